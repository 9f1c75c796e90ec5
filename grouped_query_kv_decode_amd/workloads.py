"""Seeded synthetic decode workloads (shared by tests and the benchmark).

This module only draws inputs; it holds none of the attention arithmetic.
Shapes follow the models the pages name (wikillm "Grouped-query attention
(GQA)", Variants: Mistral 7B has 32 query heads and 8 K/V heads; the paper's
T5-XXL setting has 64 heads and sweeps the group count; Gemma 2 uses two query
heads per K/V head, 32 / 16 for the 27B model).  The pages measure on T5 tasks
that are not available here; seeded Gaussian caches of these shapes stand in.

Recipe: q, K and V are drawn as float32 N(0, 1) from a torch generator seeded
per workload, multiplied by the workload's value scale, optionally given
outliers (K elements picked with probability p multiplied by a factor), and
rounded once to the storage dtype.  Ragged lengths are drawn on the CPU
(uniform integers in [1, Lmax]) so they do not depend on the device.  Cache
positions at or beyond a sequence's length hold NaN (``pad="nan"``), zeros,
or are left unwritten (``pad="none"``).
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    G: int
    d: int
    Lmax: int
    dtype: str          # "f32" or "bf16"
    seed: int
    value_scale: float = 1.0
    k_outlier_p: float = 0.0
    k_outlier_x: float = 1.0
    ragged: bool = False  # lengths ~ U{1..Lmax}; otherwise every length is Lmax

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def r(self) -> int:
        return self.H // self.G

    @property
    def d_model(self) -> int:
        """Width of the token's hidden state for the projections: H * d."""
        return self.H * self.d

    def with_(self, **kw) -> "Workload":
        return dataclasses.replace(self, **kw)


TINY_F32 = Workload("tiny_f32_B1_H8_G2_d64_L256", 1, 8, 2, 64, 256, "f32", 1000)
MISTRAL_7B = Workload("mistral7b_bf16_B16_H32_G8_d128_L4096", 16, 32, 8, 128, 4096, "bf16", 1001)
T5XXL_G8 = Workload("t5xxl_bf16_B32_H64_G8_d64_L2048", 32, 64, 8, 64, 2048, "bf16", 1002, value_scale=0.5)
GEMMA2_27B = Workload("gemma2_27b_bf16_B8_H32_G16_d128_L8192", 8, 32, 16, 128, 8192, "bf16", 1003,
                      k_outlier_p=0.01, k_outlier_x=20.0)
RAGGED = Workload("ragged_bf16_B64_H64_G8_d128_Lmax32768", 64, 64, 8, 128, 32768, "bf16", 1004, ragged=True)


def t5xxl_sweep(G: int) -> Workload:
    """The T5-XXL-shaped workload at another group count (H = 64 throughout)."""
    if G == 8:
        return T5XXL_G8
    return T5XXL_G8.with_(name="t5xxl_bf16_B32_H64_G%d_d64_L2048" % G, G=G, seed=1002 + G)


T5XXL_SWEEP_G = (1, 4, 8, 16, 64)

WORKLOADS = {w.name: w for w in [TINY_F32, MISTRAL_7B, T5XXL_G8, GEMMA2_27B, RAGGED]}
for _g in T5XXL_SWEEP_G:
    WORKLOADS[t5xxl_sweep(_g).name] = t5xxl_sweep(_g)


def seq_lens_for(w: Workload, seed_offset: int = 0):
    """int32 lengths [B] on the CPU."""
    import torch
    if not w.ragged:
        return torch.full((w.B,), w.Lmax, dtype=torch.int32)
    gen = torch.Generator("cpu").manual_seed(w.seed * 7919 + seed_offset)
    return torch.randint(1, w.Lmax + 1, (w.B,), generator=gen, dtype=torch.int64).to(torch.int32)


def _torch_dtype(w: Workload):
    import torch
    return torch.float32 if w.dtype == "f32" else torch.bfloat16


def make_inputs(w: Workload, device="cpu", pad: str = "nan", seed_offset: int = 0, seq_lens=None):
    """Seeded (q, k_cache, v_cache, seq_lens) for a workload.

    q [B,H,d], k/v [B,G,Lmax,d] in the workload dtype on ``device``;
    seq_lens [B] int32 on ``device``.  Each sequence's cache is drawn
    separately, so peak temporary memory is one sequence's float32 K or V.
    """
    import torch
    dev = torch.device(device)
    dt = _torch_dtype(w)
    gen = torch.Generator(dev.type if dev.type != "cuda" else dev).manual_seed(w.seed + 100003 * seed_offset)
    lens = seq_lens_for(w, seed_offset) if seq_lens is None else seq_lens.to("cpu", torch.int32)

    q = (torch.randn((w.B, w.H, w.d), generator=gen, device=dev) * w.value_scale).to(dt)
    alloc = torch.empty if pad == "none" else (torch.zeros if pad == "zero" else None)
    if alloc is None:
        k = torch.full((w.B, w.G, w.Lmax, w.d), float("nan"), dtype=dt, device=dev)
        v = torch.full((w.B, w.G, w.Lmax, w.d), float("nan"), dtype=dt, device=dev)
    else:
        k = alloc((w.B, w.G, w.Lmax, w.d), dtype=dt, device=dev)
        v = alloc((w.B, w.G, w.Lmax, w.d), dtype=dt, device=dev)
    for b in range(w.B):
        n = int(lens[b])
        if n == 0:
            continue
        kb = torch.randn((w.G, n, w.d), generator=gen, device=dev) * w.value_scale
        if w.k_outlier_p > 0:
            mask = torch.rand((w.G, n, w.d), generator=gen, device=dev) < w.k_outlier_p
            kb = torch.where(mask, kb * w.k_outlier_x, kb)
        k[b, :, :n] = kb.to(dt)
        del kb
        vb = torch.randn((w.G, n, w.d), generator=gen, device=dev) * w.value_scale
        v[b, :, :n] = vb.to(dt)
        del vb
    return q, k, v, lens.to(dev)


def valid_kv_positions(w: Workload, seq_lens) -> int:
    """Number of cached (sequence, position) pairs attended: sum of clamped lengths."""
    return int(seq_lens.to("cpu", copy=False).clamp(0, w.Lmax).sum())
