"""HIP path (through the C ABI) against the CPU oracle, on the GPU.

Tolerances: max |gpu - oracle| <= 1e-5 for float32 inputs and <= 2e-2 for
bfloat16 inputs (binary32 accumulation, one rounding of the output; the
oracle reads the same rounded inputs in binary64).  The mean-pool helper must
match bit for bit.
"""
import math
import os

import numpy as np
import pytest
import torch

import grouped_query_kv_decode_amd as gqa
from grouped_query_kv_decode_amd import workloads as wl
import oracle

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-5, "bf16": 2e-2}
# A second, relative bar: max|gpu - oracle| <= REL * max|oracle|.  The
# absolute tolerance is the stated one, but outputs are averages of many
# values and often far below it; the relative bar catches a lost split or
# row there.  bf16: output and probability rounding are 2^-9 relative (worst
# observed over the suite 0.43% of max|out|); fp32: binary32 rounding.
REL = {"f32": 1e-4, "bf16": 2e-2}
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    gqa.load_library()
    yield


@pytest.fixture
def env(monkeypatch):
    """Set launch-plan environment overrides for one test."""
    def set_(**kw):
        for k, v in kw.items():
            if v is None:
                monkeypatch.delenv(k, raising=False)
            else:
                monkeypatch.setenv(k, str(v))
    set_(GQA_KERNEL=None, GQA_CHUNK=None, GQA_TARGET_WGS=None, GQA_MAX_CHUNK=None, GQA_MERGE=None, GQA_WAVES=None,
         GQA_CONTIG=None, GQA_HEAD_SPLIT=None, GQA_FUSED_MAX_SPLITS=None, GQA_ORDER=None, GQA_TEMPORAL=None)
    return set_


def run_gpu(q, k, v, lens, scale):
    out = gqa.decode(q, k, v, lens, scale)
    torch.cuda.synchronize()
    return out


def oracle_out(q, k, v, lens, scale, rows=None):
    """Oracle on the host copies; rows = optional list of sequences to compute."""
    if rows is None:
        return oracle.decode(q.cpu(), k.cpu(), v.cpu(), lens.cpu(), scale)
    outs = []
    for b in rows:
        n = max(1, min(int(lens[b]), k.shape[2]))
        outs.append(oracle.decode(q[b:b + 1].cpu(), k[b:b + 1, :, :n].cpu(), v[b:b + 1, :, :n].cpu(),
                                  lens[b:b + 1].cpu(), scale)[0])
    return np.stack(outs)


def check(out, ref, dtype, what="", at_output_scale=False):
    """at_output_scale (binary32 runs of the bf16 workloads, whose outputs
    reach several units): the absolute bar is taken at the output's scale,
    TOL * max(1, max|out|), since binary32 rounding is relative."""
    got = out.detach().float().cpu().double().numpy()
    assert got.shape == ref.shape
    assert np.all(np.isfinite(got)), what + ": non-finite output"
    err = float(np.max(np.abs(got - ref))) if got.size else 0.0
    top = float(np.max(np.abs(ref))) if ref.size else 0.0
    print("%s max|err| = %.3g (max|out| = %.3g)" % (what, err, top))
    tol = TOL[dtype] * (max(1.0, top) if at_output_scale else 1.0)
    assert err <= tol, "%s: max|err| %.3g > %.3g" % (what, err, tol)
    assert err <= REL[dtype] * top or top == 0.0, "%s: max|err| %.3g > %.3g * max|out| %.3g" % (what, err, REL[dtype], top)
    return err


def check_relative(out, ref, what, rel=0.01):
    """For long sequences, whose outputs are averages of very many values and
    so far below the absolute tolerance: max|gpu - oracle| <= rel * max|oracle|
    (bf16 output rounding is 2^-9 relative; leaving out one split of a long
    sequence moves the output by several percent)."""
    got = out.detach().float().cpu().double().numpy()
    err = float(np.max(np.abs(got - ref)))
    top = float(np.max(np.abs(ref)))
    print("%s relative max|err| = %.3g" % (what, err / top))
    assert err <= rel * top, "%s: max|err| %.3g > %.3g * max|out| %.3g" % (what, err, rel, top)


def rand_case(B, H, G, d, Lmax, lens, dtype, seed, scale=None, value_scale=1.0):
    w = wl.Workload("case", B, H, G, d, Lmax, dtype, seed, value_scale=value_scale)
    q, k, v, _ = wl.make_inputs(w, DEV, pad="nan", seq_lens=torch.tensor(lens, dtype=torch.int32))
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return q, k, v, lens_t, (w.scale if scale is None else scale)


# --------------------------------------------------------------- small shapes, every path

SMALL = [
    # (B, H, G, d, Lmax, lens)
    (1, 8, 2, 64, 256, [256]),
    (3, 8, 2, 128, 600, [600, 1, 333]),
    (2, 32, 8, 128, 1000, [1000, 517]),
    (4, 12, 4, 64, 300, [129, 128, 127, 31]),     # r = 3
    (2, 16, 16, 128, 700, [700, 65]),             # G = H (MHA)
    (2, 16, 1, 64, 400, [400, 97]),               # G = 1 (MQA), r = 16
    (2, 24, 1, 128, 300, [300, 33]),              # r = 24 (two head blocks)
    (2, 64, 1, 64, 260, [260, 200]),              # r = 64 (four head blocks)
    (2, 64, 8, 64, 520, [520, 7]),                # r = 8
    (2, 6, 3, 128, 90, [90, 45]),                 # r = 2, less than one tile per wave
]


@pytest.mark.parametrize("case", SMALL, ids=lambda c: "B%d_H%d_G%d_d%d_L%d" % c[:5])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kernel", ["default", "valu"])
@pytest.mark.parametrize("chunk", [None, 32, 128, 100000])
@pytest.mark.parametrize("merge", ["fused", "kernel", "wide"])
def test_small_parity(env, case, dtype, kernel, chunk, merge):
    """merge: in the decode kernel, the per-unit merge kernel, or the wide
    merge kernel (forced for every split plan)."""
    B, H, G, d, L, lens = case
    env(GQA_KERNEL=None if kernel == "default" else kernel, GQA_CHUNK=chunk,
        GQA_MERGE="kernel" if merge == "kernel" else None, GQA_FUSED_MAX_SPLITS=1 if merge == "wide" else None)
    q, k, v, lens_t, scale = rand_case(B, H, G, d, L, lens, dtype, seed=sum(case[:5]) + 7 * len(lens))
    out = run_gpu(q, k, v, lens_t, scale)
    check(out, oracle_out(q, k, v, lens_t, scale), dtype, "%s %s chunk=%s %s" % (dtype, kernel, chunk, case))


# Binary32 on the matrix cores (v_mfma_f32_16x16x4_f32; the default for 3..64
# heads per K/V head), forced with GQA_KERNEL=mfma on every small shape: r = 1
# and 2 pad the head block with zero queries, r = 24 and 64 take a workgroup
# per block of 16 heads.  Every split and merge path, then the window, the
# cache append, ragged lengths at tile edges and a dispatch order.
F32_MFMA = SMALL


@pytest.mark.parametrize("case", F32_MFMA, ids=lambda c: "B%d_H%d_G%d_d%d_L%d" % c[:5])
@pytest.mark.parametrize("chunk", [None, 32, 128, 100000])
@pytest.mark.parametrize("merge", ["fused", "kernel", "wide"])
def test_f32_matrix_cores(env, case, chunk, merge):
    B, H, G, d, L, lens = case
    env(GQA_KERNEL="mfma", GQA_CHUNK=chunk, GQA_MERGE="kernel" if merge == "kernel" else None,
        GQA_FUSED_MAX_SPLITS=1 if merge == "wide" else None)
    assert gqa.decode_kernel_kind(B, H, G, d, L, gqa.GQA_F32) == 1
    q, k, v, lens_t, scale = rand_case(B, H, G, d, L, lens, "f32", seed=sum(case[:5]) + 3 * len(lens))
    out = run_gpu(q, k, v, lens_t, scale)
    check(out, oracle_out(q, k, v, lens_t, scale), "f32", "f32 mfma chunk=%s %s %s" % (chunk, merge, case))


@pytest.mark.parametrize("chunk", [None, 64])
def test_f32_matrix_cores_window_append_order(env, chunk):
    B, H, G, d, L = 5, 32, 8, 128, 700
    lens = [700, 1, 17, 256, 513]
    env(GQA_KERNEL="mfma", GQA_CHUNK=chunk)
    q, k, v, lens_t, scale = rand_case(B, H, G, d, L, lens, "f32", seed=41)
    for W in (1, 15, 16, 17, 300):
        out = gqa.decode_window(q, k, v, lens_t, scale, window=W)
        torch.cuda.synchronize()
        ref = oracle.decode(q.cpu(), k.cpu(), v.cpu(), lens_t.cpu(), scale, window=W)
        check(out, ref, "f32", "f32 mfma window %d chunk=%s" % (W, chunk))
    # the append writes position len-1 of each sequence (lengths count the new token)
    k_new = torch.randn(B, G, d, device=DEV)
    v_new = torch.randn(B, G, d, device=DEV)
    k2, v2 = k.clone(), v.clone()
    out = gqa.decode_append(q, k_new, v_new, k2, v2, lens_t, scale)
    torch.cuda.synchronize()
    ref, rk, rv = oracle.decode_append(q.cpu(), k_new.cpu(), v_new.cpu(), k.cpu(), v.cpu(), lens_t.cpu(), scale)
    check(out, ref, "f32", "f32 mfma append chunk=%s" % chunk)
    for b, n in enumerate(lens):
        assert np.array_equal(k2[b, :, :n].cpu().numpy(), np.asarray(rk)[b, :, :n])
        assert np.array_equal(v2[b, :, :n].cpu().numpy(), np.asarray(rv)[b, :, :n])
    # several rounds of workgroups, taken largest first by the order kernel
    env(GQA_KERNEL="mfma", GQA_CHUNK=32, GQA_ORDER=1)
    out = run_gpu(q, k, v, lens_t, scale)
    check(out, oracle_out(q, k, v, lens_t, scale), "f32", "f32 mfma ordered")


# Many splits per sequence: beyond 32 the splits are merged by the wide merge
# kernel (a workgroup per sequence, head and 32 dimensions; 32 slices of
# splits folded in order).  Sequences with few and with many splits side by
# side; slice counts that do not divide the splits.
MANY_SPLITS = [
    # (B, H, G, d, Lmax, lens, chunk)
    (3, 32, 8, 128, 9000, [9000, 4100, 300], 256),     # 36 splits, 17, 2
    (2, 8, 1, 128, 20000, [20000, 16 * 256 + 1], 256),  # r = 8: 79 splits; 17
    (2, 64, 1, 64, 12000, [12000, 5000], 256),         # head chunks: 47 and 20 splits
    (1, 8, 2, 64, 8192, [8192], 32),                    # 256 splits, the planner's maximum
]


@pytest.mark.parametrize("case", MANY_SPLITS, ids=lambda c: "B%d_H%d_G%d_d%d_L%d_c%d" % (c[:5] + (c[6],)))
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kernel", ["default", "valu"])
@pytest.mark.parametrize("merge", ["fused", "kernel"])
def test_many_splits(env, case, dtype, kernel, merge):
    B, H, G, d, L, lens, chunk = case
    env(GQA_KERNEL=None if kernel == "default" else kernel, GQA_CHUNK=chunk,
        GQA_MERGE=None if merge == "fused" else "kernel")
    q, k, v, lens_t, scale = rand_case(B, H, G, d, L, lens, dtype, seed=sum(case[:5]) + chunk)
    out = run_gpu(q, k, v, lens_t, scale)
    check(out, oracle_out(q, k, v, lens_t, scale), dtype, "%s %s %s %s" % (dtype, kernel, merge, case))


def test_many_splits_window_and_append(env):
    """Sliding window and cache append with more than 32 splits per sequence."""
    env(GQA_CHUNK=256)
    B, H, G, d, L = 2, 32, 8, 128, 9000
    lens = [9000, 6100]
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, "bf16", seed=31)
    gen = torch.Generator(DEV).manual_seed(32)
    kn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
    out_w = gqa.decode_window(q, k, v, lt, scale, window=5000)
    torch.cuda.synchronize()
    check(out_w, oracle.decode(q.cpu(), k.cpu(), v.cpu(), lt.cpu(), scale, window=5000), "bf16", "window 5000")
    k0, v0 = k.cpu(), v.cpu()
    out = gqa.decode_append(q, kn, vn, k, v, lt, scale)
    torch.cuda.synchronize()
    ref, rk, rv = oracle.decode_append(q.cpu(), kn.cpu(), vn.cpu(), k0, v0, lt.cpu(), scale)
    check(out, ref, "bf16", "append, many splits")
    assert np.array_equal(k.cpu().view(torch.int16).numpy().view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(v.cpu().view(torch.int16).numpy().view(np.uint16), rv.view(np.uint16))


def test_wide_merge_by_partial_bytes(env):
    """At most 32 splits, but 16 heads x 16 splits of 128-dimension partials
    (133 KB) for the merging workgroup to read: the plan takes the wide merge
    kernel.  Against the oracle (full, partial and one-position sequences),
    and the same bits call after call."""
    B, H, G, d, L = 3, 64, 4, 128, 4096
    lens = [4096, 2049, 1]
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, "bf16", seed=860)
    out = run_gpu(q, k, v, lt, scale).clone()
    check(out, oracle_out(q, k, v, lt, scale), "bf16", "wide merge by bytes")
    for _ in range(3):
        assert torch.equal(run_gpu(q, k, v, lt, scale), out)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_long_single_sequence(env, dtype):
    """One sequence, one K/V head, 131072 positions: the planner's 256 splits
    of 512 positions (every compute unit busy), merged by the wide kernel."""
    w = wl.Workload("long", 1, 8, 1, 128, 131072, dtype, 41)
    q, k, v, lens = wl.make_inputs(w, DEV)
    out = run_gpu(q, k, v, lens, w.scale)
    ref = oracle_out(q, k, v, lens, w.scale)
    check(out, ref, dtype, "B1 H8 G1 d128 L131072 " + dtype)
    check_relative(out, ref, "B1 H8 G1 d128 L131072 " + dtype, rel=0.01 if dtype == "bf16" else 1e-4)


@pytest.mark.parametrize("dtype,kernel", [("bf16", "default"), ("f32", "default"), ("bf16", "valu")])
def test_dispatch_order(env, dtype, kernel):
    """Grids of more than 1024 workgroups with several splits run their items
    largest first (an order kernel sorts them on the device): only the
    schedule changes, so outputs are bit-equal to blockIdx order - with the
    in-kernel merge, the merge kernel, a window and a cache append - and
    agree with the oracle."""
    B, H, G, d, L = 48, 32, 8, 128, 6000
    gen = torch.Generator().manual_seed(71)
    lens = [int(x) for x in torch.randint(1, L + 1, (B,), generator=gen)]
    lens[:3] = [L, 1, 513]
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, dtype, seed=72)
    kernel_env = None if kernel == "default" else kernel
    for merge in (None, "kernel"):
        env(GQA_KERNEL=kernel_env, GQA_CHUNK=256, GQA_MERGE=merge, GQA_ORDER=0)   # 384 units x 24 splits
        ref = run_gpu(q, k, v, lt, scale).clone()
        env(GQA_ORDER=None)
        for _ in range(3):
            assert torch.equal(run_gpu(q, k, v, lt, scale), ref)
    check(ref.cpu()[:8], oracle_out(q, k, v, lt, scale, rows=list(range(8))), dtype, "ordered grid, sampled rows")
    env(GQA_ORDER=0)
    ref_w = gqa.decode_window(q, k, v, lt, scale, window=2500).clone()
    env(GQA_ORDER=None)
    assert torch.equal(gqa.decode_window(q, k, v, lt, scale, window=2500), ref_w)
    gen = torch.Generator(DEV).manual_seed(73)
    dt = torch.float32 if dtype == "f32" else torch.bfloat16
    kn = torch.randn((B, G, d), generator=gen, device=DEV).to(dt)
    vn = torch.randn((B, G, d), generator=gen, device=DEV).to(dt)
    k0, v0 = k.clone(), v.clone()
    env(GQA_ORDER=0)
    ref_a = gqa.decode_append(q, kn, vn, k0, v0, lt, scale).clone()
    env(GQA_ORDER=None)
    k1, v1 = k.clone(), v.clone()
    assert torch.equal(gqa.decode_append(q, kn, vn, k1, v1, lt, scale), ref_a)
    bits = torch.int32 if dtype == "f32" else torch.int16
    assert torch.equal(k1.view(bits), k0.view(bits)) and torch.equal(v1.view(bits), v0.view(bits))


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_dispatch_order_large_batch(env, dtype):
    """More sequences than the order kernel stages in LDS (4096): it then reads
    each item's length from memory.  Outputs are bit-equal with the order
    forced off, forced on and left to the plan (on: 50,000 workgroups of 5
    splits), and sampled sequences - both sides of the 4096 boundary, empty
    ones included - agree with the oracle."""
    B, H, G, d, L = 5000, 8, 2, 64, 160
    gen = torch.Generator().manual_seed(81)
    lens = [int(x) for x in torch.randint(0, L + 1, (B,), generator=gen)]
    lens[:3] = [L, 0, 1]
    lens[4096] = L
    lens[-1] = 33
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, dtype, seed=82)
    env(GQA_CHUNK=32, GQA_ORDER=0)
    ref = run_gpu(q, k, v, lt, scale).clone()
    for order in (1, None):
        env(GQA_ORDER=order)
        assert torch.equal(run_gpu(q, k, v, lt, scale), ref), "order %s" % order
    picks = [int(x) for x in torch.randint(0, B, (24,), generator=gen)]
    rows = sorted(set([0, 1, 2, 4095, 4096, 4097, B - 1] + picks))
    check(ref.cpu()[rows], oracle_out(q, k, v, lt, scale, rows=rows), dtype, "B5000 ordered, sampled rows")


PLAN_SHAPES = [
    # (B, H, G, d, L, dtype): default plans chosen by the launch estimates
    (6, 32, 8, 128, 4096, "bf16"),     # 48 units: 5 splits, 240 workgroups
    (12, 32, 8, 128, 4096, "bf16"),    # 96 units: 5 splits, two full rounds
    (48, 32, 8, 128, 2048, "bf16"),    # 384 units: 2 splits, three full rounds
    (4, 32, 1, 128, 16384, "bf16"),    # 32 heads per K/V head: 1 head chunk, 64 splits (wide merge)
    (64, 64, 1, 64, 4096, "bf16"),     # 64 heads per K/V head: 2 head chunks
    (12, 32, 8, 128, 2048, "f32"),     # binary32 matrix cores, 96 units: 5 splits, two full rounds
    (4, 32, 8, 128, 8192, "f32"),      # binary32 matrix cores, 32 units: 8 splits
    (64, 32, 8, 128, 2048, "f32"),     # binary32 matrix cores, 512 units: one split each
    (1, 8, 2, 64, 1024, "f32"),        # binary32 matrix cores, one-round grid: 16 splits of 64 by the estimate
    (2, 64, 1, 64, 4096, "f32"),       # binary32 matrix cores, r = 64: four head chunks
    (8, 32, 16, 128, 4096, "f32"),     # binary32 r = 2: the VALU kernel
    (20, 32, 16, 128, 4096, "f32"),    # binary32 r = 2, 320 units (not whole rounds): matrix cores
    (3, 32, 32, 128, 8192, "f32"),     # binary32 r = 1, 96 units: matrix cores
    (4, 32, 32, 64, 512, "bf16"),      # VALU (r = 1): 2 -> 1 split by the estimate
    (64, 64, 8, 128, 16384, "bf16"),   # 8192-position split cap: 2 splits, 1024 workgroups
]


@pytest.mark.parametrize("shape", PLAN_SHAPES, ids=lambda c: "B%d_H%d_G%d_d%d_L%d_%s" % c)
def test_default_plan_shapes(env, shape):
    """Shapes whose default plans come from the split-count, head-chunk,
    binary32 and VALU split estimates and the split cap, against the
    oracle on sampled sequences (ragged lengths keep every split path busy)."""
    B, H, G, d, L, dtype = shape
    gen = torch.Generator().manual_seed(B * 131 + L)
    lens = [int(x) for x in torch.randint(1, L + 1, (B,), generator=gen)]
    lens[0] = L
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, dtype, seed=90 + B)
    out = run_gpu(q, k, v, lt, scale)
    # sampled sequences, indexed on the host copy (a bad index then raises
    # on the CPU instead of reading out of bounds on the device)
    rows = sorted(set(r for r in (0, 1, B // 2, B - 1) if r < B))
    check(out.cpu()[rows], oracle_out(q, k, v, lt, scale, rows=rows), dtype, "plan shape %s" % (shape,))


@pytest.mark.parametrize("cap", [None, 4096])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_very_long_sequence(env, cap, dtype):
    """2,097,152 positions: the default 8192-position split cap gives the
    planner's usual 256 splits; a 4096 cap gives 512 (more than 256), merged
    by the wide kernel 16 per slice.  Both matrix-core kernels (r = 8)."""
    env(GQA_MAX_CHUNK=cap)
    w = wl.Workload("very_long", 1, 8, 1, 64, 1 << 21, dtype, 43)
    q, k, v, lens = wl.make_inputs(w, DEV)
    out = run_gpu(q, k, v, lens, w.scale)
    ref = oracle_out(q, k, v, lens, w.scale)
    check(out, ref, dtype, "B1 H8 G1 d64 L2097152 %s cap %s" % (dtype, cap))
    check_relative(out, ref, "B1 H8 G1 d64 L2097152 " + dtype, rel=0.01 if dtype == "bf16" else 1e-4)


def test_tiny_workload_fp32(env):
    w = wl.TINY_F32
    q, k, v, lens = wl.make_inputs(w, DEV)
    out = run_gpu(q, k, v, lens, w.scale)
    check(out, oracle_out(q, k, v, lens, w.scale), "f32", w.name)


# --------------------------------------------------------------- edge cases

@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_empty_and_clamped_lengths(env, dtype):
    env(GQA_CHUNK=128)
    q, k, v, _, scale = rand_case(3, 8, 2, 128, 300, [300, 300, 300], dtype, seed=5)
    lens = torch.tensor([0, 1000, 1], dtype=torch.int32, device=DEV)
    out = run_gpu(q, k, v, lens, scale)
    assert torch.all(out[0] == 0)
    ref = oracle_out(q, k, v, lens, scale)
    check(out, ref, dtype, "len 0 / >Lmax / 1")
    # one position: the output is that value row, rounded once
    for h in range(8):
        assert torch.equal(out[2, h], v[2, h // 4, 0])


def test_empty_batch(env):
    q = torch.empty((0, 8, 64), dtype=torch.bfloat16, device=DEV)
    k = torch.empty((0, 2, 16, 64), dtype=torch.bfloat16, device=DEV)
    out = gqa.decode(q, k, k, torch.empty((0,), dtype=torch.int32, device=DEV), 0.125)
    assert out.shape == (0, 8, 64)


@pytest.mark.parametrize("waves", [4, 8, 16])
@pytest.mark.parametrize("contig", [0, 1])
@pytest.mark.parametrize("case", [(3, 32, 8, 128, 3000, [3000, 1, 1777]), (4, 64, 8, 64, 2100, [2100, 2047, 33, 1000]),
                                  (2, 48, 2, 128, 900, [900, 450])], ids=["d128_r4", "d64_r8", "d128_r24"])
def test_launch_variants(env, waves, contig, case):
    """Every workgroup size and tile order of the matrix-core kernel, single
    and multi-split plans (first-tile prefetch used and discarded)."""
    B, H, G, d, L, lens = case
    q, k, v, lens_t, scale = rand_case(B, H, G, d, L, lens, "bf16", seed=31 + waves + contig)
    ref = oracle_out(q, k, v, lens_t, scale)
    for chunk in (None, 512, 1000):
        env(GQA_WAVES=waves, GQA_CONTIG=contig, GQA_CHUNK=chunk)
        out = run_gpu(q, k, v, lens_t, scale)
        check(out, ref, "bf16", "waves=%d contig=%d chunk=%s %s" % (waves, contig, chunk, case[:5]))


HEAD_SPLIT_CASES = [
    # (B, H, G, d, Lmax, lens): r = 64, 24, 48 and 40 (last head chunk partly empty)
    (3, 64, 1, 64, 1500, [1500, 513, 7]),
    (2, 24, 1, 128, 900, [900, 300]),
    (2, 48, 1, 64, 700, [700, 1]),
    (2, 80, 2, 128, 600, [600, 333]),
]


@pytest.mark.parametrize("case", HEAD_SPLIT_CASES, ids=lambda c: "H%d_G%d_d%d" % c[1:4])
@pytest.mark.parametrize("split", [1, 2, 4])
@pytest.mark.parametrize("merge", ["fused", "kernel"])
def test_head_split(env, case, split, merge):
    """The matrix-core kernel with the group's head blocks spread over 1, 2
    or 4 workgroups (the planner drops to a split that leaves no workgroup
    without heads), fused or separate merge, against the oracle."""
    env(GQA_HEAD_SPLIT=split, GQA_CHUNK=256, GQA_MERGE=None if merge == "fused" else "kernel")
    q, k, v, lens, scale = rand_case(*case, "bf16", seed=sum(case[:5]) + split)
    out = run_gpu(q, k, v, lens, scale)
    check(out, oracle_out(q, k, v, lens, scale), "bf16", "head split %d %s %s" % (split, merge, case[:5]))


@pytest.mark.parametrize("split", [1, 4])
def test_head_split_append_and_window(env, split):
    env(GQA_HEAD_SPLIT=split, GQA_CHUNK=256)
    B, H, G, d, L = 3, 64, 1, 64, 1100
    lens = [1100, 700, 1]
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, "bf16", seed=900 + split)
    gen = torch.Generator(DEV).manual_seed(split)
    kn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
    k0, v0 = k.cpu(), v.cpu()
    out = gqa.decode_append(q, kn, vn, k, v, lt, scale, window=300)
    torch.cuda.synchronize()
    ref, rk, rv = oracle.decode_append(q.cpu(), kn.cpu(), vn.cpu(), k0, v0, lt.cpu(), scale, window=300)
    check(out, ref, "bf16", "head split %d append+window" % split)
    assert np.array_equal(k.cpu().view(torch.int16).numpy().view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(v.cpu().view(torch.int16).numpy().view(np.uint16), rv.view(np.uint16))


@pytest.mark.parametrize("kernel", ["default", "valu"])
def test_split_boundaries(env, kernel):
    """Lengths at chunk and tile boundaries +-1 with several splits."""
    env(GQA_KERNEL=None if kernel == "default" else kernel, GQA_CHUNK=256)
    lens = [255, 256, 257, 511, 512, 513, 31, 32, 33, 1]
    q, k, v, lens_t, scale = rand_case(len(lens), 32, 8, 128, 520, lens, "bf16", seed=77)
    out = run_gpu(q, k, v, lens_t, scale)
    check(out, oracle_out(q, k, v, lens_t, scale), "bf16", "split boundaries " + kernel)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_large_scores_stay_finite(env, dtype):
    """q and K scaled by 8: scores 64x their usual size (softmax far from
    uniform, exp2 arguments in the hundreds).  binary32: a score's rounding
    error grows with sum |q_i k_i|, 64x here, so the absolute 1e-5 bar (for
    scores of the usual size) is replaced by the binary32 relative bar,
    1e-4 of max|out| (observed 5.8e-6)."""
    q, k, v, lens, scale = rand_case(2, 16, 4, 128, 700, [700, 300], dtype, seed=8)
    q.mul_(8)
    k.mul_(8)
    out = run_gpu(q, k, v, lens, scale)
    ref = oracle_out(q, k, v, lens, scale)
    if dtype == "bf16":
        check(out, ref, dtype, "large scores")
    else:
        assert torch.isfinite(out).all()
        check_relative(out, ref, "large scores f32", rel=REL["f32"])


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_nan_inside_valid_positions_propagates(env, dtype):
    env(GQA_CHUNK=128)
    q, k, v, lens, scale = rand_case(2, 8, 2, 128, 300, [300, 300], dtype, seed=9)
    k[0, 1, 17, 5] = float("nan")
    out = run_gpu(q, k, v, lens, scale).float().cpu()
    ref = oracle_out(q, k, v, lens, scale)
    assert np.array_equal(np.isnan(out.numpy()), np.isnan(ref))
    assert torch.isnan(out[0, 4:]).all() and not torch.isnan(out[0, :4]).any() and not torch.isnan(out[1]).any()


def test_deterministic_and_workspace_reuse(env):
    env(GQA_CHUNK=128)
    a = rand_case(3, 32, 8, 128, 900, [900, 400, 129], "bf16", seed=10)
    b = rand_case(5, 16, 2, 64, 300, [300, 1, 2, 299, 150], "bf16", seed=11)
    o1 = run_gpu(*a).clone()
    o2 = run_gpu(*b).clone()
    o3 = run_gpu(*a).clone()
    assert torch.equal(o1, o3)
    check(o2, oracle_out(*b), "bf16", "second shape")
    check(o3, oracle_out(*a), "bf16", "reuse")


def test_non_default_stream(env):
    env(GQA_CHUNK=128)
    q, k, v, lens, scale = rand_case(2, 32, 8, 128, 640, [640, 300], "bf16", seed=12)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out = gqa.decode(q, k, v, lens, scale)
    s.synchronize()
    check(out, oracle_out(q, k, v, lens, scale), "bf16", "side stream")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("plan", ["fused", "merge_kernel", "wide", "ordered"])
def test_decode_in_two_phases(env, dtype, plan):
    """gqa_decode_phase: phase 1 (the split kernel, with the order kernel
    before it when the plan orders) then phase 2 (the separate merge kernel,
    nothing when the merge runs in the split kernel) on one stream give
    exactly what gqa_decode gives."""
    env(GQA_CHUNK=64 if plan != "wide" else 32, GQA_MERGE="kernel" if plan == "merge_kernel" else None,
        GQA_ORDER=1 if plan == "ordered" else None)
    q, k, v, lt, scale = rand_case(5, 32, 8, 128, 1900, [1900, 1, 640, 1899, 33], dtype, seed=16)
    ref = run_gpu(q, k, v, lt, scale).clone()
    out = torch.full_like(ref, float("nan"))
    gqa.decode_phase(1, q, k, v, lt, scale, out=out)
    gqa.decode_phase(2, q, k, v, lt, scale, out=out)
    torch.cuda.synchronize()
    assert torch.equal(out, ref), "%s %s" % (dtype, plan)
    check(out, oracle_out(q, k, v, lt, scale), dtype, "two phases %s %s" % (dtype, plan))


def test_concurrent_streams(env):
    """Two side streams (default priority) each running split plans at the
    same time, with no synchronisation between them: the binding keeps one
    workspace per stream, so the arrival counters and partials of the two
    never mix.  Every call bit-equal to the same call run alone."""
    env(GQA_CHUNK=128)
    a = rand_case(3, 32, 8, 128, 900, [900, 400, 129], "bf16", seed=14)
    b = rand_case(4, 16, 4, 128, 1000, [1000, 999, 513, 1], "f32", seed=15)
    ref_a = run_gpu(*a).clone()
    ref_b = run_gpu(*b).clone()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    outs = []
    for _ in range(5):
        with torch.cuda.stream(s1):
            oa = gqa.decode(*a)
        with torch.cuda.stream(s2):
            ob = gqa.decode(*b)
        outs.append((oa, ob))
    s1.synchronize()
    s2.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa, ref_a) and torch.equal(ob, ref_b)
    check(ref_a, oracle_out(*a), "bf16", "stream a")
    check(ref_b, oracle_out(*b), "f32", "stream b")


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_equal_queries_in_a_group(env, dtype):
    q, k, v, lens, scale = rand_case(1, 16, 4, 128, 500, [500], dtype, seed=13)
    q[0, 4:8] = q[0, 4]
    out = run_gpu(q, k, v, lens, scale)
    for h in range(4, 8):
        assert torch.equal(out[0, h], out[0, 4])


MHA_CASES = [(3, 8, 8, 128, 3000, [3000, 1, 1777]), (2, 16, 16, 64, 2100, [2100, 33])]


@pytest.mark.parametrize("case", MHA_CASES, ids=["d128", "d64"])
@pytest.mark.parametrize("plan", [(None, None), (256, None), (256, "kernel"), (100000, None)],
                         ids=["default_split", "split256", "split256_mergekernel", "unsplit"])
def test_mha_on_matrix_cores(env, case, plan):
    """r = 1 (G = H) on the matrix-core kernel, the default for bfloat16 MHA
    calls of at least 32 MiB of K and V (forced here on small shapes): one
    real head in a block of 16.  Plain decode, sliding window and the cache
    append against the oracle."""
    chunk, merge = plan
    env(GQA_KERNEL="mfma", GQA_CHUNK=chunk, GQA_MERGE=merge)
    B, H, G, d, L, lens = case
    assert gqa.decode_kernel_kind(B, H, G, d, L, gqa.GQA_BF16) == 1
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, "bf16", seed=700 + d)
    check(run_gpu(q, k, v, lt, scale), oracle_out(q, k, v, lt, scale), "bf16", "MHA mfma %s %s" % (plan, case[:5]))
    out_w = gqa.decode_window(q, k, v, lt, scale, 1000)
    torch.cuda.synchronize()
    check(out_w, oracle.decode(q.cpu(), k.cpu(), v.cpu(), lt.cpu(), scale, window=1000), "bf16", "MHA mfma window")
    gen = torch.Generator(DEV).manual_seed(701)
    kn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
    vn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
    k0, v0 = k.cpu(), v.cpu()
    out_a = gqa.decode_append(q, kn, vn, k, v, lt, scale)
    torch.cuda.synchronize()
    ref, rk, rv = oracle.decode_append(q.cpu(), kn.cpu(), vn.cpu(), k0, v0, lt.cpu(), scale)
    check(out_a, ref, "bf16", "MHA mfma append")
    assert np.array_equal(k.cpu().view(torch.int16).numpy().view(np.uint16), rk.view(np.uint16))
    assert np.array_equal(v.cpu().view(torch.int16).numpy().view(np.uint16), rv.view(np.uint16))


# Invariants of the decode-step block (softmax weights, then their weighted
# sum of value rows) on every kernel and merge path: unsplit, split with the
# in-kernel merge, split with the merge kernel; both element types.
INVARIANT_PLANS = [("default", 100000, None), ("default", 128, None), ("default", 128, "kernel"),
                   ("valu", 100000, None), ("valu", 128, None), ("valu", 128, "kernel"),
                   ("mfma", 100000, None), ("mfma", 256, None)]  # (binary32 has no matrix-core path: VALU)
INVARIANT_CASES = [(3, 32, 8, 128, 600, [600, 257, 1]),   # r = 4
                   (2, 64, 4, 64, 500, [500, 33]),        # r = 16
                   (2, 8, 8, 128, 300, [300, 129])]       # r = 1


def _invariant_env(env, plan):
    kernel, chunk, merge = plan
    env(GQA_KERNEL=None if kernel == "default" else kernel, GQA_CHUNK=chunk, GQA_MERGE=merge)


@pytest.mark.parametrize("case", INVARIANT_CASES, ids=["r4", "r16", "r1"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("plan", INVARIANT_PLANS, ids=lambda p: "%s_c%d_%s" % (p[0], p[1], p[2] or "fused"))
def test_constant_values_come_back(env, case, dtype, plan):
    """V constant over the attended positions of each (sequence, K/V head):
    the weights sum to one, so every query head of the group returns that
    constant - exactly after the final rounding for bfloat16 (the weight sum
    adds the same rounded weights that multiply V), within the binary32
    tolerance for float32.  Padding holds NaN and stays unread."""
    _invariant_env(env, plan)
    B, H, G, d, L, lens = case
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, dtype, seed=300 + d + B)
    gen = torch.Generator().manual_seed(301 + B)
    consts = (torch.rand((B, G), generator=gen) * 6 - 3).to(torch.bfloat16).float()  # exact in both types
    for b in range(B):
        for g in range(G):
            v[b, g, :lens[b]] = consts[b, g].item()
    out = run_gpu(q, k, v, lt, scale)
    want = consts.repeat_interleave(H // G, dim=1)[:, :, None].expand(B, H, d).to(torch.float64).numpy()
    if dtype == "bf16":
        assert np.array_equal(out.cpu().double().numpy(), want), "constant V did not come back exactly"
    else:
        check(out, want, dtype, "constant V %s %s" % (plan, case[:5]))


@pytest.mark.parametrize("case", INVARIANT_CASES, ids=["r4", "r16", "r1"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("plan", INVARIANT_PLANS, ids=lambda p: "%s_c%d_%s" % (p[0], p[1], p[2] or "fused"))
def test_zero_query_gives_mean_of_values(env, case, dtype, plan):
    """q = 0: every score is zero, the weights are uniform, and the output is
    the mean of the attended value rows (closed form, in binary64 on the host)."""
    _invariant_env(env, plan)
    B, H, G, d, L, lens = case
    q, k, v, lt, scale = rand_case(B, H, G, d, L, lens, dtype, seed=400 + d + B)
    q.zero_()
    out = run_gpu(q, k, v, lt, scale)
    vh = v.cpu().double().numpy()
    want = np.stack([np.repeat(vh[b, :, :lens[b]].mean(axis=1), H // G, axis=0) for b in range(B)])
    check(out, want, dtype, "q = 0 %s %s" % (plan, case[:5]))


def test_outlier_rows_alternative_reading(env):
    """Second reading of the Gemma-shaped outlier recipe: 1% of K rows x20."""
    q, k, v, lens, scale = rand_case(2, 32, 16, 128, 2048, [2048, 1500], "bf16", seed=14)
    gen = torch.Generator(DEV).manual_seed(14)
    rows = torch.rand(k.shape[:3], generator=gen, device=DEV) < 0.01
    k[rows] = (k[rows].float() * 20).to(k.dtype)
    out = run_gpu(q, k, v, lens, scale)
    check(out, oracle_out(q, k, v, lens, scale), "bf16", "outlier rows")


@pytest.mark.parametrize("kernel", ["default", "valu"])
def test_fused_merge_matches_merge_kernel(env, kernel):
    """The in-kernel merge (last-arriving workgroup) and the separate merge
    kernel do the same arithmetic in the same order: results are bit-equal,
    call after call, on shapes with many concurrent splits."""
    cases = [rand_case(16, 32, 8, 128, 4096, [4096] * 16, "bf16", seed=21),
             rand_case(32, 64, 8, 64, 2048, [2048 - 37 * i for i in range(32)], "bf16", seed=22),
             rand_case(4, 16, 4, 128, 3000, [3000, 1, 1500, 2999], "f32", seed=23),
             rand_case(3, 32, 8, 128, 9000, [9000, 4100, 300], "bf16", seed=24)]  # 36 splits: wide merge
    for q, k, v, lens, scale in cases:
        env(GQA_KERNEL=None if kernel == "default" else kernel, GQA_CHUNK=256, GQA_MERGE="kernel")
        ref = run_gpu(q, k, v, lens, scale).clone()
        env(GQA_MERGE=None)
        for _ in range(30):
            out = gqa.decode(q, k, v, lens, scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref)
        outs = [gqa.decode(q, k, v, lens, scale).clone() for _ in range(20)]
        torch.cuda.synchronize()
        for o in outs:
            assert torch.equal(o, ref)


# --------------------------------------------------------------- sliding window and cache append

WIN_CASES = [
    (4, 32, 8, 128, 3000, [3000, 2500, 100, 1]),
    (3, 64, 8, 64, 2100, [2100, 33, 1500]),
    (2, 12, 4, 128, 700, [700, 64]),   # r = 3
]


@pytest.mark.parametrize("case", WIN_CASES, ids=["d128_r4", "d64_r8", "d128_r3"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("kernel", ["default", "valu"])
def test_window_parity(env, case, dtype, kernel):
    B, H, G, d, L, lens = case
    q, k, v, lens_t, scale = rand_case(B, H, G, d, L, lens, dtype, seed=51 + d)
    for chunk in (None, 128):
        env(GQA_KERNEL=None if kernel == "default" else kernel, GQA_CHUNK=chunk)
        for W in (1, 31, 32, 33, 511, 1000, 5000):
            out = gqa.decode_window(q, k, v, lens_t, scale, W)
            torch.cuda.synchronize()
            ref = oracle.decode(q.cpu(), k.cpu(), v.cpu(), lens_t.cpu(), scale, window=W)
            check(out, ref, dtype, "window=%d chunk=%s %s" % (W, chunk, case[:5]))


APPEND_CASES = [
    (4, 32, 8, 128, 1200, [1200, 1, 32, 33]),
    (3, 64, 8, 64, 700, [700, 257, 2]),
    (2, 16, 16, 128, 300, [300, 128]),  # r = 1
    (2, 24, 1, 128, 500, [500, 17]),    # r = 24
]


@pytest.mark.parametrize("case", APPEND_CASES, ids=["d128_r4", "d64_r8", "d128_r1", "d128_r24"])
@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("plan", ["default", "valu", "split128", "mergekernel"])
def test_append_parity(env, case, dtype, plan):
    """The new key/value land in row len-1 of the caches (bit-exact, nothing
    else written) and the output matches the oracle's append-then-attend."""
    B, H, G, d, L, lens = case
    env(GQA_KERNEL="valu" if plan == "valu" else None, GQA_CHUNK=128 if plan in ("split128", "mergekernel") else None,
        GQA_MERGE="kernel" if plan == "mergekernel" else None)
    q, k, v, lens_t, scale = rand_case(B, H, G, d, L, lens, dtype, seed=61 + d + B)
    gen = torch.Generator(DEV).manual_seed(99)
    kn = torch.randn((B, G, d), generator=gen, device=DEV).to(k.dtype)
    vn = torch.randn((B, G, d), generator=gen, device=DEV).to(k.dtype)
    for W in (0, 100):
        kc, vc = k.clone(), v.clone()
        out = gqa.decode_append(q, kn, vn, kc, vc, lens_t, scale, window=W)
        torch.cuda.synchronize()
        ref, rk, rv = oracle.decode_append(q.cpu(), kn.cpu(), vn.cpu(), k.cpu(), v.cpu(), lens_t.cpu(), scale, window=W)
        check(out, ref, dtype, "append window=%d %s %s" % (W, plan, case[:5]))
        bits = torch.int16 if dtype == "bf16" else torch.int32
        # NaN padding compares by bit pattern
        assert np.array_equal(kc.cpu().view(bits).numpy().view(rk.dtype if dtype == "bf16" else np.int32),
                              rk.view(np.uint16) if dtype == "bf16" else rk.view(np.int32))
        assert np.array_equal(vc.cpu().view(bits).numpy().view(rv.dtype if dtype == "bf16" else np.int32),
                              rv.view(np.uint16) if dtype == "bf16" else rv.view(np.int32))


def test_append_matches_decode_of_updated_cache(env):
    """Append-then-attend in one launch equals a plain decode of the updated
    caches, bit for bit (same kernel arithmetic)."""
    q, k, v, lens, scale = rand_case(16, 32, 8, 128, 4096, [4096] * 8 + [4000 - 301 * i for i in range(8)], "bf16",
                                     seed=71)
    gen = torch.Generator(DEV).manual_seed(7)
    kn = torch.randn((16, 8, 128), generator=gen, device=DEV).to(torch.bfloat16)
    vn = torch.randn((16, 8, 128), generator=gen, device=DEV).to(torch.bfloat16)
    out_a = gqa.decode_append(q, kn, vn, k, v, lens, scale)
    out_d = gqa.decode(q, k, v, lens, scale)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_d)


@pytest.mark.parametrize("G", [1, 8, 64])
def test_encoder_decoder_steps(env, G):
    """A few steps of the fig. 6 setup at small size: self-attention with the
    cache append over a growing decoder cache, then cross-attention over the
    encoder positions; every step against the oracle, cache included."""
    B, H, d, T_in, T_out = 3, 64, 64, 300, 40
    q, ks, vs, _, sc = rand_case(B, H, G, d, T_out, [T_out] * B, "bf16", seed=80 + G)
    _, kx, vx, lx, _ = rand_case(B, H, G, d, T_in, [T_in, 250, 7], "bf16", seed=90 + G)
    gen = torch.Generator(DEV).manual_seed(G)
    ks_ref = ks.cpu()
    vs_ref = vs.cpu()
    for t in range(T_out):
        kn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
        vn = torch.randn((B, G, d), generator=gen, device=DEV).to(torch.bfloat16)
        lens = torch.full((B,), t + 1, dtype=torch.int32, device=DEV)
        o_self = gqa.decode_append(q, kn, vn, ks, vs, lens, sc)
        o_cross = gqa.decode(q, kx, vx, lx, sc)
        torch.cuda.synchronize()
        if t in (0, 1, 31, 32, T_out - 1):
            ref, ks_ref_np, vs_ref_np = oracle.decode_append(q.cpu(), kn.cpu(), vn.cpu(), ks_ref, vs_ref, lens.cpu(), sc)
            check(o_self, ref, "bf16", "self step %d G=%d" % (t, G))
            check(o_cross, oracle.decode(q.cpu(), kx.cpu(), vx.cpu(), lx.cpu(), sc), "bf16", "cross G=%d" % G)
        ks_ref = ks.cpu()
        vs_ref = vs.cpu()


# --------------------------------------------------------------- the named workloads at full size

FULL = [wl.MISTRAL_7B, wl.GEMMA2_27B] + [wl.t5xxl_sweep(g) for g in wl.T5XXL_SWEEP_G]


@pytest.mark.parametrize("w", FULL, ids=lambda w: w.name)
def test_full_workload(env, w):
    q, k, v, lens = wl.make_inputs(w, DEV)
    out = run_gpu(q, k, v, lens, w.scale)
    check(out, oracle_out(q, k, v, lens, w.scale), w.dtype, w.name)


# The named workloads' shapes in binary32: the binary32 matrix-core kernel at
# r = 4..64 (and the VALU kernel at the Gemma-2-27B shape's r = 2), full size,
# every sequence; the ragged batch on eight sequences incl. the shortest and
# longest (its caches are 9.3 GB in binary32).  The 1e-5 bar is the binary32
# config's, whose outputs stay below 1; here it is taken at the output's scale
# (the Gemma-2-27B shape's x20 key outliers give scores ~20x and outputs up to
# ~4.5 in magnitude, and binary32 rounding grows with both).
FULL_F32 = [w.with_(dtype="f32", name=w.name.replace("_bf16_", "_f32_"))
            for w in [wl.MISTRAL_7B, wl.GEMMA2_27B] + [wl.t5xxl_sweep(g) for g in (1, 4, 8, 16)]]


@pytest.mark.parametrize("w", FULL_F32, ids=lambda w: w.name)
def test_full_workload_binary32(env, w):
    q, k, v, lens = wl.make_inputs(w, DEV)
    out = run_gpu(q, k, v, lens, w.scale)
    check(out, oracle_out(q, k, v, lens, w.scale), w.dtype, w.name, at_output_scale=True)


def test_ragged_workload_binary32(env):
    w = wl.RAGGED.with_(dtype="f32", name=wl.RAGGED.name.replace("_bf16_", "_f32_"))
    q, k, v, lens = wl.make_inputs(w, DEV)
    out = run_gpu(q, k, v, lens, w.scale)
    lc = lens.cpu()
    rows = sorted({int(lc.argmin()), int(lc.argmax()), 0, 9, 17, 31, 42, 63})
    check(out.cpu()[rows], oracle_out(q, k, v, lens, w.scale, rows=rows), w.dtype, w.name + " rows %s" % rows,
          at_output_scale=True)


@pytest.mark.parametrize("dtype,B,H,G", [("bf16", 256, 64, 8), ("f32", 128, 32, 8), ("f32", 64, 32, 16)],
                         ids=["bf16_mfma", "f32_mfma", "f32_valu"])
def test_largest_caches(env, dtype, B, H, G):
    """Caches past 2^32 elements per tensor (d128 Lmax 32768: 8.6e9 bf16 or
    4.3e9 binary32 elements, 17 GB each), on both matrix-core kernels and
    the VALU kernel (binary32, two heads per K/V head): every address
    computed past 32 bits.  Ragged lengths (several splits, an ordered grid
    of several rounds); sequences sampled against the oracle, every output
    finite."""
    d, L = 128, 32768
    gen = torch.Generator().manual_seed(4242 + B)
    lens = [int(x) for x in torch.randint(1, L + 1, (B,), generator=gen)]
    lens[0], lens[-1] = L, L
    w = wl.Workload("largest", B, H, G, d, L, dtype, 77)
    want_kind = 0 if G == 16 else 1
    assert gqa.decode_kernel_kind(B, H, G, d, L, gqa.GQA_F32 if dtype == "f32" else gqa.GQA_BF16) == want_kind
    q, k, v, lt = wl.make_inputs(w, DEV, pad="none", seq_lens=torch.tensor(lens, dtype=torch.int32))
    out = run_gpu(q, k, v, lt, w.scale)
    assert torch.isfinite(out).all()
    rows = [0, 1, B // 2, B - 1]
    check(out.cpu()[rows], oracle_out(q, k, v, lt, w.scale, rows=rows), dtype, "largest caches %s B%d" % (dtype, B))
    del q, k, v, out
    torch.cuda.empty_cache()


def test_ragged_workload(env):
    """Ragged long-context workload at full size (B64 H64 G8 d128, lengths
    uniform in 1..32768 over a 32768-position padded cache): every one of the
    64 sequences against the oracle, each over its valid prefix (the oracle
    reads only the attended positions, ~34 GFLOP in binary64)."""
    w = wl.RAGGED
    q, k, v, lens = wl.make_inputs(w, DEV)
    out = run_gpu(q, k, v, lens, w.scale)
    ref = oracle_out(q, k, v, lens, w.scale, rows=list(range(w.B)))
    check(out, ref, w.dtype, w.name + " all sequences")
    lc = lens.cpu()
    for b in (int(lc.argmin()), int(lc.argmax())):  # shortest and longest on their own relative bar
        check_relative(out.cpu()[b:b + 1], ref[b:b + 1], "%s sequence %d (len %d)" % (w.name, b, int(lc[b])))


# --------------------------------------------------------------- mean-pool conversion

@pytest.mark.parametrize("shape", [(4096, 32, 8, 128), (512, 12, 4, 64), (256, 8, 8, 128), (300, 8, 1, 96),
                                   (1, 3, 1, 1)])
def test_meanpool_bit_exact(shape):
    d_model, H, G, h = shape
    gen = torch.Generator("cpu").manual_seed(d_model + H)
    w = torch.randn((d_model, H * h), generator=gen) * torch.exp(torch.randn((d_model, H * h), generator=gen) * 3)
    w[0, :min(4, H * h)] = -0.0
    got = gqa.meanpool_kv(w.to(DEV), H, G).cpu()
    torch.cuda.synchronize()
    ref = oracle.meanpool(w.numpy(), H, G)
    assert np.array_equal(got.numpy().view(np.uint32), ref.view(np.uint32))


# --------------------------------------------------------------- seeded random configurations

def _random_cases(n, seed):
    """Small random shapes across the plan space: group ratios 1..64 (head
    splits, padded head blocks), lengths that are not multiples of 32 (tails,
    empty sequences), windows, the cache append, both dtypes."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(n):
        d = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 3, 4, 8]))
        r = int(rng.choice([1, 2, 3, 4, 5, 7, 8, 12, 16, 24, 40, 48, 64]))
        B = int(rng.integers(1, 6))
        Lmax = int(rng.integers(1, 1400))
        lens = [int(x) for x in rng.integers(0, Lmax + 1, size=B)]
        lens[0] = Lmax  # one full sequence
        dtype = "bf16" if rng.random() < 0.75 else "f32"
        window = int(rng.integers(1, Lmax + 40)) if rng.random() < 0.3 else 0
        append = bool(rng.random() < 0.3)
        merge = "kernel" if rng.random() < 0.2 else None
        cases.append((i, B, G * r, G, d, Lmax, lens, dtype, window, append, merge))
    return cases


@pytest.mark.parametrize("case", _random_cases(48, 2026), ids=lambda c: "rand%02d" % c[0])
def test_random_configurations(env, case):
    i, B, H, G, d, Lmax, lens, dtype, window, append, merge = case
    env(GQA_MERGE=merge)
    q, k, v, lt, scale = rand_case(B, H, G, d, Lmax, lens, dtype, seed=5000 + i)
    what = "rand%02d B%d H%d G%d d%d L%d %s W%d append=%s merge=%s" % (i, B, H, G, d, Lmax, dtype, window, append,
                                                                       merge)
    if append:
        gen = torch.Generator(DEV).manual_seed(6000 + i)
        kn = torch.randn((B, G, d), generator=gen, device=DEV).to(k.dtype)
        vn = torch.randn((B, G, d), generator=gen, device=DEV).to(k.dtype)
        k0, v0 = k.cpu(), v.cpu()
        out = gqa.decode_append(q, kn, vn, k, v, lt, scale, window=window)
        torch.cuda.synchronize()
        ref, rk, rv = oracle.decode_append(q.cpu(), kn.cpu(), vn.cpu(), k0, v0, lt.cpu(), scale, window=window)
        check(out, ref, dtype, what)
        bits = torch.int16 if dtype == "bf16" else torch.int32
        nbits = np.uint16 if dtype == "bf16" else np.uint32
        assert np.array_equal(k.cpu().view(bits).numpy().view(nbits), rk.view(nbits)), what
        assert np.array_equal(v.cpu().view(bits).numpy().view(nbits), rv.view(nbits)), what
    elif window:
        out = gqa.decode_window(q, k, v, lt, scale, window)
        torch.cuda.synchronize()
        check(out, oracle.decode(q.cpu(), k.cpu(), v.cpu(), lt.cpu(), scale, window=window), dtype, what)
    else:
        out = run_gpu(q, k, v, lt, scale)
        check(out, oracle_out(q, k, v, lt, scale), dtype, what)


def _random_plans(n, seed, binary32=False, first=0):
    """Random shapes as above, each with random plan settings: split length
    (down to one tile, so up to ~250 splits), dispatch order forced on, the
    wide merge forced, plain or non-temporal cache loads, head split; larger
    batches, so that some grids exceed 1024 workgroups.  binary32: every case
    in binary32, with the kernel drawn too (the plan's, or either forced)."""
    rng = np.random.default_rng(seed)
    cases = []
    for i in range(first, first + n):
        d = int(rng.choice([64, 128]))
        G = int(rng.choice([1, 2, 4, 8]))
        r = int(rng.choice([1, 2, 3, 4, 8, 16, 24, 64]))
        B = int(rng.integers(1, 40))
        Lmax = int(rng.integers(1, 8000))
        lens = [int(x) for x in rng.integers(0, Lmax + 1, size=B)]
        lens[0] = Lmax
        dtype = "f32" if binary32 or rng.random() >= 0.8 else "bf16"
        window = int(rng.integers(1, Lmax + 40)) if rng.random() < 0.25 else 0
        append = bool(rng.random() < 0.25)
        plan = {
            "GQA_CHUNK": int(rng.choice([32, 64, 96, 256, 512, 1000])) if rng.random() < 0.7 else None,
            "GQA_ORDER": int(rng.choice([0, 1])) if rng.random() < 0.6 else None,
            "GQA_FUSED_MAX_SPLITS": int(rng.choice([1, 4, 64])) if rng.random() < 0.3 else None,
            "GQA_TEMPORAL": int(rng.choice([0, 1])) if rng.random() < 0.3 else None,
            "GQA_HEAD_SPLIT": int(rng.choice([1, 2, 4])) if rng.random() < 0.2 else None,
            "GQA_MERGE": "kernel" if rng.random() < 0.15 else None,
        }
        if binary32:
            plan["GQA_KERNEL"] = [None, "mfma", "valu"][int(rng.integers(0, 3))]
        cases.append((i, B, G * r, G, d, Lmax, lens, dtype, window, append, plan))
    return cases


@pytest.mark.parametrize("case", _random_plans(48, 4242) + _random_plans(24, 5151, binary32=True, first=100),
                         ids=lambda c: "plan%02d" % c[0] if c[0] < 100 else "f32plan%02d" % (c[0] - 100))
def test_random_plans(env, case):
    i, B, H, G, d, Lmax, lens, dtype, window, append, plan = case
    env(**plan)
    q, k, v, lt, scale = rand_case(B, H, G, d, Lmax, lens, dtype, seed=7000 + i)
    what = "plan%02d B%d H%d G%d d%d L%d %s W%d append=%s %s" % (i, B, H, G, d, Lmax, dtype, window, append,
                                                               {k_: v_ for k_, v_ in plan.items() if v_ is not None})
    rows = list(range(min(B, 6)))  # the oracle on a few sequences keeps the test fast
    if append:
        gen = torch.Generator(DEV).manual_seed(8000 + i)
        kn = torch.randn((B, G, d), generator=gen, device=DEV).to(k.dtype)
        vn = torch.randn((B, G, d), generator=gen, device=DEV).to(k.dtype)
        k0, v0 = k[:len(rows)].cpu(), v[:len(rows)].cpu()
        out = gqa.decode_append(q, kn, vn, k, v, lt, scale, window=window)
        torch.cuda.synchronize()
        ref, rk, rv = oracle.decode_append(q[:len(rows)].cpu(), kn[:len(rows)].cpu(), vn[:len(rows)].cpu(), k0, v0,
                                           lt[:len(rows)].cpu(), scale, window=window)
        check(out[:len(rows)], ref, dtype, what)
        bits = torch.int16 if dtype == "bf16" else torch.int32
        nbits = np.uint16 if dtype == "bf16" else np.uint32
        assert np.array_equal(k[:len(rows)].cpu().view(bits).numpy().view(nbits), rk.view(nbits)), what
        assert np.array_equal(v[:len(rows)].cpu().view(bits).numpy().view(nbits), rv.view(nbits)), what
    else:
        out = gqa.decode_window(q, k, v, lt, scale, window) if window else gqa.decode(q, k, v, lt, scale)
        torch.cuda.synchronize()
        ref = oracle.decode(q[:len(rows)].cpu(), k[:len(rows)].cpu(), v[:len(rows)].cpu(), lt[:len(rows)].cpu(),
                            scale, window=window)
        check(out[:len(rows)], ref, dtype, what)

