"""The C ABI without a GPU: the library loads, exports what the headers under
include/ declare, and rejects bad arguments on the host before any HIP call."""
import ctypes
import glob
import os
import re

import pytest

import grouped_query_kv_decode_amd as gqa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))

OK, NULL, SHAPE, UNSUP, ALIGN, WS, SCALE, HIP, SIZE = range(9)
F32, BF16 = 0, 1
P = 0x10000  # a 256-byte aligned dummy address; never dereferenced on these paths


@pytest.fixture(scope="module")
def lib():
    return gqa.load_library()


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names.update(re.findall(r"\b(gqa_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


def test_headers_present():
    assert [os.path.basename(h) for h in HEADERS] == ["gqa.h", "gqa_measure.h"]


C_CLIENT = r"""
#include <stdio.h>
#include "gqa.h"
#include "gqa_measure.h"
int main(void) {
  size_t ws = gqa_decode_workspace_size(16, 32, 8, 128, 4096, GQA_BF16);
  gqa_status empty = gqa_decode(NULL, NULL, NULL, NULL, 0, 32, 8, 128, 4096, 0.088f, GQA_BF16, NULL, NULL, 0, NULL);
  gqa_status bad = gqa_decode(NULL, NULL, NULL, NULL, 1, 32, 6, 128, 4096, 0.088f, GQA_BF16, NULL, NULL, 0, NULL);
  printf("%zu %d %d %d %d\n", ws, (int)empty, (int)bad, gqa_decode_kernel_kind(16, 32, 8, 128, 4096, GQA_F32),
         (int)(GQA_NOALLOC_SCRATCH_BYTES >> 20));
  return 0;
}
"""


@pytest.mark.parametrize("compiler,std", [("gcc", "-std=c11"), ("g++", "-std=c++17")])
def test_headers_serve_a_plain_c_client(tmp_path, compiler, std):
    """Both headers compile as strict C11 (and as C++17) with every warning
    an error, and a client links libgqa.so and calls it through them (host
    paths only: sizing, an empty batch, a rejected shape, the kernel choice)."""
    import shutil
    import subprocess
    if shutil.which(compiler) is None:
        pytest.skip(compiler + " not installed")
    src = tmp_path / ("client.c" if compiler == "gcc" else "client.cpp")
    src.write_text(C_CLIENT)
    exe = tmp_path / "client"
    pkg = os.path.dirname(gqa.library_path())
    cmd = [compiler, std, "-Wall", "-Wextra", "-Werror", "-pedantic", "-D__HIP_PLATFORM_AMD__",
           "-isystem", "/opt/rocm/include", "-I" + os.path.join(ROOT, "include"), str(src),
           "-L" + pkg, "-lgqa", "-Wl,-rpath," + pkg, "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stderr
    out = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert out.returncode == 0, out.stderr
    ws, empty, bad, kind, scratch_mib = (int(x) for x in out.stdout.split())
    assert ws == _decode_ws(16, 32, 2, 128)  # the Mistral-7B shape's plan: 2 splits
    assert (empty, bad, kind, scratch_mib) == (OK, SHAPE, 1, 32)


def test_header_declares_the_binding_list():
    assert declared_functions() == sorted(gqa.EXPORTED)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for s in range(9):
        txt = gqa.status_string(s)
        assert txt and txt != "unknown status"
    assert gqa.status_string(99) == "unknown status"


def decode(lib, q=P, k=P, v=P, lens=P, B=2, H=8, G=2, d=128, L=512, scale=0.125, dt=BF16, out=P, ws=P,
           ws_bytes=1 << 30):
    return lib.gqa_decode(q, k, v, lens, B, H, G, d, L, scale, dt, out, ws, ws_bytes, None)


def test_shape_errors(lib):
    assert decode(lib, H=6, G=4) == SHAPE
    assert decode(lib, B=-1) == SHAPE
    assert decode(lib, H=0) == SHAPE
    assert decode(lib, G=0) == SHAPE
    assert decode(lib, L=0) == SHAPE
    assert decode(lib, d=0) == SHAPE


def test_unsupported(lib):
    assert decode(lib, d=96) == UNSUP
    assert decode(lib, d=256) == UNSUP
    assert decode(lib, dt=7) == UNSUP


def test_empty_batch_is_a_noop(lib):
    assert decode(lib, B=0, q=None, k=None, v=None, lens=None, out=None, ws=None, ws_bytes=0) == OK


def test_null_pointers(lib):
    for kw in ("q", "k", "v", "lens", "out"):
        assert decode(lib, **{kw: None}) == NULL, kw


def test_alignment(lib):
    for kw in ("q", "k", "v", "out"):
        assert decode(lib, **{kw: P + 8}) == ALIGN, kw
    assert decode(lib, lens=P + 2) == ALIGN


def test_scale(lib):
    assert decode(lib, scale=float("nan")) == SCALE
    assert decode(lib, scale=float("inf")) == SCALE
    assert decode(lib, scale=3e38) == SCALE  # scale * log2(e) overflows binary32


def test_workspace_checks(lib, monkeypatch):
    monkeypatch.setenv("GQA_CHUNK", "128")
    need = lib.gqa_decode_workspace_size(2, 8, 2, 128, 512, BF16)
    assert need > 0
    assert decode(lib, ws_bytes=need - 1) == WS
    assert decode(lib, ws=None, ws_bytes=need) == NULL
    assert decode(lib, ws=P + 16, ws_bytes=need) == ALIGN


def test_workspace_size_model(lib, monkeypatch):
    B, H, G, d, L = 2, 8, 2, 128, 512
    monkeypatch.setenv("GQA_CHUNK", "128")
    S = 4
    need = lib.gqa_decode_workspace_size(B, H, G, d, L, BF16)
    # 256 KiB of arrival counters, (max, sum) pairs, then partial outputs
    ml = (B * H * S * 8 + 255) // 256 * 256
    assert need == 256 * 1024 + ml + B * H * S * d * 4
    monkeypatch.setenv("GQA_CHUNK", str(L))
    assert lib.gqa_decode_workspace_size(B, H, G, d, L, BF16) == 0  # one split: no workspace
    assert lib.gqa_decode_workspace_size(B, 6, 4, d, L, BF16) == 0  # rejected shape


def _decode_ws(B, H, S, d, grid=0):
    """Counters, split (max, sum) pairs, split outputs; for grids of more than
    1024 workgroups with at least 4 splits also the dispatch order, one int
    each (pass grid for those)."""
    up = lambda x: (x + 255) // 256 * 256
    if grid > 1024:
        return 256 * 1024 + up(B * H * S * 8) + up(B * H * S * d * 4) + grid * 4
    return 256 * 1024 + up(B * H * S * 8) + B * H * S * d * 4


def test_split_plan_model(lib, monkeypatch):
    """Split lengths: about 256 workgroups (on the matrix cores the count
    that fills whole rounds of 256 best), at least 256 positions on the
    bfloat16 matrix-core kernel (64 on the binary32 one, 32 on the VALU
    kernel), at least Lmax/256, at most 8192 on the matrix cores and 4096 on
    the VALU kernel."""
    for k in ("GQA_CHUNK", "GQA_TARGET_WGS", "GQA_MAX_CHUNK", "GQA_KERNEL", "GQA_HEAD_SPLIT", "GQA_MERGE", "GQA_ORDER",
              "GQA_FUSED_MAX_SPLITS"):
        monkeypatch.delenv(k, raising=False)
    cases = [
        # (B, H, G, d, L, dtype, splits)
        (16, 32, 8, 128, 4096, BF16, 2),      # 128 units: 2048-position splits
        (1, 32, 8, 128, 4096, BF16, 16),      # 8 units: 256-position floor
        (4, 32, 8, 128, 4096, BF16, 8),       # 32 units: 512
        (1, 32, 8, 128, 32768, BF16, 32),     # 8 units, long: 1024 (256 WGs)
        (64, 64, 8, 128, 32768, BF16, 4, 2048),  # 512 units: 8192 cap; 2048 workgroups, ordered
        (64, 64, 8, 128, 32768, F32, 4, 2048),   # binary32 r = 8, matrix cores: 8192 cap; ordered
        (8, 32, 16, 128, 8192, BF16, 2),      # 128 units: 4096
        # binary32 on the matrix cores, grids of one round: 64-position floor,
        # the target's split count halved while the estimate falls
        (1, 8, 2, 64, 256, F32, 4),           # 2 units: 4 splits of 64
        (1, 8, 2, 64, 1024, F32, 16),         # 2 units: 16 splits of 64
        (1, 32, 8, 128, 512, F32, 8),         # 8 units: 8 splits of 64
        (2, 32, 8, 128, 1024, F32, 8),        # 16 units: 16 -> 8 splits of 128
        (4, 32, 8, 128, 1024, F32, 8),        # 32 units: 256 workgroups
        (1, 8, 2, 64, 8192, F32, 32),         # 2 units: 128 -> 32 splits (no wide merge)
        (16, 32, 8, 128, 4096, F32, 2),       # 128 units: 2048
        (1, 16, 16, 128, 1024, BF16, 8),      # r = 1 (VALU), 16 units: 16 -> 8 splits of 128
        (1, 8, 1, 128, 131072, BF16, 256),    # one unit, long: 512-position splits (256 WGs)
        (1, 8, 1, 128, 262144, F32, 256),     # at most 256 splits: 1024 positions
        # 64 heads per K/V head: 2 or 4 head chunks, whichever moves fewer
        # bytes through the busiest compute unit (slabs + merge)
        (32, 64, 1, 64, 2048, BF16, 4),       # 2 chunks: 64 units x 512 positions
        (64, 64, 1, 64, 4096, BF16, 2),       # 2 chunks (4 would read whole slabs: 1 split)
        (32, 128, 2, 128, 4096, BF16, 2),     # 2 chunks
        (4, 64, 1, 64, 8192, BF16, 16),       # 4 chunks (2 would merge 32 heads x 32 splits)
        (8, 64, 1, 128, 8192, BF16, 8),       # 4 chunks
        (2, 64, 1, 128, 32768, BF16, 64),     # 2 chunks, 64 splits for the wide merge
        # 17..32 heads per K/V head: 1 or 2 head chunks by the same estimate
        (16, 32, 1, 128, 4096, BF16, 8),      # 2 chunks (1 would merge 32 heads x 16 splits)
        (4, 32, 1, 128, 16384, BF16, 64),     # 1 chunk: 64 splits for the wide merge
        (32, 32, 1, 128, 8192, BF16, 8),      # 1 chunk
        (96, 32, 1, 128, 2048, BF16, 2),      # 1 chunk, 2 splits: 192 workgroups in one round
        # unit counts that do not divide 256: the split count that fills whole
        # rounds of 256 workgroups, not the one that just overfills the first
        (6, 32, 8, 128, 4096, BF16, 5),       # 48 units: 240 workgroups (6 splits: 288)
        (3, 32, 8, 128, 8192, BF16, 10),      # 24 units: 240 (11 splits: 264)
        (12, 32, 8, 128, 4096, BF16, 5),      # 96 units: 480, two full rounds (3 splits: 288)
        (20, 32, 8, 128, 4096, BF16, 3),      # 160 units: 480 (2 splits: 320)
        (48, 32, 8, 128, 2048, BF16, 2),      # 384 units: 768, three full rounds (1 split: 384)
    ]
    for B, H, G, d, L, dt, S, *grid in cases:
        assert lib.gqa_decode_workspace_size(B, H, G, d, L, dt) == _decode_ws(B, H, S, d, *grid), (B, H, G, d, L, dt, S)
    # binary32 on the VALU kernel (the default for r <= 2; forced here)
    valu_cases = [
        (64, 64, 8, 128, 32768, F32, 8, 4096),   # 4096 cap; 4096 workgroups, ordered
        # grids of one round: the target's split count halved while the
        # estimate falls (fewer splits where the merge costs more than it saves)
        (1, 8, 2, 64, 1024, F32, 8),          # 2 units: 32 -> 8 splits of 128
        (1, 32, 8, 128, 512, F32, 8),         # 8 units: 16 -> 8 splits of 64
        (2, 8, 2, 128, 2048, F32, 64),        # 4 units: keeps 64 splits of 32 (wide merge)
        # 4 heads per row set: 512 workgroups where the units divide 512,
        # else 768; 8 heads per row set: 768
        (4, 32, 8, 128, 8192, F32, 16),       # 32 units: 512 workgroups
        (16, 32, 8, 128, 4096, F32, 4),       # 128 units: 512
        (12, 32, 8, 128, 2048, F32, 8),       # 96 units do not divide 512: 768
        (2, 64, 8, 128, 8192, F32, 43),       # 8 heads per row set: 768 aimed at, 192-position splits
        (1, 8, 2, 64, 8192, F32, 256),        # 2 units of 4 heads: 768 workgroups aimed at, 32-position splits
    ]
    monkeypatch.setenv("GQA_KERNEL", "valu")
    for B, H, G, d, L, dt, S, *grid in valu_cases:
        assert lib.gqa_decode_workspace_size(B, H, G, d, L, dt) == _decode_ws(B, H, S, d, *grid), (B, H, G, d, L, dt, S)
    assert lib.gqa_decode_workspace_size(1, 8, 2, 64, 256, F32) == 0     # 8 -> 1 split by the estimate
    monkeypatch.delenv("GQA_KERNEL")
    monkeypatch.setenv("GQA_ORDER", "0")  # no dispatch order: no order region
    assert lib.gqa_decode_workspace_size(64, 64, 8, 128, 32768, BF16) == _decode_ws(64, 64, 4, 128)
    # one split: no workspace
    assert lib.gqa_decode_workspace_size(4, 32, 32, 64, 512, BF16) == 0  # VALU r = 1: 2 -> 1
    monkeypatch.setenv("GQA_TARGET_WGS", "256")  # a plain target: the floors, 64 and 32 positions
    assert lib.gqa_decode_workspace_size(1, 8, 2, 64, 256, F32) == _decode_ws(1, 8, 4, 64)
    monkeypatch.setenv("GQA_KERNEL", "valu")
    assert lib.gqa_decode_workspace_size(1, 8, 2, 64, 256, F32) == _decode_ws(1, 8, 8, 64)
    monkeypatch.delenv("GQA_KERNEL")
    monkeypatch.delenv("GQA_TARGET_WGS")
    assert lib.gqa_decode_workspace_size(32, 64, 8, 64, 2048, BF16) == 0
    assert lib.gqa_decode_workspace_size(128, 32, 1, 128, 1024, BF16) == 0  # 2 head chunks, one split each


def test_noalloc_limit(lib):
    """gqa_decode_noalloc: the binding's limit is the header's, and a shape
    whose plan needs more scratch than that is rejected on the host (before
    any HIP call, so this runs without a GPU) with GQA_ERR_WORKSPACE."""
    m = re.search(r"#define GQA_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADERS[0]).read())
    assert m and int(m.group(1)) << int(m.group(2)) == gqa.NOALLOC_SCRATCH_BYTES
    big = (64, 64, 8, 128, 131072)
    assert lib.gqa_decode_workspace_size(*big, BF16) > gqa.NOALLOC_SCRATCH_BYTES
    args = (P, P, P, P, *big, 0.088, BF16, P, None)
    assert lib.gqa_decode_noalloc(*args) == WS
    assert lib.gqa_decode_noalloc(P, P, P, P, 2, 6, 4, 128, 512, 0.088, BF16, P, None) == SHAPE
    assert lib.gqa_decode_noalloc(None, None, None, None, 0, 8, 2, 128, 512, 0.088, BF16, None, None) == OK


def test_plan_reads_the_environment_only_on_reload(lib, monkeypatch):
    """A call never reads the GQA_* overrides: changing the environment
    without gqa_tuning_reload() leaves the plan (and so the workspace size)
    as it was; the reload picks the change up."""
    B, H, G, d, L = 2, 8, 2, 128, 512
    monkeypatch.delenv("GQA_CHUNK", raising=False)  # (the test hook reloads)
    base = lib.gqa_decode_workspace_size(B, H, G, d, L, BF16)
    os.environ["GQA_CHUNK"] = "128"
    try:
        assert lib.gqa_decode_workspace_size(B, H, G, d, L, BF16) == base
        gqa.tuning_reload()
        assert lib.gqa_decode_workspace_size(B, H, G, d, L, BF16) == _decode_ws(B, H, 4, d) != base
    finally:
        del os.environ["GQA_CHUNK"]
        gqa.tuning_reload()
    assert lib.gqa_decode_workspace_size(B, H, G, d, L, BF16) == base


def test_plan_lookup_cost(lib):
    """Plans are cached per shape: 100,000 workspace-size queries of the
    named shapes cost about a microsecond each, nearly all of it the ctypes
    call (the lookup itself is ~20 ns in C; evaluating a plan took 0.4-0.8 us
    when every call read the environment)."""
    import time
    shapes = [(1, 8, 2, 64, 256, F32), (16, 32, 8, 128, 4096, BF16), (32, 64, 1, 64, 2048, BF16),
              (64, 64, 8, 128, 32768, BF16)]
    f = lib.gqa_decode_workspace_size
    for sh in shapes:
        f(*sh)
        t0 = time.perf_counter()
        for _ in range(100000):
            f(*sh)
        us = (time.perf_counter() - t0) * 10
        print("plan lookup %s: %.2f us per call (ctypes included)" % (sh, us))
        assert us < 5.0, sh


def test_kernel_selection(lib, monkeypatch):
    monkeypatch.delenv("GQA_KERNEL", raising=False)
    assert lib.gqa_decode_kernel_kind(16, 32, 8, 128, 4096, BF16) == 1
    assert lib.gqa_decode_kernel_kind(1, 8, 2, 64, 256, F32) == 1     # binary32, r = 4: matrix cores
    assert lib.gqa_decode_kernel_kind(8, 48, 4, 128, 4096, F32) == 1  # r = 12
    assert lib.gqa_decode_kernel_kind(8, 32, 16, 128, 8192, F32) == 0  # r = 2: the VALU kernel
    assert lib.gqa_decode_kernel_kind(20, 32, 16, 128, 4096, F32) == 1  # r = 2, 320 units: matrix cores
    assert lib.gqa_decode_kernel_kind(6, 32, 32, 128, 4096, F32) == 1   # r = 1, 192 units: matrix cores
    assert lib.gqa_decode_kernel_kind(16, 32, 32, 128, 1024, F32) == 0  # r = 1, 512 units: VALU
    assert lib.gqa_decode_kernel_kind(3, 8, 8, 64, 256, F32) == 0       # r = 1, 24 units but 3 MiB: VALU
    assert lib.gqa_decode_kernel_kind(8, 32, 32, 128, 4096, F32) == 0  # r = 1
    assert lib.gqa_decode_kernel_kind(1, 32, 1, 64, 256, F32) == 1     # r = 32: two head blocks
    assert lib.gqa_decode_kernel_kind(1, 128, 1, 64, 256, F32) == 0    # r = 128
    assert lib.gqa_decode_kernel_kind(1, 128, 1, 64, 256, BF16) == 0  # more than 64 heads per group
    assert lib.gqa_decode_kernel_kind(32, 64, 64, 64, 2048, BF16) == 1  # r = 1, 1 GiB of K and V: matrix cores
    assert lib.gqa_decode_kernel_kind(2, 8, 8, 128, 4096, BF16) == 1    # r = 1, 32 MiB
    assert lib.gqa_decode_kernel_kind(4, 32, 32, 64, 512, BF16) == 0    # r = 1, 16 MiB: the VALU kernel
    assert lib.gqa_decode_kernel_kind(2, 8, 8, 128, 4095, BF16) == 0    # just under 32 MiB
    assert lib.gqa_decode_kernel_kind(1, 6, 4, 64, 256, BF16) == -1
    monkeypatch.setenv("GQA_KERNEL", "valu")
    assert lib.gqa_decode_kernel_kind(16, 32, 8, 128, 4096, BF16) == 0
    monkeypatch.setenv("GQA_KERNEL", "mfma")
    assert lib.gqa_decode_kernel_kind(4, 32, 32, 64, 512, BF16) == 1
    assert lib.gqa_decode_kernel_kind(8, 32, 16, 128, 8192, F32) == 1  # forced: binary32 at r = 2
    assert lib.gqa_decode_kernel_kind(1, 64, 1, 64, 256, F32) == 1     # r = 64: four head chunks


def test_plan_invariants_random_shapes(lib, monkeypatch):
    """2000 seeded random shapes through the host plan, both dtypes: the
    kernel follows the documented rule (bf16: matrix cores for r = 2..64 and
    for MHA calls of at least 32 MiB; binary32: matrix cores for r = 3..64,
    and for r <= 2 on calls of at least 32 MiB whose B*G units neither divide
    nor are a multiple of 256),
    and the workspace is zero or exactly that of one split count S (at most
    256 splits, or Lmax over the split cap where that is more), with an order
    region of one int per workgroup for ordered grids."""
    import numpy as np
    for k in ("GQA_CHUNK", "GQA_TARGET_WGS", "GQA_MAX_CHUNK", "GQA_KERNEL", "GQA_HEAD_SPLIT", "GQA_MERGE", "GQA_ORDER",
              "GQA_FUSED_MAX_SPLITS", "GQA_WAVES"):
        monkeypatch.delenv(k, raising=False)
    up = lambda x: (x + 255) // 256 * 256
    rng = np.random.default_rng(99)
    for _ in range(2000):
        G = int(rng.choice([1, 2, 3, 4, 8, 16, 32]))
        r = int(rng.choice([1, 2, 3, 4, 5, 8, 12, 16, 24, 32, 48, 64, 96, 128]))
        B = int(rng.integers(1, 300))
        d = int(rng.choice([64, 128]))
        L = int(rng.choice([1, 7, 33, 256, 1000, 4096, 8192, 32768, 131072, 1 << 21]))
        dt = int(rng.choice([F32, BF16]))
        H = G * r
        kind = lib.gqa_decode_kernel_kind(B, H, G, d, L, dt)
        big_mha = 4.0 * B * G * L * d >= 32 * 1024 * 1024
        uneven = (B * G) % 256 != 0 and 256 % (B * G) != 0
        f32_mfma = 3 <= r <= 64 or (r <= 2 and uneven and 8.0 * B * G * L * d >= 32 * 1024 * 1024)
        want = (1 if (2 <= r <= 64 or (r == 1 and big_mha)) else 0) if dt == BF16 else (1 if f32_mfma else 0)
        assert kind == want, (B, H, G, d, L, dt)
        ws = lib.gqa_decode_workspace_size(B, H, G, d, L, dt)
        if ws == 0:
            continue
        cap = 8192 if kind == 1 else 4096
        s_max = max(256, -(-L // cap))
        est = (ws - 256 * 1024) // (B * H * (8 + 4 * d))
        found = None
        # the order region (one int per workgroup, <= 16 head chunks) adds at most a quarter to est
        for S in range(max(2, est * 3 // 4 - 2), min(s_max, est + 2) + 1):
            body = 256 * 1024 + up(B * H * S * 8) + B * H * S * d * 4
            if ws == body:
                found = S
                break
            extra = ws - (256 * 1024 + up(B * H * S * 8) + up(B * H * S * d * 4))
            if extra > 0 and extra % (4 * B * G * S) == 0 and extra // (4 * B * G * S) <= 16:  # head chunks <= 16
                found = S
                break
        assert found is not None, (B, H, G, d, L, dt, ws)
        assert 2 <= found <= s_max, (B, H, G, d, L, dt, found)


def test_meanpool_argument_errors(lib):
    mp = lib.gqa_meanpool_kv
    assert mp(P, 16, 6, 4, 8, P, None) == SHAPE
    assert mp(P, -1, 8, 2, 8, P, None) == SHAPE
    assert mp(P, 16, 8, 2, 0, P, None) == UNSUP
    assert mp(None, 0, 8, 2, 8, None, None) == OK
    assert mp(None, 16, 8, 2, 8, P, None) == NULL
    assert mp(P, 16, 8, 2, 8, None, None) == NULL
    assert mp(P + 2, 16, 8, 2, 8, P, None) == ALIGN


def test_workspace_init_arguments(lib):
    assert lib.gqa_workspace_init(None, 0, None) == OK
    assert lib.gqa_workspace_init(None, 64, None) == NULL


def test_stream_read_arguments(lib):
    """The read-ceiling probe's host checks (nothing is launched)."""
    sr = lib.gqa_stream_read
    assert sr(P, 0, 1, 0, P, None) == OK          # no bytes: no-op
    assert sr(None, 64, 1, 0, P, None) == NULL
    assert sr(P, 64, 1, 0, None, None) == NULL
    assert sr(P + 8, 64, 1, 0, P, None) == ALIGN  # buffer not 16-byte aligned
    assert sr(P, 72, 1, 0, P, None) == ALIGN      # size not a multiple of 16
    assert sr(P, 64, 1, -1, P, None) == SHAPE
    assert sr(P, 64, 1, (1 << 20) + 1, P, None) == SHAPE


def test_phase_argument(lib):
    args = (P, P, P, P, 2, 8, 2, 128, 512, 0.125, BF16, P, P, 1 << 30, None)
    assert lib.gqa_decode_phase(3, *args) == UNSUP
    assert lib.gqa_decode_phase(-1, *args) == UNSUP
    assert lib.gqa_decode_phase(1, P, P, P, P, 2, 6, 4, 128, 512, 0.125, BF16, P, P, 0, None) == SHAPE
    assert lib.gqa_decode_phase(2, None, None, None, None, 0, 8, 2, 128, 512, 0.125, BF16, None, None, 0, None) == OK


def test_window_and_append_arguments(lib):
    win = lambda W, **kw: lib.gqa_decode_window(kw.get("q", P), P, P, P, kw.get("B", 2), kw.get("H", 8), 2, 128,
                                                512, W, 0.125, BF16, P, P, 1 << 30, None)
    assert win(0) == SHAPE
    assert win(-3) == SHAPE
    assert win(5, H=7) == SHAPE
    assert win(5, B=0, q=None) == OK
    assert win(5, q=None) == NULL
    app = lambda kn=P, vn=P, W=0, B=2, H=8: lib.gqa_decode_append(P, kn, vn, P, P, P, B, H, 2, 128, 512, W, 0.125,
                                                                  BF16, P, P, 1 << 30, None)
    assert app(kn=None) == NULL
    assert app(vn=None) == NULL
    assert app(kn=P + 8) == ALIGN
    assert app(W=-1) == SHAPE
    assert app(H=7) == SHAPE
    assert app(kn=None, vn=None, B=0) == OK


def _linear_ws(M, K, N):
    """Workspace model of gqa_linear: 128-column blocks, k split in whole
    32-row steps into the largest power of two of parts that keeps the grid
    within 256 workgroups and at least two steps per wave of 4."""
    ntile, ksteps = N // 128, K // 32
    ks = 1
    while 2 * ks * ntile <= 256 and 2 * ks <= ksteps // 8:
        ks *= 2
    per = -(-ksteps // ks)
    ks = -(-ksteps // per)
    return 0 if ks == 1 else 256 * 1024 + ks * M * N * 4


def test_linear_arguments(lib):
    lin = lambda x=P, w=P, y=P, M=4, K=256, N=256, dt=BF16, ws=None, nb=0: lib.gqa_linear(x, w, y, M, K, N, dt, ws,
                                                                                          nb, None)
    assert lin(dt=F32) == UNSUP
    assert lin(M=65) == UNSUP
    assert lin(K=48) == UNSUP
    assert lin(N=200) == UNSUP
    assert lin(M=-1) == SHAPE
    assert lin(K=0) == SHAPE
    assert lin(N=0) == SHAPE
    assert lin(M=0, x=None, w=None, y=None) == OK
    assert lin(x=None) == NULL
    assert lin(y=P + 2) == ALIGN
    # k split (K = 4096 over 2 column blocks): the workspace is required
    assert lin(M=4, K=4096, N=256, ws=None) == NULL
    assert lin(M=4, K=4096, N=256, ws=P, nb=_linear_ws(4, 4096, 256) - 1) == WS
    assert lin(M=4, K=4096, N=256, ws=P + 64, nb=1 << 30) == ALIGN


def test_linear_workspace_model(lib):
    for M, K, N in [(16, 4096, 6144), (16, 4096, 4096), (1, 256, 128), (64, 8192, 1024), (3, 64, 128 * 600),
                    (8, 96, 128)]:
        assert lib.gqa_linear_workspace_size(M, K, N, BF16) == _linear_ws(M, K, N), (M, K, N)
    assert lib.gqa_linear_workspace_size(16, 4096, 4096, F32) == 0
    assert lib.gqa_linear_workspace_size(0, 4096, 4096, BF16) == 0


def test_pack_and_linear_packed_arguments(lib):
    pack = lambda w=P, wp=P, K=64, N=32, dt=BF16: lib.gqa_pack_weight(w, wp, K, N, dt, None)
    assert pack(dt=F32) == UNSUP
    assert pack(K=48) == UNSUP
    assert pack(N=24) == UNSUP
    assert pack(K=0) == SHAPE
    assert pack(N=-16) == SHAPE
    assert pack(w=None) == NULL
    assert pack(wp=None) == NULL
    assert pack(w=P + 1) == ALIGN
    assert pack(wp=P + 8) == ALIGN
    lin = lambda x=P, wp=P, y=P, M=4, K=64, N=32, dt=BF16: lib.gqa_linear_packed(x, wp, y, M, K, N, dt, None)
    assert lin(dt=F32) == UNSUP
    assert lin(M=65) == UNSUP
    assert lin(K=40) == UNSUP
    assert lin(N=8) == UNSUP
    assert lin(M=-1) == SHAPE
    assert lin(M=0, x=None, wp=None, y=None) == OK
    assert lin(wp=None) == NULL
    assert lin(x=P + 2) == ALIGN
    assert lin(y=P + 8) == ALIGN


def test_decode_layer_arguments(lib):
    # Mistral-7B shape: d_model 4096, H 32, G 8, d 128
    need = lib.gqa_decode_layer_workspace_size(16, 32, 8, 128, 4096, 0, 4096, BF16)
    att = lib.gqa_decode_workspace_size(16, 32, 8, 128, 4096, BF16)
    scratch = max(att, 256 * 1024)  # the packed projections need no workspace; counters always reserved
    bufs = 2 * (16 * 32 * 128) * 2 + 2 * (16 * 8 * 128) * 2
    assert need == -(-scratch // 256) * 256 + bufs
    # a window short enough for one split: no attention scratch, but the
    # buffers still start after the 256 KiB counter region
    assert lib.gqa_decode_workspace_size(3, 8, 2, 128, 100, BF16) == 0
    assert lib.gqa_decode_layer_workspace_size(3, 8, 2, 128, 600, 100, 512, BF16) == \
        256 * 1024 + 2 * 256 * (-(-3 * 8 * 128 * 2 // 256)) + 2 * 256 * (-(-3 * 2 * 128 * 2 // 256))
    assert lib.gqa_decode_layer_workspace_size(16, 32, 8, 128, 4096, 0, 4096, F32) == 0
    assert lib.gqa_decode_layer_workspace_size(65, 32, 8, 128, 4096, 0, 4096, BF16) == 0
    assert lib.gqa_decode_layer_workspace_size(16, 32, 8, 128, 4096, 0, 4008, BF16) == 0

    def layer(x=P, w1=P, w2=P, B=2, H=8, G=2, d=128, W=0, dm=1024, dt=BF16, ws=P, nb=1 << 30):
        return lib.gqa_decode_layer(x, w1, w2, P, P, P, B, H, G, d, 512, W, dm, 0.125, dt, P, ws, nb, None)
    assert layer(dt=F32) == UNSUP
    assert layer(B=65) == UNSUP
    assert layer(dm=1000) == UNSUP
    assert layer(H=7) == SHAPE
    assert layer(W=-1) == SHAPE
    assert layer(dm=0) == SHAPE
    assert layer(H=1 << 24, G=1 << 22) == SIZE  # (H + 2G) d beyond the int range
    assert layer(B=0, x=None, ws=None) == OK
    assert layer(x=None) == NULL
    assert layer(ws=None) == NULL
    assert layer(w2=P + 4) == ALIGN
    assert layer(ws=P + 128) == ALIGN
    assert layer(nb=lib.gqa_decode_layer_workspace_size(2, 8, 2, 128, 512, 0, 1024, BF16) - 1) == WS


def test_binding_rejects_bad_tensors():
    import torch
    q = torch.zeros(2, 8, 64)
    k = torch.zeros(2, 2, 16, 64)
    with pytest.raises(ValueError):
        gqa.decode(q, k, k, torch.zeros(2, dtype=torch.int32), 0.1)  # CPU tensors
    with pytest.raises(TypeError):
        gqa.decode(q, k, k, torch.zeros(2, dtype=torch.int64), 0.1)
    with pytest.raises(ValueError):
        gqa.decode(q, k[:1], k[:1], torch.zeros(2, dtype=torch.int32), 0.1)


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(RuntimeError):
        gqa.load_library(str(tmp_path / "libgqa.so"))


def test_oracle_and_product_are_independent():
    """Neither side imports, includes or links the other."""
    pkg = os.path.join(ROOT, "grouped_query_kv_decode_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                text = open(os.path.join(dirpath, f)).read()
                assert not re.search(r"^\s*(import|from)\s+oracle\b", text, re.M), f
                assert "gqa_oracle" not in text, f
    for f in os.listdir(os.path.join(ROOT, "oracle")):
        if f.endswith((".py", ".c", ".h")):
            text = open(os.path.join(ROOT, "oracle", f)).read()
            assert "grouped_query_kv_decode_amd" not in text, f
            assert "gqa.h" not in text, f
