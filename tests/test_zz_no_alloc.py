"""gqa_decode_noalloc, the decode entry point that allocates nothing: its
split partials and arrival counters live in the library's per-device scratch
array.  Through the C ABI, two calls in a row (the second on a smaller input)
must give exactly what gqa_decode gives with a workspace - the same plan and
kernels - and so agree with the oracle to the decode tolerance."""
import numpy as np
import pytest
import torch

import grouped_query_kv_decode_amd as gqa
from grouped_query_kv_decode_amd import workloads as wl
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"
TOL = {"f32": 1e-5, "bf16": 2e-2}


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    gqa.load_library()
    yield


def _case(B, H, G, d, L, lens, dtype, seed):
    w = wl.Workload("noalloc", B, H, G, d, L, dtype, seed)
    q, k, v, _ = wl.make_inputs(w, DEV, pad="nan", seq_lens=torch.tensor(lens, dtype=torch.int32))
    return w, q, k, v, torch.tensor(lens, dtype=torch.int32, device=DEV)


def _noalloc(lib, w, q, k, v, lens, out):
    """One gqa_decode_noalloc call through the C ABI on torch's current stream."""
    code = gqa.GQA_F32 if w.dtype == "f32" else gqa.GQA_BF16
    st = lib.gqa_decode_noalloc(q.data_ptr(), k.data_ptr(), v.data_ptr(), lens.data_ptr(), w.B, w.H, w.G, w.d, w.Lmax,
                                w.scale, code, out.data_ptr(), torch.cuda.current_stream().cuda_stream)
    assert st == 0, gqa.status_string(st)


SEQUENCES = [
    # two calls in a row, the second on a smaller input
    [(16, 32, 8, 128, 4096, [4096, 1, 2049] + [4096 - 250 * i for i in range(13)], "bf16", 1),  # matrix cores, 2 splits
     (3, 8, 2, 64, 700, [700, 1, 333], "bf16", 2)],                                             # 3 splits
    [(2, 8, 1, 128, 40000, [40000, 9000], "bf16", 3),   # 157 splits: the wide merge kernel
     (1, 8, 2, 64, 1024, [1000], "f32", 4)],            # binary32 matrix cores, 16 splits
    [(4, 32, 16, 128, 3000, [3000, 17, 2999, 1500], "f32", 5),   # binary32 r = 2: the VALU kernel, split
     (2, 16, 4, 128, 900, [900, 450], "f32", 6)],                 # binary32 matrix cores, split
]


@pytest.mark.parametrize("seq", SEQUENCES, ids=["fused_merge", "wide_merge_then_f32", "f32_valu_then_mfma"])
def test_noalloc_matches_workspace_decode(seq):
    lib = gqa.load_library()
    for (B, H, G, d, L, lens, dtype, seed) in seq:
        w, q, k, v, lt = _case(B, H, G, d, L, lens, dtype, seed)
        need = gqa.decode_workspace_size(B, H, G, d, L, q.dtype)
        assert 0 < need <= gqa.NOALLOC_SCRATCH_BYTES
        ref = gqa.decode(q, k, v, lt, w.scale)
        out = torch.full_like(ref, float("nan"))
        _noalloc(lib, w, q, k, v, lt, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), "noalloc differs from gqa_decode (B%d H%d G%d d%d L%d %s)" % (B, H, G, d, L, dtype)
        got = out.float().cpu().double().numpy()
        want = oracle.decode(q.cpu(), k.cpu(), v.cpu(), lt.cpu(), w.scale)
        err = float(np.max(np.abs(got - want)))
        print("noalloc B%d H%d G%d d%d L%d %s: max|err| %.3g" % (B, H, G, d, L, dtype, err))
        assert err <= TOL[dtype]


def test_noalloc_binding_and_repeat():
    """The binding's decode_noalloc, call after call on one stream: bit-equal
    every time (the counters are left at zero by each call)."""
    w, q, k, v, lt = _case(4, 32, 8, 128, 3000, [3000, 17, 1500, 2999], "bf16", 5)
    ref = gqa.decode(q, k, v, lt, w.scale).clone()
    outs = [gqa.decode_noalloc(q, k, v, lt, w.scale).clone() for _ in range(20)]
    torch.cuda.synchronize()
    for o in outs:
        assert torch.equal(o, ref)


def test_noalloc_graph_replays():
    """The callers it is for capture it: after one eager call on the device
    (which sets the scratch up), gqa_decode_noalloc captured into a HIP graph
    and replayed five times with new queries written between replays, every
    replay bit-equal to gqa_decode with a workspace on the same inputs."""
    lib = gqa.load_library()
    w, q, k, v, lt = _case(4, 32, 8, 128, 3000, [3000, 2047, 1, 1500], "bf16", 6)
    out = torch.empty_like(q)
    _noalloc(lib, w, q, k, v, lt, out)  # set-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc(lib, w, q, k, v, lt, out)
    gen = torch.Generator(DEV).manual_seed(7)
    for rep in range(5):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        g.replay()
        torch.cuda.synchronize()
        ref = gqa.decode(q, k, v, lt, w.scale)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
