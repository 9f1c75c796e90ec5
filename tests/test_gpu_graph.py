"""The decode entry points captured into a HIP graph (through torch's graph
capture), as a serving loop would: no allocation, no memset and no host
synchronisation inside the calls, and the arrival counters are left at zero
by every launch, so a captured call can be replayed.  Each test replays the
graph several times with new inputs written between replays (ordinary eager
work and synchronisations in between) and checks every replay bit for bit
against the same call made eagerly."""
import pytest
import torch

import grouped_query_kv_decode_amd as gqa
from grouped_query_kv_decode_amd import workloads as wl

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    gqa.load_library()
    yield


def new_ws(nbytes):
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    gqa.workspace_init(ws)
    return ws


def inputs(B, H, G, d, L, lens, seed):
    w = wl.Workload("graph", B, H, G, d, L, "bf16", seed)
    q, k, v, _ = wl.make_inputs(w, DEV, pad="zero", seq_lens=torch.tensor(lens, dtype=torch.int32))
    return q, k, v, torch.tensor(lens, dtype=torch.int32, device=DEV), w.scale


@pytest.mark.parametrize("shape", [(4, 32, 8, 128, 3000, [3000, 2047, 1, 1500]), (2, 64, 1, 64, 1200, [1200, 700])],
                         ids=["split_merge", "head_split"])
def test_decode_graph_replays(shape):
    B, H, G, d, L, lens = shape
    q, k, v, lt, scale = inputs(B, H, G, d, L, lens, seed=31)
    need = gqa.decode_workspace_size(B, H, G, d, L, torch.bfloat16)
    ws_graph, ws_eager = new_ws(need), new_ws(need)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.decode(q, k, v, lt, scale, out=out, workspace=ws_graph)
    gen = torch.Generator(DEV).manual_seed(5)
    for rep in range(5):
        q.copy_(torch.randn(q.shape, generator=gen, device=DEV).to(q.dtype))
        g.replay()
        torch.cuda.synchronize()
        ref = gqa.decode(q, k, v, lt, scale, workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep


def test_append_graph_replays():
    """Captured decode with the cache append: every replay writes row
    len-1 of the caches from the (new) k_new / v_new and attends; the eager
    call on copies of the caches gives the same output and caches."""
    B, H, G, d, L = 3, 32, 8, 128, 2500
    lens = [2500, 1200, 3]
    q, k, v, lt, scale = inputs(B, H, G, d, L, lens, seed=41)
    kn = torch.zeros((B, G, d), dtype=torch.bfloat16, device=DEV)
    vn = torch.zeros_like(kn)
    need = gqa.decode_workspace_size(B, H, G, d, L, torch.bfloat16)
    ws_graph, ws_eager = new_ws(need), new_ws(need)
    out = torch.empty_like(q)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        gqa.decode_append(q, kn, vn, k, v, lt, scale, out=out, workspace=ws_graph)
    gen = torch.Generator(DEV).manual_seed(6)
    for rep in range(4):
        kn.copy_(torch.randn(kn.shape, generator=gen, device=DEV).to(kn.dtype))
        vn.copy_(torch.randn(vn.shape, generator=gen, device=DEV).to(vn.dtype))
        k2, v2 = k.clone(), v.clone()
        g.replay()
        torch.cuda.synchronize()
        ref = gqa.decode_append(q, kn, vn, k2, v2, lt, scale, workspace=ws_eager)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), rep
        assert torch.equal(k.view(torch.int16), k2.view(torch.int16)), rep
        assert torch.equal(v.view(torch.int16), v2.view(torch.int16)), rep


def test_layer_step_graph_replays():
    """The three-kernel decode step (packed projections, append + attention)
    captured once and replayed for consecutive tokens."""
    B, H, G, d, L, d_model = 4, 16, 4, 128, 512, 2048
    lens = [300, 512, 17, 100]
    q, k, v, lt, scale = inputs(B, H, G, d, L, lens, seed=51)
    gen = torch.Generator(DEV).manual_seed(7)
    x = torch.randn((B, d_model), generator=gen, device=DEV).to(torch.bfloat16)
    w_qkv = (torch.randn((d_model, (H + 2 * G) * d), generator=gen, device=DEV) * d_model ** -0.5).to(torch.bfloat16)
    w_o = (torch.randn((H * d, d_model), generator=gen, device=DEV) * (H * d) ** -0.5).to(torch.bfloat16)
    need = gqa.decode_layer_workspace_size(B, H, G, d, L, 0, d_model, torch.bfloat16)
    k2, v2 = k.clone(), v.clone()
    step_graph = gqa.LayerStep(x, w_qkv, w_o, k, v, lt, H, G, scale, workspace=new_ws(need))
    lt2 = lt.clone()
    step_eager = gqa.LayerStep(x, w_qkv, w_o, k2, v2, lt2, H, G, scale, workspace=new_ws(need))
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step_graph()
    for rep in range(4):
        x.copy_(torch.randn(x.shape, generator=gen, device=DEV).to(x.dtype))
        g.replay()
        torch.cuda.synchronize()
        y_ref = step_eager()
        torch.cuda.synchronize()
        assert torch.equal(step_graph.out, y_ref), rep
        assert torch.equal(k.view(torch.int16), k2.view(torch.int16)), rep
        lt += 1   # the next token of every sequence
        lt2 += 1
