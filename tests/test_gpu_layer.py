"""Projections and the full decode step (HIP path through the C ABI) against
the CPU oracle, on the GPU.

gqa_linear: every output is one binary32 sum rounded once to bfloat16, so
    |gpu - oracle| <= 2^-8 |oracle| + 2^-16 sum_k |x_k w_kn|
(half an ulp of bfloat16 for the rounding, plus a generous bound on binary32
accumulation error; a wrong operand or index is off by O(|oracle|)).

gqa_linear_packed (weights in the packed layout of gqa_pack_weight): the
same bound.  gqa_pack_weight: bit-exact against the layout built by host
reshapes.

gqa_decode_layer: element-wise parity holds stage by stage - the one-call
step is bit-equal to the three public entry points called in turn, and each
of those is checked against the oracle on identical inputs (here and in
test_gpu_parity.py).  End to end against the oracle's step
(oracle.decode_layer, which rounds q, key, val and the attention output to
bfloat16 like the kernels do) the intermediates differ: where the binary32
and binary64 values straddle a bfloat16 rounding boundary they land one ulp
apart, which with a long cache (an attention output that averages thousands
of values) happens in a large share of the elements.  Those one-ulp
differences (2^-8 relative, random signs) add up in y = out @ Wo like a random
walk, about 2^-8 rms(y) per output, so each output row is checked against
    |gpu - oracle| <= 2^-8 |oracle| + 2^-5 rms(oracle row)
(eight times that estimate; a wrong column, segment or cache row is off by
O(rms)).
"""
import numpy as np
import pytest
import torch

import grouped_query_kv_decode_amd as gqa
from grouped_query_kv_decode_amd import workloads as wl
import oracle

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    gqa.load_library()
    yield


@pytest.fixture
def ksplit(monkeypatch):
    def set_(v):
        if v is None:
            monkeypatch.delenv("GQA_LINEAR_KSPLIT", raising=False)
        else:
            monkeypatch.setenv("GQA_LINEAR_KSPLIT", str(v))
    set_(None)
    return set_


def rand_bf16(shape, seed, std=1.0):
    gen = torch.Generator("cpu").manual_seed(seed)
    return (torch.randn(shape, generator=gen) * std).to(torch.bfloat16)


def check_linear(y, x, w, what):
    ref = oracle.matmul(x, w)
    mag = np.abs(x.float().double().numpy()) @ np.abs(w.float().double().numpy())
    got = y.float().cpu().double().numpy()
    err = np.abs(got - ref)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -16 * mag
    worst = float(np.max(err / bound)) if err.size else 0.0
    print("%s max|err| = %.3g, worst err/bound = %.3f" % (what, float(err.max()) if err.size else 0.0, worst))
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), "%s: err/bound %.3f" % (what, worst)


LINEAR_CASES = [
    # (M, K, N)
    (1, 32, 128),            # one k step, one column block
    (5, 96, 384),            # ragged tokens, three k steps
    (16, 4096, 6144),        # fused q/k/v projection, d_model 4096, H 32, G 8, d 128
    (16, 4096, 4096),        # output projection of the same layer
    (17, 1024, 256),         # two token tiles
    (33, 512, 640),          # three token tiles (rounded up to four)
    (64, 4096, 128),         # most tokens, one column block, k split
    (3, 8192, 1024),
]


@pytest.mark.parametrize("case", LINEAR_CASES, ids=lambda c: "M%d_K%d_N%d" % c)
@pytest.mark.parametrize("split", [None, 1])
def test_linear_parity(ksplit, case, split):
    M, K, N = case
    ksplit(split)
    x = rand_bf16((M, K), seed=M + K)
    w = rand_bf16((K, N), seed=N + 7, std=K ** -0.5)
    y = gqa.linear(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    check_linear(y, x, w, "linear M%d K%d N%d split=%s" % (M, K, N, split))


@pytest.mark.parametrize("split", [2, 3, 7, 64, 128])
def test_linear_forced_splits(ksplit, split):
    """Uneven and extreme k splits (the last split shorter, one step per split)."""
    ksplit(split)
    M, K, N = 9, 4096, 256
    x = rand_bf16((M, K), seed=11)
    w = rand_bf16((K, N), seed=12, std=K ** -0.5)
    y = gqa.linear(x.to(DEV), w.to(DEV))
    torch.cuda.synchronize()
    check_linear(y, x, w, "linear split=%d" % split)


def test_linear_deterministic_and_workspace_reuse(ksplit):
    M, K, N = 16, 4096, 6144
    x = rand_bf16((M, K), seed=21).to(DEV)
    w = rand_bf16((K, N), seed=22, std=K ** -0.5).to(DEV)
    ws = torch.empty(gqa.linear_workspace_size(M, K, N, torch.bfloat16), dtype=torch.uint8, device=DEV)
    gqa.workspace_init(ws)
    a = gqa.linear(x, w, workspace=ws).clone()
    # a smaller product in between reuses the counters and partials
    x2 = rand_bf16((2, 1024), seed=23).to(DEV)
    w2 = rand_bf16((1024, 512), seed=24).to(DEV)
    gqa.linear(x2, w2, workspace=ws)
    b = gqa.linear(x, w, workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_linear_special_values(ksplit):
    """Zero rows give zeros; a row with a NaN gives NaN in every column; an
    identity block reproduces x."""
    M, K, N = 4, 256, 256
    x = rand_bf16((M, K), seed=31)
    x[1] = 0
    x[2, 17] = float("nan")
    w = torch.zeros((K, N), dtype=torch.bfloat16)
    w[:N, :] = torch.eye(N, dtype=torch.bfloat16)
    y = gqa.linear(x.to(DEV), w.to(DEV)).cpu()
    torch.cuda.synchronize()
    assert torch.equal(y[0], x[0, :N])
    assert torch.equal(y[1], torch.zeros(N, dtype=torch.bfloat16))
    assert torch.isnan(y[2]).all()
    assert torch.equal(y[3], x[3, :N])


# --------------------------------------------------------------- packed weights

def host_pack(w):
    """The packed layout of gqa_pack_weight, by host reshapes: element
    (kb, nb, c, n, e) = w[32kb + 8c + e, 16nb + n]."""
    K, N = w.shape
    return w.reshape(K // 32, 4, 8, N // 16, 16).permute(0, 3, 1, 4, 2).reshape(-1).contiguous()


@pytest.mark.parametrize("shape", [(32, 16), (64, 48), (4096, 6144), (96, 4096)])
def test_pack_weight_layout(shape):
    K, N = shape
    w = rand_bf16((K, N), seed=K + N)
    wp = gqa.pack_weight(w.to(DEV)).cpu()
    torch.cuda.synchronize()
    assert torch.equal(wp.view(torch.int16), host_pack(w).view(torch.int16))


PACKED_CASES = [
    # (M, K, N)
    (1, 32, 16),             # one block
    (5, 96, 48),             # ragged tokens, three strips, a partial chunk
    (4, 1056, 64),           # two whole chunks and a partial one (loop)
    (16, 4096, 6144),        # fused q/k/v projection, d_model 4096, H 32, G 8, d 128 (2 strips, unrolled)
    (16, 4096, 4096),        # output projection of the same layer (1 strip, unrolled)
    (16, 2048, 4096),        # 4 unrolled chunks
    (8, 2048, 6144),         # 2 strips, 4 unrolled chunks
    (1, 8192, 6144),         # 2 strips, 16 unrolled chunks, one token
    (12, 4096, 8192),        # 4 strips per workgroup
    (17, 1024, 272),         # two token tiles
    (33, 512, 640),          # three token tiles (rounded up to four)
    (64, 4096, 128),         # most tokens
    (3, 8192, 1024),         # 16 unrolled chunks
    (2, 4096, 1088),         # fused projection of H 16, G 1, d 64
]


@pytest.mark.parametrize("case", PACKED_CASES, ids=lambda c: "M%d_K%d_N%d" % c)
@pytest.mark.parametrize("plan", [(None, None), ("1", None), ("2", None), ("4", None), (None, "0"), ("2", "0")],
                         ids=["default", "strips1", "strips2", "strips4", "loop", "strips2_loop"])
def test_linear_packed_parity(monkeypatch, case, plan):
    """Every kernel variant of the packed projection (strips per workgroup,
    unrolled or looped chunks; strip counts that do not divide the output
    fall back to one) against the oracle."""
    M, K, N = case
    for name, v in (("GQA_LINEAR_STRIPS", plan[0]), ("GQA_LINEAR_UNROLL", plan[1])):
        if v is None:
            monkeypatch.delenv(name, raising=False)
        else:
            monkeypatch.setenv(name, v)
    x = rand_bf16((M, K), seed=M + K)
    w = rand_bf16((K, N), seed=N + 7, std=K ** -0.5)
    wp = gqa.pack_weight(w.to(DEV))
    y = gqa.linear_packed(x.to(DEV), wp, N)
    torch.cuda.synchronize()
    check_linear(y, x, w, "linear_packed M%d K%d N%d plan=%s" % (M, K, N, plan))


def test_linear_packed_special_values():
    M, K, N = 4, 256, 256
    x = rand_bf16((M, K), seed=31)
    x[1] = 0
    x[2, 17] = float("nan")
    w = torch.eye(N, dtype=torch.bfloat16)
    y = gqa.linear_packed(x.to(DEV), gqa.pack_weight(w.to(DEV)), N).cpu()
    torch.cuda.synchronize()
    assert torch.equal(y[0], x[0])
    assert torch.equal(y[1], torch.zeros(N, dtype=torch.bfloat16))
    assert torch.isnan(y[2]).all()
    assert torch.equal(y[3], x[3])


def test_linear_packed_deterministic():
    M, K, N = 16, 4096, 6144
    x = rand_bf16((M, K), seed=41).to(DEV)
    wp = gqa.pack_weight(rand_bf16((K, N), seed=42, std=K ** -0.5).to(DEV))
    a = gqa.linear_packed(x, wp, N).clone()
    b = gqa.linear_packed(x, wp, N)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


# --------------------------------------------------------------- full decode step

LAYER_CASES = [
    # (B, H, G, d, Lmax, d_model, lens, window)
    (3, 8, 2, 128, 600, 512, [600, 1, 333], 0),
    (3, 8, 2, 128, 600, 512, [600, 1, 333], 100),
    (4, 12, 4, 64, 300, 384, [300, 129, 0, 64], 0),
    (2, 16, 16, 128, 200, 256, [200, 17], 0),          # MHA
    (5, 16, 1, 64, 256, 1024, [256, 255, 1, 2, 100], 0),  # MQA
]


def layer_inputs(B, H, G, d, Lmax, d_model, lens, seed):
    w = wl.Workload("layer", B, H, G, d, Lmax, "bf16", seed)
    _, k, v, _ = wl.make_inputs(w, DEV, pad="nan", seq_lens=torch.tensor(lens, dtype=torch.int32))
    x = rand_bf16((B, d_model), seed=seed + 1)
    w_qkv = rand_bf16((d_model, (H + 2 * G) * d), seed=seed + 2, std=d_model ** -0.5)
    w_o = rand_bf16((H * d, d_model), seed=seed + 3, std=(H * d) ** -0.5)
    lens_t = torch.tensor(lens, dtype=torch.int32, device=DEV)
    return x.to(DEV), w_qkv.to(DEV), w_o.to(DEV), k, v, lens_t, d ** -0.5


def composed(x, w_qkv, w_o, k, v, lens, H, G, scale, window):
    """The same step from the public entry points, one call at a time."""
    B = x.shape[0]
    d = k.shape[3]
    qkv = gqa.linear_packed(x, gqa.pack_weight(w_qkv), w_qkv.shape[1])
    q = qkv[:, :H * d].reshape(B, H, d).contiguous()
    kn = qkv[:, H * d:(H + G) * d].reshape(B, G, d).contiguous()
    vn = qkv[:, (H + G) * d:].reshape(B, G, d).contiguous()
    att = gqa.decode_append(q, kn, vn, k, v, lens, scale, window=window)
    return gqa.linear_packed(att.reshape(B, H * d), gqa.pack_weight(w_o), w_o.shape[1])


def check_layer(y, ref, what):
    got = y.float().cpu().double().numpy()
    err = np.abs(got - ref)
    rms = np.sqrt(np.mean(ref ** 2, axis=1, keepdims=True))
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -5 * rms
    print("%s max|err| = %.3g, rms(y) = %.3g, worst err/bound = %.3f" % (what, float(err.max()), float(rms.mean()),
                                                                         float(np.max(err / np.maximum(bound, 1e-300)))))
    assert np.all(np.isfinite(got)), what
    assert np.all(err <= bound), what


@pytest.mark.parametrize("case", LAYER_CASES, ids=lambda c: "B%d_H%d_G%d_d%d_W%d" % (c[:4] + (c[7],)))
def test_decode_layer_parity(ksplit, case):
    B, H, G, d, Lmax, d_model, lens, window = case
    x, w_qkv, w_o, k, v, lens_t, scale = layer_inputs(B, H, G, d, Lmax, d_model, lens, seed=500 + B + H)
    k0, v0 = k.cpu(), v.cpu()
    y = gqa.decode_layer(x, w_qkv, w_o, k, v, lens_t, H, G, scale, window=window)
    torch.cuda.synchronize()
    ref, rk, rv, (_, rkn, rvn, _) = oracle.decode_layer(x.cpu(), w_qkv.cpu(), w_o.cpu(), k0, v0, lens_t.cpu(), H, G,
                                                        scale, window)
    check_layer(y, ref, "layer %s" % (case,))
    # caches: only row len-1 of each (b, g) changed; it holds the new key/value
    kc, vc = k.cpu(), v.cpu()
    for b, n in enumerate(lens):
        n = min(max(n, 0), Lmax)
        rows = [t for t in range(Lmax) if t != n - 1]
        assert torch.equal(kc[b, :, rows].view(torch.int16), k0[b, :, rows].view(torch.int16))
        assert torch.equal(vc[b, :, rows].view(torch.int16), v0[b, :, rows].view(torch.int16))
        if n > 0:
            for new, ref_new in ((kc[b, :, n - 1], rkn[b]), (vc[b, :, n - 1], rvn[b])):
                diff = (new.float() - ref_new.float()).abs()
                assert torch.all(diff <= 2.0 ** -7 * ref_new.float().abs() + 1e-30), (b, n)


@pytest.mark.parametrize("window", [0, 1000])
def test_decode_layer_equals_composition(ksplit, window):
    """The one-call step is bit-equal to the three entry points in turn
    (same kernels, same plans), caches included; Mistral-7B layer shape."""
    B, H, G, d, Lmax, d_model = 16, 32, 8, 128, 4096, 4096
    lens = [4096] * 8 + [4000 - 301 * i for i in range(8)]
    x, w_qkv, w_o, k, v, lens_t, scale = layer_inputs(B, H, G, d, Lmax, d_model, lens, seed=600)
    k2, v2 = k.clone(), v.clone()
    y1 = gqa.decode_layer(x, w_qkv, w_o, k, v, lens_t, H, G, scale, window=window)
    y2 = composed(x, w_qkv, w_o, k2, v2, lens_t, H, G, scale, window)
    torch.cuda.synchronize()
    assert torch.equal(y1, y2)
    assert torch.equal(k.view(torch.int16), k2.view(torch.int16))
    assert torch.equal(v.view(torch.int16), v2.view(torch.int16))


def test_decode_layer_full_size_against_oracle(ksplit):
    """Mistral-7B layer shape (d_model 4096, H 32, G 8, d 128, 4096 cached
    positions, 16 sequences) against the oracle's step."""
    B, H, G, d, Lmax, d_model = 16, 32, 8, 128, 4096, 4096
    lens = [4096] * B
    x, w_qkv, w_o, k, v, lens_t, scale = layer_inputs(B, H, G, d, Lmax, d_model, lens, seed=700)
    k0, v0 = k.cpu(), v.cpu()
    y = gqa.decode_layer(x, w_qkv, w_o, k, v, lens_t, H, G, scale)
    torch.cuda.synchronize()
    ref, _, _, _ = oracle.decode_layer(x.cpu(), w_qkv.cpu(), w_o.cpu(), k0, v0, lens_t.cpu(), H, G, scale, 0)
    check_layer(y, ref, "layer mistral7b")


def test_layer_step_reuse(ksplit):
    """A bound LayerStep called for consecutive tokens (lengths growing by
    one) matches fresh calls of the composition."""
    B, H, G, d, Lmax, d_model = 2, 8, 2, 128, 64, 256
    x, w_qkv, w_o, k, v, _, scale = layer_inputs(B, H, G, d, Lmax, d_model, [10, 3], seed=800)
    k2, v2 = k.clone(), v.clone()
    lens = torch.tensor([10, 3], dtype=torch.int32, device=DEV)
    step = gqa.LayerStep(x, w_qkv, w_o, k, v, lens, H, G, scale)
    for t in range(4):
        y1 = step().clone()
        y2 = composed(x, w_qkv, w_o, k2, v2, lens, H, G, scale, 0)
        torch.cuda.synchronize()
        assert torch.equal(y1, y2), t
        lens += 1
    assert torch.equal(k.view(torch.int16), k2.view(torch.int16))


# --------------------------------------------------------------- seeded random shapes

def _random_linear(n, seed):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        M = int(rng.integers(1, 65))
        K = 32 * int(rng.integers(1, 97))
        N = 16 * int(rng.integers(1, 161))
        out.append((i, M, K, N))
    return out


@pytest.mark.parametrize("case", _random_linear(24, 77), ids=lambda c: "rand%02d_M%d_K%d_N%d" % c)
def test_random_projections(ksplit, case):
    """gqa_linear_packed on random (M, K, N); gqa_linear as well where N is a
    multiple of 128."""
    i, M, K, N = case
    x = rand_bf16((M, K), seed=9000 + i)
    w = rand_bf16((K, N), seed=9100 + i, std=K ** -0.5)
    y = gqa.linear_packed(x.to(DEV), gqa.pack_weight(w.to(DEV)), N)
    torch.cuda.synchronize()
    check_linear(y, x, w, "packed rand%02d M%d K%d N%d" % case)
    if N % 128 == 0:
        y2 = gqa.linear(x.to(DEV), w.to(DEV))
        torch.cuda.synchronize()
        check_linear(y2, x, w, "row-major rand%02d M%d K%d N%d" % case)
