"""Pins that tie the CPU oracle to facts outside itself.

Every pin takes an ``oracle.Oracle`` and raises AssertionError on a mismatch,
so the same pins run against the real oracle (test_oracle_pins.py) and against
copies of it with a planted mistake (test_oracle_mutants.py), where at least
one pin must fail.

What fixes each expected value:
  * torch's CPU scaled_dot_product_attention in float64 (a library routine the
    oracle does not use): with ``enable_gqa`` (the library's own grouping), on
    K/V heads replicated per group, and at the two endpoints the glossary and
    the concept page name (G = H is multi-head, G = 1 is multi-query);
  * scipy's softmax for the attention weights themselves (value rows set to
    one-hot vectors make the output equal to the weights);
  * closed forms: one cached position, zero query, constant values, the golden
    fixtures under tests/golden/;
  * invariants of the definition: no positional term (joint permutation of the
    cached positions), positions at or beyond the length are never read, equal
    queries in one group give equal outputs, linearity of the conversion.
"""
from __future__ import annotations

import json
import math
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand_case(rng, B, H, G, d, Lmax, lens=None, scale=None, mag=1.0):
    q = rng.standard_normal((B, H, d)) * mag
    k = rng.standard_normal((B, G, Lmax, d)) * mag
    v = rng.standard_normal((B, G, Lmax, d))
    if lens is None:
        lens = np.full(B, Lmax, dtype=np.int32)
    lens = np.asarray(lens, dtype=np.int32)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    return q, k, v, lens, scale


def _sdpa(q, k, v, scale, enable_gqa):
    """torch SDPA for one sequence: q[H,d], k/v[Gk,T,d] -> [H,d] float64."""
    import torch
    import torch.nn.functional as F
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, scale=scale, enable_gqa=enable_gqa)
    return o[0, :, 0, :].numpy()


def pin_sdpa_enable_gqa(o):
    """Grouped decode equals the library's grouped-query SDPA, ragged lengths."""
    rng = np.random.default_rng(11)
    for G in (1, 2, 4, 8):
        for scale in (None, 0.37):
            q, k, v, lens, sc = _rand_case(rng, 3, 8, G, 8, 7, lens=[7, 3, 1], scale=scale)
            out = o.decode(q, k, v, lens, sc)
            for b in range(3):
                n = lens[b]
                ref = _sdpa(q[b], k[b, :, :n], v[b, :, :n], sc, enable_gqa=True)
                np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def pin_sdpa_replicated_heads(o):
    """Grouped decode equals multi-head SDPA on K/V heads copied to each of
    their H/G query heads in consecutive blocks (the sketch's assumption)."""
    rng = np.random.default_rng(12)
    H = 12
    for G in (2, 3, 4, 6):
        q, k, v, lens, sc = _rand_case(rng, 2, H, G, 4, 5, lens=[5, 2])
        out = o.decode(q, k, v, lens, sc)
        r = H // G
        for b in range(2):
            n = lens[b]
            kr = np.stack([k[b, g, :n] for g in range(G) for _ in range(r)])
            vr = np.stack([v[b, g, :n] for g in range(G) for _ in range(r)])
            ref = _sdpa(q[b], kr, vr, sc, enable_gqa=False)
            np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def pin_mha_endpoint(o):
    """G = H: ordinary multi-head attention, head h reads K/V head h."""
    rng = np.random.default_rng(13)
    q, k, v, lens, sc = _rand_case(rng, 2, 6, 6, 8, 9, lens=[9, 4])
    out = o.decode(q, k, v, lens, sc)
    for b in range(2):
        n = lens[b]
        ref = _sdpa(q[b], k[b, :, :n], v[b, :, :n], sc, enable_gqa=False)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def pin_mqa_endpoint(o):
    """G = 1: multi-query attention, every head reads the one K/V head."""
    rng = np.random.default_rng(14)
    H = 8
    q, k, v, lens, sc = _rand_case(rng, 2, H, 1, 8, 6, lens=[6, 5])
    out = o.decode(q, k, v, lens, sc)
    for b in range(2):
        n = lens[b]
        kr = np.repeat(k[b, :, :n], H, axis=0)
        vr = np.repeat(v[b, :, :n], H, axis=0)
        ref = _sdpa(q[b], kr, vr, sc, enable_gqa=False)
        np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12)


def pin_weights_are_softmax(o):
    """One-hot value rows expose the weights: they match scipy's softmax of the
    scaled scores, are non-negative and sum to 1."""
    from scipy.special import softmax
    rng = np.random.default_rng(15)
    B, H, G, d, L = 2, 4, 2, 8, 8
    q, k, _, lens, sc = _rand_case(rng, B, H, G, d, L, lens=[8, 5])
    v = np.zeros((B, G, L, d))
    for t in range(L):
        v[:, :, t, t] = 1.0
    out = o.decode(q, k, v, lens, sc)
    r = H // G
    for b in range(B):
        n = lens[b]
        for h in range(H):
            w = softmax(sc * (k[b, h // r, :n] @ q[b, h]))
            np.testing.assert_allclose(out[b, h, :n], w, rtol=0, atol=1e-14)
            assert np.all(out[b, h, n:] == 0.0)
            assert abs(out[b, h].sum() - 1.0) <= 1e-12
            assert np.all(out[b, h] >= 0.0)


def pin_large_scores(o):
    """Scores near +-1000 overflow a naive exp; the result must still match SDPA."""
    rng = np.random.default_rng(16)
    q, k, v, lens, sc = _rand_case(rng, 1, 4, 2, 4, 6, mag=1.0, scale=1.0)
    q = q * 30.0
    k = k * 30.0
    out = o.decode(q, k, v, lens, sc)
    assert np.all(np.isfinite(out))
    ref = _sdpa(q[0], k[0], v[0], sc, enable_gqa=True)
    np.testing.assert_allclose(out[0], ref, rtol=0, atol=1e-12)


def pin_constant_values(o):
    rng = np.random.default_rng(17)
    q, k, v, lens, sc = _rand_case(rng, 2, 8, 2, 8, 10, lens=[10, 3])
    v[:] = 0.0
    v[..., :] = np.arange(8) * 0.25 - 1.0  # every position carries the same row
    out = o.decode(q, k, v, lens, sc)
    np.testing.assert_allclose(out, np.broadcast_to(np.arange(8) * 0.25 - 1.0, out.shape), rtol=0, atol=1e-14)


def pin_single_position(o):
    """One cached position: its weight is exactly 1, out equals that value row bitwise."""
    rng = np.random.default_rng(18)
    q, k, v, lens, sc = _rand_case(rng, 3, 6, 3, 8, 4, lens=[1, 1, 1])
    out = o.decode(q, k, v, lens, sc)
    for b in range(3):
        for h in range(6):
            assert np.array_equal(out[b, h], v[b, h // 2, 0])


def pin_zero_query(o):
    """q = 0 gives equal scores, so out is the plain mean of the cached value rows."""
    rng = np.random.default_rng(19)
    q, k, v, lens, sc = _rand_case(rng, 2, 4, 2, 8, 7, lens=[7, 4])
    q[:] = 0.0
    out = o.decode(q, k, v, lens, sc)
    for b in range(2):
        for h in range(4):
            np.testing.assert_allclose(out[b, h], v[b, h // 2, :lens[b]].mean(axis=0), rtol=0, atol=1e-14)


def pin_permutation_invariance(o):
    """No positional term: permuting the cached positions of K and V jointly
    leaves the output unchanged."""
    rng = np.random.default_rng(20)
    q, k, v, lens, sc = _rand_case(rng, 1, 4, 2, 8, 9)
    perm = rng.permutation(9)
    a = o.decode(q, k, v, lens, sc)
    b = o.decode(q, k[:, :, perm], v[:, :, perm], lens, sc)
    np.testing.assert_allclose(a, b, rtol=0, atol=1e-13)


def pin_padding_never_read(o):
    """NaN beyond each sequence's length does not reach the output."""
    rng = np.random.default_rng(21)
    q, k, v, lens, sc = _rand_case(rng, 3, 4, 2, 8, 8, lens=[8, 5, 1])
    a = o.decode(q, k, v, lens, sc)
    k2, v2 = k.copy(), v.copy()
    for b in range(3):
        k2[b, :, lens[b]:] = np.nan
        v2[b, :, lens[b]:] = np.nan
    b_ = o.decode(q, k2, v2, lens, sc)
    assert np.all(np.isfinite(b_))
    assert np.array_equal(a, b_)


def pin_equal_queries(o):
    """Identical query rows inside one group produce identical outputs; the
    same rows in different groups do not (the groups hold different K/V)."""
    rng = np.random.default_rng(22)
    q, k, v, lens, sc = _rand_case(rng, 1, 8, 2, 8, 6)
    q[0, :] = q[0, 0]
    out = o.decode(q, k, v, lens, sc)
    for h in range(4):
        assert np.array_equal(out[0, h], out[0, 0])
        assert np.array_equal(out[0, 4 + h], out[0, 4])
    assert not np.allclose(out[0, 0], out[0, 4])


def pin_empty_and_clamped_lengths(o):
    """Length 0 gives zeros; a length above Lmax behaves as Lmax."""
    rng = np.random.default_rng(23)
    q, k, v, _, sc = _rand_case(rng, 3, 4, 2, 8, 5)
    out = o.decode(q, k, v, np.array([0, 9, 5], dtype=np.int32), sc)
    assert np.array_equal(out[0], np.zeros((4, 8)))
    assert np.array_equal(out[1], o.decode(q[1:2], k[1:2], v[1:2], np.array([5], np.int32), sc)[0])
    np.testing.assert_allclose(out[2], _sdpa(q[2], k[2], v[2], sc, True), rtol=0, atol=1e-12)


def pin_golden_decode(o):
    with open(os.path.join(GOLDEN, "decode_closed_form.json")) as f:
        fx = json.load(f)
    for c in fx["cases"]:
        out = o.decode(np.array(c["q"], np.float64), np.array(c["k"], np.float64),
                       np.array(c["v"], np.float64), np.array(c["seq_lens"], np.int32), c["scale"])
        np.testing.assert_allclose(out, np.array(c["out"]), rtol=1e-14, atol=1e-14, err_msg=c["name"])


def pin_bf16_and_f32_storage(o):
    """Stored bfloat16 / binary32 values are widened exactly: the same values
    given as binary64 give the identical output."""
    import torch
    rng = np.random.default_rng(24)
    q, k, v, lens, sc = _rand_case(rng, 2, 4, 2, 8, 6, lens=[6, 2])
    for dt in (torch.bfloat16, torch.float32):
        qt, kt, vt = (torch.from_numpy(x).to(dt) for x in (q, k, v))
        a = o.decode(qt, kt, vt, lens, sc)
        b = o.decode(qt.double().numpy(), kt.double().numpy(), vt.double().numpy(), lens, sc)
        assert np.array_equal(a, b)


def _sdpa_masked(q, k, v, scale, lo, n):
    """torch SDPA for one sequence over positions lo .. n-1 (boolean mask), grouped."""
    import torch
    import torch.nn.functional as F
    L = k.shape[1]
    mask = torch.zeros(1, 1, 1, L, dtype=torch.bool)
    mask[..., lo:n] = True
    qt = torch.from_numpy(np.ascontiguousarray(q))[None, :, None, :]
    kt = torch.from_numpy(np.ascontiguousarray(k))[None]
    vt = torch.from_numpy(np.ascontiguousarray(v))[None]
    o = F.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=scale, enable_gqa=True)
    return o[0, :, 0, :].numpy()


def pin_window_sdpa_mask(o):
    """Sliding window: only positions max(0, len-W) .. len-1 are attended
    (library SDPA with an explicit position mask)."""
    rng = np.random.default_rng(41)
    q, k, v, lens, sc = _rand_case(rng, 4, 8, 2, 8, 12, lens=[12, 7, 3, 1])
    for W in (1, 2, 5, 7, 11, 12, 40):
        out = o.decode(q, k, v, lens, sc, window=W)
        for b in range(4):
            n = int(lens[b])
            ref = _sdpa_masked(q[b], k[b], v[b], sc, max(0, n - W), n)
            np.testing.assert_allclose(out[b], ref, rtol=0, atol=1e-12, err_msg="W=%d b=%d" % (W, b))


def pin_window_closed_forms(o):
    """W = 1 gives the last value row exactly; W >= len gives the plain decode exactly."""
    rng = np.random.default_rng(42)
    q, k, v, lens, sc = _rand_case(rng, 3, 4, 2, 8, 9, lens=[9, 4, 1])
    one = o.decode(q, k, v, lens, sc, window=1)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(one[b, h], v[b, h // 2, lens[b] - 1])
    assert np.array_equal(o.decode(q, k, v, lens, sc, window=9), o.decode(q, k, v, lens, sc))
    assert np.array_equal(o.decode(q, k, v, lens, sc, window=1000), o.decode(q, k, v, lens, sc))


def _append_case(rng, B=3, H=8, G=2, d=8, L=10, lens=(10, 4, 1)):
    q, k, v, lens, sc = _rand_case(rng, B, H, G, d, L, lens=list(lens))
    k_new = rng.standard_normal((B, G, d))
    v_new = rng.standard_normal((B, G, d))
    return q, k, v, lens, sc, k_new, v_new


def pin_append_updates_the_cache(o):
    """The new key/value land at position len-1 of each sequence; nothing else changes."""
    rng = np.random.default_rng(43)
    q, k, v, lens, sc, kn, vn = _append_case(rng, lens=(10, 4, 1))
    lens = np.array([10, 4, 0], np.int32)
    _, k2, v2 = o.decode_append(q, kn, vn, k, v, lens, sc)
    ek, ev = k.copy(), v.copy()
    for b in range(2):
        ek[b, :, lens[b] - 1] = kn[b]
        ev[b, :, lens[b] - 1] = vn[b]
    assert np.array_equal(k2, ek) and np.array_equal(v2, ev)


def pin_append_matches_sdpa(o):
    """Append then attend = library SDPA over the cache with row len-1
    replaced by the new key/value; one position gives v_new exactly."""
    rng = np.random.default_rng(44)
    q, k, v, lens, sc, kn, vn = _append_case(rng, lens=(10, 5, 1))
    for W in (0, 3):
        out, _, _ = o.decode_append(q, kn, vn, k, v, lens, sc, window=W)
        for b in range(3):
            n = int(lens[b])
            kk, vv = k[b].copy(), v[b].copy()
            kk[:, n - 1] = kn[b]
            vv[:, n - 1] = vn[b]
            lo = max(0, n - W) if W else 0
            np.testing.assert_allclose(out[b], _sdpa_masked(q[b], kk, vv, sc, lo, n), rtol=0, atol=1e-12)
        for h in range(8):
            assert np.array_equal(out[2, h], vn[2, h // 4])


def pin_matmul_numpy(o):
    """The projections x @ W against numpy's matmul in float64; an identity W
    returns x; rows and columns are not swapped (non-square shapes)."""
    rng = np.random.default_rng(45)
    for M, K, N in ((1, 8, 5), (3, 16, 24), (7, 5, 3)):
        x = rng.standard_normal((M, K))
        w = rng.standard_normal((K, N))
        np.testing.assert_allclose(o.matmul(x, w), x @ w, rtol=0, atol=1e-12)
    x = rng.standard_normal((4, 6))
    assert np.array_equal(o.matmul(x, np.eye(6)), x)


def pin_decode_layer_composition(o):
    """The decode step with projections (batch, one token per sequence) equals
    its stages: library matmuls for the projections, masked library SDPA over
    the appended cache for attention."""
    import torch
    rng = np.random.default_rng(46)
    B, H, G, d, L, dm = 3, 8, 2, 8, 9, 16
    x = torch.from_numpy(rng.standard_normal((B, dm)))
    wqkv = torch.from_numpy(rng.standard_normal((dm, (H + 2 * G) * d)) / 4)
    wo = torch.from_numpy(rng.standard_normal((H * d, dm)) / 8)
    _, k, v, lens, sc = _rand_case(rng, B, H, G, d, L, lens=[9, 4, 1])
    y, kc, vc, _ = o.decode_layer(x.float(), wqkv.float(), wo.float(), k.astype(np.float32), v.astype(np.float32),
                                  lens, H, G, sc)
    qkv = (x.float().double() @ wqkv.float().double()).float().numpy().astype(np.float64)
    q = qkv[:, :H * d].reshape(B, H, d)
    kn = qkv[:, H * d:(H + G) * d].reshape(B, G, d)
    vn = qkv[:, (H + G) * d:].reshape(B, G, d)
    att = np.zeros((B, H, d))
    for b in range(B):
        n = int(lens[b])
        kk = k[b].astype(np.float32).astype(np.float64)
        vv = v[b].astype(np.float32).astype(np.float64)
        kk[:, n - 1] = kn[b]
        vv[:, n - 1] = vn[b]
        att[b] = _sdpa_masked(q[b], kk, vv, sc, 0, n)
    ref = att.astype(np.float32).astype(np.float64).reshape(B, H * d) @ wo.float().double().numpy()
    np.testing.assert_allclose(y, ref, rtol=1e-6, atol=1e-6)


DECODE_PINS = [
    pin_sdpa_enable_gqa, pin_sdpa_replicated_heads, pin_mha_endpoint, pin_mqa_endpoint,
    pin_weights_are_softmax, pin_large_scores, pin_constant_values, pin_single_position,
    pin_zero_query, pin_permutation_invariance, pin_padding_never_read, pin_equal_queries,
    pin_empty_and_clamped_lengths, pin_golden_decode, pin_bf16_and_f32_storage,
    pin_window_sdpa_mask, pin_window_closed_forms, pin_append_updates_the_cache, pin_append_matches_sdpa,
    pin_matmul_numpy, pin_decode_layer_composition,
]


# ----------------------------------------------------------------------------- meanpool

def f32_bits(x) -> int:
    return struct.unpack("<I", struct.pack("<f", float(x)))[0]


def round_fraction_to_f32(fr: Fraction) -> np.float32:
    """Correctly rounded (ties to even) binary32 of an exact rational."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        err = abs(Fraction(float(cand)) - fr)
        key = (err, f32_bits(cand) & 1)  # on a tie prefer the even significand
        if best is None or key < best[0]:
            best = (key, cand)
    return best[1]


def pin_meanpool_identity(o):
    """G = H: every group has one member, the pool is the identity bitwise."""
    rng = np.random.default_rng(31)
    w = rng.standard_normal((5, 6 * 4)).astype(np.float32)
    assert np.array_equal(o.meanpool(w, 6, 6).view(np.uint32), w.view(np.uint32))


def pin_meanpool_identical_members(o):
    rng = np.random.default_rng(32)
    blocks = rng.standard_normal((3, 2, 4)).astype(np.float32)  # [d_model, G, h]
    w = np.concatenate([blocks[:, g] for g in range(2) for _ in range(3)], axis=1)
    assert np.array_equal(o.meanpool(w, 6, 2), blocks.reshape(3, 8))


def pin_meanpool_structured(o):
    """w[:, i*h + c] = 16*i + c/64: pooled column g*h + c is
    16*(g*r + (r-1)/2) + c/64, exact in binary32; fixes the column layout."""
    H, G, h, dm = 8, 2, 4, 3
    r = H // G
    w = np.array([[16.0 * i + c / 64.0 for i in range(H) for c in range(h)]] * dm, np.float32)
    exp = np.array([[16.0 * (g * r + (r - 1) / 2.0) + c / 64.0 for g in range(G) for c in range(h)]] * dm, np.float32)
    assert np.array_equal(o.meanpool(w, H, G), exp)


def pin_meanpool_exact_rational(o):
    """Against the exact rational mean rounded once to binary32: agreement
    except where rounding the binary64 quotient first moves a tie, and then by
    at most one unit in the last place."""
    rng = np.random.default_rng(33)
    for H, G in ((8, 2), (6, 2), (12, 4), (5, 1)):
        h = 4
        w = (rng.standard_normal((16, H * h)) * rng.choice([1e-3, 1.0, 1e3], size=(16, H * h))).astype(np.float32)
        got = o.meanpool(w, H, G)
        r = H // G
        mism = 0
        for row in range(16):
            for g in range(G):
                for c in range(h):
                    fr = sum(Fraction(float(w[row, i * h + c])) for i in range(g * r, g * r + r)) / r
                    e = round_fraction_to_f32(fr)
                    gbits, ebits = f32_bits(got[row, g * h + c]), f32_bits(e)
                    if gbits != ebits:
                        mism += 1
                        assert abs(int(gbits) - int(ebits)) == 1
        assert mism <= 1


def pin_meanpool_signed_zero(o):
    w = np.array([[-0.0, -0.0, 0.0, -0.0]], np.float32)
    out = o.meanpool(w, 4, 2)
    assert f32_bits(out[0, 0]) == 0x80000000  # mean(-0, -0) = -0
    assert f32_bits(out[0, 1]) == 0x00000000  # mean(+0, -0) = +0


def pin_golden_meanpool(o):
    with open(os.path.join(GOLDEN, "meanpool_closed_form.json")) as f:
        fx = json.load(f)
    for c in fx["cases"]:
        out = o.meanpool(np.array(c["w"], np.float32), c["H"], c["G"])
        bits = [[f32_bits(x) for x in row] for row in out]
        assert bits == [[int(x, 16) for x in row] for row in c["out_hex"]], c["name"]


def pin_conversion_then_decode(o):
    """Conversion and decode together: an MHA layer whose K/V heads are
    identical within each group converts to a GQA layer with the same output;
    for any MHA layer the pooled keys/values are the per-group mean of the
    multi-head keys/values (the projection is linear)."""
    rng = np.random.default_rng(34)
    dm, H, G, h, T = 16, 8, 2, 4, 6
    r = H // G
    X = rng.standard_normal((T, dm)).astype(np.float32)      # cached tokens
    x = rng.standard_normal(dm).astype(np.float32)           # new token
    Wq = rng.standard_normal((dm, H * h)).astype(np.float32)
    base_k = rng.standard_normal((dm, G * h)).astype(np.float32)
    base_v = rng.standard_normal((dm, G * h)).astype(np.float32)
    Wk = np.concatenate([base_k[:, (i // r) * h:(i // r + 1) * h] for i in range(H)], axis=1)
    Wv = np.concatenate([base_v[:, (i // r) * h:(i // r + 1) * h] for i in range(H)], axis=1)
    X64, x64 = X.astype(np.float64), x.astype(np.float64)
    q = (x64 @ Wq.astype(np.float64)).reshape(1, H, h)
    k_mha = (X64 @ Wk.astype(np.float64)).reshape(T, H, h).transpose(1, 0, 2)[None]
    v_mha = (X64 @ Wv.astype(np.float64)).reshape(T, H, h).transpose(1, 0, 2)[None]
    lens = np.array([T], np.int32)
    mha = o.decode(q, k_mha, v_mha, lens, 0.5)
    Wk_g, Wv_g = o.meanpool(Wk, H, G), o.meanpool(Wv, H, G)
    k_g = (X64 @ Wk_g.astype(np.float64)).reshape(T, G, h).transpose(1, 0, 2)[None]
    v_g = (X64 @ Wv_g.astype(np.float64)).reshape(T, G, h).transpose(1, 0, 2)[None]
    gqa = o.decode(q, k_g, v_g, lens, 0.5)
    np.testing.assert_allclose(gqa, mha, rtol=0, atol=1e-12)

    Wk = rng.standard_normal((dm, H * h)).astype(np.float32)
    k_mha = (X64 @ Wk.astype(np.float64)).reshape(T, H, h)
    k_g = (X64 @ o.meanpool(Wk, H, G).astype(np.float64)).reshape(T, G, h)
    mean_k = k_mha.reshape(T, G, r, h).mean(axis=2)
    np.testing.assert_allclose(k_g, mean_k, rtol=0, atol=1e-4)


MEANPOOL_PINS = [
    pin_meanpool_identity, pin_meanpool_identical_members, pin_meanpool_structured,
    pin_meanpool_exact_rational, pin_meanpool_signed_zero, pin_golden_meanpool,
    pin_conversion_then_decode,
]

ALL_PINS = DECODE_PINS + MEANPOOL_PINS
