"""Runs every entry point of one build of the C oracle over a fixed set of
seeded small cases and saves the outputs (test infrastructure, used by
test_oracle_sanitized.py).  It imports only numpy, so it can run in a process
with a sanitizer runtime preloaded:

    python oracle_sanitize_driver.py <liboracle.so> <out.npz>

bfloat16 inputs are passed as their uint16 bit patterns with the oracle's
bfloat16 element code.  Cases cover empty and clamped lengths, windows, the
cache append (including an empty sequence), several thread counts, the
projection product and the mean-pool, and calls the oracle must reject."""
import os
import sys

sys.modules["torch"] = None  # keep torch out of this process (the oracle wrapper then works on numpy alone)
sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))

import numpy as np  # noqa: E402

import oracle  # noqa: E402


def bf16_bits(x):
    """float32 -> bfloat16 bits, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def main(lib_path, out_path):
    ora = oracle.Oracle(lib_path)
    raw = ora._lib
    rng = np.random.default_rng(20261203)
    res = {}
    B, H, G, d, Lmax = 4, 8, 2, 16, 37
    lens = np.array([37, 0, 50, 1], dtype=np.int32)  # full, empty, clamped, one position
    q = rng.standard_normal((B, H, d)).astype(np.float32)
    k = rng.standard_normal((B, G, Lmax, d)).astype(np.float32)
    v = rng.standard_normal((B, G, Lmax, d)).astype(np.float32)
    for nt in (1, 3, 8):
        for win in (0, 1, 5, 100):
            res["f32_t%d_w%d" % (nt, win)] = ora.decode(q, k, v, lens, 0.25, nthreads=nt, window=win)
            res["f64_t%d_w%d" % (nt, win)] = ora.decode(q.astype(np.float64), k.astype(np.float64),
                                                        v.astype(np.float64), lens, 0.25, nthreads=nt, window=win)
            qb, kb, vb = bf16_bits(q), bf16_bits(k), bf16_bits(v)
            out = np.empty((B, H, d), dtype=np.float64)
            rc = raw.gqa_oracle_decode_window(qb.ctypes.data, kb.ctypes.data, vb.ctypes.data, oracle.ELEM_BF16,
                                              lens.ctypes.data, B, H, G, d, Lmax, win, 0.25, out.ctypes.data, nt)
            assert rc == 0
            res["bf16_t%d_w%d" % (nt, win)] = out
    kn = rng.standard_normal((B, G, d)).astype(np.float32)
    vn = rng.standard_normal((B, G, d)).astype(np.float32)
    for win in (0, 3):
        out, kc, vc = ora.decode_append(q, kn, vn, k, v, lens, 0.25, nthreads=2, window=win)
        res["append_w%d" % win], res["append_k_w%d" % win], res["append_v_w%d" % win] = out, kc, vc
    x = rng.standard_normal((5, 64)).astype(np.float32)
    w = rng.standard_normal((64, 48)).astype(np.float32)
    res["matmul_f32"] = ora.matmul(x, w)
    y = np.empty((5, 48), dtype=np.float64)
    xb, wb = bf16_bits(x), bf16_bits(w)  # held: .ctypes.data does not keep an array alive
    assert raw.gqa_oracle_matmul(xb.ctypes.data, wb.ctypes.data, oracle.ELEM_BF16, 5, 64, 48, y.ctypes.data) == 0
    res["matmul_bf16"] = y
    wm = (rng.standard_normal((7, 12 * 5)) * np.exp(rng.standard_normal((7, 12 * 5)) * 3)).astype(np.float32)
    for g in (1, 3, 4, 12):
        res["meanpool_G%d" % g] = ora.meanpool(wm, 12, g)
    # rejected arguments: no memory is touched
    bad = np.empty((1, 6, d), dtype=np.float64)
    assert raw.gqa_oracle_decode_window(q.ctypes.data, k.ctypes.data, v.ctypes.data, oracle.ELEM_F32,
                                        lens.ctypes.data, 1, 6, 4, d, Lmax, 0, 0.25, bad.ctypes.data, 1) != 0
    assert raw.gqa_oracle_meanpool(wm.ctypes.data, 7, 12, 5, 5, res["meanpool_G1"].ctypes.data) != 0
    np.savez(out_path, **res)
    print("driver ok: %d results" % len(res))


if __name__ == "__main__":
    main(sys.argv[1], sys.argv[2])
