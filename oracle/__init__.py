"""CPU oracle for grouped-query decode attention (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It loads ``liboracle.so`` built from
``gqa_oracle.c`` (plain C, binary64) and shares no code with the HIP path.

What it computes is stated in ``gqa_oracle.c``: the decode-step block and the
conversion block of the Implementation sketch on the wikillm page
"Grouped-query attention (GQA)", with the block head-to-group assignment that
the sketch assumes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gqa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

# binary64 throughout; no contraction into fused multiply-adds, no fast-math,
# SSE2 arithmetic (the x86-64 default), so every operation rounds once.
GCC_FLAGS = ["-O2", "-std=c11", "-fno-fast-math", "-ffp-contract=off", "-fPIC", "-shared", "-pthread"]

ELEM_F32, ELEM_BF16, ELEM_F64 = 0, 1, 2


def build(src: str = _SRC, out: str = _LIB, extra_flags=()) -> str:
    """Compile the oracle with gcc; returns the path of the shared library."""
    tmp = out + ".tmp%d" % os.getpid()
    cmd = ["gcc", *GCC_FLAGS, *extra_flags, src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


class Oracle:
    """ctypes view of one compiled oracle library (the real one or a test mutant)."""

    def __init__(self, path: str):
        self.path = path
        lib = ctypes.CDLL(path)
        lib.gqa_oracle_decode.restype = ctypes.c_int
        lib.gqa_oracle_decode.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.gqa_oracle_decode_window.restype = ctypes.c_int
        lib.gqa_oracle_decode_window.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.gqa_oracle_decode_append.restype = ctypes.c_int
        lib.gqa_oracle_decode_append.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
            ctypes.c_int, ctypes.c_int, ctypes.c_double, ctypes.c_void_p, ctypes.c_int,
        ]
        lib.gqa_oracle_matmul.restype = ctypes.c_int
        lib.gqa_oracle_matmul.argtypes = [
            ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        lib.gqa_oracle_meanpool.restype = ctypes.c_int
        lib.gqa_oracle_meanpool.argtypes = [
            ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_void_p,
        ]
        self._lib = lib

    def decode(self, q, k_cache, v_cache, seq_lens, scale: float, nthreads: int | None = None,
               window: int = 0) -> np.ndarray:
        """out[B,H,d] float64 for q[B,H,d], k/v[B,G,Lmax,d], seq_lens[B].

        Inputs may be numpy arrays (float32/float64) or CPU torch tensors
        (float32/float64/bfloat16); q, k and v must share one element type.
        window > 0 attends only the last `window` positions of each sequence.
        """
        qa, elem_q = _host_array(q)
        ka, elem_k = _host_array(k_cache)
        va, elem_v = _host_array(v_cache)
        if not (elem_q == elem_k == elem_v):
            raise TypeError("q, k_cache and v_cache must have one element type")
        if qa.ndim != 3 or ka.ndim != 4 or va.shape != ka.shape:
            raise ValueError("expected q[B,H,d] and k/v[B,G,Lmax,d]")
        B, H, d = qa.shape
        Bk, G, Lmax, dk = ka.shape
        if Bk != B or dk != d:
            raise ValueError("q and the caches disagree on B or d")
        sl = np.ascontiguousarray(_to_numpy(seq_lens), dtype=np.int32)
        if sl.shape != (B,):
            raise ValueError("seq_lens must have shape [B]")
        out = np.empty((B, H, d), dtype=np.float64)
        if nthreads is None:
            nthreads = len(os.sched_getaffinity(0))
        rc = self._lib.gqa_oracle_decode_window(
            qa.ctypes.data, ka.ctypes.data, va.ctypes.data, elem_q, sl.ctypes.data,
            B, H, G, d, Lmax, int(window), float(scale), out.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("oracle decode rejected its arguments (rc=%d)" % rc)
        return out

    def decode_append(self, q, k_new, v_new, k_cache, v_cache, seq_lens, scale: float,
                      nthreads: int | None = None, window: int = 0):
        """(out[B,H,d] float64, k_cache', v_cache'): append k_new/v_new [B,G,d] at
        position len-1 of copies of the caches, then decode.  The returned
        caches are numpy arrays in the input storage (bfloat16 as uint16 bits)."""
        qa, e0 = _host_array(q)
        kn, e1 = _host_array(k_new)
        vn, e2 = _host_array(v_new)
        ka, e3 = _host_array(k_cache)
        va, e4 = _host_array(v_cache)
        if len({e0, e1, e2, e3, e4}) != 1:
            raise TypeError("all tensors must have one element type")
        ka, va = ka.copy(), va.copy()
        B, H, d = qa.shape
        _, G, Lmax, _ = ka.shape
        if kn.shape != (B, G, d) or vn.shape != (B, G, d):
            raise ValueError("k_new/v_new must have shape [B,G,d]")
        sl = np.ascontiguousarray(_to_numpy(seq_lens), dtype=np.int32)
        out = np.empty((B, H, d), dtype=np.float64)
        if nthreads is None:
            nthreads = len(os.sched_getaffinity(0))
        rc = self._lib.gqa_oracle_decode_append(
            qa.ctypes.data, kn.ctypes.data, vn.ctypes.data, ka.ctypes.data, va.ctypes.data, e0, sl.ctypes.data,
            B, H, G, d, Lmax, int(window), float(scale), out.ctypes.data, int(nthreads))
        if rc != 0:
            raise ValueError("oracle decode_append rejected its arguments (rc=%d)" % rc)
        return out, ka, va

    def matmul(self, x, w) -> np.ndarray:
        """y[M,N] float64 = x[M,K] @ w[K,N] (same element type; bfloat16 exactly widened)."""
        xa, ex = _host_array(x)
        wa, ew = _host_array(w)
        if ex != ew or xa.ndim != 2 or wa.ndim != 2 or xa.shape[1] != wa.shape[0]:
            raise ValueError("expected x[M,K] and w[K,N] of one element type")
        M, K = xa.shape
        N = wa.shape[1]
        y = np.empty((M, N), dtype=np.float64)
        rc = self._lib.gqa_oracle_matmul(xa.ctypes.data, wa.ctypes.data, ex, M, K, N, y.ctypes.data)
        if rc != 0:
            raise ValueError("oracle matmul rejected its arguments (rc=%d)" % rc)
        return y

    def decode_layer(self, x, w_qkv, w_o, k_cache, v_cache, seq_lens, H: int, G: int, scale: float, window: int = 0):
        """One decode step of the Implementation sketch's decode-step block for a
        batch of tokens, in the storage type of its inputs (bfloat16 or binary32):
        qkv = x @ w_qkv (columns: H query heads, then G key heads, then G value
        heads, d each), rounded to the storage type; the new key/value appended
        at position len-1; attention; the attention output rounded to the
        storage type; y = out @ w_o.  Returns (y float64 [M, d_model], caches)."""
        import torch
        is_bf16 = isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16
        dt = torch.bfloat16 if is_bf16 else torch.float32
        M = x.shape[0]
        d = w_qkv.shape[1] // (H + 2 * G)
        qkv = torch.from_numpy(self.matmul(x, w_qkv)).to(dt)
        q = qkv[:, :H * d].reshape(M, H, d).contiguous()
        kn = qkv[:, H * d:(H + G) * d].reshape(M, G, d).contiguous()
        vn = qkv[:, (H + G) * d:].reshape(M, G, d).contiguous()
        out, kc, vc = self.decode_append(q, kn, vn, k_cache, v_cache, seq_lens, scale, window=window)
        att = torch.from_numpy(out).to(dt).reshape(M, H * d).contiguous()
        return self.matmul(att, w_o), kc, vc, (q, kn, vn, att)

    def meanpool(self, w, H: int, G: int) -> np.ndarray:
        """w_out[d_model, G*h] float32 from w[d_model, H*h] float32."""
        wa = np.ascontiguousarray(_to_numpy(w))
        if wa.dtype != np.float32 or wa.ndim != 2 or wa.shape[1] % H:
            raise ValueError("expected float32 w[d_model, H*h]")
        d_model = wa.shape[0]
        h = wa.shape[1] // H
        out = np.empty((d_model, G * h), dtype=np.float32)
        rc = self._lib.gqa_oracle_meanpool(wa.ctypes.data, d_model, H, G, h, out.ctypes.data)
        if rc != 0:
            raise ValueError("oracle meanpool rejected its arguments (rc=%d)" % rc)
        return out


def _to_numpy(x):
    if isinstance(x, np.ndarray):
        return x
    try:
        import torch
    except ImportError:  # pragma: no cover
        torch = None
    if torch is not None and isinstance(x, torch.Tensor):
        x = x.detach()
        if x.device.type != "cpu":
            x = x.cpu()
        if x.dtype == torch.bfloat16:
            return x.contiguous().view(torch.int16).numpy().view(np.uint16)
        return x.contiguous().numpy()
    return np.asarray(x)


def _host_array(x):
    """(contiguous numpy array, element code); bfloat16 arrives as uint16 bits."""
    is_bf16 = False
    try:
        import torch
        is_bf16 = isinstance(x, torch.Tensor) and x.dtype == torch.bfloat16
    except ImportError:  # pragma: no cover
        pass
    a = np.ascontiguousarray(_to_numpy(x))
    if is_bf16:
        return a, ELEM_BF16
    if a.dtype == np.float32:
        return a, ELEM_F32
    if a.dtype == np.float64:
        return a, ELEM_F64
    raise TypeError("unsupported oracle input dtype %s" % a.dtype)


_default: Oracle | None = None


def get() -> Oracle:
    """The oracle built from ``gqa_oracle.c``, compiling it when absent or stale."""
    global _default
    if _default is None:
        if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
            build()
        _default = Oracle(_LIB)
    return _default


def decode(q, k_cache, v_cache, seq_lens, scale, nthreads=None, window=0):
    return get().decode(q, k_cache, v_cache, seq_lens, scale, nthreads, window)


def decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale, nthreads=None, window=0):
    return get().decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale, nthreads, window)


def meanpool(w, H, G):
    return get().meanpool(w, H, G)


def matmul(x, w):
    return get().matmul(x, w)


def decode_layer(x, w_qkv, w_o, k_cache, v_cache, seq_lens, H, G, scale, window=0):
    return get().decode_layer(x, w_qkv, w_o, k_cache, v_cache, seq_lens, H, G, scale, window)
