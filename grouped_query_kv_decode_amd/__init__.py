"""Grouped-query decode attention for AMD Instinct MI355X (gfx950).

Thin ctypes binding over ``libgqa.so`` (C ABI in ``include/gqa.h``): argument
marshalling only.  Every step of the computation runs in the HIP kernels; if
the library is missing or cannot be loaded the calls raise - there is no
fallback path.  PyTorch supplies device memory and the stream.

Entry points (same names as the C ABI, without the ``gqa_`` prefix):
    decode(q, k_cache, v_cache, seq_lens, scale, out=None, workspace=None)
    decode_noalloc(q, k_cache, v_cache, seq_lens, scale, out=None)   no workspace (library scratch)
    decode_workspace_size(B, H, G, d, Lmax, dtype)
    decode_phase(phase, ...)           (split kernel / merge kernel separately)
    decode_window(q, k_cache, v_cache, seq_lens, scale, window, ...)
    decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale, window=0, ...)
    workspace_init(workspace)
    linear(x, w, out=None, workspace=None)              y = x @ w (bfloat16 projections, row-major w)
    pack_weight(w)                                      w in the packed matrix-core layout
    linear_packed(x, w_packed, N, out=None)             y = x @ w from the packed layout
    decode_layer(x, w_qkv, w_o, k_cache, v_cache, seq_lens, H, G, scale, window=0)
    meanpool_kv(w, H, G, out=None)
    decode_kernel_kind(B, H, G, d, Lmax, dtype)
    stream_read(buf, nontemporal=True, grid=0, sink=None)   the read-ceiling probe (measurement only)
    tuning_reload()                    re-read the GQA_* launch-plan overrides (tuning and tests)
"""
from __future__ import annotations

import ctypes
import os

__all__ = [
    "GQAError", "decode", "decode_noalloc", "decode_phase", "decode_window", "decode_append", "decode_workspace_size", "workspace_init", "meanpool_kv",
    "linear", "linear_workspace_size", "pack_weight", "linear_packed", "decode_layer", "decode_layer_workspace_size", "LayerStep",
    "decode_kernel_kind", "stream_read", "tuning_reload", "status_string", "library_path", "load_library", "Decoder",
    "GQA_F32", "GQA_BF16",
]

_PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_PKG, "libgqa.so")

GQA_F32, GQA_BF16 = 0, 1
NOALLOC_SCRATCH_BYTES = 32 << 20  # GQA_NOALLOC_SCRATCH_BYTES of gqa.h: the scratch of decode_noalloc
STATUS_NAMES = {
    0: "GQA_OK", 1: "GQA_ERR_NULL", 2: "GQA_ERR_SHAPE", 3: "GQA_ERR_UNSUPPORTED", 4: "GQA_ERR_ALIGN",
    5: "GQA_ERR_WORKSPACE", 6: "GQA_ERR_SCALE", 7: "GQA_ERR_HIP", 8: "GQA_ERR_SIZE",
}
EXPORTED = [
    "gqa_decode_workspace_size", "gqa_workspace_init", "gqa_decode", "gqa_decode_noalloc", "gqa_decode_phase",
    "gqa_decode_window",
    "gqa_decode_append", "gqa_linear_workspace_size", "gqa_linear", "gqa_pack_weight", "gqa_linear_packed",
    "gqa_decode_layer_workspace_size",
    "gqa_decode_layer", "gqa_meanpool_kv",
    "gqa_status_string", "gqa_last_hip_error", "gqa_decode_kernel_kind", "gqa_stream_read", "gqa_tuning_reload",
]

_lib = None


class GQAError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        msg = "%s failed: %s (%s)" % (where, STATUS_NAMES.get(status, status), status_string(status))
        if status == 7:
            msg += ": " + load_library().gqa_last_hip_error().decode()
        super().__init__(msg)


def library_path() -> str:
    return _LIB_PATH


def load_library(path: str | None = None):
    """Load libgqa.so (raises if it has not been built)."""
    global _lib
    if _lib is not None and path is None:
        return _lib
    p = path or _LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError("libgqa.so not found at %s; build it with `python -m grouped_query_kv_decode_amd.build`" % p)
    lib = ctypes.CDLL(p)
    vp, ci, sz = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t
    lib.gqa_decode_workspace_size.restype = sz
    lib.gqa_decode_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.gqa_workspace_init.restype = ci
    lib.gqa_workspace_init.argtypes = [vp, sz, vp]
    lib.gqa_decode_phase.restype = ci
    lib.gqa_decode_phase.argtypes = [ci, vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp, vp, sz, vp]
    lib.gqa_decode.restype = ci
    lib.gqa_decode.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp, vp, sz, vp]
    lib.gqa_decode_noalloc.restype = ci
    lib.gqa_decode_noalloc.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp, vp]
    lib.gqa_decode_window.restype = ci
    lib.gqa_decode_window.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp, vp, sz, vp]
    lib.gqa_decode_append.restype = ci
    lib.gqa_decode_append.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp, vp, sz,
                                      vp]
    lib.gqa_linear_workspace_size.restype = sz
    lib.gqa_linear_workspace_size.argtypes = [ci, ci, ci, ci]
    lib.gqa_linear.restype = ci
    lib.gqa_linear.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp, sz, vp]
    lib.gqa_pack_weight.restype = ci
    lib.gqa_pack_weight.argtypes = [vp, vp, ci, ci, ci, vp]
    lib.gqa_linear_packed.restype = ci
    lib.gqa_linear_packed.argtypes = [vp, vp, vp, ci, ci, ci, ci, vp]
    lib.gqa_decode_layer_workspace_size.restype = sz
    lib.gqa_decode_layer_workspace_size.argtypes = [ci, ci, ci, ci, ci, ci, ci, ci]
    lib.gqa_decode_layer.restype = ci
    lib.gqa_decode_layer.argtypes = [vp, vp, vp, vp, vp, vp, ci, ci, ci, ci, ci, ci, ci, ctypes.c_float, ci, vp, vp,
                                     sz, vp]
    lib.gqa_meanpool_kv.restype = ci
    lib.gqa_meanpool_kv.argtypes = [vp, ci, ci, ci, ci, vp, vp]
    lib.gqa_status_string.restype = ctypes.c_char_p
    lib.gqa_status_string.argtypes = [ci]
    lib.gqa_last_hip_error.restype = ctypes.c_char_p
    lib.gqa_last_hip_error.argtypes = []
    lib.gqa_decode_kernel_kind.restype = ci
    lib.gqa_decode_kernel_kind.argtypes = [ci, ci, ci, ci, ci, ci]
    lib.gqa_stream_read.restype = ci
    lib.gqa_stream_read.argtypes = [vp, sz, ci, ci, vp, vp]
    lib.gqa_tuning_reload.restype = None
    lib.gqa_tuning_reload.argtypes = []
    if path is None:
        _lib = lib
    return lib


def tuning_reload() -> None:
    """Re-read the GQA_* launch-plan overrides from the environment (the
    library reads them once when it loads; see include/gqa_measure.h)."""
    load_library().gqa_tuning_reload()


def status_string(status: int) -> str:
    return load_library().gqa_status_string(int(status)).decode()


def _dtype_code(dt) -> int:
    import torch
    if dt == torch.float32:
        return GQA_F32
    if dt == torch.bfloat16:
        return GQA_BF16
    raise TypeError("unsupported dtype %s (float32 or bfloat16)" % dt)


def _stream_handle(device) -> int:
    import torch
    return torch.cuda.current_stream(device).cuda_stream


def decode_workspace_size(B, H, G, d, Lmax, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().gqa_decode_workspace_size(B, H, G, d, Lmax, code))


def decode_kernel_kind(B, H, G, d, Lmax, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().gqa_decode_kernel_kind(B, H, G, d, Lmax, code))


def workspace_init(workspace) -> None:
    """Clear a workspace (uint8 tensor) before its first use."""
    st = load_library().gqa_workspace_init(workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                           _stream_handle(workspace.device))
    if st:
        raise GQAError(st, "gqa_workspace_init")


# One cleared workspace per (device, stream), grown on demand.
_ws_cache: dict = {}


def _workspace_for(nbytes: int, device):
    import torch
    key = (device.index, _stream_handle(device))
    ws = _ws_cache.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        workspace_init(ws)
        _ws_cache[key] = ws
    return ws


def _prepare(q, k_cache, v_cache, seq_lens, scale, out, workspace, window=0, no_workspace=False):
    """Checks the tensors and returns (ctypes argument tuple without the stream, out, workspace)."""
    import torch
    B, H, d = q.shape
    Bk, G, Lmax, dk = k_cache.shape
    if Bk != B or dk != d or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("shape mismatch: q %s, k %s, v %s" % (tuple(q.shape), tuple(k_cache.shape), tuple(v_cache.shape)))
    if not (q.dtype == k_cache.dtype == v_cache.dtype):
        raise TypeError("q, k_cache and v_cache must share one dtype")
    if seq_lens.dtype != torch.int32 or tuple(seq_lens.shape) != (B,):
        raise TypeError("seq_lens must be int32 of shape [B]")
    for name, t in (("q", q), ("k_cache", k_cache), ("v_cache", v_cache), ("seq_lens", seq_lens)):
        if not t.is_contiguous():
            raise ValueError("%s must be contiguous" % name)
        if t.device != q.device or t.device.type != "cuda":
            raise ValueError("%s must be on the GPU of q" % name)
    code = _dtype_code(q.dtype)
    if out is None:
        out = torch.empty((B, H, d), dtype=q.dtype, device=q.device)
    elif tuple(out.shape) != (B, H, d) or out.dtype != q.dtype or not out.is_contiguous() or out.device != q.device:
        raise ValueError("out must be a contiguous [B,H,d] tensor of q's dtype on q's GPU")
    need = 0 if no_workspace else decode_workspace_size(B, H, G, d, min(Lmax, window) if window > 0 else Lmax, code)
    if workspace is None and need > 0:
        workspace = _workspace_for(need, q.device)
    ws_ptr = workspace.data_ptr() if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    args = (q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(), seq_lens.data_ptr(), B, H, G, d, Lmax,
            float(scale), code, out.data_ptr(), ws_ptr, ws_bytes)
    return args, out, workspace


def decode(q, k_cache, v_cache, seq_lens, scale: float, out=None, workspace=None):
    """out[B,H,d] = grouped-query decode attention (see include/gqa.h).

    q [B,H,d], k_cache/v_cache [B,G,Lmax,d] (float32 or bfloat16, one dtype,
    contiguous, on one GPU), seq_lens [B] int32 on the same GPU.  Enqueued on
    torch's current stream.
    """
    args, out, _ = _prepare(q, k_cache, v_cache, seq_lens, scale, out, workspace)
    st = load_library().gqa_decode(*args, _stream_handle(q.device))
    if st:
        raise GQAError(st, "gqa_decode")
    return out


def decode_noalloc(q, k_cache, v_cache, seq_lens, scale: float, out=None):
    """decode() without a workspace: the library's per-device scratch holds the
    split partials (gqa_decode_noalloc; for callers that cannot allocate).
    Calls on one GPU must not overlap in time."""
    import torch
    if out is None:
        out = torch.empty(q.shape, dtype=q.dtype, device=q.device)
    args, out, _ = _prepare(q, k_cache, v_cache, seq_lens, scale, out, None, no_workspace=True)
    st = load_library().gqa_decode_noalloc(*args[:12], _stream_handle(q.device))
    if st:
        raise GQAError(st, "gqa_decode_noalloc")
    return out


def decode_phase(phase: int, q, k_cache, v_cache, seq_lens, scale: float, out=None, workspace=None):
    """One phase of decode (1: split kernel, 2: merge kernel, 0: both); see gqa.h."""
    args, out, _ = _prepare(q, k_cache, v_cache, seq_lens, scale, out, workspace)
    st = load_library().gqa_decode_phase(int(phase), *args, _stream_handle(q.device))
    if st:
        raise GQAError(st, "gqa_decode_phase")
    return out


def decode_window(q, k_cache, v_cache, seq_lens, scale: float, window: int, out=None, workspace=None):
    """Sliding-window decode: each sequence attends its last `window` positions."""
    args, out, _ = _prepare(q, k_cache, v_cache, seq_lens, scale, out, workspace, window=int(window))
    a = args[:9] + (int(window),) + args[9:]
    st = load_library().gqa_decode_window(*a, _stream_handle(q.device))
    if st:
        raise GQAError(st, "gqa_decode_window")
    return out


def _check_new(k_new, v_new, k_cache):
    B, G, _, d = k_cache.shape
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if tuple(t.shape) != (B, G, d) or t.dtype != k_cache.dtype or not t.is_contiguous() \
                or t.device != k_cache.device:
            raise ValueError("%s must be a contiguous [B,G,d] tensor of the cache dtype on its GPU" % name)


def decode_append(q, k_new, v_new, k_cache, v_cache, seq_lens, scale: float, window: int = 0, out=None,
                  workspace=None):
    """Write k_new/v_new [B,G,d] at position seq_lens[b]-1 of the caches (in
    place), then decode over the updated caches (window > 0: sliding window)."""
    _check_new(k_new, v_new, k_cache)
    args, out, _ = _prepare(q, k_cache, v_cache, seq_lens, scale, out, workspace, window=int(window))
    a = (args[0], k_new.data_ptr(), v_new.data_ptr()) + args[1:9] + (int(window),) + args[9:]
    st = load_library().gqa_decode_append(*a, _stream_handle(q.device))
    if st:
        raise GQAError(st, "gqa_decode_append")
    return out


class Decoder:
    """A decode call bound to fixed tensors and to the stream current at
    construction; each call() is one C-ABI call with pre-marshalled
    arguments (for tight loops: serving steps, benchmarks)."""

    def __init__(self, q, k_cache, v_cache, seq_lens, scale: float, out=None, workspace=None, window: int = 0,
                 k_new=None, v_new=None):
        self._keep = (q, k_cache, v_cache, seq_lens, k_new, v_new)
        args, self.out, self.workspace = _prepare(q, k_cache, v_cache, seq_lens, scale, out, workspace,
                                                  window=int(window))
        stream = (_stream_handle(q.device),)
        lib = load_library()
        self._phase_args = args + stream
        if k_new is not None:
            _check_new(k_new, v_new, k_cache)
            self._fn, self._name = lib.gqa_decode_append, "gqa_decode_append"
            self._args = (args[0], k_new.data_ptr(), v_new.data_ptr()) + args[1:9] + (int(window),) + args[9:] + stream
        elif window > 0:
            self._fn, self._name = lib.gqa_decode_window, "gqa_decode_window"
            self._args = args[:9] + (int(window),) + args[9:] + stream
        else:
            self._fn, self._name = lib.gqa_decode, "gqa_decode"
            self._args = args + stream
        self._phase = lib.gqa_decode_phase
        self._plain = k_new is None and window <= 0

    def __call__(self):
        st = self._fn(*self._args)
        if st:
            raise GQAError(st, self._name)
        return self.out

    def phase(self, phase: int):
        if not self._plain:
            raise ValueError("phases are available for plain decode only")
        st = self._phase(phase, *self._phase_args)
        if st:
            raise GQAError(st, "gqa_decode_phase")
        return self.out


def linear_workspace_size(M, K, N, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().gqa_linear_workspace_size(M, K, N, code))


def _check_dev(name, t, ref, shape, dtype):
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or not t.is_contiguous() or t.device != ref.device \
            or t.device.type != "cuda":
        raise ValueError("%s must be a contiguous %s %s tensor on %s" % (name, list(shape), dtype, ref.device))


def _ws_args(need, device, workspace):
    if workspace is None and need > 0:
        workspace = _workspace_for(need, device)
    if workspace is None:
        return None, 0, None
    return workspace.data_ptr(), workspace.numel() * workspace.element_size(), workspace


def linear(x, w, out=None, workspace=None):
    """y[M,N] = x[M,K] @ w[K,N] in bfloat16 (binary32 sums, rounded once)."""
    import torch
    M, K = x.shape
    N = w.shape[1]
    _check_dev("x", x, x, (M, K), torch.bfloat16)
    _check_dev("w", w, x, (K, N), torch.bfloat16)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check_dev("out", out, x, (M, N), torch.bfloat16)
    ws_ptr, ws_bytes, _ = _ws_args(linear_workspace_size(M, K, N, GQA_BF16), x.device, workspace)
    st = load_library().gqa_linear(x.data_ptr(), w.data_ptr(), out.data_ptr(), M, K, N, GQA_BF16, ws_ptr, ws_bytes,
                                   _stream_handle(x.device))
    if st:
        raise GQAError(st, "gqa_linear")
    return out


def pack_weight(w, out=None):
    """w [K, N] bfloat16 (row-major, on the GPU) in the packed matrix-core
    layout of gqa_pack_weight (a flat tensor of the same size)."""
    import torch
    K, N = w.shape
    _check_dev("w", w, w, (K, N), torch.bfloat16)
    if out is None:
        out = torch.empty(K * N, dtype=torch.bfloat16, device=w.device)
    _check_dev("out", out, w, (K * N,), torch.bfloat16)
    st = load_library().gqa_pack_weight(w.data_ptr(), out.data_ptr(), K, N, GQA_BF16, _stream_handle(w.device))
    if st:
        raise GQAError(st, "gqa_pack_weight")
    return out


def linear_packed(x, w_packed, N: int, out=None):
    """y[M,N] = x[M,K] @ W with W given packed (pack_weight)."""
    import torch
    M, K = x.shape
    _check_dev("x", x, x, (M, K), torch.bfloat16)
    _check_dev("w_packed", w_packed, x, (K * N,), torch.bfloat16)
    if out is None:
        out = torch.empty((M, N), dtype=x.dtype, device=x.device)
    _check_dev("out", out, x, (M, N), torch.bfloat16)
    st = load_library().gqa_linear_packed(x.data_ptr(), w_packed.data_ptr(), out.data_ptr(), M, K, N, GQA_BF16,
                                          _stream_handle(x.device))
    if st:
        raise GQAError(st, "gqa_linear_packed")
    return out


def decode_layer_workspace_size(B, H, G, d, Lmax, window, d_model, dtype) -> int:
    code = dtype if isinstance(dtype, int) else _dtype_code(dtype)
    return int(load_library().gqa_decode_layer_workspace_size(B, H, G, d, Lmax, window, d_model, code))


class LayerStep:
    """The full decode step (projections, cache append, attention, output
    projection; gqa_decode_layer) bound to fixed tensors; each call runs on
    torch's current stream.  w_qkv [d_model, (H+2G)d] and w_o [H d, d_model]
    are row-major; they are packed once here (pack_weight)."""

    def __init__(self, x, w_qkv, w_o, k_cache, v_cache, seq_lens, H: int, G: int, scale: float, window: int = 0,
                 out=None, workspace=None):
        import torch
        B, d_model = x.shape
        Bk, Gk, Lmax, d = k_cache.shape
        if Bk != B or Gk != G or H % G:
            raise ValueError("shape mismatch: x %s, k_cache %s, H=%d, G=%d" % (tuple(x.shape), tuple(k_cache.shape),
                                                                               H, G))
        bf = torch.bfloat16
        _check_dev("x", x, x, (B, d_model), bf)
        _check_dev("w_qkv", w_qkv, x, (d_model, (H + 2 * G) * d), bf)
        _check_dev("w_o", w_o, x, (H * d, d_model), bf)
        _check_dev("k_cache", k_cache, x, (B, G, Lmax, d), bf)
        _check_dev("v_cache", v_cache, x, (B, G, Lmax, d), bf)
        _check_dev("seq_lens", seq_lens, x, (B,), torch.int32)
        if out is None:
            out = torch.empty((B, d_model), dtype=bf, device=x.device)
        _check_dev("out", out, x, (B, d_model), bf)
        need = decode_layer_workspace_size(B, H, G, d, Lmax, int(window), d_model, GQA_BF16)
        if need == 0 and B > 0:
            raise GQAError(3, "gqa_decode_layer_workspace_size")
        ws_ptr, ws_bytes, self.workspace = _ws_args(need, x.device, workspace)
        self.out = out
        self.w_qkv_packed = pack_weight(w_qkv)
        self.w_o_packed = pack_weight(w_o)
        self._keep = (x, k_cache, v_cache, seq_lens)
        self._fn = load_library().gqa_decode_layer
        self._args = (x.data_ptr(), self.w_qkv_packed.data_ptr(), self.w_o_packed.data_ptr(), k_cache.data_ptr(),
                      v_cache.data_ptr(),
                      seq_lens.data_ptr(), B, H, G, d, Lmax, int(window), d_model, float(scale), GQA_BF16,
                      out.data_ptr(), ws_ptr, ws_bytes)
        self._device = x.device

    def __call__(self):
        """One step, enqueued on torch's current stream (so it can be
        captured into a graph)."""
        st = self._fn(*self._args, _stream_handle(self._device))
        if st:
            raise GQAError(st, "gqa_decode_layer")
        return self.out


def decode_layer(x, w_qkv, w_o, k_cache, v_cache, seq_lens, H: int, G: int, scale: float, window: int = 0,
                 out=None, workspace=None):
    """y[B, d_model] = one decode step of a GQA attention layer (see LayerStep;
    the row-major weights are packed on every call - bind a LayerStep to pack
    them once); the caches receive the new token's keys and values in place."""
    return LayerStep(x, w_qkv, w_o, k_cache, v_cache, seq_lens, H, G, scale, window, out, workspace)()


def meanpool_kv(w, H: int, G: int, out=None):
    """w_out[d_model, G*h] = per-group mean of the head column blocks of w[d_model, H*h] (float32)."""
    import torch
    if w.dtype != torch.float32 or w.dim() != 2 or not w.is_contiguous() or w.device.type != "cuda":
        raise ValueError("w must be a contiguous float32 [d_model, H*h] tensor on the GPU")
    d_model, cols = w.shape
    if H < 1 or cols % H:
        raise ValueError("w has %d columns, not a multiple of H=%d" % (cols, H))
    h = cols // H
    if out is None:
        out = torch.empty((d_model, G * h), dtype=torch.float32, device=w.device)
    st = load_library().gqa_meanpool_kv(w.data_ptr(), d_model, H, G, h, out.data_ptr(), _stream_handle(w.device))
    if st:
        raise GQAError(st, "gqa_meanpool_kv")
    return out


def stream_read(buf, nontemporal: bool = True, grid: int = 0, sink=None):
    """Read every byte of the GPU tensor `buf` once (16-byte loads,
    non-temporal by default) on `grid` workgroups (0: 2048): the read-ceiling
    probe.  Returns `sink` (one int32 on the GPU), written only when a
    thread's xor fold of its pieces equals 0x12345678."""
    import torch
    if buf.device.type != "cuda" or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous tensor on the GPU")
    if sink is None:
        sink = torch.zeros(1, dtype=torch.int32, device=buf.device)
    st = load_library().gqa_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), int(bool(nontemporal)),
                                        int(grid), sink.data_ptr(), _stream_handle(buf.device))
    if st:
        raise GQAError(st, "gqa_stream_read")
    return sink
