"""Per-phase timeline of a matrix-core decode call (measurement only).

    python -m grouped_query_kv_decode_amd.timeline build     # on any machine (hipcc cross-compiles)
    python bench.py --timeline                               # on the GPU

build() copies the library sources, inserts wall-clock stamps into the two
matrix-core decode kernels (bfloat16 and binary32) and links the copy as
libgqa_timeline.so next to libgqa.so.  The stamps are s_memrealtime reads (a constant 100 MHz counter
shared by the whole GPU) stored by lane 0 of each wave of the first 8192
workgroups: kernel entry, first tile multiplied, tile loop done, output or
partial stores issued, arrival ticket taken, end (after the merge for the
workgroup that merges); the instrumented kernel is otherwise the product
kernel, so the phases are those of a real call (the stamps add ~2 us).

run() times steady-state calls: ten calls back to back over rotated inputs,
stamps from the last one, medians over 30 such groups.  Phases are in
microseconds from the first wave's start.
"""
from __future__ import annotations

import concurrent.futures
import ctypes
import json
import math
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
LIB = os.path.join(PKG, "libgqa_timeline.so")
_SLOTS = 8192 * 4 * 8

# (anchor, replacement) per kernel source: each anchor must occur once.  The
# two kernels are separate code objects, so each gets its own stamp buffer
# and reader.


def _stamps(buf, tp, merge_call, pv_end):
    return [
        ("namespace gqa {\nnamespace {\n",
         "__device__ unsigned long long %s[8192 * 4 * 8];\n" % buf +
         "namespace gqa {\nnamespace {\n"
         "__device__ __forceinline__ void tl_put(int e, unsigned long long v) {\n"
         "  if ((threadIdx.x & 63) == 0 && blockIdx.x < 8192 && (threadIdx.x >> 6) < 4)\n"
         "    %s[(blockIdx.x * 4 + (threadIdx.x >> 6)) * 8 + e] = v;\n" % buf +
         "}\n"
         "__device__ __forceinline__ void tl_stamp(int e) { tl_put(e, __builtin_amdgcn_s_memrealtime()); }\n"),
        ("  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;\n  const int c = lane >> 4, nn = lane & 15;\n",
         "  tl_stamp(0);\n  tl_put(4, 0);\n  tl_put(6, 0);\n"
         "  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;\n  const int c = lane >> 4, nn = lane & 15;\n"
         "  bool tl_first = false;\n"),
        (pv_end + "\n  };",
         pv_end + "\n    if (!tl_first) {\n      tl_first = true;\n      tl_stamp(1);\n    }\n  };"),
        (tp, tp + "  tl_stamp(2);\n"),
        ("  if (nsplit == 1 || !p.fused) return;\n"
         "  if (!arrive_last(p.ws_cnt + ((size_t)b * p.G + g) * p.HC + hc, nsplit, p.arrive_acqrel)) return;\n"
         "  " + merge_call,
         "  tl_stamp(3);\n"
         "  if (nsplit == 1 || !p.fused) {\n    tl_stamp(5);\n    return;\n  }\n"
         "  const bool tl_last = arrive_last(p.ws_cnt + ((size_t)b * p.G + g) * p.HC + hc, nsplit, p.arrive_acqrel);\n"
         "  tl_stamp(4);\n"
         "  if (!tl_last) {\n    tl_stamp(5);\n    return;\n  }\n"
         "  " + merge_call + "\n"
         "  __builtin_amdgcn_s_waitcnt(0);\n  tl_stamp(5);\n  tl_put(6, 1);"),
    ]


_KERNELS = [  # (source, stamp buffer, reader)
    ("gqa_decode_mfma.hip", "tl_buf", "gqa_timeline_read",
     _stamps("tl_buf", "  for (int hb = 0; hb < HB; ++hb) l[hb] = group_sum(l[hb]);\n",
             "merge_heads<__bf16, D>(p, b, head0, rw, nsplit);", "    pv_steps<0, DB, HB>(o, T.vR, pB);")),
    ("gqa_decode_mfma_f32.hip", "tl_buf_f32", "gqa_timeline_read_f32",
     _stamps("tl_buf_f32", "  l_run = group_sum(l_run);\n", "merge_heads<float, D>(p, b, head0, rw, nsplit);",
             "        for (int e = 0; e < 4; ++e) o[4 * m + e] = mfma4(T.vR[i][m][e], pw[i], o[4 * m + e]);")),
]
_READER = """
extern "C" int %s(void *host, size_t bytes) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(%s), bytes, 0, hipMemcpyDeviceToHost);
}
"""


def build(verbose: bool = True) -> str:
    """Instrumented copy of the sources -> libgqa_timeline.so (beside libgqa.so)."""
    from . import build as b
    work = os.path.join(b.BUILD_DIR, "timeline")
    csrc = os.path.join(work, "csrc")
    shutil.rmtree(work, ignore_errors=True)
    shutil.copytree(b.CSRC, csrc)
    for name, buf, reader, stamps in _KERNELS:
        path = os.path.join(csrc, name)
        src = open(path).read()
        for anchor, repl in stamps:
            if src.count(anchor) != 1:
                raise RuntimeError("timeline: anchor not found once in %s: %r" % (name, anchor[:60]))
            src = src.replace(anchor, repl)
        with open(path, "w") as f:
            f.write(src + _READER % (reader, buf))
    def compile_one(item):
        name, extra = item
        obj = os.path.join(work, os.path.splitext(name)[0] + ".o")
        cmd = [b.HIPCC, *[c for c in b.COMMON if not c.startswith("-I")], "-I" + b.INCLUDE, "-I" + csrc, *extra,
               "-c", os.path.join(csrc, name), "-o", obj]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError("hipcc failed for %s:\n%s" % (name, res.stderr))
        return obj

    with concurrent.futures.ThreadPoolExecutor(max_workers=min(8, len(b.SOURCES))) as ex:
        objs = list(ex.map(compile_one, b.SOURCES))
    tmp = LIB + ".tmp%d" % os.getpid()
    subprocess.run([b.HIPCC, "--offload-arch=" + b.ARCH, "-shared", "-fPIC", *objs, "-o", tmp], check=True)
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


def _phases(st, tick_us):
    """Phase figures (us from the first wave's start) of one call's stamps [wg, wave, event]."""
    import numpy as np
    used = st[:, :, 0].max(axis=1) > 0
    s = st[used]
    t0 = s[:, :, 0][s[:, :, 0] > 0].min()
    rel = lambda x: (x - t0) * tick_us
    first = s[:, :, 1]
    lend = s[:, :, 2].max(axis=1)
    pub = s[:, :, 3].max(axis=1)
    tick = s[:, :, 4].max(axis=1)
    merger = s[:, 0, 6] == 1
    arr = (tick[tick > 0] - pub[tick > 0]) * tick_us if (tick > 0).any() else np.zeros(1)
    mdur = ((s[merger][:, :, 5].max(axis=1) - s[merger][:, :, 4].min(axis=1)) * tick_us if merger.any()
            else np.zeros(1))
    return dict(workgroups=int(used.sum()), launch_spread=float(rel(s[:, :, 0].min(axis=1)).max()),
                first_tile_p50=float(np.median(rel(first[first > 0]))), first_tile_max=float(rel(first[first > 0]).max()),
                loop_end_p10=float(np.percentile(rel(lend[lend > 0]), 10)),
                loop_end_p50=float(np.median(rel(lend[lend > 0]))), loop_end_max=float(rel(lend[lend > 0]).max()),
                stores_issued_max=float(rel(pub[pub > 0]).max()), arrival_p50=float(np.median(arr)),
                merge_p50=float(np.median(mdur)), mergers=int(merger.sum()),
                end=float(rel(s[:, :, 5].max(axis=1)).max()))


def run(cases, tick_us: float = 0.01, groups: int = 30):
    """cases: [(workload name, window)].  Prints and returns one dict per case."""
    import numpy as np
    import torch
    import grouped_query_kv_decode_amd as gqa
    from grouped_query_kv_decode_amd import workloads as wl
    if not os.path.exists(LIB):
        raise RuntimeError("%s not built: python -m grouped_query_kv_decode_amd.timeline build" % LIB)
    lib = gqa.load_library(LIB)
    for _, _, reader, _ in _KERNELS:
        getattr(lib, reader).argtypes = [ctypes.c_void_p, ctypes.c_size_t]
    saved = gqa._lib
    gqa._lib = lib
    host = np.zeros(_SLOTS, dtype=np.uint64)
    dev = torch.device("cuda:0")
    results = []
    try:
        for name, window in cases:
            w = wl.WORKLOADS[name]
            code = gqa.GQA_F32 if w.dtype == "f32" else gqa.GQA_BF16
            if gqa.decode_kernel_kind(w.B, w.H, w.G, w.d, w.Lmax, code) != 1:
                raise RuntimeError("timeline: %s does not run on a matrix-core kernel" % name)
            read = lib.gqa_timeline_read_f32 if w.dtype == "f32" else lib.gqa_timeline_read
            kvb = 2 * w.B * w.G * w.Lmax * w.d * (4 if w.dtype == "f32" else 2)
            rot = min(64, max(1, math.ceil((1 << 30) / kvb)))
            decs = [gqa.Decoder(*wl.make_inputs(w, dev, pad="none", seed_offset=i), w.scale, window=window)
                    for i in range(rot)]
            for i in range(20):
                decs[i % rot]()
            torch.cuda.synchronize()
            rows = []
            for it in range(groups):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record()
                for j in range(10):
                    decs[(it * 10 + j) % rot]()
                e1.record()
                torch.cuda.synchronize()
                if read(host.ctypes.data, host.nbytes) != 0:
                    raise RuntimeError("timeline read failed")
                ph = _phases(host.reshape(8192, 4, 8).astype(np.int64), tick_us)
                ph["call_us"] = e0.elapsed_time(e1) * 1e3 / 10
                rows.append(ph)
            agg = {k: float(np.median([r[k] for r in rows])) for k in rows[0]}
            agg.update(mode="timeline", workload=name, window=window, groups=groups)
            print(json.dumps(agg), flush=True)
            results.append(agg)
            del decs
            torch.cuda.empty_cache()
    finally:
        gqa._lib = saved
    return results


if __name__ == "__main__":
    if len(sys.argv) > 1 and sys.argv[1] == "build":
        build()
    else:
        print(__doc__)
