// Device-side pieces shared by the decode kernels: launch parameters, the
// split-partial format, and the in-kernel merge of split partials.
//
// Decode semantics follow the decode-step block of the Implementation sketch
// on the wikillm page "Grouped-query attention (GQA)": per query head, softmax
// of the scaled scores against the keys of its group's K/V head, then the
// probability-weighted sum of that head's value rows.  The softmax is taken
// online over tiles and across context splits; merging (m, l, o) partials with
// weights exp2(m_s - max_s m_s) gives the same quotient as the plain softmax.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

struct DecodeParams {
  const void *q;           // [B, H, D]
  const void *k;           // [B, G, Lmax, D]
  const void *v;           // [B, G, Lmax, D]
  const void *k_new;       // [B, G, D] new token's keys (cache append), or null
  const void *v_new;       // [B, G, D] new token's values, or null
  const int32_t *seq_lens; // [B]
  void *out;               // [B, H, D]
  float *ws_o;             // [B, H, S, D]  un-normalised split outputs
  float2 *ws_ml;           // [B, H, S]     (running max in log2 units, sum of weights)
  float *ws_o1;            // [B, H, NG, D] group partials (more than kOneLevel splits)
  float2 *ws_ml1;          // [B, H, NG]
  unsigned *ws_cnt;        // arrival counters; zero between calls: [0, units) per unit, then
                           // NG per unit for the groups when NG > 0
  int NG;                  // split groups per unit: 0 when S <= kOneLevel
  int fused;               // 1: the last split of a unit merges; 0: a merge kernel follows
  int contig;              // matrix-core kernel: contiguous per-wave tile runs instead of interleaved tiles
  int B, H, G, Lmax;
  int window;              // > 0: attend only the last `window` positions
  int r;                   // query heads per K/V head, H / G
  int S;                   // splits per (b, g) in the grid
  int chunk;               // positions per split
  int HC;                  // head chunks per (b, g) in the grid (VALU kernel: RC heads each;
                           // matrix-core kernel: its HB head blocks of 16 each)
  float scale_log2;        // scale * log2(e): scores are kept in log2 units
};


constexpr float kLog2e = 1.44269504088896340736f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// A load of data that is read once (KV cache, weights): non-temporal, so it
// streams through the caches without displacing data that is reused.
template <typename V>
__device__ __forceinline__ V stream_load(const V *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ uint4 stream_load(const uint4 *p) {
  typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));
  const u32x4_t v = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t *>(p));
  return make_uint4(v[0], v[1], v[2], v[3]);
}

// Shift used with a running maximum: keeps exp2(x - shift) free of
// (-inf) - (-inf) when nothing has been seen yet.
__device__ __forceinline__ float safe_shift(float m) { return m == kNegInf ? 0.f : m; }

__device__ __forceinline__ int clamp_len(const DecodeParams &p, int b) {
  int n = p.seq_lens[b];
  return n < 0 ? 0 : (n > p.Lmax ? p.Lmax : n);
}

__device__ __forceinline__ int num_splits(int n, int chunk) { return n > 0 ? (n + chunk - 1) / chunk : 1; }

// First attended position: 0, or len - window under a sliding window.  Splits
// cover [lo, len) from lo on.
__device__ __forceinline__ int window_lo(const DecodeParams &p, int n) {
  return (p.window > 0 && n > p.window) ? n - p.window : 0;
}

// Cache append (the decode-step block appends the new token's key and value,
// then attends): the workgroup whose split holds position n-1 writes the new
// row into the cache.  Threads 0 .. D*sizeof(T)/16-1 move 16 bytes each.
template <typename T, int D>
__device__ __forceinline__ void append_row(const DecodeParams &p, int b, int g, int n) {
  constexpr int kLanes = D * (int)sizeof(T) / 16;
  if ((int)threadIdx.x < kLanes) {
    const size_t src = ((size_t)b * p.G + g) * D + threadIdx.x * (16 / sizeof(T));
    const size_t dst = (((size_t)b * p.G + g) * (size_t)p.Lmax + (size_t)(n - 1)) * D + threadIdx.x * (16 / sizeof(T));
    *reinterpret_cast<uint4 *>(static_cast<T *>(const_cast<void *>(p.k)) + dst) =
        *reinterpret_cast<const uint4 *>(static_cast<const T *>(p.k_new) + src);
    *reinterpret_cast<uint4 *>(static_cast<T *>(const_cast<void *>(p.v)) + dst) =
        *reinterpret_cast<const uint4 *>(static_cast<const T *>(p.v_new) + src);
  }
}

template <typename T> struct Store;
template <> struct Store<float> {
  __device__ static void four(void *base, size_t idx, float a, float b, float c, float d) {
    *reinterpret_cast<float4 *>(static_cast<float *>(base) + idx) = make_float4(a, b, c, d);
  }
};
template <> struct Store<__bf16> {
  __device__ static void four(void *base, size_t idx, float a, float b, float c, float d) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
    bf16x4 v = {(__bf16)a, (__bf16)b, (__bf16)c, (__bf16)d};  // round to nearest even
    *reinterpret_cast<bf16x4 *>(static_cast<__bf16 *>(base) + idx) = v;
  }
};

// out[b, head0 .. head0+nh-1, :] = 0 (a sequence with no cached positions).
template <typename T, int D>
__device__ void write_zero_heads(const DecodeParams &p, int b, int head0, int nh) {
  for (int idx = threadIdx.x; idx < nh * (D / 4); idx += blockDim.x) {
    const int j = idx / (D / 4), c = (idx % (D / 4)) * 4;
    Store<T>::four(p.out, ((size_t)b * p.H + head0 + j) * D + c, 0.f, 0.f, 0.f, 0.f);
  }
}

// Split partials are written and read with device-scope (sc1) accesses: they
// are coherent across the XCDs' L2 caches without a cache write-back, so the
// arrival protocol below needs no release fence.
__device__ __forceinline__ void store_partial4(float *dst, float a, float b, float c, float d) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(dst),
                     (unsigned long long)__float_as_uint(a) | ((unsigned long long)__float_as_uint(b) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(dst + 2),
                     (unsigned long long)__float_as_uint(c) | ((unsigned long long)__float_as_uint(d) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_ml(float2 *dst, float m, float l) {
  __hip_atomic_store(reinterpret_cast<unsigned long long *>(dst),
                     (unsigned long long)__float_as_uint(m) | ((unsigned long long)__float_as_uint(l) << 32),
                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float2 load_pair(const float *src) {
  const unsigned long long v = __hip_atomic_load(reinterpret_cast<const unsigned long long *>(src), __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
  return make_float2(__uint_as_float((unsigned)v), __uint_as_float((unsigned)(v >> 32)));
}

// Called by every thread of a workgroup after it stored its split partial.
// Returns true (in all threads) in the workgroup that arrived last for its
// unit; that workgroup then merges.  Each thread waits for its own partial
// stores to complete before the barrier, so when the arrival count is seen
// every partial of the unit is visible to device-scope loads.  The last
// arrival resets the counter, so the counters are zero again at kernel end.
__device__ __forceinline__ bool arrive_last(unsigned *counter, int nsplit) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev = __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (unsigned)(nsplit - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

// Up to kOneLevel splits are merged in one fold by the last workgroup to
// arrive.  Beyond that they are merged in groups of kSplitGroup: the last
// arrival of each group folds the group into a group partial and the last
// group to finish folds those, so no workgroup reads more than kSplitGroup
// partials per head.  (At 32 splits one fold measured faster than two
// levels; allowing 256 splits, merged in two levels, took one 131072-position
// sequence of one K/V head from 70.7 to 22.3 us.)
constexpr int kOneLevel = 32;
constexpr int kSplitGroup = 16;

// Running log-sum-exp state of one head's four output dimensions.
struct Fold {
  float M = kNegInf, L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  // add a partial (max m, weight sum l, un-normalised output x, y)
  __device__ __forceinline__ void add(float2 ml, float2 x, float2 y) {
    const float mn = fmaxf(M, ml.x);
    const float sh = safe_shift(mn);
    const float a_old = fast_exp2(M - sh), a = fast_exp2(ml.x - sh);
    M = mn;
    L = L * a_old + ml.y * a;
    o0 = o0 * a_old + x.x * a;
    o1 = o1 * a_old + x.y * a;
    o2 = o2 * a_old + y.x * a;
    o3 = o3 * a_old + y.y * a;
  }
};

// Fold partials first .. first+n-1 (in index order) of one head's list:
// ml[i] and o[i * D + c .. +3].  Loads are issued sixteen at a time.
template <int D>
__device__ __forceinline__ void fold_range(Fold &f, const float2 *ml, const float *o, int c, int first, int n) {
  constexpr int kBatch = 16;
  for (int i0 = 0; i0 < n; i0 += kBatch) {
    float2 h[kBatch], x[kBatch], y[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i0 + i < n) {
        const int k = first + i0 + i;
        h[i] = load_pair(reinterpret_cast<const float *>(ml + k));
        x[i] = load_pair(o + (size_t)k * D + c);
        y[i] = load_pair(o + (size_t)k * D + c + 2);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (i0 + i < n) f.add(h[i], x[i], y[i]);
  }
}

template <typename T, int D>
__device__ __forceinline__ void store_out(const DecodeParams &p, int b, int head, int c, const Fold &f) {
  const float inv = 1.f / f.L;
  Store<T>::four(p.out, ((size_t)b * p.H + head) * D + c, f.o0 * inv, f.o1 * inv, f.o2 * inv, f.o3 * inv);
}

// Log-sum-exp merge of the nsplit partials of heads head0 .. head0+nh-1 of
// sequence b into out: one fold over the splits in index order, or, with
// more than kOneLevel splits, a fold of each group followed by a fold of
// the group results in group order - the arithmetic of the distributed
// merge below, so both give the same bits.  Deterministic; the separate
// merge kernel calls this same routine.
template <typename T, int D>
__device__ void merge_heads(const DecodeParams &p, int b, int head0, int nh, int nsplit) {
  for (int idx = threadIdx.x; idx < nh * (D / 4); idx += blockDim.x) {
    const int j = idx / (D / 4), c = (idx % (D / 4)) * 4;
    const size_t hs = ((size_t)b * p.H + head0 + j) * p.S;
    Fold f;
    if (nsplit <= kOneLevel) {
      fold_range<D>(f, p.ws_ml + hs, p.ws_o + hs * D, c, 0, nsplit);
    } else {
      for (int g0 = 0; g0 < nsplit; g0 += kSplitGroup) {
        Fold fg;
        fold_range<D>(fg, p.ws_ml + hs, p.ws_o + hs * D, c, g0, min(kSplitGroup, nsplit - g0));
        f.add(make_float2(fg.M, fg.L), make_float2(fg.o0, fg.o1), make_float2(fg.o2, fg.o3));
      }
    }
    store_out<T, D>(p, b, head0 + j, c, f);
  }
}

// After a workgroup has stored its split partial: the arrival protocol of
// the in-kernel merge.  Every workgroup of a unit calls this; the last one
// to arrive merges (two levels with more than kOneLevel splits: the last
// of each group folds the group into a group partial, the last group folds
// those).  unit = (b * G + g) * HC + hc.
template <typename T, int D>
__device__ void finish_splits(const DecodeParams &p, int b, size_t unit, int head0, int nh, int s, int nsplit) {
  if (nsplit <= kOneLevel) {
    if (!arrive_last(p.ws_cnt + unit, nsplit)) return;
    merge_heads<T, D>(p, b, head0, nh, nsplit);
    return;
  }
  const int gi = s / kSplitGroup;
  const int g0 = gi * kSplitGroup;
  const size_t units = (size_t)p.B * p.G * p.HC;
  if (!arrive_last(p.ws_cnt + units + unit * p.NG + gi, min(kSplitGroup, nsplit - g0))) return;
  for (int idx = threadIdx.x; idx < nh * (D / 4); idx += blockDim.x) {
    const int j = idx / (D / 4), c = (idx % (D / 4)) * 4;
    const size_t hs = ((size_t)b * p.H + head0 + j) * p.S;
    Fold fg;
    fold_range<D>(fg, p.ws_ml + hs, p.ws_o + hs * D, c, g0, min(kSplitGroup, nsplit - g0));
    const size_t hg = ((size_t)b * p.H + head0 + j) * p.NG + gi;
    store_partial4(p.ws_o1 + hg * D + c, fg.o0, fg.o1, fg.o2, fg.o3);
    if (c == 0) store_ml(p.ws_ml1 + hg, fg.M, fg.L);
  }
  const int ng = (nsplit + kSplitGroup - 1) / kSplitGroup;
  if (!arrive_last(p.ws_cnt + unit, ng)) return;
  for (int idx = threadIdx.x; idx < nh * (D / 4); idx += blockDim.x) {
    const int j = idx / (D / 4), c = (idx % (D / 4)) * 4;
    const size_t hg = ((size_t)b * p.H + head0 + j) * p.NG;
    Fold f;
    fold_range<D>(f, p.ws_ml1 + hg, p.ws_o1 + hg * D, c, 0, ng);
    store_out<T, D>(p, b, head0 + j, c, f);
  }
}

// Host-side launchers (one per kernel translation unit).
hipError_t launch_decode_valu(const DecodeParams &p, int dtype, int D, int RC, unsigned grid, hipStream_t stream);
hipError_t launch_decode_mfma(const DecodeParams &p, int D, int HB, int NW, unsigned grid, hipStream_t stream);
hipError_t launch_merge(const DecodeParams &p, int dtype, int D, int heads_per_unit, hipStream_t stream);
hipError_t launch_meanpool(const float *w, int d_model, int H, int G, int h, float *w_out, hipStream_t stream);
hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t stream);

}  // namespace gqa
