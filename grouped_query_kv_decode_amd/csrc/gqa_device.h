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
  unsigned *ws_cnt;        // arrival counter per unit; zero between calls
  const int *order;        // item of each workgroup (largest work first), or null: item = blockIdx
  int fused;               // 1: the last split of a unit merges; 0: a merge kernel follows
  int contig;              // matrix-core kernel: contiguous per-wave tile runs instead of interleaved tiles
  int arrive_acqrel;       // the arrival counter's increment with release/acquire ordering (agent scope)
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

// Max / sum over the four lanes l, l^16, l^32, l^48 (the lane groups of one
// matrix-core output column: one head in the decode kernels).
__device__ __forceinline__ float group_max(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group_sum(float x) {
  auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
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
__device__ __forceinline__ bool arrive_last(unsigned *counter, int nsplit, bool acq_rel = false) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned prev =
        acq_rel ? __hip_atomic_fetch_add(counter, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT)
                : __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const int last = prev == (unsigned)(nsplit - 1);
    if (last) __hip_atomic_store(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

// Log-sum-exp merge of the nsplit partials of heads head0 .. head0+nh-1 of
// sequence b into out.  Each item is one head and 4 output dimensions; its
// splits are taken in index order and folded into a running (max, weight
// sum, output) with rescaling when the max grows.  The loads of a batch of
// splits are issued together, and a thread with two items issues both
// items' loads before folding either, so a merge of up to 8 splits costs one
// memory round trip even when the items outnumber the threads (64 heads of
// 64 dimensions on 256 threads: 2.4 -> ~1.2 us).  Deterministic; the
// separate merge kernel calls this same routine.
template <typename T, int D, int kItems, int kBatch>
__device__ __forceinline__ void merge_pass(const DecodeParams &p, int b, int head0, int nsplit, int idx0, int total) {
  float M[kItems], L[kItems], o[kItems][4];
  size_t hs[kItems];
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int idx = idx0 + k * (int)blockDim.x;
    hs[k] = ((size_t)b * p.H + head0 + (idx < total ? idx : 0) / (D / 4)) * p.S;
    M[k] = kNegInf;
    L[k] = 0.f;
    o[k][0] = o[k][1] = o[k][2] = o[k][3] = 0.f;
  }
  for (int s0 = 0; s0 < nsplit; s0 += kBatch) {
    float2 h[kItems][kBatch], x[kItems][kBatch], y[kItems][kBatch];
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
      const int idx = idx0 + k * (int)blockDim.x;
      const int c = (idx % (D / 4)) * 4;
      const float *ml = reinterpret_cast<const float *>(p.ws_ml + hs[k]);
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (idx < total && s0 + i < nsplit) {
          h[k][i] = load_pair(ml + 2 * (s0 + i));
          x[k][i] = load_pair(p.ws_o + (hs[k] + s0 + i) * D + c);
          y[k][i] = load_pair(p.ws_o + (hs[k] + s0 + i) * D + c + 2);
        }
      }
    }
#pragma unroll
    for (int k = 0; k < kItems; ++k) {
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (idx0 + k * (int)blockDim.x < total && s0 + i < nsplit) {
          const float mn = fmaxf(M[k], h[k][i].x);
          const float sh = safe_shift(mn);
          const float a_old = fast_exp2(M[k] - sh), a = fast_exp2(h[k][i].x - sh);
          M[k] = mn;
          L[k] = L[k] * a_old + h[k][i].y * a;
          o[k][0] = o[k][0] * a_old + x[k][i].x * a;
          o[k][1] = o[k][1] * a_old + x[k][i].y * a;
          o[k][2] = o[k][2] * a_old + y[k][i].x * a;
          o[k][3] = o[k][3] * a_old + y[k][i].y * a;
        }
      }
    }
  }
#pragma unroll
  for (int k = 0; k < kItems; ++k) {
    const int idx = idx0 + k * (int)blockDim.x;
    if (idx < total) {
      const int j = idx / (D / 4), c = (idx % (D / 4)) * 4;
      const float inv = 1.f / L[k];
      Store<T>::four(p.out, ((size_t)b * p.H + head0 + j) * D + c, o[k][0] * inv, o[k][1] * inv, o[k][2] * inv,
                     o[k][3] * inv);
    }
  }
}

template <typename T, int D>
__device__ void merge_heads(const DecodeParams &p, int b, int head0, int nh, int nsplit) {
  const int total = nh * (D / 4);
  const int stride = (int)blockDim.x;
  if (total <= stride) {
    if ((int)threadIdx.x < total) merge_pass<T, D, 1, 16>(p, b, head0, nsplit, threadIdx.x, total);
    return;
  }
  for (int idx = threadIdx.x; idx < total; idx += 2 * stride) merge_pass<T, D, 2, 8>(p, b, head0, nsplit, idx, total);
}

// Host-side launchers (one per kernel translation unit).
// one_piece (tuning): a 16-byte piece per lane and row also where the plan takes two.
hipError_t launch_decode_valu(const DecodeParams &p, int dtype, int D, int RC, int one_piece, unsigned grid,
                              hipStream_t stream);
// nontemporal: the cache stream's loads are non-temporal (plain loads when
// head chunks read the same lines; four head blocks always stream).
hipError_t launch_decode_mfma(const DecodeParams &p, int D, int HB, int NW, int nontemporal, unsigned grid,
                              hipStream_t stream);
// binary32 on the matrix cores: one head block of up to 16 heads per workgroup
hipError_t launch_decode_mfma_f32(const DecodeParams &p, int D, int nontemporal, unsigned grid, hipStream_t stream);
hipError_t launch_merge(const DecodeParams &p, int dtype, int D, int heads_per_unit, hipStream_t stream);
hipError_t launch_merge_wide(const DecodeParams &p, int dtype, int D, hipStream_t stream);
hipError_t launch_order(const DecodeParams &p, bool valu_layout, unsigned grid, int *order, hipStream_t stream);
hipError_t launch_meanpool(const float *w, int d_model, int H, int G, int h, float *w_out, hipStream_t stream);
hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t stream);
hipError_t launch_stream_read(const void *buf, size_t bytes, bool nontemporal, unsigned grid, unsigned *sink,
                              hipStream_t stream);

}  // namespace gqa
