// Log-sum-exp merge of context-split partials into the decode output, as
// separate kernels (used when the in-kernel merge is off, and beyond 32
// splits per sequence), and the workspace fill kernel.
//
// A split s of head h leaves (m_s, l_s, o_s): the maximum of its scores in
// log2 units, the sum of exp2(score - m_s) over its positions, and the
// un-normalised weighted sum of its value rows.  With M = max_s m_s,
//   out = sum_s exp2(m_s - M) o_s / sum_s exp2(m_s - M) l_s,
// which is the plain softmax-weighted sum of the decode-step block on the
// wikillm page "Grouped-query attention (GQA)" (Implementation sketch) taken
// over all positions of all splits.
#include "gqa_device.h"

namespace gqa {
namespace {

// One workgroup per (sequence, head range of one split workgroup), using the
// same routine as the in-kernel merge: identical arithmetic, same order.
template <typename T, int D>
__global__ __launch_bounds__(256) void merge_kernel(DecodeParams p, int heads_per_unit) {
  const int units_per_b = p.H / heads_per_unit;
  const int b = blockIdx.x / units_per_b;
  const int head0 = (blockIdx.x % units_per_b) * heads_per_unit;
  const int n = clamp_len(p, b);
  const int nsplit = num_splits(n - window_lo(p, n), p.chunk);
  if (nsplit <= 1) return;  // written directly by the split kernel
  merge_heads<T, D>(p, b, head0, heads_per_unit, nsplit);
}

// Many splits (up to 256 per sequence, for few and long sequences): one
// workgroup per (sequence, head, 32 output dimensions), 256 threads = 8 groups
// of 4 dimensions x 32 slices of consecutive splits.  Each thread combines its
// slice; the slices are then combined in slice order through LDS, so the
// result is deterministic, and no thread reads more than ceil(nsplit / 32)
// partials (one batch of loads at 256 splits).
struct Fold {
  float M = kNegInf, L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  __device__ __forceinline__ void add(float m, float l, float x0, float x1, float x2, float x3) {
    const float mn = fmaxf(M, m);
    const float sh = safe_shift(mn);
    const float a_old = fast_exp2(M - sh), a = fast_exp2(m - sh);
    M = mn;
    L = L * a_old + l * a;
    o0 = o0 * a_old + x0 * a;
    o1 = o1 * a_old + x1 * a;
    o2 = o2 * a_old + x2 * a;
    o3 = o3 * a_old + x3 * a;
  }
};

template <typename T, int D>
__global__ __launch_bounds__(256) void merge_wide_kernel(DecodeParams p) {
  constexpr int kSlices = 32, kBatch = 16;
  const int bh = blockIdx.x / (D / 32);  // b * H + head
  const int b = bh / p.H;
  const int n = clamp_len(p, b);
  const int nsplit = num_splits(n - window_lo(p, n), p.chunk);
  if (nsplit <= 1) return;  // written directly by the split kernel
  const int q = threadIdx.x & 7, k = threadIdx.x >> 3;
  const int c = (blockIdx.x % (D / 32)) * 32 + 4 * q;
  const int per = (nsplit + kSlices - 1) / kSlices;
  const int first = k * per;
  const int cnt = min(per, nsplit - first);
  const float *ml = reinterpret_cast<const float *>(p.ws_ml + (size_t)bh * p.S);
  const float *o = p.ws_o + (size_t)bh * p.S * D + c;
  Fold f;
  if (cnt <= kBatch) {
    // One batch (every plan of at most 512 splits): the slice's maximum
    // first, then its weighted sums, whose exp2 terms are independent (the
    // running fold below chains two exp2 per split).
    float2 h[kBatch], x[kBatch], y[kBatch];
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < cnt) {
        const int s = first + i;
        h[i] = load_pair(ml + 2 * s);
        x[i] = load_pair(o + (size_t)s * D);
        y[i] = load_pair(o + (size_t)s * D + 2);
      }
    }
#pragma unroll
    for (int i = 0; i < kBatch; ++i)
      if (i < cnt) f.M = fmaxf(f.M, h[i].x);
    const float sh = safe_shift(f.M);
#pragma unroll
    for (int i = 0; i < kBatch; ++i) {
      if (i < cnt) {
        const float a = fast_exp2(h[i].x - sh);
        f.L += h[i].y * a;
        f.o0 += x[i].x * a;
        f.o1 += x[i].y * a;
        f.o2 += y[i].x * a;
        f.o3 += y[i].y * a;
      }
    }
  } else {
    for (int i0 = 0; i0 < cnt; i0 += kBatch) {
      float2 h[kBatch], x[kBatch], y[kBatch];
#pragma unroll
      for (int i = 0; i < kBatch; ++i) {
        if (i0 + i < cnt) {
          const int s = first + i0 + i;
          h[i] = load_pair(ml + 2 * s);
          x[i] = load_pair(o + (size_t)s * D);
          y[i] = load_pair(o + (size_t)s * D + 2);
        }
      }
#pragma unroll
      for (int i = 0; i < kBatch; ++i)
        if (i0 + i < cnt) f.add(h[i].x, h[i].y, x[i].x, x[i].y, y[i].x, y[i].y);
    }
  }
  __shared__ float sm[kSlices][8][6];
  float *e = sm[k][q];
  e[0] = f.M;
  e[1] = f.L;
  e[2] = f.o0;
  e[3] = f.o1;
  e[4] = f.o2;
  e[5] = f.o3;
  __syncthreads();
  if (k != 0) return;
  // The slices in slice order, again maximum first, then the weighted sums.
  const int used = min(kSlices, (nsplit + per - 1) / per);
  float M = kNegInf;
  for (int kk = 0; kk < used; ++kk) M = fmaxf(M, sm[kk][q][0]);
  const float sh = safe_shift(M);
  float L = 0.f, o0 = 0.f, o1 = 0.f, o2 = 0.f, o3 = 0.f;
  for (int kk = 0; kk < used; ++kk) {
    const float *v = sm[kk][q];
    const float a = fast_exp2(v[0] - sh);
    L += v[1] * a;
    o0 += v[2] * a;
    o1 += v[3] * a;
    o2 += v[4] * a;
    o3 += v[5] * a;
  }
  const float inv = 1.f / L;
  Store<T>::four(p.out, (size_t)bh * D + c, o0 * inv, o1 * inv, o2 * inv, o3 * inv);
}

template <typename T>
hipError_t launch_t(const DecodeParams &p, int D, int heads_per_unit, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)p.B * (p.H / heads_per_unit));
  if (D == 64)
    hipLaunchKernelGGL((merge_kernel<T, 64>), dim3(grid), dim3(256), 0, stream, p, heads_per_unit);
  else
    hipLaunchKernelGGL((merge_kernel<T, 128>), dim3(grid), dim3(256), 0, stream, p, heads_per_unit);
  return hipGetLastError();
}

__global__ __launch_bounds__(256) void fill_zero_kernel(uint4 *p, size_t n16, unsigned char *tail, size_t ntail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n16) p[i] = make_uint4(0u, 0u, 0u, 0u);
  if (i < ntail) tail[i] = 0;
}

}  // namespace

hipError_t launch_merge(const DecodeParams &p, int dtype, int D, int heads_per_unit, hipStream_t stream) {
  return dtype == 0 ? launch_t<float>(p, D, heads_per_unit, stream) : launch_t<__bf16>(p, D, heads_per_unit, stream);
}

hipError_t launch_merge_wide(const DecodeParams &p, int dtype, int D, hipStream_t stream) {
  const unsigned grid = (unsigned)((size_t)p.B * p.H * (D / 32));
  if (dtype == 0) {
    if (D == 64)
      hipLaunchKernelGGL((merge_wide_kernel<float, 64>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_wide_kernel<float, 128>), dim3(grid), dim3(256), 0, stream, p);
  } else {
    if (D == 64)
      hipLaunchKernelGGL((merge_wide_kernel<__bf16, 64>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((merge_wide_kernel<__bf16, 128>), dim3(grid), dim3(256), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  const size_t n = n16 > ntail ? n16 : ntail;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<uint4 *>(ptr), n16, static_cast<unsigned char *>(ptr) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace gqa
