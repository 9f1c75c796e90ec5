// Log-sum-exp merge of context-split partials into the decode output, as a
// separate kernel (used when the in-kernel merge is off), and the workspace
// fill kernel.
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

hipError_t launch_fill_zero(void *ptr, size_t bytes, hipStream_t stream) {
  const size_t n16 = bytes / 16, ntail = bytes % 16;
  const size_t n = n16 > ntail ? n16 : ntail;
  if (n == 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, stream,
                     static_cast<uint4 *>(ptr), n16, static_cast<unsigned char *>(ptr) + n16 * 16, ntail);
  return hipGetLastError();
}

}  // namespace gqa
