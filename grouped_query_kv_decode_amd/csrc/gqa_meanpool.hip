// Grouped mean-pool of K/V projection columns (the checkpoint conversion of
// the wikillm page "Grouped-query attention (GQA)", Implementation sketch,
// conversion block; Variants, "Converted and uptrained checkpoints").
//
// This translation unit is compiled with -ffp-contract=off.  Each output is
// the binary64 sum of the group's members in ascending head order (starting
// from the first member), divided once by r in binary64 (IEEE division) and
// rounded once to binary32 - a fixed sequence of correctly rounded
// operations, so the result is bit-reproducible.
#include "gqa_device.h"

namespace gqa {
namespace {

// V consecutive output columns per thread (V = 4: 16-byte loads and stores,
// when h % 4 == 0 and the pointers are 16-byte aligned; else V = 1).  The
// members' loads are issued kBatch at a time before they are added; each
// element still takes exactly the sequence above.
template <int V>
__global__ __launch_bounds__(256) void meanpool_kernel(const float *__restrict__ w, int H, int G, int h,
                                                       size_t total_v, float *__restrict__ w_out) {
  typedef float fv __attribute__((ext_vector_type(V)));
  constexpr int kBatch = 8;
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total_v) return;
  const size_t cols_v = (size_t)G * h / V;
  const int col = (int)(idx % cols_v) * V;  // first output column g*h + c
  const size_t row = idx / cols_v;
  const int g = col / h, c = col % h;
  const int r = H / G;
  const float *wr = w + row * (size_t)H * h + c;
  double acc[V];
  {
    const fv first = stream_load(reinterpret_cast<const fv *>(wr + (size_t)(g * r) * h));
#pragma unroll
    for (int e = 0; e < V; ++e) acc[e] = (double)first[e];
  }
  for (int i0 = 1; i0 < r; i0 += kBatch) {
    fv m[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (i0 + j < r) m[j] = stream_load(reinterpret_cast<const fv *>(wr + (size_t)(g * r + i0 + j) * h));
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (i0 + j < r) {
#pragma unroll
        for (int e = 0; e < V; ++e) acc[e] += (double)m[j][e];
      }
  }
  fv o;
#pragma unroll
  for (int e = 0; e < V; ++e) o[e] = (float)(acc[e] / (double)r);
  *reinterpret_cast<fv *>(w_out + idx * V) = o;
}

}  // namespace

hipError_t launch_meanpool(const float *w, int d_model, int H, int G, int h, float *w_out, hipStream_t stream) {
  const size_t total = (size_t)d_model * G * h;
  if (total == 0) return hipSuccess;
  const bool vec = h % 4 == 0 && (uintptr_t)w % 16 == 0 && (uintptr_t)w_out % 16 == 0;
  const size_t total_v = vec ? total / 4 : total;
  const size_t blocks = (total_v + 255) / 256;
  if (vec)
    hipLaunchKernelGGL(meanpool_kernel<4>, dim3((unsigned)blocks), dim3(256), 0, stream, w, H, G, h, total_v, w_out);
  else
    hipLaunchKernelGGL(meanpool_kernel<1>, dim3((unsigned)blocks), dim3(256), 0, stream, w, H, G, h, total_v, w_out);
  return hipGetLastError();
}

}  // namespace gqa
