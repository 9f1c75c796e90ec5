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

__global__ __launch_bounds__(256) void meanpool_kernel(const float *__restrict__ w, int H, int G, int h,
                                                       size_t total, float *__restrict__ w_out) {
  const size_t idx = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  const int col = (int)(idx % ((size_t)G * h));  // output column g*h + c
  const size_t row = idx / ((size_t)G * h);
  const int g = col / h, c = col % h;
  const int r = H / G;
  const float *wr = w + row * (size_t)H * h;
  double acc = (double)wr[(size_t)(g * r) * h + c];
  for (int i = g * r + 1; i < g * r + r; ++i) acc += (double)wr[(size_t)i * h + c];
  w_out[idx] = (float)(acc / (double)r);
}

}  // namespace

hipError_t launch_meanpool(const float *w, int d_model, int H, int G, int h, float *w_out, hipStream_t stream) {
  const size_t total = (size_t)d_model * G * h;
  if (total == 0) return hipSuccess;
  const size_t blocks = (total + 255) / 256;
  hipLaunchKernelGGL(meanpool_kernel, dim3((unsigned)blocks), dim3(256), 0, stream, w, H, G, h, total, w_out);
  return hipGetLastError();
}

}  // namespace gqa
