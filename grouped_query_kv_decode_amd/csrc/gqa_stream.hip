// Streaming-read probe: the practical HBM read ceiling that the decode
// kernels are measured against (a kernel that only reads, with the same
// 16-byte loads).  Every thread reads 16-byte pieces of the buffer
// grid-stride and folds them with xor; one word is written only if a
// thread's fold equals a fixed value, so no read can be dropped.
#include "gqa_device.h"

namespace gqa {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr unsigned kSentinel = 0x12345678u;

template <bool NT>
__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4 *__restrict__ p, size_t n16, unsigned *sink) {
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  unsigned acc = 0;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n16; i += stride) {
    u32x4 v;
    if constexpr (NT)
      v = __builtin_nontemporal_load(p + i);
    else
      v = p[i];
    acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
  }
  if (acc == kSentinel) sink[0] = acc;
}

}  // namespace

hipError_t launch_stream_read(const void *buf, size_t bytes, bool nontemporal, unsigned grid, unsigned *sink,
                              hipStream_t stream) {
  const u32x4 *p = static_cast<const u32x4 *>(buf);
  if (nontemporal)
    hipLaunchKernelGGL((stream_read_kernel<true>), dim3(grid), dim3(256), 0, stream, p, bytes / 16, sink);
  else
    hipLaunchKernelGGL((stream_read_kernel<false>), dim3(grid), dim3(256), 0, stream, p, bytes / 16, sink);
  return hipGetLastError();
}

}  // namespace gqa
