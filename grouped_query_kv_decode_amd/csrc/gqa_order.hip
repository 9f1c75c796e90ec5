// Dispatch order of the decode workgroups for grids that run in several
// rounds (more workgroups than the GPU holds at once).  The dispatcher hands
// workgroups out in blockIdx order as slots free up, so the last ones to
// start decide when the call ends; with ragged lengths, split-major order
// starts full-length splits of the longest sequences last.  This kernel
// sorts the items (split s, unit) by their number of attended positions,
// largest first (the classic longest-processing-time-first rule), and the
// decode kernels read their item from the result.  Only the schedule
// changes: every item's arithmetic, and the merge order of each unit's
// splits, stay the same, so outputs are bit-identical with and without it.
#include "gqa_device.h"

namespace gqa {
namespace {

constexpr int kClasses = 129;   // work sizes in 1/128ths of a split, 0 .. 128
constexpr int kStagedLens = 4096;  // lengths read once into LDS up to this batch size

// One workgroup of 1024 threads: counting sort of the grid's items by size
// class, largest first.  Whole splits (the first class) keep their index
// order - the split-major order that deals the units round-robin over the
// XCDs - through a stable compaction, so a batch of equal lengths gets the
// identity order; the smaller items follow by size, in any order within a
// class (LDS counters).
__global__ __launch_bounds__(1024) void order_kernel(DecodeParams p, bool valu_layout, unsigned grid, int *order) {
  __shared__ unsigned count[kClasses], cursor[kClasses];
  __shared__ unsigned wave_full[16], base_full;
  __shared__ int lens[kStagedLens];
  const unsigned bg = (unsigned)p.B * p.G;
  const unsigned units = bg * p.HC;
  const bool staged = p.B <= kStagedLens;
  for (int k = threadIdx.x; k < kClasses; k += blockDim.x) count[k] = 0;
  if (staged)
    for (int b = threadIdx.x; b < p.B; b += blockDim.x) lens[b] = clamp_len(p, b);
  __syncthreads();
  // key 0 = a whole split, kClasses-1 = no positions
  auto key_of = [&](unsigned item) {
    const int s = item / units;
    const unsigned rem = item % units;
    const int b = valu_layout ? (int)(rem / p.HC / p.G) : (int)((rem % bg) / p.G);
    const int n = staged ? lens[b] : clamp_len(p, b);
    const long m = (long)(n - window_lo(p, n)) - (long)s * p.chunk;
    const long size = m < 0 ? 0 : (m > p.chunk ? p.chunk : m);
    return (kClasses - 1) - (int)((size * (kClasses - 1) + p.chunk - 1) / p.chunk);
  };
  for (unsigned i = threadIdx.x; i < grid; i += blockDim.x) atomicAdd(&count[key_of(i)], 1u);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned acc = 0;
    for (int k = 0; k < kClasses; ++k) {
      cursor[k] = acc;
      acc += count[k];
    }
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  if (threadIdx.x == 0) base_full = 0;  // whole splits take positions [0, count[0])
  __syncthreads();
  for (unsigned i0 = 0; i0 < grid; i0 += blockDim.x) {
    const unsigned i = i0 + threadIdx.x;
    const int key = i < grid ? key_of(i) : -1;
    const unsigned long long full = __ballot(key == 0);
    if (lane == 0) wave_full[wave] = (unsigned)__popcll(full);
    __syncthreads();
    if (key == 0) {
      unsigned pos = base_full + (unsigned)__popcll(full & ((1ull << lane) - 1));
      for (int w = 0; w < wave; ++w) pos += wave_full[w];
      order[pos] = (int)i;
    } else if (key > 0) {
      order[atomicAdd(&cursor[key], 1u)] = (int)i;
    }
    __syncthreads();
    if (threadIdx.x == 0)
      for (int w = 0; w < 16; ++w) base_full += wave_full[w];
    __syncthreads();
  }
}

}  // namespace

hipError_t launch_order(const DecodeParams &p, bool valu_layout, unsigned grid, int *order, hipStream_t stream) {
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(1024), 0, stream, p, valu_layout, grid, order);
  return hipGetLastError();
}

}  // namespace gqa
