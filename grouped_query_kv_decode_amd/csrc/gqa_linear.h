// Launchers of the projection kernels (y = x @ W, bfloat16): row-major W
// with a k split across workgroups, and W in the packed matrix-core layout.
#pragma once
#include "gqa_device.h"

namespace gqa {

// Projection y[M, N] = x[M, K] @ W[K, N] (bfloat16, row-major).
struct LinearParams {
  const __bf16 *x;   // [M, K]
  const __bf16 *w;   // [K, N]
  __bf16 *y[3];      // output segments (see seg_lo)
  int seg_lo[4];     // output column c in [seg_lo[s], seg_lo[s+1]) goes to y[s], row stride seg_lo[s+1]-seg_lo[s]
  int nseg;
  float *ws_part;    // [KS, M, N] k-split partial sums
  unsigned *ws_cnt;  // arrival counter per 128-column block; zero between calls
  int M, K, N;
  int KS;            // k splits
  int ksteps_per_split;  // 32-row steps per split
};

hipError_t launch_linear(const LinearParams &p, int NW, int TPI, unsigned grid, hipStream_t stream);
// tb: token tiles (1, 2 or 4); sw: strips per workgroup; nch: chunks of
// linear_packed_chunk_blocks(tb, sw) k-blocks unrolled at compile time (K must
// then equal nch chunks), 0 for the loop over any K.
hipError_t launch_linear_packed(const LinearParams &p, int tb, int sw, int nch, hipStream_t stream);
int linear_packed_chunk_blocks(int tb, int sw);
hipError_t launch_pack_weight(const void *w, void *w_packed, int K, int N, hipStream_t stream);

}  // namespace gqa
