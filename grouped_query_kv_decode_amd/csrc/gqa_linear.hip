// Projections of the decode step on the matrix cores (bfloat16, gfx950):
// y[M, N] = x[M, K] @ W[K, N], one row of x per token (M <= 64 tokens), W
// row-major - the q = x@Wq, key = x@Wk, val = x@Wv and y = out@Wo products of
// the decode-step block on the wikillm page "Grouped-query attention (GQA)"
// (Implementation sketch).  With a handful of tokens the product is bound by
// reading W once, so W is streamed with coalesced 16-byte loads.
//
// MFMA v_mfma_f32_16x16x32_bf16 computes y^T = W^T . x^T: the A operand needs
// 8 consecutive k of one output column per lane, while W is contiguous along
// the columns.  Lane (c, n) loads rows k+8c .. k+8c+7, columns 8n .. 8n+7 of a
// 32 x 128 block (four full 256-byte rows per load instruction) and transposes
// the 8x8 block in registers; MFMA number db then produces columns 8m + db,
// m = 0..15.  The B operand is x, 8 consecutive k per lane straight from
// memory.  A workgroup owns 128 output columns and a range of k; its waves take
// 32-row steps in turn and are summed through LDS in wave order; k-split
// partials are summed in split order by the workgroup that finishes its
// column block last (same arrival protocol as the decode kernel), so the
// result is deterministic.
#include "gqa_device.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

template <int E>
__device__ __forceinline__ u32x4 column(const u32x4 *rows) {
  constexpr unsigned sel = (E & 1) ? 0x07060302u : 0x05040100u;
  u32x4 a;
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = __builtin_amdgcn_perm(rows[2 * k + 1][E >> 1], rows[2 * k][E >> 1], sel);
  return a;
}

// Output columns [seg_lo[s], seg_lo[s+1]) go to y[s] with row stride
// seg_lo[s+1] - seg_lo[s] (a fused projection can write q, key and value into
// three separate tensors).
__device__ __forceinline__ __bf16 *out_ptr(const LinearParams &p, int row, int col) {
  int s = 0;
  if (p.nseg > 1 && col >= p.seg_lo[1]) s = 1;
  if (p.nseg > 2 && col >= p.seg_lo[2]) s = 2;
  const int w = p.seg_lo[s + 1] - p.seg_lo[s];
  return p.y[s] + (size_t)row * w + (col - p.seg_lo[s]);
}

template <int TB, int NW>
__global__ __launch_bounds__(64 * NW) void linear_mfma(LinearParams p) {
  constexpr int kCols = 128;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4, nn = lane & 15;
  const int ntile = p.N / kCols;
  const int tile = blockIdx.x % ntile;
  const int ks = blockIdx.x / ntile;
  const int col0 = tile * kCols;
  const int kstep_total = p.K / 32;
  const int kstep0 = ks * p.ksteps_per_split;
  const int kstep1 = min(kstep_total, kstep0 + p.ksteps_per_split);

  f32x4 acc[TB][8];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb)
#pragma unroll
    for (int db = 0; db < 8; ++db) acc[tb][db] = f32x4{0.f, 0.f, 0.f, 0.f};

  const __bf16 *wl = p.w + (size_t)(8 * c) * p.N + col0 + 8 * nn;  // lane's first row / column
  for (int st = kstep0 + wave; st < kstep1; st += NW) {
    const int k = st * 32;
    u32x4 wR[8];
    const __bf16 *wk = wl + (size_t)k * p.N;
#pragma unroll
    for (int u = 0; u < 8; ++u) wR[u] = *reinterpret_cast<const u32x4 *>(wk + (size_t)u * p.N);
    u32x4 xB[TB];
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) {
      const int row = tb * 16 + nn;
      xB[tb] = row < p.M ? *reinterpret_cast<const u32x4 *>(p.x + (size_t)row * p.K + k + 8 * c)
                         : u32x4{0u, 0u, 0u, 0u};
    }
#define GQA_LIN_STEP(DB)                                                              \
  {                                                                                   \
    const u32x4 a = column<DB>(wR);                                                   \
    _Pragma("unroll") for (int tb = 0; tb < TB; ++tb) acc[tb][DB] = mfma(a, xB[tb], acc[tb][DB]); \
  }
    GQA_LIN_STEP(0) GQA_LIN_STEP(1) GQA_LIN_STEP(2) GQA_LIN_STEP(3)
    GQA_LIN_STEP(4) GQA_LIN_STEP(5) GQA_LIN_STEP(6) GQA_LIN_STEP(7)
#undef GQA_LIN_STEP
  }

  // Sum the waves in wave order through LDS: sm[token][column].
  constexpr int LD = kCols + 4;
  __shared__ float sm[TB * 16 * LD];
  for (int w = 0; w < NW; ++w) {
    if (wave == w) {
#pragma unroll
      for (int tb = 0; tb < TB; ++tb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int db = 0; db < 8; ++db) {
            float *e = sm + (tb * 16 + nn) * LD + 8 * (4 * c + i) + db;
            *e = w == 0 ? acc[tb][db][i] : *e + acc[tb][db][i];
          }
    }
    __syncthreads();
  }

  // One k split: round and store.  Several: device-scope partials, and the
  // last workgroup of the column block sums them in split order.
  const int rows = p.M;
  if (p.KS == 1) {
    for (int idx = threadIdx.x; idx < rows * kCols; idx += blockDim.x) {
      const int row = idx / kCols, col = idx % kCols;
      *out_ptr(p, row, col0 + col) = (__bf16)sm[row * LD + col];
    }
    return;
  }
  for (int idx = threadIdx.x * 4; idx < rows * kCols; idx += blockDim.x * 4) {
    const int row = idx / kCols, col = idx % kCols;
    const float *e = sm + row * LD + col;
    store_partial4(p.ws_part + ((size_t)ks * p.M + row) * p.N + col0 + col, e[0], e[1], e[2], e[3]);
  }
  if (!arrive_last(p.ws_cnt + tile, p.KS)) return;
  for (int idx = threadIdx.x * 2; idx < rows * kCols; idx += blockDim.x * 2) {
    const int row = idx / kCols, col = idx % kCols;
    float s0 = 0.f, s1 = 0.f;
    for (int s = 0; s < p.KS; ++s) {
      const float2 v = load_pair(p.ws_part + ((size_t)s * p.M + row) * p.N + col0 + col);
      s0 += v.x;
      s1 += v.y;
    }
    *out_ptr(p, row, col0 + col) = (__bf16)s0;
    *out_ptr(p, row, col0 + col + 1) = (__bf16)s1;
  }
}

template <int TB>
hipError_t launch_tb(const LinearParams &p, int NW, unsigned grid, hipStream_t stream) {
  if (NW == 8)
    hipLaunchKernelGGL((linear_mfma<TB, 8>), dim3(grid), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((linear_mfma<TB, 4>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_linear(const LinearParams &p, int NW, unsigned grid, hipStream_t stream) {
  switch ((p.M + 15) / 16) {
    case 1: return launch_tb<1>(p, NW, grid, stream);
    case 2: return launch_tb<2>(p, NW, grid, stream);
    case 3:
    case 4: return launch_tb<4>(p, NW, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
