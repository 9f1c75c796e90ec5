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
#include "gqa_linear.h"

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

// A wave's steps are kstep0 + wave + j*NW.  TPI steps are loaded before any
// is used (one memory round trip for all of them); a step past the split's
// end re-reads the split's last step (in bounds, from cache) and is skipped.
template <int TB, int NW, int TPI>
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
  for (int base = kstep0 + wave; base < kstep1; base += TPI * NW) {
    u32x4 wR[TPI][8];
    u32x4 xB[TPI][TB];
#pragma unroll
    for (int j = 0; j < TPI; ++j) {
      const int k = min(base + j * NW, kstep1 - 1) * 32;
      const __bf16 *wk = wl + (size_t)k * p.N;
#pragma unroll
      for (int u = 0; u < 8; ++u) wR[j][u] = stream_load(reinterpret_cast<const u32x4 *>(wk + (size_t)u * p.N));
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const int row = tb * 16 + nn;
        xB[j][tb] = row < p.M ? *reinterpret_cast<const u32x4 *>(p.x + (size_t)row * p.K + k + 8 * c)
                              : u32x4{0u, 0u, 0u, 0u};
      }
    }
#pragma unroll
    for (int j = 0; j < TPI; ++j) {
      if (base + j * NW >= kstep1) break;
#define GQA_LIN_STEP(DB)                                                                           \
  {                                                                                                \
    const u32x4 a = column<DB>(wR[j]);                                                             \
    _Pragma("unroll") for (int tb = 0; tb < TB; ++tb) acc[tb][DB] = mfma(a, xB[j][tb], acc[tb][DB]); \
  }
      GQA_LIN_STEP(0) GQA_LIN_STEP(1) GQA_LIN_STEP(2) GQA_LIN_STEP(3)
      GQA_LIN_STEP(4) GQA_LIN_STEP(5) GQA_LIN_STEP(6) GQA_LIN_STEP(7)
#undef GQA_LIN_STEP
    }
  }

  // Sum the waves in wave order through LDS into sm[token][column].  When
  // every wave's accumulator fits, all waves write their own slice and the
  // sum is read back in parallel after one barrier; otherwise the waves add
  // into one slice in turn.
  constexpr int LD = kCols + 4;
  constexpr bool kSlices = NW * TB * 16 * LD * 4 <= 64 * 1024;
  __shared__ float sm[(kSlices ? NW : 1) * TB * 16 * LD];
  if constexpr (kSlices) {
    float *mine = sm + wave * (TB * 16 * LD);
#pragma unroll
    for (int tb = 0; tb < TB; ++tb)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < 8; ++db) mine[(tb * 16 + nn) * LD + 8 * (4 * c + i) + db] = acc[tb][db][i];
    __syncthreads();
  } else {
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
  }
  // total of element (row, col) over the waves, in wave order
  auto total = [&](int row, int col) {
    float t = sm[row * LD + col];
    if constexpr (kSlices) {
#pragma unroll
      for (int w = 1; w < NW; ++w) t += sm[w * (TB * 16 * LD) + row * LD + col];
    }
    return t;
  };

  // One k split: round and store.  Several: device-scope partials, and the
  // last workgroup of the column block sums them in split order.
  const int rows = p.M;
  if (p.KS == 1) {
    for (int idx = threadIdx.x; idx < rows * kCols; idx += blockDim.x) {
      const int row = idx / kCols, col = idx % kCols;
      *out_ptr(p, row, col0 + col) = (__bf16)total(row, col);
    }
    return;
  }
  for (int idx = threadIdx.x * 4; idx < rows * kCols; idx += blockDim.x * 4) {
    const int row = idx / kCols, col = idx % kCols;
    store_partial4(p.ws_part + ((size_t)ks * p.M + row) * p.N + col0 + col, total(row, col), total(row, col + 1),
                   total(row, col + 2), total(row, col + 3));
  }
  if (!arrive_last(p.ws_cnt + tile, p.KS)) return;
  // Each thread sums kPairs column pairs; the loads of kBatch splits for all
  // of them are issued before the adds.
  constexpr int kPairs = 4, kBatch = 8;
  const int npairs = rows * kCols / 2;
  for (int base = threadIdx.x; base < npairs; base += blockDim.x * kPairs) {
    float2 sum[kPairs];
#pragma unroll
    for (int i = 0; i < kPairs; ++i) sum[i] = make_float2(0.f, 0.f);
    for (int s0 = 0; s0 < p.KS; s0 += kBatch) {
      float2 v[kPairs][kBatch];
#pragma unroll
      for (int i = 0; i < kPairs; ++i) {
        const int pr = base + i * blockDim.x;
        const int row = (2 * pr) / kCols, col = (2 * pr) % kCols;
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (pr < npairs && s0 + u < p.KS)
            v[i][u] = load_pair(p.ws_part + ((size_t)(s0 + u) * p.M + row) * p.N + col0 + col);
      }
#pragma unroll
      for (int i = 0; i < kPairs; ++i)
#pragma unroll
        for (int u = 0; u < kBatch; ++u)
          if (s0 + u < p.KS) {
            sum[i].x += v[i][u].x;
            sum[i].y += v[i][u].y;
          }
    }
#pragma unroll
    for (int i = 0; i < kPairs; ++i) {
      const int pr = base + i * blockDim.x;
      if (pr < npairs) {
        const int row = (2 * pr) / kCols, col = (2 * pr) % kCols;
        *out_ptr(p, row, col0 + col) = (__bf16)sum[i].x;
        *out_ptr(p, row, col0 + col + 1) = (__bf16)sum[i].y;
      }
    }
  }
}

template <int TB, int TPI>
hipError_t launch_tb(const LinearParams &p, int NW, unsigned grid, hipStream_t stream) {
  if constexpr (TB * TPI > 8) {  // does not fit the register file
    return hipErrorInvalidValue;
  } else if (NW == 8)
    hipLaunchKernelGGL((linear_mfma<TB, 8, TPI>), dim3(grid), dim3(512), 0, stream, p);
  else
    hipLaunchKernelGGL((linear_mfma<TB, 4, TPI>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int TPI>
hipError_t launch_tpi(const LinearParams &p, int NW, unsigned grid, hipStream_t stream) {
  switch ((p.M + 15) / 16) {
    case 1: return launch_tb<1, TPI>(p, NW, grid, stream);
    case 2: return launch_tb<2, TPI>(p, NW, grid, stream);
    case 3:
    case 4: return launch_tb<4, TPI>(p, NW, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_linear(const LinearParams &p, int NW, int TPI, unsigned grid, hipStream_t stream) {
  switch (TPI) {
    case 1: return launch_tpi<1>(p, NW, grid, stream);
    case 2: return launch_tpi<2>(p, NW, grid, stream);
    case 4: return launch_tpi<4>(p, NW, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
