// Projections of the decode step over weights packed for the matrix cores
// (bfloat16, gfx950): y[M, N] = x[M, K] @ W[K, N], M <= 64 tokens - the
// q = x Wq, key = x Wk, val = x Wv and output products of the decode-step
// block on the wikillm page "Grouped-query attention (GQA)" (Implementation
// sketch).
//
// Packed layout (written once by pack_kernel; weights are constants of the
// model): W is cut into 32 x 16 blocks, block (kb, nb) holding rows
// 32kb .. 32kb+31 and columns 16nb .. 16nb+15.  Inside a block, lane
// l = 16c + n of a wave finds its v_mfma_f32_16x16x32_bf16 A operand - the 8
// values W[32kb + 8c + e][16nb + n], e = 0..7 - as 16 contiguous bytes at
// byte 16 l, so one wave-wide 16-byte load fetches one 1 KiB block and feeds
// one MFMA with no data movement.  Blocks are ordered k first (kb slow, nb
// fast): the workgroups, one per strip, start together on neighbouring
// blocks and move down the rows together, so at any moment the GPU reads one
// contiguous band of W (a plain streaming pattern); strip-contiguous order
// would have every workgroup reading at the same offset of its own strip, a
// fixed stride apart.
//
// Kernel: one workgroup per 16-column strip streams the strip over all of K
// (no split of k, so no partial sums leave the workgroup); its waves take
// blocks in turn, TPI at a time with all loads issued before the first MFMA,
// and are summed through LDS in wave order.  x, the B operand, is small and
// every workgroup reads all of it (from L2), staged through LDS.
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

// y[row][col .. col+3] for the segment holding col (segments start at
// multiples of 16, so four consecutive columns never straddle two).
__device__ __forceinline__ void store4(const LinearParams &p, int row, int col, f32x4 v) {
  int s = 0;
  if (p.nseg > 1 && col >= p.seg_lo[1]) s = 1;
  if (p.nseg > 2 && col >= p.seg_lo[2]) s = 2;
  const int w = p.seg_lo[s + 1] - p.seg_lo[s];
  __bf16 *dst = p.y[s] + (size_t)row * w + (col - p.seg_lo[s]);
  typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
  bf16x4 o;
  o[0] = (__bf16)v[0];
  o[1] = (__bf16)v[1];
  o[2] = (__bf16)v[2];
  o[3] = (__bf16)v[3];
  *reinterpret_cast<bf16x4 *>(dst) = o;
}

template <int TB, int NW, int TPI, int PD>
__global__ __launch_bounds__(64 * NW) void linear_packed(LinearParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4, nn = lane & 15;
  const int nb = blockIdx.x;
  const int kblocks = p.K / 32;
  // lane's 16 bytes of block (kb = 0) of this strip; blocks of a strip are N/16 KiB apart
  const int nstrips = p.N / 16;
  const __bf16 *wl = p.w + (size_t)nb * 512 + lane * 8;

  // x is staged through LDS a chunk of KC blocks (KC*32 values of k) at a
  // time: read from memory as whole row segments, then each lane takes its
  // B operand (token nn, 8 values of k) from LDS.  Read straight from memory
  // the operand would touch 16 half-used cache lines per wave-wide load.
  // Software pipeline: while chunk i is multiplied, x of chunk i+1 and the
  // weights of chunks i+1 .. i+PD-1 are in flight (PD register sets for the
  // weights, two LDS buffers for x, one barrier per chunk).
  constexpr int KC = NW * TPI;
  constexpr int ROWB = KC * 64 + 16;         // bytes per token row (+16: spreads the LDS banks)
  constexpr int PPR = KC * 4;                // 16-byte pieces per row
  constexpr int XPT = (TB * 16 * PPR + 64 * NW - 1) / (64 * NW);  // pieces per thread
  constexpr int BUFB = TB * 16 * ROWB;
  __shared__ __attribute__((aligned(16))) unsigned char xs[2 * BUFB];

  f32x4 acc[TB];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) acc[tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  auto load_x = [&](u32x4 (&xr)[XPT], int kb0) {
    const int nkb = min(KC, kblocks - kb0);
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + i * 64 * NW;
      const int row = idx / PPR, pc = idx % PPR;
      xr[i] = (row < p.M && pc < nkb * 4)
                  ? *reinterpret_cast<const u32x4 *>(p.x + (size_t)row * p.K + kb0 * 32 + pc * 8)
                  : u32x4{0u, 0u, 0u, 0u};
    }
  };
  // this wave's weight blocks of a chunk; past the end: re-read the last
  // block (in bounds), skipped in the products
  auto load_w = [&](u32x4 (&a)[TPI], int kb0) {
#pragma unroll
    for (int j = 0; j < TPI; ++j) {
      const int kb = min(kb0 + wave + j * NW, kblocks - 1);
      a[j] = stream_load(reinterpret_cast<const u32x4 *>(wl + (size_t)kb * nstrips * 512));
    }
  };
  auto store_x = [&](const u32x4 (&xr)[XPT], unsigned char *buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + i * 64 * NW;
      const int row = idx / PPR, pc = idx % PPR;
      if (row < TB * 16) *reinterpret_cast<u32x4 *>(buf + row * ROWB + pc * 16) = xr[i];
    }
  };
  auto products = [&](const u32x4 (&a)[TPI], const unsigned char *buf, int kb0) {
    const int nkb = min(KC, kblocks - kb0);
#pragma unroll
    for (int j = 0; j < TPI; ++j) {
      const int kl = wave + j * NW;  // block within the chunk
      if (kl >= nkb) break;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const u32x4 b = *reinterpret_cast<const u32x4 *>(buf + (tb * 16 + nn) * ROWB + (kl * 32 + 8 * c) * 2);
        acc[tb] = mfma(a[j], b, acc[tb]);
      }
    }
  };

  u32x4 xr[XPT], a[PD][TPI];
  load_x(xr, 0);
#pragma unroll
  for (int d = 0; d < PD - 1; ++d)
    if (d * KC < kblocks) load_w(a[d], d * KC);
  int buf = 0;
  for (int kb0 = 0; kb0 < kblocks; kb0 += PD * KC) {
#pragma unroll
    for (int ph = 0; ph < PD; ++ph) {
      const int kc = kb0 + ph * KC;  // this chunk; its weights are in a[ph]
      if (kc >= kblocks) break;
      store_x(xr, xs + buf * BUFB);
      if (kc + KC < kblocks) load_x(xr, kc + KC);
      if (kc + (PD - 1) * KC < kblocks) load_w(a[(ph + PD - 1) % PD], kc + (PD - 1) * KC);
      __syncthreads();
      products(a[ph], xs + buf * BUFB, kc);
      buf ^= 1;
    }
  }

  // acc[tb][i] of lane (c, nn) = y[token tb*16 + nn][column 16nb + 4c + i]
  // of this wave's blocks.  Sum the waves in wave order.
  __shared__ f32x4 sm[NW > 1 ? NW - 1 : 1][TB][64];
  if (wave > 0) {
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) sm[wave - 1][tb][lane] = acc[tb];
  }
  __syncthreads();
  if (wave != 0) return;
#pragma unroll
  for (int w = 1; w < NW; ++w)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[tb] += sm[w - 1][tb][lane];
#pragma unroll
  for (int tb = 0; tb < TB; ++tb) {
    const int row = tb * 16 + nn;
    if (row < p.M) store4(p, row, nb * 16 + 4 * c, acc[tb]);
  }
}

// One thread per 16-byte group of the packed layout: gathers W[32kb+8c+e][16nb+n].
__global__ __launch_bounds__(256) void pack_kernel(const __bf16 *__restrict__ w, __bf16 *__restrict__ wp, int K, int N) {
  const size_t g = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t groups = (size_t)K * N / 8;
  if (g >= groups) return;
  const int l = (int)(g % 64);
  const size_t blk = g / 64;
  const int nstrips = N / 16;
  const int nb = (int)(blk % nstrips), kb = (int)(blk / nstrips);
  const int c = l >> 4, n = l & 15;
  const __bf16 *src = w + (size_t)(32 * kb + 8 * c) * N + 16 * nb + n;
  typedef unsigned short u16x8 __attribute__((ext_vector_type(8)));
  u16x8 v;
#pragma unroll
  for (int e = 0; e < 8; ++e) v[e] = __builtin_bit_cast(unsigned short, src[(size_t)e * N]);
  *reinterpret_cast<u16x8 *>(wp + g * 8) = v;
}

// Two x chunks in LDS, TB*16 rows of NW*TPI*64 bytes each: at most ~66 KiB.
// PD*TPI weight operands per lane in registers.
template <int TB, int NW, int TPI, int PD>
hipError_t launch_one(const LinearParams &p, hipStream_t stream) {
  if constexpr (TB * NW * TPI > 32 || PD * TPI > 16) {
    return hipErrorInvalidValue;
  } else {
    hipLaunchKernelGGL((linear_packed<TB, NW, TPI, PD>), dim3(p.N / 16), dim3(64 * NW), 0, stream, p);
    return hipGetLastError();
  }
}

template <int TB, int TPI, int PD>
hipError_t launch_nw(const LinearParams &p, int NW, hipStream_t stream) {
  return NW == 8 ? launch_one<TB, 8, TPI, PD>(p, stream) : launch_one<TB, 4, TPI, PD>(p, stream);
}

template <int TPI, int PD>
hipError_t launch_tb(const LinearParams &p, int NW, hipStream_t stream) {
  switch ((p.M + 15) / 16) {
    case 1: return launch_nw<1, TPI, PD>(p, NW, stream);
    case 2: return launch_nw<2, TPI, PD>(p, NW, stream);
    case 3:
    case 4: return launch_nw<4, TPI, PD>(p, NW, stream);
    default: return hipErrorInvalidValue;
  }
}

template <int PD>
hipError_t launch_tpi(const LinearParams &p, int NW, int TPI, hipStream_t stream) {
  switch (TPI) {
    case 1: return launch_tb<1, PD>(p, NW, stream);
    case 2: return launch_tb<2, PD>(p, NW, stream);
    case 4: return launch_tb<4, PD>(p, NW, stream);
    case 8: return launch_tb<8, PD>(p, NW, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_linear_packed(const LinearParams &p, int NW, int TPI, int PD, hipStream_t stream) {
  // prefetch distance 2 (one chunk ahead) measured best; deeper rings are
  // available to the template but not instantiated
  return PD == 2 ? launch_tpi<2>(p, NW, TPI, stream) : hipErrorInvalidValue;
}

hipError_t launch_pack_weight(const void *w, void *w_packed, int K, int N, hipStream_t stream) {
  const size_t groups = (size_t)K * N / 8;
  const unsigned grid = (unsigned)((groups + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const __bf16 *>(w),
                     static_cast<__bf16 *>(w_packed), K, N);
  return hipGetLastError();
}

}  // namespace gqa
