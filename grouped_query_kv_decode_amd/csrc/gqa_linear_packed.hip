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
// Kernel: one workgroup per 1, 2 or 4 adjacent 16-column strips streams them
// over all of K (no split of k, so no partial sums leave the workgroup); its
// waves take blocks in turn and are summed through LDS in wave order.  x, the
// B operand, is small and every workgroup reads all of it (from L2), staged
// through LDS; wider workgroups read less x in total.
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

// Workgroup: SW adjacent strips (16 SW output columns) over all of K.  Its
// NW waves take the blocks of a chunk of KC = NW*TPI consecutive k-blocks
// in turn (wave w: blocks w, w+NW, ...), each block feeding SW MFMAs (one per
// strip) with the same x operand.
//
// Pipeline: a ring of PD chunks - the weights and x of chunk i are requested
// PD-1 chunks before chunk i is multiplied.  Every chunk issues the same
// loads (addresses past the end are clamped in bounds and their data never
// used), so the wait before a chunk's products covers that chunk's loads
// only and leaves the later ones in flight; with conditional loads the
// compiler drains every load at each chunk, and the kernel then runs at one
// memory latency per chunk.  NCH > 0 unrolls all NCH chunks at compile time
// (K = NCH*KC*32): no loop back edge, whose register copies would also force
// a full drain; NCH = 0 loops over any K.
template <int TB, int NW, int TPI, int SW, int PD, int NCH>
__global__ __launch_bounds__(64 * NW) void linear_packed(LinearParams p) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4, nn = lane & 15;
  const int nstrips = p.N / 16;
  const int nb0 = blockIdx.x * SW;  // first strip
  const int kblocks = p.K / 32;
  // lane's 16 bytes of block (kb = 0) of strip nb0; blocks of one strip are N/16 KiB apart
  const __bf16 *wl = p.w + (size_t)nb0 * 512 + lane * 8;

  // x staged through LDS a chunk at a time: read from memory as whole row
  // segments (16-byte pieces, XPT per thread), then each lane takes its B
  // operand (token nn, 8 values of k) from LDS.  Read straight from memory
  // the operand would touch 16 half-used cache lines per wave-wide load.
  constexpr int KC = NW * TPI;
  constexpr int ROWB = KC * 64 + 16;  // bytes per token row (+16: spreads the LDS banks)
  constexpr int PPR = KC * 4;         // 16-byte pieces per row
  constexpr int XPT = TB * 16 * PPR / (64 * NW);
  static_assert(XPT * 64 * NW == TB * 16 * PPR, "x pieces split evenly over the threads");
  constexpr int BUFB = TB * 16 * ROWB;
  __shared__ __attribute__((aligned(16))) unsigned char xs[2 * BUFB];

  f32x4 acc[SW][TB];
#pragma unroll
  for (int s = 0; s < SW; ++s)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) acc[s][tb] = f32x4{0.f, 0.f, 0.f, 0.f};

  // Rows past M repeat row M-1 (they only feed outputs past M, never
  // stored); pieces past the last k-block repeat it (never read from LDS).
  auto load_x = [&](u32x4 (&xr)[XPT], int kb0) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + i * 64 * NW;
      const int row = min(idx / PPR, p.M - 1), pc = idx % PPR;
      const int kb = min(kb0 + pc / 4, kblocks - 1);
      xr[i] = *reinterpret_cast<const u32x4 *>(p.x + (size_t)row * p.K + kb * 32 + (pc % 4) * 8);
    }
  };
  // this wave's blocks of a chunk, one per strip; past the end: the last
  // block again (in bounds, skipped in the products)
  auto load_w = [&](u32x4 (&a)[TPI][SW], int kb0) {
#pragma unroll
    for (int j = 0; j < TPI; ++j) {
      const int kb = min(kb0 + wave + j * NW, kblocks - 1);
#pragma unroll
      for (int s = 0; s < SW; ++s)
        a[j][s] = stream_load(reinterpret_cast<const u32x4 *>(wl + ((size_t)kb * nstrips + s) * 512));
    }
  };
  auto store_x = [&](const u32x4 (&xr)[XPT], unsigned char *buf) {
#pragma unroll
    for (int i = 0; i < XPT; ++i) {
      const int idx = threadIdx.x + i * 64 * NW;
      *reinterpret_cast<u32x4 *>(buf + (idx / PPR) * ROWB + (idx % PPR) * 16) = xr[i];
    }
  };
  auto products = [&](const u32x4 (&a)[TPI][SW], const unsigned char *buf, int nkb) {
#pragma unroll
    for (int j = 0; j < TPI; ++j) {
      const int kl = wave + j * NW;  // block within the chunk
      if (kl >= nkb) break;
#pragma unroll
      for (int tb = 0; tb < TB; ++tb) {
        const u32x4 b = *reinterpret_cast<const u32x4 *>(buf + (tb * 16 + nn) * ROWB + (kl * 32 + 8 * c) * 2);
#pragma unroll
        for (int s = 0; s < SW; ++s) acc[s][tb] = mfma(a[j][s], b, acc[s][tb]);
      }
    }
  };

  u32x4 xr[PD][XPT], a[PD][TPI][SW];
#pragma unroll
  for (int d = 0; d < PD - 1; ++d) {
    load_x(xr[d], d * KC);
    load_w(a[d], d * KC);
  }
  if constexpr (NCH > 0) {
#pragma unroll
    for (int i = 0; i < NCH; ++i) {
      if (i + PD - 1 < NCH) {
        load_x(xr[(i + PD - 1) % PD], (i + PD - 1) * KC);
        load_w(a[(i + PD - 1) % PD], (i + PD - 1) * KC);
      }
      store_x(xr[i % PD], xs + (i & 1) * BUFB);
      __syncthreads();
      products(a[i % PD], xs + (i & 1) * BUFB, KC);
    }
  } else {
    int buf = 0;
    for (int kb0 = 0; kb0 < kblocks; kb0 += PD * KC) {
#pragma unroll
      for (int ph = 0; ph < PD; ++ph) {
        const int kc = kb0 + ph * KC;  // this chunk; its x and weights are in slot ph
        if (kc >= kblocks) break;
        load_x(xr[(ph + PD - 1) % PD], kc + (PD - 1) * KC);
        load_w(a[(ph + PD - 1) % PD], kc + (PD - 1) * KC);
        store_x(xr[ph], xs + buf * BUFB);
        __syncthreads();
        products(a[ph], xs + buf * BUFB, min(KC, kblocks - kc));
        buf ^= 1;
      }
    }
  }

  // acc[s][tb][i] of lane (c, nn) = y[token tb*16 + nn][column 16 (nb0 + s) + 4c + i]
  // of this wave's blocks.  Sum the waves in wave order.
  __shared__ f32x4 sm[NW][SW][TB][64];
#pragma unroll
  for (int s = 0; s < SW; ++s)
#pragma unroll
    for (int tb = 0; tb < TB; ++tb) sm[wave][s][tb][lane] = acc[s][tb];
  __syncthreads();
  for (int it = threadIdx.x; it < SW * TB * 64; it += 64 * NW) {
    const int l = it % 64, tb = (it / 64) % TB, s = it / (64 * TB);
    const int row = tb * 16 + (l & 15);
    if (row >= p.M) continue;
    f32x4 t = sm[0][s][tb][l];
#pragma unroll
    for (int w = 1; w < NW; ++w) t += sm[w][s][tb][l];
    store4(p, row, 16 * (nb0 + s) + 4 * (l >> 4), t);
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

template <int TB, int NW, int TPI, int SW, int PD, int NCH>
hipError_t launch_one(const LinearParams &p, hipStream_t stream) {
  hipLaunchKernelGGL((linear_packed<TB, NW, TPI, SW, PD, NCH>), dim3(p.N / 16 / SW), dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

// The instantiated shapes (x chunks of TB*16 rows x KC blocks staged twice in
// LDS, at most ~68 KiB; the wave partial sums NW*SW*TB KiB):
//   one token tile: 1 strip, 4 waves x 4 blocks, ring of 3 (unrolled) or 2;
//                   2 strips, 8 waves x 2 blocks, ring of 4 (unrolled) or 2;
//                   4 strips, 4 waves x 1 block, ring of 2;
//   two / four token tiles: 1 strip, 4 waves x 4 / 2 blocks, ring of 2.
// Unrolled for K = 2048, 4096 and 8192 (4, 8 and 16 chunks of 16 blocks).
int linear_packed_chunk_blocks(int tb, int sw) { return tb == 4 ? 8 : (sw == 4 ? 4 : 16); }

hipError_t launch_linear_packed(const LinearParams &p, int tb, int sw, int nch, hipStream_t stream) {
  if (tb == 1 && sw == 1) {
    switch (nch) {
      case 0: return launch_one<1, 4, 4, 1, 2, 0>(p, stream);
      case 4: return launch_one<1, 4, 4, 1, 3, 4>(p, stream);
      case 8: return launch_one<1, 4, 4, 1, 3, 8>(p, stream);
      case 16: return launch_one<1, 4, 4, 1, 3, 16>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (tb == 1 && sw == 2) {
    switch (nch) {
      case 0: return launch_one<1, 8, 2, 2, 2, 0>(p, stream);
      case 4: return launch_one<1, 8, 2, 2, 4, 4>(p, stream);
      case 8: return launch_one<1, 8, 2, 2, 4, 8>(p, stream);
      case 16: return launch_one<1, 8, 2, 2, 4, 16>(p, stream);
      default: return hipErrorInvalidValue;
    }
  }
  if (nch != 0) return hipErrorInvalidValue;
  if (tb == 1 && sw == 4) return launch_one<1, 4, 1, 4, 2, 0>(p, stream);
  if (tb == 2 && sw == 1) return launch_one<2, 4, 4, 1, 2, 0>(p, stream);
  if (tb == 4 && sw == 1) return launch_one<4, 4, 2, 1, 2, 0>(p, stream);
  return hipErrorInvalidValue;
}
hipError_t launch_pack_weight(const void *w, void *w_packed, int K, int N, hipStream_t stream) {
  const size_t groups = (size_t)K * N / 8;
  const unsigned grid = (unsigned)((groups + 255) / 256);
  hipLaunchKernelGGL(pack_kernel, dim3(grid), dim3(256), 0, stream, static_cast<const __bf16 *>(w),
                     static_cast<__bf16 *>(w_packed), K, N);
  return hipGetLastError();
}

}  // namespace gqa
