// Grouped-query decode attention on the matrix cores in binary32 (gfx950).
//
// The work split of the bfloat16 matrix-core kernel: one workgroup (4 waves)
// owns (sequence b, K/V head g, head chunk hc, split s), streams that K/V
// head's positions of the split from HBM once and serves up to 16 query
// heads of the group from every tile (wikillm "Grouped-query attention
// (GQA)", Overview; the decode-step block of its Implementation sketch gives
// the per-head softmax(scale * q.K) . V computed here).
//
// Each wave takes 16-position tiles.  With v_mfma_f32_16x16x4_f32 (A: 16x4,
// B: 4x16, one binary32 per lane; lane l = 16c + n holds row / column n at
// reduction index c):
//   scores^T[16 pos x 16 heads] = K_tile[16 x D] . Q^T[D x 16]
//     lane (c, n) loads K row n, dims 16j + 4c .. +3 (16 bytes); MFMA (j, e)
//     takes element e, so its reduction index c stands for dimension
//     16j + 4c + e, and q is loaded in the same layout.  Lane (c, n) then
//     holds the scores of positions 4c .. 4c+3 for head n.
//   out^T[16 dims x 16 heads] += V_tile^T[16 dims x 4 pos] . P^T[4 pos x 16]
//     step i (0..3) takes positions 4c + i, so B is the lane's own weight i
//     (no data movement); lane (c, n) loads V row 4c + i, dims 64m + 4n .. +3
//     (a 256-byte run per row), and element e is A of output block (m, e),
//     whose row n is dimension 64m + 4n + e.
// The reduction index order inside an MFMA is free, which is why these
// permutations need no fix-up.  Heads beyond the group in a 16-head block
// are zero queries whose results are discarded.
#include "gqa_device.h"

namespace gqa {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D, bool NT>
__global__ __launch_bounds__(256) void decode_mfma_f32(DecodeParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int NW = 4;
  constexpr int KJ = D / 16;  // K loads per tile, 4 score MFMAs each
  constexpr int VM = D / 64;  // V loads per position step
  constexpr int DB = D / 16;  // output blocks (m, e)
  constexpr int kTile = 16;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4, nn = lane & 15;

  // Item order as in the bfloat16 matrix-core kernel: split slowest, then
  // head chunk, then (b, g) units.
  const unsigned item = p.order ? (unsigned)p.order[blockIdx.x] : blockIdx.x;
  const unsigned bg = (unsigned)p.B * p.G;
  const unsigned units = bg * p.HC;
  const int s = item / units;
  const unsigned rem = item % units;
  const int hc = rem / bg;
  const unsigned u = rem % bg;
  const int g = u % p.G;
  const int b = u / p.G;

  const int head0 = g * p.r + hc * 16;
  const int rw = min(p.r - hc * 16, 16);  // query heads of this workgroup
  const int t0 = s * p.chunk;

  // B operand of the score MFMAs: q of head nn, dims 16j + 4c .. +3.
  f32x4 qB[KJ];
  {
    const float *qp = static_cast<const float *>(p.q) + ((size_t)b * p.H + head0 + nn) * D + 4 * c;
#pragma unroll
    for (int j = 0; j < KJ; ++j)
      qB[j] = nn < rw ? *reinterpret_cast<const f32x4 *>(qp + 16 * j) : f32x4{0.f, 0.f, 0.f, 0.f};
  }

  const size_t slab = ((size_t)b * p.G + g) * (size_t)p.Lmax * D;
  const float *kbase = static_cast<const float *>(p.k) + slab;
  const float *vbase = static_cast<const float *>(p.v) + slab;
  const int koff = nn * D + 4 * c;      // K row nn
  const int voff = 4 * c * D + 4 * nn;  // V row 4c (+ step i)

  auto kv_load = [](const float *ptr) {
    if constexpr (NT)
      return __builtin_nontemporal_load(reinterpret_cast<const f32x4 *>(ptr));
    else
      return *reinterpret_cast<const f32x4 *>(ptr);
  };

  struct Tile {
    f32x4 kA[KJ];
    f32x4 vR[4][VM];
  };
  auto load_full = [&](Tile &T, int tt) {
    const float *kt = kbase + (size_t)tt * D;
    const float *vt = vbase + (size_t)tt * D;
#pragma unroll
    for (int j = 0; j < KJ; ++j) T.kA[j] = kv_load(kt + koff + 16 * j);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < VM; ++m) T.vR[i][m] = kv_load(vt + voff + i * D + 64 * m);
  };

  // The wave's first tile is requested before the sequence length arrives,
  // as in the bfloat16 kernel (rows inside the slab; used only if the whole
  // tile is inside the split), on grids of one round when a window is set.
  const int lo_guess = p.window > 0 && p.Lmax > p.window ? p.Lmax - p.window : 0;
  const int t_first = lo_guess + t0 + kTile * wave;
  const bool spec = (p.window <= 0 || gridDim.x <= 256) && (s == 0 || p.S <= 2) &&
                    t_first + kTile <= min(lo_guess + t0 + p.chunk, p.Lmax);
  Tile T_first;
  if (spec) load_full(T_first, t_first);

  const int n = clamp_len(p, b);
  const int lo = window_lo(p, n);
  const int nsplit = num_splits(n - lo, p.chunk);
  if (s >= nsplit) return;
  if (n == 0) {
    write_zero_heads<float, D>(p, b, head0, rw);
    return;
  }
  const int ts = lo + t0;  // this split: positions [ts, t1)
  const int t1 = min(ts + p.chunk, n);
  const bool append = p.k_new != nullptr;
  const int t_full = append ? min(t1, n - 1) : t1;
  if (append && s == nsplit - 1 && hc == 0) append_row<float, D>(p, b, g, n);
  const float *knew = append ? static_cast<const float *>(p.k_new) + ((size_t)b * p.G + g) * D : nullptr;
  const float *vnew = append ? static_cast<const float *>(p.v_new) + ((size_t)b * p.G + g) * D : nullptr;

  f32x4 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) o[db] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kNegInf, l_run = 0.f;

  // The split's last tile: rows past the split end are clamped to its last
  // row and masked out of the softmax; the appended row n-1 comes from
  // k_new / v_new.
  auto load_tail = [&](Tile &T, int tt) {
    {
      const int t = min(tt + nn, t1 - 1);
      const float *src = (append && t == n - 1) ? knew : kbase + (size_t)t * D;
#pragma unroll
      for (int j = 0; j < KJ; ++j) T.kA[j] = kv_load(src + 4 * c + 16 * j);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = min(tt + 4 * c + i, t1 - 1);
      const float *src = (append && t == n - 1) ? vnew : vbase + (size_t)t * D;
#pragma unroll
      for (int m = 0; m < VM; ++m) T.vR[i][m] = kv_load(src + 4 * nn + 64 * m);
    }
  };

  // Scores, softmax weights and the weighted V sum of one tile, with the
  // lazy rescale of the bfloat16 kernel (the reference max moves only when a
  // tile exceeds it by more than 2^kSlack).  The weights enter p.V and the
  // weight sum unrounded.
  constexpr float kSlack = 10.f;
  auto compute = [&](const Tile &T, int tt, bool tail) {
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < KJ; j += 2)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc0 = mfma4(T.kA[j][e], qB[j][e], acc0);
        acc1 = mfma4(T.kA[j + 1][e], qB[j + 1][e], acc1);
      }
    // lane (c, nn): scores of positions tt + 4c + i, head nn
    float sc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc[i] = (acc0[i] + acc1[i]) * p.scale_log2;
      if (tail && tt + 4 * c + i >= t1) sc[i] = kNegInf;
    }
    float mt = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    mt = group_max(mt);
    if (__builtin_amdgcn_ballot_w64(mt > m_run + kSlack)) {
      const float mn = mt > m_run + kSlack ? mt : m_run;
      const float alpha = fast_exp2(m_run - safe_shift(mn));
      m_run = mn;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db) o[db] *= alpha;
    }
    const float sh = safe_shift(m_run);
    float pw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      pw[i] = fast_exp2(sc[i] - sh);
      l_run += pw[i];
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int m = 0; m < VM; ++m)
#pragma unroll
        for (int e = 0; e < 4; ++e) o[4 * m + e] = mfma4(T.vR[i][m][e], pw[i], o[4 * m + e]);
  };

  // Wave w takes every NW-th tile; whole tiles through a ring of two (the
  // next tile's loads in flight while a tile is multiplied), then the
  // split's last, partial tile.
  int tt = ts + kTile * wave;
  constexpr int kStride = kTile * NW;
  if (spec && lo == lo_guess && tt + kTile <= t_full) {  // the prefetched first tile is tile tt and whole
    compute(T_first, tt, false);
    tt += kStride;
  }
  {
    const int nfull = tt + kTile <= t_full ? (t_full - kTile - tt) / kStride + 1 : 0;
    if (nfull > 0) {
      Tile R0, R1;
      load_full(R0, tt);
      int i = 0;
      for (; i + 2 < nfull; i += 2) {
        load_full(R1, tt + (i + 1) * kStride);
        compute(R0, tt + i * kStride, false);
        load_full(R0, tt + (i + 2) * kStride);
        compute(R1, tt + (i + 1) * kStride, false);
      }
      if (i + 1 < nfull) {
        load_full(R1, tt + (i + 1) * kStride);
        compute(R0, tt + i * kStride, false);
        compute(R1, tt + (i + 1) * kStride, false);
      } else {
        compute(R0, tt + i * kStride, false);
      }
      tt += nfull * kStride;
    }
  }
  for (; tt < t1; tt += kStride) {
    Tile T;
    if (tt + kTile <= t_full) {
      load_full(T, tt);
      compute(T, tt, false);
    } else {
      load_tail(T, tt);
      compute(T, tt, true);
    }
  }

  l_run = group_sum(l_run);

  // Merge the waves through LDS in wave order (deterministic).
  constexpr int LD = D + 4;
  __shared__ float sm_m[NW][16], sm_l[NW][16];
  __shared__ __align__(16) float sm_o[NW * 16 * LD];
  if (c == 0) {
    sm_m[wave][nn] = m_run;
    sm_l[wave][nn] = l_run;
  }
  // output row 4c + i of block (m, e) holds dimension 64m + 16c + 4i + e
  {
    float *row = sm_o + (wave * 16 + nn) * LD;
#pragma unroll
    for (int m = 0; m < VM; ++m)
#pragma unroll
      for (int i = 0; i < 4; ++i)
        *reinterpret_cast<f32x4 *>(row + 64 * m + 16 * c + 4 * i) =
            f32x4{o[4 * m][i], o[4 * m + 1][i], o[4 * m + 2][i], o[4 * m + 3][i]};
  }
  __syncthreads();

  for (int idx = threadIdx.x; idx < rw * (D / 4); idx += blockDim.x) {
    const int j = idx / (D / 4), cc = (idx % (D / 4)) * 4;
    float M = sm_m[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][j]);
    const float shj = safe_shift(M);
    float L = 0.f, r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      const float a = fast_exp2(sm_m[w][j] - shj);
      const float *row = sm_o + (w * 16 + j) * LD + cc;
      L += sm_l[w][j] * a;
      r0 += row[0] * a;
      r1 += row[1] * a;
      r2 += row[2] * a;
      r3 += row[3] * a;
    }
    if (nsplit == 1) {
      const float inv = 1.f / L;
      Store<float>::four(p.out, ((size_t)b * p.H + head0 + j) * D + cc, r0 * inv, r1 * inv, r2 * inv, r3 * inv);
    } else {
      const size_t hs = ((size_t)b * p.H + head0 + j) * p.S + s;
      store_partial4(p.ws_o + hs * D + cc, r0, r1, r2, r3);
      if (cc == 0) store_ml(p.ws_ml + hs, M, L);
    }
  }
  if (nsplit == 1 || !p.fused) return;
  if (!arrive_last(p.ws_cnt + ((size_t)b * p.G + g) * p.HC + hc, nsplit, p.arrive_acqrel)) return;
  merge_heads<float, D>(p, b, head0, rw, nsplit);
}

template <int D>
hipError_t launch_d(const DecodeParams &p, bool nontemporal, unsigned grid, hipStream_t stream) {
  if (nontemporal)
    hipLaunchKernelGGL((decode_mfma_f32<D, true>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_mfma_f32<D, false>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_mfma_f32(const DecodeParams &p, int D, int nontemporal, unsigned grid, hipStream_t stream) {
  if (D == 64) return launch_d<64>(p, nontemporal != 0, grid, stream);
  if (D == 128) return launch_d<128>(p, nontemporal != 0, grid, stream);
  return hipErrorInvalidValue;
}

}  // namespace gqa
