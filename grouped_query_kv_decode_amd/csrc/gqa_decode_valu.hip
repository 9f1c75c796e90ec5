// Grouped-query decode attention on the vector ALUs (binary32 and bfloat16).
//
// One workgroup (4 waves) owns (sequence b, K/V head g, head chunk hc, split
// s): it streams positions [lo + s*chunk, min(lo + (s+1)*chunk, len_b)) of
// K/V head g once (lo = 0, or the first position of the sliding window) and
// serves up to RC query heads of the group from every row it loads
// (wikillm "Grouped-query attention (GQA)", Overview: every query head of a
// group attends with the group's single key and value head).
//
// Lane layout: a cache row of D elements is spread over LPR lanes, 16 bytes
// per lane, so one wave-wide 128-bit load covers RPW consecutive rows.  Each
// row group keeps its own online softmax state; states are merged across row
// groups with cross-lane shuffles and across waves through LDS.
#include "gqa_device.h"

namespace gqa {
namespace {

template <typename T> struct Elems;
template <> struct Elems<float> {
  static constexpr int kPerLane = 4;
  __device__ static void widen(const uint4 &u, float *f) {
    f[0] = __uint_as_float(u.x);
    f[1] = __uint_as_float(u.y);
    f[2] = __uint_as_float(u.z);
    f[3] = __uint_as_float(u.w);
  }
};
template <> struct Elems<__bf16> {
  static constexpr int kPerLane = 8;
  // bfloat16 -> binary32 is exact: the bf16 bits become the upper half.
  __device__ static void widen(const uint4 &u, float *f) {
    const unsigned w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __uint_as_float(w[i] << 16);
      f[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
    }
  }
};

// Sum over aligned groups of LPR lanes; every lane of the group gets the sum.
template <int LPR>
__device__ __forceinline__ float row_sum(float x) {
  // xor 1 and xor 2 inside each quad, then the half-row and row mirrors
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xF, 0xF, false));
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xF, 0xF, false));
  if (LPR >= 8) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x141, 0xF, 0xF, false));
  if (LPR >= 16) x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x140, 0xF, 0xF, false));
  if (LPR >= 32) x += __shfl_xor(x, 16);
  return x;
}

// VPL: 16-byte pieces a lane holds of each row (1, or 2 for binary32 rows
// of 128 elements, which then span 16 lanes instead of 32: fewer cross-lane
// reduction steps per score).  Piece v of every lane lies in the v-th 1/VPL
// of the row, so each load instruction reads one contiguous run per row.
template <typename T, int D, int RC, int U, bool SPEC, int VPL>
__global__ __launch_bounds__(256) void decode_valu(DecodeParams p) {
  constexpr int PPL = Elems<T>::kPerLane;  // elements per 16-byte piece
  constexpr int EPL = PPL * VPL;           // elements per lane per row
  constexpr int PSTRIDE = D / VPL;         // elements between a lane's pieces
  constexpr int LPR = D / EPL;             // lanes per row
  constexpr int RPW = 64 / LPR;            // rows per wave per load
  constexpr int NRG = 4 * RPW;             // row groups per workgroup
  static_assert(LPR >= 4 && LPR <= 32, "row must span 4..32 lanes");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int sub = lane % LPR;
  const int rg = wave * RPW + lane / LPR;

  // Split index slowest (see the MFMA kernel): units spread over the XCDs.
  const unsigned item = p.order ? (unsigned)p.order[blockIdx.x] : blockIdx.x;
  const unsigned units = (unsigned)p.B * p.G * p.HC;
  const int s = item / units;
  unsigned id = item % units;
  const int hc = id % p.HC;
  id /= p.HC;
  const int g = id % p.G;
  const int b = id / p.G;

  const int jbase = hc * RC;
  const int nh = min(RC, p.r - jbase);
  const int head0 = g * p.r + jbase;
  const bool append = p.k_new != nullptr;
  const size_t slab = ((size_t)b * p.G + g) * (size_t)p.Lmax * D;
  const T *kp = static_cast<const T *>(p.k) + slab + sub * PPL;
  const T *vp = static_cast<const T *>(p.v) + slab + sub * PPL;

  // Query rows of the served heads (they do not depend on the length).
  uint4 qraw[RC][VPL];
#pragma unroll
  for (int j = 0; j < RC; ++j)
#pragma unroll
    for (int v = 0; v < VPL; ++v)
      qraw[j][v] = j < nh ? *reinterpret_cast<const uint4 *>(static_cast<const T *>(p.q) +
                                                            ((size_t)b * p.H + head0 + j) * D + sub * PPL + v * PSTRIDE)
                          : make_uint4(0u, 0u, 0u, 0u);

  // A slot of rows: U rows per row group, their validity in the split.
  struct Rows {
    uint4 kr[U][VPL], vr[U][VPL];
    bool ok[U];
  };
  constexpr int kStep = NRG * U;
  // SPEC (grids of one round, no cache append): the first slot is
  // requested before the sequence length arrives (as in the matrix-core
  // kernel), for a full-length sequence, rows clamped inside the slab.  Once
  // the length is known, the slot is used if the split starts where
  // guessed: rows past the split are masked and their V set to zero
  // (padding may hold anything), so the products equal those of the plain
  // path.  Only on the leading splits.  Tiny binary32 B1 H8 G2 d64 L256:
  // 9.1 -> 8.5 us; on larger grids the variant's code streamed slower
  // (binary32 Mistral-7B shape 93 -> 109 us), so they run without it.
  const int lo_guess = p.window > 0 && p.Lmax > p.window ? p.Lmax - p.window : 0;
  const int ts_guess = lo_guess + s * p.chunk;
  const bool spec = SPEC && (s == 0 || p.S <= 2) && ts_guess < p.Lmax;
  Rows first;
  if (spec) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int row = min(ts_guess + u * NRG + rg, p.Lmax - 1);
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        first.kr[u][v] = stream_load(reinterpret_cast<const uint4 *>(kp + (size_t)row * D + v * PSTRIDE));
        first.vr[u][v] = stream_load(reinterpret_cast<const uint4 *>(vp + (size_t)row * D + v * PSTRIDE));
      }
    }
  }

  const int n = clamp_len(p, b);
  const int lo = window_lo(p, n);
  const int nsplit = num_splits(n - lo, p.chunk);
  if (s >= nsplit) return;
  if (n == 0) {
    write_zero_heads<T, D>(p, b, head0, nh);
    return;
  }
  const int t0 = lo + s * p.chunk, t1 = min(t0 + p.chunk, n);
  // Cache append: position n-1 is read from k_new / v_new and written into
  // the cache by one workgroup of the last split.
  if (append && s == nsplit - 1 && hc == 0) append_row<T, D>(p, b, g, n);
  const bool use_first = spec && t0 == ts_guess;

  // Query rows pre-multiplied by scale*log2(e) (zero rows past the group).
  float qf[RC][EPL];
#pragma unroll
  for (int j = 0; j < RC; ++j) {
#pragma unroll
    for (int v = 0; v < VPL; ++v) Elems<T>::widen(qraw[j][v], qf[j] + v * PPL);
#pragma unroll
    for (int e = 0; e < EPL; ++e) qf[j][e] *= p.scale_log2;
  }

  const T *knew = append ? static_cast<const T *>(p.k_new) + ((size_t)b * p.G + g) * D + sub * PPL : nullptr;
  const T *vnew = append ? static_cast<const T *>(p.v_new) + ((size_t)b * p.G + g) * D + sub * PPL : nullptr;

  float m[RC], l[RC], o[RC][EPL];
#pragma unroll
  for (int j = 0; j < RC; ++j) {
    m[j] = kNegInf;
    l[j] = 0.f;
#pragma unroll
    for (int e = 0; e < EPL; ++e) o[j][e] = 0.f;
  }

  auto load = [&](Rows &R, int tb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int t = tb + u * NRG + rg;
      R.ok[u] = t < t1;
      const int row = R.ok[u] ? t : t1 - 1;  // never past the length
      const bool fresh = append && row == n - 1;
#pragma unroll
      for (int v = 0; v < VPL; ++v) {
        R.kr[u][v] = stream_load(reinterpret_cast<const uint4 *>((fresh ? knew : kp + (size_t)row * D) + v * PSTRIDE));
        R.vr[u][v] = stream_load(reinterpret_cast<const uint4 *>((fresh ? vnew : vp + (size_t)row * D) + v * PSTRIDE));
      }
    }
  };
  // The speculative slot once the split is known: rows past it masked, with V zero.
  auto settle = [&](Rows &R, int tb) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      R.ok[u] = tb + u * NRG + rg < t1;
      if (!R.ok[u])
#pragma unroll
        for (int v = 0; v < VPL; ++v) R.vr[u][v] = make_uint4(0u, 0u, 0u, 0u);
    }
  };
  auto process = [&](const Rows &R) {
    const bool *ok = R.ok;
    float sc[U][RC];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float kf[EPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) Elems<T>::widen(R.kr[u][v], kf + v * PPL);
#pragma unroll
      for (int j = 0; j < RC; ++j) {
        float acc = 0.f;
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc = fmaf(qf[j][e], kf[e], acc);
        acc = row_sum<LPR>(acc);
        sc[u][j] = ok[u] ? acc : kNegInf;
      }
    }
    float sh[RC];
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      float mt = sc[0][j];
#pragma unroll
      for (int u = 1; u < U; ++u) mt = fmaxf(mt, sc[u][j]);
      const float mn = fmaxf(m[j], mt);
      sh[j] = safe_shift(mn);
      const float alpha = fast_exp2(m[j] - sh[j]);
      m[j] = mn;
      l[j] *= alpha;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] *= alpha;
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      float vf[EPL];
#pragma unroll
      for (int v = 0; v < VPL; ++v) Elems<T>::widen(R.vr[u][v], vf + v * PPL);
#pragma unroll
      for (int j = 0; j < RC; ++j) {
        const float pj = fast_exp2(sc[u][j] - sh[j]);
        l[j] += pj;
#pragma unroll
        for (int e = 0; e < EPL; ++e) o[j][e] = fmaf(pj, vf[e], o[j][e]);
      }
    }
  };
  // Rows through a ring of two slots with 4 heads per row set: the next
  // slot's loads are in flight while one is multiplied (loop unrolled by two
  // with fixed slots, every load unconditional, so the compiler's wait before
  // a slot's products covers that slot only).  Only the schedule changes.
  // Binary32 Mistral-7B shape 102.6 -> 92.6 us, B1 L32768 62.7 -> 56.5 us,
  // the tiny B1 H8 G2 d64 L256 case 8.8 -> 8.0 us.  With 1, 2 or 8 heads
  // the slots' registers cost occupancy (2 heads, B8 H32 G16 d128 L8192:
  // 156.5 -> 209.5 us), so those load and multiply one slot at a time.
  constexpr bool kRing = RC == 4;
  if constexpr (kRing) {
    const int nit = (t1 - t0 + kStep - 1) / kStep;
    Rows &A = first;
    Rows B;
    if (use_first)
      settle(A, t0);
    else
      load(A, t0);
    int i = 0;
    for (; i + 2 < nit; i += 2) {
      load(B, t0 + (i + 1) * kStep);
      process(A);
      load(A, t0 + (i + 2) * kStep);
      process(B);
    }
    if (i + 1 < nit) {
      load(B, t0 + (i + 1) * kStep);
      process(A);
      process(B);
    } else {
      process(A);
    }
  } else {
    int tb = t0;
    if (use_first) {
      settle(first, t0);
      process(first);
      tb += kStep;
    }
    for (; tb < t1; tb += kStep) {
      Rows R;
      load(R, tb);
      process(R);
    }
  }

  // Merge the row groups of this wave (lanes lane ^ LPR, ^ 2LPR, ...).
#pragma unroll
  for (int off = LPR; off < 64; off <<= 1) {
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      const float m2 = __shfl_xor(m[j], off);
      const float l2 = __shfl_xor(l[j], off);
      const float mn = fmaxf(m[j], m2);
      const float shj = safe_shift(mn);
      const float a1 = fast_exp2(m[j] - shj), a2 = fast_exp2(m2 - shj);
      m[j] = mn;
      l[j] = l[j] * a1 + l2 * a2;
#pragma unroll
      for (int e = 0; e < EPL; ++e) o[j][e] = o[j][e] * a1 + __shfl_xor(o[j][e], off) * a2;
    }
  }

  // Merge the four waves through LDS, in wave order.
  __shared__ float sm_m[4][RC], sm_l[4][RC];
  __shared__ float sm_o[RC][D];
  if (lane == 0) {
#pragma unroll
    for (int j = 0; j < RC; ++j) {
      sm_m[wave][j] = m[j];
      sm_l[wave][j] = l[j];
    }
  }
  __syncthreads();
  float a_self[RC];
#pragma unroll
  for (int j = 0; j < RC; ++j) {
    const float M = fmaxf(fmaxf(sm_m[0][j], sm_m[1][j]), fmaxf(sm_m[2][j], sm_m[3][j]));
    a_self[j] = fast_exp2(m[j] - safe_shift(M));
  }
  for (int w = 0; w < 4; ++w) {
    if (wave == w && lane < LPR) {
#pragma unroll
      for (int j = 0; j < RC; ++j)
#pragma unroll
        for (int e = 0; e < EPL; ++e) {
          const int x = (e / PPL) * PSTRIDE + sub * PPL + e % PPL;  // element of piece e / PPL
          const float add = o[j][e] * a_self[j];
          sm_o[j][x] = w == 0 ? add : sm_o[j][x] + add;
        }
    }
    __syncthreads();
  }

  // This workgroup's result for its heads: final output, or a split partial.
  for (int idx = threadIdx.x; idx < nh * (D / 4); idx += blockDim.x) {
    const int j = idx / (D / 4), c = (idx % (D / 4)) * 4;
    const float M = fmaxf(fmaxf(sm_m[0][j], sm_m[1][j]), fmaxf(sm_m[2][j], sm_m[3][j]));
    const float shj = safe_shift(M);
    float L = 0.f;
#pragma unroll
    for (int w = 0; w < 4; ++w) L += sm_l[w][j] * fast_exp2(sm_m[w][j] - shj);
    if (nsplit == 1) {
      const float inv = 1.f / L;
      Store<T>::four(p.out, ((size_t)b * p.H + head0 + j) * D + c, sm_o[j][c] * inv, sm_o[j][c + 1] * inv,
                     sm_o[j][c + 2] * inv, sm_o[j][c + 3] * inv);
    } else {
      const size_t hs = ((size_t)b * p.H + head0 + j) * p.S + s;
      store_partial4(p.ws_o + hs * D + c, sm_o[j][c], sm_o[j][c + 1], sm_o[j][c + 2], sm_o[j][c + 3]);
      if (c == 0) store_ml(p.ws_ml + hs, M, L);
    }
  }
  if (nsplit == 1 || !p.fused) return;
  if (!arrive_last(p.ws_cnt + ((size_t)b * p.G + g) * p.HC + hc, nsplit, p.arrive_acqrel)) return;
  merge_heads<T, D>(p, b, head0, nh, nsplit);
}

template <typename T, int D, int RC>
hipError_t launch_t(const DecodeParams &p, bool one_piece, unsigned grid, hipStream_t stream) {
  // Two pieces per lane for binary32 rows of 128 elements serving 8 heads
  // per row set (GQA_VALU_PIECES=1 restores one), with half the rows per slot
  // (same bytes in flight): B2 H64 G8 d128 L8192 50.7 -> 46.0 us.  With 1 or
  // 2 heads it measured neutral, with 4 heads 2-9% slower (Mistral-7B shape
  // 87.8 -> 91.2 us), so those keep one piece.
  constexpr int VPL = (std::is_same<T, float>::value && D == 128 && RC == 8) ? 2 : 1;
  constexpr int U = (RC <= 4 ? 8 : 4) / VPL;
  if (VPL == 2 && one_piece) {
    constexpr int U1 = RC <= 4 ? 8 : 4;
    if (grid <= 256 && p.k_new == nullptr)
      hipLaunchKernelGGL((decode_valu<T, D, RC, U1, true, 1>), dim3(grid), dim3(256), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_valu<T, D, RC, U1, false, 1>), dim3(grid), dim3(256), 0, stream, p);
    return hipGetLastError();
  }
  if (grid <= 256 && p.k_new == nullptr)
    hipLaunchKernelGGL((decode_valu<T, D, RC, U, true, VPL>), dim3(grid), dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL((decode_valu<T, D, RC, U, false, VPL>), dim3(grid), dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rc(const DecodeParams &p, int RC, bool one_piece, unsigned grid, hipStream_t stream) {
  switch (RC) {
    case 1: return launch_t<T, D, 1>(p, one_piece, grid, stream);
    case 2: return launch_t<T, D, 2>(p, one_piece, grid, stream);
    case 4: return launch_t<T, D, 4>(p, one_piece, grid, stream);
    case 8: return launch_t<T, D, 8>(p, one_piece, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_valu(const DecodeParams &p, int dtype, int D, int RC, int one_piece, unsigned grid,
                              hipStream_t stream) {
  const bool op = one_piece != 0;
  if (dtype == 0)
    return D == 64 ? launch_rc<float, 64>(p, RC, op, grid, stream) : launch_rc<float, 128>(p, RC, op, grid, stream);
  return D == 64 ? launch_rc<__bf16, 64>(p, RC, op, grid, stream) : launch_rc<__bf16, 128>(p, RC, op, grid, stream);
}

}  // namespace gqa
