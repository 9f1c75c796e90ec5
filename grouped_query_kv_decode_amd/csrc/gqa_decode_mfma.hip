// Grouped-query decode attention on the matrix cores (bfloat16, gfx950).
//
// One workgroup (4 waves) owns (sequence b, K/V head g, split s) and streams
// that K/V head's positions of the split from HBM once, serving all r = H/G
// query heads of the group from each tile (wikillm "Grouped-query attention
// (GQA)", Overview; the decode-step block of its Implementation sketch gives
// the per-head softmax(scale * q.K) . V that is computed here).
//
// Each wave takes 32-position tiles.  With v_mfma_f32_16x16x32_bf16
// (A: 16x32, B: 32x16, both 8 bf16 per lane; lane l holds row / column l%16):
//   scores^T[16 pos x 16 heads] = K_tile[16 x D] . Q^T[D x 16]
//     A = K rows straight from global memory (16 bytes per lane), B = q.
//     Row m of half h is position 8*(m/4) + 4*h + m%4 of the tile, so lane
//     group c = l/16 ends up holding the scores of positions 8c .. 8c+7.
//   out^T[16 dims x 16 heads] += V_tile^T[16 x 32 pos] . P^T[32 pos x 16]
//     B = the probabilities already in the lane (no data movement); A needs
//     8 positions of one dimension per lane.  Lane (c, n) loads rows 8c+u,
//     dims 8n .. 8n+7 (D = 128) with coalesced 16-byte loads and transposes
//     the 8x8 block in registers; MFMA number db then covers dimensions
//     8m + db, m = 0..15, so the output lands as 32 contiguous dims per lane.
// Heads beyond r in a 16-head block are zero queries whose results are
// discarded.  The reduction index order inside an MFMA is free, which is
// why the position and dimension permutations above need no other fix-up.
#include <type_traits>

#include "gqa_device.h"

namespace gqa {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x4 mfma(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Element e (0..7) of eight 16-bit rows, packed as one MFMA operand:
// dword k = (row 2k element e, row 2k+1 element e).
template <int E, typename Row>
__device__ __forceinline__ u32x4 column(const Row *rows) {
  constexpr unsigned sel = (E & 1) ? 0x07060302u : 0x05040100u;
  u32x4 a;
#pragma unroll
  for (int k = 0; k < 4; ++k) a[k] = __builtin_amdgcn_perm(rows[2 * k + 1][E >> 1], rows[2 * k][E >> 1], sel);
  return a;
}

// out^T += V^T . P^T for dimension blocks DBI .. DB-1.
template <int DBI, int DB, int HB, typename Row>
__device__ __forceinline__ void pv_steps(f32x4 (&o)[HB][DB], const Row *vR, const u32x4 *pB) {
  if constexpr (DBI < DB) {
    const u32x4 a = column<DBI>(vR);
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) o[hb][DBI] = mfma(a, pB[hb], o[hb][DBI]);
    pv_steps<DBI + 1, DB, HB>(o, vR, pB);
  }
}

template <int D, int HB, int NW, bool NT>
__global__ __launch_bounds__(64 * NW) void decode_mfma(DecodeParams p) {
  static_assert(D == 64 || D == 128, "head dim");
  constexpr int KB = D / 32;  // QK MFMAs per 16-position half
  constexpr int DB = D / 16;  // PV MFMAs (dimension blocks)
  typedef typename std::conditional<D == 128, u32x4, u32x2>::type VRow;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane >> 4, nn = lane & 15;

  // Split index slowest: consecutive workgroups (which the dispatcher deals
  // round-robin to the XCDs) are different (b, g) units of one split, so
  // every XCD gets an even share of the units whatever their lengths.  With
  // the group's head blocks spread over p.HC workgroups (head chunk hc), the
  // chunks of one (b, g, split) are B*G apart in dispatch order - on the same
  // XCD when B*G is a multiple of 8, so the tiles they all read come from
  // that XCD's L2 after the first.
  // (With p.order, the workgroups take the items in the order it gives:
  // largest work first, for grids that run in several rounds.)
  const unsigned item = p.order ? (unsigned)p.order[blockIdx.x] : blockIdx.x;
  const unsigned bg = (unsigned)p.B * p.G;
  const unsigned units = bg * p.HC;
  const int s = item / units;
  const unsigned rem = item % units;
  const int hc = rem / bg;
  const unsigned u = rem % bg;
  const int g = u % p.G;
  const int b = u / p.G;

  const int head0 = g * p.r + hc * 16 * HB;
  const int rw = min(p.r - hc * 16 * HB, 16 * HB);  // query heads of this workgroup
  const int t0 = s * p.chunk;

  // B operand of the score MFMAs: q of head hb*16 + nn, dims kb*32 + 8c .. +7.
  u32x4 qB[HB][KB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    const int j = hb * 16 + nn;
    const __bf16 *qp = static_cast<const __bf16 *>(p.q) + ((size_t)b * p.H + head0 + j) * D + 8 * c;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
      qB[hb][kb] = j < rw ? *reinterpret_cast<const u32x4 *>(qp + kb * 32) : u32x4{0u, 0u, 0u, 0u};
  }

  const size_t slab = ((size_t)b * p.G + g) * (size_t)p.Lmax * D;
  const __bf16 *kbase = static_cast<const __bf16 *>(p.k) + slab;
  const __bf16 *vbase = static_cast<const __bf16 *>(p.v) + slab;
  // Lane offsets inside a tile (elements): K row of score half 0 (half 1 is
  // 4 rows further), dims 8c..; V row 8c, dims VPL*nn ..
  constexpr int VPL = D == 128 ? 8 : 4;
  const int koff = (8 * (nn >> 2) + (nn & 3)) * D + 8 * c;
  const int voff = 8 * c * D + VPL * nn;

  // Cache loads: non-temporal, or plain where the head chunks of a group read
  // the same tiles (they then find each other's lines in L2).
  auto kv_load = [](const auto *ptr) {
    if constexpr (NT)
      return stream_load(ptr);
    else
      return *ptr;
  };

  // One 32-position tile: K rows for the two score halves, V rows 8c .. 8c+7.
  struct Tile {
    u32x4 kA[2][KB];
    VRow vR[8];
  };
  // A whole tile inside the split: tile base is uniform, lane offsets fixed.
  // The cache is read once per call, so its loads are non-temporal: the
  // stream then does not evict what is reused (q, partial sums, counters)
  // from the caches, which measured 10% faster on a 268 MB cache.
  auto load_full = [&](Tile &T, int tt) {
    const __bf16 *kt = kbase + (size_t)tt * D;
    const __bf16 *vt = vbase + (size_t)tt * D;
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        T.kA[h][kb] = kv_load(reinterpret_cast<const u32x4 *>(kt + koff + h * 4 * D + kb * 32));
#pragma unroll
    for (int u = 0; u < 8; ++u) T.vR[u] = kv_load(reinterpret_cast<const VRow *>(vt + voff + u * D));
  };

  // The wave's first tile is requested before the sequence length arrives
  // (q, that tile and the length then share one memory latency).  Its rows
  // lie inside the cache slab; they are used only if the whole tile turns
  // out to be inside the split, otherwise the tile is loaded again below.
  // Limited to the leading splits, so workgroups of splits past a short
  // sequence's end waste little.  With a window the splits start where the
  // window does, which depends on the length: the guess is a full-length
  // sequence, and the tile is used only if the window starts there.  That
  // only on grids of one round (all workgroups wait for their first tile at
  // once): Mistral-7B shape with W = 1024 14.6 -> 14.0 us, while ragged
  // lengths with W = 4096 (512 workgroups) wasted most guesses, 157 -> 162 us.
  const int lo_guess = p.window > 0 && p.Lmax > p.window ? p.Lmax - p.window : 0;
  const int t_first = lo_guess + t0 + 32 * wave;
  const bool spec = !p.contig && (p.window <= 0 || gridDim.x <= 256) && (s == 0 || p.S <= 2) &&
                    t_first + 32 <= min(lo_guess + t0 + p.chunk, p.Lmax);
  Tile T_first;
  if (spec) load_full(T_first, t_first);

  const int n = clamp_len(p, b);
  const int lo = window_lo(p, n);
  const int nsplit = num_splits(n - lo, p.chunk);
  if (s >= nsplit) return;
  if (n == 0) {
    write_zero_heads<__bf16, D>(p, b, head0, rw);
    return;
  }
  const int ts = lo + t0;  // this split: positions [ts, t1)
  const int t1 = min(ts + p.chunk, n);
  // With a cache append, position n-1 comes from k_new / v_new: whole tiles
  // must end before it, the tile holding it takes the per-row path.
  const bool append = p.k_new != nullptr;
  const int t_full = append ? min(t1, n - 1) : t1;
  if (append && s == nsplit - 1 && hc == 0) append_row<__bf16, D>(p, b, g, n);
  const __bf16 *knew = append ? static_cast<const __bf16 *>(p.k_new) + ((size_t)b * p.G + g) * D : nullptr;
  const __bf16 *vnew = append ? static_cast<const __bf16 *>(p.v_new) + ((size_t)b * p.G + g) * D : nullptr;

  f32x4 o[HB][DB];
  float m[HB], l[HB];
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    m[hb] = kNegInf;
    l[hb] = 0.f;
#pragma unroll
    for (int db = 0; db < DB; ++db) o[hb][db] = f32x4{0.f, 0.f, 0.f, 0.f};
  }

  // The last tile of a split: rows past the split end are clamped to its last
  // row (never past the sequence length) and masked out of the softmax; the
  // appended row n-1 is read from k_new / v_new.
  auto load_tail = [&](Tile &T, int tt) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int t = min(tt + 8 * (nn >> 2) + 4 * h + (nn & 3), t1 - 1);
      const __bf16 *src = (append && t == n - 1) ? knew : kbase + (size_t)t * D;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) T.kA[h][kb] = kv_load(reinterpret_cast<const u32x4 *>(src + 8 * c + kb * 32));
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int t = min(tt + 8 * c + u, t1 - 1);
      const __bf16 *src = (append && t == n - 1) ? vnew : vbase + (size_t)t * D;
      T.vR[u] = kv_load(reinterpret_cast<const VRow *>(src + VPL * nn));
    }
  };
  // Scores, softmax weights and the weighted V sum of one tile.  The running
  // reference m only moves when a tile's maximum exceeds it by more than
  // 2^kSlack (then o and l are rescaled), so weights stay below 2^kSlack and
  // the accumulators are touched by the matrix cores only.
  constexpr float kSlack = 10.f;
  auto compute = [&](const Tile &T, int tt, bool tail) {
    u32x4 pB[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      f32x4 acc[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        acc[h] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < KB; ++kb) acc[h] = mfma(T.kA[h][kb], qB[hb][kb], acc[h]);
      }
      // lane (c, nn): scores of positions tt + 8c + u, u = 4h + i, head nn
      float sc[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        sc[u] = acc[u >> 2][u & 3] * p.scale_log2;
        if (tail && tt + 8 * c + u >= t1) sc[u] = kNegInf;
      }
      float mt = fmaxf(fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3])), fmaxf(fmaxf(sc[4], sc[5]), fmaxf(sc[6], sc[7])));
      mt = group_max(mt);
      if (__builtin_amdgcn_ballot_w64(mt > m[hb] + kSlack)) {
        const float mn = mt > m[hb] + kSlack ? mt : m[hb];
        const float alpha = fast_exp2(m[hb] - safe_shift(mn));
        m[hb] = mn;
        l[hb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db) o[hb][db] *= alpha;
      }
      const float sh = safe_shift(m[hb]);
      float pv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) pv[u] = fast_exp2(sc[u] - sh);
      // The weights enter p.V rounded to bfloat16; the weight sum adds those
      // same rounded values (widening bfloat16 is exact), so the output is a
      // convex combination of value rows: a constant V comes back exactly.
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        const bf16x2 t2 = {(__bf16)pv[2 * k], (__bf16)pv[2 * k + 1]};  // round to nearest even
        const unsigned bits = __builtin_bit_cast(unsigned, t2);
        pB[hb][k] = bits;
        l[hb] += __uint_as_float(bits << 16) + __uint_as_float(bits & 0xffff0000u);
      }
    }
    pv_steps<0, DB, HB>(o, T.vR, pB);
  };

  // Tiles of the split go to the waves either interleaved (wave w takes
  // every NW-th 32-position tile) or as contiguous runs (p.contig).
  int tt, te, kStride;
  if (p.contig) {
    const int ntiles = (t1 - ts + 31) / 32;
    const int per = (ntiles + NW - 1) / NW;
    tt = ts + 32 * per * wave;
    te = min(t1, tt + 32 * per);
    kStride = 32;
  } else {
    tt = ts + 32 * wave;
    te = t1;
    kStride = 32 * NW;
    if (spec && lo == lo_guess && tt + 32 <= t_full) {  // the prefetched first tile is tile tt and whole: use it
      compute(T_first, tt, false);
      tt += kStride;
    }
  }
  // Whole tiles through a ring of two: the next tile's loads are in flight
  // while a tile is multiplied.  The loop is unrolled by two with fixed
  // slots and every load in it is of a whole tile, so the compiler's wait
  // before a tile's products covers that tile only.  Measured (bit-equal):
  // Mistral-7B shape 42.5 -> 41.7 us, T5-XXL G = 8 23.8 -> 21.9 us, B64 H64
  // G1 d64 L4096 23.1 -> 20.5 us.  Not with two or four head blocks at
  // d = 128, whose products then need 272-428 registers (B32 H64 G1 d128
  // L2048 with four: 28.0 -> 29.6 us); those load and multiply one tile at
  // a time below.
  constexpr bool kRing = D == 64 || HB == 1;
  if constexpr (kRing) {
    const int lim = min(te, t_full);
    const int nfull = tt + 32 <= lim ? (lim - 32 - tt) / kStride + 1 : 0;  // whole tiles left
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
  for (; tt < te; tt += kStride) {
    Tile T;
    if (tt + 32 <= t_full) {
      load_full(T, tt);
      compute(T, tt, false);
    } else {  // the split's last tile (partial, or holding the appended row)
      load_tail(T, tt);
      compute(T, tt, true);
    }
  }

  // Per-head weight sums: add the four lane groups.
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) l[hb] = group_sum(l[hb]);

  // Merge the NW waves through LDS, in wave order (deterministic).  When the
  // per-wave outputs fit in 64 KiB each wave stores its own and one barrier
  // suffices; otherwise the waves add into one buffer in turn.
  constexpr int NHB = 16 * HB;
  constexpr int LD = D + 4;
  constexpr bool kParallel = NW * NHB * LD * 4 <= 64 * 1024;
  constexpr int kRegions = kParallel ? NW : 1;
  __shared__ float sm_m[NW][NHB], sm_l[NW][NHB];
  __shared__ float sm_o[kRegions * NHB * LD];
  if (c == 0) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      sm_m[wave][hb * 16 + nn] = m[hb];
      sm_l[wave][hb * 16 + nn] = l[hb];
    }
  }
  // output row m = 4c + i of PV MFMA db holds dimension VPL*m + db
  if (kParallel) {
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      float *row = sm_o + (wave * NHB + hb * 16 + nn) * LD;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int db = 0; db < DB; ++db) row[VPL * (4 * c + i) + db] = o[hb][db][i];
    }
    __syncthreads();
  } else {
    __syncthreads();
    float a_self[HB];
#pragma unroll
    for (int hb = 0; hb < HB; ++hb) {
      const int j = hb * 16 + nn;
      float M = sm_m[0][j];
#pragma unroll
      for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][j]);
      a_self[hb] = fast_exp2(m[hb] - safe_shift(M));
    }
    for (int w = 0; w < NW; ++w) {
      if (wave == w) {
#pragma unroll
        for (int hb = 0; hb < HB; ++hb) {
          float *row = sm_o + (hb * 16 + nn) * LD;
#pragma unroll
          for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int db = 0; db < DB; ++db) {
              const int dim = VPL * (4 * c + i) + db;
              const float add = o[hb][db][i] * a_self[hb];
              row[dim] = w == 0 ? add : row[dim] + add;
            }
        }
      }
      __syncthreads();
    }
  }

  for (int idx = threadIdx.x; idx < rw * (D / 4); idx += blockDim.x) {
    const int j = idx / (D / 4), cc = (idx % (D / 4)) * 4;
    float M = sm_m[0][j];
#pragma unroll
    for (int w = 1; w < NW; ++w) M = fmaxf(M, sm_m[w][j]);
    const float shj = safe_shift(M);
    float L = 0.f, r0 = 0.f, r1 = 0.f, r2 = 0.f, r3 = 0.f;
    if (kParallel) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float a = fast_exp2(sm_m[w][j] - shj);
        const float *row = sm_o + (w * NHB + j) * LD + cc;
        L += sm_l[w][j] * a;
        r0 += row[0] * a;
        r1 += row[1] * a;
        r2 += row[2] * a;
        r3 += row[3] * a;
      }
    } else {
#pragma unroll
      for (int w = 0; w < NW; ++w) L += sm_l[w][j] * fast_exp2(sm_m[w][j] - shj);
      const float *row = sm_o + j * LD + cc;
      r0 = row[0];
      r1 = row[1];
      r2 = row[2];
      r3 = row[3];
    }
    if (nsplit == 1) {
      const float inv = 1.f / L;
      Store<__bf16>::four(p.out, ((size_t)b * p.H + head0 + j) * D + cc, r0 * inv, r1 * inv, r2 * inv, r3 * inv);
    } else {
      const size_t hs = ((size_t)b * p.H + head0 + j) * p.S + s;
      store_partial4(p.ws_o + hs * D + cc, r0, r1, r2, r3);
      if (cc == 0) store_ml(p.ws_ml + hs, M, L);
    }
  }
  if (nsplit == 1 || !p.fused) return;
  if (!arrive_last(p.ws_cnt + ((size_t)b * p.G + g) * p.HC + hc, nsplit, p.arrive_acqrel)) return;
  merge_heads<__bf16, D>(p, b, head0, rw, nsplit);
}

template <int D, int HB, int NW>
hipError_t launch_t(const DecodeParams &p, bool nontemporal, unsigned grid, hipStream_t stream) {
  if constexpr (HB <= 2) {
    if (!nontemporal) {
      hipLaunchKernelGGL((decode_mfma<D, HB, NW, false>), dim3(grid), dim3(64 * NW), 0, stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((decode_mfma<D, HB, NW, true>), dim3(grid), dim3(64 * NW), 0, stream, p);
  return hipGetLastError();
}

// Larger workgroups only where the register budget (64 KiB per SIMD split
// over more waves) holds the head blocks without spilling.
template <int D, int HB>
hipError_t launch_nw(const DecodeParams &p, int NW, bool nt, unsigned grid, hipStream_t stream) {
  if constexpr (HB == 1 && D == 64) {
    if (NW == 16) return launch_t<D, HB, 16>(p, nt, grid, stream);
  }
  if constexpr (HB <= 2) {
    if (NW == 8) return launch_t<D, HB, 8>(p, nt, grid, stream);
  }
  return launch_t<D, HB, 4>(p, nt, grid, stream);
}

template <int D>
hipError_t launch_hb(const DecodeParams &p, int HB, int NW, bool nt, unsigned grid, hipStream_t stream) {
  switch (HB) {
    case 1: return launch_nw<D, 1>(p, NW, nt, grid, stream);
    case 2: return launch_nw<D, 2>(p, NW, nt, grid, stream);
    case 4: return launch_nw<D, 4>(p, NW, nt, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_decode_mfma(const DecodeParams &p, int D, int HB, int NW, int nontemporal, unsigned grid,
                              hipStream_t stream) {
  const bool nt = nontemporal != 0;
  return D == 64 ? launch_hb<64>(p, HB, NW, nt, grid, stream) : launch_hb<128>(p, HB, NW, nt, grid, stream);
}

}  // namespace gqa
