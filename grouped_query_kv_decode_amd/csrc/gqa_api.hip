// Host side of libgqa.so: argument checks, launch planning and the C ABI
// declared in include/gqa.h.  No allocation, no synchronisation.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <string>

#include "gqa.h"
#include "gqa_measure.h"
#include "gqa_device.h"
#include "gqa_linear.h"

namespace {

thread_local std::string g_last_hip_error;

enum { KIND_VALU = 0, KIND_MFMA = 1 };

gqa_status hip_fail(hipError_t e) {
  g_last_hip_error = hipGetErrorString(e);
  return GQA_ERR_HIP;
}

int env_int(const char *name, int dflt) {
  const char *v = getenv(name);
  if (!v || !*v) return dflt;
  char *end = nullptr;
  const long x = strtol(v, &end, 10);
  return (end && *end == 0 && x > 0 && x < (1L << 30)) ? (int)x : dflt;
}

bool env_is(const char *name, const char *value) {
  const char *v = getenv(name);
  return v && strcmp(v, value) == 0;
}

// Launch-plan overrides for tuning and tests.  They are read from the
// environment once, when the library is loaded, and again only on
// gqa_tuning_reload(); a decode call never reads the environment, so the
// plan a call takes cannot change between gqa_decode_workspace_size and the
// call.  Zero (or -1) means "the measured default plan".
struct Tuning {
  int kernel;        // GQA_KERNEL=valu|mfma: 1 + KIND_VALU / 1 + KIND_MFMA, 0 the plan's choice
  int target_wgs;    // GQA_TARGET_WGS: plain workgroup target (split count rounded up to it)
  int max_chunk;     // GQA_MAX_CHUNK: split length cap
  int chunk;         // GQA_CHUNK: split length
  int fused_max;     // GQA_FUSED_MAX_SPLITS: splits merged inside the decode kernel at most
  int waves;         // GQA_WAVES=8|16: matrix-core workgroup waves
  int head_split;    // GQA_HEAD_SPLIT=1|2|4
  int contig;        // GQA_CONTIG=1: contiguous per-wave tile runs
  int temporal;      // GQA_TEMPORAL=0|1: non-temporal / plain cache loads (-1: the plan's)
  int merge_kernel;  // GQA_MERGE=kernel
  int order;         // GQA_ORDER=0|1 (-1: the plan's)
  int valu_pieces;   // GQA_VALU_PIECES=1: one 16-byte piece per lane and row
  int arrive_acqrel; // GQA_ARRIVE=acqrel: release/acquire ordering on the arrival counter
  int linear_waves, linear_ksplit, linear_tpi, linear_strips;  // GQA_LINEAR_*
  int linear_unroll;                                           // GQA_LINEAR_UNROLL=0: 0, else -1
};

Tuning read_tuning() {
  Tuning t;
  t.kernel = env_is("GQA_KERNEL", "valu") ? 1 + KIND_VALU : (env_is("GQA_KERNEL", "mfma") ? 1 + KIND_MFMA : 0);
  t.target_wgs = env_int("GQA_TARGET_WGS", 0);
  t.max_chunk = env_int("GQA_MAX_CHUNK", 0);
  t.chunk = env_int("GQA_CHUNK", 0);
  t.fused_max = env_int("GQA_FUSED_MAX_SPLITS", 0);
  t.waves = env_int("GQA_WAVES", 0);
  t.head_split = env_int("GQA_HEAD_SPLIT", 0);
  t.contig = env_int("GQA_CONTIG", 0) == 1;
  const char *tmp = getenv("GQA_TEMPORAL");
  t.temporal = tmp && tmp[0] ? (tmp[0] == '1') : -1;
  t.merge_kernel = env_is("GQA_MERGE", "kernel");
  t.order = env_is("GQA_ORDER", "0") ? 0 : (env_is("GQA_ORDER", "1") ? 1 : -1);
  const char *pieces = getenv("GQA_VALU_PIECES");
  t.valu_pieces = pieces && pieces[0] == '1';
  t.arrive_acqrel = env_is("GQA_ARRIVE", "acqrel");
  t.linear_waves = env_int("GQA_LINEAR_WAVES", 0);
  t.linear_ksplit = env_int("GQA_LINEAR_KSPLIT", 0);
  t.linear_tpi = env_int("GQA_LINEAR_TPI", 0);
  t.linear_strips = env_int("GQA_LINEAR_STRIPS", 0);
  t.linear_unroll = env_is("GQA_LINEAR_UNROLL", "0") ? 0 : -1;
  return t;
}

Tuning g_tuning = read_tuning();              // at library load
std::atomic<unsigned> g_tuning_gen{1};        // bumped by gqa_tuning_reload: cached plans go stale

size_t round_up(size_t x, size_t a) { return (x + a - 1) / a * a; }
int ceil_div(long a, long b) { return (int)((a + b - 1) / b); }
int next_pow2(int x) {
  int p = 1;
  while (p < x) p <<= 1;
  return p;
}


// Workspace layout when some sequence may span several splits:
//   [0, kCounterBytes)  arrival counters, one per (b, g, head chunk) unit;
//                       zero between calls (each call leaves them zero)
//   ml region           float2 [B, H, S]   split (max, weight sum)
//   o region            float  [B, H, S, d] split un-normalised outputs
//   order region        int    [grid]       dispatch order (multi-round grids)
// The counter region is never used for anything else, whatever the shape,
// so one cleared workspace serves calls of any shape.
constexpr size_t kCounterBytes = 256 * 1024;
constexpr long kMaxFusedUnits = kCounterBytes / sizeof(unsigned);  // counters
constexpr int kMaxSplits = 256;     // splits per sequence the planner uses at most
constexpr int kMaxFusedSplits = 32; // more splits: merged by the wide merge kernel
constexpr unsigned kOrderMinGrid = 1024;  // larger split grids run largest items first ...
constexpr int kOrderMinSplits = 4;        // ... with at least this many splits per sequence

struct Plan {
  int kind;
  int chunk, S, HC, RC, HB;
  int NW;  // waves per workgroup (matrix-core kernel)
  int fused;
  int wide;     // merge by the wide merge kernel
  int ordered;  // workgroups take their items largest first (order region of the workspace)
  int nontemporal;  // matrix-core cache loads non-temporal (plain when head chunks share lines)
  int contig;       // matrix-core tiles as contiguous per-wave runs (tuning only)
  int valu_pieces;  // VALU kernel forced to one 16-byte piece per lane and row (tuning only)
  int arrive_acqrel;  // release/acquire arrival counter
  unsigned grid;
  size_t ml_off, o_off, order_off, ws_bytes;
};

gqa_status check_shape(int B, int H, int G, int d, int Lmax, gqa_dtype dt) {
  if (dt != GQA_F32 && dt != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (B < 0 || H < 1 || G < 1 || d < 1 || Lmax < 1 || H % G != 0) return GQA_ERR_SHAPE;
  if (d != 64 && d != 128) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

// Decode launch plan (tuned on MI355X with the workload sweep):
//  - kernel: bfloat16 uses the matrix-core kernel for r = H/G in 2..64, and
//    for r = 1 on calls that stream at least 32 MiB of K and V (smaller MHA
//    calls take the VALU kernel, whose one-round plan splits less); binary32
//    uses its own matrix-core kernel for r = 3..64 (one workgroup per block
//    of 16 heads), and for r <= 2 on calls of at least 32 MiB whose (b, g)
//    units do not fill whole rounds of 256 workgroups; otherwise the VALU
//    kernel.  GQA_KERNEL=valu|mfma overrides.
//  - workgroups of the matrix-core kernels have 4 waves (GQA_WAVES = 8 or 16
//    overrides for bfloat16 where the register budget for the head blocks
//    allows).
//  - with fewer (b, g) units than compute units the matrix-core kernel
//    spreads a group's head blocks over up to 2 or 4 workgroups (head chunks;
//    how many by an estimate of the busiest compute unit's work, see
//    plan_cost; GQA_HEAD_SPLIT overrides), which then load the cache with
//    plain instead of non-temporal loads (GQA_TEMPORAL=0/1 overrides) so
//    that they share its lines in L2.
//  - splits: one workgroup per (b, g, head chunk, split), split lengths of
//    at least 256 positions (bfloat16 matrix cores), 64 (binary32 matrix
//    cores) or 32 (VALU), at least Lmax/256,
//    at most GQA_MAX_CHUNK = 8192 on the matrix cores, 4096 on the VALU
//    kernel (the cap keeps ragged batches balanced).
//    The VALU kernel aims at one workgroup per compute unit (three on
//    binary32 with 4 or more heads per row set); the matrix-core kernels take
//    the split count of lowest plan_cost among those filling 1..4 rounds of
//    256 workgroups (binary32 grids of one round: their own estimate).
//    GQA_TARGET_WGS (a plain workgroup target) and GQA_CHUNK override.
//  - when a sequence spans several splits, the workgroup that finishes its
//    (b, g) unit last merges the partials inside the same kernel; with more
//    units than counters (or GQA_MERGE=kernel) a second kernel merges instead.
//    Beyond GQA_FUSED_MAX_SPLITS = 32 splits, or when that workgroup would
//    read more than 96 KiB of partials, the wide merge kernel does (a launch
//    of its own costs more than the in-kernel merge saves below that).
//  - grids of more than 1024 workgroups with at least 4 splits per sequence
//    (several dispatch rounds) take their items largest first, in an order a
//    small kernel sorts from the lengths on the device (GQA_ORDER=0/1).
gqa_status make_plan(int B, int H, int G, int d, int Lmax, gqa_dtype dt, const Tuning &tu, Plan *pl) {
  const int r = H / G;
  // bfloat16 runs on the matrix cores for r = 2..64, and for r = 1 (MHA)
  // once the call streams at least 32 MiB of K and V: rocprofv3 / graph-
  // replay times, matrix cores against VALU, B8 H32 G32 d128 L8192 150.8 /
  // 158.9 us, B4 H16 G16 d128 L32768 153.0 / 161.9, B64 H8 G8 d128 L4096
  // 153.0 / 157.3, B32 H64 G64 d64 L2048 156.1 / 157.6, B8 H16 G16 d64
  // L2048 (67 MB) 14.8 / 16.1, B2 H8 G8 d128 L4096 (33.5 MB) 12.7 / 13.5;
  // below, the VALU kernel's one-round plan (fewer splits) wins: B4 H32 G32
  // d64 L512 (16.8 MB) 7.61 / 7.30 us, B1 H16 G16 d128 L1024 (8.4 MB)
  // 8.71 / 8.07 us.
  //
  // binary32 runs on the matrix cores (v_mfma_f32_16x16x4_f32) for r = 3..64,
  // a workgroup per block of 16 heads (HIP-event times, matrix cores / VALU):
  // B16 H32 G8 d128 L4096 82.9 / 91.0 us, B32 H64 G8 d64 L2048 42.0 / 61.0,
  // B32 H64 G4 d64 L2048 25.0 / 62.7, B8 H48 G4 d128 L4096 27.2 / 64.5,
  // B1 H8 G2 d64 L256 6.8 / 8.8; r = 24..64: B16 H48 G2 d128 L4096 33.3 /
  // 88.8, B8 H64 G2 d128 L4096 21.7 / 66.9, B32 H64 G1 d64 L2048 18.9 / 66.8,
  // B4 H64 G1 d128 L8192 23.7 / 75.9.  At r = 2 and r = 1 the kernels
  // themselves tie (B8 H32 G16 d128 L8192 156.9 / 156.0, B16 H16 G8 d128
  // L4096 82.0 / 81.8, B8 H32 G32 d128 L4096 154.8 / 153.5, B16 H32 G32 d128
  // L1024 82.4 / 79.1), and the VALU kernel stays - except on calls of at
  // least 32 MiB whose (b, g) units do not fill whole rounds of 256
  // workgroups (neither divides the other), where the matrix-core plan's
  // split count, chosen to fill whole rounds, wins (graph replays): r = 2
  // B20 H32 G16 d128 L4096 (320 units) 202.4 / 230.7 us, B6 H32 G16 d128
  // L8192 123.1 / 154.2, B3 H32 G16 d128 L8192 65.4 / 80.4, B12 H32 G16 d128
  // L4096 121.8 / 126.3, B40 H32 G16 d128 L2048 196.8 / 199.9; r = 1 B3 H32
  // G32 d128 L8192 121.5 / 151.8, B20 H16 G16 d128 L4096 201.2 / 226.0, B6
  // H32 G32 d128 L4096 120.6 / 123.3.
  const double kv_bytes = 4.0 * B * G * (double)Lmax * d;
  const bool mha_on_mfma = r == 1 && kv_bytes >= 32.0 * 1024 * 1024;
  const long bg = (long)B * G;
  const bool uneven_rounds = bg % 256 != 0 && 256 % bg != 0;
  const bool f32_mfma = dt == GQA_F32 && ((r >= 3 && r <= 64) ||
                                          (r <= 2 && uneven_rounds && 2.0 * kv_bytes >= 32.0 * 1024 * 1024));
  int kind = (dt == GQA_BF16 && ((r >= 2 && r <= 64) || mha_on_mfma)) || f32_mfma ? KIND_MFMA : KIND_VALU;
  if (tu.kernel == 1 + KIND_VALU) kind = KIND_VALU;
  if (tu.kernel == 1 + KIND_MFMA && r <= 64) kind = KIND_MFMA;
  pl->kind = kind;
  pl->NW = 4;
  const int target = tu.target_wgs > 0 ? tu.target_wgs : 256;
  // Split cap: 8192 positions on the matrix cores, measured against 4096 and
  // 6144 (ragged B64 H64 G8 d128 Lmax 32768 715 -> 707 us, B64 H64 G8 L16384
  // 664 -> 652 us, B32 H64 G8 L8192 164.5 -> 159 us, B8 H32 G8 L131072
  // 652 -> 641 us, no shape slower; 6144 leaves odd round counts).
  const int max_chunk = tu.max_chunk > 0 ? tu.max_chunk : (kind == KIND_MFMA ? 8192 : 4096);
  const int chunk_env = tu.chunk;
  const bool target_env = tu.target_wgs > 0;
  const int fused_max = tu.fused_max > 0 ? tu.fused_max : kMaxFusedSplits;
  // Split length for about S splits: the floors (the matrix-core kernel's 4
  // waves take 8 tiles of 32 positions per 256, and shorter splits cost more
  // in epilogue and merge than they gain; the VALU kernel's rows are
  // shorter), at most kMaxSplits splits per sequence (beyond kMaxFusedSplits
  // merged by a second kernel), at most max_chunk positions.
  auto chunk_of = [&](long S) {
    int chunk = (int)round_up((size_t)ceil_div(Lmax, S < 1 ? 1 : S), 32);
    const int min_chunk = kind == KIND_MFMA ? (dt == GQA_F32 ? 64 : 256) : 32;
    if (chunk < min_chunk) chunk = min_chunk;
    const int min_for_merge = (int)round_up((size_t)ceil_div(Lmax, kMaxSplits), 32);
    if (chunk < min_for_merge) chunk = min_for_merge;
    if (chunk > max_chunk) chunk = max_chunk;
    return chunk > Lmax ? Lmax : chunk;
  };
  // Estimated time of a matrix-core launch, in KiB through the busiest
  // compute unit (its memory path moves ~35 GB/s, from L2 or HBM alike):
  // per dispatch round one slab (a split's K and V, bfloat16) plus ~64 KiB of
  // fixed cost (first latency, epilogue); when the sequence is split, ~128
  // KiB for the split protocol's tail (partial stores, arrival) plus the
  // merge - the in-kernel one is a single workgroup reading heads x splits
  // partials at the very end (x4), the wide merge kernel a launch of its own
  // (~128 KiB).
  auto plan_cost = [&](long units, int heads, int chunk) {
    const long S = ceil_div(Lmax, chunk);
    const long rounds = (units * S + 255) / 256;
    double e = rounds * ((double)chunk * d * (dt == GQA_F32 ? 8 : 4) / 1024 + 64.0);
    if (S > 1) e += 128.0 + (S > fused_max ? 128.0 : 4.0 * heads * S * (d + 2) * 4 / 1024);
    return e;
  };
  // VALU kernel, grids of at most one round (256 workgroups): fewer, longer
  // splits where the split protocol costs more than the shorter stream
  // saves.  Estimated time in us: a workgroup streams ~40 KiB of K and V per
  // us plus ~1 us fixed; a split plan adds ~2.5 us for the partial stores,
  // arrival and in-kernel merge, plus ~0.2 us per split the merge reads
  // (~5 us for the separate wide merge kernel).  Candidates: the target's
  // split count halved down to 1.  Measured with HIP-graph replays, cold
  // caches (split count: default -> chosen): B1 H8 G2 d64 L1024 f32
  // 32 -> 8 splits 10.25 -> 8.31 us, B1 H32 G8 d128 L512 f32 16 -> 8
  // 10.07 -> 8.90, B1 H16 G16 d128 L1024 bf16 16 -> 8 10.28 -> 8.15,
  // B4 H32 G32 d64 L512 bf16 2 -> 1 8.45 -> 7.31, B1 H8 G2 d64 L256 f32
  // 8 -> 1 8.31 -> 7.95; B2 H8 G2 d128 L2048 f32 keeps its 64 splits (12.99;
  // 8 splits 18.69).
  auto valu_chunk = [&](long units, int base) {
    const long S0 = ceil_div(Lmax, base);
    if (S0 <= 1 || units * S0 > 256) return base;
    const double kib_per_pos = d * (dt == GQA_F32 ? 8.0 : 4.0) / 1024;
    auto est = [&](int chunk) {
      const long S = ceil_div(Lmax, chunk);
      double e = chunk * kib_per_pos / 40.0 + 1.0;
      if (S > 1) e += S > fused_max ? 5.0 : 2.5 + 0.2 * S;
      return e;
    };
    int best = base;
    double best_e = est(base);
    for (long S = S0 / 2; S >= 1; S /= 2) {
      const int c = chunk_of(S);
      const double e = est(c);
      if (e < best_e) {
        best_e = e;
        best = c;
      }
    }
    return best;
  };
  // Binary32 on the matrix cores, grids of one round: the split count of
  // lowest estimated time among the target's count halved down to 1.  In us:
  // a workgroup streams ~40 KiB of K and V per us (its 16-position tiles
  // take one per wave, so a 64-position split is one tile per wave) and the
  // merging one reads its unit's partials at that rate; ~1.4 us for the
  // split protocol (partial stores, arrival), ~4 us for a separate wide
  // merge kernel, ~0.012 us per workgroup dispatched.  Fitted to HIP-graph
  // replays (split length: us): B1 H8 G2 d64 L256 64: 5.64, 128: 6.61,
  // 256: 6.75; B1 H8 G2 d64 L1024 64: 6.75, 128: 7.19, 256: 8.39; B1 H32 G8
  // d128 L512 64: 7.85, 128: 9.11, 256: 12.24; B2 H32 G8 d128 L1024 64:
  // 11.20, 128: 10.69, 256: 13.01; B4 H32 G8 d128 L1024 128: 11.48, 256: 13.66.
  auto f32_mfma_chunk = [&](long units, int heads, int base) {
    auto est = [&](int chunk) {
      const long S = ceil_div(Lmax, chunk);
      double e = chunk * d * 8.0 / 1024 / 40 + 0.012 * units * S;
      if (S > 1) {
        const double part_kib = (double)heads * S * (d + 2) * 4 / 1024;
        e += 1.4 + ((S > fused_max || part_kib > 96) ? 4.0 : part_kib / 40);
      }
      return e;
    };
    int best = base;
    double best_e = est(base);
    for (long S = ceil_div(Lmax, base) / 2; S >= 1; S /= 2) {
      const int c = chunk_of(S);
      const double e = est(c);
      if (e < best_e) {
        best_e = e;
        best = c;
      }
    }
    return best;
  };
  // Split length for a grid of `units` (b, g, head chunk) units of `heads`
  // query heads each: about `target` workgroups (one per compute unit).  On
  // the matrix cores the split count is then the one of lowest plan_cost
  // among the counts that fill 1..4 rounds of 256 workgroups.  Rounding the
  // count up to fill the GPU leaves a few compute units with two workgroups
  // that set the pace: B6 H32 G8 d128 L4096 (48 units) 6 splits 26.4 us,
  // 5 splits 21.2 us; B5 L16384 78.3 -> 56.2 us; B48 L2048 (384 units)
  // 1 split 72.3 us, 2 splits 64.8 us.  The count stays within the fused
  // merge's limit unless the length needs more.
  auto chunk_for = [&](long units, int heads) {
    if (chunk_env > 0) return chunk_env > Lmax ? Lmax : chunk_env;
    // The VALU kernel on binary32 serving 4 or more heads per row it loads
    // needs several workgroups per compute unit to hide its dependent FMA
    // chains: 768 (B16 H32 G8 d128 L4096 214.8 -> 101.5 us, B12 L2048
    // 80.4 -> 44.0 us); with 1 or 2 heads one per compute unit stays best
    // (B8 H32 G16 d128 L8192: 154.3 us, 166.0 with 768), and on bfloat16
    // (only run there when forced) 768 is slower on the T5-XXL shapes.
    // With 4 heads per row set and the row ring, two workgroups per compute
    // unit do as well where they divide evenly (units dividing 512): binary32
    // Mistral-7B shape 93.1 -> 90.4 us, B4 H32 G8 d128 L8192 56.0 -> 50.6,
    // B32 L1024 52.8 -> 49.7, B1 L32768 57.3 -> 53.1; where they would not
    // (B12 L2048: 576 workgroups, 47.7 against 44.5 us with 768) and with 8
    // heads per row set (B2 H64 G8 d128 L8192 58.7 against 50.5 us) 768 stays.
    long tgt = target;
    if (kind == KIND_VALU && dt == GQA_F32 && heads >= 4 && !target_env)
      tgt = (heads == 4 && 512 % units == 0) ? 512 : 768;
    const int base = chunk_of((tgt + units - 1) / units);
    if (target_env) return base;
    if (kind != KIND_MFMA) return valu_chunk(units, base);
    if (dt == GQA_F32 && units * ceil_div(Lmax, base) <= 256) return f32_mfma_chunk(units, heads, base);
    const long s_max = ceil_div(Lmax, base) > fused_max ? ceil_div(Lmax, base) : (long)fused_max;
    auto est = [&](int chunk) { return plan_cost(units, heads, chunk); };
    int best = base;
    double best_e = est(base);
    for (long k = 1; k <= 4; ++k) {
      for (long S : {256 * k / units, (256 * k + units - 1) / units}) {
        if (S < 1) continue;
        const int c = chunk_of(S);
        if (ceil_div(Lmax, c) > s_max) continue;
        const double e = est(c);
        if (e < best_e) {
          best_e = e;
          best = c;
        }
      }
    }
    return best;
  };
  if (kind == KIND_MFMA) {
    const int hb = (r + 15) / 16;
    const int hb_all = hb <= 1 ? 1 : (hb <= 2 ? 2 : 4);
    // Spread the head blocks over workgroups when there are fewer (b, g)
    // units than compute units: a workgroup's tile loop serves each of its
    // head blocks in turn, so with few units the loop, not HBM, sets the pace.
    int hc = ((long)B * G < 256) ? hb_all : 1;
    auto fit = [&](int h) {  // no chunk without heads
      while (h > 1 && (h - 1) * (hb_all / h) * 16 >= r) h /= 2;
      return h;
    };
    hc = fit(hc);
    if (hc > 1) {
      // Every head chunk reads the whole slab through a compute unit's memory
      // path; fewer chunks read less, more chunks keep the splits, and so the
      // merge, small.  Of the two candidates (1 or 2 chunks for two head
      // blocks, 2 or 4 for four) the one of lower plan_cost wins.  Measured
      // (bf16): 64 heads per K/V head, 2 chunks B64 d64 L4096 29.0 -> 23.2
      // us, B2 d128 L32768 32.9 -> 22.8 us, 4 chunks B4 d64 L8192 12.8 us
      // (19.6 with 2); 32 heads, 1 chunk B4 d128 L16384 25.1 -> 19.0 us,
      // B1 d128 L131072 28.2 -> 23.2 us, 2 chunks B8 d64 L8192 13.1 us
      // (19.5 with 1).
      auto cost = [&](int h) {
        const long units = (long)B * G * h;
        const int heads = (hb_all / h) * 16 < r ? (hb_all / h) * 16 : r;
        return plan_cost(units, heads, chunk_for(units, heads));
      };
      const int other = fit(hc / 2);  // at most two head blocks per workgroup (four measured slower)
      if (other != hc && hb_all / other <= 2 && cost(other) < cost(hc)) hc = other;
    }
    const int hc_env = tu.head_split;
    if (hc_env == 1 || hc_env == 2 || hc_env == 4) hc = fit(hc_env > hb_all ? hb_all : hc_env);
    pl->HC = hc;
    pl->HB = hb_all / hc;
    if (dt == GQA_F32) {  // the binary32 kernel serves one head block: a workgroup per block
      pl->HC = hb;
      pl->HB = 1;
    }
    pl->NW = 4;  // chosen below, once the split length is known
    pl->RC = 0;
  } else {
    pl->RC = next_pow2(r < 8 ? r : 8);
    pl->HC = ceil_div(r, pl->RC);
    pl->HB = 0;
  }
  const long units = (long)B * G * pl->HC;
  const int chunk = chunk_for(units, kind == KIND_MFMA ? (16 * pl->HB < r ? 16 * pl->HB : r) : pl->RC);
  pl->chunk = chunk;
  if (kind == KIND_MFMA) {
    // 4 waves (measured best on every workload with the non-temporal cache
    // stream); 8 or 16 on request where the head blocks fit the register
    // budget of the larger workgroup.
    const int nw_max = dt == GQA_F32 ? 4 : (pl->HB == 1 && d == 64) ? 16 : (pl->HB <= 2 ? 8 : 4);
    const int nw_def = 4;
    const int nw = tu.waves > 0 ? tu.waves : nw_def;
    pl->NW = (nw == 8 || nw == 16) && nw <= nw_max ? nw : 4;
  }
  pl->S = ceil_div(Lmax, chunk);
  const unsigned long long grid = (unsigned long long)units * pl->S;
  if (grid == 0 || grid > 0x7fffffffULL) return GQA_ERR_SIZE;
  pl->grid = (unsigned)grid;
  // In-kernel merge: one counter per unit, and a merging workgroup that
  // reads every split of its heads, which pays up to kMaxFusedSplits; beyond
  // that, or when that one workgroup would read more than 96 KiB of partials
  // through its compute unit, a merge kernel spread over heads, dimensions
  // and splits.  Graph replays, in-kernel / merge kernel: B3 H64 G4 d128
  // L8192 (16 heads x 21 splits, 175 KB) 20.8 / 17.9 us, B4 H64 G4 d128
  // L8192 (133 KB) 21.3 / 20.0 us; at 66 KB and below the in-kernel merge
  // wins (B1 H32 G8 d128 L32768 28.1 / 27.8, B20 H8 G1 d128 L4096 54 KB
  // 13.9 / 14.8, T5-XXL G = 1 34 KB 11.4 / 16.4, Mistral-7B shape 42.5 / 45.5).
  const long partial_bytes = (long)(pl->kind == KIND_MFMA ? (16 * pl->HB < r ? 16 * pl->HB : r) : pl->RC) *
                             pl->S * (d + 2) * 4;
  pl->wide = pl->S > fused_max || (pl->S > 1 && partial_bytes > 96 * 1024);
  pl->fused = units <= kMaxFusedUnits && !pl->wide && !tu.merge_kernel;
  // Grids of several rounds with at least kOrderMinSplits splits per
  // sequence: the order kernel sorts the items largest first (ragged lengths
  // otherwise leave whole splits of the longest sequences to the last round:
  // ragged B64 H64 G8 d128 Lmax 32768, 8 splits, 785 -> 725 us).  It costs
  // each workgroup one dependent load at its start, ~1% on a batch of equal
  // lengths (B64 H32 G16 d128 L8192, 2 splits: 646.7 -> 654.6 us), hence the
  // split floor.
  pl->ordered = (pl->S >= kOrderMinSplits && pl->grid > kOrderMinGrid && tu.order != 0) || (tu.order == 1 && pl->S > 1);
  // Cache loads: non-temporal, or plain where head chunks share the lines in L2.
  pl->nontemporal = tu.temporal >= 0 ? !tu.temporal : pl->HC == 1 || kind != KIND_MFMA;
  pl->contig = tu.contig;
  pl->valu_pieces = tu.valu_pieces;
  pl->arrive_acqrel = tu.arrive_acqrel;
  if (pl->S > 1) {
    pl->ml_off = kCounterBytes;
    pl->o_off = pl->ml_off + round_up((size_t)B * H * pl->S * sizeof(float2), 256);
    pl->order_off = pl->o_off + round_up((size_t)B * H * pl->S * d * sizeof(float), 256);
    pl->ws_bytes = pl->ordered ? pl->order_off + (size_t)pl->grid * sizeof(int)
                               : pl->o_off + (size_t)B * H * pl->S * d * sizeof(float);
  } else {
    pl->ml_off = pl->o_off = pl->order_off = pl->ws_bytes = 0;
  }
  return GQA_OK;
}

// Plans of the last few shapes each host thread used, keyed by the shape and
// the tuning generation (a serving loop repeats a handful of shapes; the
// plan then costs a lookup instead of the estimates).
struct PlanEntry {
  int B, H, G, d, Lmax, dt;
  unsigned gen;  // 0: empty
  gqa_status st;
  Plan plan;
};
constexpr int kPlanCache = 8;
thread_local PlanEntry t_plans[kPlanCache];
thread_local unsigned t_plan_next;

gqa_status get_plan(int B, int H, int G, int d, int Lmax, gqa_dtype dt, Plan *pl) {
  const unsigned gen = g_tuning_gen.load(std::memory_order_acquire);
  for (const PlanEntry &e : t_plans) {
    if (e.gen == gen && e.B == B && e.H == H && e.G == G && e.d == d && e.Lmax == Lmax && e.dt == (int)dt) {
      *pl = e.plan;
      return e.st;
    }
  }
  const gqa_status st = make_plan(B, H, G, d, Lmax, dt, g_tuning, pl);
  PlanEntry &e = t_plans[t_plan_next++ % kPlanCache];
  e = PlanEntry{B, H, G, d, Lmax, (int)dt, gen, st, *pl};
  return st;
}

bool aligned(const void *p, size_t a) { return ((uintptr_t)p % a) == 0; }

// Projection plan: 128-column blocks x k splits; a split takes whole 32-row
// steps.  k is split in a power of two of parts, the largest that keeps the
// grid within one workgroup of 4 waves per compute unit (256) and at least
// two steps per wave: every split adds partial sums that the last workgroup
// of the column block reads back, so more workgroups than compute units
// cost more in that tail than they gain.
struct LinearPlan {
  int KS, ksteps_per_split, NW, TPI;
  unsigned grid;
  size_t ws_bytes;  // counters + partials, 0 when k is not split
};

gqa_status check_linear(int M, int K, int N, gqa_dtype dt) {
  if (dt != GQA_F32 && dt != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (M < 0 || K < 1 || N < 1) return GQA_ERR_SHAPE;
  if (dt != GQA_BF16 || M > 64 || K % 32 != 0 || N % 128 != 0) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

gqa_status make_linear_plan(int M, int K, int N, LinearPlan *pl) {
  const Tuning &tu = g_tuning;
  const int ntile = N / 128;
  const int ksteps = K / 32;
  pl->NW = tu.linear_waves == 8 ? 8 : 4;
  int KS = tu.linear_ksplit;
  if (KS == 0) {
    const int max_ks = ksteps / (2 * pl->NW);
    KS = 1;
    while (2 * KS * ntile <= 256 && 2 * KS <= max_ks) KS *= 2;
  }
  if (KS > ksteps) KS = ksteps;
  pl->ksteps_per_split = ceil_div(ksteps, KS);
  pl->KS = ceil_div(ksteps, pl->ksteps_per_split);
  // steps loaded together: a wave's whole share when it fits the registers
  const int per_wave = ceil_div(pl->ksteps_per_split, pl->NW);
  const int tb = ceil_div(M, 16) > 2 ? 4 : ceil_div(M, 16);
  const int max_tpi = tb == 4 ? 2 : 4;
  pl->TPI = per_wave >= 3 ? 4 : per_wave;
  if (pl->TPI < 1) pl->TPI = 1;
  if (pl->TPI > max_tpi) pl->TPI = max_tpi;
  const int tpi_env = tu.linear_tpi;
  if (tpi_env == 1 || tpi_env == 2 || (tpi_env == 4 && max_tpi == 4)) pl->TPI = tpi_env;
  const unsigned long long grid = (unsigned long long)ntile * pl->KS;
  if (grid == 0 || grid > 0x7fffffffULL || ntile > kMaxFusedUnits) return GQA_ERR_SIZE;
  pl->grid = (unsigned)grid;
  pl->ws_bytes = pl->KS > 1 ? kCounterBytes + (size_t)pl->KS * M * N * sizeof(float) : 0;
  return GQA_OK;
}

gqa_status linear_impl(const void *x, const void *w, void *const y[3], const int seg_lo[4], int nseg, int M, int K,
                       int N, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  LinearPlan pl;
  gqa_status st = make_linear_plan(M, K, N, &pl);
  if (st != GQA_OK) return st;
  if (pl.ws_bytes > 0) {
    if (!workspace) return GQA_ERR_NULL;
    if (workspace_bytes < pl.ws_bytes) return GQA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GQA_ERR_ALIGN;
  }
  gqa::LinearParams p;
  p.x = static_cast<const __bf16 *>(x);
  p.w = static_cast<const __bf16 *>(w);
  for (int i = 0; i < 3; ++i) p.y[i] = static_cast<__bf16 *>(y[i]);
  for (int i = 0; i < 4; ++i) p.seg_lo[i] = seg_lo[i];
  p.nseg = nseg;
  p.ws_cnt = pl.ws_bytes ? static_cast<unsigned *>(workspace) : nullptr;
  p.ws_part = pl.ws_bytes ? reinterpret_cast<float *>(static_cast<char *>(workspace) + kCounterBytes) : nullptr;
  p.M = M;
  p.K = K;
  p.N = N;
  p.KS = pl.KS;
  p.ksteps_per_split = pl.ksteps_per_split;
  const hipError_t e = gqa::launch_linear(p, pl.NW, pl.TPI, pl.grid, stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e);
}

// Packed projections: one workgroup per 16-column strip over all of k, so
// no workspace.  TPI blocks per wave are loaded before they are used.
gqa_status check_packed(int M, int K, int N, gqa_dtype dt) {
  if (dt != GQA_F32 && dt != GQA_BF16) return GQA_ERR_UNSUPPORTED;
  if (M < 0 || K < 1 || N < 1) return GQA_ERR_SHAPE;
  if (dt != GQA_BF16 || M > 64 || K % 32 != 0 || N % 16 != 0) return GQA_ERR_UNSUPPORTED;
  if ((unsigned long long)K * N > (1ULL << 40)) return GQA_ERR_SIZE;
  return GQA_OK;
}

gqa_status check_layer(int B, int H, int G, int d, int Lmax, int window, int d_model, gqa_dtype dtype) {
  gqa_status st = check_shape(B, H, G, d, Lmax, dtype);
  if (st != GQA_OK) return st;
  if (window < 0 || d_model < 1) return GQA_ERR_SHAPE;
  if ((long long)(H + 2LL * G) * d > 0x7fffffffLL) return GQA_ERR_SIZE;
  st = check_packed(B, d_model, (H + 2 * G) * d, dtype);
  if (st == GQA_OK) st = check_packed(B, H * d, d_model, dtype);
  return st;
}

gqa_status packed_impl(const void *x, const void *wp, void *const y[3], const int seg_lo[4], int nseg, int M, int K,
                       int N, hipStream_t stream) {
  gqa::LinearParams p{};
  p.x = static_cast<const __bf16 *>(x);
  p.w = static_cast<const __bf16 *>(wp);
  for (int i = 0; i < 3; ++i) p.y[i] = static_cast<__bf16 *>(y[i]);
  for (int i = 0; i < 4; ++i) p.seg_lo[i] = seg_lo[i];
  p.nseg = nseg;
  p.M = M;
  p.K = K;
  p.N = N;
  // One token tile: 2 or 4 strips per workgroup where one strip each would
  // leave more than ~1.5 workgroups per compute unit, as long as at least
  // 192 workgroups remain (each workgroup reads all of x, so fewer and wider
  // ones read less of it: [4096 x 6144] 12.3 -> 10.7 us with 2 strips);
  // K of 4, 8 or 16 chunks runs the unrolled kernel (measured 0.5-1 us
  // faster than the loop: [4096 x 4096] 7.9 us).  GQA_LINEAR_STRIPS=1|2|4
  // and GQA_LINEAR_UNROLL=0 override.
  const int tb = ceil_div(M, 16) > 2 ? 4 : ceil_div(M, 16);
  const int nstrips = N / 16;
  int sw = 1;
  if (tb == 1) {
    for (int cand : {4, 2})
      if (sw == 1 && nstrips % cand == 0 && nstrips / cand >= 192) sw = cand;
    const int sw_env = g_tuning.linear_strips;
    if ((sw_env == 1 || sw_env == 2 || sw_env == 4) && nstrips % sw_env == 0) sw = sw_env;
  }
  const int kc = gqa::linear_packed_chunk_blocks(tb, sw);
  const int nch = (K / 32) % kc == 0 ? K / 32 / kc : 0;
  const bool unroll = tb == 1 && sw <= 2 && (nch == 4 || nch == 8 || nch == 16) && g_tuning.linear_unroll != 0;
  const hipError_t e = gqa::launch_linear_packed(p, tb, sw, unroll ? nch : 0, stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e);
}

// Workspace of the full decode step (gqa_decode_layer): the decode kernel's
// scratch (counters + split partials; at least the counter region), then q,
// the new keys and values, and the attention output.
struct LayerPlan {
  size_t scratch, q_off, kn_off, vn_off, att_off, total;
};

gqa_status make_layer_plan(int B, int H, int G, int d, int Lmax, int window, int d_model, LayerPlan *lp) {
  (void)d_model;
  Plan ap;
  const int Leff = (window > 0 && window < Lmax) ? window : Lmax;
  gqa_status st = get_plan(B, H, G, d, Leff, GQA_BF16, &ap);
  if (st != GQA_OK) return st;
  // The counter region stays reserved even when the attention needs no
  // split: a workspace may be shared with other calls, which rely on its
  // first kCounterBytes holding zeroed counters.
  const size_t scratch = ap.ws_bytes > kCounterBytes ? ap.ws_bytes : kCounterBytes;
  lp->scratch = round_up(scratch, 256);
  lp->q_off = lp->scratch;
  lp->kn_off = lp->q_off + round_up((size_t)B * H * d * 2, 256);
  lp->vn_off = lp->kn_off + round_up((size_t)B * G * d * 2, 256);
  lp->att_off = lp->vn_off + round_up((size_t)B * G * d * 2, 256);
  lp->total = lp->att_off + round_up((size_t)B * H * d * 2, 256);
  return GQA_OK;
}

}  // namespace

extern "C" {

size_t gqa_decode_workspace_size(int B, int H, int G, int d, int Lmax, gqa_dtype dtype) {
  if (check_shape(B, H, G, d, Lmax, dtype) != GQA_OK || B == 0) return 0;
  Plan pl;
  if (get_plan(B, H, G, d, Lmax, dtype, &pl) != GQA_OK) return 0;
  return pl.ws_bytes;
}

int gqa_decode_kernel_kind(int B, int H, int G, int d, int Lmax, gqa_dtype dtype) {
  if (check_shape(B, H, G, d, Lmax, dtype) != GQA_OK) return -1;
  Plan pl;
  if (get_plan(B > 0 ? B : 1, H, G, d, Lmax, dtype, &pl) != GQA_OK) return -1;
  return pl.kind;
}

void gqa_tuning_reload(void) {
  g_tuning = read_tuning();
  g_tuning_gen.fetch_add(1, std::memory_order_acq_rel);
}

gqa_status gqa_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream) {
  if (workspace_bytes == 0) return GQA_OK;
  if (!workspace) return GQA_ERR_NULL;
  const hipError_t e = gqa::launch_fill_zero(workspace, workspace_bytes, stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e);
}

}  // extern "C"

namespace {

// Shared body of the decode entry points.  k_new / v_new (both or neither)
// switch on the cache append; window > 0 the sliding window.
gqa_status decode_impl(int phase, const void *q, const void *k_new, const void *v_new, const void *k_cache,
                       const void *v_cache, const int32_t *seq_lens, int B, int H, int G, int d, int Lmax,
                       int window, float scale, gqa_dtype dtype, void *out, void *workspace,
                       size_t workspace_bytes, hipStream_t stream) {
  if (phase != 0 && phase != 1 && phase != 2) return GQA_ERR_UNSUPPORTED;
  gqa_status st = check_shape(B, H, G, d, Lmax, dtype);
  if (st != GQA_OK) return st;
  if (window < 0) return GQA_ERR_SHAPE;
  if (B == 0) return GQA_OK;
  if (!q || !k_cache || !v_cache || !seq_lens || !out) return GQA_ERR_NULL;
  if ((k_new == nullptr) != (v_new == nullptr)) return GQA_ERR_NULL;
  if (!aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(out, 16) || !aligned(seq_lens, 4))
    return GQA_ERR_ALIGN;
  if (k_new && (!aligned(k_new, 16) || !aligned(v_new, 16))) return GQA_ERR_ALIGN;
  const double sl2 = (double)scale * 1.4426950408889634;
  if (!isfinite(scale) || !isfinite((float)sl2)) return GQA_ERR_SCALE;
  // a window shorter than the cache plans splits over the window only
  const int Leff = (window > 0 && window < Lmax) ? window : Lmax;
  Plan pl;
  st = get_plan(B, H, G, d, Leff, dtype, &pl);
  if (st != GQA_OK) return st;
  if (pl.ws_bytes > 0) {
    if (!workspace) return GQA_ERR_NULL;
    if (workspace_bytes < pl.ws_bytes) return GQA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return GQA_ERR_ALIGN;
  }

  gqa::DecodeParams p;
  p.q = q;
  p.k = k_cache;
  p.v = v_cache;
  p.k_new = k_new;
  p.v_new = v_new;
  p.seq_lens = seq_lens;
  p.out = out;
  char *ws = static_cast<char *>(workspace);
  p.ws_cnt = pl.ws_bytes ? reinterpret_cast<unsigned *>(ws) : nullptr;
  p.ws_ml = pl.ws_bytes ? reinterpret_cast<float2 *>(ws + pl.ml_off) : nullptr;
  p.ws_o = pl.ws_bytes ? reinterpret_cast<float *>(ws + pl.o_off) : nullptr;
  int *order = pl.ordered ? reinterpret_cast<int *>(ws + pl.order_off) : nullptr;
  p.order = order;
  p.fused = pl.fused;
  p.contig = pl.contig;
  p.arrive_acqrel = pl.arrive_acqrel;
  p.B = B;
  p.H = H;
  p.G = G;
  p.Lmax = Lmax;
  p.window = window;
  p.r = H / G;
  p.S = pl.S;
  p.chunk = pl.chunk;
  p.HC = pl.HC;
  p.scale_log2 = (float)sl2;

  if (phase != 2 && order) {
    const hipError_t e = gqa::launch_order(p, pl.kind == KIND_VALU, pl.grid, order, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (phase != 2) {
    const hipError_t e =
        pl.kind != KIND_MFMA ? gqa::launch_decode_valu(p, (int)dtype, d, pl.RC, pl.valu_pieces, pl.grid, stream)
        : dtype == GQA_F32   ? gqa::launch_decode_mfma_f32(p, d, pl.nontemporal, pl.grid, stream)
                             : gqa::launch_decode_mfma(p, d, pl.HB, pl.NW, pl.nontemporal, pl.grid, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  if (phase != 1 && pl.S > 1 && !pl.fused) {
    // up to kMaxFusedSplits: one merge workgroup per (sequence, K/V head), all
    // r heads of the group (the in-kernel merge's arithmetic); beyond, the
    // wide merge kernel
    const hipError_t e = pl.wide ? gqa::launch_merge_wide(p, (int)dtype, d, stream)
                                 : gqa::launch_merge(p, (int)dtype, d, p.r, stream);
    if (e != hipSuccess) return hip_fail(e);
  }
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_decode_phase(int phase, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *seq_lens, int B, int H, int G, int d, int Lmax, float scale,
                            gqa_dtype dtype, void *out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(phase, q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, H, G, d, Lmax, 0, scale, dtype, out,
                     workspace, workspace_bytes, stream);
}

gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens, int B, int H,
                      int G, int d, int Lmax, float scale, gqa_dtype dtype, void *out, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  return decode_impl(0, q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, H, G, d, Lmax, 0, scale, dtype, out,
                     workspace, workspace_bytes, stream);
}

}  // extern "C"

// The no-allocation entry point's scratch: split partials, arrival counters
// and dispatch order of gqa_decode_noalloc, one copy on every GPU the library
// runs on, held until the process ends.  Host code never passes this name to
// a kernel (on the host it is only a stand-in for the device copy): each
// device's address comes from hipGetSymbolAddress, taken once with that
// device current.
static __device__ __align__(256) unsigned char scratch[GQA_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxScratchDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxScratchDevices];  // device address of `scratch`, per device (null: not set up)

// The scratch of the device that `stream` belongs to; on the first call on
// that device the address is looked up and the counter region cleared by a
// fill kernel enqueued on `stream` (ordered before the decode that follows;
// the kernels leave the counters zero again after every call).
gqa_status scratch_for(hipStream_t stream, void **ptr) {
  int dev = -1;
  hipError_t e = stream ? hipStreamGetDevice(stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= kMaxScratchDevices) return GQA_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    int cur = -1;
    e = hipGetDevice(&cur);
    if (e != hipSuccess) return hip_fail(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return hip_fail(e);
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return hip_fail(e);
    if (e2 != hipSuccess) return hip_fail(e2);
    if (!p || !aligned(p, 256)) return GQA_ERR_ALIGN;
    e = gqa::launch_fill_zero(p, kCounterBytes, stream);
    if (e != hipSuccess) return hip_fail(e);
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return GQA_OK;
}

}  // namespace

extern "C" {

gqa_status gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                              int B, int H, int G, int d, int Lmax, float scale, gqa_dtype dtype, void *out,
                              hipStream_t stream) {
  gqa_status st = check_shape(B, H, G, d, Lmax, dtype);
  if (st != GQA_OK) return st;
  if (B == 0) return GQA_OK;
  Plan pl;
  st = get_plan(B, H, G, d, Lmax, dtype, &pl);
  if (st != GQA_OK) return st;
  if (pl.ws_bytes > GQA_NOALLOC_SCRATCH_BYTES) return GQA_ERR_WORKSPACE;
  void *ws = nullptr;
  if (pl.ws_bytes > 0 && (st = scratch_for(stream, &ws)) != GQA_OK) return st;
  return decode_impl(0, q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, H, G, d, Lmax, 0, scale, dtype, out, ws,
                     ws ? (size_t)GQA_NOALLOC_SCRATCH_BYTES : 0, stream);
}

gqa_status gqa_decode_window(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                             int B, int H, int G, int d, int Lmax, int window, float scale, gqa_dtype dtype,
                             void *out, void *workspace, size_t workspace_bytes, hipStream_t stream) {
  const gqa_status st = check_shape(B, H, G, d, Lmax, dtype);
  if (st != GQA_OK) return st;
  if (window < 1) return GQA_ERR_SHAPE;
  return decode_impl(0, q, nullptr, nullptr, k_cache, v_cache, seq_lens, B, H, G, d, Lmax, window, scale, dtype,
                     out, workspace, workspace_bytes, stream);
}

gqa_status gqa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                             const int32_t *seq_lens, int B, int H, int G, int d, int Lmax, int window, float scale,
                             gqa_dtype dtype, void *out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream) {
  const gqa_status st = check_shape(B, H, G, d, Lmax, dtype);
  if (st != GQA_OK) return st;
  if (window < 0) return GQA_ERR_SHAPE;
  if (B > 0 && (!k_new || !v_new)) return GQA_ERR_NULL;
  return decode_impl(0, q, k_new, v_new, k_cache, v_cache, seq_lens, B, H, G, d, Lmax, window, scale, dtype, out,
                     workspace, workspace_bytes, stream);
}

size_t gqa_linear_workspace_size(int M, int K, int N, gqa_dtype dtype) {
  if (check_linear(M, K, N, dtype) != GQA_OK || M == 0) return 0;
  LinearPlan pl;
  return make_linear_plan(M, K, N, &pl) == GQA_OK ? pl.ws_bytes : 0;
}

gqa_status gqa_linear(const void *x, const void *w, void *y, int M, int K, int N, gqa_dtype dtype, void *workspace,
                      size_t workspace_bytes, hipStream_t stream) {
  const gqa_status st = check_linear(M, K, N, dtype);
  if (st != GQA_OK) return st;
  if (M == 0) return GQA_OK;
  if (!x || !w || !y) return GQA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w, 16) || !aligned(y, 16)) return GQA_ERR_ALIGN;
  void *ys[3] = {y, nullptr, nullptr};
  const int seg[4] = {0, N, N, N};
  return linear_impl(x, w, ys, seg, 1, M, K, N, workspace, workspace_bytes, stream);
}

gqa_status gqa_pack_weight(const void *w, void *w_packed, int K, int N, gqa_dtype dtype, hipStream_t stream) {
  const gqa_status st = check_packed(1, K, N, dtype);
  if (st != GQA_OK) return st;
  if (!w || !w_packed) return GQA_ERR_NULL;
  if (!aligned(w, 2) || !aligned(w_packed, 16)) return GQA_ERR_ALIGN;
  if (((unsigned long long)K * N / 8 + 255) / 256 > 0x7fffffffULL) return GQA_ERR_SIZE;
  const hipError_t e = gqa::launch_pack_weight(w, w_packed, K, N, stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e);
}

gqa_status gqa_linear_packed(const void *x, const void *w_packed, void *y, int M, int K, int N, gqa_dtype dtype,
                             hipStream_t stream) {
  const gqa_status st = check_packed(M, K, N, dtype);
  if (st != GQA_OK) return st;
  if (M == 0) return GQA_OK;
  if (!x || !w_packed || !y) return GQA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_packed, 16) || !aligned(y, 16)) return GQA_ERR_ALIGN;
  void *ys[3] = {y, nullptr, nullptr};
  const int seg[4] = {0, N, N, N};
  return packed_impl(x, w_packed, ys, seg, 1, M, K, N, stream);
}

size_t gqa_decode_layer_workspace_size(int B, int H, int G, int d, int Lmax, int window, int d_model,
                                       gqa_dtype dtype) {
  if (check_layer(B, H, G, d, Lmax, window, d_model, dtype) != GQA_OK || B == 0) return 0;
  LayerPlan lp;
  return make_layer_plan(B, H, G, d, Lmax, window, d_model, &lp) == GQA_OK ? lp.total : 0;
}

gqa_status gqa_decode_layer(const void *x, const void *w_qkv_packed, const void *w_o_packed, void *k_cache,
                            void *v_cache, const int32_t *seq_lens, int B, int H, int G, int d, int Lmax, int window,
                            int d_model, float scale, gqa_dtype dtype, void *y, void *workspace,
                            size_t workspace_bytes, hipStream_t stream) {
  gqa_status st = check_layer(B, H, G, d, Lmax, window, d_model, dtype);
  if (st != GQA_OK) return st;
  if (B == 0) return GQA_OK;
  if (!x || !w_qkv_packed || !w_o_packed || !k_cache || !v_cache || !seq_lens || !y || !workspace)
    return GQA_ERR_NULL;
  if (!aligned(x, 16) || !aligned(w_qkv_packed, 16) || !aligned(w_o_packed, 16) || !aligned(y, 16))
    return GQA_ERR_ALIGN;
  if (!aligned(workspace, 256)) return GQA_ERR_ALIGN;
  LayerPlan lp;
  st = make_layer_plan(B, H, G, d, Lmax, window, d_model, &lp);
  if (st != GQA_OK) return st;
  if (workspace_bytes < lp.total) return GQA_ERR_WORKSPACE;
  char *ws = static_cast<char *>(workspace);
  void *q = ws + lp.q_off, *kn = ws + lp.kn_off, *vn = ws + lp.vn_off, *att = ws + lp.att_off;
  // 1. q, key, val = x @ [Wq | Wk | Wv], written as three tensors
  void *ys[3] = {q, kn, vn};
  const int seg[4] = {0, H * d, (H + G) * d, (H + 2 * G) * d};
  st = packed_impl(x, w_qkv_packed, ys, seg, 3, B, d_model, (H + 2 * G) * d, stream);
  if (st != GQA_OK) return st;
  // 2. append the new key/value to the caches, attend
  st = decode_impl(0, q, kn, vn, k_cache, v_cache, seq_lens, B, H, G, d, Lmax, window, scale, dtype, att, ws,
                   lp.scratch, stream);
  if (st != GQA_OK) return st;
  // 3. y = out @ Wo
  void *yo[3] = {y, nullptr, nullptr};
  const int seg_o[4] = {0, d_model, d_model, d_model};
  return packed_impl(att, w_o_packed, yo, seg_o, 1, B, H * d, d_model, stream);
}

gqa_status gqa_meanpool_kv(const float *w, int d_model, int H, int G, int h, float *w_out, hipStream_t stream) {
  if (d_model < 0 || H < 1 || G < 1 || H % G != 0) return GQA_ERR_SHAPE;
  if (h < 1) return GQA_ERR_UNSUPPORTED;
  if (d_model == 0) return GQA_OK;
  if (!w || !w_out) return GQA_ERR_NULL;
  if (!aligned(w, 4) || !aligned(w_out, 4)) return GQA_ERR_ALIGN;
  const unsigned long long total = (unsigned long long)d_model * G * h;
  if ((unsigned long long)d_model * H * h > (1ULL << 40) || (total + 255) / 256 > 0x7fffffffULL) return GQA_ERR_SIZE;
  const hipError_t e = gqa::launch_meanpool(w, d_model, H, G, h, w_out, stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e);
}

const char *gqa_status_string(gqa_status s) {
  switch (s) {
    case GQA_OK: return "ok";
    case GQA_ERR_NULL: return "a required pointer is NULL";
    case GQA_ERR_SHAPE: return "invalid shape (sizes must be positive and H divisible by G)";
    case GQA_ERR_UNSUPPORTED: return "unsupported head dimension or dtype";
    case GQA_ERR_ALIGN: return "pointer not aligned (16 bytes for tensors, 256 for the workspace)";
    case GQA_ERR_WORKSPACE: return "workspace smaller than gqa_decode_workspace_size()";
    case GQA_ERR_SCALE: return "scale is not finite";
    case GQA_ERR_HIP: return "HIP runtime error";
    case GQA_ERR_SIZE: return "problem size exceeds the supported index range";
  }
  return "unknown status";
}

gqa_status gqa_stream_read(const void *buf, size_t bytes, int nontemporal, int grid, unsigned *sink,
                           hipStream_t stream) {
  if (grid < 0 || grid > 1 << 20) return GQA_ERR_SHAPE;
  if (bytes == 0) return GQA_OK;
  if (!buf || !sink) return GQA_ERR_NULL;
  if (!aligned(buf, 16) || bytes % 16 != 0) return GQA_ERR_ALIGN;
  const hipError_t e = gqa::launch_stream_read(buf, bytes, nontemporal != 0, grid == 0 ? 2048u : (unsigned)grid, sink,
                                               stream);
  return e == hipSuccess ? GQA_OK : hip_fail(e);
}

const char *gqa_last_hip_error(void) { return g_last_hip_error.c_str(); }

}  // extern "C"
