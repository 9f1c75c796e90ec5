/*
 * gqa.h - grouped-query decode attention on AMD Instinct MI355X (gfx950).
 *
 * C ABI of libgqa.so.  Plain pointers and sizes; device buffers are owned by
 * the caller.  The library never allocates, frees or synchronises; every call
 * only enqueues work on the given HIP stream and returns.
 *
 * What is computed (sources are the public pages on grouped-query attention,
 * cited by title and section):
 *   wikillm "Grouped-query attention (GQA)", Overview and Implementation
 *   sketch (decode-step block): the H query heads form G groups; each query
 *   head attends with its group's single key head and value head over every
 *   cached position:
 *       out[b,h,:] = sum_t softmax_t( scale * q[b,h,:] . K[b,g,t,:] ) * V[b,g,t,:]
 *   with g = h / (H/G) - the block assignment of consecutive query heads to a
 *   group that the sketch assumes (the paper does not state it).
 *   elemedex glossary "grouped-query attention", paragraph "Grouped (GQA)":
 *   G = 1 is multi-query attention, G = H is multi-head attention; both are
 *   ordinary calls of the same entry point.
 *
 * Conventions shared by all entry points:
 *   - Tensors are dense, row-major, contiguous; element type per gqa_dtype.
 *   - Argument errors are reported on the host, before anything is enqueued.
 *   - GQA_ERR_HIP means a HIP launch or runtime call failed; the HIP error
 *     text is available from gqa_last_hip_error().
 *   - Nothing throws across the ABI.  Calls are reentrant; two calls that
 *     share one workspace must not overlap in time (use one stream).
 */
#ifndef GQA_H_
#define GQA_H_

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  GQA_F32 = 0,  /* IEEE binary32 */
  GQA_BF16 = 1  /* bfloat16: the upper 16 bits of a binary32 */
} gqa_dtype;

typedef enum {
  GQA_OK = 0,
  GQA_ERR_NULL = 1,        /* a required pointer is NULL */
  GQA_ERR_SHAPE = 2,       /* a size is negative, H, G, d or Lmax < 1, or H % G != 0 */
  GQA_ERR_UNSUPPORTED = 3, /* d not in {64, 128} (or h < 1 for meanpool), unknown dtype */
  GQA_ERR_ALIGN = 4,       /* q, k_cache, v_cache or out not 16-byte aligned; workspace not 256-byte aligned */
  GQA_ERR_WORKSPACE = 5,   /* workspace_bytes < gqa_decode_workspace_size(...) */
  GQA_ERR_SCALE = 6,       /* scale is NaN or infinite */
  GQA_ERR_HIP = 7,         /* a HIP call failed */
  GQA_ERR_SIZE = 8         /* a size product overflows the supported index range */
} gqa_status;

/*
 * Bytes of device workspace that gqa_decode needs for this shape (0 when it
 * needs none).  The workspace holds per-split partial results and, in its
 * first 256 KiB, arrival counters.  Returns 0 for arguments gqa_decode would
 * reject.
 */
size_t gqa_decode_workspace_size(int B, int H, int G, int d, int Lmax, gqa_dtype dtype);

/*
 * Clears a workspace before its first use (enqueues a fill kernel on
 * `stream`; the same as filling it with zero bytes).  Every completed
 * gqa_decode call leaves the counter region zero again, so a cleared
 * workspace serves any number of later calls, of any shape whose size
 * requirement it meets.  workspace_bytes = 0 is a no-op.
 */
gqa_status gqa_workspace_init(void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Grouped-query decode attention for one new token per sequence.
 *
 *   q         [B, H, d]        dtype, device.  Query heads of the new token.
 *   k_cache   [B, G, Lmax, d]  dtype, device.  Key cache; K/V head g of
 *   v_cache   [B, G, Lmax, d]  sequence b is one contiguous Lmax*d slab.
 *   seq_lens  [B] int32, device.  Positions 0 .. seq_lens[b]-1 are attended;
 *             the new token's key/value must already be in the cache (the
 *             sketch appends before attending).  Values are clamped to
 *             [0, Lmax] on the device; 0 gives out[b] = 0.  Positions at or
 *             beyond seq_lens[b] never reach the output (a workgroup may
 *             prefetch one 32-row tile below Lmax before the length is
 *             known and discards it if it crosses the length).
 *   B, H, G, d, Lmax  B >= 0 (B = 0 is a no-op; pointers are then not
 *             checked), H >= 1, G >= 1, H % G == 0, d in {64, 128}, Lmax >= 1.
 *   scale     multiplies q . k before the softmax (1/sqrt(d) in the pages'
 *             sketch); must be finite.
 *   dtype     element type of q, k_cache, v_cache and out.
 *   out       [B, H, d] dtype, device.  Must not alias the inputs.  Rounded
 *             once (to nearest even) from binary32 accumulation.
 *   workspace device buffer of workspace_bytes >= gqa_decode_workspace_size
 *             (may be NULL when that size is 0), 256-byte aligned, cleared
 *             once before first use (gqa_workspace_init or any zero fill),
 *             and owned by this call until the work completes on `stream`.
 *   stream    HIP stream the work is enqueued on (NULL: the null stream).
 *
 * Enqueues the decode kernel: a workgroup per (sequence, K/V head, context
 * split) streams that part of the cache once for all query heads of the group
 * (with few (sequence, K/V head) units, the group's heads are spread over 2
 * or 4 workgroups that read the same part); when a sequence spans several
 * splits (at most 256), the workgroup that finishes its unit last merges the
 * split results (log-sum-exp) into out.  Beyond 32 splits per sequence or
 * above 65536 units a second kernel does that merge instead (beyond 32
 * splits one spread over sequences, heads, dimensions and slices of the
 * splits).  Grids of more than 1024 workgroups with at least 4 splits per
 * sequence are preceded by a one-workgroup kernel that orders their work
 * items largest first (from seq_lens, on the device; the outputs do not
 * depend on it).  The launch plan depends only on the shape and dtype (and
 * on the tuning overrides of gqa_measure.h, read when the library loads).  The call
 * allocates nothing, does not synchronise and issues no memset, so it can be
 * captured into a HIP graph (with a workspace cleared beforehand).
 * NaN or Inf inside the attended positions propagate to the output.
 */
gqa_status gqa_decode(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                      int B, int H, int G, int d, int Lmax, float scale, gqa_dtype dtype, void *out,
                      void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gqa_decode in two phases, for callers that schedule or time them apart:
 * phase 1 enqueues the split kernel (which completes out by itself unless the
 * merge runs as a separate kernel), phase 2 only that separate merge kernel
 * (nothing when it is not needed), phase 0 both - exactly gqa_decode.  Phase 2
 * must follow phase 1 of the same arguments on the same stream with the
 * workspace untouched in between.  Other arguments and status codes as for
 * gqa_decode; an unknown phase gives GQA_ERR_UNSUPPORTED.
 */
gqa_status gqa_decode_phase(int phase, const void *q, const void *k_cache, const void *v_cache,
                            const int32_t *seq_lens, int B, int H, int G, int d, int Lmax, float scale,
                            gqa_dtype dtype, void *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * gqa_decode for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): no
 * workspace argument.  The split partials, arrival counters and dispatch
 * order live in a scratch array of GQA_NOALLOC_SCRATCH_BYTES inside the
 * library, one per GPU, which each GPU the library runs on holds until the
 * process ends.  The plan, the kernels and so the results are those of
 * gqa_decode with a workspace.
 *   Returns GQA_ERR_WORKSPACE when the shape's plan needs more than the
 *   scratch holds (gqa_decode_workspace_size(...) > GQA_NOALLOC_SCRATCH_BYTES);
 *   other arguments and status codes as for gqa_decode.
 *   The first call on a device looks the scratch up (with that device made
 *   current for the lookup) and enqueues a fill kernel on `stream` that clears
 *   its counters; every completed call leaves them zero again.
 *   All calls on one GPU share its scratch: calls that overlap in time on one
 *   GPU (on different streams or from several threads) race and give wrong
 *   results; order them on one stream.  The call allocates and frees nothing.
 */
#define GQA_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
gqa_status gqa_decode_noalloc(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                              int B, int H, int G, int d, int Lmax, float scale, gqa_dtype dtype, void *out,
                              hipStream_t stream);

/*
 * Sliding-window decode: as gqa_decode, but sequence b attends only its last
 * `window` cached positions, [max(0, len_b - window), len_b).  The wikillm
 * page "Grouped-query attention (GQA)" (Variants, decoder-only models) notes
 * that Mistral 7B pairs GQA with sliding-window attention, which the GQA
 * paper does not cover; this is the plain reading of a window of `window`
 * positions ending at the new token.
 *   window >= 1 (GQA_ERR_SHAPE otherwise).  Positions before the window are
 *   not read.  Workspace: gqa_decode_workspace_size(B, H, G, d,
 *   min(Lmax, window), dtype) bytes; other arguments as for gqa_decode.
 */
gqa_status gqa_decode_window(const void *q, const void *k_cache, const void *v_cache, const int32_t *seq_lens,
                             int B, int H, int G, int d, int Lmax, int window, float scale, gqa_dtype dtype,
                             void *out, void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * Decode with the cache append of the decode-step block (wikillm "Grouped-
 * query attention (GQA)", Implementation sketch: the new token's G key heads
 * and G value heads are appended to the cache, then attended) in one launch:
 *   k_new, v_new  [B, G, d] dtype, device (16-byte aligned): the new token's
 *                 keys and values.
 *   k_cache, v_cache  [B, G, Lmax, d], updated in place: row len_b - 1 of each
 *                 (b, g) slab receives k_new[b, g] / v_new[b, g], where
 *                 len_b = clamp(seq_lens[b], 0, Lmax) counts the new token;
 *                 nothing else in the caches is written.  len_b = 0 appends
 *                 nothing and gives out[b] = 0.
 *   window        0 for none, else as for gqa_decode_window (workspace sized
 *                 with min(Lmax, window) then).
 * The output equals gqa_decode (or gqa_decode_window) over the updated
 * caches.  Other arguments as for gqa_decode.
 */
gqa_status gqa_decode_append(const void *q, const void *k_new, const void *v_new, void *k_cache, void *v_cache,
                             const int32_t *seq_lens, int B, int H, int G, int d, int Lmax, int window, float scale,
                             gqa_dtype dtype, void *out, void *workspace, size_t workspace_bytes,
                             hipStream_t stream);

/*
 * Projection of the decode-step block (wikillm "Grouped-query attention
 * (GQA)", Implementation sketch: q = x Wq, key = x Wk, val = x Wv, and the
 * output projection Wo), for a batch of M tokens:
 *   y[M, N] = x[M, K] @ w[K, N]
 *   x  [M, K] bfloat16, row-major, device, 16-byte aligned; one row per token.
 *   w  [K, N] bfloat16, row-major, device, 16-byte aligned (read once).
 *   y  [M, N] bfloat16, device, 16-byte aligned; each element is the binary32
 *      sum rounded once to bfloat16 (nearest even).
 *   M in 0..64 (M = 0 is a no-op), K a multiple of 32, N a multiple of 128,
 *   dtype GQA_BF16 (GQA_ERR_UNSUPPORTED otherwise; GQA_ERR_SHAPE for K or
 *   N < 1 or M < 0).
 *   workspace  gqa_linear_workspace_size(M, K, N, dtype) bytes (0: may be
 *      NULL), cleared once with gqa_workspace_init, 256-byte aligned; when K is
 *      split across workgroups it holds arrival counters (left at zero after
 *      each call) and binary32 partial sums, added in a fixed order, so
 *      results are deterministic.  Calls that share a workspace must be
 *      ordered (one stream).
 * Status codes as for gqa_decode.
 */
size_t gqa_linear_workspace_size(int M, int K, int N, gqa_dtype dtype);
gqa_status gqa_linear(const void *x, const void *w, void *y, int M, int K, int N, gqa_dtype dtype, void *workspace,
                      size_t workspace_bytes, hipStream_t stream);

/*
 * Weight layout for the matrix cores (a one-time conversion of a model's
 * projection weights, like gqa_meanpool_kv): w [K, N] bfloat16 row-major is
 * rewritten into w_packed (same size, K*N*2 bytes) as 32 x 16 blocks:
 *   block (kb, nb), kb < K/32, nb < N/16, starts at element (kb*(N/16) + nb)*512;
 *   inside it, element 8*l + e (l = 16c + n, c < 4, n < 16, e < 8) is
 *   w[32kb + 8c + e][16nb + n].
 * A wave then fetches the A operand of one v_mfma_f32_16x16x32_bf16 as one
 * contiguous 1 KiB load, and the workgroups of the product (one per 16-column
 * strip) together read contiguous bands of rows.
 *   K a multiple of 32, N a multiple of 16, dtype GQA_BF16
 *   (GQA_ERR_UNSUPPORTED otherwise; GQA_ERR_SHAPE for K or N < 1).
 *   w 2-byte aligned, w_packed 16-byte aligned, not overlapping.
 * Status codes as for gqa_decode.
 */
gqa_status gqa_pack_weight(const void *w, void *w_packed, int K, int N, gqa_dtype dtype, hipStream_t stream);

/*
 * gqa_linear over a packed weight (gqa_pack_weight): y[M, N] = x[M, K] @ W.
 * Each workgroup reads 1, 2 or 4 adjacent 16-column strips once over all of
 * K, so no workspace is needed and each output is one binary32 sum (in an
 * order fixed by the shape) rounded once to bfloat16.
 *   x [M, K], y [M, N] bfloat16 row-major, 16-byte aligned; M in 0..64
 *   (0 is a no-op); K a multiple of 32; N a multiple of 16; dtype GQA_BF16.
 * Status codes as for gqa_linear.
 */
gqa_status gqa_linear_packed(const void *x, const void *w_packed, void *y, int M, int K, int N, gqa_dtype dtype,
                             hipStream_t stream);

/*
 * The whole decode-step block of wikillm "Grouped-query attention (GQA)"
 * (Implementation sketch) for B sequences, one new token each, enqueued as
 * three kernels on `stream`:
 *   1. [q | key | val] = x @ w_qkv           (gqa_linear_packed, output split in three)
 *   2. key/val appended at row len_b - 1 of the caches; out = attention
 *      (gqa_decode_append, with `window` as there)
 *   3. y = out @ w_o                           (gqa_linear_packed)
 *   x             [B, d_model] bfloat16, device: the token's hidden state.
 *   w_qkv_packed  [d_model, (H + 2G) d] bfloat16 in the packed layout
 *                 (gqa_pack_weight): columns H d of query heads, then G d of
 *                 key heads, then G d of value heads (head i owns d columns).
 *   w_o_packed    [H d, d_model] bfloat16, packed.
 *   k_cache, v_cache, seq_lens, B, H, G, d, Lmax, window, scale: as for
 *                 gqa_decode_append (caches updated in place).
 *   y             [B, d_model] bfloat16.
 * q, key, val and out are rounded to bfloat16 between the steps (they live in
 * the workspace).  dtype must be GQA_BF16, B <= 64 and d_model a multiple of
 * 32 (GQA_ERR_UNSUPPORTED otherwise).  Other status codes as for gqa_decode.
 * Workspace: gqa_decode_layer_workspace_size(...) bytes, 256-byte aligned,
 * cleared once with gqa_workspace_init.
 */
size_t gqa_decode_layer_workspace_size(int B, int H, int G, int d, int Lmax, int window, int d_model,
                                       gqa_dtype dtype);
gqa_status gqa_decode_layer(const void *x, const void *w_qkv_packed, const void *w_o_packed, void *k_cache,
                            void *v_cache, const int32_t *seq_lens, int B, int H, int G, int d, int Lmax, int window,
                            int d_model, float scale, gqa_dtype dtype, void *y, void *workspace,
                            size_t workspace_bytes, hipStream_t stream);

/*
 * The pages' checkpoint conversion step, numeric core only: wikillm
 * "Grouped-query attention (GQA)", Implementation sketch (conversion block)
 * and Variants ("Converted and uptrained checkpoints"): the key (or value)
 * projection columns of the H/G heads of each group are mean-pooled.
 *
 *   w      [d_model, H*h] binary32, device; head i owns columns i*h .. (i+1)*h-1.
 *   w_out  [d_model, G*h] binary32, device; column block g is the mean of the
 *          blocks of heads g*r .. g*r+r-1, r = H/G (block assignment).
 *
 * Arithmetic (bit-exact, deterministic): binary64 sum of the members in
 * ascending head order starting from the first member, one binary64 division
 * by r, one rounding to binary32 (nearest even).  Call once for W_K and once
 * for W_V; W_Q and W_O are left as they are.  d_model = 0 is a no-op.
 */
gqa_status gqa_meanpool_kv(const float *w, int d_model, int H, int G, int h, float *w_out, hipStream_t stream);

/* Static description of a status code. */
const char *gqa_status_string(gqa_status status);

/* Text of the HIP error behind the last GQA_ERR_HIP in this thread ("" if none). */
const char *gqa_last_hip_error(void);

/*
 * Which decode kernel a shape runs on: 0 = VALU kernel (binary32 or bfloat16
 * dot products on the vector ALUs), 1 = a matrix-core kernel (bfloat16, or
 * binary32 with 3..64 query heads per K/V head).  Returns -1 for arguments
 * gqa_decode would reject.  (The tuning override GQA_KERNEL=valu|mfma of
 * gqa_measure.h forces a kernel; mfma up to 64 query heads per K/V head.)
 */
int gqa_decode_kernel_kind(int B, int H, int G, int d, int Lmax, gqa_dtype dtype);

#ifdef __cplusplus
}
#endif

#endif /* GQA_H_ */
