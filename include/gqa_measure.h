/*
 * gqa_measure.h - measurement and tuning utilities of libgqa.so.
 *
 * Not part of the decode path: a read-only streaming probe that gives the
 * practical HBM read ceiling the decode kernels are measured against, and
 * the reload of the launch-plan overrides used by tuning sweeps and tests.
 * Same conventions as gqa.h (status codes, caller-owned device memory, work
 * enqueued on the given stream).
 */
#ifndef GQA_MEASURE_H_
#define GQA_MEASURE_H_

#include <stddef.h>

#include "gqa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads `bytes` of `buf` once with 16-byte loads, non-temporal if
 * `nontemporal` is nonzero - the loads of the decode kernels' cache stream -
 * on `grid` workgroups of 256 threads (0: 2048), each thread taking pieces
 * grid-stride.  Every thread folds its pieces with xor and writes the fold to
 * sink[0] only if it equals 0x12345678, so no read can be skipped and sink is
 * normally left untouched.
 *   buf   device, 16-byte aligned; bytes a multiple of 16 (GQA_ERR_ALIGN).
 *   sink  device, one unsigned; grid in 0..2^20 (GQA_ERR_SHAPE otherwise).
 * bytes = 0 is a no-op.  Enqueued on `stream`.
 */
gqa_status gqa_stream_read(const void *buf, size_t bytes, int nontemporal, int grid, unsigned *sink,
                           hipStream_t stream);

/*
 * Launch-plan overrides.  The library reads its GQA_* environment variables
 * (GQA_KERNEL=valu|mfma, GQA_CHUNK, GQA_TARGET_WGS, GQA_MAX_CHUNK,
 * GQA_FUSED_MAX_SPLITS, GQA_WAVES, GQA_HEAD_SPLIT, GQA_CONTIG, GQA_TEMPORAL,
 * GQA_MERGE=kernel, GQA_ORDER, GQA_ARRIVE, GQA_VALU_PIECES, GQA_LINEAR_*) once, when it
 * is loaded; unset, every call takes the measured default plan.  Calls never
 * read the environment themselves.  gqa_tuning_reload() reads the variables
 * again and drops the plans cached per shape.  It must not run while another
 * thread is inside the library, and a workspace sized before a reload may no
 * longer be large enough after it.
 */
void gqa_tuning_reload(void);

#ifdef __cplusplus
}
#endif

#endif /* GQA_MEASURE_H_ */
