/*
 * zo_placement.h -- measurement and placement calls of libzo.so that are not steps of the
 * method: the in-place streaming diagnostic and the per-buffer choice of how the passes
 * over a large parameter buffer are issued (one launch, or consecutive launches over
 * slices).  They exist because on MI355X the bandwidth of a large allocation depends on
 * the physical memory it lands on.  Conventions (contexts, streams, errors) as in zo.h.
 */
#ifndef ZO_PLACEMENT_H
#define ZO_PLACEMENT_H

#include "zo.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Diagnostic, not a step of the method: every 32-bit word of d_buf becomes word ^ mask,
 * in place, streaming in the same order as zo_perturb (mask = 0 leaves the buffer
 * unchanged; a non-zero mask makes the pass checkable).  The bandwidth of this call on a
 * parameter buffer (2 * bytes / time) is the in-place read-modify-write ceiling of the
 * physical memory that buffer occupies; a large buffer's ceiling varies with where the
 * allocation lands, so a benchmark can compare zo_perturb with it on the very buffer it
 * times.  d_buf: device, 16-byte aligned, bytes a multiple of 16 (other kernels must not
 * use d_buf concurrently).  Errors (ZO_EINVAL): NULL ctx, NULL or misaligned d_buf with
 * bytes > 0, bytes not a multiple of 16. */
zo_status zo_stream_rmw(zo_ctx *ctx, void *d_buf, uint64_t bytes, uint32_t mask, void *stream);

/* Placement of a large parameter buffer, a property of MI355X's HBM rather than of the
 * method (the callers are those who stream a buffer in place many times, as every pass of
 * a step does): the bandwidth one launch reaches over a large buffer depends on where the
 * allocation's physical memory lies -- on some placements a launch whose eight XCD streams
 * lie far apart in the buffer runs well below what the memory allows -- while a pass issued
 * as consecutive launches over 1 GiB slices (every wave in flight inside one slice) runs
 * at nearly the same rate on every placement.  zo_tune_placement times both forms on the
 * caller's buffer (a read and write-back of every word, contents unchanged; synchronizes
 * `stream`), keeps the faster in the context, and reports both (GB/s of in-place traffic;
 * the sliced figure is 0 for buffers under 2 GiB, which always use one launch).  From then
 * on zo_perturb, zo_perturb2 and zo_stream_rmw on this context issue their passes in that
 * form; results do not depend on it.  zo_set_slice_bytes sets the form directly (0: one
 * launch per pass; otherwise a multiple of 1 MiB), zo_get_slice_bytes reads it.
 * Errors (ZO_EINVAL): NULL ctx, NULL or misaligned d_buf, bytes not a multiple of 16,
 * slice bytes not a multiple of 1 MiB; ZO_EHIP if the runtime reports an error. */
zo_status zo_tune_placement(zo_ctx *ctx, void *d_buf, uint64_t bytes, void *stream,
                            uint64_t *out_slice_bytes, double *out_gbps_whole,
                            double *out_gbps_sliced);
zo_status zo_set_slice_bytes(zo_ctx *ctx, uint64_t slice_bytes);
uint64_t zo_get_slice_bytes(const zo_ctx *ctx);

#ifdef __cplusplus
}
#endif

#endif /* ZO_PLACEMENT_H */
