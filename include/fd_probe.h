/*
 * fd_probe.h -- HBM read probe of the split-KV decode library (gfx950).
 *
 * A measurement aid, not part of the decode path. Decode attention re-reads
 * the whole cached history at every step, so it is bound by memory traffic
 * (the Bifurcated Attention abstract in the "Related papers" list makes this
 * point for incremental decoding); the split kernel's bandwidth is judged
 * against the 8 TB/s HBM peak and against what a kernel that does nothing
 * but stream the same bytes achieves on the same device. This call is that
 * kernel: each of `workgroups` workgroups of `waves` waves reads its
 * contiguous share of `bytes` with non-temporal 16-byte loads, keeping
 * 16 * loads_per_lane bytes per lane in flight (the next batch is requested
 * as the current one lands), and folds what it reads into one word per
 * workgroup that is written only if it equals an improbable value, so
 * nothing is skipped. The caller times it (e.g. events around a graph of
 * launches over buffers rotated so no launch is served from the
 * Infinity Cache).
 *
 *   buf             device, 16-byte aligned, `bytes` readable bytes
 *   bytes           > 0, a multiple of
 *                   workgroups * waves * 64 * 16 * loads_per_lane
 *   workgroups      1 .. 65535
 *   waves           4, 8 or 16 per workgroup
 *   loads_per_lane  2, 4 or 8 sixteen-byte loads per lane per batch, or
 *                   16 with at most 8 waves
 *   sink            device uint32 [workgroups] (written only in the
 *                   improbable case; must be valid)
 *   stream          hipStream_t as void* (NULL = null stream)
 * Returns 0 (FD_OK), -1 for a bad argument (nothing launched), -4 for a
 * launch error.
 */
#ifndef FD_PROBE_H
#define FD_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

int fd_read_probe(const void* buf, size_t bytes, int workgroups, int waves,
                  int loads_per_lane, uint32_t* sink, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* FD_PROBE_H */
