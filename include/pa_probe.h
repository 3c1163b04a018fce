/*
 * pa_probe.h — measurement aid shipped beside libpa (libpa_probe.so), not
 * part of the decode path.
 *
 * pa_probe_stream_read: enqueues one streaming read of `bytes` bytes of
 * device memory at `buf` (16-byte aligned) on `stream` (hipStream_t as void*,
 * NULL = null stream) with `workgroups` workgroups of 256 threads. Each lane
 * keeps `loads_per_lane` (1, 2, 4 or 8) independent 16-byte loads in flight,
 * with the streaming (non-temporal) cache policy if `nontemporal` is
 * nonzero, else the plain one. The best rate over a sweep of these shapes is
 * the practical HBM read ceiling that the decode kernels' rates are compared
 * with. `sink` is a device word written only if the folded data equal a
 * sentinel (keeps the reads live). Returns 0, 1 for a bad argument (nothing
 * enqueued), 6 if the launch failed.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int pa_probe_stream_read(const void* buf, size_t bytes, int workgroups, int loads_per_lane,
                         int nontemporal, void* sink, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_PROBE_H */
