/*
 * pa_probe.h — measurement aid shipped beside libpa (libpa_probe.so), not
 * part of the decode path.
 *
 * pa_probe_stream_read: enqueues one read of `bytes` bytes of device memory
 * at `buf` (16-byte aligned) on `stream` (hipStream_t as void*, NULL = null
 * stream) with `workgroups` workgroups of 256 threads. Each lane keeps
 * `loads_per_lane` independent 16-byte loads in flight, with the streaming
 * (non-temporal) cache policy if `nontemporal` is nonzero, else the plain
 * one. `pattern`: 0 = grid-stride (loads 1, 2, 4, 8; each wave load covers
 * 1 KiB of consecutive bytes), 1 = each wave reads loads_per_lane KiB of
 * consecutive bytes per iteration (loads 1, 2, 4, 8), 2 = random 4 KiB tiles
 * from each half of the buffer at one pseudo-random tile index per
 * iteration, like paged decode's K and V blocks (loads 4: one tile at a
 * time, 8: both halves' tiles together; bytes >= 8 KiB; the tiles covered
 * per half are a power of two, so up to half of the buffer is read: the
 * achieved rate counts the bytes actually read, see the bench). The best
 * rate over a sweep of these shapes is the practical HBM read ceiling that
 * the decode kernels' rates are compared with. `sink` is a device word
 * written only if the folded data equal a sentinel (keeps the reads live).
 * Returns 0, 1 for a bad argument (nothing enqueued), 6 if the launch
 * failed.
 *
 * pa_probe_mfma_valu: enqueues `workgroups` workgroups of 8 waves on
 * `stream`; each wave runs `iters` iterations of matrix-core work (16
 * independent v_mfma_f32_16x16x32_bf16 on four accumulators) and/or vector
 * work (64 fp32 FMAs on eight independent chains), by `mode`: 0 MFMAs only,
 * 1 FMAs only, 2 both in every wave, interleaved, 3 waves 0-3 MFMAs and
 * waves 4-7 FMAs (one wave of each kind per SIMD), 4 MFMAs only as one
 * dependent chain, 5 16 exp2 per iteration only. Timing the modes shows how
 * far the two kinds of work overlap on one SIMD. `out` [dev] float
 * [workgroups * 512] receives one value per thread (keeps the work live).
 * Returns 0, 1 for a bad argument (nothing enqueued), 6 if the launch
 * failed.
 */
#ifndef PA_PROBE_H
#define PA_PROBE_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

int pa_probe_stream_read(const void* buf, size_t bytes, int workgroups, int loads_per_lane,
                         int nontemporal, int pattern, void* sink, void* stream);
int pa_probe_mfma_valu(int mode, int workgroups, int iters, float* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* PA_PROBE_H */
