/*
 * libtopk_probe.h -- the streaming-read probe that measures the HBM read
 * rate a plain kernel reaches on the device, the second denominator of the
 * top-k kernels' roofline (the first is the published 8 TB/s).  It is a
 * measurement tool beside libtopk, not part of the selection path.
 *
 * The sglang PR #39305 page, section "Performance", times its kernels on
 * inputs rotated past the on-chip caches; the same probe, run over a buffer
 * larger than the 256 MB Infinity Cache, also evicts earlier inputs before a
 * timed region.
 */
#ifndef LIBTOPK_PROBE_H
#define LIBTOPK_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Reads `bytes` bytes of device memory at `src` once, with one 16-byte
 * load per lane of 256-thread workgroups, consecutive lanes on consecutive
 * 16-byte vectors (every load instruction of a wave covers 1 KB).  Nothing is
 * written unless the XOR of a vector's four words equals 0x9E3779B9, in
 * which case one word of `sink` (device, 256 words, caller-owned) receives
 * it; callers pass a zero-filled buffer, so the probe writes nothing.
 *   src     device pointer, 16-byte aligned
 *   bytes   a multiple of 16, 0 .. 2^40
 *   sink    device uint32 [256]
 *   stream  hipStream_t, NULL for the default stream
 * Returns 0, -1 for a bad argument (nothing enqueued), -3 when the launch
 * fails.  Asynchronous. */
int topk_probe_stream_read(const void *src, int64_t bytes, uint32_t *sink, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* LIBTOPK_PROBE_H */
