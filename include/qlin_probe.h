/*
 * qlin_probe.h -- measurement aid of the quantized skinny linear layer
 * (libqlin_probe.so): a plain streaming read of a device buffer on gfx950,
 * the HBM read ceiling that the GEMM's achieved bandwidth is compared with.
 * It is not part of the linear layer and libqlin.so does not depend on it.
 */
#ifndef QLIN_PROBE_H
#define QLIN_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Reads every byte of buf[0, bytes) once with 16-byte non-temporal vector
 * loads (the faster policy for a read that streams through once) from
 * `blocks` workgroups of 256 threads (a grid-stride loop with 8 loads in
 * flight per thread), and folds the data into one word per workgroup, which
 * is stored to sink[b] only in the (practically impossible) case that it
 * equals a fixed constant, so the loads cannot be removed and sink is almost
 * never written.
 *   buf    device pointer, 16-byte aligned, caller-owned
 *   bytes  a multiple of 16, > 0
 *   sink   device pointer to `blocks` uint32 words, caller-owned
 *   blocks 1 .. 65535
 *   stream hipStream_t (NULL = default stream); the read is only enqueued
 * Returns 0, or 1 for an invalid argument (nothing enqueued), or the
 * hipError_t of the launch.
 */
int qlin_probe_read(const void *buf, size_t bytes, uint32_t *sink, int blocks, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* QLIN_PROBE_H */
