/*
 * ipttt_probe.h: C ABI of libipttt_probe, micro-benchmarks of the chip's
 * achievable rates (measurement only; not part of the layer library).
 *
 * The layer's kernels are reported against the rates these launches reach on
 * the same GPU: bf16 MFMA issue with no memory traffic, a streaming read of
 * HBM, conflict-free LDS reads and direct copies from L2 into LDS. Each call
 * enqueues ONE launch on hip_stream (NULL = the null stream) for the caller to
 * time with events on that stream, and returns the launch's work.
 *
 * Kinds:
 *   IPTTT_PROBE_MFMA16: two waves per SIMD on every CU issue back-to-back
 *     independent v_mfma_f32_16x16x32_bf16, n iterations of 8 per wave, no
 *     memory traffic; src unused; dst receives one float per thread.
 *   IPTTT_PROBE_MFMA32: the same with v_mfma_f32_32x32x16_bf16, n iterations
 *     of 4 per wave.
 *   IPTTT_PROBE_READ: streams n bytes of src (n a multiple of 16, n <=
 *     src_bytes) through the CUs; dst receives one folded value per thread.
 *   IPTTT_PROBE_LDS: two 256-thread blocks per CU read 32 KB of their LDS n
 *     times over in conflict-free 16-byte pieces; src unused; dst receives one
 *     folded value per thread.
 *   IPTTT_PROBE_COPY: two four-wave blocks per CU copy 8 KB per wave and
 *     iteration from 64 KB windows of src (4 MiB read in all, L2-resident after
 *     the first pass; src_bytes must be at least 4 MiB) into LDS with direct
 *     global-to-LDS copies, two iterations in flight, n iterations; dst must
 *     be non-NULL (nothing is written to it).
 *
 * Arguments. src, dst: device pointers, 16-byte aligned; src_bytes, dst_bytes:
 * their sizes. dst must hold one 32-bit value per thread of the launch
 * (MFMA, LDS: 512 x CUs values; READ: 2048 x CUs values). *work (host)
 * receives the launch's FLOPs (MFMA kinds) or bytes read, copied or moved
 * through LDS.
 *
 * Errors. Returns 0 (IPTTT_OK) on success; -1 (IPTTT_E_INVALID) for an unknown
 * kind, n < 1, a NULL or misaligned buffer, NULL work, or buffers too small
 * for the launch, all checked before any device work; -3 (IPTTT_E_HIP) if a
 * device query or the launch fails.
 */
#ifndef IPTTT_PROBE_H
#define IPTTT_PROBE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IPTTT_PROBE_MFMA16 = 0,
  IPTTT_PROBE_MFMA32 = 1,
  IPTTT_PROBE_READ = 2,
  IPTTT_PROBE_LDS = 3,
  IPTTT_PROBE_COPY = 4
} ipttt_probe_kind;

int ipttt_probe(int32_t kind, int64_t n, const void *src, size_t src_bytes, void *dst,
                size_t dst_bytes, double *work, void *hip_stream);

#ifdef __cplusplus
}
#endif

#endif /* IPTTT_PROBE_H */
