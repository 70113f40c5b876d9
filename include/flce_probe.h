/* Measurement probes (libflce_probe.so), used by the benchmark only.
 *
 * They are not part of the fused linear cross-entropy boundary (flce.h):
 * they measure what the chip itself sustains, so that the path's kernels can
 * be compared with a ceiling that holds on this machine as well as with the
 * published peaks.  All pointers are device pointers; every call is
 * asynchronous on `stream` (a hipStream_t, NULL for the default stream) and
 * returns 0 on success, 1 for invalid arguments (nothing launched), 2 if the
 * launch failed.  The caller owns every buffer.
 */
#ifndef FLCE_PROBE_H
#define FLCE_PROBE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* bf16 MFMA throughput with no memory traffic in the loop.
 * `blocks` workgroups of flce_probe_mfma_threads() threads (eight waves,
 * one workgroup per CU) each run `iters` iterations of 32 independent
 * v_mfma_f32_32x32x16_bf16, i.e. blocks * 8 waves * iters * 32 * 32768 flops.
 * Each lane takes its eight 16-byte operand fragments from `operands`
 * (operand_bytes >= 16; fragment f of lane t is 16-byte element
 * (8 t + f) mod (operand_bytes / 16)), so random operands give the toggling
 * of a real GEMM and zero operands none.  `sink` receives one float per
 * thread: sink_floats >= blocks * flce_probe_mfma_threads(). */
int flce_probe_mfma_loop(const void* operands, int64_t operand_bytes, float* sink,
                         int64_t sink_floats, int blocks, int iters, void* stream);

/* The same loop with v_mfma_f32_16x16x32_bf16: each iteration runs 64
 * independent 16x16x32 MFMAs (16 accumulators), the same flops as one
 * iteration above, from the same operand fragments; arguments, sink and
 * return codes as for flce_probe_mfma_loop. */
int flce_probe_mfma16_loop(const void* operands, int64_t operand_bytes, float* sink,
                           int64_t sink_floats, int blocks, int iters, void* stream);

/* A read of `bytes` bytes of `src` (a multiple of 16) by `blocks` workgroups
 * of flce_probe_stream_threads() threads; workgroup b reads the b-th of
 * `blocks` contiguous segments (about 1 MiB each is what the benchmark uses),
 * 16 bytes per lane, four loads in flight per lane.  `sink` receives 16 bytes
 * per thread: sink_bytes >= blocks * flce_probe_stream_threads() * 16. */
int flce_probe_read_stream(const void* src, int64_t bytes, void* sink, int64_t sink_bytes,
                           int blocks, void* stream);

/* Threads per workgroup of the two probes. */
int flce_probe_mfma_threads(void);
int flce_probe_stream_threads(void);

#ifdef __cplusplus
}
#endif

#endif /* FLCE_PROBE_H */
