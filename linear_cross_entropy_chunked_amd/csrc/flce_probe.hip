// Measurement probes for the benchmark (libflce_probe.so), outside the fused
// cross-entropy path: what this chip sustains on its own, as the ceilings the
// path's kernels are compared with.
//
//   flce_probe_mfma_loop   bf16 32x32x16 MFMAs on register operands only,
//                          eight waves per CU, no memory traffic in the loop.
//                          With random operands the multipliers toggle as in
//                          a real GEMM and the chip's power limit sets the
//                          clock; with zero operands it does not.
//   flce_probe_mfma16_loop the same with bf16 16x16x32 MFMAs, twice as many
//                          per iteration (the same flops).
//   flce_probe_read_stream a read of one large buffer in contiguous segments,
//                          one per workgroup, 16 bytes per lane, four loads in
//                          flight per lane: the HBM read rate.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "flce_probe.h"

namespace {

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) unsigned u32x4_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;

constexpr int kMfmaThreads = 512;   // eight waves: one workgroup per CU, two waves per SIMD
constexpr int kStreamThreads = 256;

// Each lane keeps four A and four B fragments, rotated every iteration so
// that consecutive MFMAs see different operand bits; eight accumulators keep
// the MFMA pipe free of dependences.  The accumulators' sum is written out so
// nothing is dead.
__global__ __launch_bounds__(kMfmaThreads) void mfma_loop_kernel(const u32x4_t* __restrict__ ops,
                                                                 int64_t nops, float* sink,
                                                                 int iters) {
  const int64_t t = (int64_t)blockIdx.x * kMfmaThreads + threadIdx.x;
  u32x4_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[(t * 8 + i) % nops];
    b[i] = ops[(t * 8 + 4 + i) % nops];
  }
  f32x16_t acc[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) acc[j] = f32x16_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 8; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a[(s + j) & 3]),
                                                         __builtin_bit_cast(bf16x8_t, b[(s + 3 * j) & 3]),
                                                         acc[j], 0, 0, 0);
    const u32x4_t x = a[0];
    a[0] = a[1]; a[1] = a[2]; a[2] = a[3]; a[3] = b[0];
    b[0] = b[1]; b[1] = b[2]; b[2] = b[3]; b[3] = x;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  sink[t] = s;
}

// The same operand rotation with 16x16x32 MFMAs: sixteen accumulators of four
// floats, 64 MFMAs of 16384 flops per iteration.
__global__ __launch_bounds__(kMfmaThreads) void mfma16_loop_kernel(const u32x4_t* __restrict__ ops,
                                                                   int64_t nops, float* sink,
                                                                   int iters) {
  const int64_t t = (int64_t)blockIdx.x * kMfmaThreads + threadIdx.x;
  u32x4_t a[4], b[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    a[i] = ops[(t * 8 + i) % nops];
    b[i] = ops[(t * 8 + 4 + i) % nops];
  }
  f32x4_t acc[16];
#pragma unroll
  for (int j = 0; j < 16; ++j) acc[j] = f32x4_t{};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 4; ++s)
#pragma unroll
      for (int j = 0; j < 16; ++j)
        acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a[(s + j) & 3]),
                                                         __builtin_bit_cast(bf16x8_t, b[(s + 3 * j) & 3]),
                                                         acc[j], 0, 0, 0);
    const u32x4_t x = a[0];
    a[0] = a[1]; a[1] = a[2]; a[2] = a[3]; a[3] = b[0];
    b[0] = b[1]; b[1] = b[2]; b[2] = b[3]; b[3] = x;
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 16; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) s += acc[j][e];
  sink[t] = s;
}

// Workgroup b reads the b-th of gridDim.x contiguous segments, four 16-byte
// loads in flight per lane (contiguous segments of about 1 MiB measured
// faster than a grid-strided sweep of the whole buffer: 5.9 against 5.3 TB/s).
__global__ __launch_bounds__(kStreamThreads) void read_stream_kernel(const u32x4_t* __restrict__ src,
                                                                     int64_t n, int64_t seg,
                                                                     u32x4_t* sink) {
  const int64_t b0 = (int64_t)blockIdx.x * seg;
  const int64_t e = b0 + seg < n ? b0 + seg : n;
  int64_t i = b0 + threadIdx.x;
  u32x4_t acc = {0u, 0u, 0u, 0u};
  for (; i + 3 * kStreamThreads < e; i += 4 * kStreamThreads) {
    const u32x4_t p = src[i], q = src[i + kStreamThreads], r = src[i + 2 * kStreamThreads],
                  u = src[i + 3 * kStreamThreads];
    acc ^= p ^ q ^ r ^ u;
  }
  for (; i < e; i += kStreamThreads) acc ^= src[i];
  sink[(int64_t)blockIdx.x * kStreamThreads + threadIdx.x] = acc;
}

}  // namespace

extern "C" int flce_probe_mfma_loop(const void* operands, int64_t operand_bytes, float* sink,
                                    int64_t sink_floats, int blocks, int iters, void* stream) {
  if (!operands || !sink || operand_bytes < 16 || blocks <= 0 || iters < 0 ||
      sink_floats < (int64_t)blocks * kMfmaThreads)
    return 1;
  hipLaunchKernelGGL(mfma_loop_kernel, dim3(blocks), dim3(kMfmaThreads), 0, (hipStream_t)stream,
                     (const u32x4_t*)operands, operand_bytes / 16, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int flce_probe_mfma16_loop(const void* operands, int64_t operand_bytes, float* sink,
                                      int64_t sink_floats, int blocks, int iters, void* stream) {
  if (!operands || !sink || operand_bytes < 16 || blocks <= 0 || iters < 0 ||
      sink_floats < (int64_t)blocks * kMfmaThreads)
    return 1;
  hipLaunchKernelGGL(mfma16_loop_kernel, dim3(blocks), dim3(kMfmaThreads), 0, (hipStream_t)stream,
                     (const u32x4_t*)operands, operand_bytes / 16, sink, iters);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int flce_probe_read_stream(const void* src, int64_t bytes, void* sink,
                                      int64_t sink_bytes, int blocks, void* stream) {
  if (!src || !sink || bytes < 16 || (bytes & 15) || blocks <= 0 ||
      sink_bytes < (int64_t)blocks * kStreamThreads * 16)
    return 1;
  const int64_t n = bytes / 16;
  hipLaunchKernelGGL(read_stream_kernel, dim3(blocks), dim3(kStreamThreads), 0, (hipStream_t)stream,
                     (const u32x4_t*)src, n, (n + blocks - 1) / blocks, (u32x4_t*)sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

extern "C" int flce_probe_mfma_threads(void) { return kMfmaThreads; }
extern "C" int flce_probe_stream_threads(void) { return kStreamThreads; }
