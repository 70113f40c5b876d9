// Device-side building blocks for the gfx950 kernels: element types, exact
// conversions, the MFMA tile step, wave reductions and the XCD-aware block
// order.  Everything here is CDNA4 (wave64) specific.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace flce {

typedef unsigned short u16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(8))) _Float16 f16x8_t;
typedef __attribute__((ext_vector_type(16))) float f32x16_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
typedef __attribute__((ext_vector_type(4))) unsigned int u32x4_t;
typedef __attribute__((ext_vector_type(2))) unsigned int u32x2_t;

constexpr int kWave = 64;

// ---------------------------------------------------------------- conversions
__device__ __forceinline__ float bf16_to_f32(u16 b) { return __uint_as_float(uint32_t(b) << 16); }

// fp32 -> bf16, IEEE round-to-nearest-even (gfx950's v_cvt_pk_bf16_f32);
// NaN stays NaN.  The pair form converts two values in one instruction.
typedef __bf16 bf16x2_native_t __attribute__((ext_vector_type(2)));
typedef float f32x2_native_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  const f32x2_native_t v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_native_t));
}
__device__ __forceinline__ u16 f32_to_bf16(float f) {
  return __builtin_bit_cast(u16, static_cast<__bf16>(f));
}

__device__ __forceinline__ float f16_to_f32(u16 h) {
  _Float16 x = __builtin_bit_cast(_Float16, h);
  return float(x);
}

__device__ __forceinline__ u16 f32_to_f16(float f) {
  _Float16 x = _Float16(f);  // v_cvt_f16_f32, round-to-nearest-even
  return __builtin_bit_cast(u16, x);
}

// ------------------------------------------------------------ element traits
// 16-bit types: the 32x32x16 MFMA takes 8 consecutive k per lane (16 bytes).
// fp32: the 32x32x2 MFMA takes 1 k per lane.  `base` names the element type
// itself, also through Mfma16 below; `sub16` is set by Mfma16.
//
// Mfma16<T> (16-bit T) computes the same 32x32 accumulator blocks with four
// 16x16x32 MFMAs each: 32 k per step, 8 consecutive k per lane.  For one
// 16x16 sub-block, lane l holds A[l % 16][8 (l / 16) + 0..7] and
// B[8 (l / 16) + 0..7][l % 16] and receives D[4 (l / 16) + e][l % 16],
// e = 0..3; sub-block q = 2 (row half) + (column half) lives in accumulator
// elements 4 q .. 4 q + 3.  Under this chip's power limit a loop of 16x16x32
// MFMAs on random data sustains 1.96-1.98 PFLOP/s against 1.68-1.82 for
// 32x32x16 (2.44 and 2.43 with zero operands, where the clock stays at its
// maximum).  The fragment bytes per flop are the same for both shapes, but a
// k-step covers 32 k, so a k-tile holds half as many steps to hide each
// step's reads behind.
template <int Q, class V>
__device__ __forceinline__ void mma16_sub(f32x16_t& c, V a, V b) {
  f32x4_t d = {c[4 * Q], c[4 * Q + 1], c[4 * Q + 2], c[4 * Q + 3]};
  if constexpr (__is_same(V, bf16x8_t))
    d = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, d, 0, 0, 0);
  else
    d = __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, d, 0, 0, 0);
  c[4 * Q] = d[0];
  c[4 * Q + 1] = d[1];
  c[4 * Q + 2] = d[2];
  c[4 * Q + 3] = d[3];
}

struct BF16 {
  typedef u16 storage;
  typedef BF16 base;
  static constexpr bool sub16 = false;
  static constexpr int kpack = 8;   // k per lane per MFMA
  static constexpr int kstep = 16;  // k per MFMA
  static constexpr int vec = 8;     // elements per 16-byte vector
  __device__ static float to_f32(u16 x) { return bf16_to_f32(x); }
  __device__ static u16 from_f32(float x) { return f32_to_bf16(x); }
  __device__ static void mma(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
  }
  template <int Q>
  __device__ static void mma16(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    mma16_sub<Q>(c, __builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b));
  }
};

struct F16 {
  typedef u16 storage;
  typedef F16 base;
  static constexpr bool sub16 = false;
  static constexpr int kpack = 8;
  static constexpr int kstep = 16;
  static constexpr int vec = 8;
  __device__ static float to_f32(u16 x) { return f16_to_f32(x); }
  __device__ static u16 from_f32(float x) { return f32_to_f16(x); }
  __device__ static void mma(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a),
                                                __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  }
  template <int Q>
  __device__ static void mma16(const u32x4_t& a, const u32x4_t& b, f32x16_t& c) {
    mma16_sub<Q>(c, __builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b));
  }
};

template <class T>
struct Mfma16 : T {
  static_assert(sizeof(typename T::storage) == 2, "16x16x32 MFMAs take 16-bit operands");
  static constexpr bool sub16 = true;
  static constexpr int kstep = 32;
};

struct F32 {
  typedef float storage;
  typedef F32 base;
  static constexpr bool sub16 = false;
  static constexpr int kpack = 1;
  static constexpr int kstep = 2;
  static constexpr int vec = 4;
  __device__ static float to_f32(float x) { return x; }
  __device__ static float from_f32(float x) { return x; }
  __device__ static void mma(float a, float b, f32x16_t& c) {
    c = __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
};

// Element store in a destination dtype chosen at run time (0 f32, 1 f16, 2 bf16).
__device__ __forceinline__ void store_as(void* base, int64_t i, float v, int dt) {
  if (dt == 0)
    static_cast<float*>(base)[i] = v;
  else if (dt == 1)
    static_cast<u16*>(base)[i] = f32_to_f16(v);
  else
    static_cast<u16*>(base)[i] = f32_to_bf16(v);
}

__device__ __forceinline__ float load_as(const void* base, int64_t i, int dt) {
  if (dt == 0) return static_cast<const float*>(base)[i];
  if (dt == 1) return f16_to_f32(static_cast<const u16*>(base)[i]);
  return bf16_to_f32(static_cast<const u16*>(base)[i]);
}

// ------------------------------------------------------------ wave reductions
// Reductions over the 32 lanes of one half-wave (xor masks below 32 stay in
// the half), used where the 32x32 MFMA tile spreads a row over 32 lanes.
__device__ __forceinline__ float half_wave_max(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ float half_wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < 32; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
__device__ __forceinline__ int wave_min_int(int v) {
#pragma unroll
  for (int m = 1; m < kWave; m <<= 1) {
    const int o = __shfl_xor(v, m, kWave);
    v = o < v ? o : v;
  }
  return v;
}

// -------------------------------------------------------- XCD-aware ordering
// Workgroups are handed to the 8 XCDs round-robin (hardware id i runs on XCD
// i % 8).  This maps hardware ids to logical tile ids so that consecutive
// logical ids run on one XCD and share its L2: XCD x receives the contiguous
// logical range [x*q + min(x, r), ...), q = n / 8, r = n % 8.
__device__ __forceinline__ int xcd_remap(int hw_id, int n) {
  const int q = n >> 3, r = n & 7;
  const int x = hw_id & 7, j = hw_id >> 3;
  return x * q + (x < r ? x : r) + j;
}

}  // namespace flce
