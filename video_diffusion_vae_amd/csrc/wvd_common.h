// Shared device helpers of the wvd HIP library (gfx950, wave64).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

// Storage formats: activations, prepared weights and MFMA operands are fp16
// (h16_t bit patterns); the latents and weights handed in may be bf16 or
// fp32; the video handed out is bf16.
typedef uint16_t h16_t;
typedef uint16_t bf16_t;
typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef unsigned u32x4_t __attribute__((ext_vector_type(4)));

namespace wvd {

constexpr int kWave = 64;
constexpr float kF16Max = 65504.0f;

// Input tensor element types accepted at the C ABI.
enum DType { DT_BF16 = 0, DT_F32 = 1 };

__device__ __forceinline__ float bf2f(uint32_t u16) { return __uint_as_float(u16 << 16); }

// fp32 -> bf16, round to nearest even; a NaN stays a (quiet) NaN.
__device__ __forceinline__ uint32_t f2bf(float f) {
  if (f != f) return 0x7fc0u;
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float h2f(uint32_t u16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u16);
}

// Range events of the values this code object stores as fp16, one word per
// translation unit and device: bit 0 (kRangeSaturated) a finite value beyond
// the fp16 range was stored as +-65504, bit 1 (kRangeNaN) a NaN was stored.
// The host reads and clears them through wvd_range_flags.
constexpr unsigned kRangeSaturated = 1u;
constexpr unsigned kRangeNaN = 2u;
static __device__ unsigned int g_range_flags;

// |f| as bits: above kF16MaxBits means beyond +-65504, inf or NaN.
constexpr uint32_t kF16MaxBits = 0x477fe000u;  // 65504.0f
__device__ __forceinline__ uint32_t abs_bits(float f) { return __float_as_uint(f) & 0x7fffffffu; }

__device__ __forceinline__ uint32_t h16_bits(float f) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// The rare path of the fp16 conversions: a finite value beyond +-65504
// saturates and a NaN stays NaN; `flags` collects which of the two occurred.
__device__ __forceinline__ uint32_t f2h_saturate(float f, uint32_t& flags) {
  if (abs_bits(f) > kF16MaxBits) flags |= f != f ? kRangeNaN : kRangeSaturated;
  return h16_bits(f != f ? f : fminf(fmaxf(f, -kF16Max), kF16Max));
}
__device__ __forceinline__ void raise_range_flags(uint32_t flags) {
  if (flags) __hip_atomic_fetch_or(&g_range_flags, flags, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __noinline__ uint32_t f2h_out_of_range(float f) {
  uint32_t fl = 0;
  const uint32_t r = f2h_saturate(f, fl);
  raise_range_flags(fl);
  return r;
}

// |f| <= 65504, false for a NaN (one compare with an abs modifier).
__device__ __forceinline__ bool in_f16_range(float f) { return __builtin_fabsf(f) <= kF16Max; }

// max(|a|, |b|, |c|) that propagates a NaN (IEEE 754-2019 maximum: one
// v_maximum3_f32 with abs modifiers), so !(result <= 65504) tests all three
// values against the fp16 range and for NaN at once.
__device__ __forceinline__ float max3_abs_nan(float a, float b, float c) {
  return __builtin_elementwise_maximum(
      __builtin_elementwise_maximum(__builtin_fabsf(a), __builtin_fabsf(b)), __builtin_fabsf(c));
}

// fp32 -> fp16, round to nearest even.  A finite value beyond +-65504
// saturates there and a NaN stays NaN; either one sets the range flags.
__device__ __forceinline__ uint32_t f2h(float f) {
  return in_f16_range(f) ? h16_bits(f) : f2h_out_of_range(f);
}

// Norm scale 1 / max(||v||, 1e-12) of a channel sum of squares ss >= 0, as
// the Winograd input transforms compute it: min(rsqrt(ss), 1e12), one
// hardware reciprocal square root (the conversion self-test, wvd_f16_probe,
// bounds its error).
__device__ __forceinline__ float norm_scale(float ss) { return fminf(__builtin_amdgcn_rsqf(ss), 1e12f); }

// clamp(v, -1, 1) that keeps a NaN (the video's final clamp).
__device__ __forceinline__ float clamp_unit(float v) { return v != v ? v : fminf(fmaxf(v, -1.0f), 1.0f); }

// Element of an input tensor of type dt as fp32.
__device__ __forceinline__ float load_in(const void* p, long long i, int dt) {
  return dt == DT_F32 ? static_cast<const float*>(p)[i] : bf2f(static_cast<const bf16_t*>(p)[i]);
}

// Two values in one conversion instruction (v_cvt_pk_f16_f32, round to
// nearest even like the scalar conversion), lo in the low half.
typedef float f32x2v_t __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2v_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t h16x2_bits(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v_t){lo, hi}, f16x2v_t));
}

// The rare paths of pack2h / pack8h (leaf functions: no stack frame).
__device__ __noinline__ uint32_t pack2h_out_of_range(float lo, float hi) {
  uint32_t fl = 0;
  const uint32_t r = f2h_saturate(lo, fl) | (f2h_saturate(hi, fl) << 16);
  raise_range_flags(fl);
  return r;
}
__device__ __noinline__ uint4 pack8h_out_of_range(float f0, float f1, float f2, float f3, float f4, float f5,
                                                  float f6, float f7) {
  uint32_t fl = 0;
  const uint4 r = make_uint4(f2h_saturate(f0, fl) | (f2h_saturate(f1, fl) << 16),
                             f2h_saturate(f2, fl) | (f2h_saturate(f3, fl) << 16),
                             f2h_saturate(f4, fl) | (f2h_saturate(f5, fl) << 16),
                             f2h_saturate(f6, fl) | (f2h_saturate(f7, fl) << 16));
  raise_range_flags(fl);
  return r;
}

// The common path converts unconditionally; only an out-of-range value
// branches, and then the rare path recomputes the whole result.
__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  uint32_t r = h16x2_bits(lo, hi);
  if (!(__builtin_elementwise_maximum(__builtin_fabsf(lo), __builtin_fabsf(hi)) <= kF16Max))
    r = pack2h_out_of_range(lo, hi);
  return r;
}

// Unpack 8 fp16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8h(const uint4& v, float* f) {
  f[0] = h2f(v.x & 0xffffu); f[1] = h2f(v.x >> 16);
  f[2] = h2f(v.y & 0xffffu); f[3] = h2f(v.y >> 16);
  f[4] = h2f(v.z & 0xffffu); f[5] = h2f(v.z >> 16);
  f[6] = h2f(v.w & 0xffffu); f[7] = h2f(v.w >> 16);
}

// Eight values at once: one range test for all eight on the common path
// (four NaN-propagating maxima of the magnitudes and one compare).
__device__ __forceinline__ uint4 pack8h(const float* f) {
  const float m = max3_abs_nan(
      f[6], f[7], __builtin_elementwise_maximum(max3_abs_nan(f[0], f[1], f[2]), max3_abs_nan(f[3], f[4], f[5])));
  uint4 r = make_uint4(h16x2_bits(f[0], f[1]), h16x2_bits(f[2], f[3]), h16x2_bits(f[4], f[5]),
                       h16x2_bits(f[6], f[7]));
  if (!(m <= kF16Max)) r = pack8h_out_of_range(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
  return r;
}

// pack8h with the range test on the magnitudes' bit patterns (an AND and an
// unsigned maximum per value): the same result and flags, more instructions,
// but fewer registers live where the values are produced and stored one
// group at a time (wino_out_kernel keeps three waves per SIMD with it and
// drops to two with pack8h; norm_silu_kernel keeps five).
__device__ __forceinline__ uint4 pack8h_int(const float* f) {
  uint32_t m = 0;
#pragma unroll
  for (int k = 0; k < 8; ++k) m = max(m, abs_bits(f[k]));
  uint4 r = make_uint4(h16x2_bits(f[0], f[1]), h16x2_bits(f[2], f[3]), h16x2_bits(f[4], f[5]),
                       h16x2_bits(f[6], f[7]));
  if (m > kF16MaxBits) r = pack8h_out_of_range(f[0], f[1], f[2], f[3], f[4], f[5], f[6], f[7]);
  return r;
}

// SiLU(t) = t / (1 + e^-t) as every kernel evaluates it: __expf (the
// hardware exp2 of t * log2(e)) and the hardware reciprocal.  Its error
// against the exact value is bounded by the math self-test
// (wvd_math_probe) over the activations' input range.
__device__ __forceinline__ float silu_hw(float t) { return t * __builtin_amdgcn_rcpf(1.0f + __expf(-t)); }

// e^t as the attention softmax evaluates it (hardware exp2 of t * log2(e)).
__device__ __forceinline__ float exp_hw(float t) { return __expf(t); }

}  // namespace wvd
