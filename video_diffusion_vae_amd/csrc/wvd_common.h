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

namespace wvd {

constexpr int kWave = 64;
constexpr float kF16Max = 65504.0f;

// Input tensor element types accepted at the C ABI.
enum DType { DT_BF16 = 0, DT_F32 = 1 };

__device__ __forceinline__ float bf2f(uint32_t u16) { return __uint_as_float(u16 << 16); }

// fp32 -> bf16, round to nearest even (inputs are finite).
__device__ __forceinline__ uint32_t f2bf(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

__device__ __forceinline__ float h2f(uint32_t u16) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)u16);
}

// fp32 -> fp16, round to nearest even, saturating at +-65504.
__device__ __forceinline__ uint32_t f2h(float f) {
  f = fminf(fmaxf(f, -kF16Max), kF16Max);
  return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}

// Element of an input tensor of type dt as fp32.
__device__ __forceinline__ float load_in(const void* p, long long i, int dt) {
  return dt == DT_F32 ? static_cast<const float*>(p)[i] : bf2f(static_cast<const bf16_t*>(p)[i]);
}

__device__ __forceinline__ uint32_t pack2h(float lo, float hi) { return f2h(lo) | (f2h(hi) << 16); }

// Unpack 8 fp16 held in a uint4 into floats.
__device__ __forceinline__ void unpack8h(const uint4& v, float* f) {
  f[0] = h2f(v.x & 0xffffu); f[1] = h2f(v.x >> 16);
  f[2] = h2f(v.y & 0xffffu); f[3] = h2f(v.y >> 16);
  f[4] = h2f(v.z & 0xffffu); f[5] = h2f(v.z >> 16);
  f[6] = h2f(v.w & 0xffffu); f[7] = h2f(v.w >> 16);
}

__device__ __forceinline__ uint4 pack8h(const float* f) {
  uint4 r;
  r.x = pack2h(f[0], f[1]); r.y = pack2h(f[2], f[3]);
  r.z = pack2h(f[4], f[5]); r.w = pack2h(f[6], f[7]);
  return r;
}

// SiLU(v) = v / (1 + exp(-v)); exp via the hardware exp2 path.
__device__ __forceinline__ float silu(float v) { return v / (1.0f + __expf(-v)); }

}  // namespace wvd
