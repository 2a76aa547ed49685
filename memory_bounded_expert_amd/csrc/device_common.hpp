// Device-side helpers shared by the HIP kernels of libmoebound (gfx950).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 bit pattern as stored in memory
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;
typedef __attribute__((ext_vector_type(4))) float f32x4_t;
// 16 bytes as a native vector: a first-class value, so staging arrays of it
// stay in registers (HIP's uint4 is a struct and copies of it go through memory).
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4_t;

constexpr int kThreads = 256;  // work-group size of every kernel but the planner's

__device__ __forceinline__ float bf2f(bf16_t v) { return __uint_as_float(((uint32_t)v) << 16); }

// fp32 -> bf16, round to nearest even (gfx950 v_cvt_pk_bf16_f32).
__device__ __forceinline__ bf16_t f2bf(float f) {
  return __builtin_bit_cast(bf16_t, static_cast<__bf16>(f));
}

// The logistic 1 / (1 + e^-a), the reciprocal by the hardware instruction
// (about 1 ulp; every bf16 value formed from it is rounded right after)
__device__ __forceinline__ float logistic(float a) { return __builtin_amdgcn_rcpf(1.f + __expf(-a)); }
// h = silu(a) u = a u / (1 + e^-a)
__device__ __forceinline__ float swiglu_h(float a, float u) { return a * logistic(a) * u; }

template <typename T> struct Elem;
template <> struct Elem<float> {
  static constexpr int kPer16B = 4;
  __device__ static __forceinline__ float to_f(float v) { return v; }
  __device__ static __forceinline__ float from_f(float v) { return v; }
};
template <> struct Elem<bf16_t> {
  static constexpr int kPer16B = 8;
  __device__ static __forceinline__ float to_f(bf16_t v) { return bf2f(v); }
  __device__ static __forceinline__ bf16_t from_f(float v) { return f2bf(v); }
};

// Unpack / pack one 16-byte chunk to / from fp32 lanes.
__device__ __forceinline__ void unpack16(const u32x4_t& v, float* out, float) {
  out[0] = __uint_as_float(v.x); out[1] = __uint_as_float(v.y);
  out[2] = __uint_as_float(v.z); out[3] = __uint_as_float(v.w);
}
__device__ __forceinline__ void unpack16(const u32x4_t& v, float* out, bf16_t) {
  const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
  }
}
__device__ __forceinline__ u32x4_t pack16(const float* in, float) {
  return u32x4_t{__float_as_uint(in[0]), __float_as_uint(in[1]), __float_as_uint(in[2]),
                 __float_as_uint(in[3])};
}
__device__ __forceinline__ u32x4_t pack16(const float* in, bf16_t) {
  uint32_t w[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
    w[i] = (uint32_t)f2bf(in[2 * i]) | ((uint32_t)f2bf(in[2 * i + 1]) << 16);
  return u32x4_t{w[0], w[1], w[2], w[3]};
}

}  // namespace moe
