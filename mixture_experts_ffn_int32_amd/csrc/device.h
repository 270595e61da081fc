// Device-side types and helpers shared by the HIP kernels of libhmm (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace hmm {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x8 __attribute__((ext_vector_type(8)));
typedef int32_t i32x2 __attribute__((ext_vector_type(2)));

// bfloat16 <-> float.  The float -> bf16 cast is IEEE round-to-nearest-even
// (one v_cvt_pk_bf16_f32 on gfx950).
__device__ __forceinline__ float bf2f(uint16_t b) { return __uint_as_float((uint32_t)b << 16); }
__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }
__device__ __forceinline__ float round_bf(float f) { return bf2f(f2bf(f)); }

// unpack / pack 8 bf16 held in a 16-byte vector
__device__ __forceinline__ void unpack8(const u32x4 v, float (&f)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    f[2 * i] = __uint_as_float(v[i] << 16);
    f[2 * i + 1] = __uint_as_float(v[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ u32x4 pack8(const float (&f)[8]) {
  u32x4 v;
#pragma unroll
  for (int i = 0; i < 4; ++i) v[i] = (uint32_t)f2bf(f[2 * i]) | ((uint32_t)f2bf(f[2 * i + 1]) << 16);
  return v;
}

// The logistic function on the hardware exponential and reciprocal (v_exp_f32,
// v_rcp_f32: about one ulp each), not an IEEE division: a few ulps of float32,
// far below the bf16 rounding that follows every use.
__device__ __forceinline__ float sigmoidf_(float g) { return __builtin_amdgcn_rcpf(1.0f + __expf(-g)); }

// A 16-byte store of a product's output with the streaming (non-temporal) hint:
// the outputs are far larger than the L2 caches and read back, if at all, by a
// later launch, so they should not evict the operand tiles that the workgroups
// of an XCD share (measured per fwd+bwd step: -0.6% at T=8192, H=7168, I=2048,
// E=32, K=8 with one hot expert; -1.6% at T=4000, H=2048, I=768, E=128, K=8, Zipf).
__device__ __forceinline__ void store16_stream(uint16_t* p, u32x4 v) {
  __builtin_nontemporal_store(v, reinterpret_cast<u32x4*>(p));
}

}  // namespace hmm
