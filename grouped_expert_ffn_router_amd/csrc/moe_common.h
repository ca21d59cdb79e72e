// Device helpers shared by the kernels of libmoe (gfx950 / CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace moe {

typedef uint16_t bf16_t;  // bfloat16 storage

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ float bf16_to_f32(bf16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}

// float -> bfloat16, round to nearest, ties to even; NaN stays NaN.  gfx950
// converts in hardware (v_cvt_pk_bf16_f32, two values per instruction); an
// exhaustive comparison over every non-NaN float bit pattern gave the same
// bits as the integer round-to-nearest-even formula (u + 0x7fff + lsb) >> 16.
__device__ __forceinline__ bf16_t f32_to_bf16(float f) { return __builtin_bit_cast(bf16_t, (__bf16)f); }

// Two floats -> packed bfloat16 pair (lo in the low half), one instruction.
__device__ __forceinline__ uint32_t f32x2_to_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Storage <-> float for the two activation types.
template <class T> struct Act;
template <> struct Act<bf16_t> {
  __device__ __forceinline__ static float load(bf16_t v) { return bf16_to_f32(v); }
  __device__ __forceinline__ static bf16_t store(float v) { return f32_to_bf16(v); }
};
template <> struct Act<float> {
  __device__ __forceinline__ static float load(float v) { return v; }
  __device__ __forceinline__ static float store(float v) { return v; }
};

// silu(a) = a * sigmoid(a); the reciprocal is the hardware one (within 1 ulp).
__device__ __forceinline__ float silu(float a) { return a * __builtin_amdgcn_rcpf(1.0f + __expf(-a)); }

__device__ __forceinline__ int lane_id() { return (int)__lane_id(); }

// Mask of lanes below the calling lane (wave64).
__device__ __forceinline__ uint64_t lanemask_lt() {
  const int l = lane_id();
  return l == 0 ? 0ull : (~0ull >> (64 - l));
}

}  // namespace moe
