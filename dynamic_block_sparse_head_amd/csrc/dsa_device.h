// Device-side helpers shared by the gfx950 kernels of libdsa.so.
#pragma once

#include <stdint.h>

#include <hip/hip_runtime.h>

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float floatx16 __attribute__((ext_vector_type(16)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr int kNumXcd = 8;   // MI355X: 8 accelerator complex dies, WGs dispatched round-robin

// bf16 bits -> float (exact)
__device__ __forceinline__ float bf16_to_f32(uint16_t x) { return __uint_as_float(uint32_t(x) << 16); }
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// float -> bf16 bits, round to nearest even (v_cvt_pk_bf16_f32)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 v;
  v[0] = static_cast<__bf16>(lo);
  v[1] = static_cast<__bf16>(hi);
  return __builtin_bit_cast(uint32_t, v);
}

// double -> bf16 bits, rounded once to nearest even.  The double is first
// rounded to float toward zero with the last bit forced to 1 when inexact
// ("round to odd": the discarded bits survive as a sticky bit), then the
// float is rounded to bf16 to nearest even; with 16 spare bits between the
// two formats the result equals direct rounding of the double.
__device__ __forceinline__ uint16_t f64_to_bf16(double x) {
  const float f = static_cast<float>(x);
  uint32_t u = __float_as_uint(f);
  const double back = static_cast<double>(f);
  if (back != x && (u & 0x7f800000u) != 0x7f800000u) {
    if (__builtin_fabs(back) > __builtin_fabs(x)) u -= 1u;   // one step toward zero
    u |= 1u;
  }
  return f32_to_bf16(__uint_as_float(u));
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Raw buffer descriptor over `bytes` bytes from `base`: buffer loads at byte
// offsets outside [0, bytes) return zero instead of touching memory.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, int(bytes), 0x00020000);
}

// Work-item order that keeps consecutive work ids on one XCD: the hardware
// hands workgroup b to XCD b % 8, so id = (b % 8) * per_xcd + b / 8 puts a
// contiguous range of work on each die (its L2 then serves their shared K/V).
__device__ __forceinline__ int xcd_work_id(int per_xcd) {
  const int b = blockIdx.x;
  return (b % kNumXcd) * per_xcd + b / kNumXcd;
}

}  // namespace dsa
