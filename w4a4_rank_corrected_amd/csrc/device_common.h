// Device-side helpers shared by the HIP kernels of the library (gfx950 only).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace svdq {
namespace dev {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// 1.5 * 2^23: adding it to |v| < 2^22 rounds v to an integer (nearest-even) and
// leaves that integer in the low mantissa bits; as an i32 accumulator seed it
// makes the MFMA's integer result read back as the float 1.5*2^23 + sum.
constexpr float kMagic = 12582912.0f;
constexpr int32_t kMagicBits = 0x4B400000;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Two floats -> packed bf16 pair (round to nearest even; v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  __bf16 a = (__bf16)lo;
  __bf16 b = (__bf16)hi;
  return (uint32_t)__builtin_bit_cast(uint16_t, a) | ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

__device__ __forceinline__ uint16_t bf16_bits(float f) { return __builtin_bit_cast(uint16_t, (__bf16)f); }

__device__ __forceinline__ float f16_to_f32(uint16_t h) { return (float)__builtin_bit_cast(_Float16, h); }

__device__ __forceinline__ u32x4 ldg16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }

// Raw buffer resource over [base, base + bytes): loads whose offset falls
// outside read 0 without touching memory (the hardware range check), so edge
// tiles need no clamping or masking.  Word 3 is the gfx9 raw-buffer format.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Wave-wide max over the four lanes l, l^16, l^32, l^48 (one row of an MFMA
// operand): ds_swizzle for the xor-16 partner, permlane32_swap for xor-32.
__device__ __forceinline__ float max4_rows(float v) {
  float s = __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
  v = fmaxf(v, s);
  auto pr = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(pr[0]), __uint_as_float(pr[1]));
}

}  // namespace dev
}  // namespace svdq
