// device_common.h — device-side helpers shared by the stage-1 kernels (stage1.hip, prefill.hip):
// vector types, scalar loads of uniform inputs, the row reductions over the four lanes that hold
// one MFMA row's keys, and bf16 packing. Internal to libdecode_attn.so.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace decode_attn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309417f;

// Read-only kernel inputs (block table, context lengths) are read through the constant address
// space so uniform indices become scalar loads.
typedef const __attribute__((address_space(4))) int32_t* const_i32_ptr;

__device__ __forceinline__ int32_t load_uniform(const int32_t* p, size_t idx) {
  return ((const_i32_ptr)(p))[idx];
}

#ifndef DECODE_ATTN_PERMLANE
#define DECODE_ATTN_PERMLANE 1
#endif

// Reductions of a value with its copies in lanes l ^ 16 and l ^ 32 (the four lanes holding one
// row's keys). gfx950's row-swap permutes (v_permlane16/32_swap) exchange the two halves of a
// 32-lane (or 64-lane) span in the VALU; each lane then holds the pair {x[l], x[l ^ 16]} (resp.
// ^ 32) and combines it, with no LDS round trip as ds_bpermute would need.
__device__ __forceinline__ float max_xor16_32(float v) {
#if DECODE_ATTN_PERMLANE
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const float m16 = fmaxf(__builtin_bit_cast(float, (uint32_t)r16[0]),
                          __builtin_bit_cast(float, (uint32_t)r16[1]));
  const uint32_t c = __builtin_bit_cast(uint32_t, m16);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return fmaxf(__builtin_bit_cast(float, (uint32_t)r32[0]),
               __builtin_bit_cast(float, (uint32_t)r32[1]));
#else
  v = fmaxf(v, __shfl_xor(v, 16));
  return fmaxf(v, __shfl_xor(v, 32));
#endif
}

__device__ __forceinline__ float sum_xor16_32(float v) {
#if DECODE_ATTN_PERMLANE
  const uint32_t b = __builtin_bit_cast(uint32_t, v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(b, b, false, false);
  const float s16 = __builtin_bit_cast(float, (uint32_t)r16[0]) +
                    __builtin_bit_cast(float, (uint32_t)r16[1]);
  const uint32_t c = __builtin_bit_cast(uint32_t, s16);
  const auto r32 = __builtin_amdgcn_permlane32_swap(c, c, false, false);
  return __builtin_bit_cast(float, (uint32_t)r32[0]) + __builtin_bit_cast(float, (uint32_t)r32[1]);
#else
  v += __shfl_xor(v, 16);
  return v + __shfl_xor(v, 32);
#endif
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  const __bf16 a = (__bf16)lo, b = (__bf16)hi;  // round to nearest even
  return (uint32_t)__builtin_bit_cast(uint16_t, a) |
         ((uint32_t)__builtin_bit_cast(uint16_t, b) << 16);
}

}  // namespace
}  // namespace decode_attn
