// mma16.h -- the 32x32x16 MFMA on 16-bit operands (bf16 or fp16, fp32
// accumulation) and the packing helpers that go with it, shared by every
// kernel file: v_mfma_f32_32x32x16_{bf16,f16}, rounding of an fp32 pair to
// the input type (nearest-even), its inverse, and the sum of a rounded pair
// (v_dot2 with (1, 1)).  Each including file keeps its own copy in an
// anonymous namespace.
#ifndef FA_MMA16_H
#define FA_MMA16_H

#include <hip/hip_runtime.h>

#include <stdint.h>

namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));

template <typename T> struct Mma;

template <> struct Mma<__bf16> {
  typedef bf16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  // (a, b) rounded to nearest-even bf16, a in the low half.
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, bf16x2));
  }
  static __device__ __forceinline__ f32x2 unpack2(uint32_t x) {
    return __builtin_convertvector(__builtin_bit_cast(bf16x2, x), f32x2);
  }
  // acc + x.lo + x.hi for a packed pair (v_dot2 with (1, 1)): sums values as
  // rounded to bf16
  static __device__ __forceinline__ float pair_sum(uint32_t x, float acc) {
    const bf16x2 one = {(__bf16)1.0f, (__bf16)1.0f};
    return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, x), one, acc, false);
  }
};

template <> struct Mma<_Float16> {
  typedef f16x8 frag;
  static __device__ __forceinline__ f32x16 mma(frag a, frag b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  static __device__ __forceinline__ uint32_t pack2(float a, float b) {
    const f32x2 x = {a, b};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(x, f16x2));
  }
  static __device__ __forceinline__ f32x2 unpack2(uint32_t x) {
    return __builtin_convertvector(__builtin_bit_cast(f16x2, x), f32x2);
  }
  static __device__ __forceinline__ float pair_sum(uint32_t x, float acc) {
    const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
    return __builtin_amdgcn_fdot2(__builtin_bit_cast(f16x2, x), one, acc, false);
  }
};

}  // namespace

#endif  // FA_MMA16_H
