// Device helpers shared by the gfx950 kernels of the W4A16 MoE layer.
//
// Number formats (the NVFP4 and group-64 INT4 weights named in "[Model] Add
// Flint (RecursiveSI/flint)", section "What happened", and in "Recursive
// Flint: 125 tok/s on an M4 Pro, measured where it matters least", table
// under "What actually shipped"):
//   e2m1 codes are decoded by the CDNA4 FP4 conversion instructions with a
//   unit scale (the instruction applies only the exponent of its scale
//   operand, so block scales are applied separately); e4m3fn block scales by
//   the gfx950 FP8 conversion, which decodes the OCP e4m3fn encoding;
//   INT4 codes become the bf16 value 128 + q by OR-ing them into the
//   mantissa of the bf16 constant 128.0 (0x4300).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define MOE_DEV __device__ __forceinline__

typedef __bf16 moe_bf16x2 __attribute__((ext_vector_type(2)));
typedef float moe_f32x2 __attribute__((ext_vector_type(2)));

namespace moe {

constexpr int kFmtNvfp4 = 1;
constexpr int kFmtInt4 = 2;

MOE_DEV float bf16_to_f32(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

MOE_DEV float f16_to_f32(uint32_t bits16) { return (float)__builtin_bit_cast(_Float16, (uint16_t)bits16); }

// fp32 -> bf16, round to nearest, ties to even (NaN kept quiet NaN).
MOE_DEV uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return (u >> 16) | 0x40u;
  u += 0x7fffu + ((u >> 16) & 1u);
  return u >> 16;
}

// e4m3fn byte `sel` (0..3) of `word` -> fp32 (exact).
MOE_DEV float e4m3_to_f32(uint32_t word, int sel) {
  switch (sel) {
    case 0: return __builtin_amdgcn_cvt_f32_fp8((int)word, 0);
    case 1: return __builtin_amdgcn_cvt_f32_fp8((int)word, 1);
    case 2: return __builtin_amdgcn_cvt_f32_fp8((int)word, 2);
    default: return __builtin_amdgcn_cvt_f32_fp8((int)word, 3);
  }
}

// The two e2m1 codes of byte `SEL` of `word` -> fp32 pair (low nibble in .x).
template <int SEL>
MOE_DEV moe_f32x2 e2m1x2_to_f32(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(word, 1.0f, SEL);
}

// The two e2m1 codes of byte `SEL` of `word` -> bf16 pair (low nibble first), exact.
template <int SEL>
MOE_DEV moe_bf16x2 e2m1x2_to_bf16(uint32_t word) {
  return __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(word, 1.0f, SEL);
}

// INT4: nibbles S and S+4 of `word` -> bf16 pair (128 + q_S, 128 + q_{S+4}), exact.
template <int S>
MOE_DEV moe_bf16x2 int4x2_to_bf16_off128(uint32_t word) {
  uint32_t v = ((word >> (4 * S)) & 0x000F000Fu) | 0x43004300u;
  return __builtin_bit_cast(moe_bf16x2, v);
}

MOE_DEV float dot2_bf16(moe_bf16x2 a, uint32_t b_bits, float c) {
  return __builtin_amdgcn_fdot2_f32_bf16(a, __builtin_bit_cast(moe_bf16x2, b_bits), c, false);
}

MOE_DEV float silu_f32(float z) { return z / (1.0f + expf(-z)); }

// Sum over groups of G consecutive lanes (G a power of two <= 64).
template <int G>
MOE_DEV float group_sum(float v) {
#pragma unroll
  for (int off = G / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

MOE_DEV uint32_t ld_nc_u32(const void* p) { return __builtin_nontemporal_load((const uint32_t*)p); }

}  // namespace moe
