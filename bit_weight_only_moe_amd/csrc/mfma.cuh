// Matrix-core building blocks shared by the prefill and decode kernels:
// bf16 MFMA 32x32x16 operands, exact dequantisation of 32 weights into bf16
// operand chunks, the swizzled LDS tile index, and a written-out step chain.
//
// v_mfma_f32_32x32x16_bf16: lane l supplies row (A) or column (B) l % 32 and
// 8 consecutive k values; accumulator register i of lane l holds row
// (i / 4) * 8 + (l / 32) * 4 + i % 4, column l % 32.
#pragma once

#include <type_traits>

#include "common.cuh"

namespace moe {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

MOE_DEV uint4 to_uint4(u32x4_t v) { return make_uint4(v[0], v[1], v[2], v[3]); }

MOE_DEV int swz(int row, int chunk) { return row * 8 + (chunk ^ (row & 7)); }  // in 16-byte units

MOE_DEV uint32_t pack_bf16(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  const bf16x2_t v = {(__bf16)lo, (__bf16)hi};
  return __builtin_bit_cast(uint32_t, v);
}

// Dequantise 32 consecutive weights (16 bytes of codes) of one row into 4
// bf16 chunks of 8.  NVFP4: two e4m3 block scales (bytes 0, 1 of `sc`).
// INT4: zero point z; the result is the exact integer q - z.  Every value is
// exact in fp32 and in bf16, so the hardware fp32 -> bf16 conversion does
// not round.
template <int FMT>
MOE_DEV void dequant32(uint4 c, uint32_t sc, int z, uint4 (&o)[4]) {
  const uint32_t w[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    float v[8];
    if (FMT == kFmtNvfp4) {
      const float b = e4m3_to_f32(sc, q >> 1);
      const moe_f32x2 p0 = e2m1x2_to_f32<0>(w[q]), p1 = e2m1x2_to_f32<1>(w[q]);
      const moe_f32x2 p2 = e2m1x2_to_f32<2>(w[q]), p3 = e2m1x2_to_f32<3>(w[q]);
      v[0] = p0.x * b; v[1] = p0.y * b; v[2] = p1.x * b; v[3] = p1.y * b;
      v[4] = p2.x * b; v[5] = p2.y * b; v[6] = p3.x * b; v[7] = p3.y * b;
    } else {
      // 2^23 + q as fp32 bits, minus 2^23 + z: exact
      const float off = 8388608.0f + (float)z;
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = __uint_as_float(0x4B000000u | ((w[q] >> (4 * j)) & 15u)) - off;
    }
    o[q].x = pack_bf16(v[0], v[1]);
    o[q].y = pack_bf16(v[2], v[3]);
    o[q].z = pack_bf16(v[4], v[5]);
    o[q].w = pack_bf16(v[6], v[7]);
  }
}

MOE_DEV bf16x8_t lds_frag(const uint4* tile, int row, int chunk) {
  return __builtin_bit_cast(bf16x8_t, tile[swz(row, chunk)]);
}

MOE_DEV f32x16_t mfma(bf16x8_t a, bf16x8_t b, f32x16_t c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// f(kt) for kt = KT .. nk - 1 as compile-time constants, written out.
template <int KT, int NMAX, class F>
MOE_DEV void unrolled_steps(int nk, F& f) {
  if constexpr (KT < NMAX) {
    if (KT >= nk) return;
    f(std::integral_constant<int, KT>{});
    unrolled_steps<KT + 1, NMAX>(nk, f);
  }
}

}  // namespace moe
