// VALU GEMV building blocks for the decode path: packed 4-bit expert rows
// streamed from HBM with 16-byte loads, dequantised in registers, and
// dot-multiplied against a few token vectors staged in LDS (the
// "expert-indexed GEMVs" of "[Model] Add Flint (RecursiveSI/flint)",
// section "What happened").
//
// A row of K weights is cut into pieces of 32 weights (16 bytes of codes).
// LPR lanes share a row; lane `lir` of the group takes pieces lir, lir+LPR,
// ... so each load instruction of a lane group reads LPR*16 consecutive
// bytes.  64/LPR rows are in flight per wave.
//
// Token staging in LDS, per token, K values, stored piece-transposed: the
// c-th 16-byte chunk (c = 0..3) of piece p sits at chunk index c*(K/32) + p,
// so the 64 lanes of a wave, which work on consecutive pieces, read
// consecutive 16-byte chunks (no LDS bank conflicts).  Within a chunk:
//   NVFP4: bf16 in natural order (the FP4 convert yields element pairs 2i, 2i+1);
//   INT4:  bf16 permuted inside every 8-element chunk as x0 x4 x1 x5 x2 x6 x3 x7
//          (the magic-number unpack yields nibble pairs (s, s+4)), plus the fp32
//          sum of each 32-element piece, used to remove the +128 offset and
//          the zero point: sum (q - z) x = sum (128 + q) x - (128 + z) sum x.
#pragma once

#include "common.cuh"

namespace moe {

// Stage rows row_of(0) .. row_of(nt - 1) of `src` (K bf16 values each) into
// LDS in the FMT layout, piece-transposed: row t at dst + t*K, its INT4
// piece sums at dsum + t*(K/32).  Each thread takes whole 32-element pieces and issues the
// loads of two pieces before it writes either, so up to 512 pieces cost one
// memory round trip.
// 32 bf16 values (one piece of a token row) in four 16-byte registers.
struct Piece64 {
  uint4 a, b, c, d;
};

// Store one piece (chunks at a stride of `np` 16-byte chunks) in the FMT layout.
template <int FMT>
MOE_DEV void store_piece(uint4* __restrict__ dst, int np, float* __restrict__ dsum, const Piece64& v) {
  if (!int_layout(FMT)) {
    dst[0] = v.a;
    dst[np] = v.b;
    dst[2 * np] = v.c;
    dst[3 * np] = v.d;
  } else {
    float sum = 0.f;
    const uint4 w4[4] = {v.a, v.b, v.c, v.d};
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const uint4 w = w4[c];
      // elements 0..7 as 16-bit halves of w.x .. w.w
      const uint32_t e0 = w.x & 0xffffu, e1 = w.x >> 16, e2 = w.y & 0xffffu, e3 = w.y >> 16;
      const uint32_t e4 = w.z & 0xffffu, e5 = w.z >> 16, e6 = w.w & 0xffffu, e7 = w.w >> 16;
      uint4 o;
      o.x = e0 | (e4 << 16);
      o.y = e1 | (e5 << 16);
      o.z = e2 | (e6 << 16);
      o.w = e3 | (e7 << 16);
      dst[c * np] = o;
      sum += ((bf16_to_f32(e0) + bf16_to_f32(e1)) + (bf16_to_f32(e2) + bf16_to_f32(e3))) +
             ((bf16_to_f32(e4) + bf16_to_f32(e5)) + (bf16_to_f32(e6) + bf16_to_f32(e7)));
    }
    *dsum = sum;
  }
}

MOE_DEV Piece64 load_piece64(const uint16_t* __restrict__ src) {
  const uint4* s = (const uint4*)src;
  return Piece64{s[0], s[1], s[2], s[3]};
}

// Stage rows row_of(0) .. row_of(nt - 1) of `src` (K bf16 values each) into
// LDS in the FMT layout, piece-transposed: row t at dst + t*K, its INT4
// piece sums at dsum + t*(K/32).  Each thread takes whole 32-element pieces and issues the
// loads of two pieces before it writes either, so up to 512 pieces cost one
// memory round trip.
//
// scl (LDS, may be NULL): the rows are RMS-normalised while staged, element
// v of row t becoming bf16_RNE(v * scl[t]), scl[t] the row's reciprocal root
// (rms_apply8, the same arithmetic as the normalisation kernel).
template <int FMT, typename RowOf>
MOE_DEV void stage_rows(uint16_t* __restrict__ dst, float* __restrict__ dsum, const uint16_t* __restrict__ src,
                        RowOf row_of, int nt, int K, const float* scl = nullptr) {
  const int ppt = K / 32, total = nt * ppt, nthr = blockDim.x;
  for (int p0 = threadIdx.x; p0 < total; p0 += 2 * nthr) {
    const int p1 = p0 + nthr;
    const int t0 = p0 / ppt, t1 = p1 / ppt;
    const int c0 = p0 - t0 * ppt, c1 = p1 - t1 * ppt;
    Piece64 v0 = load_piece64(src + (size_t)row_of(t0) * K + 32 * c0);
    Piece64 v1;
    if (p1 < total) v1 = load_piece64(src + (size_t)row_of(t1) * K + 32 * c1);
    if (scl) {
      const float s0 = scl[t0];
      v0 = Piece64{rms_apply8(v0.a, s0), rms_apply8(v0.b, s0), rms_apply8(v0.c, s0), rms_apply8(v0.d, s0)};
      if (p1 < total) {
        const float s1 = scl[t1];
        v1 = Piece64{rms_apply8(v1.a, s1), rms_apply8(v1.b, s1), rms_apply8(v1.c, s1), rms_apply8(v1.d, s1)};
      }
    }
    store_piece<FMT>((uint4*)(dst + (size_t)t0 * K) + c0, ppt, dsum + p0, v0);
    if (p1 < total) store_piece<FMT>((uint4*)(dst + (size_t)t1 * K) + c1, ppt, dsum + p1, v1);
  }
}

// Raw bytes of one 32-weight piece: 16 bytes of codes, its scale bits and zero
// (INT4 scale + bias: the bias bits).
struct RawPiece {
  uint4 c;
  uint32_t s;
  uint32_t z;
};

// Load piece p of a packed row.
//   codes_row : K/2 bytes;  scales_row: NVFP4 K/16 e4m3 bytes, INT4 K/64 fp16
//   zeros_row : INT4 K/64 bytes; INT4 scale + bias: the biases, K/64 fp16
template <int FMT>
MOE_DEV RawPiece load_piece(const uint8_t* __restrict__ codes_row, const uint8_t* __restrict__ scales_row,
                            const uint8_t* __restrict__ zeros_row, int p) {
  RawPiece r;
  r.c = *(const uint4*)(codes_row + 16 * p);
  if (FMT == kFmtBf16) {
    r.s = r.z = 0;
  } else if (FMT == kFmtNvfp4) {
    r.s = *(const uint16_t*)(scales_row + 2 * p);
    r.z = 0;
  } else {
    r.s = ((const uint16_t*)scales_row)[p >> 1];
    r.z = FMT == kFmtInt4Sb ? (uint32_t)((const uint16_t*)zeros_row)[p >> 1] : (uint32_t)zeros_row[p >> 1];
  }
  return r;
}

// Accumulate the dot products of piece p (already loaded) with nt <= NT
// staged tokens into acc[t] (without the NVFP4 tensor scale).
//   xs   : LDS tokens, token t at xs + t*xstride (bf16 elements), piece-transposed
//   xsum : LDS piece sums (INT4), token t at xsum + t*sstride; sstride = xstride / 32
template <int FMT, int NT>
MOE_DEV void piece_dot(const RawPiece& r, int p, const uint16_t* __restrict__ xs, int xstride,
                       const float* __restrict__ xsum, int sstride, int nt, float (&acc)[NT]) {
  if constexpr (FMT == kFmtBf16) {
    // piece p = 8 weights = chunk p % 4 of staged token piece p / 4
    const int pp = p >> 2, cc = p & 3;
    const moe_bf16x2 w0 = __builtin_bit_cast(moe_bf16x2, r.c.x), w1 = __builtin_bit_cast(moe_bf16x2, r.c.y);
    const moe_bf16x2 w2 = __builtin_bit_cast(moe_bf16x2, r.c.z), w3 = __builtin_bit_cast(moe_bf16x2, r.c.w);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (t < nt) {
        const uint4 xv = ((const uint4*)(xs + t * xstride))[cc * sstride + pp];
        float d = 0.f;
        d = dot2_bf16(w0, xv.x, d);
        d = dot2_bf16(w1, xv.y, d);
        d = dot2_bf16(w2, xv.z, d);
        d = dot2_bf16(w3, xv.w, d);
        acc[t] += d;
      }
    }
    return;
  }
  moe_bf16x2 q[16];
  float b0, b1, zc = 0.f;
  const uint4 c = r.c;
  if (FMT == kFmtNvfp4) {
    b0 = e4m3_to_f32(r.s, 0);
    b1 = e4m3_to_f32(r.s, 1);
    q[0] = e2m1x2_to_bf16<0>(c.x); q[1] = e2m1x2_to_bf16<1>(c.x);
    q[2] = e2m1x2_to_bf16<2>(c.x); q[3] = e2m1x2_to_bf16<3>(c.x);
    q[4] = e2m1x2_to_bf16<0>(c.y); q[5] = e2m1x2_to_bf16<1>(c.y);
    q[6] = e2m1x2_to_bf16<2>(c.y); q[7] = e2m1x2_to_bf16<3>(c.y);
    q[8] = e2m1x2_to_bf16<0>(c.z); q[9] = e2m1x2_to_bf16<1>(c.z);
    q[10] = e2m1x2_to_bf16<2>(c.z); q[11] = e2m1x2_to_bf16<3>(c.z);
    q[12] = e2m1x2_to_bf16<0>(c.w); q[13] = e2m1x2_to_bf16<1>(c.w);
    q[14] = e2m1x2_to_bf16<2>(c.w); q[15] = e2m1x2_to_bf16<3>(c.w);
  } else {
    // The scale and zero are converted here, at their use: left visible, the
    // conversions are hoisted next to their loads and each piece's loads then
    // wait for the previous piece's scale and zero before issuing.
    uint32_t rs = r.s, rz = r.z;
    asm volatile("" : "+v"(rs), "+v"(rz));
    b0 = f16_to_f32((unsigned short)rs);
    if (FMT == kFmtInt4Sb) {
      // sum (s q + b) x = s sum (128 + q) x + (b - 128 s) sum x
      b1 = f16_to_f32((unsigned short)rz) - 128.0f * b0;
    } else {
      b1 = 0.f;
      zc = 128.0f + (float)rz;
    }
    const uint32_t mg = int4_magic();
    q[0] = int4x2_to_bf16_off128<0>(c.x, mg); q[1] = int4x2_to_bf16_off128<1>(c.x, mg);
    q[2] = int4x2_to_bf16_off128<2>(c.x, mg); q[3] = int4x2_to_bf16_off128<3>(c.x, mg);
    q[4] = int4x2_to_bf16_off128<0>(c.y, mg); q[5] = int4x2_to_bf16_off128<1>(c.y, mg);
    q[6] = int4x2_to_bf16_off128<2>(c.y, mg); q[7] = int4x2_to_bf16_off128<3>(c.y, mg);
    q[8] = int4x2_to_bf16_off128<0>(c.z, mg); q[9] = int4x2_to_bf16_off128<1>(c.z, mg);
    q[10] = int4x2_to_bf16_off128<2>(c.z, mg); q[11] = int4x2_to_bf16_off128<3>(c.z, mg);
    q[12] = int4x2_to_bf16_off128<0>(c.w, mg); q[13] = int4x2_to_bf16_off128<1>(c.w, mg);
    q[14] = int4x2_to_bf16_off128<2>(c.w, mg); q[15] = int4x2_to_bf16_off128<3>(c.w, mg);
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (t < nt) {
      const uint4* xp = (const uint4*)(xs + t * xstride) + p;
      const uint4 x0 = xp[0], x1 = xp[sstride], x2 = xp[2 * sstride], x3 = xp[3 * sstride];
      float d0 = 0.f, d1 = 0.f;
      d0 = dot2_bf16(q[0], x0.x, d0); d0 = dot2_bf16(q[1], x0.y, d0);
      d0 = dot2_bf16(q[2], x0.z, d0); d0 = dot2_bf16(q[3], x0.w, d0);
      d0 = dot2_bf16(q[4], x1.x, d0); d0 = dot2_bf16(q[5], x1.y, d0);
      d0 = dot2_bf16(q[6], x1.z, d0); d0 = dot2_bf16(q[7], x1.w, d0);
      d1 = dot2_bf16(q[8], x2.x, d1); d1 = dot2_bf16(q[9], x2.y, d1);
      d1 = dot2_bf16(q[10], x2.z, d1); d1 = dot2_bf16(q[11], x2.w, d1);
      d1 = dot2_bf16(q[12], x3.x, d1); d1 = dot2_bf16(q[13], x3.y, d1);
      d1 = dot2_bf16(q[14], x3.z, d1); d1 = dot2_bf16(q[15], x3.w, d1);
      if (FMT == kFmtNvfp4) {
        acc[t] = fmaf(b0, d0, acc[t]);
        acc[t] = fmaf(b1, d1, acc[t]);
        // one token's staged values at a time: without this the compiler reads
        // every token's chunks first, and the several-token NVFP4 gate/up kernels
        // need 104-106 registers (four waves per SIMD) instead of 90-92 (five);
        // measured: 4/16/64 tokens -3.4/-1/-2%, the 8-token chain -2.2%
        if (NT > 1) __builtin_amdgcn_sched_barrier(0);
      } else if (FMT == kFmtInt4Sb) {
        acc[t] = fmaf(b0, d0 + d1, fmaf(b1, xsum[t * sstride + p], acc[t]));
      } else {
        acc[t] = fmaf(b0, fmaf(-zc, xsum[t * sstride + p], d0 + d1), acc[t]);
      }
    }
  }
}

// A packed matrix stack as the kernels see it.
struct MatDev {
  const uint8_t* codes;
  const uint8_t* scales;
  const uint8_t* zeros;      // INT4 zeros; scale + bias: the biases
  const float* ts;
  int rows, cols;
};

template <int FMT>
MOE_DEV const uint8_t* row_codes(const MatDev& m, int e, int r) {
  return m.codes + ((size_t)e * m.rows + r) * (size_t)(FMT == kFmtBf16 ? m.cols * 2 : m.cols / 2);
}
template <int FMT>
MOE_DEV const uint8_t* row_scales(const MatDev& m, int e, int r) {
  return m.scales + ((size_t)e * m.rows + r) * (size_t)(FMT == kFmtNvfp4 ? m.cols / 16 : (m.cols / 64) * 2);
}
// INT4 zeros (u8) or, for scale + bias, the biases (fp16) of row r.
template <int FMT>
MOE_DEV const uint8_t* row_zeros(const MatDev& m, int e, int r) {
  return m.zeros ? m.zeros + ((size_t)e * m.rows + r) * (size_t)(FMT == kFmtInt4Sb ? (m.cols / 64) * 2 : m.cols / 64)
                 : nullptr;
}
template <int FMT>
MOE_DEV float tensor_scale(const MatDev& m, int e) {
  return FMT == kFmtNvfp4 ? m.ts[e] : 1.0f;
}

// Lanes per row: the largest power of two <= 64 dividing K/32.
inline int lanes_per_row(int K) {
  int pieces = K / 32, l = 64;
  while (l > 1 && (pieces % l)) l >>= 1;
  return l;
}

MOE_DEV float group_sum_dyn(float v, int lpr) {
  for (int off = lpr / 2; off >= 1; off >>= 1) v += __shfl_xor(v, off, 64);
  return v;
}

}  // namespace moe
