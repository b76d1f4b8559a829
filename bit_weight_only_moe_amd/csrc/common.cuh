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
constexpr int kFmtInt4Sb = 3;  // INT4 with scale and bias per group of 64
constexpr int kFmtBf16 = 4;    // 16-bit weights, no quantisation
// Weights per GEMV piece (one 16-byte load of a row): 32 four-bit codes, or 8
// bf16 weights (one 16-byte chunk of a staged token piece).
constexpr int piece_w(int fmt) { return fmt == kFmtBf16 ? 8 : 32; }
// Token staging layout: the INT4 forms stage permuted chunks plus piece sums.
constexpr bool int_layout(int fmt) { return fmt == kFmtInt4 || fmt == kFmtInt4Sb; }

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
// magic: 0x43004300 (the bf16 pair (128, 128)) held in a VGPR (int4_magic()):
// with both constants literal the compiler emits an AND and an OR (CDNA's
// three-operand encoding takes no literal), with the magic in a register a
// single v_and_or_b32 (the mask goes in a scalar register).  Written as an
// asm statement (no side effects, so still scheduled freely): in plain C the
// compiler unpacks every resident piece as soon as its codes arrive, which
// held the multi-token gate/up kernels compiled for the Flint shape at 128
// registers with 73 spilled and the down kernel at 180; as asm they take 106
// and 108 and spill nothing.
template <int S>
MOE_DEV moe_bf16x2 int4x2_to_bf16_off128(uint32_t word, uint32_t magic) {
  uint32_t v;
  if constexpr (S == 0)
    asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(v) : "v"(word), "s"(0x000F000Fu), "v"(magic));
  else
    asm("v_lshrrev_b32 %0, %4, %1\n\tv_and_or_b32 %0, %0, %2, %3"
        : "=&v"(v)
        : "v"(word), "s"(0x000F000Fu), "v"(magic), "i"(4 * S));
  return __builtin_bit_cast(moe_bf16x2, v);
}

MOE_DEV uint32_t int4_magic() {
  uint32_t m = 0x43004300u;
  asm("" : "+v"(m));
  return m;
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

namespace moe {

// ---- DPP-based wave reductions (gfx9 row_shr / row_bcast) ---------------
// Each helper leaves the full result in every lane.

template <int CTRL, int ROW_MASK = 0xf, int BANK_MASK = 0xf>
MOE_DEV uint32_t dpp_u32(uint32_t old, uint32_t v) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)v, CTRL, ROW_MASK, BANK_MASK, false);
}

MOE_DEV uint64_t max_u64(uint64_t a, uint64_t b) { return a > b ? a : b; }

template <int CTRL, int ROW_MASK, int BANK_MASK>
MOE_DEV uint64_t dpp_max_step(uint64_t v) {
  const uint32_t lo = dpp_u32<CTRL, ROW_MASK, BANK_MASK>(0u, (uint32_t)v);
  const uint32_t hi = dpp_u32<CTRL, ROW_MASK, BANK_MASK>(0u, (uint32_t)(v >> 32));
  return max_u64(v, ((uint64_t)hi << 32) | lo);
}

// Maximum of a 64-bit key over the wave (0 is the identity): inclusive
// max-scan with row_shr 1, 2, 3, 4, 8 and row_bcast 15, 31; lane 63 holds
// the result, which is broadcast to all lanes.
MOE_DEV uint64_t wave_max_u64(uint64_t v) {
  v = dpp_max_step<0x111, 0xf, 0xf>(v);
  v = dpp_max_step<0x112, 0xf, 0xf>(v);
  v = dpp_max_step<0x113, 0xf, 0xf>(v);
  v = dpp_max_step<0x114, 0xf, 0xe>(v);
  v = dpp_max_step<0x118, 0xf, 0xc>(v);
  v = dpp_max_step<0x142, 0xa, 0xf>(v);
  v = dpp_max_step<0x143, 0xc, 0xf>(v);
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, 63);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), 63);
  return ((uint64_t)hi << 32) | lo;
}

// fp32 -> uint32 whose unsigned order is the numeric order (-0 folded onto +0).
MOE_DEV uint32_t f32_order_key(float f) {
  uint32_t u = __float_as_uint(f == 0.0f ? 0.0f : f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
MOE_DEV float f32_from_order_key(uint32_t k) {
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : ~k);
}

// ---- workgroup / device synchronisation ---------------------------------
MOE_DEV void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

}  // namespace moe

namespace moe {

// ---- device-coherent accesses for data exchanged between blocks ---------
// Agent-scope relaxed atomic loads/stores are coherent across the chip's
// separate L2 caches without the cache write-back / invalidate that an
// agent-scope fence implies: on gfx950 they carry the device-scope cache
// policy bit (sc1), so a store is written through to the device-coherent
// level and is acknowledged (its vmcnt decrement) only once it is there.
// A producer block stores with st_dev, then block_stores_done() (every wave
// waits for its own stores, then the block barrier), then one thread bumps
// a counter; the consumer that sees the final count issues an agent-scope
// acquire before it reads.
MOE_DEV void st_dev(int32_t* p, int32_t v) { __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); }
MOE_DEV void st_dev(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV void st_dev(float* p, float v) {
  __hip_atomic_store((uint32_t*)p, __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV int32_t ld_dev(const int32_t* p) {
  return __hip_atomic_load(const_cast<int32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV uint32_t ld_dev(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
MOE_DEV float ld_dev(const float* p) {
  return __uint_as_float(__hip_atomic_load((uint32_t*)const_cast<float*>(p), __ATOMIC_RELAXED,
                                           __HIP_MEMORY_SCOPE_AGENT));
}
MOE_DEV uint64_t ld_dev(const uint64_t* p) {
  return __hip_atomic_load(const_cast<uint64_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Every wave of the block waits until all of its own outstanding vector
// memory operations, st_dev stores included, have completed; the barrier
// then orders all of those waits before whatever one thread does next (the
// ticket atomic).  A workgroup-scope release fence would not do here: on
// this target, outside thread-group-split mode, it waits for LDS traffic
// only and leaves global stores in flight.
MOE_DEV void block_stores_done() {
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
  __syncthreads();
}

}  // namespace moe

namespace moe {

// ---- DPP group sums ------------------------------------------------------
template <int CTRL, int ROW_MASK, int BANK_MASK>
MOE_DEV float dpp_f32(float v) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, v), CTRL, ROW_MASK,
                                                               BANK_MASK, false));
}

// Sum over each group of G consecutive lanes (G a power of two <= 64); the
// total lands in the LAST lane of each group (other lanes hold partial sums).
// Built from row_shr (within 16-lane rows) and row_bcast (across rows).
template <int G>
MOE_DEV float group_sum_last(float x) {
  float v = x;
  if (G == 2) {
    v = x + dpp_f32<0x111, 0xf, 0xf>(x);
  } else if (G >= 4) {
    v = x + dpp_f32<0x111, 0xf, 0xf>(x) + dpp_f32<0x112, 0xf, 0xf>(x) + dpp_f32<0x113, 0xf, 0xf>(x);
  }
  if (G >= 8) v += dpp_f32<0x114, 0xf, 0xa>(v);
  if (G >= 16) v += dpp_f32<0x118, 0xf, 0xc>(v);
  if (G >= 32) v += dpp_f32<0x142, 0xa, 0xf>(v);
  if (G >= 64) v += dpp_f32<0x143, 0xc, 0xf>(v);
  return v;
}

MOE_DEV float group_sum_last_dyn(float v, int g) {
  switch (g) {
    case 64: return group_sum_last<64>(v);
    case 32: return group_sum_last<32>(v);
    case 16: return group_sum_last<16>(v);
    case 8: return group_sum_last<8>(v);
    case 4: return group_sum_last<4>(v);
    case 2: return group_sum_last<2>(v);
    default: return v;
  }
}

// Full-wave sum broadcast to every lane.
MOE_DEV float wave_sum(float v) {
  v = group_sum_last<64>(v);
  return __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), 63));
}

// Gain-free RMS normalisation of one bf16 row of H values (H % 8 == 0) by one
// wave: s = sqrt(mean(r^2) + eps) with the squares summed in a fixed order
// (lane l takes the 8-element chunks l, l + 64, ... in element order, then a
// wave sum), q = 1 / s (rounded once), and x = bf16_RNE(r * q) per element.
// Every caller (the norm kernel, the chained step's first decode launch) goes
// through these functions, so they agree bit for bit.
MOE_DEV float rms_scale_wave(const uint16_t* __restrict__ r, int H, float eps, int lane) {
  const uint4* rr = (const uint4*)r;
  float ss = 0.f;
  for (int i = lane; i < H / 8; i += 64) {
    const uint4 v = rr[i];
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      const float a = bf16_to_f32(w[q] & 0xffffu), b = bf16_to_f32(w[q] >> 16);
      ss = fmaf(a, a, ss);
      ss = fmaf(b, b, ss);
    }
  }
  return 1.0f / sqrtf(wave_sum(ss) / (float)H + eps);
}

// Two bf16 values (packed) times q, rounded to bf16 (packed).
MOE_DEV uint32_t rms_apply2(uint32_t w, float q) {
  return f32_to_bf16_rne(bf16_to_f32(w & 0xffffu) * q) | (f32_to_bf16_rne(bf16_to_f32(w >> 16) * q) << 16);
}

MOE_DEV uint4 rms_apply8(uint4 v, float q) {
  return make_uint4(rms_apply2(v.x, q), rms_apply2(v.y, q), rms_apply2(v.z, q), rms_apply2(v.w, q));
}

// x = rms_norm(r) for one row by one wave, written to dst (and to dst2 when
// not NULL; either may be LDS or global memory).  A lane writes only the
// chunks it reads, after the wave's sum, so dst may alias r.
MOE_DEV void rms_norm_row_wave(const uint16_t* r, int H, float eps, int lane, uint16_t* dst, uint16_t* dst2) {
  const float s = rms_scale_wave(r, H, eps, lane);
  const uint4* rr = (const uint4*)r;
  for (int i = lane; i < H / 8; i += 64) {
    const uint4 o = rms_apply8(rr[i], s);
    ((uint4*)dst)[i] = o;
    if (dst2) ((uint4*)dst2)[i] = o;
  }
}

}  // namespace moe
