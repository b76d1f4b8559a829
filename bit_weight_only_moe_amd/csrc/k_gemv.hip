// Grouped SwiGLU experts on the VALU (decode-sized token counts): the
// "expert-indexed GEMVs" of "[Model] Add Flint (RecursiveSI/flint)", section
// "What happened".  Weights are read once per touched expert, however many of
// the batch's tokens chose it.
//
// Work units: every routed expert with at least one sorted row (listed in
// `active`), plus optionally the always-on shared expert over all tokens
// ("Recursive Flint: 125 tok/s on an M4 Pro, measured where it matters
// least", table under "What actually shipped").  A block takes one unit and
// a slice of its output rows; tokens are staged in LDS in batches of kNT.
#include "gemv.cuh"
#include "launch.h"
#include "route.cuh"

namespace moe {

constexpr int kNT = 8;

// active[0] = number of experts with rows, active[1 + a] = their ids (increasing).
__global__ void __launch_bounds__(1024) k_active_list(const int32_t* __restrict__ offsets, int E,
                                                      int32_t* __restrict__ active) {
  __shared__ int scan_lds[17];
  const int e = threadIdx.x;
  const int flag = (e < E) && (offsets[e + 1] > offsets[e]);
  int total;
  const int pos = block_exclusive_scan(flag, scan_lds, total);
  if (flag) active[1 + pos] = e;
  if (e == 0) active[0] = total;
}

struct UnitTable {
  const int32_t* active;        // [0] = count, [1 + a] = expert id
  const int32_t* offsets;       // [E + 1] sorted rows per expert
  const int32_t* sorted_pairs;  // token of sorted row r = sorted_pairs[r] / k (NULL: r)
  int k;
  int max_active;               // grid slots for routed units
  int shared_T;                 // > 0: unit max_active is the shared expert over tokens [0, shared_T)
};

struct Unit {
  int e, r0, r1;
  bool shared;
};

MOE_DEV bool resolve_unit(const UnitTable& u, int a, Unit& out) {
  if (u.shared_T > 0 && a == u.max_active) {
    out.e = 0;
    out.r0 = 0;
    out.r1 = u.shared_T;
    out.shared = true;
    return true;
  }
  if (a >= u.max_active || a >= u.active[0]) return false;
  out.e = u.active[1 + a];
  out.r0 = u.offsets[out.e];
  out.r1 = u.offsets[out.e + 1];
  out.shared = false;
  return true;
}

// h[r, i] = bf16(silu(gate_e[i] . x_r) * (up_e[i] . x_r)) for the unit's rows r.
template <int FMT>
__global__ void __launch_bounds__(256) k_gateup(UnitTable u, const uint16_t* __restrict__ x, int H, MatDev gate,
                                                MatDev up, MatDev sgate, MatDev sup, uint16_t* __restrict__ h_routed,
                                                uint16_t* __restrict__ h_shared, int rows_per_block, int nslices,
                                                int lpr) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + (size_t)kNT * H * sizeof(uint16_t));
  Unit un;
  if (!resolve_unit(u, blockIdx.x / nslices, un)) return;
  const MatDev& G = un.shared ? sgate : gate;
  const MatDev& U = un.shared ? sup : up;
  const int Iu = G.rows;
  uint16_t* hout = un.shared ? h_shared : h_routed;
  const int i0 = (blockIdx.x % nslices) * rows_per_block;
  if (i0 >= Iu) return;
  const int i1 = min(Iu, i0 + rows_per_block);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = (H / 32) / lpr;
  const float tsg = tensor_scale<FMT>(G, un.e), tsu = tensor_scale<FMT>(U, un.e);

  for (int rb = un.r0; rb < un.r1; rb += kNT) {
    const int nt = min(kNT, un.r1 - rb);
    __syncthreads();
    for (int t = 0; t < nt; ++t) {
      const int r = rb + t;
      const int tok = (un.shared || !u.sorted_pairs) ? r : u.sorted_pairs[r] / u.k;
      stage_token<FMT>(xs + t * H, xsum + t * (H / 32), x + (size_t)tok * H, H, tid, 256);
    }
    __syncthreads();
    for (int base = i0 + wave * rpw; base < i1; base += 4 * rpw) {
      const int i = base + rsub;
      const bool valid = i < i1;
      float ag[kNT], au[kNT];
#pragma unroll
      for (int t = 0; t < kNT; ++t) ag[t] = au[t] = 0.f;
      if (valid) {
        const uint8_t *gc = row_codes(G, un.e, i), *gs = row_scales<FMT>(G, un.e, i), *gz = row_zeros(G, un.e, i);
        const uint8_t *uc = row_codes(U, un.e, i), *us = row_scales<FMT>(U, un.e, i), *uz = row_zeros(U, un.e, i);
        for (int j0 = 0; j0 < ppl; j0 += 4) {
          RawPiece rg[4], ru[4];
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j0 + j < ppl) {
              const int p = lir + (j0 + j) * lpr;
              rg[j] = load_piece<FMT>(gc, gs, gz, p);
              ru[j] = load_piece<FMT>(uc, us, uz, p);
            }
          }
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            if (j0 + j < ppl) {
              const int p = lir + (j0 + j) * lpr;
              piece_dot<FMT, kNT>(rg[j], p, xs, H, xsum, H / 32, nt, ag);
              piece_dot<FMT, kNT>(ru[j], p, xs, H, xsum, H / 32, nt, au);
            }
          }
        }
      }
#pragma unroll
      for (int t = 0; t < kNT; ++t) {
        if (t < nt) {
          ag[t] = group_sum_dyn(ag[t], lpr);
          au[t] = group_sum_dyn(au[t], lpr);
        }
      }
      if (valid && lir == 0) {
#pragma unroll
        for (int t = 0; t < kNT; ++t) {
          if (t < nt) {
            const float g = ag[t] * tsg, uu = au[t] * tsu;
            hout[(size_t)(rb + t) * Iu + i] = (uint16_t)f32_to_bf16_rne(silu_f32(g) * uu);
          }
        }
      }
    }
  }
}

// out[r, n] = down_e[n] . h_r (fp32, unweighted) for the unit's rows r.
template <int FMT>
__global__ void __launch_bounds__(256) k_down(UnitTable u, const uint16_t* __restrict__ h_routed,
                                              const uint16_t* __restrict__ h_shared, MatDev down, MatDev sdown,
                                              float* __restrict__ out_routed, float* __restrict__ out_shared,
                                              int rows_per_block, int nslices, int lpr_r, int lpr_s, int Kmax) {
  extern __shared__ __align__(16) uint8_t smem[];
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + (size_t)kNT * Kmax * sizeof(uint16_t));
  Unit un;
  if (!resolve_unit(u, blockIdx.x / nslices, un)) return;
  const MatDev& D = un.shared ? sdown : down;
  const int K = D.cols, H = D.rows;
  const uint16_t* hin = un.shared ? h_shared : h_routed;
  float* out = un.shared ? out_shared : out_routed;
  const int n0 = (blockIdx.x % nslices) * rows_per_block;
  if (n0 >= H) return;
  const int n1 = min(H, n0 + rows_per_block);
  const int lpr = un.shared ? lpr_s : lpr_r;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = (K / 32) / lpr;
  const float ts = tensor_scale<FMT>(D, un.e);

  for (int rb = un.r0; rb < un.r1; rb += kNT) {
    const int nt = min(kNT, un.r1 - rb);
    __syncthreads();
    for (int t = 0; t < nt; ++t)
      stage_token<FMT>(xs + t * K, xsum + t * (K / 32), hin + (size_t)(rb + t) * K, K, tid, 256);
    __syncthreads();
    for (int base = n0 + wave * rpw; base < n1; base += 4 * rpw) {
      const int n = base + rsub;
      const bool valid = n < n1;
      float acc[kNT];
#pragma unroll
      for (int t = 0; t < kNT; ++t) acc[t] = 0.f;
      if (valid) {
        const uint8_t *dc = row_codes(D, un.e, n), *ds = row_scales<FMT>(D, un.e, n), *dz = row_zeros(D, un.e, n);
        for (int j0 = 0; j0 < ppl; j0 += 4) {
          RawPiece rd[4];
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j0 + j < ppl) rd[j] = load_piece<FMT>(dc, ds, dz, lir + (j0 + j) * lpr);
#pragma unroll
          for (int j = 0; j < 4; ++j)
            if (j0 + j < ppl) piece_dot<FMT, kNT>(rd[j], lir + (j0 + j) * lpr, xs, K, xsum, K / 32, nt, acc);
        }
      }
#pragma unroll
      for (int t = 0; t < kNT; ++t)
        if (t < nt) acc[t] = group_sum_dyn(acc[t], lpr);
      if (valid && lir == 0) {
#pragma unroll
        for (int t = 0; t < kNT; ++t)
          if (t < nt) out[(size_t)(rb + t) * H + n] = acc[t] * ts;
      }
    }
  }
}

static MatDev to_dev(const moe_w4_matrix& m) {
  MatDev d;
  d.codes = m.codes;
  d.scales = (const uint8_t*)m.scales;
  d.zeros = m.zeros;
  d.ts = m.tensor_scale;
  d.rows = m.rows;
  d.cols = m.cols;
  return d;
}

static const moe_w4_matrix kNoMatrix = {0, 0, 0, 64, nullptr, nullptr, nullptr, nullptr};

constexpr int kGateupRows = 16;
constexpr int kDownRows = 64;

hipError_t launch_gemv_ffn(const moe_ffn_weights* routed, const int32_t* active, const int32_t* offsets,
                           const int32_t* sorted_pairs, int k, int max_active, const moe_ffn_weights* shared,
                           int shared_T, const uint16_t* x, int H, uint16_t* h_routed, uint16_t* h_shared,
                           float* out_routed, float* out_shared, hipStream_t s) {
  UnitTable u;
  u.active = active;
  u.offsets = offsets;
  u.sorted_pairs = sorted_pairs;
  u.k = k;
  u.max_active = max_active;
  u.shared_T = shared ? shared_T : 0;
  const int fmt = routed ? routed->gate.fmt : shared->gate.fmt;
  const moe_w4_matrix& rg = routed ? routed->gate : kNoMatrix;
  const moe_w4_matrix& ru = routed ? routed->up : kNoMatrix;
  const moe_w4_matrix& rd = routed ? routed->down : kNoMatrix;
  const moe_w4_matrix& sg = shared ? shared->gate : kNoMatrix;
  const moe_w4_matrix& su = shared ? shared->up : kNoMatrix;
  const moe_w4_matrix& sd = shared ? shared->down : kNoMatrix;
  const int I = routed ? rg.rows : 0, Is = shared ? sg.rows : 0;
  const int units = max_active + (u.shared_T > 0 ? 1 : 0);
  if (units == 0) return hipSuccess;
  // gate/up
  {
    const int nslices = (std::max(I, Is) + kGateupRows - 1) / kGateupRows;
    const int lpr = lanes_per_row(H);
    const size_t lds = (size_t)kNT * H * sizeof(uint16_t) + (size_t)kNT * (H / 32) * sizeof(float);
    dim3 grid(units * nslices);
    if (fmt == kFmtNvfp4)
      hipLaunchKernelGGL(k_gateup<kFmtNvfp4>, grid, dim3(256), lds, s, u, x, H, to_dev(rg), to_dev(ru), to_dev(sg),
                         to_dev(su), h_routed, h_shared, kGateupRows, nslices, lpr);
    else
      hipLaunchKernelGGL(k_gateup<kFmtInt4>, grid, dim3(256), lds, s, u, x, H, to_dev(rg), to_dev(ru), to_dev(sg),
                         to_dev(su), h_routed, h_shared, kGateupRows, nslices, lpr);
  }
  // down
  {
    const int nslices = (H + kDownRows - 1) / kDownRows;
    const int Kmax = std::max(I, Is);
    const int lpr_r = I ? lanes_per_row(I) : 64, lpr_s = Is ? lanes_per_row(Is) : 64;
    const size_t lds = (size_t)kNT * Kmax * sizeof(uint16_t) + (size_t)kNT * (Kmax / 32) * sizeof(float);
    dim3 grid(units * nslices);
    if (fmt == kFmtNvfp4)
      hipLaunchKernelGGL(k_down<kFmtNvfp4>, grid, dim3(256), lds, s, u, h_routed, h_shared, to_dev(rd), to_dev(sd),
                         out_routed, out_shared, kDownRows, nslices, lpr_r, lpr_s, Kmax);
    else
      hipLaunchKernelGGL(k_down<kFmtInt4>, grid, dim3(256), lds, s, u, h_routed, h_shared, to_dev(rd), to_dev(sd),
                         out_routed, out_shared, kDownRows, nslices, lpr_r, lpr_s, Kmax);
  }
  return hipGetLastError();
}

hipError_t launch_active_list(const int32_t* offsets, int E, int32_t* active, hipStream_t s) {
  hipLaunchKernelGGL(k_active_list, dim3(1), dim3(1024), 0, s, offsets, E, active);
  return hipGetLastError();
}

}  // namespace moe
