// The MoE layer for decode-sized batches (T <= 64) in three launches (gfx950).
//
// The layer of "[Model] Add Flint (RecursiveSI/flint)", section "What
// happened" (fused top-k router, expert-indexed GEMVs over W4A16 weights),
// with the always-on shared expert of "Recursive Flint: 125 tok/s on an M4
// Pro, measured where it matters least" (table under "What actually
// shipped").  No block ever waits for another (spinning blocks starve the
// memory system on this chip); cross-block hand-offs inside a launch use
// the "last one out" pattern: producers store results with device-coherent
// stores and take a ticket from an atomic counter, and the block that takes
// the final ticket continues with a device-scope acquire.
//
//   launch 1  router blocks: logits of 4 experts (one per wave); the last
//             router block does top-k, softmax and the expert grouping.
//             shared-expert blocks (same grid): gate/up + SwiGLU, which needs
//             no routing, so its weights stream while the router runs.
//   launch 2  routed gate/up + SwiGLU: one (touched expert, 16-row slice) per
//             block; each touched expert's weights are read once for all the
//             tokens that chose it.
//   launch 3  down projection: one (unit = touched or shared expert, 64-row
//             slice of H) per block, fp32 outputs to the workspace; the last
//             block of each slice combines y = residual + sum_j w_j o_j +
//             o_shared in that fixed order and rounds to bf16.
//
// Every block loads all of its weight pieces before it uses any, so one
// memory round trip covers a block's whole share of the expert bytes.
#include "gemv.cuh"
#include "launch.h"
#include "route.cuh"

namespace moe {

#ifdef MOE_TRACE
// Per-block phase timestamps (100 MHz constant clock) for development builds.
__device__ unsigned long long g_trace[3][65536 * 4];
#define MOE_TRACE_AT(kern, slot)                                                      \
  do {                                                                                \
    if (threadIdx.x == 0 && blockIdx.x < 65536)                                       \
      g_trace[kern][blockIdx.x * 4 + (slot)] = __builtin_amdgcn_s_memrealtime();      \
  } while (0)
#else
#define MOE_TRACE_AT(kern, slot) \
  do {                           \
  } while (0)
#endif

constexpr int kRG = 16;      // gate/up rows per block
constexpr int kRD = 64;      // down rows per block
constexpr int kMaxPc = 8;    // weight pieces per lane held in registers per matrix

// Synchronisation words (ints) at the start of the workspace, 64 bytes apart.
constexpr int kTicketRouter = 0;
constexpr int kTicketSlice = 16;  // + 16 * slice

struct LayerArgs {
  int T, H, I, Is, E, k;
  const uint16_t* x;
  const uint16_t* residual;
  uint16_t* y;
  const float* w_router;
  MatDev gate, up, down;
  MatDev sgate, sup, sdown;  // sgate.codes == nullptr: no shared expert
  int* sync;
  float* logits;             // [T, E]
  int32_t* ids;              // [T*k]
  float* w;                  // [T*k]
  int32_t* offsets;          // [E + 1]
  int32_t* sorted_pairs;     // [T*k]
  int32_t* pair_pos;         // [T*k]
  int32_t* active;           // [1 + E]
  uint16_t* h_routed;        // [T*k, I]
  uint16_t* h_shared;        // [T, Is]
  float* o_routed;           // [T*k, H]
  float* o_shared;           // [T, H]
  int32_t* ids_out;
  float* w_out;
  int nR, nS;                // launch 1 layout
  int slices_r;              // launch 2: gate/up slices per routed expert
  int slices_d;              // launch 3: row slices of H
  int lpr_h, lpr_i, lpr_is;
};

// ------------------------------------------------------------------ gate/up
// Load this lane's pieces c0 .. c0+kMaxPc-1 (row iteration c / ppl, piece
// c % ppl) of the gate and up rows into registers.
template <int FMT>
MOE_DEV void load_gateup_chunk(const MatDev& G, const MatDev& U, int e, int c0, int npc, int ppl, int lpr, int lir,
                               int row0, int row_step, int i1, RawPiece (&rg)[kMaxPc], RawPiece (&ru)[kMaxPc]) {
#pragma unroll
  for (int q = 0; q < kMaxPc; ++q) {
    const int c = c0 + q;
    const int i = row0 + row_step * (c / ppl);
    if (c < npc && i < i1) {
      const int p = lir + (c % ppl) * lpr;
      rg[q] = load_piece<FMT>(row_codes(G, e, i), row_scales<FMT>(G, e, i), row_zeros(G, e, i), p);
      ru[q] = load_piece<FMT>(row_codes(U, e, i), row_scales<FMT>(U, e, i), row_zeros(U, e, i), p);
    }
  }
}

// h[r, i] = bf16(silu(gate_e[i] . x_tok(r)) * (up_e[i] . x_tok(r))) for the
// rows r in [r0, r1) and output rows i in [i0, i1).  tok_of(r): token index.
template <int FMT, int NT, typename TokOf>
MOE_DEV void gateup_rows(const MatDev& G, const MatDev& U, int e, int r0, int r1, int i0, int i1, int H,
                         const uint16_t* __restrict__ x, TokOf tok_of, uint16_t* __restrict__ hout, int Iu,
                         int lpr, uint8_t* smem, int kern) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = (H / 32) / lpr;
  const int iters = (i1 - i0 + 4 * rpw - 1) / (4 * rpw);  // row iterations per wave
  const int npc = iters * ppl;                            // pieces per lane per matrix
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + (size_t)NT * H * sizeof(uint16_t));
  const float tsg = tensor_scale<FMT>(G, e), tsu = tensor_scale<FMT>(U, e);
  // When every piece fits in registers they are loaded once, before the
  // tokens are staged, so both memory latencies overlap.
  const bool resident = npc <= kMaxPc;
  RawPiece rg[kMaxPc], ru[kMaxPc];
  const int row0 = i0 + wave * rpw + rsub;
  if (resident) load_gateup_chunk<FMT>(G, U, e, 0, npc, ppl, lpr, lir, row0, 4 * rpw, i1, rg, ru);
  for (int rb = r0; rb < r1; rb += NT) {
    const int nt = min(NT, r1 - rb);
    __syncthreads();
    for (int t = 0; t < nt; ++t)
      stage_token<FMT>(xs + t * H, xsum + t * (H / 32), x + (size_t)tok_of(rb + t) * H, H, tid, 256);
    __syncthreads();
    MOE_TRACE_AT(kern, 1);
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ag[t] = au[t] = 0.f;
    for (int c0 = 0; c0 < npc; c0 += kMaxPc) {
      // piece c of this lane: row iteration c / ppl, piece index c % ppl
      if (!resident) load_gateup_chunk<FMT>(G, U, e, c0, npc, ppl, lpr, lir, row0, 4 * rpw, i1, rg, ru);
#pragma unroll
      for (int q = 0; q < kMaxPc; ++q) {
        const int c = c0 + q;
        if (c < npc) {
          const int i = i0 + wave * rpw + rsub + 4 * rpw * (c / ppl);
          if (i < i1) {
            const int p = lir + (c % ppl) * lpr;
            piece_dot<FMT, NT>(rg[q], p, xs, H, xsum, H / 32, nt, ag);
            piece_dot<FMT, NT>(ru[q], p, xs, H, xsum, H / 32, nt, au);
          }
          if (c % ppl == ppl - 1) {  // the row's last piece: reduce over its lanes and emit
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if (t < nt) {
                ag[t] = group_sum_last_dyn(ag[t], lpr);
                au[t] = group_sum_last_dyn(au[t], lpr);
              }
            }
            if (i < i1 && lir == lpr - 1) {
#pragma unroll
              for (int t = 0; t < NT; ++t)
                if (t < nt)
                  hout[(size_t)(rb + t) * Iu + i] = (uint16_t)f32_to_bf16_rne(silu_f32(ag[t] * tsg) * (au[t] * tsu));
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) ag[t] = au[t] = 0.f;
          }
        }
      }
    }
  }
  MOE_TRACE_AT(kern, 2);
}

// ------------------------------------------------------------------ down
// out[r, n] = down_e[n] . h_r (fp32, unweighted) for rows r in [r0, r1) of
// `hin` (row stride K) and output rows n in [n0, n1).  Stores with st_dev
// when `coherent` (another block of the same launch reads them).
template <int FMT, int NT>
MOE_DEV void down_rows(const MatDev& D, int e, int r0, int r1, int n0, int n1, const uint16_t* __restrict__ hin,
                       float* __restrict__ out, int lpr, bool coherent, uint8_t* smem) {
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = D.cols, H = D.rows;
  const int rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = (K / 32) / lpr;
  const int iters = (n1 - n0 + 4 * rpw - 1) / (4 * rpw);
  const int npc = iters * ppl;
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + (size_t)NT * K * sizeof(uint16_t));
  const float ts = tensor_scale<FMT>(D, e);
  const bool resident = npc <= kMaxPc;  // every piece stays in registers across token batches
  RawPiece rd[kMaxPc];
  if (resident) {
#pragma unroll
    for (int q = 0; q < kMaxPc; ++q) {
      const int n = n0 + wave * rpw + rsub + 4 * rpw * (q / ppl);
      if (q < npc && n < n1) rd[q] = load_piece<FMT>(row_codes(D, e, n), row_scales<FMT>(D, e, n), row_zeros(D, e, n),
                                                      lir + (q % ppl) * lpr);
    }
  }
  for (int rb = r0; rb < r1; rb += NT) {
    const int nt = min(NT, r1 - rb);
    __syncthreads();
    for (int t = 0; t < nt; ++t) stage_token<FMT>(xs + t * K, xsum + t * (K / 32), hin + (size_t)(rb + t) * K, K, tid, 256);
    __syncthreads();
    MOE_TRACE_AT(2, 1);
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
    for (int c0 = 0; c0 < npc; c0 += kMaxPc) {
      if (!resident) {
#pragma unroll
        for (int q = 0; q < kMaxPc; ++q) {
          const int c = c0 + q;
          const int n = n0 + wave * rpw + rsub + 4 * rpw * (c / ppl);
          if (c < npc && n < n1)
            rd[q] = load_piece<FMT>(row_codes(D, e, n), row_scales<FMT>(D, e, n), row_zeros(D, e, n),
                                    lir + (c % ppl) * lpr);
        }
      }
#pragma unroll
      for (int q = 0; q < kMaxPc; ++q) {
        const int c = c0 + q;
        if (c < npc) {
          const int n = n0 + wave * rpw + rsub + 4 * rpw * (c / ppl);
          if (n < n1) piece_dot<FMT, NT>(rd[q], lir + (c % ppl) * lpr, xs, K, xsum, K / 32, nt, acc);
          if (c % ppl == ppl - 1) {  // the row's last piece
#pragma unroll
            for (int t = 0; t < NT; ++t)
              if (t < nt) acc[t] = group_sum_last_dyn(acc[t], lpr);
            if (n < n1 && lir == lpr - 1) {
#pragma unroll
              for (int t = 0; t < NT; ++t) {
                if (t < nt) {
                  float* dst = out + (size_t)(rb + t) * H + n;
                  if (coherent) st_dev(dst, acc[t] * ts);
                  else *dst = acc[t] * ts;
                }
              }
            }
#pragma unroll
            for (int t = 0; t < NT; ++t) acc[t] = 0.f;
          }
        }
      }
    }
  }
}

// ------------------------------------------------------------------ launch 1
template <int FMT, int NT>
__global__ void __launch_bounds__(256) k_layer_route_shared(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int ticket;
  MOE_TRACE_AT(0, 0);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = a.T, H = a.H, E = a.E;
  if ((int)blockIdx.x >= a.nR) {
    const int slice = blockIdx.x - a.nR;
    const int i0 = slice * kRG, i1 = min(a.Is, i0 + kRG);
    gateup_rows<FMT, NT>(a.sgate, a.sup, 0, 0, T, i0, i1, H, a.x, [](int r) { return r; }, a.h_shared, a.Is,
                         a.lpr_h, smem, 0);
    MOE_TRACE_AT(0, 3);
    return;
  }
  // router: one expert per wave, all tokens; tokens staged in LDS 8 at a time,
  // the router row streamed in chunks of 4 float4 per lane
  const int e = blockIdx.x * 4 + wave;
  constexpr int kC = 4;
  constexpr int kTB = 8;
  const int nc = H / 4;
  uint2* xs = (uint2*)smem;  // [kTB][H / 4]
  for (int t0 = 0; t0 < T; t0 += kTB) {
    const int nt = min(kTB, T - t0);
    __syncthreads();
    for (int i = tid; i < nt * nc; i += 256) xs[i] = ((const uint2*)(a.x + (size_t)t0 * H))[i];
    __syncthreads();
    if (e < E) {
      const float4* wr = (const float4*)(a.w_router + (size_t)e * H);
      float s[kTB];
#pragma unroll
      for (int tt = 0; tt < kTB; ++tt) s[tt] = 0.f;
      for (int cb = 0; cb < nc; cb += 64 * kC) {
        float4 wv[kC];
#pragma unroll
        for (int q = 0; q < kC; ++q)
          if (cb + lane + 64 * q < nc) wv[q] = wr[cb + lane + 64 * q];
#pragma unroll
        for (int tt = 0; tt < kTB; ++tt) {
          if (tt < nt) {
#pragma unroll
            for (int q = 0; q < kC; ++q) {
              const int c = cb + lane + 64 * q;
              if (c < nc) {
                const uint2 xv = xs[tt * nc + c];
                s[tt] = fmaf(wv[q].x, bf16_to_f32(xv.x & 0xffffu), s[tt]);
                s[tt] = fmaf(wv[q].y, bf16_to_f32(xv.x >> 16), s[tt]);
                s[tt] = fmaf(wv[q].z, bf16_to_f32(xv.y & 0xffffu), s[tt]);
                s[tt] = fmaf(wv[q].w, bf16_to_f32(xv.y >> 16), s[tt]);
              }
            }
          }
        }
      }
#pragma unroll
      for (int tt = 0; tt < kTB; ++tt) {
        if (tt < nt) {
          const float v = group_sum_last<64>(s[tt]);
          if (lane == 63) a.logits[(size_t)(t0 + tt) * E + e] = v;
        }
      }
    }
  }
  MOE_TRACE_AT(0, 1);
  __syncthreads();
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    ticket = __hip_atomic_fetch_add(a.sync + kTicketRouter, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  MOE_TRACE_AT(0, 2);
  if (ticket != a.nR - 1) return;

  // Last router block: all logits are stored.  Top-k + softmax per token,
  // then the stable grouping of pairs p = t*k + j by expert.  ids within a
  // token are distinct, so the rank of (t, j) among its expert's pairs is the
  // number of earlier tokens that chose the same expert (a 64-bit mask per
  // expert, T <= 64).
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    a.sync[kTicketRouter] = 0;  // ready for the next call
  }
  __syncthreads();
  const int k = a.k, n = T * k;
  unsigned long long* mask = (unsigned long long*)smem;  // [E]
  int32_t* s_ids = (int32_t*)(mask + E);                  // [n]
  float* s_w = (float*)(s_ids + n);                       // [n]
  int32_t* off = (int32_t*)(s_w + n);                     // [E + 1]
  int* scan_tmp = (int*)(off + E + 1);                    // [17]
  for (int t = wave; t < T; t += 4) wave_topk_softmax(a.logits + (size_t)t * E, E, k, lane, s_ids + t * k, s_w + t * k);
  for (int i = tid; i < E; i += 256) mask[i] = 0ull;
  __syncthreads();
  for (int p = tid; p < n; p += 256) atomicOr(&mask[s_ids[p]], 1ull << (p / k));
  __syncthreads();
  int cnt[4], loc = 0, nz = 0;
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = tid * 4 + q;
    cnt[q] = ee < E ? __popcll(mask[ee]) : 0;
    loc += cnt[q];
    nz += cnt[q] > 0;
  }
  int total, ntot;
  int pre = block_exclusive_scan(loc, scan_tmp, total);
  int apre = block_exclusive_scan(nz, scan_tmp, ntot);
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = tid * 4 + q;
    if (ee < E) {
      off[ee] = pre;
      a.offsets[ee] = pre;
      if (cnt[q] > 0) a.active[1 + apre++] = ee;
      pre += cnt[q];
    }
  }
  if (tid == 0) {
    off[E] = total;
    a.offsets[E] = total;
    a.active[0] = ntot;
  }
  __syncthreads();
  for (int p = tid; p < n; p += 256) {
    const int t = p / k, ee = s_ids[p];
    const int pos = off[ee] + __popcll(mask[ee] & ((1ull << t) - 1ull));
    a.sorted_pairs[pos] = p;
    a.pair_pos[p] = pos;
    a.ids[p] = ee;
    a.w[p] = s_w[p];
    if (a.ids_out) {
      a.ids_out[p] = ee;
      a.w_out[p] = s_w[p];
    }
  }
  MOE_TRACE_AT(0, 3);
}

// ------------------------------------------------------------------ launch 2
template <int FMT, int NT>
__global__ void __launch_bounds__(256) k_layer_gateup(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  MOE_TRACE_AT(1, 0);
  const int unit = blockIdx.x / a.slices_r;
  if (unit >= a.active[0]) return;
  const int e = a.active[1 + unit];
  const int i0 = (blockIdx.x % a.slices_r) * kRG, i1 = min(a.I, i0 + kRG);
  const int32_t* sp = a.sorted_pairs;
  const int k = a.k;
  gateup_rows<FMT, NT>(a.gate, a.up, e, a.offsets[e], a.offsets[e + 1], i0, i1, a.H, a.x,
                       [sp, k](int r) { return sp[r] / k; }, a.h_routed, a.I, a.lpr_h, smem, 1);
  MOE_TRACE_AT(1, 3);
}

// ------------------------------------------------------------------ launch 3
template <int FMT, int NT>
__global__ void __launch_bounds__(256) k_layer_down_combine(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int ticket;
  MOE_TRACE_AT(2, 0);
  const int tid = threadIdx.x;
  const int T = a.T, H = a.H, k = a.k;
  const int slice = blockIdx.x % a.slices_d, unit = blockIdx.x / a.slices_d;
  const int n_active = a.active[0];
  const bool has_shared = a.sgate.codes != nullptr;
  const int units = n_active + (has_shared ? 1 : 0);
  if (unit >= units) return;
  const int n0 = slice * kRD, n1 = min(H, n0 + kRD);
  if (unit < n_active) {
    const int e = a.active[1 + unit];
    down_rows<FMT, NT>(a.down, e, a.offsets[e], a.offsets[e + 1], n0, n1, a.h_routed, a.o_routed, a.lpr_i, true,
                       smem);
  } else {
    down_rows<FMT, NT>(a.sdown, 0, 0, T, n0, n1, a.h_shared, a.o_shared, a.lpr_is, true, smem);
  }
  MOE_TRACE_AT(2, 2);
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __syncthreads();
  int* ctr = a.sync + kTicketSlice + 16 * slice;
  if (tid == 0) ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (ticket != units - 1) return;
  // last block of this slice: every unit's rows [n0, n1) are stored
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *ctr = 0;
  }
  __syncthreads();
  const int rows = n1 - n0;
  for (int idx = tid; idx < T * rows; idx += 256) {
    const int t = idx / rows, n = n0 + idx % rows;
    float acc = 0.f;
    for (int j = 0; j < k; ++j) acc = fmaf(a.w[t * k + j], a.o_routed[(size_t)a.pair_pos[t * k + j] * H + n], acc);
    if (has_shared) acc += a.o_shared[(size_t)t * H + n];
    if (a.residual) acc += bf16_to_f32(a.residual[(size_t)t * H + n]);
    a.y[(size_t)t * H + n] = (uint16_t)f32_to_bf16_rne(acc);
  }
  MOE_TRACE_AT(2, 3);
}

// ------------------------------------------------------------------ grouped FFN (composed path)
struct GroupedArgs {
  int H, I, k;
  const uint16_t* x;
  const int32_t* sorted_pairs;  // NULL: sorted row r is token r
  const int32_t* offsets;       // [E + 1]; NULL: one expert (0) over rows [0, rows)
  const int32_t* active;        // [0] = count, [1 + a] = expert id
  int rows;
  MatDev gate, up, down;
  uint16_t* h;                  // [total_rows, I]
  float* out;                   // [total_rows, H]
  int slices_r, slices_d, lpr_h, lpr_i;
};

MOE_DEV bool grouped_unit(const GroupedArgs& g, int unit, int& e, int& r0, int& r1) {
  if (!g.offsets) {
    e = 0;
    r0 = 0;
    r1 = g.rows;
    return unit == 0;
  }
  if (unit >= g.active[0]) return false;
  e = g.active[1 + unit];
  r0 = g.offsets[e];
  r1 = g.offsets[e + 1];
  return true;
}

template <int FMT, int NT>
__global__ void __launch_bounds__(256) k_grouped_gateup(GroupedArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];
  int e, r0, r1;
  if (!grouped_unit(g, blockIdx.x / g.slices_r, e, r0, r1)) return;
  const int i0 = (blockIdx.x % g.slices_r) * kRG, i1 = min(g.I, i0 + kRG);
  const int32_t* sp = g.sorted_pairs;
  const int k = g.k;
  gateup_rows<FMT, NT>(g.gate, g.up, e, r0, r1, i0, i1, g.H, g.x,
                       [sp, k](int r) { return sp ? sp[r] / k : r; }, g.h, g.I, g.lpr_h, smem, 1);
}

template <int FMT, int NT>
__global__ void __launch_bounds__(256) k_grouped_down(GroupedArgs g) {
  extern __shared__ __align__(16) uint8_t smem[];
  int e, r0, r1;
  if (!grouped_unit(g, blockIdx.x / g.slices_d, e, r0, r1)) return;
  const int n0 = (blockIdx.x % g.slices_d) * kRD, n1 = min(g.H, n0 + kRD);
  down_rows<FMT, NT>(g.down, e, r0, r1, n0, n1, g.h, g.out, g.lpr_i, false, smem);
}

// ------------------------------------------------------------------ host side
static MatDev mat_dev(const moe_w4_matrix& m) {
  MatDev d;
  d.codes = m.codes;
  d.scales = (const uint8_t*)m.scales;
  d.zeros = m.zeros;
  d.ts = m.tensor_scale;
  d.rows = m.rows;
  d.cols = m.cols;
  return d;
}

static int layer_nt(int T) { return T == 1 ? 1 : (T <= 4 ? 4 : 8); }

size_t layer_decode_lds(int T, int H, int I, int Is, int E, int k) {
  if (T < 1 || T > 64 || E > 1024 || H > 4096) return 0;
  const int NT = layer_nt(T), Kmax = std::max(I, Is);
  const size_t stage_h = (size_t)NT * H * 2 + (size_t)NT * (H / 32) * 4;
  const size_t stage_i = (size_t)NT * Kmax * 2 + (size_t)NT * (Kmax / 32) * 4;
  const size_t route = (size_t)E * 8 + (size_t)T * k * 8 + (size_t)(E + 1) * 4 + 17 * 4;
  const size_t lds = std::max(stage_h, std::max(stage_i, route));
  return lds <= 64 * 1024 ? lds : 0;
}

int layer_decode_sync_words(int H) { return kTicketSlice + 16 * ((H + kRD - 1) / kRD); }

hipError_t launch_grouped_gemv(const moe_ffn_weights* w, const int32_t* active, const int32_t* offsets,
                               const int32_t* sorted_pairs, int k, int max_active, const uint16_t* x, int H, int I,
                               uint16_t* h, float* out, int rows, hipStream_t s) {
  GroupedArgs g;
  g.rows = rows;
  g.H = H;
  g.I = I;
  g.k = k;
  g.x = x;
  g.sorted_pairs = sorted_pairs;
  g.offsets = offsets;
  g.active = active;
  g.gate = mat_dev(w->gate);
  g.up = mat_dev(w->up);
  g.down = mat_dev(w->down);
  g.h = h;
  g.out = out;
  g.slices_r = (I + kRG - 1) / kRG;
  g.slices_d = (H + kRD - 1) / kRD;
  g.lpr_h = lanes_per_row(H);
  g.lpr_i = lanes_per_row(I);
  constexpr int NT = 8;
  const size_t lds = std::max((size_t)NT * H * 2 + (size_t)NT * (H / 32) * 4,
                              (size_t)NT * I * 2 + (size_t)NT * (I / 32) * 4);
  if (w->gate.fmt == kFmtNvfp4) {
    hipLaunchKernelGGL((k_grouped_gateup<kFmtNvfp4, NT>), dim3(max_active * g.slices_r), dim3(256), lds, s, g);
    hipLaunchKernelGGL((k_grouped_down<kFmtNvfp4, NT>), dim3(max_active * g.slices_d), dim3(256), lds, s, g);
  } else {
    hipLaunchKernelGGL((k_grouped_gateup<kFmtInt4, NT>), dim3(max_active * g.slices_r), dim3(256), lds, s, g);
    hipLaunchKernelGGL((k_grouped_down<kFmtInt4, NT>), dim3(max_active * g.slices_d), dim3(256), lds, s, g);
  }
  return hipGetLastError();
}

template <int FMT, int NT>
static void launch_all(const LayerArgs& a, int max_active, size_t lds, hipStream_t s) {
  hipLaunchKernelGGL((k_layer_route_shared<FMT, NT>), dim3(a.nR + a.nS), dim3(256), lds, s, a);
  hipLaunchKernelGGL((k_layer_gateup<FMT, NT>), dim3(max_active * a.slices_r), dim3(256), lds, s, a);
  const int units = max_active + (a.sgate.codes ? 1 : 0);
  hipLaunchKernelGGL((k_layer_down_combine<FMT, NT>), dim3(units * a.slices_d), dim3(256), lds, s, a);
}

hipError_t launch_layer_decode(const moe_layer_weights* L, const uint16_t* x, const uint16_t* residual, int T,
                               uint16_t* y, int* sync, float* logits, int32_t* ids, float* w, int32_t* offsets,
                               int32_t* sorted_pairs, int32_t* pair_pos, int32_t* active, uint16_t* h_routed,
                               uint16_t* h_shared, float* o_routed, float* o_shared, int32_t* ids_out, float* w_out,
                               hipStream_t s) {
  LayerArgs a;
  a.T = T;
  a.H = L->H;
  a.I = L->I;
  a.E = L->E;
  a.k = L->k;
  a.Is = L->shared ? L->shared->gate.rows : 0;
  a.x = x;
  a.residual = residual;
  a.y = y;
  a.w_router = L->w_router;
  a.gate = mat_dev(L->experts.gate);
  a.up = mat_dev(L->experts.up);
  a.down = mat_dev(L->experts.down);
  if (L->shared) {
    a.sgate = mat_dev(L->shared->gate);
    a.sup = mat_dev(L->shared->up);
    a.sdown = mat_dev(L->shared->down);
  } else {
    a.sgate = a.sup = a.sdown = MatDev{nullptr, nullptr, nullptr, nullptr, 0, 64};
  }
  a.sync = sync;
  a.logits = logits;
  a.ids = ids;
  a.w = w;
  a.offsets = offsets;
  a.sorted_pairs = sorted_pairs;
  a.pair_pos = pair_pos;
  a.active = active;
  a.h_routed = h_routed;
  a.h_shared = h_shared;
  a.o_routed = o_routed;
  a.o_shared = o_shared;
  a.ids_out = ids_out;
  a.w_out = w_out;
  const int max_active = std::min(a.E, T * a.k);
  a.nR = (a.E + 3) / 4;
  a.nS = L->shared ? (a.Is + kRG - 1) / kRG : 0;
  a.slices_r = (a.I + kRG - 1) / kRG;
  a.slices_d = (a.H + kRD - 1) / kRD;
  a.lpr_h = lanes_per_row(a.H);
  a.lpr_i = lanes_per_row(a.I);
  a.lpr_is = a.Is ? lanes_per_row(a.Is) : 64;
  const size_t lds = layer_decode_lds(T, a.H, a.I, a.Is, a.E, a.k);
  const bool nv = L->experts.gate.fmt == kFmtNvfp4;
  switch (layer_nt(T)) {
    case 1:
      nv ? launch_all<kFmtNvfp4, 1>(a, max_active, lds, s) : launch_all<kFmtInt4, 1>(a, max_active, lds, s);
      break;
    case 4:
      nv ? launch_all<kFmtNvfp4, 4>(a, max_active, lds, s) : launch_all<kFmtInt4, 4>(a, max_active, lds, s);
      break;
    default:
      nv ? launch_all<kFmtNvfp4, 8>(a, max_active, lds, s) : launch_all<kFmtInt4, 8>(a, max_active, lds, s);
  }
  return hipGetLastError();
}

}  // namespace moe

#ifdef MOE_TRACE
extern "C" void* moe_trace_ptr() {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(moe::g_trace)) != hipSuccess) return nullptr;
  return p;
}
#endif
