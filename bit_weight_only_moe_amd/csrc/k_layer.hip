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
//   launch 1  router blocks: logits of 4 experts (one per wave) for a batch
//             of tokens (one token up to 8 tokens, else up to 4).  The last
//             router block of a batch does the batch's top-k + softmax (a lone
//             token with all four waves, else one token per wave); the last
//             batch to finish groups every (token, choice) pair by expert and
//             writes one record per touched expert (from 2 to 8 tokens the
//             gate/up blocks group instead).  Shared-expert blocks (same
//             grid): gate/up + SwiGLU, which needs no routing, so its weights
//             stream while the router runs.
//   launch 2  routed gate/up + SwiGLU: one (record, row slice of I) per
//             block; each touched expert's weights are read once for all the
//             tokens that chose it.
//   launch 3  down projection: one (unit = record or shared-expert token
//             batch, row slice of H) per block (NVFP4 at 2 to 16 tokens:
//             about 1024 blocks, each taking several units of its slice),
//             fp32 outputs to the workspace; the last block of each slice
//             combines y = residual + sum_j w_j o_j + o_shared in that fixed
//             order and rounds to bf16.  A lone token instead: each block
//             takes a few output rows of every unit and combines them in LDS
//             itself.
//
// Every block loads all of its weight pieces before it uses any, so one
// memory round trip covers a block's whole share of the expert bytes.
#include "gemv.cuh"
#include "launch.h"
#include "route.cuh"

namespace moe {

// Rows per block (measured: 8 or 32 gate/up rows, 32 or 128 down rows are
// slower from 4 to 64 tokens).
constexpr int kRG = 16;      // gate/up rows per block (4 when T == 1)
constexpr int kRD = 64;      // down rows per block (32 when T == 1)
constexpr int kRDMin = 32;   // smallest down slice: bounds the number of slice tickets
// Lanes per gate/up row when a block's rows meet several tokens: each lane
// group's partial dot products are summed across the group once per (row,
// token), so a quarter wave per row (4 rows reduced at once) costs a quarter of
// the reductions of a whole wave per row (measured, 4 to 64 tokens: 9 to 17%
// faster layer calls; 8 lanes is slower).
constexpr int kLprTokens = 16;
constexpr int kLprDownTokens = 4;  // the same for down rows (I = 768: 2% faster at 64 tokens than 8)
constexpr int kMaxPcG = 4;   // gate/up weight pieces per lane held in registers, per matrix
constexpr int kMaxPcD = 8;   // down weight pieces per lane held in registers
constexpr int kSepCombineT = 16;  // above this many tokens the combine is a launch of its own
constexpr int kSharedInGateupT = 8;  // up to this many tokens (NVFP4) the shared gate/up runs in launch 2
constexpr bool fmt_shared_early(int fmt) { return fmt == kFmtNvfp4; }
constexpr int kRouteT = 4;   // tokens per router block (a batch; its last block routes them, one per wave)
constexpr int kMaxBatches = 16;  // 64 tokens / kRouteT
constexpr int kRec = 4 + 64; // ints per routed-unit record: expert, first row, rows, 0, token[rows]
// From 2 to kGroupInGateupT tokens one wave of each gate/up block groups the
// pairs it needs itself instead of one block at the end of launch 1 (measured:
// 4 tokens 32.8 -> 31.3 us; the 8-token chain 2147 -> 2113 us once the grouping
// took one wave and no block barriers; with the four-wave grouping 8 and 16
// tokens lost 0.5% and 2.5%).  At most 8 tokens: the T*k <= 64 pairs fit one wave.
constexpr int kGroupInGateupT = 8;
// Down blocks of the looping down kernel: about four blocks per CU, each taking
// several units of its slice (measured against one unit per block, the 8-token
// 47-layer chain 2238 -> 2148 us, 16 tokens 66.4 -> 63.9 us; at 64 tokens and in
// the runtime-shape kernels the loop's extra registers cost more than it saves).
constexpr int kDownBlocks = 1024;
constexpr int kMaxDownUnits = 8;
constexpr bool down_loops(int fmt, int nt, int ip) { return fmt == kFmtNvfp4 && nt == 2 && ip > 0; }

// Compile-time shapes: GP = H / 32 and IP = I / 32 pieces per gate/up and down
// row (0: the runtime shape).  Lanes per row as the launcher picks them at
// runtime: the largest power of two up to a cap that divides the pieces.
constexpr int lanes_for(int pieces, int cap) {
  int l = cap;
  while (l > 1 && pieces % l) l >>= 1;
  return l;
}
constexpr int gate_lpr(int NT, int GP) { return GP ? lanes_for(GP, NT == 1 ? 64 : kLprTokens) : 0; }
constexpr int down_lpr(int NT, int IP) { return IP ? lanes_for(IP, NT == 1 ? 64 : kLprDownTokens) : 0; }

// Synchronisation words (ints) at the start of the workspace, 64 bytes apart.
constexpr int kTicketGroup = 0;                         // batches routed
constexpr int kTicketBatch = 16;                        // + 16 * batch: router blocks of a batch done
constexpr int kTicketSlice = 16 * (1 + kMaxBatches);    // + 16 * slice: down units of a slice done

struct LayerArgs {
  int T, H, I, Is, E, k;
  const uint16_t* x;
  // chained step: launch 1 computes x = rms_norm(norm_r) (eps) itself and
  // writes it to x_w (== x) for launches 2 and 3; NULL: x is given
  const uint16_t* norm_r;
  uint16_t* x_w;
  float eps;
  const uint16_t* residual;
  uint16_t* y;
  const float* w_router;
  MatDev gate, up, down;
  MatDev sgate, sup, sdown;  // sgate.codes == nullptr: no shared expert
  int* sync;
  float* logits;             // [T, E]
  int32_t* ids;              // [T*k]
  float* w;                  // [T*k]
  int32_t* pair_pos;         // [T*k]
  int32_t* n_active;         // [1]
  int32_t* rec;              // [max_active, kRec]
  uint16_t* h_routed;        // [T*k, I]
  uint16_t* h_shared;        // [T, Is]
  float* o_routed;           // [T*k, H]
  float* o_shared;           // [T, H]
  int32_t* ids_out;
  float* w_out;
  int max_active;            // min(E, T*k)
  int rt;                    // tokens per router block
  int nRe, nR;               // router blocks: expert groups of 4, total (expert groups x token batches)
  int nsb;                   // shared-expert token batches of NT tokens (0: no shared expert)
  int rg, rd;                // rows per gate/up block, per down block
  int ss_r;                  // shared gate/up row slices
  int slices_r;              // routed gate/up row slices per expert
  int slices_d;              // down row slices of H
  int lpr_h, lpr_i, lpr_is;
  int down_stage_bytes;      // launch 3: LDS bytes of the token staging (16-byte multiple)
  int rows_t1;               // one token: output rows per down block, every unit (0: not used)
  int sync_slices;           // slice tickets in the workspace (cleared by launch 1)
  int sep_combine;           // launch 3 only projects; a fourth launch (k_combine) combines
  int down_groups;           // launch 3: unit groups per slice (block g takes units g, g + G, ...)
  int shared_in_gateup;      // the shared expert's gate/up runs in launch 2 instead of launch 1
};


// ------------------------------------------------------------------ gate/up
// Load this lane's pieces c0 .. c0+kMaxPcG-1 (row iteration c / ppl, piece
// c % ppl) of the gate and up rows into registers.
template <int FMT, int PC>
MOE_DEV void load_gateup_chunk(const MatDev& G, const MatDev& U, int e, int c0, int npc, int ppl, int lpr, int lir,
                               int row0, int row_step, int i1, RawPiece (&rg)[PC], RawPiece (&ru)[PC]) {
#pragma unroll
  for (int q = 0; q < PC; ++q) {
    const int c = c0 + q;
    const int i = row0 + row_step * (c / ppl);
    if (c < npc && i < i1) {
      const int p = lir + (c % ppl) * lpr;
      rg[q] = load_piece<FMT>(row_codes<FMT>(G, e, i), row_scales<FMT>(G, e, i), row_zeros<FMT>(G, e, i), p);
      ru[q] = load_piece<FMT>(row_codes<FMT>(U, e, i), row_scales<FMT>(U, e, i), row_zeros<FMT>(U, e, i), p);
    }
  }
}

// Tokens normalised while staged: x_tok = rms_norm(r_tok) (eps).  Used where
// the rows [r0, r1) are at most 4 tokens (one wave computes each scale);
// scale: LDS for their 4 scales.  r == NULL: the tokens are staged as given.
struct NormIn {
  const uint16_t* r = nullptr;
  float eps = 0.f;
  float* scale = nullptr;
};

// h[r, i] = bf16(silu(gate_e[i] . x_tok(r)) * (up_e[i] . x_tok(r))) for the
// rows r in [r0, r1) and output rows i in [i0, i1).  tok_of(r): token index.
// KP > 0: the rows have KP pieces (H = 32 KP) and LPR lanes share a row, both
// compile-time, and the block's rows take one iteration of its waves (i1 - i0
// <= 4 * 64 / LPR): the piece loop, its row and piece indices and the lane
// reductions are then constants.  KP == 0: the same computation with the
// runtime shape.
template <int FMT, int NT, int KP = 0, int LPR = 0, typename TokOf>
MOE_DEV void gateup_rows(const MatDev& G, const MatDev& U, int e, int r0, int r1, int i0, int i1, int H_rt,
                         const uint16_t* __restrict__ x, TokOf tok_of, uint16_t* __restrict__ hout, int Iu,
                         int lpr_rt, uint8_t* smem, const NormIn& nrm = NormIn{}) {
  constexpr bool FIX = KP > 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = FIX ? 32 * KP : H_rt;
  const int lpr = FIX ? LPR : lpr_rt;
  const int rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = (H / piece_w(FMT)) / lpr;
  const int iters = FIX ? 1 : (i1 - i0 + 4 * rpw - 1) / (4 * rpw);  // row iterations per wave
  const int npc = iters * ppl;                                       // pieces per lane per matrix
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + (size_t)NT * H * sizeof(uint16_t));
  const float tsg = tensor_scale<FMT>(G, e), tsu = tensor_scale<FMT>(U, e);
  // When every piece fits in registers they are loaded once, before the
  // tokens are staged, so both memory latencies overlap.
  constexpr int PC = kMaxPcG;
  const bool resident = npc <= PC;
  RawPiece rg[PC], ru[PC];
  const int row0 = i0 + wave * rpw + rsub;
  if (resident) load_gateup_chunk<FMT, PC>(G, U, e, 0, npc, ppl, lpr, lir, row0, 4 * rpw, i1, rg, ru);
  // normalised tokens: their scales, one wave per token, with the weight loads in flight
  if (nrm.r && wave < r1 - r0) {
    const float sc = rms_scale_wave(nrm.r + (size_t)tok_of(r0 + wave) * H, H, nrm.eps, lane);
    if (lane == 0) nrm.scale[wave] = sc;
  }
  const uint16_t* xsrc = nrm.r ? nrm.r : x;
  for (int rb = r0; rb < r1; rb += NT) {
    const int nt = min(NT, r1 - rb);
    __syncthreads();
    stage_rows<FMT>(xs, xsum, xsrc, [&](int t) { return tok_of(rb + t); }, nt, H,
                    nrm.r ? nrm.scale + (rb - r0) : nullptr);
    __syncthreads();
    float ag[NT], au[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) ag[t] = au[t] = 0.f;
    for (int c0 = 0; c0 < npc; c0 += PC) {
      // piece c of this lane: row iteration c / ppl, piece index c % ppl
      if (!resident) load_gateup_chunk<FMT, PC>(G, U, e, c0, npc, ppl, lpr, lir, row0, 4 * rpw, i1, rg, ru);
#pragma unroll
      for (int q = 0; q < PC; ++q) {
        const int c = c0 + q;
        if (c < npc) {
          const int i = FIX ? row0 : row0 + 4 * rpw * (c / ppl);
          if (i < i1) {
            const int p = lir + (FIX ? c : c % ppl) * lpr;
            piece_dot<FMT, NT>(rg[q], p, xs, H, xsum, H / 32, nt, ag);
            piece_dot<FMT, NT>(ru[q], p, xs, H, xsum, H / 32, nt, au);
          }
          if ((FIX ? c : c % ppl) == ppl - 1) {  // the row's last piece: reduce over its lanes and emit
#pragma unroll
            for (int t = 0; t < NT; ++t) {
              if (t < nt) {
                if (FIX) {
                  ag[t] = group_sum_last<LPR>(ag[t]);
                  au[t] = group_sum_last<LPR>(au[t]);
                } else {
                  ag[t] = group_sum_last_dyn(ag[t], lpr);
                  au[t] = group_sum_last_dyn(au[t], lpr);
                }
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
}

// ------------------------------------------------------------------ down
// out[r, n] = down_e[n] . h_r (fp32, unweighted) for rows r in [r0, r1) of
// `hin` (row stride K) and output rows n in [n0, n1).  Stores with st_dev
// when `coherent` (another block of the same launch reads them).
// KP, LPR as for gateup_rows (K = 32 KP; n1 - n0 <= 4 * 64 / LPR when KP > 0).
template <int FMT, int NT, int KP = 0, int LPR = 0>
MOE_DEV void down_rows(const MatDev& D, int e, int r0, int r1, int n0, int n1, const uint16_t* __restrict__ hin,
                       float* __restrict__ out, int lpr_rt, bool coherent, uint8_t* smem) {
  constexpr bool FIX = KP > 0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int K = FIX ? 32 * KP : D.cols, H = D.rows;
  const int lpr = FIX ? LPR : lpr_rt;
  const int rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = (K / piece_w(FMT)) / lpr;
  const int iters = FIX ? 1 : (n1 - n0 + 4 * rpw - 1) / (4 * rpw);
  const int npc = iters * ppl;
  uint16_t* xs = (uint16_t*)smem;
  float* xsum = (float*)(smem + (size_t)NT * K * sizeof(uint16_t));
  const float ts = tensor_scale<FMT>(D, e);
  constexpr int PC = kMaxPcD;
  const bool resident = npc <= PC;  // every piece stays in registers across token batches
  const int row0 = n0 + wave * rpw + rsub;
  RawPiece rd[PC];
  if (resident) {
#pragma unroll
    for (int q = 0; q < PC; ++q) {
      const int n = FIX ? row0 : row0 + 4 * rpw * (q / ppl);
      if (q < npc && n < n1) rd[q] = load_piece<FMT>(row_codes<FMT>(D, e, n), row_scales<FMT>(D, e, n), row_zeros<FMT>(D, e, n),
                                                      lir + (FIX ? q : q % ppl) * lpr);
    }
  }
  for (int rb = r0; rb < r1; rb += NT) {
    const int nt = min(NT, r1 - rb);
    __syncthreads();
    stage_rows<FMT>(xs, xsum, hin, [rb](int t) { return rb + t; }, nt, K);
    __syncthreads();
    float acc[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) acc[t] = 0.f;
    for (int c0 = 0; c0 < npc; c0 += PC) {
      if (!resident) {
#pragma unroll
        for (int q = 0; q < PC; ++q) {
          const int c = c0 + q;
          const int n = row0 + 4 * rpw * (c / ppl);
          if (c < npc && n < n1)
            rd[q] = load_piece<FMT>(row_codes<FMT>(D, e, n), row_scales<FMT>(D, e, n), row_zeros<FMT>(D, e, n),
                                    lir + (c % ppl) * lpr);
        }
      }
#pragma unroll
      for (int q = 0; q < PC; ++q) {
        const int c = c0 + q;
        if (c < npc) {
          const int n = FIX ? row0 : row0 + 4 * rpw * (c / ppl);
          if (n < n1) piece_dot<FMT, NT>(rd[q], lir + (FIX ? c : c % ppl) * lpr, xs, K, xsum, K / 32, nt, acc);
          if ((FIX ? c : c % ppl) == ppl - 1) {  // the row's last piece
#pragma unroll
            for (int t = 0; t < NT; ++t)
              if (t < nt) acc[t] = FIX ? group_sum_last<LPR>(acc[t]) : group_sum_last_dyn(acc[t], lpr);
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
// Blocks [0, nR): router, 4 experts (one per wave) x up to rt tokens.  The
// block that takes the last router ticket does top-k + softmax for every
// token and groups the (token, choice) pairs by expert.
// Blocks [nR, ...): shared expert gate/up, one (row slice, token batch) each.
template <int FMT, int NT, int GP, int IP>
__global__ void __launch_bounds__(256) k_layer_route_shared(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int ticket;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int T = a.T, H = a.H, E = a.E;
  // The down launch's slice tickets are cleared here (that launch starts after
  // this one ends), the router tickets by the gate/up launch: every call
  // leaves its counters at zero, and a call also clears the other launch's
  // counters, so a call that never finished cannot upset the next one.
  if (blockIdx.x == 0)
    for (int q = tid; q < a.sync_slices; q += 256) a.sync[kTicketSlice + 16 * q] = 0;
  if ((int)blockIdx.x >= a.nR) {
    const int b = blockIdx.x - a.nR;
    const int slice = b % a.ss_r, r0 = (b / a.ss_r) * NT;
    const int i0 = slice * a.rg, i1 = min(a.Is, i0 + a.rg);
    __shared__ float s_nscale[4];
    NormIn nrm;
    if (a.norm_r) nrm = NormIn{a.norm_r, a.eps, s_nscale};
    gateup_rows<FMT, NT, GP, gate_lpr(NT, GP)>(a.sgate, a.sup, 0, r0, min(T, r0 + NT), i0, i1, H, a.x,
                                               [](int r) { return r; }, a.h_shared, a.Is, a.lpr_h, smem, nrm);
    return;
  }
  const int nb = a.nR / a.nRe;  // token batches
  const int batch = blockIdx.x / a.nRe;
  const int t0 = batch * a.rt, nt = min(a.rt, T - t0);
  {
    const int e = (blockIdx.x % a.nRe) * 4 + wave;
    float4 wv[kRouterC];
    // a wave past the last expert loads the last expert's row (never used):
    // no branch around the loads, whose registers the token copy then reuses
    router_prefetch(a.w_router + (size_t)min(e, E - 1) * H, H, lane, wv);
    if (a.norm_r) {
      // the batch's tokens normalised here, one wave each; one block per batch also
      // stores them for the gate/up launch
      if (wave < nt)
        rms_norm_row_wave(a.norm_r + (size_t)(t0 + wave) * H, H, a.eps, lane, (uint16_t*)smem + (size_t)wave * H,
                          blockIdx.x % a.nRe == 0 ? a.x_w + (size_t)(t0 + wave) * H : nullptr);
    } else {
      copy_to_lds((uint4*)smem, (const uint4*)(a.x + (size_t)t0 * H), nt * H / 8);
    }
    __syncthreads();
    if (e < E) {
      // device-coherent stores: the block that takes the batch's last ticket reads them
      auto dots = [&](auto rt) __attribute__((always_inline)) {
        constexpr int RT = decltype(rt)::value;
        float acc[RT];
        router_dots<RT>(a.w_router + (size_t)e * H, (const uint16_t*)smem, H, nt, lane, acc, wv);
#pragma unroll
        for (int t = 0; t < RT; ++t)
          if (t < nt && lane == 63) st_dev(a.logits + (size_t)(t0 + t) * E + e, acc[t]);
      };
      // a lone token (or batches of one token) computes one chain
      if (NT == 1 || a.rt == 1)
        dots(std::integral_constant<int, 1>{});
      else
        dots(std::integral_constant<int, kRouteT>{});
    }
  }
  block_stores_done();  // every logit this block stored is visible chip-wide
  int* ctr = a.sync + kTicketBatch + 16 * batch;
  if (tid == 0) ticket = __hip_atomic_fetch_add(ctr, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (ticket != a.nRe - 1) return;

  // Last router block of this token batch: every logit of its nt <= 4 tokens
  // is stored.  Top-k + softmax, one token per wave.
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *ctr = 0;  // ready for the next call
  }
  __syncthreads();
  const int k = a.k, n = T * k;
  // Byte offsets into smem: pointers formed as smem + offset stay LDS
  // pointers for the compiler (an integer round trip would turn every access
  // below into a slower flat access).
  const int o_w = 4 * n, o_log = 8 * n;
  const int o_mask = (o_log + 4 * kRouteT * E + 7) & ~7, o_off = o_mask + 8 * E;
  const int o_scan = o_off + 4 * (E + 1), o_cv = o_scan + 4 * 17, o_ce = o_cv + 4 * 32;
  const int o_rk = (o_ce + 4 * 32 + 15) & ~15;
  int32_t* s_ids = (int32_t*)smem;                                // [n]
  float* s_w = (float*)(smem + o_w);                              // [n]
  float* s_log = (float*)(smem + o_log);                          // [kRouteT, E]
  unsigned long long* mask = (unsigned long long*)(smem + o_mask);  // [E]
  int32_t* off = (int32_t*)(smem + o_off);                        // [E + 1]
  int* scan_tmp = (int*)(smem + o_scan);                          // [17]
  float* cand_v = (float*)(smem + o_cv);                          // [4 * 8]
  int32_t* cand_e = (int32_t*)(smem + o_ce);                      // [4 * 8]
  uint64_t* rk = (uint64_t*)(smem + o_rk);                        // [kRankScratch]
  copy_f32_to_lds(s_log, a.logits + (size_t)t0 * E, nt * E);
  __syncthreads();
  // a lone token: all four waves share its selection (rank counting for up
  // to 256 experts); several tokens: one per wave (rank counting over the
  // lanes' largest keys for up to 256 experts, else k rounds of a wave maximum)
  if (nt == 1 && E <= 256)
    block_topk_rank(s_log, E, k, rk, s_ids + t0 * k, s_w + t0 * k);
  else if (nt == 1)
    block_topk_softmax(s_log, E, k, wave, lane, cand_v, cand_e, s_ids + t0 * k, s_w + t0 * k);
  else if (wave < nt && E <= 256)
    wave_topk_rank(s_log + wave * E, E, k, lane, rk + wave * kWaveRankScratch, s_ids + (t0 + wave) * k,
                   s_w + (t0 + wave) * k);
  else if (wave < nt)
    wave_topk_softmax(s_log + wave * E, E, k, lane, s_ids + (t0 + wave) * k, s_w + (t0 + wave) * k);
  __syncthreads();
  const int p0 = t0 * k, p1 = (t0 + nt) * k;  // this batch's pairs
  if (NT == 2 && T <= kGroupInGateupT) {
    // each gate/up block groups the pairs it needs itself (group_unit_wave), so this
    // batch only publishes its choices for the next launch
    for (int p = p0 + tid; p < p1; p += 256) {
      a.ids[p] = s_ids[p];
      a.w[p] = s_w[p];
      if (a.ids_out) {
        a.ids_out[p] = s_ids[p];
        a.w_out[p] = s_w[p];
      }
    }
    return;
  }
  if (nb > 1) {
    // Publish this batch's choices; the last batch to finish groups all tokens.
    for (int p = p0 + tid; p < p1; p += 256) {
      st_dev(a.ids + p, s_ids[p]);
      st_dev(a.w + p, s_w[p]);
    }
    block_stores_done();
    if (tid == 0)
      ticket = __hip_atomic_fetch_add(a.sync + kTicketGroup, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __syncthreads();
    if (ticket != nb - 1) return;
    if (tid == 0) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      a.sync[kTicketGroup] = 0;
    }
    __syncthreads();
    for (int p = tid; p < n; p += 256) {
      if (p < p0 || p >= p1) {
        s_ids[p] = a.ids[p];
        s_w[p] = a.w[p];
      }
    }
    __syncthreads();
  }

  if (T == 1) {
    // One token, k distinct experts: each is a unit of one row, and its
    // record index is its rank among the chosen ids.
    if (tid < k) {
      const int ee = s_ids[tid];
      int rank = 0;
      for (int j = 0; j < k; ++j) rank += s_ids[j] < ee;
      int32_t* r = a.rec + (size_t)rank * kRec;
      r[0] = ee;
      r[1] = rank;
      r[2] = 1;
      r[3] = 0;
      r[4] = 0;
      a.pair_pos[tid] = rank;
      a.ids[tid] = ee;
      a.w[tid] = s_w[tid];
      if (a.ids_out) {
        a.ids_out[tid] = ee;
        a.w_out[tid] = s_w[tid];
      }
    }
    if (tid == 0) a.n_active[0] = k;
    return;
  }

  // Every token's choices are in LDS.  Stable grouping of pairs p = t*k + j
  // by expert: ids within a token are distinct, so the rank of (t, j) among
  // its expert's pairs is the number of earlier tokens that chose the same
  // expert (a 64-bit mask per expert, T <= 64).  Each touched expert, in
  // ascending id order, gets a record: expert, first row of its pairs in the
  // grouped order, row count, and the token of each row; records past the
  // last touched expert get expert -1.
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
  // one scan for both prefix sums: pair counts in the low 16 bits (at most
  // T*k <= 512 in all), touched experts in the high 16 bits (at most E)
  int ptot;
  const int pk = block_exclusive_scan(loc | (nz << 16), scan_tmp, ptot);
  int pre = pk & 0xffff, apre = pk >> 16;
  const int ntot = ptot >> 16;
  int32_t* ridx = (int32_t*)s_log;  // [E] record index of each touched expert (the logits are done with)
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int ee = tid * 4 + q;
    if (ee < E) {
      off[ee] = pre;
      if (cnt[q] > 0) {
        ridx[ee] = apre;
        int32_t* r = a.rec + (size_t)(apre++) * kRec;
        r[0] = ee;
        r[1] = pre;
        r[2] = cnt[q];
        r[3] = 0;
      }
      pre += cnt[q];
    }
  }
  for (int u = ntot + tid; u < a.max_active; u += 256) a.rec[(size_t)u * kRec] = -1;
  if (tid == 0) a.n_active[0] = ntot;
  __syncthreads();
  // one thread per pair: its rank among its expert's tokens gives both its
  // grouped row and its slot in the expert's record token list
  for (int p = tid; p < n; p += 256) {
    const int t = p / k, ee = s_ids[p];
    const int rank = __popcll(mask[ee] & ((1ull << t) - 1ull));
    a.pair_pos[p] = off[ee] + rank;
    a.rec[(size_t)ridx[ee] * kRec + 4 + rank] = t;
    if (nb == 1) {
      a.ids[p] = ee;
      a.w[p] = s_w[p];
    }
    if (a.ids_out) {
      a.ids_out[p] = ee;
      a.w_out[p] = s_w[p];
    }
  }
}

// ------------------------------------------------------------------ grouping in launch 2
// Record of unit u (the u-th smallest touched expert) built by one wave of a
// gate/up block from the T*k <= 64 chosen ids of every token (one pair per
// lane): the same expert, first grouped row, row count and token list
// (ascending tokens) that a single grouping block would write, so the grouped
// order is unchanged.  The block of each unit's first slice (`publish`) also
// stores the record and its pairs' grouped rows for the down launch, and unit
// 0's block the number of touched experts.  Units past the last touched
// expert get expert -1.  Called by wave 0 only (the wave's LDS traffic is in
// order, so no block barrier); s_rec is the block's LDS copy, valid after the
// caller's barrier.
MOE_DEV void group_unit_wave(const LayerArgs& a, int u, bool publish, int* s_rec, uint32_t* s_mask) {
  const int lane = threadIdx.x & 63;
  const int k = a.k, n = a.T * k;
  const int id = lane < n ? a.ids[lane] : -1;
  if (lane < 32) s_mask[lane] = 0u;  // touched experts, E <= 1024
  wave_lds_sync();
  if (id >= 0) atomicOr(&s_mask[id >> 5], 1u << (id & 31));
  wave_lds_sync();
  const uint32_t m = lane < 32 ? s_mask[lane] : 0u;
  const int c = __popc(m);
  const int inc = wave_inclusive_scan(c);
  const int total = __shfl(inc, 63, 64);
  int mine = -1;
  if (inc - c <= u && u < inc) {
    uint32_t mm = m;  // drop the set bits below the wanted one
    for (int q = u - (inc - c); q > 0; --q) mm &= mm - 1u;
    mine = lane * 32 + __ffs(mm) - 1;
  }
  const uint64_t who = __ballot(mine >= 0);
  const int e = who ? __shfl(mine, __ffsll((long long)who) - 1, 64) : -1;
  if (publish && u == 0 && lane == 0) a.n_active[0] = total;
  int32_t* rec = a.rec + (size_t)u * kRec;
  if (e < 0) {
    if (lane == 0) {
      s_rec[0] = -1;
      if (publish) rec[0] = -1;
    }
    return;
  }
  const uint64_t beq = __ballot(id == e);
  const int r0 = __popcll(__ballot(id >= 0 && id < e)), cnt = __popcll(beq);
  if (id == e) {
    const int rank = __popcll(beq & ((1ull << lane) - 1ull));
    s_rec[4 + rank] = lane / k;
    if (publish) {
      rec[4 + rank] = lane / k;
      a.pair_pos[lane] = r0 + rank;
    }
  }
  if (lane == 0) {
    s_rec[0] = e;
    s_rec[1] = r0;
    s_rec[2] = cnt;
    s_rec[3] = 0;
    if (publish) {
      rec[0] = e;
      rec[1] = r0;
      rec[2] = cnt;
      rec[3] = 0;
    }
  }
}

// ------------------------------------------------------------------ launch 2
// One (routed-unit record, 16-row slice of I) per block.
// INT4 with several tokens: bounded to 128 registers (4 waves per SIMD; it
// fits without spilling, 5 registers under its unbounded allocation, and
// runs T=16/64 4-6% faster than at 3 waves)
template <int FMT, int NT, int GP, int IP>
__global__ void __launch_bounds__(256, FMT != kFmtNvfp4 && NT > 1 ? 4 : 1) k_layer_gateup(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_rec[kRec];
  if (blockIdx.x == 0 && threadIdx.x <= kMaxBatches) a.sync[16 * threadIdx.x] = 0;  // router tickets
  const int nsh = a.shared_in_gateup ? a.ss_r * a.nsb : 0;
  if ((int)blockIdx.x < nsh) {
    // the shared expert first (its units carry NT tokens each): one (row slice, token batch) per block
    const int slice = blockIdx.x % a.ss_r, r0 = (blockIdx.x / a.ss_r) * NT;
    const int i0 = slice * a.rg, i1 = min(a.Is, i0 + a.rg);
    gateup_rows<FMT, NT, GP, gate_lpr(NT, GP)>(a.sgate, a.sup, 0, r0, min(a.T, r0 + NT), i0, i1, a.H, a.x,
                                               [](int r) { return r; }, a.h_shared, a.Is, a.lpr_h, smem);
    return;
  }
  const int unit = (blockIdx.x - nsh) / a.slices_r;
  if (NT == 2 && a.T <= kGroupInGateupT) {
    __shared__ uint32_t s_mask[32];
    if (threadIdx.x < 64) group_unit_wave(a, unit, (blockIdx.x - nsh) % a.slices_r == 0, s_rec, s_mask);
  } else if (threadIdx.x < kRec)
    s_rec[threadIdx.x] = a.rec[(size_t)unit * kRec + threadIdx.x];
  __syncthreads();
  const int e = s_rec[0];
  if (e < 0) return;
  const int r0 = s_rec[1];
  const int i0 = ((blockIdx.x - nsh) % a.slices_r) * a.rg, i1 = min(a.I, i0 + a.rg);
  gateup_rows<FMT, NT, GP, gate_lpr(NT, GP)>(a.gate, a.up, e, r0, r0 + s_rec[2], i0, i1, a.H, a.x,
                       [r0](int r) { return s_rec[4 + r - r0]; }, a.h_routed, a.I, a.lpr_h, smem);
}

// ------------------------------------------------------------------ launch 3
// One (unit, 64-row slice of H) per block; units are the shared expert's
// token batches, then the routed records.  fp32 outputs go to the
// workspace; the last block of each slice combines
// y = residual + sum_j w_j o_j + o_shared in that fixed order.
template <int FMT, int NT, int GP, int IP>
__global__ void __launch_bounds__(256) k_layer_down_combine(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_rec[kMaxDownUnits][3];
  __shared__ int ticket, s_nact;
  const int tid = threadIdx.x;
  const int T = a.T, H = a.H, k = a.k, n = T * k;
  // Block (group g, slice) takes units g, g + G, g + 2G, ... of its slice
  // (G = down_groups; one unit per block, G = every unit, except in the
  // compiled-shape NVFP4 kernel for 2 to 16 tokens: the others would need more
  // registers for the loop).  The shared expert's units come first: they
  // carry NT tokens each and would otherwise be the launch's tail.
  constexpr bool LOOP = down_loops(FMT, NT, IP);
  const int max_units = a.nsb + a.max_active;
  const int slice = blockIdx.x % a.slices_d, g = blockIdx.x / a.slices_d, G = LOOP ? a.down_groups : max_units;
  const int nmine = g < max_units ? (LOOP ? (max_units - 1 - g) / G + 1 : 1) : 0;  // <= kMaxDownUnits
  // the combine's weights and pair positions (written by launch 1), loaded
  // with the records so the last block needs one more round trip only
  float* s_w = (float*)(smem + a.down_stage_bytes);  // [n]
  int32_t* s_pp = (int32_t*)(s_w + n);                // [n]
  // every candidate unit's record head (expert, first row, rows) in one round trip
  if (tid < 3 * nmine) {
    const int j = tid / 3, u = g + G * j;
    if (u >= a.nsb) s_rec[j][tid % 3] = a.rec[(size_t)(u - a.nsb) * kRec + tid % 3];
  }
  if (tid == 255) s_nact = a.n_active[0];
  if (!a.sep_combine) {
    for (int p = tid; p < n; p += 256) {
      s_w[p] = a.w[p];
      s_pp[p] = a.pair_pos[p];
    }
  }
  __syncthreads();
  const int n0 = slice * a.rd, n1 = min(H, n0 + a.rd);
  int done = 0;  // units of this slice this block projected
  if constexpr (LOOP) {
    for (int j = 0; j < nmine; ++j) {
      // one projection site for both kinds of unit (the matrix and buffers picked per unit)
      const int u = g + G * j;
      const bool sh = u < a.nsb;
      int e = 0, r0 = u * NT, r1 = min(T, r0 + NT);
      if (!sh) {
        e = s_rec[j][0];
        if (e < 0) break;  // past the last touched expert (records are in unit order)
        r0 = s_rec[j][1];
        r1 = r0 + s_rec[j][2];
      }
      down_rows<FMT, NT, IP, down_lpr(NT, IP)>(sh ? a.sdown : a.down, e, r0, r1, n0, n1,
                                               sh ? a.h_shared : a.h_routed, sh ? a.o_shared : a.o_routed,
                                               sh ? a.lpr_is : a.lpr_i, !a.sep_combine, smem);
      ++done;
    }
  } else if (nmine > 0) {
    if (g >= a.nsb) {
      const int e = s_rec[0][0];
      if (e < 0) return;  // past the last touched expert
      down_rows<FMT, NT, IP, down_lpr(NT, IP)>(a.down, e, s_rec[0][1], s_rec[0][1] + s_rec[0][2], n0, n1,
                                               a.h_routed, a.o_routed, a.lpr_i, !a.sep_combine, smem);
    } else {
      const int r0 = g * NT;
      down_rows<FMT, NT, IP, down_lpr(NT, IP)>(a.sdown, 0, r0, min(T, r0 + NT), n0, n1, a.h_shared, a.o_shared,
                                               a.lpr_is, !a.sep_combine, smem);
    }
    done = 1;
  }
  if (a.sep_combine || done == 0) return;  // a combine launch reads the outputs after this launch
  block_stores_done();
  const int units = s_nact + a.nsb;
  int* ctr = a.sync + kTicketSlice + 16 * slice;
  if (tid == 0) ticket = __hip_atomic_fetch_add(ctr, done, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (ticket + done != units) return;
  // last block of this slice: every unit's rows [n0, n1) are stored
  if (tid == 0) {
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    *ctr = 0;
  }
  __syncthreads();
  const bool has_shared = a.nsb > 0;
  const int rows = n1 - n0, total = T * rows;
  // U (token, column) outputs per thread and round, U = 1, 2 or 4 as the
  // slice needs, all of their loads issued before the first sum: one memory
  // round trip per round instead of one per output (this block is the
  // launch's tail).  The loads are unconditional so that no branch splits
  // them: outputs past the end re-read the last one, choices past k re-read
  // choice k - 1, a missing shared expert or residual reads the routed
  // outputs or the tokens instead; none of these enters a stored sum.
  const float* osrc = has_shared ? a.o_shared : a.o_routed;
  const uint16_t* rsrc = a.residual ? a.residual : a.x;
  auto rounds = [&](auto uc) __attribute__((always_inline)) {
    constexpr int U = decltype(uc)::value;
    for (int base = tid; base < total; base += U * 256) {
      float o[U][8], os[U];
      uint32_t rsb[U];  // residual bits, converted at their use (converted here, the
                        // shift would wait for every load issued so far)
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = min(base + u * 256, total - 1);
        const int t = idx / rows, c = n0 + idx % rows;
#pragma unroll
        for (int j = 0; j < 8; ++j) o[u][j] = a.o_routed[(size_t)s_pp[t * k + min(j, k - 1)] * H + c];
        os[u] = osrc[(size_t)t * H + c];
        rsb[u] = rsrc[(size_t)t * H + c];
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int idx = base + u * 256;
        if (idx < total) {
          const int t = idx / rows, c = n0 + idx % rows;
          float acc = 0.f;
#pragma unroll
          for (int j = 0; j < 8; ++j)
            if (j < k) acc = fmaf(s_w[t * k + j], o[u][j], acc);
          if (has_shared) acc += os[u];
          if (a.residual) {
            uint32_t rb = rsb[u];
            asm volatile("" : "+v"(rb));
            acc += bf16_to_f32((uint16_t)rb);
          }
          a.y[(size_t)t * H + c] = (uint16_t)f32_to_bf16_rne(acc);
        }
      }
    }
  };
  const int per_thread = (total + 255) / 256;
  if (per_thread <= 1)
    rounds(std::integral_constant<int, 1>{});
  else if (per_thread <= 2)
    rounds(std::integral_constant<int, 2>{});
  else
    rounds(std::integral_constant<int, 4>{});
}

// ------------------------------------------------------------------ launch 3, one token
// A lone token meets each of its k experts and the shared expert once, so
// one block takes rows [n0, n0 + R) of every unit: R * units row-dots, one
// per lane group, in a single pass.  The outputs meet in LDS and the block
// writes y for its rows itself, so no slice ticket and no reload of the
// other units' outputs.  Each row-dot uses the lanes, pieces and reduction
// of down_rows, and the combine takes the same order as the multi-block
// combine: the results are those of the general launch 3, bit for bit.
constexpr int kMaxUnitsT1 = 9;   // k <= 8 routed experts + the shared expert
constexpr int kT1Threads = 256;  // measured: 512 (8 rows per block) the same, 1024 slower
template <int FMT, int IP>
__global__ void __launch_bounds__(kT1Threads) k_layer_down_t1(LayerArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  __shared__ int s_e[kMaxUnitsT1];
  __shared__ float s_w[kMaxUnitsT1];
  __shared__ int s_pp[kMaxUnitsT1];
  __shared__ float s_o[kT1Threads];  // [unit][row]: units * R <= lane groups <= threads
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int H = a.H, I = a.I, k = a.k, R = a.rows_t1;
  const bool has_shared = a.nsb > 0;
  const int nu = k + (has_shared ? 1 : 0);
  const int n0 = blockIdx.x * R;
  // record r holds the expert of rank r, whose h row is r (written by launch 1)
  if (tid < k) {
    s_e[tid] = a.rec[(size_t)tid * kRec];
    s_w[tid] = a.w[tid];
    s_pp[tid] = a.pair_pos[tid];
  } else if (tid < kMaxUnitsT1) {  // padding read by the combine, never used
    s_w[tid] = 0.f;
    s_pp[tid] = 0;
  }
  __syncthreads();
  constexpr int LPR_C = down_lpr(1, IP);
  const int lpr = IP ? LPR_C : a.lpr_i, rpw = 64 / lpr, lir = lane % lpr, rsub = lane / lpr;
  const int ppl = IP ? IP / LPR_C : (I / piece_w(FMT)) / lpr;
  const int d = wave * rpw + rsub;  // this lane group's row-dot: unit d / R, row n0 + d % R
  const int u = d / R, n = n0 + d % R;
  const bool active = u < nu && n < H;
  // idle lane groups load a valid row too (results unused): no divergent
  // branch among the loads
  const int uc = min(u, nu - 1), nc = min(n, H - 1);
  const bool sh = uc == k;
  const MatDev& D = sh ? a.sdown : a.down;
  const int e = sh ? 0 : s_e[uc];
  // The h rows (unit t < k: routed row t; unit k: the shared row) go to LDS
  // piece-transposed.  Their loads are issued before the weight loads, so the
  // LDS stores wait for them alone.
  uint16_t* xs = (uint16_t*)smem;                                  // nu rows of I
  float* xsum = (float*)(smem + (size_t)nu * I * sizeof(uint16_t));  // INT4 piece sums
  const int ppt = I / 32, total = nu * ppt;
  auto h_piece = [&](int p) {
    const int t = p / ppt;
    return load_piece64((t < k ? a.h_routed + (size_t)t * I : a.h_shared) + 32 * (p - t * ppt));
  };
  Piece64 hv0, hv1;
  const int hp0 = tid, hp1 = tid + kT1Threads;
  if (hp0 < total) hv0 = h_piece(hp0);
  if (hp1 < total) hv1 = h_piece(hp1);
  RawPiece rd[kMaxPcD];
  {
    const uint8_t* rc = row_codes<FMT>(D, e, nc);
    const uint8_t* rs = row_scales<FMT>(D, e, nc);
    const uint8_t* rz = row_zeros<FMT>(D, e, nc);
#pragma unroll
    for (int q = 0; q < kMaxPcD; ++q)
      if (q < ppl) rd[q] = load_piece<FMT>(rc, rs, rz, lir + q * lpr);
  }
  auto h_store = [&](int p, const Piece64& v) {
    const int t = p / ppt, c = p - t * ppt;
    store_piece<FMT>((uint4*)(xs + (size_t)t * I) + c, ppt, xsum + p, v);
  };
  if (hp0 < total) h_store(hp0, hv0);
  if (hp1 < total) h_store(hp1, hv1);
  for (int p = tid + 2 * kT1Threads; p < total; p += kT1Threads) h_store(p, h_piece(p));
  __syncthreads();
  float acc[1] = {0.f};
#pragma unroll
  for (int q = 0; q < kMaxPcD; ++q)
    if (q < ppl) piece_dot<FMT, 1>(rd[q], lir + q * lpr, xs + (size_t)uc * I, I, xsum + uc * (I / 32), I / 32, 1, acc);
  acc[0] = IP ? group_sum_last<LPR_C>(acc[0]) : group_sum_last_dyn(acc[0], lpr);
  if (active && lir == lpr - 1) s_o[d] = acc[0] * tensor_scale<FMT>(D, e);
  __syncthreads();
  if (tid < R && n0 + tid < H) {
    const int c = n0 + tid;
    // every LDS read issued before the first use (a chain of dependent
    // reads would cost one LDS round trip per choice)
    float ow[kMaxUnitsT1 - 1], oo[kMaxUnitsT1 - 1];
#pragma unroll
    for (int j = 0; j < kMaxUnitsT1 - 1; ++j) {
      ow[j] = s_w[j];
      oo[j] = s_o[s_pp[j] * R + tid];
    }
    const float os = has_shared ? s_o[k * R + tid] : 0.f;
    float acc2 = 0.f;
#pragma unroll
    for (int j = 0; j < kMaxUnitsT1 - 1; ++j)
      if (j < k) acc2 = fmaf(ow[j], oo[j], acc2);
    if (has_shared) acc2 += os;
    if (a.residual) acc2 += bf16_to_f32(a.residual[c]);
    a.y[c] = (uint16_t)f32_to_bf16_rne(acc2);
  }
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
                       [sp, k](int r) { return sp ? sp[r] / k : r; }, g.h, g.I, g.lpr_h, smem);
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
  d.zeros = m.fmt == kFmtInt4Sb ? (const uint8_t*)m.biases : m.zeros;
  d.ts = m.tensor_scale;
  d.rows = m.rows;
  d.cols = m.cols;
  return d;
}

// Tokens staged per block (and per shared-expert batch).  Measured: 2 rather
// than 4 tokens up to 16 tokens (T=4 39.1 -> 36.8 us, T=16 75.0 -> 74.2 us,
// the batch-8 chain -2%; INT4 T=4/16 -6%/-2.5%), 4 at 64 tokens (2: 175 -> 183 us).
static int layer_nt(int T) { return T == 1 ? 1 : T <= 16 ? 2 : 4; }

static size_t stage_bytes(int NT, int K) { return (size_t)NT * K * 2 + (size_t)NT * (K / 32) * 4; }

// Dynamic LDS of the three decode launches; 0 when the shape is outside the
// decode path (more than 64 tokens, E > 1024, H > 4096, or > 64 KB).
struct DecodeLds {
  size_t route, gateup, down;
};

// Tokens per router batch.  Up to kRouteOneT tokens each token is a batch of its own: the
// batches' last blocks then rank their tokens in parallel, each with all four waves
// (measured against batches of 4: 4 tokens 33.5 -> 32.6 us, the 8-token 47-layer chain
// 2294 -> 2238 us; the router weights are read once per token batch, from the caches).
constexpr int kRouteOneT = 8;
static int router_tokens(int T) { return T <= kRouteOneT ? 1 : std::min(kRouteT, T); }

static size_t align16(size_t v) { return (v + 15) & ~(size_t)15; }

static DecodeLds decode_lds(int T, int H, int I, int Is, int E, int k) {
  DecodeLds d{0, 0, 0};
  if (T < 1 || T > 64 || E > 1024 || H > 4096) return d;
  const int NT = layer_nt(T);
  const size_t tables =
      (size_t)T * k * 8 + (size_t)kRouteT * E * 4 + 8 + (size_t)E * 8 + (size_t)(E + 1) * 4 + 17 * 4 + 64 * 4 + 16 + kRankScratch * 8;
  const size_t route = std::max((size_t)router_tokens(T) * H * 2, std::max(tables, stage_bytes(NT, H)));
  const size_t gateup = stage_bytes(NT, H);
  const size_t down = align16(stage_bytes(NT, std::max(I, Is))) + (size_t)T * k * 8;
  if (std::max(route, std::max(gateup, down)) > 64 * 1024) return d;
  return DecodeLds{route, gateup, down};
}

size_t layer_decode_lds(int T, int H, int I, int Is, int E, int k) {
  const DecodeLds d = decode_lds(T, H, I, Is, E, k);
  return std::max(d.route, std::max(d.gateup, d.down));
}

int layer_decode_sync_words(int H) { return kTicketSlice + 16 * ((H + kRDMin - 1) / kRDMin); }

size_t layer_decode_rec_ints(int T, int E, int k) { return (size_t)std::min(E, T * k) * kRec; }

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
  const int pw = piece_w(w->gate.fmt);
  g.lpr_h = lanes_for(H / pw, kLprTokens);
  g.lpr_i = lanes_for(I / pw, kLprDownTokens);
  constexpr int NT = 8;
  const size_t lds = std::max((size_t)NT * H * 2 + (size_t)NT * (H / 32) * 4,
                              (size_t)NT * I * 2 + (size_t)NT * (I / 32) * 4);
  if (w->gate.fmt == kFmtNvfp4) {
    MOE_LAUNCH((k_grouped_gateup<kFmtNvfp4, NT>), dim3(max_active * g.slices_r), dim3(256), lds, s, g);
    MOE_LAUNCH((k_grouped_down<kFmtNvfp4, NT>), dim3(max_active * g.slices_d), dim3(256), lds, s, g);
  } else if (w->gate.fmt == kFmtInt4Sb) {
    MOE_LAUNCH((k_grouped_gateup<kFmtInt4Sb, NT>), dim3(max_active * g.slices_r), dim3(256), lds, s, g);
    MOE_LAUNCH((k_grouped_down<kFmtInt4Sb, NT>), dim3(max_active * g.slices_d), dim3(256), lds, s, g);
  } else if (w->gate.fmt == kFmtBf16) {
    MOE_LAUNCH((k_grouped_gateup<kFmtBf16, NT>), dim3(max_active * g.slices_r), dim3(256), lds, s, g);
    MOE_LAUNCH((k_grouped_down<kFmtBf16, NT>), dim3(max_active * g.slices_d), dim3(256), lds, s, g);
  } else {
    MOE_LAUNCH((k_grouped_gateup<kFmtInt4, NT>), dim3(max_active * g.slices_r), dim3(256), lds, s, g);
    MOE_LAUNCH((k_grouped_down<kFmtInt4, NT>), dim3(max_active * g.slices_d), dim3(256), lds, s, g);
  }
  return hipGetLastError();
}

// Rows per block of the single-token down launch, or 0 where the general
// launch 3 is used: the shared expert (if any) must have the routed inter
// size (its h row shares the staging layout), every unit's row-dots must fit
// one pass of the block's lane groups, and a lane's pieces its registers.
static int down_t1_rows(int T, int I, int Is, int k, bool shared, int pw) {
  if (T != 1 || (shared && Is != I) || k > 8) return 0;
  const int lpr = lanes_for(I / pw, 64);
  if ((I / pw) / lpr > kMaxPcD) return 0;
  const int units = k + (shared ? 1 : 0);
  const int rows = (kT1Threads / lpr) / units;
  if (rows < 1 || (size_t)units * I * 2 + (size_t)units * (I / 32) * 4 > 64 * 1024) return 0;
  return rows;
}

template <int FMT, int NT, int GP, int IP>
static hipError_t launch_all(const LayerArgs& a, const DecodeLds& lds, hipStream_t s) {
  const int nsh = a.ss_r * a.nsb;
  MOE_LAUNCH((k_layer_route_shared<FMT, NT, GP, IP>), dim3(a.nR + (a.shared_in_gateup ? 0 : nsh)), dim3(256),
             lds.route, s, a);
  MOE_LAUNCH((k_layer_gateup<FMT, NT, GP, IP>), dim3((a.shared_in_gateup ? nsh : 0) + a.max_active * a.slices_r),
             dim3(256), lds.gateup, s, a);
  if (NT == 1 && a.rows_t1 > 0) {
    const int units = a.k + (a.nsb > 0 ? 1 : 0);
    const size_t l1 = (size_t)units * a.I * 2 + (size_t)units * (a.I / 32) * 4;
    MOE_LAUNCH((k_layer_down_t1<FMT, IP>), dim3((a.H + a.rows_t1 - 1) / a.rows_t1), dim3(kT1Threads), l1, s, a);
    return hipSuccess;
  }
  const int groups = down_loops(FMT, NT, IP) ? a.down_groups : a.max_active + a.nsb;
  MOE_LAUNCH((k_layer_down_combine<FMT, NT, GP, IP>), dim3(groups * a.slices_d), dim3(256), lds.down, s, a);
  if (!a.sep_combine) return hipSuccess;
  return launch_combine(a.o_routed, a.pair_pos, a.w, a.nsb > 0 ? a.o_shared : nullptr, a.residual, a.T, a.k, a.H,
                        a.y, nullptr, s);
}

// The Flint shape (hidden 2048, inter 768, the shared expert as wide as the
// routed ones) runs kernels compiled for it; every other shape the same
// kernels with its runtime shape.  Measured (NVFP4, 1/4/16/64 tokens):
// 21.9/38.8/78.3/190 -> 20.4/34.6/68.1/148 us.  The INT4 forms fit their
// register bounds compiled for the Flint shape since their nibble unpack is
// an asm statement (int4x2_to_bf16_off128).
template <int FMT, int NT>
static hipError_t launch_shape(const LayerArgs& a, const DecodeLds& lds, hipStream_t s) {
  if (a.H == 2048 && a.I == 768 && (a.Is == 0 || a.Is == 768) && FMT != kFmtBf16)
    return launch_all<FMT, NT, 64, 24>(a, lds, s);
  return launch_all<FMT, NT, 0, 0>(a, lds, s);
}

hipError_t launch_layer_decode(const moe_layer_weights* L, const uint16_t* x, const uint16_t* residual, int T,
                               uint16_t* y, const LayerDecodeBufs& b, int32_t* ids_out, float* w_out, hipStream_t s,
                               const uint16_t* norm_r, float eps) {
  LayerArgs a;
  a.norm_r = norm_r;
  a.x_w = const_cast<uint16_t*>(x);
  a.eps = eps;
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
  a.sync = b.sync;
  a.logits = b.logits;
  a.ids = b.ids;
  a.w = b.w;
  a.pair_pos = b.pair_pos;
  a.n_active = b.n_active;
  a.rec = b.rec;
  a.h_routed = b.h_routed;
  a.h_shared = b.h_shared;
  a.o_routed = b.o_routed;
  a.o_shared = b.o_shared;
  a.ids_out = ids_out;
  a.w_out = w_out;
  const int NT = layer_nt(T);
  a.max_active = std::min(a.E, T * a.k);
  a.rt = router_tokens(T);
  a.nRe = (a.E + 3) / 4;
  a.nR = a.nRe * ((T + a.rt - 1) / a.rt);
  a.nsb = L->shared ? (T + NT - 1) / NT : 0;
  // a single token has little work per block: smaller slices spread it over more CUs
  const bool bf = L->experts.gate.fmt == kFmtBf16;
  // bf16 weights: 64 lanes per gate/up row (4 pieces of 8 weights per lane at
  // hidden 2048) and 4 rows per block, 32 down rows per block, so a block's
  // pieces stay in registers
  a.rg = (T == 1 || bf) ? 4 : kRG;
  a.rd = (T == 1 || bf) ? kRDMin : kRD;
  a.ss_r = L->shared ? (a.Is + a.rg - 1) / a.rg : 0;
  a.slices_r = (a.I + a.rg - 1) / a.rg;
  a.slices_d = (a.H + a.rd - 1) / a.rd;
  const int pw = bf ? 8 : 32;
  a.lpr_h = lanes_for(a.H / pw, (NT == 1 || bf) ? 64 : kLprTokens);
  a.lpr_i = lanes_for(a.I / pw, NT == 1 ? 64 : bf ? 32 : kLprDownTokens);
  a.lpr_is = a.Is ? lanes_for(a.Is / pw, NT == 1 ? 64 : bf ? 32 : kLprDownTokens) : 64;
  a.down_stage_bytes = (int)align16(stage_bytes(NT, std::max(a.I, a.Is)));
  a.rows_t1 = down_t1_rows(T, a.I, a.Is, a.k, L->shared != nullptr, pw);
  a.sync_slices = (a.H + kRDMin - 1) / kRDMin;
  // many tokens: the last down block of each slice would combine T x 64 outputs at the
  // launch's end (a serial tail); a combine launch of its own spreads that over the chip
  a.sep_combine = T > kSepCombineT;
  {
    // the looping down kernel: one unit per block while the units' slices fit kDownBlocks,
    // above that each block takes several units of its slice (their record heads in one
    // round trip, one slice ticket per block)
    const int max_units = a.max_active + a.nsb;
    const int fit = std::max(1, kDownBlocks / a.slices_d);
    a.down_groups = std::min(max_units, std::max(fit, (max_units + kMaxDownUnits - 1) / kMaxDownUnits));
  }
  // NVFP4, few tokens: the first launch's critical path is the router and its routing tail;
  // the shared expert's gate/up then runs beside the routed gate/up instead (measured, same
  // box: 1 token 19.7 -> 19.3 us, 4 tokens 33.4 -> 33.0 us, the 8-token chain -0.8%; at 16
  // and 64 tokens +1-2%; the INT4 forms and BF16 lose 5% at one token and 2-3% at 4 and 16,
  // their gate/up launch being the busier one)
  a.shared_in_gateup = fmt_shared_early(L->experts.gate.fmt) && T <= kSharedInGateupT;
  const DecodeLds lds = decode_lds(T, a.H, a.I, a.Is, a.E, a.k);
  const int fmt = L->experts.gate.fmt;
  auto by_fmt = [&](auto nt) -> hipError_t {
    constexpr int N = decltype(nt)::value;
    if (fmt == kFmtNvfp4) return launch_shape<kFmtNvfp4, N>(a, lds, s);
    if (fmt == kFmtInt4Sb) return launch_shape<kFmtInt4Sb, N>(a, lds, s);
    if (fmt == kFmtBf16) return launch_shape<kFmtBf16, N>(a, lds, s);
    return launch_shape<kFmtInt4, N>(a, lds, s);
  };
  if (NT == 1) return by_fmt(std::integral_constant<int, 1>{});
  if (NT == 2) return by_fmt(std::integral_constant<int, 2>{});
  return by_fmt(std::integral_constant<int, 4>{});
}

}  // namespace moe
