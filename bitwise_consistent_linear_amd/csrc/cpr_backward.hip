// HIP kernels for the backward of CPR Gated DeltaNet (the trainer's gradients) on gfx950.
//
// Per row i of (n, h), dL/ds (sh) runs backward over the tokens:
//   sh += g q;  dh = sh . k;  dv_i = b dh;  xh = sh - dv_i k;  [shares];  sh = a xh
// (row_bwd_* in cpr_row.hpp, in the contract's binary32 order). The shares of dq, dk, da
// and db need the forward states, the recurrence of sh does not. So:
//   1. plan:    one workgroup maps chunk slots to (sequence, chunk) and computes each
//               sequence's first chunk-state index;
//   2. state:   a reverse scan of sh per row (as parallel as the forward scan), writing dv,
//               dS0 and sh at every chunk boundary;
//   3. chunk:   for every (chunk, value head, block of 32 rows) in parallel: the forward
//               states recomputed from the trainer's chunk state (checkpoints every 8 tokens
//               in registers, each token's v_i - u in LDS), sh re-run from the boundary value the state pass stored (the
//               same operations, so the same bits), and every token's shares summed over
//               the block's rows: pairwise in natural row order, within the wave by row
//               swaps, then across the 8 waves through LDS; one partial per (token, head,
//               row block);
//   4. combine: the pairwise tree continued over the row blocks, then the value heads of a
//               q/k group left to right.
// A pair of the row tree whose second half holds no row (d_v not a power of two) passes its
// first half through unchanged, at every level; that is what makes the hierarchical sums
// equal the contract's single tree over the d_v rows.

#include <algorithm>
#include <mutex>
#include <type_traits>
#include <utility>

#include "cpr_io.hpp"
#include "cpr_row.hpp"
#include "internal.h"

namespace gdn {
namespace {

using namespace io;

constexpr int kThreads = 256;
constexpr int kStateStage = 16;                   // tokens staged at a time by the state pass
constexpr int kSub = 8;                           // tokens per recomputed sub-block
constexpr int kMaxSub = 8;                        // sub-blocks per segment
constexpr int kSeg = kSub * kMaxSub;              // tokens per segment: a chunk of C > 64 is
                                                  // processed as segments of 64, last first
constexpr int kChunkLanes = 16;                   // lanes per row in the chunk kernel
constexpr int kChunkWaves = 8;                    // waves per chunk-kernel workgroup
constexpr int kChunkThreads = 64 * kChunkWaves;
constexpr int kChunkRows = kChunkThreads / kChunkLanes;

// f(std::integral_constant<int, i>) for i = 0 .. N-1 (REVERSE: N-1 .. 0), each with its own
// compile-time index, so register arrays indexed by i stay in registers.
template <bool REVERSE, int N, typename F, int... I>
__device__ __forceinline__ void static_for_impl(F &&f, std::integer_sequence<int, I...>) {
  (f(std::integral_constant<int, REVERSE ? N - 1 - I : I>{}), ...);
}
template <int N, bool REVERSE = false, typename F>
__device__ __forceinline__ void static_for(F &&f) {
  static_for_impl<REVERSE, N>(f, std::make_integer_sequence<int, N>{});
}

// --------------------------------------------------------------------------------- plan

__global__ __launch_bounds__(kThreads) void cpr_bwd_plan_kernel(const BwdArgs p) {
  chunk_plan(p.cu_seqlens, p.num_seqs, p.total_tokens, p.chunk, p.total_chunks, p.slots_max,
             p.plan, p.plan_cbase);
}

// ---------------------------------------------------------------------------- state pass

template <int D, int L, bool BF16>
__global__ __launch_bounds__(kThreads) void cpr_bwd_state_kernel(const BwdArgs p) {
  constexpr int ROWS = kThreads / L;
  constexpr int M = D / L;
  constexpr int TS = kStateStage;
  constexpr int GROUPS = D / 4;
  constexpr int KQ_ITEMS = TS * GROUPS, V_ITEMS = TS * ROWS;
  constexpr int KQ_PER = (KQ_ITEMS + kThreads - 1) / kThreads;
  constexpr int V_PER = (V_ITEMS + kThreads - 1) / kThreads;
  using raw_t = typename Raw4<BF16>::type;

  __shared__ __align__(16) float sk[2][TS * D];
  __shared__ __align__(16) float sq[2][TS * D];
  __shared__ float sg[2][V_ITEMS];   // dL/do of the block's rows
  __shared__ float sdv[2][V_ITEMS];  // dv of the block's rows, stored coalesced after a stage
  __shared__ float sa[2][TS], sb[2][TS];
  __shared__ int s_len[kMaxRankedSeqs];
  __shared__ int s_pick;

  const int tid = threadIdx.x, row = tid / L, lane = tid % L;
  const int Hv = p.num_v_heads, Hk = p.num_qk_heads, dv = p.d_v;
  const int rblocks = (dv + ROWS - 1) / ROWS;
  int pair, rblock;
  block_work(blockIdx.x, p.num_seqs * Hv, rblocks, Hv / Hk, pair, rblock);
  const int rank = pair / Hv;
  const int h = pair % Hv;
  const int r0 = rblock * ROWS;
  const int64_t T = p.total_tokens;
  const int n = ranked_sequence(p.cu_seqlens, p.num_seqs, T, rank, s_len, &s_pick);
  int64_t bos, eos;
  seq_range(p.cu_seqlens, n, T, bos, eos);
  const int64_t Tn = eos - bos;
  const int64_t cbase = p.plan_cbase[n];
  const int hk = h / (Hv / Hk);
  const int i = r0 + row;
  const bool valid = i < dv;
  const int64_t row_off = (((int64_t)n * Hv + h) * dv + i) * D + lane * M;
  const int64_t vstride = (int64_t)Hv * dv;

  float sh[M];
  if (p.d_final_state && valid) {
    load_row<M>(p.d_final_state + row_off, sh);
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) sh[e] = 0.0f;
  }
#pragma unroll
  for (int e = 0; e < M; ++e) asm volatile("" ::"v"(sh[e]));

  raw_t rk[KQ_PER], rq[KQ_PER];
  float rg[V_PER], ra, rb;
  auto fetch = [&](int64_t t0) {
    const int64_t last = Tn - 1;
#pragma unroll
    for (int j = 0; j < KQ_PER; ++j) {
      const int g = (tid + j * kThreads) % KQ_ITEMS;
      const int64_t t = t0 + g / GROUPS < last ? t0 + g / GROUPS : last;
      const int64_t src = ((bos + t) * Hk + hk) * D + 4 * (g % GROUPS);
      rk[j] = load_raw4<BF16>(p.k, src);
      rq[j] = load_raw4<BF16>(p.q, src);
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int e = (tid + j * kThreads) % V_ITEMS;
      const int64_t t = t0 + e / ROWS < last ? t0 + e / ROWS : last;
      const int r = r0 + e % ROWS < dv ? r0 + e % ROWS : dv - 1;
      rg[j] = p.d_o[(bos + t) * vstride + (int64_t)h * dv + r];
    }
    const int64_t t = t0 + tid % TS < last ? t0 + tid % TS : last;
    ra = p.a[(bos + t) * Hv + h];
    rb = p.b[(bos + t) * Hv + h];
  };
  auto deposit = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KQ_PER; ++j) {
      const int g = tid + j * kThreads;
      if (KQ_ITEMS % kThreads == 0 || g < KQ_ITEMS) {
        const int off = (g / GROUPS) * D + stage_slot<D, L>(g % GROUPS);
        *reinterpret_cast<float4 *>(&sk[buf][off]) = widen4<BF16>(rk[j]);
        *reinterpret_cast<float4 *>(&sq[buf][off]) = widen4<BF16>(rq[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int e = tid + j * kThreads;
      if (V_ITEMS % kThreads == 0 || e < V_ITEMS) sg[buf][e] = rg[j];
    }
    if (tid < TS) {
      sa[buf][tid] = ra;
      sb[buf][tid] = rb;
    }
  };
  auto write_dv = [&](int64_t t0, int nt, int buf) {
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int e = tid + j * kThreads;
      const int tt = e / ROWS, r = e % ROWS;
      if ((V_ITEMS % kThreads == 0 || e < V_ITEMS) && tt < nt && r0 + r < dv)
        p.dv[(bos + t0 + tt) * vstride + (int64_t)h * dv + r0 + r] = sdv[buf][e];
    }
  };
  auto run_token = [&](int buf, int tt) {
    float kr[M], qr[M], xh[M], dh;
    lds_slice<D, L>(&sk[buf][tt * D], lane, kr);
    lds_slice<D, L>(&sq[buf][tt * D], lane, qr);
    row_bwd_absorb<D, L>(sh, sg[buf][tt * ROWS + row], qr);
    sdv[buf][tt * ROWS + row] = row_bwd_delta<D, L>(sh, kr, sb[buf][tt], xh, dh);
    row_bwd_decay<D, L>(sh, sa[buf][tt], xh);
  };

  const int chunk_shift = __builtin_ctz((unsigned)p.chunk);
  const int64_t nstages = (Tn + TS - 1) / TS;
  if (Tn > 0) {
    fetch((nstages - 1) * TS);
    deposit(0);
  }
  __syncthreads();
  for (int64_t idx = 0; idx < nstages; ++idx) {
    const int64_t st = nstages - 1 - idx;
    const int buf = (int)(idx & 1);
    const int64_t t0 = st * TS;
    const int nt = (int)(Tn - t0 < TS ? Tn - t0 : TS);
    const bool more = st > 0;
    if (more) fetch(t0 - TS);
    if (nt == TS) {
      // dL/d(state after a full chunk's last token), from everything after it
      const int64_t done = t0 + TS;
      if ((done & (p.chunk - 1)) == 0) {
        const int64_t c = cbase + (done >> chunk_shift) - 1;
        if (valid && c < p.total_chunks)
          store_row<M>(p.dsh_bnd + ((c * Hv + h) * dv + i) * D + lane * M, sh);
      }
#pragma unroll
      for (int tt = TS - 1; tt >= 0; --tt) run_token(buf, tt);
    } else {
#pragma unroll 1
      for (int tt = nt - 1; tt >= 0; --tt) run_token(buf, tt);
    }
    if (more) deposit(buf ^ 1);
    __syncthreads();
    write_dv(t0, nt, buf);
  }
  if (valid) store_row<M>(p.d_initial_state + row_off, sh);
}

// ---------------------------------------------------------------------------- chunk pass

// Lane swaps between the 16-lane rows of a wave (gfx950): swap16 exchanges the odd rows of
// `hi` with the even rows of `lo`; swap32 exchanges the upper 32 lanes of `hi` with the lower
// 32 lanes of `lo`. (a, b) are the two registers afterwards.
__device__ __forceinline__ void swap16(float hi, float lo, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(hi), __float_as_uint(lo),
                                                  false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float hi, float lo, float &a, float &b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(hi), __float_as_uint(lo),
                                                  false, false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}

// One token's shares summed over the four rows of a wave (row r in lanes 16r .. 16r+15) in
// the row tree's order, (r0 + r1) + (r2 + r3), scattered over the lanes. Each level is one
// swap and one add: after a swap, register a holds the pair's first row and b its second,
// so a + b is the pair's sum on both rows' lanes, and a alone is the pass-through value.
// On return, lane (r, c) holds the 4-row sums of z[0 .. H-1] = elements
// (r odd ? dq : dk)[c M + (r < 2 ? H : 0) + 0 .. H-1] (H = M / 2; for M = 1 every lane holds
// element c, and lanes of rows 0 and 1 report it), and y = (r odd ? da : db).
// c1: this lane's level-one pair is combined; c2: the two halves are combined. FULL: all
// four rows hold rows below d_v (no pass-through).
template <int M, bool FULL>
__device__ __forceinline__ void rows4_sum(const float (&pq)[M], const float (&pk)[M], float pa,
                                          float pb, bool c1, bool c2,
                                          float (&z)[M >= 2 ? M / 2 : 1], float &y) {
  float w[M], a, b;
#pragma unroll
  for (int j = 0; j < M; ++j) {
    swap16(pk[j], pq[j], a, b);
    w[j] = (FULL || c1) ? a + b : a;
  }
  if constexpr (M >= 2) {
    constexpr int H = M / 2;
#pragma unroll
    for (int j = 0; j < H; ++j) {
      swap32(w[H + j], w[j], a, b);
      z[j] = (FULL || c2) ? a + b : a;
    }
  } else {
    swap32(w[0], w[0], a, b);
    z[0] = (FULL || c2) ? a + b : a;
  }
  swap16(pb, pa, a, b);
  const float x = (FULL || c1) ? a + b : a;
  swap32(x, x, a, b);
  y = (FULL || c2) ? a + b : a;
}

// The chunk pass, in one of two schedules with the same arithmetic (so the same bits):
//   SEQ = false: one workgroup per (chunk slot, value head, row block); dL/ds at the chunk's
//                end comes from the state pass (or dL/dS_final for a sequence's last chunk);
//   SEQ = true:  one workgroup per (sequence, value head, row block), sweeping the
//                sequence's chunks from last to first and carrying dL/ds in registers; it
//                writes dv and dS0 itself, so the state pass does not run.
// Checkpoints and a sub-block of recomputed states live in registers: allow up to 256
// VGPRs (two waves per SIMD) rather than spill.
// WHOLE: every sub-block it takes is whole (8 tokens) and d_v is a multiple of the four rows
// of a wave, so no token is skipped and no row of a wave that counts passes through: the
// token loops (the forward sweep's included) run a fixed 8 tokens with no per-token branch,
// every lane of a row stores the row's values to LDS (the same value to the same place),
// and the scheduler can overlap one token's reduction trees with its neighbours'
// arithmetic. Where d_v allows and C <= 64 the host sets p.whole and launches the general
// kernel, then the WHOLE one. Only a sequence's last chunk can hold a partial sub-block (C
// is a multiple of 8), so the general kernel then takes just those chunks of ragged
// sequences (length not a multiple of 8): on the sequence schedule it runs that chunk and
// leaves dL/ds at its start in the boundary buffer (or dS0 for a one-chunk sequence), and
// the WHOLE kernel sweeps the chunks below it from there. The same operations either way.
template <int D, bool BF16, bool SEQ, bool LONG, bool WHOLE>
__global__ __launch_bounds__(kChunkThreads) __attribute__((amdgpu_waves_per_eu(1, 2)))
void cpr_bwd_chunk_kernel(const BwdArgs p) {
  static_assert(!(WHOLE && LONG), "chunks longer than a segment take the general loops");
  constexpr int kThreads = kChunkThreads;
  constexpr int L = kChunkLanes, ROWS = kChunkRows, M = D / L, SB = kSub;
  constexpr int WAVES = kChunkWaves, RPW = 64 / L;  // rows per wave
  constexpr int PWP = 2 * D + 4;  // shares of a token (dq, dk, da, db) padded to whole float4:
                                  // their LDS row and their row in the partial sums
  constexpr int H = M >= 2 ? M / 2 : 1;               // elements each lane holds after rows4_sum
  constexpr int GROUPS = D / 4;
  constexpr int KQ_ITEMS = SB * GROUPS, V_ITEMS = SB * ROWS;
  constexpr int KQ_PER = (KQ_ITEMS + kThreads - 1) / kThreads;
  static_assert(V_ITEMS <= kThreads && SB <= kThreads, "one v/g and a/b item per thread");
  using raw_t = typename Raw4<BF16>::type;
  __shared__ __align__(16) float sk[2][SB * D];
  __shared__ __align__(16) float sq[2][SB * D];
  __shared__ float sv[2][V_ITEMS], sg[2][V_ITEMS], sa[2][SB], sb[2][SB];
  // wave sums of a sub-block's tokens, two buffers: sub-block sbi uses swave[sbi & 1], so the
  // next sub-block's tokens can be summed while other waves still read these (one barrier
  // per sub-block). The sequence ranking's lengths, used once before the first chunk, share
  // the second buffer.
  __shared__ __align__(16) float swave[2][SB][WAVES][PWP];
  static_assert(kMaxRankedSeqs <= SB * WAVES * PWP, "ranking lengths fit one wave-sum buffer");
  int *const s_len = reinterpret_cast<int *>(&swave[1][0][0][0]);
  // v_i - u of every token of the chunk; once the reverse pass has rebuilt a sub-block's
  // states from its entries, the sequence schedule keeps that sub-block's dv_i there
  __shared__ float sdif[kMaxSub * SB][ROWS];
  __shared__ int s_pick;

  const int Hv = p.num_v_heads, Hk = p.num_qk_heads, dv = p.d_v, RB = p.row_blocks;
  int pair, rblock, n, h, c_hi, c_lo;
  int64_t bos, eos;
  bool from_bnd = !SEQ;  // dL/ds at the end of chunk c_hi comes from the boundary buffer
  if constexpr (SEQ) {
    block_work(blockIdx.x, p.num_seqs * Hv, RB, 1, pair, rblock);
    h = pair % Hv;
    n = ranked_sequence(p.cu_seqlens, p.num_seqs, p.total_tokens, pair / Hv, s_len, &s_pick);
    seq_range(p.cu_seqlens, n, p.total_tokens, bos, eos);
    c_hi = (int)((eos - bos + p.chunk - 1) / p.chunk) - 1;
    c_lo = 0;
    if (p.whole && (eos - bos) % SB != 0) {  // uniform: a ragged sequence
      if constexpr (WHOLE) {
        if (c_hi == 0) return;  // its only chunk is the general kernel's
        c_hi -= 1;              // from the boundary the general kernel left
        from_bnd = true;
      } else {
        c_lo = c_hi;  // its last chunk only
      }
    } else if (!WHOLE && p.whole) {
      return;  // uniform: the WHOLE kernel has this sequence
    }
  } else {
    block_work(blockIdx.x, p.slots_max * Hv, RB, 1, pair, rblock);
    const int slot = pair / Hv;
    h = pair % Hv;
    if (slot >= p.plan[0]) return;  // uniform: this workgroup has no chunk
    n = p.plan[kPlanHeader + 2 * slot];
    c_hi = c_lo = p.plan[kPlanHeader + 2 * slot + 1];
    seq_range(p.cu_seqlens, n, p.total_tokens, bos, eos);
    if ((int64_t)c_hi * p.chunk >= eos - bos) return;  // uniform
    if (p.whole) {  // uniform: a chunk with a partial sub-block is the general kernel's
      const int64_t clen = eos - bos - (int64_t)c_hi * p.chunk;
      const bool ragged = (clen < p.chunk ? clen : p.chunk) % SB != 0;
      if (ragged == WHOLE) return;
    }
  }
  const int64_t Tn = eos - bos;
  const int64_t cbase = p.plan_cbase[n];
  const int hk = h / (Hv / Hk);
  const int r0 = rblock * ROWS;
  const int64_t vstride = (int64_t)Hv * dv;
  auto row_offset = [&](int i, int lane) { return (((int64_t)n * Hv + h) * dv + i) * D + lane * M; };

  // dL/ds after the last chunk processed here, carried from chunk to chunk
  float sh[M];
#pragma unroll
  for (int e = 0; e < M; ++e) sh[e] = 0.0f;
  {
    const int lane = threadIdx.x % L, i = r0 + (int)threadIdx.x / L;
    if (i < dv) {
      if (from_bnd && ((int64_t)c_hi + 1) * p.chunk <= Tn) {
        if (cbase + c_hi < p.total_chunks)
          load_row<M>(p.dsh_bnd + (((cbase + c_hi) * Hv + h) * dv + i) * D + lane * M, sh);
      } else if (p.d_final_state) {
        load_row<M>(p.d_final_state + row_offset(i, lane), sh);
      }
    }
  }

  raw_t rk[KQ_PER], rq[KQ_PER];
  uint32_t rv = 0;
  float rg = 0.0f, ra = 0.0f, rb = 0.0f;
  for (int c = c_hi; c >= c_lo; --c) {
   const int64_t cstart = (int64_t)c * p.chunk;
   const int clen = (int)(Tn - cstart < p.chunk ? Tn - cstart : p.chunk);
   const int nseg = LONG ? (clen + kSeg - 1) / kSeg : 1;  // LONG: chunks longer than kSeg
   for (int seg = nseg - 1; seg >= 0; --seg) {
    // Thread-derived values come from an opaque copy of the thread index, once per segment,
    // so that the addresses of the unrolled body are not held live across segments.
    int tid = threadIdx.x;
    asm volatile("" : "+v"(tid));
    const int row = tid / L, lane = tid % L;
    const int wave = tid / 64, wl = tid % 64, r4 = wl / L, c16 = wl % L;
    const int i = r0 + row;
    const bool valid = i < dv;
    const int wrow0 = r0 + wave * RPW;  // first row of this wave
    const bool full4 = wrow0 + RPW - 1 < dv;
    const bool c1 = r4 < 2 ? wrow0 + 1 < dv : wrow0 + 3 < dv, c2 = wrow0 + 2 < dv;
    // where this lane stores its row sums in swave[j][wave][.] (see rows4_sum)
    int zofs = (M >= 2) ? ((r4 & 1) ? 0 : D) + c16 * M + (r4 < 2 ? H : 0)
                        : ((r4 & 1) ? 0 : D) + c16;
    int yofs = 2 * D + ((r4 & 1) ? 0 : 1);
    asm volatile("" : "+v"(zofs), "+v"(yofs));  // kept in registers, not recomputed per token
    const bool zwrite = M >= 2 || r4 < 2, ywrite = c16 == 0 && r4 < 2;

    // the state at the chunk's start: the initial state or the trainer's chunk state
    float s[M];
#pragma unroll
    for (int e = 0; e < M; ++e) s[e] = 0.0f;
    if (valid) {
      if (c == 0) {
        if (p.initial_state) load_row<M>(p.initial_state + row_offset(i, lane), s);
      } else if (cbase + c - 1 < p.total_chunks) {
        load_row<M>(p.chunk_states + (((cbase + c - 1) * Hv + h) * dv + i) * D + lane * M, s);
      }
    }

    // Tokens [c0 + j0, c0 + j0 + nt) of the chunk: global memory -> registers (fetch), then
    // registers -> LDS buffer (deposit), so the loads of the next sub-block overlap the
    // arithmetic of this one. Items past nt repeat the last token and are never read.
    auto fetch = [&](int64_t c0, int j0, int nt) {
#pragma unroll
      for (int jj = 0; jj < KQ_PER; ++jj) {
        const int g = (tid + jj * kThreads) % KQ_ITEMS;
        const int tt = g / GROUPS < nt ? g / GROUPS : nt - 1;
        const int64_t src = ((bos + c0 + j0 + tt) * Hk + hk) * D + 4 * (g % GROUPS);
        rk[jj] = load_raw4<BF16>(p.k, src);
        rq[jj] = load_raw4<BF16>(p.q, src);
      }
      {
        const int e = tid % V_ITEMS;
        const int tt = e / ROWS < nt ? e / ROWS : nt - 1;
        const int r = r0 + e % ROWS < dv ? r0 + e % ROWS : dv - 1;
        const int64_t at = (bos + c0 + j0 + tt) * vstride + (int64_t)h * dv + r;
        rv = load_raw1<BF16>(p.v, at);
        rg = p.d_o[at];
      }
      const int tt = tid % SB < nt ? tid % SB : nt - 1;
      ra = p.a[(bos + c0 + j0 + tt) * Hv + h];
      rb = p.b[(bos + c0 + j0 + tt) * Hv + h];
    };
    auto deposit = [&](int buf) {
#pragma unroll
      for (int jj = 0; jj < KQ_PER; ++jj) {
        const int g = tid + jj * kThreads;
        if (KQ_ITEMS % kThreads == 0 || g < KQ_ITEMS) {
          const int off = (g / GROUPS) * D + stage_slot<D, L>(g % GROUPS);
          *reinterpret_cast<float4 *>(&sk[buf][off]) = widen4<BF16>(rk[jj]);
          *reinterpret_cast<float4 *>(&sq[buf][off]) = widen4<BF16>(rq[jj]);
        }
      }
      if (tid < V_ITEMS) {
        const bool ok = r0 + tid % ROWS < dv;
        sv[buf][tid] = ok ? widen1<BF16>(rv) : 0.0f;
        sg[buf][tid] = ok ? rg : 0.0f;
      }
      if (tid < SB) {
        sa[buf][tid] = ra;
        sb[buf][tid] = rb;
      }
    };

    // The state at this segment's start: the chunk's start state carried forward over the
    // segments before it, token by token in the forward order (the row update of the trainer,
    // so the same bits). One staged sub-block at a time, buffer 0, no overlap: this runs only
    // for chunks longer than a segment.
    if constexpr (LONG) {
     for (int j0 = 0; j0 < seg * kSeg; j0 += SB) {
      fetch(cstart, j0, SB);
      __syncthreads();  // buffer 0's previous readers are done
      deposit(0);
      __syncthreads();
      for (int j = 0; j < SB; ++j) {
        float kr[M], x[M];
        lds_slice<D, L>(&sk[0][j * D], lane, kr);
        row_decay<D, L>(s, sa[0][j], x);
        const float u = contract_dot<D, L>(x, kr);
        row_update<D, L>(s, row_delta(sb[0][j], sv[0][j * ROWS + row], u), kr, x);
      }
     }
     if (seg > 0) __syncthreads();  // the advance's readers of buffer 0 are done
    }

    const int64_t c0 = cstart + (int64_t)seg * kSeg;
    const int len = clen - seg * kSeg < kSeg ? clen - seg * kSeg : kSeg;
    const int nsb = (len + SB - 1) / SB;
    auto sub_len = [&](int sbi) { return len - sbi * SB < SB ? len - sbi * SB : SB; };
    fetch(c0, 0, sub_len(0));
    deposit(0);  // buffer 0's last reader (the previous chunk) finished before its barrier
    __syncthreads();

    // forward over the chunk, keeping the state at the start of every sub-block
    float ck[kMaxSub][M];
    static_for<kMaxSub>([&](auto sbi_c) {
      constexpr int sbi = decltype(sbi_c)::value, buf = sbi & 1;
      if (sbi < nsb) {
        const bool next = sbi + 1 < nsb;
        if (next) fetch(c0, (sbi + 1) * SB, sub_len(sbi + 1));
#pragma unroll
        for (int e = 0; e < M; ++e) ck[sbi][e] = s[e];
        const int nt = WHOLE ? SB : sub_len(sbi);
        for (int j = 0; j < nt; ++j) {
          float kr[M], x[M];
          lds_slice<D, L>(&sk[buf][j * D], lane, kr);
          row_decay<D, L>(s, sa[buf][j], x);
          const float u = contract_dot<D, L>(x, kr);
          const float dif = sv[buf][j * ROWS + row] - u;  // d = b (v_i - u), as row_delta
          if (WHOLE || lane == 0) sdif[sbi * SB + j][row] = dif;
          row_update<D, L>(s, sb[buf][j] * dif, kr, x);
        }
        if (next) deposit(buf ^ 1);  // its last reader finished before the previous barrier
        __syncthreads();
      }
    });

    // sub-blocks in reverse: recompute the states, run sh back, sum the shares over rows
    static_for<kMaxSub, true>([&](auto sbi_c) {
      constexpr int sbi = decltype(sbi_c)::value, buf = sbi & 1;
      if (sbi < nsb) {
        const int nt = WHOLE ? SB : sub_len(sbi);
        if (sbi > 0) fetch(c0, (sbi - 1) * SB, SB);
        float st[SB + 1][M], dif[SB], del[SB];
#pragma unroll
        for (int e = 0; e < M; ++e) st[0][e] = ck[sbi][e];
#pragma unroll
        for (int j = 0; j < SB; ++j) {
          if (WHOLE || j < nt) {  // the forward sweep left v_i - u of each token: no dot here
            float kr[M], x[M];
            lds_slice<D, L>(&sk[buf][j * D], lane, kr);
            row_decay<D, L>(st[j], sa[buf][j], x);
            dif[j] = sdif[sbi * SB + j][row];
            del[j] = sb[buf][j] * dif[j];
#pragma unroll
            for (int e = 0; e < M; ++e) st[j + 1][e] = st[j][e];
            row_update<D, L>(st[j + 1], del[j], kr, x);
          }
        }
#pragma unroll
        for (int j = SB - 1; j >= 0; --j) {
          if (WHOLE || j < nt) {
            float kr[M], qr[M], x[M], xh[M], pq[M], pk[M], dh;
            lds_slice<D, L>(&sk[buf][j * D], lane, kr);
            lds_slice<D, L>(&sq[buf][j * D], lane, qr);
            const float g = sg[buf][j * ROWS + row], a = sa[buf][j], b = sb[buf][j];
            row_bwd_absorb<D, L>(sh, g, qr);
#pragma unroll
            for (int e = 0; e < M; ++e) pq[e] = g * st[j + 1][e];
            const float dv_i = row_bwd_delta<D, L>(sh, kr, b, xh, dh);
            if constexpr (SEQ) {  // this row's entry was read by the rebuild above (this wave)
              if (WHOLE || lane == 0) sdif[sbi * SB + j][row] = dv_i;
            }
            const float pb = dh * dif[j];
            const float uh = -dv_i;
            row_decay<D, L>(st[j], a, x);
#pragma unroll
            for (int e = 0; e < M; ++e) {
              const float ds = del[j] * sh[e];
              pk[e] = __builtin_fmaf(uh, x[e], ds);
            }
            const float pa = contract_dot<D, L>(xh, st[j]);
            row_bwd_decay<D, L>(sh, a, xh);
            float z[H], y;
            if (WHOLE || full4)
              rows4_sum<M, true>(pq, pk, pa, pb, c1, c2, z, y);
            else
              rows4_sum<M, false>(pq, pk, pa, pb, c1, c2, z, y);
            float *dst = &swave[sbi & 1][j][wave][0];
            if constexpr (H == 4) {
              *reinterpret_cast<float4 *>(dst + zofs) = make_float4(z[0], z[1], z[2], z[3]);
            } else if constexpr (H == 2) {
              *reinterpret_cast<float2 *>(dst + zofs) = make_float2(z[0], z[1]);
            } else {
              if (zwrite) dst[zofs] = z[0];
            }
            if (ywrite) dst[yofs] = y;
          }
        }
        // the previous sub-block's inputs: buffer buf ^ 1 was last read by sub-block sbi + 1,
        // before the barrier that ended it; its readers come after the barrier below
        if (sbi > 0) deposit(buf ^ 1);
        __syncthreads();
        // across the waves (wave w holds rows r0 + 4w .. r0 + 4w + 3), pairwise, pass-through;
        // four consecutive shares per thread (one 16-byte read per wave, one 16-byte store).
        // The last group of a token holds da, db and two padding slots, whose sums nothing
        // reads.
        constexpr int G4 = PWP / 4;
        for (int e = tid; e < nt * G4; e += kThreads) {
          const int j = e / G4, f = 4 * (e % G4);
          float4 w[WAVES];
#pragma unroll
          for (int x = 0; x < WAVES; ++x)
            w[x] = *reinterpret_cast<const float4 *>(&swave[sbi & 1][j][x][f]);
#pragma unroll
          for (int st = 1; st < WAVES; st *= 2)
#pragma unroll
            for (int x = 0; x + st < WAVES; x += 2 * st)
              if (r0 + (x + st) * RPW < dv) {
                w[x].x = w[x].x + w[x + st].x;
                w[x].y = w[x].y + w[x + st].y;
                w[x].z = w[x].z + w[x + st].z;
                w[x].w = w[x].w + w[x + st].w;
              }
          const int64_t t = bos + c0 + sbi * SB + j;
          *reinterpret_cast<float4 *>(&p.partials[((t * Hv + h) * RB + rblock) * PWP + f]) = w[0];
        }
        if constexpr (SEQ) {
          for (int e = tid; e < nt * ROWS; e += kThreads) {
            const int j = e / ROWS, r = e % ROWS;
            if (r0 + r < dv)
              p.dv[(bos + c0 + sbi * SB + j) * vstride + (int64_t)h * dv + r0 + r] =
                  sdif[sbi * SB + j][r];
          }
        }
        // No barrier here: the next sub-block writes the other wave-sum buffer and its own
        // sdif rows, and reads the input buffer deposited before the barrier above.
      }
    });
   }  // segments
  }
  if constexpr (SEQ) {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));  // recomputed here rather than held across the chunk loop
    const int lane = t % L, i = r0 + t / L;
    if (i < dv) {
      if (!WHOLE && c_lo > 0) {  // a ragged sequence's last chunk: dL/ds at its start
        if (cbase + c_lo - 1 < p.total_chunks)
          store_row<M>(p.dsh_bnd + (((cbase + c_lo - 1) * Hv + h) * dv + i) * D + lane * M, sh);
      } else {
        store_row<M>(p.d_initial_state + row_offset(i, lane), sh);
      }
    }
  }
}

// -------------------------------------------------------------------------- combine pass

// Pairwise tree over the RB row-block sums (natural order, pass-through); RBMAX is the power
// of two at or above RB.
template <int RBMAX>
__device__ __forceinline__ float rb_tree(const float *base, int64_t stride, int RB) {
  constexpr int kMaxRB = RBMAX;
  float v[kMaxRB];
#pragma unroll
  for (int j = 0; j < kMaxRB; ++j) v[j] = j < RB ? base[j * stride] : 0.0f;
#pragma unroll
  for (int w = 1; w < kMaxRB; w *= 2)
#pragma unroll
    for (int j = 0; j + w < kMaxRB; j += 2 * w)
      if (j + w < RB) v[j] = v[j] + v[j + w];
  return v[0];
}

// One token per workgroup iteration (grid-stride over tokens): its Hk * d_k elements of dq
// and dk and Hv pairs (da, db), indexed in 32 bits (d_k a power of two).
template <int RBMAX>
__global__ __launch_bounds__(kThreads) void cpr_bwd_combine_kernel(const BwdArgs p) {
  const int D = p.d_k, PW = 2 * D + 4, RB = p.row_blocks;  // partial rows padded to float4
  const int Hv = p.num_v_heads, Hk = p.num_qk_heads, G = Hv / Hk;
  const int dshift = __builtin_ctz((unsigned)D), nqk = Hk << dshift;
  const int64_t T = p.total_tokens;
  for (int64_t t = blockIdx.x; t < T; t += gridDim.x) {
    const float *tok = p.partials + t * Hv * RB * PW;
    for (int i = threadIdx.x; i < nqk + Hv; i += kThreads) {
      if (i < nqk) {
        const int hk = i >> dshift, e = i & (D - 1);
        float aq = 0.0f, ak = 0.0f;
        for (int g = 0; g < G; ++g) {
          const float *base = tok + ((hk * G + g) * RB) * PW;
          const float vq = rb_tree<RBMAX>(base + e, PW, RB);
          const float vk = rb_tree<RBMAX>(base + D + e, PW, RB);
          aq = g == 0 ? vq : aq + vq;
          ak = g == 0 ? vk : ak + vk;
        }
        p.dq[(t * Hk + hk) * D + e] = aq;
        p.dk[(t * Hk + hk) * D + e] = ak;
      } else {
        const int h = i - nqk;
        const float *base = tok + (h * RB) * PW;
        p.da[t * Hv + h] = rb_tree<RBMAX>(base + 2 * D, PW, RB);
        p.db[t * Hv + h] = rb_tree<RBMAX>(base + 2 * D + 1, PW, RB);
      }
    }
  }
}

// ---------------------------------------------------------------------------- launchers

template <typename Args>
hipError_t launch1(const void *fn, int64_t grid, Args args, hipStream_t stream,
                   int threads = kThreads) {
  if (grid <= 0) return hipSuccess;
  void *kargs[] = {&args};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), kargs, 0, stream);
}

template <int D>
const void *state_fn(int L, bool bf16) {
  switch (L) {
    case 16: return bf16 ? (const void *)cpr_bwd_state_kernel<D, 16, true>
                         : (const void *)cpr_bwd_state_kernel<D, 16, false>;
    case 8: return bf16 ? (const void *)cpr_bwd_state_kernel<D, 8, true>
                        : (const void *)cpr_bwd_state_kernel<D, 8, false>;
    default: return bf16 ? (const void *)cpr_bwd_state_kernel<D, 4, true>
                         : (const void *)cpr_bwd_state_kernel<D, 4, false>;
  }
}

template <int D, bool LONG, bool WHOLE>
const void *chunk_fn_len(bool bf16, bool seq) {
  if (seq)
    return bf16 ? (const void *)cpr_bwd_chunk_kernel<D, true, true, LONG, WHOLE>
                : (const void *)cpr_bwd_chunk_kernel<D, false, true, LONG, WHOLE>;
  return bf16 ? (const void *)cpr_bwd_chunk_kernel<D, true, false, LONG, WHOLE>
              : (const void *)cpr_bwd_chunk_kernel<D, false, false, LONG, WHOLE>;
}

// Chunks of at most kSeg tokens take the kernels without the segment advance; `whole`
// picks their branch-free variant (nullptr for longer chunks).
template <int D>
const void *chunk_fn(bool bf16, bool seq, int chunk, bool whole) {
  if (chunk > kSeg) return whole ? nullptr : chunk_fn_len<D, true, false>(bf16, seq);
  return whole ? chunk_fn_len<D, false, true>(bf16, seq) : chunk_fn_len<D, false, false>(bf16, seq);
}

}  // namespace

// ------------------------------------------------------- fixed scratch for the no-alloc call

// The workspace of gdn_cpr_trainer_bwd_noalloc: one array per GPU the library runs on, held
// until the process ends. On the host, `scratch` names a stand-in, not device memory: every
// host use goes through the address hipGetSymbolAddress returns for the current device.
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

hipError_t noalloc_scratch(void **ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void *addr[kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {  // once per device, with that device current
    void *p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (!p) return hipErrorInvalidSymbol;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

int backward_row_blocks(int d_v) { return (d_v + kChunkRows - 1) / kChunkRows; }

BwdWorkspace backward_workspace(int64_t num_seqs, int64_t num_v_heads, int64_t d_k,
                                int64_t d_v, int64_t total_tokens, int64_t total_chunks) {
  auto up256 = [](int64_t x) { return (x + 255) / 256 * 256; };
  BwdWorkspace w{};
  const int64_t slots = total_chunks + num_seqs;
  w.plan_off = 0;
  w.plan_bytes = up256((kPlanHeader + 2 * slots) * 4);
  w.cbase_off = w.plan_off + w.plan_bytes;
  w.cbase_bytes = up256(std::max<int64_t>(num_seqs, 1) * 4);
  w.dsh_off = w.cbase_off + w.cbase_bytes;
  w.dsh_bytes = up256(total_chunks * num_v_heads * d_v * d_k * 4);
  w.partials_off = w.dsh_off + w.dsh_bytes;
  w.partials_bytes =
      up256(total_tokens * num_v_heads * backward_row_blocks((int)d_v) * (2 * d_k + 4) * 4);
  w.total = w.partials_off + w.partials_bytes;
  w.slots_max = slots;
  return w;
}

int64_t backward_state_grid(const BwdArgs &a, int L) {
  const int64_t rows = kThreads / L;
  return (int64_t)a.num_seqs * a.num_v_heads * ((a.d_v + rows - 1) / rows);
}

int64_t backward_chunk_grid(const BwdArgs &a, bool seq) {
  return (int64_t)(seq ? a.num_seqs : a.slots_max) * a.num_v_heads * a.row_blocks;
}

hipError_t launch_backward(const BwdArgs &args, int L, bool seq, hipStream_t st) {
  if (args.row_blocks < 1 || args.row_blocks > 32) return hipErrorInvalidValue;  // d_v <= 1024
  BwdArgs a = args;
  // The branch-free chunk kernel needs whole waves of rows (every wave's four rows below d_v
  // or none) and chunks of one segment; it runs after the general kernel, which then takes
  // only the chunks with a partial sub-block.
  a.whole = a.chunk <= kSeg && a.d_v % (64 / kChunkLanes) == 0;
  hipError_t e = launch1((const void *)cpr_bwd_plan_kernel, 1, a, st);
  if (e != hipSuccess) return e;
  const void *sf, *cf, *wf;
  switch (a.d_k) {
    case 16: sf = state_fn<16>(L, a.bf16); cf = chunk_fn<16>(a.bf16, seq, a.chunk, false);
             wf = chunk_fn<16>(a.bf16, seq, a.chunk, true); break;
    case 32: sf = state_fn<32>(L, a.bf16); cf = chunk_fn<32>(a.bf16, seq, a.chunk, false);
             wf = chunk_fn<32>(a.bf16, seq, a.chunk, true); break;
    case 64: sf = state_fn<64>(L, a.bf16); cf = chunk_fn<64>(a.bf16, seq, a.chunk, false);
             wf = chunk_fn<64>(a.bf16, seq, a.chunk, true); break;
    case 128: sf = state_fn<128>(L, a.bf16); cf = chunk_fn<128>(a.bf16, seq, a.chunk, false);
              wf = chunk_fn<128>(a.bf16, seq, a.chunk, true); break;
    default: return hipErrorInvalidValue;
  }
  if (!seq && (e = launch1(sf, backward_state_grid(a, L), a, st)) != hipSuccess) return e;
  const int64_t cgrid = backward_chunk_grid(a, seq);
  if ((e = launch1(cf, cgrid, a, st, kChunkThreads)) != hipSuccess) return e;
  if (a.whole && (e = launch1(wf, cgrid, a, st, kChunkThreads)) != hipSuccess) return e;
  const int64_t grid = std::min<int64_t>(a.total_tokens, 65536);  // tokens, grid-strided
  const void *comb;
  if (a.row_blocks <= 1) comb = (const void *)cpr_bwd_combine_kernel<1>;
  else if (a.row_blocks <= 2) comb = (const void *)cpr_bwd_combine_kernel<2>;
  else if (a.row_blocks <= 4) comb = (const void *)cpr_bwd_combine_kernel<4>;
  else if (a.row_blocks <= 8) comb = (const void *)cpr_bwd_combine_kernel<8>;
  else if (a.row_blocks <= 16) comb = (const void *)cpr_bwd_combine_kernel<16>;
  else comb = (const void *)cpr_bwd_combine_kernel<32>;  // d_v <= 1024: at most 32 blocks
  return launch1(comb, grid, a, st);
}

}  // namespace gdn
