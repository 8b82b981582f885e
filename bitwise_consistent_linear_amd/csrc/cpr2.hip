// Two-level CPR on gfx950: the IsoExec pages' literal reading of Chunkwise-Parallel
// Recurrent Gated DeltaNet, in which the chunk-boundary states come from a chunkwise
// transition and the outputs from the recurrence run in parallel between the boundaries,
// and decode resynchronises its state every C tokens.
//
// For a full chunk of C tokens the rows' update is affine: S_end = S_start A_c + B_c.
//   rows kernel, TRANSITION: A_c's d_k rows start as unit rows e_j and absorb the chunk's
//       tokens with v = +0; B_c's d_v rows start at +0 and absorb them with v (the contract
//       row update, cpr_row.hpp); all chunks in parallel;
//   boundary kernel: S_{c+1} = B_c + S_c A_c, chunk after chunk per sequence, on the binary32
//       matrix instructions, whose every step is a fused multiply-add in ascending k with the
//       accumulator first: the accumulator starts as B_c, so each element is B_c[i, j] plus
//       the products in ascending k, one rounding each;
//   rows kernel, OUTPUT: every chunk's rows restart from S_c and absorb its tokens, writing o
//       (and, for a sequence that ends part-way through a chunk, the final state).
// Decode: the running rows take one token per step (the decode kernel of cpr_kernels.hip);
// the token also goes into a C-slot cache; after a chunk's last token the rows kernel
// rebuilds A_c and B_c from the cache and the boundary kernel sets S_{c+1}, which becomes the
// running rows, the boundary state and the resync checkpoint.

#include <algorithm>
#include <type_traits>

#include "cpr_io.hpp"
#include "cpr_row.hpp"
#include "internal.h"

namespace gdn {
namespace {

using namespace io;

constexpr int kThreads = 256;
// Lanes per state row in the rows kernel. Its grids hold every chunk of every head side by
// side, so occupancy is plentiful: 4 lanes per row (8 whole leaves per lane at d_k = 128)
// keeps the cross-lane part of each dot at two DPP levels.
constexpr int kLanes = 4;
constexpr int kRows = kThreads / kLanes;   // rows per workgroup
// Tokens staged at a time: 16 for the transitions, whose next block is loaded into
// registers meanwhile; 32 for the outputs, which load between blocks (fewer waits per chunk)
constexpr int kSubTransition = 16, kSubOutput = 32;
enum Cpr2Mode : int { kTransition = 0, kOutput = 1 };
// Word 3 of a raw buffer resource on gfx9-family chips (32-bit data format, no swizzle).
constexpr int kBufferWord3 = 0x00020000;

using f32x4 = float __attribute__((ext_vector_type(4)));

__global__ __launch_bounds__(kThreads) void cpr2_plan_kernel(const Cpr2Args p) {
  chunk_plan(p.cu_seqlens, p.num_seqs, p.total_tokens, p.chunk, p.total_chunks, p.slots_max,
             p.plan, p.plan_cbase);
}

// Which chunk a unit of the rows kernel works on. Batch: slot s of the plan. Decode: entry s
// of the list of sequences whose step ends a chunk (their caches hold the chunk's tokens:
// rows n C .. n C + C - 1 of the cache arrays).
struct ChunkWork {
  bool active;
  int n, c;
  int64_t t0;    // first token row of the chunk in the token arrays
  int len;       // tokens in the chunk
  int64_t cidx;  // index of its transition / of the state after it
  bool last;     // the sequence's last chunk (batch)
};

__device__ __forceinline__ ChunkWork chunk_work(const Cpr2Args &p, int unit) {
  ChunkWork w{};
  if (p.decode) {
    w.n = p.plan[kPlanHeader + unit];
    w.t0 = (int64_t)w.n * p.chunk;
    w.len = p.chunk;
    w.cidx = w.n;
    w.active = true;
    return w;
  }
  if (unit >= p.plan[0]) return w;
  w.n = p.plan[kPlanHeader + 2 * unit];
  w.c = p.plan[kPlanHeader + 2 * unit + 1];
  int64_t bos, eos;
  seq_range(p.cu_seqlens, w.n, p.total_tokens, bos, eos);
  w.t0 = bos + (int64_t)w.c * p.chunk;
  if (w.t0 >= eos) return w;
  w.len = (int)(eos - w.t0 < p.chunk ? eos - w.t0 : p.chunk);
  w.cidx = (int64_t)p.plan_cbase[w.n] + w.c;
  w.last = w.t0 + w.len == eos;
  w.active = true;
  return w;
}

// Decode: the sequences whose step ends a chunk, in order, into plan[kPlanHeader ..] with
// their count in plan[0]; run by one workgroup of kThreads threads.
__device__ void list_chunk_ends(const Cpr2Args &p) {
  __shared__ int s_wave[kThreads / 64];
  __shared__ int s_base;
  const int tid = threadIdx.x, wave = tid / 64, lane = tid % 64;
  if (tid == 0) s_base = 0;
  __syncthreads();
  for (int b0 = 0; b0 < p.num_seqs; b0 += kThreads) {
    const int n = b0 + tid;
    bool ends = false;
    if (n < p.num_seqs) {
      const int32_t pos = p.pos[n];
      ends = pos >= 0 && (pos + 1) % p.chunk == 0;
    }
    const unsigned long long m = __ballot(ends);
    const int below = __popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) s_wave[wave] = __popcll(m);
    __syncthreads();
    int off = s_base;
    for (int w = 0; w < wave; ++w) off += s_wave[w];
    if (ends) p.plan[kPlanHeader + off + below] = n;
    __syncthreads();
    if (tid == 0)
      for (int w = 0; w < kThreads / 64; ++w) s_base += s_wave[w];
    __syncthreads();
  }
  if (tid == 0) p.plan[0] = s_base;
}

// kRows rows of one (chunk, value head) per unit. TRANSITION rows r < d_k are A_c's (unit
// start, v = +0), rows d_k <= r < d_k + d_v are B_c's (zero start); OUTPUT rows are S's.
// Batch: one unit per workgroup. LISTED (decode): workgroups take the units of the listed
// sequences in a grid-stride loop.
template <int D, bool BF16, int MODE, bool LISTED>
__global__ __launch_bounds__(kThreads) void cpr2_rows_kernel(const Cpr2Args p) {
  constexpr bool OUT = MODE == kOutput;
  constexpr int L = kLanes, M = D / L, ROWS = kRows, GROUPS = D / 4;
  constexpr int SB = OUT ? kSubOutput : kSubTransition;
  constexpr int KQ_ITEMS = SB * GROUPS, V_ITEMS = SB * ROWS;
  constexpr int KQ_PER = (KQ_ITEMS + kThreads - 1) / kThreads;
  constexpr int V_PER = (V_ITEMS + kThreads - 1) / kThreads;
  using raw_t = typename Raw4<BF16>::type;
  // Transitions: two buffers, sub-block s computes from buffer s & 1 while the loads of s + 1
  // are in flight and then deposited in the other. Outputs: one buffer, loaded between
  // sub-blocks; their rows need more registers, and the prefetch would cost a wave per SIMD.
  constexpr bool PF = !OUT;
  constexpr int NB = PF ? 2 : 1;
  __shared__ __align__(16) float sk[NB][SB * D];
  __shared__ __align__(16) float sq[NB][OUT ? SB * D : 4];
  __shared__ float sv[NB][V_ITEMS], sa[NB][SB], sb[NB][SB];
  __shared__ float so[NB][OUT ? V_ITEMS : 1];

  const int tid = threadIdx.x, row = tid / L, lane = tid % L;
  const int Hv = p.num_v_heads, Hk = p.num_qk_heads, dk = p.d_k, dv = p.d_v;
  const int rows = OUT ? dv : dk + dv;
  const int RB = (rows + ROWS - 1) / ROWS;
  const int units = LISTED ? p.plan[0] : p.slots_max;

  auto unit = [&](int blk) {
    int pair, rblock;
    block_work(blk, units * Hv, RB, 1, pair, rblock);
    const int h = pair % Hv;
    const ChunkWork w = chunk_work(p, pair / Hv);
    if (!w.active || (!OUT && w.len < p.chunk)) return;  // uniform: full chunks' transitions
    if (!OUT && !p.decode && w.cidx >= p.total_chunks) return;  // lengths past the claims
    const int hk = h / (Hv / Hk);
    const int r0 = rblock * ROWS, r = r0 + row;
    const bool valid = r < rows;
    const bool arow = !OUT && r < dk;  // a row of A_c
    const int vi = OUT ? r : r - dk;   // the value row this row reads
    const int64_t vstride = (int64_t)Hv * dv;
    const int64_t st = (int64_t)dv * D;  // floats per (head) state

    float s[M];
#pragma unroll
    for (int e = 0; e < M; ++e) s[e] = (arow && lane * M + e == r) ? 1.0f : 0.0f;
    if (OUT && valid) {
      const float *src = nullptr;
      if (w.c == 0) {
        if (p.initial_state) src = p.initial_state + ((int64_t)w.n * Hv + h) * st;
      } else if (w.cidx - 1 < p.total_chunks) {
        src = p.chunk_states + ((w.cidx - 1) * Hv + h) * st;
      }
      if (src) load_row<M>(src + (int64_t)r * D + lane * M, s);
    }

    // A sub-block's inputs in registers between their global loads and their LDS deposit.
    // Token indices are clamped to the chunk's last token, so the loads need no branches;
    // the extra values land in slots the token loop never reads.
    raw_t rk[KQ_PER], rq[OUT ? KQ_PER : 1];
    uint32_t rv[V_PER];
    float ra = 0.0f, rb = 0.0f;
    auto fetch = [&](int j0) {
      const int last = w.len - 1;
#pragma unroll
      for (int j = 0; j < KQ_PER; ++j) {
        const int g = (tid + j * kThreads) % KQ_ITEMS;
        const int t = j0 + g / GROUPS < last ? j0 + g / GROUPS : last;
        const int64_t src = ((w.t0 + t) * Hk + hk) * D + 4 * (g % GROUPS);
        rk[j] = load_raw4<BF16>(p.k, src);
        if constexpr (OUT) rq[j] = load_raw4<BF16>(p.q, src);
      }
#pragma unroll
      for (int j = 0; j < V_PER; ++j) {
        const int e = (tid + j * kThreads) % V_ITEMS;
        const int t = j0 + e / ROWS < last ? j0 + e / ROWS : last;
        const int rr = r0 + e % ROWS, vr = OUT ? rr : rr - dk;
        rv[j] = (rr < rows && vr >= 0)
                    ? load_raw1<BF16>(p.v, (w.t0 + t) * vstride + (int64_t)h * dv + vr)
                    : 0u;  // +0 for A_c's rows and rows past the block
      }
      const int t = j0 + tid % SB < last ? j0 + tid % SB : last;
      ra = p.a[(w.t0 + t) * Hv + h];
      rb = p.b[(w.t0 + t) * Hv + h];
    };
    auto deposit = [&](int buf) {
#pragma unroll
      for (int j = 0; j < KQ_PER; ++j) {
        const int g = tid + j * kThreads;
        if (KQ_ITEMS % kThreads == 0 || g < KQ_ITEMS) {
          const int off = (g / GROUPS) * D + stage_slot<D, L>(g % GROUPS);
          *reinterpret_cast<float4 *>(&sk[buf][off]) = widen4<BF16>(rk[j]);
          if constexpr (OUT) *reinterpret_cast<float4 *>(&sq[buf][off]) = widen4<BF16>(rq[j]);
        }
      }
#pragma unroll
      for (int j = 0; j < V_PER; ++j) {
        const int e = tid + j * kThreads;
        if (V_ITEMS % kThreads == 0 || e < V_ITEMS) sv[buf][e] = widen1<BF16>(rv[j]);
      }
      if (tid < SB) {
        sa[buf][tid] = ra;
        sb[buf][tid] = rb;
      }
    };

    const int nsub = (w.len + SB - 1) / SB;
    if constexpr (PF) {
      fetch(0);
      __syncthreads();  // the previous unit's readers of both buffers are done
      deposit(0);
      __syncthreads();
    }
    for (int sbk = 0; sbk < nsub; ++sbk) {
      const int buf = PF ? sbk & 1 : 0, j0 = sbk * SB;
      const int nt = w.len - j0 < SB ? w.len - j0 : SB;
      const bool more = sbk + 1 < nsub;
      if constexpr (PF) {
        if (more) fetch(j0 + SB);  // global loads in flight while this sub-block computes
      } else {
        fetch(j0);
        __syncthreads();  // the previous sub-block's (or unit's) readers are done
        deposit(0);
        __syncthreads();
      }
      if constexpr (OUT) {
        // token j's readout dot runs side by side with token j+1's key dot (both read the
        // state after token j): the same operations on the same operands as row_token
        float kr[M], qr[M], x[M];
        lds_slice<D, L>(&sk[buf][0], lane, kr);
        row_decay<D, L>(s, sa[buf][0], x);
        float u = contract_dot<D, L>(x, kr);
        for (int j = 0; j < nt; ++j) {
          row_update<D, L>(s, row_delta(sb[buf][j], sv[buf][j * ROWS + row], u), kr, x);
          lds_slice<D, L>(&sq[buf][j * D], lane, qr);
          float o_i;
          if (j + 1 < nt) {
            lds_slice<D, L>(&sk[buf][(j + 1) * D], lane, kr);
            row_decay<D, L>(s, sa[buf][j + 1], x);
            float xs[2][M], ys[2][M], res[2];
#pragma unroll
            for (int e = 0; e < M; ++e) {
              xs[0][e] = s[e];
              ys[0][e] = qr[e];
              xs[1][e] = x[e];
              ys[1][e] = kr[e];
            }
            contract_dots<D, L, 2>(xs, ys, res);
            o_i = res[0];
            u = res[1];
          } else {
            o_i = contract_dot<D, L>(s, qr);
          }
          if (lane == 0) so[buf][j * ROWS + row] = o_i;
        }
      } else {
        for (int j = 0; j < nt; ++j) {
          float kr[M], x[M];
          lds_slice<D, L>(&sk[buf][j * D], lane, kr);
          row_decay<D, L>(s, sa[buf][j], x);
          const float u = contract_dot<D, L>(x, kr);
          // A_c's rows absorb v = +0 (their staged v is +0)
          row_update<D, L>(s, row_delta(sb[buf][j], sv[buf][j * ROWS + row], u), kr, x);
        }
      }
      if constexpr (PF) {
        if (more) deposit(buf ^ 1);
      }
      __syncthreads();
      if constexpr (OUT) {
        for (int e = tid; e < nt * ROWS; e += kThreads) {
          const int tt = e / ROWS, rr = r0 + e % ROWS;
          if (rr < dv) p.o[(w.t0 + j0 + tt) * vstride + (int64_t)h * dv + rr] = so[buf][e];
        }
      }
    }
    if (!valid) return;
    if constexpr (OUT) {
      // a sequence that ends part-way through a chunk ends with these rows
      if (p.final_state && w.last && w.len < p.chunk)
        store_row<M>(p.final_state + ((int64_t)w.n * Hv + h) * st + (int64_t)r * D + lane * M,
                     s);
    } else {
      float *dst = arow ? p.trans_a + ((w.cidx * Hv + h) * (int64_t)D + r) * D
                        : p.trans_b + (w.cidx * Hv + h) * st + (int64_t)vi * D;
      store_row<M>(dst + lane * M, s);
    }
  };

  if constexpr (LISTED) {
    const int total = units * Hv * RB;
    for (int blk = blockIdx.x; blk < total; blk += gridDim.x) unit(blk);
  } else {
    unit(blockIdx.x);
  }
}

// A byte offset that every buffer range check rejects: loads from it read +0 and stores to it
// are dropped (the offset sits in the address register, which the check always covers).
constexpr int kOutOfRange = (int)0x80000000u;

// A lane's 16 values of a 32 x 32 block into a state of `bytes` bytes at dst; off[v] is the
// byte offset of value v (kOutOfRange for rows past d_v, which are dropped).
__device__ __forceinline__ void store_rows(float *dst, int bytes, const int (&off)[16],
                                           const float (&out)[16]) {
  const __amdgpu_buffer_rsrc_t R = __builtin_amdgcn_make_buffer_rsrc(dst, 0, bytes, kBufferWord3);
#pragma unroll
  for (int v = 0; v < 16; ++v)
    __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(unsigned, out[v]), R, off[v], 0, 0);
}

// One workgroup: 32 rows of one (sequence, value head); wave w owns state columns
// 32 w .. 32 w + 31. For each full chunk in order, S <- B_c + S A_c on the matrix units:
// v_mfma_f32_16x16x4_f32 adds S[i, k] A[k, j] for k ascending, four k per instruction, each
// a fused multiply-add, onto an accumulator that starts as B_c. A wave's 32 x 32 block is
// four independent 16 x 16 accumulator chains (two row halves x two column halves), so the
// matrix unit always has an instruction whose operands are ready. The wave's B operands, its
// 32 columns of A_c (D / 2 values per lane), live in registers, and with PREFETCH the next
// chunk's columns and accumulator start are loaded while the current chunk's chains run.
// S's 32 rows are shared by the waves through LDS, double-buffered. Workgroups take
// (sequence, head, row block) units in a grid-stride loop; decode's units are those of the
// listed sequences only, on a capped grid, so a step on which no chunk ends costs little.
template <int D, bool PREFETCH>
__global__ __launch_bounds__(D * 2) void cpr2_boundary_kernel(const Cpr2Args p) {
  // S[i][k] sits at sS[buf][i][(k % 4) KQ + k / 4]: a lane's A operands for four steps
  // (k = 4 g + lq .. 4 (g + 3) + lq) are one 16-byte read. Rows padded by 4 floats.
  constexpr int KQ = D / 4, SS = D + 4;
  __shared__ __align__(16) float sS[2][32][SS];  // the rows' state, current and next
  auto slot = [](int k) { return (k % 4) * KQ + k / 4; };
  const int tid = threadIdx.x, wave = tid / 64, l = tid % 64, lq = l / 16, li = l % 16;
  const int Hv = p.num_v_heads, dv = p.d_v;
  const int RB = (dv + 31) / 32;
  const int seqs = p.decode ? p.plan[0] : p.num_seqs;
  const int total = seqs * Hv * RB;  // below 2^31: checked on the host
  const int64_t st = (int64_t)dv * D;
  for (int blk = blockIdx.x; blk < total; blk += gridDim.x) {
    // the row blocks of a (sequence, head) on one XCD: they read the same A_c, once from HBM
    int pair, rblock;
    block_work(blk, seqs * Hv, RB, 1, pair, rblock);
    const int h = pair % Hv;
    const int n = p.decode ? p.plan[kPlanHeader + pair / Hv] : pair / Hv;
    const int r0 = rblock * 32;
    int64_t first, count;  // transitions to apply, by index
    const float *start;    // S before the first of them
    if (p.decode) {
      first = n;
      count = 1;
      start = p.boundary + ((int64_t)n * Hv + h) * st;
    } else {
      int64_t bos, eos;
      seq_range(p.cu_seqlens, n, p.total_tokens, bos, eos);
      first = p.plan_cbase[n];
      count = (eos - bos) / p.chunk;
      if (first + count > p.total_chunks) count = p.total_chunks - first;
      if (count < 0) count = 0;
      start = p.initial_state ? p.initial_state + ((int64_t)n * Hv + h) * st : nullptr;
    }
    // Accumulator value v = 4 (2 rh + ch) + r of this lane: row r0 + 16 rh + 4 lq + r,
    // column 32 wave + 16 ch + li. Its byte offset in a state (out of range past d_v: such
    // rows read +0 and their stores drop); A_c by buffer loads with one address register per
    // column half and the k steps as scalar offsets (always in range).
    int off[16];
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int rh = v / 8, ch = (v / 4) % 2, r = v % 4;
      const int i = r0 + 16 * rh + 4 * lq + r, j = 32 * wave + 16 * ch + li;
      off[v] = i < dv ? (i * D + j) * 4 : kOutOfRange;
    }
    const int va0 = (lq * D + 32 * wave + li) * 4, va1 = va0 + 16 * 4;
    auto load_ab = [&](int64_t cidx, float (&a)[2][KQ], float (&b)[16]) {
      const __amdgpu_buffer_rsrc_t A = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float *>(p.trans_a + (cidx * Hv + h) * (int64_t)D * D), 0, D * D * 4,
          kBufferWord3);
      const __amdgpu_buffer_rsrc_t B = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<float *>(p.trans_b + (cidx * Hv + h) * st), 0, (int)(st * 4), kBufferWord3);
#pragma unroll
      for (int g = 0; g < KQ; ++g) {
        a[0][g] = __builtin_bit_cast(float,
                                     __builtin_amdgcn_raw_buffer_load_b32(A, va0, 16 * D * g, 0));
        a[1][g] = __builtin_bit_cast(float,
                                     __builtin_amdgcn_raw_buffer_load_b32(A, va1, 16 * D * g, 0));
      }
#pragma unroll
      for (int v = 0; v < 16; ++v)
        b[v] = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(B, off[v], 0, 0));
    };
    float ca[2][KQ], cb[16];
    if (count > 0) load_ab(first, ca, cb);
    __syncthreads();  // the previous unit's readers of sS are done
    for (int e = tid; e < 32 * D; e += blockDim.x) {
      const int i = e / D, k = e % D;
      sS[0][i][slot(k)] = (start && r0 + i < dv) ? start[(int64_t)(r0 + i) * D + k] : 0.0f;
    }
    int cur = 0;
    for (int64_t c = 0; c < count; ++c) {
      const int64_t cidx = first + c;
      __syncthreads();  // sS[cur] is complete
      float na[PREFETCH ? 2 : 1][PREFETCH ? KQ : 1], nb[PREFETCH ? 16 : 1];
      if constexpr (PREFETCH) {
        if (c + 1 < count) load_ab(cidx + 1, na, nb);
      }
      f32x4 acc[2][2];
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[v / 8][(v / 4) % 2][v % 4] = cb[v];
      // the chunk's A operands from LDS first (one wait), then the four chains interleaved
      float4 sv4[2][KQ / 4];
#pragma unroll
      for (int rh = 0; rh < 2; ++rh)
#pragma unroll
        for (int g = 0; g < KQ / 4; ++g)
          sv4[rh][g] = *reinterpret_cast<const float4 *>(&sS[cur][16 * rh + li][lq * KQ + 4 * g]);
#pragma unroll
      for (int g = 0; g < KQ / 4; ++g) {
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int step = 4 * g + u;
#pragma unroll
          for (int rh = 0; rh < 2; ++rh) {
            const float sa = u == 0 ? sv4[rh][g].x : u == 1 ? sv4[rh][g].y
                           : u == 2 ? sv4[rh][g].z : sv4[rh][g].w;
#pragma unroll
            for (int ch = 0; ch < 2; ++ch)
              acc[rh][ch] = __builtin_amdgcn_mfma_f32_16x16x4f32(sa, ca[ch][step], acc[rh][ch],
                                                                 0, 0, 0);
          }
        }
      }
      const int nxt = cur ^ 1;
      float out[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int rh = v / 8, ch = (v / 4) % 2, r = v % 4;
        out[v] = acc[rh][ch][r];
        sS[nxt][16 * rh + 4 * lq + r][slot(32 * wave + 16 * ch + li)] = out[v];
      }
      if constexpr (PREFETCH) {
        // take the prefetched operands before this chunk's stores are issued: stores and
        // loads share one in-order counter, so waiting for the loads after the stores would
        // wait for the stores to reach memory too
        if (c + 1 < count) {
#pragma unroll
          for (int g = 0; g < KQ; ++g) {
            ca[0][g] = na[0][g];
            ca[1][g] = na[1][g];
          }
#pragma unroll
          for (int v = 0; v < 16; ++v) cb[v] = nb[v];
        }
        __builtin_amdgcn_sched_barrier(0);
      }
      // S_{c+1} to HBM by buffer stores (rows past d_v are dropped), a fixed number per
      // variant with no branch, so the compiler's waits can count them exactly
      if constexpr (PREFETCH) {  // batch: chunk_states is set whenever a chunk exists
        store_rows(p.chunk_states + (cidx * Hv + h) * st, (int)(st * 4), off, out);
      } else {  // decode: boundary, state, resync (a range of 0 bytes when there is none:
                // every store then falls outside it and is dropped)
        const int64_t base = ((int64_t)n * Hv + h) * st;
        store_rows(p.boundary + base, (int)(st * 4), off, out);
        store_rows(p.state + base, (int)(st * 4), off, out);
        store_rows((p.resync ? p.resync : p.boundary) + base, p.resync ? (int)(st * 4) : 0, off,
                   out);
      }
      cur = nxt;
    }
    // a sequence whose length is a multiple of C (zero included) ends on its boundary state
    if (!p.decode && p.final_state) {
      int64_t bos, eos;
      seq_range(p.cu_seqlens, n, p.total_tokens, bos, eos);
      if ((eos - bos) % p.chunk == 0) {
        __syncthreads();
        for (int e = tid; e < 32 * D; e += blockDim.x) {
          const int i = e / D, k = e % D;
          if (r0 + i < dv)
            p.final_state[((int64_t)n * Hv + h) * st + (int64_t)(r0 + i) * D + k] =
                sS[cur][i][slot(k)];
        }
      }
    }
  }
}

// Decode: the step's token into slot pos % C of its sequence's cache; workgroup 0 also lists
// the sequences whose step ends a chunk, for the transition and boundary launches after it.
template <bool BF16>
__global__ __launch_bounds__(kThreads) void cpr2_cache_kernel(const Cpr2Args p, const void *k,
                                                               const void *v, const float *a,
                                                               const float *b) {
  const int n = blockIdx.x;
  if (n == 0) list_chunk_ends(p);
  const int32_t pos = p.pos[n];
  if (pos < 0) return;
  const int Hk = p.num_qk_heads, Hv = p.num_v_heads, dk = p.d_k, dv = p.d_v, C = p.chunk;
  const int64_t row = (int64_t)n * C + pos % C;
  using T = typename std::conditional<BF16, uint16_t, float>::type;
  // 16 bytes per lane where both ends of a copy are 16-byte aligned (the usual case: whole
  // rows of a contiguous tensor), element by element otherwise
  auto copy = [&](void *dst_base, const void *src_base, int count) {
    T *dst = static_cast<T *>(dst_base) + row * count;
    const T *src = static_cast<const T *>(src_base) + (int64_t)n * count;
    constexpr int V = 16 / sizeof(T);
    if ((reinterpret_cast<uintptr_t>(dst) | reinterpret_cast<uintptr_t>(src)) % 16 == 0 &&
        count % V == 0) {
      for (int e = threadIdx.x; e < count / V; e += kThreads)
        reinterpret_cast<uint4 *>(dst)[e] = reinterpret_cast<const uint4 *>(src)[e];
    } else {
      for (int e = threadIdx.x; e < count; e += kThreads) dst[e] = src[e];
    }
  };
  copy(p.cache_k, k, Hk * dk);
  copy(p.cache_v, v, Hv * dv);
  for (int e = threadIdx.x; e < Hv; e += kThreads) {
    p.cache_a[row * Hv + e] = a[(int64_t)n * Hv + e];
    p.cache_b[row * Hv + e] = b[(int64_t)n * Hv + e];
  }
}

template <typename Args>
hipError_t launch(const void *fn, int64_t grid, int threads, Args args, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  void *kargs[] = {&args};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), kargs, 0, stream);
}

// batch transitions and outputs, one unit per workgroup; decode transitions, listed
template <int D>
const void *rows_fn(bool bf16, int mode, bool decode) {
  if (decode)
    return bf16 ? (const void *)cpr2_rows_kernel<D, true, kTransition, true>
                : (const void *)cpr2_rows_kernel<D, false, kTransition, true>;
  if (mode == kTransition)
    return bf16 ? (const void *)cpr2_rows_kernel<D, true, kTransition, false>
                : (const void *)cpr2_rows_kernel<D, false, kTransition, false>;
  return bf16 ? (const void *)cpr2_rows_kernel<D, true, kOutput, false>
              : (const void *)cpr2_rows_kernel<D, false, kOutput, false>;
}

const void *rows_kernel(int d_k, bool bf16, int mode, bool decode) {
  switch (d_k) {
    case 32: return rows_fn<32>(bf16, mode, decode);
    case 64: return rows_fn<64>(bf16, mode, decode);
    default: return rows_fn<128>(bf16, mode, decode);
  }
}

// batch: prefetching sweeps over many chunks; decode: one chunk per unit, lighter on
// registers so more units are in flight
const void *boundary_kernel(int d_k, bool decode) {
  switch (d_k) {
    case 32: return decode ? (const void *)cpr2_boundary_kernel<32, false>
                           : (const void *)cpr2_boundary_kernel<32, true>;
    case 64: return decode ? (const void *)cpr2_boundary_kernel<64, false>
                           : (const void *)cpr2_boundary_kernel<64, true>;
    default: return decode ? (const void *)cpr2_boundary_kernel<128, false>
                           : (const void *)cpr2_boundary_kernel<128, true>;
  }
}

// Decode launches cap their grids: most steps end no chunk, and a workgroup per possible
// unit would cost a dispatch each just to find that out.
constexpr int64_t kDecodeGridCap = 4096;

int64_t boundary_grid(const Cpr2Args &a) {
  const int64_t g = (int64_t)a.num_seqs * a.num_v_heads * ((a.d_v + 31) / 32);
  return a.decode ? std::min(g, kDecodeGridCap) : g;
}

int64_t rows_units(const Cpr2Args &a, int rows) {
  const int64_t units = a.decode ? a.num_seqs : a.slots_max;
  return units * a.num_v_heads * ((rows + kRows - 1) / kRows);
}

int64_t rows_grid(const Cpr2Args &a, int rows) {
  return a.decode ? std::min(rows_units(a, rows), kDecodeGridCap) : rows_units(a, rows);
}

}  // namespace

bool cpr2_dk_admitted(int d_k) { return d_k == 32 || d_k == 64 || d_k == 128; }

Cpr2Layout cpr2_layout(int64_t num_seqs, int64_t num_v_heads, int64_t d_k, int64_t d_v,
                       int64_t total_chunks, bool decode, bool need_states) {
  auto up256 = [](int64_t x) { return (x + 255) / 256 * 256; };
  const int64_t n_trans = decode ? num_seqs : total_chunks;
  Cpr2Layout w{};
  w.plan_off = 0;  // batch: the chunk plan; decode: the list of sequences ending a chunk
  w.cbase_off = up256((kPlanHeader + (decode ? num_seqs : 2 * (total_chunks + num_seqs))) * 4);
  w.ta_off = w.cbase_off + (decode ? 0 : up256(std::max<int64_t>(num_seqs, 1) * 4));
  w.tb_off = w.ta_off + up256(n_trans * num_v_heads * d_k * d_k * 4);
  w.cs_off = w.tb_off + up256(n_trans * num_v_heads * d_v * d_k * 4);
  w.total = w.cs_off + (need_states ? up256(total_chunks * num_v_heads * d_v * d_k * 4) : 0);
  return w;
}

int64_t cpr2_max_grid(const Cpr2Args &a) {
  const int64_t units = a.decode ? a.num_seqs : a.slots_max;
  return std::max<int64_t>(units * a.num_v_heads * ((a.d_k + a.d_v + kRows - 1) / kRows),
                           (int64_t)a.num_seqs * a.num_v_heads * ((a.d_v + 31) / 32));
}

hipError_t launch_cpr2_scan(const Cpr2Args &a, hipStream_t st) {
  hipError_t e = launch((const void *)cpr2_plan_kernel, 1, kThreads, a, st);
  if (e != hipSuccess) return e;
  const int D = a.d_k;
  if ((e = launch(rows_kernel(D, a.bf16, kTransition, false), rows_grid(a, a.d_k + a.d_v),
                  kThreads, a, st)) != hipSuccess)
    return e;
  if ((e = launch(boundary_kernel(D, false), boundary_grid(a), 2 * D, a, st)) != hipSuccess)
    return e;
  return launch(rows_kernel(D, a.bf16, kOutput, false), rows_grid(a, a.d_v), kThreads, a, st);
}

hipError_t launch_cpr2_decode_tail(const Cpr2Args &a, const void *k, const void *v,
                                   const float *av, const float *bv, hipStream_t st) {
  // the token into the cache, then (for sequences whose step ends a chunk) the transition
  // rebuilt from the cache and the new boundary state
  void *kargs[] = {const_cast<Cpr2Args *>(&a), &k, &v, &av, &bv};
  const void *cache = a.bf16 ? (const void *)cpr2_cache_kernel<true>
                             : (const void *)cpr2_cache_kernel<false>;
  hipError_t e = hipLaunchKernel(cache, dim3((unsigned)a.num_seqs), dim3(kThreads), kargs, 0, st);
  if (e != hipSuccess) return e;
  Cpr2Args t = a;  // the transition reads the cache as its token arrays
  t.k = a.cache_k;
  t.v = a.cache_v;
  t.a = a.cache_a;
  t.b = a.cache_b;
  if ((e = launch(rows_kernel(a.d_k, a.bf16, kTransition, true), rows_grid(t, a.d_k + a.d_v),
                  kThreads, t, st)) != hipSuccess)
    return e;
  return launch(boundary_kernel(a.d_k, true), boundary_grid(t), 2 * a.d_k, t, st);
}

}  // namespace gdn
