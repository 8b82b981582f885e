// HIP kernels for CPR Gated DeltaNet on gfx950: the packed-batch scan (trainer_fwd and
// engine_prefill) and the one-token decode step.
//
// Work decomposition: every state row (sequence n, value head h, row i) evolves on its own
// (the gated delta rule updates S row by row: row i only sees v_i). A workgroup of NT
// threads (256; 512 for the two-waves-per-SIMD trainer shape) owns ROWS = NT/L consecutive
// rows of one (n, h); each row sits in the VGPRs of L lanes (cpr_row.hpp). No MFMA: each token is a matrix-vector step on a d_k x d_v state
// whose every element is touched four times, not a dense contraction.
//
// Scan: tokens are staged TS at a time - q and k of the (n, q/k head) in the order the
// lanes read them, v of the workgroup's rows, a and b - into LDS as binary32 (bf16 widened
// exactly) with coalesced loads; the token loop then runs from LDS and registers only. The
// outputs o of a stage go back through LDS so that each token's rows are stored
// contiguously. Chunk-boundary states (trainer) and the final state (prefill) are stored
// straight from the registers, each lane its contiguous slice of the row.
//
// Decode: one launch per step; each row's d_k floats are read from HBM, updated once and
// written back (plus the resync checkpoint on C-token boundaries). For d_k >= 32 a row sits
// on 32 lanes (row_token_split), so that each lane moves 16 bytes of the row at d_k = 128.
//
// Scheduling: workgroups of the longest sequences are dispatched first (for up to 1024
// sequences the rank of every sequence by length is computed in LDS), so that the long
// serial scans overlap with the short ones.

#include "cpr_io.hpp"
#include "cpr_row.hpp"
#include "internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;  // decode, and the scan unless the launcher picks 512
// TS, the tokens staged in LDS at a time, is chosen by the launcher: 64 for a lone wave per
// SIMD at 16 lanes per row with bf16 inputs and in 512-thread workgroups (a trainer launch
// only when C >= 64), 32 for 8 or 16 lanes per row otherwise, 16 for 4 (where occupancy
// matters). Longer stages halve
// the per-stage barrier and pipeline restart but take more LDS. Stages start at in-sequence
// index 0 and every admitted C is a multiple of 16, so a chunk boundary falls on a token
// 16 m - 1 of a stage.
// ----------------------------------------------------------------------------- kernels

using namespace io;

// At 4 lanes per row the scan is issue-bound with many waves to run: it asks for three
// waves per SIMD (at most 168 registers), which hides each wave's dependency chains.
// NT threads per workgroup: 256, or 512 for two waves per SIMD from one workgroup per CU
// (64-token stages staged once for 32 rows). With 512 the o buffer has one stage, not two,
// to fit the LDS, and each wave stores only its own rows' o from it, so that a wave's next
// stage cannot overwrite what another wave is still reading.
template <int D, int L, int TS, bool BF16, int MODE, int NT, int R>
__global__ __launch_bounds__(NT)
__attribute__((amdgpu_waves_per_eu(L == 4 ? 4 - R : 1)))
void cpr_scan_kernel(const ScanArgs p) {
  static_assert(R == 1 || (R == 2 && L == 4 && NT == 256), "row pairs at 4 lanes per row");
  static_assert(TS % 16 == 0, "a stage holds whole 16-token groups");
  constexpr int kThreads = NT;
  constexpr int SO_BUFS = NT == 512 ? 1 : 2;
  // GR groups of L lanes; group g holds the R rows g, g + GR, ... of the workgroup's ROWS.
  constexpr int GR = kThreads / L;
  constexpr int ROWS = R * GR;
  constexpr int M = D / L;
  // Chunk boundaries inside a full stage (after its tokens 15, 31, ...) are kept from the
  // registers and stored after the stage; a trainer launch with 64-token stages is made only
  // for C >= 64, whose boundaries fall on stage ends.
  constexpr bool INNER = MODE == kTrainer && TS <= 32;
  constexpr int SNAPS = INNER && TS / 16 > 1 ? TS / 16 - 1 : 1;
  constexpr int GROUPS = D / 4;  // float4 groups per staged k or q vector
  constexpr int KQ_ITEMS = TS * GROUPS, V_ITEMS = TS * ROWS;
  constexpr int KQ_PER = (KQ_ITEMS + kThreads - 1) / kThreads;
  constexpr int V_PER = (V_ITEMS + kThreads - 1) / kThreads;
  using raw_t = typename Raw4<BF16>::type;

  // Two stage buffers: stage s is computed from buffer s&1 while stage s+1 is deposited
  // into the other. A buffer holds the stage's k, then its q.
  constexpr int KQ_FLOATS = TS * D;
  constexpr int POOL = 2 * KQ_FLOATS;
  // One block with the small arrays first, so that they sit below 64 KiB and every read of
  // them takes an immediate offset from a fixed base. The sequence lengths are read only
  // by the ranking, which ends with a barrier before the first deposit, so they share the
  // v buffers.
  static_assert(2 * V_ITEMS >= kMaxRankedSeqs, "the ranking fits in the v buffers");
  struct alignas(16) Lds {
    float sa[2][TS], sb[2][TS];
    union {
      float sv[2][V_ITEMS];
      int s_len[kMaxRankedSeqs];
    };
    float so[SO_BUFS][V_ITEMS];
    int s_pick;
    unsigned long long s_acc;
    alignas(16) float pool[2][POOL];
  };
  __shared__ Lds lds;
  auto &sa = lds.sa;
  auto &sb = lds.sb;
  auto &sv = lds.sv;
  auto &so = lds.so;
  auto &pool = lds.pool;
  int *const s_len = lds.s_len;
  int &s_pick = lds.s_pick;
  unsigned long long &s_acc = lds.s_acc;

  const int tid = threadIdx.x, row = tid / L, lane = tid % L;
  auto SK = [&](int buf) { return &pool[buf][0]; };
  auto SQ = [&](int buf) { return &pool[buf][KQ_FLOATS]; };
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
  int64_t cbase = 0;
  if constexpr (MODE == kTrainer)
    cbase = first_chunk_slot(p.cu_seqlens, n, T, p.chunk, p.total_chunks, &s_acc);

  const int hk = h / (Hv / Hk);
  int irow[R];
  bool valid[R];
  int64_t row_off[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    irow[rr] = r0 + row + GR * rr;
    valid[rr] = irow[rr] < dv;
    row_off[rr] = (((int64_t)n * Hv + h) * dv + irow[rr]) * D + lane * M;
  }
  const int64_t vstride = (int64_t)Hv * dv;

  float s[R][M];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (p.initial_state && valid[rr]) {
      load_row<M>(p.initial_state + row_off[rr], s[rr]);
    } else {
#pragma unroll
      for (int e = 0; e < M; ++e) s[rr][e] = 0.0f;
    }
  }
  float(&s_first)[M] = s[0];
  // Complete the state loads here, once: otherwise the first use of s inside the stage
  // loop waits on the in-order load counter and with it on that stage's prefetch loads.
#pragma unroll
  for (int rr = 0; rr < R; ++rr)
#pragma unroll
    for (int e = 0; e < M; ++e) asm volatile("" ::"v"(s[rr][e]));

  // Staged inputs in registers, between their global load and their LDS deposit. Token and
  // row indices are clamped to valid addresses so the loads need no branches; the extra
  // values land in LDS slots that the token loop never reads.
  raw_t rk[KQ_PER], rq[KQ_PER];
  uint32_t rv[V_PER];
  float ra, rb;
  // Generic fetch of the stage starting at in-sequence token t0 (any length, indices clamped
  // to the sequence's last token): used for a sequence's last, partial stage.
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
      rv[j] = load_raw1<BF16>(p.v, (bos + t) * vstride + (int64_t)h * dv + r);
    }
    const int64_t t = t0 + tid % TS < last ? t0 + tid % TS : last;
    ra = p.a[(bos + t) * Hv + h];
    rb = p.b[(bos + t) * Hv + h];
  };
  // Byte offsets of this thread's staged loads and o stores inside one full stage. A full
  // stage adds them to scalar stage bases, so its global accesses need no per-stage 64-bit
  // address arithmetic. The host admits Hv * max(d_k, d_v) <= 2^20, so every offset inside a
  // stage of at most 64 tokens fits in 32 bits. Where stages are pipelined (L >= 8) they are
  // computed once and held for the whole scan (FIXED); at 4 lanes per row the registers go
  // to a third wave instead, and each full stage recomputes them in 32-bit arithmetic.
  constexpr bool FIXED = L >= 8;
  constexpr uint32_t EL = BF16 ? 2 : 4;
  const uint32_t kq_tok = (uint32_t)Hk * D;  // q/k elements per token
  // (t is the thread index; !FIXED passes an opaque copy so that the offsets are
  // recomputed where used instead of being hoisted into registers held across the scan)
  auto kq_offset = [&](int t, int j) -> uint32_t {
    const uint32_t g = (uint32_t)(t + j * kThreads) % KQ_ITEMS;
    return ((g / GROUPS) * kq_tok + (uint32_t)hk * D + 4 * (g % GROUPS)) * EL;
  };
  auto v_offset = [&](int t, int j) -> uint32_t {
    const uint32_t e = (uint32_t)(t + j * kThreads) % V_ITEMS;
    const int r = r0 + (int)(e % ROWS) < dv ? r0 + (int)(e % ROWS) : dv - 1;
    return ((e / ROWS) * (uint32_t)vstride + (uint32_t)(h * dv + r)) * EL;
  };
  auto o_offset = [&](int t, int j) -> uint32_t {
    const int eo = t + j * kThreads;
    return ((uint32_t)(eo / ROWS) * (uint32_t)vstride + (uint32_t)(h * dv + r0 + eo % ROWS)) * 4;
  };
  auto o_store_ok = [&](int t, int j) -> bool {
    const int eo = t + j * kThreads;
    return (V_ITEMS % kThreads == 0 || eo < V_ITEMS) && r0 + eo % ROWS < dv;
  };
  uint32_t kq_off[KQ_PER], v_off[V_PER], o_off[V_PER];
  bool o_ok[V_PER];
  if constexpr (FIXED) {
#pragma unroll
    for (int j = 0; j < KQ_PER; ++j) kq_off[j] = kq_offset(tid, j);
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      v_off[j] = v_offset(tid, j);
      o_off[j] = o_offset(tid, j);
      o_ok[j] = o_store_ok(tid, j);
    }
  }
  const uint32_t ab_off = (uint32_t)((tid % TS) * Hv + h) * 4;
  // Fetch of a full stage (t0 + TS <= Tn): scalar bases plus the 32-bit offsets.
  auto opaque_tid = [&]() {
    int t = tid;
    if constexpr (!FIXED) asm volatile("" : "+v"(t));
    return t;
  };
  auto fetch_full = [&](int64_t t0) {
    const int t = opaque_tid();
    const int64_t tok = bos + t0;
    const char *kb = static_cast<const char *>(p.k) + tok * kq_tok * EL;
    const char *qb = static_cast<const char *>(p.q) + tok * kq_tok * EL;
    const char *vb = static_cast<const char *>(p.v) + tok * vstride * EL;
    const char *ab = reinterpret_cast<const char *>(p.a + tok * Hv);
    const char *bb = reinterpret_cast<const char *>(p.b + tok * Hv);
#pragma unroll
    for (int j = 0; j < KQ_PER; ++j) {
      const uint32_t off = FIXED ? kq_off[j] : kq_offset(t, j);
      rk[j] = *reinterpret_cast<const raw_t *>(kb + off);
      rq[j] = *reinterpret_cast<const raw_t *>(qb + off);
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const uint32_t off = FIXED ? v_off[j] : v_offset(t, j);
      if constexpr (BF16)
        rv[j] = *reinterpret_cast<const uint16_t *>(vb + off);
      else
        rv[j] = *reinterpret_cast<const uint32_t *>(vb + off);
    }
    ra = *reinterpret_cast<const float *>(ab + ab_off);
    rb = *reinterpret_cast<const float *>(bb + ab_off);
  };
  auto deposit = [&](int buf) {
#pragma unroll
    for (int j = 0; j < KQ_PER; ++j) {
      const int g = tid + j * kThreads;
      if (KQ_ITEMS % kThreads == 0 || g < KQ_ITEMS) {
        const int off = (g / GROUPS) * D + stage_slot<D, L>(g % GROUPS);
        *reinterpret_cast<float4 *>(&SK(buf)[off]) = widen4<BF16>(rk[j]);
        *reinterpret_cast<float4 *>(&SQ(buf)[off]) = widen4<BF16>(rq[j]);
      }
    }
#pragma unroll
    for (int j = 0; j < V_PER; ++j) {
      const int e = tid + j * kThreads;
      if (V_ITEMS % kThreads == 0 || e < V_ITEMS) sv[buf][e] = widen1<BF16>(rv[j]);
    }
    if (tid < TS) {
      sa[buf][tid] = ra;
      sb[buf][tid] = rb;
    }
  };
  auto write_o = [&](int64_t t0, int nt, int buf) {
    if constexpr (SO_BUFS == 1) {
      // this wave's own rows (64 / L of them) for every token of the stage
      constexpr int RW = 64 / L;
      const int wave = tid / 64, wl = tid % 64;
#pragma unroll
      for (int j = 0; j < TS * RW / 64; ++j) {
        const int e = wl + 64 * j, tt = e / RW, r = wave * RW + e % RW;
        if (tt < nt && r0 + r < dv)
          p.o[(bos + t0 + tt) * vstride + (int64_t)h * dv + r0 + r] = so[0][tt * ROWS + r];
      }
    } else if (nt == TS) {  // full stage: scalar base plus the 32-bit offsets
      char *ob = reinterpret_cast<char *>(p.o + (bos + t0) * vstride);
      const int t = opaque_tid();
#pragma unroll
      for (int j = 0; j < V_PER; ++j)
        if (FIXED ? o_ok[j] : o_store_ok(t, j))
          *reinterpret_cast<float *>(ob + (FIXED ? o_off[j] : o_offset(t, j))) =
              so[buf][tid + j * kThreads];
    } else {
#pragma unroll
      for (int j = 0; j < V_PER; ++j) {
        const int e = tid + j * kThreads;
        const int tt = e / ROWS, r = e % ROWS;
        if ((V_ITEMS % kThreads == 0 || e < V_ITEMS) && tt < nt && r0 + r < dv)
          p.o[(bos + t0 + tt) * vstride + (int64_t)h * dv + r0 + r] = so[buf][e];
      }
    }
  };
  // o of token tt of the stage for the group's row rr, into the coalescing buffer
  auto store_o = [&](int buf, int tt, int rr, float value) {
    so[SO_BUFS == 1 ? 0 : buf][tt * ROWS + row + GR * rr] = value;
  };
  // One token of a stage, in row_token's order of operations (decay, key dot, delta,
  // update, readout) on each of the group's R rows, whose dots run side by side and share
  // the k and q read from LDS; q is read only once k is no longer needed, so the two are
  // never held together. Every lane of a row holds the same o_i and stores it (no branch),
  // which keeps an unrolled stage in one basic block.
  auto run_token = [&](int buf, int tt) {
    float kr[M], qr[M], x[R][M], y[R][M], r[R];
    lds_slice<D, L>(&SK(buf)[tt * D], lane, kr);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) {
      row_decay<D, L>(s[rr], sa[buf][tt], x[rr]);
#pragma unroll
      for (int e = 0; e < M; ++e) y[rr][e] = kr[e];
    }
    contract_dots<D, L, R>(x, y, r);
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
      row_update<D, L>(s[rr], row_delta(sb[buf][tt], sv[buf][tt * ROWS + row + GR * rr], r[rr]),
                       kr, x[rr]);
    lds_slice<D, L>(&SQ(buf)[tt * D], lane, qr);
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
#pragma unroll
      for (int e = 0; e < M; ++e) y[rr][e] = qr[e];
    contract_dots<D, L, R>(s, y, r);
#pragma unroll
    for (int rr = 0; rr < R; ++rr) store_o(buf, tt, rr, r[rr]);
  };

  // A full stage, software-pipelined: the inputs of token t+2 are read from LDS while token
  // t computes (a three-slot register ring), and token t's readout dot runs side by side
  // with token t+1's key dot (both read only the state after token t). Every operation is
  // one that row_token performs, on the same operands; only independent operations are
  // interleaved, so the bits are the same. Used where few waves share a SIMD and latency,
  // not issue, bounds the stage.
  auto run_stage_pipelined = [&](int buf, float (&snap)[SNAPS][M]) {
    float(&s)[M] = s_first;
    float rk_[3][M], rq_[3][M], ra_[3], rb_[3], rv_[3], x[M];
    auto load_token = [&](int tt, int slot) {
      lds_slice<D, L>(&SK(buf)[tt * D], lane, rk_[slot]);
      lds_slice<D, L>(&SQ(buf)[tt * D], lane, rq_[slot]);
      ra_[slot] = sa[buf][tt];
      rb_[slot] = sb[buf][tt];
      rv_[slot] = sv[buf][tt * ROWS + row];
    };
    load_token(0, 0);
    load_token(1, 1);
    row_decay<D, L>(s, ra_[0], x);
    float u = contract_dot<D, L>(x, rk_[0]);
#pragma unroll
    for (int tt = 0; tt < TS; ++tt) {
      const int cur = tt % 3, nxt = (tt + 1) % 3;
      if (tt + 2 < TS) load_token(tt + 2, (tt + 2) % 3);
      row_update<D, L>(s, row_delta(rb_[cur], rv_[cur], u), rk_[cur], x);
      if (INNER && tt % 16 == 15 && tt + 1 < TS) {  // the state at a possible chunk boundary
#pragma unroll
        for (int e = 0; e < M; ++e) snap[tt / 16][e] = s[e];
      }
      if (tt + 1 < TS) {
        row_decay<D, L>(s, ra_[nxt], x);
        float xs[2][M], ys[2][M], r[2];
#pragma unroll
        for (int e = 0; e < M; ++e) {
          xs[0][e] = s[e];
          ys[0][e] = rq_[cur][e];
          xs[1][e] = x[e];
          ys[1][e] = rk_[nxt][e];
        }
        contract_dots<D, L, 2>(xs, ys, r);
        store_o(buf, tt, 0, r[0]);
        u = r[1];
      } else {
        store_o(buf, tt, 0, contract_dot<D, L>(s, rq_[cur]));
      }
    }
  };

  // A chunk boundary (j + 1) % C == 0 falls on a token 16 m - 1 of a stage (see TS above).
  // `done` = tokens absorbed.
  const int chunk_shift = __builtin_ctz((unsigned)p.chunk);
  auto store_chunk_state = [&](int64_t done, int rr, const float (&st)[M]) {
    if constexpr (MODE == kTrainer) {
      if ((done & (p.chunk - 1)) == 0) {
        const int64_t c = cbase + (done >> chunk_shift) - 1;
        if (valid[rr] && c >= 0 && c < p.total_chunks)
          store_row<M>(p.chunk_states + ((c * Hv + h) * dv + irow[rr]) * D + lane * M, st);
      }
    }
  };
  auto store_chunk_states = [&](int64_t done) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr) store_chunk_state(done, rr, s[rr]);
  };
  const int64_t nstages = (Tn + TS - 1) / TS;

  if (Tn > 0) {
    if (Tn >= TS)
      fetch_full(0);
    else
      fetch(0);
    deposit(0);
  }
  __syncthreads();
  // Full stages in the loop; a sequence's last stage, if partial, after it. Keeping the
  // partial stage's token loop out of the stage loop lets the state stay in one set of
  // registers across stages (with both in the loop the compiler copied the state in and
  // out of the full stage, 128 moves per stage at 4 lanes per row and two rows per group).
  const int64_t nfull = Tn / TS;
  for (int64_t st = 0; st < nfull; ++st) {
    const int buf = (int)(st & 1);
    const int64_t t0 = st * TS;
    const bool more = st + 1 < nstages;
    if (more) {  // global loads in flight while this stage computes
      if (t0 + 2 * TS <= Tn)
        fetch_full(t0 + TS);
      else
        fetch(t0 + TS);
    }
    if constexpr (L >= 8) {
      float snap[SNAPS][M];
      run_stage_pipelined(buf, snap);
      if constexpr (INNER) {
#pragma unroll
        for (int m = 0; m + 1 < TS / 16; ++m) store_chunk_state(t0 + 16 * (m + 1), 0, snap[m]);
      }
    } else {
#pragma unroll
      for (int tt = 0; tt < TS; ++tt) run_token(buf, tt);
    }
    store_chunk_states(t0 + TS);
    if (more) deposit(buf ^ 1);
    __syncthreads();
    write_o(t0, TS, buf);
  }
  if (nfull < nstages) {  // the last stage, partial: its inputs were deposited already
    const int buf = (int)(nfull & 1);
    const int64_t t0 = nfull * TS;
    const int nt = (int)(Tn - t0);
#pragma unroll 1
    for (int tt = 0; tt < nt; ++tt) {
      run_token(buf, tt);
      store_chunk_states(t0 + tt + 1);
    }
    __syncthreads();
    write_o(t0, nt, buf);
  }
  if constexpr (MODE == kPrefill) {
#pragma unroll
    for (int rr = 0; rr < R; ++rr)
      if (valid[rr]) store_row<M>(p.final_state + row_off[rr], s[rr]);
  }
}

// On 32 lanes per row each group of lanes holds two rows, g and g + 8 of a 16-row block, so
// that a wave keeps as many bytes in flight as on 16 lanes (one 16-byte load per lane and
// row, each load instruction covering two whole rows).
constexpr int decode_rows_per_group(int L) { return L == 32 ? 2 : 1; }

template <int D, int L, bool BF16>
__global__ __launch_bounds__(kThreads) void cpr_decode_kernel(const DecodeArgs p) {
  constexpr int R = decode_rows_per_group(L);
  constexpr int GR = kThreads / L;
  constexpr int ROWS = R * GR;
  constexpr int M = D / L;
  const int tid = threadIdx.x, row = tid / L, lane = tid % L;
  const int Hv = p.num_v_heads, Hk = p.num_qk_heads, dv = p.d_v;
  const int rblocks = (dv + ROWS - 1) / ROWS;
  int pair, rblock;
  block_work(blockIdx.x, p.num_seqs * Hv, rblocks, Hv / Hk, pair, rblock);
  const int n = pair / Hv;
  const int h = pair % Hv;
  const int pos = p.pos[n];
  if (pos < 0) return;  // idle slot: uniform over the workgroup
  const int hk = h / (Hv / Hk);

  float kr[M], qr[M];
  const int64_t qk_off = ((int64_t)n * Hk + hk) * D + lane * M;
  load_input<M, BF16>(p.k, qk_off, kr);
  load_input<M, BF16>(p.q, qk_off, qr);
  const int64_t nh = (int64_t)n * Hv + h;
  const float a = p.a[nh], b = p.b[nh];
  int i[R];
  bool valid[R];
  float v_i[R], s[R][M], oi[R];
  int64_t row_off[R];
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    i[rr] = rblock * ROWS + row + GR * rr;
    valid[rr] = i[rr] < dv;
    row_off[rr] = (nh * dv + i[rr]) * D + lane * M;
    if constexpr (L == 32) {
      // Rows past d_v load (and compute on) the last row, so that every load is issued
      // unconditionally and both rows' loads are in flight together (measured 187 against
      // 210 us per step on the engine_decode workload with the loads behind branches);
      // only valid rows store.
      const int ic = valid[rr] ? i[rr] : dv - 1;
      v_i[rr] = load1<BF16>(p.v, nh * dv + ic);
      load_row<M>(p.state + (nh * dv + ic) * D + lane * M, s[rr]);
    } else {
      v_i[rr] = valid[rr] ? load1<BF16>(p.v, nh * dv + i[rr]) : 0.0f;
      if (valid[rr]) {
        load_row<M>(p.state + row_off[rr], s[rr]);
      } else {
#pragma unroll
        for (int e = 0; e < M; ++e) s[rr][e] = 0.0f;
      }
    }
  }
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if constexpr (L == 32)
      oi[rr] = row_token_split<D>(s[rr], a, b, v_i[rr], kr, qr);
    else
      oi[rr] = row_token<D, L>(s[rr], a, b, v_i[rr], kr, qr);
  }
  const bool resync = p.resync_states && (((int64_t)pos + 1) & (p.chunk - 1)) == 0;
#pragma unroll
  for (int rr = 0; rr < R; ++rr) {
    if (valid[rr]) {
      store_row<M>(p.state + row_off[rr], s[rr]);
      if (lane == 0) p.o[nh * dv + i[rr]] = oi[rr];
      if (resync) store_row<M>(p.resync_states + row_off[rr], s[rr]);
    }
  }
}

// ---------------------------------------------------------------------------- launchers

template <typename Args>
hipError_t launch(const void *fn, int64_t grid, Args args, hipStream_t stream,
                  int threads = kThreads) {
  if (grid <= 0) return hipSuccess;
  void *kargs[] = {&args};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(threads), kargs, 0, stream);
}

template <int D, int L, int TS, int NT = kThreads, int R = 1>
hipError_t scan_dl(const ScanArgs &a, hipStream_t st) {
  const int64_t grid = scan_grid(a, L, NT, R);
  const void *fn;
  if constexpr (NT == 512) {  // bf16, d_v a multiple of 32; a trainer launch needs C >= TS
    if (!a.bf16 || a.d_v % 32 != 0 || (a.mode == kTrainer && a.chunk < TS))
      return hipErrorInvalidValue;
    fn = a.mode == kTrainer ? (const void *)cpr_scan_kernel<D, L, TS, true, kTrainer, NT, R>
                            : (const void *)cpr_scan_kernel<D, L, TS, true, kPrefill, NT, R>;
  } else if constexpr (TS > 32) {  // bf16 inputs only; a trainer launch needs C >= TS
    if (!a.bf16 || (a.mode == kTrainer && a.chunk < TS)) return hipErrorInvalidValue;
    fn = a.mode == kTrainer ? (const void *)cpr_scan_kernel<D, L, TS, true, kTrainer, NT, R>
                            : (const void *)cpr_scan_kernel<D, L, TS, true, kPrefill, NT, R>;
  } else if (a.mode == kTrainer) {
    fn = a.bf16 ? (const void *)cpr_scan_kernel<D, L, TS, true, kTrainer, NT, R>
                : (const void *)cpr_scan_kernel<D, L, TS, false, kTrainer, NT, R>;
  } else {
    fn = a.bf16 ? (const void *)cpr_scan_kernel<D, L, TS, true, kPrefill, NT, R>
                : (const void *)cpr_scan_kernel<D, L, TS, false, kPrefill, NT, R>;
  }
  return launch(fn, grid, a, st, NT);
}

template <int D, int L>
hipError_t decode_dl(const DecodeArgs &a, hipStream_t st) {
  const void *fn = a.bf16 ? (const void *)cpr_decode_kernel<D, L, true>
                          : (const void *)cpr_decode_kernel<D, L, false>;
  return launch(fn, decode_grid(a, L), a, st);
}

template <int D>
hipError_t scan_d(const ScanArgs &a, int L, int TS, int NT, int R, hipStream_t st) {
  if (R == 2)
    return L == 4 && TS == 16 && NT == 256 ? scan_dl<D, 4, 16, 256, 2>(a, st)
                                           : hipErrorInvalidValue;
  if (R != 1) return hipErrorInvalidValue;
  if (NT == 512) return L == 16 && TS == 64 ? scan_dl<D, 16, 64, 512>(a, st) : hipErrorInvalidValue;
  if (L == 16 && TS == 64 && a.bf16) return scan_dl<D, 16, 64>(a, st);
  if (L == 16 && TS == 32) return scan_dl<D, 16, 32>(a, st);
  if (L == 8 && TS == 32) return scan_dl<D, 8, 32>(a, st);
  if (L == 4 && TS == 16) return scan_dl<D, 4, 16>(a, st);
  return hipErrorInvalidValue;
}

template <int D>
hipError_t decode_d(const DecodeArgs &a, int L, hipStream_t st) {
  if constexpr (D >= 32) {
    if (L == 32) return decode_dl<D, 32>(a, st);
  }
  switch (L) {
    case 16: return decode_dl<D, 16>(a, st);
    case 8: return decode_dl<D, 8>(a, st);
    case 4: return decode_dl<D, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t scan_grid(const ScanArgs &a, int L, int threads, int rows_per_group) {
  const int64_t rows = (int64_t)rows_per_group * (threads / L);
  return (int64_t)a.num_seqs * a.num_v_heads * ((a.d_v + rows - 1) / rows);
}

int64_t decode_grid(const DecodeArgs &a, int L) {
  const int64_t rows = decode_rows_per_group(L) * (kThreads / L);
  return (int64_t)a.num_seqs * a.num_v_heads * ((a.d_v + rows - 1) / rows);
}

hipError_t launch_scan(const ScanArgs &a, int L, int TS, int threads, int rows_per_group,
                       hipStream_t st) {
  switch (a.d_k) {
    case 16: return scan_d<16>(a, L, TS, threads, rows_per_group, st);
    case 32: return scan_d<32>(a, L, TS, threads, rows_per_group, st);
    case 64: return scan_d<64>(a, L, TS, threads, rows_per_group, st);
    case 128: return scan_d<128>(a, L, TS, threads, rows_per_group, st);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode(const DecodeArgs &a, int L, hipStream_t st) {
  switch (a.d_k) {
    case 16: return decode_d<16>(a, L, st);
    case 32: return decode_d<32>(a, L, st);
    case 64: return decode_d<64>(a, L, st);
    case 128: return decode_d<128>(a, L, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdn
