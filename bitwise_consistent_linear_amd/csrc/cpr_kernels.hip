// HIP kernels for CPR Gated DeltaNet on gfx950: the packed-batch scan (trainer_fwd and
// engine_prefill) and the one-token decode step.
//
// Work decomposition: every state row (sequence n, value head h, row i) evolves on its own
// (the gated delta rule updates S row by row: row i only sees v_i). A workgroup of 256
// threads owns ROWS = 256/L consecutive rows of one (n, h); each row sits in the VGPRs of
// L lanes (cpr_row.hpp). No MFMA: each token is a matrix-vector step on a d_k x d_v state
// whose every element is touched four times, not a dense contraction.
//
// Scan: tokens are staged 16 at a time - q and k of the (n, q/k head) in the order the
// lanes read them, v of the workgroup's rows, a and b - into LDS as binary32 (bf16 widened
// exactly) with coalesced loads; the token loop then runs from LDS and registers only. The
// outputs o of a stage go back through LDS so that each token's ROWS values are stored
// contiguously. Chunk-boundary states (trainer) and the final state (prefill) are stored
// straight from the registers, each lane its contiguous slice of the row.
//
// Decode: one launch per step; each row's d_k floats are read from HBM, updated once and
// written back (plus the resync checkpoint on C-token boundaries).
//
// Scheduling: workgroups of the longest sequences are dispatched first (for up to 1024
// sequences the rank of every sequence by length is computed in LDS), so that the long
// serial scans overlap with the short ones.

#include "cpr_row.hpp"
#include "internal.h"

namespace gdn {
namespace {

constexpr int kThreads = 256;
constexpr int kStageTokens = 16;
constexpr int kMaxRankedSeqs = 1024;

// ---------------------------------------------------------------------- loads and stores

template <bool BF16>
__device__ __forceinline__ float load1(const void *base, int64_t idx) {
  if constexpr (BF16)
    return __uint_as_float((uint32_t)static_cast<const uint16_t *>(base)[idx] << 16);
  else
    return static_cast<const float *>(base)[idx];
}

// Four consecutive input elements starting at idx (idx % 4 == 0), widened to binary32.
template <bool BF16>
__device__ __forceinline__ float4 load4(const void *base, int64_t idx) {
  if constexpr (BF16) {
    const uint2 w = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
    return make_float4(__uint_as_float(w.x << 16), __uint_as_float(w.x & 0xFFFF0000u),
                       __uint_as_float(w.y << 16), __uint_as_float(w.y & 0xFFFF0000u));
  } else {
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
  }
}

template <int M, bool BF16>
__device__ __forceinline__ void load_input(const void *base, int64_t idx, float (&r)[M]) {
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int g = 0; g < M / 4; ++g) {
      const float4 x = load4<BF16>(base, idx + 4 * g);
      r[4 * g] = x.x; r[4 * g + 1] = x.y; r[4 * g + 2] = x.z; r[4 * g + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) r[e] = load1<BF16>(base, idx + e);
  }
}

template <int M>
__device__ __forceinline__ void load_row(const float *src, float (&r)[M]) {
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int g = 0; g < M / 4; ++g) {
      const float4 x = reinterpret_cast<const float4 *>(src)[g];
      r[4 * g] = x.x; r[4 * g + 1] = x.y; r[4 * g + 2] = x.z; r[4 * g + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) r[e] = src[e];
  }
}

template <int M>
__device__ __forceinline__ void store_row(float *dst, const float (&r)[M]) {
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int g = 0; g < M / 4; ++g)
      reinterpret_cast<float4 *>(dst)[g] =
          make_float4(r[4 * g], r[4 * g + 1], r[4 * g + 2], r[4 * g + 3]);
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) dst[e] = r[e];
  }
}

// LDS layout of one staged k or q vector (D floats). When a lane's slice (M floats) is a
// whole number of float4, group g of lane l sits at float4 slot g*L + l, so one ds_read_b128
// per group covers L*16 contiguous bytes across the lanes of a row; otherwise plain order.
template <int D, int L>
__device__ __forceinline__ int stage_slot(int c) {  // float offset of logical floats 4c..4c+3
  constexpr int M = D / L;
  if constexpr (M % 4 == 0) {
    const int e = 4 * c;
    return (((e % M) / 4) * L + e / M) * 4;
  } else {
    return 4 * c;
  }
}

template <int D, int L>
__device__ __forceinline__ void lds_slice(const float *vec, int lane, float (&r)[D / L]) {
  constexpr int M = D / L;
  if constexpr (M % 4 == 0) {
#pragma unroll
    for (int g = 0; g < M / 4; ++g) {
      const float4 x = *reinterpret_cast<const float4 *>(vec + (g * L + lane) * 4);
      r[4 * g] = x.x; r[4 * g + 1] = x.y; r[4 * g + 2] = x.z; r[4 * g + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) r[e] = vec[lane * M + e];
  }
}

// --------------------------------------------------------------------------- scheduling

// Token range of sequence n, clamped to [0, T) so that bad cu_seqlens cannot address
// outside the buffers.
__device__ __forceinline__ void seq_range(const int32_t *cu, int n, int64_t T, int64_t &bos,
                                          int64_t &eos) {
  int64_t lo = cu[n], hi = cu[n + 1];
  lo = lo < 0 ? 0 : (lo > T ? T : lo);
  hi = hi < lo ? lo : (hi > T ? T : hi);
  bos = lo;
  eos = hi;
}

// The sequence of the given rank when sequences are ordered by decreasing length (ties by
// index); natural order beyond kMaxRankedSeqs sequences. Uniform over the workgroup.
__device__ int ranked_sequence(const int32_t *cu, int N, int64_t T, int rank, int *s_len,
                               int *s_pick) {
  if (N > kMaxRankedSeqs) return rank;
  for (int j = threadIdx.x; j < N; j += blockDim.x) {
    int64_t b, e;
    seq_range(cu, j, T, b, e);
    s_len[j] = (int)(e - b);
  }
  if (threadIdx.x == 0) *s_pick = rank;  // overwritten below: ranks are a permutation
  __syncthreads();
  for (int j = threadIdx.x; j < N; j += blockDim.x) {
    const int lj = s_len[j];
    int r = 0;
    for (int m = 0; m < N; ++m) {
      const int lm = s_len[m];
      r += (lm > lj) | ((lm == lj) & (m < j));
    }
    if (r == rank) *s_pick = j;
  }
  __syncthreads();
  return *s_pick;
}

// Index of sequence n's first chunk-boundary state: sum over m < n of floor(T_m / C).
__device__ int64_t first_chunk_slot(const int32_t *cu, int n, int64_t T, int C, int *s_acc) {
  if (threadIdx.x == 0) *s_acc = 0;
  __syncthreads();
  int local = 0;
  for (int m = threadIdx.x; m < n; m += blockDim.x) {
    int64_t b, e;
    seq_range(cu, m, T, b, e);
    local += (int)((e - b) / C);
  }
  atomicAdd(s_acc, local);
  __syncthreads();
  return *s_acc;
}

// ----------------------------------------------------------------------------- kernels

template <int D, int L, bool BF16, int MODE>
__global__ __launch_bounds__(kThreads) void cpr_scan_kernel(const ScanArgs p) {
  constexpr int ROWS = kThreads / L;
  constexpr int M = D / L;
  constexpr int TS = kStageTokens;
  constexpr int GROUPS = D / 4;  // float4 groups per staged k or q vector
  __shared__ __align__(16) float sk[TS * D];
  __shared__ __align__(16) float sq[TS * D];
  __shared__ float sv[TS * ROWS];
  __shared__ float so[TS * ROWS];
  __shared__ float sa[TS], sb[TS];
  __shared__ int s_len[kMaxRankedSeqs];
  __shared__ int s_pick, s_acc;

  const int tid = threadIdx.x, row = tid / L, lane = tid % L;
  const int Hv = p.num_v_heads, Hk = p.num_qk_heads, dv = p.d_v;
  const int rblocks = (dv + ROWS - 1) / ROWS;
  const int per_seq = Hv * rblocks;
  const int rank = blockIdx.x / per_seq;
  const int h = (blockIdx.x % per_seq) / rblocks;
  const int r0 = (blockIdx.x % rblocks) * ROWS;
  const int64_t T = p.total_tokens;

  const int n = ranked_sequence(p.cu_seqlens, p.num_seqs, T, rank, s_len, &s_pick);
  int64_t bos, eos;
  seq_range(p.cu_seqlens, n, T, bos, eos);
  const int64_t Tn = eos - bos;
  int64_t cbase = 0;
  if constexpr (MODE == kTrainer) cbase = first_chunk_slot(p.cu_seqlens, n, T, p.chunk, &s_acc);

  const int hk = h / (Hv / Hk);
  const int i = r0 + row;
  const bool valid = i < dv;
  const int64_t row_off = (((int64_t)n * Hv + h) * dv + i) * D + lane * M;
  const int64_t vstride = (int64_t)Hv * dv;

  float s[M];
  if (p.initial_state && valid) {
    load_row<M>(p.initial_state + row_off, s);
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) s[e] = 0.0f;
  }

  auto stage = [&](int64_t t0, int nt) {
    for (int g = tid; g < nt * GROUPS; g += kThreads) {
      const int tt = g / GROUPS, c = g % GROUPS;
      const int64_t src = ((bos + t0 + tt) * Hk + hk) * D + 4 * c;
      *reinterpret_cast<float4 *>(sk + tt * D + stage_slot<D, L>(c)) = load4<BF16>(p.k, src);
      *reinterpret_cast<float4 *>(sq + tt * D + stage_slot<D, L>(c)) = load4<BF16>(p.q, src);
    }
    for (int e = tid; e < nt * ROWS; e += kThreads) {
      const int tt = e / ROWS, r = e % ROWS;
      sv[e] = (r0 + r < dv) ? load1<BF16>(p.v, (bos + t0 + tt) * vstride + (int64_t)h * dv + r0 + r)
                            : 0.0f;
    }
    for (int tt = tid; tt < nt; tt += kThreads) {
      const int64_t ab = (bos + t0 + tt) * Hv + h;
      sa[tt] = p.a[ab];
      sb[tt] = p.b[ab];
    }
  };

  auto write_o = [&](int64_t t0, int nt) {
    for (int e = tid; e < nt * ROWS; e += kThreads) {
      const int tt = e / ROWS, r = e % ROWS;
      if (r0 + r < dv) p.o[(bos + t0 + tt) * vstride + (int64_t)h * dv + r0 + r] = so[e];
    }
  };

  auto step = [&](int tt) {
    float kr[M], qr[M];
    lds_slice<D, L>(sk + tt * D, lane, kr);
    lds_slice<D, L>(sq + tt * D, lane, qr);
    const float oi = row_token<D, L>(s, sa[tt], sb[tt], sv[tt * ROWS + row], kr, qr);
    if (lane == 0) so[tt * ROWS + row] = oi;
  };

  // Every admitted C is a multiple of the stage length and stages start at in-sequence
  // index 0, so a chunk boundary (j + 1) % C == 0 can only be the last token of a full stage.
  static_assert(16 % TS == 0, "stage length must divide every admitted chunk size");
  const int chunk_shift = __builtin_ctz((unsigned)p.chunk);

  if (Tn > 0) stage(0, (int)(Tn < TS ? Tn : TS));
  __syncthreads();
  for (int64_t t0 = 0; t0 < Tn; t0 += TS) {
    const int nt = (int)(Tn - t0 < TS ? Tn - t0 : TS);
    if (nt == TS) {
#pragma unroll
      for (int tt = 0; tt < TS; ++tt) step(tt);
      if constexpr (MODE == kTrainer) {
        const int64_t done = t0 + TS;  // tokens absorbed
        if ((done & (p.chunk - 1)) == 0) {
          const int64_t c = cbase + (done >> chunk_shift) - 1;
          if (valid && c < p.total_chunks)
            store_row<M>(p.chunk_states + ((c * Hv + h) * dv + i) * D + lane * M, s);
        }
      }
    } else {
      for (int tt = 0; tt < nt; ++tt) step(tt);
    }
    __syncthreads();
    write_o(t0, nt);
    if (t0 + TS < Tn) stage(t0 + TS, (int)(Tn - t0 - TS < TS ? Tn - t0 - TS : TS));
    __syncthreads();
  }
  if constexpr (MODE == kPrefill) {
    if (valid) store_row<M>(p.final_state + row_off, s);
  }
}

template <int D, int L, bool BF16>
__global__ __launch_bounds__(kThreads) void cpr_decode_kernel(const DecodeArgs p) {
  constexpr int ROWS = kThreads / L;
  constexpr int M = D / L;
  const int tid = threadIdx.x, row = tid / L, lane = tid % L;
  const int Hv = p.num_v_heads, Hk = p.num_qk_heads, dv = p.d_v;
  const int rblocks = (dv + ROWS - 1) / ROWS;
  const int per_seq = Hv * rblocks;
  const int n = blockIdx.x / per_seq;
  const int h = (blockIdx.x % per_seq) / rblocks;
  const int i = (blockIdx.x % rblocks) * ROWS + row;
  const int pos = p.pos[n];
  if (pos < 0) return;  // idle slot: uniform over the workgroup
  const bool valid = i < dv;
  const int hk = h / (Hv / Hk);

  float kr[M], qr[M];
  const int64_t qk_off = ((int64_t)n * Hk + hk) * D + lane * M;
  load_input<M, BF16>(p.k, qk_off, kr);
  load_input<M, BF16>(p.q, qk_off, qr);
  const int64_t nh = (int64_t)n * Hv + h;
  const float a = p.a[nh], b = p.b[nh];
  const float v_i = valid ? load1<BF16>(p.v, nh * dv + i) : 0.0f;
  const int64_t row_off = (nh * dv + i) * D + lane * M;
  float s[M];
  if (valid) {
    load_row<M>(p.state + row_off, s);
  } else {
#pragma unroll
    for (int e = 0; e < M; ++e) s[e] = 0.0f;
  }
  const float oi = row_token<D, L>(s, a, b, v_i, kr, qr);
  if (valid) {
    store_row<M>(p.state + row_off, s);
    if (lane == 0) p.o[nh * dv + i] = oi;
    if (p.resync_states && (((int64_t)pos + 1) & (p.chunk - 1)) == 0)
      store_row<M>(p.resync_states + row_off, s);
  }
}

// ---------------------------------------------------------------------------- launchers

template <typename Args>
hipError_t launch(const void *fn, int64_t grid, Args args, hipStream_t stream) {
  if (grid <= 0) return hipSuccess;
  void *kargs[] = {&args};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

template <int D, int L>
hipError_t scan_dl(const ScanArgs &a, hipStream_t st) {
  const int64_t grid = scan_grid(a, L);
  const bool trainer = a.mode == kTrainer;
  const void *fn;
  if (a.bf16)
    fn = trainer ? (const void *)cpr_scan_kernel<D, L, true, kTrainer>
                 : (const void *)cpr_scan_kernel<D, L, true, kPrefill>;
  else
    fn = trainer ? (const void *)cpr_scan_kernel<D, L, false, kTrainer>
                 : (const void *)cpr_scan_kernel<D, L, false, kPrefill>;
  return launch(fn, grid, a, st);
}

template <int D, int L>
hipError_t decode_dl(const DecodeArgs &a, hipStream_t st) {
  const void *fn = a.bf16 ? (const void *)cpr_decode_kernel<D, L, true>
                          : (const void *)cpr_decode_kernel<D, L, false>;
  return launch(fn, decode_grid(a, L), a, st);
}

template <int D>
hipError_t scan_d(const ScanArgs &a, int L, hipStream_t st) {
  switch (L) {
    case 16: return scan_dl<D, 16>(a, st);
    case 8: return scan_dl<D, 8>(a, st);
    case 4: return scan_dl<D, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

template <int D>
hipError_t decode_d(const DecodeArgs &a, int L, hipStream_t st) {
  switch (L) {
    case 16: return decode_dl<D, 16>(a, st);
    case 8: return decode_dl<D, 8>(a, st);
    case 4: return decode_dl<D, 4>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

int64_t scan_grid(const ScanArgs &a, int L) {
  const int64_t rows = kThreads / L;
  return (int64_t)a.num_seqs * a.num_v_heads * ((a.d_v + rows - 1) / rows);
}

int64_t decode_grid(const DecodeArgs &a, int L) {
  const int64_t rows = kThreads / L;
  return (int64_t)a.num_seqs * a.num_v_heads * ((a.d_v + rows - 1) / rows);
}

hipError_t launch_scan(const ScanArgs &a, int L, hipStream_t st) {
  switch (a.d_k) {
    case 16: return scan_d<16>(a, L, st);
    case 32: return scan_d<32>(a, L, st);
    case 64: return scan_d<64>(a, L, st);
    case 128: return scan_d<128>(a, L, st);
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
