// Device helpers shared by the forward and backward kernels: input loads (bf16 widened
// exactly), state-row transfers, the LDS layout of staged k/q vectors, and the mapping of
// workgroups to sequences and head pairs.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace gdn {
namespace io {

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
__host__ __device__ __forceinline__ void seq_range(const int32_t *cu, int n, int64_t T,
                                                   int64_t &bos, int64_t &eos) {
  int64_t lo = cu[n], hi = cu[n + 1];
  lo = lo < 0 ? 0 : (lo > T ? T : lo);
  hi = hi < lo ? lo : (hi > T ? T : hi);
  bos = lo;
  eos = hi;
}

// The sequence of the given rank when sequences are ordered by decreasing length (ties by
// index); natural order beyond kMaxRankedSeqs sequences. Uniform over the workgroup.
__device__ inline int ranked_sequence(const int32_t *cu, int N, int64_t T, int rank, int *s_len,
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
  return __builtin_amdgcn_readfirstlane(*s_pick);  // the same in every lane: keep it scalar
}

// Workgroup -> (head pair, row block), XCD-aware. The dispatcher hands workgroups to the
// 8 XCDs (each with its own L2) in round-robin order of workgroup id. A pair is one
// sequence (in scheduling order) and value head; pair = unit * G + g, where a unit is one
// sequence and q/k head and g runs over the G value heads that share that q/k head. Units
// are taken 8 at a time; within such a group, unit u*8+x gets every workgroup id congruent
// to x mod 8, so all row blocks of all G heads of a unit run on one XCD and read its q, k
// (and each head's a and b) through one L2; consecutive workgroups of a unit alternate
// between its heads, so the heads advance through the tokens side by side. A last group of
// fewer than 8 units is laid out linearly. A bijection from [0, pairs * rblocks) onto
// (pair, row block) for any G dividing pairs.
constexpr int kXcds = 8;

__host__ __device__ __forceinline__ void block_work(int b, int pairs, int rblocks, int G,
                                                    int &pair, int &rb) {
  const int per_unit = G * rblocks, units = pairs / G;
  const int group = b / (kXcds * per_unit), within = b % (kXcds * per_unit);
  int unit, w;
  if (group < units / kXcds) {
    unit = group * kXcds + within % kXcds;
    w = within / kXcds;
  } else {
    unit = group * kXcds + within / per_unit;
    w = within % per_unit;
  }
  pair = unit * G + w % G;
  rb = w / G;
}

// The chunk slots of a packed batch, listed by one workgroup of 256 threads:
// plan[0] = slots used (at most slots_max); slot s holds (sequence, chunk) in
// plan[kPlanHeader + 2 s], plan[kPlanHeader + 2 s + 1], sequences in order, one slot per
// chunk including a last partial one; cbase[n] = sum over m < n of floor(T_m / C), the
// index of sequence n's first chunk state, clamped to total_chunks. The sums run in 64 bits:
// lengths come from device memory the host cannot check, and whatever they hold, every slot
// and base written stays inside its buffer.
constexpr int kPlanHeader = 4;

__device__ inline void chunk_plan(const int32_t *cu, int N, int64_t T, int C, int64_t total_chunks,
                                  int slots_max, int32_t *plan, int32_t *cbase) {
  constexpr int kThreads = 256;
  __shared__ int64_t s_ceil[kThreads], s_floor[kThreads];
  __shared__ int64_t s_carry_ceil, s_carry_floor;
  const int tid = threadIdx.x;
  if (tid == 0) {
    s_carry_ceil = 0;
    s_carry_floor = 0;
  }
  __syncthreads();
  for (int base = 0; base < N; base += kThreads) {
    const int m = base + tid;
    int64_t len = 0;
    if (m < N) {
      int64_t b, e;
      seq_range(cu, m, T, b, e);
      len = e - b;
    }
    const int64_t nc = (len + C - 1) / C, nf = len / C;
    s_ceil[tid] = nc;
    s_floor[tid] = nf;
    __syncthreads();
    for (int off = 1; off < kThreads; off *= 2) {  // inclusive scan
      const int64_t vc = tid >= off ? s_ceil[tid - off] : 0;
      const int64_t vf = tid >= off ? s_floor[tid - off] : 0;
      __syncthreads();
      s_ceil[tid] += vc;
      s_floor[tid] += vf;
      __syncthreads();
    }
    const int64_t ex_ceil = s_carry_ceil + s_ceil[tid] - nc;
    const int64_t ex_floor = s_carry_floor + s_floor[tid] - nf;
    if (m < N) {
      cbase[m] = (int32_t)(ex_floor < total_chunks ? ex_floor : total_chunks);
      for (int64_t c = 0; c < nc && ex_ceil + c < slots_max; ++c) {
        const int64_t slot = ex_ceil + c;
        plan[kPlanHeader + 2 * slot] = m;
        plan[kPlanHeader + 2 * slot + 1] = (int32_t)c;
      }
    }
    __syncthreads();
    if (tid == kThreads - 1) {
      s_carry_ceil += s_ceil[tid];
      s_carry_floor += s_floor[tid];
    }
    __syncthreads();
  }
  if (tid == 0) plan[0] = (int32_t)(s_carry_ceil < slots_max ? s_carry_ceil : slots_max);
}

// Full chunks of sequence m after clamping its range: floor(T_m / C) >= 0.
__host__ __device__ __forceinline__ unsigned long long full_chunks(const int32_t *cu, int m,
                                                                   int64_t T, int C) {
  int64_t b, e;
  seq_range(cu, m, T, b, e);  // e >= b
  return (unsigned long long)((e - b) / C);
}

// A sum of full_chunks terms as a chunk-state index in [0, total_chunks]. At most 2^31
// sequences of fewer than 2^31 tokens each, so the 64-bit sum cannot wrap.
__host__ __device__ __forceinline__ int64_t clamp_chunk_index(unsigned long long sum,
                                                              int64_t total_chunks) {
  return sum < (unsigned long long)total_chunks ? (int64_t)sum : total_chunks;
}

// Index of sequence n's first chunk-boundary state: sum over m < n of floor(T_m / C), in
// 64 bits and clamped to total_chunks. The lengths come from device memory the host cannot
// check; whatever they hold, the index is in [0, total_chunks].
__device__ inline int64_t first_chunk_slot(const int32_t *cu, int n, int64_t T, int C,
                                           int64_t total_chunks, unsigned long long *s_acc) {
  if (threadIdx.x == 0) *s_acc = 0;
  __syncthreads();
  unsigned long long local = 0;
  for (int m = threadIdx.x; m < n; m += blockDim.x) local += full_chunks(cu, m, T, C);
  atomicAdd(s_acc, local);
  __syncthreads();
  return clamp_chunk_index(*s_acc, total_chunks);
}

// Raw register copy of four input elements: bf16 stays packed until it is written to LDS.
template <bool BF16>
struct Raw4 {
  using type = float4;
};
template <>
struct Raw4<true> {
  using type = uint2;
};

template <bool BF16>
__device__ __forceinline__ typename Raw4<BF16>::type load_raw4(const void *base, int64_t idx) {
  if constexpr (BF16)
    return *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(base) + idx);
  else
    return *reinterpret_cast<const float4 *>(static_cast<const float *>(base) + idx);
}

// One input element kept raw (bf16 bits or binary32 bits) until it is written to LDS, so
// that no arithmetic on it forces the prefetch loads to complete early.
template <bool BF16>
__device__ __forceinline__ uint32_t load_raw1(const void *base, int64_t idx) {
  if constexpr (BF16)
    return static_cast<const uint16_t *>(base)[idx];
  else
    return __float_as_uint(static_cast<const float *>(base)[idx]);
}

template <bool BF16>
__device__ __forceinline__ float widen1(uint32_t r) {
  return __uint_as_float(BF16 ? r << 16 : r);
}

template <bool BF16>
__device__ __forceinline__ float4 widen4(typename Raw4<BF16>::type r) {
  if constexpr (BF16)
    return make_float4(__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xFFFF0000u),
                       __uint_as_float(r.y << 16), __uint_as_float(r.y & 0xFFFF0000u));
  else
    return r;
}

}  // namespace io
}  // namespace gdn
