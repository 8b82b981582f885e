// The linear region on gfx950: Y = X W, every output the contract dot of a row of X and a
// column of W (K split into 16 contiguous leaves; a leaf is the rounded product of its first
// pair followed by fused multiply-adds in ascending k; the 16 leaf sums added pairwise in
// natural order), on the matrix cores.
//
// gfx950's binary32 matrix instruction v_mfma_f32_32x32x2_f32 computes, for every output,
// fma(a[k+1], b[k+1], fma(a[k], b[k], c)): two fused steps in ascending k with the
// accumulator first, rounded to nearest even with denormals kept. So a leaf is a run of
// these instructions over its k range starting from an accumulator of -0.0 (fma(a, b, -0)
// is the rounded product a*b, the sign of an exact zero included), and the leaf sums are
// combined by the same pairwise tree as the gated delta rule's dots. The bits of Y[m, n]
// therefore depend on neither the tile, nor the number of rows M, nor the schedule.
//
// Workgroup: 8 waves, a 128 x 128 tile of Y; wave (wm, wn) owns rows 64 wm .. 64 wm + 63 and
// columns 32 wn .. 32 wn + 31 as two 32 x 32 blocks that share the B operand (two
// independent accumulator chains); two waves per SIMD. K is staged KS at a time into LDS as
// binary32, double-buffered, the next stage's global loads held in registers as loaded (bf16
// bits or binary32) while the current one computes: W k-major; X row-major with each row's
// even and odd k apart, so one 16-byte read gives a lane its A operands for four steps.
// KS = 64 for bf16 X and W when a leaf is whole 64-k stages and N is a multiple of 128 (one
// workgroup barrier per 64 k; 141 KiB of LDS; W's columns interleaved over the lanes so that
// its deposit is free of LDS bank conflicts), 32 otherwise. KS changes which instructions wait for which, never an
// operation or its operands, so both give the same bits.

#include <type_traits>

#include "internal.h"

namespace gdn {
namespace {

using f32x16 = float __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int TM = 128, TN = 128;  // workgroup tile
constexpr int kLeaves = 16;

__device__ __forceinline__ uint32_t comp(const uint4 &v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}
__device__ __forceinline__ float comp(const float4 &v, int c) {
  return c == 0 ? v.x : c == 1 ? v.y : c == 2 ? v.z : v.w;
}

// V consecutive inputs of one row, kept as loaded (bf16 bits or binary32) until they are
// written to LDS; get(e) widens element e exactly (e a compile-time index).
template <bool BF16, int V>
struct Run {
  static constexpr int NV = BF16 ? V / 8 : V / 4;
  using vec = std::conditional_t<BF16, uint4, float4>;
  vec r[NV];
  // elements [idx, idx + V) of base; the run is 16-byte aligned
  __device__ __forceinline__ void load(const void *base, int64_t idx) {
    const vec *src = BF16 ? reinterpret_cast<const vec *>(static_cast<const uint16_t *>(base) + idx)
                          : reinterpret_cast<const vec *>(static_cast<const float *>(base) + idx);
#pragma unroll
    for (int i = 0; i < NV; ++i) r[i] = src[i];
  }
  // element e from base[row + min(c0 + e, n - 1)]: columns past n repeat the last one
  __device__ __forceinline__ void load_clamped(const void *base, int64_t row, int64_t c0,
                                               int64_t n) {
    auto col = [&](int e) { return row + (c0 + e < n ? c0 + e : n - 1); };
    if constexpr (BF16) {
      const uint16_t *b = static_cast<const uint16_t *>(base);
      uint32_t w[V / 2];
#pragma unroll
      for (int e = 0; e < V / 2; ++e)
        w[e] = (uint32_t)b[col(2 * e)] | ((uint32_t)b[col(2 * e + 1)] << 16);
#pragma unroll
      for (int i = 0; i < NV; ++i) r[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    } else {
      const float *b = static_cast<const float *>(base);
      float f[V];
#pragma unroll
      for (int e = 0; e < V; ++e) f[e] = b[col(e)];
#pragma unroll
      for (int i = 0; i < NV; ++i) r[i] = make_float4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3]);
    }
  }
  __device__ __forceinline__ float get(int e) const {
    if constexpr (BF16) {
      const uint32_t w = comp(r[e / 8], (e % 8) / 2);
      return __uint_as_float(e % 2 == 0 ? w << 16 : w & 0xFFFF0000u);
    } else {
      return comp(r[e / 4], e % 4);
    }
  }
};

template <bool XBF16, bool WBF16, int KS>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_leaf_kernel(const LinearArgs p) {
  constexpr int QS = KS / 2 + 4, WS = TN + 4;  // LDS row strides (conflict-free reads)
  constexpr int XPT = TM * KS / kThreads;      // staged X values per thread (8 or 16)
  constexpr int WPT = KS * TN / kThreads;      // staged W values per thread (8 or 16)
  static_assert((KS == 32 || KS == 64) && XPT % 8 == 0 && WPT % 8 == 0, "staging shape");
  static_assert(KS == 32 || (XBF16 && WBF16), "64-k stages stage bf16 X and W");
  __shared__ __align__(16) float sx[2][2][TM][QS];  // sx[buf][k % 2][row][k / 2]
  __shared__ __align__(16) float sw[2][KS][WS];      // sw[buf][k][col]

  const int tid = threadIdx.x, wave = tid / 64, l = tid % 64;
  const int wm = wave / 4, wn = wave % 4;  // 2 x 4 waves of 64 x 32
  const int64_t M = p.m, N = p.n;
  const int K = p.k;
  const int64_t tiles_n = (N + TN - 1) / TN;
  const int64_t tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int64_t m0 = tile_m * TM, n0 = tile_n * TN;

  // staging: X tile [128 rows x KS k]: one row, XPT consecutive k per thread;
  //          W tile [KS k x 128 cols]: one k, WPT consecutive columns per thread
  const int xr = tid / (KS / XPT), xk = (tid % (KS / XPT)) * XPT;
  const int wk = tid / (TN / WPT), wc = (tid % (TN / WPT)) * WPT;
  const int64_t xrow = m0 + xr < M ? m0 + xr : M - 1;  // rows past M repeat the last row
  const bool w_vec = N % (WBF16 ? 8 : 4) == 0;           // every W row 16-byte aligned
  Run<XBF16, XPT> xv;
  Run<WBF16, WPT> wv;  // KS = 32
  // KS = 64 (bf16 W): lane c of a W row (eight lanes per row) holds columns 32 j + 4 c .. + 3,
  // j = 0 .. 3, so that each of the four 16-byte LDS writes of the deposit puts the row's
  // eight lanes in eight different groups of four banks (consecutive 16-column runs per
  // lane put them in two, a four-way conflict)
  uint2 wq[4];
  const int wcl = tid % (TN / WPT);
  auto fetch = [&](int k0) {
    xv.load(p.x, xrow * K + k0 + xk);
    const int64_t wrow = (int64_t)(k0 + wk) * N;
    if constexpr (KS == 64) {  // launched only for N a multiple of the tile: every column in range
#pragma unroll
      for (int j = 0; j < 4; ++j)
        wq[j] = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(p.w) + wrow + n0 +
                                                 32 * j + 4 * wcl);
    } else if (w_vec && n0 + wc + WPT <= N) {  // all columns in range, rows 16-byte aligned
      wv.load(p.w, wrow + n0 + wc);
    } else {
      wv.load_clamped(p.w, wrow, n0 + wc, N);
    }
  };
  auto deposit = [&](int buf) {
    // k = xk + e: even k to half 0, odd k to half 1, at position k / 2
#pragma unroll
    for (int h = 0; h < XPT / 8; ++h) {
      *reinterpret_cast<float4 *>(&sx[buf][0][xr][xk / 2 + 4 * h]) =
          make_float4(xv.get(8 * h), xv.get(8 * h + 2), xv.get(8 * h + 4), xv.get(8 * h + 6));
      *reinterpret_cast<float4 *>(&sx[buf][1][xr][xk / 2 + 4 * h]) =
          make_float4(xv.get(8 * h + 1), xv.get(8 * h + 3), xv.get(8 * h + 5), xv.get(8 * h + 7));
    }
    if constexpr (KS == 64) {
#pragma unroll
      for (int j = 0; j < 4; ++j)
        *reinterpret_cast<float4 *>(&sw[buf][wk][32 * j + 4 * wcl]) =
            make_float4(__uint_as_float(wq[j].x << 16), __uint_as_float(wq[j].x & 0xFFFF0000u),
                        __uint_as_float(wq[j].y << 16), __uint_as_float(wq[j].y & 0xFFFF0000u));
    } else {
#pragma unroll
      for (int e = 0; e < WPT; e += 4)
        *reinterpret_cast<float4 *>(&sw[buf][wk][wc + e]) =
            make_float4(wv.get(e), wv.get(e + 1), wv.get(e + 2), wv.get(e + 3));
    }
  };

  // per lane: A operands for both blocks (rows 64 wm + l%32 and 32 more, k = 2q + l/32), the
  // shared B operand (column 32 wn + l%32)
  const int arow = 64 * wm + l % 32, bcol = 32 * wn + l % 32, kl = l / 32;
  const int stages_per_leaf = K / (KS * kLeaves);  // KS * 16 divides K: a leaf is whole stages
  f32x16 acc0, acc1;              // the current leaf, blocks 0 and 1
  f32x16 t0[4], t1[4];            // pending subtrees: slot j holds a sum of 2^j leaves
  int leaf = 0;

  auto fold = [&]() {             // leaf `leaf` is complete: add it into the pairwise tree
    f32x16 x0 = acc0, x1 = acc1;
    if (leaf & 1) {
      x0 = t0[0] + x0; x1 = t1[0] + x1;
      if (leaf & 2) {
        x0 = t0[1] + x0; x1 = t1[1] + x1;
        if (leaf & 4) {
          x0 = t0[2] + x0; x1 = t1[2] + x1;
          if (leaf & 8) {
            x0 = t0[3] + x0; x1 = t1[3] + x1;  // leaf 15: the root
          }
          t0[3] = x0; t1[3] = x1;
        } else { t0[2] = x0; t1[2] = x1; }
      } else { t0[1] = x0; t1[1] = x1; }
    } else { t0[0] = x0; t1[0] = x1; }
    ++leaf;
  };

  const int stages = K / KS;
  fetch(0);
  deposit(0);
  __syncthreads();
  for (int s = 0, in_leaf = 0; s < stages; ++s) {
    const int buf = s & 1;
    if (s + 1 < stages) fetch((s + 1) * KS);
    if (in_leaf == 0) {  // a leaf starts: fma(a, b, -0) is the rounded product
#pragma unroll
      for (int r = 0; r < 16; ++r) { acc0[r] = -0.0f; acc1[r] = -0.0f; }
    }
#pragma unroll
    for (int g = 0; g < KS / 8; ++g) {  // steps q = 4 g .. 4 g + 3, k = 2 q + kl
      const float4 x0 = *reinterpret_cast<const float4 *>(&sx[buf][kl][arow][4 * g]);
      const float4 x1 = *reinterpret_cast<const float4 *>(&sx[buf][kl][arow + 32][4 * g]);
      const float a0[4] = {x0.x, x0.y, x0.z, x0.w}, a1[4] = {x1.x, x1.y, x1.z, x1.w};
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const float b = sw[buf][2 * (4 * g + u) + kl][bcol];
        acc0 = __builtin_amdgcn_mfma_f32_32x32x2f32(a0[u], b, acc0, 0, 0, 0);
        acc1 = __builtin_amdgcn_mfma_f32_32x32x2f32(a1[u], b, acc1, 0, 0, 0);
      }
    }
    if (++in_leaf == stages_per_leaf) {
      in_leaf = 0;
      fold();
    }
    if (s + 1 < stages) deposit(buf ^ 1);  // its last reader finished before the last barrier
    __syncthreads();
  }

  // the root is in t0[3], t1[3]; lane l, register r holds row 8 (r/4) + 4 (l/32) + r%4,
  // column l%32 of its block (block 1 is 32 rows below block 0)
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    const int64_t row = m0 + 64 * wm + 8 * (r / 4) + 4 * kl + r % 4;
    const int64_t col = n0 + 32 * wn + l % 32;
    if (col < N) {
      if (row < M) p.y[row * N + col] = t0[3][r];
      if (row + 32 < M) p.y[(row + 32) * N + col] = t1[3][r];
    }
  }
}

}  // namespace

bool linear_k_admitted(int64_t k) {  // leaves of whole 32-k stages: K a multiple of 16 * 32
  return k >= 32 * kLeaves && k <= (1 << 24) && k % (32 * kLeaves) == 0;
}

int64_t linear_grid(const LinearArgs &a) { return ((a.m + TM - 1) / TM) * ((a.n + TN - 1) / TN); }

hipError_t launch_linear(const LinearArgs &a, hipStream_t stream) {
  const int64_t grid = linear_grid(a);
  if (grid <= 0) return hipSuccess;
  // 64-k stages for bf16 inputs whose leaves are whole 64-k stages (K a multiple of 1024) and
  // whose tiles are all whole in N (that kernel has no path for columns past N)
  const bool deep = a.x_bf16 && a.w_bf16 && a.k % (64 * kLeaves) == 0 && a.n % TN == 0;
  const void *fn = deep       ? (const void *)linear_leaf_kernel<true, true, 64>
                   : a.x_bf16 ? (a.w_bf16 ? (const void *)linear_leaf_kernel<true, true, 32>
                                          : (const void *)linear_leaf_kernel<true, false, 32>)
                              : (a.w_bf16 ? (const void *)linear_leaf_kernel<false, true, 32>
                                          : (const void *)linear_leaf_kernel<false, false, 32>);
  LinearArgs args = a;
  void *kargs[] = {&args};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace gdn
