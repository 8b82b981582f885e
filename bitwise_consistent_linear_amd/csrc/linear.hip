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
// independent accumulator chains); two waves per SIMD. K is staged 32 at a time into LDS as
// binary32, double-buffered, the next stage's global loads in registers while the current
// one computes: W k-major; X row-major with each row's even and odd k apart, so one 16-byte
// read gives a lane its A operands for four steps.

#include "internal.h"

namespace gdn {
namespace {

using f32x16 = float __attribute__((ext_vector_type(16)));

constexpr int kWaves = 8, kThreads = 64 * kWaves;
constexpr int TM = 128, TN = 128, KS = 32;     // workgroup tile, k per stage
constexpr int QS = KS / 2 + 4, WS = TN + 4;    // LDS row strides (conflict-free reads)
constexpr int kLeaves = 16;
constexpr int XPT = TM * KS / kThreads;        // staged X values per thread (8)
constexpr int WPT = KS * TN / kThreads;        // staged W values per thread (8)
static_assert(XPT == 8 && WPT == 8, "staging assumes 8 values per thread");

__device__ __forceinline__ float widen_bf16(uint32_t bits16) { return __uint_as_float(bits16 << 16); }

template <bool XBF16, bool WBF16>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void linear_leaf_kernel(const LinearArgs p) {
  __shared__ __align__(16) float sx[2][2][TM][QS];  // sx[buf][k % 2][row][k / 2]
  __shared__ __align__(16) float sw[2][KS][WS];      // sw[buf][k][col]

  const int tid = threadIdx.x, wave = tid / 64, l = tid % 64;
  const int wm = wave / 4, wn = wave % 4;  // 2 x 4 waves of 64 x 32
  const int64_t M = p.m, N = p.n;
  const int K = p.k;
  const int64_t tiles_n = (N + TN - 1) / TN;
  const int64_t tile_m = blockIdx.x / tiles_n, tile_n = blockIdx.x % tiles_n;
  const int64_t m0 = tile_m * TM, n0 = tile_n * TN;

  // staging: X tile [128 rows x 32 k]: one row, 8 consecutive k per thread;
  //          W tile [32 k x 128 cols]: one k, 8 consecutive columns per thread
  const int xr = tid / 4, xk = (tid % 4) * 8;
  const int wk = tid / 16, wc = (tid % 16) * 8;
  const int64_t xrow = m0 + xr < M ? m0 + xr : M - 1;  // rows past M repeat the last row
  const bool w_vec = N % (WBF16 ? 8 : 4) == 0;           // every W row 16-byte aligned
  float xv[XPT], wv[WPT];
  auto fetch = [&](int k0) {
    const int64_t xo = xrow * K + k0 + xk;
    if constexpr (XBF16) {
      const uint4 r = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.x) + xo);
      const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        xv[2 * e] = widen_bf16(u[e] & 0xFFFFu);
        xv[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
      }
    } else {
      const float4 a = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.x) + xo);
      const float4 b = *reinterpret_cast<const float4 *>(static_cast<const float *>(p.x) + xo + 4);
      xv[0] = a.x; xv[1] = a.y; xv[2] = a.z; xv[3] = a.w;
      xv[4] = b.x; xv[5] = b.y; xv[6] = b.z; xv[7] = b.w;
    }
    const int64_t wrow = (int64_t)(k0 + wk) * N;
    if (w_vec && n0 + wc + WPT <= N) {  // all columns in range, rows 16-byte aligned
      if constexpr (WBF16) {
        const uint4 r = *reinterpret_cast<const uint4 *>(static_cast<const uint16_t *>(p.w) +
                                                         wrow + n0 + wc);
        const uint32_t u[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          wv[2 * e] = widen_bf16(u[e] & 0xFFFFu);
          wv[2 * e + 1] = __uint_as_float(u[e] & 0xFFFF0000u);
        }
      } else {
        const float4 *src = reinterpret_cast<const float4 *>(static_cast<const float *>(p.w) +
                                                             wrow + n0 + wc);
#pragma unroll
        for (int e = 0; e < 2; ++e) {
          const float4 r = src[e];
          wv[4 * e] = r.x; wv[4 * e + 1] = r.y; wv[4 * e + 2] = r.z; wv[4 * e + 3] = r.w;
        }
      }
    } else {
#pragma unroll
      for (int e = 0; e < WPT; ++e) {  // columns past N repeat the last column
        const int64_t c = n0 + wc + e < N ? n0 + wc + e : N - 1;
        if constexpr (WBF16)
          wv[e] = widen_bf16(static_cast<const uint16_t *>(p.w)[wrow + c]);
        else
          wv[e] = static_cast<const float *>(p.w)[wrow + c];
      }
    }
  };
  auto deposit = [&](int buf) {
    // k = xk + e: even k to half 0, odd k to half 1, at position k / 2
    *reinterpret_cast<float4 *>(&sx[buf][0][xr][xk / 2]) = make_float4(xv[0], xv[2], xv[4], xv[6]);
    *reinterpret_cast<float4 *>(&sx[buf][1][xr][xk / 2]) = make_float4(xv[1], xv[3], xv[5], xv[7]);
#pragma unroll
    for (int e = 0; e < WPT; e += 4)
      *reinterpret_cast<float4 *>(&sw[buf][wk][wc + e]) =
          make_float4(wv[e], wv[e + 1], wv[e + 2], wv[e + 3]);
  };

  // per lane: A operands for both blocks (rows 64 wm + l%32 and 32 more, k = 2q + l/32), the
  // shared B operand (column 32 wn + l%32)
  const int arow = 64 * wm + l % 32, bcol = 32 * wn + l % 32, kl = l / 32;
  const int stages_per_leaf = K / (KS * kLeaves);  // K % 512 == 0: a leaf is whole stages
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

bool linear_k_admitted(int64_t k) {  // leaves of whole stages: K a multiple of 16 * 32
  return k >= KS * kLeaves && k <= (1 << 24) && k % (KS * kLeaves) == 0;
}

int64_t linear_grid(const LinearArgs &a) { return ((a.m + TM - 1) / TM) * ((a.n + TN - 1) / TN); }

hipError_t launch_linear(const LinearArgs &a, hipStream_t stream) {
  const int64_t grid = linear_grid(a);
  if (grid <= 0) return hipSuccess;
  const void *fn = a.x_bf16 ? (a.w_bf16 ? (const void *)linear_leaf_kernel<true, true>
                                        : (const void *)linear_leaf_kernel<true, false>)
                            : (a.w_bf16 ? (const void *)linear_leaf_kernel<false, true>
                                        : (const void *)linear_leaf_kernel<false, false>);
  LinearArgs args = a;
  void *kargs[] = {&args};
  return hipLaunchKernel(fn, dim3((unsigned)grid), dim3(kThreads), kargs, 0, stream);
}

}  // namespace gdn
