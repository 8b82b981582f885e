// Per-token update of one state row, spread over L lanes of a wavefront (gfx950).
//
// The scan kernel (trainer_fwd, prefill) calls these steps, and the decode kernel calls
// row_token, so the three cases run the same sequence of binary32 operations and agree bit
// for bit. The wide decode kernel holds a row on 32 lanes (row_token_split below): the same
// operations on the same operands in the same order, with each leaf's chain handed from
// one lane to the next half-way.
//
// A row s of d_k = D binary32 values lives in the VGPRs of L consecutive lanes: lane l
// holds elements [l*M, (l+1)*M) with M = D/L, i.e. P = 16/L whole leaves of W = D/16
// contiguous elements. The contract's dot product is then:
//   1. per leaf, a serial chain: rounded product of the first pair, fmaf for the rest;
//   2. within the lane, the pairwise tree over its P leaves (natural order);
//   3. across lanes, the remaining levels by DPP: partner lane l^1 (quad_perm [1,0,3,2]),
//      l^2 (quad_perm [2,3,0,1]), then the other half of the 8-lane group (row_half_mirror)
//      and the other half of the 16-lane row (row_mirror).
// After step 2 every lane of a 2^j-lane group holds the same partial sum, so any partner
// in the other group gives the natural pairing; IEEE addition is commutative, so every
// lane ends with identical bits. Fixed binary tree with fp32 accumulation: IsoExec,
// agentlenshq.com, section on achieving parallel invariance.
#pragma once

#include <hip/hip_runtime.h>

namespace gdn {

// DPP controls (GCN/CDNA encoding).
constexpr int kDppQuadXor1 = 0xB1;    // quad_perm [1,0,3,2]
constexpr int kDppQuadXor2 = 0x4E;    // quad_perm [2,3,0,1]
constexpr int kDppRowHalfMirror = 0x141;
constexpr int kDppRowMirror = 0x140;
constexpr int kDppQuadEven = 0xA0;    // quad_perm [0,0,2,2]: each lane reads its even lane
constexpr int kDppQuadOdd = 0xF5;     // quad_perm [1,1,3,3]: each lane reads its odd lane

template <int CTRL>
__device__ __forceinline__ float dpp_partner(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, true));
}

template <int D, int L>
struct RowShape {
  static_assert(D % 16 == 0, "d_k must be a multiple of the 16 leaves");
  static_assert(L == 1 || L == 2 || L == 4 || L == 8 || L == 16, "lanes per row");
  static constexpr int M = D / L;   // row elements per lane
  static constexpr int P = 16 / L;  // leaves per lane
  static constexpr int W = D / 16;  // leaf width
};

// N contract dot products computed side by side: dot n of the row slice x[n] with the
// matching slice y[n] of k or q. Each dot performs exactly the contract's sequence of
// operations (the same for every N); computing several together only lets independent
// instructions fill each other's latencies and DPP wait states.
template <int D, int L, int N>
__device__ __forceinline__ void contract_dots(const float (&x)[N][D / L],
                                              const float (&y)[N][D / L], float (&r)[N]) {
  constexpr int P = RowShape<D, L>::P, W = RowShape<D, L>::W;
  float leaf[N][P];
#pragma unroll
  for (int p = 0; p < P; ++p)
#pragma unroll
    for (int n = 0; n < N; ++n) leaf[n][p] = x[n][p * W] * y[n][p * W];
#pragma unroll
  for (int e = 1; e < W; ++e)
#pragma unroll
    for (int p = 0; p < P; ++p)
#pragma unroll
      for (int n = 0; n < N; ++n)
        leaf[n][p] = __builtin_fmaf(x[n][p * W + e], y[n][p * W + e], leaf[n][p]);
#pragma unroll
  for (int w = 1; w < P; w *= 2)
#pragma unroll
    for (int p = 0; p < P; p += 2 * w)
#pragma unroll
      for (int n = 0; n < N; ++n) leaf[n][p] = leaf[n][p] + leaf[n][p + w];
#pragma unroll
  for (int n = 0; n < N; ++n) r[n] = leaf[n][0];
  if constexpr (L >= 2) {
#pragma unroll
    for (int n = 0; n < N; ++n) r[n] = r[n] + dpp_partner<kDppQuadXor1>(r[n]);
  }
  if constexpr (L >= 4) {
#pragma unroll
    for (int n = 0; n < N; ++n) r[n] = r[n] + dpp_partner<kDppQuadXor2>(r[n]);
  }
  if constexpr (L >= 8) {
#pragma unroll
    for (int n = 0; n < N; ++n) r[n] = r[n] + dpp_partner<kDppRowHalfMirror>(r[n]);
  }
  if constexpr (L >= 16) {
#pragma unroll
    for (int n = 0; n < N; ++n) r[n] = r[n] + dpp_partner<kDppRowMirror>(r[n]);
  }
}

template <int D, int L>
__device__ __forceinline__ float contract_dot(const float (&x)[D / L], const float (&y)[D / L]) {
  constexpr int M = RowShape<D, L>::M;
  float xs[1][M], ys[1][M], r[1];
#pragma unroll
  for (int e = 0; e < M; ++e) {
    xs[0][e] = x[e];
    ys[0][e] = y[e];
  }
  contract_dots<D, L, 1>(xs, ys, r);
  return r[0];
}

// The steps of one token on one row (s: the row's slice in this lane).
template <int D, int L>
__device__ __forceinline__ void row_decay(const float (&s)[D / L], float a, float (&x)[D / L]) {
#pragma unroll
  for (int e = 0; e < RowShape<D, L>::M; ++e) x[e] = a * s[e];
}

__device__ __forceinline__ float row_delta(float b, float v_i, float u) {
  const float diff = v_i - u;
  return b * diff;
}

template <int D, int L>
__device__ __forceinline__ void row_update(float (&s)[D / L], float delta, const float (&k)[D / L],
                                           const float (&x)[D / L]) {
#pragma unroll
  for (int e = 0; e < RowShape<D, L>::M; ++e) s[e] = __builtin_fmaf(delta, k[e], x[e]);
}

// One token on one row: decay, key dot, delta, fused rank-1 update, query readout.
// s is updated in place; returns o_i (identical in all L lanes of the row).
template <int D, int L>
__device__ __forceinline__ float row_token(float (&s)[D / L], float a, float b, float v_i,
                                           const float (&k)[D / L], const float (&q)[D / L]) {
  float x[RowShape<D, L>::M];
  row_decay<D, L>(s, a, x);
  const float u = contract_dot<D, L>(x, k);
  row_update<D, L>(s, row_delta(b, v_i, u), k, x);
  return contract_dot<D, L>(s, q);
}

// --------------------------------------------------------------------------- backward
// The backward steps of one token on one row, sh being the lane's slice of dL/ds. The
// reverse scan and the chunk kernel both use these, so they produce the same dL/ds bits.

// sh_e = fmaf(g, q_e, sh_e): adds the readout's share, g = dL/do_i.
template <int D, int L>
__device__ __forceinline__ void row_bwd_absorb(float (&sh)[D / L], float g,
                                               const float (&q)[D / L]) {
#pragma unroll
  for (int e = 0; e < RowShape<D, L>::M; ++e) sh[e] = __builtin_fmaf(g, q[e], sh[e]);
}

// dh = dot(sh, k); dv_i = b * dh; xh_e = fmaf(-dv_i, k_e, sh_e). Returns dv_i.
template <int D, int L>
__device__ __forceinline__ float row_bwd_delta(const float (&sh)[D / L], const float (&k)[D / L],
                                               float b, float (&xh)[D / L], float &dh) {
  dh = contract_dot<D, L>(sh, k);
  const float dv_i = b * dh;
  const float uh = -dv_i;
#pragma unroll
  for (int e = 0; e < RowShape<D, L>::M; ++e) xh[e] = __builtin_fmaf(uh, k[e], sh[e]);
  return dv_i;
}

// sh_e = a * xh_e: dL/ds of the previous state.
template <int D, int L>
__device__ __forceinline__ void row_bwd_decay(float (&sh)[D / L], float a, const float (&xh)[D / L]) {
#pragma unroll
  for (int e = 0; e < RowShape<D, L>::M; ++e) sh[e] = a * xh[e];
}

// ------------------------------------------------------------ a row on 32 lanes (decode)
// Lane l of a 32-lane row holds elements [l*M, (l+1)*M), M = D/32: the first or second half
// of leaf l/2 (leaf width 2M), so a lane's slice is 16 bytes at d_k = 128. A leaf's chain
// starts in its even lane (rounded first product, fmaf for the rest of that half) and
// continues in its odd lane from the even lane's partial, copied by DPP; the odd lane's
// result, copied back, is the leaf in both lanes. The tree then pairs leaves 2m and 2m+1
// (lanes two apart: quad_perm [2,3,0,1]), leaf pairs (the other half of each 8-lane group:
// row_half_mirror), groups of four (the other half of the 16-lane row: row_mirror) and the
// two halves of the 32-lane row (a lane swap between 16-lane rows): the natural pairing of
// the contract's tree, every lane of the row ending with the same bits.
__device__ __forceinline__ float swap16_sum(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

template <int D>
__device__ __forceinline__ float contract_dot_split(const float (&x)[D / 32],
                                                    const float (&y)[D / 32]) {
  static_assert(D % 32 == 0, "a leaf spans two lanes");
  constexpr int M = D / 32;
  float part = x[0] * y[0];
#pragma unroll
  for (int e = 1; e < M; ++e) part = __builtin_fmaf(x[e], y[e], part);
  float leaf = dpp_partner<kDppQuadEven>(part);  // odd lanes: continue the even lane's chain
#pragma unroll
  for (int e = 0; e < M; ++e) leaf = __builtin_fmaf(x[e], y[e], leaf);
  float r = dpp_partner<kDppQuadOdd>(leaf);
  r = r + dpp_partner<kDppQuadXor2>(r);
  r = r + dpp_partner<kDppRowHalfMirror>(r);
  r = r + dpp_partner<kDppRowMirror>(r);
  return swap16_sum(r);
}

// row_token on a 32-lane row: decay, key dot, delta, fused rank-1 update, query readout.
template <int D>
__device__ __forceinline__ float row_token_split(float (&s)[D / 32], float a, float b,
                                                 float v_i, const float (&k)[D / 32],
                                                 const float (&q)[D / 32]) {
  constexpr int M = D / 32;
  float x[M];
#pragma unroll
  for (int e = 0; e < M; ++e) x[e] = a * s[e];
  const float u = contract_dot_split<D>(x, k);
  const float delta = row_delta(b, v_i, u);
#pragma unroll
  for (int e = 0; e < M; ++e) s[e] = __builtin_fmaf(delta, k[e], x[e]);
  return contract_dot_split<D>(s, q);
}

}  // namespace gdn
