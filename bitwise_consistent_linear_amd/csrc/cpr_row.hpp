// Per-token update of one state row, spread over L lanes of a wavefront (gfx950).
//
// This is the only implementation of the recurrence's arithmetic on the GPU; the scan
// kernel (trainer_fwd, prefill) and the decode kernel both call row_token, so the three
// cases run the same sequence of binary32 operations and agree bit for bit.
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

// Contract dot product of the row slice x with the matching slice y of k or q.
template <int D, int L>
__device__ __forceinline__ float contract_dot(const float (&x)[D / L], const float (&y)[D / L]) {
  constexpr int P = RowShape<D, L>::P, W = RowShape<D, L>::W;
  float leaf[P];
#pragma unroll
  for (int p = 0; p < P; ++p) {
    float acc = x[p * W] * y[p * W];
#pragma unroll
    for (int e = 1; e < W; ++e) acc = __builtin_fmaf(x[p * W + e], y[p * W + e], acc);
    leaf[p] = acc;
  }
#pragma unroll
  for (int w = 1; w < P; w *= 2)
#pragma unroll
    for (int p = 0; p < P; p += 2 * w) leaf[p] = leaf[p] + leaf[p + w];
  float r = leaf[0];
  if constexpr (L >= 2) r = r + dpp_partner<kDppQuadXor1>(r);
  if constexpr (L >= 4) r = r + dpp_partner<kDppQuadXor2>(r);
  if constexpr (L >= 8) r = r + dpp_partner<kDppRowHalfMirror>(r);
  if constexpr (L >= 16) r = r + dpp_partner<kDppRowMirror>(r);
  return r;
}

// One token on one row: decay, key dot, delta, fused rank-1 update, query readout.
// s is updated in place; returns o_i (identical in all L lanes of the row).
template <int D, int L>
__device__ __forceinline__ float row_token(float (&s)[D / L], float a, float b, float v_i,
                                           const float (&k)[D / L], const float (&q)[D / L]) {
  constexpr int M = RowShape<D, L>::M;
  float x[M];
#pragma unroll
  for (int e = 0; e < M; ++e) x[e] = a * s[e];
  const float u = contract_dot<D, L>(x, k);
  const float diff = v_i - u;
  const float delta = b * diff;
#pragma unroll
  for (int e = 0; e < M; ++e) s[e] = __builtin_fmaf(delta, k[e], x[e]);
  return contract_dot<D, L>(s, q);
}

}  // namespace gdn
