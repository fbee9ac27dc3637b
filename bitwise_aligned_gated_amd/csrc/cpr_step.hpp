// cpr_step.hpp -- the one per-token step of the gated delta rule shared by every kernel.
//
// CPR ("Solving the linear-attention headache", IsoExec articles) makes the per-token recurrence
// the reference computation and obtains bitwise agreement between prefill, training and decode by
// having every path apply the same per-token rounding schedule.  This header is that schedule; the
// boundary pass, the output pass and the decode step all call cpr_step() below and nothing else
// touches the state's arithmetic.
//
// Pinned schedule (schedule 1), for each value column j of the fp32 state S (d_k x d_v):
//   leaf partials  the d_k rows form d_k/8 leaves of 8 consecutive rows; a leaf's partial is
//                  p = S[r0][j]*x[r0], then p = fma(S[r][j], x[r], p) for r = r0+1 .. r0+7
//   tree           the leaf partials are summed by a balanced pairwise tree: leaf 2m with 2m+1,
//                  then those sums pairwise, and so on (IEEE add is commutative, so both lanes of
//                  a DPP butterfly pair hold the same bits)
//   update         u = tree(S, k); w = fma(-a, u, v_j); c = b*w; S[r][j] = fma(k[r], c, a*S[r][j])
//   output         o_j = tree(S_updated, q)
// All in fp32 with IEEE denormals and round-to-nearest-even, built with -ffp-contract=off so no
// other fusion can appear.  Which lane holds which leaf is free: a lane may hold NL consecutive
// leaves and sum them in-lane with the same pairwise tree before the cross-lane levels, so any
// (leaves per lane, lanes per column) mapping yields identical bits.
#pragma once

#include <hip/hip_runtime.h>

#include "cpr_schedule.hpp"

namespace cpr {

// One butterfly level across lanes inside a DPP row: x + x[partner].
template <int CTRL>
__device__ __forceinline__ float dpp_pair_add(float x) {
  const int y = __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xF, 0xF, false);
  return x + __builtin_bit_cast(float, y);
}

// Balanced all-reduce over G consecutive lanes (G in {1, 2, 4, 8, 16}, groups aligned to G).
// Level 1 pairs lane l with l^1 (quad_perm [1,0,3,2]); level 2 with l^2 (quad_perm [2,3,0,1]);
// level 3 uses row_half_mirror (l <-> 7-l) and level 4 row_mirror (l <-> 15-l).  After level m
// every lane of an aligned 2^m block holds the same bits, so each mirror pairs whole blocks
// exactly as an xor-butterfly would.
template <int G>
__device__ __forceinline__ float lane_tree(float x) {
  static_assert(G == 1 || G == 2 || G == 4 || G == 8 || G == 16, "lanes per column");
  if constexpr (G >= 2) x = dpp_pair_add<0xB1>(x);   // quad_perm [1,0,3,2]
  if constexpr (G >= 4) x = dpp_pair_add<0x4E>(x);   // quad_perm [2,3,0,1]
  if constexpr (G >= 8) x = dpp_pair_add<0x141>(x);  // row_half_mirror
  if constexpr (G >= 16) x = dpp_pair_add<0x140>(x); // row_mirror
  return x;
}

// The pinned dot product of one column slice with x: NL leaves in this lane (rows
// [0, NL*kLeaf) of the arrays), the in-lane part of the tree, then the cross-lane levels.
template <int NL, int G>
__device__ __forceinline__ float pinned_dot(const float (&s)[NL * kLeaf], const float (&x)[NL * kLeaf]) {
  float p[NL];
#pragma unroll
  for (int l = 0; l < NL; ++l) {
    float acc = s[l * kLeaf] * x[l * kLeaf];
#pragma unroll
    for (int r = 1; r < kLeaf; ++r) acc = __builtin_fmaf(s[l * kLeaf + r], x[l * kLeaf + r], acc);
    p[l] = acc;
  }
#pragma unroll
  for (int w = 1; w < NL; w *= 2) {
#pragma unroll
    for (int l = 0; l + w < NL; l += 2 * w) p[l] = p[l] + p[l + w];
  }
  return lane_tree<G>(p[0]);
}

// The update's last step on one column slice held by this lane: S[r][j] = fma(k[r], c, a*S[r][j]).
template <int N>
__device__ __forceinline__ void cpr_apply(float (&s)[N], const float (&k)[N], float a, float c) {
#pragma unroll
  for (int r = 0; r < N; ++r) s[r] = __builtin_fmaf(k[r], c, a * s[r]);
}

// The state update of one token on one column slice held by this lane (steps 1-4 of the
// schedule); u, w and c are returned for the passes that keep them.
template <int NL, int G>
__device__ __forceinline__ void cpr_update(float (&s)[NL * kLeaf], const float (&k)[NL * kLeaf], float v, float a,
                                           float b, float& u, float& w, float& c) {
  u = pinned_dot<NL, G>(s, k);
  w = __builtin_fmaf(-a, u, v);
  c = b * w;
  cpr_apply(s, k, a, c);
}

// One token applied to one column slice held by this lane.
//   s   this lane's NL*8 rows of column j (updated in place)
//   k   the same rows of k_t; q the same rows of q_t (read only when WITH_OUT)
//   v   v_t[j]; a, b the token's gates.  Returns o_t[j] when WITH_OUT (every lane of the
//   column's G-lane group returns the same bits), else 0.
template <int NL, int G, bool WITH_OUT>
__device__ __forceinline__ float cpr_step(float (&s)[NL * kLeaf], const float (&k)[NL * kLeaf],
                                          const float (&q)[NL * kLeaf], float v, float a, float b) {
  float u, w, c;
  cpr_update<NL, G>(s, k, v, a, b, u, w, c);
  if constexpr (WITH_OUT) return pinned_dot<NL, G>(s, q);
  return 0.0f;
}

// The same step with output when c_t[j] is already known (kept by an earlier pass that ran this
// very step on the same state): the update's last step and the output, the same bits as cpr_step.
template <int NL, int G>
__device__ __forceinline__ float cpr_step_given_c(float (&s)[NL * kLeaf], const float (&k)[NL * kLeaf],
                                                  const float (&q)[NL * kLeaf], float a, float c) {
  cpr_apply(s, k, a, c);
  return pinned_dot<NL, G>(s, q);
}

// fp32 -> bf16 bits, round to nearest even (finite values), the one conversion every kernel uses.
__device__ __forceinline__ unsigned short f32_to_bf16_rne(float f) {
  unsigned int u = __builtin_bit_cast(unsigned int, f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return static_cast<unsigned short>(u >> 16);
}

__device__ __forceinline__ float bf16_to_f32(unsigned short h) {
  return __builtin_bit_cast(float, static_cast<unsigned int>(h) << 16);
}

// Resynchronisation to a bf16 boundary dtype: every state element rounded to the nearest bf16
// (ties to even).  Applied to the state entering a chunk-start position, just before that
// position's token, by every path; with the fp32 boundary dtype nothing is applied.
template <int N>
__device__ __forceinline__ void resync_round(float (&s)[N]) {
#pragma unroll
  for (int r = 0; r < N; ++r) s[r] = bf16_to_f32(f32_to_bf16_rne(s[r]));
}

}  // namespace cpr
