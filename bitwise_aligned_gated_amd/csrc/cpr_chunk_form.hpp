// cpr_chunk_form.hpp -- matrix-core helpers and the per-chunk workspace layout shared by the
// chunkwise (WY/UT) forward (cpr_chunked.hip) and its backward (cpr_chunked_bwd.hip).
#pragma once

#include <hip/hip_runtime.h>

#include "cpr_common.hpp"

namespace cpr {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4c __attribute__((ext_vector_type(4)));

// v_mfma_f32_16x16x32_bf16 on a wave of 64 lanes, lane l = j + 16 g (j < 16, g < 4):
//   A (16 x 32): lane holds A[j][8 g + e], e < 8;  B (32 x 16): lane holds B[8 g + e][j];
//   D (16 x 16): lane holds D[4 g + r][j] in register r.
// Both operands are read from arrays laid out with the contraction index contiguous (A as
// [row][k], B as [column][k]), so a lane's eight elements are consecutive.
__device__ __forceinline__ f32x4c mma(const bf16x8& a, const bf16x8& b, f32x4c c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// v_mfma_f32_16x16x4f32 (same lane layout with one A and one B element per lane: A[j][g], B[g][j])
// for the small fp32 products of the triangular inverse.
__device__ __forceinline__ f32x4c mma_f32(float a, float b, f32x4c c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

struct Split {
  bf16x8 hi, lo;
};

__device__ __forceinline__ Split split8(const float4& x0, const float4& x1) {
  const float x[8] = {x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
  Split s;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const __bf16 h = static_cast<__bf16>(x[e]);
    s.hi[e] = h;
    s.lo[e] = static_cast<__bf16>(x[e] - static_cast<float>(h));
  }
  return s;
}

// Eight consecutive fp32 values (16-byte aligned) as a split operand.
__device__ __forceinline__ Split frag_f32(const float* p) {
  return split8(reinterpret_cast<const float4*>(p)[0], reinterpret_cast<const float4*>(p)[1]);
}

// Eight consecutive bf16 values (16-byte aligned) as an exact operand.
__device__ __forceinline__ bf16x8 frag_bf16(const __bf16* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

__device__ __forceinline__ f32x4c mma_split(const Split& a, const Split& b, f32x4c c) {
  c = mma(a.hi, b.hi, c);
  c = mma(a.hi, b.lo, c);
  return mma(a.lo, b.hi, c);
}
__device__ __forceinline__ f32x4c mma_split_a(const Split& a, const bf16x8& b, f32x4c c) {
  c = mma(a.hi, b, c);
  return mma(a.lo, b, c);
}
__device__ __forceinline__ f32x4c mma_split_b(const bf16x8& a, const Split& b, f32x4c c) {
  c = mma(a, b.hi, c);
  return mma(a, b.lo, c);
}

template <int D>
struct ChunkCfg {
  static constexpr int L = 64;                   // token rows of a chunk tile (4 waves x 16)
  static constexpr int NS = 32;                  // state columns per state-pass workgroup
  static constexpr int SB = D + 8;               // bf16 row stride of [L][D] tiles
  static constexpr int ST = L + 8;               // bf16 row stride of [D][L] tiles
  static constexpr int SF = L + 4;               // fp32 row stride of [L][L] / [NS][L] tiles
  static constexpr int SS = D + 4;               // fp32 row stride of the [NS][D] state slice
  static constexpr int WS_MAT = L * D;           // floats of one [L][D] workspace matrix
  static constexpr int WS_LG = 72;               // doubles reserved for the log gate products
};

// Workspace of one (chunk row, value head): W [L][D], U [L][D], C^T [D][L] (fp32), then the
// log gate products lgd[0..L] (fp64; lgd[t] = sum of log a over the chunk's first t tokens).
template <int D>
__host__ __device__ constexpr int64_t chunk_ws_floats() {
  return 3 * ChunkCfg<D>::WS_MAT + 2 * ChunkCfg<D>::WS_LG;
}

// The token range [t0, t1) (within the sequence) of chunk row c of a sequence starting at p0.
__device__ __forceinline__ void chunk_range(const SeqMeta& m, int64_t c, int C, int* t0, int* t1) {
  const int64_t first = m.p0 / C;
  const int64_t b0 = (first + c) * C - m.p0, b1 = (first + c + 1) * C - m.p0;
  *t0 = static_cast<int>(b0 > 0 ? b0 : 0);
  *t1 = static_cast<int>(b1 < m.len ? b1 : m.len);
}

// Rows t < n of an io-bf16 [tokens][D] operand (row t at src + (tok + t) * stride), written
// transposed into dst [D][ST] (zero for t >= n).  Each thread takes two consecutive tokens of one
// 8-column unit, so consecutive threads store consecutive 32-bit words.
template <int D, int ST>
__device__ __forceinline__ void stage_transposed(__bf16* dst, const __bf16* src, int64_t tok, int64_t stride, int n) {
  constexpr int L = 64;
  for (int e = threadIdx.x; e < (L / 2) * (D / 8); e += 256) {
    const int tp = e % (L / 2), c8 = e / (L / 2), t = 2 * tp;
    bf16x8 x0 = {}, x1 = {};
    if (t < n) x0 = *reinterpret_cast<const bf16x8*>(src + (tok + t) * stride + 8 * c8);
    if (t + 1 < n) x1 = *reinterpret_cast<const bf16x8*>(src + (tok + t + 1) * stride + 8 * c8);
#pragma unroll
    for (int y = 0; y < 8; ++y) {
      __bf16 pr[2] = {x0[y], x1[y]};
      *reinterpret_cast<unsigned*>(&dst[(8 * c8 + y) * ST + t]) = __builtin_bit_cast(unsigned, pr);
    }
  }
}

// stage_transposed in two steps: the loads into registers (issued early), then the transposed LDS
// stores (once the destination is free).  Same threads, units and values.
template <int D>
struct TransposedRegs {
  static constexpr int U = ((64 / 2) * (D / 8) + 255) / 256;   // units (two tokens of 8 columns) per thread
  bf16x8 x[2 * U];
};

template <int D>
__device__ __forceinline__ void fetch_transposed(TransposedRegs<D>& R, const __bf16* src, int64_t tok, int64_t stride,
                                                 int n) {
  constexpr int L = 64;
#pragma unroll
  for (int u = 0; u < TransposedRegs<D>::U; ++u) {
    const int e = threadIdx.x + 256 * u, tp = e % (L / 2), c8 = e / (L / 2), t = 2 * tp;
    R.x[2 * u] = R.x[2 * u + 1] = bf16x8{};
    if (e < (L / 2) * (D / 8)) {
      if (t < n) R.x[2 * u] = *reinterpret_cast<const bf16x8*>(src + (tok + t) * stride + 8 * c8);
      if (t + 1 < n) R.x[2 * u + 1] = *reinterpret_cast<const bf16x8*>(src + (tok + t + 1) * stride + 8 * c8);
    }
  }
}

template <int D, int ST>
__device__ __forceinline__ void commit_transposed(__bf16* dst, const TransposedRegs<D>& R) {
  constexpr int L = 64;
#pragma unroll
  for (int u = 0; u < TransposedRegs<D>::U; ++u) {
    const int e = threadIdx.x + 256 * u, tp = e % (L / 2), c8 = e / (L / 2), t = 2 * tp;
    if (e < (L / 2) * (D / 8)) {
#pragma unroll
      for (int y = 0; y < 8; ++y) {
        __bf16 pr[2] = {R.x[2 * u][y], R.x[2 * u + 1][y]};
        *reinterpret_cast<unsigned*>(&dst[(8 * c8 + y) * ST + t]) = __builtin_bit_cast(unsigned, pr);
      }
    }
  }
}

// What the chunkwise forward keeps for its backward, per (chunk row, value head), after the
// workspace above: T^T [L][L] (T^T[t][s] = T[s][t]) and W^T [D][L], fp32.
template <int D>
__host__ __device__ constexpr int64_t chunk_bwd_floats() {
  return static_cast<int64_t>(ChunkCfg<D>::L) * ChunkCfg<D>::L + ChunkCfg<D>::WS_MAT;
}

}  // namespace cpr
