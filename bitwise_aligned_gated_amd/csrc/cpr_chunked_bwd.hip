// cpr_chunked_bwd.hip -- the backward of the chunkwise (WY/UT) trainer forward: the "native" trainer
// column of the per-layer table in "Solving the linear-attention headache" (IsoExec articles), the
// evaluation CPR's trainer forward and backward are compared against.
//
// With G = dL/dS, the adjoint recurrence G_{t-1} = a_t (I - b_t k_t k_t^T)(G_t + q_t dO_t^T), which
// the CPR backward walks token by token, has a chunk form.  Per chunk of L tokens with gate
// products Gam_t = a_1 ... a_t, chunk-end adjoint G_L, the forward's T = (I + A)^{-1} and
// W = T diag(b Gam) K, the gradients reaching the write vectors, dc_t = (G_t + q_t dO_t^T)^T k_t,
// solve the transposed system of the forward's:
//     (I + A^T) dC = R,   R = (M . Q K^T)^T dO + diag(Gam_L / Gam) K G_L,   so dC = T^T R,
// and the adjoint at the chunk start is
//     G_0 = Gam_L G_L + Q^T diag(Gam) dO - K^T diag(b Gam) dC = Gam_L G_L + Q^T diag(Gam) dO - W^T R.
// The forward's w_t = v_t - a_t S_{t-1}^T k_t (for db) is, per chunk,
//     w = V - diag(Gam) K S_0 - (N . K K^T) C,   N[t][s] = Gam_t / Gam_s (s < t).
// Kernels: intra (per chunk and value head, all chunks at once: w, and the part of R that does not
// depend on G), state (per sequence, value head and column slice, last chunk first: R, dc, G at every
// chunk boundary and <G, S_0> at every chunk start).  dq, dk, dv, da and db then come from the
// per-token and chunk-gradient kernels of the CPR backward, which take dc, G and the forward's c from
// here.  Products run on v_mfma_f32_16x16x32_bf16 with split (hi + lo bf16) operands where a value
// is not exactly bf16, as in the forward.
#include <hip/hip_runtime.h>

#include "cpr_chunk_form.hpp"
#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

// ---- intra: w and the G-independent part of R, per (chunk row, value head) ----------------------
template <int D>
struct alignas(16) IntraLds {
  using M = ChunkCfg<D>;
  static constexpr int KS = D + 8;                            // bf16 row stride of the K rows
  float pm[M::L * M::SF];       // (M . Q K^T)^T, then N . K K^T
  union {
    __bf16 dt[D * M::ST];       // dO^T (zero past the chunk)
    __bf16 kr[M::L * KS];       // then the K rows (zero past the chunk)
  };
  double lgd[M::L + 1];
};

template <int D>
__global__ void __launch_bounds__(256) nbwd_intra_kernel(BackwardArgs A) {
  using M = ChunkCfg<D>;
  constexpr int L = M::L, ST = M::ST, SF = M::SF, NT = D / 16;
  __shared__ IntraLds<D> S;
  __shared__ int64_t red[6];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio);
  const int64_t w = gs.group / A.h_k;
  const int kh = static_cast<int>(gs.group % A.h_k);
  const int h = kh * ratio + gs.member;
  if (w >= A.rows_cap) return;                                // uniform across the block
  int i;
  int64_t c;
  if (!plan_find_row(A, w, &i, &c, red)) return;              // uniform across the block
  const SeqMeta m = seq_meta(A, i);
  int t0, t1;
  chunk_range(m, c, A.chunk, &t0, &t1);
  const int n = t1 - t0;                                      // tokens, 1..64
  const int64_t tok = m.tok0 + t0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lg = lane >> 4;
  const int row = 16 * wave + lj;                             // this lane's A row
  const __bf16* qin = static_cast<const __bf16*>(A.q);
  const __bf16* kin = static_cast<const __bf16*>(A.k);
  const __bf16* vin = static_cast<const __bf16*>(A.v);
  const __bf16* din = static_cast<const __bf16*>(A.d_o);
  const float* wsb = A.fws + (w * A.h_v + h) * chunk_ws_floats<D>();
  const double* lgw = reinterpret_cast<const double*>(wsb + 3 * M::WS_MAT);
  for (int e = tid; e <= L; e += 256) S.lgd[e] = lgw[e];
  // K fragments of this lane's row (exact bf16; zero past the chunk)
  bf16x8 kf[D / 32];
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    kf[p] = bf16x8{};
    if (row < n) kf[p] = *reinterpret_cast<const bf16x8*>(kin + ((tok + row) * A.h_k + kh) * D + 32 * p + 8 * lg);
  }
  stage_transposed<D, ST>(S.dt, din + static_cast<int64_t>(h) * D, tok, static_cast<int64_t>(A.h_v) * D, n);
  __syncthreads();
  // pm[t][s] = (Gam_s / Gam_t) k_t . q_s for t <= s: the transpose of the forward's M . Q K^T
  {
    f32x4c acc[4] = {};
#pragma unroll
    for (int p = 0; p < D / 32; ++p)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int s = 16 * nt + lj;
        bf16x8 qf = {};
        if (s < n) qf = *reinterpret_cast<const bf16x8*>(qin + ((tok + s) * A.h_k + kh) * D + 32 * p + 8 * lg);
        acc[nt] = mma(kf[p], qf, acc[nt]);
      }
    double lrow[4], lcol[4];                                   // read before any use
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      lrow[x] = S.lgd[16 * wave + 4 * lg + x + 1];
      lcol[x] = S.lgd[16 * x + lj + 1];
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * lg + r, s = 16 * nt + lj;
        float x = 0.f;
        if (t <= s && s < n) x = __expf(static_cast<float>(lcol[nt] - lrow[r])) * acc[nt][r];
        S.pm[t * SF + s] = x;
      }
  }
  __syncthreads();
  // the G-independent part of R, pm dO, into the dc buffer (the state pass completes it)
  {
    f32x4c acc[NT] = {};
#pragma unroll
    for (int p = 0; p < L / 32; ++p) {
      const Split af = frag_f32(&S.pm[row * SF + 32 * p + 8 * lg]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        acc[nt] = mma_split_a(af, frag_bf16(&S.dt[(16 * nt + lj) * ST + 32 * p + 8 * lg]), acc[nt]);
    }
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * lg + r;
        if (t < n) A.dc[((tok + t) * A.h_v + h) * D + 16 * nt + lj] = acc[nt][r];
      }
  }
  __syncthreads();                                            // pm reads done
  // pm[t][s] = (Gam_t / Gam_s) k_t . k_s for s < t
  {
    f32x4c acc[4] = {};
#pragma unroll
    for (int p = 0; p < D / 32; ++p)
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int s = 16 * nt + lj;
        bf16x8 kb = {};
        if (s < n) kb = *reinterpret_cast<const bf16x8*>(kin + ((tok + s) * A.h_k + kh) * D + 32 * p + 8 * lg);
        acc[nt] = mma(kf[p], kb, acc[nt]);
      }
    double lrow[4], lcol[4];                                   // read before any use
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      lrow[x] = S.lgd[16 * wave + 4 * lg + x + 1];
      lcol[x] = S.lgd[16 * x + lj + 1];
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * lg + r, s = 16 * nt + lj;
        float x = 0.f;
        if (s < t && t < n) x = __expf(static_cast<float>(lrow[r] - lcol[nt])) * acc[nt][r];
        S.pm[t * SF + s] = x;
      }
  }
  __syncthreads();
  // w = V - diag(Gam) K S_0 - (N . K K^T) C.  Each wave takes whole 16-column tiles over all 64 rows,
  // so the block reads S_0 and C^T once: the tile's S_0 and C^T fragments are split once and used for
  // the four row blocks, whose K rows come from LDS.
  constexpr int KS = IntraLds<D>::KS;
  for (int e = tid; e < L * (D / 8); e += 256) {              // dO^T is no longer read
    const int t = e / (D / 8), c8 = e % (D / 8);
    bf16x8 x = {};
    if (t < n) x = *reinterpret_cast<const bf16x8*>(kin + ((tok + t) * A.h_k + kh) * D + 8 * c8);
    *reinterpret_cast<bf16x8*>(&S.kr[t * KS + 8 * c8]) = x;
  }
  __syncthreads();
  const float* s0 = A.chunk_states + (w * A.h_v + h) * static_cast<int64_t>(D) * D;   // S^T [column][d]
  const float* ctw = wsb + 2 * M::WS_MAT;                                              // C^T [D][L]
#pragma unroll 1
  for (int nt = wave; nt < NT; nt += 4) {
    Split sf[D / 32], cf[L / 32];
#pragma unroll
    for (int p = 0; p < D / 32; ++p) sf[p] = frag_f32(s0 + (16 * nt + lj) * D + 32 * p + 8 * lg);
#pragma unroll
    for (int p = 0; p < L / 32; ++p) cf[p] = frag_f32(ctw + (16 * nt + lj) * L + 32 * p + 8 * lg);
#pragma unroll 1
    for (int rb = 0; rb < L / 16; ++rb) {
      f32x4c acc = {};
#pragma unroll
      for (int p = 0; p < D / 32; ++p) acc = mma_split_b(frag_bf16(&S.kr[(16 * rb + lj) * KS + 32 * p + 8 * lg]), sf[p], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[r] *= __expf(static_cast<float>(S.lgd[16 * rb + 4 * lg + r + 1]));
#pragma unroll
      for (int p = 0; p < L / 32; ++p) acc = mma_split(frag_f32(&S.pm[(16 * rb + lj) * SF + 32 * p + 8 * lg]), cf[p], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * rb + 4 * lg + r;
        if (t < n) {
          const int64_t e = ((tok + t) * A.h_v + h) * D + 16 * nt + lj;
          A.ww[e] = static_cast<float>(vin[e]) - acc[r];
        }
      }
    }
  }
}

// ---- state: the chunk chain of the adjoint, last chunk first, per (sequence, value head, slice) ----
template <int D>
struct alignas(16) BwdStateLds {
  using M = ChunkCfg<D>;
  float gt[M::NS * M::SS];      // G^T slice [column][d]
  float rt[M::NS * M::SF];      // R^T [column][token]
  float ot[M::NS * M::SF];      // (diag(Gam) dO)^T [column][token]
  __bf16 qt[D * M::ST];         // Q^T of the chunk
  double lgd[M::L + 1];
};

// One chunk's inputs of the chain that do not depend on G, loaded a chunk ahead into registers.
template <int D>
struct BwdRegs {
  using M = ChunkCfg<D>;
  static constexpr int QU = ((M::L / 2) * (D / 8) + 255) / 256;   // token pairs of 8 Q columns per thread
  bf16x8 q[2 * QU];
  bf16x8 k[D / 32];                                            // this lane's K row, as A fragments
  float ri[M::NS / 16][4];                                     // R's intra part at this lane's positions
  float dov[M::NS / 16][4];                                    // dO there
  double lg;                                                   // lgd[tid] (threads 0..L)
};

template <int D>
__device__ __forceinline__ void bwd_fetch(const BackwardArgs& A, const SeqMeta& m, int64_t row0, int64_t c, int h,
                                          int kh, int j0, BwdRegs<D>& R) {
  using M = ChunkCfg<D>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lg = lane >> 4;
  const int row = 16 * wave + lj;
  int t0, t1;
  chunk_range(m, c, A.chunk, &t0, &t1);
  const int n = t1 - t0;
  const int64_t tok = m.tok0 + t0;
  const __bf16* qin = static_cast<const __bf16*>(A.q);
  const __bf16* kin = static_cast<const __bf16*>(A.k);
  const __bf16* din = static_cast<const __bf16*>(A.d_o);
#pragma unroll
  for (int x = 0; x < BwdRegs<D>::QU; ++x) {
    const int e = tid + 256 * x, t = 2 * (e % (M::L / 2)), c8 = e / (M::L / 2);
    R.q[2 * x] = R.q[2 * x + 1] = bf16x8{};
    if (e < (M::L / 2) * (D / 8)) {
      if (t < n) R.q[2 * x] = *reinterpret_cast<const bf16x8*>(qin + ((tok + t) * A.h_k + kh) * D + 8 * c8);
      if (t + 1 < n) R.q[2 * x + 1] = *reinterpret_cast<const bf16x8*>(qin + ((tok + t + 1) * A.h_k + kh) * D + 8 * c8);
    }
  }
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    R.k[p] = bf16x8{};
    if (row < n) R.k[p] = *reinterpret_cast<const bf16x8*>(kin + ((tok + row) * A.h_k + kh) * D + 32 * p + 8 * lg);
  }
#pragma unroll
  for (int nt = 0; nt < M::NS / 16; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * wave + 4 * lg + r;
      R.ri[nt][r] = R.dov[nt][r] = 0.f;
      if (t < n) {
        const int64_t e = ((tok + t) * A.h_v + h) * D + j0 + 16 * nt + lj;
        R.ri[nt][r] = A.dc[e];
        R.dov[nt][r] = static_cast<float>(din[e]);
      }
    }
  const float* wsb = A.fws + ((row0 + c) * A.h_v + h) * chunk_ws_floats<D>();
  R.lg = tid <= M::L ? reinterpret_cast<const double*>(wsb + 3 * M::WS_MAT)[tid] : 0.0;
}

template <int D>
__host__ __device__ constexpr int bwd_state_parts() {
  return (D / ChunkCfg<D>::NS) * 4;                            // slices x waves
}

template <int D>
__global__ void __launch_bounds__(256) nbwd_state_kernel(BackwardArgs A) {
  using M = ChunkCfg<D>;
  constexpr int L = M::L, NS = M::NS, SS = M::SS, SF = M::SF, ST = M::ST;
  constexpr int NSL = D / NS;                                  // column slices per value head
  __shared__ BwdStateLds<D> S;
  __shared__ int64_t red[6];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio * NSL);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k), kh = static_cast<int>(gs.group % A.h_k);
  const int h = kh * ratio + gs.member / NSL, sl = gs.member % NSL;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = plan_row_offset(A, i, red);
  const int64_t brow0 = row0 + i;                              // boundary b of sequence i: row brow0 + b
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lg = lane >> 4;
  const int row = 16 * wave + lj;
  const int64_t plane = static_cast<int64_t>(D) * D;
  const int j0 = sl * NS;
  const int64_t nrows = row0 + m.nrows <= A.rows_cap ? m.nrows : (A.rows_cap > row0 ? A.rows_cap - row0 : 0);
  // G at the last token: dL/dS_T, or zero
  for (int e = tid; e < NS * D / 4; e += 256) {
    const int jj = e / (D / 4), c4 = e % (D / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (A.d_state != nullptr)
      x = reinterpret_cast<const float4*>(A.d_state + (static_cast<int64_t>(i) * A.h_v + h) * plane +
                                          static_cast<int64_t>(j0 + jj) * D)[c4];
    *reinterpret_cast<float4*>(&S.gt[jj * SS + 4 * c4]) = x;
  }
  __syncthreads();
  auto store_g = [&](int64_t brow) {                           // the slice of G to boundary row brow
    if (brow >= A.adj_rows) return;
    for (int e = tid; e < NS * D / 4; e += 256) {
      const int jj = e / (D / 4), c4 = e % (D / 4);
      reinterpret_cast<float4*>(A.adjoint + (brow * A.h_v + h) * plane + static_cast<int64_t>(j0 + jj) * D)[c4] =
          *reinterpret_cast<const float4*>(&S.gt[jj * SS + 4 * c4]);
    }
  };
  store_g(brow0 + nrows);
  BwdRegs<D> R;
  if (nrows > 0) bwd_fetch<D>(A, m, row0, nrows - 1, h, kh, j0, R);
  for (int64_t c = nrows - 1; c >= 0; --c) {
    const int64_t wr = row0 + c;
    int t0, t1;
    chunk_range(m, c, A.chunk, &t0, &t1);
    const int n = t1 - t0;
    const int64_t tok = m.tok0 + t0;
    const float* bwb = A.fbw + (wr * A.h_v + h) * chunk_bwd_floats<D>();
    // commit the fetched Q^T (two consecutive tokens per thread: 32-bit stores) and log products
#pragma unroll
    for (int x = 0; x < BwdRegs<D>::QU; ++x) {
      const int e = tid + 256 * x, tp = e % (L / 2), c8 = e / (L / 2);
      if (e < (L / 2) * (D / 8)) {
#pragma unroll
        for (int y = 0; y < 8; ++y) {
          __bf16 pr[2] = {R.q[2 * x][y], R.q[2 * x + 1][y]};
          *reinterpret_cast<unsigned*>(&S.qt[(8 * c8 + y) * ST + 2 * tp]) = __builtin_bit_cast(unsigned, pr);
        }
      }
    }
    if (tid <= L) S.lgd[tid] = R.lg;
    // this chunk's T^T row fragments, in flight through the R step
    float4 tt[L / 32][2];
#pragma unroll
    for (int p = 0; p < L / 32; ++p) {
      const float4* src = reinterpret_cast<const float4*>(bwb + row * L + 32 * p + 8 * lg);
      tt[p][0] = src[0];
      tt[p][1] = src[1];
    }
    __syncthreads();
    // R = (the intra part) + diag(Gam_L / Gam) K G_L; R^T and (diag(Gam) dO)^T to LDS
    {
      f32x4c acc[NS / 16] = {};
#pragma unroll
      for (int p = 0; p < D / 32; ++p)
#pragma unroll
        for (int nt = 0; nt < NS / 16; ++nt)
          acc[nt] = mma_split_b(R.k[p], frag_f32(&S.gt[(16 * nt + lj) * SS + 32 * p + 8 * lg]), acc[nt]);
      const double lgL = S.lgd[n];
#pragma unroll
      for (int nt = 0; nt < NS / 16; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * wave + 4 * lg + r, jj = 16 * nt + lj;
          float rv = 0.f, ov = 0.f;
          if (t < n) {
            rv = R.ri[nt][r] + __expf(static_cast<float>(lgL - S.lgd[t + 1])) * acc[nt][r];
            ov = __expf(static_cast<float>(S.lgd[t + 1])) * R.dov[nt][r];
          }
          S.rt[jj * SF + t] = rv;
          S.ot[jj * SF + t] = ov;
        }
    }
    __syncthreads();
    if (c > 0) bwd_fetch<D>(A, m, row0, c - 1, h, kh, j0, R);  // the next chunk's inputs, in flight
    // dC = T^T R -> the dc buffer (the same elements this thread read as R's intra part)
    {
      f32x4c acc[NS / 16] = {};
#pragma unroll
      for (int p = 0; p < L / 32; ++p) {
        const Split af = split8(tt[p][0], tt[p][1]);
#pragma unroll
        for (int nt = 0; nt < NS / 16; ++nt)
          acc[nt] = mma_split(af, frag_f32(&S.rt[(16 * nt + lj) * SF + 32 * p + 8 * lg]), acc[nt]);
      }
#pragma unroll
      for (int nt = 0; nt < NS / 16; ++nt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 16 * wave + 4 * lg + r;
          if (t < n) A.dc[((tok + t) * A.h_v + h) * D + j0 + 16 * nt + lj] = acc[nt][r];
        }
    }
    // G^T <- Gam_L G^T + (diag(Gam) dO)^T Q - R^T W, and this wave's part of <G_0, S_0>
    const float gL = __expf(static_cast<float>(S.lgd[n]));
    const float* s0 = A.chunk_states + (wr * A.h_v + h) * plane;
    double hp = 0.0;
    constexpr int TILES = (NS / 16) * (D / 16);
#pragma unroll
    for (int q = 0; q < TILES / 4; ++q) {
      const int tile = wave * (TILES / 4) + q;
      const int jt = tile / (D / 16), dt = tile % (D / 16);
      float sv[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) sv[r] = s0[static_cast<int64_t>(j0 + 16 * jt + 4 * lg + r) * D + 16 * dt + lj];
      f32x4c u = {}, v = {};
#pragma unroll
      for (int p = 0; p < L / 32; ++p) {
        u = mma_split_a(frag_f32(&S.ot[(16 * jt + lj) * SF + 32 * p + 8 * lg]),
                        frag_bf16(&S.qt[(16 * dt + lj) * ST + 32 * p + 8 * lg]), u);
        v = mma_split(frag_f32(&S.rt[(16 * jt + lj) * SF + 32 * p + 8 * lg]),
                      frag_f32(bwb + L * L + (16 * dt + lj) * L + 32 * p + 8 * lg), v);
      }
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float& g = S.gt[(16 * jt + 4 * lg + r) * SS + 16 * dt + lj];
        const float ng = __builtin_fmaf(gL, g, u[r] - v[r]);
        g = ng;
        hp = __builtin_fma(static_cast<double>(ng), static_cast<double>(sv[r]), hp);
      }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) hp += __shfl_xor(hp, o, 64);
    if (lane == 0 && brow0 + c < A.adj_rows)
      A.hpart[((brow0 + c) * A.h_v + h) * A.hparts + sl * 4 + wave] = hp;
    __syncthreads();                                           // G^T complete; rt, ot, qt, lgd free
    store_g(brow0 + c);
  }
  if (A.d_state0 != nullptr) {
    for (int e = tid; e < NS * D / 4; e += 256) {
      const int jj = e / (D / 4), c4 = e % (D / 4);
      reinterpret_cast<float4*>(A.d_state0 + (static_cast<int64_t>(i) * A.h_v + h) * plane +
                                static_cast<int64_t>(j0 + jj) * D)[c4] = *reinterpret_cast<const float4*>(&S.gt[jj * SS + 4 * c4]);
    }
  }
}

template <int D>
static hipError_t launch_backward_chunked_t(const BackwardArgs& A, hipStream_t stream) {
  const int ratio = A.h_v / A.h_k;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0 && A.rows_cap > 0) {
    const int64_t g = xcd_grid(A.rows_cap * A.h_k, ratio);
    if (g > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((nbwd_intra_kernel<D>), dim3(static_cast<unsigned>(g)), dim3(256), 0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if (A.num_seqs > 0) {
    const int64_t g = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, ratio * (D / ChunkCfg<D>::NS));
    if (g > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((nbwd_state_kernel<D>), dim3(static_cast<unsigned>(g)), dim3(256), 0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return record_event(A.events, 1, stream);
}

hipError_t launch_backward_chunked(int d, const BackwardArgs& A, hipStream_t stream) {
  if (A.hparts != backward_chunked_parts(d)) return hipErrorInvalidValue;
  if (d == 32) return launch_backward_chunked_t<32>(A, stream);
  if (d == 64) return launch_backward_chunked_t<64>(A, stream);
  if (d == 128) return launch_backward_chunked_t<128>(A, stream);
  return hipErrorInvalidValue;
}

int backward_chunked_parts(int d) {
  if (d == 32) return bwd_state_parts<32>();
  if (d == 64) return bwd_state_parts<64>();
  if (d == 128) return bwd_state_parts<128>();
  return 0;
}

}  // namespace cpr
