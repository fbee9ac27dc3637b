// cpr_chunked.hip -- the chunkwise (WY/UT) evaluation of the gated delta rule on bf16 matrix
// cores, used two ways:
//   native  every output from the chunk form: the pages' "native" column of the per-layer table
//           in "Solving the linear-attention headache" (IsoExec articles), the evaluation CPR is
//           compared against;
//   R2      the chunk form computes only the states at chunk starts (a value-changing boundary
//           pass); the outputs then come from the pinned per-token step started at those states
//           (the CPR output pass), the other reading of the CPR passes.
//
// Algebra, per chunk of L tokens with gate products Gam_t = a_1 ... a_t and entering state S_0:
//   the per-token write vectors c_t = b_t (v_t - a_t S_{t-1}^T k_t) satisfy
//       (I + A) C = diag(b) V - diag(b Gam) K S_0,   A[s][r] = b_s (Gam_s/Gam_r) k_s . k_r (r < s),
//   so with T = (I + A)^{-1}, W = T diag(b Gam) K and U = T diag(b) V:
//       C = U - W S_0,   S_L = Gam_L S_0 + K^T diag(Gam_L / Gam) C,
//       O = diag(Gam) Q S_0 + (M . Q K^T) C,   M[t][s] = Gam_t / Gam_s (s <= t).
// Kernels: prep (per chunk and value head: T by forward substitution in fp32, then W and U),
// state (per sequence, value head and column slice, sequential over the chunks: C and the next
// state), output (per chunk and value head: O).  Products run on v_mfma_f32_16x16x32_bf16 with
// fp32 accumulation; an operand that is not exactly bf16 is split into a bf16 high part and a
// bf16 low part and the product taken as hi*hi + hi*lo + lo*hi, which keeps fp32-level accuracy.
// Log gate products are summed in fp64; decay ratios are exp of their fp32 differences.
#include <hip/hip_runtime.h>

#include "cpr_chunk_form.hpp"
#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

// ---- prep: T, W, U per (chunk row, value head) ------------------------------------------------
template <int D>
struct alignas(16) PrepLds {
  using M = ChunkCfg<D>;
  float am[M::L * M::SF];       // A, then T
  float tp[M::L * M::SF];       // T, then T diag(b Gam), then T diag(b)
  union {
    float ty[M::L * M::SF];     // blocked-inverse scratch
    __bf16 kt[D * M::ST];       // then K^T (zero past the chunk)
    __bf16 vt[D * M::ST];       // then V^T
  };
  double lgd[M::L + 1];
  float bb[M::L];
};

// One (chunk row w, value head h) of the prep pass.  Uniform across the block; it returns early
// for rows with no work.
template <int D>
__device__ __forceinline__ void prep_item(const PrefillArgs& A, float* ws, PrepLds<D>& S, int64_t* red, int64_t w,
                                          int kh, int h) {
  using M = ChunkCfg<D>;
  constexpr int L = M::L, ST = M::ST, SF = M::SF, NT = D / 16;
  int i;
  int64_t c;
  if (A.gate != nullptr) {                                    // one row per sequence, run where gated in
    i = static_cast<int>(w);
    c = 0;
    if (A.gate[i] == 0) return;                               // uniform across the block
  } else if (!plan_find_row(A, w, &i, &c, red)) {
    return;                                                   // uniform across the block
  }
  const SeqMeta m = seq_meta(A, i);
  int t0, t1;
  chunk_range(m, c, A.chunk, &t0, &t1);
  const int n = t1 - t0;                                      // tokens, 1..64
  const int64_t tok = m.tok0 + t0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lg = lane >> 4;
  const __bf16* kin = static_cast<const __bf16*>(A.k);
  const __bf16* vin = static_cast<const __bf16*>(A.v);

  // K^T and V^T (zero past the chunk) into registers, committed to LDS once the inverse is done
  // with its scratch; gates and their log products
  TransposedRegs<D> kreg, vreg;
  fetch_transposed<D>(kreg, kin + kh * D, tok, static_cast<int64_t>(A.h_k) * D, n);
  fetch_transposed<D>(vreg, vin + static_cast<int64_t>(h) * D, tok, static_cast<int64_t>(A.h_v) * D, n);
  if (tid < L) {
    float a = 1.f, b = 0.f;
    if (tid < n) {
      a = A.a[(tok + tid) * A.h_v + h];
      b = A.b[(tok + tid) * A.h_v + h];
    }
    S.bb[tid] = b;
    double x = tid < n ? log(static_cast<double>(a)) : 0.0;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const double y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    S.lgd[tid + 1] = x;
    if (tid == 0) S.lgd[0] = 0.0;
  }
  __syncthreads();

  // A = strictly lower (b_s Gam_s / Gam_r) k_s . k_r, K rows read straight from memory
  {
    f32x4c acc[4] = {};
    const int ra = 16 * wave + lj;
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      bf16x8 af = {};
      if (ra < n) af = *reinterpret_cast<const bf16x8*>(kin + ((tok + ra) * A.h_k + kh) * D + 32 * p + 8 * lg);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int rb = 16 * nt + lj;
        bf16x8 bfr = {};
        if (rb < n) bfr = *reinterpret_cast<const bf16x8*>(kin + ((tok + rb) * A.h_k + kh) * D + 32 * p + 8 * lg);
        acc[nt] = mma(af, bfr, acc[nt]);
      }
    }
    // the log products of this lane's rows and columns, read before any use (unconditional reads
    // issue together)
    double lrow[4], lcol[4];
    float brow[4];
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      lrow[x] = S.lgd[16 * wave + 4 * lg + x + 1];
      brow[x] = S.bb[16 * wave + 4 * lg + x];
      lcol[x] = S.lgd[16 * x + lj + 1];
    }
#pragma unroll
    for (int nt = 0; nt < 4; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 16 * wave + 4 * lg + r, rr = 16 * nt + lj;
        float v = 0.f;
        if (rr < s && s < n) v = brow[r] * __expf(static_cast<float>(lrow[r] - lcol[nt])) * acc[nt][r];
        S.am[s * SF + rr] = v;
      }
  }
  __syncthreads();
  // T = (I + A)^{-1} (unit lower triangular), blocked: the four 16 x 16 diagonal blocks by
  // forward substitution, then the off-diagonal blocks level by level, X = -T_B A_BA T_A
  if (tid < L) {                                               // column j of block bk in registers
    const int bk = tid >> 4, j = tid & 15, o0 = 16 * bk;
    float tc[16];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      float acc = s == j ? 1.f : 0.f;
#pragma unroll
      for (int r = 0; r < s; ++r) acc = __builtin_fmaf(-S.am[(o0 + s) * SF + o0 + r], tc[r], acc);   // tc[r] = 0 for r < j
      tc[s] = s < j ? 0.f : acc;
    }
#pragma unroll
    for (int s = 0; s < 16; ++s) S.tp[(o0 + s) * SF + o0 + j] = tc[s];
  }
  for (int e = tid; e < L * L; e += 256) {                     // zero the off-diagonal blocks
    const int t = e / L, s = e % L;
    if ((t >> 4) != (s >> 4)) S.tp[t * SF + s] = 0.f;
  }
  __syncthreads();
  for (int half = 16; half < L; half *= 2) {
    // pairs of half x half blocks at offsets (q, q + half), q = 0, 2 half, ...; 16 x 16 tiles of
    // the off-diagonal block, one wave per tile, on fp32 matrix cores
    const int tps = (half / 16) * (half / 16), ntiles = (L / (2 * half)) * tps;
    // Y = A_BA T_A
    for (int tile = wave; tile < ntiles; tile += 4) {
      const int q = 2 * half * (tile / tps), it = (tile % tps) / (half / 16), jt = tile % (half / 16);
      f32x4c acc = {};
      for (int kk = 0; kk < half / 4; ++kk)
        acc = mma_f32(S.am[(q + half + 16 * it + lj) * SF + q + 4 * kk + lg],
                      S.tp[(q + 4 * kk + lg) * SF + q + 16 * jt + lj], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) S.ty[(q + half + 16 * it + 4 * lg + r) * SF + q + 16 * jt + lj] = acc[r];
    }
    __syncthreads();
    // X = -T_B Y
    for (int tile = wave; tile < ntiles; tile += 4) {
      const int q = 2 * half * (tile / tps), it = (tile % tps) / (half / 16), jt = tile % (half / 16);
      f32x4c acc = {};
      for (int kk = 0; kk < half / 4; ++kk)
        acc = mma_f32(S.tp[(q + half + 16 * it + lj) * SF + q + half + 4 * kk + lg],
                      S.ty[(q + half + 4 * kk + lg) * SF + q + 16 * jt + lj], acc);
#pragma unroll
      for (int r = 0; r < 4; ++r) S.tp[(q + half + 16 * it + 4 * lg + r) * SF + q + 16 * jt + lj] = -acc[r];
    }
    __syncthreads();
  }
  // keep T in am; tp = T diag(b Gam); K^T into the scratch's space
  for (int e = tid; e < L * L; e += 256) {
    const int t = e / L, s = e % L;
    const float tv = S.tp[t * SF + s];
    S.am[t * SF + s] = tv;
    S.tp[t * SF + s] = tv * (S.bb[s] * __expf(static_cast<float>(S.lgd[s + 1])));
  }
  commit_transposed<D, ST>(S.kt, kreg);
  __syncthreads();
  float* wsb = ws + (w * A.h_v + h) * chunk_ws_floats<D>();
  float* bwb = A.chunk_bwd != nullptr ? A.chunk_bwd + (w * A.h_v + h) * chunk_bwd_floats<D>() : nullptr;
  if (bwb != nullptr)                                          // T^T for the backward: row t holds T[.][t]
    for (int e = tid; e < L * L; e += 256) bwb[e] = S.am[(e % L) * SF + e / L];
  // W = T diag(b Gam) K, then U = T diag(b) V
  for (int which = 0; which < 2; ++which) {
    f32x4c acc[NT] = {};
#pragma unroll
    for (int p = 0; p < L / 32; ++p) {
      const Split af = frag_f32(&S.tp[(16 * wave + lj) * SF + 32 * p + 8 * lg]);
#pragma unroll
      for (int nt = 0; nt < NT; ++nt) {
        const __bf16* bt = which == 0 ? S.kt : S.vt;
        acc[nt] = mma_split_a(af, frag_bf16(&bt[(16 * nt + lj) * ST + 32 * p + 8 * lg]), acc[nt]);
      }
    }
    float* dst = wsb + which * M::WS_MAT;
#pragma unroll
    for (int nt = 0; nt < NT; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) dst[(16 * wave + 4 * lg + r) * D + 16 * nt + lj] = acc[nt][r];
    if (which == 0 && bwb != nullptr) {                        // W^T for the backward: [D][L]
#pragma unroll
      for (int nt = 0; nt < NT; ++nt)
        *reinterpret_cast<float4*>(bwb + L * L + (16 * nt + lj) * L + 16 * wave + 4 * lg) =
            make_float4(acc[nt][0], acc[nt][1], acc[nt][2], acc[nt][3]);
    }
    if (which == 0) {
      __syncthreads();                                         // K^T and tp reads done
      for (int e = tid; e < L * L; e += 256) {
        const int t = e / L, s = e % L;
        S.tp[t * SF + s] = S.am[t * SF + s] * S.bb[s];
      }
      commit_transposed<D, ST>(S.vt, vreg);                    // V^T over K^T
      __syncthreads();
    }
  }
  double* lgw = reinterpret_cast<double*>(wsb + 3 * M::WS_MAT);
  for (int e = tid; e <= L; e += 256) lgw[e] = S.lgd[e];
}

template <int D>
__global__ void __launch_bounds__(256) chunk_prep_kernel(PrefillArgs A, float* ws) {
  __shared__ PrepLds<D> S;
  __shared__ int64_t red[6];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio);
  const int64_t w = gs.group / A.h_k;
  const int kh = static_cast<int>(gs.group % A.h_k);
  if (w >= A.rows_cap) return;                                // uniform across the block
  prep_item<D>(A, ws, S, red, w, kh, kh * ratio + gs.member);
}

// The prep pass over the rows of a listed set of sequences only (one row each, A.gate set): the
// workgroups take (listed sequence, value head) items in turn, so the grid need not cover every
// sequence.  list[0 .. *count) are sequence indices.
template <int D>
__global__ void __launch_bounds__(256) chunk_prep_list_kernel(PrefillArgs A, float* ws, const int32_t* list,
                                                              const int32_t* count) {
  __shared__ PrepLds<D> S;
  __shared__ int64_t red[6];
  const int ratio = A.h_v / A.h_k;
  const int64_t items = static_cast<int64_t>(*count < A.num_seqs ? *count : A.num_seqs) * A.h_v;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int h = static_cast<int>(it % A.h_v);
    prep_item<D>(A, ws, S, red, list[it / A.h_v], h / ratio, h);
    __syncthreads();                                          // LDS free for the next item
  }
}

// ---- state: sequential over chunks per (sequence, value head, column slice) ---------------------
template <int D>
struct alignas(16) StateLds {
  using M = ChunkCfg<D>;
  float st[M::NS * M::SS];      // S^T slice [column][d]
  float ct[M::NS * M::SF];      // diag(Gam_L / Gam) C, transposed: [column][token]
  __bf16 kt[D * M::ST];         // K^T of the chunk
  double lgd[M::L + 1];
};

// One chunk's inputs of the state pass, loaded ahead into registers.
template <int D>
struct StateRegs {
  using M = ChunkCfg<D>;
  static constexpr int KU = ((M::L / 2) * (D / 8) + 255) / 256;   // token pairs of 8 K columns per thread
  bf16x8 k[2 * KU];
  float4 w[D / 32][2];                                         // W fragments of this lane's row
  float u[M::NS / 16][4];                                      // U at this lane's C positions
  double lg;                                                   // lgd[tid] (threads 0..L)
};

template <int D>
__device__ __forceinline__ void state_fetch(const PrefillArgs& A, const float* ws, const SeqMeta& m, int64_t row0,
                                            int64_t c, int h, int kh, int j0, StateRegs<D>& R) {
  using M = ChunkCfg<D>;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lg = lane >> 4;
  int t0, t1;
  chunk_range(m, c, A.chunk, &t0, &t1);
  const int n = t1 - t0;
  const int64_t tok = m.tok0 + t0;
  const __bf16* kin = static_cast<const __bf16*>(A.k);
#pragma unroll
  for (int x = 0; x < StateRegs<D>::KU; ++x) {
    const int e = tid + 256 * x, t = 2 * (e % (M::L / 2)), c8 = e / (M::L / 2);
    R.k[2 * x] = R.k[2 * x + 1] = bf16x8{};
    if (e < (M::L / 2) * (D / 8)) {
      if (t < n) R.k[2 * x] = *reinterpret_cast<const bf16x8*>(kin + ((tok + t) * A.h_k + kh) * D + 8 * c8);
      if (t + 1 < n) R.k[2 * x + 1] = *reinterpret_cast<const bf16x8*>(kin + ((tok + t + 1) * A.h_k + kh) * D + 8 * c8);
    }
  }
  const float* wsb = ws + ((row0 + c) * A.h_v + h) * chunk_ws_floats<D>();
#pragma unroll
  for (int p = 0; p < D / 32; ++p) {
    const float4* src = reinterpret_cast<const float4*>(wsb + (16 * wave + lj) * D + 32 * p + 8 * lg);
    R.w[p][0] = src[0];
    R.w[p][1] = src[1];
  }
#pragma unroll
  for (int nt = 0; nt < M::NS / 16; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) R.u[nt][r] = wsb[M::WS_MAT + (16 * wave + 4 * lg + r) * D + j0 + 16 * nt + lj];
  R.lg = tid <= M::L ? reinterpret_cast<const double*>(wsb + 3 * M::WS_MAT)[tid] : 0.0;
}

// One (sequence i, value head h, column slice sl) of the state pass.  Uniform across the block;
// it returns early for sequences with no work.
template <int D>
__device__ __forceinline__ void state_item(const PrefillArgs& A, float* ws, int write_final, StateLds<D>& S,
                                           int64_t* red, int i, int kh, int h, int sl) {
  using M = ChunkCfg<D>;
  constexpr int L = M::L, NS = M::NS, SS = M::SS, SF = M::SF, ST = M::ST;
  if (A.gate != nullptr && A.gate[i] == 0) return;            // uniform across the block
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = A.gate != nullptr ? i : plan_row_offset(A, i, red);
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lg = lane >> 4;
  const int64_t plane = static_cast<int64_t>(D) * D;
  const int j0 = sl * NS;
  if (m.slot < 0) return;                                      // uniform: nothing to do
  // chunks whose workspace exists (rows beyond the launch's capacity are never planned)
  const int64_t nrows = row0 + m.nrows <= A.rows_cap ? m.nrows : (A.rows_cap > row0 ? A.rows_cap - row0 : 0);
  StateRegs<D> R;
  if (nrows > 0) state_fetch<D>(A, ws, m, row0, 0, h, kh, j0, R);
  // the entering state: the slot's (continuation; from state_in when given) or zero
  const float* sin = A.state_in != nullptr ? A.state_in : A.state;
  for (int e = tid; e < NS * D / 4; e += 256) {
    const int jj = e / (D / 4), c4 = e % (D / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (A.from_state) x = reinterpret_cast<const float4*>(sin + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane +
                                                          static_cast<int64_t>(j0 + jj) * D)[c4];
    *reinterpret_cast<float4*>(&S.st[jj * SS + 4 * c4]) = x;
  }
  __syncthreads();
  for (int64_t c = 0; c < nrows; ++c) {
    const int64_t w = row0 + c;
    int t0, t1;
    chunk_range(m, c, A.chunk, &t0, &t1);
    const int n = t1 - t0;
    // the state entering this chunk -> its chunk-state row (when rows are kept)
    for (int e = tid; A.chunk_states != nullptr && e < NS * D / 4; e += 256) {
      const int jj = e / (D / 4), c4 = e % (D / 4);
      reinterpret_cast<float4*>(A.chunk_states + (w * A.h_v + h) * plane + static_cast<int64_t>(j0 + jj) * D)[c4] =
          *reinterpret_cast<const float4*>(&S.st[jj * SS + 4 * c4]);
    }
    // commit the fetched K^T (two consecutive tokens per thread: 32-bit stores) and log products
#pragma unroll
    for (int x = 0; x < StateRegs<D>::KU; ++x) {
      const int e = tid + 256 * x, tp = e % (L / 2), c8 = e / (L / 2);
      if (e < (L / 2) * (D / 8)) {
#pragma unroll
        for (int y = 0; y < 8; ++y) {
          __bf16 pr[2] = {R.k[2 * x][y], R.k[2 * x + 1][y]};
          *reinterpret_cast<unsigned*>(&S.kt[(8 * c8 + y) * ST + 2 * tp]) = __builtin_bit_cast(unsigned, pr);
        }
      }
    }
    if (tid <= L) S.lgd[tid] = R.lg;
    // P = W S: rows 16 wave.., columns j0 + 16 nt + j
    f32x4c acc[NS / 16] = {};
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      const Split af = split8(R.w[p][0], R.w[p][1]);
#pragma unroll
      for (int nt = 0; nt < NS / 16; ++nt) acc[nt] = mma_split(af, frag_f32(&S.st[(16 * nt + lj) * SS + 32 * p + 8 * lg]), acc[nt]);
    }
    float uc[NS / 16][4];
#pragma unroll
    for (int nt = 0; nt < NS / 16; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) uc[nt][r] = R.u[nt][r];
    __syncthreads();                                           // kt, lgd committed; st reads done
    if (c + 1 < nrows) state_fetch<D>(A, ws, m, row0, c + 1, h, kh, j0, R);   // next chunk, in flight
    // C = U - P; C^T to the workspace (and, for the backward, every token's c); diag(Gam_L / Gam) C^T
    // to LDS
    float* wsb = ws + (w * A.h_v + h) * chunk_ws_floats<D>();
    const double lgL = S.lgd[n];
    float* cst = A.c_stash != nullptr ? A.c_stash + ((m.tok0 + t0) * A.h_v + h) * D + j0 : nullptr;
#pragma unroll
    for (int nt = 0; nt < NS / 16; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * lg + r, jj = 16 * nt + lj;
        const float cv = uc[nt][r] - acc[nt][r];
        wsb[2 * M::WS_MAT + (j0 + jj) * L + t] = cv;
        if (cst != nullptr && t < n) cst[static_cast<int64_t>(t) * A.h_v * D + jj] = cv;
        S.ct[jj * SF + t] = t < n ? cv * __expf(static_cast<float>(lgL - S.lgd[t + 1])) : 0.f;
      }
    __syncthreads();
    // S^T <- Gam_L S^T + (diag(Gam_L/Gam) C)^T K
    const float gL = __expf(static_cast<float>(lgL));
    constexpr int TILES = (NS / 16) * (D / 16);
#pragma unroll
    for (int q = 0; q < TILES / 4; ++q) {
      const int tile = wave * (TILES / 4) + q;
      const int jt = tile / (D / 16), dt = tile % (D / 16);
      f32x4c u = {};
#pragma unroll
      for (int p = 0; p < L / 32; ++p)
        u = mma_split_a(frag_f32(&S.ct[(16 * jt + lj) * SF + 32 * p + 8 * lg]),
                        frag_bf16(&S.kt[(16 * dt + lj) * ST + 32 * p + 8 * lg]), u);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        float& sv = S.st[(16 * jt + 4 * lg + r) * SS + 16 * dt + lj];
        sv = __builtin_fmaf(gL, sv, u[r]);
      }
    }
    __syncthreads();
  }
  if (write_final || m.len == 0) {                             // an empty sequence keeps its entering state
    for (int e = tid; e < NS * D / 4; e += 256) {
      const int jj = e / (D / 4), c4 = e % (D / 4);
      reinterpret_cast<float4*>(A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane +
                                static_cast<int64_t>(j0 + jj) * D)[c4] = *reinterpret_cast<const float4*>(&S.st[jj * SS + 4 * c4]);
    }
  }
}

template <int D>
__global__ void __launch_bounds__(256) chunk_state_kernel(PrefillArgs A, float* ws, int write_final) {
  constexpr int NSL = D / ChunkCfg<D>::NS;                     // column slices per value head
  __shared__ StateLds<D> S;
  __shared__ int64_t red[6];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio * NSL);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k), kh = static_cast<int>(gs.group % A.h_k);
  state_item<D>(A, ws, write_final, S, red, i, kh, kh * ratio + gs.member / NSL, gs.member % NSL);
}

// The state pass over a listed set of sequences only (A.gate set): the workgroups take (listed
// sequence, value head, column slice) items in turn.  list[0 .. *count) are sequence indices.
template <int D>
__global__ void __launch_bounds__(256) chunk_state_list_kernel(PrefillArgs A, float* ws, int write_final,
                                                               const int32_t* list, const int32_t* count) {
  constexpr int NSL = D / ChunkCfg<D>::NS;
  __shared__ StateLds<D> S;
  __shared__ int64_t red[6];
  const int ratio = A.h_v / A.h_k;
  const int64_t per = static_cast<int64_t>(A.h_v) * NSL;
  const int64_t items = static_cast<int64_t>(*count < A.num_seqs ? *count : A.num_seqs) * per;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    const int r = static_cast<int>(it % per), h = r / NSL;
    state_item<D>(A, ws, write_final, S, red, list[it / per], h / ratio, h, r % NSL);
    __syncthreads();                                          // LDS free for the next item
  }
}

// ---- output: O = diag(Gam) Q S_0 + (M . Q K^T) C per (chunk row, value head) ------------------------
template <int D>
struct alignas(16) OutLds {
  using M = ChunkCfg<D>;
  float qk[M::L * M::SF];       // M . Q K^T
  __bf16 q[M::L * M::SB];       // Q rows (zero past the chunk)
  __bf16 k[M::L * M::SB];       // K rows (zero past the chunk)
  double lgd[M::L + 1];
};

// One workgroup per (chunk row, value head).  Wave w first forms rows [16 w, 16 w + 16) of
// M . Q K^T; then the 4 D/16 (row block, column tile) output tiles are dealt out so that each
// wave owns whole column tiles (D >= 64) or half of one (D = 32): the S_0 and C^T fragments of a
// column tile are read from memory by one wave only, once (the first tile's before anything
// else, so that those loads overlap the staging and M . Q K^T), and Q, K and M . Q K^T come from
// LDS.
// Each output element's products run in one fixed order (Q S_0 over the D/32 blocks, the row's
// Gam, then (M . Q K^T) C) whichever wave forms it, so the bits do not depend on the mapping.
template <int D>
__global__ void __launch_bounds__(256) chunk_output_kernel(PrefillArgs A, const float* ws) {
  using M = ChunkCfg<D>;
  constexpr int L = M::L, SF = M::SF, SB = M::SB, NT = D / 16;
  static_assert(NT % 2 == 0, "column tiles");
  __shared__ OutLds<D> S;
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
  const int n = t1 - t0;
  const int64_t tok = m.tok0 + t0;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lg = lane >> 4;
  const __bf16* qin = static_cast<const __bf16*>(A.q);
  const __bf16* kin = static_cast<const __bf16*>(A.k);
  const float* wsb = ws + (w * A.h_v + h) * chunk_ws_floats<D>();
  const double* lgw = reinterpret_cast<const double*>(wsb + 3 * M::WS_MAT);
  const float* s0 = A.chunk_states + (w * A.h_v + h) * static_cast<int64_t>(D) * D;
  const float* ctw = wsb + 2 * M::WS_MAT;                      // C^T [D][L]
  Split sf[D / 32], cf[L / 32];                                // S_0 and C^T fragments of a column tile
  auto fetch_tile = [&](int nt) {
#pragma unroll
    for (int p = 0; p < D / 32; ++p) sf[p] = frag_f32(s0 + (16 * nt + lj) * D + 32 * p + 8 * lg);
#pragma unroll
    for (int p = 0; p < L / 32; ++p) cf[p] = frag_f32(ctw + (16 * nt + lj) * L + 32 * p + 8 * lg);
  };
  fetch_tile(wave * NT / 4);
  for (int e = tid; e <= L; e += 256) S.lgd[e] = lgw[e];
  // Q and K rows to LDS (exact bf16; zero past the chunk), 8 values per unit
  for (int e = tid; e < L * (D / 8); e += 256) {
    const int t = e / (D / 8), c8 = e % (D / 8);
    bf16x8 x = {}, y = {};
    if (t < n) {
      x = *reinterpret_cast<const bf16x8*>(qin + ((tok + t) * A.h_k + kh) * D + 8 * c8);
      y = *reinterpret_cast<const bf16x8*>(kin + ((tok + t) * A.h_k + kh) * D + 8 * c8);
    }
    *reinterpret_cast<bf16x8*>(&S.q[t * SB + 8 * c8]) = x;
    *reinterpret_cast<bf16x8*>(&S.k[t * SB + 8 * c8]) = y;
  }
  __syncthreads();
  // M . Q K^T -> LDS, rows of this wave's block
  {
    const int row = 16 * wave + lj;
    f32x4c acc[4] = {};
#pragma unroll
    for (int p = 0; p < D / 32; ++p) {
      const bf16x8 qf = frag_bf16(&S.q[row * SB + 32 * p + 8 * lg]);
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) acc[nt] = mma(qf, frag_bf16(&S.k[(16 * nt + lj) * SB + 32 * p + 8 * lg]), acc[nt]);
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
        float v = 0.f;
        if (s <= t && t < n) v = __expf(static_cast<float>(lrow[r] - lcol[nt])) * acc[nt][r];
        S.qk[t * SF + s] = v;
      }
  }
  __syncthreads();
  // O = diag(Gam) Q S_0 + (M . Q K^T) C: wave w takes tiles w NT .. w NT + NT - 1 of the 4 NT
  // (column tile it / 4, row block it % 4)
  unsigned short* o = static_cast<unsigned short*>(A.o);
#pragma unroll
  for (int k = 0; k < NT; ++k) {
    const int it = wave * NT + k, nt = it / 4, rb = it % 4;
    if (k > 0 && rb == 0) fetch_tile(nt);                      // this wave's next column tile
    const int row = 16 * rb + lj;
    f32x4c acc = {};
#pragma unroll
    for (int p = 0; p < D / 32; ++p) acc = mma_split_b(frag_bf16(&S.q[row * SB + 32 * p + 8 * lg]), sf[p], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[r] *= __expf(static_cast<float>(S.lgd[16 * rb + 4 * lg + r + 1]));
#pragma unroll
    for (int p = 0; p < L / 32; ++p) acc = mma_split(frag_f32(&S.qk[row * SF + 32 * p + 8 * lg]), cf[p], acc);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int t = 16 * rb + 4 * lg + r;
      if (t < n) o[((tok + t) * A.h_v + h) * D + 16 * nt + lj] = f32_to_bf16_rne(acc[r]);
    }
  }
}

// ---- R2 resynchronisation in decode -----------------------------------------------------------
// Under the R2 reading a chunk-start state is the chunk form's state, computed from the previous
// chunk-start state over the chunk's tokens, and the tokens in between run the pinned per-token
// step from it.  A decode step keeps, per slot, the chunk-start state of the chunk its last token
// fell in (the pool's boundary record) and that chunk's tokens so far (the ring, indexed by
// position mod C).  When a slot reaches the next chunk start, the chunk form over the ring's C
// tokens from the recorded state gives the new chunk-start state: the same chunk_prep and
// chunk_state kernels as the chunked prefill, run over the ring as a batch of one-chunk sequences
// (one per slot, gated to the slots at a chunk start), so the state has the bits a chunked R2
// prefill over the same tokens computes.  The decode step then applies the token from it and
// records it, and the token is appended to the ring.

// Ring layout (num_slots x C token positions): q, k [S C][H_k][D] bf16, v [S C][H_v][D] bf16,
// a, b [S C][H_v] fp32, each part 256-byte aligned.
struct RingParts {
  __bf16* q;
  __bf16* k;
  __bf16* v;
  float* a;
  float* b;
};

static int64_t pad256(int64_t x) { return (x + 255) / 256 * 256; }

int64_t r2_ring_bytes(int h_k, int h_v, int d, int chunk, int num_slots) {
  const int64_t n = static_cast<int64_t>(num_slots) * chunk;
  return 2 * pad256(n * h_k * d * 2) + pad256(n * h_v * d * 2) + 2 * pad256(n * h_v * 4);
}

static RingParts ring_parts(void* ring, int h_k, int h_v, int d, int chunk, int num_slots) {
  const int64_t n = static_cast<int64_t>(num_slots) * chunk;
  char* p = static_cast<char*>(ring);
  RingParts r;
  r.q = reinterpret_cast<__bf16*>(p);
  p += pad256(n * h_k * d * 2);
  r.k = reinterpret_cast<__bf16*>(p);
  p += pad256(n * h_k * d * 2);
  r.v = reinterpret_cast<__bf16*>(p);
  p += pad256(n * h_v * d * 2);
  r.a = reinterpret_cast<float*>(p);
  p += pad256(n * h_v * 4);
  r.b = reinterpret_cast<float*>(p);
  return r;
}

// Workspace: the one-chunk batch's cu_seqlens [S + 1], slot ids [S], gate [S] (int32), positions
// [S] (int64, zero), then the chunk-form workspace of S rows.
struct R2Work {
  int32_t* cu;
  int32_t* ids;
  int32_t* gate;
  int64_t* vpos;
  int32_t* list;     // the slots gated in this step, in any order
  int32_t* lent;     // their batch entries, in the same order
  int32_t* count;    // how many
  float* ws;
};

int64_t r2_workspace_bytes(int h_v, int d, int num_slots) {
  const int64_t S = num_slots;
  return pad256((S + 1) * 4) + 2 * pad256(S * 4) + pad256(S * 8) + 2 * pad256(S * 4) + pad256(4) +
         S * h_v * chunked_workspace_floats(d) * 4;
}

static R2Work r2_work(void* work, int num_slots) {
  const int64_t S = num_slots;
  char* p = static_cast<char*>(work);
  R2Work w;
  w.cu = reinterpret_cast<int32_t*>(p);
  p += pad256((S + 1) * 4);
  w.ids = reinterpret_cast<int32_t*>(p);
  p += pad256(S * 4);
  w.gate = reinterpret_cast<int32_t*>(p);
  p += pad256(S * 4);
  w.vpos = reinterpret_cast<int64_t*>(p);
  p += pad256(S * 8);
  w.list = reinterpret_cast<int32_t*>(p);
  p += pad256(S * 4);
  w.lent = reinterpret_cast<int32_t*>(p);
  p += pad256(S * 4);
  w.count = reinterpret_cast<int32_t*>(p);
  p += pad256(4);
  w.ws = reinterpret_cast<float*>(p);
  return w;
}

// The one-chunk batch over every slot, then the step's slots that stand at a chunk start with a
// chunk behind them gated in and listed.  One workgroup: the list is built by a block scan in batch
// order, so it needs no atomics.
constexpr int kR2PrepareThreads = 1024;

__global__ void __launch_bounds__(kR2PrepareThreads) r2_prepare_kernel(R2Work W, const int32_t* slot_ids, int batch,
                                                                      const int64_t* pos, int num_slots, int chunk) {
  __shared__ int64_t red[kR2PrepareThreads / 64 + 2];
  for (int s = threadIdx.x; s <= num_slots; s += kR2PrepareThreads) {
    W.cu[s] = s * chunk;
    if (s < num_slots) {
      W.ids[s] = s;
      W.gate[s] = 0;
      W.vpos[s] = 0;
    }
  }
  __syncthreads();                                            // every gate cleared before any is set
  int64_t listed = 0;
  for (int base = 0; base < batch; base += kR2PrepareThreads) {   // uniform across the block
    const int j = base + static_cast<int>(threadIdx.x);
    int32_t s = -1;
    if (j < batch) {
      s = slot_ids[j];
      if (s < 0 || s >= num_slots) {
        s = -1;
      } else {
        const int64_t p = pos[s];
        if (!(p > 0 && p % chunk == 0)) s = -1;
      }
    }
    int64_t total;
    const int64_t at = listed + block_excl_scan_i64(s >= 0 ? 1 : 0, red, &total);
    if (s >= 0) {
      W.gate[s] = 1;
      if (at < num_slots) {                                   // a slot listed twice could overflow it
        W.list[at] = s;
        W.lent[at] = j;
      }
    }
    listed += total;
  }
  if (threadIdx.x == 0) *W.count = static_cast<int32_t>(listed < num_slots ? listed : num_slots);
}

// After the step, which leaves the positions alone here: each listed slot's token to ring position
// pos mod C, then its position advanced.  One workgroup per batch entry.
template <int D>
__global__ void __launch_bounds__(256) r2_ring_append_kernel(DecodeArgs A, RingParts R) {
  const int j = blockIdx.x;
  const int32_t s = A.slot_ids[j];
  if (s < 0 || s >= A.num_slots) return;                      // uniform across the block
  const int64_t p = A.pos[s];
  if (p >= 0) {
    const int64_t dst = static_cast<int64_t>(s) * A.chunk + p % A.chunk;
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(A.q) + static_cast<int64_t>(j) * A.h_k * D);
    const uint4* k = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(A.k) + static_cast<int64_t>(j) * A.h_k * D);
    const uint4* v = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(A.v) + static_cast<int64_t>(j) * A.h_v * D);
    uint4* rq = reinterpret_cast<uint4*>(R.q + dst * A.h_k * D);
    uint4* rk = reinterpret_cast<uint4*>(R.k + dst * A.h_k * D);
    uint4* rv = reinterpret_cast<uint4*>(R.v + dst * A.h_v * D);
    for (int e = threadIdx.x; e < A.h_k * D / 8; e += 256) {
      rq[e] = q[e];
      rk[e] = k[e];
    }
    for (int e = threadIdx.x; e < A.h_v * D / 8; e += 256) rv[e] = v[e];
    for (int e = threadIdx.x; e < A.h_v; e += 256) {
      R.a[dst * A.h_v + e] = A.a[static_cast<int64_t>(j) * A.h_v + e];
      R.b[dst * A.h_v + e] = A.b[static_cast<int64_t>(j) * A.h_v + e];
    }
  }
  __syncthreads();                                            // every thread has read the position
  if (threadIdx.x == 0) A.pos[s] = p + 1;
}

// After a chunked R2 prefill (before its position update): each sequence's tokens from the start
// of its last chunk on go to the ring, and the state entering that chunk (its last chunk-state
// row) to the boundary record.  One workgroup per sequence.
template <int D>
__global__ void __launch_bounds__(256) r2_ring_fill_kernel(PrefillArgs A, RingParts R, float* boundary,
                                                           int64_t* boundary_pos) {
  __shared__ int64_t red[6];
  const int i = blockIdx.x;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = plan_row_offset(A, i, red);
  if (m.slot < 0 || m.len == 0) return;                      // uniform across the block
  const int64_t C = A.chunk, p_end = m.p0 + m.len;
  const int64_t bpos = (p_end - 1) / C * C, first = bpos > m.p0 ? bpos : m.p0;
  for (int64_t p = first; p < p_end; ++p) {
    const int64_t src = m.tok0 + (p - m.p0), dst = static_cast<int64_t>(m.slot) * C + p % C;
    const uint4* q = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(A.q) + src * A.h_k * D);
    const uint4* k = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(A.k) + src * A.h_k * D);
    const uint4* v = reinterpret_cast<const uint4*>(static_cast<const __bf16*>(A.v) + src * A.h_v * D);
    uint4* rq = reinterpret_cast<uint4*>(R.q + dst * A.h_k * D);
    uint4* rk = reinterpret_cast<uint4*>(R.k + dst * A.h_k * D);
    uint4* rv = reinterpret_cast<uint4*>(R.v + dst * A.h_v * D);
    for (int e = threadIdx.x; e < A.h_k * D / 8; e += 256) {
      rq[e] = q[e];
      rk[e] = k[e];
    }
    for (int e = threadIdx.x; e < A.h_v * D / 8; e += 256) rv[e] = v[e];
    for (int e = threadIdx.x; e < A.h_v; e += 256) {
      R.a[dst * A.h_v + e] = A.a[src * A.h_v + e];
      R.b[dst * A.h_v + e] = A.b[src * A.h_v + e];
    }
  }
  const int64_t row = row0 + m.nrows - 1;
  if (row >= A.rows_cap) return;
  const int64_t plane = static_cast<int64_t>(A.h_v) * D * D;
  const float4* srow = reinterpret_cast<const float4*>(A.chunk_states + row * plane);
  float4* brow = reinterpret_cast<float4*>(boundary + static_cast<int64_t>(m.slot) * plane);
  for (int64_t e = threadIdx.x; e < plane / 4; e += 256) brow[e] = srow[e];
  if (threadIdx.x == 0) boundary_pos[m.slot] = bpos;
}

// Workgroups of the list-driven chunk-form kernels in an R2 decode step, two per CU: a step's
// usual few slots at a chunk start give a few hundred state-pass items, one turn each.
constexpr int64_t kR2ListGrid = 512;

template <int D>
static hipError_t launch_decode_r2_t(const DecodeArgs& A, void* ring, void* work, hipStream_t stream,
                                     hipStream_t side, hipEvent_t fork, hipEvent_t join) {
  using M = ChunkCfg<D>;
  const int S = A.num_slots;
  const RingParts R = ring_parts(ring, A.h_k, A.h_v, D, A.chunk, S);
  const R2Work W = r2_work(work, S);
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess || A.batch == 0) return e != hipSuccess ? e : record_event(A.events, 1, stream);
  hipLaunchKernelGGL(r2_prepare_kernel, dim3(1), dim3(kR2PrepareThreads), 0, stream, W, A.slot_ids, A.batch, A.pos, S,
                     A.chunk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // With a second stream, the listed slots' chain (chunk form, then their step) runs there, beside
  // the step of every other slot, whose state stream it would otherwise wait for.
  const bool split = side != nullptr;
  if (split &&
      ((e = hipEventRecord(fork, stream)) != hipSuccess || (e = hipStreamWaitEvent(side, fork, 0)) != hipSuccess))
    return e;
  const hipStream_t cs = split ? side : stream;
  // the chunk form over every gated slot's ring: recorded chunk-start state in, new one into the slot
  PrefillArgs F{};
  F.cu = W.cu;
  F.slot_ids = W.ids;
  F.pos = W.vpos;
  F.pos_out = W.vpos;
  F.q = R.q; F.k = R.k; F.v = R.v; F.a = R.a; F.b = R.b;
  F.o = nullptr;
  F.state = A.state;
  F.state_in = A.boundary;
  F.chunk_states = nullptr;
  F.total_tokens = static_cast<int64_t>(S) * A.chunk;
  F.rows_cap = S;
  F.num_seqs = S;
  F.num_slots = S;
  F.from_state = 1;
  F.h_k = A.h_k; F.h_v = A.h_v; F.chunk = A.chunk;
  F.gate = W.gate;
  // grids sized for a few slots at a chunk start (the usual case); the workgroups take the listed
  // slots' items in turn, so more slots only take more turns
  const int64_t np = static_cast<int64_t>(S) * A.h_v, ns = np * (D / M::NS);
  const unsigned gp = static_cast<unsigned>(np < kR2ListGrid ? np : kR2ListGrid);
  const unsigned gs = static_cast<unsigned>(ns < kR2ListGrid ? ns : kR2ListGrid);
  hipLaunchKernelGGL((chunk_prep_list_kernel<D>), dim3(gp), dim3(256), 0, cs, F, W.ws, W.list, W.count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((chunk_state_list_kernel<D>), dim3(gs), dim3(256), 0, cs, F, W.ws, 1, W.list, W.count);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // the token from that state (recorded at the chunk start), then the ring and the positions
  DecodeArgs B = A;
  B.events = nullptr;
  B.skip_advance = 1;
  if (split) {
    // the listed entries' step after their chunk form; every other slot's step meanwhile
    const int64_t gl = A.max_wgs > 0 && A.max_wgs < kR2ListGrid ? A.max_wgs : kR2ListGrid;
    if ((e = launch_decode_list(D, D, IO_BF16, B, W.lent, W.count, static_cast<unsigned>(gl), cs)) != hipSuccess)
      return e;
    if ((e = hipEventRecord(join, cs)) != hipSuccess) return e;
    B.skip_slot = W.gate;
    if ((e = launch_decode(D, D, IO_BF16, B, stream)) != hipSuccess) return e;
    if ((e = hipStreamWaitEvent(stream, join, 0)) != hipSuccess) return e;
  } else {
    if ((e = launch_decode(D, D, IO_BF16, B, stream)) != hipSuccess) return e;
  }
  hipLaunchKernelGGL((r2_ring_append_kernel<D>), dim3(static_cast<unsigned>(A.batch)), dim3(256), 0, stream, A, R);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return record_event(A.events, 1, stream);
}

hipError_t launch_decode_r2(int d, const DecodeArgs& A, void* ring, void* work, hipStream_t stream,
                            hipStream_t side, hipEvent_t fork, hipEvent_t join) {
  if (d == 32) return launch_decode_r2_t<32>(A, ring, work, stream, side, fork, join);
  if (d == 64) return launch_decode_r2_t<64>(A, ring, work, stream, side, fork, join);
  if (d == 128) return launch_decode_r2_t<128>(A, ring, work, stream, side, fork, join);
  return hipErrorInvalidValue;
}

template <int D>
static hipError_t launch_chunked_t(const PrefillArgs& A, float* ws, int mode, hipStream_t stream) {
  using M = ChunkCfg<D>;
  const int ratio = A.h_v / A.h_k;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0 && A.rows_cap > 0) {
    const int64_t g = xcd_grid(A.rows_cap * A.h_k, ratio);
    if (g > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((chunk_prep_kernel<D>), dim3(static_cast<unsigned>(g)), dim3(256), 0, stream, A, ws);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0) {
    const int64_t g = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, ratio * (D / M::NS));
    if (g > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((chunk_state_kernel<D>), dim3(static_cast<unsigned>(g)), dim3(256), 0, stream, A, ws,
                       mode == 0 ? 1 : 0);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 2, stream)) != hipSuccess) return e;
  if (mode == 0) {
    if (A.num_seqs > 0 && A.rows_cap > 0) {
      const int64_t g = xcd_grid(A.rows_cap * A.h_k, ratio);
      hipLaunchKernelGGL((chunk_output_kernel<D>), dim3(static_cast<unsigned>(g)), dim3(256), 0, stream, A,
                         static_cast<const float*>(ws));
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = launch_prefill_finish(A, stream)) != hipSuccess) return e;
  } else {
    // R2: the CPR output pass (pinned per-token step) from the chunk-form states just stored; with a
    // decode ring attached, each sequence's last chunk goes to the ring and its entering state to
    // the boundary record before the positions move
    if (A.r2_ring == nullptr) {
      if ((e = launch_output_pass(D, D, IO_BF16, A, stream)) != hipSuccess) return e;
    } else {
      if ((e = launch_output_pass_only(D, D, IO_BF16, A, stream)) != hipSuccess) return e;
      const RingParts R = ring_parts(A.r2_ring, A.h_k, A.h_v, D, A.chunk, A.num_slots);
      if (A.num_seqs > 0) {
        hipLaunchKernelGGL((r2_ring_fill_kernel<D>), dim3(static_cast<unsigned>(A.num_seqs)), dim3(256), 0, stream, A,
                           R, A.r2_boundary, A.r2_boundary_pos);
        if ((e = hipGetLastError()) != hipSuccess) return e;
      }
      if ((e = launch_prefill_finish(A, stream)) != hipSuccess) return e;
    }
  }
  return record_event(A.events, 3, stream);
}

hipError_t launch_prefill_chunked(int dk, int dv, int io, const PrefillArgs& A, void* ws, int mode, hipStream_t stream) {
  if (io != IO_BF16 || dk != dv) return hipErrorInvalidValue;
  float* w = static_cast<float*>(ws);
  if (dk == 32) return launch_chunked_t<32>(A, w, mode, stream);
  if (dk == 64) return launch_chunked_t<64>(A, w, mode, stream);
  if (dk == 128) return launch_chunked_t<128>(A, w, mode, stream);
  return hipErrorInvalidValue;
}

int64_t chunked_bwd_floats(int d) {
  if (d == 32) return chunk_bwd_floats<32>();
  if (d == 64) return chunk_bwd_floats<64>();
  if (d == 128) return chunk_bwd_floats<128>();
  return 0;
}

int64_t chunked_workspace_floats(int d) {
  if (d == 32) return chunk_ws_floats<32>();
  if (d == 64) return chunk_ws_floats<64>();
  if (d == 128) return chunk_ws_floats<128>();
  return 0;
}

}  // namespace cpr
