// cpr_backward.hip -- gradients of the gated delta rule for the trainer, evaluated the CPR way.
//
// The per-layer table of "Solving the linear-attention headache" (IsoExec articles) times CPR for
// the trainer's forward and backward.  The backward mirrors the forward's two passes:
//   adjoint pass   G = dL/dS runs backward in time, G_{t-1} = a_t (G_t + q_t dO_t^T) + k_t du_t^T
//                  with du_t = -a_t b_t (G_t + q_t dO_t^T)^T k_t.  It needs no forward state and
//                  is column-independent, so, like pass 1, it runs each sequence's columns from the
//                  last token back to the end of chunk 0 and stores G at every chunk end.
//   gradient pass  one workgroup per (chunk, value head, column group): the chunk's forward states
//                  are replayed from the stashed chunk-start state (checkpoints every SUB tokens,
//                  the SUB states of a sub-chunk in registers), G is replayed from the stored
//                  chunk-end adjoint, and every token's dq, dk, dv, da, db follow.  dv is a
//                  per-column value and is stored directly; dq, dk, da, db sum over the value
//                  columns, so each workgroup stores its columns' sum (fixed pairwise order).
//   reduce         per (token, key head): dq, dk sum the partials of its value heads and column
//                  groups, da, db of a value head sum its column groups, all in a fixed pairwise
//                  order, so the gradients are bitwise reproducible for any batch or packing.
// Arithmetic (fp32, IEEE, round to nearest even; leaves and trees as in the forward schedule):
//   Ghat = fma(q_i, dO_j, G);  dc = tree(Ghat, k);  dw = b*dc;  du = (-a)*dw;
//   G    = fma(k_i, du, a*Ghat);  dv_j = dw;  db_j = dc*w;  da_j = fma(-dw, u, tree(Ghat, S_{t-1}));
//   dq_i = sum_j S_t[i][j]*dO_j;  dk_i = sum_j fma(S_{t-1}[i][j], du_j, Ghat[i][j]*c_j).
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

template <int DK, int DV>
struct BwdCfg {
  static constexpr int G = DK / kLeaf;                         // lanes per column, one leaf each
  static constexpr int R = kLeaf;
  static constexpr int WG_COLS = (256 / G < DV) ? 256 / G : DV;
  static constexpr int THREADS = WG_COLS * G;
  static constexpr int NCG = DV / WG_COLS;                     // column groups per value head
  static constexpr int TT = 16;                                // tokens per staged tile
  static constexpr int SUB = 8;                                // tokens per replayed sub-chunk
  static constexpr int MAXC = 64;                              // largest chunk supported
  static constexpr int NSUB = MAXC / SUB;
  static constexpr int PW = 2 * DK + 2;                        // partial: dq[DK], dk[DK], da, db
  static_assert(DV % WG_COLS == 0 && WG_COLS % 8 == 0, "shape");
};

template <int DK, int DV>
struct alignas(16) BwdLds {
  using Cfg = BwdCfg<DK, DV>;
  float k[Cfg::TT][DK];
  float q[Cfg::TT][DK];
  float v[Cfg::TT][Cfg::WG_COLS];
  float d[Cfg::TT][Cfg::WG_COLS];       // dO
  float2 ab[Cfg::TT];
  float rq[Cfg::WG_COLS][DK];           // per-column partials of dq and dk for one token
  float rk[Cfg::WG_COLS][DK];
  float2 rs[Cfg::WG_COLS];              // per-column da, db
};

// Stage tokens [t0, t0 + n) (packed indices, n <= TT) into LDS: k and q of key head kh, v and dO of
// the workgroup's columns of value head h, a and b.  Synchronous; the caller synchronises.
template <int DK, int DV, int IO, bool WITH_Q>
__device__ __forceinline__ void stage(const BackwardArgs& A, BwdLds<DK, DV>& L, int t0, int n, int kh, int h,
                                      int col0) {
  using Cfg = BwdCfg<DK, DV>;
  for (int u = threadIdx.x; u < n * (DK / 8); u += Cfg::THREADS) {
    const int tt = u / (DK / 8), c8 = u % (DK / 8);
    const int64_t e = (static_cast<int64_t>(t0 + tt) * A.h_k + kh) * DK + c8 * 8;
    float x[8];
    widen8<IO>(load_raw8<IO>(A.k, e), x);
    store_f32x8(&L.k[tt][c8 * 8], x);
    if constexpr (WITH_Q) {
      widen8<IO>(load_raw8<IO>(A.q, e), x);
      store_f32x8(&L.q[tt][c8 * 8], x);
    }
  }
  for (int u = threadIdx.x; u < n * (Cfg::WG_COLS / 8); u += Cfg::THREADS) {
    const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
    const int64_t e = (static_cast<int64_t>(t0 + tt) * A.h_v + h) * DV + col0 + c8 * 8;
    float x[8];
    widen8<IO>(load_raw8<IO>(A.v, e), x);
    store_f32x8(&L.v[tt][c8 * 8], x);
    if constexpr (WITH_Q) {
      widen8<IO>(load_raw8<IO>(A.d_o, e), x);
      store_f32x8(&L.d[tt][c8 * 8], x);
    }
  }
  for (int u = threadIdx.x; u < n; u += Cfg::THREADS) {
    const int64_t e = static_cast<int64_t>(t0 + u) * A.h_v + h;
    L.ab[u] = make_float2(A.a[e], A.b[e]);
  }
}

// ---- adjoint pass -------------------------------------------------------------------------------
template <int DK, int DV, int IO>
__global__ void __launch_bounds__((BwdCfg<DK, DV>::THREADS)) adjoint_pass_kernel(BackwardArgs A) {
  using Cfg = BwdCfg<DK, DV>;
  constexpr int G = Cfg::G;
  __shared__ BwdLds<DK, DV> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio * Cfg::NCG);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k), kh = static_cast<int>(gs.group % A.h_k);
  const int h = kh * ratio + gs.member / Cfg::NCG, cg = gs.member % Cfg::NCG;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = plan_row_offset(A, i, red);
  const int tid = threadIdx.x, lc = tid / G, g = tid % G;
  const int col0 = cg * Cfg::WG_COLS;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t off = static_cast<int64_t>(col0 + lc) * DK + g * Cfg::R;
  float Gs[Cfg::R];
  if (A.d_state != nullptr) {
    load_f32x8(A.d_state + (static_cast<int64_t>(i) * A.h_v + h) * plane + off, Gs);
  } else {
#pragma unroll
    for (int r = 0; r < Cfg::R; ++r) Gs[r] = 0.0f;
  }
  if (m.len == 0) {                                          // nothing to go through: dS0 = dS_T
    if (A.d_state0 != nullptr) store_f32x8(A.d_state0 + (static_cast<int64_t>(i) * A.h_v + h) * plane + off, Gs);
    return;
  }
  const int C = A.chunk;
  const int64_t last_row = row0 + m.nrows - 1;
  if (last_row < A.rows_cap) store_f32x8(A.adjoint + (last_row * A.h_v + h) * plane + off, Gs);
  // tokens from the last one down to the first token of chunk 1
  const int first = C;
  for (int t1 = m.len; t1 > first; t1 -= Cfg::TT) {
    const int t0 = t1 - Cfg::TT > first ? t1 - Cfg::TT : first;
    __syncthreads();
    stage<DK, DV, IO, true>(A, L, static_cast<int>(m.tok0) + t0, t1 - t0, kh, h, col0);
    __syncthreads();
    for (int tt = t1 - t0 - 1; tt >= 0; --tt) {
      float kr[Cfg::R], qr[Cfg::R], gh[Cfg::R];
      load_f32x8(&L.k[tt][g * Cfg::R], kr);
      load_f32x8(&L.q[tt][g * Cfg::R], qr);
      const float dO = L.d[tt][lc];
      const float2 ab = L.ab[tt];
#pragma unroll
      for (int r = 0; r < Cfg::R; ++r) gh[r] = __builtin_fmaf(qr[r], dO, Gs[r]);
      const float dc = pinned_dot<1, G>(gh, kr);
      const float dw = ab.y * dc;
      const float du = -ab.x * dw;
#pragma unroll
      for (int r = 0; r < Cfg::R; ++r) Gs[r] = __builtin_fmaf(kr[r], du, ab.x * gh[r]);
      const int t = t0 + tt;
      if (t % C == 0) {                                      // G is now dL/dS at the end of chunk t/C - 1
        const int64_t row = row0 + t / C - 1;
        if (row < A.rows_cap) store_f32x8(A.adjoint + (row * A.h_v + h) * plane + off, Gs);
      }
    }
  }
}

// ---- gradient pass ------------------------------------------------------------------------------
// Register checkpoints indexed by a block-uniform sub-chunk number, through constant indices only.
template <int R, int N, int M = 0>
__device__ __forceinline__ void ckpt_save(float (&cp)[N][R], int idx, const float (&s)[R]) {
  if constexpr (M < N) {
    if (idx == M) {
#pragma unroll
      for (int r = 0; r < R; ++r) cp[M][r] = s[r];
    } else {
      ckpt_save<R, N, M + 1>(cp, idx, s);
    }
  }
}

template <int R, int N, int M = 0>
__device__ __forceinline__ void ckpt_load(const float (&cp)[N][R], int idx, float (&s)[R]) {
  if constexpr (M < N) {
    if (idx == M) {
#pragma unroll
      for (int r = 0; r < R; ++r) s[r] = cp[M][r];
    } else {
      ckpt_load<R, N, M + 1>(cp, idx, s);
    }
  }
}

// Sum x over the WG_COLS column slots in a fixed balanced pairwise order.
template <int N>
__device__ __forceinline__ float pair_sum(float (&x)[N]) {
#pragma unroll
  for (int w = 1; w < N; w *= 2) {
#pragma unroll
    for (int l = 0; l + w < N; l += 2 * w) x[l] = x[l] + x[l + w];
  }
  return x[0];
}

template <int DK, int DV, int IO>
__global__ void __launch_bounds__((BwdCfg<DK, DV>::THREADS)) grad_chunk_kernel(BackwardArgs A) {
  using Cfg = BwdCfg<DK, DV>;
  constexpr int G = Cfg::G, R = Cfg::R, SUB = Cfg::SUB, NCOL = Cfg::WG_COLS;
  __shared__ BwdLds<DK, DV> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio * Cfg::NCG);
  const int64_t w = gs.group / A.h_k;
  const int kh = static_cast<int>(gs.group % A.h_k);
  const int h = kh * ratio + gs.member / Cfg::NCG, cg = gs.member % Cfg::NCG;
  if (w >= A.rows_cap) return;                               // uniform across the block
  int i;
  int64_t c;
  if (!plan_find_row(A, w, &i, &c, red)) return;             // uniform across the block
  const SeqMeta m = seq_meta(A, i);
  const int C = A.chunk;
  const int tb = static_cast<int>(c) * C;
  const int te = tb + C < m.len ? tb + C : m.len;
  const int tok0 = static_cast<int>(m.tok0);
  const int tid = threadIdx.x, lc = tid / G, g = tid % G;
  const int col0 = cg * Cfg::WG_COLS;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t off = static_cast<int64_t>(col0 + lc) * DK + g * R;

  float s[R], Gs[R];
  load_f32x8(A.chunk_states + (w * A.h_v + h) * plane + off, s);
  load_f32x8(A.adjoint + (w * A.h_v + h) * plane + off, Gs);

  // replay the chunk forward once, keeping the state entering every sub-chunk
  float cp[Cfg::NSUB][R];
  for (int t0 = tb; t0 < te; t0 += Cfg::TT) {
    const int n = te - t0 < Cfg::TT ? te - t0 : Cfg::TT;
    __syncthreads();
    stage<DK, DV, IO, false>(A, L, tok0 + t0, n, kh, h, col0);
    __syncthreads();
    for (int tt = 0; tt < n; ++tt) {
      const int j = t0 + tt - tb;
      if (j % SUB == 0) ckpt_save<R, Cfg::NSUB>(cp, j / SUB, s);
      float kr[R], u, ww, cc;
      load_f32x8(&L.k[tt][g * R], kr);
      const float2 ab = L.ab[tt];
      cpr_update<1, G>(s, kr, L.v[tt][lc], ab.x, ab.y, u, ww, cc);
    }
  }

  // sub-chunks from the last to the first: replay their states, then walk them backwards
  const int nsub = (te - tb + SUB - 1) / SUB;
  for (int sc = nsub - 1; sc >= 0; --sc) {
    const int ts = tb + sc * SUB;
    const int n = te - ts < SUB ? te - ts : SUB;
    __syncthreads();
    stage<DK, DV, IO, true>(A, L, tok0 + ts, n, kh, h, col0);
    __syncthreads();
    float st[SUB + 1][R], uu[SUB], wv[SUB], cv[SUB];
    ckpt_load<R, Cfg::NSUB>(cp, sc, st[0]);
#pragma unroll
    for (int j = 0; j < SUB; ++j) {
#pragma unroll
      for (int r = 0; r < R; ++r) st[j + 1][r] = st[j][r];
      if (j < n) {
        float kr[R];
        load_f32x8(&L.k[j][g * R], kr);
        const float2 ab = L.ab[j];
        cpr_update<1, G>(st[j + 1], kr, L.v[j][lc], ab.x, ab.y, uu[j], wv[j], cv[j]);
      }
    }
#pragma unroll
    for (int j = SUB - 1; j >= 0; --j) {
      if (j < n) {
        float kr[R], qr[R], gh[R], pq[R], pk[R];
        load_f32x8(&L.k[j][g * R], kr);
        load_f32x8(&L.q[j][g * R], qr);
        const float dO = L.d[j][lc];
        const float2 ab = L.ab[j];
#pragma unroll
        for (int r = 0; r < R; ++r) gh[r] = __builtin_fmaf(qr[r], dO, Gs[r]);
#pragma unroll
        for (int r = 0; r < R; ++r) pq[r] = st[j + 1][r] * dO;
        const float dc = pinned_dot<1, G>(gh, kr);
        const float dS = pinned_dot<1, G>(gh, st[j]);
        const float dw = ab.y * dc;
        const float du = -ab.x * dw;
        const float da_col = __builtin_fmaf(-dw, uu[j], dS);
        const float db_col = dc * wv[j];
#pragma unroll
        for (int r = 0; r < R; ++r) pk[r] = __builtin_fmaf(st[j][r], du, gh[r] * cv[j]);
#pragma unroll
        for (int r = 0; r < R; ++r) Gs[r] = __builtin_fmaf(kr[r], du, ab.x * gh[r]);
        const int t = tok0 + ts + j;
        if (g == 0) {
          A.dv[(static_cast<int64_t>(t) * A.h_v + h) * DV + col0 + lc] = dw;
          L.rs[lc] = make_float2(da_col, db_col);
        }
        store_f32x8(&L.rq[lc][g * R], pq);
        store_f32x8(&L.rk[lc][g * R], pk);
        __syncthreads();
        float* part = A.partial + ((static_cast<int64_t>(t) * A.h_v + h) * Cfg::NCG + cg) * Cfg::PW;
        for (int e = tid; e < Cfg::PW; e += Cfg::THREADS) {
          float x[NCOL];
          if (e < DK) {
#pragma unroll
            for (int l = 0; l < NCOL; ++l) x[l] = L.rq[l][e];
          } else if (e < 2 * DK) {
#pragma unroll
            for (int l = 0; l < NCOL; ++l) x[l] = L.rk[l][e - DK];
          } else if (e == 2 * DK) {
#pragma unroll
            for (int l = 0; l < NCOL; ++l) x[l] = L.rs[l].x;
          } else {
#pragma unroll
            for (int l = 0; l < NCOL; ++l) x[l] = L.rs[l].y;
          }
          part[e] = pair_sum<NCOL>(x);
        }
        __syncthreads();
      }
    }
  }
  if (c == 0 && A.d_state0 != nullptr)
    store_f32x8(A.d_state0 + (static_cast<int64_t>(i) * A.h_v + h) * plane + off, Gs);
}

// ---- reduce ---------------------------------------------------------------------------------------
// One workgroup per token.  dq and dk of a key head: each of its value heads' column-group
// partials summed pairwise, then the value heads added in head order.  da and db of a value head:
// its column-group partials summed pairwise.
template <int DK, int DV>
__global__ void __launch_bounds__(256) grad_reduce_kernel(BackwardArgs A) {
  using Cfg = BwdCfg<DK, DV>;
  constexpr int NCG = Cfg::NCG, PW = Cfg::PW;
  const int64_t t = blockIdx.x;
  if (t >= A.total_tokens) return;
  const int ratio = A.h_v / A.h_k;
  const float* pt = A.partial + t * A.h_v * NCG * PW;
  for (int e = threadIdx.x; e < A.h_k * 2 * DK; e += blockDim.x) {
    const int kh = e / (2 * DK), idx = e % (2 * DK);
    float acc = 0.0f;
    for (int m = 0; m < ratio; ++m) {
      const float* p = pt + (kh * ratio + m) * NCG * PW + idx;
      float x[NCG];
#pragma unroll
      for (int cg = 0; cg < NCG; ++cg) x[cg] = p[cg * PW];
      const float s = pair_sum<NCG>(x);
      acc = m == 0 ? s : acc + s;
    }
    float* out = idx < DK ? A.dq : A.dk;
    out[(t * A.h_k + kh) * DK + idx % DK] = acc;
  }
  for (int e = threadIdx.x; e < A.h_v * 2; e += blockDim.x) {
    const int h = e / 2, which = e % 2;
    const float* p = pt + h * NCG * PW + 2 * DK + which;
    float x[NCG];
#pragma unroll
    for (int cg = 0; cg < NCG; ++cg) x[cg] = p[cg * PW];
    (which == 0 ? A.da : A.db)[t * A.h_v + h] = pair_sum<NCG>(x);
  }
}

template <int DK, int DV, int IO>
static hipError_t launch_backward_t(const BackwardArgs& A, hipStream_t stream) {
  using Cfg = BwdCfg<DK, DV>;
  const int ratio = A.h_v / A.h_k;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0) {
    const int64_t g1 = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, ratio * Cfg::NCG);
    if (g1 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((adjoint_pass_kernel<DK, DV, IO>), dim3(static_cast<unsigned>(g1)), dim3(Cfg::THREADS), 0,
                       stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0 && A.rows_cap > 0) {
    const int64_t g2 = xcd_grid(A.rows_cap * A.h_k, ratio * Cfg::NCG);
    if (g2 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((grad_chunk_kernel<DK, DV, IO>), dim3(static_cast<unsigned>(g2)), dim3(Cfg::THREADS), 0, stream,
                       A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 2, stream)) != hipSuccess) return e;
  if (A.total_tokens > 0) {
    hipLaunchKernelGGL((grad_reduce_kernel<DK, DV>), dim3(static_cast<unsigned>(A.total_tokens)), dim3(256), 0, stream,
                       A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return record_event(A.events, 3, stream);
}

hipError_t launch_backward(int dk, int dv, int io, const BackwardArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_backward_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

int backward_column_groups(int dk, int dv) {
  if (dk == dv && (dk == 16 || dk == 32 || dk == 64 || dk == 128)) {
    switch (dk) {
      case 16: return BwdCfg<16, 16>::NCG;
      case 32: return BwdCfg<32, 32>::NCG;
      case 64: return BwdCfg<64, 64>::NCG;
      default: return BwdCfg<128, 128>::NCG;
    }
  }
  return 0;
}

}  // namespace cpr
