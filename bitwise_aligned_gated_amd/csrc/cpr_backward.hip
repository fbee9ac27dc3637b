// cpr_backward.hip -- gradients of the gated delta rule for the trainer.
//
// The per-layer table of "Solving the linear-attention headache" (IsoExec articles) times CPR for
// the trainer's forward and backward.  The pages give no backward; this is reverse-mode
// differentiation of the recurrence
//     u_t = S_{t-1}^T k_t,  w_t = v_t - a_t u_t,  c_t = b_t w_t,  S_t = a_t S_{t-1} + k_t c_t^T,
//     o_t = S_t^T q_t,
// evaluated in four kernels over the forward's stash of chunk-start states.
//
// adjoint (column-parallel, one token at a time, last token first)
//     G = dL/dS satisfies G_{t-1} = a_t (I - b_t k_t k_t^T) Ghat_t with Ghat_t = G_t + q_t dO_t^T;
//     it needs no forward state.  Each (sequence, value head, column group) walks its tokens
//     backward and writes dc_t = Ghat_t^T k_t for every token, G at every chunk boundary, and
//     dL/dS_0.
// replay (column-parallel, one chunk per workgroup)
//     the forward step of the shared pinned schedule from the stashed chunk-start state, writing
//     c_t and w_t for every token: the same bits the forward computed.  Skipped when the trainer
//     forward kept them.
// per-token gradients (streaming, D/8 lanes per (token, value head))
//     dv_t = b_t dc_t, db_t = dc_t . w_t and v_t . dv_t for the h recurrence below.
// chunk gradients (matrix cores, one workgroup per (chunk, key head))
//     Inside a chunk with gate products Gam_t = a_1 ... a_t, every state and adjoint is the
//     chunk-start (or chunk-end) matrix plus rank-one terms, so with dU_t = -a_t b_t dc_t
//       dq_t = Gam_t S_0 dO_t + sum_{s<=t} (Gam_t/Gam_s) k_s (c_s . dO_t)
//       dk_t = (Gam_L/Gam_t) G_L c_t + sum_{s>=t} (Gam_s/Gam_t) q_s (dO_s . c_t)
//            + Gam_{t-1} S_0 dU_t + sum_{s<t} (Gam_{t-1}/Gam_s) k_s (c_s . dU_t)
//            + sum_{s>t} (Gam_{s-1}/Gam_t) k_s (dU_s . c_t)
//     which are dense products on 16x16x4 fp32 MFMA tiles with decay-masked L x L factors.  The
//     remaining gradients are per token: dv_t = b_t dc_t, db_t = dc_t . w_t, and
//     a_t da_t = <G_{t-1}, S_{t-1}> =: h_{t-1}, where h_0 = <G at the chunk start, S_0> and
//     h_t = h_{t-1} - q_t . dq_t + v_t . (b_t dc_t) (the per-value-head dq), accumulated in fp64.
//     h_0 is formed by the adjoint pass, which holds G at the chunk start anyway: each wave adds its
//     lanes' part of <G, S_0> (S_0 prefetched from the stash a chunk ahead) and stores it, and the
//     chunk-gradient pass adds the parts in a fixed order.
//     dq and dk of a key head accumulate its value heads in head order in the workgroup's
//     matrix-core accumulators, and are stored once.
// Every sum has a fixed order, so the gradients are bitwise reproducible for any batch
// composition or packing.
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

// ---- column-parallel passes ------------------------------------------------------------------
template <int DK, int DV>
struct ColCfg {
  static constexpr int G = DK / kLeaf;                         // lanes per column, one leaf each
  static constexpr int R = kLeaf;
  static constexpr int WG_COLS = (256 / G < DV) ? 256 / G : DV;
  static constexpr int THREADS = WG_COLS * G;
  static constexpr int NCG = DV / WG_COLS;                     // column groups per value head
  static constexpr int TT = 16;                                // tokens per staged tile
  static constexpr int WAVES = (THREADS + 63) / 64;
  static constexpr int PARTS = NCG * WAVES;                    // parts of <G, S_0> per chunk and head
  static_assert(DV % WG_COLS == 0 && WG_COLS % 8 == 0, "shape");
};

template <int D>
__host__ __device__ constexpr int adjoint_parts_of() {
  return ColCfg<D, D>::PARTS;
}

int adjoint_parts(int d) {
  switch (d) {
    case 16: return ColCfg<16, 16>::PARTS;
    case 32: return ColCfg<32, 32>::PARTS;
    case 64: return ColCfg<64, 64>::PARTS;
    case 128: return ColCfg<128, 128>::PARTS;
    default: return 0;
  }
}

template <int DK, int DV>
struct alignas(16) ColLds {
  using Cfg = ColCfg<DK, DV>;
  float k[Cfg::TT][DK];                 // lane-interleaved rows (kq_slot)
  float q[Cfg::TT][DK];
  float v[Cfg::TT][Cfg::WG_COLS];
  float d[Cfg::TT][Cfg::WG_COLS];       // dO
  float2 ab[Cfg::TT];
  float out0[Cfg::TT][Cfg::WG_COLS];    // per-token column values awaiting a coalesced store
  float out1[Cfg::TT][Cfg::WG_COLS];
};

// Stage tokens [t0, t0 + n) (packed indices, n <= TT): k (and q) of key head kh, v (and dO) of
// the workgroup's columns of value head h, a and b.  The caller synchronises around it.
template <int DK, int DV, int IO, bool WITH_Q>
__device__ __forceinline__ void stage(const BackwardArgs& A, ColLds<DK, DV>& L, int64_t t0, int n, int kh, int h,
                                      int col0) {
  using Cfg = ColCfg<DK, DV>;
  for (int u = threadIdx.x; u < n * (DK / 8); u += Cfg::THREADS) {
    const int tt = u / (DK / 8), c8 = u % (DK / 8);
    const int64_t e = ((t0 + tt) * A.h_k + kh) * DK + c8 * 8;
    float x[8];
    widen8<IO>(load_raw8<IO>(A.k, e), x);
    store_kq8<Cfg::G, Cfg::R>(&L.k[tt][0], c8 * 8, x);
    if constexpr (WITH_Q) {
      widen8<IO>(load_raw8<IO>(A.q, e), x);
      store_kq8<Cfg::G, Cfg::R>(&L.q[tt][0], c8 * 8, x);
    }
  }
  for (int u = threadIdx.x; u < n * (Cfg::WG_COLS / 8); u += Cfg::THREADS) {
    const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
    const int64_t e = ((t0 + tt) * A.h_v + h) * DV + col0 + c8 * 8;
    float x[8];
    widen8<IO>(load_raw8<IO>(A.v, e), x);
    store_f32x8(&L.v[tt][c8 * 8], x);
    if constexpr (WITH_Q) {
      widen8<IO>(load_raw8<IO>(A.d_o, e), x);
      store_f32x8(&L.d[tt][c8 * 8], x);
    }
  }
  for (int u = threadIdx.x; u < n; u += Cfg::THREADS) {
    const int64_t e = (t0 + u) * A.h_v + h;
    L.ab[u] = make_float2(A.a[e], A.b[e]);
  }
}

// Store the staged per-token column values of tokens [t0, t0 + n) to dst [N][H_v][DV] (fp32).
template <int DK, int DV>
__device__ __forceinline__ void store_cols(const BackwardArgs& A,
                                           const float (&src)[ColCfg<DK, DV>::TT][ColCfg<DK, DV>::WG_COLS],
                                           float* dst, int64_t t0, int n, int h, int col0) {
  using Cfg = ColCfg<DK, DV>;
  for (int e = threadIdx.x; e < n * Cfg::WG_COLS; e += Cfg::THREADS) {
    const int tt = e / Cfg::WG_COLS, col = e % Cfg::WG_COLS;
    dst[((t0 + tt) * A.h_v + h) * DV + col0 + col] = src[tt][col];
  }
}

// One tile's inputs of the adjoint, loaded ahead into registers (raw io units).
template <int DK, int DV, int IO>
struct AdjRegs {
  using Cfg = ColCfg<DK, DV>;
  static constexpr int KU = (Cfg::TT * DK / 8 + Cfg::THREADS - 1) / Cfg::THREADS;
  static constexpr int VU = (Cfg::TT * Cfg::WG_COLS / 8 + Cfg::THREADS - 1) / Cfg::THREADS;
  static constexpr int AU = (2 * Cfg::TT + Cfg::THREADS - 1) / Cfg::THREADS;
  Raw8<IO> k[KU], q[KU], v[VU], d[VU];
  float ab[AU];
};

// Fetch tokens [t0, t0 + n) (packed indices, n <= TT).  Tile bases are uniform and each lane's
// offsets within a tile do not depend on t0; units past n keep what they held (no token reads
// them) and are never read from memory.
template <int DK, int DV, int IO>
__device__ __forceinline__ void adj_fetch(const BackwardArgs& A, AdjRegs<DK, DV, IO>& R, int64_t t0, int n, int kh,
                                          int h, int col0) {
  using Cfg = ColCfg<DK, DV>;
  constexpr int64_t ES = IO == IO_F32 ? 4 : 2;
  const int tid = threadIdx.x;
  const char* kb = static_cast<const char*>(A.k) + (t0 * A.h_k + kh) * DK * ES;
  const char* qb = static_cast<const char*>(A.q) + (t0 * A.h_k + kh) * DK * ES;
  const char* vb = static_cast<const char*>(A.v) + ((t0 * A.h_v + h) * DV + col0) * ES;
  const char* db = static_cast<const char*>(A.d_o) + ((t0 * A.h_v + h) * DV + col0) * ES;
  const float* ga = A.a + t0 * A.h_v + h;
  const float* gb = A.b + t0 * A.h_v + h;
#pragma unroll
  for (int x = 0; x < AdjRegs<DK, DV, IO>::KU; ++x) {
    const int u = tid + x * Cfg::THREADS, tt = u / (DK / 8), c8 = u % (DK / 8);
    const uint32_t off = static_cast<uint32_t>(tt * A.h_k * DK + c8 * 8);
    if (u < Cfg::TT * DK / 8 && tt < n) {
      R.k[x] = load_raw8<IO>(kb, off);
      R.q[x] = load_raw8<IO>(qb, off);
    }
  }
#pragma unroll
  for (int x = 0; x < AdjRegs<DK, DV, IO>::VU; ++x) {
    const int u = tid + x * Cfg::THREADS, tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
    const uint32_t off = static_cast<uint32_t>(tt * A.h_v * DV + c8 * 8);
    if (u < Cfg::TT * Cfg::WG_COLS / 8 && tt < n) {
      R.v[x] = load_raw8<IO>(vb, off);
      R.d[x] = load_raw8<IO>(db, off);
    }
  }
#pragma unroll
  for (int x = 0; x < AdjRegs<DK, DV, IO>::AU; ++x) {
    const int u = tid + x * Cfg::THREADS, tt = u % Cfg::TT;
    const uint32_t off = static_cast<uint32_t>(tt * A.h_v);
    if (tt < n) {                    // lanes [0, TT) fetch a, lanes [TT, 2 TT) fetch b
      if (u < Cfg::TT)
        R.ab[x] = ga[off];
      else if (u < 2 * Cfg::TT)
        R.ab[x] = gb[off];
    }
  }
}

template <int DK, int DV, int IO>
__device__ __forceinline__ void adj_commit(const AdjRegs<DK, DV, IO>& R, ColLds<DK, DV>& L) {
  using Cfg = ColCfg<DK, DV>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int x = 0; x < AdjRegs<DK, DV, IO>::KU; ++x) {
    const int u = tid + x * Cfg::THREADS, tt = u / (DK / 8), c8 = u % (DK / 8);
    if (u < Cfg::TT * DK / 8) {
      float y[8];
      widen8<IO>(R.k[x], y);
      store_kq8<Cfg::G, Cfg::R>(&L.k[tt][0], c8 * 8, y);
      widen8<IO>(R.q[x], y);
      store_kq8<Cfg::G, Cfg::R>(&L.q[tt][0], c8 * 8, y);
    }
  }
#pragma unroll
  for (int x = 0; x < AdjRegs<DK, DV, IO>::VU; ++x) {
    const int u = tid + x * Cfg::THREADS, tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
    if (u < Cfg::TT * Cfg::WG_COLS / 8) {
      float y[8];
      widen8<IO>(R.v[x], y);
      store_f32x8(&L.v[tt][c8 * 8], y);
      widen8<IO>(R.d[x], y);
      store_f32x8(&L.d[tt][c8 * 8], y);
    }
  }
#pragma unroll
  for (int x = 0; x < AdjRegs<DK, DV, IO>::AU; ++x) {
    const int u = tid + x * Cfg::THREADS;
    if (u < Cfg::TT)
      L.ab[u].x = R.ab[x];
    else if (u < 2 * Cfg::TT)
      L.ab[u - Cfg::TT].y = R.ab[x];
  }
}

// adjoint: one workgroup per (sequence, value head, column group), grouped per key head.
template <int DK, int DV, int IO>
__global__ void __launch_bounds__((ColCfg<DK, DV>::THREADS)) adjoint_kernel(BackwardArgs A) {
  using Cfg = ColCfg<DK, DV>;
  constexpr int G = Cfg::G, R = Cfg::R;
  __shared__ ColLds<DK, DV> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio * Cfg::NCG);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k), kh = static_cast<int>(gs.group % A.h_k);
  const int h = kh * ratio + gs.member / Cfg::NCG, cg = gs.member % Cfg::NCG;
  const SeqMeta m = seq_meta(A, i);
  const int64_t brow0 = plan_row_offset(A, i, red) + i;   // boundary b of sequence i: row brow0 + b
  const int tid = threadIdx.x, lc = tid / G, g = tid % G;
  const int col0 = cg * Cfg::WG_COLS;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t off = static_cast<int64_t>(col0 + lc) * DK + g * R;
  float Gs[R];
  if (A.d_state != nullptr) {
    load_f32x8(A.d_state + (static_cast<int64_t>(i) * A.h_v + h) * plane + off, Gs);
  } else {
#pragma unroll
    for (int r = 0; r < R; ++r) Gs[r] = 0.0f;
  }
  const int C = A.chunk;
  // the boundary at the last token (position len) holds dL/dS_T
  if (brow0 + m.nrows < A.adj_rows) store_f32x8(A.adjoint + ((brow0 + m.nrows) * A.h_v + h) * plane + off, Gs);
  // tiles of TT tokens from the last one back: the tile ending at t1 starts at max(t1 - TT, 0);
  // the next tile's inputs are fetched into registers while this one runs
  AdjRegs<DK, DV, IO> Rg = {};
  if (m.len > 0) {
    const int t0 = m.len - Cfg::TT > 0 ? m.len - Cfg::TT : 0;
    adj_fetch<DK, DV, IO>(A, Rg, m.tok0 + t0, m.len - t0, kh, h, col0);
    adj_commit<DK, DV, IO>(Rg, L);
  }
  // the stash row of the chunk start the walk reaches next (the last chunk's first), a chunk ahead
  const int64_t srow0 = brow0 - i;                           // chunk c of sequence i: stash row srow0 + c
  float sb[R];
  if (m.len > 0) load_f32x8(A.chunk_states + ((srow0 + (m.len - 1) / C) * A.h_v + h) * plane + off, sb);
  __syncthreads();
  for (int t1 = m.len; t1 > 0; t1 -= Cfg::TT) {
    const int t0 = t1 - Cfg::TT > 0 ? t1 - Cfg::TT : 0;
    const int n = t1 - t0;
    const bool more = t0 > 0;
    if (more) {
      const int p0 = t0 - Cfg::TT > 0 ? t0 - Cfg::TT : 0;
      adj_fetch<DK, DV, IO>(A, Rg, m.tok0 + p0, t0 - p0, kh, h, col0);
    }
    // token t0 + tt leaves G at dL/dS of position t0 + tt, a boundary when that is a multiple of
    // C; rem counts down to it.  Each token's dc goes to LDS at the start of the next one, so that
    // the lane-masked write does not split a token's own arithmetic.
    int rem = __builtin_amdgcn_readfirstlane((t1 - 1) % C);
    int64_t brow = brow0 + (t1 - 1) / C;
    float pdc = 0.0f;
    int ptt = -1;
    auto token = [&](int tt) {
      float kr[R], qr[R], gh[R];
      lds_read_kq<G, R>(&L.k[tt][0], g, kr);
      lds_read_kq<G, R>(&L.q[tt][0], g, qr);
      const float dO = L.d[tt][lc];
      const float2 ab = L.ab[tt];
      if (ptt >= 0 && g == 0) L.out0[ptt][lc] = pdc;
#pragma unroll
      for (int r = 0; r < R; ++r) gh[r] = __builtin_fmaf(qr[r], dO, Gs[r]);
      const float dc = pinned_dot<1, G>(gh, kr);
      const float du = -ab.x * (ab.y * dc);
#pragma unroll
      for (int r = 0; r < R; ++r) Gs[r] = __builtin_fmaf(kr[r], du, ab.x * gh[r]);
      pdc = dc;
      ptt = tt;
      if (rem == 0) {                                        // G is now dL/dS at a chunk boundary
        if (brow < A.adj_rows) {
          store_f32x8(A.adjoint + (brow * A.h_v + h) * plane + off, Gs);
          // this wave's part of <G, S> at the chunk start: rows in order, then a lane butterfly
          double hp = 0.0;
#pragma unroll
          for (int r = 0; r < R; ++r) hp = __builtin_fma(static_cast<double>(Gs[r]), static_cast<double>(sb[r]), hp);
#pragma unroll
          for (int o = (Cfg::THREADS < 64 ? Cfg::THREADS : 64) / 2; o >= 1; o >>= 1) hp += __shfl_xor(hp, o, 64);
          if ((tid & 63) == 0)
            A.hpart[(brow * A.h_v + h) * Cfg::PARTS + cg * Cfg::WAVES + (tid >> 6)] = hp;
          if (brow > brow0)                                  // the next chunk start's row, a chunk ahead
            load_f32x8(A.chunk_states + ((brow - 1 - i) * A.h_v + h) * plane + off, sb);
        }
        rem = C;
        --brow;
      }
      --rem;
    };
    if (n == Cfg::TT) {                                      // full tile: unrolled, immediate offsets
#pragma unroll
      for (int tt = Cfg::TT - 1; tt >= 0; --tt) token(tt);
    } else {
      for (int tt = n - 1; tt >= 0; --tt) token(tt);
    }
    if (g == 0) L.out0[ptt][lc] = pdc;
    __syncthreads();
    store_cols<DK, DV>(A, L.out0, A.dc, m.tok0 + t0, n, h, col0);
    if (more) adj_commit<DK, DV, IO>(Rg, L);
    __syncthreads();
  }
  if (A.d_state0 != nullptr) store_f32x8(A.d_state0 + (static_cast<int64_t>(i) * A.h_v + h) * plane + off, Gs);
}

// replay: one workgroup per (chunk, value head, column group), grouped per key head.
template <int DK, int DV, int IO>
__global__ void __launch_bounds__((ColCfg<DK, DV>::THREADS)) replay_kernel(BackwardArgs A) {
  using Cfg = ColCfg<DK, DV>;
  constexpr int G = Cfg::G, R = Cfg::R;
  __shared__ ColLds<DK, DV> L;
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
  const int tb = static_cast<int>(c) * A.chunk;
  const int te = tb + A.chunk < m.len ? tb + A.chunk : m.len;
  const int tid = threadIdx.x, lc = tid / G, g = tid % G;
  const int col0 = cg * Cfg::WG_COLS;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  float s[R];
  load_f32x8(A.chunk_states + (w * A.h_v + h) * plane + static_cast<int64_t>(col0 + lc) * DK + g * R, s);
  for (int t0 = tb; t0 < te; t0 += Cfg::TT) {
    const int n = te - t0 < Cfg::TT ? te - t0 : Cfg::TT;
    __syncthreads();
    stage<DK, DV, IO, false>(A, L, m.tok0 + t0, n, kh, h, col0);
    __syncthreads();
    for (int tt = 0; tt < n; ++tt) {
      float kr[R], u, ww, cc;
      lds_read_kq<G, R>(&L.k[tt][0], g, kr);
      const float2 ab = L.ab[tt];
      cpr_update<1, G>(s, kr, L.v[tt][lc], ab.x, ab.y, u, ww, cc);
      if (g == 0) {
        L.out0[tt][lc] = cc;
        L.out1[tt][lc] = ww;
      }
    }
    __syncthreads();
    store_cols<DK, DV>(A, L.out0, A.cc, m.tok0 + t0, n, h, col0);
    store_cols<DK, DV>(A, L.out1, A.ww, m.tok0 + t0, n, h, col0);
  }
}

// ---- chunk gradients on matrix cores --------------------------------------------------------
// v_mfma_f32_16x16x4f32 on a wave of 64 lanes, lane l = j + 16 g (j < 16, g < 4):
//   A (16 x 4): lane holds A[j][g];  B (4 x 16): lane holds B[g][j];
//   D (16 x 16): lane holds D[4 g + r][j] in register r.
// In a product over a k range, a lane of group g feeds the k values 16 p + 4 g + e (e < 4) of
// panel p, so that its A elements are four consecutive columns of a row.
typedef float f32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

template <int D>
struct MCfg {
  static constexpr int L = 64;                  // token rows of a chunk tile: 4 waves x 16
  static constexpr int SB = D + 4;              // row stride of D-wide matrices in LDS
  static constexpr int SC = L + 4;              // row stride of C^T (rows of L tokens)
  static constexpr int SA = L + 4;              // row stride of the L x L products
  static constexpr int NT = D / 16;             // 16-wide tiles across D
  static constexpr int HR = D < 64 ? D : 64;    // rows of a D x D matrix (and of C^T) staged at once
  static constexpr int NH = D / HR;             // staged parts per matrix
  // With DIRECT staging (D = 128, bf16 io) the S0 / G_end rows are loaded straight into LDS,
  // 64 lanes x 16 bytes = two rows per load; pairs of rows sit PP floats apart, so the four rows
  // one MFMA operand read touches (r, r + 4, r + 8, r + 12) start 16 banks apart.  Otherwise rows
  // go through registers with a padded row stride SB (the fp32-io kernel has no registers to
  // spare for the wider dO loads and the direct path together).
  static constexpr int PP = 2 * D + 8;
  static_assert(HR / 2 * PP <= HR * SB || D != 128, "the direct layout fits the padded one");
};

template <int D, int IO>
constexpr bool direct_staging() {
  return D == 128 && IO == IO_BF16;
}

// Offset of row r of the staged matrix part, and of row r0 + e from row r0 (r0 even, e < 4).
template <int D, bool DIRECT>
__device__ __forceinline__ int mrow(int r) {
  using M = MCfg<D>;
  if constexpr (DIRECT) return (r >> 1) * M::PP + (r & 1) * D;
  return r * M::SB;
}
template <int D, bool DIRECT>
constexpr int mrow_step(int e) {
  return DIRECT ? (e >> 1) * MCfg<D>::PP + (e & 1) * D : e * MCfg<D>::SB;
}

// LDS of the chunk-gradient kernel: the products with S0 and G_end stream those matrices (and
// C^T) in parts of HR rows; the decay-masked products then hold A1, A2 and K (later Q).
template <int D>
struct alignas(16) MLds {
  using M = MCfg<D>;
  union {
    struct {
      float mat[M::HR * M::SB];     // rows [j0, j0 + HR) of S0 or G_end ([dv][dk] layout)
      float ct[M::HR * M::SC];      // rows [j0, j0 + HR) of C^T
    } p;
    struct {
      float a1[M::L * M::SA];       // dO C^T
      float a2[M::L * M::SA];       // dU C^T
      float kq[M::L * M::SB];       // K, then Q (zero past the chunk)
    } m;
  } u;
  double lgd[M::L + 1];             // sum of log a over the chunk's tokens before token t
  float2 ab[M::L];
  float xq[M::L];                   // q_t . dq_t of the current value head
};

template <int IO>
__device__ __forceinline__ float4 load4(const void* base, int64_t elem) {
  if constexpr (IO == IO_F32) {
    return *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
  } else {
    const uint2 u = *reinterpret_cast<const uint2*>(static_cast<const unsigned short*>(base) + elem);
    return make_float4(__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xFFFF0000u),
                       __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xFFFF0000u));
  }
}

// Four consecutive io-typed values kept as raw bits until used, and their exact widening.
template <int IO>
struct Raw4;
template <>
struct Raw4<IO_F32> {
  float4 x;
};
template <>
struct Raw4<IO_BF16> {
  uint2 x;
};

template <int IO>
__device__ __forceinline__ Raw4<IO> load_raw4(const void* base, int64_t elem) {
  Raw4<IO> r;
  if constexpr (IO == IO_F32)
    r.x = *reinterpret_cast<const float4*>(static_cast<const float*>(base) + elem);
  else
    r.x = *reinterpret_cast<const uint2*>(static_cast<const unsigned short*>(base) + elem);
  return r;
}

template <int IO>
__device__ __forceinline__ float4 widen4(const Raw4<IO>& r) {
  if constexpr (IO == IO_F32) {
    return r.x;
  } else {
    const uint2 u = r.x;
    return make_float4(__builtin_bit_cast(float, u.x << 16), __builtin_bit_cast(float, u.x & 0xFFFF0000u),
                       __builtin_bit_cast(float, u.y << 16), __builtin_bit_cast(float, u.y & 0xFFFF0000u));
  }
}

__device__ __forceinline__ float comp(const float4& v, int e) {
  return e == 0 ? v.x : e == 1 ? v.y : e == 2 ? v.z : v.w;
}

// Stage rows [j0, j0 + HR) of a D x D fp32 matrix in [dv][dk] layout into S.u.p.mat (row r at
// mrow(r)), and the same
// rows of C^T (C [t][j] of this chunk, zero past its n tokens) into S.u.p.ct.
template <int D, bool DIRECT, bool CT = true>
__device__ __forceinline__ void stage_part(MLds<D>& S, const float* mat, const float* cc, int64_t tok, int n,
                                           int h_v, int h, int j0) {
  using M = MCfg<D>;
  if constexpr (DIRECT) {
    // wave w loads row pairs w, w + 4, ...: lane l takes 16 bytes of row 2 p + l / 32, which the
    // load writes to LDS at the pair's base + 16 l
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const float* src = mat + static_cast<int64_t>(j0 + (lane >> 5)) * D + 4 * (lane & 31);
#if defined(__HIP_DEVICE_COMPILE__)   // a device builtin; the host pass only needs the declaration
#pragma unroll 1
    for (int p = wave; p < M::HR / 2; p += 4)
      __builtin_amdgcn_global_load_lds(src + static_cast<int64_t>(2 * p) * D, &S.u.p.mat[p * M::PP], 16, 0, 0);
#endif
  } else {
    for (int e = threadIdx.x; e < M::HR * D / 4; e += 256) {
      const int r = e / (D / 4), c4 = e % (D / 4);
      *reinterpret_cast<float4*>(&S.u.p.mat[r * M::SB + 4 * c4]) =
          reinterpret_cast<const float4*>(mat + static_cast<int64_t>(j0 + r) * D)[c4];
    }
  }
  for (int e = threadIdx.x; CT && e < M::L * M::HR / 4; e += 256) {
    const int t = e / (M::HR / 4), c4 = e % (M::HR / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < n) x = *reinterpret_cast<const float4*>(cc + ((tok + t) * h_v + h) * D + j0 + 4 * c4);
    S.u.p.ct[(4 * c4 + 0) * M::SC + t] = x.x;
    S.u.p.ct[(4 * c4 + 1) * M::SC + t] = x.y;
    S.u.p.ct[(4 * c4 + 2) * M::SC + t] = x.z;
    S.u.p.ct[(4 * c4 + 3) * M::SC + t] = x.w;
  }
  if constexpr (DIRECT) __builtin_amdgcn_s_waitcnt(0);   // this wave's loads into LDS have landed
}

// K or Q rows of the chunk (io dtype, zero past its n tokens) into S.u.m.kq.
template <int D, int IO>
__device__ __forceinline__ void stage_kq(MLds<D>& S, const void* src, int64_t tok, int n, int h_k, int kh) {
  using M = MCfg<D>;
  for (int e = threadIdx.x; e < M::L * D / 4; e += 256) {
    const int t = e / (D / 4), c4 = e % (D / 4);
    float4 x = make_float4(0.f, 0.f, 0.f, 0.f);
    if (t < n) x = load4<IO>(src, ((tok + t) * h_k + kh) * D + 4 * c4);
    *reinterpret_cast<float4*>(&S.u.m.kq[t * M::SB + 4 * c4]) = x;
  }
}

// The per-token gradients that need no chunk form, over every (token, value head): dv_t = b_t dc_t,
// db_t = dc_t . w_t, and v_t . dv_t for the chunk pass's h recurrence.  D/8 lanes per token-head,
// eight columns each, summed in column order per lane and then by the DPP tree over the lanes; each
// lane group takes two token-heads, their loads issued together.
template <int D, int IO>
__global__ void __launch_bounds__(256) token_grads_kernel(BackwardArgs A) {
  constexpr int LPT = D / 8;                                    // lanes per token-head
  constexpr int PER_BLOCK = 2 * 256 / LPT;                      // token-heads per workgroup
  const int64_t n = A.total_tokens * A.h_v;
  const int c8 = threadIdx.x % LPT;
  int64_t th[2];
  float4 dc[2][2], w[2][2], v[2][2];
  float bt[2];
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    th[u] = static_cast<int64_t>(blockIdx.x) * PER_BLOCK + u * (256 / LPT) + threadIdx.x / LPT;
    const int64_t base = (th[u] < n ? th[u] : 0) * D + 8 * c8;   // [t][h][D] with th = t H_v + h
    dc[u][0] = reinterpret_cast<const float4*>(A.dc + base)[0];
    dc[u][1] = reinterpret_cast<const float4*>(A.dc + base)[1];
    w[u][0] = reinterpret_cast<const float4*>(A.ww + base)[0];
    w[u][1] = reinterpret_cast<const float4*>(A.ww + base)[1];
    v[u][0] = load4<IO>(A.v, base);
    v[u][1] = load4<IO>(A.v, base + 4);
    bt[u] = A.b[th[u] < n ? th[u] : 0];
  }
#pragma unroll
  for (int u = 0; u < 2; ++u) {
    const float x[8] = {dc[u][0].x, dc[u][0].y, dc[u][0].z, dc[u][0].w, dc[u][1].x, dc[u][1].y, dc[u][1].z, dc[u][1].w};
    const float y[8] = {w[u][0].x, w[u][0].y, w[u][0].z, w[u][0].w, w[u][1].x, w[u][1].y, w[u][1].z, w[u][1].w};
    const float z[8] = {v[u][0].x, v[u][0].y, v[u][0].z, v[u][0].w, v[u][1].x, v[u][1].y, v[u][1].z, v[u][1].w};
    float dv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dv[e] = bt[u] * x[e];
    float sv = z[0] * dv[0], sd = x[0] * y[0];
#pragma unroll
    for (int e = 1; e < 8; ++e) {
      sv = __builtin_fmaf(z[e], dv[e], sv);
      sd = __builtin_fmaf(x[e], y[e], sd);
    }
    sv = lane_tree<LPT>(sv);
    sd = lane_tree<LPT>(sd);
    if (th[u] < n) {
      float* dst = A.dv + th[u] * D + 8 * c8;
      reinterpret_cast<float4*>(dst)[0] = make_float4(dv[0], dv[1], dv[2], dv[3]);
      reinterpret_cast<float4*>(dst)[1] = make_float4(dv[4], dv[5], dv[6], dv[7]);
      if (c8 == 0) {
        A.db[th[u]] = sd;
        A.xv[th[u]] = sv;
      }
    }
  }
}

template <int D, int IO>
__global__ void __launch_bounds__(256, 2) grad_chunk_kernel(BackwardArgs A) {
  using M = MCfg<D>;
  constexpr int NT = M::NT, SB = M::SB, SC = M::SC, SA = M::SA, LT = M::L, HR = M::HR, NH = M::NH;
  constexpr bool DS = direct_staging<D, IO>();
  __shared__ MLds<D> S;
  __shared__ int64_t red[6];
  const int64_t w = blockIdx.x / A.h_k;
  const int kh = static_cast<int>(blockIdx.x % A.h_k);
  if (w >= A.rows_cap) return;                               // uniform across the block
  int i;
  int64_t c;
  if (!plan_find_row(A, w, &i, &c, red)) return;             // uniform across the block
  const SeqMeta m = seq_meta(A, i);
  const int tb = static_cast<int>(c) * A.chunk;
  const int L = A.chunk < m.len - tb ? A.chunk : m.len - tb; // tokens in this chunk, 1..64
  const int64_t tok = m.tok0 + tb;
  const int ratio = A.h_v / A.h_k;
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lj = lane & 15, lgp = lane >> 4;
  const int row = 16 * wave + lj;                            // this lane's A row (token in chunk)
  const bool rv = row < L;
  const int64_t plane = static_cast<int64_t>(D) * D;
  const int64_t gstart = w + i;                              // boundary rows around this chunk

  // the key head's dq and dk: each value head's products accumulate onto the previous heads' in the
  // matrix-core accumulators, heads in order; xprev holds q_t . dq_t of the heads before
  f32x4 acc_dq[NT], acc_dk[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) acc_dq[n] = acc_dk[n] = f32x4{0.f, 0.f, 0.f, 0.f};
  float xprev[4] = {0.f, 0.f, 0.f, 0.f};
  for (int hh = 0; hh < ratio; ++hh) {
    const int h = kh * ratio + hh;
    __syncthreads();                                         // the previous head is done with LDS
    if (tid < LT) {
      float2 ab = make_float2(1.f, 0.f);
      if (tid < L) ab = make_float2(A.a[(tok + tid) * A.h_v + h], A.b[(tok + tid) * A.h_v + h]);
      S.ab[tid] = ab;
      // log of the gate product up to and including token tid, an inclusive scan in fp64
      double x = tid < L ? log(static_cast<double>(ab.x)) : 0.0;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(x, off, 64);
        if (lane >= off) x += y;
      }
      S.lgd[tid + 1] = x;
      if (tid == 0) S.lgd[0] = 0.0;
    }
    __syncthreads();
    const double lr0 = S.lgd[row], lr1 = S.lgd[row + 1];
    const float2 abr = S.ab[row];
    const float fq = rv ? __expf(static_cast<float>(lr1)) : 0.f;                 // Gam after the row
    const float fu = rv ? __expf(static_cast<float>(lr0)) : 0.f;                 // Gam before it
    const float fc = rv ? __expf(static_cast<float>(S.lgd[L] - lr1)) : 0.f;     // Gam_L / Gam_row
    const float su = -abr.x * abr.y;                                              // dU = su * dc
    const float* s0 = A.chunk_states + (w * A.h_v + h) * plane;
    const float* ge = A.adjoint + ((gstart + 1) * A.h_v + h) * plane;

    // dq += Gam_t dO S0^T; dk += Gam_{t-1} dU S0^T; A1 = dO C^T; A2 = dU C^T; h_0 = <G_start, S0>
    f32x4 a1[4], a2[4];
#pragma unroll
    for (int n = 0; n < 4; ++n) a1[n] = a2[n] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll 1
    for (int part = 0; part < NH; ++part) {
      const int j0 = part * HR;
      __syncthreads();
      stage_part<D, DS>(S, s0, A.cc, tok, L, A.h_v, h, j0);
      __syncthreads();
      // this lane's dO and dc elements of panel p are fetched while panel p - 1 runs: raw bits, a
      // row past the chunk reading row 0 (its values are then replaced by zeros at use)
      const int64_t arow = ((tok + (rv ? row : 0)) * A.h_v + h) * D + j0 + 4 * lgp;
      Raw4<IO> o_next = load_raw4<IO>(A.d_o, arow);
      float4 c_next = *reinterpret_cast<const float4*>(A.dc + arow);
#pragma unroll 1
      for (int p = 0; p < HR / 16; ++p) {
        const int kl = 16 * p + 4 * lgp;                     // k within the part
        const int mk = mrow<D, DS>(kl);
        const Raw4<IO> o_raw = o_next;
        const float4 c_cur = c_next;
        const int pn = p + 1 < HR / 16 ? p + 1 : p;          // the last panel fetches itself again
        o_next = load_raw4<IO>(A.d_o, arow + 16 * pn);
        c_next = *reinterpret_cast<const float4*>(A.dc + arow + 16 * pn);
        const float4 zero = make_float4(0.f, 0.f, 0.f, 0.f);
        const float4 o4 = rv ? widen4<IO>(o_raw) : zero, c4 = rv ? c_cur : zero;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = kl + e;
          const float ao = comp(o4, e), au = su * comp(c4, e);
          const float aq = ao * fq, ak = au * fu;
#pragma unroll
          for (int n = 0; n < NT; ++n) {
            const float bs = S.u.p.mat[mk + mrow_step<D, DS>(e) + 16 * n + lj];
            acc_dq[n] = mfma4(aq, bs, acc_dq[n]);
            acc_dk[n] = mfma4(ak, bs, acc_dk[n]);
          }
#pragma unroll
          for (int n = 0; n < 4; ++n) {
            const float bc = S.u.p.ct[k * SC + 16 * n + lj];
            a1[n] = mfma4(ao, bc, a1[n]);
            a2[n] = mfma4(au, bc, a2[n]);
          }
        }
      }
      // dk += (Gam_L / Gam_t) C G_end^T over the same columns, while their C^T is staged
      __syncthreads();
      stage_part<D, DS, false>(S, ge, A.cc, tok, L, A.h_v, h, j0);   // C^T of this part stays
      __syncthreads();
#pragma unroll 1
      for (int p = 0; p < HR / 16; ++p) {
        const int mk = mrow<D, DS>(16 * p + 4 * lgp);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int k = 16 * p + 4 * lgp + e;
          const float ac = S.u.p.ct[k * SC + row] * fc;
#pragma unroll
          for (int n = 0; n < NT; ++n)
            acc_dk[n] = mfma4(ac, S.u.p.mat[mk + mrow_step<D, DS>(e) + 16 * n + lj], acc_dk[n]);
        }
      }
    }
    __syncthreads();                                         // C^T and G_end reads done
    // A1, A2 -> LDS; K rows -> LDS
#pragma unroll
    for (int n = 0; n < 4; ++n)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * lgp + r;
        S.u.m.a1[t * SA + 16 * n + lj] = a1[n][r];
        S.u.m.a2[t * SA + 16 * n + lj] = a2[n][r];
      }
    stage_kq<D, IO>(S, A.k, tok, L, A.h_k, kh);
    __syncthreads();
    // dq += (M_incl . A1) K;  dk += (M_strict . A2 + N_strict . A2^T) K
#pragma unroll 1
    for (int p = 0; p < LT / 16; ++p) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 16 * p + 4 * lgp + e;
        const double ls0 = S.lgd[s], ls1 = S.lgd[s + 1];
        float aq = 0.f, ak2 = 0.f;
        if (rv) {
          if (s <= row) aq = S.u.m.a1[row * SA + s] * __expf(static_cast<float>(lr1 - ls1));
          if (s < row) ak2 = S.u.m.a2[row * SA + s] * __expf(static_cast<float>(lr0 - ls1));
          if (s > row) ak2 = S.u.m.a2[s * SA + row] * __expf(static_cast<float>(ls0 - lr1));
        }
#pragma unroll
        for (int n = 0; n < NT; ++n) {
          const float kbv = S.u.m.kq[s * SB + 16 * n + lj];
          acc_dq[n] = mfma4(aq, kbv, acc_dq[n]);
          acc_dk[n] = mfma4(ak2, kbv, acc_dk[n]);
        }
      }
    }
    __syncthreads();
    stage_kq<D, IO>(S, A.q, tok, L, A.h_k, kh);
    __syncthreads();
    // dk += (N_incl . A1^T) Q
#pragma unroll 1
    for (int p = 0; p < LT / 16; ++p) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int s = 16 * p + 4 * lgp + e;
        const double ls1 = S.lgd[s + 1];
        float ak1 = 0.f;
        if (rv && s >= row) ak1 = S.u.m.a1[s * SA + row] * __expf(static_cast<float>(ls1 - lr1));
#pragma unroll
        for (int n = 0; n < NT; ++n) acc_dk[n] = mfma4(ak1, S.u.m.kq[s * SB + 16 * n + lj], acc_dk[n]);
      }
    }
    // per-token terms of this value head: q_t . dq_t over this head's dq, the accumulated dq's dot
    // less that of the heads before (rows 16 wave + 4 g + r, columns 16 n + j)
    {
      float xr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int t = 16 * wave + 4 * lgp + r;
        float x = 0.f;
#pragma unroll
        for (int n = 0; n < NT; ++n) x = __builtin_fmaf(acc_dq[n][r], S.u.m.kq[t * SB + 16 * n + lj], x);
        const float xc = lane_tree<16>(x);
        xr[r] = xc - xprev[r];
        xprev[r] = xc;
      }
      if (lj == 0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) S.xq[16 * wave + 4 * lgp + r] = xr[r];
      }
    }
    __syncthreads();
    // h_{t-1} = h_0 - sum_{s<t} (q_s . dq_s - v_s . dv_s); da_t = h_{t-1} / a_t
    if (tid < LT) {
      const double x = tid < L ? static_cast<double>(S.xq[tid]) - static_cast<double>(A.xv[(tok + tid) * A.h_v + h])
                               : 0.0;
      double incl = x;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const double y = __shfl_up(incl, off, 64);
        if (lane >= off) incl += y;
      }
      double excl = __shfl_up(incl, 1, 64);
      if (lane == 0) excl = 0.0;
      // h_0 = <G_start, S_0>: the parts the adjoint pass stored, added in order
      const double* hpp = A.hpart + (gstart * A.h_v + h) * A.hparts;
      double h0 = 0.0;
#pragma unroll 1
      for (int p = 0; p < A.hparts; ++p) h0 += hpp[p];
      if (tid < L) A.da[(tok + tid) * A.h_v + h] = static_cast<float>((h0 - excl) / static_cast<double>(S.ab[tid].x));
    }
  }
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int t = 16 * wave + 4 * lgp + r;
    if (t < L) {
      const int64_t base = ((tok + t) * A.h_k + kh) * D;
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        A.dq[base + 16 * n + lj] = acc_dq[n][r];
        A.dk[base + 16 * n + lj] = acc_dk[n][r];
      }
    }
  }
}

// One block per sequence: where its rows start in the caller's stash (chunk A.chunk), as a slot
// id over that stash, with a zero position there, so that pass 1 at the gradient tile's chunk
// starts every sequence from the state it began with.
__global__ void __launch_bounds__(256) rechunk_setup_kernel(BackwardArgs A, int32_t* slot_ids, int64_t* pos) {
  __shared__ int64_t red[(256 + 63) / 64 + 2];
  const int j = blockIdx.x;
  const int64_t r0 = plan_row_offset(A, j, red);
  if (threadIdx.x == 0) {
    slot_ids[j] = static_cast<int32_t>(r0 < A.rows_cap ? r0 : A.rows_cap);
    if (r0 < A.rows_cap) pos[r0] = 0;
  }
}

hipError_t launch_rechunk_setup(const BackwardArgs& A, int32_t* slot_ids, int64_t* pos, hipStream_t stream) {
  if (A.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(rechunk_setup_kernel, dim3(static_cast<unsigned>(A.num_seqs)), dim3(256), 0, stream, A,
                     slot_ids, pos);
  return hipGetLastError();
}

// The per-token gradients (after which event 2 is recorded) and the chunk gradients (event 3),
// from dc, G at every chunk boundary, the <G, S> parts, c and w.
template <int D, int IO>
static hipError_t launch_gradient_passes_t(const BackwardArgs& A, hipStream_t stream) {
  hipError_t e;
  if (A.total_tokens > 0) {
    const int64_t per_block = 2 * 256 / (D / 8);
    const int64_t g = (A.total_tokens * A.h_v + per_block - 1) / per_block;
    if (g > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((token_grads_kernel<D, IO>), dim3(static_cast<unsigned>(g)), dim3(256), 0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 2, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0 && A.rows_cap > 0) {
    const int64_t g3 = A.rows_cap * A.h_k;
    if (g3 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((grad_chunk_kernel<D, IO>), dim3(static_cast<unsigned>(g3)), dim3(256), 0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return record_event(A.events, 3, stream);
}

hipError_t launch_gradient_passes(int d, int io, const BackwardArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (d == D && io == IOV) return launch_gradient_passes_t<D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

template <int DK, int DV, int IO>
static hipError_t launch_backward_t(const BackwardArgs& A, hipStream_t stream) {
  using Cfg = ColCfg<DK, DV>;
  const int ratio = A.h_v / A.h_k;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0) {
    const int64_t g1 = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, ratio * Cfg::NCG);
    if (g1 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((adjoint_kernel<DK, DV, IO>), dim3(static_cast<unsigned>(g1)), dim3(Cfg::THREADS), 0, stream,
                       A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0 && A.rows_cap > 0 && !A.have_cw) {
    const int64_t g2 = xcd_grid(A.rows_cap * A.h_k, ratio * Cfg::NCG);
    if (g2 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((replay_kernel<DK, DV, IO>), dim3(static_cast<unsigned>(g2)), dim3(Cfg::THREADS), 0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return launch_gradient_passes_t<DK, IO>(A, stream);
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

}  // namespace cpr
