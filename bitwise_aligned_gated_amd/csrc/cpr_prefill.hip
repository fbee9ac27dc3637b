// cpr_prefill.hip -- the two CPR passes over a packed varlen batch.
//
// "Solving the linear-attention headache" (IsoExec articles): one pass finds the state at the
// start of every chunk; a second pass, parallel over chunks, produces each chunk's outputs
// starting from that state.  Both passes here apply the shared pinned step (cpr_step.hpp)
// to every token, so the states pass 1 stores are exactly the states pass 2 and decode reach.
//
// Work mapping.  A column's d_k rows are split over G consecutive lanes, each holding NL leaves
// of 8 rows (R = 8*NL rows), and a lane owns NC columns; the state lives in registers.  Token
// tiles (k, q widened to fp32, the workgroup's v columns, a and b) are staged through LDS and
// the next tile is fetched into registers while the current one is computed.
//   pass 1 (boundary_pass)  parallel only over (sequence, value head, column): G = d_k/8 so a
//                           sequence's chain is spread over as many lanes as possible.  One
//                           workgroup per (sequence, value head, column group); runs each
//                           sequence up to its last chunk start and stores the state entering
//                           every chunk.
//   pass 2 (output_pass)    parallel over chunks too, so lanes take more rows (G <= 4) and two
//                           columns each, which cuts the tree and per-column overhead per
//                           element.  One workgroup per (boundary row, value head, column
//                           group); a row is one chunk: load its entering state, run its tokens
//                           with output, store o; the last chunk also stores the final state.
// Workgroups are ordered XCD-aware (cpr_common.hpp): those reading one key head's tokens share
// an XCD and its L2.
//   fused (fused_pass)      the one-pass variant: pass 1's mapping and grid, every token with
//                           output, chunk-start rows only when a stash is given.
//   finish                  pos[slot] = p0 + length, after the passes have read pos.
// The schedule fixes the leaves and the tree, not the lane mapping, so both mappings (and the
// decode kernel's) produce identical bits.
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

// What a token loop does: pass 1 stores chunk-start states, pass 2 writes outputs, the fused
// one-pass variant does both (it runs a whole sequence like pass 1, with outputs like pass 2).
// With a stash, pass 1 runs every token and also keeps each token's write value c (and w when
// asked), and pass 2 applies the kept c instead of predicting it again: the same values enter
// the same update, so the bits do not change, and pass 2 skips the prediction's dot product.
// Pass 1 comes in two lane mappings: one 8-row leaf per lane (kBoundary, kBoundaryC) or two
// (kBoundary2, kBoundaryC2).  Two leaves per lane halve the tree levels and the per-column work
// (w, c) per state element, so a column costs ~11% fewer instructions per token, but a column
// chain then occupies half as many lanes: the launcher picks the mapping that loads the busiest
// SIMD least (launch_pass1 below).  The schedule fixes leaves and tree, not lanes, so both give the
// same bits.
enum : int { kBoundary = 0, kOutput = 1, kFused = 2, kOutputC = 3, kBoundaryC = 4, kBoundary2 = 5, kBoundaryC2 = 6 };
constexpr bool has_out(int mode) { return mode == kOutput || mode == kFused || mode == kOutputC; }
constexpr bool is_pass1(int mode) {
  return mode == kBoundary || mode == kBoundaryC || mode == kBoundary2 || mode == kBoundaryC2;
}
constexpr bool two_leaves(int mode) { return mode == kBoundary2 || mode == kBoundaryC2; }
constexpr bool has_rows(int mode) { return is_pass1(mode) || mode == kFused; }
constexpr bool is_wide(int mode) { return mode == kOutput || mode == kOutputC; }
constexpr bool reads_c(int mode) { return mode == kOutputC; }      // c from the stash instead of v, b
constexpr bool keeps_c(int mode) { return mode == kBoundaryC || mode == kBoundaryC2; }    // writes the stash
constexpr bool stops_at_last_start(int mode) { return mode == kBoundary || mode == kBoundary2; }

template <int DK, int DV, int MODE>
struct PassCfg {
  static constexpr bool WIDE = is_wide(MODE);     // parallel over chunks: fewer, longer lanes
  static constexpr int G = WIDE ? (DK / kLeaf < 4 ? DK / kLeaf : 4)
                                : (two_leaves(MODE) && DK >= 2 * kLeaf ? DK / (2 * kLeaf) : DK / kLeaf);  // lanes per column
  static constexpr int NL = DK / (kLeaf * G);                                  // leaves per lane
  static constexpr int R = NL * kLeaf;                                         // rows per lane
  static constexpr int NC = WIDE ? 2 : 1;                                      // columns per lane
  static constexpr int WG_MAX_COLS = 256 / G * NC;                             // 4 waves
  static constexpr int WG_COLS = WG_MAX_COLS < DV ? WG_MAX_COLS : DV;
  static constexpr int THREADS = WG_COLS / NC * G;
  static constexpr int TT = is_pass1(MODE) ? 32 : 16;  // tokens per tile
  static constexpr int K_UNITS = TT * DK / 8;          // 8-element units of a k (or q) tile
  static constexpr int V_UNITS = TT * WG_COLS / 8;
  static constexpr int K_PER_T = (K_UNITS + THREADS - 1) / THREADS;
  static constexpr int V_PER_T = (V_UNITS + THREADS - 1) / THREADS;
  static constexpr int NAB = reads_c(MODE) ? TT : 2 * TT;        // gates per tile: a (and b)
  static constexpr int AB_PER_T = (NAB + THREADS - 1) / THREADS;
  static_assert(DK % (kLeaf * G) == 0 && DV % WG_COLS == 0 && WG_COLS % 8 == 0, "shape");
  static_assert(THREADS % 64 == 0 || (THREADS & (THREADS - 1)) == 0, "block size");
};

// One tile in flight (global -> registers -> LDS).
template <int DK, int DV, int IO, int MODE>
struct TileRegs {
  using Cfg = PassCfg<DK, DV, MODE>;
  Raw8<IO> k[Cfg::K_PER_T];
  Raw8<IO> q[has_out(MODE) ? Cfg::K_PER_T : 1];
  Raw8<reads_c(MODE) ? IO_F32 : IO> v[Cfg::V_PER_T];   // v, or the stashed c (fp32)
  float ab[Cfg::AB_PER_T];
};

template <int DK, int DV, int MODE>
struct TileLds {
  using Cfg = PassCfg<DK, DV, MODE>;
  float k[Cfg::TT][DK];                                 // lane-interleaved rows (kq_slot)
  float q[has_out(MODE) ? Cfg::TT : 1][DK];
  float v[Cfg::TT][Cfg::WG_COLS];                       // v, or the stashed c
  float o[MODE == kFused ? Cfg::TT : 1][Cfg::WG_COLS];  // fused: outputs gathered for row stores
  float cs[keeps_c(MODE) ? Cfg::TT : 1][Cfg::WG_COLS];  // stash: c and w gathered for row stores
  float ws[keeps_c(MODE) ? Cfg::TT : 1][Cfg::WG_COLS];
  float2 ab[Cfg::TT];   // (a, b) of each token (stashed c: a only)
};

// Fetch packed tokens [t0, t0 + n) (n <= TT) of key head kh / value head h into registers.
// The tile's base addresses are uniform and each lane's offsets within a tile do not depend on
// t0, so per unit the loop pays one compare and a load.  Units past n keep what they held (they
// are committed to LDS but no token reads them) and are never read from memory.
template <int DK, int DV, int IO, int MODE>
__device__ __forceinline__ void fetch_tile(const PrefillArgs& A, TileRegs<DK, DV, IO, MODE>& R, int t0, int n,
                                           int kh, int h, int col0) {
  using Cfg = PassCfg<DK, DV, MODE>;
  constexpr int64_t ES = IO == IO_F32 ? 4 : 2;
  const int tid = threadIdx.x;
  const char* kb = static_cast<const char*>(A.k) + (static_cast<int64_t>(t0) * A.h_k + kh) * DK * ES;
  const char* qb = static_cast<const char*>(A.q) + (static_cast<int64_t>(t0) * A.h_k + kh) * DK * ES;
  const char* vb = reads_c(MODE)
                       ? reinterpret_cast<const char*>(A.c_stash + (static_cast<int64_t>(t0) * A.h_v + h) * DV + col0)
                       : static_cast<const char*>(A.v) + ((static_cast<int64_t>(t0) * A.h_v + h) * DV + col0) * ES;
#pragma unroll
  for (int i = 0; i < Cfg::K_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    const int tt = u / (DK / 8), c8 = u % (DK / 8);
    const uint32_t off = static_cast<uint32_t>(tt * A.h_k * DK + c8 * 8);
    if (u < Cfg::K_UNITS && tt < n) {
      R.k[i] = load_raw8<IO>(kb, off);
      if constexpr (has_out(MODE)) R.q[i] = load_raw8<IO>(qb, off);
    }
  }
#pragma unroll
  for (int i = 0; i < Cfg::V_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
    const uint32_t off = static_cast<uint32_t>(tt * A.h_v * DV + c8 * 8);
    if (u < Cfg::V_UNITS && tt < n) R.v[i] = load_raw8<reads_c(MODE) ? IO_F32 : IO>(vb, off);
  }
  const float* ga = A.a + static_cast<int64_t>(t0) * A.h_v + h;
  const float* gb = A.b + static_cast<int64_t>(t0) * A.h_v + h;
#pragma unroll
  for (int i = 0; i < Cfg::AB_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    const int tt = u % Cfg::TT;
    const uint32_t off = static_cast<uint32_t>(tt * A.h_v);
    if (tt < n) {                    // lanes [0, TT) fetch a, lanes [TT, 2 TT) fetch b
      if (u < Cfg::TT)
        R.ab[i] = ga[off];
      else if (u < Cfg::NAB)
        R.ab[i] = gb[off];
    }
  }
}

template <int DK, int DV, int IO, int MODE>
__device__ __forceinline__ void commit_tile(const TileRegs<DK, DV, IO, MODE>& R, TileLds<DK, DV, MODE>& L) {
  using Cfg = PassCfg<DK, DV, MODE>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg::K_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    if (u < Cfg::K_UNITS) {
      const int tt = u / (DK / 8), c8 = u % (DK / 8);
      float x[8];
      widen8<IO>(R.k[i], x);
      store_kq8<Cfg::G, Cfg::R>(&L.k[tt][0], c8 * 8, x);
      if constexpr (has_out(MODE)) {
        widen8<IO>(R.q[i], x);
        store_kq8<Cfg::G, Cfg::R>(&L.q[tt][0], c8 * 8, x);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < Cfg::V_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    if (u < Cfg::V_UNITS) {
      const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
      float x[8];
      widen8<reads_c(MODE) ? IO_F32 : IO>(R.v[i], x);
      store_f32x8(&L.v[tt][c8 * 8], x);
    }
  }
#pragma unroll
  for (int i = 0; i < Cfg::AB_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    if (u < Cfg::TT)
      L.ab[u].x = R.ab[i];
    else if (u < Cfg::NAB)
      L.ab[u - Cfg::TT].y = R.ab[i];
  }
}

// Run tokens [tb, te) (offsets from the sequence start; tb < te) of one sequence through this
// lane's columns.  Modes with output write o for every token; modes with rows store the state
// entering every chunk start reached after a token, as rows row0 + 1, row0 + 2, ... below
// row_end (the first one `first_nb` tokens after tb).
template <int DK, int DV, int IO, int MODE>
__device__ __forceinline__ void run_tokens(const PrefillArgs& A, TileLds<DK, DV, MODE>& L,
                                           float (&s)[PassCfg<DK, DV, MODE>::NC][PassCfg<DK, DV, MODE>::R],
                                           int tok0, int tb, int te, int h, int cg, int64_t row0, int64_t row_end,
                                           int first_nb) {
  using Cfg = PassCfg<DK, DV, MODE>;
  constexpr int G = Cfg::G, NL = Cfg::NL, R = Cfg::R, NC = Cfg::NC;
  constexpr bool OUT = has_out(MODE);
  const int tid = threadIdx.x;
  const int cp = tid / G, g = tid % G;
  const int col0 = cg * Cfg::WG_COLS;
  const int kh = h / (A.h_v / A.h_k);
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  int nb = __builtin_amdgcn_readfirstlane(first_nb);   // tokens until the next chunk start
  int64_t row = row0 + 1;                              // row the next chunk-start state goes to
  const bool rows_on = has_rows(MODE) && A.chunk_states != nullptr;
  const bool keep_w = A.w_stash != nullptr;

  TileRegs<DK, DV, IO, MODE> Rg = {};
  fetch_tile<DK, DV, IO, MODE>(A, Rg, tok0 + tb, te - tb < Cfg::TT ? te - tb : Cfg::TT, kh, h, col0);
  commit_tile<DK, DV, IO, MODE>(Rg, L);
  __syncthreads();
  for (int t0 = tb; t0 < te; t0 += Cfg::TT) {
    const int n = te - t0 < Cfg::TT ? te - t0 : Cfg::TT;
    const int t1 = t0 + Cfg::TT;
    const bool more = t1 < te;
    if (more) fetch_tile<DK, DV, IO, MODE>(A, Rg, tok0 + t1, te - t1 < Cfg::TT ? te - t1 : Cfg::TT, kh, h, col0);
    // Stash modes hand each token's c (and w) to LDS at the start of the next token, so that the
    // lane-masked write does not split a token's own arithmetic.
    float pc = 0.0f, pw = 0.0f;
    int ptt = -1;
    auto hand_over = [&]() {
      if constexpr (keeps_c(MODE)) {
        if (ptt >= 0 && g == 0) {
          L.cs[ptt][cp] = pc;
          if (keep_w) L.ws[ptt][cp] = pw;
        }
      }
    };
    // A token's inputs from the tile.  Pass 1 reads token tt + 1's while token tt computes, so
    // that a lone sequence's chain does not wait on LDS at every token (the one-pass variant
    // would need more registers than five waves per SIMD allow).
    struct In {
      float kr[R], qr[R], vv[NC];
      float2 ab;
    };
    auto read_in = [&](int tt, In& x) {
      lds_read_kq<G, R>(&L.k[tt][0], g, x.kr);
      if constexpr (OUT) lds_read_kq<G, R>(&L.q[tt][0], g, x.qr);
      x.ab = L.ab[tt];
#pragma unroll
      for (int c = 0; c < NC; ++c) x.vv[c] = L.v[tt][cp * NC + c];
    };
    auto token = [&](int tt, In& x) {
      float (&kr)[R] = x.kr;
      float (&qr)[R] = x.qr;
      float (&vv)[NC] = x.vv;
      const float2 ab = x.ab;
      hand_over();
      float o[NC];
      if constexpr (MODE == kOutputC) {                    // vv holds the stashed c
#pragma unroll
        for (int c = 0; c < NC; ++c) o[c] = cpr_step_given_c<NL, G>(s[c], kr, qr, ab.x, vv[c]);
      } else if constexpr (keeps_c(MODE)) {
        float u;
        cpr_update<NL, G>(s[0], kr, vv[0], ab.x, ab.y, u, pw, pc);
        ptt = tt;
        o[0] = 0.0f;
      } else {
#pragma unroll
        for (int c = 0; c < NC; ++c) o[c] = cpr_step<NL, G, OUT>(s[c], kr, qr, vv[c], ab.x, ab.y);
      }
      if constexpr (is_wide(MODE)) {
        if (g == 0) {
          const int64_t oe = (static_cast<int64_t>(tok0 + t0 + tt) * A.h_v + h) * DV + col0 + cp * NC;
          if constexpr (NC == 2) {
            store2<IO>(A.o, oe, o[0], o[1]);
          } else {
#pragma unroll
            for (int c = 0; c < NC; ++c) store1<IO>(A.o, oe + c, o[c]);
          }
        }
      } else if constexpr (MODE == kFused) {
        if (g == 0) L.o[tt][cp] = o[0];
      }
      if constexpr (has_rows(MODE)) {
        if (--nb == 0) {                                   // the new state enters a chunk start
          nb = A.chunk;
          // resynchronise where a token at this position follows (pass 2 applies it after pass 1)
          if (A.round_boundary && (stops_at_last_start(MODE) || t0 + tt + 1 < te)) {
#pragma unroll
            for (int c = 0; c < NC; ++c) resync_round(s[c]);
          }
          if (rows_on && row < row_end && row < A.rows_cap) {
#pragma unroll
            for (int c = 0; c < NC; ++c)
#pragma unroll
              for (int r = 0; r < R; r += 8)
                store_f32x8(A.chunk_states + (row * A.h_v + h) * plane +
                                static_cast<int64_t>(col0 + cp * NC + c) * DK + g * R + r,
                            *reinterpret_cast<float(*)[8]>(&s[c][r]));
          }
          ++row;
        }
      }
    };
    if constexpr (is_pass1(MODE)) {
      In nx;
      read_in(0, nx);
      if (n == Cfg::TT) {                      // full tile: unrolled, immediate offsets
#pragma unroll
        for (int tt = 0; tt < Cfg::TT; ++tt) {
          In cur = nx;
          if (tt + 1 < Cfg::TT) read_in(tt + 1, nx);
          token(tt, cur);
        }
      } else {
        for (int tt = 0; tt < n; ++tt) {
          In cur = nx;
          if (tt + 1 < n) read_in(tt + 1, nx);
          token(tt, cur);
        }
      }
    } else if (!is_wide(MODE) && n == Cfg::TT) {   // one-leaf lanes, full tile: unrolled
#pragma unroll
      for (int tt = 0; tt < Cfg::TT; ++tt) {
        In cur;
        read_in(tt, cur);
        token(tt, cur);
      }
    } else {
      for (int tt = 0; tt < n; ++tt) {
        In cur;
        read_in(tt, cur);
        token(tt, cur);
      }
    }
    hand_over();
    ptt = -1;
    __syncthreads();
    if constexpr (MODE == kFused) {                    // the tile's outputs, 8 columns per unit
      for (int u = tid; u < n * (Cfg::WG_COLS / 8); u += Cfg::THREADS) {
        const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = L.o[tt][c8 * 8 + i];
        store8<IO>(A.o, (static_cast<int64_t>(tok0 + t0 + tt) * A.h_v + h) * DV + col0 + c8 * 8, x);
      }
    }
    if constexpr (keeps_c(MODE)) {                     // the tile's c (and w), 4 columns per unit
      for (int u = tid; u < n * (Cfg::WG_COLS / 4); u += Cfg::THREADS) {
        const int tt = u / (Cfg::WG_COLS / 4), c4 = u % (Cfg::WG_COLS / 4);
        const int64_t e = (static_cast<int64_t>(tok0 + t0 + tt) * A.h_v + h) * DV + col0 + c4 * 4;
        *reinterpret_cast<float4*>(A.c_stash + e) = *reinterpret_cast<const float4*>(&L.cs[tt][c4 * 4]);
        if (A.w_stash != nullptr)
          *reinterpret_cast<float4*>(A.w_stash + e) = *reinterpret_cast<const float4*>(&L.ws[tt][c4 * 4]);
      }
    }
    if (more) commit_tile<DK, DV, IO, MODE>(Rg, L);
    __syncthreads();
  }
}

// MODE kBoundary(2): tokens up to the last chunk start; kBoundaryC(2): every token, keeping c (and w).
template <int DK, int DV, int IO, int MODE>
__device__ __forceinline__ void boundary_pass_item(const PrefillArgs& A, int64_t vb) {
  using Cfg = PassCfg<DK, DV, MODE>;
  static_assert(Cfg::R % kLeaf == 0 && Cfg::NC == 1, "pass 1 holds whole leaves of one column per lane");
  static_assert(is_pass1(MODE), "pass 1 modes");
  __shared__ TileLds<DK, DV, MODE> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  // group = (sequence, key head); members = its value heads x column groups
  const int ratio = A.h_v / A.h_k, ncg = DV / Cfg::WG_COLS;
  const GroupSlot gs = xcd_group(vb, ratio * ncg);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k);
  const int h = static_cast<int>(gs.group % A.h_k) * ratio + gs.member / ncg, cg = gs.member % ncg;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = plan_row_offset(A, i, red);
  const int tid = threadIdx.x, lc = tid / Cfg::G, g = tid % Cfg::G;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t col_off = static_cast<int64_t>(cg * Cfg::WG_COLS + lc) * DK + g * Cfg::R;
  float s[1][Cfg::R];
  auto store_s = [&](float* p) {
#pragma unroll
    for (int r = 0; r < Cfg::R; r += 8) store_f32x8(p + r, *reinterpret_cast<float(*)[8]>(&s[0][r]));
  };
  if (m.slot >= 0 && m.len == 0 && !A.from_state) {          // an empty sequence from zero: zero slot
#pragma unroll
    for (int r = 0; r < Cfg::R; ++r) s[0][r] = 0.0f;
    store_s(A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane + col_off);
  }
  if (m.nrows == 0 || row0 >= A.rows_cap) return;            // uniform across the block
  if (A.from_state) {
    const float* src = A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane + col_off;
#pragma unroll
    for (int r = 0; r < Cfg::R; r += 8) load_f32x8(src + r, *reinterpret_cast<float(*)[8]>(&s[0][r]));
  } else {
#pragma unroll
    for (int r = 0; r < Cfg::R; ++r) s[0][r] = 0.0f;
  }
  if (A.round_boundary && m.p0 % A.chunk == 0) resync_round(s[0]);   // the first token is a chunk start
  store_s(A.chunk_states + (row0 * A.h_v + h) * plane + col_off);
  if (stops_at_last_start(MODE) && m.nrows < 2) return;
  // tokens up to the last recorded chunk start (or all of them); the first chunk start is
  // C - p0 % C tokens in
  const int64_t C = A.chunk;
  const int first_nb = static_cast<int>(C - m.p0 % C);
  const int last = keeps_c(MODE) ? m.len : static_cast<int>((m.p0 / C + m.nrows - 1) * C - m.p0);
  run_tokens<DK, DV, IO, MODE>(A, L, s, static_cast<int>(m.tok0), 0, last, h, cg, row0, row0 + m.nrows, first_nb);
}

template <int DK, int DV, int IO, int MODE>
__global__ void __launch_bounds__((PassCfg<DK, DV, MODE>::THREADS)) boundary_pass_kernel(PrefillArgs A) {
  boundary_pass_item<DK, DV, IO, MODE>(A, blockIdx.x);
}

// The same items under a capped grid: each workgroup takes items b, b + gridDim.x, ...
template <int DK, int DV, int IO, int MODE>
__global__ void __launch_bounds__((PassCfg<DK, DV, MODE>::THREADS)) boundary_pass_strided_kernel(PrefillArgs A) {
  for (int64_t vb = blockIdx.x; vb < A.grid_items; vb += gridDim.x) {
    if (vb != blockIdx.x) __syncthreads();                 // the previous item is done with LDS
    boundary_pass_item<DK, DV, IO, MODE>(A, vb);
  }
}

// MODE kOutput: every step predicts c from v; kOutputC: c comes from pass 1's stash.
template <int DK, int DV, int IO, int MODE>
__device__ __forceinline__ void output_pass_item(const PrefillArgs& A, int64_t vb) {
  using Cfg = PassCfg<DK, DV, MODE>;
  static_assert(MODE == kOutput || MODE == kOutputC, "pass 2 modes");
  __shared__ TileLds<DK, DV, MODE> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  // group = (boundary row, key head); members = its value heads x column groups
  const int ratio = A.h_v / A.h_k, ncg = DV / Cfg::WG_COLS;
  const GroupSlot gs = xcd_group(vb, ratio * ncg);
  const int64_t w = gs.group / A.h_k;
  const int h = static_cast<int>(gs.group % A.h_k) * ratio + gs.member / ncg, cg = gs.member % ncg;
  if (w >= A.rows_cap) return;                               // uniform across the block
  int i;
  int64_t c;
  if (!plan_find_row(A, w, &i, &c, red)) return;             // uniform across the block
  const SeqMeta m = seq_meta(A, i);
  const int64_t C = A.chunk;
  const int64_t tb = c == 0 ? 0 : (m.p0 / C + c) * C - m.p0;
  const int64_t next = (m.p0 / C + c + 1) * C - m.p0;
  const int64_t te = next < m.len ? next : m.len;
  const int tid = threadIdx.x, cp = tid / Cfg::G, g = tid % Cfg::G;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  float s[Cfg::NC][Cfg::R];
  const float* src = A.chunk_states + (w * A.h_v + h) * plane;
#pragma unroll
  for (int cc = 0; cc < Cfg::NC; ++cc) {
    const int64_t off = static_cast<int64_t>(cg * Cfg::WG_COLS + cp * Cfg::NC + cc) * DK + g * Cfg::R;
#pragma unroll
    for (int r = 0; r < Cfg::R; r += 8) load_f32x8(src + off + r, *reinterpret_cast<float(*)[8]>(&s[cc][r]));
  }
  run_tokens<DK, DV, IO, MODE>(A, L, s, static_cast<int>(m.tok0), static_cast<int>(tb), static_cast<int>(te), h, cg,
                               0, 0, 0);
  if (c == m.nrows - 1) {
    float* dst = A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane;
#pragma unroll
    for (int cc = 0; cc < Cfg::NC; ++cc) {
      const int64_t off = static_cast<int64_t>(cg * Cfg::WG_COLS + cp * Cfg::NC + cc) * DK + g * Cfg::R;
#pragma unroll
      for (int r = 0; r < Cfg::R; r += 8) store_f32x8(dst + off + r, *reinterpret_cast<float(*)[8]>(&s[cc][r]));
    }
  }
}

template <int DK, int DV, int IO, int MODE>
__global__ void __launch_bounds__((PassCfg<DK, DV, MODE>::THREADS)) output_pass_kernel(PrefillArgs A) {
  output_pass_item<DK, DV, IO, MODE>(A, blockIdx.x);
}

// The same items under a capped grid: each workgroup takes items b, b + gridDim.x, ...
template <int DK, int DV, int IO, int MODE>
__global__ void __launch_bounds__((PassCfg<DK, DV, MODE>::THREADS)) output_pass_strided_kernel(PrefillArgs A) {
  for (int64_t vb = blockIdx.x; vb < A.grid_items; vb += gridDim.x) {
    if (vb != blockIdx.x) __syncthreads();                 // the previous item is done with LDS
    output_pass_item<DK, DV, IO, MODE>(A, vb);
  }
}

// The one-pass variant: every token of a sequence in one launch, with outputs, and (when a stash
// is given) the same chunk-start rows as pass 1.  Same step, same bits as the two passes.
template <int DK, int DV, int IO>
__device__ __forceinline__ void fused_pass_item(const PrefillArgs& A, int64_t vb) {
  using Cfg = PassCfg<DK, DV, kFused>;
  __shared__ TileLds<DK, DV, kFused> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  const int ratio = A.h_v / A.h_k, ncg = DV / Cfg::WG_COLS;
  const GroupSlot gs = xcd_group(vb, ratio * ncg);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k);
  const int h = static_cast<int>(gs.group % A.h_k) * ratio + gs.member / ncg, cg = gs.member % ncg;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = A.chunk_states != nullptr ? plan_row_offset(A, i, red) : 0;
  if (m.slot < 0) return;                                    // uniform across the block
  const int tid = threadIdx.x, lc = tid / Cfg::G, g = tid % Cfg::G;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t col_off = static_cast<int64_t>(cg * Cfg::WG_COLS + lc) * DK + g * Cfg::R;
  float* slot_state = A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane + col_off;
  float s[1][Cfg::R];
  if (A.from_state) {
    load_f32x8(slot_state, s[0]);
  } else {
#pragma unroll
    for (int r = 0; r < Cfg::R; ++r) s[0][r] = 0.0f;
  }
  if (m.len > 0) {
    if (A.round_boundary && m.p0 % A.chunk == 0) resync_round(s[0]);
    if (A.chunk_states != nullptr && row0 < A.rows_cap)
      store_f32x8(A.chunk_states + (row0 * A.h_v + h) * plane + col_off, s[0]);
    const int64_t C = A.chunk;
    const int first_nb = static_cast<int>(C - m.p0 % C);
    run_tokens<DK, DV, IO, kFused>(A, L, s, static_cast<int>(m.tok0), 0, m.len, h, cg, row0, row0 + m.nrows,
                                   first_nb);
  }
  store_f32x8(slot_state, s[0]);
}

template <int DK, int DV, int IO>
__global__ void __launch_bounds__((PassCfg<DK, DV, kFused>::THREADS)) fused_pass_kernel(PrefillArgs A) {
  fused_pass_item<DK, DV, IO>(A, blockIdx.x);
}

// The same items under a capped grid: each workgroup takes items b, b + gridDim.x, ...
template <int DK, int DV, int IO>
__global__ void __launch_bounds__((PassCfg<DK, DV, kFused>::THREADS)) fused_pass_strided_kernel(PrefillArgs A) {
  for (int64_t vb = blockIdx.x; vb < A.grid_items; vb += gridDim.x) {
    if (vb != blockIdx.x) __syncthreads();                 // the previous item is done with LDS
    fused_pass_item<DK, DV, IO>(A, vb);
  }
}

__global__ void prefill_finish_kernel(PrefillArgs A) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= A.num_seqs) return;
  const SeqMeta m = seq_meta(A, i);
  if (m.slot < 0) return;
  A.pos_out[m.slot] = m.p0 + m.len;
}

template <int DK, int DV, int IO, int MODE>
static hipError_t launch_pass1_mode(const PrefillArgs& A, hipStream_t stream) {
  using C1 = PassCfg<DK, DV, MODE>;
  const int64_t g1 = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, A.h_v / A.h_k * (DV / C1::WG_COLS));
  if (g1 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  return launch_items(boundary_pass_kernel<DK, DV, IO, MODE>, boundary_pass_strided_kernel<DK, DV, IO, MODE>, g1,
                      C1::THREADS, stream, A);
}

// Pass 1's lane mapping for a launch.  Two leaves per lane issue fewer instructions per state
// element, but a column's chain then runs on half as many lanes, so each wave carries twice the
// columns and the per-token dependent chain (two leaves, the in-lane add, three DPP levels, w, c,
// the update) is exposed unless many waves share each SIMD -- and the two-leaf kernel's 138 VGPRs
// leave room for only three resident waves per SIMD.  Measured at d_k = 128 (pass 1 with the c
// stash, ms, one leaf / two leaves): 5 x 2048 tokens 0.562 / 0.568; the 10240-token trainer batch
// 0.592 / 0.623; 8 x 2048 0.860 / 0.917; 16 x 2048 1.667 / 1.614; 256 prompts of 1..2048 tokens
// 13.08 / 12.09.  Two leaves are taken from 8 waves per SIMD on (16 or more sequences of
// 32 x 128 columns) on; other head dims, and launches under a workgroup cap, keep one leaf per lane.
bool pass1_two_leaves(int dk, const PrefillArgs& A) {
  if (dk != 128 || A.num_seqs <= 0 || A.max_wgs > 0) return false;
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess || hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) !=
                                              hipSuccess || cus <= 0)
    return false;
  const int64_t simds = 4 * static_cast<int64_t>(cus);
  const int64_t waves2 = static_cast<int64_t>(A.num_seqs) * A.h_v * 128 * 8 / 64;   // columns x 8 lanes
  return waves2 >= 8 * simds;
}

template <int DK, int DV, int IO>
static hipError_t launch_pass1(const PrefillArgs& A, hipStream_t stream) {
  if constexpr (DK == 128) {
    if (pass1_two_leaves(DK, A))
      return A.c_stash != nullptr ? launch_pass1_mode<DK, DV, IO, kBoundaryC2>(A, stream)
                                  : launch_pass1_mode<DK, DV, IO, kBoundary2>(A, stream);
  }
  return A.c_stash != nullptr ? launch_pass1_mode<DK, DV, IO, kBoundaryC>(A, stream)
                              : launch_pass1_mode<DK, DV, IO, kBoundary>(A, stream);
}

template <int DK, int DV, int IO>
static hipError_t launch_prefill_t(const PrefillArgs& A, hipStream_t stream) {
  using C2 = PassCfg<DK, DV, kOutput>;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0) {
    e = launch_pass1<DK, DV, IO>(A, stream);
    if (e != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0 && A.rows_cap > 0) {
    const int64_t g2 = xcd_grid(A.rows_cap * A.h_k, A.h_v / A.h_k * (DV / C2::WG_COLS));
    if (g2 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    if (A.c_stash != nullptr)
      e = launch_items(output_pass_kernel<DK, DV, IO, kOutputC>, output_pass_strided_kernel<DK, DV, IO, kOutputC>, g2,
                       C2::THREADS, stream, A);
    else
      e = launch_items(output_pass_kernel<DK, DV, IO, kOutput>, output_pass_strided_kernel<DK, DV, IO, kOutput>, g2,
                       C2::THREADS, stream, A);
    if (e != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 2, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0) {
    hipLaunchKernelGGL(prefill_finish_kernel, dim3((A.num_seqs + 255) / 256), dim3(256), 0, stream, A);
    e = hipGetLastError();
  }
  return e;
}

template <int DK, int DV, int IO>
static hipError_t launch_fused_t(const PrefillArgs& A, hipStream_t stream) {
  using CF = PassCfg<DK, DV, kFused>;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0) {
    const int64_t gf = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, A.h_v / A.h_k * (DV / CF::WG_COLS));
    if (gf > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    e = launch_items(fused_pass_kernel<DK, DV, IO>, fused_pass_strided_kernel<DK, DV, IO>, gf, CF::THREADS, stream, A);
    if (e != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0) {
    hipLaunchKernelGGL(prefill_finish_kernel, dim3((A.num_seqs + 255) / 256), dim3(256), 0, stream, A);
    e = hipGetLastError();
  }
  return e;
}

hipError_t launch_prefill_fused(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_fused_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefill_finish(const PrefillArgs& A, hipStream_t stream) {
  if (A.num_seqs <= 0) return hipSuccess;
  hipLaunchKernelGGL(prefill_finish_kernel, dim3((A.num_seqs + 255) / 256), dim3(256), 0, stream, A);
  return hipGetLastError();
}

template <int DK, int DV, int IO>
static hipError_t launch_output_pass_only_t(const PrefillArgs& A, hipStream_t stream) {
  using C2 = PassCfg<DK, DV, kOutput>;
  if (A.num_seqs > 0 && A.rows_cap > 0) {
    const int64_t g2 = xcd_grid(A.rows_cap * A.h_k, A.h_v / A.h_k * (DV / C2::WG_COLS));
    if (g2 > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    return launch_items(output_pass_kernel<DK, DV, IO, kOutput>, output_pass_strided_kernel<DK, DV, IO, kOutput>, g2,
                        C2::THREADS, stream, A);
  }
  return hipSuccess;
}

template <int DK, int DV, int IO>
static hipError_t launch_output_pass_t(const PrefillArgs& A, hipStream_t stream) {
  const hipError_t e = launch_output_pass_only_t<DK, DV, IO>(A, stream);
  if (e != hipSuccess) return e;
  return launch_prefill_finish(A, stream);
}

template <int DK, int DV, int IO>
static hipError_t launch_boundary_pass_t(const PrefillArgs& A, hipStream_t stream) {
  if (A.num_seqs <= 0) return hipSuccess;
  return launch_pass1<DK, DV, IO>(A, stream);
}

hipError_t launch_boundary_pass(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_boundary_pass_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_output_pass_only(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_output_pass_only_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_output_pass(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_output_pass_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_prefill(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_prefill_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

}  // namespace cpr
