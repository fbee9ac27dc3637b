// cpr_prefill.hip -- the two CPR passes over a packed varlen batch.
//
// "Solving the linear-attention headache" (IsoExec articles): a first pass computes the
// recurrent state at chunk boundaries, then the outputs inside each chunk are filled in parallel
// from that chunk's boundary state.  Both passes here apply the shared pinned step (cpr_step.hpp)
// to every token, so the states pass 1 stores are exactly the states pass 2 and decode reach.
//
// Work mapping (both passes): one workgroup owns WG_COLS value columns of one value head; a
// column's d_k rows are spread over G = d_k/8 consecutive lanes, one 8-row leaf per lane, so the
// state lives in registers (8 floats per lane).  Token tiles of TT tokens (k, q as fp32, the
// workgroup's v columns, a and b) are staged through LDS; the next tile is fetched into registers
// while the current one is computed.
//   pass 1 (boundary_pass)  grid (sequence, value head, column group); runs each sequence up to
//                           its last chunk start and stores the state entering every chunk.
//   pass 2 (output_pass)    grid (boundary row, value head, column group); a row is one chunk:
//                           load its entering state, run its tokens with output, store o; the
//                           last chunk of a sequence also stores the final state in the slot.
//   finish                  pos[slot] = p0 + length, after both passes have read pos.
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

template <int DK, int DV, int IO>
struct PrefillCfg {
  static constexpr int G = DK / kLeaf;                       // lanes per column
  static constexpr int WG_COLS = (256 / G < DV) ? 256 / G : DV;
  static constexpr int THREADS = WG_COLS * G;
  static constexpr int TT = 32;                              // tokens per LDS tile
  static constexpr int K_UNITS = TT * DK / 8;                // 8-element units per k (or q) tile
  static constexpr int V_UNITS = TT * WG_COLS / 8;
  static constexpr int K_PER_T = (K_UNITS + THREADS - 1) / THREADS;
  static constexpr int V_PER_T = (V_UNITS + THREADS - 1) / THREADS;
  static constexpr int AB_PER_T = (2 * TT + THREADS - 1) / THREADS;
  static_assert(DK % 8 == 0 && DV % WG_COLS == 0 && WG_COLS % 8 == 0, "shape");
  static_assert(THREADS % 64 == 0 || (THREADS & (THREADS - 1)) == 0, "block size");
};

// Registers holding one tile in flight (global -> registers -> LDS).
template <int DK, int DV, int IO, bool OUT>
struct TileRegs {
  using Cfg = PrefillCfg<DK, DV, IO>;
  Raw8<IO> k[Cfg::K_PER_T];
  Raw8<IO> q[OUT ? Cfg::K_PER_T : 1];
  Raw8<IO> v[Cfg::V_PER_T];
  float ab[Cfg::AB_PER_T];
};

template <int DK, int DV, int IO, bool OUT>
struct TileLds {
  using Cfg = PrefillCfg<DK, DV, IO>;
  float k[Cfg::TT][DK];
  float q[OUT ? Cfg::TT : 1][DK];
  float v[Cfg::TT][Cfg::WG_COLS];
  float o[OUT ? Cfg::TT : 1][Cfg::WG_COLS];
  float a[Cfg::TT];
  float b[Cfg::TT];
};

// Fetch tokens [t0, t0 + n) (packed indices, n <= TT) of key head g / value head h into registers.
// Tokens past n are zero-filled and never read from memory.
template <int DK, int DV, int IO, bool OUT>
__device__ __forceinline__ void fetch_tile(const PrefillArgs& A, TileRegs<DK, DV, IO, OUT>& R, int64_t t0,
                                           int n, int kh, int h, int col0) {
  using Cfg = PrefillCfg<DK, DV, IO>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg::K_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    const int tt = u / (DK / 8), c8 = u % (DK / 8);
    const bool ok = u < Cfg::K_UNITS && tt < n;
    const int64_t e = ((t0 + tt) * A.h_k + kh) * DK + c8 * 8;
    R.k[i] = ok ? load_raw8<IO>(A.k, e) : zero_raw8<IO>();
    if constexpr (OUT) R.q[i] = ok ? load_raw8<IO>(A.q, e) : zero_raw8<IO>();
  }
#pragma unroll
  for (int i = 0; i < Cfg::V_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
    const bool ok = u < Cfg::V_UNITS && tt < n;
    const int64_t e = ((t0 + tt) * A.h_v + h) * DV + col0 + c8 * 8;
    R.v[i] = ok ? load_raw8<IO>(A.v, e) : zero_raw8<IO>();
  }
#pragma unroll
  for (int i = 0; i < Cfg::AB_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    const int tt = u % Cfg::TT;
    const bool ok = u < 2 * Cfg::TT && tt < n;
    const float* src = u < Cfg::TT ? A.a : A.b;
    R.ab[i] = ok ? src[(t0 + tt) * A.h_v + h] : 0.0f;
  }
}

template <int DK, int DV, int IO, bool OUT>
__device__ __forceinline__ void commit_tile(const TileRegs<DK, DV, IO, OUT>& R, TileLds<DK, DV, IO, OUT>& L) {
  using Cfg = PrefillCfg<DK, DV, IO>;
  const int tid = threadIdx.x;
#pragma unroll
  for (int i = 0; i < Cfg::K_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    if (u < Cfg::K_UNITS) {
      const int tt = u / (DK / 8), c8 = u % (DK / 8);
      float x[8];
      widen8<IO>(R.k[i], x);
      store_f32x8(&L.k[tt][c8 * 8], x);
      if constexpr (OUT) {
        widen8<IO>(R.q[i], x);
        store_f32x8(&L.q[tt][c8 * 8], x);
      }
    }
  }
#pragma unroll
  for (int i = 0; i < Cfg::V_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    if (u < Cfg::V_UNITS) {
      const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
      float x[8];
      widen8<IO>(R.v[i], x);
      store_f32x8(&L.v[tt][c8 * 8], x);
    }
  }
#pragma unroll
  for (int i = 0; i < Cfg::AB_PER_T; ++i) {
    const int u = tid + i * Cfg::THREADS;
    if (u < Cfg::TT)
      L.a[u] = R.ab[i];
    else if (u < 2 * Cfg::TT)
      L.b[u - Cfg::TT] = R.ab[i];
  }
}

// Run tokens [tb, te) (offsets from the sequence start) of one sequence through this lane's column
// slice.  OUT: write o for every token.  !OUT: store the state entering every chunk start reached
// inside (tb, te] into chunk_states.
template <int DK, int DV, int IO, bool OUT>
__device__ __forceinline__ void run_tokens(const PrefillArgs& A, TileLds<DK, DV, IO, OUT>& L, float (&s)[8],
                                           const SeqMeta& m, int64_t row0, int64_t tb, int64_t te, int h,
                                           int cg) {
  using Cfg = PrefillCfg<DK, DV, IO>;
  constexpr int G = Cfg::G;
  const int tid = threadIdx.x;
  const int lc = tid / G, g = tid % G;
  const int col0 = cg * Cfg::WG_COLS;
  const int kh = h / (A.h_v / A.h_k);
  const int64_t C = A.chunk;
  const int64_t plane = static_cast<int64_t>(DV) * DK;      // one head's state

  TileRegs<DK, DV, IO, OUT> R;
  if (tb < te) {
    fetch_tile<DK, DV, IO, OUT>(A, R, m.tok0 + tb, static_cast<int>(te - tb < Cfg::TT ? te - tb : Cfg::TT), kh, h,
                                col0);
    commit_tile<DK, DV, IO, OUT>(R, L);
  }
  __syncthreads();
  for (int64_t t0 = tb; t0 < te; t0 += Cfg::TT) {
    const int n = static_cast<int>(te - t0 < Cfg::TT ? te - t0 : Cfg::TT);
    const int64_t t1 = t0 + Cfg::TT;
    const bool more = t1 < te;
    if (more)
      fetch_tile<DK, DV, IO, OUT>(A, R, m.tok0 + t1, static_cast<int>(te - t1 < Cfg::TT ? te - t1 : Cfg::TT), kh, h,
                                  col0);
    for (int tt = 0; tt < n; ++tt) {
      float kr[8], qr[8];
      load_f32x8(&L.k[tt][g * 8], kr);
      if constexpr (OUT) load_f32x8(&L.q[tt][g * 8], qr);
      const float o = cpr_step<1, G, OUT>(s, kr, qr, L.v[tt][lc], L.a[tt], L.b[tt]);
      if constexpr (OUT) {
        if (g == 0) L.o[tt][lc] = o;
      } else {
        const int64_t p = m.p0 + t0 + tt + 1;               // position the new state enters
        if (p % C == 0 && t0 + tt + 1 <= te) {
          const int64_t row = row0 + (p / C - m.p0 / C);
          if (row < A.rows_cap)
            store_f32x8(A.chunk_states + (row * A.h_v + h) * plane + static_cast<int64_t>(col0 + lc) * DK + g * 8, s);
        }
      }
    }
    __syncthreads();
    if constexpr (OUT) {
      // the tile's outputs, 8 columns per unit
      for (int u = tid; u < n * (Cfg::WG_COLS / 8); u += Cfg::THREADS) {
        const int tt = u / (Cfg::WG_COLS / 8), c8 = u % (Cfg::WG_COLS / 8);
        float x[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) x[i] = L.o[tt][c8 * 8 + i];
        store8<IO>(A.o, ((m.tok0 + t0 + tt) * A.h_v + h) * DV + col0 + c8 * 8, x);
      }
    }
    if (more) commit_tile<DK, DV, IO, OUT>(R, L);
    __syncthreads();
  }
}

template <int DK, int DV, int IO>
__global__ void __launch_bounds__((PrefillCfg<DK, DV, IO>::THREADS)) boundary_pass_kernel(PrefillArgs A) {
  using Cfg = PrefillCfg<DK, DV, IO>;
  __shared__ TileLds<DK, DV, IO, false> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  const int i = blockIdx.x, h = blockIdx.y, cg = blockIdx.z;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = plan_row_offset(A, i, red);
  const int tid = threadIdx.x, lc = tid / Cfg::G, g = tid % Cfg::G;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t col_off = static_cast<int64_t>(cg * Cfg::WG_COLS + lc) * DK + g * 8;
  float s[8];
  if (m.slot >= 0 && m.len == 0 && !A.from_state) {          // an empty sequence from zero: zero slot
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = 0.0f;
    store_f32x8(A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane + col_off, s);
  }
  if (m.nrows == 0 || row0 >= A.rows_cap) return;            // uniform across the block
  if (A.from_state) {
    load_f32x8(A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane + col_off, s);
  } else {
#pragma unroll
    for (int r = 0; r < 8; ++r) s[r] = 0.0f;
  }
  store_f32x8(A.chunk_states + (row0 * A.h_v + h) * plane + col_off, s);
  // tokens up to the last recorded chunk start
  const int64_t C = A.chunk;
  const int64_t last = m.nrows > 1 ? (m.p0 / C + m.nrows - 1) * C - m.p0 : 0;
  run_tokens<DK, DV, IO, false>(A, L, s, m, row0, 0, last, h, cg);
}

template <int DK, int DV, int IO>
__global__ void __launch_bounds__((PrefillCfg<DK, DV, IO>::THREADS)) output_pass_kernel(PrefillArgs A) {
  using Cfg = PrefillCfg<DK, DV, IO>;
  __shared__ TileLds<DK, DV, IO, true> L;
  __shared__ int64_t red[(Cfg::THREADS + 63) / 64 + 2];
  const int64_t w = blockIdx.x;
  const int h = blockIdx.y, cg = blockIdx.z;
  if (w >= A.rows_cap) return;
  int i;
  int64_t c;
  if (!plan_find_row(A, w, &i, &c, red)) return;             // uniform across the block
  const SeqMeta m = seq_meta(A, i);
  const int64_t C = A.chunk;
  const int64_t tb = c == 0 ? 0 : (m.p0 / C + c) * C - m.p0;
  const int64_t next = (m.p0 / C + c + 1) * C - m.p0;
  const int64_t te = next < m.len ? next : m.len;
  const int tid = threadIdx.x, lc = tid / Cfg::G, g = tid % Cfg::G;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t col_off = static_cast<int64_t>(cg * Cfg::WG_COLS + lc) * DK + g * 8;
  float s[8];
  load_f32x8(A.chunk_states + (w * A.h_v + h) * plane + col_off, s);
  run_tokens<DK, DV, IO, true>(A, L, s, m, w - c, tb, te, h, cg);
  if (c == m.nrows - 1) store_f32x8(A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane + col_off, s);
}

__global__ void prefill_finish_kernel(PrefillArgs A) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= A.num_seqs) return;
  const SeqMeta m = seq_meta(A, i);
  if (m.slot < 0) return;
  A.pos_out[m.slot] = m.p0 + m.len;
}

template <int DK, int DV, int IO>
static hipError_t launch_prefill_t(const PrefillArgs& A, hipStream_t stream) {
  using Cfg = PrefillCfg<DK, DV, IO>;
  const dim3 block(Cfg::THREADS);
  const unsigned ncg = DV / Cfg::WG_COLS;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0) {
    hipLaunchKernelGGL((boundary_pass_kernel<DK, DV, IO>), dim3(A.num_seqs, A.h_v, ncg), block, 0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0 && A.rows_cap > 0) {
    hipLaunchKernelGGL((output_pass_kernel<DK, DV, IO>), dim3(static_cast<unsigned>(A.rows_cap), A.h_v, ncg), block, 0,
                       stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 2, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0) {
    hipLaunchKernelGGL(prefill_finish_kernel, dim3((A.num_seqs + 255) / 256), dim3(256), 0, stream, A);
    e = hipGetLastError();
  }
  return e;
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
