// cpr_overlap.hip -- prefill with the chunk outputs produced while pass 1 runs on.
//
// "Solving the linear-attention headache" (IsoExec articles): pass 1 walks each sequence to find
// the state at every chunk start, pass 2 fills in each chunk's outputs from that state.  When the
// batch is a few long sequences, pass 1 has one wave per SIMD (its columns are all the
// parallelism there is) and each token's dependent chain leaves most issue slots idle, so pass 2
// run afterwards is pure added time.  Here one workgroup owns a group of columns of one value
// head and holds three kinds of waves:
//   P pass-1 waves (raised issue priority) run every token of the sequence with the shared pinned
//     step, one leaf of 8 rows per lane, and hand each finished chunk over through LDS: the state
//     entering the chunk and every token's c;
//   NH pass-2 waves take the handed-over chunks in turn (chunk c to wave c mod NH), apply each
//     token's c to the chunk's state -- the same bits as the output pass given pass 1's c --
//     store the chunk-start row and write o; with NH = 4 each SIMD holds one pass-1 and one
//     pass-2 wave, so pass 2's arithmetic fills the slots pass 1's chain leaves idle;
//   one staging wave loads pass 1's inputs a tile ahead (k widened to fp32 in the lane order pass
//     1 reads, v, the gates), so pass 1 reads them from LDS with fixed offsets and spends no
//     issue slots on addressing or widening.
// The waves meet only through LDS counters (chunks handed over, chunks released, tiles staged,
// tiles consumed), on the same CU, so no data crosses XCDs or L2s; NH + 1 hand-off buffers let
// pass 1 run up to NH chunks ahead.  Every wait is bounded, so a wave that is never signalled
// still finishes.  A wave whose wait gives up touches no shared buffer afterwards: it ORs a flag
// into the device's status word (read back by gdn_device_status, which then reports GDN_EHIP) and
// leaves the item, so the call's results are refused rather than silently wrong (section "The
// execution contract": refuse to run rather than run mismatched numerics).
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

template <int DK, int DV>
struct OvCfg {
  static constexpr int G = DK / kLeaf;                        // pass 1: lanes per column, one leaf each
  static constexpr int CP = 64 / G;                           // pass 1: columns per wave
  static constexpr int CW = (4 * CP < DV) ? 4 * CP : DV;      // columns of a workgroup
  static constexpr int P = (CW * G + 63) / 64;                // pass-1 waves
  static constexpr int G2 = (64 / CW < DK / kLeaf) ? 64 / CW : DK / kLeaf;   // pass 2: lanes per column
  static constexpr int NL2 = DK / (kLeaf * G2);               // pass 2: leaves per lane
  static constexpr int R2 = NL2 * kLeaf;                      // pass 2: rows per lane
  static constexpr int NCG = DV / CW;                         // column groups per value head
  static constexpr int NH = 4;                                // pass-2 waves: with the pass-1 waves,
                                                              //   two waves on each SIMD
  static constexpr int THREADS = (P + NH + 1) * 64;          // and one wave staging pass 1's inputs
  static constexpr int TT = 32;                               // pass 1: tokens per staged tile
  static constexpr int NT = 2;                                // staged tiles in flight
  static constexpr int KU = (TT * DK / 8 + 63) / 64;          // staging: k units per lane
  static constexpr int VU = (TT * CW / 8 + 63) / 64;          // staging: v units per lane
  static constexpr int TH = 4;                                // pass 2: tokens per tile
  static constexpr int CMAX = 64;                             // largest chunk this kernel takes
  static constexpr int NB = NH + 1;                           // hand-off buffers
  static constexpr int KU2 = (TH * DK / 8 + 63) / 64;         // pass 2: k (and q) units per lane
  static_assert(DV % CW == 0 && CW % 8 == 0 && CW * G2 <= 64 && DK % (kLeaf * G2) == 0, "shape");
};

template <int DK, int DV>
struct alignas(16) OvTile {
  using O = OvCfg<DK, DV>;
  float k[O::TT][DK];                 // widened, lane-interleaved for one-leaf lanes
  float v[O::TT][O::CW];
  float2 ab[O::TT];
};

template <int DK, int DV>
struct alignas(16) OvLds {
  using O = OvCfg<DK, DV>;
  OvTile<DK, DV> tile[O::NT];         // pass 1's inputs, staged a tile ahead
  float hk[O::NH][O::TH][DK];         // pass 2, per wave: k and q rows of its tile (lane-interleaved),
  float hq[O::NH][O::TH][DK];         //   a, and the chunk's outputs gathered for wider stores
  float ha[O::NH][O::TH];
  float ho[O::NH][O::CMAX][O::CW];
  float hs[O::NB][O::CW][DK];         // state entering a handed-over chunk ([column][row])
  float hc[O::NB][O::CMAX][O::CW];    // c of each of its tokens, by position within the chunk
  int handed[O::P];                   // chunks each pass-1 wave has completed
  int consumed[O::P];                 // staged tiles each pass-1 wave has finished with
  int loaded;                         // tiles staged
  int released[O::NH];                // chunks each pass-2 wave has finished with
};

constexpr uint32_t kSpinLimit = 1u << 22;   // ~0.2 s of s_sleep polls: far beyond any real wait

// Which wait gave up, as bits of the status word.
enum : uint32_t {
  kGaveUpTile = 1u,       // a pass-1 wave waiting for its staged input tile
  kGaveUpBuffer = 2u,     // a pass-1 wave waiting for a free hand-off buffer
  kGaveUpHandOff = 4u,    // a pass-2 wave waiting for a handed-over chunk
  kGaveUpStaging = 8u,    // the staging wave waiting for a free tile buffer
};

// The device's status word: flags of bounded waits that gave up since the host last read it.
__device__ uint32_t g_wait_status;

// Wait until *cnt >= target (workgroup-scope acquire), polling at most `limit` times; false if
// the bound ran out.  The result is the same in every lane of the wave.
__device__ __forceinline__ bool wait_count(const int* cnt, int target, uint32_t limit) {
  for (uint32_t it = 0; it < limit; ++it) {
    const int seen = __builtin_amdgcn_readfirstlane(__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP));
    if (seen >= target) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

// Record that a wait of this wave gave up (one lane's vector atomic).
__device__ __forceinline__ void gave_up(const PrefillArgs& A, uint32_t what) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_fetch_or(A.status, what, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A pass-1 token's inputs for one lane: its 8 rows of k, its column's v, the gates.
struct OvIn {
  float k[kLeaf];
  float v;
  float2 ab;
};

template <int DK, int DV, int IO>
__device__ __forceinline__ void overlap_item(const PrefillArgs& A, int64_t vb) {
  using O = OvCfg<DK, DV>;
  constexpr int G = O::G, CW = O::CW, P = O::P, G2 = O::G2, NL2 = O::NL2, R2 = O::R2, TH = O::TH, TT = O::TT;
  __shared__ OvLds<DK, DV> L;
  __shared__ int64_t red[(O::THREADS + 63) / 64 + 2];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(vb, ratio * O::NCG);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k), kh = static_cast<int>(gs.group % A.h_k);
  const int h = kh * ratio + gs.member / O::NCG, col0 = (gs.member % O::NCG) * CW;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = plan_row_offset(A, i, red);
  if (m.slot < 0) return;                                      // uniform across the block
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t C = A.chunk;
  if (m.len == 0) {                                            // nothing to run; from zero: zero slot
    if (wave < P && !A.from_state) {
      const int cw = wave * O::CP + lane / G;
      if (cw < CW) {
        float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
        store_f32x8(A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane +
                        static_cast<int64_t>(col0 + cw) * DK + (lane % G) * kLeaf, z);
      }
    }
    return;
  }
  if (threadIdx.x == 0) {
    for (int p = 0; p < P; ++p) L.handed[p] = 0;
    for (int p = 0; p < P; ++p) L.consumed[p] = 0;
    L.loaded = 0;
    for (int p = 0; p < O::NH; ++p) L.released[p] = 0;
  }
  __syncthreads();                      // the last block-wide barrier: the waves now meet only in LDS
  const int nchunks = static_cast<int>(m.nrows);
  const bool rows_on = A.chunk_states != nullptr;
  const uint32_t limit = A.wait_limit != 0 ? A.wait_limit : kSpinLimit;

  if (wave < P) {
    // ---------------------------------------------------------------- pass 1
    __builtin_amdgcn_s_setprio(3);
    const int lc = lane / G, g = lane % G, cw = wave * O::CP + lc;
    const bool act = cw < CW;                                  // lanes past the columns idle
    const int64_t col_off = static_cast<int64_t>(col0 + (act ? cw : 0)) * DK + g * kLeaf;
    float* slot_state = A.state + (static_cast<int64_t>(m.slot) * A.h_v + h) * plane + col_off;
    float s[kLeaf];
    if (A.from_state) {
      load_f32x8(slot_state, s);
    } else {
#pragma unroll
      for (int r = 0; r < kLeaf; ++r) s[r] = 0.0f;
    }
    if (A.round_boundary && m.p0 % C == 0) resync_round(s);   // the first token is a chunk start
    if (act) store_f32x8(&L.hs[0][cw][g * kLeaf], s);
    const int first = static_cast<int>(C - m.p0 % C);          // tokens until the next chunk start
    int left = first < m.len ? first : m.len;                  // tokens of this chunk still to run
    int c = 0;                                                 // chunk being run
    int cbuf = 0, pos = static_cast<int>(m.p0 % C);            // its hand-off buffer; token position
    float pc = 0.0f;                                           // c of the previous token, not yet in LDS
    int pslot = -1;
    bool stop = false;                                         // a wait gave up: no further token runs
    auto read_in = [&](const OvTile<DK, DV>& T, int tt, OvIn& x) {
      lds_read_kq<G, kLeaf>(&T.k[tt][0], g, x.k);
      x.v = T.v[tt][act ? cw : 0];
      x.ab = T.ab[tt];
    };
    auto run_token = [&](int t, const OvIn& x) {
      if (stop) return;                                        // uniform across the wave
      // the previous token's c goes to LDS first, so the lane-masked write does not split this
      // token's arithmetic
      if (pslot >= 0 && g == 0 && act) L.hc[cbuf][pslot][cw] = pc;
      float u, w;
      cpr_update<1, G>(s, x.k, x.v, x.ab.x, x.ab.y, u, w, pc);
      pslot = pos++;
      if (--left == 0) {                                       // chunk c is complete
        if (g == 0 && act) L.hc[cbuf][pslot][cw] = pc;
        pslot = -1;
        const bool last = t + 1 == m.len;
        if (!last) {
          if (A.round_boundary) resync_round(s);               // a chunk start with a token to follow
          // chunk c + 1 goes to the buffer chunk c + 1 - NB = c - NH used: wait until its pass-2
          // wave (c mod NH) is done with it, i.e. has released c / NH chunks.  If that wait gives
          // up the buffer may still be in use: chunk c is not handed over and the wave stops.
          if (c >= O::NH && !wait_count(&L.released[c % O::NH], c / O::NH, limit)) {
            gave_up(A, kGaveUpBuffer);
            stop = true;
            return;
          }
          cbuf = cbuf + 1 == O::NB ? 0 : cbuf + 1;
          if (act) store_f32x8(&L.hs[cbuf][cw][g * kLeaf], s);
          pos = 0;
          left = m.len - (t + 1) < C ? m.len - (t + 1) : static_cast<int>(C);
        }
        ++c;
        if (lane == 0) __hip_atomic_store(&L.handed[wave], c, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    };
    // tile by tile as the staging wave provides them; within a tile the next token's inputs are
    // read from LDS while the current one runs
    for (int it = 0, t0 = 0; t0 < m.len && !stop; ++it, t0 += TT) {
      if (!wait_count(&L.loaded, it + 1, limit)) {
        gave_up(A, kGaveUpTile);
        stop = true;
        break;
      }
      const OvTile<DK, DV>& T = L.tile[it % O::NT];
      const int n = m.len - t0 < TT ? m.len - t0 : TT;
      OvIn nx;
      read_in(T, 0, nx);
      if (n == TT) {                                           // full tile: unrolled, immediate offsets
#pragma unroll
        for (int tt = 0; tt < TT; ++tt) {
          const OvIn cur = nx;
          if (tt + 1 < TT) read_in(T, tt + 1, nx);
          run_token(t0 + tt, cur);
        }
      } else {
        for (int tt = 0; tt < n; ++tt) {
          const OvIn cur = nx;
          if (tt + 1 < n) read_in(T, tt + 1, nx);
          run_token(t0 + tt, cur);
        }
      }
      if (lane == 0 && !stop)                                  // the tile's buffer may be refilled
        __hip_atomic_store(&L.consumed[wave], it + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
    if (act && !stop) store_f32x8(slot_state, s);
  } else if (wave < P + O::NH) {
    // ---------------------------------------------------------------- pass 2
    // Wave P + w takes chunks w, w + NH, ... with G2 lanes per column and R2 rows per lane.  Its
    // tiles' inputs (k, q, a) do not depend on pass 1, so the next tile -- also the first of its
    // next chunk -- is fetched while one runs; only the chunk hand-offs wait on pass 1.
    const int w = wave - P;
    const int col = lane / G2, g2 = lane % G2;
    const bool act = col < CW;
    const int64_t p0 = m.p0;
    auto chunk_span = [&](int cc, int* tb, int* te) {
      *tb = cc == 0 ? 0 : static_cast<int>((p0 / C + cc) * C - p0);
      const int64_t next = (p0 / C + cc + 1) * C - p0;
      *te = next < m.len ? static_cast<int>(next) : m.len;
    };
    Raw8<IO> rk[O::KU2], rq[O::KU2];
    float ra = 0.0f;
    auto fetch = [&](int h0, int n) {
#pragma unroll
      for (int x = 0; x < O::KU2; ++x) {
        const int u = lane + 64 * x, tt = u / (DK / 8), c8 = u % (DK / 8);
        if (u < TH * DK / 8 && tt < n) {
          const int64_t e = ((m.tok0 + h0 + tt) * A.h_k + kh) * DK + c8 * 8;
          rk[x] = load_raw8<IO>(A.k, e);
          rq[x] = load_raw8<IO>(A.q, e);
        }
      }
      if (lane < n) ra = A.a[(m.tok0 + h0 + lane) * A.h_v + h];
    };
    auto commit = [&]() {
#pragma unroll
      for (int x = 0; x < O::KU2; ++x) {
        const int u = lane + 64 * x;
        if (u < TH * DK / 8) {
          float y[8];
          widen8<IO>(rk[x], y);
          store_kq8<G2, R2>(&L.hk[w][u / (DK / 8)][0], (u % (DK / 8)) * 8, y);
          widen8<IO>(rq[x], y);
          store_kq8<G2, R2>(&L.hq[w][u / (DK / 8)][0], (u % (DK / 8)) * 8, y);
        }
      }
      if (lane < TH) L.ha[w][lane] = ra;
    };
    int tb = 0, te = 0;
    if (w < nchunks) {
      chunk_span(w, &tb, &te);
      fetch(tb, te - tb < TH ? te - tb : TH);
    }
    for (int c = w; c < nchunks; c += O::NH) {
      bool ready = true;                                       // every pass-1 wave is past chunk c
#pragma unroll
      for (int p = 0; p < P; ++p) ready = ready && wait_count(&L.handed[p], c + 1, limit);
      if (!ready) {
        gave_up(A, kGaveUpHandOff);
        break;
      }
      const int off = c == 0 ? static_cast<int>(p0 % C) : 0;  // position of token tb in the chunk
      float s[R2];
#pragma unroll
      for (int r = 0; r < R2; r += 8)
        load_f32x8(&L.hs[c % O::NB][act ? col : 0][g2 * R2 + r], *reinterpret_cast<float(*)[8]>(&s[r]));
      if (rows_on && act && row0 + c < A.rows_cap) {           // the chunk-start row, stored from here
        float* rp = A.chunk_states + ((row0 + c) * A.h_v + h) * plane + static_cast<int64_t>(col0 + col) * DK + g2 * R2;
#pragma unroll
        for (int r = 0; r < R2; r += 8) store_f32x8(rp + r, *reinterpret_cast<float(*)[8]>(&s[r]));
      }
      for (int h0 = tb; h0 < te; h0 += TH) {
        const int n = te - h0 < TH ? te - h0 : TH;
        commit();
        __builtin_amdgcn_wave_barrier();
        if (h0 + TH < te) {                                    // the chunk's next tile
          fetch(h0 + TH, te - h0 - TH < TH ? te - h0 - TH : TH);
        } else if (c + O::NH < nchunks) {                      // the first tile of the next chunk
          int nb0, ne0;
          chunk_span(c + O::NH, &nb0, &ne0);
          fetch(nb0, ne0 - nb0 < TH ? ne0 - nb0 : TH);
        }
        for (int tt = 0; tt < n; ++tt) {
          const int t = h0 + tt;
          float kr[R2], qr[R2];
          lds_read_kq<G2, R2>(&L.hk[w][tt][0], g2, kr);
          lds_read_kq<G2, R2>(&L.hq[w][tt][0], g2, qr);
          const float cv = act ? L.hc[c % O::NB][t - tb + off][col] : 0.0f;
          const float o = cpr_step_given_c<NL2, G2>(s, kr, qr, L.ha[w][tt], cv);
          if (g2 == 0 && act) L.ho[w][t - tb][col] = o;
        }
        __builtin_amdgcn_wave_barrier();                       // the tile's reads come before its refill
      }
      if (lane == 0)                                           // hs and hc of chunk c are free again
        __hip_atomic_store(&L.released[w], c / O::NH + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
      __builtin_amdgcn_wave_barrier();
      for (int r = lane; r < te - tb; r += 64) {               // the chunk's outputs, a token per lane
        const int64_t oe = (static_cast<int64_t>(m.tok0 + tb + r) * A.h_v + h) * DV + col0;
#pragma unroll
        for (int j = 0; j < CW; j += 8) {
          float y[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) y[e] = L.ho[w][r][j + e];
          store8<IO>(A.o, oe + j, y);
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (c + O::NH < nchunks) chunk_span(c + O::NH, &tb, &te);
    }
  } else {
    // ---------------------------------------------------------------- staging
    // Tile it of pass 1's inputs goes to buffer it mod NT once every pass-1 wave is done with
    // tile it - NT: k widened to fp32 in the one-leaf lane-interleaved order, v, and a with b.
    for (int it = 0, t0 = 0; t0 < m.len; ++it, t0 += TT) {
      bool free_ = true;
      if (it >= O::NT) {
#pragma unroll
        for (int p = 0; p < P; ++p) free_ = free_ && wait_count(&L.consumed[p], it - O::NT + 1, limit);
      }
      if (!free_) {
        gave_up(A, kGaveUpStaging);
        break;
      }
      OvTile<DK, DV>& T = L.tile[it % O::NT];
      const int n = m.len - t0 < TT ? m.len - t0 : TT;
      Raw8<IO> rk[O::KU], rv[O::VU];
      float2 ab = make_float2(0.0f, 0.0f);
#pragma unroll
      for (int x = 0; x < O::KU; ++x) {
        const int u = lane + 64 * x, tt = u / (DK / 8);
        if (u < TT * DK / 8 && tt < n)
          rk[x] = load_raw8<IO>(A.k, ((m.tok0 + t0 + tt) * A.h_k + kh) * DK + (u % (DK / 8)) * 8);
      }
#pragma unroll
      for (int x = 0; x < O::VU; ++x) {
        const int u = lane + 64 * x, tt = u / (CW / 8);
        if (u < TT * CW / 8 && tt < n)
          rv[x] = load_raw8<IO>(A.v, ((m.tok0 + t0 + tt) * A.h_v + h) * DV + col0 + (u % (CW / 8)) * 8);
      }
      if (lane < n) {
        const int64_t e = (m.tok0 + t0 + lane) * A.h_v + h;
        ab = make_float2(A.a[e], A.b[e]);
      }
#pragma unroll
      for (int x = 0; x < O::KU; ++x) {
        const int u = lane + 64 * x, tt = u / (DK / 8);
        if (u < TT * DK / 8 && tt < n) {
          float y[8];
          widen8<IO>(rk[x], y);
          store_kq8<G, kLeaf>(&T.k[tt][0], (u % (DK / 8)) * 8, y);
        }
      }
#pragma unroll
      for (int x = 0; x < O::VU; ++x) {
        const int u = lane + 64 * x, tt = u / (CW / 8);
        if (u < TT * CW / 8 && tt < n) {
          float y[8];
          widen8<IO>(rv[x], y);
          float4* d = reinterpret_cast<float4*>(&T.v[tt][(u % (CW / 8)) * 8]);
          d[0] = make_float4(y[0], y[1], y[2], y[3]);
          d[1] = make_float4(y[4], y[5], y[6], y[7]);
        }
      }
      if (lane < n) T.ab[lane] = ab;
      if (lane == 0) __hip_atomic_store(&L.loaded, it + 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
    }
  }
}

template <int DK, int DV, int IO>
__global__ void __launch_bounds__((OvCfg<DK, DV>::THREADS)) overlap_kernel(PrefillArgs A) {
  overlap_item<DK, DV, IO>(A, blockIdx.x);
}

// The same items under a capped grid: each workgroup takes items b, b + gridDim.x, ...
template <int DK, int DV, int IO>
__global__ void __launch_bounds__((OvCfg<DK, DV>::THREADS)) overlap_strided_kernel(PrefillArgs A) {
  for (int64_t vb = blockIdx.x; vb < A.grid_items; vb += gridDim.x) {
    if (vb != blockIdx.x) __syncthreads();                 // every wave is done with the previous item
    overlap_item<DK, DV, IO>(A, vb);
  }
}

template <int DK, int DV, int IO>
static hipError_t launch_overlap_t(const PrefillArgs& A0, hipStream_t stream) {
  using O = OvCfg<DK, DV>;
  PrefillArgs A = A0;
  hipError_t e = wait_status_word(&A.status);
  if (e != hipSuccess) return e;
  if ((e = record_event(A.events, 0, stream)) != hipSuccess) return e;
  if (A.num_seqs > 0) {
    const int64_t grid = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, A.h_v / A.h_k * O::NCG);
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    e = launch_items(overlap_kernel<DK, DV, IO>, overlap_strided_kernel<DK, DV, IO>, grid, O::THREADS, stream, A);
    if (e != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  return launch_prefill_finish(A, stream);
}

int overlap_max_chunk() { return OvCfg<128, 128>::CMAX; }

// The status word of the current device, found once per device by symbol (its host-side name is
// no device address).
hipError_t wait_status_word(uint32_t** out) {
  constexpr int kMaxDevices = 64;
  static uint32_t* words[kMaxDevices] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  uint32_t* w = __atomic_load_n(&words[dev], __ATOMIC_ACQUIRE);
  if (w == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(g_wait_status));
    if (e != hipSuccess) return e;
    w = static_cast<uint32_t*>(p);
    __atomic_store_n(&words[dev], w, __ATOMIC_RELEASE);
  }
  *out = w;
  return hipSuccess;
}

// The kernel's LDS holds one workgroup per CU, so a grid larger than the CU count would run in
// rounds, each as long as the longest sequence; the one-pass kernel is faster there.
bool overlap_fits(int dk, int dv, const PrefillArgs& A) {
  int ncg = 0;
  if (dk == dv) {
    switch (dk) {
      case 16: ncg = OvCfg<16, 16>::NCG; break;
      case 32: ncg = OvCfg<32, 32>::NCG; break;
      case 64: ncg = OvCfg<64, 64>::NCG; break;
      case 128: ncg = OvCfg<128, 128>::NCG; break;
      default: return false;
    }
  }
  int dev = 0, cus = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
    return false;
  const int64_t items = static_cast<int64_t>(A.num_seqs) * A.h_v * ncg;
  return (A.max_wgs > 0 && A.max_wgs < items ? A.max_wgs : items) <= cus;
}

hipError_t launch_prefill_overlap(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_overlap_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

}  // namespace cpr
