// cpr_overlap.hip -- prefill with the chunk outputs produced while pass 1 runs on.
//
// "Solving the linear-attention headache" (IsoExec articles): pass 1 walks each sequence to find
// the state at every chunk start, pass 2 fills in each chunk's outputs from that state.  When the
// batch is a few long sequences, pass 1 has one wave per SIMD (its columns are all the
// parallelism there is) and each token's dependent chain leaves most issue slots idle, so pass 2
// run afterwards is pure added time.  Here one workgroup holds three waves over the same columns:
//   wave 0 (pass 1, raised issue priority) runs every token of the sequence with the shared
//     pinned step, stores the chunk-start rows and the final state, and hands each finished
//     chunk over through LDS: the state entering the chunk and every token's c;
//   waves 1 and 2 (pass 2) take the handed-over chunks in turn, apply each token's c to the
//     chunk's state and write o -- the same bits as the output pass given pass 1's c.  Each
//     token of pass 2 is a short dependent chain too, so two waves share the chunks to keep pace.
// The waves meet only through LDS counters (chunks handed over; chunks each pass-2 wave has
// released), on the same CU, so no data crosses XCDs or L2s; three hand-off buffers let wave 0
// run up to two chunks ahead.  Every wait is bounded, so a wave that is never signalled still
// finishes.
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

template <int DK, int DV>
struct OvCfg {
  static constexpr int G = DK / kLeaf;                        // lanes per column, one leaf each
  static constexpr int COLS = (64 / G < DV) ? 64 / G : DV;    // columns of a workgroup (one wave)
  static constexpr int NCG = DV / COLS;                       // column groups per value head
  static constexpr int TT = 32;                               // tokens per pass-1 tile
  static constexpr int TH = 4;                                // tokens per pass-2 tile
  static constexpr int NB = 3;                                // hand-off buffers
  static constexpr int CMAX = 64;                             // largest chunk this kernel takes
  static constexpr int KU1 = TT * DK / 8 / 64;                // 8-element k units per lane, pass 1
  static constexpr int KU2 = (TH * DK / 8 + 63) / 64;         // k (and q) units per lane, pass 2
  static_assert(DV % COLS == 0 && KU1 >= 1, "shape");
};

template <int DK, int DV, int IO>
struct alignas(16) OvLds {
  using O = OvCfg<DK, DV>;
  float k[O::TT][DK];              // pass 1: k rows of the tile (lane-interleaved, kq_slot)
  float v[O::TT][O::COLS];
  float2 ab[O::TT];
  float hk[2][O::TH][DK];          // pass 2, per wave: k and q rows of its tile (lane-interleaved),
  float hq[2][O::TH][DK];          //   a, and the chunk's outputs gathered for wider stores
  float ha[2][O::TH];
  float ho[2][O::CMAX][O::COLS];
  float hs[O::NB][O::COLS][DK];    // state entering a handed-over chunk ([column][row])
  float hc[O::NB][O::CMAX][O::COLS];  // c of each of its tokens, by position within the chunk
  int handed;                      // chunks wave 0 has handed over
  int released[2];                 // chunks each pass-2 wave has finished with
};

constexpr uint32_t kSpinLimit = 1u << 22;   // ~0.2 s of s_sleep polls: far beyond any real wait

// Wait until *cnt >= target (workgroup-scope acquire); false if the bound ran out.
__device__ __forceinline__ bool wait_count(const int* cnt, int target) {
  for (uint32_t it = 0; it < kSpinLimit; ++it) {
    if (__hip_atomic_load(cnt, __ATOMIC_ACQUIRE, __HIP_MEMORY_SCOPE_WORKGROUP) >= target) return true;
    __builtin_amdgcn_s_sleep(2);
  }
  return false;
}

__device__ __forceinline__ void post_count(int* cnt, int value) {
  if ((threadIdx.x & 63) == 0) __hip_atomic_store(cnt, value, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Pass 1's tile in registers (raw io units), fetched one tile ahead.
template <int DK, int DV, int IO>
struct OvRegs {
  using O = OvCfg<DK, DV>;
  static constexpr int VE = O::TT * O::COLS / 64;            // v values per lane
  Raw8<IO> k[O::KU1];
  float v[VE];
  float ab;
};

template <int DK, int DV, int IO>
__device__ __forceinline__ void ov_fetch(const PrefillArgs& A, OvRegs<DK, DV, IO>& R, int64_t t0, int n, int kh,
                                         int h, int col0) {
  using O = OvCfg<DK, DV>;
  constexpr int64_t ES = IO == IO_F32 ? 4 : 2;
  const int lane = threadIdx.x & 63;
  const char* kb = static_cast<const char*>(A.k) + (t0 * A.h_k + kh) * DK * ES;
  const char* vb = static_cast<const char*>(A.v) + ((t0 * A.h_v + h) * DV + col0) * ES;
#pragma unroll
  for (int x = 0; x < O::KU1; ++x) {
    const int u = lane + 64 * x, tt = u / (DK / 8), c8 = u % (DK / 8);
    if (tt < n) R.k[x] = load_raw8<IO>(kb, static_cast<uint32_t>(tt * A.h_k * DK + c8 * 8));
  }
#pragma unroll
  for (int x = 0; x < OvRegs<DK, DV, IO>::VE; ++x) {
    const int e = lane + 64 * x, tt = e / O::COLS, j = e % O::COLS;
    if (tt < n) R.v[x] = load1<IO>(vb, static_cast<uint32_t>(tt * A.h_v * DV + j));
  }
  const int tt = lane & (O::TT - 1);
  if (tt < n) {                          // lanes [0, TT) fetch a, lanes [TT, 2 TT) fetch b
    const int64_t e = (t0 + tt) * A.h_v + h;
    if (lane < O::TT)
      R.ab = A.a[e];
    else
      R.ab = A.b[e];
  }
}

template <int DK, int DV, int IO>
__device__ __forceinline__ void ov_commit(const OvRegs<DK, DV, IO>& R, OvLds<DK, DV, IO>& L) {
  using O = OvCfg<DK, DV>;
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int x = 0; x < O::KU1; ++x) {
    const int u = lane + 64 * x, tt = u / (DK / 8), c8 = u % (DK / 8);
    float y[8];
    widen8<IO>(R.k[x], y);
    store_kq8<O::G, kLeaf>(&L.k[tt][0], c8 * 8, y);
  }
#pragma unroll
  for (int x = 0; x < OvRegs<DK, DV, IO>::VE; ++x) {
    const int e = lane + 64 * x;
    L.v[e / O::COLS][e % O::COLS] = R.v[x];
  }
  if (lane < O::TT)
    L.ab[lane].x = R.ab;
  else
    L.ab[lane - O::TT].y = R.ab;
}

template <int DK, int DV, int IO>
__global__ void __launch_bounds__(192) overlap_kernel(PrefillArgs A) {
  using O = OvCfg<DK, DV>;
  constexpr int G = O::G, COLS = O::COLS, TT = O::TT, TH = O::TH;
  __shared__ OvLds<DK, DV, IO> L;
  __shared__ int64_t red[4];
  const int ratio = A.h_v / A.h_k;
  const GroupSlot gs = xcd_group(blockIdx.x, ratio * O::NCG);
  if (gs.group >= static_cast<int64_t>(A.num_seqs) * A.h_k) return;   // uniform across the block
  const int i = static_cast<int>(gs.group / A.h_k), kh = static_cast<int>(gs.group % A.h_k);
  const int h = kh * ratio + gs.member / O::NCG, col0 = (gs.member % O::NCG) * COLS;
  const SeqMeta m = seq_meta(A, i);
  const int64_t row0 = plan_row_offset(A, i, red);
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63, lc = lane / G, g = lane % G;
  const bool act = lc < COLS;                                  // lanes past the columns idle
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t col_off = static_cast<int64_t>(col0 + (act ? lc : 0)) * DK + g * kLeaf;
  float* slot_state = A.state + (static_cast<int64_t>(m.slot < 0 ? 0 : m.slot) * A.h_v + h) * plane + col_off;
  if (m.slot < 0) return;                                      // uniform across the block
  if (m.len == 0) {                                            // nothing to run; from zero: zero slot
    if (wave == 0 && act && !A.from_state) {
      float z[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
      store_f32x8(slot_state, z);
    }
    return;
  }
  if (threadIdx.x == 0) {
    L.handed = 0;
    L.released[0] = 0;
    L.released[1] = 0;
  }
  __syncthreads();                      // the last block-wide barrier: the waves now meet only in LDS
  const int64_t C = A.chunk;
  const int nchunks = static_cast<int>(m.nrows);
  const bool rows_on = A.chunk_states != nullptr;

  if (wave == 0) {
    // ---------------------------------------------------------------- pass 1
    __builtin_amdgcn_s_setprio(3);
    float s[kLeaf];
    if (A.from_state) {
      load_f32x8(slot_state, s);
    } else {
#pragma unroll
      for (int r = 0; r < kLeaf; ++r) s[r] = 0.0f;
    }
    if (A.round_boundary && m.p0 % C == 0) resync_round(s);   // the first token is a chunk start
    if (rows_on && act && row0 < A.rows_cap) store_f32x8(A.chunk_states + (row0 * A.h_v + h) * plane + col_off, s);
    if (act) store_f32x8(&L.hs[0][lc][g * kLeaf], s);
    int nb = static_cast<int>(C - m.p0 % C);                   // tokens until the next chunk start
    float pc = 0.0f;                                           // c of the previous token, not yet in LDS
    int pbuf = 0, pslot = -1;
    int c = 0;                                                 // chunk being run
    int64_t row = row0 + 1;
    OvRegs<DK, DV, IO> Rg = {};
    ov_fetch<DK, DV, IO>(A, Rg, m.tok0, m.len < TT ? m.len : TT, kh, h, col0);
    for (int t0 = 0; t0 < m.len; t0 += TT) {
      const int n = m.len - t0 < TT ? m.len - t0 : TT;
      ov_commit<DK, DV, IO>(Rg, L);
      __builtin_amdgcn_wave_barrier();
      if (t0 + TT < m.len) {
        const int n1 = m.len - t0 - TT < TT ? m.len - t0 - TT : TT;
        ov_fetch<DK, DV, IO>(A, Rg, m.tok0 + t0 + TT, n1, kh, h, col0);
      }
      for (int tt = 0; tt < n; ++tt) {
        const int t = t0 + tt;
        float kr[kLeaf];
        lds_read_kq<G, kLeaf>(&L.k[tt][0], g, kr);
        const float2 ab = L.ab[tt];
        // the previous token's c goes to LDS first, so the lane-masked write does not split this
        // token's arithmetic
        if (pslot >= 0 && g == 0 && act) L.hc[pbuf][pslot][lc] = pc;
        float u, w;
        cpr_update<1, G>(s, kr, act ? L.v[tt][lc] : 0.0f, ab.x, ab.y, u, w, pc);
        pbuf = c % O::NB;
        pslot = static_cast<int>(C) - nb;                      // the token's position within the chunk
        const bool last = t + 1 == m.len;
        if (--nb == 0 || last) {                               // chunk c is complete
          if (g == 0 && act) L.hc[pbuf][pslot][lc] = pc;
          pslot = -1;
          if (nb == 0) {
            nb = static_cast<int>(C);
            if (!last) {
              if (A.round_boundary) resync_round(s);           // a chunk start with a token to follow
              if (rows_on && act && row < row0 + m.nrows && row < A.rows_cap)
                store_f32x8(A.chunk_states + (row * A.h_v + h) * plane + col_off, s);
            }
            ++row;
          }
          if (!last) {
            // chunk c + 1 goes to the buffer chunk c - 2 used: wait until its pass-2 wave (the
            // chunk's parity) is done with it, i.e. has released (c - 2) / 2 + 1 chunks
            if (c >= 2) wait_count(&L.released[c & 1], (c - 2) / 2 + 1);
            if (act) store_f32x8(&L.hs[(c + 1) % O::NB][lc][g * kLeaf], s);
          }
          post_count(&L.handed, c + 1);
          ++c;
        }
      }
      __builtin_amdgcn_wave_barrier();                         // the tile's reads come before its refill
    }
    if (act) store_f32x8(slot_state, s);
  } else {
    // ---------------------------------------------------------------- pass 2
    // Wave 1 + w takes chunks w, w + 2, ...  Its tiles' inputs (k, q, a) do not depend on pass 1,
    // so the next tile -- also the first of its next chunk -- is fetched while one runs; only the
    // chunk hand-offs wait on pass 1.
    const int w = wave - 1;
    const int64_t p0 = m.p0;
    unsigned short* o16 = static_cast<unsigned short*>(A.o);
    float* o32 = static_cast<float*>(A.o);
    auto chunk_span = [&](int c, int* tb, int* te) {
      *tb = c == 0 ? 0 : static_cast<int>((p0 / C + c) * C - p0);
      const int64_t next = (p0 / C + c + 1) * C - p0;
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
          store_kq8<G, kLeaf>(&L.hk[w][u / (DK / 8)][0], (u % (DK / 8)) * 8, y);
          widen8<IO>(rq[x], y);
          store_kq8<G, kLeaf>(&L.hq[w][u / (DK / 8)][0], (u % (DK / 8)) * 8, y);
        }
      }
      if (lane < TH) L.ha[w][lane] = ra;
    };
    int tb, te;
    if (w < nchunks) {
      chunk_span(w, &tb, &te);
      fetch(tb, te - tb < TH ? te - tb : TH);
    }
    for (int c = w; c < nchunks; c += 2) {
      if (!wait_count(&L.handed, c + 1)) break;
      const int off = c == 0 ? static_cast<int>(p0 % C) : 0;  // position of token tb in the chunk
      float s[kLeaf];
      load_f32x8(&L.hs[c % O::NB][act ? lc : 0][g * kLeaf], s);
      for (int h0 = tb; h0 < te; h0 += TH) {
        const int n = te - h0 < TH ? te - h0 : TH;
        commit();
        __builtin_amdgcn_wave_barrier();
        if (h0 + TH < te) {                                    // the chunk's next tile
          fetch(h0 + TH, te - h0 - TH < TH ? te - h0 - TH : TH);
        } else if (c + 2 < nchunks) {                          // the first tile of the next chunk
          int nb0, ne0;
          chunk_span(c + 2, &nb0, &ne0);
          fetch(nb0, ne0 - nb0 < TH ? ne0 - nb0 : TH);
        }
        for (int tt = 0; tt < n; ++tt) {
          const int t = h0 + tt;
          float kr[kLeaf], qr[kLeaf];
          lds_read_kq<G, kLeaf>(&L.hk[w][tt][0], g, kr);
          lds_read_kq<G, kLeaf>(&L.hq[w][tt][0], g, qr);
          const float cv = act ? L.hc[c % O::NB][t - tb + off][lc] : 0.0f;
          const float o = cpr_step_given_c<1, G>(s, kr, qr, L.ha[w][tt], cv);
          if (g == 0 && act) L.ho[w][t - tb][lc] = o;
        }
        __builtin_amdgcn_wave_barrier();                       // the tile's reads come before its refill
      }
      post_count(&L.released[w], c / 2 + 1);                   // hs and hc of chunk c are free again
      __builtin_amdgcn_wave_barrier();
      for (int r = lane; r < te - tb; r += 64) {               // the chunk's outputs, a token per lane
        const int64_t oe = (static_cast<int64_t>(m.tok0 + tb + r) * A.h_v + h) * DV + col0;
#pragma unroll
        for (int j = 0; j < COLS; ++j) {
          if constexpr (IO == IO_F32)
            o32[oe + j] = L.ho[w][r][j];
          else
            o16[oe + j] = f32_to_bf16_rne(L.ho[w][r][j]);
        }
      }
      __builtin_amdgcn_wave_barrier();
      if (c + 2 < nchunks) chunk_span(c + 2, &tb, &te);
    }
  }
}

template <int DK, int DV, int IO>
static hipError_t launch_overlap_t(const PrefillArgs& A, hipStream_t stream) {
  using O = OvCfg<DK, DV>;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.num_seqs > 0) {
    const int64_t grid = xcd_grid(static_cast<int64_t>(A.num_seqs) * A.h_k, A.h_v / A.h_k * O::NCG);
    if (grid > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL((overlap_kernel<DK, DV, IO>), dim3(static_cast<unsigned>(grid)), dim3(192), 0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  return launch_prefill_finish(A, stream);
}

int overlap_max_chunk() { return OvCfg<128, 128>::CMAX; }

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
