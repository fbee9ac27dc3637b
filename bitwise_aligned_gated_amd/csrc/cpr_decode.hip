// cpr_decode.hip -- CPR decode: one token per slot with the shared pinned step, and the
// once-per-chunk resynchronisation (section "Solving the linear-attention headache" of the
// IsoExec articles: decode advances the state a token at a time and re-bases it at every chunk
// start so that its rounding agrees with prefill and training).
//
// A slot's state is read from HBM, advanced by one token in registers and written back; the
// kernel is bound by those 2 x d_k x d_v x 4 bytes per (slot, value head).  Work mapping: G =
// d_k/8 lanes per column with one 8-row leaf each (the boundary pass's mapping).
//
// Workgroups are small (one column per lane: 8 KiB of state at d = 128) and numbered in state
// order, so the workgroups in flight together stream through one compact window of the pool.
// The slot's position is needed only for chunk-start work (bf16 boundaries, a boundary record):
//  - without such work no workgroup reads it, and one workgroup per slot advances it;
//  - with it every workgroup reads it, and a second, one-thread-per-entry kernel advances it
//    after the step, so no workgroup of the step ever sees a moved position.
//
// Resynchronisation: a slot whose position is a multiple of C holds a chunk-start state.  With
// the fp32 boundary dtype re-basing it on the boundary state is exact and leaves the values as
// they are; with bf16 the state is rounded.  The state is then committed to the pool's boundary
// record when the pool has one.
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

#ifndef CPR_DECODE_NC
#define CPR_DECODE_NC 1         // step kernel, columns per lane
#endif
#ifndef CPR_RESYNC_NC
#define CPR_RESYNC_NC 8         // explicit resync, columns per lane (one workgroup per (slot, value head) at d = 128)
#endif
#ifndef CPR_DECODE_NT
#define CPR_DECODE_NT 0       // streaming (non-temporal) state access: bit 0 loads, bit 1 stores
#endif

__device__ __forceinline__ void state_load(const float* p, float (&x)[8]) {
  if constexpr ((CPR_DECODE_NT & 1) != 0) load_f32x8_nt(p, x); else load_f32x8(p, x);
}
__device__ __forceinline__ void state_store(float* p, const float (&x)[8]) {
  if constexpr ((CPR_DECODE_NT & 2) != 0) store_f32x8_nt(p, x); else store_f32x8(p, x);
}

template <int DK, int DV, int NC_MAX>
struct DecodeCfg {
  static constexpr int G = DK / kLeaf;                         // lanes per column, one leaf each
  static constexpr int SLOTS = (256 / G < DV) ? 256 / G : DV;  // column slots per workgroup
  static constexpr int NC_ALL = DV / SLOTS;
  static constexpr int NC = NC_ALL < NC_MAX ? NC_ALL : NC_MAX;  // columns per lane
  static constexpr int WG_COLS = SLOTS * NC;                   // columns per workgroup
  static constexpr int THREADS = SLOTS * G;
  static_assert(DV % SLOTS == 0 && NC_ALL % NC == 0 && WG_COLS % 8 == 0, "shape");
};

// One work item per (entry, value head, column group): every lane first issues the streaming
// loads of all its NC columns (NC x 32 bytes of state), then runs the step on each column; lane
// (slot, g) owns columns col0 + slot + SLOTS * c, so each load instruction of a wave covers whole
// 512-byte columns.
template <int DK, int DV>
using StepCfg = DecodeCfg<DK, DV, CPR_DECODE_NC>;

template <int DK, int DV, int IO>
__device__ __forceinline__ void decode_step_item(const DecodeArgs& A, int64_t vb) {
  using Cfg = StepCfg<DK, DV>;
  constexpr int G = Cfg::G, NC = Cfg::NC, SLOTS = Cfg::SLOTS, NCG = DV / Cfg::WG_COLS;
  __shared__ float o_lds[Cfg::WG_COLS];
  const int per_entry = A.h_v * NCG;
  // state order: column groups fastest, then value heads, then entries
  const int z = static_cast<int>(vb % NCG), h = static_cast<int>(vb / NCG % A.h_v);
  const int e = static_cast<int>(vb / per_entry);
  const int col0 = z * Cfg::WG_COLS;
  const int32_t slot = A.slot_ids[e];
  if (slot < 0 || slot >= A.num_slots) return;                  // uniform across the block
  if (A.skip_slot != nullptr && A.skip_slot[slot] != 0) return; // uniform: a later launch steps it
  // With chunk-start work the position is read here and advanced by decode_advance_kernel after
  // this launch; without it the position is not read, and one workgroup advances it below.
  const bool chunk_work = A.boundary != nullptr || A.round_boundary != 0;
  const int64_t p = chunk_work ? A.pos[slot] : 0;
  const int tid = threadIdx.x, cs = tid / G, g = tid % G;
  const int64_t head = (static_cast<int64_t>(slot) * A.h_v + h) * DV * DK;
  const int kh = h / (A.h_v / A.h_k);
  const int64_t kq = (static_cast<int64_t>(e) * A.h_k + kh) * DK + g * kLeaf;
  const int64_t vo = (static_cast<int64_t>(e) * A.h_v + h) * DV + col0;
  const float* src = A.state + head + static_cast<int64_t>(col0) * DK + g * kLeaf;

  float s[NC][kLeaf];
#pragma unroll
  for (int c = 0; c < NC; ++c) state_load(src + static_cast<int64_t>(cs + SLOTS * c) * DK, s[c]);
  float kr[kLeaf], qr[kLeaf], v[NC];
  widen8<IO>(load_raw8<IO>(A.k, kq), kr);
  widen8<IO>(load_raw8<IO>(A.q, kq), qr);
#pragma unroll
  for (int c = 0; c < NC; ++c) v[c] = load1<IO>(A.v, vo + cs + SLOTS * c);
  const float a = A.a[static_cast<int64_t>(e) * A.h_v + h];
  const float b = A.b[static_cast<int64_t>(e) * A.h_v + h];

  const bool at_chunk_start = chunk_work && p % A.chunk == 0;
  if (A.round_boundary && at_chunk_start) {                      // resynchronise: re-base on bf16
#pragma unroll
    for (int c = 0; c < NC; ++c) resync_round(s[c]);
  }
  if (A.boundary != nullptr && at_chunk_start) {                 // commit the chunk-start state
#pragma unroll
    for (int c = 0; c < NC; ++c)
      state_store(A.boundary + head + static_cast<int64_t>(col0 + cs + SLOTS * c) * DK + g * kLeaf, s[c]);
    if (h == 0 && z == 0 && tid == 0) A.boundary_pos[slot] = p;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c) {
    const float o = cpr_step<1, G, true>(s[c], kr, qr, v[c], a, b);
    if (g == 0) o_lds[cs + SLOTS * c] = o;
  }
#pragma unroll
  for (int c = 0; c < NC; ++c)
    state_store(A.state + head + static_cast<int64_t>(col0 + cs + SLOTS * c) * DK + g * kLeaf, s[c]);
  __syncthreads();
  if (tid < Cfg::WG_COLS / 8) {
    float x[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = o_lds[tid * 8 + i];
    store8<IO>(A.o, vo + tid * 8, x);
  }
  // Slot ids are distinct and, without chunk-start work, no other work item touches pos[slot].
  if (!chunk_work && h == 0 && z == 0 && tid == 0) A.pos[slot] += 1;
}

template <int DK, int DV, int IO>
__global__ void __launch_bounds__((StepCfg<DK, DV>::THREADS)) decode_step_kernel(DecodeArgs A) {
  decode_step_item<DK, DV, IO>(A, blockIdx.x);
}

// The same items under a capped grid: each workgroup takes items b, b + gridDim.x, ...
template <int DK, int DV, int IO>
__global__ void __launch_bounds__((StepCfg<DK, DV>::THREADS)) decode_step_strided_kernel(DecodeArgs A) {
  for (int64_t vb = blockIdx.x; vb < A.grid_items; vb += gridDim.x) {
    if (vb != blockIdx.x) __syncthreads();                 // the previous item is done with LDS
    decode_step_item<DK, DV, IO>(A, vb);
  }
}

// The step over listed batch entries only: the workgroups take (listed entry, value head, column
// group) items in turn.  entries[0 .. *count) are batch indices; the count is known on the device.
template <int DK, int DV, int IO>
__global__ void __launch_bounds__((StepCfg<DK, DV>::THREADS)) decode_step_list_kernel(DecodeArgs A,
                                                                                     const int32_t* entries,
                                                                                     const int32_t* count) {
  constexpr int NCG = DV / StepCfg<DK, DV>::WG_COLS;
  const int64_t per = static_cast<int64_t>(A.h_v) * NCG;
  const int32_t n = *count < A.batch ? *count : A.batch;
  const int64_t items = static_cast<int64_t>(n > 0 ? n : 0) * per;
  for (int64_t it = blockIdx.x; it < items; it += gridDim.x) {
    if (it != blockIdx.x) __syncthreads();                 // the previous item is done with LDS
    const int32_t en = entries[it / per];
    if (en < 0 || en >= A.batch) continue;                 // uniform across the block
    decode_step_item<DK, DV, IO>(A, static_cast<int64_t>(en) * per + it % per);
  }
}

// pos[slot] += 1 for every listed slot, after a step with chunk-start work (entries taken in turn
// when the grid is capped).
__global__ void __launch_bounds__(256) decode_advance_kernel(DecodeArgs A) {
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < A.batch;
       e += static_cast<int64_t>(gridDim.x) * 256) {
    const int32_t slot = A.slot_ids[e];
    if (slot >= 0 && slot < A.num_slots) A.pos[slot] += 1;
  }
}

template <int DK, int DV>
__global__ void __launch_bounds__((DecodeCfg<DK, DV, CPR_RESYNC_NC>::THREADS)) resync_kernel(DecodeArgs A) {
  using Cfg = DecodeCfg<DK, DV, CPR_RESYNC_NC>;
  const int e = blockIdx.x, h = blockIdx.y;
  const int32_t slot = A.slot_ids[e];
  if (slot < 0 || slot >= A.num_slots) return;
  const int64_t p = A.pos[slot];
  if (p < 0 || p % A.chunk != 0) return;
  if (A.boundary == nullptr && !A.round_boundary) return;
  const int tid = threadIdx.x, cs = tid / Cfg::G, g = tid % Cfg::G;
  const int col0 = blockIdx.z * Cfg::WG_COLS;
  const int64_t head = (static_cast<int64_t>(slot) * A.h_v + h) * DV * DK;
#pragma unroll
  for (int c = 0; c < Cfg::NC; ++c) {
    const int64_t off = head + static_cast<int64_t>(col0 + cs + Cfg::SLOTS * c) * DK + g * kLeaf;
    float s[kLeaf];
    load_f32x8(A.state + off, s);
    if (A.round_boundary) {
      resync_round(s);
      store_f32x8(A.state + off, s);
    }
    if (A.boundary != nullptr) store_f32x8(A.boundary + off, s);
  }
  if (A.boundary != nullptr && h == 0 && blockIdx.z == 0 && tid == 0) A.boundary_pos[slot] = p;
}

template <int DK, int DV, int IO>
static hipError_t launch_decode_t(const DecodeArgs& A, hipStream_t stream) {
  using Cfg = StepCfg<DK, DV>;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.batch > 0) {
    const int64_t items = static_cast<int64_t>(A.batch) * A.h_v * (DV / Cfg::WG_COLS);
    e = launch_items(decode_step_kernel<DK, DV, IO>, decode_step_strided_kernel<DK, DV, IO>, items, Cfg::THREADS,
                     stream, A);
    if (e != hipSuccess) return e;
    if ((A.boundary != nullptr || A.round_boundary != 0) && !A.skip_advance) {
      int64_t wgs = (static_cast<int64_t>(A.batch) + 255) / 256;
      if (A.max_wgs > 0 && A.max_wgs < wgs) wgs = A.max_wgs;
      hipLaunchKernelGGL(decode_advance_kernel, dim3(static_cast<unsigned>(wgs)), dim3(256), 0, stream, A);
      e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
  }
  return record_event(A.events, 1, stream);
}

template <int DK, int DV>
static hipError_t launch_resync_t(const DecodeArgs& A, hipStream_t stream) {
  using Cfg = DecodeCfg<DK, DV, CPR_RESYNC_NC>;
  if (A.batch == 0 || (A.boundary == nullptr && !A.round_boundary)) return hipSuccess;
  hipLaunchKernelGGL((resync_kernel<DK, DV>), dim3(A.batch, A.h_v, DV / Cfg::WG_COLS), dim3(Cfg::THREADS), 0, stream, A);
  return hipGetLastError();
}

hipError_t launch_decode(int dk, int dv, int io, const DecodeArgs& A, hipStream_t stream) {
#define CPR_CASE(D, IOV) \
  if (dk == D && dv == D && io == IOV) return launch_decode_t<D, D, IOV>(A, stream);
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_decode_list(int dk, int dv, int io, const DecodeArgs& A, const int32_t* entries,
                              const int32_t* count, unsigned grid, hipStream_t stream) {
#define CPR_CASE(D, IOV)                                                                                         \
  if (dk == D && dv == D && io == IOV) {                                                                         \
    hipLaunchKernelGGL((decode_step_list_kernel<D, D, IOV>), dim3(grid), dim3(StepCfg<D, D>::THREADS), 0, stream, \
                       A, entries, count);                                                                       \
    return hipGetLastError();                                                                                    \
  }
  CPR_CASE(16, IO_F32) CPR_CASE(16, IO_BF16)
  CPR_CASE(32, IO_F32) CPR_CASE(32, IO_BF16)
  CPR_CASE(64, IO_F32) CPR_CASE(64, IO_BF16)
  CPR_CASE(128, IO_F32) CPR_CASE(128, IO_BF16)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

hipError_t launch_resync(int dk, int dv, const DecodeArgs& A, hipStream_t stream) {
#define CPR_CASE(D) \
  if (dk == D && dv == D) return launch_resync_t<D, D>(A, stream);
  CPR_CASE(16) CPR_CASE(32) CPR_CASE(64) CPR_CASE(128)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

}  // namespace cpr
