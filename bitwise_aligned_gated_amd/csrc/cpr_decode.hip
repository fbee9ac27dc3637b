// cpr_decode.hip -- CPR decode: one token per slot with the shared pinned step, and the
// chunk-cadence resynchronisation ("For decode, the recurrent form runs but resynchronizes the
// hidden state every chunk-size tokens", section "Solving the linear-attention headache" of the
// IsoExec articles).
//
// A slot's state is read from HBM, advanced by one token in registers and written back; the
// kernel is bound by those 2 x d_k x d_v x 4 bytes per (slot, value head).  Work mapping is the
// prefill one (G = d_k/8 lanes per column, one 8-row leaf per lane), so a wave reads and writes
// 64/G whole columns = contiguous 512-byte runs at d_k = 128.
//
// Resynchronisation: a slot whose position is a multiple of C holds a chunk-start state.  The
// boundary dtype is fp32, so re-basing it on the boundary state is exact and leaves the values
// as they are; the state is committed to the pool's boundary record when the pool has one.
#include <hip/hip_runtime.h>

#include "cpr_common.hpp"
#include "cpr_launch.hpp"

namespace cpr {

template <int DK, int DV>
struct DecodeCfg {
  static constexpr int G = DK / kLeaf;
  static constexpr int WG_COLS = (256 / G < DV) ? 256 / G : DV;
  static constexpr int THREADS = WG_COLS * G;
};

template <int DK, int DV, int IO>
__global__ void __launch_bounds__((DecodeCfg<DK, DV>::THREADS)) decode_step_kernel(DecodeArgs A) {
  using Cfg = DecodeCfg<DK, DV>;
  constexpr int G = Cfg::G;
  const int e = blockIdx.x, h = blockIdx.y, cg = blockIdx.z;
  const int32_t slot = A.slot_ids[e];
  if (slot < 0 || slot >= A.num_slots) return;
  const int64_t p = A.pos[slot];
  const int tid = threadIdx.x, lc = tid / G, g = tid % G;
  const int col = cg * Cfg::WG_COLS + lc;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t soff = (static_cast<int64_t>(slot) * A.h_v + h) * plane + static_cast<int64_t>(col) * DK + g * 8;
  const int kh = h / (A.h_v / A.h_k);
  const int64_t kq = (static_cast<int64_t>(e) * A.h_k + kh) * DK + g * 8;

  float s[8], kr[8], qr[8];
  load_f32x8(A.state + soff, s);
  widen8<IO>(load_raw8<IO>(A.k, kq), kr);
  widen8<IO>(load_raw8<IO>(A.q, kq), qr);
  const int64_t vo = (static_cast<int64_t>(e) * A.h_v + h) * DV + col;
  const float v = load1<IO>(A.v, vo);
  const float a = A.a[static_cast<int64_t>(e) * A.h_v + h];
  const float b = A.b[static_cast<int64_t>(e) * A.h_v + h];

  if (A.boundary != nullptr && p >= 0 && p % A.chunk == 0) {
    store_f32x8(A.boundary + soff, s);
    if (h == 0 && cg == 0 && tid == 0) A.boundary_pos[slot] = p;
  }
  const float o = cpr_step<1, G, true>(s, kr, qr, v, a, b);
  store_f32x8(A.state + soff, s);
  if (g == 0) store1<IO>(A.o, vo, o);
}

__global__ void decode_advance_kernel(DecodeArgs A) {
  const int e = blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= A.batch) return;
  const int32_t slot = A.slot_ids[e];
  if (slot < 0 || slot >= A.num_slots) return;
  A.pos[slot] += 1;
}

template <int DK, int DV>
__global__ void __launch_bounds__((DecodeCfg<DK, DV>::THREADS)) resync_kernel(DecodeArgs A) {
  using Cfg = DecodeCfg<DK, DV>;
  const int e = blockIdx.x, h = blockIdx.y, cg = blockIdx.z;
  const int32_t slot = A.slot_ids[e];
  if (slot < 0 || slot >= A.num_slots || A.boundary == nullptr) return;
  const int64_t p = A.pos[slot];
  if (p < 0 || p % A.chunk != 0) return;
  const int tid = threadIdx.x, lc = tid / Cfg::G, g = tid % Cfg::G;
  const int64_t plane = static_cast<int64_t>(DV) * DK;
  const int64_t soff = (static_cast<int64_t>(slot) * A.h_v + h) * plane +
                       static_cast<int64_t>(cg * Cfg::WG_COLS + lc) * DK + g * 8;
  float s[8];
  load_f32x8(A.state + soff, s);
  store_f32x8(A.boundary + soff, s);
  if (h == 0 && cg == 0 && tid == 0) A.boundary_pos[slot] = p;
}

template <int DK, int DV, int IO>
static hipError_t launch_decode_t(const DecodeArgs& A, hipStream_t stream) {
  using Cfg = DecodeCfg<DK, DV>;
  hipError_t e = record_event(A.events, 0, stream);
  if (e != hipSuccess) return e;
  if (A.batch > 0) {
    hipLaunchKernelGGL((decode_step_kernel<DK, DV, IO>), dim3(A.batch, A.h_v, DV / Cfg::WG_COLS), dim3(Cfg::THREADS),
                       0, stream, A);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  if ((e = record_event(A.events, 1, stream)) != hipSuccess) return e;
  if (A.batch > 0) {
    hipLaunchKernelGGL(decode_advance_kernel, dim3((A.batch + 255) / 256), dim3(256), 0, stream, A);
    e = hipGetLastError();
  }
  return e;
}

template <int DK, int DV>
static hipError_t launch_resync_t(const DecodeArgs& A, hipStream_t stream) {
  using Cfg = DecodeCfg<DK, DV>;
  if (A.batch == 0 || A.boundary == nullptr) return hipSuccess;
  hipLaunchKernelGGL((resync_kernel<DK, DV>), dim3(A.batch, A.h_v, DV / Cfg::WG_COLS), dim3(Cfg::THREADS), 0, stream,
                     A);
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

hipError_t launch_resync(int dk, int dv, const DecodeArgs& A, hipStream_t stream) {
#define CPR_CASE(D) \
  if (dk == D && dv == D) return launch_resync_t<D, D>(A, stream);
  CPR_CASE(16) CPR_CASE(32) CPR_CASE(64) CPR_CASE(128)
#undef CPR_CASE
  return hipErrorInvalidValue;
}

}  // namespace cpr
