// cpr_common.hpp -- device helpers shared by the CPR kernels: typed 8-element loads, the varlen
// chunk plan computed from cu_seqlens on the device, and the kernel argument blocks.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cpr_args.hpp"
#include "cpr_step.hpp"

namespace cpr {

enum : int { IO_F32 = 0, IO_BF16 = 1 };

// ---- raw 8-element units (what one lane moves from HBM for 8 consecutive elements) ----------
template <int IO>
struct Raw8;
template <>
struct Raw8<IO_F32> {
  uint4 w[2];
};
template <>
struct Raw8<IO_BF16> {
  uint4 w[1];
};

template <int IO>
__device__ __forceinline__ Raw8<IO> load_raw8(const void* base, int64_t elem) {
  Raw8<IO> r;
  if constexpr (IO == IO_F32) {
    const uint4* p = reinterpret_cast<const uint4*>(static_cast<const float*>(base) + elem);
    r.w[0] = p[0];
    r.w[1] = p[1];
  } else {
    r.w[0] = *reinterpret_cast<const uint4*>(static_cast<const unsigned short*>(base) + elem);
  }
  return r;
}

template <int IO>
__device__ __forceinline__ Raw8<IO> zero_raw8() {
  Raw8<IO> r;
#pragma unroll
  for (int i = 0; i < (IO == IO_F32 ? 2 : 1); ++i) r.w[i] = make_uint4(0, 0, 0, 0);
  return r;
}

// Widen a raw unit to 8 floats (exact for both dtypes).
template <int IO>
__device__ __forceinline__ void widen8(const Raw8<IO>& r, float (&x)[8]) {
  if constexpr (IO == IO_F32) {
    const unsigned int u[8] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w,
                               r.w[1].x, r.w[1].y, r.w[1].z, r.w[1].w};
#pragma unroll
    for (int i = 0; i < 8; ++i) x[i] = __builtin_bit_cast(float, u[i]);
  } else {
    const unsigned int u[4] = {r.w[0].x, r.w[0].y, r.w[0].z, r.w[0].w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      x[2 * i] = __builtin_bit_cast(float, u[i] << 16);
      x[2 * i + 1] = __builtin_bit_cast(float, u[i] & 0xFFFF0000u);
    }
  }
}

// Store 8 floats to an io-typed array (bf16: round to nearest even).
template <int IO>
__device__ __forceinline__ void store8(void* base, int64_t elem, const float (&x)[8]) {
  if constexpr (IO == IO_F32) {
    uint4* p = reinterpret_cast<uint4*>(static_cast<float*>(base) + elem);
    p[0] = make_uint4(__builtin_bit_cast(unsigned int, x[0]), __builtin_bit_cast(unsigned int, x[1]),
                      __builtin_bit_cast(unsigned int, x[2]), __builtin_bit_cast(unsigned int, x[3]));
    p[1] = make_uint4(__builtin_bit_cast(unsigned int, x[4]), __builtin_bit_cast(unsigned int, x[5]),
                      __builtin_bit_cast(unsigned int, x[6]), __builtin_bit_cast(unsigned int, x[7]));
  } else {
    unsigned int u[4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      u[i] = static_cast<unsigned int>(f32_to_bf16_rne(x[2 * i])) |
             (static_cast<unsigned int>(f32_to_bf16_rne(x[2 * i + 1])) << 16);
    *reinterpret_cast<uint4*>(static_cast<unsigned short*>(base) + elem) = make_uint4(u[0], u[1], u[2], u[3]);
  }
}

template <int IO>
__device__ __forceinline__ void store1(void* base, int64_t elem, float x) {
  if constexpr (IO == IO_F32)
    static_cast<float*>(base)[elem] = x;
  else
    static_cast<unsigned short*>(base)[elem] = f32_to_bf16_rne(x);
}

// Store two consecutive outputs with one 4-byte (bf16) or 8-byte (fp32) write.
template <int IO>
__device__ __forceinline__ void store2(void* base, int64_t elem, float x0, float x1) {
  if constexpr (IO == IO_F32) {
    *reinterpret_cast<float2*>(static_cast<float*>(base) + elem) = make_float2(x0, x1);
  } else {
    *reinterpret_cast<unsigned int*>(static_cast<unsigned short*>(base) + elem) =
        static_cast<unsigned int>(f32_to_bf16_rne(x0)) | (static_cast<unsigned int>(f32_to_bf16_rne(x1)) << 16);
  }
}

template <int IO>
__device__ __forceinline__ float load1(const void* base, int64_t elem) {
  if constexpr (IO == IO_F32)
    return static_cast<const float*>(base)[elem];
  else
    return bf16_to_f32(static_cast<const unsigned short*>(base)[elem]);
}

__device__ __forceinline__ void load_f32x8(const float* p, float (&x)[8]) {
  const float4 a = reinterpret_cast<const float4*>(p)[0];
  const float4 b = reinterpret_cast<const float4*>(p)[1];
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

// Streaming (non-temporal) variants for data touched once per launch, such as a decode step's
// state: they keep the stream from displacing reusable lines in L2.
typedef float f32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ void load_f32x8_nt(const float* p, float (&x)[8]) {
  const f32x4_t a = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p));
  const f32x4_t b = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p) + 1);
  x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
  x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
}

__device__ __forceinline__ void store_f32x8_nt(float* p, const float (&x)[8]) {
  const f32x4_t a = {x[0], x[1], x[2], x[3]};
  const f32x4_t b = {x[4], x[5], x[6], x[7]};
  __builtin_nontemporal_store(a, reinterpret_cast<f32x4_t*>(p));
  __builtin_nontemporal_store(b, reinterpret_cast<f32x4_t*>(p) + 1);
}

__device__ __forceinline__ void store_f32x8(float* p, const float (&x)[8]) {
  reinterpret_cast<float4*>(p)[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(p)[1] = make_float4(x[4], x[5], x[6], x[7]);
}

// ---- lane-interleaved k / q tile rows in LDS -------------------------------------------------
// A staged k (or q) row is kept lane-interleaved: lane g of a column reads its rows
// [g R, g R + R) as R/4 float4s, and float4 i of lane g sits at slot i G + g, so the G lanes'
// i-th reads cover G consecutive float4s (no LDS bank conflicts) instead of G strided ones.
template <int G, int R>
__device__ __forceinline__ int kq_slot(int row) {
  return ((row % R) / 4 * G + row / R) * 4 + row % 4;
}

// Rows [r0, r0 + 8) of a lane-interleaved tile row (r0 a multiple of 8; R a multiple of 8, so the
// eight rows belong to one lane and form two of its float4s).
template <int G, int R>
__device__ __forceinline__ void store_kq8(float* row, int r0, const float (&x)[8]) {
  reinterpret_cast<float4*>(row + kq_slot<G, R>(r0))[0] = make_float4(x[0], x[1], x[2], x[3]);
  reinterpret_cast<float4*>(row + kq_slot<G, R>(r0 + 4))[0] = make_float4(x[4], x[5], x[6], x[7]);
}

// Lane g's R rows of a lane-interleaved tile row.
template <int G, int R>
__device__ __forceinline__ void lds_read_kq(const float* row, int g, float (&x)[R]) {
#pragma unroll
  for (int i = 0; i < R / 4; ++i) {
    const float4 f = reinterpret_cast<const float4*>(row)[i * G + g];
    x[4 * i] = f.x; x[4 * i + 1] = f.y; x[4 * i + 2] = f.z; x[4 * i + 3] = f.w;
  }
}

// Record events[i] on the stream when the caller asked for timing events.
inline hipError_t record_event(void* const* events, int i, hipStream_t stream) {
  if (events == nullptr || events[i] == nullptr) return hipSuccess;
  return hipEventRecord(static_cast<hipEvent_t>(events[i]), stream);
}

// ---- XCD-aware workgroup order ---------------------------------------------------------------
// MI355X hands linear workgroup ids to its 8 XCDs round-robin, and each XCD has its own L2.
// Workgroups that read the same inputs (a key head's k and q, shared by its value heads and
// column groups) form a group; a group's members get ids with one residue mod 8, consecutive in
// that XCD's order, so the shared lines are fetched into one L2 once.  Launch
// xcd_grid(n_groups, group_size) workgroups; ids past the last group have no work.
constexpr int kXcds = 8;

inline int64_t xcd_grid(int64_t n_groups, int group_size) {
  return (n_groups + kXcds - 1) / kXcds * kXcds * group_size;
}

// Launch shape of a kernel with `items` work items: one workgroup each, or at most max_wgs
// workgroups that take items b, b + gridDim.x, ... in turn.  Every item's arithmetic is the same
// either way, so the shape moves no bit.
template <typename Args>
inline Args with_items(const Args& A, int64_t items) {
  Args B = A;
  B.grid_items = items;
  return B;
}
// Launch `items` work items: the natural kernel with one workgroup per item, or, when the caller
// capped the grid below that, the strided kernel with max_wgs workgroups.
template <typename Args>
inline hipError_t launch_items(void (*natural)(Args), void (*strided)(Args), int64_t items, unsigned threads,
                               hipStream_t stream, const Args& A) {
  if (items > 0x7FFFFFFF) return hipErrorInvalidConfiguration;
  if (A.max_wgs > 0 && A.max_wgs < items)
    hipLaunchKernelGGL(strided, dim3(static_cast<unsigned>(A.max_wgs)), dim3(threads), 0, stream, with_items(A, items));
  else
    hipLaunchKernelGGL(natural, dim3(static_cast<unsigned>(items)), dim3(threads), 0, stream, with_items(A, items));
  return hipGetLastError();
}

struct GroupSlot {
  int64_t group;
  int member;
};

__device__ __forceinline__ GroupSlot xcd_group(int64_t b, int group_size) {
  const int64_t x = b % kXcds, u = b / kXcds;
  GroupSlot r;
  r.group = (u / group_size) * kXcds + x;
  r.member = static_cast<int>(u % group_size);
  return r;
}

// ---- varlen plan ------------------------------------------------------------------------------
// Metadata of packed sequence j.  A sequence with malformed cu_seqlens entries, an out-of-range
// slot or a negative start position is treated as empty (no rows, no tokens) so no kernel ever
// indexes outside the buffers.
struct SeqMeta {
  int64_t tok0;   // first packed token
  int64_t p0;     // absolute position of that token
  int32_t len;    // tokens
  int32_t slot;
  int64_t nrows;  // boundary rows: states entering p0 and every chunk start inside the range
};

__device__ __forceinline__ SeqMeta seq_meta(const PrefillArgs& A, int j) {
  SeqMeta m;
  m.tok0 = 0; m.p0 = 0; m.len = 0; m.slot = -1; m.nrows = 0;
  const int32_t c0 = A.cu[j], c1 = A.cu[j + 1];
  if (c0 < 0 || c1 < c0 || static_cast<int64_t>(c1) > A.total_tokens) return m;
  const int32_t slot = A.slot_ids[j];
  if (slot < 0 || slot >= A.num_slots) return m;
  const int64_t p0 = A.from_state ? A.pos[slot] : 0;
  if (p0 < 0) return m;
  m.tok0 = c0;
  m.p0 = p0;
  m.len = c1 - c0;
  m.slot = slot;
  const int64_t C = A.chunk;
  m.nrows = m.len == 0 ? 0 : 1 + (p0 + m.len - 1) / C - p0 / C;
  return m;
}

// The same metadata for a gradient pass: every sequence started at position 0, no slots.
__device__ __forceinline__ SeqMeta seq_meta(const BackwardArgs& A, int j) {
  SeqMeta m;
  m.tok0 = 0; m.p0 = 0; m.len = 0; m.slot = 0; m.nrows = 0;
  const int32_t c0 = A.cu[j], c1 = A.cu[j + 1];
  if (c0 < 0 || c1 < c0 || static_cast<int64_t>(c1) > A.total_tokens) return m;
  m.tok0 = c0;
  m.len = c1 - c0;
  m.nrows = m.len == 0 ? 0 : 1 + (m.len - 1) / A.chunk;
  return m;
}

// Block-wide sum of one int64 per thread.  All threads must call; result valid in every thread.
// `red` is __shared__ scratch of at least (blockDim.x + 63) / 64 entries.
// Blocks narrower than a wave must have a power-of-two size so the butterfly stays on live lanes.
__device__ __forceinline__ int64_t block_sum_i64(int64_t x, int64_t* red) {
  const int width = blockDim.x < 64 ? static_cast<int>(blockDim.x) : 64;
  for (int off = width >> 1; off >= 1; off >>= 1) x += __shfl_xor(x, off, width);
  const int wave = threadIdx.x >> 6;
  const int nwaves = (blockDim.x + 63) >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[wave] = x;
  __syncthreads();
  int64_t s = 0;
  for (int w = 0; w < nwaves; ++w) s += red[w];
  return s;
}

// Block-wide exclusive prefix of one int64 per thread; *total receives the block's sum.
// `red` is __shared__ scratch of at least (blockDim.x + 63) / 64 entries.
__device__ __forceinline__ int64_t block_excl_scan_i64(int64_t x, int64_t* red, int64_t* total) {
  const int lane = threadIdx.x & 63;
  int64_t incl = x;
  for (int off = 1; off < 64; off <<= 1) {
    const int64_t y = __shfl_up(incl, off, 64);
    if (lane >= off) incl += y;
  }
  const int wave = threadIdx.x >> 6;
  const int nwaves = (blockDim.x + 63) >> 6;
  __syncthreads();
  // the last live lane of each wave publishes the wave total
  if (lane == 63 || threadIdx.x == blockDim.x - 1) red[wave] = incl;
  __syncthreads();
  int64_t before = 0, all = 0;
  for (int w = 0; w < nwaves; ++w) {
    if (w < wave) before += red[w];
    all += red[w];
  }
  *total = all;
  return before + incl - x;
}

// First boundary row of sequence i (sum of the rows of sequences 0 .. i-1).  Block-wide.
template <class Args>
__device__ inline int64_t plan_row_offset(const Args& A, int i, int64_t* red) {
  int64_t acc = 0;
  for (int base = 0; base < i; base += blockDim.x) {
    const int j = base + static_cast<int>(threadIdx.x);
    const int64_t n = j < i ? seq_meta(A, j).nrows : 0;
    acc += block_sum_i64(n, red);
  }
  return acc;
}

// Which (sequence, row within it) owns global boundary row w.  Block-wide; returns false when w
// is past the last row (the block has no work).  `red` needs (blockDim.x+63)/64 + 2 entries.
template <class Args>
__device__ inline bool plan_find_row(const Args& A, int64_t w, int* seq, int64_t* row_in_seq, int64_t* red) {
  int64_t* found = red + ((blockDim.x + 63) >> 6);   // [0]: sequence, [1]: row in it
  if (threadIdx.x == 0) found[0] = -1;
  int64_t offset = 0;
  for (int base = 0; base < A.num_seqs; base += blockDim.x) {
    const int j = base + static_cast<int>(threadIdx.x);
    const int64_t n = j < A.num_seqs ? seq_meta(A, j).nrows : 0;
    int64_t total;
    const int64_t start = offset + block_excl_scan_i64(n, red, &total);
    if (n > 0 && w >= start && w < start + n) {
      found[0] = j;
      found[1] = w - start;
    }
    __syncthreads();
    const int64_t f = found[0];
    if (f >= 0) {
      *seq = static_cast<int>(f);
      *row_in_seq = found[1];
      return true;
    }
    offset += total;
    if (offset > w) break;
  }
  return false;
}

}  // namespace cpr
