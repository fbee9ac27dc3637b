// cpr_launch.hpp -- internal launchers between the C ABI (cpr_host.cpp) and the kernels.
#pragma once

#include <hip/hip_runtime.h>

namespace cpr {

struct PrefillArgs;
struct DecodeArgs;
struct BackwardArgs;

// Each returns hipErrorInvalidValue for a (dk, dv, io) combination that is not compiled in.
hipError_t launch_prefill(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream);
hipError_t launch_prefill_fused(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream);
// Pass 1 and the chunk outputs in one workgroup per column group (chunks up to overlap_max_chunk()).
hipError_t launch_prefill_overlap(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream);
int overlap_max_chunk();
// The current device's status word of the overlapped kernel's bounded waits (device address).
hipError_t wait_status_word(uint32_t** out);
// The library-owned scratch of gdn_prefill_static on the current device (its device address, taken
// once per device), kStaticScratchBytes long and 256-byte aligned.
constexpr size_t kStaticScratchBytes = size_t(256) << 20;
hipError_t static_scratch(void** out);
// Whether every workgroup of the overlapped kernel is resident at once (one per CU).
bool overlap_fits(int dk, int dv, const PrefillArgs& A);
hipError_t launch_decode(int dk, int dv, int io, const DecodeArgs& A, hipStream_t stream);
// The step over the batch entries entries[0 .. *count) only, on `grid` workgroups taking them in turn.
hipError_t launch_decode_list(int dk, int dv, int io, const DecodeArgs& A, const int32_t* entries,
                              const int32_t* count, unsigned grid, hipStream_t stream);
hipError_t launch_resync(int dk, int dv, const DecodeArgs& A, hipStream_t stream);
hipError_t launch_backward(int dk, int dv, int io, const BackwardArgs& A, hipStream_t stream);
// Parts of <G, S_0> the adjoint pass stores per chunk start and value head (head dim d).
int adjoint_parts(int d);
// The backward's per-token and chunk gradient kernels alone (events 2 and 3), given dc, the
// adjoint rows, the <G, S> parts, c and w.
hipError_t launch_gradient_passes(int d, int io, const BackwardArgs& A, hipStream_t stream);
// The chunk-form backward's own passes (events 0 and 1): w and the intra-chunk part of dC, then
// the reverse chunk chain (G at every chunk boundary, dc, the <G, S> parts), from what the
// chunk-form trainer forward kept.  Head dims 32, 64 and 128, bf16 io.
hipError_t launch_backward_chunked(int d, const BackwardArgs& A, hipStream_t stream);
int backward_chunked_parts(int d);
int64_t chunked_bwd_floats(int d);
// The position update that ends every prefill, and the CPR output pass (with that update) alone,
// started from chunk states already stored.
hipError_t launch_prefill_finish(const PrefillArgs& A, hipStream_t stream);
hipError_t launch_output_pass(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream);
// The CPR output pass alone, without the position update.
hipError_t launch_output_pass_only(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream);
// Pass 1 alone (chunk-start states up to each sequence's last chunk start, no c, no finish).
hipError_t launch_boundary_pass(int dk, int dv, int io, const PrefillArgs& A, hipStream_t stream);
// For a backward at a chunk above the chunk-gradient tile: slot_ids[j] = the first row of sequence
// j in a stash at chunk A.chunk, and a zero position at each such row.
hipError_t launch_rechunk_setup(const BackwardArgs& A, int32_t* slot_ids, int64_t* pos, hipStream_t stream);
// Chunkwise evaluation on matrix cores: mode 0 native outputs, mode 1 chunk-form boundary states
// followed by the CPR output pass.  ws holds chunked_workspace_floats(d) floats per chunk row and
// value head.
hipError_t launch_prefill_chunked(int dk, int dv, int io, const PrefillArgs& A, void* ws, int mode,
                                  hipStream_t stream);
int64_t chunked_workspace_floats(int d);
// R2 resynchronisation in decode: ring and workspace sizes, and the step (the chunk form over the
// ring for slots at a chunk start, then the pinned step, then the ring append).
int64_t r2_ring_bytes(int h_k, int h_v, int d, int chunk, int num_slots);
int64_t r2_workspace_bytes(int h_v, int d, int num_slots);
// The chunk form and the listed slots' step run on the second stream `side` (forked from `stream`
// and joined back before the ring append by the two events), beside the other slots' step; side
// NULL: all in sequence on `stream`.
hipError_t launch_decode_r2(int d, const DecodeArgs& A, void* ring, void* work, hipStream_t stream,
                            hipStream_t side, hipEvent_t fork, hipEvent_t join);

}  // namespace cpr
