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
hipError_t launch_decode(int dk, int dv, int io, const DecodeArgs& A, hipStream_t stream);
hipError_t launch_resync(int dk, int dv, const DecodeArgs& A, hipStream_t stream);
hipError_t launch_backward(int dk, int dv, int io, const BackwardArgs& A, hipStream_t stream);

}  // namespace cpr
