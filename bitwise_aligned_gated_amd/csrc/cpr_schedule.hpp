// cpr_schedule.hpp -- constants of the pinned per-token schedule (host and device).
#pragma once

namespace cpr {

constexpr int kSchedule = 1;  // schedule version (see cpr_step.hpp)
constexpr int kLeaf = 8;      // rows per leaf of the pinned dot product
// Version of the kernels' work mapping (lanes per column, columns per lane, tile sizes, workgroup
// order, which kernels a call launches).  The schedule fixes leaves and tree, so the mapping never
// moves a bit; it enters only the deployment digest.  Raised with every change of a kernel's work
// mapping (4: one-column-per-lane decode in state order with a separate position update, the
// overlapped prefill, and the chunk-64 backward under fp32 boundaries; 5: the chunk-form output
// kernel with whole column tiles per wave, and the R2 decode step's four launches; 6: the R2 step's
// listed slots resynchronised and stepped on a second stream, 512 list-driven workgroups).
constexpr int kMappingVersion = 6;

}  // namespace cpr
