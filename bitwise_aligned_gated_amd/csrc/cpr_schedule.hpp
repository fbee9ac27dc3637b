// cpr_schedule.hpp -- constants of the pinned per-token schedule (host and device).
#pragma once

namespace cpr {

constexpr int kSchedule = 1;  // schedule version (see cpr_step.hpp)
constexpr int kLeaf = 8;      // rows per leaf of the pinned dot product

}  // namespace cpr
