// Host-only soundness check of a logical schedule, run before a step
// implementation's launches when the library is loaded with AR_DEBUG=1, and
// by the sanitized host tests.  Pure C++; the kernels do not include it.
#pragma once

#include <cstdint>
#include <vector>

#include "plan.hpp"

namespace ar {

// Why `steps`, the schedule of `coll` for (n, count, root), could not run one
// launch per step with the counters telling the truth; nullptr if it can.
// Checked: every transfer lies inside [0, count) between two distinct ranks
// of [0, n); within a step no transfer writes what another one of the step
// reads or writes, so that all of a step's transfers can run at once in
// place (the ring's within-step disjointness; AllToAll, whose one step pairs
// its transfers into swaps that its kernel performs together, is exempt);
// the step count is expected_steps(coll, n) (when n > 1 and count > 0); the
// bytes the transfers move per rank equal logical_bytes(), which the
// counters add.  The result is a static string.
const char* schedule_violation(ar_collective_t coll, const std::vector<Step>& steps, int n,
                               uint64_t count, int root);

}  // namespace ar
