// Kernel launchers for the collectives (gfx950).  Every launcher enqueues on
// `stream` and returns the hipError_t of the launch; none synchronises.
// `vec` selects 16-byte packs (every rank buffer 16-byte aligned) or the
// element-at-a-time path (buffers aligned only to the element size); the two
// give identical results.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "ar.h"
#include "plan.hpp"

namespace ar {

struct RankPtrs {
  void* p[AR_MAX_RANKS];
};

// Fused ring fold: for every element i of chunk c, fold ranks c+1, c+2, ...,
// c in that order (each hop: rank's own value (+) incoming partial) and store
// the result into every rank (all_ranks, AllReduce) or into rank c only
// (ReduceScatter).
hipError_t launch_ring_fold(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                            ar_op_t op, bool all_ranks, bool vec, hipStream_t stream);

// Fused fan-out copy: for every element i of chunk c, copy from rank c
// (allgather) or from `root` (broadcast) into every other rank.
hipError_t launch_fanout(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                         bool from_root, int root, bool vec, hipStream_t stream);

// The double tree's broadcast as one fan-out: elements [0, ceil(T/2)) copied
// from rank 0 (tree 0's root), [ceil(T/2), T) from rank N-1 (tree 1's root),
// into every other rank.
hipError_t launch_tree_broadcast(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                                 bool vec, hipStream_t stream);

// AllToAll: block j of rank i and block i of rank j swap places for every
// pair i < j (count must be a multiple of n).
hipError_t launch_alltoall(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype, bool vec,
                           hipStream_t stream);

// Fused binomial tree fold.  root < 0: the double tree, per element the
// pairwise fold of the tree that owns it, stored into every rank (or, with
// to_roots, into the owning tree's root only: rank 0 for [0, ceil(T/2)),
// rank N-1 for the rest).  root >= 0: Reduce, one tree over the whole buffer
// on roles (rank - root) mod N, stored into bufs[root] only.
hipError_t launch_tree_fold(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                            ar_op_t op, int root, bool to_roots, bool vec, hipStream_t stream);

// One schedule step: all of its transfers in one launch.
hipError_t launch_step(const RankPtrs& ptrs, const Step& step, ar_dtype_t dtype, ar_op_t op,
                       bool vec, hipStream_t stream);

}  // namespace ar
