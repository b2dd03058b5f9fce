// Host-side planning for the collectives: argument validation, the chunk
// layout and the logical schedules (which rank sends which element range to
// which rank at each step).  Pure C++, no HIP: it runs without a GPU.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "ar.h"

namespace ar {

// One logical transfer inside a step: elements [lo, hi) of rank `src` go to
// rank `dst`, which either combines them into its own copy (reduce steps) or
// overwrites its copy (copy steps).
struct Transfer {
  int src;
  int dst;
  uint64_t lo;
  uint64_t hi;
};

struct Step {
  bool reduce;                   // true: dst = dst (+) src; false: dst = src
  std::vector<Transfer> xfers;   // disjoint destinations within a step
};

size_t itemsize(ar_dtype_t dtype);
bool dtype_ok(int dtype);
bool op_ok(int op);

// Ring chunks: C = ceil(T/N); chunk c = [min(cC, T), min((c+1)C, T)).
uint64_t chunk_size(int n, uint64_t count);
void chunk_bounds(int n, uint64_t count, int c, uint64_t* lo, uint64_t* hi);

// Binomial tree depth ceil(log2 n).
int tree_depth(int n);

// Double-tree split: tree 0 owns [0, h), tree 1 owns [h, T), h = ceil(T/2).
uint64_t tree_split(uint64_t count);
// Rank that plays `role` in tree 0 (identity) or tree 1 (mirror).
inline int tree_rank(int tree, int role, int n) { return tree == 0 ? role : n - 1 - role; }

// Logical schedules.  A ring AllReduce is the ReduceScatter steps followed by
// the AllGather steps; the tree is its reduce rounds then its broadcast rounds.
std::vector<Step> ring_reduce_scatter_schedule(int n, uint64_t count);
std::vector<Step> ring_allgather_schedule(int n, uint64_t count);
std::vector<Step> tree_allreduce_schedule(int n, uint64_t count);
std::vector<Step> broadcast_schedule(int n, uint64_t count, int root);
std::vector<Step> reduce_schedule(int n, uint64_t count, int root);
std::vector<Step> scatter_schedule(int n, uint64_t count, int root, bool to_root);
std::vector<Step> alltoall_schedule(int n, uint64_t count);
std::vector<Step> schedule_for(ar_collective_t coll, int n, uint64_t count, int root);

// Adds the bytes of every transfer to sent[src] / recv[dst].
void count_bytes(const std::vector<Step>& steps, size_t isz, uint64_t* sent, uint64_t* recv);

// The same per-rank totals as count_bytes over schedule_for(coll, ...), from
// closed forms, without building the schedule (sent / recv are overwritten).
void logical_bytes(ar_collective_t coll, int n, uint64_t count, int root, size_t isz,
                   uint64_t* sent, uint64_t* recv);

int expected_steps(ar_collective_t coll, int n);

// Kernel launches and HBM bytes of one call of `coll` with implementation
// `impl`: the fused kernels run once and move the algorithmic bytes (every
// input read once, every output written once); the step implementation
// launches once per schedule step and moves 3 bytes per element of each
// reduce transfer (read both sides, write one) and 2 per element of each copy
// transfer.
// The fused AllReduces of many ranks run as two launches (see
// allreduce_split), moving (2N + 1) * T * s bytes.
int impl_launches(ar_collective_t coll, ar_impl_t impl, int n, uint64_t count, size_t isz);
uint64_t impl_hbm_bytes(ar_collective_t coll, ar_impl_t impl, int n, uint64_t count, size_t isz);

// Whether the fused AllReduces run in two launches instead of one fold that
// stores into all N ranks: the ring as the fused ReduceScatter (every
// element folded in ring order into its owner's chunk) then the fused
// AllGather (each owner's chunk copied to every other rank); the double tree
// as its two trees' folds stored into their roots only (rank 0 and rank N-1)
// then each root's half copied to every other rank.  Both give the same bits
// as the one-pass folds: AllReduce is AllGather after ReduceScatter [Lecture
// 09 section 3.9], a tree AllReduce is its reduce then its broadcast [Lecture
// 09 section 5.2], and the first launch leaves exactly the value the one-pass
// fold stores.  With many ranks the one-pass fold writes every tile into all
// N buffers at once, which HBM serves poorly, while the copy writes one
// buffer after another.  Measured on gfx950 (in-process A/B, float32, warm
// clocks): with 384 MiB to 4.8 GB of inputs the two launches are 1-13 %
// faster than the one-pass folds from 16 to 64 ranks (ring at 24 ranks and
// 805 MB: even), 1-9 % faster at 11-16 ranks, within 2 % at 8-10 and 8 %
// slower at 6; with exactly 256 MiB (the Infinity Cache's size) they are
// 1-7 % slower for most rank counts.  So both split from 12 ranks and
// 384 MiB of inputs.
bool allreduce_split(int n, uint64_t count, size_t isz);

// Validation shared by every collective call.  `op` < 0 means "not used",
// `root` < 0 means "not used".  Checks: bufs non-NULL, n in range, dtype /
// op / root ranges, count * itemsize overflow, and, when count > 0, entries
// non-NULL, element alignment and pairwise overlap of the
// [ptr, ptr + count * itemsize) ranges.
ar_status_t validate(void* const* bufs, int n, size_t count, int dtype, int op, int root);

}  // namespace ar
