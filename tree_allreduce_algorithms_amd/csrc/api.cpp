// C ABI of libar.so: argument validation, implementation dispatch, counters.
//
// Every call validates its arguments before touching the HIP runtime, so
// argument errors are reported with nothing enqueued (and can be exercised
// on a machine without a GPU).  Kernels run on the caller's stream; the
// library never synchronises and never allocates.
#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <vector>

#include "ar.h"
#include "kernels.hpp"
#include "plan.hpp"
#include "plan_check.hpp"

namespace {

std::mutex g_counter_mu;
uint64_t g_sent[AR_MAX_RANKS];
uint64_t g_recv[AR_MAX_RANKS];
uint64_t g_steps = 0;

ar_impl_t impl_from_env() {
  const char* v = std::getenv("AR_IMPL");
  return (v != nullptr && std::strcmp(v, "step") == 0) ? AR_IMPL_STEP : AR_IMPL_FUSED;
}
std::atomic<int> g_impl{static_cast<int>(impl_from_env())};

// AR_DEBUG (set and not "0" at load): before enqueuing anything, every call
// with work to do builds the logical schedule it follows and checks it with
// schedule_violation(); a violation (a defect of this library) is printed
// and aborts the process.
bool debug_from_env() {
  const char* v = std::getenv("AR_DEBUG");
  return v != nullptr && v[0] != '\0' && std::strcmp(v, "0") != 0;
}
const bool g_debug = debug_from_env();

void debug_check_schedule(ar_collective_t coll, int n, size_t count, int root) {
  const int r = root < 0 ? 0 : root;
  const char* why = ar::schedule_violation(coll, ar::schedule_for(coll, n, count, r), n, count, r);
  if (why != nullptr) {
    std::fprintf(stderr, "libar: AR_DEBUG: the schedule of collective %d (N=%d, T=%zu, root %d) "
                 "fails its check: %s\n", static_cast<int>(coll), n, count, r, why);
    std::abort();
  }
}

thread_local int t_last_hip_error = 0;

// Launch-failure injection (ar_debug_fail_launch): while the counter is
// positive, every launch the library is about to make takes one from it, and
// the launch that takes it from 1 to 0 returns hipErrorLaunchFailure without
// reaching the HIP runtime.
std::atomic<int> g_fail_launch{0};

template <class F>
hipError_t enqueue(F&& launch_fn) {
  int k = g_fail_launch.load(std::memory_order_relaxed);
  while (k > 0 && !g_fail_launch.compare_exchange_weak(k, k - 1, std::memory_order_relaxed)) {
  }
  if (k == 1) return hipErrorLaunchFailure;
  return launch_fn();
}

// Cost model coefficients (alpha_us per launch, gbps of HBM traffic) per
// collective and implementation.  The AllReduce pairs are the least-squares
// fit of launches * alpha + bytes / gbps to the N=4 float32 message-size sweep
// (1 KiB to 256 MiB per rank, Infinity Cache flushed before every call) on
// one MI355X.  The fused ring and the fused double tree are one launch of the
// same work each (N reads and N writes per element) and measure within 1-2 %
// of each other at every size, so their points are fitted together and they
// share one pair: the model ties them and the ring runs.  The other
// collectives were measured at one size each (N=64 x 64 MB per rank; AllToAll
// N=8 x 128 MiB), which fixes their bandwidth given the AllReduce fit's
// per-launch alpha (the fused one for fused kernels, a ring step's for step
// launches, Scatter, Gather and AllToAll).
struct CostCoeff {
  double alpha_us;
  double gbps;
};
std::mutex g_cost_mu;
CostCoeff g_cost[9][2] = {
    {{7.66, 6546.0}, {3.32, 6669.0}},   // ring AllReduce: fused, step
    {{7.66, 6604.0}, {3.32, 6600.0}},   // ReduceScatter
    {{7.66, 7247.0}, {3.32, 7451.0}},   // AllGather
    {{7.66, 7247.0}, {3.32, 5846.0}},   // Broadcast
    {{7.66, 6546.0}, {3.22, 6071.0}},   // double-tree AllReduce
    {{7.66, 6706.0}, {7.66, 6706.0}},   // Reduce (fused either way)
    {{3.32, 4224.0}, {3.32, 4224.0}},   // Scatter (one step either way)
    {{3.32, 5556.0}, {3.32, 5556.0}},   // Gather (one step either way)
    {{3.32, 6060.0}, {3.32, 6060.0}},   // AllToAll (one kernel either way)
};

bool coll_ok(int coll) { return coll >= AR_RING_ALLREDUCE && coll <= AR_ALLTOALL; }
bool impl_ok(int impl) { return impl == AR_IMPL_FUSED || impl == AR_IMPL_STEP; }

// The implementation a call runs: bfloat16 with float32 partials runs its
// reductions fused whatever the setting.
ar_impl_t effective_impl(ar_collective_t coll, ar_impl_t impl, ar_dtype_t dtype) {
  if (dtype == AR_BFLOAT16_ACC32 &&
      (coll == AR_RING_ALLREDUCE || coll == AR_REDUCE_SCATTER || coll == AR_TREE_ALLREDUCE))
    return AR_IMPL_FUSED;
  return impl;
}

double predict_us(ar_collective_t coll, ar_impl_t impl, int n, size_t count, ar_dtype_t dtype) {
  impl = effective_impl(coll, impl, dtype);
  CostCoeff c;
  {
    std::lock_guard<std::mutex> lock(g_cost_mu);
    c = g_cost[coll][impl];
  }
  const double launches = ar::impl_launches(coll, impl, n, count, ar::itemsize(dtype));
  const double bytes = static_cast<double>(ar::impl_hbm_bytes(coll, impl, n, count, ar::itemsize(dtype)));
  return launches * c.alpha_us + bytes / (c.gbps * 1e3);
}

ar_collective_t choose_allreduce(int n, size_t count, ar_dtype_t dtype) {
  const ar_impl_t impl = static_cast<ar_impl_t>(g_impl.load());
  const double ring = predict_us(AR_RING_ALLREDUCE, impl, n, count, dtype);
  const double tree = predict_us(AR_TREE_ALLREDUCE, impl, n, count, dtype);
  return tree < ring ? AR_TREE_ALLREDUCE : AR_RING_ALLREDUCE;
}

void add_counters(ar_collective_t coll, int n, uint64_t count, int root, size_t isz) {
  uint64_t sent[AR_MAX_RANKS];
  uint64_t recv[AR_MAX_RANKS];
  ar::logical_bytes(coll, n, count, root < 0 ? 0 : root, isz, sent, recv);
  std::lock_guard<std::mutex> lock(g_counter_mu);
  for (int r = 0; r < n; ++r) {
    g_sent[r] += sent[r];
    g_recv[r] += recv[r];
  }
  g_steps += static_cast<uint64_t>(ar::expected_steps(coll, n));
}

ar_status_t run(ar_collective_t coll, void* const* bufs, int n, size_t count, ar_dtype_t dtype,
                int op, int root, hipStream_t stream) {
  // dtype may be rewritten below (bfloat16 copies); counters use its size,
  // which the rewrite keeps
  const ar_status_t v = ar::validate(bufs, n, count, static_cast<int>(dtype), op, root);
  if (v != AR_SUCCESS) return v;
  const ar_op_t aop = op >= 0 ? static_cast<ar_op_t>(op) : AR_SUM;
  if (n == 1 || count == 0) {
    add_counters(coll, n, count, root, ar::itemsize(dtype));
    return AR_SUCCESS;
  }

  if (g_debug) debug_check_schedule(coll, n, count, root);

  ar::RankPtrs ptrs;
  std::memset(&ptrs, 0, sizeof(ptrs));
  bool aligned16 = true;
  for (int r = 0; r < n; ++r) {
    ptrs.p[r] = bufs[r];
    aligned16 = aligned16 && (reinterpret_cast<uintptr_t>(bufs[r]) % 16 == 0);
  }
  // bfloat16 with float32 partials: the reductions can only run fused (a
  // partial cannot live in a bfloat16 buffer between launches); the copies
  // are bfloat16 copies.
  const bool acc32 = dtype == AR_BFLOAT16_ACC32;
  const bool reduction = coll == AR_RING_ALLREDUCE || coll == AR_REDUCE_SCATTER ||
                         coll == AR_TREE_ALLREDUCE || coll == AR_REDUCE;
  const ar_impl_t impl =
      (acc32 && reduction) ? AR_IMPL_FUSED : static_cast<ar_impl_t>(g_impl.load());
  if (acc32 && !reduction) dtype = AR_BFLOAT16;

  // 16-byte packs need every buffer 16-byte aligned (pack p of every rank
  // then covers the same elements); otherwise the kernels move one element
  // at a time, with the same arithmetic in the same order.
  const bool vec = aligned16;

  hipError_t err = hipSuccess;
  if (coll == AR_REDUCE) {
    // one implementation: the partials of the rounds live in registers, so
    // no rank other than the root is written
    err = enqueue([&] { return ar::launch_tree_fold(ptrs, n, count, dtype, aop, root, false, vec, stream); });
  } else if (coll == AR_ALLTOALL) {
    err = enqueue([&] { return ar::launch_alltoall(ptrs, n, count, dtype, vec, stream); });
  } else if (impl == AR_IMPL_STEP || coll == AR_SCATTER || coll == AR_GATHER) {
    // the literal schedule: one launch per step (the schedule is built only here)
    const std::vector<ar::Step> sched = ar::schedule_for(coll, n, count, root < 0 ? 0 : root);
    for (const ar::Step& s : sched) {
      err = enqueue([&] { return ar::launch_step(ptrs, s, dtype, aop, vec, stream); });
      if (err != hipSuccess) break;
    }
  } else {
    switch (coll) {
      case AR_RING_ALLREDUCE:
        if (ar::allreduce_split(n, count, ar::itemsize(dtype))) {
          // fused ReduceScatter, then the owners' chunks fanned out: the same
          // bits as the one-pass fold (AllReduce = AllGather after
          // ReduceScatter), faster for many ranks
          err = enqueue([&] { return ar::launch_ring_fold(ptrs, n, count, dtype, aop, false, vec, stream); });
          if (err == hipSuccess)
            err = enqueue([&] { return ar::launch_fanout(ptrs, n, count, dtype, false, 0, vec, stream); });
        } else {
          err = enqueue([&] { return ar::launch_ring_fold(ptrs, n, count, dtype, aop, true, vec, stream); });
        }
        break;
      case AR_REDUCE_SCATTER:
        err = enqueue([&] { return ar::launch_ring_fold(ptrs, n, count, dtype, aop, false, vec, stream); });
        break;
      case AR_ALLGATHER:
        err = enqueue([&] { return ar::launch_fanout(ptrs, n, count, dtype, false, 0, vec, stream); });
        break;
      case AR_BROADCAST:
        err = enqueue([&] { return ar::launch_fanout(ptrs, n, count, dtype, true, root, vec, stream); });
        break;
      case AR_TREE_ALLREDUCE:
        if (ar::allreduce_split(n, count, ar::itemsize(dtype))) {
          // both trees' folds stored into their roots, then each root's half
          // fanned out: the reduce and broadcast passes, the same bits as the
          // one-pass fold, faster for many ranks
          err = enqueue([&] { return ar::launch_tree_fold(ptrs, n, count, dtype, aop, -1, true, vec, stream); });
          if (err == hipSuccess)
            err = enqueue([&] { return ar::launch_tree_broadcast(ptrs, n, count, dtype, vec, stream); });
        } else {
          err = enqueue([&] { return ar::launch_tree_fold(ptrs, n, count, dtype, aop, -1, false, vec, stream); });
        }
        break;
      default:   // Reduce, Scatter, Gather and AllToAll are dispatched above
        break;
    }
  }
  if (err != hipSuccess) {
    t_last_hip_error = static_cast<int>(err);
    return AR_ERROR_HIP;
  }
  add_counters(coll, n, count, root, ar::itemsize(dtype));
  return AR_SUCCESS;
}

}  // namespace

extern "C" {

ar_status_t ar_ring_allreduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                              ar_op_t op, hipStream_t stream) {
  if (!ar::op_ok(static_cast<int>(op))) return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_RING_ALLREDUCE, bufs, nranks, count, dtype, static_cast<int>(op), -1, stream);
}

ar_status_t ar_reduce_scatter(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                              ar_op_t op, hipStream_t stream) {
  if (!ar::op_ok(static_cast<int>(op))) return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_REDUCE_SCATTER, bufs, nranks, count, dtype, static_cast<int>(op), -1, stream);
}

ar_status_t ar_allgather(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                         hipStream_t stream) {
  return run(AR_ALLGATHER, bufs, nranks, count, dtype, -1, -1, stream);
}

ar_status_t ar_broadcast(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, int root,
                         hipStream_t stream) {
  if (root < 0) return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_BROADCAST, bufs, nranks, count, dtype, -1, root, stream);
}

ar_status_t ar_tree_allreduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                              ar_op_t op, hipStream_t stream) {
  if (!ar::op_ok(static_cast<int>(op))) return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_TREE_ALLREDUCE, bufs, nranks, count, dtype, static_cast<int>(op), -1, stream);
}

ar_status_t ar_reduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, ar_op_t op,
                      int root, hipStream_t stream) {
  if (!ar::op_ok(static_cast<int>(op)) || root < 0) return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_REDUCE, bufs, nranks, count, dtype, static_cast<int>(op), root, stream);
}

ar_status_t ar_scatter(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, int root,
                       hipStream_t stream) {
  if (root < 0) return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_SCATTER, bufs, nranks, count, dtype, -1, root, stream);
}

ar_status_t ar_gather(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, int root,
                      hipStream_t stream) {
  if (root < 0) return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_GATHER, bufs, nranks, count, dtype, -1, root, stream);
}

ar_status_t ar_alltoall(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype,
                        hipStream_t stream) {
  if (nranks >= 1 && nranks <= AR_MAX_RANKS && count % static_cast<size_t>(nranks) != 0)
    return AR_ERROR_INVALID_ARGUMENT;
  return run(AR_ALLTOALL, bufs, nranks, count, dtype, -1, -1, stream);
}

ar_status_t ar_allreduce(void* const* bufs, int nranks, size_t count, ar_dtype_t dtype, ar_op_t op,
                         hipStream_t stream) {
  if (!ar::op_ok(static_cast<int>(op))) return AR_ERROR_INVALID_ARGUMENT;
  if (nranks < 1 || nranks > AR_MAX_RANKS || !ar::dtype_ok(static_cast<int>(dtype)))
    return AR_ERROR_INVALID_ARGUMENT;
  return run(choose_allreduce(nranks, count, dtype), bufs, nranks, count, dtype,
             static_cast<int>(op), -1, stream);
}

ar_status_t ar_allreduce_choice(int nranks, size_t count, ar_dtype_t dtype, ar_collective_t* choice) {
  if (nranks < 1 || nranks > AR_MAX_RANKS || !ar::dtype_ok(static_cast<int>(dtype)) ||
      choice == nullptr)
    return AR_ERROR_INVALID_ARGUMENT;
  *choice = choose_allreduce(nranks, count, dtype);
  return AR_SUCCESS;
}

ar_status_t ar_predict_time(ar_collective_t coll, ar_impl_t impl, int nranks, size_t count,
                            ar_dtype_t dtype, double* microseconds) {
  if (!coll_ok(coll) || !impl_ok(impl) || nranks < 1 || nranks > AR_MAX_RANKS ||
      !ar::dtype_ok(static_cast<int>(dtype)) || microseconds == nullptr)
    return AR_ERROR_INVALID_ARGUMENT;
  *microseconds = predict_us(coll, impl, nranks, count, dtype);
  return AR_SUCCESS;
}

ar_status_t ar_launch_plan(ar_collective_t coll, ar_impl_t impl, int nranks, size_t count,
                           ar_dtype_t dtype, int* launches, uint64_t* hbm_bytes) {
  if (!coll_ok(coll) || !impl_ok(impl) || nranks < 1 || nranks > AR_MAX_RANKS ||
      !ar::dtype_ok(static_cast<int>(dtype)) || launches == nullptr || hbm_bytes == nullptr)
    return AR_ERROR_INVALID_ARGUMENT;
  const ar_impl_t run = effective_impl(coll, impl, dtype);
  const size_t isz = ar::itemsize(dtype);
  *launches = ar::impl_launches(coll, run, nranks, count, isz);
  *hbm_bytes = ar::impl_hbm_bytes(coll, run, nranks, count, isz);
  return AR_SUCCESS;
}

ar_status_t ar_set_cost_model(ar_collective_t coll, ar_impl_t impl, double alpha_us, double gbps) {
  if (!coll_ok(coll) || !impl_ok(impl) || !(alpha_us >= 0.0) || !(gbps > 0.0))
    return AR_ERROR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(g_cost_mu);
  g_cost[coll][impl] = {alpha_us, gbps};
  return AR_SUCCESS;
}

ar_status_t ar_get_cost_model(ar_collective_t coll, ar_impl_t impl, double* alpha_us, double* gbps) {
  if (!coll_ok(coll) || !impl_ok(impl)) return AR_ERROR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(g_cost_mu);
  if (alpha_us != nullptr) *alpha_us = g_cost[coll][impl].alpha_us;
  if (gbps != nullptr) *gbps = g_cost[coll][impl].gbps;
  return AR_SUCCESS;
}

size_t ar_chunk_size(int nranks, size_t count) {
  return static_cast<size_t>(ar::chunk_size(nranks, count));
}

ar_status_t ar_chunk_range(int nranks, size_t count, int chunk, size_t* begin, size_t* end) {
  if (nranks < 1 || nranks > AR_MAX_RANKS || chunk < 0 || chunk >= nranks || begin == nullptr ||
      end == nullptr)
    return AR_ERROR_INVALID_ARGUMENT;
  uint64_t lo, hi;
  ar::chunk_bounds(nranks, count, chunk, &lo, &hi);
  *begin = static_cast<size_t>(lo);
  *end = static_cast<size_t>(hi);
  return AR_SUCCESS;
}

ar_status_t ar_expected_bytes(ar_collective_t coll, int nranks, size_t count, ar_dtype_t dtype,
                              int root, uint64_t* sent, uint64_t* recv) {
  if (nranks < 1 || nranks > AR_MAX_RANKS || !ar::dtype_ok(static_cast<int>(dtype)) ||
      sent == nullptr || recv == nullptr || ar::expected_steps(coll, nranks) < 0)
    return AR_ERROR_INVALID_ARGUMENT;
  const bool rooted =
      coll == AR_BROADCAST || coll == AR_REDUCE || coll == AR_SCATTER || coll == AR_GATHER;
  if (rooted && (root < 0 || root >= nranks)) return AR_ERROR_INVALID_ARGUMENT;
  if (coll == AR_ALLTOALL && count % static_cast<size_t>(nranks) != 0)
    return AR_ERROR_INVALID_ARGUMENT;
  ar::logical_bytes(coll, nranks, count, rooted ? root : 0, ar::itemsize(dtype), sent, recv);
  return AR_SUCCESS;
}

int ar_expected_steps(ar_collective_t coll, int nranks) { return ar::expected_steps(coll, nranks); }

ar_status_t ar_counters_read(int nranks, uint64_t* sent, uint64_t* recv) {
  if (nranks < 0 || nranks > AR_MAX_RANKS) return AR_ERROR_INVALID_ARGUMENT;
  std::lock_guard<std::mutex> lock(g_counter_mu);
  for (int r = 0; r < nranks; ++r) {
    if (sent != nullptr) sent[r] = g_sent[r];
    if (recv != nullptr) recv[r] = g_recv[r];
  }
  return AR_SUCCESS;
}

uint64_t ar_counters_steps(void) {
  std::lock_guard<std::mutex> lock(g_counter_mu);
  return g_steps;
}

void ar_counters_reset(void) {
  std::lock_guard<std::mutex> lock(g_counter_mu);
  for (int r = 0; r < AR_MAX_RANKS; ++r) g_sent[r] = g_recv[r] = 0;
  g_steps = 0;
}

ar_status_t ar_set_impl(ar_impl_t impl) {
  if (impl != AR_IMPL_FUSED && impl != AR_IMPL_STEP) return AR_ERROR_INVALID_ARGUMENT;
  g_impl.store(static_cast<int>(impl));
  return AR_SUCCESS;
}

ar_impl_t ar_get_impl(void) { return static_cast<ar_impl_t>(g_impl.load()); }

const char* ar_status_string(ar_status_t status) {
  switch (status) {
    case AR_SUCCESS: return "success";
    case AR_ERROR_INVALID_ARGUMENT: return "invalid argument";
    case AR_ERROR_UNSUPPORTED: return "unsupported";
    case AR_ERROR_HIP: return "HIP error";
  }
  return "unknown status";
}

int ar_last_hip_error(void) { return t_last_hip_error; }

ar_status_t ar_debug_fail_launch(int k) {
  if (k < 0) return AR_ERROR_INVALID_ARGUMENT;
  g_fail_launch.store(k);
  return AR_SUCCESS;
}

int ar_version(void) { return AR_VERSION; }

}  // extern "C"
