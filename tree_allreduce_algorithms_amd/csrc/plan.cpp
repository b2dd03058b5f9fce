// Host-side planning: validation, chunk layout, logical schedules, counters.
//
// Schedules follow "Collectives from scratch" (从零实现集合通信), section
// "two-pass ring allreduce": rank r sends to r+1; the ReduceScatter pass has
// rank r forward chunk (r - s) mod N at step s = 1..N-1 (so rank r finishes
// owning chunk r), the AllGather pass forwards the completed chunks around
// once more.  The tree follows Lecture 09 section 5.2 and Chapter 4 section
// 4.3.2 (two trees, half the data each), read as two binomial trees, the
// second on mirrored roles.
#include "plan.hpp"
#include "plan_check.hpp"

#include <algorithm>
#include <utility>

namespace ar {

size_t itemsize(ar_dtype_t dtype) {
  return (dtype == AR_BFLOAT16 || dtype == AR_BFLOAT16_ACC32) ? 2 : 4;
}

bool dtype_ok(int dtype) {
  return dtype == AR_INT32 || dtype == AR_FLOAT32 || dtype == AR_BFLOAT16 ||
         dtype == AR_BFLOAT16_ACC32;
}

bool op_ok(int op) { return op == AR_SUM || op == AR_PROD || op == AR_MAX || op == AR_MIN; }

uint64_t chunk_size(int n, uint64_t count) {
  if (n < 1) return 0;
  const uint64_t un = static_cast<uint64_t>(n);
  return count / un + (count % un != 0 ? 1 : 0);
}

void chunk_bounds(int n, uint64_t count, int c, uint64_t* lo, uint64_t* hi) {
  const uint64_t size = chunk_size(n, count);
  const uint64_t a = static_cast<uint64_t>(c) * size;
  *lo = std::min(a, count);
  *hi = std::min(a + size, count);
}

int tree_depth(int n) {
  int d = 0;
  while ((1 << d) < n) ++d;
  return d;
}

uint64_t tree_split(uint64_t count) { return count / 2 + (count % 2); }

std::vector<Step> ring_reduce_scatter_schedule(int n, uint64_t count) {
  std::vector<Step> out;
  for (int t = 0; t + 1 < n; ++t) {
    Step s{true, {}};
    for (int r = 0; r < n; ++r) {
      const int c = ((r - t - 1) % n + n) % n;
      uint64_t lo, hi;
      chunk_bounds(n, count, c, &lo, &hi);
      s.xfers.push_back({r, (r + 1) % n, lo, hi});
    }
    out.push_back(std::move(s));
  }
  return out;
}

std::vector<Step> ring_allgather_schedule(int n, uint64_t count) {
  std::vector<Step> out;
  for (int t = 0; t + 1 < n; ++t) {
    Step s{false, {}};
    for (int r = 0; r < n; ++r) {
      const int c = ((r - t) % n + n) % n;
      uint64_t lo, hi;
      chunk_bounds(n, count, c, &lo, &hi);
      s.xfers.push_back({r, (r + 1) % n, lo, hi});
    }
    out.push_back(std::move(s));
  }
  return out;
}

std::vector<Step> tree_allreduce_schedule(int n, uint64_t count) {
  const int depth = tree_depth(n);
  const uint64_t h = tree_split(count);
  const uint64_t seg_lo[2] = {0, h};
  const uint64_t seg_hi[2] = {h, count};
  std::vector<Step> out;
  for (int k = 0; k < depth; ++k) {            // reduce rounds, leaves first
    const int stride = 1 << k;
    Step s{true, {}};
    for (int tree = 0; tree < 2; ++tree)
      for (int q = 0; q + stride < n; q += 2 * stride)
        s.xfers.push_back({tree_rank(tree, q + stride, n), tree_rank(tree, q, n), seg_lo[tree],
                           seg_hi[tree]});
    out.push_back(std::move(s));
  }
  for (int k = depth - 1; k >= 0; --k) {       // broadcast rounds, root first
    const int stride = 1 << k;
    Step s{false, {}};
    for (int tree = 0; tree < 2; ++tree)
      for (int q = 0; q + stride < n; q += 2 * stride)
        s.xfers.push_back({tree_rank(tree, q, n), tree_rank(tree, q + stride, n), seg_lo[tree],
                           seg_hi[tree]});
    out.push_back(std::move(s));
  }
  return out;
}

std::vector<Step> broadcast_schedule(int n, uint64_t count, int root) {
  std::vector<Step> out;
  for (int k = tree_depth(n) - 1; k >= 0; --k) {
    const int stride = 1 << k;
    Step s{false, {}};
    for (int q = 0; q + stride < n; q += 2 * stride)
      s.xfers.push_back({(q + root) % n, (q + stride + root) % n, 0, count});
    out.push_back(std::move(s));
  }
  return out;
}

// Reduce to `root`: the binomial reduce rounds on roles (rank - root) mod N
// over the whole buffer.  The fused kernel evaluates these rounds in
// registers; the schedule gives the counters.
std::vector<Step> reduce_schedule(int n, uint64_t count, int root) {
  std::vector<Step> out;
  for (int k = 0; k < tree_depth(n); ++k) {
    const int stride = 1 << k;
    Step s{true, {}};
    for (int q = 0; q + stride < n; q += 2 * stride)
      s.xfers.push_back({(q + stride + root) % n, (q + root) % n, 0, count});
    out.push_back(std::move(s));
  }
  return out;
}

// Scatter / Gather: one step of direct transfers of chunk c between the root
// and rank c.
std::vector<Step> scatter_schedule(int n, uint64_t count, int root, bool to_root) {
  std::vector<Step> out;
  if (n < 2) return out;
  Step s{false, {}};
  for (int c = 0; c < n; ++c) {
    if (c == root) continue;
    uint64_t lo, hi;
    chunk_bounds(n, count, c, &lo, &hi);
    s.xfers.push_back(to_root ? Transfer{c, root, lo, hi} : Transfer{root, c, lo, hi});
  }
  out.push_back(std::move(s));
  return out;
}

// AllToAll: one step in which rank i sends its block j to rank j (block i
// there), for every i != j.  Transfer ranges name the source block; the
// kernel swaps block pairs instead of replaying these transfers.
std::vector<Step> alltoall_schedule(int n, uint64_t count) {
  std::vector<Step> out;
  if (n < 2) return out;
  const uint64_t b = count / static_cast<uint64_t>(n);
  Step s{false, {}};
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j)
      if (i != j) s.xfers.push_back({i, j, static_cast<uint64_t>(j) * b, static_cast<uint64_t>(j + 1) * b});
  out.push_back(std::move(s));
  return out;
}

std::vector<Step> schedule_for(ar_collective_t coll, int n, uint64_t count, int root) {
  switch (coll) {
    case AR_RING_ALLREDUCE: {
      std::vector<Step> a = ring_reduce_scatter_schedule(n, count);
      std::vector<Step> b = ring_allgather_schedule(n, count);
      a.insert(a.end(), b.begin(), b.end());
      return a;
    }
    case AR_REDUCE_SCATTER: return ring_reduce_scatter_schedule(n, count);
    case AR_ALLGATHER: return ring_allgather_schedule(n, count);
    case AR_BROADCAST: return broadcast_schedule(n, count, root);
    case AR_TREE_ALLREDUCE: return tree_allreduce_schedule(n, count);
    case AR_REDUCE: return reduce_schedule(n, count, root);
    case AR_SCATTER: return scatter_schedule(n, count, root, false);
    case AR_GATHER: return scatter_schedule(n, count, root, true);
    case AR_ALLTOALL: return alltoall_schedule(n, count);
  }
  return {};
}

namespace {

// Binomial-tree traffic of role q in a tree over n roles: q sends its segment
// to its parent once (q != 0) and receives one segment from each child.
uint64_t tree_children(int q, int n) {
  uint64_t c = 0;
  for (int k = 0; (1 << k) < n; ++k) {
    if (q % (1 << (k + 1)) != 0) break;
    if (q + (1 << k) < n) ++c;
  }
  return c;
}

uint64_t chunk_len(int n, uint64_t count, int c) {
  uint64_t lo, hi;
  chunk_bounds(n, count, c, &lo, &hi);
  return hi - lo;
}

}  // namespace

void logical_bytes(ar_collective_t coll, int n, uint64_t count, int root, size_t isz,
                   uint64_t* sent, uint64_t* recv) {
  for (int r = 0; r < n; ++r) sent[r] = recv[r] = 0;
  if (n < 2) return;
  auto add = [&](uint64_t* v, int r, uint64_t elems) { v[r] += elems * isz; };
  const bool rs = coll == AR_RING_ALLREDUCE || coll == AR_REDUCE_SCATTER;
  const bool ag = coll == AR_RING_ALLREDUCE || coll == AR_ALLGATHER;
  for (int r = 0; r < n; ++r) {
    const int prev = (r + n - 1) % n, next = (r + 1) % n;
    if (rs) {   // ReduceScatter: r sends every chunk but its own, gets every chunk but r-1's
      add(sent, r, count - chunk_len(n, count, r));
      add(recv, r, count - chunk_len(n, count, prev));
    }
    if (ag) {   // AllGather: r forwards every chunk but r+1's, gets every chunk but its own
      add(sent, r, count - chunk_len(n, count, next));
      add(recv, r, count - chunk_len(n, count, r));
    }
  }
  switch (coll) {
    case AR_TREE_ALLREDUCE: {   // both trees: reduce rounds then the mirrored broadcast rounds
      const uint64_t h = tree_split(count);
      for (int tree = 0; tree < 2; ++tree) {
        const uint64_t seg = tree == 0 ? h : count - h;
        for (int q = 0; q < n; ++q) {
          const int r = tree_rank(tree, q, n);
          const uint64_t moved = seg * (tree_children(q, n) + (q != 0 ? 1 : 0));
          add(sent, r, moved);
          add(recv, r, moved);
        }
      }
      break;
    }
    case AR_BROADCAST:
    case AR_REDUCE:   // one rooted tree over the whole buffer, one direction
      for (int q = 0; q < n; ++q) {
        const int r = (q + root) % n;
        const uint64_t to_children = count * tree_children(q, n);
        const uint64_t to_parent = q != 0 ? count : 0;
        add(coll == AR_BROADCAST ? sent : recv, r, to_children);
        add(coll == AR_BROADCAST ? recv : sent, r, to_parent);
      }
      break;
    case AR_SCATTER:
    case AR_GATHER:
      for (int c = 0; c < n; ++c) {
        if (c == root) continue;
        const uint64_t len = chunk_len(n, count, c);
        add(coll == AR_SCATTER ? sent : recv, root, len);
        add(coll == AR_SCATTER ? recv : sent, c, len);
      }
      break;
    case AR_ALLTOALL: {
      const uint64_t b = count / static_cast<uint64_t>(n);
      for (int r = 0; r < n; ++r) {
        add(sent, r, b * static_cast<uint64_t>(n - 1));
        add(recv, r, b * static_cast<uint64_t>(n - 1));
      }
      break;
    }
    default:
      break;
  }
}

void count_bytes(const std::vector<Step>& steps, size_t isz, uint64_t* sent, uint64_t* recv) {
  for (const Step& s : steps)
    for (const Transfer& x : s.xfers) {
      const uint64_t b = (x.hi - x.lo) * isz;
      sent[x.src] += b;
      recv[x.dst] += b;
    }
}

int expected_steps(ar_collective_t coll, int n) {
  if (n < 1 || n > AR_MAX_RANKS) return -1;
  switch (coll) {
    case AR_RING_ALLREDUCE: return 2 * (n - 1);
    case AR_REDUCE_SCATTER:
    case AR_ALLGATHER: return n - 1;
    case AR_BROADCAST:
    case AR_REDUCE: return tree_depth(n);
    case AR_TREE_ALLREDUCE: return 2 * tree_depth(n);
    case AR_SCATTER:
    case AR_GATHER:
    case AR_ALLTOALL: return n > 1 ? 1 : 0;
  }
  return -1;
}

bool allreduce_split(int n, uint64_t count, size_t isz) {
  constexpr int kMinRanks = 12;
  constexpr uint64_t kMinInputBytes = 3ull << 27;   // 384 MiB
  return n >= kMinRanks && static_cast<uint64_t>(n) * count * isz >= kMinInputBytes;
}

int impl_launches(ar_collective_t coll, ar_impl_t impl, int n, uint64_t count, size_t isz) {
  if (n <= 1) return 0;
  if (impl == AR_IMPL_FUSED && (coll == AR_RING_ALLREDUCE || coll == AR_TREE_ALLREDUCE) &&
      allreduce_split(n, count, isz))
    return 2;
  // Reduce has one (fused) implementation; Scatter, Gather and AllToAll are
  // one step.
  if (impl == AR_IMPL_FUSED || coll == AR_REDUCE || coll == AR_ALLTOALL) return 1;
  return expected_steps(coll, n);
}

uint64_t impl_hbm_bytes(ar_collective_t coll, ar_impl_t impl, int n, uint64_t count, size_t isz) {
  if (n <= 1) return 0;
  const uint64_t un = static_cast<uint64_t>(n);
  // Reduce runs fused under either implementation, AllToAll one swap kernel
  // (every off-diagonal block read and written once); Scatter and Gather
  // run their one schedule step under either (modelled with root 0).
  const bool fused = impl == AR_IMPL_FUSED || coll == AR_REDUCE;
  if (fused && coll != AR_SCATTER && coll != AR_GATHER && coll != AR_ALLTOALL) {
    switch (coll) {
      case AR_RING_ALLREDUCE:
      case AR_TREE_ALLREDUCE:
        return (allreduce_split(n, count, isz) ? 2 * un + 1 : 2 * un) * count * isz;
      case AR_REDUCE_SCATTER:
      case AR_REDUCE: return (un + 1) * count * isz;
      default: return un * count * isz;   // AllGather, Broadcast
    }
  }
  // The literal schedule: 3 bytes per element of each reduce transfer (read
  // both sides, write one), 2 per element of each copy transfer.
  uint64_t sent[AR_MAX_RANKS];
  uint64_t recv[AR_MAX_RANKS];
  logical_bytes(coll, n, count, 0, 1, sent, recv);
  uint64_t moved = 0;
  for (int r = 0; r < n; ++r) moved += sent[r];
  uint64_t reduced = 0;
  if (coll == AR_RING_ALLREDUCE || coll == AR_TREE_ALLREDUCE) reduced = moved / 2;
  if (coll == AR_REDUCE_SCATTER) reduced = moved;
  return (3 * reduced + 2 * (moved - reduced)) * isz;
}

ar_status_t validate(void* const* bufs, int n, size_t count, int dtype, int op, int root) {
  if (!dtype_ok(dtype)) return AR_ERROR_INVALID_ARGUMENT;
  if (op >= 0 && !op_ok(op)) return AR_ERROR_INVALID_ARGUMENT;
  if (bufs == nullptr || n < 1 || n > AR_MAX_RANKS) return AR_ERROR_INVALID_ARGUMENT;
  if (root >= n) return AR_ERROR_INVALID_ARGUMENT;
  const size_t isz = itemsize(static_cast<ar_dtype_t>(dtype));
  if (count > SIZE_MAX / isz) return AR_ERROR_INVALID_ARGUMENT;
  if (count == 0) return AR_SUCCESS;   // no element is touched: entries are not inspected
  const uint64_t bytes = static_cast<uint64_t>(count) * isz;
  std::pair<uintptr_t, int> order[AR_MAX_RANKS];
  for (int r = 0; r < n; ++r) {
    const uintptr_t p = reinterpret_cast<uintptr_t>(bufs[r]);
    if (p == 0 || p % isz != 0) return AR_ERROR_INVALID_ARGUMENT;
    if (bytes > UINTPTR_MAX - p) return AR_ERROR_INVALID_ARGUMENT;
    order[r] = {p, r};
  }
  if (bytes > 0) {
    std::sort(order, order + n);
    for (int i = 0; i + 1 < n; ++i)
      if (order[i].first + bytes > order[i + 1].first) return AR_ERROR_INVALID_ARGUMENT;
  }
  return AR_SUCCESS;
}

namespace {

// Transfers a and b touch overlapping elements of ranks ra and rb.
bool collide(const Transfer& a, int ra, const Transfer& b, int rb) {
  return ra == rb && a.lo < a.hi && b.lo < b.hi && a.lo < b.hi && b.lo < a.hi;
}

}  // namespace

const char* schedule_violation(ar_collective_t coll, const std::vector<Step>& steps, int n,
                               uint64_t count, int root) {
  if (n < 1 || n > AR_MAX_RANKS) return "rank count out of range";
  if (n > 1 && count > 0 && static_cast<int>(steps.size()) != expected_steps(coll, n))
    return "the step count differs from the documented one";
  for (const Step& s : steps) {
    for (const Transfer& t : s.xfers) {
      if (t.src < 0 || t.src >= n || t.dst < 0 || t.dst >= n || t.src == t.dst)
        return "a transfer between ranks out of range or from a rank to itself";
      if (t.lo > t.hi || t.hi > count) return "a transfer outside the buffer";
    }
    if (coll == AR_ALLTOALL) continue;
    // a transfer writes its destination's range (and reads it too when the
    // step reduces), and reads its source's range
    for (size_t i = 0; i < s.xfers.size(); ++i) {
      const Transfer& w = s.xfers[i];
      for (size_t j = 0; j < s.xfers.size(); ++j) {
        if (i == j) continue;
        const Transfer& o = s.xfers[j];
        if (collide(w, w.dst, o, o.dst)) return "two transfers of a step write the same elements";
        if (collide(w, w.dst, o, o.src)) return "a transfer of a step writes what another one reads";
      }
    }
  }
  uint64_t sent[AR_MAX_RANKS] = {};
  uint64_t recv[AR_MAX_RANKS] = {};
  uint64_t want_sent[AR_MAX_RANKS];
  uint64_t want_recv[AR_MAX_RANKS];
  count_bytes(steps, 1, sent, recv);
  logical_bytes(coll, n, count, root, 1, want_sent, want_recv);
  for (int r = 0; r < n; ++r)
    if (sent[r] != want_sent[r] || recv[r] != want_recv[r])
      return "the schedule's bytes differ from the counters' closed forms";
  return nullptr;
}

}  // namespace ar
