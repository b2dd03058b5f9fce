// Host check of the library's planning code (plan.cpp), built by
// tests/test_host_sanitized.py with AddressSanitizer and UndefinedBehavior-
// Sanitizer (host code only; nothing here touches a GPU).  Exit status 0 and
// a final "OK" line when every check holds.
//
// Checks, over seeded random and edge-case arguments:
//  * every transfer of every schedule lies inside [0, count) and between two
//    distinct ranks in [0, n);
//  * within one step no transfer writes what another transfer of the step
//    reads or writes (the property that lets one launch run a whole step;
//    AllToAll is exempt: its kernel performs each pair of transfers as one
//    swap);
//  * the closed-form per-rank byte counts equal the counts summed over the
//    schedule, and the step count is the documented one;
//  * the library's own check, schedule_violation() (what AR_DEBUG=1 runs
//    before every call), accepts every schedule above, and names the fault
//    in schedules with a planted one (two writes of the same elements, a
//    write of what another transfer reads, a range past the buffer, a
//    transfer from a rank to itself, a missing step, bytes that differ from
//    the closed forms);
//  * the chunk bounds tile [0, count) in order;
//  * validate() accepts good arguments and rejects NULL entries, misaligned
//    or overlapping buffers, out-of-range roots and sizes whose byte length
//    overflows.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <random>
#include <vector>

#include "plan.hpp"
#include "plan_check.hpp"

namespace {

int g_failures = 0;

#define CHECK(cond, ...)                                        \
  do {                                                          \
    if (!(cond)) {                                              \
      if (g_failures < 20) {                                    \
        std::printf("FAIL %s:%d: %s: ", __FILE__, __LINE__, #cond); \
        std::printf(__VA_ARGS__);                               \
        std::printf("\n");                                      \
      }                                                         \
      ++g_failures;                                             \
    }                                                           \
  } while (0)

bool overlap(uint64_t a0, uint64_t a1, uint64_t b0, uint64_t b1) {
  return a0 < b1 && b0 < a1 && a0 < a1 && b0 < b1;
}

void check_schedule(ar_collective_t coll, int n, uint64_t count, int root) {
  const std::vector<ar::Step> steps = ar::schedule_for(coll, n, count, root);
  if (n > 1 && count > 0)
    CHECK(static_cast<int>(steps.size()) == ar::expected_steps(coll, n),
          "coll %d n %d count %llu: %zu steps", coll, n, (unsigned long long)count, steps.size());
  for (const ar::Step& s : steps) {
    for (size_t i = 0; i < s.xfers.size(); ++i) {
      const ar::Transfer& t = s.xfers[i];
      CHECK(t.src >= 0 && t.src < n && t.dst >= 0 && t.dst < n && t.src != t.dst,
            "coll %d n %d: ranks %d -> %d", coll, n, t.src, t.dst);
      CHECK(t.lo <= t.hi && t.hi <= count, "coll %d n %d: range [%llu, %llu) of %llu", coll, n,
            (unsigned long long)t.lo, (unsigned long long)t.hi, (unsigned long long)count);
    }
    if (coll == AR_ALLTOALL) continue;
    for (size_t i = 0; i < s.xfers.size(); ++i) {
      const ar::Transfer& w = s.xfers[i];
      for (size_t j = 0; j < s.xfers.size(); ++j) {
        if (i == j) continue;
        const ar::Transfer& o = s.xfers[j];
        // w writes (w.dst, range); o reads (o.src, range) and, if it reduces, (o.dst, range)
        const bool hits_read = (o.src == w.dst && overlap(w.lo, w.hi, o.lo, o.hi)) ||
                               (s.reduce && o.dst == w.dst && overlap(w.lo, w.hi, o.lo, o.hi));
        const bool hits_write = o.dst == w.dst && overlap(w.lo, w.hi, o.lo, o.hi);
        CHECK(!hits_read && !hits_write, "coll %d n %d count %llu: transfers %zu and %zu collide",
              coll, n, (unsigned long long)count, i, j);
      }
    }
  }
  const char* why = ar::schedule_violation(coll, steps, n, count, root);
  CHECK(why == nullptr, "coll %d n %d count %llu root %d: schedule_violation: %s", coll, n,
        (unsigned long long)count, root, why ? why : "");
  for (size_t isz : {size_t(2), size_t(4)}) {
    std::vector<uint64_t> s1(n, 0), r1(n, 0), s2(n, 0), r2(n, 0);
    ar::count_bytes(steps, isz, s1.data(), r1.data());
    ar::logical_bytes(coll, n, count, root, isz, s2.data(), r2.data());
    for (int r = 0; r < n; ++r)
      CHECK(s1[r] == s2[r] && r1[r] == r2[r],
            "coll %d n %d count %llu root %d rank %d: schedule %llu/%llu, closed form %llu/%llu",
            coll, n, (unsigned long long)count, root, r, (unsigned long long)s1[r],
            (unsigned long long)r1[r], (unsigned long long)s2[r], (unsigned long long)r2[r]);
  }
}

// schedule_violation() on schedules with one planted fault each: it must
// report the fault named by `expect` (a substring of its message).
void planted(const char* what, ar_collective_t coll, const std::vector<ar::Step>& steps, int n,
             uint64_t count, const char* expect) {
  const char* why = ar::schedule_violation(coll, steps, n, count, 0);
  CHECK(why != nullptr && std::strstr(why, expect) != nullptr, "%s: got \"%s\"", what,
        why ? why : "(accepted)");
}

void check_planted() {
  const int n = 4;
  const uint64_t t = 16;
  const std::vector<ar::Step> rs = ar::ring_reduce_scatter_schedule(n, t);
  CHECK(ar::schedule_violation(AR_REDUCE_SCATTER, rs, n, t, 0) == nullptr, "unplanted schedule");
  std::vector<ar::Step> bad = rs;
  bad[0].xfers.push_back(bad[0].xfers[0]);
  planted("a transfer repeated in its step", AR_REDUCE_SCATTER, bad, n, t, "write the same");
  bad = rs;
  ar::Transfer& x = bad[1].xfers[1];
  x.src = bad[1].xfers[0].dst;   // reads what transfer 0 of the step writes
  x.lo = bad[1].xfers[0].lo;
  x.hi = bad[1].xfers[0].hi;
  if (x.dst == x.src) x.dst = (x.src + 2) % n;
  planted("a transfer reading what another one writes", AR_REDUCE_SCATTER, bad, n, t,
          "writes what another one reads");
  bad = rs;
  bad[0].xfers[0].hi = t + 1;
  planted("a range past the buffer", AR_REDUCE_SCATTER, bad, n, t, "outside the buffer");
  bad = rs;
  bad[0].xfers[0].dst = bad[0].xfers[0].src;
  planted("a transfer to its own rank", AR_REDUCE_SCATTER, bad, n, t, "to itself");
  bad = rs;
  bad.pop_back();
  planted("a missing step", AR_REDUCE_SCATTER, bad, n, t, "step count");
  bad = rs;
  bad[2].xfers[3].hi -= 1;
  planted("a shortened transfer", AR_REDUCE_SCATTER, bad, n, t, "closed forms");
  // a copy step's transfer widened to its destination's whole buffer, part
  // of which the transfer out of that rank reads in the same step
  std::vector<ar::Step> ag = ar::ring_allgather_schedule(n, t);
  ag[0].xfers[2].lo = 0;
  ag[0].xfers[2].hi = t;
  planted("a widened copy", AR_ALLGATHER, ag, n, t, "writes what another one reads");
}

void check_chunks(int n, uint64_t count) {
  uint64_t next = 0;
  for (int c = 0; c < n; ++c) {
    uint64_t lo = 0, hi = 0;
    ar::chunk_bounds(n, count, c, &lo, &hi);
    CHECK(lo == next && lo <= hi && hi <= count, "n %d count %llu chunk %d: [%llu, %llu)", n,
          (unsigned long long)count, c, (unsigned long long)lo, (unsigned long long)hi);
    next = hi;
  }
  CHECK(next == count, "n %d count %llu: chunks end at %llu", n, (unsigned long long)count,
        (unsigned long long)next);
}

void check_validate() {
  alignas(64) static char arena[1 << 16];
  void* good[4] = {arena, arena + 4096, arena + 8192, arena + 12288};
  CHECK(ar::validate(good, 4, 1024, AR_FLOAT32, AR_SUM, -1) == AR_SUCCESS, "good arguments");
  CHECK(ar::validate(good, 4, 1024, AR_FLOAT32, AR_SUM, 3) == AR_SUCCESS, "root 3");
  CHECK(ar::validate(good, 4, 1024, AR_FLOAT32, AR_SUM, 4) == AR_ERROR_INVALID_ARGUMENT, "root 4");
  CHECK(ar::validate(good, 4, 1025, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT,
        "overlap by one element");
  CHECK(ar::validate(good, 4, 0, AR_FLOAT32, AR_SUM, -1) == AR_SUCCESS, "empty");
  void* nulls[4] = {nullptr, nullptr, nullptr, nullptr};
  CHECK(ar::validate(nulls, 4, 0, AR_FLOAT32, AR_SUM, -1) == AR_SUCCESS, "empty, NULL entries");
  CHECK(ar::validate(nulls, 4, 1, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT, "NULL entries");
  void* odd[2] = {arena + 2, arena + 4098};
  CHECK(ar::validate(odd, 2, 16, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT, "2-byte aligned fp32");
  CHECK(ar::validate(odd, 2, 16, AR_BFLOAT16, AR_SUM, -1) == AR_SUCCESS, "2-byte aligned bf16");
  CHECK(ar::validate(good, 4, SIZE_MAX / 2, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT,
        "byte length overflows");
  CHECK(ar::validate(good, 4, SIZE_MAX / 4 - 1, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT,
        "ranges run past the address space");
  CHECK(ar::validate(good, 0, 16, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT, "n = 0");
  CHECK(ar::validate(good, 65, 16, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT, "n = 65");
  CHECK(ar::validate(good, 4, 16, 7, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT, "dtype 7");
  CHECK(ar::validate(good, 4, 16, AR_FLOAT32, 9, -1) == AR_ERROR_INVALID_ARGUMENT, "op 9");
  CHECK(ar::validate(nullptr, 4, 16, AR_FLOAT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT, "bufs NULL");
  void* same[2] = {arena, arena};
  CHECK(ar::validate(same, 2, 1, AR_INT32, AR_SUM, -1) == AR_ERROR_INVALID_ARGUMENT, "same buffer twice");
}

}  // namespace

int main() {
  const ar_collective_t colls[] = {AR_RING_ALLREDUCE, AR_REDUCE_SCATTER, AR_ALLGATHER,
                                   AR_BROADCAST,      AR_TREE_ALLREDUCE, AR_REDUCE,
                                   AR_SCATTER,        AR_GATHER,         AR_ALLTOALL};
  std::mt19937_64 rng(20261202);
  std::vector<std::pair<int, uint64_t>> shapes;
  for (int n = 1; n <= 64; ++n)
    for (uint64_t t : {uint64_t(0), uint64_t(1), uint64_t(n - 1), uint64_t(n), uint64_t(n + 1),
                       uint64_t(3 * n + 2), uint64_t(1000003)})
      shapes.push_back({n, t});
  for (int i = 0; i < 300; ++i)
    shapes.push_back({1 + static_cast<int>(rng() % 64), rng() % (uint64_t(1) << (rng() % 44))});
  shapes.push_back({64, (uint64_t(1) << 40) + 17});
  shapes.push_back({7, (uint64_t(1) << 36) - 3});
  for (const auto& [n, t] : shapes) {
    check_chunks(n, t);
    for (ar_collective_t c : colls) {
      const uint64_t count = c == AR_ALLTOALL ? t - t % n : t;
      const int root = static_cast<int>(rng() % n);
      check_schedule(c, n, count, root);
    }
  }
  check_validate();
  check_planted();
  if (g_failures) {
    std::printf("%d checks failed\n", g_failures);
    return 1;
  }
  std::printf("OK (%zu shapes x 9 collectives)\n", shapes.size());
  return 0;
}
