// One schedule step per launch (gfx950): the literal ring / tree schedules.
#include "device_common.hpp"

namespace ar {
namespace {

constexpr int kStepUnroll = 4;

// ---------------------------------------------------------------------------
// One schedule step: transfer j (blockIdx.y) moves elements [lo, hi) from
// src[j] to dst[j], combining (reduce steps) or overwriting (copy steps).
// Destinations of one step never overlap and no transfer reads what another
// transfer of the same step writes (a ring ReduceScatter step has rank r read
// its chunk r-t-1 and update its chunk r-t-2; an AllGather step reads chunk
// r-t and writes chunk r-t-1; a tree round's receivers and senders are
// disjoint role sets), so one launch per step is race-free.
// ---------------------------------------------------------------------------
struct StepArgs {
  const void* src[AR_MAX_RANKS];
  void* dst[AR_MAX_RANKS];
  uint64_t lo[AR_MAX_RANKS];
  uint64_t hi[AR_MAX_RANKS];
  uint64_t tiles;
};

template <ar_dtype_t DT, ar_op_t OP, bool REDUCE, bool VEC>
__global__ __launch_bounds__(kBlock) void step_kernel(StepArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int K = PackOf<T, VEC>::K;
  constexpr int U = VEC ? kStepUnroll : 1;
  using P = typename PackOf<T, VEC>::P;
  using S = Pack<T, 1>;

  const int j = blockIdx.y;
  const uint64_t lo = a.lo[j];
  const uint64_t hi = a.hi[j];
  if (lo >= hi) return;
  const void* src = a.src[j];
  void* dst = a.dst[j];
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t tp = TileGrid<U>::first_pack(s.plo, tile);
    if (tp >= s.phi) break;
    const uint64_t toff = tp * sizeof(P);
    const TileLanes<U, sizeof(P)> ln(tp, s.plo, s.phi);
    const char* sp = at(src, toff);
    char* dp = at(dst, toff);
    P in[U];
    P own[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ln.live[u]) {
        in[u] = load_stream<P>(sp, ln.off[u]);
        if (REDUCE) own[u] = load_stream<P>(dp, ln.off[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ln.live[u])
        store_cached<P>(dp, ln.off[u], REDUCE ? combine<DT, OP>(own[u], in[u]) : in[u]);
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    const S in = load<S>(src, e);
    store<S>(dst, e, REDUCE ? combine<DT, OP>(load<S>(dst, e), in) : in);
  }
}

template <ar_dtype_t DT, ar_op_t OP>
hipError_t step_typed(const StepArgs& a, int nxfers, bool reduce, bool vec, hipStream_t stream) {
  const dim3 grid(grid_x(a.tiles), nxfers);
  const void* fn;
  if (reduce)
    fn = vec ? reinterpret_cast<const void*>(&step_kernel<DT, OP, true, true>)
             : reinterpret_cast<const void*>(&step_kernel<DT, OP, true, false>);
  else
    fn = vec ? reinterpret_cast<const void*>(&step_kernel<DT, AR_SUM, false, true>)
             : reinterpret_cast<const void*>(&step_kernel<DT, AR_SUM, false, false>);
  return launch(fn, grid, a, stream);
}

}  // namespace

hipError_t launch_step(const RankPtrs& ptrs, const Step& step, ar_dtype_t dtype, ar_op_t op,
                       bool vec, hipStream_t stream) {
  const int nx = static_cast<int>(step.xfers.size());
  if (nx == 0) return hipSuccess;
  if (nx > AR_MAX_RANKS) return hipErrorInvalidValue;
  StepArgs a;
  uint64_t longest = 0;
  for (int j = 0; j < nx; ++j) {
    const Transfer& x = step.xfers[j];
    a.src[j] = ptrs.p[x.src];
    a.dst[j] = ptrs.p[x.dst];
    a.lo[j] = x.lo;
    a.hi[j] = x.hi;
    longest = std::max(longest, x.hi - x.lo);
  }
  if (longest == 0) return hipSuccess;
  a.tiles = vec ? tiles_for(longest, static_cast<int>(16 / itemsize(dtype)), kStepUnroll)
              : tiles_for(longest, 1, 1);
  AR_DISPATCH(step_typed, dtype, op, a, nx, step.reduce, vec, stream);
}

}  // namespace ar
