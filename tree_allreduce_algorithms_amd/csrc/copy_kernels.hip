// Fused fan-out copy (gfx950): AllGather (chunk c comes from rank c, its
// owner after ReduceScatter) or Broadcast (every chunk comes from the root).
// The chunk split only spreads the work over blockIdx.y; each element is read
// once from its source rank and written into every other rank.
#include "device_common.hpp"

namespace ar {
namespace {

struct FanoutArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t chunk;
  uint64_t tiles;
  int n;
  int root;   // < 0: AllGather
};

template <class T, int U, bool VEC>
__global__ __launch_bounds__(kBlock) void fanout_kernel(FanoutArgs a) {
  constexpr int K = PackOf<T, VEC>::K;
  using P = typename PackOf<T, VEC>::P;
  using S = Pack<T, 1>;

  const int n = a.n;
  const int c = blockIdx.y;
  const uint64_t lo = umin(static_cast<uint64_t>(c) * a.chunk, a.count);
  const uint64_t hi = umin(lo + a.chunk, a.count);
  if (lo >= hi) return;
  const int src = a.root < 0 ? c : a.root;
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t tp = TileGrid<U>::first_pack(s.plo, tile);
    if (tp >= s.phi) break;
    const uint64_t toff = tp * sizeof(P);
    const TileLanes<U, sizeof(P)> ln(tp, s.plo, s.phi);
    const char* sp = at(a.ptrs.p[src], toff);
    P v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (ln.live[u]) v[u] = load_stream<P>(sp, ln.off[u]);
    for (int r = 0; r < n; ++r) {
      if (r == src) continue;
      char* dp = at(a.ptrs.p[r], toff);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ln.live[u]) store_stream<P>(dp, ln.off[u], v[u]);
    }
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    const S v = load<S>(a.ptrs.p[src], e);
    for (int r = 0; r < n; ++r)
      if (r != src) store<S>(a.ptrs.p[r], e, v);
  }
}

template <class T>
const void* fanout_fn(int u, bool vec) {
  if (!vec) return reinterpret_cast<const void*>(&fanout_kernel<T, 1, false>);
  if (u == 4) return reinterpret_cast<const void*>(&fanout_kernel<T, 4, true>);
  if (u == 2) return reinterpret_cast<const void*>(&fanout_kernel<T, 2, true>);
  return reinterpret_cast<const void*>(&fanout_kernel<T, 1, true>);
}

}  // namespace

hipError_t launch_fanout(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                         bool from_root, int root, bool vec, hipStream_t stream) {
  FanoutArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.chunk = chunk_size(n, count);
  a.n = n;
  a.root = from_root ? root : -1;
  const int pack = vec ? static_cast<int>(16 / itemsize(dtype)) : 1;
  const int u = vec ? pick_unroll(UnrollFor::kFanout, n) : 1;
  a.tiles = tiles_for(a.chunk, pack, u);
  const dim3 grid(grid_x(a.tiles), n);
  const void* fn = itemsize(dtype) == 2 ? fanout_fn<uint16_t>(u, vec) : fanout_fn<uint32_t>(u, vec);
  return launch(fn, grid, a, stream);
}

}  // namespace ar
