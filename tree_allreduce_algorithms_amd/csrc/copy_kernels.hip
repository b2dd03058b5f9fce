// Copy kernels (gfx950).
//
// Fan-out: AllGather (chunk c comes from rank c, its owner after
// ReduceScatter) or Broadcast (every chunk comes from the root).  The chunk
// split only spreads the work over blockIdx.y; each element is read once
// from its source rank and written into every other rank.
//
// AllToAll: block j of rank i and block i of rank j trade places, one thread
// per pack of the pair, so every off-diagonal element is read once and
// written once and no two threads touch the same location.
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
        if (ln.live[u]) store_cached<P>(dp, ln.off[u], v[u]);
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

// AllToAll block swap: blockIdx.y = i * n + j; pairs with i >= j exit (the
// diagonal stays in place, and each pair is swapped once, by i < j).
struct AllToAllArgs {
  RankPtrs ptrs;
  uint64_t block;   // elements per block (count / n)
  uint64_t tiles;
  int n;
};

template <class T, int U, bool VEC>
__global__ __launch_bounds__(kBlock) void alltoall_kernel(AllToAllArgs a) {
  using P = typename PackOf<T, VEC>::P;
  constexpr int K = PackOf<T, VEC>::K;
  const int i = static_cast<int>(blockIdx.y) / a.n;
  const int j = static_cast<int>(blockIdx.y) % a.n;
  if (i >= j) return;
  const uint64_t npacks = a.block / K;   // VEC only when K divides the block
  const uint64_t bbytes = a.block * sizeof(T);
  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t tp = TileGrid<U>::first_pack(0, tile);
    if (tp >= npacks) break;
    const uint64_t toff = tp * sizeof(P);
    const TileLanes<U, sizeof(P)> ln(tp, 0, npacks);
    char* bi = at(a.ptrs.p[i], static_cast<uint64_t>(j) * bbytes + toff);   // rank i, block j
    char* bj = at(a.ptrs.p[j], static_cast<uint64_t>(i) * bbytes + toff);   // rank j, block i
    P x[U], y[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ln.live[u]) {
        x[u] = load_stream<P>(bi, ln.off[u]);
        y[u] = load_stream<P>(bj, ln.off[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (ln.live[u]) {
        store_stream<P>(bi, ln.off[u], y[u]);
        store_stream<P>(bj, ln.off[u], x[u]);
      }
    }
  }
}

template <class T>
const void* alltoall_fn(bool vec) {
  return vec ? reinterpret_cast<const void*>(&alltoall_kernel<T, 2, true>)
             : reinterpret_cast<const void*>(&alltoall_kernel<T, 1, false>);
}

}  // namespace

hipError_t launch_alltoall(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype, bool vec,
                           hipStream_t stream) {
  AllToAllArgs a;
  a.ptrs = ptrs;
  a.n = n;
  a.block = count / static_cast<uint64_t>(n);
  const size_t isz = itemsize(dtype);
  // 16-byte packs need every block start 16-byte aligned as well
  vec = vec && (a.block * isz) % 16 == 0;
  const int pack = vec ? static_cast<int>(16 / isz) : 1;
  const int u = vec ? 2 : 1;
  a.tiles = tiles_for(a.block, pack, u);
  const dim3 grid(grid_x(a.tiles), static_cast<uint32_t>(n * n));
  const void* fn = isz == 2 ? alltoall_fn<uint16_t>(vec) : alltoall_fn<uint32_t>(vec);
  return launch(fn, grid, a, stream);
}

hipError_t launch_fanout(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                         bool from_root, int root, bool vec, hipStream_t stream) {
  FanoutArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.chunk = chunk_size(n, count);
  a.n = n;
  a.root = from_root ? root : -1;
  const int pack = vec ? static_cast<int>(16 / itemsize(dtype)) : 1;
  const int u = vec ? pick_fanout_unroll(n) : 1;
  a.tiles = tiles_for(a.chunk, pack, u);
  const dim3 grid(grid_x(a.tiles), n);
  const void* fn = itemsize(dtype) == 2 ? fanout_fn<uint16_t>(u, vec) : fanout_fn<uint32_t>(u, vec);
  return launch(fn, grid, a, stream);
}

}  // namespace ar
