// Copy kernels (gfx950).
//
// Fan-out: AllGather (chunk c comes from rank c, its owner after
// ReduceScatter), Broadcast (every chunk comes from the root) or the double
// tree's broadcast (two chunks, the halves, from the trees' roots: rank 0 and
// rank N-1).  Each element is read from its source rank and written into
// every other rank.
//
// AllToAll: block j of rank i and block i of rank j trade places, one thread
// per pack of the pair, so every off-diagonal element is read once and
// written once and no two threads touch the same location.  The pairs i < j
// are taken two at a time, their tiles dealt alternately.
#include "device_common.hpp"

namespace ar {
namespace {

struct FanoutArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t chunk;
  uint64_t tiles;
  int n;
  int root;     // >= 0: Broadcast
  int halves;   // the double tree's two halves (else AllGather)
};

// The rank chunk c is copied from.
__device__ __forceinline__ int fanout_source(int c, int root, int halves, int n) {
  return root >= 0 ? root : halves ? (c == 0 ? 0 : n - 1) : c;
}

// The fan-out one element per lane: the path for rank buffers aligned only to
// the element size (16-byte aligned buffers take the grouped kernel below).
// blockIdx.y is the chunk.
template <class T>
__global__ __launch_bounds__(kBlock) void fanout_kernel(FanoutArgs a) {
  constexpr int U = 1;
  constexpr bool VEC = false;
  constexpr int K = PackOf<T, VEC>::K;
  using P = typename PackOf<T, VEC>::P;
  using S = Pack<T, 1>;

  const int n = a.n;
  const int c = blockIdx.y;
  const uint64_t lo = umin(static_cast<uint64_t>(c) * a.chunk, a.count);
  const uint64_t hi = umin(lo + a.chunk, a.count);
  if (lo >= hi) return;
  const int src = fanout_source(c, a.root, a.halves, n);
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

// The fan-out for 16-byte packs, in destination passes.  Written as above
// (every block storing its tile into all N-1 other ranks), the blocks in
// flight at any moment write into every rank buffer at once.  Measured on
// gfx950, a write stream spread that way over 63 buffers runs at about 71 %
// of HBM peak where the same bytes written one buffer after another run at
// 78 %, and the fan-out itself ran at 65-68 %.  So the tile slots (a.slots
// per chunk, chunk after chunk) are cut into groups of a.group slots, and
// each group is copied pass by pass: a pass writes every tile of the group
// into one rank, so the blocks in flight together fill one contiguous
// stretch of one buffer.  Within a pass the units are dealt to the XCDs so
// that each XCD writes one contiguous eighth of the group: blocks go to the 8
// XCDs in turn, so unit w of a pass runs on XCD w mod 8 and takes slot
// (w mod 8) * (a.group / 8) + w / 8.  Measured on gfx950, a write stream in
// which every XCD fills its own contiguous range runs at 86 % of HBM peak
// against 77 % when the XCDs interleave tile by tile (the folds, which mix
// reads and writes, measured 4-16 % slower with that order and keep the
// plain one).  Every pass re-reads the group's source tiles: a slot runs on
// the same XCD in every pass, and the group fits in the XCDs' L2, so HBM still
// sees each source byte read once (FETCH_SIZE confirms it).  Unit b of the
// flattened launch is (group, pass, w).
struct FanoutGroupArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t chunk;
  uint32_t slots;   // tile slots per chunk
  uint32_t group;   // tile slots per group (a multiple of 8)
  uint32_t units;   // groups * passes * group
  int n;
  int nchunks;      // n, or 2 for the double tree's halves
  int passes;
  int root;         // >= 0: Broadcast
  int halves;       // the double tree's halves (else AllGather)
  int rotate;       // pass j writes rank src + 1 + j (else rank j, or j + 1 past the root)
};

template <class T, int U, bool NTL, bool NTS>
__global__ __launch_bounds__(kBlock) void fanout_group_kernel(FanoutGroupArgs a) {
  constexpr int K = 16 / sizeof(T);
  using S = Pack<T, 1>;
  const int n = a.n;
  const uint32_t per_group = a.group * static_cast<uint32_t>(a.passes);

  // (the host keeps units + gridDim.x below 2^32)
  for (uint32_t b = blockIdx.x; b < a.units; b += gridDim.x) {
    // the unit's coordinates are wave-uniform; readfirstlane keeps them (and
    // the rank pointers they select) in scalar registers
    const uint32_t g = b / per_group;
    const uint32_t rem = b - g * per_group;
    const int j = wave_uniform(static_cast<int>(rem / a.group));
    const uint32_t w = rem - static_cast<uint32_t>(j) * a.group;
    // the pass's units on XCD w mod 8 take one contiguous eighth of the group
    const uint32_t q = g * a.group + (w % 8) * (a.group / 8) + w / 8;
    const int c = wave_uniform(static_cast<int>(q / a.slots));
    if (c >= a.nchunks) continue;   // padding of the last group
    const uint32_t lt = static_cast<uint32_t>(wave_uniform(static_cast<int>(q - static_cast<uint32_t>(c) * a.slots)));
    const int src = fanout_source(c, a.root, a.halves, n);
    const int dst = a.rotate ? wrap_rank(src + 1 + j, n) : (a.root >= 0 && j >= a.root) ? j + 1 : j;
    if (dst == src) continue;
    const uint64_t lo = umin(static_cast<uint64_t>(c) * a.chunk, a.count);
    const uint64_t hi = umin(lo + a.chunk, a.count);
    if (lo >= hi) continue;
    const Span s = make_span<K>(lo, hi);

    const uint64_t tp = TileGrid<U>::first_pack(s.plo, lt);
    if (tp < s.phi) {
      const uint64_t toff = tp * 16;
      const TileLanes<U, 16> ln(tp, s.plo, s.phi);
      // plain loads, so that the later passes find these lines in L2; with
      // a single pass (two ranks) nothing is read twice and the loads stream
      const char* sp = at(a.ptrs.p[src], toff);
      char* dp = at(a.ptrs.p[dst], toff);
      Raw16 v[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ln.live[u]) {
          const Raw16* ap = reinterpret_cast<const Raw16*>(sp + ln.off[u]);
          v[u] = NTL ? __builtin_nontemporal_load(ap) : *ap;
        }
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (ln.live[u]) {
          Raw16* bp = reinterpret_cast<Raw16*>(dp + ln.off[u]);
          if (NTS)
            __builtin_nontemporal_store(v[u], bp);
          else
            *bp = v[u];
        }
      }
    }

    // the chunk's elements outside whole packs: one unit per chunk (its first
    // slot, in the pass of the rank after the source) copies them everywhere
    if (lt == 0 && dst == wrap_rank(src + 1, n) && threadIdx.x < s.scalar_count()) {
      const uint64_t e = s.scalar_index(threadIdx.x);
      const S v = load<S>(a.ptrs.p[src], e);
      for (int r = 0; r < n; ++r)
        if (r != src) store<S>(a.ptrs.p[r], e, v);
    }
  }
}

// Bytes of source per group (before balancing): 12 MiB, 1.5 MiB of each
// XCD's 4 MiB L2.  Measured on gfx950 against 4, 8 and 16 MiB, balanced and
// not, over AllGathers of 4 to 64 ranks, it was fastest or within the noise
// of the fastest.
constexpr uint64_t kFanoutGroupBytes = 12ull << 20;

// Loads and stores of the grouped fan-out, chosen by measurement on gfx950:
// with two ranks (one pass, nothing read twice) the loads carry the
// non-temporal hint and the stores go through the caches, as in a plain copy;
// with more ranks the loads go through L2 (the later passes re-read them
// there) and the stores carry the non-temporal hint.
struct FanoutFlavour {
  int unroll;
  bool stream_loads;
  bool stream_stores;
};

inline FanoutFlavour fanout_flavour(int n) {
  if (n == 2) return {4, true, false};
  return {2, false, true};
}

template <class T, int U>
const void* fanout_group_fn(bool ntl, bool nts) {
  if (ntl) {
    return nts ? reinterpret_cast<const void*>(&fanout_group_kernel<T, U, true, true>)
               : reinterpret_cast<const void*>(&fanout_group_kernel<T, U, true, false>);
  }
  return nts ? reinterpret_cast<const void*>(&fanout_group_kernel<T, U, false, true>)
             : reinterpret_cast<const void*>(&fanout_group_kernel<T, U, false, false>);
}

template <class T>
const void* fanout_group_fn(int u, bool ntl, bool nts) {
  if (u == 4) return fanout_group_fn<T, 4>(ntl, nts);
  if (u == 2) return fanout_group_fn<T, 2>(ntl, nts);
  return fanout_group_fn<T, 1>(ntl, nts);
}

// AllToAll block swap over the pairs i < j (the diagonal stays in place),
// numbered row by row: p = 0 is (0, 1), then (0, 2), ..., (0, n-1), (1, 2), ...
// Unit u of the flattened launch is tile (u mod 2T) / 2 of pair
// 2 (u / 2T) + u mod 2, T = a.tiles: two pairs at a time, their tiles
// alternating; when the number of pairs is odd the last one runs alone, unit
// u then being its tile u mod 2T.  Measured on gfx950 against one pair at a time (in-process
// A/B): N=8 x 128 MiB -3.6 %, N=8 x 512 MiB -4.4 %, N=16 x 256 MiB -5.2 %;
// four pairs at a time -1 to -4 %, every pair at once +5 to +8 %.
struct AllToAllArgs {
  RankPtrs ptrs;
  uint64_t block;   // elements per block (count / n)
  uint64_t tiles;   // tiles per pair
  uint32_t units;   // pairs times a.tiles
  int n;
};

// The pair (i, j), i < j, numbered p in row order.
__device__ __forceinline__ void alltoall_pair(uint32_t p, int n, int* i, int* j) {
  int r = 0;
  while (p >= static_cast<uint32_t>(n - 1 - r)) {
    p -= static_cast<uint32_t>(n - 1 - r);
    ++r;
  }
  *i = r;
  *j = r + 1 + static_cast<int>(p);
}

template <class T, int U, bool VEC>
__global__ __launch_bounds__(kBlock) void alltoall_kernel(AllToAllArgs a) {
  using P = typename PackOf<T, VEC>::P;
  constexpr int K = PackOf<T, VEC>::K;
  const uint64_t npacks = a.block / K;   // VEC only when K divides the block
  const uint64_t bbytes = a.block * sizeof(T);
  const uint32_t pairs = static_cast<uint32_t>(a.n * (a.n - 1) / 2);
  const uint32_t per_two = 2u * static_cast<uint32_t>(a.tiles);
  // (the host keeps units + gridDim.x below 2^32)
  for (uint32_t unit = blockIdx.x; unit < a.units; unit += gridDim.x) {
    const uint32_t two = unit / per_two;
    const uint32_t rem = unit - two * per_two;
    const bool alone = 2u * two + 1u >= pairs;
    const uint32_t p = wave_uniform(static_cast<int>(alone ? 2u * two : 2u * two + (rem & 1u)));
    int i, j;
    alltoall_pair(p, a.n, &i, &j);
    const uint64_t tile = alone ? rem : (rem >> 1);
    const uint64_t tp = TileGrid<U>::first_pack(0, tile);
    if (tp >= npacks) continue;
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
  const uint64_t pairs = static_cast<uint64_t>(n) * (n - 1) / 2;
  const uint64_t units = pairs * a.tiles;
  // the decode runs in 32 bits: N - 1 halves of one rank's buffer in tiles
  // of at least 1 KiB stay far below 2^32 for buffers that fit in HBM
  if (units + kMaxGridX > UINT32_MAX) return hipErrorInvalidValue;
  a.units = static_cast<uint32_t>(units);
  const void* fn = isz == 2 ? alltoall_fn<uint16_t>(vec) : alltoall_fn<uint32_t>(vec);
  return launch(fn, dim3(grid_x(units)), a, stream);
}

namespace {

// One fan-out launch: `nchunks` chunks of `chunk` elements, chunk c copied
// from fanout_source(c, root, halves, n) into every other rank.
hipError_t launch_fanout_chunks(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                                uint64_t chunk, int nchunks, int root, bool halves, bool vec,
                                hipStream_t stream) {
  if (vec) {
    FanoutGroupArgs a;
    a.ptrs = ptrs;
    a.count = count;
    a.chunk = chunk;
    a.n = n;
    a.nchunks = nchunks;
    a.root = root;
    a.halves = halves ? 1 : 0;
    const FanoutFlavour fl = fanout_flavour(n);
    const int u = pick_fanout_unroll(fl.unroll);
    const int pack = static_cast<int>(16 / itemsize(dtype));
    const uint64_t slots = tiles_for(chunk, pack, u);
    const uint64_t tile_bytes = static_cast<uint64_t>(kBlock) * u * 16;
    const uint64_t all_slots = slots * static_cast<uint64_t>(nchunks);
    // groups of about kFanoutGroupBytes, balanced so that the last one is
    // not mostly padding
    const uint64_t group_max = std::max<uint64_t>(8, kFanoutGroupBytes / tile_bytes / 8 * 8);
    const uint64_t groups = (all_slots + group_max - 1) / group_max;
    const uint64_t group = ((all_slots + groups - 1) / groups + 7) / 8 * 8;
    // A group inside one or two chunks has one source per tile, so pass j can
    // write rank src + 1 + j: n - 1 passes, each one buffer.  A Broadcast
    // (one source for every chunk) always takes that order.  A group over
    // many small chunks of an AllGather or the tree's halves keeps one
    // destination per pass instead: pass j writes rank j, and the tiles whose
    // source is rank j have nothing to do.  (The kernel's other order also
    // skips a root, so either order is valid for any call.)
    a.rotate = (root >= 0 || slots * 2 >= group) ? 1 : 0;
    a.passes = (a.rotate || root >= 0) ? n - 1 : n;
    const uint64_t units = (all_slots + group - 1) / group * group * static_cast<uint64_t>(a.passes);
    // the decode runs in 32 bits; all rank buffers together would have to
    // exceed the GPU's memory many times over to need more (the element
    // path below takes such a call)
    if (units + kMaxGridX <= UINT32_MAX) {
      a.slots = static_cast<uint32_t>(slots);
      a.group = static_cast<uint32_t>(group);
      a.units = static_cast<uint32_t>(units);
      const void* fn = itemsize(dtype) == 2 ? fanout_group_fn<uint16_t>(u, fl.stream_loads, fl.stream_stores)
                                            : fanout_group_fn<uint32_t>(u, fl.stream_loads, fl.stream_stores);
      return launch(fn, dim3(grid_x(units)), a, stream);
    }
  }
  FanoutArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.chunk = chunk;
  a.n = n;
  a.root = root;
  a.halves = halves ? 1 : 0;
  a.tiles = tiles_for(chunk, 1, 1);
  const dim3 grid(grid_x(a.tiles), static_cast<uint32_t>(nchunks));
  const void* fn = itemsize(dtype) == 2 ? reinterpret_cast<const void*>(&fanout_kernel<uint16_t>)
                                        : reinterpret_cast<const void*>(&fanout_kernel<uint32_t>);
  return launch(fn, grid, a, stream);
}

}  // namespace

hipError_t launch_fanout(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                         bool from_root, int root, bool vec, hipStream_t stream) {
  return launch_fanout_chunks(ptrs, n, count, dtype, chunk_size(n, count), n, from_root ? root : -1,
                              false, vec, stream);
}

hipError_t launch_tree_broadcast(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                                 bool vec, hipStream_t stream) {
  return launch_fanout_chunks(ptrs, n, count, dtype, tree_split(count), 2, -1, true, vec, stream);
}

}  // namespace ar
