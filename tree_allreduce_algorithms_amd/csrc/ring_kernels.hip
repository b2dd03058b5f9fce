// Fused ring fold (ReduceScatter / AllReduce in one pass), gfx950.
//
// For chunk c the ring's ReduceScatter pass starts with rank c+1's value and
// has ranks c+2, ..., c each add their own value to the incoming partial, rank
// c finishing the sum ("Collectives from scratch", two-pass ring: rank r ends
// up owning chunk r).  Doing those N-1 hops for one element in registers
// gives bit-for-bit the value the step-by-step ring leaves in rank c; the
// AllGather pass then only copies it, so AllReduce stores it in every rank.
// (AR_BFLOAT16_ACC32 runs the same hops on float32 partials and rounds once.)
#include "device_common.hpp"

namespace ar {
namespace {

constexpr int kFoldBatch = 8;   // rank loads issued before folding them

struct FoldArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t chunk;
  uint64_t tiles;
  int n;
};

// The fold in registers, one element per lane: the path for rank buffers
// aligned only to the element size (16-byte aligned buffers take the staged
// kernel below).  ALL: store into every rank (AllReduce) or only into the
// chunk's owner (ReduceScatter).
template <ar_dtype_t DT, ar_op_t OP, bool ALL>
__global__ __launch_bounds__(kBlock) void ring_fold_kernel(FoldArgs a) {
  constexpr int U = 1;
  constexpr bool VEC = false;
  using T = typename Elem<DT>::T;
  constexpr int K = PackOf<T, VEC>::K;
  constexpr int B = kFoldBatch;
  using P = typename PackOf<T, VEC>::P;
  using S = Pack<T, 1>;

  const int n = a.n;
  const int c = blockIdx.y;
  const uint64_t lo = umin(static_cast<uint64_t>(c) * a.chunk, a.count);
  const uint64_t hi = umin(lo + a.chunk, a.count);
  if (lo >= hi) return;
  const int first = wrap_rank(c + 1, n);
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t tp = TileGrid<U>::first_pack(s.plo, tile);
    if (tp >= s.phi) break;
    const uint64_t toff = tp * sizeof(P);
    const TileLanes<U, sizeof(P)> ln(tp, s.plo, s.phi);

    using F = Fold<DT, OP, P>;
    typename F::A acc[U];
    for (int k0 = 0; k0 < n; k0 += B) {
      P in[B][U];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (k0 + j < n) {
          const char* src = at(a.ptrs.p[wrap_rank(first + k0 + j, n)], toff);
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (ln.live[u]) in[j][u] = load_stream<P>(src, ln.off[u]);
        }
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (k0 + j < n) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            acc[u] = (k0 + j == 0) ? F::widen(in[j][u]) : F::combine(F::widen(in[j][u]), acc[u]);
        }
      }
    }
    P out[U];
#pragma unroll
    for (int u = 0; u < U; ++u) out[u] = F::narrow(acc[u]);
    if (ALL) {
      for (int r = 0; r < n; ++r) {
        char* dst = at(a.ptrs.p[r], toff);
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (ln.live[u]) store_stream<P>(dst, ln.off[u], out[u]);
      }
    } else {
      char* dst = at(a.ptrs.p[c], toff);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ln.live[u]) store_stream<P>(dst, ln.off[u], out[u]);
    }
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    using FS = Fold<DT, OP, S>;
    const uint64_t e = s.scalar_index(threadIdx.x);
    typename FS::A acc = FS::widen(load<S>(a.ptrs.p[first], e));
    for (int k = 1; k < n; ++k)
      acc = FS::combine(FS::widen(load<S>(a.ptrs.p[wrap_rank(first + k, n)], e)), acc);
    const S out = FS::narrow(acc);
    if (ALL) {
      for (int r = 0; r < n; ++r) store<S>(a.ptrs.p[r], e, out);
    } else {
      store<S>(a.ptrs.p[c], e, out);
    }
  }
}

// The same fold through staged tiles (16-byte packs only).  LDS slot s holds
// ring position s of the fold (rank c+1+s), M runs of 64 packs each; each
// thread folds whole 32-bit words of the tile's columns (the hops above, on
// the word's one or two elements) in slot order, and the results go to every
// rank (ALL) or to rank c.  More than kStageGroup ranks are staged in groups
// of equal size, each thread carrying its partials in registers.
// The blocks take the chunks one after another (blockIdx.y is the chunk), or
// with PAIRS two chunks at a time: block b of a one-dimensional grid is tile
// (b mod 2T) / 2 of chunk 2 (b / 2T) + b mod 2, T = a.tiles, one tile each;
// with N odd the last chunk runs alone, block b being its tile b mod 2T (see
// fold_in_pairs).
template <ar_dtype_t DT, ar_op_t OP, bool ALL, int NMAX, bool PAIRS>
__global__ __launch_bounds__(kBlock) void ring_stage_kernel(FoldArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int K = 16 / sizeof(T);
  constexpr int M = stage_runs(NMAX);
  constexpr int TP = kRun * M;
  constexpr int G = stage_slots(NMAX);
  using WP = Pack<T, 4 / sizeof(T)>;
  using S = Pack<T, 1>;
  using F = Fold<DT, OP, WP>;
  extern __shared__ Raw16 stage[];

  const int n = a.n;
  int c;
  uint64_t tile0, tstride;
  if constexpr (PAIRS) {
    const uint32_t per_pair = 2u * static_cast<uint32_t>(a.tiles);
    const uint32_t pair = blockIdx.x / per_pair;
    const uint32_t rem = blockIdx.x - pair * per_pair;
    const bool alone = 2u * pair + 1u >= static_cast<uint32_t>(n);
    c = static_cast<int>(alone ? 2u * pair : 2u * pair + (rem & 1u));
    tile0 = alone ? rem : rem >> 1;
    tstride = a.tiles;
  } else {
    c = static_cast<int>(blockIdx.y);
    tile0 = blockIdx.x;
    tstride = gridDim.x;
  }
  const uint64_t lo = umin(static_cast<uint64_t>(c) * a.chunk, a.count);
  const uint64_t hi = umin(lo + a.chunk, a.count);
  if (lo >= hi) return;
  const int first = wrap_rank(c + 1, n);
  const Span s = make_span<K>(lo, hi);
  Raw16* res = stage + stage_slots(n) * TP;   // the layout stage_bytes(n) allocates
  // groups of equal size (at most G): 33 ranks go as 17 + 16, not 32 + 1
  const int groups = (n + G - 1) / G;
  const int gsize = (n + groups - 1) / groups;

  for (uint64_t tile = tile0; tile < a.tiles; tile += tstride) {
    const uint64_t tp0 = (s.plo / TP + tile) * TP;
    if (tp0 >= s.phi || s.plo >= s.phi) break;
    const StageTile t{tp0, s.plo, s.phi};
    typename F::A acc[M];
    for (int g0 = 0; g0 < n; g0 += gsize) {
      const int slots = n - g0 < gsize ? n - g0 : gsize;
      stage_in<G, M>(a.ptrs, slots, t, RingSlot{first, g0, n}, stage);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int it = static_cast<int>(threadIdx.x) + i * kBlock;
        const uint64_t col = tp0 + (it >> 2);
        if (col >= s.plo && col < s.phi) {
          const StageWord<WP, M> word{reinterpret_cast<const uint32_t*>(stage), it};
          int k = 0;
          if (g0 == 0) {
            acc[i] = F::widen(word(0));
            k = 1;
          }
          for (; k < slots; ++k) acc[i] = F::combine(F::widen(word(k)), acc[i]);
          if (g0 + slots == n)
            reinterpret_cast<uint32_t*>(res)[it] = __builtin_bit_cast(uint32_t, F::narrow(acc[i]));
        }
      }
      // orders this group's reads of the stage before the next group's
      // loads overwrite it, and the results before the stores read them
      __syncthreads();
    }
    // (the next tile's first barrier orders these reads of res before its
    // fold overwrites them)
    if (ALL)
      stage_out<NMAX, M>(a.ptrs, 0, n, t, res);
    else
      stage_out<1, M>(a.ptrs, c, c + 1, t, res);
  }

  if (tile0 == 0 && threadIdx.x < s.scalar_count()) {
    using FS = Fold<DT, OP, S>;
    const uint64_t e = s.scalar_index(threadIdx.x);
    typename FS::A acc = FS::widen(load<S>(a.ptrs.p[first], e));
    for (int k = 1; k < n; ++k)
      acc = FS::combine(FS::widen(load<S>(a.ptrs.p[wrap_rank(first + k, n)], e)), acc);
    const S out = FS::narrow(acc);
    if (ALL) {
      for (int r = 0; r < n; ++r) store<S>(a.ptrs.p[r], e, out);
    } else {
      store<S>(a.ptrs.p[c], e, out);
    }
  }
}

template <ar_dtype_t DT, ar_op_t OP, bool ALL, bool PAIRS = false>
const void* ring_stage_fn(int n) {
  if (n <= 2) return reinterpret_cast<const void*>(&ring_stage_kernel<DT, OP, ALL, 2, PAIRS>);
  if (n <= 4) return reinterpret_cast<const void*>(&ring_stage_kernel<DT, OP, ALL, 4, PAIRS>);
  if (n <= 8) return reinterpret_cast<const void*>(&ring_stage_kernel<DT, OP, ALL, 8, PAIRS>);
  if (n <= 16) return reinterpret_cast<const void*>(&ring_stage_kernel<DT, OP, ALL, 16, PAIRS>);
  if (n <= 32) return reinterpret_cast<const void*>(&ring_stage_kernel<DT, OP, ALL, 32, PAIRS>);
  return reinterpret_cast<const void*>(&ring_stage_kernel<DT, OP, ALL, AR_MAX_RANKS, PAIRS>);
}

// Whether the one-pass AllReduce deals its blocks over two chunks at a time.
// Chunk after chunk, the blocks in flight read and write one narrow stretch
// of each of the N buffers; over all N chunks at once (tiles dealt round the
// chunks), N stretches of each.  Measured on gfx950 (in-process A/B, three
// processes, float32 unless noted), two chunks at a time against one: N=8 x
// 1.2 GB -0.5 to -1.1 %, N=8 x 600 MB bfloat16 -2 to -3 %, N=8 x 512 MiB -1
// to -7 %, N=10 x 480 MB -1.4 to -2.4 %, N=16 x 600 MB -2.4 %, N=4 x 2.4 GB
// -2 %, N=2 x 4.8 GB -2.3 %; but N=4 x 256 MiB +9 %, N=6-8 at 64-256 MiB +2
// to +5 %, N=8 x 26 MB +0.4 to +2.4 %, and every chunk at once N=8 x 1.2 GB
// +5 %, the ReduceScatter +4 to +12 %.  So pairs from 384 MiB per rank,
// AllReduce only.
inline bool fold_in_pairs(bool all, uint64_t count, size_t isz) {
  return all && count * isz >= (384ull << 20);
}

template <ar_dtype_t DT, ar_op_t OP>
hipError_t ring_fold_typed(FoldArgs a, bool all, bool vec, hipStream_t stream) {
  constexpr int K = 16 / sizeof(typename Elem<DT>::T);
  if (vec && stage_ring(a.n)) {
    a.tiles = stage_tiles_for(a.chunk, K, stage_runs(a.n));
    const uint64_t pair_blocks = static_cast<uint64_t>(a.n) * a.tiles;
    if (fold_in_pairs(all, a.count, sizeof(typename Elem<DT>::T)) && pair_blocks <= kMaxGridX) {
      return launch(ring_stage_fn<DT, OP, true, true>(a.n), dim3(static_cast<uint32_t>(pair_blocks)), a,
                    stream, stage_bytes(a.n));
    }
    const dim3 grid(grid_x(a.tiles), a.n);
    const void* fn = all ? ring_stage_fn<DT, OP, true>(a.n) : ring_stage_fn<DT, OP, false>(a.n);
    return launch(fn, grid, a, stream, stage_bytes(a.n));
  }
  a.tiles = tiles_for(a.chunk, 1, 1);
  const dim3 grid(grid_x(a.tiles), a.n);
  return launch(all ? reinterpret_cast<const void*>(&ring_fold_kernel<DT, OP, true>)
                    : reinterpret_cast<const void*>(&ring_fold_kernel<DT, OP, false>),
                grid, a, stream);
}

}  // namespace

hipError_t launch_ring_fold(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                            ar_op_t op, bool all_ranks, bool vec, hipStream_t stream) {
  FoldArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.chunk = chunk_size(n, count);
  a.n = n;
  a.tiles = 0;
  AR_DISPATCH_FOLD(ring_fold_typed, dtype, op, a, all_ranks, vec, stream);
}

}  // namespace ar
