// Device-side building blocks shared by the collective kernels (gfx950).
//
// All of the work is streaming: every kernel reads each input element once
// and writes each output element once, so HBM bandwidth bounds everything and
// no matrix cores are involved.  Common structure:
//
// * A kernel processes "segments" (a ring chunk, a tree's half, a transfer's
//   element range), one per blockIdx.y.  Within a segment, elements are
//   grouped into 16-byte packs aligned to the element index (every rank
//   buffer is 16-byte aligned when these kernels run, so a pack maps to one
//   dwordx4 access in every buffer).  Packs are split into tiles of
//   kBlock * U packs; a block walks tiles blockIdx.x, blockIdx.x + gridDim.x,
//   ...  The unaligned head and tail of a segment (fewer than one pack each)
//   are handled element by element by block x == 0.
// * Everything about which rank to read or write is uniform per block (the
//   segment fixes it).  A tile's byte offset is uniform too, so rank pointer
//   plus tile offset sits in scalar registers and each lane adds only a
//   32-bit offset below 64 KiB: one VGPR of addressing per pack instead of a
//   64-bit address per (rank, pack).
// * Each element is owned by exactly one thread (or, in the staged folds
//   below, one block), which reads all the values it needs before writing
//   any of them, so the in-place updates never race.
//
// Arithmetic of one hop is `local (+) incoming` at the receiving rank
// (Lecture 09 section 7.1 and Chapter 4 section 4.3.1 update the receiver's
// own chunk in place): int32 wraps, float32 is one IEEE operation (built with
// -ffp-contract=off, subnormals kept), bfloat16 widens to float32, applies
// the operation and rounds back to nearest-even after every hop.
#pragma once

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>

#include "kernels.hpp"

namespace ar {
namespace {

constexpr int kBlock = 256;
constexpr uint32_t kMaxGridX = 1u << 22;   // grid-stride loops cover any excess

template <ar_dtype_t DT> struct Elem;
template <> struct Elem<AR_INT32> { using T = int32_t; };
template <> struct Elem<AR_FLOAT32> { using T = float; };
template <> struct Elem<AR_BFLOAT16> { using T = uint16_t; };
template <> struct Elem<AR_BFLOAT16_ACC32> { using T = uint16_t; };

__device__ __forceinline__ float bf16_widen(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16 bits, round to nearest, ties to even.  gfx950 converts
// in one instruction (v_cvt_pk_bf16_f32, which rounds by the current mode:
// nearest-even).
__device__ __forceinline__ uint16_t bf16_round(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f));
}

using F32x2 = float __attribute__((ext_vector_type(2)));
using BF16x2 = __bf16 __attribute__((ext_vector_type(2)));

// Two float32 values -> two bfloat16 in one 32-bit word (lo in bits 0-15).
__device__ __forceinline__ uint32_t bf16x2_round(float lo, float hi) {
  const F32x2 v = {lo, hi};
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, BF16x2));
}

template <ar_dtype_t DT, ar_op_t OP> struct Combine;

template <ar_op_t OP> struct Combine<AR_INT32, OP> {
  static __device__ __forceinline__ int32_t apply(int32_t local, int32_t in) {
    if constexpr (OP == AR_SUM)
      return static_cast<int32_t>(static_cast<uint32_t>(local) + static_cast<uint32_t>(in));
    else if constexpr (OP == AR_PROD)
      return static_cast<int32_t>(static_cast<uint32_t>(local) * static_cast<uint32_t>(in));
    else if constexpr (OP == AR_MAX)
      return in > local ? in : local;
    else
      return in < local ? in : local;
  }
};

template <ar_op_t OP> struct Combine<AR_FLOAT32, OP> {
  static __device__ __forceinline__ float apply(float local, float in) {
    if constexpr (OP == AR_SUM)
      return local + in;
    else if constexpr (OP == AR_PROD)
      return local * in;
    else if constexpr (OP == AR_MAX)
      return in > local ? in : local;
    else
      return in < local ? in : local;
  }
};

template <ar_op_t OP> struct Combine<AR_BFLOAT16, OP> {
  static __device__ __forceinline__ uint16_t apply(uint16_t local, uint16_t in) {
    const float a = bf16_widen(local);
    const float b = bf16_widen(in);
    if constexpr (OP == AR_SUM)
      return bf16_round(a + b);
    else if constexpr (OP == AR_PROD)
      return bf16_round(a * b);
    else if constexpr (OP == AR_MAX)
      return b > a ? in : local;
    else
      return b < a ? in : local;
  }
};

// K elements moved as one aligned access (K * sizeof(T) == 16 -> dwordx4).
template <class T, int K> struct alignas(sizeof(T) * K) Pack {
  T e[K];
};

template <int W> struct Words {
  uint32_t w[W];
};

template <ar_dtype_t DT, ar_op_t OP, class T, int K>
__device__ __forceinline__ Pack<T, K> combine(const Pack<T, K>& local, const Pack<T, K>& in) {
  if constexpr (DT == AR_BFLOAT16 && (OP == AR_SUM || OP == AR_PROD) && K % 2 == 0) {
    // Two bfloat16 per 32-bit word: widening is a shift (low half) or a mask
    // (high half), and one conversion rounds both results.
    const Words<K / 2> lw = __builtin_bit_cast(Words<K / 2>, local);
    const Words<K / 2> iw = __builtin_bit_cast(Words<K / 2>, in);
    Words<K / 2> r;
#pragma unroll
    for (int j = 0; j < K / 2; ++j) {
      const float a0 = __uint_as_float(lw.w[j] << 16);
      const float a1 = __uint_as_float(lw.w[j] & 0xffff0000u);
      const float b0 = __uint_as_float(iw.w[j] << 16);
      const float b1 = __uint_as_float(iw.w[j] & 0xffff0000u);
      if constexpr (OP == AR_SUM)
        r.w[j] = bf16x2_round(a0 + b0, a1 + b1);
      else
        r.w[j] = bf16x2_round(a0 * b0, a1 * b1);
    }
    return __builtin_bit_cast(Pack<T, K>, r);
  } else {
    Pack<T, K> r;
#pragma unroll
    for (int j = 0; j < K; ++j) r.e[j] = Combine<DT, OP>::apply(local.e[j], in.e[j]);
    return r;
  }
}

// How a fold accumulates.  Every dtype but AR_BFLOAT16_ACC32 folds in its
// own element type (each hop is `combine`, rounding to that type); for
// AR_BFLOAT16_ACC32 the loaded bfloat16 values are widened to float32, the
// hops are float32 operations, and the result is rounded to bfloat16 once.
// combine(local, incoming) keeps the receiver-side operand order.
template <ar_dtype_t DT, ar_op_t OP, class P> struct Fold {
  using A = P;
  static __device__ __forceinline__ A widen(const P& p) { return p; }
  static __device__ __forceinline__ P narrow(const A& a) { return a; }
  static __device__ __forceinline__ A combine(const A& local, const A& incoming) {
    return ::ar::combine<DT, OP>(local, incoming);
  }
};

template <ar_op_t OP, int K> struct Fold<AR_BFLOAT16_ACC32, OP, Pack<uint16_t, K>> {
  using P = Pack<uint16_t, K>;
  using A = Pack<float, K>;
  static __device__ __forceinline__ A widen(const P& p) {
    A a;
#pragma unroll
    for (int j = 0; j < K; ++j) a.e[j] = bf16_widen(p.e[j]);
    return a;
  }
  static __device__ __forceinline__ P narrow(const A& a) {
    if constexpr (K % 2 == 0) {
      Words<K / 2> w;
#pragma unroll
      for (int j = 0; j < K / 2; ++j) w.w[j] = bf16x2_round(a.e[2 * j], a.e[2 * j + 1]);
      return __builtin_bit_cast(P, w);
    } else {
      P p;
#pragma unroll
      for (int j = 0; j < K; ++j) p.e[j] = bf16_round(a.e[j]);
      return p;
    }
  }
  static __device__ __forceinline__ A combine(const A& local, const A& incoming) {
    return ::ar::combine<AR_FLOAT32, OP>(local, incoming);
  }
};

// Plain element accesses (the unaligned head and tail of a segment).
template <class P> __device__ __forceinline__ P load(const void* base, uint64_t i) {
  return reinterpret_cast<const P*>(base)[i];
}
template <class P> __device__ __forceinline__ void store(void* base, uint64_t i, const P& v) {
  reinterpret_cast<P*>(base)[i] = v;
}

// Streaming 16-byte accesses for the pack paths.  A collective touches every
// byte of every rank buffer once (a read, a write, or a read then a write by
// the same thread), so there is no reuse for L2 to capture; the non-temporal
// hint lets the loads (and the folds' stores) stream past it.  Measured on gfx950 with
// 8 x 1.2 GB buffers, the hint raises a pure read stream from about 6.4 to
// 7.0 TB/s and the 8-rank fold from about 5.2 to 5.5 TB/s.
using Raw16 = uint32_t __attribute__((ext_vector_type(4)));

// `base` is uniform (rank pointer + tile offset); `off` is the lane's byte
// offset inside the tile.
__device__ __forceinline__ const char* at(const void* p, uint64_t byte_off) {
  return static_cast<const char*>(p) + byte_off;
}
__device__ __forceinline__ char* at(void* p, uint64_t byte_off) {
  return static_cast<char*>(p) + byte_off;
}

// 16-byte packs go through the streaming hint; single elements (the path for
// buffers aligned only to the element size) are plain accesses.
template <class P> __device__ __forceinline__ P load_stream(const char* base, uint32_t off) {
  if constexpr (sizeof(P) == 16) {
    const Raw16 v = __builtin_nontemporal_load(reinterpret_cast<const Raw16*>(base + off));
    return __builtin_bit_cast(P, v);
  } else {
    return *reinterpret_cast<const P*>(base + off);
  }
}
template <class P>
__device__ __forceinline__ void store_stream(char* base, uint32_t off, const P& v) {
  if constexpr (sizeof(P) == 16) {
    __builtin_nontemporal_store(__builtin_bit_cast(Raw16, v), reinterpret_cast<Raw16*>(base + off));
  } else {
    *reinterpret_cast<P*>(base + off) = v;
  }
}

// Stores that go through the caches.  The copies (the AllGather and Broadcast
// fan-out, and every step of the literal schedules) write each value they
// read to one or more other buffers; measured on gfx950 they run faster when
// their stores are ordinary write-back stores: the fan-out 4-6 % at N = 8
// and 64, the step AllGather at N = 64 about 30 %.  The folds keep
// store_stream, whose hint measured 6 % faster for them.
template <class P>
__device__ __forceinline__ void store_cached(char* base, uint32_t off, const P& v) {
  *reinterpret_cast<P*>(base + off) = v;
}

// Element type T moved either as 16-byte packs (VEC: every rank buffer is
// 16-byte aligned) or one element at a time (buffers aligned only to the
// element size).  Both paths apply the same per-element arithmetic in the
// same order, so their results are identical.
template <class T, bool VEC> struct PackOf {
  static constexpr int K = VEC ? static_cast<int>(16 / sizeof(T)) : 1;
  using P = Pack<T, K>;
};

// Elements [lo, hi) of a segment split into an element-wise head, whole
// K-element packs [plo, phi) and an element-wise tail.
struct Span {
  uint64_t lo, hi, plo, phi, head_end, tail_begin;
  __device__ uint32_t scalar_count() const {
    return static_cast<uint32_t>((head_end - lo) + (hi - tail_begin));
  }
  __device__ uint64_t scalar_index(uint32_t t) const {
    const uint32_t head = static_cast<uint32_t>(head_end - lo);
    return t < head ? lo + t : tail_begin + (t - head);
  }
};

template <int K> __device__ __forceinline__ Span make_span(uint64_t lo, uint64_t hi) {
  Span s;
  s.lo = lo;
  s.hi = hi;
  s.plo = (lo + K - 1) / K;
  const uint64_t ph = hi / K;
  s.phi = ph > s.plo ? ph : s.plo;
  s.head_end = hi < s.plo * K ? hi : s.plo * K;
  const uint64_t tb = s.phi * K > s.head_end ? s.phi * K : s.head_end;
  s.tail_begin = tb < hi ? tb : hi;
  return s;
}

// Tiles lie on a grid of kBlock * U packs anchored at element 0 of the
// buffer, not at the segment's start: tile t covers packs [t*TP, (t+1)*TP).
// When a segment starts mid-line (a ragged chunk, the second tree half) its
// first and last tiles are partly masked, but every wave still writes whole,
// line-aligned 1 KiB runs.  Anchoring tiles at the segment start instead
// shifts every store off the 128-byte lines, so neighbouring waves each write
// half of the same lines; with streaming stores that measured about 25 % slower
// on a 64-rank AllGather.
template <int U> struct TileGrid {
  static constexpr uint64_t kPacks = static_cast<uint64_t>(kBlock) * U;
  // First pack of the segment's `tile`-th tile (tile counts from the tile
  // holding the segment's first pack).
  static __device__ __forceinline__ uint64_t first_pack(uint64_t plo, uint64_t tile) {
    return (plo / kPacks + tile) * kPacks;
  }
};

// Per-tile lane setup: live[u] says whether the lane's pack u lies inside the
// segment's packs [plo, phi), off[u] is its byte offset inside the tile (PB
// bytes per pack).
template <int U, int PB> struct TileLanes {
  bool live[U];
  uint32_t off[U];
  __device__ TileLanes(uint64_t tile_pack, uint64_t plo, uint64_t phi) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const uint32_t lane_pack = threadIdx.x + static_cast<uint32_t>(u * kBlock);
      const uint64_t p = tile_pack + lane_pack;
      live[u] = p >= plo && p < phi;
      off[u] = lane_pack * static_cast<uint32_t>(PB);
    }
  }
};

// ---------------------------------------------------------------------------
// Staged tiles: the folds' exchange through LDS.
//
// A fold needs the same element of all N ranks before it can write any of
// them.  Loading all N packs in one lane and storing N results from it makes
// every wave alternate N-deep load bursts with N-deep store bursts; measured
// on gfx950 (8 x 1.2 GB float32 AllReduce) that runs at about 70 % of HBM
// peak, while a 1:1 copy with one load and one store per lane reaches 81 %.
// A staged tile spreads the loads over the block's waves instead.  The tile
// is M runs of 64 packs (1 KiB, one wave instruction) of every rank:
//   1. wave w reads the (slot, run) pairs q = w, w + 4, ... (slot q / M,
//      run q % M) into LDS slot q, where a slot is a rank in the fold's order
//      (the ring's positions, the tree's roles);
//   2. after a barrier, each thread folds whole 32-bit words of the tile's
//      columns over the slots in order and, after the last group of slots,
//      leaves the results in LDS;
//   3. after a second barrier, wave w stores the results into the
//      (rank, run) pairs w, w + 4, ... of its destination ranks.
// Same bits as folding in registers; on the same buffers the 8-rank fold
// runs at 75-78 % of peak.  Tiles are anchored at pack 0 of the buffer like
// TileGrid, so every wave still reads and writes whole 1 KiB runs.  M grows
// for small N so that each wave still issues two loads; more than 32 ranks
// are staged 32 (or, for the ring, an equal share) at a time.
// ---------------------------------------------------------------------------
constexpr int kRun = 64;                    // packs per run
constexpr int kStageWaves = kBlock / 64;

// Runs per rank per staged tile for n ranks: at least two (rank, run) pairs
// per wave.
constexpr int stage_runs(int n) { return n <= 2 ? 4 : n <= 4 ? 2 : 1; }

// Ranks staged at once.  A fold of more ranks stages them in groups of this
// many, in the fold's order, each thread carrying its partial in registers
// from group to group.
constexpr int kStageGroup = 32;
constexpr int stage_slots(int n) { return n < kStageGroup ? n : kStageGroup; }

// LDS bytes of a staged tile: one group of rows of M runs, plus M runs of
// results.
inline size_t stage_bytes(int n) {
  return static_cast<size_t>(stage_slots(n) + 1) * stage_runs(n) * kRun * 16;
}

// A value the whole wave agrees on, kept in a scalar register.
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The lane's packs of one staged tile: run m covers packs
// [tp0 + 64 m, tp0 + 64 (m + 1)) of every rank; the segment's whole packs are
// [plo, phi).
struct StageTile {
  uint64_t tp0, plo, phi;
  __device__ uint64_t pack(int m) const { return tp0 + m * kRun + (threadIdx.x & 63); }
  __device__ bool live(int m) const {
    const uint64_t p = pack(m);
    return p >= plo && p < phi;
  }
  // The lane's pack if live, else the segment's first whole pack (a valid
  // address whose value is discarded).
  __device__ uint64_t safe(int m) const { return live(m) ? pack(m) : plo; }
};

// Which rank fills LDS slot s of a staged tile.
struct SlotIsRank {   // slot s holds rank s
  __device__ int operator()(int s) const { return s; }
};
struct RingSlot {     // slot s holds ring position base + s of the fold that starts at `first`
  int first, base, n;
  __device__ int operator()(int s) const {
    const int r = first + base + s;
    return r >= n ? r - n : r;
  }
};

// Phase 1 for a wave holding exactly C (slot, run) pairs: all C loads are
// issued before the first is waited for, with no lane-dependent branch
// between them.
template <int M, int C, class RankOf>
__device__ __forceinline__ void stage_rows(const RankPtrs& ptrs, int w, const StageTile& t,
                                           const RankOf& rank_of, Raw16* stage) {
  const int lane = threadIdx.x & 63;
  Raw16 v[C];
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int q = w + i * kStageWaves;
    v[i] = __builtin_nontemporal_load(reinterpret_cast<const Raw16*>(ptrs.p[rank_of(q / M)]) +
                                      t.safe(q % M));
  }
#pragma unroll
  for (int i = 0; i < C; ++i) {
    const int q = w + i * kStageWaves;
    if (t.live(q % M)) stage[q * kRun + lane] = v[i];
  }
}

template <int M, int C, class RankOf>
__device__ __forceinline__ void stage_rows_upto(int count, const RankPtrs& ptrs, int w,
                                                const StageTile& t, const RankOf& rank_of,
                                                Raw16* stage) {
  if constexpr (C > 0) {
    if (count == C)
      stage_rows<M, C>(ptrs, w, t, rank_of, stage);
    else
      stage_rows_upto<M, C - 1>(count, ptrs, w, t, rank_of, stage);
  }
}

// Phase 1: every (slot, run) pair of slots [0, slots), slots <= SMAX, into
// LDS slot * M + run, slot s read from rank rank_of(s).  The segment must hold
// at least one whole pack.
template <int SMAX, int M, class RankOf>
__device__ __forceinline__ void stage_in(const RankPtrs& ptrs, int slots, const StageTile& t,
                                         const RankOf& rank_of, Raw16* stage) {
  constexpr int R = (SMAX * M + kStageWaves - 1) / kStageWaves;
  const int w = wave_uniform(threadIdx.x >> 6);
  const int pairs = slots * M;
  const int count = w < pairs ? (pairs - w + kStageWaves - 1) / kStageWaves : 0;
  stage_rows_upto<M, R>(count, ptrs, w, t, rank_of, stage);
}

// Phase 3: result run m (res[64 m, 64 m + 64)) into run m of ranks [r0, r1),
// r1 - r0 <= NMAX.
template <int NMAX, int M>
__device__ __forceinline__ void stage_out(const RankPtrs& ptrs, int r0, int r1,
                                          const StageTile& t, const Raw16* res) {
  constexpr int R = (NMAX * M + kStageWaves - 1) / kStageWaves;
  const int lane = threadIdx.x & 63;
  const int w = wave_uniform(threadIdx.x >> 6);
  const int pairs = (r1 - r0) * M;
#pragma unroll
  for (int i = 0; i < R; ++i) {
    const int q = w + i * kStageWaves;
    if (q < pairs && t.live(q % M))
      __builtin_nontemporal_store(res[(q % M) * kRun + lane],
                                  reinterpret_cast<Raw16*>(ptrs.p[r0 + q / M]) + t.pack(q % M));
  }
}

// Phase 2 addressing: in a tile of M runs, thread-word `it` in [0, 256 M) is
// word (it & 3) of column (it >> 2); rank k's copy sits at stage word
// k * 256 M + it, the result at res word it.
template <class WP, int M> struct StageWord {
  const uint32_t* words;
  int it;
  __device__ WP operator()(int rank) const {
    return __builtin_bit_cast(WP, words[rank * (kBlock * M) + it]);
  }
};

__device__ __forceinline__ int wrap_rank(int r, int n) { return r >= n ? r - n : r; }

__device__ __forceinline__ uint64_t umin(uint64_t a, uint64_t b) { return a < b ? a : b; }

// ---------------------------------------------------------------------------
// Host-side launch helpers.
// ---------------------------------------------------------------------------
// Upper bound on the tiles of the buffer-anchored grid that one segment of
// at most max_elems elements touches (its packs plus one partial tile at each
// end).
inline uint64_t tiles_for(uint64_t max_elems, int pack, int unroll) {
  const uint64_t packs = max_elems / pack + 1;
  const uint64_t per_tile = static_cast<uint64_t>(kBlock) * unroll;
  return (packs + per_tile - 1) / per_tile + 1;
}

// Packs per lane per tile of the fan-out copy: `preferred` unless
// AR_TUNE_UNROLL (1, 2 or 4, read at the first launch) overrides it for
// measurements; the choice changes nothing but the pack grouping, never any
// element's arithmetic.  (The folds stage their tiles through LDS and have
// no such choice.)
inline int pick_fanout_unroll(int preferred) {
  static const int forced = [] {
    const char* v = std::getenv("AR_TUNE_UNROLL");
    const int u = v != nullptr ? std::atoi(v) : 0;
    return (u == 1 || u == 2 || u == 4) ? u : 0;
  }();
  return forced != 0 ? forced : preferred;
}

inline uint32_t grid_x(uint64_t tiles) {
  return static_cast<uint32_t>(std::min<uint64_t>(tiles, kMaxGridX));
}

template <class Args>
hipError_t launch(const void* fn, dim3 grid, const Args& args, hipStream_t stream,
                  size_t lds_bytes = 0) {
  Args copy = args;
  void* kargs[] = {&copy};
  return hipLaunchKernel(fn, grid, dim3(kBlock), kargs, lds_bytes, stream);
}

// The folds use staged tiles from 2 ranks up (at most 33 KiB of LDS per
// block).  Measured on gfx950 against folding in registers, float32, about
// 9.6 GB of inputs: ring AllReduce 7-10 % faster at N = 5 to 16,
// ReduceScatter 12 % at 8 and 16 and 6-8 % at 40 to 64 (two groups), double
// tree and Reduce 5-12 % at 3 to 16; within placement noise (+-5 %) at N = 2
// to 4.
inline bool stage_ring(int n) { return n >= 2; }
inline bool stage_tree(int n) { return n >= 2; }

// Tiles of the staged grid (M runs each, anchored at pack 0) that a segment
// of at most max_elems elements touches.
inline uint64_t stage_tiles_for(uint64_t max_elems, int pack, int runs) {
  const uint64_t packs = max_elems / pack + 1;
  const uint64_t per_tile = static_cast<uint64_t>(kRun) * runs;
  return (packs + per_tile - 1) / per_tile + 1;
}

// dtype x op dispatch onto a template taking <ar_dtype_t, ar_op_t>.
// AR_DISPATCH covers the per-hop dtypes (the step kernels);
// AR_DISPATCH_FOLD also covers AR_BFLOAT16_ACC32 (the fused folds).
#define AR_DISPATCH_OPS(FN, DT, OP, ...)                                         \
  switch (OP) {                                                                   \
    case AR_SUM: return FN<DT, AR_SUM>(__VA_ARGS__);                              \
    case AR_PROD: return FN<DT, AR_PROD>(__VA_ARGS__);                            \
    case AR_MAX: return FN<DT, AR_MAX>(__VA_ARGS__);                              \
    case AR_MIN: return FN<DT, AR_MIN>(__VA_ARGS__);                              \
  }

#define AR_DISPATCH(FN, DTYPE, OP, ...)                                          \
  do {                                                                            \
    switch (DTYPE) {                                                              \
      case AR_INT32: AR_DISPATCH_OPS(FN, AR_INT32, OP, __VA_ARGS__) break;        \
      case AR_FLOAT32: AR_DISPATCH_OPS(FN, AR_FLOAT32, OP, __VA_ARGS__) break;    \
      case AR_BFLOAT16: AR_DISPATCH_OPS(FN, AR_BFLOAT16, OP, __VA_ARGS__) break;  \
      default: break;                                                             \
    }                                                                             \
    return hipErrorInvalidValue;                                                  \
  } while (0)

#define AR_DISPATCH_FOLD(FN, DTYPE, OP, ...)                                     \
  do {                                                                            \
    switch (DTYPE) {                                                              \
      case AR_INT32: AR_DISPATCH_OPS(FN, AR_INT32, OP, __VA_ARGS__) break;        \
      case AR_FLOAT32: AR_DISPATCH_OPS(FN, AR_FLOAT32, OP, __VA_ARGS__) break;    \
      case AR_BFLOAT16: AR_DISPATCH_OPS(FN, AR_BFLOAT16, OP, __VA_ARGS__) break;  \
      case AR_BFLOAT16_ACC32:                                                     \
        AR_DISPATCH_OPS(FN, AR_BFLOAT16_ACC32, OP, __VA_ARGS__) break;            \
    }                                                                             \
    return hipErrorInvalidValue;                                                  \
  } while (0)

}  // namespace
}  // namespace ar
