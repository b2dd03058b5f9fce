// HIP kernels (gfx950) for the ring / tree collectives over N rank buffers
// in one GPU's HBM.
//
// All of the work is streaming: every kernel reads each input element once
// and writes each output element once, so HBM bandwidth bounds everything and
// no matrix cores are involved.  Common structure:
//
// * A kernel processes "segments" (a ring chunk, a tree's half, a transfer's
//   element range), one per blockIdx.y.  Within a segment, elements are
//   grouped into 16-byte packs aligned to the element index (every rank
//   buffer is 16-byte aligned when the fast path is taken, so a pack maps to
//   one dwordx4 access in every buffer).  Packs are split into tiles of
//   kBlock * U packs; a block walks tiles blockIdx.x, blockIdx.x + gridDim.x,
//   ...  The unaligned head and tail of a segment (fewer than one pack each)
//   are handled element by element by block x == 0.
// * Everything about which rank to read or write is uniform per block (the
//   segment fixes it), so rank pointers are loaded from the kernel arguments
//   into scalar registers.
// * Each element is owned by exactly one thread, which reads all the values
//   it needs before writing any of them, so the in-place updates never race.
//
// Arithmetic of one hop is `local (+) incoming` at the receiving rank
// (Lecture 09 section 7.1 and Chapter 4 section 4.3.1 update the receiver's
// own chunk in place): int32 wraps, float32 is one IEEE operation (built with
// -ffp-contract=off, subnormals kept), bfloat16 widens to float32, applies
// the operation and rounds back to nearest-even after every hop.
#include "kernels.hpp"

#include <algorithm>

namespace ar {
namespace {

constexpr int kBlock = 256;
constexpr int kRingUnroll = 2;   // packs per thread per tile in the ring fold
constexpr int kRingBatch = 8;    // rank loads issued before folding them
constexpr int kCopyUnroll = 2;
constexpr int kStepUnroll = 2;
constexpr uint32_t kMaxGridX = 1u << 24;

template <ar_dtype_t DT> struct Elem;
template <> struct Elem<AR_INT32> { using T = int32_t; };
template <> struct Elem<AR_FLOAT32> { using T = float; };
template <> struct Elem<AR_BFLOAT16> { using T = uint16_t; };

__device__ __forceinline__ float bf16_widen(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// float32 -> bfloat16, round to nearest, ties to even.  Adding 0x7FFF plus the
// lowest kept bit carries into the kept half exactly when the dropped half is
// above one half, or equal to it with an odd kept half.  NaN is quieted.
__device__ __forceinline__ uint16_t bf16_round(float f) {
  const uint32_t u = __float_as_uint(f);
  if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x0040u);
  return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
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

template <ar_dtype_t DT, ar_op_t OP, class T, int K>
__device__ __forceinline__ Pack<T, K> combine(const Pack<T, K>& local, const Pack<T, K>& in) {
  Pack<T, K> r;
#pragma unroll
  for (int j = 0; j < K; ++j) r.e[j] = Combine<DT, OP>::apply(local.e[j], in.e[j]);
  return r;
}

template <class P> __device__ __forceinline__ P load(const void* base, uint64_t i) {
  return reinterpret_cast<const P*>(base)[i];
}
template <class P> __device__ __forceinline__ void store(void* base, uint64_t i, const P& v) {
  reinterpret_cast<P*>(base)[i] = v;
}

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

__device__ __forceinline__ int wrap_rank(int r, int n) { return r >= n ? r - n : r; }

__device__ __forceinline__ uint64_t umin(uint64_t a, uint64_t b) { return a < b ? a : b; }

// ---------------------------------------------------------------------------
// Fused ring fold (ReduceScatter / AllReduce in one pass).
//
// For chunk c the ring's ReduceScatter pass starts with rank c+1's value and
// has ranks c+2, ..., c each add their own value to the incoming partial, rank
// c finishing the sum ("Collectives from scratch", two-pass ring: rank r ends
// up owning chunk r).  Doing those N-1 hops for one element in registers
// gives bit-for-bit the value the step-by-step ring leaves in rank c; the
// AllGather pass then only copies it, so AllReduce stores it in every rank.
// ---------------------------------------------------------------------------
struct FoldArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t chunk;
  uint64_t tiles;
  int n;
};

template <ar_dtype_t DT, ar_op_t OP, bool ALL>
__global__ __launch_bounds__(kBlock) void ring_fold_kernel(FoldArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int K = 16 / sizeof(T);
  constexpr int U = kRingUnroll;
  constexpr int B = kRingBatch;
  using P = Pack<T, K>;
  using S = Pack<T, 1>;

  const int n = a.n;
  const int c = blockIdx.y;
  const uint64_t lo = umin(static_cast<uint64_t>(c) * a.chunk, a.count);
  const uint64_t hi = umin(lo + a.chunk, a.count);
  if (lo >= hi) return;
  const int first = wrap_rank(c + 1, n);
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t p0 = s.plo + tile * (kBlock * U) + threadIdx.x;
    if (p0 >= s.phi) break;
    bool live[U];
#pragma unroll
    for (int u = 0; u < U; ++u) live[u] = p0 + u * kBlock < s.phi;

    P acc[U];
    for (int k0 = 0; k0 < n; k0 += B) {
      P in[B][U];
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (k0 + j < n) {
          const void* src = a.ptrs.p[wrap_rank(first + k0 + j, n)];
#pragma unroll
          for (int u = 0; u < U; ++u)
            if (live[u]) in[j][u] = load<P>(src, p0 + u * kBlock);
        }
      }
#pragma unroll
      for (int j = 0; j < B; ++j) {
        if (k0 + j < n) {
#pragma unroll
          for (int u = 0; u < U; ++u)
            acc[u] = (k0 + j == 0) ? in[j][u] : combine<DT, OP>(in[j][u], acc[u]);
        }
      }
    }
    if (ALL) {
      for (int r = 0; r < n; ++r) {
#pragma unroll
        for (int u = 0; u < U; ++u)
          if (live[u]) store<P>(a.ptrs.p[r], p0 + u * kBlock, acc[u]);
      }
    } else {
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (live[u]) store<P>(a.ptrs.p[c], p0 + u * kBlock, acc[u]);
    }
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    S acc = load<S>(a.ptrs.p[first], e);
    for (int k = 1; k < n; ++k)
      acc = combine<DT, OP>(load<S>(a.ptrs.p[wrap_rank(first + k, n)], e), acc);
    if (ALL) {
      for (int r = 0; r < n; ++r) store<S>(a.ptrs.p[r], e, acc);
    } else {
      store<S>(a.ptrs.p[c], e, acc);
    }
  }
}

// ---------------------------------------------------------------------------
// Fused fan-out copy: AllGather (chunk c comes from rank c) or Broadcast
// (every chunk comes from the root).  The chunk split only spreads the work.
// ---------------------------------------------------------------------------
struct FanoutArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t chunk;
  uint64_t tiles;
  int n;
  int root;   // < 0: AllGather
};

template <class T>
__global__ __launch_bounds__(kBlock) void fanout_kernel(FanoutArgs a) {
  constexpr int K = 16 / sizeof(T);
  constexpr int U = kCopyUnroll;
  using P = Pack<T, K>;
  using S = Pack<T, 1>;

  const int n = a.n;
  const int c = blockIdx.y;
  const uint64_t lo = umin(static_cast<uint64_t>(c) * a.chunk, a.count);
  const uint64_t hi = umin(lo + a.chunk, a.count);
  if (lo >= hi) return;
  const int src = a.root < 0 ? c : a.root;
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t p0 = s.plo + tile * (kBlock * U) + threadIdx.x;
    if (p0 >= s.phi) break;
    P v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (p0 + u * kBlock < s.phi) v[u] = load<P>(a.ptrs.p[src], p0 + u * kBlock);
    for (int r = 0; r < n; ++r) {
      if (r == src) continue;
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (p0 + u * kBlock < s.phi) store<P>(a.ptrs.p[r], p0 + u * kBlock, v[u]);
    }
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    const S v = load<S>(a.ptrs.p[src], e);
    for (int r = 0; r < n; ++r)
      if (r != src) store<S>(a.ptrs.p[r], e, v);
  }
}

// ---------------------------------------------------------------------------
// Fused double binomial tree.  Tree 0 owns [0, half) with role == rank, tree 1
// owns [half, count) with role == N-1-rank.  Reduce round k combines role q
// (q mod 2^(k+1) == 0) with role q + 2^k when that role exists: role q keeps
// own (+) incoming.  Doing every round in registers leaves role 0's value,
// which the broadcast rounds would copy to every rank.
// NMAX bounds N at compile time so that the per-role values live in
// statically indexed registers; K is the pack width per role.
// ---------------------------------------------------------------------------
struct TreeArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t half;
  uint64_t tiles;
  int n;
};

template <ar_dtype_t DT, ar_op_t OP, int NMAX, int K>
__global__ __launch_bounds__(kBlock) void tree_fold_kernel(TreeArgs a) {
  using T = typename Elem<DT>::T;
  using P = Pack<T, K>;
  using S = Pack<T, 1>;

  const int n = a.n;
  const int tree = blockIdx.y;
  const uint64_t lo = tree == 0 ? 0 : a.half;
  const uint64_t hi = tree == 0 ? a.half : a.count;
  if (lo >= hi) return;
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t p = s.plo + tile * kBlock + threadIdx.x;
    if (p >= s.phi) break;
    P v[NMAX];
#pragma unroll
    for (int q = 0; q < NMAX; ++q)
      if (q < n) v[q] = load<P>(a.ptrs.p[tree == 0 ? q : n - 1 - q], p);
#pragma unroll
    for (int stride = 1; stride < NMAX; stride *= 2) {
#pragma unroll
      for (int q = 0; q + stride < NMAX; q += 2 * stride)
        if (q + stride < n) v[q] = combine<DT, OP>(v[q], v[q + stride]);
    }
    for (int r = 0; r < n; ++r) store<P>(a.ptrs.p[r], p, v[0]);
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    S v[NMAX];
#pragma unroll
    for (int q = 0; q < NMAX; ++q)
      if (q < n) v[q] = load<S>(a.ptrs.p[tree == 0 ? q : n - 1 - q], e);
#pragma unroll
    for (int stride = 1; stride < NMAX; stride *= 2) {
#pragma unroll
      for (int q = 0; q + stride < NMAX; q += 2 * stride)
        if (q + stride < n) v[q] = combine<DT, OP>(v[q], v[q + stride]);
    }
    for (int r = 0; r < n; ++r) store<S>(a.ptrs.p[r], e, v[0]);
  }
}

// ---------------------------------------------------------------------------
// One schedule step: transfer j (blockIdx.y) moves elements [lo, hi) from
// src[j] to dst[j], combining (reduce steps) or overwriting (copy steps).
// Destinations of one step never overlap and no transfer reads what another
// transfer of the same step writes (a ring step reads chunk c-1 of the rank it
// writes chunk c-2 of ... ; a tree round's receivers and senders are disjoint
// role sets), so one launch per step is race-free.
// ---------------------------------------------------------------------------
struct StepArgs {
  const void* src[AR_MAX_RANKS];
  void* dst[AR_MAX_RANKS];
  uint64_t lo[AR_MAX_RANKS];
  uint64_t hi[AR_MAX_RANKS];
  uint64_t tiles;
};

template <ar_dtype_t DT, ar_op_t OP, bool REDUCE>
__global__ __launch_bounds__(kBlock) void step_kernel(StepArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int K = 16 / sizeof(T);
  constexpr int U = kStepUnroll;
  using P = Pack<T, K>;
  using S = Pack<T, 1>;

  const int j = blockIdx.y;
  const uint64_t lo = a.lo[j];
  const uint64_t hi = a.hi[j];
  if (lo >= hi) return;
  const void* src = a.src[j];
  void* dst = a.dst[j];
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t p0 = s.plo + tile * (kBlock * U) + threadIdx.x;
    if (p0 >= s.phi) break;
    P in[U];
    P own[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (p0 + u * kBlock < s.phi) {
        in[u] = load<P>(src, p0 + u * kBlock);
        if (REDUCE) own[u] = load<P>(dst, p0 + u * kBlock);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (p0 + u * kBlock < s.phi)
        store<P>(dst, p0 + u * kBlock, REDUCE ? combine<DT, OP>(own[u], in[u]) : in[u]);
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    const S in = load<S>(src, e);
    store<S>(dst, e, REDUCE ? combine<DT, OP>(load<S>(dst, e), in) : in);
  }
}

// ---------------------------------------------------------------------------
// Host-side launch helpers.
// ---------------------------------------------------------------------------
uint64_t tiles_for(uint64_t max_elems, int pack, int unroll) {
  const uint64_t packs = max_elems / pack + 1;
  const uint64_t per_tile = static_cast<uint64_t>(kBlock) * unroll;
  return std::max<uint64_t>(1, (packs + per_tile - 1) / per_tile);
}

uint32_t grid_x(uint64_t tiles) {
  return static_cast<uint32_t>(std::min<uint64_t>(tiles, kMaxGridX));
}

template <class Args>
hipError_t launch(const void* fn, dim3 grid, const Args& args, hipStream_t stream) {
  Args copy = args;
  void* kargs[] = {&copy};
  return hipLaunchKernel(fn, grid, dim3(kBlock), kargs, 0, stream);
}

template <ar_dtype_t DT, ar_op_t OP>
hipError_t ring_fold_typed(const FoldArgs& a, bool all, hipStream_t stream) {
  const dim3 grid(grid_x(a.tiles), a.n);
  if (all) return launch(reinterpret_cast<const void*>(&ring_fold_kernel<DT, OP, true>), grid, a, stream);
  return launch(reinterpret_cast<const void*>(&ring_fold_kernel<DT, OP, false>), grid, a, stream);
}

template <ar_dtype_t DT, ar_op_t OP>
hipError_t tree_fold_typed(const TreeArgs& a, hipStream_t stream) {
  using T = typename Elem<DT>::T;
  constexpr int K = 16 / sizeof(T);
  TreeArgs b = a;
  const uint64_t longest = a.half;   // tree 0's half is never the shorter one
  if (a.n <= 8) {
    b.tiles = tiles_for(longest, K, 1);
    return launch(reinterpret_cast<const void*>(&tree_fold_kernel<DT, OP, 8, K>),
                  dim3(grid_x(b.tiles), 2), b, stream);
  }
  b.tiles = tiles_for(longest, 1, 1);
  return launch(reinterpret_cast<const void*>(&tree_fold_kernel<DT, OP, AR_MAX_RANKS, 1>),
                dim3(grid_x(b.tiles), 2), b, stream);
}

template <ar_dtype_t DT, ar_op_t OP>
hipError_t step_typed(const StepArgs& a, int nxfers, bool reduce, hipStream_t stream) {
  const dim3 grid(grid_x(a.tiles), nxfers);
  if (reduce) return launch(reinterpret_cast<const void*>(&step_kernel<DT, OP, true>), grid, a, stream);
  return launch(reinterpret_cast<const void*>(&step_kernel<DT, AR_SUM, false>), grid, a, stream);
}

// dtype x op dispatch onto a template taking <ar_dtype_t, ar_op_t>.
#define AR_DISPATCH(FN, DTYPE, OP, ...)                                          \
  do {                                                                            \
    switch (DTYPE) {                                                              \
      case AR_INT32:                                                              \
        switch (OP) {                                                             \
          case AR_SUM: return FN<AR_INT32, AR_SUM>(__VA_ARGS__);                  \
          case AR_PROD: return FN<AR_INT32, AR_PROD>(__VA_ARGS__);                \
          case AR_MAX: return FN<AR_INT32, AR_MAX>(__VA_ARGS__);                  \
          case AR_MIN: return FN<AR_INT32, AR_MIN>(__VA_ARGS__);                  \
        }                                                                         \
        break;                                                                    \
      case AR_FLOAT32:                                                            \
        switch (OP) {                                                             \
          case AR_SUM: return FN<AR_FLOAT32, AR_SUM>(__VA_ARGS__);                \
          case AR_PROD: return FN<AR_FLOAT32, AR_PROD>(__VA_ARGS__);              \
          case AR_MAX: return FN<AR_FLOAT32, AR_MAX>(__VA_ARGS__);                \
          case AR_MIN: return FN<AR_FLOAT32, AR_MIN>(__VA_ARGS__);                \
        }                                                                         \
        break;                                                                    \
      case AR_BFLOAT16:                                                           \
        switch (OP) {                                                             \
          case AR_SUM: return FN<AR_BFLOAT16, AR_SUM>(__VA_ARGS__);               \
          case AR_PROD: return FN<AR_BFLOAT16, AR_PROD>(__VA_ARGS__);             \
          case AR_MAX: return FN<AR_BFLOAT16, AR_MAX>(__VA_ARGS__);               \
          case AR_MIN: return FN<AR_BFLOAT16, AR_MIN>(__VA_ARGS__);               \
        }                                                                         \
        break;                                                                    \
    }                                                                             \
    return hipErrorInvalidValue;                                                  \
  } while (0)

}  // namespace

hipError_t launch_ring_fold(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                            ar_op_t op, bool all_ranks, hipStream_t stream) {
  FoldArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.chunk = chunk_size(n, count);
  a.n = n;
  a.tiles = tiles_for(a.chunk, static_cast<int>(16 / itemsize(dtype)), kRingUnroll);
  AR_DISPATCH(ring_fold_typed, dtype, op, a, all_ranks, stream);
}

hipError_t launch_fanout(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                         bool from_root, int root, hipStream_t stream) {
  FanoutArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.chunk = chunk_size(n, count);
  a.n = n;
  a.root = from_root ? root : -1;
  const int pack = static_cast<int>(16 / itemsize(dtype));
  a.tiles = tiles_for(a.chunk, pack, kCopyUnroll);
  const dim3 grid(grid_x(a.tiles), n);
  if (itemsize(dtype) == 2)
    return launch(reinterpret_cast<const void*>(&fanout_kernel<uint16_t>), grid, a, stream);
  return launch(reinterpret_cast<const void*>(&fanout_kernel<uint32_t>), grid, a, stream);
}

hipError_t launch_tree_fold(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                            ar_op_t op, hipStream_t stream) {
  TreeArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.half = tree_split(count);
  a.n = n;
  a.tiles = 0;
  AR_DISPATCH(tree_fold_typed, dtype, op, a, stream);
}

hipError_t launch_step(const RankPtrs& ptrs, const Step& step, ar_dtype_t dtype, ar_op_t op,
                       hipStream_t stream) {
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
  a.tiles = tiles_for(longest, static_cast<int>(16 / itemsize(dtype)), kStepUnroll);
  AR_DISPATCH(step_typed, dtype, op, a, nx, step.reduce, stream);
}

}  // namespace ar
