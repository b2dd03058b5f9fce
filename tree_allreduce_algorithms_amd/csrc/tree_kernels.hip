// Fused binomial-tree folds (gfx950): the double-tree AllReduce and the
// Reduce to one root.
#include "device_common.hpp"

namespace ar {
namespace {

// ---------------------------------------------------------------------------
// Fused double binomial tree.  Tree 0 owns [0, half) with role == rank, tree 1
// owns [half, count) with role == N-1-rank.  Reduce round k combines role q
// (q mod 2^(k+1) == 0) with role q + 2^k when that role exists: role q keeps
// own (+) incoming.  Doing every round in registers leaves role 0's value,
// which the broadcast rounds would copy to every rank.
//
// The rounds are evaluated while streaming the roles in order 0, 1, ..., N-1,
// like a binary counter: slot[l] holds the combined value of the latest
// complete block of 2^l roles.  Role q arrives as a block of one; while bit l
// of q is set, the block in slot[l] (lower roles, the receiving side) absorbs
// it: cur = slot[l] (+) cur.  After role N-1 the occupied slots are the set
// bits of N, and the reduce rounds combine them from the smallest block (the
// highest roles) upward, each larger block receiving the result.  This is
// exactly the pairing of the rounds above, with log2(N) + 1 values live
// instead of N.  Roles are loaded in batches of kTreeBatch so that many loads
// are in flight before the first combine.
// ---------------------------------------------------------------------------
struct TreeArgs {
  RankPtrs ptrs;
  uint64_t count;
  uint64_t half;
  uint64_t tiles;
  int n;
  int root;       // >= 0: Reduce to `root` (one tree over the whole buffer)
  int to_roots;   // double tree: store each tree's result into its root only
};

constexpr int kTreeBatch = 8;

constexpr int ilog2_ceil(int v) { return v <= 1 ? 0 : 1 + ilog2_ceil((v + 1) / 2); }

// The rank that plays `role` in tree 0 (role == rank), tree 1 (N-1-role) or,
// for a Reduce (root >= 0), the tree on roles (rank - root) mod N.
__device__ __forceinline__ int tree_role_rank(int role, int tree, int root, int n) {
  return root >= 0 ? wrap_rank(role + root, n) : (tree == 0 ? role : n - 1 - role);
}

// The ranks [lo, hi) that receive tree `tree`'s result: the root of a Reduce,
// the tree's own root (role 0) when the double tree stores into its roots
// only, every rank otherwise.
struct OutRanks {
  int lo, hi;
  __device__ OutRanks(const TreeArgs& a, int tree) {
    if (a.root >= 0 || a.to_roots) {
      lo = tree_role_rank(0, tree, a.root, a.n);
      hi = lo + 1;
    } else {
      lo = 0;
      hi = a.n;
    }
  }
};

// The binary counter over roles 0, 1, ..., N-1 described above, for U values
// per role.  push() takes the roles in order; its role must be a compile-time
// constant after unrolling at the call site, so that the bit tests and the
// slot indices resolve at compile time and the slots stay in registers.
template <ar_dtype_t DT, ar_op_t OP, int NMAX, int U, class P> struct TreeCounter {
  using F = Fold<DT, OP, P>;
  using A = typename F::A;
  static constexpr int L = ilog2_ceil(NMAX) + 1;
  A slot[L][U];

  __device__ __forceinline__ void push(int q, const P (&in)[U]) {
    A cur[U];
#pragma unroll
    for (int u = 0; u < U; ++u) cur[u] = F::widen(in[u]);
    int l = 0;
#pragma unroll
    for (int bit = 0; bit < L; ++bit) {
      if (((q >> bit) & 1) == 0) break;
#pragma unroll
      for (int u = 0; u < U; ++u) cur[u] = F::combine(slot[bit][u], cur[u]);
      l = bit + 1;
    }
#pragma unroll
    for (int ll = 0; ll < L; ++ll)
      if (ll == l) {
#pragma unroll
        for (int u = 0; u < U; ++u) slot[ll][u] = cur[u];
      }
  }

  // After roles 0..n-1: the occupied slots are the set bits of n; combine
  // them from the smallest block upward, each larger block receiving.
  __device__ __forceinline__ void finish(int n, P (&out)[U]) const {
    A res[U];
    bool have = false;
#pragma unroll
    for (int l = 0; l < L; ++l) {
      if ((n >> l) & 1) {
#pragma unroll
        for (int u = 0; u < U; ++u) res[u] = have ? F::combine(slot[l][u], res[u]) : slot[l][u];
        have = true;
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) out[u] = F::narrow(res[u]);
  }
};

// Folds U packs of every role of one tree; load(rank, u) loads rank's pack u.
// Roles are loaded in batches of kTreeBatch so that many loads are in flight
// before the first combine.
template <ar_dtype_t DT, ar_op_t OP, int NMAX, int U, class P, class Load>
__device__ __forceinline__ void tree_fold_values(int n, int tree, int root, const Load& load,
                                                 P (&out)[U]) {
  TreeCounter<DT, OP, NMAX, U, P> tc;
#pragma unroll
  for (int q0 = 0; q0 < NMAX; q0 += kTreeBatch) {
    if (q0 >= n) break;
    P in[kTreeBatch][U];
#pragma unroll
    for (int j = 0; j < kTreeBatch; ++j) {
      const int q = q0 + j;
      if (q < n) {
        const int rank = tree_role_rank(q, tree, root, n);
#pragma unroll
        for (int u = 0; u < U; ++u) in[j][u] = load(rank, u);
      }
    }
#pragma unroll
    for (int j = 0; j < kTreeBatch; ++j) {
      const int q = q0 + j;   // compile-time after unrolling
      if (q < n) tc.push(q, in[j]);
    }
  }
  tc.finish(n, out);
}

// The folds in registers, one element per lane: the path for rank buffers
// aligned only to the element size (16-byte aligned buffers take the staged
// kernel below).
template <ar_dtype_t DT, ar_op_t OP, int NMAX>
__global__ __launch_bounds__(kBlock) void tree_fold_kernel(TreeArgs a) {
  constexpr bool VEC = false;
  constexpr int U = 1;
  using T = typename Elem<DT>::T;
  constexpr int K = PackOf<T, VEC>::K;
  using P = typename PackOf<T, VEC>::P;
  using S = Pack<T, 1>;

  const int n = a.n;
  const int tree = blockIdx.y;
  const int root = a.root;
  const uint64_t lo = (root >= 0 || tree == 0) ? 0 : a.half;
  const uint64_t hi = (root >= 0 || tree != 0) ? a.count : a.half;
  if (lo >= hi) return;
  const Span s = make_span<K>(lo, hi);

  for (uint64_t tile = blockIdx.x; tile < a.tiles; tile += gridDim.x) {
    const uint64_t tp = TileGrid<U>::first_pack(s.plo, tile);
    if (tp >= s.phi) break;
    const uint64_t toff = tp * sizeof(P);
    const TileLanes<U, sizeof(P)> ln(tp, s.plo, s.phi);
    P v[U];
    tree_fold_values<DT, OP, NMAX, U, P>(
        n, tree, root,
        [&](int rank, int u) {
          return ln.live[u] ? load_stream<P>(at(a.ptrs.p[rank], toff), ln.off[u]) : P{};
        },
        v);
    const OutRanks out(a, tree);
    for (int r = out.lo; r < out.hi; ++r) {
      char* dst = at(a.ptrs.p[r], toff);
#pragma unroll
      for (int u = 0; u < U; ++u)
        if (ln.live[u]) store_stream<P>(dst, ln.off[u], v[u]);
    }
  }

  if (blockIdx.x == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    S v[1];
    tree_fold_values<DT, OP, NMAX, 1, S>(
        n, tree, root, [&](int rank, int) { return load<S>(a.ptrs.p[rank], e); }, v);
    const OutRanks out(a, tree);
    for (int r = out.lo; r < out.hi; ++r) store<S>(a.ptrs.p[r], e, v[0]);
  }
}

// Slot s of a staged tree group holds role base + s.
struct TreeSlot {
  int base, tree, root, n;
  __device__ int operator()(int s) const { return tree_role_rank(base + s, tree, root, n); }
};

// The same folds through staged tiles (16-byte packs only): the block stages
// M runs of 64 packs of each role in LDS, a group of kStageGroup roles at a
// time (roles 0-31, then 32-63), each thread pushes whole 32-bit words of the
// tile's columns through the counter above in role order, and the results go
// to every rank (double tree), to the tree's root (double tree, to_roots) or
// to the root (Reduce).  blockIdx.y is the tree, or with HALVES (double tree
// only) the blocks of a one-dimensional grid alternate between the two
// trees: block b is tile b / 2 of tree b mod 2 (see interleave_halves).
template <ar_dtype_t DT, ar_op_t OP, int NMAX, bool HALVES>
__global__ __launch_bounds__(kBlock) void tree_stage_kernel(TreeArgs a) {
  using T = typename Elem<DT>::T;
  constexpr int K = 16 / sizeof(T);
  constexpr int M = stage_runs(NMAX);
  constexpr int TP = kRun * M;
  constexpr int G = stage_slots(NMAX);
  using WP = Pack<T, 4 / sizeof(T)>;
  using S = Pack<T, 1>;
  extern __shared__ Raw16 stage[];

  const int n = a.n;
  const int tree = HALVES ? static_cast<int>(blockIdx.x & 1u) : static_cast<int>(blockIdx.y);
  const uint64_t tile0 = HALVES ? (blockIdx.x >> 1) : blockIdx.x;
  const uint64_t tstride = HALVES ? (gridDim.x >> 1) : gridDim.x;
  const int root = a.root;
  const uint64_t lo = (root >= 0 || tree == 0) ? 0 : a.half;
  const uint64_t hi = (root >= 0 || tree != 0) ? a.count : a.half;
  if (lo >= hi) return;
  const Span s = make_span<K>(lo, hi);
  Raw16* res = stage + stage_slots(n) * TP;   // the layout stage_bytes(n) allocates

  for (uint64_t tile = tile0; tile < a.tiles; tile += tstride) {
    const uint64_t tp0 = (s.plo / TP + tile) * TP;
    if (tp0 >= s.phi || s.plo >= s.phi) break;
    const StageTile t{tp0, s.plo, s.phi};
    TreeCounter<DT, OP, NMAX, 1, WP> tc[M];
#pragma unroll
    for (int g0 = 0; g0 < NMAX; g0 += G) {
      if (g0 >= n) break;
      const int slots = n - g0 < G ? n - g0 : G;
      stage_in<G, M>(a.ptrs, slots, t, TreeSlot{g0, tree, root, n}, stage);
      __syncthreads();
#pragma unroll
      for (int i = 0; i < M; ++i) {
        const int it = static_cast<int>(threadIdx.x) + i * kBlock;
        const uint64_t col = tp0 + (it >> 2);
        if (col >= s.plo && col < s.phi) {
          const StageWord<WP, M> word{reinterpret_cast<const uint32_t*>(stage), it};
#pragma unroll
          for (int j = 0; j < G; ++j) {
            const WP v[1] = {word(j)};
            if (g0 + j < n) tc[i].push(g0 + j, v);   // role compile-time after unrolling
          }
          if (g0 + slots == n) {
            WP out[1];
            tc[i].finish(n, out);
            reinterpret_cast<uint32_t*>(res)[it] = __builtin_bit_cast(uint32_t, out[0]);
          }
        }
      }
      // orders this group's reads of the stage before the next group's
      // loads overwrite it, and the results before the stores read them
      __syncthreads();
    }
    // (the next tile's first barrier orders these reads of res before its
    // fold overwrites them)
    if (root >= 0 || a.to_roots) {
      const int r = tree_role_rank(0, tree, root, n);
      stage_out<1, M>(a.ptrs, r, r + 1, t, res);
    } else {
      stage_out<NMAX, M>(a.ptrs, 0, n, t, res);
    }
  }

  if (tile0 == 0 && threadIdx.x < s.scalar_count()) {
    const uint64_t e = s.scalar_index(threadIdx.x);
    S v[1];
    tree_fold_values<DT, OP, NMAX, 1, S>(
        n, tree, root, [&](int rank, int) { return load<S>(a.ptrs.p[rank], e); }, v);
    const OutRanks out(a, tree);
    for (int r = out.lo; r < out.hi; ++r) store<S>(a.ptrs.p[r], e, v[0]);
  }
}

template <ar_dtype_t DT, ar_op_t OP, bool HALVES = false>
const void* tree_stage_fn(int n) {
  if (n <= 2) return reinterpret_cast<const void*>(&tree_stage_kernel<DT, OP, 2, HALVES>);
  if (n <= 4) return reinterpret_cast<const void*>(&tree_stage_kernel<DT, OP, 4, HALVES>);
  if (n <= 8) return reinterpret_cast<const void*>(&tree_stage_kernel<DT, OP, 8, HALVES>);
  if (n <= 16) return reinterpret_cast<const void*>(&tree_stage_kernel<DT, OP, 16, HALVES>);
  if (n <= 32) return reinterpret_cast<const void*>(&tree_stage_kernel<DT, OP, 32, HALVES>);
  return reinterpret_cast<const void*>(&tree_stage_kernel<DT, OP, AR_MAX_RANKS, HALVES>);
}

// Whether the one-pass double tree runs its two trees' tiles in alternation
// (HALVES) instead of tree 0's half and then tree 1's.  Measured on gfx950
// (in-process A/B against the plain order): N=8 x 1.2 GB float32 even, N=8 x
// 600 MB bfloat16 -2.7 %, N=4 x 2.4 GB -5.7 %, N=8 x 26 MB -0.9 %; the folds
// into the roots of the two-launch double tree +2 % (N=64 x 64 MB).  So the
// one-pass double tree alternates from 384 MiB per rank, as the ring
// AllReduce takes its chunks in pairs there.
inline bool interleave_halves(int root, bool to_roots, uint64_t count, size_t isz) {
  return root < 0 && !to_roots && count * isz >= (384ull << 20);
}

template <ar_dtype_t DT, ar_op_t OP>
const void* tree_fold_fn(int n) {
  if (n <= 8) return reinterpret_cast<const void*>(&tree_fold_kernel<DT, OP, 8>);
  if (n <= 16) return reinterpret_cast<const void*>(&tree_fold_kernel<DT, OP, 16>);
  if (n <= 32) return reinterpret_cast<const void*>(&tree_fold_kernel<DT, OP, 32>);
  return reinterpret_cast<const void*>(&tree_fold_kernel<DT, OP, AR_MAX_RANKS>);
}

template <ar_dtype_t DT, ar_op_t OP>
hipError_t tree_fold_typed(const TreeArgs& a, bool vec, hipStream_t stream) {
  constexpr int K = 16 / sizeof(typename Elem<DT>::T);
  TreeArgs b = a;
  // Reduce: one segment, the whole buffer; double tree: tree 0's half, never
  // the shorter one, bounds both segments.
  const uint64_t longest = a.root >= 0 ? a.count : a.half;
  if (vec && stage_tree(a.n)) {
    b.tiles = stage_tiles_for(longest, K, stage_runs(a.n));
    if (interleave_halves(a.root, a.to_roots != 0, a.count, sizeof(typename Elem<DT>::T))) {
      const dim3 grid(2u * static_cast<uint32_t>(std::min<uint64_t>(b.tiles, kMaxGridX / 2)));
      return launch(tree_stage_fn<DT, OP, true>(a.n), grid, b, stream, stage_bytes(a.n));
    }
    const dim3 grid(grid_x(b.tiles), a.root >= 0 ? 1 : 2);
    return launch(tree_stage_fn<DT, OP>(a.n), grid, b, stream, stage_bytes(a.n));
  }
  b.tiles = tiles_for(longest, 1, 1);
  const dim3 grid(grid_x(b.tiles), a.root >= 0 ? 1 : 2);
  return launch(tree_fold_fn<DT, OP>(a.n), grid, b, stream);
}

}  // namespace

hipError_t launch_tree_fold(const RankPtrs& ptrs, int n, uint64_t count, ar_dtype_t dtype,
                            ar_op_t op, int root, bool to_roots, bool vec, hipStream_t stream) {
  TreeArgs a;
  a.ptrs = ptrs;
  a.count = count;
  a.half = tree_split(count);
  a.n = n;
  a.tiles = 0;
  a.root = root;
  a.to_roots = (root < 0 && to_roots) ? 1 : 0;
  AR_DISPATCH_FOLD(tree_fold_typed, dtype, op, a, vec, stream);
}

}  // namespace ar
