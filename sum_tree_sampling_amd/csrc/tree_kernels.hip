// tree_kernels.hip -- initialisation, batched priority update, ring intake and
// top-level rebuild of the sum + min tree on gfx950.
//
// Tree layout ("Putting prioritized replay's segment tree on a GPU", section
// "The Tree Under Every Prioritized Replay"): node i has children 2i and
// 2i+1, leaves at [n, 2n).  The sum tree and its twin min tree are two
// separate arrays of 2n f32 with the same indexing.
//
// Both writers (update and intake) follow the same plan:
//  1. The leaves are cut into 2^P aligned partitions of 2^S leaves (S <= 12);
//     one 256-thread workgroup owns one partition, i.e. one subtree, so no
//     two workgroups ever write the same node.
//  2. The workgroup collects the leaves it must set (for the update: the last
//     batch position per slot wins; for the intake: the ring range), writes
//     them, and repairs every dirty node of its subtree up to the partition
//     root.  Sparse partitions (<= 64 new leaves, the common case) are
//     repaired by one wave: each leaf's lane walks up its own chain until it
//     meets the chain of its right neighbour; siblings along the chains are
//     fetched in one round of independent loads and values meet through lane
//     shuffles, so the levels stay ordered without a barrier.  Crowded
//     partitions are rebuilt level by level in LDS, one 1024-leaf
//     sub-partition at a time, a barrier between levels.  A contiguous intake
//     run is rebuilt from its range and the two boundary paths.
//  3. The 2^P - 1 nodes above the partitions are not touched by the writers.
//     They are a pure function of the partition roots, and the sampler
//     rebuilds them in LDS anyway to walk the top of the tree, without
//     storing them.  top_kernel rebuilds the stored ones for readers of the
//     stored tree (total, min, inspection, a sampler without an LDS top).
// Every node is recomputed from its two children, never updated by adding a
// delta, and no level is read before the level below it is complete (the
// dependency rule of section "The Race Condition Worth Writing Down").
//
// The running max priority lives in two slots of the control block.  A call
// that may raise it reads the committed slot (its value at the start of the
// call) and raises the other slot with atomicMax on the f32 bit patterns
// (all priorities are >= 0, so the bit patterns order like the values); the
// host flips the committed slot after enqueueing the call.

#include <type_traits>

#include "lanes.h"
#include "per_internal.h"
#include "pow_f32.h"

// Phase stamps of the update kernels, in the measurement build only
// (libper_stamps.so, PER_PHASE_STAMPS defined): lane 0 of wave w of block b
// stores the 100 MHz real-time clock at the end of phase k into
// per_phase_stamps[b * kStampPhases + k] (phases: include/per_stamps.h).
// Each stamp waits for its own scalar read of the clock.  In the product
// build the stamps are empty statements.
#ifdef PER_PHASE_STAMPS
constexpr int kStampBlocks = 4096, kStampPhases = 16;
__device__ unsigned long long per_phase_stamps[kStampBlocks * kStampPhases];
#define PER_STAMP(w, k)                                                        \
  do {                                                                         \
    if (threadIdx.x == 64u * (w) && blockIdx.x < (unsigned)kStampBlocks)       \
      per_phase_stamps[blockIdx.x * kStampPhases + (k)] = __builtin_amdgcn_s_memrealtime(); \
  } while (0)

extern "C" int per_stamps_clear(hipStream_t stream) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(per_phase_stamps)) != hipSuccess) return -4;
  return hipMemsetAsync(p, 0, sizeof(per_phase_stamps), stream) == hipSuccess ? 0 : -4;
}

extern "C" int per_stamps_read(unsigned long long* out, long long count, hipStream_t stream) {
  if (!out || count < 0 || count > (long long)(kStampBlocks * kStampPhases)) return -1;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(per_phase_stamps)) != hipSuccess) return -4;
  if (hipMemcpyAsync(out, p, (size_t)count * sizeof(unsigned long long), hipMemcpyDeviceToHost,
                     stream) != hipSuccess)
    return -4;
  return hipStreamSynchronize(stream) == hipSuccess ? 0 : -4;
}
#else
#define PER_STAMP(w, k) \
  do {                  \
  } while (0)
#endif

namespace per {
namespace {

constexpr int kSubBits = 10;  // crowded partitions are rebuilt in 2^10-leaf pieces
// Whether the scan path (small batches) also takes its low siblings from
// the leaf's line (line_siblings).  It does not: there a partition holds one
// or two entries and the step is bound by latency, which the line's extra
// loads and adds lengthen (measured: Ape-X update + intake 6.1 -> 6.6 us,
// DQN update 6.4 -> 7.4 us), while the bucketed path, bound by the count of
// lines its many entries touch, gains (2^24 leaves, 65536 entries: 32.9 ->
// 27.3 us).
constexpr bool kScanLine = false;
constexpr int kUpdThreads = 256;  // threads of an update block
constexpr int kSub = 1 << kSubBits;

// The min of two tree values.  Every value stored in or compared by these
// trees is a priority or a sum of priorities: +0, a positive finite value or
// +inf, never NaN or -0 (a given -0 priority is stored as +0).  For those the
// f32 bit patterns order like the values, so the min is one integer min of
// the bits, with the same result as (b < a) ? b : a.
__device__ __forceinline__ float min_f32(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}

// Priority of one TD error: f32 of (|td| + eps)^alpha in f64
// ("GPU-Resident Prioritized Experience Replay", section "Priority update";
// NaN / Inf clamp of section "Error Handling & Fallback": NaN takes the value
// of td = 0, computed on the host as p_nan, and +/-Inf the max at batch start).
// pow_f32 gives the f64 pow's f32 value by the shorter exp2(alpha log2 y)
// wherever that rounds the same way.
__device__ __forceinline__ float priority_of(float td, float max_at_start, double alpha,
                                             double eps, float p_nan) {
  const float x = fabsf(td);
  if (__builtin_isnan(x)) return p_nan;
  if (__builtin_isinf(x)) return max_at_start;
  return pow_f32((double)x + eps, alpha);
}

// ------------------------------------------------------------ block helpers

struct BlockScratch {
  int wsum[kTreeThreads / 64];
  uint32_t wmax[kTreeThreads / 64];
};

// Exclusive scan of one int per thread over the 256-thread block.
__device__ int block_excl_scan(int v, BlockScratch& sx, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sx.wsum[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kTreeThreads / 64; ++k) {
    off += (k < w) ? sx.wsum[k] : 0;
    tot += sx.wsum[k];
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// Block max of f32 bit patterns of non-negative values (0 if none); NT
// threads per block.
template <int NT = kTreeThreads>
__device__ uint32_t block_max_bits(uint32_t v, BlockScratch& sx) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  v = wave_max_u32(v);
  if (NT == 64) return v;
  if (lane == 0) sx.wmax[w] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int k = 0; k < NT / 64; ++k) r = max(r, sx.wmax[k]);
  __syncthreads();
  return r;
}

// ------------------------------------------------------------ sparse chains

// Leaves per partition as a power of two.  FULL: the usual 2^kMaxSpanBits,
// known when compiling, so that the per-level loops of the sparse update
// carry no test of the level against it (the tests also held the scalar
// registers of the update kernels past their budget); else the geometry's.
template <bool FULL>
__device__ __forceinline__ int span_bits(const Geom& g) {
  return FULL ? kMaxSpanBits : g.S;
}

// Sparse repair by one wave.  Lanes [0, m) hold the new leaves of the
// partition sorted by offset (offset off, value p); `valid` marks one lane
// per distinct offset (the others are ignored) and ps / pm hold the stored
// values of the siblings of the lane's ancestors (index k: the sibling of
// the ancestor k levels above the leaf, 0 = the leaf's own sibling).  d_i is
// the depth of the lowest common ancestor of the leaves of lanes i and i+1
// (P-1 for the last lane, whose chain ends at the partition root).  Lane i
// computes the nodes of its chain at depths L-1 .. d_i+1: it is the last
// (rightmost) new leaf under each of them.  When lane i's path enters a node
// X from the right child, X's left child holds new leaves iff the nearest
// valid lane j < i with d_j <= depth(X) has d_j == depth(X); that lane's
// chain ends exactly at the left child, whose value it holds, frozen.
// Otherwise the other child is unchanged and its stored value is the
// sibling's.  Must be called by all 64 lanes of the wave.  PAIR: the lanes
// hold the leaves of two consecutive partitions, part and part + 1 (off up
// to 2^(S+1)); a lane whose right neighbour lies in the other partition
// takes d = P - 1 like the last lane, so each chain stops at its own
// partition's root, and the first partition's last chain, with d below
// every depth the loop visits, ends no chain of the second.
template <bool FULL, bool PAIR = false>
__device__ __forceinline__ void sparse_chain(const TreePtrs& t, const Geom& g, uint32_t part, int m, bool valid,
                             uint32_t off, float p, const float* ps, const float* pm) {
  const int S = span_bits<FULL>(g);
  const int lane = threadIdx.x & 63;
  const uint32_t leaf = (part << S) + off;
  const uint32_t node = g.n + leaf;
  if (valid) {
    t.sum[node] = p;
    t.mn[node] = p;
  }
  const uint32_t next_leaf = next_lane(leaf);
  int d = g.P - 1;
  if (lane < m - 1) d = g.L - 1 - (31 - __clz(leaf ^ next_leaf));
  if constexpr (PAIR) d = max(d, (int)g.P - 1);

  float vs = p, vm = p;
  const uint64_t lanes_below = (1ull << lane) - 1ull;
  // Bit k: some chain ends at step k (d == L - 1 - k); the last lane's
  // chain ends at the partition root, past every step.
  const uint32_t ends = wave_or_u32(valid ? 1u << (g.L - 1 - d) : 0u);
#pragma unroll
  for (int k = 0; k < kMaxSpanBits; ++k) {
    if (k >= S) continue;       // uniform across the wave (none when FULL)
    const int l = g.L - 1 - k;  // depth of the node computed at this step
    const bool active = valid && d < l;
    const uint32_t child = node >> k;
    const bool right = child & 1u;
    float os = ps[k], om = pm[k];
    // Chains ending here (d == l) deliver their value to the right; most
    // levels have none, so the lookup runs only when one does (uniform test).
    if ((ends >> k) & 1u) {
      const uint64_t eq = __ballot(valid && d == l);
      const uint64_t le = __ballot(valid && d <= l);
      const uint64_t below = le & lanes_below;
      const int src = below ? 63 - __clzll(below) : lane;
      const bool take = active && right && below != 0ull && ((eq >> src) & 1ull);
      const float s_src = __shfl(vs, src);
      const float m_src = __shfl(vm, src);
      if (take) {
        os = s_src;
        om = m_src;
      }
    }
    if (active) {
      // f32 addition is commutative, and so is the min of priorities (never
      // NaN or -0): the side of the child does not matter.
      vs = vs + os;
      vm = min_f32(vm, om);
      t.sum[child >> 1] = vs;
      t.mn[child >> 1] = vm;
    }
  }
}

// ------------------------------------------------------------ update LDS

struct SparseSmem {
  float sib_s[kSparseMax][kMaxSpanBits];  // stored siblings along each of the
  float sib_m[kSparseMax][kMaxSpanBits];  // first 64 entries' leaf paths
  uint64_t key[kSparseMax];               // (offset << 32 | batch position)
  float pval[kSparseMax];                 // priorities
};

struct DenseSmem {
  int owner[kSub];         // last batch position per offset of the sub-partition
  float val[kSub];         // its new leaf values
  float hs[kSub], hm[kSub];  // local heap [1, 2^sb) of the sub-partition
  uint8_t dirty[kSub];     // node has a new leaf below it
  uint32_t bits[kSub / 32];  // offsets that receive a new leaf
};

// A wave's batch entries listed for the scan's collect when some lane holds
// more than one of them (scan_update), one list per wave; kept only by the
// blocks of the variants that use them (WL).
struct WaveList {
  int64_t idx[64];
  float td[64];
  uint32_t pos[64];
};
struct WaveLists {
  WaveList w[kUpdThreads / 64];
};
struct NoWaveLists {};

// LDS of an update block that owns PPB consecutive partitions: one sparse
// area per partition (wave w repairs partition w of the block), sharing its
// memory with the block-wide rebuild of a crowded partition.
template <int PPB, bool WL = false>
struct UpdSmem {
  union {
    SparseSmem sp[PPB];
    DenseSmem dn;
  } u;
  BlockScratch sx;
  int count[PPB];      // entries collected per partition
  uint32_t mtot[PPB];  // entries per partition (bucketed path)
  uint32_t bmax;       // max priority bits of the block's entries
  uint32_t ball;       // max priority bits of the whole batch (fused intake blocks)
  int flag;
  std::conditional_t<WL, WaveLists, NoWaveLists> wl;  // last: the others' offsets stay put
};

// The parent of two tree values: their f32 sum, or their min.
template <bool MIN>
__device__ __forceinline__ float join(float a, float b) {
  return MIN ? min_f32(a, b) : a + b;
}

template <bool MIN>
__device__ __forceinline__ float join4(float4 v) {
  return join<MIN>(join<MIN>(v.x, v.y), join<MIN>(v.z, v.w));
}

// Heights of a leaf's path whose siblings lie in the leaf's aligned 32-leaf
// line (128 bytes): the sibling at height h < 5 is the subtree over the 2^h
// leaves of block (node >> h) ^ 1, next to the leaf's own block.
constexpr int kLineHeights = 5;

// The stored siblings at heights 0..4 of the path from leaf node `node`
// (n a multiple of 32), from the leaves of its line: the leaves of each
// sibling block, reduced pairwise in heap order (a stored node is exactly
// the f32 sum, or the min, of its two children, so this is its stored value
// bit for bit).  Nine loads that all fall in one line, instead of one line
// per height.
template <bool MIN>
__device__ __forceinline__ void line_siblings(const float* tree, uint32_t node, float* sib) {
  const float s0 = tree[node ^ 1u];
  const float2 s1 = *reinterpret_cast<const float2*>(tree + (((node >> 1) ^ 1u) << 1));
  const float4 s2 = *reinterpret_cast<const float4*>(tree + (((node >> 2) ^ 1u) << 2));
  const float4* p3 = reinterpret_cast<const float4*>(tree + (((node >> 3) ^ 1u) << 3));
  const float4* p4 = reinterpret_cast<const float4*>(tree + (((node >> 4) ^ 1u) << 4));
  const float4 s3a = p3[0], s3b = p3[1];
  const float4 s4a = p4[0], s4b = p4[1], s4c = p4[2], s4d = p4[3];
  sib[0] = s0;
  sib[1] = join<MIN>(s1.x, s1.y);
  sib[2] = join4<MIN>(s2);
  sib[3] = join<MIN>(join4<MIN>(s3a), join4<MIN>(s3b));
  sib[4] = join<MIN>(join<MIN>(join4<MIN>(s4a), join4<MIN>(s4b)),
                     join<MIN>(join4<MIN>(s4c), join4<MIN>(s4d)));
}

// Collect entry k of a partition (any thread): for the first 64 entries the
// stored siblings along its leaf's whole path to the partition root go to
// the partition's sparse area, loaded before the priority's pow so that both
// latencies overlap.  LINE (with FULL): the siblings of heights 0..4 come
// from the leaf's line (line_siblings), the others one load each.  Returns
// the priority.
template <bool FULL, bool LINE>
__device__ __forceinline__ float collect(SparseSmem& sp, int k, const TreePtrs& t,
                                         const Geom& g, uint32_t part, uint32_t off,
                                         uint32_t pos, float td, float m0, double alpha,
                                         double eps, float p_nan) {
  const int S = span_bits<FULL>(g);
  float ps[kMaxSpanBits], pm[kMaxSpanBits];
  const uint32_t node = g.n + (part << S) + off;
  if (k < kSparseMax) {
    if constexpr (FULL && LINE) {
      line_siblings<false>(t.sum, node, ps);
      line_siblings<true>(t.mn, node, pm);
    }
#pragma unroll
    for (int q = (FULL && LINE) ? kLineHeights : 0; q < kMaxSpanBits; ++q) {
      if (q < S) {
        const uint32_t sib = (node >> q) ^ 1u;
        ps[q] = t.sum[sib];
        pm[q] = t.mn[sib];
      }
    }
  }
  const float p = priority_of(td, m0, alpha, eps, p_nan);
  if (k < kSparseMax) {
    sp.key[k] = ((uint64_t)off << 32) | pos;
    sp.pval[k] = p;
#pragma unroll
    for (int q = 0; q < kMaxSpanBits; ++q) {
      if (q < S) {
        sp.sib_s[k][q] = ps[q];
        sp.sib_m[k][q] = pm[q];
      }
    }
  }
  return p;
}

// Raise the running-max slot by max priority bits mb (one thread).  The block
// holding partition 0 carries the value at the start of the call over
// (carry); every other caller has something to add only when it exceeds
// that value, which spares the one contended address nearly all atomics.
__device__ __forceinline__ void publish_max(uint32_t mb, bool carry, float m0,
                                            uint32_t* max_dst) {
  const uint32_t m0b = __float_as_uint(m0);
  if (carry)
    atomicMax(max_dst, max(mb, m0b));
  else if (mb > m0b)
    atomicMax(max_dst, mb);
}

// One wave updates a partition holding m <= 64 collected entries: sort them
// by (offset, batch position) -- the rank of each key among the m keys,
// counted from LDS (m is small) -- so that the last batch position of each
// offset is the last of its run, and repair the chains of those winners with
// the prefetched siblings.
template <bool FULL, bool PAIR = false>
__device__ __forceinline__ void wave_update(SparseSmem& sp, const TreePtrs& t, const Geom& g, uint32_t part,
                            int m) {
  const int lane = threadIdx.x & 63;
  const bool in = lane < m;
  const uint64_t mine = in ? sp.key[lane] : ~0ull;
  // The ranks (a permutation of [0, m), lanes past m keeping their own
  // index) are inverted by one lane permute, which gives each sorted
  // position its entry.
  int rank = 0;
#pragma unroll 4
  for (int j = 0; j < m; ++j) rank += (sp.key[j] < mine) ? 1 : 0;
  if (!in) rank = lane;
  const int sorted = __builtin_amdgcn_ds_permute(rank << 2, lane);  // every lane takes part
  const int src = in ? sorted : 0;
  const uint64_t key = sp.key[src];
  const uint32_t off = (uint32_t)(key >> 32);
  const float p = sp.pval[src];
  PER_STAMP(0, 13);
  const uint32_t next_off = next_lane(off);  // lane m - 1 does not look at it
  const bool win = in && (lane == m - 1 || next_off != off);
  float ps[kMaxSpanBits], pm[kMaxSpanBits];
#pragma unroll
  for (int k = 0; k < kMaxSpanBits; ++k) {
    ps[k] = sp.sib_s[src][k];
    pm[k] = sp.sib_m[src][k];
  }
  PER_STAMP(0, 14);
  sparse_chain<FULL, PAIR>(t, g, part, m, win, in ? off : 0u, p, ps, pm);
}

// ------------------------------------------------------------ crowded partitions

__device__ __forceinline__ bool has_bit(const DenseSmem& dn, uint32_t off) {
  return (dn.bits[off >> 5] >> (off & 31)) & 1u;
}

// Rebuild one sub-partition of 2^sb leaves (sb <= kSubBits) in LDS from its
// new leaves (dn.val / dn.bits) and its stored old ones, and write back the
// new leaves and every node with a new leaf below it.  subroot: node index
// of the sub-partition's root; leaf0: node index of its first leaf.  All old
// leaves are loaded before anything is stored.
template <int NT>
__device__ void dense_sub_rebuild(DenseSmem& dn, const TreePtrs& t, uint32_t subroot,
                                  uint32_t leaf0, int sb) {
  constexpr int kPairs = kSub / 2 / NT;
  const uint32_t span = 1u << sb, half = span >> 1;
  float2 os[kPairs], om[kPairs];
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    os[r] = om[r] = make_float2(0.0f, 0.0f);
    const uint32_t h = half + threadIdx.x + r * NT;
    if (h < span) {
      const uint32_t a = 2 * h - span;
      if (!(has_bit(dn, a) && has_bit(dn, a + 1))) {
        os[r] = *reinterpret_cast<const float2*>(t.sum + leaf0 + a);
        om[r] = *reinterpret_cast<const float2*>(t.mn + leaf0 + a);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < kPairs; ++r) {
    const uint32_t h = half + threadIdx.x + r * NT;
    if (h < span) {
      const uint32_t a = 2 * h - span;
      const bool ba = has_bit(dn, a), bb = has_bit(dn, a + 1);
      const float ls = ba ? dn.val[a] : os[r].x, lm = ba ? dn.val[a] : om[r].x;
      const float rs = bb ? dn.val[a + 1] : os[r].y, rm = bb ? dn.val[a + 1] : om[r].y;
      dn.hs[h] = ls + rs;
      dn.hm[h] = min_f32(lm, rm);
      dn.dirty[h] = ba | bb;
    }
  }
  // The levels above in LDS, nothing stored to global memory in between: a
  // barrier waits for every outstanding memory operation, stores included.
  for (uint32_t width = half >> 1; width >= 1; width >>= 1) {
    __syncthreads();
    for (uint32_t h = width + threadIdx.x; h < 2 * width; h += NT) {
      dn.hs[h] = dn.hs[2 * h] + dn.hs[2 * h + 1];
      dn.hm[h] = min_f32(dn.hm[2 * h], dn.hm[2 * h + 1]);
      dn.dirty[h] = dn.dirty[2 * h] | dn.dirty[2 * h + 1];
    }
  }
  __syncthreads();
  // New leaves, then every node with a new leaf below it; local heap index
  // h in [1, span) is global node ((subroot - 1) << depth(h)) + h.
  for (uint32_t a = threadIdx.x; a < span; a += NT) {
    if (has_bit(dn, a)) {
      t.sum[leaf0 + a] = dn.val[a];
      t.mn[leaf0 + a] = dn.val[a];
    }
  }
  for (uint32_t h = 1 + threadIdx.x; h < span; h += NT) {
    if (dn.dirty[h]) {
      const uint32_t x = ((subroot - 1u) << (31 - __clz(h))) + h;
      t.sum[x] = dn.hs[h];
      t.mn[x] = dn.hm[h];
    }
  }
}

// Block-wide update of a crowded partition.  each(f) calls f(off, pos, p)
// for every entry of the partition, spread over the block's threads (the
// same entries, in any order, on every call).  The sub-partitions are
// handled one at a time: last batch position per offset through an LDS
// owner table, then an LDS rebuild; the few levels between the
// sub-partition roots and the partition root follow from the stored nodes.
// Returns the block max of all entries' priority bits.
template <int NT, typename Each>
__device__ uint32_t dense_update(DenseSmem& dn, int& flag, BlockScratch& sx, const TreePtrs& t,
                                 const Geom& g, uint32_t part, Each each) {
  const int sb = g.S < kSubBits ? g.S : kSubBits;
  const int e = g.S - sb;
  const uint32_t sspan = 1u << sb, smask = sspan - 1u;
  const uint32_t nwords = (sspan + 31) >> 5;
  const uint32_t root = (1u << g.P) + part;
  uint32_t mb = 0;
  for (uint32_t q = 0; q < (1u << e); ++q) {
    for (uint32_t k = threadIdx.x; k < sspan; k += NT) dn.owner[k] = -1;
    for (uint32_t k = threadIdx.x; k < nwords; k += NT) dn.bits[k] = 0u;
    if (threadIdx.x == 0) flag = 0;
    __syncthreads();
    each([&](uint32_t off, uint32_t pos, float p) {
      if (q == 0) mb = max(mb, __float_as_uint(p));
      if ((off >> sb) == q) atomicMax(&dn.owner[off & smask], (int)pos);
    });
    __syncthreads();
    each([&](uint32_t off, uint32_t pos, float p) {
      const uint32_t o = off & smask;
      if ((off >> sb) == q && dn.owner[o] == (int)pos) {
        dn.val[o] = p;
        atomicOr(&dn.bits[o >> 5], 1u << (o & 31));
        flag = 1;
      }
    });
    __syncthreads();
    if (flag) dense_sub_rebuild<NT>(dn, t, (root << e) + q, g.n + (part << g.S) + (q << sb), sb);
    __syncthreads();
  }
  if (e > 0 && threadIdx.x == 0) {
    for (int j = e - 1; j >= 0; --j) {
      for (uint32_t r = 0; r < (1u << j); ++r) {
        const uint32_t x = (root << j) + r;
        t.sum[x] = t.sum[2 * x] + t.sum[2 * x + 1];
        t.mn[x] = min_f32(t.mn[2 * x], t.mn[2 * x + 1]);
      }
    }
  }
  return block_max_bits<NT>(mb, sx);
}

// ------------------------------------------------------------ intake range

struct RangeSmem {
  float val[kMaxSpan];                      // new leaf values by offset
  float ns[kMaxSpan + 2 * kMaxSpanBits];    // dirty nodes of heights 1..S, packed
  float nm[kMaxSpan + 2 * kMaxSpanBits];    // height after height: sums, mins
  float bnd_s[2][kMaxSpanBits];             // boundary siblings per level: left, right
  float bnd_m[2][kMaxSpanBits];
};

struct AddSmem {
  union {
    RangeSmem r;
    DenseSmem dn;
  } u;
  BlockScratch sx;
  int flag;
};

// The boundary siblings of a contiguous run of new leaves, offsets [lo, hi)
// of the partition: at every level the dirty nodes form a contiguous range
// and only its two end nodes can have an unchanged child -- the sibling left
// of the range's first node when that node is a right child, and the sibling
// right of its last node when that node is a left child.  Loaded by the
// block's first wave, up front with the caller's other loads.
__device__ __forceinline__ void prefetch_range_boundaries(RangeSmem& r, const TreePtrs& t,
                                                          const Geom& g, uint32_t part,
                                                          uint32_t lo, uint32_t hi) {
  const uint32_t a = g.n + (part << g.S) + lo, b = g.n + (part << g.S) + hi - 1;
  const int q = threadIdx.x & 31;
  if (threadIdx.x < 64 && q < g.S) {
    const bool left = threadIdx.x < 32;
    const uint32_t x = (left ? a : b) >> q;
    const bool need = left ? (x & 1u) : !(x & 1u);
    if (need) {
      const uint32_t sib = left ? x - 1 : x + 1;
      r.bnd_s[left ? 0 : 1][q] = t.sum[sib];
      r.bnd_m[left ? 0 : 1][q] = t.mn[sib];
    }
  }
}

// The boundary sibling of height q = lane & 31 of a run [lo, hi) of new
// leaves, into the registers of the block's first wave: lanes 0..31 the
// sibling left of the run's first node at height q (needed when that node
// is a right child), lanes 32..63 the sibling right of its last node (needed
// when that node is a left child); other lanes and unneeded siblings: 0.
template <bool FULL>
__device__ __forceinline__ void load_range_boundary(const TreePtrs& t, const Geom& g,
                                                    uint32_t part, uint32_t lo, uint32_t hi,
                                                    float& sib_s, float& sib_m) {
  const int S = span_bits<FULL>(g);
  const uint32_t a = g.n + (part << S) + lo, b = g.n + (part << S) + hi - 1;
  const int q = threadIdx.x & 31;
  if (threadIdx.x < 64 && q < S) {
    const bool left = threadIdx.x < 32;
    const uint32_t x = (left ? a : b) >> q;
    if (left ? (x & 1u) : !(x & 1u)) {
      const uint32_t sib = left ? x - 1 : x + 1;
      sib_s = t.sum[sib];
      sib_m = t.mn[sib];
    }
  }
}

// The climb of uniform_range: the two boundary paths over `levels` heights
// from the new leaves' value v, one add and one min per path and height with
// the other children other[k] (left path's sum and min, right path's sum and
// min) at height k, or the other path where merges has bit k.  Lane k keeps
// the nodes of height k + 1.
// FIXED: levels is kMaxSpanBits, so the unrolled climb tests no level.
template <bool FIXED>
__device__ __forceinline__ void climb_paths(int levels, int lane, uint64_t merges, float v,
                                            const float4* other, float& oLs, float& oLm,
                                            float& oRs, float& oRm) {
  float sL = v, mL = v, sR = v, mR = v;  // the paths' nodes at the current height
#pragma unroll
  for (int k = 0; k < kMaxSpanBits; ++k) {
    if (FIXED || k < levels) {  // uniform
      // Where the paths meet, each takes the other as its other child (the
      // two sums and the two mins are then equal).
      const bool meet = (merges >> k) & 1ull;
      const float4 c = other[k];  // the same LDS word for every lane
      const float aLs = meet ? sR : c.x;
      const float aLm = meet ? mR : c.y;
      const float aRs = meet ? sL : c.z;
      const float aRm = meet ? mL : c.w;
      sL = sL + aLs;
      mL = min_f32(mL, aLm);
      sR = sR + aRs;
      mR = min_f32(mR, aRm);
      const bool mine = lane == k;
      oLs = mine ? sL : oLs;
      oLm = mine ? mL : oLm;
      oRs = mine ? sR : oRs;
      oRm = mine ? mR : oRm;
    }
  }
}

// Repair after a contiguous run [lo, hi) of new leaves that all take the
// value v.  A node strictly between the run's first and last node of its
// height k covers 2^k new leaves and nothing else: its sum is v doubled k
// times, which is exactly what the pairwise adds of its subtree give, and
// its min is v.  Those nodes and the leaves are stored by the whole block,
// independently.  Only the first and last node of each height (the run's two
// boundary paths) can have an old leaf below, and the block's first wave
// computes them.  Lane q first works out, for height q, the other child of
// each path's node: a stored boundary sibling (from the registers
// load_range_boundary filled: lane q the left one, lane 32 + q the right
// one), an interior node, or -- where the paths meet -- the other path.
// The wave then climbs the heights with one add and one min per path and
// height (f32 addition is commutative, and so is the min of priorities,
// which are never NaN or -0, so the order of the two children does not
// matter), lane q keeping the two nodes of height q + 1; the lanes store
// them together at the end.  A single instruction stream climbing S levels
// costs several cycles per instruction, so the climb does nothing else, and
// the other waves store the leaves and the interior nodes meanwhile.  No
// barrier anywhere.
template <bool FULL>
__device__ __forceinline__ void uniform_range(const TreePtrs& t, const Geom& g, uint32_t part,
                                              uint32_t lo, uint32_t hi, float v, float sib_s,
                                              float sib_m) {
  const int S = span_bits<FULL>(g);
  const uint32_t leaf0 = g.n + (part << S);
  // Every load is complete before the first store: a wait placed after
  // stores (the compiler joins the paths of the waves below) would also
  // wait for those stores.
  asm volatile("" ::"v"(v), "v"(sib_s), "v"(sib_m));
  if (threadIdx.x < 64) {
    const int lane = threadIdx.x;
    const int q = lane & 31;
    const float brs = __shfl(sib_s, 32 + q);  // right boundary siblings of height q
    const float brm = __shfl(sib_m, 32 + q);
    const uint32_t A = (leaf0 + lo) >> q, Bn = (leaf0 + hi - 1) >> q;  // the paths' nodes
    const float full = v * __int_as_float((127 + q) << 23);           // v doubled q times
    const bool merge = !(A & 1u) && A + 1u == Bn;  // the two paths share a parent
    // The other child of each path's node at height q.
    const float cls = (A & 1u) ? sib_s : ((A + 1u < Bn) ? full : brs);
    const float clm = (A & 1u) ? sib_m : ((A + 1u < Bn) ? v : brm);
    const float crs = (Bn & 1u) ? ((Bn - 1u > A) ? full : sib_s) : brs;
    const float crm = (Bn & 1u) ? ((Bn - 1u > A) ? v : sib_m) : brm;
    const uint64_t merges = __ballot(merge);
    // Handed to the climb through LDS: a lane reading the word of height k
    // is an ordinary load the compiler may schedule early, where reading it
    // from lane k's registers is an operation it must not hoist.
    __shared__ float4 other[kMaxSpanBits];
    if (lane < S) other[lane] = make_float4(cls, clm, crs, crm);
    __builtin_amdgcn_wave_barrier();
    float oLs = 0.0f, oLm = 0.0f, oRs = 0.0f, oRm = 0.0f;  // lane q: the parents of height q
    climb_paths<FULL>(S, lane, merges, v, other, oLs, oLm, oRs, oRm);
    if (lane < S) {
      const uint32_t pa = A >> 1, pb = Bn >> 1;
      t.sum[pa] = oLs;
      t.mn[pa] = oLm;
      if (pb != pa) {
        t.sum[pb] = oRs;
        t.mn[pb] = oRm;
      }
    }
    PER_STAMP(0, 5);
  }
  // The leaves and the interior nodes, by the other waves, while the first
  // wave climbs.
  if (threadIdx.x >= 64) {
    float full = v;  // sum of a node of height k covering new leaves only
    for (int k = 0; k <= S; ++k) {
      const uint32_t A = (leaf0 + lo) >> k, Bn = (leaf0 + hi - 1) >> k;
      const uint32_t first = (k == 0) ? A : A + 1;
      for (uint32_t x = first + threadIdx.x - 64; x < Bn + (k == 0 ? 1u : 0u);
           x += kTreeThreads - 64) {
        t.sum[x] = full;
        t.mn[x] = v;
      }
      full = full + full;
    }
  }
}

// Rebuild after a contiguous run [lo, hi) of new leaves (values in r.val),
// level by level in LDS with a barrier between levels (whole block).
__device__ void range_repair(RangeSmem& r, const TreePtrs& t, const Geom& g, uint32_t part,
                             uint32_t lo, uint32_t hi) {
  // Heights 1..S in LDS first: a barrier waits for every outstanding memory
  // operation of the block, stores included, so nothing is stored to
  // global memory until the last one.
  const uint32_t leaf0 = g.n + (part << g.S);
  uint32_t A = leaf0 + lo, Bn = leaf0 + hi - 1;  // children range (node indices)
  const float* cs = r.val + lo;                   // children values, index x - A
  const float* cm = r.val + lo;
  uint32_t at = 0;                                // packed position of the height
  for (int k = 0; k < g.S; ++k) {
    const uint32_t pa = A >> 1, pb = Bn >> 1;
    float* ns = r.ns + at;
    float* nm = r.nm + at;
    for (uint32_t x = pa + threadIdx.x; x <= pb; x += kTreeThreads) {
      const uint32_t l = 2 * x, rr = 2 * x + 1;
      const float ls = (l >= A) ? cs[l - A] : r.bnd_s[0][k];
      const float lm = (l >= A) ? cm[l - A] : r.bnd_m[0][k];
      const float rs = (rr <= Bn) ? cs[rr - A] : r.bnd_s[1][k];
      const float rm = (rr <= Bn) ? cm[rr - A] : r.bnd_m[1][k];
      ns[x - pa] = ls + rs;
      nm[x - pa] = min_f32(lm, rm);
    }
    __syncthreads();
    cs = ns;
    cm = nm;
    at += pb - pa + 1;
    A = pa;
    Bn = pb;
  }
  for (uint32_t off = lo + threadIdx.x; off < hi; off += kTreeThreads) {
    t.sum[leaf0 + off] = r.val[off];
    t.mn[leaf0 + off] = r.val[off];
  }
  A = leaf0 + lo;
  Bn = leaf0 + hi - 1;
  at = 0;
  for (int k = 0; k < g.S; ++k) {
    const uint32_t pa = A >> 1, pb = Bn >> 1;
    for (uint32_t x = pa + threadIdx.x; x <= pb; x += kTreeThreads) {
      t.sum[x] = r.ns[at + x - pa];
      t.mn[x] = r.nm[at + x - pa];
    }
    at += pb - pa + 1;
    A = pa;
    Bn = pb;
  }
}

// ------------------------------------------------------------------ kernels

__global__ void __launch_bounds__(256) init_kernel(TreePtrs t, Buckets bk, Geom g) {
  const uint64_t total = 2ull * g.n;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride)
  {
    t.sum[i] = 0.0f;
    t.mn[i] = __builtin_inff();
  }
  const uint32_t np = 1u << g.P;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < np; i += stride)
    bk.counts[i * kCountStride] = 0u;
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    t.ctrl->maxp_bits[0] = __float_as_uint(1.0f);
    t.ctrl->maxp_bits[1] = __float_as_uint(1.0f);
    for (int k = 0; k < 2; ++k) {
      t.ctrl->cursor[k] = 0u;
      t.ctrl->size[k] = 0u;
    }
    bk.ovf_n[0] = 0u;
    bk.ovf_n[1] = 0u;
  }
}

__global__ void __launch_bounds__(256) bucket_clear_kernel(Buckets bk, uint32_t np) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < np; i += gridDim.x * blockDim.x)
    bk.counts[i * kCountStride] = 0u;
  if (blockIdx.x == 0 && threadIdx.x < 2) bk.ovf_n[threadIdx.x] = 0u;
}

struct UpdateArgs {
  const int64_t* idx;
  const float* td;
  uint32_t B;
  uint32_t size;  // filled slots (host-tracked; see ring)
  double alpha, eps;
  float p_nan;
  int src, dst;  // running-max slots: read / raise
  int ovf;       // overflow counter of this call (bucketed path)
  RingRef ring;  // graph mode: the size comes from ring_ctrl->size[ring.slot]
  const Ctrl* ring_ctrl;
};

__device__ __forceinline__ uint32_t filled_size(const UpdateArgs& a) {
  return a.ring.dev ? a.ring_ctrl->size[a.ring.slot] : a.size;
}

// Entries b0 + c kUpdThreads + threadIdx.x (c < kChunk) of a batch of B:
// their slots (-1 past the end) and TD errors, all loads issued before any
// is used.
template <int kChunk>
__device__ __forceinline__ void load_chunk(const int64_t* idx, const float* td, uint32_t B,
                                           uint32_t b0, int64_t* ix, float* tx) {
#pragma unroll
  for (int c = 0; c < kChunk; ++c) {
    const uint32_t b = b0 + c * kUpdThreads + threadIdx.x;
    ix[c] = -1;
    tx[c] = 0.0f;
    if (b < B) {
      ix[c] = idx[b];
      tx[c] = td[b];
    }
  }
}

// Word `slot` (0 or 1) of a two-slot field of the control block, from a
// copy loaded whole at kernel start (one scalar trip through the preloaded
// pointer, issued before the slot is known).
__device__ __forceinline__ uint32_t ctrl_word(const uint32_t (&w)[2], int slot) {
  return slot ? w[1] : w[0];
}

// Small batches: each block owns PPB consecutive partitions and scans the
// whole batch for their slots; wave w repairs partition w of the block when
// it is sparse, crowded partitions are rebuilt by the whole block after.
// m0: the running max at the start of the call.  FUSED (one partition per
// block): entries at offsets skip(off) are left out of the repair, their
// priorities still raising the running max; sm.ball is cleared for the
// caller's batch max.  Returns whether a partition was crowded (then
// rebuilt by the whole block, which has passed a barrier since); otherwise
// wave w returns right after its sparse repair.  ix0, tx0: the batch's
// first chunk (load_chunk at b0 = 0), loaded by the caller at kernel start.
template <int PPB, bool FUSED, bool FULL, int kChunk, bool LINE, typename SM, typename Skip>
__device__ __forceinline__ bool scan_update(SM& sm, const TreePtrs& t, const Geom& g,
                                            const UpdateArgs& a, uint32_t part0, uint32_t size,
                                            float m0, const int64_t* ix0, const float* tx0,
                                            Skip skip) {
  const int nparts = (int)min((uint32_t)PPB, (1u << g.P) - part0);
  uint32_t* max_dst = &t.ctrl->maxp_bits[a.dst];
  if (threadIdx.x < PPB) sm.count[threadIdx.x] = 0;
  if (threadIdx.x == 0) {
    sm.bmax = 0u;
    sm.ball = 0u;
  }
  __syncthreads();
  // Each thread loads its share of the batch in chunks of kChunk entries, all
  // loads of a chunk issued before any of them is looked at (kChunk is sized
  // to the batch when launching: no idle slots for small batches).
  for (uint32_t b0 = 0; b0 < a.B; b0 += kUpdThreads * kChunk) {
    int64_t ix[kChunk];
    float tx[kChunk];
    if (b0 == 0) {
#pragma unroll
      for (int c = 0; c < kChunk; ++c) {
        ix[c] = ix0[c];
        tx[c] = tx0[c];
      }
    } else {
      load_chunk<kChunk>(a.idx, a.td, a.B, b0, ix, tx);
    }
#pragma unroll
    for (int c = 0; c < kChunk; ++c) asm volatile("" ::"v"(tx[c]), "v"(ix[c]));
    // The entries this lane looks at (bit c: slot c of the chunk).
    uint32_t pending = 0u;
#pragma unroll
    for (int c = 0; c < kChunk; ++c) {
      const int64_t i = ix[c];
      if (i < 0 || i >= (int64_t)size) continue;
      const uint32_t q = (uint32_t)((uint64_t)i >> span_bits<FULL>(g)) - part0;  // wraps below part0
      if (q < (uint32_t)nparts) pending |= 1u << c;
    }
    // A lane holding several entries would collect them one round (one
    // sibling trip and power) after another.  Then the wave lists its
    // entries in LDS first -- entry e counted lane by lane in slot order --
    // and lane e mod 64 takes entry e, 64 entries per round.  Compiled for
    // the larger batches (four or more entries per thread and chunk), where
    // a busy partition's entries often share a lane: the code costs the
    // smaller ones more than it saves.
    if constexpr (kChunk >= 4 && FULL) {
     const uint32_t cnt = (uint32_t)__builtin_popcount(pending);
     if (__ballot(cnt > 1u) != 0ull) {
      WaveList& wl = sm.wl.w[threadIdx.x >> 6];
      const int lane = threadIdx.x & 63;
      const uint64_t below = (1ull << lane) - 1ull;
      uint32_t pre = 0u, total = 0u;  // entries of the lower lanes; of the wave
#pragma unroll
      for (int bit = 0; (1 << bit) <= kChunk; ++bit) {
        const uint64_t bm = __ballot((cnt >> bit) & 1u);
        pre += (uint32_t)__popcll(bm & below) << bit;
        total += (uint32_t)__popcll(bm) << bit;
      }
      for (uint32_t r0 = 0; r0 < total; r0 += 64u) {
        uint32_t e = pre;
#pragma unroll
        for (int c = 0; c < kChunk; ++c) {
          if ((pending >> c) & 1u) {
            if (e - r0 < 64u) {
              wl.idx[e - r0] = ix[c];
              wl.td[e - r0] = tx[c];
              wl.pos[e - r0] = b0 + (uint32_t)c * kUpdThreads + threadIdx.x;
            }
            ++e;
          }
        }
        // The wave reads what its own lanes wrote: LDS operations of one
        // wave complete in order.
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (r0 + (uint32_t)lane < total) {
          // the entry is the block's (as in the rounds below)
          const int64_t i = wl.idx[lane];
          const uint32_t q = (uint32_t)((uint64_t)i >> span_bits<FULL>(g)) - part0;
          const uint32_t part = part0 + q;
          const uint32_t off = (uint32_t)i - (part << span_bits<FULL>(g));
          bool keep = true;
          if constexpr (FUSED) keep = !skip(off);
          const int k = keep ? atomicAdd(&sm.count[q], 1) : kSparseMax;
          const float p = collect<FULL, LINE>(sm.u.sp[q], k, t, g, part, off, wl.pos[lane],
                                              wl.td[lane], m0, a.alpha, a.eps, a.p_nan);
          atomicMax(&sm.bmax, __float_as_uint(p));
        }
        // and overwrites the list only after every lane has read its entry
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      }
      pending = 0u;
     }
    }
    // One entry per lane per round: entries of one wave in different slots
    // are collected together, their sibling loads and pows overlapping,
    // instead of one slot after the other.
    while (__ballot(pending != 0u) != 0ull) {
      if (pending != 0u) {
        const int c = __builtin_ctz(pending);
        pending &= pending - 1u;
        int64_t i = ix[0];
        float td = tx[0];
#pragma unroll
        for (int cc = 1; cc < kChunk; ++cc) {
          if (c == cc) {
            i = ix[cc];
            td = tx[cc];
          }
        }
        const uint32_t b = b0 + (uint32_t)c * kUpdThreads + threadIdx.x;
        const uint32_t q = (uint32_t)((uint64_t)i >> span_bits<FULL>(g)) - part0;
        // The entry is the block's: collect() issues no loads for an entry
        // index >= kSparseMax, which left-out entries take.
        const uint32_t part = part0 + q;
        const uint32_t off = (uint32_t)i - (part << span_bits<FULL>(g));
        bool keep = true;
        if constexpr (FUSED) keep = !skip(off);
        const int k = keep ? atomicAdd(&sm.count[q], 1) : kSparseMax;
        const float p = collect<FULL, LINE>(sm.u.sp[q], k, t, g, part, off, b, td, m0, a.alpha,
                                            a.eps, a.p_nan);
        atomicMax(&sm.bmax, __float_as_uint(p));
      }
    }
  }
  PER_STAMP(0, 1);
  PER_STAMP(1, 10);
  PER_STAMP(2, 11);
  PER_STAMP(3, 12);
  __syncthreads();
  PER_STAMP(0, 8);
  if (threadIdx.x == 64) publish_max(sm.bmax, blockIdx.x == 0, m0, max_dst);
  const int w = threadIdx.x >> 6;
  bool crowded = false;
  for (int q = 0; q < nparts; ++q) crowded |= sm.count[q] > kSparseMax;
  if (w < nparts) {
    const int m = sm.count[w];
    if (m > 0 && m <= kSparseMax) wave_update<FULL>(sm.u.sp[w], t, g, part0 + w, m);
  }
  PER_STAMP(0, 2);
  if (!crowded) return false;
  // The dense rebuild reuses the sparse areas: every wave is done with them.
  __syncthreads();
  for (int q = 0; q < nparts; ++q) {
    if (sm.count[q] <= kSparseMax) continue;
    const uint32_t part = part0 + q, base = part << g.S;
    // Its entries are read from the batch again.
    dense_update<kUpdThreads>(sm.u.dn, sm.flag, sm.sx, t, g, part, [&](auto f) {
      for (uint32_t b = threadIdx.x; b < a.B; b += kUpdThreads) {
        const int64_t i = a.idx[b];
        if (i >= 0 && i < (int64_t)size && ((uint64_t)i >> g.S) == part &&
            !(FUSED && skip((uint32_t)i - base)))
          f((uint32_t)i - base, b, priority_of(a.td[b], m0, a.alpha, a.eps, a.p_nan));
      }
    });
  }
  return true;
}

template <int PPB, bool FULL, int CH, bool LINE>
__global__ void __launch_bounds__(kUpdThreads) update_scan_kernel(const int64_t* bidx, const float* btd,
                                                                  uint32_t bB, Ctrl* ctrl, TreePtrs t,
                                                                  Geom g, UpdateArgs a) {
  __shared__ UpdSmem<PPB, (CH >= 4 && FULL)> sm;
  // The batch and the control block arrive in scalar registers with the
  // wave (the leading arguments, preloaded; the same as a's and t's), so
  // the batch's first chunk is loaded before anything else.
  int64_t ix0[CH];
  float tx0[CH];
  load_chunk<CH>(bidx, btd, bB, 0, ix0, tx0);
  const Ctrl c = *ctrl;
  a.idx = bidx;
  a.td = btd;
  a.B = bB;
  t.ctrl = ctrl;
  // The other arguments the first steps need, fetched in one batch.
  asm volatile("" ::"s"(a.src), "s"(a.size), "s"(a.ring.dev), "s"(a.ring.slot), "s"(g.n),
               "s"(g.S));
  const float m0 = __uint_as_float(ctrl_word(c.maxp_bits, a.src));
  const uint32_t size = a.ring.dev ? ctrl_word(c.size, a.ring.slot) : a.size;
  scan_update<PPB, false, FULL, CH, LINE>(sm, t, g, a, blockIdx.x * PPB, size, m0, ix0, tx0,
                                          [](uint32_t) { return false; });
}

// Large batches, step 1: every valid entry goes to its partition's bucket
// (kBucketCap entries per partition); past the cap, to an overflow list.
__global__ void __launch_bounds__(256) bucket_kernel(const int64_t* idx, const float* td, uint32_t B,
                                                     uint32_t* counts, Buckets bk, Geom g,
                                                     UpdateArgs a) {
  // The batch and the counts arrive in scalar registers with the wave (the
  // leading arguments, preloaded; the same as a's and bk's), so the entry's
  // loads issue at once.
  const uint32_t b = blockIdx.x * kTreeThreads + threadIdx.x;  // launched with kTreeThreads
  if (b >= B) return;
  const int64_t i = idx[b];
  const float x = td[b];
  // The other arguments the next steps need, fetched in one batch.
  asm volatile("" ::"s"(a.size), "s"(a.ring.dev), "s"(g.S));
  asm volatile("" ::"v"(i), "v"(x));  // both loads out before either is looked at
  if (i < 0 || i >= (int64_t)filled_size(a)) return;
  const uint32_t part = (uint32_t)((uint64_t)i >> g.S);
  const uint32_t k = atomicAdd(&counts[part * kCountStride], 1u);
  if (k < kBucketCap) {
    const uint32_t e = part * kBucketCap + k;
    bk.slot[e] = (uint32_t)i;
    bk.pos[e] = b;
    bk.td[e] = x;
  } else {
    const uint32_t e = atomicAdd(&bk.ovf_n[a.ovf], 1u);
    bk.oslot[e] = (uint32_t)i;
    bk.opos[e] = b;
    bk.otd[e] = x;
  }
}

// Large batches, step 2: each block owns PPB consecutive partitions; wave w
// reads the bucket of partition w of the block and repairs it (lane k takes
// entry k), crowded partitions (more entries than a bucket holds) are
// rebuilt by the whole block after, from their bucket and the overflow list.
template <int PPB, bool FULL>
__global__ void __launch_bounds__(kUpdThreads) update_bucket_kernel(uint32_t* counts, const uint32_t* slot,
                                                                    const uint32_t* pos,
                                                                    const float* etd, uint32_t np,
                                                                    TreePtrs t, Buckets bk, Geom g,
                                                                    UpdateArgs a) {
  __shared__ UpdSmem<PPB> sm;
  // The buckets and the partition count arrive in scalar registers with the
  // wave (the leading arguments, preloaded; the same as bk's and 2^g.P), so
  // the counts and entries are loaded before anything else.
  const uint32_t part0 = blockIdx.x * PPB;
  const int nparts = (int)min((uint32_t)PPB, np - part0);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t cnt = 0u;
  if (threadIdx.x < (unsigned)nparts) cnt = counts[(part0 + threadIdx.x) * kCountStride];
  // Every lane loads its entry of the wave's bucket before the count is
  // known, so that the entries arrive together with the counts instead of
  // one trip after them (the lanes past the count drop theirs).
  uint32_t es = 0u, ep = 0u;
  float et = 0.0f;
  if (w < nparts) {
    const uint32_t e = (part0 + w) * kBucketCap + lane;
    es = slot[e];
    ep = pos[e];
    et = etd[e];
  }
  // The other arguments the next steps need, fetched in one batch.
  asm volatile("" ::"s"(t.ctrl), "s"(a.src), "s"(a.dst), "s"(a.ovf), "s"(g.S), "s"(g.n));
  const float m0 = __uint_as_float(t.ctrl->maxp_bits[a.src]);
  uint32_t* max_dst = &t.ctrl->maxp_bits[a.dst];
  if (threadIdx.x < (unsigned)nparts) {
    sm.mtot[threadIdx.x] = cnt;
    counts[(part0 + threadIdx.x) * kCountStride] = 0u;  // ready for the next call's bucketing
  }
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    bk.ovf_n[a.ovf ^ 1] = 0u;  // the next call's overflow counter
    publish_max(0u, true, m0, max_dst);
  }
  __syncthreads();
  bool crowded = false;
  for (int q = 0; q < nparts; ++q) crowded |= sm.mtot[q] > (uint32_t)kBucketCap;
  if (w < nparts) {
    const uint32_t part = part0 + w, m = sm.mtot[w];
    if (m > 0 && m <= (uint32_t)kBucketCap) {
      SparseSmem& sp = sm.u.sp[w];
      uint32_t pb = 0u;
      if ((uint32_t)lane < m) {
        const float p = collect<FULL, true>(sp, lane, t, g, part,
                                            es - (part << span_bits<FULL>(g)), ep, et, m0,
                                            a.alpha, a.eps, a.p_nan);
        pb = __float_as_uint(p);
      }
      pb = wave_max_u32(pb);
      if (lane == 0) publish_max(pb, false, m0, max_dst);
      // The wave reads what its own lanes wrote to its sparse area: LDS
      // operations of one wave complete in order.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      wave_update<FULL>(sp, t, g, part, (int)m);
    }
  }
  if (!crowded) return;
  // The dense rebuild reuses the sparse areas: every wave is done with them.
  __syncthreads();
  const uint32_t novf = bk.ovf_n[a.ovf];
  for (int q = 0; q < nparts; ++q) {
    if (sm.mtot[q] <= (uint32_t)kBucketCap) continue;
    const uint32_t part = part0 + q, base = part << g.S;
    const uint32_t* bslot = bk.slot + part * kBucketCap;
    const uint32_t* bpos = bk.pos + part * kBucketCap;
    const float* btd = bk.td + part * kBucketCap;
    const uint32_t mb = dense_update<kUpdThreads>(sm.u.dn, sm.flag, sm.sx, t, g, part, [&](auto f) {
      for (uint32_t k = threadIdx.x; k < kBucketCap; k += kUpdThreads)
        f(bslot[k] - base, bpos[k], priority_of(btd[k], m0, a.alpha, a.eps, a.p_nan));
      for (uint32_t k = threadIdx.x; k < novf; k += kUpdThreads) {
        const uint32_t i = bk.oslot[k];
        if ((i >> g.S) == part)
          f(i - base, bk.opos[k], priority_of(bk.otd[k], m0, a.alpha, a.eps, a.p_nan));
      }
    });
    if (threadIdx.x == 0) publish_max(mb, false, m0, max_dst);
  }
}

// The sparse repair of m <= 64 bucket entries by one wave (lane k holding
// entry k: slot es, batch position ep, TD error et) in partition part, or
// in part and part + 1 (PAIR, the first's entries first).
template <bool PAIR>
__device__ __forceinline__ void bucket_repair(SparseSmem& sp, const TreePtrs& t, const Geom& g,
                                              const UpdateArgs& a, uint32_t part, uint32_t m,
                                              uint32_t es, uint32_t ep, float et, float m0,
                                              uint32_t* max_dst) {
  const int lane = threadIdx.x & 63;
  uint32_t pb = 0u;
  if ((uint32_t)lane < m) {
    const float p = collect<true, true>(sp, lane, t, g, part, es - (part << kMaxSpanBits), ep, et,
                                        m0, a.alpha, a.eps, a.p_nan);
    pb = __float_as_uint(p);
  }
  pb = wave_max_u32(pb);
  if (lane == 0) publish_max(pb, false, m0, max_dst);
  // The wave reads what its own lanes wrote to its sparse area: LDS
  // operations of one wave complete in order.
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  wave_update<true, PAIR>(sp, t, g, part, (int)m);
}

// Large batches, step 2, for thin batches over many full partitions: as
// update_bucket_kernel, with eight partitions per block and the pair 2w,
// 2w + 1 to wave w.  When the two buckets fit one wave together, lane k
// takes entry k of the first and the second's entries follow it (moved
// down the lanes by a shuffle), and one sort and one chain repair both
// partitions.  A wave's chain costs the same instructions whether it
// carries 16 entries or 32, and with every wave of the grid resident the
// chains are bound by instruction issue, so this halves their cost.  Two
// buckets that do not fit one wave are repaired one after the other;
// crowded partitions are rebuilt by the whole block after.
__global__ void __launch_bounds__(kUpdThreads) update_bucket_pair_kernel(uint32_t* counts,
                                                                         const uint32_t* slot,
                                                                         const uint32_t* pos,
                                                                         const float* etd, uint32_t np,
                                                                         TreePtrs t, Buckets bk, Geom g,
                                                                         UpdateArgs a) {
  constexpr int PPB = 8;
  __shared__ UpdSmem<PPB> sm;
  // As in update_bucket_kernel: the counts and both buckets' entries are
  // loaded first, through the preloaded leading arguments.
  const uint32_t part0 = blockIdx.x * PPB;
  const int nparts = (int)min((uint32_t)PPB, np - part0);
  const int w = threadIdx.x >> 6, lane = threadIdx.x & 63;
  uint32_t cnt = 0u;
  if (threadIdx.x < (unsigned)nparts) cnt = counts[(part0 + threadIdx.x) * kCountStride];
  uint32_t es[2] = {0u, 0u}, ep[2] = {0u, 0u};
  float et[2] = {0.0f, 0.0f};
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (2 * w + h < nparts) {
      const uint32_t e = (part0 + 2 * w + h) * kBucketCap + lane;
      es[h] = slot[e];
      ep[h] = pos[e];
      et[h] = etd[e];
    }
  }
  asm volatile("" ::"s"(t.ctrl), "s"(a.src), "s"(a.dst), "s"(a.ovf), "s"(g.n));
  const float m0 = __uint_as_float(t.ctrl->maxp_bits[a.src]);
  uint32_t* max_dst = &t.ctrl->maxp_bits[a.dst];
  if (threadIdx.x < (unsigned)nparts) {
    sm.mtot[threadIdx.x] = cnt;
    counts[(part0 + threadIdx.x) * kCountStride] = 0u;  // ready for the next call's bucketing
  }
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    bk.ovf_n[a.ovf ^ 1] = 0u;  // the next call's overflow counter
    publish_max(0u, true, m0, max_dst);
  }
  __syncthreads();
  bool crowded = false;
  for (int q = 0; q < nparts; ++q) crowded |= sm.mtot[q] > (uint32_t)kBucketCap;
  const uint32_t pa = part0 + 2 * w;  // the wave's first partition
  const uint32_t ma = 2 * w < nparts ? sm.mtot[2 * w] : 0u;
  const uint32_t mb = 2 * w + 1 < nparts ? sm.mtot[2 * w + 1] : 0u;
  const bool sa = ma > 0u && ma <= (uint32_t)kBucketCap;
  const bool sb = mb > 0u && mb <= (uint32_t)kBucketCap;
  if (sa && sb && ma + mb <= (uint32_t)kSparseMax) {  // uniform across the wave
    const int src = lane >= (int)ma ? lane - (int)ma : 0;
    const uint32_t s1 = (uint32_t)__shfl((int)es[1], src);
    const uint32_t p1 = (uint32_t)__shfl((int)ep[1], src);
    const float t1 = __shfl(et[1], src);
    const bool first = (uint32_t)lane < ma;
    bucket_repair<true>(sm.u.sp[2 * w], t, g, a, pa, ma + mb, first ? es[0] : s1,
                        first ? ep[0] : p1, first ? et[0] : t1, m0, max_dst);
  } else {
    if (sa) bucket_repair<false>(sm.u.sp[2 * w], t, g, a, pa, ma, es[0], ep[0], et[0], m0, max_dst);
    if (sb)
      bucket_repair<false>(sm.u.sp[2 * w + 1], t, g, a, pa + 1u, mb, es[1], ep[1], et[1], m0,
                           max_dst);
  }
  if (!crowded) return;
  // The dense rebuild reuses the sparse areas: every wave is done with them.
  __syncthreads();
  const uint32_t novf = bk.ovf_n[a.ovf];
  for (int q = 0; q < nparts; ++q) {
    if (sm.mtot[q] <= (uint32_t)kBucketCap) continue;
    const uint32_t part = part0 + q, base = part << g.S;
    const uint32_t* bslot = bk.slot + part * kBucketCap;
    const uint32_t* bpos = bk.pos + part * kBucketCap;
    const float* btd = bk.td + part * kBucketCap;
    const uint32_t mbits = dense_update<kUpdThreads>(sm.u.dn, sm.flag, sm.sx, t, g, part, [&](auto f) {
      for (uint32_t k = threadIdx.x; k < kBucketCap; k += kUpdThreads)
        f(bslot[k] - base, bpos[k], priority_of(btd[k], m0, a.alpha, a.eps, a.p_nan));
      for (uint32_t k = threadIdx.x; k < novf; k += kUpdThreads) {
        const uint32_t i = bk.oslot[k];
        if ((i >> g.S) == part)
          f(i - base, bk.opos[k], priority_of(bk.otd[k], m0, a.alpha, a.eps, a.p_nan));
      }
    });
    if (threadIdx.x == 0) publish_max(mbits, false, m0, max_dst);
  }
}

// Partitions touched by the ring range [cursor, cursor + count): one run,
// or two when the range wraps past the end and the runs stay apart.
struct TouchedRuns {
  uint32_t first[2], len[2];
};

__host__ __device__ inline TouchedRuns touched_runs(uint32_t cursor, uint32_t count,
                                                    const Geom& g) {
  const uint64_t end = (uint64_t)cursor + count;
  const uint32_t hi0 = (uint32_t)(end < g.n ? end : g.n);
  uint32_t f0 = cursor >> g.S, l0 = (hi0 - 1) >> g.S;  // inclusive
  uint32_t l1 = 0;
  bool second = end > g.n;
  if (second) {
    l1 = (uint32_t)(end - g.n - 1) >> g.S;
    if (l1 + 1 >= f0) {  // the two runs meet or overlap: one run over every partition
      f0 = 0;
      l0 = (1u << g.P) - 1;
      second = false;
    }
  }
  TouchedRuns r;
  r.first[0] = f0;
  r.len[0] = l0 - f0 + 1;
  r.first[1] = 0;
  r.len[1] = second ? l1 + 1 : 0;
  return r;
}

struct AddArgs {
  uint32_t cursor, count;  // cursor: host-tracked, unless ring.dev
  uint32_t size;           // filled slots before the intake: host-tracked, unless ring.dev
  RingRef ring;            // ring.dev: cursor and size come from ctrl slot ring.slot
  const float* prio;
  uint32_t ntree;  // blocks set aside for tree work (the rest copy rows)
  uint32_t last;   // the launch's last block, which commits the ring state
  int src, dst;    // running-max slots: read / raise
  const float* states;
  const float* next_states;
  const uint32_t* actions;
  const float* rewards;
  const uint8_t* dones;
};

// The ring state before an intake: the launch's, or the device's (graph mode).
__device__ __forceinline__ void ring_state(const TreePtrs& t, const AddArgs& a, uint32_t& cursor,
                                           uint32_t& size) {
  cursor = a.cursor;
  size = a.size;
  if (a.ring.dev) {
    cursor = t.ctrl->cursor[a.ring.slot];
    size = t.ctrl->size[a.ring.slot];
  }
}

// The ring state after the intake goes to the other slot, so that no block
// of the launch reads a value another block has changed.  One thread of the
// last block: a row-copy block whenever rows are kept, with no barrier to
// wait on the store.
__device__ __forceinline__ void commit_ring(const TreePtrs& t, const Geom& g, const AddArgs& a,
                                            uint32_t cursor, uint32_t size) {
  if (blockIdx.x == a.last && threadIdx.x == 0) {
    const uint64_t next = (uint64_t)cursor + a.count;
    const uint64_t filled = (uint64_t)size + a.count;
    t.ctrl->cursor[a.ring.slot ^ 1] = (uint32_t)(next >= g.n ? next - g.n : next);
    t.ctrl->size[a.ring.slot ^ 1] = (uint32_t)(filled < g.n ? filled : g.n);
  }
}

// Row copy of the intake's transitions into their ring slots, by the blocks
// [first, a.last] of the launch.
__device__ __forceinline__ void copy_intake_rows(const Storage& st, const Geom& g, const AddArgs& a,
                                 uint32_t cursor, uint32_t first) {
  const uint32_t nb = a.last + 1u - first;
  const uint32_t tid = (blockIdx.x - first) * kTreeThreads + threadIdx.x;
  const uint32_t stride = nb * kTreeThreads;
  const uint32_t D = (uint32_t)st.D;
  if ((D & 3u) == 0u) {
    const uint32_t c4 = D >> 2;
    const uint64_t total = (uint64_t)a.count * c4;
    for (uint64_t e = tid; e < total; e += stride) {
      const uint32_t j = (uint32_t)(e / c4), c = (uint32_t)(e % c4);
      uint32_t slot = cursor + j;
      if (slot >= g.n) slot -= g.n;
      const uint64_t so = (uint64_t)j * D + 4u * c, dof = (uint64_t)slot * D + 4u * c;
      *reinterpret_cast<float4*>(st.states + dof) =
          *reinterpret_cast<const float4*>(a.states + so);
      *reinterpret_cast<float4*>(st.next_states + dof) =
          *reinterpret_cast<const float4*>(a.next_states + so);
    }
  } else {
    const uint64_t total = (uint64_t)a.count * D;
    for (uint64_t e = tid; e < total; e += stride) {
      const uint32_t j = (uint32_t)(e / D), c = (uint32_t)(e % D);
      uint32_t slot = cursor + j;
      if (slot >= g.n) slot -= g.n;
      st.states[(uint64_t)slot * D + c] = a.states[e];
      st.next_states[(uint64_t)slot * D + c] = a.next_states[e];
    }
  }
  for (uint32_t j = tid; j < a.count; j += stride) {
    uint32_t slot = cursor + j;
    if (slot >= g.n) slot -= g.n;
    st.actions[slot] = a.actions[j];
    st.rewards[slot] = a.rewards[j];
    st.dones[slot] = a.dones[j];
  }
}

// The ring range [cursor, cursor + count) split at the wrap -- [cursor,
// min(end, n)) and, past the wrap, [0, end - n) -- and clipped to partition
// `part`: runs of offsets [lo0, hi0) and, when both meet it, [0, hi1).
struct IntakeRuns {
  int runs;  // 0, 1 or 2
  uint32_t lo0, hi0, hi1;

  __device__ bool has(uint32_t off) const {
    return (off >= lo0 && off < hi0) || (runs == 2 && off < hi1);
  }
};

template <bool FULL>
__device__ __forceinline__ IntakeRuns intake_runs(uint32_t cursor, uint32_t count, const Geom& g,
                                                  uint32_t part) {
  const uint32_t span = 1u << span_bits<FULL>(g);
  const uint32_t base = part << span_bits<FULL>(g);
  const uint64_t end = (uint64_t)cursor + count;
  const uint32_t a_lo = max(cursor, base);
  const uint32_t a_hi = min((uint32_t)(end < g.n ? end : g.n), base + span);
  const uint32_t b_hi = min((uint32_t)(end > g.n ? end - g.n : 0u), base + span);
  const bool has_a = a_lo < a_hi, has_b = base < b_hi;
  IntakeRuns r;
  r.runs = (int)has_a + (int)has_b;
  r.lo0 = has_a ? a_lo - base : 0u;
  r.hi0 = has_a ? a_hi - base : (has_b ? b_hi - base : 0u);
  r.hi1 = has_b ? b_hi - base : 0u;
  return r;
}

// The intake's slots in partition `part` -- the ring range [cursor, cursor +
// count) clipped to it: one run, or two when the ring wraps inside it --
// take the given priorities (prio[j] for the range's j-th slot) or v, and
// the nodes above them are repaired up to the partition root.  Given
// priorities raise the running max at max_dst: thread 0 publishes the
// block's max, carrying v over when carry is set and otherwise only when it
// exceeds v (v must then already be there).  RANGE: sm holds a RangeSmem
// for the LDS repair of a single run of given priorities; without one such
// a run is rebuilt like two.  Returns at once when the range misses the
// partition.  Every argument is block-uniform.
template <bool RANGE, bool FULL, typename SM>
__device__ __forceinline__ void intake_partition(SM& sm, const TreePtrs& t, const Geom& g,
                                                 uint32_t part, uint32_t cursor, uint32_t count,
                                                 const float* prio, float v, bool carry,
                                                 uint32_t* max_dst) {
  const uint32_t base = part << g.S;
  const IntakeRuns ir = intake_runs<FULL>(cursor, count, g, part);
  const int runs = ir.runs;
  const uint32_t lo0 = ir.lo0, hi0 = ir.hi0, hi1 = ir.hi1;
  if (runs == 0) return;
  if (runs == 1 && !prio) {
    // One run at the running max (the usual intake): no LDS, no barrier.
    float sib_s = 0.0f, sib_m = 0.0f;
    load_range_boundary<FULL>(t, g, part, lo0, hi0, sib_s, sib_m);
    uniform_range<FULL>(t, g, part, lo0, hi0, v, sib_s, sib_m);
    return;
  }
  // One run: its boundary siblings go out with the other loads.
  if constexpr (RANGE) {
    if (runs == 1) prefetch_range_boundaries(sm.u.r, t, g, part, lo0, hi0);
  }
  auto value_of = [&](uint32_t off) -> float {
    const uint32_t slot = base + off;
    const uint32_t j = (slot >= cursor) ? slot - cursor : slot + (g.n - cursor);
    return prio ? prio[j] + 0.0f : v;
  };
  // f(off) for every new offset of the partition, spread over the block.
  auto each_offset = [&](auto f) {
    for (uint32_t off = lo0 + threadIdx.x; off < hi0; off += kTreeThreads) f(off);
    if (runs == 2)
      for (uint32_t off = threadIdx.x; off < hi1; off += kTreeThreads) f(off);
  };
  uint32_t mb = 0;
  each_offset([&](uint32_t off) {
    const float p = value_of(off);
    mb = max(mb, __float_as_uint(p));
    if constexpr (RANGE) {
      if (runs == 1) sm.u.r.val[off] = p;
    }
  });
  if (prio) {
    mb = block_max_bits<kTreeThreads>(mb, sm.sx);
    if (threadIdx.x == 0) publish_max(mb, carry, v, max_dst);
  }
  __syncthreads();
  if constexpr (RANGE) {
    if (runs == 1) {
      range_repair(sm.u.r, t, g, part, lo0, hi0);
      return;
    }
  }
  // Two runs in one partition (the ring wrapped inside it): general rebuild;
  // slots are distinct, so the offset doubles as the batch position.
  dense_update<kTreeThreads>(sm.u.dn, sm.flag, sm.sx, t, g, part, [&](auto f) {
    each_offset([&](uint32_t off) { f(off, off, value_of(off)); });
  });
}

// Ring intake ("GPU-Resident Prioritized Experience Replay", section
// "Experience Insertion"): new slots take the given priority or the running
// max priority; rows are copied by the blocks past the tree blocks.
template <bool FULL>
__global__ void __launch_bounds__(256) add_kernel(TreePtrs t, Geom g, Storage st, AddArgs a) {
  __shared__ AddSmem sm;
  // The arguments the first steps need, fetched in one batch.
  asm volatile("" ::"s"(t.ctrl), "s"(a.cursor), "s"(a.count), "s"(a.size), "s"(a.ring.dev),
               "s"(a.last), "s"(a.ntree), "s"(a.src), "s"(a.prio), "s"(g.n), "s"(g.S));
  uint32_t cursor, size;
  ring_state(t, a, cursor, size);
  commit_ring(t, g, a, cursor, size);
  if (blockIdx.x >= a.ntree) {
    copy_intake_rows(st, g, a, cursor, a.ntree);
    return;
  }
  const uint32_t w = blockIdx.x;
  const TouchedRuns tr = touched_runs(cursor, a.count, g);
  if (w >= tr.len[0] + tr.len[1]) return;  // spare block of a worst-case grid
  const uint32_t part = (w < tr.len[0]) ? tr.first[0] + w : tr.first[1] + (w - tr.len[0]);
  const float m0 = __uint_as_float(t.ctrl->maxp_bits[a.src]);
  intake_partition<true, FULL>(sm, t, g, part, cursor, a.count, a.prio, m0, w == 0,
                               &t.ctrl->maxp_bits[a.dst]);
}

// LDS of the fused update + intake block when the intake brings its own
// priorities: the update's areas and the intake's range repair share it.
template <bool WL = false>
struct UpdAddSmem {
  union {
    SparseSmem sp[1];
    DenseSmem dn;
    RangeSmem r;
  } u;
  BlockScratch sx;
  int count[1];
  uint32_t mtot[1];
  uint32_t bmax;
  uint32_t ball;
  int flag;
  std::conditional_t<WL, WaveLists, NoWaveLists> wl;  // last: the others' offsets stay put
};

// Whether f32(pow(y, alpha)) <= m0 for every y <= ys, decided by f32
// logarithms (2^-16 <= alpha <= 16): true when alpha log2(ys) lies below
// log2(m0) by more than 2^-12 (1 + |alpha log2 ys| + |log2 m0|).  Rounding ys
// and alpha to f32, the product and each logarithm (taken as within 2^-20 +
// 2^-21 |result|) move the two sides by under 2^-15 (1 + |alpha log2 ys| +
// |log2 m0|) together, so then ys^alpha < m0 (1 - 2^-13), and the f64 pow,
// within a few of its ulps, rounds to at most m0.  Zero, infinite and NaN
// operands make a side infinite or NaN and the answer false.
__device__ __forceinline__ bool stays_below(double ys, float m0, double alpha) {
  if (alpha > 16.0) return false;
  const float za = (float)alpha * log2f((float)ys), lm = log2f(m0);
  return za < lm - 0x1p-12f * (1.0f + fabsf(za) + fabsf(lm));
}

// The max priority bits over the batch entries b = first, first + stride,
// ... with an index in [0, size): what priority_of gives each (NaN and
// infinite TD errors included).  Called by whole waves (stride a multiple of
// 64).  p = f32(pow(|td| + eps, alpha)) rises with |td|, and an entry whose y
// = |td| + eps lies below y* (1 - 2^-24), y* the largest finite one of its
// wave and chunk, has an exact p at least a factor (1 - 2^-24)^alpha <= 1 -
// 2^-41 (alpha >= 2^-16) below that of y*: far more than the few-ulp error
// of the f64 pow, so it cannot exceed the max after rounding.  So only the
// entries at or above that bound are raised to alpha, and none when even y*
// cannot lift the priority above m0 (stays_below): the caller takes the max
// with m0, so a result below m0 is as good as the exact one there.
__device__ __forceinline__ uint32_t batch_max_bits(const UpdateArgs& a, uint32_t size, float m0,
                                                   uint32_t first, uint32_t stride) {
  constexpr int kC = 4;
  const bool few = a.alpha >= 0x1p-16;
  uint32_t mall = 0u;
  for (uint32_t b0 = 0; b0 < a.B; b0 += stride * kC) {  // the same trips in every wave
    int64_t ix[kC];
    float tx[kC];
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      const uint32_t b = b0 + c * stride + first;
      ix[c] = -1;
      tx[c] = 0.0f;
      if (b < a.B) {
        ix[c] = a.idx[b];
        tx[c] = a.td[b];
      }
    }
    uint32_t pend = 0u, xb = 0u;
#pragma unroll
    for (int c = 0; c < kC; ++c) {
      if (ix[c] < 0 || ix[c] >= (int64_t)size) continue;
      const float x = fabsf(tx[c]);
      if (__builtin_isnan(x)) {
        mall = max(mall, __float_as_uint(a.p_nan));
      } else if (__builtin_isinf(x)) {
        mall = max(mall, __float_as_uint(m0));
      } else {
        xb = max(xb, __float_as_uint(x));
        pend |= 1u << c;
      }
    }
    if (few) {
      const double ys = (double)__uint_as_float(wave_max_u32(xb)) + a.eps;
      const double bound = ys - ys * 0x1p-24;
#pragma unroll
      for (int c = 0; c < kC; ++c)
        if (((pend >> c) & 1u) && (double)fabsf(tx[c]) + a.eps < bound) pend &= ~(1u << c);
      if (stays_below(ys, m0, a.alpha)) pend = 0u;
    }
    while (__ballot(pend != 0u) != 0ull) {  // one entry per lane per round
      if (pend != 0u) {
        const int c = __builtin_ctz(pend);
        pend &= pend - 1u;
        float td = tx[0];
#pragma unroll
        for (int cc = 1; cc < kC; ++cc)
          if (c == cc) td = tx[cc];
        mall = max(mall, __float_as_uint(priority_of(td, m0, a.alpha, a.eps, a.p_nan)));
      }
    }
  }
  return mall;
}

// An update batch followed by an intake in one launch, with the result of
// the two calls in that order.  Block `part` of the first 2^P updates its
// partition from the batch as the scan path does, then applies the intake's
// slots in it, if the ring range meets it, on top of the repaired subtree.
// At the running max (PRIO false) those slots take the max after the
// update: the value at the start or a larger priority of the batch, which
// such a block gathers from the whole batch while scanning it.  Both raise
// the running max in the same slot (a.dst == b.dst).  Blocks past the first
// 2^P copy the intake's rows.
template <bool PRIO, bool FULL, int CH>
__global__ void __launch_bounds__(kUpdThreads) update_add_kernel(const int64_t* bidx, const float* btd,
                                                                 uint32_t bB, Ctrl* ctrl, TreePtrs t,
                                                                 Geom g, Storage st, UpdateArgs a,
                                                                 AddArgs b) {
  __shared__ std::conditional_t<PRIO, UpdAddSmem<(CH >= 4 && FULL)>, UpdSmem<1, (CH >= 4 && FULL)>> sm;
  // The batch and the control block arrive in scalar registers with the
  // wave (the leading arguments, preloaded; the same as a's and t's), so
  // the batch's first chunk is loaded before anything else.
  int64_t ix0[CH];
  float tx0[CH];
  load_chunk<CH>(bidx, btd, bB, 0, ix0, tx0);
  const Ctrl c = *ctrl;
  a.idx = bidx;
  a.td = btd;
  a.B = bB;
  t.ctrl = ctrl;
  // The other arguments the first steps need, fetched in one batch: left to
  // itself, the compiler loads each after the branch that first needs it,
  // one dependent trip each.
  asm volatile("" ::"s"(a.src), "s"(b.cursor), "s"(b.count), "s"(b.size), "s"(b.ring.dev),
               "s"(b.ring.slot), "s"(b.last), "s"(g.n), "s"(g.S));
  PER_STAMP(0, 0);
  PER_STAMP(1, 7);
  // The ring state before the intake: the launch's, or the device's (graph
  // mode), from the control block's copy.
  const uint32_t cursor = b.ring.dev ? ctrl_word(c.cursor, b.ring.slot) : b.cursor;
  const uint32_t size = b.ring.dev ? ctrl_word(c.size, b.ring.slot) : b.size;
  commit_ring(t, g, b, cursor, size);
  const uint32_t np = 1u << g.P;
  if (blockIdx.x >= np) {
    copy_intake_rows(st, g, b, cursor, np);
    return;
  }
  const uint32_t part = blockIdx.x;
  const IntakeRuns ir = intake_runs<FULL>(cursor, b.count, g, part);
  const float m0 = __uint_as_float(ctrl_word(c.maxp_bits, a.src));
  // Update entries at slots the intake takes are left out of the repair
  // (the intake overwrites them; their priorities still count).
  const bool crowded = scan_update<1, true, FULL, CH, kScanLine>(
      sm, t, g, a, part, size, m0, ix0, tx0, [&](uint32_t off) { return ir.has(off); });
  if (ir.runs == 0) return;
  if constexpr (PRIO) {
    // The update's repair is complete, and visible to the whole block,
    // before the intake reads the nodes around its run.
    __syncthreads();
    intake_partition<PRIO, FULL>(sm, t, g, part, cursor, b.count, b.prio, m0, false,
                                 &t.ctrl->maxp_bits[b.dst]);
  } else {
    // At the running max the intake takes the max priority over the whole
    // batch (the value at the start or a larger one of the batch): waves 1-3
    // compute it while wave 0 finishes the partition's sparse repair and, for
    // the usual single run, loads the run's boundary siblings, which in
    // program order see that repair's stores.  The update's new leaves are
    // all outside the run, so its repaired nodes meet the intake's only on
    // the run's two boundary paths, which wave 0 climbs; the run's interior
    // nodes are the intake's alone.
    const bool one = ir.runs == 1 && !crowded;
    float sib_s = 0.0f, sib_m = 0.0f;
    if (threadIdx.x >= 64) {
      const uint32_t wm = wave_max_u32(batch_max_bits(a, size, m0, threadIdx.x - 64,
                                                      kUpdThreads - 64));
      if ((threadIdx.x & 63) == 0) atomicMax(&sm.ball, wm);
      PER_STAMP(1, 6);
    } else if (one) {
      load_range_boundary<FULL>(t, g, part, ir.lo0, ir.hi0, sib_s, sib_m);
    }
    PER_STAMP(0, 3);
    __syncthreads();
    PER_STAMP(0, 4);
    const float v = __uint_as_float(max(__float_as_uint(m0), sm.ball));
    if (one) {
      uniform_range<FULL>(t, g, part, ir.lo0, ir.hi0, v, sib_s, sib_m);
      return;
    }
    intake_partition<PRIO, FULL>(sm, t, g, part, cursor, b.count, b.prio, v, false,
                                 &t.ctrl->maxp_bits[b.dst]);
  }
}

// Nodes [1, 2^P) above the partitions, recomputed from depth P upwards.
struct TopSmem {
  float s[1 << kMaxTopBits];
  float m[1 << kMaxTopBits];
};

__global__ void __launch_bounds__(256) top_kernel(TreePtrs t, Geom g) {
  __shared__ TopSmem sm;
  const uint32_t np = 1u << g.P;
  if (g.P <= kMaxTopBits) {
    const uint32_t half = np >> 1;
    for (uint32_t h = half + threadIdx.x; h < np; h += kTreeThreads) {
      const float2 cs = *reinterpret_cast<const float2*>(t.sum + 2 * h);
      const float2 cm = *reinterpret_cast<const float2*>(t.mn + 2 * h);
      sm.s[h] = cs.x + cs.y;
      sm.m[h] = min_f32(cm.x, cm.y);
    }
    // In LDS level by level, stored once after the last barrier (a barrier
    // also waits for outstanding global stores).
    for (uint32_t width = half >> 1; width >= 1; width >>= 1) {
      __syncthreads();
      for (uint32_t h = width + threadIdx.x; h < 2 * width; h += kTreeThreads) {
        sm.s[h] = sm.s[2 * h] + sm.s[2 * h + 1];
        sm.m[h] = min_f32(sm.m[2 * h], sm.m[2 * h + 1]);
      }
    }
    __syncthreads();
    for (uint32_t h = 1 + threadIdx.x; h < np; h += kTreeThreads) {
      t.sum[h] = sm.s[h];
      t.mn[h] = sm.m[h];
    }
  } else {
    // More top nodes than LDS holds: level by level through global memory.
    for (int l = g.P - 1; l >= 0; --l) {
      const uint32_t lo = 1u << l;
      for (uint32_t h = lo + threadIdx.x; h < 2 * lo; h += kTreeThreads) {
        t.sum[h] = t.sum[2 * h] + t.sum[2 * h + 1];
        t.mn[h] = min_f32(t.mn[2 * h], t.mn[2 * h + 1]);
      }
      __threadfence_block();
      __syncthreads();
    }
  }
}

// Batch entries per thread and chunk of the update scan: the batch over the
// block's threads, rounded up to 2, 4, 8 or 16 (larger batches take more
// chunks; the fused update + intake stops at 8).  One chunk means that every
// load of the batch goes out at kernel entry (2^21 leaves, 4096 entries:
// update 8.25 -> 7.7 us with 16 against two chunks of 8).
inline int scan_chunk(int64_t B) {
  return B <= 2 * kUpdThreads ? 2 : (B <= 4 * kUpdThreads ? 4 : (B <= 8 * kUpdThreads ? 8 : 16));
}

// The fewest blocks the bucketed repair with two partitions per wave is
// launched with: one per CU of the MI355X.
constexpr uint32_t kPairMinBlocks = 256;

inline unsigned grid_for(uint64_t work, unsigned per_block, unsigned cap) {
  uint64_t b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_init(const TreePtrs& t, const Buckets& bk, const Geom& g, hipStream_t s) {
  const unsigned grid = grid_for(2ull * g.n, kTreeThreads * 8, 4096);
  return launch_kernel(init_kernel, dim3(grid), dim3(kTreeThreads), 0, s, t, bk, g);
}

hipError_t launch_top(const TreePtrs& t, const Geom& g, hipStream_t s) {
  return launch_kernel(top_kernel, dim3(1), dim3(kTreeThreads), 0, s, t, g);
}

hipError_t launch_bucket_clear(const Buckets& bk, const Geom& g, hipStream_t s) {
  const uint32_t np = 1u << g.P;
  return launch_kernel(bucket_clear_kernel, dim3(grid_for(np, kTreeThreads, 64)),
                       dim3(kTreeThreads), 0, s, bk, np);
}

bool update_uses_buckets(const Geom& g, int64_t B) {
  // Every partition's block scans the batch: np * B loads in all.  Past 2^21
  // of them, bucket the batch first (measured: 4096 entries on 512
  // partitions update in 8.6 us by the scan, 10.2 us bucketed).
  const uint64_t np = 1ull << g.P;
  return np * (uint64_t)B > (1ull << 21);
}

hipError_t launch_update(const TreePtrs& t, const Buckets& bk, const Geom& g, RingRef ring,
                         uint32_t size, int64_t B, const int64_t* idx, const float* td,
                         double alpha, double eps, int src, int dst, int ovf, hipStream_t s) {
  UpdateArgs a;
  a.ring = ring;
  a.ring_ctrl = t.ctrl;
  a.idx = idx;
  a.td = td;
  a.B = (uint32_t)B;
  a.size = size;
  a.alpha = alpha;
  a.eps = eps;
  a.p_nan = (float)pow(eps, alpha);
  a.src = src;
  a.dst = dst;
  a.ovf = ovf;
  const uint64_t np = 1ull << g.P;
  if (!update_uses_buckets(g, B)) {
    // One partition per block: the batch scan is spread over the most blocks.
    const int ch = scan_chunk(B);
    const dim3 grid((unsigned)np), block(kUpdThreads);
    if (g.S == kMaxSpanBits && ch == 2)
      return launch_kernel(update_scan_kernel<1, true, 2, kScanLine>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, a);
    if (g.S == kMaxSpanBits && ch == 4)
      return launch_kernel(update_scan_kernel<1, true, 4, kScanLine>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, a);
    if (g.S == kMaxSpanBits && ch == 8)
      return launch_kernel(update_scan_kernel<1, true, 8, kScanLine>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, a);
    if (g.S == kMaxSpanBits)
      return launch_kernel(update_scan_kernel<1, true, 16, kScanLine>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, a);
    return launch_kernel(update_scan_kernel<1, false, 8, false>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, a);
  }
  // Bucketed: four partitions per block, one wave each, while the batch
  // spreads thin over the partitions (<= 16 entries each on average), so
  // that every wave of a block repairs; denser batches take one partition
  // per block, so that crowded partitions are rebuilt in parallel.
  const bool thin = (uint64_t)B <= 16 * np;
  const unsigned grid = thin ? (unsigned)((np + 3) / 4) : (unsigned)np;
  const unsigned eb = grid_for((uint64_t)B, kTreeThreads, 1u << 30);
  hipError_t e = launch_kernel(bucket_kernel, dim3(eb), dim3(kTreeThreads), 0, s, a.idx, a.td, a.B,
                               bk.counts, bk, g, a);
  if (e != hipSuccess) return e;
  const bool full = g.S == kMaxSpanBits;
  // Two partitions per wave while eight per block still give at least one
  // block per CU.
  if (thin && full && np >= 8u * kPairMinBlocks)
    return launch_kernel(update_bucket_pair_kernel, dim3((unsigned)(np / 8)), dim3(kUpdThreads), 0, s,
                         bk.counts, bk.slot, bk.pos, bk.td, np, t, bk, g, a);
  if (thin && full)
    return launch_kernel(update_bucket_kernel<4, true>, dim3(grid), dim3(kUpdThreads), 0, s,
                         bk.counts, bk.slot, bk.pos, bk.td, np, t, bk, g, a);
  if (thin)
    return launch_kernel(update_bucket_kernel<4, false>, dim3(grid), dim3(kUpdThreads), 0, s,
                         bk.counts, bk.slot, bk.pos, bk.td, np, t, bk, g, a);
  if (full)
    return launch_kernel(update_bucket_kernel<1, true>, dim3(grid), dim3(kUpdThreads), 0, s,
                         bk.counts, bk.slot, bk.pos, bk.td, np, t, bk, g, a);
  return launch_kernel(update_bucket_kernel<1, false>, dim3(grid), dim3(kUpdThreads), 0, s,
                         bk.counts, bk.slot, bk.pos, bk.td, np, t, bk, g, a);
}

hipError_t launch_add(const TreePtrs& t, const Geom& g, const Storage& st, RingRef ring,
                      uint32_t size, uint32_t cursor, uint32_t count, const float* states,
                      const float* next_states, const uint32_t* actions, const float* rewards,
                      const uint8_t* dones, const float* prio, int src, int dst, hipStream_t s) {
  AddArgs a;
  a.cursor = cursor;
  a.count = count;
  a.size = size;
  a.ring = ring;
  a.prio = prio;
  a.src = src;
  a.dst = dst;
  a.states = states;
  a.next_states = next_states;
  a.actions = actions;
  a.rewards = rewards;
  a.dones = dones;
  const uint32_t np = 1u << g.P;
  if (ring.dev) {
    // The cursor is known only on the device: enough tree blocks for any
    // placement of count slots (a cyclic range of c slots meets at most
    // c / span + 2 partitions); the spare ones return at once.
    const uint64_t worst = ((uint64_t)count >> g.S) + 2;
    a.ntree = worst < np ? (uint32_t)worst : np;
  } else {
    const TouchedRuns tr = touched_runs(cursor, count, g);
    a.ntree = tr.len[0] + tr.len[1];
  }
  unsigned ncopy = 0;
  if (st.D > 0)
    ncopy = grid_for((uint64_t)count * (uint64_t)st.D / 4 + count, kTreeThreads * 4, 2048);
  a.last = a.ntree + ncopy - 1u;
  if (g.S == kMaxSpanBits)
    return launch_kernel(add_kernel<true>, dim3(a.ntree + ncopy), dim3(kTreeThreads), 0, s, t, g,
                         st, a);
  return launch_kernel(add_kernel<false>, dim3(a.ntree + ncopy), dim3(kTreeThreads), 0, s, t, g,
                       st, a);
}

hipError_t launch_update_add(const TreePtrs& t, const Geom& g, const Storage& st, RingRef ring,
                             uint32_t size, uint32_t cursor, int64_t B, const int64_t* idx,
                             const float* td, double alpha, double eps, uint32_t count,
                             const float* states, const float* next_states,
                             const uint32_t* actions, const float* rewards, const uint8_t* dones,
                             const float* prio, int src, int dst, hipStream_t s) {
  UpdateArgs a;
  a.ring = ring;
  a.ring_ctrl = t.ctrl;
  a.idx = idx;
  a.td = td;
  a.B = (uint32_t)B;
  a.size = size;
  a.alpha = alpha;
  a.eps = eps;
  a.p_nan = (float)pow(eps, alpha);
  a.src = src;
  a.dst = dst;
  a.ovf = 0;
  AddArgs b;
  b.cursor = cursor;
  b.count = count;
  b.size = size;
  b.ring = ring;
  b.prio = prio;
  b.src = src;
  b.dst = dst;
  b.states = states;
  b.next_states = next_states;
  b.actions = actions;
  b.rewards = rewards;
  b.dones = dones;
  const uint32_t np = 1u << g.P;
  b.ntree = np;
  unsigned ncopy = 0;
  if (st.D > 0)
    ncopy = grid_for((uint64_t)count * (uint64_t)st.D / 4 + count, kTreeThreads * 4, 2048);
  b.last = np + ncopy - 1u;
  const bool full = g.S == kMaxSpanBits;
  const int ch = scan_chunk(B);
  const dim3 grid(np + ncopy), block(kUpdThreads);
  if (!full && prio)
    return launch_kernel(update_add_kernel<true, false, 8>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
  if (!full)
    return launch_kernel(update_add_kernel<false, false, 8>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
  if (prio && ch == 2)
    return launch_kernel(update_add_kernel<true, true, 2>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
  if (prio && ch == 4)
    return launch_kernel(update_add_kernel<true, true, 4>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
  if (prio)
    return launch_kernel(update_add_kernel<true, true, 8>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
  if (ch == 2)
    return launch_kernel(update_add_kernel<false, true, 2>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
  if (ch == 4)
    return launch_kernel(update_add_kernel<false, true, 4>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
  return launch_kernel(update_add_kernel<false, true, 8>, grid, block, 0, s, a.idx, a.td, a.B, t.ctrl, t, g, st, a, b);
}

}  // namespace per
