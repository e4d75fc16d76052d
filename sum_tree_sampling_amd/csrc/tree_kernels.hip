// tree_kernels.hip -- initialisation, batched priority update and ring intake
// of the sum + min tree on gfx950.
//
// Tree layout ("Putting prioritized replay's segment tree on a GPU", section
// "The Tree Under Every Prioritized Replay"): node i has children 2i and
// 2i+1, leaves at [n, 2n), sum tree and twin min tree in two [2n] f32 arrays.
//
// Both writers (update and intake) follow the same plan:
//  1. The leaves are cut into 2^P aligned partitions of 2^S leaves (S <= 12);
//     one 256-thread workgroup owns one partition, i.e. one subtree.
//  2. The workgroup collects the leaves it must set (for the update: the last
//     batch position per slot wins; for the intake: the ring range), writes
//     them, and repairs every dirty node of its subtree up to the partition
//     root.  Sparse partitions (<= 64 new leaves) are repaired by one wave:
//     each leaf's lane walks up its own chain until it meets the chain of its
//     right neighbour; siblings along the chains are fetched in one round of
//     independent loads and values meet through lane shuffles, so the levels
//     stay ordered without a barrier.  Dense partitions are rebuilt level by
//     level in LDS with a barrier between levels.
//  3. The last workgroup to finish (a device-scope completion counter)
//     rebuilds the 2^P - 1 nodes above the partitions and updates the running
//     max priority.
// Every node is recomputed from its two children, never updated by adding a
// delta, and no level is read before the level below it is complete (the
// dependency rule of section "The Race Condition Worth Writing Down").

#include "per_internal.h"

namespace per {
namespace {

__device__ __forceinline__ float min_f32(float a, float b) { return (b < a) ? b : a; }

// Priority of one TD error: f32 of (|td| + eps)^alpha in f64
// ("GPU-Resident Prioritized Experience Replay", section "Priority update";
// NaN / Inf clamp of section "Error Handling & Fallback": NaN takes the value
// of td = 0, computed on the host as p_nan, and +/-Inf the max at batch start).
__device__ __forceinline__ float priority_of(float td, float max_at_start, double alpha,
                                             double eps, float p_nan) {
  const float x = fabsf(td);
  if (__builtin_isnan(x)) return p_nan;
  if (__builtin_isinf(x)) return max_at_start;
  return (float)pow((double)x + eps, alpha);
}

struct PartSmem {
  float val[kMaxSpan];                 // new leaf value by offset in the partition
  union {
    int owner[kMaxSpan];               // last batch position per offset (update dedupe)
    struct {
      float s[kMaxSpan];
      float m[kMaxSpan];
    } heap;                            // local heap [1, 2^S) / top nodes [1, 2^P)
  } u;
  uint32_t bits[kMaxSpan / 32];        // offsets that receive a new leaf
  uint8_t dirty[kMaxSpan];             // dense repair: node has a new leaf below it
  uint16_t list[kSparseMax];           // sparse repair: sorted offsets
  int wsum[kTreeThreads / 64];
  uint32_t wmax[kTreeThreads / 64];
  int total;
  uint32_t last;
};

// Exclusive scan of one int per thread over the 256-thread block.
__device__ int block_excl_scan(int v, PartSmem& sm, int* total) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    int y = __shfl_up(x, o);
    if (lane >= o) x += y;
  }
  if (lane == 63) sm.wsum[w] = x;
  __syncthreads();
  int off = 0, tot = 0;
#pragma unroll
  for (int k = 0; k < kTreeThreads / 64; ++k) {
    off += (k < w) ? sm.wsum[k] : 0;
    tot += sm.wsum[k];
  }
  __syncthreads();
  *total = tot;
  return off + x - v;
}

// Block max of non-negative f32 values held as bits + 1 (0 = none).
__device__ uint32_t block_max_tagged(uint32_t v, PartSmem& sm) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, o));
  if (lane == 0) sm.wmax[w] = v;
  __syncthreads();
  uint32_t r = 0;
#pragma unroll
  for (int k = 0; k < kTreeThreads / 64; ++k) r = max(r, sm.wmax[k]);
  __syncthreads();
  return r;
}

__device__ __forceinline__ bool has_bit(const PartSmem& sm, uint32_t off) {
  return (sm.bits[off >> 5] >> (off & 31)) & 1u;
}

// Sparse repair by wave 0: U <= 64 sorted new leaves, lane i owns leaf i.
// d_i is the depth of the lowest common ancestor of leaves i and i+1 (P-1
// for the last leaf, whose chain ends at the partition root).  Lane i
// computes the nodes of its chain at depths L-1 .. d_i+1: it is the last
// (rightmost) new leaf under each of them.  When lane i's path enters a node
// X from the right child, X's left child holds new leaves iff the nearest
// lane j < i with d_j <= depth(X) has d_j == depth(X); that lane's chain ends
// exactly at the left child, whose value it holds, frozen.  Otherwise the
// other child is unchanged and its value was prefetched.
__device__ void sparse_repair(const PartSmem& sm, const TreePtrs& t, const Geom& g,
                              uint32_t part, int U) {
  const int lane = threadIdx.x;
  const bool valid = lane < U;
  const uint32_t off = valid ? sm.list[lane] : 0u;
  const uint32_t leaf = (part << g.S) + off;
  const uint32_t node = g.n + leaf;
  const float p = sm.val[off];
  if (valid) {
    t.sum[node] = p;
    t.mn[node] = p;
  }
  const uint32_t next_leaf = __shfl_down(leaf, 1);
  int d = g.P - 1;
  if (lane < U - 1) d = g.L - 1 - (31 - __clz(leaf ^ next_leaf));

  float ps[kMaxSpanBits], pm[kMaxSpanBits];
#pragma unroll
  for (int k = 0; k < kMaxSpanBits; ++k) {
    ps[k] = 0.0f;
    pm[k] = 0.0f;
    if (k < g.S && valid && (g.L - 1 - k) > d) {
      const uint32_t sib = (node >> k) ^ 1u;
      ps[k] = t.sum[sib];
      pm[k] = t.mn[sib];
    }
  }

  float vs = p, vm = p;
  const uint64_t lanes_below = (1ull << lane) - 1ull;
#pragma unroll
  for (int k = 0; k < kMaxSpanBits; ++k) {
    if (k >= g.S) continue;     // uniform across the wave
    const int l = g.L - 1 - k;  // depth of the node computed at this step
    const uint64_t le = __ballot(valid && d <= l);
    const uint64_t below = le & lanes_below;
    const int src = below ? 63 - __clzll(below) : lane;
    const int d_src = __shfl(d, src);
    const float s_src = __shfl(vs, src);
    const float m_src = __shfl(vm, src);
    if (valid && d < l) {
      const uint32_t child = node >> k;
      const bool right = child & 1u;
      float os = ps[k], om = pm[k];
      if (right && below != 0ull && d_src == l) {
        os = s_src;
        om = m_src;
      }
      if (right) {
        vs = os + vs;
        vm = min_f32(om, vm);
      } else {
        vs = vs + os;
        vm = min_f32(vm, om);
      }
      const uint32_t parent = child >> 1;
      t.sum[parent] = vs;
      t.mn[parent] = vm;
    }
  }
}

// Dense repair by the whole block: rebuild the partition's subtree in LDS and
// write back the nodes with a new leaf below them.
__device__ void dense_repair(PartSmem& sm, const TreePtrs& t, const Geom& g, uint32_t part) {
  const uint32_t span = 1u << g.S, half = span >> 1;
  const uint32_t root = (1u << g.P) + part;
  const uint32_t leaf0 = g.n + (part << g.S);
  for (uint32_t k = threadIdx.x; k < span; k += kTreeThreads) {
    if (has_bit(sm, k)) {
      t.sum[leaf0 + k] = sm.val[k];
      t.mn[leaf0 + k] = sm.val[k];
    }
  }
  // local heap index h in [1, span) <-> global node ((root - 1) << depth(h)) + h
  for (uint32_t h = half + threadIdx.x; h < span; h += kTreeThreads) {
    const uint32_t a = 2 * h - span;
    const bool ba = has_bit(sm, a), bb = has_bit(sm, a + 1);
    float ls, lm, rs, rm;
    if (ba && bb) {
      ls = lm = sm.val[a];
      rs = rm = sm.val[a + 1];
    } else {
      const float2 os = *reinterpret_cast<const float2*>(t.sum + leaf0 + a);
      const float2 om = *reinterpret_cast<const float2*>(t.mn + leaf0 + a);
      ls = ba ? sm.val[a] : os.x;
      lm = ba ? sm.val[a] : om.x;
      rs = bb ? sm.val[a + 1] : os.y;
      rm = bb ? sm.val[a + 1] : om.y;
    }
    const float s = ls + rs, m = min_f32(lm, rm);
    sm.u.heap.s[h] = s;
    sm.u.heap.m[h] = m;
    sm.dirty[h] = ba | bb;
    if (ba | bb) {
      const uint32_t gnode = ((root - 1u) << (g.S - 1)) + h;
      t.sum[gnode] = s;
      t.mn[gnode] = m;
    }
  }
  for (uint32_t width = half >> 1, dl = g.S - 2; width >= 1; width >>= 1, --dl) {
    __syncthreads();
    for (uint32_t h = width + threadIdx.x; h < 2 * width; h += kTreeThreads) {
      const float s = sm.u.heap.s[2 * h] + sm.u.heap.s[2 * h + 1];
      const float m = min_f32(sm.u.heap.m[2 * h], sm.u.heap.m[2 * h + 1]);
      const uint8_t dv = sm.dirty[2 * h] | sm.dirty[2 * h + 1];
      sm.u.heap.s[h] = s;
      sm.u.heap.m[h] = m;
      sm.dirty[h] = dv;
      if (dv) {
        const uint32_t gnode = ((root - 1u) << dl) + h;
        t.sum[gnode] = s;
        t.mn[gnode] = m;
      }
    }
  }
}

// Repair the partition after sm.val / sm.bits hold its new leaves.
__device__ void repair_partition(PartSmem& sm, const TreePtrs& t, const Geom& g,
                                 uint32_t part) {
  const uint32_t nwords = ((1u << g.S) + 31) >> 5;
  const uint32_t w = (threadIdx.x < nwords) ? sm.bits[threadIdx.x] : 0u;
  int U;
  const int before = block_excl_scan(__popc(w), sm, &U);
  if (U == 0) return;
  if (U <= kSparseMax) {
    uint32_t x = w;
    int r = before;
    while (x) {
      const int b = __ffs(x) - 1;
      sm.list[r++] = (uint16_t)(threadIdx.x * 32 + b);
      x &= x - 1;
    }
    __syncthreads();
    if (threadIdx.x < 64) sparse_repair(sm, t, g, part, U);
  } else {
    dense_repair(sm, t, g, part);
  }
}

// Nodes [1, 2^P) above the partitions, recomputed from depth P upwards.
__device__ void top_rebuild(PartSmem& sm, const TreePtrs& t, const Geom& g) {
  const uint32_t np = 1u << g.P;
  if (g.P <= kMaxTopBits) {
    const uint32_t half = np >> 1;
    for (uint32_t h = half + threadIdx.x; h < np; h += kTreeThreads) {
      const float2 cs = *reinterpret_cast<const float2*>(t.sum + 2 * h);
      const float2 cm = *reinterpret_cast<const float2*>(t.mn + 2 * h);
      const float s = cs.x + cs.y, m = min_f32(cm.x, cm.y);
      sm.u.heap.s[h] = s;
      sm.u.heap.m[h] = m;
      t.sum[h] = s;
      t.mn[h] = m;
    }
    for (uint32_t width = half >> 1; width >= 1; width >>= 1) {
      __syncthreads();
      for (uint32_t h = width + threadIdx.x; h < 2 * width; h += kTreeThreads) {
        const float s = sm.u.heap.s[2 * h] + sm.u.heap.s[2 * h + 1];
        const float m = min_f32(sm.u.heap.m[2 * h], sm.u.heap.m[2 * h + 1]);
        sm.u.heap.s[h] = s;
        sm.u.heap.m[h] = m;
        t.sum[h] = s;
        t.mn[h] = m;
      }
    }
  } else {
    // More top nodes than LDS holds: level by level through global memory.
    for (int l = g.P - 1; l >= 0; --l) {
      const uint32_t lo = 1u << l;
      for (uint32_t h = lo + threadIdx.x; h < 2 * lo; h += kTreeThreads) {
        const float2 cs = *reinterpret_cast<const float2*>(t.sum + 2 * h);
        const float2 cm = *reinterpret_cast<const float2*>(t.mn + 2 * h);
        t.sum[h] = cs.x + cs.y;
        t.mn[h] = min_f32(cm.x, cm.y);
      }
      __threadfence();
      __syncthreads();
    }
  }
}

// Completion: the last block to finish rebuilds the top levels and folds the
// call's max priority into the running max.
__device__ void finish(PartSmem& sm, const TreePtrs& t, const Geom& g, float max_at_start,
                       uint32_t nblocks, uint32_t* reset_a, uint32_t* reset_b) {
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) sm.last = (atomicAdd(&t.ctrl->ticket, 1u) == nblocks - 1u) ? 1u : 0u;
  __syncthreads();
  if (!sm.last) return;
  __threadfence();
  if (g.P > 0) top_rebuild(sm, t, g);
  if (threadIdx.x == 0) {
    const uint32_t bm = atomicExch(&t.ctrl->batch_max, 0u);
    if (bm != 0u) {
      const float pm = __uint_as_float(bm - 1u);
      if (pm > max_at_start) t.ctrl->maxp = pm;
    }
    atomicExch(&t.ctrl->ticket, 0u);
  }
  if (reset_a) {
    const uint32_t np = 1u << g.P;
    for (uint32_t k = threadIdx.x; k < np; k += kTreeThreads) {
      reset_a[k] = 0u;
      reset_b[k] = 0u;
    }
  }
}

__device__ void clear_partition_tables(PartSmem& sm, const Geom& g, bool with_owner) {
  const uint32_t span = 1u << g.S;
  if (with_owner)
    for (uint32_t k = threadIdx.x; k < span; k += kTreeThreads) sm.u.owner[k] = -1;
  const uint32_t nwords = (span + 31) >> 5;
  for (uint32_t k = threadIdx.x; k < nwords; k += kTreeThreads) sm.bits[k] = 0u;
}

// Record entry (slot offset, batch position) as a candidate; the last batch
// position per slot wins.
__device__ __forceinline__ void note_position(PartSmem& sm, uint32_t off, int pos) {
  atomicMax(&sm.u.owner[off], pos);
}

__device__ __forceinline__ void set_winner(PartSmem& sm, uint32_t off, float p) {
  sm.val[off] = p;
  atomicOr(&sm.bits[off >> 5], 1u << (off & 31));
}

__device__ void publish_batch_max(PartSmem& sm, const TreePtrs& t, float pmax_local, bool any) {
  const uint32_t tag = any ? __float_as_uint(pmax_local) + 1u : 0u;
  const uint32_t m = block_max_tagged(tag, sm);
  if (threadIdx.x == 0 && m != 0u) atomicMax(&t.ctrl->batch_max, m);
}

// ------------------------------------------------------------------ kernels

__global__ void __launch_bounds__(256) init_kernel(TreePtrs t, Buckets bk, Geom g) {
  const uint64_t total = 2ull * g.n;
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < total; i += stride) {
    t.sum[i] = 0.0f;
    t.mn[i] = __builtin_inff();
  }
  const uint32_t np = 1u << g.P;
  for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < np; i += stride) {
    bk.counts[i] = 0u;
    bk.fill[i] = 0u;
  }
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    t.ctrl->maxp = 1.0f;
    t.ctrl->ticket = 0u;
    t.ctrl->batch_max = 0u;
  }
}

struct UpdateArgs {
  const int64_t* idx;
  const float* td;
  uint32_t B;
  uint32_t size;
  double alpha, eps;
  float p_nan;
};

// Small batches: every partition's block scans the whole batch for its slots.
__global__ void __launch_bounds__(256) update_scan_kernel(TreePtrs t, Geom g, UpdateArgs a) {
  __shared__ PartSmem sm;
  const uint32_t part = blockIdx.x;
  const uint32_t base = part << g.S;
  const float m0 = t.ctrl->maxp;
  clear_partition_tables(sm, g, true);
  __syncthreads();
  for (uint32_t b = threadIdx.x; b < a.B; b += kTreeThreads) {
    const int64_t i = a.idx[b];
    if (i >= 0 && i < (int64_t)a.size && ((uint64_t)i >> g.S) == part)
      note_position(sm, (uint32_t)i - base, (int)b);
  }
  __syncthreads();
  float pmax = 0.0f;
  bool any = false;
  for (uint32_t b = threadIdx.x; b < a.B; b += kTreeThreads) {
    const int64_t i = a.idx[b];
    if (i >= 0 && i < (int64_t)a.size && ((uint64_t)i >> g.S) == part) {
      const float p = priority_of(a.td[b], m0, a.alpha, a.eps, a.p_nan);
      pmax = any ? fmaxf(pmax, p) : p;
      any = true;
      const uint32_t off = (uint32_t)i - base;
      if (sm.u.owner[off] == (int)b) set_winner(sm, off, p);
    }
  }
  publish_batch_max(sm, t, pmax, any);
  __syncthreads();
  repair_partition(sm, t, g, part);
  finish(sm, t, g, m0, gridDim.x, nullptr, nullptr);
}

// Large batches, step 1: entries per partition.
__global__ void __launch_bounds__(256) bucket_count_kernel(Buckets bk, Geom g, UpdateArgs a) {
  const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int64_t i = a.idx[b];
  if (i >= 0 && i < (int64_t)a.size) atomicAdd(&bk.counts[(uint64_t)i >> g.S], 1u);
}

// Large batches, step 2: exclusive prefix of the counts (one block).
__global__ void __launch_bounds__(256) bucket_scan_kernel(Buckets bk, Geom g) {
  __shared__ PartSmem sm;
  const uint32_t np = 1u << g.P;
  uint32_t carry = 0;
  for (uint32_t lo = 0; lo < np; lo += kTreeThreads) {
    const uint32_t k = lo + threadIdx.x;
    const int c = (k < np) ? (int)bk.counts[k] : 0;
    int tot;
    const int ex = block_excl_scan(c, sm, &tot);
    if (k < np) bk.offs[k] = carry + (uint32_t)ex;
    carry += (uint32_t)tot;
  }
  if (threadIdx.x == 0) bk.offs[np] = carry;
}

// Large batches, step 3: scatter the valid entries into their buckets.
__global__ void __launch_bounds__(256) bucket_fill_kernel(Buckets bk, Geom g, UpdateArgs a) {
  const uint32_t b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= a.B) return;
  const int64_t i = a.idx[b];
  if (i < 0 || i >= (int64_t)a.size) return;
  const uint32_t part = (uint32_t)((uint64_t)i >> g.S);
  const uint32_t at = bk.offs[part] + atomicAdd(&bk.fill[part], 1u);
  bk.slot[at] = (uint32_t)i;
  bk.pos[at] = b;
  bk.td[at] = a.td[b];
}

// Large batches, step 4: one block per partition reads its bucket.
__global__ void __launch_bounds__(256) update_bucket_kernel(TreePtrs t, Buckets bk, Geom g,
                                                            UpdateArgs a) {
  __shared__ PartSmem sm;
  const uint32_t part = blockIdx.x;
  const uint32_t base = part << g.S;
  const float m0 = t.ctrl->maxp;
  const uint32_t lo = bk.offs[part], hi = bk.offs[part + 1];
  clear_partition_tables(sm, g, true);
  __syncthreads();
  for (uint32_t e = lo + threadIdx.x; e < hi; e += kTreeThreads)
    note_position(sm, bk.slot[e] - base, (int)bk.pos[e]);
  __syncthreads();
  float pmax = 0.0f;
  bool any = false;
  for (uint32_t e = lo + threadIdx.x; e < hi; e += kTreeThreads) {
    const float p = priority_of(bk.td[e], m0, a.alpha, a.eps, a.p_nan);
    pmax = any ? fmaxf(pmax, p) : p;
    any = true;
    const uint32_t off = bk.slot[e] - base;
    if (sm.u.owner[off] == (int)bk.pos[e]) set_winner(sm, off, p);
  }
  publish_batch_max(sm, t, pmax, any);
  __syncthreads();
  repair_partition(sm, t, g, part);
  finish(sm, t, g, m0, gridDim.x, bk.counts, bk.fill);
}

struct AddArgs {
  uint32_t cursor, count;
  const float* prio;
  uint32_t run_first[2], run_len[2];   // touched partitions: two disjoint runs
  uint32_t ntree;                      // blocks doing tree work (the rest copy rows)
  const float* states;
  const float* next_states;
  const uint32_t* actions;
  const float* rewards;
  const uint8_t* dones;
};

// Ring intake ("GPU-Resident Prioritized Experience Replay", section
// "Experience Insertion"): new slots take the given priority or the running
// max priority; rows are copied by the blocks past the tree blocks.
__global__ void __launch_bounds__(256) add_kernel(TreePtrs t, Geom g, Storage st, AddArgs a) {
  __shared__ PartSmem sm;
  if (blockIdx.x >= a.ntree) {
    // Row copy of the transitions into their ring slots.
    const uint32_t nb = gridDim.x - a.ntree;
    const uint32_t tid = (blockIdx.x - a.ntree) * kTreeThreads + threadIdx.x;
    const uint32_t stride = nb * kTreeThreads;
    const uint32_t D = (uint32_t)st.D;
    if ((D & 3u) == 0u) {
      const uint32_t c4 = D >> 2;
      const uint64_t total = (uint64_t)a.count * c4;
      for (uint64_t e = tid; e < total; e += stride) {
        const uint32_t j = (uint32_t)(e / c4), c = (uint32_t)(e % c4);
        uint32_t slot = a.cursor + j;
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
        uint32_t slot = a.cursor + j;
        if (slot >= g.n) slot -= g.n;
        st.states[(uint64_t)slot * D + c] = a.states[e];
        st.next_states[(uint64_t)slot * D + c] = a.next_states[e];
      }
    }
    for (uint32_t j = tid; j < a.count; j += stride) {
      uint32_t slot = a.cursor + j;
      if (slot >= g.n) slot -= g.n;
      st.actions[slot] = a.actions[j];
      st.rewards[slot] = a.rewards[j];
      st.dones[slot] = a.dones[j];
    }
    return;
  }
  const uint32_t w = blockIdx.x;
  const uint32_t part = (w < a.run_len[0]) ? a.run_first[0] + w : a.run_first[1] + (w - a.run_len[0]);
  const uint32_t span = 1u << g.S;
  const uint32_t base = part << g.S;
  const float m0 = t.ctrl->maxp;
  clear_partition_tables(sm, g, false);
  __syncthreads();
  // The ring range [cursor, cursor + count) split at the wrap.
  const uint64_t end = (uint64_t)a.cursor + a.count;
  const uint32_t r_lo[2] = {a.cursor, 0u};
  const uint32_t r_hi[2] = {(uint32_t)(end < g.n ? end : g.n),
                            (uint32_t)(end > g.n ? end - g.n : 0u)};
  float pmax = 0.0f;
  bool any = false;
  for (int r = 0; r < 2; ++r) {
    const uint32_t lo = max(r_lo[r], base), hi = min(r_hi[r], base + span);
    for (uint32_t slot = lo + threadIdx.x; slot < hi; slot += kTreeThreads) {
      const uint32_t j = (slot >= a.cursor) ? slot - a.cursor : slot + (g.n - a.cursor);
      float p = m0;
      if (a.prio) {
        p = a.prio[j] + 0.0f;
        pmax = any ? fmaxf(pmax, p) : p;
        any = true;
      }
      set_winner(sm, slot - base, p);
    }
  }
  if (a.prio) publish_batch_max(sm, t, pmax, any);
  __syncthreads();
  repair_partition(sm, t, g, part);
  finish(sm, t, g, m0, a.ntree, nullptr, nullptr);
}

inline unsigned grid_for(uint64_t work, unsigned per_block, unsigned cap) {
  uint64_t b = (work + per_block - 1) / per_block;
  if (b < 1) b = 1;
  if (b > cap) b = cap;
  return (unsigned)b;
}

}  // namespace

hipError_t launch_init(const TreePtrs& t, const Buckets& bk, const Geom& g, hipStream_t s) {
  const unsigned grid = grid_for(2ull * g.n, kTreeThreads * 8, 4096);
  hipLaunchKernelGGL(init_kernel, dim3(grid), dim3(kTreeThreads), 0, s, t, bk, g);
  return hipGetLastError();
}

hipError_t launch_update(const TreePtrs& t, const Buckets& bk, const Geom& g, uint32_t size,
                         int64_t B, const int64_t* idx, const float* td, double alpha,
                         double eps, hipStream_t s) {
  UpdateArgs a;
  a.idx = idx;
  a.td = td;
  a.B = (uint32_t)B;
  a.size = size;
  a.alpha = alpha;
  a.eps = eps;
  a.p_nan = (float)pow(eps, alpha);
  const uint64_t np = 1ull << g.P;
  // Scanning costs np * B loads; past ~4M use the bucketed path.
  if (np * (uint64_t)B <= (1ull << 22)) {
    hipLaunchKernelGGL(update_scan_kernel, dim3((unsigned)np), dim3(kTreeThreads), 0, s, t, g,
                       a);
    return hipGetLastError();
  }
  const unsigned eb = grid_for((uint64_t)B, kTreeThreads, 1u << 30);
  hipLaunchKernelGGL(bucket_count_kernel, dim3(eb), dim3(kTreeThreads), 0, s, bk, g, a);
  hipLaunchKernelGGL(bucket_scan_kernel, dim3(1), dim3(kTreeThreads), 0, s, bk, g);
  hipLaunchKernelGGL(bucket_fill_kernel, dim3(eb), dim3(kTreeThreads), 0, s, bk, g, a);
  hipLaunchKernelGGL(update_bucket_kernel, dim3((unsigned)np), dim3(kTreeThreads), 0, s, t, bk,
                     g, a);
  return hipGetLastError();
}

hipError_t launch_add(const TreePtrs& t, const Geom& g, const Storage& st, uint32_t cursor,
                      uint32_t count, const float* states, const float* next_states,
                      const uint32_t* actions, const float* rewards, const uint8_t* dones,
                      const float* prio, hipStream_t s) {
  AddArgs a;
  a.cursor = cursor;
  a.count = count;
  a.prio = prio;
  a.states = states;
  a.next_states = next_states;
  a.actions = actions;
  a.rewards = rewards;
  a.dones = dones;
  // Touched partitions of [cursor, cursor+count) and, past the wrap, [0, end-n).
  const uint64_t end = (uint64_t)cursor + count;
  const uint32_t hi0 = (uint32_t)(end < g.n ? end : g.n);
  uint32_t f0 = cursor >> g.S, l0 = (hi0 - 1) >> g.S;  // inclusive
  uint32_t f1 = 0, l1 = 0;
  bool second = end > g.n;
  if (second) {
    l1 = (uint32_t)(end - g.n - 1) >> g.S;
    f1 = 0;
    if (l1 >= f0) {  // the runs meet: one run covers everything touched
      f0 = 0;
      l0 = (1u << g.P) - 1;
      second = false;
    } else if (l1 + 1 == f0) {
      f0 = 0;
      second = false;
    }
  }
  a.run_first[0] = f0;
  a.run_len[0] = l0 - f0 + 1;
  a.run_first[1] = second ? f1 : 0;
  a.run_len[1] = second ? (l1 - f1 + 1) : 0;
  a.ntree = a.run_len[0] + a.run_len[1];
  unsigned ncopy = 0;
  if (st.D > 0) ncopy = grid_for((uint64_t)count * (uint64_t)st.D / 4 + count, kTreeThreads * 4, 2048);
  hipLaunchKernelGGL(add_kernel, dim3(a.ntree + ncopy), dim3(kTreeThreads), 0, s, t, g, st, a);
  return hipGetLastError();
}

}  // namespace per
