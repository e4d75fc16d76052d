// rank_kernels.hip -- rank-based prioritisation on gfx950: the ranking of
// the filled slots by priority and the tree over the rank weights.
//
// "GPU-Resident Prioritized Experience Replay", section "Sampling Kernels",
// rank-based: the (priority, index) pairs are sorted descending, then samples
// are drawn with probabilities 1/rank^alpha through their cumulative sum,
// gathered, and weighted.  Here:
//  * the ranking is a stable least-significant-digit radix sort of the slots
//    [0, count) on the key ~bits(priority) (for priorities >= 0 the f32 bit
//    patterns order like the values, so ascending keys are descending
//    priorities; stability keeps equal priorities in slot order): eight
//    passes of 4-bit digits over tiles of 4096 items -- a histogram of each
//    tile, one scan of all tile histograms, and a scatter in which every
//    thread writes its 16 consecutive items in order, so that each digit's
//    items keep their order;
//  * the cumulative sum is a tree over the rank weights f32((r+1)^-alpha)
//    built with the priority trees' rules (sum and min of the two children),
//    so the proportional descent over it gives the rank of a mass exactly.
//    One block per 4096-leaf partition builds its subtree in LDS; the top
//    kernel of the priority trees finishes the nodes above.

#include "per_internal.h"

namespace per {
namespace {

constexpr int kRankThreads = 256;
constexpr int kItems = 16;                                // consecutive items per thread
constexpr uint32_t kTile = kRankThreads * kItems;         // 4096
constexpr int kDigitBits = 4;
constexpr int kDigits = 1 << kDigitBits;

__device__ __forceinline__ float rank_min(float a, float b) { return (b < a) ? b : a; }

// Keys and values of the first pass, straight from the priority leaves.
__global__ void __launch_bounds__(256) rank_seed_kernel(const float* leaves, uint32_t count,
                                                        uint32_t* keys, uint32_t* vals) {
  const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) {
    keys[i] = ~__float_as_uint(leaves[i]);
    vals[i] = i;
  }
}

// Per-thread digit counts of one tile in LDS, digit-major (cnt[d][t]); on
// return cnt holds, for every digit, the exclusive prefix over the threads
// (the tile-local position of each thread's first item of that digit), and
// tot[d] the tile's count of digit d.
struct TileSmem {
  uint32_t cnt[kDigits * kRankThreads];
  uint32_t tot[kDigits];
};

__device__ __forceinline__ void tile_counts(TileSmem& sm, const uint32_t* k, int nvalid,
                                            int shift) {
  const int t = threadIdx.x;
#pragma unroll
  for (int d = 0; d < kDigits; ++d) sm.cnt[d * kRankThreads + t] = 0u;
  // Own column only, so no two threads touch one counter; LDS adds without a
  // returned value issue back to back instead of as 16 dependent round trips.
#pragma unroll
  for (int i = 0; i < kItems; ++i)
    if (i < nvalid) atomicAdd(&sm.cnt[((k[i] >> shift) & (kDigits - 1)) * kRankThreads + t], 1u);
  __syncthreads();
  // Thread t scans the 16 entries [16t, 16t + 16) (digit t / 16), then the
  // 16 segments of a digit (16 consecutive lanes of one wave) meet by shuffle.
  uint32_t* seg = sm.cnt + t * kItems;
  uint32_t run = 0;
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const uint32_t c = seg[i];
    seg[i] = run;
    run += c;
  }
  uint32_t inc = run;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o, 16);
    if ((t & 15) >= o) inc += y;
  }
  const uint32_t excl = inc - run;
#pragma unroll
  for (int i = 0; i < kItems; ++i) seg[i] += excl;
  if ((t & 15) == 15) sm.tot[t >> 4] = inc;
  __syncthreads();
}

__device__ __forceinline__ int load_tile(const uint32_t* src, uint32_t count, uint32_t* k) {
  const uint32_t first = blockIdx.x * kTile + threadIdx.x * kItems;
  const int nvalid = (first >= count) ? 0 : (int)min((uint32_t)kItems, count - first);
  if (nvalid == kItems) {
#pragma unroll
    for (int i = 0; i < kItems; i += 4) {
      const uint4 q = *reinterpret_cast<const uint4*>(src + first + i);
      k[i] = q.x;
      k[i + 1] = q.y;
      k[i + 2] = q.z;
      k[i + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < kItems; ++i) k[i] = (i < nvalid) ? src[first + i] : 0u;
  }
  return nvalid;
}

// Tile histograms of one pass: hist[d * ntiles + tile].
__global__ void __launch_bounds__(kRankThreads) rank_hist_kernel(const uint32_t* keys,
                                                                 uint32_t count, int shift,
                                                                 uint32_t* hist) {
  __shared__ TileSmem sm;
  uint32_t k[kItems];
  const int nvalid = load_tile(keys, count, k);
  tile_counts(sm, k, nvalid, shift);
  if (threadIdx.x < kDigits) hist[threadIdx.x * gridDim.x + blockIdx.x] = sm.tot[threadIdx.x];
}

// Exclusive scan of the m = 16 * ntiles histogram entries in place (one
// block; digit-major order, so entry (d, tile) becomes the global position
// of the tile's first item of digit d).  m is a multiple of 16: a thread
// owns 16-entry chunks, read and written as four 16-byte accesses each, all
// of a chunk's loads issued together.
__global__ void __launch_bounds__(1024) rank_scan_kernel(uint32_t* hist, uint32_t m) {
  __shared__ uint32_t wsum[16];
  const uint32_t nchunks = m / 16;
  const uint32_t per = (nchunks + 1023) / 1024;  // chunks per thread
  const uint32_t c0 = threadIdx.x * per, c1 = min(c0 + per, nchunks);
  uint32_t s = 0;
  for (uint32_t c = c0; c < c1; ++c) {
    uint4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = reinterpret_cast<const uint4*>(hist)[4 * c + j];
#pragma unroll
    for (int j = 0; j < 4; ++j) s += q[j].x + q[j].y + q[j].z + q[j].w;
  }
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t inc = s;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t y = __shfl_up(inc, o);
    if (lane >= o) inc += y;
  }
  if (lane == 63) wsum[w] = inc;
  __syncthreads();
  uint32_t run = inc - s;
  for (int k = 0; k < w; ++k) run += wsum[k];
  for (uint32_t c = c0; c < c1; ++c) {
    uint4 q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) q[j] = reinterpret_cast<const uint4*>(hist)[4 * c + j];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      uint4 o;
      o.x = run;
      run += q[j].x;
      o.y = run;
      run += q[j].y;
      o.z = run;
      run += q[j].z;
      o.w = run;
      run += q[j].w;
      reinterpret_cast<uint4*>(hist)[4 * c + j] = o;
    }
  }
}

// Stable scatter of one pass.  The tile is first put in digit order in LDS
// (every thread places its items, in order, after the tile's earlier items
// of the same digit), then written out with consecutive threads on
// consecutive items, so that each digit's run of the tile goes to
// consecutive addresses.
struct ScatterSmem {
  TileSmem tc;
  uint32_t key[kTile];
  uint32_t val[kTile];
  uint32_t dbase[kDigits];  // tile-local start of each digit
  uint32_t gbase[kDigits];  // global start of this tile's run of each digit
};

__global__ void __launch_bounds__(kRankThreads) rank_scatter_kernel(
    const uint32_t* keys, const uint32_t* vals, uint32_t count, int shift,
    const uint32_t* hist, uint32_t* keys_out, uint32_t* vals_out) {
  __shared__ ScatterSmem sm;
  uint32_t k[kItems], v[kItems];
  const int nvalid = load_tile(keys, count, k);
  load_tile(vals, count, v);
  tile_counts(sm.tc, k, nvalid, shift);
  const int t = threadIdx.x;
  if (t < kDigits) {
    uint32_t b = 0;
    for (int d = 0; d < t; ++d) b += sm.tc.tot[d];
    sm.dbase[t] = b;
    sm.gbase[t] = hist[t * gridDim.x + blockIdx.x];
  }
  __syncthreads();
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    if (i < nvalid) {
      const uint32_t d = (k[i] >> shift) & (kDigits - 1);
      const uint32_t pos = sm.dbase[d] + sm.tc.cnt[d * kRankThreads + t]++;
      sm.key[pos] = k[i];
      sm.val[pos] = v[i];
    }
  }
  __syncthreads();
  const uint32_t tile_n = min(kTile, count - blockIdx.x * kTile);
  for (uint32_t i = t; i < tile_n; i += kRankThreads) {
    const uint32_t kk = sm.key[i];
    const uint32_t d = (kk >> shift) & (kDigits - 1);
    const uint32_t pos = sm.gbase[d] + (i - sm.dbase[d]);
    keys_out[pos] = kk;
    vals_out[pos] = sm.val[i];
  }
}

// Leaves and subtree of one 2^S-leaf partition of the rank-weight trees:
// leaf r holds f32((r+1)^-alpha) for r < count, else sum 0 / min +inf.  The
// subtree is a local heap in LDS (h in [1, 2 span): leaves at [span, 2 span),
// local node h of depth d is global node (root << d) + h - 2^d with root the
// partition root), built level by level and stored after the last barrier.
// Dynamic LDS: 2 x 2 span floats.
__global__ void __launch_bounds__(kRankThreads) rank_build_kernel(TreePtrs t, Geom g,
                                                                  uint32_t count, double alpha) {
  extern __shared__ float heap[];
  const uint32_t span = 1u << g.S;
  float* hs = heap;
  float* hm = heap + 2 * span;
  const uint32_t r0 = blockIdx.x << g.S;  // first rank of the partition
  const uint32_t root = (1u << g.P) + blockIdx.x;
  for (uint32_t o = threadIdx.x; o < span; o += kRankThreads) {
    const uint32_t r = r0 + o;
    const float w = (r < count) ? (float)pow((double)(r + 1), -alpha) : 0.0f;
    hs[span + o] = w;
    hm[span + o] = (r < count) ? w : __builtin_inff();
  }
  for (uint32_t width = span >> 1; width >= 1; width >>= 1) {
    __syncthreads();
    for (uint32_t h = width + threadIdx.x; h < 2 * width; h += kRankThreads) {
      const float2 cs = reinterpret_cast<const float2*>(hs)[h];  // children 2h, 2h+1
      const float2 cm = reinterpret_cast<const float2*>(hm)[h];
      hs[h] = cs.x + cs.y;
      hm[h] = rank_min(cm.x, cm.y);
    }
  }
  __syncthreads();
  for (uint32_t h = 1 + threadIdx.x; h < 2 * span; h += kRankThreads) {
    const int d = 31 - __clz(h);
    const uint32_t x = (root << d) + (h - (1u << d));
    t.sum[x] = hs[h];
    t.mn[x] = hm[h];
  }
}

}  // namespace

hipError_t launch_rank_sort(const float* leaves, uint32_t count, uint32_t* const keys[2],
                            uint32_t* const vals[2], uint32_t* hist, hipStream_t s) {
  if (count == 0) return hipSuccess;
  const unsigned ntiles = (count + kTile - 1) / kTile;
  hipLaunchKernelGGL(rank_seed_kernel, dim3((count + 255) / 256), dim3(256), 0, s, leaves, count,
                     keys[0], vals[0]);
  for (int p = 0; p < 32 / kDigitBits; ++p) {
    const int shift = kDigitBits * p;
    hipLaunchKernelGGL(rank_hist_kernel, dim3(ntiles), dim3(kRankThreads), 0, s, keys[p & 1],
                       count, shift, hist);
    hipLaunchKernelGGL(rank_scan_kernel, dim3(1), dim3(1024), 0, s, hist,
                       (uint32_t)kDigits * ntiles);
    hipLaunchKernelGGL(rank_scatter_kernel, dim3(ntiles), dim3(kRankThreads), 0, s, keys[p & 1],
                       vals[p & 1], count, shift, hist, keys[(p + 1) & 1], vals[(p + 1) & 1]);
  }
  return hipGetLastError();
}

hipError_t launch_rank_build(const TreePtrs& rt, const Geom& g, uint32_t count, double alpha,
                             hipStream_t s) {
  const size_t lds = sizeof(float) * 4 * (size_t(1) << g.S);
  hipLaunchKernelGGL(rank_build_kernel, dim3(1u << g.P), dim3(kRankThreads), lds, s, rt, g, count,
                     alpha);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || g.P == 0) return e;
  return launch_top(rt, g, s);
}

uint32_t rank_tiles(int64_t n) { return (uint32_t)((n + kTile - 1) / kTile); }

}  // namespace per
