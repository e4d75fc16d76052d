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
//    priorities; stability keeps equal priorities in slot order): four
//    passes of 8-bit digits over tiles of 4096 items.  A tile is read
//    striped (wave w, step i, lane l holds item 1024 w + 64 i + l), so a
//    wave's steps visit its items in order; in each step the lanes holding
//    one digit find each other by eight ballots, which ranks every item
//    among the earlier items of its digit without a per-thread counter
//    table.  A pass is the tile histograms, a scan of each digit's row of
//    tile counts, and a scatter that stages the tile in digit order in LDS
//    and writes each digit's run to consecutive addresses.  The first pass
//    reads the priorities themselves.
//  * the cumulative sum is a tree over the rank weights f32((r+1)^-alpha)
//    built with the priority trees' rules (sum and min of the two children),
//    so the proportional descent over it gives the rank of a mass exactly.
//    One block per 4096-leaf partition builds its subtree in LDS; the top
//    kernel of the priority trees finishes the nodes above.

#include "per_internal.h"
#include "pow_f32.h"

namespace per {
namespace {

constexpr int kRankThreads = 256;                   // four waves
constexpr int kItems = 16;                          // steps per wave
constexpr uint32_t kTile = kRankThreads * kItems;   // 4096
constexpr uint32_t kWaveItems = kTile / 4;          // 1024
constexpr int kDigitBits = 8;
constexpr int kDigits = 1 << kDigitBits;            // 256 = kRankThreads
constexpr int kPasses = 32 / kDigitBits;

__device__ __forceinline__ float rank_min(float a, float b) { return (b < a) ? b : a; }

// Item `i` of this lane in its tile's striped order, as an index into [0, count).
__device__ __forceinline__ uint32_t striped_item(int i) {
  return blockIdx.x * kTile + (threadIdx.x >> 6) * kWaveItems + (uint32_t)i * 64u +
         (threadIdx.x & 63u);
}

// The tile's keys (and values) of this lane; FIRST: from the priorities, the
// value being the slot.  ok[i]: the item exists.
template <bool FIRST, bool VALS>
__device__ __forceinline__ void load_striped(const uint32_t* keys, const uint32_t* vals,
                                             const float* leaves, uint32_t count,
                                             uint32_t k[kItems], uint32_t v[kItems],
                                             bool ok[kItems]) {
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const uint32_t x = striped_item(i);
    ok[i] = x < count;
    const uint32_t xs = ok[i] ? x : 0u;
    if constexpr (FIRST) {
      k[i] = ~__float_as_uint(leaves[xs]);
      if constexpr (VALS) v[i] = x;
    } else {
      k[i] = keys[xs];
      if constexpr (VALS) v[i] = vals[xs];
    }
  }
}

// The lanes of the wave whose item exists and has digit d (this lane's own
// digit): one ballot per digit bit.  Every lane of the wave takes part.
__device__ __forceinline__ uint64_t digit_peers(uint32_t d, bool ok) {
  uint64_t m = __ballot(ok);
#pragma unroll
  for (int b = 0; b < kDigitBits; ++b) {
    const bool bit = (d >> b) & 1u;
    const uint64_t bal = __ballot(bit);
    m &= bit ? bal : ~bal;
  }
  return m;
}

// Per-wave digit counts of a tile in wc[w][d], each wave counting its own
// items in its own row (so no barrier and no atomics); in step i the lowest
// lane of each digit adds the digit's lanes.  my[i]: the item's position
// among the wave's items of its digit.
__device__ __forceinline__ void wave_digit_counts(uint32_t (*wc)[kDigits], const uint32_t k[kItems],
                                                  const bool ok[kItems], int shift,
                                                  uint32_t my[kItems]) {
  const int w = threadIdx.x >> 6;
  const uint32_t lane = threadIdx.x & 63u;
  const uint64_t below = (1ull << lane) - 1ull;
#pragma unroll
  for (int d = 0; d < kDigits / 64; ++d) wc[w][lane + 64 * d] = 0u;
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    const uint32_t d = (k[i] >> shift) & (kDigits - 1);
    const uint64_t m = digit_peers(d, ok[i]);
    const uint32_t before = (uint32_t)__popcll(m & below);
    const uint32_t base = wc[w][d];  // every lane reads before the leaders write
    my[i] = base + before;
    if (ok[i] && before == 0u) wc[w][d] = base + (uint32_t)__popcll(m);
  }
}

// Exclusive prefix over the block's 256 threads of a and b at once.
__device__ __forceinline__ void block_excl2(uint32_t a, uint32_t b, uint32_t* wsum, uint32_t& ea,
                                            uint32_t& eb) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  uint32_t ia = a, ib = b;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const uint32_t ya = __shfl_up(ia, o), yb = __shfl_up(ib, o);
    if (lane >= o) {
      ia += ya;
      ib += yb;
    }
  }
  if (lane == 63) {
    wsum[w] = ia;
    wsum[4 + w] = ib;
  }
  __syncthreads();
  ea = ia - a;
  eb = ib - b;
  for (int q = 0; q < w; ++q) {
    ea += wsum[q];
    eb += wsum[4 + q];
  }
}

// Tile histograms of one pass: hist[d * ntiles + tile].  MATCH: count by
// ballots (the last pass, on the exponent's high bits, where most keys share
// a few digits and LDS adds to one address would serialise), else by LDS
// adds.
template <bool FIRST, bool MATCH>
__global__ void __launch_bounds__(kRankThreads) rank_hist_kernel(const uint32_t* keys,
                                                                 const float* leaves,
                                                                 uint32_t count, int shift,
                                                                 uint32_t ntiles, uint32_t* hist) {
  __shared__ uint32_t wc[4][kDigits];
  uint32_t k[kItems];
  bool ok[kItems];
  load_striped<FIRST, false>(keys, nullptr, leaves, count, k, nullptr, ok);
  if constexpr (MATCH) {
    uint32_t my[kItems];
    wave_digit_counts(wc, k, ok, shift, my);
  } else {
    // Order does not matter for the counts: LDS adds without a returned
    // value, issued back to back, each wave into its own row.
    const int w = threadIdx.x >> 6;
#pragma unroll
    for (int d = 0; d < kDigits / 64; ++d) wc[w][(threadIdx.x & 63) + 64 * d] = 0u;
#pragma unroll
    for (int i = 0; i < kItems; ++i)
      if (ok[i]) atomicAdd(&wc[w][(k[i] >> shift) & (kDigits - 1)], 1u);
  }
  __syncthreads();
  const int t = threadIdx.x;
  hist[(size_t)t * ntiles + blockIdx.x] = wc[0][t] + wc[1][t] + wc[2][t] + wc[3][t];
}

// Exclusive scan of each digit's row of tile counts in place (one block per
// digit); tot[d] = the digit's count over all tiles.
__global__ void __launch_bounds__(kRankThreads) rank_rowscan_kernel(uint32_t* hist,
                                                                    uint32_t ntiles,
                                                                    uint32_t* tot) {
  __shared__ uint32_t wsum[8];
  constexpr uint32_t kHeld = 16;  // entries a thread keeps in registers (up to 2^24 slots)
  uint32_t* row = hist + (size_t)blockIdx.x * ntiles;
  const uint32_t per = (ntiles + kRankThreads - 1) / kRankThreads;
  const uint32_t c0 = min(threadIdx.x * per, ntiles), c1 = min(c0 + per, ntiles);
  uint32_t s = 0, run, unused;
  if (per <= kHeld) {
    // All of a thread's loads issued together, the entries kept for the
    // writes.
    uint32_t x[kHeld];
#pragma unroll
    for (uint32_t j = 0; j < kHeld; ++j) x[j] = (c0 + j < c1) ? row[c0 + j] : 0u;
#pragma unroll
    for (uint32_t j = 0; j < kHeld; ++j) s += x[j];
    block_excl2(s, 0u, wsum, run, unused);
#pragma unroll
    for (uint32_t j = 0; j < kHeld; ++j) {
      if (c0 + j < c1) {
        row[c0 + j] = run;
        run += x[j];
      }
    }
  } else {
    for (uint32_t c = c0; c < c1; ++c) s += row[c];
    block_excl2(s, 0u, wsum, run, unused);
    for (uint32_t c = c0; c < c1; ++c) {
      const uint32_t x = row[c];
      row[c] = run;
      run += x;
    }
  }
  if (threadIdx.x == kRankThreads - 1) tot[blockIdx.x] = run;
}

// Stable scatter of one pass.  Each wave ranks its items per digit; the
// tile's digit starts and the waves' starts within each digit follow from
// the counts; the tile is staged in digit order in LDS, then written out
// with consecutive threads on consecutive staged items, so that each digit's
// run goes to consecutive addresses from the digit's global start for this
// tile (its row scan plus the counts of all smaller digits).
struct ScatterSmem {
  uint32_t key[kTile];
  uint32_t val[kTile];
  uint32_t wc[4][kDigits];  // per-wave counts, then per-wave starts in the tile
  uint32_t dstart[kDigits];  // tile-local start of each digit
  uint32_t gbase[kDigits];   // global start of this tile's run of each digit
  uint32_t wsum[8];
};

template <bool FIRST>
__global__ void __launch_bounds__(kRankThreads) rank_scatter_kernel(
    const uint32_t* keys, const uint32_t* vals, const float* leaves, uint32_t count, int shift,
    uint32_t ntiles, const uint32_t* hist, const uint32_t* tot, uint32_t* keys_out,
    uint32_t* vals_out) {
  __shared__ ScatterSmem sm;
  uint32_t k[kItems], v[kItems], my[kItems];
  bool ok[kItems];
  load_striped<FIRST, true>(keys, vals, leaves, count, k, v, ok);
  const int t = threadIdx.x;
  const uint32_t row = hist[(size_t)t * ntiles + blockIdx.x];  // thread t: digit t
  const uint32_t dtot = tot[t];
  wave_digit_counts(sm.wc, k, ok, shift, my);
  __syncthreads();
  const uint32_t c0 = sm.wc[0][t], c1 = sm.wc[1][t], c2 = sm.wc[2][t], c3 = sm.wc[3][t];
  uint32_t start, dbefore;
  block_excl2(c0 + c1 + c2 + c3, dtot, sm.wsum, start, dbefore);
  sm.dstart[t] = start;
  sm.gbase[t] = dbefore + row;
  sm.wc[0][t] = start;
  sm.wc[1][t] = start + c0;
  sm.wc[2][t] = start + c0 + c1;
  sm.wc[3][t] = start + c0 + c1 + c2;
  __syncthreads();
  const int w = t >> 6;
#pragma unroll
  for (int i = 0; i < kItems; ++i) {
    if (ok[i]) {
      const uint32_t pos = sm.wc[w][(k[i] >> shift) & (kDigits - 1)] + my[i];
      sm.key[pos] = k[i];
      sm.val[pos] = v[i];
    }
  }
  __syncthreads();
  const uint32_t tile_n = min(kTile, count - blockIdx.x * kTile);
  for (uint32_t i = t; i < tile_n; i += kRankThreads) {
    const uint32_t kk = sm.key[i];
    const uint32_t d = (kk >> shift) & (kDigits - 1);
    const uint32_t pos = sm.gbase[d] + (i - sm.dstart[d]);
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
    const float w = (r < count) ? pow_f32((double)(r + 1), -alpha) : 0.0f;
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
  const uint32_t ntiles = (count + kTile - 1) / kTile;
  uint32_t* tot = hist + (size_t)kDigits * ntiles;
  for (int p = 0; p < kPasses; ++p) {
    const int shift = kDigitBits * p;
    const uint32_t* kin = keys[p & 1];
    const uint32_t* vin = vals[p & 1];
    uint32_t* kout = keys[(p + 1) & 1];
    uint32_t* vout = vals[(p + 1) & 1];
    hipError_t e;
    if (p == 0)
      e = launch_kernel(rank_hist_kernel<true, false>, dim3(ntiles), dim3(kRankThreads), 0, s,
                        nullptr, leaves, count, shift, ntiles, hist);
    else if (p < kPasses - 1)
      e = launch_kernel(rank_hist_kernel<false, false>, dim3(ntiles), dim3(kRankThreads), 0, s,
                        kin, nullptr, count, shift, ntiles, hist);
    else
      e = launch_kernel(rank_hist_kernel<false, true>, dim3(ntiles), dim3(kRankThreads), 0, s,
                        kin, nullptr, count, shift, ntiles, hist);
    if (e != hipSuccess) return e;
    e = launch_kernel(rank_rowscan_kernel, dim3(kDigits), dim3(kRankThreads), 0, s, hist, ntiles,
                      tot);
    if (e != hipSuccess) return e;
    if (p == 0)
      e = launch_kernel(rank_scatter_kernel<true>, dim3(ntiles), dim3(kRankThreads), 0, s,
                        nullptr, nullptr, leaves, count, shift, ntiles, hist, tot, kout, vout);
    else
      e = launch_kernel(rank_scatter_kernel<false>, dim3(ntiles), dim3(kRankThreads), 0, s, kin,
                        vin, nullptr, count, shift, ntiles, hist, tot, kout, vout);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

hipError_t launch_rank_build(const TreePtrs& rt, const Geom& g, uint32_t count, double alpha,
                             hipStream_t s) {
  const size_t lds = sizeof(float) * 4 * (size_t(1) << g.S);
  hipError_t e = launch_kernel(rank_build_kernel, dim3(1u << g.P), dim3(kRankThreads), lds, s, rt,
                               g, count, alpha);
  if (e != hipSuccess || g.P == 0) return e;
  return launch_top(rt, g, s);
}

size_t rank_hist_words(int64_t n) {
  return (size_t)kDigits * ((size_t)((n + kTile - 1) / kTile) + 1);
}

}  // namespace per
