// sample_kernels.hip -- batched proportional sampling on gfx950: root-to-leaf
// descent, importance-sampling weights and the gather of the sampled rows,
// fused in one kernel.
//
// Descent rule ("Putting prioritized replay's segment tree on a GPU",
// section "Sampling Is a Descent"): each level decides one bit of the leaf
// offset.  The right child is taken when the left child's sum is at most the
// remaining mass and the right child's sum is not 0; the left sum is then
// taken off the mass (an f32 subtraction).
//
// Layout of the work: a group of G lanes (G = 16: four samples per wave;
// G = 1: one lane per sample; G = 64: one wave per sample) carries one
// sample.  The top of the tree is walked on chip: each block first rebuilds
// the 2^P - 1 nodes above the update partitions from the 2^P partition roots
// (coalesced loads), which also gives it the total and the min priority --
// in LDS, or, with one sample per wave over 2^8 .. 2^10 roots, in each
// wave's registers.  The rebuilt nodes stay on chip: the stored ones are
// refreshed only by top_kernel (per_flush, or before a sampler that reads
// them from memory).  (Trees of at most 2^10 leaves are staged whole.)  The
// remaining levels are covered in rounds: a round of R levels below node c
// loads the 2^R contiguous
// descendants of c at depth +R (G lanes x V values, 16-byte vector loads),
// rebuilds the R-1 intermediate levels by pairwise adds -- bit-identical to
// the stored nodes, since every stored node is exactly the f32 sum of its
// children -- and takes all R decisions from registers.  A round is one
// dependent trip to memory instead of R.
//
// Weights ("GPU-Resident Prioritized Experience Replay", section "Sampling
// Kernels"): w = (N*P(i))^-beta normalised by the weight of the min-tree root
// priority; N and the total cancel, so w = (p_i / p_min)^-beta, in f64.
// Rows are copied by the whole wave, 16 bytes per lane per access, straight
// into the caller's buffers ("True Single-Graph Implementation Plan", Task
// 3).

#include <type_traits>

#include "lanes.h"
#include "per_internal.h"
#include "pow_f32.h"

// Start and end stamps of the proportional sampler's waves, in the
// measurement build only (libper_stamps.so, PER_PHASE_STAMPS defined): lane 0
// of wave w (of 4) of block b stores the 100 MHz real-time clock when the
// wave starts into per_sample_stamps[b * 8 + w] and when it is done into
// per_sample_stamps[b * 8 + 4 + w] (include/per_stamps.h).  In the product
// build the stamps are empty statements.
#ifdef PER_PHASE_STAMPS
constexpr int kSampleStampBlocks = 4096;
__device__ unsigned long long per_sample_stamps[kSampleStampBlocks * 8];
#define PER_SAMPLE_STAMP(k)                                                               \
  do {                                                                                    \
    if ((threadIdx.x & 63u) == 0 && blockIdx.x < (unsigned)kSampleStampBlocks)           \
      per_sample_stamps[blockIdx.x * 8 + (k) * 4 + (threadIdx.x >> 6)] =                  \
          __builtin_amdgcn_s_memrealtime();                                               \
  } while (0)

extern "C" int per_sample_stamps_clear(hipStream_t stream) {
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(per_sample_stamps)) != hipSuccess) return -4;
  return hipMemsetAsync(p, 0, sizeof(per_sample_stamps), stream) == hipSuccess ? 0 : -4;
}

extern "C" int per_sample_stamps_read(unsigned long long* out, long long count,
                                      hipStream_t stream) {
  if (!out || count < 0 || count > (long long)(kSampleStampBlocks * 8)) return -1;
  void* p = nullptr;
  if (hipGetSymbolAddress(&p, HIP_SYMBOL(per_sample_stamps)) != hipSuccess) return -4;
  if (hipMemcpyAsync(out, p, (size_t)count * sizeof(unsigned long long), hipMemcpyDeviceToHost,
                     stream) != hipSuccess)
    return -4;
  return hipStreamSynchronize(stream) == hipSuccess ? 0 : -4;
}
#else
#define PER_SAMPLE_STAMP(k) \
  do {                      \
  } while (0)
#endif

namespace per {
namespace {

constexpr int kSampleThreads = 256;

// The min of two tree values.  Every value stored in or compared by these
// trees is a priority or a sum of priorities: +0, a positive finite value or
// +inf, never NaN or -0 (a given -0 priority is stored as +0).  For those the
// f32 bit patterns order like the values, so the min is one integer min of
// the bits, with the same result as (b < a) ? b : a.
__device__ __forceinline__ float min_f32(float a, float b) {
  return __uint_as_float(min(__float_as_uint(a), __float_as_uint(b)));
}

struct SampleArgs {
  float* sum;
  float* mn;
  uint32_t n;
  uint32_t size;
  const uint32_t* dev_size;  // uniform mode in graph mode: the filled size, read on the device
  uint32_t B;
  const uint32_t* order;  // rank-based: the slot of each leaf (rank), or NULL
  const float* u;       // masses, or NULL: from the generator stream
  uint64_t seed;        // generator key (seed, 0)
  uint64_t offset;      // stream word of sample 0
  double beta;
  int64_t* idx_out;
  float* w_out;
  float* states_out;
  float* next_out;
  uint32_t* actions_out;
  float* rewards_out;
  void* dones_out;      // u8 [B], or f32 [B] when dones_f32
  uint32_t out_stride;  // floats per output state row, >= D; columns D.. are 0
  int dones_f32;
  Storage st;
  int P;          // partitions = 2^P; the top P levels are rebuilt in LDS
  int top_mode;   // kTopNone / kTopRebuild / kTopWhole
  int top;        // levels walked in LDS
  int nrounds;
  int rounds[kMaxRounds];
};

// Pairwise (heap-order) sum of LEN register values: the value of their
// common ancestor node.
template <int LEN>
__device__ __forceinline__ float pair_sum(const float* x) {
  if constexpr (LEN == 1) {
    return x[0];
  } else {
    return pair_sum<LEN / 2>(x) + pair_sum<LEN / 2>(x + LEN / 2);
  }
}

// Descent through the V values one lane holds (the bottom log2(V) levels of
// a round).  Returns the chosen offset; leaf receives its value.
template <int V>
__device__ __forceinline__ int lane_descent(const float* x, float& m, float& leaf) {
  if constexpr (V == 1) {
    leaf = x[0];
    return 0;
  } else {
    constexpr int H = V / 2;
    const float ls = pair_sum<H>(x), rs = pair_sum<H>(x + H);
    const bool right = !(ls > m || rs == 0.0f);
    if (right) m = m - ls;
    float y[H];
#pragma unroll
    for (int i = 0; i < H; ++i) y[i] = right ? x[H + i] : x[i];
    return (right ? H : 0) + lane_descent<H>(y, m, leaf);
  }
}

template <int V>
__device__ __forceinline__ void load_values(const float* p, float* x) {
  if constexpr (V == 1) {
    x[0] = p[0];
  } else if constexpr (V == 2) {
    const float2 q = *reinterpret_cast<const float2*>(p);
    x[0] = q.x;
    x[1] = q.y;
  } else {
#pragma unroll
    for (int i = 0; i < V; i += 4) {
      const float4 q = *reinterpret_cast<const float4*>(p + i);
      x[i] = q.x;
      x[i + 1] = q.y;
      x[i + 2] = q.z;
      x[i + 3] = q.w;
    }
  }
}

constexpr int ilog2(int v) { return v <= 1 ? 0 : 1 + ilog2(v / 2); }

// Wave-cooperative row copy of a wave's SPW samples (sample s's slot in lane
// s*G), in batches of kBatch accesses per lane: every load of a batch is
// issued before the first store, so each lane keeps kBatch reads in flight
// (16 bytes each when VEC).  An output row has W >= D floats; its columns
// D .. W-1 are stored as 0 ("True Single-Graph Implementation Plan", Task 2:
// padded rows).  A padding column re-reads the row's first column (the same
// line, so the load stays unconditional and in its batch); the zero is
// selected at the store, after the batch's loads.
// kBatch (1, 2, 4 or 8) is chosen from the wave's access count so that a
// wave copying a few short rows issues no idle loads.  mid() runs once,
// between the first batch's loads and its stores, so that its work overlaps
// their trip.  With one lane per sample (G = 1) a wave copies 64 samples'
// rows alone, batch after batch: there the loads of batch k + 1 are issued
// before the stores of batch k, and those stores wait for every load in
// flight, so they go out one trip after their own loads.  Loads and stores
// share the wave's one memory counter: waiting only for batch k's loads
// would also wait for batch k - 1's stores, issued just before them, and is
// slower (2^24 leaves, 65536 rows of 128 floats: 36.2 against 34.1 us).
// Elsewhere the wave's few batches go one after the other.  NT: the rows are read with
// the non-temporal hint, so that a large gather streams past the caches
// instead of evicting the tree nodes the descents and updates reuse.
template <bool VEC, bool NT, int SPW, int G, int kBatch, typename Mid>
__device__ __forceinline__ void copy_rows(const SampleArgs& a, uint32_t wave_b0, uint32_t slot,
                                          int lane, uint32_t D, uint32_t W, Mid mid) {
  constexpr uint32_t kW = VEC ? 4u : 1u;      // floats per access
  const uint32_t per_src = D / kW;            // loads per row
  const uint32_t per_row = W / kW;            // stores per row
  const uint32_t total = SPW * 2u * per_row;
  using T = typename std::conditional<VEC, float4, float>::type;
  // The four row pointers as values: a per-lane choice between two fields of
  // the argument block would otherwise become a per-lane load of a pointer
  // (and a wait) in front of every row access.
  const float* const src_s = a.st.states;
  const float* const src_n = a.st.next_states;
  float* const dst_s = a.states_out;
  float* const dst_n = a.next_out;
  // With at most four samples per wave their slots are read once, from the
  // lanes that hold them; otherwise each access fetches its sample's slot.
  uint32_t few[SPW <= 4 ? SPW : 1];
  if constexpr (SPW <= 4) {
#pragma unroll
    for (int k = 0; k < SPW; ++k) few[k] = (uint32_t)__builtin_amdgcn_readlane((int)slot, k * G);
  }
  // The loads of the batch at access t0: buf receives the values, dst the
  // output addresses, ok whether the access exists, pad whether it is a
  // padding column.
  auto issue = [&](uint32_t t0, T* buf, T** dst, bool* ok, bool* pad) {
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      const uint32_t t = t0 + q * 64 + lane;
      uint32_t s = t / (2u * per_row);
      if (s >= SPW) s = SPW - 1;
      uint32_t slot_s;
      if constexpr (SPW <= 4) {
        slot_s = few[0];
#pragma unroll
        for (int k = 1; k < SPW; ++k)
          if (s == (uint32_t)k) slot_s = few[k];
      } else {
        slot_s = (uint32_t)__shfl((int)slot, (int)s * G);
      }
      const uint32_t bs = wave_b0 + s;
      ok[q] = t < total && bs < a.B;
      const uint32_t rem = t - s * 2u * per_row;
      const bool nxt = rem >= per_row;
      const uint32_t c = nxt ? rem - per_row : rem;
      pad[q] = c >= per_src;
      const float* src = (nxt ? src_n : src_s) + (uint64_t)slot_s * D;
      dst[q] = reinterpret_cast<T*>((nxt ? dst_n : dst_s) + (uint64_t)bs * W) + c;
      // Unconditional: s is clamped to a sample of the wave (a descent of an
      // inactive lane still ends on a leaf) and past-the-end or padding
      // accesses read column 0, so the address is always in the row store.
      const uint32_t col = (pad[q] || !ok[q]) ? 0u : c;
      if constexpr (NT && VEC) {
        typedef float f32x4 __attribute__((ext_vector_type(4)));
        const f32x4 x = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src) + col);
        buf[q] = make_float4(x.x, x.y, x.z, x.w);
      } else if constexpr (NT) {
        buf[q] = __builtin_nontemporal_load(src + col);
      } else {
        buf[q] = reinterpret_cast<const T*>(src)[col];
      }
    }
  };
  auto store = [&](const T* buf, T* const* dst, const bool* ok, const bool* pad) {
#pragma unroll
    for (int q = 0; q < kBatch; ++q) {
      if (ok[q]) *dst[q] = pad[q] ? T{} : buf[q];
    }
  };
  if constexpr (G == 1) {
    T buf[kBatch];
    T* dst[kBatch];
    bool ok[kBatch], pad[kBatch];
    if (total > 0) {
      issue(0, buf, dst, ok, pad);
      mid();
    }
    for (uint32_t t0 = 0; t0 < total; t0 += 64 * kBatch) {
      T nbuf[kBatch];
      T* ndst[kBatch];
      bool nok[kBatch], npad[kBatch];
      const bool more = t0 + 64 * kBatch < total;  // uniform
      if (more) issue(t0 + 64 * kBatch, nbuf, ndst, nok, npad);
      store(buf, dst, ok, pad);
      if (more) {
#pragma unroll
        for (int q = 0; q < kBatch; ++q) {
          buf[q] = nbuf[q];
          dst[q] = ndst[q];
          ok[q] = nok[q];
          pad[q] = npad[q];
        }
      }
    }
  } else {
    // Written out in the loop: captured by a lambda, the slots in few[]
    // would live in scratch memory.
    for (uint32_t t0 = 0; t0 < total; t0 += 64 * kBatch) {
      T buf[kBatch];
      T* dst[kBatch];
      bool ok[kBatch], pad[kBatch];
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        const uint32_t t = t0 + q * 64 + lane;
        uint32_t s = t / (2u * per_row);
        if (s >= SPW) s = SPW - 1;
        uint32_t slot_s;
        if constexpr (SPW <= 4) {
          slot_s = few[0];
#pragma unroll
          for (int k = 1; k < SPW; ++k)
            if (s == (uint32_t)k) slot_s = few[k];
        } else {
          slot_s = (uint32_t)__shfl((int)slot, (int)s * G);
        }
        const uint32_t bs = wave_b0 + s;
        ok[q] = t < total && bs < a.B;
        const uint32_t rem = t - s * 2u * per_row;
        const bool nxt = rem >= per_row;
        const uint32_t c = nxt ? rem - per_row : rem;
        pad[q] = c >= per_src;
        const float* src = (nxt ? src_n : src_s) + (uint64_t)slot_s * D;
        dst[q] = reinterpret_cast<T*>((nxt ? dst_n : dst_s) + (uint64_t)bs * W) + c;
        // Unconditional: s is clamped to a sample of the wave and
        // past-the-end or padding accesses read column 0.
        const uint32_t col = (pad[q] || !ok[q]) ? 0u : c;
        if constexpr (NT && VEC) {
          typedef float f32x4 __attribute__((ext_vector_type(4)));
          const f32x4 x =
              __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(src) + col);
          buf[q] = make_float4(x.x, x.y, x.z, x.w);
        } else if constexpr (NT) {
          buf[q] = __builtin_nontemporal_load(src + col);
        } else {
          buf[q] = reinterpret_cast<const T*>(src)[col];
        }
      }
      if (t0 == 0) mid();
#pragma unroll
      for (int q = 0; q < kBatch; ++q) {
        if (ok[q]) *dst[q] = pad[q] ? T{} : buf[q];
      }
    }
  }
  if (total == 0) mid();
}

// Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers: As
// Easy as 1, 2, 3", SC 2011): ten rounds over a 4 x 64-bit counter and a
// 2 x 64-bit key; a round takes the 128-bit products of counter words 0 and
// 2 with the two round multipliers and mixes their halves with words 1 and 3
// and the key, which gains the two Weyl increments between rounds.  Word j of
// a seed's stream is word j % 4 of the block at counter (j / 4, 0, 0, 0)
// under key (seed, 0).
__device__ __forceinline__ uint64_t stream_word(uint64_t seed, uint64_t j) {
  uint64_t c0 = j >> 2, c1 = 0, c2 = 0, c3 = 0;
  uint64_t k0 = seed, k1 = 0;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B97F4A7C15ull;
      k1 += 0xBB67AE8584CAA73Bull;
    }
    const uint64_t m0 = 0xD2E7470EE14C6C93ull, m1 = 0xCA5A826395121157ull;
    const uint64_t hi0 = __umul64hi(m0, c0), lo0 = m0 * c0;
    const uint64_t hi1 = __umul64hi(m1, c2), lo1 = m1 * c2;
    const uint64_t n0 = hi1 ^ c1 ^ k0, n2 = hi0 ^ c3 ^ k1;
    c0 = n0;
    c1 = lo1;
    c2 = n2;
    c3 = lo0;
  }
  const uint32_t w = (uint32_t)(j & 3u);
  return w == 0 ? c0 : (w == 1 ? c1 : (w == 2 ? c2 : c3));
}

// The mass uniform of a stream word: its top 24 bits times 2^-24, in [0, 1).
__device__ __forceinline__ float stream_uniform(uint64_t w) {
  return (float)(uint32_t)(w >> 40) * 0x1p-24f;
}

// Outputs of one sample (lead: the lane of its group that writes them): the
// index, the IS weight and, cooperatively over the wave, the row copy (NT:
// rows read with the non-temporal hint).
// The IS weight (p / pmin)^-beta of a sampled priority p >= pmin > 0.  With
// both normal and 0 <= beta <= 1: p = 2^e1 m1, pmin = 2^e0 m0 (m in [1, 2)),
// so log2(p / pmin) = L = (e1 - e0) + log2 m1 - log2 m0, the integer part
// exact and each f32 logarithm of a significand within 2^-24 of the true
// value; z = -beta L in f64, n the integer nearest z and w = 2^n 2^(z - n)
// with the fraction's power in f32.  The exponent is then off by at most
// beta 2^-23 + 2^-26 (the fraction rounded to f32) and the f32 power by one
// unit in its last place, so w lies within 2.1e-7 relative of the exact
// value, and of the f64 formula's value rounded to f32 within 2.7e-7.
// Otherwise, or where w would leave the f32 normal range, the f64 power
// (pow_f32).
__device__ __forceinline__ float is_weight(float p, float pmin, double beta) {
  const uint32_t pb = __float_as_uint(p), qb = __float_as_uint(pmin);
  const uint32_t pe = pb >> 23, qe = qb >> 23;  // sign and exponent: positive normal in [1, 254]
  if (pe - 1u < 254u && qe - 1u < 254u && beta >= 0.0 && beta <= 1.0) {
    const float m1 = __uint_as_float((pb & 0x007FFFFFu) | 0x3F800000u);
    const float m0 = __uint_as_float((qb & 0x007FFFFFu) | 0x3F800000u);
    const double L = (double)((int)pe - (int)qe) + ((double)log2f(m1) - (double)log2f(m0));
    const double z = -beta * L;
    const double n = rint(z);
    if (n >= -125.0 && n <= 127.0) return ldexpf(exp2f((float)(z - n)), (int)n);
  }
  return pow_f32((double)p / (double)pmin, -beta);
}

template <int G, int SPW, bool NT>
__device__ __forceinline__ void emit(const SampleArgs& a, uint32_t wave, int lane, uint32_t b,
                                     bool lead, uint32_t slot, float leaf, float pmin) {
  // The scalar fields of the sampled transition: loaded now, stored after
  // the rows, so that their trip to memory overlaps the row copy.
  uint32_t act = 0u;
  float rew = 0.0f;
  uint8_t done = 0;
  if (lead && a.states_out) {
    act = a.st.actions[slot];
    rew = a.st.rewards[slot];
    done = a.st.dones[slot];
  }
  if (lead) a.idx_out[b] = (int64_t)slot;
  // The weight, computed while the rows' loads are in flight.
  auto weight = [&]() {
    if (lead && a.w_out) {
      // (N P_i)^-beta / (N P_min)^-beta = (p_i / p_min)^-beta: one power
      // (is_weight).  With p_min > 0 every stored priority, the sampled one
      // included, is > 0; with p_min = 0 the normaliser is infinite and w = 0.
      float w = 0.0f;
      if (pmin > 0.0f) w = is_weight(leaf, pmin, a.beta);
      a.w_out[b] = w;
    }
  };

  if (!a.states_out) weight();
  if (a.states_out) {
    const uint32_t D = (uint32_t)a.st.D, W = a.out_stride;
    const bool vec = ((D | W) & 3u) == 0u;
    const uint32_t per_lane = (SPW * 2u * (vec ? W / 4 : W) + 63u) / 64u;  // accesses per lane
    if (vec) {
      if (per_lane <= 1)
        copy_rows<true, NT, SPW, G, 1>(a, wave * SPW, slot, lane, D, W, weight);
      else if (per_lane <= 2)
        copy_rows<true, NT, SPW, G, 2>(a, wave * SPW, slot, lane, D, W, weight);
      else if (per_lane <= 4)
        copy_rows<true, NT, SPW, G, 4>(a, wave * SPW, slot, lane, D, W, weight);
      else
        copy_rows<true, NT, SPW, G, 8>(a, wave * SPW, slot, lane, D, W, weight);
    } else {
      if (per_lane <= 2)
        copy_rows<false, NT, SPW, G, 2>(a, wave * SPW, slot, lane, D, W, weight);
      else
        copy_rows<false, NT, SPW, G, 8>(a, wave * SPW, slot, lane, D, W, weight);
    }
  }
  if (lead && a.states_out) {
    a.actions_out[b] = act;  // the stored bits, read as u32 or i32 by the caller
    a.rewards_out[b] = rew;
    if (a.dones_f32)
      static_cast<float*>(a.dones_out)[b] = (float)done;
    else
      static_cast<uint8_t*>(a.dones_out)[b] = done;
  }
}

// STREAM: masses from the generator stream instead of a.u.  FN > 0: the
// levels below the top are exactly FN rounds of FR levels (the usual
// 4096-leaf partitions), known when compiling, so that the rounds are
// unrolled and test no lane count; else a.nrounds rounds of a.rounds[r].
// TP > 0: the top is rebuilt from 2^TP partition roots (a.P == TP), so
// that the rebuild's and the walk's loops are fixed too.
template <int G, int V, bool STREAM, int FR, int FN, int TP>
__global__ void __launch_bounds__(kSampleThreads) sample_kernel(const float* u, float* sum, float* mn,
                                                                uint32_t B, SampleArgs a) {
  // The masses, the trees and the batch size arrive in scalar registers with
  // the wave (the leading arguments, preloaded; the same as a's), so the
  // first loads issue at once.
  extern __shared__ float top[];  // nodes [0, 2^(K+1)) of the sum tree
  // The other arguments the first steps need, fetched in one batch: left to
  // itself, the compiler loads each after the branch that first needs it,
  // one dependent trip each.  With the top's depth fixed when compiling they
  // are fetched once the first loads are in flight (below).
  if constexpr (TP == 0)
    asm volatile("" ::"s"(a.top_mode), "s"(a.P), "s"(a.top), "s"(a.nrounds));
  PER_SAMPLE_STAMP(0);
  constexpr int LOGG = ilog2(G);
  constexpr int LOGV = ilog2(V);
  constexpr int SPW = 64 / G;  // samples per wave

  const int lane = threadIdx.x & 63;
  const int j = lane & (G - 1);
  const int gbase = lane & ~(G - 1);
  const uint32_t wave = blockIdx.x * (kSampleThreads / 64) + (threadIdx.x >> 6);
  const uint32_t b = wave * SPW + (uint32_t)(lane / G);
  const bool active = b < B;
  // The sample's mass is fetched first, so that its trip overlaps the
  // top rebuild's loads instead of following them.
  float ub = 0.0f;
  if (!STREAM && active) ub = u[b];

  // One sample per wave and a top of 2^8 .. 2^10 roots: each wave keeps the
  // whole top in registers instead of sharing an LDS copy with its block.
  constexpr bool kWaveTop = G == 64 && TP >= 8 && TP <= 10;
  float T, pmin;
  uint32_t node = 1;
  if constexpr (kWaveTop) {
    // Lane l holds roots [C l, C l + C), sums and mins.  The nodes above
    // them follow by pairwise adds: within the lane (lane_descent forms
    // them as it goes), then across lanes, where after step k lane l holds
    // the node over the 2^k aligned lanes around it (f32 addition is
    // commutative, so both lanes of a pair get the node's value).  The walk
    // through the cross-lane levels reads the two children of the current
    // node from the first lane of each half (the path is wave-uniform, so
    // these are lane reads), and the last log2(C) levels run inside the
    // chosen lane.  Bit for bit the stored nodes, as every other top
    // rebuild; no LDS and no barrier.
    constexpr int C = (1 << TP) / 64;
    const uint32_t np = 1u << TP;
    float r[C], mr[C];
#pragma unroll
    for (int i = 0; i < C; i += 4) {
      const float4 q = *reinterpret_cast<const float4*>(sum + np + (uint32_t)lane * C + i);
      const float4 w = *reinterpret_cast<const float4*>(mn + np + (uint32_t)lane * C + i);
      r[i] = q.x;
      r[i + 1] = q.y;
      r[i + 2] = q.z;
      r[i + 3] = q.w;
      mr[i] = w.x;
      mr[i + 1] = w.y;
      mr[i + 2] = w.z;
      mr[i + 3] = w.w;
    }
    asm volatile("" ::"s"(a.top), "s"(a.nrounds));
    float x[6];
    x[0] = pair_sum<C>(r);
    float mm = mr[0];
#pragma unroll
    for (int i = 1; i < C; ++i) mm = min_f32(mm, mr[i]);
#pragma unroll
    for (int k = 1; k < 6; ++k) x[k] = x[k - 1] + xor_lanes(x[k - 1], k - 1);
#pragma unroll
    for (int k = 0; k < 5; ++k) mm = min_f32(mm, xor_lanes(mm, k));
    const float left0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[5]), 0));
    const float right0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[5]), 32));
    T = left0 + right0;
    pmin = min_f32(__int_as_float(__builtin_amdgcn_readlane(__float_as_int(mm), 0)),
                   __int_as_float(__builtin_amdgcn_readlane(__float_as_int(mm), 32)));
    if (STREAM && active) ub = stream_uniform(stream_word(a.seed, a.offset + b));
    // The wave's one mass, made visibly uniform so that the walk's decisions
    // and lane numbers stay scalar.
    ub = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(ub)));
    float m = ub * T;
    if (!(m < T)) m = __uint_as_float(__float_as_uint(T) - 1u);  // largest f32 below T
    int base = 0;  // first lane under the current node
#pragma unroll
    for (int k = 5; k >= 0; --k) {  // each child covers 2^k lanes
      const float cl = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[k]), base));
      const float cr =
          __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x[k]), base + (1 << k)));
      const bool right = !(cl > m || cr == 0.0f);
      if (right) {
        m = m - cl;
        base += 1 << k;
      }
    }
    float lm = m, lv;
    const int e = lane_descent<C>(r, lm, lv);
    m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lm), base));
    node = np + (uint32_t)(base * C + __builtin_amdgcn_readlane(e, base));
    ub = m;  // carried to the rounds below
  } else if (TP > 0 || a.top_mode == kTopRebuild) {
    // Nodes [1, 2^P) from the partition roots at depth P: sums in top[],
    // mins in mtop[].  With more than 512 roots the levels down to depth 8
    // are reduced block-wide first, two levels per pass: a thread takes four
    // consecutive nodes (one 16-byte access), stores them and forms their two
    // parents and their grandparent in registers, so that a barrier separates
    // every second level only; the first pass reads the roots from global
    // memory.  Thread t ends holding node 2^8 + t.  Then each wave reduces a
    // contiguous segment of depth 8 (or, with at most 512 roots, of the roots
    // themselves, at most two per lane) in registers and lane shuffles,
    // every node formed on the way stored to LDS.  Only the joins of the four
    // segment roots wait for a barrier.
    const int P = TP > 0 ? TP : a.P;
    const uint32_t np = 1u << P;
    float* mtop = top + 2 * np;
    const int wv = threadIdx.x >> 6;
    const int lgw = (P >= 8) ? 2 : 0;  // log2 of the waves of the wave stage
    const int Pw = (P - lgw > 7) ? lgw + 6 : P;
    const int lgseg = Pw - lgw;                 // log2 of a wave's nodes at depth Pw
    const int lgc = lgseg > 6 ? lgseg - 6 : 0;  // log2 of nodes per lane (<= 1)
    const int lgl = lgseg - lgc;                // log2 of the lanes used
    // Four nodes of depth d at index q (a multiple of 4): stored when they
    // come from global memory, and their parents and grandparent formed and
    // stored; returns the grandparent.
    auto quad = [&](int d, uint32_t q, float4 cs, float4 cm, bool fresh, float& gm) {
      if (fresh) {
        *reinterpret_cast<float4*>(top + (1u << d) + q) = cs;
        *reinterpret_cast<float4*>(mtop + (1u << d) + q) = cm;
      }
      const float2 ps = make_float2(cs.x + cs.y, cs.z + cs.w);
      const float2 pm = make_float2(min_f32(cm.x, cm.y), min_f32(cm.z, cm.w));
      *reinterpret_cast<float2*>(top + (1u << (d - 1)) + (q >> 1)) = ps;
      *reinterpret_cast<float2*>(mtop + (1u << (d - 1)) + (q >> 1)) = pm;
      const float gs = ps.x + ps.y;
      gm = min_f32(pm.x, pm.y);
      top[(1u << (d - 2)) + (q >> 2)] = gs;
      mtop[(1u << (d - 2)) + (q >> 2)] = gm;
      return gs;
    };
    float hs = 0.0f, hm = 0.0f;  // node 2^Pw + threadIdx.x, when Pw < P
    if (Pw < P) {
      constexpr int kG = (1 << kMaxTopBits) / 4 / kSampleThreads;  // root quads per thread
      const uint32_t nq = np >> 2;
      float4 rs[kG], rm[kG];
#pragma unroll
      for (int c = 0; c < kG; ++c) {
        const uint32_t g = threadIdx.x + c * kSampleThreads;
        if (g < nq) {
          rs[c] = *reinterpret_cast<const float4*>(sum + np + 4 * g);
          rm[c] = *reinterpret_cast<const float4*>(mn + np + 4 * g);
        }
      }
      if constexpr (TP > 0) asm volatile("" ::"s"(a.top), "s"(a.nrounds));
#pragma unroll
      for (int c = 0; c < kG; ++c) {
        const uint32_t g = threadIdx.x + c * kSampleThreads;
        if (g < nq) {
          float m2;
          const float s2 = quad(P, 4 * g, rs[c], rm[c], true, m2);
          if (c == 0) {  // with 2^10 roots this is node 2^8 + threadIdx.x
            hs = s2;
            hm = m2;
          }
        }
      }
      // Down to depth 8 in LDS; each pass that reaches it leaves thread t
      // with node 2^8 + t.
      for (int d = P - 2; d > Pw;) {
        __syncthreads();
        if (d - Pw >= 2) {
          for (uint32_t g = threadIdx.x; g < (1u << (d - 2)); g += kSampleThreads) {
            const float4 cs = reinterpret_cast<const float4*>(top + (1u << d))[g];
            const float4 cm = reinterpret_cast<const float4*>(mtop + (1u << d))[g];
            float m2;
            const float s2 = quad(d, 4 * g, cs, cm, false, m2);
            hs = s2;
            hm = m2;
          }
          d -= 2;
        } else {
          for (uint32_t g = threadIdx.x; g < (1u << (d - 1)); g += kSampleThreads) {
            const float2 cs = reinterpret_cast<const float2*>(top + (1u << d))[g];
            const float2 cm = reinterpret_cast<const float2*>(mtop + (1u << d))[g];
            hs = cs.x + cs.y;
            hm = min_f32(cm.x, cm.y);
            top[(1u << (d - 1)) + g] = hs;
            mtop[(1u << (d - 1)) + g] = hm;
          }
          d -= 1;
        }
      }
    }
    if (wv < (1 << lgw)) {
      const uint32_t k0 = (1u << Pw) + ((uint32_t)wv << lgseg) + ((uint32_t)lane << lgc);
      const bool on = lane < (1 << lgl);
      const uint32_t c = 1u << lgc;
      float v[2], mv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        v[i] = 0.0f;
        mv[i] = 0.0f;
        if (on && (uint32_t)i < c) {
          if (Pw < P) {  // lgc == 0: the node this thread formed above
            v[i] = hs;
            mv[i] = hm;
          } else {
            v[i] = sum[k0 + i];
            mv[i] = mn[k0 + i];
          }
        }
      }
      if (on && Pw == P) {
#pragma unroll
        for (int i = 0; i < 2; ++i) {
          if ((uint32_t)i < c) {
            top[k0 + i] = v[i];
            mtop[k0 + i] = mv[i];
          }
        }
      }
      if (lgc == 1) {
        v[0] = v[0] + v[1];
        mv[0] = min_f32(mv[0], mv[1]);
        if (on) {
          top[k0 >> 1] = v[0];
          mtop[k0 >> 1] = mv[0];
        }
      }
      float s0 = v[0], m0 = mv[0];
#pragma unroll
      for (int q = 0; q < 6; ++q) {
        if (q < lgl) {  // uniform
          const float sr = down_lanes(s0, q);
          const float mr = down_lanes(m0, q);
          if (on && (lane & ((2 << q) - 1)) == 0) {
            s0 = s0 + sr;
            m0 = min_f32(m0, mr);
            const uint32_t x = k0 >> (lgc + q + 1);
            top[x] = s0;
            mtop[x] = m0;
          }
        }
      }
    }
    __syncthreads();
    if (lgw > 0) {
      // The four segment roots are nodes 4..7.
      if (threadIdx.x == 0) {
        const float s2 = top[4] + top[5], s3 = top[6] + top[7];
        const float m2 = min_f32(mtop[4], mtop[5]), m3 = min_f32(mtop[6], mtop[7]);
        top[2] = s2;
        top[3] = s3;
        mtop[2] = m2;
        mtop[3] = m3;
        top[1] = s2 + s3;
        mtop[1] = min_f32(m2, m3);
      }
      __syncthreads();
    }
    T = top[1];
    pmin = mtop[1];
    // Taken here, from LDS: left to itself the compiler merges the two
    // branches' reads into one generic load behind a wait for all memory.
    asm volatile("" ::"v"(T), "v"(pmin));
  } else {
    if (a.top_mode == kTopWhole) {
      const uint32_t cnt = 1u << (a.top + 1);  // whole tree, >= 4 floats
      for (uint32_t i = threadIdx.x * 4; i < cnt; i += kSampleThreads * 4)
        *reinterpret_cast<float4*>(top + i) = *reinterpret_cast<const float4*>(sum + i);
      __syncthreads();
    }
    T = sum[1];
    pmin = mn[1];
  }

  float m;
  if constexpr (kWaveTop) {
    m = ub;  // the mass left after the wave's walk through the top
  } else {
    if (STREAM && active) ub = stream_uniform(stream_word(a.seed, a.offset + b));
    m = ub * T;
    if (!(m < T)) m = __uint_as_float(__float_as_uint(T) - 1u);  // largest f32 below T
    const int levels_in_lds = TP > 0 ? TP : a.top;
#pragma unroll
    for (int l = 0; l < levels_in_lds; ++l) {
      const float2 c = reinterpret_cast<const float2*>(top)[node];  // children 2node, 2node+1
      const bool right = !(c.x > m || c.y == 0.0f);
      if (right) m = m - c.x;
      node = 2 * node + (right ? 1u : 0u);
    }
  }
  float leaf = 0.0f;
  if (!kWaveTop && a.nrounds == 0) leaf = top[node];

  auto round = [&](const int R) {
    const int lg = R - LOGV;  // log2 of the lanes used this round (<= LOGG)
    const uint32_t base = node << R;
    const bool used = j < (1 << lg);
    float x[V];
    if (used) {
      load_values<V>(sum + base + (uint32_t)j * V, x);
    } else {
#pragma unroll
      for (int i = 0; i < V; ++i) x[i] = 0.0f;
    }
    float v = pair_sum<V>(x);
    float lrec[LOGG + 1], rrec[LOGG + 1];
#pragma unroll
    for (int s = 1; s <= LOGG; ++s) {
      lrec[s] = rrec[s] = 0.0f;
      if (s <= lg) {
        const float pv = xor_lanes(v, s - 1);
        const bool hi = (j >> (s - 1)) & 1;
        lrec[s] = hi ? pv : v;
        rrec[s] = hi ? v : pv;
        v = lrec[s] + rrec[s];
      }
    }
    bool on = used;
#pragma unroll
    for (int s = LOGG; s >= 1; --s) {
      if (s <= lg) {
        const bool right = !(lrec[s] > m || rrec[s] == 0.0f);
        if (right) m = m - lrec[s];
        on = on && (((j >> (s - 1)) & 1) == (right ? 1 : 0));
      }
    }
    float lv;
    const int e = lane_descent<V>(x, m, lv);
    uint32_t pos = (uint32_t)j * V + (uint32_t)e;
    if constexpr (G == 64) {
      // One sample per wave: the lane that holds the path is wave-uniform.
      const uint64_t mask = __ballot(on);
      const int src = mask ? (__ffsll((unsigned long long)mask) - 1) : 0;
      m = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(m), src));
      pos = (uint32_t)__builtin_amdgcn_readlane((int)pos, src);
      lv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(lv), src));
    } else if constexpr (G > 1) {
      const uint64_t mask = __ballot(on);
      const uint64_t gm = (mask >> gbase) & ((1ull << G) - 1ull);
      const int src = gbase + (gm ? (__ffsll((unsigned long long)gm) - 1) : 0);
      m = __shfl(m, src);
      pos = (uint32_t)__shfl((int)pos, src);
      lv = __shfl(lv, src);
    }
    node = base + pos;
    leaf = lv;
  };
  if constexpr (FN > 0) {
#pragma unroll
    for (int r = 0; r < FN; ++r) round(FR);
  } else {
    for (int r = 0; r < a.nrounds; ++r) round(a.rounds[r]);
  }

  uint32_t slot = node - a.n;
  if (a.order) slot = a.order[slot];  // rank-based: the descent gave a rank
  emit<G, SPW, true>(a, wave, lane, b, active && j == 0, slot, leaf, pmin);
  PER_SAMPLE_STAMP(1);
}

// Uniform sample over the filled slots ("GPU-Resident Prioritized
// Experience Replay", section "Experience Insertion": without
// prioritisation the same ring is sampled uniformly from generated indices
// into [0, size)): G lanes per sample (as the proportional sampler: 16 for
// small batches, so that they spread over more of the chip, else 1), slot =
// ((word >> 32) * size) >> 32, then the rows.  Lanes past B still land on a
// filled slot, which the wave's row copy relies on.
template <int G>
__global__ void __launch_bounds__(kSampleThreads) uniform_kernel(SampleArgs a) {
  // The arguments the first steps need, fetched in one batch.
  asm volatile("" ::"s"(a.seed), "s"(a.offset), "s"(a.size), "s"(a.dev_size), "s"(a.B),
               "s"(a.idx_out), "s"(a.st.D));
  constexpr int SPW = 64 / G;
  const int lane = threadIdx.x & 63;
  const uint32_t wave = blockIdx.x * (kSampleThreads / 64) + (threadIdx.x >> 6);
  const uint32_t b = wave * SPW + (uint32_t)(lane / G);
  const uint32_t size = a.dev_size ? *a.dev_size : a.size;
  const uint64_t hi = stream_word(a.seed, a.offset + b) >> 32;
  const uint32_t slot = (uint32_t)((hi * (uint64_t)size) >> 32);
  emit<G, SPW, false>(a, wave, lane, b, b < a.B && (lane & (G - 1)) == 0, slot, 0.0f, 0.0f);
}

template <int G, int V, bool STREAM, int FR, int FN, int TP>
hipError_t launch_one(const SampleArgs& a, unsigned grid, size_t lds, hipStream_t s) {
  return launch_kernel(sample_kernel<G, V, STREAM, FR, FN, TP>, dim3(grid), dim3(kSampleThreads),
                       lds, s, a.u, a.sum, a.mn, a.B, a);
}

// The usual round shape (FR, FN) with the top depth of trees of 2^20 to
// 2^24 leaves fixed when compiling; other depths at run time.
template <int G, int V, bool STREAM, int FR, int FN>
hipError_t launch_fixed(const SampleArgs& a, unsigned grid, size_t lds, hipStream_t s) {
  switch (a.top_mode == kTopRebuild ? a.P : 0) {
    case 8:
      return launch_one<G, V, STREAM, FR, FN, 8>(a, grid, lds, s);
    case 9:
      return launch_one<G, V, STREAM, FR, FN, 9>(a, grid, lds, s);
    case 10:
      return launch_one<G, V, STREAM, FR, FN, 10>(a, grid, lds, s);
    case 11:
      return launch_one<G, V, STREAM, FR, FN, 11>(a, grid, lds, s);
    case 12:
      return launch_one<G, V, STREAM, FR, FN, 12>(a, grid, lds, s);
    default:
      return launch_one<G, V, STREAM, FR, FN, 0>(a, grid, lds, s);
  }
}

// FR, FN: the round shape of the usual partition for this G and V, taken
// when the plan has exactly that shape.
template <int G, int V, int FR, int FN>
hipError_t launch_variant(const SampleArgs& a, hipStream_t s) {
  constexpr int SPW = 64 / G;
  const uint64_t waves = (a.B + SPW - 1) / SPW;
  const unsigned grid = (unsigned)((waves + 3) / 4);
  size_t lds = 0;
  if (a.top_mode == kTopRebuild) lds = 2 * (sizeof(float) << (a.P + 1));
  // One sample per wave over 2^8 .. 2^10 roots: the top lives in registers.
  if (G == 64 && a.top_mode == kTopRebuild && a.P >= 8 && a.P <= 10) lds = 0;
  if (a.top_mode == kTopWhole) lds = sizeof(float) << (a.top + 1);
  bool fixed = a.nrounds == FN;
  for (int r = 0; r < a.nrounds; ++r) fixed = fixed && a.rounds[r] == FR;
  if (a.u && fixed) return launch_fixed<G, V, false, FR, FN>(a, grid, lds, s);
  if (a.u) return launch_one<G, V, false, 0, 0, 0>(a, grid, lds, s);
  if (fixed) return launch_fixed<G, V, true, FR, FN>(a, grid, lds, s);
  return launch_one<G, V, true, 0, 0, 0>(a, grid, lds, s);
}

// Split `levels` into rounds of lo..hi levels, larger rounds first.
void split_rounds(int levels, int hi, SamplePlan& p) {
  p.nrounds = 0;
  if (levels <= 0) return;
  const int k = (levels + hi - 1) / hi;
  const int base = levels / k, extra = levels % k;
  for (int r = 0; r < k; ++r) p.rounds[p.nrounds++] = base + (r < extra ? 1 : 0);
}

}  // namespace

// Modes: 1 = one wave per sample (G=64, V=4, rounds of up to 8 levels);
// 2 = 16 lanes per sample (G=16, V=4, up to 6 levels);
// 3 = one lane per sample (G=1, V=16, rounds of exactly 4 levels).
// Batches of a few hundred samples take one wave per sample, up to a few
// thousand when they gather rows of 32 floats or more: the row copies then
// spread over four times as many waves (measured on the DQN step, 2^20
// slots of 64 floats, B = 1024: 0.65 us less per step; without rows, 2^21
// slots and B = 512: 0.1 us less).  With very few samples, or thousands
// without rows, the extra blocks and top rebuilds cost more than they give.
SamplePlan make_sample_plan(const Geom& g, int64_t B, uint32_t row_floats, int forced_mode) {
  SamplePlan p{};
  p.mode = (B <= 16384) ? 2 : 3;
  if (B >= 256 && B <= (row_floats >= 32 ? 2048 : 1024)) p.mode = 1;
  if (forced_mode >= 1 && forced_mode <= 3) p.mode = forced_mode;
  if (g.P > 0 && g.P <= kMaxTopBits) {
    p.top_mode = kTopRebuild;
    p.top_levels = g.P;
  } else if (g.P == 0 && g.L <= 10) {
    p.top_mode = kTopWhole;
    p.top_levels = g.L;
  } else {
    p.top_mode = kTopNone;
    p.top_levels = 0;
  }
  const int levels = g.L - p.top_levels;
  if (p.mode == 3 && levels % 4 != 0) p.mode = 2;
  if (p.mode == 2 && levels > 0 && levels < 2) p.mode = 1;
  const int hi = (p.mode == 1) ? 8 : (p.mode == 2 ? 6 : 4);
  split_rounds(levels, hi, p);
  return p;
}

hipError_t launch_sample(const TreePtrs& t, const Geom& g, const Storage& st,
                         const SamplePlan& plan, uint32_t size, int64_t B, const float* u,
                         uint64_t seed, uint64_t offset, double beta, int64_t* idx_out,
                         float* w_out, float* states_out,
                         float* next_out, uint32_t* actions_out, float* rewards_out,
                         void* dones_out, uint32_t out_stride, bool dones_f32,
                         hipStream_t s, const uint32_t* order) {
  SampleArgs a{};
  a.sum = t.sum;
  a.mn = t.mn;
  a.n = g.n;
  a.size = size;
  a.B = (uint32_t)B;
  a.order = order;
  a.u = u;
  a.seed = seed;
  a.offset = offset;
  a.beta = beta;
  a.idx_out = idx_out;
  a.w_out = w_out;
  a.states_out = states_out;
  a.next_out = next_out;
  a.actions_out = actions_out;
  a.rewards_out = rewards_out;
  a.dones_out = dones_out;
  a.out_stride = out_stride;
  a.dones_f32 = dones_f32 ? 1 : 0;
  a.st = st;
  a.P = g.P;
  a.top_mode = plan.top_mode;
  a.top = plan.top_levels;
  a.nrounds = plan.nrounds;
  for (int r = 0; r < kMaxRounds; ++r) a.rounds[r] = plan.rounds[r];
  switch (plan.mode) {
    case 2:
      return launch_variant<16, 4, 6, 2>(a, s);
    case 3:
      return launch_variant<1, 16, 4, 3>(a, s);
    default:
      return launch_variant<64, 4, 6, 2>(a, s);
  }
}

hipError_t launch_uniform(const Storage& st, const Ctrl* ctrl, RingRef ring, uint32_t size,
                          int64_t B, uint64_t seed, uint64_t offset, int64_t* idx_out,
                          float* states_out, float* next_out, uint32_t* actions_out,
                          float* rewards_out, void* dones_out, uint32_t out_stride,
                          bool dones_f32, hipStream_t s) {
  SampleArgs a{};
  a.size = size;
  a.dev_size = ring.dev ? &ctrl->size[ring.slot] : nullptr;
  a.B = (uint32_t)B;
  a.seed = seed;
  a.offset = offset;
  a.idx_out = idx_out;
  a.states_out = states_out;
  a.next_out = next_out;
  a.actions_out = actions_out;
  a.rewards_out = rewards_out;
  a.dones_out = dones_out;
  a.out_stride = out_stride;
  a.dones_f32 = dones_f32 ? 1 : 0;
  a.st = st;
  if (B <= 16384) {
    const uint64_t waves = ((uint64_t)B + 3) / 4;
    return launch_kernel(uniform_kernel<16>, dim3((unsigned)((waves + 3) / 4)),
                         dim3(kSampleThreads), 0, s, a);
  }
  const uint64_t waves = ((uint64_t)B + 63) / 64;
  return launch_kernel(uniform_kernel<1>, dim3((unsigned)((waves + 3) / 4)), dim3(kSampleThreads),
                       0, s, a);
}

}  // namespace per
