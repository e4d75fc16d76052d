// per_internal.h -- shared definitions of the HIP sum-tree library (not
// installed; the public ABI is include/per.h).
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace per {

// Kernel-timing request of the calling host thread (per_time_next): while
// set, launches go through hipExtLaunchKernel, the first one recording
// `start` as it begins and each one recording `stop` as it ends, so that the
// two events bracket the call's kernels on the device.
struct KernelTiming {
  hipEvent_t start = nullptr;
  hipEvent_t stop = nullptr;
};
KernelTiming& kernel_timing();

// Every kernel of the library is launched through here.
template <typename... KArgs, typename... Args>
hipError_t launch_kernel(void (*kern)(KArgs...), dim3 grid, dim3 block, size_t lds, hipStream_t s,
                         Args... args) {
  KernelTiming& t = kernel_timing();
  if (t.start || t.stop) {
    hipExtLaunchKernelGGL(kern, grid, block, (uint32_t)lds, s, t.start, t.stop, 0u,
                          static_cast<KArgs>(args)...);
    t.start = nullptr;  // only the call's first kernel opens the interval
  } else {
    kern<<<grid, block, lds, s>>>(static_cast<KArgs>(args)...);
  }
  return hipGetLastError();
}

// Leaves per partition = 2^kMaxSpanBits.  The batched update and the intake
// work one workgroup per partition (an aligned subtree); the few levels above
// the partitions are rebuilt lazily (by the sampler, or by top_kernel).
constexpr int kMaxSpanBits = 12;
constexpr int kMaxSpan = 1 << kMaxSpanBits;
// Partitions holding at most this many updated leaves are repaired by one
// wave walking the leaf-to-partition-root chains; denser ones are rebuilt
// in LDS.
constexpr int kSparseMax = 64;
// Top levels (above the partitions) that fit in the workgroup's LDS.
constexpr int kMaxTopBits = 12;
constexpr int kTreeThreads = 256;

// Device control block at the start of the workspace's control area.
// The running max priority is kept in two slots (f32 bit patterns, raised
// with atomicMax): a call that may raise it reads the committed slot and
// raises the other, and the host then commits the other slot.  The ring
// state (cursor, size) is kept the same way: every intake reads slot r and
// writes the next state to slot r ^ 1, and the host flips r.  In graph mode
// the kernels take the ring state from these slots instead of from their
// launch arguments, so that a captured sequence of calls replays with the
// state of the replay, not of the capture.
struct Ctrl {
  uint32_t maxp_bits[2];
  uint32_t cursor[2];
  uint32_t size[2];
  uint32_t pad[2];
};

// Where a kernel takes the ring state from: its arguments (dev == 0), or
// slot `slot` of the control block (dev != 0, graph mode).
struct RingRef {
  int dev;
  int slot;
};

// Geometry shared by host and kernels.
struct Geom {
  uint32_t n;      // capacity (leaves)
  int L;           // log2(n)
  int S;           // leaves per partition = 2^S, S = min(L, kMaxSpanBits)
  int P;           // partitions = 2^P, P = L - S
};

struct TreePtrs {
  float* sum;      // [2n] sum tree; index 0 unused
  float* mn;       // [2n] min tree
  Ctrl* ctrl;
};

// Scratch of the bucketed (large-batch) update: a bucket of kBucketCap
// entries per partition and an overflow list for the rest.
constexpr int kBucketCap = kSparseMax;
// Words between two partitions' bucket counts: one count per 128-byte line,
// so that the bucketing pass's atomic adds to different partitions do not
// queue behind each other on a shared line (2^24 leaves, 65536 entries:
// update 25.2 -> 24.0 us against packed counts).
constexpr uint32_t kCountStride = 32;
struct Buckets {
  uint32_t* counts;   // [2^P * kCountStride] entries of partition p at [p * kCountStride] (reset by the update)
  uint32_t* ovf_n;    // [2] overflow counters, used by alternate calls
  uint32_t* slot;     // [2^P * kBucketCap] leaf slot of each bucketed entry
  uint32_t* pos;      // its batch position
  float* td;          // its TD error
  uint32_t* oslot;    // [max_batch] overflow entries
  uint32_t* opos;
  float* otd;
};

struct Storage {
  float* states;
  float* next_states;
  uint32_t* actions;
  float* rewards;
  uint8_t* dones;
  int D;
};

// Workspace layout (byte offsets from the 256-byte aligned base).
struct Layout {
  size_t sum, mn, ctrl, counts, ovf_n, slot, pos, td, oslot, opos, otd, total;
};
Layout workspace_layout(int64_t n, int64_t max_batch);
// The bucketed update's scratch for np partitions and max_batch entries laid
// out from base (256-byte aligned); *end receives the bytes it spans.
Buckets bucket_layout(char* base, size_t np, int64_t max_batch, size_t* end);

// Descent plan of the sampler.  The top of the tree reaches LDS either by a
// rebuild from the partition roots (kTopRebuild, 0 < P <= kMaxTopBits), by
// staging a whole small tree (kTopWhole, n <= 2^10), or not at all.
constexpr int kMaxRounds = 12;
constexpr int kTopNone = 0, kTopRebuild = 1, kTopWhole = 2;
struct SamplePlan {
  int mode;                 // kernel variant (group size, values per lane)
  int top_mode;             // how the top of the tree reaches LDS
  int top_levels;           // levels walked in the LDS copy of the tree top
  int nrounds;              // global rounds after the LDS top
  int rounds[kMaxRounds];   // levels per round
};

// ----------------------------------------------------------------- launchers
hipError_t launch_init(const TreePtrs& t, const Buckets& bk, const Geom& g, hipStream_t s);

// Batched update; B > 0.  src / dst: running-max slots to read / raise.
// ovf: overflow counter of this call when the batch is bucketed (see
// update_uses_buckets); alternate calls must alternate it.
// The filled size bounds the accepted indices: size, or ctrl->size[ring.slot]
// when ring.dev.
hipError_t launch_update(const TreePtrs& t, const Buckets& bk, const Geom& g, RingRef ring,
                         uint32_t size, int64_t B, const int64_t* idx, const float* td,
                         double alpha, double eps, int src, int dst, int ovf, hipStream_t s);
bool update_uses_buckets(const Geom& g, int64_t B);
// Zero the bucket counts of the 2^P partitions and both overflow counters
// (a fill kernel, so that a captured sequence clears them on every replay).
hipError_t launch_bucket_clear(const Buckets& bk, const Geom& g, hipStream_t s);

// Rebuild of the nodes above the partitions (one block).
hipError_t launch_top(const TreePtrs& t, const Geom& g, hipStream_t s);

// Ring intake of count > 0 items at cursor into a ring holding size items
// (both read from ctrl slot ring.slot instead when ring.dev).  Either way the
// ring state after the intake is written to ctrl slot ring.slot ^ 1.
hipError_t launch_add(const TreePtrs& t, const Geom& g, const Storage& st, RingRef ring,
                      uint32_t size, uint32_t cursor, uint32_t count, const float* states,
                      const float* next_states, const uint32_t* actions, const float* rewards,
                      const uint8_t* dones, const float* prio, int src, int dst, hipStream_t s);

// An update batch (B > 0, not bucketed: !update_uses_buckets(g, B)) and then
// an intake of count > 0 items, in one launch; the running max is read from
// slot src and raised in slot dst by both parts.
hipError_t launch_update_add(const TreePtrs& t, const Geom& g, const Storage& st, RingRef ring,
                             uint32_t size, uint32_t cursor, int64_t B, const int64_t* idx,
                             const float* td, double alpha, double eps, uint32_t count,
                             const float* states, const float* next_states,
                             const uint32_t* actions, const float* rewards, const uint8_t* dones,
                             const float* prio, int src, int dst, hipStream_t s);

hipError_t launch_sample(const TreePtrs& t, const Geom& g, const Storage& st,
                         const SamplePlan& plan, uint32_t size, int64_t B, const float* u,
                         uint64_t seed, uint64_t offset, double beta, int64_t* idx_out,
                         float* w_out, float* states_out,
                         float* next_out, uint32_t* actions_out, float* rewards_out,
                         void* dones_out, uint32_t out_stride, bool dones_f32,
                         hipStream_t s, const uint32_t* order = nullptr);

// forced_mode: 0 chooses the layout by batch and row width; 1, 2, 3 force
// one wave, 16 lanes or one lane per sample.
SamplePlan make_sample_plan(const Geom& g, int64_t B, uint32_t row_floats, int forced_mode);

// Rank-based prioritisation: a stable radix sort of the slots [0, count) by
// descending leaf priority (keys / vals: two ping-pong buffers of n words,
// the ranking ends in vals[0]; hist: rank_hist_words(n) words), and the
// build of the trees over the rank weights (count filled ranks).
hipError_t launch_rank_sort(const float* leaves, uint32_t count, uint32_t* const keys[2],
                            uint32_t* const vals[2], uint32_t* hist, hipStream_t s);
hipError_t launch_rank_build(const TreePtrs& rt, const Geom& g, uint32_t count, double alpha,
                             hipStream_t s);
size_t rank_hist_words(int64_t n);

// Uniform sample of B slots over [0, size) from the generator stream (size
// read from ctrl slot ring.slot when ring.dev).
hipError_t launch_uniform(const Storage& st, const Ctrl* ctrl, RingRef ring, uint32_t size,
                          int64_t B, uint64_t seed, uint64_t offset, int64_t* idx_out, float* states_out, float* next_out,
                          uint32_t* actions_out, float* rewards_out, void* dones_out,
                          uint32_t out_stride, bool dones_f32, hipStream_t s);

}  // namespace per
