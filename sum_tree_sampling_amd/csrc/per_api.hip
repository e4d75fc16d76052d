// per_api.hip -- the C ABI declared in include/per.h: argument checks,
// workspace layout, handle state and kernel launches.  Nothing here
// allocates device memory, and only leaving graph mode waits for the device.

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <cstdlib>
#include <mutex>
#include <new>
#include <string>

#include "../../include/per.h"
#include "per_internal.h"

struct per_s {
  per::Geom g;
  int64_t max_batch;
  double alpha, eps;
  per::TreePtrs t;
  per::Buckets bk;
  per::Storage st;
  int64_t size, cursor;
  int epoch;       // committed running-max slot
  int ovf;         // overflow counter for the next bucketed update
  int ring;        // control-block slot holding the current ring state
  bool top_stale;  // nodes above the partitions not yet rebuilt
  bool graph;      // graph mode: ring state read on the device, top always rebuilt
  int sample_mode;  // descent layout forced by per_set_sample_lanes (0: by batch)
  int entry_epoch, entry_ovf, entry_ring;  // parities when graph mode was entered
  int device;
  // rank-based prioritisation (after per_rank_attach)
  bool rank_attached;
  per::TreePtrs rt;      // trees over the rank weights (ctrl unused)
  uint32_t* rkeys[2];    // radix-sort ping-pong buffers, n words each
  uint32_t* rvals[2];    // rvals[0] holds the ranking after a refresh
  uint32_t* rhist;       // 16 words per 4096-item tile
  int64_t rank_size;     // filled slots at the last refresh (0: none)
  int64_t rank_built;    // count the rank-weight trees were built for (-1: none)
};

namespace {

thread_local std::string g_last_error;
thread_local per::KernelTiming g_timing;

// Every entry point returns through fail() or ok(), which also drop a
// pending timing request: per_time_next applies to one call only.
int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  g_timing = per::KernelTiming{};
  return code;
}

int ok() {
  g_last_error.clear();
  g_timing = per::KernelTiming{};
  return PER_OK;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(PER_EHIP, "%s: %s", what, hipGetErrorString(e));
}

bool pow2(int64_t v) { return v > 0 && (v & (v - 1)) == 0; }

// Ring state for a launch: the host's copy, or (graph mode) the device's.
per::RingRef ring_ref(const per_s* h) { return per::RingRef{h->graph ? 1 : 0, h->ring}; }

// Graph mode always rebuilds the nodes above the partitions: a replay cannot
// know what ran before it.
bool top_may_be_stale(const per_s* h) { return h->top_stale || (h->graph && h->g.P > 0); }

int log2i(int64_t v) {
  int l = 0;
  while ((int64_t(1) << l) < v) ++l;
  return l;
}

size_t align256(size_t v) { return (v + 255) & ~size_t(255); }

int check_capacity(int64_t capacity) {
  if (!pow2(capacity) || capacity < 2 || capacity > PER_MAX_CAPACITY)
    return fail(PER_EINVAL, "capacity %lld is not a power of two in [2, 2^30]",
                (long long)capacity);
  return PER_OK;
}

int check_batch_limit(int64_t max_batch) {
  if (max_batch < 1 || max_batch > PER_MAX_BATCH)
    return fail(PER_EINVAL, "max_batch %lld outside [1, 2^24]", (long long)max_batch);
  return PER_OK;
}

per::Geom make_geom(int64_t capacity) {
  per::Geom g;
  g.n = (uint32_t)capacity;
  g.L = log2i(capacity);
  g.S = g.L < per::kMaxSpanBits ? g.L : per::kMaxSpanBits;
  g.P = g.L - g.S;
  return g;
}

// ---------------------------------------------------- static update scratch
//
// per_update_static takes the bucketed update's scratch (bucket counts,
// overflow counters, buckets, overflow list) from this array instead of the
// handle's workspace.  Each device that loads the library holds its own copy
// until the process ends; host code reaches it only through the address
// hipGetSymbolAddress gives on that device (the array's name on the host is
// a stand-in, not a device address).  Sized for 2^12 partitions of 4096
// leaves (capacity <= 2^24) and batches of up to 2^16 entries.
constexpr int64_t kStaticMaxParts = int64_t(1) << 12;
constexpr int64_t kStaticMaxBatch = int64_t(1) << 16;
constexpr size_t kStaticScratchBytes = size_t(5) << 20;
constexpr int kMaxDevices = 64;

static __device__ __align__(256) unsigned char scratch[kStaticScratchBytes];

std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];  // the array's address on each device (NULL: not resolved)

// Resolves the array's address on `device`, which must be the current
// device.  Once per device; later calls return at once.
int resolve_static_scratch(int device) {
  if (device < 0 || device >= kMaxDevices) return PER_OK;  // per_update_static refuses it
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[device]) return PER_OK;
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (e != hipSuccess) return hip_fail(e, "static update scratch: hipGetSymbolAddress");
  g_scratch_ptr[device] = p;
  return PER_OK;
}

}  // namespace

namespace per {

KernelTiming& kernel_timing() { return g_timing; }

// The bucketed update's scratch for np partitions and max_batch entries,
// laid out from `base` (256-byte aligned) with the workspace's rules; the
// layout's end is returned in *end.
Buckets bucket_layout(char* base, size_t np, int64_t max_batch, size_t* end) {
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return base + at;
  };
  const size_t nb = np * kBucketCap;
  Buckets b;
  b.counts = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * np * kCountStride));
  b.ovf_n = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * 2));
  b.slot = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * nb));
  b.pos = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * nb));
  b.td = reinterpret_cast<float*>(take(sizeof(float) * nb));
  b.oslot = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)max_batch));
  b.opos = reinterpret_cast<uint32_t*>(take(sizeof(uint32_t) * (size_t)max_batch));
  b.otd = reinterpret_cast<float*>(take(sizeof(float) * (size_t)max_batch));
  if (end) *end = o;
  return b;
}

Layout workspace_layout(int64_t n, int64_t max_batch) {
  const Geom g = make_geom(n);
  const size_t np = size_t(1) << g.P;
  const size_t nb = np * kBucketCap;
  Layout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  l.sum = take(sizeof(float) * 2 * (size_t)n);
  l.mn = take(sizeof(float) * 2 * (size_t)n);
  l.ctrl = take(sizeof(Ctrl));
  l.counts = take(sizeof(uint32_t) * np * kCountStride);
  l.ovf_n = take(sizeof(uint32_t) * 2);
  l.slot = take(sizeof(uint32_t) * nb);
  l.pos = take(sizeof(uint32_t) * nb);
  l.td = take(sizeof(float) * nb);
  l.oslot = take(sizeof(uint32_t) * (size_t)max_batch);
  l.opos = take(sizeof(uint32_t) * (size_t)max_batch);
  l.otd = take(sizeof(float) * (size_t)max_batch);
  l.total = o;
  return l;
}

}  // namespace per

extern "C" {

int per_workspace_bytes(int64_t capacity, int64_t max_batch, size_t* out) {
  if (!out) return fail(PER_EINVAL, "out is NULL");
  int rc = check_capacity(capacity);
  if (rc) return rc;
  rc = check_batch_limit(max_batch);
  if (rc) return rc;
  *out = per::workspace_layout(capacity, max_batch).total;
  return ok();
}

int per_create(per_t** out, int64_t capacity, int32_t state_dim, int64_t max_batch,
               double alpha, double eps, void* d_ws, size_t ws_bytes, float* d_states,
               float* d_next_states, uint32_t* d_actions, float* d_rewards,
               uint8_t* d_dones, hipStream_t stream) {
  if (!out) return fail(PER_EINVAL, "out is NULL");
  *out = nullptr;
  int rc = check_capacity(capacity);
  if (rc) return rc;
  rc = check_batch_limit(max_batch);
  if (rc) return rc;
  if (state_dim < 0) return fail(PER_EINVAL, "state_dim %d < 0", (int)state_dim);
  if (!(alpha > 0.0) || !(alpha < 1e300) || !(eps >= 0.0) || !(eps < 1e300))
    return fail(PER_EINVAL, "alpha must be finite and > 0, eps finite and >= 0");
  if (!d_ws) return fail(PER_EINVAL, "workspace is NULL");
  if (reinterpret_cast<uintptr_t>(d_ws) & 255u)
    return fail(PER_EINVAL, "workspace is not 256-byte aligned");
  const per::Layout lay = per::workspace_layout(capacity, max_batch);
  if (ws_bytes < lay.total)
    return fail(PER_ENOSPC, "workspace of %zu bytes, %zu needed", ws_bytes, lay.total);
  const bool any_storage = d_states || d_next_states || d_actions || d_rewards || d_dones;
  const bool all_storage = d_states && d_next_states && d_actions && d_rewards && d_dones;
  if (state_dim > 0 && !all_storage)
    return fail(PER_EINVAL, "state_dim > 0 needs all five storage arrays");
  if (state_dim == 0 && any_storage)
    return fail(PER_EINVAL, "state_dim == 0 takes no storage arrays");
  if (state_dim > 0 && ((reinterpret_cast<uintptr_t>(d_states) |
                         reinterpret_cast<uintptr_t>(d_next_states)) & 15u))
    return fail(PER_EINVAL, "state arrays must be 16-byte aligned");

  per_s* h = new (std::nothrow) per_s();
  if (!h) return fail(PER_EINVAL, "out of host memory");
  h->g = make_geom(capacity);
  h->max_batch = max_batch;
  h->alpha = alpha;
  h->eps = eps;
  char* base = static_cast<char*>(d_ws);
  h->t.sum = reinterpret_cast<float*>(base + lay.sum);
  h->t.mn = reinterpret_cast<float*>(base + lay.mn);
  h->t.ctrl = reinterpret_cast<per::Ctrl*>(base + lay.ctrl);
  h->bk.counts = reinterpret_cast<uint32_t*>(base + lay.counts);
  h->bk.ovf_n = reinterpret_cast<uint32_t*>(base + lay.ovf_n);
  h->bk.slot = reinterpret_cast<uint32_t*>(base + lay.slot);
  h->bk.pos = reinterpret_cast<uint32_t*>(base + lay.pos);
  h->bk.td = reinterpret_cast<float*>(base + lay.td);
  h->bk.oslot = reinterpret_cast<uint32_t*>(base + lay.oslot);
  h->bk.opos = reinterpret_cast<uint32_t*>(base + lay.opos);
  h->bk.otd = reinterpret_cast<float*>(base + lay.otd);
  h->st.states = d_states;
  h->st.next_states = d_next_states;
  h->st.actions = d_actions;
  h->st.rewards = d_rewards;
  h->st.dones = d_dones;
  h->st.D = state_dim;
  h->size = 0;
  h->cursor = 0;
  h->epoch = 0;
  h->ovf = 0;
  h->ring = 0;
  h->top_stale = false;
  h->graph = false;
  h->sample_mode = 0;
  h->rank_attached = false;
  h->rank_size = 0;
  h->rank_built = -1;
  if (hipGetDevice(&h->device) != hipSuccess) h->device = -1;
  rc = resolve_static_scratch(h->device);
  if (rc) {
    delete h;
    return rc;
  }
  hipError_t e = per::launch_init(h->t, h->bk, h->g, stream);
  if (e != hipSuccess) {
    delete h;
    return hip_fail(e, "per_create: init launch");
  }
  *out = h;
  return ok();
}

int per_destroy(per_t* h) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  delete h;
  return ok();
}

namespace {

int check_add(const per_t* h, int64_t count, const float* d_states, const float* d_next_states,
              const uint32_t* d_actions, const float* d_rewards, const uint8_t* d_dones) {
  if (count < 0 || count > (int64_t)h->g.n)
    return fail(PER_EINVAL, "count %lld outside [0, capacity]", (long long)count);
  if (count > 0 && h->st.D > 0) {
    if (!(d_states && d_next_states && d_actions && d_rewards && d_dones))
      return fail(PER_EINVAL, "the handle has storage: all five row arrays are required");
    if ((reinterpret_cast<uintptr_t>(d_states) | reinterpret_cast<uintptr_t>(d_next_states)) &
        15u)
      return fail(PER_EINVAL, "state rows must be 16-byte aligned");
  }
  return PER_OK;
}

int check_update(const per_t* h, int64_t B, const int64_t* d_idx, const float* d_td) {
  if (B < 0 || B > h->max_batch)
    return fail(PER_EINVAL, "B %lld outside [0, max_batch=%lld]", (long long)B,
                (long long)h->max_batch);
  if (B > 0 && (!d_idx || !d_td)) return fail(PER_EINVAL, "idx and td are required");
  return PER_OK;
}

// Host state after an intake of count items was enqueued.
void advance_ring(per_t* h, int64_t count) {
  h->ring ^= 1;
  h->top_stale = h->g.P > 0;
  h->cursor = (h->cursor + count) % (int64_t)h->g.n;
  h->size = (h->size + count < (int64_t)h->g.n) ? h->size + count : (int64_t)h->g.n;
}

}  // namespace

int per_add(per_t* h, int64_t count, const float* d_states, const float* d_next_states,
            const uint32_t* d_actions, const float* d_rewards, const uint8_t* d_dones,
            const float* d_prio, hipStream_t stream) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  int rc = check_add(h, count, d_states, d_next_states, d_actions, d_rewards, d_dones);
  if (rc) return rc;
  if (count == 0) return ok();
  const int src = h->epoch, dst = d_prio ? (h->epoch ^ 1) : h->epoch;
  hipError_t e = per::launch_add(h->t, h->g, h->st, ring_ref(h), (uint32_t)h->size,
                                 (uint32_t)h->cursor, (uint32_t)count, d_states, d_next_states,
                                 d_actions, d_rewards, d_dones, d_prio, src, dst, stream);
  if (e != hipSuccess) return hip_fail(e, "per_add");
  h->epoch = dst;
  advance_ring(h, count);
  return ok();
}

int per_update(per_t* h, int64_t B, const int64_t* d_idx, const float* d_td,
               hipStream_t stream) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  int rc = check_update(h, B, d_idx, d_td);
  if (rc) return rc;
  if (B == 0) return ok();
  hipError_t e = per::launch_update(h->t, h->bk, h->g, ring_ref(h), (uint32_t)h->size, B, d_idx,
                                    d_td, h->alpha, h->eps, h->epoch, h->epoch ^ 1, h->ovf,
                                    stream);
  if (e != hipSuccess) return hip_fail(e, "per_update");
  h->epoch ^= 1;
  if (per::update_uses_buckets(h->g, B)) h->ovf ^= 1;
  h->top_stale = h->g.P > 0;
  return ok();
}

int per_update_static(per_t* h, int64_t B, const int64_t* d_idx, const float* d_td,
                      hipStream_t stream) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  int rc = check_update(h, B, d_idx, d_td);
  if (rc) return rc;
  if (B == 0) return ok();
  const int64_t np = int64_t(1) << h->g.P;
  const bool bucketed = per::update_uses_buckets(h->g, B);
  if (bucketed && (np > kStaticMaxParts || B > kStaticMaxBatch))
    return fail(PER_EINVAL,
                "per_update_static: a bucketed batch needs capacity <= 2^24 and B <= 2^16 "
                "(capacity %lld, B %lld)", (long long)h->g.n, (long long)B);
  if (h->device < 0 || h->device >= kMaxDevices || !g_scratch_ptr[h->device])
    return fail(PER_EHIP, "per_update_static: no static scratch on device %d", h->device);
  size_t end = 0;
  const per::Buckets sb =
      per::bucket_layout(static_cast<char*>(g_scratch_ptr[h->device]), (size_t)np,
                         kStaticMaxBatch, &end);
  if (end > kStaticScratchBytes)
    return fail(PER_EINVAL, "per_update_static: scratch layout exceeds the array");
  hipError_t e = hipSuccess;
  // The array keeps the previous call's counters (of any handle on this
  // device): clear them, then always use overflow counter 0.
  if (bucketed) e = per::launch_bucket_clear(sb, h->g, stream);
  if (e == hipSuccess)
    e = per::launch_update(h->t, sb, h->g, ring_ref(h), (uint32_t)h->size, B, d_idx, d_td,
                           h->alpha, h->eps, h->epoch, h->epoch ^ 1, 0, stream);
  if (e != hipSuccess) return hip_fail(e, "per_update_static");
  h->epoch ^= 1;
  h->top_stale = h->g.P > 0;
  return ok();
}

int per_update_add(per_t* h, int64_t B, const int64_t* d_idx, const float* d_td, int64_t count,
                   const float* d_states, const float* d_next_states, const uint32_t* d_actions,
                   const float* d_rewards, const uint8_t* d_dones, const float* d_prio,
                   hipStream_t stream) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  int rc = check_update(h, B, d_idx, d_td);
  if (rc) return rc;
  rc = check_add(h, count, d_states, d_next_states, d_actions, d_rewards, d_dones);
  if (rc) return rc;
  if (count == 0) return per_update(h, B, d_idx, d_td, stream);
  if (B == 0 || per::update_uses_buckets(h->g, B)) {
    // Nothing to fuse, or a batch large enough for the bucketed update: the
    // two calls, one after the other (both checked above, so neither fails
    // on its arguments).
    rc = per_update(h, B, d_idx, d_td, stream);
    if (rc) return rc;
    return per_add(h, count, d_states, d_next_states, d_actions, d_rewards, d_dones, d_prio,
                   stream);
  }
  const int src = h->epoch, dst = h->epoch ^ 1;
  hipError_t e = per::launch_update_add(h->t, h->g, h->st, ring_ref(h), (uint32_t)h->size,
                                        (uint32_t)h->cursor, B, d_idx, d_td, h->alpha, h->eps,
                                        (uint32_t)count, d_states, d_next_states, d_actions,
                                        d_rewards, d_dones, d_prio, src, dst, stream);
  if (e != hipSuccess) return hip_fail(e, "per_update_add");
  h->epoch = dst;
  advance_ring(h, count);
  return ok();
}

namespace {

enum SampleKind { kGivenMasses, kStreamMasses, kUniform, kRank };

// Shared by the sample entry points: masses given (d_u), drawn from the
// generator stream (seed, offset), or a uniform sample from the stream;
// out_stride floats per output state row (>= state_dim), dones as u8 or f32.
int sample_impl(per_t* h, int64_t B, SampleKind kind, const float* d_u, uint64_t seed,
                uint64_t offset, double beta, int64_t* d_idx_out, float* d_w_out,
                float* d_states_out, float* d_next_states_out, int64_t out_stride,
                uint32_t* d_actions_out, float* d_rewards_out, void* d_dones_out, bool dones_f32,
                hipStream_t stream, const char* what) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  if (B < 0 || B > h->max_batch)
    return fail(PER_EINVAL, "B %lld outside [0, max_batch=%lld]", (long long)B,
                (long long)h->max_batch);
  if (out_stride < h->st.D || out_stride > PER_MAX_OUT_STRIDE)
    return fail(PER_EINVAL, "out_stride %lld outside [state_dim=%d, %lld]", (long long)out_stride,
                (int)h->st.D, (long long)PER_MAX_OUT_STRIDE);
  if (B == 0) return ok();
  if (!d_idx_out) return fail(PER_EINVAL, "idx_out is required");
  if ((kind == kGivenMasses || kind == kRank) && !d_u) return fail(PER_EINVAL, "u is required");
  if (!(beta >= 0.0) || !(beta < 1e300)) return fail(PER_EINVAL, "beta must be finite, >= 0");
  const bool any_rows = d_states_out || d_next_states_out || d_actions_out || d_rewards_out ||
                        d_dones_out;
  const bool all_rows = d_states_out && d_next_states_out && d_actions_out && d_rewards_out &&
                        d_dones_out;
  if (any_rows && !all_rows) return fail(PER_EINVAL, "row outputs go all together");
  if (any_rows && h->st.D == 0) return fail(PER_EINVAL, "the handle keeps no rows");
  if (any_rows && ((reinterpret_cast<uintptr_t>(d_states_out) |
                    reinterpret_cast<uintptr_t>(d_next_states_out)) & 15u))
    return fail(PER_EINVAL, "state outputs must be 16-byte aligned");
  if (h->size == 0) return fail(PER_EEMPTY, "sample from an empty buffer");
  if (kind == kRank) {
    if (h->rank_size == 0) return fail(PER_EEMPTY, "rank sample before per_rank_refresh");
    const per::SamplePlan plan =
        per::make_sample_plan(h->g, B, any_rows ? (uint32_t)h->st.D : 0u, h->sample_mode);
    hipError_t e = per::launch_sample(h->rt, h->g, h->st, plan, (uint32_t)h->rank_size, B, d_u,
                                      0, 0, beta, d_idx_out, d_w_out,
                                      any_rows ? d_states_out : nullptr, d_next_states_out,
                                      d_actions_out, d_rewards_out, d_dones_out,
                                      (uint32_t)out_stride, dones_f32, stream,
                                      h->rvals[0]);
    return e == hipSuccess ? ok() : hip_fail(e, what);
  }
  if (kind == kUniform) {
    hipError_t e = per::launch_uniform(h->st, h->t.ctrl, ring_ref(h), (uint32_t)h->size, B, seed,
                                       offset, d_idx_out, any_rows ? d_states_out : nullptr,
                                       d_next_states_out,
                                       d_actions_out, d_rewards_out, d_dones_out,
                                       (uint32_t)out_stride, dones_f32, stream);
    return e == hipSuccess ? ok() : hip_fail(e, what);
  }
  const per::SamplePlan plan =
      per::make_sample_plan(h->g, B, any_rows ? (uint32_t)h->st.D : 0u, h->sample_mode);
  const bool stale = top_may_be_stale(h);
  if (stale && plan.top_mode != per::kTopRebuild) {  // the sampler will not rebuild the top itself
    hipError_t e = per::launch_top(h->t, h->g, stream);
    if (e != hipSuccess) return hip_fail(e, "per_sample: top rebuild");
    h->top_stale = false;
  }
  hipError_t e = per::launch_sample(h->t, h->g, h->st, plan, (uint32_t)h->size, B,
                                    kind == kGivenMasses ? d_u : nullptr, seed, offset, beta,
                                    d_idx_out, d_w_out, any_rows ? d_states_out : nullptr,
                                    d_next_states_out, d_actions_out, d_rewards_out,
                                    d_dones_out, (uint32_t)out_stride, dones_f32, stream);
  if (e != hipSuccess) return hip_fail(e, what);
  // A rebuilding sampler keeps its top in LDS: the stored top stays pending
  // until per_flush (or a sampler that reads it from memory) rebuilds it.
  return ok();
}

}  // namespace

int per_sample(per_t* h, int64_t B, const float* d_u, double beta, int64_t* d_idx_out,
               float* d_w_out, float* d_states_out, float* d_next_states_out,
               uint32_t* d_actions_out, float* d_rewards_out, uint8_t* d_dones_out,
               hipStream_t stream) {
  return sample_impl(h, B, kGivenMasses, d_u, 0, 0, beta, d_idx_out, d_w_out, d_states_out,
                     d_next_states_out, h ? h->st.D : 0, d_actions_out, d_rewards_out,
                     d_dones_out, false, stream, "per_sample");
}

int per_sample_philox(per_t* h, int64_t B, uint64_t seed, uint64_t offset, double beta,
                      int64_t* d_idx_out, float* d_w_out, float* d_states_out,
                      float* d_next_states_out, uint32_t* d_actions_out, float* d_rewards_out,
                      uint8_t* d_dones_out, hipStream_t stream) {
  return sample_impl(h, B, kStreamMasses, nullptr, seed, offset, beta, d_idx_out, d_w_out,
                     d_states_out, d_next_states_out, h ? h->st.D : 0, d_actions_out,
                     d_rewards_out, d_dones_out, false, stream, "per_sample_philox");
}

int per_sample_uniform(per_t* h, int64_t B, uint64_t seed, uint64_t offset, int64_t* d_idx_out,
                       float* d_states_out, float* d_next_states_out, uint32_t* d_actions_out,
                       float* d_rewards_out, uint8_t* d_dones_out, hipStream_t stream) {
  return sample_impl(h, B, kUniform, nullptr, seed, offset, 0.0, d_idx_out, nullptr, d_states_out,
                     d_next_states_out, h ? h->st.D : 0, d_actions_out, d_rewards_out,
                     d_dones_out, false, stream, "per_sample_uniform");
}

int per_sample_padded(per_t* h, int64_t B, const float* d_u, double beta, int64_t* d_idx_out,
                      float* d_w_out, float* d_states_out, float* d_next_states_out,
                      int64_t out_stride, int32_t* d_actions_out, float* d_rewards_out,
                      float* d_dones_out, hipStream_t stream) {
  return sample_impl(h, B, kGivenMasses, d_u, 0, 0, beta, d_idx_out, d_w_out, d_states_out,
                     d_next_states_out, out_stride, reinterpret_cast<uint32_t*>(d_actions_out),
                     d_rewards_out, d_dones_out, true, stream, "per_sample_padded");
}

static int copy_scalar(per_t* h, const void* src, float* d_out, hipStream_t stream,
                       const char* what) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  if (!d_out) return fail(PER_EINVAL, "out is NULL");
  hipError_t e = hipMemcpyAsync(d_out, src, sizeof(float), hipMemcpyDeviceToDevice, stream);
  if (e != hipSuccess) return hip_fail(e, what);
  return ok();
}

int per_flush(per_t* h, hipStream_t stream) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  if (top_may_be_stale(h)) {
    hipError_t e = per::launch_top(h->t, h->g, stream);
    if (e != hipSuccess) return hip_fail(e, "per_flush");
    h->top_stale = false;
  }
  return ok();
}

int per_total(per_t* h, float* d_out, hipStream_t stream) {
  if (!h || !d_out) return fail(PER_EINVAL, "NULL argument");
  int rc = per_flush(h, stream);
  if (rc) return rc;
  return copy_scalar(h, h->t.sum + 1, d_out, stream, "per_total");
}

int per_min(per_t* h, float* d_out, hipStream_t stream) {
  if (!h || !d_out) return fail(PER_EINVAL, "NULL argument");
  int rc = per_flush(h, stream);
  if (rc) return rc;
  return copy_scalar(h, h->t.mn + 1, d_out, stream, "per_min");
}

int per_max_priority(per_t* h, float* d_out, hipStream_t stream) {
  if (!h || !d_out) return fail(PER_EINVAL, "NULL argument");
  return copy_scalar(h, &h->t.ctrl->maxp_bits[h->epoch], d_out, stream, "per_max_priority");
}

int per_graph_mode(per_t* h, int32_t on, hipStream_t stream) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  if (on) {
    if (h->graph) return fail(PER_EINVAL, "already in graph mode");
    h->graph = true;
    h->entry_epoch = h->epoch;
    h->entry_ovf = h->ovf;
    h->entry_ring = h->ring;
    return ok();
  }
  if (!h->graph) return fail(PER_EINVAL, "not in graph mode");
  // Replays have moved the ring on the device: take its state back.
  per::Ctrl c;
  hipError_t e = hipMemcpyAsync(&c, h->t.ctrl, sizeof c, hipMemcpyDeviceToHost, stream);
  if (e == hipSuccess) e = hipStreamSynchronize(stream);
  if (e != hipSuccess) return hip_fail(e, "per_graph_mode: ring state");
  h->cursor = c.cursor[h->ring];
  h->size = c.size[h->ring];
  h->graph = false;
  h->top_stale = h->g.P > 0;
  if (h->epoch != h->entry_epoch || h->ovf != h->entry_ovf || h->ring != h->entry_ring)
    return fail(PER_EINVAL,
                "the calls made in graph mode flip a slot parity an odd number of times "
                "(running max %d, overflow %d, ring %d): replaying them reads stale slots",
                h->epoch ^ h->entry_epoch, h->ovf ^ h->entry_ovf, h->ring ^ h->entry_ring);
  return ok();
}

int per_set_sample_lanes(per_t* h, int32_t lanes) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  int mode;
  switch (lanes) {
    case 0: mode = 0; break;
    case 64: mode = 1; break;
    case 16: mode = 2; break;
    case 1: mode = 3; break;
    default: return fail(PER_EINVAL, "lanes per sample must be 0, 1, 16 or 64 (got %d)", lanes);
  }
  h->sample_mode = mode;
  return ok();
}

int per_time_next(hipEvent_t start, hipEvent_t stop) {
  g_last_error.clear();
  g_timing.start = start;
  g_timing.stop = stop;
  return PER_OK;
}

int64_t per_size(const per_t* h) { return h ? h->size : -1; }
int64_t per_cursor(const per_t* h) { return h ? h->cursor : -1; }
int64_t per_capacity(const per_t* h) { return h ? (int64_t)h->g.n : -1; }
int32_t per_state_dim(const per_t* h) { return h ? h->st.D : -1; }

namespace {

struct RankLayout {
  size_t rsum, rmn, keys0, keys1, vals0, vals1, hist, total;
};

RankLayout rank_layout(int64_t n) {
  RankLayout l;
  size_t o = 0;
  auto take = [&](size_t bytes) {
    const size_t at = o;
    o = align256(o + bytes);
    return at;
  };
  l.rsum = take(sizeof(float) * 2 * (size_t)n);
  l.rmn = take(sizeof(float) * 2 * (size_t)n);
  l.keys0 = take(sizeof(uint32_t) * (size_t)n);
  l.keys1 = take(sizeof(uint32_t) * (size_t)n);
  l.vals0 = take(sizeof(uint32_t) * (size_t)n);
  l.vals1 = take(sizeof(uint32_t) * (size_t)n);
  l.hist = take(sizeof(uint32_t) * per::rank_hist_words(n));
  l.total = o;
  return l;
}

}  // namespace

int per_rank_workspace_bytes(int64_t capacity, size_t* out) {
  if (!out) return fail(PER_EINVAL, "out is NULL");
  int rc = check_capacity(capacity);
  if (rc) return rc;
  *out = rank_layout(capacity).total;
  return ok();
}

int per_rank_attach(per_t* h, void* d_ws, size_t ws_bytes) {
  if (!h || !d_ws) return fail(PER_EINVAL, "NULL argument");
  if (reinterpret_cast<uintptr_t>(d_ws) & 255u)
    return fail(PER_EINVAL, "rank workspace is not 256-byte aligned");
  const RankLayout l = rank_layout(h->g.n);
  if (ws_bytes < l.total)
    return fail(PER_ENOSPC, "rank workspace of %zu bytes, %zu needed", ws_bytes, l.total);
  char* base = static_cast<char*>(d_ws);
  h->rt.sum = reinterpret_cast<float*>(base + l.rsum);
  h->rt.mn = reinterpret_cast<float*>(base + l.rmn);
  h->rt.ctrl = nullptr;
  h->rkeys[0] = reinterpret_cast<uint32_t*>(base + l.keys0);
  h->rkeys[1] = reinterpret_cast<uint32_t*>(base + l.keys1);
  h->rvals[0] = reinterpret_cast<uint32_t*>(base + l.vals0);
  h->rvals[1] = reinterpret_cast<uint32_t*>(base + l.vals1);
  h->rhist = reinterpret_cast<uint32_t*>(base + l.hist);
  h->rank_attached = true;
  h->rank_size = 0;
  h->rank_built = -1;
  return ok();
}

int per_rank_refresh(per_t* h, hipStream_t stream) {
  if (!h) return fail(PER_EINVAL, "handle is NULL");
  if (h->graph) return fail(PER_EINVAL, "per_rank_refresh needs the ring size: leave graph mode");
  if (!h->rank_attached) return fail(PER_EINVAL, "no rank workspace: call per_rank_attach");
  if (h->size == 0) return fail(PER_EEMPTY, "ranking an empty buffer");
  hipError_t e = per::launch_rank_sort(h->t.sum + h->g.n, (uint32_t)h->size, h->rkeys, h->rvals,
                                       h->rhist, stream);
  if (e != hipSuccess) return hip_fail(e, "per_rank_refresh: sort");
  if (h->rank_built != h->size) {
    e = per::launch_rank_build(h->rt, h->g, (uint32_t)h->size, h->alpha, stream);
    if (e != hipSuccess) return hip_fail(e, "per_rank_refresh: rank weights");
    h->rank_built = h->size;
  }
  h->rank_size = h->size;
  return ok();
}

int per_sample_rank(per_t* h, int64_t B, const float* d_u, double beta, int64_t* d_idx_out,
                    float* d_w_out, float* d_states_out, float* d_next_states_out,
                    uint32_t* d_actions_out, float* d_rewards_out, uint8_t* d_dones_out,
                    hipStream_t stream) {
  return sample_impl(h, B, kRank, d_u, 0, 0, beta, d_idx_out, d_w_out, d_states_out,
                     d_next_states_out, h ? h->st.D : 0, d_actions_out, d_rewards_out,
                     d_dones_out, false, stream, "per_sample_rank");
}

int per_rank_ptrs(const per_t* h, const uint32_t** d_order, const float** d_rank_sum,
                  const float** d_rank_min) {
  if (!h || !d_order || !d_rank_sum || !d_rank_min) return fail(PER_EINVAL, "NULL argument");
  if (!h->rank_attached) return fail(PER_EINVAL, "no rank workspace: call per_rank_attach");
  *d_order = h->rvals[0];
  *d_rank_sum = h->rt.sum;
  *d_rank_min = h->rt.mn;
  return ok();
}

int per_tree_ptrs(const per_t* h, const float** d_sum, const float** d_min) {
  if (!h || !d_sum || !d_min) return fail(PER_EINVAL, "NULL argument");
  *d_sum = h->t.sum;
  *d_min = h->t.mn;
  return ok();
}

const char* per_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
