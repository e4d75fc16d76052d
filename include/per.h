/*
 * per.h -- C ABI of the MI355X (gfx950) prioritized-replay sum tree.
 *
 * A flat implicit sum tree and a twin min tree over 2n f32 nodes ("Putting
 * prioritized replay's segment tree on a GPU", section "The Tree Under Every
 * Prioritized Replay": leaves at [n, 2n), node i has children 2i and 2i+1,
 * internal nodes hold the sum -- or, in the twin tree, the min -- of their
 * children, the root at index 1), plus ring storage of transitions
 * ("GPU-Resident Prioritized Experience Replay", section "Architecture").
 *
 * Conventions shared by every entry point
 *  - Pointers prefixed d_ are device pointers (HBM of the device the handle
 *    was created on).  Every device buffer is owned by the caller; the
 *    library never allocates or frees device memory.
 *  - Work is enqueued on the caller's stream and is ordered by it; no entry
 *    point synchronises the host with the device, except per_graph_mode
 *    when it leaves graph mode.  Inputs must stay alive and unchanged, and
 *    outputs untouched, until the stream has passed the call.
 *  - Host-side checks happen before anything is enqueued: on an error return
 *    nothing was enqueued and the handle is unchanged.
 *  - A handle may be used from one host thread at a time, and calls on one
 *    handle must go to streams that are ordered with respect to each other.
 *  - Return codes: PER_OK, or a negative PER_E* code; per_last_error() then
 *    describes the failure (text is per host thread).
 *  - Numerics: every f32 tree node is recomputed as the round-to-nearest f32
 *    sum (min) of its two children, never by adding a delta, so the trees are
 *    a pure function of the leaves; no flush-to-zero, no fused multiply-add.
 */
#ifndef PER_H
#define PER_H

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define PER_OK 0
#define PER_EINVAL (-1) /* an argument is out of range or a required pointer is NULL */
#define PER_ENOSPC (-2) /* the workspace is smaller than per_workspace_bytes() */
#define PER_EEMPTY (-3) /* sampling from a buffer that holds no transition */
#define PER_EHIP (-4)   /* the HIP runtime reported an error (see per_last_error) */

#define PER_MAX_CAPACITY (1LL << 30)
#define PER_MAX_BATCH (1LL << 24)
#define PER_MAX_OUT_STRIDE (1LL << 20)

typedef struct per_s per_t;

/*
 * Bytes of device workspace a handle needs: both trees (2 x 2n f32), a small
 * control block (running max priority, completion counters) and the scratch
 * the batched update uses for batches of up to max_batch entries.
 * capacity: number of leaves, a power of two in [2, PER_MAX_CAPACITY].
 * max_batch: largest B later passed to per_update / per_sample, in
 * [1, PER_MAX_BATCH].  Writes *out and returns PER_OK, or PER_EINVAL.
 */
int per_workspace_bytes(int64_t capacity, int64_t max_batch, size_t* out);

/*
 * Creates a handle over caller-owned memory and enqueues the initialisation
 * of the trees on `stream`: every sum node 0, every min node +inf (the
 * neutral elements, so empty slots never count), running max priority 1.0;
 * size = cursor = 0.
 *  d_ws / ws_bytes: device workspace, 256-byte aligned, at least
 *    per_workspace_bytes(capacity, max_batch) bytes (else PER_ENOSPC).
 *  alpha, eps: priority exponent and offset, p = (|td| + eps)^alpha
 *    ("GPU-Resident Prioritized Experience Replay", section "Priority
 *    update"); alpha > 0, eps >= 0, both finite.
 *  state_dim: floats per state row, >= 0.  With state_dim > 0 the five
 *    storage arrays (section "Architecture" of the same page) must all be
 *    given: d_states and d_next_states [capacity x state_dim] f32 row-major,
 *    16-byte aligned; d_actions [capacity] u32; d_rewards [capacity] f32;
 *    d_dones [capacity] u8.  With state_dim == 0 they must all be NULL and the
 *    handle keeps priorities only.  The storage must outlive the handle.
 * On success *out receives the handle (free with per_destroy).
 */
int per_create(per_t** out, int64_t capacity, int32_t state_dim, int64_t max_batch,
               double alpha, double eps, void* d_ws, size_t ws_bytes, float* d_states,
               float* d_next_states, uint32_t* d_actions, float* d_rewards,
               uint8_t* d_dones, hipStream_t stream);

/* Frees the host-side handle only (no device work, no synchronisation). */
int per_destroy(per_t* h);

/*
 * Ring intake ("GPU-Resident Prioritized Experience Replay", section
 * "Experience Insertion"; overflow overwrites the oldest slots, section
 * "Error Handling & Fallback").  Transition j of the call goes to slot
 * (cursor + j) mod capacity; afterwards cursor = (cursor + count) mod
 * capacity and size = min(size + count, capacity).
 *  count in [0, capacity] (0 enqueues nothing).
 *  Rows: d_states / d_next_states [count x state_dim] f32 (16-byte aligned),
 *    d_actions / d_rewards / d_dones [count]; required when the handle has
 *    storage, ignored otherwise.
 *  d_prio: [count] f32 priorities, finite and >= 0 (-0.0 is stored as +0.0;
 *    not checked on the device).  NULL gives every new slot the running max
 *    priority (the new items' priority at the time the stream runs the call).
 *    Given priorities raise the running max to their maximum.
 */
int per_add(per_t* h, int64_t count, const float* d_states, const float* d_next_states,
            const uint32_t* d_actions, const float* d_rewards, const uint8_t* d_dones,
            const float* d_prio, hipStream_t stream);

/*
 * Batched priority update ("GPU-Resident Prioritized Experience Replay",
 * sections "Priority update" and "Error Handling & Fallback"; the batch
 * update of "Putting prioritized replay's segment tree on a GPU", section
 * "Second Port: Make the Update GPU-Shaped", with the level-synchronous
 * dependency rule of section "The Race Condition Worth Writing Down").
 *  B in [0, max_batch]; d_idx [B] i64 slot indices; d_td [B] f32 TD errors.
 * The result equals applying the entries one by one in batch order: for a
 * slot repeated in the batch the last position wins.  Entry b sets slot
 * d_idx[b] to p = f32(pow_f64(|td| + eps, alpha)); NaN td gives the td = 0
 * value and +/-Inf td the running max priority as of the start of the call.
 * Indices outside [0, size) are skipped (defined, not an error).  The
 * running max priority becomes the max of itself and every p of the call.
 */
int per_update(per_t* h, int64_t B, const int64_t* d_idx, const float* d_td,
               hipStream_t stream);

/*
 * per_update for callers that cannot allocate device memory at the call:
 * code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation.  Same arguments, result and errors as per_update.  A batch
 * that takes the bucketed update (more than 2^21 / 2^P entries, 2^P =
 * capacity / 4096 partitions) keeps its buckets, overflow list and counters
 * in a static device array of the library (5 MiB, one per device, held until
 * the process ends) instead of in the handle's workspace; the call clears
 * its counters first with a small kernel.  Limits of that array: capacity
 * <= 2^24 and B <= 2^16 for a bucketed batch, else PER_EINVAL; smaller
 * batches need no scratch and take any size per_update takes.  The call
 * allocates nothing and launches no allocating routine.  Every handle on a
 * device shares the one array: per_update_static calls that may overlap on
 * one device (on different streams or from different host threads) race on
 * it and must be ordered by the caller.
 */
int per_update_static(per_t* h, int64_t B, const int64_t* d_idx, const float* d_td,
                      hipStream_t stream);

/*
 * per_update(h, B, d_idx, d_td) followed by per_add(h, count, rows..., d_prio)
 * in one kernel launch where possible ("Putting prioritized replay's segment
 * tree on a GPU", section "The Tree Under Every Prioritized Replay": the
 * replay rank takes a priority update for every learner batch plus intake
 * batches from the actors; "True Single-Graph Implementation Plan", its
 * goal: fewer launches per step).  The result -- trees, running max, ring
 * state, stored rows -- is that of the two calls in that order: the intake
 * overwrites slots the update just set, and NULL d_prio gives the new slots
 * the running max after the update.  Arguments and errors as for the two
 * calls, all checked before anything is enqueued.  B == 0 or count == 0
 * reduces to the other call; a batch large enough for the bucketed update
 * (more than 2^21 / 2^P entries, 2^P = capacity / 4096 partitions) is
 * enqueued as the two calls.
 */
int per_update_add(per_t* h, int64_t B, const int64_t* d_idx, const float* d_td, int64_t count,
                   const float* d_states, const float* d_next_states, const uint32_t* d_actions,
                   const float* d_rewards, const uint8_t* d_dones, const float* d_prio,
                   hipStream_t stream);

/*
 * Batched proportional sample ("Putting prioritized replay's segment tree on a
 * GPU", section "Sampling Is a Descent"; importance weights and gather,
 * "GPU-Resident Prioritized Experience Replay", section "Sampling Kernels";
 * writing straight into caller buffers, "True Single-Graph Implementation
 * Plan", Task 3).
 *  B in [0, max_batch]; PER_EEMPTY if size == 0 (checked on the host).
 *  d_u [B] f32 uniforms in [0, 1) (unchecked).  Sample b uses the mass
 *    m = f32(u_b * total), clamped below total, and picks one child per
 *    level from the root: the right one when the left child's sum is at
 *    most m and the right child's sum is not 0 (then m = f32(m - left sum)),
 *    else the left one.
 *  d_idx_out [B] i64: sampled slots (required).
 *  d_w_out [B] f32 or NULL: w_b = (N*P_b)^-beta / (N*P_min)^-beta, N = size,
 *    P_b = p_b / total, P_min = min-tree root / total, i.e. (p_b / p_min)^-beta;
 *    0 when the min priority is 0.  For 0 <= beta <= 1 and normal priorities
 *    it is taken from the exact exponent difference, f32 logarithms of the
 *    significands and an f32 power of two, within 3e-7 relative of the f64
 *    value rounded to f32; otherwise the f32 of the f64 power.
 *  Row outputs (all NULL, or all given when the handle has storage):
 *    d_states_out / d_next_states_out [B x state_dim] f32 (16-byte aligned),
 *    d_actions_out [B] u32, d_rewards_out [B] f32, d_dones_out [B] u8: byte
 *    copies of the sampled slots.
 * Preconditions (unchecked): total finite and > 0.
 */
int per_sample(per_t* h, int64_t B, const float* d_u, double beta, int64_t* d_idx_out,
               float* d_w_out, float* d_states_out, float* d_next_states_out,
               uint32_t* d_actions_out, float* d_rewards_out, uint8_t* d_dones_out,
               hipStream_t stream);

/*
 * per_sample with the masses drawn on the device ("GPU-Resident Prioritized
 * Experience Replay", section "Sampling Kernels": the uniform values come
 * from a generator on the GPU, not from the host).  The generator is
 * Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
 * As Easy as 1, 2, 3", SC 2011); word j of the stream of a seed is word
 * j % 4 of the block at counter (j / 4, 0, 0, 0) under key (seed, 0).
 * Sample b uses u_b = (word(offset + b) >> 40) * 2^-24, i.e. a 24-bit
 * uniform in [0, 1); everything else is per_sample with d_u = those u_b.
 * The caller advances offset (by B per call for fresh masses).
 */
int per_sample_philox(per_t* h, int64_t B, uint64_t seed, uint64_t offset, double beta,
                      int64_t* d_idx_out, float* d_w_out, float* d_states_out,
                      float* d_next_states_out, uint32_t* d_actions_out, float* d_rewards_out,
                      uint8_t* d_dones_out, hipStream_t stream);

/*
 * Uniform sample over the filled slots, for prioritisation switched off
 * ("GPU-Resident Prioritized Experience Replay", section "Experience
 * Insertion": the same ring sampled uniformly from generated indices into
 * [0, size)).  Slot b = ((word(offset + b) >> 32) * size) >> 32 with the
 * stream of per_sample_philox; no weights (all equal).  Row outputs and
 * errors as per_sample.
 */
int per_sample_uniform(per_t* h, int64_t B, uint64_t seed, uint64_t offset, int64_t* d_idx_out,
                       float* d_states_out, float* d_next_states_out, uint32_t* d_actions_out,
                       float* d_rewards_out, uint8_t* d_dones_out, hipStream_t stream);

/*
 * Rank-based prioritisation ("GPU-Resident Prioritized Experience Replay",
 * section "Sampling Kernels", rank-based: the (priority, index) pairs sorted
 * descending, then sampling with probabilities 1/rank^alpha through their
 * cumulative sum, gather and IS weights).
 *
 * per_rank_workspace_bytes: bytes of the extra device workspace a handle of
 *   this capacity needs for it (the trees over the rank weights, 2 x 2 x
 *   capacity f32; the sort's buffers, 4 x capacity u32; its tile counts).
 * per_rank_attach: hands that workspace (caller-owned, 256-byte aligned,
 *   kept until per_destroy) to the handle.  PER_ENOSPC if too small.
 * per_rank_refresh: ranks the filled slots [0, size) by descending leaf
 *   priority, equal priorities by ascending slot (stable radix sort), and,
 *   when size changed since the last refresh, rebuilds the trees over the
 *   rank weights w_r = f32(pow_f64(r + 1, -alpha)) for ranks r < size (sum 0
 *   / min +inf beyond), with the pairwise rules of the priority trees.
 *   Later per_update / per_add calls do not change the ranking until the
 *   next refresh.  PER_EEMPTY if size == 0; PER_EINVAL without a workspace.
 * per_sample_rank: per_sample over the rank-weight trees as of the last
 *   refresh: the descent on mass f32(u_b * W), W = the sum of the rank
 *   weights, gives a rank r, and the sample is the slot of rank r; the IS
 *   weight is per_sample's with the rank weights as priorities and N = the
 *   size at the refresh.  Arguments, row outputs and errors as per_sample;
 *   PER_EEMPTY before the first refresh.
 * per_rank_ptrs: read-only device views for inspection: the ranking
 *   (d_order[r] = slot of rank r, r < size at the refresh) and the two
 *   rank-weight trees (2 x capacity f32 each, node 0 unused).
 */
int per_rank_workspace_bytes(int64_t capacity, size_t* out);
int per_rank_attach(per_t* h, void* d_ws, size_t ws_bytes);
int per_rank_refresh(per_t* h, hipStream_t stream);
int per_sample_rank(per_t* h, int64_t B, const float* d_u, double beta, int64_t* d_idx_out,
                    float* d_w_out, float* d_states_out, float* d_next_states_out,
                    uint32_t* d_actions_out, float* d_rewards_out, uint8_t* d_dones_out,
                    hipStream_t stream);
int per_rank_ptrs(const per_t* h, const uint32_t** d_order, const float** d_rank_sum,
                  const float** d_rank_min);

/*
 * per_sample written straight into a trainer's input buffers ("True
 * Single-Graph Implementation Plan", Task 2: rows gathered into a padded
 * destination, scalars gathered as f32 / i32; Task 3: the sampler writes the
 * trainer's buffers directly).  Same masses, descent, indices and weights
 * as per_sample.  Differences, all in the row outputs:
 *  out_stride: floats per output state row, in [state_dim,
 *    PER_MAX_OUT_STRIDE] (else PER_EINVAL); d_states_out / d_next_states_out
 *    are [B x out_stride] f32 (16-byte aligned): columns [0, state_dim) hold
 *    the stored row, columns [state_dim, out_stride) are written as +0.0.
 *  d_actions_out [B] i32: the stored 32 bits of the action.
 *  d_dones_out [B] f32: the stored done byte's value (0.0 or 1.0 for 0 / 1).
 * Row outputs all NULL (then out_stride is only range-checked) or all given
 * when the handle has storage.  Errors as per_sample.
 */
int per_sample_padded(per_t* h, int64_t B, const float* d_u, double beta, int64_t* d_idx_out,
                      float* d_w_out, float* d_states_out, float* d_next_states_out,
                      int64_t out_stride, int32_t* d_actions_out, float* d_rewards_out,
                      float* d_dones_out, hipStream_t stream);

/*
 * Lanes that carry one sample through the descent: 64 (one wave per
 * sample), 16 (four samples per wave) or 1 (one lane per sample); 0, the
 * default, lets the library choose by batch size and row width.  Every
 * layout computes the same indices, weights and rows ("Putting prioritized
 * replay's segment tree on a GPU", section "Sampling Is a Descent": each
 * descent is independent of the others); the choice only changes how the
 * batch spreads over the chip.  Applies to the handle's later sampling
 * calls.  PER_EINVAL for any other value.
 */
int per_set_sample_lanes(per_t* h, int32_t lanes);

/*
 * Device-side timing of one call ("Putting prioritized replay's segment
 * tree on a GPU", section "Measuring the Trade Honestly": each operation
 * timed on its own).  The next entry point called on this host thread that
 * enqueues kernels records `start` (if not NULL) as its first kernel begins
 * and `stop` (if not NULL) as its last kernel ends, through
 * hipExtLaunchKernel; hipEventElapsedTime(start, stop) then gives the span
 * of the call's kernels on the device without the dispatch gap before the
 * first one.  The request is dropped when that call returns, whatever it
 * returns.  The events must be created by the caller; do not request timing
 * for a call issued into a stream under graph capture.  Returns PER_OK.
 */
int per_time_next(hipEvent_t start, hipEvent_t stop);

/*
 * The nodes above the update partitions (the top levels of both trees,
 * "Putting prioritized replay's segment tree on a GPU", section "The Tree
 * Under Every Prioritized Replay": every internal node is the sum -- or
 * min -- of its two children) are rebuilt lazily: per_add and per_update
 * leave them stale, and per_sample rebuilds them in on-chip memory for its
 * own descent without storing them (on trees too deep for that it stores
 * them first).  per_flush enqueues the rebuild of the stored top now if it
 * is pending (one small kernel; a no-op otherwise), so that the arrays of
 * per_tree_ptrs hold every node.  per_total and per_min call it themselves.
 */
int per_flush(per_t* h, hipStream_t stream);

/*
 * Enqueue a 4-byte device copy of the sum-tree root (total priority), the
 * min-tree root (min priority over written slots; +inf when empty) or the
 * running max priority into d_out.  The caller synchronises to read it.
 * The two roots are node 1 of the flat trees ("Putting prioritized replay's
 * segment tree on a GPU", section "The Tree Under Every Prioritized Replay":
 * the root holds the total that masses are drawn from, and the twin min
 * tree gives the smallest priority for the importance-weight
 * normalisation); the running max priority is what new transitions enter
 * with ("GPU-Resident Prioritized Experience Replay", section "Experience
 * Insertion").  per_total and per_min flush the top levels first.
 */
int per_total(per_t* h, float* d_out, hipStream_t stream);
int per_min(per_t* h, float* d_out, hipStream_t stream);
int per_max_priority(per_t* h, float* d_out, hipStream_t stream);

/*
 * Graph mode ("True Single-Graph Implementation Plan", its goal and
 * architecture: one graph launch per training step, with counters kept on
 * the GPU instead of written by the host; "H100 GPU Pipeline Optimization
 * Design", section 2, CUDA Graph for experience collection: a captured loop
 * reads the replay buffer's changing size through the device; "GPU-Resident
 * Prioritized Experience Replay", section "Approach": no CPU involvement per
 * training step).
 *
 * per_graph_mode(h, 1, s) makes the calls that follow capturable and
 * replayable: per_add, per_update and per_sample_uniform read the ring's
 * cursor and filled size from the device control block (every per_add
 * writes the next state there, in either mode), and every sampling call
 * rebuilds the nodes above the partitions instead of trusting the host's
 * record of whether they are current.  Nothing is enqueued and nothing waits.
 *
 * Replay rule: the device keeps the running max, the bucketed update's
 * overflow list and the ring state in two slots each, and a call reads one
 * slot and writes the other, chosen on the host when it is issued.  A
 * captured sequence therefore replays correctly only if it flips each of
 * these slot parities an even number of times, so that each replay starts
 * on the slots the capture started on.  One training step (per_add with
 * running-max priorities, a sample, per_update) flips the running-max and
 * ring parities once each: capture two steps.  Random-number offsets of
 * per_sample_philox / per_sample_uniform are fixed at capture time.
 * per_rank_refresh fails in graph mode; per_size / per_cursor report the
 * host's count of the calls issued, which replays do not advance.
 *
 * per_graph_mode(h, 0, s) leaves graph mode: it waits for stream s, copies
 * the ring state back from the device (so per_size / per_cursor count every
 * replay) and marks the top levels stale.  It returns PER_EINVAL if the
 * calls issued in graph mode broke the replay rule (the handle has left
 * graph mode all the same), and PER_EHIP if the copy fails.  Entering twice
 * or leaving when not in graph mode is PER_EINVAL.  Never call it while s is
 * being captured.
 */
int per_graph_mode(per_t* h, int32_t on, hipStream_t stream);

/* Host-side state: number of written slots, next slot to write, capacity,
 * floats per state row.  -1 for a NULL handle. */
int64_t per_size(const per_t* h);
int64_t per_cursor(const per_t* h);
int64_t per_capacity(const per_t* h);
int32_t per_state_dim(const per_t* h);

/* Read-only device pointers to the two [2 x capacity] f32 trees (index 0
 * unused), for inspection after the stream has passed per_flush. */
int per_tree_ptrs(const per_t* h, const float** d_sum, const float** d_min);

/* Text of the last error on this host thread ("" if none). */
const char* per_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* PER_H */
