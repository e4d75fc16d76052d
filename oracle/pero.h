/*
 * pero.h -- CPU oracle for the prioritized-replay sum tree.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may include, link,
 * load or call this code: only the test suite, the package smoke check and the
 * CPU-baseline leg of the benchmark do.  It shares no source with the HIP
 * library and is deliberately plain: single-threaded loops, one element at a
 * time, in the order the method is described.
 *
 * What it models (citations are to the source pages by title and section):
 *  - "Putting prioritized replay's segment tree on a GPU",
 *    section "The Tree Under Every Prioritized Replay": a flat implicit binary
 *    tree in an array of 2n entries, leaves at [n, 2n), node i with children
 *    2i and 2i+1, every internal node the sum of its children, root at 1; and
 *    a twin tree with min in place of sum.
 *  - same page, section "Sampling Is a Descent": proportional sampling by a
 *    root-to-leaf walk that goes left while the left sum exceeds the
 *    remaining mass, else subtracts it and goes right.
 *  - "GPU-Resident Prioritized Experience Replay", sections "Architecture"
 *    (ring storage layout), "Experience Insertion" (new items at the current
 *    max priority, cursor wrap), "Priority update" (|td| to the power alpha
 *    plus epsilon), "Sampling Kernels" (importance-sampling weights), and
 *    "Error Handling & Fallback" (NaN/Inf clamp).
 *
 * Readings taken where the pages are silent or disagree (each is listed in
 * the design notes of the repository):
 *  - nodes are f32; every internal node is recomputed as the f32 sum (round to
 *    nearest) of its two children, never updated by adding a delta;
 *  - the descent carries the mass in f32 and also goes left when the right
 *    child is exactly zero;
 *  - priority p = f32( pow_f64(|td| + eps, alpha) ); NaN td gives the td = 0
 *    value, +/-Inf td gives the running max priority at batch start;
 *  - the running max priority starts at 1.0 and takes the max of every
 *    priority written;
 *  - update indices outside [0, size) are skipped; duplicates follow batch
 *    order (the last position wins);
 *  - IS weight w = f32( (N*P(i))^-beta / (N*P_min)^-beta ) in f64 with
 *    N = size, P(i) = p_i / total, P_min = min-tree root / total; w = 0 when
 *    the min-tree root is 0.
 */
#ifndef PERO_H
#define PERO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pero pero_t;

/* Returns NULL if capacity is not a power of two in [2, 2^30], state_dim < 0
 * or memory cannot be had.  state_dim == 0 keeps no transition storage. */
pero_t* pero_create(int64_t capacity, int32_t state_dim, double alpha, double eps);
void pero_destroy(pero_t* t);

/* Ring intake of count transitions; prio == NULL gives each new item the
 * running max priority.  Row pointers are ignored when state_dim == 0.
 * Returns 0, or -1 if count is outside [0, capacity]. */
int pero_add(pero_t* t, int64_t count, const float* states, const float* next_states,
             const uint32_t* actions, const float* rewards, const uint8_t* dones,
             const float* prio);

/* Priority update in batch order.  Returns 0, or -1 if B < 0. */
int pero_update(pero_t* t, int64_t B, const int64_t* idx, const float* td);

/* Proportional sample of B transitions for the uniforms u in [0, 1).
 * w_out and the row outputs may be NULL.  Returns 0, -1 if B < 0, or -3
 * when the buffer is empty. */
int pero_sample(const pero_t* t, int64_t B, const float* u, double beta, int64_t* idx_out,
                float* w_out, float* states_out, float* next_states_out,
                uint32_t* actions_out, float* rewards_out, uint8_t* dones_out);

/* Philox4x64-10 block, and word j of a seed's stream (word j % 4 of the
 * block at counter (j / 4, 0, 0, 0) under key (seed, 0)). */
void pero_philox4x64(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]);
uint64_t pero_stream_word(uint64_t seed, uint64_t j);

/* pero_sample with u_b = (word(offset + b) >> 40) * 2^-24. */
int pero_sample_philox(const pero_t* t, int64_t B, uint64_t seed, uint64_t offset, double beta,
                       int64_t* idx_out, float* w_out, float* states_out,
                       float* next_states_out, uint32_t* actions_out, float* rewards_out,
                       uint8_t* dones_out);

/* Uniform sample: idx_b = ((word(offset + b) >> 32) * size) >> 32; rows as
 * pero_sample.  -3 if size == 0. */
int pero_sample_uniform(const pero_t* t, int64_t B, uint64_t seed, uint64_t offset,
                        int64_t* idx_out, float* states_out, float* next_states_out,
                        uint32_t* actions_out, float* rewards_out, uint8_t* dones_out);

/* Rank-based sampling: pero_rank_refresh ranks the filled slots (order[r]
 * = slot of rank r + 1, by descending priority, ties by ascending slot) and
 * builds the tree over the rank weights f32((r+1)^-alpha); pero_sample_rank
 * descends that tree and samples order[r].  The rank arrays are valid after
 * a refresh (NULL before the first). */
int pero_rank_refresh(pero_t* t);
int pero_sample_rank(const pero_t* t, int64_t B, const float* u, double beta, int64_t* idx_out,
                     float* w_out, float* states_out, float* next_states_out,
                     uint32_t* actions_out, float* rewards_out, uint8_t* dones_out);
const int64_t* pero_rank_order(const pero_t* t);
const float* pero_rank_sum_tree(const pero_t* t);
const float* pero_rank_min_tree(const pero_t* t);

/* pero_sample written into padded trainer buffers: state rows of out_stride
 * >= D floats, zero past column D; actions i32 (stored bits), rewards f32,
 * dones f32.  -1 if out_stride < D. */
int pero_sample_padded(const pero_t* t, int64_t B, const float* u, double beta, int64_t* idx_out,
                       float* w_out, float* states_out, float* next_states_out,
                       int64_t out_stride, int32_t* actions_out, float* rewards_out,
                       float* dones_out);

float pero_total(const pero_t* t);
float pero_min(const pero_t* t);
float pero_max_priority(const pero_t* t);
int64_t pero_size(const pero_t* t);
int64_t pero_cursor(const pero_t* t);
int64_t pero_capacity(const pero_t* t);
int32_t pero_state_dim(const pero_t* t);

/* Read-only views of the 2n-entry trees (index 0 unused). */
const float* pero_sum_tree(const pero_t* t);
const float* pero_min_tree(const pero_t* t);

#ifdef __cplusplus
}
#endif
#endif /* PERO_H */
