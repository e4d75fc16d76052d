/*
 * pero.c -- CPU oracle for the prioritized-replay sum tree.
 *
 * TEST INFRASTRUCTURE ONLY (see pero.h).  Plain C, one element at a time,
 * built with -O2 -ffp-contract=off and no fast-math so that every f32 add,
 * subtract and min is a single IEEE round-to-nearest operation.
 */
#include "pero.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

struct pero {
    int64_t n;          /* capacity = number of leaves, a power of two */
    int32_t D;          /* state_dim; 0 = no transition storage */
    double alpha, eps;
    float* sum;         /* [2n], index 0 unused, leaves at [n, 2n) */
    float* mn;          /* [2n], same layout, min in place of sum */
    float* states;      /* [n*D] */
    float* next_states; /* [n*D] */
    uint32_t* actions;  /* [n] */
    float* rewards;     /* [n] */
    uint8_t* dones;     /* [n] */
    int64_t size, cursor;
    float maxp;         /* running max priority */
    /* rank-based sampling, as of the last pero_rank_refresh */
    int64_t rank_size;  /* filled slots when refreshed; 0 = never */
    int64_t* order;     /* [n] slots by descending priority, ties by slot */
    float* rsum;        /* [2n] tree over the rank weights, as sum */
    float* rmn;         /* [2n] and its twin min tree */
};

/* Recompute every ancestor of tree node i, from its parent up to the root.
 * "The Tree Under Every Prioritized Replay": an internal node holds the sum of
 * its children (and, in the twin tree, their min); a point update touches one
 * leaf-to-root path. */
static void walk_to_root(pero_t* t, int64_t i) {
    for (i >>= 1; i >= 1; i >>= 1) {
        float l = t->sum[2 * i], r = t->sum[2 * i + 1];
        t->sum[i] = l + r;
        float a = t->mn[2 * i], b = t->mn[2 * i + 1];
        t->mn[i] = (b < a) ? b : a;
    }
}

static void set_leaf(pero_t* t, int64_t slot, float p) {
    int64_t i = t->n + slot;
    t->sum[i] = p;
    t->mn[i] = p;
    walk_to_root(t, i);
}

pero_t* pero_create(int64_t capacity, int32_t state_dim, double alpha, double eps) {
    if (capacity < 2 || capacity > ((int64_t)1 << 30)) return NULL;
    if ((capacity & (capacity - 1)) != 0) return NULL;
    if (state_dim < 0) return NULL;
    pero_t* t = (pero_t*)calloc(1, sizeof(pero_t));
    if (!t) return NULL;
    t->n = capacity;
    t->D = state_dim;
    t->alpha = alpha;
    t->eps = eps;
    t->sum = (float*)malloc(sizeof(float) * 2 * capacity);
    t->mn = (float*)malloc(sizeof(float) * 2 * capacity);
    if (!t->sum || !t->mn) { pero_destroy(t); return NULL; }
    /* Empty slots are the neutral elements: 0 for sum, +inf for min. */
    for (int64_t i = 0; i < 2 * capacity; ++i) {
        t->sum[i] = 0.0f;
        t->mn[i] = INFINITY;
    }
    if (state_dim > 0) {
        t->states = (float*)calloc((size_t)capacity * state_dim, sizeof(float));
        t->next_states = (float*)calloc((size_t)capacity * state_dim, sizeof(float));
        t->actions = (uint32_t*)calloc((size_t)capacity, sizeof(uint32_t));
        t->rewards = (float*)calloc((size_t)capacity, sizeof(float));
        t->dones = (uint8_t*)calloc((size_t)capacity, sizeof(uint8_t));
        if (!t->states || !t->next_states || !t->actions || !t->rewards || !t->dones) {
            pero_destroy(t);
            return NULL;
        }
    }
    t->size = 0;
    t->cursor = 0;
    t->maxp = 1.0f;
    return t;
}

void pero_destroy(pero_t* t) {
    if (!t) return;
    free(t->sum);
    free(t->mn);
    free(t->states);
    free(t->next_states);
    free(t->actions);
    free(t->rewards);
    free(t->dones);
    free(t->order);
    free(t->rsum);
    free(t->rmn);
    free(t);
}

/* "GPU-Resident Prioritized Experience Replay", section "Experience
 * Insertion": new experiences take the current max priority and the write
 * cursor wraps modulo capacity; section "Error Handling & Fallback": ring
 * overflow overwrites the oldest items.  Given priorities replace the max
 * priority and raise it; -0.0 is read as +0.0. */
int pero_add(pero_t* t, int64_t count, const float* states, const float* next_states,
             const uint32_t* actions, const float* rewards, const uint8_t* dones,
             const float* prio) {
    if (count < 0 || count > t->n) return -1;
    const int64_t D = t->D;
    for (int64_t j = 0; j < count; ++j) {
        int64_t slot = (t->cursor + j) % t->n;
        if (D > 0) {
            memcpy(t->states + slot * D, states + j * D, sizeof(float) * D);
            memcpy(t->next_states + slot * D, next_states + j * D, sizeof(float) * D);
            t->actions[slot] = actions[j];
            t->rewards[slot] = rewards[j];
            t->dones[slot] = dones[j];
        }
        float p;
        if (prio) {
            p = prio[j] + 0.0f;
            if (p > t->maxp) t->maxp = p;
        } else {
            p = t->maxp;
        }
        set_leaf(t, slot, p);
    }
    t->cursor = (t->cursor + count) % t->n;
    t->size = (t->size + count < t->n) ? t->size + count : t->n;
    return 0;
}

/* Priority of one TD error.  "GPU-Resident Prioritized Experience Replay",
 * section "Priority update" (|td| to the power alpha, plus epsilon; read here
 * as (|td| + eps)^alpha, evaluated in f64 and rounded once to f32) and
 * section "Error Handling & Fallback" (NaN/Inf are clamped: NaN to the td = 0
 * value, the lowest priority; Inf to the running max at batch start). */
static float priority_of(const pero_t* t, float td, float max_at_start) {
    float x = fabsf(td);
    if (isnan(x)) return (float)pow(t->eps, t->alpha);
    if (isinf(x)) return max_at_start;
    return (float)pow((double)x + t->eps, t->alpha);
}

/* Batch update, element by element in batch order so that a later position
 * of a repeated index wins; each element walks its leaf-to-root path
 * ("Putting prioritized replay's segment tree on a GPU", section "Second
 * Port: Make the Update GPU-Shaped", the per-element propagation it starts
 * from). */
int pero_update(pero_t* t, int64_t B, const int64_t* idx, const float* td) {
    if (B < 0) return -1;
    const float max_at_start = t->maxp;
    for (int64_t b = 0; b < B; ++b) {
        int64_t slot = idx[b];
        if (slot < 0 || slot >= t->size) continue;
        float p = priority_of(t, td[b], max_at_start);
        if (p > t->maxp) t->maxp = p;
        set_leaf(t, slot, p);
    }
    return 0;
}

/* The leaf offset that mass m in [0, total) selects ("Putting prioritized
 * replay's segment tree on a GPU", section "Sampling Is a Descent").  The
 * offset is built one bit per level, most significant first: at depth d the
 * walk stands on node 2^d + off and compares the remaining mass with its two
 * children.  The bit is 1 -- the right child -- when the left child's sum
 * does not exceed the mass, and then that sum is taken off the mass.
 * Readings: the mass is an f32 and every subtraction is rounded to f32, and
 * a right child whose sum is 0 is never taken. */
static int64_t descend_tree(const float* sum, int64_t n, float m) {
    int levels = 0;
    while (((int64_t)1 << levels) < n) ++levels;
    int64_t off = 0;
    for (int d = 0; d < levels; ++d) {
        const int64_t node = ((int64_t)1 << d) + off;
        const float left = sum[2 * node], right = sum[2 * node + 1];
        const int bit = !(left > m) && right != 0.0f;
        if (bit) m -= left;
        off = 2 * off + bit;
    }
    return off;
}

/* IS weight of a sampled priority p: (N*P(i))^-beta normalised by its
 * largest value, which belongs to the minimum priority ("GPU-Resident
 * Prioritized Experience Replay", section "Sampling Kernels"); 0 when the
 * minimum priority is 0. */
static float is_weight(double N, float p, float pmin, float total, double beta) {
    if (!(pmin > 0.0f)) return 0.0f;
    double P_i = (double)p / (double)total;
    double P_min = (double)pmin / (double)total;
    return (float)(pow(N * P_i, -beta) / pow(N * P_min, -beta));
}

/* "GPU-Resident Prioritized Experience Replay", section "Sampling Kernels":
 * masses in [0, total), one search per sample, gather of the sampled rows,
 * then IS weights.  The weight is (N*P(i))^-beta normalised by its largest
 * value, which belongs to the minimum priority (the min tree serves this
 * normalisation: "The Tree Under Every Prioritized Replay"). */
int pero_sample(const pero_t* t, int64_t B, const float* u, double beta, int64_t* idx_out,
                float* w_out, float* states_out, float* next_states_out,
                uint32_t* actions_out, float* rewards_out, uint8_t* dones_out) {
    if (B < 0) return -1;
    if (B == 0) return 0;
    if (t->size == 0) return -3;
    const float total = t->sum[1];
    const float pmin = t->mn[1];
    const double N = (double)t->size;
    const int64_t D = t->D;
    for (int64_t b = 0; b < B; ++b) {
        float m = u[b] * total;
        if (!(m < total)) m = nextafterf(total, 0.0f);
        int64_t slot = descend_tree(t->sum, t->n, m);
        idx_out[b] = slot;
        if (w_out) w_out[b] = is_weight(N, t->sum[t->n + slot], pmin, total, beta);
        if (D > 0 && states_out) {
            memcpy(states_out + b * D, t->states + slot * D, sizeof(float) * D);
            memcpy(next_states_out + b * D, t->next_states + slot * D, sizeof(float) * D);
            actions_out[b] = t->actions[slot];
            rewards_out[b] = t->rewards[slot];
            dones_out[b] = t->dones[slot];
        }
    }
    return 0;
}

/* The same sample written straight into a trainer's buffers ("True
 * Single-Graph Implementation Plan", Tasks 2 and 3): indices and weights are
 * those of pero_sample; each state row goes into a destination row of
 * out_stride >= D floats whose columns D .. out_stride-1 are 0; actions are
 * written as i32 (the stored 32 bits), rewards as f32 and dones as f32 (the
 * stored byte's value).  Row outputs all NULL, or all given. */
int pero_sample_padded(const pero_t* t, int64_t B, const float* u, double beta, int64_t* idx_out,
                       float* w_out, float* states_out, float* next_states_out,
                       int64_t out_stride, int32_t* actions_out, float* rewards_out,
                       float* dones_out) {
    const int64_t D = t->D;
    if (out_stride < D) return -1;
    int rc = pero_sample(t, B, u, beta, idx_out, w_out, NULL, NULL, NULL, NULL, NULL);
    if (rc != 0 || D == 0 || !states_out) return rc;
    for (int64_t b = 0; b < B; ++b) {
        const int64_t slot = idx_out[b];
        for (int64_t c = 0; c < out_stride; ++c) {
            states_out[b * out_stride + c] = (c < D) ? t->states[slot * D + c] : 0.0f;
            next_states_out[b * out_stride + c] = (c < D) ? t->next_states[slot * D + c] : 0.0f;
        }
        memcpy(&actions_out[b], &t->actions[slot], sizeof(int32_t));
        rewards_out[b] = t->rewards[slot];
        dones_out[b] = (float)t->dones[slot];
    }
    return 0;
}

/* Philox4x64-10 (Salmon, Moraes, Dror and Shaw, "Parallel Random Numbers:
 * As Easy as 1, 2, 3", SC 2011): ten rounds over a 4 x 64-bit counter with
 * a 2 x 64-bit key; a round multiplies counter words 0 and 2 by the two
 * round constants into 128-bit products and mixes their halves with words
 * 1 and 3 and the key; the key gains the two Weyl constants between rounds. */
void pero_philox4x64(const uint64_t ctr_in[4], const uint64_t key_in[2], uint64_t out[4]) {
    uint64_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint64_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        if (r > 0) {
            k0 += 0x9E3779B97F4A7C15ull;
            k1 += 0xBB67AE8584CAA73Bull;
        }
        unsigned __int128 p0 = (unsigned __int128)0xD2E7470EE14C6C93ull * c0;
        unsigned __int128 p1 = (unsigned __int128)0xCA5A826395121157ull * c2;
        uint64_t n0 = (uint64_t)(p1 >> 64) ^ c1 ^ k0;
        uint64_t n1 = (uint64_t)p1;
        uint64_t n2 = (uint64_t)(p0 >> 64) ^ c3 ^ k1;
        uint64_t n3 = (uint64_t)p0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* Word j of the stream of a seed: word j % 4 of the block at counter
 * (j / 4, 0, 0, 0) under key (seed, 0). */
uint64_t pero_stream_word(uint64_t seed, uint64_t j) {
    const uint64_t ctr[4] = {j / 4, 0, 0, 0};
    const uint64_t key[2] = {seed, 0};
    uint64_t out[4];
    pero_philox4x64(ctr, key, out);
    return out[j % 4];
}

/* Proportional sample with the masses drawn on the device side of the
 * method ("GPU-Resident Prioritized Experience Replay", section "Sampling
 * Kernels": the uniform values come from a generator, not from the host):
 * sample b uses u_b = (word(offset + b) >> 40) * 2^-24, then pero_sample. */
int pero_sample_philox(const pero_t* t, int64_t B, uint64_t seed, uint64_t offset, double beta,
                       int64_t* idx_out, float* w_out, float* states_out,
                       float* next_states_out, uint32_t* actions_out, float* rewards_out,
                       uint8_t* dones_out) {
    if (B < 0) return -1;
    if (B == 0) return 0;
    float* u = (float*)malloc(sizeof(float) * (size_t)B);
    if (!u) return -1;
    for (int64_t b = 0; b < B; ++b)
        u[b] = (float)(pero_stream_word(seed, offset + (uint64_t)b) >> 40) * 0x1p-24f;
    int rc = pero_sample(t, B, u, beta, idx_out, w_out, states_out, next_states_out,
                         actions_out, rewards_out, dones_out);
    free(u);
    return rc;
}

/* Uniform sample over the filled slots (the same section: without
 * prioritisation the ring is sampled uniformly from generated indices into
 * [0, size)): idx_b = ((word(offset + b) >> 32) * size) >> 32, rows as in
 * pero_sample. */
int pero_sample_uniform(const pero_t* t, int64_t B, uint64_t seed, uint64_t offset,
                        int64_t* idx_out, float* states_out, float* next_states_out,
                        uint32_t* actions_out, float* rewards_out, uint8_t* dones_out) {
    if (B < 0) return -1;
    if (B == 0) return 0;
    if (t->size == 0) return -3;
    const int64_t D = t->D;
    for (int64_t b = 0; b < B; ++b) {
        const uint64_t hi = pero_stream_word(seed, offset + (uint64_t)b) >> 32;
        const int64_t slot = (int64_t)((hi * (uint64_t)t->size) >> 32);
        idx_out[b] = slot;
        if (D > 0 && states_out) {
            memcpy(states_out + b * D, t->states + slot * D, sizeof(float) * D);
            memcpy(next_states_out + b * D, t->next_states + slot * D, sizeof(float) * D);
            actions_out[b] = t->actions[slot];
            rewards_out[b] = t->rewards[slot];
            dones_out[b] = t->dones[slot];
        }
    }
    return 0;
}

/* Rank-based prioritisation ("GPU-Resident Prioritized Experience Replay",
 * section "Sampling Kernels", rank-based: sort the (priority, index) pairs
 * descending, then sample with probabilities 1/rank^alpha through their
 * cumulative sum, gather, IS weights).  The refresh ranks the filled slots:
 * order[r] is the slot of rank r + 1, by descending priority, equal
 * priorities by ascending slot; the rank weights w_r = f32((r+1)^-alpha) are
 * the leaves of a second tree built like the priority trees (sums and mins
 * of children), which holds their cumulative sums for the descent. */
typedef struct {
    float p;
    int64_t slot;
} rank_pair;

static int by_priority_desc(const void* a, const void* b) {
    const rank_pair* x = (const rank_pair*)a;
    const rank_pair* y = (const rank_pair*)b;
    if (x->p > y->p) return -1;
    if (x->p < y->p) return 1;
    return (x->slot < y->slot) ? -1 : (x->slot > y->slot);
}

int pero_rank_refresh(pero_t* t) {
    const int64_t n = t->n;
    if (!t->order) {
        t->order = (int64_t*)calloc((size_t)n, sizeof(int64_t));
        t->rsum = (float*)calloc((size_t)(2 * n), sizeof(float));
        t->rmn = (float*)calloc((size_t)(2 * n), sizeof(float));
        if (!t->order || !t->rsum || !t->rmn) return -1;
    }
    rank_pair* pairs = (rank_pair*)malloc(sizeof(rank_pair) * (size_t)(t->size ? t->size : 1));
    if (!pairs) return -1;
    for (int64_t s = 0; s < t->size; ++s) {
        pairs[s].p = t->sum[n + s];
        pairs[s].slot = s;
    }
    qsort(pairs, (size_t)t->size, sizeof(rank_pair), by_priority_desc);
    for (int64_t r = 0; r < t->size; ++r) t->order[r] = pairs[r].slot;
    free(pairs);
    for (int64_t r = 0; r < n; ++r) {
        const float w = (r < t->size) ? (float)pow((double)(r + 1), -t->alpha) : 0.0f;
        t->rsum[n + r] = w;
        t->rmn[n + r] = (r < t->size) ? w : INFINITY;
    }
    for (int64_t i = n - 1; i >= 1; --i) {
        float l = t->rsum[2 * i], r = t->rsum[2 * i + 1];
        t->rsum[i] = l + r;
        float a = t->rmn[2 * i], b = t->rmn[2 * i + 1];
        t->rmn[i] = (b < a) ? b : a;
    }
    t->rank_size = t->size;
    return 0;
}

/* Rank-based sample as of the last refresh: the descent of pero_sample on
 * the rank-weight tree gives a rank r; the sampled slot is order[r]; the IS
 * weight is that of pero_sample with the rank weights as priorities and
 * N = the filled size at the refresh.  -3 if never refreshed or empty. */
int pero_sample_rank(const pero_t* t, int64_t B, const float* u, double beta, int64_t* idx_out,
                     float* w_out, float* states_out, float* next_states_out,
                     uint32_t* actions_out, float* rewards_out, uint8_t* dones_out) {
    if (B < 0) return -1;
    if (B == 0) return 0;
    if (t->rank_size == 0) return -3;
    const float total = t->rsum[1];
    const float pmin = t->rmn[1];
    const double N = (double)t->rank_size;
    const int64_t D = t->D;
    for (int64_t b = 0; b < B; ++b) {
        float m = u[b] * total;
        if (!(m < total)) m = nextafterf(total, 0.0f);
        const int64_t r = descend_tree(t->rsum, t->n, m);
        const int64_t slot = t->order[r];
        idx_out[b] = slot;
        if (w_out) w_out[b] = is_weight(N, t->rsum[t->n + r], pmin, total, beta);
        if (D > 0 && states_out) {
            memcpy(states_out + b * D, t->states + slot * D, sizeof(float) * D);
            memcpy(next_states_out + b * D, t->next_states + slot * D, sizeof(float) * D);
            actions_out[b] = t->actions[slot];
            rewards_out[b] = t->rewards[slot];
            dones_out[b] = t->dones[slot];
        }
    }
    return 0;
}

const int64_t* pero_rank_order(const pero_t* t) { return t->order; }
const float* pero_rank_sum_tree(const pero_t* t) { return t->rsum; }
const float* pero_rank_min_tree(const pero_t* t) { return t->rmn; }

float pero_total(const pero_t* t) { return t->sum[1]; }
float pero_min(const pero_t* t) { return t->mn[1]; }
float pero_max_priority(const pero_t* t) { return t->maxp; }
int64_t pero_size(const pero_t* t) { return t->size; }
int64_t pero_cursor(const pero_t* t) { return t->cursor; }
int64_t pero_capacity(const pero_t* t) { return t->n; }
int32_t pero_state_dim(const pero_t* t) { return t->D; }
const float* pero_sum_tree(const pero_t* t) { return t->sum; }
const float* pero_min_tree(const pero_t* t) { return t->mn; }
