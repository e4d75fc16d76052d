/*
 * per_probe.h -- measurement aids for the latency floor of the tree's short
 * launches (libper_probe.so, gfx950).  Not part of the replay buffer: a
 * batch of a few hundred samples and updates on a 2^21-leaf tree moves a
 * fraction of a megabyte, so its time is set by launch overhead and by
 * chains of dependent loads, one per tree level ("Putting prioritized
 * replay's segment tree on a GPU", section "Sampling Is a Descent": a
 * descent reads one node pair per level, each read depending on the last).
 * The first two calls measure those two costs on their own; the third
 * measures what an argument block adds to a launch.
 *
 * Device pointers are prefixed d_ and owned by the caller; work goes to the
 * caller's stream; nothing is allocated and nothing waits (except in
 * per_probe_launch_cost, which says so).  Return 0, or -1 for a bad argument
 * (checked on the host), or -4 for a HIP error.
 */
#ifndef PER_PROBE_H
#define PER_PROBE_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue `launches` (>= 1) launches of an empty kernel, one 64-lane block
 * each, back to back. */
int per_probe_empty(int64_t launches, hipStream_t stream);

/* Enqueue one kernel in which a single lane follows the chain i <- d_next[i]
 * for `depth` (>= 1) dependent loads from i = 0, and stores the last i to
 * d_out[0].  d_next: [length] u32, length a power of two in [1, 2^30]; each
 * index is reduced modulo length before it is used, so any content stays in
 * bounds.  A random cyclic permutation makes every load wait for the one
 * before and land on a line the others rarely share. */
int per_probe_chain(const uint32_t* d_next, int64_t length, int64_t depth, uint32_t* d_out,
                    hipStream_t stream);

/* The cost of one launch of an empty kernel (one 64-lane block) that takes
 * an argument block of arg_bytes (16, 256 or 512) bytes, in us, into
 * *us_per_launch: `launches` (in [100, 100000], a multiple of 100) launches
 * back to back on a stream of the call's own, timed with events after a
 * warm-up; with graph != 0 the same launches are captured 100 at a time into
 * a HIP graph and replayed, so that no host work stands between them.
 * Creates and destroys its stream, events and graph; waits for the work. */
int per_probe_launch_cost(int64_t launches, int arg_bytes, int graph, double* us_per_launch);

#ifdef __cplusplus
}
#endif

#endif  // PER_PROBE_H
