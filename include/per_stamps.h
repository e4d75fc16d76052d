/*
 * per_stamps.h -- phase stamps of the update kernels and the sampler
 * (libper_stamps.so, gfx950): a measurement build of libper.so, the same
 * sources compiled with PER_PHASE_STAMPS, that exports every call of per.h
 * plus the four below.
 * Not part of the replay buffer.
 *
 * A batch of a few hundred updates on a 2^21-leaf tree moves a fraction of
 * a megabyte, so the fused update + intake kernel's time is set by chains
 * of dependent trips and by one wave's serial repair ("Putting prioritized
 * replay's segment tree on a GPU", section "Second Port: Make the Update
 * GPU-Shaped": the update walks each dirty path up to the root).  In this
 * build, lane 0 of wave w of block b stores the 100 MHz real-time clock
 * (s_memrealtime) at the end of phase k into slot [b * 16 + k] of a device
 * array of 4096 x 16 u64 (blocks past 4096 store nothing):
 *
 *   k  wave  end of
 *   0   0    the kernel's argument fetch (the block's start)
 *   1   0    its share of the batch scan (entries and their siblings collected)
 *   2   0    the partition's sparse repair (its last store issued)
 *   3   0    the intake's boundary loads issued (blocks that meet the ring range)
 *   4   0    the barrier after them
 *   5   0    the intake's boundary climb stored
 *   6   1    the batch max (blocks that meet the ring range)
 *   7   1    the argument fetch
 *   8   0    the barrier after the scan (the repair's start)
 *  10-12 1-3 their share of the batch scan
 *  13   0    the repair's sort (entries in order)
 *  14   0    the repair's sibling reads from LDS
 *
 * Slots 0-7 are stored by the fused update + intake kernel only; 1, 2, 8 and
 * 10-14 also by the other update kernels that share those phases.
 *
 * The proportional sampler (section "Sampling Is a Descent" of the same page)
 * keeps a second array of 4096 x 8 u64: lane 0 of wave w (of 4) of block b
 * stores the clock when the wave starts into slot [b * 8 + w] and when it is
 * done (descent, weights and rows) into slot [b * 8 + 4 + w].
 *
 * Each stamp waits for its own scalar read of the clock, so a phase ending in
 * a stamp reads long by that wait.
 *
 * Work goes to the caller's stream.  Return 0, -1 for a bad argument
 * (checked on the host) or -4 for a HIP error.
 */
#ifndef PER_STAMPS_H
#define PER_STAMPS_H

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Enqueue the zeroing of every slot (a memset: not for a stream being
 * captured into a graph). */
int per_stamps_clear(hipStream_t stream);

/* Copy the first `count` slots (0 <= count <= 4096 * 16) to host memory at
 * `out`, then wait for the stream. */
int per_stamps_read(unsigned long long* out, long long count, hipStream_t stream);

/* The same for the sampler's array (0 <= count <= 4096 * 8). */
int per_sample_stamps_clear(hipStream_t stream);
int per_sample_stamps_read(unsigned long long* out, long long count, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif  // PER_STAMPS_H
