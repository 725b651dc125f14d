/* bitnet_i2s_stamps.h -- launch timing of the instrumented build.
 *
 * libbitnet_i2s_stamps.so is the same library built with -DBITNET_STAMPS: it
 * exports every function of bitnet_i2s.h with identical results, and its
 * decode GEMV (bitnet_gemv_i2s_i8, its grouped form and bitnet_linear_i2s up
 * to BITNET_LINEAR_FUSED_MAX_N tokens) records, for every launch, the device
 * time at which the launch's first workgroup started and its last wave
 * finished (s_memrealtime, 100 MHz ticks, by atomic min / max).  A launch's
 * own duration is then end - start, with no tracer serialising the launches
 * and no launch gap included.  The product library libbitnet_i2s.so has no
 * such slots and does not export these functions.
 *
 * Slots are taken in launch order by the host call that enqueues the launch
 * (for a captured graph: at capture time, so every replay writes the same
 * slots) and wrap after 512 launches.  One device at a time; calls that
 * launch from several host threads at once interleave their slots.
 */
#ifndef BITNET_I2S_STAMPS_H
#define BITNET_I2S_STAMPS_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Clears every slot on the current device (start = UINT64_MAX, end = 0) by a
 * kernel enqueued on `stream` (a hipStream_t, NULL = default stream); with
 * rewind != 0 the next launch also takes slot 0 again.  Returns 0, or
 * BITNET_E_HIP when the slots cannot be reached. */
int bitnet_stamps_reset(int rewind, void *stream);

/* Synchronises the device, then copies the [start, end] pairs of the launches
 * made since the last rewind (at most max_launches of them, in launch order)
 * to the host array `out` (2 * max_launches uint64_t, caller-owned).  Returns
 * the number of pairs copied, or -1 on a HIP error or a NULL `out`. */
int bitnet_stamps_read(uint64_t *out, int max_launches);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_I2S_STAMPS_H */
