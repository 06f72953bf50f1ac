/*
 * gpu_clock.h -- shader-clock sampling for throughput measurements.
 *
 * Not part of the attention operation.  A matrix-bound kernel's time scales with
 * the shader clock the GPU sustains while it runs, and that clock moves with power
 * and temperature from box to box and within a run.  These calls let a benchmark
 * record it next to the time it measures, from inside the GPU, without any other
 * process: the shader core's cycle counter (s_memtime) is read against the
 * constant-rate wall-clock counter (s_memrealtime) on one wave.
 *
 * Both counters are 64-bit and read on the device.  Calls are stream-ordered and
 * return before the work finishes; results are valid after the stream synchronises.
 * Buffers are device memory owned by the caller.  Status codes are those of attn.h
 * (0 on success, negative on error, nothing launched on error).
 */
#ifndef EXACT_ATTENTION_89_GPU_CLOCK_H
#define EXACT_ATTENTION_89_GPU_CLOCK_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/*
 * attn_clock_sampler -- one wave records (wall ticks, shader cycles, phase) triples.
 *
 * samples: device buffer of 3 * max_samples + 1 uint64 values; samples[0] receives the
 * number of triples written, triple i is samples[1 + 3i .. 3 + 3i]: the wave's
 * wall-clock ticks, its shader cycles, and the value of the int at `phase` (device
 * memory, read with agent scope) when the triple was taken.  Both counters are the
 * sampling wave's own, so only differences between triples are meaningful (counters
 * of different XCDs need not agree).  A triple is taken every interval_ticks wall
 * ticks (the wave sleeps in between); the wave ends after the first triple whose
 * phase equals stop_value, or once duration_ticks have passed, or after max_samples
 * triples, whichever comes first, so the kernel always ends.  Launched on a stream of
 * its own it runs beside other work and occupies one wave slot of one CU; an
 * attn_clock_mark(phase, stop_value) enqueued behind that work ends it, so that a
 * device-wide synchronisation after the work does not wait out the duration.
 * Errors: ATTN_ERR_NULL (samples or phase NULL), ATTN_ERR_ALIGN (samples not 8-byte
 * or phase not 4-byte aligned), ATTN_ERR_SHAPE (max_samples < 1 or > 1 << 20,
 * interval_ticks or duration_ticks 0).
 */
int attn_clock_sampler(uint64_t* samples, const int* phase, int stop_value, int max_samples,
                       uint64_t interval_ticks, uint64_t duration_ticks, void* stream);

/*
 * attn_clock_mark -- store `value` into the int at `phase` (agent scope) when `stream`
 * reaches this point: a marker between other launches, which a running sampler records
 * with every later triple.  Errors: ATTN_ERR_NULL, ATTN_ERR_ALIGN.
 */
int attn_clock_mark(int* phase, int value, void* stream);

/* Frequency of the wall-clock counter of the current device, in Hz (> 0), or a
 * negative status (ATTN_ERR_HIP) if the runtime cannot report it. */
int64_t attn_clock_wall_hz(void);

#ifdef __cplusplus
}
#endif

#endif
