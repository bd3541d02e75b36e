/*
 * spec_debug.h -- kernel timing for benchmarks and profiling tools.
 *
 * Not part of the operations' contract (spec.h): these calls keep one
 * process-wide record of HIP events, guarded by a mutex, and are meant for a
 * benchmark driving one stream at a time.  With timing off (the default)
 * every launch skips the records entirely.
 */
#ifndef SPEC_DEBUG_H
#define SPEC_DEBUG_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* on != 0: every later kernel launch of the library, on any stream, records
 * a HIP event pair on its own stream around itself (the events timestamp
 * the kernel on the stream it runs on).  0 stops recording.  Returns 0. */
int spec_profile_enable(int on);
/* Drop every record (events are kept for reuse).  Returns 0. */
int spec_profile_reset(void);
/* Synchronise the recorded events of the kernel named `kernel` (host
 * string) and return, through the host pointers, the number of launches
 * and their total duration in milliseconds since the last reset.  Returns
 * 0, SPEC_EINVAL (1) for a NULL argument, or SPEC_ELAUNCH (4) if an event
 * could not be read. */
int spec_profile_read(const char* kernel, int* launches, double* total_ms);
/* Names of kernels with records, separated by ',', into buf (host, buf_len
 * bytes, always NUL-terminated when buf_len > 0); returns the length needed
 * including the NUL. */
int spec_profile_names(char* buf, int buf_len);

/* The kernels' own Philox4x32-10 (the function every draw of spec.h calls),
 * exposed so that tests can compare it bit for bit with an independent
 * implementation: for i = 0..n-1, out[4i .. 4i+3] (device, uint32) = the
 * four output words at key = seed and counter (i mod 2^16, i / 2^16,
 * round_lo, round_hi).  n <= 2^32.  Enqueued on stream; returns 0, or
 * SPEC_EINVAL (1) for a NULL out, SPEC_ELAUNCH (4) on a launch error. */
int spec_philox_words(uint64_t seed, uint64_t round, size_t n, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* SPEC_DEBUG_H */
