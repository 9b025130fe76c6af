/*
 * msda_bench.h - measurement hooks of the MSDA library (libmsda.so), kept
 * apart from the operator's C ABI in msda.h.  Nothing here is needed to run
 * the operator; a benchmark uses these calls to time the library's kernels
 * and to measure the memory-path ceilings it compares them against.  The
 * pages ask for each design choice on this path to be backed by measured
 * bandwidth and atomic throughput ("Efficient Multi-Scale Deformable Attention
 * on GPUs", sections "Key findings" and "The backward pass is an atomics
 * problem").
 */
#ifndef MSDA_BENCH_H
#define MSDA_BENCH_H

#include <stddef.h>
#include <stdint.h>

#include "msda.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * Kernel timing for benchmarks.  Between msda_profile_start() and
 * msda_profile_stop() on one thread, every kernel this library enqueues from
 * that thread is bracketed by two HIP events recorded on its stream.
 * msda_profile_stop() waits for the last recorded event, copies at most `max`
 * records (kernel name, milliseconds between its events) into `out`, ends the
 * session and returns the number of kernels recorded (which may exceed `max`),
 * or -1 when a HIP event call failed.  Records past `capacity` are dropped.
 * The events are created by the library (host-side HIP objects, no device
 * memory) and kept for reuse until the process ends.
 */
typedef struct {
    const char *name; /* static string, e.g. "fwd_kernel<f32,32>" */
    float ms;
} msda_kernel_time;

msda_status msda_profile_start(int capacity);
int msda_profile_stop(msda_kernel_time *out, int max);
/*
 * Restrict the sessions of this thread to the kernels named `name` (the names
 * msda_profile_stop reports); NULL or "" records every kernel again.  Kernels
 * left out get no events at all, so a session can time one kernel while
 * disturbing the others as little as possible.  The events are created with
 * hipEventDisableSystemFence: recording one does not write back or invalidate
 * caches.
 */
void msda_profile_select(const char *name);

/*
 * Test hook: later binned backward plans made on this thread poll an earlier
 * plan block's totals at most `polls` times before giving up (default 2^24,
 * which never expires on a working device).  0 makes every plan block after
 * the first give up at once, which exercises the MSDA_BWD_PLAN_EXPIRED path
 * with every kernel still ending normally.
 */
void msda_test_set_plan_wait_limit(uint32_t polls);

/*
 * Test hook: the schedule of later forward launches (msda_forward,
 * msda_forward_softmax) on this thread.  0 (default): the LDS-window gather
 * when the launch has enough queries per (batch, head) for its staging to pay
 * off, else the direct gather; 1: always the direct gather; 2: the LDS-window
 * gather whenever the device's LDS holds its tables.  Both compute the same
 * sums; only the order of the fp32 additions may differ.
 */
void msda_test_set_forward_schedule(int schedule);

/*
 * Test hook: with wide != 0, later binned backward calls on this thread run
 * the tile pass with 64-bit sample-id division and grad_out addresses, the
 * path it otherwise takes only when a launch's sample ids or grad_out image
 * reach 2^31 (sizes too large to check against the oracle element by
 * element).  0 restores the default.  Both paths compute the same sums.
 */
void msda_test_set_tile_wide_addressing(int wide);

/*
 * Diagnostic: shader-clock sums of the phases of the last binned tile pass on
 * the current device, one row of 12 unsigned 64-bit values per tile block
 * (row = block index), copied into out (host memory, nblocks * 12 values,
 * owned by the caller).  Each row is wave 0's view of its block: slot 0
 * staging and the chunk claim, 1 cell pass, 2 cell scan, plan and record sort,
 * 3 item loop, 4 the next chunk's position, 5 its loads issued, 6 result pass,
 * 7 pixel pass, 8 the last barrier, 9 and 10 unused, 11 chunks processed.
 * Only a library built with -DMSDA_TILE_PHASE_CLOCKS records them; any other
 * build returns MSDA_ERR_UNSUPPORTED without touching the device.  Errors:
 * MSDA_ERR_NULL_POINTER, MSDA_ERR_INVALID_DIMS (nblocks outside 0..2048),
 * MSDA_ERR_HIP.
 */
msda_status msda_test_tile_phase_clocks(unsigned long long *out, int nblocks);

/* Memory-path microbenchmarks (msda_microbench_run). */
typedef enum {
    /* streaming read of the buffer (16-byte loads); units = bytes read */
    MSDA_MB_READ = 0,
    /* copy of the buffer's first half into its second half; units = bytes read + written */
    MSDA_MB_COPY = 1,
    /* no-return fp32 global atomic adds, each wavefront instruction covering two whole
     * 128-byte rows picked at random among span / 128 rows; units = element adds */
    MSDA_MB_ATOMIC_F32 = 2,
    /* the same with packed bf16 pairs (four rows per instruction); units = pair adds */
    MSDA_MB_ATOMIC_PK_BF16 = 3,
    /* random 128-byte rows gathered by 8-lane groups (16 bytes per lane, 8 rows in flight
     * per lane, 4 FMAs per 16 bytes) from a span of `span` bytes at the buffer's head:
     * a span of 16 KiB stays in the vector L1, 45 MiB is the size of an encoder-scale
     * value tensor; units = bytes gathered */
    MSDA_MB_GATHER_GLOBAL = 4,
    /* the same gather from a 64 KiB copy in LDS; units = bytes gathered */
    MSDA_MB_GATHER_LDS = 5,
    /* no-return LDS fp32 atomic adds (ds_add_f32) to random words of 64 KiB; units =
     * lane adds */
    MSDA_MB_LDS_ATOMIC_F32 = 6
} msda_microbench;

/*
 * Run microbenchmark `kind` on the caller's device buffer `buf` (`bytes` bytes,
 * 256-byte aligned, at least 1 MiB; its contents are overwritten; the last 4 KiB
 * serve as a sink).  `span`: for the atomic kinds, the bytes of the row set the
 * adds land on (a power of two, at least 128, at most the buffer); for
 * MSDA_MB_GATHER_GLOBAL, the gathered span (a power of two from 4 KiB to 1 GiB,
 * at most the buffer); ignored otherwise.  One warm-up launch, then `reps`
 * launches back to back on `stream`, bracketed by two HIP events; the call
 * waits for them.  Writes the mean milliseconds per launch and the units one
 * launch processes.  Returns 0, 1 for invalid arguments (nothing enqueued), or
 * 2 for a failed HIP call.
 */
int msda_microbench_run(msda_microbench kind, void *buf, size_t bytes, size_t span, int reps,
                        void *stream, double *ms_per_launch, double *units_per_launch);

#ifdef __cplusplus
}
#endif

#endif /* MSDA_BENCH_H */
