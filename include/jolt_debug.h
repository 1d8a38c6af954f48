/*
 * jolt_debug.h -- measurement and inspection entry points of libjolt.so.
 * Not part of the compression API; used by the benchmark and the tests.
 */
#ifndef JOLT_DEBUG_H
#define JOLT_DEBUG_H

#include "jolt.h"

#ifdef __cplusplus
extern "C" {
#endif

/* Runs the factor stages of jolt_build_tables once (same arguments and workspace),
 * then launches the fused score pass `reps` times between two HIP events recorded
 * on `stream` (the stream the score kernels are launched on), and returns the mean
 * duration of one score launch in *ms_out.  Synchronises `stream`. */
jolt_status jolt_debug_score_pass(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                                  const void* const* omega_dev, void* workspace, size_t workspace_bytes,
                                  int32_t reps, jolt_stream_t stream, double* ms_out);

/* Launch timer of one kernel of the path, for the benchmark.  kernel: 0 = the fused
 * score pass of jolt_build_tables.  jolt_debug_timer_enable(kernel, 1) makes every
 * later launch of that kernel record a HIP event before and after it on the stream it
 * is launched on; jolt_debug_timer_read synchronises those events, returns the summed
 * duration in *total_ms and the number of timed launches in *launches, and clears the
 * record.  Host-side state of the library (not thread-safe against concurrent builds);
 * enabling adds two event records per launch and changes no results. */
jolt_status jolt_debug_timer_enable(int32_t kernel, int32_t enable);
jolt_status jolt_debug_timer_read(int32_t kernel, double* total_ms, int32_t* launches);

/* Copies `bytes` bytes of the workspace region `which` after a build into host memory:
 * 0 = U_d (fp64 [n_tables][D][32]), 1 = stored U_T (fp16 [n_tables][5][T][32]),
 * 2 = stored cores of the r_d chains (fp16 [n_tables][5][N][32][D]),
 * 3 = stored core of the full-token chain (fp16 [n_tables][N][T][32]); working precision
 * (fp32, or fp64 when the factors run in fp64) intermediates of the token factor:
 * 4 = token Grams [n_tables][5][T][T] (exact mode), 5 and 6 = subspace blocks
 * [n_tables * 5][T][64] (exact) or [.][T][40] (randomized), 7 = Rayleigh-Ritz / B B^T
 * matrices (fp64 [n_tables * 5][64 or 40]^2), 8 = their top-32 eigenvectors
 * [n_tables * 5][64 or 40][32], 9 = U_T [n_tables * 5][T][32], 10 = the row-chunk Gram
 * partials of the last orthonormalisation (fp64 [batch][chunks][64 or 40]^2). */
jolt_status jolt_debug_read(const jolt_config* cfg, const void* workspace, int32_t which, void* host_out,
                            size_t bytes);

#ifdef __cplusplus
}
#endif
#endif /* JOLT_DEBUG_H */
