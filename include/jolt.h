/*
 * jolt.h -- C ABI of the JoLT KV-cache candidate-table engine for MI355X (gfx950).
 *
 * The engine implements the method described on the pages about arXiv:2607.12550
 * ("A JoLT for the KV cache"):
 *   [JTRA] "Joint Tucker-rank and residual-bit KV allocator": Formulas (residual and
 *          decoded cache; normalised distortion D; Lagrangian; byte cost C),
 *          Mathematical statement, Implementation notes (grid
 *          r_T in {4,8,16,32,T}, r_d in {4,8,16,32,D}, b in {0,2,4,8}; candidate
 *          tables per group and K/V; binary search on lambda; storage-exact bytes).
 *   [RTR]  "Rotated Tucker residual for outlier-resistant KV quantization": Key
 *          formulas (Y = QR, block quantizer Q_b, decode), Implementation notes
 *          (normalized Hadamard rotation, blocks of 64 or 128 values).
 *   [TS]   "Technical Summary: A JOLT for the KV Cache": Methodology 1 (partial
 *          Tucker by ST-HOSVD), 2 (rotated residual), 3 (joint Lagrangian
 *          allocation), 4 (FlashJoLT randomized token-mode SVD).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * A "table" is one (layer group g, cache kind c) tensor X in bf16, shape [N, T, D]
 * row-major (D fastest), where N = layers-in-group x heads (never compressed),
 * T = tokens, D = head width.  Table index t = 2*g + c (c: 0 = K, 1 = V) by
 * convention of the caller; the library treats tables independently.
 *
 * Candidate index i = (i_rT * 5 + i_rd) * 4 + i_b over the ascending grids above,
 * so i = 99 is (T, D, 8).  r_T = T and r_d = D mean the identity factor (nothing
 * stored); (T, D) stores X verbatim and has distortion 0.
 *
 * Memory: every buffer is owned by the caller.  "dev" pointers are device memory
 * of the current HIP device, "host" pointers are host memory.  The library never
 * allocates device memory: the caller passes a workspace whose size is obtained
 * from jolt_workspace_size().  Functions that take a hipStream_t enqueue their
 * work on that stream; jolt_build_tables synchronises it (it returns host tables).
 * jolt_build_tables copies its small results back through one pinned host buffer per
 * host thread (hipHostMalloc, grown when a larger configuration needs it, held until
 * the process ends; pageable memory is used if it cannot be allocated).
 *
 * Errors: every function returns a jolt_status and never throws across the ABI.
 * Output buffers are written only when JOLT_OK is returned, except that device
 * outputs of the asynchronous calls may be partially written when a later device
 * error is reported.
 */
#ifndef JOLT_H
#define JOLT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct ihipStream_t* jolt_stream_t; /* identical to hipStream_t */

typedef enum {
  JOLT_OK = 0,
  JOLT_EINVAL = -1,      /* bad argument or unsupported configuration            */
  JOLT_ENOMEM = -2,      /* workspace too small                                  */
  JOLT_EDEVICE = -3,     /* a HIP runtime call failed                            */
  JOLT_EINFEASIBLE = -4, /* even the cheapest candidate of every table exceeds B */
  JOLT_ERANGE = -5,      /* a stored fp16 core/factor value would overflow fp16  */
  JOLT_ENONFINITE = -6   /* the input tensor contains Inf or NaN                 */
} jolt_status;

typedef enum { JOLT_TOKEN_EXACT = 0, JOLT_TOKEN_RANDOMIZED = 1 } jolt_token_mode;

enum { JOLT_N_RT = 5, JOLT_N_RD = 5, JOLT_N_B = 4, JOLT_N_CAND = 100, JOLT_MAX_TABLES = 64 };

typedef struct {
  int32_t N;            /* slices per table (layers in group x heads), 1..65536        */
  int32_t T;            /* tokens; power of two, 64..65536                             */
  int32_t D;            /* head width; 64 or 128                                       */
  int32_t n_tables;     /* 1..JOLT_MAX_TABLES                                          */
  int32_t quant_block;  /* values per quantization block; must equal D                 */
  int32_t s_bytes;      /* bytes per stored factor/core value; must be 2 (fp16)        */
  int32_t align_bytes;  /* section alignment of a record; must be 256                  */
  int32_t token_mode;   /* jolt_token_mode                                             */
  int32_t q_cap;        /* token directions kept by the randomized finder; must be 32  */
  int32_t oversample;   /* extra sketch columns; must be 8                             */
  int32_t power_iters;  /* randomized subspace iterations; 0..4                        */
  int32_t exact_iters;  /* exact mode, T > 128: subspace iterations (64 columns) before the
                           first Ritz-residual test (12)                                  */
  int32_t factor_precision; /* factor-stage arithmetic: 0 auto (fp64 when N*T*D <= 2^20),
                               1 fp64, 2 fp32-accurate (fp16 hi/lo MFMA, fp64 block sums) */
  int32_t exact_max_iters;  /* exact mode, T > 128: most subspace iterations in total
                               (exact_iters..256, default 64); see jolt_last_build_info  */
} jolt_config;

/* Default configuration for the given shape (exact mode, first residual test after 12
 * subspace iterations and at most 64 in total, q_cap 32, oversample 8, 2 power iterations,
 * block D, fp16 storage, 256 alignment, automatic factor precision). */
void jolt_default_config(jolt_config* cfg, int32_t N, int32_t T, int32_t D, int32_t n_tables);

/* Human-readable name of a status code (static string). */
const char* jolt_status_string(jolt_status s);

/* Device workspace bytes needed by jolt_build_tables and jolt_encode for cfg.
 * Host-only; no device call. */
jolt_status jolt_workspace_size(const jolt_config* cfg, size_t* bytes_out);

/* Storage-exact byte cost of every candidate ([JTRA] Formulas, cost display, with
 * the Implementation notes' "actual storage": header 256 B, fp16 factors shared by
 * the N slices, fp16 core, packed b-bit codes, fp32 scale per block, every section
 * padded to align_bytes).  C_out: host uint64[100].  Host-only. */
jolt_status jolt_cost_table(const jolt_config* cfg, uint64_t* C_out);

/* Candidate table of every table ([JTRA] Implementation notes: partial Tucker on the
 * token and feature unfoldings, reconstruct, residual, fixed orthogonal transform,
 * quantize, normalised Frobenius distortion).
 *   x_dev      host array [n_tables] of device pointers to bf16 [N, T, D]
 *   signs_dev  device int8 [n_tables, D], entries +1/-1: the random signs sigma of
 *              the rotation Q = H_D diag(sigma) / sqrt(D) of each table
 *   omega_dev  randomized mode only (else NULL): host array [n_tables] of device
 *              pointers to bf16 sketch matrices, concatenated over r_d = 4, 8, 16,
 *              32, D: block r_d is [N * r_d, q_cap + oversample] row-major, row
 *              n * r_d + j multiplies column (n, j) of the token unfolding
 *   D_out      host double [n_tables, 100]: normalised distortion of the stored
 *              representation ||X - X^||^2 / ||X||^2 (0 when ||X|| = 0)
 *   C_out      host uint64 [n_tables, 100]: bytes (same for every table)
 *   xnorm2_out host double [n_tables] or NULL: ||X||^2 of the bf16 input
 * Synchronises `stream`.  Inputs are not modified. */
jolt_status jolt_build_tables(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                              const void* const* omega_dev, double* D_out, uint64_t* C_out,
                              double* xnorm2_out, void* workspace, size_t workspace_bytes,
                              jolt_stream_t stream);

/* How the token factors of the last call that computed factors in `workspace`
 * (jolt_build_tables, jolt_model_tables or jolt_encode) were obtained.  Exact mode with
 * T > 128 runs subspace iteration in rounds: exact_iters iterations, then Rayleigh-Ritz and
 * the residual ||M u_i - theta_i u_i|| of the 32 leading Ritz pairs of every token Gram M
 * (the converged top eigenpairs the exact mode stands for).  A problem converges when its
 * largest residual is at most 1e-6 of its leading Ritz value.  Further rounds, sized from the
 * measured contraction per iteration (0.5 assumed before two residuals of a problem are
 * known), run while a problem is above that and still
 * contracting, up to exact_max_iters; a round that leaves a residual above 0.8 of its
 * previous value marks the floor of the working precision (about 1e-6 with fp32
 * products), and such a problem counts as converged if the floor is below 1e-5.
 *   iterations     subspace iterations of the exact mode (0 for T <= 128, where a direct
 *                  eigensolver runs); power_iters in randomized mode
 *   max_residual   largest relative Ritz residual left over all (table, r_d) problems
 *                  (0 where not computed)
 *   converged      1 if every problem converged as above (always 1 outside the exact
 *                  subspace iteration)
 * Host-only; JOLT_EINVAL if no call has computed factors in this workspace. */
typedef struct {
  int32_t iterations;
  int32_t converged;
  double max_residual;
} jolt_factor_info;
jolt_status jolt_last_build_info(const void* workspace, jolt_factor_info* info_out);

/* Budget-feasible allocation ([JTRA] Mathematical statement and Implementation
 * notes: for a price lambda every table takes argmin D + lambda*C independently;
 * lambda is searched until the allocation fits).  lambda+ = inf{lambda : sum C <= B}
 * is one of the slopes between consecutive vertices of the tables' lower convex hulls
 * of (C, D); a binary search over those slopes finds it exactly, and z*(lambda) is
 * returned at lambda = lambda+ (1 + 1e-12), just above the tie; ties go to the lower C,
 * then the lower index.
 *   D, C         host [n_tables, n_cand]
 *   choice_out   host int32 [n_tables]
 *   lambda_out   host double (may be NULL)
 *   total_out    host uint64 sum of chosen costs (may be NULL)
 * Host-only and pure. */
jolt_status jolt_allocate(const double* D, const uint64_t* C, int32_t n_tables, int32_t n_cand,
                          uint64_t budget_bytes, int32_t* choice_out, double* lambda_out,
                          uint64_t* total_out);

/* Modelled candidate tables from spectra only (the separable error model D ~ eps^2(b) tau
 * that the allocation of "A JoLT for the KV cache" optimises, with eps^2(b) calibrated on a
 * Gaussian round trip; "Technical Summary: A JOLT for the KV Cache", Methodology 4:
 * FlashJoLT tail-mass accounting).  The factor stages run as in jolt_build_tables up to the
 * feature and token eigenvalues; no cores, reconstruction or residual pass.
 *   D(z) = eps^2(b) * tau(r_T, r_d); tau = 1 - E/||X||^2 with E the energy of the top r_T
 *   token eigen-directions of Y(r_d) (randomized mode: those B = Q^T A captures; what the
 *   sketch misses counts as residual), the top r_d feature directions when r_T = T, 0 for
 *   (T, D); eps^2(0) = 1, eps^2(b) = sum |g - Q_b(g)|^2 / sum |g|^2 over the rows of
 *   gauss_dev, one quantization block per row.
 *   gauss_dev    device fp32 [gauss_rows, D] standard normal rows, 1 <= gauss_rows <= 65536
 *   eps2_out     host double [4]: eps^2 for b = 0, 2, 4, 8 (may be NULL)
 *   other arguments and errors as for jolt_build_tables (same workspace size).
 * Synchronises the stream.  Writes the workspace without cores: a later jolt_encode_built
 * on it returns JOLT_EINVAL until jolt_build_tables or jolt_encode has run again. */
jolt_status jolt_model_tables(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                              const void* const* omega_dev, const float* gauss_dev, int32_t gauss_rows,
                              double* D_out, uint64_t* C_out, double* xnorm2_out, double* eps2_out,
                              void* workspace, size_t workspace_bytes, jolt_stream_t stream);

/* Greedy improvement of a budget-feasible allocation ("Joint Tucker-rank and
 * residual-bit KV allocator", Implementation notes: after the price search, swap
 * candidates with the best distortion reduction per added byte).  A move replaces one
 * table's candidate by one of strictly lower distortion whose added cost keeps the
 * total within budget_bytes; the best move is applied until none is left.  Moves adding
 * no bytes rank first (larger reduction first), the others by
 * (D_cur - D_new) / (C_new - C_cur) in fp64; ties go to the lower table, then the lower
 * candidate index.
 *   D, C          host [n_tables, n_cand] (as for jolt_allocate)
 *   choice_inout  host int32 [n_tables]: the starting allocation, replaced by the result
 *   total_out     host uint64 sum of the resulting costs (may be NULL)
 *   moves_out     host int32: number of moves applied (may be NULL)
 * JOLT_EINVAL for a choice outside [0, n_cand), non-finite or negative D, or a start
 * above the budget (choice_inout is then unchanged).  Host-only and pure. */
jolt_status jolt_refine_swap(const double* D, const uint64_t* C, int32_t n_tables, int32_t n_cand,
                             uint64_t budget_bytes, int32_t* choice_inout, uint64_t* total_out,
                             int32_t* moves_out);

/* Fixed baseline allocation (same page, Implementation notes: fixed-rank or fixed-bit
 * baselines; the pages' toy baseline gives every group the same (r_T, r_d, b)): one
 * candidate index shared by all tables, the allowed candidate of least total
 * distortion whose total cost fits budget_bytes (ties: lower total cost, then lower
 * index).  Total distortion is summed over tables in table order in fp64.
 *   allowed       host uint8 [n_cand], nonzero = candidate allowed (NULL: all)
 *   cand_out      host int32 candidate index
 *   total_out     host uint64 total cost (may be NULL)
 *   dist_out      host double total distortion (may be NULL)
 * JOLT_EINFEASIBLE when no allowed candidate fits.  Host-only and pure. */
jolt_status jolt_allocate_common(const double* D, const uint64_t* C, int32_t n_tables, int32_t n_cand,
                                 uint64_t budget_bytes, const uint8_t* allowed, int32_t* cand_out,
                                 uint64_t* total_out, double* dist_out);

/* Bytes of the record of candidate `cand` (equals C[cand]).  Host-only. */
jolt_status jolt_record_bytes(const jolt_config* cfg, int32_t cand, uint64_t* bytes_out);

/* Compressed record of every table at its chosen candidate ([RTR] Implementation
 * notes: store Tucker factors, core, per-block scale and integer codes).  The
 * factors are recomputed with the same kernels as jolt_build_tables, so they are
 * bitwise those the table was scored with.  X~ and the residual R = X - X~ are formed in
 * fp64; the rotation, scale and codes in fp32 (their errors scale with |R|: about 1e-5 of
 * the codes differ by one from an exact evaluation).
 *   choice     host int32 [n_tables] candidate indices
 *   rec_dev    host array [n_tables] of device pointers, each >= C[choice] bytes
 * Record layout (little-endian): 256-byte header {u32 magic "JOLT", u32 version 1,
 * i32 N, T, D, r_T, r_d, b, blk, flags; u64 total bytes, offsets of the U_T, U_d,
 * core, codes and scales sections (0 if absent); at byte 128 the sign bits, bit i
 * set when sigma_i = -1}, then 256-aligned sections: U_T fp16 [T, r_T] (r_T < T),
 * U_d fp16 [D, r_d] (r_d < D), core fp16 [N, r_T, r_d] (or X bf16 [N, T, D] for
 * (T, D)), codes (b > 0) b-bit two's complement packed little-endian in row-major
 * element order, scales (b > 0) fp32 [N, T, D / blk].
 * Asynchronous on `stream`. */
jolt_status jolt_encode(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                        const void* const* omega_dev, const int32_t* choice, void* const* rec_dev,
                        void* workspace, size_t workspace_bytes, jolt_stream_t stream);

/* The same records as jolt_encode without recomputing the factors: the Tucker factors
 * and cores are taken from `workspace`, where the last successful jolt_build_tables
 * (or jolt_encode) on that workspace left them.  This follows the method's order
 * ([JTRA] Implementation notes: candidate tables from one calibration pass, a choice
 * per group and K/V, then storage of the chosen candidate), computing the factors once.
 * Precondition: the previous call that wrote `workspace` was a successful
 * jolt_build_tables or jolt_encode with an identical cfg, the same x_dev and signs_dev
 * pointers and the same workspace_bytes, and neither the inputs nor the workspace were
 * modified since.  The pointer and config part of this is checked on the host (a
 * registry keyed by the workspace address); a mismatch returns JOLT_EINVAL and writes
 * nothing.  Contents cannot be checked: changed inputs give records of the old factors
 * with the new residual.
 *   x_dev, signs_dev, choice, rec_dev, stream as for jolt_encode (no sketch needed).
 * Asynchronous on `stream`; errors as jolt_encode plus the precondition check. */
jolt_status jolt_encode_built(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                              const int32_t* choice, void* const* rec_dev, void* workspace,
                              size_t workspace_bytes, jolt_stream_t stream);

/* Decoded cache X^ = X~ + Q^T Q_b(Q R) rounded to bf16 (RNE) ([JTRA] Formulas, first
 * display; [RTR] Implementation notes: multiply codes by the scale, inverse
 * transform, add X~; b = 0 returns X~).
 *   rec_dev    host array [n_tables] of device pointers to records made by jolt_encode
 *   choice     host int32 [n_tables] the candidates the records were made with
 *   xhat_dev   host array [n_tables] of device pointers to bf16 [N, T, D] outputs
 * Asynchronous on `stream`; needs no workspace. */
jolt_status jolt_decode(const jolt_config* cfg, const void* const* rec_dev, const int32_t* choice,
                        void* const* xhat_dev, jolt_stream_t stream);

/* Attention over layer groups' compressed K and V, decoded inside the attention
 * ("Joint Tucker-rank and residual-bit KV allocator", Implementation notes:
 * reconstruct the low-rank part and the residual immediately before attention,
 * preferably in a fused kernel).  For group g, slice n (layer x KV head), query i:
 *   O_g[n, i, :] = sum_t softmax_t(scale * Q_g[n, i, :] . K^_g[n, t, :]) V^_g[n, t, :]
 * where K^_g and V^_g are, bit for bit, the bf16 caches jolt_decode would write from
 * the group's two records; they are rebuilt tile by tile in LDS and never stored.
 * Scores, softmax and the weighted sum are fp32.
 *   n_groups       number of groups (>= 1)
 *   rec_k, rec_v   host arrays [n_groups] of device pointers to the K and V records
 *                  (made by jolt_encode with the same config); cand_k, cand_v host int32
 *                  [n_groups], their candidates
 *   q_dev          host array [n_groups] of device bf16 [N, nq, D], 1 <= nq <= 16
 *                  (queries per slice, e.g. the query heads sharing a KV head)
 *   scale          score scale (1/sqrt(D) for standard attention)
 *   o_dev          host array [n_groups] of device fp32 [N, nq, D] outputs
 *   workspace      device scratch of at least jolt_attend_workspace_size bytes
 * Asynchronous on `stream`.  JOLT_EINVAL for a bad config, count, candidate, nq, pointer
 * or a short workspace. */
jolt_status jolt_attend_workspace_size(const jolt_config* cfg, int32_t n_groups, int32_t nq, size_t* bytes_out);
jolt_status jolt_attend(const jolt_config* cfg, int32_t n_groups, const void* const* rec_k, const int32_t* cand_k,
                        const void* const* rec_v, const int32_t* cand_v, const void* const* q_dev, int32_t nq,
                        float scale, float* const* o_dev, void* workspace, size_t workspace_bytes,
                        jolt_stream_t stream);

/* Streaming admission of incoming token blocks against frozen records ("Rotated Tucker
 * residual for outlier-resistant KV quantization", Implementation notes: keep the Tucker
 * factors and form R = X - X~ for each incoming token block; "Joint Tucker-rank and
 * residual-bit KV allocator", Implementation notes: at KV-cache admission time).
 * A record made by jolt_encode is frozen: its feature factor, cores and rotation stay
 * fixed.  For an incoming block X' [N, t', D] of the same table the token rows L of the
 * block are the least-squares fit of every token against the record's reconstruction
 * operator (X~'_n = L R_n):
 *   r_T < T:  one row per token shared by the slices, R_n = G_n U_d^T (G_n if r_d = D),
 *             L [t', r_T];
 *   r_T = T:  one row per token and slice, R = U_d^T, L [N, t', r_d];
 *   (T, D):   the block is stored verbatim.
 * L = P A+ with P = sum_n X'_n R_n^T and A = sum_n R_n R_n^T in fp64; A+ keeps the
 * eigen-directions of A above 1e-12 of its largest eigenvalue (the minimum-norm solution
 * when the operator is rank deficient).  L is stored as fp16 (RNE) and the rotated residual
 * X' - L R as b-bit codes and fp32 scales, exactly as jolt_encode does for its rows.
 *
 * Block record: 256-byte header (uint32 words: 0 magic 0x42544C4A "JLTB", 1 version 1,
 * 2 N, 3 t', 4 D, 5 r_T, 6 r_d, 7 b, 8 quantization block (= D), 9 T of the frozen record;
 * words 10-17 little-endian uint64 total bytes, offsets of L, codes and scales; word 18
 * flags, bit 0 = an L value overflowed fp16), then 256-aligned sections: L fp16 (or the
 * verbatim bf16 block), packed b-bit two's-complement codes in row-major element order,
 * fp32 scales [N, t'].  Codes and scales are absent when b = 0.
 *
 * t' (t_new) is a multiple of 64 in [64, 65536].  Every pointer argument holds one entry
 * per table of cfg (n_tables), as in jolt_decode; cand[t] is the candidate record t was
 * made with.  Records, blocks, inputs and outputs are 16-byte aligned device buffers. */

/* Bytes of one table's frozen state (A+ and the eigenvalues of A, fp64). */
jolt_status jolt_stream_state_bytes(size_t* bytes_out);
/* Bytes of the block record of candidate `cand` for t_new tokens. */
jolt_status jolt_stream_block_bytes(const jolt_config* cfg, int32_t cand, int32_t t_new, uint64_t* bytes_out);
/* Device workspace of jolt_stream_encode for t_new tokens (per-workgroup error sums). */
jolt_status jolt_stream_workspace_size(const jolt_config* cfg, int32_t t_new, size_t* bytes_out);

/* Freeze: compute each table's state from its record (once per record; A from the stored
 * fp16 factors, Jacobi eigendecomposition, pseudo-inverse).
 *   state_dev  host array of device pointers to jolt_stream_state_bytes each (8-byte aligned)
 * Asynchronous on `stream`.  JOLT_EINVAL for a bad config, candidate or pointer. */
jolt_status jolt_stream_prepare(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                                void* const* state_dev, jolt_stream_t stream);

/* Encode one incoming block per table against its frozen record and state.
 *   xnew_dev   host array of device pointers to bf16 [N, t_new, D]
 *   block_dev  host array of device pointers to jolt_stream_block_bytes each
 *   dist_dev   device double [n_tables] or NULL: ||X' - X^'||^2 / ||X'||^2 of each block
 *              (X^' in fp64 before the bf16 rounding of decode; 0 for an all-zero block or
 *              a verbatim record; NaN when an L value overflowed fp16)
 *   workspace  device scratch of at least jolt_stream_workspace_size bytes (8-byte aligned)
 * Asynchronous on `stream` (overflow is reported in the block header and dist_dev, not by
 * the return code).  JOLT_EINVAL for a bad config, t_new, candidate or pointer;
 * JOLT_ENOMEM for a short workspace. */
jolt_status jolt_stream_encode(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                               const void* const* state_dev, const void* const* xnew_dev, int32_t t_new,
                               void* const* block_dev, double* dist_dev, void* workspace, size_t workspace_bytes,
                               jolt_stream_t stream);

/* For callers that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops on the cache write path, harnesses that forbid hipMalloc): the same encode
 * as jolt_stream_encode, with the workspace taken from a scratch array that the library
 * holds in device memory, JOLT_NOALLOC_SCRATCH_BYTES per device (a static device array of
 * the code object: each device the library runs on holds its copy until the process ends).
 * It calls no hipMalloc, hipFree or allocating library routine; the first call on a device
 * looks up that device's scratch address once.
 *   Limit: jolt_stream_workspace_size(cfg, t_new) <= JOLT_NOALLOC_SCRATCH_BYTES (e.g.
 *   16 tables of N >= 8 slices up to t_new = 960), else JOLT_ENOMEM before any device work.
 *   Every call on a device shares that device's scratch: calls that overlap on one device
 *   (on different streams, or from different host threads) race and must be serialised by
 *   the caller.  The scratch keeps the last call's partial sums; every value a call reads
 *   there it has written itself first.
 * Other arguments, errors and results are those of jolt_stream_encode. */
#define JOLT_NOALLOC_SCRATCH_BYTES (32u << 20)
jolt_status jolt_stream_encode_noalloc(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                                       const void* const* state_dev, const void* const* xnew_dev, int32_t t_new,
                                       void* const* block_dev, double* dist_dev, jolt_stream_t stream);

/* Decoded block X^' = L R + Q^T Q_b(Q R') rounded to bf16 (RNE), with the same tile
 * arithmetic as jolt_decode.
 *   out_dev    host array of device pointers to bf16 [N, t_new, D]
 * Asynchronous on `stream`; needs no workspace. */
jolt_status jolt_stream_decode(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                               const void* const* block_dev, int32_t t_new, void* const* out_dev,
                               jolt_stream_t stream);

#ifdef __cplusplus
}
#endif
#endif /* JOLT_H */
