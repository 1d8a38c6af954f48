// Internal interfaces between the host orchestration and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "common.h"

namespace jolt {

// ---------------------------------------------------------------- generic GEMM
struct GemmOperand {
  const void* p;    // base pointer (ignored when tbl != 0)
  int32_t tbl;      // 1: base = table pointer [b / bdiv]
  int32_t type;     // 0 fp32, 1 bf16, 2 fp16, 3 fp64
  int32_t bdiv;     // batch index b -> (b / bdiv, b % bdiv)
  int64_t sb1, sb2; // element strides of the two batch parts
  int32_t rsh;      // row r -> (r >> rsh) * sr1 + (r & (2^rsh - 1)) * sr2
  int64_t sr1, sr2;
  int32_t ksh;      // k -> (k >> ksh) * sk1 + (k & (2^ksh - 1)) * sk2
  int64_t sk1, sk2;
  int32_t lmode;    // load pattern, set by launch_gemm: 0 generic, 1 8-wide along k, 2 along rows
  int64_t off0;     // constant element offset added to the base
  int32_t novar;    // 1: the operand ignores the variant digit of the batch index (see GemmArgs)
};

struct GemmVariant {
  GemmOperand A;  // rows = m
  GemmOperand B;  // rows = n
  int32_t M, N, K;
};

struct GemmArgs {
  GemmVariant v[6];
  int32_t nvar;  // variant = (b / vdiv) % nvar; operands with novar see
  int32_t vdiv;  // b' = (b / (vdiv * nvar)) * vdiv + b % vdiv instead of b
  void* C;
  int32_t c_type;  // 0 fp32, 1 fp64
  int32_t cbdiv;
  int64_t csb1, csb2, csm, csn;
  const void* Cin;
  _Float16* C16;
  int32_t* flags;
  float alpha;
  const double* alpha_norm;
  int32_t alpha_div;
  int32_t acc64;
  int32_t mode;     // GEMM_SPLIT, GEMM_BF16 or GEMM_F64
  // checkpoints (split / bf16 modes): after k reaches ck[i] (a multiple of 32, < K) the
  // partial result is also stored at C + (i - nck) * ck_stride elements, i.e. the final
  // result at C and the checkpoints below it
  int32_t nck;
  int32_t ck[3];
  int64_t ck_stride;
  // split-K: with a scratch buffer, launch_gemm may split K over ksplit workgroups per
  // tile (workgroup z: batch z / ksplit, k slice z % ksplit) that write raw partial sums
  // [batch][ksplit][pm][pn] (fp64 with acc64, else fp32) to `scratch`; a second kernel adds
  // the slices in order and applies the epilogue (alpha, Cin, C, C16, flags)
  void* scratch;
  int64_t scratch_bytes;
  int32_t ksplit;  // set by launch_gemm
  int32_t pm, pn;  // set by launch_gemm
  // XCD grouping: when xgrp > 0, the tiles of every xgrp consecutive batches (a unit that
  // shares operands) are dispatched to one XCD, so the shared operand is fetched into one
  // L2.  Workgroups go to the 8 XCDs round-robin by linear index; launch_gemm falls back to
  // the plain order when the units do not divide evenly.
  int32_t xgrp;
};
enum { GEMM_SPLIT = 0, GEMM_BF16 = 1, GEMM_F64 = 2 };

hipError_t launch_gemm(const GemmArgs& g, const TablePtrs& tp, int batch, hipStream_t s);

// fp16 cores of the five r_d chains of every table (fp32 working precision, D = 128):
// G16[t][cc][n][0..31][0..r_d) = U_T(t, cc)^T Y_n(r_d), UT fp32 [t][5][T][32], Y32 fp32
// [t][N][T][32], X (r_d = D chain) the bf16 tables tp.p[t]
// feature projection Y32 [ntab][N][T][32] = X U_d (fp32 working precision) with its fp16
// copy G16T and, when YT is given (N <= 32), YT[t][tk][j * N + n] = Y[t][n][tk][j]
hipError_t launch_project(const TablePtrs& tp, const float* Ud32, int N, int T, int D, int ntab, float* Y32,
                          _Float16* G16T, float* YT, int32_t* flags, hipStream_t s);

// With Wh (and Wl, V32 [ntab][D][32], signs [ntab][D]) the kernel also writes the rotated
// reconstruction operands of the score pass, as launch_prep_w would
// randomized finder, r_d = D chain: P[t][n D + f][c] = sum_tk X_t[n][tk][f] S[t][tk][c]
// (c < 40; S at S + t * s_tab, P at P + t * p_tab, fp32), through k-slice partials `part`
// of ntab * N * xts_slices(T) * D * 40 floats
int xts_slices(int T);
hipError_t launch_xts(const TablePtrs& tp, const float* S, int64_t s_tab, int N, int T, int D, int ntab,
                      float* part, float* P, int64_t p_tab, hipStream_t s);

// randomized finder, chains r_d = 4 << cc < D: P[t][cc][n r_d + j][c] = sum_tk Y[t][n][tk][j]
// S[t][cc][tk][c] (j < r_d, c < 40; S chain blocks [T][40], P chain blocks of p_chain floats),
// through partials `part` of ntab * N * xts_slices(T) * 4 * 32 * 40 floats
hipError_t launch_yts(const float* Y, const float* S, int N, int T, int ntab, float* part, float* P,
                      int64_t p_chain, hipStream_t s);

// randomized finder, r_d = D chain: S[t][tk][c] = sum_{n, f} X_t[n][tk][f] B[t][n D + f][c]
// (c < 40) from B^T (rows c of stride b_ld, table stride b_tab; bf16 with exact products,
// or fp32 split into fp16 hi/lo), the generic GEMM's arithmetic; S fp32, table stride s_tab
// S of the randomized finder's r_d < D chains (all four from one pass over Y32): BT the
// transposed operand (fp32 or bf16), chain cc at element offset boff[cc] (4 entries)
hipError_t launch_yw4(const float* Y, const void* BT, bool bf16, int64_t b_tab, int64_t b_ld, const int64_t* boff,
                      int N, int T, int ntab, float* S, int64_t s_tab, int64_t s_chain, hipStream_t s);
hipError_t launch_xw(const TablePtrs& tp, const void* BT, bool bf16, int64_t b_tab, int64_t b_ld, int N, int T,
                     int D, int ntab, float* S, int64_t s_tab, hipStream_t s);

hipError_t launch_cores(const float* UT, const float* Y32, const TablePtrs& tp, int N, int T, int D, int ntab,
                        _Float16* G16, int32_t* flags, const float* V32, const int8_t* signs, _Float16* Wh,
                        _Float16* Wl, double* part, hipStream_t s);
// P_b = M_b Q_b for the exact subspace iteration (M_b [T][T] at M + (b / div) s1 + (b % div) s2,
// Q_b, P_b [T][64], fp32); with W, the Gram partials P^T P of the T / 64 row blocks
// ([batch][T / 64][64][64] fp64, both triangles)
hipError_t launch_mq(const float* M, int div, int64_t s1, int64_t s2, const float* Q, float* P, int T, int batch,
                     double* W, hipStream_t s);
// cores and reconstruction operands of the randomized token mode from the finder's last
// product P = A^T Q ([table][5][p_chain floats], rows n r_d + j, 40 columns) and the
// eigenvectors V ([table][5][40][32]) that form U_T = Q V (fp32 working precision, D = 128)
hipError_t launch_cores_rr(const float* V, const float* P, int64_t p_chain, int N, int D, int ntab, _Float16* G16,
                           int32_t* flags, const float* V32, const int8_t* signs, _Float16* Wh, _Float16* Wl,
                           hipStream_t s);
// token slices the core kernel splits each slice's tokens into (1: no partial sums), and the
// fp64 partial-sum doubles it then needs: nks * N * ntab * 26 tiles * 256
int cores_slices(int N, int T, int ntab);

// helpers to describe operands
inline GemmOperand op_plain(const void* p, int type, int64_t sb1, int64_t sr, int64_t sk) {
  GemmOperand o{};
  o.p = p; o.tbl = 0; o.type = type; o.bdiv = 1; o.sb1 = sb1; o.sb2 = 0;
  o.rsh = 30; o.sr1 = 0; o.sr2 = sr; o.ksh = 30; o.sk1 = 0; o.sk2 = sk;
  return o;
}

// ---------------------------------------------------------------- small dense kernels
// top-k eigenpairs of `batch` symmetric n x n fp64 matrices (n <= 128, k <= 32):
// eigenvalues descending; eigenvectors sign-normalised (largest |entry| positive).
// A: [batch][n][n] fp64; U64: [batch][n][k] fp64 (nullable); U32: [batch][n][k] fp32 (nullable);
// lam: [batch][k] (nullable)
hipError_t launch_syev_topk(const double* A, int n, int k, int batch, double* U64, float* U32,
                            double* lam, hipStream_t s);

// Partial Grams of the CholeskyQR passes: W[b][q] = Z_bq^T Z_bq in fp64, Z_bq the q-th of
// `nparts` equal row chunks of the row-major [rows][p] block b (fp32 or fp64 values;
// p <= 64, p % 4 == 0, rows % nparts == 0).  Output [batch][nparts][p][p].
hipError_t launch_gram64(const void* src, bool f64in, int64_t rows, int p, int nparts, int batch, double* W,
                         hipStream_t s);
// U[b][t][m] = sum_c S[b][t][c] V[b][c][m] for c < p (40 or 64), m < 32: fp32 rows and their fp16
// copy at (b / div) u1 + (b % div) u2 + 32 t (a token factor from its basis and eigenvectors)
hipError_t launch_ut_rows(const float* S, const float* V, int p, int T, int batch, float* U32, _Float16* U16,
                          int div, int64_t u1, int64_t u2, hipStream_t s);
// W[b][q] = Z_b^T P_b over row chunk q (fp32 [batch][rows][64] blocks, fp64 [64][64] partials)
hipError_t launch_gram_cross(const float* Z, const float* P, int64_t rows, int nparts, int batch, double* W,
                             hipStream_t s);
// out[b][i] = sum over q < nparts of W[(b nparts + q) len + i], in order (fp64)
hipError_t launch_sum_parts(const double* W, int nparts, int len, int batch, double* out, hipStream_t s);

// Cholesky W = R^T R of `batch` p x p fp64 Grams, summed from `nparts` partials
// [batch][nparts][p][p]; writes R^{-1} (upper) [batch][p][p] as fp32, or fp64 when f64out.
hipError_t launch_chol_inv(const double* Wparts, int nparts, int p, int batch, void* Rinv, bool f64out,
                           hipStream_t s);

// dst[b] = src[b] R_b^{-1} for fp32 [rows][p] blocks, R_b the Cholesky factor of the Gram
// summed from `nparts` fp64 partials [batch][nparts][p][p] (p <= 64, p % 4 == 0)
// (Rinv: fp32 [batch][p][p] scratch for the factors' inverses, required)
hipError_t launch_chol_apply(const double* Wparts, int nparts, int p, const float* src, float* dst, int64_t rows,
                             int batch, float* Rinv, hipStream_t s);

// Gaussian round trip of the block quantizer: part [rows][4] = (sum g^2, error sums at
// b = 2, 4, 8) of fp32 rows G [rows][D]
hipError_t launch_eps2(const float* G, int rows, int D, double* part, hipStream_t s);

// general entry of the eigensolver: input fp32 or fp64, outputs fp64 / fp32 / fp16 (nullable)
hipError_t launch_syev_topk_any(const void* A, bool f32in, int n, int k, int batch, double* U64, float* U32,
                                _Float16* U16, double* lam, hipStream_t s);

// sum `nparts` fp64 [D][D] partial Grams per table; xnorm2 = trace; flag non-finite.
// With upper_tiles the partials hold only the 16 x 16 tiles on and above the diagonal
// (launch_fgram) and each sum is stored at (m, n) and (n, m).
hipError_t launch_reduce_gram(const double* parts, int nparts, int D, int ntab, double* G, double* xn2,
                              int32_t* flags, hipStream_t s, bool upper_tiles = false);

// feature Gram partials parts[t][q] (fp64 [D][D], tiles on and above the diagonal) of the
// row chunks q < nchunk of `rows` rows of every bf16 table viewed as [N T][D]; the same
// values, bit for bit, as the generic GEMM's bf16 mode with fp64 flushes (D = 64 or 128)
hipError_t launch_fgram(const TablePtrs& tp, int64_t rows, int D, int nchunk, int ntab, double* parts,
                        hipStream_t s);

// token Gram of the tensor: M[t * msb + ...] = s sum_n X_n X_n^T (T x T fp32, s the power-of-two
// scale of the table's norm xn2[t]) for bf16 tables [N][T][128]; T a multiple of 128.  The sum
// over n is split into tgram_splits(N, T, nt) parts; when there are several, parts holds
// tgram_part_floats(N, T, nt) floats of partial sums (a second launch adds them)
int tgram_splits(int N, int T, int nt);
int64_t tgram_part_floats(int N, int T, int nt);
hipError_t launch_tgram(const TablePtrs& tp, int N, int T, int D, int nt, const double* xn2, float* M, int64_t msb,
                        float* parts, hipStream_t s);

// nested token Grams of the projection: M[t * msb + c * T * T] = s sum_{j < 4 * 2^c} sum_n
// y_{n,j} y_{n,j}^T (c = 0 .. 3, fp32 T x T) from the token-major copy YT [t][T][32][N] (fp32,
// N = 32; split fp16 arithmetic); T a multiple of 128
hipError_t launch_tgram_y(const float* YT, int N, int T, int nt, const double* xn2, float* M, int64_t msb,
                          hipStream_t s);

// feature factor products: Ud32 = fp32(U_d[:, :32]); Ud16 = fp16(U_d[:, :32]);
// V32[:, j] = Q Ud16[:, j] (normalised random-sign Hadamard); V split into negated
// fp16 hi/lo [D][32] for the score kernel.
hipError_t launch_prep_feature(const double* Ud64, const int8_t* signs, int D, int ntab, float* Ud32,
                               _Float16* Ud16, float* V32, _Float16* Vneg_hi, _Float16* Vneg_lo,
                               hipStream_t s);

// YT[t][tk][j * N + n] = Y[t][n][tk][j] for fp32 Y [ntab][N][T][32] (N <= 256)
hipError_t launch_transpose_y(const float* Y, int N, int T, int ntab, float* YT, hipStream_t s);
// dst[b][c][t] = src[b][t][c] for the slices b = table * N + n ([T][C] each, C % 8 == 0):
// src from the bf16 tables tp (tp != nullptr) or one contiguous buffer
hipError_t launch_transpose_tc(const TablePtrs* tp, const void* src, bool bf16, int N, int T, int C, int ntab,
                               void* dst, hipStream_t s);

// deterministic start block for the exact token subspace iteration: [batch][T][64]
hipError_t launch_init_subspace(void* Q, bool f64, int T, int batch, hipStream_t s);

// res[b] = max_i ||(P_b - theta_i Z_b) v_i|| / theta_0 over the 32 Ritz pairs of problem b:
// P, Z [batch][T][p], V [batch][p][32] in working precision, lam [batch][32] fp64; part
// (batch * T / 64 * 32 doubles, nullable) holds row-chunk partial sums for the fp32, p = 64 case
hipError_t launch_ritz_residual(const void* P, const void* Z, const void* V, bool f64, const double* lam, int T,
                                int p, int batch, double* res, double* part, hipStream_t s);

// W_rot for the r_d chains: for chain c < 5 and slice n, rows k < 32 of
// Q (G16_n[k, :] U_d~^T) as negated fp16 hi/lo in [f][k] layout.
hipError_t launch_prep_w(const _Float16* G16, const float* V32, const int8_t* signs, int N, int D,
                         int ntab, _Float16* Wneg_hi, _Float16* Wneg_lo, int32_t* flags, hipStream_t s);

// ---------------------------------------------------------------- fused score pass
struct ScoreArgs {
  int N, T, D, ntab;
  const int8_t* signs;      // [ntab][D]
  const _Float16* UT16;     // [ntab][5][T][32]   stored token factors of the r_d chains
  const _Float16* G16T;     // [ntab][N][T][32]   stored core of the full-token chain
  const _Float16* Wneg_hi;  // [ntab][5][N][D][32]
  const _Float16* Wneg_lo;
  const _Float16* Vneg_hi;  // [ntab][D][32]
  const _Float16* Vneg_lo;
  double* part;             // [ntab][score_partials(N, T)][100]
};
hipError_t launch_score(const ScoreArgs& a, const TablePtrs& x, hipStream_t s);
int score_partials(int N, int T);  // workgroup partials per table written by the score pass
hipError_t launch_score_reduce(const double* part, int nparts, int ntab, double* E, hipStream_t s);

// ---------------------------------------------------------------- encode / decode
struct EncodeTable {
  int rT, rd, b;           // chosen candidate
  int chain;               // 0..4 r_d chain, 5 full-token chain, -1 verbatim (T, D)
  char* rec;               // record base (device)
  uint64_t off_ut, off_ud, off_core, off_codes, off_scales, total;
};
#define JOLT_TAB_CHUNK 16  // table descriptors per codec launch (kernel-argument size)
struct EncodeArgs {
  int N, T, D, ntab;       // ntab <= JOLT_TAB_CHUNK tables starting at t0
  int t0;
  const int8_t* signs;
  const _Float16* UT16;    // [ntab][5][T][32]
  const _Float16* Ud16;    // [ntab][D][32]
  const _Float16* G16;     // [ntab][5][N][32][D] stored cores
  const _Float16* G16T;    // [ntab][N][T][32]
  EncodeTable t[JOLT_TAB_CHUNK];
  const void* xsrc[JOLT_TAB_CHUNK];
};
hipError_t launch_encode(const EncodeArgs& a, hipStream_t s);

struct DecodeArgs {
  int N, T, D, ntab;  // ntab <= JOLT_TAB_CHUNK
  EncodeTable t[JOLT_TAB_CHUNK];
  void* out[JOLT_TAB_CHUNK];
};
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);

// ---------------------------------------------------------------- streaming admission
// An incoming token block of each table is encoded against that table's frozen record:
// token rows L of the block by least squares against the record's reconstruction
// operator, then the rotated residual codes of X' - L R, into a block record.
struct StreamTable {
  EncodeTable f;              // the frozen record (f.rec = its base)
  char* blk;                  // block record base
  uint64_t off_l, off_codes, off_scales, total;  // block record sections
  const uint16_t* x;          // incoming block, bf16 [N][tn][D]
  double* state;              // pseudo-inverse A+ [32][32] fp64, then the eigenvalues of A [32]
  uint16_t* out;              // decoded block, bf16 [N][tn][D]
};
#define STREAM_TAB_CHUNK 16   // tables per streaming launch (kernel-argument size)
#define STREAM_CHUNK 256      // block tokens per residual / decode workgroup
#define STREAM_GROUPS 8       // slice groups of the left-factor pass (fewer when N < 8)
#define STREAM_STATE_DOUBLES (32 * 32 + 32)
#define STREAM_RCUT 1e-12     // eigenvalues of A below this fraction of the largest are dropped
#define BLOCK_MAGIC 0x42544C4Au
struct StreamArgs {
  int N, T, D, tn, ntab, t0;  // ntab <= STREAM_TAB_CHUNK tables starting at global index t0
  int nchunk;                 // token chunks of 256 per slice of the block
  double* part;               // [n_tables][N][nchunk][2]: sum x^2, sum of squared errors
  double* dist;               // [n_tables] block distortion (nullable)
  int ng, spg;                // slice groups of the left-factor pass, slices per group
  double* pfold;              // [n_tables][ng][tn / 64][4][2][4][64] partial P^T of the groups
  StreamTable t[STREAM_TAB_CHUNK];
};
hipError_t launch_stream_prepare(const StreamArgs& a, hipStream_t s);
hipError_t launch_stream_encode(const StreamArgs& a, hipStream_t s);
hipError_t launch_stream_decode(const StreamArgs& a, hipStream_t s);

#define ATT_QMAX 16    // queries per slice
#define ATT_CHMAX 2048 // tokens per attention chunk
#define ATT_GMAX 8     // layer groups per launch
struct AttendArgs {
  int N, T, D, nq, ng;          // ng <= ATT_GMAX groups
  int ach, nchunk;              // tokens per chunk, chunks per slice
  float scale;                  // score scale
  EncodeTable k[ATT_GMAX], v[ATT_GMAX];  // each group's K and V records
  const uint16_t* q[ATT_GMAX];  // bf16 [N][nq][D] per group
  float* out[ATT_GMAX];         // fp32 [N][nq][D] per group
  float* part;                  // [ng][N][nchunk][nq][D + 2]: unnormalised output, chunk max, chunk sum
};
hipError_t launch_attend(const AttendArgs& a, hipStream_t s);

}  // namespace jolt
