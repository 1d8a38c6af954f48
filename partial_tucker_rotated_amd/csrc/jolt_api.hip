// C ABI of the JoLT engine: validation, byte cost, lambda bisection, workspace
// planning and the launch sequence of the table build, encode and decode.
#include <math.h>
#include <stdlib.h>
#include <string.h>

#include <algorithm>
#include <mutex>
#include <unordered_map>
#include <vector>

#include "../../include/jolt.h"
#include "../../include/jolt_debug.h"
#include "jolt_internal.h"

using namespace jolt;

namespace {

const int kRTIdx = 5, kRDIdx = 5, kNB = 4;
const int kBits[4] = {0, 2, 4, 8};
const int kRanks[4] = {4, 8, 16, 32};

inline uint64_t pad_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }
inline bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
inline int ilog2(int64_t x) {
  int r = 0;
  while ((1ll << r) < x) ++r;
  return r;
}

jolt_status validate(const jolt_config* c) {
  if (!c) return JOLT_EINVAL;
  if (c->N < 1 || c->N > 65536) return JOLT_EINVAL;
  if (!pow2(c->T) || c->T < 64 || c->T > 65536) return JOLT_EINVAL;
  if (c->D != 64 && c->D != 128) return JOLT_EINVAL;
  if (c->n_tables < 1 || c->n_tables > JOLT_MAX_TABLES) return JOLT_EINVAL;
  if (c->quant_block != c->D || c->s_bytes != 2 || c->align_bytes != 256) return JOLT_EINVAL;
  if (c->q_cap != 32 || c->oversample != 8) return JOLT_EINVAL;
  if (c->token_mode != JOLT_TOKEN_EXACT && c->token_mode != JOLT_TOKEN_RANDOMIZED) return JOLT_EINVAL;
  if (c->power_iters < 0 || c->power_iters > 4) return JOLT_EINVAL;
  if (c->exact_iters < 1 || c->exact_iters > c->exact_max_iters || c->exact_max_iters > 256) return JOLT_EINVAL;
  if (c->token_mode == JOLT_TOKEN_EXACT && c->T > 2048) return JOLT_EINVAL;  // T x T Grams
  if (c->token_mode == JOLT_TOKEN_RANDOMIZED && c->N * 4 < c->q_cap + c->oversample) return JOLT_EINVAL;
  if ((int64_t)c->N * c->T > (1ll << 30)) return JOLT_EINVAL;
  if (c->factor_precision < 0 || c->factor_precision > 2) return JOLT_EINVAL;
  return JOLT_OK;
}

// fp64 factor arithmetic: needed where single fp16 storage-rounding flips of a factor
// entry would be visible in the table (few rows), and cheap there
bool precise_factors(const jolt_config* c) {
  if (c->factor_precision == 1) return true;
  if (c->factor_precision == 2) return false;
  return (int64_t)c->N * c->T * c->D <= (1ll << 20);
}

void cand_params(const jolt_config* c, int i, int& rT, int& rd, int& b, int& irT, int& ird) {
  irT = i / (kRDIdx * kNB);
  ird = (i / kNB) % kRDIdx;
  b = kBits[i % kNB];
  rT = irT < 4 ? kRanks[irT] : c->T;
  rd = ird < 4 ? kRanks[ird] : c->D;
}

uint64_t cand_cost(const jolt_config* c, int i) {
  int rT, rd, b, irT, ird;
  cand_params(c, i, rT, rd, b, irT, ird);
  const uint64_t A = (uint64_t)c->align_bytes, s = (uint64_t)c->s_bytes;
  const uint64_t N = c->N, T = c->T, D = c->D;
  uint64_t bytes = 256;
  if (rT == c->T && rd == c->D) {
    bytes += pad_up(s * N * T * D, A);
  } else {
    if (rT < c->T) bytes += pad_up(s * T * rT, A);
    if (rd < c->D) bytes += pad_up(s * D * rd, A);
    bytes += pad_up(s * N * rT * rd, A);
  }
  if (b > 0) {
    bytes += pad_up((b * N * T * D + 7) / 8, A);
    bytes += pad_up(4 * N * T * (D / c->quant_block), A);
  }
  return bytes;
}

EncodeTable record_layout(const jolt_config* c, int i) {
  int rT, rd, b, irT, ird;
  cand_params(c, i, rT, rd, b, irT, ird);
  EncodeTable e{};
  e.rT = rT;
  e.rd = rd;
  e.b = b;
  e.chain = (irT == 4 && ird == 4) ? -1 : (irT == 4 ? 5 : ird);
  const uint64_t A = 256, N = c->N, T = c->T, D = c->D;
  uint64_t off = 256;
  if (rT < c->T) {
    e.off_ut = off;
    off += pad_up(2 * T * rT, A);
  }
  if (rd < c->D) {
    e.off_ud = off;
    off += pad_up(2 * D * rd, A);
  }
  e.off_core = off;
  off += pad_up(2 * N * (uint64_t)rT * rd, A);
  if (b > 0) {
    e.off_codes = off;
    off += pad_up((b * N * T * D + 7) / 8, A);
    e.off_scales = off;
    off += pad_up(4 * N * T, A);
  }
  e.total = off;
  return e;
}

// ------------------------------------------------------------------ workspace plan
struct Plan {
  size_t total = 0;
  int nchunk = 1;   // feature Gram row chunks
  size_t flags, xn2, E, gparts, Gd, Ud64, lamd, Ud32, Ud16, V32, Vh, Vl, Y32, G16T, Mtok, Qs, Zs, Wp, Rinv,
      Hrr, Vrr, Om, Pz, Pq, UT32, UT16, Gc, G16, Wh, Wl, part, YT, gscr, lamT, PqT, OmT, XSp, XSp2, res, CoP, TGp;
  size_t gscr_bytes = 0;
  size_t put(size_t bytes) {
    const size_t o = total;
    total += pad_up(bytes, 256);
    return o;
  }
};

// The four token Grams of the r_d = 4..32 chains in one GEMM over the feature-major
// token unfolding (fp32 working precision; checkpoints at K = 4N, 8N, 16N on 32-aligned
// bounds; the row-block transpose holds N <= 256)
// The r_d = D token Gram of the exact mode by its own kernel (fp32 working precision)
bool tgram_kernel(const jolt_config* c) {
  return !precise_factors(c) && c->D == 128 && c->T % 128 == 0 && c->n_tables <= 64;
}

bool token_grams_fused(const jolt_config* c) {
  const int N = c->N;
  return c->token_mode == JOLT_TOKEN_EXACT && !precise_factors(c) && (N & (N - 1)) == 0 && N >= 8 && N <= 256;
}

// The randomized range finder's products A^T S (K = T) run in kernels of their own that
// stream the tensor or Y once per slice (launch_xts, launch_yts), and its products A B take
// the shared operand B transposed, so that lanes load runs of k (fp32 working precision).
bool rf_token_contig(const jolt_config* c) {
  return c->token_mode == JOLT_TOKEN_RANDOMIZED && !precise_factors(c);
}

Plan make_plan(const jolt_config* c) {
  Plan p;
  const size_t nt = c->n_tables, N = c->N, T = c->T, D = c->D, NT = N * T;
  const size_t nb = nt * 5;
  const int tiles = (int)((D / 64) * (D / 64));
  while ((int64_t)nt * p.nchunk * tiles < 2048 && (int64_t)NT % (2 * p.nchunk) == 0 &&
         (int64_t)NT / (2 * p.nchunk) >= 256)
    p.nchunk *= 2;
  const bool exact = c->token_mode == JOLT_TOKEN_EXACT;
  const size_t pc = exact ? JOLT_PSUB : 40;
  const size_t fe = precise_factors(c) ? 8 : 4;  // working-precision element bytes
  p.flags = p.put(64);
  p.xn2 = p.put(8 * nt);
  p.E = p.put(8 * nt * 100);
  p.gparts = p.put(8 * nt * p.nchunk * D * D);
  p.Gd = p.put(8 * nt * D * D);
  p.Ud64 = p.put(8 * nt * D * JOLT_KMAX);
  p.lamd = p.put(8 * nt * JOLT_KMAX);
  p.Ud32 = p.put(4 * nt * D * JOLT_KMAX);
  p.Ud16 = p.put(2 * nt * D * JOLT_KMAX);
  p.V32 = p.put(4 * nt * D * JOLT_KMAX);
  p.Vh = p.put(2 * nt * D * JOLT_KMAX);
  p.Vl = p.put(2 * nt * D * JOLT_KMAX);
  p.Y32 = p.put(fe * nt * NT * JOLT_KMAX);
  p.G16T = p.put(2 * nt * NT * JOLT_KMAX);
  p.Mtok = exact ? p.put(fe * nb * T * T) : 0;
  // split sums of the r_d = D token Gram's own kernel (side stream)
  {
    const int64_t pf = exact && tgram_kernel(c) ? tgram_part_floats((int)N, (int)T, (int)nt) : 0;
    p.TGp = pf > 0 ? p.put(4 * (size_t)pf) : 0;
  }
  p.Qs = p.put(fe * nb * T * pc);
  p.Zs = p.put(fe * nb * T * pc);
  p.Wp = p.put(8 * nb * (size_t)JOLT_GRAM_PARTS * pc * pc);
  p.Rinv = p.put(fe * nb * pc * pc);
  p.Hrr = p.put(8 * nb * pc * pc);
  p.Vrr = p.put(fe * nb * pc * JOLT_KMAX);
  p.lamT = p.put(8 * nb * JOLT_KMAX);  // token eigenvalues (modelled tables)
  p.res = p.put(8 * nb);               // Ritz residuals of the exact subspace iteration
  p.Om = exact ? 0 : p.put(2 * nt * N * (4 + 8 + 16 + 32 + D) * 40);
  p.Pz = exact ? 0 : p.put(fe * nb * N * D * 40);
  p.Pq = exact ? 0 : p.put(fe * nb * N * D * 40);
  p.UT32 = p.put(fe * nb * T * JOLT_KMAX);
  p.UT16 = p.put(2 * nb * T * JOLT_KMAX);
  p.Gc = p.put(fe * nb * N * JOLT_KMAX * D);
  p.G16 = p.put(2 * nb * N * JOLT_KMAX * D);
  p.Wh = p.put(2 * nb * N * D * JOLT_KMAX);
  p.Wl = p.put(2 * nb * N * D * JOLT_KMAX);
  p.part = p.put(8 * nt * (NT / 64) * 100);
  p.YT = token_grams_fused(c) ? p.put(4 * nt * NT * JOLT_KMAX) : 0;
  // k-slice partials of the finder's A^T S kernels (one launch at a time on the main stream)
  p.XSp = rf_token_contig(c) ? p.put(4 * nt * N * (size_t)xts_slices((int)T) * std::max<size_t>(D, 128) * 40) : 0;
  // the tensor chain's A^T S runs beside the r_d < D chains' (side stream) when the token axis
  // is one k slice: partials of its own
  p.XSp2 = rf_token_contig(c) && xts_slices((int)T) == 1 ? p.put(4 * nt * N * std::max<size_t>(D, 128) * 40) : 0;
  p.PqT = rf_token_contig(c) ? p.put(4 * nb * N * D * 40) : 0;
  p.OmT = rf_token_contig(c) ? p.put(2 * nt * N * (4 + 8 + 16 + 32 + D) * 40) : 0;
  // token-slice partial sums of the core kernel (fp32 working precision, D = 128)
  {
    const int nks = (exact && !precise_factors(c) && D == 128) ? cores_slices((int)N, (int)T, (int)nt) : 1;
    p.CoP = nks > 1 ? p.put(8 * (size_t)nks * N * nt * 26 * 256) : 0;
  }
  // split-K partial sums of the factor-stage GEMMs: a quarter of the input bytes,
  // between 64 MiB and 1 GiB
  {
    const size_t xb = 2 * nt * NT * D;
    size_t g = xb / 4;
    g = g < ((size_t)64 << 20) ? ((size_t)64 << 20) : g;
    g = g > ((size_t)1 << 30) ? ((size_t)1 << 30) : g;
    p.gscr_bytes = g;
    p.gscr = p.put(g);
  }
  return p;
}

#define HIPCHK(x)                                 \
  do {                                            \
    if ((x) != hipSuccess) return JOLT_EDEVICE;   \
  } while (0)

struct Ctx {
  const jolt_config* c;
  Plan p;
  char* ws;
  TablePtrs x;
  hipStream_t s;
  bool f64;     // fp64 factor arithmetic
  int wt;       // operand type code of working buffers (0 fp32, 3 fp64)
  int we;       // bytes per working element
  // exact token mode: subspace iterations run, largest Ritz residual left (relative to the
  // leading Ritz value), whether every problem met the tolerance
  mutable int exact_iters_used = 0;
  mutable double exact_residual = 0.0;
  mutable int exact_converged = 1;
  template <typename T>
  T* at(size_t off) const {
    return (T*)(ws + off);
  }
  void* w(size_t off, int64_t elems = 0) const { return ws + off + elems * we; }
  int mode_any() const { return f64 ? GEMM_F64 : GEMM_SPLIT; }
  int mode_bf16() const { return f64 ? GEMM_F64 : GEMM_BF16; }
};

// A second stream (default priority) and two events per device, created on first use and
// kept for the process: work that does not depend on the feature factor (the token Gram of
// X in exact mode) runs beside the feature eigensolver, which occupies one workgroup per
// table.
struct SideStream {
  hipStream_t s = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
// `which` selects one of two side streams of the device (default priority, non-blocking)
static hipError_t side_stream(SideStream& out, int which = 0) {
  static std::mutex mu;
  static std::unordered_map<int, SideStream> per_dev;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  dev = 2 * dev + which;
  std::lock_guard<std::mutex> lk(mu);
  auto it = per_dev.find(dev);
  if (it == per_dev.end()) {
    SideStream ss;
    if ((e = hipStreamCreateWithFlags(&ss.s, hipStreamNonBlocking)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.fork, hipEventDisableTiming)) != hipSuccess) return e;
    if ((e = hipEventCreateWithFlags(&ss.join, hipEventDisableTiming)) != hipSuccess) return e;
    it = per_dev.emplace(dev, ss).first;
  }
  out = it->second;
  return hipSuccess;
}

GemmArgs gemm_base(const Ctx& x) {
  GemmArgs g;
  memset(&g, 0, sizeof(g));
  g.scratch = x.ws + x.p.gscr;
  g.scratch_bytes = (int64_t)x.p.gscr_bytes;
  g.nvar = 1;
  g.vdiv = 1;
  g.cbdiv = 1;
  g.alpha = 1.0f;
  g.alpha_div = 1;
  return g;
}

GemmOperand wop(const Ctx& x, const void* p, int64_t sb1, int64_t sr, int64_t sk) {
  return op_plain(p, x.wt, sb1, sr, sk);
}

// token-unfolding operand of chain c (r_d = 4 << c, or D for c = 4):
// element (row t, k = n * r_d + j); batch b -> table b / bdiv
GemmOperand op_unfold(const Ctx& x, int c, int bdiv) {
  const int T = x.c->T, D = x.c->D, N = x.c->N;
  GemmOperand o{};
  o.bdiv = bdiv;
  o.rsh = 30;
  if (c < 4) {
    const int rd = 4 << c;
    o.p = x.w(x.p.Y32);
    o.type = x.wt;
    o.sb1 = (int64_t)N * T * JOLT_KMAX;
    o.sr2 = JOLT_KMAX;
    o.ksh = ilog2(rd);
    o.sk1 = (int64_t)T * JOLT_KMAX;
    o.sk2 = 1;
  } else {
    o.tbl = 1;
    o.type = 1;
    o.sr2 = D;
    o.ksh = ilog2(D);
    o.sk1 = (int64_t)T * D;
    o.sk2 = 1;
  }
  return o;
}
// transposed unfolding: element (row k = n * r_d + j, col t)
GemmOperand op_unfold_t(const Ctx& x, int c, int bdiv) {
  const int T = x.c->T, D = x.c->D, N = x.c->N;
  GemmOperand o{};
  o.bdiv = bdiv;
  o.ksh = 30;
  if (c < 4) {
    const int rd = 4 << c;
    o.p = x.w(x.p.Y32);
    o.type = x.wt;
    o.sb1 = (int64_t)N * T * JOLT_KMAX;
    o.rsh = ilog2(rd);
    o.sr1 = (int64_t)T * JOLT_KMAX;
    o.sr2 = 1;
    o.sk2 = JOLT_KMAX;
  } else {
    o.tbl = 1;
    o.type = 1;
    o.rsh = ilog2(D);
    o.sr1 = (int64_t)T * D;
    o.sr2 = 1;
    o.sk2 = D;
  }
  return o;
}

// output description of a working buffer [batch][rows][cols]
void out_w(const Ctx& x, GemmArgs& g, void* C, int64_t rows, int64_t cols) {
  g.C = C;
  g.c_type = x.f64 ? 1 : 0;
  g.csb1 = rows * cols;
  g.csm = cols;
  g.csn = 1;
}

// dst[b] = orth(src[b]) for `batch` row-major [rows][p] working-precision matrices
// (one CholeskyQR pass: Gram, Cholesky, dst = src R^{-1}).  The Gram is formed in fp64
// from the working values in either precision: in a subspace iteration the columns of
// src are dominated by the leading direction, and the squared spread of the directions
// the block must keep apart (down to 1e-7 of the leading one, squared) is far below
// what an fp32-accumulated Gram resolves; lost there, a direction does not come back.
// The Gram is summed from up to JOLT_GRAM_PARTS row chunks of at least 128 rows, one
// workgroup each.
// row chunks of the Gram partials of a [rows][p] block
static int orth_parts(int64_t rows) {
  int nsplit = 1;
  while (nsplit * 2 <= JOLT_GRAM_PARTS && rows % (nsplit * 2) == 0 && rows / (nsplit * 2) >= 128) nsplit *= 2;
  return nsplit;
}

// As orth, on stream s with the given Gram-partial and R^{-1} scratch (problem 0's slots).
jolt_status orth_at(const Ctx& x, hipStream_t s, const void* src, void* dst, int64_t rows, int p, int batch,
                    double* Wp, void* Rinv) {
  const int nsplit = orth_parts(rows);
  HIPCHK(launch_gram64(src, x.f64, rows, p, nsplit, batch, Wp, s));
  if (!x.f64) {  // Cholesky and inverse, then dst = src R^{-1}
    HIPCHK(launch_chol_apply(Wp, nsplit, p, (const float*)src, (float*)dst, rows, batch, (float*)Rinv, s));
    return JOLT_OK;
  }
  HIPCHK(launch_chol_inv(Wp, nsplit, p, batch, Rinv, x.f64, s));
  GemmArgs q = gemm_base(x);
  q.scratch = nullptr;
  q.scratch_bytes = 0;
  q.v[0].A = wop(x, src, rows * p, p, 1);
  q.v[0].B = wop(x, Rinv, (int64_t)p * p, 1, p);
  q.v[0].M = (int32_t)rows;
  q.v[0].N = p;
  q.v[0].K = p;
  q.mode = x.mode_any();
  out_w(x, q, dst, rows, p);
  HIPCHK(launch_gemm(q, x.x, batch, s));
  return JOLT_OK;
}

jolt_status orth(const Ctx& x, const void* src, void* dst, int64_t rows, int p, int batch) {
  return orth_at(x, x.s, src, dst, rows, p, batch, x.at<double>(x.p.Wp), x.w(x.p.Rinv));
}

hipError_t syev_at(const Ctx& x, hipStream_t s, const void* A, bool Af64, int n, int batch, void* U,
                   _Float16* U16, double* lam) {
  // U (working precision) [batch][n][32]; lam [batch][32] (nullable)
  return jolt::launch_syev_topk_any(A, !Af64, n, JOLT_KMAX, batch, x.f64 ? (double*)U : nullptr,
                                    x.f64 ? nullptr : (float*)U, U16, lam, s);
}
hipError_t syev(const Ctx& x, const void* A, bool Af64, int n, int batch, void* U, _Float16* U16, double* lam) {
  return syev_at(x, x.s, A, Af64, n, batch, U, U16, lam);
}

// Exact token factors of `nprob` problems by subspace iteration (64 columns, CholeskyQR after
// every product) on stream s, with Rayleigh-Ritz and a Ritz-residual test at the end of each
// round.  Problem b reads its token Gram at M + (b / div) s1 + (b % div) s2 elements and
// writes U_T (working precision and fp16) at the same split of UT / UT16 with strides u1,
// u2; its subspace buffers are the slots boff + b of Qs, Zs, Wp, Rinv, Hrr, Vrr, lamT and
// res.  After a round the orthonormal basis is in one of Qs / Zs and its product with M in
// the other (bas_in_z tells which); a further round continues from that product.
struct SubspaceJob {
  hipStream_t s;
  int nprob;
  int64_t boff;
  void* M;
  int div;
  int64_t s1, s2;
  void* UT;
  _Float16* UT16;
  int64_t u1, u2;
  bool bas_in_z;  // set by each round
};

struct SubspaceOps {
  const Ctx& x;
  SubspaceJob& j;
  int T, p;
  int64_t blk;
  void *Q, *Z;
  double* Wp;
  void* Rinv;
  double* Hrr;
  void* Vrr;
  double* lam;
  double* res;
  SubspaceOps(const Ctx& x_, SubspaceJob& j_) : x(x_), j(j_) {
    const Plan& P = x.p;
    T = x.c->T;
    p = JOLT_PSUB;
    blk = (int64_t)T * p;
    Q = x.w(P.Qs, j.boff * blk);
    Z = x.w(P.Zs, j.boff * blk);
    Wp = x.at<double>(P.Wp) + j.boff * JOLT_GRAM_PARTS * p * p;
    Rinv = x.w(P.Rinv, j.boff * p * p);
    Hrr = x.at<double>(P.Hrr) + j.boff * p * p;
    Vrr = x.w(P.Vrr, j.boff * p * JOLT_KMAX);
    lam = x.at<double>(P.lamT) + j.boff * JOLT_KMAX;
    res = x.at<double>(P.res) + j.boff;
  }
  // the product kernel with Gram partials applies (fp32 working precision)
  bool mq() const { return !x.f64 && p == 64 && T % 64 == 0 && T / 64 <= JOLT_GRAM_PARTS; }
  // dst = M src for every problem; with gram (and mq()), also the Gram partials of dst in Wp
  hipError_t product(const void* src, void* dst, bool gram = false) {
    if (mq())
      return launch_mq((const float*)j.M, j.div, j.s1, j.s2, (const float*)src, (float*)dst, T, j.nprob,
                       gram ? Wp : nullptr, j.s);
    GemmArgs g = gemm_base(x);
    g.scratch = nullptr;  // short reductions: no split-K (and no sharing between streams)
    g.scratch_bytes = 0;
    GemmOperand mo = wop(x, j.M, j.s1, T, 1);
    mo.bdiv = j.div;
    mo.sb2 = j.s2;
    g.v[0].A = mo;
    g.v[0].B = wop(x, src, blk, 1, p);
    g.v[0].M = T;
    g.v[0].N = p;
    g.v[0].K = T;
    g.mode = x.mode_any();
    out_w(x, g, dst, T, p);
    g.xgrp = 1;  // operand shared by the unit's tiles: one XCD
    return launch_gemm(g, x.x, j.nprob, j.s);
  }
  jolt_status orth(const void* src, void* dst) { return orth_at(x, j.s, src, dst, T, p, j.nprob, Wp, Rinv); }
  // src = M q as product(q, src, true) left it: one CholeskyQR pass into dst
  jolt_status orth_product(const void* src, void* dst) {
    if (!mq()) return orth(src, dst);
    HIPCHK(launch_chol_apply(Wp, T / 64, p, (const float*)src, (float*)dst, T, j.nprob, (float*)Rinv, j.s));
    return JOLT_OK;
  }
  // basis in `bas` (orthonormal up to one CholeskyQR pass): second pass into `oth`, then
  // Rayleigh-Ritz (product into `bas`, H = Z^T M Z, its top 32 eigenpairs, U_T = Z V) and
  // the Ritz residuals; afterwards the basis is in `oth` and its product in `bas`
  jolt_status finalize(void* bas, void* oth) {
    jolt_status st = orth(bas, oth);
    if (st != JOLT_OK) return st;
    HIPCHK(product(oth, bas));
    if (mq()) {  // H = Z^T (M Z) from row-chunk partials, U_T = Z V row by row
      const int np = orth_parts(T);
      HIPCHK(launch_gram_cross((const float*)oth, (const float*)bas, T, np, j.nprob, Wp, j.s));
      HIPCHK(launch_sum_parts(Wp, np, p * p, j.nprob, Hrr, j.s));
      HIPCHK(syev_at(x, j.s, Hrr, true, p, j.nprob, Vrr, nullptr, lam));
      HIPCHK(launch_ut_rows((const float*)oth, (const float*)Vrr, p, T, j.nprob, (float*)j.UT, j.UT16, j.div, j.u1,
                            j.u2, j.s));
      HIPCHK(launch_ritz_residual(bas, oth, Vrr, x.f64, lam, T, p, j.nprob, res, Wp, j.s));
      j.bas_in_z = oth == Z;
      return JOLT_OK;
    }
    GemmArgs h = gemm_base(x);
    h.scratch = nullptr;
    h.scratch_bytes = 0;
    h.v[0].A = wop(x, oth, blk, 1, p);
    h.v[0].B = wop(x, bas, blk, 1, p);
    h.v[0].M = p;
    h.v[0].N = p;
    h.v[0].K = T;
    h.C = Hrr;
    h.c_type = 1;
    h.csb1 = (int64_t)p * p;
    h.csm = p;
    h.csn = 1;
    h.acc64 = 1;
    h.mode = x.mode_any();
    HIPCHK(launch_gemm(h, x.x, j.nprob, j.s));
    HIPCHK(syev_at(x, j.s, Hrr, true, p, j.nprob, Vrr, nullptr, lam));
    GemmArgs u = gemm_base(x);
    u.scratch = nullptr;
    u.scratch_bytes = 0;
    u.v[0].A = wop(x, oth, blk, p, 1);
    u.v[0].B = wop(x, Vrr, (int64_t)p * JOLT_KMAX, 1, JOLT_KMAX);
    u.v[0].M = T;
    u.v[0].N = JOLT_KMAX;
    u.v[0].K = p;
    u.mode = x.mode_any();
    u.C = j.UT;
    u.c_type = x.f64 ? 1 : 0;
    u.cbdiv = j.div;
    u.csb1 = j.u1;
    u.csb2 = j.u2;
    u.csm = JOLT_KMAX;
    u.csn = 1;
    u.C16 = j.UT16;
    u.xgrp = 1;  // operand shared by the unit's tiles: one XCD
    HIPCHK(launch_gemm(u, x.x, j.nprob, j.s));
    // (the job's Gram-partial slots are free here: T / 64 * 32 <= orth_parts(T) * p * p doubles)
    HIPCHK(launch_ritz_residual(bas, oth, Vrr, x.f64, lam, T, p, j.nprob, res, Wp, j.s));
    j.bas_in_z = oth == Z;
    return JOLT_OK;
  }
};

// First round: a fixed start block, `iters` products each followed by CholeskyQR, then the
// Rayleigh-Ritz step and the residuals: subspace_begin_n.
// `iters` (>= 1) further iterations from the last round's product, then Rayleigh-Ritz and the
// residuals again: subspace_more_n.
// The same rounds for several jobs on their own streams, their launches queued iteration by
// iteration in turn, so that no stream waits for the host to queue another stream's round.
jolt_status subspace_begin_n(const Ctx& x, SubspaceJob* const* js, int n, int iters) {
  std::vector<SubspaceOps> o;
  o.reserve(n);
  for (int k = 0; k < n; ++k) o.emplace_back(x, *js[k]);
  for (int k = 0; k < n; ++k) HIPCHK(launch_init_subspace(o[k].Q, x.f64, o[k].T, js[k]->nprob, js[k]->s));
  for (int it = 0; it < iters; ++it) {
    for (int k = 0; k < n; ++k) HIPCHK(o[k].product(o[k].Q, o[k].Z, true));
    for (int k = 0; k < n; ++k) {
      jolt_status st = o[k].orth_product(o[k].Z, o[k].Q);
      if (st != JOLT_OK) return st;
    }
  }
  for (int k = 0; k < n; ++k) {
    jolt_status st = o[k].finalize(o[k].Q, o[k].Z);
    if (st != JOLT_OK) return st;
  }
  return JOLT_OK;
}

jolt_status subspace_more_n(const Ctx& x, SubspaceJob* const* js, int n, int iters) {
  std::vector<SubspaceOps> o;
  o.reserve(n);
  std::vector<void*> bas(n), prod(n);
  for (int k = 0; k < n; ++k) {
    o.emplace_back(x, *js[k]);
    bas[k] = js[k]->bas_in_z ? o[k].Z : o[k].Q;
    prod[k] = js[k]->bas_in_z ? o[k].Q : o[k].Z;
  }
  for (int k = 0; k < n; ++k) {  // the product held by the last round: one iteration
    jolt_status st = o[k].orth(prod[k], bas[k]);
    if (st != JOLT_OK) return st;
  }
  for (int it = 1; it < iters; ++it) {
    for (int k = 0; k < n; ++k) HIPCHK(o[k].product(bas[k], prod[k], true));
    for (int k = 0; k < n; ++k) {
      jolt_status st = o[k].orth_product(prod[k], bas[k]);
      if (st != JOLT_OK) return st;
    }
  }
  for (int k = 0; k < n; ++k) {
    jolt_status st = o[k].finalize(bas[k], prod[k]);
    if (st != JOLT_OK) return st;
  }
  return JOLT_OK;
}

// Relative Ritz residual below which a token eigenpair counts as converged: the largest
// residual of the 32 leading Ritz pairs, ||M u - theta u||, at most this fraction of the
// leading Ritz value.
#define JOLT_EXACT_TOL 1e-6
// A round that leaves a problem's residual above this fraction of its previous value has
// reached the floor of the working precision (about 1e-6 of theta_0 with fp32 products and
// an fp32 Gram); the problem then stops iterating, and counts as converged when that floor
// is below JOLT_EXACT_FLOOR.
#define JOLT_EXACT_STALL 0.8
#define JOLT_EXACT_FLOOR 1e-5

// Contraction per iteration assumed for the first further round, before two residuals of a
// problem have been measured (measured at 512 and 1024 tokens: about 0.3 and 0.4).
#define JOLT_EXACT_RATE0 0.5

// Host side of the convergence test.  Every job's first round is queued and the main stream
// has joined the other streams.  Read every problem's residual; while a problem is above the
// tolerance and still contracting, run further rounds of the job that holds it (each job on
// its own stream, batched over its problems; the main stream joins the other streams before
// the next read), sized from the slowest contraction per iteration among such problems
// (JOLT_EXACT_RATE0 before it has been measured), up to exact_max_iters in total.  jobs[k]
// holds the problems (subspace slots) boff .. boff + nprob - 1; joins[k] is the event that
// the main stream waits on after a round of jobs[k] on another stream.
jolt_status subspace_converge(const Ctx& x, SubspaceJob* const* jobs, const hipEvent_t* joins, int njobs, int first) {
  const jolt_config* c = x.c;
  const int nt = c->n_tables, nb = 5 * nt;
  double* res_dev = x.at<double>(x.p.res);
  std::vector<double> res(nb), prev(nb, -1.0);
  std::vector<char> stalled(nb, 0);
  auto read = [&]() -> jolt_status {
    HIPCHK(hipMemcpyAsync(res.data(), res_dev, sizeof(double) * nb, hipMemcpyDeviceToHost, x.s));
    HIPCHK(hipStreamSynchronize(x.s));
    return JOLT_OK;
  };
  auto job_of = [&](int b) {
    for (int k = 0; k < njobs; ++k)
      if (b >= jobs[k]->boff && b < jobs[k]->boff + jobs[k]->nprob) return k;
    return -1;
  };
  jolt_status st = read();
  if (st != JOLT_OK) return st;
  int iters = first, prev_iters = 0;
  for (;;) {
    std::vector<char> active(njobs, 0);
    bool any = false;
    double need = 0.0, worst = 0.0;
    bool all_conv = true;
    for (int b = 0; b < nb; ++b) {
      worst = std::max(worst, res[b]);
      if (!(res[b] > JOLT_EXACT_TOL)) continue;
      if (prev_iters > 0 && !stalled[b] && !(res[b] < JOLT_EXACT_STALL * prev[b])) stalled[b] = 1;
      if (stalled[b]) {
        all_conv = all_conv && res[b] <= JOLT_EXACT_FLOOR;
        continue;
      }
      all_conv = false;
      const int k = job_of(b);
      if (k >= 0) {
        active[k] = 1;
        any = true;
      }
      const double rate =
          prev_iters > 0 ? std::pow(res[b] / prev[b], 1.0 / (iters - prev_iters)) : JOLT_EXACT_RATE0;
      need = std::max(need, std::log(JOLT_EXACT_TOL / res[b]) / std::log(rate));
    }
    x.exact_iters_used = iters;
    x.exact_residual = worst;
    x.exact_converged = all_conv;
    if (!any || iters >= c->exact_max_iters) break;
    int more = std::max(2, (int)std::ceil(need) + 1);
    more = std::min(more, c->exact_max_iters - iters);
    prev = res;
    prev_iters = iters;
    std::vector<SubspaceJob*> run;
    for (int k = 0; k < njobs; ++k)
      if (active[k] && jobs[k]->nprob > 0) run.push_back(jobs[k]);
    st = subspace_more_n(x, run.data(), (int)run.size(), more);
    if (st != JOLT_OK) return st;
    for (int k = 0; k < njobs; ++k) {  // the other streams' rounds complete before the read
      if (!active[k] || jobs[k]->nprob == 0 || jobs[k]->s == x.s) continue;
      HIPCHK(hipEventRecord(joins[k], jobs[k]->s));
      HIPCHK(hipStreamWaitEvent(x.s, joins[k], 0));
    }
    iters += more;
    st = read();
    if (st != JOLT_OK) return st;
  }
  return JOLT_OK;
}

// the all-chain core kernel (fp32 working precision, D = 128) also writes the score pass's
// reconstruction operands; otherwise launch_prep_w forms them after run_factors
static bool cores_make_w(const Ctx& x) { return !x.f64 && x.c->D == 128; }

jolt_status run_factors(const Ctx& x, const int8_t* signs_dev, bool cores = true) {
  const jolt_config* c = x.c;
  const Plan& P = x.p;
  const int nt = c->n_tables, N = c->N, T = c->T, D = c->D;
  const int64_t NT = (int64_t)N * T;
  const int nb = nt * 5;
  SideStream side;
  SubspaceJob jd{};  // exact mode: the r_d = D chain's subspace iteration (side stream)
  // randomized mode: the sketch product of the r_d = D chain goes ahead on the side stream
  // when its kernel applies (the conditions of the range finder's own launch below)
  const bool xw_early = rf_token_contig(c) && !x.f64 && ((int64_t)N * (4 + 8 + 16 + 32 + D)) % 8 == 0 &&
                        (uintptr_t)(x.at<uint16_t>(P.OmT) + (int64_t)N * (4 + 8 + 16 + 32)) % 16 == 0;
  x.exact_iters_used = 0;
  x.exact_residual = 0.0;
  x.exact_converged = 1;
  HIPCHK(hipMemsetAsync(x.at<int32_t>(P.flags), 0, 64, x.s));

  // ---- feature Gram sum_n X_n^T X_n in row chunks (bf16 products exact, fp64 across chunks)
  {
    if (!x.f64 && (D == 64 || D == 128)) {  // dedicated kernel: the GEMM's arithmetic, upper tiles only
      HIPCHK(launch_fgram(x.x, NT / P.nchunk, D, P.nchunk, nt, x.at<double>(P.gparts), x.s));
      HIPCHK(launch_reduce_gram(x.at<double>(P.gparts), P.nchunk, D, nt, x.at<double>(P.Gd),
                                x.at<double>(P.xn2), x.at<int32_t>(P.flags), x.s, true));
    } else {
      const int64_t rows = NT / P.nchunk;
      GemmArgs g = gemm_base(x);
      GemmOperand a{};
      a.tbl = 1;
      a.type = 1;
      a.bdiv = P.nchunk;
      a.sb2 = rows * D;
      a.rsh = 30;
      a.sr2 = 1;
      a.ksh = 30;
      a.sk2 = D;
      g.v[0].A = a;
      g.v[0].B = a;
      g.v[0].M = D;
      g.v[0].N = D;
      g.v[0].K = (int32_t)rows;
      g.C = x.at<double>(P.gparts);
      g.c_type = 1;
      g.cbdiv = P.nchunk;
      g.csb1 = (int64_t)P.nchunk * D * D;
      g.csb2 = (int64_t)D * D;
      g.csm = D;
      g.csn = 1;
      g.acc64 = 1;
      g.mode = x.mode_bf16();
      g.xgrp = 1;  // operand shared by the unit's tiles: one XCD
      HIPCHK(launch_gemm(g, x.x, nt * P.nchunk, x.s));
      HIPCHK(launch_reduce_gram(x.at<double>(P.gparts), P.nchunk, D, nt, x.at<double>(P.Gd),
                                x.at<double>(P.xn2), x.at<int32_t>(P.flags), x.s));
    }
    // randomized mode: the tensor chain's sketch product S = X Omega needs neither the
    // feature factor nor Y; it runs on the side stream beside the feature eigensolve and the
    // projection, and is joined before the first orthonormalisation
    if (xw_early) {
      const int64_t omrows = (int64_t)N * (4 + 8 + 16 + 32 + D);
      HIPCHK(launch_transpose_tc(nullptr, x.w(P.Om), true, 1, (int)omrows, 40, nt, x.w(P.OmT), x.s));
      HIPCHK(side_stream(side));
      HIPCHK(hipEventRecord(side.fork, x.s));
      HIPCHK(hipStreamWaitEvent(side.s, side.fork, 0));
      HIPCHK(launch_xw(x.x, x.at<uint16_t>(P.OmT) + (int64_t)N * (4 + 8 + 16 + 32), true, omrows * 40, omrows, N, T,
                       D, nt, x.at<float>(P.Zs) + 4 * (int64_t)T * 40, 5 * (int64_t)T * 40, side.s));
      HIPCHK(hipEventRecord(side.join, side.s));
    }
    const bool fork = c->token_mode == JOLT_TOKEN_EXACT;
    if (fork) {
      HIPCHK(side_stream(side));
      HIPCHK(hipEventRecord(side.fork, x.s));
    }
    // the feature eigensolver goes into the main stream before the host queues the side
    // stream's long launch sequence, so that it does not wait for that queueing
    HIPCHK(launch_syev_topk(x.at<double>(P.Gd), D, JOLT_KMAX, nt, x.at<double>(P.Ud64), nullptr,
                            x.at<double>(P.lamd), x.s));
    HIPCHK(launch_prep_feature(x.at<double>(P.Ud64), signs_dev, D, nt, x.at<float>(P.Ud32), x.at<_Float16>(P.Ud16),
                               x.at<float>(P.V32), x.at<_Float16>(P.Vh), x.at<_Float16>(P.Vl), x.s));
    if (fork) {
      // r_d = D token Gram sum_n X_n X_n^T (bf16 products exact, scaled by 1 / ||X||^2) on
      // the side stream, beside the feature eigensolver; joined before the token factors
      HIPCHK(hipStreamWaitEvent(side.s, side.fork, 0));
      if (tgram_kernel(c)) {  // its own kernel (fp32 working precision)
        HIPCHK(launch_tgram(x.x, N, T, D, nt, x.at<double>(P.xn2), x.at<float>(P.Mtok) + 4 * (int64_t)T * T,
                            5 * (int64_t)T * T, P.TGp ? x.at<float>(P.TGp) : nullptr, side.s));
      } else {
        GemmArgs g = gemm_base(x);
        g.scratch = nullptr;  // the scratch belongs to the main stream's launches
        g.scratch_bytes = 0;
        GemmOperand a = op_unfold(x, 4, 1);
        g.v[0].A = a;
        g.v[0].B = a;
        g.v[0].M = T;
        g.v[0].N = T;
        g.v[0].K = N * D;
        out_w(x, g, x.w(P.Mtok, 4 * (int64_t)T * T), T, T);
        g.csb1 = 5 * (int64_t)T * T;
        g.acc64 = 1;
        g.mode = x.mode_bf16();
        g.alpha_norm = x.at<double>(P.xn2);
        g.xgrp = 1;  // operand shared by the unit's tiles: one XCD
        HIPCHK(launch_gemm(g, x.x, nt, side.s));
      }
      if (T > 128) {  // the r_d = D token factors (subspace slots 4 nt ..) follow on this stream;
        // their launches are queued with the other chains' after the main stream's projection
        // and nested Grams, so that those do not wait for the host to queue them
        const int64_t TT = (int64_t)T * T, TK = (int64_t)T * JOLT_KMAX;
        jd = SubspaceJob{side.s, nt, 4 * (int64_t)nt, x.w(P.Mtok, 4 * TT), 1, 5 * TT, 0,
                         x.w(P.UT32, 4 * TK), x.at<_Float16>(P.UT16) + 4 * TK, 5 * TK, 0, false};
      } else {
        HIPCHK(hipEventRecord(side.join, side.s));
      }
    }
  }
  // ---- feature projection Y = X U_d[:, :32]; its fp16 copy is the core of the r_T = T chain
  // (fp32 working precision: one kernel that also writes the token-major copy for the
  // fused token Grams when N <= 32; otherwise the generic GEMM)
  const bool proj_kernel = !x.f64 && (D == 64 || D == 128);
  const bool proj_yt = proj_kernel && token_grams_fused(c) && N <= 32;
  if (proj_kernel) {
    HIPCHK(launch_project(x.x, x.at<float>(P.Ud32), N, T, D, nt, x.at<float>(P.Y32), x.at<_Float16>(P.G16T),
                          proj_yt ? x.at<float>(P.YT) : nullptr, x.at<int32_t>(P.flags), x.s));
  } else {
    GemmArgs g = gemm_base(x);
    GemmOperand a{};
    a.tbl = 1;
    a.type = 1;
    a.bdiv = 1;
    a.rsh = 30;
    a.sr2 = D;
    a.ksh = 30;
    a.sk2 = 1;
    g.v[0].A = a;
    g.v[0].B = x.f64 ? op_plain(x.at<double>(P.Ud64), 3, (int64_t)D * JOLT_KMAX, 1, JOLT_KMAX)
                     : op_plain(x.at<float>(P.Ud32), 0, (int64_t)D * JOLT_KMAX, 1, JOLT_KMAX);
    g.v[0].M = (int32_t)NT;
    g.v[0].N = JOLT_KMAX;
    g.v[0].K = D;
    g.mode = x.mode_any();
    out_w(x, g, x.w(P.Y32), NT, JOLT_KMAX);
    g.C16 = x.at<_Float16>(P.G16T);
    g.flags = x.at<int32_t>(P.flags);
    HIPCHK(launch_gemm(g, x.x, nt, x.s));
  }
  // ---- token factor of every (table, r_d)
  void* UT = x.w(P.UT32);
  _Float16* UT16 = x.at<_Float16>(P.UT16);
  if (c->token_mode == JOLT_TOKEN_EXACT) {
    void* M = x.w(P.Mtok);
    const int64_t TT = (int64_t)T * T;
    // the r_d = D token Gram was launched on the side stream
    if (token_grams_fused(c)) {
      // M(r_d) = sum_{j < r_d} sum_n y_{n,j} y_{n,j}^T: one pass over K = 32 N columns
      // ordered (j, n); the partial sums at K = 4N, 8N, 16N are M(4), M(8), M(16)
      if (!proj_yt) HIPCHK(launch_transpose_y(x.at<float>(P.Y32), N, T, nt, x.at<float>(P.YT), x.s));
      if (!x.f64 && N == 32 && T % 128 == 0) {  // its own kernel (fp32 working precision)
        HIPCHK(launch_tgram_y(x.at<float>(P.YT), N, T, nt, x.at<double>(P.xn2), x.at<float>(P.Mtok), 5 * TT, x.s));
      } else {
        GemmArgs g = gemm_base(x);
        GemmOperand a = op_plain(x.at<float>(P.YT), 0, NT * JOLT_KMAX, (int64_t)JOLT_KMAX * N, 1);
        g.v[0].A = a;
        g.v[0].B = a;
        g.v[0].M = T;
        g.v[0].N = T;
        g.v[0].K = JOLT_KMAX * N;
        out_w(x, g, x.w(P.Mtok, 3 * TT), T, T);
        g.csb1 = 5 * TT;
        g.acc64 = 1;
        g.mode = x.mode_any();
        g.alpha_norm = x.at<double>(P.xn2);
        g.nck = 3;
        g.ck[0] = 4 * N;
        g.ck[1] = 8 * N;
        g.ck[2] = 16 * N;
        g.ck_stride = TT;
        g.xgrp = 1;  // operand shared by the unit's tiles: one XCD
        HIPCHK(launch_gemm(g, x.x, nt, x.s));
      }
    } else {
      const int j0s[4] = {0, 4, 8, 16}, ws[4] = {4, 4, 8, 16};
      for (int cc = 0; cc < 4; ++cc) {  // r_d = 4, 8, 16, 32 as running sums over feature blocks
        GemmArgs g = gemm_base(x);
        GemmOperand a{};
        a.p = x.w(P.Y32, j0s[cc]);
        a.type = x.wt;
        a.bdiv = 1;
        a.sb1 = NT * JOLT_KMAX;
        a.rsh = 30;
        a.sr2 = JOLT_KMAX;
        a.ksh = ilog2(ws[cc]);
        a.sk1 = (int64_t)T * JOLT_KMAX;
        a.sk2 = 1;
        g.v[0].A = a;
        g.v[0].B = a;
        g.v[0].M = T;
        g.v[0].N = T;
        g.v[0].K = N * ws[cc];
        out_w(x, g, x.w(P.Mtok, cc * TT), T, T);
        g.Cin = cc > 0 ? x.w(P.Mtok, (cc - 1) * TT) : nullptr;
        g.csb1 = 5 * TT;
        g.acc64 = 1;
        g.mode = x.mode_any();
        g.alpha_norm = x.at<double>(P.xn2);
            HIPCHK(launch_gemm(g, x.x, nt, x.s));
      }
    }
    if (T <= 128) {
      HIPCHK(hipStreamWaitEvent(x.s, side.join, 0));
      HIPCHK(syev(x, M, x.f64, T, nb, UT, UT16, x.at<double>(P.lamT)));
    } else {
      // chains r_d = 4 .. 32 (subspace slots 4 t + chain): the first half of the tables here,
      // the second half on a second side stream (its launches are small, so the two halves
      // run side by side); r_d = D (slots 4 nt + t) on the first side stream
      const int64_t TT = (int64_t)T * T, TK = (int64_t)T * JOLT_KMAX;
      const int na = (nt + 1) / 2;
      SubspaceJob jm{x.s, 4 * na, 0, M, 4, 5 * TT, TT, UT, UT16, 5 * TK, TK, false};
      SubspaceJob jb{};
      SideStream s2;
      if (nt > na) {
        HIPCHK(side_stream(s2, 1));
        HIPCHK(hipEventRecord(s2.fork, x.s));
        HIPCHK(hipStreamWaitEvent(s2.s, s2.fork, 0));
        jb = SubspaceJob{s2.s, 4 * (nt - na), 4 * (int64_t)na, x.w(P.Mtok, (int64_t)na * 5 * TT), 4, 5 * TT, TT,
                         x.w(P.UT32, (int64_t)na * 5 * TK), UT16 + (int64_t)na * 5 * TK, 5 * TK, TK, false};
      }
      // first rounds of all three jobs (the r_d = D job's stream already holds its token Gram)
      SubspaceJob* first[3] = {&jd, &jm, &jb};
      jolt_status st = subspace_begin_n(x, first, nt > na ? 3 : 2, c->exact_iters);
      if (st != JOLT_OK) return st;
      HIPCHK(hipEventRecord(side.join, side.s));
      if (nt > na) HIPCHK(hipEventRecord(s2.join, s2.s));
      HIPCHK(hipStreamWaitEvent(x.s, side.join, 0));
      if (nt > na) HIPCHK(hipStreamWaitEvent(x.s, s2.join, 0));
      SubspaceJob* jobs[3] = {&jm, &jb, &jd};
      const hipEvent_t joins[3] = {nullptr, s2.join, side.join};
      st = subspace_converge(x, jobs, joins, 3, c->exact_iters);
      if (st != JOLT_OK) return st;
    }
  } else {
    // FlashJoLT randomized range finder on every (table, r_d)
    const int p = 40;
    const int64_t NDmax = (int64_t)N * D;
    void* S = x.w(P.Zs);
    void* Q = x.w(P.Qs);
    void* Pz = x.w(P.Pz);
    void* Pq = x.w(P.Pq);
    const int64_t omrows = (int64_t)N * (4 + 8 + 16 + 32 + D);
    HIPCHK(hipMemsetAsync(Pz, 0, (size_t)x.we * nb * NDmax * p, x.s));
    HIPCHK(hipMemsetAsync(Pq, 0, (size_t)x.we * nb * NDmax * p, x.s));
    // S = A B (B = the sketch, or the orthonormal basis Pq of the row space), then
    // orthonormalised in place.  Only the last basis is orthonormalised twice (CholeskyQR2:
    // S -> Q -> S), since U_T = S V and B = S^T A need it orthonormal to working precision;
    // the intermediate bases only carry their span to the next product, which one
    // CholeskyQR pass preserves as well as two (the second pass corrects orthogonality, not
    // span), and they are well conditioned after one pass.  fp64 factors keep two passes
    // everywhere (their generic-GEMM apply cannot run in place).
    // The chains go out in three launches so that each can take the GEMM's vector loaders:
    // r_d = 4 (only 4 contiguous values along k: the generic loader), r_d = 8 .. 32, and
    // the unprojected tensor (bf16 products, exact, when multiplied by the bf16 sketch).
    // Launch (c0, cnt) takes batch b = table * cnt + (chain - c0).
    const int groups[3][2] = {{0, 1}, {1, 3}, {4, 1}};
    // the shared operand (the sketch, or the row-space basis) as columns of contiguous rows:
    // lanes then load runs of k instead of values 40 apart
    const bool contigA = rf_token_contig(c);
    // the tensor chain's products run beside the r_d < D chains' (two streams) when the token
    // axis is one k slice of the A^T S kernels; for longer token axes each product fills the
    // chip alone and running two at once was slower (32k tokens: build +0.4 ms; 2048
    // tokens: -0.7 ms)
    const bool rf_side = xts_slices(T) == 1;
    auto apply_A = [&](bool omega, bool last) -> jolt_status {
      if (contigA && omega) {
        if (!xw_early) HIPCHK(launch_transpose_tc(nullptr, x.w(P.Om), true, 1, (int)omrows, p, nt, x.w(P.OmT), x.s));
      } else if (contigA) {
        HIPCHK(launch_transpose_tc(nullptr, Pq, false, 1, (int)NDmax, p, nb, x.w(P.PqT), x.s));
      }
      // the tensor chain's S = X Pq on the side stream, beside the r_d < D chains' products
      // on the main stream; joined before the orthonormalisation
      const bool xw_side = rf_side && contigA && !omega && NDmax % 8 == 0 &&
                           (uintptr_t)(x.at<float>(P.PqT) + 4 * NDmax * p) % 16 == 0;
      if (xw_side) {
        HIPCHK(side_stream(side));
        HIPCHK(hipEventRecord(side.fork, x.s));
        HIPCHK(hipStreamWaitEvent(side.s, side.fork, 0));
        HIPCHK(launch_xw(x.x, x.at<float>(P.PqT) + 4 * NDmax * p, false, 5 * NDmax * p, NDmax, N, T, D, nt,
                         x.at<float>(P.Zs) + 4 * (int64_t)T * p, 5 * (int64_t)T * p, side.s));
        HIPCHK(hipEventRecord(side.join, side.s));
      }
      bool yw_done = false;
      for (const auto& gr : groups) {
        const int c0 = gr[0], cnt = gr[1];
        if (c0 < 4 && contigA && !yw_done) {  // the four r_d < D chains from one pass over Y
          int64_t boff[4];
          for (int cc = 0, roff = 0; cc < 4; roff += N * (4 << cc), ++cc)
            boff[cc] = omega ? (int64_t)roff : (int64_t)cc * NDmax * p;
          const void* BT = omega ? (const void*)x.at<uint16_t>(P.OmT) : (const void*)x.at<float>(P.PqT);
          const int64_t btab = omega ? omrows * p : 5 * NDmax * p, bld = omega ? omrows : NDmax;
          bool fits = T % 128 == 0 && btab % 8 == 0 && bld % 8 == 0 && (uintptr_t)BT % 16 == 0;
          for (int cc = 0; cc < 4; ++cc) fits = fits && boff[cc] % 8 == 0;
          if (fits) {  // otherwise the GEMM below
            HIPCHK(launch_yw4(x.at<float>(P.Y32), BT, omega, btab, bld, boff, N, T, nt, x.at<float>(P.Zs),
                              5 * (int64_t)T * p, (int64_t)T * p, x.s));
            yw_done = true;
            continue;
          }
        }
        if (c0 < 4 && yw_done) continue;
        if (c0 == 4 && ((omega && xw_early) || xw_side)) {  // launched on the side stream: joined here
          HIPCHK(hipStreamWaitEvent(x.s, side.join, 0));
          continue;
        }
        if (c0 == 4 && contigA) {  // the tensor itself: its own kernel (same arithmetic as the GEMM)
          const int64_t roff4 = (int64_t)N * (4 + 8 + 16 + 32);
          const void* BT = omega ? (const void*)(x.at<uint16_t>(P.OmT) + roff4)
                                 : (const void*)(x.at<float>(P.PqT) + 4 * NDmax * p);
          const int64_t btab = omega ? omrows * p : 5 * NDmax * p, bld = omega ? omrows : NDmax;
          if (bld % 8 == 0 && btab % 8 == 0 && (uintptr_t)BT % 16 == 0) {
            HIPCHK(launch_xw(x.x, BT, omega, btab, bld, N, T, D, nt, x.at<float>(P.Zs) + 4 * (int64_t)T * p,
                             5 * (int64_t)T * p, x.s));
            continue;
          }
        }
        GemmArgs g = gemm_base(x);
        g.nvar = cnt;
        for (int v = 0; v < cnt; ++v) {
          const int cc = c0 + v;
          const int rd = cc < 4 ? (4 << cc) : D;
          int64_t roff = 0;
          for (int c2 = 0; c2 < cc; ++c2) roff += (int64_t)N * (c2 < 4 ? (4 << c2) : D);
          g.v[v].A = op_unfold(x, cc, cnt);
          if (omega) {
            GemmOperand o = contigA ? op_plain(x.at<uint16_t>(P.OmT) + roff, 1, omrows * p, omrows, 1)
                                    : op_plain(x.at<uint16_t>(P.Om) + roff * p, 1, omrows * p, 1, p);
            o.bdiv = cnt;
            g.v[v].B = o;
          } else {
            GemmOperand o = contigA ? op_plain(x.w(P.PqT), 0, 5 * NDmax * p, NDmax, 1)
                                    : wop(x, Pq, 5 * NDmax * p, 1, p);  // block (table, chain)
            o.bdiv = cnt;
            o.sb2 = NDmax * p;
            o.off0 = (int64_t)c0 * NDmax * p;
            g.v[v].B = o;
          }
          g.v[v].M = T;
          g.v[v].N = p;
          g.v[v].K = N * rd;
        }
        g.mode = (omega && c0 == 4) ? x.mode_bf16() : x.mode_any();
        out_w(x, g, x.w(P.Zs, (int64_t)c0 * T * p), T, p);
        g.cbdiv = cnt;
        g.csb1 = 5 * (int64_t)T * p;
        g.csb2 = (int64_t)T * p;
        g.xgrp = 1;  // operand shared by the unit's tiles: one XCD
        HIPCHK(launch_gemm(g, x.x, nt * cnt, x.s));
      }
      if (!last && !x.f64) return orth(x, S, S, T, p, nb);
      jolt_status st = orth(x, S, Q, T, p, nb);
      if (st != JOLT_OK) return st;
      return orth(x, Q, S, T, p, nb);
    };
    // P = A^T S  (rows n * r_d + j; rows beyond N r_d stay zero)
    const bool contig = rf_token_contig(c);
    auto apply_At = [&](void* dstP) -> jolt_status {
      const int groups_t[2][2] = {{0, 4}, {4, 1}};  // r_d < D, the tensor itself
      if (contig && rf_side) {
        // the tensor itself, X_n^T S per slice by its own kernel, on the side stream (its
        // partials in a buffer of their own), beside the r_d < D chains' Y_n^T S(r_d) on the
        // main stream (all four chains at once); joined before the result is read
        static_assert(p == 40, "sketch width of launch_xts");
        HIPCHK(side_stream(side));
        HIPCHK(hipEventRecord(side.fork, x.s));
        HIPCHK(hipStreamWaitEvent(side.s, side.fork, 0));
        HIPCHK(launch_xts(x.x, (const float*)S + (int64_t)4 * T * p, 5 * (int64_t)T * p, N, T, D, nt,
                          x.at<float>(P.XSp2), (float*)dstP + (int64_t)4 * NDmax * p, 5 * NDmax * p, side.s));
        HIPCHK(hipEventRecord(side.join, side.s));
        HIPCHK(launch_yts(x.at<float>(P.Y32), (const float*)S, N, T, nt, x.at<float>(P.XSp), (float*)dstP,
                          NDmax * p, x.s));
        HIPCHK(hipStreamWaitEvent(x.s, side.join, 0));
        return JOLT_OK;
      }
      for (const auto& gr : groups_t) {
        const int c0 = gr[0], cnt = gr[1];
        if (c0 == 0 && contig) {  // r_d < D: Y_n^T S(r_d) per slice, all four chains at once
          HIPCHK(launch_yts(x.at<float>(P.Y32), (const float*)S, N, T, nt, x.at<float>(P.XSp), (float*)dstP,
                            NDmax * p, x.s));
          continue;
        }
        if (c0 == 4 && contig) {  // the tensor itself: X_n^T S per slice by its own kernel
          HIPCHK(launch_xts(x.x, (const float*)S + (int64_t)4 * T * p, 5 * (int64_t)T * p, N, T, D, nt,
                            x.at<float>(P.XSp), (float*)dstP + (int64_t)4 * NDmax * p, 5 * NDmax * p, x.s));
          continue;
        }
        GemmArgs g = gemm_base(x);
        g.nvar = cnt;
        for (int v = 0; v < cnt; ++v) {
          const int cc = c0 + v;
          const int rd = cc < 4 ? (4 << cc) : D;
          g.v[v].A = op_unfold_t(x, cc, cnt);
          GemmOperand o = wop(x, S, 5 * (int64_t)T * p, 1, p);
          o.bdiv = cnt;
          o.sb2 = (int64_t)T * p;
          o.off0 = (int64_t)c0 * T * p;
          g.v[v].B = o;
          g.v[v].M = N * rd;
          g.v[v].N = p;
          g.v[v].K = T;
        }
        g.mode = x.mode_any();
        out_w(x, g, (char*)dstP + (size_t)x.we * c0 * NDmax * p, NDmax, p);
        g.cbdiv = cnt;
        g.csb1 = 5 * NDmax * p;
        g.csb2 = NDmax * p;
        g.xgrp = 1;  // operand shared by the unit's tiles: one XCD
        HIPCHK(launch_gemm(g, x.x, nt * cnt, x.s));
      }
      return JOLT_OK;
    };
    jolt_status st = apply_A(true, c->power_iters == 0);
    if (st != JOLT_OK) return st;
    for (int it = 0; it < c->power_iters; ++it) {
      // the row-space basis Pq = orth(A^T S) (one pass; two with fp64 factors)
      st = apply_At(Pz);
      if (st != JOLT_OK) return st;
      if (x.f64) {
        st = orth(x, Pz, Pq, NDmax, p, nb);
        if (st != JOLT_OK) return st;
        st = orth(x, Pq, Pz, NDmax, p, nb);
        if (st != JOLT_OK) return st;
        HIPCHK(hipMemcpyAsync(Pq, Pz, (size_t)x.we * nb * NDmax * p, hipMemcpyDeviceToDevice, x.s));
      } else {
        st = orth(x, Pz, Pq, NDmax, p, nb);
        if (st != JOLT_OK) return st;
      }
      st = apply_A(false, it == c->power_iters - 1);
      if (st != JOLT_OK) return st;
    }
    // B^T = A^T S; B B^T = (A^T S)^T (A^T S) (40 x 40); its eigenvectors are the left
    // singular vectors of B
    st = apply_At(Pz);
    if (st != JOLT_OK) return st;
    {  // the Gram in fp64 from row-chunk partials (the orthonormalisations' buffers are free)
      const int nsplit = orth_parts(NDmax);
      HIPCHK(launch_gram64(Pz, x.f64, NDmax, p, nsplit, nb, x.at<double>(P.Wp), x.s));
      HIPCHK(launch_sum_parts(x.at<double>(P.Wp), nsplit, p * p, nb, x.at<double>(P.Hrr), x.s));
    }
    HIPCHK(syev(x, x.at<double>(P.Hrr), true, p, nb, x.w(P.Vrr), nullptr, x.at<double>(P.lamT)));
    if (!x.f64) {  // U_T = S V row by row (fp32)
      HIPCHK(launch_ut_rows((const float*)S, x.at<float>(P.Vrr), p, T, nb, (float*)UT, UT16, 1,
                            (int64_t)T * JOLT_KMAX, 0, x.s));
    } else {
      GemmArgs u = gemm_base(x);
      u.v[0].A = wop(x, S, (int64_t)T * p, p, 1);
      u.v[0].B = wop(x, x.w(P.Vrr), (int64_t)p * JOLT_KMAX, 1, JOLT_KMAX);
      u.v[0].M = T;
      u.v[0].N = JOLT_KMAX;
      u.v[0].K = p;
      u.mode = x.mode_any();
      out_w(x, u, UT, T, JOLT_KMAX);
      u.C16 = UT16;
      u.xgrp = 1;  // operand shared by the unit's tiles: one XCD
      HIPCHK(launch_gemm(u, x.x, nb, x.s));
    }
  }
  if (!cores) {  // spectra only (modelled tables): the side stream has been joined above
    return JOLT_OK;
  }
  // ---- cores G_n = U_T^T Y_n(r_d) of the r_d chains as fp16 storage copies: fp32 working
  // precision at D = 128 by the all-chain kernel (one workgroup per table and slice)
  if (cores_make_w(x) && c->token_mode == JOLT_TOKEN_RANDOMIZED) {
    // from the finder's last product P = A^T Q and U_T = Q V: G_n = V^T P_n^T (no pass over
    // the tensor)
    HIPCHK(launch_cores_rr(x.at<float>(P.Vrr), x.at<float>(P.Pz), (int64_t)N * D * 40, N, D, nt,
                           x.at<_Float16>(P.G16), x.at<int32_t>(P.flags), x.at<float>(P.V32), signs_dev,
                           x.at<_Float16>(P.Wh), x.at<_Float16>(P.Wl), x.s));
    return JOLT_OK;
  }
  if (cores_make_w(x)) {  // and the score pass's reconstruction operands
    HIPCHK(launch_cores(x.at<float>(P.UT32), x.at<float>(P.Y32), x.x, N, T, D, nt, x.at<_Float16>(P.G16),
                        x.at<int32_t>(P.flags), x.at<float>(P.V32), signs_dev, x.at<_Float16>(P.Wh),
                        x.at<_Float16>(P.Wl), P.CoP ? x.at<double>(P.CoP) : nullptr, x.s));
    return JOLT_OK;
  }
  // otherwise one generic GEMM launch: batch b = (table * 5 + chain) * N + n, variant = chain
  {
    GemmArgs g = gemm_base(x);
    g.nvar = 5;
    g.vdiv = N;
    for (int cc = 0; cc < 5; ++cc) {
      const int rd = cc < 4 ? (4 << cc) : D;
      GemmOperand a = wop(x, UT, (int64_t)T * JOLT_KMAX, 1, JOLT_KMAX);  // b / N = table * 5 + chain
      a.bdiv = N;
      g.v[cc].A = a;
      GemmOperand bo{};
      bo.novar = 1;  // b' = table * N + n
      bo.bdiv = N;
      bo.rsh = 30;
      bo.sr2 = 1;
      bo.ksh = 30;
      if (cc < 4) {
        bo.p = x.w(P.Y32);
        bo.type = x.wt;
        bo.sb1 = NT * JOLT_KMAX;
        bo.sb2 = (int64_t)T * JOLT_KMAX;
        bo.sk2 = JOLT_KMAX;
      } else {
        bo.tbl = 1;
        bo.type = 1;
        bo.sb2 = (int64_t)T * D;
        bo.sk2 = D;
      }
      g.v[cc].B = bo;
      g.v[cc].M = JOLT_KMAX;
      g.v[cc].N = rd;
      g.v[cc].K = T;
    }
    g.mode = x.mode_any();
    g.C = x.w(P.Gc);
    g.c_type = x.f64 ? 1 : 0;
    g.csb1 = (int64_t)JOLT_KMAX * D;
    g.csm = D;
    g.csn = 1;
    g.C16 = x.at<_Float16>(P.G16);
    g.flags = x.at<int32_t>(P.flags);
    g.xgrp = N;  // operand shared by the unit's tiles: one XCD
    HIPCHK(launch_gemm(g, x.x, nt * 5 * N, x.s));
  }
  return JOLT_OK;
}

// Launch timer of the score kernel (benchmark support)
struct KernelTimer {
  bool on = false;
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev;
};
std::mutex g_timer_mu;
KernelTimer g_score_timer;

hipError_t timed_score(const ScoreArgs& sa, const TablePtrs& x, hipStream_t s) {
  std::lock_guard<std::mutex> lk(g_timer_mu);
  if (!g_score_timer.on) return launch_score(sa, x, s);
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t err = hipEventCreate(&e0);
  if (err == hipSuccess) err = hipEventCreate(&e1);
  if (err == hipSuccess) err = hipEventRecord(e0, s);
  if (err == hipSuccess) err = launch_score(sa, x, s);
  if (err == hipSuccess) err = hipEventRecord(e1, s);
  if (err != hipSuccess) {
    if (e0) (void)hipEventDestroy(e0);
    if (e1) (void)hipEventDestroy(e1);
    return err;
  }
  g_score_timer.ev.emplace_back(e0, e1);
  return hipSuccess;
}

// How the last call that computed factors in a workspace obtained its token factors.
std::mutex g_info_mu;
std::unordered_map<const void*, jolt_factor_info> g_info;
void info_set(const Ctx& x) {
  jolt_factor_info f;
  const bool sub = x.c->token_mode == JOLT_TOKEN_EXACT && x.c->T > 128;
  f.iterations = x.c->token_mode == JOLT_TOKEN_EXACT ? (sub ? x.exact_iters_used : 0) : x.c->power_iters;
  f.converged = sub ? x.exact_converged : 1;
  f.max_residual = sub ? x.exact_residual : 0.0;
  std::lock_guard<std::mutex> lk(g_info_mu);
  g_info[x.ws] = f;
}

// Which inputs the factors held by a workspace belong to: set when a call has computed
// them, cleared when a call starts overwriting the workspace.
struct FactorStamp {
  jolt_config cfg;
  std::vector<const void*> x;
  const int8_t* signs;
  size_t bytes;
};
std::mutex g_stamp_mu;
std::unordered_map<const void*, FactorStamp> g_stamps;

void stamp_clear(const void* ws) {
  std::lock_guard<std::mutex> lk(g_stamp_mu);
  g_stamps.erase(ws);
}
void stamp_set(const Ctx& x, const int8_t* signs, size_t bytes) {
  FactorStamp f;
  f.cfg = *x.c;
  f.x.assign(x.x.p, x.x.p + x.c->n_tables);
  f.signs = signs;
  f.bytes = bytes;
  std::lock_guard<std::mutex> lk(g_stamp_mu);
  g_stamps[x.ws] = f;
}
bool stamp_matches(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs, const void* ws,
                   size_t bytes) {
  std::lock_guard<std::mutex> lk(g_stamp_mu);
  auto it = g_stamps.find(ws);
  if (it == g_stamps.end()) return false;
  const FactorStamp& f = it->second;
  if (memcmp(&f.cfg, cfg, sizeof(jolt_config)) != 0 || f.signs != signs || f.bytes != bytes) return false;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (f.x[t] != x_dev[t]) return false;
  return true;
}

jolt_status prepare(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                    const void* const* omega_dev, void* workspace, size_t workspace_bytes, hipStream_t s,
                    Ctx& x) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!x_dev || !signs_dev || !workspace) return JOLT_EINVAL;
  if (cfg->token_mode == JOLT_TOKEN_RANDOMIZED && !omega_dev) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (!x_dev[t] || (cfg->token_mode == JOLT_TOKEN_RANDOMIZED && !omega_dev[t])) return JOLT_EINVAL;
  x.c = cfg;
  x.p = make_plan(cfg);
  x.f64 = precise_factors(cfg);
  x.wt = x.f64 ? 3 : 0;
  x.we = x.f64 ? 8 : 4;
  if (workspace_bytes < x.p.total) return JOLT_ENOMEM;
  x.ws = (char*)workspace;
  stamp_clear(workspace);
  x.s = s;
  memset(&x.x, 0, sizeof(x.x));
  for (int t = 0; t < cfg->n_tables; ++t) x.x.p[t] = x_dev[t];
  if (cfg->token_mode == JOLT_TOKEN_RANDOMIZED) {
    const size_t per = sizeof(uint16_t) * (size_t)cfg->N * (4 + 8 + 16 + 32 + cfg->D) * 40;
    for (int t = 0; t < cfg->n_tables; ++t)
      HIPCHK(hipMemcpyAsync(x.ws + x.p.Om + per * t, omega_dev[t], per, hipMemcpyDeviceToDevice, s));
  }
  return JOLT_OK;
}

}  // namespace

extern "C" {

void jolt_default_config(jolt_config* cfg, int32_t N, int32_t T, int32_t D, int32_t n_tables) {
  if (!cfg) return;
  cfg->N = N;
  cfg->T = T;
  cfg->D = D;
  cfg->n_tables = n_tables;
  cfg->quant_block = D;
  cfg->s_bytes = 2;
  cfg->align_bytes = 256;
  cfg->token_mode = JOLT_TOKEN_EXACT;
  cfg->q_cap = 32;
  cfg->oversample = 8;
  cfg->power_iters = 2;
  cfg->exact_iters = 12;
  cfg->factor_precision = 0;
  cfg->exact_max_iters = 64;
}

jolt_status jolt_last_build_info(const void* workspace, jolt_factor_info* info_out) {
  if (!workspace || !info_out) return JOLT_EINVAL;
  std::lock_guard<std::mutex> lk(g_info_mu);
  auto it = g_info.find(workspace);
  if (it == g_info.end()) return JOLT_EINVAL;
  *info_out = it->second;
  return JOLT_OK;
}

const char* jolt_status_string(jolt_status s) {
  switch (s) {
    case JOLT_OK: return "ok";
    case JOLT_EINVAL: return "invalid argument or unsupported configuration";
    case JOLT_ENOMEM: return "workspace too small";
    case JOLT_EDEVICE: return "HIP runtime error";
    case JOLT_EINFEASIBLE: return "budget below the cheapest allocation";
    case JOLT_ERANGE: return "fp16 storage overflow";
    case JOLT_ENONFINITE: return "non-finite input";
  }
  return "unknown status";
}

jolt_status jolt_workspace_size(const jolt_config* cfg, size_t* bytes_out) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!bytes_out) return JOLT_EINVAL;
  *bytes_out = make_plan(cfg).total;
  return JOLT_OK;
}

jolt_status jolt_cost_table(const jolt_config* cfg, uint64_t* C_out) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!C_out) return JOLT_EINVAL;
  for (int i = 0; i < JOLT_N_CAND; ++i) C_out[i] = cand_cost(cfg, i);
  return JOLT_OK;
}

jolt_status jolt_record_bytes(const jolt_config* cfg, int32_t cand, uint64_t* bytes_out) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!bytes_out || cand < 0 || cand >= JOLT_N_CAND) return JOLT_EINVAL;
  *bytes_out = cand_cost(cfg, cand);
  return JOLT_OK;
}

static ScoreArgs score_args(const Ctx& x, const int8_t* signs_dev) {
  const jolt_config* cfg = x.c;
  ScoreArgs sa{};
  sa.N = cfg->N;
  sa.T = cfg->T;
  sa.D = cfg->D;
  sa.ntab = cfg->n_tables;
  sa.signs = signs_dev;
  sa.UT16 = x.at<_Float16>(x.p.UT16);
  sa.G16T = x.at<_Float16>(x.p.G16T);
  sa.Wneg_hi = x.at<_Float16>(x.p.Wh);
  sa.Wneg_lo = x.at<_Float16>(x.p.Wl);
  sa.Vneg_hi = x.at<_Float16>(x.p.Vh);
  sa.Vneg_lo = x.at<_Float16>(x.p.Vl);
  sa.part = x.at<double>(x.p.part);
  return sa;
}

// Pinned host staging for the small results a build brings back (flags, norms, error sums),
// one buffer per host thread, grown when needed and kept until the process ends (it is not
// freed at exit, when the runtime may already be gone).  nullptr when pinned memory is not
// available: the caller then copies into pageable memory.
static thread_local void* g_pin = nullptr;
static thread_local size_t g_pin_bytes = 0;
static void* pinned_staging(size_t bytes) {
  if (g_pin_bytes >= bytes) return g_pin;
  if (g_pin) (void)hipHostFree(g_pin);  // the previous call synchronised its copy
  g_pin = nullptr;
  g_pin_bytes = 0;
  void* p = nullptr;
  if (hipHostMalloc(&p, bytes, hipHostMallocDefault) != hipSuccess) return nullptr;
  g_pin = p;
  g_pin_bytes = bytes;
  return p;
}

jolt_status jolt_build_tables(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                              const void* const* omega_dev, double* D_out, uint64_t* C_out, double* xnorm2_out,
                              void* workspace, size_t workspace_bytes, jolt_stream_t stream) {
  if (!D_out || !C_out) return JOLT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  Ctx x;
  jolt_status st = prepare(cfg, x_dev, signs_dev, omega_dev, workspace, workspace_bytes, s, x);
  if (st != JOLT_OK) return st;
  const int nt = cfg->n_tables;
  st = run_factors(x, signs_dev);
  if (st != JOLT_OK) return st;
  info_set(x);
  if (!cores_make_w(x))
    HIPCHK(launch_prep_w(x.at<_Float16>(x.p.G16), x.at<float>(x.p.V32), signs_dev, cfg->N, cfg->D, nt,
                         x.at<_Float16>(x.p.Wh), x.at<_Float16>(x.p.Wl), x.at<int32_t>(x.p.flags), s));
  const ScoreArgs sa = score_args(x, signs_dev);
  HIPCHK(timed_score(sa, x.x, s));
  const int nwg = score_partials(cfg->N, cfg->T);
  HIPCHK(launch_score_reduce(x.at<double>(x.p.part), nwg, nt, x.at<double>(x.p.E), s));
  std::vector<double> E((size_t)nt * 100), xn2(nt);
  int32_t flags = 0;
  // flags, norms and error sums are consecutive in the workspace: one copy into pinned memory
  const size_t span = x.p.E + sizeof(double) * E.size() - x.p.flags;
  char* pin = (x.p.flags < x.p.xn2 && x.p.xn2 < x.p.E) ? (char*)pinned_staging(span) : nullptr;
  if (pin) {
    HIPCHK(hipMemcpyAsync(pin, x.ws + x.p.flags, span, hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
    memcpy(&flags, pin, sizeof(int32_t));
    memcpy(xn2.data(), pin + (x.p.xn2 - x.p.flags), sizeof(double) * nt);
    memcpy(E.data(), pin + (x.p.E - x.p.flags), sizeof(double) * E.size());
  } else {
    HIPCHK(hipMemcpyAsync(E.data(), x.at<double>(x.p.E), sizeof(double) * E.size(), hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(xn2.data(), x.at<double>(x.p.xn2), sizeof(double) * nt, hipMemcpyDeviceToHost, s));
    HIPCHK(hipMemcpyAsync(&flags, x.at<int32_t>(x.p.flags), sizeof(int32_t), hipMemcpyDeviceToHost, s));
    HIPCHK(hipStreamSynchronize(s));
  }
  if (flags & 2) return JOLT_ENONFINITE;
  for (int t = 0; t < nt; ++t)
    if (!isfinite(xn2[t])) return JOLT_ENONFINITE;
  if (flags & 1) return JOLT_ERANGE;
  for (int t = 0; t < nt; ++t) {
    for (int i = 0; i < JOLT_N_CAND; ++i) {
      const double d = xn2[t] > 0.0 ? E[(size_t)t * 100 + i] / xn2[t] : 0.0;
      if (!isfinite(d)) return JOLT_ENONFINITE;
      D_out[(size_t)t * JOLT_N_CAND + i] = d;
      C_out[(size_t)t * JOLT_N_CAND + i] = cand_cost(cfg, i);
    }
    if (xnorm2_out) xnorm2_out[t] = xn2[t];
  }
  stamp_set(x, signs_dev, workspace_bytes);  // only a build that succeeded leaves reusable factors
  return JOLT_OK;
}

static uint64_t choose_all(const double* D, const uint64_t* C, int nt, int nc, double lam, int32_t* ch) {
  uint64_t tot = 0;
  for (int t = 0; t < nt; ++t) {
    int best = 0;
    double bl = D[(size_t)t * nc] + lam * (double)C[(size_t)t * nc];
    for (int i = 1; i < nc; ++i) {
      const double l = D[(size_t)t * nc + i] + lam * (double)C[(size_t)t * nc + i];
      const uint64_t ci = C[(size_t)t * nc + i], cb = C[(size_t)t * nc + best];
      if (l < bl || (l == bl && ci < cb)) {
        best = i;
        bl = l;
      }
    }
    ch[t] = best;
    tot += C[(size_t)t * nc + best];
  }
  return tot;
}

// Slopes (D_a - D_b) / (C_b - C_a) between consecutive vertices of every table's lower
// convex hull of the points (C_i, D_i), from the cheapest point to the least distorted one;
// sorted ascending, duplicates removed.
static std::vector<double> hull_slopes(const double* D, const uint64_t* C, int nt, int nc) {
  std::vector<double> out;
  std::vector<int> byc(nc), idx(nc), hull;
  for (int t = 0; t < nt; ++t) {
    const double* Dt = D + (size_t)t * nc;
    const uint64_t* Ct = C + (size_t)t * nc;
    // candidates in the order (C, D, index): the order by (C, index) is shared by tables with
    // the same cost row (the usual case), then each run of equal C is ordered by (D, index)
    if (t == 0 || memcmp(Ct, Ct - nc, sizeof(uint64_t) * nc) != 0) {
      for (int i = 0; i < nc; ++i) byc[i] = i;
      std::sort(byc.begin(), byc.end(), [&](int a, int b) { return Ct[a] != Ct[b] ? Ct[a] < Ct[b] : a < b; });
    }
    idx = byc;
    for (int r0 = 0; r0 < nc;) {
      int r1 = r0 + 1;
      while (r1 < nc && Ct[idx[r1]] == Ct[idx[r0]]) ++r1;
      for (int k = r0 + 1; k < r1; ++k) {  // insertion sort of the run by (D, index)
        const int v = idx[k];
        int j = k;
        while (j > r0 && (Dt[idx[j - 1]] != Dt[v] ? Dt[idx[j - 1]] > Dt[v] : idx[j - 1] > v)) {
          idx[j] = idx[j - 1];
          --j;
        }
        idx[j] = v;
      }
      r0 = r1;
    }
    hull.clear();
    double dmin = 0.0;
    for (int k = 0; k < nc; ++k) {
      const int i = idx[k];
      if (!hull.empty() && !(Dt[i] < dmin)) continue;  // no better than a cheaper point
      dmin = Dt[i];
      while (hull.size() >= 2) {  // drop the middle point unless the chain turns strictly convex
        const int a = hull[hull.size() - 2], b = hull.back();
        const double s1 = (Dt[a] - Dt[b]) / (double)(Ct[b] - Ct[a]);
        const double s2 = (Dt[b] - Dt[i]) / (double)(Ct[i] - Ct[b]);
        if (s2 < s1) break;
        hull.pop_back();
      }
      hull.push_back(i);
    }
    for (size_t k = 1; k < hull.size(); ++k) {
      const int a = hull[k - 1], b = hull[k];
      out.push_back((Dt[a] - Dt[b]) / (double)(Ct[b] - Ct[a]));
    }
  }
  std::sort(out.begin(), out.end());
  out.erase(std::unique(out.begin(), out.end()), out.end());
  return out;
}

jolt_status jolt_allocate(const double* D, const uint64_t* C, int32_t n_tables, int32_t n_cand, uint64_t budget,
                          int32_t* choice_out, double* lambda_out, uint64_t* total_out) {
  if (!D || !C || !choice_out || n_tables < 1 || n_cand < 1) return JOLT_EINVAL;
  uint64_t minsum = 0;
  for (int t = 0; t < n_tables; ++t) {
    uint64_t m = C[(size_t)t * n_cand];
    for (int i = 0; i < n_cand; ++i) {
      if (!isfinite(D[(size_t)t * n_cand + i]) || D[(size_t)t * n_cand + i] < 0.0) return JOLT_EINVAL;
      m = C[(size_t)t * n_cand + i] < m ? C[(size_t)t * n_cand + i] : m;
    }
    minsum += m;
  }
  if (minsum > budget) return JOLT_EINFEASIBLE;
  std::vector<int32_t> ch(n_tables);
  double lam = 0.0;
  uint64_t tot = choose_all(D, C, n_tables, n_cand, 0.0, ch.data());
  if (tot > budget) {
    // The chosen total is a non-increasing step function of the price that changes only
    // at the slopes between consecutive vertices of a table's lower convex hull of
    // (C, D), and takes the lower-cost side there.  lambda+ is therefore the smallest such
    // slope whose allocation fits; it is found by binary search over the sorted slopes,
    // each evaluated just above the slope (relative 1e-12) so that rounding cannot put a
    // tie on the expensive side.
    std::vector<double> bps = hull_slopes(D, C, n_tables, n_cand);
    const double up = 1.0 + 1e-12;
    size_t lo = 0, hi = bps.size();  // the answer lies in [lo, hi); at the largest slope it fits
    if (bps.empty()) return JOLT_EINFEASIBLE;
    hi = bps.size() - 1;
    while (lo < hi) {
      const size_t mid = lo + (hi - lo) / 2;
      if (choose_all(D, C, n_tables, n_cand, bps[mid] * up, ch.data()) <= budget)
        hi = mid;
      else
        lo = mid + 1;
    }
    lam = bps[lo] * up;
    tot = choose_all(D, C, n_tables, n_cand, lam, ch.data());
    if (tot > budget) return JOLT_EINFEASIBLE;
  }
  for (int t = 0; t < n_tables; ++t) choice_out[t] = ch[t];
  if (lambda_out) *lambda_out = lam;
  if (total_out) *total_out = tot;
  return JOLT_OK;
}

static bool valid_tables(const double* D, int32_t n_tables, int32_t n_cand) {
  for (size_t i = 0; i < (size_t)n_tables * n_cand; ++i)
    if (!isfinite(D[i]) || D[i] < 0.0) return false;
  return true;
}

jolt_status jolt_refine_swap(const double* D, const uint64_t* C, int32_t n_tables, int32_t n_cand, uint64_t budget,
                             int32_t* choice_inout, uint64_t* total_out, int32_t* moves_out) {
  if (!D || !C || !choice_inout || n_tables < 1 || n_cand < 1 || !valid_tables(D, n_tables, n_cand))
    return JOLT_EINVAL;
  std::vector<int32_t> ch(choice_inout, choice_inout + n_tables);
  uint64_t total = 0;
  for (int t = 0; t < n_tables; ++t) {
    if (ch[t] < 0 || ch[t] >= n_cand) return JOLT_EINVAL;
    total += C[(size_t)t * n_cand + ch[t]];
  }
  if (total > budget) return JOLT_EINVAL;
  int32_t moves = 0;
  for (;;) {
    bool found = false, bfree = false;
    double bscore = 0.0;
    int bt = -1, bi = -1;
    for (int t = 0; t < n_tables; ++t) {
      const double* Dt = D + (size_t)t * n_cand;
      const uint64_t* Ct = C + (size_t)t * n_cand;
      const double dc = Dt[ch[t]];
      const uint64_t cc = Ct[ch[t]];
      for (int i = 0; i < n_cand; ++i) {
        const double dn = Dt[i];
        const uint64_t cn = Ct[i];
        if (!(dn < dc) || total - cc + cn > budget) continue;
        const bool fr = cn <= cc;
        const double score = fr ? dc - dn : (dc - dn) / (double)(cn - cc);
        if (!found || (fr && !bfree) || (fr == bfree && score > bscore)) {
          found = true;
          bfree = fr;
          bscore = score;
          bt = t;
          bi = i;
        }
      }
    }
    if (!found) break;
    total = total - C[(size_t)bt * n_cand + ch[bt]] + C[(size_t)bt * n_cand + bi];
    ch[bt] = bi;
    ++moves;
  }
  for (int t = 0; t < n_tables; ++t) choice_inout[t] = ch[t];
  if (total_out) *total_out = total;
  if (moves_out) *moves_out = moves;
  return JOLT_OK;
}

jolt_status jolt_allocate_common(const double* D, const uint64_t* C, int32_t n_tables, int32_t n_cand,
                                 uint64_t budget, const uint8_t* allowed, int32_t* cand_out, uint64_t* total_out,
                                 double* dist_out) {
  if (!D || !C || !cand_out || n_tables < 1 || n_cand < 1 || !valid_tables(D, n_tables, n_cand)) return JOLT_EINVAL;
  int best = -1;
  double bdist = 0.0;
  uint64_t bcost = 0;
  for (int i = 0; i < n_cand; ++i) {
    if (allowed && !allowed[i]) continue;
    uint64_t cost = 0;
    double dist = 0.0;
    for (int t = 0; t < n_tables; ++t) {
      cost += C[(size_t)t * n_cand + i];
      dist += D[(size_t)t * n_cand + i];
    }
    if (cost > budget) continue;
    if (best < 0 || dist < bdist || (dist == bdist && cost < bcost)) {
      best = i;
      bdist = dist;
      bcost = cost;
    }
  }
  if (best < 0) return JOLT_EINFEASIBLE;
  *cand_out = best;
  if (total_out) *total_out = bcost;
  if (dist_out) *dist_out = bdist;
  return JOLT_OK;
}

jolt_status jolt_model_tables(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                              const void* const* omega_dev, const float* gauss_dev, int32_t gauss_rows, double* D_out,
                              uint64_t* C_out, double* xnorm2_out, double* eps2_out, void* workspace,
                              size_t workspace_bytes, jolt_stream_t stream) {
  if (!D_out || !C_out || !gauss_dev || gauss_rows < 1 || gauss_rows > 65536) return JOLT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  Ctx x;
  jolt_status st = prepare(cfg, x_dev, signs_dev, omega_dev, workspace, workspace_bytes, s, x);
  if (st != JOLT_OK) return st;
  if ((size_t)gauss_rows * 4 * sizeof(double) > x.p.gscr_bytes) return JOLT_EINVAL;
  const int nt = cfg->n_tables, T = cfg->T, D = cfg->D, nb = nt * 5;
  st = run_factors(x, signs_dev, false);
  if (st != JOLT_OK) return st;
  info_set(x);
  double* epart = x.at<double>(x.p.gscr);
  HIPCHK(launch_eps2(gauss_dev, gauss_rows, D, epart, s));
  std::vector<double> lamd((size_t)nt * JOLT_KMAX), lamT((size_t)nb * JOLT_KMAX), xn2(nt), ep((size_t)gauss_rows * 4);
  int32_t flags = 0;
  HIPCHK(hipMemcpyAsync(lamd.data(), x.at<double>(x.p.lamd), sizeof(double) * lamd.size(), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(lamT.data(), x.at<double>(x.p.lamT), sizeof(double) * lamT.size(), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(xn2.data(), x.at<double>(x.p.xn2), sizeof(double) * nt, hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(ep.data(), epart, sizeof(double) * ep.size(), hipMemcpyDeviceToHost, s));
  HIPCHK(hipMemcpyAsync(&flags, x.at<int32_t>(x.p.flags), sizeof(int32_t), hipMemcpyDeviceToHost, s));
  HIPCHK(hipStreamSynchronize(s));
  if (flags & 2) return JOLT_ENONFINITE;
  for (int t = 0; t < nt; ++t)
    if (!isfinite(xn2[t])) return JOLT_ENONFINITE;
  // eps^2(b): error sums over the calibration rows, in row order
  double e[4] = {0.0, 0.0, 0.0, 0.0};
  for (int r = 0; r < gauss_rows; ++r)
    for (int k = 0; k < 4; ++k) e[k] += ep[(size_t)r * 4 + k];
  const double eps2[4] = {1.0, e[0] > 0 ? e[1] / e[0] : 0.0, e[0] > 0 ? e[2] / e[0] : 0.0,
                          e[0] > 0 ? e[3] / e[0] : 0.0};
  const bool exact = cfg->token_mode == JOLT_TOKEN_EXACT;
  for (int t = 0; t < nt; ++t) {
    const double xn = xn2[t];
    // the exact-mode token Grams carry the power-of-two scale 2^(14 - e), ||X||^2 = f 2^e
    double tscale = 1.0;
    if (exact && xn > 0.0) {
      int ex = 0;
      (void)frexp(xn, &ex);
      tscale = (double)ldexpf(1.0f, 14 - ex);  // the fp32 factor the Gram launches applied
    }
    for (int i = 0; i < JOLT_N_CAND; ++i) {
      int rT, rd, b, irT, ird;
      cand_params(cfg, i, rT, rd, b, irT, ird);
      double tau = 0.0;
      if (!(rT == T && rd == D) && xn > 0.0) {
        double total = xn;
        if (rd < D) {
          total = 0.0;
          for (int k = 0; k < rd; ++k) total += lamd[(size_t)t * JOLT_KMAX + k];
        }
        double captured = total;
        if (rT < T) {
          size_t slot;
          if (exact && T > 128) slot = ird < 4 ? (size_t)t * 4 + ird : (size_t)4 * nt + t;
          else slot = (size_t)t * 5 + ird;
          captured = 0.0;
          for (int k = 0; k < rT; ++k) captured += lamT[slot * JOLT_KMAX + k];
          captured /= tscale;
        }
        tau = (xn - captured) / xn;
        if (!(tau > 0.0)) tau = 0.0;
      }
      const int ib = b == 0 ? 0 : (b == 2 ? 1 : (b == 4 ? 2 : 3));
      if (!isfinite(tau)) return JOLT_ENONFINITE;
      D_out[(size_t)t * JOLT_N_CAND + i] = eps2[ib] * tau;
      C_out[(size_t)t * JOLT_N_CAND + i] = cand_cost(cfg, i);
    }
    if (xnorm2_out) xnorm2_out[t] = xn;
  }
  if (eps2_out)
    for (int k = 0; k < 4; ++k) eps2_out[k] = eps2[k];
  return JOLT_OK;
}

static jolt_status encode_records(const Ctx& x, const void* const* x_dev, const int8_t* signs_dev,
                                  const int32_t* choice, void* const* rec_dev) {
  const jolt_config* cfg = x.c;
  for (int t0 = 0; t0 < cfg->n_tables; t0 += JOLT_TAB_CHUNK) {
    EncodeArgs a;
    memset(&a, 0, sizeof(a));
    a.N = cfg->N;
    a.T = cfg->T;
    a.D = cfg->D;
    a.t0 = t0;
    a.ntab = cfg->n_tables - t0 < JOLT_TAB_CHUNK ? cfg->n_tables - t0 : JOLT_TAB_CHUNK;
    a.signs = signs_dev;
    a.UT16 = x.at<_Float16>(x.p.UT16);
    a.Ud16 = x.at<_Float16>(x.p.Ud16);
    a.G16 = x.at<_Float16>(x.p.G16);
    a.G16T = x.at<_Float16>(x.p.G16T);
    for (int i = 0; i < a.ntab; ++i) {
      a.t[i] = record_layout(cfg, choice[t0 + i]);
      a.t[i].rec = (char*)rec_dev[t0 + i];
      a.xsrc[i] = x_dev[t0 + i];
    }
    HIPCHK(launch_encode(a, x.s));
  }
  return JOLT_OK;
}

static jolt_status check_choice(const jolt_config* cfg, const int32_t* choice, void* const* rec_dev) {
  if (!choice || !rec_dev) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (choice[t] < 0 || choice[t] >= JOLT_N_CAND || !rec_dev[t]) return JOLT_EINVAL;
  return JOLT_OK;
}

jolt_status jolt_encode(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                        const void* const* omega_dev, const int32_t* choice, void* const* rec_dev, void* workspace,
                        size_t workspace_bytes, jolt_stream_t stream) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  st = check_choice(cfg, choice, rec_dev);
  if (st != JOLT_OK) return st;
  hipStream_t s = (hipStream_t)stream;
  Ctx x;
  st = prepare(cfg, x_dev, signs_dev, omega_dev, workspace, workspace_bytes, s, x);
  if (st != JOLT_OK) return st;
  st = run_factors(x, signs_dev);
  if (st != JOLT_OK) return st;
  info_set(x);
  stamp_set(x, signs_dev, workspace_bytes);
  return encode_records(x, x_dev, signs_dev, choice, rec_dev);
}

jolt_status jolt_encode_built(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                              const int32_t* choice, void* const* rec_dev, void* workspace, size_t workspace_bytes,
                              jolt_stream_t stream) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  st = check_choice(cfg, choice, rec_dev);
  if (st != JOLT_OK) return st;
  if (!x_dev || !signs_dev || !workspace) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (!x_dev[t]) return JOLT_EINVAL;
  if (!stamp_matches(cfg, x_dev, signs_dev, workspace, workspace_bytes)) return JOLT_EINVAL;
  Ctx x;
  x.c = cfg;
  x.p = make_plan(cfg);
  x.f64 = precise_factors(cfg);
  x.wt = x.f64 ? 3 : 0;
  x.we = x.f64 ? 8 : 4;
  x.ws = (char*)workspace;
  x.s = (hipStream_t)stream;
  memset(&x.x, 0, sizeof(x.x));
  for (int t = 0; t < cfg->n_tables; ++t) x.x.p[t] = x_dev[t];
  return encode_records(x, x_dev, signs_dev, choice, rec_dev);
}

jolt_status jolt_debug_score_pass(const jolt_config* cfg, const void* const* x_dev, const int8_t* signs_dev,
                                  const void* const* omega_dev, void* workspace, size_t workspace_bytes,
                                  int32_t reps, jolt_stream_t stream, double* ms_out) {
  if (!ms_out || reps < 1) return JOLT_EINVAL;
  hipStream_t s = (hipStream_t)stream;
  Ctx x;
  jolt_status st = prepare(cfg, x_dev, signs_dev, omega_dev, workspace, workspace_bytes, s, x);
  if (st != JOLT_OK) return st;
  st = run_factors(x, signs_dev);
  if (st != JOLT_OK) return st;
  info_set(x);
  stamp_set(x, signs_dev, workspace_bytes);
  if (!cores_make_w(x))
    HIPCHK(launch_prep_w(x.at<_Float16>(x.p.G16), x.at<float>(x.p.V32), signs_dev, cfg->N, cfg->D,
                         cfg->n_tables, x.at<_Float16>(x.p.Wh), x.at<_Float16>(x.p.Wl), x.at<int32_t>(x.p.flags), s));
  const ScoreArgs sa = score_args(x, signs_dev);
  HIPCHK(launch_score(sa, x.x, s));  // warm
  hipEvent_t e0, e1;
  HIPCHK(hipEventCreate(&e0));
  HIPCHK(hipEventCreate(&e1));
  HIPCHK(hipEventRecord(e0, s));
  for (int r = 0; r < reps; ++r) HIPCHK(launch_score(sa, x.x, s));
  HIPCHK(hipEventRecord(e1, s));
  HIPCHK(hipEventSynchronize(e1));
  float ms = 0.f;
  HIPCHK(hipEventElapsedTime(&ms, e0, e1));
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  *ms_out = (double)ms / reps;
  return JOLT_OK;
}

jolt_status jolt_debug_timer_enable(int32_t kernel, int32_t enable) {
  if (kernel != 0) return JOLT_EINVAL;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  g_score_timer.on = enable != 0;
  return JOLT_OK;
}

jolt_status jolt_debug_timer_read(int32_t kernel, double* total_ms, int32_t* launches) {
  if (kernel != 0 || !total_ms || !launches) return JOLT_EINVAL;
  std::lock_guard<std::mutex> lk(g_timer_mu);
  double tot = 0.0;
  jolt_status st = JOLT_OK;
  for (auto& pr : g_score_timer.ev) {
    float ms = 0.f;
    if (hipEventSynchronize(pr.second) != hipSuccess || hipEventElapsedTime(&ms, pr.first, pr.second) != hipSuccess)
      st = JOLT_EDEVICE;
    tot += ms;
    (void)hipEventDestroy(pr.first);
    (void)hipEventDestroy(pr.second);
  }
  *launches = (int32_t)g_score_timer.ev.size();
  *total_ms = tot;
  g_score_timer.ev.clear();
  return st;
}

jolt_status jolt_debug_read(const jolt_config* cfg, const void* workspace, int32_t which, void* host_out,
                            size_t bytes) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!workspace || !host_out) return JOLT_EINVAL;
  const Plan p = make_plan(cfg);
  const size_t nt = cfg->n_tables, N = cfg->N, T = cfg->T, D = cfg->D;
  size_t off, avail;
  const size_t fe = precise_factors(cfg) ? 8 : 4, nb = nt * 5;
  const size_t pc = cfg->token_mode == JOLT_TOKEN_EXACT ? JOLT_PSUB : 40;
  switch (which) {
    case 0: off = p.Ud64; avail = 8 * nt * D * JOLT_KMAX; break;
    case 1: off = p.UT16; avail = 2 * nt * 5 * T * JOLT_KMAX; break;
    case 2: off = p.G16; avail = 2 * nt * 5 * N * JOLT_KMAX * D; break;
    case 3: off = p.G16T; avail = 2 * nt * N * T * JOLT_KMAX; break;
    case 4: off = p.Mtok; avail = p.Mtok ? fe * nb * T * T : 0; break;
    case 5: off = p.Qs; avail = fe * nb * T * pc; break;
    case 6: off = p.Zs; avail = fe * nb * T * pc; break;
    case 7: off = p.Hrr; avail = 8 * nb * pc * pc; break;
    case 8: off = p.Vrr; avail = fe * nb * pc * JOLT_KMAX; break;
    case 9: off = p.UT32; avail = fe * nb * T * JOLT_KMAX; break;
    case 10: off = p.Wp; avail = 8 * nb * (size_t)JOLT_GRAM_PARTS * pc * pc; break;
    default: return JOLT_EINVAL;
  }
  if (bytes > avail) return JOLT_EINVAL;
  HIPCHK(hipMemcpy(host_out, (const char*)workspace + off, bytes, hipMemcpyDeviceToHost));
  return JOLT_OK;
}

jolt_status jolt_decode(const jolt_config* cfg, const void* const* rec_dev, const int32_t* choice,
                        void* const* xhat_dev, jolt_stream_t stream) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!rec_dev || !choice || !xhat_dev) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (choice[t] < 0 || choice[t] >= JOLT_N_CAND || !rec_dev[t] || !xhat_dev[t]) return JOLT_EINVAL;
  for (int t0 = 0; t0 < cfg->n_tables; t0 += JOLT_TAB_CHUNK) {
    DecodeArgs a;
    memset(&a, 0, sizeof(a));
    a.N = cfg->N;
    a.T = cfg->T;
    a.D = cfg->D;
    a.ntab = cfg->n_tables - t0 < JOLT_TAB_CHUNK ? cfg->n_tables - t0 : JOLT_TAB_CHUNK;
    for (int i = 0; i < a.ntab; ++i) {
      a.t[i] = record_layout(cfg, choice[t0 + i]);
      a.t[i].rec = (char*)rec_dev[t0 + i];
      a.out[i] = xhat_dev[t0 + i];
    }
    HIPCHK(launch_decode(a, (hipStream_t)stream));
  }
  return JOLT_OK;
}

// tokens per attention chunk: 256 (which amortises the per-workgroup reconstruction
// operands), halved (down to 64 and the tile) while the launch would have fewer than 512
// workgroups
static int attend_chunk(const jolt_config* c, int n_groups) {
  const int cp = c->D == 128 ? 32 : 64;
  const int ng = n_groups < ATT_GMAX ? n_groups : ATT_GMAX;
  int ach = ATT_CHMAX;
  while (ach > cp && ach > 64 && (int64_t)c->N * ng * ((c->T + ach - 1) / ach) < 512) ach /= 2;
  return ach;
}

jolt_status jolt_attend_workspace_size(const jolt_config* cfg, int32_t n_groups, int32_t nq, size_t* bytes_out) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!bytes_out || nq < 1 || nq > ATT_QMAX || n_groups < 1) return JOLT_EINVAL;
  const int ach = attend_chunk(cfg, n_groups);
  const size_t nchunk = (cfg->T + ach - 1) / ach;
  const size_t ng = n_groups < ATT_GMAX ? n_groups : ATT_GMAX;
  *bytes_out = ng * cfg->N * nchunk * nq * (cfg->D + 2) * sizeof(float);
  return JOLT_OK;
}

jolt_status jolt_attend(const jolt_config* cfg, int32_t n_groups, const void* const* rec_k, const int32_t* cand_k,
                        const void* const* rec_v, const int32_t* cand_v, const void* const* q_dev, int32_t nq,
                        float scale, float* const* o_dev, void* workspace, size_t workspace_bytes,
                        jolt_stream_t stream) {
  size_t need = 0;
  jolt_status st = jolt_attend_workspace_size(cfg, n_groups, nq, &need);
  if (st != JOLT_OK) return st;
  if (!rec_k || !rec_v || !cand_k || !cand_v || !q_dev || !o_dev || !workspace || workspace_bytes < need ||
      !isfinite(scale))
    return JOLT_EINVAL;
  for (int g = 0; g < n_groups; ++g)
    if (!rec_k[g] || !rec_v[g] || !q_dev[g] || !o_dev[g] || cand_k[g] < 0 || cand_k[g] >= JOLT_N_CAND ||
        cand_v[g] < 0 || cand_v[g] >= JOLT_N_CAND)
      return JOLT_EINVAL;
  const int ach = attend_chunk(cfg, n_groups);
  for (int g0 = 0; g0 < n_groups; g0 += ATT_GMAX) {  // the launches share the workspace in order
    AttendArgs a;
    memset(&a, 0, sizeof(a));
    a.N = cfg->N;
    a.T = cfg->T;
    a.D = cfg->D;
    a.nq = nq;
    a.ng = n_groups - g0 < ATT_GMAX ? n_groups - g0 : ATT_GMAX;
    a.ach = ach;
    a.nchunk = (cfg->T + ach - 1) / ach;
    a.scale = scale;
    for (int i = 0; i < a.ng; ++i) {
      a.k[i] = record_layout(cfg, cand_k[g0 + i]);
      a.k[i].rec = (char*)rec_k[g0 + i];
      a.v[i] = record_layout(cfg, cand_v[g0 + i]);
      a.v[i].rec = (char*)rec_v[g0 + i];
      a.q[i] = (const uint16_t*)q_dev[g0 + i];
      a.out[i] = o_dev[g0 + i];
    }
    a.part = (float*)workspace;
    HIPCHK(launch_attend(a, (hipStream_t)stream));
  }
  return JOLT_OK;
}

}  // extern "C"

// ------------------------------------------------------------------ streaming admission
namespace {

StreamTable block_layout(const jolt_config* c, int cand, int tn) {
  StreamTable b{};
  b.f = record_layout(c, cand);
  const uint64_t A = 256, N = c->N, D = c->D, tt = (uint64_t)tn;
  uint64_t off = 256;
  b.off_l = off;
  if (b.f.chain < 0) {
    off += pad_up(2 * N * tt * D, A);
  } else {
    off += b.f.chain == 5 ? pad_up(2 * N * tt * (uint64_t)b.f.rd, A) : pad_up(2 * tt * (uint64_t)b.f.rT, A);
    if (b.f.b > 0) {
      b.off_codes = off;
      off += pad_up(((uint64_t)b.f.b * N * tt * D + 7) / 8, A);
      b.off_scales = off;
      off += pad_up(4 * N * tt, A);
    }
  }
  b.total = off;
  return b;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

jolt_status stream_check(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand, int32_t t_new) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!rec_dev || !cand || t_new < 64 || t_new > 65536 || t_new % 64) return JOLT_EINVAL;
  if ((int64_t)cfg->N * t_new > (1ll << 30)) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (cand[t] < 0 || cand[t] >= JOLT_N_CAND || !rec_dev[t] || !aligned16(rec_dev[t])) return JOLT_EINVAL;
  return JOLT_OK;
}

StreamArgs stream_args(const jolt_config* cfg, int t0, int tn) {
  StreamArgs a;
  memset(&a, 0, sizeof(a));
  a.N = cfg->N;
  a.T = cfg->T;
  a.D = cfg->D;
  a.tn = tn;
  a.t0 = t0;
  a.ntab = cfg->n_tables - t0 < STREAM_TAB_CHUNK ? cfg->n_tables - t0 : STREAM_TAB_CHUNK;
  a.nchunk = (tn + STREAM_CHUNK - 1) / STREAM_CHUNK;
  a.ng = cfg->N < STREAM_GROUPS ? cfg->N : STREAM_GROUPS;
  a.spg = (cfg->N + a.ng - 1) / a.ng;
  return a;
}

// jolt_stream_encode with the workspace at `ws` (device memory of at least `ws_bytes`).
jolt_status stream_encode_at(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                             const void* const* state_dev, const void* const* xnew_dev, int32_t t_new,
                             void* const* block_dev, double* dist_dev, void* ws, size_t ws_bytes,
                             hipStream_t stream) {
  jolt_status st = stream_check(cfg, rec_dev, cand, t_new);
  if (st != JOLT_OK) return st;
  if (!state_dev || !xnew_dev || !block_dev || !ws) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (!state_dev[t] || !xnew_dev[t] || !block_dev[t] || !aligned16(xnew_dev[t]) || !aligned16(block_dev[t]))
      return JOLT_EINVAL;
  size_t need = 0;
  st = jolt_stream_workspace_size(cfg, t_new, &need);
  if (st != JOLT_OK) return st;
  if (ws_bytes < need || ((uintptr_t)ws & 7u)) return JOLT_ENOMEM;
  for (int t0 = 0; t0 < cfg->n_tables; t0 += STREAM_TAB_CHUNK) {
    StreamArgs a = stream_args(cfg, t0, t_new);
    a.part = (double*)ws;
    a.pfold = a.part + (size_t)2 * cfg->n_tables * cfg->N * a.nchunk;
    a.dist = dist_dev;
    for (int i = 0; i < a.ntab; ++i) {
      a.t[i] = block_layout(cfg, cand[t0 + i], t_new);
      a.t[i].f.rec = (char*)rec_dev[t0 + i];
      a.t[i].state = (double*)state_dev[t0 + i];
      a.t[i].x = (const uint16_t*)xnew_dev[t0 + i];
      a.t[i].blk = (char*)block_dev[t0 + i];
    }
    HIPCHK(launch_stream_encode(a, stream));
  }
  return JOLT_OK;
}

// The scratch of jolt_stream_encode_noalloc: one copy per device in the code object's
// device memory, held until the process ends.  Host code never passes `scratch` itself to
// a kernel (in host code the name is a host-side stand-in, not a device address): the
// device address comes from hipGetSymbolAddress, taken once per device with that device
// current, and kept.
static __device__ __align__(256) unsigned char scratch[JOLT_NOALLOC_SCRATCH_BYTES];
std::mutex g_scratch_mu;
std::unordered_map<int, void*> g_scratch_ptr;

jolt_status scratch_address(void** out) {
  int dev = 0;
  HIPCHK(hipGetDevice(&dev));
  std::lock_guard<std::mutex> lk(g_scratch_mu);
  auto it = g_scratch_ptr.find(dev);
  if (it == g_scratch_ptr.end()) {
    void* ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return JOLT_EDEVICE;
    it = g_scratch_ptr.emplace(dev, ptr).first;
  }
  *out = it->second;
  return JOLT_OK;
}

}  // namespace

extern "C" {

jolt_status jolt_stream_state_bytes(size_t* bytes_out) {
  if (!bytes_out) return JOLT_EINVAL;
  *bytes_out = sizeof(double) * STREAM_STATE_DOUBLES;
  return JOLT_OK;
}

jolt_status jolt_stream_block_bytes(const jolt_config* cfg, int32_t cand, int32_t t_new, uint64_t* bytes_out) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!bytes_out || cand < 0 || cand >= JOLT_N_CAND || t_new < 64 || t_new > 65536 || t_new % 64)
    return JOLT_EINVAL;
  *bytes_out = block_layout(cfg, cand, t_new).total;
  return JOLT_OK;
}

jolt_status jolt_stream_workspace_size(const jolt_config* cfg, int32_t t_new, size_t* bytes_out) {
  jolt_status st = validate(cfg);
  if (st != JOLT_OK) return st;
  if (!bytes_out || t_new < 64 || t_new > 65536 || t_new % 64) return JOLT_EINVAL;
  const size_t nchunk = (size_t)(t_new + STREAM_CHUNK - 1) / STREAM_CHUNK;
  const size_t ng = cfg->N < STREAM_GROUPS ? (size_t)cfg->N : STREAM_GROUPS;
  // error sums [n_tables][N][nchunk][2], then the left-factor partials [n_tables][ng][t/64][2048]
  *bytes_out = sizeof(double) * ((size_t)2 * cfg->n_tables * cfg->N * nchunk +
                                 (size_t)cfg->n_tables * ng * (t_new / 64) * 2048);
  return JOLT_OK;
}

jolt_status jolt_stream_prepare(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                                void* const* state_dev, jolt_stream_t stream) {
  jolt_status st = stream_check(cfg, rec_dev, cand, 64);
  if (st != JOLT_OK) return st;
  if (!state_dev) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (!state_dev[t] || ((uintptr_t)state_dev[t] & 7u)) return JOLT_EINVAL;
  for (int t0 = 0; t0 < cfg->n_tables; t0 += STREAM_TAB_CHUNK) {
    StreamArgs a = stream_args(cfg, t0, 64);
    for (int i = 0; i < a.ntab; ++i) {
      a.t[i] = block_layout(cfg, cand[t0 + i], 64);
      a.t[i].f.rec = (char*)rec_dev[t0 + i];
      a.t[i].state = (double*)state_dev[t0 + i];
    }
    HIPCHK(launch_stream_prepare(a, (hipStream_t)stream));
  }
  return JOLT_OK;
}

jolt_status jolt_stream_encode(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                               const void* const* state_dev, const void* const* xnew_dev, int32_t t_new,
                               void* const* block_dev, double* dist_dev, void* workspace, size_t workspace_bytes,
                               jolt_stream_t stream) {
  return stream_encode_at(cfg, rec_dev, cand, state_dev, xnew_dev, t_new, block_dev, dist_dev, workspace,
                          workspace_bytes, (hipStream_t)stream);
}

jolt_status jolt_stream_encode_noalloc(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                                       const void* const* state_dev, const void* const* xnew_dev, int32_t t_new,
                                       void* const* block_dev, double* dist_dev, jolt_stream_t stream) {
  jolt_status st = stream_check(cfg, rec_dev, cand, t_new);
  if (st != JOLT_OK) return st;
  size_t need = 0;
  st = jolt_stream_workspace_size(cfg, t_new, &need);
  if (st != JOLT_OK) return st;
  if (need > JOLT_NOALLOC_SCRATCH_BYTES) return JOLT_ENOMEM;
  void* ptr = nullptr;
  st = scratch_address(&ptr);
  if (st != JOLT_OK) return st;
  return stream_encode_at(cfg, rec_dev, cand, state_dev, xnew_dev, t_new, block_dev, dist_dev, ptr,
                          JOLT_NOALLOC_SCRATCH_BYTES, (hipStream_t)stream);
}

jolt_status jolt_stream_decode(const jolt_config* cfg, const void* const* rec_dev, const int32_t* cand,
                               const void* const* block_dev, int32_t t_new, void* const* out_dev,
                               jolt_stream_t stream) {
  jolt_status st = stream_check(cfg, rec_dev, cand, t_new);
  if (st != JOLT_OK) return st;
  if (!block_dev || !out_dev) return JOLT_EINVAL;
  for (int t = 0; t < cfg->n_tables; ++t)
    if (!block_dev[t] || !out_dev[t] || !aligned16(block_dev[t]) || !aligned16(out_dev[t])) return JOLT_EINVAL;
  for (int t0 = 0; t0 < cfg->n_tables; t0 += STREAM_TAB_CHUNK) {
    StreamArgs a = stream_args(cfg, t0, t_new);
    for (int i = 0; i < a.ntab; ++i) {
      a.t[i] = block_layout(cfg, cand[t0 + i], t_new);
      a.t[i].f.rec = (char*)rec_dev[t0 + i];
      a.t[i].blk = (char*)block_dev[t0 + i];
      a.t[i].out = (uint16_t*)out_dev[t0 + i];
    }
    HIPCHK(launch_stream_decode(a, (hipStream_t)stream));
  }
  return JOLT_OK;
}

}  // extern "C"
