// Streaming admission: an incoming token block X' [N, t', D] of a table is encoded against
// the table's frozen record.  Both pages put the compressor on the cache write path: the
// selected Tucker factors are kept and every incoming token block is reconstructed and its
// residual R = X - X~ rotated and quantized ("Rotated Tucker residual for outlier-resistant
// KV quantization", Implementation notes; "Joint Tucker-rank and residual-bit KV
// allocator", Implementation notes).
//
// The record's feature factor and cores stay fixed.  With X~_n = L R_n (R_n = G_n U_d^T, or
// G_n when r_d = D, for r_T < T; R = U_d^T for r_T = T) an incoming token needs only its
// rows of L: one row shared by all slices when r_T < T (as U_T's rows are), one row per
// slice when r_T = T.  They are the least-squares fit of the token against the operator,
// through the normal equations L = P A+, P = sum_n X'_n R_n^T, A = sum_n R_n R_n^T (K x K,
// K <= 32).  A+ keeps the eigen-directions of A above STREAM_RCUT of the largest eigenvalue
// (the minimum-norm solution when the operator is rank deficient, e.g. N r_d < r_T).
//
//   k_stream_prepare  once per frozen record: A in fp64 from the stored fp16 factors,
//                     cyclic Jacobi eigendecomposition, A+ into the state buffer
//   k_block_header    block record header
//   k_stream_fold     per 64 tokens and slice group: P with fp64 MFMA (per-slice rows of
//                     r_T = T records: L = P A+ written here)
//   k_stream_fold_fin per 64 tokens: the groups' P added, L = P A+, fp16 rows into the block
//   k_stream_resid    per 256 tokens and slice: X~ tiles from the frozen operator and the
//                     block's rows (the decoder's tile code), rotation, b-bit codes, fp32
//                     scales, and the sums of x^2 and of the squared error
//   k_stream_dist     per table: the block's distortion ||X' - X^'||^2 / ||X'||^2
//   k_stream_decode   block record + frozen record -> bf16 X^' (the decoder's tile code)
#include "codec_tiles.h"

namespace jolt {

static_assert(STREAM_CHUNK == CODEC_CHUNK, "the streaming launches use the codec's token chunk");

// ------------------------------------------------------------------ frozen state
// One workgroup per table.  Thread tid owns the entries tid + 256 m (m < 4) of the 32 x 32
// matrix A (zero beyond K).  Then Jacobi sweeps in the round-robin order of 16 disjoint
// pairs per step (31 steps per sweep) until the off-diagonal mass is below 1e-30 of the
// total (at most 30 sweeps); A+ = sum over kept m of v_m v_m^T / lambda_m.
__device__ __forceinline__ void stream_pair(int r, int k, int& p, int& q) {
  int a, b;
  if (k == 0) {
    a = 31;
    b = r;
  } else {
    a = (r + k) % 31;
    b = (r - k + 31) % 31;
  }
  p = a < b ? a : b;
  q = a < b ? b : a;
}

__global__ __launch_bounds__(256) void k_stream_prepare(const StreamArgs a) {
  const StreamTable& st = a.t[blockIdx.x];
  const EncodeTable& f = st.f;
  const int tid = threadIdx.x, D = a.D, N = a.N;
  __shared__ double A[32][33], V[32][33], Bm[32][33], Hs[32][33];
  __shared__ double Gs[32][129];
  __shared__ double rot[16][2];
  __shared__ double red[2][4];
  __shared__ int stop;
  const int chain = f.chain;
  const int rT = f.rT, rd = f.rd;
  const int K = chain < 0 ? 0 : (chain == 5 ? rd : rT);
  const _Float16* Ud = (const _Float16*)(f.rec + f.off_ud);
  const _Float16* Gc = (const _Float16*)(f.rec + f.off_core);
  double acc[4] = {0.0, 0.0, 0.0, 0.0};
  if (chain >= 0 && chain != 4) {  // Bm = U_d^T U_d (r_d x r_d)
    for (int e = tid; e < 32 * 32; e += 256) {
      const int i = e >> 5, j = e & 31;
      double v = 0.0;
      if (i < rd && j < rd)
        for (int x = 0; x < D; ++x) v = fma((double)Ud[x * rd + i], (double)Ud[x * rd + j], v);
      Bm[i][j] = v;
    }
    __syncthreads();
  }
  if (chain == 5) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = tid + 256 * m;
      acc[m] = Bm[e >> 5][e & 31];
    }
  } else if (chain >= 0) {
    const int gw = chain == 4 ? D : rd;  // row length of a stored core slice
    for (int n = 0; n < N; ++n) {
      const _Float16* G = Gc + (int64_t)n * rT * gw;
      for (int e = tid; e < rT * gw; e += 256) Gs[e / gw][e % gw] = (double)G[e];
      __syncthreads();
      if (chain == 4) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int e = tid + 256 * m, i = e >> 5, j = e & 31;
          if (i < K && j < K) {
            double v = 0.0;
            for (int x = 0; x < D; ++x) v = fma(Gs[i][x], Gs[j][x], v);
            acc[m] += v;
          }
        }
      } else {
        for (int e = tid; e < 32 * 32; e += 256) {  // H = G_n Bm (r_T x r_d)
          const int i = e >> 5, c = e & 31;
          double v = 0.0;
          if (i < rT && c < rd)
            for (int x = 0; x < rd; ++x) v = fma(Gs[i][x], Bm[x][c], v);
          Hs[i][c] = v;
        }
        __syncthreads();
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          const int e = tid + 256 * m, i = e >> 5, j = e & 31;
          if (i < K && j < K) {
            double v = 0.0;
            for (int x = 0; x < rd; ++x) v = fma(Hs[i][x], Gs[j][x], v);
            acc[m] += v;
          }
        }
      }
      __syncthreads();  // Gs, Hs are rewritten for the next slice
    }
  }
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int e = tid + 256 * m, i = e >> 5, j = e & 31;
    A[i][j] = acc[m];
    V[i][j] = i == j ? 1.0 : 0.0;
  }
  __syncthreads();
  for (int sweep = 0; sweep < 30; ++sweep) {
    double off = 0.0, tot = 0.0;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int e = tid + 256 * m, i = e >> 5, j = e & 31;
      const double v = A[i][j] * A[i][j];
      tot += v;
      if (i != j) off += v;
    }
    off = wave_sum_f64(off);
    tot = wave_sum_f64(tot);
    if ((tid & 63) == 0) {
      red[0][tid >> 6] = off;
      red[1][tid >> 6] = tot;
    }
    __syncthreads();
    if (tid == 0) {
      const double o = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
      const double t = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
      stop = !(o > 1e-30 * t);
    }
    __syncthreads();
    if (stop) break;
    for (int r = 0; r < 31; ++r) {
      if (tid < 16) {
        int p, q;
        stream_pair(r, tid, p, q);
        const double app = A[p][p], aqq = A[q][q], apq = A[p][q];
        double c = 1.0, s = 0.0;
        if (apq != 0.0) {
          const double th = (aqq - app) / (2.0 * apq);
          const double at = fabs(th);
          double t = at > 1e150 ? 0.5 / at : 1.0 / (at + sqrt(1.0 + th * th));
          if (th < 0.0) t = -t;
          c = 1.0 / sqrt(1.0 + t * t);
          s = t * c;
        }
        rot[tid][0] = c;
        rot[tid][1] = s;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 2; ++m) {  // columns p, q of A and V
        const int it = tid + 256 * m, k = it & 15, row = it >> 4;
        int p, q;
        stream_pair(r, k, p, q);
        const double c = rot[k][0], s = rot[k][1];
        const double ap = A[row][p], aq = A[row][q];
        A[row][p] = c * ap - s * aq;
        A[row][q] = s * ap + c * aq;
        const double vp = V[row][p], vq = V[row][q];
        V[row][p] = c * vp - s * vq;
        V[row][q] = s * vp + c * vq;
      }
      __syncthreads();
#pragma unroll
      for (int m = 0; m < 2; ++m) {  // rows p, q of A
        const int it = tid + 256 * m, k = it & 15, col = it >> 4;
        int p, q;
        stream_pair(r, k, p, q);
        const double c = rot[k][0], s = rot[k][1];
        const double bp = A[p][col], bq = A[q][col];
        A[p][col] = c * bp - s * bq;
        A[q][col] = s * bp + c * bq;
      }
      __syncthreads();
    }
  }
  double lmax = 0.0;
  for (int m = 0; m < 32; ++m) lmax = fmax(lmax, A[m][m]);
  const double cut = STREAM_RCUT * lmax;
#pragma unroll
  for (int m4 = 0; m4 < 4; ++m4) {
    const int e = tid + 256 * m4, i = e >> 5, j = e & 31;
    double v = 0.0;
    if (lmax > 0.0)
      for (int m = 0; m < 32; ++m) {
        const double lam = A[m][m];
        if (lam > cut) v += V[i][m] * V[j][m] / lam;
      }
    st.state[e] = v;
  }
  if (tid < 32) st.state[32 * 32 + tid] = A[tid][tid];
}

// ------------------------------------------------------------------ block records
// Header words: 0 magic "JLTB", 1 version, 2 N, 3 t', 4 D, 5 r_T, 6 r_d, 7 b, 8 values per
// quantization block, 9 T of the frozen record, 10-17 64-bit total and the offsets of the
// left factor, codes and scales, 18 flags (bit 0: a left-factor value overflowed fp16).
__global__ void k_block_header(const StreamArgs a) {
  const StreamTable& st = a.t[blockIdx.x];
  uint32_t* h = (uint32_t*)st.blk;
  const int i = threadIdx.x;
  uint32_t w = 0;
  switch (i) {
    case 0: w = BLOCK_MAGIC; break;
    case 1: w = 1u; break;
    case 2: w = (uint32_t)a.N; break;
    case 3: w = (uint32_t)a.tn; break;
    case 4: w = (uint32_t)a.D; break;
    case 5: w = (uint32_t)st.f.rT; break;
    case 6: w = (uint32_t)st.f.rd; break;
    case 7: w = (uint32_t)st.f.b; break;
    case 8: w = (uint32_t)a.D; break;
    case 9: w = (uint32_t)a.T; break;
    default: break;
  }
  if (i >= 10 && i < 18) {
    const int q = (i - 10) >> 1;
    const uint64_t v = q == 0 ? st.total : q == 1 ? st.off_l : q == 2 ? st.off_codes : st.off_scales;
    w = (i & 1) ? (uint32_t)(v >> 32) : (uint32_t)v;
  }
  h[i] = w;
}

// fp16 rows of L from L^T tiles (element (i = 16 kt + 4 r + lk, token) in register r of
// tile kt): dst[rowbase + i] for i < K; an overflow sets bit 0 of header word 18.
__device__ __forceinline__ void stream_store_rows(const StreamTable& st, const double4_t (&Lt)[2], int nkt, int K,
                                                  int64_t rowbase, int lk) {
  _Float16* dst = (_Float16*)(st.blk + st.off_l);
  bool ovf = false;
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
    if (kt < nkt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int i = 16 * kt + 4 * r + lk;
        if (i < K) {
          const _Float16 h = f64_to_f16(Lt[kt][r]);
          ovf |= (__builtin_bit_cast(uint16_t, h) & 0x7C00u) == 0x7C00u;
          dst[rowbase + i] = h;
        }
      }
  if (ovf) atomicOr((uint32_t*)st.blk + 18, 1u);
}

// Left factor, first pass: workgroup (64-token tile bx, slice group g, table).  Wave w takes
// tokens tok0 + 16 w .. + 15 of slices n = g S .. g S + S - 1.  fp64 MFMA 16x16x4 tiles:
// A(i, k) in lane i + 16 k, B(k, j) in lane j + 16 k, result (i, j) in lane 16 (i & 3) + j,
// register i >> 2, so register s of a result tile is the B operand of k-step s of the next
// product.  Products are held transposed (rows = factor index, columns = tokens):
//   Y^T = U_d^T X'^T (r_d x 16),  P^T = sum_n G_n Y_n^T (or G_n X'^T when r_d = D).
// r_T < T: the slice group's P^T is written, register by register, to the partial buffer
// (k_stream_fold_fin adds the groups and applies A+).  r_T = T: every slice has its own
// rows, L^T = A+ Y^T, written here.
template <int D>
__global__ __launch_bounds__(256) void k_stream_fold(const StreamArgs a) {
  const StreamTable& st = a.t[blockIdx.z];
  const EncodeTable& f = st.f;
  const int chain = f.chain;
  if (chain < 0) return;
  const int N = a.N, tn = a.tn, rT = f.rT, rd = f.rd, S = a.spg;
  const int n0 = blockIdx.y * S, n1 = min(N, n0 + S);
  if (n0 >= n1) return;
  const bool per_slice = chain == 5;
  const int K = per_slice ? rd : rT;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int tok0 = blockIdx.x * 64;
  __shared__ __attribute__((aligned(16))) uint16_t Xs[64][D + 8];
  __shared__ _Float16 Uds[D][33];
  const _Float16* Udg = (const _Float16*)(f.rec + f.off_ud);
  const _Float16* Gg = (const _Float16*)(f.rec + f.off_core);
  if (chain != 4)
    for (int idx = tid; idx < D * 32; idx += 256) {
      const int r = idx >> 5, c = idx & 31;
      Uds[r][c] = c < rd ? Udg[r * rd + c] : (_Float16)0.0f;
    }
  const int nkt = (K + 15) / 16;    // 16-row tiles of P and L
  const int nrt = rd > 16 ? 2 : 1;  // 16-row tiles of Y
  const double4_t z4 = {0.0, 0.0, 0.0, 0.0};
  double4_t P[2] = {z4, z4};
  for (int n = n0; n < n1; ++n) {
    __syncthreads();  // the previous slice's rows are consumed (and Uds is staged)
    const uint4* src = (const uint4*)(st.x + ((int64_t)n * tn + tok0) * D);
    for (int idx = tid; idx < 64 * D / 8; idx += 256) {
      const int r = idx / (D / 8), c = idx - r * (D / 8);
      *(uint4*)&Xs[r][c * 8] = src[idx];
    }
    __syncthreads();
    const uint16_t* xrow = &Xs[16 * w + li][0];
    if (chain == 4) {
      const _Float16* G = Gg + (int64_t)n * rT * D;
      double4_t Q[2] = {z4, z4};  // odd k-steps: a second dependency chain
      for (int f0 = 0; f0 < D; f0 += 8) {
        const double b0 = (double)bf16_to_f32(xrow[f0 + lk]);
        const double b1 = (double)bf16_to_f32(xrow[f0 + 4 + lk]);
#pragma unroll
        for (int kt = 0; kt < 2; ++kt)
          if (kt < nkt) {
            const int i = 16 * kt + li;
            const double a0 = i < K ? (double)G[i * D + f0 + lk] : 0.0;
            const double a1 = i < K ? (double)G[i * D + f0 + 4 + lk] : 0.0;
            P[kt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a0, b0, P[kt], 0, 0, 0);
            Q[kt] = __builtin_amdgcn_mfma_f64_16x16x4f64(a1, b1, Q[kt], 0, 0, 0);
          }
      }
      P[0] += Q[0];
      P[1] += Q[1];
    } else {
      double4_t Y[2] = {z4, z4}, Y2[2] = {z4, z4};
      for (int f0 = 0; f0 < D; f0 += 8) {
        const double b0 = (double)bf16_to_f32(xrow[f0 + lk]);
        const double b1 = (double)bf16_to_f32(xrow[f0 + 4 + lk]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
          if (rt < nrt) {
            Y[rt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)Uds[f0 + lk][16 * rt + li], b0, Y[rt], 0, 0, 0);
            Y2[rt] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)Uds[f0 + 4 + lk][16 * rt + li], b1, Y2[rt], 0, 0, 0);
          }
      }
      Y[0] += Y2[0];
      Y[1] += Y2[1];
      if (per_slice) {
        // L^T = A+ Y^T for this slice's rows
        double4_t Lt[2] = {z4, z4};
        for (int s = 0; s < K / 4; ++s) {
          const double bv = Y[s >> 2][s & 3];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            if (kt < nkt)
              Lt[kt] = __builtin_amdgcn_mfma_f64_16x16x4f64(st.state[(16 * kt + li) * 32 + 4 * s + lk], bv, Lt[kt],
                                                            0, 0, 0);
        }
        stream_store_rows(st, Lt, nkt, K, ((int64_t)n * tn + tok0 + 16 * w + li) * rd, lk);
      } else {
        const _Float16* G = Gg + (int64_t)n * rT * rd;
        for (int s = 0; s < rd / 4; ++s) {
          const double bv = Y[s >> 2][s & 3];
#pragma unroll
          for (int kt = 0; kt < 2; ++kt)
            if (kt < nkt) {
              const int i = 16 * kt + li;
              const double av = i < K ? (double)G[i * rd + 4 * s + lk] : 0.0;
              P[kt] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, P[kt], 0, 0, 0);
            }
        }
      }
    }
  }
  if (per_slice) return;
  // partial P^T of this slice group: [table][group][token tile][wave][kt][register][lane]
  double* pp = a.pfold + ((((int64_t)(a.t0 + blockIdx.z) * a.ng + blockIdx.y) * (tn / 64) + blockIdx.x) * 4 + w) *
                             (2 * 4 * 64);
#pragma unroll
  for (int kt = 0; kt < 2; ++kt)
    if (kt < nkt)
#pragma unroll
      for (int r = 0; r < 4; ++r) pp[(kt * 4 + r) * 64 + lane] = P[kt][r];
}

// Left factor, second pass (r_T < T): P^T = the slice groups' partials added in group
// order, L^T = A+ P^T, fp16 rows into the block.  Workgroup (64-token tile, table).
__global__ __launch_bounds__(256) void k_stream_fold_fin(const StreamArgs a) {
  const StreamTable& st = a.t[blockIdx.z];
  const EncodeTable& f = st.f;
  if (f.chain < 0 || f.chain == 5) return;
  const int tn = a.tn, K = f.rT, ng = min(a.ng, (a.N + a.spg - 1) / a.spg);
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int nkt = (K + 15) / 16;
  const double4_t z4 = {0.0, 0.0, 0.0, 0.0};
  double4_t P[2] = {z4, z4};
  const int64_t gstride = (int64_t)(tn / 64) * 4 * (2 * 4 * 64);
  const double* pp = a.pfold + ((((int64_t)(a.t0 + blockIdx.z) * a.ng) * (tn / 64) + blockIdx.x) * 4 + w) *
                                   (2 * 4 * 64);
  for (int g = 0; g < ng; ++g)
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      if (kt < nkt)
#pragma unroll
        for (int r = 0; r < 4; ++r) P[kt][r] += pp[g * gstride + (kt * 4 + r) * 64 + lane];
  double4_t Lt[2] = {z4, z4};
  for (int s = 0; s < K / 4; ++s) {
    const double bv = P[s >> 2][s & 3];
#pragma unroll
    for (int kt = 0; kt < 2; ++kt)
      if (kt < nkt)
        Lt[kt] = __builtin_amdgcn_mfma_f64_16x16x4f64(st.state[(16 * kt + li) * 32 + 4 * s + lk], bv, Lt[kt], 0, 0, 0);
  }
  stream_store_rows(st, Lt, nkt, K, (int64_t)(blockIdx.x * 64 + 16 * w + li) * K, lk);
}

// Residual codes, scales and error sums of 256 tokens of slice n (verbatim records: the
// block's rows are copied).  Partial sums (x^2, squared error) per workgroup, in a fixed
// order, for k_stream_dist.
template <int D>
__global__ __launch_bounds__(256) void k_stream_resid(const StreamArgs a) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  constexpr int CP = CodecLds<D>::CP;
  const int tl = blockIdx.z, tg = a.t0 + tl, n = blockIdx.y, c = blockIdx.x;
  const StreamTable& st = a.t[tl];
  const EncodeTable& f = st.f;
  const int tn = a.tn;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  const int tb = c * CODEC_CHUNK, te = min(tn, tb + CODEC_CHUNK);
  __shared__ CodecLds<D> L;
  __shared__ double sgs[D];
  __shared__ int8_t sg8[D];
  __shared__ double red[2][4];
  double ex = 0.0, ee = 0.0;
  if (f.chain < 0) {  // (T, D): the block keeps X' verbatim
    const uint4* src = (const uint4*)(st.x + ((int64_t)n * tn + tb) * D);
    uint4* dst = (uint4*)(st.blk + st.off_l) + ((int64_t)n * tn + tb) * D / 8;
    for (int64_t i = tid; i < (int64_t)(te - tb) * D / 8; i += 256) dst[i] = src[i];
  } else {
    DecodeSrc d = codec_prepare<D>(L, sgs, f, n, a.T);
    const _Float16* Lbk = (const _Float16*)(st.blk + st.off_l);
    d.Lb = f.chain == 5 ? Lbk + (int64_t)n * tn * f.rd : Lbk;
    d.ls = f.chain == 5 ? f.rd : f.rT;
    for (int x = tid; x < D; x += 256) sg8[x] = sgs[x] < 0.0 ? (int8_t)-1 : (int8_t)1;
    const int b = f.b;
    const int qmax = b > 0 ? (1 << (b - 1)) - 1 : 0;
    uint32_t* codes = (uint32_t*)(st.blk + st.off_codes);
    float* scales = (float*)(st.blk + st.off_scales);
    __syncthreads();
    TileIn cur;
    codec_fetch_a<D>(cur, d.Lb, d.ls, d.K, tb);
    codec_fetch_row<D>(cur, st.x, (int64_t)n * tn + tb + rloc);
    for (int t0 = tb; t0 < te; t0 += CP) {
      const bool more = t0 + CP < te;  // uniform
      TileIn nxt;
      if (more) {
        codec_fetch_a<D>(nxt, d.Lb, d.ls, d.K, t0 + CP);
        codec_fetch_row<D>(nxt, st.x, (int64_t)n * tn + t0 + CP + rloc);
      }
      codec_xtilde_in<D>(L, cur, d.K);
      __syncthreads();
      const int64_t row = (int64_t)n * tn + t0 + rloc;
      const double* xt = &L.Xt[rloc][sg * FPT];
      double y[FPT];
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        const double x = (double)bf16_to_f32((uint16_t)(cur.w[i >> 1] >> (16 * (i & 1))));
        ex = fma(x, x, ex);
        y[i] = x - xt[i];
      }
      if (b > 0) {
        int q[FPT];
        const float sc = codec_rotq<D>(y, sg8 + sg * FPT, sg, qmax, q);
        codec_store_codes(q, codes, row, D, sg, b);
        if (sg == 0) scales[row] = sc;
        const double sd = (double)sc;
#pragma unroll
        for (int i = 0; i < FPT; ++i) {
          const double e = y[i] - sd * (double)q[i];
          ee = fma(e, e, ee);
        }
      } else {
#pragma unroll
        for (int i = 0; i < FPT; ++i) ee = fma(y[i], y[i], ee);
      }
      __syncthreads();  // X~ tile is rewritten by the next pass
      if (more) cur = nxt;
    }
  }
  ex = wave_sum_f64(ex);
  ee = wave_sum_f64(ee);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = ex;
    red[1][tid >> 6] = ee;
  }
  __syncthreads();
  if (tid == 0) {
    double* p = a.part + (((int64_t)tg * a.N + n) * a.nchunk + c) * 2;
    p[0] = (red[0][0] + red[0][1]) + (red[0][2] + red[0][3]);
    p[1] = (red[1][0] + red[1][1]) + (red[1][2] + red[1][3]);
  }
}

// dist[t] = sum of squared errors / sum of x^2 over the block (0 for an all-zero block or
// a verbatim record; NaN when the left factor overflowed fp16).  One wave per table.
__global__ void k_stream_dist(const StreamArgs a) {
  const int tl = blockIdx.x, tg = a.t0 + tl, lane = threadIdx.x;
  const StreamTable& st = a.t[tl];
  const int64_t np = (int64_t)a.N * a.nchunk;
  const double* p = a.part + (int64_t)tg * np * 2;
  double ex = 0.0, ee = 0.0;
  for (int64_t i = lane; i < np; i += 64) {
    ex += p[2 * i];
    ee += p[2 * i + 1];
  }
  ex = wave_sum_f64(ex);
  ee = wave_sum_f64(ee);
  if (lane == 0) {
    const uint32_t flags = ((const uint32_t*)st.blk)[18];
    double d = st.f.chain < 0 ? 0.0 : (ex > 0.0 ? ee / ex : 0.0);
    if (flags & 1u) d = __builtin_nan("");
    a.dist[tg] = d;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_stream_decode(const StreamArgs a) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  constexpr int CP = CodecLds<D>::CP;
  const int tl = blockIdx.z, n = blockIdx.y;
  const StreamTable& st = a.t[tl];
  const EncodeTable& f = st.f;
  const int tn = a.tn;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  const int tb = blockIdx.x * CODEC_CHUNK, te = min(tn, tb + CODEC_CHUNK);
  if (f.chain < 0) {
    const uint4* src = (const uint4*)(st.blk + st.off_l) + ((int64_t)n * tn + tb) * D / 8;
    uint4* dst = (uint4*)st.out + ((int64_t)n * tn + tb) * D / 8;
    for (int64_t i = tid; i < (int64_t)(te - tb) * D / 8; i += 256) dst[i] = src[i];
    return;
  }
  __shared__ DecLds<D> L;
  __shared__ float sgs[D];
  DecSrc d = dec_prepare<D>(L, sgs, f, n, a.T);
  const _Float16* Lbk = (const _Float16*)(st.blk + st.off_l);
  d.Lb = f.chain == 5 ? Lbk + (int64_t)n * tn * f.rd : Lbk;
  d.ls = f.chain == 5 ? f.rd : f.rT;
  d.codes = (const uint8_t*)(st.blk + st.off_codes);
  d.scales = (const float*)(st.blk + st.off_scales);
  dec_bops<D>(L);
  DecIn cur;
  dec_fetch<D>(cur, d, f.b, n, tn, tb);
  for (int t0 = tb; t0 < te; t0 += CP) {
    const bool more = t0 + CP < te;  // uniform
    DecIn nxt;
    if (more) dec_fetch<D>(nxt, d, f.b, n, tn, t0 + CP);
    float4_t v[4];
    dec_vals<D>(&L.Bh[0][0][0][0], &L.Bl[0][0][0][0], sgs, d, f.b, cur, v);
    dec_store<D>(st.out, (int64_t)n * tn + t0, v);
    if (more) cur = nxt;
  }
}

static bool stream_args_ok(const StreamArgs& a) {
  return a.ntab >= 1 && a.ntab <= STREAM_TAB_CHUNK && a.N >= 1 && a.tn >= 64 && a.tn % 64 == 0 &&
         (a.D == 64 || a.D == 128) && a.nchunk == (a.tn + CODEC_CHUNK - 1) / CODEC_CHUNK;
}

hipError_t launch_stream_prepare(const StreamArgs& a, hipStream_t s) {
  if (a.ntab < 1 || a.ntab > STREAM_TAB_CHUNK || a.D > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_stream_prepare, dim3(a.ntab), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_encode(const StreamArgs& a, hipStream_t s) {
  if (!stream_args_ok(a) || !a.part || !a.pfold || a.spg < 1 || a.ng < 1 || (int64_t)a.ng * a.spg < a.N)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_block_header, dim3(a.ntab), dim3(64), 0, s, a);
  const dim3 gf(a.tn / 64, a.ng, a.ntab), gfin(a.tn / 64, 1, a.ntab), gr(a.nchunk, a.N, a.ntab);
  if (a.D == 128)
    hipLaunchKernelGGL(k_stream_fold<128>, gf, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_stream_fold<64>, gf, dim3(256), 0, s, a);
  hipLaunchKernelGGL(k_stream_fold_fin, gfin, dim3(256), 0, s, a);
  if (a.D == 128)
    hipLaunchKernelGGL(k_stream_resid<128>, gr, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_stream_resid<64>, gr, dim3(256), 0, s, a);
  if (a.dist) hipLaunchKernelGGL(k_stream_dist, dim3(a.ntab), dim3(64), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_stream_decode(const StreamArgs& a, hipStream_t s) {
  if (!stream_args_ok(a)) return hipErrorInvalidValue;
  const dim3 g(a.nchunk, a.N, a.ntab);
  if (a.D == 128)
    hipLaunchKernelGGL(k_stream_decode<128>, g, dim3(256), 0, s, a);
  else
    hipLaunchKernelGGL(k_stream_decode<64>, g, dim3(256), 0, s, a);
  return hipGetLastError();
}

}  // namespace jolt
