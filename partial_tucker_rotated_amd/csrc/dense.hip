// Small dense kernels of the factor stage: the symmetric top-k eigensolver used for
// the feature Gram, the small token Grams and the Rayleigh-Ritz matrices; the
// Cholesky inverse of CholeskyQR; Gram reduction; feature-factor preparation.
#include "jolt_internal.h"

namespace jolt {

// ============================================================ symmetric top-k eigensolver
// Householder tridiagonalisation (matrix in LDS), multisection bisection with Sturm
// counts for the k largest eigenvalues, inverse iteration with an LDL^T solve and
// modified Gram-Schmidt inside clusters, back-transformation, sign normalisation.
#define SY_N 128
#define SY_K 32
#define SY_IB 16  // eigenvectors per inverse-iteration batch
#define SY_S 8    // bisection samples per eigenvalue and round
#define SY_ROUNDS 16

// eigenvector j, component i, stored in the upper-right quadrant of the matrix
// array (free once the matrix is tridiagonal), rotated so that lanes j do not collide
__device__ __forceinline__ int sy_yidx(int j, int i) { return (2 * j + (i >> 6)) * SY_N + 64 + ((i + 2 * j) & 63); }

template <typename TIn>
__global__ __launch_bounds__(256) void k_syev_topk(const TIn* Aall, int n, int k, double* U64, float* U32,
                                                   _Float16* U16, double* lam_out) {
  __shared__ double A[SY_N * SY_N];
  __shared__ double scr[SY_IB * 130];  // LDL^T pivots of a batch; reused as scratch earlier
  __shared__ double d[SY_N], e[SY_N], e2[SY_N], tau[SY_N];
  __shared__ double lo[SY_K], hi[SY_K], red[64];
  __shared__ int cnt[256];
  __shared__ double sh_misc[4];
  double* vv = scr;            // Householder vector (tridiagonalisation only)
  double* ww = scr + SY_N;     // p, then w
  double* ww2 = scr + 2 * SY_N;
  double* xs = scr;            // bisection sample points (bisection only)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const TIn* Ain = Aall + (int64_t)b * n * n;
  for (int idx = tid; idx < n * n; idx += 256) A[(idx / n) * SY_N + idx % n] = (double)Ain[idx];
  __syncthreads();

  // ---- tridiagonalisation: A = Q T Q^T, Q = H_0 ... H_{n-3}
  for (int kk = 0; kk < n - 2; ++kk) {
    const int m = n - kk - 1;  // size of the trailing block
    if (wave == 0) {
      double s = 0.0;
      for (int i = kk + 2 + lane; i < n; i += 64) s += A[i * SY_N + kk] * A[i * SY_N + kk];
      s = wave_sum_f64(s);
      if (lane == 0) {
        const double x0 = A[(kk + 1) * SY_N + kk];
        d[kk] = A[kk * SY_N + kk];
        if (s == 0.0) {
          tau[kk] = 0.0;
          e[kk] = x0;
          sh_misc[0] = 0.0;
        } else {
          const double nx = sqrt(x0 * x0 + s);
          const double beta = x0 >= 0.0 ? -nx : nx;
          tau[kk] = (beta - x0) / beta;
          e[kk] = beta;
          sh_misc[0] = 1.0 / (x0 - beta);
        }
      }
    }
    __syncthreads();
    const double t = tau[kk];
    if (t == 0.0) continue;  // uniform across the block
    const double sc = sh_misc[0];
    for (int i = tid; i < m; i += 256) {
      const double v = i == 0 ? 1.0 : A[(kk + 1 + i) * SY_N + kk] * sc;
      vv[i] = v;
      if (i > 0) A[(kk + 1 + i) * SY_N + kk] = v;
    }
    __syncthreads();
    // p = tau * A22 v: thread i sums column i of the symmetric block over half the rows
    {
      const int i = tid & 127, half = tid >> 7;
      double s = 0.0;
      if (i < m) {
        const int j0 = half ? (m >> 1) : 0, j1 = half ? m : (m >> 1);
        for (int j = j0; j < j1; ++j) s += A[(kk + 1 + j) * SY_N + kk + 1 + i] * vv[j];
      }
      if (half) ww2[i] = s;
      __syncthreads();
      if (!half && i < m) ww[i] = t * (s + ww2[i]);
    }
    __syncthreads();
    if (wave == 0) {
      double s = 0.0;
      for (int i = lane; i < m; i += 64) s += ww[i] * vv[i];
      s = wave_sum_f64(s);
      if (lane == 0) sh_misc[1] = 0.5 * t * s;
    }
    __syncthreads();
    {
      const double K = sh_misc[1];
      for (int i = tid; i < m; i += 256) ww[i] = ww[i] - K * vv[i];
    }
    __syncthreads();
    for (int r = wave; r < m; r += 4) {
      const double vr = vv[r], wr = ww[r];
      double* row = &A[(kk + 1 + r) * SY_N + kk + 1];
      for (int c = lane; c < m; c += 64) row[c] -= vr * ww[c] + wr * vv[c];
    }
    __syncthreads();
  }
  if (tid == 0) {
    if (n >= 2) {
      d[n - 2] = A[(n - 2) * SY_N + n - 2];
      e[n - 2] = A[(n - 1) * SY_N + n - 2];
      tau[n - 2] = 0.0;
    }
    d[n - 1] = A[(n - 1) * SY_N + n - 1];
    e[n - 1] = 0.0;
    tau[n - 1] = 0.0;
    double glo = 1e300, ghi = -1e300, tmax = 0.0, emax = 0.0;
    for (int i = 0; i < n; ++i) {
      const double r = (i > 0 ? fabs(e[i - 1]) : 0.0) + (i < n - 1 ? fabs(e[i]) : 0.0);
      glo = fmin(glo, d[i] - r);
      ghi = fmax(ghi, d[i] + r);
      tmax = fmax(tmax, fabs(d[i]) + r);
      if (i < n - 1) emax = fmax(emax, e[i] * e[i]);
      e2[i] = i < n - 1 ? e[i] * e[i] : 0.0;
    }
    const double span = fmax(ghi - glo, 1e-300);
    sh_misc[0] = glo - 1e-3 * span - 1e-300;
    sh_misc[1] = ghi + 1e-3 * span + 1e-300;
    sh_misc[2] = fmax(2.2250738585072014e-308, 4.930380657631324e-32 * fmax(1.0, emax));  // eps^2 * max e^2
    sh_misc[3] = tmax;
  }
  __syncthreads();
  const double pivmin = sh_misc[2], tnorm = sh_misc[3];
  if (tid < k) {
    lo[tid] = sh_misc[0];
    hi[tid] = sh_misc[1];
  }
  __syncthreads();

  // ---- multisection bisection for the k largest eigenvalues
  for (int round = 0; round < SY_ROUNDS; ++round) {
    const int j = tid / SY_S, s = tid % SY_S;
    if (j < k) {
      const double x = lo[j] + (hi[j] - lo[j]) * (double)(s + 1) / (double)(SY_S + 1);
      int c = 0;
      double q = d[0] - x;
      if (fabs(q) < pivmin) q = -pivmin;
      c += q < 0.0;
      for (int i = 1; i < n; ++i) {
        q = (d[i] - x) - e2[i - 1] / q;
        if (fabs(q) < pivmin) q = -pivmin;
        c += q < 0.0;
      }
      cnt[tid] = c;
      xs[tid] = x;
    }
    __syncthreads();
    if (tid < k) {
      const int idx = n - 1 - tid;  // ascending index of the tid-th largest
      double l = lo[tid], h = hi[tid];
      for (int s2 = 0; s2 < SY_S; ++s2) {
        const int c = cnt[tid * SY_S + s2];
        const double x = xs[tid * SY_S + s2];
        if (c <= idx) l = fmax(l, x);
        if (c >= idx + 1) h = fmin(h, x);
      }
      lo[tid] = l;
      hi[tid] = h;
    }
    __syncthreads();
  }
  if (tid < k) {
    const double lam = 0.5 * (lo[tid] + hi[tid]);
    lo[tid] = lam;  // lo[] now holds the eigenvalues
    if (lam_out) lam_out[(int64_t)b * k + tid] = lam;
  }
  __syncthreads();

  // ---- inverse iteration on T - lambda I (LDL^T, no pivoting), batches of SY_IB vectors
  const double clus = 1e-9 * fmax(tnorm, 1e-300);
  const double ptiny = fmax(pivmin, 2.220446049250313e-16 * 1e-3 * tnorm);
  for (int b0 = 0; b0 < k; b0 += SY_IB) {
    const int j = b0 + tid;
    if (tid < SY_IB && j < k) {
      const double lam = lo[j];
      double* Dp = &scr[tid * 130];
      for (int i = 0; i < n; ++i) A[sy_yidx(j, i)] = 1.0 + 0.5 * cos((double)((i + 1) * (j + 1)) * 0.7);
      for (int it = 0; it < 2; ++it) {
        double Dprev = d[0] - lam;
        if (fabs(Dprev) < ptiny) Dprev = Dprev < 0.0 ? -ptiny : ptiny;
        Dp[0] = Dprev;
        double z = A[sy_yidx(j, 0)];
        for (int i = 1; i < n; ++i) {
          const double L = e[i - 1] / Dprev;
          double Di = (d[i] - lam) - L * e[i - 1];
          if (fabs(Di) < ptiny) Di = Di < 0.0 ? -ptiny : ptiny;
          Dp[i] = Di;
          z = A[sy_yidx(j, i)] - L * z;
          A[sy_yidx(j, i)] = z;
          Dprev = Di;
        }
        double y = A[sy_yidx(j, n - 1)] / Dp[n - 1];
        A[sy_yidx(j, n - 1)] = y;
        double nrm = y * y;
        for (int i = n - 2; i >= 0; --i) {
          y = (A[sy_yidx(j, i)] - e[i] * y) / Dp[i];
          A[sy_yidx(j, i)] = y;
          nrm += y * y;
        }
        const double inv = 1.0 / sqrt(nrm);
        for (int i = 0; i < n; ++i) A[sy_yidx(j, i)] *= inv;
      }
    }
    __syncthreads();
  }
  // modified Gram-Schmidt inside clusters of (numerically) equal eigenvalues
  for (int j = 1; j < k; ++j) {
    for (int i = 0; i < j; ++i) {
      if (fabs(lo[i] - lo[j]) > clus) continue;  // uniform across the block
      if (wave == 0) {
        double s = 0.0;
        for (int c = lane; c < n; c += 64) s += A[sy_yidx(i, c)] * A[sy_yidx(j, c)];
        s = wave_sum_f64(s);
        for (int c = lane; c < n; c += 64) A[sy_yidx(j, c)] -= s * A[sy_yidx(i, c)];
        double s2 = 0.0;
        for (int c = lane; c < n; c += 64) s2 += A[sy_yidx(j, c)] * A[sy_yidx(j, c)];
        s2 = wave_sum_f64(s2);
        const double inv = s2 > 0.0 ? 1.0 / sqrt(s2) : 0.0;
        for (int c = lane; c < n; c += 64) A[sy_yidx(j, c)] *= inv;
      }
      __syncthreads();
    }
  }

  // ---- back-transformation x = H_0 (H_1 (... H_{n-3} y))
  for (int kk = n - 3; kk >= 0; --kk) {
    const double t = tau[kk];
    if (t == 0.0) continue;
    const int m = n - kk - 1;
    // w_j = v^T y_j over rows kk+1 .. n-1 (v_0 = 1); thread (j, part) partial sums
    {
      const int j = tid >> 3, part = tid & 7;
      double s = 0.0;
      if (j < k) {
        for (int r = part; r < m; r += 8) {
          const double v = r == 0 ? 1.0 : A[(kk + 1 + r) * SY_N + kk];
          s += v * A[sy_yidx(j, kk + 1 + r)];
        }
      }
      cnt[tid] = 0;
      scr[tid] = s;
    }
    __syncthreads();
    if (tid < k) {
      double s = 0.0;
      for (int p = 0; p < 8; ++p) s += scr[tid * 8 + p];
      red[tid] = t * s;
    }
    __syncthreads();
    {
      const int j = tid >> 3, part = tid & 7;
      if (j < k) {
        const double wj = red[j];
        for (int r = part; r < m; r += 8) {
          const double v = r == 0 ? 1.0 : A[(kk + 1 + r) * SY_N + kk];
          A[sy_yidx(j, kk + 1 + r)] -= v * wj;
        }
      }
    }
    __syncthreads();
  }

  // ---- sign normalisation and output
  if (tid < k) {
    const int j = tid;
    double best = -1.0, sgn = 1.0;
    for (int i = 0; i < n; ++i) {
      const double v = A[sy_yidx(j, i)];
      if (fabs(v) > best) {
        best = fabs(v);
        sgn = v < 0.0 ? -1.0 : 1.0;
      }
    }
    red[j] = sgn;
  }
  __syncthreads();
  for (int idx = tid; idx < n * k; idx += 256) {
    const int i = idx / k, j = idx % k;
    const double v = A[sy_yidx(j, i)] * red[j];
    const int64_t o = (int64_t)b * n * k + idx;
    if (U64) U64[o] = v;
    if (U32) U32[o] = (float)v;
    if (U16) U16[o] = f64_to_f16(v);
  }
}

hipError_t launch_syev_topk_any(const void* A, bool f32in, int n, int k, int batch, double* U64, float* U32,
                                _Float16* U16, double* lam, hipStream_t s) {
  if (n > SY_N || k > SY_K || k > n || n < 3) return hipErrorInvalidValue;
  if (f32in)
    hipLaunchKernelGGL(k_syev_topk<float>, dim3(batch), dim3(256), 0, s, (const float*)A, n, k, U64, U32, U16, lam);
  else
    hipLaunchKernelGGL(k_syev_topk<double>, dim3(batch), dim3(256), 0, s, (const double*)A, n, k, U64, U32, U16,
                       lam);
  return hipGetLastError();
}

hipError_t launch_syev_topk(const double* A, int n, int k, int batch, double* U64, float* U32, double* lam,
                            hipStream_t s) {
  return launch_syev_topk_any(A, false, n, k, batch, U64, U32, nullptr, lam, s);
}

// ============================================================ Cholesky inverse (CholeskyQR)
// W = sum of partial Grams (fp64); W = R^T R; writes R^{-1} (upper triangular) as fp32.
// A column whose pivot falls below 1e-13 * trace gets that floor (rank-deficient input).
__global__ __launch_bounds__(64) void k_chol_inv(const double* Wparts, int nparts, int p, void* Rinv, int f64out) {
  __shared__ double W[64][65];
  __shared__ double R[64][65];
  const int b = blockIdx.x, c = threadIdx.x;
  const double* src = Wparts + (int64_t)b * nparts * p * p;
  for (int r = 0; r < p; ++r) {
    if (c < p) {
      double s = 0.0;
      for (int q = 0; q < nparts; ++q) s += src[(int64_t)q * p * p + r * p + c];
      W[r][c] = s;
      R[r][c] = 0.0;
    }
  }
  __syncthreads();
  double tr = 0.0;
  for (int r = 0; r < p; ++r) tr += W[r][r];
  const double floor_ = fmax(1e-13 * tr, 1e-300);
  for (int j = 0; j < p; ++j) {
    double dj = W[j][j];
    if (!(dj > floor_)) dj = floor_;
    const double rjj = sqrt(dj);
    __syncthreads();
    if (c >= j && c < p) R[j][c] = c == j ? rjj : W[j][c] / rjj;
    __syncthreads();
    if (c > j && c < p) {
      const double rjc = R[j][c];
      for (int r = j + 1; r <= c; ++r) {
        W[r][c] -= R[j][r] * rjc;
        if (r != c) W[c][r] = W[r][c];
      }
    }
    __syncthreads();
  }
  // R^{-1}: column c by back substitution
  if (c < p) {
    double x[64];
    for (int i = p - 1; i >= 0; --i) {
      double s = i == c ? 1.0 : 0.0;
      for (int l = i + 1; l < p; ++l) s -= R[i][l] * x[l];
      x[i] = i > c ? 0.0 : s / R[i][i];
    }
    for (int i = 0; i < p; ++i) {
      const int64_t o = (int64_t)b * p * p + i * p + c;
      if (f64out) ((double*)Rinv)[o] = x[i];
      else ((float*)Rinv)[o] = (float)x[i];
    }
  }
}

hipError_t launch_chol_inv(const double* Wparts, int nparts, int p, int batch, void* Rinv, bool f64out,
                           hipStream_t s) {
  if (p > 64) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_chol_inv, dim3(batch), dim3(64), 0, s, Wparts, nparts, p, Rinv, f64out ? 1 : 0);
  return hipGetLastError();
}

// ============================================================ Gram reduction
__global__ void k_reduce_gram(const double* parts, int nparts, int DD, double* G) {
  const int t = blockIdx.y;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= DD) return;
  const double* src = parts + (int64_t)t * nparts * DD + idx;
  double s = 0.0;
  for (int q = 0; q < nparts; ++q) s += src[(int64_t)q * DD];
  G[(int64_t)t * DD + idx] = s;
}
__global__ void k_trace(const double* G, int D, int ntab, double* xn2, int32_t* flags) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= ntab) return;
  double s = 0.0;
  for (int i = 0; i < D; ++i) s += G[(int64_t)t * D * D + i * D + i];
  xn2[t] = s;
  if (!isfinite(s)) atomicOr(flags, 2);
}

hipError_t launch_reduce_gram(const double* parts, int nparts, int D, int ntab, double* G, double* xn2,
                              int32_t* flags, hipStream_t s) {
  const int DD = D * D;
  hipLaunchKernelGGL(k_reduce_gram, dim3((DD + 255) / 256, ntab), dim3(256), 0, s, parts, nparts, DD, G);
  hipLaunchKernelGGL(k_trace, dim3((ntab + 63) / 64), dim3(64), 0, s, G, D, ntab, xn2, flags);
  return hipGetLastError();
}

// ============================================================ feature factor preparation
__device__ __forceinline__ double hsign(int f, int i) { return (__popc(f & i) & 1) ? -1.0 : 1.0; }

__global__ void k_prep_feature(const double* Ud64, const int8_t* signs, int D, float* Ud32, _Float16* Ud16,
                               float* V32, _Float16* Vh, _Float16* Vl) {
  const int t = blockIdx.y;
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;  // f * 32 + j
  if (idx >= D * JOLT_KMAX) return;
  const int f = idx / JOLT_KMAX, j = idx % JOLT_KMAX;
  const int64_t base = (int64_t)t * D * JOLT_KMAX;
  const double u = Ud64[base + idx];
  Ud32[base + idx] = (float)u;
  Ud16[base + idx] = f64_to_f16(u);
  // V[f][j] = (1/sqrt(D)) sum_i H[f][i] sigma_i fp16(U_d[i][j])
  double s = 0.0;
  for (int i = 0; i < D; ++i) s += hsign(f, i) * (double)signs[t * D + i] * (double)f64_to_f16(Ud64[base + i * JOLT_KMAX + j]);
  const float v = (float)(s / sqrt((double)D));
  V32[base + idx] = v;
  const float nv = -v;
  const _Float16 h = (_Float16)nv;
  Vh[base + idx] = h;
  Vl[base + idx] = (_Float16)(nv - (float)h);
}

hipError_t launch_prep_feature(const double* Ud64, const int8_t* signs, int D, int ntab, float* Ud32,
                               _Float16* Ud16, float* V32, _Float16* Vneg_hi, _Float16* Vneg_lo, hipStream_t s) {
  hipLaunchKernelGGL(k_prep_feature, dim3((D * JOLT_KMAX + 255) / 256, ntab), dim3(256), 0, s, Ud64, signs, D, Ud32,
                     Ud16, V32, Vneg_hi, Vneg_lo);
  return hipGetLastError();
}

// ============================================================ subspace start block
__global__ void k_init_subspace(void* Q, int f64, int T, int64_t total) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= total) return;
  uint32_t h = (uint32_t)(idx % ((int64_t)T * JOLT_PSUB)) * 2654435761u;
  h ^= h >> 15;
  h *= 2246822519u;
  h ^= h >> 13;
  const float v = ((h & 1u) ? 1.0f : -1.0f) * rsqrtf((float)T) * (1.0f + 0.25f * (float)((h >> 8) & 7u) / 7.0f);
  if (f64) ((double*)Q)[idx] = (double)v;
  else ((float*)Q)[idx] = v;
}

hipError_t launch_init_subspace(void* Q, bool f64, int T, int batch, hipStream_t s) {
  const int64_t total = (int64_t)batch * T * JOLT_PSUB;
  hipLaunchKernelGGL(k_init_subspace, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, Q, f64 ? 1 : 0, T,
                     total);
  return hipGetLastError();
}

// ============================================================ rotated reconstruction operands
// For chain c < 4 (r_d = 4 << c): W[k][f] = sum_{j < r_d} G16[k][j] V[f][j];
// chain 4 (r_d = D): W[k][f] = (1/sqrt(D)) sum_i H[f][i] sigma_i G16[k][i].
// Stored negated, split into fp16 hi/lo, layout [t][c][n][f][k].
__global__ __launch_bounds__(256) void k_prep_w(const _Float16* G16, const float* V32, const int8_t* signs, int N,
                                                int D, _Float16* Wh, _Float16* Wl, int32_t* flags) {
  const int n = blockIdx.x, c = blockIdx.y, t = blockIdx.z;
  __shared__ float g[JOLT_KMAX][129];
  const int64_t gbase = (((int64_t)t * 5 + c) * N + n) * JOLT_KMAX * D;
  const int rd = c < 4 ? (4 << c) : D;
  for (int idx = threadIdx.x; idx < JOLT_KMAX * rd; idx += 256) {
    const int kk = idx / rd, j = idx % rd;
    g[kk][j] = (float)G16[gbase + (int64_t)kk * D + j];
  }
  __syncthreads();
  int overflow = 0;
  for (int idx = threadIdx.x; idx < D * JOLT_KMAX; idx += 256) {
    const int f = idx / JOLT_KMAX, kk = idx % JOLT_KMAX;
    double s = 0.0;
    if (c < 4) {
      const float* vrow = V32 + ((int64_t)t * D + f) * JOLT_KMAX;
      for (int j = 0; j < rd; ++j) s += (double)g[kk][j] * (double)vrow[j];
    } else {
      for (int i = 0; i < D; ++i) s += hsign(f, i) * (double)signs[t * D + i] * (double)g[kk][i];
      s /= sqrt((double)D);
    }
    const float w = -(float)s;
    const _Float16 h = (_Float16)w;
    if (!(fabsf((float)h) <= 65504.f)) overflow = 1;
    Wh[gbase / D * D + idx] = h;  // same base: [t][c][n] block of D*32 values
    Wl[gbase / D * D + idx] = (_Float16)(w - (float)h);
  }
  if (overflow) atomicOr(flags, 1);
}

hipError_t launch_prep_w(const _Float16* G16, const float* V32, const int8_t* signs, int N, int D, int ntab,
                         _Float16* Wneg_hi, _Float16* Wneg_lo, int32_t* flags, hipStream_t s) {
  hipLaunchKernelGGL(k_prep_w, dim3(N, 5, ntab), dim3(256), 0, s, G16, V32, signs, N, D, Wneg_hi, Wneg_lo, flags);
  return hipGetLastError();
}

}  // namespace jolt
