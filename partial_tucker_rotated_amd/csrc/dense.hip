// Small dense kernels of the factor stage: the symmetric top-k eigensolver used for
// the feature Gram, the small token Grams and the Rayleigh-Ritz matrices; the
// Cholesky inverse of CholeskyQR; Gram reduction; feature-factor preparation.
#include "jolt_internal.h"
#include "w_operands.h"

namespace jolt {

// ============================================================ symmetric top-k eigensolver
// Householder tridiagonalisation in fp64 (matrix in LDS); fp32 multisection bisection
// with Sturm counts for approximate k largest eigenvalues; fp64 inverse iteration on
// T - lambda I (LDL^T factored once, three solves), modified Gram-Schmidt inside
// clusters of nearly equal eigenvalues; back-transformation by the Householder
// vectors; sign normalisation (largest-magnitude entry positive).
#define SY_N 128
#define SY_LD 129   // LDS row stride of A: columns as well as rows read without bank conflicts
#define SY_K 32
#define SY_IB 16     // eigenvectors per inverse-iteration batch (LDS for the pivots)
#define SY_S 16      // bisection samples per eigenvalue and round
#define SY_ROUNDS 6  // 17^6 ~ 2.4e7: fp32 resolution of the spectrum
#define SY_THREADS 512

// eigenvector j, component i, stored in the upper-right quadrant of the matrix
// array (free once the matrix is tridiagonal), rotated so that lanes j do not collide
// 1 / x: hardware reciprocal refined by one Newton step y <- y (2 - x y) (a few ulp)
__device__ __forceinline__ double recip(double x) {
  const double y = __builtin_amdgcn_rcp(x);
  return fma(y, fma(-x, y, 1.0), y);
}

__device__ __forceinline__ int sy_yidx(int j, int i) { return (2 * j + (i >> 6)) * SY_LD + 64 + ((i + 2 * j) & 63); }

template <typename TIn>
__global__ __launch_bounds__(SY_THREADS) void k_syev_topk(const TIn* Aall, int n, int k, double* U64, float* U32,
                                                          _Float16* U16, double* lam_out) {
  __shared__ double A[SY_N * SY_LD];
  __shared__ double scr[SY_IB * 130];  // 1/pivots of an inverse-iteration batch; earlier: partials, v copies
  static_assert(SY_IB * 130 >= 12 * SY_N, "partials and eight wave copies of v");
  __shared__ double d[SY_N], e[SY_N], tau[SY_N], sgn[SY_K];
  __shared__ float lo[SY_K], hi[SY_K], lamf[SY_K];
  __shared__ float df[SY_N], e2f[SY_N];
  __shared__ float xs[SY_THREADS];
  __shared__ int cnt[SY_THREADS];
  __shared__ double red[8], red2[8];
  __shared__ double sh_misc[4];
  double* parts = scr;  // [4][SY_N] partial matvec sums (tridiagonalisation)

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int b = blockIdx.x;
  const TIn* Ain = Aall + (int64_t)b * n * n;
  for (int idx = tid; idx < n * n; idx += SY_THREADS) A[(idx / n) * SY_LD + idx % n] = (double)Ain[idx];
  __syncthreads();

  // ---- tridiagonalisation: A = Q T Q^T, Q = H_0 ... H_{n-3}
  // The squared norm of the next column below its subdiagonal is accumulated by the
  // update of the current step (lane 0 of every wave owns column 0 of its rows).
  // Two barriers per step: every wave builds its own copy of v (so no barrier publishes
  // it), and after the matvec partials every wave forms p, p^T v and w for itself; rows'
  // entries of p are read across lanes (row indices are wave-uniform).
  bool have_sigma = false;
  double* vw = scr + 4 * SY_N + wave * SY_N;  // this wave's copy of v
  for (int kk = 0; kk < n - 2; ++kk) {
    const int m = n - kk - 1;  // size of the trailing block
    if (!have_sigma) {
      if (wave == 0) {
        double s = 0.0;
        for (int i = kk + 2 + lane; i < n; i += 64) s += A[i * SY_LD + kk] * A[i * SY_LD + kk];
        s = wave_sum_f64(s);
        if (lane == 0) red2[0] = s;
      }
      if (tid < SY_THREADS / 64 && tid > 0) red2[tid] = 0.0;
      __syncthreads();
    }
    double sigma = 0.0;
#pragma unroll
    for (int w = 0; w < SY_THREADS / 64; ++w) sigma += red2[w];
    const double x0 = A[(kk + 1) * SY_LD + kk];
    double t = 0.0, sc = 0.0, beta = x0;
    if (sigma != 0.0) {
      const double nx = sqrt(x0 * x0 + sigma);
      beta = x0 >= 0.0 ? -nx : nx;
      t = (beta - x0) * recip(beta);
      sc = recip(x0 - beta);
    }
    if (tid == 0) {
      d[kk] = A[kk * SY_LD + kk];
      tau[kk] = t;
      e[kk] = beta;
    }
    have_sigma = false;
    if (t == 0.0) {  // uniform: the column is already reduced
      __syncthreads();
      continue;
    }
    const bool c0in = lane < m, c1in = lane + 64 < m;
    const double v0 = c0in ? (lane == 0 ? 1.0 : A[(kk + 1 + lane) * SY_LD + kk] * sc) : 0.0;
    const double v1 = c1in ? A[(kk + 65 + lane) * SY_LD + kk] * sc : 0.0;
    vw[lane] = v0;
    vw[lane + 64] = v1;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    {  // partial sums of A22 v: thread (column i, quarter q) over a quarter of the rows,
       // 8 rows per batch of loads
      const int i = tid & 127, q = tid >> 7;
      double sv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) sv[u] = 0.0;
      if (i < m) {
        const int j0 = (m * q) >> 2, j1 = (m * (q + 1)) >> 2;
        const double* col = &A[(kk + 1) * SY_LD + kk + 1 + i];
        int j = j0;
        for (; j + 7 < j1; j += 8) {
          double av[8], vr[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            av[u] = col[(j + u) * SY_LD];
            vr[u] = vw[j + u];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) sv[u] = fma(av[u], vr[u], sv[u]);
        }
        for (; j < j1; ++j) sv[0] = fma(col[j * SY_LD], vw[j], sv[0]);
      }
      parts[q * SY_N + i] = ((sv[0] + sv[1]) + (sv[2] + sv[3])) + ((sv[4] + sv[5]) + (sv[6] + sv[7]));
    }
    __syncthreads();  // B3: the partials are complete; column kk is no longer read
    {  // p = tau (A22 v), p^T v and w = p - (tau/2)(p^T v) v in every wave; then
       // A22 -= v w^T + w v^T; lane 0 accumulates the next step's column norm (rows kk + 3 ...)
      const double p0 = c0in ? t * ((parts[lane] + parts[SY_N + lane]) + (parts[2 * SY_N + lane] + parts[3 * SY_N + lane]))
                             : 0.0;
      const double p1 = c1in ? t * ((parts[lane + 64] + parts[SY_N + lane + 64]) +
                                    (parts[2 * SY_N + lane + 64] + parts[3 * SY_N + lane + 64]))
                             : 0.0;
      const double pv = wave_sum_f64(fma(p1, v1, p0 * v0));
      const double K = 0.5 * t * pv;
      const double w0 = p0 - K * v0, w1 = p1 - K * v1;
      if (wave == 0) {  // the Householder vector is kept below the subdiagonal of column kk
        if (c0in && lane > 0) A[(kk + 1 + lane) * SY_LD + kk] = v0;
        if (c1in) A[(kk + 65 + lane) * SY_LD + kk] = v1;
      }
      // rows wave, wave + 8, ... in groups of 4 whose loads are all issued before the
      // group's stores
      double nsq = 0.0;
      constexpr int RS = SY_THREADS / 64;
      int r = wave;
      for (; r + 3 * RS < m; r += 4 * RS) {
        double vr[4], wr[4], a0[4], a1[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rr = r + u * RS;
          const double* row = &A[(kk + 1 + rr) * SY_LD + kk + 1];
          vr[u] = vw[rr];
          wr[u] = rr < 64 ? readlane_f64(w0, rr) : readlane_f64(w1, rr - 64);
          a0[u] = c0in ? row[lane] : 0.0;
          a1[u] = c1in ? row[lane + 64] : 0.0;
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int rr = r + u * RS;
          double* row = &A[(kk + 1 + rr) * SY_LD + kk + 1];
          const double n0 = a0[u] - (vr[u] * w0 + wr[u] * v0);
          const double n1 = a1[u] - (vr[u] * w1 + wr[u] * v1);
          if (c0in) row[lane] = n0;
          if (c1in) row[lane + 64] = n1;
          if (lane == 0 && rr >= 2) nsq += n0 * n0;
        }
      }
      for (; r < m; r += RS) {
        const double vr = vw[r], wr = r < 64 ? readlane_f64(w0, r) : readlane_f64(w1, r - 64);
        double* row = &A[(kk + 1 + r) * SY_LD + kk + 1];
        if (c0in) {
          const double nv = row[lane] - (vr * w0 + wr * v0);
          row[lane] = nv;
          if (lane == 0 && r >= 2) nsq += nv * nv;
        }
        if (c1in) row[lane + 64] -= vr * w1 + wr * v1;
      }
      if (lane == 0) red2[wave] = nsq;
    }
    have_sigma = true;
    __syncthreads();  // B5
  }
  if (tid == 0) {
    if (n >= 2) {
      d[n - 2] = A[(n - 2) * SY_LD + n - 2];
      e[n - 2] = A[(n - 1) * SY_LD + n - 2];
      tau[n - 2] = 0.0;
    }
    d[n - 1] = A[(n - 1) * SY_LD + n - 1];
    e[n - 1] = 0.0;
    tau[n - 1] = 0.0;
    double glo = 1e300, ghi = -1e300, tmax = 0.0;
    for (int i = 0; i < n; ++i) {
      const double r = (i > 0 ? fabs(e[i - 1]) : 0.0) + (i < n - 1 ? fabs(e[i]) : 0.0);
      glo = fmin(glo, d[i] - r);
      ghi = fmax(ghi, d[i] + r);
      tmax = fmax(tmax, fabs(d[i]) + r);
    }
    if (!(tmax > 0.0)) tmax = 1.0;  // zero matrix: any scale works
    const double span = fmax(ghi - glo, tmax * 1e-6);
    sh_misc[0] = glo - 1e-3 * span;
    sh_misc[1] = ghi + 1e-3 * span;
    sh_misc[3] = tmax;
  }
  __syncthreads();
  const double tnorm = sh_misc[3];
  // fp32 copies for the counts (scaled by 1 / ||T|| to stay well inside the fp32 range)
  const double inv_tn = 1.0 / tnorm;
  if (tid < k) {
    lo[tid] = (float)(sh_misc[0] * inv_tn);
    hi[tid] = (float)(sh_misc[1] * inv_tn);
  }
  for (int i = tid; i < n; i += SY_THREADS) {
    df[i] = (float)(d[i] * inv_tn);
    const float ei = (float)(e[i] * inv_tn);
    e2f[i] = ei * ei;
  }
  __syncthreads();

  // ---- fp32 multisection: eigenvalue index n-1-j (the j-th largest) lies in [lo_j, hi_j)
  {
    const float pivmin = 1e-30f;
    for (int round = 0; round < SY_ROUNDS; ++round) {
      const int j = tid / SY_S, s = tid % SY_S;
      if (j < k) {
        const float x = lo[j] + (hi[j] - lo[j]) * (float)(s + 1) / (float)(SY_S + 1);
        int c = 0;
        float q = df[0] - x;
        if (fabsf(q) < pivmin) q = -pivmin;
        c += q < 0.f;
        for (int i = 1; i < n; ++i) {
          q = (df[i] - x) - e2f[i - 1] * __builtin_amdgcn_rcpf(q);
          if (fabsf(q) < pivmin) q = -pivmin;
          c += q < 0.f;
        }
        cnt[tid] = c;
        xs[tid] = x;
      }
      __syncthreads();
      if (tid < k) {
        const int idx = n - 1 - tid;
        float l = lo[tid], h = hi[tid];
        for (int s2 = 0; s2 < SY_S; ++s2) {
          const int c = cnt[tid * SY_S + s2];
          const float x = xs[tid * SY_S + s2];
          if (c <= idx) l = fmaxf(l, x);
          if (c >= idx + 1) h = fminf(h, x);
        }
        lo[tid] = l;
        hi[tid] = h;
      }
      __syncthreads();
    }
    if (tid < k) lamf[tid] = 0.5f * (lo[tid] + hi[tid]);
    __syncthreads();
  }

  // ---- inverse iteration on T - lambda I (LDL^T without pivoting, factored once);
  // passes over the vector move 8 entries at a time between LDS and registers
  // Pivots are kept at least eps * ||T|| in magnitude, so one step of either recurrence
  // grows the vector by at most ~2 / eps; after every 8 entries a vector that has grown
  // past 1e100 is rescaled as a whole (processed and unprocessed entries: only its
  // direction matters), which keeps it finite for any shift, also inside clusters of
  // (near-)zero eigenvalues of rank-deficient inputs.
  const double ptiny = 2.220446049250313e-16 * tnorm;
  const double big = 1e100;
  for (int b0 = 0; b0 < k; b0 += SY_IB) {
    const int j = b0 + tid;
    if (tid < SY_IB && j < k) {
      const double lam = (double)lamf[j] * tnorm;
      double* iD = &scr[tid * 130];
      double Dprev = d[0] - lam;
      if (fabs(Dprev) < ptiny) Dprev = Dprev < 0.0 ? -ptiny : ptiny;
      double idp = recip(Dprev);
      iD[0] = idp;
      for (int i = 1; i < n; ++i) {
        double Di = (d[i] - lam) - e[i - 1] * e[i - 1] * idp;
        if (fabs(Di) < ptiny) Di = Di < 0.0 ? -ptiny : ptiny;
        idp = recip(Di);
        iD[i] = idp;
      }
      // start vector: deterministic pseudo-random entries in [0.5, 1.5)
      for (int i = 0; i < n; ++i) {
        uint32_t h = (uint32_t)(i * 0x9E3779B1u) ^ (uint32_t)((j + 1) * 0x85EBCA77u);
        h ^= h >> 15;
        h *= 0x2C1B3C6Du;
        h ^= h >> 12;
        A[sy_yidx(j, i)] = 0.5 + (double)(h >> 8) * (1.0 / 16777216.0);
      }
      // three solves; only the direction matters, so the vector is normalised once at
      // the end (the rescaling guards keep it finite in between)
      double gmx = 0.0;  // largest magnitude of the last solve's entries
      for (int it = 0; it < 3; ++it) {
        // L z = x (L_{i,i-1} = e_{i-1} / D_{i-1})
        double z = 0.0, lprev = 0.0;
        for (int i0 = 0; i0 < n; i0 += 8) {
          double xv[8], ev[8], dv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            xv[u] = A[sy_yidx(j, i0 + u)];
            ev[u] = e[i0 + u];
            dv[u] = iD[i0 + u];
          }
          double mx = 0.0;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            z = xv[u] - lprev * z;
            xv[u] = z;
            lprev = ev[u] * dv[u];
            mx = fmax(mx, fabs(z));
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) A[sy_yidx(j, i0 + u)] = xv[u];
          if (mx > big) {  // rare: rescale the whole vector
            const double sc = 1.0 / mx;
            for (int i = 0; i < n; ++i) A[sy_yidx(j, i)] *= sc;
            z *= sc;
          }
        }
        // D L^T y = z
        double y = 0.0;
        gmx = 0.0;
        for (int i0 = n - 8; i0 >= 0; i0 -= 8) {
          double zv[8], ev[8], dv[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            zv[u] = A[sy_yidx(j, i0 + u)];
            ev[u] = e[i0 + u];
            dv[u] = iD[i0 + u];
          }
          double mx = 0.0;
#pragma unroll
          for (int u = 7; u >= 0; --u) {
            y = (zv[u] - ev[u] * y) * dv[u];  // e[n-1] = 0 starts the recurrence
            zv[u] = y;
            mx = fmax(mx, fabs(y));
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) A[sy_yidx(j, i0 + u)] = zv[u];
          gmx = fmax(gmx, mx);
          if (gmx > big) {
            const double sc = 1.0 / gmx;
            for (int i = 0; i < n; ++i) A[sy_yidx(j, i)] *= sc;
            y *= sc;
            gmx = 1.0;
          }
        }
      }
      // normalise: scale by the largest entry first so the sum of squares cannot overflow
      const double sm = gmx > 0.0 ? 1.0 / gmx : 0.0;
      double nrm = 0.0;
      for (int i0 = 0; i0 < n; i0 += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = A[sy_yidx(j, i0 + u)] * sm;
#pragma unroll
        for (int u = 0; u < 8; ++u) nrm = fma(v[u], v[u], nrm);
      }
      const double inv = nrm > 0.0 ? sm / sqrt(nrm) : 0.0;
      for (int i0 = 0; i0 < n; i0 += 8) {
        double v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) v[u] = A[sy_yidx(j, i0 + u)];
#pragma unroll
        for (int u = 0; u < 8; ++u) A[sy_yidx(j, i0 + u)] = v[u] * inv;
      }
    }
    __syncthreads();
  }
  // modified Gram-Schmidt inside clusters of eigenvalues the fp32 bisection cannot separate
  const float clus = 1e-5f;
  float lamr[SY_K];
#pragma unroll
  for (int i = 0; i < SY_K; ++i) lamr[i] = i < k ? lamf[i] : 0.f;
  for (int j = 1; j < k; ++j) {
    bool any = false;
    for (int i = 0; i < j; ++i) any |= fabsf(lamr[i] - lamr[j]) <= clus;
    if (!any) continue;  // uniform across the block
    for (int i = 0; i < j; ++i) {
      if (fabsf(lamr[i] - lamr[j]) > clus) continue;  // uniform across the block
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

  // ---- back-transformation x = H_0 (H_1 (... H_{n-3} y)); 16 lanes per eigenvector,
  // lane g keeping entries g, g + 16, ... in registers; a step is one batch of loads of
  // the reflector (prefetched a step ahead), one 16-lane reduction and 8 FMAs.  Each wave
  // owns its vectors: no block barriers inside the loop.
  {
    const int j = tid >> 4, g = tid & 15;
    const bool own = j < k;
    double y[8], hn[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = g + 16 * u;
      y[u] = (own && i < n) ? A[sy_yidx(j, i)] : 0.0;
    }
    // reflector kk at entries i: 0 for i <= kk, 1 at kk + 1, A(i, kk) below
    auto load_h = [&](int kk, double (&h)[8]) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const int i = g + 16 * u;
        const double x = A[(i < n ? i : n - 1) * SY_LD + kk];
        h[u] = i > kk + 1 && i < n ? x : (i == kk + 1 ? 1.0 : 0.0);
      }
    };
    load_h(n - 3, hn);
    for (int kk = n - 3; kk >= 0; --kk) {
      double hv[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) hv[u] = hn[u];
      if (kk > 0) load_h(kk - 1, hn);
      const double t = tau[kk];
      if (t == 0.0) continue;
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int u = 0; u < 8; u += 2) {
        s0 = fma(hv[u], y[u], s0);
        s1 = fma(hv[u + 1], y[u + 1], s1);
      }
      const double ts = t * row16_sum_f64(s0 + s1);
#pragma unroll
      for (int u = 0; u < 8; ++u) y[u] = fma(-ts, hv[u], y[u]);
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = g + 16 * u;
      if (own && i < n) A[sy_yidx(j, i)] = y[u];
    }
  }
  __syncthreads();
  // ---- sign normalisation and output
  if (tid < k) {
    const int j = tid;
    double best = -1.0, sg = 1.0;
    for (int i = 0; i < n; ++i) {
      const double v = A[sy_yidx(j, i)];
      if (fabs(v) > best) {
        best = fabs(v);
        sg = v < 0.0 ? -1.0 : 1.0;
      }
    }
    sgn[j] = sg;
    if (lam_out) lam_out[(int64_t)b * k + j] = (double)lamf[j] * tnorm;
  }
  __syncthreads();
  for (int idx = tid; idx < n * k; idx += SY_THREADS) {
    const int i = idx / k, j = idx % k;
    const double v = A[sy_yidx(j, i)] * sgn[j];
    const int64_t o = (int64_t)b * n * k + idx;
    if (U64) U64[o] = v;
    if (U32) U32[o] = (float)v;
    if (U16) U16[o] = f64_to_f16(v);
  }
}

hipError_t launch_syev_topk_any(const void* A, bool f32in, int n, int k, int batch, double* U64, float* U32,
                                _Float16* U16, double* lam, hipStream_t s) {
  // inverse iteration walks the vectors 8 entries at a time
  if (n > SY_N || k > SY_K || k > n || n < 8 || (n & 7)) return hipErrorInvalidValue;
  if (f32in)
    hipLaunchKernelGGL(k_syev_topk<float>, dim3(batch), dim3(SY_THREADS), 0, s, (const float*)A, n, k, U64, U32,
                       U16, lam);
  else
    hipLaunchKernelGGL(k_syev_topk<double>, dim3(batch), dim3(SY_THREADS), 0, s, (const double*)A, n, k, U64, U32,
                       U16, lam);
  return hipGetLastError();
}

hipError_t launch_syev_topk(const double* A, int n, int k, int batch, double* U64, float* U32, double* lam,
                            hipStream_t s) {
  return launch_syev_topk_any(A, false, n, k, batch, U64, U32, nullptr, lam, s);
}

// ============================================================ CholeskyQR Grams (fp64 MFMA)
// One workgroup per (row chunk, block): the chunk passes through LDS in slabs of 64 rows
// (columns p .. 16 NT - 1 zero-filled, NT = ceil(p / 16)); wave w takes rows 16 w .. 16 w + 15
// of every slab and accumulates the NT (NT + 1) / 2 tiles on and above the diagonal of
// Z^T Z with v_mfma_f64_16x16x4f64; the four waves' sums are added in wave order at the
// end and each tile is written with its mirror.  Tile operands: A(i, k) = Z[k][16 I + i] in
// lane i + 16 k, B(k, j) = Z[k][16 J + j] in lane j + 16 k; result (i, j) in lane
// 16 (i & 3) + j, register i >> 2.  Every product and sum is fp64 (fp32 inputs are exact
// in fp64), so the Gram carries no rounding beyond fp64's.
typedef double gram_d4 __attribute__((ext_vector_type(4)));
constexpr int GRAM_SLAB = 64;
constexpr int GRAM_LS = 80;  // LDS row stride (elements): 4 consecutive rows hit disjoint banks

template <typename TIn, int NT>
__global__ __launch_bounds__(256) void k_gram64(const TIn* src, int64_t rows, int p, int nparts, double* W) {
  constexpr int NU = NT * (NT + 1) / 2;
  __shared__ __align__(16) TIn Zs[GRAM_SLAB][GRAM_LS];
  __shared__ double red[4][256];
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int64_t chunk = rows / nparts;
  const TIn* Z = src + ((int64_t)b * rows + (int64_t)q * chunk) * p;
  const int li = lane & 15, lk = lane >> 4;
  constexpr int VEC = 16 / sizeof(TIn);  // elements per 16-byte load
  constexpr int GPR = 16 * NT / VEC;     // 16-byte groups per staged row
  gram_d4 acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = (gram_d4){0.0, 0.0, 0.0, 0.0};
  for (int64_t r0 = 0; r0 < chunk; r0 += GRAM_SLAB) {
    const int nr = (int)(chunk - r0 < GRAM_SLAB ? chunk - r0 : GRAM_SLAB);
    // slab rows r0 .. r0 + 63 (zero past the chunk and past column p); p % 4 == 0 and the
    // block starts 16-byte aligned, so each 16-byte group of a row lies wholly inside or
    // outside p
    for (int e = tid; e < GRAM_SLAB * GPR; e += 256) {
      const int r = e / GPR, c = (e - r * GPR) * VEC;
      uint4 v = make_uint4(0u, 0u, 0u, 0u);
      if (r < nr && c < p) v = *(const uint4*)(Z + (r0 + r) * p + c);
      *(uint4*)&Zs[r][c] = v;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // rows past nr are zero
      const int k = 16 * w + 4 * ks + lk;
      double a[NT];
#pragma unroll
      for (int I = 0; I < NT; ++I) a[I] = (double)Zs[k][16 * I + li];
      int u = 0;
#pragma unroll
      for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = I; J < NT; ++J, ++u) acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[I], a[J], acc[u], 0, 0, 0);
    }
    __syncthreads();
  }
  double* out = W + ((int64_t)b * nparts + q) * p * p;
  int u = 0;
#pragma unroll
  for (int I = 0; I < NT; ++I)
#pragma unroll
    for (int J = I; J < NT; ++J, ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][r * 64 + lane] = acc[u][r];
      __syncthreads();
      {  // element (4 r + lk', li') of the tile, r = tid >> 6, lane' = tid & 63
        const double v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        const int r = tid >> 6, l = tid & 63;
        const int i = 16 * I + 4 * r + (l >> 4), j = 16 * J + (l & 15);
        if (i < p && j < p) {
          out[i * p + j] = v;
          if (I != J) out[j * p + i] = v;
        }
      }
      __syncthreads();
    }
}

// Cross Gram of two fp32 [rows][64] blocks, W[b][q] = Z_q^T P_q over row chunk q (fp64 MFMA,
// all 16 tiles; the layout and order of k_gram64, with A from Z and B from P).
__global__ __launch_bounds__(256) void k_gram_cross(const float* Z, const float* Pm, int64_t rows, int nparts,
                                                    double* W) {
  __shared__ __align__(16) float Zs[GRAM_SLAB][GRAM_LS], Ps[GRAM_SLAB][GRAM_LS];
  __shared__ double red[4][256];
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, li = lane & 15, lk = lane >> 4;
  const int64_t chunk = rows / nparts;
  const float* Zb = Z + ((int64_t)b * rows + (int64_t)q * chunk) * 64;
  const float* Pb = Pm + ((int64_t)b * rows + (int64_t)q * chunk) * 64;
  gram_d4 acc[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) acc[u] = (gram_d4){0.0, 0.0, 0.0, 0.0};
  for (int64_t r0 = 0; r0 < chunk; r0 += GRAM_SLAB) {
    const int nr = (int)(chunk - r0 < GRAM_SLAB ? chunk - r0 : GRAM_SLAB);
    for (int e = tid; e < GRAM_SLAB * 16; e += 256) {
      const int r = e >> 4, c = (e & 15) * 4;
      uint4 vz = make_uint4(0u, 0u, 0u, 0u), vp = vz;
      if (r < nr) {
        vz = *(const uint4*)(Zb + (r0 + r) * 64 + c);
        vp = *(const uint4*)(Pb + (r0 + r) * 64 + c);
      }
      *(uint4*)&Zs[r][c] = vz;
      *(uint4*)&Ps[r][c] = vp;
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      const int k = 16 * w + 4 * ks + lk;
      double a[4], bb[4];
#pragma unroll
      for (int I = 0; I < 4; ++I) {
        a[I] = (double)Zs[k][16 * I + li];
        bb[I] = (double)Ps[k][16 * I + li];
      }
#pragma unroll
      for (int I = 0; I < 4; ++I)
#pragma unroll
        for (int J = 0; J < 4; ++J)
          acc[4 * I + J] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[I], bb[J], acc[4 * I + J], 0, 0, 0);
    }
    __syncthreads();
  }
  double* out = W + ((int64_t)b * nparts + q) * 64 * 64;
#pragma unroll
  for (int u = 0; u < 16; ++u) {
#pragma unroll
    for (int r = 0; r < 4; ++r) red[w][r * 64 + lane] = acc[u][r];
    __syncthreads();
    {
      const double v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
      const int r = tid >> 6, l = tid & 63;
      out[(16 * (u >> 2) + 4 * r + (l >> 4)) * 64 + 16 * (u & 3) + (l & 15)] = v;
    }
    __syncthreads();
  }
}

hipError_t launch_gram_cross(const float* Z, const float* P, int64_t rows, int nparts, int batch, double* W,
                             hipStream_t s) {
  if (nparts < 1 || rows < nparts || rows % nparts || batch < 1 || batch > 65535 || nparts > 65535)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_gram_cross, dim3(nparts, batch), dim3(256), 0, s, Z, P, rows, nparts, W);
  return hipGetLastError();
}

hipError_t launch_gram64(const void* src, bool f64in, int64_t rows, int p, int nparts, int batch, double* W,
                         hipStream_t s) {
  if (p > 64 || p < 4 || (p & 3) || nparts < 1 || rows < nparts || rows % nparts || batch < 1 ||
      batch > 65535 || nparts > 65535)
    return hipErrorInvalidValue;
  const dim3 g(nparts, batch);
  const int nt = (p + 15) / 16;
#define JOLT_GRAM(T_, NT_) hipLaunchKernelGGL((k_gram64<T_, NT_>), g, dim3(256), 0, s, (const T_*)src, rows, p, nparts, W)
  if (f64in) {
    if (nt == 1) JOLT_GRAM(double, 1);
    else if (nt == 2) JOLT_GRAM(double, 2);
    else if (nt == 3) JOLT_GRAM(double, 3);
    else JOLT_GRAM(double, 4);
  } else {
    if (nt == 1) JOLT_GRAM(float, 1);
    else if (nt == 2) JOLT_GRAM(float, 2);
    else if (nt == 3) JOLT_GRAM(float, 3);
    else JOLT_GRAM(float, 4);
  }
#undef JOLT_GRAM
  return hipGetLastError();
}

// Sum of `nparts` consecutive fp64 blocks of `len` values per batch entry, in block order:
// out[b][i] = sum_q W[(b nparts + q) len + i].
__global__ __launch_bounds__(256) void k_sum_parts(const double* __restrict__ W, int nparts, int len,
                                                   double* __restrict__ out) {
  const int b = blockIdx.y;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < len; i += gridDim.x * 256) {
    const double* src = W + (int64_t)b * nparts * len + i;
    double a = 0.0;
    for (int q = 0; q < nparts; ++q) a += src[(int64_t)q * len];
    out[(int64_t)b * len + i] = a;
  }
}

hipError_t launch_sum_parts(const double* W, int nparts, int len, int batch, double* out, hipStream_t s) {
  if (nparts < 1 || len < 1 || batch < 1 || batch > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_sum_parts, dim3((len + 255) / 256, batch), dim3(256), 0, s, W, nparts, len, out);
  return hipGetLastError();
}

// Token factor from a basis and the eigenvectors of its Rayleigh quotient:
// U_b[t][m] = sum_c S[b][t][c] V[b][c][m] (c < P = 40 or 64 basis columns, m < 32), fp32 FMAs
// in ascending c; written in fp32 and as fp16 (one rounding of the fp32 value) at
// (b / div) u1 + (b % div) u2 + 32 t.  One thread per row t; V of the workgroup's problem b
// in LDS (every lane reads the same V entries: broadcast).
template <int P>
__global__ __launch_bounds__(256) void k_ut_rows(const float* __restrict__ S, const float* __restrict__ V, int T,
                                                 float* __restrict__ U32, _Float16* __restrict__ U16, int div,
                                                 int64_t u1, int64_t u2) {
  constexpr int KM = JOLT_KMAX;
  const int b = blockIdx.y, tid = threadIdx.x;
  __shared__ __align__(16) float vs[P][KM];
  for (int idx = tid; idx < P * KM; idx += 256) (&vs[0][0])[idx] = V[(int64_t)b * P * KM + idx];
  __syncthreads();
  const int t = blockIdx.x * 256 + tid;
  if (t >= T) return;
  const float4* srow = (const float4*)(S + ((int64_t)b * T + t) * P);
  float sv[P];
#pragma unroll
  for (int q = 0; q < P / 4; ++q) {
    const float4 v = srow[q];
    sv[4 * q] = v.x; sv[4 * q + 1] = v.y; sv[4 * q + 2] = v.z; sv[4 * q + 3] = v.w;
  }
  float u[KM];
#pragma unroll
  for (int m = 0; m < KM; ++m) u[m] = 0.f;
#pragma unroll
  for (int c = 0; c < P; ++c)
#pragma unroll
    for (int q = 0; q < KM / 4; ++q) {
      const float4 v = *(const float4*)&vs[c][4 * q];
      u[4 * q] = fmaf(sv[c], v.x, u[4 * q]);
      u[4 * q + 1] = fmaf(sv[c], v.y, u[4 * q + 1]);
      u[4 * q + 2] = fmaf(sv[c], v.z, u[4 * q + 2]);
      u[4 * q + 3] = fmaf(sv[c], v.w, u[4 * q + 3]);
    }
  const int64_t o = (int64_t)(b / div) * u1 + (int64_t)(b % div) * u2 + (int64_t)t * KM;
#pragma unroll
  for (int q = 0; q < KM / 4; ++q) *(float4*)(U32 + o + 4 * q) = make_float4(u[4 * q], u[4 * q + 1], u[4 * q + 2], u[4 * q + 3]);
#pragma unroll
  for (int q = 0; q < KM / 8; ++q) {
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e)
      w[e] = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)u[8 * q + 2 * e]) |
             ((uint32_t)__builtin_bit_cast(uint16_t, (_Float16)u[8 * q + 2 * e + 1]) << 16);
    *(uint4*)(U16 + o + 8 * q) = make_uint4(w[0], w[1], w[2], w[3]);
  }
}

hipError_t launch_ut_rows(const float* S, const float* V, int p, int T, int batch, float* U32, _Float16* U16,
                          int div, int64_t u1, int64_t u2, hipStream_t s) {
  if ((p != 40 && p != 64) || T < 1 || batch < 1 || batch > 65535 || div < 1) return hipErrorInvalidValue;
  const dim3 g((T + 255) / 256, batch);
  if (p == 40) hipLaunchKernelGGL(k_ut_rows<40>, g, dim3(256), 0, s, S, V, T, U32, U16, div, u1, u2);
  else hipLaunchKernelGGL(k_ut_rows<64>, g, dim3(256), 0, s, S, V, T, U32, U16, div, u1, u2);
  return hipGetLastError();
}

// ============================================================ Cholesky inverse (CholeskyQR)
// r = sqrt(x), iv = 1 / sqrt(x) for x > 0: hardware reciprocal square root refined by one
// Newton step y <- y (3 - x y^2) / 2 (a few ulp, no IEEE divide or square-root sequence)
__device__ __forceinline__ void sqrt_and_inv(double x, double& r, double& iv) {
  double y = __builtin_amdgcn_rsq(x);
  const double h = 0.5 * x;
  y = fma(y, fma(-h * y, y, 0.5), y);
  iv = y;
  r = x * y;
}

// Relative shift of the CholeskyQR factorisations.  Their Grams are summed in fp64 from
// the working values, so the shift only has to cover fp64 rounding; directions down to
// about sqrt(kOrthShift) = 1e-7 of the block's largest singular value are normalised.
constexpr double kOrthShift = 1e-14;

// ------------------------------------------------------------ blocked Cholesky inverse
// One workgroup (4 waves) per Gram; the Gram is padded to 64 x 64 with the identity
// (the factor of the padded matrix is blockdiag(R, I)).  Lower Cholesky W + s I = L L^T in
// four 16-column panels: wave 0 factors a panel with one lane per row (the pivot and the
// multipliers of a column are broadcast with readlane), the four waves subtract the panel's
// outer product from the trailing blocks with v_mfma_f64_16x16x4f64.  Then Y = L^{-1}:
// the diagonal blocks by forward substitution with one lane per column, the blocks below
// by levels, Y_IJ = -Y_II sum_K L_IK Y_KJ with fp64 MFMA (the register layout of a
// product tile is the layout of a B operand, so the two products chain in registers).
// R^{-1} = Y^T.  All arithmetic is fp64.
#define CB_LD 66  // LDS row stride (doubles): the 16 x 4 operand reads hit distinct banks
typedef double cb_d4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ double cb_readlane(double v, int l) { return readlane_f64(v, l); }

__global__ __launch_bounds__(256) void k_chol_inv_blk(const double* Wparts, int nparts, int p, double rel_shift,
                                                      void* Rinv, int f64out) {
  __shared__ double W[64][CB_LD];   // the Gram, then L (lower)
  __shared__ double Ys[64][CB_LD];  // Y = L^{-1} (lower)
  __shared__ double red[4];
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const double* src = Wparts + (int64_t)b * nparts * p * p;
  // ---- sum of the partial Grams, padded with the identity; the 16 entries of a thread
  // are loaded together for each partial (independent loads in flight)
  {
    double v[16];
    int off[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + 256 * e, i = idx >> 6, j = idx & 63;
      const bool in = i < p && j < p;
      off[e] = in ? i * p + j : 0;
      v[e] = 0.0;
    }
    for (int q = 0; q < nparts; ++q) {
      const double* sp = src + (int64_t)q * p * p;
      double t[16];
#pragma unroll
      for (int e = 0; e < 16; ++e) t[e] = sp[off[e]];
#pragma unroll
      for (int e = 0; e < 16; ++e) v[e] += t[e];
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const int idx = tid + 256 * e, i = idx >> 6, j = idx & 63;
      W[i][j] = (i < p && j < p) ? v[e] : (i == j ? 1.0 : 0.0);
    }
  }
  __syncthreads();
  if (wave == 0) {
    const double dg = lane < p ? W[lane][lane] : 0.0;
    const double tr = wave_sum_f64(dg);
    if (lane == 0) red[0] = tr;
  }
  __syncthreads();
  const double shift = rel_shift * red[0];
  const double floor_ = fmax(0.5 * shift, 1e-300);  // below the shift: rounding only
  if (tid < p) W[tid][tid] += shift;
  __syncthreads();

  // ---- L L^T = W by 16-column panels
  const int li = lane & 15, lk = lane >> 4;
  for (int K = 0; K < 4; ++K) {
    const int r0 = 16 * K;
    if (wave == 0) {
      const int r = r0 + lane;
      const bool rin = r < 64;
      double pr[16];
#pragma unroll
      for (int c = 0; c < 16; ++c) pr[c] = rin ? W[r][r0 + c] : 0.0;
#pragma unroll
      for (int c = 0; c < 16; ++c) {
        double piv = cb_readlane(pr[c], c);
        if (!(piv > floor_)) piv = floor_;
        double sq, is;
        sqrt_and_inv(piv, sq, is);
        pr[c] = lane == c ? sq : pr[c] * is;  // rows below: L(r, r0 + c)
#pragma unroll
        for (int c2 = c + 1; c2 < 16; ++c2) pr[c2] = fma(-pr[c], cb_readlane(pr[c], c2), pr[c2]);
      }
      if (rin) {
#pragma unroll
        for (int c = 0; c < 16; ++c) W[r][r0 + c] = lane >= c ? pr[c] : 0.0;
      }
    }
    __syncthreads();
    // trailing tiles (I, J), K < J <= I < 4: W_IJ -= L_IK L_JK^T
    const int nt = (3 - K) * (4 - K) / 2;
    for (int t = wave; t < nt; t += 4) {
      int I = K + 1, J = K + 1, u = t;
      while (u > I - K - 1) {  // tiles in row-major order of the lower triangle
        u -= I - K;
        ++I;
      }
      J = K + 1 + u;
      cb_d4 acc;
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[e] = W[16 * I + 4 * e + lk][16 * J + li];
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const double a = -W[16 * I + li][r0 + 4 * s4 + lk];
        const double bb = W[16 * J + li][r0 + 4 * s4 + lk];
        acc = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, acc, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) W[16 * I + 4 * e + lk][16 * J + li] = acc[e];
    }
    __syncthreads();
  }

  // ---- Y = L^{-1}: diagonal blocks, lane (block I = lane >> 4, column j = lane & 15)
  if (wave == 0) {
    const int I = lane >> 4, j = lane & 15, o = 16 * I;
    double y[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      double sum = i == j ? 1.0 : 0.0;
#pragma unroll
      for (int k = 0; k < i; ++k) sum = fma(-W[o + i][o + k], y[k], sum);
      y[i] = i < j ? 0.0 : sum * recip(W[o + i][o + i]);
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) Ys[o + i][o + j] = y[i];
  }
  __syncthreads();
  // blocks below the diagonal by levels d = I - J (each reads Y blocks of lower levels)
  for (int d = 1; d < 4; ++d) {
    const int I = wave + d, J = wave;
    cb_d4 Tt = {0.0, 0.0, 0.0, 0.0}, Yt = {0.0, 0.0, 0.0, 0.0};
    if (I < 4) {
      // T = sum_{K = J}^{I-1} L_IK Y_KJ
      for (int K = J; K < I; ++K) {
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const double a = W[16 * I + li][16 * K + 4 * s4 + lk];
          const double bb = Ys[16 * K + 4 * s4 + lk][16 * J + li];
          Tt = __builtin_amdgcn_mfma_f64_16x16x4f64(a, bb, Tt, 0, 0, 0);
        }
      }
      // Y_IJ = -Y_II T: register s4 of T holds rows 4 s4 .. 4 s4 + 3, lane 16 k + j: the B
      // operand of k step s4
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const double a = -Ys[16 * I + li][16 * I + 4 * s4 + lk];
        Yt = __builtin_amdgcn_mfma_f64_16x16x4f64(a, Tt[s4], Yt, 0, 0, 0);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) Ys[16 * I + 4 * e + lk][16 * J + li] = Yt[e];
    }
    __syncthreads();
  }
  // ---- R^{-1} = Y^T (upper): entry (k, c) = Y(c, k)
  for (int idx = tid; idx < p * p; idx += 256) {
    const int k = idx / p, c = idx - k * p;
    const double v = k <= c ? Ys[c][k] : 0.0;
    const int64_t o = (int64_t)b * p * p + idx;
    if (f64out) ((double*)Rinv)[o] = v;
    else ((float*)Rinv)[o] = (float)v;
  }
}

// dst = src R^{-1} for `rpb` rows of one fp32 [rows][p] block per workgroup
// (grid (ceil(rows / rpb), batch)), R^{-1} (fp32 [p][p] per batch) written by
// k_chol_inv_blk: the rows are multiplied with the fp16 hi/lo split MFMA (hi*hi + hi*lo +
// lo*hi, fp32 accumulation), the same arithmetic as the split GEMM.
__global__ __launch_bounds__(256) void k_chol_apply(int p, const float* Rinv, const float* src, float* dst,
                                                    int64_t rows, int rpb) {
  __shared__ __align__(16) uint16_t Bh[64][72];  // R^{-1} transposed: [column][k], fp16 hi / lo
  __shared__ __align__(16) uint16_t Bl[64][72];
  const int b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int r0 = 4 * (tid >> 4), c0 = 4 * (tid & 15);
  double xf[4][4];
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      xf[u][v] = (r0 + u < p && c0 + v < p) ? (double)Rinv[(int64_t)b * p * p + (r0 + u) * p + c0 + v] : 0.0;
  // R^{-1} is applied as (2^-e R^{-1}) with the largest entry below 1, so its fp16 hi/lo
  // split stays in range whatever the scale and conditioning of the block; the result is
  // multiplied back by 2^e (exact)
  __shared__ double wmax[4];
  double mloc = 0.0;
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (r0 + u < p && c0 + v < p) mloc = fmax(mloc, fabs(xf[u][v]));
  for (int o = 32; o > 0; o >>= 1) mloc = fmax(mloc, __shfl_xor(mloc, o, 64));
  if (lane == 0) wmax[wave] = mloc;
  __syncthreads();
  const double rmax = fmax(fmax(wmax[0], wmax[1]), fmax(wmax[2], wmax[3]));
  int ex = 0;
  if (rmax > 0.0) (void)frexp(rmax, &ex);  // rmax = f 2^ex, f in [0.5, 1)
  const double down = ldexp(1.0, -ex);
  const float up = (float)ldexp(1.0, ex);
#pragma unroll
  for (int u = 0; u < 4; ++u)
#pragma unroll
    for (int v = 0; v < 4; ++v) {  // entry (k = r0 + u, column c0 + v); zero outside p
      const float x = (r0 + u < p && c0 + v < p) ? (float)(xf[u][v] * down) : 0.f;
      const _Float16 h = (_Float16)x;
      Bh[c0 + v][r0 + u] = __builtin_bit_cast(uint16_t, h);
      Bl[c0 + v][r0 + u] = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)h));
    }
  __syncthreads();
  const int kt = (p + 15) / 16;  // 16-wide k slices and column tiles
  const float* S = src + (int64_t)b * rows * p;
  float* Q = dst + (int64_t)b * rows * p;
  const int64_t rbeg = (int64_t)blockIdx.x * rpb;
  const int64_t rend = rbeg + rpb < rows ? rbeg + rpb : rows;
  const int fr = lane & 15, fk = 4 * (lane >> 4);
  for (int64_t rt = rbeg + 16 * wave; rt < rend; rt += 64) {
    // A fragments: row rt + fr, k = 16 s + fk .. + 3 (zero beyond p or the last row)
    half4_t ah[4], al[4];
    const int64_t row = rt + fr;
#pragma unroll
    for (int sl = 0; sl < 4; ++sl) {
      float v4[4] = {0.f, 0.f, 0.f, 0.f};
      const int k = 16 * sl + fk;
      if (sl < kt && row < rend && k < p) {
        const float4 q = *(const float4*)(S + row * p + k);  // p is a multiple of 4
        v4[0] = q.x; v4[1] = q.y; v4[2] = q.z; v4[3] = q.w;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const _Float16 h = (_Float16)v4[e];
        ah[sl][e] = h;
        al[sl][e] = (_Float16)(v4[e] - (float)h);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      if (ct >= kt) break;
      float4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int sl = 0; sl < 4; ++sl) {
        if (sl >= kt) break;
        const half4_t bh = *(const half4_t*)&Bh[16 * ct + fr][16 * sl + fk];
        const half4_t bl = *(const half4_t*)&Bl[16 * ct + fr][16 * sl + fk];
        acc = mfma16(ah[sl], bh, acc);
        acc = mfma16(ah[sl], bl, acc);
        acc = mfma16(al[sl], bh, acc);
      }
      const int col = 16 * ct + fr;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int64_t orow = rt + fk + e;
        if (orow < rend && col < p) Q[orow * p + col] = acc[e] * up;
      }
    }
  }
  __syncthreads();
}

hipError_t launch_chol_apply(const double* Wparts, int nparts, int p, const float* src, float* dst, int64_t rows,
                             int batch, float* Rinv, hipStream_t s) {
  if (p > 64 || p < 4 || (p & 3) || rows < 1 || batch < 1 || batch > 65535 || !Rinv) return hipErrorInvalidValue;
  const int rpb = 128;
  const int64_t nblk = (rows + rpb - 1) / rpb;
  if (nblk > 65535) return hipErrorInvalidValue;
  // factor once per matrix, then apply
  hipLaunchKernelGGL(k_chol_inv_blk, dim3(batch), dim3(256), 0, s, Wparts, nparts, p, kOrthShift, (void*)Rinv, 0);
  hipLaunchKernelGGL(k_chol_apply, dim3((unsigned)nblk, batch), dim3(256), 0, s, p, (const float*)Rinv, src, dst,
                     rows, rpb);
  return hipGetLastError();
}

hipError_t launch_chol_inv(const double* Wparts, int nparts, int p, int batch, void* Rinv, bool f64out,
                           hipStream_t s) {
  if (p > 64 || p < 4 || (p & 3) || batch < 1 || batch > 65535) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_chol_inv_blk, dim3(batch), dim3(256), 0, s, Wparts, nparts, p, kOrthShift, Rinv,
                     f64out ? 1 : 0);
  return hipGetLastError();
}

// ============================================================ Gram reduction
// With `upper` the partials hold the 16 x 16 tiles on and above the diagonal only: the
// sum of entry (m, n) of such a tile is stored at (m, n) and, off the diagonal tiles, at (n, m).
__global__ void k_reduce_gram(const double* parts, int nparts, int D, int upper, double* G) {
  const int t = blockIdx.y;
  const int DD = D * D;
  const int idx = blockIdx.x * 256 + threadIdx.x;
  if (idx >= DD) return;
  const int m = idx / D, n = idx % D;
  if (upper && (m >> 4) > (n >> 4)) return;
  const double* src = parts + (int64_t)t * nparts * DD + idx;
  double s = 0.0;
  for (int q = 0; q < nparts; ++q) s += src[(int64_t)q * DD];
  G[(int64_t)t * DD + idx] = s;
  if (upper && (m >> 4) != (n >> 4)) G[(int64_t)t * DD + (int64_t)n * D + m] = s;
}
__global__ __launch_bounds__(128) void k_trace(const double* G, int D, double* xn2, int32_t* flags) {
  const int t = blockIdx.x;
  __shared__ double red[128];
  const int i = threadIdx.x;
  red[i] = i < D ? G[(int64_t)t * D * D + (int64_t)i * D + i] : 0.0;
  __syncthreads();
  for (int o = 64; o > 0; o >>= 1) {
    if (i < o) red[i] += red[i + o];
    __syncthreads();
  }
  if (i == 0) {
    xn2[t] = red[0];
    if (!isfinite(red[0])) atomicOr(flags, 2);
  }
}

hipError_t launch_reduce_gram(const double* parts, int nparts, int D, int ntab, double* G, double* xn2,
                              int32_t* flags, hipStream_t s, bool upper_tiles) {
  const int DD = D * D;
  if (upper_tiles && (D & 15)) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_reduce_gram, dim3((DD + 255) / 256, ntab), dim3(256), 0, s, parts, nparts, D,
                     upper_tiles ? 1 : 0, G);
  if (D > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_trace, dim3(ntab), dim3(128), 0, s, G, D, xn2, flags);
  return hipGetLastError();
}

// ============================================================ feature factor preparation

// One block per table.  V[:, j] = Q fp16(U_d[:, j]) = H (sigma . u) / sqrt(D) by a fast
// Walsh-Hadamard transform of each column in LDS (fp64).
__global__ __launch_bounds__(256) void k_prep_feature(const double* Ud64, const int8_t* signs, int D, float* Ud32,
                                                      _Float16* Ud16, float* V32, _Float16* Vh, _Float16* Vl) {
  const int t = blockIdx.x;
  __shared__ double v[128][JOLT_KMAX + 1];
  const int64_t base = (int64_t)t * D * JOLT_KMAX;
  for (int idx = threadIdx.x; idx < D * JOLT_KMAX; idx += 256) {
    const int f = idx / JOLT_KMAX, j = idx % JOLT_KMAX;
    const double u = Ud64[base + idx];
    const _Float16 h = f64_to_f16(u);
    Ud32[base + idx] = (float)u;
    Ud16[base + idx] = h;
    v[f][j] = signs[t * D + f] < 0 ? -(double)h : (double)h;
  }
  __syncthreads();
  for (int st = 1; st < D; st <<= 1) {
    for (int idx = threadIdx.x; idx < (D / 2) * JOLT_KMAX; idx += 256) {
      const int pr = idx / JOLT_KMAX, j = idx % JOLT_KMAX;
      const int i0 = ((pr / st) * 2 * st) + (pr % st), i1 = i0 + st;
      const double a = v[i0][j], b = v[i1][j];
      v[i0][j] = a + b;
      v[i1][j] = a - b;
    }
    __syncthreads();
  }
  const double isq = 1.0 / sqrt((double)D);
  for (int idx = threadIdx.x; idx < D * JOLT_KMAX; idx += 256) {
    const int f = idx / JOLT_KMAX, j = idx % JOLT_KMAX;
    const float val = (float)(v[f][j] * isq);
    V32[base + idx] = val;
    const float nv = -val;
    const _Float16 h = (_Float16)nv;
    Vh[base + idx] = h;
    Vl[base + idx] = (_Float16)(nv - (float)h);
  }
}

hipError_t launch_prep_feature(const double* Ud64, const int8_t* signs, int D, int ntab, float* Ud32,
                               _Float16* Ud16, float* V32, _Float16* Vneg_hi, _Float16* Vneg_lo, hipStream_t s) {
  if (D > 128) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_prep_feature, dim3(ntab), dim3(256), 0, s, Ud64, signs, D, Ud32, Ud16, V32, Vneg_hi,
                     Vneg_lo);
  return hipGetLastError();
}

// ============================================================ token-major copy of Y
// YT[t][tk][j * N + n] = Y[t][n][tk][j] (fp32): rows of the token unfolding with the
// feature index outermost, so that the columns of features j < r_d form a prefix.
// One block per (token, table); N <= 256.
__global__ __launch_bounds__(256) void k_transpose_y(const float* Y, int N, int T, float* YT) {
  const int tk = blockIdx.x, t = blockIdx.y;
  __shared__ float s[256][JOLT_KMAX + 1];
  const float* src = Y + (int64_t)t * N * T * JOLT_KMAX + (int64_t)tk * JOLT_KMAX;
  for (int idx = threadIdx.x; idx < N * JOLT_KMAX; idx += 256) {
    const int n = idx / JOLT_KMAX, j = idx % JOLT_KMAX;
    s[n][j] = src[(int64_t)n * T * JOLT_KMAX + j];
  }
  __syncthreads();
  float* dst = YT + ((int64_t)t * T + tk) * JOLT_KMAX * N;
  for (int idx = threadIdx.x; idx < N * JOLT_KMAX; idx += 256) {
    const int j = idx / N, n = idx % N;
    dst[idx] = s[n][j];
  }
}

hipError_t launch_transpose_y(const float* Y, int N, int T, int ntab, float* YT, hipStream_t s) {
  if (N > 256) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_transpose_y, dim3(T, ntab), dim3(256), 0, s, Y, N, T, YT);
  return hipGetLastError();
}

// ============================================================ token-contiguous copies
// dst[b][c][t] = src[b][t][c] for every slice b = table * N + n of T rows of C values
// (C a multiple of 8): the transposed operands of the randomized range finder then run
// along contiguous rows.  Source: the bf16 tables (tp) or one contiguous buffer; 64 rows x
// 32 values per block through LDS.
template <typename E>
__global__ __launch_bounds__(256) void k_transpose_tc(const TablePtrs tp, const E* __restrict__ src, int N,
                                                      int T, int C, E* __restrict__ dst) {
  const int t0 = blockIdx.x * 64, c0 = blockIdx.y * 32, b = blockIdx.z;
  __shared__ E tile[32][65];
  const E* sb = src ? src + (int64_t)b * T * C : (const E*)tp.p[b / N] + (int64_t)(b % N) * T * C;
  const int cn = min(32, C - c0), rn = min(64, T - t0);  // this block's columns and rows
  for (int idx = threadIdx.x; idx < 64 * 32; idx += 256) {
    const int r = idx >> 5, c = idx & 31;
    if (c < cn && r < rn) tile[c][r] = sb[(int64_t)(t0 + r) * C + c0 + c];
  }
  __syncthreads();
  E* db = dst + (int64_t)b * T * C;
  for (int idx = threadIdx.x; idx < 64 * 32; idx += 256) {
    const int c = idx >> 6, r = idx & 63;
    if (c < cn && r < rn) db[(int64_t)(c0 + c) * T + t0 + r] = tile[c][r];
  }
}

hipError_t launch_transpose_tc(const TablePtrs* tp, const void* src, bool bf16, int N, int T, int C, int ntab,
                               void* dst, hipStream_t s) {
  if (T < 1 || C % 8 || C < 8 || N < 1 || ntab < 1 || (int64_t)N * ntab > 65535 || (T + 63) / 64 > 65535 ||
      (!tp && !src))
    return hipErrorInvalidValue;
  TablePtrs none{};
  const dim3 grid((T + 63) / 64, (C + 31) / 32, N * ntab);
  if (bf16)
    hipLaunchKernelGGL(k_transpose_tc<uint16_t>, grid, dim3(256), 0, s, tp ? *tp : none, (const uint16_t*)src, N,
                       T, C, (uint16_t*)dst);
  else
    hipLaunchKernelGGL(k_transpose_tc<float>, grid, dim3(256), 0, s, tp ? *tp : none, (const float*)src, N, T, C,
                       (float*)dst);
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

// ============================================================ Ritz residuals
// Convergence test of the exact token subspace iteration.  Problem b holds the orthonormal
// basis Z_b [T][p], the product P_b = M_b Z_b [T][p] (working precision), the eigenvectors
// V_b [p][32] of H_b = Z_b^T P_b (working precision) and their eigenvalues theta_b [32]
// (fp64, descending).  The Ritz pair i is (theta_i, u_i = Z_b v_i), and its residual is
// M u_i - theta_i u_i = (P_b - theta_i Z_b) v_i.  res[b] = max_i ||residual_i|| / theta_0
// over the 32 pairs, in fp64 (0 when theta_0 <= 0).  One workgroup per problem; thread
// tid takes rows tid, tid + 256, ...; column sums of squares reduced in a fixed order.
template <typename W>
__global__ __launch_bounds__(256) void k_ritz_residual(const W* P, const W* Z, const W* V, const double* lam,
                                                       int T, int p, double* res) {
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
  __shared__ double Vs[JOLT_PSUB][JOLT_KMAX];
  __shared__ double th[JOLT_KMAX];
  __shared__ double part[4][JOLT_KMAX];
  const W* Pb = P + (int64_t)b * T * p;
  const W* Zb = Z + (int64_t)b * T * p;
  const W* Vb = V + (int64_t)b * p * JOLT_KMAX;
  for (int e = tid; e < p * JOLT_KMAX; e += 256) Vs[e / JOLT_KMAX][e % JOLT_KMAX] = (double)Vb[e];
  if (tid < JOLT_KMAX) th[tid] = lam[(int64_t)b * JOLT_KMAX + tid];
  __syncthreads();
  double ss[JOLT_KMAX];
#pragma unroll
  for (int i = 0; i < JOLT_KMAX; ++i) ss[i] = 0.0;
  for (int t = tid; t < T; t += 256) {
    double r[JOLT_KMAX];
#pragma unroll
    for (int i = 0; i < JOLT_KMAX; ++i) r[i] = 0.0;
    for (int k = 0; k < p; ++k) {
      const double pk = (double)Pb[(int64_t)t * p + k], zk = (double)Zb[(int64_t)t * p + k];
#pragma unroll
      for (int i = 0; i < JOLT_KMAX; ++i) r[i] = fma(fma(-th[i], zk, pk), Vs[k][i], r[i]);
    }
#pragma unroll
    for (int i = 0; i < JOLT_KMAX; ++i) ss[i] = fma(r[i], r[i], ss[i]);
  }
#pragma unroll
  for (int i = 0; i < JOLT_KMAX; ++i) {
    double v = ss[i];
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    if (lane == 0) part[wv][i] = v;
  }
  __syncthreads();
  if (tid == 0) {
    double m = 0.0;
    for (int i = 0; i < JOLT_KMAX; ++i) {
      const double v = ((part[0][i] + part[1][i]) + part[2][i]) + part[3][i];
      m = fmax(m, sqrt(v));
    }
    res[b] = th[0] > 0.0 ? m / th[0] : 0.0;
  }
}

// The same residuals for fp32 P, Z, V with p = 64, by fp64 MFMA: workgroup (64-row chunk q,
// problem b), wave w the 16 rows 64 q + 16 w ..; PV and ZV tiles (16 rows x 32 columns) by
// v_mfma_f64_16x16x4f64 over k in steps of 4 (lane (i, g) supplies P[row i][16 kc + 4 g + t]
// in step 4 kc + t, from one float4 load), R = PV - theta ZV per column, and the column sums
// of R^2 of the chunk to part[(b nchunk + q) 32 + i] (waves added in order);
// k_ritz_final then adds the chunks in order and takes max_i sqrt(.) / theta_0.
__global__ __launch_bounds__(256) void k_ritz_mfma(const float* __restrict__ P, const float* __restrict__ Z,
                                                   const float* __restrict__ V, const double* __restrict__ lam,
                                                   int T, double* __restrict__ part) {
  constexpr int p = 64, KM = JOLT_KMAX;
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x, lane = tid & 63, w = tid >> 6;
  const int li = lane & 15, g = lane >> 4;
  __shared__ float vs[p][KM];
  __shared__ double th[KM];
  __shared__ double red[4][KM];
  for (int idx = tid; idx < p * KM; idx += 256) (&vs[0][0])[idx] = V[(int64_t)b * p * KM + idx];
  if (tid < KM) th[tid] = lam[(int64_t)b * KM + tid];
  __syncthreads();
  const int64_t row = (int64_t)q * 64 + 16 * w + li;
  const float4* pr = (const float4*)(P + ((int64_t)b * T + row) * p);
  const float4* zr = (const float4*)(Z + ((int64_t)b * T + row) * p);
  gram_d4 pv[2], zv[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    pv[ct] = (gram_d4){0.0, 0.0, 0.0, 0.0};
    zv[ct] = (gram_d4){0.0, 0.0, 0.0, 0.0};
  }
#pragma unroll
  for (int kc = 0; kc < p / 16; ++kc) {
    const float4 a4 = pr[4 * kc + g], z4 = zr[4 * kc + g];  // k = 16 kc + 4 g .. + 3
    const float av[4] = {a4.x, a4.y, a4.z, a4.w}, zz[4] = {z4.x, z4.y, z4.z, z4.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int k = 16 * kc + 4 * g + t;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const double bv = (double)vs[k][16 * ct + li];
        pv[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)av[t], bv, pv[ct], 0, 0, 0);
        zv[ct] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)zz[t], bv, zv[ct], 0, 0, 0);
      }
    }
  }
  // element (row 4 r + g, column 16 ct + li) in register r
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const double tc = th[16 * ct + li];
    double ssum = 0.0;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const double rr = fma(-tc, zv[ct][r], pv[ct][r]);
      ssum = fma(rr, rr, ssum);
    }
    ssum += __shfl_xor(ssum, 16, 64);
    ssum += __shfl_xor(ssum, 32, 64);
    if (g == 0) red[w][16 * ct + li] = ssum;
  }
  __syncthreads();
  if (tid < KM)
    part[((int64_t)b * gridDim.x + q) * KM + tid] = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
}

__global__ __launch_bounds__(64) void k_ritz_final(const double* __restrict__ part, int nchunk,
                                                   const double* __restrict__ lam, double* __restrict__ res) {
  const int b = blockIdx.x, i = threadIdx.x;
  double v = 0.0;
  if (i < JOLT_KMAX)
    for (int q = 0; q < nchunk; ++q) v += part[((int64_t)b * nchunk + q) * JOLT_KMAX + i];
  double m = i < JOLT_KMAX ? sqrt(v) : 0.0;
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  if (i == 0) {
    const double t0 = lam[(int64_t)b * JOLT_KMAX];
    res[b] = t0 > 0.0 ? m / t0 : 0.0;
  }
}

hipError_t launch_ritz_residual(const void* P, const void* Z, const void* V, bool f64, const double* lam, int T,
                                int p, int batch, double* res, double* part, hipStream_t s) {
  if (p > JOLT_PSUB || batch <= 0) return hipErrorInvalidValue;
  if (!f64 && p == 64 && T % 64 == 0 && part) {
    hipLaunchKernelGGL(k_ritz_mfma, dim3(T / 64, batch), dim3(256), 0, s, (const float*)P, (const float*)Z,
                       (const float*)V, lam, T, part);
    hipLaunchKernelGGL(k_ritz_final, dim3(batch), dim3(64), 0, s, part, T / 64, lam, res);
    return hipGetLastError();
  }
  if (f64)
    hipLaunchKernelGGL(k_ritz_residual<double>, dim3(batch), dim3(256), 0, s, (const double*)P, (const double*)Z,
                       (const double*)V, lam, T, p, res);
  else
    hipLaunchKernelGGL(k_ritz_residual<float>, dim3(batch), dim3(256), 0, s, (const float*)P, (const float*)Z,
                       (const float*)V, lam, T, p, res);
  return hipGetLastError();
}

// ============================================================ Gaussian calibration of eps^2(b)
// One wave per row g of length D (one quantization block): part[row] = (sum g^2, and for
// b = 2, 4, 8 the error sum (g - s q)^2 with s = fp32(max|g| / (2^(b-1) - 1)) and
// q = clip(rint(g / s)) decided in fp64, as the encoder does).  Sums in fixed order.
__global__ __launch_bounds__(256) void k_eps2(const float* G, int rows, int D, double* part) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (row >= rows) return;  // uniform per wave
  const float* g = G + row * D;
  double m = 0.0, e0 = 0.0;
  for (int f = lane; f < D; f += 64) {
    const double v = (double)g[f];
    m = fmax(m, fabs(v));
    e0 = fma(v, v, e0);
  }
  for (int o = 32; o > 0; o >>= 1) m = fmax(m, __shfl_xor(m, o, 64));
  double e[3];
#pragma unroll
  for (int bi = 0; bi < 3; ++bi) {
    const int b = 2 << bi;
    const int qmax = (1 << (b - 1)) - 1;
    const double sc = (double)(float)(m / qmax);
    double acc = 0.0;
    for (int f = lane; f < D; f += 64) {
      const double v = (double)g[f];
      double q = sc > 0.0 ? rint(v / sc) : 0.0;
      q = fmin(fmax(q, (double)(-qmax - 1)), (double)qmax);
      const double r = v - sc * q;
      acc = fma(r, r, acc);
    }
    e[bi] = acc;
  }
  const double s0 = wave_sum_f64(e0), s2 = wave_sum_f64(e[0]), s4 = wave_sum_f64(e[1]), s8 = wave_sum_f64(e[2]);
  if (lane == 0) {
    part[row * 4 + 0] = s0;
    part[row * 4 + 1] = s2;
    part[row * 4 + 2] = s4;
    part[row * 4 + 3] = s8;
  }
}

hipError_t launch_eps2(const float* G, int rows, int D, double* part, hipStream_t s) {
  if (rows < 1 || D < 1 || D > 4096) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_eps2, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, s, G, rows, D, part);
  return hipGetLastError();
}

// ============================================================ rotated reconstruction operands
// (the operands and their layout: w_operands.h) one workgroup per (slice, chain, table)
__global__ __launch_bounds__(256) void k_prep_w(const _Float16* G16, const float* V32, const int8_t* signs, int N,
                                                int D, _Float16* Wh, _Float16* Wl, int32_t* flags) {
  const int n = blockIdx.x, c = blockIdx.y, t = blockIdx.z;
  __shared__ double g[JOLT_KMAX][129];  // core rows (r_d chains), or their transform (chain 4)
  __shared__ __align__(16) float vs[128][PW_VS];
  const int64_t gbase = (((int64_t)t * 5 + c) * N + n) * JOLT_KMAX * D;
  const int lD = 31 - __clz(D);  // D, r_d and the butterfly strides are powers of two
  const int lrd = c < 4 ? 2 + c : lD, rd = 1 << lrd;
  for (int idx = threadIdx.x; idx < JOLT_KMAX * rd; idx += 256) {
    const int kk = idx >> lrd, j = idx & (rd - 1);
    double v = (double)G16[gbase + (int64_t)kk * D + j];
    if (c == 4 && signs[t * D + j] < 0) v = -v;
    g[kk][j] = v;
  }
  if (c < 4)
    for (int idx = threadIdx.x; idx < D * JOLT_KMAX; idx += 256)
      vs[idx / JOLT_KMAX][idx % JOLT_KMAX] = V32[(int64_t)t * D * JOLT_KMAX + idx];
  __syncthreads();
  int overflow = 0;
  const int64_t obase = gbase;  // [t][c][n] block of D*32 values
  switch (c) {
    case 0: prep_w_rows<4>(&g[0][0], 129, &vs[0][0], D, obase, Wh, Wl, overflow); break;
    case 1: prep_w_rows<8>(&g[0][0], 129, &vs[0][0], D, obase, Wh, Wl, overflow); break;
    case 2: prep_w_rows<16>(&g[0][0], 129, &vs[0][0], D, obase, Wh, Wl, overflow); break;
    case 3: prep_w_rows<32>(&g[0][0], 129, &vs[0][0], D, obase, Wh, Wl, overflow); break;
    default: prep_w_hadamard(&g[0][0], 129, lD, obase, Wh, Wl, overflow); break;
  }
  if (overflow) atomicOr(flags, 1);
}

hipError_t launch_prep_w(const _Float16* G16, const float* V32, const int8_t* signs, int N, int D, int ntab,
                         _Float16* Wneg_hi, _Float16* Wneg_lo, int32_t* flags, hipStream_t s) {
  if (D != 64 && D != 128) return hipErrorInvalidValue;  // the kernel's index arithmetic takes powers of two
  hipLaunchKernelGGL(k_prep_w, dim3(N, 5, ntab), dim3(256), 0, s, G16, V32, signs, N, D, Wneg_hi, Wneg_lo, flags);
  return hipGetLastError();
}

}  // namespace jolt
