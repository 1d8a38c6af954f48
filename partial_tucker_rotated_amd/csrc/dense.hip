// Small dense kernels of the factor stage: the symmetric top-k eigensolver used for
// the feature Gram, the small token Grams and the Rayleigh-Ritz matrices; the
// Cholesky inverse of CholeskyQR; Gram reduction; feature-factor preparation.
#include "jolt_internal.h"
#include "w_operands.h"

namespace jolt {

// ============================================================ symmetric top-k eigensolver
// One workgroup of 512 threads per matrix (n <= 128, the k <= 32 largest eigenpairs):
// - Householder tridiagonalisation in fp64 with the matrix in registers: a row is held by
//   NP consecutive lanes (CP columns each), so the matrix-vector product needs only a
//   reduction across those lanes; each step has two barriers (v published; p and the p^T v
//   partials published), and waves whose rows are all reduced only take part in them.
// - fp32 multisection bisection with Sturm counts, each eigenvalue's 16 samples in 16
//   lanes of one wave, the interval narrowed from a ballot (no barrier);
// - fp64 inverse iteration on T - lambda I (LDL^T factored once, three solves), all k
//   vectors at once, one lane each; modified Gram-Schmidt inside clusters of nearly equal
//   eigenvalues (only where the bisection finds any);
// - back-transformation by the Householder vectors (kept packed in LDS), 16 lanes per
//   eigenvector; sign normalisation (largest-magnitude entry positive) in registers.
#define SY_N 128
#define SY_K 32
#define SY_S 16      // bisection samples per eigenvalue and round
#define SY_ROUNDS 6  // 17^6 ~ 2.4e7: fp32 resolution of the spectrum
#define SY_THREADS 512

// 1 / x: hardware reciprocal refined by one Newton step y <- y (2 - x y) (a few ulp)
__device__ __forceinline__ double recip(double x) {
  const double y = __builtin_amdgcn_rcp(x);
  return fma(y, fma(-x, y, 1.0), y);
}

// packed Householder vectors: reflector q keeps its entries q + 2 .. n - 1 (entry q + 1 is 1)
__device__ __forceinline__ int sy_voff(int q, int n) { return q * (n - 2) - (q * (q - 1)) / 2; }

// sum over groups of NP (4 or 8) consecutive lanes, returned to every lane of the group
template <int NP>
__device__ __forceinline__ double sy_group_sum(double v) {
  v += dpp_f64<0xB1>(v);
  v += dpp_f64<0x4E>(v);
  if (NP == 8) v += dpp_f64<0x141>(v);
  return v;
}

template <typename TIn, int NR>
__global__ __launch_bounds__(SY_THREADS) void k_syev_topk(const TIn* Aall, int n, int k, double* U64, float* U32,
                                                          _Float16* U16, double* lam_out) {
  constexpr int NP = SY_THREADS / NR;  // lanes per row: 4 (NR = 128) or 8 (NR = 64)
  constexpr int CP = NR / NP;          // columns per lane
  constexpr int RPW = 64 / NP;         // rows per wave
  constexpr int VST = CP + 2;          // padded stride of a lane's columns in the broadcast vectors
  constexpr int YLD = NR + 1;          // row stride of the eigenvector and pivot arrays
  constexpr int NU = NR / 16;          // entries per lane in the back-transformation
  // Householder vectors: whole rows (NR = 64) or packed below the subdiagonal (NR = 128)
  __shared__ double VR[NR == 64 ? (NR - 2) * NR : (NR - 2) * (NR - 1) / 2];
  __shared__ double Y[SY_K * YLD], iDs[SY_K * YLD];
  __shared__ double vb[NP * VST], pb[NP * VST], rb[NP * VST];
  __shared__ double d[NR], e[NR], es[NR], tau[NR];
  __shared__ double pvw[8], taus[2], gred[2][3], ysc[SY_K];
  __shared__ float df[NR], e2s[NR], lamf[SY_K];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int row = tid / NP, part = tid % NP;
  const int b = blockIdx.x;
  const TIn* Ain = Aall + (int64_t)b * n * n;
  double a[CP];
#pragma unroll
  for (int u = 0; u < CP; ++u) {
    const int j = part * CP + u;
    a[u] = (row < n && j < n) ? (double)Ain[row * n + j] : 0.0;
  }

  // ---- tridiagonalisation: A = Q T Q^T, Q = H_0 ... H_{n-3}, H_q = I - tau_q v_q v_q^T
  for (int kk = 0; kk < n - 2; ++kk) {
    if (wave == (kk * NP) >> 6) {  // the wave holding row kk (= column kk) builds v
      if (row == kk) {  // the row goes through LDS; lane l then takes columns l and l + 64
#pragma unroll
        for (int u = 0; u < CP; ++u) rb[part * VST + u] = a[u];
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      const int j0 = lane, j1 = lane + 64;
      const double r0 = rb[(j0 / CP) * VST + j0 % CP];
      const double r1 = NR > 64 ? rb[(j1 / CP) * VST + j1 % CP] : 0.0;
      const double x0 = rb[((kk + 1) / CP) * VST + (kk + 1) % CP], dkk = rb[(kk / CP) * VST + kk % CP];
      const double s = wave_sum_f64((j0 >= kk + 2 ? r0 * r0 : 0.0) + (j1 >= kk + 2 ? r1 * r1 : 0.0));
      double t = 0.0, sc = 0.0, beta = x0;
      if (s != 0.0) {
        const double nx = sqrt(x0 * x0 + s);
        beta = x0 >= 0.0 ? -nx : nx;
        t = (beta - x0) * recip(beta);
        sc = recip(x0 - beta);
      }
      const double v0 = j0 == kk + 1 ? 1.0 : (j0 >= kk + 2 ? r0 * sc : 0.0);
      const double v1 = j1 == kk + 1 ? 1.0 : (j1 >= kk + 2 ? r1 * sc : 0.0);
      vb[(j0 / CP) * VST + j0 % CP] = v0;
      if constexpr (NR == 64) {
        VR[kk * NR + j0] = v0;
      } else {
        const int vo = sy_voff(kk, n) - kk - 2;
        vb[(j1 / CP) * VST + j1 % CP] = v1;
        if (j0 >= kk + 2 && j0 < n) VR[vo + j0] = v0;
        if (j1 >= kk + 2 && j1 < n) VR[vo + j1] = v1;
      }
      if (lane == 0) {
        d[kk] = dkk;
        e[kk] = beta;
        tau[kk] = t;
        taus[kk & 1] = t;
      }
    }
    __syncthreads();  // v and tau of this step are published
    // rows 0 .. kk are final; a wave takes part while it holds a row kk + 1 .. n - 1
    const bool act = (wave + 1) * RPW - 1 > kk && wave * RPW < n;
    double vp[CP], vi = 0.0, pi = 0.0;
    const double t = taus[kk & 1];
    if (act) {
#pragma unroll
      for (int u = 0; u < CP; ++u) vp[u] = vb[part * VST + u];
      vi = vb[(row / CP) * VST + row % CP];
    }
    if (t == 0.0) continue;  // uniform: the column is already reduced
    if (act) {
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int u = 0; u < CP; u += 2) {
        s0 = fma(a[u], vp[u], s0);
        s1 = fma(a[u + 1], vp[u + 1], s1);
      }
      const double av = sy_group_sum<NP>(s0 + s1);
      pi = (row > kk && row < n) ? t * av : 0.0;  // p = tau A v on the trailing rows
      const double pv = wave_sum_f64(part == 0 ? pi * vi : 0.0);
      if (lane == 0) pvw[wave] = pv;
    } else if (lane == 0) {
      pvw[wave] = 0.0;
    }
    if (part == 0) pb[(row / CP) * VST + row % CP] = pi;  // zero on reduced rows
    __syncthreads();  // p and the p^T v partials are published
    if (act) {
      double pv = 0.0;
#pragma unroll
      for (int w = 0; w < SY_THREADS / 64; ++w) pv += pvw[w];
      const double K = 0.5 * t * pv;
      const double wi = pi - K * vi;  // w = p - (tau / 2)(p^T v) v;  A -= v w^T + w v^T
#pragma unroll
      for (int u = 0; u < CP; ++u) {
        const double wj = pb[part * VST + u] - K * vp[u];
        a[u] = fma(-vi, wj, fma(-wi, vp[u], a[u]));
      }
    }
  }
#pragma unroll
  for (int u = 0; u < CP; ++u) {  // the trailing 2 x 2 block
    const int j = part * CP + u;
    if (row == n - 2 && j == n - 2) d[n - 2] = a[u];
    if (row == n - 2 && j == n - 1) e[n - 2] = a[u];
    if (row == n - 1 && j == n - 1) d[n - 1] = a[u];
  }
  if (tid == 0) {
    e[n - 1] = 0.0;
    tau[n - 2] = 0.0;
    tau[n - 1] = 0.0;
  }
  __syncthreads();

  // ---- Gershgorin bounds of T and its scale
  if (tid < 128) {
    double glo = 1e300, ghi = -1e300, tm = 0.0;
    if (tid < n) {
      const double r = (tid > 0 ? fabs(e[tid - 1]) : 0.0) + (tid < n - 1 ? fabs(e[tid]) : 0.0);
      glo = d[tid] - r;
      ghi = d[tid] + r;
      tm = fabs(d[tid]) + r;
    }
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) {
      glo = fmin(glo, __shfl_xor(glo, o, 64));
      ghi = fmax(ghi, __shfl_xor(ghi, o, 64));
      tm = fmax(tm, __shfl_xor(tm, o, 64));
    }
    if (lane == 0) {
      gred[wave][0] = glo;
      gred[wave][1] = ghi;
      gred[wave][2] = tm;
    }
  }
  __syncthreads();
  const double glo = fmin(gred[0][0], gred[1][0]), ghi = fmax(gred[0][1], gred[1][1]);
  double tnorm = fmax(gred[0][2], gred[1][2]);
  if (!(tnorm > 0.0)) tnorm = 1.0;  // zero matrix: any scale works
  const double span = fmax(ghi - glo, tnorm * 1e-6);
  const double inv_tn = 1.0 / tnorm;
  // fp32 copies for the counts (scaled by 1 / ||T|| to stay well inside the fp32 range);
  // e2s[i] = e[i - 1]^2 and es[i] = e[i - 1] (zero at i = 0)
  for (int i = tid; i < n; i += SY_THREADS) {
    df[i] = (float)(d[i] * inv_tn);
    const float ei = i > 0 ? (float)(e[i - 1] * inv_tn) : 0.f;
    e2s[i] = ei * ei;
    es[i] = i > 0 ? e[i - 1] : 0.0;
  }
  __syncthreads();

  // ---- fp32 multisection: eigenvalue index n-1-j (the j-th largest) lies in [L, H)
  {
    const float pivmin = 1e-30f;
    const int j = tid / SY_S, s = tid % SY_S;
    if (j < k) {
      float L = (float)((glo - 1e-3 * span) * inv_tn), H = (float)((ghi + 1e-3 * span) * inv_tn);
      const int idx = n - 1 - j;
      for (int round = 0; round < SY_ROUNDS; ++round) {
        auto sample = [&](int q) { return L + (H - L) * (float)(q + 1) / (float)(SY_S + 1); };
        const float x = sample(s);
        int c = 0;
        float q = 1.0f;  // e2s[0] = 0: the first pivot is df[0] - x
        for (int i0 = 0; i0 < n; i0 += 8) {
          float dv[8], ev[8];
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            dv[u] = df[i0 + u] - x;
            ev[u] = e2s[i0 + u];
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            q = dv[u] - ev[u] * __builtin_amdgcn_rcpf(q);
            if (fabsf(q) < pivmin) q = -pivmin;
            c += q < 0.f;
          }
        }
        // the samples grow with s: L moves to the last one with count <= idx, H to the
        // first one above
        const unsigned int m = (unsigned int)((__ballot(c <= idx) >> (lane & 48)) & 0xFFFFull);
        const unsigned int z = ~m & 0xFFFFu;
        const float nL = m ? sample(31 - __clz(m)) : L;
        const float nH = z ? sample(__ffs(z) - 1) : H;
        L = nL;
        H = nH;
      }
      if (s == 0) lamf[j] = 0.5f * (L + H);
    }
  }
  __syncthreads();

  // ---- inverse iteration on T - lambda I (LDL^T without pivoting, factored once), one
  // lane per eigenvector; passes over the vector move 8 entries at a time between LDS and
  // registers, the next 8 loaded while the current ones are processed.  Pivots are kept at
  // least eps * ||T|| in magnitude, so one step of either recurrence grows the vector by at
  // most ~2 / eps; after every 8 entries a vector that has grown past 1e100 is rescaled as a
  // whole (processed and unprocessed entries: only its direction matters; in the first
  // solve the start entries not yet generated stay as they are, which only changes the
  // start vector), which keeps it finite for any shift, also inside clusters of
  // (near-)zero eigenvalues of rank-deficient inputs.
  if (tid < k) {
    const int j = tid;
    const double ptiny = 2.220446049250313e-16 * tnorm;
    const double big = 1e100;
    const double lam = (double)lamf[j] * tnorm;
    double* iD = &iDs[j * YLD];
    double* yv = &Y[j * YLD];
    double c0[8], c1[8], c2[8], n0[8], n1[8], n2[8];
    auto shift = [&]() {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        c0[u] = n0[u];
        c1[u] = n1[u];
        c2[u] = n2[u];
      }
    };
    // factorisation fused with the first solve L z = x (L_{i,i-1} = e_{i-1} / D_{i-1}), the
    // start entries deterministic pseudo-random in [0.5, 1.5)
    {
      auto ld = [&](int i0, double (&dd)[8], double (&ee2)[8], double (&ee)[8]) {
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          dd[u] = d[i0 + u] - lam;
          ee2[u] = es[i0 + u] * es[i0 + u];  // es[0] = 0: the first pivot is d[0] - lam
          ee[u] = e[i0 + u];
        }
      };
      double idp = 0.0, z = 0.0, lprev = 0.0;
      ld(0, c0, c1, c2);
      for (int i0 = 0; i0 < n; i0 += 8) {
        if (i0 + 8 < n) ld(i0 + 8, n0, n1, n2);
        double zs[8], ids[8], mx = 0.0;
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          double Di = c0[u] - c1[u] * idp;
          if (fabs(Di) < ptiny) Di = Di < 0.0 ? -ptiny : ptiny;
          idp = recip(Di);
          ids[u] = idp;
          uint32_t h = (uint32_t)((i0 + u) * 0x9E3779B1u) ^ (uint32_t)((j + 1) * 0x85EBCA77u);
          h ^= h >> 15;
          h *= 0x2C1B3C6Du;
          h ^= h >> 12;
          z = (0.5 + (double)(h >> 8) * (1.0 / 16777216.0)) - lprev * z;
          zs[u] = z;
          lprev = c2[u] * idp;
          mx = fmax(mx, fabs(z));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          iD[i0 + u] = ids[u];
          yv[i0 + u] = zs[u];
        }
        if (mx > big) {  // rare: rescale what is stored so far
          const double sc = 1.0 / mx;
          for (int i = 0; i < i0 + 8; ++i) yv[i] *= sc;
          z *= sc;
        }
        shift();
      }
    }
    auto ld_sol = [&](int i0, double (&xx)[8], double (&ee)[8], double (&dd)[8]) {
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        xx[u] = yv[i0 + u];
        ee[u] = e[i0 + u];
        dd[u] = iD[i0 + u];
      }
    };
    double gmx = 0.0;  // largest magnitude of the last solve's entries
    for (int it = 0; it < 3; ++it) {
      if (it > 0) {  // L z = x
        double z = 0.0, lprev = 0.0;
        ld_sol(0, c0, c1, c2);
        for (int i0 = 0; i0 < n; i0 += 8) {
          if (i0 + 8 < n) ld_sol(i0 + 8, n0, n1, n2);
          double mx = 0.0;
#pragma unroll
          for (int u = 0; u < 8; ++u) {
            z = c0[u] - lprev * z;
            c0[u] = z;
            lprev = c1[u] * c2[u];
            mx = fmax(mx, fabs(z));
          }
#pragma unroll
          for (int u = 0; u < 8; ++u) yv[i0 + u] = c0[u];
          if (mx > big) {  // rare: rescale the whole vector and the entries loaded ahead
            const double sc = 1.0 / mx;
            for (int i = 0; i < n; ++i) yv[i] *= sc;
#pragma unroll
            for (int u = 0; u < 8; ++u) n0[u] *= sc;
            z *= sc;
          }
          shift();
        }
      }
      // D L^T y = z
      double y = 0.0;
      gmx = 0.0;
      ld_sol(n - 8, c0, c1, c2);
      for (int i0 = n - 8; i0 >= 0; i0 -= 8) {
        if (i0 >= 8) ld_sol(i0 - 8, n0, n1, n2);
        double mx = 0.0;
#pragma unroll
        for (int u = 7; u >= 0; --u) {
          y = (c0[u] - c1[u] * y) * c2[u];  // e[n-1] = 0 starts the recurrence
          c0[u] = y;
          mx = fmax(mx, fabs(y));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) yv[i0 + u] = c0[u];
        gmx = fmax(gmx, mx);
        if (gmx > big) {
          const double sc = 1.0 / gmx;
          for (int i = 0; i < n; ++i) yv[i] *= sc;
#pragma unroll
          for (int u = 0; u < 8; ++u) n0[u] *= sc;
          y *= sc;
          gmx = 1.0;
        }
        shift();
      }
    }
    // the norm, formed after scaling by the largest entry so the sum of squares cannot
    // overflow; the vector is scaled when it is read for the back-transformation
    const double sm = gmx > 0.0 ? 1.0 / gmx : 0.0;
    double nrm = 0.0;
    for (int i0 = 0; i0 < n; i0 += 8) {
      double v[8];
#pragma unroll
      for (int u = 0; u < 8; ++u) v[u] = yv[i0 + u] * sm;
#pragma unroll
      for (int u = 0; u < 8; ++u) nrm = fma(v[u], v[u], nrm);
    }
    ysc[j] = nrm > 0.0 ? sm / sqrt(nrm) : 0.0;
  }
  // modified Gram-Schmidt inside clusters of eigenvalues the fp32 bisection cannot separate
  const float clus = 1e-5f;
  bool near = false;
  if (tid < k)
    for (int i = 0; i < tid; ++i) near |= fabsf(lamf[i] - lamf[tid]) <= clus;
  if (__syncthreads_or(near)) {
    for (int idx = tid; idx < k * n; idx += SY_THREADS) Y[(idx / n) * YLD + idx % n] *= ysc[idx / n];
    __syncthreads();
    if (tid < k) ysc[tid] = 1.0;
    for (int j = 1; j < k; ++j) {
      for (int i = 0; i < j; ++i) {
        if (fabsf(lamf[i] - lamf[j]) > clus) continue;  // uniform across the block
        if (wave == 0) {
          double s = 0.0;
          for (int c = lane; c < n; c += 64) s += Y[i * YLD + c] * Y[j * YLD + c];
          s = wave_sum_f64(s);
          for (int c = lane; c < n; c += 64) Y[j * YLD + c] -= s * Y[i * YLD + c];
          double s2 = 0.0;
          for (int c = lane; c < n; c += 64) s2 += Y[j * YLD + c] * Y[j * YLD + c];
          s2 = wave_sum_f64(s2);
          const double inv = s2 > 0.0 ? 1.0 / sqrt(s2) : 0.0;
          for (int c = lane; c < n; c += 64) Y[j * YLD + c] *= inv;
        }
        __syncthreads();
      }
    }
  }

  // ---- back-transformation x = H_0 (H_1 (... H_{n-3} y)); 16 lanes per eigenvector,
  // lane g keeping entries g, g + 16, ... in registers; a step is one batch of loads of
  // the reflector and its tau (both prefetched a step ahead), one 16-lane reduction and NU
  // FMAs.  Each wave owns its vectors: no block barriers inside the loop.
  const int j = tid >> 4, g = tid & 15;
  const bool own = j < k;
  double y[NU];
  {
    const double sy = own ? ysc[j] : 0.0;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int i = g + 16 * u;
      y[u] = (own && i < n) ? Y[j * YLD + i] * sy : 0.0;
    }
  }
  {
    double hn[NU], tn;
    // reflector kk at entries i: 0 for i <= kk, 1 at kk + 1, v below
    auto load_h = [&](int kk, double (&h)[NU]) {
      if constexpr (NR == 64) {
#pragma unroll
        for (int u = 0; u < NU; ++u) h[u] = VR[kk * NR + g + 16 * u];
      } else {
        const int vo = sy_voff(kk, n) - kk - 2;
#pragma unroll
        for (int u = 0; u < NU; ++u) {
          const int i = g + 16 * u;
          h[u] = i > kk + 1 && i < n ? VR[vo + i] : (i == kk + 1 ? 1.0 : 0.0);
        }
      }
    };
    load_h(n - 3, hn);
    tn = tau[n - 3];
    for (int kk = n - 3; kk >= 0; --kk) {
      double hv[NU];
#pragma unroll
      for (int u = 0; u < NU; ++u) hv[u] = hn[u];
      const double t = tn;  // zero for a column that needed no reflection
      if (kk > 0) {
        load_h(kk - 1, hn);
        tn = tau[kk - 1];
      }
      double s0 = 0.0, s1 = 0.0;
#pragma unroll
      for (int u = 0; u < NU; u += 2) {
        s0 = fma(hv[u], y[u], s0);
        s1 = fma(hv[u + 1], y[u + 1], s1);
      }
      const double ts = t * row16_sum_f64(s0 + s1);
#pragma unroll
      for (int u = 0; u < NU; ++u) y[u] = fma(-ts, hv[u], y[u]);
    }
  }
  // ---- sign normalisation (the first entry of largest magnitude made positive) and output
  double bv = 0.0;
  int bi = 1 << 30;
#pragma unroll
  for (int u = 0; u < NU; ++u) {
    const int i = g + 16 * u;
    if (i < n && (fabs(y[u]) > fabs(bv) || (fabs(y[u]) == fabs(bv) && i < bi))) {
      bv = y[u];
      bi = i;
    }
  }
  auto pick = [&](double ov, int oi) {
    if (fabs(ov) > fabs(bv) || (fabs(ov) == fabs(bv) && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  };
  pick(dpp_f64<0xB1>(bv), __builtin_amdgcn_mov_dpp(bi, 0xB1, 0xF, 0xF, true));
  pick(dpp_f64<0x4E>(bv), __builtin_amdgcn_mov_dpp(bi, 0x4E, 0xF, 0xF, true));
  pick(dpp_f64<0x141>(bv), __builtin_amdgcn_mov_dpp(bi, 0x141, 0xF, 0xF, true));
  pick(dpp_f64<0x140>(bv), __builtin_amdgcn_mov_dpp(bi, 0x140, 0xF, 0xF, true));
  const double sg = bv < 0.0 ? -1.0 : 1.0;
  if (own) {
    if (g == 0 && lam_out) lam_out[(int64_t)b * k + j] = (double)lamf[j] * tnorm;
#pragma unroll
    for (int u = 0; u < NU; ++u) {
      const int i = g + 16 * u;
      if (i >= n) continue;
      const double v = y[u] * sg;
      const int64_t o = (int64_t)b * n * k + (int64_t)i * k + j;
      if (U64) U64[o] = v;
      if (U32) U32[o] = (float)v;
      if (U16) U16[o] = f64_to_f16(v);
    }
  }
}

hipError_t launch_syev_topk_any(const void* A, bool f32in, int n, int k, int batch, double* U64, float* U32,
                                _Float16* U16, double* lam, hipStream_t s) {
  // inverse iteration walks the vectors 8 entries at a time
  if (n > SY_N || k > SY_K || k > n || n < 8 || (n & 7)) return hipErrorInvalidValue;
  if (n <= 64) {
    if (f32in)
      hipLaunchKernelGGL((k_syev_topk<float, 64>), dim3(batch), dim3(SY_THREADS), 0, s, (const float*)A, n, k, U64,
                         U32, U16, lam);
    else
      hipLaunchKernelGGL((k_syev_topk<double, 64>), dim3(batch), dim3(SY_THREADS), 0, s, (const double*)A, n, k,
                         U64, U32, U16, lam);
  } else {
    if (f32in)
      hipLaunchKernelGGL((k_syev_topk<float, 128>), dim3(batch), dim3(SY_THREADS), 0, s, (const float*)A, n, k, U64,
                         U32, U16, lam);
    else
      hipLaunchKernelGGL((k_syev_topk<double, 128>), dim3(batch), dim3(SY_THREADS), 0, s, (const double*)A, n, k,
                         U64, U32, U16, lam);
  }
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
  constexpr int VEC = 16 / sizeof(TIn);          // elements per 16-byte load
  constexpr int GPR = 16 * NT / VEC;             // 16-byte groups per staged row
  constexpr int NL = (GRAM_SLAB * GPR + 255) / 256;  // groups per thread and slab
  __shared__ __align__(16) TIn Zs[2][GRAM_SLAB][GRAM_LS];
  static_assert(sizeof(Zs) >= 4 * 256 * sizeof(double), "the wave sums fit the slab buffers");
  const int q = blockIdx.x, b = blockIdx.y, tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6;
  const int64_t chunk = rows / nparts;
  const TIn* Z = src + ((int64_t)b * rows + (int64_t)q * chunk) * p;
  const int li = lane & 15, lk = lane >> 4;
  gram_d4 acc[NU];
#pragma unroll
  for (int u = 0; u < NU; ++u) acc[u] = (gram_d4){0.0, 0.0, 0.0, 0.0};
  // slab rows r0 .. r0 + 63 (zero past the chunk and past column p); p % 4 == 0 and the block
  // starts 16-byte aligned, so each 16-byte group of a row lies wholly inside or outside p.
  // The next slab is loaded into registers during the current slab's products and stored
  // into the other buffer after them (one barrier per slab).
  uint4 ld[NL];
  auto fetch = [&](int64_t r0) {
    const int nr = (int)(chunk - r0 < GRAM_SLAB ? chunk - r0 : GRAM_SLAB);
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + 256 * i, r = e / GPR, c = (e - r * GPR) * VEC;
      ld[i] = make_uint4(0u, 0u, 0u, 0u);
      if (e < GRAM_SLAB * GPR && r < nr && c < p) ld[i] = *(const uint4*)(Z + (r0 + r) * p + c);
    }
  };
  auto put = [&](int buf) {
#pragma unroll
    for (int i = 0; i < NL; ++i) {
      const int e = tid + 256 * i, r = e / GPR, c = (e - r * GPR) * VEC;
      if (e < GRAM_SLAB * GPR) *(uint4*)&Zs[buf][r][c] = ld[i];
    }
  };
  fetch(0);
  put(0);
  __syncthreads();
  int buf = 0;
  for (int64_t r0 = 0; r0 < chunk; r0 += GRAM_SLAB) {
    const bool more = r0 + GRAM_SLAB < chunk;
    if (more) fetch(r0 + GRAM_SLAB);
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {  // rows past the chunk are zero
      const int k = 16 * w + 4 * ks + lk;
      double a[NT];
#pragma unroll
      for (int I = 0; I < NT; ++I) a[I] = (double)Zs[buf][k][16 * I + li];
      int u = 0;
#pragma unroll
      for (int I = 0; I < NT; ++I)
#pragma unroll
        for (int J = I; J < NT; ++J, ++u) acc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64(a[I], a[J], acc[u], 0, 0, 0);
    }
    if (more) put(buf ^ 1);  // its last readers passed the previous barrier
    __syncthreads();
    buf ^= 1;
  }
  // the four waves' sums go through the slab buffers (free after the last barrier)
  double(*red)[256] = reinterpret_cast<double(*)[256]>(&Zs[0][0][0]);
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
