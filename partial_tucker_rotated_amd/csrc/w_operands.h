// Rotated reconstruction operands of the score pass, shared by the kernel that forms them
// on their own (k_prep_w) and the core kernel that forms them after the cores (k_cores),
// so that both give the same values to the bit.
//
// Per table t, chain c and slice n, from the fp16 cores G (32 rows k, r_d columns j):
//   chain c < 4 (r_d = 4 << c): W[k][f] = sum_{j < r_d} G[k][j] V[f][j]   (V = Q fp16(U_d), fp32)
//   chain 4     (r_d = D):      W[k][f] = (1/sqrt(D)) sum_i H[f][i] sigma_i G[k][i]
// (Q = H diag(sigma) / sqrt(D) acting on the feature axis, "Rotated Tucker residual for
// outlier-resistant KV quantization", Key formulas), stored negated and split into fp16
// hi = fp16(w), lo = fp16(w - hi), layout [t][c][n][f][k].  Sums in fp64, j ascending.
// All helpers run on the 256 threads of a workgroup.
#pragma once
#include "common.h"

constexpr int PW_VS = JOLT_KMAX + 4;  // row stride of the V rows in LDS (16-byte aligned)

__device__ __forceinline__ void prep_w_store(float w, int64_t o, _Float16* Wh, _Float16* Wl, int& overflow) {
  const _Float16 h = (_Float16)w;
  if (!(fabsf((float)h) <= 65504.f)) overflow = 1;
  Wh[o] = h;
  Wl[o] = (_Float16)(w - (float)h);
}

// chains c < 4: g = core rows (row stride gs doubles), vs = V rows [D][PW_VS] in LDS.
// Thread (k = tid % 32) keeps core row k in registers and forms W[k][f] for
// f = tid / 32, tid / 32 + 8, ..., U outputs at a time (U independent FMA chains; the
// order within each sum does not depend on U; D is a multiple of 8 U)
template <int RD, int U = 1>
__device__ __forceinline__ void prep_w_rows(const double* g, int gs, const float* vs, int D, int64_t obase,
                                            _Float16* Wh, _Float16* Wl, int& overflow) {
  const int kk = threadIdx.x & 31;
  double gr[RD];
#pragma unroll
  for (int j = 0; j < RD; ++j) gr[j] = g[kk * gs + j];
  for (int f0 = threadIdx.x >> 5; f0 < D; f0 += 8 * U) {
    double sum[U];
#pragma unroll
    for (int u = 0; u < U; ++u) sum[u] = 0.0;
#pragma unroll
    for (int j = 0; j < RD; j += 4) {
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float4 v = *(const float4*)&vs[(f0 + 8 * u) * PW_VS + j];
        sum[u] = fma(gr[j], (double)v.x, sum[u]);
        sum[u] = fma(gr[j + 1], (double)v.y, sum[u]);
        sum[u] = fma(gr[j + 2], (double)v.z, sum[u]);
        sum[u] = fma(gr[j + 3], (double)v.w, sum[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      prep_w_store(-(float)sum[u], obase + (f0 + 8 * u) * JOLT_KMAX + kk, Wh, Wl, overflow);
  }
}

// chain 4: g = the 32 sign-flipped core rows (row stride gs doubles) in LDS, transformed in
// place by the fast Walsh-Hadamard transform (strides 1, 2, ..., D/2 in that order, one
// barrier per stage; D = 2^lD), then scaled, negated, split and stored
__device__ __forceinline__ void prep_w_hadamard(double* g, int gs, int lD, int64_t obase, _Float16* Wh,
                                                _Float16* Wl, int& overflow) {
  const int D = 1 << lD;
  for (int ls = 0; ls < lD; ++ls) {
    const int st = 1 << ls;
    for (int idx = threadIdx.x; idx < JOLT_KMAX * (D / 2); idx += 256) {
      const int kk = idx >> (lD - 1), pr = idx & (D / 2 - 1);
      const int i0 = ((pr >> ls) << (ls + 1)) + (pr & (st - 1)), i1 = i0 + st;
      const double a = g[kk * gs + i0], b = g[kk * gs + i1];
      g[kk * gs + i0] = a + b;
      g[kk * gs + i1] = a - b;
    }
    __syncthreads();
  }
  const double isq = 1.0 / sqrt((double)D);
  for (int idx = threadIdx.x; idx < D * JOLT_KMAX; idx += 256) {
    const int f = idx / JOLT_KMAX, kk = idx % JOLT_KMAX;
    prep_w_store(-(float)(g[kk * gs + f] * isq), obase + idx, Wh, Wl, overflow);
  }
}
