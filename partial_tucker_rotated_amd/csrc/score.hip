// Fused candidate scoring pass.
//
// For one table, the 24 non-trivial (r_T, r_d) pairs form six chains whose
// reconstructions are nested partial sums:
//   chain c < 5 (r_d = 4, 8, 16, 32, D):  X~ = U_T[:, :r_T] W_c,  r_T = 4 -> 8 -> 16 -> 32
//   chain 5     (r_T = T):                X~ = G_T[:, :r_d] U_d^T, r_d = 4 -> 8 -> 16 -> 32
// Because the rotation Q acts on the feature axis and is linear, the rotated
// residual is Y = Q R = Z - U_T (W Q^T) with Z = Q X computed once per tile, so no
// transform is applied per candidate ("Joint Tucker-rank and residual-bit KV
// allocator", Formulas: D is measured on X~ + Q^T Q_b(QR); Q^T Q = I lets the error
// be summed in the rotated domain).  Each wave owns one chain: MFMA accumulates the
// negated, fp16 hi/lo split operand into the fp32 Z tile, and after ranks 4, 8, 16
// and 32 the block quantizer of "Rotated Tucker residual for outlier-resistant KV
// quantization" (Key formulas: s = max|Y| / (2^(b-1) - 1), q = clip(round(Y/s))) is
// scored for b = 0, 2, 4, 8 on every row of D values:
//   e_0 = sum Y^2
//   e_2 = sum min(Y^2, (m - |Y|)^2) = e_0 - 2 m^2 sum max(0, |Y|/m - 1/2)
//   e_b = (m / (2^(b-1) - 1))^2 sum (u - rne(u))^2,  u = Y (2^(b-1) - 1) / m   (b = 4, 8)
// (the clip never binds because |Y| <= m).
#include "jolt_internal.h"

namespace jolt {

struct ScoreAcc {
  float e0, e2, e4, e8;
};

// value of lane ^ 1 (CTRL 0xB1) or lane ^ 2 (CTRL 0x4E) of the same quad, by DPP quad permute
template <int CTRL>
__device__ __forceinline__ float quad_xor(float v) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

template <int NJ>
__device__ __forceinline__ void score_rows(const float4_t (&Y)[NJ], ScoreAcc& acc) {
  float m = 0.f;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) m = fmaxf(m, fabsf(Y[jt][i]));
  m = fmaxf(m, __shfl_xor(m, 16, 64));
  m = fmaxf(m, __shfl_xor(m, 32, 64));
  const float im = m > 0.f ? __builtin_amdgcn_rcpf(m) : 0.f;
  const float c4 = 7.f * im, c8 = 127.f * im;
  float s0 = 0.f, s2 = 0.f, s4 = 0.f, s8 = 0.f;
#pragma unroll
  for (int jt = 0; jt < NJ; ++jt)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float y = Y[jt][i];
      s0 = fmaf(y, y, s0);
      s2 += __builtin_amdgcn_fmed3f(fmaf(fabsf(y), im, -0.5f), 0.f, 1.f);
      const float u4 = y * c4;
      const float d4 = u4 - __builtin_rintf(u4);
      s4 = fmaf(d4, d4, s4);
      const float u8 = y * c8;
      const float d8 = u8 - __builtin_rintf(u8);
      s8 = fmaf(d8, d8, s8);
    }
  const float m2 = m * m;
  acc.e0 += s0;
  acc.e2 += fmaf(-2.f * m2, s2, s0);
  acc.e4 = fmaf(s4, m2 * (1.f / 49.f), acc.e4);
  acc.e8 = fmaf(s8, m2 * (1.f / 16129.f), acc.e8);
}

// K-slot map of the five MFMAs of a chain: rank checkpoints after slots 0, 1, 2, 4.
// A operand (negated W, hi/lo): slot s, lane group g -> (k base, lo part?, zero?)
__device__ __forceinline__ void a_slot(int s, int g, int& kb, bool& lo, bool& zero) {
  zero = false;
  if (s < 2) {
    kb = 4 * s;
    lo = g == 1;
    zero = g >= 2;
  } else {
    const int base = s == 2 ? 8 : (s == 3 ? 16 : 24);
    kb = base + 4 * (g & 1);
    lo = g >= 2;
  }
}
__device__ __forceinline__ void b_slot(int s, int g, int& kb, bool& zero) {
  zero = false;
  if (s < 2) {
    kb = 4 * s;
    zero = g >= 2;
  } else {
    const int base = s == 2 ? 8 : (s == 3 ? 16 : 24);
    kb = base + 4 * (g & 1);
  }
}

constexpr int SCORE_CHUNK = 512;  // tokens per workgroup (looped in tiles of 64)
// Two waves per chain, each scoring two of a tile's four 16-token subtiles: twelve
// waves put three on every SIMD, each with the same work (six waves, one per chain,
// left two SIMDs with one wave and two with two).  The chains' A fragments live in
// LDS, where both waves of a chain read them, instead of in 80 VGPRs per wave.
constexpr int SCORE_WAVES = 12;

template <int D>
__global__ __launch_bounds__(64 * SCORE_WAVES) void k_score(const ScoreArgs a, const TablePtrs xp) {
  constexpr int NJ = D / 16;  // 16-feature MFMA row tiles
  constexpr int ZS = D + 4;   // LDS row stride in floats
  constexpr int SEG = D / 32; // 32-value segments per token row
  constexpr int NF = 6 * 5 * NJ * 64;  // A fragments: [chain][slot][row tile][lane]
  __shared__ __align__(16) float Z[64 * ZS];
  __shared__ __align__(16) half4_t AF[NF];

  const int n = blockIdx.x, t = blockIdx.y, ch = blockIdx.z;
  const int T = a.T, N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int tbeg = ch * SCORE_CHUNK, tend = min(T, tbeg + SCORE_CHUNK);

  // ---- operand fragments of the six chains, staged once for every tile of the chunk
  // (ordered before their first read by the barrier after the first tile's Z)
  for (int idx = tid; idx < NF; idx += 64 * SCORE_WAVES) {
    const int ln = idx & 63, jt = (idx >> 6) % NJ, s = (idx >> 6) / NJ % 5, cc = idx / (64 * NJ * 5);
    const int gg = ln >> 4;  // the slot map of a_slot, with the slot a run-time value
    const bool zero = s < 2 && gg >= 2;
    const bool lo = s < 2 ? gg == 1 : gg >= 2;
    const int kb = s < 2 ? 4 * s : (s == 2 ? 8 : (s == 3 ? 16 : 24)) + 4 * (gg & 1);
    const _Float16* src;
    if (cc < 5) {
      const int64_t base = (((int64_t)t * 5 + cc) * N + n) * D * JOLT_KMAX;
      src = (lo ? a.Wneg_lo : a.Wneg_hi) + base;
    } else {
      src = (lo ? a.Vneg_lo : a.Vneg_hi) + (int64_t)t * D * JOLT_KMAX;
    }
    AF[idx] = zero ? (half4_t){0, 0, 0, 0} : *(const half4_t*)(src + (jt * 16 + (ln & 15)) * JOLT_KMAX + kb);
  }

  const int c = wave >> 1, h = wave & 1;  // chain, subtile parity
  const int g = lane >> 4, r = lane & 15;
  const half4_t* Ac = AF + c * 5 * NJ * 64 + lane;
  ScoreAcc acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) acc[i] = ScoreAcc{0.f, 0.f, 0.f, 0.f};
  const int8_t* sgn_base = a.signs + t * D;
  const float isq = (float)(1.0 / __builtin_sqrt((double)D));

  // the rotating threads' 32 input values of the next tile, loaded one tile ahead
  const bool rot = tid < 64 * SEG;
  const int tk = tid / SEG, sg = tid % SEG;
  const uint16_t* xrow = (const uint16_t*)xp.p[t] + ((int64_t)n * T + tk) * D + sg * 32;
  uint4 xin[4];
  if (rot) {
#pragma unroll
    for (int q = 0; q < 4; ++q) xin[q] = *(const uint4*)(xrow + (int64_t)tbeg * D + q * 8);
  }

  for (int tok0 = tbeg; tok0 < tend; tok0 += 64) {
    // ---- Z = Q x = H (sigma . x) / sqrt(D) for the 64 token rows of this tile
    if (rot) {
      const int8_t* sgn = sgn_base + sg * 32;
      float v[32];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const uint4 raw = xin[q];
        const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
        for (int hh = 0; hh < 4; ++hh) {
          v[q * 8 + 2 * hh] = __uint_as_float(w[hh] << 16);
          v[q * 8 + 2 * hh + 1] = __uint_as_float(w[hh] & 0xFFFF0000u);
        }
      }
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = sgn[i] < 0 ? -v[i] : v[i];
#pragma unroll
      for (int s = 1; s < 32; s <<= 1)
#pragma unroll
        for (int i = 0; i < 32; ++i)
          if (!(i & s)) {
            const float p = v[i], q2 = v[i + s];
            v[i] = p + q2;
            v[i + s] = p - q2;
          }
      // segments of a token row sit in consecutive lanes (SEG = 2 or 4 of a quad)
      const float sv1 = (sg & 1) ? -1.f : 1.f, sv2 = (sg & 2) ? -1.f : 1.f;
#pragma unroll
      for (int i = 0; i < 32; ++i) v[i] = quad_xor<0xB1>(v[i]) + sv1 * v[i];
      if constexpr (SEG == 4) {
#pragma unroll
        for (int i = 0; i < 32; ++i) v[i] = quad_xor<0x4E>(v[i]) + sv2 * v[i];
      }
#pragma unroll
      for (int i = 0; i < 32; i += 4)
        *(float4_t*)&Z[tk * ZS + sg * 32 + i] =
            (float4_t){v[i] * isq, v[i + 1] * isq, v[i + 2] * isq, v[i + 3] * isq};
    }
    __syncthreads();
    if (rot && tok0 + 64 < tend) {
#pragma unroll
      for (int q = 0; q < 4; ++q) xin[q] = *(const uint4*)(xrow + (int64_t)(tok0 + 64) * D + q * 8);
    }

#pragma unroll 1
    for (int i2 = 0; i2 < 2; ++i2) {
      // keeps the fragment loads inside the loop: hoisted, they would hold 80 VGPRs
      asm volatile("" ::: "memory");
      const int tt = 2 * i2 + h;
      const int tok = tok0 + tt * 16 + r;
      const _Float16* Bsrc = c < 5 ? a.UT16 + (((int64_t)t * 5 + c) * T + tok) * JOLT_KMAX
                                   : a.G16T + (((int64_t)t * N + n) * T + tok) * JOLT_KMAX;
      half4_t Bf[5];
#pragma unroll
      for (int s = 0; s < 5; ++s) {
        int kb;
        bool zero;
        b_slot(s, g, kb, zero);
        Bf[s] = zero ? (half4_t){0, 0, 0, 0} : *(const half4_t*)(Bsrc + kb);
      }
      float4_t Y[NJ];
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) Y[jt] = *(const float4_t*)&Z[(tt * 16 + r) * ZS + jt * 16 + 4 * g];
#pragma unroll
      for (int s = 0; s < 3; ++s) {
#pragma unroll
        for (int jt = 0; jt < NJ; ++jt) Y[jt] = mfma16(Ac[(s * NJ + jt) * 64], Bf[s], Y[jt]);
        score_rows<NJ>(Y, acc[s]);
      }
#pragma unroll
      for (int jt = 0; jt < NJ; ++jt) {
        Y[jt] = mfma16(Ac[(3 * NJ + jt) * 64], Bf[3], Y[jt]);
        Y[jt] = mfma16(Ac[(4 * NJ + jt) * 64], Bf[4], Y[jt]);
      }
      score_rows<NJ>(Y, acc[3]);
    }
    __syncthreads();  // Z is rewritten by the next tile
  }

  // ---- partial sums of this workgroup: part[t][wg][pair][b]; the odd wave of each
  // chain hands its sums to the even one through LDS (Z is free after the last barrier)
  const int nch = (T + SCORE_CHUNK - 1) / SCORE_CHUNK;
  const int nwg = N * nch;
  const int wg = n * nch + ch;
  double* dst = a.part + ((int64_t)t * nwg + wg) * 100;
  double* xch = (double*)Z + c * 16;
  double sums[16];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    sums[4 * i + 0] = wave_sum_f64((double)acc[i].e0);
    sums[4 * i + 1] = wave_sum_f64((double)acc[i].e2);
    sums[4 * i + 2] = wave_sum_f64((double)acc[i].e4);
    sums[4 * i + 3] = wave_sum_f64((double)acc[i].e8);
  }
  if (h == 1 && lane == 0) {
#pragma unroll
    for (int e = 0; e < 16; ++e) xch[e] = sums[e];
  }
  __syncthreads();
  if (h == 0 && lane == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int pair = c < 5 ? i * 5 + c : 20 + i;  // (i_rT * 5 + i_rd)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[pair * 4 + e] = sums[4 * i + e] + xch[4 * i + e];
    }
  }
  if (wave == 0 && lane < 4) dst[24 * 4 + lane] = 0.0;  // (T, D): stored verbatim, no residual
}

int score_partials(int N, int T) { return N * ((T + SCORE_CHUNK - 1) / SCORE_CHUNK); }

hipError_t launch_score(const ScoreArgs& a, const TablePtrs& x, hipStream_t s) {
  dim3 grid(a.N, a.ntab, (a.T + SCORE_CHUNK - 1) / SCORE_CHUNK);
  if (a.D == 128)
    hipLaunchKernelGGL(k_score<128>, grid, dim3(64 * SCORE_WAVES), 0, s, a, x);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_score<64>, grid, dim3(64 * SCORE_WAVES), 0, s, a, x);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// E[t][e] = sum over workgroups of part[t][wg][e] (fixed order)
__global__ __launch_bounds__(256) void k_score_reduce(const double* part, int nwg, double* E) {
  const int e = blockIdx.x, t = blockIdx.y;
  __shared__ double red[256];
  double s = 0.0;
  for (int w = threadIdx.x; w < nwg; w += 256) s += part[((int64_t)t * nwg + w) * 100 + e];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int o = 128; o > 0; o >>= 1) {
    if (threadIdx.x < o) red[threadIdx.x] += red[threadIdx.x + o];
    __syncthreads();
  }
  if (threadIdx.x == 0) E[t * 100 + e] = red[0];
}

hipError_t launch_score_reduce(const double* part, int nparts, int ntab, double* E, hipStream_t s) {
  hipLaunchKernelGGL(k_score_reduce, dim3(100, ntab), dim3(256), 0, s, part, nparts, E);
  return hipGetLastError();
}

}  // namespace jolt
