// Record writer (encode) and reader (decode) for one chosen candidate per table.
//
// Encode follows "Rotated Tucker residual for outlier-resistant KV quantization",
// Implementation notes: with the stored Tucker factors, reconstruct X~, form
// R = X - X~, rotate each row of D values with Q = H diag(sigma) / sqrt(D), and store
// per block (one row) the scale s = max|Y| / (2^(b-1) - 1) (fp32) and the codes
// clip(round(Y / s), -2^(b-1), 2^(b-1) - 1).  The residual path runs in fp64.
// Decode follows "Joint Tucker-rank and residual-bit KV allocator", Formulas, first
// display: X^ = X~ + Q^T Q_b(Q R), in fp64, rounded once to bf16.
//
// Launches cover up to JOLT_TAB_CHUNK tables: blockIdx.y is the local table index,
// workspace arrays are indexed by the global table index t0 + local.
#include "jolt_internal.h"

namespace jolt {

#define REC_MAGIC 0x544C4F4Au

__global__ void k_rec_header(const EncodeArgs a) {
  const int tl = blockIdx.x, tg = a.t0 + tl;
  const EncodeTable& e = a.t[tl];
  uint32_t* h = (uint32_t*)e.rec;
  const int i = threadIdx.x;  // 64 words of the 256-byte header
  uint32_t w = 0;
  switch (i) {
    case 0: w = REC_MAGIC; break;
    case 1: w = 1u; break;
    case 2: w = (uint32_t)a.N; break;
    case 3: w = (uint32_t)a.T; break;
    case 4: w = (uint32_t)a.D; break;
    case 5: w = (uint32_t)e.rT; break;
    case 6: w = (uint32_t)e.rd; break;
    case 7: w = (uint32_t)e.b; break;
    case 8: w = (uint32_t)a.D; break;  // quantization block = one row of D values
    default: break;
  }
  if (i >= 10 && i < 22) {
    const int q = (i - 10) >> 1;
    const uint64_t v = q == 0 ? e.total : q == 1 ? e.off_ut : q == 2 ? e.off_ud : q == 3 ? e.off_core
                     : q == 4 ? e.off_codes : e.off_scales;
    w = (i & 1) ? (uint32_t)(v >> 32) : (uint32_t)v;
  }
  if (i >= 32 && i < 32 + (a.D + 31) / 32) {
    uint32_t bits = 0;
    for (int j = 0; j < 32; ++j) {
      const int f = (i - 32) * 32 + j;
      if (f < a.D && a.signs[tg * a.D + f] < 0) bits |= 1u << j;
    }
    w = bits;
  }
  h[i] = w;
}

// Copy a 16-bit matrix into a record section and zero the section's padding.
// which: 0 = U_T, 1 = U_d, 2 = core (or X verbatim)
__global__ void k_rec_section(const EncodeArgs a, int which) {
  const int tl = blockIdx.y, tg = a.t0 + tl;
  const EncodeTable& e = a.t[tl];
  const int N = a.N, T = a.T, D = a.D;
  uint64_t off = 0, padded = 0;
  int64_t rows = 0, cols = 1;
  if (which == 0) {
    if (e.chain < 0 || e.chain == 5) return;
    off = e.off_ut;
    rows = T;
    cols = e.rT;
    padded = (e.off_ud ? e.off_ud : e.off_core) - off;
  } else if (which == 1) {
    if (e.chain < 0 || e.chain == 4) return;
    off = e.off_ud;
    rows = D;
    cols = e.rd;
    padded = e.off_core - off;
  } else {
    off = e.off_core;
    padded = (e.off_codes ? e.off_codes : e.total) - off;
    if (e.chain < 0) {
      rows = (int64_t)N * T;
      cols = D;
    } else if (e.chain == 5) {
      rows = (int64_t)N * T;
      cols = e.rd;
    } else {
      rows = (int64_t)N * e.rT;
      cols = e.rd;
    }
  }
  uint16_t* dst = (uint16_t*)(e.rec + off);
  const int64_t nel = rows * cols, nhalf = (int64_t)(padded / 2);
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nhalf; i += stride) {
    uint16_t v = 0;
    if (i < nel) {
      const int64_t rr = i / cols, cc = i - rr * cols;
      if (which == 0) {
        v = __builtin_bit_cast(uint16_t, a.UT16[(((int64_t)tg * 5 + e.chain) * T + rr) * JOLT_KMAX + cc]);
      } else if (which == 1) {
        v = __builtin_bit_cast(uint16_t, a.Ud16[((int64_t)tg * D + rr) * JOLT_KMAX + cc]);
      } else if (e.chain < 0) {
        v = ((const uint16_t*)a.xsrc[tl])[i];
      } else if (e.chain == 5) {
        v = __builtin_bit_cast(uint16_t, a.G16T[((int64_t)tg * N * T + rr) * JOLT_KMAX + cc]);
      } else {
        const int64_t nn = rr / e.rT, kk = rr - nn * e.rT;
        v = __builtin_bit_cast(uint16_t,
                               a.G16[((((int64_t)tg * 5 + e.chain) * N + nn) * JOLT_KMAX + kk) * D + cc]);
      }
    }
    dst[i] = v;
  }
}

// 16 codes of B bits -> B/2 words (element j of the group at bits [j*B, j*B+B) of the stream)
template <int B>
__device__ __forceinline__ void pack_codes(const int (&q)[16], uint32_t* dst) {
  constexpr uint32_t mask = (1u << B) - 1u;
#pragma unroll
  for (int w = 0; w < B / 2; ++w) {
    uint32_t word = 0;
#pragma unroll
    for (int j = 0; j < 32 / B; ++j) word |= ((uint32_t)q[w * (32 / B) + j] & mask) << (j * B);
    dst[w] = word;
  }
}

// Residual codes and scales (b > 0).  One block per (slice n, table); loops over the
// tokens.  SEG = D/32 threads per row, each owning 32 consecutive features.
template <int D>
__global__ __launch_bounds__(256) void k_encode_resid(const EncodeArgs a) {
  constexpr int FPT = 16;         // features per thread
  constexpr int SEG = D / FPT;    // threads per row
  constexpr int RPP = 256 / SEG;  // rows per pass
  const int n = blockIdx.x, tl = blockIdx.y, tg = a.t0 + tl;
  const EncodeTable& e = a.t[tl];
  if (e.b == 0) return;
  const int N = a.N, T = a.T;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  const int qmax = (1 << (e.b - 1)) - 1;
  // X~ row = sum_k L_row[k] Rm[k][:]; rows k >= K are zero
  __shared__ double Rm[JOLT_KMAX][D];
  const int K = e.chain < 0 ? 0 : (e.chain == 5 ? e.rd : e.rT);
  for (int idx = tid; idx < JOLT_KMAX * D; idx += 256) {
    const int k = idx / D, f = idx % D;
    double v = 0.0;
    if (k < K) {
      if (e.chain == 5) {
        v = (double)a.Ud16[((int64_t)tg * D + f) * JOLT_KMAX + k];
      } else {
        const _Float16* Gk = a.G16 + ((((int64_t)tg * 5 + e.chain) * N + n) * JOLT_KMAX + k) * D;
        if (e.chain == 4) {
          v = (double)Gk[f];
        } else {
          for (int j = 0; j < e.rd; ++j) v += (double)Gk[j] * (double)a.Ud16[((int64_t)tg * D + f) * JOLT_KMAX + j];
        }
      }
    }
    Rm[k][f] = v;
  }
  __syncthreads();
  const double isq = 1.0 / sqrt((double)D);
  const int8_t* sgn = a.signs + tg * D + sg * FPT;
  uint32_t* codes = (uint32_t*)(e.rec + e.off_codes);
  float* scales = (float*)(e.rec + e.off_scales);
  for (int t0 = 0; t0 < T; t0 += RPP) {
    // rows of a thread group share `valid`; invalid groups compute a duplicate row and store nothing
    const bool valid = t0 + rloc < T;
    const int tok = valid ? t0 + rloc : T - 1;
    const int64_t row = (int64_t)n * T + tok;
    const uint16_t* xr = (const uint16_t*)a.xsrc[tl] + row * D + sg * FPT;
    double L[JOLT_KMAX];
    if (e.chain >= 0) {
      const _Float16* Ls = e.chain == 5 ? a.G16T + (((int64_t)tg * N + n) * T + tok) * JOLT_KMAX
                                        : a.UT16 + (((int64_t)tg * 5 + e.chain) * T + tok) * JOLT_KMAX;
#pragma unroll
      for (int k = 0; k < JOLT_KMAX; ++k) L[k] = k < K ? (double)Ls[k] : 0.0;
    } else {
#pragma unroll
      for (int k = 0; k < JOLT_KMAX; ++k) L[k] = 0.0;
    }
    double y[FPT];
    for (int i = 0; i < FPT; ++i) {
      const int f = sg * FPT + i;
      double xt = 0.0;
#pragma unroll
      for (int k = 0; k < JOLT_KMAX; ++k) xt = fma(L[k], Rm[k][f], xt);
      const double x = (double)bf16_to_f32(xr[i]);
      const double rres = e.chain >= 0 ? x - xt : 0.0;
      y[i] = sgn[i] < 0 ? -rres : rres;
    }
#pragma unroll
    for (int s = 1; s < FPT; s <<= 1)
#pragma unroll
      for (int i = 0; i < FPT; ++i)
        if (!(i & s)) {
          const double p = y[i], q2 = y[i + s];
          y[i] = p + q2;
          y[i + s] = p - q2;
        }
#pragma unroll
    for (int s = 1; s < SEG; s <<= 1)
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        const double p = __shfl_xor(y[i], s, 64);
        y[i] = (sg & s) ? (p - y[i]) : (y[i] + p);
      }
    double m = 0.0;
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      y[i] *= isq;
      m = fmax(m, fabs(y[i]));
    }
#pragma unroll
    for (int s = 1; s < SEG; s <<= 1) m = fmax(m, __shfl_xor(m, s, 64));
    const float sc = (float)(m / (double)qmax);
    const double sd = (double)sc;
    int q[FPT];
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      double v = sd > 0.0 ? rint(y[i] / sd) : 0.0;
      v = fmin(fmax(v, (double)(-qmax - 1)), (double)qmax);
      q[i] = (int)v;
    }
    if (valid) {
      uint32_t* cw = codes + (row * D + sg * FPT) * e.b / 32;
      if (e.b == 2) pack_codes<2>(q, cw);
      else if (e.b == 4) pack_codes<4>(q, cw);
      else pack_codes<8>(q, cw);
      if (sg == 0) scales[row] = sc;
    }
  }
}

template <int B>
__device__ __forceinline__ void unpack_codes(const uint32_t* src, double s, double (&y)[16]) {
  constexpr int PER = 32 / B;
#pragma unroll
  for (int w = 0; w < B / 2; ++w) {
    const uint32_t word = src[w];
#pragma unroll
    for (int j = 0; j < PER; ++j) {
      const int q = (int)(word << (32 - B * (j + 1))) >> (32 - B);  // sign-extended field j
      y[w * PER + j] = s * (double)q;
    }
  }
}

// Decoded rows of slice n in fp64, rounded once to bf16 (the only rounding of the output).
template <int D, int K>
__device__ __forceinline__ void decode_rows(const DecodeArgs& a, const EncodeTable& e, int n, int tl,
                                            double (*Rm)[D], const double* sgs) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  constexpr int RPP = 256 / SEG;
  const int T = a.T;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  const char* rec = e.rec;
  uint16_t* out = (uint16_t*)a.out[tl];
  const _Float16* Ut = (const _Float16*)(rec + e.off_ut);
  const _Float16* Gc = (const _Float16*)(rec + e.off_core);
  const uint32_t* codes = (const uint32_t*)(rec + e.off_codes);
  const float* scales = (const float*)(rec + e.off_scales);
  for (int t0 = 0; t0 < T; t0 += RPP) {
    const bool valid = t0 + rloc < T;
    const int tok = valid ? t0 + rloc : T - 1;
    const int64_t row = (int64_t)n * T + tok;
    uint16_t* orow = out + row * D + sg * FPT;
    double y[FPT];
    if (e.b > 0) {
      const double s = (double)scales[row];
      const uint32_t* cw = codes + (row * D + sg * FPT) * e.b / 32;
      if (e.b == 2) unpack_codes<2>(cw, s, y);
      else if (e.b == 4) unpack_codes<4>(cw, s, y);
      else unpack_codes<8>(cw, s, y);
#pragma unroll
      for (int st = 1; st < FPT; st <<= 1)
#pragma unroll
        for (int i = 0; i < FPT; ++i)
          if (!(i & st)) {
            const double p = y[i], q2 = y[i + st];
            y[i] = p + q2;
            y[i + st] = p - q2;
          }
#pragma unroll
      for (int st = 1; st < SEG; st <<= 1)
#pragma unroll
        for (int i = 0; i < FPT; ++i) {
          const double p = __shfl_xor(y[i], st, 64);
          y[i] = (sg & st) ? (p - y[i]) : (y[i] + p);
        }
    } else {
#pragma unroll
      for (int i = 0; i < FPT; ++i) y[i] = 0.0;
    }
    double L[K];
    const _Float16* Ls = e.chain == 5 ? Gc + row * e.rd : Ut + (int64_t)tok * e.rT;
#pragma unroll
    for (int k = 0; k < K; ++k) L[k] = (double)Ls[k];
    if (!valid) continue;
#pragma unroll
    for (int i = 0; i < FPT; i += 2) {
      double o[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int f = sg * FPT + i + h;
        double xt = 0.0;
#pragma unroll
        for (int k = 0; k < K; ++k) xt = fma(L[k], Rm[k][f], xt);
        o[h] = fma(sgs[f], y[i + h], xt);
      }
      *(uint32_t*)&orow[i] = (uint32_t)f64_to_bf16(o[0]) | ((uint32_t)f64_to_bf16(o[1]) << 16);
    }
  }
}

// Reconstruction, dequantization, inverse rotation, bf16 output.
// One block per (slice n, table); loops over the tokens.
template <int D>
__global__ __launch_bounds__(256) void k_decode(const DecodeArgs a) {
  const int n = blockIdx.x, tl = blockIdx.y;
  const EncodeTable& e = a.t[tl];
  const int T = a.T;
  const int tid = threadIdx.x;
  const char* rec = e.rec;
  __shared__ double Rm[JOLT_KMAX][D];
  __shared__ double sgs[D];  // sigma_f / sqrt(D)
  if (e.chain < 0) {  // (T, D): X stored verbatim
    const uint4* src = (const uint4*)(rec + e.off_core) + (int64_t)n * T * D / 8;
    uint4* dst = (uint4*)a.out[tl] + (int64_t)n * T * D / 8;
    for (int64_t i = tid; i < (int64_t)T * D / 8; i += 256) dst[i] = src[i];
    return;
  }
  const uint32_t* sbits = (const uint32_t*)(rec + 128);
  const double isq = 1.0 / sqrt((double)D);
  for (int f = tid; f < D; f += 256) sgs[f] = ((sbits[f >> 5] >> (f & 31)) & 1u) ? -isq : isq;
  const _Float16* Ud = (const _Float16*)(rec + e.off_ud);
  const _Float16* Gc = (const _Float16*)(rec + e.off_core);
  const int K = e.chain == 5 ? e.rd : e.rT;
  for (int idx = tid; idx < K * D; idx += 256) {
    const int k = idx / D, f = idx % D;
    double v;
    if (e.chain == 5) {
      v = (double)Ud[f * e.rd + k];
    } else if (e.chain == 4) {
      v = (double)Gc[((int64_t)n * e.rT + k) * D + f];
    } else {
      v = 0.0;
      for (int j = 0; j < e.rd; ++j)
        v = fma((double)Gc[((int64_t)n * e.rT + k) * e.rd + j], (double)Ud[f * e.rd + j], v);
    }
    Rm[k][f] = v;
  }
  __syncthreads();
  switch (K) {
    case 4: decode_rows<D, 4>(a, e, n, tl, Rm, sgs); break;
    case 8: decode_rows<D, 8>(a, e, n, tl, Rm, sgs); break;
    case 16: decode_rows<D, 16>(a, e, n, tl, Rm, sgs); break;
    default: decode_rows<D, 32>(a, e, n, tl, Rm, sgs); break;
  }
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_rec_header, dim3(a.ntab), dim3(64), 0, s, a);
  for (int which = 0; which < 3; ++which)
    hipLaunchKernelGGL(k_rec_section, dim3(512, a.ntab), dim3(256), 0, s, a, which);
  if (a.D == 128)
    hipLaunchKernelGGL(k_encode_resid<128>, dim3(a.N, a.ntab), dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_encode_resid<64>, dim3(a.N, a.ntab), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  if (a.D == 128)
    hipLaunchKernelGGL(k_decode<128>, dim3(a.N, a.ntab), dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_decode<64>, dim3(a.N, a.ntab), dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jolt
