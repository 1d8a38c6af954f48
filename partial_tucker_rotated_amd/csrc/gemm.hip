// Generic batched GEMM for the non-fused contractions of the path: feature and token
// Grams, the feature projection, the range-finder products, the core and the
// subspace-iteration products.
//
// C[b](m, n) = alpha_b * sum_k A[b](m, k) * B[b](k, n)  (+ Cin[b](m, n))
//
// Operands are addressed through strides with power-of-two index splits, so that
// unfoldings (e.g. column n*r + j of the token unfolding) are read in place.  Modes:
//  * GEMM_BF16: both operands bf16; products exact in fp32 (bf16 MFMA).
//  * GEMM_SPLIT: every operand value x is split into fp16 hi = fp16(x) and
//    lo = fp16(x - hi); the product is hi*hi + hi*lo + lo*hi (about 22 significant
//    bits, fp32 accumulation).  Operand values must lie in the fp16 range; fp16
//    subnormals are kept by gfx950 MFMA.
//  * GEMM_F64: operands widened to fp64, fp64 FMA accumulation (small problems where
//    fp64 factors are needed to reproduce fp16 storage rounding exactly).
// With acc64 the fp32 MFMA accumulators are flushed into fp64 every 256 values of k.
#include <algorithm>

#include "jolt_internal.h"
#include "w_operands.h"

namespace jolt {

__device__ __forceinline__ int64_t op_offset(const GemmOperand& o, int r, int k) {
  const int rm = (1 << o.rsh) - 1, km = (1 << o.ksh) - 1;
  return (int64_t)(r >> o.rsh) * o.sr1 + (int64_t)(r & rm) * o.sr2 + (int64_t)(k >> o.ksh) * o.sk1 +
         (int64_t)(k & km) * o.sk2;
}

__device__ __forceinline__ int op_esize(int type) { return type == 0 ? 4 : (type == 3 ? 8 : 2); }

__device__ __forceinline__ const char* op_base(const GemmOperand& o, const TablePtrs& tp, int b, int vdiv,
                                               int nvar) {
  const int esz = op_esize(o.type);
  if (o.novar) b = (b / (vdiv * nvar)) * vdiv + b % vdiv;
  const int hi = b / o.bdiv, lo = b - hi * o.bdiv;
  const char* base = o.tbl ? (const char*)tp.p[hi] : (const char*)o.p + (int64_t)hi * o.sb1 * esz;
  return base + ((int64_t)lo * o.sb2 + o.off0) * esz;
}

__device__ __forceinline__ int64_t row_off(const GemmOperand& o, int r) {
  const int rm = (1 << o.rsh) - 1;
  return (int64_t)(r >> o.rsh) * o.sr1 + (int64_t)(r & rm) * o.sr2;
}
__device__ __forceinline__ int64_t k_off(const GemmOperand& o, int k) {
  const int km = (1 << o.ksh) - 1;
  return (int64_t)(k >> o.ksh) * o.sk1 + (int64_t)(k & km) * o.sk2;
}

// 8 values (rows r, k .. k+7) of an operand as floats (split mode) or raw bf16 (bf16 mode)
template <bool BF>
__device__ __forceinline__ void load8(const GemmOperand& o, const char* base, int r, int k, int R, int K,
                                      float (&v)[8], uint16_t (&raw)[8]) {
  const bool rin = r < R;
  if (o.lmode == 1 && rin && k + 7 < K) {
    const int64_t off = row_off(o, r) + k_off(o, k);
    if (BF || o.type != 0) {
      const uint4 q = *(const uint4*)((const uint16_t*)base + off);
      const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
      for (int h = 0; h < 4; ++h) {
        raw[2 * h] = (uint16_t)(w[h] & 0xFFFFu);
        raw[2 * h + 1] = (uint16_t)(w[h] >> 16);
      }
      if (!BF) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
          v[i] = o.type == 1 ? bf16_to_f32(raw[i]) : (float)__builtin_bit_cast(_Float16, raw[i]);
      }
    } else {
      const float4 a = *(const float4*)((const float*)base + off);
      const float4 b = *(const float4*)((const float*)base + off + 4);
      v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
      v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    return;
  }
  // generic strided path: the type branch is taken once and the eight loads are issued
  // back to back (an element outside the operand reads offset 0, which is in bounds, and
  // is replaced by zero)
  const int64_t ro = rin ? row_off(o, r) : 0;
  int64_t off[8];
  bool ok[8];
  if (o.ksh >= 30) {  // no split of k: offsets advance by a constant stride
    const int64_t o0 = ro + (int64_t)k * o.sk2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ok[i] = rin && k + i < K;
      off[i] = ok[i] ? o0 + i * o.sk2 : 0;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      ok[i] = rin && k + i < K;
      off[i] = ok[i] ? ro + k_off(o, k + i) : 0;
    }
  }
  if (BF || o.type == 1 || o.type == 2) {
    const uint16_t* p = (const uint16_t*)base;
    uint16_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = p[off[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t u = ok[i] ? t[i] : (uint16_t)0;
      if (BF) raw[i] = u;
      else v[i] = o.type == 1 ? bf16_to_f32(u) : (float)__builtin_bit_cast(_Float16, u);
    }
  } else if (o.type == 0) {
    const float* p = (const float*)base;
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = p[off[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ok[i] ? t[i] : 0.f;
  } else {
    const double* p = (const double*)base;
    double t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = p[off[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ok[i] ? (float)t[i] : 0.f;
  }
}

// Loader specialised on the operand's load pattern L (the kernel is instantiated per
// pattern pair, so each instantiation holds one load path per operand):
//  L = 1: 8 consecutive k of one row as one or two 16-byte loads (K a multiple of 8);
//  L = 2: lanes along consecutive rows, k advancing by a constant stride (no k split);
//  L = 0: any operand (per-element offsets).
template <bool BF, int L>
__device__ __forceinline__ void load8s(const GemmOperand& o, const char* base, int r, int k, int R, int K,
                                       float (&v)[8], uint16_t (&raw)[8]) {
  if (L == 0) {
    load8<BF>(o, base, r, k, R, K, v, raw);
    return;
  }
  const bool rin = r < R;
  if (L == 1) {
    if (rin && k < K) {
      const int64_t off = row_off(o, r) + k_off(o, k);
      if (BF || o.type != 0) {
        const uint4 q = *(const uint4*)((const uint16_t*)base + off);
        const uint32_t w[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          raw[2 * h] = (uint16_t)(w[h] & 0xFFFFu);
          raw[2 * h + 1] = (uint16_t)(w[h] >> 16);
        }
        if (!BF) {
#pragma unroll
          for (int i = 0; i < 8; ++i)
            v[i] = o.type == 1 ? bf16_to_f32(raw[i]) : (float)__builtin_bit_cast(_Float16, raw[i]);
        }
      } else {
        const float4 a = *(const float4*)((const float*)base + off);
        const float4 b = *(const float4*)((const float*)base + off + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
      }
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        v[i] = 0.f;
        raw[i] = 0;
      }
    }
    return;
  }
  // L == 2
  const int64_t o0 = (rin ? row_off(o, r) : 0) + (int64_t)k * o.sk2;
  int64_t off[8];
  bool ok[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    ok[i] = rin && k + i < K;
    off[i] = ok[i] ? o0 + i * o.sk2 : 0;
  }
  if (BF || o.type != 0) {
    const uint16_t* p = (const uint16_t*)base;
    uint16_t t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = p[off[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t u = ok[i] ? t[i] : (uint16_t)0;
      raw[i] = u;
      if (!BF) v[i] = o.type == 1 ? bf16_to_f32(u) : (float)__builtin_bit_cast(_Float16, u);
    }
  } else {
    const float* p = (const float*)base;
    float t[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) t[i] = p[off[i]];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = ok[i] ? t[i] : 0.f;
  }
}

// 8 fp16/bf16 bit patterns packed for one 16-byte LDS store
__device__ __forceinline__ uint4 pack8(const uint16_t (&h)[8]) {
  uint4 q;
  q.x = (uint32_t)h[0] | ((uint32_t)h[1] << 16);
  q.y = (uint32_t)h[2] | ((uint32_t)h[3] << 16);
  q.z = (uint32_t)h[4] | ((uint32_t)h[5] << 16);
  q.w = (uint32_t)h[6] | ((uint32_t)h[7] << 16);
  return q;
}

// shared epilogue for one output element
__device__ __forceinline__ void store_out(const GemmArgs& g, int64_t off, double val, double alpha, int& overflow) {
  val *= alpha;
  if (g.c_type == 1) {
    if (g.Cin) val += ((const double*)g.Cin)[off];
    ((double*)g.C)[off] = val;
  } else {
    float fv = (float)val;
    if (g.Cin) fv += ((const float*)g.Cin)[off];
    if (g.C) ((float*)g.C)[off] = fv;
    val = fv;
  }
  if (g.C16) {
    const _Float16 h = f64_to_f16(val);
    if (!(fabsf((float)h) <= 65504.f)) overflow = 1;
    g.C16[off] = h;
  }
}

__device__ __forceinline__ double batch_alpha(const GemmArgs& g, int b) {
  double alpha = g.alpha;
  if (g.alpha_norm) alpha *= (double)gram_scale_from_norm(g.alpha_norm[b / g.alpha_div]);
  return alpha;
}

// Workgroup with linear index L runs on XCD L % 8.  Units of `ugrp` consecutive grid
// z-slices (all their x, y tiles) are dealt to the XCDs round-robin, so that XCD x runs
// units x, x + 8, x + 16, ... in order.  The launcher guarantees (gridDim.z / ugrp) % 8 == 0.
__device__ __forceinline__ void xcd_remap(int ugrp, int& bx, int& by, int& bz) {
  const int gx = gridDim.x, gy = gridDim.y;
  const int64_t tpb = (int64_t)gx * gy;
  const int64_t L = bx + gx * ((int64_t)by + (int64_t)gy * bz);
  const int xcd = (int)(L & 7);
  const int64_t i = L >> 3;
  const int64_t us = tpb * ugrp;  // workgroups per unit
  const int64_t u = (i / us) * 8 + xcd;
  const int64_t o = i % us;
  bz = (int)(u * ugrp + o / tpb);
  const int64_t t = o % tpb;
  bx = (int)(t % gx);
  by = (int)(t / gx);
}

// stores this thread's 2 x 2 tiles of 16 x 16 (rows wm0 + 16 i + fk + v, columns wn0 + 16 j + fr)
__device__ __forceinline__ void gemm_epilogue(const GemmArgs& g, int b, int wm0, int wn0, int fk, int fr, int M,
                                              int N, const float4_t (&acc)[2][2], const double (&dacc)[2][2][4],
                                              int64_t extra, int& overflow) {
  const double alpha = batch_alpha(g, b);
  const int cb = b / g.cbdiv;
  const int64_t cbase = (int64_t)cb * g.csb1 + (int64_t)(b - cb * g.cbdiv) * g.csb2 + extra;
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int m = wm0 + 16 * i + fk + v;
        const int n = wn0 + 16 * j + fr;
        if (m >= M || n >= N) continue;
        const int64_t off = cbase + (int64_t)m * g.csm + (int64_t)n * g.csn;
        store_out(g, off, g.acc64 ? dacc[i][j][v] : (double)acc[i][j][v], alpha, overflow);
      }
}

// BK = k values per step (32, 64 or 128).  Each thread moves BK/32 chunks of 8 values
// per operand per step; the global loads of step k0 + BK are issued before the MFMAs of
// step k0 and stored to LDS after them (register double buffering), so one load round
// trip is spread over BK / 16 MFMA k-slices.
template <bool BF, int BK, int LA, int LB>
__global__ __launch_bounds__(256) void k_gemm(const GemmArgs g, const TablePtrs tp) {
  constexpr int KC = BK / 32;   // 8-value chunks per thread per operand
  constexpr int LS = BK + 8;    // LDS row stride (halves)
  int bx = blockIdx.x, by = blockIdx.y, zb = blockIdx.z;
  if (g.xgrp > 0) xcd_remap(g.xgrp, bx, by, zb);
  const int b = g.ksplit > 1 ? zb / g.ksplit : zb;
  const GemmVariant& V = g.v[(b / g.vdiv) % g.nvar];
  const int m0 = by * 64, n0 = bx * 64;
  if (m0 >= V.M || n0 >= V.N) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int M = V.M, N = V.N;
  int kb0 = 0, K = V.K;  // k range [kb0, K) of this workgroup
  if (g.ksplit > 1) {
    const int kc = ((V.K + g.ksplit - 1) / g.ksplit + 31) & ~31;
    kb0 = (zb % g.ksplit) * kc;
    K = min(V.K, kb0 + kc);
  }

  __shared__ __align__(16) uint16_t sAh[64][LS];
  __shared__ __align__(16) uint16_t sBh[64][LS];
  __shared__ __align__(16) uint16_t sAl[BF ? 1 : 64][LS];
  __shared__ __align__(16) uint16_t sBl[BF ? 1 : 64][LS];

  const char* baseA = op_base(V.A, tp, b, g.vdiv, g.nvar);
  const char* baseB = op_base(V.B, tp, b, g.vdiv, g.nvar);
  const int lr = tid >> 2, lk = (tid & 3) * 8;

  float4_t acc[2][2];
  double dacc[2][2][4];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int v = 0; v < 4; ++v) dacc[i][j][v] = 0.0;
    }
  const int wm = (wave >> 1) * 32, wn = (wave & 1) * 32;
  const int fr = lane & 15, fk = 4 * (lane >> 4);

  constexpr bool acol = LA == 2, bcol = LB == 2;
  const int ar = acol ? (tid & 63) : lr, ak = acol ? (tid >> 6) * 8 : lk;
  const int br = bcol ? (tid & 63) : lr, bk = bcol ? (tid >> 6) * 8 : lk;
  float va[KC][8], vb[KC][8];
  uint16_t ra[KC][8], rb[KC][8];
  int ck_i = 0, overflow = 0;
  if (K > kb0) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      load8s<BF, LA>(V.A, baseA, m0 + ar, kb0 + ak + 32 * c, M, K, va[c], ra[c]);
      load8s<BF, LB>(V.B, baseB, n0 + br, kb0 + bk + 32 * c, N, K, vb[c], rb[c]);
    }
  }
  for (int k0 = kb0; k0 < K; k0 += BK) {
#pragma unroll
    for (int c = 0; c < KC; ++c) {
      if (BF) {
        *(uint4*)&sAh[ar][ak + 32 * c] = pack8(ra[c]);
        *(uint4*)&sBh[br][bk + 32 * c] = pack8(rb[c]);
      } else {
        uint16_t ah[8], al[8], bh[8], bl[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const _Float16 xa = (_Float16)va[c][i], xb = (_Float16)vb[c][i];
          ah[i] = __builtin_bit_cast(uint16_t, xa);
          bh[i] = __builtin_bit_cast(uint16_t, xb);
          al[i] = __builtin_bit_cast(uint16_t, (_Float16)(va[c][i] - (float)xa));
          bl[i] = __builtin_bit_cast(uint16_t, (_Float16)(vb[c][i] - (float)xb));
        }
        *(uint4*)&sAh[ar][ak + 32 * c] = pack8(ah);
        *(uint4*)&sBh[br][bk + 32 * c] = pack8(bh);
        *(uint4*)&sAl[ar][ak + 32 * c] = pack8(al);
        *(uint4*)&sBl[br][bk + 32 * c] = pack8(bl);
      }
    }
    __syncthreads();
    if (k0 + BK < K) {
#pragma unroll
      for (int c = 0; c < KC; ++c) {
        load8s<BF, LA>(V.A, baseA, m0 + ar, k0 + BK + ak + 32 * c, M, K, va[c], ra[c]);
        load8s<BF, LB>(V.B, baseB, n0 + br, k0 + BK + bk + 32 * c, N, K, vb[c], rb[c]);
      }
    }
#pragma unroll
    for (int ks = 0; ks < BK; ks += 16) {
#pragma unroll
      for (int i = 0; i < 2; ++i) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          if (BF) {
            const short4_t a = *(const short4_t*)&sAh[wm + 16 * i + fr][ks + fk];
            const short4_t bb = *(const short4_t*)&sBh[wn + 16 * j + fr][ks + fk];
            acc[i][j] = mfma16bf(a, bb, acc[i][j]);
          } else {
            const half4_t ah = *(const half4_t*)&sAh[wm + 16 * i + fr][ks + fk];
            const half4_t bh = *(const half4_t*)&sBh[wn + 16 * j + fr][ks + fk];
            const half4_t al = *(const half4_t*)&sAl[wm + 16 * i + fr][ks + fk];
            const half4_t bl = *(const half4_t*)&sBl[wn + 16 * j + fr][ks + fk];
            acc[i][j] = mfma16(ah, bh, acc[i][j]);
            acc[i][j] = mfma16(ah, bl, acc[i][j]);
            acc[i][j] = mfma16(al, bh, acc[i][j]);
          }
        }
      }
    }
    __syncthreads();
    const bool ckpt = ck_i < g.nck && k0 + BK == g.ck[ck_i];
    if (g.acc64 && (((k0 - kb0 + BK) & 255) == 0 || k0 + BK >= K || ckpt)) {
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) {
#pragma unroll
          for (int v = 0; v < 4; ++v) dacc[i][j][v] += (double)acc[i][j][v];
          acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
        }
    }
    if (ckpt) {  // partial result up to this k, stored below the final one
      gemm_epilogue(g, b, m0 + wm, n0 + wn, fk, fr, M, N, acc, dacc, (int64_t)(ck_i - g.nck) * g.ck_stride, overflow);
      ++ck_i;
    }
  }
  if (g.ksplit > 1) {  // raw partial sums of this k slice
    const int64_t pbase = (int64_t)zb * g.pm * g.pn;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int m = m0 + wm + 16 * i + fk + v, n = n0 + wn + 16 * j + fr;
          if (m >= M || n >= N) continue;
          if (g.acc64) ((double*)g.scratch)[pbase + (int64_t)m * g.pn + n] = dacc[i][j][v];
          else ((float*)g.scratch)[pbase + (int64_t)m * g.pn + n] = acc[i][j][v];
        }
    return;
  }
  gemm_epilogue(g, b, m0 + wm, n0 + wn, fk, fr, M, N, acc, dacc, 0, overflow);
  if (overflow && g.flags) atomicOr(g.flags, 1);
}

// sum of the k-slice partials in slice order, then the epilogue of one output element
__global__ __launch_bounds__(256) void k_gemm_reduce(const GemmArgs g, int batch) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int64_t per = (int64_t)g.pm * g.pn;
  if (idx >= per * batch) return;
  const int b = (int)(idx / per);
  const int rem = (int)(idx - (int64_t)b * per);
  const int m = rem / g.pn, n = rem - m * g.pn;
  const GemmVariant& V = g.v[(b / g.vdiv) % g.nvar];
  if (m >= V.M || n >= V.N) return;
  double sum = 0.0;
  for (int sp = 0; sp < g.ksplit; ++sp) {
    const int64_t o = ((int64_t)b * g.ksplit + sp) * per + rem;
    sum += g.acc64 ? ((const double*)g.scratch)[o] : (double)((const float*)g.scratch)[o];
  }
  if (!g.acc64) sum = (double)(float)sum;  // the unsplit kernel's fp32 accumulator type
  const int cb = b / g.cbdiv;
  const int64_t off = (int64_t)cb * g.csb1 + (int64_t)(b - cb * g.cbdiv) * g.csb2 + (int64_t)m * g.csm +
                      (int64_t)n * g.csn;
  int overflow = 0;
  store_out(g, off, sum, batch_alpha(g, b), overflow);
  if (overflow && g.flags) atomicOr(g.flags, 1);
}

// 4 values (row r, k .. k+3) of an operand widened to fp64; loads issued back to back
__device__ __forceinline__ void load4_f64(const GemmOperand& o, const char* base, int r, int k, int R, int K,
                                          double (&v)[4]) {
  int64_t off[4];
  bool ok[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    ok[i] = r < R && k + i < K;
    off[i] = ok[i] ? op_offset(o, r, k + i) : 0;
  }
  if (o.type == 3) {
    double t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = ((const double*)base)[off[i]];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ok[i] ? t[i] : 0.0;
  } else if (o.type == 0) {
    float t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = ((const float*)base)[off[i]];
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ok[i] ? (double)t[i] : 0.0;
  } else {
    uint16_t t[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) t[i] = ((const uint16_t*)base)[off[i]];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint16_t u = ok[i] ? t[i] : (uint16_t)0;
      v[i] = o.type == 1 ? (double)bf16_to_f32(u) : (double)__builtin_bit_cast(_Float16, u);
    }
  }
}

// fp64 tiles: 64 x 64 outputs per block, 4 x 4 per thread, k step 16
__global__ __launch_bounds__(256) void k_gemm_f64(const GemmArgs g, const TablePtrs tp) {
  const int b = blockIdx.z;
  const GemmVariant& V = g.v[(b / g.vdiv) % g.nvar];
  const int m0 = blockIdx.y * 64, n0 = blockIdx.x * 64;
  if (m0 >= V.M || n0 >= V.N) return;
  const int tid = threadIdx.x;
  const int M = V.M, N = V.N, K = V.K;
  __shared__ double sA[16][65];
  __shared__ double sB[16][65];
  const char* baseA = op_base(V.A, tp, b, g.vdiv, g.nvar);
  const char* baseB = op_base(V.B, tp, b, g.vdiv, g.nvar);
  const int lr = tid & 63, lk = (tid >> 6) * 4;
  const int tr = (tid >> 4) * 4, tc = (tid & 15) * 4;
  double acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = 0.0;
  for (int k0 = 0; k0 < K; k0 += 16) {
    {
      double ta[4], tb[4];
      load4_f64(V.A, baseA, m0 + lr, k0 + lk, M, K, ta);
      load4_f64(V.B, baseB, n0 + lr, k0 + lk, N, K, tb);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        sA[lk + i][lr] = ta[i];
        sB[lk + i][lr] = tb[i];
      }
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      double a[4], bb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        a[i] = sA[kk][tr + i];
        bb[i] = sB[kk][tc + i];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fma(a[i], bb[j], acc[i][j]);
    }
    __syncthreads();
  }
  const double alpha = batch_alpha(g, b);
  const int cb = b / g.cbdiv;
  const int64_t cbase = (int64_t)cb * g.csb1 + (int64_t)(b - cb * g.cbdiv) * g.csb2;
  int overflow = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int m = m0 + tr + i, n = n0 + tc + j;
      if (m >= M || n >= N) continue;
      store_out(g, cbase + (int64_t)m * g.csm + (int64_t)n * g.csn, acc[i][j], alpha, overflow);
    }
  if (overflow && g.flags) atomicOr(g.flags, 1);
}

static int pick_lmode(const GemmOperand& o, int K, bool split_or_bf) {
  if (!split_or_bf || o.type == 3) return 0;
  const int64_t vec = o.type == 0 ? 4 : 8;  // elements per 16 bytes
  auto al = [&](int64_t x) { return x % vec == 0; };
  const bool kfull = o.ksh >= 3;
  if (o.sk2 == 1 && kfull && K % 8 == 0 && al(o.sk1) && al(o.sr1) && al(o.sr2) && al(o.sb1) && al(o.sb2) &&
      al(o.off0) && (o.tbl || ((uintptr_t)o.p % 16) == 0))
    return 1;
  if (o.sr2 == 1 && o.rsh >= 6 && o.ksh >= 30) return 2;
  return 0;
}

template <bool BF, int BK>
static void launch_k(const GemmArgs& g, const TablePtrs& tp, dim3 grid, int la, int lb, hipStream_t s) {
  if (la == 1 && lb == 1) hipLaunchKernelGGL((k_gemm<BF, BK, 1, 1>), grid, dim3(256), 0, s, g, tp);
  else if (la == 1 && lb == 2) hipLaunchKernelGGL((k_gemm<BF, BK, 1, 2>), grid, dim3(256), 0, s, g, tp);
  else if (la == 2 && lb == 1) hipLaunchKernelGGL((k_gemm<BF, BK, 2, 1>), grid, dim3(256), 0, s, g, tp);
  else if (la == 2 && lb == 2) hipLaunchKernelGGL((k_gemm<BF, BK, 2, 2>), grid, dim3(256), 0, s, g, tp);
  else hipLaunchKernelGGL((k_gemm<BF, BK, 0, 0>), grid, dim3(256), 0, s, g, tp);
}

hipError_t launch_gemm(const GemmArgs& g0, const TablePtrs& tp, int batch, hipStream_t s) {
  GemmArgs g = g0;
  for (int v = 0; v < g.nvar; ++v) {
    g.v[v].A.lmode = pick_lmode(g.v[v].A, g.v[v].K, g.mode != GEMM_F64);
    g.v[v].B.lmode = pick_lmode(g.v[v].B, g.v[v].K, g.mode != GEMM_F64);
  }
  int maxM = 0, maxN = 0;
  for (int v = 0; v < g.nvar; ++v) {
    maxM = maxM > g.v[v].M ? maxM : g.v[v].M;
    maxN = maxN > g.v[v].N ? maxN : g.v[v].N;
  }
  if (batch <= 0 || maxM <= 0 || maxN <= 0) return hipSuccess;
  if (g.vdiv < 1 || g.nvar < 1 || g.nvar > 6 || g.nck < 0 || g.nck > 3) return hipErrorInvalidValue;
  if (g.nck > 0) {  // checkpoints: 32-aligned, increasing, inside K of every variant; not in fp64 mode
    if (g.mode == GEMM_F64) return hipErrorInvalidValue;
    for (int i = 0; i < g.nck; ++i) {
      if (g.ck[i] <= 0 || (g.ck[i] & 31) || (i > 0 && g.ck[i] <= g.ck[i - 1])) return hipErrorInvalidValue;
      for (int v = 0; v < g.nvar; ++v)
        if (g.ck[i] >= g.v[v].K) return hipErrorInvalidValue;
    }
  }
  if (batch > 65535 || (maxM + 63) / 64 > 65535) return hipErrorInvalidValue;
  dim3 grid((maxN + 63) / 64, (maxM + 63) / 64, batch);
  // k step: the largest of 128, 64, 32 not above the longest K that divides every checkpoint
  int maxK = 0;
  for (int v = 0; v < g.nvar; ++v) maxK = maxK > g.v[v].K ? maxK : g.v[v].K;
  // k step: 128 for long reductions (K >= 2048, where it halves the time), else 32 (the
  // smaller register and LDS footprint keeps more workgroups resident on short ones)
  int bk = maxK >= 2048 ? 128 : 32;
  for (int i = 0; i < g.nck; ++i)
    if (g.ck[i] % bk) bk = 32;
  // one load pattern per operand across the variants, else the generic loader
  int la = g.v[0].A.lmode, lb = g.v[0].B.lmode;
  for (int v = 1; v < g.nvar; ++v) {
    if (g.v[v].A.lmode != la) la = 0;
    if (g.v[v].B.lmode != lb) lb = 0;
  }
  if (la == 0 || lb == 0) la = lb = 0;
  // split-K for long reductions only: halve the slices while they are longer than 4096
  // values of k (and the partials fit the scratch).  Short slices do not pay: the fixed
  // cost of a workgroup outweighs a shorter k loop.
  g.ksplit = 1;
  g.pm = maxM;
  g.pn = maxN;
  if (g.scratch && g.nck == 0 && g.mode != GEMM_F64) {
    int64_t active = 0;  // workgroups inside their variant's M x N
    for (int b = 0; b < batch; ++b) {
      const GemmVariant& V = g.v[(b / g.vdiv) % g.nvar];
      active += (int64_t)((V.M + 63) / 64) * ((V.N + 63) / 64);
    }
    const int64_t esz = g.acc64 ? 8 : 4;
    int ks = 1;
    while (ks < 64 && maxK / ks > 4096 && active * ks < (1 << 16) &&
           (int64_t)batch * ks * 2 * maxM * maxN * esz <= g.scratch_bytes && (int64_t)batch * ks * 2 <= 65535)
      ks *= 2;
    g.ksplit = ks;
    if (ks > 1) {
      grid.z = batch * ks;
      const int kslice = (maxK + ks - 1) / ks;
      bk = kslice >= 2048 ? 128 : 32;
    }
  }
  if (g.xgrp > 0) {  // unit = xgrp batches (times the k slices of each)
    const int64_t units = (int64_t)batch / g.xgrp;
    if (batch % g.xgrp || units % 8) g.xgrp = 0;
    else g.xgrp *= g.ksplit;
  }
  if (g.mode == GEMM_F64) {
    g.xgrp = 0;
    hipLaunchKernelGGL(k_gemm_f64, grid, dim3(256), 0, s, g, tp);
  }
  else if (g.mode == GEMM_BF16) {
    if (bk == 128) launch_k<true, 128>(g, tp, grid, la, lb, s);
    else launch_k<true, 32>(g, tp, grid, la, lb, s);
  } else {
    if (bk == 128) launch_k<false, 128>(g, tp, grid, la, lb, s);
    else launch_k<false, 32>(g, tp, grid, la, lb, s);
  }
  if (g.ksplit > 1) {
    const int64_t total = (int64_t)batch * maxM * maxN;
    hipLaunchKernelGGL(k_gemm_reduce, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, s, g, batch);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- cores of all r_d chains
// G(t, cc)_n = U_T(t, cc)^T Y_n(r_d(cc)) for the five chains of table t and slice n in one
// workgroup (grid (N, tables)): the slice's Y rows (fp32, the first 32 feature
// components) and X rows (bf16) pass once, in 32-token chunks, through LDS as fp16 hi/lo
// pairs with the five U_T chunks; the 26 output tiles (rows 0..31; columns 0..15 of chains
// r_d = 4, 8, 16 of which the first r_d are stored, 0..31 of r_d = 32, 0..127 of r_d = D)
// accumulate hi*hi + hi*lo + lo*hi with fp16 MFMA in fp32, flushed to fp64 every 256
// tokens.  Output: the fp16 cores, [t][5][N][32][D] (row stride D); an fp16 overflow sets
// flags[0].  D = 128.  With Wh, the workgroup then forms the slice's rotated reconstruction
// operands of the five chains from the fp16 cores it stored (w_operands.h: the same
// arithmetic as k_prep_w), so that no separate launch is needed.
constexpr int CO_KC = 32;   // tokens per chunk
constexpr int CO_LS = 40;   // LDS row stride (halves)
constexpr int CO_TILES = 26;
// LDS: the main loop's staging, then (aliasing it) the cores of chains 0..3 as doubles at
// row stride r_d + 1 (conflict-free rows), the V rows, and the chain-4 core rows (stride 129)
constexpr int CO_STAGE = 2 * (5 * JOLT_KMAX + JOLT_KMAX + 128) * CO_LS * 2;
constexpr int CO_GC_OFF[4] = {0, 32 * 5, 32 * 5 + 32 * 9, 32 * 5 + 32 * 9 + 32 * 17};  // doubles
constexpr int CO_GC = 8 * (32 * 5 + 32 * 9 + 32 * 17 + 32 * 33);
constexpr int CO_VS = 4 * 128 * PW_VS;
constexpr int CO_G4 = 8 * 32 * 129;
constexpr int CO_SMEM = CO_STAGE > CO_GC + CO_VS + CO_G4 ? CO_STAGE : CO_GC + CO_VS + CO_G4;

__device__ __forceinline__ void co_tile(int t, int& cc, int& mt, int& nt) {
  // tiles 0..9: chains 0..3 (chain 3 has two column tiles); 10..25: chain 4
  if (t < 6) { cc = t >> 1; mt = t & 1; nt = 0; return; }
  if (t < 10) { cc = 3; mt = (t - 6) >> 1; nt = (t - 6) & 1; return; }
  cc = 4; mt = (t - 10) >> 3; nt = (t - 10) & 7;
}

// Epilogue of the core kernels: this thread's fp64 tile sums dacc -> the fp16 cores (and, with
// Wh, the slice's reconstruction operands).  The staging LDS is free when it runs.
__device__ void cores_epilogue(unsigned char* co_smem, const double (&dacc)[(CO_TILES + 3) / 4][4], int n, int tb,
                               int N, _Float16* __restrict__ G16, int32_t* flags, const float* __restrict__ V32,
                               const int8_t* __restrict__ signs, _Float16* __restrict__ Wh,
                               _Float16* __restrict__ Wl, int lD);

// Partial sums of the cores over the tokens [k_lo, k_hi) of a slice: with part, the fp64 tile
// sums go to part[((tb * N + n) * nks + ks) * CO_TILES * 256 + tile * 256 + v * 64 + lane]
// (ks = blockIdx.z) and the epilogue runs in k_cores_fin; without, here.
__global__ __launch_bounds__(256) void k_cores(const float* __restrict__ UT, const float* __restrict__ Y32,
                                               const TablePtrs tp, int N, int T, _Float16* __restrict__ G16,
                                               int32_t* flags, const float* __restrict__ V32,
                                               const int8_t* __restrict__ signs, _Float16* __restrict__ Wh,
                                               _Float16* __restrict__ Wl, int lD, int kslice,
                                               double* __restrict__ part) {
  constexpr int D = 128, KM = JOLT_KMAX;
  const int n = blockIdx.x, tb = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int ks = blockIdx.z, k_lo = ks * kslice, k_hi = min(T, k_lo + kslice);
  __shared__ __align__(16) unsigned char co_smem[CO_SMEM];
  typedef uint16_t ChainTile[5][KM][CO_LS];
  typedef uint16_t RowTile[KM][CO_LS];
  typedef uint16_t XTile[D][CO_LS];
  ChainTile& sUh = *(ChainTile*)co_smem;  // [chain][m][k]
  ChainTile& sUl = *(ChainTile*)(co_smem + sizeof(ChainTile));
  RowTile& sYh = *(RowTile*)(co_smem + 2 * sizeof(ChainTile));  // [j][k]
  RowTile& sYl = *(RowTile*)(co_smem + 2 * sizeof(ChainTile) + sizeof(RowTile));
  XTile& sXh = *(XTile*)(co_smem + 2 * sizeof(ChainTile) + 2 * sizeof(RowTile));  // [j][k]
  XTile& sXl = *(XTile*)(co_smem + 2 * sizeof(ChainTile) + 2 * sizeof(RowTile) + sizeof(XTile));
  static_assert(2 * sizeof(ChainTile) + 2 * sizeof(RowTile) + 2 * sizeof(XTile) == CO_STAGE, "staging size");
  const float* U = UT + (int64_t)tb * 5 * T * KM;             // [5][T][32]
  const float* Y = Y32 + ((int64_t)tb * N + n) * T * KM;      // [T][32]
  const uint16_t* X = (const uint16_t*)tp.p[tb] + (int64_t)n * T * D;  // [T][D]
  const int fr = lane & 15, fk = 4 * (lane >> 4);
  constexpr int TPW = (CO_TILES + 3) / 4;  // tiles per wave
  float4_t acc[TPW];
  double dacc[TPW][4];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    acc[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) dacc[i][v] = 0.0;
  }
  // staging: thread loads U (5 x 32 tokens x 32 = 5120 floats: 20 per thread), Y (1024: 4),
  // X (4096 bf16: 16)
  float ru[20], ry[4];
  uint16_t rx[16];
  auto load = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 5; ++i) {  // U chain i, token k0 + (tid >> 3), columns 4 (tid & 7) ..
      const float4 v = *(const float4*)(U + ((int64_t)i * T + k0 + (tid >> 3)) * KM + 4 * (tid & 7));
      ru[4 * i] = v.x; ru[4 * i + 1] = v.y; ru[4 * i + 2] = v.z; ru[4 * i + 3] = v.w;
    }
    {
      const float4 v = *(const float4*)(Y + (int64_t)(k0 + (tid >> 3)) * KM + 4 * (tid & 7));
      ry[0] = v.x; ry[1] = v.y; ry[2] = v.z; ry[3] = v.w;
    }
    {  // X token k0 + (tid >> 3), features 16 (tid & 7) ..
      const uint4* p = (const uint4*)(X + (int64_t)(k0 + (tid >> 3)) * D + 16 * (tid & 7));
      const uint4 a = p[0], b = p[1];
      const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        rx[2 * i] = (uint16_t)(w[i] & 0xFFFFu);
        rx[2 * i + 1] = (uint16_t)(w[i] >> 16);
      }
    }
  };
  auto split = [](float x, uint16_t& h, uint16_t& l) {
    const _Float16 hh = (_Float16)x;
    h = __builtin_bit_cast(uint16_t, hh);
    l = __builtin_bit_cast(uint16_t, (_Float16)(x - (float)hh));
  };
  load(k_lo);
  const int kk = tid >> 3;  // token within the chunk
  for (int k0 = k_lo; k0 < k_hi; k0 += CO_KC) {
#pragma unroll
    for (int i = 0; i < 5; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c) split(ru[4 * i + c], sUh[i][4 * (tid & 7) + c][kk], sUl[i][4 * (tid & 7) + c][kk]);
#pragma unroll
    for (int c = 0; c < 4; ++c) split(ry[c], sYh[4 * (tid & 7) + c][kk], sYl[4 * (tid & 7) + c][kk]);
#pragma unroll
    for (int c = 0; c < 16; ++c) split(__uint_as_float((uint32_t)rx[c] << 16), sXh[16 * (tid & 7) + c][kk],
                                       sXl[16 * (tid & 7) + c][kk]);
    __syncthreads();
    if (k0 + CO_KC < k_hi) load(k0 + CO_KC);
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + 4 * i;
      if (t >= CO_TILES) break;
      int cc, mt, nt;
      co_tile(t, cc, mt, nt);
#pragma unroll
      for (int ks = 0; ks < CO_KC; ks += 16) {
        const half4_t ah = *(const half4_t*)&sUh[cc][16 * mt + fr][ks + fk];
        const half4_t al = *(const half4_t*)&sUl[cc][16 * mt + fr][ks + fk];
        half4_t bh, bl;
        if (cc < 4) {
          bh = *(const half4_t*)&sYh[16 * nt + fr][ks + fk];
          bl = *(const half4_t*)&sYl[16 * nt + fr][ks + fk];
        } else {
          bh = *(const half4_t*)&sXh[16 * nt + fr][ks + fk];
          bl = *(const half4_t*)&sXl[16 * nt + fr][ks + fk];
        }
        acc[i] = mfma16(ah, bh, acc[i]);
        acc[i] = mfma16(ah, bl, acc[i]);
        acc[i] = mfma16(al, bh, acc[i]);
      }
    }
    __syncthreads();
    if (((k0 + CO_KC) & 255) == 0 || k0 + CO_KC >= k_hi) {
#pragma unroll
      for (int i = 0; i < TPW; ++i) {
#pragma unroll
        for (int v = 0; v < 4; ++v) dacc[i][v] += (double)acc[i][v];
        acc[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
      }
    }
  }
  if (part) {
    double* pp = part + (((int64_t)tb * N + n) * gridDim.z + ks) * CO_TILES * 256;
#pragma unroll
    for (int i = 0; i < TPW; ++i) {
      const int t = wave + 4 * i;
      if (t >= CO_TILES) break;
#pragma unroll
      for (int v = 0; v < 4; ++v) pp[t * 256 + v * 64 + lane] = dacc[i][v];
    }
    return;
  }
  // (the last barrier of the loop has passed: the staging may be overwritten)
  cores_epilogue(co_smem, dacc, n, tb, N, G16, flags, V32, signs, Wh, Wl, lD);
}

// The cores from the k slices' partial sums (added in slice order, fp64), then the epilogue.
__global__ __launch_bounds__(256) void k_cores_fin(const double* __restrict__ part, int nks, int N,
                                                   _Float16* __restrict__ G16, int32_t* flags,
                                                   const float* __restrict__ V32, const int8_t* __restrict__ signs,
                                                   _Float16* __restrict__ Wh, _Float16* __restrict__ Wl, int lD) {
  const int n = blockIdx.x, tb = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ __align__(16) unsigned char co_smem[CO_SMEM];
  constexpr int TPW = (CO_TILES + 3) / 4;
  double dacc[TPW][4];
  const double* pp = part + ((int64_t)tb * N + n) * nks * CO_TILES * 256;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave + 4 * i;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      double a = 0.0;
      if (t < CO_TILES)
        for (int q = 0; q < nks; ++q) a += pp[(int64_t)q * CO_TILES * 256 + t * 256 + v * 64 + lane];
      dacc[i][v] = a;
    }
  }
  cores_epilogue(co_smem, dacc, n, tb, N, G16, flags, V32, signs, Wh, Wl, lD);
}

__device__ void cores_epilogue(unsigned char* co_smem, const double (&dacc)[(CO_TILES + 3) / 4][4], int n, int tb,
                               int N, _Float16* __restrict__ G16, int32_t* flags, const float* __restrict__ V32,
                               const int8_t* __restrict__ signs, _Float16* __restrict__ Wh,
                               _Float16* __restrict__ Wl, int lD) {
  constexpr int D = 128, KM = JOLT_KMAX;
  constexpr int TPW = (CO_TILES + 3) / 4;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fk = 4 * (lane >> 4);
  double* gc = (double*)co_smem;                       // chains 0..3, [32][r_d + 1]
  float* vs = (float*)(co_smem + CO_GC);               // [D][PW_VS]
  double* g4 = (double*)(co_smem + CO_GC + CO_VS);     // [32][129], sign-flipped
  int overflow = 0;
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave + 4 * i;
    if (t >= CO_TILES) break;
    int cc, mt, nt;
    co_tile(t, cc, mt, nt);
    const int rd = cc < 4 ? (4 << cc) : D;
    _Float16* out = G16 + (((int64_t)tb * 5 + cc) * N + n) * KM * D;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int m = 16 * mt + fk + v, j = 16 * nt + fr;
      if (j >= rd) continue;
      const _Float16 h = f64_to_f16(dacc[i][v]);
      if (!(fabsf((float)h) <= 65504.f)) overflow = 1;
      out[m * D + j] = h;
      if (Wh) {
        const double hv = (double)h;
        if (cc < 4) gc[CO_GC_OFF[cc] + m * (rd + 1) + j] = hv;
        else g4[m * 129 + j] = signs[tb * D + j] < 0 ? -hv : hv;
      }
    }
  }
  if (Wh) {
    for (int idx = tid; idx < D * KM; idx += 256)
      vs[(idx >> 5) * PW_VS + (idx & 31)] = V32[(int64_t)tb * D * KM + idx];
    __syncthreads();
    const int64_t wb = ((int64_t)tb * 5 * N + n) * KM * D, cs = (int64_t)N * KM * D;  // chain stride
    prep_w_rows<4, 4>(gc + CO_GC_OFF[0], 5, vs, D, wb, Wh, Wl, overflow);
    prep_w_rows<8, 4>(gc + CO_GC_OFF[1], 9, vs, D, wb + cs, Wh, Wl, overflow);
    prep_w_rows<16, 4>(gc + CO_GC_OFF[2], 17, vs, D, wb + 2 * cs, Wh, Wl, overflow);
    prep_w_rows<32, 4>(gc + CO_GC_OFF[3], 33, vs, D, wb + 3 * cs, Wh, Wl, overflow);
    // lD = log2 D arrives at run time, so 1/sqrt(D) is computed as in k_prep_w (not folded)
    prep_w_hadamard(g4, 129, lD, wb + 4 * cs, Wh, Wl, overflow);
  }
  if (overflow && flags) atomicOr(flags, 1);
}

// token slices of the core kernel: enough workgroups to fill the chip, at least 1024 tokens
// (a multiple of 256) per slice
int cores_slices(int N, int T, int ntab) {
  int nks = 1;
  while ((int64_t)N * ntab * nks < 2048 && T / (2 * nks) >= 1024 && (T / (2 * nks)) % 256 == 0) nks *= 2;
  return nks;
}

hipError_t launch_cores(const float* UT, const float* Y32, const TablePtrs& tp, int N, int T, int D, int ntab,
                        _Float16* G16, int32_t* flags, const float* V32, const int8_t* signs, _Float16* Wh,
                        _Float16* Wl, double* part, hipStream_t s) {
  if (D != 128 || T % CO_KC || N < 1 || ntab < 1 || N > 65535 || ntab > 65535) return hipErrorInvalidValue;
  if (Wh && (!Wl || !V32 || !signs)) return hipErrorInvalidValue;
  const int nks = cores_slices(N, T, ntab);
  if (nks > 1) {
    if (!part) return hipErrorInvalidValue;
    hipLaunchKernelGGL(k_cores, dim3(N, ntab, nks), dim3(256), 0, s, UT, Y32, tp, N, T, G16, flags, V32, signs, Wh,
                       Wl, 7, T / nks, part);
    hipLaunchKernelGGL(k_cores_fin, dim3(N, ntab), dim3(256), 0, s, part, nks, N, G16, flags, V32, signs, Wh, Wl, 7);
  } else {
    hipLaunchKernelGGL(k_cores, dim3(N, ntab, 1), dim3(256), 0, s, UT, Y32, tp, N, T, G16, flags, V32, signs, Wh, Wl,
                       7, T, (double*)nullptr);
  }
  return hipGetLastError();
}

// ============================================================ feature projection
// Product of the exact mode's subspace iteration, P_b = M_b Q_b for the token Grams M_b
// ([T][T], fp32, at M + (b / div) s1 + (b % div) s2) and the bases Q_b ([T][64], fp32): the
// generic GEMM's split arithmetic (both operands as fp16 hi + lo, products hi hi, hi lo,
// lo hi by v_mfma_f32_16x16x32_f16, fp32 sums in ascending k).  Workgroup (64-row block q,
// problem b); wave w owns rows 64 q + 16 w .. + 15 and all 64 columns.  M's rows stream from
// HBM once (the A fragments straight into registers, the next k step's loaded during the
// current products); Q passes through a double-buffered LDS stage as fp16 hi / lo.  With W,
// the block's Gram partial P^T P (fp64 MFMA from the fp32 values stored, the four waves
// added in order) goes to W[(b nblk + q) 64 64 ..] with both triangles, so that the
// CholeskyQR that follows needs no Gram pass of its own.
__global__ __launch_bounds__(256) void k_mq(const float* __restrict__ M, int div, int64_t s1, int64_t s2,
                                            const float* __restrict__ Q, float* __restrict__ P, int T,
                                            double* __restrict__ W) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  typedef double d4 __attribute__((ext_vector_type(4)));
  const int q = blockIdx.x, b = blockIdx.y, nblk = gridDim.x;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  __shared__ __align__(16) h8 sQh[2][4][4][16], sQl[2][4][4][16];  // [buf][ct][g][li]
  __shared__ double red[4][256];
  const float* Mb = M + (int64_t)(b / div) * s1 + (int64_t)(b % div) * s2;
  const float* Qb = Q + (int64_t)b * T * 64;
  const float* mrow = Mb + (int64_t)(64 * q + 16 * w + li) * T + 8 * g;
  // staging item of thread tid: (ct, gq, lq) = (tid >> 6, (tid >> 4) & 3, tid & 15),
  // values Q[k0 + 8 gq + e][16 ct + lq], e < 8
  const int sct = tid >> 6, sg = (tid >> 4) & 3, sl = tid & 15;
  float qraw[8];
  auto fetch_q = [&](int k0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) qraw[e] = Qb[(int64_t)(k0 + 8 * sg + e) * 64 + 16 * sct + sl];
  };
  auto put_q = [&](int bf) {
    h8 hv, lv;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const _Float16 hh = (_Float16)qraw[e];
      hv[e] = hh;
      lv[e] = (_Float16)(qraw[e] - (float)hh);
    }
    sQh[bf][sct][sg][sl] = hv;
    sQl[bf][sct][sg][sl] = lv;
  };
  float4 ma[2];
  auto fetch_a = [&](int k0) {
    ma[0] = *(const float4*)(mrow + k0);
    ma[1] = *(const float4*)(mrow + k0 + 4);
  };
  float4_t acc[4];
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) acc[ct] = (float4_t){0.f, 0.f, 0.f, 0.f};
  fetch_q(0);
  put_q(0);
  fetch_a(0);
  __syncthreads();
  for (int k0 = 0; k0 < T; k0 += 32) {
    const int bf = (k0 >> 5) & 1;
    h8 ah, al;
    {
      const float v[8] = {ma[0].x, ma[0].y, ma[0].z, ma[0].w, ma[1].x, ma[1].y, ma[1].z, ma[1].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 hh = (_Float16)v[e];
        ah[e] = hh;
        al[e] = (_Float16)(v[e] - (float)hh);
      }
    }
    const bool more = k0 + 32 < T;  // uniform
    if (more) {
      fetch_a(k0 + 32);
      fetch_q(k0 + 32);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const h8 bh = sQh[bf][ct][g][li], bl = sQl[bf][ct][g][li];
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bh, acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah, bl, acc[ct], 0, 0, 0);
      acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al, bh, acc[ct], 0, 0, 0);
    }
    if (more) put_q(bf ^ 1);  // the other buffer: its readers passed the previous barrier
    __syncthreads();
  }
  // P rows 64 q + 16 w + 4 g + r, column 16 ct + li in register r of tile ct
  float* prow = P + ((int64_t)b * T + 64 * q + 16 * w + 4 * g) * 64 + li;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) prow[r * 64 + 16 * ct] = acc[ct][r];
  if (!W) return;
  // Gram partial of the block: tile (I, J), I <= J: sum over rows 4 kk + r of P[.][16 I + i]
  // P[.][16 J + j]; for fixed r the registers r of tiles I and J are the A (i, k = g) and
  // B (k = g, j) operands of v_mfma_f64_16x16x4f64 over the rows 4 g + r
  d4 gacc[10];
#pragma unroll
  for (int u = 0; u < 10; ++u) gacc[u] = (d4){0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    int u = 0;
#pragma unroll
    for (int I = 0; I < 4; ++I)
#pragma unroll
      for (int J = I; J < 4; ++J, ++u)
        gacc[u] = __builtin_amdgcn_mfma_f64_16x16x4f64((double)acc[I][r], (double)acc[J][r], gacc[u], 0, 0, 0);
  }
  double* out = W + ((int64_t)b * nblk + q) * 64 * 64;
  int u = 0;
#pragma unroll
  for (int I = 0; I < 4; ++I)
#pragma unroll
    for (int J = I; J < 4; ++J, ++u) {
#pragma unroll
      for (int r = 0; r < 4; ++r) red[w][r * 64 + lane] = gacc[u][r];
      __syncthreads();
      {  // element (16 I + 4 r + (l >> 4), 16 J + (l & 15)), r = tid >> 6, l = tid & 63
        const double v = ((red[0][tid] + red[1][tid]) + red[2][tid]) + red[3][tid];
        const int r = tid >> 6, l = tid & 63;
        const int i = 16 * I + 4 * r + (l >> 4), j = 16 * J + (l & 15);
        out[i * 64 + j] = v;
        if (I != J) out[j * 64 + i] = v;
      }
      __syncthreads();
    }
}

hipError_t launch_mq(const float* M, int div, int64_t s1, int64_t s2, const float* Q, float* P, int T, int batch,
                     double* W, hipStream_t s) {
  if (T < 64 || T % 64 || T / 64 > JOLT_GRAM_PARTS || batch < 1 || batch > 65535 || div < 1)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_mq, dim3(T / 64, batch), dim3(256), 0, s, M, div, s1, s2, Q, P, T, W);
  return hipGetLastError();
}

// Cores of the randomized token mode without a pass over the tensor.  The finder's last
// product is P = A^T Q (rows n r_d + j of chain r_d, 40 columns) for the orthonormal basis Q,
// and its token factor is U_T = Q V with V [40][32] the eigenvectors of P^T P, so
// G_n[m][j] = sum_t U_T[t][m] Y_n[t][j] = sum_c V[c][m] P[n r_d + j][c]: the same core in
// exact arithmetic, here a 40-term sum per value in fp64 from the working-precision P and V.
// Workgroup (slice n, table), the tile layout and epilogue of k_cores (D = 128): the five
// chains' V and the slice's 188 P rows are staged in LDS, each thread forms its tiles'
// values, then cores_epilogue stores the fp16 cores and the reconstruction operands.
constexpr int CR_P = 40;       // sketch columns
constexpr int CR_LS = CR_P + 1;  // LDS row stride of the P rows (floats)
constexpr int CR_ROWS = 4 + 8 + 16 + 32 + 128;
constexpr int CR_ROW0[5] = {0, 4, 12, 28, 60};

__global__ __launch_bounds__(256) void k_cores_rr(const float* __restrict__ V, const float* __restrict__ P,
                                                  int64_t p_chain, int N, _Float16* __restrict__ G16,
                                                  int32_t* flags, const float* __restrict__ V32,
                                                  const int8_t* __restrict__ signs, _Float16* __restrict__ Wh,
                                                  _Float16* __restrict__ Wl, int lD) {
  constexpr int D = 128, KM = JOLT_KMAX;
  constexpr int TPW = (CO_TILES + 3) / 4;
  const int n = blockIdx.x, tb = blockIdx.y, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fk = 4 * (lane >> 4);
  __shared__ __align__(16) unsigned char co_smem[CO_SMEM];
  __shared__ __align__(16) float vs[5][CR_P][KM];
  __shared__ float ps[CR_ROWS][CR_LS];
  for (int idx = tid; idx < 5 * CR_P * KM; idx += 256)
    (&vs[0][0][0])[idx] = V[((int64_t)tb * 5) * CR_P * KM + idx];
  for (int idx = tid; idx < CR_ROWS * CR_P; idx += 256) {
    const int r = idx / CR_P, c = idx - r * CR_P;
    const int cc = r < 4 ? 0 : r < 12 ? 1 : r < 28 ? 2 : r < 60 ? 3 : 4;
    const int rd = cc < 4 ? (4 << cc) : D, j = r - CR_ROW0[cc];
    ps[r][c] = P[((int64_t)tb * 5 + cc) * p_chain + ((int64_t)n * rd + j) * CR_P + c];
  }
  __syncthreads();
  double dacc[TPW][4];
#pragma unroll
  for (int i = 0; i < TPW; ++i) {
    const int t = wave + 4 * i;
#pragma unroll
    for (int v = 0; v < 4; ++v) dacc[i][v] = 0.0;
    if (t >= CO_TILES) continue;
    int cc, mt, nt;
    co_tile(t, cc, mt, nt);
    const int rd = cc < 4 ? (4 << cc) : D, j = 16 * nt + fr;
    if (j >= rd) continue;  // columns beyond r_d are not stored
    const float* prow = ps[CR_ROW0[cc] + j];
    for (int c = 0; c < CR_P; ++c) {
      const double pc = (double)prow[c];
      const float4 vv = *(const float4*)&vs[cc][c][16 * mt + fk];
      dacc[i][0] = fma((double)vv.x, pc, dacc[i][0]);
      dacc[i][1] = fma((double)vv.y, pc, dacc[i][1]);
      dacc[i][2] = fma((double)vv.z, pc, dacc[i][2]);
      dacc[i][3] = fma((double)vv.w, pc, dacc[i][3]);
    }
  }
  cores_epilogue(co_smem, dacc, n, tb, N, G16, flags, V32, signs, Wh, Wl, lD);
}

hipError_t launch_cores_rr(const float* V, const float* P, int64_t p_chain, int N, int D, int ntab, _Float16* G16,
                           int32_t* flags, const float* V32, const int8_t* signs, _Float16* Wh, _Float16* Wl,
                           hipStream_t s) {
  if (D != 128 || N < 1 || ntab < 1 || N > 65535 || ntab > 65535 || p_chain < (int64_t)N * D * CR_P)
    return hipErrorInvalidValue;
  if (!Wh || !Wl || !V32 || !signs) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_cores_rr, dim3(N, ntab), dim3(256), 0, s, V, P, p_chain, N, G16, flags, V32, signs, Wh, Wl, 7);
  return hipGetLastError();
}

// Y_n = X_n U_d[:, :32] for every slice of a table (fp32 working precision) with its fp16
// copy (the core of the r_T = T chain) and, optionally, the token-major copy
// YT[tk][j N + n] that the fused token Grams read.  Workgroup (16 tokens, table); wave w
// takes the slices n = w, w + 4, ...  The arithmetic is the generic GEMM's split mode,
// operation for operation: both operands split into fp16 hi + lo, per 16-wide k step the
// products hi*hi, hi*lo, lo*hi (v_mfma_f32_16x16x16f16) accumulated in fp32 in ascending
// k, so Y is the same to the bit.  The A operand of a step (16 tokens x 16 features) is read
// straight from the table; the result tile holds token 4 (lane >> 4) + r, column lane & 15
// in register r.  With YT (N <= 32) the 16 x 32N token-major rows are staged in LDS and
// written out whole.
#define PJ_TOK 16
#define PJ_NMAX 32
template <int D>
__global__ __launch_bounds__(256) void k_project(const TablePtrs tp, const float* __restrict__ Ud32, int N, int T,
                                                 float* __restrict__ Y32, _Float16* __restrict__ G16T,
                                                 float* __restrict__ YT, int32_t* __restrict__ flags) {
  const int t = blockIdx.y, tok0 = blockIdx.x * PJ_TOK;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, lk = lane >> 4;
  __shared__ __align__(16) _Float16 Us[2][JOLT_KMAX][D + 8];  // U_d^T as fp16 hi, lo
  __shared__ __align__(16) float YTs[PJ_TOK][JOLT_KMAX * PJ_NMAX + 4];
  const float* U = Ud32 + (int64_t)t * D * JOLT_KMAX;
  for (int idx = tid; idx < D * JOLT_KMAX; idx += 256) {
    const int f = idx / JOLT_KMAX, j = idx - f * JOLT_KMAX;
    const float u = U[idx];
    const _Float16 h = (_Float16)u;
    Us[0][j][f] = h;
    Us[1][j][f] = (_Float16)(u - (float)h);
  }
  __syncthreads();
  const uint16_t* X = (const uint16_t*)tp.p[t];
  int ovf = 0;
  for (int n = w; n < N; n += 4) {
    const uint16_t* xr = X + ((int64_t)n * T + tok0 + li) * D + 4 * lk;
    uint2 raw[D / 16];
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) raw[ks] = *(const uint2*)(xr + 16 * ks);
    float4_t acc[2] = {(float4_t){0.f, 0.f, 0.f, 0.f}, (float4_t){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const uint32_t wv[2] = {raw[ks].x, raw[ks].y};
      half4_t ah, al;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xv = bf16_to_f32((uint16_t)(wv[e >> 1] >> (16 * (e & 1))));
        const _Float16 hx = (_Float16)xv;
        ah[e] = hx;
        al[e] = (_Float16)(xv - (float)hx);
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        const half4_t bh = *(const half4_t*)&Us[0][16 * ct + li][16 * ks + 4 * lk];
        const half4_t bl = *(const half4_t*)&Us[1][16 * ct + li][16 * ks + 4 * lk];
        acc[ct] = mfma16(ah, bh, acc[ct]);
        acc[ct] = mfma16(ah, bl, acc[ct]);
        acc[ct] = mfma16(al, bh, acc[ct]);
      }
    }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int tl = 4 * lk + r, col = 16 * ct + li;
        const float y = acc[ct][r];
        const int64_t o = (((int64_t)t * N + n) * T + tok0 + tl) * JOLT_KMAX + col;
        Y32[o] = y;
        const _Float16 h = f64_to_f16((double)y);
        if (!(fabsf((float)h) <= 65504.f)) ovf = 1;
        G16T[o] = h;
        if (YT) YTs[tl][col * N + n] = y;
      }
  }
  if (ovf && flags) atomicOr(flags, 1);
  if (YT) {
    __syncthreads();
    const int rowlen = JOLT_KMAX * N;
    for (int idx = tid; idx < PJ_TOK * rowlen; idx += 256) {
      const int i = idx / rowlen, c = idx - i * rowlen;
      YT[((int64_t)t * T + tok0 + i) * rowlen + c] = YTs[i][c];
    }
  }
}

// The same projection without the token-major copy, 64 tokens per workgroup: the tensor's
// bf16 rows enter v_mfma_f32_16x16x32_bf16 straight from global memory (token i in lane
// i + 16 g, features 32 kb + 8 g .. + 7), U_d[:, :32] as three bf16 pieces u1 + u2 + u3
// staged once per workgroup, so every product is exact in fp32 (fp32 sums in ascending k).
// Column j of product tile ct is column 2 j + ct of U_d, so a lane ends up with two
// adjacent columns of each of its tokens (8-byte fp32 and 4-byte fp16 stores; 16 lanes
// cover a token's 32 columns).  Wave w owns tokens 16 w .. 16 w + 15 and loops over the
// slices, the next slice's rows loaded during the products; fp16 copy by one rounding of
// the fp32 value.
template <int D>
__global__ __launch_bounds__(256) void k_project4(const TablePtrs tp, const float* __restrict__ Ud32, int N, int T,
                                                  float* __restrict__ Y32, _Float16* __restrict__ G16T,
                                                  int32_t* __restrict__ flags) {
  typedef __bf16 b8 __attribute__((ext_vector_type(8)));
  constexpr int KB = D / 32;
  const int t = blockIdx.y, tok0 = blockIdx.x * 64;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  __shared__ __align__(16) b8 sU[3][KB][2][4][16];  // [piece][kb][ct][g][li]: U[32 kb + 8 g + e][2 li + ct]
  const float* U = Ud32 + (int64_t)t * D * JOLT_KMAX;
  for (int idx = tid; idx < KB * 2 * 4 * 16; idx += 256) {
    const int lq = idx & 15, gq = (idx >> 4) & 3, ct = (idx >> 6) & 1, kb = idx >> 7;
    b8 p0, p1, p2;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float u = U[(32 * kb + 8 * gq + e) * JOLT_KMAX + 2 * lq + ct];
      const __bf16 h1 = (__bf16)u;
      const float r1 = u - (float)h1;
      const __bf16 h2 = (__bf16)r1;
      p0[e] = h1;
      p1[e] = h2;
      p2[e] = (__bf16)(r1 - (float)h2);
    }
    sU[0][kb][ct][gq][lq] = p0;
    sU[1][kb][ct][gq][lq] = p1;
    sU[2][kb][ct][gq][lq] = p2;
  }
  __syncthreads();
  const uint16_t* X = (const uint16_t*)tp.p[t];
  uint4 xa[KB];
  auto load = [&](int n) {
    const uint16_t* xr = X + ((int64_t)n * T + tok0 + 16 * w + li) * D + 8 * g;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) xa[kb] = *(const uint4*)(xr + 32 * kb);
  };
  int ovf = 0;
  load(0);
  for (int n = 0; n < N; ++n) {
    b8 af[KB];
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) af[kb] = __builtin_bit_cast(b8, xa[kb]);
    if (n + 1 < N) load(n + 1);
    float4_t acc[2] = {(float4_t){0.f, 0.f, 0.f, 0.f}, (float4_t){0.f, 0.f, 0.f, 0.f}};
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
          acc[ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[kb], sU[pc][kb][ct][g][li], acc[ct], 0, 0, 0);
    // element (token 16 w + 4 g + r, column 2 li + ct)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t o = (((int64_t)t * N + n) * T + tok0 + 16 * w + 4 * g + r) * JOLT_KMAX + 2 * li;
      const float y0 = acc[0][r], y1 = acc[1][r];
      *(float2*)&Y32[o] = make_float2(y0, y1);
      const _Float16 h0 = (_Float16)y0, h1 = (_Float16)y1;
      if (!(fabsf((float)h0) <= 65504.f) || !(fabsf((float)h1) <= 65504.f)) ovf = 1;
      typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
      *(h2_t*)&G16T[o] = (h2_t){h0, h1};
    }
  }
  if (ovf && flags) atomicOr(flags, 1);
}

hipError_t launch_project(const TablePtrs& tp, const float* Ud32, int N, int T, int D, int ntab, float* Y32,
                          _Float16* G16T, float* YT, int32_t* flags, hipStream_t s) {
  if ((D != 64 && D != 128) || T % PJ_TOK || N < 1 || ntab < 1 || ntab > 65535 || T / PJ_TOK > 65535 ||
      (YT && N > PJ_NMAX))
    return hipErrorInvalidValue;
  if (!YT && T % 64 == 0) {  // no token-major copy: 64 tokens per workgroup
    const dim3 g4(T / 64, ntab);
    if (D == 128)
      hipLaunchKernelGGL(k_project4<128>, g4, dim3(256), 0, s, tp, Ud32, N, T, Y32, G16T, flags);
    else
      hipLaunchKernelGGL(k_project4<64>, g4, dim3(256), 0, s, tp, Ud32, N, T, Y32, G16T, flags);
    return hipGetLastError();
  }
  const dim3 grid(T / PJ_TOK, ntab);
  if (D == 128)
    hipLaunchKernelGGL(k_project<128>, grid, dim3(256), 0, s, tp, Ud32, N, T, Y32, G16T, YT, flags);
  else
    hipLaunchKernelGGL(k_project<64>, grid, dim3(256), 0, s, tp, Ud32, N, T, Y32, G16T, YT, flags);
  return hipGetLastError();
}

// ============================================================ feature Gram partials
// P[t][q] = X_q^T X_q for row chunk q (rows q R .. q R + R - 1 of table t viewed as
// [N T][D], bf16), one workgroup per (chunk, table).  The arithmetic is the generic GEMM's
// bf16 mode, operation for operation: v_mfma_f32_16x16x16bf16_1k over 16-row k blocks
// counted from the chunk start in ascending order (rows past the chunk end read as zero),
// exact products, fp32 accumulators flushed into fp64 after every 256 rows and at the
// end; so the partials are the same to the bit.  Only the 16 x 16 tiles on and above the
// diagonal are formed (the tile below sums the same exact products in the same order as
// its transpose): wave w < D/32 owns tile rows w and D/16 - 1 - w, D/16 + 1 tiles.  Rows
// pass through LDS as dwords (row 2p, row 2p + 1) of one feature, [feature][row pair],
// so an operand fragment (4 consecutive rows of one feature) is two dwords; each lane
// loads 2 features of a row, so a row is one coalesced 2D-byte read.
constexpr int FG_BK = 64;             // rows per LDS stage
constexpr int FG_RS = FG_BK / 2 + 1;  // LDS row stride in dwords (odd)

template <int D, int W>
__device__ __forceinline__ void fgram_stage(const uint32_t* sT, int lane, float4_t (&acc)[D / 16 + 1]) {
  constexpr int TD = D / 16;
  constexpr int W2 = TD - 1 - W;
  const int fr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int ks = 0; ks < FG_BK; ks += 16) {
    short4_t f[TD];  // fragments of the column tiles W .. TD - 1 (rows W and W2 among them)
#pragma unroll
    for (int j = W; j < TD; ++j) {
      const uint32_t* q = sT + (16 * j + fr) * FG_RS + ks / 2 + 2 * g;
      uint2 u;
      u.x = q[0];
      u.y = q[1];
      f[j] = __builtin_bit_cast(short4_t, u);
    }
#pragma unroll
    for (int j = W; j < TD; ++j) acc[j - W] = mfma16bf(f[W], f[j], acc[j - W]);
#pragma unroll
    for (int j = W2; j < TD; ++j) acc[TD - W + j - W2] = mfma16bf(f[W2], f[j], acc[TD - W + j - W2]);
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_fgram(const TablePtrs tp, int64_t rows, int nchunk, double* parts) {
  constexpr int TD = D / 16, NTW = TD + 1;
  constexpr int PPP = 512 / D;          // row pairs per load pass
  constexpr int NP = (FG_BK / 2) / PPP;  // load passes per stage
  __shared__ uint32_t sT[2][D * FG_RS];
  const int q = blockIdx.x, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const uint32_t* X = (const uint32_t*)tp.p[t] + (int64_t)q * rows * (D / 2);
  const int f2 = tid % (D / 2), pp = tid / (D / 2);  // feature pair, first row pair
  uint32_t ld[NP][2];
  auto load = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int64_t r = k0 + 2 * (pp + i * PPP);
      ld[i][0] = r < rows ? X[r * (D / 2) + f2] : 0u;
      ld[i][1] = r + 1 < rows ? X[(r + 1) * (D / 2) + f2] : 0u;
    }
  };
  float4_t acc[NTW];
  double dacc[NTW][4];
#pragma unroll
  for (int i = 0; i < NTW; ++i) {
    acc[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int v = 0; v < 4; ++v) dacc[i][v] = 0.0;
  }
  load(0);
  int buf = 0;
  for (int64_t k0 = 0; k0 < rows; k0 += FG_BK) {
    uint32_t* st = sT[buf];
#pragma unroll
    for (int i = 0; i < NP; ++i) {
      const int p = pp + i * PPP;
      const uint32_t a = ld[i][0], b = ld[i][1];
      st[(2 * f2) * FG_RS + p] = (a & 0xFFFFu) | (b << 16);
      st[(2 * f2 + 1) * FG_RS + p] = (a >> 16) | (b & 0xFFFF0000u);
    }
    __syncthreads();  // (a stage's buffer is rewritten two stages later, past this barrier)
    if (k0 + FG_BK < rows) load(k0 + FG_BK);
    if (wave < TD / 2) {
      switch (wave) {
        case 0: fgram_stage<D, 0>(st, lane, acc); break;
        case 1: fgram_stage<D, 1>(st, lane, acc); break;
        case 2: if constexpr (TD / 2 > 2) fgram_stage<D, 2>(st, lane, acc); break;
        default: if constexpr (TD / 2 > 3) fgram_stage<D, 3>(st, lane, acc); break;
      }
      if (((k0 + FG_BK) & 255) == 0 || k0 + FG_BK >= rows) {
#pragma unroll
        for (int i = 0; i < NTW; ++i) {
#pragma unroll
          for (int v = 0; v < 4; ++v) dacc[i][v] += (double)acc[i][v];
          acc[i] = (float4_t){0.f, 0.f, 0.f, 0.f};
        }
      }
    }
    buf ^= 1;
  }
  if (wave >= TD / 2) return;
  double* P = parts + ((int64_t)t * nchunk + q) * D * D;
  const int fr = lane & 15, g = lane >> 4;
#pragma unroll
  for (int s = 0; s < NTW; ++s) {
    // tile s of this wave: row tile w, columns w .. TD - 1, then row tile TD - 1 - w
    const int i = s < TD - wave ? wave : TD - 1 - wave;
    const int j = s < TD - wave ? wave + s : (TD - 1 - wave) + (s - (TD - wave));
#pragma unroll
    for (int v = 0; v < 4; ++v) P[(int64_t)(16 * i + 4 * g + v) * D + 16 * j + fr] = dacc[s][v];
  }
}

hipError_t launch_fgram(const TablePtrs& tp, int64_t rows, int D, int nchunk, int ntab, double* parts,
                        hipStream_t s) {
  if ((D != 64 && D != 128) || rows < 1 || nchunk < 1 || nchunk > 65535 || ntab < 1 || ntab > 65535)
    return hipErrorInvalidValue;
  const dim3 grid(nchunk, ntab);
  if (D == 128)
    hipLaunchKernelGGL(k_fgram<128>, grid, dim3(256), 0, s, tp, rows, nchunk, parts);
  else
    hipLaunchKernelGGL(k_fgram<64>, grid, dim3(256), 0, s, tp, rows, nchunk, parts);
  return hipGetLastError();
}

// ============================================================ token Gram of the tensor
// M = s sum_n X_n X_n^T (T x T per table, fp32) for bf16 X [N][T][128], s the power-of-two
// scale of the table's norm (as the generic GEMM applies it).  Work unit = one 128 x 128
// output tile (I, J), I <= J, of one table over a contiguous range of slices n (part p of S,
// S chosen on the host so that the units fill two workgroups per CU); four waves, wave
// (wr, wc) the 64 x 64 block of rows 64 wr.. and columns 64 wc...  The k axis of a slice
// (128 features) goes through LDS in two stages of 64: the rows 128 I .. and 128 J .. of a
// stage sit in LDS as 128-byte rows whose 16-byte chunks are permuted by an XOR of the row
// (the 16 rows of a fragment read, and the two rows of 16 lanes' stores, fall on distinct
// banks), double-buffered.  Each stage's rows are loaded into registers two stages ahead
// and stored into the free buffer after the current stage's products (one barrier per
// stage).  At 64 KB of LDS two workgroups share a CU, so every SIMD holds two waves.
// Fragments: A(i, k) = X_n[128 I + 64 wr + 16 a + i][k] and B(k, j) = X_n[128 J + 64 wc +
// 16 b + j][k], both row-major along k, 8 consecutive k per lane (v_mfma_f32_16x16x32_bf16:
// exact products, each 32-term sum added to the part's running fp32 totals).  With S > 1
// every part stores its totals in the
// fragment layout and k_tgram_fin, the next launch on the stream, adds the S parts in the
// order p = 0 .. S - 1 and stores the tile; with S = 1 the unit stores it.  A tile goes out
// with its mirror (J, I), transposed through LDS with row-contiguous stores.  Tiles of one
// table run on one XCD when the table count is a multiple of 8 (the shared rows stay in
// that XCD's L2).
constexpr int TG_TILE = 128;
constexpr int TG_KS = 64;                  // k per LDS stage (one 128-byte row run)
constexpr int TG_PANEL = TG_TILE * TG_KS;  // bf16 per panel buffer
typedef __bf16 bf16x8_g __attribute__((ext_vector_type(8)));
typedef unsigned int u32x4_g __attribute__((ext_vector_type(4)));
constexpr int TG_TS = 132;  // row stride (fp32) of the transposed tile in LDS
constexpr int TG_LDS = TG_TILE * TG_TS * 2 > 4 * TG_PANEL ? TG_TILE * TG_TS * 2 : 4 * TG_PANEL;  // bf16 units

// bf16 offset of chunk c (8 k values) of row r in a panel buffer
__device__ __forceinline__ int tg_off(int r, int c) { return r * TG_KS + ((c ^ ((r >> 1) & 7)) << 3); }

// Parts per tile: the S in 1..4 (S <= N) with the least estimated time, the busiest CU's
// units (two per CU on 256 CUs) times the part size, plus a tenth per extra part for the
// partial sums' traffic
int tgram_splits(int N, int T, int nt) {
  const int64_t tiles = T / TG_TILE, units = tiles * (tiles + 1) / 2 * nt;
  int best = 1;
  double bt = 1e300;
  for (int S = 1; S <= 4 && S <= N; ++S) {
    const int64_t per_cu = (units * S + 255) / 256;
    const double t = (double)per_cu / S * (1.0 + 0.1 * (S - 1));
    if (t < bt - 1e-12) {
      bt = t;
      best = S;
    }
  }
  return best;
}

// a finished 128 x 128 tile (fragment layout of the four waves) and its mirror
template <bool DIAG>
__device__ __forceinline__ void tgram_store(uint16_t* lds, const float4_t (&tot)[4][4], int T, int I, int J, float sc,
                                            float* out) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4, wr = wave >> 1, wc = wave & 1;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = TG_TILE * I + 64 * wr + 16 * a + 4 * lk + r, col = TG_TILE * J + 64 * wc + 16 * b + li;
        out[(int64_t)row * T + col] = tot[a][b][r] * sc;
      }
  if (!DIAG) {  // the mirror tile (J, I), transposed through LDS (free after the last barrier)
    float* Ts = (float*)lds;  // [128][TG_TS]: Ts[c][r] = tile(r, c)
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b)
#pragma unroll
        for (int r = 0; r < 4; ++r) Ts[(64 * wc + 16 * b + li) * TG_TS + 64 * wr + 16 * a + 4 * lk + r] = tot[a][b][r] * sc;
    __syncthreads();
    for (int idx = tid; idx < TG_TILE * TG_TILE / 4; idx += 256) {
      const int c = idx >> 5, r4 = (idx & 31) * 4;
      const float4_t v = *(const float4_t*)&Ts[c * TG_TS + r4];
      *(float4_t*)&out[(int64_t)(TG_TILE * J + c) * T + TG_TILE * I + r4] = v;
    }
  }
}

// one unit; DIAG: I == J (one panel serves both operands)
template <bool DIAG>
__device__ __forceinline__ void tgram_tile(uint16_t* lds, const uint16_t* X, int T, int I, int J, int n0, int n1,
                                           float sc, float* out, float* part) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4, wr = wave >> 1, wc = wave & 1;
  uint16_t* sA = lds;                 // [2][TG_PANEL]
  uint16_t* sB = lds + 2 * TG_PANEL;  // [2][TG_PANEL]
  // loader: thread t moves chunk t % 8 of rows t / 8 + 32 q (q < 4) of a stage (8 consecutive
  // lanes read one row's 128-byte run); the XOR of the chunk is the same for every q
  const int r0 = tid >> 3, ch = tid & 7;
  const int so = tg_off(r0, ch);
  const uint16_t* ga = X + (int64_t)(I * TG_TILE + r0) * 128 + ch * 8;
  const uint16_t* gb = X + (int64_t)(J * TG_TILE + r0) * 128 + ch * 8;
  const int64_t slice = (int64_t)T * 128;
  const int nst = 2 * (n1 - n0);  // even, >= 2
  auto koff = [&](int s) { return (int64_t)(n0 + (s >> 1)) * slice + (s & 1) * TG_KS; };
  auto load = [&](u32x4_g (&ra)[4], u32x4_g (&rb)[4], int s) {
    const int64_t ko = koff(s);
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      ra[q] = *(const u32x4_g*)(ga + ko + q * 32 * 128);
      if (!DIAG) rb[q] = *(const u32x4_g*)(gb + ko + q * 32 * 128);
    }
  };
  auto store = [&](const u32x4_g (&ra)[4], const u32x4_g (&rb)[4], int buf) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      *(u32x4_g*)&sA[buf * TG_PANEL + so + q * 32 * TG_KS] = ra[q];
      if (!DIAG) *(u32x4_g*)&sB[buf * TG_PANEL + so + q * 32 * TG_KS] = rb[q];
    }
  };
  // fragment offsets: row 64 w + 16 a + li, chunk 4 st + lk, XOR (li >> 1) & 7
  const int swz = (li >> 1) & 7;
  const int fa = (64 * wr + li) * TG_KS, fb = (64 * wc + li) * TG_KS;
  float4_t tot[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) tot[a][b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  // the stage's fragments of both 32-deep steps are read first, so that the LDS reads of
  // the second step overlap the products of the first
  auto compute = [&](int buf) {
    const uint16_t* pa = &sA[buf * TG_PANEL + fa];
    const uint16_t* pb = DIAG ? &sA[buf * TG_PANEL + fb] : &sB[buf * TG_PANEL + fb];
    bf16x8_g af[2][4], bf[2][4];
#pragma unroll
    for (int st = 0; st < 2; ++st) {
      const int co = ((4 * st + lk) ^ swz) << 3;
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        af[st][a] = *(const bf16x8_g*)(pa + 16 * a * TG_KS + co);
        bf[st][a] = *(const bf16x8_g*)(pb + 16 * a * TG_KS + co);
      }
    }
#pragma unroll
    for (int st = 0; st < 2; ++st)
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
          tot[a][b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[st][a], bf[st][b], tot[a][b], 0, 0, 0);
  };
  u32x4_g ra0[4], rb0[4], ra1[4], rb1[4];
  load(ra0, rb0, 0);
  load(ra1, rb1, 1);
  store(ra0, rb0, 0);
  __syncthreads();
  // The loads and stores run without conditions (past the end they repeat the last stage,
  // whose copy is never read): with no branch around them the compiler's wait counts let the
  // loads of two stages ahead stay in flight across each stage's LDS stores.
  for (int s = 0; s < nst; s += 2) {
    // stage s (buffer 0): stage s + 2 loaded, stage s + 1 stored
    load(ra0, rb0, min(s + 2, nst - 1));
    __builtin_amdgcn_sched_barrier(0);  // the loads go out before the stage's products
    compute(0);
    store(ra1, rb1, 1);
    __syncthreads();
    // stage s + 1 (buffer 1): stage s + 3 loaded, stage s + 2 stored
    load(ra1, rb1, min(s + 3, nst - 1));
    __builtin_amdgcn_sched_barrier(0);
    compute(1);
    store(ra0, rb0, 0);
    __syncthreads();
  }
  if (part) {  // one of several parts: its totals in the fragment layout [wave][a][b][lane]
    float4_t* mine = (float4_t*)part;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) mine[((wave * 4 + a) * 4 + b) * 64 + lane] = tot[a][b];
    return;
  }
  tgram_store<DIAG>(lds, tot, T, I, J, sc, out);
}

// decode of tile index u < tiles (tiles + 1) / 2 into (I, J), I <= J, row-major over the upper triangle
__device__ __forceinline__ void tgram_ij(int tiles, int u, int& I, int& J) {
  I = 0;
  while (u >= tiles - I) {  // row I of the upper triangle holds tiles - I tiles
    u -= tiles - I;
    ++I;
  }
  J = I + u;
}

__global__ __launch_bounds__(256, 2) void k_tgram(const TablePtrs tp, int N, int T, int nt, int S, const double* xn2,
                                                  float* M, int64_t msb, float* parts) {
  __shared__ __align__(16) uint16_t lds[TG_LDS];
  const int tiles = T / TG_TILE, ntile = tiles * (tiles + 1) / 2;  // tiles I <= J
  const int per = ntile * S;                                         // units of a table
  const int L = blockIdx.x;
  int tab, u;
  if (nt % 8 == 0) {  // XCD L % 8 takes tables x, x + 8, ...
    const int i = L >> 3;
    tab = (L & 7) + 8 * (i / per);
    u = i % per;
  } else {
    tab = L / per;
    u = L % per;
  }
  const int tile = u / S, p = u - tile * S;
  int I, J;
  tgram_ij(tiles, tile, I, J);
  const int n0 = (int)((int64_t)p * N / S), n1 = (int)((int64_t)(p + 1) * N / S);
  const uint16_t* X = (const uint16_t*)tp.p[tab];
  const float sc = gram_scale_from_norm(xn2[tab]);  // a power of two: exact
  float* out = M + (int64_t)tab * msb;
  float* part = S > 1 ? parts + ((int64_t)(tab * ntile + tile) * S + p) * TG_TILE * TG_TILE : nullptr;
  if (I == J)
    tgram_tile<true>(lds, X, T, I, J, n0, n1, sc, out, part);
  else
    tgram_tile<false>(lds, X, T, I, J, n0, n1, sc, out, part);
}

// The S parts of a tile added in the order p = 0 .. S - 1, scaled and stored with the mirror:
// one wave per 64 x 64 quadrant (wr, wc) of a tile, its block stored from the fragments and
// (off the diagonal) its mirror block transposed through LDS with row-contiguous stores
constexpr int TGF_TS = 65;  // row stride (fp32) of the transposed block
__global__ __launch_bounds__(64) void k_tgram_fin(int T, int nt, int S, const double* xn2, float* M, int64_t msb,
                                                  const float* parts) {
  __shared__ float Ts[64 * TGF_TS];
  const int tiles = T / TG_TILE, ntile = tiles * (tiles + 1) / 2;
  const int wave = blockIdx.x & 3, ut = blockIdx.x >> 2;
  const int tab = ut / ntile, tile = ut - tab * ntile;
  const int lane = threadIdx.x, li = lane & 15, lk = lane >> 4, wr = wave >> 1, wc = wave & 1;
  int I, J;
  tgram_ij(tiles, tile, I, J);
  const float4_t* src = (const float4_t*)(parts + (int64_t)ut * S * TG_TILE * TG_TILE);
  float4_t tot[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) tot[a][b] = src[((wave * 4 + a) * 4 + b) * 64 + lane];
  for (int q = 1; q < S; ++q) {
    src += TG_TILE * TG_TILE / 4;
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) tot[a][b] += src[((wave * 4 + a) * 4 + b) * 64 + lane];
  }
  const float sc = gram_scale_from_norm(xn2[tab]);
  float* out = M + (int64_t)tab * msb;
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int rl = 16 * a + 4 * lk + r, cl = 16 * b + li;
        const float v = tot[a][b][r] * sc;
        out[(int64_t)(TG_TILE * I + 64 * wr + rl) * T + TG_TILE * J + 64 * wc + cl] = v;
        Ts[cl * TGF_TS + rl] = v;
      }
  if (I == J) return;  // a diagonal tile is whole without mirrors
  __syncthreads();
  for (int idx = lane; idx < 64 * 16; idx += 64) {
    const int c = idx >> 4, r4 = (idx & 15) * 4;
    const float* t = &Ts[c * TGF_TS + r4];
    *(float4_t*)&out[(int64_t)(TG_TILE * J + 64 * wc + c) * T + TG_TILE * I + 64 * wr + r4] =
        (float4_t){t[0], t[1], t[2], t[3]};
  }
}

int64_t tgram_part_floats(int N, int T, int nt) {
  const int S = tgram_splits(N, T, nt);
  const int64_t tiles = T / TG_TILE, ntile = tiles * (tiles + 1) / 2;
  return S > 1 ? (int64_t)S * ntile * nt * TG_TILE * TG_TILE : 0;
}

// parts: tgram_part_floats(N, T, nt) floats (unused when that is 0)
hipError_t launch_tgram(const TablePtrs& tp, int N, int T, int D, int nt, const double* xn2, float* M, int64_t msb,
                        float* parts, hipStream_t s) {
  if (D != 128 || T < TG_TILE || T % TG_TILE || N < 1 || nt < 1 || nt > 64) return hipErrorInvalidValue;
  const int S = tgram_splits(N, T, nt);
  if (S > 1 && parts == nullptr) return hipErrorInvalidValue;
  const int64_t ntile = (int64_t)(T / TG_TILE) * (T / TG_TILE + 1) / 2 * nt;
  if (ntile * S > 0x7FFFFFFF || ntile * 4 > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tgram, dim3((unsigned)(ntile * S)), dim3(256), 0, s, tp, N, T, nt, S, xn2, M, msb, parts);
  if (S > 1) hipLaunchKernelGGL(k_tgram_fin, dim3((unsigned)(ntile * 4)), dim3(64), 0, s, T, nt, S, xn2, M, msb, parts);
  return hipGetLastError();
}

// ============================================================ nested token Grams of the projection
// M(r) = s sum_{j < r} sum_n y_{n,j} y_{n,j}^T for r = 4, 8, 16, 32 (T x T fp32 each), from
// the token-major copy YT [T][32][N] (fp32, N = 32) of Y = X U_d[:, :32]: one pass over
// k = (j, n), the running sums stored after j = 3, 7, 15 and 31.  Same tiling as k_tgram
// (128 x 128 tiles I <= J with their mirrors, four waves of 64 x 64); k block j is the 32
// values n of feature j, split on the way into LDS into fp16 hi = fp16(y) and lo =
// fp16(y - hi), and multiplied as hi hi + hi lo + lo hi (v_mfma_f32_16x16x32_f16, the
// generic GEMM's split arithmetic); each block's sums start from zero and are added to the
// running fp32 totals.  The mirror tiles go out through a transposed LDS tile of their own.
constexpr int TY_RS = 40;  // LDS row stride of a split panel in fp16 (80 B: 16 rows on distinct banks)
typedef _Float16 f16x8_g __attribute__((ext_vector_type(8)));

template <bool DIAG>
__device__ __forceinline__ void tgram_y_tile(_Float16 (*sP)[4][TG_TILE * TY_RS], float* Ts, const float* Y, int T,
                                             int I, int J, float sc, float* out, int64_t slot) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4, wr = wave >> 1, wc = wave & 1;
  // loader: thread t moves the 16-byte chunks c = t + 256 q (q < 4) of a block's panel: row
  // c / 8, values 4 (c % 8) .. + 3 of the row's 32 (8 consecutive lanes read one 128-byte run)
  const int r0 = tid >> 3, c4 = (tid & 7) * 4;
  const float* ga = Y + (int64_t)(I * TG_TILE + r0) * 1024 + c4;
  const float* gb = Y + (int64_t)(J * TG_TILE + r0) * 1024 + c4;
  float4_t ra[4], rb[4];
  auto split_store = [&](int buf, int pan, int r, const float4_t& v) {
    _Float16 h[4], l[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      h[e] = (_Float16)v[e];
      l[e] = (_Float16)(v[e] - (float)h[e]);
    }
    *(uint2*)&sP[buf][pan][r * TY_RS + c4] =
        make_uint2((uint32_t)__builtin_bit_cast(uint16_t, h[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[1]) << 16),
                   (uint32_t)__builtin_bit_cast(uint16_t, h[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, h[3]) << 16));
    *(uint2*)&sP[buf][pan + 1][r * TY_RS + c4] =
        make_uint2((uint32_t)__builtin_bit_cast(uint16_t, l[0]) | ((uint32_t)__builtin_bit_cast(uint16_t, l[1]) << 16),
                   (uint32_t)__builtin_bit_cast(uint16_t, l[2]) | ((uint32_t)__builtin_bit_cast(uint16_t, l[3]) << 16));
  };
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    ra[q] = *(const float4_t*)(ga + q * 32 * 1024);
    if (!DIAG) rb[q] = *(const float4_t*)(gb + q * 32 * 1024);
  }
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    split_store(0, 0, r0 + 32 * q, ra[q]);
    if (!DIAG) split_store(0, 2, r0 + 32 * q, rb[q]);
  }
  __syncthreads();
  float4_t tot[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) tot[a][b] = (float4_t){0.f, 0.f, 0.f, 0.f};
  for (int j = 0; j < JOLT_KMAX; ++j) {
    const int buf = j & 1;
    if (j + 1 < JOLT_KMAX) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        ra[q] = *(const float4_t*)(ga + (j + 1) * 32 + q * 32 * 1024);
        if (!DIAG) rb[q] = *(const float4_t*)(gb + (j + 1) * 32 + q * 32 * 1024);
      }
    }
    const int pbo = DIAG ? 0 : 2;
    f16x8_g ah[4], al[4], bh[4], bl[4];
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const int ro = (64 * wr + 16 * a + li) * TY_RS + 8 * lk, co = (64 * wc + 16 * a + li) * TY_RS + 8 * lk;
      ah[a] = *(const f16x8_g*)&sP[buf][0][ro];
      al[a] = *(const f16x8_g*)&sP[buf][1][ro];
      bh[a] = *(const f16x8_g*)&sP[buf][pbo][co];
      bl[a] = *(const f16x8_g*)&sP[buf][pbo + 1][co];
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < 4; ++b) {
        float4_t blk = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[a], bh[b], (float4_t){0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
        blk = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[a], bl[b], blk, 0, 0, 0);
        blk = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[a], bh[b], blk, 0, 0, 0);
        tot[a][b] += blk;
      }
    if (j + 1 < JOLT_KMAX) {
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        split_store(buf ^ 1, 0, r0 + 32 * q, ra[q]);
        if (!DIAG) split_store(buf ^ 1, 2, r0 + 32 * q, rb[q]);
      }
    }
    if (j == 3 || j == 7 || j == 15 || j == 31) {  // M(j + 1): this tile and its mirror
      float* o = out + (j == 3 ? 0 : j == 7 ? 1 : j == 15 ? 2 : 3) * slot;
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int rl = 64 * wr + 16 * a + 4 * lk + r, cl = 64 * wc + 16 * b + li;
            const float v = tot[a][b][r] * sc;
            o[(int64_t)(TG_TILE * I + rl) * T + TG_TILE * J + cl] = v;
            if (!DIAG) Ts[cl * TG_TS + rl] = v;
          }
      if (!DIAG) {
        __syncthreads();
        for (int idx = tid; idx < TG_TILE * TG_TILE / 4; idx += 256) {
          const int c = idx >> 5, r4 = (idx & 31) * 4;
          *(float4_t*)&o[(int64_t)(TG_TILE * J + c) * T + TG_TILE * I + r4] = *(const float4_t*)&Ts[c * TG_TS + r4];
        }
      }
    }
    __syncthreads();
  }
}

__global__ __launch_bounds__(256) void k_tgram_y(const float* YT, int T, int nt, const double* xn2, float* M,
                                                 int64_t msb) {
  __shared__ __align__(16) _Float16 sP[2][4][TG_TILE * TY_RS];  // [buffer][A hi, A lo, B hi, B lo]
  __shared__ __align__(16) float Ts[TG_TILE * TG_TS];
  const int tiles = T / TG_TILE, ntile = tiles * (tiles + 1) / 2;  // tiles I <= J
  const int L = blockIdx.x;
  int tab, tile;
  if (nt % 8 == 0) {  // XCD L % 8 takes tables x, x + 8, ...
    const int i = L >> 3;
    tab = (L & 7) + 8 * (i / ntile);
    tile = i % ntile;
  } else {
    tab = L / ntile;
    tile = L % ntile;
  }
  int I = 0;
  while (tile >= tiles - I) {
    tile -= tiles - I;
    ++I;
  }
  const int J = I + tile;
  const float* Y = YT + (int64_t)tab * T * 1024;
  const float sc = gram_scale_from_norm(xn2[tab]);
  float* out = M + (int64_t)tab * msb;
  if (I == J)
    tgram_y_tile<true>(sP, Ts, Y, T, I, J, sc, out, (int64_t)T * T);
  else
    tgram_y_tile<false>(sP, Ts, Y, T, I, J, sc, out, (int64_t)T * T);
}

hipError_t launch_tgram_y(const float* YT, int N, int T, int nt, const double* xn2, float* M, int64_t msb,
                          hipStream_t s) {
  if (N != 32 || T < TG_TILE || T % TG_TILE || nt < 1) return hipErrorInvalidValue;
  const int64_t grid = (int64_t)(T / TG_TILE) * (T / TG_TILE + 1) / 2 * nt;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(k_tgram_y, dim3((unsigned)grid), dim3(256), 0, s, YT, T, nt, xn2, M, msb);
  return hipGetLastError();
}

// ============================================================ X^T S of the randomized finder
// For the r_d = D chain the finder's A^T S is, per slice n, P_n = X_n^T S (D x 40), X_n the
// bf16 slice [T][D] and S [T][40] fp32.  One workgroup per (k slice of XS_KS tokens, slice,
// table) streams its tokens in chunks of 64 through LDS, as fp16 pairs (token 2p, 2p + 1) per
// feature and per sketch column, both operands split into fp16 hi + lo as in the generic
// GEMM's split mode (products hi hi, hi lo, lo hi, in that order).  MFMA 16x16x16
// accumulates in fp32 over the k slice; the partials are summed over the slices in order, in
// fp64, by k_xts_reduce.  Wave w owns feature tiles 2w, 2w + 1 (D = 128; w for D = 64) and
// the three 16-column tiles of the (padded) 48 sketch columns.
constexpr int XS_KS = 4096;  // tokens per k slice
constexpr int XS_P = 40;     // sketch columns
constexpr int XS_LS = 33;    // LDS row stride in dwords (32 token pairs + 1)

template <int D>
__global__ __launch_bounds__(256) void k_xts(const TablePtrs tp, const float* __restrict__ S, int64_t s_tab, int N,
                                             int T, int nks, float* __restrict__ part) {
  constexpr int RT = D / 64;  // feature tiles per wave
  const int ks = blockIdx.x, n = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint32_t sX[D * XS_LS], sXl[D * XS_LS];  // [f][pair] fp16 hi / lo of x (tokens 2p, 2p + 1)
  __shared__ uint32_t sSh[48 * XS_LS], sSl[48 * XS_LS];  // [c][pair] fp16 hi / lo of S
  const uint32_t* X = (const uint32_t*)tp.p[t] + (int64_t)n * T * (D / 2);  // [T][D/2] feature pairs
  const float* St = S + (int64_t)t * s_tab;
  const int k0 = ks * XS_KS, k1 = min(T, k0 + XS_KS);
  const int fr = lane & 15, g = lane >> 4;
  float4_t acc[RT][3];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto f16bits = [](float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v); };
  auto lo = [](float v) { return v - (float)(_Float16)v; };
  // the next chunk's X words and S values are loaded while the current chunk is multiplied
  constexpr int NQ = D / 16;                 // X word pairs per thread and chunk
  constexpr int NSI = (32 * 48 + 255) / 256;  // S (pair, column) items per thread and chunk
  uint32_t xa[NQ], xb[NQ];
  float sa[NSI], sb[NSI];
  auto load = [&](int c0) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int f2 = tid % (D / 2), pp = tid / (D / 2) + q * (512 / D), r = c0 + 2 * pp;
      xa[q] = r < k1 ? X[(int64_t)r * (D / 2) + f2] : 0u;
      xb[q] = r + 1 < k1 ? X[(int64_t)(r + 1) * (D / 2) + f2] : 0u;
    }
#pragma unroll
    for (int i = 0; i < NSI; ++i) {
      const int idx = tid + 256 * i, c = idx % 48, pp = idx / 48, r = c0 + 2 * pp;
      const bool ok = idx < 32 * 48 && c < XS_P;
      sa[i] = (ok && r < k1) ? St[(int64_t)r * XS_P + c] : 0.f;
      sb[i] = (ok && r + 1 < k1) ? St[(int64_t)(r + 1) * XS_P + c] : 0.f;
    }
  };
  if (k0 < k1) load(k0);
  for (int c0 = k0; c0 < k1; c0 += 64) {
#pragma unroll
    for (int q = 0; q < NQ; ++q) {
      const int f2 = tid % (D / 2), pp = tid / (D / 2) + q * (512 / D);
      const uint32_t a = xa[q], b = xb[q];
      const float a0 = __uint_as_float(a << 16), a1 = __uint_as_float(a & 0xFFFF0000u);
      const float b0 = __uint_as_float(b << 16), b1 = __uint_as_float(b & 0xFFFF0000u);
      sX[(2 * f2) * XS_LS + pp] = f16bits(a0) | (f16bits(b0) << 16);
      sX[(2 * f2 + 1) * XS_LS + pp] = f16bits(a1) | (f16bits(b1) << 16);
      sXl[(2 * f2) * XS_LS + pp] = f16bits(lo(a0)) | (f16bits(lo(b0)) << 16);
      sXl[(2 * f2 + 1) * XS_LS + pp] = f16bits(lo(a1)) | (f16bits(lo(b1)) << 16);
    }
#pragma unroll
    for (int i = 0; i < NSI; ++i) {
      const int idx = tid + 256 * i, c = idx % 48, pp = idx / 48;
      if (idx < 32 * 48) {
        sSh[c * XS_LS + pp] = f16bits(sa[i]) | (f16bits(sb[i]) << 16);
        sSl[c * XS_LS + pp] = f16bits(lo(sa[i])) | (f16bits(lo(sb[i])) << 16);
      }
    }
    __syncthreads();
    if (c0 + 64 < k1) load(c0 + 64);
#pragma unroll
    for (int kb = 0; kb < 64; kb += 16) {
      const int pq = kb / 2 + 2 * g;  // fragment: tokens kb + 4 g .. + 3 = pairs pq, pq + 1
      half4_t bh[3], bl[3];
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int c = 16 * j + fr;
        uint2 u, v;
        u.x = sSh[c * XS_LS + pq];
        u.y = sSh[c * XS_LS + pq + 1];
        v.x = sSl[c * XS_LS + pq];
        v.y = sSl[c * XS_LS + pq + 1];
        bh[j] = __builtin_bit_cast(half4_t, u);
        bl[j] = __builtin_bit_cast(half4_t, v);
      }
#pragma unroll
      for (int i = 0; i < RT; ++i) {
        const int f = 16 * (RT * wave + i) + fr;
        uint2 u, w;
        u.x = sX[f * XS_LS + pq];
        u.y = sX[f * XS_LS + pq + 1];
        w.x = sXl[f * XS_LS + pq];
        w.y = sXl[f * XS_LS + pq + 1];
        const half4_t ax = __builtin_bit_cast(half4_t, u), axl = __builtin_bit_cast(half4_t, w);
#pragma unroll
        for (int j = 0; j < 3; ++j) {
          acc[i][j] = mfma16(ax, bh[j], acc[i][j]);
          acc[i][j] = mfma16(ax, bl[j], acc[i][j]);
          acc[i][j] = mfma16(axl, bh[j], acc[i][j]);
        }
      }
    }
    __syncthreads();
  }
  // partial [t][n][ks][f][c]: result tile rows f = 16 rt + 4 g + v, columns c = 16 j + fr
  float* out = part + (((int64_t)t * N + n) * nks + ks) * D * XS_P;
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int f = 16 * (RT * wave + i) + 4 * g + v, c = 16 * j + fr;
        if (c < XS_P) out[f * XS_P + c] = acc[i][j][v];
      }
}

// The same products with four slices per workgroup and bf16 MFMA: the tensor is bf16, so its
// values enter v_mfma_f32_16x16x32_bf16 unchanged (transposed through LDS to feature rows of
// token pairs), and S enters as three bf16 pieces s1 + s2 + s3 (24 bits of the fp32 value,
// staged once for the four slices), so every product is exact in fp32.  Workgroup (k slice,
// group of 4 slices, table); wave w owns slice 4 grp + w: its D features (D / 16 row tiles)
// against the three 16-column tiles of the (padded) 48 sketch columns.  Chunks of 32 tokens;
// the next chunk is loaded during the products.  Partials as k_xts.
constexpr int XG = 4;          // slices per workgroup
constexpr int XC = 32;         // tokens per chunk
constexpr int XLS = XC + 8;    // LDS row stride (bf16 values)

template <int D>
__global__ __launch_bounds__(256) void k_xts4(const TablePtrs tp, const float* __restrict__ S, int64_t s_tab, int N,
                                              int T, int nks, float* __restrict__ part) {
  typedef __bf16 b8 __attribute__((ext_vector_type(8)));
  constexpr int RT = D / 16;  // feature tiles per wave
  const int ks = blockIdx.x, grp = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, g = lane >> 4;
  __shared__ __align__(16) uint16_t sX[XG][D][XLS];     // [slice][f][token]
  __shared__ __align__(16) uint16_t sS[3][48][XLS];     // [piece][c][token]
  const int n0 = grp * XG;
  const uint16_t* X = (const uint16_t*)tp.p[t] + (int64_t)n0 * T * D;  // slice s at + s T D
  const float* St = S + (int64_t)t * s_tab;
  const int k0 = ks * XS_KS, k1 = min(T, k0 + XS_KS);
  // items per chunk: X (slice, 8 features, token pair): 4 x D/8 x 16, token pairs on consecutive
  // lanes (consecutive LDS words); S (token pair, 4 columns): 16 x 10
  constexpr int NXI = XG * 16 * (D / 8) / 256;
  uint4 xa[NXI], xb[NXI];
  float4_t sa, sb;
  const float4_t z4 = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto load = [&](int c0) {
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int idx = tid + 256 * i, pp = idx & 15, f8 = (idx >> 4) % (D / 8), sl = (idx >> 4) / (D / 8);
      const int r = c0 + 2 * pp;
      const uint16_t* xr = X + ((int64_t)sl * T + r) * D + 8 * f8;
      xa[i] = r < k1 ? *(const uint4*)xr : make_uint4(0u, 0u, 0u, 0u);
      xb[i] = r + 1 < k1 ? *(const uint4*)(xr + D) : make_uint4(0u, 0u, 0u, 0u);
    }
    {
      const int pp = tid / 10, c4 = tid % 10, r = c0 + 2 * pp;
      const bool ok = tid < 160;
      sa = ok && r < k1 ? *(const float4_t*)(St + (int64_t)r * XS_P + 4 * c4) : z4;
      sb = ok && r + 1 < k1 ? *(const float4_t*)(St + (int64_t)(r + 1) * XS_P + 4 * c4) : z4;
    }
  };
  float4_t acc[RT][3];
#pragma unroll
  for (int i = 0; i < RT; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  // the padding columns 40..47 of S stay zero
  for (int idx = tid; idx < 3 * 8 * XLS; idx += 256) sS[idx / (8 * XLS)][40 + (idx / XLS) % 8][idx % XLS] = 0;
  if (k0 < k1) load(k0);
  for (int c0 = k0; c0 < k1; c0 += XC) {
#pragma unroll
    for (int i = 0; i < NXI; ++i) {
      const int idx = tid + 256 * i, pp = idx & 15, f8 = (idx >> 4) % (D / 8), sl = (idx >> 4) / (D / 8);
      const uint32_t wa[4] = {xa[i].x, xa[i].y, xa[i].z, xa[i].w}, wb[4] = {xb[i].x, xb[i].y, xb[i].z, xb[i].w};
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t va = (wa[e >> 1] >> (16 * (e & 1))) & 0xFFFFu, vb = (wb[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
        *(uint32_t*)&sX[sl][8 * f8 + e][2 * pp] = va | (vb << 16);
      }
    }
    if (tid < 160) {
      const int pp = tid / 10, c4 = tid % 10;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float a = sa[e], b = sb[e];
        const __bf16 a1 = (__bf16)a, b1 = (__bf16)b;
        const float ar = a - (float)a1, br = b - (float)b1;
        const __bf16 a2 = (__bf16)ar, b2 = (__bf16)br;
        const __bf16 a3 = (__bf16)(ar - (float)a2), b3 = (__bf16)(br - (float)b2);
        const int c = 4 * c4 + e;
        *(uint32_t*)&sS[0][c][2 * pp] =
            (uint32_t)__builtin_bit_cast(uint16_t, a1) | ((uint32_t)__builtin_bit_cast(uint16_t, b1) << 16);
        *(uint32_t*)&sS[1][c][2 * pp] =
            (uint32_t)__builtin_bit_cast(uint16_t, a2) | ((uint32_t)__builtin_bit_cast(uint16_t, b2) << 16);
        *(uint32_t*)&sS[2][c][2 * pp] =
            (uint32_t)__builtin_bit_cast(uint16_t, a3) | ((uint32_t)__builtin_bit_cast(uint16_t, b3) << 16);
      }
    }
    __syncthreads();
    if (c0 + XC < k1) load(c0 + XC);
    b8 bv[3][3];
#pragma unroll
    for (int pc = 0; pc < 3; ++pc)
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) bv[pc][ct] = *(const b8*)&sS[pc][16 * ct + li][8 * g];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) {
      const b8 av = *(const b8*)&sX[wave][16 * rt + li][8 * g];
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int pc = 0; pc < 3; ++pc)
          acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bv[pc][ct], acc[rt][ct], 0, 0, 0);
    }
    __syncthreads();
  }
  // partial [t][n][ks][f][c]: tile element (row f = 16 rt + 4 g + v, column c = 16 ct + li)
  const int n = n0 + wave;
  float* out = part + (((int64_t)t * N + n) * nks + ks) * D * XS_P;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int ct = 0; ct < 3; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int f = 16 * rt + 4 * g + v, c = 16 * ct + li;
        if (c < XS_P) out[f * XS_P + c] = acc[rt][ct][v];
      }
}

// P[t][n D + f][c] (row stride XS_P, table stride p_tab) = sum over k slices in order (fp64)
__global__ __launch_bounds__(256) void k_xts_reduce(const float* __restrict__ part, int N, int D, int nks,
                                                    float* __restrict__ P, int64_t p_tab) {
  const int t = blockIdx.y;
  const int64_t per = (int64_t)N * D * XS_P;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < per; idx += (int64_t)gridDim.x * 256) {
    const int64_t n = idx / ((int64_t)D * XS_P), r = idx - n * D * XS_P;  // r = f * XS_P + c
    const float* src = part + (((int64_t)t * N + n) * nks) * D * XS_P + r;
    double s = 0.0;
    for (int q = 0; q < nks; ++q) s += (double)src[(int64_t)q * D * XS_P];
    P[(int64_t)t * p_tab + idx] = (float)s;
  }
}

int xts_slices(int T) { return (T + XS_KS - 1) / XS_KS; }

hipError_t launch_xts(const TablePtrs& tp, const float* S, int64_t s_tab, int N, int T, int D, int ntab,
                      float* part, float* P, int64_t p_tab, hipStream_t s) {
  if ((D != 64 && D != 128) || T < 1 || T % 2 || N < 1 || N > 65535 || ntab < 1 || ntab > 65535)
    return hipErrorInvalidValue;
  const int nks = xts_slices(T);
  if (N % XG == 0 && (int64_t)nks * (N / XG) * ntab >= 512) {  // four slices per workgroup
    const dim3 g4(nks, N / XG, ntab);
    if (D == 128)
      hipLaunchKernelGGL(k_xts4<128>, g4, dim3(256), 0, s, tp, S, s_tab, N, T, nks, part);
    else
      hipLaunchKernelGGL(k_xts4<64>, g4, dim3(256), 0, s, tp, S, s_tab, N, T, nks, part);
  } else {
    const dim3 grid(nks, N, ntab);
    if (D == 128)
      hipLaunchKernelGGL(k_xts<128>, grid, dim3(256), 0, s, tp, S, s_tab, N, T, nks, part);
    else
      hipLaunchKernelGGL(k_xts<64>, grid, dim3(256), 0, s, tp, S, s_tab, N, T, nks, part);
  }
  const int64_t per = (int64_t)N * D * XS_P;
  hipLaunchKernelGGL(k_xts_reduce, dim3((unsigned)std::min<int64_t>((per + 255) / 256, 4096), ntab), dim3(256), 0, s,
                     part, N, D, nks, P, p_tab);
  return hipGetLastError();
}

// For the r_d < D chains the finder's A^T S is, per slice n and chain cc (r_d = 4 << cc),
// P_n(cc) = Y_n[:, :r_d]^T S(cc) (r_d x 40), Y_n [T][32] fp32.  One workgroup per (k slice,
// slice, table) reads each 64-token chunk of Y_n once and multiplies it against the four
// chains' S (rows j < 32 for every chain; the first r_d are kept), both operands split into
// fp16 hi + lo through LDS as in k_xts.  Wave w owns chain w: two 16-row tiles of j and the
// three 16-column tiles of the (padded) 48 sketch columns.
template <int UNUSED = 0>
__global__ __launch_bounds__(256) void k_yts(const float* __restrict__ Y, const float* __restrict__ S, int N,
                                             int T, int nks, float* __restrict__ part) {
  const int ks = blockIdx.x, n = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  __shared__ uint32_t sYh[32 * XS_LS], sYl[32 * XS_LS];            // [j][pair]
  __shared__ uint32_t sSh[4 * 48 * XS_LS], sSl[4 * 48 * XS_LS];    // [chain][c][pair]
  const float* Yn = Y + ((int64_t)t * N + n) * T * JOLT_KMAX;      // [T][32]
  const float* St = S + (int64_t)t * 5 * T * XS_P;                 // chains 0..3: [cc][T][40]
  const int k0 = ks * XS_KS, k1 = min(T, k0 + XS_KS);
  const int fr = lane & 15, g = lane >> 4;
  float4_t acc[2][3];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 3; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto f16bits = [](float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v); };
  auto lo = [](float v) { return v - (float)(_Float16)v; };
  constexpr int NY = 32 * 32 / 256;       // (pair, j) items per thread
  constexpr int NS = 4 * 32 * 48 / 256;   // (chain, pair, c) items per thread
  float ya[NY], yb[NY], sa[NS], sb[NS];
  auto load = [&](int c0) {
#pragma unroll
    for (int i = 0; i < NY; ++i) {
      const int idx = tid + 256 * i, j = idx & 31, pp = idx >> 5, r = c0 + 2 * pp;
      ya[i] = r < k1 ? Yn[(int64_t)r * JOLT_KMAX + j] : 0.f;
      yb[i] = r + 1 < k1 ? Yn[(int64_t)(r + 1) * JOLT_KMAX + j] : 0.f;
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int idx = tid + 256 * i, c = idx % 48, pp = (idx / 48) & 31, cc = idx / (48 * 32), r = c0 + 2 * pp;
      const float* Sc = St + (int64_t)cc * T * XS_P;
      sa[i] = (c < XS_P && r < k1) ? Sc[(int64_t)r * XS_P + c] : 0.f;
      sb[i] = (c < XS_P && r + 1 < k1) ? Sc[(int64_t)(r + 1) * XS_P + c] : 0.f;
    }
  };
  if (k0 < k1) load(k0);
  for (int c0 = k0; c0 < k1; c0 += 64) {
#pragma unroll
    for (int i = 0; i < NY; ++i) {
      const int idx = tid + 256 * i, j = idx & 31, pp = idx >> 5;
      sYh[j * XS_LS + pp] = f16bits(ya[i]) | (f16bits(yb[i]) << 16);
      sYl[j * XS_LS + pp] = f16bits(lo(ya[i])) | (f16bits(lo(yb[i])) << 16);
    }
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      const int idx = tid + 256 * i, c = idx % 48, pp = (idx / 48) & 31, cc = idx / (48 * 32);
      sSh[(cc * 48 + c) * XS_LS + pp] = f16bits(sa[i]) | (f16bits(sb[i]) << 16);
      sSl[(cc * 48 + c) * XS_LS + pp] = f16bits(lo(sa[i])) | (f16bits(lo(sb[i])) << 16);
    }
    __syncthreads();
    if (c0 + 64 < k1) load(c0 + 64);
#pragma unroll
    for (int kb = 0; kb < 64; kb += 16) {
      const int pq = kb / 2 + 2 * g;
      half4_t bh[3], bl[3];
#pragma unroll
      for (int jt = 0; jt < 3; ++jt) {
        const int c = wave * 48 + 16 * jt + fr;
        uint2 u, v;
        u.x = sSh[c * XS_LS + pq];
        u.y = sSh[c * XS_LS + pq + 1];
        v.x = sSl[c * XS_LS + pq];
        v.y = sSl[c * XS_LS + pq + 1];
        bh[jt] = __builtin_bit_cast(half4_t, u);
        bl[jt] = __builtin_bit_cast(half4_t, v);
      }
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const int j = 16 * it + fr;
        uint2 u, w;
        u.x = sYh[j * XS_LS + pq];
        u.y = sYh[j * XS_LS + pq + 1];
        w.x = sYl[j * XS_LS + pq];
        w.y = sYl[j * XS_LS + pq + 1];
        const half4_t ah = __builtin_bit_cast(half4_t, u), al = __builtin_bit_cast(half4_t, w);
#pragma unroll
        for (int jt = 0; jt < 3; ++jt) {
          acc[it][jt] = mfma16(ah, bh[jt], acc[it][jt]);
          acc[it][jt] = mfma16(ah, bl[jt], acc[it][jt]);
          acc[it][jt] = mfma16(al, bh[jt], acc[it][jt]);
        }
      }
    }
    __syncthreads();
  }
  // partial [t][n][ks][chain w][j < 32][c < 40]
  float* out = part + ((((int64_t)t * N + n) * nks + ks) * 4 + wave) * JOLT_KMAX * XS_P;
#pragma unroll
  for (int it = 0; it < 2; ++it)
#pragma unroll
    for (int jt = 0; jt < 3; ++jt)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * it + 4 * g + v, c = 16 * jt + fr;
        if (c < XS_P) out[j * XS_P + c] = acc[it][jt][v];
      }
}

// The same products for N a multiple of 8, eight slices per workgroup: the four chains' S
// chunk is staged once for eight slices instead of once per slice.  One workgroup of 512
// threads per (k slice, group of 8 slices, table); wave w owns slice 8 grp + w: its 32 rows
// j (two 16-row tiles) against all 160 columns (chain cc = column / 40, c = column % 40; ten
// 16-column tiles).  Chunks of 32 tokens go through LDS as fp16 hi + lo, token-contiguous
// rows for both operands (Y transposed on the way in); v_mfma_f32_16x16x32_f16 with the
// products hi hi, hi lo, lo hi; the next chunk is loaded during the products.  The partials
// have the layout of k_yts.
constexpr int YG = 8;        // slices per workgroup
constexpr int YC = 32;       // tokens per chunk
constexpr int YLS = YC + 8;  // LDS row stride (halves)

__global__ __launch_bounds__(512, 4) void k_yts8(const float* __restrict__ Y, const float* __restrict__ S, int N,
                                              int T, int nks, float* __restrict__ part) {
  const int ks = blockIdx.x, grp = blockIdx.y, t = blockIdx.z;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, g = lane >> 4;
  __shared__ __align__(16) uint16_t sYh[YG * 32][YLS], sYl[YG * 32][YLS];  // [slice * 32 + j][token]
  __shared__ __align__(16) uint16_t sSh[4 * XS_P][YLS], sSl[4 * XS_P][YLS];  // [cc * 40 + c][token]
  const int n0 = grp * YG;
  const float* Yg = Y + ((int64_t)t * N + n0) * T * JOLT_KMAX;  // slice s at + s T 32
  const float* St = S + (int64_t)t * 5 * T * XS_P;               // chains 0..3: [cc][T][40]
  const int k0 = ks * XS_KS, k1 = min(T, k0 + XS_KS);
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  float4_t acc[2][10];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int j = 0; j < 10; ++j) acc[i][j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto hb = [](float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v); };
  auto lb = [](float v) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)(v - (float)(_Float16)v)); };
  // items per chunk: Y (slice, token pair, 4 values of j): 8 x 16 x 8 = 1024, two per thread;
  // S (chain, token pair, 4 columns): 4 x 16 x 10 = 640, at most two per thread
  float4_t ya[2], yb[2], sa[2], sb[2];
  const float4_t z4 = (float4_t){0.f, 0.f, 0.f, 0.f};
  auto load = [&](int c0) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i, sl = idx >> 7, pp = (idx >> 3) & 15, j4 = idx & 7, r = c0 + 2 * pp;
      const float* yr = Yg + ((int64_t)sl * T + r) * JOLT_KMAX + 4 * j4;
      ya[i] = r < k1 ? *(const float4_t*)yr : z4;
      yb[i] = r + 1 < k1 ? *(const float4_t*)(yr + JOLT_KMAX) : z4;
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i, cc = idx / 160, rem = idx % 160, pp = rem / 10, c4 = rem % 10, r = c0 + 2 * pp;
      const bool ok = idx < 640;
      const float* sr = St + ((int64_t)cc * T + r) * XS_P + 4 * c4;
      sa[i] = ok && r < k1 ? *(const float4_t*)sr : z4;
      sb[i] = ok && r + 1 < k1 ? *(const float4_t*)(sr + XS_P) : z4;
    }
  };
  if (k0 < k1) load(k0);
  for (int c0 = k0; c0 < k1; c0 += YC) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i, sl = idx >> 7, pp = (idx >> 3) & 15, j4 = idx & 7;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int row = sl * 32 + 4 * j4 + e;
        *(uint32_t*)&sYh[row][2 * pp] = hb(ya[i][e]) | (hb(yb[i][e]) << 16);
        *(uint32_t*)&sYl[row][2 * pp] = lb(ya[i][e]) | (lb(yb[i][e]) << 16);
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i, cc = idx / 160, rem = idx % 160, pp = rem / 10, c4 = rem % 10;
      if (idx < 640) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int col = cc * XS_P + 4 * c4 + e;
          *(uint32_t*)&sSh[col][2 * pp] = hb(sa[i][e]) | (hb(sb[i][e]) << 16);
          *(uint32_t*)&sSl[col][2 * pp] = lb(sa[i][e]) | (lb(sb[i][e]) << 16);
        }
      }
    }
    __syncthreads();
    if (c0 + YC < k1) load(c0 + YC);
    h8 ah[2], al[2];
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) {
      ah[rt] = *(const h8*)&sYh[wave * 32 + 16 * rt + li][8 * g];
      al[rt] = *(const h8*)&sYl[wave * 32 + 16 * rt + li][8 * g];
    }
#pragma unroll
    for (int ct = 0; ct < 10; ++ct) {
      const h8 bh = *(const h8*)&sSh[16 * ct + li][8 * g];
      const h8 bl = *(const h8*)&sSl[16 * ct + li][8 * g];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt) {
        // rows j = 16 .. 31 are read only by the r_d = 32 chain (columns 120 .. 159, tiles
        // 7 .. 9); its other tiles stay zero and are never read back
        if (rt == 1 && 16 * ct + 15 < 3 * XS_P) continue;
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt], bh, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[rt], bl, acc[rt][ct], 0, 0, 0);
        acc[rt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[rt], bh, acc[rt][ct], 0, 0, 0);
      }
    }
    __syncthreads();
  }
  // partial [t][n][ks][chain][j < 32][c < 40]; tile element (row 4 g + v, column li)
  const int n = n0 + wave;
  float* out = part + (((int64_t)t * N + n) * nks + ks) * 4 * JOLT_KMAX * XS_P;
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int ct = 0; ct < 10; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int j = 16 * rt + 4 * g + v, col = 16 * ct + li, cc = col / XS_P, c = col - cc * XS_P;
        out[(cc * JOLT_KMAX + j) * XS_P + c] = acc[rt][ct][v];
      }
}

// P[t][cc][n r_d + j][c] (chain block stride p_chain, table stride 5 p_chain) for j < r_d
__global__ __launch_bounds__(256) void k_yts_reduce(const float* __restrict__ part, int N, int nks,
                                                    float* __restrict__ P, int64_t p_chain) {
  const int cc = blockIdx.y % 4, t = blockIdx.y / 4, rd = 4 << cc;
  const int64_t per = (int64_t)N * rd * XS_P;
  for (int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x; idx < per; idx += (int64_t)gridDim.x * 256) {
    const int64_t row = idx / XS_P;
    const int c = (int)(idx - row * XS_P);
    const int64_t n = row / rd;
    const int j = (int)(row - n * rd);
    const float* src = part + ((((int64_t)t * N + n) * nks) * 4 + cc) * JOLT_KMAX * XS_P + j * XS_P + c;
    double s = 0.0;
    for (int q = 0; q < nks; ++q) s += (double)src[(int64_t)q * 4 * JOLT_KMAX * XS_P];
    P[((int64_t)t * 5 + cc) * p_chain + idx] = (float)s;
  }
}

hipError_t launch_yts(const float* Y, const float* S, int N, int T, int ntab, float* part, float* P,
                      int64_t p_chain, hipStream_t s) {
  if (T < 1 || T % 2 || N < 1 || N > 65535 || ntab < 1 || ntab > 65535 / 4) return hipErrorInvalidValue;
  const int nks = xts_slices(T);
  if (N % YG == 0 && (int64_t)nks * (N / YG) * ntab >= 256)
    hipLaunchKernelGGL(k_yts8, dim3(nks, N / YG, ntab), dim3(512), 0, s, Y, S, N, T, nks, part);
  else
    hipLaunchKernelGGL(k_yts<0>, dim3(nks, N, ntab), dim3(256), 0, s, Y, S, N, T, nks, part);
  const int64_t per = (int64_t)N * 32 * XS_P;
  hipLaunchKernelGGL(k_yts_reduce, dim3((unsigned)std::min<int64_t>((per + 255) / 256, 2048), ntab * 4), dim3(256), 0,
                     s, part, N, nks, P, p_chain);
  return hipGetLastError();
}

// The r_d < D chains' A B of the randomized finder, all four from one pass over Y:
// S_cc[t][tk][c] = sum_n sum_{j < r_d} Y_t[n][tk][j] B_cc[n r_d + j][c] (r_d = 4 << cc,
// c < 40), B given transposed (BT: element t b_tab + boff[cc] + c b_ld + row; fp32, or bf16
// with BF).  Every chain uses the same A fragments, j = 0..31 of a slice in one 32-deep
// product per slice and chain, with the B rows j >= r_d zero.  Operands split into fp16 hi
// + lo (products hi hi, hi lo, lo hi; a bf16 B has no lo part), fp32 accumulation over the
// slices in order.  One workgroup per 128 tokens of a table; wave w owns tokens
// 32 w .. 32 w + 31 (two 16-token tiles).  The slices' B fragments go through LDS (double
// buffer), the Y fragments from global memory straight into registers; the next slice is
// loaded during the products.
struct YwOff {
  int64_t b[4];
};

template <bool BF>
__global__ __launch_bounds__(256) void k_yw4(const float* __restrict__ Y, const void* __restrict__ BT, int64_t b_tab,
                                             int64_t b_ld, const YwOff boff, int N, int T, float* __restrict__ Sout,
                                             int64_t s_tab, int64_t s_chain) {
  typedef _Float16 h8 __attribute__((ext_vector_type(8)));
  const int t0 = blockIdx.x * 128, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, g = lane >> 4;
  __shared__ __align__(16) h8 sBh[2][4][3][4][16], sBl[2][4][3][4][16];  // [buf][cc][ct][g][li]
  const float* Yt = Y + (int64_t)t * N * T * JOLT_KMAX;
  // B fragments of slice n into buffer bf: item (cc, ct, g, li) = 768 items, 3 per thread.
  // fetch_b loads a slice's raw values into registers before the products of the current
  // slice; put_b converts them and stores them after those products, so that the loads'
  // latency overlaps the products.
  uint32_t braw[3][8];
  auto b_item = [&](int i, int& lq, int& gq, int& ct, int& cc, int& cnt) {
    const int idx = tid + 256 * i;
    lq = idx & 15;
    gq = (idx >> 4) & 3;
    ct = (idx >> 6) % 3;
    cc = idx / 192;
    const int rd = 4 << cc, col = 16 * ct + lq;
    cnt = (col < XS_P && 8 * gq < rd) ? min(8, rd - 8 * gq) : 0;
  };
  // per item: the offset of slice 0 (the chain's offset selected, not indexed, so that it
  // stays in scalar registers) and r_d
  int64_t bbase[3];
#pragma unroll
  for (int i = 0; i < 3; ++i) {
    int lq, gq, ct, cc, cnt;
    b_item(i, lq, gq, ct, cc, cnt);
    const int64_t off = cc == 0 ? boff.b[0] : cc == 1 ? boff.b[1] : cc == 2 ? boff.b[2] : boff.b[3];
    bbase[i] = (int64_t)t * b_tab + off + (int64_t)(16 * ct + lq) * b_ld + 8 * gq;
  }
  // Branch-free, so that no wait for earlier loads is needed before the products: every
  // item loads two 16-byte pieces (an item with fewer values reads the table's first
  // element instead, which is in bounds), and put_b zeroes what lies beyond the item's count.
  auto fetch_b = [&](int n) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      int lq, gq, ct, cc, cnt;
      b_item(i, lq, gq, ct, cc, cnt);
      const int rd = 4 << cc;
      const int64_t o = bbase[i] + (int64_t)n * rd, t0b = (int64_t)t * b_tab;
      if (BF) {  // 4 bf16 values per 8-byte piece
        const int64_t oa = cnt >= 4 ? o : t0b, ob = cnt == 8 ? o + 4 : t0b;
        const uint2 u = *(const uint2*)((const uint16_t*)BT + oa), w = *(const uint2*)((const uint16_t*)BT + ob);
        braw[i][0] = u.x; braw[i][1] = u.y; braw[i][2] = w.x; braw[i][3] = w.y;
      } else {
        const int64_t oa = cnt >= 4 ? o : t0b, ob = cnt == 8 ? o + 4 : t0b;
        const uint4 a = *(const uint4*)((const float*)BT + oa), b = *(const uint4*)((const float*)BT + ob);
        braw[i][0] = a.x; braw[i][1] = a.y; braw[i][2] = a.z; braw[i][3] = a.w;
        braw[i][4] = b.x; braw[i][5] = b.y; braw[i][6] = b.z; braw[i][7] = b.w;
      }
    }
  };
  auto put_b = [&](int bf) {
#pragma unroll
    for (int i = 0; i < 3; ++i) {
      int lq, gq, ct, cc, cnt;
      b_item(i, lq, gq, ct, cc, cnt);
      float v[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) {  // a bf16 pair per dword, or one float per dword
        const float x = BF ? __uint_as_float(((braw[i][e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16)
                           : __uint_as_float(braw[i][e]);
        v[e] = e < cnt ? x : 0.f;
      }
      h8 hv, lv;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const _Float16 hh = (_Float16)v[e];
        hv[e] = hh;
        lv[e] = (_Float16)(v[e] - (float)hh);
      }
      sBh[bf][cc][ct][gq][lq] = hv;
      sBl[bf][cc][ct][gq][lq] = lv;
    }
  };
  // this lane's Y values of slice n: token t0 + 32 wave + 16 tt + li, j = 8 g .. 8 g + 7
  float4_t ya[2][2];
  auto load_a = [&](int n) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const float* yr = Yt + ((int64_t)n * T + t0 + 32 * wave + 16 * tt + li) * JOLT_KMAX + 8 * g;
      ya[tt][0] = *(const float4_t*)yr;
      ya[tt][1] = *(const float4_t*)(yr + 4);
    }
  };
  float4_t acc[4][2][3];
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) acc[cc][tt][ct] = (float4_t){0.f, 0.f, 0.f, 0.f};
  fetch_b(0);
  put_b(0);
  load_a(0);
  __syncthreads();
  for (int n = 0; n < N; ++n) {
    const int bf = n & 1;
    h8 ah[2], al[2];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float v = ya[tt][e >> 2][e & 3];
        const _Float16 hh = (_Float16)v;
        ah[tt][e] = hh;
        al[tt][e] = (_Float16)(v - (float)hh);
      }
    if (n + 1 < N) {
      load_a(n + 1);
      fetch_b(n + 1);
    }
#pragma unroll
    for (int cc = 0; cc < 4; ++cc)
#pragma unroll
      for (int ct = 0; ct < 3; ++ct) {
        const h8 bh = sBh[bf][cc][ct][g][li], bl = sBl[bf][cc][ct][g][li];
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) {
          acc[cc][tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[tt], bh, acc[cc][tt][ct], 0, 0, 0);
          acc[cc][tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(ah[tt], bl, acc[cc][tt][ct], 0, 0, 0);
          acc[cc][tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_f16(al[tt], bh, acc[cc][tt][ct], 0, 0, 0);
        }
      }
    // the other buffer: its last readers passed the previous barrier
    if (n + 1 < N) put_b(bf ^ 1);
    __syncthreads();
  }
  // element (token 4 g + v of tile tt, column 16 ct + li)
#pragma unroll
  for (int cc = 0; cc < 4; ++cc)
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int tk = t0 + 32 * wave + 16 * tt + 4 * g + v, c = 16 * ct + li;
          if (c < XS_P) Sout[(int64_t)t * s_tab + cc * s_chain + (int64_t)tk * XS_P + c] = acc[cc][tt][ct][v];
        }
}

hipError_t launch_yw4(const float* Y, const void* BT, bool bf16, int64_t b_tab, int64_t b_ld, const int64_t* boff,
                      int N, int T, int ntab, float* S, int64_t s_tab, int64_t s_chain, hipStream_t s) {
  YwOff o;
  bool ok = T % 128 == 0 && N >= 1 && ntab >= 1 && ntab <= 65535 && T / 128 <= 65535 && b_tab % 8 == 0 &&
            b_ld % 8 == 0 && ((uintptr_t)BT % 16) == 0;
  for (int c = 0; c < 4; ++c) {
    o.b[c] = boff[c];
    ok = ok && boff[c] % 8 == 0;
  }
  if (!ok) return hipErrorInvalidValue;
  const dim3 grid(T / 128, ntab);
  if (bf16) hipLaunchKernelGGL(k_yw4<true>, grid, dim3(256), 0, s, Y, BT, b_tab, b_ld, o, N, T, S, s_tab, s_chain);
  else hipLaunchKernelGGL(k_yw4<false>, grid, dim3(256), 0, s, Y, BT, b_tab, b_ld, o, N, T, S, s_tab, s_chain);
  return hipGetLastError();
}

// The r_d = D chain's A B of the randomized finder: S[t][tk][c] = sum_n sum_f X_t[n][tk][f]
// B[t][n D + f][c] (c < 40), given B^T ([c][row n D + f], row stride b_ld, table stride b_tab).
// The generic GEMM's arithmetic operation for operation, so S is the same to the bit: k in
// ascending order (n outer, f inner) in 16-wide blocks, fp32 accumulation; with BF (the
// bf16 sketch) exact bf16 products, else both operands split into fp16 hi + lo and the
// products hi hi, hi lo, lo hi in that order.  One workgroup per 64 tokens of a table loops
// over the slices, staging X_n's rows and B_n^T in LDS (the next slice is loaded during the
// products); wave w owns tokens 16 w .. 16 w + 15 and the three 16-column tiles of the
// (padded) 48 columns.
template <int D, bool BF>
__global__ __launch_bounds__(256) void k_xw(const TablePtrs tp, const void* __restrict__ BT, int64_t b_tab,
                                            int64_t b_ld, int N, int T, float* __restrict__ Sout, int64_t s_tab) {
  constexpr int LS = D + 8;  // LDS row stride (halves)
  const int t0 = blockIdx.x * 64, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, fr = lane & 15, g = lane >> 4;
  __shared__ __align__(16) uint16_t sXh[64 * LS], sXl[BF ? 8 : 64 * LS];
  __shared__ __align__(16) uint16_t sBh[48 * LS], sBl[BF ? 8 : 48 * LS];
  const uint16_t* X = (const uint16_t*)tp.p[t];
  constexpr int NX = 64 * D / 8 / 256;            // 16-byte X loads per thread and slice
  constexpr int NB = (48 * D / 4 + 255) / 256;     // 4-value B loads per thread and slice
  uint4 xr[NX];
  float4 br[NB];
  uint2 br16[NB];
  auto load = [&](int n) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 8), seg = idx % (D / 8);
      xr[i] = *(const uint4*)(X + ((int64_t)n * T + t0 + row) * D + 8 * seg);
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int idx = tid + 256 * i, c = idx / (D / 4), q = idx % (D / 4);
      const bool ok = idx < 48 * D / 4 && c < XS_P;
      const int64_t o = (int64_t)t * b_tab + (int64_t)c * b_ld + (int64_t)n * D + 4 * q;
      if (BF) br16[i] = ok ? *(const uint2*)((const uint16_t*)BT + o) : make_uint2(0u, 0u);
      else br[i] = ok ? *(const float4*)((const float*)BT + o) : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto h16 = [](float v) { return __builtin_bit_cast(uint16_t, (_Float16)v); };
  auto l16 = [](float v) { return __builtin_bit_cast(uint16_t, (_Float16)(v - (float)(_Float16)v)); };
  float4_t acc[3];
#pragma unroll
  for (int j = 0; j < 3; ++j) acc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  load(0);
  for (int n = 0; n < N; ++n) {
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int idx = tid + 256 * i, row = idx / (D / 8), seg = idx % (D / 8);
      const uint32_t w[4] = {xr[i].x, xr[i].y, xr[i].z, xr[i].w};
      if (BF) {
        *(uint4*)&sXh[row * LS + 8 * seg] = xr[i];
      } else {
        uint16_t hh[8], ll[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = __uint_as_float(((w[e >> 1] >> (16 * (e & 1))) & 0xFFFFu) << 16);
          hh[e] = h16(v);
          ll[e] = l16(v);
        }
        *(uint4*)&sXh[row * LS + 8 * seg] = pack8(hh);
        *(uint4*)&sXl[row * LS + 8 * seg] = pack8(ll);
      }
    }
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int idx = tid + 256 * i, c = idx / (D / 4), q = idx % (D / 4);
      if (idx < 48 * D / 4) {
        if (BF) {
          *(uint2*)&sBh[c * LS + 4 * q] = br16[i];
        } else {
          const float v[4] = {br[i].x, br[i].y, br[i].z, br[i].w};
          uint2 hh, ll;
          hh.x = (uint32_t)h16(v[0]) | ((uint32_t)h16(v[1]) << 16);
          hh.y = (uint32_t)h16(v[2]) | ((uint32_t)h16(v[3]) << 16);
          ll.x = (uint32_t)l16(v[0]) | ((uint32_t)l16(v[1]) << 16);
          ll.y = (uint32_t)l16(v[2]) | ((uint32_t)l16(v[3]) << 16);
          *(uint2*)&sBh[c * LS + 4 * q] = hh;
          *(uint2*)&sBl[c * LS + 4 * q] = ll;
        }
      }
    }
    __syncthreads();
    if (n + 1 < N) load(n + 1);
#pragma unroll
    for (int kb = 0; kb < D; kb += 16) {
      const int ar = (16 * wave + fr) * LS + kb + 4 * g;
#pragma unroll
      for (int j = 0; j < 3; ++j) {
        const int brow = (16 * j + fr) * LS + kb + 4 * g;
        if (BF) {
          acc[j] = mfma16bf(*(const short4_t*)&sXh[ar], *(const short4_t*)&sBh[brow], acc[j]);
        } else {
          const half4_t ah = *(const half4_t*)&sXh[ar], al = *(const half4_t*)&sXl[ar];
          const half4_t bh = *(const half4_t*)&sBh[brow], bl = *(const half4_t*)&sBl[brow];
          acc[j] = mfma16(ah, bh, acc[j]);
          acc[j] = mfma16(ah, bl, acc[j]);
          acc[j] = mfma16(al, bh, acc[j]);
        }
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int j = 0; j < 3; ++j)
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const int tk = t0 + 16 * wave + 4 * g + v, c = 16 * j + fr;
      if (c < XS_P) Sout[(int64_t)t * s_tab + (int64_t)tk * XS_P + c] = acc[j][v];
    }
}

// The same product with 256 tokens per workgroup and no LDS for X: the tensor is bf16, so its
// rows enter bf16 MFMA (v_mfma_f32_16x16x32_bf16) straight from global memory as A operands
// (token i in lane i + 16 g, features 32 kb + 8 g .. + 7: 16 contiguous bytes), exact.  B_n
// (the slice's D x 40 block) goes through a double-buffered LDS stage as three bf16 pieces
// b1 + b2 + b3 (24 bits of the fp32 value; one piece for the bf16 sketch), so every product
// is exact in fp32; the products run over the slices in order, fp32 accumulation.  Wave w
// owns tokens 32 w .. 32 w + 31 (two 16-token tiles) of the workgroup's 256; the next slice's
// rows are loaded during the products.
template <int D, bool BF>
__global__ __launch_bounds__(512) void k_xw8(const TablePtrs tp, const void* __restrict__ BT, int64_t b_tab,
                                             int64_t b_ld, int N, int T, float* __restrict__ Sout, int64_t s_tab) {
  typedef __bf16 b8 __attribute__((ext_vector_type(8)));
  constexpr int KB = D / 32;       // 32-deep products per slice
  constexpr int NP = BF ? 1 : 3;   // bf16 pieces of B
  constexpr int ITEMS = KB * 3 * 4 * 16;  // (kb, ct, g, li) fragments per piece
  const int t0 = blockIdx.x * 256, t = blockIdx.y;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, li = lane & 15, g = lane >> 4;
  __shared__ __align__(16) b8 sB[2][NP][KB][3][4][16];
  const uint16_t* X = (const uint16_t*)tp.p[t];
  // B fragments of slice n: item (kb, ct, g, li), ITEMS of them, at most two per thread.
  // fetch_b loads a slice's raw values into registers before the products of the current
  // slice; put_b splits them into bf16 pieces and stores them after those products, so
  // that the loads' latency overlaps the products.
  // Branch-free, so that no wait for earlier loads is needed before the products: an item
  // beyond the 40 columns reads the table's first element instead (in bounds), and put_b
  // stores zeros for it.
  constexpr int BW = BF ? 4 : 8;  // dwords per item
  uint32_t braw[2][BW];
  auto fetch_b = [&](int n) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i;
      if (idx >= ITEMS) break;  // uniform per wave (ITEMS is a multiple of 64)
      const int lq = idx & 15, gq = (idx >> 4) & 3, ct = (idx >> 6) % 3, kb = idx / 192;
      const int col = 16 * ct + lq;
      const int64_t o = col < XS_P ? (int64_t)t * b_tab + (int64_t)col * b_ld + (int64_t)n * D + 32 * kb + 8 * gq
                                   : (int64_t)t * b_tab;
      if (BF) {
        const uint4 u = *(const uint4*)((const uint16_t*)BT + o);
        braw[i][0] = u.x; braw[i][1] = u.y; braw[i][2] = u.z; braw[i][3] = u.w;
      } else {
        const uint4 a = *(const uint4*)((const float*)BT + o), b = *(const uint4*)((const float*)BT + o + 4);
        braw[i][0] = a.x; braw[i][1] = a.y; braw[i][2] = a.z; braw[i][3] = a.w;
        braw[i][BW > 4 ? 4 : 0] = b.x; braw[i][BW > 5 ? 5 : 0] = b.y;
        braw[i][BW > 6 ? 6 : 0] = b.z; braw[i][BW > 7 ? 7 : 0] = b.w;
      }
    }
  };
  auto put_b = [&](int bf) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int idx = tid + 512 * i;
      if (idx >= ITEMS) break;
      const int lq = idx & 15, gq = (idx >> 4) & 3, ct = (idx >> 6) % 3, kb = idx / 192;
      const bool ok = 16 * ct + lq < XS_P;
      if (BF) {
        sB[bf][0][kb][ct][gq][lq] = __builtin_bit_cast(
            b8, ok ? make_uint4(braw[i][0], braw[i][1], braw[i][2], braw[i][3]) : make_uint4(0u, 0u, 0u, 0u));
      } else {
        b8 p0, p1, p2;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float v = ok ? __uint_as_float(braw[i][e < BW ? e : 0]) : 0.f;
          const __bf16 h1 = (__bf16)v;
          const float r1 = v - (float)h1;
          const __bf16 h2 = (__bf16)r1;
          p0[e] = h1;
          p1[e] = h2;
          p2[e] = (__bf16)(r1 - (float)h2);
        }
        sB[bf][0][kb][ct][gq][lq] = p0;
        sB[bf][NP > 1 ? 1 : 0][kb][ct][gq][lq] = p1;
        sB[bf][NP > 2 ? 2 : 0][kb][ct][gq][lq] = p2;
      }
    }
  };
  uint4 xa[2][KB];
  auto load_a = [&](int n) {
#pragma unroll
    for (int tt = 0; tt < 2; ++tt) {
      const uint16_t* xr = X + ((int64_t)n * T + t0 + 32 * wave + 16 * tt + li) * D + 8 * g;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) xa[tt][kb] = *(const uint4*)(xr + 32 * kb);
    }
  };
  float4_t acc[2][3];
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int ct = 0; ct < 3; ++ct) acc[tt][ct] = (float4_t){0.f, 0.f, 0.f, 0.f};
  fetch_b(0);
  put_b(0);
  load_a(0);
  __syncthreads();
  for (int n = 0; n < N; ++n) {
    const int bf = n & 1;
    b8 af[2][KB];
#pragma unroll
    for (int tt = 0; tt < 2; ++tt)
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) af[tt][kb] = __builtin_bit_cast(b8, xa[tt][kb]);
    // B first, then X, both unconditional (the index clamped: the last slice is fetched
    // again at the end): put_b then waits only for the B loads, and the next slice's X loads
    // stay in flight across the barrier (fetched after them, B made it wait for them as
    // well: 1056 -> 826 us at 32k tokens).
    const int nn = n + 1 < N ? n + 1 : N - 1;
    fetch_b(nn);
    load_a(nn);
#pragma unroll
    for (int kb = 0; kb < KB; ++kb)
#pragma unroll
      for (int ct = 0; ct < 3; ++ct)
#pragma unroll
        for (int pc = 0; pc < NP; ++pc) {
          const b8 bv = sB[bf][pc][kb][ct][g][li];
#pragma unroll
          for (int tt = 0; tt < 2; ++tt)
            acc[tt][ct] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[tt][kb], bv, acc[tt][ct], 0, 0, 0);
        }
    // the other buffer: its last readers passed the previous barrier
    put_b(bf ^ 1);
    __syncthreads();
  }
#pragma unroll
  for (int tt = 0; tt < 2; ++tt)
#pragma unroll
    for (int ct = 0; ct < 3; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int tk = t0 + 32 * wave + 16 * tt + 4 * g + v, c = 16 * ct + li;
        if (c < XS_P) Sout[(int64_t)t * s_tab + (int64_t)tk * XS_P + c] = acc[tt][ct][v];
      }
}

hipError_t launch_xw(const TablePtrs& tp, const void* BT, bool bf16, int64_t b_tab, int64_t b_ld, int N, int T,
                     int D, int ntab, float* S, int64_t s_tab, hipStream_t s) {
  if ((D != 64 && D != 128) || T % 64 || N < 1 || ntab < 1 || ntab > 65535 || T / 64 > 65535 || b_ld % 8 ||
      b_tab % 8 || ((uintptr_t)BT % 16))
    return hipErrorInvalidValue;
  if (T % 256 == 0) {  // 256 tokens per workgroup, X straight into registers
    const dim3 g8(T / 256, ntab);
    if (D == 128) {
      if (bf16) hipLaunchKernelGGL((k_xw8<128, true>), g8, dim3(512), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
      else hipLaunchKernelGGL((k_xw8<128, false>), g8, dim3(512), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
    } else {
      if (bf16) hipLaunchKernelGGL((k_xw8<64, true>), g8, dim3(512), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
      else hipLaunchKernelGGL((k_xw8<64, false>), g8, dim3(512), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
    }
    return hipGetLastError();
  }
  const dim3 grid(T / 64, ntab);
  if (D == 128) {
    if (bf16) hipLaunchKernelGGL((k_xw<128, true>), grid, dim3(256), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
    else hipLaunchKernelGGL((k_xw<128, false>), grid, dim3(256), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
  } else {
    if (bf16) hipLaunchKernelGGL((k_xw<64, true>), grid, dim3(256), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
    else hipLaunchKernelGGL((k_xw<64, false>), grid, dim3(256), 0, s, tp, BT, b_tab, b_ld, N, T, S, s_tab);
  }
  return hipGetLastError();
}

}  // namespace jolt
