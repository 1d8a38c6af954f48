// Record writer (encode) and reader (decode) for one chosen candidate per table.
//
// Encode follows "Rotated Tucker residual for outlier-resistant KV quantization",
// Implementation notes: with the stored Tucker factors, reconstruct X~, form
// R = X - X~, rotate each row of D values with Q = H diag(sigma) / sqrt(D), and store
// per block (one row) the scale s = max|Y| / (2^(b-1) - 1) (fp32) and the codes
// clip(round(Y / s), -2^(b-1), 2^(b-1) - 1).  The residual path runs in fp64.
// Decode follows "Joint Tucker-rank and residual-bit KV allocator", Formulas, first
// display: X^ = X~ + Q^T Q_b(Q R), in fp64, rounded once to bf16.
// X~ is formed per token tile with fp64 MFMA; the rest runs with one thread per 16
// consecutive features of a row (D / 16 threads per row).
//
// Launches cover up to JOLT_TAB_CHUNK tables: blockIdx.y is the local table index,
// workspace arrays are indexed by the global table index t0 + local.
#include "jolt_internal.h"

namespace jolt {

#ifdef JOLT_CODEC_TIMING  // phase timestamps of block (0, 0, 0) (probe builds only)
__device__ unsigned long long g_codec_t[8];
#define CD_MARK(i)                                                                      \
  do {                                                                                  \
    if (blockIdx.x == 0 && blockIdx.y == 0 && blockIdx.z == 0 && threadIdx.x == 0)      \
      g_codec_t[i] = __builtin_amdgcn_s_memrealtime();                                   \
  } while (0)
#else
#define CD_MARK(i) \
  do {             \
  } while (0)
#endif

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

// ---------------------------------------------------------------- shared reconstruction
// X~ rows of one slice n are L (tokens x K) times Rm (K x D): L is U_T (r_d chains, K =
// r_T) or the per-token core of the r_T = T chain (K = r_d); Rm is G_n U_d~^T, G_n, or
// U_d~^T.  Rm is formed once per workgroup in fp64 (exact sums of fp16 products up to
// fp64 rounding); each pass computes the X~ tile of CP tokens with fp64 MFMA
// (v_mfma_f64_16x16x4f64) into LDS, where the row-layout stages read it.
typedef double double4_t __attribute__((ext_vector_type(4)));

constexpr int CODEC_CHUNK = 256;  // tokens per workgroup

template <int D>
struct CodecLds {
  static constexpr int CP = D == 128 ? 32 : 64;  // tokens per pass (256 threads x 16 features)
  static constexpr int RS = D + 4;               // Rm row stride (doubles)
  static constexpr int XS = D + 2;               // X~ row stride (doubles)
  double Rm[JOLT_KMAX][RS];
  double Xt[CP][XS];
  double Gs[JOLT_KMAX][JOLT_KMAX];  // staged core rows (r_d chains < 4)
};

// Rm[k][f] for k < K (rows K.. zero).  kind: 0 = G_n U_d~^T (G fp16 [K][rd] with row
// stride gs, U_d fp16 [D][rd] with row stride us), 1 = G_n itself ([K][D], stride gs),
// 2 = U_d~^T (U_d [D][K], stride us).
template <int D>
__device__ void codec_setup_rm(CodecLds<D>& L, int kind, int K, int rd, const _Float16* G, int64_t gs,
                               const _Float16* Ud, int64_t us) {
  const int tid = threadIdx.x;
  if (kind == 0) {
    for (int idx = tid; idx < K * rd; idx += 256) {
      const int k = idx / rd, j = idx - k * rd;
      L.Gs[k][j] = (double)G[k * gs + j];
    }
    __syncthreads();
  }
  for (int idx = tid; idx < JOLT_KMAX * D; idx += 256) {
    const int k = idx / D, f = idx - k * D;
    double v = 0.0;
    if (k < K) {
      if (kind == 1) {
        v = (double)G[k * gs + f];
      } else if (kind == 2) {
        v = (double)Ud[f * us + k];
      } else {
        const _Float16* u = Ud + f * us;
        for (int j = 0; j < rd; ++j) v = fma(L.Gs[k][j], (double)u[j], v);
      }
    }
    L.Rm[k][f] = v;
  }
  __syncthreads();
}

// X~ of tokens tok0 .. tok0 + CP - 1 into L.Xt.  Lrow(t) = fp16 row of L for token t
// (row stride ls); K a multiple of 4.  Wave w computes token tile w / (CT/4) and column
// tiles 4 (w % (CT/4)) ..+3 (CT = D/16).  Output of a 16 x 16 tile: element (i, j) in
// lane 16 (i & 3) + j, register i >> 2; A element (i, k) in lane i + 16 k, B element
// (k, j) in lane j + 16 k.
template <int D>
__device__ __forceinline__ void codec_xtilde(CodecLds<D>& L, const _Float16* Lb, int64_t ls, int K, int tok0) {
  constexpr int CT = D / 16;
  constexpr int WPT = CT / 4;  // waves per token tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, c0 = (w % WPT) * 4;
  const int li = lane & 15, lk = lane >> 4;
  double4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (double4_t){0.0, 0.0, 0.0, 0.0};
  const _Float16* arow = Lb + (int64_t)(tok0 + 16 * tt + li) * ls + lk;
  for (int kk = 0; kk < K; kk += 4) {
    const double av = (double)arow[kk];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const double bv = L.Rm[kk + lk][16 * (c0 + c) + li];
      acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[c], 0, 0, 0);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) L.Xt[16 * tt + 4 * r + lk][16 * (c0 + c) + li] = acc[c][r];
}

// Residual codes and scales (b > 0).  Block (token chunk, slice n, local table).
template <int D>
__global__ __launch_bounds__(256) void k_encode_resid(const EncodeArgs a) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;  // threads per row
  constexpr int CP = CodecLds<D>::CP;
  const int tl = blockIdx.z, tg = a.t0 + tl, n = blockIdx.y;
  const EncodeTable& e = a.t[tl];
  if (e.b == 0) return;
  const int N = a.N, T = a.T;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  const int qmax = (1 << (e.b - 1)) - 1;
  const int tb = blockIdx.x * CODEC_CHUNK, te = min(T, tb + CODEC_CHUNK);
  __shared__ CodecLds<D> L;
  int K = 0;
  const _Float16* Lb = nullptr;
  int64_t ls = JOLT_KMAX;
  if (e.chain == 5) {
    K = e.rd;
    codec_setup_rm<D>(L, 2, K, e.rd, nullptr, 0, a.Ud16 + (int64_t)tg * D * JOLT_KMAX, JOLT_KMAX);
    Lb = a.G16T + ((int64_t)tg * N + n) * T * JOLT_KMAX;
  } else if (e.chain >= 0) {
    K = e.rT;
    const _Float16* G = a.G16 + (((int64_t)tg * 5 + e.chain) * N + n) * JOLT_KMAX * D;
    if (e.chain == 4) codec_setup_rm<D>(L, 1, K, D, G, D, nullptr, 0);
    else codec_setup_rm<D>(L, 0, K, e.rd, G, D, a.Ud16 + (int64_t)tg * D * JOLT_KMAX, JOLT_KMAX);
    Lb = a.UT16 + ((int64_t)tg * 5 + e.chain) * T * JOLT_KMAX;
  }
  const double isq = 1.0 / sqrt((double)D);
  const int8_t* sgn = a.signs + tg * D + sg * FPT;
  uint32_t* codes = (uint32_t*)(e.rec + e.off_codes);
  float* scales = (float*)(e.rec + e.off_scales);
  for (int t0 = tb; t0 < te; t0 += CP) {
    if (K > 0) codec_xtilde<D>(L, Lb, ls, K, t0);
    __syncthreads();
    const int tok = t0 + rloc;
    const int64_t row = (int64_t)n * T + tok;
    const uint4* xr = (const uint4*)((const uint16_t*)a.xsrc[tl] + row * D + sg * FPT);
    double y[FPT];
    {
      const uint4 q0 = xr[0], q1 = xr[1];
      const uint32_t wv[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
      const double* xt = &L.Xt[rloc][sg * FPT];
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        const uint16_t hb = (uint16_t)(wv[i >> 1] >> (16 * (i & 1)));
        const double x = (double)bf16_to_f32(hb);
        const double r = K > 0 ? x - xt[i] : 0.0;
        y[i] = sgn[i] < 0 ? -r : r;
      }
    }
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
    double m = 0.0;
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      y[i] *= isq;
      m = fmax(m, fabs(y[i]));
    }
#pragma unroll
    for (int st = 1; st < SEG; st <<= 1) m = fmax(m, __shfl_xor(m, st, 64));
    const float sc = (float)(m / (double)qmax);
    const double sd = (double)sc;
    int q[FPT];
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      double v = sd > 0.0 ? rint(y[i] / sd) : 0.0;
      v = fmin(fmax(v, (double)(-qmax - 1)), (double)qmax);
      q[i] = (int)v;
    }
    uint32_t* cw = codes + (row * D + sg * FPT) * e.b / 32;
    if (e.b == 2) pack_codes<2>(q, cw);
    else if (e.b == 4) pack_codes<4>(q, cw);
    else pack_codes<8>(q, cw);
    if (sg == 0) scales[row] = sc;
    __syncthreads();  // X~ tile is rewritten by the next pass
  }
}

// 16 codes of B bits (sign-extended fields) from B/2 words
template <int B>
__device__ __forceinline__ void unpack_codes(const uint32_t* src, int (&q)[16]) {
  constexpr int PER = 32 / B;
#pragma unroll
  for (int w = 0; w < B / 2; ++w) {
    const uint32_t word = src[w];
#pragma unroll
    for (int j = 0; j < PER; ++j) q[w * PER + j] = (int)(word << (32 - B * (j + 1))) >> (32 - B);
  }
}

// Reconstruction, dequantization, inverse rotation, bf16 output.  Block (token chunk,
// slice n, local table).  The inverse Hadamard runs on the integer codes (exact); the
// residual s (H q)_f sigma_f / sqrt(D) is added to X~ with one fp64 rounding, and the sum
// is rounded once to bf16.
// ---------------------------------------------------------------- decode of row tiles
// What a workgroup needs to rebuild rows of slice n of one record (chain >= 0).
struct DecodeSrc {
  int K;                 // inner dimension of X~ = L Rm
  const _Float16* Lb;    // L rows (token-major, stride ls)
  int64_t ls;
  const uint32_t* codes;
  const float* scales;
};

// Signs sigma_f / sqrt(D) from the record header into sgs, and the slice's Rm into L.
template <int D>
__device__ DecodeSrc codec_prepare(CodecLds<D>& L, double* sgs, const EncodeTable& e, int n, int T) {
  const int tid = threadIdx.x;
  const char* rec = e.rec;
  const uint32_t* sbits = (const uint32_t*)(rec + 128);
  const double isq = 1.0 / sqrt((double)D);
  for (int f = tid; f < D; f += 256) sgs[f] = ((sbits[f >> 5] >> (f & 31)) & 1u) ? -isq : isq;
  const _Float16* Ut = (const _Float16*)(rec + e.off_ut);
  const _Float16* Ud = (const _Float16*)(rec + e.off_ud);
  const _Float16* Gc = (const _Float16*)(rec + e.off_core);
  DecodeSrc d;
  if (e.chain == 5) {
    d.K = e.rd;
    codec_setup_rm<D>(L, 2, d.K, e.rd, nullptr, 0, Ud, e.rd);
    d.Lb = Gc + (int64_t)n * T * e.rd;
    d.ls = e.rd;
  } else {
    d.K = e.rT;
    const _Float16* G = Gc + (int64_t)n * e.rT * (e.chain == 4 ? D : e.rd);
    if (e.chain == 4) codec_setup_rm<D>(L, 1, d.K, D, G, D, nullptr, 0);
    else codec_setup_rm<D>(L, 0, d.K, e.rd, G, e.rd, Ud, e.rd);
    d.Lb = Ut;
    d.ls = e.rT;
  }
  d.codes = (const uint32_t*)(rec + e.off_codes);
  d.scales = (const float*)(rec + e.off_scales);
  return d;
}

// Decoded bf16 values of tokens t0 .. t0 + CP - 1 of slice n: this thread's 16 features
// (segment sg of token t0 + rloc, rloc = tid / (D / 16)), packed two per word.
// X~ goes through L.Xt; the caller synchronises before L.Xt is written again.
template <int D>
__device__ __forceinline__ void codec_decode_tile(CodecLds<D>& L, const double* sgs, const EncodeTable& e,
                                                  const DecodeSrc& d, int n, int T, int t0, uint32_t (&ow)[8]) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  codec_xtilde<D>(L, d.Lb, d.ls, d.K, t0);
  __syncthreads();
  const int tok = t0 + rloc;
  const int64_t row = (int64_t)n * T + tok;
  double s = 0.0;
  int h[FPT];
  if (e.b > 0) {
    s = (double)d.scales[row];
    const uint32_t* cw = d.codes + (row * D + sg * FPT) * e.b / 32;
    if (e.b == 2) unpack_codes<2>(cw, h);
    else if (e.b == 4) unpack_codes<4>(cw, h);
    else unpack_codes<8>(cw, h);
#pragma unroll
    for (int st = 1; st < FPT; st <<= 1)
#pragma unroll
      for (int i = 0; i < FPT; ++i)
        if (!(i & st)) {
          const int p = h[i], q2 = h[i + st];
          h[i] = p + q2;
          h[i + st] = p - q2;
        }
#pragma unroll
    for (int st = 1; st < SEG; st <<= 1)
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        const int p = __shfl_xor(h[i], st, 64);
        h[i] = (sg & st) ? (p - h[i]) : (h[i] + p);
      }
  } else {
#pragma unroll
    for (int i = 0; i < FPT; ++i) h[i] = 0;
  }
  const double* xt = &L.Xt[rloc][sg * FPT];
#pragma unroll
  for (int i = 0; i < FPT; i += 2) {
    uint32_t pk = 0;
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int f = sg * FPT + i + u;
      const double o = fma(sgs[f], s * (double)h[i + u], xt[i + u]);
      pk |= (uint32_t)f64_to_bf16(o) << (16 * u);
    }
    ow[i / 2] = pk;
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_decode(const DecodeArgs a) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  constexpr int CP = CodecLds<D>::CP;
  const int tl = blockIdx.z, n = blockIdx.y;
  const EncodeTable& e = a.t[tl];
  const int T = a.T;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  const int tb = blockIdx.x * CODEC_CHUNK, te = min(T, tb + CODEC_CHUNK);
  if (e.chain < 0) {  // (T, D): X stored verbatim
    const uint4* src = (const uint4*)(e.rec + e.off_core) + ((int64_t)n * T + tb) * D / 8;
    uint4* dst = (uint4*)a.out[tl] + ((int64_t)n * T + tb) * D / 8;
    for (int64_t i = tid; i < (int64_t)(te - tb) * D / 8; i += 256) dst[i] = src[i];
    return;
  }
  __shared__ CodecLds<D> L;
  __shared__ double sgs[D];  // sigma_f / sqrt(D)
  CD_MARK(0);
  const DecodeSrc d = codec_prepare<D>(L, sgs, e, n, T);
  uint16_t* out = (uint16_t*)a.out[tl];
  CD_MARK(1);
  for (int t0 = tb; t0 < te; t0 += CP) {
    uint32_t ow[FPT / 2];
    codec_decode_tile<D>(L, sgs, e, d, n, T, t0, ow);
    if (t0 == tb) CD_MARK(2);
    const int64_t row = (int64_t)n * T + t0 + rloc;
    uint4* orow = (uint4*)(out + row * D + sg * FPT);
    orow[0] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
    orow[1] = make_uint4(ow[4], ow[5], ow[6], ow[7]);
    __syncthreads();
    if (t0 == tb) CD_MARK(3);
  }
  CD_MARK(4);
}

// ---------------------------------------------------------------- fused decode + attention
// O = softmax(Q K^T * scale) V for one layer group, K and V rebuilt tile by tile from their
// records exactly as k_decode writes them (bf16 values), never stored.  Workgroup (chunk c,
// slice n, group g) takes the tokens [c ach, (c + 1) ach) of slice n and all nq queries of
// that slice: scores of the chunk from the K tiles, the chunk's softmax statistics (max m and
// sum l of exp(s - m)), then sum_t exp(s_t - m) V_t from the V tiles, all in fp32.
// k_attend_merge combines the chunks: O = sum_c e^{m_c - M} O_c / sum_c e^{m_c - M} l_c.
template <int D>
__device__ __forceinline__ void attend_rows(CodecLds<D>& L, const double* sgs, const EncodeTable& e,
                                            const DecodeSrc& d, int n, int T, int t0, float (*Xd)[D + 4]) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  uint32_t ow[FPT / 2];
  if (e.chain < 0) {  // (T, D): the record holds X
    const uint4* src = (const uint4*)((const uint16_t*)(e.rec + e.off_core) + ((int64_t)n * T + t0 + rloc) * D +
                                      sg * FPT);
    const uint4 w0 = src[0], w1 = src[1];
    ow[0] = w0.x; ow[1] = w0.y; ow[2] = w0.z; ow[3] = w0.w;
    ow[4] = w1.x; ow[5] = w1.y; ow[6] = w1.z; ow[7] = w1.w;
  } else {
    codec_decode_tile<D>(L, sgs, e, d, n, T, t0, ow);
  }
#pragma unroll
  for (int i = 0; i < FPT / 2; ++i) {
    Xd[rloc][sg * FPT + 2 * i] = bf16_to_f32((uint16_t)(ow[i] & 0xFFFFu));
    Xd[rloc][sg * FPT + 2 * i + 1] = bf16_to_f32((uint16_t)(ow[i] >> 16));
  }
}

template <int D>
__global__ __launch_bounds__(256) void k_attend(const AttendArgs a) {
  constexpr int CP = CodecLds<D>::CP;
  constexpr int OPT = ATT_QMAX * D / 256;  // outputs per thread at most
  const int c = blockIdx.x, n = blockIdx.y, g = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int T = a.T, nq = a.nq;
  const EncodeTable& ek = a.k[g];
  const EncodeTable& ev = a.v[g];
  const int tb = c * a.ach, te = min(T, tb + a.ach), ntok = te - tb;
  __shared__ CodecLds<D> L;
  __shared__ double sgs[D];
  __shared__ float Xd[CP][D + 4];
  __shared__ float Qs[ATT_QMAX][D];
  __shared__ float P[ATT_QMAX][ATT_CHMAX];  // scaled scores, then exp(s - m)
  __shared__ float stat[ATT_QMAX][2];
  for (int idx = tid; idx < nq * D; idx += 256)
    Qs[idx / D][idx % D] = bf16_to_f32(a.q[g][((int64_t)n * nq) * D + idx]);
  // ---- scores of the chunk against the K tiles
  DecodeSrc d{};
  if (ek.chain >= 0) d = codec_prepare<D>(L, sgs, ek, n, T);
  __syncthreads();
  for (int t0 = tb; t0 < te; t0 += CP) {
    attend_rows<D>(L, sgs, ek, d, n, T, t0, Xd);
    __syncthreads();
    for (int pr = tid; pr < nq * CP; pr += 256) {
      const int i = pr / CP, tt = pr - i * CP;
      float s0 = 0.f, s1 = 0.f;
#pragma unroll 8
      for (int f = 0; f < D; f += 2) {
        s0 = fmaf(Qs[i][f], Xd[tt][f], s0);
        s1 = fmaf(Qs[i][f + 1], Xd[tt][f + 1], s1);
      }
      P[i][t0 - tb + tt] = (s0 + s1) * a.scale;
    }
    __syncthreads();
  }
  // ---- softmax statistics of the chunk, one wave per query
  for (int i = wave; i < nq; i += 4) {
    float m = -INFINITY;
    for (int t = lane; t < ntok; t += 64) m = fmaxf(m, P[i][t]);
    m = wave_max_f32(m);
    float l = 0.f;
    for (int t = lane; t < ntok; t += 64) {
      const float p = expf(P[i][t] - m);
      P[i][t] = p;
      l += p;
    }
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    if (lane == 0) {
      stat[i][0] = m;
      stat[i][1] = l;
    }
  }
  __syncthreads();
  // ---- sum_t p_t V_t from the V tiles; thread owns outputs tid, tid + 256, ...
  float acc[OPT];
#pragma unroll
  for (int j = 0; j < OPT; ++j) acc[j] = 0.f;
  if (ev.chain >= 0) d = codec_prepare<D>(L, sgs, ev, n, T);
  __syncthreads();
  for (int t0 = tb; t0 < te; t0 += CP) {
    attend_rows<D>(L, sgs, ev, d, n, T, t0, Xd);
    __syncthreads();
#pragma unroll
    for (int j = 0; j < OPT; ++j) {
      const int o = tid + 256 * j;
      if (o < nq * D) {
        const int i = o / D, f = o - i * D;
        float s = acc[j];
#pragma unroll 8
        for (int tt = 0; tt < CP; ++tt) s = fmaf(P[i][t0 - tb + tt], Xd[tt][f], s);
        acc[j] = s;
      }
    }
    __syncthreads();
  }
  float* part = a.part + ((((int64_t)g * a.N + n) * a.nchunk + c) * nq) * (D + 2);
#pragma unroll
  for (int j = 0; j < OPT; ++j) {
    const int o = tid + 256 * j;
    if (o < nq * D) part[(o / D) * (D + 2) + (o % D)] = acc[j];
  }
  if (tid < nq) {
    part[tid * (D + 2) + D] = stat[tid][0];
    part[tid * (D + 2) + D + 1] = stat[tid][1];
  }
}

__global__ __launch_bounds__(256) void k_attend_merge(const AttendArgs a) {
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  const int D = a.D, g = blockIdx.y;
  if (idx >= (int64_t)a.N * a.nq * D) return;
  const int f = (int)(idx % D);
  const int64_t ni = idx / D;  // n * nq + i
  const int64_t n = ni / a.nq, i = ni - n * a.nq;
  const float* base = a.part + (((int64_t)g * a.N + n) * a.nchunk * a.nq + i) * (D + 2);
  const int64_t cs = (int64_t)a.nq * (D + 2);  // chunk stride
  float M = -INFINITY;
  for (int c = 0; c < a.nchunk; ++c) M = fmaxf(M, base[c * cs + D]);
  float num = 0.f, den = 0.f;
  for (int c = 0; c < a.nchunk; ++c) {
    const float w = expf(base[c * cs + D] - M);
    num = fmaf(w, base[c * cs + f], num);
    den = fmaf(w, base[c * cs + D + 1], den);
  }
  a.out[g][idx] = num / den;
}

hipError_t launch_attend(const AttendArgs& a, hipStream_t s) {
  if (a.nq < 1 || a.nq > ATT_QMAX || a.ach < 1 || a.ach > ATT_CHMAX || a.nchunk < 1 || a.N < 1 || a.ng < 1 ||
      a.ng > ATT_GMAX)
    return hipErrorInvalidValue;
  const int cp = a.D == 128 ? CodecLds<128>::CP : CodecLds<64>::CP;
  if (a.T % cp || a.ach % cp || (int64_t)a.nchunk * a.ach < a.T) return hipErrorInvalidValue;
  const dim3 grid(a.nchunk, a.N, a.ng);
  if (a.D == 128)
    hipLaunchKernelGGL(k_attend<128>, grid, dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_attend<64>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  const int64_t tot = (int64_t)a.N * a.nq * a.D;
  hipLaunchKernelGGL(k_attend_merge, dim3((unsigned)((tot + 255) / 256), a.ng), dim3(256), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_encode(const EncodeArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(k_rec_header, dim3(a.ntab), dim3(64), 0, s, a);
  for (int which = 0; which < 3; ++which)
    hipLaunchKernelGGL(k_rec_section, dim3(512, a.ntab), dim3(256), 0, s, a, which);
  const dim3 grid((a.T + CODEC_CHUNK - 1) / CODEC_CHUNK, a.N, a.ntab);
  if (a.T % CodecLds<64>::CP) return hipErrorInvalidValue;
  if (a.D == 128)
    hipLaunchKernelGGL(k_encode_resid<128>, grid, dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_encode_resid<64>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((a.T + CODEC_CHUNK - 1) / CODEC_CHUNK, a.N, a.ntab);
  if (a.T % CodecLds<64>::CP) return hipErrorInvalidValue;
  if (a.D == 128)
    hipLaunchKernelGGL(k_decode<128>, grid, dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_decode<64>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jolt
