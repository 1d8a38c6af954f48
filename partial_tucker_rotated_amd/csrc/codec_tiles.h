// Tile-level pieces of the record codec shared by the encoder, the decoder, fused
// attention and streaming admission: b-bit code packing, the encoder's fp64 reconstruction
// operand Rm and X~ tiles (fp64 MFMA), the row rotation + block quantizer, and the fp32
// register decode of one token tile.  Included by the codec translation units only.
#pragma once
#include "jolt_internal.h"


namespace jolt {

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

// ---------------------------------------------------------------- encoder reconstruction
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
  // kind 0 stages U_d transposed ([j][f], rd x D doubles) in the X~ tile, which is not in use
  // before the first tile of the workgroup
  double* Us = &L.Xt[0][0];
  static_assert(sizeof(L.Xt) >= sizeof(double) * JOLT_KMAX * D, "U_d staging fits the X~ tile");
  if (kind == 0) {
    for (int idx = tid; idx < K * rd; idx += 256) {
      const int k = idx / rd, j = idx - k * rd;
      L.Gs[k][j] = (double)G[k * gs + j];
    }
    for (int idx = tid; idx < rd * D; idx += 256) {
      const int j = idx / D, f = idx - j * D;
      Us[idx] = (double)Ud[f * us + j];
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
        for (int j = 0; j < rd; ++j) v = fma(L.Gs[k][j], Us[j * D + f], v);
      }
    }
    L.Rm[k][f] = v;
  }
  __syncthreads();
}

// Per-thread global inputs of one pass of CP tokens.  The codec kernels fetch them one pass
// ahead, so that their memory latency overlaps the previous pass's arithmetic.
struct TileIn {
  _Float16 a[JOLT_KMAX / 4];  // A operands of the X~ products (this lane's token, k = 4 st + lk)
  uint32_t w[8];              // decode: the b-bit codes of the thread's 16 features (b / 2 words);
                              // encode and verbatim rows: the 16 bf16 values (8 words)
  float s;                    // decode: the row's scale
};

// X~ of tokens tok0 .. tok0 + CP - 1 into L.Xt.  Lrow(t) = fp16 row of L for token t
// (row stride ls); K a multiple of 4.  Wave w computes token tile w / (CT/4) and column
// tiles 4 (w % (CT/4)) ..+3 (CT = D/16).  Output of a 16 x 16 tile: element (i, j) in
// lane 16 (i & 3) + j, register i >> 2; A element (i, k) in lane i + 16 k, B element
// (k, j) in lane j + 16 k.  codec_fetch_a loads this lane's A operands, codec_xtilde_in
// forms the tile from them.
template <int D>
__device__ __forceinline__ void codec_fetch_a(TileIn& in, const _Float16* Lb, int64_t ls, int K, int tok0) {
  constexpr int WPT = D / 64;  // waves per token tile
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, li = lane & 15, lk = lane >> 4;
  const _Float16* arow = Lb + (int64_t)(tok0 + 16 * tt + li) * ls + lk;
#pragma unroll
  for (int st = 0; st < JOLT_KMAX / 4; ++st) in.a[st] = 4 * st < K ? arow[4 * st] : (_Float16)0.0f;
}

template <int D>
__device__ __forceinline__ void codec_xtilde_in(CodecLds<D>& L, const TileIn& in, int K) {
  constexpr int WPT = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, c0 = (w % WPT) * 4;
  const int li = lane & 15, lk = lane >> 4;
  double4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (double4_t){0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int st = 0; st < JOLT_KMAX / 4; ++st)
    if (4 * st < K) {
      const double av = (double)in.a[st];
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const double bv = L.Rm[4 * st + lk][16 * (c0 + c) + li];
        acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, bv, acc[c], 0, 0, 0);
      }
    }
#pragma unroll
  for (int c = 0; c < 4; ++c)
#pragma unroll
    for (int r = 0; r < 4; ++r) L.Xt[16 * tt + 4 * r + lk][16 * (c0 + c) + li] = acc[c][r];
}

template <int D>
__device__ __forceinline__ void codec_xtilde(CodecLds<D>& L, const _Float16* Lb, int64_t ls, int K, int tok0) {
  TileIn in;
  codec_fetch_a<D>(in, Lb, ls, K, tok0);
  codec_xtilde_in<D>(L, in, K);
}

// the 16 bf16 values of this thread's segment of row `row` (rows of D values at x)
template <int D>
__device__ __forceinline__ void codec_fetch_row(TileIn& in, const uint16_t* x, int64_t row) {
  const int sg = threadIdx.x % (D / 16);
  const uint4* xr = (const uint4*)(x + row * D + sg * 16);
  const uint4 q0 = xr[0], q1 = xr[1];
  in.w[0] = q0.x; in.w[1] = q0.y; in.w[2] = q0.z; in.w[3] = q0.w;
  in.w[4] = q1.x; in.w[5] = q1.y; in.w[6] = q1.z; in.w[7] = q1.w;
}

// Partner value of an fp64 across lanes l and l ^ X (X = 1, 2: quad permutation by DPP;
// X = 4: ds_swizzle in xor mode within groups of 32 lanes).  All lanes must be active.
template <int X>
__device__ __forceinline__ double lane_xor_f64(double v) {
  if (X == 1) return dpp_f64<0xB1>(v);
  if (X == 2) return dpp_f64<0x4E>(v);
  const long long u = __double_as_longlong(v);
  constexpr int pat = (X << 10) | 0x1F;  // and mask 31, or mask 0, xor mask X
  const int lo = __builtin_amdgcn_ds_swizzle((int)u, pat);
  const int hi = __builtin_amdgcn_ds_swizzle((int)(u >> 32), pat);
  return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Rotation and block quantization of one row of D residual values held by D / 16
// consecutive lanes, 16 features each (segment sg): y holds this thread's residual on
// entry and Q r (Q = H diag(sigma) / sqrt(D)) on exit; q receives the codes
// clip(rint(y / s), -qmax - 1, qmax) decided in fp64 with the fp32 scale s = max|y| / qmax,
// which is returned.  sgn points at sigma for this thread's 16 features.  Called by all
// threads of the workgroup.
// y / s is formed as y * (1 / s); where that product lies within 2^-36 of a rounding tie
// (it is within a few ulp, about 2^-45, of the correctly rounded quotient) the quotient
// itself decides, so the codes equal those of rint(y / s) with an IEEE fp64 division.
template <int D>
__device__ __forceinline__ float codec_rotq(double (&y)[16], const int8_t* sgn, int sg, int qmax, int (&q)[16]) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  static_assert(SEG == 4 || SEG == 8, "rows of 64 or 128 values");
#pragma unroll
  for (int i = 0; i < FPT; ++i) y[i] = sgn[i] < 0 ? -y[i] : y[i];
#pragma unroll
  for (int st = 1; st < FPT; st <<= 1)
#pragma unroll
    for (int i = 0; i < FPT; ++i)
      if (!(i & st)) {
        const double p = y[i], q2 = y[i + st];
        y[i] = p + q2;
        y[i + st] = p - q2;
      }
  // butterflies across the row's lanes: lane sg keeps p + y (bit clear) or p - y (bit set)
  // of its value y and its partner's p, i.e. fma(+-1, y, p)
  auto cross = [&](auto xs) {
    constexpr int X = decltype(xs)::value;
    const double sn = (sg & X) ? -1.0 : 1.0;
#pragma unroll
    for (int i = 0; i < FPT; ++i) y[i] = fma(sn, y[i], lane_xor_f64<X>(y[i]));
  };
  cross(std::integral_constant<int, 1>());
  cross(std::integral_constant<int, 2>());
  if (SEG == 8) cross(std::integral_constant<int, 4>());
  const double isq = 1.0 / sqrt((double)D);
  double m = 0.0;
#pragma unroll
  for (int i = 0; i < FPT; ++i) {
    y[i] *= isq;
    m = fmax(m, fabs(y[i]));
  }
  m = fmax(m, lane_xor_f64<1>(m));
  m = fmax(m, lane_xor_f64<2>(m));
  if (SEG == 8) m = fmax(m, lane_xor_f64<4>(m));
  const float sc = (float)(m / (double)qmax);
  const double sd = (double)sc;
  const double inv = sd > 0.0 ? 1.0 / sd : 0.0;
#pragma unroll
  for (int i = 0; i < FPT; ++i) {
    double u = y[i] * inv;
    double v = rint(u);
    if (fabs(fabs(u - v) - 0.5) < 0x1p-36) v = rint(y[i] / sd);  // near a tie (never when sd = 0)
    v = fmin(fmax(v, (double)(-qmax - 1)), (double)qmax);
    q[i] = (int)v;
  }
  return sc;
}

// b-bit codes of this thread's 16 features of row `row` into the packed code stream
__device__ __forceinline__ void codec_store_codes(const int (&q)[16], uint32_t* codes, int64_t row, int D, int sg,
                                                  int b) {
  uint32_t* cw = codes + (row * D + sg * 16) * b / 32;
  if (b == 2) pack_codes<2>(q, cw);
  else if (b == 4) pack_codes<4>(q, cw);
  else pack_codes<8>(q, cw);
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

// ---------------------------------------------------------------- decode in registers (fp32)
// X^ = X~ + sigma_f / sqrt(D) * s_t * (H q)_f, evaluated in fp32 and rounded once to bf16
// (round to nearest even).  Wave w owns token tile tt = w / WPT (16 tokens) and the
// features 64 h .. 64 h + 63, h = w % WPT (WPT = D / 64 waves per token tile).  Column
// j = li of product tile c stands for feature f = 64 h + 4 li + c, so a lane ends up with 4
// consecutive features of its tokens (one 8-byte store per token).  Both products land in
// the same register layout, element (token 4 lk + r, feature 64 h + 4 li + c) in lane
// 16 lk + li, register r of tile c:
//   X~ = L Rm with v_mfma_f32_16x16x32_f16: A = the fp16 rows of L (row i in lane i + 16 g,
//   k = 8 g .. 8 g + 7), B = Rm split into fp16 hi + lo parts (k = 8 g .. 8 g + 7 of column
//   j in lane j + 16 g): fp16 products are exact in fp32, the split keeps ~22 bits of Rm;
//   Rm itself (G_n U_d^T, G_n or U_d^T) is formed once per workgroup in fp32 from the fp16
//   record values.  The lo product is skipped where Rm is fp16 already (G_n, U_d^T).
//   (H q) with v_mfma_i32_16x16x32_i8: q the b-bit codes as int8, H the Sylvester Hadamard
//   matrix (+-1 as int8), exact in int32 (|H q| <= 128 * 128), A = the codes of token i in
//   lane i + 16 g, product s taking k = (D / 4) g + 8 s .. + 7 (the order of k in a sum is
//   free, and this one gives each lane D b / 32 contiguous bytes of codes).
//   H[k][f] = (-1)^popcount(k & f): for k = (D / 4) g + 8 s + e (e < 8) the bits of e and of
//   (D / 4) g + 8 s do not overlap, so the 8 bytes a lane feeds are a pattern fixed by f & 7 =
//   4 (li & 1) + c, negated when popcount(((D / 4) g + 8 s) & f) is odd.
// The residual term is (sigma_f / sqrt(D) * s_t) * (H q)_f, added to X~ by one fp32 FMA.
typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef int int4_v __attribute__((ext_vector_type(4)));

template <int D>
struct DecLds {
  float Rm[JOLT_KMAX][D + 4];             // reconstruction operand, rows k < K
  union {
    struct {                              // while Rm is formed (G_n U_d^T only)
      float Gs[JOLT_KMAX][JOLT_KMAX + 1];  // staged core rows
      float Us[JOLT_KMAX][D + 4];          // staged U_d^T
    };
    struct {                              // afterwards: the B operands of the X~ product,
      half8_t Bh[D / 64][4][4][16];       // [h][c][g][li] for lane (li, g) of the waves of
      half8_t Bl[D / 64][4][4][16];       // feature block h (16 lanes: 256 consecutive bytes)
    };
  };
};

// What a workgroup needs to rebuild rows of slice n of one record (chain >= 0).
struct DecSrc {
  int K;                 // inner dimension of X~ = L Rm
  int lo;                // Rm needs its lo part (G_n U_d^T)
  const _Float16* Lb;    // L rows (token-major, stride ls)
  int64_t ls;
  const uint8_t* codes;
  const float* scales;
};

// Signs sigma_f / sqrt(D) from the record header into sgs (fp32), and the slice's Rm (fp32)
// into L.Rm.  Ends with a barrier.
template <int D>
__device__ DecSrc dec_prepare(DecLds<D>& L, float* sgs, const EncodeTable& e, int n, int T) {
  const int tid = threadIdx.x;
  const char* rec = e.rec;
  const uint32_t* sbits = (const uint32_t*)(rec + 128);
  const float isq = (float)(1.0 / sqrt((double)D));
  for (int f = tid; f < D; f += 256) sgs[f] = ((sbits[f >> 5] >> (f & 31)) & 1u) ? -isq : isq;
  const _Float16* Ut = (const _Float16*)(rec + e.off_ut);
  const _Float16* Ud = (const _Float16*)(rec + e.off_ud);
  const _Float16* Gc = (const _Float16*)(rec + e.off_core);
  DecSrc d;
  d.codes = (const uint8_t*)(rec + e.off_codes);
  d.scales = (const float*)(rec + e.off_scales);
  if (e.chain == 5) {  // Rm = U_d^T, L = the slice's per-token core rows
    d.K = e.rd;
    d.lo = 0;
    d.Lb = Gc + (int64_t)n * T * e.rd;
    d.ls = e.rd;
    for (int idx = tid; idx < JOLT_KMAX * D; idx += 256) {
      const int k = idx / D, f = idx - k * D;
      L.Rm[k][f] = k < d.K ? (float)Ud[f * e.rd + k] : 0.0f;
    }
  } else if (e.chain == 4) {  // Rm = G_n (r_d = D), L = U_T
    d.K = e.rT;
    d.lo = 0;
    d.Lb = Ut;
    d.ls = e.rT;
    const _Float16* G = Gc + (int64_t)n * e.rT * D;
    for (int idx = tid; idx < JOLT_KMAX * D; idx += 256) {
      const int k = idx / D, f = idx - k * D;
      L.Rm[k][f] = k < d.K ? (float)G[k * D + f] : 0.0f;
    }
  } else {  // Rm = G_n U_d^T, L = U_T; fp16 products exact in fp32, summed over j in order
    d.K = e.rT;
    d.lo = 1;
    d.Lb = Ut;
    d.ls = e.rT;
    const int rd = e.rd;
    const _Float16* G = Gc + (int64_t)n * e.rT * rd;
    for (int idx = tid; idx < d.K * rd; idx += 256) {
      const int k = idx / rd, j = idx - k * rd;
      L.Gs[k][j] = (float)G[k * rd + j];
    }
    for (int idx = tid; idx < rd * D; idx += 256) {
      const int j = idx / D, f = idx - j * D;
      L.Us[j][f] = (float)Ud[f * rd + j];
    }
    __syncthreads();
    for (int idx = tid; idx < JOLT_KMAX * D; idx += 256) {
      const int k = idx / D, f = idx - k * D;
      float v = 0.0f;
      if (k < d.K)
        for (int j = 0; j < rd; ++j) v = fmaf(L.Gs[k][j], L.Us[j][f], v);
      L.Rm[k][f] = v;
    }
  }
  __syncthreads();
  return d;
}

// The B operands of the X~ product into L.Bh / L.Bl: Rm[8 g + e][64 h + 4 li + c] split into
// fp16 hi and lo parts (zero for k >= K), for every (h, c, g, li).  Ends with a barrier.
template <int D>
__device__ __forceinline__ void dec_bops(DecLds<D>& L) {
  for (int idx = threadIdx.x; idx < (D / 64) * 4 * 4 * 16; idx += 256) {
    const int li = idx & 15, g = (idx >> 4) & 3, c = (idx >> 6) & 3, h = idx >> 8;
    const int f = 64 * h + 4 * li + c;
    half8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = L.Rm[8 * g + e][f];
      const _Float16 hv = (_Float16)v;
      hi[e] = hv;
      lo[e] = (_Float16)(v - (float)hv);
    }
    L.Bh[h][c][g][li] = hi;
    L.Bl[h][c][g][li] = lo;
  }
  __syncthreads();
}

struct DecIn {
  half8_t a;   // L row of token li, k = 8 lk .. 8 lk + 7
  uint2 q[4];  // codes of token li, k = (D / 4) lk + 8 s .. + 7 (b bytes each)
  float4_t s;  // scales of tokens 4 lk + r
};

// WIDE: the token tile of wave w is w (one wave covers all D features of its tile);
// otherwise w / (D / 64).  TOKSCALE: in.s[0] is the scale of the lane's own token li (the
// transposed tiles of fused attention) instead of those of tokens 4 lk + r.
template <int D, bool WIDE = false, bool TOKSCALE = false>
__device__ __forceinline__ void dec_fetch(DecIn& in, const DecSrc& d, int b, int n, int T, int t0) {
  constexpr int WPT = WIDE ? 1 : D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, li = lane & 15, lk = lane >> 4;
  const int tok = t0 + 16 * tt + li;
  const _Float16* arow = d.Lb + (int64_t)tok * d.ls + 8 * lk;
  if (8 * lk + 8 <= d.K) {
    in.a = *(const half8_t*)arow;
  } else {
#pragma unroll
    for (int e = 0; e < 8; ++e) in.a[e] = (_Float16)0.0f;
    if (8 * lk < d.K) {  // K = 4: half a group
      const uint2 v = *(const uint2*)arow;
      in.a[0] = __builtin_bit_cast(_Float16, (uint16_t)(v.x & 0xFFFFu));
      in.a[1] = __builtin_bit_cast(_Float16, (uint16_t)(v.x >> 16));
      in.a[2] = __builtin_bit_cast(_Float16, (uint16_t)(v.y & 0xFFFFu));
      in.a[3] = __builtin_bit_cast(_Float16, (uint16_t)(v.y >> 16));
    }
  }
  if (b > 0) {
    // the lane's codes are k = (D / 4) lk .. (D / 4) lk + D / 4 - 1 of its token: D b / 32
    // contiguous bytes (k block st of the products takes k = (D / 4) lk + 8 st .. + 7)
    const int64_t row = (int64_t)n * T + tok;
    const uint8_t* cb = d.codes + ((row * D + (D / 4) * lk) * b >> 3);
    if (D == 128) {
      if (b == 8) {
        const uint4 u = *(const uint4*)cb, v = *(const uint4*)(cb + 16);
        in.q[0] = make_uint2(u.x, u.y);
        in.q[1] = make_uint2(u.z, u.w);
        in.q[2] = make_uint2(v.x, v.y);
        in.q[3] = make_uint2(v.z, v.w);
      } else if (b == 4) {
        const uint4 u = *(const uint4*)cb;
        in.q[0] = make_uint2(u.x, 0u);
        in.q[1] = make_uint2(u.y, 0u);
        in.q[2] = make_uint2(u.z, 0u);
        in.q[3] = make_uint2(u.w, 0u);
      } else {
        const uint2 u = *(const uint2*)cb;
        in.q[0] = make_uint2(u.x & 0xFFFFu, 0u);
        in.q[1] = make_uint2(u.x >> 16, 0u);
        in.q[2] = make_uint2(u.y & 0xFFFFu, 0u);
        in.q[3] = make_uint2(u.y >> 16, 0u);
      }
    } else {  // D = 64: two k blocks
      if (b == 8) {
        const uint4 u = *(const uint4*)cb;
        in.q[0] = make_uint2(u.x, u.y);
        in.q[1] = make_uint2(u.z, u.w);
      } else if (b == 4) {
        const uint2 u = *(const uint2*)cb;
        in.q[0] = make_uint2(u.x, 0u);
        in.q[1] = make_uint2(u.y, 0u);
      } else {
        const uint32_t u = *(const uint32_t*)cb;
        in.q[0] = make_uint2(u & 0xFFFFu, 0u);
        in.q[1] = make_uint2(u >> 16, 0u);
      }
    }
    if (TOKSCALE) in.s[0] = d.scales[(int64_t)n * T + tok];
    else in.s = *(const float4_t*)(d.scales + (int64_t)n * T + t0 + 16 * tt + 4 * lk);
  }
}

// 8 b-bit codes (packed little-endian in the first b bytes of w) as 8 sign-extended int8
// bytes
__device__ __forceinline__ uint2 codes_to_i8(uint2 w, int b) {
  if (b == 8) return w;
  uint32_t lo = 0, hi = 0;
  const int m = (1 << b) - 1, sb = 1 << (b - 1);
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const int f0 = (int)((w.x >> (b * e)) & m), f1 = (int)((w.x >> (b * (e + 4))) & m);
    lo |= (uint32_t)(uint8_t)((f0 ^ sb) - sb) << (8 * e);
    hi |= (uint32_t)(uint8_t)((f1 ^ sb) - sb) << (8 * e);
  }
  return make_uint2(lo, hi);
}

// decoded values of this lane in fp32: out[c][r] = X^(token 4 lk + r, feature 64 h + 4 li + c)
// Bh, Bl: the B operands in the [h][c][g][li] layout of DecLds (a record's own, or a copy)
template <int D>
__device__ __forceinline__ void dec_vals(const half8_t* Bh, const half8_t* Bl, const float* sgs, const DecSrc& d,
                                         int b, const DecIn& in, float4_t (&out)[4]) {
  constexpr int WPT = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int h = w % WPT, li = lane & 15;
  const int f0 = 64 * h + 4 * li, lk = lane >> 4;
  long av[D / 32];  // the codes as int8 A operands, shared by the four tiles
  if (b > 0) {
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      const uint2 q8 = codes_to_i8(in.q[st], b);
      av[st] = (long)(((uint64_t)q8.y << 32) | q8.x);
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const int bi = ((h * 4 + c) * 4 + lk) * 16 + li;
    out[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(in.a, Bh[bi], (float4_t){0.0f, 0.0f, 0.0f, 0.0f}, 0, 0, 0);
    if (d.lo) out[c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(in.a, Bl[bi], out[c], 0, 0, 0);
    if (b > 0) {
      // byte e of the Hadamard operand: (-1)^popcount(e & (f & 7)), f & 7 = 4 (li & 1) + c
      const int f7 = (f0 + c) & 7;
      uint64_t pat = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) pat |= (uint64_t)((__builtin_popcount(e & f7) & 1) ? 0xFFu : 0x01u) << (8 * e);
      int4_v hq = (int4_v){0, 0, 0, 0};
#pragma unroll
      for (int st = 0; st < D / 32; ++st) {
        const bool odd = __builtin_popcount(((D / 4) * lk + 8 * st) & (f0 + c)) & 1;
        const long bv = (long)(odd ? (pat ^ 0xFEFEFEFEFEFEFEFEull) : pat);
        hq = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[st], bv, hq, 0, 0, 0);
      }
      const float sg = sgs[f0 + c];
#pragma unroll
      for (int r = 0; r < 4; ++r) out[c][r] = fmaf(sg * in.s[r], (float)hq[r], out[c][r]);
    }
  }
}

__device__ __forceinline__ uint16_t dec_bf16(float v) { return __builtin_bit_cast(uint16_t, (__bf16)v); }

// stores a pass decoded by dec_vals: rows of slice n from rowbase = n T + t0, tokens
// 16 tt + 4 lk + r, 4 consecutive features per lane (8 bytes), bf16 round to nearest even
template <int D>
__device__ __forceinline__ void dec_store(uint16_t* out, int64_t rowbase, const float4_t (&v)[4]) {
  constexpr int WPT = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, f0 = 64 * (w % WPT) + 4 * (lane & 15), lk = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint2 pk = make_uint2((uint32_t)dec_bf16(v[0][r]) | ((uint32_t)dec_bf16(v[1][r]) << 16),
                                (uint32_t)dec_bf16(v[2][r]) | ((uint32_t)dec_bf16(v[3][r]) << 16));
    *(uint2*)(out + (rowbase + 16 * tt + 4 * lk + r) * D + f0) = pk;
  }
}

// ---------------------------------------------------------------- wide register decode
// The decoder's own layout: wave w owns the 16 tokens 16 w .. 16 w + 15 of a pass of 64 and
// all D features, so the codes and L rows of a token are read once and the int8 A operands
// serve every output tile of the wave.  Column li of product tile (h, c), h < NH = D / 64,
// stands for feature f = 4 NH li + 4 h + c: a lane holds 4 NH consecutive features of each of
// its tokens (one 16-byte store per token at D = 128).  The Hadamard B operands depend only
// on (h, c, k block, lane) and b; they are formed once per workgroup into LDS.  For b = 4
// the bytes of a k block carry the codes in the order 0, 2, 4, 6, 1, 3, 5, 7 (even nibbles,
// then odd nibbles), and the Hadamard operands follow the same order.
template <int D>
__device__ __forceinline__ int dw_feat(int h, int c, int li) {
  return 4 * (D / 64) * li + 4 * h + c;
}

// code index carried by byte p of a k block
__device__ __forceinline__ int dw_code_of_byte(int p, int b) { return b == 4 ? (p < 4 ? 2 * p : 2 * p - 7) : p; }

// B operands of the X~ product for the wide layout: L.Bh / L.Bl [h][c][g][li] =
// Rm[8 g + e][dw_feat(h, c, li)] split into fp16 hi and lo.  Ends with a barrier.
template <int D>
__device__ __forceinline__ void dec_bops_w(DecLds<D>& L) {
  for (int idx = threadIdx.x; idx < (D / 64) * 4 * 4 * 16; idx += 256) {
    const int li = idx & 15, g = (idx >> 4) & 3, c = (idx >> 6) & 3, h = idx >> 8;
    const int f = dw_feat<D>(h, c, li);
    half8_t hi, lo;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float v = L.Rm[8 * g + e][f];
      const _Float16 hv = (_Float16)v;
      hi[e] = hv;
      lo[e] = (_Float16)(v - (float)hv);
    }
    L.Bh[h][c][g][li] = hi;
    L.Bl[h][c][g][li] = lo;
  }
  __syncthreads();
}

// Hadamard B operands [h][c][st][lane] (NH * 4 * D / 32 * 64 entries of 8 bytes): byte p of
// lane (li, g) in k block st is H[k][f] = (-1)^popcount(k & f) as int8 for
// k = (D / 4) g + 8 st + dw_code_of_byte(p, b), f = dw_feat(h, c, li).  No barrier.
template <int D>
__device__ __forceinline__ void dec_hops_w(uint64_t* Hb, int b) {
  constexpr int NST = D / 32;
  for (int idx = threadIdx.x; idx < (D / 64) * 4 * NST * 64; idx += 256) {
    const int lane = idx & 63, st = (idx >> 6) % NST, hc = idx / (64 * NST);
    const int h = hc >> 2, c = hc & 3, li = lane & 15, g = lane >> 4;
    const int f = dw_feat<D>(h, c, li), kb = (D / 4) * g + 8 * st;
    uint64_t v = 0;
#pragma unroll
    for (int p = 0; p < 8; ++p)
      v |= (uint64_t)((__builtin_popcount((kb + dw_code_of_byte(p, b)) & f) & 1) ? 0xFFu : 0x01u) << (8 * p);
    Hb[idx] = v;
  }
}

// 8 b-bit codes (packed little-endian in the first b bytes of w) as 8 int8 bytes in the
// order of dw_code_of_byte
__device__ __forceinline__ uint64_t codes_to_i8_w(uint2 w, int b) {
  if (b == 8) return ((uint64_t)w.y << 32) | w.x;
  if (b == 4) {  // nibbles 0, 2, 4, 6 -> bytes 0..3, nibbles 1, 3, 5, 7 -> bytes 4..7
    const uint32_t lo = w.x & 0x0F0F0F0Fu, hi = (w.x >> 4) & 0x0F0F0F0Fu;
    // sign extension within each byte: bit 3 set -> bits 4..7 set (no carry across bytes)
    const uint32_t slo = lo | ((lo & 0x08080808u) * 0x1Eu), shi = hi | ((hi & 0x08080808u) * 0x1Eu);
    return ((uint64_t)shi << 32) | slo;
  }
  const uint2 q = codes_to_i8(w, b);
  return ((uint64_t)q.y << 32) | q.x;
}

// decoded values of this lane in fp32: out[h][c][r] = X^(token 4 lk + r of the wave's tile,
// feature dw_feat(h, c, li))
template <int D>
__device__ __forceinline__ void dec_vals_w(const DecLds<D>& L, const uint64_t* Hb, const float* sgs,
                                           const DecSrc& d, int b, const DecIn& in,
                                           float4_t (&out)[D / 64][4]) {
  constexpr int NH = D / 64, NST = D / 32;
  const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
  long av[NST];
  if (b > 0) {
#pragma unroll
    for (int st = 0; st < NST; ++st) av[st] = (long)codes_to_i8_w(in.q[st], b);
  }
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      out[h][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(in.a, L.Bh[h][c][lk][li], (float4_t){0.0f, 0.0f, 0.0f, 0.0f},
                                                         0, 0, 0);
      if (d.lo) out[h][c] = __builtin_amdgcn_mfma_f32_16x16x32_f16(in.a, L.Bl[h][c][lk][li], out[h][c], 0, 0, 0);
      if (b > 0) {
        int4_v hq = (int4_v){0, 0, 0, 0};
#pragma unroll
        for (int st = 0; st < NST; ++st)
          hq = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[st], (long)Hb[((h * 4 + c) * NST + st) * 64 + lane], hq, 0,
                                                     0, 0);
        const float sg = sgs[dw_feat<D>(h, c, li)];
#pragma unroll
        for (int r = 0; r < 4; ++r) out[h][c][r] = fmaf(sg * in.s[r], (float)hq[r], out[h][c][r]);
      }
    }
}

// stores a pass decoded by dec_vals_w: rows of slice n from rowbase = n T + t0, tokens
// 16 w + 4 lk + r, 4 NH consecutive features per lane, bf16 round to nearest even
template <int D>
__device__ __forceinline__ void dec_store_w(uint16_t* out, int64_t rowbase, const float4_t (&v)[D / 64][4]) {
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int li = lane & 15, lk = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    uint16_t* dst = out + (rowbase + 16 * w + 4 * lk + r) * D + dw_feat<D>(0, 0, li);
    const uint2 p0 = make_uint2((uint32_t)dec_bf16(v[0][0][r]) | ((uint32_t)dec_bf16(v[0][1][r]) << 16),
                                (uint32_t)dec_bf16(v[0][2][r]) | ((uint32_t)dec_bf16(v[0][3][r]) << 16));
    if (D == 128) {
      const int h1 = D / 64 - 1;  // 1
      const uint2 p1 = make_uint2((uint32_t)dec_bf16(v[h1][0][r]) | ((uint32_t)dec_bf16(v[h1][1][r]) << 16),
                                  (uint32_t)dec_bf16(v[h1][2][r]) | ((uint32_t)dec_bf16(v[h1][3][r]) << 16));
      *(uint4*)dst = make_uint4(p0.x, p0.y, p1.x, p1.y);
    } else {
      *(uint2*)dst = p0;
    }
  }
}

}  // namespace jolt
