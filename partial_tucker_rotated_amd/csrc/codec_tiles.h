// Tile-level pieces of the record codec shared by the encoder, the decoder, fused
// attention and streaming admission: b-bit code packing, the fp64 reconstruction
// operand Rm and X~ tiles (fp64 MFMA), the row rotation + block quantizer, and the
// decode of one token tile.  Included by the codec translation units only.
#pragma once
#include "jolt_internal.h"

#ifndef CODEC_TILE_MARK  // phase timestamps of probe builds (defined by codec.hip there)
#define CODEC_TILE_MARK(i)
#endif

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

// Rotation and block quantization of one row of D residual values held by D / 16
// consecutive lanes, 16 features each (segment sg): y holds this thread's residual on
// entry and Q r (Q = H diag(sigma) / sqrt(D)) on exit; q receives the codes
// clip(rint(y / s), -qmax - 1, qmax) decided in fp64 with the fp32 scale s = max|y| / qmax,
// which is returned.  sgn points at sigma for this thread's 16 features.
template <int D>
__device__ __forceinline__ float codec_rotq(double (&y)[16], const int8_t* sgn, int sg, int qmax, int (&q)[16]) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
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
#pragma unroll
  for (int st = 1; st < SEG; st <<= 1)
#pragma unroll
    for (int i = 0; i < FPT; ++i) {
      const double p = __shfl_xor(y[i], st, 64);
      y[i] = (sg & st) ? (p - y[i]) : (y[i] + p);
    }
  const double isq = 1.0 / sqrt((double)D);
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
#pragma unroll
  for (int i = 0; i < FPT; ++i) {
    double v = sd > 0.0 ? rint(y[i] / sd) : 0.0;
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

// codes and scale of this thread's 16 features of row `row`
template <int D>
__device__ __forceinline__ void codec_fetch_res(TileIn& in, const DecodeSrc& d, int b, int64_t row) {
  const int sg = threadIdx.x % (D / 16);
  in.s = 0.0f;
  if (b > 0) {
    in.s = d.scales[row];
    const uint32_t* cw = d.codes + (row * D + sg * 16) * b / 32;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      if (2 * i < b) in.w[i] = cw[i];
  }
}

// everything one pass of a decode needs: the X~ operands, the codes and the scale
template <int D>
__device__ __forceinline__ void codec_fetch_tile(TileIn& in, const DecodeSrc& d, int b, int n, int T, int t0) {
  codec_fetch_a<D>(in, d.Lb, d.ls, d.K, t0);
  codec_fetch_res<D>(in, d, b, (int64_t)n * T + t0 + (int)threadIdx.x / (D / 16));
}

// Decoded bf16 values of this thread's 16 features (segment sg of token t0 + rloc, rloc =
// tid / (D / 16)) from the X~ tile in L.Xt and the codes in `in`, packed two per word.
template <int D>
__device__ __forceinline__ void codec_decode_rows(const CodecLds<D>& L, const double* sgs, int b, const TileIn& in,
                                                  uint32_t (&ow)[8]) {
  constexpr int FPT = 16;
  constexpr int SEG = D / FPT;
  const int tid = threadIdx.x, sg = tid % SEG, rloc = tid / SEG;
  double s = 0.0;
  int h[FPT];
  if (b > 0) {
    s = (double)in.s;
    if (b == 2) unpack_codes<2>(in.w, h);
    else if (b == 4) unpack_codes<4>(in.w, h);
    else unpack_codes<8>(in.w, h);
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
      pk |= (uint32_t)f64_to_bf16_rto(o) << (16 * u);
    }
    ow[i / 2] = pk;
  }
}

// One pass of a decode from inputs already fetched: X~ tile, synchronisation, rows.  The
// caller synchronises before L.Xt is written again.
template <int D>
__device__ __forceinline__ void codec_decode_pass(CodecLds<D>& L, const double* sgs, int b, int K, const TileIn& in,
                                                  uint32_t (&ow)[8]) {
  CODEC_TILE_MARK(5);
  codec_xtilde_in<D>(L, in, K);
  __syncthreads();
  CODEC_TILE_MARK(6);
  codec_decode_rows<D>(L, sgs, b, in, ow);
}

// ---------------------------------------------------------------- decode in registers
// A decode pass without the X~ round trip through LDS.  Wave w owns token tile tt = w / WPT
// (16 tokens) and the features 64 h .. 64 h + 63, h = w % WPT (WPT = D / 64 waves per token
// tile).  Column j = li of product tile c stands for feature f = 64 h + 4 li + c, so a lane
// ends up with 4 consecutive features of its tokens (one 8-byte store per token).  Both
// products land in the same register layout, element (token 4 r + lk, feature
// 64 h + 4 li + c) in lane 16 lk + li, register r of tile c:
//   X~ with fp64 MFMA as above (B operand: column f of Rm);
//   (H q) with v_mfma_i32_16x16x32_i8: q the b-bit codes (int8), H the Sylvester Hadamard
//   matrix (+-1 as int8), exact in int32 (|H q| <= 128 * 128).  That product's A operand
//   holds row i in lane i + 16 g (bytes k = 8 g .. 8 g + 7) and its result row 4 g + r in
//   register r, so the lane of row i fetches the codes of token 4 (i % 4) + i / 4, which puts
//   token 4 r + lk in register r as in the fp64 tile.
//   H[k][f] = (-1)^popcount(k & f): for k = 32 s + 8 g + e (e < 8) the bits of e and of
//   8 g + 32 s do not overlap, so the 8 bytes a lane feeds are a pattern fixed by f & 7 =
//   4 (li & 1) + c, negated when popcount((8 g + 32 s) & f) is odd.
// The decoded value is fma(sigma_f / sqrt(D), s_t (H q)_f, X~), rounded once to bf16, as in
// codec_decode_rows.
typedef int int4_v __attribute__((ext_vector_type(4)));

struct DecIn {
  _Float16 a[JOLT_KMAX / 4];  // A operands of the X~ product
  uint2 q[4];                 // this lane's codes: token 4 (li % 4) + li / 4, k = 32 s + 8 lk .. + 7
  float s[4];                 // scales of tokens 4 r + lk
};

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

template <int D>
__device__ __forceinline__ void dec_fetch(DecIn& in, const DecodeSrc& d, int b, int n, int T, int t0) {
  constexpr int WPT = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, li = lane & 15, lk = lane >> 4;
  const _Float16* arow = d.Lb + (int64_t)(t0 + 16 * tt + li) * d.ls + lk;
#pragma unroll
  for (int st = 0; st < JOLT_KMAX / 4; ++st) in.a[st] = 4 * st < d.K ? arow[4 * st] : (_Float16)0.0f;
  if (b > 0) {
    const int64_t row = (int64_t)n * T + t0 + 16 * tt + 4 * (li & 3) + (li >> 2);
    const uint8_t* cb = (const uint8_t*)d.codes;
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      const int64_t byte = ((row * D + 32 * st + 8 * lk) * b) >> 3;  // b bytes, b-aligned
      if (b == 8) in.q[st] = *(const uint2*)(cb + byte);
      else if (b == 4) in.q[st] = make_uint2(*(const uint32_t*)(cb + byte), 0u);
      else in.q[st] = make_uint2((uint32_t)*(const uint16_t*)(cb + byte), 0u);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) in.s[r] = d.scales[(int64_t)n * T + t0 + 16 * tt + 4 * r + lk];
  }
}

// decoded values of this lane: out[c][r] = bf16 bits of (token 4 r + lk, feature 64 h + 4 li + c)
template <int D>
__device__ __forceinline__ void dec_regs(const CodecLds<D>& L, const double* sgs, int b, int K, const DecIn& in,
                                         uint16_t (&out)[4][4]) {
  constexpr int WPT = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int f0 = 64 * (w % WPT) + 4 * (lane & 15), lk = lane >> 4;
  double4_t acc[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) acc[c] = (double4_t){0.0, 0.0, 0.0, 0.0};
#pragma unroll
  for (int st = 0; st < JOLT_KMAX / 4; ++st)
    if (4 * st < K) {
      const double av = (double)in.a[st];
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, L.Rm[4 * st + lk][f0 + c], acc[c], 0, 0, 0);
    }
  int4_v hq[4];
#pragma unroll
  for (int c = 0; c < 4; ++c) hq[c] = (int4_v){0, 0, 0, 0};
  if (b > 0) {
    long pos[4];  // per tile: byte e = (-1)^popcount(e & (f & 7))
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int f7 = (f0 + c) & 7;
      uint64_t pat = 0;
#pragma unroll
      for (int e = 0; e < 8; ++e) pat |= (uint64_t)((__builtin_popcount(e & f7) & 1) ? 0xFFu : 0x01u) << (8 * e);
      pos[c] = (long)pat;
    }
#pragma unroll
    for (int st = 0; st < D / 32; ++st) {
      const uint2 q8 = codes_to_i8(in.q[st], b);
      const long av = (long)(((uint64_t)q8.y << 32) | q8.x);
#pragma unroll
      for (int c = 0; c < 4; ++c) {
        const bool odd = __builtin_popcount((8 * lk + 32 * st) & (f0 + c)) & 1;
        const long bv = odd ? (pos[c] ^ (long)0xFEFEFEFEFEFEFEFEull) : pos[c];
        hq[c] = __builtin_amdgcn_mfma_i32_16x16x32_i8(av, bv, hq[c], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int c = 0; c < 4; ++c) {
    const double sg = sgs[f0 + c];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const double sv = b > 0 ? (double)in.s[r] : 0.0;
      out[c][r] = f64_to_bf16_rto(fma(sg, sv * (double)hq[c][r], acc[c][r]));
    }
  }
}

// stores a pass decoded by dec_regs: rows of slice n from rowbase = n T + t0, tokens
// 16 tt + 4 r + lk, 4 consecutive features per lane (8 bytes)
template <int D>
__device__ __forceinline__ void dec_store(uint16_t* out, int64_t rowbase, const uint16_t (&v)[4][4]) {
  constexpr int WPT = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, f0 = 64 * (w % WPT) + 4 * (lane & 15), lk = lane >> 4;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const uint2 pk = make_uint2((uint32_t)v[0][r] | ((uint32_t)v[1][r] << 16),
                                (uint32_t)v[2][r] | ((uint32_t)v[3][r] << 16));
    *(uint2*)(out + (rowbase + 16 * tt + 4 * r + lk) * D + f0) = pk;
  }
}

}  // namespace jolt
