// Record writer (encode) and reader (decode) for one chosen candidate per table.
//
// Encode follows "Rotated Tucker residual for outlier-resistant KV quantization",
// Implementation notes: with the stored Tucker factors, reconstruct X~, form
// R = X - X~, rotate each row of D values with Q = H diag(sigma) / sqrt(D), and store
// per block (one row) the scale s = max|Y| / (2^(b-1) - 1) (fp32) and the codes
// clip(round(Y / s), -2^(b-1), 2^(b-1) - 1).  X~ and R are formed in fp64, the rotation and
// the quantizer in fp32.
// Decode follows "Joint Tucker-rank and residual-bit KV allocator", Formulas, first
// display: X^ = X~ + Q^T Q_b(Q R), evaluated in fp32 and rounded once to bf16.
// The encoder forms X~ per token tile with fp64 MFMA and runs the residual with one thread
// per 16 consecutive features of a row (D / 16 threads per row); the decoder keeps each
// token tile in registers (fp16 split MFMA for X~, int8 MFMA for the inverse Hadamard).
//
// Launches cover up to JOLT_TAB_CHUNK tables: blockIdx.y is the local table index,
// workspace arrays are indexed by the global table index t0 + local.
#include "jolt_internal.h"

#include "codec_tiles.h"

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

// Residual codes and scales (b > 0), in registers.  Block (chunk of ENC_CHUNK tokens, slice
// n, local table), passes of 64 tokens: wave w owns tokens 16 w .. 16 w + 15 of a pass and all
// D features.  X~ = L Rm by v_mfma_f64_16x16x4f64 (A: the fp16 L row of token i, k = 4 st + g
// in lane i + 16 g; B: Rm in LDS, formed once per block in fp64); result (token 4 r + g,
// feature f(c, l)) in lane 16 g + l, register r of tile c, with f(c, l) = NCT l + c
// (NCT = D / 16 tiles), so a lane holds NCT consecutive features of each of its 4 tokens:
// its input rows are 16-byte loads and its codes are one contiguous b NCT / 8 bytes.  X~ and
// the residual R = X - X~ are fp64 (R rounded once to fp32), so the cancellation between X
// and X~ costs no precision; the rotation, scale and codes then run in fp32, whose errors
// scale with |R|: the rotation's butterflies over c run in registers, those over l across
// the 16 lanes of the token (DPP quad permutations for l ^ 1, l ^ 2, ds_swizzle for l ^ 4,
// l ^ 8); 1 / sqrt(D) is applied with the scale, s = (max |y| / sqrt(D)) / qmax rounded to
// fp32, and y / (s sqrt(D)) is rounded to nearest even by adding 1.5 * 2^23 (the low bits
// of the sum are the two's-complement code).  No LDS or barrier inside the loop; the next
// pass's rows are fetched during the current one.
constexpr int ENC_CHUNK = 1024;

template <int D>
struct EncLds {
  static constexpr int NCT = D / 16;
  double Bs[JOLT_KMAX / 4][NCT][64];  // B operands of X~: Rm[4 st + g][f(c, l)] in lane l + 16 g
  _Float16 Gs[JOLT_KMAX][JOLT_KMAX];  // staged core rows (r_d < D chains)
  _Float16 Us[JOLT_KMAX][D];          // staged U_d^T (r_d < D chains)
};

template <int X>
__device__ __forceinline__ float enc_xor_f32(float v) {  // partner within the 16-lane group
  if (X == 1) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0xB1, 0xF, 0xF, true));
  if (X == 2) return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x4E, 0xF, 0xF, true));
  constexpr int pat = (X << 10) | 0x1F;  // ds_swizzle xor mode
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), pat));
}

template <int D>
__global__ __launch_bounds__(256, 3) void k_encode_resid(const EncodeArgs a) {
  constexpr int NCT = D / 16;  // column tiles = features per lane
  const int tl = blockIdx.z, tg = a.t0 + tl, n = blockIdx.y;
  const EncodeTable& e = a.t[tl];
  if (e.b == 0) return;
  const int T = a.T, N = a.N;
  const int tid = threadIdx.x, lane = tid & 63, w = tid >> 6, li = lane & 15, g = lane >> 4;
  const int qmax = (1 << (e.b - 1)) - 1;
  const int tb = blockIdx.x * ENC_CHUNK, te = min(T, tb + ENC_CHUNK);
  if (e.chain < 0) {  // (T, D) with b > 0: X stored verbatim, a zero residual (codes 0, scale 0)
    uint32_t* cz = (uint32_t*)(e.rec + e.off_codes + (((int64_t)n * T + tb) * D * e.b >> 3));
    for (int64_t i = tid; i < ((int64_t)(te - tb) * D * e.b >> 5); i += 256) cz[i] = 0u;
    float* sz = (float*)(e.rec + e.off_scales) + (int64_t)n * T + tb;
    for (int i = tid; i < te - tb; i += 256) sz[i] = 0.0f;
    return;
  }
  __shared__ __align__(16) EncLds<D> L;
  // ---- reconstruction operand in the B layout: Rm = G_n U_d^T, G_n or U_d^T (fp64 sums of
  // fp16 products over j in ascending order)
  int K;
  const _Float16* Lb;  // L rows (token-major, stride 32)
  const _Float16* Ud = a.Ud16 + (int64_t)tg * D * JOLT_KMAX;  // [D][32]
  if (e.chain == 5) {
    K = e.rd;
    Lb = a.G16T + ((int64_t)tg * N + n) * T * JOLT_KMAX;
  } else {
    K = e.rT;
    Lb = a.UT16 + ((int64_t)tg * 5 + e.chain) * T * JOLT_KMAX;
  }
  const _Float16* G = a.G16 + (((int64_t)tg * 5 + (e.chain < 5 ? e.chain : 0)) * N + n) * JOLT_KMAX * D;
  const bool kind0 = e.chain < 4;
  if (kind0) {
    const int rd = e.rd;
    for (int idx = tid; idx < K * rd; idx += 256) {
      const int k = idx / rd, j = idx - k * rd;
      L.Gs[k][j] = G[k * D + j];
    }
    for (int idx = tid; idx < rd * D; idx += 256) {
      const int f = idx / rd, j = idx - f * rd;
      L.Us[j][f] = Ud[f * JOLT_KMAX + j];
    }
    __syncthreads();
  }
  for (int idx = tid; idx < (K / 4) * NCT * 64; idx += 256) {
    const int ln = idx & 63, c = (idx >> 6) % NCT, st = idx / (64 * NCT);
    const int k = 4 * st + (ln >> 4), f = NCT * (ln & 15) + c;
    double v;
    if (e.chain == 5) {
      v = (double)Ud[f * JOLT_KMAX + k];
    } else if (e.chain == 4) {
      v = (double)G[k * D + f];
    } else {
      v = 0.0;
      for (int j = 0; j < e.rd; ++j) v = fma((double)L.Gs[k][j], (double)L.Us[j][f], v);
    }
    L.Bs[st][c][ln] = v;
  }
  __syncthreads();
  // this lane's rotation signs sigma_f for f = NCT li + c, as sign bits
  uint32_t sbits = 0;
#pragma unroll
  for (int c = 0; c < NCT; ++c) sbits |= (a.signs[tg * D + NCT * li + c] < 0 ? 1u : 0u) << c;
  const float isq = (float)(1.0 / sqrt((double)D));
  const uint16_t* xsrc = (const uint16_t*)a.xsrc[tl];
  uint8_t* codes = (uint8_t*)(e.rec + e.off_codes);
  float* scales = (float*)(e.rec + e.off_scales);
  // inputs of one pass: the lane's L values (token li, k = 4 st + g) and its x rows
  // (tokens 4 r + g, features NCT li .. NCT li + NCT - 1)
  struct In {
    uint32_t a[JOLT_KMAX / 8];  // fp16 bits of k = 4 st + g, st even in the low half
    uint32_t x[4][NCT / 2];
  };
  auto fetch = [&](In& in, int t0) {
    const int t0w = t0 + 16 * w;
    const uint16_t* lr = (const uint16_t*)Lb + (int64_t)(t0w + li) * JOLT_KMAX + g;
#pragma unroll
    for (int s2 = 0; s2 < JOLT_KMAX / 8; ++s2) {
      const uint32_t lo = 8 * s2 < K ? lr[8 * s2] : 0u, hi = 8 * s2 + 4 < K ? lr[8 * s2 + 4] : 0u;
      in.a[s2] = lo | (hi << 16);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const uint16_t* xr = xsrc + ((int64_t)n * T + t0w + 4 * r + g) * D + NCT * li;
      if (NCT == 8) {
        const uint4 u = *(const uint4*)xr;
        in.x[r][0] = u.x; in.x[r][1] = u.y; in.x[r][NCT > 4 ? 2 : 0] = u.z; in.x[r][NCT > 4 ? 3 : 0] = u.w;
      } else {
        const uint2 u = *(const uint2*)xr;
        in.x[r][0] = u.x; in.x[r][1] = u.y;
      }
    }
  };
  In cur, nxt;
  fetch(cur, tb);
  for (int t0 = tb; t0 < te; t0 += 64) {
    const bool more = t0 + 64 < te;  // uniform
    if (more) fetch(nxt, t0 + 64);
    // ---- X~ tiles
    double4_t xt[NCT];
#pragma unroll
    for (int c = 0; c < NCT; ++c) xt[c] = (double4_t){0.0, 0.0, 0.0, 0.0};
#pragma unroll
    for (int st = 0; st < JOLT_KMAX / 4; ++st)
      if (4 * st < K) {
        const double av = (double)__builtin_bit_cast(_Float16, (uint16_t)(cur.a[st >> 1] >> (16 * (st & 1))));
#pragma unroll
        for (int c = 0; c < NCT; ++c)
          xt[c] = __builtin_amdgcn_mfma_f64_16x16x4f64(av, L.Bs[st][c][lane], xt[c], 0, 0, 0);
      }
    // ---- per token 4 r + g: residual in fp64 (one rounding to fp32), then the rotation,
    // scale and codes in fp32
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      float y[NCT];
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const uint16_t hb = (uint16_t)(cur.x[r][c >> 1] >> (16 * (c & 1)));
        const float d = (float)((double)bf16_to_f32(hb) - xt[c][r]);
        y[c] = __uint_as_float(__float_as_uint(d) ^ (((sbits >> c) & 1u) << 31));
      }
#pragma unroll
      for (int st = 1; st < NCT; st <<= 1)
#pragma unroll
        for (int c = 0; c < NCT; ++c)
          if (!(c & st)) {
            const float p = y[c], q2 = y[c + st];
            y[c] = p + q2;
            y[c + st] = p - q2;
          }
      auto cross = [&](auto xs) {
        constexpr int X = decltype(xs)::value;
        const float sn = (li & X) ? -1.0f : 1.0f;
#pragma unroll
        for (int c = 0; c < NCT; ++c) y[c] = fmaf(sn, y[c], enc_xor_f32<X>(y[c]));
      };
      cross(std::integral_constant<int, 1>());
      cross(std::integral_constant<int, 2>());
      cross(std::integral_constant<int, 4>());
      cross(std::integral_constant<int, 8>());
      float m = 0.0f;
#pragma unroll
      for (int c = 0; c < NCT; ++c) m = fmaxf(m, fabsf(y[c]));
      m = fmaxf(m, enc_xor_f32<1>(m));
      m = fmaxf(m, enc_xor_f32<2>(m));
      m = fmaxf(m, enc_xor_f32<4>(m));
      m = fmaxf(m, enc_xor_f32<8>(m));
      const float sc = (m * isq) / (float)qmax;  // max |Q r| / qmax
      const float inv = sc > 0.0f ? isq / sc : 0.0f;
      const uint32_t bm = (1u << e.b) - 1u;
      uint64_t word = 0;
#pragma unroll
      for (int c = 0; c < NCT; ++c) {
        const float u = __builtin_amdgcn_fmed3f(y[c] * inv, (float)(-qmax - 1), (float)qmax);
        const uint32_t qb = __float_as_uint(u + 12582912.0f) & bm;  // rint(u), two's complement
        word |= (uint64_t)qb << (c * e.b);
      }
      const int64_t row = (int64_t)n * T + t0 + 16 * w + 4 * r + g;
      uint8_t* cw = codes + ((row * D + NCT * li) * e.b >> 3);  // NCT b / 8 bytes
      const int nbytes = NCT * e.b / 8;
      if (nbytes == 8) *(uint2*)cw = make_uint2((uint32_t)word, (uint32_t)(word >> 32));
      else if (nbytes == 4) *(uint32_t*)cw = (uint32_t)word;
      else if (nbytes == 2) *(uint16_t*)cw = (uint16_t)word;
      else *cw = (uint8_t)word;
      if (li == 0) scales[row] = sc;
    }
    if (more) cur = nxt;
  }
}

// Reconstruction, dequantization, inverse rotation, bf16 output.  The inverse Hadamard runs
// on the integer codes (exact); the residual s (H q)_f sigma_f / sqrt(D) is added to X~ by one
// fp32 FMA, and the sum is rounded once to bf16.
// Decode: workgroup (chunk of DEC_CHUNK tokens, slice n, table), passes of 64 tokens in the
// wide register layout (wave w: tokens 16 w .. 16 w + 15 of a pass, all D features).  Rm and
// the B operands are set up once per workgroup; the inputs of a pass (L rows, codes, scales)
// are fetched two passes ahead, so that two passes' loads are in flight while one is decoded.
constexpr int DEC_CHUNK = 1024;

template <int D>
__global__ __launch_bounds__(256, 3) void k_decode(const DecodeArgs a) {
  constexpr int CP = 64;  // tokens per pass
  const int tl = blockIdx.z, n = blockIdx.y;
  const EncodeTable& e = a.t[tl];
  const int T = a.T;
  const int tid = threadIdx.x;
  const int tb = blockIdx.x * DEC_CHUNK, te = min(T, tb + DEC_CHUNK);
  if (e.chain < 0) {  // (T, D): X stored verbatim
    const uint4* src = (const uint4*)(e.rec + e.off_core) + ((int64_t)n * T + tb) * D / 8;
    uint4* dst = (uint4*)a.out[tl] + ((int64_t)n * T + tb) * D / 8;
    for (int64_t i = tid; i < (int64_t)(te - tb) * D / 8; i += 256) dst[i] = src[i];
    return;
  }
  __shared__ __align__(16) DecLds<D> L;
  __shared__ float sgs[D];  // sigma_f / sqrt(D)
  // the Hadamard operands take the place of Rm once the B operands are formed from it
  uint64_t* Hb = (uint64_t*)&L.Rm[0][0];
  static_assert(sizeof(L.Rm) >= sizeof(uint64_t) * (D / 64) * 4 * (D / 32) * 64, "Hadamard operands fit Rm");
  const DecSrc d = dec_prepare<D>(L, sgs, e, n, T);
  dec_bops_w<D>(L);  // ends with a barrier: Rm is free
  if (e.b > 0) {     // uniform
    dec_hops_w<D>(Hb, e.b);
    __syncthreads();
  }
  uint16_t* out = (uint16_t*)a.out[tl];
  const int np = (te - tb) / CP;  // passes (te - tb is a multiple of 64)
  DecIn in0, in1, in2;
  float4_t v[D / 64][4];
  auto pass = [&](const DecIn& in, int p) {
    dec_vals_w<D>(L, Hb, sgs, d, e.b, in, v);
    dec_store_w<D>(out, (int64_t)n * T + tb + p * CP, v);
  };
  dec_fetch<D, true>(in0, d, e.b, n, T, tb);
  if (np > 1) dec_fetch<D, true>(in1, d, e.b, n, T, tb + CP);
  for (int p = 0; p < np; p += 3) {  // np is uniform: every branch below is
    if (p + 2 < np) dec_fetch<D, true>(in2, d, e.b, n, T, tb + (p + 2) * CP);
    pass(in0, p);
    if (p + 1 >= np) break;
    if (p + 3 < np) dec_fetch<D, true>(in0, d, e.b, n, T, tb + (p + 3) * CP);
    pass(in1, p + 1);
    if (p + 2 >= np) break;
    if (p + 4 < np) dec_fetch<D, true>(in1, d, e.b, n, T, tb + (p + 4) * CP);
    pass(in2, p + 2);
  }
}

// ---------------------------------------------------------------- fused decode + attention
// O = softmax(Q K^T * scale) V for one layer group, K and V rebuilt from their records with the
// decoder's arithmetic (the same fp32 expression, rounded once to bf16), never stored.
// Workgroup (chunk c, slice n, group g) takes the tokens [c ach, (c + 1) ach) of slice n and
// all nq queries of that slice.  Each wave works alone on 16-token tiles (tokens
// 16 w .. 16 w + 15 of every 64), with its own running softmax, entirely in registers:
//   1. K tile transposed: K^T(f, t) = Rm^T L^T + sigma_f s_t (H q)(f, t) / sqrt(D) by the
//      decoder's MFMAs with the operands swapped (fp16 split for Rm^T L^T, int8 for H q^T),
//      so lane (t, g) holds features f(hc, 4 g + r) of token t: the A operand of the scores;
//   2. scores S(t, q) = K Q^T * scale by bf16 MFMA (exact products, fp32 sums); lane (q, g)
//      then holds the scores of query q for tokens 4 g + r;
//   3. running softmax per query (max and sum over the 16 tokens: registers and lanes
//      q, q + 16, q + 32, q + 48), P = exp(S - m), the factor exp(m_old - m) for the output;
//   4. V tile as the decoder computes it: lane (f, g) holds V(4 g + r, f), the A operand of
//      O^T = V^T P^T by v_mfma_f32_16x16x16_bf16 with P split into bf16 hi + lo (16 bits).
// At the end the four waves' states are merged (log-sum-exp) through LDS, and the chunk's O
// (unnormalised), m and l go to the workspace; k_attend_merge combines the chunks:
// O = sum_c e^{m_c - M} O_c / sum_c e^{m_c - M} l_c.
// Features follow the wide decode layout: tile hc = 4 h + c, f(hc, i) = dw_feat(h, c, i).
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef short4_t bf16x4_s;
constexpr int ATT_BLK = 64;  // tokens per step of a workgroup (16 per wave)

template <int D>
struct AttLds {
  union {
    DecLds<D> L;                      // set-up; then K's B operands (L.Bh, L.Bl) and, in
                                      // place of L.Rm, K's Hadamard operands
    float Ow[4][ATT_QMAX][D];         // after the loop: each wave's unnormalised output
  };
  half8_t Bvh[D / 64][4][4][16];      // V's B operands (copied out of L during set-up)
  half8_t Bvl[D / 64][4][4][16];
  uint64_t Hv[(D / 64) * 4 * (D / 32) * 64];  // V's Hadamard operands
  float sgk[D], sgv[D];               // sigma_f / sqrt(D) of K and V
  float mw[4][ATT_QMAX], lw[4][ATT_QMAX];
};

__device__ __forceinline__ uint32_t att_pk(float a, float b) {
  return (uint32_t)dec_bf16(a) | ((uint32_t)dec_bf16(b) << 16);
}

// The wave's K tiles u < NTL (tokens t0[u] + li, as bf16 bits kb[u][hc][r] of feature
// f(hc, 4 lk + r)).  B (the code width, 0 for none) and LO (Rm has an fp16 lo part) are
// compile-time, so the products of all NTL tiles form one block the compiler can interleave.
template <int D, int NTL, bool B, bool LO>
__device__ __forceinline__ void att_k_mfma(const AttLds<D>& S, const uint64_t* Hk, int b, const DecIn* in,
                                           uint32_t (&kb)[NTL][D / 64 * 4][2]) {
  constexpr int NH = D / 64, NST = D / 32;
  const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
  long av[NTL][NST];
  if (B) {
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
      for (int st = 0; st < NST; ++st) av[u][st] = (long)codes_to_i8_w(in[u].q[st], b);
  }
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float4_t x[NTL];
#pragma unroll
      for (int u = 0; u < NTL; ++u) {
        x[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(S.L.Bh[h][c][lk][li], in[u].a, (float4_t){0.0f, 0.0f, 0.0f, 0.0f},
                                                      0, 0, 0);
        if (LO) x[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(S.L.Bl[h][c][lk][li], in[u].a, x[u], 0, 0, 0);
      }
      if (B) {
#pragma unroll
        for (int u = 0; u < NTL; ++u) {
          int4_v hq = (int4_v){0, 0, 0, 0};
#pragma unroll
          for (int st = 0; st < NST; ++st)
            hq = __builtin_amdgcn_mfma_i32_16x16x32_i8((long)Hk[((h * 4 + c) * NST + st) * 64 + lane], av[u][st], hq, 0,
                                                       0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r)
            x[u][r] = fmaf(S.sgk[dw_feat<D>(h, c, 4 * lk + r)] * in[u].s[0], (float)hq[r], x[u][r]);
        }
      }
#pragma unroll
      for (int u = 0; u < NTL; ++u) {
        kb[u][h * 4 + c][0] = att_pk(x[u][0], x[u][1]);
        kb[u][h * 4 + c][1] = att_pk(x[u][2], x[u][3]);
      }
    }
}

template <int D, int NTL>
__device__ __forceinline__ void att_k_tiles(const AttLds<D>& S, const uint64_t* Hk, const EncodeTable& e,
                                            const DecSrc& d, const DecIn* in, int n, int T, const int* t0,
                                            uint32_t (&kb)[NTL][D / 64 * 4][2]) {
  constexpr int NH = D / 64;
  const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
  if (e.chain < 0) {  // verbatim rows: token t0 + li, features f(hc, 4 lk + r) = 4 NH (4 lk + r) + hc
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
      const uint16_t* row = (const uint16_t*)(e.rec + e.off_core) + ((int64_t)n * T + t0[u] + li) * D;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int f0 = 4 * NH * (4 * lk + r);
        uint32_t w[2 * NH];
        if (NH == 2) {
          const uint4 v = *(const uint4*)(row + f0);
          w[0] = v.x; w[1] = v.y; w[NH > 1 ? 2 : 0] = v.z; w[NH > 1 ? 3 : 0] = v.w;
        } else {
          const uint2 v = *(const uint2*)(row + f0);
          w[0] = v.x; w[1] = v.y;
        }
#pragma unroll
        for (int hc = 0; hc < NH * 4; ++hc) {
          const uint32_t v = (w[hc >> 1] >> (16 * (hc & 1))) & 0xFFFFu;
          if (r & 1) kb[u][hc][r >> 1] |= v << 16;
          else kb[u][hc][r >> 1] = v;
        }
      }
    }
    return;
  }
  if (e.b > 0) {
    if (d.lo) att_k_mfma<D, NTL, true, true>(S, Hk, e.b, in, kb);
    else att_k_mfma<D, NTL, true, false>(S, Hk, e.b, in, kb);
  } else {
    if (d.lo) att_k_mfma<D, NTL, false, true>(S, Hk, e.b, in, kb);
    else att_k_mfma<D, NTL, false, false>(S, Hk, e.b, in, kb);
  }
}

// The wave's V tiles u < NTL (tokens t0[u] + 4 lk + r, as bf16 bits vb[u][hc][.] of feature
// f(hc, li)); B and LO as for K.
template <int D, int NTL, bool B, bool LO>
__device__ __forceinline__ void att_v_mfma(const AttLds<D>& S, int b, const DecIn* in,
                                           uint32_t (&vb)[NTL][D / 64 * 4][2]) {
  constexpr int NH = D / 64, NST = D / 32;
  const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
  long av[NTL][NST];
  if (B) {
#pragma unroll
    for (int u = 0; u < NTL; ++u)
#pragma unroll
      for (int st = 0; st < NST; ++st) av[u][st] = (long)codes_to_i8_w(in[u].q[st], b);
  }
#pragma unroll
  for (int h = 0; h < NH; ++h)
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      float4_t x[NTL];
#pragma unroll
      for (int u = 0; u < NTL; ++u) {
        x[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(in[u].a, S.Bvh[h][c][lk][li], (float4_t){0.0f, 0.0f, 0.0f, 0.0f},
                                                      0, 0, 0);
        if (LO) x[u] = __builtin_amdgcn_mfma_f32_16x16x32_f16(in[u].a, S.Bvl[h][c][lk][li], x[u], 0, 0, 0);
      }
      if (B) {
        const float sg = S.sgv[dw_feat<D>(h, c, li)];
#pragma unroll
        for (int u = 0; u < NTL; ++u) {
          int4_v hq = (int4_v){0, 0, 0, 0};
#pragma unroll
          for (int st = 0; st < NST; ++st)
            hq = __builtin_amdgcn_mfma_i32_16x16x32_i8(av[u][st], (long)S.Hv[((h * 4 + c) * NST + st) * 64 + lane], hq,
                                                       0, 0, 0);
#pragma unroll
          for (int r = 0; r < 4; ++r) x[u][r] = fmaf(sg * in[u].s[r], (float)hq[r], x[u][r]);
        }
      }
#pragma unroll
      for (int u = 0; u < NTL; ++u) {
        vb[u][h * 4 + c][0] = att_pk(x[u][0], x[u][1]);
        vb[u][h * 4 + c][1] = att_pk(x[u][2], x[u][3]);
      }
    }
}

template <int D, int NTL>
__device__ __forceinline__ void att_v_tiles(const AttLds<D>& S, const EncodeTable& e, const DecSrc& d,
                                            const DecIn* in, int n, int T, const int* t0,
                                            uint32_t (&vb)[NTL][D / 64 * 4][2]) {
  constexpr int NH = D / 64;
  const int lane = threadIdx.x & 63, li = lane & 15, lk = lane >> 4;
  if (e.chain < 0) {  // verbatim rows t0 + 4 lk + r, features 4 NH li .. 4 NH li + 4 NH - 1
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
      const uint16_t* base =
          (const uint16_t*)(e.rec + e.off_core) + ((int64_t)n * T + t0[u] + 4 * lk) * D + 4 * NH * li;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        uint32_t w[2 * NH];
        if (NH == 2) {
          const uint4 v = *(const uint4*)(base + r * D);
          w[0] = v.x; w[1] = v.y; w[NH > 1 ? 2 : 0] = v.z; w[NH > 1 ? 3 : 0] = v.w;
        } else {
          const uint2 v = *(const uint2*)(base + r * D);
          w[0] = v.x; w[1] = v.y;
        }
#pragma unroll
        for (int hc = 0; hc < NH * 4; ++hc) {
          const uint32_t v = (w[hc >> 1] >> (16 * (hc & 1))) & 0xFFFFu;
          if (r & 1) vb[u][hc][r >> 1] |= v << 16;
          else vb[u][hc][r >> 1] = v;
        }
      }
    }
    return;
  }
  if (e.b > 0) {
    if (d.lo) att_v_mfma<D, NTL, true, true>(S, e.b, in, vb);
    else att_v_mfma<D, NTL, true, false>(S, e.b, in, vb);
  } else {
    if (d.lo) att_v_mfma<D, NTL, false, true>(S, e.b, in, vb);
    else att_v_mfma<D, NTL, false, false>(S, e.b, in, vb);
  }
}

// One step of a wave's flash attention over NTL tiles of 16 tokens (t0[u] + 16 w ..), in two
// parts (the caller loads the next step's K inputs in between): att_scores forms the K tiles
// and their scores; att_pv takes the running softmax over the step's 16 NTL tokens, forms
// the V tiles and adds V^T P^T to O^T.
template <int D, int NTL>
__device__ __forceinline__ void att_scores(const AttLds<D>& S, const uint64_t* Hk, const EncodeTable& ek,
                                           const DecSrc& dk, const DecIn* kin, int n, int T, const int* t0,
                                           const bf16x8_t (&qf)[D / 32], float4_t (&sc)[NTL]) {
  constexpr int NT = D / 64 * 4, KS = D / 32;
  uint32_t kb[NTL][NT][2];
  att_k_tiles<D, NTL>(S, Hk, ek, dk, kin, n, T, t0, kb);
#pragma unroll
  for (int u = 0; u < NTL; ++u) {
    sc[u] = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const bf16x8_t kf = __builtin_bit_cast(
          bf16x8_t, make_uint4(kb[u][2 * s][0], kb[u][2 * s][1], kb[u][2 * s + 1][0], kb[u][2 * s + 1][1]));
      sc[u] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[s], sc[u], 0, 0, 0);
    }
  }
}

template <int D, int NTL>
__device__ __forceinline__ void att_pv(const AttLds<D>& S, const EncodeTable& ev, const DecSrc& dv,
                                       const DecIn* vin, int n, int T, const int* t0, float4_t (&sc)[NTL],
                                       float scale, float& m, float& l, float4_t (&acc)[D / 64 * 4]) {
  constexpr int NT = D / 64 * 4;
  float bm = -INFINITY;
#pragma unroll
  for (int u = 0; u < NTL; ++u)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      sc[u][r] *= scale;
      bm = fmaxf(bm, sc[u][r]);
    }
  bm = fmaxf(bm, __shfl_xor(bm, 16, 64));
  bm = fmaxf(bm, __shfl_xor(bm, 32, 64));
  const float mn = fmaxf(m, bm);
  const float cf = expf(m - mn);  // 0 on the first step (m = -inf)
  float ps = 0.0f;
  bf16x4_s pbh[NTL], pbl[NTL];  // P as the B operand of O^T (k = token 4 lk + r, column = query li)
#pragma unroll
  for (int u = 0; u < NTL; ++u) {
    float hv[4], lv[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float p = expf(sc[u][r] - mn);
      ps += p;
      const __bf16 hb = (__bf16)p;
      hv[r] = (float)hb;
      lv[r] = p - hv[r];
    }
    pbh[u] = __builtin_bit_cast(bf16x4_s, make_uint2(att_pk(hv[0], hv[1]), att_pk(hv[2], hv[3])));
    pbl[u] = __builtin_bit_cast(bf16x4_s, make_uint2(att_pk(lv[0], lv[1]), att_pk(lv[2], lv[3])));
  }
  ps += __shfl_xor(ps, 16, 64);
  ps += __shfl_xor(ps, 32, 64);
  l = l * cf + ps;
  m = mn;
  uint32_t vb[NTL][NT][2];
  att_v_tiles<D, NTL>(S, ev, dv, vin, n, T, t0, vb);
#pragma unroll
  for (int j = 0; j < NT; ++j) {
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[j][r] *= cf;
#pragma unroll
    for (int u = 0; u < NTL; ++u) {
      const bf16x4_s va = __builtin_bit_cast(bf16x4_s, make_uint2(vb[u][j][0], vb[u][j][1]));
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pbh[u], acc[j], 0, 0, 0);
      acc[j] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pbl[u], acc[j], 0, 0, 0);
    }
  }
}


template <int D>
__global__ __launch_bounds__(256, 2) void k_attend(const AttendArgs a) {
  constexpr int NH = D / 64, NT = NH * 4, KS = D / 32;
  const int c = blockIdx.x, n = blockIdx.y, g = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lk = lane >> 4;
  const int T = a.T, nq = a.nq;
  const EncodeTable& ek = a.k[g];
  const EncodeTable& ev = a.v[g];
  const int tb = c * a.ach, te = min(T, tb + a.ach);
  __shared__ __align__(16) AttLds<D> S;
  uint64_t* Hk = (uint64_t*)&S.L.Rm[0][0];
  static_assert(sizeof(S.L.Rm) >= sizeof(uint64_t) * (D / 64) * 4 * (D / 32) * 64, "Hadamard operands fit Rm");
  // ---- set-up: V's operands first (copied aside), then K's (left in S.L)
  DecSrc dv{}, dk{};
  if (ev.chain >= 0) {
    dv = dec_prepare<D>(S.L, S.sgv, ev, n, T);
    dec_bops_w<D>(S.L);
    for (int idx = tid; idx < (D / 64) * 4 * 4 * 16; idx += 256) {
      (&S.Bvh[0][0][0][0])[idx] = (&S.L.Bh[0][0][0][0])[idx];
      (&S.Bvl[0][0][0][0])[idx] = (&S.L.Bl[0][0][0][0])[idx];
    }
    if (ev.b > 0) dec_hops_w<D>(S.Hv, ev.b);
    __syncthreads();
  }
  if (ek.chain >= 0) {
    dk = dec_prepare<D>(S.L, S.sgk, ek, n, T);
    dec_bops_w<D>(S.L);  // ends with a barrier: Rm is free
    if (ek.b > 0) dec_hops_w<D>(Hk, ek.b);
  }
  __syncthreads();
  // the scores' B operand for k step s: element 4 j + r of lane (q, g) = Q[q][f(2 s + j, 4 g + r)]
  bf16x8_t qf[KS];
  {
    const uint16_t* qr = a.q[g] + ((int64_t)n * nq + (li < nq ? li : 0)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      uint16_t u[8];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int hc = 2 * s + j;
          u[4 * j + r] = li < nq ? qr[dw_feat<D>(hc >> 2, hc & 3, 4 * lk + r)] : (uint16_t)0;
        }
      qf[s] = __builtin_bit_cast(bf16x8_t, make_uint4(u[0] | ((uint32_t)u[1] << 16), u[2] | ((uint32_t)u[3] << 16),
                                                      u[4] | ((uint32_t)u[5] << 16), u[6] | ((uint32_t)u[7] << 16)));
    }
  }
  // O^T tiles: acc[hc][r] = O(query li, feature f(hc, 4 lk + r)); running max m and sum l of
  // query li
  float4_t acc[NT];
#pragma unroll
  for (int j = 0; j < NT; ++j) acc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY, l = 0.0f;
  // steps of 64 tokens, two at a time (the wave's tiles t0 + 16 w and t0 + 64 + 16 w; an odd
  // last step alone); the next step's K inputs are loaded once the K tiles are formed, its V
  // inputs once the V tiles are
  const int nstep = (te - tb) / ATT_BLK;
  DecIn kin[2], vin[2];
  auto kfetch = [&](DecIn& q, int t0) {
    if (ek.chain >= 0) dec_fetch<D, true, true>(q, dk, ek.b, n, T, t0);
  };
  auto vfetch = [&](DecIn& q, int t0) {
    if (ev.chain >= 0) dec_fetch<D, true>(q, dv, ev.b, n, T, t0);
  };
  if (nstep > 0) {
    kfetch(kin[0], tb);
    vfetch(vin[0], tb);
  }
  if (nstep > 1) {
    kfetch(kin[1], tb + ATT_BLK);
    vfetch(vin[1], tb + ATT_BLK);
  }
  for (int i = 0; i < nstep; i += 2) {
    const int t0 = tb + i * ATT_BLK, tn = t0 + 2 * ATT_BLK;
    const bool n0 = i + 2 < nstep, n1 = i + 3 < nstep;
    if (i + 1 < nstep) {
      const int tt[2] = {t0 + 16 * wave, t0 + ATT_BLK + 16 * wave};
      float4_t sc[2];
      att_scores<D, 2>(S, Hk, ek, dk, kin, n, T, tt, qf, sc);
      if (n0) kfetch(kin[0], tn);
      if (n1) kfetch(kin[1], tn + ATT_BLK);
      att_pv<D, 2>(S, ev, dv, vin, n, T, tt, sc, a.scale, m, l, acc);
    } else {
      const int tt[1] = {t0 + 16 * wave};
      float4_t sc[1];
      att_scores<D, 1>(S, Hk, ek, dk, kin, n, T, tt, qf, sc);
      att_pv<D, 1>(S, ev, dv, vin, n, T, tt, sc, a.scale, m, l, acc);
    }
    if (n0) vfetch(vin[0], tn);
    if (n1) vfetch(vin[1], tn + ATT_BLK);
  }
  // ---- merge of the four waves (S.L is no longer read: every wave has passed the loop)
  __syncthreads();
  if (lk == 0 && li < nq) {
    S.mw[wave][li] = m;
    S.lw[wave][li] = l;
  }
#pragma unroll
  for (int j = 0; j < NT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      if (li < nq) S.Ow[wave][li][dw_feat<D>(j >> 2, j & 3, 4 * lk + r)] = acc[j][r];
  __syncthreads();
  float* part = a.part + ((((int64_t)g * a.N + n) * a.nchunk + c) * nq) * (D + 2);
  for (int idx = tid; idx < nq * D; idx += 256) {
    const int q = idx / D, f = idx - q * D;
    const float M = fmaxf(fmaxf(S.mw[0][q], S.mw[1][q]), fmaxf(S.mw[2][q], S.mw[3][q]));
    float o = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) o = fmaf(expf(S.mw[w][q] - M), S.Ow[w][q][f], o);
    part[q * (D + 2) + f] = o;
  }
  if (tid < nq) {
    const float M = fmaxf(fmaxf(S.mw[0][tid], S.mw[1][tid]), fmaxf(S.mw[2][tid], S.mw[3][tid]));
    float ls = 0.0f;
#pragma unroll
    for (int w = 0; w < 4; ++w) ls = fmaf(expf(S.mw[w][tid] - M), S.lw[w][tid], ls);
    part[tid * (D + 2) + D] = M;
    part[tid * (D + 2) + D + 1] = ls;
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
  if (a.T % ATT_BLK || a.ach % ATT_BLK || (int64_t)a.nchunk * a.ach < a.T) return hipErrorInvalidValue;
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
  const dim3 grid((a.T + ENC_CHUNK - 1) / ENC_CHUNK, a.N, a.ntab);
  if (a.T % 64) return hipErrorInvalidValue;  // passes of 64 tokens
  if (a.D == 128)
    hipLaunchKernelGGL(k_encode_resid<128>, grid, dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_encode_resid<64>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
  const dim3 grid((a.T + DEC_CHUNK - 1) / DEC_CHUNK, a.N, a.ntab);
  if (a.T % 64) return hipErrorInvalidValue;  // passes of 64 tokens
  if (a.D == 128)
    hipLaunchKernelGGL(k_decode<128>, grid, dim3(256), 0, s, a);
  else if (a.D == 64)
    hipLaunchKernelGGL(k_decode<64>, grid, dim3(256), 0, s, a);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace jolt
