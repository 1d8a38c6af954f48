// Record writer (encode) and reader (decode) for one chosen candidate per table.
//
// Encode follows "Rotated Tucker residual for outlier-resistant KV quantization",
// Implementation notes: with the stored Tucker factors, reconstruct X~, form
// R = X - X~, rotate each row of D values with Q = H diag(sigma) / sqrt(D), and store
// per block (one row) the scale s = max|Y| / (2^(b-1) - 1) (fp32) and the codes
// clip(round(Y / s), -2^(b-1), 2^(b-1) - 1).  The residual path runs in fp64.
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
  const int8_t* sgn = a.signs + tg * D + sg * FPT;
  uint32_t* codes = (uint32_t*)(e.rec + e.off_codes);
  float* scales = (float*)(e.rec + e.off_scales);
  const uint16_t* xsrc = (const uint16_t*)a.xsrc[tl];
  TileIn cur;
  codec_fetch_a<D>(cur, Lb, ls, K, tb);
  codec_fetch_row<D>(cur, xsrc, (int64_t)n * T + tb + rloc);
  for (int t0 = tb; t0 < te; t0 += CP) {
    const bool more = t0 + CP < te;  // uniform
    TileIn nxt;
    if (more) {
      codec_fetch_a<D>(nxt, Lb, ls, K, t0 + CP);
      codec_fetch_row<D>(nxt, xsrc, (int64_t)n * T + t0 + CP + rloc);
    }
    if (K > 0) codec_xtilde_in<D>(L, cur, K);
    __syncthreads();
    const int64_t row = (int64_t)n * T + t0 + rloc;
    double y[FPT];
    {
      const double* xt = &L.Xt[rloc][sg * FPT];
#pragma unroll
      for (int i = 0; i < FPT; ++i) {
        const uint16_t hb = (uint16_t)(cur.w[i >> 1] >> (16 * (i & 1)));
        const double x = (double)bf16_to_f32(hb);
        y[i] = K > 0 ? x - xt[i] : 0.0;
      }
    }
    int q[FPT];
    const float sc = codec_rotq<D>(y, sgn, sg, qmax, q);
    codec_store_codes(q, codes, row, D, sg, e.b);
    if (sg == 0) scales[row] = sc;
    __syncthreads();  // X~ tile is rewritten by the next pass
    if (more) cur = nxt;
  }
}

// Reconstruction, dequantization, inverse rotation, bf16 output.  The inverse Hadamard runs
// on the integer codes (exact); the residual s (H q)_f sigma_f / sqrt(D) is added to X~ by one
// fp32 FMA, and the sum is rounded once to bf16.
// Decode: workgroup (chunk of DEC_CHUNK tokens, slice n, table).  Rm and the B operands are
// set up once per workgroup; each pass of CP tokens fetches the next pass's L rows, codes and
// scales before its own products (no barrier inside the loop).
constexpr int DEC_CHUNK = 1024;

template <int D>
__global__ __launch_bounds__(256, 4) void k_decode(const DecodeArgs a) {
  constexpr int CP = 16 * 4 * 64 / D;  // tokens per pass: 16 per token tile, D / 64 waves per tile
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
  __shared__ DecLds<D> L;
  __shared__ float sgs[D];  // sigma_f / sqrt(D)
  const DecSrc d = dec_prepare<D>(L, sgs, e, n, T);
  dec_bops<D>(L);
  uint16_t* out = (uint16_t*)a.out[tl];
  DecIn cur;
  dec_fetch<D>(cur, d, e.b, n, T, tb);
  for (int t0 = tb; t0 < te; t0 += CP) {
    const bool more = t0 + CP < te;  // uniform
    DecIn nxt;
    if (more) dec_fetch<D>(nxt, d, e.b, n, T, t0 + CP);
    float4_t v[4];
    dec_vals<D>(&L.Bh[0][0][0][0], &L.Bl[0][0][0][0], sgs, d, e.b, cur, v);
    dec_store<D>(out, (int64_t)n * T + t0, v);
    if (more) cur = nxt;
  }
}

// ---------------------------------------------------------------- fused decode + attention
// O = softmax(Q K^T * scale) V for one layer group, K and V rebuilt from their records exactly
// as k_decode writes them (bf16 values), never stored.  Workgroup (chunk c, slice n, group g)
// takes the tokens [c ach, (c + 1) ach) of slice n and all nq queries of that slice, in blocks
// of 64 tokens, with the running softmax of flash attention:
//   1. K block: decode passes into LDS (bf16, token-major); scores S = K Q^T by bf16 MFMA
//      (exact products, fp32 sums), times `scale`;
//   2. per query: block maximum, new running maximum m, P = exp(S - m), running sum l and
//      the factor exp(m_old - m) for the output rows;
//   3. V block: decode passes into LDS (bf16, feature-major);
//   4. O = O exp(m_old - m) + P V by bf16 MFMA with P split into bf16 hi + lo (16 bits).
// The chunk's O (unnormalised), m and l go to the workspace; k_attend_merge combines the
// chunks: O = sum_c e^{m_c - M} O_c / sum_c e^{m_c - M} l_c.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int ATT_BLK = 64;  // tokens per block

template <int D>
struct AttLds {
  DecLds<D> L;                        // K's reconstruction operand and B operands
  half8_t Bvh[D / 64][4][4][16];      // V's B operands (copied out of L during set-up)
  half8_t Bvl[D / 64][4][4][16];
  float sgk[D], sgv[D];               // sigma_f / sqrt(D) of K and V
  union {
    uint16_t Kb[ATT_BLK][D + 8];      // K block, token-major bf16
    uint16_t Vt[D][ATT_BLK + 8];      // V block, feature-major bf16
  };
  float Sc[ATT_QMAX][ATT_BLK + 4];    // scores, then P
  float m[ATT_QMAX], l[ATT_QMAX], corr[ATT_QMAX];
};

// One decode pass of a record into the block buffer: token-major (K) or feature-major (V).
// Verbatim records (chain < 0) are copied from the record's bf16 rows.
template <int D, bool VT>
__device__ __forceinline__ void att_pass(AttLds<D>& S, const half8_t* Bh, const half8_t* Bl, const float* sg,
                                         const EncodeTable& e, const DecSrc& d, const DecIn& in, int n, int T, int t0,
                                         int row0) {
  if (e.chain < 0) {  // uniform; 256 threads x 16 values = CP rows of D
    const int sgm = threadIdx.x % (D / 16), rloc = threadIdx.x / (D / 16);
    const uint4* xr = (const uint4*)((const uint16_t*)(e.rec + e.off_core) + ((int64_t)n * T + t0 + rloc) * D + sgm * 16);
    const uint4 q0 = xr[0], q1 = xr[1];
    const uint32_t w[8] = {q0.x, q0.y, q0.z, q0.w, q1.x, q1.y, q1.z, q1.w};
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const uint16_t v = (uint16_t)(w[i >> 1] >> (16 * (i & 1)));
      if (VT) S.Vt[sgm * 16 + i][row0 + rloc] = v;
      else S.Kb[row0 + rloc][sgm * 16 + i] = v;
    }
    return;
  }
  constexpr int WPT = D / 64;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int tt = w / WPT, f0 = 64 * (w % WPT) + 4 * (lane & 15), lk = lane >> 4;
  float4_t v[4];
  dec_vals<D>(Bh, Bl, sg, d, e.b, in, v);
  if (VT) {  // 4 consecutive tokens of feature f0 + c
#pragma unroll
    for (int c = 0; c < 4; ++c)
      *(uint2*)&S.Vt[f0 + c][row0 + 16 * tt + 4 * lk] =
          make_uint2((uint32_t)dec_bf16(v[c][0]) | ((uint32_t)dec_bf16(v[c][1]) << 16),
                     (uint32_t)dec_bf16(v[c][2]) | ((uint32_t)dec_bf16(v[c][3]) << 16));
  } else {   // 4 consecutive features of token 16 tt + 4 lk + r
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *(uint2*)&S.Kb[row0 + 16 * tt + 4 * lk + r][f0] =
          make_uint2((uint32_t)dec_bf16(v[0][r]) | ((uint32_t)dec_bf16(v[1][r]) << 16),
                     (uint32_t)dec_bf16(v[2][r]) | ((uint32_t)dec_bf16(v[3][r]) << 16));
  }
}

template <int D>
__global__ __launch_bounds__(256, 2) void k_attend(const AttendArgs a) {
  constexpr int CP = 16 * 4 * 64 / D;        // tokens per decode pass
  constexpr int PPB = ATT_BLK / CP;          // decode passes per block
  constexpr int CT = D / 16 / 4;             // output feature tiles per wave
  const int c = blockIdx.x, n = blockIdx.y, g = blockIdx.z, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int li = lane & 15, lg = lane >> 4;
  const int T = a.T, nq = a.nq;
  const EncodeTable& ek = a.k[g];
  const EncodeTable& ev = a.v[g];
  const int tb = c * a.ach, te = min(T, tb + a.ach);
  __shared__ AttLds<D> S;
  // ---- set-up: V's operands first (copied aside), then K's (left in S.L)
  DecSrc dv{}, dk{};
  if (ev.chain >= 0) {
    dv = dec_prepare<D>(S.L, S.sgv, ev, n, T);
    dec_bops<D>(S.L);
    for (int idx = tid; idx < (D / 64) * 4 * 4 * 16; idx += 256) {
      (&S.Bvh[0][0][0][0])[idx] = (&S.L.Bh[0][0][0][0])[idx];
      (&S.Bvl[0][0][0][0])[idx] = (&S.L.Bl[0][0][0][0])[idx];
    }
    __syncthreads();
  }
  if (ek.chain >= 0) {
    dk = dec_prepare<D>(S.L, S.sgk, ek, n, T);
    dec_bops<D>(S.L);
  }
  if (tid < ATT_QMAX) {
    S.m[tid] = -INFINITY;
    S.l[tid] = 0.0f;
  }
  // queries as the B operand of the scores (column = query li, k = 32 kb + 8 lg .. + 7)
  bf16x8_t qf[D / 32];
#pragma unroll
  for (int kb = 0; kb < D / 32; ++kb) {
    uint4 u = make_uint4(0u, 0u, 0u, 0u);
    if (li < nq) u = *(const uint4*)(a.q[g] + ((int64_t)n * nq + li) * D + 32 * kb + 8 * lg);
    qf[kb] = __builtin_bit_cast(bf16x8_t, u);
  }
  float4_t acc[CT];
#pragma unroll
  for (int j = 0; j < CT; ++j) acc[j] = (float4_t){0.f, 0.f, 0.f, 0.f};
  __syncthreads();
  // decode passes in the order K passes of a block, then its V passes; each pass's inputs are
  // fetched one pass ahead
  auto fetch = [&](DecIn& in, int q) {
    const int blk = q / (2 * PPB), p = q % (2 * PPB);
    const int tp = tb + blk * ATT_BLK + (p % PPB) * CP;
    if (p < PPB) {
      if (ek.chain >= 0) dec_fetch<D>(in, dk, ek.b, n, T, tp);
    } else if (ev.chain >= 0) {
      dec_fetch<D>(in, dv, ev.b, n, T, tp);
    }
  };
  const int npass = (te - tb) / ATT_BLK * 2 * PPB;
  int q = 0;
  DecIn cur;
  if (npass > 0) fetch(cur, 0);
  for (int t0 = tb; t0 < te; t0 += ATT_BLK) {
    // ---- 1. K block and its scores
#pragma unroll
    for (int p = 0; p < PPB; ++p, ++q) {
      DecIn nxt;
      if (q + 1 < npass) fetch(nxt, q + 1);
      att_pass<D, false>(S, &S.L.Bh[0][0][0][0], &S.L.Bl[0][0][0][0], S.sgk, ek, dk, cur, n, T, t0 + p * CP,
                         p * CP);
      cur = nxt;
    }
    __syncthreads();
    {
      float4_t sc = (float4_t){0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < D / 32; ++kb) {
        const bf16x8_t kf = *(const bf16x8_t*)&S.Kb[16 * wave + li][32 * kb + 8 * lg];
        sc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[kb], sc, 0, 0, 0);
      }
      // element (token 16 wave + 4 lg + r, query li)
      if (li < nq)
#pragma unroll
        for (int r = 0; r < 4; ++r) S.Sc[li][16 * wave + 4 * lg + r] = sc[r] * a.scale;
    }
    __syncthreads();
    // ---- 2. running softmax: wave w takes queries w, w + 4, ...; lane = token
    for (int q = wave; q < nq; q += 4) {
      const float sv = S.Sc[q][lane];
      const float mo = S.m[q];
      const float mn = fmaxf(mo, wave_max_f32(sv));
      const float pv = expf(sv - mn);
      float ls = pv;
      for (int o = 32; o > 0; o >>= 1) ls += __shfl_xor(ls, o, 64);
      S.Sc[q][lane] = pv;
      if (lane == 0) {
        const float cf = expf(mo - mn);  // 0 on the first block (mo = -inf)
        S.corr[q] = cf;
        S.l[q] = S.l[q] * cf + ls;
        S.m[q] = mn;
      }
    }
    // ---- 3. V block, feature-major (the K block is consumed)
#pragma unroll
    for (int p = 0; p < PPB; ++p, ++q) {
      DecIn nxt;
      if (q + 1 < npass) fetch(nxt, q + 1);
      att_pass<D, true>(S, &S.Bvh[0][0][0][0], &S.Bvl[0][0][0][0], S.sgv, ev, dv, cur, n, T, t0 + p * CP,
                        p * CP);
      cur = nxt;
    }
    __syncthreads();
    // ---- 4. O = O corr + P V; output tile (query 4 lg + r, feature 16 ct + li)
    {
      float cr[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) cr[r] = 4 * lg + r < nq ? S.corr[4 * lg + r] : 0.0f;
#pragma unroll
      for (int j = 0; j < CT; ++j)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[j][r] *= cr[r];
#pragma unroll
      for (int ks = 0; ks < ATT_BLK / 32; ++ks) {
        bf16x8_t ph, pl;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const float pv = li < nq ? S.Sc[li][32 * ks + 8 * lg + e] : 0.0f;
          const __bf16 hb = (__bf16)pv;
          ph[e] = hb;
          pl[e] = (__bf16)(pv - (float)hb);
        }
#pragma unroll
        for (int j = 0; j < CT; ++j) {
          const int f = 16 * (CT * wave + j) + li;
          const bf16x8_t vf = *(const bf16x8_t*)&S.Vt[f][32 * ks + 8 * lg];
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ph, vf, acc[j], 0, 0, 0);
          acc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pl, vf, acc[j], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }
  float* part = a.part + ((((int64_t)g * a.N + n) * a.nchunk + c) * nq) * (D + 2);
#pragma unroll
  for (int j = 0; j < CT; ++j)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int q = 4 * lg + r, f = 16 * (CT * wave + j) + li;
      if (q < nq) part[q * (D + 2) + f] = acc[j][r];
    }
  if (tid < nq) {
    part[tid * (D + 2) + D] = S.m[tid];
    part[tid * (D + 2) + D + 1] = S.l[tid];
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
  const dim3 grid((a.T + DEC_CHUNK - 1) / DEC_CHUNK, a.N, a.ntab);
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
