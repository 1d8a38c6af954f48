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

#ifdef JOLT_CODEC_TIMING
#define CODEC_TILE_MARK(i) CD_MARK(i)
#endif
}  // namespace jolt
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

// Reconstruction, dequantization, inverse rotation, bf16 output.  Block (token chunk,
// slice n, local table).  The inverse Hadamard runs on the integer codes (exact); the
// residual s (H q)_f sigma_f / sqrt(D) is added to X~ with one fp64 rounding, and the sum
// is rounded once to bf16.
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
  __syncthreads();  // Rm and the signs are read-only from here: no barrier inside the loop
  DecIn cur;
  dec_fetch<D>(cur, d, e.b, n, T, tb);
  for (int t0 = tb; t0 < te; t0 += CP) {
    const bool more = t0 + CP < te;  // uniform
    DecIn nxt;
    if (more) dec_fetch<D>(nxt, d, e.b, n, T, t0 + CP);
    uint16_t v[4][4];
    dec_regs<D>(L, sgs, e.b, d.K, cur, v);
    dec_store<D>(out, (int64_t)n * T + t0, v);
    if (t0 == tb) CD_MARK(2);
    if (more) cur = nxt;
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
// One pass of rebuilt rows for the attention: fetch (one pass ahead) and decode into Xd as
// fp32 (the bf16 values jolt_decode writes).  Verbatim records hold X itself: the pass then
// carries this thread's 16 values of its row segment in q.
template <int D>
__device__ __forceinline__ void attend_fetch(DecIn& in, const EncodeTable& e, const DecodeSrc& d, int n, int T,
                                             int t0) {
  if (e.chain < 0) {
    const int sg = threadIdx.x % (D / 16), rloc = threadIdx.x / (D / 16);
    const uint4* xr = (const uint4*)((const uint16_t*)(e.rec + e.off_core) + ((int64_t)n * T + t0 + rloc) * D + sg * 16);
    const uint4 q0 = xr[0], q1 = xr[1];
    in.q[0] = make_uint2(q0.x, q0.y);
    in.q[1] = make_uint2(q0.z, q0.w);
    in.q[2] = make_uint2(q1.x, q1.y);
    in.q[3] = make_uint2(q1.z, q1.w);
  } else {
    dec_fetch<D>(in, d, e.b, n, T, t0);
  }
}

template <int D>
__device__ __forceinline__ void attend_rows(const CodecLds<D>& L, const double* sgs, const EncodeTable& e,
                                            const DecodeSrc& d, const DecIn& in, float (*Xd)[D + 4]) {
  if (e.chain < 0) {  // uniform: row layout, 16 values of segment sg of row rloc
    const int sg = threadIdx.x % (D / 16), rloc = threadIdx.x / (D / 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const uint32_t w0 = in.q[i].x, w1 = in.q[i].y;
      Xd[rloc][sg * 16 + 4 * i] = bf16_to_f32((uint16_t)(w0 & 0xFFFFu));
      Xd[rloc][sg * 16 + 4 * i + 1] = bf16_to_f32((uint16_t)(w0 >> 16));
      Xd[rloc][sg * 16 + 4 * i + 2] = bf16_to_f32((uint16_t)(w1 & 0xFFFFu));
      Xd[rloc][sg * 16 + 4 * i + 3] = bf16_to_f32((uint16_t)(w1 >> 16));
    }
  } else {  // tile layout of dec_regs
    constexpr int WPT = D / 64;
    const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const int tt = w / WPT, f0 = 64 * (w % WPT) + 4 * (lane & 15), lk = lane >> 4;
    uint16_t v[4][4];
    dec_regs<D>(L, sgs, e.b, d.K, in, v);
#pragma unroll
    for (int r = 0; r < 4; ++r)
#pragma unroll
      for (int c = 0; c < 4; ++c) Xd[16 * tt + 4 * r + lk][f0 + c] = bf16_to_f32(v[c][r]);
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
  DecIn cur;
  attend_fetch<D>(cur, ek, d, n, T, tb);
  for (int t0 = tb; t0 < te; t0 += CP) {
    const bool more = t0 + CP < te;  // uniform
    DecIn nxt;
    if (more) attend_fetch<D>(nxt, ek, d, n, T, t0 + CP);
    attend_rows<D>(L, sgs, ek, d, cur, Xd);
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
    if (more) cur = nxt;
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
  attend_fetch<D>(cur, ev, d, n, T, tb);
  for (int t0 = tb; t0 < te; t0 += CP) {
    const bool more = t0 + CP < te;  // uniform
    DecIn nxt;
    if (more) attend_fetch<D>(nxt, ev, d, n, T, t0 + CP);
    attend_rows<D>(L, sgs, ev, d, cur, Xd);
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
    if (more) cur = nxt;
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
