// bf16 window-attention backward on MFMA (gfx950), d = 32, any M <= 32.
//
// Backward of exact window attention with window-local 2D RoPE, recomputing P from the forward's
// log-sum-exp so that no score matrix is ever stored (FlashSwin paper card, "FLASHSWIN: Unlocking
// Large Windows and Dense Tokens in Swin Vision Transformers with Memory Efficient Attention":
// Abstract, flat training memory in the window size; Table S1).  In the log2 domain with
// q^ = q~ log2(e) / sqrt(d):  P = exp2(q^ . k~ - LSE log2(e)),  dS = P (dO . v - Delta),
// dq~ = sum_j dS k~ / sqrt(d),  dk~ = sum_i dS q~ / sqrt(d),  dv = sum_i P dO,
// dq = R^T dq~, dk = R^T dk~, and dtheta += p (dx~_b x~_a - dx~_a x~_b) over Q and K tokens.
//
// Three kernels, all deterministic (no atomics):
//  * prologue, one workgroup per window-head: Delta = rowsum(dO * O) per token, and the window's
//    largest |dO| and |v| components, which fix power-of-two scales for the fp16 operands below;
//  * dK/dV, key-stationary: a wave owns 32 keys (lane = key); queries stream through LDS in
//    chunks.  S = Q^ K~^T and dP = dO V^T start from -LSE / -Delta tiles read from LDS (one value
//    per query row), so P = exp2(S) and dS = P * dP cost one exp and one multiply per score;
//    dV^T += dO^T P and dK~^T += Q^T dS;
//  * dQ, query-stationary: a wave owns 32 queries (lane = query); keys stream through LDS.
//    S^T = K~ Q^T and dP^T = V dO^T start from the lane's -LSE and -Delta; dQ~^T += K~^T dS^T.
// Operand precision: the inputs q, k, v, dO are bf16, so dP = dO V^T is exact on bf16 MFMA.  The
// derived operands (rotated Q^ and K~, P, dS, the scaled dO of the dV product) go to fp16 MFMAs,
// 8x finer than bf16; dS and dO are pre-scaled by powers of two derived from the prologue's
// bounds (|dS| <= 64 max|dO| max|v|), so they cannot leave fp16 range.  A chunk whose rotated
// Q^ or K~ exceeds the fp16 range is done with bf16 operands instead.  Each workgroup reduces its
// dtheta terms in a fixed order into one partials row; a last kernel sums the rows in order.
#include <algorithm>
#include <mutex>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"

namespace fsw {

namespace {

constexpr int kCh = 128;       // tokens per LDS chunk
constexpr int kMaxChunks = 8;  // NP <= 1024
constexpr int kNW = 4;         // waves per workgroup: 128 queries (dQ) or 128 keys (dK/dV)

__host__ __device__ inline int chunk_len(int NP) { return NP < kCh ? NP : kCh; }
__host__ __device__ inline size_t table_bytes(int M) { return (size_t)2 * 2 * M * 8 * 4; }

__device__ inline void fill_table(float* sn, float* cs, const float* th_row, const float* th_col, int head, int M,
                                  int tid, int nt) {
  for (int i = tid; i < 2 * M * 8; i += nt) {
    const int axis = i / (M * 8);
    const int p = (i / 8) % M;
    const int j = i % 8;
    const float th = axis ? th_col[head * 8 + j] : th_row[head * 8 + j];
    float s, c;
    rope_sincos(th, p, &s, &c);
    sn[i] = s;
    cs[i] = c;
  }
}

// Labels of the tokens of one chunk and the per-32-block summaries (labels present, all valid).
__device__ inline void chunk_labels(const Geom& g, const WinHead& w, int c0, int ch, uint8_t* lab, int tid, int nt) {
  for (int n = tid; n < ch; n += nt) {
    const int t = c0 + n;
    lab[n] = t < g.N ? (uint8_t)token_label(g, w.wy, w.wx, t / g.M, t % g.M) : (uint8_t)0xff;
  }
}
__device__ inline void block_info(const uint8_t* lab, int ch, uint32_t* blk, int tid, int nt) {
  for (int b = tid; b < ch / 32; b += nt) {
    uint32_t bits = 0, full = 1;
    for (int j = 0; j < 32; ++j) {
      const uint8_t lb = lab[b * 32 + j];
      if (lb == 0xff)
        full = 0;
      else
        bits |= 1u << lb;
    }
    blk[b] = bits | (full << 9);
  }
}

// Write 8 16-bit values (one 16-byte part of a token row) into a transposed [32][stride] array.
__device__ __forceinline__ void write_t(uint16_t* t, int stride, int part, int pos, uint4 val) {
  const uint32_t w4[4] = {val.x, val.y, val.z, val.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    t[(size_t)(part * 8 + 2 * e) * stride + pos] = (uint16_t)(w4[e] & 0xffffu);
    t[(size_t)(part * 8 + 2 * e + 1) * stride + pos] = (uint16_t)(w4[e] >> 16);
  }
}

__device__ __forceinline__ bool any_big(const float (&x)[8]) {
  bool b = false;
#pragma unroll
  for (int e = 0; e < 8; ++e) b |= !(fabsf(x[e]) < kF16Limit);
  return b;
}

// Power of two 2^k with 2^k * bound <= 2^14 (1 when bound is 0 or not finite).
__device__ __forceinline__ float pow2_scale(float bound) {
  if (!(bound > 0.f) || !(bound < INFINITY)) return 1.f;
  int e;
  frexpf(bound, &e);  // bound < 2^e
  return ldexpf(1.f, 14 - e);
}

template <bool H16>
__device__ __forceinline__ uint32_t pack_op2(float a, float b) {
  if constexpr (H16)
    return pack2h(a, b);
  else
    return pack2(a, b);
}

// Stage rotated rows (times `scale`) of tokens c0 .. c0+CH of `src`: row-major into `rows` and,
// when tr != nullptr, transposed into `tr`; fp16 (h16) or bf16.  Sets *flag when a value is out
// of fp16 range (only checked when h16).
__device__ inline void stage_rotated(const uint16_t* __restrict__ src, const Geom& g, const WinHead& w, int c0, int CH,
                                     const float* sn, const float* cs, float scale, bool h16, uint16_t* rows,
                                     uint16_t* tr, int tst, uint32_t* flag, int tid, int nt) {
  const int M = g.M, N = g.N;
  const int64_t rowstride = (int64_t)g.heads * 32;
  for (int it = tid; it < CH * 4; it += nt) {
    const int n = it >> 2, part = it & 3;
    const int tn = c0 + n;
    float x[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    if (tn < N) {
      const int r = tn / M, c = tn - (tn / M) * M;
      const int64_t off = token_index(g, w.b, w.wy, w.wx, r, c) * rowstride + w.h * 32 + part * 8;
      unpack8(*reinterpret_cast<const uint4*>(src + off), x);
      const int axis = part >> 1;
      rotate8(x, sn, cs, axis, M, axis ? c : r, (part & 1) * 4);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= scale;
    }
    const uint4 packed = pack8_op(x, h16);
    *reinterpret_cast<uint4*>(rows + n * kKStride + part * 8) = packed;
    if (tr) write_t(tr, tst, part, vt_pos(n), packed);
    if (h16 && flag && any_big(x)) atomicOr(flag, 1u);
  }
}

// Rows of tokens c0 .. c0+CH of `src` (bf16, unchanged) into `rows` (when not null); when tr is
// not null also `scale * src` transposed into `tr` in fp16 (h16) or bf16.
__device__ inline void stage_plain(const uint16_t* __restrict__ src, const Geom& g, const WinHead& w, int c0, int CH,
                                   uint16_t* rows, uint16_t* tr, int tst, float scale, bool h16, int tid, int nt) {
  const int M = g.M, N = g.N;
  const int64_t rowstride = (int64_t)g.heads * 32;
  for (int it = tid; it < CH * 4; it += nt) {
    const int n = it >> 2, part = it & 3;
    const int tn = c0 + n;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (tn < N) {
      const int r = tn / M, c = tn - (tn / M) * M;
      val = *reinterpret_cast<const uint4*>(src + token_index(g, w.b, w.wy, w.wx, r, c) * rowstride + w.h * 32 +
                                            part * 8);
    }
    if (rows) *reinterpret_cast<uint4*>(rows + n * kKStride + part * 8) = val;
    if (tr) {
      float x[8];
      unpack8(val, x);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= scale;
      write_t(tr, tst, part, vt_pos(n), pack8_op(x, h16));
    }
  }
}

// Fixed-order reduction of each lane's 8 dtheta slots (for its channels 8g + 4h + {0..3}) over
// the workgroup into one 16-float partials row: slots 0..7 row-axis pairs, 8..15 column-axis.
// Lane slot (g, u) = pair 4(g&1) + 2h + u of axis g>>1.
template <int NW>
__device__ inline void reduce_dtheta(float (&t)[8], float* red, float* dst, int lane, int wave, int tid) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) t[i] += __shfl_xor(t[i], o, 64);
  }
  if ((lane & 31) == 0) {
    const int h = lane >> 5;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq)
#pragma unroll
      for (int u = 0; u < 2; ++u) red[wave * 16 + (gq >> 1) * 8 + 4 * (gq & 1) + 2 * h + u] = t[2 * gq + u];
  }
  __syncthreads();
  if (tid < 16) {
    float s = 0.f;
    for (int i = 0; i < NW; ++i) s += red[i * 16 + tid];
    dst[tid] = s;
  }
}

// Epilogue shared by the dQ and dK kernels: for the lane's token, take the gradient w.r.t. the
// rotated vector (dxt[v] * scale, channel 8*(v/4) + 4h + v%4), recompute the rotated input,
// accumulate dtheta slots, un-rotate and store bf16.
// The dtheta integrand uses the rotated input exactly as the gradient products saw it (rounded
// to fp16 or bf16 after scaling by `op_scale`, then scaled back): the Q-side and K-side sums of
// the integrand cancel in their position-independent part, and that cancellation only survives
// rounding when both sides are formed from the same operand values the products used.
__device__ inline void unrotate_store(const f32x16_t& dxt, float scale, float op_scale, bool op16,
                                      const uint16_t* xsrc, uint16_t* dst, const float* sn, const float* cs, int M,
                                      int r, int c, int h, float (&t)[8]) {
  const float inv_op = 1.f / op_scale;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    const uint2 raw = *reinterpret_cast<const uint2*>(xsrc + 8 * gq + 4 * h);
    const float xin[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                          __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
    const int axis = gq >> 1;
    const int pos = axis ? c : r;
    float res[4];
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int j = 4 * (gq & 1) + 2 * h + u;
      const float s = sn[(axis * M + pos) * 8 + j];
      const float co = cs[(axis * M + pos) * 8 + j];
      const float a = xin[2 * u], b = xin[2 * u + 1];
      const float ar = (a * co - b * s) * op_scale, br = (a * s + b * co) * op_scale;
      float at, bt;
      if (op16) {
        at = (float)(_Float16)ar * inv_op;
        bt = (float)(_Float16)br * inv_op;
      } else {
        at = bf16_bits_to_float(float_to_bf16_bits(ar)) * inv_op;
        bt = bf16_bits_to_float(float_to_bf16_bits(br)) * inv_op;
      }
      const float da = dxt[4 * gq + 2 * u] * scale, db = dxt[4 * gq + 2 * u + 1] * scale;
      t[2 * gq + u] += (float)pos * (db * at - da * bt);
      res[2 * u] = da * co + db * s;  // R^T (da, db)
      res[2 * u + 1] = -da * s + db * co;
    }
    uint2 o;
    o.x = pack2(res[0], res[1]);
    o.y = pack2(res[2], res[3]);
    *reinterpret_cast<uint2*>(dst + 8 * gq + 4 * h) = o;
  }
}

// ------------------------------------------------------------------------------------ prologue

// One workgroup per window-head: Delta for every token, and scal[wh] = {max |dO|, max |v|}.
__global__ __launch_bounds__(256) void bwd_pre_kernel(const uint16_t* __restrict__ out,
                                                      const uint16_t* __restrict__ dout,
                                                      const uint16_t* __restrict__ v, float* __restrict__ delta,
                                                      float* __restrict__ scal, Geom g) {
  __shared__ float red[2][4];
  const int64_t wh = blockIdx.x;
  const WinHead w = decode_winhead(g, wh);
  const int tid = threadIdx.x;
  const int64_t rowstride = (int64_t)g.heads * 32;
  float gmax = 0.f, vmax = 0.f;
  const int items = g.N * 4;
  const int iters = (items + 255) / 256;
  for (int i = 0; i < iters; ++i) {  // uniform trip count: the shuffles below see every lane
    const int it = i * 256 + tid;
    float s = 0.f;
    int64_t tok = 0;
    const bool ok = it < items;
    if (ok) {
      const int n = it >> 2, part = it & 3;
      const int r = n / g.M, c = n - (n / g.M) * g.M;
      tok = token_index(g, w.b, w.wy, w.wx, r, c);
      const int64_t off = tok * rowstride + w.h * 32 + part * 8;
      float o[8], d[8], vv[8];
      unpack8(*reinterpret_cast<const uint4*>(out + off), o);
      unpack8(*reinterpret_cast<const uint4*>(dout + off), d);
      unpack8(*reinterpret_cast<const uint4*>(v + off), vv);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s = __builtin_fmaf(o[e], d[e], s);
        gmax = fmaxf(gmax, fabsf(d[e]));
        vmax = fmaxf(vmax, fabsf(vv[e]));
      }
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    if (ok && (it & 3) == 0) delta[tok * g.heads + w.h] = s;
  }
  gmax = wave_max(gmax);
  vmax = wave_max(vmax);
  if ((tid & 63) == 0) {
    red[0][tid >> 6] = gmax;
    red[1][tid >> 6] = vmax;
  }
  __syncthreads();
  if (tid == 0) {
    scal[wh * 2] = fmaxf(fmaxf(red[0][0], red[0][1]), fmaxf(red[0][2], red[0][3]));
    scal[wh * 2 + 1] = fmaxf(fmaxf(red[1][0], red[1][1]), fmaxf(red[1][2], red[1][3]));
  }
}

// ---------------------------------------------------------------------------------------- dQ

template <bool H16>
__device__ __forceinline__ void dq_chunk(const uint16_t* sK, const uint16_t* sV, const uint16_t* sKt,
                                         const uint8_t* sLab, const uint32_t* sBlk, int kst, int nblk, int col, int h,
                                         uint32_t wave_labels, bool wave_single, int qlab, uint4 qo0, uint4 qo1,
                                         const bf16x8_t& gb0, const bf16x8_t& gb1, const f32x16_t& cL,
                                         const f32x16_t& cD, float ds_scale, f32x16_t& acc) {
  for (int kb = 0; kb < nblk; ++kb) {
    const uint32_t info = sBlk[kb];
    const uint32_t bl = info & 0x1ffu;
    if ((bl & wave_labels) == 0) continue;
    const bool need_mask = !((info >> 9) & 1u) || !wave_single || bl != wave_labels;
    const uint16_t* krow = sK + (kb * 32 + col) * kKStride + 8 * h;
    const uint16_t* vrow = sV + (kb * 32 + col) * kKStride + 8 * h;
    f32x16_t s = mfma_op<H16>(*reinterpret_cast<const uint4*>(krow), qo0, cL);
    s = mfma_op<H16>(*reinterpret_cast<const uint4*>(krow + 16), qo1, s);
    f32x16_t dp = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(vrow)), gb0, cD);
    dp = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 16)), gb1, dp);
    const uint32_t live = need_mask ? live_bits(sLab, kb, h, qlab) : 0xffffu;
    float ds[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float p = __builtin_amdgcn_exp2f(s[e]) * ds_scale;
      ds[e] = ((live >> e) & 1u) ? p * dp[e] : 0.f;
    }
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[e] = pack_op2<H16>(ds[2 * e], ds[2 * e + 1]);
    const uint16_t* ktrow = sKt + col * kst + kb * 32 + 8 * h;
    acc = mfma_op<H16>(*reinterpret_cast<const uint4*>(ktrow), make_uint4(pk[0], pk[1], pk[2], pk[3]), acc);
    acc = mfma_op<H16>(*reinterpret_cast<const uint4*>(ktrow + 16), make_uint4(pk[4], pk[5], pk[6], pk[7]), acc);
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dq_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dq, float* __restrict__ partials, Geom g, int nb, int NP) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int D = 32;
  constexpr int NT = NW * 64;
  const int M = g.M, N = g.N;
  const int CH = chunk_len(NP);
  const int kst = vt_stride(CH);
  uint16_t* sK = reinterpret_cast<uint16_t*>(smem_raw);
  uint16_t* sV = sK + CH * kKStride;
  uint16_t* sKt = sV + CH * kKStride;
  float* sn = reinterpret_cast<float*>(sKt + 32 * kst);
  float* cs = sn + 2 * M * 8;
  float* red = cs + 2 * M * 8;
  uint32_t* sBlk = reinterpret_cast<uint32_t*>(red + NW * 16);
  uint32_t* sFlag = sBlk + kCh / 32;  // [0]: some |q^| out of fp16 range; [1 + chunk]: some |k~| in the chunk
  uint8_t* sLab = reinterpret_cast<uint8_t*>(sFlag + 1 + kMaxChunks);

  const int64_t blk = blockIdx.x;
  const int64_t wh = blk / nb;
  const WinHead w = decode_winhead(g, wh);
  const int qblock = (int)(blk % nb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int64_t rowstride = (int64_t)g.heads * D;
  const float qscale = kLog2e * 0.17677669529663687f;
  // |dS| <= |dO . v| + |Delta| <= 64 max|dO| max|v|: scale so the fp16 dS stays in range
  const float ds_scale = pow2_scale(64.f * scal[wh * 2] * scal[wh * 2 + 1]);

  fill_table(sn, cs, th_row, th_col, w.h, M, tid, NT);
  if (tid <= kMaxChunks) sFlag[tid] = 0;
  __syncthreads();

  // the lane's query: Q^ in both operand formats, dO as bf16 B operands, -LSE and -Delta
  const int qi = qblock * NW * 32 + wave * 32 + col;
  const bool valid = qi < N;
  int r = 0, c = 0, qlab = 0xff;
  int64_t tok = 0;
  uint4 qh0 = make_uint4(0, 0, 0, 0), qh1 = qh0, qf0 = qh0, qf1 = qh0, g0 = qh0, g1 = qh0;
  float lse2 = 0.f, del = 0.f;
  if (valid) {
    r = qi / M;
    c = qi - r * M;
    tok = token_index(g, w.b, w.wy, w.wx, r, c);
    qlab = token_label(g, w.wy, w.wx, r, c);
    const int64_t off = tok * rowstride + w.h * D;
    float x[8], y[8];
    unpack8(*reinterpret_cast<const uint4*>(q + off + 8 * h), x);
    unpack8(*reinterpret_cast<const uint4*>(q + off + 16 + 8 * h), y);
    rotate8(x, sn, cs, 0, M, r, 4 * h);
    rotate8(y, sn, cs, 1, M, c, 4 * h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] *= qscale;
      y[e] *= qscale;
    }
    qh0 = pack8_op(x, true);
    qh1 = pack8_op(y, true);
    qf0 = pack8_op(x, false);
    qf1 = pack8_op(y, false);
    if (any_big(x) || any_big(y)) atomicOr(&sFlag[0], 1u);
    g0 = *reinterpret_cast<const uint4*>(dout + off + 8 * h);
    g1 = *reinterpret_cast<const uint4*>(dout + off + 16 + 8 * h);
    lse2 = lse[tok * g.heads + w.h] * kLog2e;
    del = delta[tok * g.heads + w.h];
  }
  const bf16x8_t gb0 = as_bf16x8(g0), gb1 = as_bf16x8(g1);
  f32x16_t cL, cD, acc;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    cL[e] = -lse2;
    cD[e] = -del;
    acc[e] = 0.f;
  }
  const uint32_t wave_labels = wave_or(valid ? (1u << qlab) : 0u);
  const bool wave_single = __builtin_popcount(wave_labels) == 1;
  bool all16 = true;

  for (int c0 = 0, ci = 0; c0 < NP; c0 += CH, ++ci) {
    __syncthreads();
    const bool qbig = sFlag[0] != 0;
    stage_rotated(k, g, w, c0, CH, sn, cs, 1.f, !qbig, sK, sKt, kst, &sFlag[1 + ci], tid, NT);
    stage_plain(v, g, w, c0, CH, sV, nullptr, 0, 1.f, false, tid, NT);
    chunk_labels(g, w, c0, CH, sLab, tid, NT);
    __syncthreads();
    block_info(sLab, CH, sBlk, tid, NT);
    const bool h16 = !qbig && sFlag[1 + ci] == 0;
    if (!h16 && !qbig) stage_rotated(k, g, w, c0, CH, sn, cs, 1.f, false, sK, sKt, kst, nullptr, tid, NT);
    __syncthreads();
    all16 = all16 && h16;
    if (wave_labels == 0) continue;
    const int nblk = min(CH, NP - c0) / 32;
    if (h16)
      dq_chunk<true>(sK, sV, sKt, sLab, sBlk, kst, nblk, col, h, wave_labels, wave_single, qlab, qh0, qh1, gb0, gb1,
                     cL, cD, ds_scale, acc);
    else
      dq_chunk<false>(sK, sV, sKt, sLab, sBlk, kst, nblk, col, h, wave_labels, wave_single, qlab, qf0, qf1, gb0, gb1,
                      cL, cD, ds_scale, acc);
  }

  float t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (valid) {
    const int64_t off = tok * rowstride + w.h * D;
    // dq~ = acc / ds_scale / sqrt(d); the dtheta integrand takes q~ as the dK product saw it
    unrotate_store(acc, 0.17677669529663687f / ds_scale, qscale, all16, q + off, dq + off, sn, cs, M, r, c, h, t);
  }
  const int64_t prow = ((int64_t)w.h * 2 + 1) * (g.B * g.nH * g.nW * nb) + wh / g.heads * nb + qblock;
  reduce_dtheta<NW>(t, red, partials + prow * 16, lane, wave, tid);
}

// -------------------------------------------------------------------------------------- dK / dV

template <bool H16>
__device__ __forceinline__ void dkdv_chunk(const uint16_t* sQ, const uint16_t* sG, const uint16_t* sQt,
                                           const uint16_t* sGt, const float* sL, const float* sD, const uint8_t* sLab,
                                           const uint32_t* sBlk, int tst, int nblk, int col, int h,
                                           uint32_t wave_labels, bool wave_single, int klab, uint4 ko0, uint4 ko1,
                                           const bf16x8_t& vb0, const bf16x8_t& vb1, float ds_scale,
                                           f32x16_t& accv, f32x16_t& acck) {
  for (int qb = 0; qb < nblk; ++qb) {
    const uint32_t info = sBlk[qb];
    const uint32_t bl = info & 0x1ffu;
    if ((bl & wave_labels) == 0) continue;
    const bool need_mask = !((info >> 9) & 1u) || !wave_single || bl != wave_labels;
    // -LSE and -Delta of the 16 query rows this lane's accumulators hold: 8g + 4h + j
    f32x16_t cL, cD;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const float4 l4 = *reinterpret_cast<const float4*>(sL + qb * 32 + 8 * gq + 4 * h);
      const float4 d4 = *reinterpret_cast<const float4*>(sD + qb * 32 + 8 * gq + 4 * h);
      cL[4 * gq] = -l4.x;
      cL[4 * gq + 1] = -l4.y;
      cL[4 * gq + 2] = -l4.z;
      cL[4 * gq + 3] = -l4.w;
      cD[4 * gq] = -d4.x;
      cD[4 * gq + 1] = -d4.y;
      cD[4 * gq + 2] = -d4.z;
      cD[4 * gq + 3] = -d4.w;
    }
    const uint16_t* qrow = sQ + (qb * 32 + col) * kKStride + 8 * h;
    const uint16_t* grow = sG + (qb * 32 + col) * kKStride + 8 * h;
    f32x16_t s = mfma_op<H16>(*reinterpret_cast<const uint4*>(qrow), ko0, cL);
    s = mfma_op<H16>(*reinterpret_cast<const uint4*>(qrow + 16), ko1, s);
    f32x16_t dp = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(grow)), vb0, cD);
    dp = mfma32x32x16(as_bf16x8(*reinterpret_cast<const uint4*>(grow + 16)), vb1, dp);
    const uint32_t live = need_mask ? live_bits(sLab, qb, h, klab) : 0xffffu;
    float p[16], ds[16];
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      const float pe = ((live >> e) & 1u) ? __builtin_amdgcn_exp2f(s[e]) : 0.f;
      p[e] = pe;
      ds[e] = pe * ds_scale * dp[e];
    }
    uint32_t pp[8], pd[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      pp[e] = pack_op2<H16>(p[2 * e], p[2 * e + 1]);
      pd[e] = pack_op2<H16>(ds[2 * e], ds[2 * e + 1]);
    }
    const uint16_t* gtrow = sGt + col * tst + qb * 32 + 8 * h;
    const uint16_t* qtrow = sQt + col * tst + qb * 32 + 8 * h;
    accv = mfma_op<H16>(*reinterpret_cast<const uint4*>(gtrow), make_uint4(pp[0], pp[1], pp[2], pp[3]), accv);
    accv = mfma_op<H16>(*reinterpret_cast<const uint4*>(gtrow + 16), make_uint4(pp[4], pp[5], pp[6], pp[7]), accv);
    acck = mfma_op<H16>(*reinterpret_cast<const uint4*>(qtrow), make_uint4(pd[0], pd[1], pd[2], pd[3]), acck);
    acck = mfma_op<H16>(*reinterpret_cast<const uint4*>(qtrow + 16), make_uint4(pd[4], pd[5], pd[6], pd[7]), acck);
  }
}

template <int NW>
__global__ __launch_bounds__(NW * 64) void bwd_dkdv_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ partials, Geom g, int nb, int NP) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int D = 32;
  constexpr int NT = NW * 64;
  const int M = g.M, N = g.N;
  const int CH = chunk_len(NP);
  const int tst = vt_stride(CH);
  uint16_t* sQ = reinterpret_cast<uint16_t*>(smem_raw);
  uint16_t* sG = sQ + CH * kKStride;
  uint16_t* sQt = sG + CH * kKStride;
  uint16_t* sGt = sQt + 32 * tst;
  float* sL = reinterpret_cast<float*>(sGt + 32 * tst);
  float* sD = sL + kCh;
  float* sn = sD + kCh;
  float* cs = sn + 2 * M * 8;
  float* red = cs + 2 * M * 8;
  uint32_t* sBlk = reinterpret_cast<uint32_t*>(red + NW * 16);
  uint32_t* sFlag = sBlk + kCh / 32;  // [0]: some |k~| out of fp16 range; [1 + chunk]: some |q^| in the chunk
  uint8_t* sLab = reinterpret_cast<uint8_t*>(sFlag + 1 + kMaxChunks);

  const int64_t blk = blockIdx.x;
  const int64_t wh = blk / nb;
  const WinHead w = decode_winhead(g, wh);
  const int kblock = (int)(blk % nb);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int64_t rowstride = (int64_t)g.heads * D;
  const float qscale = kLog2e * 0.17677669529663687f;
  const float g_scale = pow2_scale(scal[wh * 2]);                             // fp16 dO of the dV product
  const float ds_scale = pow2_scale(64.f * scal[wh * 2] * scal[wh * 2 + 1]);  // fp16 dS of the dK product

  fill_table(sn, cs, th_row, th_col, w.h, M, tid, NT);
  if (tid <= kMaxChunks) sFlag[tid] = 0;
  __syncthreads();

  // the lane's key: K~ in both operand formats, V as bf16 B operands
  const int kj = kblock * NW * 32 + wave * 32 + col;
  const bool valid = kj < N;
  int r = 0, c = 0, klab = 0xff;
  int64_t tok = 0;
  uint4 kh0 = make_uint4(0, 0, 0, 0), kh1 = kh0, kf0 = kh0, kf1 = kh0, v0 = kh0, v1 = kh0;
  if (valid) {
    r = kj / M;
    c = kj - r * M;
    tok = token_index(g, w.b, w.wy, w.wx, r, c);
    klab = token_label(g, w.wy, w.wx, r, c);
    const int64_t off = tok * rowstride + w.h * D;
    float x[8], y[8];
    unpack8(*reinterpret_cast<const uint4*>(k + off + 8 * h), x);
    unpack8(*reinterpret_cast<const uint4*>(k + off + 16 + 8 * h), y);
    rotate8(x, sn, cs, 0, M, r, 4 * h);
    rotate8(y, sn, cs, 1, M, c, 4 * h);
    kh0 = pack8_op(x, true);
    kh1 = pack8_op(y, true);
    kf0 = pack8_op(x, false);
    kf1 = pack8_op(y, false);
    if (any_big(x) || any_big(y)) atomicOr(&sFlag[0], 1u);
    v0 = *reinterpret_cast<const uint4*>(v + off + 8 * h);
    v1 = *reinterpret_cast<const uint4*>(v + off + 16 + 8 * h);
  }
  const bf16x8_t vb0 = as_bf16x8(v0), vb1 = as_bf16x8(v1);
  f32x16_t accv, acck;
#pragma unroll
  for (int e = 0; e < 16; ++e) accv[e] = acck[e] = 0.f;
  const uint32_t wave_labels = wave_or(valid ? (1u << klab) : 0u);
  const bool wave_single = __builtin_popcount(wave_labels) == 1;
  bool all16 = true;

  for (int c0 = 0, ci = 0; c0 < NP; c0 += CH, ++ci) {
    __syncthreads();
    const bool kbig = sFlag[0] != 0;
    stage_rotated(q, g, w, c0, CH, sn, cs, qscale, !kbig, sQ, sQt, tst, &sFlag[1 + ci], tid, NT);
    stage_plain(dout, g, w, c0, CH, sG, sGt, tst, g_scale, !kbig, tid, NT);
    for (int n = tid; n < CH; n += NT) {
      const int qn = c0 + n;
      float l2 = 0.f, dl = 0.f;
      if (qn < N) {
        const int64_t t_ = token_index(g, w.b, w.wy, w.wx, qn / M, qn % M);
        l2 = lse[t_ * g.heads + w.h] * kLog2e;
        dl = delta[t_ * g.heads + w.h];
      }
      sL[n] = l2;
      sD[n] = dl;
    }
    chunk_labels(g, w, c0, CH, sLab, tid, NT);
    __syncthreads();
    block_info(sLab, CH, sBlk, tid, NT);
    const bool h16 = !kbig && sFlag[1 + ci] == 0;
    if (!h16 && !kbig) {
      stage_rotated(q, g, w, c0, CH, sn, cs, qscale, false, sQ, sQt, tst, nullptr, tid, NT);
      stage_plain(dout, g, w, c0, CH, nullptr, sGt, tst, g_scale, false, tid, NT);
    }
    __syncthreads();
    all16 = all16 && h16;
    if (wave_labels == 0) continue;
    const int nblk = min(CH, NP - c0) / 32;
    if (h16)
      dkdv_chunk<true>(sQ, sG, sQt, sGt, sL, sD, sLab, sBlk, tst, nblk, col, h, wave_labels, wave_single, klab, kh0,
                       kh1, vb0, vb1, ds_scale, accv, acck);
    else
      dkdv_chunk<false>(sQ, sG, sQt, sGt, sL, sD, sLab, sBlk, tst, nblk, col, h, wave_labels, wave_single, klab, kf0,
                        kf1, vb0, vb1, ds_scale, accv, acck);
  }

  float t[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  if (valid) {
    const int64_t off = tok * rowstride + w.h * D;
    // dV = accv / g_scale: lane holds channels 8g + 4h + j of its key
    const float inv_g = 1.f / g_scale;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint2 o;
      o.x = pack2(accv[4 * gq] * inv_g, accv[4 * gq + 1] * inv_g);
      o.y = pack2(accv[4 * gq + 2] * inv_g, accv[4 * gq + 3] * inv_g);
      *reinterpret_cast<uint2*>(dv + off + 8 * gq + 4 * h) = o;
    }
    // dk~ = acck * ln 2 / ds_scale (the Q operand carried log2(e) / sqrt(d))
    unrotate_store(acck, kLn2 / ds_scale, 1.0f, all16, k + off, dk + off, sn, cs, M, r, c, h, t);
  }
  const int64_t prow = ((int64_t)w.h * 2 + 0) * (g.B * g.nH * g.nW * nb) + wh / g.heads * nb + kblock;
  reduce_dtheta<NW>(t, red, partials + prow * 16, lane, wave, tid);
}

size_t dq_smem(int NP, int M) {
  const int CH = chunk_len(NP);
  return (size_t)CH * kKStride * 2 * 2 + (size_t)32 * vt_stride(CH) * 2 + table_bytes(M) + kNW * 16 * 4 +
         (kCh / 32) * 4 + (1 + kMaxChunks) * 4 + kCh;
}
size_t dkdv_smem(int NP, int M) {
  const int CH = chunk_len(NP);
  return (size_t)CH * kKStride * 2 * 2 + (size_t)32 * vt_stride(CH) * 2 * 2 + kCh * 4 * 2 + table_bytes(M) +
         kNW * 16 * 4 + (kCh / 32) * 4 + (1 + kMaxChunks) * 4 + kCh;
}

}  // namespace

int64_t bwd_mfma_partials(const Geom& g) {
  const int64_t nb = (g.N + kNW * 32 - 1) / (kNW * 32);
  return (int64_t)g.heads * 2 * g.B * g.nH * g.nW * nb;
}

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  hipLaunchKernelGGL(bwd_pre_kernel, dim3((unsigned)nwh), dim3(256), 0, st, (const uint16_t*)a.out,
                     (const uint16_t*)a.dout, (const uint16_t*)a.v, a.delta, a.scal, g);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int NP = (g.N + 31) / 32 * 32;
  const int nb = (g.N + kNW * 32 - 1) / (kNW * 32);
  const int64_t blocks = nwh * nb;
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute((const void*)bwd_dq_mfma_kernel<kNW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
    (void)hipFuncSetAttribute((const void*)bwd_dkdv_mfma_kernel<kNW>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
  });
  hipLaunchKernelGGL(bwd_dkdv_mfma_kernel<kNW>, dim3((unsigned)blocks), dim3(kNW * 64), dkdv_smem(NP, g.M), st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                     a.lse, a.delta, a.scal, a.th_row, a.th_col, (uint16_t*)a.dk, (uint16_t*)a.dv, a.partials, g, nb,
                     NP);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(bwd_dq_mfma_kernel<kNW>, dim3((unsigned)blocks), dim3(kNW * 64), dq_smem(NP, g.M), st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                     a.lse, a.delta, a.scal, a.th_row, a.th_col, (uint16_t*)a.dq, a.partials, g, nb, NP);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows_per_head = 2 * g.B * g.nH * g.nW * nb;
  return launch_dtheta_reduce(a.partials, a.n_partials, rows_per_head, g, a.dth_row, a.dth_col, st);
}

}  // namespace fsw
