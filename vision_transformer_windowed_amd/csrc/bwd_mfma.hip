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
// Kernels, all deterministic (no atomics on results):
//  * prologue, one workgroup per window-head: Delta = rowsum(dO * O) per token and the window's
//    largest |dO|, |v|, |q|, |k| components, which fix the operand format and power-of-two scales;
//  * dK/dV, key-stationary: a wave owns 32 keys (lane = key); queries stream through LDS in
//    chunks.  S = Q^ K~^T and tau (dP - Delta) = dO (tau V)^T start from -LSE / -tau Delta tiles
//    read from LDS, so P = exp2(S) and tau dS = P * (tau dP') cost one exp and one multiply per
//    score; dV^T += (g dO)^T P and dK~^T += Q^T (tau dS), with the Q^T and dO^T operands read
//    transposed from row-major LDS (ds_read_b64_tr_b16);
//  * dQ, query-stationary: a wave owns 32 queries (lane = query); keys stream through LDS.
//    S^T = K~ Q^T and tau dP'^T = V (tau dO)^T start from the lane's -LSE and -tau Delta;
//    dQ~^T += K~^T (tau dS)^T.
// Operand precision: dP = dO V^T multiplies bf16 inputs exactly (tau is a power of two).  The
// derived operands (rotated Q^ and K~, P, tau dS, g dO) go to fp16 MFMAs, 8x finer than bf16, when
// the prologue's maxima put every one of them in fp16 range (|tau dS| <= 2^14 by construction:
// |dS| <= |dO . v| + |Delta| <= 64 max|dO| max|v|); otherwise the window uses bf16 operands.
// Each workgroup reduces its dtheta terms in a fixed order into one partials row; a last kernel
// sums the rows in a fixed order.
#include <algorithm>
#include <mutex>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"
#include "fsw_stream.h"

namespace fsw {

namespace {

constexpr float kSqrt2 = 1.4142135623730951f;
constexpr float kQScale = kLog2e * 0.17677669529663687f;  // log2(e) / sqrt(32)

// Power of two 2^k (k clamped to [-100, 100]) with 2^k * bound <= 2^14 (1 when bound is 0 or not
// finite).
__device__ __forceinline__ float pow2_scale(float bound) {
  if (!(bound > 0.f) || !(bound < INFINITY)) return 1.f;
  int e;
  frexpf(bound, &e);  // bound < 2^e
  return ldexpf(1.f, min(100, max(-100, 14 - e)));
}

// Operand format of a window-head: fp16 when every rotated, scaled score operand is in range.
__device__ __forceinline__ bool window_h16(const float* scal, int64_t wh) {
  return kSqrt2 * scal[wh * 4 + 2] * kQScale < kF16Limit && kSqrt2 * scal[wh * 4 + 3] < kF16Limit;
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

// One workgroup per window and group of up to kPreHeads heads: Delta for every token and head, and
// scal[wh] = {max |dO|, max |v|, max |q|, max |k|} over each window-head's components.  The heads of
// a token sit side by side in one row, so the group's slice of every token row is read whole and
// each fetched line is used in full.  A thread keeps one 8-channel part p of the slice (head p / 4)
// for every token it handles, so its maxima belong to one head; kPreBatch tokens per step have
// their 5 x 16-byte loads issued together.  The work per 16 bytes is kept to a few packed
// instructions (dot products of bf16 pairs, 16-bit integer maxima), and the loads bypass the caches;
// the kernel runs at the HBM rate of a plain copy.
constexpr int kPreThreads = 256;
constexpr int kPreBatch = 4;
constexpr int kPreHeads = 16;
// Off is the type of byte offsets into the tensors: uint32_t when every offset fits (the host checks),
// which keeps the per-item address arithmetic to a few 32-bit instructions.
template <typename Off, bool STATS>
__global__ __launch_bounds__(kPreThreads) void bwd_pre_kernel(const uint16_t* __restrict__ out,
                                                              const uint16_t* __restrict__ dout,
                                                              const uint16_t* __restrict__ v,
                                                              const uint16_t* __restrict__ q,
                                                              const uint16_t* __restrict__ k,
                                                              float* __restrict__ delta, float* __restrict__ scal,
                                                              const float* __restrict__ stats, Geom g) {
  // STATS: the forward's per-window-head maxima of q, k and v (stats[wh] = {max |q| of a first and of
  // a second workgroup's queries, max |k|, max |v|}) stand in for those rows, and only O and dO are
  // read, twice as many tokens per batch.
  constexpr int kBatch = STATS ? 2 * kPreBatch : kPreBatch;
  __shared__ float red[4][kPreThreads];
  const int groups = (g.heads + kPreHeads - 1) / kPreHeads;
  const int64_t blk = xcd_order(blockIdx.x, gridDim.x);
  const int64_t win = blk / groups;
  const int h0 = (int)(blk - win * groups) * kPreHeads;
  const int hc = min(kPreHeads, g.heads - h0);
  const int wx = (int)(win % g.nW);
  const int wy = (int)((win / g.nW) % g.nH);
  const int64_t b = win / g.nW / g.nH;
  const int P = 4 * hc, T = kPreThreads / P;  // parts per token slice, tokens per pass
  const int tid = threadIdx.x;
  const bool act = tid < P * T;  // P * T is a multiple of 4: the 4 parts of a head stay together
  const int p = tid % P, t0 = tid / P;
  // byte strides of a token and the byte offset of the thread's part within the token row
  const Off os2 = (Off)(2 * g.os), xs2 = (Off)(2 * g.xs), ch2 = (Off)(2 * (h0 * 32 + p * 8));
  const Off img = (Off)(b * g.Hg);  // first grid row of the image
  const char* const po = reinterpret_cast<const char*>(out);
  const char* const pd = reinterpret_cast<const char*>(dout);
  const char* const pv = reinterpret_cast<const char*>(v);
  const char* const pq = reinterpret_cast<const char*>(q);
  const char* const pk = reinterpret_cast<const char*>(k);
  // the thread's tokens are t0, t0 + T, ...: window (row, column) advanced by (dr, dc) per token
  const int dr = T / g.M, dc = T - dr * g.M;
  int r = t0 / g.M, c = t0 - (t0 / g.M) * g.M;
  uint32_t am[4] = {0u, 0u, 0u, 0u};
  const int steps = (g.N + T * kBatch - 1) / (T * kBatch);
  for (int st = 0; st < steps; ++st) {  // uniform trip count: the shuffles below see every lane
    uint4 ro[kBatch], rd[kBatch], rv[STATS ? 1 : kBatch], rq[STATS ? 1 : kBatch], rk[STATS ? 1 : kBatch];
    Off tok[kBatch];
    bool ok[kBatch];
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const int n = (st * kBatch + u) * T + t0;
      const bool in = act && n < g.N;
      // Positions wrap at the padded extents.  An item past the end reads the window's first slot
      // again, and a padding position (or a padding first slot) reads the image's last row or column
      // instead: the maxima can only grow, which keeps every operand in range, and no Delta is stored
      // for either.
      const int yp = grid_coord(wy * g.M + (in ? r : 0), g.shift, g.Hp);
      const int xp = grid_coord(wx * g.M + (in ? c : 0), g.shift, g.Wp);
      ok[u] = in && yp < g.Hg && xp < g.Wg;
      const int y = min(yp, g.Hg - 1), x = min(xp, g.Wg - 1);
      tok[u] = (img + (Off)y) * (Off)g.Wg + (Off)x;
      const Off oo = tok[u] * os2 + ch2;
      ro[u] = load_stream(po + oo);
      rd[u] = load_stream(pd + oo);
      if constexpr (!STATS) {
        const Off xo = tok[u] * xs2 + ch2;
        rv[u] = load_stream(pv + xo);
        rq[u] = load_stream(pq + xo);
        rk[u] = load_stream(pk + xo);
      }
      c += dc;
      r += dr;
      if (c >= g.M) {
        c -= g.M;
        ++r;
      }
    }
#pragma unroll
    for (int u = 0; u < kBatch; ++u) {
      const uint32_t wo[4] = {ro[u].x, ro[u].y, ro[u].z, ro[u].w}, wd[4] = {rd[u].x, rd[u].y, rd[u].z, rd[u].w};
      float s = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        s = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, wo[e]), __builtin_bit_cast(bf16x2_t, wd[e]),
                                            s, false);
        am[0] = absmax_pair(am[0], wd[e]);
      }
      if constexpr (!STATS) {
        am[1] = absmax_x8(am[1], rv[u]);
        am[2] = absmax_x8(am[2], rq[u]);
        am[3] = absmax_x8(am[3], rk[u]);
      }
      // Delta of the token and head: its four 8-channel parts sit in four consecutive lanes
      s += __shfl_xor(s, 1, 64);
      s += __shfl_xor(s, 2, 64);
      if (ok[u] && (p & 3) == 0) delta[tok[u] * (Off)g.heads + (Off)(h0 + (p >> 2))] = s;
    }
  }
  constexpr int kRed = STATS ? 1 : 4;  // quantities reduced here
#pragma unroll
  for (int i = 0; i < kRed; ++i) red[i][tid] = absmax_value(am[i]);
  __syncthreads();
  if (tid < P) {  // one thread per (head, quantity): the maximum over its head's parts and tokens
    const int i = tid & 3, hh = tid >> 2;
    const int64_t wh = win * g.heads + h0 + hh;
    float m = 0.f;
    if (STATS && i > 0) {
      const float* s4 = stats + wh * 4;
      m = i == 1 ? s4[3] : i == 2 ? fmaxf(s4[0], s4[1]) : s4[2];
    } else {
      for (int t = 0; t < T; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) m = fmaxf(m, red[i][t * P + hh * 4 + j]);
    }
    scal[wh * 4 + i] = m;
  }
}

// Both main kernels stream the window's other side through LDS in chunks of up to chunk_max(MT)
// tokens:
//   load (global -> registers, chunk c + 1)  |  compute on chunk c from LDS
//   barrier; registers -> LDS (RoPE, scaling, operand format); barrier
// Block summaries (which labels a 32-token block holds) are double-buffered, so the buffer that
// the next chunk's stores OR into was cleared during the previous chunk's stores.
// Tile rows use the swizzled 64-byte layout (srow), so row and transposed operand reads are free
// of LDS bank conflicts, and every operand address is a per-lane base plus a constant.

// ---------------------------------------------------------------------------------------- dQ

struct DqSmem {
  uint16_t* K;    // [CH] swizzled rows: rotated K~ (operand format)
  uint16_t* V;    // [CH] swizzled rows: bf16 V
  float* sn;
  float* cs;
  float* red;     // [NW * 16]
  uint32_t* blk;  // [2][chunk / 32]
  uint8_t* lab;   // [chunk]
};
template <int NW>
__host__ __device__ inline size_t dq_smem(int NP, int M, int cmax) {
  const int CH = chunk_len(NP, cmax);
  return (size_t)CH * 32 * 2 * 2 + (size_t)2 * 2 * M * 8 * 4 + NW * 16 * 4 + 2 * (cmax / 32) * 4 + cmax;
}

// Each wave owns S sets of 32 queries (lane = query within a set).  The sets share every LDS
// operand read (K~ and V rows, the transposed K~^T), so staging and LDS traffic per tile shrink
// with S, and the S independent tiles give the scheduler work to interleave.
template <int NW, int MT, int S, bool H16, bool PAD>
__device__ inline void dq_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                               const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                               const float* __restrict__ lse, const float* __restrict__ delta,
                               const float* __restrict__ scal, uint16_t* __restrict__ dq,
                               float* __restrict__ partials, const Geom& g, int nb, int NP, const DqSmem& sm,
                               const WinHead& w, int64_t wh, int qblock) {
  constexpr int D = 32;
  constexpr int KC = chunk_max(MT);
  constexpr int NT = NW * 64;
  constexpr int IPT = (KC * 4 + NT - 1) / NT;
  const int M = MT > 0 ? MT : g.M;
  const int N = M * M;
  const WinOrder wo = win_order(g, M, w.wy, w.wx);
  // padding tokens of a padded grid are neither loaded nor stored (PAD instances only)
  const bool gpad = PAD && (g.Hp != g.Hg || g.Wp != g.Wg);
  const int CH = chunk_len(NP, KC);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int64_t xs = g.xs;
  const float ds_scale = pow2_scale(64.f * scal[wh * 4] * scal[wh * 4 + 1]);

  uint4 ik[IPT], iv[IPT];
  // Branch-free, so that the loads go out in one batch: an item that is none (past the chunk or the
  // window, or padding) reads a grid token of the image, and its bit in iok stays clear.
  uint32_t iok = 0;
  auto load_chunk = [&](int c0) {
    iok = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + i * NT;
      const int kn = c0 + (it >> 2);
      int r_ = 0, c_ = 0;
      if (kn < N) slot_rc(wo, kn, r_, c_);
      const bool ok = it < CH * 4 && kn < N && (!gpad || token_real(g, w.wy, w.wx, r_, c_));
      iok |= ok ? 1u << i : 0u;
      const int64_t tok = ok ? token_index(g, w.b, w.wy, w.wx, r_, c_) : w.b * g.Hg * g.Wg;
      const int64_t off = tok * xs + w.h * D + (it & 3) * 8;
      ik[i] = *reinterpret_cast<const uint4*>(k + off);
      iv[i] = *reinterpret_cast<const uint4*>(v + off);
    }
  };
  // In a window split by the shift, chunks holding none of the labels of this workgroup's queries
  // are neither loaded, staged nor visited (each region band is one contiguous slot range).
  const bool split = wo.ra != M || wo.ca != M;  // one window per workgroup: uniform
  const int own0 = qblock * NW * 32 * S;
  const uint32_t own = split ? range_labels(g, w, wo, own0, min(N, own0 + NW * 32 * S)) : 0u;
  auto next_chunk = [&](int c) {
    if (split)
      while (c < NP && (range_labels(g, w, wo, c, c + CH) & own) == 0) c += CH;
    return c;
  };
  int c0 = next_chunk(0);
  if (c0 < NP) load_chunk(c0);

  // the lane's queries: Q^ operands, tau * dO as bf16 B operands, -LSE and -tau Delta.  The loads of
  // every set go out before any is used (branch-free: a lane without a query reads a grid token of the
  // image and zeroes it), so that their latencies overlap.
  const int qbase = (qblock * NW + wave) * 32 * S + col;
  uint4 qb0[S], qb1[S], gb0[S], gb1[S];
  f32x16_t cL[S], cD[S], acc[S];
  int qlab[S], qr[S], qc[S];
  bool qval[S];
  float ql[S], qd[S];
  uint32_t wl = 0;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const int qi = qbase + 32 * t;
    bool valid = qi < N;
    int r = 0, c = 0;
    if (valid) {
      slot_rc(wo, qi, r, c);
      valid = !gpad || token_real(g, w.wy, w.wx, r, c);  // a padding query is no query
    }
    qval[t] = valid;
    qr[t] = r;
    qc[t] = c;
    const int64_t tok = valid ? token_index(g, w.b, w.wy, w.wx, r, c) : w.b * g.Hg * g.Wg;
    const int64_t off = tok * xs + w.h * D, goff = tok * g.os + w.h * D;
    qb0[t] = *reinterpret_cast<const uint4*>(q + off + 8 * h);
    qb1[t] = *reinterpret_cast<const uint4*>(q + off + 16 + 8 * h);
    gb0[t] = *reinterpret_cast<const uint4*>(dout + goff + 8 * h);
    gb1[t] = *reinterpret_cast<const uint4*>(dout + goff + 16 + 8 * h);
    ql[t] = lse[tok * g.heads + w.h];
    qd[t] = delta[tok * g.heads + w.h];
  }
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const bool valid = qval[t];
    qlab[t] = valid ? token_label(g, w.wy, w.wx, qr[t], qc[t]) : 0xff;
    wl |= valid ? (1u << qlab[t]) : 0u;
    float lse2 = 0.f, del = 0.f;
    if (valid) {
      lse2 = ql[t] * kLog2e;
      del = qd[t] * ds_scale;
      qb0[t] = rotated_part<H16>(qb0[t], sm.sn, sm.cs, M, qr[t], qc[t], h, kQScale);
      qb1[t] = rotated_part<H16>(qb1[t], sm.sn, sm.cs, M, qr[t], qc[t], 2 + h, kQScale);
      gb0[t] = scaled_part<false>(gb0[t], ds_scale);
      gb1[t] = scaled_part<false>(gb1[t], ds_scale);
    } else {
      qb0[t] = qb1[t] = gb0[t] = gb1[t] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      cL[t][e] = -lse2;
      cD[t][e] = -del;
      acc[t][e] = 0.f;
    }
  }
  const uint32_t wave_labels = uniform(wave_or(wl));
  const bool wave_single = __builtin_popcount(wave_labels) == 1;
  int tlo, thi;
  srow_tr_offsets(lane, tlo, thi);
  const int ro0 = srow(col, h), ro1 = srow(col, 2 + h);

  int buf = 0;
  for (int cn; c0 < NP; c0 = cn, buf ^= 1) {
    cn = next_chunk(c0 + CH);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + i * NT;
      if (it < CH * 4) {
        const int n = it >> 2, part = it & 3, kn = c0 + n;
        const bool ok = (iok >> i) & 1u;  // padding and slots past the window stay zero
        uint4 kr = make_uint4(0, 0, 0, 0);
        if (ok) {
          int r_, c_;
          slot_rc(wo, kn, r_, c_);
          kr = rotated_part<H16>(ik[i], sm.sn, sm.cs, M, r_, c_, part, 1.f);
        }
        *reinterpret_cast<uint4*>(sm.K + srow(n, part)) = kr;
        *reinterpret_cast<uint4*>(sm.V + srow(n, part)) = ok ? iv[i] : make_uint4(0, 0, 0, 0);
        if (part == 0) sm.lab[n] = chunk_label<PAD>(g, w, wo, kn, sm.blk + buf * (KC / 32), n);
      }
    }
    if (tid < KC / 32) sm.blk[(buf ^ 1) * (KC / 32) + tid] = 0;
    __syncthreads();
    if (cn < NP) load_chunk(cn);
    if (wave_labels == 0) continue;
    uint32_t info4[KC / 32];
#pragma unroll
    for (int i = 0; i < KC / 128; ++i) {
      const uint4 bw = *reinterpret_cast<const uint4*>(sm.blk + buf * (KC / 32) + 4 * i);
      info4[4 * i] = uniform(bw.x);
      info4[4 * i + 1] = uniform(bw.y);
      info4[4 * i + 2] = uniform(bw.z);
      info4[4 * i + 3] = uniform(bw.w);
    }
    const int nblk = min(CH, NP - c0) >> 5;
#pragma unroll
    for (int kb = 0; kb < KC / 32; ++kb) {
      if (kb >= nblk) break;
      const uint32_t info = info4[kb];
      const uint32_t bl = info & 0x1ffu;
      if ((bl & wave_labels) == 0) continue;
      const bool need_mask = ((info >> 10) & 1u) || !wave_single || bl != wave_labels;
      const uint16_t* Kb = sm.K + kb * 1024;
      const uint16_t* Vb = sm.V + kb * 1024;
      const uint4 ka0 = *reinterpret_cast<const uint4*>(Kb + ro0);
      const uint4 ka1 = *reinterpret_cast<const uint4*>(Kb + ro1);
      const uint4 va0 = *reinterpret_cast<const uint4*>(Vb + ro0);
      const uint4 va1 = *reinterpret_cast<const uint4*>(Vb + ro1);
      // S^T = K~ Q^T from -LSE, tau (dP - Delta)^T = V (tau dO)^T from -tau Delta
      f32x16_t sc[S], dc[S];
#pragma unroll
      for (int t = 0; t < S; ++t) {
        sc[t] = mfma_op<H16>(ka1, qb1[t], mfma_op<H16>(ka0, qb0[t], cL[t]));
        dc[t] = mfma_op<false>(va1, gb1[t], mfma_op<false>(va0, gb0[t], cD[t]));
      }
      // tau dS^T = exp2(S^T) * tau (dP - Delta)^T, the float32 product rounded once to the operand format
      uint32_t pk[S][8];
#pragma unroll
      for (int t = 0; t < S; ++t) {
        float p[16];
        if (need_mask) {
          const uint32_t live = live_bits(sm.lab, kb, h, qlab[t]);
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] = ((live >> e) & 1u) ? __builtin_amdgcn_exp2f(sc[t][e]) : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(sc[t][e]);
        }
        if constexpr (H16) {
#pragma unroll
          for (int e = 0; e < 8; ++e) pk[t][e] = mul2h(p[2 * e], dc[t][2 * e], p[2 * e + 1], dc[t][2 * e + 1]);
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) pk[t][e] = pack2(p[2 * e] * dc[t][2 * e], p[2 * e + 1] * dc[t][2 * e + 1]);
        }
      }
      // dQ~^T += K~^T (tau dS)^T
      const uint4 kt0 = tr_operand_at(Kb, tlo, thi);
      const uint4 kt1 = tr_operand_at(Kb + 512, tlo, thi);
#pragma unroll
      for (int t = 0; t < S; ++t) {
        acc[t] = mfma_op<H16>(kt0, make_uint4(pk[t][0], pk[t][1], pk[t][2], pk[t][3]), acc[t]);
        acc[t] = mfma_op<H16>(kt1, make_uint4(pk[t][4], pk[t][5], pk[t][6], pk[t][7]), acc[t]);
      }
    }
  }

  float th[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const int qi = qbase + 32 * t;
    int r = 0, c = 0;
    if (qi < N) slot_rc(wo, qi, r, c);
    if (qi < N && (!gpad || token_real(g, w.wy, w.wx, r, c))) {
      const int64_t off = token_index(g, w.b, w.wy, w.wx, r, c) * xs + w.h * D;
      // dq~ = acc / tau / sqrt(d); the dtheta integrand takes q~ as the dK product saw it
      unrotate_store(acc[t], 0.17677669529663687f / ds_scale, kQScale, H16, q + off, dq + off, sm.sn, sm.cs, M, r, c,
                     h, th);
    }
  }
  const int64_t prow = ((int64_t)w.h * 2 + 1) * (g.B * g.nH * g.nW * nb) + wh / g.heads * nb + qblock;
  reduce_dtheta<NW>(th, sm.red, partials + prow * 16, lane, wave, tid);
}

template <int NW, int MT, int S, bool PAD>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dq_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dq, float* __restrict__ partials, Geom g, int nb, int NP) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int KC = chunk_max(MT);
  if constexpr (MT > 0) NP = (MT * MT + 31) / 32 * 32;  // compile-time chunk geometry
  const int M = MT > 0 ? MT : g.M;
  const int CH = chunk_len(NP, KC);
  DqSmem sm;
  sm.K = reinterpret_cast<uint16_t*>(smem_raw);
  sm.V = sm.K + CH * 32;
  sm.sn = reinterpret_cast<float*>(sm.V + CH * 32);
  sm.cs = sm.sn + 2 * M * 8;
  sm.red = sm.cs + 2 * M * 8;
  sm.blk = reinterpret_cast<uint32_t*>(sm.red + NW * 16);
  sm.lab = reinterpret_cast<uint8_t*>(sm.blk + 2 * (KC / 32));
  const int64_t lb = xcd_order(blockIdx.x, gridDim.x);
  const int64_t wh = lb / nb;
  const WinHead w = decode_winhead(g, wh);
  if (threadIdx.x < 2 * (KC / 32)) sm.blk[threadIdx.x] = 0;
  fill_table(sm.sn, sm.cs, th_row, th_col, w.h, M, threadIdx.x, NW * 64);
  __syncthreads();
  if (window_h16(scal, wh))
    dq_body<NW, MT, S, true, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, nb, NP, sm, w, wh, (int)(lb % nb));
  else
    dq_body<NW, MT, S, false, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, nb, NP, sm, w, wh, (int)(lb % nb));
}

// -------------------------------------------------------------------------------------- dK / dV

struct DkdvSmem {
  uint16_t* Q;    // [CH] swizzled rows: rotated, scaled Q^ (operand format)
  uint16_t* G;    // [CH] swizzled rows: bf16 dO
  uint16_t* Gs;   // [CH] swizzled rows: g * dO (operand format)
  float* L;       // [chunk] -LSE log2(e)
  float* Dl;      // [chunk] -tau Delta
  float* sn;
  float* cs;
  float* red;     // [NW * 16]
  uint32_t* blk;  // [2][chunk / 32]
  uint8_t* lab;   // [chunk]
};
template <int NW>
__host__ __device__ inline size_t dkdv_smem(int NP, int M, int cmax) {
  const int CH = chunk_len(NP, cmax);
  return (size_t)CH * 32 * 2 * 3 + cmax * 4 * 2 + (size_t)2 * 2 * M * 8 * 4 + NW * 16 * 4 + 2 * (cmax / 32) * 4 + cmax;
}

// Each wave owns S sets of 32 keys (lane = key within a set); the sets share the LDS reads of the
// query-side operands (Q^ and dO rows, -LSE and -tau Delta, the transposed Q^T and (g dO)^T).
template <int NW, int MT, int S, bool H16, bool PAD>
__device__ inline void dkdv_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                                 const float* __restrict__ lse, const float* __restrict__ delta,
                                 const float* __restrict__ scal, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                 float* __restrict__ partials, const Geom& g, int nb, int NP, const DkdvSmem& sm,
                                 const WinHead& w, int64_t wh, int kblock) {
  constexpr int D = 32;
  constexpr int KC = chunk_max(MT);
  constexpr int NT = NW * 64;
  constexpr int IPT = (KC * 4 + NT - 1) / NT;
  const int M = MT > 0 ? MT : g.M;
  const int N = M * M;
  const WinOrder wo = win_order(g, M, w.wy, w.wx);
  // padding tokens of a padded grid are neither loaded nor stored (PAD instances only)
  const bool gpad = PAD && (g.Hp != g.Hg || g.Wp != g.Wg);
  const int CH = chunk_len(NP, KC);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const int64_t xs = g.xs;
  const float g_scale = pow2_scale(scal[wh * 4]);                              // dO of the dV product
  const float ds_scale = pow2_scale(64.f * scal[wh * 4] * scal[wh * 4 + 1]);  // dS of the dK product

  uint4 iq[IPT], ig[IPT];
  float il[IPT], id[IPT];
  // Branch-free, so that the loads go out in one batch: an item that is none (past the chunk or the
  // window, or padding) reads a grid token of the image, and its bit in iok stays clear; LSE and Delta
  // are read by every part and kept by part 0.
  uint32_t iok = 0;
  auto load_chunk = [&](int c0) {
    iok = 0;
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + i * NT;
      const int qn = c0 + (it >> 2);
      int r_ = 0, c_ = 0;
      if (qn < N) slot_rc(wo, qn, r_, c_);
      const bool ok = it < CH * 4 && qn < N && (!gpad || token_real(g, w.wy, w.wx, r_, c_));
      iok |= ok ? 1u << i : 0u;
      const int64_t t_ = ok ? token_index(g, w.b, w.wy, w.wx, r_, c_) : w.b * g.Hg * g.Wg;
      iq[i] = *reinterpret_cast<const uint4*>(q + t_ * xs + w.h * D + (it & 3) * 8);
      ig[i] = *reinterpret_cast<const uint4*>(dout + t_ * g.os + w.h * D + (it & 3) * 8);
      il[i] = lse[t_ * g.heads + w.h];
      id[i] = delta[t_ * g.heads + w.h];
    }
  };
  // In a window split by the shift, chunks holding none of the labels of this workgroup's keys are
  // neither loaded, staged nor visited (each region band is one contiguous slot range).
  const bool split = wo.ra != M || wo.ca != M;  // one window per workgroup: uniform
  const int own0 = kblock * NW * 32 * S;
  const uint32_t own = split ? range_labels(g, w, wo, own0, min(N, own0 + NW * 32 * S)) : 0u;
  auto next_chunk = [&](int c) {
    if (split)
      while (c < NP && (range_labels(g, w, wo, c, c + CH) & own) == 0) c += CH;
    return c;
  };
  int c0 = next_chunk(0);
  if (c0 < NP) load_chunk(c0);

  // the lane's keys (one per set): K~ operands, tau * V as bf16 B operands.  The loads of every set
  // go out before any is used (branch-free: a lane without a key reads a grid token of the image and
  // zeroes it), so that their latencies overlap.
  const int kbase = (kblock * NW + wave) * 32 * S + col;
  uint4 kb0[S], kb1[S], vb0[S], vb1[S];
  f32x16_t accv[S], acck[S];
  int klab[S], kr[S], kc[S];
  bool kval[S];
  uint32_t wl = 0;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const int kj = kbase + 32 * t;
    bool valid = kj < N;
    int r = 0, c = 0;
    if (valid) {
      slot_rc(wo, kj, r, c);
      valid = !gpad || token_real(g, w.wy, w.wx, r, c);  // a padding key is no key
    }
    kval[t] = valid;
    kr[t] = r;
    kc[t] = c;
    const int64_t off = (valid ? token_index(g, w.b, w.wy, w.wx, r, c) : w.b * g.Hg * g.Wg) * xs + w.h * D;
    kb0[t] = *reinterpret_cast<const uint4*>(k + off + 8 * h);
    kb1[t] = *reinterpret_cast<const uint4*>(k + off + 16 + 8 * h);
    vb0[t] = *reinterpret_cast<const uint4*>(v + off + 8 * h);
    vb1[t] = *reinterpret_cast<const uint4*>(v + off + 16 + 8 * h);
  }
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const bool valid = kval[t];
    klab[t] = valid ? token_label(g, w.wy, w.wx, kr[t], kc[t]) : 0xff;
    wl |= valid ? (1u << klab[t]) : 0u;
    if (valid) {
      kb0[t] = rotated_part<H16>(kb0[t], sm.sn, sm.cs, M, kr[t], kc[t], h, 1.f);
      kb1[t] = rotated_part<H16>(kb1[t], sm.sn, sm.cs, M, kr[t], kc[t], 2 + h, 1.f);
      vb0[t] = scaled_part<false>(vb0[t], ds_scale);
      vb1[t] = scaled_part<false>(vb1[t], ds_scale);
    } else {
      kb0[t] = kb1[t] = vb0[t] = vb1[t] = make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) accv[t][e] = acck[t][e] = 0.f;
  }
  const uint32_t wave_labels = uniform(wave_or(wl));
  const bool wave_single = __builtin_popcount(wave_labels) == 1;
  int tlo, thi;
  srow_tr_offsets(lane, tlo, thi);
  const int ro0 = srow(col, h), ro1 = srow(col, 2 + h);

  int buf = 0;
  for (int cn; c0 < NP; c0 = cn, buf ^= 1) {
    cn = next_chunk(c0 + CH);
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      const int it = tid + i * NT;
      if (it < CH * 4) {
        const int n = it >> 2, part = it & 3, qn = c0 + n;
        const bool ok = (iok >> i) & 1u;  // padding and slots past the window stay zero
        uint4 qr = make_uint4(0, 0, 0, 0);
        if (ok) {
          int r_, c_;
          slot_rc(wo, qn, r_, c_);
          qr = rotated_part<H16>(iq[i], sm.sn, sm.cs, M, r_, c_, part, kQScale);
        }
        const uint4 gr = ok ? ig[i] : make_uint4(0, 0, 0, 0);
        *reinterpret_cast<uint4*>(sm.Q + srow(n, part)) = qr;
        *reinterpret_cast<uint4*>(sm.G + srow(n, part)) = gr;
        *reinterpret_cast<uint4*>(sm.Gs + srow(n, part)) = scaled_part<H16>(gr, g_scale);
        if (part == 0) {
          sm.L[n] = ok ? -il[i] * kLog2e : 0.f;
          sm.Dl[n] = ok ? -id[i] * ds_scale : 0.f;
          sm.lab[n] = chunk_label<PAD>(g, w, wo, qn, sm.blk + buf * (KC / 32), n);
        }
      }
    }
    if (tid < KC / 32) sm.blk[(buf ^ 1) * (KC / 32) + tid] = 0;
    __syncthreads();
    if (cn < NP) load_chunk(cn);
    if (wave_labels == 0) continue;
    uint32_t info4[KC / 32];
#pragma unroll
    for (int i = 0; i < KC / 128; ++i) {
      const uint4 bw = *reinterpret_cast<const uint4*>(sm.blk + buf * (KC / 32) + 4 * i);
      info4[4 * i] = uniform(bw.x);
      info4[4 * i + 1] = uniform(bw.y);
      info4[4 * i + 2] = uniform(bw.z);
      info4[4 * i + 3] = uniform(bw.w);
    }
    const int nblk = min(CH, NP - c0) >> 5;
#pragma unroll
    for (int qb = 0; qb < KC / 32; ++qb) {
      if (qb >= nblk) break;
      const uint32_t info = info4[qb];
      const uint32_t bl = info & 0x1ffu;
      if ((bl & wave_labels) == 0) continue;
      const bool need_mask = ((info >> 10) & 1u) || !wave_single || bl != wave_labels;
      const uint16_t* Qb = sm.Q + qb * 1024;
      const uint16_t* Gb = sm.G + qb * 1024;
      // -LSE and -tau Delta of the 16 query rows this lane's accumulators hold: 8g + 4h + j
      f32x16_t cL, cD;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        const float4 l4 = *reinterpret_cast<const float4*>(sm.L + qb * 32 + 8 * gq + 4 * h);
        const float4 d4 = *reinterpret_cast<const float4*>(sm.Dl + qb * 32 + 8 * gq + 4 * h);
        cL[4 * gq] = l4.x;
        cL[4 * gq + 1] = l4.y;
        cL[4 * gq + 2] = l4.z;
        cL[4 * gq + 3] = l4.w;
        cD[4 * gq] = d4.x;
        cD[4 * gq + 1] = d4.y;
        cD[4 * gq + 2] = d4.z;
        cD[4 * gq + 3] = d4.w;
      }
      const uint4 qa0 = *reinterpret_cast<const uint4*>(Qb + ro0);
      const uint4 qa1 = *reinterpret_cast<const uint4*>(Qb + ro1);
      const uint4 ga0 = *reinterpret_cast<const uint4*>(Gb + ro0);
      const uint4 ga1 = *reinterpret_cast<const uint4*>(Gb + ro1);
      // S = Q^ K~^T from -LSE, tau (dP - Delta) = dO (tau V)^T from -tau Delta
      f32x16_t sc[S], dc[S];
#pragma unroll
      for (int t = 0; t < S; ++t) {
        sc[t] = mfma_op<H16>(qa1, kb1[t], mfma_op<H16>(qa0, kb0[t], cL));
        dc[t] = mfma_op<false>(ga1, vb1[t], mfma_op<false>(ga0, vb0[t], cD));
      }
      // P = exp2(S), tau dS = P * tau (dP - Delta)
      uint32_t pp[S][8], pd[S][8];
#pragma unroll
      for (int t = 0; t < S; ++t) {
        float p[16];
        if (need_mask) {
          const uint32_t live = live_bits(sm.lab, qb, h, klab[t]);
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] = ((live >> e) & 1u) ? __builtin_amdgcn_exp2f(sc[t][e]) : 0.f;
        } else {
#pragma unroll
          for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(sc[t][e]);
        }
        if constexpr (H16) {
          // tau dS as a packed fp16 product of the fp16 P and tau (dP - Delta)
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pp[t][e] = pack2h(p[2 * e], p[2 * e + 1]);
            const f16x2_t a = __builtin_bit_cast(f16x2_t, pp[t][e]);
            const f16x2_t b = __builtin_bit_cast(f16x2_t, pack2h(dc[t][2 * e], dc[t][2 * e + 1]));
            pd[t][e] = __builtin_bit_cast(uint32_t, a * b);
          }
        } else {
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            pp[t][e] = pack2(p[2 * e], p[2 * e + 1]);
            pd[t][e] = pack2(p[2 * e] * dc[t][2 * e], p[2 * e + 1] * dc[t][2 * e + 1]);
          }
        }
      }
      // dV^T += (g dO)^T P, dK~^T += Q^T (tau dS)
      const uint16_t* Gsb = sm.Gs + qb * 1024;
      const uint4 gt0 = tr_operand_at(Gsb, tlo, thi);
      const uint4 gt1 = tr_operand_at(Gsb + 512, tlo, thi);
#pragma unroll
      for (int t = 0; t < S; ++t) {
        accv[t] = mfma_op<H16>(gt0, make_uint4(pp[t][0], pp[t][1], pp[t][2], pp[t][3]), accv[t]);
        accv[t] = mfma_op<H16>(gt1, make_uint4(pp[t][4], pp[t][5], pp[t][6], pp[t][7]), accv[t]);
      }
      const uint4 qt0 = tr_operand_at(Qb, tlo, thi);
      const uint4 qt1 = tr_operand_at(Qb + 512, tlo, thi);
#pragma unroll
      for (int t = 0; t < S; ++t) {
        acck[t] = mfma_op<H16>(qt0, make_uint4(pd[t][0], pd[t][1], pd[t][2], pd[t][3]), acck[t]);
        acck[t] = mfma_op<H16>(qt1, make_uint4(pd[t][4], pd[t][5], pd[t][6], pd[t][7]), acck[t]);
      }
    }
  }

  float th[8] = {0, 0, 0, 0, 0, 0, 0, 0};
  const float inv_g = 1.f / g_scale;
#pragma unroll
  for (int t = 0; t < S; ++t) {
    const int kj = kbase + 32 * t;
    int r = 0, c = 0;
    if (kj < N) slot_rc(wo, kj, r, c);
    if (kj < N && (!gpad || token_real(g, w.wy, w.wx, r, c))) {
      const int64_t off = token_index(g, w.b, w.wy, w.wx, r, c) * xs + w.h * D;
      // dV = accv / g: lane holds channels 8g + 4h + j of its key
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint2 o;
        o.x = pack2(accv[t][4 * gq] * inv_g, accv[t][4 * gq + 1] * inv_g);
        o.y = pack2(accv[t][4 * gq + 2] * inv_g, accv[t][4 * gq + 3] * inv_g);
        *reinterpret_cast<uint2*>(dv + off + 8 * gq + 4 * h) = o;
      }
      // dk~ = acck * ln 2 / tau (the Q operand carried log2(e) / sqrt(d))
      unrotate_store(acck[t], kLn2 / ds_scale, 1.0f, H16, k + off, dk + off, sm.sn, sm.cs, M, r, c, h, th);
    }
  }
  const int64_t prow = ((int64_t)w.h * 2 + 0) * (g.B * g.nH * g.nW * nb) + wh / g.heads * nb + kblock;
  reduce_dtheta<NW>(th, sm.red, partials + prow * 16, lane, wave, tid);
}

template <int NW, int MT, int S, bool PAD>
__global__ __launch_bounds__(NW * 64, 2) void bwd_dkdv_mfma_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ partials, Geom g, int nb, int NP) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int KC = chunk_max(MT);
  if constexpr (MT > 0) NP = (MT * MT + 31) / 32 * 32;  // compile-time chunk geometry
  const int M = MT > 0 ? MT : g.M;
  const int CH = chunk_len(NP, KC);
  DkdvSmem sm;
  sm.Q = reinterpret_cast<uint16_t*>(smem_raw);
  sm.G = sm.Q + CH * 32;
  sm.Gs = sm.G + CH * 32;
  sm.L = reinterpret_cast<float*>(sm.Gs + CH * 32);
  sm.Dl = sm.L + KC;
  sm.sn = sm.Dl + KC;
  sm.cs = sm.sn + 2 * M * 8;
  sm.red = sm.cs + 2 * M * 8;
  sm.blk = reinterpret_cast<uint32_t*>(sm.red + NW * 16);
  sm.lab = reinterpret_cast<uint8_t*>(sm.blk + 2 * (KC / 32));
  const int64_t lb = xcd_order(blockIdx.x, gridDim.x);
  const int64_t wh = lb / nb;
  const WinHead w = decode_winhead(g, wh);
  if (threadIdx.x < 2 * (KC / 32)) sm.blk[threadIdx.x] = 0;
  fill_table(sm.sn, sm.cs, th_row, th_col, w.h, M, threadIdx.x, NW * 64);
  __syncthreads();
  if (window_h16(scal, wh))
    dkdv_body<NW, MT, S, true, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, nb, NP, sm, w, wh,
                               (int)(lb % nb));
  else
    dkdv_body<NW, MT, S, false, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, nb, NP, sm, w, wh,
                                (int)(lb % nb));
}

// Waves per workgroup and 32-token sets per wave for N tokens per window; the workgroups of a
// window-head each cover waves * sets * 32 tokens of the stationary side.
struct MainShape {
  int waves, sets;
};
MainShape main_shape(int N) {
  if (N > 256) return {8, 2};
  if (N > 128) return {4, 2};
  return {N > 64 ? 4 : 2, 1};
}
// The shape the dispatch launches for a geometry.  The grid, the dtheta partial rows (and so the
// workspace size) all follow it; launch_main refuses a template shape that differs.
MainShape bwd_shape(const Geom& g) {
  if (g.M == 32 || g.M == 16) return {g.M == 32 ? 8 : 4, 2};
  if (g.M == 8) return {2, 1};
  return main_shape(g.N);
}
int64_t blocks_per_windowhead(const Geom& g) {
  const MainShape m = bwd_shape(g);
  return (g.N + m.waves * m.sets * 32 - 1) / (m.waves * m.sets * 32);
}

template <int NW, int MT, int S, bool PAD = false>
hipError_t launch_main(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  const int NP = (g.N + 31) / 32 * 32;
  const MainShape m = bwd_shape(g);
  if (m.waves != NW || m.sets != S) return hipErrorInvalidConfiguration;
  const int nb = (int)blocks_per_windowhead(g);
  const int64_t blocks = nwh * nb;
  hipLaunchKernelGGL((bwd_dkdv_mfma_kernel<NW, MT, S, PAD>), dim3((unsigned)blocks), dim3(NW * 64),
                     dkdv_smem<NW>(NP, g.M, chunk_max(MT)), st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.lse, a.delta, a.scal, a.th_row, a.th_col, (uint16_t*)a.dk,
                     (uint16_t*)a.dv, a.partials, g, nb, NP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_mfma_kernel<NW, MT, S, PAD>), dim3((unsigned)blocks), dim3(NW * 64), dq_smem<NW>(NP, g.M, chunk_max(MT)),
                     st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout,
                     a.lse, a.delta, a.scal, a.th_row, a.th_col, (uint16_t*)a.dq, a.partials, g, nb, NP);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t rows_per_head = 2 * g.B * g.nH * g.nW * nb;
  return launch_dtheta_reduce(a.partials, a.n_partials, rows_per_head, g, a.dth_row, a.dth_col, st);
}

}  // namespace

int64_t bwd_mfma_partials(const Geom& g) {
  return (int64_t)g.heads * 2 * g.B * g.nH * g.nW * blocks_per_windowhead(g);
}

hipError_t launch_bwd_pre32(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int64_t pre_blocks = g.B * g.nH * g.nW * ((g.heads + kPreHeads - 1) / kPreHeads);
  // every byte offset the pre-kernel forms is below 2 * tokens * max(xs, os)
  const bool off32 = (double)g.B * g.Hg * g.Wg * 2.0 * (double)std::max(g.xs, g.os) < 4294967296.0;
  auto* const kern = off32 ? (a.stats ? bwd_pre_kernel<uint32_t, true> : bwd_pre_kernel<uint32_t, false>)
                            : (a.stats ? bwd_pre_kernel<int64_t, true> : bwd_pre_kernel<int64_t, false>);
  hipLaunchKernelGGL(kern, dim3((unsigned)pre_blocks), dim3(kPreThreads), 0, st, (const uint16_t*)a.out,
                     (const uint16_t*)a.dout, (const uint16_t*)a.v, (const uint16_t*)a.q, (const uint16_t*)a.k, a.delta,
                     a.scal, a.stats, g);
  return hipGetLastError();
}

hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const hipError_t e = launch_bwd_pre32(a, st);
  if (e != hipSuccess) return e;
  const MainShape m = bwd_shape(g);
  if (g.Hp != g.Hg || g.Wp != g.Wg) {  // padded grid: the run-time-M instances with padding checks
    if (m.waves == 8) return launch_main<8, 0, 2, true>(a, st);
    if (m.waves == 4) return m.sets == 2 ? launch_main<4, 0, 2, true>(a, st) : launch_main<4, 0, 1, true>(a, st);
    return launch_main<2, 0, 1, true>(a, st);
  }
  if (g.M == 32) return launch_main<8, 32, 2>(a, st);
  if (g.M == 8) return launch_main<2, 8, 1>(a, st);
  if (g.M == 16) return launch_main<4, 16, 2>(a, st);
  if (m.waves == 8) return launch_main<8, 0, 2>(a, st);
  if (m.waves == 4) return m.sets == 2 ? launch_main<4, 0, 2>(a, st) : launch_main<4, 0, 1>(a, st);
  return launch_main<2, 0, 1>(a, st);
}

}  // namespace fsw
