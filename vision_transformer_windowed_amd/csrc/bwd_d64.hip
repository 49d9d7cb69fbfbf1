// bf16 window-attention backward on MFMA (gfx950) for d = 64 and windows of up to 256 tokens (M <= 16).
//
// Backward of exact window attention with window-local 2D RoPE, recomputing P from the forward's
// log-sum-exp so that no score matrix is stored (FlashSwin paper card, "FLASHSWIN: Unlocking Large
// Windows and Dense Tokens in Swin Vision Transformers with Memory Efficient Attention": Abstract, flat
// training memory in the window size; Table S1).  In the log2 domain with q^ = q~ log2(e) / sqrt(d):
// P = exp2(q^ . k~ - LSE log2(e)), dS = P (dO . v - Delta), dq~ = sum_j dS k~ / sqrt(d),
// dk~ = sum_i dS q~ / sqrt(d), dv = sum_i P dO, dq = R^T dq~, dk = R^T dk~, and
// dtheta += p (dx~_b x~_a - dx~_a x~_b) over Q and K tokens.
//
// A window of at most 256 tokens of 64 channels fits LDS whole, so each kernel stages one side of a
// window-head once and walks it without chunking or per-chunk barriers:
//  * prologue, one workgroup per window-head: Delta = rowsum(dO * O) per token and the window-head's
//    largest |dO|, |v|, |q|, |k| components, which fix the operand format and power-of-two scales;
//  * dK/dV, key-stationary: a wave owns 32 keys (lane = key) held as B operands; the workgroup stages
//    the window's rotated, scaled queries Q^, dO and g dO in LDS (rows of 64 channels and 16 bytes of
//    pad), with -LSE and -tau Delta.  Per 32-query block: S = Q^ K~^T from -LSE and
//    tau (dP - Delta) = dO (tau V)^T from -tau Delta (4 MFMAs each), P = exp2(S),
//    tau dS = P * tau (dP - Delta), dV^T += (g dO)^T P and dK~^T += Q^T (tau dS) (2 output tiles of 32
//    channels, 4 MFMAs each, the transposed operands read by ds_read_b64_tr_b16);
//  * dQ, query-stationary: a wave owns 32 queries; the workgroup stages the rotated K~ and V.  Per
//    32-key block: S^T = K~ Q^T and tau dP'^T = V (tau dO)^T, dQ~^T += K~^T (tau dS)^T.
// Operand precision as in the d = 32 kernels: the derived operands (Q^, K~, P, tau dS, g dO) are fp16
// when the prologue's maxima put all of them in range, else bf16; dP = dO V^T multiplies bf16 inputs
// exactly.  Each workgroup reduces its dtheta terms in a fixed order into one partials row of 32
// floats; the shared reduce kernel sums the rows in a fixed order.
#include <algorithm>
#include <mutex>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"
#include "fsw_stream.h"

namespace fsw {

namespace {

constexpr int D6 = 64;
constexpr int kRS = D6 + 8;   // LDS row stride (elements): 144-byte rows, conflict-free row and transposed reads
constexpr int kMaxN6 = 256;   // largest window (tokens) these kernels serve
constexpr float kQScale6 = kLog2e * 0.125f;  // log2(e) / sqrt(64)
constexpr float kRoot2 = 1.4142135623730951f;

// Power of two 2^k (k clamped to [-100, 100]) with 2^k * bound <= 2^14 (1 when bound is 0 or not finite).
__device__ __forceinline__ float scale_to_2p14(float bound) {
  if (!(bound > 0.f) || !(bound < INFINITY)) return 1.f;
  int e;
  frexpf(bound, &e);  // bound < 2^e
  return ldexpf(1.f, min(100, max(-100, 14 - e)));
}

// fp16 score operands when every rotated, scaled component is in range (a rotation grows a component
// by at most sqrt(2)).
__device__ __forceinline__ bool h16_window(const float* scal, int64_t wh) {
  return kRoot2 * scal[wh * 4 + 2] * kQScale6 < kF16Limit && kRoot2 * scal[wh * 4 + 3] < kF16Limit;
}

// RoPE sin/cos table of one head, [2 axes][M positions][16 pairs].
__device__ inline void fill_table64(float* sn, float* cs, const float* th_row, const float* th_col, int head, int M,
                                    int tid, int nt) {
  for (int i = tid; i < 2 * M * 16; i += nt) {
    const int axis = i / (M * 16);
    const int p = (i / 16) % M;
    const int j = i % 16;
    const float th = axis ? th_col[head * 16 + j] : th_row[head * 16 + j];
    float s, c;
    rope_sincos(th, p, &s, &c);
    sn[i] = s;
    cs[i] = c;
  }
}

// Channels 8 part .. 8 part + 7 of token (r, c), rotated (parts 0..3: row axis, 4..7: column axis),
// scaled, packed to the operand format.
template <bool H16>
__device__ __forceinline__ uint4 rot_part64(uint4 raw, const float* sn, const float* cs, int M, int r, int c, int part,
                                            float scale) {
  float x[8];
  unpack8(raw, x);
  const int axis = part >> 2;
  rotate8(x, sn, cs, axis, M, axis ? c : r, (part & 3) * 4, 16);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= scale;
  return pack8_op(x, H16);
}

// Live mask of the lane's 16 accumulator rows 8g + 4h + j of 32-token block blk for label lab.
__device__ __forceinline__ uint32_t live16(const uint8_t* labs, int blk, int h, int lab) {
  uint32_t bits = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(labs + blk * 32 + 8 * g + 4 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (((w >> (8 * j)) & 0xff) == (uint32_t)lab) bits |= 1u << (4 * g + j);
  }
  return bits;
}

// Epilogue of the dK and dQ kernels for the lane's token: gradient w.r.t. the rotated vector in tile c
// (value v of acc[c]: channel 32c + 8(v/4) + 4h + v%4, times `scale`), recompute the rotated input as
// the products saw it (scaled by op_scale, rounded to the operand format, scaled back), accumulate the
// 16 dtheta slots of the lane (slot 8c + 2g + u: pair 4g + 2h + u of axis c), un-rotate, store bf16.
__device__ inline void unrotate_store64(const f32x16_t (&acc)[2], float scale, float op_scale, bool op16,
                                        const uint16_t* xsrc, uint16_t* dst, const float* sn, const float* cs, int M,
                                        int r, int c, int h, float (&t)[16]) {
  const float inv_op = 1.f / op_scale;
#pragma unroll
  for (int ct = 0; ct < 2; ++ct) {
    const int pos = ct ? c : r;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ch = 32 * ct + 8 * gq + 4 * h;
      const uint2 raw = *reinterpret_cast<const uint2*>(xsrc + ch);
      const float xin[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                            __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
      float res[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 4 * gq + 2 * h + u;  // pair within the axis
        const float s = sn[(ct * M + pos) * 16 + j];
        const float co = cs[(ct * M + pos) * 16 + j];
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
        const float da = acc[ct][4 * gq + 2 * u] * scale, db = acc[ct][4 * gq + 2 * u + 1] * scale;
        t[8 * ct + 2 * gq + u] += (float)pos * (db * at - da * bt);
        res[2 * u] = da * co + db * s;  // R^T (da, db)
        res[2 * u + 1] = -da * s + db * co;
      }
      uint2 o;
      o.x = pack2(res[0], res[1]);
      o.y = pack2(res[2], res[3]);
      *reinterpret_cast<uint2*>(dst + ch) = o;
    }
  }
}

// Fixed-order reduction of the lanes' 16 dtheta slots over the workgroup into one 32-float partials row
// (row-axis pairs 0..15, then column-axis pairs): a butterfly over the 32 lanes of each half-wave, then
// the waves in order.
template <int NW>
__device__ inline void reduce_dtheta64(float (&t)[16], float* red, float* dst, int lane, int wave, int tid) {
#pragma unroll
  for (int i = 0; i < 16; ++i) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) t[i] += __shfl_xor(t[i], o, 64);
  }
  if ((lane & 31) == 0) {
    const int h = lane >> 5;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq)
#pragma unroll
        for (int u = 0; u < 2; ++u) red[wave * 32 + 16 * ct + 4 * gq + 2 * h + u] = t[8 * ct + 2 * gq + u];
  }
  __syncthreads();
  if (tid < 32) {
    float s = 0.f;
    for (int i = 0; i < NW; ++i) s += red[i * 32 + tid];
    dst[tid] = s;
  }
}

// ------------------------------------------------------------------------------------ prologue

// One workgroup per window-head: Delta of its tokens and scal[wh] = {max |dO|, max |v|, max |q|, max |k|}.
// Thread: 16-byte part p = tid % 8 of tokens tid / 8, tid / 8 + 32, ...
__global__ __launch_bounds__(256) void bwd_pre64_kernel(const uint16_t* __restrict__ out,
                                                        const uint16_t* __restrict__ dout,
                                                        const uint16_t* __restrict__ v, const uint16_t* __restrict__ q,
                                                        const uint16_t* __restrict__ k, float* __restrict__ delta,
                                                        float* __restrict__ scal, Geom g) {
  __shared__ float red[4][4];
  const int64_t wh = xcd_order(blockIdx.x, gridDim.x);
  const WinHead w = decode_winhead(g, wh);
  const int tid = threadIdx.x, p = tid & 7;
  float mx[4] = {0.f, 0.f, 0.f, 0.f};
  for (int n0 = 0; n0 < g.N; n0 += 32) {  // uniform trip count: every lane reaches the shuffles
    const int n = n0 + (tid >> 3);
    const bool ok = n < g.N && token_real(g, w.wy, w.wx, n / g.M, n % g.M);
    float s = 0.f;
    int64_t tok = 0;
    if (ok) {
      tok = token_index(g, w.b, w.wy, w.wx, n / g.M, n % g.M);
      const int64_t xo = tok * g.xs + w.h * D6 + 8 * p, oo = tok * g.os + w.h * D6 + 8 * p;
      float o8[8], d8[8], v8[8], q8[8], k8[8];
      unpack8(*reinterpret_cast<const uint4*>(out + oo), o8);
      unpack8(*reinterpret_cast<const uint4*>(dout + oo), d8);
      unpack8(*reinterpret_cast<const uint4*>(v + xo), v8);
      unpack8(*reinterpret_cast<const uint4*>(q + xo), q8);
      unpack8(*reinterpret_cast<const uint4*>(k + xo), k8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        s = __builtin_fmaf(o8[e], d8[e], s);
        // a NaN component counts as infinity (fmaxf would drop it)
        mx[0] = fmaxf(mx[0], d8[e] != d8[e] ? INFINITY : fabsf(d8[e]));
        mx[1] = fmaxf(mx[1], v8[e] != v8[e] ? INFINITY : fabsf(v8[e]));
        mx[2] = fmaxf(mx[2], q8[e] != q8[e] ? INFINITY : fabsf(q8[e]));
        mx[3] = fmaxf(mx[3], k8[e] != k8[e] ? INFINITY : fabsf(k8[e]));
      }
    }
    s += __shfl_xor(s, 1, 64);
    s += __shfl_xor(s, 2, 64);
    s += __shfl_xor(s, 4, 64);
    if (ok && p == 0) delta[tok * g.heads + w.h] = s;
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = wave_max(mx[i]);
  if ((tid & 63) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[tid >> 6][i] = mx[i];
  }
  __syncthreads();
  if (tid < 4) scal[wh * 4 + tid] = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
}

// ---------------------------------------------------------------------------------------- dK / dV

// LDS of the dK/dV kernel for NP padded tokens.
struct KvSmem {
  uint16_t* Q;    // [NP][kRS] rotated, scaled Q^ (operand format)
  uint16_t* G;    // [NP][kRS] bf16 dO
  uint16_t* Gs;   // [NP][kRS] g dO (operand format)
  float* L;       // [NP] -LSE log2(e)
  float* Dl;      // [NP] -tau Delta
  float* sn;      // [2][M][16]
  float* cs;
  float* red;     // [NW][32]
  uint8_t* lab;   // [NP]
};
__host__ __device__ inline size_t kv_smem_bytes(int NP, int M, int NW) {
  return (size_t)NP * kRS * 2 * 3 + (size_t)NP * 4 * 2 + (size_t)2 * 2 * M * 16 * 4 + (size_t)NW * 32 * 4 + NP;
}

template <int NW, bool H16, bool PAD>
__device__ inline void dkdv64_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                   const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                                   const float* __restrict__ lse, const float* __restrict__ delta,
                                   const float* __restrict__ scal, uint16_t* __restrict__ dk,
                                   uint16_t* __restrict__ dv, float* __restrict__ partials, const Geom& g, int NP,
                                   const KvSmem& sm, const WinHead& w, int64_t wh, bool masked) {
  constexpr int NT = NW * 64;
  constexpr int IPT = kMaxN6 * 8 / NT;  // staged 16-byte items per thread, at most
  const int M = g.M, N = g.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const float g_scale = scale_to_2p14(scal[wh * 4]);                               // dO of the dV product
  const float ds_scale = scale_to_2p14(128.f * scal[wh * 4] * scal[wh * 4 + 1]);  // |tau dS| <= 2^14

  // 1. stage every query-side row of the window (item it: part it % 8 of token it / 8)
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int it = tid + i * NT;
    if (it >= NP * 8) break;  // uniform across a wave: NP * 8 is a multiple of 256
    const int n = it >> 3, part = it & 7;
    uint4 qo = make_uint4(0, 0, 0, 0), go = qo, gs = qo;
    float lv = 0.f, dl = 0.f;
    uint8_t lb = 0xff;
    if (n < N && (!PAD || token_real(g, w.wy, w.wx, n / M, n % M))) {  // padding stays zero, label 0xff
      const int r = n / M, c = n - (n / M) * M;
      const int64_t tok = token_index(g, w.b, w.wy, w.wx, r, c);
      const uint4 qr = *reinterpret_cast<const uint4*>(q + tok * g.xs + w.h * D6 + 8 * part);
      go = *reinterpret_cast<const uint4*>(dout + tok * g.os + w.h * D6 + 8 * part);
      qo = rot_part64<H16>(qr, sm.sn, sm.cs, M, r, c, part, kQScale6);
      gs = scaled_part<H16>(go, g_scale);
      if (part == 0) {
        lv = -lse[tok * g.heads + w.h] * kLog2e;
        dl = -delta[tok * g.heads + w.h] * ds_scale;
        lb = (uint8_t)token_label(g, w.wy, w.wx, r, c);
      }
    }
    *reinterpret_cast<uint4*>(sm.Q + n * kRS + 8 * part) = qo;
    *reinterpret_cast<uint4*>(sm.G + n * kRS + 8 * part) = go;
    *reinterpret_cast<uint4*>(sm.Gs + n * kRS + 8 * part) = gs;
    if (part == 0) {
      sm.L[n] = lv;
      sm.Dl[n] = dl;
      sm.lab[n] = lb;
    }
  }

  // 2. the lane's key: K~ operands (k-step t: channels 16t + 8h ..), tau V as bf16 B operands
  const int kj = wave * 32 + col;
  const bool kvalid = kj < N && (!PAD || token_real(g, w.wy, w.wx, kj / M, kj % M));  // a padding key is no key
  const int kr = kvalid ? kj / M : 0, kc = kvalid ? kj - (kj / M) * M : 0;
  int64_t koff = 0;
  uint4 kb[4], vb[4];
  int klab = 0xff;
#pragma unroll
  for (int t = 0; t < 4; ++t) kb[t] = vb[t] = make_uint4(0, 0, 0, 0);
  if (kvalid) {
    koff = token_index(g, w.b, w.wy, w.wx, kr, kc) * g.xs + w.h * D6;
    klab = token_label(g, w.wy, w.wx, kr, kc);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      kb[t] = rot_part64<H16>(*reinterpret_cast<const uint4*>(k + koff + 16 * t + 8 * h), sm.sn, sm.cs, M, kr, kc,
                              2 * t + h, 1.f);
      vb[t] = scaled_part<false>(*reinterpret_cast<const uint4*>(v + koff + 16 * t + 8 * h), ds_scale);
    }
  }
  f32x16_t accv[2], acck[2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) accv[ct][e] = acck[ct][e] = 0.f;
  __syncthreads();

  // 3. every 32-query block against the wave's 32 keys
  const int NB = NP >> 5;
  for (int qb = 0; qb < NB; ++qb) {
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
    // S = Q^ K~^T from -LSE, tau (dP - Delta) = dO (tau V)^T from -tau Delta
    const uint16_t* qrow = sm.Q + (qb * 32 + col) * kRS + 8 * h;
    const uint16_t* grow = sm.G + (qb * 32 + col) * kRS + 8 * h;
    f32x16_t sc = cL, dc = cD;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc = mfma_op<H16>(*reinterpret_cast<const uint4*>(qrow + 16 * t), kb[t], sc);
      dc = mfma_op<false>(*reinterpret_cast<const uint4*>(grow + 16 * t), vb[t], dc);
    }
    // P = exp2(S) (queries of other regions, or past the window, masked), tau dS = P * tau (dP - Delta)
    float p[16];
    const uint32_t live = masked ? live16(sm.lab, qb, h, klab) : 0xffffu;
#pragma unroll
    for (int e = 0; e < 16; ++e) p[e] = ((live >> e) & 1u) ? __builtin_amdgcn_exp2f(sc[e]) : 0.f;
    uint32_t pp[8], pd[8];
    if constexpr (H16) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pp[e] = pack2h(p[2 * e], p[2 * e + 1]);
        const f16x2_t a = __builtin_bit_cast(f16x2_t, pp[e]);
        const f16x2_t b = __builtin_bit_cast(f16x2_t, pack2h(dc[2 * e], dc[2 * e + 1]));
        pd[e] = __builtin_bit_cast(uint32_t, a * b);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        pp[e] = pack2(p[2 * e], p[2 * e + 1]);
        pd[e] = pack2(p[2 * e] * dc[2 * e], p[2 * e + 1] * dc[2 * e + 1]);
      }
    }
    // dV^T += (g dO)^T P and dK~^T += Q^T (tau dS), per 32-channel tile
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint4 gt0 = tr_operand(sm.Gs + 32 * ct, kRS, qb * 32, lane);
      const uint4 gt1 = tr_operand(sm.Gs + 32 * ct, kRS, qb * 32 + 16, lane);
      accv[ct] = mfma_op<H16>(gt0, make_uint4(pp[0], pp[1], pp[2], pp[3]), accv[ct]);
      accv[ct] = mfma_op<H16>(gt1, make_uint4(pp[4], pp[5], pp[6], pp[7]), accv[ct]);
      const uint4 qt0 = tr_operand(sm.Q + 32 * ct, kRS, qb * 32, lane);
      const uint4 qt1 = tr_operand(sm.Q + 32 * ct, kRS, qb * 32 + 16, lane);
      acck[ct] = mfma_op<H16>(qt0, make_uint4(pd[0], pd[1], pd[2], pd[3]), acck[ct]);
      acck[ct] = mfma_op<H16>(qt1, make_uint4(pd[4], pd[5], pd[6], pd[7]), acck[ct]);
    }
  }

  // 4. dV = accv / g; dk~ = acck ln 2 / tau (the Q^ operand carried log2(e) / sqrt(d)); dtheta terms
  float th[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) th[i] = 0.f;
  if (kvalid) {
    const float inv_g = 1.f / g_scale;
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint2 o;
        o.x = pack2(accv[ct][4 * gq] * inv_g, accv[ct][4 * gq + 1] * inv_g);
        o.y = pack2(accv[ct][4 * gq + 2] * inv_g, accv[ct][4 * gq + 3] * inv_g);
        *reinterpret_cast<uint2*>(dv + koff + 32 * ct + 8 * gq + 4 * h) = o;
      }
    unrotate_store64(acck, kLn2 / ds_scale, 1.f, H16, k + koff, dk + koff, sm.sn, sm.cs, M, kr, kc, h, th);
  }
  const int64_t nwin = g.B * g.nH * g.nW;
  reduce_dtheta64<NW>(th, sm.red, partials + (((int64_t)w.h * 2 + 0) * nwin + wh / g.heads) * 32, lane, wave, tid);
}

template <int NW, bool PAD>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv64_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ partials, Geom g, int NP) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  KvSmem sm;
  sm.Q = reinterpret_cast<uint16_t*>(smem_raw);
  sm.G = sm.Q + NP * kRS;
  sm.Gs = sm.G + NP * kRS;
  sm.L = reinterpret_cast<float*>(sm.Gs + NP * kRS);
  sm.Dl = sm.L + NP;
  sm.sn = sm.Dl + NP;
  sm.cs = sm.sn + 2 * g.M * 16;
  sm.red = sm.cs + 2 * g.M * 16;
  sm.lab = reinterpret_cast<uint8_t*>(sm.red + NW * 32);
  const int64_t wh = xcd_order(blockIdx.x, gridDim.x);
  const WinHead w = decode_winhead(g, wh);
  // Several Swin regions only in the last window row and column of a shifted grid.  Padding can sit
  // in the last two window rows or columns of a shifted padded grid: every window of a padded grid is
  // masked (a padding key must get P = 0 exactly, not exp2(0 - LSE)).
  const bool edge = w.wy == g.nH - 1 || w.wx == g.nW - 1;
  const bool masked = (g.shift > 0 && edge) || PAD || NP != g.N;
  fill_table64(sm.sn, sm.cs, th_row, th_col, w.h, g.M, threadIdx.x, NW * 64);
  __syncthreads();
  if (h16_window(scal, wh))
    dkdv64_body<NW, true, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, NP, sm, w, wh, masked);
  else
    dkdv64_body<NW, false, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, NP, sm, w, wh, masked);
}

// ---------------------------------------------------------------------------------------- dQ

struct QSmem {
  uint16_t* K;    // [NP][kRS] rotated K~ (operand format)
  uint16_t* V;    // [NP][kRS] bf16 V
  float* sn;
  float* cs;
  float* red;     // [NW][32]
  uint8_t* lab;   // [NP]
};
__host__ __device__ inline size_t q_smem_bytes(int NP, int M, int NW) {
  return (size_t)NP * kRS * 2 * 2 + (size_t)2 * 2 * M * 16 * 4 + (size_t)NW * 32 * 4 + NP;
}

template <int NW, bool H16, bool PAD>
__device__ inline void dq64_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                                 const float* __restrict__ lse, const float* __restrict__ delta,
                                 const float* __restrict__ scal, uint16_t* __restrict__ dq,
                                 float* __restrict__ partials, const Geom& g, int NP, const QSmem& sm,
                                 const WinHead& w, int64_t wh, bool masked) {
  constexpr int NT = NW * 64;
  constexpr int IPT = kMaxN6 * 8 / NT;
  const int M = g.M, N = g.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const float ds_scale = scale_to_2p14(128.f * scal[wh * 4] * scal[wh * 4 + 1]);

  // 1. stage the window's rotated K~ and V rows
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int it = tid + i * NT;
    if (it >= NP * 8) break;
    const int n = it >> 3, part = it & 7;
    uint4 ko = make_uint4(0, 0, 0, 0), vo = ko;
    uint8_t lb = 0xff;
    if (n < N && (!PAD || token_real(g, w.wy, w.wx, n / M, n % M))) {  // padding stays zero, label 0xff
      const int r = n / M, c = n - (n / M) * M;
      const int64_t off = token_index(g, w.b, w.wy, w.wx, r, c) * g.xs + w.h * D6 + 8 * part;
      ko = rot_part64<H16>(*reinterpret_cast<const uint4*>(k + off), sm.sn, sm.cs, M, r, c, part, 1.f);
      vo = *reinterpret_cast<const uint4*>(v + off);
      if (part == 0) lb = (uint8_t)token_label(g, w.wy, w.wx, r, c);
    }
    *reinterpret_cast<uint4*>(sm.K + n * kRS + 8 * part) = ko;
    *reinterpret_cast<uint4*>(sm.V + n * kRS + 8 * part) = vo;
    if (part == 0) sm.lab[n] = lb;
  }

  // 2. the lane's query: Q^ operands, tau dO as bf16 B operands, -LSE and -tau Delta
  const int qi = wave * 32 + col;
  const bool qvalid = qi < N && (!PAD || token_real(g, w.wy, w.wx, qi / M, qi % M));  // a padding query is no query
  const int qr = qvalid ? qi / M : 0, qc = qvalid ? qi - (qi / M) * M : 0;
  int64_t qoff = 0;
  uint4 qb[4], gb[4];
  int qlab = 0xff;
  float lse2 = 0.f, del = 0.f;
#pragma unroll
  for (int t = 0; t < 4; ++t) qb[t] = gb[t] = make_uint4(0, 0, 0, 0);
  if (qvalid) {
    const int64_t tok = token_index(g, w.b, w.wy, w.wx, qr, qc);
    qoff = tok * g.xs + w.h * D6;
    const int64_t goff = tok * g.os + w.h * D6;
    qlab = token_label(g, w.wy, w.wx, qr, qc);
    lse2 = lse[tok * g.heads + w.h] * kLog2e;
    del = delta[tok * g.heads + w.h] * ds_scale;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      qb[t] = rot_part64<H16>(*reinterpret_cast<const uint4*>(q + qoff + 16 * t + 8 * h), sm.sn, sm.cs, M, qr, qc,
                              2 * t + h, kQScale6);
      gb[t] = scaled_part<false>(*reinterpret_cast<const uint4*>(dout + goff + 16 * t + 8 * h), ds_scale);
    }
  }
  f32x16_t cL, cD, acc[2];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    cL[e] = -lse2;
    cD[e] = -del;
    acc[0][e] = acc[1][e] = 0.f;
  }
  __syncthreads();

  // 3. every 32-key block against the wave's 32 queries
  const int NB = NP >> 5;
  for (int kb = 0; kb < NB; ++kb) {
    const uint16_t* krow = sm.K + (kb * 32 + col) * kRS + 8 * h;
    const uint16_t* vrow = sm.V + (kb * 32 + col) * kRS + 8 * h;
    // S^T = K~ Q^T from -LSE, tau (dP - Delta)^T = V (tau dO)^T from -tau Delta
    f32x16_t sc = cL, dc = cD;
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      sc = mfma_op<H16>(*reinterpret_cast<const uint4*>(krow + 16 * t), qb[t], sc);
      dc = mfma_op<false>(*reinterpret_cast<const uint4*>(vrow + 16 * t), gb[t], dc);
    }
    const uint32_t live = masked ? live16(sm.lab, kb, h, qlab) : 0xffffu;
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float p0 = ((live >> (2 * e)) & 1u) ? __builtin_amdgcn_exp2f(sc[2 * e]) : 0.f;
      const float p1 = ((live >> (2 * e + 1)) & 1u) ? __builtin_amdgcn_exp2f(sc[2 * e + 1]) : 0.f;
      // tau dS^T, the float32 product rounded once to the operand format
      if constexpr (H16)
        pk[e] = mul2h(p0, dc[2 * e], p1, dc[2 * e + 1]);
      else
        pk[e] = pack2(p0 * dc[2 * e], p1 * dc[2 * e + 1]);
    }
    // dQ~^T += K~^T (tau dS)^T, per 32-channel tile
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      const uint4 kt0 = tr_operand(sm.K + 32 * ct, kRS, kb * 32, lane);
      const uint4 kt1 = tr_operand(sm.K + 32 * ct, kRS, kb * 32 + 16, lane);
      acc[ct] = mfma_op<H16>(kt0, make_uint4(pk[0], pk[1], pk[2], pk[3]), acc[ct]);
      acc[ct] = mfma_op<H16>(kt1, make_uint4(pk[4], pk[5], pk[6], pk[7]), acc[ct]);
    }
  }

  // 4. dq~ = acc / tau / sqrt(d); the dtheta integrand takes q~ as the dK product saw it
  float th[16];
#pragma unroll
  for (int i = 0; i < 16; ++i) th[i] = 0.f;
  if (qvalid) unrotate_store64(acc, 0.125f / ds_scale, kQScale6, H16, q + qoff, dq + qoff, sm.sn, sm.cs, M, qr, qc, h, th);
  const int64_t nwin = g.B * g.nH * g.nW;
  reduce_dtheta64<NW>(th, sm.red, partials + (((int64_t)w.h * 2 + 1) * nwin + wh / g.heads) * 32, lane, wave, tid);
}

template <int NW, bool PAD>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq64_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dq, float* __restrict__ partials, Geom g, int NP) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  QSmem sm;
  sm.K = reinterpret_cast<uint16_t*>(smem_raw);
  sm.V = sm.K + NP * kRS;
  sm.sn = reinterpret_cast<float*>(sm.V + NP * kRS);
  sm.cs = sm.sn + 2 * g.M * 16;
  sm.red = sm.cs + 2 * g.M * 16;
  sm.lab = reinterpret_cast<uint8_t*>(sm.red + NW * 32);
  const int64_t wh = xcd_order(blockIdx.x, gridDim.x);
  const WinHead w = decode_winhead(g, wh);
  const bool edge = w.wy == g.nH - 1 || w.wx == g.nW - 1;
  const bool masked = (g.shift > 0 && edge) || PAD || NP != g.N;  // as in the dK/dV kernel
  fill_table64(sm.sn, sm.cs, th_row, th_col, w.h, g.M, threadIdx.x, NW * 64);
  __syncthreads();
  if (h16_window(scal, wh))
    dq64_body<NW, true, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, NP, sm, w, wh, masked);
  else
    dq64_body<NW, false, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, NP, sm, w, wh, masked);
}

// The dynamic-LDS limit of a kernel is raised on the current device, once per device (beyond
// kMaxDevices: on every call).
template <typename F>
void raise_lds_limit(F* kernel, std::once_flag (&once)[64]) {
  const auto raise = [kernel] {
    (void)hipFuncSetAttribute((const void*)kernel, hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  };
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64)
    std::call_once(once[dev], raise);
  else
    raise();
}

template <int NW, bool PAD>
hipError_t launch_d64(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int NP = (g.N + 31) / 32 * 32;
  if (NP > NW * 32) return hipErrorInvalidConfiguration;
  static std::once_flag once_kv[64], once_q[64];
  raise_lds_limit(bwd_dkdv64_kernel<NW, PAD>, once_kv);
  raise_lds_limit(bwd_dq64_kernel<NW, PAD>, once_q);
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  hipLaunchKernelGGL((bwd_dkdv64_kernel<NW, PAD>), dim3((unsigned)nwh), dim3(NW * 64), kv_smem_bytes(NP, g.M, NW), st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                     a.delta, a.scal, a.th_row, a.th_col, (uint16_t*)a.dk, (uint16_t*)a.dv, a.partials, g, NP);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq64_kernel<NW, PAD>), dim3((unsigned)nwh), dim3(NW * 64), q_smem_bytes(NP, g.M, NW), st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse,
                     a.delta, a.scal, a.th_row, a.th_col, (uint16_t*)a.dq, a.partials, g, NP);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_dtheta_reduce(a.partials, a.n_partials, 2 * g.B * g.nH * g.nW, g, a.dth_row, a.dth_col, st);
}

}  // namespace

bool bwd_d64_supported(const Geom& g) { return g.d == 64 && g.N <= kMaxN6; }

int64_t bwd_d64_partials(const Geom& g) { return (int64_t)g.heads * 2 * g.B * g.nH * g.nW; }

hipError_t launch_bwd_d64(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  if (!bwd_d64_supported(g)) return hipErrorInvalidValue;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  hipLaunchKernelGGL(bwd_pre64_kernel, dim3((unsigned)nwh), dim3(256), 0, st, (const uint16_t*)a.out,
                     (const uint16_t*)a.dout, (const uint16_t*)a.v, (const uint16_t*)a.q, (const uint16_t*)a.k, a.delta,
                     a.scal, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.Hp != g.Hg || g.Wp != g.Wg) {  // padded grid: the instances with padding checks
    if (g.N <= 64) return launch_d64<2, true>(a, st);
    if (g.N <= 128) return launch_d64<4, true>(a, st);
    return launch_d64<8, true>(a, st);
  }
  if (g.N <= 64) return launch_d64<2, false>(a, st);
  if (g.N <= 128) return launch_d64<4, false>(a, st);
  return launch_d64<8, false>(a, st);
}

}  // namespace fsw
