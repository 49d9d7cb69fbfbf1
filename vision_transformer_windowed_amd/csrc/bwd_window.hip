// bf16 window-attention backward on MFMA (gfx950) for windows of up to 256 tokens (M <= 16) that fit
// LDS whole: head dim d = 64, and d = 32 with a rank-r additive bias (r <= 32) whose factors travel as
// extra channels of the score products.
//
// Backward of exact window attention with window-local 2D RoPE, recomputing P from the forward's
// log-sum-exp so that no score matrix is stored (FlashSwin paper card, "FLASHSWIN: Unlocking Large
// Windows and Dense Tokens in Swin Vision Transformers with Memory Efficient Attention": Abstract, flat
// training memory in the window size; Table S1).  In the log2 domain with q^ = q~ log2(e) / sqrt(d):
// P = exp2(q^ . k~ - LSE log2(e)), dS = P (dO . v - Delta), dq~ = sum_j dS k~ / sqrt(d),
// dk~ = sum_i dS q~ / sqrt(d), dv = sum_i P dO, dq = R^T dq~, dk = R^T dk~, and
// dtheta += p (dx~_b x~_a - dx~_a x~_b) over Q and K tokens.
//
// A window of at most 256 tokens fits LDS whole, so each kernel stages one side of a window-head once
// and walks it without chunking or per-chunk barriers:
//  * prologue, one workgroup per window-head: Delta = rowsum(dO * O) per token and the window-head's
//    largest |dO|, |v|, |q|, |k| components, which fix the operand format and power-of-two scales;
//  * dK/dV, key-stationary: a wave owns 32 keys (lane = key) held as B operands; the workgroup stages
//    the window's rotated, scaled queries Q^, dO and g dO in LDS (rows of 64 channels and 16 bytes of
//    pad), with -LSE and -tau Delta.  Per 32-query block: S = Q^ K~^T from -LSE and
//    tau (dP - Delta) = dO (tau V)^T from -tau Delta, P = exp2(S), tau dS = P * tau (dP - Delta),
//    dV^T += (g dO)^T P and dK~^T += Q^T (tau dS) (32-channel output tiles, the transposed operands read
//    by ds_read_b64_tr_b16);
//  * dQ, query-stationary: a wave owns 32 queries; the workgroup stages the rotated K~ and V.  Per
//    32-key block: S^T = K~ Q^T and tau dP'^T = V (tau dO)^T, dQ~^T += K~^T (tau dS)^T.
// Operand precision as in the d = 32 chunked kernels: the derived operands (Q^, K~, P, tau dS, g dO)
// are fp16 when the prologue's maxima put all of them in range, else bf16; dP = dO V^T multiplies bf16
// inputs exactly.  Each workgroup reduces its dtheta terms in a fixed order into one partials row of
// d/2 floats; the shared reduce kernel sums the rows in a fixed order.
//
// Rank-r bias (FlashBias-style factors U, W [heads, M*M, r] over in-window positions; the paper card's
// Table S1 and Table 4 caption): the term U[n_i] . W[n_j] joins each scaled score before the softmax.
// The score operands carry it as extra channels, Q^' = [q^ | log2(e) U] and K~' = [k~ | W] (zero past
// r), so S needs (32 + r) / 16 k-steps.  The same operands then give the factor gradients in the
// extra output rows of the dK and dQ products: dW[n_j] = sum_i dS_ij U[n_i] and
// dU[n_i] = sum_j dS_ij W[n_j].  Both are sums over windows: a workgroup walks G windows of one head,
// adds each window's rows (unscaled by that window's tau) into registers of the lane's key or query, and
// writes one partial row per group; a fixed-order reduce sums the groups.
#include <algorithm>
#include <mutex>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"
#include "fsw_stream.h"

namespace fsw {

namespace {

constexpr int kRS = 72;       // LDS row stride (elements): 64 channels and 16 bytes of pad (144-byte rows,
                              // conflict-free row and transposed reads)
constexpr int kMaxNW = 256;   // largest window (tokens) these kernels serve
constexpr float kRoot2 = 1.4142135623730951f;

// 1 / sqrt(d)
template <int D>
__host__ __device__ constexpr float inv_sqrt_d() {
  return D == 64 ? 0.125f : 0.17677669529663687f;
}

// Channel layout of an instance: head dim D (64, or 32 with a bias) and RK bias channels (0, 16 or 32)
// appended to the score operands.  Score rows hold DK = D + RK channels (zero beyond), so at most 64.
template <int D, int RK>
struct WDim {
  static_assert((D == 64 && RK == 0) || (D == 32 && (RK == 16 || RK == 32)), "unsupported channel layout");
  static constexpr int DK = D + RK;          // channels of the score products
  static constexpr int KST = DK / 16;        // their k-steps
  static constexpr int DST = D / 16;         // k-steps of dP = dO V^T
  static constexpr int VT = D / 32;          // 32-channel tiles of dV
  static constexpr int KT = (DK + 31) / 32;  // tiles of the score-side gradient: dK~ (dQ~), then the factor's
  static constexpr int PA = D / 4;           // RoPE pairs per axis
  static constexpr float kInvSqrtD = inv_sqrt_d<D>();
  static constexpr float kQScale = kLog2e * kInvSqrtD;  // log2(e) / sqrt(d)
};

// Power of two 2^k (k clamped to [-100, 100]) with 2^k * bound <= 2^14 (1 when bound is 0 or not finite).
__device__ __forceinline__ float scale_to_2p14(float bound) {
  if (!(bound > 0.f) || !(bound < INFINITY)) return 1.f;
  int e;
  frexpf(bound, &e);  // bound < 2^e
  return ldexpf(1.f, min(100, max(-100, 14 - e)));
}

// fp16 score operands when every rotated, scaled component is in range (a rotation grows a component
// by at most sqrt(2)).
template <int D>
__device__ __forceinline__ bool h16_window(const float* scal, int64_t wh) {
  return kRoot2 * scal[wh * 4 + 2] * (kLog2e * inv_sqrt_d<D>()) < kF16Limit &&
         kRoot2 * scal[wh * 4 + 3] < kF16Limit;
}

// RoPE sin/cos table of one head, [2 axes][M positions][D/4 pairs].
template <int D>
__device__ inline void fill_table(float* sn, float* cs, const float* th_row, const float* th_col, int head, int M,
                                  int tid, int nt) {
  constexpr int PA = D / 4;
  for (int i = tid; i < 2 * M * PA; i += nt) {
    const int axis = i / (M * PA);
    const int p = (i / PA) % M;
    const int j = i % PA;
    const float th = axis ? th_col[head * PA + j] : th_row[head * PA + j];
    float s, c;
    rope_sincos(th, p, &s, &c);
    sn[i] = s;
    cs[i] = c;
  }
}

// Channels 8 part .. 8 part + 7 of token (r, c), rotated (the first D/16 parts: row axis, the rest:
// column axis), scaled, packed to the operand format.
template <int D, bool H16>
__device__ __forceinline__ uint4 rot_part(uint4 raw, const float* sn, const float* cs, int M, int r, int c, int part,
                                          float scale) {
  float x[8];
  unpack8(raw, x);
  const int axis = part / (D / 16);
  rotate8(x, sn, cs, axis, M, axis ? c : r, (part % (D / 16)) * 4, D / 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= scale;
  return pack8_op(x, H16);
}

// Channels c0 .. c0 + 7 (c0 a multiple of 8 below RK) of row n of a head's zero-padded bias factor
// (float32 [heads][N][RK], written by factor_prep_kernel): two aligned 16-byte words.
template <int RK>
__device__ __forceinline__ const uint4* factor_row8(const float* f, int head, int n, int c0, int N) {
  return reinterpret_cast<const uint4*>(f + ((int64_t)head * N + n) * RK + c0);
}

// Eight factor values (two words of factor_row8) times `scale`, packed to the operand format.
template <bool H16>
__device__ __forceinline__ uint4 factor_op(uint4 a, uint4 b, float scale) {
  const float x[8] = {__uint_as_float(a.x) * scale, __uint_as_float(a.y) * scale, __uint_as_float(a.z) * scale,
                      __uint_as_float(a.w) * scale, __uint_as_float(b.x) * scale, __uint_as_float(b.y) * scale,
                      __uint_as_float(b.z) * scale, __uint_as_float(b.w) * scale};
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

// Epilogue of the dK and dQ kernels for the lane's token: gradient w.r.t. the rotated vector in the first
// D/32 tiles (value v of acc[ct]: channel 32 ct + 8(v/4) + 4h + v%4, times `scale`), recompute the
// rotated input as the products saw it (scaled by op_scale, rounded to the operand format, scaled back),
// accumulate the D/4 dtheta slots of the lane (slot (D/8) axis + 2 gg + u: pair 4 gg + 2h + u of the
// axis), un-rotate, store bf16.
template <int D, int NA>
__device__ inline void unrotate_store(const f32x16_t (&acc)[NA], float scale, float op_scale, bool op16,
                                      const uint16_t* xsrc, uint16_t* dst, const float* sn, const float* cs, int M,
                                      int r, int c, int h, float (&t)[D / 4]) {
  constexpr int PA = D / 4;
  const float inv_op = 1.f / op_scale;
  uint2 rawg[D / 32][4];  // every load first: one wait instead of one per group
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct)
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) rawg[ct][gq] = *reinterpret_cast<const uint2*>(xsrc + 32 * ct + 8 * gq + 4 * h);
#pragma unroll
  for (int ct = 0; ct < D / 32; ++ct) {
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      const int ach = 32 * ct + 8 * gq;   // first channel of the lane's group (plus 4h)
      const int axis = ach / (D / 2);
      const int gg = (ach % (D / 2)) / 8;
      const int pos = axis ? c : r;
      const int ch = ach + 4 * h;
      const uint2 raw = rawg[ct][gq];
      const float xin[4] = {__uint_as_float(raw.x << 16), __uint_as_float(raw.x & 0xffff0000u),
                            __uint_as_float(raw.y << 16), __uint_as_float(raw.y & 0xffff0000u)};
      float res[4];
#pragma unroll
      for (int u = 0; u < 2; ++u) {
        const int j = 4 * gg + 2 * h + u;  // pair within the axis
        const float s = sn[(axis * M + pos) * PA + j];
        const float co = cs[(axis * M + pos) * PA + j];
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
        t[(PA / 2) * axis + 2 * gg + u] += (float)pos * (db * at - da * bt);
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

// Fixed-order reduction of the lanes' D/4 dtheta slots over the workgroup into one partials row of D/2
// floats (row-axis pairs, then column-axis pairs): a butterfly over the 32 lanes of each half-wave, then
// the waves in order.
template <int NW, int D>
__device__ inline void reduce_dtheta(float (&t)[D / 4], float* red, float* dst, int lane, int wave, int tid) {
  constexpr int PA = D / 4;
#pragma unroll
  for (int i = 0; i < PA; ++i) {
#pragma unroll
    for (int o = 1; o < 32; o <<= 1) t[i] += __shfl_xor(t[i], o, 64);
  }
  if ((lane & 31) == 0) {
    const int h = lane >> 5;
#pragma unroll
    for (int axis = 0; axis < 2; ++axis)
#pragma unroll
      for (int gg = 0; gg < PA / 4; ++gg)
#pragma unroll
        for (int u = 0; u < 2; ++u)
          red[wave * (D / 2) + PA * axis + 4 * gg + 2 * h + u] = t[(PA / 2) * axis + 2 * gg + u];
  }
  __syncthreads();
  if (tid < D / 2) {
    float s = 0.f;
    for (int i = 0; i < NW; ++i) s += red[i * (D / 2) + tid];
    dst[tid] = s;
  }
}

// ------------------------------------------------------------------------------------ prologue

// What a prologue workgroup reads and writes.
enum PreMode {
  kPreFull = 0,    // O, dO, q, k, v: Delta and scal
  kPreStats = 1,   // O and dO: Delta and max |dO|; the other maxima come from the forward's stats
  kPreMaxima = 2,  // q, k, v: the forward's stats, for the forward kernels that do not produce them
};

// One workgroup per window-head: Delta of its tokens and scal[wh] = {max |dO|, max |v|, max |q|, max |k|}
// (or, kPreMaxima, stats[wh] = {max |q|, 0, max |k|, max |v|}).  Thread: 16-byte part p = tid % (D/8)
// of tokens tid / (D/8), tid / (D/8) + 256 / (D/8), ...  The full prologue is launched for d = 64; the
// bias kernels (d = 32) take the prologue of the chunked d = 32 kernels, which reads several heads'
// slices of a token row at once.
template <int D, int MODE>
__global__ __launch_bounds__(256) void bwd_pre_win_kernel(const uint16_t* __restrict__ out,
                                                          const uint16_t* __restrict__ dout,
                                                          const uint16_t* __restrict__ v,
                                                          const uint16_t* __restrict__ q,
                                                          const uint16_t* __restrict__ k, float* __restrict__ delta,
                                                          float* __restrict__ scal, float* __restrict__ stats,
                                                          Geom g) {
  constexpr int PPT = D / 8;        // parts per token
  constexpr int TPP = 256 / PPT;    // tokens per pass
  __shared__ float red[4][4];
  const int64_t wh = xcd_order(blockIdx.x, gridDim.x);
  const WinHead w = decode_winhead(g, wh);
  const int tid = threadIdx.x, p = tid % PPT;
  float mx[4] = {0.f, 0.f, 0.f, 0.f};  // max |dO|, |v|, |q|, |k|
  // a NaN component counts as infinity (fmaxf would drop it)
  const auto amax = [](float m, float x) { return fmaxf(m, x != x ? INFINITY : fabsf(x)); };
  for (int n0 = 0; n0 < g.N; n0 += TPP) {  // uniform trip count: every lane reaches the shuffles
    const int n = n0 + tid / PPT;
    const bool ok = n < g.N && token_real(g, w.wy, w.wx, n / g.M, n % g.M);
    float s = 0.f;
    int64_t tok = 0;
    if (ok) {
      tok = token_index(g, w.b, w.wy, w.wx, n / g.M, n % g.M);
      const int64_t xo = tok * g.xs + w.h * D + 8 * p, oo = tok * g.os + w.h * D + 8 * p;
      if constexpr (MODE != kPreMaxima) {
        float o8[8], d8[8];
        unpack8(*reinterpret_cast<const uint4*>(out + oo), o8);
        unpack8(*reinterpret_cast<const uint4*>(dout + oo), d8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          s = __builtin_fmaf(o8[e], d8[e], s);
          mx[0] = amax(mx[0], d8[e]);
        }
      }
      if constexpr (MODE != kPreStats) {
        float v8[8], q8[8], k8[8];
        unpack8(*reinterpret_cast<const uint4*>(v + xo), v8);
        unpack8(*reinterpret_cast<const uint4*>(q + xo), q8);
        unpack8(*reinterpret_cast<const uint4*>(k + xo), k8);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          mx[1] = amax(mx[1], v8[e]);
          mx[2] = amax(mx[2], q8[e]);
          mx[3] = amax(mx[3], k8[e]);
        }
      }
    }
    if constexpr (MODE != kPreMaxima) {
#pragma unroll
      for (int o = 1; o < PPT; o <<= 1) s += __shfl_xor(s, o, 64);
      if (ok && p == 0) delta[tok * g.heads + w.h] = s;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) mx[i] = wave_max(mx[i]);
  if ((tid & 63) == 0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) red[tid >> 6][i] = mx[i];
  }
  __syncthreads();
  if (tid < 4) {
    const auto total = [&](int i) { return fmaxf(fmaxf(red[0][i], red[1][i]), fmaxf(red[2][i], red[3][i])); };
    if constexpr (MODE == kPreMaxima) {
      stats[wh * 4 + tid] = tid == 0 ? total(2) : tid == 1 ? 0.f : tid == 2 ? total(3) : total(1);
    } else if constexpr (MODE == kPreStats) {
      const float* s4 = stats + wh * 4;
      scal[wh * 4 + tid] = tid == 0 ? total(0) : tid == 1 ? s4[3] : tid == 2 ? fmaxf(s4[0], s4[1]) : s4[2];
    } else {
      scal[wh * 4 + tid] = total(tid);
    }
  }
}

// Per head: the bias factors zero-padded from rank to RK channels (upad, wpad [heads][N][RK], so that
// the kernels read eight channels as two aligned 16-byte words), and their largest |component|:
// fmax[2h] = max |U[h]|, fmax[2h + 1] = max |W[h]| (a NaN counts as infinity).  One workgroup per head.
template <int RK>
__global__ __launch_bounds__(256) void factor_prep_kernel(const float* __restrict__ u, const float* __restrict__ w,
                                                          int rank, int N, float* __restrict__ upad,
                                                          float* __restrict__ wpad, float* __restrict__ fmax) {
  __shared__ float red[4][2];
  const int h = blockIdx.x, tid = threadIdx.x;
  float mu = 0.f, mw = 0.f;
  for (int i = tid; i < N * RK; i += 256) {
    const int n = i / RK, c = i % RK;
    const int64_t src = ((int64_t)h * N + n) * rank + c;
    const float a = c < rank ? u[src] : 0.f, b = c < rank ? w[src] : 0.f;
    upad[(int64_t)h * N * RK + i] = a;
    wpad[(int64_t)h * N * RK + i] = b;
    mu = fmaxf(mu, a != a ? INFINITY : fabsf(a));
    mw = fmaxf(mw, b != b ? INFINITY : fabsf(b));
  }
  mu = wave_max(mu);
  mw = wave_max(mw);
  if ((tid & 63) == 0) {
    red[tid >> 6][0] = mu;
    red[tid >> 6][1] = mw;
  }
  __syncthreads();
  if (tid < 2) fmax[2 * h + tid] = fmaxf(fmaxf(red[0][tid], red[1][tid]), fmaxf(red[2][tid], red[3][tid]));
}

// fp16 operands for a head's bias channels: log2(e) U and W in fp16 range.
__device__ __forceinline__ bool factors_h16(const float* fmax, int h) {
  return kLog2e * fmax[2 * h] < kF16Limit && fmax[2 * h + 1] < kF16Limit;
}

// ---------------------------------------------------------------------------------------- dK / dV

// LDS of the dK/dV kernel for NP padded tokens.
struct KvSmem {
  uint16_t* Q;    // [NP][kRS] rotated, scaled Q^ (operand format), then log2(e) U
  uint16_t* G;    // [NP][kRS] bf16 dO
  uint16_t* Gs;   // [NP][kRS] g dO (operand format)
  float* L;       // [NP] -LSE log2(e)
  float* Dl;      // [NP] -tau Delta
  float* sn;      // [2][M][D/4]
  float* cs;
  float* red;     // [NW][D/2]
  uint8_t* lab;   // [NP]
};
template <int D>
__host__ __device__ inline size_t kv_smem_bytes(int NP, int M, int NW) {
  return (size_t)NP * kRS * 2 * 3 + (size_t)NP * 4 * 2 + (size_t)2 * 2 * M * (D / 4) * 4 + (size_t)NW * (D / 2) * 4 +
         NP;
}

// One window-head.  fac (RK > 0): the lane's key's factor-gradient rows, to which this window's
// dW = sum_i dS U is added.
template <int D, int RK, int NW, bool H16, bool PAD>
__device__ inline void dkdv_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                 const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                                 const float* __restrict__ lse, const float* __restrict__ delta,
                                 const float* __restrict__ scal, uint16_t* __restrict__ dk, uint16_t* __restrict__ dv,
                                 float* __restrict__ partials, const Geom& g, int NP, const KvSmem& sm,
                                 const WinHead& w, int64_t wh, bool masked, const LowRank& lr, float (&fac)[16]) {
  using WD = WDim<D, RK>;
  constexpr int NT = NW * 64;
  constexpr int IPT = 4;  // staged 16-byte items per thread: NP <= 32 NW tokens of 8 items
  const int M = g.M, N = g.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const float g_scale = scale_to_2p14(scal[wh * 4]);                                   // dO of the dV product
  const float ds_scale = scale_to_2p14(2.f * D * scal[wh * 4] * scal[wh * 4 + 1]);  // |tau dS| <= 2^14

  // 1. every global load first (the staged items: part it % 8 of token it / 8; then the lane's key), so
  //    that their latencies overlap; the transforms follow
  // (the loads of an item are unconditional inside one test, so the compiler keeps them in one batch:
  //  a part beyond the head's channels reads channels of part D/8 - 1, and LSE and Delta are read by
  //  every part, kept by part 0)
  uint4 ra[IPT], rb[IPT];
  float rl[IPT], rd[IPT];
  const int64_t tok0 = w.b * g.Hg * g.Wg;  // a grid token of the image: the address of items that are none
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int it = tid + i * NT;
    const int n = it >> 3, part = it & 7;
    const bool ok = it < NP * 8 && n < N && (!PAD || token_real(g, w.wy, w.wx, n / M, n % M));
    const int64_t tok = ok ? token_index(g, w.b, w.wy, w.wx, n / M, n % M) : tok0;
    const int pc = min(part, D / 8 - 1);
    const uint4* pa = reinterpret_cast<const uint4*>(q + tok * g.xs + w.h * D + 8 * pc);
    const uint4* pb = reinterpret_cast<const uint4*>(dout + tok * g.os + w.h * D + 8 * pc);
    if constexpr (RK > 0) {
      if (part >= D / 8) {  // a bias part: its eight padded U channels instead
        pa = factor_row8<RK>(lr.u, w.h, ok ? n : 0, min(8 * part - D, RK - 8), N);
        pb = pa + 1;
      }
    }
    ra[i] = *pa;
    rb[i] = *pb;
    rl[i] = lse[tok * g.heads + w.h];
    rd[i] = delta[tok * g.heads + w.h];
  }
  const int kj = wave * 32 + col;
  const bool kvalid = kj < N && (!PAD || token_real(g, w.wy, w.wx, kj / M, kj % M));  // a padding key is no key
  const int kr = kvalid ? kj / M : 0, kc = kvalid ? kj - (kj / M) * M : 0;
  int64_t koff = 0;
  uint4 kb[WD::KST], vb[WD::DST], fw[WD::KST - WD::DST + 1];
  koff = (kvalid ? token_index(g, w.b, w.wy, w.wx, kr, kc) : tok0) * g.xs + w.h * D;
#pragma unroll
  for (int t = 0; t < WD::DST; ++t) {
    kb[t] = *reinterpret_cast<const uint4*>(k + koff + 16 * t + 8 * h);
    vb[t] = *reinterpret_cast<const uint4*>(v + koff + 16 * t + 8 * h);
  }
#pragma unroll
  for (int t = WD::DST; t < WD::KST; ++t) {
    const uint4* f = factor_row8<RK>(lr.w, w.h, kvalid ? kj : 0, 16 * t + 8 * h - D, N);
    kb[t] = f[0];
    fw[t - WD::DST] = f[1];
  }

  // 2. stage every query-side row of the window
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int it = tid + i * NT;
    if (it >= NP * 8) break;  // uniform across a wave: NP * 8 is a multiple of 256
    const int n = it >> 3, part = it & 7;
    uint4 qo = make_uint4(0, 0, 0, 0), go = qo, gs = qo;
    uint8_t lb = 0xff;
    if (n < N && (!PAD || token_real(g, w.wy, w.wx, n / M, n % M))) {  // padding stays zero, label 0xff
      const int r = n / M, c = n - (n / M) * M;
      if (part < D / 8) {
        go = rb[i];
        qo = rot_part<D, H16>(ra[i], sm.sn, sm.cs, M, r, c, part, WD::kQScale);
        gs = scaled_part<H16>(go, g_scale);
      } else if (part < WD::DK / 8) {
        qo = factor_op<H16>(ra[i], rb[i], kLog2e);
      }
      if (part == 0) lb = (uint8_t)token_label(g, w.wy, w.wx, r, c);
    }
    *reinterpret_cast<uint4*>(sm.Q + n * kRS + 8 * part) = qo;
    if (part < D / 8) {
      *reinterpret_cast<uint4*>(sm.G + n * kRS + 8 * part) = go;
      *reinterpret_cast<uint4*>(sm.Gs + n * kRS + 8 * part) = gs;
    }
    if (part == 0) {
      sm.L[n] = lb != 0xff ? -rl[i] * kLog2e : 0.f;  // lb: the label of a grid token, 0xff otherwise
      sm.Dl[n] = lb != 0xff ? -rd[i] * ds_scale : 0.f;
      sm.lab[n] = lb;
    }
  }

  // 3. the lane's key: K~' operands (k-step t: channels 16t + 8h ..), tau V as bf16 B operands (zero for
  //    a lane without a key)
  int klab = 0xff;
  if (kvalid) {
    klab = token_label(g, w.wy, w.wx, kr, kc);
#pragma unroll
    for (int t = 0; t < WD::DST; ++t) {
      kb[t] = rot_part<D, H16>(kb[t], sm.sn, sm.cs, M, kr, kc, 2 * t + h, 1.f);
      vb[t] = scaled_part<false>(vb[t], ds_scale);
    }
#pragma unroll
    for (int t = WD::DST; t < WD::KST; ++t)
      kb[t] = factor_op<H16>(kb[t], fw[t - WD::DST], 1.f);
  } else {
#pragma unroll
    for (int t = 0; t < WD::KST; ++t) kb[t] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < WD::DST; ++t) vb[t] = make_uint4(0, 0, 0, 0);
  }
  f32x16_t accv[WD::VT], acck[WD::KT];
#pragma unroll
  for (int ct = 0; ct < WD::VT; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) accv[ct][e] = 0.f;
#pragma unroll
  for (int ct = 0; ct < WD::KT; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) acck[ct][e] = 0.f;
  __syncthreads();

  // 4. every 32-query block against the wave's 32 keys
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
    // S = Q^' K~'^T from -LSE, tau (dP - Delta) = dO (tau V)^T from -tau Delta
    const uint16_t* qrow = sm.Q + (qb * 32 + col) * kRS + 8 * h;
    const uint16_t* grow = sm.G + (qb * 32 + col) * kRS + 8 * h;
    f32x16_t sc = cL, dc = cD;
#pragma unroll
    for (int t = 0; t < WD::KST; ++t) {
      sc = mfma_op<H16>(*reinterpret_cast<const uint4*>(qrow + 16 * t), kb[t], sc);
      if (t < WD::DST) dc = mfma_op<false>(*reinterpret_cast<const uint4*>(grow + 16 * t), vb[t], dc);
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
    // dV^T += (g dO)^T P and dK~'^T += Q^'^T (tau dS), per 32-channel tile
#pragma unroll
    for (int ct = 0; ct < WD::KT; ++ct) {
      if (ct < WD::VT) {
        const uint4 gt0 = tr_operand(sm.Gs + 32 * ct, kRS, qb * 32, lane);
        const uint4 gt1 = tr_operand(sm.Gs + 32 * ct, kRS, qb * 32 + 16, lane);
        accv[ct] = mfma_op<H16>(gt0, make_uint4(pp[0], pp[1], pp[2], pp[3]), accv[ct]);
        accv[ct] = mfma_op<H16>(gt1, make_uint4(pp[4], pp[5], pp[6], pp[7]), accv[ct]);
      }
      const uint4 qt0 = tr_operand(sm.Q + 32 * ct, kRS, qb * 32, lane);
      const uint4 qt1 = tr_operand(sm.Q + 32 * ct, kRS, qb * 32 + 16, lane);
      acck[ct] = mfma_op<H16>(qt0, make_uint4(pd[0], pd[1], pd[2], pd[3]), acck[ct]);
      acck[ct] = mfma_op<H16>(qt1, make_uint4(pd[4], pd[5], pd[6], pd[7]), acck[ct]);
    }
  }

  // 5. dV = accv / g; dk~ = acck ln 2 / tau (the Q^ operand carried log2(e) / sqrt(d)); dW rows
  //    (the log2(e) U channels) likewise ln 2 / tau; dtheta terms
  float th[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) th[i] = 0.f;
  if (kvalid) {
    const float inv_g = 1.f / g_scale;
#pragma unroll
    for (int ct = 0; ct < WD::VT; ++ct)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint2 o;
        o.x = pack2(accv[ct][4 * gq] * inv_g, accv[ct][4 * gq + 1] * inv_g);
        o.y = pack2(accv[ct][4 * gq + 2] * inv_g, accv[ct][4 * gq + 3] * inv_g);
        *reinterpret_cast<uint2*>(dv + koff + 32 * ct + 8 * gq + 4 * h) = o;
      }
    unrotate_store<D>(acck, kLn2 / ds_scale, 1.f, H16, k + koff, dk + koff, sm.sn, sm.cs, M, kr, kc, h, th);
    if constexpr (RK > 0) {
      const float fs = kLn2 / ds_scale;
#pragma unroll
      for (int e = 0; e < 16; ++e) fac[e] += acck[WD::KT - 1][e] * fs;
    }
  }
  const int64_t nwin = g.B * g.nH * g.nW;
  reduce_dtheta<NW, D>(th, sm.red, partials + (((int64_t)w.h * 2 + 0) * nwin + wh / g.heads) * (D / 2), lane, wave,
                       tid);
}

// Lane's factor-gradient rows (the lane's token n = 32 wave + lane % 32, channels 8(e/4) + 4h + e%4 of
// its 16 values) into row n of one [N][rank] partial.
__device__ inline void store_factor_rows(const float (&fac)[16], float* dst, int N, int rank) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int n = wave * 32 + (lane & 31), h = lane >> 5;
  if (n >= N) return;
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    const int c = 8 * (e >> 2) + 4 * h + (e & 3);
    if (c < rank) dst[(int64_t)n * rank + c] = fac[e];
  }
}

// Several Swin regions only in the last window row and column of a shifted grid.  Padding can sit in
// the last two window rows or columns of a shifted padded grid: every window of a padded grid is masked
// (a padding key must get P = 0 exactly, not exp2(0 - LSE)).
template <bool PAD>
__device__ __forceinline__ bool window_masked(const Geom& g, const WinHead& w, int NP) {
  const bool edge = w.wy == g.nH - 1 || w.wx == g.nW - 1;
  return (g.shift > 0 && edge) || PAD || NP != g.N;
}

// Without a bias (RK == 0): one window-head per workgroup.  With a bias: workgroup grp walks windows
// G (grp / heads) .. of head grp % heads and writes its dW partial row block to fparts.
template <int D, int RK, int NW, bool PAD>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dkdv_win_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dk, uint16_t* __restrict__ dv, float* __restrict__ partials, Geom g, int NP, LowRank lr,
    const float* __restrict__ fmax, float* __restrict__ fparts, int G) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  KvSmem sm;
  sm.Q = reinterpret_cast<uint16_t*>(smem_raw);
  sm.G = sm.Q + NP * kRS;
  sm.Gs = sm.G + NP * kRS;
  sm.L = reinterpret_cast<float*>(sm.Gs + NP * kRS);
  sm.Dl = sm.L + NP;
  sm.sn = sm.Dl + NP;
  sm.cs = sm.sn + 2 * g.M * (D / 4);
  sm.red = sm.cs + 2 * g.M * (D / 4);
  sm.lab = reinterpret_cast<uint8_t*>(sm.red + NW * (D / 2));
  const int64_t grp = xcd_order(blockIdx.x, gridDim.x);
  float fac[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) fac[e] = 0.f;
  if constexpr (RK == 0) {
    const WinHead w = decode_winhead(g, grp);
    const bool masked = window_masked<PAD>(g, w, NP);
    fill_table<D>(sm.sn, sm.cs, th_row, th_col, w.h, g.M, threadIdx.x, NW * 64);
    __syncthreads();
    if (h16_window<D>(scal, grp))
      dkdv_body<D, RK, NW, true, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, NP, sm, w, grp, masked, lr,
                                      fac);
    else
      dkdv_body<D, RK, NW, false, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, NP, sm, w, grp, masked,
                                       lr, fac);
  } else {
    const int head = (int)(grp % g.heads);
    const int64_t nwin = g.B * g.nH * g.nW, wg = grp / g.heads, w0 = wg * G;
    const int nw = (int)min((int64_t)G, nwin - w0);
    const bool fh16 = factors_h16(fmax, head);
    fill_table<D>(sm.sn, sm.cs, th_row, th_col, head, g.M, threadIdx.x, NW * 64);
    __syncthreads();
    for (int i = 0; i < nw; ++i) {  // the body's barriers separate one window's LDS use from the next
      const int64_t wh = (w0 + i) * g.heads + head;
      const WinHead w = decode_winhead(g, wh);
      const bool masked = window_masked<PAD>(g, w, NP);
      if (fh16 && h16_window<D>(scal, wh))
        dkdv_body<D, RK, NW, true, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, NP, sm, w, wh, masked,
                                        lr, fac);
      else
        dkdv_body<D, RK, NW, false, PAD>(q, k, v, dout, lse, delta, scal, dk, dv, partials, g, NP, sm, w, wh, masked,
                                         lr, fac);
    }
    store_factor_rows(fac, fparts + (wg * g.heads + head) * (int64_t)g.N * lr.rank, g.N, lr.rank);
  }
}

// ---------------------------------------------------------------------------------------- dQ

struct QSmem {
  uint16_t* K;    // [NP][kRS] rotated K~ (operand format), then W
  uint16_t* V;    // [NP][kRS] bf16 V
  float* sn;
  float* cs;
  float* red;     // [NW][D/2]
  uint8_t* lab;   // [NP]
};
template <int D>
__host__ __device__ inline size_t q_smem_bytes(int NP, int M, int NW) {
  return (size_t)NP * kRS * 2 * 2 + (size_t)2 * 2 * M * (D / 4) * 4 + (size_t)NW * (D / 2) * 4 + NP;
}

// One window-head.  fac (RK > 0): the lane's query's factor-gradient rows, to which this window's
// dU = sum_j dS W is added.
template <int D, int RK, int NW, bool H16, bool PAD>
__device__ inline void dq_body(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                               const uint16_t* __restrict__ v, const uint16_t* __restrict__ dout,
                               const float* __restrict__ lse, const float* __restrict__ delta,
                               const float* __restrict__ scal, uint16_t* __restrict__ dq, float* __restrict__ partials,
                               const Geom& g, int NP, const QSmem& sm, const WinHead& w, int64_t wh, bool masked,
                               const LowRank& lr, float (&fac)[16]) {
  using WD = WDim<D, RK>;
  constexpr int NT = NW * 64;
  constexpr int IPT = 4;  // staged 16-byte items per thread: NP <= 32 NW tokens of 8 items
  const int M = g.M, N = g.N;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int h = lane >> 5, col = lane & 31;
  const float ds_scale = scale_to_2p14(2.f * D * scal[wh * 4] * scal[wh * 4 + 1]);

  // 1. every global load first (the staged K, V or W items, then the lane's query), so that their
  //    latencies overlap; the transforms follow
  // (as in the dK/dV kernel, the loads of an item are unconditional inside one test)
  uint4 ra[IPT], rb[IPT];
  const int64_t tok0 = w.b * g.Hg * g.Wg;  // a grid token of the image: the address of items that are none
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int it = tid + i * NT;
    const int n = it >> 3, part = it & 7;
    const bool ok = it < NP * 8 && n < N && (!PAD || token_real(g, w.wy, w.wx, n / M, n % M));
    const int64_t off = (ok ? token_index(g, w.b, w.wy, w.wx, n / M, n % M) : tok0) * g.xs + w.h * D +
                        8 * min(part, D / 8 - 1);
    const uint4* pa = reinterpret_cast<const uint4*>(k + off);
    const uint4* pb = reinterpret_cast<const uint4*>(v + off);
    if constexpr (RK > 0) {
      if (part >= D / 8) {  // a bias part: its eight padded W channels instead
        pa = factor_row8<RK>(lr.w, w.h, ok ? n : 0, min(8 * part - D, RK - 8), N);
        pb = pa + 1;
      }
    }
    ra[i] = *pa;
    rb[i] = *pb;
  }
  const int qi = wave * 32 + col;
  const bool qvalid = qi < N && (!PAD || token_real(g, w.wy, w.wx, qi / M, qi % M));  // a padding query is no query
  const int qr = qvalid ? qi / M : 0, qc = qvalid ? qi - (qi / M) * M : 0;
  int64_t qoff = 0;
  uint4 qb[WD::KST], gb[WD::DST], fu[WD::KST - WD::DST + 1];
  const int64_t qtok = qvalid ? token_index(g, w.b, w.wy, w.wx, qr, qc) : tok0;
  qoff = qtok * g.xs + w.h * D;
  const int64_t goff = qtok * g.os + w.h * D;
  float lse2 = lse[qtok * g.heads + w.h], del = delta[qtok * g.heads + w.h];
#pragma unroll
  for (int t = 0; t < WD::DST; ++t) {
    qb[t] = *reinterpret_cast<const uint4*>(q + qoff + 16 * t + 8 * h);
    gb[t] = *reinterpret_cast<const uint4*>(dout + goff + 16 * t + 8 * h);
  }
#pragma unroll
  for (int t = WD::DST; t < WD::KST; ++t) {
    const uint4* f = factor_row8<RK>(lr.u, w.h, qvalid ? qi : 0, 16 * t + 8 * h - D, N);
    qb[t] = f[0];
    fu[t - WD::DST] = f[1];
  }

  // 2. stage the window's rotated K~ (then W) and V rows
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int it = tid + i * NT;
    if (it >= NP * 8) break;
    const int n = it >> 3, part = it & 7;
    uint4 ko = make_uint4(0, 0, 0, 0), vo = ko;
    uint8_t lb = 0xff;
    if (n < N && (!PAD || token_real(g, w.wy, w.wx, n / M, n % M))) {  // padding stays zero, label 0xff
      const int r = n / M, c = n - (n / M) * M;
      if (part < D / 8) {
        ko = rot_part<D, H16>(ra[i], sm.sn, sm.cs, M, r, c, part, 1.f);
        vo = rb[i];
      } else if (part < WD::DK / 8) {
        ko = factor_op<H16>(ra[i], rb[i], 1.f);
      }
      if (part == 0) lb = (uint8_t)token_label(g, w.wy, w.wx, r, c);
    }
    *reinterpret_cast<uint4*>(sm.K + n * kRS + 8 * part) = ko;
    if (part < D / 8) *reinterpret_cast<uint4*>(sm.V + n * kRS + 8 * part) = vo;
    if (part == 0) sm.lab[n] = lb;
  }

  // 3. the lane's query: Q^' operands, tau dO as bf16 B operands, -LSE and -tau Delta
  int qlab = 0xff;
  if (qvalid) {
    qlab = token_label(g, w.wy, w.wx, qr, qc);
    lse2 *= kLog2e;
    del *= ds_scale;
#pragma unroll
    for (int t = 0; t < WD::DST; ++t) {
      qb[t] = rot_part<D, H16>(qb[t], sm.sn, sm.cs, M, qr, qc, 2 * t + h, WD::kQScale);
      gb[t] = scaled_part<false>(gb[t], ds_scale);
    }
#pragma unroll
    for (int t = WD::DST; t < WD::KST; ++t)
      qb[t] = factor_op<H16>(qb[t], fu[t - WD::DST], kLog2e);
  } else {  // a lane without a query: zero operands, reference 0
    lse2 = del = 0.f;
#pragma unroll
    for (int t = 0; t < WD::KST; ++t) qb[t] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int t = 0; t < WD::DST; ++t) gb[t] = make_uint4(0, 0, 0, 0);
  }
  f32x16_t cL, cD, acc[WD::KT];
#pragma unroll
  for (int e = 0; e < 16; ++e) {
    cL[e] = -lse2;
    cD[e] = -del;
  }
#pragma unroll
  for (int ct = 0; ct < WD::KT; ++ct)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[ct][e] = 0.f;
  __syncthreads();

  // 4. every 32-key block against the wave's 32 queries
  const int NB = NP >> 5;
  for (int kb = 0; kb < NB; ++kb) {
    const uint16_t* krow = sm.K + (kb * 32 + col) * kRS + 8 * h;
    const uint16_t* vrow = sm.V + (kb * 32 + col) * kRS + 8 * h;
    // S^T = K~' Q^'^T from -LSE, tau (dP - Delta)^T = V (tau dO)^T from -tau Delta
    f32x16_t sc = cL, dc = cD;
#pragma unroll
    for (int t = 0; t < WD::KST; ++t) {
      sc = mfma_op<H16>(*reinterpret_cast<const uint4*>(krow + 16 * t), qb[t], sc);
      if (t < WD::DST) dc = mfma_op<false>(*reinterpret_cast<const uint4*>(vrow + 16 * t), gb[t], dc);
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
    // dQ~'^T += K~'^T (tau dS)^T, per 32-channel tile
#pragma unroll
    for (int ct = 0; ct < WD::KT; ++ct) {
      const uint4 kt0 = tr_operand(sm.K + 32 * ct, kRS, kb * 32, lane);
      const uint4 kt1 = tr_operand(sm.K + 32 * ct, kRS, kb * 32 + 16, lane);
      acc[ct] = mfma_op<H16>(kt0, make_uint4(pk[0], pk[1], pk[2], pk[3]), acc[ct]);
      acc[ct] = mfma_op<H16>(kt1, make_uint4(pk[4], pk[5], pk[6], pk[7]), acc[ct]);
    }
  }

  // 5. dq~ = acc / tau / sqrt(d); the dtheta integrand takes q~ as the dK product saw it; dU rows
  //    (the W channels) acc / tau
  float th[D / 4];
#pragma unroll
  for (int i = 0; i < D / 4; ++i) th[i] = 0.f;
  if (qvalid) {
    unrotate_store<D>(acc, WD::kInvSqrtD / ds_scale, WD::kQScale, H16, q + qoff, dq + qoff, sm.sn, sm.cs, M, qr, qc, h,
                      th);
    if constexpr (RK > 0) {
      const float fs = 1.f / ds_scale;
#pragma unroll
      for (int e = 0; e < 16; ++e) fac[e] += acc[WD::KT - 1][e] * fs;
    }
  }
  const int64_t nwin = g.B * g.nH * g.nW;
  reduce_dtheta<NW, D>(th, sm.red, partials + (((int64_t)w.h * 2 + 1) * nwin + wh / g.heads) * (D / 2), lane, wave,
                       tid);
}

// Work assignment as in the dK/dV kernel; with a bias the dU partial row block goes to fparts.
template <int D, int RK, int NW, bool PAD>
__global__ __launch_bounds__(NW * 64, 1) void bwd_dq_win_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const uint16_t* __restrict__ dout, const float* __restrict__ lse, const float* __restrict__ delta,
    const float* __restrict__ scal, const float* __restrict__ th_row, const float* __restrict__ th_col,
    uint16_t* __restrict__ dq, float* __restrict__ partials, Geom g, int NP, LowRank lr, const float* __restrict__ fmax,
    float* __restrict__ fparts, int G) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  QSmem sm;
  sm.K = reinterpret_cast<uint16_t*>(smem_raw);
  sm.V = sm.K + NP * kRS;
  sm.sn = reinterpret_cast<float*>(sm.V + NP * kRS);
  sm.cs = sm.sn + 2 * g.M * (D / 4);
  sm.red = sm.cs + 2 * g.M * (D / 4);
  sm.lab = reinterpret_cast<uint8_t*>(sm.red + NW * (D / 2));
  const int64_t grp = xcd_order(blockIdx.x, gridDim.x);
  float fac[16];
#pragma unroll
  for (int e = 0; e < 16; ++e) fac[e] = 0.f;
  if constexpr (RK == 0) {
    const WinHead w = decode_winhead(g, grp);
    const bool masked = window_masked<PAD>(g, w, NP);
    fill_table<D>(sm.sn, sm.cs, th_row, th_col, w.h, g.M, threadIdx.x, NW * 64);
    __syncthreads();
    if (h16_window<D>(scal, grp))
      dq_body<D, RK, NW, true, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, NP, sm, w, grp, masked, lr, fac);
    else
      dq_body<D, RK, NW, false, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, NP, sm, w, grp, masked, lr, fac);
  } else {
    const int head = (int)(grp % g.heads);
    const int64_t nwin = g.B * g.nH * g.nW, wg = grp / g.heads, w0 = wg * G;
    const int nw = (int)min((int64_t)G, nwin - w0);
    const bool fh16 = factors_h16(fmax, head);
    fill_table<D>(sm.sn, sm.cs, th_row, th_col, head, g.M, threadIdx.x, NW * 64);
    __syncthreads();
    for (int i = 0; i < nw; ++i) {
      const int64_t wh = (w0 + i) * g.heads + head;
      const WinHead w = decode_winhead(g, wh);
      const bool masked = window_masked<PAD>(g, w, NP);
      if (fh16 && h16_window<D>(scal, wh))
        dq_body<D, RK, NW, true, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, NP, sm, w, wh, masked, lr, fac);
      else
        dq_body<D, RK, NW, false, PAD>(q, k, v, dout, lse, delta, scal, dq, partials, g, NP, sm, w, wh, masked, lr,
                                       fac);
    }
    store_factor_rows(fac, fparts + (wg * g.heads + head) * (int64_t)g.N * lr.rank, g.N, lr.rank);
  }
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

// Windows per workgroup of the bias kernels: enough workgroups to fill the chip (about 1024 window-heads
// per window of a group), at most 8.
int64_t windows_per_group(const Geom& g) {
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  return std::max<int64_t>(1, std::min<int64_t>(8, nwh / 1024));
}

template <int D, int RK, int NW, bool PAD>
hipError_t launch_win(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int NP = (g.N + 31) / 32 * 32;
  if (NP > NW * 32) return hipErrorInvalidConfiguration;
  static std::once_flag once_kv[64], once_q[64];
  raise_lds_limit(bwd_dkdv_win_kernel<D, RK, NW, PAD>, once_kv);
  raise_lds_limit(bwd_dq_win_kernel<D, RK, NW, PAD>, once_q);
  const int64_t nwin = g.B * g.nH * g.nW;
  const int64_t G = RK > 0 ? windows_per_group(g) : 1;
  const int64_t ngroups = (nwin + G - 1) / G;
  const int64_t blocks = ngroups * g.heads;
  const int64_t per_group = (int64_t)g.heads * g.N * a.lr.rank;  // entries of one factor
  // bias workspace: dW partials [ngroups][heads][N][rank], dU partials; from the first 256-byte
  // boundary past the float32 kernels' two [windows][heads][N][rank] blocks: the padded factors
  // [heads][N][RK] and the factor maxima
  float* wparts = a.lr_parts;
  float* uparts = RK > 0 ? a.lr_parts + ngroups * per_group : nullptr;
  float* extra = a.lr_parts + (2 * nwin * per_group + 63) / 64 * 64;
  LowRank lrp = a.lr;
  float* fmax = nullptr;
  if constexpr (RK > 0) {
    float* upad = extra;
    float* wpad = upad + (int64_t)g.heads * g.N * RK;
    fmax = wpad + (int64_t)g.heads * g.N * RK;
    hipLaunchKernelGGL(factor_prep_kernel<RK>, dim3((unsigned)g.heads), dim3(256), 0, st, a.lr.u, a.lr.w, a.lr.rank,
                       g.N, upad, wpad, fmax);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    lrp.u = upad;
    lrp.w = wpad;
  }
  hipLaunchKernelGGL((bwd_dkdv_win_kernel<D, RK, NW, PAD>), dim3((unsigned)blocks), dim3(NW * 64),
                     kv_smem_bytes<D>(NP, g.M, NW), st, (const uint16_t*)a.q, (const uint16_t*)a.k,
                     (const uint16_t*)a.v, (const uint16_t*)a.dout, a.lse, a.delta, a.scal, a.th_row, a.th_col,
                     (uint16_t*)a.dk, (uint16_t*)a.dv, a.partials, g, NP, lrp, fmax, wparts, (int)G);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_win_kernel<D, RK, NW, PAD>), dim3((unsigned)blocks), dim3(NW * 64),
                     q_smem_bytes<D>(NP, g.M, NW), st, (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v,
                     (const uint16_t*)a.dout, a.lse, a.delta, a.scal, a.th_row, a.th_col, (uint16_t*)a.dq, a.partials,
                     g, NP, lrp, fmax, uparts, (int)G);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (RK > 0) {
    e = launch_lowrank_reduce(wparts, ngroups, per_group, a.dw, st);
    if (e != hipSuccess) return e;
    e = launch_lowrank_reduce(uparts, ngroups, per_group, a.du, st);
    if (e != hipSuccess) return e;
  }
  return launch_dtheta_reduce(a.partials, a.n_partials, 2 * nwin, g, a.dth_row, a.dth_col, st);
}

template <int D, int RK, bool PAD>
hipError_t launch_win_nw(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  if (g.N <= 64) return launch_win<D, RK, 2, PAD>(a, st);
  if (g.N <= 128) return launch_win<D, RK, 4, PAD>(a, st);
  return launch_win<D, RK, 8, PAD>(a, st);
}

}  // namespace

bool bwd_d64_supported(const Geom& g) { return g.d == 64 && g.N <= kMaxNW; }

bool bwd_lowrank_mfma_supported(const Geom& g, int rank) {
  return g.d == 32 && g.N <= kMaxNW && rank >= 1 && rank <= kMaxRank && g.Hp == g.Hg && g.Wp == g.Wg;
}

int64_t bwd_window_partials(const Geom& g) { return (int64_t)g.heads * 2 * g.B * g.nH * g.nW; }

hipError_t launch_bwd_d64(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  if (!bwd_d64_supported(g)) return hipErrorInvalidValue;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  if (a.stats)
    hipLaunchKernelGGL((bwd_pre_win_kernel<64, kPreStats>), dim3((unsigned)nwh), dim3(256), 0, st,
                       (const uint16_t*)a.out, (const uint16_t*)a.dout, (const uint16_t*)a.v, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, a.delta, a.scal, const_cast<float*>(a.stats), g);
  else
    hipLaunchKernelGGL((bwd_pre_win_kernel<64, kPreFull>), dim3((unsigned)nwh), dim3(256), 0, st,
                       (const uint16_t*)a.out, (const uint16_t*)a.dout, (const uint16_t*)a.v, (const uint16_t*)a.q,
                       (const uint16_t*)a.k, a.delta, a.scal, nullptr, g);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (g.Hp != g.Hg || g.Wp != g.Wg) return launch_win_nw<64, 0, true>(a, st);  // the instances with padding checks
  return launch_win_nw<64, 0, false>(a, st);
}

hipError_t launch_operand_maxima(const FwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  if (!a.stats || a.dtype != 1 || (g.d != 32 && g.d != 64)) return hipErrorInvalidValue;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  if (g.d == 32)
    hipLaunchKernelGGL((bwd_pre_win_kernel<32, kPreMaxima>), dim3((unsigned)nwh), dim3(256), 0, st, nullptr, nullptr,
                       (const uint16_t*)a.v, (const uint16_t*)a.q, (const uint16_t*)a.k, nullptr, nullptr, a.stats, g);
  else
    hipLaunchKernelGGL((bwd_pre_win_kernel<64, kPreMaxima>), dim3((unsigned)nwh), dim3(256), 0, st, nullptr, nullptr,
                       (const uint16_t*)a.v, (const uint16_t*)a.q, (const uint16_t*)a.k, nullptr, nullptr, a.stats, g);
  return hipGetLastError();
}

hipError_t launch_bwd_lowrank_mfma(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  if (!bwd_lowrank_mfma_supported(g, a.lr.rank) || !a.lr.u || !a.lr.w || !a.du || !a.dw || !a.lr_parts)
    return hipErrorInvalidValue;
  const hipError_t e = launch_bwd_pre32(a, st);  // the d = 32 prologue: several heads per workgroup
  if (e != hipSuccess) return e;
  if (a.lr.rank <= 16) return launch_win_nw<32, 16, false>(a, st);
  return launch_win_nw<32, 32, false>(a, st);
}

}  // namespace fsw
