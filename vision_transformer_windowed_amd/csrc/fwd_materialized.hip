// Materialized window attention (bf16, d = 32): the standard Swin route that FlashSwin replaces, kept as
// an on-device comparison of memory and time against the fused kernels.
//
// Standard Swin window attention materializes the M^2 x M^2 score matrix of every window, adds the
// learned relative-position bias elementwise, takes the softmax and multiplies by V; its memory grows
// as O(M^4) per window, which is what FlashSwin removes (FlashSwin paper card, "FLASHSWIN: Unlocking
// Large Windows and Dense Tokens in Swin Vision Transformers with Memory Efficient Attention":
// Abstract; Figure 1(C) and Table S1 for memory against M, Figure S1 for throughput).  Here the same
// attention as the fused path (window-local 2D RoPE on Q and K, Swin's shift and region mask), with an
// optional relative-position bias table, runs as three kernels with the scores in HBM:
//   1. scores: S = q~ . k~ / sqrt(d) (+ bias) on MFMA, masked pairs -inf, float32 rows of NP = N
//      rounded up to 32 entries per query (the padding entries -inf); slots are row-major, n = r*M + c;
//   2. softmax: one wave per row reads it whole, writes P = exp(S - max) / sum as bf16 over the first
//      half of the same row, and LSE;
//   3. P.V: O^T = V^T P^T on MFMA, V staged in LDS, P read from HBM.
// The workspace holds the score rows: window-heads x N x NP x 4 bytes.
#include <algorithm>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"

namespace fsw {

namespace {

constexpr float kMatScale = 0.17677669529663687f;  // 1 / sqrt(32)

// ---------------------------------------------------------------------------------------- scores

// Workgroup = one window-head and 4 query tiles of 32 (one per wave); the head's RoPE sin/cos table is
// built in LDS.  A wave rotates its 32 queries once (lane l: query qt*32 + l%32, channels 8h.. and
// 16+8h.., h = l/32, in float32) and walks the key tiles: the lanes load and rotate key kt*32 + l%32,
// the score tile S^T = K~ Q^T (fp16 operands when every rotated component of the pair of tiles fits,
// else bf16) leaves each lane the 16 scores of its query with keys kt*32 + 8g + 4h + j, which it writes
// with the bias added and masked pairs at -inf.
constexpr int kScWaves = 4;
__global__ __launch_bounds__(kScWaves * 64) void mat_scores_kernel(const uint16_t* __restrict__ q,
                                                                   const uint16_t* __restrict__ k,
                                                                   const float* __restrict__ th_row,
                                                                   const float* __restrict__ th_col,
                                                                   const float* __restrict__ bias,
                                                                   float* __restrict__ S, Geom g, int NB,
                                                                   int qgroups) {
  __shared__ float tsn[2 * 32 * 8], tcs[2 * 32 * 8];
  const int64_t wh = blockIdx.x / qgroups;
  const int qg = (int)(blockIdx.x - wh * qgroups);
  const WinHead w = decode_winhead(g, wh);
  const int M = g.M, N = g.N, NP = NB * 32;
  for (int i = threadIdx.x; i < 2 * M * 8; i += kScWaves * 64) {
    const int axis = i / (M * 8), p = (i / 8) % M, j = i % 8;
    float sv, cv;
    rope_sincos(axis ? th_col[w.h * 8 + j] : th_row[w.h * 8 + j], p, &sv, &cv);
    tsn[i] = sv;
    tcs[i] = cv;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qt = qg * kScWaves + wave;
  if (qt >= NB) return;  // whole wave
  const int h = lane >> 5, col = lane & 31;

  // channels 8h..8h+7 (row axis, pairs 4h..) and 16+8h.. (column axis, pairs 4h..) of slot n, rotated
  auto operand = [&](const uint16_t* x, int n, float scale, float (&a)[8], float (&b)[8]) {
#pragma unroll
    for (int e = 0; e < 8; ++e) a[e] = b[e] = 0.f;
    if (n >= N) return;
    const int r = n / M, c = n - (n / M) * M;
    const int64_t off = token_index(g, w.b, w.wy, w.wx, r, c) * g.xs + w.h * 32;
    unpack8(*reinterpret_cast<const uint4*>(x + off + 8 * h), a);
    unpack8(*reinterpret_cast<const uint4*>(x + off + 16 + 8 * h), b);
    rotate8(a, tsn, tcs, 0, M, r, 4 * h);
    rotate8(b, tsn, tcs, 1, M, c, 4 * h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      a[e] *= scale;
      b[e] *= scale;
    }
  };
  const int qi = qt * 32 + col;
  float qa[8], qb[8];
  operand(q, qi, kMatScale, qa, qb);
  float qmx = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) qmx = fmaxf(qmx, fmaxf(fabsf(qa[e]), fabsf(qb[e])));
  const int qr = qi / M, qc = qi - (qi / M) * M;
  const int qlab = qi < N ? token_label(g, w.wy, w.wx, qr, qc) : -1;
  float* row = S + (wh * N + min(qi, N - 1)) * (int64_t)NP + 4 * h;
  for (int kt = 0; kt < NB; ++kt) {
    float ka[8], kb[8];
    operand(k, kt * 32 + col, 1.f, ka, kb);
    float mx = qmx;
#pragma unroll
    for (int e = 0; e < 8; ++e) mx = fmaxf(mx, fmaxf(fabsf(ka[e]), fabsf(kb[e])));
    const bool h16 = __builtin_amdgcn_ballot_w64(!(mx < kF16Limit)) == 0;
    f32x16_t s;
#pragma unroll
    for (int e = 0; e < 16; ++e) s[e] = 0.f;
    if (h16) {
      s = mfma_op<true>(pack8_op(ka, true), pack8_op(qa, true), s);
      s = mfma_op<true>(pack8_op(kb, true), pack8_op(qb, true), s);
    } else {
      s = mfma_op<false>(pack8_op(ka, false), pack8_op(qa, false), s);
      s = mfma_op<false>(pack8_op(kb, false), pack8_op(qb, false), s);
    }
    if (qi >= N) continue;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      float4 o;
      float* ov = &o.x;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int key = kt * 32 + 8 * gq + 4 * h + j;
        float val = -INFINITY;
        if (key < N) {
          const int kr = key / M, kc = key - (key / M) * M;
          if (token_label(g, w.wy, w.wx, kr, kc) == qlab) {
            val = s[4 * gq + j];
            if (bias) val += bias[((int64_t)w.h * (2 * M - 1) + (qr - kr + M - 1)) * (2 * M - 1) + (qc - kc + M - 1)];
          }
        }
        ov[j] = val;
      }
      *reinterpret_cast<float4*>(row + kt * 32 + 8 * gq) = o;
    }
  }
}

// --------------------------------------------------------------------------------------- softmax

// One wave per score row (query qi of window-head wh), four rows per workgroup.  The row's NP <= 1024
// floats are read whole into registers before P (bf16, normalised) overwrites its first 2*NP bytes.
template <int PER>  // floats per lane: NP / 64 rounded up
__global__ __launch_bounds__(256) void mat_softmax_kernel(float* __restrict__ S, float* __restrict__ lse, Geom g, int NP,
                                                          int64_t nrows) {
  const int lane = threadIdx.x & 63;
  const int64_t rowi = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (rowi >= nrows) return;
  float* row = S + rowi * NP;
  float x[PER];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = i * 64 + lane;
    x[i] = j < NP ? row[j] : -INFINITY;
    m = fmaxf(m, x[i]);
  }
  m = wave_max(m);
  float sum = 0.f;
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    x[i] = __expf(x[i] - m);
    sum += x[i];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) sum += __shfl_xor(sum, o, 64);
  const float inv = 1.f / sum;
  uint16_t* p = reinterpret_cast<uint16_t*>(row);
  // every lane has read its values (and the shuffles above made the wave wait for them) before any write
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int j = i * 64 + lane;
    if (j < NP) p[j] = float_to_bf16_bits(x[i] * inv);
  }
  if (lse && lane == 0) {
    const int64_t wh = rowi / g.N;
    const int qi = (int)(rowi - wh * g.N);
    const WinHead w = decode_winhead(g, wh);
    const int qr = qi / g.M, qc = qi - (qi / g.M) * g.M;
    lse[token_index(g, w.b, w.wy, w.wx, qr, qc) * g.heads + w.h] = m + __logf(sum);
  }
}

// ------------------------------------------------------------------------------------------- P.V

// Workgroup = one window-head and 8 query tiles of 32 (8 waves); the window's V rows are staged in LDS
// ([NP][32] bf16, zero past N).  Lane l holds O^T for query qt*32 + l%32, channels 8g + 4h + j; per 16
// keys the B operand is P of keys 4h + {0..3} and 8 + 4h + {0..3} (the order tr_operand presents V^T).
constexpr int kPvWaves = 8;
__global__ __launch_bounds__(kPvWaves * 64) void mat_pv_kernel(const float* __restrict__ S,
                                                               const uint16_t* __restrict__ v,
                                                               uint16_t* __restrict__ out, Geom g, int NB,
                                                               int qgroups) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  uint16_t* Vs = reinterpret_cast<uint16_t*>(smem_raw);
  const int NP = NB * 32;
  const int64_t wh = blockIdx.x / qgroups;
  const int qg = (int)(blockIdx.x - wh * qgroups);
  const WinHead w = decode_winhead(g, wh);
  const int M = g.M, N = g.N;
  for (int it = threadIdx.x; it < NP * 4; it += kPvWaves * 64) {
    const int key = it >> 2, part = it & 3;
    uint4 val = make_uint4(0, 0, 0, 0);
    if (key < N) {
      const int r = key / M, c = key - (key / M) * M;
      val = *reinterpret_cast<const uint4*>(v + token_index(g, w.b, w.wy, w.wx, r, c) * g.xs + w.h * 32 + part * 8);
    }
    *reinterpret_cast<uint4*>(Vs + key * 32 + part * 8) = val;
  }
  __syncthreads();
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int qt = qg * kPvWaves + wave;
  if (qt >= NB) return;
  const int h = lane >> 5, col = lane & 31;
  const int qi = qt * 32 + col;
  const uint16_t* prow = reinterpret_cast<const uint16_t*>(S + (wh * N + std::min(qi, N - 1)) * (int64_t)NP);
  f32x16_t o;
#pragma unroll
  for (int e = 0; e < 16; ++e) o[e] = 0.f;
  for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const int k0 = kb * 32 + half * 16;
      const uint2 lo = *reinterpret_cast<const uint2*>(prow + k0 + 4 * h);
      const uint2 hi = *reinterpret_cast<const uint2*>(prow + k0 + 8 + 4 * h);
      const uint4 pb = make_uint4(lo.x, lo.y, hi.x, hi.y);
      o = mfma32x32x16(as_bf16x8(tr_operand(Vs, 32, k0, lane)), as_bf16x8(pb), o);
    }
  }
  if (qi >= N) return;
  const int qr = qi / M, qc = qi - (qi / M) * M;
  uint16_t* dst = out + token_index(g, w.b, w.wy, w.wx, qr, qc) * g.os + w.h * 32 + 4 * h;
#pragma unroll
  for (int gq = 0; gq < 4; ++gq) {
    uint2 pr;
    pr.x = pack2(o[4 * gq], o[4 * gq + 1]);
    pr.y = pack2(o[4 * gq + 2], o[4 * gq + 3]);
    *reinterpret_cast<uint2*>(dst + 8 * gq) = pr;
  }
}

template <int PER>
hipError_t launch_softmax(float* S, float* lse, const Geom& g, int NP, int64_t nrows, hipStream_t st) {
  hipLaunchKernelGGL((mat_softmax_kernel<PER>), dim3((unsigned)((nrows + 3) / 4)), dim3(256), 0, st, S, lse, g, NP,
                     nrows);
  return hipGetLastError();
}

}  // namespace

size_t materialized_workspace_bytes(const Geom& g) {
  const int64_t NP = (g.N + 31) / 32 * 32;
  return (size_t)(g.B * g.nH * g.nW * g.heads) * (size_t)g.N * (size_t)NP * sizeof(float);
}

hipError_t launch_fwd_materialized(const FwdArgs& a, const float* bias, void* workspace, hipStream_t st) {
  const Geom& g = a.g;
  const int NB = (g.N + 31) / 32, NP = NB * 32;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  float* S = static_cast<float*>(workspace);
  const int sgroups = (NB + kScWaves - 1) / kScWaves;
  hipLaunchKernelGGL(mat_scores_kernel, dim3((unsigned)(nwh * sgroups)), dim3(kScWaves * 64), 0, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, a.th_row, a.th_col, bias, S, g, NB, sgroups);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t nrows = nwh * g.N;
  if (NP <= 64)
    e = launch_softmax<1>(S, a.lse, g, NP, nrows, st);
  else if (NP <= 256)
    e = launch_softmax<4>(S, a.lse, g, NP, nrows, st);
  else
    e = launch_softmax<16>(S, a.lse, g, NP, nrows, st);
  if (e != hipSuccess) return e;
  const int qgroups = (NB + kPvWaves - 1) / kPvWaves;
  const size_t smem = (size_t)NP * 32 * 2;
  if (smem > 64 * 1024) {
    e = hipFuncSetAttribute((const void*)mat_pv_kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(mat_pv_kernel, dim3((unsigned)(nwh * qgroups)), dim3(kPvWaves * 64), smem, st, (const float*)S,
                     (const uint16_t*)a.v, (uint16_t*)a.out, g, NB, qgroups);
  return hipGetLastError();
}

}  // namespace fsw
