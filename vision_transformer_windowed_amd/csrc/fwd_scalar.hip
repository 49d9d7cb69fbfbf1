// Generic window-attention forward: one thread per query, float32 arithmetic, streamed keys.
//
// Exact softmax window attention with window-local 2D RoPE on Q and K, computed with an online
// softmax so no score matrix is stored (FlashSwin paper card, "FLASHSWIN: Unlocking Large Windows
// and Dense Tokens in Swin Vision Transformers with Memory Efficient Attention": Abstract and
// Figure 1(B)).  This path serves float32 tensors (all arithmetic in float32, no reduced-precision
// products) and every (M, d) the MFMA path does not cover, and grids padded to a multiple of M
// (padding tokens are neither queries nor keys).  Keys are staged per tile in LDS after rotation;
// each thread keeps its query's running max, running sum and output accumulator in registers.
// With LR it also adds a rank-r bias U[n_i] . W[n_j] to every score (the learned low-rank bias
// factorization of the FlashBias comparison model on the same paper card, Table S1): the query's U
// row lives in registers (zero past the rank), the keys' W rows are staged beside K.
#include "fsw_common.h"
#include "fsw_launch.h"

namespace fsw {

constexpr int kScalarThreads = 128;  // queries per workgroup == keys per LDS tile
constexpr int kChunk = 16;           // scores held in registers between max updates

template <typename IO, int D, bool LR>
__global__ __launch_bounds__(kScalarThreads) void fwd_scalar_kernel(const IO* __restrict__ q, const IO* __restrict__ k,
                                                                     const IO* __restrict__ v,
                                                                     const float* __restrict__ th_row,
                                                                     const float* __restrict__ th_col,
                                                                     IO* __restrict__ out, float* __restrict__ lse,
                                                                     Geom g, int nqb, LowRank lr) {
  constexpr int R = LR ? kMaxRank : 1;
  __shared__ float sK[kScalarThreads][D];
  __shared__ float sV[kScalarThreads][D];
  __shared__ float sW[LR ? kScalarThreads : 1][R];
  __shared__ int sLab[kScalarThreads];

  const int64_t blk = blockIdx.x;
  const WinHead w = decode_winhead(g, blk / nqb);
  const int qb = (int)(blk % nqb);
  const int tid = threadIdx.x;
  const int N = g.N;
  const int n = qb * kScalarThreads + tid;
  const bool active = n < N && token_real(g, w.wy, w.wx, n / g.M, n % g.M);
  const float* tr = th_row + w.h * (D / 4);
  const float* tc = th_col + w.h * (D / 4);
  const int64_t xs = g.xs, os = g.os;

  float qv[D];
  float ub[R];  // the query's U row times log2(e) (scores are kept in log2 units)
#pragma unroll
  for (int t = 0; t < R; ++t) ub[t] = 0.f;
  int qlab = 0;
  int64_t qtok = 0;
  if (active) {
    if (LR) {
      const float* urow = lr.u + ((int64_t)w.h * N + n) * lr.rank;
#pragma unroll
      for (int t = 0; t < R; ++t)
        if (t < lr.rank) ub[t] = urow[t] * kLog2e;
    }
    const int r = n / g.M, c = n - (n / g.M) * g.M;
    qtok = token_index(g, w.b, w.wy, w.wx, r, c);
    load_row<D>(q + qtok * xs + w.h * D, qv);
    rope_rotate<D>(qv, tr, tc, r, c);
    const float sc = kLog2e * rsqrtf((float)D);
#pragma unroll
    for (int i = 0; i < D; ++i) qv[i] *= sc;
    qlab = token_label(g, w.wy, w.wx, r, c);
  } else {
#pragma unroll
    for (int i = 0; i < D; ++i) qv[i] = 0.f;
  }

  float acc[D];
#pragma unroll
  for (int i = 0; i < D; ++i) acc[i] = 0.f;
  float m = -INFINITY, l = 0.f;

  for (int t0 = 0; t0 < N; t0 += kScalarThreads) {
    __syncthreads();
    {
      const int j = t0 + tid;
      if (j < N && token_real(g, w.wy, w.wx, j / g.M, j % g.M)) {
        const int r = j / g.M, c = j - (j / g.M) * g.M;
        const int64_t tok = token_index(g, w.b, w.wy, w.wx, r, c);
        float kv[D], vv[D];
        load_row<D>(k + tok * xs + w.h * D, kv);
        load_row<D>(v + tok * xs + w.h * D, vv);
        rope_rotate<D>(kv, tr, tc, r, c);
#pragma unroll
        for (int i = 0; i < D; ++i) {
          sK[tid][i] = kv[i];
          sV[tid][i] = vv[i];
        }
        sLab[tid] = token_label(g, w.wy, w.wx, r, c);
        if (LR) {
          const float* wrow = lr.w + ((int64_t)w.h * N + j) * lr.rank;
#pragma unroll
          for (int t = 0; t < R; ++t) sW[tid][t] = t < lr.rank ? wrow[t] : 0.f;
        }
      } else {
        // past the end of the window, or padding: never matches a query label; zero rows keep 0 * row
        // finite
#pragma unroll
        for (int i = 0; i < D; ++i) {
          sK[tid][i] = 0.f;
          sV[tid][i] = 0.f;
        }
        if (LR) {
#pragma unroll
          for (int t = 0; t < R; ++t) sW[tid][t] = 0.f;
        }
        sLab[tid] = -1;
      }
    }
    __syncthreads();
    const int tn = min(kScalarThreads, N - t0);
    for (int c0 = 0; c0 < tn; c0 += kChunk) {
      float s[kChunk];
      float cmax = -INFINITY;
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int j = c0 + u;
        float dot = 0.f;
        if (j < tn && sLab[j] == qlab) {
#pragma unroll
          for (int i = 0; i < D; ++i) dot = __builtin_fmaf(qv[i], sK[j][i], dot);
          if (LR) {
#pragma unroll
            for (int t = 0; t < R; ++t) dot = __builtin_fmaf(ub[t], sW[j][t], dot);
          }
        } else {
          dot = -INFINITY;
        }
        s[u] = dot;
        cmax = fmaxf(cmax, dot);
      }
      if (cmax == -INFINITY) continue;  // every key of the chunk masked for this query
      if (cmax > m) {
        const float alpha = exp2f(m - cmax);  // m == -inf gives 0
        l *= alpha;
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] *= alpha;
        m = cmax;
      }
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const float p = exp2f(s[u] - m);  // masked: exp2(-inf) = 0
        l += p;
        const int j = min(c0 + u, kScalarThreads - 1);
#pragma unroll
        for (int i = 0; i < D; ++i) acc[i] = __builtin_fmaf(p, sV[j][i], acc[i]);
      }
    }
  }

  if (active) {
    const float inv = 1.f / l;
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] *= inv;
    store_row<D>(out + qtok * os + w.h * D, acc);
    if (lse) lse[qtok * g.heads + w.h] = m * kLn2 + logf(l);
  }
}

template <typename IO, int D>
static hipError_t launch_fwd_scalar_t(const FwdArgs& a, hipStream_t st) {
  const int nqb = (a.g.N + kScalarThreads - 1) / kScalarThreads;
  const int64_t nwh = a.g.B * a.g.nH * a.g.nW * a.g.heads;
  const int64_t blocks = nwh * nqb;
  if (a.lr.rank > 0)
    hipLaunchKernelGGL((fwd_scalar_kernel<IO, D, true>), dim3((unsigned)blocks), dim3(kScalarThreads), 0, st,
                       (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.th_row, a.th_col, (IO*)a.out, a.lse, a.g, nqb,
                       a.lr);
  else
    hipLaunchKernelGGL((fwd_scalar_kernel<IO, D, false>), dim3((unsigned)blocks), dim3(kScalarThreads), 0, st,
                       (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, a.th_row, a.th_col, (IO*)a.out, a.lse, a.g, nqb,
                       a.lr);
  return hipGetLastError();
}

hipError_t launch_fwd_scalar(const FwdArgs& a, hipStream_t st) {
  const bool bf = a.dtype == 1;
  switch (a.g.d) {
    case 8: return bf ? launch_fwd_scalar_t<uint16_t, 8>(a, st) : launch_fwd_scalar_t<float, 8>(a, st);
    case 16: return bf ? launch_fwd_scalar_t<uint16_t, 16>(a, st) : launch_fwd_scalar_t<float, 16>(a, st);
    case 32: return bf ? launch_fwd_scalar_t<uint16_t, 32>(a, st) : launch_fwd_scalar_t<float, 32>(a, st);
    case 64: return bf ? launch_fwd_scalar_t<uint16_t, 64>(a, st) : launch_fwd_scalar_t<float, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fsw
