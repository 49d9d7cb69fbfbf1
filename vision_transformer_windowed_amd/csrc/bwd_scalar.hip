// Generic window-attention backward: float32 arithmetic, recomputation from the saved LSE.
//
// Backward of exact window attention with window-local 2D RoPE (FlashSwin paper card, "FLASHSWIN:
// Unlocking Large Windows and Dense Tokens in Swin Vision Transformers with Memory Efficient
// Attention": Abstract, flat training memory in M; Table S1).  P is never stored: every kernel
// recomputes it as exp(S - LSE).  With Delta_i = sum_d dO_i O_i:
//   dV_j = sum_i P_ij dO_i,   dS_ij = P_ij (dO_i . V_j - Delta_i),
//   dq~_i = sum_j dS_ij k~_j / sqrt(d),   dk~_j = sum_i dS_ij q~_i / sqrt(d),
//   dq = R^T dq~, dk = R^T dk~, and for a rotated pair (a, b) at angle theta * p,
//   dtheta += p (dx~_b x~_a - dx~_a x~_b) over all Q and K tokens.
// With a rank-r bias U[n_i] . W[n_j] on the scores (the FlashBias factorization on the same paper card,
// Table S1), dW[n_j] = sum_i dS_ij U[n_i] and dU[n_i] = sum_j dS_ij W[n_j] per window: the dK/dV and dQ
// kernels write them per window and position, and a last kernel sums the windows in a fixed order.
// Three kernels: Delta; dK/dV with one thread per key; dQ with one thread per query.  Padding tokens
// of a padded grid are neither queries nor keys (no loads, no stores, no dtheta terms).  The theta
// gradient is reduced per workgroup in a fixed order into a partials buffer, then summed over
// workgroups in a fixed order, so results are bit-reproducible.
#include <algorithm>

#include "fsw_common.h"
#include "fsw_launch.h"

namespace fsw {

constexpr int kBwdThreads = 128;

// Delta[t, h] = sum_d dO[t, h, d] * O[t, h, d]
template <typename IO, int D>
__global__ __launch_bounds__(256) void bwd_delta_kernel(const IO* __restrict__ out, const IO* __restrict__ dout,
                                                        float* __restrict__ delta, int64_t rows) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < rows; i += stride) {
    float o[D], g[D];
    load_row<D>(out + i * D, o);
    load_row<D>(dout + i * D, g);
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < D; ++e) s = __builtin_fmaf(o[e], g[e], s);
    delta[i] = s;
  }
}

// Fixed-order workgroup reduction of each thread's D/2 dtheta terms into one partials row.
template <int D>
__device__ __forceinline__ void reduce_dtheta_block(float (&t)[D / 2], float* dst) {
  __shared__ float red[kBwdThreads][D / 2 + 1];
  const int tid = threadIdx.x;
  __syncthreads();
#pragma unroll
  for (int e = 0; e < D / 2; ++e) red[tid][e] = t[e];
  __syncthreads();
  for (int half = kBwdThreads / 2; half > 0; half >>= 1) {
    if (tid < half) {
#pragma unroll
      for (int e = 0; e < D / 2; ++e) red[tid][e] += red[tid + half][e];
    }
    __syncthreads();
  }
  if (tid < D / 2) dst[tid] = red[0][tid];
}

// Per-pair dtheta terms of one token: p * (dx_b * x_a - dx_a * x_b), row pairs then column pairs.
template <int D>
__device__ __forceinline__ void dtheta_terms(const float (&x)[D], const float (&dx)[D], int r, int c, float (&t)[D / 2]) {
#pragma unroll
  for (int j = 0; j < D / 4; ++j) {
    t[j] += (float)r * (dx[2 * j + 1] * x[2 * j] - dx[2 * j] * x[2 * j + 1]);
    t[D / 4 + j] += (float)c * (dx[D / 2 + 2 * j + 1] * x[D / 2 + 2 * j] - dx[D / 2 + 2 * j] * x[D / 2 + 2 * j + 1]);
  }
}

// Partials layout: [heads][2 kernels][windows * blocks_per_windowhead][D/2].
__device__ __forceinline__ int64_t partial_row(const Geom& g, int64_t blk, int nb, int which) {
  const int64_t wh = blk / nb;
  const int h = (int)(wh % g.heads);
  const int64_t win = wh / g.heads;
  const int64_t per_head = g.B * g.nH * g.nW * nb;
  return ((int64_t)h * 2 + which) * per_head + win * nb + (blk % nb);
}

template <typename IO, int D, bool LR>
__global__ __launch_bounds__(kBwdThreads) void bwd_dkdv_scalar_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v, const IO* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, const float* __restrict__ th_row,
    const float* __restrict__ th_col, IO* __restrict__ dk, IO* __restrict__ dv, float* __restrict__ partials, Geom g,
    int nb, LowRank lr, float* __restrict__ wparts) {
  constexpr int R = LR ? kMaxRank : 1;
  __shared__ float sQ[kBwdThreads][D];  // q~ * log2(e) / sqrt(d)
  __shared__ float sG[kBwdThreads][D];  // dO
  __shared__ float sL[kBwdThreads];     // lse * log2(e)
  __shared__ float sDel[kBwdThreads];
  __shared__ float sU[LR ? kBwdThreads : 1][R];  // the queries' U rows
  __shared__ int sLab[kBwdThreads];

  const int64_t blk = blockIdx.x;
  const WinHead w = decode_winhead(g, blk / nb);
  const int tid = threadIdx.x;
  const int N = g.N;
  const int j = (int)(blk % nb) * kBwdThreads + tid;
  const bool active = j < N && token_real(g, w.wy, w.wx, j / g.M, j % g.M);  // padding is no key
  const float* tr = th_row + w.h * (D / 4);
  const float* tc = th_col + w.h * (D / 4);
  const int64_t xs = g.xs, os = g.os;
  const float qscale = kLog2e * rsqrtf((float)D);

  float kt[D], vv[D];
  float wk[R], dwk[R];  // the key's W row times log2(e), and its gradient
#pragma unroll
  for (int t = 0; t < R; ++t) wk[t] = dwk[t] = 0.f;
  int klab = -2, kr = 0, kc = 0;
  int64_t ktok = 0;
  if (active) {
    if (LR) {
      const float* wrow = lr.w + ((int64_t)w.h * N + j) * lr.rank;
#pragma unroll
      for (int t = 0; t < R; ++t)
        if (t < lr.rank) wk[t] = wrow[t] * kLog2e;
    }
    kr = j / g.M;
    kc = j - kr * g.M;
    ktok = token_index(g, w.b, w.wy, w.wx, kr, kc);
    load_row<D>(k + ktok * xs + w.h * D, kt);
    load_row<D>(v + ktok * xs + w.h * D, vv);
    rope_rotate<D>(kt, tr, tc, kr, kc);
    klab = token_label(g, w.wy, w.wx, kr, kc);
  } else {
#pragma unroll
    for (int e = 0; e < D; ++e) kt[e] = vv[e] = 0.f;
  }
  float dkt[D], dvv[D];
#pragma unroll
  for (int e = 0; e < D; ++e) dkt[e] = dvv[e] = 0.f;

  for (int t0 = 0; t0 < N; t0 += kBwdThreads) {
    __syncthreads();
    {
      const int i = t0 + tid;
      if (i < N && token_real(g, w.wy, w.wx, i / g.M, i % g.M)) {
        const int r = i / g.M, c = i - (i / g.M) * g.M;
        const int64_t tok = token_index(g, w.b, w.wy, w.wx, r, c);
        float qv[D], gv[D];
        load_row<D>(q + tok * xs + w.h * D, qv);
        load_row<D>(dout + tok * os + w.h * D, gv);
        rope_rotate<D>(qv, tr, tc, r, c);
#pragma unroll
        for (int e = 0; e < D; ++e) {
          sQ[tid][e] = qv[e] * qscale;
          sG[tid][e] = gv[e];
        }
        sL[tid] = lse[tok * g.heads + w.h] * kLog2e;
        sDel[tid] = delta[tok * g.heads + w.h];
        sLab[tid] = token_label(g, w.wy, w.wx, r, c);
        if (LR) {
          const float* urow = lr.u + ((int64_t)w.h * N + i) * lr.rank;
#pragma unroll
          for (int t = 0; t < R; ++t) sU[tid][t] = t < lr.rank ? urow[t] : 0.f;
        }
      } else {
        sLab[tid] = -1;
      }
    }
    __syncthreads();
    const int tn = min(kBwdThreads, N - t0);
    for (int i = 0; i < tn; ++i) {
      if (sLab[i] != klab) continue;
      float s2 = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        s2 = __builtin_fmaf(sQ[i][e], kt[e], s2);
        dp = __builtin_fmaf(sG[i][e], vv[e], dp);
      }
      if (LR) {
#pragma unroll
        for (int t = 0; t < R; ++t) s2 = __builtin_fmaf(sU[i][t], wk[t], s2);
      }
      const float p = exp2f(s2 - sL[i]);
      const float ds = p * (dp - sDel[i]) * kLn2;  // dS / log2(e), pairs with the log2(e) in sQ
#pragma unroll
      for (int e = 0; e < D; ++e) {
        dvv[e] = __builtin_fmaf(p, sG[i][e], dvv[e]);
        dkt[e] = __builtin_fmaf(ds, sQ[i][e], dkt[e]);
      }
      if (LR) {
        const float dsn = p * (dp - sDel[i]);  // dS
#pragma unroll
        for (int t = 0; t < R; ++t) dwk[t] = __builtin_fmaf(dsn, sU[i][t], dwk[t]);
      }
    }
  }

  float terms[D / 2];
#pragma unroll
  for (int e = 0; e < D / 2; ++e) terms[e] = 0.f;
  if (active) {
    dtheta_terms<D>(kt, dkt, kr, kc, terms);
    rope_unrotate<D>(dkt, tr, tc, kr, kc);
    store_row<D>(dk + ktok * xs + w.h * D, dkt);
    store_row<D>(dv + ktok * xs + w.h * D, dvv);
  }
  if (LR && j < N) {  // this window's dW row of position j (zero for padding)
    float* dst = wparts + ((blk / nb) * N + j) * lr.rank;
#pragma unroll
    for (int t = 0; t < R; ++t)
      if (t < lr.rank) dst[t] = dwk[t];
  }
  reduce_dtheta_block<D>(terms, partials + partial_row(g, blk, nb, 0) * (D / 2));
}

template <typename IO, int D, bool LR>
__global__ __launch_bounds__(kBwdThreads) void bwd_dq_scalar_kernel(
    const IO* __restrict__ q, const IO* __restrict__ k, const IO* __restrict__ v, const IO* __restrict__ dout,
    const float* __restrict__ lse, const float* __restrict__ delta, const float* __restrict__ th_row,
    const float* __restrict__ th_col, IO* __restrict__ dq, float* __restrict__ partials, Geom g, int nb, LowRank lr,
    float* __restrict__ uparts) {
  constexpr int R = LR ? kMaxRank : 1;
  __shared__ float sK[kBwdThreads][D];  // k~
  __shared__ float sV[kBwdThreads][D];
  __shared__ float sW[LR ? kBwdThreads : 1][R];  // the keys' W rows
  __shared__ int sLab[kBwdThreads];

  const int64_t blk = blockIdx.x;
  const WinHead w = decode_winhead(g, blk / nb);
  const int tid = threadIdx.x;
  const int N = g.N;
  const int i = (int)(blk % nb) * kBwdThreads + tid;
  const bool active = i < N && token_real(g, w.wy, w.wx, i / g.M, i % g.M);  // padding is no query
  const float* tr = th_row + w.h * (D / 4);
  const float* tc = th_col + w.h * (D / 4);
  const int64_t xs = g.xs, os = g.os;
  const float qscale = kLog2e * rsqrtf((float)D);
  const float kscale = rsqrtf((float)D);

  float qt[D], qs[D], gv[D];
  float uq[R], duq[R];  // the query's U row times log2(e), and its gradient
#pragma unroll
  for (int t = 0; t < R; ++t) uq[t] = duq[t] = 0.f;
  float l2 = 0.f, del = 0.f;
  int qlab = -2, qr = 0, qc = 0;
  int64_t qtok = 0;
  if (active) {
    if (LR) {
      const float* urow = lr.u + ((int64_t)w.h * N + i) * lr.rank;
#pragma unroll
      for (int t = 0; t < R; ++t)
        if (t < lr.rank) uq[t] = urow[t] * kLog2e;
    }
    qr = i / g.M;
    qc = i - qr * g.M;
    qtok = token_index(g, w.b, w.wy, w.wx, qr, qc);
    load_row<D>(q + qtok * xs + w.h * D, qt);
    load_row<D>(dout + qtok * os + w.h * D, gv);
    rope_rotate<D>(qt, tr, tc, qr, qc);
    l2 = lse[qtok * g.heads + w.h] * kLog2e;
    del = delta[qtok * g.heads + w.h];
    qlab = token_label(g, w.wy, w.wx, qr, qc);
  } else {
#pragma unroll
    for (int e = 0; e < D; ++e) qt[e] = gv[e] = 0.f;
  }
#pragma unroll
  for (int e = 0; e < D; ++e) qs[e] = qt[e] * qscale;
  float dqt[D];
#pragma unroll
  for (int e = 0; e < D; ++e) dqt[e] = 0.f;

  for (int t0 = 0; t0 < N; t0 += kBwdThreads) {
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
        for (int e = 0; e < D; ++e) {
          sK[tid][e] = kv[e];
          sV[tid][e] = vv[e];
        }
        sLab[tid] = token_label(g, w.wy, w.wx, r, c);
        if (LR) {
          const float* wrow = lr.w + ((int64_t)w.h * N + j) * lr.rank;
#pragma unroll
          for (int t = 0; t < R; ++t) sW[tid][t] = t < lr.rank ? wrow[t] : 0.f;
        }
      } else {
        sLab[tid] = -1;
      }
    }
    __syncthreads();
    const int tn = min(kBwdThreads, N - t0);
    for (int j = 0; j < tn; ++j) {
      if (sLab[j] != qlab) continue;
      float s2 = 0.f, dp = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) {
        s2 = __builtin_fmaf(qs[e], sK[j][e], s2);
        dp = __builtin_fmaf(gv[e], sV[j][e], dp);
      }
      if (LR) {
#pragma unroll
        for (int t = 0; t < R; ++t) s2 = __builtin_fmaf(uq[t], sW[j][t], s2);
      }
      const float p = exp2f(s2 - l2);
      const float ds = p * (dp - del) * kscale;
#pragma unroll
      for (int e = 0; e < D; ++e) dqt[e] = __builtin_fmaf(ds, sK[j][e], dqt[e]);
      if (LR) {
        const float dsn = p * (dp - del);  // dS
#pragma unroll
        for (int t = 0; t < R; ++t) duq[t] = __builtin_fmaf(dsn, sW[j][t], duq[t]);
      }
    }
  }

  float terms[D / 2];
#pragma unroll
  for (int e = 0; e < D / 2; ++e) terms[e] = 0.f;
  if (active) {
    dtheta_terms<D>(qt, dqt, qr, qc, terms);
    rope_unrotate<D>(dqt, tr, tc, qr, qc);
    store_row<D>(dq + qtok * xs + w.h * D, dqt);
  }
  if (LR && i < N) {  // this window's dU row of position i (zero for padding)
    float* dst = uparts + ((blk / nb) * N + i) * lr.rank;
#pragma unroll
    for (int t = 0; t < R; ++t)
      if (t < lr.rank) dst[t] = duq[t];
  }
  reduce_dtheta_block<D>(terms, partials + partial_row(g, blk, nb, 1) * (D / 2));
}

// Factor gradients: out[e] = sum over rows r of parts[r][e] (parts laid out [rows][heads][N][rank]).
// A workgroup takes 16 entries; thread (slice s, entry) sums rows s, s + 16, ... in order, then thread
// s = 0 adds the 16 slice sums in order.
__global__ __launch_bounds__(256) void lowrank_reduce_kernel(const float* __restrict__ parts, int64_t nrows,
                                                             int64_t per_row, float* __restrict__ out) {
  __shared__ float red[16][16];
  const int el = threadIdx.x & 15, sl = threadIdx.x >> 4;
  const int64_t e = (int64_t)blockIdx.x * 16 + el;
  float s = 0.f;
  if (e < per_row)
    for (int64_t r = sl; r < nrows; r += 16) s += parts[r * per_row + e];
  red[sl][el] = s;
  __syncthreads();
  if (sl == 0 && e < per_row) {
    float t = 0.f;
#pragma unroll
    for (int i = 0; i < 16; ++i) t += red[i][el];
    out[e] = t;
  }
}

// Sum the partial rows of one (head, pair-slot) in a fixed order: thread t takes rows t, t+256, ...
// then a fixed tree over the 256 threads.  Grid: heads * (D/2) workgroups.
__global__ __launch_bounds__(256) void dtheta_reduce_kernel(const float* __restrict__ partials, int64_t rows_per_head,
                                                            int half_d, int quarter_d, float* __restrict__ dth_row,
                                                            float* __restrict__ dth_col) {
  __shared__ float red[256];
  const int h = blockIdx.x / half_d;
  const int e = blockIdx.x % half_d;
  const float* base = partials + (int64_t)h * rows_per_head * half_d + e;
  float s = 0.f;
  for (int64_t r = threadIdx.x; r < rows_per_head; r += 256) s += base[r * half_d];
  red[threadIdx.x] = s;
  __syncthreads();
  for (int half = 128; half > 0; half >>= 1) {
    if ((int)threadIdx.x < half) red[threadIdx.x] += red[threadIdx.x + half];
    __syncthreads();
  }
  if (threadIdx.x == 0) {
    if (e < quarter_d)
      dth_row[h * quarter_d + e] = red[0];
    else
      dth_col[h * quarter_d + e - quarter_d] = red[0];
  }
}

hipError_t launch_lowrank_reduce(const float* parts, int64_t nrows, int64_t per_row, float* out, hipStream_t st) {
  if (per_row <= 0) return hipSuccess;
  hipLaunchKernelGGL(lowrank_reduce_kernel, dim3((unsigned)((per_row + 15) / 16)), dim3(256), 0, st, parts, nrows,
                     per_row, out);
  return hipGetLastError();
}

hipError_t launch_dtheta_reduce(const float* partials, int64_t n_partials, int64_t rows_per_head, const Geom& g,
                                float* dth_row, float* dth_col, hipStream_t st) {
  (void)n_partials;
  hipLaunchKernelGGL(dtheta_reduce_kernel, dim3(g.heads * (g.d / 2)), dim3(256), 0, st, partials, rows_per_head,
                     g.d / 2, g.d / 4, dth_row, dth_col);
  return hipGetLastError();
}

int64_t bwd_scalar_partials(const Geom& g) {
  const int64_t nb = (g.N + kBwdThreads - 1) / kBwdThreads;
  return (int64_t)g.heads * 2 * g.B * g.nH * g.nW * nb;
}

template <typename IO, int D>
static hipError_t launch_bwd_scalar_t(const BwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int64_t rows = g.B * g.Hg * g.Wg * g.heads;
  const int64_t dblocks = std::min<int64_t>((rows + 255) / 256, 65536);
  hipLaunchKernelGGL((bwd_delta_kernel<IO, D>), dim3((unsigned)dblocks), dim3(256), 0, st, (const IO*)a.out,
                     (const IO*)a.dout, a.delta, rows);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int nb = (g.N + kBwdThreads - 1) / kBwdThreads;
  const int64_t nwin = g.B * g.nH * g.nW;
  const int64_t blocks = nwin * g.heads * nb;
  const int64_t per_win = (int64_t)g.heads * g.N * a.lr.rank;  // entries of one factor
  float* wparts = a.lr_parts;
  float* uparts = a.lr.rank > 0 ? a.lr_parts + nwin * per_win : nullptr;
  if (a.lr.rank > 0)
    hipLaunchKernelGGL((bwd_dkdv_scalar_kernel<IO, D, true>), dim3((unsigned)blocks), dim3(kBwdThreads), 0, st,
                       (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, (const IO*)a.dout, a.lse, a.delta, a.th_row,
                       a.th_col, (IO*)a.dk, (IO*)a.dv, a.partials, g, nb, a.lr, wparts);
  else
    hipLaunchKernelGGL((bwd_dkdv_scalar_kernel<IO, D, false>), dim3((unsigned)blocks), dim3(kBwdThreads), 0, st,
                       (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, (const IO*)a.dout, a.lse, a.delta, a.th_row,
                       a.th_col, (IO*)a.dk, (IO*)a.dv, a.partials, g, nb, a.lr, wparts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.lr.rank > 0)
    hipLaunchKernelGGL((bwd_dq_scalar_kernel<IO, D, true>), dim3((unsigned)blocks), dim3(kBwdThreads), 0, st,
                       (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, (const IO*)a.dout, a.lse, a.delta, a.th_row,
                       a.th_col, (IO*)a.dq, a.partials, g, nb, a.lr, uparts);
  else
    hipLaunchKernelGGL((bwd_dq_scalar_kernel<IO, D, false>), dim3((unsigned)blocks), dim3(kBwdThreads), 0, st,
                       (const IO*)a.q, (const IO*)a.k, (const IO*)a.v, (const IO*)a.dout, a.lse, a.delta, a.th_row,
                       a.th_col, (IO*)a.dq, a.partials, g, nb, a.lr, uparts);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.lr.rank > 0) {
    e = launch_lowrank_reduce(wparts, nwin, per_win, a.dw, st);
    if (e != hipSuccess) return e;
    e = launch_lowrank_reduce(uparts, nwin, per_win, a.du, st);
    if (e != hipSuccess) return e;
  }
  const int64_t rows_per_head = 2 * g.B * g.nH * g.nW * nb;
  return launch_dtheta_reduce(a.partials, a.n_partials, rows_per_head, g, a.dth_row, a.dth_col, st);
}

hipError_t launch_bwd_scalar(const BwdArgs& a, hipStream_t st) {
  const bool bf = a.dtype == 1;
  switch (a.g.d) {
    case 8: return bf ? launch_bwd_scalar_t<uint16_t, 8>(a, st) : launch_bwd_scalar_t<float, 8>(a, st);
    case 16: return bf ? launch_bwd_scalar_t<uint16_t, 16>(a, st) : launch_bwd_scalar_t<float, 16>(a, st);
    case 32: return bf ? launch_bwd_scalar_t<uint16_t, 32>(a, st) : launch_bwd_scalar_t<float, 32>(a, st);
    case 64: return bf ? launch_bwd_scalar_t<uint16_t, 64>(a, st) : launch_bwd_scalar_t<float, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fsw
