// bf16 window-attention forward on MFMA (gfx950), d = 32, any M <= 32.
//
// Exact softmax attention inside each window with window-local 2D RoPE on Q and K, without storing
// the score matrix (FlashSwin paper card, "FLASHSWIN: Unlocking Large Windows and Dense Tokens in
// Swin Vision Transformers with Memory Efficient Attention": Abstract; Figure 1(B)).
//
// Workgroup = (window, head, block of NWAVES*64 queries).  The window's K (rotated, bf16) and V
// (transposed) are staged once in LDS; each wave owns 64 queries (two 32-query MFMA tiles) held as
// bf16 B operands, and walks the keys in 32-key blocks: S^T = K~ Q^T (2 MFMAs), P = exp2(S^T),
// O^T += V^T P^T (2 MFMAs).  The shift and window partition are index arithmetic on the loads and
// stores; the Swin region mask is applied per element only in key blocks whose labels are mixed,
// and key blocks with no label in common with the wave are skipped.
//
// Softmax reference: softmax is unchanged by subtracting any per-row constant.  Instead of a
// running maximum, each wave subtracts the Cauchy-Schwarz bound B = max_i |q_i| * max_j |k_j| of its
// scores, folded into the MFMA accumulator initialisation (so the subtraction costs nothing), and
// the sum is accumulated without rescaling.  Every exponent is then <= 0 (no overflow).  If a
// query's sum comes out below 2^-80 (a bound so loose that small terms could underflow), the wave
// recomputes its tiles with the exact row maximum in a second pass; results are exact either way.
#include <algorithm>
#include <mutex>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"

namespace fsw {

namespace {

constexpr float kLowSum = 8.271806125530277e-25f;  // 2^-80

struct FwdSmem {
  uint16_t* K;     // [NP][kKStride]
  uint16_t* Vt;    // [32][NP + 8]
  float* sn;       // [2][M][8]  sin of RoPE angle (row axis, column axis)
  float* cs;       // [2][M][8]  cos
  uint8_t* lab;    // [NP]  key labels, 0xff past the window
  uint32_t* blk;   // [NP/32]  bits 0..8: labels present, bit 9: all 32 keys valid
  float* red;      // [16]: per-wave max |k~|^2 (0..7), max |q^|^2 (8..15)
};

__host__ __device__ inline size_t fwd_smem_bytes(int NP, int M) {
  size_t b = (size_t)NP * kKStride * 2 + (size_t)32 * vt_stride(NP) * 2;
  b += (size_t)2 * 2 * M * 8 * 4;
  b += (size_t)NP;
  b = (b + 3) & ~(size_t)3;
  b += (size_t)(NP / 32) * 4 + 16 * 4;
  return b;
}

__device__ inline FwdSmem carve(unsigned char* base, int NP, int M) {
  FwdSmem s;
  s.K = reinterpret_cast<uint16_t*>(base);
  s.Vt = s.K + (size_t)NP * kKStride;
  s.sn = reinterpret_cast<float*>(s.Vt + (size_t)32 * vt_stride(NP));
  s.cs = s.sn + 2 * M * 8;
  s.lab = reinterpret_cast<uint8_t*>(s.cs + 2 * M * 8);
  size_t off = ((size_t)(s.lab + NP - base) + 3) & ~(size_t)3;
  s.blk = reinterpret_cast<uint32_t*>(base + off);
  s.red = reinterpret_cast<float*>(s.blk + NP / 32);
  return s;
}

// One pass over the key blocks for the wave's two query tiles.
//  MODE 0: scores offset by the accumulator init `cinit`; p = exp2(s); accumulate l and O.
//  MODE 1: exact maximum only: m[t] = max over live keys of the raw score.
//  MODE 2: p = exp2(s - m[t]) with the exact per-query maximum; accumulate l and O.
// H16: the score operands (K~ rows in LDS, Q^ in registers) are fp16, else bf16.
template <int MODE, bool H16>
__device__ __forceinline__ void key_pass(const FwdSmem& sm, int NB, int lane, uint32_t wave_labels, bool wave_single,
                                         const uint4 (&qb)[2][2], const int (&qlab)[2], const f32x16_t& cinit,
                                         float (&m)[2], float (&l)[2], f32x16_t (&o)[2]) {
  const int h = lane >> 5;
  const int row = lane & 31;
  const int vst = vt_stride(NB * 32);
  for (int kb = 0; kb < NB; ++kb) {
    const uint32_t info = sm.blk[kb];
    const uint32_t bl = info & 0x1ffu;
    if ((bl & wave_labels) == 0) continue;  // no query of this wave may see these keys
    const bool need_mask = !((info >> 9) & 1u) || !wave_single || bl != wave_labels;
    const uint16_t* krow = sm.K + (size_t)(kb * 32 + row) * kKStride + 8 * h;
    const uint4 ka0 = *reinterpret_cast<const uint4*>(krow);
    const uint4 ka1 = *reinterpret_cast<const uint4*>(krow + 16);
    f32x16_t s[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      s[t] = mfma_op<H16>(ka0, qb[t][0], cinit);
      s[t] = mfma_op<H16>(ka1, qb[t][1], s[t]);
    }
    uint32_t live[2] = {0xffffu, 0xffffu};
    if (need_mask) {
#pragma unroll
      for (int t = 0; t < 2; ++t) live[t] = live_bits(sm.lab, kb, h, qlab[t]);
    }
    if (MODE == 1) {
#pragma unroll
      for (int t = 0; t < 2; ++t) {
#pragma unroll
        for (int v = 0; v < 16; ++v)
          if ((live[t] >> v) & 1u) m[t] = fmaxf(m[t], s[t][v]);
      }
      continue;
    }
    const uint16_t* vrow = sm.Vt + (size_t)row * vst + kb * 32 + 8 * h;
    const bf16x8_t va0 = as_bf16x8(*reinterpret_cast<const uint4*>(vrow));
    const bf16x8_t va1 = as_bf16x8(*reinterpret_cast<const uint4*>(vrow + 16));
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      float p[16];
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const float x = (MODE == 2) ? s[t][v] - m[t] : s[t][v];
        p[v] = __builtin_amdgcn_exp2f(x);
      }
      if (need_mask) {
#pragma unroll
        for (int v = 0; v < 16; ++v) p[v] = ((live[t] >> v) & 1u) ? p[v] : 0.f;
      }
      uint32_t pk[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pk[e] = pack2(p[2 * e], p[2 * e + 1]);
      float acc0 = l[t], acc1 = 0.f;
#pragma unroll
      for (int e = 0; e < 8; e += 2) {
        acc0 = add_pair(pk[e], acc0);
        acc1 = add_pair(pk[e + 1], acc1);
      }
      l[t] = acc0 + acc1;
      const uint4 b0 = make_uint4(pk[0], pk[1], pk[2], pk[3]);
      const uint4 b1 = make_uint4(pk[4], pk[5], pk[6], pk[7]);
      o[t] = mfma32x32x16(va0, as_bf16x8(b0), o[t]);
      o[t] = mfma32x32x16(va1, as_bf16x8(b1), o[t]);
    }
  }
}

// Stage the rotated K~ rows of the window into LDS in fp16 (h16) or bf16; returns this thread's
// max |k~|^2 over the keys it staged (float32 values before rounding).
__device__ inline float stage_k_rows(const FwdSmem& sm, const uint16_t* __restrict__ k, const Geom& g,
                                     const WinHead& w, int NP, int tid, int nt, bool h16) {
  constexpr int D = 32;
  const int M = g.M, N = g.N;
  const int64_t rowstride = (int64_t)g.heads * D;
  float kmax2 = 0.f;
  for (int it = tid; it < NP * 4; it += nt) {
    const int key = it >> 2;
    const int part = it & 3;
    uint4 kr = make_uint4(0, 0, 0, 0);
    float ss = 0.f;
    if (key < N) {
      const int r = key / M, c = key - (key / M) * M;
      const int64_t off = token_index(g, w.b, w.wy, w.wx, r, c) * rowstride + w.h * D + part * 8;
      float x[8];
      unpack8(*reinterpret_cast<const uint4*>(k + off), x);
      const int axis = part >> 1;
      rotate8(x, sm.sn, sm.cs, axis, M, axis ? c : r, (part & 1) * 4);
      kr = pack8_op(x, h16);
#pragma unroll
      for (int e = 0; e < 8; ++e) ss = __builtin_fmaf(x[e], x[e], ss);
    }
    *reinterpret_cast<uint4*>(sm.K + (size_t)key * kKStride + part * 8) = kr;
    ss += __shfl_xor(ss, 1, 64);
    ss += __shfl_xor(ss, 2, 64);
    kmax2 = fmaxf(kmax2, ss);
  }
  return kmax2;
}

// Main pass with the bound as softmax reference, then the exact-maximum fallback if needed.
template <bool H16>
__device__ __forceinline__ void attend(const FwdSmem& sm, int NB, int lane, uint32_t wave_labels, bool wave_single,
                                       const uint4 (&qb)[2][2], const int (&qlab)[2], const bool (&qvalid)[2],
                                       float bound, float (&ref)[2], float (&l)[2], f32x16_t (&o)[2]) {
  f32x16_t cinit;
#pragma unroll
  for (int v2 = 0; v2 < 16; ++v2) cinit[v2] = -bound;
  float m[2] = {-bound, -bound};
  if (wave_labels != 0) key_pass<0, H16>(sm, NB, lane, wave_labels, wave_single, qb, qlab, cinit, m, l, o);
  ref[0] = ref[1] = bound;
  bool low = false;
#pragma unroll
  for (int t = 0; t < 2; ++t) low |= qvalid[t] && !(l[t] + __shfl_xor(l[t], 32, 64) >= kLowSum);
  if (__builtin_amdgcn_ballot_w64(low) != 0) {
    f32x16_t zero;
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) zero[v2] = 0.f;
    m[0] = m[1] = -INFINITY;
    key_pass<1, H16>(sm, NB, lane, wave_labels, wave_single, qb, qlab, zero, m, l, o);
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      m[t] = fmaxf(m[t], __shfl_xor(m[t], 32, 64));
      if (!(m[t] > -INFINITY)) m[t] = 0.f;  // invalid query lanes
      l[t] = 0.f;
#pragma unroll
      for (int v2 = 0; v2 < 16; ++v2) o[t][v2] = 0.f;
    }
    key_pass<2, H16>(sm, NB, lane, wave_labels, wave_single, qb, qlab, zero, m, l, o);
    ref[0] = m[0];
    ref[1] = m[1];
  }
}

template <int NWAVES>
__global__ __launch_bounds__(NWAVES * 64) void fwd_mfma_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               const float* __restrict__ th_row,
                                                               const float* __restrict__ th_col,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse,
                                                               Geom g, int nqb, int NP) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int D = 32;
  constexpr int NT = NWAVES * 64;
  const int M = g.M;
  const int N = g.N;
  const int NB = NP / 32;
  const FwdSmem sm = carve(smem_raw, NP, M);

  const int64_t blk = blockIdx.x;
  const WinHead w = decode_winhead(g, blk / nqb);
  const int qblock = (int)(blk % nqb);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int64_t rowstride = (int64_t)g.heads * D;
  const int h = lane >> 5;
  const int col = lane & 31;

  // 1. RoPE sin/cos table and key labels
  for (int i = tid; i < 2 * M * 8; i += NT) {
    const int axis = i / (M * 8);
    const int p = (i / 8) % M;
    const int j = i % 8;
    const float th = axis ? th_col[w.h * 8 + j] : th_row[w.h * 8 + j];
    float s, c;
    rope_sincos(th, p, &s, &c);
    sm.sn[i] = s;
    sm.cs[i] = c;
  }
  for (int n = tid; n < NP; n += NT) {
    uint8_t lb = 0xff;
    if (n < N) lb = (uint8_t)token_label(g, w.wy, w.wx, n / M, n % M);
    sm.lab[n] = lb;
  }
  __syncthreads();

  // 2. stage K~ (rotated, fp16) and V^T (bf16, keys in vt_pos order); track max |k~|^2
  float kmax2 = stage_k_rows(sm, k, g, w, NP, tid, NT, true);
  for (int it = tid; it < NP * 4; it += NT) {
    const int key = it >> 2;
    const int part = it & 3;
    uint4 vr = make_uint4(0, 0, 0, 0);
    if (key < N) {
      const int r = key / M, c = key - (key / M) * M;
      const int64_t off = token_index(g, w.b, w.wy, w.wx, r, c) * rowstride + w.h * D + part * 8;
      vr = *reinterpret_cast<const uint4*>(v + off);
    }
    const int pos = vt_pos(key);
    const uint32_t vw[4] = {vr.x, vr.y, vr.z, vr.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      sm.Vt[(size_t)(part * 8 + 2 * e) * vt_stride(NP) + pos] = (uint16_t)(vw[e] & 0xffffu);
      sm.Vt[(size_t)(part * 8 + 2 * e + 1) * vt_stride(NP) + pos] = (uint16_t)(vw[e] >> 16);
    }
  }
  // block label summaries
  for (int b = tid; b < NB; b += NT) {
    uint32_t bits = 0, full = 1;
    for (int j = 0; j < 32; ++j) {
      const uint8_t lb = sm.lab[b * 32 + j];
      if (lb == 0xff)
        full = 0;
      else
        bits |= 1u << lb;
    }
    sm.blk[b] = bits | (full << 9);
  }

  // 3. the wave's queries (two 32-query tiles): raw loads, labels and |q^| (rotation keeps norms)
  const float qscale = kLog2e * 0.17677669529663687f;  // log2(e) / sqrt(32)
  uint4 qraw[2][2];
  int qlab[2], qr[2], qc[2];
  bool qvalid[2];
  int64_t qtok[2];
  float qn2max = 0.f;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int qi = qblock * NT + wave * 64 + t * 32 + col;
    qvalid[t] = qi < N;
    qlab[t] = 0xff;
    qtok[t] = 0;
    qr[t] = qc[t] = 0;
    qraw[t][0] = qraw[t][1] = make_uint4(0, 0, 0, 0);
    float n2 = 0.f;
    if (qvalid[t]) {
      qr[t] = qi / M;
      qc[t] = qi - qr[t] * M;
      qtok[t] = token_index(g, w.b, w.wy, w.wx, qr[t], qc[t]);
      qlab[t] = token_label(g, w.wy, w.wx, qr[t], qc[t]);
      const int64_t off = qtok[t] * rowstride + w.h * D;
      qraw[t][0] = *reinterpret_cast<const uint4*>(q + off + 8 * h);
      qraw[t][1] = *reinterpret_cast<const uint4*>(q + off + 16 + 8 * h);
      float x[8], y[8];
      unpack8(qraw[t][0], x);
      unpack8(qraw[t][1], y);
#pragma unroll
      for (int e = 0; e < 8; ++e) n2 = __builtin_fmaf(x[e], x[e], __builtin_fmaf(y[e], y[e], n2));
    }
    n2 += __shfl_xor(n2, 32, 64);
    qn2max = fmaxf(qn2max, n2);
  }
  qn2max = wave_max(qn2max) * (qscale * qscale);
  kmax2 = wave_max(kmax2);
  if (lane == 0) {
    sm.red[wave] = kmax2;
    sm.red[8 + wave] = qn2max;
  }
  __syncthreads();
  float kmax2_all = 0.f, qmax2_all = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    kmax2_all = fmaxf(kmax2_all, sm.red[i]);
    qmax2_all = fmaxf(qmax2_all, sm.red[8 + i]);
  }
  const float kmax = sqrtf(kmax2_all);
  // fp16 score operands unless some |k~| or |q^| (hence some component) could leave fp16 range
  const bool h16 = kmax < kF16Limit && sqrtf(qmax2_all) < kF16Limit;
  if (!h16) {
    __syncthreads();
    stage_k_rows(sm, k, g, w, NP, tid, NT, false);
    __syncthreads();
  }

  uint4 qb[2][2];
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    float x[8], y[8];
    unpack8(qraw[t][0], x);
    unpack8(qraw[t][1], y);
    rotate8(x, sm.sn, sm.cs, 0, M, qr[t], 4 * h);
    rotate8(y, sm.sn, sm.cs, 1, M, qc[t], 4 * h);
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      x[e] *= qscale;
      y[e] *= qscale;
    }
    qb[t][0] = pack8_op(x, h16);
    qb[t][1] = pack8_op(y, h16);
  }
  const float bound = sqrtf(qn2max) * kmax;  // >= every score of this wave (log2 units)
  uint32_t wl = 0;
#pragma unroll
  for (int t = 0; t < 2; ++t)
    if (qvalid[t]) wl |= 1u << qlab[t];
  const uint32_t wave_labels = wave_or(wl);
  const bool wave_single = __builtin_popcount(wave_labels) == 1;

  f32x16_t o[2];
  float l[2] = {0.f, 0.f};
  float ref[2];
#pragma unroll
  for (int t = 0; t < 2; ++t)
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) o[t][v2] = 0.f;
  if (h16)
    attend<true>(sm, NB, lane, wave_labels, wave_single, qb, qlab, qvalid, bound, ref, l, o);
  else
    attend<false>(sm, NB, lane, wave_labels, wave_single, qb, qlab, qvalid, bound, ref, l, o);

  // 4. epilogue: O = O^T / l (lane: query col, channels 8g + 4h + j), LSE = (ref + log2 l) ln 2
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const float lt = l[t] + __shfl_xor(l[t], 32, 64);
    if (!qvalid[t]) continue;
    const float inv = 1.f / lt;
    uint16_t* dst = out + qtok[t] * rowstride + w.h * D + 4 * h;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint2 pr;
      pr.x = pack2(o[t][4 * gq] * inv, o[t][4 * gq + 1] * inv);
      pr.y = pack2(o[t][4 * gq + 2] * inv, o[t][4 * gq + 3] * inv);
      *reinterpret_cast<uint2*>(dst + 8 * gq) = pr;
    }
    if (lse && h == 0) lse[qtok[t] * g.heads + w.h] = (ref[t] + __log2f(lt)) * kLn2;
  }
}

template <int NWAVES>
hipError_t launch_nw(const FwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int NP = (g.N + 31) / 32 * 32;
  const int nqb = (g.N + NWAVES * 64 - 1) / (NWAVES * 64);
  const size_t smem = fwd_smem_bytes(NP, g.M);
  static std::once_flag once;
  std::call_once(once, [] {
    (void)hipFuncSetAttribute((const void*)fwd_mfma_kernel<NWAVES>, hipFuncAttributeMaxDynamicSharedMemorySize,
                              160 * 1024);
  });
  const int64_t blocks = g.B * g.nH * g.nW * g.heads * nqb;
  hipLaunchKernelGGL(fwd_mfma_kernel<NWAVES>, dim3((unsigned)blocks), dim3(NWAVES * 64), smem, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.th_row, a.th_col,
                     (uint16_t*)a.out, a.lse, g, nqb, NP);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st) {
  const int N = a.g.N;
  if (N <= 64) return launch_nw<1>(a, st);
  if (N <= 128) return launch_nw<2>(a, st);
  if (N <= 256) return launch_nw<4>(a, st);
  return launch_nw<8>(a, st);
}

}  // namespace fsw
