// bf16 window-attention forward for M = 8 windows (N = 64 tokens), d = 32, on MFMA (gfx950).
//
// Exact softmax attention inside each window with window-local 2D RoPE on Q and K (FlashSwin paper
// card, "FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision Transformers with Memory
// Efficient Attention": Abstract; Figure 1(B)).  Small windows move ~12 KB per window-head for
// ~0.5 MFLOP, so this path is bound by HBM and by load latency, not by the matrix cores.
//
// One wave owns one window-head and computes it with 16x16x32 MFMA products, which keep the
// accumulators small (4 registers per 16x16 block): the kernel fits 95 registers, so four waves
// share a SIMD.  Lane (c16, g4) = (lane % 16, lane / 16) loads channels 8 g4 .. 8 g4 + 7 of token
// 16 b + c16 of K and of Q (b = 0..3) straight into the registers that hold them as operands and
// rotates them there.  V travels from HBM into the wave's LDS buffer (global_load_lds, 16 bytes
// per lane, four lanes per row) and stays row-major for the transposed ds_read_b64_tr_b16 reads of
// the P.V product.  The queries go in four 16-query blocks: S^T of two 16-key blocks at a time,
// P = exp2(S^T - ref) taken straight from those accumulators as the B operand of P.V (in a key
// order the V operand follows), O^T in two 16-channel blocks.  The RoPE sin/cos tables of every
// head are built once per workgroup while the loads are in flight.
// The softmax reference is the Cauchy-Schwarz bound max|q^| * max|k~| of the block, widened by the
// operand rounding error (bound_margin) so that no score exceeds it, with an exact-maximum
// recomputation of a block whose row sums come out below 2^-80 or not finite.  Only windows that
// hold several Swin regions (the last window row and column of a shifted grid) run the masked code.
#include <algorithm>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"

namespace fsw {

namespace {

constexpr int kM8Waves = 4;                                 // waves (window-heads) per workgroup
constexpr int kM8MaxHeads = 32;                             // tables: heads * 1 KB of LDS
constexpr int kM8WaveLds = 64 * 32 + 32;                    // per wave, 16-bit units: V rows, labels
constexpr float kM8LowSum = 8.271806125530277e-25f;         // 2^-80
constexpr float kM8QScale = kLog2e * 0.17677669529663687f;  // log2(e) / sqrt(32)

typedef float f32x4_t __attribute__((ext_vector_type(4)));

// 16x16x32 products (gfx950): A[i][k] sits in lane i + 16 (k / 8), element k % 8; B[k][j] in lane
// j + 16 (k / 8), element k % 8; D[i][j] in lane j + 16 (i / 4), element i % 4.
template <bool H16>
__device__ __forceinline__ f32x4_t mfma16_op(uint4 a, uint4 b, const f32x4_t& c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// Issue every load of window-head wh.  Lane (c16, g4) = (lane % 16, lane / 16): K and Q of token
// 16 b + c16 of block b = 0..3, channels 8 g4 .. 8 g4 + 7 (16 bytes), into the registers that hold
// them as operands.  V: HBM -> LDS, instruction i moving 64 x 16 bytes into slots i*64 .. i*64+63
// (lane L's bytes land in slot i*64 + L: row (i*64+L)/4, 16-byte chunk (i*64+L)%4), row-major.
__device__ __forceinline__ void m8_issue(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v, const Geom& g, int64_t wh, int lane,
                                         uint16_t* vs, uint4 (&kr)[4], uint4 (&qr)[4]) {
  typedef __attribute__((address_space(3))) void lds_t;
  const WinHead w = decode_winhead(g, wh);
  const int g4 = lane >> 4, c16 = lane & 15;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int n = b * 16 + c16;
    const int64_t base = token_index(g, w.b, w.wy, w.wx, n >> 3, n & 7) * g.xs + w.h * 32 + 8 * g4;
    kr[b] = *reinterpret_cast<const uint4*>(k + base);
    qr[b] = *reinterpret_cast<const uint4*>(q + base);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = i * 64 + lane;
    const int row = slot >> 2, pc = slot & 3;
    const int64_t base = token_index(g, w.b, w.wy, w.wx, row >> 3, row & 7) * g.xs + w.h * 32;
    __builtin_amdgcn_global_load_lds((const void*)(v + base + pc * 8), (lds_t*)(vs + i * 512), 16, 0, 0);
  }
}

// The lane's 8 channels 8 g4 .. 8 g4 + 7 of token n, rotated with the head's table (channels
// [0, 16) by the row position, [16, 32) by the column position), scaled, in the operand format.
template <bool H16>
__device__ __forceinline__ uint4 m8_operand(uint4 raw, const float* sn, const float* cs, int n, int g4, float scale) {
  float x[8];
  unpack8(raw, x);
  const int axis = g4 >> 1;
  rotate8(x, sn, cs, axis, 8, axis ? (n & 7) : (n >> 3), 4 * (g4 & 1));
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= scale;
  return pack8_op(x, H16);
}

// Sum and maximum over the four lanes that share lane % 16 (the parts of one token or query).
__device__ __forceinline__ float groups_sum(float x) { return halves_sum(x + __shfl_xor(x, 16, 64)); }
__device__ __forceinline__ float groups_max(float x) { return halves_max(fmaxf(x, __shfl_xor(x, 16, 64))); }

// A operand of the P.V product for key group kg (32 keys) and channel block cb: lane (c16, g4)
// holds channel 16 cb + c16 of keys 32 kg + 4 g4 + {0..3} and 32 kg + 16 + 4 g4 + {0..3}, read
// transposed from the row-major V rows (each 16-lane group transposes a 4 x 16 block).
__device__ __forceinline__ uint4 m8_vt(const uint16_t* vbuf, int kg, int cb, int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  const uint16_t* p = vbuf + (kg * 32 + 4 * g4 + (c16 >> 2)) * 32 + cb * 16 + 4 * (c16 & 3);
  const uint2 lo = lds_read_tr16(p);
  const uint2 hi = lds_read_tr16(p + 16 * 32);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Live mask of the lane's 4 scores in key block kb (keys 16 kb + 4 g4 + {0..3}) for label qlab.
__device__ __forceinline__ uint32_t m8_live4(const uint8_t* lab, int kb, int g4, int qlab) {
  const uint32_t wd = *reinterpret_cast<const uint32_t*>(lab + kb * 16 + 4 * g4);
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e)
    if (((wd >> (8 * e)) & 0xff) == (uint32_t)qlab) bits |= 1u << e;
  return bits;
}

// Attention of one 16-query block over the window's 64 keys with softmax reference `ref`: scores
// S^T of two 16-key blocks at a time, P = exp2(S^T - ref) straight into the B operand of the P.V
// product (key slots 8 g4 + {0..3} from the first block, 8 g4 + {4..7} from the second, the same
// order as the V operand), l per lane (over its 16 keys) and O^T (two 16-channel blocks).
template <bool H16, bool MASKED>
__device__ __forceinline__ void m8_block(const uint4 (&kop)[4], uint4 qop, const uint16_t* vbuf, const uint8_t* lab,
                                         int qlab, int lane, float ref, float& l, f32x4_t (&o)[2]) {
  const int g4 = lane >> 4;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  float la = 0.f, lb = 0.f;
#pragma unroll
  for (int kg = 0; kg < 2; ++kg) {
    const f32x4_t s0 = mfma16_op<H16>(kop[2 * kg], qop, zero);
    const f32x4_t s1 = mfma16_op<H16>(kop[2 * kg + 1], qop, zero);
    float p[8];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      p[e] = __builtin_amdgcn_exp2f(s0[e] - ref);
      p[4 + e] = __builtin_amdgcn_exp2f(s1[e] - ref);
    }
    if (MASKED) {
      const uint32_t b0 = m8_live4(lab, 2 * kg, g4, qlab), b1 = m8_live4(lab, 2 * kg + 1, g4, qlab);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        p[e] = ((b0 >> e) & 1u) ? p[e] : 0.f;
        p[4 + e] = ((b1 >> e) & 1u) ? p[4 + e] : 0.f;
      }
    }
    uint32_t pk[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) pk[e] = pack2(p[2 * e], p[2 * e + 1]);
    la = add_pair(pk[0], la);
    lb = add_pair(pk[1], lb);
    la = add_pair(pk[2], la);
    lb = add_pair(pk[3], lb);
    const uint4 pb = make_uint4(pk[0], pk[1], pk[2], pk[3]);
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) o[cb] = mfma16_op<false>(m8_vt(vbuf, kg, cb, lane), pb, o[cb]);
  }
  l = la + lb;
}

// Exact row maximum of one 16-query block over the live keys (raw scores, log2 units).
template <bool H16, bool MASKED>
__device__ __forceinline__ float m8_rowmax(const uint4 (&kop)[4], uint4 qop, const uint8_t* lab, int qlab, int lane) {
  const int g4 = lane >> 4;
  const f32x4_t zero = {0.f, 0.f, 0.f, 0.f};
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    const f32x4_t s = mfma16_op<H16>(kop[kb], qop, zero);
    const uint32_t live = MASKED ? m8_live4(lab, kb, g4, qlab) : 0xfu;
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if ((live >> e) & 1u) m = fmaxf(m, s[e]);
  }
  return groups_max(m);
}

// Operands and attention of one window-head: the four 16-query blocks in turn, each with the
// exact-maximum pass when its bound was too loose, then O and LSE stores.
template <bool H16, bool MASKED>
__device__ __forceinline__ void m8_attend(const uint4 (&kr)[4], const uint4 (&qr)[4], const float* sn, const float* cs,
                                          uint16_t* __restrict__ out, float* __restrict__ lse, const Geom& g,
                                          const WinHead& w, const uint16_t* vbuf, const uint8_t* lab, float kmax,
                                          const float (&qn2)[4], int lane) {
  const int g4 = lane >> 4, c16 = lane & 15;
  uint4 kop[4];
#pragma unroll
  for (int b = 0; b < 4; ++b) kop[b] = m8_operand<H16>(kr[b], sn, cs, b * 16 + c16, g4, 1.f);
#pragma unroll
  for (int qb = 0; qb < 4; ++qb) {
    const int n = qb * 16 + c16;
    const uint4 qop = m8_operand<H16>(qr[qb], sn, cs, n, g4, kM8QScale);
    const int qlab = MASKED ? lab[n] : 0;
    // >= every computed score of this block (log2 units)
    const float bound = sqrtf(qn2[qb]) * kM8QScale * kmax * bound_margin<H16>();
    f32x4_t o[2];
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) o[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
    float l;
    m8_block<H16, MASKED>(kop, qop, vbuf, lab, qlab, lane, bound, l, o);
    float lt = groups_sum(l);
    float ref = bound;
    if (__builtin_amdgcn_ballot_w64(!(lt >= kM8LowSum && lt < INFINITY)) != 0) {
      // the bound was too loose for some query of the block: exact maximum, second pass
      ref = m8_rowmax<H16, MASKED>(kop, qop, lab, qlab, lane);
#pragma unroll
      for (int cb = 0; cb < 2; ++cb) o[cb] = f32x4_t{0.f, 0.f, 0.f, 0.f};
      m8_block<H16, MASKED>(kop, qop, vbuf, lab, qlab, lane, ref, l, o);
      lt = groups_sum(l);
    }
    // O = O^T / l (lane: query c16, channels 16 cb + 4 g4 + {0..3}), LSE = (ref + log2 l) ln 2
    const int64_t qtok = token_index(g, w.b, w.wy, w.wx, n >> 3, n & 7);
    const float inv = 1.f / lt;
    uint16_t* dst = out + qtok * g.os + w.h * 32 + 4 * g4;
#pragma unroll
    for (int cb = 0; cb < 2; ++cb) {
      uint2 pr;
      pr.x = pack2(o[cb][0] * inv, o[cb][1] * inv);
      pr.y = pack2(o[cb][2] * inv, o[cb][3] * inv);
      *reinterpret_cast<uint2*>(dst + 16 * cb) = pr;
    }
    if (lse && g4 == 0) lse[qtok * g.heads + w.h] = (ref + __log2f(lt)) * kLn2;
    __builtin_amdgcn_sched_barrier(0);  // one block at a time: bounded register pressure
  }
}

// Workgroup b (in XCD order) owns window-heads b * kM8Waves .. + kM8Waves - 1, one per wave, so a
// workgroup's waves work on neighbouring window-heads (the heads of one window share cache lines).
__global__ __launch_bounds__(kM8Waves * 64, 4) void fwd_m8_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               const float* __restrict__ th_row,
                                                               const float* __restrict__ th_col,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse,
                                                               float* __restrict__ stats, Geom g, int64_t nwh) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // [heads][2 axes][8 positions][8 pairs] sin, then cos; per wave: V rows [64][32], labels [64]
  float* tsn = reinterpret_cast<float*>(smem_raw);
  float* tcs = tsn + g.heads * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint16_t* vs = reinterpret_cast<uint16_t*>(tcs + g.heads * 128) + wave * kM8WaveLds;
  uint8_t* lab = reinterpret_cast<uint8_t*>(vs + 64 * 32);

  const int64_t wh = xcd_order(blockIdx.x, gridDim.x) * kM8Waves + wave;
  const bool active = wh < nwh;
  uint4 kr[4], qr[4];
  if (active) m8_issue(q, k, v, g, wh, lane, vs, kr, qr);  // in flight while the tables are built

  for (int i = tid; i < g.heads * 128; i += kM8Waves * 64) {
    const int head = i >> 7, axis = (i >> 6) & 1, p = (i >> 3) & 7, j = i & 7;
    const float th = axis ? th_col[head * 8 + j] : th_row[head * 8 + j];
    float s, c;
    rope_sincos(th, p, &s, &c);
    tsn[i] = s;
    tcs[i] = c;
  }
  __syncthreads();
  if (!active) return;

  const WinHead w = decode_winhead(g, wh);
  // A window holds several Swin regions exactly when the grid is shifted and the window lies in the
  // last window row or column; only then are scores masked, by the tokens' region labels.
  const bool masked = g.shift > 0 && (w.wy == g.nH - 1 || w.wx == g.nW - 1);
  if (masked) lab[lane] = (uint8_t)token_label(g, w.wy, w.wx, lane >> 3, lane & 7);
  // the wave's V transfers are complete once its vector-memory count drains (the asm also keeps
  // the compiler from moving LDS reads above it)
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");

  // norms: |k|^2 max over the 64 keys, |q|^2 max per 16-query block (rotation keeps norms)
  float kn = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) kn = fmaxf(kn, groups_sum(norm2_bf16x8(kr[b], 0.f)));
  const float kmax = sqrtf(wave_max(kn));
  float qn2[4], qm = 0.f;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    qn2[b] = wave_max(groups_sum(norm2_bf16x8(qr[b], 0.f)));
    qm = fmaxf(qm, qn2[b]);
  }
  const bool h16 = kmax < kF16Limit && sqrtf(qm) * kM8QScale < kF16Limit;
  if (stats) {  // the window-head's largest |component| of q, k (registers) and v (LDS row of the lane)
    uint32_t aq = 0, ak = 0, av = 0;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      aq = absmax_x8(aq, qr[b]);
      ak = absmax_x8(ak, kr[b]);
      av = absmax_x8(av, *reinterpret_cast<const uint4*>(vs + lane * 32 + b * 8));
    }
    const float mq = wave_max(absmax_value(aq)), mk = wave_max(absmax_value(ak)), mv = wave_max(absmax_value(av));
    if (lane == 0) {
      float* const s4 = stats + wh * 4;
      s4[0] = mq;
      s4[1] = 0.f;
      s4[2] = mk;
      s4[3] = mv;
    }
  }
  const float* sn = tsn + w.h * 128;
  const float* cs = tcs + w.h * 128;
  if (h16) {
    if (masked)
      m8_attend<true, true>(kr, qr, sn, cs, out, lse, g, w, vs, lab, kmax, qn2, lane);
    else
      m8_attend<true, false>(kr, qr, sn, cs, out, lse, g, w, vs, lab, kmax, qn2, lane);
  } else {
    if (masked)
      m8_attend<false, true>(kr, qr, sn, cs, out, lse, g, w, vs, lab, kmax, qn2, lane);
    else
      m8_attend<false, false>(kr, qr, sn, cs, out, lse, g, w, vs, lab, kmax, qn2, lane);
  }
}

}  // namespace

bool fwd_m8_supported(const Geom& g) {
  return g.M == 8 && g.d == 32 && g.heads <= kM8MaxHeads && g.Hp == g.Hg && g.Wp == g.Wg;  // no padding
}

hipError_t launch_fwd_m8(const FwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  const size_t smem = (size_t)g.heads * 128 * 4 * 2 + (size_t)kM8Waves * kM8WaveLds * 2;
  const int64_t grid = (nwh + kM8Waves - 1) / kM8Waves;
  hipLaunchKernelGGL(fwd_m8_kernel, dim3((unsigned)grid), dim3(kM8Waves * 64), smem, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.th_row, a.th_col, (uint16_t*)a.out, a.lse, a.stats,
                     g, nwh);
  return hipGetLastError();
}

}  // namespace fsw
