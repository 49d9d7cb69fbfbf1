// bf16 window-attention forward for M = 8 windows (N = 64 tokens), d = 32, on MFMA (gfx950).
//
// Exact softmax attention inside each window with window-local 2D RoPE on Q and K (FlashSwin paper
// card, "FLASHSWIN: Unlocking Large Windows and Dense Tokens in Swin Vision Transformers with Memory
// Efficient Attention": Abstract; Figure 1(B)).  Small windows move ~12 KB per window-head for
// ~0.5 MFLOP, so this path is bound by HBM and by load latency, not by the matrix cores.
//
// One wave owns one window-head.  Q and K are loaded straight into the registers that hold them as
// MFMA operands (lane = token, the two 16-byte channel chunks a lane half needs; the two halves
// together read each 64-byte head row whole) and rotated there: the 64 keys become two A blocks
// (lane = key), the 64 queries two B tiles (lane = query).  V travels from HBM into the wave's LDS
// buffer (global_load_lds, 16 bytes per lane, four lanes per row) and stays row-major for the
// transposed ds_read_b64_tr_b16 reads of the P.V product.  With 4 KB of LDS per wave, four waves
// share a SIMD (at most 128 registers each).  The RoPE sin/cos tables of every head are built once
// per workgroup while the loads are in flight.
// The softmax reference is the Cauchy-Schwarz bound max|q^| * max|k~| of the tile, with an
// exact-maximum recomputation of a tile whose row sums come out below 2^-80.  Only windows that hold
// several Swin regions (the last window row and column of a shifted grid) run the masked code.
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

__device__ __forceinline__ uint32_t uniform_u32(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)x);
}

// Issue every load of window-head wh.  K and Q: the lane's token n = t * 32 + (lane % 32) of tile
// t, channel chunks h and 2 + h (h = lane / 32), into registers.  V: HBM -> LDS, instruction i
// moving 64 x 16 bytes into slots i*64 .. i*64+63 (lane L's bytes land in slot i*64 + L: row
// (i*64+L)/4, 16-byte chunk (i*64+L)%4), row-major.
__device__ __forceinline__ void m8_issue(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                         const uint16_t* __restrict__ v, const Geom& g, int64_t wh, int lane,
                                         uint16_t* vs, uint4 (&kr)[2][2], uint4 (&qr)[2][2]) {
  typedef __attribute__((address_space(3))) void lds_t;
  const WinHead w = decode_winhead(g, wh);
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = t * 32 + col;
    const int64_t base = token_index(g, w.b, w.wy, w.wx, n >> 3, n & 7) * g.xs + w.h * 32;
    kr[t][0] = *reinterpret_cast<const uint4*>(k + base + 8 * h);
    kr[t][1] = *reinterpret_cast<const uint4*>(k + base + 16 + 8 * h);
    qr[t][0] = *reinterpret_cast<const uint4*>(q + base + 8 * h);
    qr[t][1] = *reinterpret_cast<const uint4*>(q + base + 16 + 8 * h);
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int slot = i * 64 + lane;
    const int row = slot >> 2, pc = slot & 3;
    const int64_t base = token_index(g, w.b, w.wy, w.wx, row >> 3, row & 7) * g.xs + w.h * 32;
    __builtin_amdgcn_global_load_lds((const void*)(v + base + pc * 8), (lds_t*)(vs + i * 512), 16, 0, 0);
  }
}

// 8 channels of one lane, rotated with the head's table (row axis: part 0, column axis: part 1;
// pairs 4h .. 4h+3), scaled, packed to the operand format.
template <bool H16>
__device__ __forceinline__ uint4 m8_rotate(uint4 raw, const float* sn, const float* cs, int axis, int pos, int h,
                                           float scale) {
  float x[8];
  unpack8(raw, x);
  rotate8(x, sn, cs, axis, 8, pos, 4 * h);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= scale;
  return pack8_op(x, H16);
}

// Sum of squares of the 16 channels a lane holds for one token (halves add across h afterwards):
// bf16 pair dot products on the raw words (the products are exact in float32).
__device__ __forceinline__ float m8_norm2(uint4 a, uint4 b) {
  const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  float s0 = 0.f, s1 = 0.f;
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e]), __builtin_bit_cast(bf16x2_t, w[e]), s0,
                                         false);
    s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w[e + 1]),
                                         __builtin_bit_cast(bf16x2_t, w[e + 1]), s1, false);
  }
  return s0 + s1;
}

// Attention of one query tile over the window's two key blocks with softmax reference `ref` (the
// tile's bound, or a query's exact row maximum); returns l (per lane half) and O^T.
template <bool H16, bool MASKED>
__device__ __forceinline__ void m8_tile(const uint4 (&kop)[2][2], uint4 qa, uint4 qb, const uint16_t* vbuf,
                                        const uint8_t* lab, int qlab, int lane, float ref, float& l, f32x16_t& o) {
  const int h = lane >> 5;
  f32x16_t zero;
#pragma unroll
  for (int e = 0; e < 16; ++e) zero[e] = 0.f;
  float la = 0.f, lb = 0.f;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    // the reference is subtracted on the VALU (memory-bound path: registers matter more than ALU)
    f32x16_t s = mfma_op<H16>(kop[kb][0], qa, zero);
    s = mfma_op<H16>(kop[kb][1], qb, s);
    float p[16];
    if (MASKED) {
      const uint32_t live = live_bits(lab, kb, h, qlab);
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const float x = __builtin_amdgcn_exp2f(s[e] - ref);
        p[e] = ((live >> e) & 1u) ? x : 0.f;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 16; ++e) p[e] = __builtin_amdgcn_exp2f(s[e] - ref);
    }
    uint32_t pk[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pk[e] = pack2(p[2 * e], p[2 * e + 1]);
#pragma unroll
    for (int e = 0; e < 8; e += 2) {
      la = add_pair(pk[e], la);
      lb = add_pair(pk[e + 1], lb);
    }
    o = mfma32x32x16(as_bf16x8(tr_operand(vbuf, 32, kb * 32, lane)), as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3])),
                     o);
    o = mfma32x32x16(as_bf16x8(tr_operand(vbuf, 32, kb * 32 + 16, lane)),
                     as_bf16x8(make_uint4(pk[4], pk[5], pk[6], pk[7])), o);
  }
  l = la + lb;
}

// Exact row maximum of one query tile over the live keys (raw scores, log2 units).
template <bool H16, bool MASKED>
__device__ __forceinline__ float m8_rowmax(const uint4 (&kop)[2][2], uint4 qa, uint4 qb, const uint8_t* lab,
                                           int qlab, int lane) {
  const int h = lane >> 5;
  f32x16_t zero;
#pragma unroll
  for (int e = 0; e < 16; ++e) zero[e] = 0.f;
  float m = -INFINITY;
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    f32x16_t s = mfma_op<H16>(kop[kb][0], qa, zero);
    s = mfma_op<H16>(kop[kb][1], qb, s);
    const uint32_t live = MASKED ? live_bits(lab, kb, h, qlab) : 0xffffu;
#pragma unroll
    for (int e = 0; e < 16; ++e)
      if ((live >> e) & 1u) m = fmaxf(m, s[e]);
  }
  return halves_max(m);
}

// Both query tiles: attention, exact-maximum pass when needed, O and LSE stores.
template <bool H16, bool MASKED>
__device__ __forceinline__ void m8_attend(const uint4 (&kop)[2][2], const uint4 (&qop)[2][2],
                                          uint16_t* __restrict__ out, float* __restrict__ lse, const Geom& g,
                                          const WinHead& w, const uint16_t* vbuf, const uint8_t* lab, float kmax,
                                          const float (&qn2)[2], int lane) {
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = t * 32 + col;
    const int qr = n >> 3, qc = n & 7;
    const int qlab = MASKED ? lab[n] : 0;
    const float bound = sqrtf(qn2[t]) * kM8QScale * kmax;  // >= every score of this tile (log2 units)
    f32x16_t o;
#pragma unroll
    for (int e = 0; e < 16; ++e) o[e] = 0.f;
    float l;
    m8_tile<H16, MASKED>(kop, qop[t][0], qop[t][1], vbuf, lab, qlab, lane, bound, l, o);
    float lt = halves_sum(l);
    float ref = bound;
    if (__builtin_amdgcn_ballot_w64(!(lt >= kM8LowSum)) != 0) {
      // the bound was too loose for some query of the tile: exact maximum, second pass
      ref = m8_rowmax<H16, MASKED>(kop, qop[t][0], qop[t][1], lab, qlab, lane);
#pragma unroll
      for (int e = 0; e < 16; ++e) o[e] = 0.f;
      m8_tile<H16, MASKED>(kop, qop[t][0], qop[t][1], vbuf, lab, qlab, lane, ref, l, o);
      lt = halves_sum(l);
    }
    // O = O^T / l (lane: query col, channels 8g + 4h + j), LSE = (ref + log2 l) ln 2
    const int64_t qtok = token_index(g, w.b, w.wy, w.wx, qr, qc);
    const float inv = 1.f / lt;
    uint16_t* dst = out + qtok * g.os + w.h * 32 + 4 * h;
#pragma unroll
    for (int gq = 0; gq < 4; ++gq) {
      uint2 pr;
      pr.x = pack2(o[4 * gq] * inv, o[4 * gq + 1] * inv);
      pr.y = pack2(o[4 * gq + 2] * inv, o[4 * gq + 3] * inv);
      *reinterpret_cast<uint2*>(dst + 8 * gq) = pr;
    }
    if (lse && h == 0) lse[qtok * g.heads + w.h] = (ref + __log2f(lt)) * kLn2;
    __builtin_amdgcn_sched_barrier(0);  // one tile at a time: bounded register pressure
  }
}

// Rotated operands from the raw rows: keys as A blocks, queries (scaled by log2(e)/sqrt(d)) as
// B tiles; token n = tile * 32 + col sits at position (n / 8, n % 8).
template <bool H16>
__device__ __forceinline__ void m8_operands(const uint4 (&kr)[2][2], const uint4 (&qr)[2][2], const float* sn,
                                            const float* cs, int lane, uint4 (&kop)[2][2], uint4 (&qop)[2][2]) {
  const int h = lane >> 5, col = lane & 31;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int n = t * 32 + col;
    kop[t][0] = m8_rotate<H16>(kr[t][0], sn, cs, 0, n >> 3, h, 1.f);
    kop[t][1] = m8_rotate<H16>(kr[t][1], sn, cs, 1, n & 7, h, 1.f);
    qop[t][0] = m8_rotate<H16>(qr[t][0], sn, cs, 0, n >> 3, h, kM8QScale);
    qop[t][1] = m8_rotate<H16>(qr[t][1], sn, cs, 1, n & 7, h, kM8QScale);
  }
}

// Operands and attention of one window-head, dispatched on the operand format and on whether the
// window holds several Swin regions (only then are scores masked).
__device__ __forceinline__ void m8_compute(const uint4 (&kr)[2][2], const uint4 (&qr)[2][2], const float* sn,
                                           const float* cs, uint16_t* __restrict__ out, float* __restrict__ lse,
                                           const Geom& g, const WinHead& w, const uint16_t* vbuf,
                                           const uint8_t* lab, bool masked, bool h16, float kmax,
                                           const float (&qn2)[2], int lane) {
  uint4 kop[2][2], qop[2][2];
  if (h16) {
    m8_operands<true>(kr, qr, sn, cs, lane, kop, qop);
    if (masked)
      m8_attend<true, true>(kop, qop, out, lse, g, w, vbuf, lab, kmax, qn2, lane);
    else
      m8_attend<true, false>(kop, qop, out, lse, g, w, vbuf, lab, kmax, qn2, lane);
  } else {
    m8_operands<false>(kr, qr, sn, cs, lane, kop, qop);
    if (masked)
      m8_attend<false, true>(kop, qop, out, lse, g, w, vbuf, lab, kmax, qn2, lane);
    else
      m8_attend<false, false>(kop, qop, out, lse, g, w, vbuf, lab, kmax, qn2, lane);
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
                                                               Geom g, int64_t nwh) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  // [heads][2 axes][8 positions][8 pairs] sin, then cos; per wave: Q, K, V rows [64][32], labels [64]
  float* tsn = reinterpret_cast<float*>(smem_raw);
  float* tcs = tsn + g.heads * 128;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint16_t* vs = reinterpret_cast<uint16_t*>(tcs + g.heads * 128) + wave * kM8WaveLds;
  uint8_t* lab = reinterpret_cast<uint8_t*>(vs + 64 * 32);

  const int64_t wh = xcd_order(blockIdx.x, gridDim.x) * kM8Waves + wave;
  const bool active = wh < nwh;
  uint4 kr[2][2], qr[2][2];
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

  // norms: |k|^2 max over the 64 keys, |q|^2 max per query tile (rotation keeps norms)
  const float kn0 = halves_sum(m8_norm2(kr[0][0], kr[0][1]));
  const float kn1 = halves_sum(m8_norm2(kr[1][0], kr[1][1]));
  const float kmax = sqrtf(wave_max(fmaxf(kn0, kn1)));
  float qn2[2];
#pragma unroll
  for (int t = 0; t < 2; ++t) qn2[t] = wave_max(halves_sum(m8_norm2(qr[t][0], qr[t][1])));
  const bool h16 = kmax < kF16Limit && sqrtf(fmaxf(qn2[0], qn2[1])) * kM8QScale < kF16Limit;
  const float* sn = tsn + w.h * 128;
  const float* cs = tcs + w.h * 128;
  m8_compute(kr, qr, sn, cs, out, lse, g, w, vs, lab, masked, h16, kmax, qn2, lane);
}


}  // namespace

bool fwd_m8_supported(const Geom& g) { return g.M == 8 && g.d == 32 && g.heads <= kM8MaxHeads; }

hipError_t launch_fwd_m8(const FwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  const size_t smem = (size_t)g.heads * 128 * 4 * 2 + (size_t)kM8Waves * kM8WaveLds * 2;
  const int64_t grid = (nwh + kM8Waves - 1) / kM8Waves;
  hipLaunchKernelGGL(fwd_m8_kernel, dim3((unsigned)grid), dim3(kM8Waves * 64), smem, st, (const uint16_t*)a.q,
                     (const uint16_t*)a.k, (const uint16_t*)a.v, a.th_row, a.th_col, (uint16_t*)a.out, a.lse, g, nwh);
  return hipGetLastError();
}

}  // namespace fsw
