// MFMA forward kernel and its launch dispatch, included by the two translation units that instantiate
// it: fwd_mfma.hip (the plain kernels) and fwd_mfma_stats.hip (the kernels that also write the
// backward's operand maxima).  Keeping the two instance families apart keeps the code generation of
// each one independent of the other's (the compiler's module-wide choices change with the instance
// count, and the plain kernels sit at their register limit).
//
// bf16 window-attention forward on MFMA (gfx950), d = 32 (any M <= 32) and d = 64 (windows of up to
// 512 tokens, M <= 22, whose K~ and V fit LDS).
//
// Exact softmax attention inside each window with window-local 2D RoPE on Q and K, without storing
// the score matrix (FlashSwin paper card, "FLASHSWIN: Unlocking Large Windows and Dense Tokens in
// Swin Vision Transformers with Memory Efficient Attention": Abstract; Figure 1(B)).
//
// Workgroup = (window, head, block of NWAVES*32 queries).  The window's K (rotated) and V rows are
// staged once in LDS (the P.V operands are read transposed by ds_read_b64_tr_b16); each wave owns
// 32 queries (one MFMA tile) held as B operands and walks the keys in 32-key blocks:
// S^T = K~ Q^T (d/16 MFMAs), P = exp2(S^T), O^T += V^T P^T (d/16 MFMAs: d/32 output tiles of 32
// channels).  One tile per wave keeps a wave
// under 128 registers at d = 32, so four waves share each SIMD and hide each other's latencies
// (d = 64 doubles the query operands and O^T accumulators: two waves per SIMD, up to 256).  The shift
// and window partition are index arithmetic on the loads and stores; the padding tokens of a grid
// padded to a multiple of M are neither loaded nor stored and carry no query's label.  A window with a single Swin
// region and an even number of whole 32-key blocks takes a branch-free, software-pipelined loop
// (the score MFMAs of block b+1 are issued before the exponentials of block b).  Other windows mask
// per element in key blocks whose labels are mixed and skip blocks with no label in common with
// the wave.
//
// Softmax reference: softmax is unchanged by subtracting any per-row constant.  Instead of a
// running maximum, each wave subtracts the Cauchy-Schwarz bound B = max_i |q_i| * max_j |k_j| of its
// scores, widened by the operand rounding error (bound_margin), folded into the MFMA accumulator
// initialisation (so the subtraction costs nothing), and the sum is accumulated without rescaling.
// No computed score exceeds the widened bound, so every exponent is <= 0 up to float32 rounding
// and none overflows.  If a query's sum comes out below 2^-80 (a bound so loose that small terms
// could underflow) or not finite, the wave recomputes its tile with the exact row maximum in a
// second pass; results are exact either way.
//
// Precision: the score operands (rotated, scaled Q^ and K~) are rounded to fp16 when every one of
// them is in fp16 range (else bf16); P is bf16 (it may be far below 1 under the bound reference,
// where bf16 keeps the exponent range); V is the bf16 input; accumulation is float32.
#pragma once

#include <algorithm>
#include <mutex>

#include "fsw_common.h"
#include "fsw_launch.h"
#include "fsw_mfma.h"

namespace fsw {

namespace {

constexpr float kLowSum = 8.271806125530277e-25f;  // 2^-80
constexpr int kMaxWaves = 16;
constexpr int kMaxQBlocks = 2;
constexpr int kMaxNP64 = 512;  // d = 64: largest padded window whose K~ and V rows fit LDS
constexpr int kMaxNPLowRank = 512;  // d = 32 with bias channels: largest padded window served

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

// Row strides (elements) of the staged K~ and V rows for head dim D and RK channels of a low-rank
// bias (the factors' rank rounded up to 16; 0 without one).  K~ rows hold the D rotated channels,
// then the key's W factor row, then 16 bytes of pad (conflict-free 16-byte row reads); 64-channel V
// rows are padded too (128-byte rows would put the four rows of a transposing read in two bank
// groups), 32-channel V rows need none.
template <int D, int RK = 0>
struct FwdDim {
  static constexpr int KS = D + RK + 8;
  static constexpr int VS = D == 32 ? 32 : D + 8;
  static constexpr int P4 = D / 4;             // RoPE pairs per axis
  static constexpr int PARTS = D / 8;          // 16-byte parts of a token row
  static constexpr int DSTEPS = D / 16;        // k-steps over the head channels
  static constexpr int KSTEPS = (D + RK) / 16; // k-steps of a score product (head, then bias channels)
  static constexpr int OT = D / 32;            // O^T tiles of 32 channels
};
static_assert(FwdDim<32>::KS == kKStride, "d = 32 K~ stride");

struct FwdSmem {
  uint16_t* K;     // [NP][KS]
  uint16_t* V;     // [NP][VS] row-major; P.V operands come from transposing LDS reads
  float* sn;       // [2][M][D/4]  sin of RoPE angle (row axis, column axis)
  float* cs;       // [2][M][D/4]  cos
  uint16_t* rc;    // [NP]  r << 8 | c of every slot (see WinOrder); read in windows split by a shift
  uint8_t* lab;    // [NP]  key labels, 0xff past the window
  uint32_t* blk;   // [NP/32]  bits 0..8: labels present, bit 9: all 32 keys valid
  float* red;      // [2 * kMaxWaves + 12]: per-wave max |k~|^2, max |q^|^2; 4 slots each of max |q|, |k|, |v|
};

template <int D, int RK = 0>
__host__ __device__ inline size_t fwd_smem_bytes(int NP, int M) {
  size_t b = (size_t)NP * FwdDim<D, RK>::KS * 2 + (size_t)NP * FwdDim<D>::VS * 2;
  b += (size_t)2 * 2 * M * FwdDim<D>::P4 * 4;
  b += (size_t)NP * 2 + (size_t)NP;
  b = (b + 3) & ~(size_t)3;
  b += (size_t)(NP / 32) * 4 + (2 * kMaxWaves + 12) * 4;
  return b;
}

template <int D, int RK = 0>
__device__ inline FwdSmem carve(unsigned char* base, int NP, int M) {
  FwdSmem s;
  s.K = reinterpret_cast<uint16_t*>(base);
  s.V = s.K + (size_t)NP * FwdDim<D, RK>::KS;
  s.sn = reinterpret_cast<float*>(s.V + (size_t)NP * FwdDim<D>::VS);
  s.cs = s.sn + 2 * M * FwdDim<D>::P4;
  s.rc = reinterpret_cast<uint16_t*>(s.cs + 2 * M * FwdDim<D>::P4);
  s.lab = reinterpret_cast<uint8_t*>(s.rc + NP);
  size_t off = ((size_t)(s.lab + NP - base) + 3) & ~(size_t)3;
  s.blk = reinterpret_cast<uint32_t*>(base + off);
  s.red = reinterpret_cast<float*>(s.blk + NP / 32);
  return s;
}

// Slot range [bs, be) of the region band that holds slot j (see WinOrder).
__device__ __forceinline__ void band_of(const WinOrder& o, int j, int& bs, int& be) {
  const int M = o.M;
  const int e0 = o.ra * o.ca, e1 = e0 + o.ra * (M - o.ca), e2 = e1 + (M - o.ra) * o.ca;
  if (j < e0) {
    bs = 0;
    be = e0;
  } else if (j < e1) {
    bs = e0;
    be = e1;
  } else if (j < e2) {
    bs = e1;
    be = e2;
  } else {
    bs = e2;
    be = M * M;
  }
}

// Grid token of in-window position (r, c) with the window size M passed explicitly (a constant in
// the specialised kernels, so the index arithmetic folds); the position must not be padding.
__device__ __forceinline__ int64_t tok_of(const Geom& g, const WinHead& w, int M, int r, int c) {
  int y = w.wy * M + r + g.shift;
  y = y >= g.Hp ? y - g.Hp : y;
  int x = w.wx * M + c + g.shift;
  x = x >= g.Wp ? x - g.Wp : x;
  return (w.b * g.Hg + y) * g.Wg + x;
}

// Whether in-window position (r, c) is a grid token rather than padding of a padded grid.
__device__ __forceinline__ bool tok_real(const Geom& g, const WinHead& w, int M, int r, int c) {
  int y = w.wy * M + r + g.shift;
  y = y >= g.Hp ? y - g.Hp : y;
  int x = w.wx * M + c + g.shift;
  x = x >= g.Wp ? x - g.Wp : x;
  return y < g.Hg && x < g.Wg;
}

// Whether window (wy, wx) holds padding tokens: some row or column of it maps past the grid.
__device__ inline bool window_padded(const Geom& g, const WinHead& w, int M) {
  if (g.Hp == g.Hg && g.Wp == g.Wg) return false;
  bool p = false;
  for (int i = 0; i < M; ++i) p |= !tok_real(g, w, M, i, 0) || !tok_real(g, w, M, 0, i);
  return p;
}

// The wave's query operands: k-step t of the score product takes channels 16t + 8h .. 16t + 8h + 7.
template <int D, int RK = 0>
using QOps = uint4[FwdDim<D, RK>::KSTEPS];
// The wave's O^T accumulators: tile t holds channels 32t .. 32t + 31.
template <int D>
using OAcc = f32x16_t[FwdDim<D>::OT];

// Score tile S^T = K~ Q^T + cinit of key block b.
template <bool H16, int D, int RK = 0>
__device__ __forceinline__ f32x16_t block_scores(const FwdSmem& sm, int b, int row, int h, const QOps<D, RK>& qop,
                                                 const f32x16_t& cinit) {
  const uint16_t* krow = sm.K + (size_t)(b * 32 + row) * FwdDim<D, RK>::KS + 8 * h;
  f32x16_t s = mfma_op<H16>(*reinterpret_cast<const uint4*>(krow), qop[0], cinit);
#pragma unroll
  for (int t = 1; t < FwdDim<D, RK>::KSTEPS; ++t)
    s = mfma_op<H16>(*reinterpret_cast<const uint4*>(krow + 16 * t), qop[t], s);
  return s;
}

// P = exp2(S^T - m) of key block b (masked by `live` when MASK), row sums, O^T += V^T P^T.
template <bool MASK, bool SUBM, int D>
__device__ __forceinline__ void block_consume(const FwdSmem& sm, int b, int lane, uint32_t live, float m,
                                              const f32x16_t& s, float& la, float& lb, OAcc<D>& o) {
  constexpr int OT = FwdDim<D>::OT, VS = FwdDim<D>::VS;
  bf16x8_t va0[OT], va1[OT];
#pragma unroll
  for (int t = 0; t < OT; ++t) {
    va0[t] = as_bf16x8(tr_operand(sm.V + 32 * t, VS, b * 32, lane));
    va1[t] = as_bf16x8(tr_operand(sm.V + 32 * t, VS, b * 32 + 16, lane));
  }
  float p[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) p[v] = __builtin_amdgcn_exp2f(SUBM ? s[v] - m : s[v]);
  if (MASK) {
#pragma unroll
    for (int v = 0; v < 16; ++v) p[v] = ((live >> v) & 1u) ? p[v] : 0.f;
  }
  uint32_t pk[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) pk[e] = pack2(p[2 * e], p[2 * e + 1]);
#pragma unroll
  for (int e = 0; e < 8; e += 2) {
    la = add_pair(pk[e], la);
    lb = add_pair(pk[e + 1], lb);
  }
#pragma unroll
  for (int t = 0; t < OT; ++t) {
    o[t] = mfma32x32x16(va0[t], as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3])), o[t]);
    o[t] = mfma32x32x16(va1[t], as_bf16x8(make_uint4(pk[4], pk[5], pk[6], pk[7])), o[t]);
  }
}

// Pipelined pass over an even number of key blocks kb0 .. kb1-1, all whole and of the wave's one
// label: no masks, no skips, two score buffers.
template <bool H16, int D, int RK = 0>
__device__ __forceinline__ void pass_uniform(const FwdSmem& sm, int kb0, int kb1, int lane, const QOps<D, RK>& qop,
                                             const f32x16_t& cinit, float& l, OAcc<D>& o) {
  const int h = lane >> 5, row = lane & 31;
  float la = 0.f, lb = 0.f;
  if constexpr (D == 64) {  // no prefetch: the second score tile does not fit the register budget
    for (int kb = kb0; kb < kb1; ++kb) {
      const f32x16_t sa = block_scores<H16, D, RK>(sm, kb, row, h, qop, cinit);
      block_consume<false, false, D>(sm, kb, lane, 0xffffu, 0.f, sa, la, lb, o);
    }
    l = la + lb;
    return;
  }
  // the prefetch after the last pair recomputes block kb1-1 and is not used
  f32x16_t sa = block_scores<H16, D, RK>(sm, kb0, row, h, qop, cinit);
  for (int kb = kb0; kb < kb1; kb += 2) {
    const f32x16_t sb = block_scores<H16, D, RK>(sm, kb + 1, row, h, qop, cinit);
    block_consume<false, false, D>(sm, kb, lane, 0xffffu, 0.f, sa, la, lb, o);
    sa = block_scores<H16, D, RK>(sm, min(kb + 2, kb1 - 1), row, h, qop, cinit);
    block_consume<false, false, D>(sm, kb + 1, lane, 0xffffu, 0.f, sb, la, lb, o);
  }
  l = la + lb;
}

// General pass over the key blocks (regions mixed, ragged last block):
//  MODE 0: scores offset by `cinit`; p = exp2(s); accumulate l and O.
//  MODE 1: exact maximum only: m = max over live keys of the raw score.
//  MODE 2: p = exp2(s - m) with the exact per-query maximum; accumulate l and O.
template <int MODE, bool H16, int D, int RK = 0>
__device__ __forceinline__ void pass_general(const FwdSmem& sm, int NB, int lane, uint32_t wave_labels,
                                             bool wave_single, const QOps<D, RK>& qop, int qlab,
                                             const f32x16_t& cinit, float& m, float& l, OAcc<D>& o) {
  const int h = lane >> 5, row = lane & 31;
  float la = l, lb = 0.f;
  for (int kb = 0; kb < NB; ++kb) {
    const uint32_t info = uniform(sm.blk[kb]);
    const uint32_t bl = info & 0x1ffu;
    if ((bl & wave_labels) == 0) continue;  // no query of this wave may see these keys
    const bool need_mask = !((info >> 9) & 1u) || !wave_single || bl != wave_labels;
    const f32x16_t s = block_scores<H16, D, RK>(sm, kb, row, h, qop, cinit);
    const uint32_t live = need_mask ? live_bits(sm.lab, kb, h, qlab) : 0xffffu;
    if (MODE == 1) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((live >> v) & 1u) m = fmaxf(m, s[v]);
      continue;
    }
    if (need_mask)
      block_consume<true, MODE == 2, D>(sm, kb, lane, live, m, s, la, lb, o);
    else
      block_consume<false, MODE == 2, D>(sm, kb, lane, live, m, s, la, lb, o);
  }
  l = la + lb;
}

// The attention of the wave's tile: the pipelined pass when its live keys are one even run of
// whole blocks kb0 .. kb1-1 of its own label (run), else the general pass; then the exact-maximum fallback
// when the bound reference was too loose for some query.
template <bool H16, int D, int RK = 0>
__device__ __forceinline__ void attend(const FwdSmem& sm, int NB, int lane, bool run, int kb0, int kb1,
                                       uint32_t wave_labels,
                                       bool wave_single, const QOps<D, RK>& qop, int qlab, bool qvalid, float bound,
                                       float& ref, float& l, OAcc<D>& o) {
  const float refb = bound * bound_margin<H16>();
  f32x16_t cinit;
#pragma unroll
  for (int v2 = 0; v2 < 16; ++v2) cinit[v2] = -refb;
  float m = 0.f;
  if (run)
    pass_uniform<H16, D, RK>(sm, kb0, kb1, lane, qop, cinit, l, o);
  else if (wave_labels != 0)
    pass_general<0, H16, D, RK>(sm, NB, lane, wave_labels, wave_single, qop, qlab, cinit, m, l, o);
  ref = refb;
  const float lsum = halves_sum(l);
  const bool low = qvalid && !(lsum >= kLowSum && lsum < INFINITY);
  if (__builtin_amdgcn_ballot_w64(low) != 0) {
    f32x16_t zero;
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) zero[v2] = 0.f;
    m = -INFINITY;
    pass_general<1, H16, D, RK>(sm, NB, lane, wave_labels, wave_single, qop, qlab, zero, m, l, o);
    m = halves_max(m);
    if (!(m > -INFINITY)) m = 0.f;  // invalid query lanes
    l = 0.f;
#pragma unroll
    for (int t = 0; t < FwdDim<D>::OT; ++t)
#pragma unroll
      for (int v2 = 0; v2 < 16; ++v2) o[t][v2] = 0.f;
    pass_general<2, H16, D, RK>(sm, NB, lane, wave_labels, wave_single, qop, qlab, zero, m, l, o);
    ref = m;
  }
}

// Rotated K~ rows of the staged items (raw bf16 loads in kraw) into LDS in fp16 (h16) or bf16;
// returns this thread's max |k|^2 (rotation keeps norms).  Item it is 16-byte part it % PARTS of
// key it / PARTS; the PARTS parts of a key are consecutive lanes.
template <int MAXIT, int D, int RK = 0>
__device__ __forceinline__ float stage_k(const FwdSmem& sm, const uint4 (&kraw)[MAXIT], int M, bool split, int NP,
                                         int tid, int nt, bool h16) {
  constexpr int PARTS = FwdDim<D>::PARTS, AXP = PARTS / 2;
  const int N = M * M;
  float kmax2 = 0.f;
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const int it = tid + i * nt;
    if (it >= NP * PARTS) break;  // uniform across a wave: NP * PARTS is a multiple of 64
    const int key = it / PARTS;
    const int part = it % PARTS;
    uint4 kr = make_uint4(0, 0, 0, 0);
    float ss = 0.f;
    if (key < N) {
      const int rc = split ? (int)sm.rc[key] : (key / M) << 8 | (key - (key / M) * M);
      const int r = rc >> 8, c = rc & 255;
      ss = norm2_bf16x8(kraw[i], 0.f);
      float x[8];
      unpack8(kraw[i], x);
      const int axis = part / AXP;
      rotate8(x, sm.sn, sm.cs, axis, M, axis ? c : r, (part % AXP) * 4, FwdDim<D>::P4);
      kr = pack8_op(x, h16);
    }
    *reinterpret_cast<uint4*>(sm.K + (size_t)key * FwdDim<D, RK>::KS + part * 8) = kr;
    ss = quad_sum(ss);  // the parts of the key
    if (PARTS == 8)  // the other quad of the 8 lanes (row_half_mirror: lane i <- lane 7 - i)
      ss += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(ss), 0x141, 0xf, 0xf, false));
    kmax2 = fmaxf(kmax2, ss);
  }
  return kmax2;
}

// Raw W factor values of the thread's staged items (item it = tid + i nt: 8-channel part it % (RK/8)
// of slot it / (RK/8); the slot's in-window position n = r*M + c indexes the factor).  The loads are
// unconditional (slot and channel clamped into the factor), so they go out in one batch with the K
// and V loads; stage_w zeroes what lies past the rank or the window.
template <int RK, int WIT>
__device__ __forceinline__ void load_w(const FwdSmem& sm, const LowRank& lr, int head, int M, bool split, int NP,
                                       int tid, int nt, float (&wr)[WIT][8]) {
  constexpr int WP = RK / 8;
  const int N = M * M;
#pragma unroll
  for (int i = 0; i < WIT; ++i) {
    const int it = tid + i * nt;
    const int key = it < NP * WP && it / WP < N ? it / WP : 0, part = it % WP;
    const int rc = split ? (int)sm.rc[key] : (key / M) << 8 | (key - (key / M) * M);
    const float* wrow = lr.w + ((int64_t)head * N + (rc >> 8) * M + (rc & 255)) * lr.rank;
#pragma unroll
    for (int e = 0; e < 8; ++e) wr[i][e] = wrow[min(part * 8 + e, lr.rank - 1)];
  }
}

// The W factor rows of the staged keys (load_w) into channels D .. D + RK of their K~ rows (zero past
// the rank and past the window), in fp16 (h16) or bf16; returns this thread's largest |W[n]|^2 (the key
// norms that bound the scores add it to the largest |k~|^2).
template <int D, int RK, int WIT>
__device__ inline float stage_w(const FwdSmem& sm, const float (&wr)[WIT][8], int rank, int M, int NP, int tid,
                                int nt, bool h16) {
  constexpr int WP = RK / 8;
  const int N = M * M;
  float wmax2 = 0.f;
#pragma unroll
  for (int i = 0; i < WIT; ++i) {
    const int it = tid + i * nt;
    if (it >= NP * WP) break;  // uniform across a wave: NP * WP is a multiple of 64
    const int key = it / WP, part = it % WP;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = key < N && part * 8 + e < rank ? wr[i][e] : 0.f;
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    // the WP parts of a slot are consecutive lanes
#pragma unroll
    for (int o = 1; o < WP; o <<= 1) ss += __shfl_xor(ss, o, 64);
    wmax2 = fmaxf(wmax2, ss);
    *reinterpret_cast<uint4*>(sm.K + (size_t)key * FwdDim<D, RK>::KS + D + part * 8) = pack8_op(x, h16);
  }
  return wmax2;
}

// stage_w for the run-time-M instances, whose registers the batched loads would overflow: each item's
// W channels loaded as it is staged (zero past the rank and past the window).
template <int D, int RK>
__device__ inline float stage_w_direct(const FwdSmem& sm, const LowRank& lr, int head, int M, bool split, int NP,
                                       int tid, int nt, bool h16) {
  constexpr int WP = RK / 8;
  const int N = M * M;
  float wmax2 = 0.f;
  for (int it = tid; it < NP * WP; it += nt) {
    const int key = it / WP, part = it % WP;
    float x[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = 0.f;
    if (key < N) {
      const int rc = split ? (int)sm.rc[key] : (key / M) << 8 | (key - (key / M) * M);
      const float* wrow = lr.w + ((int64_t)head * N + (rc >> 8) * M + (rc & 255)) * lr.rank;
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (part * 8 + e < lr.rank) x[e] = wrow[part * 8 + e];
    }
    float ss = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) ss += x[e] * x[e];
    // the WP parts of a slot are consecutive lanes (NP * WP is a multiple of 64: uniform trip count)
#pragma unroll
    for (int o = 1; o < WP; o <<= 1) ss += __shfl_xor(ss, o, 64);
    wmax2 = fmaxf(wmax2, ss);
    *reinterpret_cast<uint4*>(sm.K + (size_t)key * FwdDim<D, RK>::KS + D + part * 8) = pack8_op(x, h16);
  }
  return wmax2;
}

// Raw U factor values of the lane's bias channels 16t + 8h + e (t < RK / 16, e < 8) of query slot rc
// (r << 8 | c), into u[8t + e]: unconditional loads (channel clamped into the rank); u_val masks them.
template <int RK>
__device__ __forceinline__ void load_u(const LowRank& lr, int head, int N, int rc, int M, int h, float (&u)[RK / 2]) {
  const float* urow = lr.u + ((int64_t)head * N + (rc >> 8) * M + (rc & 255)) * lr.rank;
#pragma unroll
  for (int t = 0; t < RK / 16; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) u[8 * t + e] = urow[min(16 * t + 8 * h + e, lr.rank - 1)];
}
// load_u for the run-time-M instances: log2(e) U[n] of the lane's channels 16t + 8h + e, each loaded
// only when within the rank (zero past it), into u[8t + e].
template <int RK>
__device__ __forceinline__ void load_u_direct(const LowRank& lr, int head, int N, int rc, int M, int h,
                                              float (&u)[RK / 2]) {
  const float* urow = lr.u + ((int64_t)head * N + (rc >> 8) * M + (rc & 255)) * lr.rank;
#pragma unroll
  for (int t = 0; t < RK / 16; ++t)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int ch = 16 * t + 8 * h + e;
      u[8 * t + e] = ch < lr.rank ? urow[ch] * kLog2e : 0.f;
    }
}
// log2(e) U of bias channel 16t + 8h + e (zero past the rank) from load_u's values.
template <int RK>
__device__ __forceinline__ float u_val(const float (&u)[RK / 2], int t, int e, int h, int rank) {
  return 16 * t + 8 * h + e < rank ? u[8 * t + e] * kLog2e : 0.f;
}

// Global loads of the thread's K and V items (16 bytes each), issued together.
template <int MAXIT, int D>
__device__ __forceinline__ void load_kv(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const Geom& g,
                                        const WinHead& w, const uint16_t* rc, int M, int NP, int tid, int nt,
                                        bool with_v, bool pad, uint4 (&kraw)[MAXIT], uint4 (&vraw)[MAXIT]) {
  constexpr int PARTS = FwdDim<D>::PARTS;
  const int N = M * M;
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const int it = tid + i * nt;
    const int key = it / PARTS;
    kraw[i] = vraw[i] = make_uint4(0, 0, 0, 0);
    if (it < NP * PARTS && key < N) {
      int r, c;
      if (rc) {
        const int rk = rc[key];
        r = rk >> 8;
        c = rk & 255;
      } else {  // row-major slots
        r = key / M;
        c = key - (key / M) * M;
      }
      if (!pad || tok_real(g, w, M, r, c)) {  // padding stays zero
        const int64_t off = tok_of(g, w, M, r, c) * g.xs + w.h * D + (it % PARTS) * 8;
        kraw[i] = *reinterpret_cast<const uint4*>(k + off);
        if (with_v) vraw[i] = *reinterpret_cast<const uint4*>(v + off);
      }
    }
  }
}

// Waves per SIMD the register budget is set for: four (128 registers) for workgroups of 8 or more waves
// at d = 32; d = 64 holds twice the query operands and O^T accumulators and takes two (256).
template <int NWAVES, int D>
constexpr int fwd_min_waves() {
  return D == 32 ? (NWAVES >= 8 ? 4 : 1) : (NWAVES >= 4 ? 2 : 1);
}

// NWAVES waves of one 32-query tile each; one workgroup per window-head stages the window's K/V
// once and then walks its query blocks of NWAVES*32 queries.  MT: compile-time window size
// (0 = g.M at run time).  NPMAX: the largest padded window this configuration serves.  D: head dim.
// PAD: the grid is padded to a multiple of M (the padding checks cost a few percent, so grids that M
// divides run an instance without them).  RK: channels of a low-rank bias U[n_i] . W[n_j] (the rank
// rounded up to 16, 0 for none), folded into the score product as extra channels: the query operand
// carries log2(e) U[n_i] after its rotated, scaled channels, the staged key row W[n_j] after K~.
// STATS: also write the window-head's largest |component| of q, k and v into stats (an instance of its
// own, so that the kernel without them keeps its register allocation).
template <int NWAVES, int MT, int NPMAX, int D, bool PAD, int RK, bool STATS>
__global__ __launch_bounds__(NWAVES * 64, (fwd_min_waves<NWAVES, D>())) void fwd_mfma_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               const float* __restrict__ th_row,
                                                               const float* __restrict__ th_col,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse,
                                                               Geom g, int nqb, int NP, int nsplit, LowRank lr,
                                                               float* __restrict__ stats) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  using Dim = FwdDim<D, RK>;
  constexpr int NT = NWAVES * 64;
  constexpr int MAXIT = (NPMAX * Dim::PARTS + NT - 1) / NT;
  constexpr int QBM = (NPMAX + NWAVES * 32 - 1) / (NWAVES * 32);  // query blocks per window, at most
  static_assert(NWAVES <= kMaxWaves, "too many waves");
  static_assert(QBM <= kMaxQBlocks, "too many query blocks");
  const int M = MT > 0 ? MT : g.M;
  const int N = M * M;
  const int NB = NP / 32;
  const FwdSmem sm = carve<D, RK>(smem_raw, NP, M);

  // Work of this workgroup: window-head wh, query blocks qoff .. qoff + nqw - 1.  The first nsplit
  // window-heads are split into one workgroup per query block, dispatched first (the first
  // 2*nsplit/8 slots of every XCD): those CUs finish their first task early, so from then on the
  // CUs stage K/V at staggered times instead of all at once.  The rest are ordered per XCD so a
  // window's heads share one L2.
  int64_t wh;
  int qoff = 0, nqw = nqb;
  {
    const int64_t b = blockIdx.x, shorts = 2 * (int64_t)nsplit, pos = b >> 3, x = b & 7;
    if (pos < shorts / 8) {
      const int64_t sidx = x * (shorts / 8) + pos;
      wh = sidx >> 1;
      qoff = (int)(sidx & 1);
      nqw = 1;
    } else {
      wh = nsplit + xcd_order(b - shorts, (int64_t)gridDim.x - shorts);
    }
  }
  const WinHead w = decode_winhead(g, wh);
  const WinOrder wo = win_order(g, M, w.wy, w.wx);
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int h = lane >> 5;
  const int col = lane & 31;

  // 0. slot order: in-window position and label of every slot.  In a window split by the shift the
  // loads below take their addresses from this table; otherwise slots are row-major.
  // Padding tokens of a padded grid get label 0xff, like the slots past the window: no query's label.
  const bool split = wo.ra != M || wo.ca != M;  // one window per workgroup: uniform
  const bool pad = PAD && window_padded(g, w, M);
  for (int n = tid; n < NP; n += NT) {
    uint8_t lb = 0xff;
    if (n < N) {
      int r, c;
      slot_rc(wo, n, r, c);
      sm.rc[n] = (uint16_t)(r << 8 | c);
      if (!pad || tok_real(g, w, M, r, c)) lb = (uint8_t)token_label(g, w.wy, w.wx, r, c);
    }
    sm.lab[n] = lb;
  }
  if (STATS && tid < 12) sm.red[2 * kMaxWaves + tid] = 0.f;  // slots of the workgroup's operand maxima
  if (split) __syncthreads();

  // 1. every global load of the thread (K and V items, the queries of every block)
  uint4 kraw[MAXIT], vraw[MAXIT];
  load_kv<MAXIT, D>(k, v, g, w, split ? sm.rc : nullptr, M, NP, tid, NT, true, pad, kraw, vraw);
  // the lane's query of block qb (16-byte pieces: channels 16t + 8h .. 16t + 8h + 7)
  auto load_q = [&](int qb, uint4 (&a)[Dim::DSTEPS]) {
    const int qi = (qoff + qb) * NT / 2 + wave * 32 + col;
#pragma unroll
    for (int t = 0; t < Dim::DSTEPS; ++t) a[t] = make_uint4(0, 0, 0, 0);
    if (qb < nqw && qi < N) {
      const int rc = split ? (int)sm.rc[qi] : (qi / M) << 8 | (qi - (qi / M) * M);
      if (!pad || tok_real(g, w, M, rc >> 8, rc & 255)) {  // padding stays zero
        const int64_t off = tok_of(g, w, M, rc >> 8, rc & 255) * g.xs + w.h * D;
#pragma unroll
        for (int t = 0; t < Dim::DSTEPS; ++t) a[t] = *reinterpret_cast<const uint4*>(q + off + 16 * t + 8 * h);
      }
    }
  };
  uint4 qraw[QBM][Dim::DSTEPS];
#pragma unroll
  for (int qb = 0; qb < QBM; ++qb) load_q(qb, qraw[qb]);
  // The bias factors of the staged keys and of the queries: with the window size fixed at compile
  // time, in the same batch (kEarly); in the run-time-M instances, whose registers that would
  // overflow, each in a batch of its own right before its use.
  constexpr bool kEarly = MT > 0;
  constexpr int WIT = RK > 0 ? (NPMAX * (RK / 8) + NT - 1) / NT : 1;
  float wraw[WIT][8];
  float uraw[kEarly ? QBM : 1][RK > 0 ? RK / 2 : 1];
  // the lane's query slot of block qb (r << 8 | c), 0 past the window
  auto q_rc = [&](int qb) {
    const int qi = (qoff + qb) * NT / 2 + wave * 32 + col;
    if (!(qb < nqw && qi < N)) return 0;
    return split ? (int)sm.rc[qi] : (qi / M) << 8 | (qi - (qi / M) * M);
  };
  if constexpr (RK > 0 && kEarly) {
    load_w<RK, WIT>(sm, lr, w.h, M, split, NP, tid, NT, wraw);
#pragma unroll
    for (int qb = 0; qb < QBM; ++qb) load_u<RK>(lr, w.h, N, q_rc(qb), M, h, uraw[qb]);
  }

  // 2. RoPE sin/cos table (while the loads are in flight)
  constexpr int P4 = Dim::P4;
  for (int i = tid; i < 2 * M * P4; i += NT) {
    const int axis = i / (M * P4);
    const int p = (i / P4) % M;
    const int j = i % P4;
    const float th = axis ? th_col[w.h * P4 + j] : th_row[w.h * P4 + j];
    float s, c;
    rope_sincos(th, p, &s, &c);
    sm.sn[i] = s;
    sm.cs[i] = c;
  }
  __syncthreads();

  // 3. K~ rows (rotated, fp16), V rows, block label summaries, norms.  With STATS: the largest
  // |component| of the raw k, v and q rows the threads hold (items past the window and padding were
  // loaded as zeros), gathered in sm.red where those rows are live anyway.
  // Every lane takes an LDS atomic maximum on the float bits (non-negative floats order as unsigned
  // integers) into one of four slots per quantity (lane % 4): no cross-lane reduction and no registers
  // held for it.  (Sixteen slots, or a wave reduction first, measured slower at M = 16: the kernel is
  // at its register limit there and spills.)  The slots were cleared before the barrier that ends
  // step 2; one thread folds them after the barrier below.
  unsigned* const red_u = reinterpret_cast<unsigned*>(sm.red + 2 * kMaxWaves);
  const auto fold_absmax = [&](int slot, uint32_t acc) {
    atomicMax(red_u + slot * 4 + (lane & 3), __float_as_uint(absmax_value(acc)));
  };
  if constexpr (STATS) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < MAXIT; ++i) a = absmax_x8(a, kraw[i]);
    fold_absmax(1, a);
  }
  float kmax2 = stage_k<MAXIT, D, RK>(sm, kraw, M, split, NP, tid, NT, true);
  if constexpr (RK > 0) {
    if constexpr (kEarly)
      kmax2 += stage_w<D, RK, WIT>(sm, wraw, lr.rank, M, NP, tid, NT, true);
    else
      kmax2 += stage_w_direct<D, RK>(sm, lr, w.h, M, split, NP, tid, NT, true);
  }
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const int it = tid + i * NT;
    if (it < NP * Dim::PARTS)
      *reinterpret_cast<uint4*>(sm.V + (size_t)(it / Dim::PARTS) * Dim::VS + (it % Dim::PARTS) * 8) = vraw[i];
  }
  if constexpr (STATS) {
    uint32_t a = 0;
#pragma unroll
    for (int i = 0; i < MAXIT; ++i) a = absmax_x8(a, vraw[i]);
    fold_absmax(2, a);
  }
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
  // log2(e) / sqrt(d)
  const float qscale = kLog2e * (D == 32 ? 0.17677669529663687f : 0.125f);
  float qn2max[QBM];
#pragma unroll
  for (int qb = 0; qb < QBM; ++qb) {
    float qn2 = 0.f;
#pragma unroll
    for (int t = 0; t < Dim::DSTEPS; ++t) qn2 = norm2_bf16x8(qraw[qb][t], qn2);
    if constexpr (RK > 0) {  // plus |log2(e) U[n_q]|^2 of the bias channels
      qn2 *= qscale * qscale;
      const int qi = (qoff + qb) * NT / 2 + wave * 32 + col;
      if (qb < nqw && qi < N) {
        if constexpr (kEarly) {
#pragma unroll
          for (int t = 0; t < RK / 16; ++t)
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const float u = u_val<RK>(uraw[kEarly ? qb : 0], t, e, h, lr.rank);
              qn2 += u * u;
            }
        } else {
          float u[RK / 2];
          load_u_direct<RK>(lr, w.h, N, q_rc(qb), M, h, u);
#pragma unroll
          for (int e = 0; e < RK / 2; ++e) qn2 += u[e] * u[e];
        }
      }
      qn2max[qb] = wave_max(halves_sum(qn2));
    } else {
      qn2max[qb] = wave_max(halves_sum(qn2)) * (qscale * qscale);
    }
  }
  kmax2 = wave_max(kmax2);
  if (lane == 0) {
    float qm = 0.f;
#pragma unroll
    for (int qb = 0; qb < QBM; ++qb) qm = fmaxf(qm, qn2max[qb]);
    sm.red[wave] = kmax2;
    sm.red[kMaxWaves + wave] = qm;
  }
  if constexpr (STATS) {
    uint32_t a = 0;
#pragma unroll
    for (int qb = 0; qb < QBM; ++qb)
#pragma unroll
      for (int t = 0; t < Dim::DSTEPS; ++t) a = absmax_x8(a, qraw[qb][t]);
    fold_absmax(0, a);
  }
  __syncthreads();
  if (STATS && tid == 0) {
    // stats[wh] = {max |q| over the queries of the first workgroup, over those of the second (0 when
    // one workgroup takes them all), max |k|, max |v|}: every slot written, by one workgroup each
    float mq = 0.f, mk = 0.f, mv = 0.f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      mq = fmaxf(mq, sm.red[2 * kMaxWaves + i]);
      mk = fmaxf(mk, sm.red[2 * kMaxWaves + 4 + i]);
      mv = fmaxf(mv, sm.red[2 * kMaxWaves + 8 + i]);
    }
    float* const s4 = stats + wh * 4;
    if (qoff == 0) {
      s4[0] = mq;
      if (nqw == nqb) s4[1] = 0.f;
      s4[2] = mk;
      s4[3] = mv;
    } else {
      s4[1] = mq;
    }
  }
  float kmax2_all = 0.f, qmax2_all = 0.f;
#pragma unroll
  for (int i = 0; i < NWAVES; ++i) {
    kmax2_all = fmaxf(kmax2_all, sm.red[i]);
    qmax2_all = fmaxf(qmax2_all, sm.red[kMaxWaves + i]);
  }
  const float kmax = sqrtf(kmax2_all);
  // fp16 score operands unless some |k~| or |q^| (hence some component) could leave fp16 range
  const bool h16 = kmax < kF16Limit && sqrtf(qmax2_all) < kF16Limit;
  if (!h16) {
    load_kv<MAXIT, D>(k, v, g, w, split ? sm.rc : nullptr, M, NP, tid, NT, false, pad, kraw, vraw);
    __syncthreads();
    stage_k<MAXIT, D, RK>(sm, kraw, M, split, NP, tid, NT, false);
    if constexpr (RK > 0 && kEarly) {
      load_w<RK, WIT>(sm, lr, w.h, M, split, NP, tid, NT, wraw);
      stage_w<D, RK, WIT>(sm, wraw, lr.rank, M, NP, tid, NT, false);
    } else if constexpr (RK > 0) {
      stage_w_direct<D, RK>(sm, lr, w.h, M, split, NP, tid, NT, false);
    }
    __syncthreads();
  }
#pragma unroll
  for (int qb = 0; qb < QBM; ++qb) {
    if (qb >= nqw) break;
    // 4. the wave's query operands (rotated, scaled by log2(e)/sqrt(d)), reference bound, labels
    const int qi = (qoff + qb) * NT / 2 + wave * 32 + col;
    const bool qvalid = qi < N && (!pad || sm.lab[qi] != 0xff);
    const int qrc = !qvalid ? 0 : split ? (int)sm.rc[qi] : (qi / M) << 8 | (qi - (qi / M) * M);
    const int qr = qrc >> 8, qc = qrc & 255;
    QOps<D, RK> qop;
    // block 0's query was loaded with K and V; later blocks reload theirs (an L2 hit) during the
    // previous block's epilogue: keeping every block's raw query live across attend() costs registers.
    // Piece t holds channels 16t + 8h ..: axis (16t) / (d/2), pairs from ((16t) % (d/2) + 8h) / 2.
#pragma unroll
    for (int t = 0; t < Dim::DSTEPS; ++t) {
      constexpr int HALF = D / 2;
      const int axis = (16 * t) / HALF;
      float x[8];
      unpack8(qraw[qb][t], x);
      rotate8(x, sm.sn, sm.cs, axis, M, axis ? qc : qr, ((16 * t) % HALF) / 2 + 4 * h, P4);
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] *= qscale;
      qop[t] = pack8_op(x, h16);
    }
    if constexpr (RK > 0) {  // the bias channels: log2(e) U[n_q], lane h holding 8h.. of each 16
      float ul[RK / 2];
#pragma unroll
      for (int e = 0; e < RK / 2; ++e) ul[e] = 0.f;
      if constexpr (!kEarly) {
        if (qvalid) load_u_direct<RK>(lr, w.h, N, qrc, M, h, ul);
      }
#pragma unroll
      for (int t = 0; t < RK / 16; ++t) {
        float x[8];
#pragma unroll
        for (int e = 0; e < 8; ++e)
          x[e] = kEarly ? (qvalid ? u_val<RK>(uraw[kEarly ? qb : 0], t, e, h, lr.rank) : 0.f) : ul[8 * t + e];
        qop[Dim::DSTEPS + t] = pack8_op(x, h16);
      }
    }
    const float bound = sqrtf(qn2max[qb]) * kmax;  // >= every score of this wave (log2 units)
    const int qlab = qvalid ? token_label(g, w.wy, w.wx, qr, qc) : 0xff;
    const uint32_t wave_labels = uniform(wave_or(qvalid ? 1u << qlab : 0u));
    const bool wave_single = __builtin_popcount(wave_labels) == 1;
    // A single-label wave sees exactly the keys of its region band, one contiguous slot range [bs, be).
    // When the band is whole 32-slot blocks, even in number, the wave takes the pipelined pass over
    // them (every window without a shift, and the bands of the usual shifted shapes).
    int kb0 = 0, kb1 = 0;
    bool run = false;
    if (wave_single && !pad) {  // a padded window's bands hold padding: the masked general pass
      int bs, be;
      band_of(wo, uniform((qoff + qb) * NT / 2 + wave * 32), bs, be);
      run = ((bs | be) & 31) == 0 && (((be - bs) >> 5) & 1) == 0;
      kb0 = bs >> 5;
      kb1 = be >> 5;
    }

    OAcc<D> o;
    float l = 0.f, ref;
#pragma unroll
    for (int t = 0; t < Dim::OT; ++t)
#pragma unroll
      for (int v2 = 0; v2 < 16; ++v2) o[t][v2] = 0.f;
    if (h16)
      attend<true, D, RK>(sm, NB, lane, run, kb0, kb1, wave_labels, wave_single, qop, qlab, qvalid, bound, ref, l, o);
    else
      attend<false, D, RK>(sm, NB, lane, run, kb0, kb1, wave_labels, wave_single, qop, qlab, qvalid, bound, ref, l, o);

    // the next block's query loads go out before this block's epilogue
    if (qb + 1 < QBM) {
      load_q(qb + 1, qraw[qb + 1]);  // zeros past the last block
      if constexpr (RK > 0 && kEarly) load_u<RK>(lr, w.h, N, q_rc(qb + 1), M, h, uraw[qb + 1]);
    }
    // 5. epilogue: O = O^T / l (lane: query col, channels 32t + 8g + 4h + j), LSE = (ref + log2 l) ln 2
    const float lt = halves_sum(l);
    if (qvalid) {
      const int64_t qtok = tok_of(g, w, M, qr, qc);
      const float inv = 1.f / lt;
#pragma unroll
      for (int t = 0; t < Dim::OT; ++t) {
        uint16_t* dst = out + qtok * g.os + w.h * D + 32 * t + 4 * h;
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          uint2 pr;
          pr.x = pack2(o[t][4 * gq] * inv, o[t][4 * gq + 1] * inv);
          pr.y = pack2(o[t][4 * gq + 2] * inv, o[t][4 * gq + 3] * inv);
          *reinterpret_cast<uint2*>(dst + 8 * gq) = pr;
        }
      }
      if (lse && h == 0) lse[qtok * g.heads + w.h] = (ref + __log2f(lt)) * kLn2;
    }
  }
}

template <bool STATS, int NWAVES, int MT, int NPMAX, int D, bool PAD = false, int RK = 0>
hipError_t launch_nw(const FwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int NP = (g.N + 31) / 32 * 32;
  const int nqb = (g.N + NWAVES * 32 - 1) / (NWAVES * 32);
  const size_t smem = fwd_smem_bytes<D, RK>(NP, g.M);
  // The dynamic-LDS limit is raised on the current device, once per device (beyond kMaxDevices:
  // on every call).
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  const auto raise = [] {
    (void)hipFuncSetAttribute((const void*)fwd_mfma_kernel<NWAVES, MT, NPMAX, D, PAD, RK, STATS>,
                              hipFuncAttributeMaxDynamicSharedMemorySize, 160 * 1024);
  };
  int dev = 0;
  if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < kMaxDevices)
    std::call_once(once[dev], raise);
  else
    raise();
  const int64_t nwh = g.B * g.nH * g.nW * g.heads;
  // staggered start (see the kernel): 64 window-heads split into 128 half tasks when there are
  // two query blocks and enough work for several rounds of workgroups per CU
  const int nsplit = (nqb == 2 && nwh >= 64 * 8) ? 64 : 0;
  const int64_t blocks = nwh + nsplit;
  hipLaunchKernelGGL((fwd_mfma_kernel<NWAVES, MT, NPMAX, D, PAD, RK, STATS>), dim3((unsigned)blocks),
                     dim3(NWAVES * 64), smem, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.th_row, a.th_col,
                     (uint16_t*)a.out, a.lse, g, nqb, NP, nsplit, a.lr, a.stats);
  return hipGetLastError();
}

// d = 32 with RK bias channels, run-time M (windows of up to kMaxNPLowRank padded tokens).
template <bool STATS, int RK>
hipError_t launch_lowrank(const FwdArgs& a, hipStream_t st) {
  const int N = a.g.N;
  if (N <= 64) return launch_nw<STATS, 2, 0, 64, 32, false, RK>(a, st);
  if (N <= 128) return launch_nw<STATS, 4, 0, 128, 32, false, RK>(a, st);
  if (a.g.M == 16) return launch_nw<STATS, 8, 16, 256, 32, false, RK>(a, st);  // window size fixed at compile time
  if (N <= 256) return launch_nw<STATS, 8, 0, 256, 32, false, RK>(a, st);
  return launch_nw<STATS, 8, 0, kMaxNPLowRank, 32, false, RK>(a, st);
}
// The instances of one STATS value for a forward call (the MFMA shapes; the M = 8 shapes of the one-wave
// kernel, which writes the maxima itself when a.stats is set).
template <bool STATS>
hipError_t launch_fwd_mfma_impl(const FwdArgs& a, hipStream_t st) {
  const int N = a.g.N;
  if (a.lr.rank > 0) {
    if (!fwd_mfma_lowrank_supported(a.g, a.lr.rank)) return hipErrorInvalidValue;
    return a.lr.rank <= 16 ? launch_lowrank<STATS, 16>(a, st) : launch_lowrank<STATS, 32>(a, st);
  }
  if (!fwd_mfma_supported(a.g)) return hipErrorInvalidValue;
  if (a.g.Hp != a.g.Hg || a.g.Wp != a.g.Wg) {  // padded grid: the run-time-M instances with padding checks
    if (a.g.d == 64) {
      if (N <= 64) return launch_nw<STATS, 2, 0, 64, 64, true>(a, st);
      if (N <= 128) return launch_nw<STATS, 4, 0, 128, 64, true>(a, st);
      if (N <= 256) return launch_nw<STATS, 4, 0, 256, 64, true>(a, st);
      return launch_nw<STATS, 8, 0, kMaxNP64, 64, true>(a, st);
    }
    if (N <= 64) return launch_nw<STATS, 2, 0, 64, 32, true>(a, st);
    if (N <= 128) return launch_nw<STATS, 4, 0, 128, 32, true>(a, st);
    if (N <= 256) return launch_nw<STATS, 8, 0, 256, 32, true>(a, st);
    return launch_nw<STATS, 16, 0, 1024, 32, true>(a, st);
  }
  if (a.g.d == 64) {
    if (N <= 64) return launch_nw<STATS, 2, 0, 64, 64>(a, st);
    if (N <= 128) return launch_nw<STATS, 4, 0, 128, 64>(a, st);
    // four waves of two query tiles: two workgroups share a CU (LDS), one stages while the other computes
    if (a.g.M == 16) return launch_nw<STATS, 4, 16, 256, 64>(a, st);
    if (N <= 256) return launch_nw<STATS, 4, 0, 256, 64>(a, st);
    return launch_nw<STATS, 8, 0, kMaxNP64, 64>(a, st);
  }
  if (a.g.M == 32) return launch_nw<STATS, 16, 32, 1024, 32>(a, st);
  if (fwd_m8_supported(a.g)) return launch_fwd_m8(a, st);
  if (a.g.M == 8) return launch_nw<STATS, 2, 8, 64, 32>(a, st);
  if (a.g.M == 16) return launch_nw<STATS, 8, 16, 256, 32>(a, st);
  if (N <= 64) return launch_nw<STATS, 2, 0, 64, 32>(a, st);
  if (N <= 128) return launch_nw<STATS, 4, 0, 128, 32>(a, st);
  if (N <= 256) return launch_nw<STATS, 8, 0, 256, 32>(a, st);
  return launch_nw<STATS, 16, 0, 1024, 32>(a, st);
}

}  // namespace

}  // namespace fsw
