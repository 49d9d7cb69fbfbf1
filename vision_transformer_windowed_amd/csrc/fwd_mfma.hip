// bf16 window-attention forward on MFMA (gfx950), d = 32, any M <= 32.
//
// Exact softmax attention inside each window with window-local 2D RoPE on Q and K, without storing
// the score matrix (FlashSwin paper card, "FLASHSWIN: Unlocking Large Windows and Dense Tokens in
// Swin Vision Transformers with Memory Efficient Attention": Abstract; Figure 1(B)).
//
// Workgroup = (window, head, block of NWAVES*32 queries).  The window's K (rotated) and V rows are
// staged once in LDS (the P.V operands are read transposed by ds_read_b64_tr_b16); each wave owns
// 32 queries (one MFMA tile) held as B operands and walks the keys in 32-key blocks:
// S^T = K~ Q^T (2 MFMAs), P = exp2(S^T), O^T += V^T P^T (2 MFMAs).  One tile per wave keeps a wave
// under 128 registers, so four waves share each SIMD and hide each other's latencies.  The shift
// and window partition are index arithmetic on the loads and stores.  A window with a single Swin
// region and an even number of whole 32-key blocks takes a branch-free, software-pipelined loop
// (the score MFMAs of block b+1 are issued before the exponentials of block b).  Other windows mask
// per element in key blocks whose labels are mixed and skip blocks with no label in common with
// the wave.
//
// Softmax reference: softmax is unchanged by subtracting any per-row constant.  Instead of a
// running maximum, each wave subtracts the Cauchy-Schwarz bound B = max_i |q_i| * max_j |k_j| of its
// scores, folded into the MFMA accumulator initialisation (so the subtraction costs nothing), and
// the sum is accumulated without rescaling.  Every exponent is then <= 0 (no overflow).  If a
// query's sum comes out below 2^-80 (a bound so loose that small terms could underflow), the wave
// recomputes its tile with the exact row maximum in a second pass; results are exact either way.
//
// Precision: the score operands (rotated, scaled Q^ and K~) are rounded to fp16 when every one of
// them is in fp16 range (else bf16); P is bf16 (it may be far below 1 under the bound reference,
// where bf16 keeps the exponent range); V is the bf16 input; accumulation is float32.
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

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

struct FwdSmem {
  uint16_t* K;     // [NP][kKStride]
  uint16_t* V;     // [NP][32] row-major; P.V operands come from transposing LDS reads
  float* sn;       // [2][M][8]  sin of RoPE angle (row axis, column axis)
  float* cs;       // [2][M][8]  cos
  uint16_t* rc;    // [NP]  r << 8 | c of every slot (see WinOrder); read in windows split by a shift
  uint8_t* lab;    // [NP]  key labels, 0xff past the window
  uint32_t* blk;   // [NP/32]  bits 0..8: labels present, bit 9: all 32 keys valid
  float* red;      // [2 * kMaxWaves]: per-wave max |k~|^2, then max |q^|^2
};

__host__ __device__ inline size_t fwd_smem_bytes(int NP, int M) {
  size_t b = (size_t)NP * kKStride * 2 + (size_t)NP * 32 * 2;
  b += (size_t)2 * 2 * M * 8 * 4;
  b += (size_t)NP * 2 + (size_t)NP;
  b = (b + 3) & ~(size_t)3;
  b += (size_t)(NP / 32) * 4 + 2 * kMaxWaves * 4;
  return b;
}

__device__ inline FwdSmem carve(unsigned char* base, int NP, int M) {
  FwdSmem s;
  s.K = reinterpret_cast<uint16_t*>(base);
  s.V = s.K + (size_t)NP * kKStride;
  s.sn = reinterpret_cast<float*>(s.V + (size_t)NP * 32);
  s.cs = s.sn + 2 * M * 8;
  s.rc = reinterpret_cast<uint16_t*>(s.cs + 2 * M * 8);
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
// the specialised kernels, so the index arithmetic folds).
__device__ __forceinline__ int64_t tok_of(const Geom& g, const WinHead& w, int M, int r, int c) {
  int y = w.wy * M + r + g.shift;
  y = y >= g.Hg ? y - g.Hg : y;
  int x = w.wx * M + c + g.shift;
  x = x >= g.Wg ? x - g.Wg : x;
  return (w.b * g.Hg + y) * g.Wg + x;
}

// Score tile S^T = K~ Q^T + cinit of key block b.
template <bool H16>
__device__ __forceinline__ f32x16_t block_scores(const FwdSmem& sm, int b, int row, int h, uint4 qb0, uint4 qb1,
                                                 const f32x16_t& cinit) {
  const uint16_t* krow = sm.K + (size_t)(b * 32 + row) * kKStride + 8 * h;
  f32x16_t s = mfma_op<H16>(*reinterpret_cast<const uint4*>(krow), qb0, cinit);
  return mfma_op<H16>(*reinterpret_cast<const uint4*>(krow + 16), qb1, s);
}

// P = exp2(S^T - m) of key block b (masked by `live` when MASK), row sums, O^T += V^T P^T.
template <bool MASK, bool SUBM>
__device__ __forceinline__ void block_consume(const FwdSmem& sm, int b, int lane, uint32_t live, float m,
                                              const f32x16_t& s, float& la, float& lb, f32x16_t& o) {
  const bf16x8_t va0 = as_bf16x8(tr_operand(sm.V, 32, b * 32, lane));
  const bf16x8_t va1 = as_bf16x8(tr_operand(sm.V, 32, b * 32 + 16, lane));
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
  o = mfma32x32x16(va0, as_bf16x8(make_uint4(pk[0], pk[1], pk[2], pk[3])), o);
  o = mfma32x32x16(va1, as_bf16x8(make_uint4(pk[4], pk[5], pk[6], pk[7])), o);
}

// Pipelined pass over an even number of key blocks kb0 .. kb1-1, all whole and of the wave's one
// label: no masks, no skips, two score buffers.
template <bool H16>
__device__ __forceinline__ void pass_uniform(const FwdSmem& sm, int kb0, int kb1, int lane, uint4 qb0, uint4 qb1,
                                             const f32x16_t& cinit, float& l, f32x16_t& o) {
  const int h = lane >> 5, row = lane & 31;
  float la = 0.f, lb = 0.f;
  // the prefetch after the last pair recomputes block kb1-1 and is not used
  f32x16_t sa = block_scores<H16>(sm, kb0, row, h, qb0, qb1, cinit);
  for (int kb = kb0; kb < kb1; kb += 2) {
    const f32x16_t sb = block_scores<H16>(sm, kb + 1, row, h, qb0, qb1, cinit);
    block_consume<false, false>(sm, kb, lane, 0xffffu, 0.f, sa, la, lb, o);
    sa = block_scores<H16>(sm, min(kb + 2, kb1 - 1), row, h, qb0, qb1, cinit);
    block_consume<false, false>(sm, kb + 1, lane, 0xffffu, 0.f, sb, la, lb, o);
  }
  l = la + lb;
}

// General pass over the key blocks (regions mixed, ragged last block):
//  MODE 0: scores offset by `cinit`; p = exp2(s); accumulate l and O.
//  MODE 1: exact maximum only: m = max over live keys of the raw score.
//  MODE 2: p = exp2(s - m) with the exact per-query maximum; accumulate l and O.
template <int MODE, bool H16>
__device__ __forceinline__ void pass_general(const FwdSmem& sm, int NB, int lane, uint32_t wave_labels,
                                             bool wave_single, uint4 qb0, uint4 qb1, int qlab,
                                             const f32x16_t& cinit, float& m, float& l, f32x16_t& o) {
  const int h = lane >> 5, row = lane & 31;
  float la = l, lb = 0.f;
  for (int kb = 0; kb < NB; ++kb) {
    const uint32_t info = uniform(sm.blk[kb]);
    const uint32_t bl = info & 0x1ffu;
    if ((bl & wave_labels) == 0) continue;  // no query of this wave may see these keys
    const bool need_mask = !((info >> 9) & 1u) || !wave_single || bl != wave_labels;
    const f32x16_t s = block_scores<H16>(sm, kb, row, h, qb0, qb1, cinit);
    const uint32_t live = need_mask ? live_bits(sm.lab, kb, h, qlab) : 0xffffu;
    if (MODE == 1) {
#pragma unroll
      for (int v = 0; v < 16; ++v)
        if ((live >> v) & 1u) m = fmaxf(m, s[v]);
      continue;
    }
    if (need_mask)
      block_consume<true, MODE == 2>(sm, kb, lane, live, m, s, la, lb, o);
    else
      block_consume<false, MODE == 2>(sm, kb, lane, live, m, s, la, lb, o);
  }
  l = la + lb;
}

// The attention of the wave's tile: the pipelined pass when its live keys are one even run of
// whole blocks kb0 .. kb1-1 of its own label (run), else the general pass; then the exact-maximum fallback
// when the bound reference was too loose for some query.
template <bool H16>
__device__ __forceinline__ void attend(const FwdSmem& sm, int NB, int lane, bool run, int kb0, int kb1,
                                       uint32_t wave_labels,
                                       bool wave_single, uint4 qb0, uint4 qb1, int qlab, bool qvalid, float bound,
                                       float& ref, float& l, f32x16_t& o) {
  f32x16_t cinit;
#pragma unroll
  for (int v2 = 0; v2 < 16; ++v2) cinit[v2] = -bound;
  float m = 0.f;
  if (run)
    pass_uniform<H16>(sm, kb0, kb1, lane, qb0, qb1, cinit, l, o);
  else if (wave_labels != 0)
    pass_general<0, H16>(sm, NB, lane, wave_labels, wave_single, qb0, qb1, qlab, cinit, m, l, o);
  ref = bound;
  const bool low = qvalid && !(halves_sum(l) >= kLowSum);
  if (__builtin_amdgcn_ballot_w64(low) != 0) {
    f32x16_t zero;
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) zero[v2] = 0.f;
    m = -INFINITY;
    pass_general<1, H16>(sm, NB, lane, wave_labels, wave_single, qb0, qb1, qlab, zero, m, l, o);
    m = halves_max(m);
    if (!(m > -INFINITY)) m = 0.f;  // invalid query lanes
    l = 0.f;
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) o[v2] = 0.f;
    pass_general<2, H16>(sm, NB, lane, wave_labels, wave_single, qb0, qb1, qlab, zero, m, l, o);
    ref = m;
  }
}

// Rotated K~ rows of the staged items (raw bf16 loads in kraw) into LDS in fp16 (h16) or bf16;
// returns this thread's max |k|^2 (rotation keeps norms).
template <int MAXIT>
__device__ __forceinline__ float stage_k(const FwdSmem& sm, const uint4 (&kraw)[MAXIT], int M, bool split, int NP,
                                         int tid, int nt, bool h16) {
  const int N = M * M;
  float kmax2 = 0.f;
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const int it = tid + i * nt;
    if (it >= NP * 4) break;  // uniform across a wave: NP * 4 is a multiple of 64
    const int key = it >> 2;
    const int part = it & 3;
    uint4 kr = make_uint4(0, 0, 0, 0);
    float ss = 0.f;
    if (key < N) {
      const int rc = split ? (int)sm.rc[key] : (key / M) << 8 | (key - (key / M) * M);
      const int r = rc >> 8, c = rc & 255;
      ss = norm2_bf16x8(kraw[i], 0.f);
      float x[8];
      unpack8(kraw[i], x);
      const int axis = part >> 1;
      rotate8(x, sm.sn, sm.cs, axis, M, axis ? c : r, (part & 1) * 4);
      kr = pack8_op(x, h16);
    }
    *reinterpret_cast<uint4*>(sm.K + (size_t)key * kKStride + part * 8) = kr;
    ss = quad_sum(ss);  // the 4 parts of the key
    kmax2 = fmaxf(kmax2, ss);
  }
  return kmax2;
}

// Global loads of the thread's K and V items (16 bytes each), issued together.
template <int MAXIT>
__device__ __forceinline__ void load_kv(const uint16_t* __restrict__ k, const uint16_t* __restrict__ v, const Geom& g,
                                        const WinHead& w, const uint16_t* rc, int M, int NP, int tid, int nt,
                                        bool with_v, uint4 (&kraw)[MAXIT], uint4 (&vraw)[MAXIT]) {
  const int N = M * M;
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const int it = tid + i * nt;
    const int key = it >> 2;
    kraw[i] = vraw[i] = make_uint4(0, 0, 0, 0);
    if (it < NP * 4 && key < N) {
      int r, c;
      if (rc) {
        const int rk = rc[key];
        r = rk >> 8;
        c = rk & 255;
      } else {  // row-major slots
        r = key / M;
        c = key - (key / M) * M;
      }
      const int64_t off = tok_of(g, w, M, r, c) * g.xs + w.h * 32 + (it & 3) * 8;
      kraw[i] = *reinterpret_cast<const uint4*>(k + off);
      if (with_v) vraw[i] = *reinterpret_cast<const uint4*>(v + off);
    }
  }
}

// NWAVES waves of one 32-query tile each; one workgroup per window-head stages the window's K/V
// once and then walks its query blocks of NWAVES*32 queries.  MT: compile-time window size
// (0 = g.M at run time).  NPMAX: the largest padded window this configuration serves.
template <int NWAVES, int MT, int NPMAX>
__global__ __launch_bounds__(NWAVES * 64, NWAVES >= 8 ? 4 : 1) void fwd_mfma_kernel(const uint16_t* __restrict__ q,
                                                               const uint16_t* __restrict__ k,
                                                               const uint16_t* __restrict__ v,
                                                               const float* __restrict__ th_row,
                                                               const float* __restrict__ th_col,
                                                               uint16_t* __restrict__ out, float* __restrict__ lse,
                                                               Geom g, int nqb, int NP, int nsplit) {
  extern __shared__ __align__(16) unsigned char smem_raw[];
  constexpr int D = 32;
  constexpr int NT = NWAVES * 64;
  constexpr int MAXIT = (NPMAX * 4 + NT - 1) / NT;
  constexpr int QBM = (NPMAX + NWAVES * 32 - 1) / (NWAVES * 32);  // query blocks per window, at most
  static_assert(NWAVES <= kMaxWaves, "too many waves");
  static_assert(QBM <= kMaxQBlocks, "too many query blocks");
  const int M = MT > 0 ? MT : g.M;
  const int N = M * M;
  const int NB = NP / 32;
  const FwdSmem sm = carve(smem_raw, NP, M);

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
  const bool split = wo.ra != M || wo.ca != M;  // one window per workgroup: uniform
  for (int n = tid; n < NP; n += NT) {
    uint8_t lb = 0xff;
    if (n < N) {
      int r, c;
      slot_rc(wo, n, r, c);
      sm.rc[n] = (uint16_t)(r << 8 | c);
      lb = (uint8_t)token_label(g, w.wy, w.wx, r, c);
    }
    sm.lab[n] = lb;
  }
  if (split) __syncthreads();

  // 1. every global load of the thread (K and V items, the queries of every block)
  uint4 kraw[MAXIT], vraw[MAXIT];
  load_kv<MAXIT>(k, v, g, w, split ? sm.rc : nullptr, M, NP, tid, NT, true, kraw, vraw);
  // the lane's query of block qb (two 16-byte halves: channels 8h.., 16+8h..)
  auto load_q = [&](int qb, uint4& a, uint4& b) {
    const int qi = (qoff + qb) * NT / 2 + wave * 32 + col;
    a = b = make_uint4(0, 0, 0, 0);
    if (qb < nqw && qi < N) {
      const int rc = split ? (int)sm.rc[qi] : (qi / M) << 8 | (qi - (qi / M) * M);
      const int64_t off = tok_of(g, w, M, rc >> 8, rc & 255) * g.xs + w.h * D;
      a = *reinterpret_cast<const uint4*>(q + off + 8 * h);
      b = *reinterpret_cast<const uint4*>(q + off + 16 + 8 * h);
    }
  };
  uint4 qraw[QBM][2];
#pragma unroll
  for (int qb = 0; qb < QBM; ++qb) load_q(qb, qraw[qb][0], qraw[qb][1]);

  // 2. RoPE sin/cos table (while the loads are in flight)
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
  __syncthreads();

  // 3. K~ rows (rotated, fp16), V rows, block label summaries, norms
  float kmax2 = stage_k<MAXIT>(sm, kraw, M, split, NP, tid, NT, true);
#pragma unroll
  for (int i = 0; i < MAXIT; ++i) {
    const int it = tid + i * NT;
    if (it < NP * 4) *reinterpret_cast<uint4*>(sm.V + (size_t)(it >> 2) * 32 + (it & 3) * 8) = vraw[i];
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
  const float qscale = kLog2e * 0.17677669529663687f;  // log2(e) / sqrt(32)
  float qn2max[QBM];
#pragma unroll
  for (int qb = 0; qb < QBM; ++qb) {
    const float qn2 = halves_sum(norm2_bf16x8(qraw[qb][1], norm2_bf16x8(qraw[qb][0], 0.f)));
    qn2max[qb] = wave_max(qn2) * (qscale * qscale);
  }
  kmax2 = wave_max(kmax2);
  if (lane == 0) {
    float qm = 0.f;
#pragma unroll
    for (int qb = 0; qb < QBM; ++qb) qm = fmaxf(qm, qn2max[qb]);
    sm.red[wave] = kmax2;
    sm.red[kMaxWaves + wave] = qm;
  }
  __syncthreads();
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
    load_kv<MAXIT>(k, v, g, w, split ? sm.rc : nullptr, M, NP, tid, NT, false, kraw, vraw);
    __syncthreads();
    stage_k<MAXIT>(sm, kraw, M, split, NP, tid, NT, false);
    __syncthreads();
  }
#pragma unroll
  for (int qb = 0; qb < QBM; ++qb) {
    if (qb >= nqw) break;
    // 4. the wave's query operands (rotated, scaled by log2(e)/sqrt(d)), reference bound, labels
    const int qi = (qoff + qb) * NT / 2 + wave * 32 + col;
    const bool qvalid = qi < N;
    const int qrc = !qvalid ? 0 : split ? (int)sm.rc[qi] : (qi / M) << 8 | (qi - (qi / M) * M);
    const int qr = qrc >> 8, qc = qrc & 255;
    uint4 qb0, qb1;
    {
      // block 0's query was loaded with K and V; later blocks reload theirs (an L2 hit) during
      // the previous block's epilogue: keeping every block's raw query live across attend() costs
      // registers
      const uint4 qa = qraw[qb][0], qc2 = qraw[qb][1];
      float x[8], y[8];
      unpack8(qa, x);
      unpack8(qc2, y);
      rotate8(x, sm.sn, sm.cs, 0, M, qr, 4 * h);
      rotate8(y, sm.sn, sm.cs, 1, M, qc, 4 * h);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        x[e] *= qscale;
        y[e] *= qscale;
      }
      qb0 = pack8_op(x, h16);
      qb1 = pack8_op(y, h16);
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
    if (wave_single) {
      int bs, be;
      band_of(wo, uniform((qoff + qb) * NT / 2 + wave * 32), bs, be);
      run = ((bs | be) & 31) == 0 && (((be - bs) >> 5) & 1) == 0;
      kb0 = bs >> 5;
      kb1 = be >> 5;
    }

    f32x16_t o;
    float l = 0.f, ref;
#pragma unroll
    for (int v2 = 0; v2 < 16; ++v2) o[v2] = 0.f;
    if (h16)
      attend<true>(sm, NB, lane, run, kb0, kb1, wave_labels, wave_single, qb0, qb1, qlab, qvalid, bound, ref, l, o);
    else
      attend<false>(sm, NB, lane, run, kb0, kb1, wave_labels, wave_single, qb0, qb1, qlab, qvalid, bound, ref, l, o);

    // the next block's query loads go out before this block's epilogue
    if (qb + 1 < QBM) load_q(qb + 1, qraw[qb + 1][0], qraw[qb + 1][1]);  // zeros past the last block
    // 5. epilogue: O = O^T / l (lane: query col, channels 8g + 4h + j), LSE = (ref + log2 l) ln 2
    const float lt = halves_sum(l);
    if (qvalid) {
      const int64_t qtok = tok_of(g, w, M, qr, qc);
      const float inv = 1.f / lt;
      uint16_t* dst = out + qtok * g.os + w.h * D + 4 * h;
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) {
        uint2 pr;
        pr.x = pack2(o[4 * gq] * inv, o[4 * gq + 1] * inv);
        pr.y = pack2(o[4 * gq + 2] * inv, o[4 * gq + 3] * inv);
        *reinterpret_cast<uint2*>(dst + 8 * gq) = pr;
      }
      if (lse && h == 0) lse[qtok * g.heads + w.h] = (ref + __log2f(lt)) * kLn2;
    }
  }
}

template <int NWAVES, int MT, int NPMAX>
hipError_t launch_nw(const FwdArgs& a, hipStream_t st) {
  const Geom& g = a.g;
  const int NP = (g.N + 31) / 32 * 32;
  const int nqb = (g.N + NWAVES * 32 - 1) / (NWAVES * 32);
  const size_t smem = fwd_smem_bytes(NP, g.M);
  // The dynamic-LDS limit is raised on the current device, once per device (beyond kMaxDevices:
  // on every call).
  constexpr int kMaxDevices = 64;
  static std::once_flag once[kMaxDevices];
  const auto raise = [] {
    (void)hipFuncSetAttribute((const void*)fwd_mfma_kernel<NWAVES, MT, NPMAX>,
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
  hipLaunchKernelGGL((fwd_mfma_kernel<NWAVES, MT, NPMAX>), dim3((unsigned)blocks), dim3(NWAVES * 64), smem, st,
                     (const uint16_t*)a.q, (const uint16_t*)a.k, (const uint16_t*)a.v, a.th_row, a.th_col,
                     (uint16_t*)a.out, a.lse, g, nqb, NP, nsplit);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st) {
  const int N = a.g.N;
  if (a.g.M == 32) return launch_nw<16, 32, 1024>(a, st);
  if (fwd_m8_supported(a.g)) return launch_fwd_m8(a, st);
  if (a.g.M == 8) return launch_nw<2, 8, 64>(a, st);
  if (a.g.M == 16) return launch_nw<8, 16, 256>(a, st);
  if (N <= 64) return launch_nw<2, 0, 64>(a, st);
  if (N <= 128) return launch_nw<4, 0, 128>(a, st);
  if (N <= 256) return launch_nw<8, 0, 256>(a, st);
  return launch_nw<16, 0, 1024>(a, st);
}

}  // namespace fsw
