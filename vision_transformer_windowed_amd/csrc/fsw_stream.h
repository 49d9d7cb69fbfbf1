// Helpers shared by the kernels that stream one side of a window through LDS in chunks
// (the backward's dK/dV and dQ kernels).
#pragma once

#include "fsw_common.h"
#include "fsw_mfma.h"

namespace fsw {

constexpr int kCh = 128;  // tokens per LDS chunk by default (chunk lengths are multiples of 128)

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ uint32_t uniform(uint32_t x) { return (uint32_t)__builtin_amdgcn_readfirstlane((int)x); }

// Chunk length of the kernels specialised for window size MT (0: run-time size): a window of 256
// tokens (M = 16) streams as one chunk, so each workgroup passes one pair of barriers, not two.
__host__ __device__ constexpr int chunk_max(int MT) { return MT == 16 ? 256 : kCh; }
__host__ __device__ constexpr int chunk_len(int NP, int cmax = kCh) { return NP < cmax ? NP : cmax; }

template <bool H16>
__device__ __forceinline__ uint32_t pack_op2(float a, float b) {
  if constexpr (H16)
    return pack2h(a, b);
  else
    return pack2(a, b);
}

__device__ inline void fill_table(float* sn, float* cs, const float* th_row, const float* th_col, int head, int M,
                                  int tid, int nt) {
  for (int i = tid; i < 2 * M * 8; i += nt) {
    const int axis = i / (M * 8);
    const int p = (i / 8) % M;
    const int j = i % 8;
    const float th = axis ? th_col[head * 8 + j] : th_row[head * 8 + j];
    float s, c;
    rope_sincos(th, p, &s, &c);
    sn[i] = s;
    cs[i] = c;
  }
}

// Rotate the 8 channels of `raw` (part `part` of token (r, c)), scale, pack to the operand format.
template <bool H16>
__device__ __forceinline__ uint4 rotated_part(uint4 raw, const float* sn, const float* cs, int M, int r, int c,
                                              int part, float scale) {
  float x[8];
  unpack8(raw, x);
  const int axis = part >> 1;
  rotate8(x, sn, cs, axis, M, axis ? c : r, (part & 1) * 4);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= scale;
  return pack8_op(x, H16);
}

// Scale 8 bf16 values by a power of two; result in the operand format.
template <bool H16>
__device__ __forceinline__ uint4 scaled_part(uint4 raw, float scale) {
  float x[8];
  unpack8(raw, x);
#pragma unroll
  for (int e = 0; e < 8; ++e) x[e] *= scale;
  return pack8_op(x, H16);
}

// Labels (bit L for label L) of the tokens in slots [a, b) of a window, from its region bands: each
// band is one contiguous slot range of one label (see WinOrder).
__device__ inline uint32_t range_labels(const Geom& g, const WinHead& w, const WinOrder& o, int a, int b) {
  const int M = o.M;
  const int e[5] = {0, o.ra * o.ca, o.ra * M, o.ra * M + (M - o.ra) * o.ca, M * M};
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (e[i] < e[i + 1] && e[i] < b && a < e[i + 1]) {
      int r, c;
      slot_rc(o, e[i], r, c);
      m |= 1u << token_label(g, w.wy, w.wx, r, c);
    }
  }
  return m;
}

// Label of chunk slot tn, staged at chunk position n (0xff past the window and for the padding of a
// padded grid), and its block summary bit (bit L for label L, bit 10 for a position past the window or
// padding) OR-ed into blk[n / 32].
// PAD: the grid may be padded (instances for padded grids only).
template <bool PAD>
__device__ __forceinline__ uint8_t chunk_label(const Geom& g, const WinHead& w, const WinOrder& wo, int tn,
                                               uint32_t* blk, int n) {
  const int N = wo.M * wo.M;
  uint8_t lb = 0xff;
  if (tn < N) {
    int r, c;
    slot_rc(wo, tn, r, c);
    if (!PAD || token_real(g, w.wy, w.wx, r, c)) lb = (uint8_t)token_label(g, w.wy, w.wx, r, c);
  }
  atomicOr(&blk[n >> 5], lb == 0xff ? (1u << 10) : (1u << lb));
  return lb;
}

}  // namespace fsw
