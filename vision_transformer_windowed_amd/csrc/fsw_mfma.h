// MFMA helpers for gfx950 (CDNA4): bf16 32x32x16 tiles, operand layouts, LDS layout of a window.
//
// v_mfma_f32_32x32x16_bf16, D[32x32] += A[32x16] * B[16x32], wave64.  Lane l (h = l / 32):
//   A: row l % 32, k = 8h .. 8h+7            (8 bf16 per lane)
//   B: col l % 32, k = 8h .. 8h+7            (8 bf16 per lane)
//   D: col l % 32, value v (0..15) at row 8*(v/4) + 4h + (v%4)
// The attention tiles are transposed (S^T = K~ Q^T, O^T = V^T P^T) so that a lane owns one query:
// its 16 score values all belong to query l % 32, and its O^T values are that query's channels.
// A lane's 16 scores cover keys 8g + 4h + j (g, j in 0..3) of a 32-key block; the P.V product
// takes them as B operands of two MFMAs (keys with g in {0,1}, then {2,3}), which fixes the order
// in which V^T must present the keys: within each 16-key group, positions 4..7 and 8..11 swap.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsw {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ f32x16_t mfma32x32x16(const bf16x8_t& a, const bf16x8_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Score products S = q^ . k~ take operands that are computed in float32 (rotation, scaling), so
// they are rounded to fp16 (11-bit significand) when every operand is in fp16 range, else to bf16.
// Raw operand bits travel as uint4; H16 selects the format and the MFMA.
template <bool H16>
__device__ __forceinline__ f32x16_t mfma_op(uint4 a, uint4 b, const f32x16_t& c) {
  if constexpr (H16)
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8_t, a), __builtin_bit_cast(f16x8_t, b), c,
                                                  0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                   c, 0, 0, 0);
}

// ds_read_b64_tr_b16 (gfx950): a group of 16 lanes loads 16 x 8 bytes and redistributes the
// 16-bit elements: output lane i of the group receives, in slot m, element (i % 4) of the chunk
// addressed by lane 4m + i/4 of the group.  If lane 4m + q addresses 4 consecutive channels
// 4q..4q+3 of key row m, output lane i holds channel i of keys 0..3: a row-major [key][channel]
// tile is read transposed, as the MFMA k-dimension needs it.
__device__ __forceinline__ uint2 lds_read_tr16(const uint16_t* p) {
  typedef short v4s __attribute__((ext_vector_type(4)));
  const v4s r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) v4s*)(p));
  return __builtin_bit_cast(uint2, r);
}

// A operand (8 values of one channel) for the P.V / dO^T.P style products from a row-major
// [key][32 channels] LDS array with row stride `rs` elements: lane l supplies channel l % 32 of
// the keys in slot order 4h + {0..3}, 8 + 4h + {0..3} (h = l / 32) of the 16-key group at `k0`,
// matching the key order of the score accumulator (keys 8g + 4h + j).
__device__ __forceinline__ uint4 tr_operand(const uint16_t* rows, int rs, int k0, int lane) {
  const int j = lane & 15;
  const int key = k0 + 4 * (lane >> 5) + (j >> 2);
  const uint16_t* p = rows + (size_t)key * rs + (lane & 16) + 4 * (j & 3);
  const uint2 lo = lds_read_tr16(p);
  const uint2 hi = lds_read_tr16(p + 8 * rs);
  return make_uint4(lo.x, lo.y, hi.x, hi.y);
}

// Swizzled LDS tile of [token][32 channels] 16-bit values: 64-byte rows, and the 16-byte chunk c
// (channels 8c..8c+7) of row n stored at chunk c ^ ((n / 4) % 4).  The MFMA row reads (16 rows,
// the same chunk) and the transposed reads (4 rows x 64 bytes per 32 lanes) then touch every LDS
// bank once.  Element offset of chunk c of row n:
__host__ __device__ __forceinline__ int srow(int n, int c) { return n * 32 + ((c ^ ((n >> 2) & 3)) << 3); }

// Per-lane element offsets (relative to a 16-row group) of the two ds_read_b64_tr_b16 reads that
// build a tr_operand-ordered operand from a swizzled tile: the group at row k0 (k0 % 16 == 0) is at
// k0 * 32 + lo and k0 * 32 + hi.
__device__ __forceinline__ void srow_tr_offsets(int lane, int& lo, int& hi) {
  const int j = lane & 15;
  const int key = 4 * (lane >> 5) + (j >> 2);
  const int ch = (lane & 16) + 4 * (j & 3);
  lo = srow(key, ch >> 3) + (ch & 7);
  hi = srow(key + 8, ch >> 3) + (ch & 7);
}

__device__ __forceinline__ uint4 tr_operand_at(const uint16_t* base, int lo, int hi) {
  const uint2 a = lds_read_tr16(base + lo);
  const uint2 b = lds_read_tr16(base + hi);
  return make_uint4(a.x, a.y, b.x, b.y);
}

// Largest operand magnitude accepted for the fp16 score products (fp16 max is 65504).
constexpr float kF16Limit = 16384.f;

// Factor that turns the Cauchy-Schwarz bound max|q^| * max|k~| into a softmax reference that no
// computed score exceeds.  Rounding q^ and k~ to the operand format (unit roundoff u = 2^-11 for
// fp16, 2^-8 for bf16) moves a product sum by at most (2u + u^2) |q^| |k~|; the float32 rotation,
// norms and accumulation add far less than 2^-16 of the bound.  Without the margin a score of an
// aligned query and key with large norms can exceed the bare bound by more than 128 (log2 units),
// and exp2 of it overflows.
template <bool H16>
__device__ __forceinline__ constexpr float bound_margin() {
  return H16 ? 1.f + 0x1p-10f + 0x1p-16f : 1.f + 0x1p-7f + 0x1p-16f;
}

__device__ __forceinline__ uint32_t pack2h(float lo, float hi) {
  f16x2_t v;
  v[0] = (_Float16)lo;
  v[1] = (_Float16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// fp16 pair (lo, hi) = (a0 * b0, a1 * b1): float32 products rounded once to fp16 (v_fma_mix with
// a zero addend; ALU only).
__device__ __forceinline__ uint32_t mul2h(float a0, float b0, float a1, float b1) {
  uint32_t r;
  asm("v_fma_mixlo_f16 %0, %1, %2, 0" : "=v"(r) : "v"(a0), "v"(b0));
  asm("v_fma_mixhi_f16 %0, %1, %2, 0" : "+v"(r) : "v"(a1), "v"(b1));
  return r;
}

// Pack 8 floats into 8 fp16 (h16) or bf16 values.
__device__ __forceinline__ uint4 pack8_op(const float (&x)[8], bool h16) {
  if (h16) return make_uint4(pack2h(x[0], x[1]), pack2h(x[2], x[3]), pack2h(x[4], x[5]), pack2h(x[6], x[7]));
  typedef __bf16 b2 __attribute__((ext_vector_type(2)));
  uint32_t w[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    b2 v;
    v[0] = (__bf16)x[2 * e];
    v[1] = (__bf16)x[2 * e + 1];
    w[e] = __builtin_bit_cast(uint32_t, v);
  }
  return make_uint4(w[0], w[1], w[2], w[3]);
}

// Storage position of key w (0..15 within its 16-key group) in the V^T rows.
__device__ __forceinline__ int vt_pos(int key) {
  const int w = key & 15;
  const int sw = ((w >> 2) == 1 || (w >> 2) == 2) ? (w ^ 12) : w;  // swap quads 1 and 2
  return (key & ~15) | sw;
}

// LDS layout of one staged window-head (bf16 d = 32):
//   K~ rows: NP keys x 40 bf16 (32 channels + 16 bytes pad: conflict-free 16-byte row reads)
//   V^T rows: 32 channels x (NP + 8) bf16 (keys in vt_pos order, 16 bytes pad)
constexpr int kKStride = 40;
__host__ __device__ constexpr int vt_stride(int np) { return np + 8; }

__device__ __forceinline__ bf16x8_t as_bf16x8(uint4 u) { return __builtin_bit_cast(bf16x8_t, u); }

__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// sum of a packed bf16 pair added to acc in float32 (v_dot2 with (1, 1))
__device__ __forceinline__ float add_pair(uint32_t pair, float acc) {
  const bf16x2_t ones = {(__bf16)1.0f, (__bf16)1.0f};
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, pair), ones, acc, false);
}

// x of lane l plus x of lane l ^ 32, in both lanes (v_permlane32_swap exchanges the wave's halves:
// the two results hold, in each lane, its own value and its partner's).
__device__ __forceinline__ float halves_sum(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float halves_max(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// Sum of squares of the 8 bf16 values packed in t, by bf16 pair dot products (the products are
// exact in float32).
__device__ __forceinline__ float norm2_bf16x8(uint4 t, float acc) {
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, t.x), __builtin_bit_cast(bf16x2_t, t.x), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, t.y), __builtin_bit_cast(bf16x2_t, t.y), acc, false);
  acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, t.z), __builtin_bit_cast(bf16x2_t, t.z), acc, false);
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, t.w), __builtin_bit_cast(bf16x2_t, t.w), acc,
                                         false);
}

// Sum over each group of 4 consecutive lanes, in all four (DPP quad permutations).
__device__ __forceinline__ float quad_sum(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0xB1, 0xf, 0xf, false));  // [1,0,3,2]
  return x + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x4E, 0xf, 0xf, false));  // [2,3,0,1]
}

// Running maximum of |x| over the two bf16 values of a pair, kept as two 16-bit integers: |x| of a
// bf16 value orders as its bits with the sign cleared.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t absmax_pair(uint32_t acc, uint32_t pair) {
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, acc),
                                                                __builtin_bit_cast(u16x2_t, pair & 0x7fff7fffu)));
}
// The larger of the two maxima as a float; a NaN component counts as infinity.
__device__ __forceinline__ float absmax_value(uint32_t acc) {
  return __uint_as_float(min(max(acc & 0xffffu, acc >> 16), 0x7f80u) << 16);
}
// absmax_pair over the four pairs of eight bf16 values.
__device__ __forceinline__ uint32_t absmax_x8(uint32_t acc, const uint4& x) {
  return absmax_pair(absmax_pair(absmax_pair(absmax_pair(acc, x.x), x.y), x.z), x.w);
}

__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o, 64));
  return x;
}
__device__ __forceinline__ uint32_t wave_or(uint32_t x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x |= (uint32_t)__shfl_xor((int)x, o, 64);
  return x;
}

// Rotate 8 consecutive channels (4 pairs) with the LDS sin/cos table [axis][position][p4] (p4 = d/4
// pairs per axis); pairs j0..j0+3 of `axis`.
__device__ __forceinline__ void rotate8(float (&x)[8], const float* sn, const float* cs, int axis, int M, int p,
                                        int j0, int p4 = 8) {
  const float* s = sn + (axis * M + p) * p4 + j0;
  const float* c = cs + (axis * M + p) * p4 + j0;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const float a = x[2 * u], b = x[2 * u + 1];
    x[2 * u] = a * c[u] - b * s[u];
    x[2 * u + 1] = a * s[u] + b * c[u];
  }
}

// 16-byte load marked non-temporal, for data that is read once and need not stay in the caches.
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint4 load_stream(const void* p) {
  const u32x4_t t = __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
  return make_uint4(t.x, t.y, t.z, t.w);
}

__device__ __forceinline__ void unpack8(uint4 t, float (&x)[8]) {
  const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    x[2 * e] = __uint_as_float(w[e] << 16);
    x[2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
  }
}

// Per-element live mask for the lane's 16 scores in key block kb: keys kb*32 + 8g + 4h + j.
__device__ __forceinline__ uint32_t live_bits(const uint8_t* lab, int kb, int h, int qlab) {
  uint32_t bits = 0;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const uint32_t w = *reinterpret_cast<const uint32_t*>(lab + kb * 32 + 8 * g + 4 * h);
#pragma unroll
    for (int j = 0; j < 4; ++j)
      if (((w >> (8 * j)) & 0xff) == (uint32_t)qlab) bits |= 1u << (4 * g + j);
  }
  return bits;
}

}  // namespace fsw
