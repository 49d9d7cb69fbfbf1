// Device-side helpers shared by the window-attention kernels (gfx950).
//
// Window/shift index arithmetic, Swin region labels, 2D RoPE angles and bf16 packing.
// Conventions follow the FlashSwin paper card ("FLASHSWIN: Unlocking Large Windows and Dense
// Tokens in Swin Vision Transformers with Memory Efficient Attention"): exact window attention
// with window-local 2D RoPE on Q and K (Abstract; Figure 1(B)); the shifted-window mask follows
// Swin's cyclic shift with three row and three column regions.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fsw {

// Shape of one call, passed to kernels by value.  A grid whose sides M does not divide is taken as
// padded to Hp x Wp (the next multiples of M), as Swin pads its feature map before the shift: the
// roll, the windows and the regions are those of Hp x Wp, and the added tokens (row >= Hg or column
// >= Wg) are absent, no key of any query and no output.  Every kernel family but the M = 8 forward
// variant and the materialized comparison takes padded grids; elsewhere Hp == Hg and Wp == Wg.
struct Geom {
  int64_t B;
  int Hg, Wg, heads, d, M, shift;
  int nH, nW;  // windows per image along rows / columns: Hp / M, Wp / M
  int Hp, Wp;  // padded extents
  int N;       // tokens per window, M*M
  int64_t xs;  // elements between consecutive tokens of q, k, v and of dq, dk, dv
  int64_t os;  // elements between consecutive tokens of out and dout (heads * d)
};

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// XCD-aware workgroup order.  Workgroup b is dispatched to XCD b % 8 and each XCD has its own L2;
// the returned logical index gives every XCD a contiguous range, so workgroups with neighbouring
// logical indices (the heads and blocks of one window, which read the same token rows) share one
// L2.  A bijection of [0, n).
__device__ __forceinline__ int64_t xcd_order(int64_t b, int64_t n) {
  const int64_t q = n >> 3, r = n & 7, x = b & 7;
  return x * q + (x < r ? x : r) + (b >> 3);
}

// Grid row (or column) of shifted-frame coordinate Y: (Y + shift) mod size, with Y < size.
__device__ __forceinline__ int grid_coord(int Y, int shift, int size) {
  int y = Y + shift;
  return y >= size ? y - size : y;
}

// Swin region of shifted-frame coordinate Y: 0 for [0, size-M), 1 for [size-M, size-shift),
// 2 for [size-shift, size).  Always 0 without a shift.
__device__ __forceinline__ int region_of(int Y, int size, int M, int shift) {
  return shift ? (int)(Y >= size - M) + (int)(Y >= size - shift) : 0;
}

// Label of in-window token (r, c) of window (wy, wx); tokens attend only to equal labels.
__device__ __forceinline__ int token_label(const Geom& g, int wy, int wx, int r, int c) {
  return 3 * region_of(wy * g.M + r, g.Hp, g.M, g.shift) + region_of(wx * g.M + c, g.Wp, g.M, g.shift);
}

// Order in which the kernels enumerate a window's tokens ("slots"): grouped by Swin region, so that
// runs of consecutive slots share one label and whole 32-slot blocks are either attended without a
// mask or skipped.  In the shifted frame a window's rows fall into at most two bands, [0, ra) and
// [ra, M): ra = M - shift in the last window row of a shifted grid, ra = M (one band) elsewhere.  The
// columns likewise with ca.  Slots enumerate band (rows 0, cols 0) row-major, then (0, 1), (1, 0),
// (1, 1); a window without a split is plain row-major, slot = r * M + c.  Softmax attention does not
// depend on the order of the keys, and each query keeps its own (r, c), so results are unchanged.
struct WinOrder {
  int M, ra, ca;
};
__device__ __forceinline__ WinOrder win_order(const Geom& g, int M, int wy, int wx) {
  WinOrder o;
  o.M = M;
  o.ra = (g.shift > 0 && wy == g.nH - 1) ? M - g.shift : M;
  o.ca = (g.shift > 0 && wx == g.nW - 1) ? M - g.shift : M;
  return o;
}
// In-window position (r, c) of slot j < M * M.
__device__ __forceinline__ void slot_rc(const WinOrder& o, int j, int& r, int& c) {
  const int M = o.M;
  if (o.ra == M && o.ca == M) {  // uniform across the workgroup: one window
    r = j / M;
    c = j - r * M;
    return;
  }
  const int n00 = o.ra * o.ca, n01 = o.ra * (M - o.ca), n10 = (M - o.ra) * o.ca;
  int r0 = 0, c0 = 0, w = o.ca;
  if (j >= n00) {
    j -= n00;
    if (j < n01) {
      c0 = o.ca;
      w = M - o.ca;
    } else {
      j -= n01;
      r0 = o.ra;
      if (j >= n10) {
        j -= n10;
        c0 = o.ca;
        w = M - o.ca;
      }
    }
  }
  // j / w by a float reciprocal: with j < 4096 and w <= 64 (M <= 64) the quotient (j + 1/2) / w lies at
  // least 1/(2w) >= 2^-7 from an integer, far beyond the float error of the product (< 2^-10)
  const int qt = (int)(((float)j + 0.5f) * __builtin_amdgcn_rcpf((float)w));
  r = r0 + qt;
  c = c0 + j - qt * w;
}

// Token index (b, y, x) in the grid of in-window position (r, c) of window (wy, wx) of image b; the
// position must not be padding (token_real).
__device__ __forceinline__ int64_t token_index(const Geom& g, int64_t b, int wy, int wx, int r, int c) {
  const int y = grid_coord(wy * g.M + r, g.shift, g.Hp);
  const int x = grid_coord(wx * g.M + c, g.shift, g.Wp);
  return (b * g.Hg + y) * g.Wg + x;
}

// Whether in-window position (r, c) of window (wy, wx) is a grid token rather than padding.
__device__ __forceinline__ bool token_real(const Geom& g, int wy, int wx, int r, int c) {
  return grid_coord(wy * g.M + r, g.shift, g.Hp) < g.Hg && grid_coord(wx * g.M + c, g.shift, g.Wp) < g.Wg;
}

// Decompose a flat window-head index wh = ((b*nH + wy)*nW + wx)*heads + h.
struct WinHead {
  int64_t b;
  int wy, wx, h;
};
__device__ __forceinline__ WinHead decode_winhead(const Geom& g, int64_t wh) {
  WinHead r;
  r.h = (int)(wh % g.heads);
  int64_t w = wh / g.heads;
  r.wx = (int)(w % g.nW);
  w /= g.nW;
  r.wy = (int)(w % g.nH);
  r.b = w / g.nH;
  return r;
}

// sin and cos of theta * p with the rounding error of the product folded back in to first order,
// so angles up to ~|theta| * M stay accurate to float32 resolution of sin/cos themselves.
__device__ __forceinline__ void rope_sincos(float theta, int p, float* s, float* c) {
  const float fp = (float)p;
  const float phi = theta * fp;
  const float err = __builtin_fmaf(theta, fp, -phi);
  float sv, cv;
  sincosf(phi, &sv, &cv);
  *s = __builtin_fmaf(err, cv, sv);
  *c = __builtin_fmaf(-err, sv, cv);
}

// Rotate the D channels of one token/head in place: row axis on [0, D/2), column axis on [D/2, D).
template <int D>
__device__ __forceinline__ void rope_rotate(float (&x)[D], const float* th_row, const float* th_col, int r, int c) {
#pragma unroll
  for (int j = 0; j < D / 4; ++j) {
    float s, co;
    rope_sincos(th_row[j], r, &s, &co);
    float a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * co - b * s;
    x[2 * j + 1] = a * s + b * co;
    rope_sincos(th_col[j], c, &s, &co);
    a = x[D / 2 + 2 * j];
    b = x[D / 2 + 2 * j + 1];
    x[D / 2 + 2 * j] = a * co - b * s;
    x[D / 2 + 2 * j + 1] = a * s + b * co;
  }
}

// Inverse rotation (angle -phi), used to pull gradients back through RoPE.
template <int D>
__device__ __forceinline__ void rope_unrotate(float (&x)[D], const float* th_row, const float* th_col, int r, int c) {
#pragma unroll
  for (int j = 0; j < D / 4; ++j) {
    float s, co;
    rope_sincos(th_row[j], r, &s, &co);
    float a = x[2 * j], b = x[2 * j + 1];
    x[2 * j] = a * co + b * s;
    x[2 * j + 1] = -a * s + b * co;
    rope_sincos(th_col[j], c, &s, &co);
    a = x[D / 2 + 2 * j];
    b = x[D / 2 + 2 * j + 1];
    x[D / 2 + 2 * j] = a * co + b * s;
    x[D / 2 + 2 * j + 1] = -a * s + b * co;
  }
}

// ---- element I/O -------------------------------------------------------------------------------

__device__ __forceinline__ float bf16_bits_to_float(uint16_t u) { return __uint_as_float(((uint32_t)u) << 16); }

// Round-to-nearest-even float -> bf16 bits (hardware conversion on gfx950).
__device__ __forceinline__ uint16_t float_to_bf16_bits(float f) {
  __bf16 h = (__bf16)f;
  return __builtin_bit_cast(uint16_t, h);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)lo;
  v[1] = (__bf16)hi;
  return __builtin_bit_cast(uint32_t, v);
}

// Load / store D consecutive elements of float or bf16 (uint16_t) storage as float.
template <int D>
__device__ __forceinline__ void load_row(const float* p, float (&x)[D]) {
#pragma unroll
  for (int i = 0; i < D; i += 4) {
    const float4 t = *reinterpret_cast<const float4*>(p + i);
    x[i] = t.x;
    x[i + 1] = t.y;
    x[i + 2] = t.z;
    x[i + 3] = t.w;
  }
}
template <int D>
__device__ __forceinline__ void load_row(const uint16_t* p, float (&x)[D]) {
#pragma unroll
  for (int i = 0; i < D; i += 8) {
    const uint4 t = *reinterpret_cast<const uint4*>(p + i);
    const uint32_t w[4] = {t.x, t.y, t.z, t.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      x[i + 2 * e] = __uint_as_float(w[e] << 16);
      x[i + 2 * e + 1] = __uint_as_float(w[e] & 0xffff0000u);
    }
  }
}
template <int D>
__device__ __forceinline__ void store_row(float* p, const float (&x)[D]) {
#pragma unroll
  for (int i = 0; i < D; i += 4) *reinterpret_cast<float4*>(p + i) = make_float4(x[i], x[i + 1], x[i + 2], x[i + 3]);
}
template <int D>
__device__ __forceinline__ void store_row(uint16_t* p, const float (&x)[D]) {
#pragma unroll
  for (int i = 0; i < D; i += 8) {
    uint4 t;
    t.x = pack_bf16x2(x[i], x[i + 1]);
    t.y = pack_bf16x2(x[i + 2], x[i + 3]);
    t.z = pack_bf16x2(x[i + 4], x[i + 5]);
    t.w = pack_bf16x2(x[i + 6], x[i + 7]);
    *reinterpret_cast<uint4*>(p + i) = t;
  }
}

}  // namespace fsw
