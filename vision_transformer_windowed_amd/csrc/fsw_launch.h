// Host-side launch interface between the C ABI (fsw_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fsw_common.h"

namespace fsw {

// Largest rank of the low-rank additive bias factors.
constexpr int kMaxRank = 32;

// Optional rank-r additive bias: per head, factors U, W [heads, M*M, rank] (float32) over in-window
// positions; the pair (i, j) adds U[n_i] . W[n_j] to its scaled score.  rank == 0: no bias.
struct LowRank {
  const float* u = nullptr;
  const float* w = nullptr;
  int rank = 0;
};

struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const float* th_row;
  const float* th_col;
  void* out;
  float* lse;  // may be null
  Geom g;
  int dtype;  // 0 = float32, 1 = bf16
  LowRank lr = {};
  // Optional (bf16, d 32 or 64): per window-head operand maxima for the backward, [windows*heads][4]
  // = {max |q| over the queries of a first workgroup, of a second (0 if none), max |k|, max |v|}.
  float* stats = nullptr;
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* out;
  const void* dout;
  const float* lse;
  const float* th_row;
  const float* th_col;
  void* dq;
  void* dk;
  void* dv;
  float* dth_row;
  float* dth_col;
  Geom g;
  int dtype;
  // workspace carve-up (device pointers inside the caller's workspace)
  float* delta;     // [B*Hg*Wg*heads]  rowsum(dO * O)
  float* scal;      // [windows*heads][4]  per window-head: max |dO|, max |v|, max |q|, max |k| components
  float* partials;  // [n_partials][2][d/4]  per-workgroup dtheta partial sums
  int64_t n_partials;
  LowRank lr = {};
  float* du = nullptr;      // [heads, M*M, rank]  gradient of the bias factors (rank > 0)
  float* dw = nullptr;
  float* lr_parts = nullptr;  // [2][windows][heads][M*M][rank]  per-window factor gradients (rank > 0)
  // The forward's operand maxima (FwdArgs::stats) or null: with them the prologue reads only O and dO.
  const float* stats = nullptr;
};

// Scalar (float32-arithmetic) paths: any d in {8,16,32,64}, any window size, either dtype, with or
// without a low-rank bias.
hipError_t launch_fwd_scalar(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_scalar(const BwdArgs& a, hipStream_t st);
// Number of dtheta partial rows the scalar backward writes.
int64_t bwd_scalar_partials(const Geom& g);

// bf16 MFMA forward: d == 32 with M <= 32, and d == 64 with at most 512 padded window tokens
// (M <= 22), where the window's K~ and V rows fit LDS.
bool fwd_mfma_supported(const Geom& g);
// The MFMA forward with a low-rank bias: bf16, d == 32, at most 512 padded window tokens, rank <= 32,
// grids that M divides.
bool fwd_mfma_lowrank_supported(const Geom& g, int rank);
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st);
// The same with a.stats set: the kernels that also write the operand maxima (fwd_mfma_stats.hip).
hipError_t launch_fwd_mfma_stats(const FwdArgs& a, hipStream_t st);
// FwdArgs::stats of a bf16 forward (d 32 or 64) from q, k and v, for the forward kernels that do not
// produce them.
hipError_t launch_operand_maxima(const FwdArgs& a, hipStream_t st);
// M = 8 windows: one wave per window-head.
bool fwd_m8_supported(const Geom& g);
hipError_t launch_fwd_m8(const FwdArgs& a, hipStream_t st);
// bf16 MFMA backward (d == 32, M <= 32).
hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t st);
// Its prologue alone (bf16, d == 32): Delta and the per-window-head maxima into a.delta, a.scal.
hipError_t launch_bwd_pre32(const BwdArgs& a, hipStream_t st);
int64_t bwd_mfma_partials(const Geom& g);
// bf16 MFMA backward for d == 64 and windows of at most 256 tokens.
bool bwd_d64_supported(const Geom& g);
hipError_t launch_bwd_d64(const BwdArgs& a, hipStream_t st);
// bf16 MFMA backward with a low-rank bias: d == 32, windows of at most 256 tokens, rank <= 32, grids
// that M divides.  Its workspace needs lowrank_mfma_extra_floats(g) floats after the float32 kernels'
// two [windows][heads][M*M][rank] blocks: up to a 256-byte boundary, the factors zero-padded to 32
// channels, and two maxima per head.
bool bwd_lowrank_mfma_supported(const Geom& g, int rank);
hipError_t launch_bwd_lowrank_mfma(const BwdArgs& a, hipStream_t st);
inline int64_t lowrank_mfma_extra_floats(const Geom& g) {
  return 64 + 2 * (int64_t)g.heads * g.N * kMaxRank + 2 * (int64_t)g.heads;
}
// dtheta partial rows of the whole-window kernels (d == 64, and the low-rank ones).
int64_t bwd_window_partials(const Geom& g);
constexpr bool kHaveMfmaBwd = true;

// Materialized comparison path (bf16, d == 32): scores in HBM, softmax, P.V.
size_t materialized_workspace_bytes(const Geom& g);
hipError_t launch_fwd_materialized(const FwdArgs& a, const float* bias, void* workspace, hipStream_t st);

// Factor gradients: out[e] = sum over rows r < nrows of parts[r * per_row + e], in a fixed order.
hipError_t launch_lowrank_reduce(const float* parts, int64_t nrows, int64_t per_row, float* out, hipStream_t st);

// Deterministic fixed-order reduction of dtheta partials into dth_row / dth_col.
hipError_t launch_dtheta_reduce(const float* partials, int64_t n_partials, int64_t partials_per_head_stride,
                                const Geom& g, float* dth_row, float* dth_col, hipStream_t st);

}  // namespace fsw
