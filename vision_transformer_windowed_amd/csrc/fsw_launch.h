// Host-side launch interface between the C ABI (fsw_api.hip) and the kernel files.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "fsw_common.h"

namespace fsw {

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
};

// Scalar (float32-arithmetic) paths: any d in {8,16,32,64}, any M <= 32, either dtype.
hipError_t launch_fwd_scalar(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_scalar(const BwdArgs& a, hipStream_t st);
// Number of dtheta partial rows the scalar backward writes.
int64_t bwd_scalar_partials(const Geom& g);

// bf16 MFMA paths (d == 32, M <= 32).
hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st);
// M = 8 windows: one wave per window-head.
bool fwd_m8_supported(const Geom& g);
hipError_t launch_fwd_m8(const FwdArgs& a, hipStream_t st);
hipError_t launch_bwd_mfma(const BwdArgs& a, hipStream_t st);
int64_t bwd_mfma_partials(const Geom& g);
constexpr bool kHaveMfmaBwd = true;

// Deterministic fixed-order reduction of dtheta partials into dth_row / dth_col.
hipError_t launch_dtheta_reduce(const float* partials, int64_t n_partials, int64_t partials_per_head_stride,
                                const Geom& g, float* dth_row, float* dth_col, hipStream_t st);

}  // namespace fsw
