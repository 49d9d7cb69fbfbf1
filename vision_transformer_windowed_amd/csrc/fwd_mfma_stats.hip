// The MFMA forward's kernels that also write the per-window-head operand maxima for the backward
// (FwdArgs::stats), in a translation unit of their own (see fwd_mfma_impl.h).
#include "fwd_mfma_impl.h"

namespace fsw {

hipError_t launch_fwd_mfma_stats(const FwdArgs& a, hipStream_t st) { return launch_fwd_mfma_impl<true>(a, st); }

}  // namespace fsw
