// bf16 window-attention forward on MFMA (gfx950): the shape limits and the plain kernels (the
// kernel, its design and its dispatch are in fwd_mfma_impl.h).
#include "fwd_mfma_impl.h"

namespace fsw {

bool fwd_mfma_supported(const Geom& g) {
  const int NP = (g.N + 31) / 32 * 32;
  return (g.d == 32 && g.M <= 32) || (g.d == 64 && NP <= kMaxNP64);
}

bool fwd_mfma_lowrank_supported(const Geom& g, int rank) {
  const int NP = (g.N + 31) / 32 * 32;
  return g.d == 32 && NP <= kMaxNPLowRank && rank >= 1 && rank <= 32 && g.Hp == g.Hg && g.Wp == g.Wg;
}

hipError_t launch_fwd_mfma(const FwdArgs& a, hipStream_t st) {
  return a.stats ? launch_fwd_mfma_stats(a, st) : launch_fwd_mfma_impl<false>(a, st);
}

}  // namespace fsw
