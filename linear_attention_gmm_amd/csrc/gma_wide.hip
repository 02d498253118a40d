// gma_wide.hip -- the general GMA kernel instantiated for bf16 inputs with
// d = dv = 128 and 256 (padded) components. It is built in its own translation
// unit so that its MFMA accumulators can be kept in VGPRs (the other
// instantiations are compiled without that option).
#include "gma_generic.hpp"

namespace lm {
namespace gma {

// The segment pass and the bidirectional read run eight waves of 32 components
// (two waves per SIMD: the routing latency of one wave hides behind the other);
// the causal pass keeps four waves of 64 components, since its per-wave read
// partials and state do not fit 256 registers at eight waves.
hipError_t wide_launch(const Args& a, int mode, int segments, unsigned BH, hipStream_t st) {
  if (mode == CAUSAL) return launch_mode<bf16, 128, 4, 64>(a, mode, segments, BH, st);
  return launch_mode<bf16, 128, 8, 32>(a, mode, segments, BH, st);
}

}  // namespace gma
}  // namespace lm
