// gma.hpp -- pieces of the Gaussian Mixture Attention forward shared by its
// kernels (gma.hip: parameter prep, segment scan, generic kernel, dispatch;
// gma_bf16.hip: the bf16 kernel for d <= 64 and up to 128 components).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace lm {
namespace gma {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kChunk = 64;
// Logit (log2 units) of padded components: finite, so max/subtract need no
// special case, and far enough below any real logit that exp2 of the
// difference is exactly 0.
constexpr float kPadLogit = -1.0e30f;

// AGG: per-segment state [Vtil | Z] only. CAUSAL: outputs, starting from the
// exclusive prefix of the earlier segments. BIDIR: outputs against the total.
// AGG_G and CAUSAL_G (bf16 kernels only): AGG that also stores each chunk's key
// responsibilities (the bf16 tile as it sits in LDS), and CAUSAL that loads
// them instead of routing the keys again.
enum Mode { AGG = 0, CAUSAL = 1, BIDIR = 2, AGG_G = 3, CAUSAL_G = 4 };

struct Args {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const void* W;   // [H][KP][2D]
  const float* c;  // [H][KP]
  float* agg;      // [B*H][P][KP][DV]
  float* aggz;     // [B*H][P][KP]
  int64_t N;
  int H;
  int P;         // segments in the workspace layout
  int seg_len;   // tokens per segment (multiple of 64)
  int KP;
  int has_init;  // CAUSAL/BIDIR: start from agg slot (p, or 0 for BIDIR) instead of zero
  float eps;
  void* gk;      // AGG_G / CAUSAL_G: [B*H][ceil(N/64)] key-responsibility tiles (64 x KP bf16 each)
};

// General kernel for bf16, d = dv = 128, KP = 256 (gma_wide.hip).
hipError_t wide_launch(const Args& a, int mode, int segments, unsigned BH, hipStream_t st);

// bf16 kernel for d = dv = 128 and KP = 256 (gma_long.hip): every mode.
bool long_supported(const GmaLaunch& L);
hipError_t long_launch(const Args& a, int mode, int segments, unsigned BH, hipStream_t st);

// bf16 kernel (gma_bf16.hip) for d = dv in {32, 64} and KP in {64, 128}.
bool fast_supported(const GmaLaunch& L);
hipError_t fast_launch(const GmaLaunch& L, const Args& a, int mode, int segments, hipStream_t st);

}  // namespace gma
}  // namespace lm
