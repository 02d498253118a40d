// launch.hpp -- internal interface between the C ABI layer and the kernels.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lm {

struct GmaLaunch {
  const void* q;
  const void* k;
  const void* v;
  void* out;
  const float* mu;
  const float* log_var;
  const float* logit_pi;
  void* W;      // workspace: [H][KP][2D] element type
  float* c;     // workspace: [H][KP]
  float* agg;   // workspace: [B*H][P][KP][DV]
  float* aggz;  // workspace: [B*H][P][KP]
  int64_t B, H, N, D, K, KP, P, seg_len;
  int causal;
  bool bf16;
  float eps;
};
hipError_t gma_launch(const GmaLaunch& L, hipStream_t st);

struct LinLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* w_lambda;  // CCQ only
  const float* b_lambda;  // CCQ only
  void* out;
  float* agg;  // workspace: R * P state blocks per (b,h) (see linattn.hip)
  int64_t B, H, N, D, P, seg_len;
  int64_t R;  // sub-segments per segment in the segment-state pass
  bool bf16;
  bool ccq;
};
hipError_t linattn_launch(const LinLaunch& L, hipStream_t st);

// Floats per state block written by the segment-state pass.
inline int64_t lin_state_floats(int64_t D, bool ccq) {
  // S (D x D), decay product, and for CCQ: M (D x D), m (D); padded to 64 floats
  int64_t n = D * D + 1 + (ccq ? D * D + D : 0);
  return (n + 63) / 64 * 64;
}

}  // namespace lm
