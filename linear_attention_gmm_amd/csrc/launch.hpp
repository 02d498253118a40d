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
  void* gk = nullptr;  // workspace (bf16 causal kernel, P > 1): key responsibilities per chunk
  int64_t B, H, N, D, K, KP, P, seg_len;
  int causal;
  bool bf16;
  float eps;
  // causal only (optional): memory [Vtil (K x D) | Z (K)] per (b,h) before the
  // first token and after the last
  const float* state_in;
  float* state_out;
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
  // optional: state [S (D x D) | M (D x D) | m (D)] per (b,h) before the first
  // token (holding t_in tokens) and after the last
  const float* state_in;
  float* state_out;
  int64_t t_in;
  int64_t chunk = 64;  // tokens per chunk: 64 (matrix-core kernels) or 32 (linattn_c32.hip)
};
hipError_t linattn_launch(const LinLaunch& L, hipStream_t st);
// Chunks of 32 tokens (linattn_c32.hip): one workgroup per (b, h), no segments.
hipError_t linattn_c32_launch(const LinLaunch& L, hipStream_t st);

// Chunk pass of the CCQ read for bf16 inputs at dk = dv = 128 (ccq_pipe.hip):
// one workgroup per (b, h, segment), starting from the segment's state block
// (agg, R * segment, blocks per (b, h)) or from zero when agg is null.
struct CcqPipeLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* w_lambda;
  const float* b_lambda;
  void* out;
  const float* agg;
  int64_t B, H, N, P, seg_len, blocks, R, sfl, t_off;
  float* state_out;
};
hipError_t ccq_pipe_launch(const CcqPipeLaunch& L, hipStream_t st);

// Gated delta rule with the plain or the CCQ read (deltanet.hip): a prepass
// writes W and Ut of every chunk, then a sequential pass carries the state.
// For CCQ a clean-query pass (segment sums, then one chunk pass per segment)
// first writes q' to qc, and the sequential pass reads with it.
struct DeltaLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  const float* w_lambda;  // CCQ only
  const float* b_lambda;  // CCQ only
  void* out;
  void* wbuf;  // workspace [B,H,N,D] of the input dtype: W of every chunk
  void* ubuf;  // workspace [B,H,N,dv] of the input dtype: Ut of every chunk
  void* qc;    // CCQ: workspace [B,H,N,D] of the input dtype
  float* agg;  // CCQ: workspace [B*H][P][cq_state_floats(D)]
  int64_t B, H, N, D, dv;
  int64_t P, seg_len;  // CCQ: segments of the clean-query pass
  bool bf16;
  bool ccq;
  // optional: state [S (D x dv) | M (D x D) | m (D)] (CCQ) or [S] per (b,h),
  // sstride floats apart, before the first token (holding t_in tokens) and
  // after the last
  const float* state_in;
  float* state_out;
  int64_t sstride;
  int64_t t_in;
};
hipError_t deltanet_launch(const DeltaLaunch& L, hipStream_t st);

// Floats per block of the clean-query segment pass: sum k k^T (D x D), sum k
// (D); padded to 64 floats.
inline int64_t cq_state_floats(int64_t D) { return (D * D + D + 63) / 64 * 64; }

// Decayed linear attention with a decay per key feature (linattn_vec.hip).
struct VecLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;  // [B,H,N,D]
  void* out;
  float* agg;  // workspace: P state blocks per (b,h)
  int64_t B, H, N, D, P, seg_len;
  int64_t R;  // sub-segments per segment in the segment pass
  bool bf16;
  const float* state_in;  // optional: S [B*H][D][D] before the first token
  float* state_out;       // optional: S after the last token
};
hipError_t linattn_vec_launch(const VecLaunch& L, hipStream_t st);

// Floats per segment block of the per-feature form: S (D x D), then the
// segment's decay per feature (D); padded to 64 floats.
inline int64_t vec_state_floats(int64_t D) { return (D * D + D + 63) / 64 * 64; }

// One-token steps on a carried fp32 state (decode.hip). q, k [B,H,D]; v, out
// [B,H,D]; state in place.
struct DecodeLaunch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;         // linear attention: [B,H], or [B,H,D] with vector_gates
  bool vector_gates;
  const float* w_lambda;  // CCQ
  const float* b_lambda;  // CCQ
  const float* mu;        // GMA
  const float* log_var;   // GMA
  const float* logit_pi;  // GMA
  void* out;
  float* state;
  int64_t B, H, D, K;
  int64_t t_now;  // CCQ: tokens in the state after the step
  bool bf16;
  float eps;
};
hipError_t lin_decode_launch(const DecodeLaunch& L, bool ccq, hipStream_t st);
hipError_t gma_decode_launch(const DecodeLaunch& L, hipStream_t st);

// Backward pass of decayed linear attention (linattn_bwd.hip): three chunk-
// kernel passes on reordered inputs plus the gate gradient.
struct BwdLaunch {
  LinLaunch fwd;  // shapes, segment plan and workspace of the chunk passes
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  // workspace (float32): time-reversed q, k, v, do, one reversed output,
  // shifted gates; for bf16 inputs also float32 copies of q, k, v, do and the
  // float32 gradients dq, dk, dv before rounding
  float* rq;
  float* rk;
  float* rv;
  float* rdo;
  float* rout;
  float* rg;
  float* uq;
  float* uk;
  float* uv;
  float* udo;
  float* udq;
  float* udk;
  float* udv;
  int64_t B, H, N, D;
  bool bf16;
};
hipError_t linattn_backward_launch(const BwdLaunch& L, hipStream_t st);

// Backward of decayed linear attention for bf16 inputs with d_k = d_v = 128:
// one launch of forward-sweep (dq) and reverse-sweep (dk, dv) workgroups, then
// the suffix sums of the gate gradient.
// Tokens per slice of the gate-gradient suffix sums of the bf16 backward.
constexpr int kGateSlice = 1024;
inline int64_t gate_slices(int64_t N) { return (N + kGateSlice - 1) / kGateSlice; }
struct BwdBf16Launch {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  float* dg;
  float* xk;   // workspace: B * H * N floats (k . dk per token)
  float* tot;  // workspace: B * H * gate_slices(N) floats (sums over slices of tokens)
  // optional carried state, [B*H][128][128] float32 each
  const float* state_in = nullptr;
  const float* dstate_out = nullptr;
  float* dstate_in = nullptr;
  int64_t B, H, N;
};
hipError_t linattn_backward_bf16_launch(const BwdBf16Launch& L, hipStream_t st);
// The float32 passes of that backward on float32 tensors (gates: also dg).
hipError_t linattn_backward_f32(const BwdLaunch& L, const float* q, const float* k, const float* v,
                                const float* dout, float* dq, float* dk, float* dv, bool gates, hipStream_t st);

// Time reversal of float32 rows: out[bh][t] = in[bh][N - 1 - t] (D floats per row).
hipError_t reverse_rows_f32(const float* in, float* out, int64_t BH, int64_t N, int64_t D, hipStream_t st);

// Backward pass of the CCQ read (ccq_bwd.hip): the float32 backward of the
// decayed linear attention read with q_clean, no-decay passes for M q and M u,
// two passes on the reversed sequence for the covariance term of dk, scans of
// the key sum.
struct CcqBwdLaunch {
  BwdLaunch bwd;  // inner backward (float32, real gates, dg = the output dg); its
                  // plan, segment workspace and reversal buffers also serve the
                  // no-decay passes
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* w;  // [H][D]
  const float* b;  // [H]
  void* dq;
  void* dk;
  void* dv;
  float* dw;
  float* db;
  // workspace (float32 rows [B*H][N][D]): copies of k, v, dout (bf16 inputs;
  // fq unused there, q is read in bf16),
  // m, M q, Sigma q, q_clean, u = dq_clean, the direct dk, dv (bf16), M u, the
  // values of the reversed passes, dm, its suffix sums, the two reversed sums;
  // [B*H][N]: lambda, unit gates; scan range sums [B*H][nch][D]; dw/db partials
  // [H][B*nblk][D + 1]
  float *fq, *fk, *fv, *fdo, *m, *mq, *s, *qc, *u, *dkg, *dvg, *mu, *vr1, *vr2, *dm, *sdm, *r1, *r2;
  float *lam, *ones, *csum, *part;
  int64_t B, H, N, D, nch, clen, nblk, blen;
  bool bf16;
  // bf16 at D = 128: the decayed read's gradients on the fused bf16 backward
  // kernel (linattn_bwd_bf16.hip) instead of the float32 chunk passes
  bool fused = false;
};
hipError_t ccq_backward_launch(const CcqBwdLaunch& L, hipStream_t st);

// Backward pass of GMA (gma_bwd.hip): the float32 backward of the linear
// attention with responsibilities as features and [v | 1] as values (over 2N
// rows for the bidirectional form), then the chain rule through the softmax and
// the Gaussian log joint.
struct GmaBwdLaunch {
  BwdLaunch bwd;  // inner linear attention: D = DL, float32, its workspace
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  const float* mu;
  const float* log_var;
  const float* logit_pi;
  void* dq;
  void* dk;
  void* dv;
  float* dmu;
  float* dlog_var;
  float* dlogit_pi;
  // workspace (float32): per head 1/var [H][K][D] and the constant part of the
  // log joint [H][K]; [B*H][NN] rows of DL entries: responsibilities of q and
  // k, values [v | 1], inner output, its gradient, feature and value
  // gradients; unit gates [B*H][NN]; parameter partial sums
  // [H][2 B nseg][K][2 D + 1]
  float* iv;
  float* cst;
  float* gq;
  float* gk;
  float* vx;
  float* y;
  float* dy;
  float* dgq;
  float* dgk;
  float* dvx;
  float* ones;
  float* part;
  float* sums;  // the partials summed over the slots [H][K][2 D + 1]
  int64_t B, H, N, D, K, DL, nseg, seg_len;
  int64_t NN;  // inner rows per sequence: N (causal) or 2N (bidirectional)
  // wide shapes (d = 128 or K > 128): the inner tensors above in blocks of 128
  // columns, NF blocks of responsibilities, NVB of values, bstride floats apart;
  // tq, tk, tv: one block each for the sums over the blocks
  int64_t NF = 1, NVB = 1;
  size_t bstride = 0;
  float* tq = nullptr;
  float* tk = nullptr;
  float* tv = nullptr;
  int causal;
  float eps;
  bool bf16;
};
hipError_t gma_backward_launch(const GmaBwdLaunch& L, hipStream_t st);

// Feature-axis padding (pad.hip): rows of width sw to rows of width dw >= sw
// with the new columns set to `fill`, and back (the first dw of sw columns).
// esize is 2 (bf16) or 4 (float32).
hipError_t pad_cols(const void* src, void* dst, int64_t rows, int sw, int dw, float fill, int esize, hipStream_t st);
hipError_t crop_cols(const void* src, void* dst, int64_t rows, int sw, int dw, int esize, hipStream_t st);

// Fixed device scratch of the entry point that allocates nothing (noalloc.hip):
// its size, and its address on the current device (looked up once per device).
constexpr size_t kNoallocScratchBytes = size_t(64) << 20;
hipError_t noalloc_scratch(void** ptr);

// Floats per state block written by the segment-state pass.
inline int64_t lin_state_floats(int64_t D, bool ccq) {
  // S (D x D), decay product, and for CCQ: M (D x D), m (D); padded to 64 floats
  int64_t n = D * D + 1 + (ccq ? D * D + D : 0);
  return (n + 63) / 64 * 64;
}

}  // namespace lm
