/*
 * linmix.h -- C ABI of the MI355X (gfx950) sequence-mixer forward library.
 *
 * Three forward passes, each a drop-in replacement for an attention layer:
 *
 *  gma_forward            Gaussian Mixture Attention. Rows of Q and K are routed
 *                         to K diagonal-Gaussian components; keys write a K-slot
 *                         memory, queries read it back. Causal (prefix sums) or
 *                         bidirectional.
 *                         Source: "Gaussian Mixture Attention: Linear-Time
 *                         Sequence Mixing via Probabilistic Latent Routing",
 *                         Method -> core mechanism (posterior responsibilities;
 *                         write phase, read phase with eps in the denominator)
 *                         and variants (bidirectional; causal by prefix sums;
 *                         softmax priors).
 *  linattn_chunk_forward  Decayed (gated) linear attention, S_t = g_t S_{t-1} +
 *                         k_t v_t^T, o_t = S_t^T q_t, computed chunkwise.
 *                         Source: allinfo.ai.kr post on linear attention, "Key
 *                         messages" and "Easy explanation" (matrix state,
 *                         decay gates, chunkwise-parallel form).
 *  ccq_forward            The same state read with the curvature-conditioned
 *                         query q_clean = (I - lambda_t Sigma_t) q_t, with
 *                         Sigma_t the running key covariance (weights 1/t,
 *                         current token included) and lambda_t =
 *                         sigmoid(w . q_t + b).
 *                         Source: "Don't Read Everything: A Curvature-
 *                         Conditioned Query for Linear Attention", section 2
 *                         Method (derivation, mechanism, integration).
 *
 * Conventions common to every entry point
 *  - Pointers named q, k, v, g, mu, ..., out, workspace are DEVICE pointers on
 *    the current HIP device. Tensors are dense and row-major in the layouts given
 *    below, with 16-byte aligned base addresses. The caller owns every buffer.
 *  - dtype selects the element type of q, k, v and out: LM_F32 (float) or
 *    LM_BF16 (bfloat16). Parameters (mu, log_var, logit_pi, g, w_lambda,
 *    b_lambda) are always float32. Accumulation is float32.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). Inputs are read-only. On LM_OK, out is fully overwritten once
 *    the stream reaches the call. out must not overlap any input or the
 *    workspace.
 *  - The library allocates no device memory on these calls. Scratch space
 *    comes from the caller's `workspace` of at least the size returned by the
 *    matching *_workspace_bytes function for the same arguments. Its
 *    contents on entry do not matter.
 *  - segments: how many independent pieces each sequence is cut into for
 *    parallelism (0 = choose automatically). Results do not depend on it
 *    beyond float32 rounding order.
 *  - Every argument is checked on the host before any HIP call; on an error
 *    nothing is launched and nothing is written. lm_last_error() then holds a
 *    description (thread-local). No C++ exception crosses this boundary.
 *  - NaN / Inf inputs are not checked; they propagate to the outputs they
 *    influence.
 */
#ifndef LINMIX_H
#define LINMIX_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LM_ABI_VERSION 1

typedef enum {
  LM_OK = 0,
  LM_EINVAL = 1,       /* null / misaligned pointer, bad size, aliasing, eps < 0, ... */
  LM_EUNSUPPORTED = 2, /* valid arguments outside the implemented shapes */
  LM_EWORKSPACE = 3,   /* workspace smaller than *_workspace_bytes */
  LM_EHIP = 4          /* a HIP runtime / launch error; see lm_last_error() */
} lm_status;

typedef enum { LM_F32 = 0, LM_BF16 = 1 } lm_dtype;

/* Version of this ABI (LM_ABI_VERSION of the build). */
int lm_abi_version(void);

/* Static name of a status code. */
const char* lm_status_string(int status);

/* Detail of the last non-OK return on the calling thread ("" if none). */
const char* lm_last_error(void);

/*
 * Gaussian Mixture Attention forward.
 *   q, k     [B,H,N,d]   routing vectors (dtype)
 *   v        [B,H,N,dv]  values (dtype)
 *   mu       [H,K,d]     component means (float32), one mixture per head
 *   log_var  [H,K,d]     log of the diagonal variances (float32)
 *   logit_pi [H,K]       mixing logits; priors are softmax(logit_pi) (float32)
 *   out      [B,H,N,dv]  O = Gamma_Q Vtil / (Gamma_Q Z + eps) (dtype)
 *   causal   1: row i reads the memory of keys j <= i; 0: of all keys
 *   eps      >= 0, added to the read normaliser
 * Implemented shapes: d and dv in {32, 64, 128} with d == dv, 1 <= K <= 256,
 * any N >= 1.
 */
size_t gma_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv,
                           int causal, int dtype, int64_t segments);
int gma_forward(const void* q, const void* k, const void* v, const float* mu,
                const float* log_var, const float* logit_pi, void* out, int64_t B, int64_t H,
                int64_t N, int64_t d, int64_t K, int64_t dv, int causal, float eps, int dtype,
                int64_t segments, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Decayed linear attention forward (chunkwise).
 *   q, k  [B,H,N,dk] (dtype);  v [B,H,N,dv] (dtype)
 *   g     [B,H,N]    per-token, per-head decay (float32), expected in (0, 1]
 *   out   [B,H,N,dv] o_t = S_t^T q_t with S_t = g_t S_{t-1} + k_t v_t^T, S_0 = 0
 *   chunk tokens per chunk; 64 is implemented
 * Implemented shapes: dk == dv in {32, 64, 128}, any N >= 1.
 */
size_t linattn_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                               int64_t chunk, int dtype, int64_t segments);
int linattn_chunk_forward(const void* q, const void* k, const void* v, const float* g, void* out,
                          int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                          int dtype, int64_t segments, void* workspace, size_t workspace_bytes,
                          void* stream);

/*
 * Curvature-conditioned-query read over decayed linear attention.
 *   q, k, v, g, out, chunk as for linattn_chunk_forward
 *   w_lambda [H,dk], b_lambda [H]  gate parameters (float32):
 *            lambda_t = sigmoid(w_lambda[h] . q_t + b_lambda[h])
 *   out      o_t = S_t^T (q_t - lambda_t Sigma_t q_t), Sigma_t = (1/t) sum_{j<=t}
 *            k_j k_j^T - mu_t mu_t^T, mu_t = (1/t) sum_{j<=t} k_j (no decay)
 * Implemented shapes: dk == dv in {32, 64, 128}, any N >= 1.
 */
size_t ccq_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                           int64_t chunk, int dtype, int64_t segments);
int ccq_forward(const void* q, const void* k, const void* v, const float* g,
                const float* w_lambda, const float* b_lambda, void* out, int64_t B, int64_t H,
                int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LINMIX_H */
