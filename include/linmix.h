/*
 * linmix.h -- C ABI of the MI355X (gfx950) sequence-mixer forward library.
 *
 * Four forward passes, each a drop-in replacement for an attention layer:
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
 *  linattn_vec_forward    The same with one decay per key feature,
 *                         S_t = diag(g_t) S_{t-1} + k_t v_t^T.
 *  deltanet_chunk_forward The gated delta write rule: S_t = g_t S_{t-1} -
 *                         beta_t k_t (g_t S_{t-1}^T k_t - v_t)^T, o_t = S_t^T q_t.
 *                         Source: allinfo.ai.kr linear attention post, "Key
 *                         messages" and "Easy explanation" (the update as one
 *                         gradient step on a squared key-to-value error; the
 *                         delta rule overwrites the value bound to a key; decay
 *                         gates forget).
 *  ccq_deltanet_forward   The CCQ read below over that write rule ("Don't Read
 *                         Everything", section 2 Method, integration: the read
 *                         does not depend on the write rule).
 *  ccq_forward            The same state read with the curvature-conditioned
 *                         query q_clean = (I - lambda_t Sigma_t) q_t, with
 *                         Sigma_t the running key covariance (weights 1/t,
 *                         current token included) and lambda_t =
 *                         sigmoid(w . q_t + b).
 *                         Source: "Don't Read Everything: A Curvature-
 *                         Conditioned Query for Linear Attention", section 2
 *                         Method (derivation, mechanism, integration).
 *
 * Carried state (prefill, then one token at a time). The causal forms need
 * nothing from the past but a fixed-size state per (b, h), so a sequence can
 * be continued in a later call:
 *  gma_forward_state, linattn_chunk_forward_state, ccq_forward_state,
 *  linattn_vec_forward_state, deltanet_forward_state,
 *  ccq_deltanet_forward_state
 *                         the forwards above, starting from a caller's state
 *                         (optional) and writing the state after the last
 *                         token (optional).
 *  gma_decode_step, linattn_decode_step, ccq_decode_step,
 *  linattn_vec_decode_step
 *                         one token per (b, h): advance the state in place and
 *                         read it.
 *                         Source: "Gaussian Mixture Attention", Method ->
 *                         variants (causal form as prefix sums of the memory);
 *                         allinfo.ai.kr linear attention post, "Key messages"
 *                         (a constant-size state replaces the growing cache);
 *                         "Don't Read Everything", section 2 Method ->
 *                         integration (the covariance statistics ride on the
 *                         same recurrence).
 * Backward passes (training): the gradients of sum(out * dout) for a given
 * output gradient dout, for the forwards without a carried state:
 *  linattn_chunk_backward dq, dk, dv, dg of decayed linear attention.
 *  gma_backward           dq, dk, dv, dmu, dlog_var, dlogit_pi of GMA (causal
 *                         and bidirectional).
 *  ccq_backward           dq, dk, dv, dg, dw_lambda, db_lambda of the CCQ read.
 *                         Each with a *_workspace_bytes function.
 * State layouts (float32, dense, one block per (b, h), blocks in b-major order):
 *    GMA   [Vtil (K x dv) | Z (K)]            K*dv + K floats:
 *          Vtil = sum_j gamma(k_j) v_j^T, Z = sum_j gamma(k_j)
 *    GLA   [S (dk x dv)]                      dk*dv floats:
 *          S = sum_j (prod_{s > j} g_s) k_j v_j^T (per-feature decay: the
 *          product scales row a of k_j v_j^T by prod_{s > j} g_s[a])
 *    CCQ   [S (dk x dv) | M (dk x dk) | m (dk)]  dk*dv + dk*dk + dk floats:
 *          M = sum_j k_j k_j^T, m = sum_j k_j (no decay)
 *    A zero-filled block is the state of an empty prefix. The CCQ state also
 *    needs the number of tokens it holds, which the caller passes (t_in,
 *    t_prev); all (b, h) of one call hold the same number.
 *
 * Feature widths. The forwards without a carried state (gma_forward,
 * linattn_chunk_forward, ccq_forward, linattn_vec_forward,
 * deltanet_chunk_forward, ccq_deltanet_forward) take feature widths d (dk)
 * and dv in {16, 32, 64, 128}, equal or not. d == dv in {32, 64, 128} runs
 * directly; any other pair runs on the kernels of width D, the smallest of
 * 32, 64, 128 that holds both, after zero padding of the feature axis, which
 * is exact (a routing feature with x = mu = 0 and log variance 0 adds the same
 * constant to every component's log joint; a zero key or query feature adds
 * nothing to any product, key covariance or norm; zero value columns give
 * output columns that are dropped). Such a call needs, in its workspace, the
 * padded Q, K, V and output (4 B*H*N*D elements of dtype), the padded
 * per-head parameters and the workspace of the width-D call. Carried states,
 * decode steps, backward passes and gma_forward_noalloc take d == dv in
 * {32, 64, 128} only.
 *
 * Conventions common to every entry point
 *  - Pointers named q, k, v, g, mu, ..., out, workspace are DEVICE pointers on
 *    the current HIP device. Tensors are dense and row-major in the layouts given
 *    below, with 16-byte aligned base addresses. The caller owns every buffer.
 *  - dtype selects the element type of q, k, v and out: LM_F32 (float) or
 *    LM_BF16 (bfloat16). Parameters (mu, log_var, logit_pi, g, w_lambda,
 *    b_lambda) are always float32. Accumulation is float32.
 *  - Calls are asynchronous on `stream` (a hipStream_t; NULL = the null
 *    stream). Inputs are read-only (the decode steps' state is the one
 *    argument that is both read and written). On LM_OK, out (and state_out)
 *    is fully overwritten once the stream reaches the call. out must not overlap any input or the
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

#define LM_ABI_VERSION 6

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
 * Implemented shapes: d, dv in {16, 32, 64, 128} (see "Feature widths"), 1 <= K <= 256,
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
 *   chunk tokens per chunk: 64 (the matrix-core kernels) or 32 (a float32
 *         kernel with one workgroup per (b, h), segments not used). The
 *         chunk length changes how the work is cut, not the result: the two
 *         agree to float32 rounding. The same holds for ccq_forward and the
 *         _state forms of both; the other chunked calls take 64.
 * Implemented shapes: dk, dv in {16, 32, 64, 128} (see "Feature widths"), any N >= 1.
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
 * Implemented shapes: dk, dv in {16, 32, 64, 128} (see "Feature widths"), any N >= 1.
 */
size_t ccq_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                           int64_t chunk, int dtype, int64_t segments);
int ccq_forward(const void* q, const void* k, const void* v, const float* g,
                const float* w_lambda, const float* b_lambda, void* out, int64_t B, int64_t H,
                int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                void* workspace, size_t workspace_bytes, void* stream);

/*
 * Gated delta rule (chunkwise), plain read.
 *   q, k  [B,H,N,dk] (dtype);  v [B,H,N,dv] (dtype)
 *   g     [B,H,N] per-token decay (float32), expected in (0, 1]; decays below
 *         2^-126 act as 2^-126
 *   beta  [B,H,N] per-token step size (float32), expected in [0, 1]; with keys
 *         of unit norm the step never amplifies the state
 *   out   [B,H,N,dv] o_t = S_t^T q_t, S_t = g_t S_{t-1} - beta_t k_t (g_t
 *         S_{t-1}^T k_t - v_t)^T, S_0 = 0 (one gradient step of size beta_t on
 *         1/2 ||S^T k_t - v_t||^2 after the decay)
 *   chunk 64 is implemented
 *   segments is accepted and has no effect: the state passes through every
 *         chunk of a sequence in order (the columns of S are what is split
 *         across workgroups: B*H*dv/32 of them).
 * Workspace (deltanet_workspace_bytes): W = T diag(beta gamma) K and
 * T diag(beta) V of every chunk, B*H*N*(dk + dv) elements of dtype.
 * Implemented shapes: dk, dv in {16, 32, 64, 128} (see "Feature widths")
 * whose padded width is at most 128 for bf16 and at most 64 for float32; any
 * N >= 1.
 */
size_t deltanet_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                                int64_t chunk, int dtype, int64_t segments);
int deltanet_chunk_forward(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, void* out, int64_t B, int64_t H, int64_t N,
                           int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                           void* workspace, size_t workspace_bytes, void* stream);

/*
 * The CCQ read over the gated delta rule: o_t = S_t^T (q_t - lambda_t Sigma_t
 * q_t), with S_t as for deltanet_chunk_forward and lambda_t, Sigma_t as for
 * ccq_forward (w_lambda [H,dk], b_lambda [H], float32).
 * Workspace (ccq_deltanet_workspace_bytes): that of deltanet_chunk_forward,
 * the clean queries (B*H*N*dk elements of dtype) and the running key sums of
 * each segment of the clean-query pass; segments (0 = automatic) splits that
 * pass only.
 * Implemented shapes: as for deltanet_chunk_forward.
 */
size_t ccq_deltanet_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                                    int64_t chunk, int dtype, int64_t segments);
int ccq_deltanet_forward(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, const float* w_lambda, const float* b_lambda,
                         void* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                         int64_t chunk, int dtype, int64_t segments, void* workspace,
                         size_t workspace_bytes, void* stream);

/*
 * Decayed linear attention with one decay per key feature (chunkwise).
 *   q, k, v, out, chunk as for linattn_chunk_forward
 *   g     [B,H,N,dk] float32, expected in [0, 1]: S_t = diag(g_t) S_{t-1} + k_t v_t^T,
 *         o_t = S_t^T q_t, S_0 = 0, for every such g (chunks that hold a decay
 *         below 2^-15 run the recurrence token by token, which is slower).
 *   g must be 16-byte aligned (it is read in 16-byte transfers).
 * Source: allinfo.ai.kr post on linear attention, "Key messages" (decay gates,
 * forgetting rates that can differ per channel).
 * Implemented shapes: dk, dv in {16, 32, 64, 128} (see "Feature widths"), chunk 64,
 * any N >= 1.
 */
size_t linattn_vec_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                                   int64_t chunk, int dtype, int64_t segments);
int linattn_vec_forward(const void* q, const void* k, const void* v, const float* g, void* out,
                        int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk,
                        int dtype, int64_t segments, void* workspace, size_t workspace_bytes,
                        void* stream);
/*
 * The same on a carried state S [B,H,dk*dv] (float32, the GLA layout below):
 * state_in / state_out as for linattn_chunk_forward_state (workspace from
 * linattn_vec_workspace_bytes), and the one-token step: q, k [B,H,dk], v, out
 * [B,H,dv], g [B,H,dk] float32; S = diag(g) S + k v^T in place, out = S^T q.
 * The step takes g as given (no clamp).
 */
int linattn_vec_forward_state(const void* q, const void* k, const void* v, const float* g,
                              void* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                              int64_t chunk, int dtype, int64_t segments, const float* state_in,
                              float* state_out, void* workspace, size_t workspace_bytes,
                              void* stream);
int linattn_vec_decode_step(const void* q, const void* k, const void* v, const float* g,
                            void* out, float* state, int64_t B, int64_t H, int64_t dk, int64_t dv,
                            int dtype, void* stream);

/*
 * Backward pass of decayed linear attention (scalar gate): given the output
 * gradient dout [B,H,N,dv] of linattn_chunk_forward(q, k, v, g), writes
 *   dq, dk [B,H,N,dk], dv [B,H,N,dv] (dtype) and dg [B,H,N] (float32),
 * the gradients of sum(out * dout): dq_t = S_t dout_t; dk, dv from the state
 * gradient U_t = q_t dout_t^T + g_{t+1} U_{t+1}; and
 * dg_t = (1/g_t) sum_{m >= t} (q_m . dq_m - k_m . dk_m).
 * bf16 with dk = dv = 128 and B*H >= 32: one launch of a forward sweep (dq)
 * and a reverse sweep (dk, dv) per (b, h), with dq and dk accurate to about 16
 * bits (split bf16 operands), then the suffix sums; segments is not used.
 * Other shapes: three chunkwise passes of the forward kernel in float32 (dk,
 * dv on the time-reversed sequence), over segments of each sequence.
 * Source: allinfo.ai.kr post on linear attention, "Key messages" (matrix state
 * with decay gates; the chunkwise form is what makes training parallel).
 * Outputs must not overlap each other, the inputs or the workspace (of at least
 * linattn_backward_workspace_bytes). Shapes as for linattn_chunk_forward.
 */
size_t linattn_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                                        int64_t chunk, int dtype, int64_t segments);
int linattn_chunk_backward(const void* q, const void* k, const void* v, const float* g,
                           const void* dout, void* dq, void* dk, void* dv, float* dg, int64_t B,
                           int64_t H, int64_t N, int64_t dkk, int64_t dvv, int64_t chunk, int dtype,
                           int64_t segments, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The same with a carried state (truncated backpropagation across calls): the
 * forward ran from state_in [B,H,dk*dv] (float32, S[a][b] at a*dv + b; NULL =
 * zero) and the loss also depends on the state after the last token through
 * dstate_out [B,H,dk*dv] (its gradient; NULL = none). Writes dq, dk, dv, dg as
 * above (dg then also holds the gates' effect on the carried states) and, when
 * dstate_in is not NULL, the gradient of state_in [B,H,dk*dv] (float32).
 * Chaining calls backwards (dstate_out of a call = dstate_in of the next)
 * gives the gradients of the whole sequence.
 * Source: allinfo.ai.kr post on linear attention, "Key messages" (the state is
 * all that crosses from one part of the sequence to the next).
 * Implemented: as linattn_chunk_backward; with a state pointer given, bf16 with
 * dk = dv = 128 (LM_EUNSUPPORTED otherwise). State buffers 16-byte aligned;
 * dstate_in must not overlap any other buffer. Same workspace.
 */
int linattn_chunk_backward_state(const void* q, const void* k, const void* v, const float* g,
                                 const void* dout, const float* state_in, const float* dstate_out,
                                 void* dq, void* dk, void* dv, float* dg, float* dstate_in,
                                 int64_t B, int64_t H, int64_t N, int64_t dkk, int64_t dvv,
                                 int64_t chunk, int dtype, int64_t segments, void* workspace,
                                 size_t workspace_bytes, void* stream);

/*
 * Backward pass of the CCQ read: given the output gradient dout [B,H,N,dv] of
 * ccq_forward(q, k, v, g, w_lambda, b_lambda), writes the gradients of
 * sum(out * dout):
 *   dq, dk [B,H,N,dk], dv [B,H,N,dv]                 (dtype, 16-byte aligned)
 *   dg [B,H,N], dw_lambda [H,dk], db_lambda [H]       (float32, 4-byte aligned)
 * With u the gradient of q_clean (from the backward of the decayed linear
 * attention read with q_clean, which also gives dv, dg and the direct part of
 * dk): dq = u - lambda Sigma u - (u . Sigma q) lambda (1 - lambda) w; the
 * covariance adds -sum_{t>=j} (lambda_t/t) [u_t (q_t . k_j) + q_t (u_t . k_j)]
 * plus the suffix sum of (lambda_t/t^2) [u_t (q_t . m_t) + q_t (u_t . m_t)]
 * to dk_j (m_t the running key sum); dw, db sum -(u . Sigma q) lambda
 * (1 - lambda) q and its scalar over the batch and the tokens. Computed in
 * float32 with the chunk kernel (decayed and undecayed passes, some on the
 * time-reversed sequence); bf16 gradients are rounded once. For bf16 at
 * dk = dv = 128 with B*H >= 32 the decayed read's gradients (u, dv, dg, the
 * direct part of dk) come from the kernel of linattn_chunk_backward instead,
 * with q_clean rounded once to bf16 as the forward's read takes it.
 * Source: "Don't Read Everything: A Curvature-Conditioned Query for Linear
 * Attention", section 2 Method (derivation, mechanism, integration).
 * Shapes as for ccq_forward (chunk 64, dk == dv in {32, 64, 128}); no carried
 * state. Outputs must not overlap each other, the inputs or the workspace (of
 * at least ccq_backward_workspace_bytes: about 18 float32 tensors of the
 * size of q, 22 for bf16 inputs).
 */
size_t ccq_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                                    int64_t chunk, int dtype);
int ccq_backward(const void* q, const void* k, const void* v, const float* g,
                 const float* w_lambda, const float* b_lambda, const void* dout, void* dq,
                 void* dk, void* dv, float* dg, float* dw_lambda, float* db_lambda, int64_t B,
                 int64_t H, int64_t N, int64_t dkk, int64_t dvv, int64_t chunk, int dtype,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * Backward pass of GMA: given the output gradient dout [B,H,N,dv] of
 * gma_forward(q, k, v, mu, log_var, logit_pi, causal, eps), writes the
 * gradients of sum(out * dout):
 *   dq, dk [B,H,N,d], dv [B,H,N,dv]                 (dtype, 16-byte aligned)
 *   dmu, dlog_var [H,K,d], dlogit_pi [H,K]          (float32, 4-byte aligned)
 * The causal output is a linear attention with the responsibilities as
 * features and [v | 1] as values (numerator and normaliser), so the float32
 * backward of that linear attention gives the gradients of the features and of
 * v; the chain rule through the softmax over components and the Gaussian log
 * joint gives dq, dk and the parameter gradients (summed over the batch and
 * over both the query and the key tokens, in a fixed order). The
 * bidirectional form is the same inner linear attention over 2N rows, keys and
 * values first, then the queries. Everything is computed in float32; bf16
 * gradients are rounded once.
 * Source: "Gaussian Mixture Attention", Method -> core mechanism (posterior
 * responsibilities), latent memory routing (write and read phases), variants
 * and training (trained end to end; softplus variances, softmax priors).
 * Implemented: causal 0 or 1, d == dv in {32, 64, 128}, 1 <= K <= 256,
 * N <= 2^29. With d = 128 or K > 128 the inner linear attention runs on
 * blocks of 128 feature and value columns (once per pair of blocks, summed).
 * Outputs must not overlap each other, the inputs or the workspace (of at
 * least gma_backward_workspace_bytes; float32 rows of 64 to 256 entries per
 * token, about 14 such tensors, twice as many rows when bidirectional).
 */
size_t gma_backward_workspace_bytes(int64_t B, int64_t H, int64_t N, int64_t d, int64_t K,
                                    int64_t dv, int causal, int dtype);
int gma_backward(const void* q, const void* k, const void* v, const float* mu,
                 const float* log_var, const float* logit_pi, const void* dout, void* dq,
                 void* dk, void* dv, float* dmu, float* dlog_var, float* dlogit_pi, int64_t B,
                 int64_t H, int64_t N, int64_t d, int64_t K, int64_t dvv, int causal, float eps,
                 int dtype, void* workspace, size_t workspace_bytes, void* stream);

/*
 * Forwards on a carried state. Arguments as for the forward of the same name
 * (gma_forward_state is the causal GMA forward; the workspace is the one
 * gma_workspace_bytes gives for causal = 1), plus:
 *   state_in   [B,H,state] device, float32 (layouts above): the state before
 *              the first token; NULL = empty prefix (zero state).
 *   state_out  [B,H,state] device, float32: receives the state after the last
 *              token; NULL = not written. May be the same buffer as state_in
 *              (updated in place); otherwise the two must not overlap. Neither
 *              may overlap out or the workspace. 16-byte aligned.
 *   t_in       (CCQ) tokens already held by state_in: the running statistics
 *              of token i of this call divide by t_in + i + 1. Must be 0 when
 *              state_in is NULL.
 * Cost: state_out of GMA adds the segment pass over the last segment; the
 * linear-attention forms write it from the registers of the last segment.
 */
int gma_forward_state(const void* q, const void* k, const void* v, const float* mu,
                      const float* log_var, const float* logit_pi, void* out, int64_t B,
                      int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, float eps,
                      int dtype, int64_t segments, const float* state_in, float* state_out,
                      void* workspace, size_t workspace_bytes, void* stream);
int linattn_chunk_forward_state(const void* q, const void* k, const void* v, const float* g,
                                void* out, int64_t B, int64_t H, int64_t N, int64_t dk,
                                int64_t dv, int64_t chunk, int dtype, int64_t segments,
                                const float* state_in, float* state_out, void* workspace,
                                size_t workspace_bytes, void* stream);
int ccq_forward_state(const void* q, const void* k, const void* v, const float* g,
                      const float* w_lambda, const float* b_lambda, void* out, int64_t B,
                      int64_t H, int64_t N, int64_t dk, int64_t dv, int64_t chunk, int dtype,
                      int64_t segments, int64_t t_in, const float* state_in, float* state_out,
                      void* workspace, size_t workspace_bytes, void* stream);
/* Gated delta rule on a carried state: S [B,H,dk*dv] (the GLA layout), plain
 * read; and the CCQ read on it with the CCQ layout [S | M | m] and t_in.
 * Workspaces from deltanet_workspace_bytes / ccq_deltanet_workspace_bytes. */
int deltanet_forward_state(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, void* out, int64_t B, int64_t H, int64_t N,
                           int64_t dk, int64_t dv, int64_t chunk, int dtype, int64_t segments,
                           const float* state_in, float* state_out, void* workspace,
                           size_t workspace_bytes, void* stream);
int ccq_deltanet_forward_state(const void* q, const void* k, const void* v, const float* g,
                               const float* beta, const float* w_lambda, const float* b_lambda,
                               void* out, int64_t B, int64_t H, int64_t N, int64_t dk, int64_t dv,
                               int64_t chunk, int dtype, int64_t segments, int64_t t_in,
                               const float* state_in, float* state_out, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * gma_forward without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Arguments, shapes and results as for gma_forward.
 * Scratch comes from a fixed device array of LM_NOALLOC_SCRATCH_BYTES inside
 * the library, one per GPU, held from the library's load until the process
 * ends; its address is looked up on the first call on each device. The call
 * allocates nothing and calls no allocating routine. The causal form does not
 * store the key responsibilities in this scratch (it routes the keys in both
 * of its passes), so it needs about 4 (K dv + K) bytes per (b, h) and segment
 * plus the prepared parameters (8 d K + 4 K bytes per head for bf16).
 * Errors: LM_EWORKSPACE when the shape needs more scratch than the array
 * holds (fewer segments need less); otherwise as for gma_forward.
 * Every call on one GPU uses the same scratch: calls that overlap in time on
 * one GPU (two streams, two threads) race and must not be issued.
 */
#define LM_NOALLOC_SCRATCH_BYTES ((size_t)64 << 20)
int gma_forward_noalloc(const void* q, const void* k, const void* v, const float* mu,
                        const float* log_var, const float* logit_pi, void* out, int64_t B,
                        int64_t H, int64_t N, int64_t d, int64_t K, int64_t dv, int causal,
                        float eps, int dtype, int64_t segments, void* stream);

/*
 * One-token steps. Per (b, h) one new token: q, k [B,H,d] and v, out [B,H,dv]
 * (dtype, 16-byte aligned); g [B,H] float32 (linear attention); parameters as
 * for the forwards. state [B,H,state] (device float32, layouts above, 16-byte
 * aligned) is read, advanced by the token and written back in place; out is
 * the read of the advanced state (the token sees itself, as in the causal
 * forwards). Equal to the matching forward over the prefix plus this token.
 *   gma_decode_step      Vtil += gamma(k) v^T, Z += gamma(k);
 *                        out = gamma(q) Vtil / (gamma(q) Z + eps).
 *   linattn_decode_step  S = g S + k v^T; out = S^T q.
 *   ccq_decode_step      also M += k k^T, m += k; with t = t_prev + 1 tokens,
 *                        out = S^T (q - lambda Sigma q), Sigma = M / t - m m^T / t^2.
 *                        t_prev: tokens held by the state before the step (>= 0).
 * Implemented: d == dv in {32, 64, 128}, 1 <= K <= 256, B*H <= 2^24. No
 * workspace. state must not overlap q, k, v or out. Calls that share a state
 * buffer must be ordered on one stream.
 */
int gma_decode_step(const void* q, const void* k, const void* v, const float* mu,
                    const float* log_var, const float* logit_pi, void* out, float* state,
                    int64_t B, int64_t H, int64_t d, int64_t K, int64_t dv, float eps, int dtype,
                    void* stream);
int linattn_decode_step(const void* q, const void* k, const void* v, const float* g, void* out,
                        float* state, int64_t B, int64_t H, int64_t dk, int64_t dv, int dtype,
                        void* stream);
int ccq_decode_step(const void* q, const void* k, const void* v, const float* g,
                    const float* w_lambda, const float* b_lambda, void* out, float* state,
                    int64_t B, int64_t H, int64_t dk, int64_t dv, int64_t t_prev, int dtype,
                    void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LINMIX_H */
