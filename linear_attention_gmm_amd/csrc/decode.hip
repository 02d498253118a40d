// decode.hip -- one-token steps of the three mixers on a carried fp32 state.
//
// A causal mixer needs nothing from the past but its state, so generation
// after a prefill advances the state one token at a time:
//  * GMA ("Gaussian Mixture Attention", Method -> core mechanism, causal
//    variant): route q and k to the K components, add gamma(k) v^T and
//    gamma(k) to the memory [Vtil | Z], read gamma(q) Vtil / (gamma(q) Z + eps).
//  * Decayed linear attention (allinfo.ai.kr linear attention post, "Key
//    messages": decay gates on the matrix state): S <- g S + k v^T, o = S^T q,
//    with one g per (b, h) or one per key feature (row of S).
//  * CCQ ("Don't Read Everything", section 2 Method): the key sums M += k k^T,
//    m += k and the count t advance with every token; the read uses
//    q_clean = q - lambda (M q / t - m (m . q) / t^2), lambda = sigmoid(w . q + b).
//
// Each step reads and rewrites the whole state once, so it is bound by HBM
// traffic on the state. One workgroup of 256 threads per (b, h): every state
// row is read as float4 by D/4 consecutive threads (coalesced), all loads of a
// pass are issued before their use so that each CU keeps many requests in
// flight, and the updated rows are written back in place.
#include "mfma.hpp"
#include "launch.hpp"

namespace lm {
namespace dec {

constexpr int NT = 256;

__device__ __forceinline__ float wave_sum(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x += __shfl_xor(x, o);
  return x;
}
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) x = fmaxf(x, __shfl_xor(x, o));
  return x;
}

__device__ __forceinline__ float4 ld4(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ void st4(float* p, float4 x) { *reinterpret_cast<float4*>(p) = x; }
__device__ __forceinline__ float dot4(float4 a, float4 b) { return a.x * b.x + a.y * b.y + a.z * b.z + a.w * b.w; }
__device__ __forceinline__ float4 fma4(float s, float4 a, float4 b) {  // s a + b
  return make_float4(fmaf(s, a.x, b.x), fmaf(s, a.y, b.y), fmaf(s, a.z, b.z), fmaf(s, a.w, b.w));
}

// Row-pass geometry over a matrix with D floats per row: D/4 threads per row,
// RPP rows per pass of the workgroup.
template <int D>
struct Rows {
  static constexpr int C4 = D / 4;
  static constexpr int RPP = NT / C4;
};

// Reduces a float4 per thread over the RPP row groups into one value per column
// (thread e < D receives column e).
template <int D>
__device__ __forceinline__ float column_sum(float4 acc, float (*sred)[D]) {
  typedef Rows<D> R;
  const int j = threadIdx.x % R::C4, r0 = threadIdx.x / R::C4;
  st4(&sred[r0][4 * j], acc);
  __syncthreads();
  float s = 0.f;
  if (threadIdx.x < D) {
#pragma unroll
    for (int r = 0; r < R::RPP; ++r) s += sred[r][threadIdx.x];
  }
  return s;
}

// ---------------------------------------------------------------------------
// Decayed linear attention and CCQ. State per (b,h): [S (D x D) | M (D x D) |
// m (D)] (M, m for CCQ only). t_now: tokens in the state after this step. VG:
// one decay per key feature (row of S), g [B,H,D].
template <typename T, int D, bool CCQ, bool VG>
__global__ __launch_bounds__(NT) void lin_step(const T* __restrict__ q, const T* __restrict__ k,
                                               const T* __restrict__ v, const float* __restrict__ g,
                                               const float* __restrict__ wl, const float* __restrict__ bl,
                                               T* __restrict__ out, float* __restrict__ state, int H,
                                               float t_now) {
  typedef Rows<D> R;
  constexpr int NP = D / R::RPP;  // passes over D rows
  constexpr size_t SF = (size_t)D * D + (CCQ ? (size_t)D * D + D : 0);
  __shared__ float sq[D], sk[D], sv[D], sqc[D], sm[D], sMq[D], sg[VG ? D : 1];
  __shared__ float sred[R::RPP][D];
  __shared__ float sdot[2];
  const int bh = blockIdx.x, h = bh % H, tid = threadIdx.x;
  const int j = tid % R::C4, r0 = tid / R::C4;
  float* S = state + (size_t)bh * SF;
  if (tid < D) {
    sq[tid] = to_f32(q[(size_t)bh * D + tid]);
    sk[tid] = to_f32(k[(size_t)bh * D + tid]);
    sv[tid] = to_f32(v[(size_t)bh * D + tid]);
    if constexpr (VG) sg[tid] = g[(size_t)bh * D + tid];
  }
  const float gt = VG ? 0.f : g[bh];
  __syncthreads();

  if constexpr (CCQ) {
    float* M = S + (size_t)D * D;
    float* m = M + (size_t)D * D;
    float4 mv[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p) mv[p] = ld4(M + (size_t)(r0 + p * R::RPP) * D + 4 * j);
    const float4 kc = ld4(&sk[4 * j]), qc4 = ld4(&sq[4 * j]);
#pragma unroll
    for (int p = 0; p < NP; ++p) {
      const int a = r0 + p * R::RPP;
      mv[p] = fma4(sk[a], kc, mv[p]);  // M <- M + k k^T
      st4(M + (size_t)a * D + 4 * j, mv[p]);
      float part = dot4(mv[p], qc4);  // (M q)_a over this thread's four columns
#pragma unroll
      for (int o = R::C4 / 2; o > 0; o >>= 1) part += __shfl_xor(part, o);
      if (j == 0) sMq[a] = part;
    }
    if (tid < D) {
      const float mn = m[tid] + sk[tid];  // m <- m + k
      m[tid] = mn;
      sm[tid] = mn;
    }
    __syncthreads();
    if (tid < 64) {
      float mq = 0.f, wq = 0.f;
      for (int i = tid; i < D; i += 64) {
        mq += sm[i] * sq[i];
        wq += wl[(size_t)h * D + i] * sq[i];
      }
      mq = wave_sum(mq);
      wq = wave_sum(wq);
      if (tid == 0) {
        sdot[0] = mq;
        sdot[1] = wq;
      }
    }
    __syncthreads();
    const float inv_t = 1.f / t_now;
    const float lam = 1.f / (1.f + expf(-(sdot[1] + bl[h])));
    if (tid < D) sqc[tid] = sq[tid] - lam * (sMq[tid] * inv_t - sm[tid] * (sdot[0] * inv_t * inv_t));
    __syncthreads();
  }
  const float* qr = CCQ ? sqc : sq;

  // S <- g S + k v^T, o = S^T q_read
  float4 sv4[NP];
#pragma unroll
  for (int p = 0; p < NP; ++p) sv4[p] = ld4(S + (size_t)(r0 + p * R::RPP) * D + 4 * j);
  const float4 vc = ld4(&sv[4 * j]);
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int p = 0; p < NP; ++p) {
    const int a = r0 + p * R::RPP;
    float4 s = sv4[p];
    const float ga = VG ? sg[a] : gt;
    s = make_float4(ga * s.x, ga * s.y, ga * s.z, ga * s.w);
    s = fma4(sk[a], vc, s);
    st4(S + (size_t)a * D + 4 * j, s);
    acc = fma4(qr[a], s, acc);
  }
  const float o = column_sum<D>(acc, sred);
  if (tid < D) out[(size_t)bh * D + tid] = from_f32<T>(o);
}

// ---------------------------------------------------------------------------
// GMA. State per (b,h): [Vtil (K x D) | Z (K)]. The responsibilities come
// straight from the Gaussian log-densities, log pi_c - (1/2) sum_i (log var_ci +
// (x_i - mu_ci)^2 / var_ci); the terms common to all components (the
// normaliser of the priors, (D/2) log 2 pi) cancel in the posterior.
// One workgroup serves NB batch entries of one head, so the parameters are
// read and the precisions exp(-log var) formed once for NB tokens.
template <typename T, int D, int NB>
__global__ __launch_bounds__(NT) void gma_step(const T* __restrict__ q, const T* __restrict__ k,
                                               const T* __restrict__ v, const float* __restrict__ mu,
                                               const float* __restrict__ lv, const float* __restrict__ lp,
                                               T* __restrict__ out, float* __restrict__ state, int B, int H,
                                               int K, float eps) {
  typedef Rows<D> R;
  constexpr int BATCH = 8;  // passes whose loads are in flight together
  __shared__ float sq[NB][D], sk[NB][D], sv[NB][D];
  __shared__ float sgq[NB][256], sgk[NB][256];
  __shared__ float sred[R::RPP][D];
  __shared__ float sden[NT / 64];
  const int h = blockIdx.x % H, b0 = (blockIdx.x / H) * NB;
  const int nb = B - b0 < NB ? B - b0 : NB;
  const int tid = threadIdx.x, l = lane_id(), w = wave_id();
  const int j = tid % R::C4, r0 = tid / R::C4;
  for (int i = tid; i < NB * D; i += NT) {
    const int n = i / D, e = i - n * D;
    const size_t x = ((size_t)(b0 + n) * H + h) * D + e;
    sq[n][e] = n < nb ? to_f32(q[x]) : 0.f;
    sk[n][e] = n < nb ? to_f32(k[x]) : 0.f;
    sv[n][e] = n < nb ? to_f32(v[x]) : 0.f;
  }
  __syncthreads();

  // log joint of the queries and keys under every component: one thread per
  // component, over the features (q and k are LDS broadcasts)
  if (tid < K) {
    const float* mc = mu + ((size_t)h * K + tid) * D;
    const float* lc = lv + ((size_t)h * K + tid) * D;
    float aq[NB], ak[NB];
#pragma unroll
    for (int n = 0; n < NB; ++n) aq[n] = ak[n] = 0.f;
    float lsum = 0.f;
#pragma unroll 4
    for (int i = 0; i < D; ++i) {
      const float m = mc[i], lvar = lc[i];
      const float prec = expf(-lvar);
      lsum += lvar;
#pragma unroll
      for (int n = 0; n < NB; ++n) {
        const float dq = sq[n][i] - m, dk = sk[n][i] - m;
        aq[n] += dq * dq * prec;
        ak[n] += dk * dk * prec;
      }
    }
    const float pc = lp[(size_t)h * K + tid];
#pragma unroll
    for (int n = 0; n < NB; ++n) {
      sgq[n][tid] = pc - 0.5f * (lsum + aq[n]);
      sgk[n][tid] = pc - 0.5f * (lsum + ak[n]);
    }
  }
  __syncthreads();
  // posteriors: softmax over components, one wave per (entry, q or k)
  for (int sidx = w; sidx < 2 * nb; sidx += NT / 64) {
    float* s = (sidx & 1) ? sgk[sidx >> 1] : sgq[sidx >> 1];
    float mx = -INFINITY;
    for (int c = l; c < K; c += 64) mx = fmaxf(mx, s[c]);
    mx = wave_max(mx);
    float sum = 0.f;
    for (int c = l; c < K; c += 64) {
      const float e = expf(s[c] - mx);
      s[c] = e;
      sum += e;
    }
    sum = wave_sum(sum);
    const float inv = 1.f / sum;
    for (int c = l; c < K; c += 64) s[c] *= inv;
  }
  __syncthreads();

  const int npass = (K + R::RPP - 1) / R::RPP;
  for (int n = 0; n < nb; ++n) {
    const size_t bh = (size_t)(b0 + n) * H + h;
    float* Vt = state + bh * ((size_t)K * D + K);
    float* Z = Vt + (size_t)K * D;
    // memory rows: Vtil <- Vtil + gamma_k v^T, numerator gamma_q^T Vtil
    const float4 vc = ld4(&sv[n][4 * j]);
    float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int p0 = 0; p0 < npass; p0 += BATCH) {
      float4 x[BATCH];
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) {
        const int c = r0 + (p0 + bb) * R::RPP;
        if (c < K) x[bb] = ld4(Vt + (size_t)c * D + 4 * j);
      }
#pragma unroll
      for (int bb = 0; bb < BATCH; ++bb) {
        const int c = r0 + (p0 + bb) * R::RPP;
        if (c < K) {
          const float4 s = fma4(sgk[n][c], vc, x[bb]);
          st4(Vt + (size_t)c * D + 4 * j, s);
          acc = fma4(sgq[n][c], s, acc);
        }
      }
    }
    // normaliser: Z <- Z + gamma_k, denominator gamma_q . Z
    float den = 0.f;
    for (int c = tid; c < K; c += NT) {
      const float z = Z[c] + sgk[n][c];
      Z[c] = z;
      den += sgq[n][c] * z;
    }
    den = wave_sum(den);
    if (l == 0) sden[w] = den;
    const float num = column_sum<D>(acc, sred);  // (its barrier publishes sden)
    if (tid < D) {
      float dsum = 0.f;
#pragma unroll
      for (int i = 0; i < NT / 64; ++i) dsum += sden[i];
      out[bh * D + tid] = from_f32<T>(num / (dsum + eps));
    }
    __syncthreads();  // sred and sden are reused by the next entry
  }
}

template <typename T, bool CCQ, bool VG>
static hipError_t lin_t(const DecodeLaunch& L, hipStream_t st) {
  const unsigned BH = (unsigned)(L.B * L.H);
  const float t_now = (float)L.t_now;
#define LM_LIN_STEP(DD)                                                                                        \
  hipLaunchKernelGGL((lin_step<T, DD, CCQ, VG>), dim3(BH), dim3(NT), 0, st, (const T*)L.q, (const T*)L.k,    \
                     (const T*)L.v, L.g, L.w_lambda, L.b_lambda, (T*)L.out, L.state, (int)L.H, t_now)
  switch (L.D) {
    case 32: LM_LIN_STEP(32); break;
    case 64: LM_LIN_STEP(64); break;
    case 128: LM_LIN_STEP(128); break;
    default: return hipErrorInvalidValue;
  }
#undef LM_LIN_STEP
  return hipGetLastError();
}

template <typename T, int NB>
static hipError_t gma_nb(const DecodeLaunch& L, hipStream_t st) {
  const unsigned grid = (unsigned)(((L.B + NB - 1) / NB) * L.H);
#define LM_GMA_STEP(DD)                                                                                        \
  hipLaunchKernelGGL((gma_step<T, DD, NB>), dim3(grid), dim3(NT), 0, st, (const T*)L.q, (const T*)L.k,       \
                     (const T*)L.v, L.mu, L.log_var, L.logit_pi, (T*)L.out, L.state, (int)L.B, (int)L.H,      \
                     (int)L.K, L.eps)
  switch (L.D) {
    case 32: LM_GMA_STEP(32); break;
    case 64: LM_GMA_STEP(64); break;
    case 128: LM_GMA_STEP(128); break;
    default: return hipErrorInvalidValue;
  }
#undef LM_GMA_STEP
  return hipGetLastError();
}

// Batch entries per workgroup: as many as fill a group without idle entries
// for small batches.
template <typename T>
static hipError_t gma_t(const DecodeLaunch& L, hipStream_t st) {
  if (L.B >= 8) return gma_nb<T, 8>(L, st);
  if (L.B >= 4) return gma_nb<T, 4>(L, st);
  return gma_nb<T, 1>(L, st);
}

}  // namespace dec

hipError_t lin_decode_launch(const DecodeLaunch& L, bool ccq, hipStream_t st) {
  if (L.vector_gates) return L.bf16 ? dec::lin_t<bf16, false, true>(L, st) : dec::lin_t<float, false, true>(L, st);
  if (L.bf16) return ccq ? dec::lin_t<bf16, true, false>(L, st) : dec::lin_t<bf16, false, false>(L, st);
  return ccq ? dec::lin_t<float, true, false>(L, st) : dec::lin_t<float, false, false>(L, st);
}

hipError_t gma_decode_launch(const DecodeLaunch& L, hipStream_t st) {
  return L.bf16 ? dec::gma_t<bf16>(L, st) : dec::gma_t<float>(L, st);
}

}  // namespace lm
