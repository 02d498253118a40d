// gma_bwd.hip -- backward pass of Gaussian Mixture Attention, causal and
// bidirectional ("Gaussian Mixture Attention: Linear-Time Sequence Mixing via
// Probabilistic Latent Routing", method: core mechanism, latent memory routing,
// variants and training: the mixer is trained end to end, the variances
// through softplus and the priors through a softmax).
//
// The causal output is a linear attention whose features are the
// responsibilities: with A_ij = gamma(q_i) . gamma(k_j),
//   N_i = sum_{j<=i} A_ij v_j,  D_i = sum_{j<=i} A_ij + eps,  O_i = N_i / D_i,
// i.e. one linear attention (no decay) with keys gamma(k), queries gamma(q) and
// values [v | 1]. Its gradients with respect to the features and the values
// are those of that linear attention for the output gradient [dN | dD] with
// dN_i = dO_i / D_i and dD_i = -(dO_i . O_i) / D_i, so the float32 backward of
// decayed linear attention (gates = 1) computes them. What is left is the chain
// rule through the softmax and the Gaussian log joint
//   l_k(x) = log pi_k - 1/2 sum_d (log var_kd + (x_d - mu_kd)^2 / var_kd):
//   dl_k   = gamma_k (dgamma_k - sum_k' gamma_k' dgamma_k')
//   dx_d   = sum_k dl_k (mu_kd - x_d) / var_kd
//   dmu_kd = sum_tokens dl_k (x_d - mu_kd) / var_kd
//   dlog var_kd = sum_tokens dl_k (-1/2 + 1/2 (x_d - mu_kd)^2 / var_kd)
//   dlogit pi_k = G_k - pi_k sum_k' G_k',  G_k = sum_tokens dl_k
// with the parameter sums running over the query and the key tokens of every
// batch entry. Everything is float32 (for bf16 inputs the value gradient's
// pass runs on the bf16 chunk kernel); the inputs and dq, dk, dv are in the
// input dtype. The constant -d/2 log 2 pi of the log density cancels in the
// softmax and is left out.
//
// Bidirectional: every query reads the memory of the whole sequence, which is
// the causal linear attention over a sequence of 2N rows with the keys and
// values in rows [0, N) and the queries in rows [N, 2N) (zero rows elsewhere):
// the same inner forward and backward then give the gradients.
//
// Kernels: prep (per head: 1/var and the constant part of the log joint),
// route (responsibilities, one thread per component, 16 tokens per step),
// pack (values [v | 1 | 0], unit gates), out_grad (dN, dD from the forward),
// chain (softmax and log-joint chain rule per token, two threads per
// component; parameter partial sums per token range), reduce (fixed-order sum of the partials), params,
// take_dv.
#include "mfma.hpp"
#include "launch.hpp"
#include "bwd.hpp"

namespace lm {
namespace gbwd {

constexpr int kTT = 16;   // tokens per step of route and chain
constexpr int kThr = 128; // threads per workgroup: one per component (K <= 128)

// Per head: iv[k][d] = exp(-log_var), cst[k] = log pi_k - 1/2 sum_d log_var_kd
// (log pi = log-softmax of the mixing logits).
template <int NT>
__global__ __launch_bounds__(NT) void prep_kernel(const float* __restrict__ log_var,
                                                  const float* __restrict__ logit_pi, float* __restrict__ iv,
                                                  float* __restrict__ cst, int K, int D) {
  __shared__ float red[NT];
  const int h = blockIdx.x, k = threadIdx.x;
  const float lp = k < K ? logit_pi[(size_t)h * K + k] : -INFINITY;
  red[k] = lp;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (k < s) red[k] = fmaxf(red[k], red[k + s]);
    __syncthreads();
  }
  const float mx = red[0];
  __syncthreads();
  red[k] = k < K ? expf(lp - mx) : 0.f;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (k < s) red[k] += red[k + s];
    __syncthreads();
  }
  const float lse = mx + logf(red[0]);
  if (k >= K) return;
  float sl = 0.f;
  for (int d = 0; d < D; ++d) {
    const float l = log_var[((size_t)h * K + k) * D + d];
    sl += l;
    iv[((size_t)h * K + k) * D + d] = expf(-l);
  }
  cst[(size_t)h * K + k] = lp - lse - 0.5f * sl;
}

// Sum over the 128 threads of the workgroup of one value per thread, for kTT
// values at once; `red` holds 2 x kTT floats.
__device__ __forceinline__ void block_sum16(float (&x)[kTT], float* red) {
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    float s = x[t];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    x[t] = s;
  }
  if (lane_id() == 0) {
#pragma unroll
    for (int t = 0; t < kTT; ++t) red[wave_id() * kTT + t] = x[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kTT; ++t) x[t] = red[t] + red[kTT + t];
  __syncthreads();
}
__device__ __forceinline__ void block_max16(float (&x)[kTT], float* red) {
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    float s = x[t];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s = fmaxf(s, __shfl_xor(s, off));
    x[t] = s;
  }
  if (lane_id() == 0) {
#pragma unroll
    for (int t = 0; t < kTT; ++t) red[wave_id() * kTT + t] = x[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kTT; ++t) x[t] = fmaxf(red[t], red[kTT + t]);
  __syncthreads();
}

// The head's mu and 1/var as [kThr][D + 1] tables in LDS (zero rows beyond K).
template <int D>
__device__ __forceinline__ void load_tables(float (*smu)[D + 1], float (*siv)[D + 1], const float* __restrict__ mu,
                                            const float* __restrict__ iv, int h, int K) {
  for (int i = threadIdx.x; i < kThr * D; i += kThr) {
    const int r = i / D, cc = i - r * D;
    const bool ok = r < K;
    smu[r][cc] = ok ? mu[((size_t)h * K + r) * D + cc] : 0.f;
    siv[r][cc] = ok ? iv[((size_t)h * K + r) * D + cc] : 0.f;
  }
}

// Responsibilities of the tokens of x (q for blockIdx.z = 0, k for 1) as
// float32 rows of DL entries (components >= K are 0). Workgroup: one (b, h),
// kTT tokens per step over a range of `len` tokens; thread = component.
template <typename T, int D>
__global__ __launch_bounds__(kThr) void route_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                     const float* __restrict__ mu, const float* __restrict__ iv,
                                                     const float* __restrict__ cst, float* __restrict__ gq,
                                                     float* __restrict__ gk, int64_t N, int64_t NN, int64_t qoff,
                                                     int H, int K, int DL, int64_t len) {
  __shared__ float sx[kTT][D];
  __shared__ float red[2 * kTT];
  const int bh = blockIdx.y, h = bh % H, c = threadIdx.x;
  const T* __restrict__ x = (blockIdx.z == 0 ? q : k) + (size_t)bh * N * D;
  float* __restrict__ out = blockIdx.z == 0 ? gq + ((size_t)bh * NN + qoff) * DL : gk + (size_t)bh * NN * DL;
  // this thread's component row of mu and 1/var, in registers
  float muk[D], ivk[D];
  {
    const float* __restrict__ mr = mu + ((size_t)h * K + (c < K ? c : 0)) * D;
    const float* __restrict__ ir = iv + ((size_t)h * K + (c < K ? c : 0)) * D;
#pragma unroll
    for (int dd = 0; dd < D; ++dd) {
      muk[dd] = mr[dd];
      ivk[dd] = ir[dd];
    }
  }
  const float ck = c < K ? cst[(size_t)h * K + c] : 0.f;
  const int64_t t_begin = (int64_t)blockIdx.x * len;
  const int64_t t_end = N < t_begin + len ? N : t_begin + len;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTT) {
    const int nv = (int)(t_end - t0 < kTT ? t_end - t0 : kTT);
    for (int i = c; i < kTT * D; i += kThr) {
      const int t = i / D, dd = i - t * D;
      sx[t][dd] = t < nv ? to_f32(x[(size_t)(t0 + t) * D + dd]) : 0.f;
    }
    __syncthreads();
    float acc[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) acc[t] = 0.f;
    if (c < K) {
#pragma unroll
      for (int dd = 0; dd < D; ++dd) {
        const float m = muk[dd], w = ivk[dd];
#pragma unroll
        for (int t = 0; t < kTT; ++t) {
          const float e = sx[t][dd] - m;
          acc[t] += e * e * w;
        }
      }
    }
    float l[kTT], mx[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) mx[t] = l[t] = c < K ? ck - 0.5f * acc[t] : -INFINITY;
    block_max16(mx, red);
    float e[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) e[t] = c < K ? expf(l[t] - mx[t]) : 0.f;
    float s[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) s[t] = e[t];
    block_sum16(s, red);
    if (c < DL) {
      for (int t = 0; t < nv; ++t) out[(size_t)(t0 + t) * DL + c] = e[t] / s[t];
    }
  }
}

// Values of the inner linear attention [v | 1 | 0 ...] (DL columns) in rows
// [0, N) of each sequence's NN inner rows.
template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ v, float* __restrict__ vx, int64_t N,
                                                   int64_t NN, int64_t total, int DV, int DL) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t r = i / DL;  // bh * N + t
  const int c = (int)(i - r * DL);
  const int64_t bh = r / N, t = r - bh * N;
  vx[((size_t)bh * NN + t) * DL + c] = c < DV ? to_f32(v[r * DV + c]) : (c == DV ? 1.f : 0.f);
}

// rows [r0, r0 + nr) of every sequence of a [BH][NN][DL] tensor set to x
// (also the unit gates: DL = 1).
__global__ __launch_bounds__(256) void fill_rows_kernel(float* __restrict__ p, int64_t NN, int64_t r0, int64_t nr,
                                                        int DL, float x, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t per = nr * DL;
  const int64_t bh = i / per, e = i - bh * per;
  p[((size_t)bh * NN + r0) * DL + e] = x;
}

// From the inner forward y = [N | D - eps | ...] and dO: the output gradient of
// the inner linear attention [dN | dD | 0 ...], one wave per token (DV <= 64).
template <typename T>
__global__ __launch_bounds__(256) void out_grad_kernel(const float* __restrict__ y, const T* __restrict__ dout,
                                                       float* __restrict__ dy, int64_t N, int64_t NN, int64_t qoff,
                                                       int64_t rows, int DV, int DL, float eps) {
  const int64_t r = (int64_t)blockIdx.x * 4 + wave_id();  // bh * N + t
  if (r >= rows) return;
  const int64_t bh = r / N, yr = bh * NN + qoff + (r - bh * N);  // the query's inner row
  const int l = lane_id();
  const float den = y[yr * DL + DV] + eps;
  const float inv = 1.f / den;
  const float gd = l < DV ? to_f32(dout[r * DV + l]) : 0.f;
  const float o = l < DV ? y[yr * DL + l] * inv : 0.f;
  float s = gd * o;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  for (int c = l; c < DL; c += 64) dy[yr * DL + c] = c < DV ? gd * inv : (c == DV ? -s * inv : 0.f);
}

// Chain rule through the softmax and the log joint for the tokens of one side
// (blockIdx.z = 0: queries, 1: keys) of one (b, h), over a range of `len`
// tokens. Writes dx in the input dtype, and this range's parameter partial sums
//   part[h][slot][k] = [sum dl (x - mu) (D) | sum dl (x - mu)^2 (D) | sum dl]
// with slot = (side * B + b) * nseg + blockIdx.x. kCT = 256 threads: for the
// partial sums thread (half hh, component c) owns features [hh D/2, (hh+1) D/2)
// of component c (half the accumulators per thread, two waves per SIMD); for
// dx thread = (feature, token group).
constexpr int kCT = 2 * kThr;

__device__ __forceinline__ void block_sum16_4(float (&x)[kTT], float* red) {
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    float s = x[t];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    x[t] = s;
  }
  if (lane_id() == 0) {
#pragma unroll
    for (int t = 0; t < kTT; ++t) red[wave_id() * kTT + t] = x[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kTT; ++t) x[t] = (red[t] + red[kTT + t]) + (red[2 * kTT + t] + red[3 * kTT + t]);
  __syncthreads();
}

template <typename T, int D>
__global__ __launch_bounds__(kCT) void chain_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                    const float* __restrict__ gq, const float* __restrict__ gk,
                                                    const float* __restrict__ dgq, const float* __restrict__ dgk,
                                                    const float* __restrict__ mu, const float* __restrict__ iv,
                                                    T* __restrict__ dq, T* __restrict__ dk, float* __restrict__ part,
                                                    int64_t N, int64_t NN, int64_t qoff, int B, int H, int K, int DL,
                                                    int64_t len, int nseg) {
  constexpr int DH = D / 2;  // features per thread in the partial sums
  __shared__ float sx[kTT][D];
  __shared__ float sdl[kTT][kThr];
  __shared__ float red[4 * kTT];
  __shared__ float smu[kThr][D + 1];
  __shared__ float siv[kThr][D + 1];
  const int tid = threadIdx.x;
  const int c = tid % kThr, hh = tid / kThr;  // component, feature half
  const int bh = blockIdx.y, b = bh / H, h = bh % H, side = blockIdx.z;
  const T* __restrict__ x = (side == 0 ? q : k) + (size_t)bh * N * D;
  T* __restrict__ dx = (side == 0 ? dq : dk) + (size_t)bh * N * D;
  const size_t row0 = (size_t)bh * NN + (side == 0 ? qoff : 0);  // inner row of this side's token 0
  const float* __restrict__ gx = (side == 0 ? gq : gk) + row0 * DL;
  const float* __restrict__ dgx = (side == 0 ? dgq : dgk) + row0 * DL;
  for (int i = tid; i < kThr * D; i += kCT) {
    const int rr = i / D, cc = i - rr * D;
    const bool ok = rr < K;
    smu[rr][cc] = ok ? mu[((size_t)h * K + rr) * D + cc] : 0.f;
    siv[rr][cc] = ok ? iv[((size_t)h * K + rr) * D + cc] : 0.f;
  }
  // dx mapping: feature fd = tid % D, tokens t = tid / D + j * (kCT / D)
  constexpr int TG = kCT / D;   // token groups
  constexpr int TPT = kTT / TG; // tokens per thread
  const int fd = tid % D, tg = tid / D;
  const int d0 = hh * DH;

  float p1[DH], p2[DH], p0 = 0.f;
#pragma unroll
  for (int i = 0; i < DH; ++i) p1[i] = p2[i] = 0.f;

  const int64_t t_begin = (int64_t)blockIdx.x * len;
  const int64_t t_end = N < t_begin + len ? N : t_begin + len;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTT) {
    const int nv = (int)(t_end - t0 < kTT ? t_end - t0 : kTT);
    for (int i = tid; i < kTT * D; i += kCT) {
      const int t = i / D, dd = i - t * D;
      sx[t][dd] = t < nv ? to_f32(x[(size_t)(t0 + t) * D + dd]) : 0.f;
    }
    float ga[kTT], dga[kTT], r[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) {
      const bool ok = c < K && t < nv;
      ga[t] = ok ? gx[(size_t)(t0 + t) * DL + c] : 0.f;
      dga[t] = ok ? dgx[(size_t)(t0 + t) * DL + c] : 0.f;
      r[t] = hh == 0 ? ga[t] * dga[t] : 0.f;  // each component counted once
    }
    block_sum16_4(r, red);  // also orders the sx writes (and the tables) before the reads below
    float dl[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) {
      dl[t] = ga[t] * (dga[t] - r[t]);
      p0 += dl[t];
    }
    if (hh == 0) {
#pragma unroll
      for (int t = 0; t < kTT; ++t) sdl[t][c] = dl[t];
    }
    if (c < K) {
#pragma unroll
      for (int i = 0; i < DH; ++i) {
        const float m = smu[c][d0 + i];
#pragma unroll
        for (int t = 0; t < kTT; ++t) {
          const float e = sx[t][d0 + i] - m;
          const float a = dl[t] * e;
          p1[i] += a;
          p2[i] += a * e;
        }
      }
    }
    __syncthreads();
    // dx_d = sum_k dl_k mu_kd iv_kd - x_d sum_k dl_k iv_kd
    float s1[TPT], s2[TPT];
#pragma unroll
    for (int j = 0; j < TPT; ++j) s1[j] = s2[j] = 0.f;
    for (int kk = 0; kk < K; ++kk) {
      const float w = siv[kk][fd];
      const float a = smu[kk][fd] * w;
#pragma unroll
      for (int j = 0; j < TPT; ++j) {
        const float d_ = sdl[tg + j * TG][kk];
        s1[j] += d_ * a;
        s2[j] += d_ * w;
      }
    }
#pragma unroll
    for (int j = 0; j < TPT; ++j) {
      const int t = tg + j * TG;
      if (t < nv) dx[(size_t)(t0 + t) * D + fd] = from_f32<T>(s1[j] - sx[t][fd] * s2[j]);
    }
    __syncthreads();
  }
  if (c < K) {
    const int slot = (side * B + b) * nseg + (int)blockIdx.x;
    float* dst = part + (((size_t)h * 2 * B * nseg + slot) * K + c) * (2 * D + 1);
#pragma unroll
    for (int i = 0; i < DH; ++i) {
      dst[d0 + i] = p1[i];
      dst[D + d0 + i] = p2[i];
    }
    if (hh == 0) dst[2 * D] = p0;
  }
}

// Sum of the partial sums over the slots, in a fixed order: one thread per
// (head, component, entry); red[h][k][F] with F = 2 D + 1.
__global__ __launch_bounds__(256) void reduce_kernel(const float* __restrict__ part, float* __restrict__ red,
                                                     int64_t n, int K, int F, int nslot) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n) return;
  const int64_t h = i / ((int64_t)K * F), e = i - h * K * F;  // e = k * F + f
  const float* src = part + (size_t)h * nslot * K * F + e;
  float s = 0.f;
  for (int sl = 0; sl < nslot; ++sl) s += src[(size_t)sl * K * F];
  red[i] = s;
}

// Parameter gradients per head from the summed partials S1, S2, S0:
// dmu = iv * S1, dlog_var = -1/2 S0 + 1/2 iv * S2, dlogit_pi = S0 - pi * sum S0.
template <int NT>
__global__ __launch_bounds__(NT) void params_kernel(const float* __restrict__ sums, const float* __restrict__ iv,
                                                    const float* __restrict__ logit_pi, float* __restrict__ dmu,
                                                    float* __restrict__ dlv, float* __restrict__ dlp, int K,
                                                    int D) {
  __shared__ float red[NT];
  const int h = blockIdx.x, c = threadIdx.x;
  const int F = 2 * D + 1;
  const float* base = sums + ((size_t)h * K + (c < K ? c : 0)) * F;
  const float g0 = c < K ? base[2 * D] : 0.f;
  if (c < K) {
    for (int dd = 0; dd < D; ++dd) {
      const float w = iv[((size_t)h * K + c) * D + dd];
      dmu[((size_t)h * K + c) * D + dd] = w * base[dd];
      dlv[((size_t)h * K + c) * D + dd] = -0.5f * g0 + 0.5f * w * base[D + dd];
    }
  }
  // pi and the total of G over the components
  const float lp = c < K ? logit_pi[(size_t)h * K + c] : -INFINITY;
  red[c] = lp;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (c < s) red[c] = fmaxf(red[c], red[c + s]);
    __syncthreads();
  }
  const float mx = red[0];
  __syncthreads();
  const float e = c < K ? expf(lp - mx) : 0.f;
  red[c] = e;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (c < s) red[c] += red[c + s];
    __syncthreads();
  }
  const float pi = e / red[0];
  __syncthreads();
  red[c] = g0;
  __syncthreads();
  for (int s = NT / 2; s > 0; s >>= 1) {
    if (c < s) red[c] += red[c + s];
    __syncthreads();
  }
  if (c < K) dlp[(size_t)h * K + c] = g0 - pi * red[0];
}

// dv = the first DV columns of the inner value gradient, in the input dtype.
template <typename T, typename TI>
__global__ __launch_bounds__(256) void take_dv_kernel(const TI* __restrict__ dvx, T* __restrict__ dv, int64_t N,
                                                      int64_t NN, int64_t rows, int DV, int DL) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= rows * DV) return;
  const int64_t r = i / DV;  // bh * N + t
  const int c = (int)(i - r * DV);
  const int64_t bh = r / N;
  dv[i] = from_f32<T>(to_f32(dvx[((size_t)bh * NN + (r - bh * N)) * DL + c]));
}

static hipError_t fill_rows(float* p, const GmaBwdLaunch& L, int64_t r0, int64_t nr, int DL, float x,
                            hipStream_t st) {
  const int64_t total = L.B * L.H * nr * DL;
  hipLaunchKernelGGL(fill_rows_kernel, dim3((unsigned)((total + 255) / 256)), dim3(256), 0, st, p, L.NN, r0, nr, DL, x,
                     total);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t run(const GmaBwdLaunch& L, hipStream_t st) {
  const int64_t BH = L.B * L.H, rows = BH * L.N;
  const int K = (int)L.K, DL = (int)L.DL, H = (int)L.H;
  const int64_t N = L.N, NN = L.NN, qoff = L.causal ? 0 : N;
  hipError_t e;
  hipLaunchKernelGGL(prep_kernel<kThr>, dim3((unsigned)H), dim3(kThr), 0, st, L.log_var, L.logit_pi, L.iv, L.cst, K,
                     D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if (!L.causal) {
    // bidirectional: queries in rows [N, 2N), keys and values in [0, N)
    if ((e = fill_rows(L.gq, L, 0, N, DL, 0.f, st)) != hipSuccess) return e;
    if ((e = fill_rows(L.gk, L, N, N, DL, 0.f, st)) != hipSuccess) return e;
    if ((e = fill_rows(L.vx, L, N, N, DL, 0.f, st)) != hipSuccess) return e;
    if ((e = fill_rows(L.dy, L, 0, N, DL, 0.f, st)) != hipSuccess) return e;
  }
  if ((e = fill_rows(L.ones, L, 0, NN, 1, 1.f, st)) != hipSuccess) return e;
  const dim3 grid((unsigned)L.nseg, (unsigned)BH, 2);
  hipLaunchKernelGGL((route_kernel<T, D>), grid, dim3(kThr), 0, st, static_cast<const T*>(L.q),
                     static_cast<const T*>(L.k), L.mu, L.iv, L.cst, L.gq, L.gk, N, NN, qoff, H, K, DL, L.seg_len);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((pack_kernel<T>), dim3((unsigned)((rows * DL + 255) / 256)), dim3(256), 0, st,
                     static_cast<const T*>(L.v), L.vx, N, NN, rows * DL, D, DL);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // inner forward: y = [N | D - eps | 0 ...] at the query rows
  LinLaunch F = L.bwd.fwd;
  F.q = L.gq;
  F.k = L.gk;
  F.v = L.vx;
  F.g = L.ones;
  F.out = L.y;
  F.bf16 = false;
  F.ccq = false;
  F.state_in = nullptr;
  F.state_out = nullptr;
  F.t_in = 0;
  if ((e = linattn_launch(F, st)) != hipSuccess) return e;
  hipLaunchKernelGGL((out_grad_kernel<T>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, L.y,
                     static_cast<const T*>(L.dout), L.dy, N, NN, qoff, rows, D, DL, L.eps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // gradients of the inner linear attention: features (dgq, dgk) and values
  BwdLaunch Bw = L.bwd;
  Bw.g = L.ones;
  bf16* dv16 = reinterpret_cast<bf16*>(L.dvx);
  if constexpr (sizeof(T) == 2) {
    // the value gradient (which nothing else uses) on bf16 operands: reversed
    // responsibilities of k and q and output gradient, in the slots of the
    // (now dead) inner output and of the inner reversed k
    const int64_t ni = BH * NN * DL;
    bf16* a16 = reinterpret_cast<bf16*>(L.y);
    bf16* b16 = reinterpret_cast<bf16*>(Bw.rk);
    if ((e = reverse_to_bf16<float>(L.gk, a16, BH, NN, DL, st)) != hipSuccess) return e;
    if ((e = reverse_to_bf16<float>(L.gq, a16 + ni, BH, NN, DL, st)) != hipSuccess) return e;
    if ((e = reverse_to_bf16<float>(L.dy, b16, BH, NN, DL, st)) != hipSuccess) return e;
    if ((e = linattn_backward_mixed(Bw, L.gq, L.gk, L.vx, L.dy, L.dgq, L.dgk, false, a16, a16 + ni, b16, b16 + ni,
                                    dv16, st)) != hipSuccess)
      return e;
  } else {
    if ((e = linattn_backward_f32(Bw, L.gq, L.gk, L.vx, L.dy, L.dgq, L.dgk, L.dvx, false, st)) != hipSuccess)
      return e;
  }
  hipLaunchKernelGGL((chain_kernel<T, D>), grid, dim3(kCT), 0, st, static_cast<const T*>(L.q),
                     static_cast<const T*>(L.k), L.gq, L.gk, L.dgq, L.dgk, L.mu, L.iv, static_cast<T*>(L.dq),
                     static_cast<T*>(L.dk), L.part, N, NN, qoff, (int)L.B, H, K, DL, L.seg_len, (int)L.nseg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int NF = 2 * D + 1;
  const int64_t nred = (int64_t)H * K * NF;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((nred + 255) / 256)), dim3(256), 0, st, L.part, L.sums, nred, K,
                     NF, (int)(2 * L.B * L.nseg));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(params_kernel<kThr>, dim3((unsigned)H), dim3(kThr), 0, st, L.sums, L.iv, L.logit_pi, L.dmu,
                     L.dlog_var, L.dlogit_pi, K, D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  if constexpr (sizeof(T) == 2)
    hipLaunchKernelGGL((take_dv_kernel<T, bf16>), dim3((unsigned)((rows * D + 255) / 256)), dim3(256), 0, st, dv16,
                       static_cast<T*>(L.dv), N, NN, rows, D, DL);
  else
    hipLaunchKernelGGL((take_dv_kernel<T, float>), dim3((unsigned)((rows * D + 255) / 256)), dim3(256), 0, st,
                       L.dvx, static_cast<T*>(L.dv), N, NN, rows, D, DL);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Wide shapes: d = 128 or more than 128 components (K <= 256). The inner
// linear attention then has more than 128 features (K) or value columns
// (d + 1), so its tensors are cut into blocks of 128 columns, each a dense
// [B*H][NN][128] float32 tensor (block b at b * bstride floats): the
// responsibilities and their gradients in NF = ceil(K / 128) blocks, the
// values [v | 1 | 0 ...], the inner output and its gradient and the value
// gradient in NVB = ceil((d + 1) / 128) blocks. The inner products are sums
// over the feature blocks, so the inner forward and backward run once per
// (feature block, value block) pair and the results are summed.
constexpr int kWT = 256;  // threads of the routing and partial-sum kernels: one per component

__device__ __forceinline__ size_t wcol(int c, size_t bstride) { return (size_t)(c >> 7) * bstride + (c & 127); }

// Sums / maxima over the 256 threads (4 waves) of kTT values at once; red holds 4 kTT floats.
template <bool MAX>
__device__ __forceinline__ void block_red4(float (&x)[kTT], float* red) {
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    float v = x[t];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) {
      const float o = __shfl_xor(v, off);
      v = MAX ? fmaxf(v, o) : v + o;
    }
    x[t] = v;
  }
  if (lane_id() == 0) {
#pragma unroll
    for (int t = 0; t < kTT; ++t) red[wave_id() * kTT + t] = x[t];
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < kTT; ++t) {
    const float a = red[t], b = red[kTT + t], c = red[2 * kTT + t], d = red[3 * kTT + t];
    x[t] = MAX ? fmaxf(fmaxf(a, b), fmaxf(c, d)) : (a + b) + (c + d);
  }
  __syncthreads();
}

// Responsibilities of q (blockIdx.z = 0) or k (1) in the block layout; thread =
// component; the component's mu and 1/var pass through registers 32 features
// at a time.
template <typename T, int D>
__global__ __launch_bounds__(kWT) void route_wide_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                         const float* __restrict__ mu, const float* __restrict__ iv,
                                                         const float* __restrict__ cst, float* __restrict__ gq,
                                                         float* __restrict__ gk, size_t bstride, int64_t N,
                                                         int64_t NN, int64_t qoff, int H, int K, int NF, int64_t len) {
  __shared__ float sx[kTT][D];
  __shared__ float red[4 * kTT];
  const int bh = blockIdx.y, h = bh % H, c = threadIdx.x;
  const T* __restrict__ x = (blockIdx.z == 0 ? q : k) + (size_t)bh * N * D;
  float* __restrict__ out = blockIdx.z == 0 ? gq + ((size_t)bh * NN + qoff) * 128 : gk + (size_t)bh * NN * 128;
  const bool live = c < K;
  const float* __restrict__ mr = mu + ((size_t)h * K + (live ? c : 0)) * D;
  const float* __restrict__ ir = iv + ((size_t)h * K + (live ? c : 0)) * D;
  const float ck = live ? cst[(size_t)h * K + c] : 0.f;
  const int64_t t_begin = (int64_t)blockIdx.x * len;
  const int64_t t_end = N < t_begin + len ? N : t_begin + len;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTT) {
    const int nv = (int)(t_end - t0 < kTT ? t_end - t0 : kTT);
    for (int i = c; i < kTT * D; i += kWT) {
      const int t = i / D, dd = i - t * D;
      sx[t][dd] = t < nv ? to_f32(x[(size_t)(t0 + t) * D + dd]) : 0.f;
    }
    __syncthreads();
    float acc[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) acc[t] = 0.f;
    if (live) {
      for (int d0 = 0; d0 < D; d0 += 32) {
        float m[32], w[32];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          m[i] = mr[d0 + i];
          w[i] = ir[d0 + i];
        }
#pragma unroll
        for (int i = 0; i < 32; ++i)
#pragma unroll
          for (int t = 0; t < kTT; ++t) {
            const float e = sx[t][d0 + i] - m[i];
            acc[t] += e * e * w[i];
          }
      }
    }
    float l[kTT], mx[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) mx[t] = l[t] = live ? ck - 0.5f * acc[t] : -INFINITY;
    block_red4<true>(mx, red);
    float e[kTT], sm[kTT];
#pragma unroll
    for (int t = 0; t < kTT; ++t) sm[t] = e[t] = live ? expf(l[t] - mx[t]) : 0.f;
    block_red4<false>(sm, red);
    if (c < NF * 128) {
      for (int t = 0; t < nv; ++t) out[(size_t)(t0 + t) * 128 + wcol(c, bstride)] = e[t] / sm[t];
    }
  }
}

// Values [v | 1 | 0 ...] of the inner linear attention in the block layout
// (rows [0, N) of each sequence's NN rows).
template <typename T>
__global__ __launch_bounds__(256) void pack_wide_kernel(const T* __restrict__ v, float* __restrict__ vx,
                                                        size_t bstride, int64_t N, int64_t NN, int64_t total, int DV,
                                                        int NVB) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int W = NVB * 128;
  const int64_t r = i / W;  // bh * N + t
  const int c = (int)(i - r * W);
  const int64_t bh = r / N, t = r - bh * N;
  vx[((size_t)bh * NN + t) * 128 + wcol(c, bstride)] = c < DV ? to_f32(v[r * DV + c]) : (c == DV ? 1.f : 0.f);
}

// Output gradient [dN | dD | 0 ...] of the inner linear attention from its
// output y = [N | D - eps | ...] and dO, one wave per token, block layout.
template <typename T>
__global__ __launch_bounds__(256) void out_grad_wide_kernel(const float* __restrict__ y, const T* __restrict__ dout,
                                                            float* __restrict__ dy, size_t bstride, int64_t N,
                                                            int64_t NN, int64_t qoff, int64_t rows, int DV, int NVB,
                                                            float eps) {
  const int64_t r = (int64_t)blockIdx.x * 4 + wave_id();  // bh * N + t
  if (r >= rows) return;
  const int64_t bh = r / N, yr = bh * NN + qoff + (r - bh * N);
  const int l = lane_id();
  const float inv = 1.f / (y[yr * 128 + wcol(DV, bstride)] + eps);
  float s = 0.f;
  for (int c = l; c < DV; c += 64) s += to_f32(dout[r * DV + c]) * y[yr * 128 + wcol(c, bstride)] * inv;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
  for (int c = l; c < NVB * 128; c += 64)
    dy[yr * 128 + wcol(c, bstride)] = c < DV ? to_f32(dout[r * DV + c]) * inv : (c == DV ? -s * inv : 0.f);
}

// a[i] += b[i]
__global__ __launch_bounds__(256) void add_kernel(float* __restrict__ a, const float* __restrict__ b, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) a[i] += b[i];
}

// Softmax backward per token of one side: dl_k = g_k (dg_k - sum_k' g_k' dg_k'),
// written as rows of 256 floats (zero past K); one wave per token.
__global__ __launch_bounds__(256) void dl_wide_kernel(const float* __restrict__ gx, const float* __restrict__ dgx,
                                                      float* __restrict__ dl, size_t bstride, int64_t N, int64_t NN,
                                                      int64_t off, int64_t rows, int K) {
  const int64_t r = (int64_t)blockIdx.x * 4 + wave_id();  // bh * N + t
  if (r >= rows) return;
  const int64_t bh = r / N, xr = bh * NN + off + (r - bh * N);
  const int l = lane_id();
  float g[4], dg[4], s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int c = l + 64 * m;
    const bool ok = c < K;
    g[m] = ok ? gx[xr * 128 + wcol(c, bstride)] : 0.f;
    dg[m] = ok ? dgx[xr * 128 + wcol(c, bstride)] : 0.f;
    s += g[m] * dg[m];
  }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) s += __shfl_xor(s, o);
  // The component with the largest responsibility: where it holds almost all
  // the mass, dg - s is a difference of two nearly equal numbers, so its dl is
  // formed as g sum_k' g_k' (dg - dg_k') instead (the same value, as the
  // responsibilities sum to 1), whose terms carry no cancellation.
  float bv = g[0];
  int bi = l;
#pragma unroll
  for (int m = 1; m < 4; ++m)
    if (g[m] > bv) {
      bv = g[m];
      bi = l + 64 * m;
    }
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) {
    const float ov = __shfl_xor(bv, o);
    const int oi = __shfl_xor(bi, o);
    if (ov > bv || (ov == bv && oi < bi)) {
      bv = ov;
      bi = oi;
    }
  }
  const int cs = __builtin_amdgcn_readfirstlane(bi);
  const float own = cs < 64 ? dg[0] : cs < 128 ? dg[1] : cs < 192 ? dg[2] : dg[3];
  const float dgs = __shfl(own, cs & 63);
  float rr = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) rr += g[m] * (dgs - dg[m]);
#pragma unroll
  for (int o = 32; o > 0; o >>= 1) rr += __shfl_xor(rr, o);
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int c = l + 64 * m;
    dl[r * 256 + c] = c == cs ? g[m] * rr : g[m] * (dg[m] - s);
  }
}

// dx_d = sum_k dl_k mu_kd / var_kd - x_d sum_k dl_k / var_kd for kTT tokens of
// one side per workgroup; thread = feature.
template <typename T, int D>
__global__ __launch_bounds__(D < 64 ? 64 : D) void dx_wide_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                                 const float* __restrict__ dlq,
                                                                 const float* __restrict__ dlk,
                                                                 const float* __restrict__ mu,
                                                                 const float* __restrict__ iv, T* __restrict__ dq,
                                                                 T* __restrict__ dk, int64_t N, int H, int K) {
  __shared__ float sdl[kTT][256];
  const int bh = blockIdx.y, h = bh % H, side = blockIdx.z, d = threadIdx.x;
  const int64_t t0 = (int64_t)blockIdx.x * kTT;
  const int nv = (int)(N - t0 < kTT ? N - t0 : kTT);
  const float* __restrict__ dl = (side == 0 ? dlq : dlk) + ((size_t)bh * N + t0) * 256;
  for (int i = threadIdx.x; i < kTT * 256; i += blockDim.x) sdl[i / 256][i % 256] = i / 256 < nv ? dl[i] : 0.f;
  __syncthreads();
  if (d >= D) return;
  float s1[kTT], s2[kTT];
#pragma unroll
  for (int t = 0; t < kTT; ++t) s1[t] = s2[t] = 0.f;
  for (int c = 0; c < K; ++c) {
    const float w = iv[((size_t)h * K + c) * D + d];
    const float a = mu[((size_t)h * K + c) * D + d] * w;
#pragma unroll
    for (int t = 0; t < kTT; ++t) {
      s1[t] += sdl[t][c] * a;
      s2[t] += sdl[t][c] * w;
    }
  }
  const T* __restrict__ x = (side == 0 ? q : k) + ((size_t)bh * N + t0) * D;
  T* __restrict__ dx = (side == 0 ? dq : dk) + ((size_t)bh * N + t0) * D;
  for (int t = 0; t < nv; ++t) dx[(size_t)t * D + d] = from_f32<T>(s1[t] - to_f32(x[(size_t)t * D + d]) * s2[t]);
}

// Parameter partial sums of one token range of one side and 32 features:
//   part[h][slot][k] = [sum dl (x - mu) (D) | sum dl (x - mu)^2 (D) | sum dl]
// (the features d0 .. d0 + 31 of the first two, and the last entry from the
// first feature chunk), slot = (side * B + b) * nseg + range; thread = component.
template <typename T, int D>
__global__ __launch_bounds__(kWT) void partial_wide_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                           const float* __restrict__ dlq,
                                                           const float* __restrict__ dlk,
                                                           const float* __restrict__ mu, float* __restrict__ part,
                                                           int64_t N, int B, int H, int K, int64_t len, int nseg) {
  __shared__ float sx[kTT][32];
  constexpr int NDC = D / 32;
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  const int side = blockIdx.z / NDC, d0 = 32 * (blockIdx.z % NDC), c = threadIdx.x;
  const T* __restrict__ x = (side == 0 ? q : k) + (size_t)bh * N * D;
  const float* __restrict__ dl = (side == 0 ? dlq : dlk) + (size_t)bh * N * 256;
  const bool live = c < K;
  float m[32], p1[32], p2[32], p0 = 0.f;
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    m[i] = live ? mu[((size_t)h * K + c) * D + d0 + i] : 0.f;
    p1[i] = p2[i] = 0.f;
  }
  const int64_t t_begin = (int64_t)blockIdx.x * len;
  const int64_t t_end = N < t_begin + len ? N : t_begin + len;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kTT) {
    const int nv = (int)(t_end - t0 < kTT ? t_end - t0 : kTT);
    for (int i = c; i < kTT * 32; i += kWT) {
      const int t = i / 32, dd = i % 32;
      sx[t][dd] = t < nv ? to_f32(x[(size_t)(t0 + t) * D + d0 + dd]) : 0.f;
    }
    __syncthreads();
    for (int t = 0; t < nv; ++t) {
      const float g = dl[(size_t)(t0 + t) * 256 + c];
      p0 += g;
#pragma unroll
      for (int i = 0; i < 32; ++i) {
        const float e = sx[t][i] - m[i];
        const float a = g * e;
        p1[i] += a;
        p2[i] += a * e;
      }
    }
    __syncthreads();
  }
  if (live) {
    const int slot = (side * B + b) * nseg + (int)blockIdx.x;
    float* dst = part + (((size_t)h * 2 * B * nseg + slot) * K + c) * (2 * D + 1);
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      dst[d0 + i] = p1[i];
      dst[D + d0 + i] = p2[i];
    }
    if (d0 == 0) dst[2 * D] = p0;
  }
}

static hipError_t add_into(float* a, const float* b, int64_t n, hipStream_t st) {
  hipLaunchKernelGGL(add_kernel, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, a, b, n);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t run_wide(const GmaBwdLaunch& L, hipStream_t st) {
  const int64_t BH = L.B * L.H, rows = BH * L.N;
  const int K = (int)L.K, H = (int)L.H, NF = (int)L.NF, NVB = (int)L.NVB;
  const int64_t N = L.N, NN = L.NN, qoff = L.causal ? 0 : N;
  const size_t bs = L.bstride;  // floats per block tensor: B*H*NN*128
  hipError_t e;
  hipLaunchKernelGGL(prep_kernel<kWT>, dim3((unsigned)H), dim3(kWT), 0, st, L.log_var, L.logit_pi, L.iv, L.cst, K, D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  for (int b = 0; b < 2; ++b) {
    if (!L.causal) {
      // bidirectional: queries in rows [N, 2N), keys and values in [0, N)
      if ((e = fill_rows(L.gq + b * bs, L, 0, N, 128, 0.f, st)) != hipSuccess) return e;
      if ((e = fill_rows(L.gk + b * bs, L, N, N, 128, 0.f, st)) != hipSuccess) return e;
      if ((e = fill_rows(L.vx + b * bs, L, N, N, 128, 0.f, st)) != hipSuccess) return e;
      if ((e = fill_rows(L.dy + b * bs, L, 0, N, 128, 0.f, st)) != hipSuccess) return e;
    }
  }
  if ((e = fill_rows(L.ones, L, 0, NN, 1, 1.f, st)) != hipSuccess) return e;
  const dim3 grid((unsigned)L.nseg, (unsigned)BH, 2);
  hipLaunchKernelGGL((route_wide_kernel<T, D>), grid, dim3(kWT), 0, st, static_cast<const T*>(L.q),
                     static_cast<const T*>(L.k), L.mu, L.iv, L.cst, L.gq, L.gk, bs, N, NN, qoff, H, K, NF, L.seg_len);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t npk = rows * NVB * 128;
  hipLaunchKernelGGL((pack_wide_kernel<T>), dim3((unsigned)((npk + 255) / 256)), dim3(256), 0, st,
                     static_cast<const T*>(L.v), L.vx, bs, N, NN, npk, D, NVB);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // inner forward, y_vb = sum_fb LA(gq_fb, gk_fb, vx_vb)
  LinLaunch F = L.bwd.fwd;
  F.g = L.ones;
  F.bf16 = false;
  F.ccq = false;
  F.state_in = nullptr;
  F.state_out = nullptr;
  F.t_in = 0;
  for (int vb = 0; vb < NVB; ++vb) {
    for (int fb = 0; fb < NF; ++fb) {
      F.q = L.gq + fb * bs;
      F.k = L.gk + fb * bs;
      F.v = L.vx + vb * bs;
      F.out = fb == 0 ? L.y + vb * bs : L.tq;
      if ((e = linattn_launch(F, st)) != hipSuccess) return e;
      if (fb > 0 && (e = add_into(L.y + vb * bs, L.tq, (int64_t)bs, st)) != hipSuccess) return e;
    }
  }
  hipLaunchKernelGGL((out_grad_wide_kernel<T>), dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, L.y,
                     static_cast<const T*>(L.dout), L.dy, bs, N, NN, qoff, rows, D, NVB, L.eps);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // inner backward per (feature block, value block), summed
  BwdLaunch Bw = L.bwd;
  Bw.g = L.ones;
  for (int fb = 0; fb < NF; ++fb) {
    for (int vb = 0; vb < NVB; ++vb) {
      float* oq = vb == 0 ? L.dgq + fb * bs : L.tq;
      float* ok = vb == 0 ? L.dgk + fb * bs : L.tk;
      float* ov = fb == 0 ? L.dvx + vb * bs : L.tv;
      if ((e = linattn_backward_f32(Bw, L.gq + fb * bs, L.gk + fb * bs, L.vx + vb * bs, L.dy + vb * bs, oq, ok, ov,
                                    false, st)) != hipSuccess)
        return e;
      if (vb > 0 && (e = add_into(L.dgq + fb * bs, L.tq, (int64_t)bs, st)) != hipSuccess) return e;
      if (vb > 0 && (e = add_into(L.dgk + fb * bs, L.tk, (int64_t)bs, st)) != hipSuccess) return e;
      if (fb > 0 && (e = add_into(L.dvx + vb * bs, L.tv, (int64_t)bs, st)) != hipSuccess) return e;
    }
  }
  // chain rule: softmax backward per token (into the dead inner output and its
  // gradient: B*H*N rows of 256 floats each), dx, parameter partial sums
  float* dlq = L.y;
  float* dlk = L.dy;
  hipLaunchKernelGGL(dl_wide_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, L.gq, L.dgq, dlq, bs, N, NN,
                     qoff, rows, K);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(dl_wide_kernel, dim3((unsigned)((rows + 3) / 4)), dim3(256), 0, st, L.gk, L.dgk, dlk, bs, N, NN,
                     (int64_t)0, rows, K);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((dx_wide_kernel<T, D>), dim3((unsigned)((N + kTT - 1) / kTT), (unsigned)BH, 2),
                     dim3(D < 64 ? 64 : D), 0, st, static_cast<const T*>(L.q), static_cast<const T*>(L.k), dlq, dlk,
                     L.mu, L.iv, static_cast<T*>(L.dq), static_cast<T*>(L.dk), N, H, K);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL((partial_wide_kernel<T, D>), dim3((unsigned)L.nseg, (unsigned)BH, (unsigned)(2 * (D / 32))),
                     dim3(kWT), 0, st, static_cast<const T*>(L.q), static_cast<const T*>(L.k), dlq, dlk, L.mu, L.part,
                     N, (int)L.B, H, K, L.seg_len, (int)L.nseg);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int NFP = 2 * D + 1;
  const int64_t nred = (int64_t)H * K * NFP;
  hipLaunchKernelGGL(reduce_kernel, dim3((unsigned)((nred + 255) / 256)), dim3(256), 0, st, L.part, L.sums, nred, K,
                     NFP, (int)(2 * L.B * L.nseg));
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(params_kernel<kWT>, dim3((unsigned)H), dim3(kWT), 0, st, L.sums, L.iv, L.logit_pi, L.dmu,
                     L.dlog_var, L.dlogit_pi, K, D);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dv: the first d columns of the value gradient (block 0)
  hipLaunchKernelGGL((take_dv_kernel<T, float>), dim3((unsigned)((rows * D + 255) / 256)), dim3(256), 0, st, L.dvx,
                     static_cast<T*>(L.dv), N, NN, rows, D, 128);
  return hipGetLastError();
}

}  // namespace gbwd

hipError_t gma_backward_launch(const GmaBwdLaunch& L, hipStream_t st) {
  using namespace gbwd;
  if (L.NF > 1 || L.NVB > 1) {
    if (L.bf16) {
      if (L.D == 32) return run_wide<bf16, 32>(L, st);
      if (L.D == 64) return run_wide<bf16, 64>(L, st);
      if (L.D == 128) return run_wide<bf16, 128>(L, st);
    } else {
      if (L.D == 32) return run_wide<float, 32>(L, st);
      if (L.D == 64) return run_wide<float, 64>(L, st);
      if (L.D == 128) return run_wide<float, 128>(L, st);
    }
    return hipErrorInvalidValue;
  }
  if (L.bf16) {
    if (L.D == 32) return run<bf16, 32>(L, st);
    if (L.D == 64) return run<bf16, 64>(L, st);
  } else {
    if (L.D == 32) return run<float, 32>(L, st);
    if (L.D == 64) return run<float, 64>(L, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lm
