// ccq_bwd.hip -- backward pass of the curvature-conditioned-query read over
// decayed linear attention ("Don't Read Everything: A Curvature-Conditioned
// Query for Linear Attention", section 2 Method: derivation, mechanism,
// integration; the read is trained with the rest of the layer).
//
// Forward (token t, count t = index + 1): m_t = sum_{j<=t} k_j,
// Mq_t = sum_{j<=t} k_j (k_j . q_t), s_t = Sigma_t q_t = (Mq_t - m_t (m_t . q_t) / t) / t,
// lambda_t = sigmoid(w . q_t + b), qc_t = q_t - lambda_t s_t, and
// o = GLA(qc, k, v, g) (S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T qc_t).
// With u = dL/dqc (from the backward of the decayed linear attention, which
// also gives dv, dg and the direct part of dk):
//   a_t   = u_t . s_t,  lambda'_t = lambda_t (1 - lambda_t)
//   dq_t  = u_t - lambda_t Sigma_t u_t - a_t lambda'_t w
//   dw    = -sum_t a_t lambda'_t q_t,  db = -sum_t a_t lambda'_t
//   dk_j += -sum_{t>=j} (lambda_t / t) [u_t (q_t . k_j) + q_t (u_t . k_j)] + sum_{t>=j} dm_t,
//   dm_t  = (lambda_t / t^2) [u_t (q_t . m_t) + q_t (u_t . m_t)]
// (dL/dSigma_t = -lambda_t u_t q_t^T, through M_t / t and m_t m_t^T / t^2).
// Mq and Sigma u are linear attentions without decay (key k, value k); the two
// sums over t >= j are linear attentions on the time-reversed sequence. All of
// them run on the chunk kernel with unit gates. Everything is float32 and bf16
// gradients are rounded once, except for bf16 inputs: there the undecayed
// passes and the dv pass run on the bf16 chunk kernel (their results enter the
// gradients as perturbations of the size of the bf16 rounding; the gradients
// of the decayed read, whose gate gradient cancels, stay in float32). At
// D = 128 with enough sequences the decayed read's backward is the fused bf16
// kernel of linattn_bwd_bf16.hip (dq and dk carried to about 16 bits there,
// the gate gradient formed inside it), fed q_clean rounded once to bf16.
#include "mfma.hpp"
#include "launch.hpp"
#include "bwd.hpp"

namespace lm {
namespace cbwd {

// Four consecutive features of a row as float32.
template <typename TI>
__device__ __forceinline__ f32x4 ld4(const TI* p) {
  if constexpr (sizeof(TI) == 2) {
    const bf16x4 v = *reinterpret_cast<const bf16x4*>(p);
    return f32x4{(float)v[0], (float)v[1], (float)v[2], (float)v[3]};
  } else {
    return *reinterpret_cast<const f32x4*>(p);
  }
}

// Per (b, h, token range) feature sums: csum[bh][c][f] = sum_{t in range c} x[t][f].
// 256 threads: D / 4 quads of features times 256 / (D / 4) row groups (rows
// t0 + group, t0 + group + groups, ...), then the groups' sums in a fixed order.
template <typename TI>
__global__ __launch_bounds__(256) void chunk_sum_kernel(const TI* __restrict__ x, float* __restrict__ csum,
                                                        int64_t N, int D, int64_t clen, int nch) {
  __shared__ f32x4 red[256];
  const int c = blockIdx.x, bh = blockIdx.y;
  const int nq = D / 4, ng = 256 / nq, fq = threadIdx.x % nq, rg = threadIdx.x / nq;
  const int64_t t0 = (int64_t)c * clen, t1 = N < t0 + clen ? N : t0 + clen;
  const TI* p = x + (size_t)bh * N * D + 4 * fq;
  f32x4 s = zero4();
  for (int64_t t = t0 + rg; t < t1; t += ng) s += ld4(p + (size_t)t * D);
  red[threadIdx.x] = s;
  __syncthreads();
  if (rg == 0) {
    for (int r = 1; r < ng; ++r) s += red[r * nq + fq];
    *reinterpret_cast<f32x4*>(csum + ((size_t)bh * nch + c) * D + 4 * fq) = s;
  }
}

// Inclusive prefix (rev = 0) or suffix (rev = 1) sums over tokens of x, per
// feature: the ranges before (after) this one from csum, then a running sum
// over the range, eight rows of loads ahead. 64 threads: 64 / (D / 4) ranges
// of D / 4 feature quads each.
template <typename TI>
__global__ __launch_bounds__(64) void scan_apply_kernel(const TI* __restrict__ x, const float* __restrict__ csum,
                                                        float* __restrict__ y, int64_t N, int D, int64_t clen,
                                                        int nch, int rev) {
  const int nq = D / 4, fq = threadIdx.x % nq;
  const int c = blockIdx.x * (64 / nq) + threadIdx.x / nq, bh = blockIdx.y;
  if (c >= nch) return;
  f32x4 off = zero4();
  const float* cs = csum + (size_t)bh * nch * D + 4 * fq;
  if (!rev) {
    for (int cc = 0; cc < c; ++cc) off += *reinterpret_cast<const f32x4*>(cs + (size_t)cc * D);
  } else {
    for (int cc = nch - 1; cc > c; --cc) off += *reinterpret_cast<const f32x4*>(cs + (size_t)cc * D);
  }
  const int64_t t0 = (int64_t)c * clen, t1 = N < t0 + clen ? N : t0 + clen;
  const TI* p = x + (size_t)bh * N * D + 4 * fq;
  float* o = y + (size_t)bh * N * D + 4 * fq;
  constexpr int U = 8;
  for (int64_t i = 0; i < t1 - t0; i += U) {
    f32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t t = rev ? t1 - 1 - (i + u) : t0 + i + u;
      v[u] = i + u < t1 - t0 ? ld4(p + (size_t)t * D) : zero4();
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (i + u < t1 - t0) {
        const int64_t t = rev ? t1 - 1 - (i + u) : t0 + i + u;
        off += v[u];
        *reinterpret_cast<f32x4*>(o + (size_t)t * D) = off;
      }
    }
  }
}

// Sum over the 64 lanes of a wave.
__device__ __forceinline__ float wsum(float x) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  return x;
}

// Per token (one wave): lambda, s = Sigma q and q_clean (q and M q in the
// input dtype; q_clean in float32, or in bf16 where only its rounded value is
// used).
template <int D, typename TM, typename TC>
__global__ __launch_bounds__(256) void pre_kernel(const TM* __restrict__ q, const float* __restrict__ m,
                                                  const TM* __restrict__ mq, const float* __restrict__ w,
                                                  const float* __restrict__ b, float* __restrict__ s,
                                                  TC* __restrict__ qc, float* __restrict__ lam, int64_t N, int H,
                                                  int64_t rows) {
  constexpr int PL = (D + 63) / 64;
  const int64_t r = (int64_t)blockIdx.x * 4 + wave_id();
  if (r >= rows) return;
  const int l = lane_id();
  const int64_t bh = r / N, tok = r - bh * N;
  const int h = (int)(bh % H);
  const float t = (float)(tok + 1);
  float qv[PL], mv[PL], wv[PL];
  float wq = 0.f, mqd = 0.f;
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int f = l + 64 * i;
    const bool ok = f < D;
    qv[i] = ok ? to_f32(q[(size_t)r * D + f]) : 0.f;
    mv[i] = ok ? m[(size_t)r * D + f] : 0.f;
    wv[i] = ok ? w[(size_t)h * D + f] : 0.f;
    wq += wv[i] * qv[i];
    mqd += mv[i] * qv[i];
  }
  wq = wsum(wq);
  mqd = wsum(mqd);
  const float la = 1.f / (1.f + expf(-(wq + b[h])));
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int f = l + 64 * i;
    if (f < D) {
      const float sv = (to_f32(mq[(size_t)r * D + f]) - mv[i] * mqd / t) / t;
      s[(size_t)r * D + f] = sv;
      qc[(size_t)r * D + f] = from_f32<TC>(qv[i] - la * sv);
    }
  }
  if (l == 0) lam[r] = la;
}

// Per token (one wave, a block of four waves over `blen` tokens of one (b, h)):
// dq, the values of the two reversed passes, dm, and this block's partial sums
// of dw and db, part[h][b * nblk + block][0 .. D) = dw, [D] = db. float32
// inputs: M u and the values in float32, in time order. bf16 inputs: M u in
// bf16, and the values and u written in bf16 at the time-reversed positions
// (the operands of the reversed passes; ru receives u).
template <typename T, int D, typename TU>
__global__ __launch_bounds__(256) void post_kernel(const T* __restrict__ q, const float* __restrict__ m,
                                                   const float* __restrict__ s, const TU* __restrict__ u,
                                                   const T* __restrict__ mu, const float* __restrict__ lam,
                                                   const float* __restrict__ w, T* __restrict__ dq,
                                                   T* __restrict__ vr1, T* __restrict__ vr2, T* __restrict__ ru,
                                                   float* __restrict__ dm, float* __restrict__ part, int64_t N, int B,
                                                   int H, int64_t blen, int nblk) {
  constexpr int PL = (D + 63) / 64;
  __shared__ float sp[4][D + 1];
  const int l = lane_id(), wv_ = wave_id();
  const int bh = blockIdx.y, b = bh / H, h = bh % H;
  float pw[PL], pb = 0.f, wl[PL];
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    pw[i] = 0.f;
    const int f = l + 64 * i;
    wl[i] = f < D ? w[(size_t)h * D + f] : 0.f;
  }
  const int64_t t_begin = (int64_t)blockIdx.x * blen;
  const int64_t t_end = N < t_begin + blen ? N : t_begin + blen;
  for (int64_t tok = t_begin + wv_; tok < t_end; tok += 4) {
    const size_t r = (size_t)bh * N + tok;
    const float t = (float)(tok + 1);
    float qv[PL], mv[PL], uv[PL];
    float a = 0.f, um = 0.f, qm = 0.f;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int f = l + 64 * i;
      const bool ok = f < D;
      qv[i] = ok ? to_f32(q[r * D + f]) : 0.f;
      mv[i] = ok ? m[r * D + f] : 0.f;
      uv[i] = ok ? to_f32(u[r * D + f]) : 0.f;
      const float sv = ok ? s[r * D + f] : 0.f;
      a += uv[i] * sv;
      um += uv[i] * mv[i];
      qm += qv[i] * mv[i];
    }
    a = wsum(a);
    um = wsum(um);
    qm = wsum(qm);
    const float la = lam[r];
    const float lp = la * (1.f - la);
    const float c1 = la / t;
#pragma unroll
    for (int i = 0; i < PL; ++i) {
      const int f = l + 64 * i;
      if (f < D) {
        const float su = (to_f32(mu[r * D + f]) - mv[i] * um / t) / t;  // Sigma u
        dq[r * D + f] = from_f32<T>(uv[i] - la * su - a * lp * wl[i]);
        if constexpr (sizeof(T) == 2) {
          const size_t rr = ((size_t)bh * N + (N - 1 - tok)) * D + f;
          vr1[rr] = from_f32<T>(c1 * uv[i]);
          vr2[rr] = from_f32<T>(c1 * qv[i]);
          ru[rr] = from_f32<T>(uv[i]);
        } else {
          vr1[r * D + f] = c1 * uv[i];
          vr2[r * D + f] = c1 * qv[i];
        }
        dm[r * D + f] = c1 / t * (uv[i] * qm + qv[i] * um);
      }
      pw[i] -= a * lp * qv[i];
    }
    pb -= a * lp;
  }
#pragma unroll
  for (int i = 0; i < PL; ++i) {
    const int f = l + 64 * i;
    if (f < D) sp[wv_][f] = pw[i];
  }
  if (l == 0) sp[wv_][D] = pb;
  __syncthreads();
  float* dst = part + ((size_t)h * B * nblk + (size_t)b * nblk + blockIdx.x) * (D + 1);
  for (int f = threadIdx.x; f <= D; f += 256) dst[f] = sp[0][f] + sp[1][f] + sp[2][f] + sp[3][f];
}

// dk = (direct part) - R1 - R2 + suffix(dm); R1 and R2 come time-reversed. The
// direct part is float32, or bf16 where the fused kernel produced it.
template <typename T, typename TD>
__global__ __launch_bounds__(256) void dk_kernel(const TD* __restrict__ dkg, const T* __restrict__ r1,
                                                 const T* __restrict__ r2, const float* __restrict__ sdm,
                                                 T* __restrict__ dk, int64_t N, int D, int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t row = i / D;
  const int f = (int)(i - row * D);
  const int64_t bh = row / N, t = row - bh * N;
  const size_t rr = ((size_t)bh * N + (N - 1 - t)) * D + f;
  dk[i] = from_f32<T>(to_f32(dkg[i]) - to_f32(r1[rr]) - to_f32(r2[rr]) + sdm[i]);
}

// dw, db per head: the block partials summed over (b, block) in a fixed order.
__global__ __launch_bounds__(256) void param_kernel(const float* __restrict__ part, float* __restrict__ dw,
                                                    float* __restrict__ db, int D, int nslot) {
  const int h = blockIdx.x;
  for (int f = threadIdx.x; f <= D; f += 256) {
    float s = 0.f;
    for (int sl = 0; sl < nslot; ++sl) s += part[((size_t)h * nslot + sl) * (D + 1) + f];
    if (f < D)
      dw[(size_t)h * D + f] = s;
    else
      db[h] = s;
  }
}

__global__ __launch_bounds__(256) void fill_kernel(float* __restrict__ p, float x, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i < n) p[i] = x;
}

// Element-wise conversion, four elements per thread (n a multiple of 4: rows
// of 32, 64 or 128 entries).
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void cvt_kernel(const TI* __restrict__ in, TO* __restrict__ out, int64_t n) {
  const int64_t i = ((int64_t)blockIdx.x * 256 + threadIdx.x) * 4;
  if (i >= n) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[i + j] = from_f32<TO>(to_f32(in[i + j]));
}

static unsigned nblocks(int64_t n) { return (unsigned)((n + 255) / 256); }

// Causal linear attention without decay: out = LA(q, k, v), on the float32 or
// the bf16 chunk kernel.
template <typename T>
static hipError_t la(const CcqBwdLaunch& L, const T* q, const T* k, const T* v, T* out, hipStream_t st) {
  LinLaunch F = L.bwd.fwd;
  F.q = q;
  F.k = k;
  F.v = v;
  F.g = L.ones;
  F.out = out;
  F.bf16 = sizeof(T) == 2;
  F.ccq = false;
  F.state_in = nullptr;
  F.state_out = nullptr;
  F.t_in = 0;
  return linattn_launch(F, st);
}

template <typename TI>
static hipError_t scan(const CcqBwdLaunch& L, const TI* x, float* y, int rev, hipStream_t st) {
  const unsigned BH = (unsigned)(L.B * L.H), per = (unsigned)(64 / (L.D / 4));
  hipLaunchKernelGGL((chunk_sum_kernel<TI>), dim3((unsigned)L.nch, BH), dim3(256), 0, st, x, L.csum, L.N, (int)L.D,
                     L.clen, (int)L.nch);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((scan_apply_kernel<TI>), dim3(((unsigned)L.nch + per - 1) / per, BH), dim3(64), 0, st, x, L.csum,
                     y, L.N, (int)L.D, L.clen, (int)L.nch, rev);
  return hipGetLastError();
}

template <typename T, int D>
static hipError_t run(const CcqBwdLaunch& L, hipStream_t st) {
  const int64_t BH = L.B * L.H, rows = BH * L.N, n = rows * D;
  const int H = (int)L.H;
  hipError_t e;
  const float *fq, *fk, *fv, *fdo;
  if constexpr (sizeof(T) == 2) {
    if (!(D == 128 && L.fused)) {
      // k, v and dout in float32 serve only the chunk passes of the decayed read
      hipLaunchKernelGGL((cvt_kernel<T, float>), dim3(nblocks(n / 4)), dim3(256), 0, st, static_cast<const T*>(L.k),
                         L.fk, n);
      hipLaunchKernelGGL((cvt_kernel<T, float>), dim3(nblocks(n / 4)), dim3(256), 0, st, static_cast<const T*>(L.v),
                         L.fv, n);
      hipLaunchKernelGGL((cvt_kernel<T, float>), dim3(nblocks(n / 4)), dim3(256), 0, st,
                         static_cast<const T*>(L.dout), L.fdo, n);
    }
    if ((e = hipGetLastError()) != hipSuccess) return e;
    fq = nullptr;  // q is read in bf16
    fk = L.fk;
    fv = L.fv;
    fdo = L.fdo;
  } else {
    fq = static_cast<const float*>(L.q);
    fk = static_cast<const float*>(L.k);
    fv = static_cast<const float*>(L.v);
    fdo = static_cast<const float*>(L.dout);
  }
  hipLaunchKernelGGL(fill_kernel, dim3(nblocks(rows)), dim3(256), 0, st, L.ones, 1.f, rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // forward quantities: m = prefix sum of k, Mq, then lambda, s = Sigma q, q_clean.
  // For bf16 inputs the undecayed passes (M q, M u and the two reversed ones)
  // run on the bf16 chunk kernel: their results enter q_clean, dq and dk as
  // perturbations of the size of the bf16 rounding, while the gradients of the
  // decayed read (with the gate gradient's cancellation) stay in float32.
  if ((e = scan<T>(L, static_cast<const T*>(L.k), L.m, 0, st)) != hipSuccess) return e;
  T* mq16 = reinterpret_cast<T*>(L.mq);  // the M q result in the input dtype
  if constexpr (sizeof(T) == 2) {
    if ((e = la<T>(L, static_cast<const T*>(L.q), static_cast<const T*>(L.k), static_cast<const T*>(L.k), mq16,
                   st)) != hipSuccess)
      return e;
  } else {
    if ((e = la<float>(L, fq, fk, fk, L.mq, st)) != hipSuccess) return e;
  }
  bool fused = false;
  if constexpr (sizeof(T) == 2 && D == 128) fused = L.fused;
  // the fused route takes q_clean rounded once to bf16 (as the forward's read
  // takes it), written straight into a free slot
  bf16* qc16 = reinterpret_cast<bf16*>(L.dvg);
  const dim3 pgrid((unsigned)((rows + 3) / 4));
  if (fused)
    hipLaunchKernelGGL((pre_kernel<D, T, bf16>), pgrid, dim3(256), 0, st, static_cast<const T*>(L.q), L.m, mq16, L.w,
                       L.b, L.s, qc16, L.lam, L.N, H, rows);
  else
    hipLaunchKernelGGL((pre_kernel<D, T, float>), pgrid, dim3(256), 0, st, static_cast<const T*>(L.q), L.m, mq16, L.w,
                       L.b, L.s, L.qc, L.lam, L.N, H, rows);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // backward of the decayed linear attention read with q_clean: u = dq_clean,
  // the direct part of dk, dv and dg
  T* mu16 = reinterpret_cast<T*>(L.mu);
  T* u16 = sizeof(T) == 2 ? mu16 + n : nullptr;  // bf16: second half of the M u slot
  if (fused) {
    // the fused bf16 kernel: dq lands in the bf16 u operand of the M u pass
    // (read as u by the later steps too), dk in the direct-dk slot (read in
    // bf16), k . dk per token and the slice sums of the gate gradient in dm
    bf16* dk16 = reinterpret_cast<bf16*>(L.dkg);
    BwdBf16Launch F{};
    F.q = qc16;
    F.k = L.k;
    F.v = L.v;
    F.g = L.bwd.g;
    F.dout = L.dout;
    F.dq = u16;
    F.dk = dk16;
    F.dv = L.dv;
    F.dg = L.bwd.dg;
    F.xk = L.dm;
    F.tot = L.dm + BH * L.N;  // the dm rows hold D floats per token
    F.B = L.B;
    F.H = L.H;
    F.N = L.N;
    if ((e = linattn_backward_bf16_launch(F, st)) != hipSuccess) return e;
  } else if constexpr (sizeof(T) == 2) {
    // dv (which dg does not use) on bf16 operands: reversed k, q_clean and
    // dout in the slots of the float32 dv and of the inner reversed k
    bf16* a16 = reinterpret_cast<bf16*>(L.dvg);
    bf16* b16 = reinterpret_cast<bf16*>(L.bwd.rk);
    if ((e = reverse_to_bf16<bf16>(static_cast<const bf16*>(L.k), a16, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = reverse_to_bf16<float>(L.qc, a16 + n, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = reverse_to_bf16<bf16>(static_cast<const bf16*>(L.dout), b16, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = linattn_backward_mixed(L.bwd, L.qc, fk, fv, fdo, L.u, L.dkg, true, a16, a16 + n, b16, b16 + n,
                                    static_cast<bf16*>(L.dv), st)) != hipSuccess)
      return e;
  } else {
    if ((e = linattn_backward_f32(L.bwd, L.qc, fk, fv, fdo, L.u, L.dkg, static_cast<float*>(L.dv), true, st)) !=
        hipSuccess)
      return e;
  }
  // Sigma u needs M u; then dq, the values of the reversed passes, dm, dw/db
  T* vr1 = reinterpret_cast<T*>(L.vr1);
  T* vr2 = reinterpret_cast<T*>(L.vr2);
  T* ru16 = sizeof(T) == 2 ? reinterpret_cast<T*>(L.vr1) + n : nullptr;  // bf16: second half of the vr1 slot
  if constexpr (sizeof(T) == 2) {
    if (!fused) {
      hipLaunchKernelGGL((cvt_kernel<float, T>), dim3(nblocks(n / 4)), dim3(256), 0, st, L.u, u16, n);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    if ((e = la<T>(L, u16, static_cast<const T*>(L.k), static_cast<const T*>(L.k), mu16, st)) != hipSuccess)
      return e;
  } else {
    if ((e = la<float>(L, L.u, fk, fk, L.mu, st)) != hipSuccess) return e;
  }
  if (fused)
    hipLaunchKernelGGL((post_kernel<T, D, bf16>), dim3((unsigned)L.nblk, (unsigned)BH), dim3(256), 0, st,
                       static_cast<const T*>(L.q), L.m, L.s, reinterpret_cast<const bf16*>(u16), mu16, L.lam, L.w,
                       static_cast<T*>(L.dq), vr1, vr2, ru16, L.dm, L.part, L.N, (int)L.B, H, L.blen, (int)L.nblk);
  else
    hipLaunchKernelGGL((post_kernel<T, D, float>), dim3((unsigned)L.nblk, (unsigned)BH), dim3(256), 0, st,
                       static_cast<const T*>(L.q), L.m, L.s, L.u, mu16, L.lam, L.w, static_cast<T*>(L.dq), vr1, vr2,
                       ru16, L.dm, L.part, L.N, (int)L.B, H, L.blen, (int)L.nblk);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // sum_{t>=j} (lambda_t/t) u_t (q_t . k_j) and (lambda_t/t) q_t (u_t . k_j): causal
  // passes over the reversed sequence (query rev k, keys rev q / rev u)
  T* r1 = reinterpret_cast<T*>(L.r1);
  T* r2 = reinterpret_cast<T*>(L.r2);
  if constexpr (sizeof(T) == 2) {
    T* rk16 = reinterpret_cast<T*>(L.bwd.rk);
    T* rq16 = rk16 + n;
    if ((e = reverse_to_bf16<bf16>(static_cast<const bf16*>(L.k), rk16, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = reverse_to_bf16<bf16>(static_cast<const bf16*>(L.q), rq16, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = la<T>(L, rk16, rq16, vr1, r1, st)) != hipSuccess) return e;
    if ((e = la<T>(L, rk16, ru16, vr2, r2, st)) != hipSuccess) return e;
  } else {
    if ((e = reverse_rows_f32(fk, L.bwd.rk, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = reverse_rows_f32(fq, L.bwd.rq, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = reverse_rows_f32(L.u, L.bwd.rv, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = reverse_rows_f32(L.vr1, L.bwd.rdo, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = reverse_rows_f32(L.vr2, L.bwd.rout, BH, L.N, D, st)) != hipSuccess) return e;
    if ((e = la<float>(L, L.bwd.rk, L.bwd.rq, L.bwd.rdo, L.r1, st)) != hipSuccess) return e;
    if ((e = la<float>(L, L.bwd.rk, L.bwd.rv, L.bwd.rout, L.r2, st)) != hipSuccess) return e;
  }
  if ((e = scan<float>(L, L.dm, L.sdm, 1, st)) != hipSuccess) return e;
  if (fused)
    hipLaunchKernelGGL((dk_kernel<T, bf16>), dim3(nblocks(n)), dim3(256), 0, st, reinterpret_cast<const bf16*>(L.dkg),
                       r1, r2, L.sdm, static_cast<T*>(L.dk), L.N, D, n);
  else
    hipLaunchKernelGGL((dk_kernel<T, float>), dim3(nblocks(n)), dim3(256), 0, st, L.dkg, r1, r2, L.sdm,
                       static_cast<T*>(L.dk), L.N, D, n);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  hipLaunchKernelGGL(param_kernel, dim3((unsigned)H), dim3(256), 0, st, L.part, L.dw, L.db, D,
                     (int)(L.B * L.nblk));
  return hipGetLastError();
}

}  // namespace cbwd

hipError_t ccq_backward_launch(const CcqBwdLaunch& L, hipStream_t st) {
  using namespace cbwd;
  switch (L.D) {
    case 32: return L.bf16 ? run<bf16, 32>(L, st) : run<float, 32>(L, st);
    case 64: return L.bf16 ? run<bf16, 64>(L, st) : run<float, 64>(L, st);
    case 128: return L.bf16 ? run<bf16, 128>(L, st) : run<float, 128>(L, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lm
