// linattn_c32.hip -- the chunkwise forwards of decayed linear attention and of
// the curvature-conditioned-query (CCQ) read with chunks of 32 tokens.
//
// Method: the same chunk algebra as the 64-token kernels (allinfo.ai.kr linear
// attention post, "Key messages" and "Easy explanation": S_t = g_t S_{t-1} +
// k_t v_t^T, o_t = S_t^T q'_t; "Don't Read Everything: A Curvature-Conditioned
// Query for Linear Attention", section 2 Method: q' = q - lambda Sigma_t q).
// Row i of a chunk, l the inclusive cumulative log2 gate inside the chunk:
//   o_i = 2^(l_i) S_prev^T q'_i + sum_{j<=i} 2^(l_i - l_j) (q'_i . k_j) v_j
//   S_next = 2^(l_last) S_prev + sum_j 2^(l_last - l_j) k_j v_j^T
// and for CCQ, with M, m the running sums of k k^T and k, P_ij = q_i . k_j,
// t the global count of token i, alpha = lambda / t,
// beta = lambda (m_prev . q_i + sum_{j<=i} P_ij) / t^2:
//   q'_i = q_i - alpha M_prev q_i + sum_{j<=i} k_j (beta - alpha P_ij) + beta m_prev.
//
// The chunk length only changes how the work is cut (how many token pairs go
// through the intra-chunk product and how many through the state), not the
// result. This kernel keeps the 32-token schedule in plain float32 arithmetic:
// one workgroup of 256 threads per (b, h) walks the sequence; thread (column
// b, part p) holds rows [p R, (p + 1) R) of column b of S (and of the
// symmetric M) in registers, R = D^2 / 256; the chunk's tiles, scores and the
// per-part partial sums of the state products sit in LDS. It serves chunk = 32
// calls; the tuned matrix-core kernels run chunk = 64.
#include "launch.hpp"
#include "mfma.hpp"

namespace lm {
namespace c32 {

constexpr int kC = 32;
constexpr int kNT = 256;
constexpr float kMinLog2G = -200.f;

template <int D>
struct Lay {
  static constexpr int TPC = kNT / D;  // threads (parts) per state column
  static constexpr int R = D / TPC;    // state rows per thread
  static constexpr int PD = D + 1;     // tile pitch (floats)
  static constexpr int PS = kC + 1;    // score pitch
  static constexpr int oQ = 0, oK = oQ + kC * PD, oV = oK + kC * PD, oQc = oV + kC * PD;
  static constexpr int oPart = oQc + kC * PD;          // [TPC][32][D]
  static constexpr int oA = oPart + TPC * kC * D;      // decayed scores [32][PS]
  static constexpr int oP = oA + kC * PS;              // raw scores (CCQ) [32][PS]
  static constexpr int oMq = oP + kC * PS;             // M_prev q [32][D]
  static constexpr int oL = oMq + kC * D;              // l [32]
  static constexpr int oAl = oL + kC;                  // alpha [32]
  static constexpr int oBe = oAl + kC;                 // beta [32]
  static constexpr int oWq = oBe + kC;                 // w . q [32]
  static constexpr int oMd = oWq + kC;                 // m_prev . q [32]
  static constexpr int om = oMd + kC;                  // m [D]
  static constexpr int total = om + D;
  static_assert(total * 4 <= 160 * 1024, "LDS budget");
};

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* wl;  // [H][D] (CCQ)
  const float* bl;  // [H] (CCQ)
  void* out;
  const float* state_in;  // optional [S | M | m] per (b, h)
  float* state_out;       // optional
  int64_t N, t_in;
  int H;
};

template <typename T, int D, bool CCQ>
__global__ __launch_bounds__(kNT) void c32_kernel(Args a) {
  typedef Lay<D> Ly;
  constexpr int TPC = Ly::TPC, R = Ly::R, PD = Ly::PD, PS = Ly::PS;
  extern __shared__ float sm_[];
  float* sQ = sm_ + Ly::oQ;
  float* sK = sm_ + Ly::oK;
  float* sV = sm_ + Ly::oV;
  float* sQc = sm_ + Ly::oQc;
  float* sPart = sm_ + Ly::oPart;
  float* sA = sm_ + Ly::oA;
  float* sP = sm_ + Ly::oP;
  float* sMq = sm_ + Ly::oMq;
  float* sL = sm_ + Ly::oL;
  float* sAl = sm_ + Ly::oAl;
  float* sBe = sm_ + Ly::oBe;
  float* sWq = sm_ + Ly::oWq;
  float* sMd = sm_ + Ly::oMd;
  float* sm = sm_ + Ly::om;
  const int tid = threadIdx.x, bh = blockIdx.x, h = bh % a.H;
  const int b = tid % D, p = tid / D, a0 = p * R;
  const int64_t N = a.N;
  const T* Q = static_cast<const T*>(a.q) + (size_t)bh * N * D;
  const T* K = static_cast<const T*>(a.k) + (size_t)bh * N * D;
  const T* V = static_cast<const T*>(a.v) + (size_t)bh * N * D;
  const float* G = a.g + (size_t)bh * N;
  T* O = static_cast<T*>(a.out) + (size_t)bh * N * D;
  constexpr size_t sfl = (size_t)D * D + (CCQ ? (size_t)D * D + D : 0);

  // state: S[a0 + r][b], M[a0 + r][b], m in LDS
  float S[R], M[CCQ ? R : 1];
  {
    const float* si = a.state_in ? a.state_in + (size_t)bh * sfl : nullptr;
#pragma unroll
    for (int r = 0; r < R; ++r) S[r] = si ? si[(size_t)(a0 + r) * D + b] : 0.f;
    if constexpr (CCQ) {
#pragma unroll
      for (int r = 0; r < R; ++r) M[r] = si ? si[(size_t)D * D + (size_t)(a0 + r) * D + b] : 0.f;
      if (p == 0) sm[b] = si ? si[2 * (size_t)D * D + b] : 0.f;
    }
  }
  const float bias = CCQ ? a.bl[h] : 0.f;
  const float* wl = CCQ ? a.wl + (size_t)h * D : nullptr;

  for (int64_t t0 = 0; t0 < N; t0 += kC) {
    const int nv = (int)(N - t0 < kC ? N - t0 : kC);
    for (int e = tid; e < kC * D; e += kNT) {
      const int i = e / D, c = e - (e / D) * D;
      const bool ok = i < nv;
      const size_t o = (size_t)(t0 + i) * D + c;
      sQ[i * PD + c] = ok ? to_f32(Q[o]) : 0.f;
      sK[i * PD + c] = ok ? to_f32(K[o]) : 0.f;
      sV[i * PD + c] = ok ? to_f32(V[o]) : 0.f;
    }
    if (tid < 64) {
      const float x = tid < nv ? fmaxf(__builtin_amdgcn_logf(G[t0 + tid]), kMinLog2G) : 0.f;
      const float lc = wave_scan_incl(x);
      if (tid < kC) sL[tid] = lc;
    }
    __syncthreads();

    const float* Qr = sQ;  // the queries the read uses
    if constexpr (CCQ) {
      // raw scores P_ij (j <= i), 4 pairs per thread
      {
        const int i = tid / 8;
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int j = tid % 8 + 8 * u;
          float s = 0.f;
          if (j <= i)
            for (int c = 0; c < D; ++c) s += sQ[i * PD + c] * sK[j * PD + c];
          sP[i * PS + j] = s;
        }
      }
      // gate logit and mean term per query
      if (tid < 2 * kC) {
        const int i = tid % kC;
        float s = 0.f;
        if (tid < kC)
          for (int c = 0; c < D; ++c) s += wl[c] * sQ[i * PD + c];
        else
          for (int c = 0; c < D; ++c) s += sm[c] * sQ[i * PD + c];
        (tid < kC ? sWq : sMd)[i] = s;
      }
      // partials of M_prev q: column b, rows of this part (M is symmetric)
      for (int i = 0; i < kC; ++i) {
        float s = 0.f;
#pragma unroll
        for (int r = 0; r < R; ++r) s += M[r] * sQ[i * PD + a0 + r];
        sPart[(p * kC + i) * D + b] = s;
      }
      __syncthreads();
      if (tid < kC) {
        const int i = tid;
        float rs = 0.f;
        for (int j = 0; j <= i; ++j) rs += sP[i * PS + j];
        const float t = (float)(a.t_in + t0 + i + 1);
        const float lam = 1.f / (1.f + expf(-(sWq[i] + bias)));
        sAl[i] = lam / t;
        sBe[i] = lam * (sMd[i] + rs) / (t * t);
      }
      for (int i = p; i < kC; i += TPC) {
        float mq = 0.f;
        for (int u = 0; u < TPC; ++u) mq += sPart[(u * kC + i) * D + b];
        sMq[i * D + b] = mq;
      }
      __syncthreads();
      // cleaned queries: column b of the rows i = p, p + TPC, ...
      for (int i = p; i < kC; i += TPC) {
        const float al = sAl[i], be = sBe[i];
        float d = -al * sMq[i * D + b] + be * sm[b];
        for (int j = 0; j <= i; ++j) d += sK[j * PD + b] * (be - al * sP[i * PS + j]);
        sQc[i * PD + b] = sQ[i * PD + b] + d;
      }
      __syncthreads();
      Qr = sQc;
    }

    // decayed scores A_ij = 2^(l_i - l_j) (q'_i . k_j), j <= i
    {
      const int i = tid / 8;
      const float li = sL[i];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int j = tid % 8 + 8 * u;
        float s = 0.f;
        if (j <= i) {
          for (int c = 0; c < D; ++c) s += Qr[i * PD + c] * sK[j * PD + c];
          s *= exp2f(li - sL[j]);
        }
        sA[i * PS + j] = s;
      }
    }
    // partials of S_prev^T q': column b, rows of this part
    for (int i = 0; i < kC; ++i) {
      float s = 0.f;
#pragma unroll
      for (int r = 0; r < R; ++r) s += S[r] * Qr[i * PD + a0 + r];
      sPart[(p * kC + i) * D + b] = s;
    }
    __syncthreads();
    // outputs: column b of the rows i = p, p + TPC, ...
    for (int i = p; i < nv; i += TPC) {
      float inter = 0.f;
      for (int u = 0; u < TPC; ++u) inter += sPart[(u * kC + i) * D + b];
      float o = exp2f(sL[i]) * inter;
      for (int j = 0; j <= i; ++j) o += sA[i * PS + j] * sV[j * PD + b];
      O[(size_t)(t0 + i) * D + b] = from_f32<T>(o);
    }
    // state update
    const float Lc = sL[kC - 1];
    const float fL = exp2f(Lc);
#pragma unroll
    for (int r = 0; r < R; ++r) S[r] *= fL;
    for (int j = 0; j < kC; ++j) {
      const float wv = exp2f(Lc - sL[j]) * sV[j * PD + b];
      const float kb = sK[j * PD + b];
#pragma unroll
      for (int r = 0; r < R; ++r) {
        const float ka = sK[j * PD + a0 + r];
        S[r] += ka * wv;
        if constexpr (CCQ) M[r] += ka * kb;
      }
    }
    if constexpr (CCQ) {
      if (p == 0) {
        float s = 0.f;
        for (int j = 0; j < kC; ++j) s += sK[j * PD + b];
        sm[b] += s;
      }
    }
    __syncthreads();
  }

  if (a.state_out) {
    float* so = a.state_out + (size_t)bh * sfl;
#pragma unroll
    for (int r = 0; r < R; ++r) so[(size_t)(a0 + r) * D + b] = S[r];
    if constexpr (CCQ) {
#pragma unroll
      for (int r = 0; r < R; ++r) so[(size_t)D * D + (size_t)(a0 + r) * D + b] = M[r];
      if (p == 0) so[2 * (size_t)D * D + b] = sm[b];
    }
  }
}

template <typename T, int D, bool CCQ>
static hipError_t launch(const LinLaunch& L, hipStream_t st) {
  Args a;
  a.q = L.q;
  a.k = L.k;
  a.v = L.v;
  a.g = L.g;
  a.wl = L.w_lambda;
  a.bl = L.b_lambda;
  a.out = L.out;
  a.state_in = L.state_in;
  a.state_out = L.state_out;
  a.N = L.N;
  a.t_in = L.t_in;
  a.H = (int)L.H;
  const size_t lds = Lay<D>::total * 4;
  auto kern = c32_kernel<T, D, CCQ>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3((unsigned)(L.B * L.H)), dim3(kNT), lds, st, a);
  return hipGetLastError();
}

template <typename T, bool CCQ>
static hipError_t by_width(const LinLaunch& L, hipStream_t st) {
  switch (L.D) {
    case 32: return launch<T, 32, CCQ>(L, st);
    case 64: return launch<T, 64, CCQ>(L, st);
    case 128: return launch<T, 128, CCQ>(L, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace c32

hipError_t linattn_c32_launch(const LinLaunch& L, hipStream_t st) {
  if (L.bf16) return L.ccq ? c32::by_width<bf16, true>(L, st) : c32::by_width<bf16, false>(L, st);
  return L.ccq ? c32::by_width<float, true>(L, st) : c32::by_width<float, false>(L, st);
}

}  // namespace lm
