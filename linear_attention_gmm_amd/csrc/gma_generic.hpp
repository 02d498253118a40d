// gma_generic.hpp -- the general GMA kernel (fp32 inputs, and bf16 shapes the
// bf16 kernel does not cover) and its launcher. Included by gma.hip, and by
// gma_wide.hip for the bf16 d = 128, 256-component instantiation, which is
// compiled with different code generation options.
#pragma once
#include "mfma.hpp"
#include "gma.hpp"

namespace lm {
namespace gma {

constexpr int kLdsBudget = 160 * 1024;

// ---------------------------------------------------------------------------
// Generic kernel (float32 inputs, and bf16 shapes outside the bf16 kernel).

template <typename T, int D, int DV, int NW, int KPW, int MODE>
struct Cfg {
  static constexpr int KS = Mma<T>::KS;
  static constexpr int RT = KPW / 16;     // component tiles per wave
  static constexpr int NKX = D / KS;      // k-steps over x features
  static constexpr int NKC = KPW / KS;    // k-steps over a wave's components
  static constexpr int NKT = kChunk / KS; // k-steps over a chunk's tokens
  static constexpr int DT = DV / 16;
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int W_VGPR = RT * (2 * D) * (int)sizeof(T) / 4 / 4;  // per lane
  // W fragments kept in registers when they are few; with eight waves (two per
  // SIMD, 256 VGPRs each) only up to 32 registers.
  static constexpr bool W_RES = W_VGPR <= (NW >= 8 ? 32 : 64);
  static constexpr int PV = DV + PAD;
  static constexpr int PE = KPW + PAD;
  static constexpr bool HAS_K = MODE != BIDIR;
  static constexpr bool HAS_Q = MODE != AGG;
  static constexpr int NXT = (HAS_K ? 1 : 0) + (HAS_Q ? 1 : 0);
  static constexpr int v_bytes = HAS_K ? kChunk * PV * (int)sizeof(T) : 0;
  static constexpr int e_bytes = HAS_K ? NW * kChunk * PE * (int)sizeof(T) : 0;
  static constexpr int st_bytes = (HAS_K && NW > 1) ? NW * kChunk * 8 : 0;
  static constexpr int rq_bytes = HAS_Q ? NW * kChunk * 16 : 0;
  static constexpr int x_bytes(bool sq) { return NXT * kChunk * ((sq ? 2 * D : D) + PAD) * (int)sizeof(T); }
  static constexpr int r_bytes(int dvb) { return HAS_Q ? NW * kChunk * (dvb + 4) * 4 : 0; }
  static constexpr int total(bool sq, int dvb) {
    return (x_bytes(sq) > r_bytes(dvb) ? x_bytes(sq) : r_bytes(dvb)) + v_bytes + e_bytes + st_bytes +
           rq_bytes;
  }
  // x*x features stored in LDS next to x when they fit, else squared on the fly.
  static constexpr bool SQ = total(true, DV <= 64 ? DV : 64) <= kLdsBudget;
  static constexpr int pick_dvb() {
    int b = DV;
    while (b > 16 && total(SQ, b) > kLdsBudget) b /= 2;
    return b;
  }
  static constexpr int DVB = pick_dvb();
  static constexpr int NDB = DV / DVB;
  static constexpr int DTB = DVB / 16;
  static constexpr int PX = (SQ ? 2 * D : D) + PAD;
  static constexpr int PR = DVB + 4;
  // byte offsets
  static constexpr int o_x = 0;  // X tiles (K first, then Q); aliased by R
  static constexpr int o_r = 0;
  static constexpr int xr_bytes = x_bytes(SQ) > r_bytes(DVB) ? x_bytes(SQ) : r_bytes(DVB);
  static constexpr int o_v = xr_bytes;
  static constexpr int o_e = o_v + v_bytes;
  static constexpr int o_st = o_e + e_bytes;
  static constexpr int o_rq = o_st + st_bytes;
  static constexpr int lds = o_rq + rq_bytes;
  static_assert(lds <= kLdsBudget, "LDS budget exceeded");
  static_assert(D % KS == 0 && KPW % KS == 0 && DV % 16 == 0, "shape");
};

// Loads a 64-row tile of routing vectors into LDS: x in columns [0, D) and, when
// SQ, x*x in [D, 2D) (squared in fp32, rounded once to T). Rows >= nvalid are 0.
template <typename T, int D, int NT, bool SQ>
__device__ __forceinline__ void load_x_tile(T* sx, int px, const T* __restrict__ src, int nvalid) {
  typedef typename Vec16<T>::type vec;
  constexpr int VN = Vec16<T>::n;
  constexpr int PER_ROW = D / VN;
  for (int i = threadIdx.x; i < kChunk * PER_ROW; i += NT) {
    const int row = i / PER_ROW, cv = i - (i / PER_ROW) * PER_ROW;
    vec x;
    if (row < nvalid) {
      x = *reinterpret_cast<const vec*>(src + (size_t)row * D + cv * VN);
    } else {
#pragma unroll
      for (int j = 0; j < VN; ++j) x[j] = from_f32<T>(0.f);
    }
    *reinterpret_cast<vec*>(sx + row * px + cv * VN) = x;
    if constexpr (SQ) {
      vec s;
#pragma unroll
      for (int j = 0; j < VN; ++j) {
        const float f = to_f32(x[j]);
        s[j] = from_f32<T>(f * f);
      }
      *reinterpret_cast<vec*>(sx + row * px + D + cv * VN) = s;
    }
  }
}

template <typename T, int DV, int NT>
__device__ __forceinline__ void load_v_tile(T* sv, int pv, const T* __restrict__ src, int nvalid) {
  typedef typename Vec16<T>::type vec;
  constexpr int VN = Vec16<T>::n;
  constexpr int PER_ROW = DV / VN;
  for (int i = threadIdx.x; i < kChunk * PER_ROW; i += NT) {
    const int row = i / PER_ROW, cv = i - (i / PER_ROW) * PER_ROW;
    vec x;
    if (row < nvalid) {
      x = *reinterpret_cast<const vec*>(src + (size_t)row * DV + cv * VN);
    } else {
#pragma unroll
      for (int j = 0; j < VN; ++j) x[j] = from_f32<T>(0.f);
    }
    *reinterpret_cast<vec*>(sv + row * pv + cv * VN) = x;
  }
}

// B-operand fragment of the routing features for k-step ks (NATURAL order).
// Steps [0, NKX) are x, steps [NKX, 2 NKX) are x*x (from LDS, or squared here).
template <typename T, int D, bool SQ>
__device__ __forceinline__ typename Mma<T>::frag feat_frag(const T* sx, int px, int row, int ks) {
  constexpr int NKX = D / Mma<T>::KS;
  if constexpr (SQ) {
    return ld_kc_nat(sx, px, row, ks);
  } else {
    typename Mma<T>::frag f = ld_kc_nat(sx, px, row, ks < NKX ? ks : ks - NKX);
    if (ks >= NKX) {
      if constexpr (sizeof(T) == 2) {
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float x = to_f32(f[j]);
          f[j] = from_f32<T>(x * x);
        }
      } else {
        f = f * f;
      }
    }
    return f;
  }
}

// A-operand fragment of W (component row `row` of this head), NATURAL order.
template <typename T, int D>
__device__ __forceinline__ typename Mma<T>::frag w_frag(const T* __restrict__ Wh, int row, int ks) {
  const int g = lane_id() >> 4;
  if constexpr (sizeof(T) == 2) {
    return *reinterpret_cast<const bf16x8*>(Wh + (size_t)row * 2 * D + ks * 32 + 8 * g);
  } else {
    return Wh[(size_t)row * 2 * D + ks * 4 + g];
  }
}

// Logits L^T [KPW x 64] of one wave's components for a 64-token tile.
// L[ct][rt] is the D tile of token tile ct and component tile rt.
template <typename T, typename C>
__device__ __forceinline__ void route(f32x4 (&L)[4][C::RT], const T* sx, const T* __restrict__ Wh,
                                      const typename Mma<T>::frag (&Wf)[C::W_RES ? C::RT : 1][C::W_RES ? 2 * C::NKX : 1],
                                      const float (&cb)[C::RT][4], int comp0) {
  typedef Mma<T> M;
  const int c16 = lane_id() & 15;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) L[ct][rt] = f32x4{cb[rt][0], cb[rt][1], cb[rt][2], cb[rt][3]};
#pragma unroll
  for (int ks = 0; ks < 2 * C::NKX; ++ks) {
    typename M::frag wk[C::RT];
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      if constexpr (C::W_RES)
        wk[rt] = Wf[rt][ks];
      else
        wk[rt] = w_frag<T, C::NKX * M::KS>(Wh, comp0 + 16 * rt + c16, ks);
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) {
      const typename M::frag f = feat_frag<T, C::NKX * M::KS, C::SQ>(sx, C::PX, 16 * ct + c16, ks);
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) L[ct][rt] = M::mma(wk[rt], f, L[ct][rt]);
    }
  }
}

// In-wave softmax pieces for token tile ct: returns the wave-local max m and
// replaces L by exp2(L - m); returns the local sum in s.
template <int RT>
__device__ __forceinline__ void local_softmax(f32x4 (&L)[RT], float& m, float& s) {
  float mx = -INFINITY;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = fmaxf(mx, L[rt][r]);
  mx = group_max(mx);
  if (mx == -INFINITY) mx = -3.0e38f;  // every component of this wave is padding
  float sum = 0.f;
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const float e = fast_exp2(L[rt][r] - mx);
      L[rt][r] = e;
      sum += e;
    }
  m = mx;
  s = group_sum(sum);
}

template <typename T, int D, int DV, int NW, int KPW, int MODE>
__global__ __launch_bounds__(NW * 64) void gma_kernel(Args a) {
  typedef Cfg<T, D, DV, NW, KPW, MODE> C;
  typedef Mma<T> M;
  typedef typename M::frag frag;
  constexpr int NT = NW * 64;
  constexpr int RT = C::RT;

  __shared__ __attribute__((aligned(16))) char smem[C::lds];
  T* sXk = reinterpret_cast<T*>(smem + C::o_x);
  T* sXq = reinterpret_cast<T*>(smem + C::o_x) + (C::HAS_K ? kChunk * C::PX : 0);
  T* sV = reinterpret_cast<T*>(smem + C::o_v);
  T* sE = reinterpret_cast<T*>(smem + C::o_e);
  float2* sSt = reinterpret_cast<float2*>(smem + C::o_st);
  float* sR = reinterpret_cast<float*>(smem + C::o_r);
  f32x4* sRQ = reinterpret_cast<f32x4*>(smem + C::o_rq);

  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int bh = blockIdx.y, p = blockIdx.x;
  const int h = bh % a.H;
  const int64_t N = a.N;
  const int64_t t_begin = (int64_t)p * a.seg_len;
  const int64_t t_end = N < t_begin + a.seg_len ? N : t_begin + a.seg_len;
  const T* __restrict__ Qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * N * D;
  const T* __restrict__ Kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * N * D;
  const T* __restrict__ Vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * N * DV;
  T* __restrict__ Og = reinterpret_cast<T*>(a.out) + (size_t)bh * N * DV;
  const T* __restrict__ Wh = reinterpret_cast<const T*>(a.W) + (size_t)h * a.KP * 2 * D;
  const float* __restrict__ ch = a.c + (size_t)h * a.KP;
  const int comp0 = w * KPW;
  T* sEw = sE + w * kChunk * C::PE;

  float cb[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) cb[rt][r] = ch[comp0 + 16 * rt + 4 * g + r];

  frag Wf[C::W_RES ? RT : 1][C::W_RES ? 2 * C::NKX : 1];
  if constexpr (C::W_RES) {
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int ks = 0; ks < 2 * C::NKX; ++ks) Wf[rt][ks] = w_frag<T, D>(Wh, comp0 + 16 * rt + c16, ks);
  }

  // State rows of this wave's components: S[dt][rt] (rows = components,
  // columns = value dims), Z[rt][r] for component 16 rt + 4 g + r.
  f32x4 S[C::DT][RT];
  float Z[RT][4];
#pragma unroll
  for (int dt = 0; dt < C::DT; ++dt)
#pragma unroll
    for (int rt = 0; rt < RT; ++rt) S[dt][rt] = zero4();
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) Z[rt][r] = 0.f;

  if constexpr (MODE != AGG) {
    if (a.has_init) {
      const int slot = MODE == CAUSAL ? p : 0;
      const float* ag = a.agg + ((size_t)bh * a.P + slot) * a.KP * DV;
      const float* az = a.aggz + ((size_t)bh * a.P + slot) * a.KP;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int comp = comp0 + 16 * rt + 4 * g + r;
#pragma unroll
          for (int dt = 0; dt < C::DT; ++dt) S[dt][rt][r] = ag[(size_t)comp * DV + 16 * dt + c16];
          Z[rt][r] = az[comp];
        }
    }
  }

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int nvalid = (int)((N - t0) < kChunk ? (N - t0) : kChunk);

    // ---- 1. tiles
    if constexpr (C::HAS_K) {
      load_x_tile<T, D, NT, C::SQ>(sXk, C::PX, Kg + (size_t)t0 * D, nvalid);
      load_v_tile<T, DV, NT>(sV, C::PV, Vg + (size_t)t0 * DV, nvalid);
    }
    if constexpr (C::HAS_Q) load_x_tile<T, D, NT, C::SQ>(sXq, C::PX, Qg + (size_t)t0 * D, nvalid);
    __syncthreads();

    // ---- 2. keys: routing, softmax, responsibilities
    frag EKf[4][C::NKC];
    float zsum[RT][4];
    if constexpr (C::HAS_K) {
      f32x4 Lk[4][RT];
      route<T, C>(Lk, sXk, Wh, Wf, cb, comp0);
      float mk[4], sk[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) local_softmax<RT>(Lk[ct], mk[ct], sk[ct]);
      float fk[4];
      if constexpr (NW > 1) {
        if (g == 0) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) sSt[w * kChunk + 16 * ct + c16] = make_float2(mk[ct], sk[ct]);
        }
        __syncthreads();
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
          const int tok = 16 * ct + c16;
          float mm = -INFINITY;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, sSt[ww * kChunk + tok].x);
          float ss = 0.f;
#pragma unroll
          for (int ww = 0; ww < NW; ++ww) {
            const float2 st = sSt[ww * kChunk + tok];
            ss += st.y * fast_exp2(st.x - mm);
          }
          fk[ct] = fast_exp2(mk[ct] - mm) / ss;
        }
      } else {
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) fk[ct] = 1.f / sk[ct];
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const float f = (16 * ct + c16 < nvalid) ? fk[ct] : 0.f;
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) Lk[ct][rt] *= f;
      }
      // normaliser increment and the transposed copy used by the state update
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          float z = 0.f;
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) z += Lk[ct][rt][r];
          zsum[rt][r] = row16_sum(z);
        }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
          T* dst = sEw + (16 * ct + c16) * C::PE + 16 * rt + 4 * g;
#pragma unroll
          for (int r = 0; r < 4; ++r) dst[r] = from_f32<T>(Lk[ct][rt][r]);
        }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct)
#pragma unroll
        for (int s = 0; s < C::NKC; ++s) EKf[ct][s] = M::chain(Lk[ct], s);
    }

    // ---- 3. queries: routing, wave-local softmax (combined across waves later)
    frag EQf[4][C::NKC];
    float mq[4], sq[4], den[4];
    if constexpr (C::HAS_Q) {
      f32x4 Lq[4][RT];
      route<T, C>(Lq, sXq, Wh, Wf, cb, comp0);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        local_softmax<RT>(Lq[ct], mq[ct], sq[ct]);
        float dn = 0.f;  // inter-chunk normaliser read: sum_k e_qk Z_k
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
#pragma unroll
          for (int r = 0; r < 4; ++r) dn += Lq[ct][rt][r] * Z[rt][r];
        den[ct] = group_sum(dn);
#pragma unroll
        for (int s = 0; s < C::NKC; ++s) EQf[ct][s] = M::chain(Lq[ct], s);
      }
    }

    // ---- 4. intra-chunk affinity A^T[kt][qt] = Gamma_K Gamma_Q^T (keys <= query)
    frag Atf[4][C::NKT];
    if constexpr (MODE == CAUSAL) {
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        f32x4 At[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          At[kt] = zero4();
          if (kt <= qt) {
#pragma unroll
            for (int s = 0; s < C::NKC; ++s) At[kt] = M::mma(EKf[kt][s], EQf[qt][s], At[kt]);
            if (kt == qt) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * g + r > c16) At[kt][r] = 0.f;
            }
          }
        }
        float dn = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) dn += At[kt][r];
        den[qt] += group_sum(dn);
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) Atf[qt][s] = M::chain(At, s);
      }
    }

    if constexpr (C::HAS_Q) __syncthreads();  // X tiles dead: the reduction area may be written

    // Gamma_K^T fragments (A operand of the update: lane = component row, k = keys).
    frag EKT[RT][C::NKT];
    if constexpr (C::HAS_K) {
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) EKT[rt][s] = ld_km_chain(sEw, C::PE, 16 * rt, s);
    }

    if constexpr (C::HAS_Q && C::HAS_K) {
      (void)0;
    }

    // ---- 5. per value block: partial reads, state update, cross-wave reduction
#pragma unroll
    for (int db = 0; db < C::NDB; ++db) {
      frag Vf[C::DTB][C::NKT];
      if constexpr (C::HAS_K) {
#pragma unroll
        for (int d = 0; d < C::DTB; ++d)
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) Vf[d][s] = ld_km_chain(sV, C::PV, 16 * (db * C::DTB + d), s);
      }
      if constexpr (C::HAS_Q) {
#pragma unroll
        for (int d = 0; d < C::DTB; ++d) {
          const int dt = db * C::DTB + d;
          frag Sf[C::NKC];
#pragma unroll
          for (int s = 0; s < C::NKC; ++s) Sf[s] = M::chain(S[dt], s);
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) {
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < C::NKC; ++s) acc = M::mma(Sf[s], EQf[qt][s], acc);
            if constexpr (MODE == CAUSAL) {
              constexpr int TPS = M::KS / 16 > 0 ? M::KS / 16 : 1;  // token tiles per k-step (bf16: 2)
#pragma unroll
              for (int s = 0; s < C::NKT; ++s) {
                // k-step s covers keys [s*KS, (s+1)*KS): needed when it starts at or before qt's tile end
                if ((s * M::KS) / 16 <= qt) acc = M::mma(Vf[d][s], Atf[qt][s], acc);
              }
              (void)TPS;
            }
            // partial numerator -> LDS [w][token][dv]
            f32x4* dst = reinterpret_cast<f32x4*>(sR + (w * kChunk + 16 * qt + c16) * C::PR + 16 * d + 4 * g);
            *dst = acc;
          }
        }
      }
      if constexpr (C::HAS_K) {
#pragma unroll
        for (int d = 0; d < C::DTB; ++d) {
          const int dt = db * C::DTB + d;
#pragma unroll
          for (int rt = 0; rt < RT; ++rt)
#pragma unroll
            for (int s = 0; s < C::NKT; ++s) S[dt][rt] = M::mma(EKT[rt][s], Vf[d][s], S[dt][rt]);
        }
      }
      if constexpr (C::HAS_Q) {
        if (db == 0 && g == 0) {
#pragma unroll
          for (int ct = 0; ct < 4; ++ct) sRQ[w * kChunk + 16 * ct + c16] = f32x4{den[ct], mq[ct], sq[ct], 0.f};
        }
        __syncthreads();
        // wave w combines tokens [w*TPW, (w+1)*TPW), 8 values per item
        constexpr int TPW = kChunk / NW;
        constexpr int IPT = C::DVB / 8;
        for (int it = l; it < TPW * IPT; it += 64) {
          const int tl = it / IPT;
          const int dv0 = (it - tl * IPT) * 8;
          const int tok = w * TPW + tl;
          if (tok < nvalid) {
            float mm = -INFINITY;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) mm = fmaxf(mm, sRQ[ww * kChunk + tok][1]);
            float ssum = 0.f, dsum = 0.f;
            float num[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) num[j] = 0.f;
#pragma unroll
            for (int ww = 0; ww < NW; ++ww) {
              const f32x4 rq = sRQ[ww * kChunk + tok];
              const float sc = fast_exp2(rq[1] - mm);
              ssum += rq[2] * sc;
              dsum += rq[0] * sc;
              const float* src = sR + (ww * kChunk + tok) * C::PR + dv0;
              const f32x4 a0 = *reinterpret_cast<const f32x4*>(src);
              const f32x4 a1 = *reinterpret_cast<const f32x4*>(src + 4);
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                num[j] += sc * a0[j];
                num[4 + j] += sc * a1[j];
              }
            }
            // O = (num / ssum) / (dsum / ssum + eps)
            const float inv = 1.f / (dsum + a.eps * ssum);
            typename Vec16<T>::type o0, o1;
            T* dst = Og + (size_t)(t0 + tok) * DV + db * C::DVB + dv0;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
              for (int j = 0; j < 8; ++j) o0[j] = from_f32<T>(num[j] * inv);
              *reinterpret_cast<bf16x8*>(dst) = o0;
            } else {
#pragma unroll
              for (int j = 0; j < 4; ++j) {
                o0[j] = num[j] * inv;
                o1[j] = num[4 + j] * inv;
              }
              *reinterpret_cast<f32x4*>(dst) = o0;
              *reinterpret_cast<f32x4*>(dst + 4) = o1;
            }
          }
        }
      }
      __syncthreads();
    }

    if constexpr (C::HAS_K) {
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) Z[rt][r] += zsum[rt][r];
    }
  }

  if constexpr (MODE == AGG) {
    float* ag = a.agg + ((size_t)bh * a.P + p) * a.KP * DV;
    float* az = a.aggz + ((size_t)bh * a.P + p) * a.KP;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int comp = comp0 + 16 * rt + 4 * g + r;
#pragma unroll
        for (int dt = 0; dt < C::DT; ++dt) ag[(size_t)comp * DV + 16 * dt + c16] = S[dt][rt][r];
        if (c16 == 0) az[comp] = Z[rt][r];
      }
  }
}


template <typename T, int D, int NW, int KPW>
inline hipError_t launch_mode(const Args& a, int mode, int segments, unsigned BH, hipStream_t st) {
  constexpr int DV = D;
  const dim3 grid((unsigned)segments, BH), block(NW * 64);
  switch (mode) {
    case AGG: hipLaunchKernelGGL((gma_kernel<T, D, DV, NW, KPW, AGG>), grid, block, 0, st, a); break;
    case CAUSAL: hipLaunchKernelGGL((gma_kernel<T, D, DV, NW, KPW, CAUSAL>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((gma_kernel<T, D, DV, NW, KPW, BIDIR>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}


}  // namespace gma
}  // namespace lm
