// linattn.hip -- chunkwise decayed linear attention and the curvature-
// conditioned-query (CCQ) read, forward, for gfx950.
//
// Method
//  * State write (allinfo.ai.kr post on linear attention, "Key messages" and
//    "Easy explanation"): S_t = g_t S_{t-1} + k_t v_t^T with a per-token decay
//    g_t in (0, 1]; plain read o_t = S_t^T q_t. The sequence is processed in
//    chunks: inside a chunk the pairwise decayed products are a masked matrix
//    product, and the state crosses only chunk boundaries.
//  * CCQ ("Don't Read Everything: A Curvature-Conditioned Query for Linear
//    Attention", section 2 Method): the read uses q_clean = q_t - lambda_t
//    Sigma_t q_t, Sigma_t the running key covariance with weights 1/t
//    (current token included, no decay), lambda_t = sigmoid(w . q_t + b). The
//    write rule is unchanged.
//
// Chunk algebra (row i of a chunk, global count t = t0 + i + 1, l = inclusive
// cumulative log2-decay inside the chunk):
//   o_i = sum_{j<=i} 2^(l_i - l_j) (q'_i . k_j) v_j + 2^(l_i) S_prev^T q'_i
//   S_next = 2^(l_last) S_prev + sum_j 2^(l_last - l_j) k_j v_j^T
// with q' = q (plain) or q_clean (CCQ). For CCQ, with M, m the running sums of
// k k^T and k carried across chunks and P_ij = q_i . k_j (j <= i):
//   delta_i = q_clean_i - q_i
//           = -alpha_i M_prev q_i + sum_{j<=i} k_j (beta_i - alpha_i P_ij) + beta_i m_prev
//   alpha_i = lambda_i / t,  beta_i = lambda_i (m_prev . q_i + sum_{j<=i} P_ij) / t^2.
// The read then uses q + delta. delta is formed in fp32 and rounded once, so the
// correction survives even where it is far below bf16 resolution of q.
//
// MI355X design: the transposed formulation (lane = query token) lets every
// product chain from registers. A workgroup of NW waves owns one (b, h,
// segment). Wave w owns the value columns [w CW, (w+1) CW) of S (and the same
// columns of the symmetric M). Q/K/V tiles sit row-major in LDS; k-major
// operands use the gfx950 transpose read. A segment pass (AGG) and a prefix
// combine at segment start give enough workgroups for short B*H.
#include "mfma.hpp"
#include "launch.hpp"

namespace lm {
namespace lin {

constexpr int kChunk = 64;

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* wl;  // [H][D]
  const float* bl;  // [H]
  void* out;
  float* agg;  // [B*H][P][sfl]
  int64_t N;
  int H;
  int P;
  int seg_len;
  int sfl;
};

template <int D>
struct Waves {
  static constexpr int NW = D / 16 < 4 ? D / 16 : 4;
  static constexpr int CW = D / NW;  // value (and M) columns per wave
  static constexpr int CT = CW / 16;
};

template <typename T, int D, bool CCQ, bool AGG>
struct Cfg {
  typedef Waves<D> Wv;
  static constexpr int NW = Wv::NW, CW = Wv::CW, CT = Wv::CT;
  static constexpr int KS = Mma<T>::KS;
  static constexpr int NKD = D / KS;      // k-steps over features
  static constexpr int NKT = kChunk / KS; // k-steps over tokens
  static constexpr int DT = D / 16;       // feature tiles
  static constexpr int PAD = 16 / (int)sizeof(T);
  static constexpr int PQ = D + PAD;
  static constexpr int tile = kChunk * PQ * (int)sizeof(T);
  static constexpr int o_q = 0;
  static constexpr int o_k = o_q + (AGG ? 0 : tile);
  static constexpr int o_v = o_k + tile;
  static constexpr int o_d = o_v + tile;                      // delta (CCQ)
  static constexpr int o_o = o_d + ((CCQ && !AGG) ? tile : 0); // output staging
  // rest of the layout without the staging tile, to decide whether it fits
  static constexpr int rest = ((CCQ && !AGG) ? 16 * PQ * (int)sizeof(T) : 0) + kChunk * 4 + (CCQ ? D * 4 : 0);
  static constexpr bool STAGE_O = !AGG && o_o + tile + rest <= 160 * 1024;
  static constexpr int o_dot = o_o + (STAGE_O ? tile : 0);    // [16][PQ] gate/mean rows (CCQ)
  static constexpr int o_l = o_dot + ((CCQ && !AGG) ? 16 * PQ * (int)sizeof(T) : 0);
  static constexpr int o_m = o_l + kChunk * 4;
  static constexpr int lds = o_m + (CCQ ? D * 4 : 0);
  static_assert(lds <= 160 * 1024, "LDS budget");
};

template <typename T, int D, int NT>
__device__ __forceinline__ void load_tile(T* s, int pq, const T* __restrict__ src, int nvalid) {
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
    *reinterpret_cast<vec*>(s + row * pq + cv * VN) = x;
  }
}

// hi/lo split of an fp32 D tile into two CHAIN fragments (bf16), or the value
// itself (f32; lo = 0).
template <typename T>
struct Split;
template <>
struct Split<bf16> {
  __device__ static __forceinline__ void chain(const f32x4* tiles, int s, bf16x8& hi, bf16x8& lo) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float x = tiles[2 * s + (i >> 2)][i & 3];
      const bf16 h = (bf16)x;
      hi[i] = h;
      lo[i] = (bf16)(x - (float)h);
    }
  }
};
template <>
struct Split<float> {
  __device__ static __forceinline__ void chain(const f32x4* tiles, int s, float& hi, float& lo) {
    hi = tiles[s >> 2][s & 3];
    lo = 0.f;
  }
};

template <typename T, int D, bool CCQ, bool AGG>
__global__ __launch_bounds__(Waves<D>::NW * 64) void lin_kernel(Args a) {
  typedef Cfg<T, D, CCQ, AGG> C;
  typedef Mma<T> M;
  typedef typename M::frag frag;
  constexpr int NW = C::NW, NT = NW * 64, CT = C::CT, DT = C::DT;

  __shared__ __attribute__((aligned(16))) char smem[C::lds];
  T* sQ = reinterpret_cast<T*>(smem + C::o_q);
  T* sK = reinterpret_cast<T*>(smem + C::o_k);
  T* sV = reinterpret_cast<T*>(smem + C::o_v);
  T* sDl = reinterpret_cast<T*>(smem + C::o_d);
  T* sO = reinterpret_cast<T*>(smem + C::o_o);
  T* sDot = reinterpret_cast<T*>(smem + C::o_dot);
  float* sL = reinterpret_cast<float*>(smem + C::o_l);
  float* sMv = reinterpret_cast<float*>(smem + C::o_m);

  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int bh = blockIdx.y, p = blockIdx.x;
  const int h = bh % a.H;
  const int64_t N = a.N;
  const int64_t t_begin = (int64_t)p * a.seg_len;
  const int64_t t_end = N < t_begin + a.seg_len ? N : t_begin + a.seg_len;
  const T* __restrict__ Qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * N * D;
  const T* __restrict__ Kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * N * D;
  const T* __restrict__ Vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * N * D;
  const float* __restrict__ Gg = a.g + (size_t)bh * N;
  T* __restrict__ Og = reinterpret_cast<T*>(a.out) + (size_t)bh * N * D;
  const int cbase = w * C::CW;

  // S[kt][ct]: rows = key features 16 kt + 4 g + r, cols = value dims cbase + 16 ct + c16.
  // M[kt][ct]: rows = features 16 kt + 4 g + r, cols = features cbase + 16 ct + c16.
  f32x4 S[DT][CT];
  f32x4 Mst[CCQ ? DT : 1][CCQ ? CT : 1];
  float mreg[CT];  // running key sum for column cbase + 16 ct + c16
#pragma unroll
  for (int kt = 0; kt < DT; ++kt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      S[kt][ct] = zero4();
      if constexpr (CCQ) Mst[kt][ct] = zero4();
    }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) mreg[ct] = 0.f;
  float lseg = 0.f;  // AGG: log2 of the segment's decay product

  if constexpr (!AGG) {
    for (int pp = 0; pp < p; ++pp) {
      const float* blk = a.agg + ((size_t)bh * a.P + pp) * a.sfl;
      const float G = blk[D * D];
#pragma unroll
      for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * kt + 4 * g + r, col = cbase + 16 * ct + c16;
            S[kt][ct][r] = G * S[kt][ct][r] + blk[row * D + col];
            if constexpr (CCQ) Mst[kt][ct][r] += blk[D * D + 1 + row * D + col];
          }
      if constexpr (CCQ) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) mreg[ct] += blk[2 * D * D + 1 + cbase + 16 * ct + c16];
      }
    }
  }
  if constexpr (CCQ && !AGG) {
    // gate rows of the dot tile: row 0 = w (hi), row 1 = w (lo); rows 2, 3 = running key sum (per chunk)
    for (int i = threadIdx.x; i < 16 * C::PQ; i += NT) {
      const int row = i / C::PQ, col = i - (i / C::PQ) * C::PQ;
      float x = 0.f;
      if (col < D && row < 2) {
        const float wv = a.wl[(size_t)h * D + col];
        const T hi = from_f32<T>(wv);
        x = row == 0 ? to_f32(hi) : wv - to_f32(hi);
      }
      sDot[i] = from_f32<T>(x);
    }
    if (g == 0) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) sMv[cbase + 16 * ct + c16] = mreg[ct];
    }
  }
  const float gate_b = CCQ ? a.bl[h] : 0.f;

  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk) {
    const int nvalid = (int)((N - t0) < kChunk ? (N - t0) : kChunk);
    __syncthreads();  // previous chunk done with the tiles; sMv complete

    // ---- 1. tiles, cumulative log2 decay, running-mean rows
    if constexpr (!AGG) load_tile<T, D, NT>(sQ, C::PQ, Qg + (size_t)t0 * D, nvalid);
    load_tile<T, D, NT>(sK, C::PQ, Kg + (size_t)t0 * D, nvalid);
    load_tile<T, D, NT>(sV, C::PQ, Vg + (size_t)t0 * D, nvalid);
    if (w == 0) {
      float x = l < nvalid ? fmaxf(log2f(Gg[t0 + l]), -200.f) : 0.f;
#pragma unroll
      for (int o = 1; o < 64; o <<= 1) {
        const float y = __shfl_up(x, o);
        if (l >= o) x += y;
      }
      sL[l] = x;
    }
    if constexpr (CCQ && !AGG) {
      for (int i = threadIdx.x; i < D; i += NT) {
        const float mv = sMv[i];
        const T hi = from_f32<T>(mv);
        sDot[2 * C::PQ + i] = hi;
        sDot[3 * C::PQ + i] = from_f32<T>(mv - to_f32(hi));
      }
    }
    __syncthreads();

    const float l_last = sL[kChunk - 1];

    if constexpr (!AGG) {
      float lq[4], bq[4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        lq[qt] = sL[16 * qt + c16];
        bq[qt] = fast_exp2(lq[qt]);
      }

      // ---- 2. raw scores P^T[kt][qt] = K Q^T (keys x queries), keys <= query
      f32x4 Pt[4][4];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt)
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          Pt[kt][qt] = zero4();
          if (kt <= qt) {
#pragma unroll
            for (int ks = 0; ks < C::NKD; ++ks)
              Pt[kt][qt] = M::mma(ld_kc_chain(sK, C::PQ, 16 * kt + c16, ks),
                                  ld_kc_chain(sQ, C::PQ, 16 * qt + c16, ks), Pt[kt][qt]);
            if (kt == qt) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * g + r > c16) Pt[kt][qt][r] = 0.f;
            }
          }
        }

      if constexpr (CCQ) {
        // ---- 3. per-query gate and mean terms
        float alpha[4], beta[4];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          f32x4 dq = zero4();
#pragma unroll
          for (int ks = 0; ks < C::NKD; ++ks)
            dq = M::mma(ld_kc_chain(sDot, C::PQ, c16, ks), ld_kc_chain(sQ, C::PQ, 16 * qt + c16, ks), dq);
          // rows 0..3 live in group 0: w.q = row0 + row1, m.q = row2 + row3
          const float wq = __shfl(dq[0] + dq[1], c16);
          const float mq = __shfl(dq[2] + dq[3], c16);
          float rs = 0.f;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
#pragma unroll
            for (int r = 0; r < 4; ++r) rs += Pt[kt][qt][r];
          rs = group_sum(rs);
          const float cnt = (float)(t0 + 16 * qt + c16 + 1);
          const float lam = 1.f / (1.f + expf(-(wq + gate_b)));
          alpha[qt] = lam / cnt;
          beta[qt] = lam * ((mq + rs) / cnt) / cnt;
        }
        // ---- 4. delta^T for this wave's feature columns
        float mprev[CT][4];
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) mprev[ct][r] = sMv[cbase + 16 * ct + 4 * g + r];
        frag Bf[4][C::NKT];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          f32x4 Bt[4];
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              const bool in = kt < qt || (kt == qt && 4 * g + r <= c16);
              Bt[kt][r] = in ? beta[qt] - alpha[qt] * Pt[kt][qt][r] : 0.f;
            }
          }
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) Bf[qt][s] = M::chain(Bt, s);
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          frag Mh[C::NKD], Ml[C::NKD];
          // A operand rows = features cbase + 16 ct + c16 (symmetric M): column tiles of M
          f32x4 Mcol[DT];
#pragma unroll
          for (int kt = 0; kt < DT; ++kt) Mcol[kt] = Mst[kt][ct];
#pragma unroll
          for (int s = 0; s < C::NKD; ++s) Split<T>::chain(Mcol, s, Mh[s], Ml[s]);
          frag KT[C::NKT];
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) KT[s] = ld_km_chain(sK, C::PQ, cbase + 16 * ct, s);
#pragma unroll
          for (int qt = 0; qt < 4; ++qt) {
            f32x4 mqv = zero4();
#pragma unroll
            for (int s = 0; s < C::NKD; ++s) {
              const frag qf = ld_kc_chain(sQ, C::PQ, 16 * qt + c16, s);
              mqv = M::mma(Mh[s], qf, mqv);
              if constexpr (sizeof(T) == 2) mqv = M::mma(Ml[s], qf, mqv);
            }
            f32x4 kb = zero4();
#pragma unroll
            for (int s = 0; s < C::NKT; ++s)
              if ((s * M::KS) / 16 <= qt) kb = M::mma(KT[s], Bf[qt][s], kb);
            T* dst = sDl + (16 * qt + c16) * C::PQ + cbase + 16 * ct + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r)
              dst[r] = from_f32<T>(-alpha[qt] * mqv[r] + kb[r] + beta[qt] * mprev[ct][r]);
          }
        }
        __syncthreads();  // delta complete
        // ---- 5. scores with the cleaned query: P^T += K delta^T (same mask)
#pragma unroll
        for (int qt = 0; qt < 4; ++qt)
#pragma unroll
          for (int kt = 0; kt < 4; ++kt) {
            if (kt <= qt) {
              f32x4 acc = zero4();
#pragma unroll
              for (int ks = 0; ks < C::NKD; ++ks)
                acc = M::mma(ld_kc_chain(sK, C::PQ, 16 * kt + c16, ks),
                             ld_kc_chain(sDl, C::PQ, 16 * qt + c16, ks), acc);
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (kt < qt || 4 * g + r <= c16) Pt[kt][qt][r] += acc[r];
            }
          }
      }

      // ---- 6. decay mask and read
      frag Pf[4][C::NKT];
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float lj = sL[16 * kt + 4 * g + r];
            Pt[kt][qt][r] = kt <= qt ? Pt[kt][qt][r] * fast_exp2(lq[qt] - lj) : 0.f;
          }
      }
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        f32x4 col[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) col[kt] = Pt[kt][qt];
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) Pf[qt][s] = M::chain(col, s);
      }
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        frag Sf[C::NKD];
        {
          f32x4 Scol[DT];
#pragma unroll
          for (int kt = 0; kt < DT; ++kt) Scol[kt] = S[kt][ct];
#pragma unroll
          for (int s = 0; s < C::NKD; ++s) Sf[s] = M::chain(Scol, s);
        }
        frag Vf[C::NKT];
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) Vf[s] = ld_km_chain(sV, C::PQ, cbase + 16 * ct, s);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          f32x4 inter = zero4();
#pragma unroll
          for (int s = 0; s < C::NKD; ++s) {
            inter = M::mma(Sf[s], ld_kc_chain(sQ, C::PQ, 16 * qt + c16, s), inter);
            if constexpr (CCQ) inter = M::mma(Sf[s], ld_kc_chain(sDl, C::PQ, 16 * qt + c16, s), inter);
          }
          f32x4 acc = zero4();
#pragma unroll
          for (int s = 0; s < C::NKT; ++s)
            if ((s * M::KS) / 16 <= qt) acc = M::mma(Vf[s], Pf[qt][s], acc);
          if constexpr (C::STAGE_O) {
            T* dst = sO + (16 * qt + c16) * C::PQ + cbase + 16 * ct + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[r] = from_f32<T>(acc[r] + bq[qt] * inter[r]);
          } else if (16 * qt + c16 < nvalid) {
            T* dst = Og + (size_t)(t0 + 16 * qt + c16) * D + cbase + 16 * ct + 4 * g;
#pragma unroll
            for (int r = 0; r < 4; ++r) dst[r] = from_f32<T>(acc[r] + bq[qt] * inter[r]);
          }
        }
      }
      if constexpr (C::STAGE_O) {
        __syncthreads();
        typedef typename Vec16<T>::type vec;
        constexpr int VN = Vec16<T>::n;
        constexpr int PER_ROW = D / VN;
        for (int i = threadIdx.x; i < nvalid * PER_ROW; i += NT) {
          const int row = i / PER_ROW, cv = i - (i / PER_ROW) * PER_ROW;
          *reinterpret_cast<vec*>(Og + (size_t)(t0 + row) * D + cv * VN) =
              *reinterpret_cast<const vec*>(sO + row * C::PQ + cv * VN);
        }
      }
    }

    // ---- 7. state updates
    {
      const float b_last = fast_exp2(l_last);
#pragma unroll
      for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) S[kt][ct] *= b_last;
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        frag Vw[C::NKT], Kc[C::NKT];
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) {
          frag vf = ld_km_chain(sV, C::PQ, cbase + 16 * ct, s);
          // scale by 2^(l_last - l_j)
          if constexpr (sizeof(T) == 2) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
              const int tok = 32 * s + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
              vf[i] = (bf16)((float)vf[i] * fast_exp2(l_last - sL[tok]));
            }
          } else {
            const int tok = 16 * (s >> 2) + 4 * g + (s & 3);
            vf = vf * fast_exp2(l_last - sL[tok]);
          }
          Vw[s] = vf;
          if constexpr (CCQ) Kc[s] = ld_km_chain(sK, C::PQ, cbase + 16 * ct, s);
        }
        if constexpr (CCQ) {
          // running key sum of this wave's columns
          float cs = 0.f;
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) {
            if constexpr (sizeof(T) == 2) {
#pragma unroll
              for (int i = 0; i < 8; ++i) cs += (float)Kc[s][i];
            } else {
              cs += Kc[s];
            }
          }
          mreg[ct] += group_sum(cs);
        }
#pragma unroll
        for (int kt = 0; kt < DT; ++kt) {
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) {
            const frag kf = ld_km_chain(sK, C::PQ, 16 * kt, s);
            S[kt][ct] = M::mma(kf, Vw[s], S[kt][ct]);
            if constexpr (CCQ) Mst[kt][ct] = M::mma(kf, Kc[s], Mst[kt][ct]);
          }
        }
      }
      if constexpr (CCQ && !AGG) {
        if (g == 0) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) sMv[cbase + 16 * ct + c16] = mreg[ct];
        }
      }
      lseg += l_last;
    }
  }

  if constexpr (AGG) {
    float* blk = a.agg + ((size_t)bh * a.P + p) * a.sfl;
#pragma unroll
    for (int kt = 0; kt < DT; ++kt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * kt + 4 * g + r, col = cbase + 16 * ct + c16;
          blk[row * D + col] = S[kt][ct][r];
          if constexpr (CCQ) blk[D * D + 1 + row * D + col] = Mst[kt][ct][r];
        }
    if (w == 0 && l == 0) blk[D * D] = exp2f(lseg);
    if constexpr (CCQ) {
      if (g == 0) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) blk[2 * D * D + 1 + cbase + 16 * ct + c16] = mreg[ct];
      }
    }
  }
}

template <typename T, int D, bool CCQ>
static hipError_t launch_d(const LinLaunch& L, hipStream_t st) {
  Args a;
  a.q = L.q;
  a.k = L.k;
  a.v = L.v;
  a.g = L.g;
  a.wl = L.w_lambda;
  a.bl = L.b_lambda;
  a.out = L.out;
  a.agg = L.agg;
  a.N = L.N;
  a.H = (int)L.H;
  a.P = (int)L.P;
  a.seg_len = (int)L.seg_len;
  a.sfl = (int)lin_state_floats(D, CCQ);
  constexpr int NT = Waves<D>::NW * 64;
  const unsigned BH = (unsigned)(L.B * L.H);
  if (L.P > 1)
    hipLaunchKernelGGL((lin_kernel<T, D, CCQ, true>), dim3((unsigned)(L.P - 1), BH), dim3(NT), 0, st, a);
  hipLaunchKernelGGL((lin_kernel<T, D, CCQ, false>), dim3((unsigned)L.P, BH), dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <typename T, bool CCQ>
static hipError_t launch_t(const LinLaunch& L, hipStream_t st) {
  switch (L.D) {
    case 32: return launch_d<T, 32, CCQ>(L, st);
    case 64: return launch_d<T, 64, CCQ>(L, st);
    case 128: return launch_d<T, 128, CCQ>(L, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace lin

hipError_t linattn_launch(const LinLaunch& L, hipStream_t st) {
  if (L.bf16) return L.ccq ? lin::launch_t<bf16, true>(L, st) : lin::launch_t<bf16, false>(L, st);
  return L.ccq ? lin::launch_t<float, true>(L, st) : lin::launch_t<float, false>(L, st);
}

}  // namespace lm
