// linattn_vec.hip -- decayed linear attention with a decay gate per key feature,
// for gfx950.
//
// Method (allinfo.ai.kr linear attention post, "Key messages": decay gates on
// the matrix state, which may forget at a different rate per channel):
//     S_t = diag(g_t) S_{t-1} + k_t v_t^T,   o_t = S_t^T q_t,   g_t in (0, 1]^dk.
//
// MI355X design
//  * One workgroup per (b, h, segment), 16 value columns per wave (D/16 waves);
//    each wave holds its columns of S (D x 16, fp32) in registers.
//  * Chunks of 64 tokens in LDS (Q, K, V double-buffered; G single-buffered
//    and turned in place into the per-feature cumulative log2 decay L).
//  * A chunk is four sub-chunks of 16 tokens, run as a short recurrence on
//    the matrix core. With P_t = L before sub-chunk t and E_t = L at its last
//    token:
//        read    o_i = (q_i * 2^(L_i - P_t))^T S + sum_{j in t, j <= i} A_ij v_j
//        update  S  <- diag(2^(E_t - P_t)) S + sum_{j in t} (k_j * 2^(E_t - L_j)) v_j^T
//    Every exponent there is <= 0. The diagonal scores A_ij = sum_a q_ia k_ja
//    2^(L_ia - L_ja) are one 16 x 16 product per sub-chunk with both operands
//    scaled about the sub-chunk's middle token; with every log2 g of the chunk
//    at or above -15, no scaled operand exceeds 2^120, so the product stays
//    finite where it is kept (j <= i).
//  * A chunk that holds a decay below 2^-15 (g = 0 included) runs the
//    recurrence itself instead, token by token on the fp32 state (the
//    one-token step's arithmetic), so every g in (0, 1] is honoured exactly;
//    the other chunks are unaffected.
//  * Long sequences are cut into segments: a segment pass computes the S and
//    the decay (per feature) of every sub-segment (two per segment when the
//    segment length allows), a fixed-order scan leaves the state at every
//    segment start, and the chunk pass starts from it.
#include "mfma.hpp"
#include "launch.hpp"

namespace lm {
namespace vec {

constexpr int kC = 64;
constexpr float kMinLog2G = -15.f;  // below this a chunk takes the token-by-token path

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const float* g;  // [B*H][N][D]
  void* out;
  float* agg;  // [B*H][P][sfl]: S (D x D), then the segment's decay per feature (D)
  int64_t N;
  int P;
  int seg_len;
  int sfl;
  int has_init;  // chunk pass: start from the state block R * (segment index)
  int R;         // sub-segments per segment in the segment pass
  float* st_out;  // chunk pass (optional): S after the last token, [B*H][D][D]
};

template <typename T, int D, bool AGG>
struct Cfg {
  static constexpr int NW = D / 16;
  static constexpr int NT = NW * 64;
  static constexpr int DT = D / 16;
  static constexpr int CPR = D * (int)sizeof(T) / 16;  // 16-byte chunks per Q/K/V row
  static constexpr int CPRG = D / 4;                   // 16-byte chunks per G/L row
  static constexpr int EPC = 16 / (int)sizeof(T);      // elements per chunk
  static constexpr int TB = kC * D * (int)sizeof(T);
  static constexpr int GB = kC * D * 4;
  static constexpr int NTL = AGG ? 2 : 3;  // tiles per buffer: (Q), K, V
  static constexpr int BUFB = NTL * TB;
  static constexpr int NBUF = (2 * BUFB + GB + 16 * 1024 <= 150 * 1024) ? 2 : 1;
  static constexpr int AP = sizeof(T) == 2 ? 24 : 20;  // pitch of the diagonal score tiles
  static constexpr int UNR = sizeof(T) == 2 ? 4 : 1;    // unrolled sub-chunks
  static constexpr int H2 = NW >= 8 ? 2 : 1;  // feature halves of the diagonal products (one per wave)
};

// L (fp32, swizzled like a DMA tile) at token row r, feature f.
template <int CPRG>
__device__ __forceinline__ float& Lat(char* sL, int r, int f) {
  return *reinterpret_cast<float*>(sL + tile_off<CPRG, 4>(r, f));
}

// L at row r for the N4 * 4 features f0 .. (f0 a multiple of 4): whole 16-byte
// chunks of the swizzled tile.
template <int CPRG, int N4>
__device__ __forceinline__ void load_l(const char* sL, int r, int f0, float* x) {
#pragma unroll
  for (int u = 0; u < N4; ++u) {
    const f32x4 c = *reinterpret_cast<const f32x4*>(sL + r * CPRG * 16 + (((f0 >> 2) + u) ^ tile_sw<CPRG>(r)) * 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) x[4 * u + i] = c[i];
  }
}

// NATURAL-order operand fragment of row `row` of a tile (k = features of k-step
// ks), each element scaled by 2^(sign (L[row] - L[ref])).
template <typename T, int CPR, int CPRG>
__device__ __forceinline__ typename Mma<T>::frag scaled_nat(const char* tile, char* sL, int row, int ks, int ref,
                                                            float sign) {
  const int g = lane_id() >> 4;
  if constexpr (sizeof(T) == 2) {
    const int f0 = ks * 32 + 8 * g;
    const bf16x8 x = tl_nat<CPR>(tile, row, ks);
    float lr[8], lf[8];
    load_l<CPRG, 2>(sL, row, f0, lr);
    load_l<CPRG, 2>(sL, ref, f0, lf);
    bf16x8 y;
#pragma unroll
    for (int i = 0; i < 8; ++i) y[i] = (bf16)((float)x[i] * fast_exp2(sign * (lr[i] - lf[i])));
    return y;
  } else {
    const int f = ks * 4 + g;
    return tl_nat_f<CPR>(tile, row, ks) * fast_exp2(sign * (Lat<CPRG>(sL, row, f) - Lat<CPRG>(sL, ref, f)));
  }
}

template <typename T, int D, bool AGG>
__global__ __launch_bounds__(D / 16 * 64) void vec_kernel(Args a) {
  typedef Cfg<T, D, AGG> C;
  typedef Mma<T> M;
  typedef typename M::frag frag;
  constexpr int NW = C::NW, NT = C::NT, DT = C::DT, CPR = C::CPR, CPRG = C::CPRG;

  __shared__ __attribute__((aligned(16))) char sBuf[C::NBUF][C::BUFB];
  __shared__ __attribute__((aligned(16))) char sG[C::GB];
  __shared__ __attribute__((aligned(16))) float sF[AGG ? 1 : 4][D];
  __shared__ __attribute__((aligned(16))) T sA[AGG ? 1 : C::H2][4][16][C::AP];
  __shared__ float sTot[NW][D];
  __shared__ float sLseg[D];
  __shared__ int sTiny[2];  // per chunk parity: the chunk holds a decay below 2^kMinLog2G

  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15, tid = threadIdx.x;
  const int bh = blockIdx.y, p = blockIdx.x;
  const int64_t N = a.N;
  const int64_t t_begin = (int64_t)p * a.seg_len;
  const int64_t t_end = N < t_begin + a.seg_len ? N : t_begin + a.seg_len;
  const T* Qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * N * D;
  const T* Kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * N * D;
  const T* Vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * N * D;
  const float* Gg = a.g + (size_t)bh * N * D;
  T* Og = reinterpret_cast<T*>(a.out) + (size_t)bh * N * D;
  const int cbase = 16 * w;

  TileDma<T, D, NW> dt;
  dt.init();
  auto issue = [&](char* buf, int64_t t0) {
    const int rows = (int)(N - t0 < kC ? N - t0 : kC);
    if constexpr (!AGG) dt.issue(buf, Qg + (size_t)t0 * D, rows);
    dt.issue(buf + (AGG ? 0 : C::TB), Kg + (size_t)t0 * D, rows);
    dt.issue(buf + (AGG ? C::TB : 2 * C::TB), Vg + (size_t)t0 * D, rows);
  };
  // The decays reach the L pass through registers: wave w owns rows
  // w TPW .. w TPW + TPW - 1, lane l features l + 64 i. They are loaded one
  // chunk ahead (rows past the end read as 1, i.e. no decay).
  constexpr int TPW = kC / NW;
  constexpr int FPL = (D + 63) / 64;
  constexpr int GR = TPW * FPL;
  auto load_g = [&](float* gd, int64_t t0) {
#pragma unroll
    for (int rr = 0; rr < TPW; ++rr)
#pragma unroll
      for (int i = 0; i < FPL; ++i) {
        const int f = l + 64 * i;
        const int64_t row = t0 + w * TPW + rr;
        gd[rr * FPL + i] = (f < D && row < N) ? Gg[(size_t)row * D + f] : 1.f;
      }
  };

  f32x4 S[DT];
#pragma unroll
  for (int kt = 0; kt < DT; ++kt) S[kt] = zero4();
  if constexpr (!AGG) {
    if (a.has_init) {
      const float* blk = a.agg + ((size_t)bh * a.P + (size_t)a.R * p) * a.sfl;
#pragma unroll
      for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[kt][r] = blk[(16 * kt + 4 * g + r) * D + cbase + c16];
    }
  }
  if (tid < D) sLseg[tid] = 0.f;
  if (tid < 2) sTiny[tid] = 0;

  float gA[GR], gB[C::NBUF == 2 ? GR : 1];
  if constexpr (C::NBUF == 2) {
    if (t_begin < t_end) {
      issue(sBuf[0], t_begin);
      load_g(gA, t_begin);
    }
  }
  // The chunk as the plain recurrence, token by token, on the fp32 state this
  // wave holds (rows a = 16 kt + 4 g + r, column cbase + c16):
  //   S <- diag(g_i) S + k_i v_i^T,  o_i = S^T q_i.
  // The decay tile sG is overwritten with the raw decays first.
  auto exact_chunk = [&](int64_t t0, const char* Qt, const char* Kt, const char* Vt) {
    for (int idx = tid; idx < kC * D; idx += NT) {
      const int r = idx / D, f = idx - (idx / D) * D;
      Lat<CPRG>(sG, r, f) = t0 + r < N ? Gg[(size_t)(t0 + r) * D + f] : 1.f;
    }
    lds_barrier();
    const int nrow = (int)(N - t0 < kC ? N - t0 : kC);
    for (int i = 0; i < nrow; ++i) {
      const float vi = to_f32(*reinterpret_cast<const T*>(Vt + tile_off<CPR, sizeof(T)>(i, cbase + c16)));
      float part = 0.f;
#pragma unroll
      for (int kt = 0; kt < DT; ++kt) {
        float gi[4];
        load_l<CPRG, 1>(sG, i, 16 * kt + 4 * g, gi);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int f = 16 * kt + 4 * g + r;
          const float ki = to_f32(*reinterpret_cast<const T*>(Kt + tile_off<CPR, sizeof(T)>(i, f)));
          S[kt][r] = gi[r] * S[kt][r] + ki * vi;
          if constexpr (!AGG) part += S[kt][r] * to_f32(*reinterpret_cast<const T*>(Qt + tile_off<CPR, sizeof(T)>(i, f)));
        }
        // keeps the loads of one feature tile from being hoisted over the
        // others (this path is for correctness, not speed, and shares the
        // kernel's registers with the chunk form)
        __builtin_amdgcn_sched_barrier(0);
      }
      if constexpr (!AGG) {
        part = group_sum(part);
        if (g == 0) Og[(size_t)(t0 + i) * D + cbase + c16] = from_f32<T>(part);
      }
    }
    if constexpr (AGG) {
      if (tid < D) {
        float ll = 0.f;
        for (int i = 0; i < nrow; ++i) ll += __builtin_amdgcn_logf(Lat<CPRG>(sG, i, tid));
        sLseg[tid] += ll;
      }
    }
  };
  // One chunk; gc holds its decays, gn receives the next chunk's.
  auto body = [&](int64_t t0, int it, float* gc, float* gn) {
    char* buf = sBuf[C::NBUF == 2 ? (it & 1) : 0];
    if constexpr (C::NBUF == 1) {
      lds_barrier();  // the previous chunk is done with every tile
      issue(buf, t0);
    }
    char* Qt = buf;
    char* Kt = buf + (AGG ? 0 : C::TB);
    char* Vt = Kt + C::TB;
    wait_vmem();
    lds_barrier();
    // the next chunk's tiles and decays load during this whole chunk (the other
    // buffer was released by the barrier above)
    if constexpr (C::NBUF == 2) {
      if (t0 + kC < t_end) issue(sBuf[(it + 1) & 1], t0 + kC);
    }

    // ---- 1. L: cumulative log2 decay per feature. Each wave scans its block of
    //      rows sequentially (lanes = features), then adds the totals of the
    //      blocks before it.
    {
      // the block's prefix stays in registers (gc is reused for it) until the
      // offset of the earlier blocks is known
      bool tiny = false;
#pragma unroll
      for (int i = 0; i < FPL; ++i) {
        float run = 0.f;
#pragma unroll
        for (int rr = 0; rr < TPW; ++rr) {
          const float lg = __builtin_amdgcn_logf(gc[rr * FPL + i]);
          tiny = tiny || !(lg >= kMinLog2G);
          run += fmaxf(lg, kMinLog2G);
          gc[rr * FPL + i] = run;
        }
        if (l + 64 * i < D) sTot[w][l + 64 * i] = run;
      }
      if (__any(tiny) && l == 0) sTiny[it & 1] = 1;
      lds_barrier();
#pragma unroll
      for (int i = 0; i < FPL; ++i) {
        const int f = l + 64 * i;
        if (f < D) {
          float off = 0.f;
#pragma unroll
          for (int u = 0; u < NW - 1; ++u)
            if (u < w) off += sTot[u][f];
#pragma unroll
          for (int rr = 0; rr < TPW; ++rr) Lat<CPRG>(sG, w * TPW + rr, f) = gc[rr * FPL + i] + off;
        }
      }
      lds_barrier();
    }
    // the flag of the chunk before this one was read by every wave long before
    // this point, so its slot is cleared for the next chunk here
    const bool exact = sTiny[it & 1] != 0;
    if (tid == 0) sTiny[(it + 1) & 1] = 0;
    if (exact) {
      exact_chunk(t0, Qt, Kt, Vt);
      if constexpr (C::NBUF == 2) {
        if (t0 + kC < t_end) load_g(gn, t0 + kC);
      }
      return;
    }

    // ---- 2a. diagonal scores of the four sub-chunks, scaled about token 16t + 8
    if constexpr (!AGG) {
      // (with eight waves each sub-chunk's product is split in two halves of
      // the features, one per wave; the read adds both)
      constexpr int KSN = D / M::KS / C::H2;
      for (int job = w; job < 4 * C::H2; job += NW) {
        const int t = job & 3, h = job >> 2;
        const int mid = 16 * t + 8;
        f32x4 acc = zero4();
#pragma unroll
        for (int kk = 0; kk < KSN; ++kk) {
          const int ks = h * KSN + kk;
          const frag qa = scaled_nat<T, CPR, CPRG>(Qt, sG, 16 * t + c16, ks, mid, 1.f);
          const frag kb = scaled_nat<T, CPR, CPRG>(Kt, sG, 16 * t + c16, ks, mid, -1.f);
          acc = M::mma(qa, kb, acc);
        }
        // lane: key j = c16, queries i = 4g + r; keep j <= i (a select, so the
        // unused entries may be anything)
#pragma unroll
        for (int r = 0; r < 4; ++r) sA[h][t][4 * g + r][c16] = from_f32<T>(c16 <= 4 * g + r ? acc[r] : 0.f);
      }
      lds_barrier();
    }

    // ---- 2b. Q -> q * 2^(L - P_t), K -> k * 2^(E - L) in place (E = E_t, or
    //      the chunk's last token in the segment pass); row decays F
    for (int idx = tid; idx < kC * CPR; idx += NT) {
      typedef typename Vec16<T>::type vec;
      constexpr int EPC = C::EPC;
      const int r = idx / CPR, pc = idx - (idx / CPR) * CPR;
      const int f0 = (pc ^ tile_sw<CPR>(r)) * EPC;
      const int t = r >> 4;
      const int re = AGG ? kC - 1 : 16 * t + 15;
      float lr[EPC], le[EPC];
      load_l<CPRG, EPC / 4>(sG, r, f0, lr);
      load_l<CPRG, EPC / 4>(sG, re, f0, le);
      vec* pk = reinterpret_cast<vec*>(Kt + r * CPR * 16 + pc * 16);
      vec kv = *pk;
#pragma unroll
      for (int e = 0; e < EPC; ++e) kv[e] = from_f32<T>(to_f32(kv[e]) * fast_exp2(le[e] - lr[e]));
      *pk = kv;
      if constexpr (!AGG) {
        float lp[EPC];
        if (t > 0) {
          load_l<CPRG, EPC / 4>(sG, 16 * t - 1, f0, lp);
        } else {
#pragma unroll
          for (int e = 0; e < EPC; ++e) lp[e] = 0.f;
        }
        vec* pq = reinterpret_cast<vec*>(Qt + r * CPR * 16 + pc * 16);
        vec qv = *pq;
#pragma unroll
        for (int e = 0; e < EPC; ++e) qv[e] = from_f32<T>(to_f32(qv[e]) * fast_exp2(lr[e] - lp[e]));
        *pq = qv;
      }
    }
    if constexpr (AGG) {
      if (tid < D) {
        const float ll = Lat<CPRG>(sG, kC - 1, tid);
        sF[0][tid] = fast_exp2(ll);
        sLseg[tid] += ll;
      }
    } else {
      for (int idx = tid; idx < 4 * D; idx += NT) {
        const int t = idx / D, f = idx - (idx / D) * D;
        const float pt = t > 0 ? Lat<CPRG>(sG, 16 * t - 1, f) : 0.f;
        sF[t][f] = fast_exp2(Lat<CPRG>(sG, 16 * t + 15, f) - pt);
      }
    }
    lds_barrier();
    // the next chunk's decays load during the sub-chunk recurrence (issued here
    // rather than with the tiles, so that the first phases do not queue behind
    // them in the address unit)
    if constexpr (C::NBUF == 2) {
      if (t0 + kC < t_end) load_g(gn, t0 + kC);
    }


    if constexpr (!AGG) {
      // ---- 3. four sub-chunks: read with the state before them, then update
      // (unrolled where the registers allow, so that tile addresses fold)
#pragma unroll C::UNR
      for (int t = 0; t < 4; ++t) {
        const int r0 = 16 * t;
        f32x4 o = zero4();
#pragma unroll
        for (int ks = 0; ks < D / M::KS; ++ks) {
          const frag qa = tl_chain_t<CPR, T>(Qt, r0 + c16, ks);
          frag sb;
          if constexpr (sizeof(T) == 2)
            sb = M::chain(S, ks);
          else
            sb = S[ks >> 2][ks & 3];
          o = M::mma(qa, sb, o);
        }
        // intra-sub-chunk: scores (rows = queries, k = keys) times V
        if constexpr (sizeof(T) == 2) {
          const bf16x4 vlo = tl_tr16<CPR>(Vt, r0 + 4 * g, cbase);
          const bf16 z = (bf16)0.f;
          const frag vb = bf16x8{vlo[0], vlo[1], vlo[2], vlo[3], z, z, z, z};
#pragma unroll
          for (int h = 0; h < C::H2; ++h) {
            const bf16x4 alo = *reinterpret_cast<const bf16x4*>(&sA[h][t][c16][4 * g]);
            o = M::mma(bf16x8{alo[0], alo[1], alo[2], alo[3], z, z, z, z}, vb, o);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t row = t0 + r0 + 4 * g + r;
            if (row < N) Og[(size_t)row * D + cbase + c16] = from_f32<T>(o[r]);
          }
          // update: S <- diag(F_t) S + Khat_t^T V_t
#pragma unroll
          for (int kt = 0; kt < DT; ++kt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) S[kt][r] *= sF[t][16 * kt + 4 * g + r];
            const bf16x4 klo = tl_tr16<CPR>(Kt, r0 + 4 * g, 16 * kt);
            const frag ka = bf16x8{klo[0], klo[1], klo[2], klo[3], z, z, z, z};
            S[kt] = M::mma(ka, vb, S[kt]);
          }
        } else {
          float vb[4];
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            vb[s] = *reinterpret_cast<const float*>(Vt + tile_off<CPR, 4>(r0 + 4 * g + s, cbase + c16));
#pragma unroll
            for (int h = 0; h < C::H2; ++h) o = M::mma(sA[h][t][c16][4 * g + s], vb[s], o);
          }
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int64_t row = t0 + r0 + 4 * g + r;
            if (row < N) Og[(size_t)row * D + cbase + c16] = from_f32<T>(o[r]);
          }
#pragma unroll
          for (int kt = 0; kt < DT; ++kt) {
#pragma unroll
            for (int r = 0; r < 4; ++r) S[kt][r] *= sF[t][16 * kt + 4 * g + r];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              const float ka = *reinterpret_cast<const float*>(Kt + tile_off<CPR, 4>(r0 + 4 * g + s, 16 * kt + c16));
              S[kt] = M::mma(ka, vb[s], S[kt]);
            }
          }
        }
      }
    } else {
      // ---- 3'. segment pass: S <- diag(2^L_last) S + Khat^T V over the chunk
#pragma unroll
      for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) S[kt][r] *= sF[0][16 * kt + 4 * g + r];
#pragma unroll
      for (int ks = 0; ks < kC / M::KS; ++ks) {
        const frag vb = tl_kmaj_t<CPR, T>(Vt, ks, cbase);
#pragma unroll
        for (int kt = 0; kt < DT; ++kt) S[kt] = M::mma(tl_kmaj_t<CPR, T>(Kt, ks, 16 * kt), vb, S[kt]);
      }
    }
  };

  if constexpr (C::NBUF == 2) {
    // two chunks per trip, so that the two decay register sets swap roles
    // without copies (a copy would wait for the loads in flight)
    int it = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += 2 * kC, it += 2) {
      body(t0, it, gA, gB);
      if (t0 + kC < t_end) body(t0 + kC, it + 1, gB, gA);
    }
  } else {
    // one buffer (large fp32 tiles): the chunk's decays load with its tiles
    int it = 0;
    for (int64_t t0 = t_begin; t0 < t_end; t0 += kC, ++it) {
      load_g(gA, t0);
      body(t0, it, gA, gB);
    }
  }

  if constexpr (!AGG) {
    // the workgroup of the last segment holds the state after the last token
    if (a.st_out && p == (int)gridDim.x - 1) {
      float* so = a.st_out + (size_t)bh * D * D;
#pragma unroll
      for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int r = 0; r < 4; ++r) so[(16 * kt + 4 * g + r) * D + cbase + c16] = S[kt][r];
    }
  }
  if constexpr (AGG) {
    float* blk = a.agg + ((size_t)bh * a.P + p) * a.sfl;
#pragma unroll
    for (int kt = 0; kt < DT; ++kt)
#pragma unroll
      for (int r = 0; r < 4; ++r) blk[(16 * kt + 4 * g + r) * D + cbase + c16] = S[kt][r];
    if (tid < D) blk[D * D + tid] = exp2f(sLseg[tid]);
  }
}

// Scan over the sub-segment states of every sequence, in a fixed order. Blocks
// 0 .. nsub-1 hold the states of consecutive sub-segments (R per segment) on
// entry; block R p becomes the state at the start of segment p:
// run <- diag(G_q) run + S_q over the sub-segments q before it, with G_q the
// sub-segment's decay per feature (left in place). run starts from the caller's
// state S (D x D) when there is one, else from zero.
__global__ __launch_bounds__(256) void vec_scan(float* __restrict__ agg, int slots, int nsub, int R, int sfl, int D,
                                                const float* __restrict__ init) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  if (e >= D * D) return;
  const int row = e / D;
  float* base = agg + (size_t)bh * slots * sfl;
  float run = init ? init[(size_t)bh * D * D + e] : 0.f;
  for (int q = 0; q < nsub; ++q) {
    float* x = base + (size_t)q * sfl + e;
    const float s = *x;
    const float gq = base[(size_t)q * sfl + D * D + row];
    if (q % R == 0) *x = run;
    run = gq * run + s;
  }
  base[(size_t)nsub * sfl + e] = run;
}

template <typename T, int D>
static hipError_t launch_d(const VecLaunch& L, hipStream_t st) {
  Args a;
  a.q = L.q;
  a.k = L.k;
  a.v = L.v;
  a.g = L.g;
  a.out = L.out;
  a.agg = L.agg;
  a.N = L.N;
  a.sfl = (int)vec_state_floats(D);
  a.has_init = 0;
  a.R = (int)L.R;
  a.P = (int)(L.R * L.P);  // state blocks per (b,h)
  a.st_out = L.state_out;
  const unsigned BH = (unsigned)(L.B * L.H);
  if (L.P > 1 || L.state_in) {
    // sub-segment states of segments 0 .. P-2, then their prefixes (from the
    // caller's state when there is one)
    const int nsub = (int)(L.R * (L.P - 1));
    a.seg_len = (int)(L.seg_len / L.R);
    hipError_t e;
    if (nsub > 0) {
      hipLaunchKernelGGL((vec_kernel<T, D, true>), dim3((unsigned)nsub, BH), dim3(Cfg<T, D, true>::NT), 0, st, a);
      if ((e = hipGetLastError()) != hipSuccess) return e;
    }
    hipLaunchKernelGGL(vec_scan, dim3((unsigned)((D * D + 255) / 256), BH), dim3(256), 0, st, L.agg, a.P, nsub, a.R,
                       a.sfl, D, L.state_in);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    a.has_init = 1;
  }
  a.seg_len = (int)L.seg_len;
  hipLaunchKernelGGL((vec_kernel<T, D, false>), dim3((unsigned)L.P, BH), dim3(Cfg<T, D, false>::NT), 0, st, a);
  return hipGetLastError();
}

template <typename T>
static hipError_t launch_t(const VecLaunch& L, hipStream_t st) {
  switch (L.D) {
    case 32: return launch_d<T, 32>(L, st);
    case 64: return launch_d<T, 64>(L, st);
    case 128: return launch_d<T, 128>(L, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace vec

hipError_t linattn_vec_launch(const VecLaunch& L, hipStream_t st) {
  return L.bf16 ? vec::launch_t<bf16>(L, st) : vec::launch_t<float>(L, st);
}

}  // namespace lm
