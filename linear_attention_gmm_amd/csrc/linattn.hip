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
// correction survives even where it is far below the bf16 resolution of q.
//
// MI355X design
//  * Transposed formulation (lane = query token): products chain from registers.
//  * A workgroup of NW waves (8 at D = 128, two per SIMD) owns one (b, h,
//    segment). Wave w owns the value columns [w CW, (w+1) CW) of S and the
//    same columns of the symmetric M and of m, in fp32 registers. The
//    per-query work (score tiles, gate and mean terms, decay mask) is shared
//    out by (query tile, key tile) pairs (see Waves) and handed to the other
//    waves through LDS; delta and the read are split by columns.
//  * Q/K/V/g tiles arrive by direct global->LDS DMA (inline asm) into
//    XOR-swizzled, double-buffered tiles; the next chunk's transfers are spread
//    over the phases of this one. k-major operands use the gfx950 LDS
//    transpose read.
//  * The decay of S is applied lazily (see State::ls), and the decay factors
//    of the score tiles never have a positive exponent (decay_tile).
//  * A segment-state pass (AGG, two sub-segments per segment) and a prefix
//    scan give the state at every segment start, so that B*H too small to
//    fill the GPU is cut into independent segments.
#include "mfma.hpp"
#include "launch.hpp"

namespace lm {
namespace lin {

constexpr int kC = 64;
constexpr int kLds = 160 * 1024;
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLazy = 64.f;

// B operand (CHAIN order, token step s) of the lower-triangular ones matrix for
// query q of the chunk: entry (token j, query q) is 1 where j <= q.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag tri_frag(int s, int q) {
  typename Mma<T>::frag f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = chain_k<T>(s, i) <= q ? (bf16)1.f : (bf16)0.f;
  } else {
    f = chain_k<T>(s, 0) <= q ? 1.f : 0.f;
  }
  return f;
}

struct Args {
  const void* q;
  const void* k;
  const void* v;
  const float* g;
  const float* wl;  // [H][D]
  const float* bl;  // [H]
  void* out;
  float* agg;  // [B*H][P][sfl] state blocks
  int64_t N;
  int H;
  int P;         // state blocks per (b,h)
  int seg_len;   // tokens per workgroup (a segment, or a sub-segment in the AGG pass)
  int sfl;
  int has_init;  // chunk pass: start from the state block R * (segment index)
  int R;
  int64_t t_off;   // tokens before the first one (held by a caller's initial state)
  float* st_out;   // chunk pass (optional): state after the last token, [S | M | m]
};

// Waves per workgroup: 16 state columns per wave (8 waves, two per SIMD, at
// D = 128 so that the MFMA work of one wave overlaps the VALU work of the
// other).
// The per-query work (score tiles of query tile qt against key tiles kt <= qt)
// is shared out by (qt, kt): with 8 waves each query tile has two owners, part 0
// taking the even key tiles and part 1 the odd ones; part-1 waves take the query
// tiles in reverse order, so that waves w and w + 4 (one SIMD) get a light and a
// heavy tile.
template <int D>
struct Waves {
  static constexpr int NW = D / 16;
  static constexpr int CW = D / NW;  // value (and M) columns per wave
  static constexpr int CT = CW / 16;
  static constexpr int SPLIT = NW >= 8 ? 2 : 1;  // owners per query tile
  static constexpr int QW = NW / SPLIT;           // waves per part
  static constexpr int QPW = QW >= 4 ? 1 : 4 / QW;  // query tiles per wave
  static constexpr int KPW = 4 / SPLIT;           // key tiles per owned query tile
  __device__ static __forceinline__ int part(int w) { return w / QW; }
  __device__ static __forceinline__ int qtile(int w, int qi) {
    const int r = w % QW + QW * qi;
    return part(w) == 0 ? r : 3 - r;
  }
  __device__ static __forceinline__ int ktile(int w, int j) { return part(w) + SPLIT * j; }
};

template <typename T, int D, bool CCQ, bool AGG>
struct Cfg {
  typedef Waves<D> Wv;
  static constexpr int NW = Wv::NW, CW = Wv::CW, CT = Wv::CT, QPW = Wv::QPW, KPW = Wv::KPW, SPLIT = Wv::SPLIT;
  static constexpr int KS = Mma<T>::KS;
  static constexpr int NKD = D / KS;   // k-steps over features
  static constexpr int NKT = kC / KS;  // k-steps over tokens
  static constexpr int DT = D / 16;    // feature tiles
  static constexpr int ES = (int)sizeof(T);
  static constexpr int CPR = D * ES / 16;
  static constexpr int TB = kC * D * ES;  // one swizzled tile
  // Pitches (elements) of the register-written tiles. For bf16 the score and
  // delta rows are 8 bytes past a multiple of 128 bytes: the 8-byte accumulator
  // writes and the 8-byte operand reads of 16 consecutive rows then hit distinct
  // LDS banks (measured). The output staging tile keeps 16-byte aligned rows
  // for its 16-byte row reads.
  static constexpr int PP = ES == 2 ? kC + 4 : kC + 4;   // scores / Bmat
  static constexpr int PDD = ES == 2 ? D + 4 : D + 4;    // delta and the gate/mean rows
  static constexpr int PD = ES == 2 ? D + 8 : D + 4;     // output staging
  static constexpr int NTILE = AGG ? 2 : 3;                 // (Q), K, V
  static constexpr int BUF = NTILE * TB + 256;              // + g
  static constexpr int o_d = 0;                             // delta [64][PDD]
  static constexpr int d_bytes = (CCQ && !AGG) ? kC * PDD * ES : 0;
  static constexpr int o_p = o_d + d_bytes;                 // scores / Bmat [64 q][PP]
  static constexpr int p_bytes = AGG ? 0 : kC * PP * ES;
  static constexpr int o_dot = o_p + p_bytes;               // [16][PDD] gate and mean rows
  static constexpr int dot_bytes = (CCQ && !AGG) ? 16 * PDD * ES : 0;
  // sL [NW][64]; sWQ [64] float2 (gate logit w.q, mean term m_prev.q); sMv [D];
  // sRS [SPLIT][64] (partial row sums of the masked scores)
  static constexpr int o_small = o_dot + dot_bytes;
  static constexpr int small_bytes = NW * kC * 4 + kC * 8 + D * 4 + SPLIT * kC * 4;
  static constexpr int o_o = o_small + small_bytes;         // output staging [64][PD]
  static constexpr int o_bytes = AGG ? 0 : kC * PD * ES;
  static constexpr bool STAGE_O = !AGG && o_o + o_bytes + BUF <= kLds;
  static constexpr int o_buf = (o_o + (STAGE_O ? o_bytes : 0) + 15) / 16 * 16;
  static constexpr int NBUF = o_buf + 2 * BUF <= kLds ? 2 : 1;
  // bf16 CCQ: the S^T q half of the read is formed in phase 3 from the Q
  // fragments read there (Q is then read once per chunk instead of twice).
  static constexpr bool IQ = CCQ && !AGG && ES == 2 && NKD >= 2 && CT == 1;
  static constexpr int lds = o_buf + NBUF * BUF;
  static_assert(lds <= kLds, "LDS budget");
};

template <typename T, int D, int NT>
__device__ __forceinline__ void store_rows(T* __restrict__ dst, const T* s, int pitch, int nrows) {
  typedef typename Vec16<T>::type vec;
  constexpr int VN = Vec16<T>::n;
  constexpr int PER_ROW = D / VN;
  for (int i = threadIdx.x; i < nrows * PER_ROW; i += NT) {
    const int row = i / PER_ROW, cv = i - (i / PER_ROW) * PER_ROW;
    *reinterpret_cast<vec*>(dst + (size_t)row * D + cv * VN) = *reinterpret_cast<const vec*>(s + row * pitch + cv * VN);
  }
}

// Four consecutive elements (accumulator rows r = 0..3 of one lane) in one store.
template <typename T>
__device__ __forceinline__ void put4v(T* dst, const f32x4& v) {
  if constexpr (sizeof(T) == 2)
    *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  else
    *reinterpret_cast<f32x4*>(dst) = v;
}

// NATURAL fragment (k contiguous along the row) of a padded tile whose rows are
// only 8-byte aligned: two 8-byte reads for bf16.
__device__ __forceinline__ bf16x8 ld_nat8(const bf16* base, int pitch, int rc, int kstep) {
  const int g = lane_id() >> 4;
  const bf16* p = base + rc * pitch + kstep * 32 + 8 * g;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 4);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ float ld_nat8(const float* base, int pitch, int rc, int kstep) {
  return ld_kc_nat(base, pitch, rc, kstep);
}

// Decay factors 2^(l_i - l_j) of the score tile (query tile qt, key tile
// kt <= qt) for this lane's query i (cumulative log2 decay lq) and key rows
// 16 kt + 4 g + r; zero above the diagonal. Off the diagonal the factor splits
// at the tile's last key p = l_{16 kt + 15} into 2^(l_i - p) 2^(p - l_j), both
// at most 1 (five exponentials instead of sixteen). On the diagonal the
// exponent is clamped to <= 0 before the mask, so that masked entries cannot
// overflow.
__device__ __forceinline__ f32x4 decay_tile(const float* sl, float lq, int kt, int qt) {
  const int g = lane_id() >> 4, c16 = lane_id() & 15;
  const f32x4 lk = *reinterpret_cast<const f32x4*>(sl + 16 * kt + 4 * g);
  f32x4 d;
  if (kt < qt) {
    const float p = sl[16 * kt + 15];
    const float a = fast_exp2(lq - p);
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = a * fast_exp2(p - lk[r]);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) d[r] = 4 * g + r <= c16 ? fast_exp2(fminf(lq - lk[r], 0.f)) : 0.f;
  }
  return d;
}

// Decay weights of the token entries (CHAIN order, step s) this lane holds in
// k-major fragments, read from the per-token weights in LDS; the same for
// every column tile.
template <typename T>
struct DecayW {
  static constexpr int NE = sizeof(T) == 2 ? 8 : 1;
  float w[NE];
  __device__ __forceinline__ void init(const float* wt, int s) {
#pragma unroll
    for (int i = 0; i < NE; ++i) w[i] = wt[chain_k<T>(s, i)];
  }
  // From the cumulative decays instead: 2^(l_last - l_j).
  __device__ __forceinline__ void init_exp(const float* sl, float l_last, int s) {
#pragma unroll
    for (int i = 0; i < NE; ++i) w[i] = fast_exp2(l_last - sl[chain_k<T>(s, i)]);
  }
  __device__ __forceinline__ typename Mma<T>::frag apply(typename Mma<T>::frag f) const {
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int i = 0; i < 8; ++i) f[i] = (bf16)((float)f[i] * w[i]);
      return f;
    } else {
      return f * w[0];
    }
  }
};

template <typename C, bool AGG>
__device__ __forceinline__ const char* tile_k(const char* buf) { return buf + (AGG ? 0 : C::TB); }
template <typename C, bool AGG>
__device__ __forceinline__ const char* tile_v(const char* buf) { return buf + (AGG ? 1 : 2) * C::TB; }
template <typename C>
__device__ __forceinline__ const float* tile_g(const char* buf) {
  return reinterpret_cast<const float*>(buf + C::NTILE * C::TB);
}

// Per-workgroup constants of the chunk loop.
template <typename T, int D, bool CCQ, bool AGG>
struct Ctx {
  typedef Cfg<T, D, CCQ, AGG> C;
  const T* Qg;
  const T* Kg;
  const T* Vg;
  const float* Gg;
  T* Og;
  int64_t N, t_end, t_off;
  float gate_b;
  int cbase;
  TileDma<T, D, C::NW> dma;

  // Issues the DMA of one tile of the chunk at c0 into `buf`: TILE 0 = Q (not
  // in AGG), 1 = K, 2 = V, 3 = the decays.
  template <int TILE>
  __device__ __forceinline__ void issue_tile(char* buf, int64_t c0) const {
    const int nv = (int)((N - c0) < kC ? (N - c0) : kC);
    if constexpr (TILE == 0) {
      static_assert(!AGG, "no Q tile in the segment pass");
      dma.issue(buf, Qg + (size_t)c0 * D, nv);
    } else if constexpr (TILE == 1) {
      dma.issue(buf + (AGG ? 0 : C::TB), Kg + (size_t)c0 * D, nv);
    } else if constexpr (TILE == 2) {
      dma.issue(buf + (AGG ? 1 : 2) * C::TB, Vg + (size_t)c0 * D, nv);
    } else {
      if (wave_id() == 0)
        lds_dma4(buf_desc(Gg + c0, (uint32_t)(nv * 4)), lane_id() * 4, lds_addr(buf + C::NTILE * C::TB));
    }
  }
  // All tiles of the chunk at c0.
  __device__ __forceinline__ void issue(char* buf, int64_t c0) const {
    if constexpr (!AGG) issue_tile<0>(buf, c0);
    issue_tile<1>(buf, c0);
    issue_tile<2>(buf, c0);
    issue_tile<3>(buf, c0);
  }
};

// Registers carried from chunk to chunk.
template <typename T, int D, bool CCQ, bool AGG>
struct State {
  typedef Cfg<T, D, CCQ, AGG> C;
  // S[kt][ct]: rows = key features 16 kt + 4 g + r, cols = value dims cbase + 16 ct + c16.
  // M[kt][ct]: rows = features 16 kt + 4 g + r, cols = features cbase + 16 ct + c16.
  f32x4 S[C::DT][C::CT];
  f32x4 Mst[CCQ ? C::DT : 1][CCQ ? C::CT : 1];
  float mreg[C::CT];  // running key sum of column cbase + 16 ct + c16
  float lseg;         // AGG: log2 of the segment's decay product
  // The decayed state is held lazily: S_true = 2^ls S. The chunk decay is
  // folded into the weights of the new terms until ls would drop below
  // -kLazy, and only then multiplied into S (bounded weights, no overflow).
  float ls;
  int64_t t_prev;     // chunk whose outputs wait in the staging tile
};

// One chunk. `cur` holds this chunk's tiles (DMA issued a chunk earlier when
// double-buffered); `nxt` receives the next chunk's tiles.
template <typename T, int D, bool CCQ, bool AGG>
__device__ __forceinline__ void chunk_step(const Ctx<T, D, CCQ, AGG>& x, State<T, D, CCQ, AGG>& st, char* cur,
                                           char* nxt, char* work, int64_t t0) {
  typedef Cfg<T, D, CCQ, AGG> C;
  typedef Mma<T> M;
  typedef typename M::frag frag;
  constexpr int NW = C::NW, NT = NW * 64, CT = C::CT, DT = C::DT, CPR = C::CPR;
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int64_t N = x.N;
  const int nvalid = (int)((N - t0) < kC ? (N - t0) : kC);
  const int cbase = x.cbase;
  const float gate_b = x.gate_b;
  T* sD = reinterpret_cast<T*>(work + C::o_d);
  T* sP = reinterpret_cast<T*>(work + C::o_p);
  T* sDot = reinterpret_cast<T*>(work + C::o_dot);
  float* sLw = reinterpret_cast<float*>(work + C::o_small) + w * kC;
  float2* sWQ = reinterpret_cast<float2*>(work + C::o_small + NW * kC * 4);
  float* sMv = reinterpret_cast<float*>(work + C::o_small + NW * kC * 4 + kC * 8);
  float* sRS = sMv + D;
  T* sO = reinterpret_cast<T*>(work + C::o_o);
  T* __restrict__ Og = x.Og;
  f32x4 (&S)[DT][CT] = st.S;
  auto& Mst = st.Mst;
  float (&mreg)[CT] = st.mreg;
  float& lseg = st.lseg;
  int64_t& t_prev = st.t_prev;
  (void)gate_b;
  (void)sWQ;
  (void)sRS;
  (void)sO;
  (void)Og;
  (void)t_prev;

  if constexpr (C::NBUF == 1) {
    lds_barrier();  // the previous chunk is done with the single buffer
    x.issue(cur, t0);
  }
  wait_vmem();
  lds_barrier();  // this chunk's tiles landed; the previous chunk is finished everywhere
  // The next chunk's DMA and the previous chunk's output stores are spread over
  // the phases of this one: issued together, the vector memory instructions of
  // all waves queue behind each other in the address unit.
  const bool pre = C::NBUF == 2 && t0 + kC < x.t_end;
  const int64_t tn = t0 + kC;
  (void)pre;
  (void)tn;
  if constexpr (AGG) {
    if (pre) {
      x.template issue_tile<1>(nxt, tn);
      x.template issue_tile<3>(nxt, tn);
    }
  } else if constexpr (!CCQ) {
    if constexpr (C::STAGE_O) {
      if (t_prev >= 0) store_rows<T, D, NT>(Og + (size_t)t_prev * D, sO, C::PD, kC);
    }
    if (pre) {
      x.template issue_tile<0>(nxt, tn);
      x.template issue_tile<3>(nxt, tn);
    }
  }
    const char* Kt = tile_k<C, AGG>(cur);
    const char* Vt = tile_v<C, AGG>(cur);

    // cumulative log2 decay of this chunk (each wave keeps a private copy)
    float l_last, l_mine;  // chunk total; this lane's token (lane = token)
    {
      // log2 g in hardware (g in (0, 1]; g = 0 gives -inf, clamped)
      float x = l < nvalid ? fmaxf(__builtin_amdgcn_logf(tile_g<C>(cur)[l]), -200.f) : 0.f;
      x = wave_scan_incl(x);
      l_mine = x;
      l_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), kC - 1));
      sLw[l] = x;
    }
    __builtin_amdgcn_wave_barrier();

    frag KTc[CCQ ? CT : 1][CCQ ? C::NKT : 1];  // K^T of this wave's columns (CCQ)
    if constexpr (CCQ) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) KTc[ct][s] = tl_kmaj_t<CPR, T>(Kt, s, cbase + 16 * ct);
    }
    if constexpr (AGG) {
      if (pre) x.template issue_tile<2>(nxt, tn);
    }

    // bf16 CCQ (IQ): bf16 snapshot of S and S^T q per query tile, from phase 3
    // to the read
    frag Sc_iq[C::IQ ? C::NKD : 1];
    f32x4 Scol_iq[C::IQ ? DT : 1];
    f32x4 iq[C::IQ ? 4 : 1];
    (void)Sc_iq;
    (void)Scol_iq;
    (void)iq;
    if constexpr (!AGG) {
      const char* Qt = cur;
      // ---- phase 1: owned (query tile, key tile) pairs: raw scores; for CCQ the
      //      masked scores, their partial row sums and the gate/mean terms, for
      //      the plain read the decayed scores
      typedef Waves<D> Wv;
      f32x4 Pr[C::QPW][C::KPW];
#pragma unroll
      for (int qi = 0; qi < C::QPW; ++qi) {
        const int qt = Wv::qtile(w, qi);
        const int q = 16 * qt + c16;
        frag QF[C::NKD];
#pragma unroll
        for (int ks = 0; ks < C::NKD; ++ks) QF[ks] = tl_nat_t<CPR, T>(Qt, q, ks);
        // bf16: all key fragments of the owned tiles are read up front (one LDS
        // round trip); fp32 fragments are single floats, read where used.
        constexpr bool HOIST = sizeof(T) == 2;
        frag KF[HOIST ? C::KPW : 1][HOIST ? C::NKD : 1];
        if constexpr (HOIST) {
#pragma unroll
          for (int j = 0; j < C::KPW; ++j) {
            const int kt = Wv::ktile(w, j);
            if (kt <= qt) {
#pragma unroll
              for (int ks = 0; ks < C::NKD; ++ks) KF[j][ks] = tl_nat_t<CPR, T>(Kt, 16 * kt + c16, ks);
            }
          }
        }
        const bool dq_owner = CCQ && Wv::part(w) == C::SPLIT - 1;
        frag DQ[CCQ && HOIST ? C::NKD : 1];
        if constexpr (CCQ && HOIST) {
          if (dq_owner) {
#pragma unroll
            for (int ks = 0; ks < C::NKD; ++ks) DQ[ks] = ld_nat8(sDot, C::PDD, c16, ks);
          }
        }
#pragma unroll
        for (int j = 0; j < C::KPW; ++j) {
          const int kt = Wv::ktile(w, j);
          Pr[qi][j] = zero4();
          if (kt <= qt) {
#pragma unroll
            for (int ks = 0; ks < C::NKD; ++ks)
              Pr[qi][j] = M::mma(HOIST ? KF[HOIST ? j : 0][HOIST ? ks : 0] : tl_nat_t<CPR, T>(Kt, 16 * kt + c16, ks),
                                 QF[ks], Pr[qi][j]);
            if (kt == qt) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * g + r > c16) Pr[qi][j][r] = 0.f;
            }
          }
        }
        T* prow = sP + q * C::PP;
        if constexpr (CCQ) {
          if (dq_owner) {
            f32x4 dq = zero4();
#pragma unroll
            for (int ks = 0; ks < C::NKD; ++ks)
              dq = M::mma(HOIST ? DQ[HOIST ? ks : 0] : ld_nat8(sDot, C::PDD, c16, ks), QF[ks], dq);
            const float wq = __shfl(dq[0] + dq[1], c16);
            const float mq = __shfl(dq[2] + dq[3], c16);
            if (g == 0) sWQ[q] = make_float2(wq, mq);
          }
          float rs = 0.f;
#pragma unroll
          for (int j = 0; j < C::KPW; ++j)
#pragma unroll
            for (int r = 0; r < 4; ++r) rs += Pr[qi][j][r];
          rs = group_sum(rs);
          if (g == 0) sRS[Wv::part(w) * kC + q] = rs;
#pragma unroll
          for (int j = 0; j < C::KPW; ++j) put4v<T>(prow + 16 * Wv::ktile(w, j) + 4 * g, Pr[qi][j]);
        } else {
          const float lq = sLw[q];
#pragma unroll
          for (int j = 0; j < C::KPW; ++j) {
            const int kt = Wv::ktile(w, j);
            f32x4 v = zero4();
            if (kt <= qt) v = Pr[qi][j] * decay_tile(sLw, lq, kt, qt);
            put4v<T>(prow + 16 * kt + 4 * g, v);
          }
        }
      }
      lds_barrier();
      if constexpr (CCQ) {
        if constexpr (C::STAGE_O) {
          if (t_prev >= 0) store_rows<T, D, NT>(Og + (size_t)t_prev * D, sO, C::PD, kC);
        }
        if (pre) x.template issue_tile<2>(nxt, tn);
      } else {
        if (pre) {
          x.template issue_tile<1>(nxt, tn);
          x.template issue_tile<2>(nxt, tn);
        }
      }

      if constexpr (CCQ) {
        // ---- phase 3: delta^T for this wave's feature columns,
        //   delta_i = -alpha_i (M_prev q_i + sum_j k_j P_ij) + beta_i (sum_{j<=i} k_j + m_prev)
        // (P masked to j <= i). The prefix sum of keys is a product with the
        // lower-triangular ones matrix, built in registers.
        // gate and mean weights, lane = query (count t = t0 + lane + 1); each
        // query tile picks its own by a lane permute
        float alpha_l, beta_l;
        {
          const float2 wm = sWQ[l];
          float rs = sRS[l];
          if constexpr (C::SPLIT > 1) rs += sRS[kC + l];
          const float lam = __builtin_amdgcn_rcpf(1.f + fast_exp2(-(wm.x + gate_b) * kLog2eF));
          const float inv_t = __builtin_amdgcn_rcpf((float)(t0 + x.t_off) + (float)(l + 1));
          alpha_l = lam * inv_t;
          beta_l = alpha_l * (wm.y + rs) * inv_t;
        }
        // bf16 diagonal blocks of the mask (tokens 32 s' .. 32 s' + 31 against
        // query tile qt with s' = qt / 2): tri0 for even qt, tri1 for odd qt
        frag ones, tri0, tri1;
        if constexpr (sizeof(T) == 2 && !C::IQ) {
#pragma unroll
          for (int i = 0; i < 8; ++i) {
            const int j = chain_k<T>(0, i);
            ones[i] = (bf16)1.f;
            tri0[i] = j <= c16 ? (bf16)1.f : (bf16)0.f;
            tri1[i] = j <= 16 + c16 ? (bf16)1.f : (bf16)0.f;
          }
        }
        (void)ones;
        (void)tri0;
        (void)tri1;
        if constexpr (C::IQ) {
          // S^T q of the read, with the bf16 snapshot of S (unchanged until the update)
#pragma unroll
          for (int kt = 0; kt < DT; ++kt) Scol_iq[kt] = S[kt][0];
#pragma unroll
          for (int s2 = 0; s2 < C::NKD; ++s2) Sc_iq[s2] = M::chain(Scol_iq, s2);
        }
        for (int ct = 0; ct < CT; ++ct) {  // (one column tile per wave)
          const int c0 = cbase + 16 * ct;
          // M_prev as the operand precision (bf16 for bf16 inputs): its rounding
          // perturbs q_clean by at most lambda |k|^2 2^-9 |q|, the size of the
          // rounding of q itself for unit-norm keys.
          frag Mh[C::NKD];
          {
            f32x4 Mcol[DT];
#pragma unroll
            for (int kt = 0; kt < DT; ++kt) Mcol[kt] = Mst[kt][ct];
#pragma unroll
            for (int s = 0; s < C::NKD; ++s) Mh[s] = M::chain(Mcol, s);
          }
          float mprev[4];
#pragma unroll
          for (int r = 0; r < 4; ++r) mprev[r] = sMv[c0 + 4 * g + r];
          auto delta_tile = [&](const int qt) {
            const int q = 16 * qt + c16;
            // bf16: every operand of this query tile is requested before the
            // first product (one LDS round trip); fp32 operands are read where used.
            constexpr bool HOIST = sizeof(T) == 2;
            frag qf[HOIST ? C::NKD : 1], pf[HOIST ? C::NKT : 1];
            if constexpr (HOIST) {
#pragma unroll
              for (int s = 0; s < C::NKD; ++s) qf[s] = tl_chain_t<CPR, T>(Qt, q, s);
#pragma unroll
              for (int s = 0; s < C::NKT; ++s) pf[s] = ld_kc_chain(sP, C::PP, q, s);
            }
            const float alpha = __shfl(alpha_l, q);
            const float beta = __shfl(beta_l, q);
            if constexpr (HOIST) __builtin_amdgcn_sched_barrier(0);
            f32x4 mqv = zero4();
#pragma unroll
            for (int s = 0; s < C::NKD; ++s)
              mqv = M::mma(Mh[s], HOIST ? qf[HOIST ? s : 0] : tl_chain_t<CPR, T>(Qt, q, s), mqv);
            if constexpr (C::IQ) {
              f32x4 a = zero4();
#pragma unroll
              for (int s = 0; s < C::NKD; ++s) a = M::mma(Sc_iq[s], qf[HOIST ? s : 0], a);
              iq[qt] = a;
            }
            f32x4 kp = zero4(), kc = zero4();
#pragma unroll
            for (int s = 0; s < C::NKT; ++s)
              if ((s * M::KS) / 16 <= qt) {
                kp = M::mma(KTc[ct][s], HOIST ? pf[HOIST ? s : 0] : ld_kc_chain(sP, C::PP, q, s), kp);
                frag tri;
                if constexpr (C::IQ) {
                  tri = tri_frag<T>(s, q);  // (qt is a constant here: unrolled)
                } else if constexpr (HOIST) {
                  // whole 32-token blocks below the diagonal are all ones
                  tri = (s + 1) * M::KS <= 16 * qt ? ones : ((qt & 1) ? tri1 : tri0);
                } else {
                  tri = tri_frag<T>(s, q);
                }
                kc = M::mma(KTc[ct][s], tri, kc);
              }
            f32x4 v;
#pragma unroll
            for (int r = 0; r < 4; ++r) v[r] = beta * (kc[r] + mprev[r]) - alpha * (mqv[r] + kp[r]);
            put4v<T>(sD + q * C::PDD + c0 + 4 * g, v);
            if constexpr (C::IQ) __builtin_amdgcn_sched_barrier(0);  // one query tile at a time
          };
          if constexpr (C::IQ) {
#pragma unroll
            for (int qt = 0; qt < 4; ++qt) delta_tile(qt);
          } else {
#pragma unroll 1
            for (int qt = 0; qt < 4; ++qt) delta_tile(qt);
          }
        }
        lds_barrier();  // delta complete; masked scores consumed

        // ---- phase 4: owned score tiles with the cleaned query, decayed
#pragma unroll
        for (int qi = 0; qi < C::QPW; ++qi) {
          const int qt = Wv::qtile(w, qi);
          const int q = 16 * qt + c16;
          frag DF[C::NKD];
#pragma unroll
          for (int ks = 0; ks < C::NKD; ++ks) DF[ks] = ld_nat8(sD, C::PDD, q, ks);
          constexpr bool HOIST = sizeof(T) == 2;
          frag KF[HOIST ? C::KPW : 1][HOIST ? C::NKD : 1];
          if constexpr (HOIST) {
#pragma unroll
            for (int j = 0; j < C::KPW; ++j) {
              const int kt = Wv::ktile(w, j);
              if (kt <= qt) {
#pragma unroll
                for (int ks = 0; ks < C::NKD; ++ks) KF[j][ks] = tl_nat_t<CPR, T>(Kt, 16 * kt + c16, ks);
              }
            }
          }
          const float lq = sLw[q];
          T* prow = sP + q * C::PP;
#pragma unroll
          for (int j = 0; j < C::KPW; ++j) {
            const int kt = Wv::ktile(w, j);
            f32x4 acc = Pr[qi][j];
            f32x4 v = zero4();
            if (kt <= qt) {
#pragma unroll
              for (int ks = 0; ks < C::NKD; ++ks)
                acc = M::mma(HOIST ? KF[HOIST ? j : 0][HOIST ? ks : 0] : tl_nat_t<CPR, T>(Kt, 16 * kt + c16, ks), DF[ks],
                             acc);
              v = acc * decay_tile(sLw, lq, kt, qt);
            }
            put4v<T>(prow + 16 * kt + 4 * g, v);
          }
        }
        lds_barrier();  // decayed scores complete
        // (K after phase 4 as well: a register reload there would also wait for it)
        if (pre) {
          x.template issue_tile<0>(nxt, tn);
          x.template issue_tile<1>(nxt, tn);
          x.template issue_tile<3>(nxt, tn);
        }
      }

      // ---- phase 5: outputs of this wave's value columns (query tile outer, so Q and
      //      delta fragments are read once)
      frag Sc[CT][C::NKD], Vf[CT][C::NKT];
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        if constexpr (C::IQ) {
#pragma unroll
          for (int s = 0; s < C::NKD; ++s) Sc[ct][s] = Sc_iq[s];
        } else {
          f32x4 Scol[DT];
#pragma unroll
          for (int kt = 0; kt < DT; ++kt) Scol[kt] = S[kt][ct];
#pragma unroll
          for (int s = 0; s < C::NKD; ++s) Sc[ct][s] = M::chain(Scol, s);
        }
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) Vf[ct][s] = tl_kmaj_t<CPR, T>(Vt, s, cbase + 16 * ct);
      }
      // Output of query q for this wave's column tiles.
      auto emit = [&](int q, const f32x4 (&acc)[CT], const f32x4 (&inter)[CT], float lq) {
        const float bq = fast_exp2(lq + st.ls);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          const int c0 = cbase + 16 * ct;
          const f32x4 o = acc[ct] + bq * inter[ct];
          if constexpr (C::STAGE_O) {
            put4v<T>(sO + q * C::PD + c0 + 4 * g, o);
          } else if (q < nvalid) {
            put4v<T>(Og + (size_t)(t0 + q) * D + c0 + 4 * g, o);
          }
        }
      };
      if constexpr (sizeof(T) == 2 && C::NKD >= 2 && C::NKT == 2) {
        // Software pipeline over half query tiles (k-steps 0 .. NKD/2-1, then
        // the rest): the LDS operands of step i+1 are requested before the
        // products of step i, with the register footprint of one whole tile.
        constexpr int HS = C::NKD / 2;
        struct Ops {
          frag q[HS], d[HS], p;
          float lq;
        };
        auto load = [&](int step, Ops& o) {
          const int qt = step >> 1, h = step & 1, q = 16 * qt + c16;
#pragma unroll
          for (int i = 0; i < HS; ++i) {
            if constexpr (!C::IQ) o.q[i] = tl_chain_t<CPR, T>(Qt, q, HS * h + i);
            if constexpr (CCQ) o.d[i] = ld_kc_chain(sD, C::PDD, q, HS * h + i);
          }
          if ((h * M::KS) / 16 <= qt) o.p = ld_kc_chain(sP, C::PP, q, h);
          if (h == 1) o.lq = sLw[q];
        };
        Ops ops[2];
        load(0, ops[0]);
        f32x4 inter[CT], acc[CT];
#pragma unroll
        for (int step = 0; step < 8; ++step) {
          const int qt = step >> 1, h = step & 1;
          if (step + 1 < 8) load(step + 1, ops[(step + 1) & 1]);
          __builtin_amdgcn_sched_barrier(0);
          const Ops& o = ops[step & 1];
          if (h == 0) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              inter[ct] = C::IQ ? iq[C::IQ ? qt : 0] : zero4();
              acc[ct] = zero4();
            }
          }
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
#pragma unroll
            for (int i = 0; i < HS; ++i) {
              if constexpr (!C::IQ) inter[ct] = M::mma(Sc[ct][HS * h + i], o.q[i], inter[ct]);
              if constexpr (CCQ) inter[ct] = M::mma(Sc[ct][HS * h + i], o.d[i], inter[ct]);
            }
            if ((h * M::KS) / 16 <= qt) acc[ct] = M::mma(Vf[ct][h], o.p, acc[ct]);
          }
          if (h == 1) emit(16 * qt + c16, acc, inter, o.lq);
        }
      } else {
#pragma unroll 1
        for (int qt = 0; qt < 4; ++qt) {
          const int q = 16 * qt + c16;
          f32x4 inter[CT], acc[CT];
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) {
            inter[ct] = zero4();
            acc[ct] = zero4();
          }
#pragma unroll
          for (int s = 0; s < C::NKD; ++s) {
            const frag qf = tl_chain_t<CPR, T>(Qt, 16 * qt + c16, s);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) inter[ct] = M::mma(Sc[ct][s], qf, inter[ct]);
            if constexpr (CCQ) {
              const frag df = ld_kc_chain(sD, C::PDD, q, s);
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) inter[ct] = M::mma(Sc[ct][s], df, inter[ct]);
            }
          }
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) {
            if ((s * M::KS) / 16 <= qt) {
              const frag pf = ld_kc_chain(sP, C::PP, q, s);
#pragma unroll
              for (int ct = 0; ct < CT; ++ct) acc[ct] = M::mma(Vf[ct][s], pf, acc[ct]);
            }
          }
          emit(q, acc, inter, sLw[q]);
        }
      }
      t_prev = t0;
    }

    // ---- state updates: S <- 2^l_last S + K^T (w V), M += K^T K, m += sum K,
    //      with S held as 2^ls S:
    //        lazy : ls <- ls + l_last,  S <- S + K^T (2^(-ls_prev - l_j) V)
    //        eager: S <- 2^(ls + l_last) S + K^T (2^(l_last - l_j) V),  ls <- 0
    //      (the lazy weights stay below 2^kLazy)
    {
      const float ls_next = st.ls + l_last;
      float wb;
      // (the segment pass, sized for 128 registers, always scales eagerly)
      if (AGG || ls_next < -kLazy) {
        const float b = fast_exp2(ls_next);
#pragma unroll
        for (int kt = 0; kt < DT; ++kt)
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) S[kt][ct] *= b;
        st.ls = 0.f;
        wb = l_last;
      } else {
        wb = -st.ls;
        st.ls = ls_next;
      }
      // per-token weights replace this wave's cumulative decays in LDS
      if constexpr (!AGG) {
        sLw[l] = fast_exp2(wb - l_mine);
        __builtin_amdgcn_wave_barrier();
      }
      frag Vw[CT][C::NKT];
#pragma unroll
      for (int s = 0; s < C::NKT; ++s) {
        DecayW<T> dw;
        if constexpr (AGG)
          dw.init_exp(sLw, l_last, s);
        else
          dw.init(sLw, s);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) Vw[ct][s] = dw.apply(tl_kmaj_t<CPR, T>(Vt, s, cbase + 16 * ct));
      }
      if constexpr (sizeof(T) == 2) {
        // K^T fragments one feature tile ahead of their products, so the LDS
        // latency of tile kt+1 overlaps the matrix-core work of tile kt.
        frag kfb[2][C::NKT];
#pragma unroll
        for (int s = 0; s < C::NKT; ++s) kfb[0][s] = tl_kmaj_t<CPR, T>(Kt, s, 0);
#pragma unroll
        for (int kt = 0; kt < DT; ++kt) {
          if (kt + 1 < DT) {
#pragma unroll
            for (int s = 0; s < C::NKT; ++s) kfb[(kt + 1) & 1][s] = tl_kmaj_t<CPR, T>(Kt, s, 16 * (kt + 1));
          }
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) {
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              S[kt][ct] = M::mma(kfb[kt & 1][s], Vw[ct][s], S[kt][ct]);
              if constexpr (CCQ) Mst[kt][ct] = M::mma(kfb[kt & 1][s], KTc[ct][s], Mst[kt][ct]);
            }
          }
          __builtin_amdgcn_sched_barrier(0);
        }
      } else {
#pragma unroll
        for (int kt = 0; kt < DT; ++kt) {
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) {
            const frag kf = tl_kmaj_t<CPR, T>(Kt, s, 16 * kt);
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) {
              S[kt][ct] = M::mma(kf, Vw[ct][s], S[kt][ct]);
              if constexpr (CCQ) Mst[kt][ct] = M::mma(kf, KTc[ct][s], Mst[kt][ct]);
            }
          }
        }
      }
      if constexpr (CCQ) {
        // column sums of K: ones^T K on the matrix core (every row of the tile
        // holds the sum of its column)
        frag ones;
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;
        } else {
          ones = 1.f;
        }
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) {
          f32x4 cs = zero4();
#pragma unroll
          for (int s = 0; s < C::NKT; ++s) cs = M::mma(ones, KTc[ct][s], cs);
          mreg[ct] += cs[0];
          if constexpr (!AGG) {
            if (g == 0) {
              const int col = cbase + 16 * ct + c16;
              const T hi = from_f32<T>(mreg[ct]);
              sMv[col] = mreg[ct];
              sDot[2 * C::PDD + col] = hi;
              sDot[3 * C::PDD + col] = from_f32<T>(mreg[ct] - to_f32(hi));
            }
          }
        }
      }
      lseg += l_last;
    }
}

// The bf16 segment-state pass is sized for two workgroups per CU (at D = 128:
// four waves per SIMD, so at most 128 VGPRs).
template <typename T, int D, bool CCQ, bool AGG>
__global__ __launch_bounds__(Waves<D>::NW * 64, AGG && sizeof(T) == 2 ? 4 : 1) void lin_kernel(Args a) {
  typedef Cfg<T, D, CCQ, AGG> C;
  constexpr int NW = C::NW, NT = NW * 64, CT = C::CT, DT = C::DT;

  // Separate arrays: the two DMA buffers and the register-written tiles.
  __shared__ __attribute__((aligned(16))) char sBuf0[C::BUF];
  __shared__ __attribute__((aligned(16))) char sBuf1[C::NBUF == 2 ? C::BUF : 16];
  __shared__ __attribute__((aligned(16))) char sWork[C::o_buf];

  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int bh = blockIdx.y, p = blockIdx.x;
  const int h = bh % a.H;
  const int64_t N = a.N;
  const int64_t t_begin = (int64_t)p * a.seg_len;
  const int64_t t_end = N < t_begin + a.seg_len ? N : t_begin + a.seg_len;

  Ctx<T, D, CCQ, AGG> x;
  x.Qg = reinterpret_cast<const T*>(a.q) + (size_t)bh * N * D;
  x.Kg = reinterpret_cast<const T*>(a.k) + (size_t)bh * N * D;
  x.Vg = reinterpret_cast<const T*>(a.v) + (size_t)bh * N * D;
  x.Gg = a.g + (size_t)bh * N;
  x.Og = reinterpret_cast<T*>(a.out) + (size_t)bh * N * D;
  x.N = N;
  x.t_end = t_end;
  x.t_off = a.t_off;
  x.gate_b = CCQ ? a.bl[h] : 0.f;
  x.cbase = w * C::CW;
  x.dma.init();
  const int cbase = x.cbase;
  T* sDot = reinterpret_cast<T*>(sWork + C::o_dot);
  float* sMv = reinterpret_cast<float*>(sWork + C::o_small + NW * kC * 4 + kC * 8);
  T* sO = reinterpret_cast<T*>(sWork + C::o_o);
  (void)sDot;
  (void)sMv;
  (void)sO;

  State<T, D, CCQ, AGG> st;
#pragma unroll
  for (int kt = 0; kt < DT; ++kt)
#pragma unroll
    for (int ct = 0; ct < CT; ++ct) {
      st.S[kt][ct] = zero4();
      if constexpr (CCQ) st.Mst[kt][ct] = zero4();
    }
#pragma unroll
  for (int ct = 0; ct < CT; ++ct) st.mreg[ct] = 0.f;
  st.lseg = 0.f;
  st.ls = 0.f;
  st.t_prev = -1;

  if constexpr (C::NBUF == 2) {
    if (t_begin < t_end) x.issue(sBuf0, t_begin);
  }

  if constexpr (!AGG) {
    // state at the segment start (exclusive prefix written by the segment scan)
    if (a.has_init) {
      const float* blk = a.agg + ((size_t)bh * a.P + (size_t)a.R * p) * a.sfl;
#pragma unroll
      for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * kt + 4 * g + r, col = cbase + 16 * ct + c16;
            st.S[kt][ct][r] = blk[row * D + col];
            if constexpr (CCQ) st.Mst[kt][ct][r] = blk[D * D + 1 + row * D + col];
          }
      if constexpr (CCQ) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) st.mreg[ct] = blk[2 * D * D + 1 + cbase + 16 * ct + c16];
      }
    }
  }
  if constexpr (CCQ && !AGG) {
    // rows 0/1: gate weights (hi/lo); rows 2/3: running key sum (hi/lo); others 0
    for (int i = threadIdx.x; i < 16 * C::PDD; i += NT) {
      const int row = i / C::PDD, col = i - (i / C::PDD) * C::PDD;
      float v = 0.f;
      if (col < D && row < 2) {
        const float wv = a.wl[(size_t)h * D + col];
        const T hi = from_f32<T>(wv);
        v = row == 0 ? to_f32(hi) : wv - to_f32(hi);
      }
      if (row < 2 || row >= 4 || col >= D) sDot[i] = from_f32<T>(v);
    }
    if (g == 0) {
#pragma unroll
      for (int ct = 0; ct < CT; ++ct) {
        const int col = cbase + 16 * ct + c16;
        const T hi = from_f32<T>(st.mreg[ct]);
        sMv[col] = st.mreg[ct];
        sDot[2 * C::PDD + col] = hi;
        sDot[3 * C::PDD + col] = from_f32<T>(st.mreg[ct] - to_f32(hi));
      }
    }
  }

  // The tile DMA is invisible to the compiler (inline asm), so the buffer of a
  // chunk can be chosen at run time without extra waits.
  int it = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kC, ++it) {
    char* cur = (C::NBUF == 2 && (it & 1)) ? sBuf1 : sBuf0;
    char* nxt = (C::NBUF == 2 && !(it & 1)) ? sBuf1 : sBuf0;
    chunk_step<T, D, CCQ, AGG>(x, st, cur, nxt, sWork, t0);
  }

  if constexpr (C::STAGE_O) {
    lds_barrier();
    if (st.t_prev >= 0) {
      const int nv = (int)((N - st.t_prev) < kC ? (N - st.t_prev) : kC);
      store_rows<T, D, NT>(x.Og + (size_t)st.t_prev * D, sO, C::PD, nv);
    }
  }

  if constexpr (!AGG) {
    // the workgroup of the last segment holds the state after the last token
    if (a.st_out && p == (int)gridDim.x - 1) {
      float* so = a.st_out + (size_t)bh * (D * D + (CCQ ? D * D + D : 0));
      const float sfin = exp2f(st.ls);
#pragma unroll
      for (int kt = 0; kt < DT; ++kt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int row = 16 * kt + 4 * g + r, col = cbase + 16 * ct + c16;
            so[row * D + col] = st.S[kt][ct][r] * sfin;
            if constexpr (CCQ) so[D * D + row * D + col] = st.Mst[kt][ct][r];
          }
      if constexpr (CCQ) {
        if (g == 0) {
#pragma unroll
          for (int ct = 0; ct < CT; ++ct) so[2 * D * D + cbase + 16 * ct + c16] = st.mreg[ct];
        }
      }
    }
  }

  if constexpr (AGG) {
    float* blk = a.agg + ((size_t)bh * a.P + p) * a.sfl;
    const float sfin = exp2f(st.ls);
#pragma unroll
    for (int kt = 0; kt < DT; ++kt)
#pragma unroll
      for (int ct = 0; ct < CT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * kt + 4 * g + r, col = cbase + 16 * ct + c16;
          blk[row * D + col] = st.S[kt][ct][r] * sfin;
          if constexpr (CCQ) blk[D * D + 1 + row * D + col] = st.Mst[kt][ct][r];
        }
    if (w == 0 && l == 0) blk[D * D] = exp2f(st.lseg);
    if constexpr (CCQ) {
      if (g == 0) {
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) blk[2 * D * D + 1 + cbase + 16 * ct + c16] = st.mreg[ct];
      }
    }
  }
}

// Scan over the sub-segment state blocks of every sequence, in a fixed order.
// Blocks 0 .. nsub-1 hold the states of consecutive sub-segments (R per
// segment) on entry; block R p becomes the state at the start of segment p:
//   S_run <- G_q S_run + S_q,  M_run <- M_run + M_q,  m_run <- m_run + m_q
// over sub-segments q (from zero, or from the caller's initial state [S | M |
// m], which has no decay slot), with G_q the decay product of sub-segment q
// (left in place).
__global__ __launch_bounds__(256) void scan_kernel(float* __restrict__ agg, int slots, int nsub, int R, int sfl,
                                                   int D, int ccq, const float* __restrict__ init) {
  const int bh = blockIdx.y;
  const int e = blockIdx.x * 256 + threadIdx.x;
  const int nS = D * D;
  const int nTot = ccq ? 2 * D * D + 1 + D : D * D + 1;
  if (e >= nTot || e == nS) return;
  float* base = agg + (size_t)bh * slots * sfl;
  float run = init ? init[(size_t)bh * (nTot - 1) + (e < nS ? e : e - 1)] : 0.f;
  for (int q = 0; q < nsub; ++q) {
    float* xp = base + (size_t)q * sfl + e;
    const float t = *xp;
    if (q % R == 0) *xp = run;
    run = e < nS ? base[(size_t)q * sfl + nS] * run + t : run + t;
  }
  base[(size_t)nsub * sfl + e] = run;
}

template <typename T, int D, bool CCQ, bool AGG>
static hipError_t launch_one(const Args& a, unsigned gx, unsigned gy, hipStream_t st) {
  typedef Cfg<T, D, CCQ, AGG> C;
  hipLaunchKernelGGL((lin_kernel<T, D, CCQ, AGG>), dim3(gx, gy), dim3(C::NW * 64), 0, st, a);
  return hipGetLastError();
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
  a.sfl = (int)lin_state_floats(D, CCQ);
  a.has_init = 0;
  a.R = (int)L.R;
  a.P = (int)(L.R * L.P);  // state blocks per (b,h)
  a.t_off = L.state_in ? L.t_in : 0;
  a.st_out = L.state_out;
  const unsigned BH = (unsigned)(L.B * L.H);
  if (L.P > 1 || L.state_in) {
    // sub-segment states of segments 0 .. P-2, then their prefixes (from the
    // initial state when there is one)
    const int nsub = (int)(L.R * (L.P - 1));
    a.seg_len = (int)(L.seg_len / L.R);
    hipError_t e;
    if (nsub > 0 && (e = launch_one<T, D, CCQ, true>(a, (unsigned)nsub, BH, st)) != hipSuccess) return e;
    const int n = CCQ ? 2 * D * D + 1 + D : D * D + 1;
    hipLaunchKernelGGL(scan_kernel, dim3((unsigned)((n + 255) / 256), BH), dim3(256), 0, st, L.agg, a.P, nsub, a.R,
                       a.sfl, D, CCQ ? 1 : 0, L.state_in);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    a.has_init = 1;
  }
  a.seg_len = (int)L.seg_len;
  if constexpr (sizeof(T) == 2 && D == 128 && CCQ) {
    CcqPipeLaunch cp;
    cp.q = L.q;
    cp.k = L.k;
    cp.v = L.v;
    cp.g = L.g;
    cp.w_lambda = L.w_lambda;
    cp.b_lambda = L.b_lambda;
    cp.out = L.out;
    cp.agg = a.has_init ? L.agg : nullptr;
    cp.B = L.B;
    cp.H = L.H;
    cp.N = L.N;
    cp.P = L.P;
    cp.seg_len = L.seg_len;
    cp.blocks = a.P;
    cp.R = a.R;
    cp.sfl = a.sfl;
    cp.t_off = a.t_off;
    cp.state_out = L.state_out;
    return ccq_pipe_launch(cp, st);
  }
  return launch_one<T, D, CCQ, false>(a, (unsigned)L.P, BH, st);
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
  if (L.chunk == 32) return linattn_c32_launch(L, st);
  if (L.bf16) return L.ccq ? lin::launch_t<bf16, true>(L, st) : lin::launch_t<bf16, false>(L, st);
  return L.ccq ? lin::launch_t<float, true>(L, st) : lin::launch_t<float, false>(L, st);
}

}  // namespace lm
