// gma_bf16.hip -- Gaussian Mixture Attention forward for bf16 inputs with
// d = dv in {32, 64} and up to 128 mixture components (padded to 64 or 128).
//
// Method ("Gaussian Mixture Attention: Linear-Time Sequence Mixing via
// Probabilistic Latent Routing", Method -> core mechanism and variants):
// responsibilities gamma(x) = p(z = k | x) of diagonal-Gaussian components for
// every query and key row; keys write Vtil = Gamma_K^T V, Z = Gamma_K^T 1;
// queries read O = Gamma_Q Vtil / (Gamma_Q Z + eps), causally by prefix sums.
//
// Workgroup of four waves per (sequence, segment), two workgroups per CU (at
// most 80 KB of LDS each). Per 64-token chunk:
//  1. Routing logits L^T = W [x | x*x]^T + c as MFMA, components split across
//     the waves (each wave keeps its W rows in registers); one lane holds one
//     token, so the softmax over a wave's components is in-lane plus two
//     cross-row lane swaps. The wave-local max and sum go to LDS.
//  2. After one barrier every wave rescales its exponentials to the posterior
//     (combining the four waves' max and sum for its tokens) and writes the
//     responsibilities Gamma_K, Gamma_Q (bf16) to LDS.
//  3. Read, split by tokens: wave w owns query tile w and computes
//     O^T = Vtil^T Gamma_Q^T (state snapshot in LDS) + V^T A^T with the masked
//     intra-chunk affinity A^T = Gamma_K Gamma_Q^T. Update, split by
//     components: [Vtil | Z] += Gamma_K^T [V | 1] into fp32 registers.
//  4. The bf16 snapshot of the state is refreshed; the next chunk's x*x
//     features are formed once per token (each wave squares the rows its own
//     DMA brought in).
// Q/K/V tiles arrive by direct global->LDS DMA into XOR-swizzled tiles, issued
// a phase ahead of their use. In the causal form over several segments, the
// segment pass (AGG_G) stores each chunk's Gamma_K tile as it sits in LDS and
// the causal pass (CAUSAL_G) brings it back by the same DMA in place of K:
// steps 1 and 2 then route the queries only.
#include "mfma.hpp"
#include "gma.hpp"

namespace lm {
namespace gma {
namespace fast {

// XOR swizzle of the 16-byte chunks of row r in a tile of CPR chunks per row,
// for the access shapes used on these tiles: 16-byte row gathers of 16
// consecutive rows, transpose reads of 8 consecutive rows, and 8- or 16-byte
// writes from accumulator tiles. gfx950 serves 16-byte LDS reads in passes of
// 16 lanes ({0-3, 12-15, 20-27}, {4-11, 16-19, 28-31}, and the same above
// lane 32) over 64 banks, 8-byte reads in passes of 32 lanes, and writes in
// passes of 128 bytes. With 16 chunks per row, (r % 8) in the upper three bits
// keeps the chunks of 8 consecutive rows apart (transpose reads), and bit 2 of
// r in bit 0 separates the two lane groups of a 16-byte gather pass.
template <int CPR>
__device__ __forceinline__ int swz(int r) {
  if constexpr (CPR == 16) return ((r & 7) << 1) | ((r >> 2) & 1);
  else if constexpr (CPR == 8) return r & 7;
  else return tile_sw<CPR>(r);
}
// Byte offset of bf16 element `col` of row `r`.
template <int CPR>
__device__ __forceinline__ int off(int r, int col) {
  return r * (CPR * 16) + (((col >> 3) ^ swz<CPR>(r)) << 4) + ((col & 7) << 1);
}
// NATURAL operand fragment: row r, elements 32 ks + 8 g .. + 7.
template <int CPR>
__device__ __forceinline__ bf16x8 gat(const char* t, int r, int ks) {
  return *reinterpret_cast<const bf16x8*>(t + off<CPR>(r, 32 * ks + 8 * (lane_id() >> 4)));
}
// CHAIN operand fragment with k along the tile rows (k-step s), operand
// row/column = tile column c0 + lane % 16 (transpose reads).
template <int CPR>
__device__ __forceinline__ bf16x4 trd(const char* t, int k0, int c0) {
  const int j = lane_id() & 15;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 LM_LDS*)(t + off<CPR>(k0 + (j >> 2), c0 + 4 * (j & 3))));
  return __builtin_bit_cast(bf16x4, v);
}
template <int CPR>
__device__ __forceinline__ bf16x8 kmaj(const char* t, int s, int c0) {
  const int g = lane_id() >> 4;
  const bf16x4 lo = trd<CPR>(t, 32 * s + 4 * g, c0);
  const bf16x4 hi = trd<CPR>(t, 32 * s + 16 + 4 * g, c0);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// 8-byte store of an accumulator tile's four rows (converted) at (r, c0).
template <int CPR>
__device__ __forceinline__ void put4(char* t, int r, int c0, const f32x4& v) {
  *reinterpret_cast<bf16x4*>(t + off<CPR>(r, c0)) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// NaN-propagating max (gfx950 v_maximum3_f32; needs no NaN quieting, unlike fmaxf).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48) with the
// gfx950 cross-row lane swaps (no LDS traffic).
__device__ __forceinline__ float rows_max(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float rows_sum(float x) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  x = __uint_as_float(a[0]) + __uint_as_float(a[1]);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Lane (g, c) holds x_g; afterwards o[i] = x_i of lane (i, c), in every row.
__device__ __forceinline__ void rows_all(float x, float (&o)[4]) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(a[0], a[0], false, false);
  const auto c = __builtin_amdgcn_permlane16_swap(a[1], a[1], false, false);
  o[0] = __uint_as_float(b[0]);
  o[1] = __uint_as_float(b[1]);
  o[2] = __uint_as_float(c[0]);
  o[3] = __uint_as_float(c[1]);
}
// Value of row-indexed x[i] for i = g (the lane's own row) without dynamic indexing.
__device__ __forceinline__ float pick(const float (&x)[4], int i) {
  return i == 0 ? x[0] : i == 1 ? x[1] : i == 2 ? x[2] : x[3];
}

template <int D, int KP, int MODE>
struct Cfg {
  static constexpr int NW = 4;
  static constexpr int RT = KP / 64;   // 16-component tiles per wave
  static constexpr int KPW = KP / NW;  // components per wave
  static constexpr int NKX = D / 32;   // k-steps over x
  static constexpr int NKF = 2 * NKX;  // over [x | x*x]
  static constexpr int NKC = KP / 32;  // over all components
  static constexpr int DT = D / 16;    // 16-wide value tiles
  static constexpr int XC = D / 8;     // 16-byte chunks per row of a Q/K/V tile
  static constexpr int GC = KP / 8;    // per row of a Gamma or state tile
  static constexpr int XB = 64 * D * 2;
  static constexpr int GB = 64 * KP * 2;
  static constexpr int SB = D * KP * 2;
  static constexpr bool IS_AGG = MODE == AGG || MODE == AGG_G;
  static constexpr bool IS_CAUSAL = MODE == CAUSAL || MODE == CAUSAL_G;
  static constexpr bool GSTORE = MODE == AGG_G;    // store the key responsibilities
  static constexpr bool GLOAD = MODE == CAUSAL_G;  // load them instead of routing the keys
  static constexpr bool HK = MODE != BIDIR;        // keys update the state
  static constexpr bool RK = HK && !GLOAD;         // keys are routed here
  static constexpr bool HQ = !IS_AGG;
  static constexpr int NS = (HK ? 1 : 0) + (HQ ? 1 : 0);
  static constexpr int INSTR = XC / NW;  // DMA instructions per wave per tile
  // Separate LDS arrays (so that the compiler can tell accesses to the DMA
  // targets from the others and does not wait for an outstanding DMA at every
  // LDS access). Unused ones keep a token size.
  static constexpr int b_xk = HK ? XB : 16;
  // AGG (keys only) double-buffers the key tile: its DMA is issued two chunks
  // ahead, a whole chunk before it is needed.
  static constexpr bool XDB = IS_AGG;
  static constexpr int b_xk1 = XDB ? XB : 16;
  static constexpr int b_xq = HQ ? XB : 16;
  static constexpr int b_v = HK ? XB : 16;
  static constexpr int b_g = NS * XB > NS * GB ? NS * XB : NS * GB;  // x*x tiles, later Gamma tiles
  static constexpr int o_x2k = 0, o_x2q = HK ? XB : 0;  // (GLOAD: queries' x*x in the key tile buffer)
  static constexpr int o_gk = 0, o_gq = HK ? GB : 0;
  static constexpr int b_st = HQ ? SB : 16;            // bf16 state snapshot Vtil^T [D][KP]
  static constexpr int b_sk = RK ? NW * 64 * 8 : 16;   // key stats [NW][64] (max, sum)
  static constexpr int GDMA = GB / (NW * 1024);        // DMA instructions per wave for a key-responsibility tile
  static constexpr int b_sq = HQ ? NW * 64 * 16 : 16;  // query stats [NW][64] (max, sum, Z-dot)
  // With two component tiles per wave, lane p of routing tile rt holds
  // component 8 (p / 4) + 4 rt + p % 4 of the wave's 32: each lane's two tiles
  // then cover 8 adjacent components (one 16-byte responsibility store), and Z
  // is read for them from a bf16 row in LDS.
  static constexpr bool PAIR = RT == 2;
  static constexpr int b_z = HQ && PAIR ? KP * 2 : 16;  // bf16 Z row of the state before the chunk
  static constexpr int lds = b_xk + b_xk1 + b_xq + b_v + b_g + b_st + b_sk + b_sq + b_z;
  static_assert(lds <= 80 * 1024, "two workgroups per CU");
  static_assert(XC % NW == 0 && KP % 64 == 0 && D % 32 == 0, "shape");
  static_assert(GDMA * NW * 1024 == GB, "a key-responsibility tile is whole 1 KB DMA pieces");
};

// Per-lane source offsets of this wave's share of a 64-row tile DMA.
template <int XC, int INSTR>
__device__ __forceinline__ void dma_init(int (&voff)[INSTR]) {
  const int l = lane_id(), w = wave_id();
#pragma unroll
  for (int i = 0; i < INSTR; ++i) {
    const int p = (w * INSTR + i) * 64 + l;
    const int r = p / XC, pc = p % XC;
    voff[i] = r * XC * 16 + ((pc ^ swz<XC>(r)) << 4);
  }
}
template <int D, int INSTR>
__device__ __forceinline__ void dma_issue(char* dst, const bf16* src, int rows, const int* voff) {
  const u32x4 d = buf_desc(src, (uint32_t)(rows * D * 2));
  const unsigned base = lds_addr(dst) + (unsigned)(wave_id() * INSTR * 1024);
#pragma unroll
  for (int i = 0; i < INSTR; ++i) lds_dma16(d, voff[i], base + (unsigned)(i * 1024));
}

// Linear DMA of one key-responsibility tile (GB bytes, stored as it sat in
// LDS) into LDS: each wave moves GDMA 1 KB pieces.
template <int GDMA>
__device__ __forceinline__ void gdma_issue(char* dst, const char* src, int bytes) {
  const u32x4 d = buf_desc(src, (uint32_t)bytes);
  const unsigned base = lds_addr(dst) + (unsigned)(wave_id() * GDMA * 1024);
#pragma unroll
  for (int i = 0; i < GDMA; ++i)
    lds_dma16(d, (wave_id() * GDMA + i) * 1024 + lane_id() * 16, base + (unsigned)(i * 1024));
}

// x*x of the 16 rows this wave's DMA wrote (same physical positions).
template <int D>
__device__ __forceinline__ void square_rows(const char* x, char* x2) {
  constexpr int CH = 16 * (D / 8);
  const int base = wave_id() * CH * 16;
#pragma unroll
  for (int i = lane_id(); i < CH; i += 64) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + base + 16 * i);
    bf16x8 s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float f = (float)v[j];
      s[j] = (bf16)(f * f);
    }
    *reinterpret_cast<bf16x8*>(x2 + base + 16 * i) = s;
  }
}

// Logits (log2 units) of this wave's components for the 64 tokens of the key
// and/or query tile: L^T = W F^T + c with F = [x | x*x]. The feature fragments
// of token tile ct + 1 are read while tile ct is multiplied.
struct Tiles {
  const char* xk;
  const char* x2k;
  const char* xq;
  const char* x2q;
};
template <typename C>
__device__ __forceinline__ void feat(const Tiles& t, int ct, bf16x8 (&fk)[C::NKF], bf16x8 (&fq)[C::NKF]) {
  const int row = 16 * ct + (lane_id() & 15);
#pragma unroll
  for (int ks = 0; ks < C::NKF; ++ks) {
    const int kk = ks < C::NKX ? ks : ks - C::NKX;
    if constexpr (C::RK) fk[ks] = gat<C::XC>(ks < C::NKX ? t.xk : t.x2k, row, kk);
    if constexpr (C::HQ) fq[ks] = gat<C::XC>(ks < C::NKX ? t.xq : t.x2q, row, kk);
  }
}
template <typename C>
__device__ __forceinline__ void route(f32x4 (&Lk)[4][C::RT], f32x4 (&Lq)[4][C::RT], const Tiles& tl,
                                      const bf16x8 (&Wf)[C::RT][C::NKF], const float (&cb)[C::RT][4]) {
  bf16x8 fk[C::NKF], fq[C::NKF];
  feat<C>(tl, 0, fk, fq);
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    bf16x8 nk[C::NKF], nq[C::NKF];
    if (ct < 3) feat<C>(tl, ct + 1, nk, nq);
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt) {
      const f32x4 c = f32x4{cb[rt][0], cb[rt][1], cb[rt][2], cb[rt][3]};
      f32x4 ak = c, aq = c;
#pragma unroll
      for (int ks = 0; ks < C::NKF; ++ks) {
        if constexpr (C::RK) ak = Mma<bf16>::mma(Wf[rt][ks], fk[ks], ak);
        if constexpr (C::HQ) aq = Mma<bf16>::mma(Wf[rt][ks], fq[ks], aq);
      }
      if constexpr (C::RK) Lk[ct][rt] = ak;
      if constexpr (C::HQ) Lq[ct][rt] = aq;
    }
#pragma unroll
    for (int ks = 0; ks < C::NKF; ++ks) {
      fk[ks] = nk[ks];
      fq[ks] = nq[ks];
    }
  }
}
// Component of row p of routing tile rt, relative to the wave's first.
template <typename C>
__device__ __forceinline__ constexpr int route_comp(int rt, int p) {
  return C::PAIR ? 8 * (p >> 2) + 4 * rt + (p & 3) : 16 * rt + p;
}
// This lane's W fragments (rows comp0 + route_comp(rt, lane % 16), NATURAL
// k-groups); wrow points at row comp0 + route_comp(0, lane % 16).
template <typename C>
__device__ __forceinline__ void load_w(bf16x8 (&Wf)[C::RT][C::NKF], const bf16* __restrict__ wrow) {
#pragma unroll
  for (int rt = 0; rt < C::RT; ++rt)
#pragma unroll
    for (int ks = 0; ks < C::NKF; ++ks)
      Wf[rt][ks] = *reinterpret_cast<const bf16x8*>(wrow + (size_t)route_comp<C>(rt, 0) * 2 * (C::NKX * 32) + 32 * ks);
}

// Wave-local softmax pieces of one token tile: L <- exp2(L - m) with m the max
// over this wave's components. Padded components have logit kPadLogit, so a
// wave of padding only has a finite max that the cross-wave combine weights
// by exp2(kPadLogit - max) = 0. Returns the
// exponentials as a bf16 B operand (k = this wave's components, CHAIN order,
// zero-padded to a full k-step) for the sums done on the matrix core.
template <int RT>
__device__ __forceinline__ bf16x8 local_exp(f32x4 (&L)[RT], float& m) {
  float mx = L[0][0];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = vmax(mx, L[rt][r]);
  mx = rows_max(mx);
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) L[rt][r] = fast_exp2(L[rt][r] - mx);
  m = mx;
  if constexpr (RT >= 2) return Mma<bf16>::chain2(L[0], L[1]);
  else return Mma<bf16>::chain2(L[0], zero4());
}

// Responsibilities of token tile ct (rows 16 ct + c16) for this wave's
// components, scaled by f[ct], into a Gamma tile.
template <typename C>
__device__ __forceinline__ void put_gamma(char* t, const f32x4 (&L)[4][C::RT], const float (&f)[4], int comp0, int g,
                                          int c16) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    if constexpr (C::PAIR) {
      const f32x4 a = L[ct][0] * f[ct], b = L[ct][1] * f[ct];
      *reinterpret_cast<bf16x8*>(t + off<C::GC>(16 * ct + c16, comp0 + 8 * g)) =
          bf16x8{(bf16)a[0], (bf16)a[1], (bf16)a[2], (bf16)a[3], (bf16)b[0], (bf16)b[1], (bf16)b[2], (bf16)b[3]};
    } else {
#pragma unroll
      for (int rt = 0; rt < C::RT; ++rt) put4<C::GC>(t, 16 * ct + c16, comp0 + 16 * rt + 4 * g, L[ct][rt] * f[ct]);
    }
  }
}
// Z of this wave's components (state layout: component 16 rt + 4 g + r) as
// the bf16 Z row.
template <typename C>
__device__ __forceinline__ void put_z(bf16* sZ, const f32x4 (&Zt)[C::RT], int comp0, int g, int c16) {
  if (c16 == 0) {
#pragma unroll
    for (int rt = 0; rt < C::RT; ++rt)
      *reinterpret_cast<bf16x4*>(sZ + comp0 + 16 * rt + 4 * g) =
          bf16x4{(bf16)Zt[rt][0], (bf16)Zt[rt][1], (bf16)Zt[rt][2], (bf16)Zt[rt][3]};
  }
}

template <int D, int KP, int MODE>
__global__ __launch_bounds__(256, 2) void kernel(Args a) {
  typedef Cfg<D, KP, MODE> C;
  typedef Mma<bf16> M;
  constexpr int RT = C::RT, DT = C::DT, NKC = C::NKC;
  __shared__ __attribute__((aligned(16))) char sXK[C::b_xk];
  __shared__ __attribute__((aligned(16))) char sXK1[C::b_xk1];
  __shared__ __attribute__((aligned(16))) char sXQ[C::b_xq];
  __shared__ __attribute__((aligned(16))) char sV[C::b_v];
  __shared__ __attribute__((aligned(16))) char sG[C::b_g];
  __shared__ __attribute__((aligned(16))) char sST[C::b_st];
  __shared__ __attribute__((aligned(16))) float2 stK[C::b_sk / 8];
  __shared__ __attribute__((aligned(16))) f32x4 stQ[C::b_sq / 16];
  __shared__ __attribute__((aligned(16))) bf16 sZ[C::b_z / 2];
  Tiles tl{sXK, sG + C::o_x2k, sXQ, C::GLOAD ? sXK : sG + C::o_x2q};

  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int bh = blockIdx.y, p = blockIdx.x;
  const int h = bh % a.H;
  const int64_t N = a.N;
  const int64_t t_begin = (int64_t)p * a.seg_len;
  const int64_t t_end = N < t_begin + a.seg_len ? N : t_begin + a.seg_len;
  const bf16* __restrict__ Qg = reinterpret_cast<const bf16*>(a.q) + (size_t)bh * N * D;
  const bf16* __restrict__ Kg = reinterpret_cast<const bf16*>(a.k) + (size_t)bh * N * D;
  const bf16* __restrict__ Vg = reinterpret_cast<const bf16*>(a.v) + (size_t)bh * N * D;
  bf16* __restrict__ Og = reinterpret_cast<bf16*>(a.out) + (size_t)bh * N * D;
  const bf16* __restrict__ Wh = reinterpret_cast<const bf16*>(a.W) + (size_t)h * KP * 2 * D;
  const float* __restrict__ ch = a.c + (size_t)h * KP;
  const int comp0 = w * C::KPW;
  const int64_t nch = (N + kChunk - 1) / kChunk;
  char* const gkh = C::GSTORE || C::GLOAD ? static_cast<char*>(a.gk) + (size_t)bh * nch * C::GB : nullptr;

  const bf16* __restrict__ wrow = Wh + (size_t)(comp0 + route_comp<C>(0, c16)) * 2 * D + 8 * g;
  float cb[RT][4];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) cb[rt][r] = ch[comp0 + route_comp<C>(rt, 4 * g + r)];

  // State rows of this wave's components: S[dt][rt] (component rows, value
  // columns) and Zt[rt] (every column holds Z of the row's component).
  f32x4 S[DT][RT], Zt[RT];
#pragma unroll
  for (int rt = 0; rt < RT; ++rt) {
    Zt[rt] = zero4();
#pragma unroll
    for (int dt = 0; dt < DT; ++dt) S[dt][rt] = zero4();
  }
  if constexpr (!C::IS_AGG) {
    if (a.has_init) {
      const int slot = C::IS_CAUSAL ? p : 0;
      const float* ag = a.agg + ((size_t)bh * a.P + slot) * KP * D;
      const float* az = a.aggz + ((size_t)bh * a.P + slot) * KP;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int comp = comp0 + 16 * rt + 4 * g + r;
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) S[dt][rt][r] = ag[(size_t)comp * D + 16 * dt + c16];
          Zt[rt][r] = az[comp];
        }
    }
#pragma unroll
    for (int dt = 0; dt < DT; ++dt)
#pragma unroll
      for (int rt = 0; rt < RT; ++rt) put4<C::GC>(sST, 16 * dt + c16, comp0 + 16 * rt + 4 * g, S[dt][rt]);
    if constexpr (C::PAIR) put_z<C>(sZ, Zt, comp0, g, c16);
  }

  int voff[C::INSTR];
  dma_init<C::XC, C::INSTR>(voff);
  {
    const int rows = (int)((N - t_begin) < kChunk ? (N - t_begin) : kChunk);
    if constexpr (C::RK) dma_issue<D, C::INSTR>(sXK, Kg + (size_t)t_begin * D, rows, voff);
    if constexpr (C::GLOAD) gdma_issue<C::GDMA>(sG + C::o_gk, gkh + (size_t)(t_begin / kChunk) * C::GB, C::GB);
    if constexpr (C::HK) dma_issue<D, C::INSTR>(sV, Vg + (size_t)t_begin * D, rows, voff);
    if constexpr (C::HQ) dma_issue<D, C::INSTR>(sXQ, Qg + (size_t)t_begin * D, rows, voff);
    if (C::XDB && t_begin + kChunk < t_end) {
      const int64_t t1 = t_begin + kChunk;
      dma_issue<D, C::INSTR>(sXK1, Kg + (size_t)t1 * D, (int)((N - t1) < kChunk ? (N - t1) : kChunk), voff);
      LM_WAIT_VMEM(C::INSTR);
    } else {
      wait_vmem();
    }
    if constexpr (C::RK) square_rows<D>(sXK, sG + C::o_x2k);
    if constexpr (C::HQ) square_rows<D>(sXQ, const_cast<char*>(tl.x2q));
    lds_barrier();
  }

  bf16x8 Wf[RT][C::NKF];
  load_w<C>(Wf, wrow);
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;

  int it = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk, ++it) {
    const int nvalid = (int)((N - t0) < kChunk ? (N - t0) : kChunk);
    const bool more = t0 + kChunk < t_end;
    const int rows_next = more ? (int)((N - t0 - kChunk) < kChunk ? (N - t0 - kChunk) : kChunk) : 0;
    // key tile of this chunk and of the next (double-buffered in AGG)
    char* xk_cur = (C::XDB && (it & 1)) ? sXK1 : sXK;
    char* xk_nxt = (C::XDB && !(it & 1)) ? sXK1 : sXK;
    tl.xk = xk_cur;
    const bool more2 = C::XDB && t0 + 2 * kChunk < t_end;

    // ---- 1. routing and wave-local softmax statistics
    f32x4 Lk[4][RT], Lq[4][RT];
    float mk[4], sk[4], mq[4], sq[4], dq[4];
    route<C>(Lk, Lq, tl, Wf, cb);
    // Sums over this wave's components on the matrix core: with A = ones every
    // row of the product is sum_k e_k; for queries the odd rows of A hold Z
    // (state before the chunk), so element 1 of each lane's tile is
    // sum_k e_k Z_k. The sums use the exponentials rounded to bf16.
    if constexpr (C::RK) {
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16x8 e = local_exp<RT>(Lk[ct], mk[ct]);
        sk[ct] = Mma<bf16>::mma(ones, e, zero4())[0];
      }
    }
    if constexpr (C::HQ) {
      bf16x8 az;  // rows: even = 1, odd = Z of this wave's components (routing order)
      {
        bf16x8 z;
        if constexpr (C::PAIR) z = *reinterpret_cast<const bf16x8*>(sZ + comp0 + 8 * g);
        else z = Mma<bf16>::chain2(Zt[0], zero4());
        az = (c16 & 1) ? z : ones;
      }
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        const bf16x8 e = local_exp<RT>(Lq[ct], mq[ct]);
        const f32x4 sd = Mma<bf16>::mma(az, e, zero4());
        sq[ct] = sd[0];
        dq[ct] = sd[1];
      }
    }
    // lane (g, c16) publishes token 16 g + c16 (every row holds every tile's stats)
    if constexpr (C::RK) stK[w * 64 + l] = make_float2(pick(mk, g), pick(sk, g));
    if constexpr (C::HQ) stQ[w * 64 + l] = f32x4{pick(mq, g), pick(sq, g), pick(dq, g), 0.f};
    lds_barrier();  // X tiles and x*x tiles are dead from here


    // ---- 2. posterior responsibilities -> LDS. Lane (g, c16) combines the four
    // waves' statistics of token 16 g + c16; the factors are then broadcast to
    // the rows that hold that token tile.
    float den_inter = 0.f;
    if constexpr (C::RK) {
      float2 st[4];
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) st[ww] = stK[ww * 64 + l];
      const float mm = vmax(vmax(st[0].x, st[1].x), vmax(st[2].x, st[3].x));
      float ss = 0.f, self = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float e = fast_exp2(st[ww].x - mm);
        ss += st[ww].y * e;
        self = ww == w ? e : self;
      }
      float f[4];
      rows_all(l < nvalid ? self * __builtin_amdgcn_rcpf(ss) : 0.f, f);
      put_gamma<C>(sG + C::o_gk, Lk, f, comp0, g, c16);
    }
    if constexpr (C::HQ) {
      f32x4 st[4];
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) st[ww] = stQ[ww * 64 + l];
      const float mm = vmax(vmax(st[0][0], st[1][0]), vmax(st[2][0], st[3][0]));
      float ss = 0.f, dd = 0.f, self = 0.f;
#pragma unroll
      for (int ww = 0; ww < 4; ++ww) {
        const float e = fast_exp2(st[ww][0] - mm);
        ss += st[ww][1] * e;
        dd += st[ww][2] * e;
        self = ww == w ? e : self;
      }
      const float inv = __builtin_amdgcn_rcpf(ss);
      float f[4], di[4];
      rows_all(self * inv, f);
      rows_all(dd * inv, di);
      den_inter = pick(di, w);
      put_gamma<C>(sG + C::o_gq, Lq, f, comp0, g, c16);
    }
    // next chunk's X tiles (their old contents died at the barrier above); in
    // AGG the key tile after next, into this chunk's key buffer
    if constexpr (C::XDB) {
      if (more2) {
        const int64_t t2 = t0 + 2 * kChunk;
        dma_issue<D, C::INSTR>(xk_cur, Kg + (size_t)t2 * D, (int)((N - t2) < kChunk ? (N - t2) : kChunk), voff);
      }
    } else if (more) {
      if constexpr (C::RK) dma_issue<D, C::INSTR>(sXK, Kg + (size_t)(t0 + kChunk) * D, rows_next, voff);
      if constexpr (C::HQ) dma_issue<D, C::INSTR>(sXQ, Qg + (size_t)(t0 + kChunk) * D, rows_next, voff);
    }
    if constexpr (C::HK) {
      // V of this chunk: its DMA was issued before the X tiles just issued (in
      // AGG also the next key tile, issued a chunk ago, is waited for here)
      if (C::XDB ? more2 : more)
        LM_WAIT_VMEM(C::INSTR * ((C::RK ? 1 : 0) + (C::HQ ? 1 : 0)));
      else
        wait_vmem();
    }
    lds_barrier();

    // ---- 3. read (query tile w) and update (this wave's components). The W
    // fragments for the next chunk are fetched now; they are waited for with
    // the next chunk's tiles. AGG keeps them in registers instead: a wait for
    // loads issued here would also wait for the tile DMA issued after them.
    if (!C::XDB && more) load_w<C>(Wf, wrow);
    if constexpr (C::GSTORE) {
      // the key-responsibility tile of this chunk, as it sits in LDS
      char* gdst = gkh + (size_t)(t0 / kChunk) * C::GB;
      for (int i = threadIdx.x; i < C::GB / 16; i += 256)
        *reinterpret_cast<u32x4*>(gdst + 16 * i) = *reinterpret_cast<const u32x4*>(sG + C::o_gk + 16 * i);
    }
    bf16x8 VB[DT][2];
    if constexpr (C::HK) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int s = 0; s < 2; ++s) VB[dt][s] = kmaj<C::XC>(sV, s, 16 * dt);
    }
    if constexpr (C::HQ) {
      const char* gq = sG + C::o_gq;
      bf16x8 GQ[NKC];
#pragma unroll
      for (int ks = 0; ks < NKC; ++ks) GQ[ks] = gat<C::GC>(gq, 16 * w + c16, ks);
      f32x4 O[DT];
#pragma unroll
      for (int dt = 0; dt < DT; ++dt) {
        O[dt] = zero4();
#pragma unroll
        for (int ks = 0; ks < NKC; ++ks) O[dt] = M::mma(gat<C::GC>(sST, 16 * dt + c16, ks), GQ[ks], O[dt]);
      }
      float den = den_inter + a.eps;
      if constexpr (C::IS_CAUSAL) {
        const char* gk = sG + C::o_gk;
        f32x4 At[4];
#pragma unroll
        for (int kt = 0; kt < 4; ++kt) {
          At[kt] = zero4();
          if (kt <= w) {
#pragma unroll
            for (int ks = 0; ks < NKC; ++ks) At[kt] = M::mma(gat<C::GC>(gk, 16 * kt + c16, ks), GQ[ks], At[kt]);
            if (kt == w) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * g + r > c16) At[kt][r] = 0.f;
            }
          }
        }
        float di = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) di += At[kt][r];
        den += rows_sum(di);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (2 * s <= w) {
            const bf16x8 Af = M::chain2(At[2 * s], At[2 * s + 1]);
#pragma unroll
            for (int dt = 0; dt < DT; ++dt) O[dt] = M::mma(VB[dt][s], Af, O[dt]);
          }
        }
      }
      const int q = 16 * w + c16;
      if (q < nvalid) {
        const float inv = 1.f / den;
        bf16* dst = Og + (size_t)(t0 + q) * D + 4 * g;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) {
          const f32x4 o = O[dt] * inv;
          *reinterpret_cast<bf16x4*>(dst + 16 * dt) = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
        }
      }
    }
    if constexpr (C::HK) {
      const char* gk = sG + C::o_gk;
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 A = kmaj<C::GC>(gk, s, comp0 + 16 * rt);
#pragma unroll
          for (int dt = 0; dt < DT; ++dt) S[dt][rt] = M::mma(A, VB[dt][s], S[dt][rt]);
          Zt[rt] = M::mma(A, ones, Zt[rt]);
        }
    }
    lds_barrier();  // Gamma tiles, the state snapshot and V are dead from here

    // ---- 4. state snapshot, next V, next x*x
    if constexpr (C::IS_CAUSAL) {
#pragma unroll
      for (int dt = 0; dt < DT; ++dt)
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) put4<C::GC>(sST, 16 * dt + c16, comp0 + 16 * rt + 4 * g, S[dt][rt]);
      if constexpr (C::PAIR) put_z<C>(sZ, Zt, comp0, g, c16);
    }
    if (more) {
      if constexpr (C::HK) {
        // Next X tiles and the W fragments first (AGG: the key tile landed
        // earlier), then the V DMA: issued after the wait, the V tile is not
        // waited for by the compiler's own wait for W at the next routing.
        if constexpr (!C::XDB) wait_vmem();
        if constexpr (C::GLOAD)
          gdma_issue<C::GDMA>(sG + C::o_gk, gkh + (size_t)(t0 / kChunk + 1) * C::GB, C::GB);
        dma_issue<D, C::INSTR>(sV, Vg + (size_t)(t0 + kChunk) * D, rows_next, voff);
      } else {
        wait_vmem();
      }
      if constexpr (C::RK) square_rows<D>(xk_nxt, sG + C::o_x2k);
      if constexpr (C::HQ) square_rows<D>(sXQ, const_cast<char*>(tl.x2q));
    }
    lds_barrier();
  }

  if constexpr (C::IS_AGG) {
    float* ag = a.agg + ((size_t)bh * a.P + p) * KP * D;
    float* az = a.aggz + ((size_t)bh * a.P + p) * KP;
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int comp = comp0 + 16 * rt + 4 * g + r;
#pragma unroll
        for (int dt = 0; dt < DT; ++dt) ag[(size_t)comp * D + 16 * dt + c16] = S[dt][rt][r];
        if (c16 == 0) az[comp] = Zt[rt][r];
      }
  }
}

template <int D, int KP>
static hipError_t launch_mode(const Args& a, int mode, int segments, unsigned BH, hipStream_t st) {
  const dim3 grid((unsigned)segments, BH), block(256);
  switch (mode) {
    case AGG: hipLaunchKernelGGL((kernel<D, KP, AGG>), grid, block, 0, st, a); break;
    case CAUSAL: hipLaunchKernelGGL((kernel<D, KP, CAUSAL>), grid, block, 0, st, a); break;
    case AGG_G: hipLaunchKernelGGL((kernel<D, KP, AGG_G>), grid, block, 0, st, a); break;
    case CAUSAL_G: hipLaunchKernelGGL((kernel<D, KP, CAUSAL_G>), grid, block, 0, st, a); break;
    default: hipLaunchKernelGGL((kernel<D, KP, BIDIR>), grid, block, 0, st, a); break;
  }
  return hipGetLastError();
}

}  // namespace fast

bool fast_supported(const GmaLaunch& L) {
  return L.bf16 && (L.D == 32 || L.D == 64) && (L.KP == 64 || L.KP == 128);
}

hipError_t fast_launch(const GmaLaunch& L, const Args& a, int mode, int segments, hipStream_t st) {
  const unsigned BH = (unsigned)(L.B * L.H);
  if (L.D == 64) {
    if (L.KP == 128) return fast::launch_mode<64, 128>(a, mode, segments, BH, st);
    if (L.KP == 64) return fast::launch_mode<64, 64>(a, mode, segments, BH, st);
  } else if (L.D == 32) {
    if (L.KP == 128) return fast::launch_mode<32, 128>(a, mode, segments, BH, st);
    if (L.KP == 64) return fast::launch_mode<32, 64>(a, mode, segments, BH, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace gma
}  // namespace lm
