// gma_long.hip -- Gaussian Mixture Attention forward for bf16 inputs with
// d = dv = 128 and 256 mixture components (the long-context shape), on gfx950.
//
// Method ("Gaussian Mixture Attention: Linear-Time Sequence Mixing via
// Probabilistic Latent Routing", Method -> core mechanism and variants):
// responsibilities gamma(x) = p(z = k | x) of diagonal-Gaussian components for
// every query and key row; keys write Vtil = Gamma_K^T V and Z = Gamma_K^T 1;
// queries read O = Gamma_Q Vtil / (Gamma_Q Z + eps), causally by prefix sums.
//
// One workgroup of eight waves per (sequence, segment), one workgroup per CU
// (two waves per SIMD). Wave w owns components 32 w .. 32 w + 31: their rows
// of W = [a | b] (bf16, in registers) and of the fp32 state [Vtil | Z]. Per
// 64-token chunk:
//  1. Routing logits L^T = W [x | x*x]^T + c (MFMA; one lane per token), the
//     wave-local softmax over the wave's 32 components, and its per-token
//     (max, sum) to LDS. The exponential sums run on the matrix core against a
//     row of ones (queries: every other row holds Z of the state before the
//     chunk, which gives the inter-chunk normaliser in the same product).
//  2. After a barrier every wave rescales its exponentials to the posterior
//     and stores its 32 columns of Gamma_K and Gamma_Q (bf16) into the LDS that
//     held the x and x*x tiles.
//  3. Read, split by (query tile, half of the value columns): partial reads
//     Vtil^T Gamma_Q^T from a bf16 snapshot of the state in LDS, the masked
//     intra-chunk affinity A^T = Gamma_K Gamma_Q^T and V^T A^T. Update, split
//     by components: [Vtil | Z] += Gamma_K^T [V | 1] into the fp32 registers.
//  4. State snapshot refresh, the next chunk's Q/K/V by direct global->LDS
//     transfer, and x*x of the rows each wave's transfer brought in.
// Within a wave, the two component tiles of the routing hold components
// 8 (p / 4) + 4 rt + p % 4 (lane p), so that a lane's eight responsibilities
// of a token are adjacent: one 16-byte store per token tile.
#include "mfma.hpp"
#include "gma.hpp"

namespace lm {
namespace gma {
namespace lng {

constexpr int kD = 128;           // d = dv
constexpr int kKP = 256;          // components (padded)
constexpr int kNW = 8;            // waves
constexpr int kNT = kNW * 64;     // threads
constexpr int kKPW = kKP / kNW;   // components per wave (two 16-row tiles)
constexpr int XCPR = kD / 8;      // 16-byte chunks per row of a Q/K/V tile
constexpr int GCPR = kKP / 8;     // per row of a Gamma tile or of the snapshot
constexpr int XB = 64 * kD * 2;   // bytes of a 64-token x tile
constexpr int GB = 64 * kKP * 2;  // of a Gamma tile
constexpr int SB = kD * kKP * 2;  // of the bf16 state snapshot Vtil^T [dv][comp]
constexpr int kInstr = XCPR * 64 * 16 / 1024 / kNW;  // DMA instructions per wave per x tile

// LDS layout (bytes) of the passes with queries: the first 64 KB hold the
// routing tiles (K, K*K, Q, Q*Q) and then Gamma_K, Gamma_Q; V; the snapshot.
constexpr int oS = 5 * XB;
constexpr int oStK = oS + SB;               // [8 waves][64 tokens] (max, sum)
constexpr int oStQ = oStK + kNW * 64 * 8;   // [8 waves][64 tokens] (max, sum, Z-dot, -)
constexpr int oZ = oStQ + kNW * 64 * 16;    // bf16 Z of the state before the chunk [KP]
constexpr int kLds = oZ + kKP * 2;
static_assert(kLds <= 160 * 1024, "LDS budget");
static_assert(2 * GB == 4 * XB, "Gamma tiles fill the routing tiles' space");
static_assert(kInstr == 2, "DMA split");

// XOR swizzle of the 16-byte chunks of row r (rows of 16 or 32 chunks). gfx950
// serves 16-byte LDS reads in passes of 16 lanes ({0-3, 12-15, 20-27}, {4-11,
// 16-19, 28-31}, and the same above lane 32) over 64 banks, 8-byte reads
// (plain or transposed) in passes of 32 lanes, and writes in passes of 128
// bytes. With (r % 8) in bits 1-3 and bit 2 of r in bit 0, the operand
// gathers of 16 rows, the transposed reads of 8 rows and the 16-byte stores
// of 8 rows are conflict-free; 8-byte stores of 16 rows take two cycles.
__device__ __forceinline__ int xsw(int r) { return ((r & 7) << 1) | ((r >> 2) & 1); }
template <int CPR>
__device__ __forceinline__ int off(int r, int col) {
  return r * (CPR * 16) + (((col >> 3) ^ xsw(r)) << 4) + ((col & 7) << 1);
}
// The lane index, hidden from the optimiser at the top of every chunk: the
// per-lane LDS addresses derived from it are then formed where they are used
// instead of being held in registers across the whole loop.
__device__ __forceinline__ int lane_opaque() {
  int x = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(x));
  return x;
}
// NATURAL operand fragment: row r, elements 32 ks + 8 g .. + 7 (lane l).
template <int CPR>
__device__ __forceinline__ bf16x8 gat(const char* t, int r, int ks, int l) {
  return *reinterpret_cast<const bf16x8*>(t + off<CPR>(r, 32 * ks + 8 * (l >> 4)));
}
// Transposed read: lane p of a 16-lane group gets column c0 + p of rows
// k0 .. k0 + 3 (the lanes supply rows k0 + j / 4, columns c0 + 4 (j % 4) ..).
template <int CPR>
__device__ __forceinline__ bf16x4 trd(const char* t, int k0, int c0, int l) {
  const int j = l & 15;
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (i16x4 LM_LDS*)(t + off<CPR>(k0 + (j >> 2), c0 + 4 * (j & 3))));
  return __builtin_bit_cast(bf16x4, v);
}
// CHAIN fragment with k along the tile rows (k-step s of 32 rows): operand
// row/column = tile column c0 + lane % 16.
template <int CPR>
__device__ __forceinline__ bf16x8 kmaj(const char* t, int s, int c0, int l) {
  const int g = l >> 4;
  const bf16x4 lo = trd<CPR>(t, 32 * s + 4 * g, c0, l);
  const bf16x4 hi = trd<CPR>(t, 32 * s + 16 + 4 * g, c0, l);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// 8-byte store of an accumulator tile's four rows (converted) at (r, c0 ..).
template <int CPR>
__device__ __forceinline__ void put4(char* t, int r, int c0, const f32x4& v) {
  *reinterpret_cast<bf16x4*>(t + off<CPR>(r, c0)) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// NaN-propagating max (gfx950 v_maximum3_f32).
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }
// Reductions over the four 16-lane rows (lanes l, l^16, l^32, l^48).
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
__device__ __forceinline__ float pick(const float (&x)[4], int i) {
  return i == 0 ? x[0] : i == 1 ? x[1] : i == 2 ? x[2] : x[3];
}

// Component (relative to the wave's first) of row p of routing tile rt.
__device__ __forceinline__ constexpr int route_comp(int rt, int p) { return 8 * (p >> 2) + 4 * rt + (p & 3); }

// Modes: AGG (segment states), AGG_G (the same, storing each chunk's Gamma_K
// tile as it sits in LDS), CAUSAL, CAUSAL_G (loading those tiles instead of
// routing the keys), BIDIR.
template <int MODE>
struct Cfg {
  static constexpr bool IS_AGG = MODE == AGG || MODE == AGG_G;
  static constexpr bool CAUS = MODE == CAUSAL || MODE == CAUSAL_G;
  static constexpr bool HK = MODE != BIDIR;        // keys update the state
  static constexpr bool GLOAD = MODE == CAUSAL_G;  // Gamma_K tiles loaded
  static constexpr bool GSTORE = MODE == AGG_G;    // Gamma_K tiles stored
  static constexpr bool RK = HK && !GLOAD;         // keys routed here
  static constexpr bool HQ = !IS_AGG;              // queries: routing, read
  // LDS. Segment passes (no queries, no snapshot) double-buffer their tiles:
  // set s holds K and K*K (then Gamma_K) at s * 2 XB and V at 4 XB + s XB.
  // The other passes hold Q and Q*Q at 2 XB, 3 XB (then Gamma_Q), K and K*K
  // at 0, XB (then Gamma_K; or the loaded Gamma_K tile), V at 4 XB and the
  // snapshot after it.
  static constexpr int oA(int s) { return IS_AGG ? s * 2 * XB : 0; }
  static constexpr int oVs(int s) { return IS_AGG ? 4 * XB + s * XB : 4 * XB; }
  static constexpr int oQx = 2 * XB, oQ2x = 3 * XB;
  static constexpr int oStK_ = IS_AGG ? 6 * XB : oStK;
  static constexpr int lds = IS_AGG ? 6 * XB + kNW * 64 * 8 : kLds;
};
constexpr int GDMA = GB / 1024 / kNW;  // DMA instructions per wave for a Gamma_K tile

// Logits (log2 units) of this wave's 64 components' two tiles for the 64
// tokens of an x tile: L[ct][rt] = W_rt [x | x*x]^T (token tile ct) + c.
__device__ __forceinline__ void route(f32x4 (&L)[4][2], const char* x, const char* x2, const bf16x8 (&Wf)[2][8],
                                      const float (&cb)[2][4], int l) {
  const int c16 = l & 15;
#pragma unroll
  for (int ct = 0; ct < 4; ++ct)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) L[ct][rt] = f32x4{cb[rt][0], cb[rt][1], cb[rt][2], cb[rt][3]};
  bf16x8 f[2];
  f[0] = gat<XCPR>(x, c16, 0, l);
#pragma unroll
  for (int i = 0; i < 32; ++i) {
    const int ct = i >> 3, ks = i & 7;
    if (i + 1 < 32) {
      const int ct1 = (i + 1) >> 3, ks1 = (i + 1) & 7;
      f[(i + 1) & 1] = gat<XCPR>(ks1 < 4 ? x : x2, 16 * ct1 + c16, ks1 & 3, l);
    }
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) L[ct][rt] = Mma<bf16>::mma(Wf[rt][ks], f[i & 1], L[ct][rt]);
  }
}

// Wave-local softmax pieces of one token tile: L <- exp2(L - m), m the max over
// the wave's components (padded components have logit kPadLogit; a wave of
// padding only is weighted by 0 in the cross-wave combine). Returns the
// exponentials as a bf16 B operand (k = the wave's 32 components in order).
__device__ __forceinline__ bf16x8 local_exp(f32x4 (&L)[2], float& m) {
  float mx = L[0][0];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) mx = vmax(mx, L[rt][r]);
  mx = rows_max(mx);
#pragma unroll
  for (int rt = 0; rt < 2; ++rt)
#pragma unroll
    for (int r = 0; r < 4; ++r) L[rt][r] = fast_exp2(L[rt][r] - mx);
  m = mx;
  return Mma<bf16>::chain2(L[0], L[1]);
}

// Responsibilities of the four token tiles: the bf16 exponentials E[ct] (the
// values the sums were taken of) scaled by f[ct], into this wave's 32 columns
// of a Gamma tile, one 16-byte store per lane and token tile.
__device__ __forceinline__ void put_gamma(char* t, const bf16x8 (&E)[4], const float (&f)[4], int comp0, int g, int c16) {
#pragma unroll
  for (int ct = 0; ct < 4; ++ct) {
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) o[i] = (bf16)((float)E[ct][i] * f[ct]);
    *reinterpret_cast<bf16x8*>(t + off<GCPR>(16 * ct + c16, comp0 + 8 * g)) = o;
  }
}

// bf16 snapshot of this wave's state rows (S[dt][rt]: component 16 rt + 4 g + r
// of the wave, value column 16 dt + c16) as Vtil^T, and its Z as the Z row.
__device__ __forceinline__ void put_state(char* sS, bf16* sZ, const f32x4 (&S)[8][2], const f32x4 (&Zt)[2], int comp0,
                                          int g, int c16) {
#pragma unroll
  for (int dt = 0; dt < 8; ++dt)
#pragma unroll
    for (int rt = 0; rt < 2; ++rt) put4<GCPR>(sS, 16 * dt + c16, comp0 + 16 * rt + 4 * g, S[dt][rt]);
  if (c16 == 0) {
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
      *reinterpret_cast<bf16x4*>(sZ + comp0 + 16 * rt + 4 * g) =
          bf16x4{(bf16)Zt[rt][0], (bf16)Zt[rt][1], (bf16)Zt[rt][2], (bf16)Zt[rt][3]};
  }
}

// x*x of the rows this wave's transfers wrote (same physical positions).
__device__ __forceinline__ void square_own(const char* x, char* x2) {
  const int base = wave_id() * kInstr * 1024 + lane_id() * 16;
#pragma unroll
  for (int i = 0; i < kInstr; ++i) {
    const bf16x8 v = *reinterpret_cast<const bf16x8*>(x + base + i * 1024);
    bf16x8 s;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float fv = (float)v[j];
      s[j] = (bf16)(fv * fv);
    }
    *reinterpret_cast<bf16x8*>(x2 + base + i * 1024) = s;
  }
}

struct Dma {
  int voff[kInstr];
  __device__ __forceinline__ void init() {
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < kInstr; ++i) {
      const int p = (w * kInstr + i) * 64 + l;
      const int r = p / XCPR, pc = p % XCPR;
      voff[i] = r * XCPR * 16 + ((pc ^ xsw(r)) << 4);
    }
  }
  // src: the tile's first row; rows: rows of the sequence left from src.
  __device__ __forceinline__ void issue(char* dst, const bf16* src, int rows) const {
    const u32x4 d = buf_desc(src, (uint32_t)((rows < 64 ? rows : 64) * kD * 2));
    const unsigned base = lds_addr(dst) + (unsigned)(wave_id() * kInstr * 1024);
#pragma unroll
    for (int i = 0; i < kInstr; ++i) lds_dma16(d, voff[i], base + (unsigned)(i * 1024));
  }
};

// Linear DMA of one stored Gamma_K tile (GB bytes, in its LDS layout).
__device__ __forceinline__ void gdma_issue(char* dst, const char* src) {
  const u32x4 d = buf_desc(src, (uint32_t)GB);
  const unsigned base = lds_addr(dst) + (unsigned)(wave_id() * GDMA * 1024);
#pragma unroll
  for (int i = 0; i < GDMA; ++i)
    lds_dma16(d, (wave_id() * GDMA + i) * 1024 + lane_id() * 16, base + (unsigned)(i * 1024));
}

template <int MODE>
__global__ __launch_bounds__(kNT, 1) void kernel(Args a) {
  typedef Cfg<MODE> C;
  typedef Mma<bf16> M;
  __shared__ __attribute__((aligned(16))) char smem[C::lds];
  float2* const stK = reinterpret_cast<float2*>(smem + C::oStK_);
  f32x4* const stQ = reinterpret_cast<f32x4*>(smem + oStQ);
  bf16* const sZ = reinterpret_cast<bf16*>(smem + oZ);
  char* const sGQ = smem + C::oQx;
  char* const sS = smem + oS;

  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int bh = blockIdx.y, p = blockIdx.x;
  const int h = bh % a.H;
  const int64_t N = a.N;
  const int64_t t_begin = (int64_t)p * a.seg_len;
  const int64_t t_end = N < t_begin + a.seg_len ? N : t_begin + a.seg_len;
  const bf16* __restrict__ Qg = reinterpret_cast<const bf16*>(a.q) + (size_t)bh * N * kD;
  const bf16* __restrict__ Kg = reinterpret_cast<const bf16*>(a.k) + (size_t)bh * N * kD;
  const bf16* __restrict__ Vg = reinterpret_cast<const bf16*>(a.v) + (size_t)bh * N * kD;
  bf16* __restrict__ Og = reinterpret_cast<bf16*>(a.out) + (size_t)bh * N * kD;
  const bf16* __restrict__ Wh = reinterpret_cast<const bf16*>(a.W) + (size_t)h * kKP * 2 * kD;
  const float* __restrict__ ch = a.c + (size_t)h * kKP;
  const int comp0 = w * kKPW;
  // stored Gamma_K tiles of this sequence, one per chunk of 64 tokens
  char* const gkh = C::GSTORE || C::GLOAD ? static_cast<char*>(a.gk) + (size_t)bh * ((N + kChunk - 1) / kChunk) * GB
                                          : nullptr;
  // read split: query tile qt, value columns 64 dh .. 64 dh + 63; the two waves
  // of a SIMD (w, w + 4) take query tiles qt and 3 - qt
  const int qt = w < 4 ? w : 7 - w;
  const int dh = w >> 2;

  // routing W fragments and biases (rows in routing order)
  bf16x8 Wf[2][8];
  float cb[2][4];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    const bf16* row = Wh + (size_t)(comp0 + route_comp(rt, c16)) * 2 * kD + 8 * g;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) Wf[rt][ks] = *reinterpret_cast<const bf16x8*>(row + 32 * ks);
#pragma unroll
    for (int r = 0; r < 4; ++r) cb[rt][r] = ch[comp0 + route_comp(rt, 4 * g + r)];
  }

  // state rows of this wave's components (component comp0 + 16 rt + 4 g + r)
  f32x4 S[8][2], Zt[2];
#pragma unroll
  for (int rt = 0; rt < 2; ++rt) {
    Zt[rt] = zero4();
#pragma unroll
    for (int dt = 0; dt < 8; ++dt) S[dt][rt] = zero4();
  }
  if constexpr (C::HQ) {
    if (a.has_init) {
      const int slot = C::CAUS ? p : 0;
      const float* ag = a.agg + ((size_t)bh * a.P + slot) * kKP * kD;
      const float* az = a.aggz + ((size_t)bh * a.P + slot) * kKP;
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int comp = comp0 + 16 * rt + 4 * g + r;
#pragma unroll
          for (int dt = 0; dt < 8; ++dt) S[dt][rt][r] = ag[(size_t)comp * kD + 16 * dt + c16];
          Zt[rt][r] = az[comp];
        }
    }
    put_state(sS, sZ, S, Zt, comp0, g, c16);
  }

  // The tiles of chunk c (set c % 2 in segment passes).
  Dma dma;
  dma.init();
  // Q first: the loaded-Gamma_K pass waits for Q only before routing and for
  // the Gamma_K and V transfers behind it just before the first barrier.
  auto issue = [&](int64_t t, int s) {
    const int rows = (int)(t_end - t);
    if constexpr (C::HQ) dma.issue(smem + C::oQx, Qg + (size_t)t * kD, rows);
    if constexpr (C::RK) dma.issue(smem + C::oA(s), Kg + (size_t)t * kD, rows);
    if constexpr (C::GLOAD) gdma_issue(smem + C::oA(s), gkh + (size_t)(t / kChunk) * GB);
    if constexpr (C::HK) dma.issue(smem + C::oVs(s), Vg + (size_t)t * kD, rows);
  };
  auto square = [&](int s) {
    if constexpr (C::RK) square_own(smem + C::oA(s), smem + C::oA(s) + XB);
    if constexpr (C::HQ) square_own(smem + C::oQx, smem + C::oQ2x);
  };
  if (t_begin < t_end) {
    issue(t_begin, 0);
    if (C::IS_AGG && t_begin + kChunk < t_end) {
      issue(t_begin + kChunk, 1);
      LM_WAIT_VMEM(2 * kInstr);  // the first chunk's tiles
    } else {
      wait_vmem();
    }
    square(0);
  }
  lds_barrier();

  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (bf16)1.f;

  int it = 0;
  for (int64_t t0 = t_begin; t0 < t_end; t0 += kChunk, ++it) {
    const int nvalid = (int)((t_end - t0) < kChunk ? (t_end - t0) : kChunk);
    const bool more = t0 + kChunk < t_end;
    const int lo = lane_opaque();  // the lane index for LDS addressing in this chunk
    const int co = lo & 15;
    const int cs = C::IS_AGG ? (it & 1) : 0;  // tile set of this chunk
    char* const sGK = smem + C::oA(cs);
    char* const sV = smem + C::oVs(cs);

    // ---- 1. routing and wave-local softmax statistics
    bf16x8 Ek[4], Eq[4];  // bf16 exponentials, k = the wave's components in order
    float mk[4], sk[4], mq[4], sq[4], dq[4];
    if constexpr (C::RK) {
      f32x4 L[4][2];
      route(L, sGK, sGK + XB, Wf, cb, lo);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        Ek[ct] = local_exp(L[ct], mk[ct]);
        sk[ct] = M::mma(ones, Ek[ct], zero4())[0];
      }
      stK[w * 64 + l] = make_float2(pick(mk, g), pick(sk, g));
    }
    if constexpr (C::HQ) {
      f32x4 L[4][2];
      route(L, smem + C::oQx, smem + C::oQ2x, Wf, cb, lo);
      // rows of A: even = 1, odd = Z of the wave's components (state before the chunk)
      const bf16x8 z = *reinterpret_cast<const bf16x8*>(sZ + comp0 + 8 * (lo >> 4));
      const bf16x8 az = (c16 & 1) ? z : ones;
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) {
        Eq[ct] = local_exp(L[ct], mq[ct]);
        const f32x4 sd = M::mma(az, Eq[ct], zero4());
        sq[ct] = sd[0];
        dq[ct] = sd[1];
      }
      stQ[w * 64 + l] = f32x4{pick(mq, g), pick(sq, g), pick(dq, g), 0.f};
    }
    if constexpr (C::GLOAD) wait_vmem();  // this chunk's Gamma_K and V transfers
    lds_barrier();  // statistics complete; the x and x*x tiles are dead

    // ---- 2. posterior responsibilities -> Gamma tiles. Lane l combines the
    // eight waves' statistics of token l; rows_all broadcasts them by tile.
    float den_inter = 0.f;
    if constexpr (C::RK) {
      float mm = stK[l].x;
#pragma unroll
      for (int ww = 1; ww < kNW; ++ww) mm = vmax(mm, stK[ww * 64 + l].x);
      float ss = 0.f, self = 0.f;
#pragma unroll
      for (int ww = 0; ww < kNW; ++ww) {
        const float2 st = stK[ww * 64 + l];
        const float e = fast_exp2(st.x - mm);
        ss += st.y * e;
        self = ww == w ? e : self;
      }
      float f[4];
      rows_all(l < nvalid ? self * __builtin_amdgcn_rcpf(ss) : 0.f, f);
      put_gamma(sGK, Ek, f, comp0, lo >> 4, co);
    }
    if constexpr (C::HQ) {
      float mm = stQ[l][0];
#pragma unroll
      for (int ww = 1; ww < kNW; ++ww) mm = vmax(mm, stQ[ww * 64 + l][0]);
      float ss = 0.f, dd = 0.f, self = 0.f;
#pragma unroll
      for (int ww = 0; ww < kNW; ++ww) {
        const f32x4 st = stQ[ww * 64 + l];
        const float e = fast_exp2(st[0] - mm);
        ss += st[1] * e;
        dd += st[2] * e;
        self = ww == w ? e : self;
      }
      const float inv = __builtin_amdgcn_rcpf(ss);
      float f[4], di[4];
      rows_all(self * inv, f);
      rows_all(dd * inv, di);
      den_inter = pick(di, qt);
      put_gamma(sGQ, Eq, f, comp0, lo >> 4, co);
    }
    lds_barrier();  // Gamma tiles complete

    // ---- 3. read (query tile qt, value columns of half dh) and update
    if constexpr (C::GSTORE) {
      // this chunk's Gamma_K tile, as it sits in LDS
      char* gdst = gkh + (size_t)(t0 / kChunk) * GB;
#pragma unroll
      for (int j = 0; j < GB / 16 / kNT; ++j) {
        const int i = (int)threadIdx.x + j * kNT;
        *reinterpret_cast<u32x4*>(gdst + 16 * i) = *reinterpret_cast<const u32x4*>(sGK + 16 * i);
      }
    }
    if constexpr (C::HQ) {
      // one k-step (32 components) at a time: the Gamma_Q fragment serves the
      // snapshot read and the intra-chunk affinity
      f32x4 O[4], At[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        O[i] = zero4();
        At[i] = zero4();
      }
#pragma unroll
      for (int ks = 0; ks < 8; ++ks) {
        const bf16x8 gq = gat<GCPR>(sGQ, 16 * qt + co, ks, lo);
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) O[d4] = M::mma(gat<GCPR>(sS, 16 * (4 * dh + d4) + co, ks, lo), gq, O[d4]);
        if constexpr (C::CAUS) {
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            if (kt <= qt) At[kt] = M::mma(gat<GCPR>(sGK, 16 * kt + co, ks, lo), gq, At[kt]);
        }
      }
      float den = den_inter + a.eps;
      if constexpr (C::CAUS) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          // keys after the query on the diagonal tile
          const float m = 4 * g + r > c16 ? 0.f : 1.f;
#pragma unroll
          for (int kt = 0; kt < 4; ++kt)
            if (kt == qt) At[kt][r] *= m;
        }
        float di = 0.f;
#pragma unroll
        for (int kt = 0; kt < 4; ++kt)
#pragma unroll
          for (int r = 0; r < 4; ++r) di += At[kt][r];
        den += rows_sum(di);
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (2 * s <= qt) {
            const bf16x8 Af = M::chain2(At[2 * s], At[2 * s + 1]);
#pragma unroll
            for (int d4 = 0; d4 < 4; ++d4) O[d4] = M::mma(kmaj<XCPR>(sV, s, 16 * (4 * dh + d4), lo), Af, O[d4]);
          }
        }
      }
      const int q = 16 * qt + c16;
      if (q < nvalid) {
        const float inv = 1.f / den;
        bf16* dst = Og + (size_t)(t0 + q) * kD + 64 * dh + 4 * g;
#pragma unroll
        for (int d4 = 0; d4 < 4; ++d4) {
          const f32x4 o = O[d4] * inv;
          *reinterpret_cast<bf16x4*>(dst + 16 * d4) = bf16x4{(bf16)o[0], (bf16)o[1], (bf16)o[2], (bf16)o[3]};
        }
      }
    }
    if constexpr (C::HK) {
      bf16x8 A[2][2];
#pragma unroll
      for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          A[rt][s] = kmaj<GCPR>(sGK, s, comp0 + 16 * rt, lo);
          Zt[rt] = M::mma(A[rt][s], ones, Zt[rt]);
        }
#pragma unroll
      for (int dt = 0; dt < 8; ++dt) {
        const bf16x8 v0 = kmaj<XCPR>(sV, 0, 16 * dt, lo), v1 = kmaj<XCPR>(sV, 1, 16 * dt, lo);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt) {
          S[dt][rt] = M::mma(A[rt][0], v0, S[dt][rt]);
          S[dt][rt] = M::mma(A[rt][1], v1, S[dt][rt]);
        }
      }
    }
    lds_barrier();  // this chunk's Gamma tiles, snapshot and V are dead

    // ---- 4. next tiles, state snapshot, x*x. Segment passes: the next
    // chunk's tiles landed during this chunk; the tiles two chunks ahead go
    // into the set just freed. Other passes: the next chunk's tiles now.
    if constexpr (C::IS_AGG) {
      wait_vmem();
      if (t0 + 2 * kChunk < t_end) issue(t0 + 2 * kChunk, cs);
      if (more) square(cs ^ 1);
    } else {
      if (more) issue(t0 + kChunk, 0);
      if constexpr (C::CAUS) put_state(sS, sZ, S, Zt, comp0, lo >> 4, co);
      if (more) {
        if constexpr (C::GLOAD) LM_WAIT_VMEM(GDMA + kInstr);  // Q (and everything before it)
        else wait_vmem();
        square(0);
      }
    }
    lds_barrier();
  }
  wait_vmem();  // output and tile stores

  if constexpr (C::IS_AGG) {
    float* ag = a.agg + ((size_t)bh * a.P + p) * kKP * kD;
    float* az = a.aggz + ((size_t)bh * a.P + p) * kKP;
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int comp = comp0 + 16 * rt + 4 * g + r;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) ag[(size_t)comp * kD + 16 * dt + c16] = S[dt][rt][r];
        if (c16 == 0) az[comp] = Zt[rt][r];
      }
  }
}

}  // namespace lng

bool long_supported(const GmaLaunch& L) { return L.bf16 && L.D == lng::kD && L.KP == lng::kKP; }

hipError_t long_launch(const Args& a, int mode, int segments, unsigned BH, hipStream_t st) {
  const dim3 grid((unsigned)segments, BH), block(lng::kNT);
  switch (mode) {
    case AGG: hipLaunchKernelGGL(lng::kernel<AGG>, grid, block, 0, st, a); break;
    case CAUSAL: hipLaunchKernelGGL(lng::kernel<CAUSAL>, grid, block, 0, st, a); break;
    case BIDIR: hipLaunchKernelGGL(lng::kernel<BIDIR>, grid, block, 0, st, a); break;
    case AGG_G: hipLaunchKernelGGL(lng::kernel<AGG_G>, grid, block, 0, st, a); break;
    case CAUSAL_G: hipLaunchKernelGGL(lng::kernel<CAUSAL_G>, grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gma
}  // namespace lm
