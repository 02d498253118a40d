// ccq_pipe.hip -- chunk pass of the curvature-conditioned-query (CCQ) read over
// decayed linear attention, for bf16 inputs with d_k = d_v = 128, on gfx950.
//
// Method ("Don't Read Everything: A Curvature-Conditioned Query for Linear
// Attention", section 2 Method; allinfo.ai.kr linear attention post, "Key
// messages" and "Easy explanation"): S_t = g_t S_{t-1} + k_t v_t^T; the read is
// o_t = S_t^T q'_t with the cleaned query q'_t = q_t - lambda_t Sigma_t q_t,
// Sigma_t the running key covariance with weights 1/t (current token included,
// no decay) and lambda_t = sigmoid(w . q_t + b). With M, m the running sums of
// k k^T and k, P_ij = q_i . k_j (j <= i, inside the chunk), alpha_i =
// lambda_i / t_i and beta_i = alpha_i (m_prev . q_i + sum_{j<=i} P_ij) / t_i:
//   q'_i - q_i = -alpha_i (M_prev q_i + sum_{j<=i} P_ij k_j)
//                + beta_i (sum_{j<=i} k_j + m_prev).
// At t = 1 the two sides cancel exactly. P enters both (as an MFMA operand and
// in the row sum) rounded to bf16 once, so that they still cancel exactly there
// and the rounding only perturbs the covariance as a centred quantity.
// The chunk's decayed read is then the plain chunkwise form with q':
//   o_i = 2^(l_i) S_prev^T q'_i + sum_{j<=i} 2^(l_i - l_j) (q'_i . k_j) v_j.
//
// MI355X design: a two-stage pipeline inside one workgroup of eight waves (one
// workgroup per CU, one producer and one consumer wave per SIMD).
//  * Producers (waves 0-3) own 32 columns each of M (fp32 registers) and of m.
//    In iteration it they clean the queries of chunk it: gate and mean terms,
//    raw scores P and M_prev q (first half), then the key products, the cleaned
//    queries q' (rounded once to bf16 and written to LDS as ready-made MFMA
//    fragments) and the update of M and m (second half).
//  * Consumers (waves 4-7) own 32 value columns each of S (fp32 registers). In
//    iteration it they read chunk it-1 with the q' made one iteration earlier:
//    decayed cleaned scores and S_prev^T q' (first half), then the intra-chunk
//    product with V, the output stores and the update of S (second half).
//  * Both halves of an iteration carry about the same matrix-core work for the
//    two waves of a SIMD, and one barrier separates them. The score tiles are
//    shared out by a fixed per-wave list, so every loop over them unrolls.
//  * Q/K/V/g tiles arrive by global->LDS DMA one iteration ahead (K in a ring
//    of three: the consumer's, the producer's and the landing one). Each wave
//    issues its share at a different point of the iteration, so that the
//    transfers do not queue behind each other in the address unit.
//  * Operand orders. Every operand read from LDS along the feature axis is a
//    NATURAL fragment (k = 8g..8g+7 of a step: one 16-byte read). Fragments
//    chained from the fp32 state (M, S) carry rows 4g..4g+3 of two 16-row
//    tiles, so the state's rows are labelled to match: row 4g + r of row
//    tile bt holds feature 32 (bt / 2) + 8g + 4 (bt % 2) + r. The key
//    operands that build the state (transposed reads of K) pick their 4-column
//    groups in the same order, and so do the columns of M and of S (tile row x
//    of column tile t is column 8 (x / 4) + 4 t + x % 4 of the wave's 32),
//    which also gives each consumer lane eight adjacent outputs of one row:
//    one 16-byte store per lane and query tile.
#include "launch.hpp"
#include "mfma.hpp"

namespace lm {
namespace ccqp {

constexpr int kC = 64;
constexpr int kD = 128;
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int TB = kC * kD * 2;  // bytes of one 64 x 128 bf16 tile
constexpr int PDD = kD + 8;      // pitch of the gate / mean rows
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLazy = 64.f;

// LDS layout (bytes).
constexpr int oK = 0;                    // K ring, 3 tiles
constexpr int oQ = oK + 3 * TB;          // Q, 2 tiles
constexpr int oV = oQ + 2 * TB;          // V, 2 tiles
constexpr int oQc = oV + 2 * TB;         // cleaned queries as fragments [qt][ks][lane] x 16 B
constexpr int oP = oQc + TB;             // raw masked scores, 64 x 64 bf16 (score layout below)
constexpr int oPc = oP + kC * kC * 2;    // cleaned decayed scores, 64 x 64 bf16
constexpr int oDot = oPc + kC * kC * 2;  // [4][PDD] bf16: w hi, w lo, m hi, m lo
constexpr int oG = oDot + 4 * PDD * 2;   // decays, 2 x 64 fp32
// per query: alpha, m_prev . q, and the row sums of P from the two slots; 16 spare
constexpr int oQR = oG + 2 * kC * 4;     // [80] float4
constexpr int oL = oQR + (kC + 16) * 16; // consumers' cumulative decays, [4][64] fp32
constexpr int oWt = oL + 4 * kC * 4;     // consumers' weights of the new state terms, [4][64] fp32
constexpr int oTri = oWt + 4 * kC * 4;   // lower-triangular ones, diagonal k-step of each query tile
constexpr int kLds = oTri + 4 * 64 * 16;
static_assert(kLds <= 160 * 1024, "LDS budget");

struct Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const float* g;
  const float* wl;  // [H][D]
  const float* bl;  // [H]
  bf16* out;
  const float* agg;  // segment start states (blocks of sfl floats), or null
  int64_t N;
  int H;
  int P;  // state blocks per (b, h)
  int R;  // block of segment p: R p
  int seg_len;
  int sfl;
  int64_t t_off;
  float* st_out;  // optional: state after the last token [S | M | m] per (b, h)
};

// ----------------------------------------------------------------------------
// LDS banking on gfx950 (measured with the bank-conflict counters): 64 banks
// of 4 bytes for reads of 8 and 16 bytes per lane. A 16-byte read is served in
// passes of 16 lanes: lanes {0-3, 12-15, 20-27} form one pass, {4-11, 16-19,
// 28-31} another, and the same for lanes 32-63. An 8-byte read (plain or
// transposed) is served in passes of 32 lanes. Writes of 8 bytes are served in
// passes of 16 lanes over 128 bytes.
//
// Tile layout. A 64 x 128 bf16 tile is 64 rows of 16 pieces of 16 bytes. Row
// block rb = r / 16 holds 256 pieces; piece c of row r sits at slot
//   rb * 256 + c * 16 + ((r % 16) ^ h(c % 4)),  h = (0, 12, 4, 8).
// An operand read (lane: row c16, piece 4 ks + g) lands on slot c16 ^ h(g) of
// 16 (the 256 bytes of the 64 banks): distinct within each pass of a 16-byte
// read. A transposed read takes one 8-byte half of 32 pieces per pass, two per
// slot at best; the XOR spreads them over all 16 slots. Row blocks, pieces and
// k-steps are constant offsets from a per-lane base. One DMA instruction fills
// 64 slots: 16 rows x 4 pieces, i.e. 64-byte runs of 16 source rows.
__device__ __forceinline__ constexpr int tile_xor(int c) { return ((0x84c0 >> (4 * (c & 3))) & 15); }
__device__ __forceinline__ int slot_off(int rb, int r16, int c) {
  return (rb * 256 + c * 16 + (r16 ^ tile_xor(c))) * 16;
}
// Score tiles (64 queries x 64 keys, bf16): piece p (8 keys) of query row r at
// 16-byte unit 8 r + (p ^ ((r / 2) % 8)). Operand reads (row c16, piece 4 s +
// g) are conflict-free; the 8-byte stores of 16 rows take two cycles, the
// least an 8-byte store of 16 lanes needs.
__device__ __forceinline__ int sc_sigma(int c16) { return (c16 >> 1) & 7; }

// The lane index, hidden from the optimiser once per chunk: the few per-lane
// LDS bases derived from it are recomputed in the loop rather than held in
// registers across it, next to the two state blocks.
struct Lane {
  int l, g, c16;
  int nat;        // NATURAL read of row c16 of a row block: piece 4 ks + g
  int trp, trp2;  // transposed read: rows 8 g + j / 4 (and + 4), piece j % 4
  int sc;         // score tiles: element offset of piece 4 s + g of row c16, s = 0
};
__device__ __forceinline__ Lane lane_opaque() {
  int x = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(x));
  Lane L;
  L.l = x;
  L.g = x >> 4;
  L.c16 = x & 15;
  const int g = L.g, j = L.c16;
  L.nat = slot_off(0, j, g);
  // rows 8 g + j / 4: row block g / 2, row 8 (g % 2) + j / 4 in it
  L.trp = slot_off(g >> 1, 8 * (g & 1) + (j >> 2), j & 3);
  L.trp2 = slot_off(g >> 1, 8 * (g & 1) + (j >> 2) + 4, j & 3);
  L.sc = j * kC + ((g ^ sc_sigma(j)) << 3);
  return L;
}
// NATURAL fragment: row 16 rb + c16, k = 32 ks + 8 g .. + 7.
__device__ __forceinline__ bf16x8 nat_rd(const char* t, int rb, int ks, const Lane& L) {
  return *reinterpret_cast<const bf16x8*>(t + rb * 4096 + ks * 1024 + L.nat);
}
// Transposed (k-major) NATURAL fragment: tokens 32 ks + 8 g .. + 7 of column
// base + 8 (p / 4) + 4 dt + p % 4 for lane p of a 16-lane group (base a
// multiple of 32): the column order of the state. Each lane of the transpose
// read supplies one row and the 4 columns its group hands to lanes
// 4 (j % 4) .. + 3; the second read covers the next 4 rows.
__device__ __forceinline__ bf16x8 trp_rd(const char* t, int ks, int base, int dt, const Lane& L) {
  const char* p = t + ks * 8192 + (base >> 3) * 256 + dt * 8;
  const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p + L.trp)));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p + L.trp2)));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// NATURAL fragment of a plain row-major bf16 array: row rc, k = 32 ks + 8 g .. + 7.
__device__ __forceinline__ bf16x8 row_rd(const bf16* base, int pitch, int rc, int ks, int g) {
  return *reinterpret_cast<const bf16x8*>(base + rc * pitch + ks * 32 + 8 * g);
}
// Score tile operand: query row 16 qt + c16, keys 32 s + 8 g .. + 7.
__device__ __forceinline__ bf16x8 sc_rd(const bf16* t, int qt, int s, const Lane& L) {
  return *reinterpret_cast<const bf16x8*>(t + qt * 16 * kC + (L.sc ^ (s << 5)));
}
// Score tile element offset of query row r, keys k .. (k a multiple of 4).
__device__ __forceinline__ int sc_off(int r, int k) {
  return r * kC + ((((k >> 3) ^ sc_sigma(r & 15)) << 3) | (k & 7));
}

// Global->LDS transfer of 16 bytes per lane (buffer_load ... lds), issued as
// inline asm without a compiler memory fence: the destination tiles of this
// kernel are read only after the wait and barrier at the top of a later
// iteration, so nothing in between has to stay ordered with the issue.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void dma16(const u32x4& desc, int voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(desc), "s"(m) : "m0");
}
__device__ __forceinline__ void dma4(const u32x4& desc, int voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(desc), "s"(m) : "m0");
}
#pragma clang diagnostic pop

// This wave's share of a tile's DMA: four of its sixteen instructions (64
// slots each), numbers 4 q .. 4 q + 3.
struct Dma {
  int voff[4];
  __device__ __forceinline__ void init(int q) {
    const int l = lane_id();
#pragma unroll
    for (int n = 0; n < 4; ++n) {
      const int i = 4 * q + n;
      const int c = (i & 3) * 4 + (l >> 4);
      const int row = 16 * (i >> 2) + ((l & 15) ^ tile_xor(c));
      voff[n] = row * (kD * 2) + c * 16;
    }
  }
  __device__ __forceinline__ void issue(char* dst, const bf16* src, int rows, int q) const {
    const u32x4 d = buf_desc(src, (uint32_t)((rows < kC ? rows : kC) * kD * 2));
    const unsigned base = lds_addr(dst) + (unsigned)(q * 4 * 1024);
#pragma unroll
    for (int n = 0; n < 4; ++n) dma16(d, voff[n], base + (unsigned)(n * 1024));
  }
};

// ----------------------------------------------------------------------------
// Score tiles (query tile, key tile <= query tile) of producer / consumer PW:
// PW 0: (0,0) (1,0) (1,1); PW 1: (2,0) (2,1) (2,2); PW 2: (3,0) (3,1);
// PW 3: (3,2) (3,3). The row sums of a query tile come from one wave, except
// query tile 3 (two partial slots).
template <int PW>
struct Tiles {
  static constexpr int n = PW < 2 ? 3 : 2;
  static constexpr int qt(int i) { return PW == 0 ? (i == 0 ? 0 : 1) : PW == 1 ? 2 : 3; }
  static constexpr int kt(int i) { return PW == 0 ? (i == 2 ? 1 : 0) : PW == 1 ? i : 2 * (PW - 2) + i; }
  static constexpr int qlast = qt(n - 1);
  static constexpr int slot = PW == 3 ? 1 : 0;
};

// Decay factors 2^(l_i - l_j) of score tile (qt, kt) for this lane's query i
// (cumulative log2 decay lq) and key rows 16 kt + 4 g + r; zero above the
// diagonal. Off the diagonal the factor is split at the tile's last key so
// that no exponent is positive; on the diagonal the exponent is clamped to
// <= 0 before the mask.
__device__ __forceinline__ f32x4 decay_tile(const float* sl, float lq, int kt, int qt, int g, int c16) {
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

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)0.f;
  return f;
}

// Lower-triangular ones as a NATURAL B operand: keys 32 s + 8 g + e (k) against
// query i (column): 1 where the key is <= i.
__device__ __forceinline__ bf16x8 tri_frag(int s, int i, int g) {
  const int t = i - 32 * s - 8 * g;  // element e is set when e <= t
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = e <= t ? (bf16)1.f : (bf16)0.f;
  return f;
}
__device__ __forceinline__ bf16x8 ones8() {
  bf16x8 f;
#pragma unroll
  for (int e = 0; e < 8; ++e) f[e] = (bf16)1.f;
  return f;
}

__device__ __forceinline__ bf16x4 pack4(const f32x4& v) {
  return bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// Writes m (this producer's 32 entries: entry (ct, r) of lane group g is
// feature 32 pw + 8 g + 4 ct + r) as the bf16 hi / lo rows 2 and 3 of the
// gate / mean operand.
__device__ __forceinline__ void put_m(bf16* sDot, const float (&m)[2][4], int pw, int g, int c16) {
  if (c16 == 0) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = 32 * pw + 8 * g + 4 * ct + r;
        const bf16 hi = (bf16)m[ct][r];
        sDot[2 * PDD + a] = hi;
        sDot[3 * PDD + a] = (bf16)(m[ct][r] - (float)hi);
      }
  }
}

// Per-workgroup constants and the transfers of one chunk's tiles.
struct Ctx {
  char* smem;
  const bf16* Qg;
  const bf16* Kg;
  const bf16* Vg;
  const float* Gg;
  bf16* Og;
  int64_t t_begin, t_end, t_tok0;
  int nch;
  float gate_b;
  Dma dma;
  __device__ __forceinline__ int rows_of(int c) const {
    const int64_t c0 = t_begin + (int64_t)c * kC;
    return (int)((t_end - c0) < kC ? (t_end - c0) : kC);
  }
  __device__ __forceinline__ const bf16* row0(const bf16* base, int c) const {
    return base + (size_t)(t_begin + (int64_t)c * kC) * kD;
  }
  __device__ __forceinline__ void issue_q(int c, int q) const { dma.issue(smem + oQ + (c & 1) * TB, row0(Qg, c), rows_of(c), q); }
  __device__ __forceinline__ void issue_k(int c, int q) const { dma.issue(smem + oK + (c % 3) * TB, row0(Kg, c), rows_of(c), q); }
  __device__ __forceinline__ void issue_v(int c, int q) const { dma.issue(smem + oV + (c & 1) * TB, row0(Vg, c), rows_of(c), q); }
  __device__ __forceinline__ void issue_g(int c) const {
    const int64_t c0 = t_begin + (int64_t)c * kC;
    dma4(buf_desc(Gg + c0, (uint32_t)(rows_of(c) * 4)), lane_id() * 4, lds_addr(smem + oG + (c & 1) * kC * 4));
  }
};

// ----------------------------------------------------------------- producer
// First half for chunk it: M_prev q for this wave's 32 columns (X), the gate
// logit and mean term of query tile PW (alpha and m_prev . q to LDS) and this
// wave's raw score tiles (bf16, with row sums of the rounded values), as one
// k-step loop whose operands are read a step ahead.
template <int PW>
__device__ __forceinline__ void producer_first(const Ctx& x, int it, const f32x4 (&St)[8][2], f32x4 (&X)[2][4],
                                               const Lane& L) {
  typedef Tiles<PW> TL;
  constexpr int NQ = TL::qlast != TL::qt(0) ? 2 : 1;  // query tiles of the score list
  const int g = L.g, c16 = L.c16;
  const char* Qt = x.smem + oQ + (it & 1) * TB;
  const char* Kt = x.smem + oK + (it % 3) * TB;
  const bf16* sDot = reinterpret_cast<const bf16*>(x.smem + oDot);
  bf16* sP = reinterpret_cast<bf16*>(x.smem + oP);
  float* sQR = reinterpret_cast<float*>(x.smem + oQR);
  // this wave's quarters of the next chunk's Q and K transfers
  if (it + 1 < x.nch) {
    x.issue_q(it + 1, PW);
    x.issue_k(it + 1, PW);
  }
  struct Ops {
    bf16x8 qc[4];      // Q, query tiles 0..3 (M_prev q, the gate and mean terms, the scores)
    bf16x8 dot;        // gate / mean rows
    bf16x8 kc[TL::n];  // K, the score list's key tiles
  };
  auto load = [&](int s, Ops& o) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) o.qc[qt] = nat_rd(Qt, qt, s, L);
    o.dot = c16 < 4 ? row_rd(sDot, PDD, c16, s, g) : zero8();
#pragma unroll
    for (int n = 0; n < TL::n; ++n) o.kc[n] = nat_rd(Kt, TL::kt(n), s, L);
  };
  Ops ops[2];
  load(0, ops[0]);
  f32x4 dq = zero4();
  f32x4 acc[TL::n];
#pragma unroll
  for (int n = 0; n < TL::n; ++n) acc[n] = zero4();
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) X[ct][qt] = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s + 1 < 4) load(s + 1, ops[(s + 1) & 1]);
    const Ops& o = ops[s & 1];
    // M_prev q, with the bf16 copy of two M row blocks
    const bf16x8 ma0 = Mma<bf16>::chain2(St[2 * s][0], St[2 * s + 1][0]);
    const bf16x8 ma1 = Mma<bf16>::chain2(St[2 * s][1], St[2 * s + 1][1]);
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      X[0][qt] = Mma<bf16>::mma(ma0, o.qc[qt], X[0][qt]);
      X[1][qt] = Mma<bf16>::mma(ma1, o.qc[qt], X[1][qt]);
    }
    // rows 0..3 of the 16-row operand hold w hi, w lo, m hi, m lo; the rest is zero
    dq = Mma<bf16>::mma(o.dot, o.qc[PW], dq);
#pragma unroll
    for (int n = 0; n < TL::n; ++n) acc[n] = Mma<bf16>::mma(o.kc[n], o.qc[TL::qt(n)], acc[n]);
  }
  {
    const int i = 16 * PW + c16;
    const float lam = __builtin_amdgcn_rcpf(1.f + fast_exp2(-(dq[0] + dq[1] + x.gate_b) * kLog2eF));
    const float inv_t = __builtin_amdgcn_rcpf((float)x.t_tok0 + (float)(it * kC + i + 1));
    // only the lanes of group 0 hold the four rows; the others write a spare slot
    *reinterpret_cast<float2*>(sQR + 4 * (g == 0 ? i : kC + c16)) = make_float2(lam * inv_t, dq[2] + dq[3]);
  }
  float rs0 = 0.f, rs1 = 0.f;
#pragma unroll
  for (int n = 0; n < TL::n; ++n) {
    const int qt = TL::qt(n), kt = TL::kt(n);
    if (kt == qt) {
#pragma unroll
      for (int r = 0; r < 4; ++r)
        if (4 * g + r > c16) acc[n][r] = 0.f;
    }
    const bf16x4 p = pack4(acc[n]);
    *reinterpret_cast<bf16x4*>(sP + sc_off(16 * qt + c16, 16 * kt + 4 * g)) = p;
    const float part = ((float)p[0] + (float)p[1]) + ((float)p[2] + (float)p[3]);
    if (qt == TL::qt(0)) rs0 += part; else rs1 += part;
  }
  rs0 = group_sum(rs0);
  sQR[4 * (g == 0 ? 16 * TL::qt(0) + c16 : kC + c16) + 2 + TL::slot] = rs0;
  if (NQ == 2) {
    rs1 = group_sum(rs1);
    sQR[4 * (g == 0 ? 16 * TL::qlast + c16 : kC + c16) + 2 + TL::slot] = rs1;
  }
}

// Second half for chunk it: alpha, beta; the key products sum_j P_ij k_j and
// sum_{j<=i} k_j for this wave's columns; q' = q + delta (bf16 fragments to
// LDS); M += K^T K[:, cols], m += column sums. The query tiles' work is
// interleaved with the row blocks of the M update (independent chains), with
// each row block's K^T fragments read one step ahead.
__device__ __forceinline__ void producer_second(const Ctx& x, int it, int pw, f32x4 (&St)[8][2], float (&mcol)[2][4],
                                                const f32x4 (&X)[2][4], const Lane& L) {
  const int g = L.g, c16 = L.c16;
  const char* Qt = x.smem + oQ + (it & 1) * TB;
  const char* Kt = x.smem + oK + (it % 3) * TB;
  const bf16* sP = reinterpret_cast<const bf16*>(x.smem + oP);
  const f32x4* sQR = reinterpret_cast<const f32x4*>(x.smem + oQR);
  const bf16x8* sTri = reinterpret_cast<const bf16x8*>(x.smem + oTri);
  bf16* sDot = reinterpret_cast<bf16*>(x.smem + oDot);
  bf16x8* sQc = reinterpret_cast<bf16x8*>(x.smem + oQc);
  // K columns of this wave in the state's column order (lane p of column tile
  // ct: feature 32 pw + 8 (p / 4) + 4 ct + p % 4; k = tokens)
  bf16x8 KC[2][2];
#pragma unroll
  for (int ct = 0; ct < 2; ++ct)
#pragma unroll
    for (int s = 0; s < 2; ++s) KC[ct][s] = trp_rd(Kt, s, 32 * pw, ct, L);
  // K columns of row tile bt in the state's row order
  bf16x8 kf[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) kf[0][s] = trp_rd(Kt, s, 0, 0, L);
  const float t_i0 = (float)x.t_tok0 + (float)(it * kC + c16 + 1);
#pragma unroll
  for (int bt = 0; bt < 8; ++bt) {
    if (bt + 1 < 8) {
#pragma unroll
      for (int s = 0; s < 2; ++s) kf[(bt + 1) & 1][s] = trp_rd(Kt, s, 32 * ((bt + 1) >> 1), (bt + 1) & 1, L);
    }
    // M += K^T K[:, cols], row block bt
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) St[bt][ct] = Mma<bf16>::mma(kf[bt & 1][s], KC[ct][s], St[bt][ct]);
    if (bt < 4) {
      const int qt = bt, i = 16 * qt + c16;
      const f32x4 qr = sQR[i];  // alpha, m_prev . q, row sums of the two slots
      const float inv_t = __builtin_amdgcn_rcpf(t_i0 + (float)(16 * qt));
      const float al = qr[0], be = qr[0] * (qr[1] + (qr[2] + qr[3])) * inv_t;
      // accumulators start from M_prev q and m_prev: kp = M_prev q + sum_j P_ij k_j,
      // kc = m_prev + sum_{j<=i} k_j
      f32x4 kp[2] = {X[0][qt], X[1][qt]};
      f32x4 kc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) kc[ct][r] = mcol[ct][r];
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s == 1 && qt < 2) continue;  // keys 32..63 lie above the diagonal
        const bf16x8 pf = sc_rd(sP, qt, s, L);
        // the query tile's diagonal k-step from the table, full steps below it
        const bf16x8 tf = s == (qt >> 1) ? sTri[qt * 64 + L.l] : ones8();
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          kp[ct] = Mma<bf16>::mma(KC[ct][s], pf, kp[ct]);
          kc[ct] = Mma<bf16>::mma(KC[ct][s], tf, kc[ct]);
        }
      }
      const bf16x8 qv = nat_rd(Qt, qt, pw, L);
      bf16x8 qc;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ct = e >> 2, r = e & 3;
        qc[e] = (bf16)((float)qv[e] + (be * kc[ct][r] - al * kp[ct][r]));
      }
      sQc[(qt * 4 + pw) * 64 + L.l] = qc;
    }
  }
  {
    const bf16x8 one = ones8();
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
      f32x4 cs = zero4();
#pragma unroll
      for (int s = 0; s < 2; ++s) cs = Mma<bf16>::mma(KC[ct][s], one, cs);
#pragma unroll
      for (int r = 0; r < 4; ++r) mcol[ct][r] += cs[r];
    }
  }
  put_m(sDot, mcol, pw, g, c16);
}

// ----------------------------------------------------------------- consumer
// Per-wave decay state of the consumer: S_true = 2^ls St (lazy decay), the ls
// this chunk's read uses, and the row sums' exponent of its new terms.
struct Lazy {
  float ls;   // after this chunk's update
  float lso;  // before it (the read of this chunk)
};

// First half for chunk c = it - 1: cumulative decays and the weights of the
// chunk's new state terms, S_prev^T q' for this wave's 32 value columns (X)
// and this wave's decayed cleaned score tiles (one k-step loop whose operands
// are read a step ahead; the q' fragments serve both), and the rare eager
// rescale of S.
template <int PW>
__device__ __forceinline__ void consumer_first(const Ctx& x, int it, f32x4 (&St)[8][2], Lazy& lz, f32x4 (&X)[2][4],
                                               const Lane& L) {
  typedef Tiles<PW> TL;
  const int l = L.l, g = L.g, c16 = L.c16;
  const int c = it - 1;
  const char* Kt = x.smem + oK + (c % 3) * TB;
  const float* gt = reinterpret_cast<const float*>(x.smem + oG + (c & 1) * kC * 4);
  float* sLw = reinterpret_cast<float*>(x.smem + oL) + PW * kC;
  float* sWt = reinterpret_cast<float*>(x.smem + oWt) + PW * kC;
  bf16* sPc = reinterpret_cast<bf16*>(x.smem + oPc);
  const bf16x8* Qc = reinterpret_cast<const bf16x8*>(x.smem + oQc);
  const int nvalid = x.rows_of(c);
  // this wave's quarter of the V transfer of chunk it (read in the next iteration)
  if (it < x.nch) {
    x.issue_v(it, PW);
    if (PW == 0) x.issue_g(it);
  }
  struct Ops {
    bf16x8 q[4];      // q', query tiles 0..3
    bf16x8 k[TL::n];  // K, the score list's key tiles
  };
  auto load = [&](int s, Ops& o) {
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) o.q[qt] = Qc[(qt * 4 + s) * 64 + l];
#pragma unroll
    for (int n = 0; n < TL::n; ++n) o.k[n] = nat_rd(Kt, TL::kt(n), s, L);
  };
  Ops ops[2];
  load(0, ops[0]);
  // cumulative log2 decay of the chunk (lane = token; g in (0, 1], 0 clamped),
  // then S <- 2^l_last S + K^T (2^(l_last - l_j) V) held as 2^ls S: the chunk
  // decay is folded into the weights of the new terms until ls would drop
  // below -kLazy, and only then multiplied into S
  bool eager;
  float ls_next;
  {
    float v = l < nvalid ? fmaxf(__builtin_amdgcn_logf(gt[l]), -200.f) : 0.f;
    v = wave_scan_incl(v);
    sLw[l] = v;
    const float l_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, v), kC - 1));
    lz.lso = lz.ls;
    ls_next = lz.ls + l_last;
    eager = ls_next < -kLazy;
    const float wb = eager ? l_last : -lz.ls;
    sWt[l] = fast_exp2(wb - v);
    lz.ls = eager ? 0.f : ls_next;
  }
  f32x4 acc[TL::n];
#pragma unroll
  for (int n = 0; n < TL::n; ++n) acc[n] = zero4();
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) X[dt][qt] = zero4();
#pragma unroll
  for (int s = 0; s < 4; ++s) {
    if (s + 1 < 4) load(s + 1, ops[(s + 1) & 1]);
    const Ops& o = ops[s & 1];
    // S_prev^T q', with the bf16 copy of two S row blocks
    const bf16x8 sa0 = Mma<bf16>::chain2(St[2 * s][0], St[2 * s + 1][0]);
    const bf16x8 sa1 = Mma<bf16>::chain2(St[2 * s][1], St[2 * s + 1][1]);
#pragma unroll
    for (int qt = 0; qt < 4; ++qt) {
      X[0][qt] = Mma<bf16>::mma(sa0, o.q[qt], X[0][qt]);
      X[1][qt] = Mma<bf16>::mma(sa1, o.q[qt], X[1][qt]);
    }
#pragma unroll
    for (int n = 0; n < TL::n; ++n) acc[n] = Mma<bf16>::mma(o.k[n], o.q[TL::qt(n)], acc[n]);
  }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int n = 0; n < TL::n; ++n) {
    const int qt = TL::qt(n), kt = TL::kt(n);
    const f32x4 d = decay_tile(sLw, sLw[16 * qt + c16], kt, qt, g, c16);
    *reinterpret_cast<bf16x4*>(sPc + sc_off(16 * qt + c16, 16 * kt + 4 * g)) = pack4(acc[n] * d);
  }
  if (eager) {
    const float b = fast_exp2(ls_next);
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) St[bt][dt] *= b;
  }
}

// Second half for chunk c = it - 1: the update of S with the weighted V,
// interleaved by row block with the query tiles' intra-chunk products and
// outputs (16-byte stores through a buffer resource that ends at the chunk's
// last valid row, so that rows past N are dropped without a branch).
__device__ __forceinline__ void consumer_second(const Ctx& x, int it, int pw, f32x4 (&St)[8][2], const Lazy& lz,
                                                const f32x4 (&X)[2][4], const Lane& L) {
  const int g = L.g, c16 = L.c16;
  const int c = it - 1;
  const char* Kt = x.smem + oK + (c % 3) * TB;
  const char* Vt = x.smem + oV + (c & 1) * TB;
  const float* sLw = reinterpret_cast<const float*>(x.smem + oL) + pw * kC;
  const float* sWt = reinterpret_cast<const float*>(x.smem + oWt) + pw * kC;
  const bf16* sPc = reinterpret_cast<const bf16*>(x.smem + oPc);
  const int64_t c0 = x.t_begin + (int64_t)c * kC;
  const int vbase = 32 * pw;
  const rsrc_t orsrc = make_rsrc(x.Og + (size_t)c0 * kD, (uint32_t)(x.rows_of(c) * kD * 2));
  bf16x8 VF[2][2], VW[2][2];
#pragma unroll
  for (int dt = 0; dt < 2; ++dt)
#pragma unroll
    for (int s = 0; s < 2; ++s) VF[dt][s] = trp_rd(Vt, s, vbase, dt, L);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
    const f32x4 w0 = *reinterpret_cast<const f32x4*>(sWt + 32 * s + 8 * g);
    const f32x4 w1 = *reinterpret_cast<const f32x4*>(sWt + 32 * s + 8 * g + 4);
#pragma unroll
    for (int dt = 0; dt < 2; ++dt)
#pragma unroll
      for (int e = 0; e < 8; ++e) VW[dt][s][e] = (bf16)((float)VF[dt][s][e] * (e < 4 ? w0[e] : w1[e - 4]));
  }
  bf16x8 kf[2][2];
#pragma unroll
  for (int s = 0; s < 2; ++s) kf[0][s] = trp_rd(Kt, s, 0, 0, L);
#pragma unroll
  for (int bt = 0; bt < 8; ++bt) {
    if (bt + 1 < 8) {
#pragma unroll
      for (int s = 0; s < 2; ++s) kf[(bt + 1) & 1][s] = trp_rd(Kt, s, 32 * ((bt + 1) >> 1), (bt + 1) & 1, L);
    }
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int dt = 0; dt < 2; ++dt) St[bt][dt] = Mma<bf16>::mma(kf[bt & 1][s], VW[dt][s], St[bt][dt]);
    if (bt < 4) {
      const int qt = bt, i = 16 * qt + c16;
      f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        if (s == 1 && qt < 2) continue;
        const bf16x8 pf = sc_rd(sPc, qt, s, L);
#pragma unroll
        for (int dt = 0; dt < 2; ++dt) acc[dt] = Mma<bf16>::mma(VF[dt][s], pf, acc[dt]);
      }
      const float bq = fast_exp2(sLw[i] + lz.lso);
      bf16x8 o;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        o[r] = (bf16)(acc[0][r] + bq * X[0][qt][r]);
        o[4 + r] = (bf16)(acc[1][r] + bq * X[1][qt][r]);
      }
      __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4, o), orsrc, (i * kD + vbase + 8 * g) * 2, 0, 0);
    }
  }
}

__global__ __launch_bounds__(kNT, 1) void chunk_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const bool producer = w < 4;
  const int pw = w & 3;
  const int bh = blockIdx.y, seg = blockIdx.x, h = bh % a.H;
  const int64_t N = a.N;

  Ctx x;
  x.smem = smem;
  x.t_begin = (int64_t)seg * a.seg_len;
  x.t_end = N < x.t_begin + a.seg_len ? N : x.t_begin + a.seg_len;
  x.t_tok0 = x.t_begin + a.t_off;
  x.nch = (int)((x.t_end - x.t_begin + kC - 1) / kC);
  x.Qg = a.q + (size_t)bh * N * kD;
  x.Kg = a.k + (size_t)bh * N * kD;
  x.Vg = a.v + (size_t)bh * N * kD;
  x.Gg = a.g + (size_t)bh * N;
  x.Og = a.out + (size_t)bh * N * kD;
  x.gate_b = a.bl[h];
  x.dma.init(pw);
  // the first chunk's Q and K: producers move Q, consumers K
  if (x.nch > 0) {
    if (producer) x.issue_q(0, pw);
    else x.issue_k(0, pw);
  }

  bf16* sPc = reinterpret_cast<bf16*>(smem + oPc);
  bf16* sP = reinterpret_cast<bf16*>(smem + oP);
  bf16* sDot = reinterpret_cast<bf16*>(smem + oDot);

  // State: producers M[frow(bt, r)][fcol(ct, c16)] as St[bt][ct] and m;
  // consumers S[frow(bt, r)][fcol(dt, c16)] as St[bt][dt].
  f32x4 St[8][2];
  float mcol[2][4];
  Lazy lz{0.f, 0.f};  // consumers: S_true = 2^ls St
  auto frow = [&](int bt, int r) { return 32 * (bt >> 1) + 8 * g + 4 * (bt & 1) + r; };
  auto fcol = [&](int t, int xx) { return 32 * pw + 8 * (xx >> 2) + 4 * t + (xx & 3); };
  {
    const float* blk = a.agg ? a.agg + ((size_t)bh * a.P + (size_t)a.R * seg) * a.sfl : nullptr;
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = frow(bt, r);
          float v = 0.f;
          if (blk) v = producer ? blk[kD * kD + 1 + row * kD + fcol(t, c16)] : blk[row * kD + fcol(t, c16)];
          St[bt][t][r] = v;
        }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) mcol[ct][r] = blk ? blk[2 * kD * kD + 1 + 32 * pw + 8 * g + 4 * ct + r] : 0.f;
  }
  // gate weights (rows 0 / 1, hi / lo), the zero score tiles above the
  // diagonal that the k-steps of 32 keys read, partial row sums slot 1
  for (int i = threadIdx.x; i < 2 * PDD; i += kNT) {
    const int row = i / PDD, col = i - (i / PDD) * PDD;
    float v = 0.f;
    if (col < kD) {
      const float wv = a.wl[(size_t)h * kD + col];
      const bf16 hi = (bf16)wv;
      v = row == 0 ? (float)hi : wv - (float)hi;
    }
    sDot[i] = (bf16)v;
  }
  for (int i = threadIdx.x; i < 2 * 16 * 16; i += kNT) {
    const int t = i >> 8, q = (i >> 4) & 15, j = i & 15;
    // tile (0, 1) and tile (2, 3) of both score buffers
    const int row = t == 0 ? q : 32 + q, col = t == 0 ? 16 + j : 48 + j;
    sP[sc_off(row, col & ~3) + (col & 3)] = (bf16)0.f;
    sPc[sc_off(row, col & ~3) + (col & 3)] = (bf16)0.f;
  }
  for (int i = threadIdx.x; i < kC + 16; i += kNT) reinterpret_cast<float*>(smem + oQR)[4 * i + 3] = 0.f;
  if (producer) {
    put_m(sDot, mcol, pw, g, c16);
    // table of the diagonal lower-triangular operands: query tile pw, k-step pw / 2
    reinterpret_cast<bf16x8*>(smem + oTri)[pw * 64 + l] = tri_frag(pw >> 1, 16 * pw + c16, g);
  }

  for (int it = 0; it <= x.nch; ++it) {
    wait_vmem();  // this wave's transfers of the previous iteration and its output stores
    lds_barrier();
    const Lane L = lane_opaque();
    // Accumulators that live across the barrier: the producer's M_prev q, or
    // the consumer's S_prev^T q' (one array for both roles).
    f32x4 X[2][4];
    if (producer) {
      if (it < x.nch) {
        switch (pw) {
          case 0: producer_first<0>(x, it, St, X, L); break;
          case 1: producer_first<1>(x, it, St, X, L); break;
          case 2: producer_first<2>(x, it, St, X, L); break;
          default: producer_first<3>(x, it, St, X, L); break;
        }
      }
    } else if (it >= 1) {
      switch (pw) {
        case 0: consumer_first<0>(x, it, St, lz, X, L); break;
        case 1: consumer_first<1>(x, it, St, lz, X, L); break;
        case 2: consumer_first<2>(x, it, St, lz, X, L); break;
        default: consumer_first<3>(x, it, St, lz, X, L); break;
      }
    } else if (x.nch > 0) {
      // iteration 0: the consumers only start the first V and decay transfers
      x.issue_v(0, pw);
      if (pw == 0) x.issue_g(0);
    }
    lds_barrier();  // score tiles, row sums, alpha and mean terms complete
    if (producer) {
      if (it < x.nch) producer_second(x, it, pw, St, mcol, X, L);
    } else if (it >= 1) {
      consumer_second(x, it, pw, St, lz, X, L);
    }
  }

  // the workgroup of the last segment holds the state after the last token
  if (a.st_out && seg == (int)gridDim.x - 1) {
    float* so = a.st_out + (size_t)bh * (2 * kD * kD + kD);
    const float sfin = producer ? 1.f : exp2f(lz.ls);
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = frow(bt, r);
          if (producer) so[kD * kD + row * kD + fcol(t, c16)] = St[bt][t][r];
          else so[row * kD + fcol(t, c16)] = St[bt][t][r] * sfin;
        }
    if (producer && c16 == 0) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) so[2 * kD * kD + 32 * pw + 8 * g + 4 * ct + r] = mcol[ct][r];
    }
  }
}

}  // namespace ccqp

hipError_t ccq_pipe_launch(const CcqPipeLaunch& L, hipStream_t st) {
  ccqp::Args a;
  a.q = static_cast<const bf16*>(L.q);
  a.k = static_cast<const bf16*>(L.k);
  a.v = static_cast<const bf16*>(L.v);
  a.g = L.g;
  a.wl = L.w_lambda;
  a.bl = L.b_lambda;
  a.out = static_cast<bf16*>(L.out);
  a.agg = L.agg;
  a.N = L.N;
  a.H = (int)L.H;
  a.P = (int)L.blocks;
  a.R = (int)L.R;
  a.seg_len = (int)L.seg_len;
  a.sfl = (int)L.sfl;
  a.t_off = L.t_off;
  a.st_out = L.state_out;
  hipLaunchKernelGGL(ccqp::chunk_kernel, dim3((unsigned)L.P, (unsigned)(L.B * L.H)), dim3(ccqp::kNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace lm
