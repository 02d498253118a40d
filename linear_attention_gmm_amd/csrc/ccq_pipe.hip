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
// lambda_i / t_i and beta_i = lambda_i (m_prev . q_i + sum_{j<=i} P_ij) / t_i^2:
//   q'_i - q_i = -alpha_i M_prev q_i + sum_j W_ij k_j + beta_i m_prev,
//   W_ij = beta_i [j <= i] - alpha_i P_ij.
// The chunk's decayed read is then the plain chunkwise form with q':
//   o_i = 2^(l_i) S_prev^T q'_i + sum_{j<=i} 2^(l_i - l_j) (q'_i . k_j) v_j.
//
// MI355X design: a two-stage pipeline inside one workgroup of eight waves (one
// workgroup per CU, one producer and one consumer wave per SIMD).
//  * Producers (waves 0-3) own 32 columns each of M (fp32 registers) and of m.
//    In iteration it they clean the queries of chunk it: raw scores P,
//    gate and mean terms, M_prev q (first half), then W K, the cleaned queries
//    q' (rounded once to bf16, written to LDS as ready-made MFMA fragments) and
//    the update of M and m (second half).
//  * Consumers (waves 4-7) own 32 value columns each of S (fp32 registers). In
//    iteration it they read chunk it-1 with the q' made one iteration earlier:
//    decayed cleaned scores and S_prev^T q' (first half), then the intra-chunk
//    product with V, the output stores and the update of S (second half).
//  * Both halves of an iteration carry about the same matrix-core work for the
//    two waves of a SIMD, and one barrier separates them. Every operand a wave
//    reuses is read from LDS once per chunk; a wave's 32 state columns give
//    each operand fragment two products.
//  * Q/K/V/g tiles arrive by global->LDS DMA one iteration ahead (K in a ring
//    of three: the consumer's, the producer's and the landing one).
//  * The consumers' value columns are permuted within a wave (tile row x of
//    column tile dt is column 8 (x / 4) + 4 dt + x % 4 of the wave's 32), so
//    that each lane ends with eight adjacent outputs of one row: one 16-byte
//    store per lane and query tile.
#include "launch.hpp"
#include "mfma.hpp"

namespace lm {
namespace ccqp {

constexpr int kC = 64;
constexpr int kD = 128;
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int CPR = kD * 2 / 16;  // 16-byte pieces per tile row
constexpr int TB = kC * kD * 2;   // bytes of one 64 x 128 bf16 tile
constexpr int PP = kC + 4;        // pitch (elements) of the score tiles
constexpr int PDD = kD + 4;       // pitch of the gate / mean rows
constexpr float kLog2eF = 1.4426950408889634f;
constexpr float kLazy = 64.f;

// LDS layout (bytes).
constexpr int oK = 0;                    // K ring, 3 swizzled tiles
constexpr int oQ = oK + 3 * TB;          // Q, 2 tiles
constexpr int oV = oQ + 2 * TB;          // V, 2 tiles
constexpr int oQc = oV + 2 * TB;         // cleaned queries as fragments [qt][ks][lane] x 16 B
constexpr int oP = oQc + TB;             // raw masked scores [64 q][PP] fp32
constexpr int oPc = oP + kC * PP * 4;    // cleaned decayed scores [64 q][PP] bf16
constexpr int oDot = oPc + kC * PP * 2;  // [4][PDD] bf16: w hi, w lo, m hi, m lo
constexpr int oG = oDot + 4 * PDD * 2;   // decays, 2 x 64 fp32
constexpr int oRS = oG + 2 * kC * 4;     // partial row sums of P, [2][64] fp32
constexpr int oWQ = oRS + 2 * kC * 4;    // (w . q, m_prev . q) per query, [64] float2
constexpr int oL = oWQ + kC * 8;         // consumers' cumulative decays, [4][64] fp32
constexpr int kLds = oL + 4 * kC * 4;
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

// Score tiles (query tile, key tile <= query tile) of producer / consumer pw.
__device__ __forceinline__ int n_tiles(int pw) { return pw < 2 ? 3 : 2; }
__device__ __forceinline__ void tile_of(int pw, int i, int& qt, int& kt) {
  // pw 0: (0,0) (1,0) (1,1); pw 1: (2,0) (2,1) (2,2); pw 2: (3,0) (3,1); pw 3: (3,2) (3,3)
  if (pw == 0) {
    qt = i == 0 ? 0 : 1;
    kt = i == 2 ? 1 : 0;
  } else if (pw == 1) {
    qt = 2;
    kt = i;
  } else {
    qt = 3;
    kt = 2 * (pw - 2) + i;
  }
}

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

// Tile layout in LDS. A 64 x 128 bf16 tile is 64 rows of 16 pieces of 16
// bytes. Row block rb = r / 16 holds 256 pieces; piece c of row r sits at slot
//   rb * 256 + c * 16 + ((r % 16) ^ 8 (c % 2)).
// Sixteen consecutive rows of one piece are then 256 contiguous bytes (the
// operand reads of 16 rows touch every bank once), a piece's neighbour sits 16
// slots on (row blocks, pieces and k-steps are constant offsets from a per-lane
// base), and the XOR keeps the two pieces of a transposed read in different
// banks. One DMA instruction fills 64 slots: 16 rows x 4 pieces, i.e. 64-byte
// runs of 16 source rows.
__device__ __forceinline__ int slot_off(int rb, int r16, int c) { return (rb * 256 + c * 16 + (r16 ^ ((c & 1) << 3))) * 16; }

// The lane index, hidden from the optimiser once per chunk: the few per-lane
// LDS bases derived from it are recomputed in the loop rather than held in
// registers across it, next to the two state blocks.
struct Lane {
  int l, g, c16;
  int chain;  // CHAIN read of row c16 of a row block, k-step 0, first half
  int kmaj;   // transposed read, rows 4 g + j / 4, first piece pair
  int vf;     // transposed read of the permuted value columns
};
__device__ __forceinline__ Lane lane_opaque() {
  int x = (int)(threadIdx.x & 63);
  asm volatile("" : "+v"(x));
  Lane L;
  L.l = x;
  L.g = x >> 4;
  L.c16 = x & 15;
  const int g = L.g, j = L.c16;
  // CHAIN: piece 4 ks + g / 2 (+2 for the second half), 8 bytes at (g % 2) 8
  L.chain = slot_off(0, j, g >> 1) + (g & 1) * 8;
  // transposed: row 4 g + j / 4, piece (j % 4) / 2, 8 bytes at (j % 2) 8
  L.kmaj = slot_off(0, 4 * g + (j >> 2), (j & 3) >> 1) + (j & 1) * 8;
  // permuted value columns: piece j % 4 (8 value columns each)
  L.vf = slot_off(0, 4 * g + (j >> 2), j & 3);
  return L;
}
// CHAIN fragment (k contiguous along the row) of row 16 rb + c16, k-step ks.
__device__ __forceinline__ bf16x8 chain_rd(const char* t, int rb, int ks, const Lane& L) {
  const char* p = t + rb * 4096 + ks * 1024 + L.chain;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 512);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// k-major CHAIN fragment (k = tokens of step ks): lane p of a 16-lane group
// gets column c0 + p (c0 a multiple of 16). Each lane of the transpose read
// supplies rows 4 g + j / 4 and the 4 columns its group hands to lanes
// 4 (j % 4) .. + 3.
__device__ __forceinline__ bf16x8 kmaj_rd(const char* t, int ks, int c0, const Lane& L) {
  const char* p = t + 2 * ks * 4096 + (c0 >> 3) * 256 + L.kmaj;
  const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p)));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p + 4096)));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// The same for the consumer's permuted value columns: lane p gets column
// base + 8 (p / 4) + 4 dt + p % 4 (base a multiple of 32).
__device__ __forceinline__ bf16x8 v_frag(const char* t, int ks, int base, int dt, const Lane& L) {
  const char* p = t + 2 * ks * 4096 + (base >> 3) * 256 + L.vf + dt * 8;
  const bf16x4 lo = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p)));
  const bf16x4 hi = __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p + 4096)));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}

// This wave's share of the DMA of a 64 x 128 bf16 tile into the layout above:
// instructions 2 w and 2 w + 1 of sixteen, each 64 slots.
struct Dma {
  int voff[2];
  __device__ __forceinline__ void init() {
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int n = 0; n < 2; ++n) {
      const int i = 2 * w + n;
      const int c = (i & 3) * 4 + (l >> 4);
      const int row = 16 * (i >> 2) + ((l & 15) ^ ((c & 1) << 3));
      voff[n] = row * (kD * 2) + c * 16;
    }
  }
  __device__ __forceinline__ void issue(char* dst, const bf16* src, int rows) const {
    const u32x4 d = buf_desc(src, (uint32_t)((rows < kC ? rows : kC) * kD * 2));
    const unsigned base = lds_addr(dst) + (unsigned)(wave_id() * 2 * 1024);
#pragma unroll
    for (int n = 0; n < 2; ++n) lds_dma16(d, voff[n], base + (unsigned)(n * 1024));
  }
};

// CHAIN fragment of a plain row-major bf16 tile (ld_kc_chain).
__device__ __forceinline__ bf16x8 kc_rd(const bf16* base, int pitch, int rc, int ks, int g) {
  const bf16* p = base + rc * pitch + ks * 32 + 4 * g;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
// token index of element e of a CHAIN fragment of step ks
__device__ __forceinline__ int chk(int ks, int e, int g) { return ks * 32 + (e < 4 ? 4 * g + e : 12 + 4 * g + e); }

__device__ __forceinline__ bf16x8 zero8() {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)0.f;
  return f;
}

__device__ __forceinline__ bf16x8 ones8() {
  bf16x8 f;
#pragma unroll
  for (int i = 0; i < 8; ++i) f[i] = (bf16)1.f;
  return f;
}

__device__ __forceinline__ void put4(bf16* dst, const f32x4& v) {
  *reinterpret_cast<bf16x4*>(dst) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}

// Writes m (this producer's 32 entries, rows 4 g + r of column tiles ct) as
// the bf16 hi / lo rows 2 and 3 of the gate / mean operand.
__device__ __forceinline__ void put_m(bf16* sDot, const float (&m)[2][4], int pw) {
  const int g = lane_id() >> 4, c16 = lane_id() & 15;
  if (c16 == 0) {
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int a = 32 * pw + 16 * ct + 4 * g + r;
        const bf16 hi = (bf16)m[ct][r];
        sDot[2 * PDD + a] = hi;
        sDot[3 * PDD + a] = (bf16)(m[ct][r] - (float)hi);
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
  const int64_t t_begin = (int64_t)seg * a.seg_len;
  const int64_t t_end = N < t_begin + a.seg_len ? N : t_begin + a.seg_len;
  const int nch = (int)((t_end - t_begin + kC - 1) / kC);
  const bf16* Qg = a.q + (size_t)bh * N * kD;
  const bf16* Kg = a.k + (size_t)bh * N * kD;
  const bf16* Vg = a.v + (size_t)bh * N * kD;
  const float* Gg = a.g + (size_t)bh * N;
  bf16* Og = a.out + (size_t)bh * N * kD;
  const float gate_b = a.bl[h];

  float* sP = reinterpret_cast<float*>(smem + oP);
  bf16* sPc = reinterpret_cast<bf16*>(smem + oPc);
  bf16* sDot = reinterpret_cast<bf16*>(smem + oDot);
  float* sRS = reinterpret_cast<float*>(smem + oRS);
  float2* sWQ = reinterpret_cast<float2*>(smem + oWQ);
  float* sLw = reinterpret_cast<float*>(smem + oL) + pw * kC;

  Dma dma;
  dma.init();
  auto issue = [&](int tile, int c) {  // tile 0 = Q, 1 = K, 2 = V, 3 = g of chunk c
    const int64_t c0 = t_begin + (int64_t)c * kC;
    const int nv = (int)((t_end - c0) < kC ? (t_end - c0) : kC);
    if (tile == 0) dma.issue(smem + oQ + (c & 1) * TB, Qg + (size_t)c0 * kD, nv);
    else if (tile == 1) dma.issue(smem + oK + (c % 3) * TB, Kg + (size_t)c0 * kD, nv);
    else if (tile == 2) dma.issue(smem + oV + (c & 1) * TB, Vg + (size_t)c0 * kD, nv);
    else if (w == 0) lds_dma4(buf_desc(Gg + c0, (uint32_t)(nv * 4)), l * 4, lds_addr(smem + oG + (c & 1) * kC * 4));
  };
  if (nch > 0) {
    issue(0, 0);
    issue(1, 0);
  }

  // State: producers M[:, 32 pw + 16 ct + c16] as St[bt][ct] (rows 16 bt + 4 g + r)
  // and m; consumers S[16 bt + 4 g + r][value column of (dt, c16)] as St[bt][dt].
  f32x4 St[8][2];
  float mcol[2][4];
  float ls = 0.f;  // consumers: S_true = 2^ls St
  // the consumer's value column for tile dt and tile column x
  const int vbase = 32 * pw;
  auto vcol = [&](int dt, int x) { return vbase + 8 * (x >> 2) + 4 * dt + (x & 3); };
  {
    const float* blk = a.agg ? a.agg + ((size_t)bh * a.P + (size_t)a.R * seg) * a.sfl : nullptr;
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * bt + 4 * g + r;
          float x = 0.f;
          if (blk) x = producer ? blk[kD * kD + 1 + row * kD + 32 * pw + 16 * t + c16] : blk[row * kD + vcol(t, c16)];
          St[bt][t][r] = x;
        }
#pragma unroll
    for (int ct = 0; ct < 2; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) mcol[ct][r] = blk ? blk[2 * kD * kD + 1 + 32 * pw + 16 * ct + 4 * g + r] : 0.f;
  }
  // gate weights (rows 0 / 1, hi / lo), the zero score tiles above the
  // diagonal that the k-steps of 32 keys read, partial row sums slot 1
  for (int i = threadIdx.x; i < 4 * PDD; i += kNT) {
    const int row = i / PDD, col = i - (i / PDD) * PDD;
    if (row == 2 || row == 3) continue;
    float v = 0.f;
    if (col < kD && row < 2) {
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
    sP[row * PP + col] = 0.f;
    sPc[row * PP + col] = (bf16)0.f;
  }
  for (int i = threadIdx.x; i < kC; i += kNT) sRS[kC + i] = 0.f;
  if (producer) put_m(sDot, mcol, pw);

  const int64_t t_tok0 = t_begin + a.t_off;  // tokens before the segment's first one (count for CCQ)

  for (int it = 0; it <= nch; ++it) {
    const Lane L = lane_opaque();
    const int l = L.l, g = L.g, c16 = L.c16;
    wait_vmem();  // this wave's DMA of the previous iteration and its output stores
    lds_barrier();
    if (it + 1 < nch) {
      issue(0, it + 1);
      issue(1, it + 1);
    }
    if (it < nch) {
      issue(2, it);
      issue(3, it);
    }

    if (producer) {
      if (it < nch) {
        // ------------------------------------------------ producer, first half
        const char* Qt = smem + oQ + (it & 1) * TB;
        const char* Kt = smem + oK + (it % 3) * TB;
        // gate logit w . q and mean term m_prev . q of query tile pw
        {
          f32x4 dq = zero4();
#pragma unroll
          for (int s = 0; s < 4; ++s)
            dq = Mma<bf16>::mma(c16 < 4 ? kc_rd(sDot, PDD, c16, s, g) : zero8(), chain_rd(Qt, pw, s, L), dq);
          if (g == 0) sWQ[16 * pw + c16] = make_float2(dq[0] + dq[1], dq[2] + dq[3]);
        }
        // raw masked scores of this producer's tiles and their row sums
        {
          const int nt = n_tiles(pw);
          float rs0 = 0.f, rs1 = 0.f;
          int qt0 = -1;
          for (int i = 0; i < nt; ++i) {
            int qt, kt;
            tile_of(pw, i, qt, kt);
            bf16x8 kf[4], qf[4];
#pragma unroll
            for (int s = 0; s < 4; ++s) {
              kf[s] = chain_rd(Kt, kt, s, L);
              qf[s] = chain_rd(Qt, qt, s, L);
            }
            f32x4 acc = zero4();
#pragma unroll
            for (int s = 0; s < 4; ++s) acc = Mma<bf16>::mma(kf[s], qf[s], acc);
            if (kt == qt) {
#pragma unroll
              for (int r = 0; r < 4; ++r)
                if (4 * g + r > c16) acc[r] = 0.f;
            }
            *reinterpret_cast<f32x4*>(sP + (16 * qt + c16) * PP + 16 * kt + 4 * g) = acc;
            const float part = acc[0] + acc[1] + acc[2] + acc[3];
            if (qt0 < 0) qt0 = qt;
            if (qt == qt0) rs0 += part; else rs1 += part;
          }
          rs0 = group_sum(rs0);
          rs1 = group_sum(rs1);
          const int slot = pw == 3 ? 1 : 0;
          if (g == 0) {
            sRS[slot * kC + 16 * qt0 + c16] = rs0;
            if (pw == 0) sRS[16 + c16] = rs1;  // producer 0 also owns query tile 1
          }
        }
      }
    } else if (it >= 1) {
      // -------------------------------------------------- consumer, first half
      const int c = it - 1;
      const float* gt = reinterpret_cast<const float*>(smem + oG + (c & 1) * kC * 4);
      const int64_t c0 = t_begin + (int64_t)c * kC;
      const int nvalid = (int)((t_end - c0) < kC ? (t_end - c0) : kC);
      // cumulative log2 decay of the chunk (lane = token; g in (0, 1], 0 clamped)
      float l_mine, l_last;
      {
        float x = l < nvalid ? fmaxf(__builtin_amdgcn_logf(gt[l]), -200.f) : 0.f;
        x = wave_scan_incl(x);
        l_mine = x;
        l_last = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), kC - 1));
        sLw[l] = x;
      }
      __builtin_amdgcn_wave_barrier();
      (void)l_mine;
      (void)l_last;
    }
    // (the consumer's first half continues below; the split keeps the
    // decay scan ahead of the fragment loads)
    if (!producer && it >= 1) {
      const int c = it - 1;
      const char* Kt = smem + oK + (c % 3) * TB;
      const bf16x8* Qc = reinterpret_cast<const bf16x8*>(smem + oQc);
      // decayed cleaned scores of this consumer's tiles
      const int nt = n_tiles(pw);
      for (int i = 0; i < nt; ++i) {
        int qt, kt;
        tile_of(pw, i, qt, kt);
        bf16x8 kf[4], qf[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          kf[s] = chain_rd(Kt, kt, s, L);
          qf[s] = Qc[(qt * 4 + s) * 64 + l];
        }
        f32x4 acc = zero4();
#pragma unroll
        for (int s = 0; s < 4; ++s) acc = Mma<bf16>::mma(kf[s], qf[s], acc);
        const f32x4 d = decay_tile(sLw, sLw[16 * qt + c16], kt, qt, g, c16);
        put4(sPc + (16 * qt + c16) * PP + 16 * kt + 4 * g, acc * d);
      }
    }
    // Accumulators that live across the barrier: the consumer's inter-chunk
    // read S_prev^T q', or the producer's M_prev q (one array for both roles).
    f32x4 X[2][4];
    if (!producer && it >= 1) {
      const bf16x8* Qc = reinterpret_cast<const bf16x8*>(smem + oQc);
      // k-step outer: one bf16 copy of two S row blocks and one q' fragment at
      // a time, eight independent accumulators
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) X[dt][qt] = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 sa0 = Mma<bf16>::chain2(St[2 * s][0], St[2 * s + 1][0]);
        const bf16x8 sa1 = Mma<bf16>::chain2(St[2 * s][1], St[2 * s + 1][1]);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const bf16x8 qf = Qc[(qt * 4 + s) * 64 + l];
          X[0][qt] = Mma<bf16>::mma(sa0, qf, X[0][qt]);
          X[1][qt] = Mma<bf16>::mma(sa1, qf, X[1][qt]);
        }
      }
    }
    if (producer && it < nch) {
      const char* Qt = smem + oQ + (it & 1) * TB;
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) X[ct][qt] = zero4();
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const bf16x8 ma0 = Mma<bf16>::chain2(St[2 * s][0], St[2 * s + 1][0]);
        const bf16x8 ma1 = Mma<bf16>::chain2(St[2 * s][1], St[2 * s + 1][1]);
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const bf16x8 qf = chain_rd(Qt, qt, s, L);
          X[0][qt] = Mma<bf16>::mma(ma0, qf, X[0][qt]);
          X[1][qt] = Mma<bf16>::mma(ma1, qf, X[1][qt]);
        }
      }
    }

    lds_barrier();  // scores, row sums, gate / mean terms, cleaned scores complete

    if (producer) {
      if (it < nch) {
        // ------------------------------------------------ producer, second half
        const char* Qt = smem + oQ + (it & 1) * TB;
        const char* Kt = smem + oK + (it % 3) * TB;
        const int64_t t0 = t_tok0 + (int64_t)it * kC;
        float al[4], be[4];
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const int i = 16 * qt + c16;
          const float2 wm = sWQ[i];
          const float rs = sRS[i] + sRS[kC + i];
          const float lam = __builtin_amdgcn_rcpf(1.f + fast_exp2(-(wm.x + gate_b) * kLog2eF));
          const float inv_t = __builtin_amdgcn_rcpf((float)t0 + (float)(i + 1));
          al[qt] = lam * inv_t;
          be[qt] = al[qt] * (wm.y + rs) * inv_t;
        }
        // K^T of this producer's 32 columns (rows a, k = tokens)
        bf16x8 KC[2][2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
          for (int s = 0; s < 2; ++s) KC[ct][s] = kmaj_rd(Kt, s, 32 * pw + 16 * ct, L);
        // W K, W_ij = beta_i [j <= i] - alpha_i P_ij, then delta and q' = q + delta
#pragma unroll
        for (int qt = 0; qt < 4; ++qt) {
          const int i = 16 * qt + c16;
          f32x4 wk[2] = {zero4(), zero4()};
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            if (s == 1 && qt < 2) continue;  // keys 32..63 lie above the diagonal
            // fp32 scores: W nearly cancels (exactly for one token), so it is
            // formed in fp32 and rounded once
            const float* prow = sP + i * PP + 32 * s + 4 * g;
            const f32x4 p0 = *reinterpret_cast<const f32x4*>(prow);
            const f32x4 p1 = *reinterpret_cast<const f32x4*>(prow + 16);
            bf16x8 wf;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int j = chk(s, e, g);
              const float pv = e < 4 ? p0[e] : p1[e - 4];
              wf[e] = (bf16)((j <= i ? be[qt] : 0.f) - al[qt] * pv);
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) wk[ct] = Mma<bf16>::mma(KC[ct][s], wf, wk[ct]);
          }
          const bf16x8 qv = chain_rd(Qt, qt, pw, L);
          bf16x8 qc;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int ct = e >> 2, r = e & 3;
            const float dl = -al[qt] * X[ct][qt][r] + wk[ct][r] + be[qt] * mcol[ct][r];
            qc[e] = (bf16)((float)qv[e] + dl);
          }
          reinterpret_cast<bf16x8*>(smem + oQc)[(qt * 4 + pw) * 64 + l] = qc;
        }
        // M += K^T K[:, cols], m += column sums of K[:, cols]
#pragma unroll
        for (int bt = 0; bt < 8; ++bt) {
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bf16x8 kf = kmaj_rd(Kt, s, 16 * bt, L);
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) St[bt][ct] = Mma<bf16>::mma(kf, KC[ct][s], St[bt][ct]);
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
        put_m(sDot, mcol, pw);
      }
    } else if (it >= 1) {
      // -------------------------------------------------- consumer, second half
      const int c = it - 1;
      const char* Kt = smem + oK + (c % 3) * TB;
      const char* Vt = smem + oV + (c & 1) * TB;
      const int64_t c0 = t_begin + (int64_t)c * kC;
      const int nvalid = (int)((t_end - c0) < kC ? (t_end - c0) : kC);
      const float l_mine = sLw[l];
      const float l_last = sLw[kC - 1];
      bf16x8 VF[2][2];
#pragma unroll
      for (int dt = 0; dt < 2; ++dt)
#pragma unroll
        for (int s = 0; s < 2; ++s) VF[dt][s] = v_frag(Vt, s, vbase, dt, L);
      // intra-chunk product, the inter-chunk part scaled by 2^(l_i + ls), stores
#pragma unroll
      for (int qt = 0; qt < 4; ++qt) {
        const int i = 16 * qt + c16;
        f32x4 acc[2] = {zero4(), zero4()};
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          if (s == 1 && qt < 2) continue;
          const bf16x8 pf = kc_rd(sPc, PP, i, s, g);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) acc[dt] = Mma<bf16>::mma(VF[dt][s], pf, acc[dt]);
        }
        const float bq = fast_exp2(sLw[i] + ls);
        bf16x8 o;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          o[r] = (bf16)(acc[0][r] + bq * X[0][qt][r]);
          o[4 + r] = (bf16)(acc[1][r] + bq * X[1][qt][r]);
        }
        if (i < nvalid) *reinterpret_cast<bf16x8*>(Og + (size_t)(c0 + i) * kD + vbase + 8 * g) = o;
      }
      // S <- 2^l_last S + K^T (2^(l_last - l_j) V), held as 2^ls S (lazy decay)
      const float ls_next = ls + l_last;
      float wb;
      if (ls_next < -kLazy) {
        const float b = fast_exp2(ls_next);
#pragma unroll
        for (int bt = 0; bt < 8; ++bt)
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) St[bt][dt] *= b;
        ls = 0.f;
        wb = l_last;
      } else {
        wb = -ls;
        ls = ls_next;
      }
      sLw[l] = fast_exp2(wb - l_mine);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        float wt[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) wt[e] = sLw[chk(s, e, g)];
#pragma unroll
        for (int dt = 0; dt < 2; ++dt)
#pragma unroll
          for (int e = 0; e < 8; ++e) VF[dt][s][e] = (bf16)((float)VF[dt][s][e] * wt[e]);
      }
#pragma unroll
      for (int bt = 0; bt < 8; ++bt) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          const bf16x8 kf = kmaj_rd(Kt, s, 16 * bt, L);
#pragma unroll
          for (int dt = 0; dt < 2; ++dt) St[bt][dt] = Mma<bf16>::mma(kf, VF[dt][s], St[bt][dt]);
        }
      }
    }
  }

  // the workgroup of the last segment holds the state after the last token
  if (a.st_out && seg == (int)gridDim.x - 1) {
    float* so = a.st_out + (size_t)bh * (2 * kD * kD + kD);
    const float sfin = producer ? 1.f : exp2f(ls);
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int row = 16 * bt + 4 * g + r;
          if (producer) so[kD * kD + row * kD + 32 * pw + 16 * t + c16] = St[bt][t][r];
          else so[row * kD + vcol(t, c16)] = St[bt][t][r] * sfin;
        }
    if (producer && c16 == 0) {
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) so[2 * kD * kD + 32 * pw + 16 * ct + 4 * g + r] = mcol[ct][r];
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
