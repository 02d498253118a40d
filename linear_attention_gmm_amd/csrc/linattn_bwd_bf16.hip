// linattn_bwd_bf16.hip -- backward pass of decayed linear attention (scalar
// gate per token) for bf16 inputs with d_k = d_v = 128, on gfx950.
//
// Method (allinfo.ai.kr linear attention post, "Key messages": the matrix
// state S_t = g_t S_{t-1} + k_t v_t^T read as o_t = S_t^T q_t, and the
// chunkwise form that makes training parallel; the gradients follow from the
// recurrence). Per (b, h) and chunk of 64 tokens, with l_i the cumulative log2
// gate inside the chunk up to token i and L = l_63:
//   dq_i = 2^(l_i) S do_i + sum_{j<=i} A_ij k_j,      A_ij = 2^(l_i - l_j) (do_i . v_j)
//   S   <- 2^L S + sum_j 2^(L - l_j) k_j v_j^T         (S before the chunk; forward sweep)
//   dk_j = 2^(L - l_j) U v_j + sum_{i>=j} A_ij q_i
//   dv_j = 2^(L - l_j) U^T k_j + sum_{i>=j} B_ij do_i, B_ij = 2^(l_i - l_j) (q_i . k_j)
//   U   <- 2^L U + sum_i 2^(l_i) q_i do_i^T            (U after the chunk; reverse sweep)
//   dg_t = (1 / g_t) sum_{m>=t} (q_m . dq_m - k_m . dk_m)
// U is the gradient of the state after the chunk (zero after the last token).
// Every decay factor above is at most 1. The gates enter as log2 g clamped at
// -200, as in the forward kernels.
//
// Precision. dg is a suffix sum of q . dq - k . dk, two terms that nearly
// cancel, so dq and dk must be accurate well beyond bf16. The inputs are exact
// in bf16; every other MFMA operand of the dq and dk products (the states S and
// U, the decayed scores A, the decay-weighted keys and queries of the state
// updates) is split into x = hi + lo with hi = bf16(x), lo = bf16(x - hi),
// which holds about 16 significant bits, and multiplied as two products. dv
// does not enter dg: its products use the bf16 hi part only, like the forward.
//
// MI355X design: one launch of 2 B H workgroups of eight waves, one per CU.
//  * Workgroups [0, BH) sweep their sequence forwards and make dq. Wave w owns
//    feature rows a = 16 w .. 16 w + 15 of S (as S^T tiles, 32 VGPRs) and of
//    dq. Each chunk: the ten lower-triangular 16 x 16 tiles of A (shared out
//    over the waves, written to LDS as hi and lo), S do, a barrier, A k, the
//    dq stores, then the state update.
//  * Workgroups [BH, 2 BH) sweep backwards. Waves 0-3 own rows a = 32 w ..
//    32 w + 31 of U (as U^T tiles) and make dk; waves 4-7 own columns b =
//    32 (w - 4) .. + 31 of a second copy of U (kept to bf16-product accuracy,
//    which is what dv needs) and make dv. Wave w and w + 4 share a SIMD, and
//    their matrix work per chunk is about the same (162 and 86 products: the
//    dk side has the split operands).
//  * The two kinds run side by side on different CUs. q . dq and k . dk are
//    summed per token across the waves through LDS and written as float32;
//    a second small kernel forms the suffix sums.
//  * Q, K, V and dO tiles arrive by global->LDS DMA into two sets of
//    swizzled tiles, one chunk ahead. Out-of-range rows of the last chunk read
//    as zeros; their gates count as 1; their stores fall outside the buffer
//    range and are dropped.
#include "launch.hpp"
#include "mfma.hpp"

namespace lm {
namespace lbw {

constexpr int kC = 64;
constexpr int kD = 128;
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int CPR = kD * 2 / 16;  // 16-byte pieces of a 128-wide bf16 row
constexpr int SPR = kC * 2 / 16;  // pieces of a 64-wide bf16 score row
constexpr int TB = kC * kD * 2;   // one 64 x 128 bf16 tile
constexpr int SB = kC * kC * 2;   // one 64 x 64 bf16 score tile
constexpr float kMinLog2G = -200.f;

enum { tQ = 0, tK = 1, tV = 2, tO = 3 };
// LDS layout (bytes): two sets of the Q, K, V, dO tiles; the score tiles A hi,
// A lo and B; per-wave partial dot products per token.
constexpr int oT = 0;
constexpr int oAh = oT + 8 * TB;
constexpr int oAl = oAh + SB;
constexpr int oB = oAl + SB;
constexpr int oX = oB + SB;
constexpr int oXs = oX + kNW * kC * 4;  // per-wave <dS_out, S_out> partials
constexpr int kLds = oXs + kNW * 4;
static_assert(kLds <= 160 * 1024, "LDS budget");

// The ten 16 x 16 tiles (query tile it >= key tile jt) of a chunk's scores.
__device__ __forceinline__ int tile_it(int p) { return p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 2 : 3; }
__device__ __forceinline__ int tile_jt(int p) { return p - (p < 1 ? 0 : p < 3 ? 1 : p < 6 ? 3 : 6); }

typedef unsigned u32x2 __attribute__((ext_vector_type(2)));

struct Args {
  const bf16* q;
  const bf16* k;
  const bf16* v;
  const bf16* dout;
  const float* g;
  bf16* dq;
  bf16* dk;
  bf16* dv;
  float* xq;  // [BH][N]: q . dq (float32)
  float* xk;  // [BH][N]: k . dk (float32)
  // optional carried state ([BH][128][128] float32, S[a][b] at a * 128 + b):
  const float* state_in;    // the state before the first token
  const float* dstate_out;  // the loss gradient of the state after the last token
  float* dstate_in;         // output: the gradient of state_in
  int64_t N;
  int BH;
};

__device__ __forceinline__ char* tile(char* smem, int set, int t) { return smem + oT + (4 * set + t) * TB; }

// hi + lo split of eight floats.
__device__ __forceinline__ void split8(const float (&x)[8], bf16x8& hi, bf16x8& lo) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    hi[e] = (bf16)x[e];
    lo[e] = (bf16)(x[e] - (float)hi[e]);
  }
}
// CHAIN fragment (rows 4g..4g+3 of two stacked 16-row tiles) of float32 tiles, split.
__device__ __forceinline__ void split_chain(const f32x4& t0, const f32x4& t1, bf16x8& hi, bf16x8& lo) {
  float x[8];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    x[r] = t0[r];
    x[4 + r] = t1[r];
  }
  split8(x, hi, lo);
}

__device__ __forceinline__ f32x4 mma(const bf16x8& a, const bf16x8& b, const f32x4& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Per-chunk decays of one wave: lc = inclusive prefix over the chunk of the
// clamped log2 gates (lane = token; 0 past the end), L = lc at token 63.
struct Decay {
  float lc, L;
  __device__ __forceinline__ void make(float gv, bool valid) {
    const float x = valid ? fmaxf(__builtin_amdgcn_logf(gv), kMinLog2G) : 0.f;
    lc = wave_scan_incl(x);
    L = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lc), kC - 1));
  }
  __device__ __forceinline__ float at(int t) const { return __shfl(lc, t); }
};

// One 16 x 16 score tile p of the chunk: rows j (key tile jt) of R, columns i
// (query tile it) of C: s_ij = 2^(l_i - l_j) (C_i . R_j) for i >= j, else 0,
// written to the row-major score tile(s) [i][j] (hi, and lo when given).
__device__ __forceinline__ void score_tile(int p, const char* tR, const char* tC, const Decay& dc, char* dhi,
                                           char* dlo) {
  const int l = lane_id(), g = l >> 4, c16 = l & 15;
  const int it = tile_it(p), jt = tile_jt(p);
  f32x4 acc = zero4();
#pragma unroll
  for (int ks = 0; ks < kD / 32; ++ks)
    acc = mma(tl_nat<CPR>(tR, 16 * jt + c16, ks), tl_nat<CPR>(tC, 16 * it + c16, ks), acc);
  const int i = 16 * it + c16;
  const float li = dc.at(i);
  // the lane shuffles run on every lane: a shuffle under the mask below
  // would read the decays of lanes it has switched off
  float lj[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) lj[r] = dc.at(16 * jt + 4 * g + r);
  bf16x4 h, lo;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int j = 16 * jt + 4 * g + r;
    const float e = fast_exp2(li - lj[r]);
    const float x = i >= j ? acc[r] * e : 0.f;
    h[r] = (bf16)x;
    lo[r] = (bf16)(x - (float)h[r]);
  }
  const int off = tile_off<SPR, 2>(i, 16 * jt + 4 * g);
  *reinterpret_cast<bf16x4*>(dhi + off) = h;
  if (dlo) *reinterpret_cast<bf16x4*>(dlo + off) = lo;
}

// Zero blocks of the score tiles that the intra-chunk products read but no
// score tile writes: rows 0-15 x columns 16-31 and rows 32-47 x columns 48-63.
__device__ __forceinline__ void zero_upper(char* smem) {
  for (int e = threadIdx.x; e < 3 * 2 * 16 * 4; e += kNT) {
    const int t = e / 128, rem = e % 128, blk = rem / 64, rr = (rem % 64) / 4, q4 = rem % 4;
    const int row = 32 * blk + rr, col = 32 * blk + 16 + 4 * q4;
    *reinterpret_cast<bf16x4*>(smem + oAh + t * SB + tile_off<SPR, 2>(row, col)) =
        bf16x4{(bf16)0.f, (bf16)0.f, (bf16)0.f, (bf16)0.f};
  }
}

// Buffer resource over one (b, h) block of a [.., N, 128] bf16 tensor; stores
// past the sequence end are dropped by the range check.
__device__ __forceinline__ rsrc_t seq_rsrc(const bf16* base, int64_t N) {
  return make_rsrc(base, (uint32_t)(N * kD * 2));
}
__device__ __forceinline__ void store4(const f32x4& x, const rsrc_t& rs, int64_t row, int col) {
  const bf16x4 o{(bf16)x[0], (bf16)x[1], (bf16)x[2], (bf16)x[3]};
  __builtin_amdgcn_raw_buffer_store_b64(__builtin_bit_cast(u32x2, o), rs, (int)((row * kD + col) * 2), 0, 0);
}

// Sum of the per-wave partials of the chunk at t0 (nw waves), one lane per
// token, written to x[t0 + lane] for tokens inside the sequence; `last` is
// added to the sequence's last token.
__device__ __forceinline__ void flush_dots(const char* smem, int nw, float* x, int64_t t0, int64_t N,
                                           float last = 0.f) {
  const int l = lane_id();
  const float* sX = reinterpret_cast<const float*>(smem + oX);
  float s = 0.f;
  for (int u = 0; u < nw; ++u) s += sX[u * kC + l];
  if (t0 + l == N - 1) s += last;
  if (t0 + l < N) x[t0 + l] = s;
}

// ---------------------------------------------------------------------------
// Forward sweep: dq and q . dq.
__device__ __forceinline__ void dq_sweep(const Args& a, char* smem, int bh) {
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const int64_t N = a.N;
  const int nch = (int)((N + kC - 1) / kC);
  const size_t base = (size_t)bh * N * kD;
  const bf16* src[4] = {a.q + base, a.k + base, a.v + base, a.dout + base};
  const float* G = a.g + (size_t)bh * N;
  const rsrc_t ors = seq_rsrc(a.dq + base, N);
  float* xq = a.xq + (size_t)bh * N;
  float* sX = reinterpret_cast<float*>(smem + oX);
  const int a0 = 16 * w;  // this wave's feature rows

  TileDma<bf16, kD, kNW> dma;
  dma.init();
  zero_upper(smem);
#pragma unroll
  for (int t = 0; t < 4; ++t) dma.issue(tile(smem, 0, t), src[t], (int)(N < kC ? N : kC));
  float gnext = l < N ? G[l] : 1.f;

  f32x4 ST[8];  // S^T: tile bt holds rows b = 16 bt + 4g + r, column a = a0 + c16
  const size_t sbase = (size_t)bh * kD * kD + (size_t)(a0 + c16) * kD;  // row a of this lane's S
#pragma unroll
  for (int bt = 0; bt < 8; ++bt)
#pragma unroll
    for (int r = 0; r < 4; ++r) ST[bt][r] = a.state_in ? a.state_in[sbase + 16 * bt + 4 * g + r] : 0.f;

  for (int c = 0; c < nch; ++c) {
    const int set = c & 1;
    const int64_t t0 = (int64_t)c * kC;
    Decay dc;
    dc.make(gnext, t0 + l < N);
    wait_vmem();
    lds_barrier();
    if (c + 1 < nch) {
      const int64_t tn = t0 + kC;
      const int rows = (int)(N - tn < kC ? N - tn : kC);
#pragma unroll
      for (int t = 0; t < 4; ++t) dma.issue(tile(smem, set ^ 1, t), src[t] + tn * kD, rows);
      gnext = tn + l < N ? G[tn + l] : 1.f;
    }
    const char* tq = tile(smem, set, tQ);
    const char* tk = tile(smem, set, tK);
    const char* tv = tile(smem, set, tV);
    const char* to = tile(smem, set, tO);
    if (c > 0 && w == kNW - 1) flush_dots(smem, kNW, xq, t0 - kC, N);

    // scores A (rows j of V, columns i of dO), hi and lo
    score_tile(w, tv, to, dc, smem + oAh, smem + oAl);
    if (w < 2) score_tile(w + 8, tv, to, dc, smem + oAh, smem + oAl);

    lds_barrier();

    // inter-chunk part: dq[a][i] = 2^(l_i) sum_b S[a][b] do_i[b]
    f32x4 acc[4];
#pragma unroll
    for (int it = 0; it < 4; ++it) acc[it] = zero4();
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      bf16x8 sh, sl;
      split_chain(ST[2 * s], ST[2 * s + 1], sh, sl);
#pragma unroll
      for (int it = 0; it < 4; ++it) {
        const bf16x8 bo = tl_chain<CPR>(to, 16 * it + c16, s);
        acc[it] = mma(sh, bo, acc[it]);
        acc[it] = mma(sl, bo, acc[it]);
      }
    }
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const float f = fast_exp2(dc.at(16 * it + c16));
#pragma unroll
      for (int r = 0; r < 4; ++r) acc[it][r] *= f;
    }
    // K^T fragments (rows a, k = tokens j), for A k and the state update
    bf16x8 kf[2];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) kf[ks] = tl_kmaj<CPR>(tk, ks, a0);

    // intra-chunk part: dq[a][i] += sum_{j<=i} k_j[a] A_ij
#pragma unroll
    for (int it = 0; it < 4; ++it) {
#pragma unroll
      for (int ks = 0; ks <= it / 2; ++ks) {
        const bf16x8 ah = tl_chain<SPR>(smem + oAh, 16 * it + c16, ks);
        const bf16x8 al = tl_chain<SPR>(smem + oAl, 16 * it + c16, ks);
        acc[it] = mma(kf[ks], ah, acc[it]);
        acc[it] = mma(kf[ks], al, acc[it]);
      }
    }
    // stores of dq (four features of token i per lane) and q . dq partials
#pragma unroll
    for (int it = 0; it < 4; ++it) {
      const int i = 16 * it + c16;
      store4(acc[it], ors, t0 + i, a0 + 4 * g);
      const bf16x4 q4 = *reinterpret_cast<const bf16x4*>(tq + tile_off<CPR, 2>(i, a0 + 4 * g));
      float p = 0.f;
#pragma unroll
      for (int r = 0; r < 4; ++r) p += (float)q4[r] * acc[it][r];
      p = group_sum(p);
      if (g == 0) sX[w * kC + i] = p;
    }

    // state update: S^T = 2^L S^T + V^T (w K), w_j = 2^(L - l_j)
    const float fL = fast_exp2(dc.L);
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int r = 0; r < 4; ++r) ST[bt][r] *= fL;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float x[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) x[e] = (float)kf[ks][e] * fast_exp2(dc.L - dc.at(chain_k<bf16>(ks, e)));
      bf16x8 kh, kl;
      split8(x, kh, kl);
#pragma unroll
      for (int bt = 0; bt < 8; ++bt) {
        const bf16x8 va = tl_kmaj<CPR>(tv, ks, 16 * bt);
        ST[bt] = mma(va, kh, ST[bt]);
        ST[bt] = mma(va, kl, ST[bt]);
      }
    }
  }
  // with a gradient for the state after the last token, the gates also reach
  // the loss through S_out: the last token's q . dq - k . dk gains <dS_out, S_out>
  if (a.dstate_out) {
    float p = 0.f;
#pragma unroll
    for (int bt = 0; bt < 8; ++bt)
#pragma unroll
      for (int r = 0; r < 4; ++r) p += ST[bt][r] * a.dstate_out[sbase + 16 * bt + 4 * g + r];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) p += __shfl_xor(p, off);
    if (l == 0) reinterpret_cast<float*>(smem + oXs)[w] = p;
  }
  lds_barrier();
  if (nch > 0 && w == kNW - 1) {
    float last = 0.f;
    if (a.dstate_out)
      for (int u = 0; u < kNW; ++u) last += reinterpret_cast<const float*>(smem + oXs)[u];
    flush_dots(smem, kNW, xq, (int64_t)(nch - 1) * kC, N, last);
  }
}

// ---------------------------------------------------------------------------
// Reverse sweep: dk, dv and k . dk.
__device__ __forceinline__ void dkv_sweep(const Args& a, char* smem, int bh) {
  const int l = lane_id(), w = wave_id(), g = l >> 4, c16 = l & 15;
  const bool kside = w < 4;          // dk waves; the others make dv
  const int f0 = 32 * (w & 3);       // first of this wave's 32 feature rows (a) or columns (b)
  const int64_t N = a.N;
  const int nch = (int)((N + kC - 1) / kC);
  const size_t base = (size_t)bh * N * kD;
  const bf16* src[4] = {a.q + base, a.k + base, a.v + base, a.dout + base};
  const float* G = a.g + (size_t)bh * N;
  const rsrc_t ors = seq_rsrc((kside ? a.dk : a.dv) + base, N);
  float* xk = a.xk + (size_t)bh * N;
  float* sX = reinterpret_cast<float*>(smem + oX);

  TileDma<bf16, kD, kNW> dma;
  dma.init();
  zero_upper(smem);
  const int64_t tl0 = (int64_t)(nch - 1) * kC;
  if (nch > 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) dma.issue(tile(smem, 0, t), src[t] + tl0 * kD, (int)(N - tl0));
  }
  float gnext = nch > 0 && tl0 + l < N ? G[tl0 + l] : 1.f;

  // dk waves: U^T, U[f][bt] rows b = 16 bt + 4g + r, column a = f0 + 16 f + c16.
  // dv waves: U, U[f][at] rows a = 16 at + 4g + r, column b = f0 + 16 f + c16.
  f32x4 U[2][8];
  // U starts as the gradient of the state after the last token (zero without one)
  const float* du = a.dstate_out ? a.dstate_out + (size_t)bh * kD * kD : nullptr;
#pragma unroll
  for (int f = 0; f < 2; ++f)
#pragma unroll
    for (int t = 0; t < 8; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int x = f0 + 16 * f + c16, y = 16 * t + 4 * g + r;  // column, row of the tile
        U[f][t][r] = du ? (kside ? du[(size_t)x * kD + y] : du[(size_t)y * kD + x]) : 0.f;
      }

  for (int c = nch - 1; c >= 0; --c) {
    const int set = (nch - 1 - c) & 1;
    const int64_t t0 = (int64_t)c * kC;
    Decay dc;
    dc.make(gnext, t0 + l < N);
    wait_vmem();
    lds_barrier();
    if (c > 0) {
      const int64_t tn = t0 - kC;
#pragma unroll
      for (int t = 0; t < 4; ++t) dma.issue(tile(smem, set ^ 1, t), src[t] + tn * kD, kC);
      gnext = G[tn + l];
    }
    const char* tq = tile(smem, set, tQ);
    const char* tk = tile(smem, set, tK);
    const char* tv = tile(smem, set, tV);
    const char* to = tile(smem, set, tO);
    if (c + 1 < nch && w == kNW - 1) flush_dots(smem, 4, xk, t0 + kC, N);

    // scores: A (rows j of V, columns i of dO; hi and lo) on the dk side,
    // B (rows j of K, columns i of Q; hi) on the dv side
    const int pw = w & 3;
    for (int p = pw; p < 10; p += 4) {
      if (kside) score_tile(p, tv, to, dc, smem + oAh, smem + oAl);
      else score_tile(p, tk, tq, dc, smem + oB, nullptr);
    }

    lds_barrier();

    // inter-chunk part, scaled by 2^(L - l_j) per key token j (the lane's column):
    //   dk[a][j] = sum_b U[a][b] v_j[b]   (split U)
    //   dv[b][j] = sum_a U[a][b] k_j[a]   (U hi)
    f32x4 acc[2][4];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int jt = 0; jt < 4; ++jt) acc[f][jt] = zero4();
    if (kside) {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 uh[2], ul[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) split_chain(U[f][2 * s], U[f][2 * s + 1], uh[f], ul[f]);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const bf16x8 bv = tl_chain<CPR>(tv, 16 * jt + c16, s);
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            acc[f][jt] = mma(uh[f], bv, acc[f][jt]);
            acc[f][jt] = mma(ul[f], bv, acc[f][jt]);
          }
        }
      }
    } else {
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        bf16x8 uh[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) uh[f] = Mma<bf16>::chain2(U[f][2 * s], U[f][2 * s + 1]);
#pragma unroll
        for (int jt = 0; jt < 4; ++jt) {
          const bf16x8 bk = tl_chain<CPR>(tk, 16 * jt + c16, s);
#pragma unroll
          for (int f = 0; f < 2; ++f) acc[f][jt] = mma(uh[f], bk, acc[f][jt]);
        }
      }
    }
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const float fj = fast_exp2(dc.L - dc.at(16 * jt + c16));
#pragma unroll
      for (int f = 0; f < 2; ++f)
#pragma unroll
        for (int r = 0; r < 4; ++r) acc[f][jt][r] *= fj;
    }
    // Q^T (dk side) or dO^T (dv side) fragments: rows f0 + 16 f + lane, k = tokens i
    bf16x8 xf[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) xf[f][ks] = tl_kmaj<CPR>(kside ? tq : to, ks, f0 + 16 * f);

    // intra-chunk part: dk[a][j] += sum_{i>=j} q_i[a] A_ij ; dv[b][j] += sum_{i>=j} do_i[b] B_ij
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
#pragma unroll
      for (int ks = jt / 2; ks < 2; ++ks) {
        if (kside) {
          const bf16x8 ah = tl_kmaj<SPR>(smem + oAh, ks, 16 * jt);
          const bf16x8 al = tl_kmaj<SPR>(smem + oAl, ks, 16 * jt);
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            acc[f][jt] = mma(xf[f][ks], ah, acc[f][jt]);
            acc[f][jt] = mma(xf[f][ks], al, acc[f][jt]);
          }
        } else {
          const bf16x8 bs = tl_kmaj<SPR>(smem + oB, ks, 16 * jt);
#pragma unroll
          for (int f = 0; f < 2; ++f) acc[f][jt] = mma(xf[f][ks], bs, acc[f][jt]);
        }
      }
    }
    // stores (four features of token j per lane); k . dk partials on the dk side
#pragma unroll
    for (int jt = 0; jt < 4; ++jt) {
      const int j = 16 * jt + c16;
      float p = 0.f;
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        store4(acc[f][jt], ors, t0 + j, f0 + 16 * f + 4 * g);
        if (kside) {
          const bf16x4 k4 = *reinterpret_cast<const bf16x4*>(tk + tile_off<CPR, 2>(j, f0 + 16 * f + 4 * g));
#pragma unroll
          for (int r = 0; r < 4; ++r) p += (float)k4[r] * acc[f][jt][r];
        }
      }
      if (kside) {
        p = group_sum(p);
        if (g == 0) sX[w * kC + j] = p;
      }
    }

    // update of U with the chunk: U = 2^L U + sum_i 2^(l_i) q_i do_i^T
    const float fL = fast_exp2(dc.L);
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) U[f][t][r] *= fL;
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      float di[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) di[e] = fast_exp2(dc.at(chain_k<bf16>(ks, e)));
      if (kside) {
        // U^T[b][a] += sum_i do_i[b] (2^(l_i) q_i[a]): split decayed Q as the B operand
        bf16x8 qh[2], ql[2];
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          float x[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) x[e] = (float)xf[f][ks][e] * di[e];
          split8(x, qh[f], ql[f]);
        }
#pragma unroll
        for (int bt = 0; bt < 8; ++bt) {
          const bf16x8 oa = tl_kmaj<CPR>(to, ks, 16 * bt);
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            U[f][bt] = mma(oa, qh[f], U[f][bt]);
            U[f][bt] = mma(oa, ql[f], U[f][bt]);
          }
        }
      } else {
        // U[a][b] += sum_i (2^(l_i) q_i[a]) do_i[b]: decayed Q^T (hi) as the A operand
#pragma unroll
        for (int at = 0; at < 8; ++at) {
          const bf16x8 qa = tl_kmaj<CPR>(tq, ks, 16 * at);
          bf16x8 qd;
#pragma unroll
          for (int e = 0; e < 8; ++e) qd[e] = (bf16)((float)qa[e] * di[e]);
#pragma unroll
          for (int f = 0; f < 2; ++f) U[f][at] = mma(qd, xf[f][ks], U[f][at]);
        }
      }
    }
  }
  // the gradient of the state before the first token is U after chunk 0 (the
  // dk waves hold it to float32 accuracy, as U^T: row b, column a)
  if (a.dstate_in && kside) {
    float* ds = a.dstate_in + (size_t)bh * kD * kD;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int t = 0; t < 8; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) ds[(size_t)(f0 + 16 * f + c16) * kD + 16 * t + 4 * g + r] = U[f][t][r];
  }
  lds_barrier();
  if (nch > 0 && w == kNW - 1) flush_dots(smem, 4, xk, 0, N);
}

__global__ __launch_bounds__(kNT, 1) void bwd_kernel(Args a) {
  __shared__ __attribute__((aligned(16))) char smem[kLds];
  const int b = blockIdx.x;
  if (b < a.BH) dq_sweep(a, smem, b);
  else dkv_sweep(a, smem, b - a.BH);
}

// dg_t = (1 / g_t) sum_{m >= t} (xq_m - xk_m) in slices of kGateSlice tokens:
// gate_tot sums each slice, gate_apply adds the totals of the later slices and
// walks its slice's tiles of 256 tokens from the last one back (thread = token:
// a suffix sum inside each wave by lane shifts, the later waves' totals from
// LDS). Every sum runs in a fixed order. dg may alias xq: gate_tot has read
// all of xq before gate_apply runs, and there each token's xq is read before
// its dg is written, by the same thread.
__global__ __launch_bounds__(256) void gate_tot(const float* xq, const float* __restrict__ xk, float* __restrict__ tot,
                                                int64_t N, int S) {
  __shared__ float red[4];
  const int sl = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, w = tid >> 6;
  const size_t base = (size_t)bh * N;
  float x = 0.f;
#pragma unroll
  for (int j = 0; j < kGateSlice / 256; ++j) {
    const int64_t t = (int64_t)sl * kGateSlice + j * 256 + tid;
    if (t < N) x += xq[base + t] - xk[base + t];
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) x += __shfl_xor(x, off);
  if (lane_id() == 0) red[w] = x;
  __syncthreads();
  if (tid == 0) tot[(size_t)bh * S + sl] = (red[0] + red[1]) + (red[2] + red[3]);
}

__global__ __launch_bounds__(256) void gate_apply(const float* __restrict__ g, const float* xq,
                                                  const float* __restrict__ xk, const float* __restrict__ tot,
                                                  float* dg, int64_t N, int S) {
  __shared__ float wtot[4];
  const int sl = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x, l = lane_id(), w = tid >> 6;
  const size_t base = (size_t)bh * N;
  float carry = 0.f;
  for (int s2 = S - 1; s2 > sl; --s2) carry += tot[(size_t)bh * S + s2];
  for (int j = kGateSlice / 256 - 1; j >= 0; --j) {
    const int64_t t = (int64_t)sl * kGateSlice + j * 256 + tid;
    const bool ok = t < N;
    float s = ok ? xq[base + t] - xk[base + t] : 0.f;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_down(s, off);  // every lane takes part; the sum masks
      if (l + off < 64) s += o;
    }
    if (l == 0) wtot[w] = s;  // lane 0 holds its wave's total
    __syncthreads();
    float after = carry;
    for (int u = w + 1; u < 4; ++u) after += wtot[u];
    const float tile = (wtot[0] + wtot[1]) + (wtot[2] + wtot[3]);
    if (ok) dg[base + t] = (s + after) / g[base + t];
    carry += tile;
    __syncthreads();  // wtot is rewritten by the next tile
  }
}

}  // namespace lbw

hipError_t linattn_backward_bf16_launch(const BwdBf16Launch& L, hipStream_t st) {
  lbw::Args a;
  a.q = static_cast<const bf16*>(L.q);
  a.k = static_cast<const bf16*>(L.k);
  a.v = static_cast<const bf16*>(L.v);
  a.dout = static_cast<const bf16*>(L.dout);
  a.g = L.g;
  a.dq = static_cast<bf16*>(L.dq);
  a.dk = static_cast<bf16*>(L.dk);
  a.dv = static_cast<bf16*>(L.dv);
  a.xq = L.dg;  // q . dq lands in dg, which the suffix pass then overwrites
  a.xk = L.xk;
  a.state_in = L.state_in;
  a.dstate_out = L.dstate_out;
  a.dstate_in = L.dstate_in;
  a.N = L.N;
  a.BH = (int)(L.B * L.H);
  hipLaunchKernelGGL(lbw::bwd_kernel, dim3((unsigned)(2 * a.BH)), dim3(lbw::kNT), 0, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int S = (int)gate_slices(L.N);
  hipLaunchKernelGGL(lbw::gate_tot, dim3((unsigned)S, (unsigned)a.BH), dim3(256), 0, st, L.dg, L.xk, L.tot, L.N, S);
  hipLaunchKernelGGL(lbw::gate_apply, dim3((unsigned)S, (unsigned)a.BH), dim3(256), 0, st, L.g, L.dg, L.xk, L.tot, L.dg,
                     L.N, S);
  return hipGetLastError();
}

}  // namespace lm
