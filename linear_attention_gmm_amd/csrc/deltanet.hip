// deltanet.hip -- chunkwise gated delta rule with the plain or the CCQ read,
// forward, for gfx950.
//
// Method
//  * Write rule (allinfo.ai.kr post on linear attention, "Key messages" and
//    "Easy explanation"): the state update is one gradient-descent step on
//    the squared error of predicting v_t from k_t, the delta rule erases the
//    value bound to the current key and writes the new one, and a decay gate
//    forgets. With S (dk x dv), decay g_t in (0, 1] and step size beta_t:
//        S_t = g_t S_{t-1} - beta_t k_t (g_t S_{t-1}^T k_t - v_t)^T,
//    read o_t = S_t^T q_t.
//  * CCQ read ("Don't Read Everything: A Curvature-Conditioned Query for
//    Linear Attention", section 2 Method, integration): the read uses
//    q_clean = q_t - lambda_t Sigma_t q_t, which depends on the queries and
//    keys only, whatever the write rule. The clean-query passes below form it
//    (running key sums M = sum k k^T, m = sum k, count t), and the chunk pass
//    then reads with it.
//
// Chunk algebra (our own derivation; the pages give no chunk form for this
// rule). Write the step as S_r = g_r S_{r-1} + k_r u_r^T with the pseudo-value
// u_r = beta_r (v_r - g_r S_{r-1}^T k_r). Inside a chunk with start state S_0
// and gamma_r = prod_{s<=r} g_s:
//   (I + A) U = diag(beta) V - diag(beta gamma) K S_0,
//   A_rj = beta_r (gamma_r / gamma_j) (k_r . k_j)  for j < r (strictly lower).
// With T = (I + A)^{-1}, W = T diag(beta gamma) K and Ut = T diag(beta) V
// (neither depends on S_0):
//   U   = Ut - W S_0
//   O   = diag(gamma) Q S_0 + (mask_{j<=r}(gamma_r / gamma_j) o Q K^T) U
//   S_C = gamma_C S_0 + K^T diag(gamma_C / gamma_j) U.
// T is formed in fp32: the four 16 x 16 diagonal blocks by forward
// substitution, then T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj for i - j = 1, 2, 3.
// Decay ratios are powers of two of differences of the running log2-decay
// with a non-positive exponent; gamma itself may underflow to 0, which only
// drops terms of that (negligible) size.
//
// MI355X design
//  * Two passes. The prepass forms T, W and Ut for every chunk at once (no
//    chunk depends on another there) and writes W and Ut, rounded to the input
//    type, in the layouts of K and V. The sequential pass then keeps only
//    the state chain S_0 -> U -> S_C per chunk (two barriers), with the
//    decayed Q K^T and the output hanging off it.
//  * The rule acts on S from the key side only, so the value columns of S
//    evolve independently: in the sequential pass a workgroup of 8 waves
//    owns 32 value columns of one (b, h) and walks every chunk in order.
//    That is B*H*dv/32 workgroups (256 at B=4, H=16, dv=128)
//    with no segment pass (a segment pass for this rule would carry a dense
//    dk x dk transition). The column groups of one (b, h) are launched
//    gridDim/groups apart, which for B*H a multiple of 8 puts them on one
//    XCD, sharing its L2 for Q, K and W.
//  * Products are 16x16 MFMA tiles (bf16 operands, fp32 accumulation; or
//    fp32), T in fp32 MFMA. S stays in fp32 registers and is rounded to the
//    operand type once per chunk for the products that read it.
//  * Each pass loads the next chunk's rows into registers while the current
//    chunk is computed (the sequential pass during its last phase only, which
//    keeps its registers within 256 per lane without spills).
#include "mfma.hpp"
#include "launch.hpp"

namespace lm {
namespace gdn {

constexpr int kC = 64;
constexpr int kNW = 8;
constexpr int kNT = kNW * 64;
constexpr int kCG = 32;  // value columns per workgroup
constexpr float kMinLog2 = -126.f;  // decays below 2^-126 act as 2^-126

// Tiles of the lower triangle of a 4 x 4 tile grid, row by row.
__device__ __forceinline__ void tri_tile(int u, int& it, int& jt) {
  it = u >= 6 ? 3 : u >= 3 ? 2 : u >= 1 ? 1 : 0;
  jt = u - it * (it + 1) / 2;
}

// k-steps over tokens 0 .. 16 r + 15 (row tile r of a lower-triangular operand).
template <typename T>
__device__ __forceinline__ constexpr int tok_steps(int r) {
  return sizeof(T) == 2 ? r / 2 + 1 : 4 * (r + 1);
}

template <typename T>
__device__ __forceinline__ T cvt(float x) {
  return (T)x;
}

// A operand, CHAIN order, of a fp32 row-major matrix (row `row`, k-step ks)
// scaled per k by sc[k], converted to T.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag scaled_row(const float* m, int pitch, int row, int ks,
                                                            const float* sc) {
  const int g = lane_id() >> 4;
  if constexpr (sizeof(T) == 2) {
    const int k0 = ks * 32 + 4 * g;
    const f32x4 a0 = *reinterpret_cast<const f32x4*>(m + row * pitch + k0);
    const f32x4 a1 = *reinterpret_cast<const f32x4*>(m + row * pitch + k0 + 16);
    const f32x4 s0 = *reinterpret_cast<const f32x4*>(sc + k0);
    const f32x4 s1 = *reinterpret_cast<const f32x4*>(sc + k0 + 16);
    bf16x8 f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (bf16)(a0[i] * s0[i]);
      f[4 + i] = (bf16)(a1[i] * s1[i]);
    }
    return f;
  } else {
    const int k = 16 * (ks >> 2) + 4 * g + (ks & 3);
    return m[row * pitch + k] * sc[k];
  }
}

// A operand of the lower-triangular ones matrix (row i of a 64-row chunk, token
// k-step ks): 1 where token <= i.
template <typename T>
__device__ __forceinline__ typename Mma<T>::frag tri_ones(int ks, int i) {
  typename Mma<T>::frag f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = chain_k<T>(ks, e) <= i ? (bf16)1.f : (bf16)0.f;
  } else {
    f = chain_k<T>(ks, 0) <= i ? 1.f : 0.f;
  }
  return f;
}

template <typename T>
__device__ __forceinline__ typename Mma<T>::frag ones_frag() {
  typename Mma<T>::frag f;
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int e = 0; e < 8; ++e) f[e] = (bf16)1.f;
  } else {
    f = 1.f;
  }
  return f;
}

// Layout of an LDS tile: rows of P elements (padded), or, with CP > 0, bf16
// rows of CP 16-byte pieces without padding and the piece index XORed by a
// function of the row. gfx950 serves 16-byte LDS reads in passes of 16 lanes
// ({0-3, 12-15, 20-27}, {4-11, 16-19, 28-31}, and the same above lane 32)
// over 64 banks of 4 bytes, 8-byte reads (plain or transposed) in passes of
// 32 lanes, and writes over 128 bytes. With CP = 16 the XOR
// ((r % 8) << 1) ^ 9 (r / 8 % 2) makes the operand gathers of 16 rows and the
// transposed reads of rows 8g .. 8g + 3 (and + 4) conflict-free; with CP = 8,
// (r / 2) % 8 does the same for the gathers. 8-byte stores of 16 rows take two
// cycles, the least for 16 lanes writing the same half of their pieces.
template <int P, int CP>
struct Lay {
  __device__ static __forceinline__ int x(int r) {
    if constexpr (CP == 16) return ((r & 7) << 1) ^ (((r >> 3) & 1) * 9);
    else return (r >> 1) & 7;
  }
  // element offset of (row r, column col)
  __device__ static __forceinline__ int off(int r, int col) {
    if constexpr (CP > 0) return r * CP * 8 + ((((col >> 3) ^ x(r)) << 3) | (col & 7));
    else return r * P + col;
  }
};
// NATURAL operand fragment of tile row rc, k-step ks.
template <typename L, typename T>
__device__ __forceinline__ typename Mma<T>::frag nat(const T* base, int rc, int ks) {
  const int g = lane_id() >> 4;
  if constexpr (sizeof(T) == 2) return *reinterpret_cast<const bf16x8*>(base + L::off(rc, ks * 32 + 8 * g));
  else return base[L::off(rc, ks * 4 + g)];
}
// Four rows (r .. r + 3) of one column of an accumulator tile, stored as four
// consecutive elements (columns c .. c + 3, c a multiple of 4) of row r' of a
// transposed tile.
template <typename L, typename T>
__device__ __forceinline__ void put4(T* base, int r, int c, const f32x4& v);

// 16-byte vectors of 64 rows of a [BH][N][width] tensor: loads into registers
// (rows past `limit` read as zero) and stores into an LDS tile of pitch `pitch`.
template <typename T, int W, int COLS>
struct RowVecs {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int VR = COLS * ES / 16;          // vectors per row
  static constexpr int NV = (kC * VR + kNT - 1) / kNT;  // per thread
  uint4 x[NV];
  // src: element (0, col0) of the (b, h) slice; width W elements per row
  __device__ __forceinline__ void load(const T* src, int64_t c0, int64_t limit) {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int p = threadIdx.x + i * kNT;
      const int row = p / VR, cv = p % VR;
      const bool ok = p < kC * VR && c0 + row < limit;
      x[i] = ok ? *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(src + (size_t)(c0 + row) * W) +
                                                  cv * 16)
                : make_uint4(0, 0, 0, 0);
    }
  }
  __device__ __forceinline__ void store(T* dst, int pitch) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int p = threadIdx.x + i * kNT;
      if (p < kC * VR) {
        const int row = p / VR, cv = p % VR;
        *reinterpret_cast<uint4*>(reinterpret_cast<char*>(dst + row * pitch) + cv * 16) = x[i];
      }
    }
  }
  // the same into a tile of layout L
  template <typename L>
  __device__ __forceinline__ void store_l(T* dst) const {
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      const int p = threadIdx.x + i * kNT;
      if (p < kC * VR) {
        const int row = p / VR, cv = p % VR;
        *reinterpret_cast<uint4*>(dst + L::off(row, cv * (16 / ES))) = x[i];
      }
    }
  }
};

// Per-token decay scalars of a chunk (wave 0, lane = token; g = 1 past the end):
// l = running log2-decay, written with what the caller needs of it.
__device__ __forceinline__ float chunk_log2_decay(float g) {
  return wave_scan_incl(fmaxf(__builtin_amdgcn_logf(g), kMinLog2));
}

// Four rows (r0 .. r0 + 3) of one column of an accumulator tile, stored as
// four consecutive elements of a transposed LDS tile.
template <typename T>
__device__ __forceinline__ void put_col4(T* p, const f32x4& v) {
  if constexpr (sizeof(T) == 2) {
    *reinterpret_cast<bf16x4*>(p) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
  } else {
    *reinterpret_cast<f32x4*>(p) = v;
  }
}
template <typename L, typename T>
__device__ __forceinline__ void put4(T* base, int r, int c, const f32x4& v) {
  put_col4(base + L::off(r, c), v);
}

// ---------------------------------------------------------------------------
// Prepass: for every chunk, T = (I + A)^{-1}, W = T diag(beta gamma) K and
// Ut = T diag(beta) V, written to the workspace in the layouts of K and V.
// Nothing here depends on the state, so every chunk is independent.

template <typename T, int D>
struct PCfg {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int KS = Mma<T>::KS;
  static constexpr int NKD = D / KS;
  static constexpr int PAD = ES == 2 ? 8 : 4;
  static constexpr int PQ = D + PAD;  // K, V, and the W / Ut staging rows
  static constexpr int PA = kC + 4;   // A, T rows (fp32)
  // The W and Ut staging tiles reuse the A and T tiles once T is formed.
  static constexpr int o_k = 0;
  static constexpr int o_v = o_k + kC * PQ * ES;
  static constexpr int o_a = o_v + kC * PQ * ES;
  static constexpr int o_t = o_a + kC * PA * 4;
  static constexpr int o_row = o_t + kC * PA * 4;  // [3][64] f32: l, beta, beta gamma
  static constexpr int o_w = o_a;
  static constexpr int o_u = o_t;
  static constexpr int bytes = o_row + 3 * kC * 4;
  static_assert(PQ * ES <= PA * 4, "staging rows fit the A and T rows");
  static_assert(bytes <= 80 * 1024, "two workgroups per CU");
  static_assert(o_v % 16 == 0 && o_a % 16 == 0 && o_t % 16 == 0 && o_row % 16 == 0, "16-byte aligned regions");
  static constexpr int FPW = D / 32;  // W (and Ut) column tiles per wave
};

struct PArgs {
  const void* k;
  const void* v;
  const float* g;
  const float* beta;
  void* w;   // [BH][N][D]
  void* ut;  // [BH][N][dv]
  int64_t N;
  int cpb;   // chunks per workgroup
};

template <typename T, int D>
__global__ __launch_bounds__(kNT, sizeof(T) == 2 ? 4 : 2) void gdn_prep_kernel(PArgs a) {
  typedef PCfg<T, D> C;
  typedef Mma<T> M;
  __shared__ __attribute__((aligned(16))) char sm[C::bytes];
  T* sK = reinterpret_cast<T*>(sm + C::o_k);
  T* sV = reinterpret_cast<T*>(sm + C::o_v);
  T* sW = reinterpret_cast<T*>(sm + C::o_w);
  T* sU = reinterpret_cast<T*>(sm + C::o_u);
  float* sA = reinterpret_cast<float*>(sm + C::o_a);
  float* sT = reinterpret_cast<float*>(sm + C::o_t);
  float* sL = reinterpret_cast<float*>(sm + C::o_row);
  float* sBt = sL + kC;
  float* sSw = sL + 2 * kC;
  const int bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), g = l >> 4, l16 = l & 15, tid = threadIdx.x;
  const int64_t nch = (a.N + kC - 1) / kC;
  const int64_t ch0 = (int64_t)blockIdx.x * a.cpb;
  const int64_t ch1 = ch0 + a.cpb < nch ? ch0 + a.cpb : nch;
  const T* kb = static_cast<const T*>(a.k) + (size_t)bh * a.N * D;
  const T* vb = static_cast<const T*>(a.v) + (size_t)bh * a.N * D;
  T* wb = static_cast<T*>(a.w) + (size_t)bh * a.N * D;
  T* ub = static_cast<T*>(a.ut) + (size_t)bh * a.N * D;
  const float* gb = a.g + (size_t)bh * a.N;
  const float* bb = a.beta + (size_t)bh * a.N;

  RowVecs<T, D, D> pk, pv;
  float pg = 1.f, pb = 0.f;
  auto fetch = [&](int64_t c0) {
    pk.load(kb, c0, a.N);
    pv.load(vb, c0, a.N);
    const bool ok = tid < kC && c0 + tid < a.N;
    pg = ok ? gb[c0 + tid] : 1.f;
    pb = ok ? bb[c0 + tid] : 0.f;
  };
  if (ch0 < ch1) fetch(ch0 * kC);

  for (int64_t ch = ch0; ch < ch1; ++ch) {
    const int64_t c0 = ch * kC;
    pk.store(sK, C::PQ);
    pv.store(sV, C::PQ);
    if (w == 0) {
      const float lr = chunk_log2_decay(pg);
      sL[l] = lr;
      sBt[l] = pb;
      sSw[l] = pb * fast_exp2(lr);
    }
    lds_barrier();

    // A = strictly lower, beta-scaled, decayed K K^T (fp32), formed as A^T
    // tiles so that a lane's four entries are consecutive in a row of A
    for (int t = w; t < 10; t += kNW) {
      int it, jt;
      tri_tile(t, it, jt);
      f32x4 acc = zero4();  // element (key j = 16 jt + 4 g + e, row i = 16 it + l16)
#pragma unroll
      for (int ks = 0; ks < C::NKD; ++ks)
        acc = M::mma(ld_kc_nat(sK, C::PQ, 16 * jt + l16, ks), ld_kc_nat(sK, C::PQ, 16 * it + l16, ks), acc);
      const int i = 16 * it + l16;
      const float li = sL[i], bi = sBt[i];
      const f32x4 lj = *reinterpret_cast<const f32x4*>(sL + 16 * jt + 4 * g);
      f32x4 av;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * jt + 4 * g + e;
        av[e] = j < i ? bi * fast_exp2(fminf(li - lj[e], 0.f)) * acc[e] : 0.f;
      }
      *reinterpret_cast<f32x4*>(sA + i * C::PA + 16 * jt + 4 * g) = av;
    }
    lds_barrier();

    // T: diagonal blocks by forward substitution (wave 0: lane group = block,
    // lane = column), two partial sums to halve the dependent chain. The other
    // waves clear tiles (0, 1) and (2, 3), which the k-steps that straddle the
    // diagonal read (the Ut staging of the previous chunk overwrote them).
    if (w > 0) {
      for (int i = tid - 64; i < 2 * 256; i += kNT - 64) {
        const int t = i >> 8, e = i & 255;
        sT[(32 * t + (e >> 4)) * C::PA + 32 * t + 16 + (e & 15)] = 0.f;
      }
    }
    if (w == 0) {
      const int b0 = 16 * g, c = l16;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float s0 = r == c ? 1.f : 0.f, s1 = 0.f;
        const float* arow = sA + (b0 + r) * C::PA + b0;
#pragma unroll
        for (int i = 0; i < r; ++i) {
          if (i & 1)
            s1 -= arow[i] * x[i];
          else
            s0 -= arow[i] * x[i];
        }
        x[r] = s0 + s1;
        __builtin_amdgcn_sched_barrier(0);  // one row's loads at a time (registers)
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sT[(b0 + r) * C::PA + b0 + c] = x[r];
    }
    lds_barrier();
    // T: off-diagonal blocks, T_ij = -T_ii sum_{m=j}^{i-1} A_im T_mj
#pragma unroll
    for (int d = 1; d < 4; ++d) {
      if (w < 4 - d) {
        const int bi = w + d, bj = w;
        f32x4 X = zero4();
        for (int m = bj; m < bi; ++m) {
#pragma unroll
          for (int ks = 0; ks < 4; ++ks)
            X = Mma<float>::mma(ld_kc_chain(sA + 16 * m, C::PA, 16 * bi + l16, ks),
                                ld_km_chain(sT + 16 * m * C::PA, C::PA, 16 * bj, ks), X);
        }
        f32x4 Y = zero4();
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
          Y = Mma<float>::mma(ld_kc_chain(sT + 16 * bi, C::PA, 16 * bi + l16, ks), X[ks], Y);
#pragma unroll
        for (int e = 0; e < 4; ++e) sT[(16 * bi + 4 * g + e) * C::PA + 16 * bj + l16] = -Y[e];
      }
      lds_barrier();
    }

    // W = T diag(beta gamma) K and Ut = T diag(beta) V: wave w takes row tile
    // w / 2 and half of the column tiles of each
    {
      const int r = w >> 1, h = w & 1;
      constexpr int NKT = tok_steps<T>(3);
      typename M::frag aw[NKT], au[NKT];
      const int nk = tok_steps<T>(r);
#pragma unroll
      for (int ks = 0; ks < NKT; ++ks)
        if (ks < nk) {
          aw[ks] = scaled_row<T>(sT, C::PA, 16 * r + l16, ks, sSw);
          au[ks] = scaled_row<T>(sT, C::PA, 16 * r + l16, ks, sBt);
        }
      lds_barrier();  // every wave holds its rows of T: the staging may overwrite A and T
      // as W^T and Ut^T tiles (rows = features of column tile f, columns =
      // tokens of row tile r), so that a lane's four entries are consecutive
      // in a row of W (Ut)
#pragma unroll 1
      for (int fi = 0; fi < C::FPW; ++fi) {
        const int f = h * C::FPW + fi;
        f32x4 cw = zero4(), cu = zero4();
#pragma unroll
        for (int ks = 0; ks < NKT; ++ks)
          if (ks < nk) {
            cw = M::mma(ld_km_chain(sK, C::PQ, 16 * f, ks), aw[ks], cw);
            cu = M::mma(ld_km_chain(sV, C::PQ, 16 * f, ks), au[ks], cu);
          }
        const int off = (16 * r + l16) * C::PQ + 16 * f + 4 * g;
        put_col4(sW + off, cw);
        put_col4(sU + off, cu);
      }
    }
    lds_barrier();
    // the next chunk's rows load while this one's are written out (issued this
    // late so that they hold no registers during T and W; the other workgroup
    // on the CU covers their latency)
    if (ch + 1 < ch1) fetch(c0 + kC);
    // rows to the workspace, 16 bytes per lane
    {
      constexpr int VR = D * (int)sizeof(T) / 16;
      for (int p = tid; p < kC * VR; p += kNT) {
        const int row = p / VR, cv = p % VR;
        if (c0 + row < a.N) {
          const size_t off = (size_t)(c0 + row) * D * sizeof(T) + (size_t)cv * 16;
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(wb) + off) =
              *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(sW + row * C::PQ) + cv * 16);
          *reinterpret_cast<uint4*>(reinterpret_cast<char*>(ub) + off) =
              *reinterpret_cast<const uint4*>(reinterpret_cast<const char*>(sU + row * C::PQ) + cv * 16);
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Sequential pass: per chunk, U = Ut - W S_0, O = diag(gamma) Q S_0 + P U with
// P the decayed lower Q K^T, S_C = gamma_C S_0 + K^T diag(gamma_C / gamma) U.
// The state chain per chunk is S_0 -> U -> S_C (two barriers); P and O hang
// off it. The operand copies of S and U sit in LDS transposed ([column][k]):
// an accumulator tile's four rows of one column are then one 8-byte store,
// and every product reads both operands as k-contiguous 16-byte fragments.

template <typename T, int D>
struct MCfg {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int KS = Mma<T>::KS;
  static constexpr int NKD = D / KS;
  static constexpr int NKC = kC / KS;
  static constexpr int PAD = ES == 2 ? 8 : 4;
  static constexpr bool SWZ = ES == 2 && D == 128;  // swizzled unpadded tiles
  static constexpr int PQ = SWZ ? D : D + PAD;      // Q, K, W rows (token-major)
  static constexpr int PV = kCG + PAD;              // Ut rows (token-major)
  static constexpr int PS = SWZ ? D : D + PAD;      // S^T rows (column-major S: [column][feature])
  static constexpr int PU = SWZ ? kC : kC + PAD;    // U^T rows ([column][token]), P rows
  typedef Lay<PQ, SWZ ? 16 : 0> LQ;                 // Q, K, W, S^T
  typedef Lay<PU, SWZ ? 8 : 0> LU;                  // U^T, P
  static constexpr int o_q = 0;
  static constexpr int o_k = o_q + kC * PQ * ES;
  static constexpr int o_w = o_k + kC * PQ * ES;
  static constexpr int o_ut = o_w + kC * PQ * ES;
  static constexpr int o_s = o_ut + kC * PV * ES;
  static constexpr int o_u = o_s + kCG * PS * ES;
  static constexpr int o_ud = o_u + kCG * PU * ES;
  static constexpr int o_p = o_ud + kCG * PU * ES;
  static constexpr int o_row = o_p + kC * PU * ES;  // [3][64] f32: l, gamma_C / gamma, gamma
  static constexpr int bytes = o_row + 3 * kC * 4;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static_assert(o_k % 16 == 0 && o_w % 16 == 0 && o_ut % 16 == 0 && o_s % 16 == 0 && o_u % 16 == 0 &&
                    o_ud % 16 == 0 && o_p % 16 == 0 && o_row % 16 == 0 && (PQ * ES) % 16 == 0 &&
                    (PS * ES) % 16 == 0 && (PU * ES) % 16 == 0,
                "16-byte aligned regions and rows");
  static constexpr int NST = 2 * D / 16;  // S tiles of the column group
  static constexpr int SPW = (NST + kNW - 1) / kNW;
};

struct Args {
  const void* q;
  const void* k;
  const void* w;   // prepass output [BH][N][D]
  const void* ut;  // prepass output [BH][N][dv]
  const float* g;
  void* out;
  const float* state_in;  // optional: S at state_in + bh * sstride
  float* state_out;
  int64_t sstride;
  const float* mfinal;  // CCQ with state_out: running sums after the last token,
                        // block P - 1 of the clean-query pass's workspace
  int P, sfl;
  int64_t N;
  int BH;
  int dv;
};

// NATURAL operand fragment with k along the rows of a token-major tile and the
// operand's row/column = tile column c0 + lane % 16 (bf16: two transpose reads).
template <typename L, typename T>
__device__ __forceinline__ typename Mma<T>::frag km_nat(const T* base, int c0, int ks) {
  const int g = lane_id() >> 4, j = lane_id() & 15;
  if constexpr (sizeof(T) == 2) {
    // lane j of a 16-lane group supplies row k0 + j / 4, columns c0 + 4 (j % 4) ..
    auto rd = [&](int k0) {
      return __builtin_bit_cast(bf16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                            (i16x4 LM_LDS*)(base + L::off(k0 + (j >> 2), c0 + 4 * (j & 3)))));
    };
    const bf16x4 lo = rd(ks * 32 + 8 * g);
    const bf16x4 hi = rd(ks * 32 + 8 * g + 4);
    return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  } else {
    return base[L::off(ks * 4 + g, c0 + j)];
  }
}

// An accumulator-layout tile (rows r0 + 4 g .. + 3, column c0 + lane % 16) of a
// token-major LDS tile.
template <typename T>
__device__ __forceinline__ f32x4 acc_tile(const T* base, int pitch, int r0, int c0) {
  const int g = lane_id() >> 4, c = lane_id() & 15;
  if constexpr (sizeof(T) == 2) {
    const bf16x4 x = tr16(base, pitch, c0, r0 + 4 * g);
    return f32x4{(float)x[0], (float)x[1], (float)x[2], (float)x[3]};
  } else {
    return f32x4{base[(r0 + 4 * g) * pitch + c0 + c], base[(r0 + 4 * g + 1) * pitch + c0 + c],
                 base[(r0 + 4 * g + 2) * pitch + c0 + c], base[(r0 + 4 * g + 3) * pitch + c0 + c]};
  }
}

template <typename T, int D>
__global__ __launch_bounds__(kNT, 2) void gdn_kernel(Args a) {
  typedef MCfg<T, D> C;
  typedef Mma<T> M;
  __shared__ __attribute__((aligned(16))) char sm[C::bytes];
  T* sQ = reinterpret_cast<T*>(sm + C::o_q);
  T* sK = reinterpret_cast<T*>(sm + C::o_k);
  T* sW = reinterpret_cast<T*>(sm + C::o_w);
  T* sUt = reinterpret_cast<T*>(sm + C::o_ut);
  T* sS = reinterpret_cast<T*>(sm + C::o_s);    // S^T: [column][feature]
  T* sU = reinterpret_cast<T*>(sm + C::o_u);    // U^T: [column][token]
  T* sUd = reinterpret_cast<T*>(sm + C::o_ud);  // (diag(gamma_C / gamma) U)^T
  T* sP = reinterpret_cast<T*>(sm + C::o_p);    // P: [query][key]
  float* sL = reinterpret_cast<float*>(sm + C::o_row);  // running log2 decay
  float* sDc = sL + kC;                                  // gamma_C / gamma_j
  float* sGm = sL + 2 * kC;                              // gamma_j

  const int bh = blockIdx.x % a.BH, cg = blockIdx.x / a.BH;
  const int w = wave_id(), l = lane_id(), g = l >> 4, l16 = l & 15;
  const int tid = threadIdx.x;
  const T* qb = static_cast<const T*>(a.q) + (size_t)bh * a.N * D;
  const T* kb = static_cast<const T*>(a.k) + (size_t)bh * a.N * D;
  const T* wb = static_cast<const T*>(a.w) + (size_t)bh * a.N * D;
  const T* ub = static_cast<const T*>(a.ut) + (size_t)bh * a.N * a.dv + cg * kCG;
  const float* gb = a.g + (size_t)bh * a.N;

  // upper tiles of P stay zero (read by the k-steps that straddle the diagonal)
  for (int i = tid; i < kC * kC; i += kNT) {
    const int r = i / kC, c = i % kC;
    if ((c >> 4) > (r >> 4)) sP[C::LU::off(r, c)] = cvt<T>(0.f);
  }

  // this wave's S tiles: t = w + kNW j, tile (t / 2, t % 2)
  f32x4 St[C::SPW];
#pragma unroll
  for (int j = 0; j < C::SPW; ++j) {
    St[j] = zero4();
    const int t = w + kNW * j;
    if (t < C::NST && a.state_in) {
      const float* src = a.state_in + (size_t)bh * a.sstride;
      const int ra = 16 * (t >> 1), col = cg * kCG + 16 * (t & 1) + l16;
#pragma unroll
      for (int e = 0; e < 4; ++e) St[j][e] = src[(size_t)(ra + 4 * g + e) * a.dv + col];
    }
  }

  RowVecs<T, D, D> pq, pk, pw;
  RowVecs<T, D, kCG> pu;  // this group's columns of rows of width dv (== D)
  float pg = 1.f;
  auto fetch = [&](int64_t c0) {
    pq.load(qb, c0, a.N);
    pk.load(kb, c0, a.N);
    pw.load(wb, c0, a.N);
    pu.load(ub, c0, a.N);
    pg = tid < kC && c0 + tid < a.N ? gb[c0 + tid] : 1.f;
  };
  fetch(0);
  const int64_t nch = (a.N + kC - 1) / kC;
  const int r_own = w >> 1, c_own = w & 1;  // the (row tile, column tile) of U and O this wave owns
  T* outp = static_cast<T*>(a.out);

  for (int64_t ch = 0; ch < nch; ++ch) {
    const int64_t c0 = ch * kC;
    // ---- inputs to LDS, the state to its operand copy
    pq.template store_l<typename C::LQ>(sQ);
    pk.template store_l<typename C::LQ>(sK);
    pw.template store_l<typename C::LQ>(sW);
    pu.store(sUt, C::PV);
#pragma unroll
    for (int j = 0; j < C::SPW; ++j) {
      const int t = w + kNW * j;
      if (t < C::NST) put4<typename C::LQ>(sS, 16 * (t & 1) + l16, 16 * (t >> 1) + 4 * g, St[j]);
    }
    if (w == 0) {
      const float lr = chunk_log2_decay(pg);
      const float lc = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, lr), 63));
      sL[l] = lr;
      sDc[l] = fast_exp2(lc - lr);
      sGm[l] = fast_exp2(lr);
    }
    lds_barrier();

    // ---- U = Ut - W S_0 (this wave's tile), stored transposed, plainly and
    //      scaled by gamma_C / gamma_j; the P tiles (as P^T tiles, so that a
    //      lane's four entries are consecutive in a row of P)
    {
      f32x4 acc = zero4();
#pragma unroll
      for (int ks = 0; ks < C::NKD; ++ks)
        acc = M::mma(nat<typename C::LQ>(sW, 16 * r_own + l16, ks), nat<typename C::LQ>(sS, 16 * c_own + l16, ks), acc);
      const f32x4 ut = acc_tile(sUt, C::PV, 16 * r_own, 16 * c_own);
      const f32x4 dc = *reinterpret_cast<const f32x4*>(sDc + 16 * r_own + 4 * g);
      f32x4 u, ud;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        u[e] = ut[e] - acc[e];
        ud[e] = u[e] * dc[e];
      }
      put4<typename C::LU>(sU, 16 * c_own + l16, 16 * r_own + 4 * g, u);
      put4<typename C::LU>(sUd, 16 * c_own + l16, 16 * r_own + 4 * g, ud);
    }
    for (int t = w; t < 10; t += kNW) {
      int it, jt;
      tri_tile(t, it, jt);
      f32x4 acc = zero4();  // element (key j = 16 jt + 4 g + e, query i = 16 it + l16)
#pragma unroll
      for (int ks = 0; ks < C::NKD; ++ks)
        acc = M::mma(nat<typename C::LQ>(sK, 16 * jt + l16, ks), nat<typename C::LQ>(sQ, 16 * it + l16, ks), acc);
      const int i = 16 * it + l16;
      const float li = sL[i];
      const f32x4 lj = *reinterpret_cast<const f32x4*>(sL + 16 * jt + 4 * g);
      f32x4 p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int j = 16 * jt + 4 * g + e;
        p[e] = j <= i ? fast_exp2(fminf(li - lj[e], 0.f)) * acc[e] : 0.f;
      }
      put4<typename C::LU>(sP, i, 16 * jt + 4 * g, p);
    }
    lds_barrier();
    if (ch + 1 < nch) fetch(c0 + kC);  // held in registers through the last phase only

    // ---- S_C = gamma_C S_0 + K^T diag(gamma_C / gamma_j) U (this wave's tiles)
    {
      const float gc = sGm[kC - 1];
#pragma unroll
      for (int j = 0; j < C::SPW; ++j) {
        const int t = w + kNW * j;
        if (t < C::NST) {
          f32x4 acc = zero4();
#pragma unroll
          for (int ks = 0; ks < C::NKC; ++ks)
            acc = M::mma(km_nat<typename C::LQ>(sK, 16 * (t >> 1), ks), nat<typename C::LU>(sUd, 16 * (t & 1) + l16, ks),
                         acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) St[j][e] = gc * St[j][e] + acc[e];
        }
      }
    }
    // ---- O = diag(gamma) Q S_0 + P U (this wave's tile)
    {
      f32x4 acc = zero4(), acc2 = zero4();
#pragma unroll
      for (int ks = 0; ks < C::NKD; ++ks)
        acc = M::mma(nat<typename C::LQ>(sQ, 16 * r_own + l16, ks), nat<typename C::LQ>(sS, 16 * c_own + l16, ks), acc);
      const int nk = tok_steps<T>(r_own);
      for (int ks = 0; ks < nk; ++ks)
        acc2 = M::mma(nat<typename C::LU>(sP, 16 * r_own + l16, ks), nat<typename C::LU>(sU, 16 * c_own + l16, ks), acc2);
      const f32x4 gm = *reinterpret_cast<const f32x4*>(sGm + 16 * r_own + 4 * g);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int i = 16 * r_own + 4 * g + e;
        if (c0 + i < a.N)
          outp[((size_t)bh * a.N + c0 + i) * a.dv + cg * kCG + 16 * c_own + l16] = cvt<T>(acc[e] * gm[e] + acc2[e]);
      }
    }
    lds_barrier();
  }

  if (a.state_out) {
    float* dst = a.state_out + (size_t)bh * a.sstride;
    if (a.mfinal && cg == 0) {
      const float* src = a.mfinal + ((size_t)bh * a.P + a.P - 1) * a.sfl;
      for (int i = tid; i < D * D + D; i += kNT) dst[D * a.dv + i] = src[i];
    }
#pragma unroll
    for (int j = 0; j < C::SPW; ++j) {
      const int t = w + kNW * j;
      if (t < C::NST) {
        const int ra = 16 * (t >> 1), col = cg * kCG + 16 * (t & 1) + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(size_t)(ra + 4 * g + e) * a.dv + col] = St[j][e];
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Clean query of the CCQ read: q' = q - lambda_t Sigma_t q_t in the chunk form
//   delta_i = -alpha_i (M_prev q_i + sum_{j<=i} P_ij k_j)
//             + beta_i (m_prev + sum_{j<=i} k_j),
//   alpha_i = lambda_i / t,  beta_i = lambda_i (m_prev . q_i + sum_{j<=i} P_ij) / t^2,
// P_ij = q_i . k_j rounded once to the operand type (row sums from the rounded
// values, so that the t = 1 case cancels). M_prev, m_prev are the running sums
// of k k^T and k before the chunk; t counts tokens from the sequence start.
// A segment pass sums k k^T and k over each segment; the chunk pass of segment
// s starts from the sums of the segments before it.

template <typename T, int D>
struct QCfg {
  static constexpr int ES = (int)sizeof(T);
  static constexpr int KS = Mma<T>::KS;
  static constexpr int NKD = D / KS;
  static constexpr int NKC = kC / KS;
  static constexpr int PAD = ES == 2 ? 8 : 4;
  static constexpr int PQ = D + PAD;
  static constexpr int PP = kC + PAD;
  static constexpr int NCT = D / 16;  // feature tiles
  static constexpr int o_q = 0;
  static constexpr int o_k = o_q + kC * PQ * ES;
  static constexpr int o_dot = o_k + kC * PQ * ES;  // [16][PQ]: w hi, w lo, m hi, m lo, zeros
  static constexpr int o_p = o_dot + 16 * PQ * ES;
  static constexpr int o_rd = o_p + kC * PP * ES;    // [64][4] f32 dot results
  static constexpr int o_ab = o_rd + kC * 4 * 4;     // [2][64] f32 alpha, beta
  static constexpr int bytes = o_ab + 2 * kC * 4;
  static_assert(bytes <= 160 * 1024, "LDS budget");
  static constexpr int VR = D * ES / 16;
  static constexpr int NQ = (kC * VR + kNT - 1) / kNT;
  static constexpr int NMT = NCT * NCT;  // M tiles (segment pass: shared out over waves)
  static constexpr int MPW = (NMT + kNW - 1) / kNW;
};

struct QArgs {
  const void* q;
  const void* k;
  const float* w_lambda;
  const float* b_lambda;
  void* qc;
  float* agg;  // [BH][P][sfl]: sum k k^T (D x D), sum k (D)
  const float* state_in;  // optional: [M | m] at state_in + bh * sstride
  int64_t sstride;
  bool keep_final;  // the last segment stores its final sums in block P - 1 of agg
  int64_t N, seg_len, t_in;
  int H, BH, P, sfl;
};

// Segment pass: sums of k k^T and k over segment blockIdx.x of (b, h) blockIdx.y.
template <typename T, int D>
__global__ __launch_bounds__(kNT) void cq_agg_kernel(QArgs a) {
  typedef QCfg<T, D> C;
  typedef Mma<T> M;
  __shared__ __attribute__((aligned(16))) char sm[C::o_dot];
  T* sK = reinterpret_cast<T*>(sm + C::o_k);
  const int s = blockIdx.x, bh = blockIdx.y;
  const int w = wave_id(), l = lane_id(), g = l >> 4, l16 = l & 15, tid = threadIdx.x;
  const int64_t t0 = (int64_t)s * a.seg_len;
  const int64_t t1 = t0 + a.seg_len < a.N ? t0 + a.seg_len : a.N;
  f32x4 acc[C::MPW];
#pragma unroll
  for (int j = 0; j < C::MPW; ++j) acc[j] = zero4();
  float msum = 0.f;
  const T* kb = static_cast<const T*>(a.k) + (size_t)bh * a.N * D;
  RowVecs<T, D, D> pk;  // the next chunk's keys (rows past the segment end read as zero)
  pk.load(kb, t0, t1);
  for (int64_t c0 = t0; c0 < t1; c0 += kC) {
    pk.store(sK, C::PQ);
    lds_barrier();
    if (c0 + kC < t1) pk.load(kb, c0 + kC, t1);
#pragma unroll
    for (int j = 0; j < C::MPW; ++j) {
      const int t = w + kNW * j;
      if (t < C::NMT) {
        const int ra = t % C::NCT, cb = t / C::NCT;
#pragma unroll
        for (int ks = 0; ks < C::NKC; ++ks)
          acc[j] = M::mma(ld_km_chain(sK, C::PQ, 16 * ra, ks), ld_km_chain(sK, C::PQ, 16 * cb, ks), acc[j]);
      }
    }
    if (tid < D)
      for (int r = 0; r < kC; ++r) msum += to_f32(sK[r * C::PQ + tid]);
    lds_barrier();
  }
  float* dst = a.agg + ((size_t)bh * a.P + s) * a.sfl;
#pragma unroll
  for (int j = 0; j < C::MPW; ++j) {
    const int t = w + kNW * j;
    if (t < C::NMT) {
      const int ra = t % C::NCT, cb = t / C::NCT;
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(16 * ra + 4 * g + e) * D + 16 * cb + l16] = acc[j][e];
    }
  }
  if (tid < D) dst[D * D + tid] = msum;
}

// Chunk pass: clean queries of segment blockIdx.x of (b, h) blockIdx.y.
template <typename T, int D>
__global__ __launch_bounds__(kNT) void cq_kernel(QArgs a) {
  typedef QCfg<T, D> C;
  typedef Mma<T> M;
  __shared__ __attribute__((aligned(16))) char sm[C::bytes];
  T* sQ = reinterpret_cast<T*>(sm + C::o_q);
  T* sK = reinterpret_cast<T*>(sm + C::o_k);
  T* sDot = reinterpret_cast<T*>(sm + C::o_dot);
  T* sP = reinterpret_cast<T*>(sm + C::o_p);
  float* sRd = reinterpret_cast<float*>(sm + C::o_rd);
  float* sAl = reinterpret_cast<float*>(sm + C::o_ab);
  float* sBe = sAl + kC;
  const int s = blockIdx.x, bh = blockIdx.y, h = bh % a.H;
  const int w = wave_id(), l = lane_id(), g = l >> 4, l16 = l & 15, tid = threadIdx.x;
  const int64_t t0 = (int64_t)s * a.seg_len;
  const int64_t t1 = t0 + a.seg_len < a.N ? t0 + a.seg_len : a.N;
  const bool owner = w < C::NCT;  // owns feature tile cw = w of delta, M's columns and m
  const int cw = w;

  // running sums before the segment: the caller's state plus the segments before it
  f32x4 Mt[C::NCT];
  float mv = 0.f;
#pragma unroll
  for (int at = 0; at < C::NCT; ++at) Mt[at] = zero4();
  if (owner) {
    const int col = 16 * cw + l16;
    if (a.state_in) {
      const float* src = a.state_in + (size_t)bh * a.sstride;
#pragma unroll
      for (int at = 0; at < C::NCT; ++at)
#pragma unroll
        for (int e = 0; e < 4; ++e) Mt[at][e] = src[(16 * at + 4 * g + e) * D + col];
      mv = src[D * D + col];
    }
    for (int sp = 0; sp < s; ++sp) {
      const float* src = a.agg + ((size_t)bh * a.P + sp) * a.sfl;
#pragma unroll
      for (int at = 0; at < C::NCT; ++at)
#pragma unroll
        for (int e = 0; e < 4; ++e) Mt[at][e] += src[(16 * at + 4 * g + e) * D + col];
      mv += src[D * D + col];
    }
  }
  // gate weights (split into two operand-type terms for bf16) and the key sum
  for (int i = tid; i < 16 * D; i += kNT) {
    const int r = i / D, f = i % D;
    float x = 0.f;
    if (r == 0 || r == 1) {
      const float wv = a.w_lambda[(size_t)h * D + f];
      x = r == 0 ? to_f32(cvt<T>(wv)) : wv - to_f32(cvt<T>(wv));
    }
    sDot[r * C::PQ + f] = cvt<T>(x);
  }
  for (int i = tid; i < kC * kC; i += kNT) {
    const int r = i / kC, c = i % kC;
    if ((c >> 4) > (r >> 4)) sP[r * C::PP + c] = cvt<T>(0.f);
  }
  lds_barrier();
  if (owner && g == 0) {
    const T hi = cvt<T>(mv);
    sDot[2 * C::PQ + 16 * cw + l16] = hi;
    sDot[3 * C::PQ + 16 * cw + l16] = cvt<T>(mv - to_f32(hi));
  }
  const float bias = a.b_lambda[h];
  T* qcp = static_cast<T*>(a.qc);

  const T* qb = static_cast<const T*>(a.q) + (size_t)bh * a.N * D;
  const T* kb = static_cast<const T*>(a.k) + (size_t)bh * a.N * D;
  RowVecs<T, D, D> pq, pk;  // the next chunk's rows (past the segment end: zero)
  pq.load(qb, t0, t1);
  pk.load(kb, t0, t1);
  for (int64_t c0 = t0; c0 < t1; c0 += kC) {
    pq.store(sQ, C::PQ);
    pk.store(sK, C::PQ);
    lds_barrier();
    if (c0 + kC < t1) {
      pq.load(qb, c0 + kC, t1);
      pk.load(kb, c0 + kC, t1);
    }
    // ---- raw scores (lower, rounded once) and the gate / key-sum dots
    for (int t = w; t < 14; t += kNW) {
      if (t < 10) {
        int it, jt;
        tri_tile(t, it, jt);
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < C::NKD; ++ks)
          acc = M::mma(ld_kc_chain(sQ, C::PQ, 16 * it + l16, ks), ld_kc_chain(sK, C::PQ, 16 * jt + l16, ks), acc);
        const int j = 16 * jt + l16;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * it + 4 * g + e;
          sP[i * C::PP + j] = cvt<T>(j <= i ? acc[e] : 0.f);
        }
      } else {
        const int r = t - 10;
        f32x4 acc = zero4();
#pragma unroll
        for (int ks = 0; ks < C::NKD; ++ks)
          acc = M::mma(ld_kc_chain(sQ, C::PQ, 16 * r + l16, ks), ld_kc_chain(sDot, C::PQ, l16, ks), acc);
        if (l16 < 4) {
#pragma unroll
          for (int e = 0; e < 4; ++e) sRd[(16 * r + 4 * g + e) * 4 + l16] = acc[e];
        }
      }
    }
    lds_barrier();
    // ---- per-row gate and coefficients
    if (w == 0) {
      const int i = l;
      float rs = 0.f;
      typedef typename Vec16<T>::type vec;
#pragma unroll
      for (int j = 0; j < kC; j += Vec16<T>::n) {
        const vec x = *reinterpret_cast<const vec*>(sP + i * C::PP + j);
#pragma unroll
        for (int e = 0; e < Vec16<T>::n; ++e) rs += to_f32(x[e]);
      }
      const float wq = sRd[i * 4 + 0] + sRd[i * 4 + 1];
      const float mq = sRd[i * 4 + 2] + sRd[i * 4 + 3];
      const float lam = 1.f / (1.f + __expf(-(wq + bias)));
      const float tc = (float)(a.t_in + c0 + i + 1);
      const bool ok = c0 + i < t1;
      const float al = ok ? lam / tc : 0.f;
      sAl[i] = al;
      sBe[i] = ok ? al * (mq + rs) / tc : 0.f;
    }
    lds_barrier();
    // ---- delta for this wave's feature tile, the clean query, the running sums
    if (owner) {
      typename M::frag mh[C::NKD], ml[C::NKD];
#pragma unroll
      for (int ks = 0; ks < C::NKD; ++ks) {
        if constexpr (sizeof(T) == 2) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float x0 = Mt[2 * ks][e], x1 = Mt[2 * ks + 1][e];
            mh[ks][e] = (bf16)x0;
            mh[ks][4 + e] = (bf16)x1;
            ml[ks][e] = (bf16)(x0 - (float)mh[ks][e]);
            ml[ks][4 + e] = (bf16)(x1 - (float)mh[ks][4 + e]);
          }
        } else {
          mh[ks] = Mt[ks >> 2][ks & 3];
        }
      }
      const int f = 16 * cw + l16;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        f32x4 acc = zero4(), z = zero4();
#pragma unroll
        for (int ks = 0; ks < C::NKD; ++ks) {
          const typename M::frag aq = ld_kc_chain(sQ, C::PQ, 16 * r + l16, ks);
          acc = M::mma(aq, mh[ks], acc);
          if constexpr (sizeof(T) == 2) acc = M::mma(aq, ml[ks], acc);
        }
        const int nk = tok_steps<T>(r);
        for (int ks = 0; ks < nk; ++ks) {
          const typename M::frag bk = ld_km_chain(sK, C::PQ, 16 * cw, ks);
          acc = M::mma(ld_kc_chain(sP, C::PP, 16 * r + l16, ks), bk, acc);
          z = M::mma(tri_ones<T>(ks, 16 * r + l16), bk, z);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 16 * r + 4 * g + e;
          if (c0 + i < t1) {
            const float d = -sAl[i] * acc[e] + sBe[i] * (z[e] + mv);
            qcp[((size_t)bh * a.N + c0 + i) * D + f] = cvt<T>(to_f32(sQ[i * C::PQ + f]) + d);
          }
        }
      }
      // running sums over the chunk's keys
      f32x4 cs = zero4();
#pragma unroll
      for (int ks = 0; ks < C::NKC; ++ks) {
        const typename M::frag bk = ld_km_chain(sK, C::PQ, 16 * cw, ks);
        cs = M::mma(ones_frag<T>(), bk, cs);
#pragma unroll
        for (int at = 0; at < C::NCT; ++at) Mt[at] = M::mma(ld_km_chain(sK, C::PQ, 16 * at, ks), bk, Mt[at]);
      }
      mv += cs[0];
    }
    lds_barrier();  // all reads of sQ, sK, sP and the key-sum row are done
    if (owner && g == 0) {
      const T hi = cvt<T>(mv);
      sDot[2 * C::PQ + 16 * cw + l16] = hi;
      sDot[3 * C::PQ + 16 * cw + l16] = cvt<T>(mv - to_f32(hi));
    }
  }
  if (a.keep_final && s == a.P - 1 && owner) {
    float* dst = a.agg + ((size_t)bh * a.P + s) * a.sfl;  // block P - 1 is not a segment sum
    const int col = 16 * cw + l16;
#pragma unroll
    for (int at = 0; at < C::NCT; ++at)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(16 * at + 4 * g + e) * D + col] = Mt[at][e];
    if (g == 0) dst[D * D + col] = mv;
  }
}

template <typename T, int D>
hipError_t run(const DeltaLaunch& L, hipStream_t st) {
  const int BH = (int)(L.B * L.H);
  const int64_t nch = (L.N + kC - 1) / kC;
  if (L.ccq) {
    QArgs q;
    q.q = L.q;
    q.k = L.k;
    q.w_lambda = L.w_lambda;
    q.b_lambda = L.b_lambda;
    q.qc = L.qc;
    q.agg = L.agg;
    q.state_in = L.state_in ? L.state_in + L.D * L.dv : nullptr;
    q.sstride = L.sstride;
    q.keep_final = L.state_out != nullptr;
    q.N = L.N;
    q.seg_len = L.seg_len;
    q.t_in = L.t_in;
    q.H = (int)L.H;
    q.BH = BH;
    q.P = (int)L.P;
    q.sfl = (int)cq_state_floats(L.D);
    if (L.P > 1) {
      hipLaunchKernelGGL((cq_agg_kernel<T, D>), dim3((unsigned)(L.P - 1), (unsigned)BH), dim3(kNT), 0, st, q);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL((cq_kernel<T, D>), dim3((unsigned)L.P, (unsigned)BH), dim3(kNT), 0, st, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  {
    PArgs p;
    p.k = L.k;
    p.v = L.v;
    p.g = L.g;
    p.beta = L.beta;
    p.w = L.wbuf;
    p.ut = L.ubuf;
    p.N = L.N;
    // about four workgroups per CU over the whole launch
    int64_t per = (nch * BH + 1023) / 1024;
    if (per < 1) per = 1;
    p.cpb = (int)per;
    const unsigned nb = (unsigned)((nch + per - 1) / per);
    hipLaunchKernelGGL((gdn_prep_kernel<T, D>), dim3(nb, (unsigned)BH), dim3(kNT), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  Args a;
  a.q = L.ccq ? L.qc : L.q;
  a.k = L.k;
  a.w = L.wbuf;
  a.ut = L.ubuf;
  a.g = L.g;
  a.out = L.out;
  a.state_in = L.state_in;
  a.state_out = L.state_out;
  a.sstride = L.sstride;
  a.mfinal = L.ccq ? L.agg : nullptr;
  a.P = (int)L.P;
  a.sfl = (int)cq_state_floats(L.D);
  a.N = L.N;
  a.BH = BH;
  a.dv = (int)L.dv;
  const unsigned groups = (unsigned)(BH * (L.dv / kCG));
  hipLaunchKernelGGL((gdn_kernel<T, D>), dim3(groups), dim3(kNT), 0, st, a);
  return hipGetLastError();
}

}  // namespace gdn

hipError_t deltanet_launch(const DeltaLaunch& L, hipStream_t st) {
  if (L.bf16) {
    switch (L.D) {
      case 32: return gdn::run<bf16, 32>(L, st);
      case 64: return gdn::run<bf16, 64>(L, st);
      case 128: return gdn::run<bf16, 128>(L, st);
    }
  } else {
    switch (L.D) {
      case 32: return gdn::run<float, 32>(L, st);
      case 64: return gdn::run<float, 64>(L, st);
    }
  }
  return hipErrorInvalidValue;
}

}  // namespace lm
