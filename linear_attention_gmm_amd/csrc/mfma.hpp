// mfma.hpp -- CDNA4 (gfx950) matrix-core and wavefront helpers shared by the
// mixer kernels.
//
// Matrix products use 16x16 output tiles:
//   bf16: v_mfma_f32_16x16x32_bf16  (k-step 32, 8 bf16 per lane per operand)
//   f32 : v_mfma_f32_16x16x4_f32    (k-step 4, 1 float per lane per operand)
// Lane layouts (verified on gfx950):
//   A (16 x k): lane l holds row l%16; its k-values come from lane group g = l/16.
//   B (k x 16): lane l holds column l%16; k-values from group g.
//   D (16 x 16, fp32): lane l holds column l%16, rows 4g..4g+3 (one f32x4).
//
// Which k-values a group holds within one k-step is a free choice, so long as
// A and B agree. Two orders are used:
//   NATURAL: bf16 k = 8g..8g+7 ; f32 k = g.
//   CHAIN  : the order in which a D tile's rows sit in registers. This lets an
//            accumulator feed the next product straight from registers.
//            bf16 (32 rows = tiles t0, t1): k = {4g..4g+3} U {16+4g..16+4g+3};
//            f32 (step s of a 16-row tile): k = 4g + s.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lm {

typedef __bf16 bf16;
typedef bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));

#define LM_LDS __attribute__((address_space(3)))

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }
// Uniform across the wave (one-dimensional workgroups of whole waves), so it is
// moved to a scalar register: offsets derived from it then take no VGPRs.
__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

template <typename T>
struct Mma;

template <>
struct Mma<bf16> {
  static constexpr int KS = 32;
  typedef bf16x8 frag;
  __device__ static __forceinline__ f32x4 mma(const frag& a, const frag& b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag zero() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.f;
    return z;
  }
  // CHAIN fragment of k-step s from D tiles stacked along k (tiles[2s], tiles[2s+1]).
  __device__ static __forceinline__ frag chain(const f32x4* tiles, int s) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (bf16)tiles[2 * s][i];
      f[4 + i] = (bf16)tiles[2 * s + 1][i];
    }
    return f;
  }
  // Same from two explicit tiles.
  __device__ static __forceinline__ frag chain2(const f32x4& t0, const f32x4& t1) {
    frag f;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[i] = (bf16)t0[i];
      f[4 + i] = (bf16)t1[i];
    }
    return f;
  }
};

template <>
struct Mma<float> {
  static constexpr int KS = 4;
  typedef float frag;
  __device__ static __forceinline__ f32x4 mma(frag a, frag b, const f32x4& c) {
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ frag zero() { return 0.f; }
  __device__ static __forceinline__ frag chain(const f32x4* tiles, int s) { return tiles[s >> 2][s & 3]; }
};

// Number of 16-row D tiles one k-step spans in CHAIN order.
template <typename T>
struct ChainTiles {
  static constexpr int value = 2;  // bf16: 32 rows
};
template <>
struct ChainTiles<float> {
  static constexpr int value = 0;  // f32: 4 steps share one tile (use Mma<float>::chain)
};

// ---------------------------------------------------------------------------
// LDS fragment loads. `base` points at element (row 0, col 0) of a row-major
// LDS tile with `pitch` elements per row.

// k contiguous in memory: operand row/column index `rc` (the lane's row of A or
// column of B) is a memory row, k runs along the row. NATURAL order.
__device__ __forceinline__ bf16x8 ld_kc_nat(const bf16* base, int pitch, int rc, int kstep) {
  const int g = lane_id() >> 4;
  return *reinterpret_cast<const bf16x8*>(base + rc * pitch + kstep * 32 + 8 * g);
}
__device__ __forceinline__ float ld_kc_nat(const float* base, int pitch, int rc, int kstep) {
  const int g = lane_id() >> 4;
  return base[rc * pitch + kstep * 4 + g];
}
// CHAIN order, k contiguous.
__device__ __forceinline__ bf16x8 ld_kc_chain(const bf16* base, int pitch, int rc, int kstep) {
  const int g = lane_id() >> 4;
  const bf16* p = base + rc * pitch + kstep * 32 + 4 * g;
  bf16x4 lo = *reinterpret_cast<const bf16x4*>(p);
  bf16x4 hi = *reinterpret_cast<const bf16x4*>(p + 16);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ float ld_kc_chain(const float* base, int pitch, int rc, int kstep) {
  const int g = lane_id() >> 4;
  return base[rc * pitch + 16 * (kstep >> 2) + 4 * g + (kstep & 3)];
}

// k-major in memory: k is the memory row, the operand's row/column index is the
// memory column. `c0` is the first column of the 16-wide tile. CHAIN order.
// bf16 uses the gfx950 LDS transpose read: each 16-lane group reads a 4 x 16
// block (lane j of the group supplies row k0 + j/4, columns c0 + 4(j%4)..+3)
// and lane p of the group receives column c0 + p of the four rows.
__device__ __forceinline__ bf16x4 tr16(const bf16* base, int pitch, int c0, int k0) {
  const int j = lane_id() & 15;
  const bf16* p = base + (k0 + (j >> 2)) * pitch + c0 + 4 * (j & 3);
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p));
  return __builtin_bit_cast(bf16x4, r);
}
__device__ __forceinline__ bf16x8 ld_km_chain(const bf16* base, int pitch, int c0, int kstep) {
  const int g = lane_id() >> 4;
  bf16x4 lo = tr16(base, pitch, c0, kstep * 32 + 4 * g);
  bf16x4 hi = tr16(base, pitch, c0, kstep * 32 + 16 + 4 * g);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
__device__ __forceinline__ float ld_km_chain(const float* base, int pitch, int c0, int kstep) {
  const int g = lane_id() >> 4;
  const int k = 16 * (kstep >> 2) + 4 * g + (kstep & 3);
  return base[k * pitch + c0 + (lane_id() & 15)];
}

// ---------------------------------------------------------------------------
// Swizzled LDS tiles filled by direct global->LDS DMA.
//
// A tile holds 64 rows of RB = D * sizeof(T) bytes, unpadded, cut into 16-byte
// chunks (CPR = RB / 16 per row). Logical chunk c of row r sits at physical
// chunk c ^ sw(r). gfx950 serves 16-byte LDS reads in passes of 16 lanes
// ({0-3, 12-15, 20-27}, {4-11, 16-19, 28-31}, and the same above lane 32) over
// 64 banks of 4 bytes, and 8-byte reads (plain or transposed) in passes of 32
// lanes. sw is chosen so that these read shapes hit distinct banks:
//   * 16 consecutive rows, same 16-byte chunk (b128 operand reads);
//   * 16 consecutive rows, same 8-byte half-chunk (b64 reads, CHAIN order);
//   * 8 consecutive rows, two adjacent chunks each (the transpose read).
// For 16 chunks per row, ((r % 8) << 1) ^ 9 (r / 8 % 2) does all three.
// The DMA writes 64 consecutive physical chunks per wave instruction, so the
// swizzle is applied to the global source addresses instead.
template <int CPR>
__device__ __forceinline__ int tile_sw(int r) {
  if constexpr (CPR == 16) {
    return ((r & 7) << 1) ^ (((r >> 3) & 1) * 9);
  } else if constexpr (CPR > 16) {
    return ((r & 7) << 1) | ((r >> 3) & 1);
  } else {
    constexpr int RPL = 16 / CPR;  // rows per 256-byte bank line
    const int u = r / RPL;
    return ((u & (CPR / 2 - 1)) << 1) | ((u / (CPR / 2)) & 1);
  }
}

// Byte offset of element `col` of row `r` (element size ES) in a swizzled tile.
template <int CPR, int ES>
__device__ __forceinline__ int tile_off(int r, int col) {
  constexpr int EPC = 16 / ES;  // elements per chunk
  return r * (CPR * 16) + (((col / EPC) ^ tile_sw<CPR>(r)) * 16) + (col % EPC) * ES;
}

// Buffer resource over `nbytes` bytes at `base` (raw, stride 0). Loads past
// nbytes return 0, which is how the tail of a sequence reads as zero rows.
typedef __amdgpu_buffer_rsrc_t rsrc_t;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}

// Buffer descriptor words over `nbytes` bytes at `base` (raw, stride 0, 32-bit
// data format), for the inline-asm transfers below.
typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
__device__ __forceinline__ u32x4 buf_desc(const void* base, uint32_t nbytes) {
  const unsigned long long a = reinterpret_cast<unsigned long long>(base);
  u32x4 d;
  d[0] = (unsigned)a;
  d[1] = (unsigned)(a >> 32) & 0xffffu;
  d[2] = nbytes;
  d[3] = 0x00020000u;
  return d;
}
// LDS byte address of a generic pointer into LDS: its low 32 bits (the high
// half is the shared aperture). Taken directly rather than by an address-space
// cast, whose null-pointer check the backend can mis-lower.
__device__ __forceinline__ unsigned lds_addr(const void* p) {
  return __builtin_amdgcn_readfirstlane((unsigned)reinterpret_cast<uintptr_t>(p));
}

// Direct global->LDS transfers written as inline asm: LDS[dst + 16 lane] (or
// 4 lane) = global[desc base + voff], 0 past the descriptor's range. The
// compiler does not see these as LDS stores, so it inserts no waits for them
// at unrelated LDS accesses; callers wait for them explicitly (vmcnt) and
// publish them with a barrier before any LDS read of the destination.
#pragma clang diagnostic push
#pragma clang diagnostic ignored "-Winline-asm"
__device__ __forceinline__ void lds_dma16(const u32x4& desc, int voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);  // keeps the operand scalar
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(desc), "s"(m)
               : "memory", "m0");
}
__device__ __forceinline__ void lds_dma4(const u32x4& desc, int voff, unsigned lds) {
  const unsigned m = __builtin_amdgcn_readfirstlane(lds);
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dword %0, %1, 0 offen lds" ::"v"(voff), "s"(desc), "s"(m)
               : "memory", "m0");
}
#pragma clang diagnostic pop

// This wave's share of the DMA of a 64 x D tile into a swizzled LDS tile: each
// wave moves INSTR blocks of 64 consecutive physical chunks. The per-lane byte
// offsets in the (row-major, unswizzled) source are fixed, so they are computed
// once; only the buffer base changes from chunk to chunk.
template <typename T, int D, int NW>
struct TileDma {
  static constexpr int CPR = D * (int)sizeof(T) / 16;
  static constexpr int INSTR = CPR / NW;
  static_assert(CPR % NW == 0, "tile split");
  int voff[INSTR];
  __device__ __forceinline__ void init() {
    const int l = lane_id(), w = wave_id();
#pragma unroll
    for (int i = 0; i < INSTR; ++i) {
      const int p = (w * INSTR + i) * 64 + l;
      const int r = p / CPR, pc = p - (p / CPR) * CPR;
      voff[i] = r * CPR * 16 + ((pc ^ tile_sw<CPR>(r)) * 16);
    }
  }
  // src: the tile's first row in global memory; rows: rows of the sequence left from src.
  __device__ __forceinline__ void issue(char* dst, const T* src, int rows) const {
    const int w = wave_id();
    const u32x4 d = buf_desc(src, (uint32_t)((rows < 64 ? rows : 64) * D * (int)sizeof(T)));
    const unsigned base = lds_addr(dst) + (unsigned)(w * INSTR * 1024);
#pragma unroll
    for (int i = 0; i < INSTR; ++i) lds_dma16(d, voff[i], base + (unsigned)(i * 1024));
  }
};

// Waits for this wave's outstanding vector memory operations (loads, LDS DMA, stores).
__device__ __forceinline__ void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// Waits until at most n (< 16) of this wave's vector memory operations are
// outstanding (they complete in order for loads).
#define LM_WAIT_VMEM(n) __builtin_amdgcn_s_waitcnt(0x0f70 | (n))

// Workgroup barrier for LDS traffic only: this wave's LDS reads and writes are
// complete, then all waves meet. Unlike __syncthreads() it does not wait for
// outstanding global loads, stores or LDS DMA (those are waited for
// explicitly where their data is needed). The empty asm statements keep the
// compiler from moving memory accesses across the barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0)
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Operand fragments from a swizzled tile.
// NATURAL order, k contiguous along the row: row `r`, k-step `ks`.
template <int CPR>
__device__ __forceinline__ bf16x8 tl_nat(const char* t, int r, int ks) {
  const int g = lane_id() >> 4;
  return *reinterpret_cast<const bf16x8*>(t + tile_off<CPR, 2>(r, ks * 32 + 8 * g));
}
template <int CPR>
__device__ __forceinline__ float tl_nat_f(const char* t, int r, int ks) {
  const int g = lane_id() >> 4;
  return *reinterpret_cast<const float*>(t + tile_off<CPR, 4>(r, ks * 4 + g));
}
// CHAIN order, k contiguous along the row.
template <int CPR>
__device__ __forceinline__ bf16x8 tl_chain(const char* t, int r, int ks) {
  const int g = lane_id() >> 4;
  const bf16x4 lo = *reinterpret_cast<const bf16x4*>(t + tile_off<CPR, 2>(r, ks * 32 + 4 * g));
  const bf16x4 hi = *reinterpret_cast<const bf16x4*>(t + tile_off<CPR, 2>(r, ks * 32 + 16 + 4 * g));
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <int CPR>
__device__ __forceinline__ float tl_chain_f(const char* t, int r, int ks) {
  const int g = lane_id() >> 4;
  return *reinterpret_cast<const float*>(t + tile_off<CPR, 4>(r, 16 * (ks >> 2) + 4 * g + (ks & 3)));
}
// k-major: k = tile row, the operand's row/column index = tile column c0 + lane%16.
// CHAIN order over k (group g holds k = 4g..4g+3 and 16+4g..16+4g+3 of the
// step), read through the transpose read: each 16-lane group reads 4 rows x 16
// columns, and the two reads of a half-wave cover 8 consecutive rows.
template <int CPR>
__device__ __forceinline__ bf16x4 tl_tr16(const char* t, int k0, int c0) {
  const int j = lane_id() & 15;
  const int r = k0 + (j >> 2);
  const char* p = t + tile_off<CPR, 2>(r, c0 + 4 * (j & 3));
  const i16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((i16x4 LM_LDS*)(p));
  return __builtin_bit_cast(bf16x4, v);
}
template <int CPR>
__device__ __forceinline__ bf16x8 tl_kmaj(const char* t, int ks, int c0) {
  const int g = lane_id() >> 4;
  const bf16x4 lo = tl_tr16<CPR>(t, ks * 32 + 4 * g, c0);
  const bf16x4 hi = tl_tr16<CPR>(t, ks * 32 + 16 + 4 * g, c0);
  return bf16x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
}
template <int CPR>
__device__ __forceinline__ float tl_kmaj_f(const char* t, int ks, int c0) {
  const int g = lane_id() >> 4;
  const int k = 16 * (ks >> 2) + 4 * g + (ks & 3);
  return *reinterpret_cast<const float*>(t + tile_off<CPR, 4>(k, c0 + (lane_id() & 15)));
}

// Type-generic front ends.
template <int CPR, typename T>
__device__ __forceinline__ typename Mma<T>::frag tl_nat_t(const char* t, int r, int ks) {
  if constexpr (sizeof(T) == 2) return tl_nat<CPR>(t, r, ks); else return tl_nat_f<CPR>(t, r, ks);
}
template <int CPR, typename T>
__device__ __forceinline__ typename Mma<T>::frag tl_chain_t(const char* t, int r, int ks) {
  if constexpr (sizeof(T) == 2) return tl_chain<CPR>(t, r, ks); else return tl_chain_f<CPR>(t, r, ks);
}
template <int CPR, typename T>
__device__ __forceinline__ typename Mma<T>::frag tl_kmaj_t(const char* t, int ks, int c0) {
  if constexpr (sizeof(T) == 2) return tl_kmaj<CPR>(t, ks, c0); else return tl_kmaj_f<CPR>(t, ks, c0);
}

// k index of element i of this lane's fragment for k-step ks, CHAIN order.
template <typename T>
__device__ __forceinline__ int chain_k(int ks, int i) {
  const int g = lane_id() >> 4;
  if constexpr (sizeof(T) == 2) return ks * 32 + (i < 4 ? 4 * g + i : 16 + 4 * g + i - 4);
  else return 16 * (ks >> 2) + 4 * g + (ks & 3);
}

// ---------------------------------------------------------------------------
// Wave reductions.

// Across the four 16-lane groups (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float group_max(float x) {
  x = fmaxf(x, __shfl_xor(x, 16));
  x = fmaxf(x, __shfl_xor(x, 32));
  return x;
}
__device__ __forceinline__ float group_sum(float x) {
  x += __shfl_xor(x, 16);
  x += __shfl_xor(x, 32);
  return x;
}

// Sum over the 16 lanes of a row (DPP row rotations); every lane gets the sum.
__device__ __forceinline__ float row16_sum(float x) {
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x128, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x124, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x122, 0xf, 0xf, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_mov_dpp(__builtin_bit_cast(int, x), 0x121, 0xf, 0xf, false));
  return x;
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Inclusive prefix sum over the 64 lanes of a wave: shifts within 16-lane rows
// (DPP, zero fill at the row start), then each row adds the totals of the rows
// before it (read from lanes 15, 31, 47).
template <int CTRL>
__device__ __forceinline__ float dpp_shr(float x) {
  return __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), CTRL, 0xf, 0xf, true));
}
__device__ __forceinline__ float wave_scan_incl(float x) {
  x += dpp_shr<0x111>(x);  // row_shr:1
  x += dpp_shr<0x112>(x);  // row_shr:2
  x += dpp_shr<0x114>(x);  // row_shr:4
  x += dpp_shr<0x118>(x);  // row_shr:8
  const float r0 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 15));
  const float r1 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 31));
  const float r2 = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, x), 47));
  const int row = lane_id() >> 4;
  return x + (row == 0 ? 0.f : row == 1 ? r0 : row == 2 ? r0 + r1 : r0 + r1 + r2);
}

// ---------------------------------------------------------------------------
// Element conversion.
template <typename T>
__device__ __forceinline__ float to_f32(T x) {
  return (float)x;
}
template <typename T>
__device__ __forceinline__ T from_f32(float x) {
  return (T)x;
}

// 16-byte vector of T.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16> {
  static constexpr int n = 8;
  typedef bf16x8 type;
};
template <>
struct Vec16<float> {
  static constexpr int n = 4;
  typedef f32x4 type;
};

}  // namespace lm
