// linattn_bwd.hip -- helper kernels of the backward pass of decayed linear
// attention (allinfo.ai.kr linear attention post, "Key messages": the matrix
// state with decay gates; the gradients follow from the recurrence).
//
// With S_t = g_t S_{t-1} + k_t v_t^T, o_t = S_t^T q_t and the output gradient
// do_t, the gradients are again decayed linear attentions, so the chunk kernel
// computes them:
//   dq_t = S_t do_t                         forward(q = do, k = v, v = k, g)
//   U_t  = q_t do_t^T + g_{t+1} U_{t+1}     (gradient of the state)
//   dk_t = U_t v_t, dv_t = U_t^T k_t        forward on the time-reversed
//                                           sequence with the gates shifted by
//                                           one token
//   dg_t = (1 / g_t) sum_{m >= t} (q_m . dq_m - k_m . dk_m)
// (the last line: the loss depends on the gates through the decays
// exp(L_i - L_j), L the cumulative log gate; the derivative with respect to L_m
// is q_m . dq_m - k_m . dk_m, and L_m sums the log gates up to m).
// The kernels below reverse sequences in time, shift the gates and form dg.
// For bf16 inputs the dq and dk passes run in float32 on float32 copies and
// those gradients are rounded once at the end: dg is a difference of two dot
// products that nearly cancel, which bf16-rounded dq and dk would not resolve.
// The dv pass, which dg does not use, runs on the bf16 inputs directly.
#include "mfma.hpp"
#include "launch.hpp"
#include "bwd.hpp"

namespace lm {
namespace bwd {

// out[bh][t][:] = in[bh][N - 1 - t][:], in 16-byte pieces (D * es a multiple of 16).
__global__ __launch_bounds__(256) void reverse_time(const char* __restrict__ in, char* __restrict__ out, int64_t N,
                                                    int row_bytes, int64_t total16) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total16) return;
  const int per_row = row_bytes / 16;
  const int64_t row = i / per_row;  // bh * N + t
  const int c = (int)(i - row * per_row);
  const int64_t bh = row / N, t = row - bh * N;
  const int64_t src = bh * N + (N - 1 - t);
  *reinterpret_cast<uint4*>(out + row * row_bytes + (int64_t)c * 16) =
      *reinterpret_cast<const uint4*>(in + src * row_bytes + (int64_t)c * 16);
}

// Gates of the reversed recurrence: gr[bh][t'] = g[bh][N - t'] for t' >= 1; the
// first reversed token has no successor, so its gate multiplies zero (1 here).
__global__ __launch_bounds__(256) void shift_gates(const float* __restrict__ g, float* __restrict__ gr, int64_t N,
                                                   int64_t total) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total) return;
  const int64_t bh = i / N, t = i - bh * N;
  gr[i] = t == 0 ? 1.f : g[bh * N + (N - t)];
}

// x_m = q_m . dq_m - k_m . dk_m for every token (float32), one wave per token:
// lanes over the features, a wave sum. Written into dg. With dq16 / dk16 the
// gradients are also written rounded to bf16 (the final outputs for bf16
// inputs, saving a separate conversion pass over dq and dk).
template <int D>
__global__ __launch_bounds__(256) void gate_dots(const float* __restrict__ q, const float* __restrict__ dq,
                                                 const float* __restrict__ k, const float* __restrict__ dk,
                                                 float* __restrict__ x, int64_t rows, bf16* __restrict__ dq16,
                                                 bf16* __restrict__ dk16) {
  const int l = lane_id();
  const int64_t row0 = ((int64_t)blockIdx.x * 4 + wave_id()) * 16;
  for (int rr = 0; rr < 16; ++rr) {
    const int64_t row = row0 + rr;
    if (row >= rows) break;
    float s = 0.f;
#pragma unroll
    for (int i = l; i < D; i += 64) {
      const size_t o = (size_t)row * D + i;
      const float a = dq[o], b = dk[o];
      s += q[o] * a - k[o] * b;
      if (dq16) {
        dq16[o] = from_f32<bf16>(a);
        dk16[o] = from_f32<bf16>(b);
      }
    }
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) s += __shfl_xor(s, off);
    if (l == 0) x[row] = s;
  }
}

// dg_t = (1 / g_t) sum_{m >= t} x_m for one (b, h) per workgroup: thread i owns
// tokens [i len, (i+1) len); the sums of the ranges after it come from LDS.
__global__ __launch_bounds__(256) void gate_suffix(const float* __restrict__ g, float* __restrict__ dg, int64_t N) {
  __shared__ float stot[256];
  const int bh = blockIdx.x, tid = threadIdx.x;
  const int64_t len = (N + 255) / 256;
  const int64_t t0 = (int64_t)tid * len, t1 = t0 + len < N ? t0 + len : N;
  const size_t base = (size_t)bh * N;
  float tot = 0.f;
  for (int64_t m = t0; m < t1; ++m) tot += dg[base + m];
  stot[tid] = tot;
  __syncthreads();
  float run = 0.f;
  for (int u = tid + 1; u < 256; ++u) run += stot[u];
  for (int64_t m = t1 - 1; m >= t0; --m) {
    run += dg[base + m];
    dg[base + m] = run / g[base + m];
  }
}

// Element-wise conversion (float32 <-> bf16), n elements (a multiple of 4).
template <typename TI, typename TO>
__global__ __launch_bounds__(256) void convert(const TI* __restrict__ in, TO* __restrict__ out, int64_t n4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= n4) return;
#pragma unroll
  for (int j = 0; j < 4; ++j) out[4 * i + j] = from_f32<TO>(to_f32(in[4 * i + j]));
}

template <typename TI, typename TO>
static hipError_t convert_n(const void* in, void* out, int64_t n, hipStream_t st) {
  const int64_t n4 = n / 4;
  hipLaunchKernelGGL((convert<TI, TO>), dim3((unsigned)((n4 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const TI*>(in), static_cast<TO*>(out), n4);
  return hipGetLastError();
}

static hipError_t gate_grad_f32(const BwdLaunch& L, const float* q, const float* dq, const float* k, const float* dk,
                                hipStream_t st, bf16* dq16 = nullptr, bf16* dk16 = nullptr) {
  const int64_t rows = L.B * L.H * L.N;
  const unsigned nb = (unsigned)((rows + 63) / 64);
#define LM_GD(DD) \
  hipLaunchKernelGGL((gate_dots<DD>), dim3(nb), dim3(256), 0, st, q, dq, k, dk, L.dg, rows, dq16, dk16)
  switch (L.D) {
    case 32: LM_GD(32); break;
    case 64: LM_GD(64); break;
    case 128: LM_GD(128); break;
    default: return hipErrorInvalidValue;
  }
#undef LM_GD
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(gate_suffix, dim3((unsigned)(L.B * L.H)), dim3(256), 0, st, L.g, L.dg, L.N);
  return hipGetLastError();
}

static hipError_t reverse(const void* in, void* out, const BwdLaunch& L, hipStream_t st, int elem_bytes = 4) {
  const int row_bytes = (int)(L.D * elem_bytes);
  const int64_t total16 = L.B * L.H * L.N * (row_bytes / 16);
  hipLaunchKernelGGL(reverse_time, dim3((unsigned)((total16 + 255) / 256)), dim3(256), 0, st,
                     static_cast<const char*>(in), static_cast<char*>(out), L.N, row_bytes, total16);
  return hipGetLastError();
}

// bf16 operands of the dv pass (for bf16 inputs): the time-reversed bf16 k, q
// and dout, a reversed output buffer, and dv itself.
struct DvBf16 {
  const bf16* rk;
  const bf16* rq;
  const bf16* rdo;
  bf16* rout;
  bf16* dv;
  bf16* dq16;  // optional: dq and dk rounded to bf16 by the gate-gradient pass
  bf16* dk16;
};

// Three chunk-kernel passes (dq; dk and dv on the reversed sequence), the
// reversals around them and (gates) the gate gradient, in float32. With h,
// the dv pass runs on the bf16 chunk kernel instead: dv does not enter the
// gate gradient, whose q . dq - k . dk cancellation is what needs float32.
static hipError_t backward(const BwdLaunch& L, const float* q, const float* k, const float* v, const float* dout,
                           float* dq, float* dk, float* dv, bool gates, const DvBf16* h, hipStream_t st) {
  hipError_t e;
  LinLaunch F = L.fwd;  // shapes, segment plan, workspace; pointers set per pass
  F.bf16 = false;
  F.ccq = false;
  F.state_in = nullptr;
  F.state_out = nullptr;
  F.t_in = 0;
  // dq = forward(q = do, k = v, v = k, g)
  F.q = dout;
  F.k = v;
  F.v = k;
  F.g = L.g;
  F.out = dq;
  if ((e = linattn_launch(F, st)) != hipSuccess) return e;
  // reversed inputs and shifted gates
  if ((e = reverse(q, L.rq, L, st)) != hipSuccess) return e;
  if (!h && (e = reverse(k, L.rk, L, st)) != hipSuccess) return e;
  if ((e = reverse(v, L.rv, L, st)) != hipSuccess) return e;
  if ((e = reverse(dout, L.rdo, L, st)) != hipSuccess) return e;
  const int64_t tot = L.B * L.H * L.N;
  hipLaunchKernelGGL(shift_gates, dim3((unsigned)((tot + 255) / 256)), dim3(256), 0, st, L.g, L.rg, L.N, tot);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // dk (reversed) = forward(q = rev v, k = rev do, v = rev q, shifted gates)
  F.q = L.rv;
  F.k = L.rdo;
  F.v = L.rq;
  F.g = L.rg;
  F.out = L.rout;
  if ((e = linattn_launch(F, st)) != hipSuccess) return e;
  if ((e = reverse(L.rout, dk, L, st)) != hipSuccess) return e;
  // dv (reversed) = forward(q = rev k, k = rev q, v = rev do, shifted gates)
  if (h) {
    F.bf16 = true;
    F.q = h->rk;
    F.k = h->rq;
    F.v = h->rdo;
    F.out = h->rout;
    if ((e = linattn_launch(F, st)) != hipSuccess) return e;
    if ((e = reverse(h->rout, h->dv, L, st, 2)) != hipSuccess) return e;
  } else {
    F.q = L.rk;
    F.k = L.rq;
    F.v = L.rdo;
    F.out = L.rout;
    if ((e = linattn_launch(F, st)) != hipSuccess) return e;
    if ((e = reverse(L.rout, dv, L, st)) != hipSuccess) return e;
  }
  return gates ? gate_grad_f32(L, q, dq, k, dk, st, h ? h->dq16 : nullptr, h ? h->dk16 : nullptr) : hipSuccess;
}

}  // namespace bwd

hipError_t linattn_backward_f32(const BwdLaunch& L, const float* q, const float* k, const float* v,
                                const float* dout, float* dq, float* dk, float* dv, bool gates, hipStream_t st) {
  return bwd::backward(L, q, k, v, dout, dq, dk, dv, gates, nullptr, st);
}

hipError_t linattn_backward_mixed(const BwdLaunch& L, const float* q, const float* k, const float* v,
                                  const float* dout, float* dq, float* dk, bool gates, const bf16* rk16,
                                  const bf16* rq16, const bf16* rdo16, bf16* rout16, bf16* dv16, hipStream_t st) {
  const bwd::DvBf16 h{rk16, rq16, rdo16, rout16, dv16, nullptr, nullptr};
  return bwd::backward(L, q, k, v, dout, dq, dk, nullptr, gates, &h, st);
}

namespace bwd {
// float32 rows to reversed bf16 rows, four entries per thread (D a multiple of 4).
__global__ __launch_bounds__(256) void reverse_to_bf16_kernel(const float* __restrict__ in, bf16* __restrict__ out,
                                                              int64_t N, int D4, int64_t total4) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= total4) return;
  const int64_t row = i / D4;  // bh * N + t
  const int c = (int)(i - row * D4);
  const int64_t bh = row / N, t = row - bh * N;
  const f32x4 v = *reinterpret_cast<const f32x4*>(in + ((bh * N + (N - 1 - t)) * D4 + c) * 4);
  *reinterpret_cast<bf16x4*>(out + i * 4) = bf16x4{(bf16)v[0], (bf16)v[1], (bf16)v[2], (bf16)v[3]};
}
}  // namespace bwd

template <typename TI>
hipError_t reverse_to_bf16(const TI* in, bf16* out, int64_t BH, int64_t N, int64_t D, hipStream_t st) {
  if constexpr (sizeof(TI) == 2) {
    // a plain reversal: 16-byte pieces of the rows
    const int row_bytes = (int)(D * 2);
    const int64_t total16 = BH * N * (row_bytes / 16);
    hipLaunchKernelGGL(bwd::reverse_time, dim3((unsigned)((total16 + 255) / 256)), dim3(256), 0, st,
                       reinterpret_cast<const char*>(in), reinterpret_cast<char*>(out), N, row_bytes, total16);
  } else {
    const int64_t total4 = BH * N * (D / 4);
    hipLaunchKernelGGL(bwd::reverse_to_bf16_kernel, dim3((unsigned)((total4 + 255) / 256)), dim3(256), 0, st, in, out,
                       N, (int)(D / 4), total4);
  }
  return hipGetLastError();
}
template hipError_t reverse_to_bf16<float>(const float*, bf16*, int64_t, int64_t, int64_t, hipStream_t);
template hipError_t reverse_to_bf16<bf16>(const bf16*, bf16*, int64_t, int64_t, int64_t, hipStream_t);

hipError_t reverse_rows_f32(const float* in, float* out, int64_t BH, int64_t N, int64_t D, hipStream_t st) {
  const int row_bytes = (int)(D * 4);
  const int64_t total16 = BH * N * (row_bytes / 16);
  hipLaunchKernelGGL(bwd::reverse_time, dim3((unsigned)((total16 + 255) / 256)), dim3(256), 0, st,
                     reinterpret_cast<const char*>(in), reinterpret_cast<char*>(out), N, row_bytes, total16);
  return hipGetLastError();
}

hipError_t linattn_backward_launch(const BwdLaunch& L, hipStream_t st) {
  using namespace bwd;
  if (!L.bf16)
    return linattn_backward_f32(L, (const float*)L.q, (const float*)L.k, (const float*)L.v, (const float*)L.dout,
                                (float*)L.dq, (float*)L.dk, (float*)L.dv, true, st);
  const int64_t n = L.B * L.H * L.N * L.D;
  hipError_t e;
  if ((e = convert_n<bf16, float>(L.q, L.uq, n, st)) != hipSuccess) return e;
  if ((e = convert_n<bf16, float>(L.k, L.uk, n, st)) != hipSuccess) return e;
  if ((e = convert_n<bf16, float>(L.v, L.uv, n, st)) != hipSuccess) return e;
  if ((e = convert_n<bf16, float>(L.dout, L.udo, n, st)) != hipSuccess) return e;
  // the dv pass on bf16 operands: the reversed bf16 k and q share the float32
  // slot that would hold the reversed float32 k, the reversed bf16 dout and its
  // output share the slot of the float32 dv (neither is used on this path)
  bf16* rk16 = reinterpret_cast<bf16*>(L.rk);
  bf16* rdo16 = reinterpret_cast<bf16*>(L.udv);
  const DvBf16 h{rk16, rk16 + n, rdo16, rdo16 + n, static_cast<bf16*>(L.dv), static_cast<bf16*>(L.dq),
                 static_cast<bf16*>(L.dk)};
  if ((e = reverse(L.k, rk16, L, st, 2)) != hipSuccess) return e;
  if ((e = reverse(L.q, rk16 + n, L, st, 2)) != hipSuccess) return e;
  if ((e = reverse(L.dout, rdo16, L, st, 2)) != hipSuccess) return e;
  // dq, dk in bf16 come from the gate-gradient pass
  return backward(L, L.uq, L.uk, L.uv, L.udo, L.udq, L.udk, nullptr, true, &h, st);
}

}  // namespace lm
