// bwd.hpp -- internal interface of the linear-attention backward for the
// other backward passes (GMA, CCQ) that run it on float32 tensors of their own.
#pragma once
#include "launch.hpp"
#include "mfma.hpp"

namespace lm {

// The backward of decayed linear attention on float32 q, k, v, dout (dq, dk in
// float32, dg when gates) with the dv pass on bf16 operands: rk16, rq16, rdo16
// are the time-reversed k, q, dout rounded to bf16 (rows of L.D entries),
// rout16 a buffer of the same size, and dv16 receives dv in bf16. L.rk is not
// used.
hipError_t linattn_backward_mixed(const BwdLaunch& L, const float* q, const float* k, const float* v,
                                  const float* dout, float* dq, float* dk, bool gates, const bf16* rk16,
                                  const bf16* rq16, const bf16* rdo16, bf16* rout16, bf16* dv16, hipStream_t st);

// out[bh][t][:] = in[bh][N - 1 - t][:] rounded to bf16 (D entries per row).
template <typename TI>
hipError_t reverse_to_bf16(const TI* in, bf16* out, int64_t BH, int64_t N, int64_t D, hipStream_t st);

}  // namespace lm
