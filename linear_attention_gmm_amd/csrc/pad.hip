// pad.hip -- zero padding of the feature axis, for the shapes that run on the
// kernels of a wider feature width (a width of 16, or d != dv): rows of width
// sw copied into rows of width dw >= sw with the new columns set to a fill
// value, and the inverse (the first dw of sw columns of every row).
//
// Padding is exact for the mixers here: a routing feature with x = mu = 0 and
// log variance 0 adds the same constant to every component's log joint (it
// cancels in the softmax), a zero key or query feature adds nothing to any
// product, key covariance or norm, a decay of 1 on a feature whose keys are
// zero leaves it zero, and a zero value column yields an output column that is
// dropped.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "launch.hpp"

namespace lm {
namespace pad {

template <typename T>
__global__ __launch_bounds__(256) void pad_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows, int sw,
                                                  int dw, float fill) {
  const int64_t n = rows * dw;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / dw;
    const int c = (int)(i - r * dw);
    dst[i] = c < sw ? src[r * sw + c] : (T)fill;
  }
}

template <typename T>
__global__ __launch_bounds__(256) void crop_kernel(const T* __restrict__ src, T* __restrict__ dst, int64_t rows, int sw,
                                                   int dw) {
  const int64_t n = rows * dw;
  for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256) {
    const int64_t r = i / dw;
    const int c = (int)(i - r * dw);
    dst[i] = src[r * sw + c];
  }
}

inline unsigned blocks(int64_t n) {
  const int64_t b = (n + 255) / 256;
  return (unsigned)(b < 8192 ? (b > 0 ? b : 1) : 8192);
}

}  // namespace pad

hipError_t pad_cols(const void* src, void* dst, int64_t rows, int sw, int dw, float fill, int esize, hipStream_t st) {
  const unsigned nb = pad::blocks(rows * dw);
  if (esize == 2)
    hipLaunchKernelGGL(pad::pad_kernel<__bf16>, dim3(nb), dim3(256), 0, st, static_cast<const __bf16*>(src),
                       static_cast<__bf16*>(dst), rows, sw, dw, fill);
  else
    hipLaunchKernelGGL(pad::pad_kernel<float>, dim3(nb), dim3(256), 0, st, static_cast<const float*>(src),
                       static_cast<float*>(dst), rows, sw, dw, fill);
  return hipGetLastError();
}

hipError_t crop_cols(const void* src, void* dst, int64_t rows, int sw, int dw, int esize, hipStream_t st) {
  const unsigned nb = pad::blocks(rows * dw);
  if (esize == 2)
    hipLaunchKernelGGL(pad::crop_kernel<__bf16>, dim3(nb), dim3(256), 0, st, static_cast<const __bf16*>(src),
                       static_cast<__bf16*>(dst), rows, sw, dw);
  else
    hipLaunchKernelGGL(pad::crop_kernel<float>, dim3(nb), dim3(256), 0, st, static_cast<const float*>(src),
                       static_cast<float*>(dst), rows, sw, dw);
  return hipGetLastError();
}

}  // namespace lm
