// Activation preparation that runs as its own launch: per-row absmax int8
// quantization.  (fp8 split staging for the MFMA path and the sign-bit
// reordering of the XOR + popcount path run inside the GEMV launch, see
// gemv.hip.)
#include "common.hpp"

namespace lowbit {
namespace {

// per-row absmax int8 quantization, one block per row
__global__ void quantize_i8(int64_t K, const uint16_t* __restrict__ X, int8_t* __restrict__ Q,
                            float* __restrict__ sx) {
  __shared__ float red[16];
  int64_t m = blockIdx.x;
  const uint16_t* row = X + m * K;
  float a = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += blockDim.x)
    a = fmaxf(a, fabsf(__uint_as_float((uint32_t)row[k] << 16)));
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = 0.0f;
  for (int w = 0; w < (int)(blockDim.x >> 6); w++) a = fmaxf(a, red[w]);
  if (a == 0.0f) {
    for (int64_t k = threadIdx.x; k < K; k += blockDim.x) Q[m * K + k] = 0;
    if (threadIdx.x == 0) sx[m] = 0.0f;
    return;
  }
  float inv = 127.0f / a;  // correctly rounded division
  for (int64_t k = threadIdx.x; k < K; k += blockDim.x) {
    float p = __fmul_rn(__uint_as_float((uint32_t)row[k] << 16), inv);
    float r = rintf(p);
    r = fminf(fmaxf(r, -127.0f), 127.0f);
    Q[m * K + k] = (int8_t)(int)r;
  }
  if (threadIdx.x == 0) sx[m] = a / 127.0f;
}

}  // namespace

hipError_t launch_quantize_i8(int64_t M, int64_t K, const uint16_t* X, int8_t* Q, float* sx,
                              hipStream_t s) {
  hipLaunchKernelGGL(quantize_i8, dim3((unsigned)M), dim3(256), 0, s, K, X, Q, sx);
  return hipGetLastError();
}

}  // namespace lowbit
