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

// The same with 16-byte loads of 8 values and 8-byte stores of their codes
// (K % 8 == 0, X 16-byte and Q 8-byte aligned): the identical per-element
// arithmetic, the row's second pass re-reading it from the cache.
__device__ __forceinline__ float absmax8(const uint4 w) {
  const uint32_t u[4] = {w.x, w.y, w.z, w.w};
  float a = 0.0f;
#pragma unroll
  for (int j = 0; j < 4; j++) {
    a = fmaxf(a, fabsf(__uint_as_float(u[j] << 16)));
    a = fmaxf(a, fabsf(__uint_as_float(u[j] & 0xFFFF0000u)));
  }
  return a;
}

__global__ __launch_bounds__(256) void quantize_i8_v8(int64_t K, const uint16_t* __restrict__ X,
                                                      int8_t* __restrict__ Q,
                                                      float* __restrict__ sx) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x, K8 = K / 8;
  const uint4* row = (const uint4*)(X + m * K);
  uint2* qrow = (uint2*)(Q + m * K);
  float a = 0.0f;
  for (int64_t i = threadIdx.x; i < K8; i += blockDim.x) a = fmaxf(a, absmax8(row[i]));
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  if (a == 0.0f) {
    for (int64_t i = threadIdx.x; i < K8; i += blockDim.x) qrow[i] = make_uint2(0u, 0u);
    if (threadIdx.x == 0) sx[m] = 0.0f;
    return;
  }
  const float inv = 127.0f / a;  // correctly rounded division
  for (int64_t i = threadIdx.x; i < K8; i += blockDim.x) {
    const uint4 w = row[i];
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
    uint32_t q[2] = {0u, 0u};
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t bits = (j & 1) ? (u[j >> 1] & 0xFFFF0000u) : (u[j >> 1] << 16);
      float r = rintf(__fmul_rn(__uint_as_float(bits), inv));
      r = fminf(fmaxf(r, -127.0f), 127.0f);
      q[j >> 2] |= (uint32_t)(uint8_t)(int8_t)(int)r << (8 * (j & 3));
    }
    qrow[i] = make_uint2(q[0], q[1]);
  }
  if (threadIdx.x == 0) sx[m] = a / 127.0f;
}

}  // namespace

hipError_t launch_quantize_i8(int64_t M, int64_t K, const uint16_t* X, int8_t* Q, float* sx,
                              hipStream_t s) {
  if (K % 8 == 0 && ((uintptr_t)X & 15) == 0 && ((uintptr_t)Q & 7) == 0)
    hipLaunchKernelGGL(quantize_i8_v8, dim3((unsigned)M), dim3(256), 0, s, K, X, Q, sx);
  else
    hipLaunchKernelGGL(quantize_i8, dim3((unsigned)M), dim3(256), 0, s, K, X, Q, sx);
  return hipGetLastError();
}

}  // namespace lowbit
