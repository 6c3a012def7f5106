// Activation staging and int8 quantization.
//
// fp8 split staging (GEMV operand A).  The MFMA GEMV multiplies fp4 weights
// (exactly +-1 / 0) by activations given as fp8 e4m3 "split terms": for
// each 32-element block of an activation row, E is chosen so the block
// maximum scaled by 2^-E lies in [128, 256); term 0 is rne_e4m3(v), and each
// next term is rne_e4m3 of 16 x the remaining residual.  Term r carries the
// E8M0 block exponent E - 4r, applied inside the scaled MFMA.  Two terms
// reproduce a bf16 value exactly (8 significant bits) for elements within
// 2^13 of the block maximum; smaller elements keep an error below
// 2^-21 x the block maximum.  Four terms give fp32 inputs 16 significant bits.
// int8 values q are split exactly as 16 * (q >> 4) + (q & 15).
//
// Layouts written here (M activation rows, R terms, MA = M * R "A rows"):
//   xa[((g * 4 + kb) * MA + a) * 32 + e]   fp8 A bytes of lane group kb; the
//       byte holds activation k = 128 g + 32 kb + e (this pairs it with the
//       packed weight of the same k)
//   xe byte [((g/4 * 4 + b) * MA + a) * 4 + g % 4]   E8M0 exponent of
//       hardware block b (supplied by lane group b)
#include "common.hpp"

namespace lowbit {
namespace {

// fp32 -> fp8 e4m3 (OCP "fn": bias 7, max 448), round to nearest even.
// Callers guarantee |v| < 256.
__device__ inline uint32_t e4m3_rne(float v) {
  uint32_t s = (__float_as_uint(v) >> 24) & 0x80;
  float a = fabsf(v);
  if (a < 0.015625f) {  // below 2^-6: subnormal grid of 2^-9 (8 -> 2^-6)
    return s | (uint32_t)rintf(a * 512.0f);
  }
  int ex;
  float f = frexpf(a, &ex);  // a = f * 2^ex, f in [0.5, 1)
  int e = ex - 1;
  int m = (int)rintf((2.0f * f - 1.0f) * 8.0f);
  if (m == 8) {
    m = 0;
    e += 1;
  }
  return s | ((uint32_t)(e + 7) << 3) | (uint32_t)m;
}

__device__ inline float e4m3_dec(uint32_t c) {
  int e = (c >> 3) & 15, m = c & 7;
  float v = e == 0 ? ldexpf((float)m, -9) : ldexpf(1.0f + m * 0.125f, e - 7);
  return (c & 0x80) ? -v : v;
}

__device__ inline float load_x(int xkind, const void* X, int64_t idx) {
  if (xkind == XK_F32) return ((const float*)X)[idx];
  if (xkind == XK_BF16) return __uint_as_float((uint32_t)((const uint16_t*)X)[idx] << 16);
  return (float)((const int8_t*)X)[idx];
}

// One thread per (row m, group g, hardware block b).  The 16x16x128 f8f6f4
// MFMA reduces over hardware positions h = 0..127; its E8M0 scale of lane
// (row, b) multiplies block h in [32b, 32b+32).  Position h = 32b + i pairs
// with fp4 weight slot i of quarter b, i.e. activation k = 128g + kmap(b, i),
// and is fed by A byte e = 16(b>>1) + (i&15) of lane group kb = 2(b&1) +
// (i>>4).  The block exponent is therefore taken over those 32 activations.
__global__ void stage_fp8(int xkind, int64_t M, int64_t K, int64_t G, const void* __restrict__ X,
                          int R, uint8_t* __restrict__ xa, uint8_t* __restrict__ xe_bytes) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= M * G * 4) return;
  int b = tid & 3;
  int64_t g = (tid >> 2) % G, m = (tid >> 2) / G;
  int64_t MA = M * R;
  float v[32];
  float amax = 0.0f;
  for (int i = 0; i < 32; i++) {
    v[i] = load_x(xkind, X, m * K + g * kGroup + kmap(b, i));
    amax = fmaxf(amax, fabsf(v[i]));
  }
  int E;
  if (xkind == XK_I8) {
    E = 0;
  } else if (amax == 0.0f) {
    E = 0;
  } else {
    int ex;
    frexpf(amax, &ex);
    E = (ex - 1) - 7;  // amax * 2^-E in [128, 256)
    int lo = -127 + kSplitShift * (R - 1);
    if (E < lo) E = lo;
  }
  int64_t gq = g >> 2;
  for (int r = 0; r < R; r++) {
    int64_t arow = m * R + r;
    uint32_t words[8];
    for (int w = 0; w < 8; w++) words[w] = 0;
    int Er;
    if (xkind == XK_I8) {
      // exact split q = 16 * (q >> 4) + (q & 15); term 0 carries 2^4
      for (int i = 0; i < 32; i++) {
        int q = (int)v[i];
        int part = r == 0 ? (q >> 4) : (q & 15);
        words[i >> 2] |= e4m3_rne((float)part) << (8 * (i & 3));
      }
      Er = r == 0 ? 4 : 0;
    } else {
      for (int i = 0; i < 32; i++) {
        float t = ldexpf(v[i], -E);
        uint32_t c = 0;
        for (int j = 0; j <= r; j++) {  // walk the residual chain to term r
          c = e4m3_rne(t);
          t = (t - e4m3_dec(c)) * 16.0f;
        }
        words[i >> 2] |= c << (8 * (i & 3));
      }
      Er = E - kSplitShift * r;
    }
    // elements 0..15 -> lane group 2(b&1), bytes 16(b>>1)..; 16..31 -> the next lane group
    const int kb0 = 2 * (b & 1), e0 = 16 * (b >> 1);
    uint4* d0 = (uint4*)(xa + (((g * 4 + kb0) * MA + arow) * 32) + e0);
    uint4* d1 = (uint4*)(xa + (((g * 4 + kb0 + 1) * MA + arow) * 32) + e0);
    *d0 = make_uint4(words[0], words[1], words[2], words[3]);
    *d1 = make_uint4(words[4], words[5], words[6], words[7]);
    xe_bytes[(((gq * 4 + b) * MA + arow) * 4) + (g & 3)] = (uint8_t)(127 + Er);
  }
}

// sign bits -> binary word order; xw[((m * GQ + gq) * 4 + q) * 4 + g % 4]
__global__ void stage_sign(int64_t M, int64_t K, int64_t G, int64_t GQ,
                           const uint8_t* __restrict__ xbits, uint32_t* __restrict__ xw) {
  int64_t tid = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (tid >= M * GQ * 16) return;
  int t = tid & 3, q = (tid >> 2) & 3;
  int64_t gq = (tid >> 4) % GQ, m = (tid >> 4) / GQ;
  int64_t g = 4 * gq + t;
  uint32_t w = 0;
  if (g < G) {
    const uint8_t* row = xbits + m * (K / 8);
    for (int b = 0; b < 32; b++) {
      int64_t k = g * kGroup + kmap(q, bin_slot(b));
      w |= (uint32_t)((row[k >> 3] >> (k & 7)) & 1) << b;
    }
  }
  xw[tid] = w;
}

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

hipError_t launch_stage_fp8(int xkind, int64_t M, int64_t K, const void* X, int R, uint8_t* xa,
                            uint32_t* xe, hipStream_t s) {
  int64_t G = K / kGroup, n = M * G * 4;
  hipLaunchKernelGGL(stage_fp8, dim3((unsigned)cdiv(n, 128)), dim3(128), 0, s, xkind, M, K, G, X,
                     R, xa, (uint8_t*)xe);
  return hipGetLastError();
}

hipError_t launch_stage_sign(int64_t M, int64_t K, const uint8_t* xbits, uint32_t* xw,
                             hipStream_t s) {
  int64_t G = K / kGroup, GQ = cdiv(G, 4), n = M * GQ * 16;
  hipLaunchKernelGGL(stage_sign, dim3((unsigned)cdiv(n, 256)), dim3(256), 0, s, M, K, G, GQ,
                     xbits, xw);
  return hipGetLastError();
}

hipError_t launch_quantize_i8(int64_t M, int64_t K, const uint16_t* X, int8_t* Q, float* sx,
                              hipStream_t s) {
  hipLaunchKernelGGL(quantize_i8, dim3((unsigned)M), dim3(256), 0, s, K, X, Q, sx);
  return hipGetLastError();
}

}  // namespace lowbit
