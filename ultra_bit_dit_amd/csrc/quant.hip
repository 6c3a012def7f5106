// Data-free quantizer front end: bf16 weights -> binary / ternary codes and
// one fp16 scale per 128-weight group, with an optional signed Hadamard
// rotation of each group (the rotation and the per-128 FP16 scale of the
// method list of the paragraph "工作原理" of the page "我开源了 OpenBonsai：
// 把你自己的 BF16 模型与微调压缩成约 2 GB 的三值 GGUF"; its
// calibrated GPTQ step needs data and is not part of this front end), and
// the matching rotation of activations.
//
// Per row n and group g (eight lanes, see the kernel):
//   v = W[n][128 g ..] * d[128 g ..]            (signs d = +-1)
//   u = H v, H[i][j] = (-1)^popcount(i & j)      (fast Walsh-Hadamard, fp64)
//   t = u r with r = 1/sqrt(128) in fp64; s = (sum |u| / 128) r (mean |t|);
//   s16 = fp16(s), round to nearest even
//   ternary: c = +1 if t > s16/2, -1 if t < -s16/2, else 0 (t / s16 rounded,
//   ties to even, clamped to [-1, 1], by exact comparison); binary: sign(t)
//   (s16 = 0: codes 0 / +1).  Without signs: u = t = v, s = mean |v|.
// The weights are bf16 (8 significant bits), so every partial sum of the
// transform and of sum |u| is exact in fp64 whenever a group's magnitudes
// span less than 2^38: the result does not depend on the summation order,
// and the rounding decisions are taken in fp64.
#include <hip/hip_runtime.h>

#include "common.hpp"

namespace lowbit {
namespace {

// fp64 -> binary16 bits, round to nearest even, from the bit pattern
__device__ __forceinline__ uint16_t f64_to_f16_bits(double x) {
  const uint64_t b = (uint64_t)__double_as_longlong(x);
  const uint16_t sign = (uint16_t)((b >> 48) & 0x8000u);
  const uint64_t a = b & 0x7FFFFFFFFFFFFFFFull;
  if (a > 0x7FF0000000000000ull) return 0x7E00;      // NaN
  if (a >= 0x40EFFE0000000000ull) return sign | 0x7C00;  // >= 65520: rounds to infinity
  int e = (int)(a >> 52) - 1023;
  if (e < -14) {
    // subnormal half (or zero): an integer multiple of 2^-24, exact scaling
    const double q = __longlong_as_double((long long)a) * 16777216.0;
    return sign | (uint16_t)__builtin_rint(q);  // 1024 becomes the smallest normal
  }
  const uint64_t mant = (a & 0x000FFFFFFFFFFFFFull) | 0x0010000000000000ull;
  uint64_t q = mant >> 42;
  const uint64_t rem = mant & 0x3FFFFFFFFFFull, half = 0x20000000000ull;
  if (rem > half || (rem == half && (q & 1))) q++;
  if (q == 2048) {
    q = 1024;
    e++;
  }
  return sign | (uint16_t)((e + 15) << 10) | (uint16_t)(q & 0x3FF);
}

__device__ __forceinline__ double f16_bits_f64(uint16_t h) {
  return (double)f16_bits_to_f32(h);
}

__device__ __forceinline__ double shfl_xor_f64(double v, int d) {
  const long long b = __double_as_longlong(v);
  const int lo = __shfl_xor((int)(b & 0xFFFFFFFF), d, 64);
  const int hi = __shfl_xor((int)(b >> 32), d, 64);
  return __longlong_as_double(((long long)hi << 32) | (unsigned)lo);
}

// Eight lanes per (row, group): lane l8 = lane % 8 of the eight holds the
// 16 consecutive elements 16 l8 .. 16 l8 + 15, so the transform's strides
// 1..8 are butterflies inside the lane and strides 16, 32, 64 exchange
// with lanes l8 ^ 1, 2, 4; a wavefront covers eight groups.  Loads are 32
// bytes and code stores 16 bytes per lane.
constexpr int kQuantGroupsPerWave = 8;

__global__ __launch_bounds__(256) void quantize_weights(int fmt, int64_t N, int64_t K, int64_t G,
                                                        const uint16_t* __restrict__ W,
                                                        const int8_t* __restrict__ signs,
                                                        int8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scales) {
  const int lane = threadIdx.x & 63, l8 = lane & 7;
  const int64_t unit = ((int64_t)blockIdx.x * 4 + (threadIdx.x >> 6)) * kQuantGroupsPerWave + (lane >> 3);
  const bool valid = unit < N * G;
  const int64_t uc = valid ? unit : N * G - 1;  // lanes past the end recompute the last group
  const int64_t n = uc / G, g = uc % G;
  const int64_t base = n * K + g * 128 + 16 * l8;
  const uint4 w0 = *(const uint4*)(W + base), w1 = *(const uint4*)(W + base + 8);
  const uint32_t wb[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
  double v[16];
#pragma unroll
  for (int i = 0; i < 8; i++) {
    v[2 * i] = (double)__uint_as_float(wb[i] << 16);
    v[2 * i + 1] = (double)__uint_as_float(wb[i] & 0xFFFF0000u);
  }
  const bool rot = signs != nullptr;
  const double r = 1.0 / __builtin_sqrt(128.0);  // folded to the fp64 constant
  if (rot) {
    const uint4 sg = *(const uint4*)(signs + g * 128 + 16 * l8);
    const uint32_t sw[4] = {sg.x, sg.y, sg.z, sg.w};
#pragma unroll
    for (int i = 0; i < 16; i++) v[i] *= (double)(int8_t)((sw[i >> 2] >> (8 * (i & 3))) & 0xFF);
    // strides 1, 2, 4, 8: inside the lane (bits 0..3 of the element index)
#pragma unroll
    for (int d = 1; d < 16; d <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        if (i & d) continue;
        const double a = v[i], b = v[i + d];
        v[i] = a + b;
        v[i + d] = a - b;
      }
    }
    // strides 16, 32, 64: lanes l8 ^ 1, 2, 4 (bits 4..6)
#pragma unroll
    for (int d = 1; d < 8; d <<= 1) {
#pragma unroll
      for (int i = 0; i < 16; i++) {
        const double p = shfl_xor_f64(v[i], d);
        v[i] = (l8 & d) ? p - v[i] : v[i] + p;
      }
    }
  }
  double S = 0.0;
#pragma unroll
  for (int i = 0; i < 16; i++) S += __builtin_fabs(v[i]);
#pragma unroll
  for (int d = 1; d < 8; d <<= 1) S += shfl_xor_f64(S, d);
  const double sc = rot ? (S / 128.0) * r : S / 128.0;
  const uint16_t s16 = f64_to_f16_bits(sc);
  const double sd = f16_bits_f64(s16), h = sd * 0.5;
  uint32_t cw[4] = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int i = 0; i < 16; i++) {
    const double t = rot ? v[i] * r : v[i];
    int8_t c;
    if (fmt == 1) c = (sd == 0.0 || !(t < 0.0)) ? 1 : -1;
    else if (sd == 0.0) c = 0;
    else c = t > h ? 1 : (t < -h ? -1 : 0);
    cw[i >> 2] |= (uint32_t)(uint8_t)c << (8 * (i & 3));
  }
  if (valid) {
    *(uint4*)(codes + base) = make_uint4(cw[0], cw[1], cw[2], cw[3]);
    if (l8 == 0) scales[n * G + g] = s16;
  }
}

// Activations rotated to match rotated weights: per 128-block,
// Xr = H (d * x) / sqrt(128) in fp32, so that sum_k Wr[n][k] Xr[m][k] equals
// sum_k W[n][k] X[m][k] (H d / sqrt(128) is orthogonal and symmetric up to d).
__global__ __launch_bounds__(256) void rotate_act(int64_t M, int64_t K, int64_t G,
                                                  const uint16_t* __restrict__ X,
                                                  const int8_t* __restrict__ signs,
                                                  float* __restrict__ Xr) {
  const int lane = threadIdx.x & 63;
  const int64_t unit = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
  if (unit >= M * G) return;
  const int64_t m = unit / G, g = unit % G;
  const int64_t base = m * K + g * 128;
  float v0 = __uint_as_float((uint32_t)X[base + lane] << 16) * (float)signs[g * 128 + lane];
  float v1 = __uint_as_float((uint32_t)X[base + lane + 64] << 16) * (float)signs[g * 128 + lane + 64];
  const float a = v0 + v1, b = v0 - v1;
  v0 = a;
  v1 = b;
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    const float p0 = __shfl_xor(v0, d, 64), p1 = __shfl_xor(v1, d, 64);
    v0 = (lane & d) ? p0 - v0 : v0 + p0;
    v1 = (lane & d) ? p1 - v1 : v1 + p1;
  }
  const float inv = 0.08838834764831845f;  // 1 / sqrt(128) rounded to fp32
  Xr[base + lane] = v0 * inv;
  Xr[base + lane + 64] = v1 * inv;
}

}  // namespace

hipError_t launch_quantize_weights(int fmt, int64_t N, int64_t K, const uint16_t* W,
                                   const int8_t* signs, int8_t* codes, uint16_t* scales,
                                   hipStream_t s) {
  const int64_t G = K / kGroup, units = N * G;
  hipLaunchKernelGGL(quantize_weights, dim3((unsigned)cdiv(units, 4 * kQuantGroupsPerWave)), dim3(256),
                     0, s, fmt, N, K, G, W, signs, codes, scales);
  return hipGetLastError();
}

hipError_t launch_rotate_act(int64_t M, int64_t K, const uint16_t* X, const int8_t* signs,
                             float* Xr, hipStream_t s) {
  const int64_t G = K / kGroup, units = M * G;
  hipLaunchKernelGGL(rotate_act, dim3((unsigned)cdiv(units, 4)), dim3(256), 0, s, M, K, G, X,
                     signs, Xr);
  return hipGetLastError();
}

}  // namespace lowbit
