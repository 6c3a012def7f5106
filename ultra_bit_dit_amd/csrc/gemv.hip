// Batch-1 (and small-M) products over packed binary / ternary weights.
//
// MFMA path.  A row-block of 16 output rows is one workgroup of S waves; the
// waves split the reduction range in whole 4-group quads and combine their
// partial sums in LDS in a fixed order.  Per group, each lane turns its 32
// packed weights into fp4 (e2m1) values +1 / -1 / 0 with 1-2 VALU ops per 8
// weights and feeds them as operand B of v_mfma_scale_f32_16x16x128_f8f6f4;
// operand A holds the staged fp8 split terms of the activations (rows of A
// beyond the staged terms are zero).  The MFMA output for the group is a
// partial dot product that the lane multiplies by the fp32 group scale and
// adds to its accumulator: the scale is applied once per group, never folded
// into a low-precision weight.
//
// Per 16 rows x 128 weights a wave issues one 16-byte vector load of codes
// (per 4 groups), one MFMA and ~10 VALU ops; the kernel is bound by HBM
// bandwidth.  Multiplications by -1 / 0 / +1 are exact in the MFMA (ternary
// products reduce to adds and sign flips: "精度保留了多少" section of the
// kongchang.com Ternary Bonsai 2 article).
//
// Sign path (binary weights x sign activations): per 32 weights one XOR and
// one popcount give the exact signed agreement 32 - 2 * popcount(w ^ x)
// (the XOR + popcount remark of the "1-bit 嘅數學" section of the
// richmindsetzone.com 1-bit diffusion page).
#include "common.hpp"

namespace lowbit {
namespace {

constexpr int kMaxWaves = 16;

template <int T>
__device__ inline v4f mfma_group(const v8i& A, const v8i& B, int sa) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // A: fp8 e4m3 (0), B: fp4 e2m1 (4); byte T of sa is the A block exponent,
  // B is unscaled (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, 0, 4, T, sa, 0, 127);
}

__device__ inline uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

struct KArgs {
  const void* pcodes;
  const uint16_t* pscales;
  const uint8_t* xa;
  const uint32_t* xe;
  const float* x_scales;
  void* y;
  int64_t N, G, GQ, GP, M, MA;
  float x_scale;
};

// FMT 1 binary, 2 ternary 2-bit.  R split terms per activation row (2 or 4).
// INTC: terms recombine to an exact integer (int8 activations).
template <int FMT, int R, bool INTC, int YK>
__global__ __launch_bounds__(1024) void gemv_mfma(KArgs a) {
  constexpr int NX = 4 / R;  // activation rows per lane group
  __shared__ float red_f[kMaxWaves][64][NX];
  __shared__ int red_i[kMaxWaves][64][NX];

  const int L = threadIdx.x & 63;
  const int w = threadIdx.x >> 6;
  const int S = blockDim.x >> 6;
  const int r = L & 15, lg = L >> 4;
  const int64_t rb = blockIdx.x;
  const int64_t q0 = (a.GQ * w) / S, q1 = (a.GQ * (w + 1)) / S;
  const bool arow = r < a.MA;

  float acc[NX];
  int iacc[NX];
#pragma unroll
  for (int j = 0; j < NX; j++) {
    acc[j] = 0.f;
    iacc[j] = 0;
  }

  const uint4* pc4 = (const uint4*)a.pcodes;
  const uint2* ps2 = (const uint2*)a.pscales;
  const uint4* xa4 = (const uint4*)a.xa;

  for (int64_t gq = q0; gq < q1; gq++) {
    // ---- loads for 4 groups
    uint4 cw0, cw1;
    if (FMT == 1) {
      cw0 = pc4[(rb * a.GQ + gq) * 64 + L];
      cw1 = make_uint4(0, 0, 0, 0);
    } else {
      cw0 = pc4[(rb * a.GP + 2 * gq) * 64 + L];
      cw1 = (2 * gq + 1 < a.GP) ? pc4[(rb * a.GP + 2 * gq + 1) * 64 + L] : make_uint4(0, 0, 0, 0);
    }
    uint2 sc = a.pscales ? ps2[(rb * a.GQ + gq) * 16 + r] : make_uint2(0x3C003C00u, 0x3C003C00u);
    uint4 av[8];
    uint32_t se = 127u * 0x01010101u;
    if (arow) {
#pragma unroll
      for (int t = 0; t < 4; t++) {
        int64_t base = ((4 * gq + t) * 4 + lg) * a.MA + r;
        av[2 * t] = xa4[base * 2];
        av[2 * t + 1] = xa4[base * 2 + 1];
      }
      se = a.xe[(gq * 4 + lg) * a.MA + r];
    } else {
#pragma unroll
      for (int t = 0; t < 8; t++) av[t] = make_uint4(0, 0, 0, 0);
    }
    const int ng = (int)min<int64_t>(4, a.G - 4 * gq);

    // ---- 4 groups: decode, MFMA, scale epilogue
#define LOWBIT_GROUP(T)                                                                     \
  if (T < ng) {                                                                             \
    uint32_t d0, d1, d2, d3;                                                                \
    if (FMT == 1) {                                                                         \
      uint32_t wv = T == 0 ? cw0.x : T == 1 ? cw0.y : T == 2 ? cw0.z : cw0.w;               \
      d0 = (wv & 0x88888888u) | 0x22222222u;                                                \
      d1 = ((wv << 1) & 0x88888888u) | 0x22222222u;                                         \
      d2 = ((wv << 2) & 0x88888888u) | 0x22222222u;                                         \
      d3 = ((wv << 3) & 0x88888888u) | 0x22222222u;                                         \
    } else {                                                                                \
      uint32_t p0 = T == 0 ? cw0.x : T == 1 ? cw0.z : T == 2 ? cw1.x : cw1.z;               \
      uint32_t p1 = T == 0 ? cw0.y : T == 1 ? cw0.w : T == 2 ? cw1.y : cw1.w;               \
      d0 = p0 & 0xAAAAAAAAu;                                                                \
      d1 = (p0 << 1) & 0xAAAAAAAAu;                                                         \
      d2 = p1 & 0xAAAAAAAAu;                                                                \
      d3 = (p1 << 1) & 0xAAAAAAAAu;                                                         \
    }                                                                                       \
    v8i B = {(int)d0, (int)d1, (int)d2, (int)d3, 0, 0, 0, 0};                               \
    uint4 x0 = av[2 * T], x1 = av[2 * T + 1];                                               \
    v8i A = {(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,                                    \
             (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};                                   \
    v4f c = mfma_group<T>(A, B, (int)se);                                                   \
    uint32_t sh = (T < 2 ? sc.x : sc.y) >> (16 * (T & 1));                                  \
    float s = f16_bits_to_f32(sh);                       \
    _Pragma("unroll") for (int j = 0; j < NX; j++) {                                        \
      float t = c[R * j];                                                                   \
      _Pragma("unroll") for (int i = 1; i < R; i++) t += c[R * j + i];                      \
      acc[j] = fmaf(s, t, acc[j]);                                                          \
      if (INTC) iacc[j] += __float2int_rn(t);                                               \
    }                                                                                       \
  }
    LOWBIT_GROUP(0)
    LOWBIT_GROUP(1)
    LOWBIT_GROUP(2)
    LOWBIT_GROUP(3)
#undef LOWBIT_GROUP
  }

  // ---- split-K reduction over the waves, fixed order
#pragma unroll
  for (int j = 0; j < NX; j++) {
    red_f[w][L][j] = acc[j];
    red_i[w][L][j] = iacc[j];
  }
  __syncthreads();
  if (w != 0) return;
#pragma unroll
  for (int j = 0; j < NX; j++) {
    float f = red_f[0][L][j];
    int iv = red_i[0][L][j];
    for (int ww = 1; ww < S; ww++) {
      f += red_f[ww][L][j];
      iv += red_i[ww][L][j];
    }
    const int64_t m = (int64_t)lg * NX + j;  // activation row
    const int64_t n = rb * 16 + r;
    if (m < a.M && n < a.N) {
      float sxm = a.x_scales ? a.x_scales[m] : a.x_scale;
      if (YK == YK_F32) ((float*)a.y)[m * a.N + n] = f * sxm;
      else if (YK == YK_BF16) ((uint16_t*)a.y)[m * a.N + n] = (uint16_t)bf16_rne(f * sxm);
      else ((int32_t*)a.y)[m * a.N + n] = iv;
    }
  }
}

// ------------------------------------------------------------ sign path
struct SArgs {
  const void* pcodes;
  const uint16_t* pscales;
  const uint32_t* xw;
  void* y;
  int64_t N, G, GQ;
  float alpha;
};

template <int YK>
__global__ __launch_bounds__(1024) void gemv_sign(SArgs a) {
  __shared__ float red_f[kMaxWaves][64];
  __shared__ int red_i[kMaxWaves][64];
  const int L = threadIdx.x & 63, w = threadIdx.x >> 6, S = blockDim.x >> 6;
  const int r = L & 15, q = L >> 4;
  const int64_t rb = blockIdx.x;
  const int64_t q0 = (a.GQ * w) / S, q1 = (a.GQ * (w + 1)) / S;
  const uint4* pc4 = (const uint4*)a.pcodes;
  const uint2* ps2 = (const uint2*)a.pscales;
  const uint4* xw4 = (const uint4*)a.xw;
  float acc = 0.f;
  int iacc = 0;
  for (int64_t gq = q0; gq < q1; gq++) {
    uint4 cw = pc4[(rb * a.GQ + gq) * 64 + L];
    uint4 xv = xw4[gq * 4 + q];
    uint2 sc = a.pscales ? ps2[(rb * a.GQ + gq) * 16 + r] : make_uint2(0x3C003C00u, 0x3C003C00u);
    const int ng = (int)min<int64_t>(4, a.G - 4 * gq);
    uint32_t wv[4] = {cw.x, cw.y, cw.z, cw.w};
    uint32_t xx[4] = {xv.x, xv.y, xv.z, xv.w};
    uint32_t ss[4] = {sc.x & 0xFFFF, sc.x >> 16, sc.y & 0xFFFF, sc.y >> 16};
#pragma unroll
    for (int t = 0; t < 4; t++) {
      if (t < ng) {
        int d = 32 - 2 * __popc(wv[t] ^ xx[t]);
        iacc += d;
        acc = fmaf(f16_bits_to_f32(ss[t]), (float)d, acc);
      }
    }
  }
  red_f[w][L] = acc;
  red_i[w][L] = iacc;
  __syncthreads();
  if (w != 0 || q != 0) return;
  float f = 0.f;
  int iv = 0;
  for (int ww = 0; ww < S; ww++)
    for (int qq = 0; qq < 4; qq++) {
      f += red_f[ww][r + 16 * qq];
      iv += red_i[ww][r + 16 * qq];
    }
  const int64_t n = rb * 16 + r;
  if (n < a.N) {
    if (YK == YK_F32) ((float*)a.y)[n] = f * a.alpha;
    else if (YK == YK_BF16) ((uint16_t*)a.y)[n] = (uint16_t)bf16_rne(f * a.alpha);
    else ((int32_t*)a.y)[n] = iv;
  }
}

int pick_waves(int64_t NB, int64_t GQ) {
  const int64_t target = 2560;  // resident waves wanted across the chip
  int64_t S = cdiv(target, NB);
  if (S > kMaxWaves) S = kMaxWaves;
  if (S > GQ) S = GQ;
  if (S < 1) S = 1;
  return (int)S;
}

template <int FMT, int R, bool INTC>
hipError_t dispatch_y(const GemvArgs& g, const KArgs& k, dim3 grid, dim3 block, hipStream_t s) {
  if (g.ykind == YK_F32)
    hipLaunchKernelGGL((gemv_mfma<FMT, R, INTC, YK_F32>), grid, block, 0, s, k);
  else if (g.ykind == YK_BF16)
    hipLaunchKernelGGL((gemv_mfma<FMT, R, INTC, YK_BF16>), grid, block, 0, s, k);
  else
    hipLaunchKernelGGL((gemv_mfma<FMT, R, INTC, YK_I32>), grid, block, 0, s, k);
  return hipGetLastError();
}

template <int FMT>
hipError_t dispatch_r(const GemvArgs& g, const KArgs& k, dim3 grid, dim3 block, hipStream_t s) {
  if (g.R == 4) return dispatch_y<FMT, 4, false>(g, k, grid, block, s);
  if (g.int_combine) return dispatch_y<FMT, 2, true>(g, k, grid, block, s);
  return dispatch_y<FMT, 2, false>(g, k, grid, block, s);
}

}  // namespace

hipError_t launch_gemv_mfma(const GemvArgs& g, hipStream_t s) {
  KArgs k;
  int64_t NB = cdiv(g.N, 16), G = g.K / kGroup;
  k.pcodes = g.pcodes;
  k.pscales = g.pscales;
  k.xa = g.xa;
  k.xe = g.xe;
  k.x_scales = g.x_scales;
  k.y = g.y;
  k.N = g.N;
  k.G = G;
  k.GQ = cdiv(G, 4);
  k.GP = cdiv(G, 2);
  k.M = g.M;
  k.MA = g.M * g.R;
  k.x_scale = g.x_scale;
  int S = pick_waves(NB, k.GQ);
  dim3 grid((unsigned)NB), block(64 * S);
  if (g.fmt == 1) return dispatch_r<1>(g, k, grid, block, s);
  if (g.fmt == 2) return dispatch_r<2>(g, k, grid, block, s);
  return hipErrorInvalidValue;
}

hipError_t launch_gemv_sign(const SignArgs& g, hipStream_t s) {
  SArgs k;
  int64_t NB = cdiv(g.N, 16), G = g.K / kGroup;
  k.pcodes = g.pcodes;
  k.pscales = g.pscales;
  k.xw = g.xw;
  k.y = g.y;
  k.N = g.N;
  k.G = G;
  k.GQ = cdiv(G, 4);
  k.alpha = g.alpha;
  int S = pick_waves(NB, k.GQ);
  dim3 grid((unsigned)NB), block(64 * S);
  if (g.ykind == YK_F32) hipLaunchKernelGGL(gemv_sign<YK_F32>, grid, block, 0, s, k);
  else if (g.ykind == YK_BF16) hipLaunchKernelGGL(gemv_sign<YK_BF16>, grid, block, 0, s, k);
  else hipLaunchKernelGGL(gemv_sign<YK_I32>, grid, block, 0, s, k);
  return hipGetLastError();
}

}  // namespace lowbit
