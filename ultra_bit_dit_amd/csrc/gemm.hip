// Large-M products Y[M][N] = X[M][K] . W[N][K]^T over packed binary or
// ternary weights (2-bit or base-3) with one fp16 scale per 128-weight group
// (the group-scaled matmul of the "1-bit 嘅數學" section of the ultra_bit_dit
// page; prefill and diffusion-transformer blocks run it as a dense
// contraction).
//
// One MFMA kernel for every format: gfx950's block-scaled
// v_mfma_scale_f32_16x16x128_f8f6f4 with fp8 e4m3 activations (two exact
// split terms per element, an E8M0 exponent per 32-element block) against fp4
// e2m1 weights decoded from the packed words in registers.  The fp16 group
// scale multiplies each group's fp32 partial; int8 activations with unit
// scales give the exact int32 product.
//
// Activations are first staged (a separate pass over X) into per-(64-row
// tile, group) images laid out exactly as the MFMA's A operand registers, so
// the GEMM copies an image to LDS and every lane reads its operand with two
// 16-byte LDS loads.  Weights are read straight from the packed layout.
#include <algorithm>

#include "common.hpp"
#include "fp4.hpp"

namespace lowbit {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------- GEMM args
struct KArgs {
  const uint8_t* xt;        // staged activation tiles
  const float* rowscale;    // per-row output multiplier, or NULL
  const uint8_t* pcodes;
  const uint16_t* pscales;  // NULL only for the exact int32 product
  void* y;
  float* part;              // split-K partial tiles
  uint32_t* cnt;            // zero-initialised arrival counters
  int64_t M, N, G, GQ, GP, NB, MT, NT;
  int KS;
};

// Workgroup -> (split, row tile, column tile).  Workgroups are dealt to the
// 8 XCDs round-robin; each XCD gets a contiguous run of the tile order
// (column tile fastest), so the workgroups resident on one XCD share their
// activation tiles in that XCD's L2.
__device__ inline void tile_of(const KArgs& a, int64_t& mt, int64_t& nt, int& ks) {
  const int64_t T = a.MT * a.NT * a.KS;
  const int64_t bid = blockIdx.x;
  int64_t id = bid;
  if (T >= 8) {
    const int64_t base = T / 8, rem = T % 8, x = bid % 8, loc = bid / 8;
    id = x * base + min(x, rem) + loc;
  }
  nt = id % a.NT;
  mt = (id / a.NT) % a.MT;
  ks = (int)(id / (a.NT * a.MT));
}

__device__ __forceinline__ float bf16_rne(float v) {
  uint32_t u = __float_as_uint(v);
  if ((u & 0x7F800000u) != 0x7F800000u) u += 0x7FFFu + ((u >> 16) & 1u);
  return __uint_as_float(u & 0xFFFF0000u);
}

template <int YK, typename T>
__device__ __forceinline__ void store_y(void* y, int64_t idx, T v) {
  if constexpr (YK == YK_I32) {
    ((int32_t*)y)[idx] = (int32_t)v;
  } else if constexpr (YK == YK_BF16) {
    ((uint16_t*)y)[idx] = (uint16_t)(__float_as_uint(bf16_rne((float)v)) >> 16);
  } else {
    ((float*)y)[idx] = (float)v;
  }
}

// Split-K: every split stores its partial tile (lane-major, so the stores
// are coalesced), makes it visible device-wide (agent-scope release) and
// bumps the tile counter; the last split to arrive (agent-scope acquire)
// adds all partials in split order (deterministic) and resets the counter.
// Its loads go out 32 values at a time, so the reduction costs a few memory
// round trips rather than one per value.  Returns true in the workgroup that
// must write Y.  INT: the values are int32 bit patterns, added as integers.
template <int NV, bool INT, int THREADS>
__device__ __forceinline__ bool split_reduce(const KArgs& a, int64_t tile, int ks, int wave,
                                             int lane, uint32_t (&v)[NV]) {
  constexpr int CH = 32;  // values per batch of loads
  static_assert(NV % CH == 0, "partial tile in whole batches");
  __shared__ uint32_t s_last;
  const int64_t per = (int64_t)(THREADS / 64) * NV * 64;  // words of one partial tile
  uint32_t* part = (uint32_t*)a.part;
  uint32_t* mine = part + (tile * a.KS + ks) * per + (int64_t)wave * NV * 64 + lane;
#pragma unroll
  for (int i = 0; i < NV; i++) mine[i * 64] = v[i];
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    const uint32_t prev = __hip_atomic_fetch_add(a.cnt + 16 + tile, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(a.KS - 1);
    if (s_last) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  }
  __syncthreads();
  if (!s_last) return false;
#pragma unroll
  for (int i0 = 0; i0 < NV; i0 += CH) {
    float fs[CH];
    int32_t is[CH];
#pragma unroll
    for (int i = 0; i < CH; i++) {
      fs[i] = 0.0f;
      is[i] = 0;
    }
    for (int k = 0; k < a.KS; k++) {
      const uint32_t* src = part + (tile * a.KS + k) * per + (int64_t)wave * NV * 64 + lane;
      uint32_t x[CH];
#pragma unroll
      for (int i = 0; i < CH; i++) x[i] = k == ks ? v[i0 + i] : src[(i0 + i) * 64];
#pragma unroll
      for (int i = 0; i < CH; i++) {
        if constexpr (INT)
          is[i] += (int32_t)x[i];
        else
          fs[i] += __uint_as_float(x[i]);
      }
    }
#pragma unroll
    for (int i = 0; i < CH; i++) v[i0 + i] = INT ? (uint32_t)is[i] : __float_as_uint(fs[i]);
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.cnt + 16 + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  return true;
}

// ---------------------------------------------- fp8 x fp4 MFMA GEMM (all formats)
// The batch-1 kernels' operand scheme at full width: activations enter
// v_mfma_scale_f32_16x16x128_f8f6f4 as two fp8 e4m3 split terms per element
// with an E8M0 exponent per 32-element hardware block (bf16: term 1 is 16x
// the residual of term 0; int8 q = 16 (q >> 4) + (q & 15) exactly), weights
// as fp4 decoded from the packed words with one or two VALU ops per 8
// weights.  One MFMA multiplies 8 activation rows (x 2 terms) by 16 weight
// rows over one group; the group's fp32 partial is scaled by the fp16 group
// scale in fp32 (int8 with unit scales: exact integer per group).
constexpr int kAT = 8;                   // activation rows per MFMA (x 2 terms = 16 A rows)
constexpr int kATBytes = 64 * 32 + 64;   // one A-tile of one group: fp8 bytes + exponents
constexpr int kF8BM = 64;                // activation rows per workgroup tile (8 A-tiles)
constexpr int kF8BN = 256;               // weight rows per workgroup tile (16 row-blocks)
constexpr int kF8Threads = 512;          // 8 waves: 2 (rows) x 4 (columns)
constexpr int kF8Img = (kF8BM / kAT) * kATBytes;  // staged bytes of one workgroup tile and group

// Staging: one thread per (row m, group g, hardware block b).  Block b of a
// group holds k = 128 g + kmap(b, i), i = 0..31 (two runs of 16); A lane
// L = r + 16 kb (A row r, lane group kb) holds bytes e of the blocks with
// b & 1 = kb >> 1, i >> 4 = kb & 1, b >> 1 = e >> 4, i & 15 = e & 15, and
// lane L also supplies the exponent of (A row L % 16, block L / 16).
// Layout: per (64-row tile, group) kF8Img bytes; A-tile a of it at a *
// kATBytes: 64 lanes x 32 fp8 bytes, then 64 exponent bytes (by lane).
// Rows >= M are staged as zeros.
template <int XK>
__global__ __launch_bounds__(256) void stage_f8(int64_t M, int64_t Mpad, int64_t K, int64_t G,
                                                const void* __restrict__ X,
                                                uint8_t* __restrict__ xs) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= Mpad * G * 4) return;
  const int b = (int)(tid & 3);
  const int64_t g = (tid >> 2) % G;
  const int64_t m = (tid >> 2) / G;
  float v[32];
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    const int64_t k0 = g * kGroup + 64 * (b & 1) + 16 * (b >> 1) + 32 * hh;
    if (m < M) {
      if constexpr (XK == XK_BF16) {
        const v4u* src = (const v4u*)((const uint16_t*)X + m * K + k0);
        const v4u w0 = src[0], w1 = src[1];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          v[16 * hh + 2 * j] = __uint_as_float(w0[j] << 16);
          v[16 * hh + 2 * j + 1] = __uint_as_float(w0[j] & 0xFFFF0000u);
          v[16 * hh + 8 + 2 * j] = __uint_as_float(w1[j] << 16);
          v[16 * hh + 8 + 2 * j + 1] = __uint_as_float(w1[j] & 0xFFFF0000u);
        }
      } else {
        const v4u w = *(const v4u*)((const int8_t*)X + m * K + k0);
#pragma unroll
        for (int j = 0; j < 16; j++) v[16 * hh + j] = (float)(int8_t)((w[j >> 2] >> (8 * (j & 3))) & 0xFF);
      }
    } else {
#pragma unroll
      for (int j = 0; j < 16; j++) v[16 * hh + j] = 0.0f;
    }
  }
  float t0[32], t1[32];
  int e0, e1;
  if constexpr (XK == XK_BF16) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
    // E puts the block maximum in [128, 256) x 2^E, clamped so that both
    // terms' exponents stay representable
    int E = 0;
    if (amax != 0.0f) {
      int ex;
      (void)frexpf(amax, &ex);
      E = max((ex - 1) - 7, -127 + kSplitShift);
    }
    const float sc = ldexpf(1.0f, -E);
#pragma unroll
    for (int j = 0; j < 32; j++) t0[j] = v[j] * sc;
    e0 = 127 + E;
    e1 = 127 + E - kSplitShift;
  } else {
#pragma unroll
    for (int j = 0; j < 32; j++) {
      const int q = (int)v[j];
      t0[j] = (float)(q >> 4);
      t1[j] = (float)(q & 15);
    }
    e0 = 127 + kSplitShift;
    e1 = 127;
  }
  uint32_t w0[8], w1[8];
#pragma unroll
  for (int j = 0; j < 8; j++) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(t0[4 * j], t0[4 * j + 1], 0, false);
    w0[j] = __builtin_amdgcn_cvt_pk_fp8_f32(t0[4 * j + 2], t0[4 * j + 3], w, true);
  }
  if constexpr (XK == XK_BF16) {
    // term 1 = rne_e4m3(16 x (t - term 0)), the residual exact in fp32
#pragma unroll
    for (int j = 0; j < 8; j++) {
      const uint32_t w = w0[j];
      t1[4 * j] = (t0[4 * j] - __builtin_amdgcn_cvt_f32_fp8(w, 0)) * 16.0f;
      t1[4 * j + 1] = (t0[4 * j + 1] - __builtin_amdgcn_cvt_f32_fp8(w, 1)) * 16.0f;
      t1[4 * j + 2] = (t0[4 * j + 2] - __builtin_amdgcn_cvt_f32_fp8(w, 2)) * 16.0f;
      t1[4 * j + 3] = (t0[4 * j + 3] - __builtin_amdgcn_cvt_f32_fp8(w, 3)) * 16.0f;
    }
  }
#pragma unroll
  for (int j = 0; j < 8; j++) {
    uint32_t w = __builtin_amdgcn_cvt_pk_fp8_f32(t1[4 * j], t1[4 * j + 1], 0, false);
    w1[j] = __builtin_amdgcn_cvt_pk_fp8_f32(t1[4 * j + 2], t1[4 * j + 3], w, true);
  }
  uint8_t* blk = xs + ((m / kF8BM) * G + g) * (int64_t)kF8Img + ((m % kF8BM) / kAT) * kATBytes;
  const int r0 = 2 * (int)(m % kAT);  // A row of term 0 (term 1 is the next row)
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    const int kb = 2 * (b & 1) + hh;
    const int e = 16 * (b >> 1);
    *(v4u*)(blk + (r0 + 16 * kb) * 32 + e) = v4u{w0[4 * hh], w0[4 * hh + 1], w0[4 * hh + 2], w0[4 * hh + 3]};
    *(v4u*)(blk + (r0 + 1 + 16 * kb) * 32 + e) = v4u{w1[4 * hh], w1[4 * hh + 1], w1[4 * hh + 2], w1[4 * hh + 3]};
  }
  blk[2048 + r0 + 16 * b] = (uint8_t)e0;
  blk[2048 + r0 + 1 + 16 * b] = (uint8_t)e1;
}

template <int T>
__device__ __forceinline__ v4f mfma_f8f4(const v8i& A, const v8i& B, int se) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // A: fp8 e4m3 (0) with the E8M0 block exponent in byte 0 of se; B: fp4 e2m1 (4), unscaled
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, 0, 4, 0, se, 0, 127);
}

// Workgroup tile 64 rows x 256 columns, 8 waves: wave (wm, wn) owns A-tiles
// 4 wm .. 4 wm + 3 (32 rows) and row-blocks 4 wn .. 4 wn + 3 (64 columns).
// Per group: the workgroup's staged activations (kF8Img bytes) sit in one of
// two LDS buffers; codes and scales are loaded a quad (4 groups) ahead.
template <int FMT, int XK, int YK, bool SCALED>
__global__ __launch_bounds__(kF8Threads) __attribute__((amdgpu_waves_per_eu(2))) void gemm_f8(KArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kF8Img];
  __shared__ uint32_t t3[256];
  constexpr bool INT = XK == XK_I8 && !SCALED;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  int64_t mt, nt;
  int ks;
  tile_of(a, mt, nt, ks);
  const int64_t q0 = a.GQ * ks / a.KS, q1 = a.GQ * (ks + 1) / a.KS;
  const int64_t g0 = 4 * q0, g1 = min<int64_t>(4 * q1, a.G);
  int64_t rbj[4];
  bool live[4];
#pragma unroll
  for (int j = 0; j < 4; j++) {
    const int64_t rb = nt * 16 + wn * 4 + j;
    live[j] = rb < a.NB;
    rbj[j] = live[j] ? rb : a.NB - 1;
  }
  if constexpr (FMT == 3) fill_trit_table(t3);
  const uint8_t* xs = a.xt + mt * a.G * (int64_t)kF8Img;
  constexpr int XR = (kF8Img / 16 + kF8Threads - 1) / kF8Threads;  // 16-byte pieces per thread
  auto xload = [&](int64_t g, v4u& x0, v4u& x1, v4u& x2) {
    const v4u* src = (const v4u*)(xs + g * kF8Img);
    constexpr int NP = kF8Img / 16;
    x0 = src[tid];
    x1 = src[min(kF8Threads + tid, NP - 1)];
    x2 = src[min(2 * kF8Threads + tid, NP - 1)];
  };
  auto xput = [&](uint8_t* dst, const v4u& x0, const v4u& x1, const v4u& x2) {
    constexpr int NP = kF8Img / 16;
    ((v4u*)dst)[tid] = x0;
    if (kF8Threads + tid < NP) ((v4u*)dst)[kF8Threads + tid] = x1;
    if (2 * kF8Threads + tid < NP) ((v4u*)dst)[2 * kF8Threads + tid] = x2;
  };
  static_assert(XR == 3, "staged group image in three 16-byte pieces per thread");

  float acc[4][4][2];
  int iacc[4][4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int u = 0; u < 2; u++) {
        acc[i][j][u] = 0.f;
        iacc[i][j][u] = 0;
      }

  v4u x0, x1, x2;
  xload(g0, x0, x1, x2);
  xput(lds[0], x0, x1, x2);
  Quad<FMT> qd[4], qn[4];
#pragma unroll
  for (int j = 0; j < 4; j++)
    load_quad_at<FMT>(a.pcodes, a.pscales, rbj[j], min<int64_t>(q0, a.GQ - 1), a.GQ, a.GP, lane, qd[j]);
  __syncthreads();

  for (int64_t q = q0; q < q1; q++) {
    // next quad's codes and scales
    const int64_t qnx = min<int64_t>(q + 1 < q1 ? q + 1 : q, a.GQ - 1);
#pragma unroll
    for (int j = 0; j < 4; j++)
      load_quad_at<FMT>(a.pcodes, a.pscales, rbj[j], qnx, a.GQ, a.GP, lane, qn[j]);
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const int64_t g = 4 * q + t;
      if (g < g1) {
        const int buf = (int)((g - g0) & 1);
        const int64_t gn = g + 1 < g1 ? g + 1 : g;
        xload(gn, x0, x1, x2);
        v8i B[4];
        float sj[4];
#pragma unroll
        for (int j = 0; j < 4; j++) {
          B[j] = decode_group<FMT>(qd[j], t, t3);
          sj[j] = a.pscales ? quad_scale<FMT>(qd[j], t) : 1.0f;
        }
        const uint8_t* L = lds[buf];
#pragma unroll
        for (int i = 0; i < 4; i++) {
          const uint8_t* at = L + (4 * wm + i) * kATBytes;
          const v4u a0 = *(const v4u*)(at + 32 * lane), a1 = *(const v4u*)(at + 32 * lane + 16);
          const v8i A = v8i{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w,
                            (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
          const int se = at[2048 + lane];
          v4f c[4];
#pragma unroll
          for (int j = 0; j < 4; j++) c[j] = mfma_f8f4<0>(A, B[j], se);
#pragma unroll
          for (int j = 0; j < 4; j++) {
            const float s0 = c[j][0] + c[j][1], s1 = c[j][2] + c[j][3];
            if constexpr (INT) {
              iacc[i][j][0] += __float2int_rn(s0);
              iacc[i][j][1] += __float2int_rn(s1);
            } else {
              acc[i][j][0] = fmaf(sj[j], s0, acc[i][j][0]);
              acc[i][j][1] = fmaf(sj[j], s1, acc[i][j][1]);
            }
          }
        }
        if (g + 1 < g1) xput(lds[buf ^ 1], x0, x1, x2);
        __syncthreads();
      }
    }
#pragma unroll
    for (int j = 0; j < 4; j++) qd[j] = qn[j];
  }

  uint32_t v[32];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int j = 0; j < 4; j++)
#pragma unroll
      for (int u = 0; u < 2; u++)
        v[(i * 4 + j) * 2 + u] = INT ? (uint32_t)iacc[i][j][u] : __float_as_uint(acc[i][j][u]);
  if (a.KS > 1 && !split_reduce<32, INT, kF8Threads>(a, mt * a.NT + nt, ks, wave, lane, v)) return;
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int u = 0; u < 2; u++) {
      const int64_t row = mt * kF8BM + 32 * wm + 8 * i + 2 * (lane >> 4) + u;
      if (row >= a.M) continue;
      const float rs = SCALED ? a.rowscale[row] : 1.0f;
#pragma unroll
      for (int j = 0; j < 4; j++) {
        const int64_t col = (nt * 16 + wn * 4 + j) * 16 + (lane & 15);
        if (!live[j] || col >= a.N) continue;
        const uint32_t x = v[(i * 4 + j) * 2 + u];
        if constexpr (INT)
          store_y<YK>(a.y, row * a.N + col, (int32_t)x);
        else
          store_y<YK>(a.y, row * a.N + col, __uint_as_float(x) * rs);
      }
    }
  }
}

// ---------------------------------------------------------------- planning
struct GemmPlan {
  int64_t MT, NT, G, KS;
  size_t xt_off, rs_off, part_off, bytes;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// K-split count: the smallest that keeps at least ~85% of a whole number of
// waves of workgroups busy on the 256 compute units (one workgroup each),
// up to 8 and at most one quad of groups per split
int64_t pick_splits(int64_t tiles, int64_t GQ) {
  const int64_t slots = 256;
  int64_t best = 1;
  double best_eff = 0.0;
  for (int64_t ks = 1; ks <= std::min<int64_t>(8, GQ); ks++) {
    const int64_t wgs = tiles * ks;
    const double eff = (double)wgs / (double)(slots * cdiv(wgs, slots));
    if (eff > best_eff + 1e-9) {
      best = ks;
      best_eff = eff;
    }
    if (eff >= 0.85) return ks;
  }
  return best;
}

GemmPlan make_gemm_plan(int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  p.G = K / kGroup;
  p.MT = cdiv(M, kF8BM);
  p.NT = cdiv(N, kF8BN);
  const int64_t tiles = p.MT * p.NT;
  p.KS = tiles > kMaxRowGroups ? 1 : pick_splits(tiles, cdiv(p.G, 4));
  p.rs_off = kCounterBytes;
  p.xt_off = p.rs_off;
  p.part_off = p.xt_off + align256((size_t)p.MT * p.G * kF8Img);
  const size_t part_tile = (size_t)kF8BM * kF8BN * 4;
  p.bytes = p.part_off + (p.KS > 1 ? (size_t)p.KS * tiles * part_tile : 0);
  return p;
}

template <int FMT>
hipError_t launch_fmt(const GemmArgs& g, const GemmPlan& p, hipStream_t s) {
  uint8_t* ws = (uint8_t*)g.ws;
  KArgs k;
  k.xt = ws + p.xt_off;
  k.pcodes = (const uint8_t*)g.pcodes;
  k.pscales = g.pscales;
  k.rowscale = g.xkind == XK_I8 ? g.x_scales : nullptr;
  k.y = g.y;
  k.part = (float*)(ws + p.part_off);
  k.cnt = (uint32_t*)ws;
  k.M = g.M;
  k.N = g.N;
  k.G = p.G;
  k.GQ = cdiv(p.G, 4);
  k.GP = cdiv(p.G, 2);
  k.NB = cdiv(g.N, 16);
  k.MT = p.MT;
  k.NT = p.NT;
  k.KS = (int)p.KS;
  const int64_t Mpad = p.MT * kF8BM;
  const int64_t units = Mpad * p.G * 4;
  const dim3 sgrid((unsigned)cdiv(units, 256));
  const dim3 grid((unsigned)(p.MT * p.NT * p.KS)), block(kF8Threads);
  if (g.xkind == XK_BF16) {
    hipLaunchKernelGGL(stage_f8<XK_BF16>, sgrid, dim3(256), 0, s, g.M, Mpad, g.K, p.G, g.x,
                       (uint8_t*)k.xt);
    if (g.ykind == YK_BF16)
      hipLaunchKernelGGL((gemm_f8<FMT, XK_BF16, YK_BF16, false>), grid, block, 0, s, k);
    else
      hipLaunchKernelGGL((gemm_f8<FMT, XK_BF16, YK_F32, false>), grid, block, 0, s, k);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(stage_f8<XK_I8>, sgrid, dim3(256), 0, s, g.M, Mpad, g.K, p.G, g.x,
                     (uint8_t*)k.xt);
  if (g.ykind == YK_I32)
    hipLaunchKernelGGL((gemm_f8<FMT, XK_I8, YK_I32, false>), grid, block, 0, s, k);
  else if (g.ykind == YK_BF16)
    hipLaunchKernelGGL((gemm_f8<FMT, XK_I8, YK_BF16, true>), grid, block, 0, s, k);
  else
    hipLaunchKernelGGL((gemm_f8<FMT, XK_I8, YK_F32, true>), grid, block, 0, s, k);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int xkind) {
  (void)xkind;
  return make_gemm_plan(M, N, K).bytes;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.xkind != XK_BF16 && g.xkind != XK_I8) return hipErrorInvalidValue;
  if (g.xkind == XK_BF16 && g.ykind == YK_I32) return hipErrorInvalidValue;
  if (g.xkind == XK_I8 && (g.ykind == YK_I32) != (g.pscales == nullptr)) return hipErrorInvalidValue;
  if (g.xkind == XK_I8 && g.ykind != YK_I32 && g.x_scales == nullptr) return hipErrorInvalidValue;
  const GemmPlan p = make_gemm_plan(g.M, g.N, g.K);
  if (p.MT * p.NT * p.KS > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (g.fmt == 1) return launch_fmt<1>(g, p, s);
  if (g.fmt == 2) return launch_fmt<2>(g, p, s);
  if (g.fmt == 3) return launch_fmt<3>(g, p, s);
  return hipErrorInvalidValue;
}

}  // namespace lowbit
