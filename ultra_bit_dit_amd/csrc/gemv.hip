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
#include <algorithm>
#include <vector>

#include "common.hpp"

namespace lowbit {
namespace {

constexpr int kMaxWaves = 16;  // waves per workgroup of the sign kernel
constexpr uint32_t kChainSpinLimit = 1u << 24;  // sleeps before a chain wait gives up
constexpr int kMaxW = 4;       // waves (row-blocks) per MFMA workgroup, at most

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

// ------------------------------------------------------- activation staging
// The MFMA multiplies fp4 weights (exactly +-1 / 0) by activations given as
// fp8 e4m3 split terms.  For each 32-element hardware block, E is chosen so
// the block maximum scaled by 2^-E lies in [128, 256); term 0 is
// rne_e4m3(v), each next term is rne_e4m3 of 16 x the remaining residual,
// and term r carries the E8M0 block exponent E - 4r, applied inside the
// MFMA.  Two terms reproduce a bf16 value exactly for elements within 2^13 of
// the block maximum (smaller ones keep an error below 2^-21 x the maximum);
// four terms give fp32 inputs 16 significant bits.  int8 values q are split
// exactly as 16 * (q >> 4) + (q & 15).  The conversions use the hardware
// v_cvt_pk_fp8_f32 / v_cvt_f32_fp8 (OCP e4m3, round to nearest even).
//
// Hardware block b of a group covers MFMA positions h = 32b + i; position h
// pairs with fp4 weight slot i of quarter b (activation k = 128g +
// kmap(b, i)) and is fed by A byte e = 16(b>>1) + (i&15) of lane group
// kb = 2(b&1) + (i>>4).  The scale of block b is read from lane group b.
//
// Each workgroup stages the quads of its K-slice into LDS (MA = M x R rows
// of A, ql = quad index inside the slice):
//   xa[((ql * 16 + t * 4 + kb) * MA + a) * 32 + e]   fp8 bytes (group t of the quad)
//   xe[((ql * 4 + b) * MA + a) * 4 + t]             E8M0 exponents

__device__ inline void load8(int xkind, const void* X, int64_t idx, float (&v)[8]) {
  if (xkind == XK_BF16) {
    const uint4 w = *(const uint4*)((const uint16_t*)X + idx);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[2 * j] = __uint_as_float(u[j] << 16);
      v[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  } else if (xkind == XK_F32) {
    const float4 a = *(const float4*)((const float*)X + idx);
    const float4 b = *(const float4*)((const float*)X + idx + 4);
    v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
    v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
  } else {
    const uint2 w = *(const uint2*)((const int8_t*)X + idx);
#pragma unroll
    for (int j = 0; j < 8; j++)
      v[j] = (float)(int8_t)(((j < 4 ? w.x : w.y) >> (8 * (j & 3))) & 0xFF);
  }
}

struct FArgs {
  const uint8_t* pcodes;
  const uint16_t* pscales;
  const void* x;
  const float* x_scales;
  void* y;
  float* part;    // split-K partial sums [KS][M][Npad]
  uint32_t* cnt;  // [16 + rg]: arrivals of the row group's K-slices
  int64_t N, K, G, GQ, GP, M, MA, NB, KS, Npad;
  float x_scale;
  int xkind;
};

// Staging of quads [q0, q1) of the M activation rows into LDS by all threads
// of the workgroup.  Work unit = 8 consecutive elements of a hardware block
// (the 4 units of a block sit in adjacent lanes); a thread handles units
// c = threadIdx + round * blockDim.  The loads of the first kStageRounds
// rounds are issued together (stage_load) so that they share one memory
// round trip with the weight loads; stage_convert then writes the terms.
constexpr int kStageRounds = 5;

__device__ __attribute__((always_inline)) inline bool stage_unit(const FArgs& a, int64_t q0,
                                                                 int64_t nq, int64_t c, int& ch,
                                                                 int& b, int& t, int64_t& ql,
                                                                 int64_t& m, int64_t& g) {
  ch = (int)(c & 3);
  b = (int)((c >> 2) & 3);
  t = (int)((c >> 4) & 3);
  const int64_t rest = c >> 6;
  ql = rest % nq;
  m = rest / nq;
  g = 4 * (q0 + ql) + t;
  return c < nq * 64 * a.M && g < a.G;
}

// raw activations of one unit: bf16 in ra, f32 in ra:rb, int8 in ra.xy.
// The load is unconditional (a unit past the end reads element 0) so that
// no control flow joins wait on it.  COH: device-coherent loads, for
// activations another workgroup may just have written.
__device__ __attribute__((always_inline)) inline uint4 coh_load4(const void* p) {
  const uint32_t* w = (const uint32_t*)p;
  return make_uint4(__hip_atomic_load(w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                    __hip_atomic_load(w + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                    __hip_atomic_load(w + 2, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT),
                    __hip_atomic_load(w + 3, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}

template <int XK, bool COH>
__device__ __attribute__((always_inline)) inline void stage_load1(const FArgs& a, int64_t q0,
                                                                  int64_t nq, int64_t rd,
                                                                  uint4& ra, uint4& rb) {
  const int64_t c = rd * blockDim.x + threadIdx.x;
  int ch, b, t;
  int64_t ql, m, g;
  const bool valid = stage_unit(a, q0, nq, c, ch, b, t, ql, m, g);
  const int64_t idx = valid ? m * a.K + g * kGroup + kmap(b, 8 * ch) : 0;
  if constexpr (XK == XK_BF16) {
    const uint16_t* p = (const uint16_t*)a.x + idx;
    ra = COH ? coh_load4(p) : *(const uint4*)p;
    rb = ra;
  } else if constexpr (XK == XK_F32) {
    const float* p = (const float*)a.x + idx;
    ra = COH ? coh_load4(p) : *(const uint4*)p;
    rb = COH ? coh_load4(p + 4) : *(const uint4*)(p + 4);
  } else {
    const uint2 w = *(const uint2*)((const int8_t*)a.x + idx);
    ra = make_uint4(w.x, w.y, w.x, w.y);
    rb = ra;
  }
}

// convert one round of units into fp8 terms and exponents in LDS
template <int R, int XK>
__device__ __attribute__((always_inline)) inline void stage_convert1(const FArgs& a, int64_t q0,
                                                                     int64_t nq, int64_t rd,
                                                                     uint4 ra, uint4 rb,
                                                                     uint8_t* xa, uint8_t* xe) {
  if (rd * blockDim.x >= nq * 64 * a.M) return;  // uniform: round past the end
  const int64_t c = rd * blockDim.x + threadIdx.x;
  int ch, b, t;
  int64_t ql, m, g;
  const bool valid = stage_unit(a, q0, nq, c, ch, b, t, ql, m, g);
  const bool inside = c < nq * 64 * a.M;  // a slot of the slice (padding groups get zeros)
  float v[8];
  if constexpr (XK == XK_BF16) {
    const uint32_t u[4] = {ra.x, ra.y, ra.z, ra.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[2 * j] = __uint_as_float(u[j] << 16);
      v[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  } else if constexpr (XK == XK_F32) {
    v[0] = __uint_as_float(ra.x); v[1] = __uint_as_float(ra.y);
    v[2] = __uint_as_float(ra.z); v[3] = __uint_as_float(ra.w);
    v[4] = __uint_as_float(rb.x); v[5] = __uint_as_float(rb.y);
    v[6] = __uint_as_float(rb.z); v[7] = __uint_as_float(rb.w);
  } else {
#pragma unroll
    for (int j = 0; j < 8; j++)
      v[j] = (float)(int8_t)(((j < 4 ? ra.x : ra.y) >> (8 * (j & 3))) & 0xFF);
  }
  if (!valid) {
#pragma unroll
    for (int j = 0; j < 8; j++) v[j] = 0.f;
  }
  float amax = 0.f;
#pragma unroll
  for (int j = 0; j < 8; j++) amax = fmaxf(amax, fabsf(v[j]));
  amax = fmaxf(amax, __shfl_xor(amax, 1));  // the 4 units of a block
  amax = fmaxf(amax, __shfl_xor(amax, 2));
  if (!inside) return;
  int E = 0;
  if (XK != XK_I8 && amax != 0.0f) {
    int ex;
    frexpf(amax, &ex);
    E = (ex - 1) - 7;
    const int lo = -127 + kSplitShift * (R - 1);
    if (E < lo) E = lo;
  }
  const int kb = 2 * (b & 1) + (ch >> 1), e = 16 * (b >> 1) + 8 * (ch & 1);
  float tv[8];
  if constexpr (XK == XK_I8) {
#pragma unroll
    for (int j = 0; j < 8; j++) tv[j] = v[j];
  } else {
    // exact power of two: E is clamped to [-127 + 4(R-1), 120]
    const float sc = ldexpf(1.0f, -E);
#pragma unroll
    for (int j = 0; j < 8; j++) tv[j] = v[j] * sc;
  }
#pragma unroll
  for (int r = 0; r < R; r++) {
    uint32_t w0, w1;
    int Er;
    if constexpr (XK == XK_I8) {
      float p[8];
#pragma unroll
      for (int j = 0; j < 8; j++) {
        const int q = (int)tv[j];
        p[j] = (float)(r == 0 ? (q >> 4) : (q & 15));
      }
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(p[0], p[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(p[2], p[3], w0, true);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(p[4], p[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(p[6], p[7], w1, true);
      Er = r == 0 ? 4 : 0;
    } else {
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(tv[0], tv[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(tv[2], tv[3], w0, true);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(tv[4], tv[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(tv[6], tv[7], w1, true);
      if (r + 1 < R) {  // residual for the next term, exact in fp32
        const float d[8] = {
            __builtin_amdgcn_cvt_f32_fp8(w0, 0), __builtin_amdgcn_cvt_f32_fp8(w0, 1),
            __builtin_amdgcn_cvt_f32_fp8(w0, 2), __builtin_amdgcn_cvt_f32_fp8(w0, 3),
            __builtin_amdgcn_cvt_f32_fp8(w1, 0), __builtin_amdgcn_cvt_f32_fp8(w1, 1),
            __builtin_amdgcn_cvt_f32_fp8(w1, 2), __builtin_amdgcn_cvt_f32_fp8(w1, 3)};
#pragma unroll
        for (int j = 0; j < 8; j++) tv[j] = (tv[j] - d[j]) * 16.0f;
      }
      Er = E - kSplitShift * r;
    }
    const int64_t arow = m * R + r;
    *(uint2*)(xa + ((ql * 16 + t * 4 + kb) * a.MA + arow) * 32 + e) = make_uint2(w0, w1);
    if (ch == 0) xe[((ql * 4 + b) * a.MA + arow) * 4 + t] = (uint8_t)(127 + Er);
  }
}

// --------------------------------------------------------------- MFMA GEMV
// Workgroup = W waves, one row-block (16 rows) per wave, all on one K-slice of
// up to QM whole 4-group quads.  Every wave issues the loads of all its codes
// and scales at once, then the workgroup stages the slice's activations into
// LDS while those loads are in flight; one staged group of activations feeds
// the MFMAs of all W row-blocks.  With several K-slices, each workgroup
// writes coherent partial sums and the last workgroup of the row group to
// arrive adds them in slice order.
//
// gemv_item does that for work item `blk` (row group blk / KS, K-slice
// blk % KS).  It is the body of the one-product kernel (item = workgroup)
// and of the persistent multi-product kernel (CHAIN: items of several
// products in turn, outputs written with device-coherent stores).  WAIT:
// the weight loads go out first, then the workgroup waits until `wait_cnt`
// reaches `wait_target` -- the previous product is complete -- and reads
// its activations with device-coherent loads.
template <int FMT, int XK, int MX, int YK, int QM, bool CHAIN, bool WAIT>
__device__ __attribute__((always_inline)) inline void gemv_item(
    const FArgs& a, int64_t blk, uint8_t* smem, const uint32_t* wait_cnt, uint32_t wait_target,
    uint32_t* err) {
  constexpr int R = XK == XK_F32 ? kSplitF32 : kSplitBF16;
  constexpr bool INTC = XK == XK_I8;
  constexpr int NC = FMT == 1 ? 1 : 2;  // 16-byte code vectors per quad (2-bit, binary)
  __shared__ uint32_t s_last;
  const int W = blockDim.x >> 6;
  const int L = threadIdx.x & 63, w = threadIdx.x >> 6, r = L & 15, lg = L >> 4;
  const int64_t rg = blk / a.KS, ks = blk % a.KS;
  // K-slices in whole quads; base-3 slices in whole octets (two quads)
  const int64_t GO = cdiv(a.GQ, 2);
  const int64_t q0 = FMT == 3 ? 2 * (GO * ks / a.KS) : a.GQ * ks / a.KS;
  const int64_t q1 = FMT == 3 ? min<int64_t>(2 * (GO * (ks + 1) / a.KS), a.GQ) : a.GQ * (ks + 1) / a.KS;
  const int nq = (int)(q1 - q0);
  const int64_t rb = (int64_t)W * rg + w;  // this wave's row-block
  const bool live = rb < a.NB;
  const bool arow = r < a.MA;
  uint8_t* xa = smem;
  uint8_t* xe = smem + (int64_t)nq * 16 * a.MA * 32;
  // 32 zero bytes + one word of unit exponents, read by lanes that hold no
  // activation row (their A operand is zero)
  uint8_t* zblk = xe + (int64_t)nq * 16 * a.MA;
  if (threadIdx.x < 9) ((uint32_t*)zblk)[threadIdx.x] = threadIdx.x < 8 ? 0u : 0x7F7F7F7Fu;
  // base-3: byte value -> its 5 trits as fp4 nibbles (trit 0 -> -1 = 0xA,
  // 1 -> 0, 2 -> +1 = 0x2), nibble e = trit e (least significant first)
  uint32_t* t3 = (uint32_t*)(zblk + 48);
  if constexpr (FMT == 3) {
    if (threadIdx.x < 243) {
      uint32_t v = threadIdx.x, nib = 0;
#pragma unroll
      for (int e = 0; e < 5; e++) {
        const uint32_t t = v % 3;
        v /= 3;
        nib |= (t == 0 ? 0xAu : t == 2 ? 0x2u : 0u) << (4 * e);
      }
      t3[threadIdx.x] = nib;
    }
  }

  uint4 ra[kStageRounds], rbv[kStageRounds];
  if constexpr (!WAIT) {
    // activation loads of the first staging rounds go out first
#pragma unroll
    for (int k = 0; k < kStageRounds; k++) stage_load1<XK, false>(a, q0, nq, k, ra[k], rbv[k]);
  }

  typedef unsigned int u4 __attribute__((ext_vector_type(4)));
  const u4* pcv = (const u4*)a.pcodes;
  const uint2* ps2 = (const uint2*)a.pscales;
  u4 cw[FMT == 3 ? 1 : QM][NC];
  typedef unsigned int u2 __attribute__((ext_vector_type(2)));
  u2 c3[FMT == 3 ? QM : 1][3];  // base-3: 24 bytes of 5-trit bytes per quad
  uint32_t c3t[FMT == 3 ? QM : 1];  // and the lane's word of 4-trit bytes
  uint2 sc[QM];
  // Every code and scale of the wave is requested before anything else.  The
  // loads are unconditional (clamped to the last valid block, results of
  // clamped loads are never used) so that none of them waits on another.
  const bool unit_scales = a.pscales == nullptr;
  const uint2* sbase = unit_scales ? (const uint2*)a.pcodes : ps2;  // any readable memory
  const int64_t rbc = live ? rb : a.NB - 1;
#pragma unroll
  for (int q = 0; q < QM; q++) {
    const int64_t gq = min<int64_t>(q0 + q, a.GQ - 1);
    if constexpr (FMT == 1) {
      cw[q][0] = __builtin_nontemporal_load(&pcv[(rbc * a.GQ + gq) * 64 + L]);
    } else if constexpr (FMT == 3) {
      // octet block (rb, gq/2): plane s of lane L at 1024 s + 16 L; the quad's
      // half h = gq % 2 takes 8-byte chunks 3h .. 3h+2 (chunk c = plane c/2,
      // half c%2) and bytes 2h, 2h+1 of the 4-byte word at 3072 + 4 L
      const uint8_t* ob = a.pcodes + (rbc * GO + (gq >> 1)) * 3328;
      const int h = (int)(gq & 1);
#pragma unroll
      for (int cc = 0; cc < 3; cc++) {
        const int c = 3 * h + cc;
        c3[q][cc] = __builtin_nontemporal_load((const u2*)(ob + 1024 * (c >> 1) + 16 * L + 8 * (c & 1)));
      }
      c3t[q] = __builtin_nontemporal_load((const uint32_t*)(ob + 3072 + 4 * L)) >> (16 * h);
    } else {
      const int64_t p0 = 2 * gq, p1 = min<int64_t>(2 * gq + 1, a.GP - 1);
      cw[q][0] = __builtin_nontemporal_load(&pcv[(rbc * a.GP + p0) * 64 + L]);
      cw[q][NC - 1] = __builtin_nontemporal_load(&pcv[(rbc * a.GP + p1) * 64 + L]);
    }
    sc[q] = sbase[(rbc * a.GQ + gq) * 16 + r];
  }
  if constexpr (WAIT) {
    // the previous product must be complete before its outputs are read; the
    // weight loads above are already in flight
    if (threadIdx.x == 0) {
      for (uint32_t spin = 0;
           __hip_atomic_load(wait_cnt, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < wait_target;
           spin++) {
        if (spin >= kChainSpinLimit) {  // never satisfied: flag it and go on
          __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < kStageRounds; k++) stage_load1<XK, true>(a, q0, nq, k, ra[k], rbv[k]);
  }
#pragma unroll
  for (int k = 0; k < kStageRounds; k++) stage_convert1<R, XK>(a, q0, nq, k, ra[k], rbv[k], xa, xe);
  // remaining rounds (small-M products with long slices), loaded and converted in turn
  const int64_t rounds = cdiv(nq * 64 * a.M, (int64_t)blockDim.x);
  for (int64_t rd = kStageRounds; rd < rounds; rd++) {
    uint4 r0, r1;
    stage_load1<XK, WAIT>(a, q0, nq, rd, r0, r1);
    stage_convert1<R, XK>(a, q0, nq, rd, r0, r1, xa, xe);
  }
  __syncthreads();

  float acc[MX];
  int iacc[MX];
#pragma unroll
  for (int j = 0; j < MX; j++) {
    acc[j] = 0.f;
    iacc[j] = 0;
  }
  if (live) {
#pragma unroll
    for (int q = 0; q < QM; q++) {
      if (q < nq) {
        // the 4 groups of the quad: operands first, then 4 independent MFMAs,
        // then the epilogues (padding groups have zero activations)
        const uint32_t se = *(const uint32_t*)(arow ? xe + ((q * 4 + lg) * a.MA + r) * 4 : zblk + 32);
        v8i A[4], B[4];
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const uint4* src =
              (const uint4*)(arow ? xa + ((q * 16 + t * 4 + lg) * a.MA + r) * 32 : zblk);
          const uint4 x0 = src[0], x1 = src[1];
          A[t] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w,
                     (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
          uint32_t d0, d1, d2, d3;
          if constexpr (FMT == 1) {
            const u4 c4 = cw[q][0];
            const uint32_t wv = t == 0 ? c4.x : t == 1 ? c4.y : t == 2 ? c4.z : c4.w;
            d0 = (wv & 0x88888888u) | 0x22222222u;
            d1 = ((wv << 1) & 0x88888888u) | 0x22222222u;
            d2 = ((wv << 2) & 0x88888888u) | 0x22222222u;
            d3 = ((wv << 3) & 0x88888888u) | 0x22222222u;
          } else if constexpr (FMT == 3) {
            // group t of the quad: bytes 6t .. 6t+5 hold slots 0..29, the
            // 4-trit byte t/2 digits 2(t%2), 2(t%2)+1 hold slots 30, 31
            const uint32_t w6[6] = {c3[q][0].x, c3[q][0].y, c3[q][1].x,
                                    c3[q][1].y, c3[q][2].x, c3[q][2].y};
            uint32_t nb[6];
#pragma unroll
            for (int i = 0; i < 6; i++) {
              const int byte = 6 * t + i;
              nb[i] = t3[(w6[byte >> 2] >> (8 * (byte & 3))) & 0xFFu];
            }
            const uint32_t tl = (t3[(c3t[q] >> (8 * (t >> 1))) & 0xFFu] >> (8 * (t & 1))) & 0xFFu;
            // slot s -> nibble s of d0..d3 (5 slots per byte)
            const uint64_t lo = (uint64_t)nb[0] | ((uint64_t)nb[1] << 20) | ((uint64_t)nb[2] << 40) |
                                ((uint64_t)nb[3] << 60);
            const uint64_t hi = (uint64_t)(nb[3] >> 4) | ((uint64_t)nb[4] << 16) |
                                ((uint64_t)nb[5] << 36) | ((uint64_t)tl << 56);
            d0 = (uint32_t)lo;
            d1 = (uint32_t)(lo >> 32);
            d2 = (uint32_t)hi;
            d3 = (uint32_t)(hi >> 32);
          } else {
            const u4 c4 = cw[q][(t >> 1) % NC];
            const uint32_t p0 = (t & 1) ? c4.z : c4.x, p1 = (t & 1) ? c4.w : c4.y;
            d0 = p0 & 0xAAAAAAAAu;
            d1 = (p0 << 1) & 0xAAAAAAAAu;
            d2 = p1 & 0xAAAAAAAAu;
            d3 = (p1 << 1) & 0xAAAAAAAAu;
          }
          B[t] = v8i{(int)d0, (int)d1, (int)d2, (int)d3, 0, 0, 0, 0};
        }
        v4f c[4];
        c[0] = mfma_group<0>(A[0], B[0], (int)se);
        c[1] = mfma_group<1>(A[1], B[1], (int)se);
        c[2] = mfma_group<2>(A[2], B[2], (int)se);
        c[3] = mfma_group<3>(A[3], B[3], (int)se);
#pragma unroll
        for (int t = 0; t < 4; t++) {
          const float s = unit_scales
                              ? 1.0f
                              : f16_bits_to_f32((t < 2 ? sc[q].x : sc[q].y) >> (16 * (t & 1)));
#pragma unroll
          for (int j = 0; j < MX; j++) {
            float tsum = c[t][R * j];
#pragma unroll
            for (int i = 1; i < R; i++) tsum += c[t][R * j + i];
            acc[j] = fmaf(s, tsum, acc[j]);
            if (INTC) iacc[j] += __float2int_rn(tsum);
          }
        }
      }
    }
  }

  // ---- output
  auto store = [&](int64_t m, int64_t n, float f, int iv) {
    const float sxm = a.x_scales ? a.x_scales[m] : a.x_scale;
    if constexpr (CHAIN) {
      if (YK == YK_F32)
        __hip_atomic_store((float*)a.y + m * a.N + n, f * sxm, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      else if (YK == YK_BF16)
        __hip_atomic_store((uint16_t*)a.y + m * a.N + n, (uint16_t)bf16_rne(f * sxm),
                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else
        __hip_atomic_store((int32_t*)a.y + m * a.N + n, iv, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
    } else {
      if (YK == YK_F32) ((float*)a.y)[m * a.N + n] = f * sxm;
      else if (YK == YK_BF16) ((uint16_t*)a.y)[m * a.N + n] = (uint16_t)bf16_rne(f * sxm);
      else ((int32_t*)a.y)[m * a.N + n] = iv;
    }
  };
  constexpr bool IPART = INTC && YK == YK_I32;
  const int64_t n = 16 * rb + r;
  if (a.KS == 1) {
#pragma unroll
    for (int j = 0; j < MX; j++) {
      const int64_t m = (int64_t)lg * (4 / R) + j;
      if (live && m < a.M && n < a.N) store(m, n, acc[j], iacc[j]);
    }
    return;
  }
  // partials: write-through (agent-coherent) stores, completed before the
  // workgroup's arrival is counted
#pragma unroll
  for (int j = 0; j < MX; j++) {
    const int64_t m = (int64_t)lg * (4 / R) + j;
    if (live && m < a.M) {
      float* dst = a.part + (ks * a.M + m) * a.Npad + n;
      if (IPART) __hip_atomic_store((int*)dst, iacc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else __hip_atomic_store(dst, acc[j], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.cnt + 16 + rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_last != (uint32_t)(a.KS - 1)) return;
  // last arrival: add the slices in order (coherent loads) and store
#pragma unroll
  for (int j = 0; j < MX; j++) {
    const int64_t m = (int64_t)lg * (4 / R) + j;
    if (live && m < a.M && n < a.N) {
      float f = 0.f;
      int iv = 0;
      for (int64_t k2 = 0; k2 < a.KS; k2++) {
        float* src = a.part + (k2 * a.M + m) * a.Npad + n;
        if (IPART) iv += __hip_atomic_load((int*)src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else f += __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      store(m, n, f, iv);
    }
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.cnt + 16 + rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int FMT, int XK, int MX, int YK, int QM>
__global__ __launch_bounds__(64 * kMaxW) void gemv_mfma(FArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  gemv_item<FMT, XK, MX, YK, QM, false, false>(a, blockIdx.x, smem, nullptr, 0, nullptr);
}

// Persistent kernel over a chain of batch-1 products (items of product s
// are [first[s], first[s+1]) in a global order that every workgroup walks
// with stride gridDim.x).  done[s] counts finished items of product s; a
// product marked `wait` reads its activations only after done[s-1] reaches
// the previous product's item count.  Workgroups never wait on an item
// later in the order than their own, and the grid is co-resident
// (cooperative launch), so every wait ends; a wait is nevertheless bounded
// by kChainSpinLimit.  The last workgroup to finish resets the counters.
struct ChainArgs {
  const FArgs* args;       // [S]
  const int64_t* first;    // [S + 1]
  const int32_t* wait;     // [S]
  uint32_t* done;          // [S], zero between launches
  uint32_t* finished;      // workgroups done, zero between launches
  uint32_t* err;           // set when a wait gave up
  int S;
};

template <int FMT, int XK, int YK, int QM>
__global__ __launch_bounds__(64 * kMaxW) __attribute__((amdgpu_waves_per_eu(2))) void gemv_chain(ChainArgs c) {
  extern __shared__ __align__(16) uint8_t smem[];
  const int64_t total = c.first[c.S];
  int s = 0;
  for (int64_t i = blockIdx.x; i < total; i += gridDim.x) {
    while (i >= c.first[s + 1]) s++;
    const FArgs a = c.args[s];
    const bool wt = s > 0 && c.wait[s] != 0;
    __syncthreads();  // the previous item's LDS reads are over
    if (wt)
      gemv_item<FMT, XK, 1, YK, QM, true, true>(a, i - c.first[s], smem, c.done + s - 1,
                                                (uint32_t)(c.first[s] - c.first[s - 1]), c.err);
    else
      gemv_item<FMT, XK, 1, YK, QM, true, false>(a, i - c.first[s], smem, nullptr, 0u, c.err);
    __builtin_amdgcn_s_waitcnt(0);  // this item's stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_fetch_add(c.done + s, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(c.finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      for (int k = 0; k < c.S; k++)
        __hip_atomic_store(c.done + k, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(c.finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

struct Plan {
  int64_t NB, NRG, G, GQ, GP, KS, Npad, MA;
  int R, W, QM;
  size_t lds, part_off, bytes;
};

int split_terms(int xkind) { return xkind == XK_F32 ? kSplitF32 : kSplitBF16; }

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

constexpr int kQuadsBinary = 16;   // quads a wave keeps in registers (binary)
constexpr int kQuadsTernary = 10;  // (2-bit ternary: twice the code bytes)

Plan make_plan(int fmt, int64_t N, int64_t K, int64_t M, int xkind) {
  Plan p;
  p.R = split_terms(xkind);
  p.MA = M * p.R;
  p.NB = cdiv(N, 16);
  p.G = K / kGroup;
  p.GQ = cdiv(p.G, 4);
  p.GP = cdiv(p.G, 2);
  p.QM = fmt == 1 ? kQuadsBinary : kQuadsTernary;
  // staged activations of a slice stay within 48 KiB of LDS
  int64_t qcap = std::min<int64_t>(p.QM, std::max<int64_t>(1, (48 * 1024) / (16 * p.MA * 33)));
  if (fmt == 3) {
    // base-3 slices are whole octets (pairs of quads)
    qcap = std::max<int64_t>(2, qcap & ~int64_t(1));
    p.KS = cdiv(cdiv(p.GQ, 2), qcap / 2);
  } else {
    p.KS = cdiv(p.GQ, qcap);
  }
  // 4 waves per workgroup: 64 rows share one staged slice, and the slice's
  // activation loads fit in the hoisted staging rounds
  p.W = kMaxW;
  p.NRG = cdiv(p.NB, p.W);
  const int64_t qmax = fmt == 3 ? 2 * cdiv(cdiv(p.GQ, 2), p.KS) : cdiv(p.GQ, p.KS);
  p.lds = (size_t)qmax * 16 * p.MA * 32 + (size_t)qmax * 16 * p.MA + 48 + (fmt == 3 ? 1024 : 0);
  p.Npad = p.NRG * p.W * 16;
  p.part_off = kCounterBytes;
  p.bytes = p.part_off + align256((size_t)(p.KS > 1 ? p.KS : 0) * M * p.Npad * 4);
  return p;
}

template <int FMT, int XK, int MX, int QM>
hipError_t launch_y(const GemvArgs& g, const FArgs& k, dim3 grid, dim3 block, size_t lds,
                    hipStream_t s) {
  if (g.ykind == YK_F32)
    hipLaunchKernelGGL((gemv_mfma<FMT, XK, MX, YK_F32, QM>), grid, block, lds, s, k);
  else if (g.ykind == YK_BF16)
    hipLaunchKernelGGL((gemv_mfma<FMT, XK, MX, YK_BF16, QM>), grid, block, lds, s, k);
  else
    hipLaunchKernelGGL((gemv_mfma<FMT, XK, MX, YK_I32, QM>), grid, block, lds, s, k);
  return hipGetLastError();
}

template <int FMT, int QM>
hipError_t launch_x(const GemvArgs& g, const FArgs& k, dim3 grid, dim3 block, size_t lds,
                    hipStream_t s) {
  if (g.xkind == XK_F32) return launch_y<FMT, XK_F32, 1, QM>(g, k, grid, block, lds, s);
  if (g.xkind == XK_I8)
    return g.M == 1 ? launch_y<FMT, XK_I8, 1, QM>(g, k, grid, block, lds, s)
                    : launch_y<FMT, XK_I8, 2, QM>(g, k, grid, block, lds, s);
  return g.M == 1 ? launch_y<FMT, XK_BF16, 1, QM>(g, k, grid, block, lds, s)
                  : launch_y<FMT, XK_BF16, 2, QM>(g, k, grid, block, lds, s);
}

}  // namespace

size_t gemv_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t M, int xkind) {
  return make_plan(fmt, N, K, M, xkind).bytes;
}

hipError_t launch_gemv_mfma(const GemvArgs& g, hipStream_t s) {
  const Plan p = make_plan(g.fmt, g.N, g.K, g.M, g.xkind);
  if (p.NRG > kMaxRowGroups || p.lds > 64 * 1024) return hipErrorInvalidValue;
  FArgs k;
  k.pcodes = (const uint8_t*)g.pcodes;
  k.pscales = g.pscales;
  k.x = g.x;
  k.x_scales = g.x_scales;
  k.y = g.y;
  k.part = (float*)((uint8_t*)g.ws + p.part_off);
  k.cnt = (uint32_t*)g.ws;
  k.N = g.N;
  k.K = g.K;
  k.G = p.G;
  k.GQ = p.GQ;
  k.GP = p.GP;
  k.M = g.M;
  k.MA = p.MA;
  k.NB = p.NB;
  k.KS = p.KS;
  k.Npad = p.Npad;
  k.x_scale = g.x_scale;
  k.xkind = g.xkind;
  const dim3 grid((unsigned)(p.NRG * p.KS)), block((unsigned)(64 * p.W));
  if (g.fmt == 1) return launch_x<1, kQuadsBinary>(g, k, grid, block, p.lds, s);
  if (g.fmt == 2) return launch_x<2, kQuadsTernary>(g, k, grid, block, p.lds, s);
  if (g.fmt == 3) return launch_x<3, kQuadsTernary>(g, k, grid, block, p.lds, s);
  return hipErrorInvalidValue;
}

// ---------------------------------------------------------------- chains
namespace {

struct ChainPlan {
  void* mem = nullptr;  // descriptors, counters and partial sums (one allocation)
  ChainArgs args;
  const void* kernel = nullptr;
  dim3 grid, block;
  size_t lds = 0;
  int device = 0;
  uint32_t* err = nullptr;
};

template <int FMT, int XK>
const void* chain_kernel(int ykind) {
  constexpr int QM = FMT == 1 ? kQuadsBinary : kQuadsTernary;
  if (ykind == YK_BF16) return (const void*)gemv_chain<FMT, XK, YK_BF16, QM>;
  return (const void*)gemv_chain<FMT, XK, YK_F32, QM>;
}

}  // namespace

hipError_t chain_create(const ChainStage* st, int S, int xkind, int ykind, void** out) {
  *out = nullptr;
  if (S < 1) return hipErrorInvalidValue;
  const int fmt = st[0].fmt;
  std::vector<FArgs> args(S);
  std::vector<int64_t> first(S + 1, 0);
  std::vector<int32_t> wait(S, 0);
  std::vector<int64_t> cnt_off(S), part_off(S);
  int64_t cnt_words = 16, part_floats = 0;
  size_t lds = 0;
  for (int i = 0; i < S; i++) {
    if (st[i].fmt != fmt) return hipErrorInvalidValue;
    const Plan p = make_plan(fmt, st[i].N, st[i].K, 1, xkind);
    if (p.lds > 64 * 1024) return hipErrorInvalidValue;
    lds = std::max(lds, p.lds);
    first[i + 1] = first[i] + p.NRG * p.KS;
    wait[i] = st[i].wait_prev ? 1 : 0;
    cnt_off[i] = cnt_words;
    cnt_words += p.NRG;
    part_off[i] = part_floats;
    if (p.KS > 1) part_floats += p.KS * p.Npad;
    FArgs& k = args[i];
    k.pcodes = (const uint8_t*)st[i].pcodes;
    k.pscales = st[i].pscales;
    k.x = st[i].x;
    k.x_scales = nullptr;
    k.y = st[i].y;
    k.N = st[i].N;
    k.K = st[i].K;
    k.G = p.G;
    k.GQ = p.GQ;
    k.GP = p.GP;
    k.M = 1;
    k.MA = p.MA;
    k.NB = p.NB;
    k.KS = p.KS;
    k.Npad = p.Npad;
    k.x_scale = 1.0f;
    k.xkind = xkind;
  }
  if (first[S] > 0x7FFFFFFF || cnt_words > 0x7FFFFFFF) return hipErrorInvalidValue;
  // layout of the one allocation
  const size_t o_args = 0;
  const size_t o_first = align256(o_args + sizeof(FArgs) * S);
  const size_t o_wait = align256(o_first + sizeof(int64_t) * (S + 1));
  const size_t o_done = align256(o_wait + sizeof(int32_t) * S);
  const size_t o_fin = align256(o_done + sizeof(uint32_t) * S);
  const size_t o_cnt = align256(o_fin + 2 * sizeof(uint32_t));
  const size_t o_part = align256(o_cnt + sizeof(uint32_t) * cnt_words);
  const size_t bytes = o_part + sizeof(float) * (size_t)part_floats;

  ChainPlan* c = new ChainPlan;
  hipError_t e = hipGetDevice(&c->device);
  if (e == hipSuccess) e = hipMalloc(&c->mem, bytes);
  if (e != hipSuccess) {
    delete c;
    return e;
  }
  uint8_t* m = (uint8_t*)c->mem;
  for (int i = 0; i < S; i++) {
    args[i].cnt = (uint32_t*)(m + o_cnt) + cnt_off[i] - 16;
    args[i].part = (float*)(m + o_part) + part_off[i];
  }
  // counters start at zero; every launch leaves them zero
  e = hipMemset(m + o_done, 0, o_part - o_done);
  if (e == hipSuccess) e = hipMemcpy(m + o_args, args.data(), sizeof(FArgs) * S, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(m + o_first, first.data(), sizeof(int64_t) * (S + 1), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(m + o_wait, wait.data(), sizeof(int32_t) * S, hipMemcpyHostToDevice);
  if (e == hipSuccess) {
    if (fmt == 1) c->kernel = xkind == XK_F32 ? chain_kernel<1, XK_F32>(ykind) : chain_kernel<1, XK_BF16>(ykind);
    else if (fmt == 2) c->kernel = xkind == XK_F32 ? chain_kernel<2, XK_F32>(ykind) : chain_kernel<2, XK_BF16>(ykind);
    else if (fmt == 3) c->kernel = xkind == XK_F32 ? chain_kernel<3, XK_F32>(ykind) : chain_kernel<3, XK_BF16>(ykind);
    else e = hipErrorInvalidValue;
  }
  int per_cu = 0, cus = 0;
  if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, c->kernel, 64 * kMaxW, lds);
  if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, c->device);
  if (e == hipSuccess && per_cu < 1) e = hipErrorInvalidConfiguration;
  if (e != hipSuccess) {
    (void)hipFree(c->mem);
    delete c;
    return e;
  }
  const int64_t want = (int64_t)per_cu * cus;
  c->grid = dim3((unsigned)std::min<int64_t>(want, first[S]));
  c->block = dim3(64 * kMaxW);
  c->lds = lds;
  c->args.args = (const FArgs*)(m + o_args);
  c->args.first = (const int64_t*)(m + o_first);
  c->args.wait = (const int32_t*)(m + o_wait);
  c->args.done = (uint32_t*)(m + o_done);
  c->args.finished = (uint32_t*)(m + o_fin);
  c->args.err = (uint32_t*)(m + o_fin) + 1;
  c->args.S = S;
  c->err = c->args.err;
  *out = c;
  return hipSuccess;
}

hipError_t chain_run(void* plan, hipStream_t s) {
  ChainPlan* c = (ChainPlan*)plan;
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev != c->device) return hipErrorInvalidDevice;
  void* kargs[] = {&c->args};
  return hipLaunchCooperativeKernel(c->kernel, c->grid, c->block, kargs, (unsigned)c->lds, s);
}

hipError_t chain_status(void* plan, int* failed_waits) {
  ChainPlan* c = (ChainPlan*)plan;
  uint32_t v = 0;
  hipError_t e = hipMemcpy(&v, c->err, sizeof(v), hipMemcpyDeviceToHost);
  *failed_waits = (int)v;
  return e;
}

void chain_destroy(void* plan) {
  ChainPlan* c = (ChainPlan*)plan;
  if (!c) return;
  (void)hipFree(c->mem);
  delete c;
}

hipError_t launch_gemv_sign(const SignArgs& g, hipStream_t s);

}  // namespace lowbit

namespace lowbit {
namespace {
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

}  // namespace

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
