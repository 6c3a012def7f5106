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
// products reduce to adds and sign flips: section "精度保留了多少" of the
// page "三值权重压缩：27B模型缩至6GB，可在浏览器本地运行").
//
// Sign path (binary weights x sign activations): per 32 weights one XOR and
// one popcount give the exact signed agreement 32 - 2 * popcount(w ^ x)
// (the XOR + popcount remark of section "1-bit 嘅數學：點解唔爆鑊？" of the
// page "瀏覽器生圖技術內幕：1-bit diffusion 點樣將 3GB 模型塞入 WebGPU？").
#include <algorithm>
#include <vector>

#include "common.hpp"
#include "fp4.hpp"

namespace lowbit {
namespace {

constexpr int kMaxWaves = 16;  // waves per workgroup of the sign kernel
constexpr uint32_t kChainSpinLimit = 1u << 24;  // sleeps before a chain wait gives up
constexpr int kMaxW = 4;       // waves (row-blocks) per MFMA workgroup, at most
constexpr int kQuadsMulti = 4;      // quads per slice of the several-row streaming kernel
constexpr int kQuadsMultiMid = 5;   // (the same with at most 15 rows of A, not base-3)
constexpr int kQuadsMultiWide = 6;  // (the same with at most 10 rows of A)
// rows of A the image buffers of a several-row streaming kernel with QM-quad
// slices hold (a slice image travels in at most ten 16-byte registers per
// thread; two workgroups' buffers fit a CU)
constexpr int multi_max_ma(int qm) { return qm == kQuadsMultiWide ? 10 : qm == kQuadsMultiMid ? 15 : 16; }
// dynamic LDS of the one-product kernel and the waiting chain: two
// workgroups per CU fit in the 160 KiB of a gfx950 CU
constexpr size_t kLdsCap = 80 * 1024;

// Operand scheme of the activations for weight format FMT and activation kind
// XK (split_terms): R terms, kShift binades apart, the block maximum scaled
// into [2^kTop, 2^(kTop+1)), A format kFmtA (0 = fp8 e4m3, 1 = bf8 e5m2).
// kCheck: how staging verifies that the terms carry the activations
// accurately enough -- 0: not needed (int8 is exact; binary rows with bf16
// are within 2^-21 of the block maximum, which every binary row weighs);
// ternary rows may weigh any subset of a block, so every element must be
// carried: 1 (bf16) exactly, 3 (fp32) within 2^-12 of itself; 2 (binary,
// fp32): the block's summed error within 2^-14 of its maximum.
template <int FMT, int XK>
struct XSplit {
  static constexpr bool kBF8 = XK == XK_BF16 && FMT != 1;
  // kCheck 1: three round-to-nearest-even bf8 terms, 3 binades apart, carry
  // every bf16 value of scaled magnitude 2^-13 or more exactly (checked over
  // every 8-bit significand at every exponent; the bound holds whether or not
  // the conversion keeps subnormal results), so a scaled magnitude below it
  // is what staging flags
  static constexpr float kMinExact = 0x1p-13f;
  static constexpr int R = split_terms(FMT, XK);
  static constexpr int kShift = kBF8 ? 3 : 4;
  static constexpr int kTop = kBF8 ? 14 : 7;
  static constexpr int kFmtA = kBF8 ? 1 : 0;
  static constexpr int kCheck = XK == XK_I8 ? 0 : FMT != 1 ? (XK == XK_F32 ? 3 : 1) : XK == XK_F32 ? 2 : 0;
};
constexpr float kStageEps = 1.0f / 4096.0f;  // 2^-12: staging error allowed per element

// Correction lists of the one-row kernels (ternary weights, bf16
// activations): the split terms carry every element within 2^27 of its
// block's maximum exactly; an element further below is listed with its
// exact residual rho = x - (what the terms carry), and the item adds
// scale x code x rho for it after its MFMAs.  Per wave a count word and up
// to kListEntries entries {slot position, rho}; a wave whose list
// overflows flags the slice for the exact recomputation.
constexpr int kListEntries = 15;
constexpr int kListWaveWords = 2 + 2 * kListEntries;  // 32
constexpr int kListBytes = 4 * kListWaveWords * kMaxW;  // 512

// two floats -> two fp8 / bf8 bytes (round to nearest even) in half HI of old
template <int FA, bool HI>
__device__ __attribute__((always_inline)) inline uint32_t cvt_pk8(float a, float b, uint32_t old) {
  if constexpr (FA == 0) return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
  else return __builtin_amdgcn_cvt_pk_bf8_f32(a, b, old, HI);
}
// the four fp8 / bf8 bytes of w as floats (exact)
template <int FA>
__device__ __attribute__((always_inline)) inline void cvt_f32x4(uint32_t w, float* d) {
  if constexpr (FA == 0) {
    d[0] = __builtin_amdgcn_cvt_f32_fp8(w, 0); d[1] = __builtin_amdgcn_cvt_f32_fp8(w, 1);
    d[2] = __builtin_amdgcn_cvt_f32_fp8(w, 2); d[3] = __builtin_amdgcn_cvt_f32_fp8(w, 3);
  } else {
    d[0] = __builtin_amdgcn_cvt_f32_bf8(w, 0); d[1] = __builtin_amdgcn_cvt_f32_bf8(w, 1);
    d[2] = __builtin_amdgcn_cvt_f32_bf8(w, 2); d[3] = __builtin_amdgcn_cvt_f32_bf8(w, 3);
  }
}

template <int T, int FA = 0>
__device__ inline v4f mfma_group(const v8i& A, const v8i& B, int sa) {
  const v4f zero = {0.f, 0.f, 0.f, 0.f};
  // A: fp8 e4m3 (0) or bf8 e5m2 (1), B: fp4 e2m1 (4); byte T of sa is the A
  // block exponent, B is unscaled (E8M0 127 = 2^0)
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, zero, FA, 4, T, sa, 0, 127);
}

// mfma_group for a run-time group index t
template <int FA>
__device__ __attribute__((always_inline)) inline v4f mfma_group_t(int t, const v8i& A, const v8i& B, int sa) {
  return t == 0 ? mfma_group<0, FA>(A, B, sa) : t == 1 ? mfma_group<1, FA>(A, B, sa)
       : t == 2 ? mfma_group<2, FA>(A, B, sa) : mfma_group<3, FA>(A, B, sa);
}

__device__ inline uint32_t bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// ------------------------------------------------------- activation staging
// The MFMA multiplies fp4 weights (exactly +-1 / 0) by activations given as
// fp8 split terms (XSplit).  For each 32-element hardware block, E is chosen
// so the block maximum scaled by 2^-E lies in [2^kTop, 2^(kTop+1)); term 0
// is the round-to-nearest-even fp8 (e4m3) or bf8 (e5m2) value of v, each
// next term that of 2^kShift x the remaining residual, and term r carries
// the E8M0 block exponent E - kShift r, applied inside the MFMA.  int8
// values q are split exactly as 16 * (q >> 4) + (q & 15).  The conversions
// use the hardware v_cvt_pk_{fp8,bf8}_f32 / v_cvt_f32_{fp8,bf8} (OCP
// formats, round to nearest even, subnormals kept).
//
// Staging also reconstructs every element from its terms (exact in fp32) and
// flags the slice when an element misses the accuracy XSplit::kCheck asks
// for: a block spanning more than the terms' range (a large element beside
// much smaller ones that a ternary row may weigh alone).  A flagged slice is
// recomputed exactly on the VALU (exact_slice), so every finite input meets
// the product bound; N(0,1) activations never raise the flag.
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
// (A row a = m R + r holds term r of activation row m.)  Images staged into
// global memory are followed by flag words (image_flag_bytes): nonzero when
// the slice must be recomputed exactly.

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
  int epi;        // 1: SiLU-mul epilogue (chains, M = 1)
  const uint8_t* xst;  // one-product kernel, M > 1: the slice images staged once
                       // per call (else null: each workgroup stages its slice)
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

// 16 bytes at byte offset `off` of x (nbytes long) read with a device-coherent
// (sc1) buffer load, for activations another workgroup may just have
// written; offsets past nbytes read zeros.
__device__ __attribute__((always_inline)) inline uint4 coh_load16(const void* x, uint32_t nbytes,
                                                                 uint32_t off) {
  const __amdgpu_buffer_rsrc_t r =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(x), (short)0, (int)nbytes, 0x00020000);
  typedef unsigned v4u_ __attribute__((ext_vector_type(4)));
  const v4u_ v = __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, 16 /* sc1 */);
  return make_uint4(v.x, v.y, v.z, v.w);
}

// raw activations of one unit: bf16 in ra, f32 in ra:rb, int8 in ra.xy.
// The load is unconditional (a unit past the end reads element 0) so that
// no control flow joins wait on it.  COH: device-coherent loads (x of M = 1
// rows shorter than 2^31 bytes).
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
    ra = COH ? coh_load16(a.x, (uint32_t)(a.M * a.K * 2), (uint32_t)(idx * 2)) : *(const uint4*)p;
    rb = ra;
  } else if constexpr (XK == XK_F32) {
    const float* p = (const float*)a.x + idx;
    ra = COH ? coh_load16(a.x, (uint32_t)(a.M * a.K * 4), (uint32_t)(idx * 4)) : *(const uint4*)p;
    rb = COH ? coh_load16(a.x, (uint32_t)(a.M * a.K * 4), (uint32_t)(idx * 4 + 16)) : *(const uint4*)(p + 4);
  } else {
    const uint2 w = *(const uint2*)((const int8_t*)a.x + idx);
    ra = make_uint4(w.x, w.y, w.x, w.y);
    rb = ra;
  }
}

// Convert one round of units into split terms and exponents in LDS (or a
// global image).  Returns true when one of the unit's elements misses the
// accuracy XSplit::kCheck asks for (never for units past the end).  LIST
// (one-row items, kCheck 1): such elements go to the wave's correction list
// wlist instead, and only a full list returns true.
template <int FMT, int XK, bool LIST = false>
__device__ __attribute__((always_inline)) inline bool stage_convert1(const FArgs& a, int64_t q0,
                                                                     int64_t nq, int64_t rd,
                                                                     uint4 ra, uint4 rb,
                                                                     uint8_t* xa, uint8_t* xe,
                                                                     uint32_t* wlist = nullptr) {
  using S = XSplit<FMT, XK>;
  constexpr int R = S::R, FA = S::kFmtA;
  if (rd * blockDim.x >= nq * 64 * a.M) return false;  // uniform: round past the end
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
  if (!inside) return false;
  int E = 0;
  if (XK != XK_I8 && amax != 0.0f) {
    int ex;
    frexpf(amax, &ex);
    E = (ex - 1) - S::kTop;
    const int lo = -127 + S::kShift * (R - 1);  // every term's exponent representable
    if (E < lo) E = lo;
  }
  const int kb = 2 * (b & 1) + (ch >> 1), e = 16 * (b >> 1) + 8 * (ch & 1);
  // tv: the part of v (scaled by 2^-E) the terms still have to carry, times
  // 2^(kShift r) before term r; t0: tv before term 0 (relative check only)
  float tv[8], t0[8];
  uint32_t lost = 0;  // kCheck 3: elements whose scaling by 2^-E underflowed to zero
  bool small = false;  // kCheck 1: a nonzero element below kMinExact
  uint32_t smallbits = 0;  // (LIST) which ones
  float amax_s = 0.f;
  if constexpr (XK == XK_I8) {
#pragma unroll
    for (int j = 0; j < 8; j++) tv[j] = v[j];
  } else {
    // exact power of two: E is clamped to [-127 + kShift (R-1), 127 - kTop]
    const float sc = ldexpf(1.0f, -E);
#pragma unroll
    for (int j = 0; j < 8; j++) {
      tv[j] = v[j] * sc;
      if constexpr (S::kCheck == 1 && LIST) {
        const bool sj = v[j] != 0.0f && fabsf(tv[j]) < S::kMinExact;
        small = small || sj;
        smallbits |= (sj ? 1u : 0u) << j;
      } else if constexpr (S::kCheck == 1) {
        small = small || (v[j] != 0.0f && fabsf(tv[j]) < S::kMinExact);
      }
      if (S::kCheck == 3) lost |= (tv[j] == 0.0f && v[j] != 0.0f) ? 1u : 0u;
      if (S::kCheck == 3) t0[j] = tv[j];
    }
    amax_s = amax * sc;
  }
  uint32_t wr[LIST ? R : 1][2];  // (LIST) the terms' bytes
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
      w0 = cvt_pk8<0, false>(p[0], p[1], 0);
      w0 = cvt_pk8<0, true>(p[2], p[3], w0);
      w1 = cvt_pk8<0, false>(p[4], p[5], 0);
      w1 = cvt_pk8<0, true>(p[6], p[7], w1);
      Er = r == 0 ? 4 : 0;
    } else {
      w0 = cvt_pk8<FA, false>(tv[0], tv[1], 0);
      w0 = cvt_pk8<FA, true>(tv[2], tv[3], w0);
      w1 = cvt_pk8<FA, false>(tv[4], tv[5], 0);
      w1 = cvt_pk8<FA, true>(tv[6], tv[7], w1);
      Er = E - S::kShift * r;
      if (S::kCheck >= 2 || r + 1 < R) {
        float d[8];
        cvt_f32x4<FA>(w0, d);
        cvt_f32x4<FA>(w1, d + 4);
        // residual, exact in fp32: the next term's input (scaled by
        // 2^kShift), or after the last term what the terms miss
#pragma unroll
        for (int j = 0; j < 8; j++) tv[j] = r + 1 < R ? (tv[j] - d[j]) * (float)(1 << S::kShift) : tv[j] - d[j];
      }
    }
    if constexpr (LIST) {
      wr[r][0] = w0;
      wr[r][1] = w1;
    }
    const int64_t arow = m * R + r;
    *(uint2*)(xa + ((ql * 16 + t * 4 + kb) * a.MA + arow) * 32 + e) = make_uint2(w0, w1);
    if (ch == 0) xe[((ql * 4 + b) * a.MA + arow) * 4 + t] = (uint8_t)(127 + Er);
  }
  // tv is now the error in units of the last term's scale, 2^(kShift (R-1))
  // below v's scale: exact comparisons with powers of two
  constexpr float kEpsR = kStageEps * (float)(1 << (S::kShift * (R - 1)));
  bool bad = false;
  if constexpr (S::kCheck == 1 && LIST) {
    if (small) {  // rare: list the elements the terms may not carry exactly
#pragma unroll
      for (int j = 0; j < 8; j++) {
        if ((smallbits >> j) & 1u) {
          // what the terms carry, term by term (each term times its power
          // of two is exact, and for such an element so are the sums)
          float carried = 0.f;
#pragma unroll
          for (int r = 0; r < R; r++) {
            const uint32_t w = wr[r][j >> 2];
            const float d = (j & 3) == 0 ? __builtin_amdgcn_cvt_f32_bf8(w, 0)
                          : (j & 3) == 1 ? __builtin_amdgcn_cvt_f32_bf8(w, 1)
                          : (j & 3) == 2 ? __builtin_amdgcn_cvt_f32_bf8(w, 2)
                                         : __builtin_amdgcn_cvt_f32_bf8(w, 3);
            carried += d * ldexpf(1.0f, E - S::kShift * r);
          }
          const float rho = v[j] - carried;
          if (rho != 0.0f) {
            const uint32_t idx = atomicAdd(wlist, 1u);
            if (idx < (uint32_t)kListEntries) {
              const uint32_t pos = (uint32_t)(8 * ch + j) | ((uint32_t)b << 5) | ((uint32_t)t << 7) |
                                   ((uint32_t)ql << 9);
              *(uint2*)(wlist + 2 + 2 * idx) = make_uint2(pos, __float_as_uint(rho));
            } else {
              bad = true;
            }
          }
        }
      }
    }
  } else if constexpr (S::kCheck == 1) {
    bad = small;
  } else if constexpr (S::kCheck == 3) {
    bad = lost != 0;
#pragma unroll
    for (int j = 0; j < 8; j++) bad = bad || fabsf(tv[j]) > kEpsR * fabsf(t0[j]);
  } else if constexpr (S::kCheck == 2) {
    float err = 0.f;
#pragma unroll
    for (int j = 0; j < 8; j++) err += fabsf(tv[j]);
    bad = err > 0.25f * kEpsR * amax_s;  // the block's four units: at most eps x its maximum
  }
  return bad;
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

// Geometry of one work item: row group rg (W row-blocks, one per wave) and
// K-slice ks of quads [q0, q1) (base-3 slices are whole octets).
struct Item {
  int64_t rg, ks, q0, rb;
  int nq;
  bool live;
};

template <int FMT>
__device__ __attribute__((always_inline)) inline Item item_of(const FArgs& a, int64_t blk) {
  Item it;
  const int W = blockDim.x >> 6, w = threadIdx.x >> 6;
  it.rg = blk / a.KS;
  it.ks = blk % a.KS;
  const int64_t GO = cdiv(a.GQ, 2);
  it.q0 = FMT == 3 ? 2 * (GO * it.ks / a.KS) : a.GQ * it.ks / a.KS;
  const int64_t q1 = FMT == 3 ? min<int64_t>(2 * (GO * (it.ks + 1) / a.KS), a.GQ)
                              : a.GQ * (it.ks + 1) / a.KS;
  it.nq = (int)(q1 - it.q0);
  it.rb = (int64_t)W * it.rg + w;
  it.live = it.rb < a.NB;
  return it;
}

// Unconditional loads (the row-block and quad are clamped into the matrix,
// results of clamped loads are never used), so no load waits on another.
template <int FMT>
__device__ __attribute__((always_inline)) inline void load_quad(const FArgs& a, const Item& it,
                                                               int q, Quad<FMT>& o) {
  const int64_t rbc = it.live ? it.rb : a.NB - 1;
  const int64_t gq = min<int64_t>(it.q0 + q, a.GQ - 1);
  load_quad_at<FMT>(a.pcodes, a.pscales, rbc, gq, a.GQ, a.GP, threadIdx.x & 63, o);
}

// Item of row group rg, K-slice ks, for callers that know both: the same
// slicing as item_of with 32-bit divisions only (a product's quads and
// slices fit 32 bits: GQ < 2^28 in every chain).
template <int FMT, int RB = 1>
__device__ __attribute__((always_inline)) inline Item item_at(const FArgs& a, int64_t rg,
                                                              int64_t ks) {
  Item it;
  // the wave index is uniform in the wave: scalar, so that the item's tests
  // are scalar branches
  const int W = blockDim.x >> 6, w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  it.rg = rg;
  it.ks = ks;
  const uint32_t KS = (uint32_t)a.KS, k = (uint32_t)ks;
  // floor(T * k / KS) without a 64-bit product: T = (T / KS) KS + T % KS
  auto split = [&](uint32_t T, uint32_t kk) { return (T / KS) * kk + (T % KS) * kk / KS; };
  uint32_t q0, q1;
  if (FMT == 3) {
    const uint32_t GO = (uint32_t)((a.GQ + 1) / 2);
    q0 = 2 * split(GO, k);
    q1 = min(2 * split(GO, k + 1), (uint32_t)a.GQ);
  } else {
    q0 = split((uint32_t)a.GQ, k);
    q1 = split((uint32_t)a.GQ, k + 1);
  }
  it.q0 = q0;
  it.nq = (int)(q1 - q0);
  it.rb = ((int64_t)W * rg + w) * RB;  // the wave's first row-block
  it.live = it.rb < a.NB;
  return it;
}

// Code and scale addresses of an item's first quad for this lane, so that
// quad q of the item is a fixed offset from them (quads past the item's end
// re-read its last quad).
struct QuadPtr {
  const uint8_t* c;
  const uint8_t* s;
  const uint8_t* c2;  // binary waves of two row-blocks: the second one's codes and scales
  const uint8_t* s2;
  int nq;
  bool p1_last;  // 2-bit: the last quad's second word block is clamped onto its first
};

template <int FMT, int RB = 1>
__device__ __attribute__((always_inline)) inline QuadPtr quad_ptr(const FArgs& a, const Item& it) {
  QuadPtr p;
  const int L = threadIdx.x & 63;
  const int64_t rbc = it.live ? it.rb : a.NB - 1;
  if constexpr (FMT == 1) {
    p.c = a.pcodes + (rbc * a.GQ + it.q0) * 1024 + 16 * L;
  } else if constexpr (FMT == 2) {
    p.c = a.pcodes + (rbc * a.GP + 2 * it.q0) * 1024 + 16 * L;
  } else {
    p.c = a.pcodes + (rbc * ((a.GQ + 1) / 2) + (it.q0 >> 1)) * 3328 + 16 * L;
  }
  const uint8_t* sb = a.pscales ? (const uint8_t*)a.pscales : a.pcodes;
  p.s = sb + ((rbc * a.GQ + it.q0) * 16 + (L & 15)) * 8;
  if constexpr (RB == 2) {
    static_assert(FMT == 1, "two row-blocks per wave: binary only");
    const int64_t rbc2 = it.rb + 1 < a.NB ? it.rb + 1 : rbc;  // past the end: a dummy re-read
    p.c2 = a.pcodes + (rbc2 * a.GQ + it.q0) * 1024 + 16 * L;
    p.s2 = sb + ((rbc2 * a.GQ + it.q0) * 16 + (L & 15)) * 8;
  } else {
    p.c2 = p.c;
    p.s2 = p.s;
  }
  p.nq = it.nq;
  p.p1_last = 2 * (it.q0 + it.nq - 1) + 1 >= a.GP;
  return p;
}

// quad q of an item through its QuadPtr (the same words as load_quad)
template <int FMT>
__device__ __attribute__((always_inline)) inline void load_quad_p(const QuadPtr& p, int q,
                                                                 Quad<FMT>& o) {
  const int qq = q < p.nq ? q : p.nq - 1;
  if constexpr (FMT == 1) {
    o.w[0] = __builtin_nontemporal_load((const u4*)(p.c + qq * 1024));
  } else if constexpr (FMT == 2) {
    const uint8_t* c = p.c + qq * 2048;
    o.w[0] = __builtin_nontemporal_load((const u4*)c);
    o.w[1] = __builtin_nontemporal_load((const u4*)(c + (p.p1_last && qq == p.nq - 1 ? 0 : 1024)));
  } else {
    // octet block qq / 2 (item slices start on whole octets), half h = qq % 2
    const uint8_t* lp = p.c + (qq >> 1) * 3328;
    const int h = qq & 1;
    o.c30 = __builtin_nontemporal_load((const u2*)(lp + (h ? 1024 + 8 : 0)));
    o.c31 = __builtin_nontemporal_load((const u2*)(lp + (h ? 2048 : 8)));
    o.c32 = __builtin_nontemporal_load((const u2*)(lp + (h ? 2048 + 8 : 1024)));
    const int L = threadIdx.x & 63;
    o.t3 = __builtin_nontemporal_load((const uint32_t*)(lp - 16 * L + 3072 + 4 * L)) >> (16 * h);
  }
  o.sc = *(const uint2*)(p.s + qq * 128);
}

// quad q of both row-blocks of a binary wave that holds two
__device__ __attribute__((always_inline)) inline void load_quad_p2(const QuadPtr& p, int q,
                                                                  Quad<1>& o, Quad<1>& o2) {
  const int qq = q < p.nq ? q : p.nq - 1;
  o.w[0] = __builtin_nontemporal_load((const u4*)(p.c + qq * 1024));
  o2.w[0] = __builtin_nontemporal_load((const u4*)(p.c2 + qq * 1024));
  o.sc = *(const uint2*)(p.s + qq * 128);
  o2.sc = *(const uint2*)(p.s2 + qq * 128);
}

// Binary waves of three row-blocks address codes and scales through buffer
// resources with wave-uniform offsets (scalar registers): only the lane's
// fixed offset stays in a vector register, which leaves the registers a
// wave needs for three row-blocks of ten quads in flight.  Every stage's
// codes and scales are shorter than 2^31 bytes.
struct QuadBuf {
  __amdgpu_buffer_rsrc_t rc, rs;
  int32_t oc, oc2, oc3, os, os2, os3;  // byte offsets of the item's first quad
  int nq;
};

__device__ __attribute__((always_inline)) inline QuadBuf quad_buf3(const FArgs& a, const Item& it) {
  QuadBuf p;
  const int64_t rbc = it.live ? it.rb : a.NB - 1;
  const int64_t rbc2 = it.rb + 1 < a.NB ? it.rb + 1 : rbc;  // past the end: a dummy re-read
  const int64_t rbc3 = it.rb + 2 < a.NB ? it.rb + 2 : rbc;
  const uint8_t* sb = a.pscales ? (const uint8_t*)a.pscales : a.pcodes;
  p.rc = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(a.pcodes), (short)0,
                                           (int)(a.NB * a.GQ * 1024), 0x00020000);
  p.rs = __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(sb), (short)0,
                                           (int)(a.NB * a.GQ * 128), 0x00020000);
  p.oc = (int32_t)((rbc * a.GQ + it.q0) * 1024);
  p.oc2 = (int32_t)((rbc2 * a.GQ + it.q0) * 1024);
  p.oc3 = (int32_t)((rbc3 * a.GQ + it.q0) * 1024);
  p.os = (int32_t)((rbc * a.GQ + it.q0) * 128);
  p.os2 = (int32_t)((rbc2 * a.GQ + it.q0) * 128);
  p.os3 = (int32_t)((rbc3 * a.GQ + it.q0) * 128);
  p.nq = it.nq;
  return p;
}

// quad q of the three row-blocks (the words load_quad_p2 reads for two);
// vc = 16 * lane, vs = 8 * (lane % 16).  Codes stream past the caches
// (non-temporal), as in load_quad_p2.
__device__ __attribute__((always_inline)) inline void load_quad_b3(const QuadBuf& p, int q,
                                                                  int vc, int vs, Quad<1>& o,
                                                                  Quad<1>& o2, Quad<1>& o3) {
  constexpr int kNT = 2;  // cache policy: non-temporal
  const int qq = q < p.nq ? q : p.nq - 1;
  o.w[0] = __builtin_amdgcn_raw_buffer_load_b128(p.rc, vc, p.oc + qq * 1024, kNT);
  o2.w[0] = __builtin_amdgcn_raw_buffer_load_b128(p.rc, vc, p.oc2 + qq * 1024, kNT);
  o3.w[0] = __builtin_amdgcn_raw_buffer_load_b128(p.rc, vc, p.oc3 + qq * 1024, kNT);
  const u2 s1 = __builtin_amdgcn_raw_buffer_load_b64(p.rs, vs, p.os + qq * 128, 0);
  const u2 s2 = __builtin_amdgcn_raw_buffer_load_b64(p.rs, vs, p.os2 + qq * 128, 0);
  const u2 s3 = __builtin_amdgcn_raw_buffer_load_b64(p.rs, vs, p.os3 + qq * 128, 0);
  o.sc = make_uint2(s1.x, s1.y);
  o2.sc = make_uint2(s2.x, s2.y);
  o3.sc = make_uint2(s3.x, s3.y);
}

// LDS of an item: staged activations (and, when copied from a global image,
// its flag words), a zero block with per-wave staging flags, the base-3 table
struct Lds {
  uint8_t* xa;
  uint8_t* xe;
  uint32_t* list;  // one-row ternary staging: the waves' correction lists
  uint8_t* zblk;   // 32 zero bytes, a word of unit exponents, then wflag
  uint32_t* wflag;  // [kMaxW]: the wave's last staging found an inaccurate element
  uint32_t* t3;
};

// bytes of the zero block and flags ahead of the base-3 table
constexpr int kZeroBlock = 64;

// bytes of the flag words that follow a slice image staged into global memory
// by `rounds` staging rounds (one word per round, padded to 16 bytes)
__host__ __device__ inline int64_t image_flag_bytes(int64_t rounds) { return (4 * rounds + 15) / 16 * 16; }

// staging rounds of a slice of nq quads and M rows (256 threads)
__host__ __device__ inline int64_t slice_rounds(int64_t nq, int64_t M) { return (nq * 64 * M + 255) / 256; }

__device__ __attribute__((always_inline)) inline Lds lds_of(const FArgs& a, uint8_t* smem, int nq,
                                                            int64_t extra = 0) {
  Lds l;
  l.xa = smem;
  l.xe = smem + (int64_t)nq * 16 * a.MA * 32;
  l.list = (uint32_t*)(l.xe + (int64_t)nq * 16 * a.MA + extra);
  l.zblk = (uint8_t*)l.list + kListBytes;
  l.wflag = (uint32_t*)(l.zblk + 48);
  l.t3 = (uint32_t*)(l.zblk + kZeroBlock);
  return l;
}

// 32 zero bytes + one word of unit exponents (read by lanes that hold no
// activation row: their A operand is zero); base-3: byte value -> its 5
// trits as fp4 nibbles (trit 0 -> -1 = 0xA, 1 -> 0, 2 -> +1 = 0x2), nibble e
// = trit e (least significant first)
template <int FMT, int TS = 1>
__device__ __attribute__((always_inline)) inline void lds_init(const Lds& l) {
  if (threadIdx.x < 9) ((uint32_t*)l.zblk)[threadIdx.x] = threadIdx.x < 8 ? 0u : 0x7F7F7F7Fu;
  if constexpr (FMT == 3) fill_trit_table<TS>(l.t3, (int)blockDim.x);
}

// copies of the base-3 table: the one-row kernels keep one per bank
// (lookups spread over the banks) in the LDS their small slice images leave
// free (16 copies: three workgroups of the streaming kernel still fit a CU)
constexpr int kTritCopies = 16;
template <int FMT, bool ONE_ROW>
constexpr int trit_copies() { return FMT == 3 && ONE_ROW ? kTritCopies : 1; }

// this wave's staging flag: lane 0 writes whether any lane saw an inaccurate element
__device__ __attribute__((always_inline)) inline void put_wave_flag(uint32_t* wflag, bool bad) {
  const bool any = __builtin_amdgcn_ballot_w64(bad) != 0;
  if ((threadIdx.x & 63) == 0) wflag[threadIdx.x >> 6] = any ? 1u : 0u;
}

// OR of the W waves' flags (after a barrier), uniform
__device__ __attribute__((always_inline)) inline bool get_flags(const uint32_t* w, int n) {
  uint32_t f = 0;
  for (int i = 0; i < n; i++) f |= w[i];
  return __builtin_amdgcn_readfirstlane(f) != 0;
}

// the 4 groups of quad q: operands first, then 4 independent MFMAs, then the
// per-group scale epilogues (padding groups have zero activations).  Several
// activation rows (MM > 1): each lane keeps one accumulator per A row it
// receives (rows 4 lg .. 4 lg + 3) and gather_rows adds the R term rows of
// every activation row afterwards.  One row (MM = 1): the R term rows sit in
// the lane's first R slots and are added before the scale is applied, in
// the order quad_mfma_m1 uses (the chains and the one-product kernel agree
// bit for bit).  (BATCH groups at a time: 4 gives the most independent
// MFMAs, 2 fewer live registers)
template <int FMT, int XK, int MM, int BATCH = 4, int TS = 1>
__device__ __attribute__((always_inline)) inline void quad_mfma(const FArgs& a, const Lds& l, int q,
                                                                const Quad<FMT>& qd,
                                                                float (&acc)[4], int (&iacc)[4]) {
  constexpr int FA = XSplit<FMT, XK>::kFmtA;
  constexpr bool INTC = XK == XK_I8;
  const int L = threadIdx.x & 63, r = L & 15, lg = L >> 4;
  const uint32_t* t3 = l.t3 + L % TS;
  const bool arow = r < a.MA;
  const uint32_t se = *(const uint32_t*)(arow ? l.xe + ((q * 4 + lg) * a.MA + r) * 4 : l.zblk + 32);
  const bool unit_scales = a.pscales == nullptr;
#pragma unroll
  for (int t0 = 0; t0 < 4; t0 += BATCH) {
    v8i A[BATCH], B[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; u++) {
      const int t = t0 + u;
      const uint4* src = (const uint4*)(arow ? l.xa + ((q * 16 + t * 4 + lg) * a.MA + r) * 32 : l.zblk);
      const uint4 x0 = src[0], x1 = src[1];
      A[u] = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
      B[u] = decode_group<FMT, TS>(qd, t, t3);
    }
    v4f c[BATCH];
#pragma unroll
    for (int u = 0; u < BATCH; u++) c[u] = mfma_group_t<FA>(t0 + u, A[u], B[u], (int)se);
#pragma unroll
    for (int u = 0; u < BATCH; u++) {
      const int t = t0 + u;
      const float s = unit_scales ? 1.0f : f16_bits_to_f32((t < 2 ? qd.sc.x : qd.sc.y) >> (16 * (t & 1)));
      if constexpr (MM == 1) {
        constexpr int R = XSplit<FMT, XK>::R;
        float tsum = c[u][0];
#pragma unroll
        for (int i = 1; i < R; i++) tsum += c[u][i];
        acc[0] = fmaf(s, tsum, acc[0]);
        if (INTC) iacc[0] += __float2int_rn(tsum);
      } else {
#pragma unroll
        for (int v = 0; v < 4; v++) {
          acc[v] = fmaf(s, c[u][v], acc[v]);
          if (INTC) iacc[v] += __float2int_rn(c[u][v]);
        }
      }
    }
  }
}

// Activation row m's value from per-A-row accumulators (quad_mfma): the sum,
// in term order, of A rows m R .. m R + R - 1, which lane group (m R + r) / 4
// holds in slot (m R + r) % 4.  Every lane calls it; the result is valid in
// lanes 0..15 (lane r = output row r of the row-block).
template <int R, int MM, typename T>
__device__ __attribute__((always_inline)) inline void gather_rows(const T (&acc)[4], T (&ym)[MM]) {
  if constexpr (MM == 1) {  // one row: quad_mfma added its terms already
    ym[0] = acc[0];
    return;
  }
#pragma unroll
  for (int m = 0; m < MM; m++) ym[m] = 0;
#pragma unroll
  for (int ar = 0; ar < MM * R; ar++) {
    const int v = ar & 3, lgs = ar >> 2;
    const T val = lgs == 0 ? acc[v] : __shfl_down(acc[v], 16 * lgs);
    ym[ar / R] += val;
  }
}

// 8 consecutive activations of row m from k0 as floats (bf16: one 16-byte
// load, fp32: two); COH: device-coherent loads (activations another
// workgroup may just have written; the row must lie within the first 2^31
// bytes of x)
template <int XK>
__device__ __attribute__((always_inline)) inline void load_x8(const FArgs& a, int64_t m, int64_t k0,
                                                              bool coh, float (&o)[8]) {
  const int64_t idx = m * a.K + k0;
  if constexpr (XK == XK_BF16) {
    const uint4 w = coh ? coh_load16(a.x, (uint32_t)(a.M * a.K * 2), (uint32_t)(idx * 2))
                        : *(const uint4*)((const uint16_t*)a.x + idx);
    const uint32_t u[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
    for (int j = 0; j < 4; j++) {
      o[2 * j] = __uint_as_float(u[j] << 16);
      o[2 * j + 1] = __uint_as_float(u[j] & 0xFFFF0000u);
    }
  } else {
#pragma unroll
    for (int h = 0; h < 2; h++) {
      const uint4 w = coh ? coh_load16(a.x, (uint32_t)(a.M * a.K * 4), (uint32_t)(idx * 4 + 16 * h))
                          : ((const uint4*)((const float*)a.x + idx))[h];
      o[4 * h] = __uint_as_float(w.x);
      o[4 * h + 1] = __uint_as_float(w.y);
      o[4 * h + 2] = __uint_as_float(w.z);
      o[4 * h + 3] = __uint_as_float(w.w);
    }
  }
}

// Exact value of an item's slice (quads [q0, q0 + nq)) for row-block rb and
// activation row m, computed on the VALU: lane L = r + 16 q multiplies its
// quarter's 32 weights of every group (decoded from the packed words) by the
// activations (products of +-1 / 0 are exact), sums each group in fp32,
// scales it by the group's fp32 scale, and the four quarters are added.
// The slow path for slices whose staging was flagged (kept small in
// registers: it sits in kernels whose main loops need them); every lane
// returns the value of row r.
template <int FMT, int XK, int TS = 1>
__device__ __attribute__((always_inline)) inline float exact_slice(const FArgs& a, int64_t rb, int64_t q0, int nq,
                                                       int64_t m, bool coh, const uint32_t* t3tab) {
  const int L = threadIdx.x & 63, qtr = L >> 4;
  const uint32_t* t3 = t3tab + L % TS;
  const int64_t rbc = rb < a.NB ? rb : a.NB - 1;
  float acc = 0.f;
#pragma unroll 1
  for (int64_t g = 4 * q0; g < 4 * (q0 + nq) && g < a.G; g++) {
    Quad<FMT> qd;
    load_quad_at<FMT>(a.pcodes, a.pscales, rbc, g >> 2, a.GQ, a.GP, L, qd);
    const int t = (int)(g & 3);
    const v8i B = t == 0 ? decode_group<FMT, TS>(qd, 0, t3) : t == 1 ? decode_group<FMT, TS>(qd, 1, t3)
                : t == 2 ? decode_group<FMT, TS>(qd, 2, t3) : decode_group<FMT, TS>(qd, 3, t3);
    const int64_t k0 = g * kGroup + 64 * (qtr & 1) + 16 * (qtr >> 1);
    float part = 0.f;
#pragma unroll 1
    for (int c = 0; c < 4; c++) {  // slots 8 c .. 8 c + 7: k0 + 32 (c >> 1) + 8 (c & 1) + i
      float xv[8];
      load_x8<XK>(a, m, k0 + 32 * (c >> 1) + 8 * (c & 1), coh, xv);
      const uint32_t w = (uint32_t)(c == 0 ? B[0] : c == 1 ? B[1] : c == 2 ? B[2] : B[3]);
#pragma unroll
      for (int i = 0; i < 8; i++) {
        const uint32_t nib = (w >> (4 * i)) & 0xFu;
        part += nib == 0x2u ? xv[i] : nib == 0xAu ? -xv[i] : 0.0f;
      }
    }
    acc = fmaf(a.pscales ? quad_scale<FMT>(qd, t) : 1.0f, part, acc);
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  return acc;
}

// quad_mfma for one activation row (M = 1, MA = R rows of A) with scales:
// `arow` points at this lane's A row of group 0 of the slice image (lanes
// with r >= R read row r mod R: their output rows are never used, and
// rows of the MFMA are independent), `erow` at its exponent word, so every
// group's operand sits at a compile-time offset.  The scale epilogue of
// group t runs after the MFMA of group t+1 is issued; the accumulation order
// (group 0..3, terms 0..R-1) is the one quad_mfma uses.  AHEAD: the A
// operands of all four groups are read from LDS first (eight more live
// registers per group), for callers with few waves per SIMD to hide the
// LDS latency behind.
template <int FMT, int XK, bool AHEAD = false, int TS = 1>
__device__ __attribute__((always_inline)) inline void quad_mfma_m1(const uint8_t* arow,
                                                                   const uint8_t* erow, int q,
                                                                   const Quad<FMT>& qd,
                                                                   const uint32_t* t3tab,
                                                                   uint32_t sign_mask,
                                                                   uint32_t one_bits, float& acc) {
  constexpr int R = XSplit<FMT, XK>::R, FA = XSplit<FMT, XK>::kFmtA;
  const uint32_t* t3 = t3tab + (threadIdx.x & 63) % TS;
  const uint32_t se = *(const uint32_t*)(erow + q * 4 * R * 4);
  uint4 xa[4][2];
  if constexpr (AHEAD) {
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const uint4* src = (const uint4*)(arow + (q * 16 + t * 4) * R * 32);
      xa[t][0] = src[0];
      xa[t][1] = src[1];
    }
  }
  v4f cp;
  float sp = 0.f;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    if constexpr (!AHEAD) {
      const uint4* src = (const uint4*)(arow + (q * 16 + t * 4) * R * 32);
      xa[t][0] = src[0];
      xa[t][1] = src[1];
    }
    const uint4 x0 = xa[t][0], x1 = xa[t][1];
    const v8i A = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    v8i B;
    if constexpr (FMT == 1) {
      const uint32_t wv = t == 0 ? qd.w[0].x : t == 1 ? qd.w[0].y : t == 2 ? qd.w[0].z : qd.w[0].w;
      B = decode_binary_reg(wv, sign_mask, one_bits);
    } else {
      B = decode_group<FMT, TS>(qd, t, t3);
    }
    const v4f c = mfma_group_t<FA>(t, A, B, (int)se);
    if (t > 0) {
      float tsum = cp[0];
#pragma unroll
      for (int i = 1; i < R; i++) tsum += cp[i];
      acc = fmaf(sp, tsum, acc);
    }
    cp = c;
    sp = quad_scale<FMT>(qd, t);
  }
  float tsum = cp[0];
#pragma unroll
  for (int i = 1; i < R; i++) tsum += cp[i];
  acc = fmaf(sp, tsum, acc);
}

// SiLU-mul epilogue of a fused gate/up product: in every 16-row block the
// rows 0..7 are gate rows and 8..15 the matching up rows, so lane r < 8 of
// a 16-lane row group holds g and lane r + 8 holds u; output 8 b + r of
// row-block b is silu(g) u = g / (1 + e^-g) u in fp32.  Every lane of the
// wave must call it (it shuffles); the result is meaningful in lanes r < 8.
__device__ __attribute__((always_inline)) inline float silu_mul_lanes(float f) {
  const float u = __shfl_down(f, 8);
  return f / (1.0f + expf(-f)) * u;
}

// quad_mfma_m1 for a binary wave of two row-blocks: each group's A operand
// is read once and feeds both row-blocks' MFMAs (two independent chains);
// each row-block's accumulation order is that of quad_mfma_m1.
template <int XK>
__device__ __attribute__((always_inline)) inline void quad_mfma_m1x2(const uint8_t* arow,
                                                                     const uint8_t* erow, int q,
                                                                     const Quad<1>& qd,
                                                                     const Quad<1>& qd2,
                                                                     uint32_t sign_mask,
                                                                     uint32_t one_bits, float& acc0,
                                                                     float& acc1) {
  constexpr int R = XSplit<1, XK>::R;
  const uint32_t se = *(const uint32_t*)(erow + q * 4 * R * 4);
  v4f cp0, cp1;
  float sp0 = 0.f, sp1 = 0.f;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint4* src = (const uint4*)(arow + (q * 16 + t * 4) * R * 32);
    const uint4 x0 = src[0], x1 = src[1];
    const v8i A = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    const uint32_t w0 = t == 0 ? qd.w[0].x : t == 1 ? qd.w[0].y : t == 2 ? qd.w[0].z : qd.w[0].w;
    const uint32_t w1 = t == 0 ? qd2.w[0].x : t == 1 ? qd2.w[0].y : t == 2 ? qd2.w[0].z : qd2.w[0].w;
    const v8i B0 = decode_binary_reg(w0, sign_mask, one_bits);
    const v8i B1 = decode_binary_reg(w1, sign_mask, one_bits);
    const v4f c0 = t == 0 ? mfma_group<0>(A, B0, (int)se) : t == 1 ? mfma_group<1>(A, B0, (int)se)
                 : t == 2 ? mfma_group<2>(A, B0, (int)se) : mfma_group<3>(A, B0, (int)se);
    const v4f c1 = t == 0 ? mfma_group<0>(A, B1, (int)se) : t == 1 ? mfma_group<1>(A, B1, (int)se)
                 : t == 2 ? mfma_group<2>(A, B1, (int)se) : mfma_group<3>(A, B1, (int)se);
    if (t > 0) {
      float s0 = cp0[0], s1 = cp1[0];
#pragma unroll
      for (int i = 1; i < R; i++) {
        s0 += cp0[i];
        s1 += cp1[i];
      }
      acc0 = fmaf(sp0, s0, acc0);
      acc1 = fmaf(sp1, s1, acc1);
    }
    cp0 = c0;
    cp1 = c1;
    sp0 = quad_scale<1>(qd, t);
    sp1 = quad_scale<1>(qd2, t);
  }
  float s0 = cp0[0], s1 = cp1[0];
#pragma unroll
  for (int i = 1; i < R; i++) {
    s0 += cp0[i];
    s1 += cp1[i];
  }
  acc0 = fmaf(sp0, s0, acc0);
  acc1 = fmaf(sp1, s1, acc1);
}

// The same for a binary wave of three row-blocks.
template <int XK>
__device__ __attribute__((always_inline)) inline void quad_mfma_m1x3(
    const uint8_t* arow, const uint8_t* erow, int q, const Quad<1>& qd, const Quad<1>& qd2,
    const Quad<1>& qd3, uint32_t sign_mask, uint32_t one_bits, float& acc0, float& acc1,
    float& acc2) {
  constexpr int R = XSplit<1, XK>::R;
  const uint32_t se = *(const uint32_t*)(erow + q * 4 * R * 4);
  v4f cp0, cp1, cp2;
  float sp0 = 0.f, sp1 = 0.f, sp2 = 0.f;
#pragma unroll
  for (int t = 0; t < 4; t++) {
    const uint4* src = (const uint4*)(arow + (q * 16 + t * 4) * R * 32);
    const uint4 x0 = src[0], x1 = src[1];
    const v8i A = v8i{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
    const uint32_t w0 = t == 0 ? qd.w[0].x : t == 1 ? qd.w[0].y : t == 2 ? qd.w[0].z : qd.w[0].w;
    const uint32_t w1 = t == 0 ? qd2.w[0].x : t == 1 ? qd2.w[0].y : t == 2 ? qd2.w[0].z : qd2.w[0].w;
    const uint32_t w2 = t == 0 ? qd3.w[0].x : t == 1 ? qd3.w[0].y : t == 2 ? qd3.w[0].z : qd3.w[0].w;
    const v8i B0 = decode_binary_reg(w0, sign_mask, one_bits);
    const v8i B1 = decode_binary_reg(w1, sign_mask, one_bits);
    const v8i B2 = decode_binary_reg(w2, sign_mask, one_bits);
    const v4f c0 = t == 0 ? mfma_group<0>(A, B0, (int)se) : t == 1 ? mfma_group<1>(A, B0, (int)se)
                 : t == 2 ? mfma_group<2>(A, B0, (int)se) : mfma_group<3>(A, B0, (int)se);
    const v4f c1 = t == 0 ? mfma_group<0>(A, B1, (int)se) : t == 1 ? mfma_group<1>(A, B1, (int)se)
                 : t == 2 ? mfma_group<2>(A, B1, (int)se) : mfma_group<3>(A, B1, (int)se);
    const v4f c2 = t == 0 ? mfma_group<0>(A, B2, (int)se) : t == 1 ? mfma_group<1>(A, B2, (int)se)
                 : t == 2 ? mfma_group<2>(A, B2, (int)se) : mfma_group<3>(A, B2, (int)se);
    if (t > 0) {
      float s0 = cp0[0], s1 = cp1[0], s2 = cp2[0];
#pragma unroll
      for (int i = 1; i < R; i++) {
        s0 += cp0[i];
        s1 += cp1[i];
        s2 += cp2[i];
      }
      acc0 = fmaf(sp0, s0, acc0);
      acc1 = fmaf(sp1, s1, acc1);
      acc2 = fmaf(sp2, s2, acc2);
    }
    cp0 = c0;
    cp1 = c1;
    cp2 = c2;
    sp0 = quad_scale<1>(qd, t);
    sp1 = quad_scale<1>(qd2, t);
    sp2 = quad_scale<1>(qd3, t);
  }
  float s0 = cp0[0], s1 = cp1[0], s2 = cp2[0];
#pragma unroll
  for (int i = 1; i < R; i++) {
    s0 += cp0[i];
    s1 += cp1[i];
    s2 += cp2[i];
  }
  acc0 = fmaf(sp0, s0, acc0);
  acc1 = fmaf(sp1, s1, acc1);
  acc2 = fmaf(sp2, s2, acc2);
}

// Output of an item: direct stores, or (several K-slices) coherent partial
// sums and, in the last workgroup of the row group to arrive, their sum in
// slice order.  ym[m] / yi[m] hold activation row m's values in lanes 0..15
// (lane r = row 16 rb + r).  COH: the outputs themselves are device-coherent
// stores.
template <int XK, int MM, int YK, bool COH>
__device__ __attribute__((always_inline)) inline void item_output(const FArgs& a, const Item& it,
                                                                  const float (&ym)[MM],
                                                                  const int (&yi)[MM]) {
  constexpr bool INTC = XK == XK_I8;
  __shared__ uint32_t s_last;
  const int L = threadIdx.x & 63, r = L & 15, lg = L >> 4;
  auto store = [&](int64_t m, int64_t n, float f, int iv) {
    const float sxm = a.x_scales ? a.x_scales[m] : a.x_scale;
    if constexpr (COH) {
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
  const int64_t n = 16 * it.rb + r;
  const bool mine = it.live && lg == 0;  // the lanes that hold the outputs
  if (a.KS == 1 && a.epi) {
    const float z = silu_mul_lanes(ym[0]);
    if (mine && r < 8) store(0, 8 * it.rb + r, z, 0);
    return;
  }
  if (a.KS == 1) {
    if (mine && n < a.N) {
#pragma unroll
      for (int m = 0; m < MM; m++)
        if (m < a.M) store(m, n, ym[m], yi[m]);
    }
    return;
  }
  // partials: write-through (agent-coherent) stores, completed before the
  // workgroup's arrival is counted
  if (mine) {
#pragma unroll
    for (int m = 0; m < MM; m++) {
      if (m < a.M) {
        float* dst = a.part + (it.ks * a.M + m) * a.Npad + n;
        if (IPART) __hip_atomic_store((int*)dst, yi[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else __hip_atomic_store(dst, ym[m], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    s_last = __hip_atomic_fetch_add(a.cnt + 16 + it.rg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_last != (uint32_t)(a.KS - 1)) return;
  // last arrival: add the slices in order (coherent loads) and store
  if (a.epi) {
    float f = 0.f;
    if (mine)
      for (int64_t k2 = 0; k2 < a.KS; k2++)
        f += __hip_atomic_load(a.part + k2 * a.Npad + n, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const float z = silu_mul_lanes(f);
    if (mine && r < 8) store(0, 8 * it.rb + r, z, 0);
    if (threadIdx.x == 0)
      __hip_atomic_store(a.cnt + 16 + it.rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  if (mine && n < a.N) {
#pragma unroll
    for (int m = 0; m < MM; m++) {
      if (m < a.M) {
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
  }
  if (threadIdx.x == 0)
    __hip_atomic_store(a.cnt + 16 + it.rg, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// The raw activations of the first kStageRounds staging rounds, in named
// registers (an array of them may be left in scratch memory by the compiler,
// and every scratch access waits for all loads in flight).
struct XRegs {
  uint4 a0, a1, a2, a3, a4, b0, b1, b2, b3, b4;
};
static_assert(kStageRounds == 5, "XRegs holds five staging rounds");

template <int K>
__device__ __attribute__((always_inline)) inline uint4& xa_reg(XRegs& x) {
  if constexpr (K == 0) return x.a0;
  else if constexpr (K == 1) return x.a1;
  else if constexpr (K == 2) return x.a2;
  else if constexpr (K == 3) return x.a3;
  else return x.a4;
}
template <int K>
__device__ __attribute__((always_inline)) inline uint4& xb_reg(XRegs& x) {
  if constexpr (K == 0) return x.b0;
  else if constexpr (K == 1) return x.b1;
  else if constexpr (K == 2) return x.b2;
  else if constexpr (K == 3) return x.b3;
  else return x.b4;
}

// NR <= kStageRounds rounds hoisted (one-row items need only as many as
// their largest slice has: 3 for 10-quad slices, 4 for 16)
template <int XK, bool COH, int NR, int K = 0>
__device__ __attribute__((always_inline)) inline void stage_load_rounds(const FArgs& a,
                                                                        const Item& it, XRegs& x) {
  stage_load1<XK, COH>(a, it.q0, it.nq, K, xa_reg<K>(x), xb_reg<K>(x));
  if constexpr (K + 1 < NR) stage_load_rounds<XK, COH, NR, K + 1>(a, it, x);
}

template <int FMT, int XK, int NR, bool LIST, int K = 0>
__device__ __attribute__((always_inline)) inline bool stage_convert_rounds(const FArgs& a,
                                                                           const Item& it,
                                                                           const Lds& l, XRegs& x,
                                                                           uint32_t* wlist) {
  bool bad = stage_convert1<FMT, XK, LIST>(a, it.q0, it.nq, K, xa_reg<K>(x), xb_reg<K>(x), l.xa, l.xe,
                                           wlist);
  if constexpr (K + 1 < NR) bad = stage_convert_rounds<FMT, XK, NR, LIST, K + 1>(a, it, l, x, wlist) || bad;
  return bad;
}

// every staging round of an item (the first NR hoisted); true if this thread
// saw an inaccurate element (LIST: that its wave's correction list is full)
template <int FMT, int XK, int SB, int NR, bool LIST = false>
__device__ __attribute__((always_inline)) inline bool stage_all(const FArgs& a, const Item& it,
                                                                const Lds& l, XRegs& x, bool coh) {
  uint32_t* wlist = LIST ? l.list + kListWaveWords * (threadIdx.x >> 6) : nullptr;
  bool bad = stage_convert_rounds<FMT, XK, NR, LIST>(a, it, l, x, wlist);
  // remaining rounds (small-M products with long slices): SB rounds' loads
  // go out together, then their conversions
  const int64_t rounds = cdiv(it.nq * 64 * a.M, (int64_t)blockDim.x);
  for (int64_t rd = NR; rd < rounds; rd += SB) {
    uint4 r0[SB], r1[SB];
#pragma unroll
    for (int u = 0; u < SB; u++) {
      if (rd + u < rounds) {
        if (coh) stage_load1<XK, true>(a, it.q0, it.nq, rd + u, r0[u], r1[u]);
        else stage_load1<XK, false>(a, it.q0, it.nq, rd + u, r0[u], r1[u]);
      }
    }
#pragma unroll
    for (int u = 0; u < SB; u++)
      if (rd + u < rounds)
        bad = stage_convert1<FMT, XK, LIST>(a, it.q0, it.nq, rd + u, r0[u], r1[u], l.xa, l.xe, wlist) || bad;
  }
  return bad;
}

// Byte stride of the slice images a one-product call with several activation
// rows stages once into xst: the image of qmax quads and its flag words.
__host__ __device__ inline int64_t image_stride(int64_t qmax, int64_t MA, int64_t M) {
  return qmax * 16 * MA * 33 + image_flag_bytes(slice_rounds(qmax, M));
}

// The one-product kernel with several activation rows: item `it`'s slice
// image and flag words, staged once per call into a.xst, copied into LDS
// with direct global -> LDS copies (1 KiB per wave instruction) and waited
// for.
template <int FMT>
__device__ __attribute__((always_inline)) inline void copy_image(const FArgs& a, const Item& it,
                                                                 const Lds& l) {
#if defined(__HIP_DEVICE_COMPILE__)
  typedef __attribute__((address_space(3))) uint8_t lds_u8_t;
  const int64_t qmax = FMT == 3 ? 2 * cdiv(cdiv(a.GQ, 2), a.KS) : cdiv(a.GQ, a.KS);
  const int64_t bytes = (int64_t)it.nq * 16 * a.MA * 33 + image_flag_bytes(slice_rounds(it.nq, a.M));
  const uint8_t* src = a.xst + it.ks * image_stride(qmax, a.MA, a.M);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, W = blockDim.x >> 6;
  for (int64_t off = 1024 * (int64_t)w; off < bytes; off += 1024 * (int64_t)W)
    if (off + 16 * lane < bytes)
      __builtin_amdgcn_global_load_lds(src + off + 16 * lane, (lds_u8_t*)(l.xa + off), 16, 0, 0);
  __builtin_amdgcn_s_waitcnt(0);  // this wave's copies have landed
#endif
}

// One work item, loads issued all at once: the body of the one-product
// kernel (CHAIN false) and of the chain kernel with waits (CHAIN: outputs
// are device-coherent; WAIT: the weight loads go out first, then the
// workgroup waits until `wait_cnt` reaches `wait_target` -- the previous
// product is complete -- and reads its activations with coherent loads).
// stage false: the workgroup's previous item was the same product and
// K-slice, so the activation image (and its staging flags) in LDS is this
// item's already.  MM: activation rows the kernel handles at most.
// The correction-list entries of a one-row item: entry {slot i of quarter b
// of group t of quad ql, rho} adds scale x code x rho to the outputs.  Lane
// r + 16 b reads row r's codes and scales of quad ql again (the item has
// just read them: L2 hits; entries are rare, and keeping every quad's codes
// in registers past the MFMAs would cost more), the output of row r is in
// lane r.
template <int FMT, int TS>
__device__ __attribute__((always_inline)) inline void list_fix(const FArgs& a, const Item& it, const Lds& l, float& acc) {
  const uint32_t* t3 = l.t3 + (threadIdx.x & 63) % TS;
  for (int w2 = 0; w2 < (int)(blockDim.x >> 6); w2++) {
    const uint32_t* wl = l.list + kListWaveWords * w2;
    const uint32_t n = min(__builtin_amdgcn_readfirstlane(wl[0]), (uint32_t)kListEntries);
    for (uint32_t e = 0; e < n; e++) {
      const uint32_t pos = __builtin_amdgcn_readfirstlane(wl[2 + 2 * e]);
      const float rho = __uint_as_float(__builtin_amdgcn_readfirstlane(wl[3 + 2 * e]));
      Quad<FMT> qd;
      load_quad<FMT>(a, it, (int)(pos >> 9), qd);
      const int i = pos & 31, b = (pos >> 5) & 3, t = (pos >> 7) & 3;
      uint32_t nib;  // the slot's fp4 code: +1 = 0x2, -1 = 0xA, 0 = 0x0
      if constexpr (FMT == 2) {
        // straight from the bit-sliced words: slot i is nibble i & 7 of
        // P0 (i < 16) or P1, shifted left once for the odd eighths
        const u4 c4 = (t >> 1) ? qd.w[1] : qd.w[0];
        const uint32_t p0 = (t & 1) ? c4.z : c4.x, p1 = (t & 1) ? c4.w : c4.y;
        const uint32_t wd = ((i < 16 ? p0 : p1) << ((i >> 3) & 1)) & 0xAAAAAAAAu;
        nib = (wd >> (4 * (i & 7))) & 0xFu;
      } else {
        const v8i B = decode_group<FMT, TS>(qd, t, t3);
        const int wi = i >> 3;
        const uint32_t wd = (uint32_t)(wi == 0 ? B[0] : wi == 1 ? B[1] : wi == 2 ? B[2] : B[3]);
        nib = (wd >> (4 * (i & 7))) & 0xFu;
      }
      const float c = nib == 0x2u ? rho : nib == 0xAu ? -rho : 0.0f;
      const float val = quad_scale<FMT>(qd, t) * c;
      acc += __shfl(val, (int)(threadIdx.x & 15) + 16 * b);
    }
  }
}

// Warming loads for the workgroup's next item: one 4-byte load per 128-byte
// line of this wave's codes (up to 24 KiB) and scales of item blk, so that
// the lines are cached when that item runs.  The values are only consumed
// (an empty asm statement), never used.
template <int FMT>
__device__ __attribute__((always_inline)) inline void warm_item(const FArgs& a, int64_t blk, uint32_t& w0,
                                                                uint32_t& w1, uint32_t& w2, uint32_t& w3) {
  const Item it = item_of<FMT>(a, blk);
  if (it.nq <= 0) return;
  const int L = threadIdx.x & 63;
  const int64_t rbc = it.live ? it.rb : a.NB - 1;
  int64_t c0, clen;
  if constexpr (FMT == 1) {
    c0 = (rbc * a.GQ + it.q0) * 1024;
    clen = (int64_t)it.nq * 1024;
  } else if constexpr (FMT == 2) {
    c0 = (rbc * a.GP + 2 * it.q0) * 1024;
    clen = (min<int64_t>(2 * (it.q0 + it.nq), a.GP) - 2 * it.q0) * 1024;
  } else {
    const int64_t o0 = it.q0 >> 1, o1 = (it.q0 + it.nq - 1) >> 1;
    c0 = (rbc * ((a.GQ + 1) / 2) + o0) * 3328;
    clen = (o1 - o0 + 1) * 3328;
  }
  const uint8_t* cb = a.pcodes + c0;
  w0 = *(const uint32_t*)(cb + min<int64_t>(128 * L, clen - 4));
  w1 = *(const uint32_t*)(cb + min<int64_t>(128 * L + 8192, clen - 4));
  w2 = *(const uint32_t*)(cb + min<int64_t>(128 * L + 16384, clen - 4));
  if (a.pscales) {
    const uint8_t* sb = (const uint8_t*)a.pscales + (rbc * a.GQ + it.q0) * 128;
    w3 = *(const uint32_t*)(sb + min<int64_t>(128 * L, (int64_t)it.nq * 128 - 4));
  }
}

template <int FMT, int XK, int MM, int YK, int QM, bool CHAIN, bool WAIT, bool ONE = false>
__device__ __attribute__((always_inline)) inline void gemv_item(
    const FArgs& a, int64_t blk, uint8_t* smem, const uint32_t* wait_cnt, uint32_t wait_target,
    uint32_t* err, bool stage = true, int64_t warm_blk = -1) {
  using S = XSplit<FMT, XK>;
  constexpr int R = S::R;
  // staging rounds whose loads go out before the weight loads: a one-row
  // slice of QM quads needs QM 64 / 256 of them
  constexpr int NR = MM == 1 ? (QM * 64 + 255) / 256 : kStageRounds;
  static_assert(NR <= kStageRounds, "hoisted staging rounds");
  const Item it = item_of<FMT>(a, blk);
  const bool pre = !CHAIN && a.xst != nullptr;  // slice image staged once per call
  // one activation row of ternary weights and bf16 activations: the elements
  // the split terms may miss go to correction lists (applied after the MFMAs)
  constexpr bool LISTED = S::kCheck == 1 && MM == 1 && CHAIN;
  const int64_t nflag = pre ? image_flag_bytes(slice_rounds(it.nq, a.M)) : 0;
  constexpr int TS = trit_copies<FMT, MM == 1>();
  const Lds l = lds_of(a, smem, it.nq, nflag);
  lds_init<FMT, TS>(l);

  XRegs xr;
  if constexpr (!WAIT) {
    // activation loads of the first staging rounds go out first
    if (stage && !pre) stage_load_rounds<XK, false, NR>(a, it, xr);
  }
  // every code and scale of the wave is requested before anything else
  Quad<FMT> qd[QM];
#pragma unroll
  for (int q = 0; q < QM; q++) load_quad<FMT>(a, it, q, qd[q]);
  uint32_t wm0 = 0, wm1 = 0, wm2 = 0, wm3 = 0;
  if constexpr (WAIT) {
    // (warm_blk: the workgroup's next item, of this product and K-slice)
    if (warm_blk >= 0) warm_item<FMT>(a, warm_blk, wm0, wm1, wm2, wm3);
    // the previous product must be complete before its outputs are read; the
    // weight loads above are already in flight
    if (threadIdx.x < 64) {
      const int L = threadIdx.x;
      for (uint32_t spin = 0;; spin++) {
        uint32_t v = L < 16 ? __hip_atomic_load(wait_cnt + 16 * L, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
        v += __shfl_xor(v, 1);
        v += __shfl_xor(v, 2);
        v += __shfl_xor(v, 4);
        v += __shfl_xor(v, 8);
        if (__builtin_amdgcn_readfirstlane(v) >= wait_target) break;
        if (spin >= kChainSpinLimit) {  // never satisfied: flag it and go on
          if (L == 0) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
    }
    __syncthreads();
    stage_load_rounds<XK, true, NR>(a, it, xr);
  }
  if (pre) {
    copy_image<FMT>(a, it, l);
  } else if (stage) {
    // (each wave's list is cleared by its own lane 0 before its lanes append:
    // one wave's LDS accesses take effect in order)
    if (LISTED && (threadIdx.x & 63) == 0) l.list[kListWaveWords * (threadIdx.x >> 6)] = 0u;
    const bool bad = stage_all<FMT, XK, ONE || !CHAIN ? 1 : 4, NR, LISTED>(a, it, l, xr, WAIT);
    put_wave_flag(l.wflag, bad);
  }
  __syncthreads();
  // the slice must be recomputed exactly (a staged element is not accurate enough)
  const bool exact = S::kCheck != 0 &&
                     (pre ? get_flags((const uint32_t*)(l.xa + (int64_t)it.nq * 16 * a.MA * 33),
                                      (int)slice_rounds(it.nq, a.M))
                          : get_flags(l.wflag, blockDim.x >> 6));

  float ym[MM];
  int yi[MM];
  if constexpr ((CHAIN && ONE) || (MM == 1 && XK != XK_I8)) {
    // one activation row with scales (float activations always have them):
    // the single-row routine
    static_assert(MM == 1, "the single-row routine keeps one row");
    float acc = 0.f;
    if (it.live) {
      const int lane = threadIdx.x & 63, rr = (lane & 15) % R, lg = lane >> 4;
      const uint8_t* arow = l.xa + (lg * R + rr) * 32;
      const uint8_t* erow = l.xe + (lg * R + rr) * 4;
      uint32_t sign_mask = 0x88888888u, one_bits = 0x22222222u;
      if constexpr (FMT == 1) {
        asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(sign_mask));
        asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(one_bits));
      }
#pragma unroll
      for (int q = 0; q < QM; q++)
        if (q < it.nq) quad_mfma_m1<FMT, XK, CHAIN, TS>(arow, erow, q, qd[q], l.t3, sign_mask, one_bits, acc);
      if constexpr (LISTED) {
        // the entries of the waves' correction lists (rare)
        uint32_t nlist = 0;
        for (int w2 = 0; w2 < (int)(blockDim.x >> 6); w2++) nlist |= l.list[kListWaveWords * w2];
        if (__builtin_amdgcn_readfirstlane(nlist) != 0) list_fix<FMT, TS>(a, it, l, acc);
      }
    }
    ym[0] = acc;
    yi[0] = 0;
  } else {
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    int iacc[4] = {0, 0, 0, 0};
    if (it.live) {
#pragma unroll
      for (int q = 0; q < QM; q++)
        if (q < it.nq) quad_mfma<FMT, XK, MM, 4, TS>(a, l, q, qd[q], acc, iacc);
    }
    gather_rows<R, MM>(acc, ym);
    gather_rows<R, MM>(iacc, yi);
  }
  if constexpr (S::kCheck != 0) {
    if (__builtin_expect(exact, 0)) {  // the slice recomputed exactly
      for (int m = 0; m < (int)a.M; m++) {  // rolled: one copy of the slow path
        const float v = exact_slice<FMT, XK, TS>(a, it.rb, it.q0, it.nq, m, WAIT, l.t3);
#pragma unroll
        for (int mm = 0; mm < MM; mm++)
          if (mm == m) ym[mm] = v;
      }
    }
  }
  // the warming loads have landed before the item's stores go out (the
  // completion count that follows waits for the stores)
  if constexpr (WAIT) asm volatile("" ::"v"(wm0), "v"(wm1), "v"(wm2), "v"(wm3));
  item_output<XK, MM, YK, CHAIN>(a, it, ym, yi);
}

// Slice images of a one-product call with several activation rows, staged
// once into xst (slice ks at ks * image_stride): block (rd, ks) converts
// round rd of slice ks, the units and lanes of the in-workgroup staging, and
// writes the round's flag word.
template <int FMT, int XK>
__global__ __launch_bounds__(256) void stage_images(FArgs a, uint8_t* xst) {
  const int64_t ks = blockIdx.y, rd = blockIdx.x;
  const Item it = item_at<FMT>(a, 0, ks);
  const int64_t qmax = FMT == 3 ? 2 * cdiv(cdiv(a.GQ, 2), a.KS) : cdiv(a.GQ, a.KS);
  uint8_t* xa = xst + ks * image_stride(qmax, a.MA, a.M);
  uint8_t* xe = xa + (int64_t)it.nq * 16 * a.MA * 32;
  uint4 r0, r1;
  stage_load1<XK, false>(a, it.q0, it.nq, rd, r0, r1);
  const bool bad = stage_convert1<FMT, XK>(a, it.q0, it.nq, rd, r0, r1, xa, xe);
  const int flagged = __syncthreads_or(bad ? 1 : 0);
  if (threadIdx.x == 0 && rd < slice_rounds(it.nq, a.M))
    ((uint32_t*)(xa + (int64_t)it.nq * 16 * a.MA * 33))[rd] = flagged ? 1u : 0u;
}

template <int FMT, int XK, int MM, int YK, int QM>
__global__ __launch_bounds__(64 * kMaxW) void gemv_mfma(FArgs a) {
  extern __shared__ __align__(16) uint8_t smem[];
  gemv_item<FMT, XK, MM, YK, QM, false, false>(a, blockIdx.x, smem, nullptr, 0, nullptr);
}

// Persistent kernel over a chain of batch-1 products (items of product s
// are [first[s], first[s+1]) in a global order that every workgroup walks
// with stride gridDim.x).  Finished items of product s are counted in 16
// counters done[256 s + 16 j], one 64-byte line each (item i adds to
// counter i mod 16, so no one address takes every workgroup's atomic), and a
// product marked `wait` reads its activations only after the 16 counters of
// product s-1, read together by 16 lanes, sum to its item count.
// Workgroups never wait on an item
// later in the order than their own, and the grid is co-resident
// (cooperative launch), so every wait ends; a wait is nevertheless bounded
// by kChainSpinLimit.  The last workgroup to finish resets the counters.
struct ChainArgs {
  const FArgs* args;       // [S]
  const int64_t* first;    // [S + 1] work items (row group x K-slice) before product s
  const int32_t* wait;     // [S]
  uint32_t* done;          // [256 S] (16 used per product), zero between launches
  uint32_t* finished;      // workgroups done, zero between launches
  uint32_t* err;           // set when a wait gave up
  // streaming kernel only
  const int64_t* ufirst;   // [S + 1] row groups before product s
  const int64_t* sfirst;   // [S + 1] K-slices before product s
  const int64_t* xoff;     // [S] byte offset of product s's staged activations in xst
  uint8_t* xst;            // staged activations of every product and K-slice
  uint32_t* bar;           // grid barrier arrivals, zero between launches
  uint32_t* flagged;       // some staged slice was flagged, zero between launches
  int S;
};

// The chain tables are read through the constant address space: scalar
// loads (counted by lgkmcnt), so reading the next item's descriptor never
// waits for the vector loads of codes in flight.
#define LOWBIT_CONST __attribute__((address_space(4)))
typedef const LOWBIT_CONST FArgs* FArgsTab;
typedef const LOWBIT_CONST int64_t* I64Tab;
typedef const LOWBIT_CONST int32_t* I32Tab;

__device__ __attribute__((always_inline)) inline FArgs load_args(FArgsTab t, int s) {
  FArgs a;
  a.pcodes = t[s].pcodes;
  a.pscales = t[s].pscales;
  a.x = t[s].x;
  a.x_scales = t[s].x_scales;
  a.y = t[s].y;
  a.part = t[s].part;
  a.cnt = t[s].cnt;
  a.N = t[s].N;
  a.K = t[s].K;
  a.G = t[s].G;
  a.GQ = t[s].GQ;
  a.GP = t[s].GP;
  a.M = t[s].M;
  a.MA = t[s].MA;
  a.NB = t[s].NB;
  a.KS = t[s].KS;
  a.Npad = t[s].Npad;
  a.x_scale = t[s].x_scale;
  a.xkind = t[s].xkind;
  a.epi = t[s].epi;
  a.xst = nullptr;
  return a;
}

// MR: several activation rows per product (lane group lg keeps 4 / R rows)
template <int FMT, int XK, int YK, int QM, bool MR>
__global__ __launch_bounds__(64 * kMaxW) __attribute__((amdgpu_waves_per_eu(2))) void gemv_chain(ChainArgs c) {
  constexpr int MX = MR ? 16 / XSplit<FMT, XK>::R : 1;  // activation rows at most
  extern __shared__ __align__(16) uint8_t smem[];
  const FArgsTab args = (FArgsTab)c.args;
  const I64Tab first = (I64Tab)c.first;
  const I32Tab waitf = (I32Tab)c.wait;
  const int64_t total = first[c.S];
  int s = 0, s_last = -1;
  int64_t ks_last = -1;
  for (int64_t i = blockIdx.x; i < total; i += gridDim.x) {
    while (i >= first[s + 1]) s++;
    const FArgs a = load_args(args, s);
    // a second item of the same product and K-slice (products with more
    // items than workgroups): its wait is met and its activations are staged
    const int64_t ks = (i - first[s]) % a.KS;
    const bool again = s == s_last && ks == ks_last;
    s_last = s;
    ks_last = ks;
    const bool wt = s > 0 && waitf[s] != 0 && !again;
    __syncthreads();  // the previous item's LDS reads are over
    // the workgroup's next item, when it is of the same product and K-slice
    // (one-row chains: the several-row kernels have no registers to spare)
    const int64_t nxt = i + gridDim.x;
    const bool warm = !MR && nxt < first[s + 1] && (nxt - first[s]) % a.KS == ks;
    if (wt)
      gemv_item<FMT, XK, MX, YK, QM, true, true, !MR>(a, i - first[s], smem, c.done + 256 * (s - 1),
                                                      (uint32_t)(first[s] - first[s - 1]), c.err, true,
                                                      warm ? nxt - first[s] : -1);
    else
      gemv_item<FMT, XK, MX, YK, QM, true, false, !MR>(a, i - first[s], smem, nullptr, 0u, c.err,
                                                       !again);
    __builtin_amdgcn_s_waitcnt(0);  // this item's stores have completed
    __syncthreads();
    if (threadIdx.x == 0) {
      const uint32_t idx = (uint32_t)(i - first[s]);
      __hip_atomic_fetch_add(c.done + 256 * s + 16 * (idx & 15), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
  __shared__ uint32_t s_prev;
  __syncthreads();
  if (threadIdx.x == 0)
    s_prev = __hip_atomic_fetch_add(c.finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __syncthreads();
  if (s_prev == gridDim.x - 1) {
    for (int k = threadIdx.x; k < 16 * c.S; k += blockDim.x)
      __hip_atomic_store(c.done + 256 * (k >> 4) + 16 * (k & 15), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (threadIdx.x == 0) __hip_atomic_store(c.finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Persistent chain without waits, software-pipelined.
//
// Prologue: the workgroups stage the activations of every product and
// K-slice (fp8 split terms + block exponents) into a global buffer, then
// meet at a grid barrier (the launch is cooperative, so all workgroups are
// resident).
//
// Main loop: a workgroup takes whole row groups (all K-slices in turn,
// accumulating in registers, so there are no split-K partial sums) of the
// products in order, row group u, u + gridDim.x, ...; each wave owns one
// row-block of it.  While a wave computes quad q of one slice, the codes
// and scales of quad q of its next slice (and the staged activations of
// the slice after) are
// already in flight, so every wave keeps a full slice of loads outstanding
// across slice, row-group and product boundaries.
// (Slice images of the streaming kernel: the image, then one 16-byte flag
// word -- nonzero when the slice must be recomputed exactly.)
template <int FMT>
__device__ __attribute__((always_inline)) inline int64_t slice_stride(const FArgs& a) {
  const int64_t qmax = FMT == 3 ? 2 * cdiv(cdiv(a.GQ, 2), a.KS) : cdiv(a.GQ, a.KS);
  return qmax * 16 * a.MA * 33 + 16;
}

// Binary weights carry half the bytes of 2-bit ternary per quad, so a
// binary wave needs more work in flight: with bf16 activations it holds
// three row-blocks (RB = 3, below); otherwise the binary kernel is held to
// 128 registers (one MFMA group in flight per step) to run four workgroups
// per CU.
//
// MR: chains of small-M products (M activation rows, M R <= 16, all stages
// alike, e.g. a verification pass over drafted tokens): the slice images
// hold M R rows of A, the quads go through the generic quad routine (one
// accumulator per A row), and each slice's rows are gathered into lanes
// 0..15 (gather_rows) before they are added up over the row's slices.
//
// RB = 3 (binary, one row): every wave holds three row-blocks, whose MFMAs
// share each A operand read (row groups of 192 rows, two workgroups per CU),
// so that two waves per SIMD keep as many bytes in flight as three ternary
// waves do; RB = 2 where a stage's codes are too long for buffer offsets.
template <int FMT, int XK, int YK, int QM, bool MR, int RB>
__global__ __launch_bounds__(64 * kMaxW) __attribute__((amdgpu_waves_per_eu(FMT == 1 && XK == XK_BF16 && !MR && RB == 1 ? 4 : 2))) void gemv_stream(ChainArgs c) {
  using S = XSplit<FMT, XK>;
  constexpr int R = S::R;
  constexpr int MM = MR ? 16 / R : 1;  // activation rows at most
  constexpr int NACC = MR ? 4 : RB;   // accumulators per lane (MR: one per A row)
  constexpr int NTOT = MR ? MM : RB;  // row sums per lane
  static_assert(RB == 1 || (FMT == 1 && !MR), "several row-blocks per wave: binary, one row");
  static_assert(RB == 1 || S::kCheck == 0, "binary bf16 rows never need the exact recomputation");
  extern __shared__ __align__(16) uint8_t smem[];
  const FArgsTab args = (FArgsTab)c.args;
  const I64Tab ufirst = (I64Tab)c.ufirst;
  const I64Tab sfirst = (I64Tab)c.sfirst;
  const I64Tab xoff = (I64Tab)c.xoff;

  // ---- prologue: stage every (product, K-slice) once
  {
    const int64_t nsl = sfirst[c.S];
    int s = 0;
    for (int64_t j = blockIdx.x; j < nsl; j += gridDim.x) {
      while (j >= sfirst[s + 1]) s++;
      const FArgs a = load_args(args, s);
      const int64_t ks = j - sfirst[s];
      const Item it = item_at<FMT>(a, 0, ks);  // row group 0 of slice ks
      uint8_t* xa = c.xst + xoff[s] + ks * slice_stride<FMT>(a);
      uint8_t* xe = xa + (int64_t)it.nq * 16 * a.MA * 32;
      const int64_t rounds = cdiv(it.nq * 64 * a.M, (int64_t)blockDim.x);
      bool bad = false;
      for (int64_t rd = 0; rd < rounds; rd++) {
        uint4 r0, r1;
        stage_load1<XK, false>(a, it.q0, it.nq, rd, r0, r1);
        bad = stage_convert1<FMT, XK>(a, it.q0, it.nq, rd, r0, r1, xa, xe) || bad;
      }
      // the slice's flag word after its image, and the launch's summary flag
      const int flagged = __syncthreads_or(bad ? 1 : 0);
      if (threadIdx.x == 0) {
        *(uint32_t*)(xa + (int64_t)it.nq * 16 * a.MA * 33) = flagged ? 1u : 0u;
        if (flagged) __hip_atomic_fetch_or(c.flagged, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
      __hip_atomic_fetch_add(c.bar, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      for (uint32_t spin = 0;
           __hip_atomic_load(c.bar, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) < gridDim.x; spin++) {
        if (spin >= kChainSpinLimit) {
          __hip_atomic_store(c.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          break;
        }
        __builtin_amdgcn_s_sleep(2);
      }
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    }
    __syncthreads();
  }

  // some slice of the launch was flagged (written before the grid barrier;
  // read now, so that the load's latency is spent under the main loop)
  bool any = false;
  if constexpr (S::kCheck != 0)
    any = __builtin_amdgcn_readfirstlane(
              __hip_atomic_load(c.flagged, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) != 0;

  // ---- main loop
  // LDS: two buffers, each the image of one staged slice (slice j uses
  // buffer j & 1), then the zero block / base-3 table and four counters:
  // filled[b] counts the waves that wrote their share of an image into
  // buffer b, consumed[b] the waves that finished computing from it.  A wave
  // writes its share of slice j+1 part-way through slice j, so waves are
  // only ever held back by a wave more than about one slice behind (there is
  // no workgroup barrier in the loop).
  // rows of A an image may hold: several-row chains use 6-quad slices up to
  // 10 rows of A, 5-quad slices up to 15 and 4-quad slices up to 16
  constexpr int MAX_MA = MR ? multi_max_ma(QM) : R;
  // (an image is followed by its 16-byte flag word)
  constexpr int XR = (QM * 16 * MAX_MA * 33 + 16 + 16 * 64 * kMaxW - 1) / (16 * 64 * kMaxW);
  constexpr int kWriteAfter = 3;  // quads computed before the next image is written
  static_assert(QM > kWriteAfter, "the next image is written part-way through a slice");
  const int64_t bufsz = (int64_t)QM * 16 * MAX_MA * 33 + 16;
  // rows of A of every stage (one M per chain)
  const int64_t MAc = MR ? args[0].MA : R;
  auto xbuf = [&](uint32_t b) { return smem + b * bufsz; };
  Lds lfix;
  lfix.zblk = smem + 2 * bufsz;
  constexpr int TS = trit_copies<FMT, !MR>();
  lfix.t3 = (uint32_t*)(lfix.zblk + kZeroBlock);
  uint32_t* filled = (uint32_t*)(lfix.zblk + kZeroBlock + trit_table_bytes(TS));
  uint32_t* consumed = filled + 2;
  lds_init<FMT, TS>(lfix);
  if (threadIdx.x < 4) filled[threadIdx.x] = 0;
  // binary decode masks, in registers (opaque to constant folding)
  uint32_t sign_mask = 0x88888888u, one_bits = 0x22222222u;
  if constexpr (FMT == 1) {
    asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(sign_mask));
    asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(one_bits));
  }

  const int64_t total = ufirst[c.S];
  int64_t u = blockIdx.x;
  const int tid = threadIdx.x;
  if (u < total) {
    int s = 0;
    while (u >= ufirst[s + 1]) s++;
    FArgs a = load_args(args, s);
    int64_t rg = u - ufirst[s], ks = 0;
    Item it = item_at<FMT, RB>(a, rg, 0);
    // staged activations of a slice, XR 16-byte pieces per thread
    auto xsrc = [&](const FArgs& f, int sidx, int64_t kslice, int nq, int k) {
      const int64_t nb = (int64_t)nq * 16 * f.MA * 33 / 16 + 1;  // image and flag word
      const int64_t piece = min<int64_t>((int64_t)k * 64 * kMaxW + tid, nb - 1);
      return (const uint4*)(c.xst + xoff[sidx] + kslice * slice_stride<FMT>(f)) + piece;
    };
    // a slice image travels in up to nine 16-byte registers per thread (named
    // registers, not an array, so that they never live in scratch memory)
    uint4 x0, x1, x2, x3, x4, x5, x6, x7, x8, x9;
    static_assert(XR <= 10, "slice image larger than ten 16-byte pieces per thread");
#define XLD(F, SI, KS_, NQ)                                                                  \
  {                                                                                          \
    x0 = *xsrc(F, SI, KS_, NQ, 0);                                                           \
    if (XR > 1) x1 = *xsrc(F, SI, KS_, NQ, 1);                                               \
    if (XR > 2) x2 = *xsrc(F, SI, KS_, NQ, 2);                                               \
    if (XR > 3) x3 = *xsrc(F, SI, KS_, NQ, 3);                                               \
    if (XR > 4) x4 = *xsrc(F, SI, KS_, NQ, 4);                                               \
    if (XR > 5) x5 = *xsrc(F, SI, KS_, NQ, 5);                                               \
    if (XR > 6) x6 = *xsrc(F, SI, KS_, NQ, 6);                                               \
    if (XR > 7) x7 = *xsrc(F, SI, KS_, NQ, 7);                                               \
    if (XR > 8) x8 = *xsrc(F, SI, KS_, NQ, 8);                                               \
    if (XR > 9) x9 = *xsrc(F, SI, KS_, NQ, 9);                                               \
  }
#define XPUT(DST, NQ)                                                                        \
  {                                                                                          \
    const int64_t nb_ = (int64_t)(NQ) * 16 * MAc * 33 / 16 + 1;                              \
    uint4* d_ = (uint4*)(DST);                                                               \
    constexpr int T_ = 64 * kMaxW;                                                           \
    if (tid < nb_) d_[tid] = x0;                                                             \
    if (XR > 1 && T_ + tid < nb_) d_[T_ + tid] = x1;                                         \
    if (XR > 2 && 2 * T_ + tid < nb_) d_[2 * T_ + tid] = x2;                                 \
    if (XR > 3 && 3 * T_ + tid < nb_) d_[3 * T_ + tid] = x3;                                 \
    if (XR > 4 && 4 * T_ + tid < nb_) d_[4 * T_ + tid] = x4;                                 \
    if (XR > 5 && 5 * T_ + tid < nb_) d_[5 * T_ + tid] = x5;                                 \
    if (XR > 6 && 6 * T_ + tid < nb_) d_[6 * T_ + tid] = x6;                                 \
    if (XR > 7 && 7 * T_ + tid < nb_) d_[7 * T_ + tid] = x7;                                 \
    if (XR > 8 && 8 * T_ + tid < nb_) d_[8 * T_ + tid] = x8;                                 \
    if (XR > 9 && 9 * T_ + tid < nb_) d_[9 * T_ + tid] = x9;                                 \
  }
    XLD(a, s, ks, it.nq);
    XPUT(xbuf(0), it.nq);
    __syncthreads();

    // next slice of this workgroup after (s, rg, ks): the same row group's
    // next K-slice, or the next row group; `more` false at the end (then the
    // current slice is returned again, as harmless dummy loads)
    auto next = [&](int s0, int64_t u0, int64_t rg0, int64_t ks0, const FArgs& f, int& s1,
                    int64_t& u1, int64_t& rg1, int64_t& ks1) {
      s1 = s0;
      u1 = u0;
      rg1 = rg0;
      ks1 = ks0 + 1;
      if (ks1 < f.KS) return true;
      ks1 = 0;
      u1 = u0 + gridDim.x;
      if (u1 >= total) {
        u1 = u0;
        ks1 = ks0;
        return false;
      }
      while (u1 >= ufirst[s1 + 1]) s1++;
      rg1 = u1 - ufirst[s1];
      return true;
    };
    int sn;
    int64_t un, rgn, ksn;
    bool more = next(s, u, rg, ks, a, sn, un, rgn, ksn);
    FArgs an = load_args(args, sn);
    Item itn = item_at<FMT, RB>(an, rgn, ksn);
    QuadPtr pn = quad_ptr<FMT, RB == 3 ? 1 : RB>(an, itn);
    QuadBuf bn;
    if constexpr (RB == 3) bn = quad_buf3(an, itn);
    const int vc = 16 * (threadIdx.x & 63), vs = 8 * (threadIdx.x & 15);
    // the current slice's codes quad by quad with the next slice's
    // activations after quad kWriteAfter - 1: the order the loop issues them
    // in, kept by scheduling barriers, so that the wait counts in the loop
    // (the stricter of loop entry and back edge) leave a whole slice of loads
    // in flight
    Quad<FMT> qd[QM];
    Quad<FMT> qd2[RB >= 2 ? QM : 1];
    Quad<FMT> qd3[RB == 3 ? QM : 1];
    {
      const QuadPtr p0 = quad_ptr<FMT, RB == 3 ? 1 : RB>(a, it);
      QuadBuf b0;
      if constexpr (RB == 3) b0 = quad_buf3(a, it);
#pragma unroll
      for (int q = 0; q < QM; q++) {
        if (q == kWriteAfter) XLD(an, sn, ksn, itn.nq);
        if constexpr (RB == 3) load_quad_b3(b0, q, vc, vs, qd[q], qd2[q], qd3[q]);
        else if constexpr (RB == 2) load_quad_p2(p0, q, qd[q], qd2[q]);
        else load_quad_p<FMT>(p0, q, qd[q]);
        __builtin_amdgcn_sched_barrier(0);
      }
    }
    float acc[NACC], tot[NTOT];  // tot: slices added in slice order, as the split-K reduction does
    int iacc[NACC];
#pragma unroll
    for (int m = 0; m < NACC; m++) {
      acc[m] = 0.f;
      iacc[m] = 0;
    }
#pragma unroll
    for (int m = 0; m < NTOT; m++) tot[m] = 0.f;
    uint32_t j = 0;   // slice number of this workgroup

    auto wait_ge = [&](uint32_t* ctr, uint32_t target) {
      if ((threadIdx.x & 63) == 0) {
        for (uint32_t spin = 0; __hip_atomic_load(ctr, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) < target; spin++) {
          if (spin >= kChainSpinLimit) {
            __hip_atomic_store(c.err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      __builtin_amdgcn_wave_barrier();
    };

    for (;;) {
      // the slice after next (its activations are loaded while this one computes)
      int s2;
      int64_t u2, rg2, ks2;
      const bool more2 = more && next(sn, un, rgn, ksn, an, s2, u2, rg2, ks2);
      if (!more) {
        s2 = sn;
        u2 = un;
        rg2 = rgn;
        ks2 = ksn;
      }
      // slice j's image is complete once every wave wrote its share (slice 0's
      // was written before the loop; buffer j & 1 is filled for slices j, j-2,
      // ... down to 1 or 2: (j + 1) / 2 times)
      const uint32_t b = j & 1;
      if (j > 0) wait_ge(filled + b, 4u * ((j + 1) >> 1));
      // this lane's A row and exponent word in the slice image (one row), or
      // the image as the generic quad routine reads it (several rows)
      const int lane = threadIdx.x & 63, rr = (lane & 15) % R, lg = lane >> 4;
      const uint8_t* arow = xbuf(b) + (lg * R + rr) * 32;
      const uint8_t* erow = xbuf(b) + it.nq * 16 * R * 32 + (lg * R + rr) * 4;
      Lds lq = lfix;
      lq.xa = xbuf(b);
      lq.xe = xbuf(b) + (int64_t)it.nq * 16 * MAc * 32;
#pragma unroll
      for (int q = 0; q < QM; q++) {
        if (q == kWriteAfter) {
          if (more) {
            // this wave's share of slice j+1's image, into the other buffer
            // once every wave is done with slice j-1
            wait_ge(consumed + (b ^ 1), 4u * ((j + 1) >> 1));
            XPUT(xbuf(b ^ 1), itn.nq);
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): the share is written
            if ((threadIdx.x & 63) == 0)
              __hip_atomic_fetch_add(filled + (b ^ 1), 1u, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_WORKGROUP);
          }
          // then the activations of the slice after next (issued on every
          // path, so that the wait counts stay exact across iterations)
          const FArgs a2 = load_args(args, s2);
          const Item it2 = item_at<FMT, RB>(a2, rg2, ks2);
          XLD(a2, s2, ks2, it2.nq);
        }
        if (it.live && q < it.nq) {
          if constexpr (MR)
            quad_mfma<FMT, XK, MM, 2>(a, lq, q, qd[q], acc, iacc);
          else if constexpr (RB == 3)
            quad_mfma_m1x3<XK>(arow, erow, q, qd[q], qd2[q], qd3[q], sign_mask, one_bits, acc[0], acc[1],
                               acc[NACC - 1]);
          else if constexpr (RB == 2)
            quad_mfma_m1x2<XK>(arow, erow, q, qd[q], qd2[q], sign_mask, one_bits, acc[0], acc[1]);
          else
            quad_mfma_m1<FMT, XK, false, TS>(arow, erow, q, qd[q], lfix.t3, sign_mask, one_bits, acc[0]);
        }
        if constexpr (RB == 3) load_quad_b3(bn, q, vc, vs, qd[q], qd2[q], qd3[q]);
        else if constexpr (RB == 2) load_quad_p2(pn, q, qd[q], qd2[q]);
        else load_quad_p<FMT>(pn, q, qd[q]);
      }
      // done reading slice j's image
      __builtin_amdgcn_s_waitcnt(0xC07F);
      if ((threadIdx.x & 63) == 0)
        __hip_atomic_fetch_add(consumed + b, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      if constexpr (MR) {
        // this slice's value of every activation row, in lanes 0..15
        float ys[MM];
        gather_rows<R, MM>(acc, ys);
#pragma unroll
        for (int m = 0; m < MM; m++) tot[m] = a.KS == 1 ? ys[m] : tot[m] + ys[m];
#pragma unroll
        for (int v = 0; v < 4; v++) acc[v] = 0.f;
      } else {
#pragma unroll
        for (int m = 0; m < NACC; m++) {
          tot[m] = a.KS == 1 ? acc[m] : tot[m] + acc[m];
          acc[m] = 0.f;
        }
      }
      if (ks == a.KS - 1) {
        // row group complete: one output per row (lanes 0..15)
        const int L = threadIdx.x & 63, r = L & 15, lg = L >> 4;
        const int64_t n = 16 * it.rb + r;
        if constexpr (MR) {
#pragma unroll
          for (int m = 0; m < MM; m++) {
            if (it.live && lg == 0 && m < a.M && n < a.N) {
              if (YK == YK_F32) ((float*)a.y)[m * a.N + n] = tot[m];
              else ((uint16_t*)a.y)[m * a.N + n] = (uint16_t)bf16_rne(tot[m]);
            }
            tot[m] = 0.f;
          }
        } else {
#pragma unroll
          for (int i = 0; i < RB; i++) {
            const int64_t rbi = it.rb + i, ni = 16 * rbi + r;
            const bool live = rbi < a.NB;
            if (a.epi) {
              const float z = silu_mul_lanes(tot[i]);
              const int64_t nz = 8 * rbi + r;
              if (live && lg == 0 && r < 8) {
                if (YK == YK_F32) ((float*)a.y)[nz] = z;
                else ((uint16_t*)a.y)[nz] = (uint16_t)bf16_rne(z);
              }
            } else if (live && lg == 0 && ni < a.N) {
              if (YK == YK_F32) ((float*)a.y)[ni] = tot[i];
              else ((uint16_t*)a.y)[ni] = (uint16_t)bf16_rne(tot[i]);
            }
            tot[i] = 0.f;
          }
        }
      }
      if (!more) break;
      s = sn; u = un; rg = rgn; ks = ksn;
      a = load_args(args, s);
      it = itn;
      sn = s2; un = u2; rgn = rg2; ksn = ks2;
      more = more2;
      an = load_args(args, sn);
      itn = item_at<FMT, RB>(an, rgn, ksn);
      if constexpr (RB == 3) bn = quad_buf3(an, itn);
      else pn = quad_ptr<FMT, RB>(an, itn);
      j++;
    }
  }

  // ---- exact recomputation of the row groups of products with a flagged
  // slice (a staged activation not accurate enough; never for N(0,1)
  // inputs): each workgroup redoes its own row groups on the VALU, after its
  // main loop so that the streaming loop keeps its registers, and overwrites
  // the outputs it wrote.
  if constexpr (S::kCheck != 0) {
    int sf = 0;
    for (int64_t uf = __builtin_expect(any, 0) ? (int64_t)blockIdx.x : total; uf < total; uf += gridDim.x) {
      while (uf >= ufirst[sf + 1]) sf++;
      const FArgs a = load_args(args, sf);
      bool flagged = false;
      for (int64_t k2 = 0; k2 < a.KS; k2++) {
        const Item itk = item_at<FMT>(a, 0, k2);
        const uint8_t* img = c.xst + xoff[sf] + k2 * slice_stride<FMT>(a);
        flagged = flagged || *(const uint32_t*)(img + (int64_t)itk.nq * 16 * a.MA * 33) != 0;
      }
      if (!__builtin_amdgcn_readfirstlane(flagged ? 1 : 0)) continue;
      const int64_t rgf = uf - ufirst[sf];
      const int L = threadIdx.x & 63, r = L & 15, lg = L >> 4;
      for (int64_t m = 0; m < a.M; m++) {
        float y = 0.f;
        Item itk;
        for (int64_t k2 = 0; k2 < a.KS; k2++) {  // slices in order, as the main loop adds them
          itk = item_at<FMT, RB>(a, rgf, k2);
          y += exact_slice<FMT, XK, TS>(a, itk.rb, itk.q0, itk.nq, m, false, lfix.t3);
        }
        const int64_t n = 16 * itk.rb + r;
        if (a.epi) {
          const float z = silu_mul_lanes(y);
          if (itk.live && lg == 0 && r < 8) {
            if (YK == YK_F32) ((float*)a.y)[8 * itk.rb + r] = z;
            else ((uint16_t*)a.y)[8 * itk.rb + r] = (uint16_t)bf16_rne(z);
          }
        } else if (itk.live && lg == 0 && n < a.N) {
          if (YK == YK_F32) ((float*)a.y)[m * a.N + n] = y;
          else ((uint16_t*)a.y)[m * a.N + n] = (uint16_t)bf16_rne(y);
        }
      }
    }
  }

#undef XLD
#undef XPUT
  // ---- the last workgroup to finish resets the barrier
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev =
        __hip_atomic_fetch_add(c.finished, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (prev == gridDim.x - 1) {
      __hip_atomic_store(c.bar, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(c.flagged, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(c.finished, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

struct Plan {
  int64_t NB, NRG, G, GQ, GP, KS, Npad, MA;
  int R, W, QM;
  size_t lds, part_off, bytes;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

constexpr int kQuadsBinary = 16;   // quads a wave keeps in registers (binary)
constexpr int kQuadsTernary = 10;  // (2-bit ternary: twice the code bytes)

Plan make_plan(int fmt, int64_t N, int64_t K, int64_t M, int xkind, int quads = 0, int rb = 1) {
  Plan p;
  p.R = split_terms(fmt, xkind);
  p.MA = M * p.R;
  p.NB = cdiv(N, 16);
  p.G = K / kGroup;
  p.GQ = cdiv(p.G, 4);
  p.GP = cdiv(p.G, 2);
  p.QM = quads > 0 ? quads : fmt == 1 ? kQuadsBinary : kQuadsTernary;
  // staged activations of a slice stay within 78 KiB of LDS (small-M
  // products of up to 15 rows of A keep a 5120-long row in one slice; two
  // workgroups still fit a CU)
  int64_t qcap = std::min<int64_t>(p.QM, std::max<int64_t>(1, (78 * 1024) / (16 * p.MA * 33)));
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
  p.NRG = cdiv(p.NB, p.W * rb);  // rb row-blocks per wave (the binary streaming kernel: 2)
  const int64_t qmax = fmt == 3 ? 2 * cdiv(cdiv(p.GQ, 2), p.KS) : cdiv(p.GQ, p.KS);
  // LDS of the one-product kernel: the slice image (with its flag words when
  // it is copied from the images staged once per call, M > 1), the zero
  // block and flags, the base-3 table
  p.lds = (size_t)qmax * 16 * p.MA * 33 + (M > 1 ? (size_t)image_flag_bytes(slice_rounds(qmax, M)) : 0) +
          kListBytes + kZeroBlock + (fmt == 3 ? trit_table_bytes(M == 1 ? kTritCopies : 1) : 0);
  p.Npad = p.NRG * p.W * rb * 16;
  p.part_off = kCounterBytes;
  p.bytes = p.part_off + align256((size_t)(p.KS > 1 ? p.KS : 0) * M * p.Npad * 4);
  return p;
}

template <int FMT, int XK, int MM, int QM>
hipError_t launch_y(const GemvArgs& g, const FArgs& k, dim3 grid, dim3 block, size_t lds,
                    hipStream_t s) {
  if (g.ykind == YK_F32)
    hipLaunchKernelGGL((gemv_mfma<FMT, XK, MM, YK_F32, QM>), grid, block, lds, s, k);
  else if (g.ykind == YK_BF16)
    hipLaunchKernelGGL((gemv_mfma<FMT, XK, MM, YK_BF16, QM>), grid, block, lds, s, k);
  else
    hipLaunchKernelGGL((gemv_mfma<FMT, XK, MM, YK_I32, QM>), grid, block, lds, s, k);
  return hipGetLastError();
}

// one activation row, or up to 16 / R of them
template <int FMT, int XK, int QM>
hipError_t launch_m(const GemvArgs& g, const FArgs& k, dim3 grid, dim3 block, size_t lds,
                    hipStream_t s) {
  constexpr int MM = 16 / split_terms(FMT, XK);
  if (g.M > MM) return hipErrorInvalidValue;
  return g.M == 1 ? launch_y<FMT, XK, 1, QM>(g, k, grid, block, lds, s)
                  : launch_y<FMT, XK, MM, QM>(g, k, grid, block, lds, s);
}

template <int FMT, int QM>
hipError_t launch_x(const GemvArgs& g, const FArgs& k, dim3 grid, dim3 block, size_t lds,
                    hipStream_t s) {
  if (g.xkind == XK_F32) return launch_m<FMT, XK_F32, QM>(g, k, grid, block, lds, s);
  if (g.xkind == XK_I8) return launch_m<FMT, XK_I8, QM>(g, k, grid, block, lds, s);
  return launch_m<FMT, XK_BF16, QM>(g, k, grid, block, lds, s);
}

}  // namespace

// bytes of the slice images a one-product call with M > 1 stages once
size_t image_bytes(const Plan& p, int fmt, int64_t M) {
  if (M <= 1) return 0;
  const int64_t qmax = fmt == 3 ? 2 * cdiv(cdiv(p.GQ, 2), p.KS) : cdiv(p.GQ, p.KS);
  return align256((size_t)(p.KS * image_stride(qmax, p.MA, M)));
}

size_t gemv_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t M, int xkind) {
  const Plan p = make_plan(fmt, N, K, M, xkind);
  return p.bytes + image_bytes(p, fmt, M);
}

hipError_t launch_gemv_mfma(const GemvArgs& g, hipStream_t s) {
  const Plan p = make_plan(g.fmt, g.N, g.K, g.M, g.xkind);
  if (p.NRG > kMaxRowGroups || p.lds > kLdsCap) return hipErrorInvalidValue;
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
  k.epi = 0;
  k.xst = nullptr;
  if (g.M > 1) {
    // several rows: the slice images are staged once, then copied by every
    // workgroup (instead of each converting M x K activations itself)
    k.xst = (const uint8_t*)g.ws + p.bytes;
    const int64_t qmax = g.fmt == 3 ? 2 * cdiv(cdiv(p.GQ, 2), p.KS) : cdiv(p.GQ, p.KS);
    const dim3 sgrid((unsigned)cdiv(qmax * 64 * g.M, (int64_t)256), (unsigned)p.KS);
    uint8_t* xst = (uint8_t*)g.ws + p.bytes;
    const bool f32 = g.xkind == XK_F32, i8 = g.xkind == XK_I8;
#define STAGE_IMG(F)                                                                          \
  {                                                                                           \
    if (f32) hipLaunchKernelGGL((stage_images<F, XK_F32>), sgrid, dim3(256), 0, s, k, xst);   \
    else if (i8) hipLaunchKernelGGL((stage_images<F, XK_I8>), sgrid, dim3(256), 0, s, k, xst); \
    else hipLaunchKernelGGL((stage_images<F, XK_BF16>), sgrid, dim3(256), 0, s, k, xst);      \
  }
    if (g.fmt == 1) STAGE_IMG(1)
    else if (g.fmt == 2) STAGE_IMG(2)
    else STAGE_IMG(3)
#undef STAGE_IMG
  }
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
const void* chain_kernel(int ykind, bool waits, int64_t M, int rb) {
  constexpr int QM = FMT == 1 ? kQuadsBinary : kQuadsTernary;
  const bool b16 = ykind == YK_BF16;
  if (waits) {
    if (M == 1)
      return b16 ? (const void*)gemv_chain<FMT, XK, YK_BF16, QM, false>
                 : (const void*)gemv_chain<FMT, XK, YK_F32, QM, false>;
    return b16 ? (const void*)gemv_chain<FMT, XK, YK_BF16, QM, true>
               : (const void*)gemv_chain<FMT, XK, YK_F32, QM, true>;
  }
  if constexpr (FMT == 1 && XK == XK_BF16) {
    if (M == 1 && rb == 3)
      return b16 ? (const void*)gemv_stream<FMT, XK, YK_BF16, kQuadsTernary, false, 3>
                 : (const void*)gemv_stream<FMT, XK, YK_F32, kQuadsTernary, false, 3>;
    if (M == 1 && rb == 2)
      return b16 ? (const void*)gemv_stream<FMT, XK, YK_BF16, kQuadsTernary, false, 2>
                 : (const void*)gemv_stream<FMT, XK, YK_F32, kQuadsTernary, false, 2>;
  }
  if (M == 1)
    return b16 ? (const void*)gemv_stream<FMT, XK, YK_BF16, kQuadsTernary, false, 1>
               : (const void*)gemv_stream<FMT, XK, YK_F32, kQuadsTernary, false, 1>;
  constexpr int R = XSplit<FMT, XK>::R;
  if (M * R <= multi_max_ma(kQuadsMultiWide))
    return b16 ? (const void*)gemv_stream<FMT, XK, YK_BF16, kQuadsMultiWide, true, 1>
               : (const void*)gemv_stream<FMT, XK, YK_F32, kQuadsMultiWide, true, 1>;
  // (base-3 slices are whole octets: an odd quad count would re-read a quad)
  if constexpr (FMT != 3)
    if (M * R <= multi_max_ma(kQuadsMultiMid))
      return b16 ? (const void*)gemv_stream<FMT, XK, YK_BF16, kQuadsMultiMid, true, 1>
                 : (const void*)gemv_stream<FMT, XK, YK_F32, kQuadsMultiMid, true, 1>;
  return b16 ? (const void*)gemv_stream<FMT, XK, YK_BF16, kQuadsMulti, true, 1>
             : (const void*)gemv_stream<FMT, XK, YK_F32, kQuadsMulti, true, 1>;
}

}  // namespace

hipError_t chain_create(const ChainStage* st, int S, int64_t M, int xkind, int ykind, void** out) {
  *out = nullptr;
  if (S < 1 || M < 1) return hipErrorInvalidValue;
  const int fmt = st[0].fmt;
  if (M * split_terms(fmt, xkind) > 16) return hipErrorInvalidValue;
  std::vector<FArgs> args(S);
  std::vector<int64_t> first(S + 1, 0);
  std::vector<int32_t> wait(S, 0);
  std::vector<int64_t> cnt_off(S), part_off(S);
  std::vector<int64_t> ufirst(S + 1, 0), sfirst(S + 1, 0), xoff(S, 0);
  int64_t cnt_words = 16, part_floats = 0, xst_bytes = 0;
  bool waits = false;
  for (int i = 1; i < S; i++) waits = waits || st[i].wait_prev != 0;
  // the streaming kernel keeps kQuadsTernary quads of every format in flight
  // (kQuadsMulti with several activation rows); its two image buffers are
  // sized for the most rows of A it handles (R, or 16)
  const int R = split_terms(fmt, xkind);
  const int quads = waits ? 0
                  : M == 1 ? kQuadsTernary
                  : M * R <= multi_max_ma(kQuadsMultiWide) ? kQuadsMultiWide
                  : fmt != 3 && M * R <= multi_max_ma(kQuadsMultiMid) ? kQuadsMultiMid
                  : kQuadsMulti;
  // binary, one bf16 row, no waits: three row-blocks per wave (buffer
  // addressing: every stage's codes shorter than 2^31 bytes), else two
  bool buf_ok = true;
  for (int i = 0; i < S; i++)
    buf_ok = buf_ok && cdiv(st[i].N, 16) * cdiv(st[i].K / kGroup, 4) * 1024 < (int64_t(1) << 31);
  const int rb = !waits && M == 1 && fmt == 1 && xkind == XK_BF16 ? (buf_ok ? 3 : 2) : 1;
  // streaming kernel: two image buffers (image + flag word), the zero block,
  // the base-3 table and four counters
  size_t lds = waits ? 0 : 2 * ((size_t)quads * 16 * (M == 1 ? R : multi_max_ma(quads)) * 33 + 16) + kZeroBlock +
                          trit_table_bytes(fmt == 3 && M == 1 ? kTritCopies : 1) + 16;
  for (int i = 0; i < S; i++) {
    if (st[i].fmt != fmt) return hipErrorInvalidValue;
    if (st[i].epi && M != 1) return hipErrorInvalidValue;
    const Plan p = make_plan(fmt, st[i].N, st[i].K, M, xkind, quads, rb);
    if (p.lds > kLdsCap) return hipErrorInvalidValue;
    if (waits) lds = std::max(lds, p.lds);
    first[i + 1] = first[i] + p.NRG * p.KS;
    ufirst[i + 1] = ufirst[i] + p.NRG;
    sfirst[i + 1] = sfirst[i] + p.KS;
    xoff[i] = xst_bytes;
    const int64_t qmax = fmt == 3 ? 2 * cdiv(cdiv(p.GQ, 2), p.KS) : cdiv(p.GQ, p.KS);
    xst_bytes += p.KS * (qmax * 16 * p.MA * 33 + 16);  // slice_stride
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
    k.M = M;
    k.MA = p.MA;
    k.NB = p.NB;
    k.KS = p.KS;
    k.Npad = p.Npad;
    k.x_scale = 1.0f;
    k.xkind = xkind;
    k.epi = st[i].epi;
    k.xst = nullptr;
  }
  if (first[S] > 0x7FFFFFFF || cnt_words > 0x7FFFFFFF) return hipErrorInvalidValue;
  // layout of the one allocation
  const size_t o_args = 0;
  const size_t o_first = align256(o_args + sizeof(FArgs) * S);
  const size_t o_wait = align256(o_first + sizeof(int64_t) * (S + 1));
  const size_t o_done = align256(o_wait + sizeof(int32_t) * S);
  const size_t o_fin = align256(o_done + sizeof(uint32_t) * S * 256);
  const size_t o_cnt = align256(o_fin + 4 * sizeof(uint32_t));
  const size_t o_part = align256(o_cnt + sizeof(uint32_t) * cnt_words);
  const size_t o_uf = align256(o_part + sizeof(float) * (size_t)part_floats);
  const size_t o_sf = align256(o_uf + sizeof(int64_t) * (S + 1));
  const size_t o_xo = align256(o_sf + sizeof(int64_t) * (S + 1));
  const size_t o_xst = align256(o_xo + sizeof(int64_t) * S);
  const size_t bytes = o_xst + (size_t)xst_bytes + 256;

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
  if (e == hipSuccess) e = hipMemcpy(m + o_uf, ufirst.data(), sizeof(int64_t) * (S + 1), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(m + o_sf, sfirst.data(), sizeof(int64_t) * (S + 1), hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(m + o_xo, xoff.data(), sizeof(int64_t) * S, hipMemcpyHostToDevice);
  if (e == hipSuccess) {
    const bool f32 = xkind == XK_F32;
    if (fmt == 1) c->kernel = f32 ? chain_kernel<1, XK_F32>(ykind, waits, M, rb) : chain_kernel<1, XK_BF16>(ykind, waits, M, rb);
    else if (fmt == 2) c->kernel = f32 ? chain_kernel<2, XK_F32>(ykind, waits, M, rb) : chain_kernel<2, XK_BF16>(ykind, waits, M, rb);
    else if (fmt == 3) c->kernel = f32 ? chain_kernel<3, XK_F32>(ykind, waits, M, rb) : chain_kernel<3, XK_BF16>(ykind, waits, M, rb);
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
  // The streaming 2-bit chain runs two workgroups per CU although three fit:
  // fewer concurrent weight streams read HBM more efficiently (a plain
  // read of the same row-group pattern: 7.0 TB/s at two workgroups of four
  // waves per CU, 6.6 at three), and its per-wave work hides the rest.
  // Base-3 keeps every resident workgroup (its table decode needs them).
  const int64_t per = !waits && fmt == 2 ? std::min(per_cu, 2) : per_cu;
  const int64_t want = per * cus;
  c->grid = dim3((unsigned)std::min<int64_t>(want, first[S]));
  c->block = dim3(64 * kMaxW);
  c->lds = lds;
  c->args.args = (const FArgs*)(m + o_args);
  c->args.first = (const int64_t*)(m + o_first);
  c->args.wait = (const int32_t*)(m + o_wait);
  c->args.done = (uint32_t*)(m + o_done);
  c->args.finished = (uint32_t*)(m + o_fin);
  c->args.err = (uint32_t*)(m + o_fin) + 1;
  c->args.bar = (uint32_t*)(m + o_fin) + 2;
  c->args.flagged = (uint32_t*)(m + o_fin) + 3;
  c->args.ufirst = (const int64_t*)(m + o_uf);
  c->args.sfirst = (const int64_t*)(m + o_sf);
  c->args.xoff = (const int64_t*)(m + o_xo);
  c->args.xst = m + o_xst;
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
  const uint8_t* xbits;  // K sign bits, bit k % 8 of byte k / 8
  void* y;
  int64_t N, K, G, GQ;
  float alpha;
};

// Sign-bit word of (group g, quarter q) in the binary weight word order:
// slot i of the quarter is k = 128 g + KMAP(q, i), i.e. the two 16-bit runs
// at bit offsets base and base + 32 of the group (base = 64 (q & 1) +
// 16 (q >> 1)); bit b of the word holds slot 8 (3 - (b & 3)) + (b >> 2),
// a 4 x 8 bit transpose of the slot-ordered word.
__device__ inline uint32_t sign_word(const uint8_t* gp, int q) {
  const int base = 64 * (q & 1) + 16 * (q >> 1);
  const uint32_t v = (uint32_t)*(const uint16_t*)(gp + base / 8) |
                     ((uint32_t)*(const uint16_t*)(gp + base / 8 + 4) << 16);
  uint32_t w = 0;
#pragma unroll
  for (int a = 0; a < 8; a++)
#pragma unroll
    for (int c = 0; c < 4; c++) w |= ((v >> (8 * (3 - c) + a)) & 1u) << (4 * a + c);
  return w;
}

// QB: quads of codes a wave loads per round (every load of a round is issued
// before any of it is used; loads past the wave's range are clamped onto its
// last quad, so the launch picks QB to fit the wave's quad count)
template <int YK, int QB>
__global__ __launch_bounds__(1024) void gemv_sign(SArgs a) {
  __shared__ float red_f[kMaxWaves][64];
  __shared__ int red_i[kMaxWaves][64];
  extern __shared__ __align__(16) uint32_t xw_lds[];  // [GQ][4 quarters][4 groups]
  const int L = threadIdx.x & 63, w = threadIdx.x >> 6, S = blockDim.x >> 6;
  const int r = L & 15, q = L >> 4;
  const int64_t rb = blockIdx.x;
  const int64_t q0 = (a.GQ * w) / S, q1 = (a.GQ * (w + 1)) / S;
  const u4* pc4 = (const u4*)a.pcodes;
  const uint2* ps2 = (const uint2*)a.pscales;
  // the first round's codes and scales go out before the row's sign words
  // are built (they do not depend on x)
  u4 cw[QB];
  uint2 sc[QB];
  auto load_round = [&](int64_t base) {
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int64_t gq = min<int64_t>(base + i, q1 - 1);  // clamped into the wave's range
      cw[i] = __builtin_nontemporal_load(&pc4[(rb * a.GQ + gq) * 64 + L]);
      sc[i] = a.pscales ? ps2[(rb * a.GQ + gq) * 16 + r] : make_uint2(0x3C003C00u, 0x3C003C00u);
    }
  };
  if (q0 < q1) load_round(q0);
  // this row's sign words, built once per workgroup: the raw sign bits (16
  // bytes per group) are copied into the words' LDS area with 16-byte loads,
  // then 16 lanes of one wave rebuild each quad's 16 words in place (a quad's
  // words depend only on its own 64 raw bytes, and a wave's reads of them
  // complete before its writes)
  {
    const uint4* xg = (const uint4*)a.xbits;
    uint4* xl = (uint4*)xw_lds;
    for (int64_t i = threadIdx.x; i < 4 * a.GQ; i += blockDim.x)
      xl[i] = i < a.G ? xg[i] : make_uint4(0u, 0u, 0u, 0u);
  }
  __syncthreads();
  for (int64_t qb = 4 * (int64_t)w + q; qb < a.GQ; qb += 4 * (int64_t)S) {
    const int t = r & 3, qq = r >> 2;
    const int64_t g = 4 * qb + t;
    const uint32_t v = g < a.G ? sign_word((const uint8_t*)xw_lds + 16 * g, qq) : 0u;
    xw_lds[qb * 16 + r] = v;
  }
  __syncthreads();
  const uint4* xw4 = (const uint4*)xw_lds;
  float acc = 0.f;
  int iacc = 0;
  // up to QB quads per round: every load of a round is issued before
  // any of it is used
  for (int64_t base = q0; base < q1; base += QB) {
    if (base != q0) load_round(base);
#pragma unroll
    for (int i = 0; i < QB; i++) {
      const int64_t gq = base + i;
      if (gq < q1) {
        const uint4 xv = xw4[gq * 4 + q];
        const int ng = (int)min<int64_t>(4, a.G - 4 * gq);
        const uint32_t wv[4] = {cw[i].x, cw[i].y, cw[i].z, cw[i].w};
        const uint32_t xx[4] = {xv.x, xv.y, xv.z, xv.w};
        const uint32_t ss[4] = {sc[i].x & 0xFFFF, sc[i].x >> 16, sc[i].y & 0xFFFF, sc[i].y >> 16};
#pragma unroll
        for (int t = 0; t < 4; t++) {
          if (t < ng) {
            const int d = 32 - 2 * __popc(wv[t] ^ xx[t]);
            iacc += d;
            acc = fmaf(f16_bits_to_f32(ss[t]), (float)d, acc);
          }
        }
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

// quads per load round for waves of `qpw` quads: as few rounds as rounds of
// 8 allow (each round waits for its loads), then the smallest round that
// still covers the quads in that many (fewest clamped duplicate loads)
int pick_sign_round(int64_t qpw) {
  const int64_t rounds = cdiv(qpw < 1 ? 1 : qpw, (int64_t)8);
  const int64_t need = cdiv(qpw < 1 ? 1 : qpw, rounds);
  for (int qb : {2, 4, 5, 8})
    if (qb >= need) return qb;
  return 8;
}

template <int QB>
hipError_t launch_sign_qb(int ykind, dim3 grid, dim3 block, size_t lds, hipStream_t s, const SArgs& k) {
  if (ykind == YK_F32) hipLaunchKernelGGL((gemv_sign<YK_F32, QB>), grid, block, lds, s, k);
  else if (ykind == YK_BF16) hipLaunchKernelGGL((gemv_sign<YK_BF16, QB>), grid, block, lds, s, k);
  else hipLaunchKernelGGL((gemv_sign<YK_I32, QB>), grid, block, lds, s, k);
  return hipGetLastError();
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
  k.xbits = g.xbits;
  k.y = g.y;
  k.N = g.N;
  k.K = g.K;
  k.G = G;
  k.GQ = cdiv(G, 4);
  k.alpha = g.alpha;
  const size_t lds = (size_t)k.GQ * 16 * 4;  // the sign words of the whole row
  if (g.K > kSignMaxK || lds > 48 * 1024) return hipErrorInvalidValue;
  int S = pick_waves(NB, k.GQ);
  dim3 grid((unsigned)NB), block(64 * S);
  const int QB = pick_sign_round(cdiv(k.GQ, (int64_t)S));
  if (QB == 2) return launch_sign_qb<2>(g.ykind, grid, block, lds, s, k);
  if (QB == 4) return launch_sign_qb<4>(g.ykind, grid, block, lds, s, k);
  if (QB == 5) return launch_sign_qb<5>(g.ykind, grid, block, lds, s, k);
  return launch_sign_qb<8>(g.ykind, grid, block, lds, s, k);
}

}  // namespace lowbit
