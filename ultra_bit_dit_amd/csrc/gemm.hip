// Large-M products Y[M][N] = X[M][K] . W[N][K]^T over packed binary or
// ternary weights (2-bit or base-3) with one fp16 scale per 128-weight group
// (the group-scaled matmul of section "1-bit 嘅數學：點解唔爆鑊？" of the page
// "瀏覽器生圖技術內幕：1-bit diffusion 點樣將 3GB 模型塞入 WebGPU？"; prefill
// and diffusion-transformer blocks run it as a dense contraction).
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
#include <type_traits>

#include "common.hpp"
#include "fp4.hpp"

namespace lowbit {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) uint8_t lds_u8;

// ---------------------------------------------------------------- GEMM args
struct KArgs {
  const uint8_t* xt;        // staged activation tiles
  const float* rowscale;    // per-row output multiplier, or NULL
  const uint8_t* pcodes;
  const uint16_t* pscales;  // NULL only for the exact int32 product
  void* y;
  float* part;              // split-K partial tiles
  uint32_t* cnt;            // zero-initialised arrival counters
  const uint16_t* x;        // the bf16 activations (exact recomputation of overflowed lists)
  int64_t M, N, K, G, GQ, GP, NB, MT, NT;
  int64_t F;                // tiles (in tile order) run whole; the others are split KS ways
  int KS;
  int row_fast;             // tile order: row tile fastest (else column tile fastest)
};

// Workgroup -> (split, row tile, column tile).  The first F tiles of the
// tile order run whole (one workgroup each); the other TT tiles are split
// KS ways along K (split ks of tail tile j is workgroup F + ks TT + j).
// Workgroups are dealt to the 8 XCDs round-robin; each XCD gets a
// contiguous run of that order -- F / 8 whole tiles, then (TT KS) / 8 split
// ones, so that every XCD gets the same share of the work when both divide
// by 8.  With the column tile fastest the workgroups resident on one XCD
// share their activation tiles in that XCD's L2 and every XCD streams all
// the weights; with the row tile fastest (products whose packed weights
// outweigh their staged activations, e.g. 512-token prefill) each XCD keeps
// its share of the weights in L2 and streams the activation tiles instead.
// nks: the splits of this workgroup's tile (1 or KS); tail: the tile's index
// among the split ones (their partial sums and counters).
__device__ inline void tile_of(const KArgs& a, int64_t& mt, int64_t& nt, int& ks, int& nks,
                               int64_t& tail) {
  const int64_t TT = a.MT * a.NT - a.F;
  const int64_t T = a.F + TT * a.KS;
  const int64_t bid = blockIdx.x;
  int64_t id = bid;
  if (T >= 8) {
    const int64_t x = bid % 8, loc = bid / 8;
    if (a.F % 8 == 0 && (TT * a.KS) % 8 == 0) {
      const int64_t fl = a.F / 8, tl = TT * a.KS / 8;
      id = loc < fl ? x * fl + loc : a.F + x * tl + (loc - fl);
    } else {
      const int64_t base = T / 8, rem = T % 8;
      id = x * base + min(x, rem) + loc;
    }
  }
  int64_t ti;
  if (id < a.F) {
    ti = id;
    ks = 0;
    nks = 1;
    tail = 0;
  } else {
    const int64_t j = id - a.F;
    tail = j % TT;
    ti = a.F + tail;
    ks = (int)(j / TT);
    nks = a.KS;
  }
  if (a.row_fast) {
    mt = ti % a.MT;
    nt = (ti / a.MT) % a.NT;
  } else {
    nt = ti % a.NT;
    mt = (ti / a.NT) % a.MT;
  }
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
// are coalesced) with device-coherent (write-through) stores, waits until
// they have completed and bumps the tile counter; the last split to arrive
// reads the other partials with device-coherent loads and adds all of them in
// split order (deterministic), then resets the counter.  No fences: an
// agent-scope fence writes back or invalidates the whole L2 of the XCD, for
// every split.  The loads go out 32 values at a time, so the reduction
// costs a few memory round trips rather than one per value.  Returns true in
// the workgroup that must write Y.  INT: the values are int32 bit patterns,
// added as integers.
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
  for (int i = 0; i < NV; i++)
    __hip_atomic_store(mine + i * 64, v[i], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  __builtin_amdgcn_s_waitcnt(0);  // this workgroup's partials have completed
  __syncthreads();
  if (threadIdx.x == 0) {
    const uint32_t prev = __hip_atomic_fetch_add(a.cnt + 16 + tile, 1u, __ATOMIC_RELAXED,
                                                 __HIP_MEMORY_SCOPE_AGENT);
    s_last = prev == (uint32_t)(a.KS - 1);
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
      for (int i = 0; i < CH; i++)
        x[i] = k == ks ? v[i0 + i]
                       : __hip_atomic_load(src + (i0 + i) * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
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
// weights.  Two MFMAs (term 0, then term 1 accumulated onto it) multiply 16
// activation rows by 16 weight rows over one group; the group's fp32
// partial is scaled by the fp16 group scale in fp32 (int8 with unit scales:
// exact integer per group).
constexpr int kRT = 16;                  // activation rows per A-tile (one term each)
constexpr int kSplitShift = 4;           // binades between the two e4m3 terms
constexpr int kATBytes = 64 * 32 + 64;   // one A-tile of one group: fp8 bytes + exponents
constexpr int kF8BM = 64;                // activation rows per workgroup tile (4 x 2 A-tiles)
constexpr int kF8Threads = 512;          // 8 waves: 2 (rows) x 4 (columns)
constexpr int kF8Tiles = (kF8BM / kRT) * 2 * kATBytes;  // the 8 A-tiles of one workgroup tile and group
// Correction lists (ternary weights, bf16 activations).  Two e4m3 terms carry
// a bf16 element exactly when it lies within 2^13 of its 32-element block's
// maximum; a ternary row may weigh only the smaller elements of a block, so
// every element the terms miss is listed with its exact residual rho =
// x - (term 0 + term 1) (an fp32 number), and the GEMM adds code x rho x
// scale for it after the group's MFMAs.  One region per 16-row tile of the
// image: a count, then up to kEntries entries {slot position, rho}.  N(0,1)
// activations list about one element per 64-row tile and group; a region
// that overflows sends its wave to an exact recomputation of its outputs.
constexpr int kEntries = 15;
constexpr int kRegionBytes = 8 + 8 * kEntries;  // 128
constexpr int kHdrBytes = (kF8BM / kRT) * kRegionBytes;  // 512
constexpr int kF8Img = kF8Tiles + kHdrBytes;  // staged bytes of one workgroup tile and group

// Staging: one thread per (row m, group g, hardware block b).  Block b of a
// group holds k = 128 g + kmap(b, i), i = 0..31 (two runs of 16); A lane
// L = r + 16 kb (A row r, lane group kb) holds bytes e of the blocks with
// b & 1 = kb >> 1, i >> 4 = kb & 1, b >> 1 = e >> 4, i & 15 = e & 15, and
// lane L also supplies the exponent of (A row L % 16, block L / 16).
// Layout: per (64-row tile, group) kF8Img bytes; A-tile a of it at a *
// kATBytes: bytes 0..15 of the 64 lanes (16 L), bytes 16..31 (1024 + 16 L),
// then 64 exponent bytes (by lane): each 16-byte LDS read of the 64 lanes is
// one contiguous KiB (no bank conflicts).
// A-tile 2 rt + u holds term u of rows 16 rt .. 16 rt + 15 (A row = row % 16).
// Rows >= M are staged as zeros.  LIST (ternary weights, bf16): region rt of
// the header at kF8Tiles receives the correction list of rows 16 rt ..
// 16 rt + 15: word 0 the number of elements the terms miss, then entries
// {row % 16 | block << 4 | slot << 6, rho bits} in (row, block, slot) order.
template <int XK, bool LIST>
__global__ __launch_bounds__(256) void stage_f8(int64_t M, int64_t Mpad, int64_t K, int64_t G,
                                                const void* __restrict__ X,
                                                uint8_t* __restrict__ xs) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= Mpad * G * 4) return;
  // thread order: b fastest, then 16 consecutive rows, then g, so that a
  // wavefront's stores fill whole 512-byte runs of one A-tile (and its 64
  // exponent bytes) and its loads read 256-byte row segments
  const int b = (int)(tid & 3);
  const int64_t g = (tid >> 6) % G;
  const int64_t m = (tid >> 6) / G * 16 + ((tid >> 2) & 15);
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
  int E = 0;
  if constexpr (XK == XK_BF16) {
    float amax = 0.0f;
#pragma unroll
    for (int j = 0; j < 32; j++) amax = fmaxf(amax, fabsf(v[j]));
    // E puts the block maximum in [128, 256) x 2^E, clamped so that both
    // terms' exponents stay representable
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
  // term u of row m: A-tile 2 rt + u of the row's 64-row tile, A row r
  const int rt = (int)((m % kF8BM) / kRT), r = (int)(m % kRT);
  uint8_t* blk0 = xs + ((m / kF8BM) * G + g) * (int64_t)kF8Img + 2 * rt * kATBytes;
  uint8_t* blk1 = blk0 + kATBytes;
#pragma unroll
  for (int hh = 0; hh < 2; hh++) {
    const int kb = 2 * (b & 1) + hh;
    const int e = 16 * (b >> 1);
    *(v4u*)(blk0 + 64 * e + (r + 16 * kb) * 16) = v4u{w0[4 * hh], w0[4 * hh + 1], w0[4 * hh + 2], w0[4 * hh + 3]};
    *(v4u*)(blk1 + 64 * e + (r + 16 * kb) * 16) = v4u{w1[4 * hh], w1[4 * hh + 1], w1[4 * hh + 2], w1[4 * hh + 3]};
  }
  blk0[2048 + r + 16 * b] = (uint8_t)e0;
  blk1[2048 + r + 16 * b] = (uint8_t)e1;
  if constexpr (LIST && XK == XK_BF16) {
    // rho = v - (term 0 2^E + term 1 2^(E-4)), all exact in fp32 (the terms
    // and the powers of two are exact; their sum spans few enough binades)
    const float p0 = ldexpf(1.0f, E), p1 = ldexpf(1.0f, E - kSplitShift);
    float rho[32];
    uint32_t miss = 0;
#pragma unroll
    for (int j = 0; j < 8; j++) {
#pragma unroll
      for (int h = 0; h < 4; h++) {
        const int i = 4 * j + h;
        const float d0 = h == 0 ? __builtin_amdgcn_cvt_f32_fp8(w0[j], 0)
                       : h == 1 ? __builtin_amdgcn_cvt_f32_fp8(w0[j], 1)
                       : h == 2 ? __builtin_amdgcn_cvt_f32_fp8(w0[j], 2)
                                : __builtin_amdgcn_cvt_f32_fp8(w0[j], 3);
        const float d1 = h == 0 ? __builtin_amdgcn_cvt_f32_fp8(w1[j], 0)
                       : h == 1 ? __builtin_amdgcn_cvt_f32_fp8(w1[j], 1)
                       : h == 2 ? __builtin_amdgcn_cvt_f32_fp8(w1[j], 2)
                                : __builtin_amdgcn_cvt_f32_fp8(w1[j], 3);
        rho[i] = v[i] - (d0 * p0 + d1 * p1);
        miss |= (rho[i] != 0.0f ? 1u : 0u) << i;
      }
    }
    // this lane's entries follow those of the lanes before it in the
    // wavefront (16 rows x 4 blocks of one 16-row tile and group)
    const int lane = threadIdx.x & 63;
    const int cnt = __popc(miss);
    int incl = cnt;
#pragma unroll
    for (int d = 1; d < 64; d *= 2) {
      const int y = __shfl_up(incl, d);
      if (lane >= d) incl += y;
    }
    const int total = __shfl(incl, 63);
    uint8_t* region = xs + ((m / kF8BM) * G + g) * (int64_t)kF8Img + kF8Tiles + rt * kRegionBytes;
    if (lane == 0) *(uint32_t*)region = (uint32_t)total;
    if (miss) {
      int idx = incl - cnt;
#pragma unroll
      for (int i = 0; i < 32; i++) {
        if ((miss >> i) & 1u) {
          if (idx < kEntries)
            *(uint2*)(region + 8 + 8 * idx) =
                make_uint2((uint32_t)(r | (b << 4) | (i << 6)), __float_as_uint(rho[i]));
          idx++;
        }
      }
    }
  }
}

// ------------------------------------------------- sign activations (fp4 A)
// Sign-bit activations (x = alpha_m (-1)^bit) enter the MFMA as fp4 +-1, the
// same encoding as binary weights, with unit block scales: every product is
// +-1 x code and each group's MFMA result is the exact integer sum that
// XOR + popcount would give.  Image per (64-row tile, group): 4 A-tiles (16
// rows each) x 64 lanes x 16 bytes, lane L = r + 16 q holding slots 8 j + n
// (register j, nibble n) at k = 128 g + KMAP(q, 8 j + n), as the packed
// weights do.
constexpr int kS1Img = 4 * 1024;

// 8 sign bits -> 8 fp4 nibbles (bit 1 -> -1 = 0xA, 0 -> +1 = 0x2)
__device__ __forceinline__ uint32_t sign_nibbles(uint32_t b8) {
  uint32_t w = 0x22222222u;
#pragma unroll
  for (int n = 0; n < 8; n++) w |= ((b8 >> n) & 1u) << (4 * n + 3);
  return w;
}

// One thread per (row m, group g, quarter q); thread order q, then 16 rows,
// then g, so that a wavefront writes one contiguous KiB.  Rows >= M get
// zero nibbles (no contribution).
__global__ __launch_bounds__(256) void stage_s1(int64_t M, int64_t Mpad, int64_t K, int64_t G,
                                                const uint8_t* __restrict__ X,
                                                uint8_t* __restrict__ xs) {
  const int64_t tid = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (tid >= Mpad * G * 4) return;
  const int q = (int)(tid & 3), r = (int)((tid >> 2) & 15);
  const int64_t g = (tid >> 6) % G;
  const int64_t m = (tid >> 6) / G * 16 + r;
  v4u out = {0u, 0u, 0u, 0u};
  if (m < M) {
    const v4u bits = *(const v4u*)(X + m * (K / 8) + g * 16);  // the group's 128 bits
    // slots 0..15: k = run0 + i, slots 16..31: k = run0 + 32 + (i - 16)
    const int run0 = 64 * (q & 1) + 16 * (q >> 1);
    auto bits16 = [&](int k0) { return (bits[k0 >> 5] >> (k0 & 31)) & 0xFFFFu; };
    const uint32_t lo = bits16(run0), hi = bits16(run0 + 32);
    out = v4u{sign_nibbles(lo & 0xFF), sign_nibbles(lo >> 8), sign_nibbles(hi & 0xFF),
              sign_nibbles(hi >> 8)};
  }
  *(v4u*)(xs + ((m / kF8BM) * G + g) * (int64_t)kS1Img + ((m % kF8BM) / kRT) * 1024 +
          (r + 16 * q) * 16) = out;
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)v >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

__device__ __forceinline__ v4f mfma_f4f4(const v4u& A, const v8i& B) {
  const v8i A8 = v8i{(int)A.x, (int)A.y, (int)A.z, (int)A.w, 0, 0, 0, 0};
  // A and B fp4 e2m1 (4), unit block scales
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A8, B, v4f{0.f, 0.f, 0.f, 0.f}, 4, 4, 0,
                                                          127, 0, 127);
}

__device__ __forceinline__ v4f mfma_f8f4(const v8i& A, const v8i& B, int se, const v4f& C) {
  // A: fp8 e4m3 (0) with the E8M0 block exponent in byte 0 of se; B: fp4 e2m1 (4), unscaled
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, C, 0, 4, 0, se, 0, 127);
}

// LDS reads of the GEMM main loop, written out so that the compiler does not
// order them after the global -> LDS copies in flight (it cannot tell the
// LDS buffers apart and would wait for every copy); each block waits for its
// own results.
//
// A operands of two consecutive A-tiles (kATBytes apart: one row tile,
// both terms): this lane's two 16-byte halves at LDS byte addresses pa and
// pa + 1024, and their exponents at pe; when CNT also the entry counts of the
// wave's two correction regions (at ph and ph + kRegionBytes).  The main
// loop reads the second row tile's A-tiles while the first one's MFMAs run.
template <bool CNT>
__device__ __forceinline__ void lds_read_a2(uint32_t pa, uint32_t pe, uint32_t ph, v4u (&A0)[2],
                                            v4u (&A1)[2], uint32_t (&se)[2], uint32_t (&cnt)[2]) {
  if constexpr (CNT) {
    __asm__ volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %2, %8 offset:1024\n\t"
        "ds_read_u8 %4, %9\n\t"
        "ds_read_b128 %1, %8 offset:2112\n\t"
        "ds_read_b128 %3, %8 offset:3136\n\t"
        "ds_read_u8 %5, %9 offset:2112\n\t"
        "ds_read_b32 %6, %10\n\t"
        "ds_read_b32 %7, %10 offset:128\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(A0[0]), "=&v"(A0[1]), "=&v"(A1[0]), "=&v"(A1[1]), "=&v"(se[0]), "=&v"(se[1]),
          "=&v"(cnt[0]), "=&v"(cnt[1])
        : "v"(pa), "v"(pe), "v"(ph)
        : "memory");
  } else {
    // (issued while MFMAs that read these registers as their accumulator
    // input may still be in flight: wait states first, so that no returning
    // load overwrites an operand an MFMA pass has yet to read)
    __asm__ volatile(
        "s_nop 7\n\t"
        "s_nop 7\n\t"
        "ds_read_b128 %0, %6\n\t"
        "ds_read_b128 %2, %6 offset:1024\n\t"
        "ds_read_u8 %4, %7\n\t"
        "ds_read_b128 %1, %6 offset:2112\n\t"
        "ds_read_b128 %3, %6 offset:3136\n\t"
        "ds_read_u8 %5, %7 offset:2112\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(A0[0]), "=&v"(A0[1]), "=&v"(A1[0]), "=&v"(A1[1]), "=&v"(se[0]), "=&v"(se[1])
        : "v"(pa), "v"(pe)
        : "memory");
  }
}

static_assert(kATBytes == 2112 && kRegionBytes == 128, "LDS offsets of the A-tile reads");

// one 8-byte correction entry from LDS, waited for
__device__ __forceinline__ uint2 lds_read_entry(uint32_t addr) {
  uint2 v;
  __asm__ volatile("ds_read_b64 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(addr) : "memory");
  return v;
}

// fp4 A operands of two consecutive sign A-tiles (1 KiB apart) at pa
__device__ __forceinline__ void lds_read_s1(uint32_t pa, v4u (&A)[2]) {
  __asm__ volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:1024\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(A[0]), "=&v"(A[1])
                   : "v"(pa)
                   : "memory");
}

// Codes and scales of four row-blocks of a quad from their code-buffer slots
// (this lane's 16 bytes of each slot; base-3 also the slot's tail word) and
// their scales, with one wait.  Base-3 slots hold planes h and h + 1 of the
// octet, h = quad % 2: the quad's 8-byte chunks are (plane h: lo, hi; plane
// h + 1: lo) for h = 0 and (plane 1: hi; plane 2: lo, hi) for h = 1.
// Slots are CodeLds::kSlot apart and scales 128 bytes apart; pc, pt and ps
// are the first row-block's addresses.
template <int FMT>
__device__ __forceinline__ void lds_read_codes4(uint32_t pc, uint32_t pt, uint32_t ps, int h,
                                                Quad<FMT>* o) {
  if constexpr (FMT == 1) {
    __asm__ volatile(
        "ds_read_b128 %0, %8\n\t"
        "ds_read_b128 %1, %8 offset:1024\n\t"
        "ds_read_b128 %2, %8 offset:2048\n\t"
        "ds_read_b128 %3, %8 offset:3072\n\t"
        "ds_read_b64 %4, %9\n\t"
        "ds_read_b64 %5, %9 offset:128\n\t"
        "ds_read_b64 %6, %9 offset:256\n\t"
        "ds_read_b64 %7, %9 offset:384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0].w[0]), "=&v"(o[1].w[0]), "=&v"(o[2].w[0]), "=&v"(o[3].w[0]),
          "=&v"(o[0].sc), "=&v"(o[1].sc), "=&v"(o[2].sc), "=&v"(o[3].sc)
        : "v"(pc), "v"(ps)
        : "memory");
  } else if constexpr (FMT == 2) {
    __asm__ volatile(
        "ds_read_b128 %0, %12\n\t"
        "ds_read_b128 %1, %12 offset:1024\n\t"
        "ds_read_b128 %2, %12 offset:2048\n\t"
        "ds_read_b128 %3, %12 offset:3072\n\t"
        "ds_read_b128 %4, %12 offset:4096\n\t"
        "ds_read_b128 %5, %12 offset:5120\n\t"
        "ds_read_b128 %6, %12 offset:6144\n\t"
        "ds_read_b128 %7, %12 offset:7168\n\t"
        "ds_read_b64 %8, %13\n\t"
        "ds_read_b64 %9, %13 offset:128\n\t"
        "ds_read_b64 %10, %13 offset:256\n\t"
        "ds_read_b64 %11, %13 offset:384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(o[0].w[0]), "=&v"(o[0].w[1]), "=&v"(o[1].w[0]), "=&v"(o[1].w[1]),
          "=&v"(o[2].w[0]), "=&v"(o[2].w[1]), "=&v"(o[3].w[0]), "=&v"(o[3].w[1]),
          "=&v"(o[0].sc), "=&v"(o[1].sc), "=&v"(o[2].sc), "=&v"(o[3].sc)
        : "v"(pc), "v"(ps)
        : "memory");
  } else {
    u4 pa[4], pb[4];
    uint32_t tw[4];
    __asm__ volatile(
        "ds_read_b128 %0, %16\n\t"
        "ds_read_b128 %4, %16 offset:1024\n\t"
        "ds_read_b128 %1, %16 offset:2304\n\t"
        "ds_read_b128 %5, %16 offset:3328\n\t"
        "ds_read_b128 %2, %16 offset:4608\n\t"
        "ds_read_b128 %6, %16 offset:5632\n\t"
        "ds_read_b128 %3, %16 offset:6912\n\t"
        "ds_read_b128 %7, %16 offset:7936\n\t"
        "ds_read_b32 %8, %17\n\t"
        "ds_read_b32 %9, %17 offset:2304\n\t"
        "ds_read_b32 %10, %17 offset:4608\n\t"
        "ds_read_b32 %11, %17 offset:6912\n\t"
        "ds_read_b64 %12, %18\n\t"
        "ds_read_b64 %13, %18 offset:128\n\t"
        "ds_read_b64 %14, %18 offset:256\n\t"
        "ds_read_b64 %15, %18 offset:384\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(pa[0]), "=&v"(pa[1]), "=&v"(pa[2]), "=&v"(pa[3]), "=&v"(pb[0]), "=&v"(pb[1]),
          "=&v"(pb[2]), "=&v"(pb[3]), "=&v"(tw[0]), "=&v"(tw[1]), "=&v"(tw[2]), "=&v"(tw[3]),
          "=&v"(o[0].sc), "=&v"(o[1].sc), "=&v"(o[2].sc), "=&v"(o[3].sc)
        : "v"(pc), "v"(pt), "v"(ps)
        : "memory");
#pragma unroll
    for (int j = 0; j < 4; j++) {
      o[j].c30 = h ? u2{pa[j].z, pa[j].w} : u2{pa[j].x, pa[j].y};
      o[j].c31 = h ? u2{pb[j].x, pb[j].y} : u2{pa[j].z, pa[j].w};
      o[j].c32 = h ? u2{pb[j].z, pb[j].w} : u2{pb[j].x, pb[j].y};
      o[j].t3 = tw[j] >> (16 * h);
    }
  }
}

// Two row-blocks of 2-bit codes (the 4-wide read leaves the widest 2-bit
// kernel without registers to spare).
__device__ __forceinline__ void lds_read_codes2_t2(uint32_t pc, uint32_t ps, Quad<2>* o) {
  __asm__ volatile(
      "ds_read_b128 %0, %6\n\t"
      "ds_read_b128 %1, %6 offset:1024\n\t"
      "ds_read_b128 %2, %6 offset:2048\n\t"
      "ds_read_b128 %3, %6 offset:3072\n\t"
      "ds_read_b64 %4, %7\n\t"
      "ds_read_b64 %5, %7 offset:128\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(o[0].w[0]), "=&v"(o[0].w[1]), "=&v"(o[1].w[0]), "=&v"(o[1].w[1]), "=&v"(o[0].sc),
        "=&v"(o[1].sc)
      : "v"(pc), "v"(ps)
      : "memory");
}

// Workgroup tile 64 rows x 64 RBW columns, 8 waves: wave (wm, wn) owns
// A-tiles 4 wm .. 4 wm + 3 (rows 32 wm .. 32 wm + 31, both terms) and
// row-blocks RBW wn .. RBW wn + RBW - 1 (16 RBW columns).  RBW = 8 halves
// the LDS operand bytes per MFMA of RBW = 4 (each A-tile read feeds 8 row-
// blocks) for wide products.
//
// Every global read of the main loop is a direct global -> LDS copy
// (global_load_lds), so one counter of this wave's copies orders everything
// and the waits below are exact:
// * group images (kF8Img bytes) go into a ring of four LDS buffers, three
//   groups ahead: group g in buffer (g - g0) % 4, the static t of the
//   unrolled quad loop; each wave copies three pieces per image;
// * codes and scales of the next quad go into one LDS code buffer at the
//   second group of a quad; each wave copies those of RBW / 2 row-blocks, and
//   at the first group of a quad every wave reads its RBW row-blocks' codes
//   and scales from there into registers.
// Copies past the end of the workgroup's K range re-read its last image or
// quad into buffers that are no longer read, so that every group issues the
// same copies.
template <int FMT, int RBW>
struct CodeLds {
  static constexpr int kRows = 4 * RBW;  // row-blocks of the workgroup tile
  // bytes per row-block slot: binary one 1 KiB block, 2-bit the P0/P1 pair,
  // base-3 two 1 KiB planes of the octet + its 256-byte tail
  static constexpr int kSlot = FMT == 1 ? 1024 : FMT == 2 ? 2048 : 2304;
  static constexpr int kScales = kRows * kSlot;  // then 128 bytes of scales per row-block
  static constexpr int kBytes = kScales + kRows * 128;
  // copy instructions per wave per quad: RBW / 2 row-blocks' codes + one for scales
  static constexpr int kCopies = (RBW / 2) * (FMT == 1 ? 1 : FMT == 2 ? 2 : 3) + 1;
};

// s_waitcnt immediate: vmcnt n (6 bits, split over two fields), lgkmcnt 0,
// expcnt at its maximum
constexpr int vm_lgkm_wait(int n) { return (n & 15) | ((n >> 4) << 14) | 0x70; }

// Code of slot i of group T of a quad, for this lane's quarter, as three bits
// (bit 0: nonzero, bit 2: negative), with few registers.  2-bit: slot
// i = 8 j + p has its z bit at 4 p + 1 - (j & 1) of word P0 (j < 2) or P1
// and its s bit two above; the caller passes HI = (j >= 2) and the bit
// position zp.  Base-3: through the trit table (fp4 nibble: +1 = 0x2,
// -1 = 0xA, 0 = 0x0, so bits 1 and 3 of the nibble).
template <int FMT, int T, bool HI>
__device__ __forceinline__ uint32_t code3_at(const Quad<FMT>& qd, int i, int zp, const uint32_t* t3) {
  if constexpr (FMT == 2) {
    const u4 c4 = qd.w[T >> 1];
    const uint32_t w = HI ? ((T & 1) ? c4.w : c4.y) : ((T & 1) ? c4.z : c4.x);
    return (w >> zp) & 5u;
  } else {
    const v8i B = decode_group<FMT>(qd, T, t3);
    const int wi = i >> 3;
    const uint32_t wd = (uint32_t)(wi == 0 ? B[0] : wi == 1 ? B[1] : wi == 2 ? B[2] : B[3]);
    return (wd >> (4 * (i & 7) + 1)) & 5u;
  }
}

// fp4 operand B of group t of a quad, t chosen at run time
template <int FMT>
__device__ __forceinline__ v8i decode_group_rt(const Quad<FMT>& qd, int t, const uint32_t* t3) {
  return t == 0 ? decode_group<FMT>(qd, 0, t3) : t == 1 ? decode_group<FMT>(qd, 1, t3)
       : t == 2 ? decode_group<FMT>(qd, 2, t3) : decode_group<FMT>(qd, 3, t3);
}

// Exact recomputation, on the VALU, of one wave's outputs over groups
// [g0, g1) (bf16 activations): lane L = r + 16 q multiplies quarter q of row
// 16 rb + r by the activations of each of the wave's rows (products of
// +-1 / 0 are exact), the quarters are added, and each group's sum is scaled
// by its fp32 scale.  The slow path of a workgroup whose correction list
// overflowed; the results go through LDS (ex, 2 RBW 4 words per lane) so
// that the loops stay rolled.
template <int FMT, int RBW>
__device__ __attribute__((always_inline)) inline void exact_wave(const KArgs& a, int64_t mt, int wm, int64_t rb0,
                                                     int g0, int g1, const uint32_t* t3, float* ex) {
  const int lane = threadIdx.x & 63, q = lane >> 4;
  for (int j = 0; j < RBW; j++) {
    const int64_t rbc = rb0 + j < a.NB ? rb0 + j : a.NB - 1;
    for (int rt = 0; rt < 2; rt++) {
      float e0 = 0.f, e1 = 0.f, e2 = 0.f, e3 = 0.f;
      for (int g = g0; g < g1; g++) {
        Quad<FMT> qd;
        load_quad_at<FMT>(a.pcodes, a.pscales, rbc, g >> 2, a.GQ, a.GP, lane, qd);
        const v8i B = decode_group_rt<FMT>(qd, g & 3, t3);
        const float sc = quad_scale<FMT>(qd, g & 3);
        const int64_t k0 = (int64_t)g * kGroup + 64 * (q & 1) + 16 * (q >> 1);
        for (int mm = 0; mm < 16; mm++) {
          const int64_t m = mt * kF8BM + 32 * wm + 16 * rt + mm;
          float part = 0.f;
          if (m < a.M) {
#pragma unroll
            for (int h = 0; h < 2; h++) {  // slots 16 h .. 16 h + 15: k0 + 32 h + (i & 15)
              const v4u* src = (const v4u*)(a.x + m * a.K + k0 + 32 * h);
              const v4u w0 = src[0], w1 = src[1];
#pragma unroll
              for (int i = 0; i < 16; i++) {
                const uint32_t wd = i < 8 ? w0[i >> 1] : w1[(i - 8) >> 1];
                const float xv = __uint_as_float((i & 1) ? (wd & 0xFFFF0000u) : (wd << 16));
                const int slot = 16 * h + i;
                const uint32_t nib = ((uint32_t)B[slot >> 3] >> (4 * (slot & 7))) & 0xFu;
                part += nib == 0x2u ? xv : nib == 0xAu ? -xv : 0.0f;
              }
            }
          }
          part += __shfl_xor(part, 16);
          part += __shfl_xor(part, 32);
          if (q == (mm >> 2)) {
            const int e = mm & 3;
            if (e == 0) e0 = fmaf(sc, part, e0);
            else if (e == 1) e1 = fmaf(sc, part, e1);
            else if (e == 2) e2 = fmaf(sc, part, e2);
            else e3 = fmaf(sc, part, e3);
          }
        }
      }
      float* o = ex + ((rt * RBW + j) * 4) * 64 + lane;
      o[0] = e0;
      o[64] = e1;
      o[128] = e2;
      o[192] = e3;
    }
  }
}

template <int FMT, int XK, int YK, bool SCALED, int RBW>
__global__ __launch_bounds__(kF8Threads) __attribute__((amdgpu_waves_per_eu(2))) void gemm_f8(KArgs a) {
#if defined(__HIP_DEVICE_COMPILE__)  // LDS address-space code: device pass only
  using CL = CodeLds<FMT, RBW>;
  constexpr int HR = RBW / 2;  // row-blocks this wave copies
  constexpr bool S1 = XK == XK_SIGN1;  // sign activations: fp4 A, one term
  constexpr int IMG = S1 ? kS1Img : kF8Img;
  constexpr int XC = S1 ? 1 : 3;       // copies per image and wave
  __shared__ __attribute__((aligned(16))) uint8_t xb0[IMG], xb1[IMG], xb2[IMG], xb3[IMG];
  __shared__ __attribute__((aligned(16))) uint8_t cbuf[CL::kBytes];
  __shared__ uint32_t t3[256];
  auto ring = [&](int t) -> lds_u8* {
    return (lds_u8*)(t == 0 ? xb0 : t == 1 ? xb1 : t == 2 ? xb2 : xb3);
  };
  constexpr bool INT = (XK == XK_I8 || S1) && !SCALED;
  // ternary weights with bf16 activations: per-group correction lists
  constexpr bool LIST = FMT != 1 && XK == XK_BF16;
  // wave-uniform values are kept in scalar registers (the copy addresses
  // below are then a scalar base plus a fixed per-lane offset)
  const int tid = threadIdx.x, lane = tid & 63, wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  int64_t mt, nt, tail;
  int ks, nks;
  tile_of(a, mt, nt, ks, nks, tail);
  mt = uniform64(mt);
  nt = uniform64(nt);
  tail = uniform64(tail);
  ks = __builtin_amdgcn_readfirstlane(ks);
  nks = __builtin_amdgcn_readfirstlane(nks);
  // group and quad indices fit 32 bits (K < 2^38)
  const int q0 = __builtin_amdgcn_readfirstlane((int)(a.GQ * ks / nks));
  const int q1 = __builtin_amdgcn_readfirstlane((int)(a.GQ * (ks + 1) / nks));
  const int g0 = 4 * q0, g1 = 4 * q1 < (int)a.G ? 4 * q1 : (int)a.G;
  const int64_t rb0 = nt * CL::kRows + RBW * wn;  // this wave's first row-block
  if constexpr (FMT == 3) fill_trit_table(t3);

  // ---- copies.  Per-lane offsets stay in the same registers for the whole
  // loop (a copy's address registers must not change while it is in flight).
  const uint8_t* xs = a.xt + mt * a.G * (int64_t)IMG;
  static_assert(kF8Img == 16 * 1024 + 1024, "image = 16 KiB + 8 x 128 bytes");
  const uint32_t vo0 = 1024 * wave + 16 * lane, vo1 = vo0 + 8192;
  const uint32_t vo2 = 16384 + 128 * wave + 16 * lane;
  // image of group g into ring buffer t: 1 KiB chunks w and w + 8, and
  // 128 bytes of the 1 KiB tail (lanes 0..7: exponents, correction lists)
  // (sign images: 512 bytes per wave, lanes 0..31)
  const uint32_t vs = 512 * wave + 16 * lane;
  auto xissue = [&](int g, int t) {
    const uint8_t* src = xs + (int64_t)g * IMG;
    lds_u8* dst = ring(t);
    if constexpr (S1) {
      if (lane < 32) __builtin_amdgcn_global_load_lds(src + vs, dst + 512 * wave, 16, 0, 0);
    } else {
      __builtin_amdgcn_global_load_lds(src + vo0, dst + 1024 * wave, 16, 0, 0);
      __builtin_amdgcn_global_load_lds(src + vo1, dst + 1024 * (wave + 8), 16, 0, 0);
      if (lane < 8) __builtin_amdgcn_global_load_lds(src + vo2, dst + 16384 + 128 * wave, 16, 0, 0);
    }
  };
  // this wave copies row-blocks RBW wn + HR wm .. + HR - 1 of the tile
  const int cr = RBW * wn + HR * wm;
  int64_t crb[HR];
#pragma unroll
  for (int u = 0; u < HR; u++) {
    const int64_t rb = nt * CL::kRows + cr + u;
    crb[u] = rb < a.NB ? rb : a.NB - 1;
  }
  const uint32_t lo16 = 16 * lane;
  const int64_t GO = (a.GQ + 1) / 2;
  const uint8_t* sbase = a.pscales ? (const uint8_t*)a.pscales : a.pcodes;
  auto cissue = [&](int gq) {
    lds_u8* cb = (lds_u8*)cbuf;
#pragma unroll
    for (int u = 0; u < HR; u++) {
      lds_u8* slot = cb + (cr + u) * CL::kSlot;
      if constexpr (FMT == 1) {
        const uint8_t* src = a.pcodes + (crb[u] * a.GQ + gq) * 1024;
        __builtin_amdgcn_global_load_lds(src + lo16, slot, 16, 0, 0);
      } else if constexpr (FMT == 2) {
        const int64_t p0 = 2 * gq, p1 = 2 * gq + 1 < a.GP ? 2 * gq + 1 : a.GP - 1;
        __builtin_amdgcn_global_load_lds(a.pcodes + (crb[u] * a.GP + p0) * 1024 + lo16, slot, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(a.pcodes + (crb[u] * a.GP + p1) * 1024 + lo16, slot + 1024,
                                         16, 0, 0);
      } else {
        // planes h, h + 1 of octet gq / 2 (h = gq % 2) and the 256-byte tail
        const uint8_t* ob = a.pcodes + (crb[u] * GO + (gq >> 1)) * 3328 + 1024 * (gq & 1);
        __builtin_amdgcn_global_load_lds(ob + lo16, slot, 16, 0, 0);
        __builtin_amdgcn_global_load_lds(ob + 1024 + lo16, slot + 1024, 16, 0, 0);
        const uint8_t* tail = a.pcodes + (crb[u] * GO + (gq >> 1)) * 3328 + 3072;
        if (lane < 16) __builtin_amdgcn_global_load_lds(tail + lo16, slot + 2048, 16, 0, 0);
      }
    }
    // scales of the HR row-blocks: lanes 8u .. 8u + 7 gather row-block u's 128 bytes
    if (lane < 8 * HR) {
      const int u = lane >> 3;
      const uint8_t* src = sbase + (crb[u] * a.GQ + gq) * 128 + 16 * (lane & 7);
      __builtin_amdgcn_global_load_lds(src, cb + CL::kScales + 128 * cr, 16, 0, 0);
    }
  };
  // Wait until the copies that the coming group reads have landed, with
  // `later` copies issued after them still in flight, and for this wave's
  // LDS accesses; then the workgroup barrier.  Copies complete in issue
  // order.  The barrier carries no memory fence: a workgroup fence would
  // also wait for every copy still in flight.
  auto xsync = [&](auto later) {
    __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(decltype(later)::value));
    __builtin_amdgcn_s_barrier();
    __asm__ volatile("" ::: "memory");
  };
  // ---- LDS reads (written out, see lds_read_a / lds_read_codes)

  // codes and scales of row-blocks RBW wn + j .. + 3 of the quad in the code buffer
  static_assert(RBW % 4 == 0, "code reads go four row-blocks at a time");
  static_assert(CL::kSlot == (FMT == 1 ? 1024 : FMT == 2 ? 2048 : 2304), "slot offsets of the code reads");
  auto cread4 = [&](int j, int gq, Quad<FMT>* o) {
    const uint32_t slot = (uint32_t)(uintptr_t)((lds_u8*)cbuf + (RBW * wn + j) * CL::kSlot);
    const uint32_t sc = (uint32_t)(uintptr_t)((lds_u8*)cbuf + CL::kScales + (RBW * wn + j) * 128) +
                        8 * (lane & 15);
    if constexpr (FMT == 2 && RBW == 8) {
      lds_read_codes2_t2(slot + lo16, sc, o);
      lds_read_codes2_t2(slot + 2 * CL::kSlot + lo16, sc + 256, o + 2);
    } else {
      lds_read_codes4<FMT>(slot + lo16, slot + 2048 + 4 * lane, sc, gq & 1, o);
    }
  };

  // acc[rt][j][e]: row 32 wm + 16 rt + 4 (lane / 16) + e, column 16 (RBW wn + j) + lane % 16
  float acc[2][RBW][4];
  int iacc[2][RBW][4];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < RBW; j++)
#pragma unroll
      for (int e = 0; e < 4; e++) {
        acc[i][j][e] = 0.f;
        iacc[i][j][e] = 0;
      }

  // prologue: codes of quad q0, then images g0 .. g0 + 2
  cissue(q0);
#pragma unroll
  for (int t = 0; t < 3; t++) xissue(g0 + t < g1 ? g0 + t : g1 - 1, t);

  Quad<FMT> qd[RBW];
  bool overflow = false;  // (LIST) one of the wave's correction lists overflowed
  // binary decode masks in registers (VOP3 takes no literal): v_and_or_b32
  uint32_t sign_mask = 0x88888888u, one_bits = 0x22222222u;
  if constexpr (FMT == 1) {
    asm volatile("v_mov_b32 %0, 0x88888888" : "=v"(sign_mask));
    asm volatile("s_mov_b32 %0, 0x22222222" : "=s"(one_bits));
  }
  for (int q = q0; q < q1; q++) {
#pragma unroll
    for (int t = 0; t < 4; t++) {
      const int g = 4 * q + t;
      if (g < g1) {
        // issued after the copies this group needs: two images, and at t =
        // 2, 3 also the next quad's codes (issued at t = 1 after its image)
        if (t < 2)
          xsync(std::integral_constant<int, 2 * XC>());
        else
          xsync(std::integral_constant<int, 2 * XC + CL::kCopies>());
        if (t == 0) {
#pragma unroll
          for (int j = 0; j < RBW; j += 4) cread4(j, q, qd + j);
        }
        xissue(g + 3 < g1 ? g + 3 : g1 - 1, (t + 3) & 3);
        if (t == 1) cissue(q + 1 < q1 ? q + 1 : q);
        v8i At[4];
        uint32_t se[4];
        v4u As[2];
        uint32_t ncorr[2] = {0u, 0u};  // (LIST) entries in the wave's two regions
        if constexpr (S1) {
          lds_read_s1((uint32_t)(uintptr_t)(ring(t) + 2 * wm * 1024) + 16 * lane, As);
        } else {
          // the first row tile's two A-tiles (and the correction counts of
          // both regions) now, the second row tile's during the first one's MFMAs
          v4u A0[2], A1[2];
          uint32_t se2[2];
          const uint32_t base = (uint32_t)(uintptr_t)(ring(t) + 4 * wm * kATBytes);
          const uint32_t ph = (uint32_t)(uintptr_t)(ring(t) + kF8Tiles + 2 * wm * kRegionBytes);
          lds_read_a2<LIST>(base + 16 * lane, base + 2048 + lane, ph, A0, A1, se2, ncorr);
#pragma unroll
          for (int i = 0; i < 2; i++) {
            At[i] = v8i{(int)A0[i].x, (int)A0[i].y, (int)A0[i].z, (int)A0[i].w,
                        (int)A1[i].x, (int)A1[i].y, (int)A1[i].z, (int)A1[i].w};
            se[i] = se2[i];
          }
        }
        if constexpr (LIST) {
          // the elements the two terms miss: acc[row][col] += s code rho
          // (added before the group's MFMA results, while few registers are live).
          // Lane 16 b + r holds block b's codes of row r (its quarter), lane
          // 16 lg + r the outputs of rows 4 lg .. 4 lg + 3 of the row tile.
          const uint32_t n0 = __builtin_amdgcn_readfirstlane(ncorr[0]);
          const uint32_t n1 = __builtin_amdgcn_readfirstlane(ncorr[1]);
          if (n0 | n1) {
            if (__builtin_expect(n0 > (uint32_t)kEntries || n1 > (uint32_t)kEntries, 0)) {
              overflow = true;
            } else {
              const uint32_t ph = (uint32_t)(uintptr_t)(ring(t) + kF8Tiles + 2 * wm * kRegionBytes);
#pragma unroll
              for (int rt = 0; rt < 2; rt++) {
                const uint32_t ne = rt == 0 ? n0 : n1;
#pragma unroll 1
                for (uint32_t ei = 0; ei < ne; ei++) {
                  const uint2 ent = lds_read_entry(ph + rt * kRegionBytes + 8 + 8 * ei);
                  const uint32_t pos = __builtin_amdgcn_readfirstlane(ent.x);
                  const float rho = __uint_as_float(__builtin_amdgcn_readfirstlane(ent.y));
                  const int row16 = pos & 15, b = (pos >> 4) & 3, i = (pos >> 6) & 31;
                  // the lanes of quarter b pack the slot's code of every
                  // row-block (three bits each); one lane move brings them to
                  // the lanes that hold row16's outputs
                  const int zp = 4 * (i & 7) + 1 - ((i >> 3) & 1);
                  uint32_t packed = 0;
                  auto pack = [&](auto hi) {
#pragma unroll
                    for (int j = 0; j < RBW; j++) {
                      const uint32_t c3 = t == 0 ? code3_at<FMT, 0, decltype(hi)::value>(qd[j], i, zp, t3)
                                        : t == 1 ? code3_at<FMT, 1, decltype(hi)::value>(qd[j], i, zp, t3)
                                        : t == 2 ? code3_at<FMT, 2, decltype(hi)::value>(qd[j], i, zp, t3)
                                                 : code3_at<FMT, 3, decltype(hi)::value>(qd[j], i, zp, t3);
                      packed |= c3 << (3 * j);
                    }
                  };
                  if (i >= 16) pack(std::true_type());  // uniform
                  else pack(std::false_type());
                  packed = (uint32_t)__shfl((int)packed, 16 * b + (lane & 15));
                  const bool dst = (lane >> 4) == (row16 >> 2);
                  const int ev = row16 & 3;
                  const float nrho = -rho;
                  float val[RBW];
#pragma unroll
                  for (int j = 0; j < RBW; j++) {
                    const uint32_t c3 = dst ? (packed >> (3 * j)) & 5u : 0u;
                    const float cr = c3 == 1u ? rho : c3 == 5u ? nrho : 0.0f;
                    val[j] = quad_scale<FMT>(qd[j], t) * cr;
                  }
#pragma unroll
                  for (int e = 0; e < 4; e++) {
                    if (ev == e) {  // uniform
#pragma unroll
                      for (int j = 0; j < RBW; j++) acc[rt][j][e] += val[j];
                    }
                  }
                }
              }
            }
          }
        }
        // row-blocks four at a time: decode, then per row-tile rt (16 rows)
        // term 0 (A-tile 2 rt) and term 1 (2 rt + 1) accumulate into one MFMA
        // result (sign activations: one fp4 A-tile per row-tile), scaled once
        // per group
#pragma unroll
        for (int h = 0; h < RBW; h += 4) {
          v8i B[4];
          float sj[4];
#pragma unroll
          for (int j = 0; j < 4; j++) {
            if constexpr (FMT == 1) {
              const u4 c4 = qd[h + j].w[0];
              B[j] = decode_binary_reg(t == 0 ? c4.x : t == 1 ? c4.y : t == 2 ? c4.z : c4.w, sign_mask,
                                       one_bits);
            } else {
              B[j] = decode_group<FMT>(qd[h + j], t, t3);
            }
            // (the exact int32 product is the only one without scales)
            sj[j] = INT ? 1.0f : quad_scale<FMT>(qd[h + j], t);
          }
#pragma unroll
          for (int rt = 0; rt < 2; rt++) {
            v4f c[4];
            if constexpr (S1) {
#pragma unroll
              for (int j = 0; j < 4; j++) c[j] = mfma_f4f4(As[rt], B[j]);
            } else {
#pragma unroll
              for (int j = 0; j < 4; j++)
                c[j] = mfma_f8f4(At[2 * rt], B[j], (int)se[2 * rt], v4f{0.f, 0.f, 0.f, 0.f});
#pragma unroll
              for (int j = 0; j < 4; j++) c[j] = mfma_f8f4(At[2 * rt + 1], B[j], (int)se[2 * rt + 1], c[j]);
              if (h == 0 && rt == 0) {
                // the second row tile's A-tiles, while these MFMAs run (before
                // their results are read)
                v4u A0[2], A1[2];
                uint32_t se2[2], nc2[2];
                const uint32_t base = (uint32_t)(uintptr_t)(ring(t) + (4 * wm + 2) * kATBytes);
                lds_read_a2<false>(base + 16 * lane, base + 2048 + lane, 0u, A0, A1, se2, nc2);
#pragma unroll
                for (int i = 0; i < 2; i++) {
                  At[2 + i] = v8i{(int)A0[i].x, (int)A0[i].y, (int)A0[i].z, (int)A0[i].w,
                                  (int)A1[i].x, (int)A1[i].y, (int)A1[i].z, (int)A1[i].w};
                  se[2 + i] = se2[i];
                }
              }
            }
#pragma unroll
            for (int j = 0; j < 4; j++) {
#pragma unroll
              for (int e = 0; e < 4; e++) {
                if constexpr (INT)
                  iacc[rt][h + j][e] += __float2int_rn(c[j][e]);
                else
                  acc[rt][h + j][e] = fmaf(sj[j], c[j][e], acc[rt][h + j][e]);
              }
            }
          }
        }
      }
    }
  }
  // no copy may still be writing LDS when the workgroup ends
  __builtin_amdgcn_s_waitcnt(vm_lgkm_wait(0));
  if constexpr (LIST) {
    // more missed elements than a list holds: the workgroup's outputs
    // exactly (every wave; the LDS buffers are free once all have left the loop)
    if (__builtin_expect(__syncthreads_or(overflow ? 1 : 0), 0)) {
      float* ex = wave < 4 ? (float*)ring(wave) : (float*)((lds_u8*)cbuf + (wave - 4) * 2 * RBW * 4 * 64 * 4);
      exact_wave<FMT, RBW>(a, mt, wm, rb0, g0, g1, t3, ex);
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int j = 0; j < RBW; j++)
#pragma unroll
          for (int e = 0; e < 4; e++) acc[i][j][e] = ex[((i * RBW + j) * 4 + e) * 64 + lane];
    }
  }

  constexpr int NV = 2 * RBW * 4;
  uint32_t v[NV];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int j = 0; j < RBW; j++)
#pragma unroll
      for (int e = 0; e < 4; e++)
        v[(i * RBW + j) * 4 + e] = INT ? (uint32_t)iacc[i][j][e] : __float_as_uint(acc[i][j][e]);
  if (nks > 1 && !split_reduce<NV, INT, kF8Threads>(a, tail, ks, wave, lane, v)) return;
#pragma unroll
  for (int i = 0; i < 2; i++) {
#pragma unroll
    for (int e = 0; e < 4; e++) {
      const int64_t row = mt * kF8BM + 32 * wm + 16 * i + 4 * (lane >> 4) + e;
      if (row >= a.M) continue;
      const float rs = SCALED ? a.rowscale[row] : 1.0f;
#pragma unroll
      for (int j = 0; j < RBW; j++) {
        const int64_t col = (rb0 + j) * 16 + (lane & 15);
        if (rb0 + j >= a.NB || col >= a.N) continue;
        const uint32_t x = v[(i * RBW + j) * 4 + e];
        if constexpr (INT)
          store_y<YK>(a.y, row * a.N + col, (int32_t)x);
        else
          store_y<YK>(a.y, row * a.N + col, __uint_as_float(x) * rs);
      }
    }
  }
#endif
}

// ---------------------------------------------------------------- planning
struct GemmPlan {
  int64_t MT, NT, G, KS, F;
  int RBW;
  int row_fast;  // tile order of the launch (see tile_of)
  size_t xt_off, rs_off, part_off, bytes;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

// K-split count when the tile grid does not fill the 256 compute units once
// (one workgroup each): the smallest that keeps at least ~85% of a whole
// number of waves of workgroups busy, up to 8 and at most one quad of groups
// per split.  Grids of a full round or more are not split (the partial sums
// would cost more HBM traffic than the idle tail).
int64_t pick_splits(int64_t tiles, int64_t GQ) {
  const int64_t slots = 256;
  if (tiles >= slots) return 1;
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

// Grids of whole rounds and a partial last one: the tiles of the last round
// may be split along K (2, 4 or 8 ways) so that their work spreads over
// every compute unit, when the round time saved (a round of whole tiles
// estimated at ~1 PFLOP/s) outweighs the partial tiles' extra HBM traffic
// (written once and read once, at ~5 TB/s).  Returns the split count (1: no
// split); the whole rounds' tiles run unsplit.
int64_t pick_tail_splits(int64_t tail, int64_t GQ, int64_t K, int RBW) {
  const double round_s = 64.0 * 64 * RBW * (double)K * 2 * 256 / 1.0e15;
  const double part_tile = 64.0 * 64 * RBW * 4;
  int64_t best = 1;
  double best_gain = 0.0;
  for (int64_t ks = 2; ks <= 8 && ks <= GQ; ks *= 2) {
    if ((tail * ks) % 8 != 0) continue;
    const double saved = (1.0 - (double)cdiv(tail * ks, (int64_t)256) / (double)ks) * round_s;
    // (with half again as much for the last arrival's reduction latency)
    const double cost = 1.5 * 2.0 * (double)tail * ks * part_tile / 5.0e12;
    if (saved - cost > best_gain) {
      best = ks;
      best_gain = saved - cost;
    }
  }
  return best;
}

GemmPlan make_gemm_plan(int fmt, int xkind, int64_t M, int64_t N, int64_t K) {
  GemmPlan p;
  p.G = K / kGroup;
  p.MT = cdiv(M, kF8BM);
  // 512-column tiles for wide products, 256 otherwise (base-3 codes need
  // more registers per row-block than a 512-column wave tile leaves)
  p.RBW = N >= 2048 && fmt != 3 ? 8 : 4;
  p.NT = cdiv(N, 64 * p.RBW);
  const int64_t tiles = p.MT * p.NT;
  if (tiles < 256) {  // less than one round: every tile split alike
    p.F = 0;
    p.KS = pick_splits(tiles, cdiv(p.G, 4));
  } else {
    const int64_t tail = tiles % 256;
    p.KS = tail == 0 ? 1 : pick_tail_splits(tail, cdiv(p.G, 4), K, p.RBW);
    p.F = p.KS > 1 ? tiles - tail : tiles;
  }
  // packed weight bytes (codes and scales) against staged activation bytes
  const double wbytes = (double)N * K * (fmt == 1 ? 1.0 : fmt == 2 ? 2.0 : 1.625) / 8 + (double)N * p.G * 2;
  const double xbytes = (double)p.MT * p.G * (xkind == XK_SIGN1 ? kS1Img : kF8Img);
  p.row_fast = wbytes > xbytes ? 1 : 0;
  p.rs_off = kCounterBytes;
  p.xt_off = p.rs_off;
  p.part_off = p.xt_off + align256((size_t)p.MT * p.G * (xkind == XK_SIGN1 ? kS1Img : kF8Img));
  const size_t part_tile = (size_t)kF8BM * 64 * p.RBW * 4;
  p.bytes = p.part_off + (p.KS > 1 ? (size_t)p.KS * (tiles - p.F) * part_tile : 0);
  return p;
}

template <int FMT, int RBW>
hipError_t launch_fmt(const GemmArgs& g, const GemmPlan& p, hipStream_t s) {
  uint8_t* ws = (uint8_t*)g.ws;
  KArgs k;
  k.xt = ws + p.xt_off;
  k.pcodes = (const uint8_t*)g.pcodes;
  k.pscales = g.pscales;
  k.rowscale = g.xkind != XK_BF16 ? g.x_scales : nullptr;
  k.y = g.y;
  k.part = (float*)(ws + p.part_off);
  k.cnt = (uint32_t*)ws;
  k.x = (const uint16_t*)g.x;
  k.K = g.K;
  k.M = g.M;
  k.N = g.N;
  k.G = p.G;
  k.GQ = cdiv(p.G, 4);
  k.GP = cdiv(p.G, 2);
  k.NB = cdiv(g.N, 16);
  k.MT = p.MT;
  k.NT = p.NT;
  k.KS = (int)p.KS;
  k.F = p.F;
  k.row_fast = p.row_fast;
  const int64_t Mpad = p.MT * kF8BM;
  const int64_t units = Mpad * p.G * 4;
  const dim3 sgrid((unsigned)cdiv(units, 256));
  const dim3 grid((unsigned)(p.F + (p.MT * p.NT - p.F) * p.KS)), block(kF8Threads);
  if (g.xkind == XK_BF16) {
    hipLaunchKernelGGL((stage_f8<XK_BF16, FMT != 1>), sgrid, dim3(256), 0, s, g.M, Mpad, g.K, p.G, g.x,
                       (uint8_t*)k.xt);
    if (g.ykind == YK_BF16)
      hipLaunchKernelGGL((gemm_f8<FMT, XK_BF16, YK_BF16, false, RBW>), grid, block, 0, s, k);
    else
      hipLaunchKernelGGL((gemm_f8<FMT, XK_BF16, YK_F32, false, RBW>), grid, block, 0, s, k);
    return hipGetLastError();
  }
  if (g.xkind == XK_SIGN1) {
    hipLaunchKernelGGL(stage_s1, sgrid, dim3(256), 0, s, g.M, Mpad, g.K, p.G, (const uint8_t*)g.x,
                       (uint8_t*)k.xt);
    if (g.ykind == YK_I32)
      hipLaunchKernelGGL((gemm_f8<FMT, XK_SIGN1, YK_I32, false, RBW>), grid, block, 0, s, k);
    else if (g.ykind == YK_BF16)
      hipLaunchKernelGGL((gemm_f8<FMT, XK_SIGN1, YK_BF16, true, RBW>), grid, block, 0, s, k);
    else
      hipLaunchKernelGGL((gemm_f8<FMT, XK_SIGN1, YK_F32, true, RBW>), grid, block, 0, s, k);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((stage_f8<XK_I8, false>), sgrid, dim3(256), 0, s, g.M, Mpad, g.K, p.G, g.x,
                     (uint8_t*)k.xt);
  if (g.ykind == YK_I32)
    hipLaunchKernelGGL((gemm_f8<FMT, XK_I8, YK_I32, false, RBW>), grid, block, 0, s, k);
  else if (g.ykind == YK_BF16)
    hipLaunchKernelGGL((gemm_f8<FMT, XK_I8, YK_BF16, true, RBW>), grid, block, 0, s, k);
  else
    hipLaunchKernelGGL((gemm_f8<FMT, XK_I8, YK_F32, true, RBW>), grid, block, 0, s, k);
  return hipGetLastError();
}

template <int FMT>
hipError_t launch_rbw(const GemmArgs& g, const GemmPlan& p, hipStream_t s) {
  if constexpr (FMT == 3)
    return launch_fmt<FMT, 4>(g, p, s);
  else
    return p.RBW == 8 ? launch_fmt<FMT, 8>(g, p, s) : launch_fmt<FMT, 4>(g, p, s);
}

}  // namespace

size_t gemm_workspace_bytes(int fmt, int xkind, int64_t M, int64_t N, int64_t K) {
  return make_gemm_plan(fmt, xkind, M, N, K).bytes;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.xkind != XK_BF16 && g.xkind != XK_I8 && g.xkind != XK_SIGN1) return hipErrorInvalidValue;
  if (g.xkind == XK_BF16 && g.ykind == YK_I32) return hipErrorInvalidValue;
  if (g.xkind != XK_BF16 && (g.ykind == YK_I32) != (g.pscales == nullptr)) return hipErrorInvalidValue;
  if (g.xkind != XK_BF16 && g.ykind != YK_I32 && g.x_scales == nullptr) return hipErrorInvalidValue;
  const GemmPlan p = make_gemm_plan(g.fmt, g.xkind, g.M, g.N, g.K);
  if (p.F + (p.MT * p.NT - p.F) * p.KS > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (g.fmt == 1) return launch_rbw<1>(g, p, s);
  if (g.fmt == 2) return launch_rbw<2>(g, p, s);
  if (g.fmt == 3) return launch_rbw<3>(g, p, s);
  return hipErrorInvalidValue;
}

}  // namespace lowbit
