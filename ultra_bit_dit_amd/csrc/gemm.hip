// Large-M products Y[M][N] = X[M][K] . W[N][K]^T over packed binary or 2-bit
// ternary weights with one fp16 scale per 128-weight group (the group-scaled
// matmul of the "1-bit 嘅數學" section of the ultra_bit_dit page; prefill and
// diffusion-transformer blocks run it as a dense contraction).
//
// Two kernels, both MFMA 32x32 on gfx950:
//
// * bf16 activations -> fp16 MFMA (32x32x16, fp32 accumulate).  The group
//   scale is folded into the weight operand: a weight is +s, -s or 0, which
//   fp16 holds exactly because s is an fp16 number.  Activations are
//   converted to fp16 after an exact per-row power-of-two rescale (bf16 has a
//   wider exponent range than fp16), so every product is exact and only the
//   fp32 accumulation rounds; the row's power of two is undone on output.
//   No per-group epilogue is needed.
// * int8 activations -> int8 MFMA (32x32x32, int32 accumulate).  Per group
//   the int32 sum is exact; it is scaled by the group scale in fp32 and,
//   after the last group, by the row's activation scale.  Without scales the
//   int32 sum over all of K is returned exactly.
//
// Activations are first staged (a separate pass over X) into 128-row tiles,
// one per (row tile, group), with the k order of each group permuted to the
// order in which the packed weight bits decode, and the 16-byte chunks of
// each tile row XOR-swizzled so that the MFMA operand reads from LDS are
// free of bank conflicts.  The GEMM copies a tile to LDS with plain
// coalesced 16-byte loads and stores.
//
// Weights are read straight from the packed layout into registers and
// decoded there (each wave decodes only the columns it owns).
#include <algorithm>

#include "common.hpp"

namespace lowbit {
namespace {

typedef unsigned v4u __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef short v2s __attribute__((ext_vector_type(2)));

constexpr int kTM = 128;          // activation rows per tile
constexpr int kTileF16 = kTM * 256;  // bytes of a staged fp16 tile (128 rows x 128 k)
constexpr int kTileI8 = kTM * 128;   // bytes of a staged int8 tile
constexpr int kThreads = 256;

// ---------------------------------------------------------------- k order
// Position p (0..127) of a staged group row <-> k offset inside the group.
//
// fp16 path: MFMA t (0..7) of the group, lane half h, operand element i
// (0..7) sits at p = 16 t + 8 h + i and multiplies the weight slot that the
// decode of the lane's words puts there.  The lane (column n, half h) owns
// quarters 2h and 2h+1 of column n's group; MFMA t takes quarter 2h + t/4.
__host__ __device__ inline int perm_f16(int fmt, int p) {
  const int t = p >> 4, h = (p >> 3) & 1, i = p & 7;
  const int q = 2 * h + (t >> 2);
  // binary: register j = 4 (t%4) + i/2 takes bit j (low half) and bit j+16 (high half)
  // ternary: word P_{(t/2)%2}; registers p' = i/2 hold slots (p', p'+4) for
  //          even t, (8+p', 12+p') for odd t
  const int slot = fmt == 1 ? bin_slot(4 * (t & 3) + (i >> 1) + 16 * (i & 1))
                            : 16 * ((t >> 1) & 1) + 8 * (t & 1) + (i >> 1) + 4 * (i & 1);
  return kmap(q, slot);
}

// int8 path: MFMA tt (0..3), half h, element i (0..15) at p = 32 tt + 16 h + i
__host__ __device__ inline int perm_i8(int fmt, int p) {
  const int tt = p >> 5, h = (p >> 4) & 1, i = p & 15;
  const int q = 2 * h + (tt >> 1);
  // binary: register j = 4 (tt%2) + i/4 holds bits j, j+8, j+16, j+24 as bytes
  // ternary: word P_{tt%2}; register v = i/4 holds slots 8 (v/2) + 2 e + v%2
  const int slot = fmt == 1 ? bin_slot(4 * (tt & 1) + (i >> 2) + 8 * (i & 3))
                            : 16 * (tt & 1) + 8 * (i >> 3) + 2 * (i & 3) + ((i >> 2) & 1);
  return kmap(q, slot);
}

// staged tile byte offset of 16-byte chunk c of tile row r (rows of 256 B
// for fp16, 128 B for int8)
__host__ __device__ inline int swz_f16(int r, int c) { return r * 256 + ((c ^ (r & 7)) << 4); }
__host__ __device__ inline int swz_i8(int r, int c) { return r * 128 + ((c ^ (r & 7)) << 4); }

// ---------------------------------------------------------------- staging
// One block per activation row: exponent of the row maximum, then the fp16
// (rescaled) values in staged order.  xinv[m] = 2^-e undoes the rescale.
template <int FMT>
__global__ __launch_bounds__(256) void stage_f16(int64_t M, int64_t K, int64_t G,
                                                 const uint16_t* __restrict__ X,
                                                 uint8_t* __restrict__ xt,
                                                 float* __restrict__ xinv) {
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const uint16_t* row = X + m * K;
  float a = 0.0f;
  for (int64_t k = threadIdx.x; k < K; k += 256)
    a = fmaxf(a, fabsf(__uint_as_float((uint32_t)row[k] << 16)));
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  // e puts the row maximum in [2^14, 2^15): every finite product with an
  // fp16 scale stays finite in fp32 and rescaling is exact
  int e = 0;
  if (a > 0.0f && a <= 3.0e38f) {
    int ex;
    (void)frexpf(a, &ex);
    e = min(max(15 - ex, -126), 126);
  }
  const float up = ldexpf(1.0f, e);
  if (threadIdx.x == 0) xinv[m] = ldexpf(1.0f, -e);
  const int64_t mt = m / kTM;
  const int r = (int)(m % kTM);
  for (int64_t ci = threadIdx.x; ci < G * 16; ci += 256) {
    const int64_t g = ci >> 4;
    const int c = (int)(ci & 15);
    const uint16_t* src = row + g * kGroup;
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float v0 = __uint_as_float((uint32_t)src[perm_f16(FMT, 8 * c + 2 * j)] << 16) * up;
      const float v1 = __uint_as_float((uint32_t)src[perm_f16(FMT, 8 * c + 2 * j + 1)] << 16) * up;
      const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;  // round to nearest even
      h[j] = (uint32_t)__builtin_bit_cast(unsigned short, h0) |
             ((uint32_t)__builtin_bit_cast(unsigned short, h1) << 16);
    }
    uint8_t* dst = xt + (mt * G + g) * (int64_t)kTileF16 + swz_f16(r, c);
    *(v4u*)dst = v4u{h[0], h[1], h[2], h[3]};
  }
}

// The same with the row read once, coalesced, into LDS (rows up to
// kStageLdsMax elements): the maximum is taken during that read and the
// permuted gather then reads LDS instead of global memory.
constexpr int64_t kStageLdsMax = 24576;  // bf16 elements (48 KiB of LDS)

template <int FMT>
__global__ __launch_bounds__(256) void stage_f16_lds(int64_t M, int64_t K, int64_t G,
                                                     const uint16_t* __restrict__ X,
                                                     uint8_t* __restrict__ xt,
                                                     float* __restrict__ xinv) {
  __shared__ __attribute__((aligned(16))) uint16_t srow[kStageLdsMax];
  __shared__ float red[4];
  const int64_t m = blockIdx.x;
  const v4u* row = (const v4u*)(X + m * K);
  float a = 0.0f;
  for (int64_t k8 = threadIdx.x; k8 < K / 8; k8 += 256) {
    const v4u w = row[k8];
    ((v4u*)srow)[k8] = w;
#pragma unroll
    for (int j = 0; j < 4; j++) {
      a = fmaxf(a, fabsf(__uint_as_float(w[j] << 16)));
      a = fmaxf(a, fabsf(__uint_as_float(w[j] & 0xFFFF0000u)));
    }
  }
  for (int off = 32; off > 0; off >>= 1) a = fmaxf(a, __shfl_xor(a, off));
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = a;
  __syncthreads();
  a = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
  int e = 0;
  if (a > 0.0f && a <= 3.0e38f) {
    int ex;
    (void)frexpf(a, &ex);
    e = min(max(15 - ex, -126), 126);
  }
  const float up = ldexpf(1.0f, e);
  if (threadIdx.x == 0) xinv[m] = ldexpf(1.0f, -e);
  const int64_t mt = m / kTM;
  const int r = (int)(m % kTM);
  for (int64_t ci = threadIdx.x; ci < G * 16; ci += 256) {
    const int64_t g = ci >> 4;
    const int c = (int)(ci & 15);
    const uint16_t* src = srow + g * kGroup;
    uint32_t h[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      const float v0 = __uint_as_float((uint32_t)src[perm_f16(FMT, 8 * c + 2 * j)] << 16) * up;
      const float v1 = __uint_as_float((uint32_t)src[perm_f16(FMT, 8 * c + 2 * j + 1)] << 16) * up;
      const _Float16 h0 = (_Float16)v0, h1 = (_Float16)v1;  // round to nearest even
      h[j] = (uint32_t)__builtin_bit_cast(unsigned short, h0) |
             ((uint32_t)__builtin_bit_cast(unsigned short, h1) << 16);
    }
    uint8_t* dst = xt + (mt * G + g) * (int64_t)kTileF16 + swz_f16(r, c);
    *(v4u*)dst = v4u{h[0], h[1], h[2], h[3]};
  }
}

template <int FMT>
__global__ __launch_bounds__(256) void stage_i8(int64_t M, int64_t K, int64_t G,
                                                const int8_t* __restrict__ X,
                                                uint8_t* __restrict__ xt) {
  const int64_t m = blockIdx.x;
  const uint8_t* row = (const uint8_t*)X + m * K;
  const int64_t mt = m / kTM;
  const int r = (int)(m % kTM);
  for (int64_t ci = threadIdx.x; ci < G * 8; ci += 256) {
    const int64_t g = ci >> 3;
    const int c = (int)(ci & 7);
    const uint8_t* src = row + g * kGroup;
    uint32_t v[4];
#pragma unroll
    for (int j = 0; j < 4; j++) {
      v[j] = 0;
#pragma unroll
      for (int b = 0; b < 4; b++) v[j] |= (uint32_t)src[perm_i8(FMT, 16 * c + 4 * j + b)] << (8 * b);
    }
    uint8_t* dst = xt + (mt * G + g) * (int64_t)kTileI8 + swz_i8(r, c);
    *(v4u*)dst = v4u{v[0], v[1], v[2], v[3]};
  }
}

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
template <int NV, bool INT>
__device__ __forceinline__ bool split_reduce(const KArgs& a, int64_t tile, int ks, int wave,
                                             int lane, uint32_t (&v)[NV]) {
  constexpr int CH = 32;  // values per batch of loads
  static_assert(NV % CH == 0, "partial tile in whole batches");
  __shared__ uint32_t s_last;
  const int64_t per = (int64_t)(kThreads / 64) * NV * 64;  // words of one partial tile
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

// ----------------------------------------------------- fp16 (bf16 input) GEMM
// Workgroup tile 128 rows x 256 columns; wave w owns columns 64w..64w+63
// (two 32-column MFMA blocks) for all 128 rows (four 32-row blocks).
constexpr int kF16Cols = 256;

// packed words of one group for the lane's two column blocks
template <int FMT>
struct WordsF16 {
  uint32_t w[2][FMT == 1 ? 2 : 4];  // [block][quarter e (binary) | 2e + P-index (ternary)]
  uint32_t s2[2];                   // fp16 scale in both halves
};

template <int FMT>
__device__ __forceinline__ WordsF16<FMT> load_words_f16(const KArgs& a, const int64_t (&rb)[2],
                                                        int r, int h, int64_t g) {
  WordsF16<FMT> o;
#pragma unroll
  for (int b = 0; b < 2; b++) {
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int L = r + 16 * (2 * h + e);
      if constexpr (FMT == 1) {
        const uint32_t* p = (const uint32_t*)a.pcodes + ((rb[b] * a.GQ + (g >> 2)) * 64 + L) * 4 + (g & 3);
        o.w[b][e] = __builtin_nontemporal_load(p);
      } else {
        const uint32_t* p = (const uint32_t*)a.pcodes + ((rb[b] * a.GP + (g >> 1)) * 64 + L) * 4 + 2 * (g & 1);
        o.w[b][2 * e] = __builtin_nontemporal_load(p);
        o.w[b][2 * e + 1] = __builtin_nontemporal_load(p + 1);
      }
    }
    const uint32_t s = a.pscales[((rb[b] * a.GQ + (g >> 2)) * 16 + r) * 4 + (g & 3)];
    o.s2[b] = s | (s << 16);
  }
  return o;
}

// weight operand of MFMA t for one column block: 8 fp16 values +-s / 0
template <int FMT>
__device__ __forceinline__ v8h decode_f16(const WordsF16<FMT>& W, int b, int t) {
  uint32_t v[4];
  const uint32_t s2 = W.s2[b];
  if constexpr (FMT == 1) {
    const uint32_t w = W.w[b][t >> 2];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int j = 4 * (t & 3) + k;
      v[k] = s2 ^ ((w << (15 - j)) & 0x80008000u);
    }
  } else {
    const uint32_t P = W.w[b][2 * (t >> 2) + ((t >> 1) & 1)];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      // even t: slots (k, k+4): z at 4k+1, s at 4k+3; odd t: slots (8+k, 12+k): z 4k, s 4k+2
      const int ss = (t & 1) ? 13 - 4 * k : 12 - 4 * k;
      const uint32_t sg = s2 ^ ((P << ss) & 0x80008000u);
      const v2s z = __builtin_bit_cast(v2s, P << (ss + 2)) >> (short)15;
      v[k] = sg & __builtin_bit_cast(uint32_t, z);
    }
  }
  return __builtin_bit_cast(v8h, v4u{v[0], v[1], v[2], v[3]});
}

template <int FMT, int YK>
__global__ __launch_bounds__(kThreads) void gemm_f16(KArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kTileF16];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int n = lane & 31, h = lane >> 5, r = n & 15;
  int64_t mt, nt;
  int ks;
  tile_of(a, mt, nt, ks);
  const int64_t g0 = a.G * ks / a.KS, g1 = a.G * (ks + 1) / a.KS;
  const int64_t col0 = nt * kF16Cols + wave * 64;
  int64_t rb[2];
#pragma unroll
  for (int b = 0; b < 2; b++) rb[b] = min((col0 + 32 * b + n) >> 4, a.NB - 1);
  const uint8_t* xt = a.xt + mt * a.G * (int64_t)kTileF16;

  v16f acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int b = 0; b < 2; b++) acc[i][b] = v16f{};

  v4u xr[8];
#pragma unroll
  for (int j = 0; j < 8; j++) xr[j] = *(const v4u*)(xt + g0 * kTileF16 + (j * kThreads + tid) * 16);
#pragma unroll
  for (int j = 0; j < 8; j++) *(v4u*)(&lds[0][(j * kThreads + tid) * 16]) = xr[j];
  WordsF16<FMT> wc = load_words_f16<FMT>(a, rb, r, h, g0);
  __syncthreads();

  for (int64_t g = g0; g < g1; g++) {
    const int buf = (int)((g - g0) & 1);
    const int64_t gn = g + 1 < g1 ? g + 1 : g;
#pragma unroll
    for (int j = 0; j < 8; j++) xr[j] = *(const v4u*)(xt + gn * kTileF16 + (j * kThreads + tid) * 16);
    const WordsF16<FMT> wn = load_words_f16<FMT>(a, rb, r, h, gn);
    const uint8_t* L = lds[buf];
    // software pipeline over the 8 MFMA steps of the group: the operands of
    // step t+1 are read from LDS and decoded while the MFMAs of step t run
    v8h A[2][4], B[2][2];
#pragma unroll
    for (int i = 0; i < 4; i++)
      A[0][i] = __builtin_bit_cast(v8h, *(const v4u*)(L + swz_f16(32 * i + n, h)));
#pragma unroll
    for (int b = 0; b < 2; b++) B[0][b] = decode_f16<FMT>(wc, b, 0);
#pragma unroll
    for (int t = 0; t < 8; t++) {
      const int cu = t & 1, nx = cu ^ 1;
      if (t + 1 < 8) {
#pragma unroll
        for (int i = 0; i < 4; i++)
          A[nx][i] = __builtin_bit_cast(v8h, *(const v4u*)(L + swz_f16(32 * i + n, 2 * (t + 1) + h)));
#pragma unroll
        for (int b = 0; b < 2; b++) B[nx][b] = decode_f16<FMT>(wc, b, t + 1);
      }
#pragma unroll
      for (int i = 0; i < 4; i++)
#pragma unroll
        for (int b = 0; b < 2; b++)
          acc[i][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(A[cu][i], B[cu][b], acc[i][b], 0, 0, 0);
      if (t == 3 && g + 1 < g1) {
        // the next group's activation tile into the other buffer
#pragma unroll
        for (int j = 0; j < 8; j++) *(v4u*)(&lds[buf ^ 1][(j * kThreads + tid) * 16]) = xr[j];
      }
    }
    wc = wn;
    __syncthreads();
  }

  uint32_t v[128];
#pragma unroll
  for (int i = 0; i < 4; i++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int q = 0; q < 16; q++) v[(i * 2 + b) * 16 + q] = __float_as_uint(acc[i][b][q]);
  if (a.KS > 1 && !split_reduce<128, false>(a, mt * a.NT + nt, ks, wave, lane, v)) return;
#pragma unroll
  for (int i = 0; i < 4; i++) {
#pragma unroll
    for (int q = 0; q < 16; q++) {
      const int64_t row = mt * kTM + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
      if (row >= a.M) continue;
      const float rs = a.rowscale[row];
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const int64_t col = col0 + 32 * b + n;
        if (col < a.N) store_y<YK>(a.y, row * a.N + col, __uint_as_float(v[(i * 2 + b) * 16 + q]) * rs);
      }
    }
  }
}

// ------------------------------------------------------------- int8 GEMM
// Workgroup tile 128 x 128; waves in a 2 x 2 grid, each 64 rows (two 32-row
// blocks) x 64 columns (two 32-column blocks).
constexpr int kI8Cols = 128;

template <int FMT>
struct WordsI8 {
  uint32_t w[2][FMT == 1 ? 2 : 4];
  float s[2];
};

template <int FMT, bool SCALED>
__device__ __forceinline__ WordsI8<FMT> load_words_i8(const KArgs& a, const int64_t (&rb)[2],
                                                      int r, int h, int64_t g) {
  WordsI8<FMT> o;
#pragma unroll
  for (int b = 0; b < 2; b++) {
#pragma unroll
    for (int e = 0; e < 2; e++) {
      const int L = r + 16 * (2 * h + e);
      if constexpr (FMT == 1) {
        const uint32_t* p = (const uint32_t*)a.pcodes + ((rb[b] * a.GQ + (g >> 2)) * 64 + L) * 4 + (g & 3);
        o.w[b][e] = __builtin_nontemporal_load(p);
      } else {
        const uint32_t* p = (const uint32_t*)a.pcodes + ((rb[b] * a.GP + (g >> 1)) * 64 + L) * 4 + 2 * (g & 1);
        o.w[b][2 * e] = __builtin_nontemporal_load(p);
        o.w[b][2 * e + 1] = __builtin_nontemporal_load(p + 1);
      }
    }
    if constexpr (SCALED)
      o.s[b] = f16_bits_to_f32(a.pscales[((rb[b] * a.GQ + (g >> 2)) * 16 + r) * 4 + (g & 3)]);
    else
      o.s[b] = 0.0f;
  }
  return o;
}

// weight operand of MFMA tt for one column block: 16 int8 values -1/0/+1,
// each byte chosen by v_perm from a two-entry (binary) or four-entry
// (ternary) table indexed by the code bits
template <int FMT>
__device__ __forceinline__ v4i decode_i8(const WordsI8<FMT>& W, int b, int tt) {
  uint32_t v[4];
  if constexpr (FMT == 1) {
    const uint32_t w = W.w[b][tt >> 1];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const uint32_t sel = (w >> (4 * (tt & 1) + k)) & 0x01010101u;  // 0 -> +1, 1 -> -1
      v[k] = __builtin_amdgcn_perm(0x0000FF01u, 0x0000FF01u, sel);
    }
  } else {
    const uint32_t P = W.w[b][2 * (tt >> 1) + (tt & 1)];
#pragma unroll
    for (int k = 0; k < 4; k++) {
      const int sh = k == 0 ? 1 : k == 1 ? 5 : k == 2 ? 0 : 4;
      // per byte: bit 0 = nonzero, bit 2 = sign -> index 0, 1, 4, 5
      const uint32_t sel = (P >> sh) & 0x05050505u;
      v[k] = __builtin_amdgcn_perm(0x0000FF00u, 0x00000100u, sel);
    }
  }
  return v4i{(int)v[0], (int)v[1], (int)v[2], (int)v[3]};
}

template <int FMT, int YK, bool SCALED>
__global__ __launch_bounds__(kThreads) void gemm_i8(KArgs a) {
  __shared__ __attribute__((aligned(16))) uint8_t lds[2][kTileI8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;
  const int n = lane & 31, h = lane >> 5, r = n & 15;
  int64_t mt, nt;
  int ks;
  tile_of(a, mt, nt, ks);
  const int64_t g0 = a.G * ks / a.KS, g1 = a.G * (ks + 1) / a.KS;
  const int64_t col0 = nt * kI8Cols + wn * 64;
  int64_t rb[2];
#pragma unroll
  for (int b = 0; b < 2; b++) rb[b] = min((col0 + 32 * b + n) >> 4, a.NB - 1);
  const uint8_t* xt = a.xt + mt * a.G * (int64_t)kTileI8;

  v16f acc[2][2];
  v16i iacc[2][2];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int b = 0; b < 2; b++) {
      acc[i][b] = v16f{};
      iacc[i][b] = v16i{};
    }

  v4u xr[4];
#pragma unroll
  for (int j = 0; j < 4; j++) xr[j] = *(const v4u*)(xt + g0 * kTileI8 + (j * kThreads + tid) * 16);
#pragma unroll
  for (int j = 0; j < 4; j++) *(v4u*)(&lds[0][(j * kThreads + tid) * 16]) = xr[j];
  WordsI8<FMT> wc = load_words_i8<FMT, SCALED>(a, rb, r, h, g0);
  __syncthreads();

  for (int64_t g = g0; g < g1; g++) {
    const int buf = (int)((g - g0) & 1);
    const int64_t gn = g + 1 < g1 ? g + 1 : g;
#pragma unroll
    for (int j = 0; j < 4; j++) xr[j] = *(const v4u*)(xt + gn * kTileI8 + (j * kThreads + tid) * 16);
    const WordsI8<FMT> wn2 = load_words_i8<FMT, SCALED>(a, rb, r, h, gn);
    const uint8_t* L = lds[buf];
    if constexpr (SCALED) {
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int b = 0; b < 2; b++) iacc[i][b] = v16i{};
    }
    // operands of step tt+1 are read and decoded while the MFMAs of step tt run
    v4i A[2][2], B[2][2];
#pragma unroll
    for (int i = 0; i < 2; i++)
      A[0][i] = __builtin_bit_cast(v4i, *(const v4u*)(L + swz_i8(64 * wm + 32 * i + n, h)));
#pragma unroll
    for (int b = 0; b < 2; b++) B[0][b] = decode_i8<FMT>(wc, b, 0);
#pragma unroll
    for (int tt = 0; tt < 4; tt++) {
      const int cu = tt & 1, nx = cu ^ 1;
      if (tt + 1 < 4) {
#pragma unroll
        for (int i = 0; i < 2; i++)
          A[nx][i] = __builtin_bit_cast(v4i, *(const v4u*)(L + swz_i8(64 * wm + 32 * i + n, 2 * (tt + 1) + h)));
#pragma unroll
        for (int b = 0; b < 2; b++) B[nx][b] = decode_i8<FMT>(wc, b, tt + 1);
      }
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int b = 0; b < 2; b++)
          iacc[i][b] = __builtin_amdgcn_mfma_i32_32x32x32_i8(A[cu][i], B[cu][b], iacc[i][b], 0, 0, 0);
    }
    if constexpr (SCALED) {
#pragma unroll
      for (int i = 0; i < 2; i++)
#pragma unroll
        for (int b = 0; b < 2; b++)
#pragma unroll
          for (int q = 0; q < 16; q++)
            acc[i][b][q] = fmaf(wc.s[b], (float)iacc[i][b][q], acc[i][b][q]);
    }
    if (g + 1 < g1) {
#pragma unroll
      for (int j = 0; j < 4; j++) *(v4u*)(&lds[buf ^ 1][(j * kThreads + tid) * 16]) = xr[j];
    }
    wc = wn2;
    __syncthreads();
  }

  uint32_t v[64];
#pragma unroll
  for (int i = 0; i < 2; i++)
#pragma unroll
    for (int b = 0; b < 2; b++)
#pragma unroll
      for (int q = 0; q < 16; q++)
        v[(i * 2 + b) * 16 + q] =
            SCALED ? __float_as_uint(acc[i][b][q]) : (uint32_t)iacc[i][b][q];
  if (a.KS > 1 && !split_reduce<64, !SCALED>(a, mt * a.NT + nt, ks, wave, lane, v)) return;
#pragma unroll
  for (int i = 0; i < 2; i++) {
#pragma unroll
    for (int q = 0; q < 16; q++) {
      const int64_t row = mt * kTM + 64 * wm + 32 * i + 8 * (q >> 2) + 4 * h + (q & 3);
      if (row >= a.M) continue;
      const float rs = SCALED ? a.rowscale[row] : 1.0f;
#pragma unroll
      for (int b = 0; b < 2; b++) {
        const int64_t col = col0 + 32 * b + n;
        if (col >= a.N) continue;
        const uint32_t x = v[(i * 2 + b) * 16 + q];
        if constexpr (SCALED)
          store_y<YK>(a.y, row * a.N + col, __uint_as_float(x) * rs);
        else
          store_y<YK>(a.y, row * a.N + col, (int32_t)x);
      }
    }
  }
}

// ---------------------------------------------------------------- planning
struct GemmPlan {
  int64_t MT, NT, G, KS;
  size_t xt_off, rs_off, part_off, bytes;
  bool f16;
};

size_t align256(size_t v) { return (v + 255) / 256 * 256; }

GemmPlan make_gemm_plan(int64_t M, int64_t N, int64_t K, int xkind) {
  GemmPlan p;
  p.f16 = xkind == XK_BF16;
  p.G = K / kGroup;
  p.MT = cdiv(M, kTM);
  p.NT = cdiv(N, p.f16 ? kF16Cols : kI8Cols);
  const int64_t tiles = p.MT * p.NT;
  // split K when the tiles alone leave most compute units idle
  p.KS = 1;
  if (tiles < 192) p.KS = std::min<int64_t>(std::min<int64_t>(cdiv(256, tiles), 8), std::max<int64_t>(1, p.G / 4));
  if (tiles > kMaxRowGroups) p.KS = 1;
  const size_t tile_bytes = p.f16 ? kTileF16 : kTileI8;
  p.rs_off = kCounterBytes;
  p.xt_off = p.rs_off + align256((size_t)M * 4);
  p.part_off = p.xt_off + align256((size_t)p.MT * p.G * tile_bytes);
  const size_t part_tile = (size_t)kTM * (p.f16 ? kF16Cols : kI8Cols) * 4;
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
  const dim3 grid((unsigned)(p.MT * p.NT * p.KS)), block(kThreads);
  if (p.f16) {
    float* rs = (float*)(ws + p.rs_off);
    k.rowscale = rs;
    if (g.K <= kStageLdsMax && ((uintptr_t)g.x % 16) == 0)
      hipLaunchKernelGGL(stage_f16_lds<FMT>, dim3((unsigned)g.M), dim3(256), 0, s, g.M, g.K, p.G,
                         (const uint16_t*)g.x, (uint8_t*)k.xt, rs);
    else
      hipLaunchKernelGGL(stage_f16<FMT>, dim3((unsigned)g.M), dim3(256), 0, s, g.M, g.K, p.G,
                         (const uint16_t*)g.x, (uint8_t*)k.xt, rs);
    if (g.ykind == YK_BF16)
      hipLaunchKernelGGL((gemm_f16<FMT, YK_BF16>), grid, block, 0, s, k);
    else
      hipLaunchKernelGGL((gemm_f16<FMT, YK_F32>), grid, block, 0, s, k);
    return hipGetLastError();
  }
  k.rowscale = g.x_scales;
  hipLaunchKernelGGL(stage_i8<FMT>, dim3((unsigned)g.M), dim3(256), 0, s, g.M, g.K, p.G,
                     (const int8_t*)g.x, (uint8_t*)k.xt);
  if (g.ykind == YK_I32)
    hipLaunchKernelGGL((gemm_i8<FMT, YK_I32, false>), grid, block, 0, s, k);
  else if (g.ykind == YK_BF16)
    hipLaunchKernelGGL((gemm_i8<FMT, YK_BF16, true>), grid, block, 0, s, k);
  else
    hipLaunchKernelGGL((gemm_i8<FMT, YK_F32, true>), grid, block, 0, s, k);
  return hipGetLastError();
}

}  // namespace

size_t gemm_workspace_bytes(int64_t M, int64_t N, int64_t K, int xkind) {
  return make_gemm_plan(M, N, K, xkind).bytes;
}

hipError_t launch_gemm(const GemmArgs& g, hipStream_t s) {
  if (g.xkind != XK_BF16 && g.xkind != XK_I8) return hipErrorInvalidValue;
  if (g.xkind == XK_BF16 && g.ykind == YK_I32) return hipErrorInvalidValue;
  if (g.xkind == XK_I8 && (g.ykind == YK_I32) != (g.pscales == nullptr)) return hipErrorInvalidValue;
  if (g.xkind == XK_I8 && g.ykind != YK_I32 && g.x_scales == nullptr) return hipErrorInvalidValue;
  const GemmPlan p = make_gemm_plan(g.M, g.N, g.K, g.xkind);
  if (p.MT * p.NT * p.KS > 0x7FFFFFFF) return hipErrorInvalidValue;
  if (g.fmt == 1) return launch_fmt<1>(g, p, s);
  if (g.fmt == 2) return launch_fmt<2>(g, p, s);
  return hipErrorInvalidValue;
}

}  // namespace lowbit
