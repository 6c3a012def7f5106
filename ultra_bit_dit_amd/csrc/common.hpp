// Internal definitions shared by the HIP sources of liblowbit (not part of
// the public ABI).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

constexpr int kGroup = 128;  // weights per FP16 scale

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));
typedef short v8s __attribute__((ext_vector_type(8)));

__host__ __device__ inline int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

// k offset inside a group of slot i (0..31) of quarter q (0..3): the order in
// which the fp4 B operand of the 16x16x128 f8f6f4 MFMA consumes k relative
// to the fp8 A operand (lane = row + 16 * quarter).
__host__ __device__ inline int kmap(int q, int i) {
  return 64 * (q & 1) + 16 * (q >> 1) + 32 * (i >> 4) + (i & 15);
}

// binary word: slot held by bit b (bit b lands in nibble b>>2 of fp4
// register 3-(b&3) after the decode shift)
__host__ __device__ inline int bin_slot(int b) { return 8 * (3 - (b & 3)) + (b >> 2); }

// fp16 bit pattern (low 16 bits of h) -> fp32, exact
__device__ inline float f16_bits_to_f32(uint32_t h) {
  return (float)__builtin_bit_cast(_Float16, (unsigned short)(h & 0xFFFFu));
}

// Activation operand scheme of the batch-1 / small-M kernels.  Activations
// enter v_mfma_scale_f32_16x16x128_f8f6f4 as R low-precision split terms per
// element, one row of A per term, each 32-element block with its own E8M0
// exponent: E puts the block maximum in [2^kTop, 2^(kTop+1)) and term r
// carries exponent E - kShift r.
//   * ternary weights, bf16 activations: three e5m2 terms (3 significant bits
//     each; exact for every element within 2^30 of its block maximum);
//   * binary weights, bf16: two e4m3 terms (exact within 2^13 of the block
//     maximum; smaller elements err by at most 2^-21 of it, and a binary row
//     always weighs the maximum, so the error stays far inside the bound);
//   * fp32: four e4m3 terms (16 significant bits);
//   * int8 q: 16 (q >> 4) + (q & 15), exact.
// Inputs the terms do not carry accurately enough are detected while staging
// and their products are recomputed exactly (see the kernels).
constexpr int split_terms(int fmt, int xkind) {
  return xkind == 1 /* F32 */ ? 4 : (xkind == 2 /* BF16 */ && fmt != 1) ? 3 : 2;
}

enum XKind { XK_F32 = 1, XK_BF16 = 2, XK_I8 = 3, XK_SIGN1 = 4 };
enum YKind { YK_F32 = 1, YK_BF16 = 2, YK_I32 = 5 };

// ------------------------------------------------------------ launchers
// (host side, defined in the .hip files; every one returns a hipError_t)

hipError_t launch_pack(int fmt, int64_t N, int64_t K, const int8_t* codes,
                       const uint16_t* scales, void* pcodes, void* pscales,
                       int32_t* bad, hipStream_t s);
hipError_t launch_unpack(int fmt, int64_t N, int64_t K, const void* pcodes,
                         const void* pscales, int8_t* codes, uint16_t* scales,
                         int32_t* bad, hipStream_t s);
hipError_t launch_quantize_i8(int64_t M, int64_t K, const uint16_t* X, int8_t* Q,
                              float* sx, hipStream_t s);


// Workspace of the fused GEMV: a fixed block of zero-initialised counters
// (self-resetting: every launch leaves them zero) followed by the staged
// activations and the split-K partial sums.
constexpr int64_t kCounterWords = 65536;
constexpr int64_t kCounterBytes = kCounterWords * 4;
constexpr int64_t kMaxRowGroups = kCounterWords - 16;  // row groups of 64 rows
// batch-1 sign activations: the reordered sign words of a row (K / 8 bytes)
// are built in 48 KiB of LDS per workgroup
constexpr int64_t kSignMaxK = 48 * 1024 * 8;

struct GemvArgs {
  int fmt;
  int64_t N, K, M;          // M activation rows (1 for a GEMV)
  const void* pcodes;
  const uint16_t* pscales;  // NULL = unit scales
  int xkind;                // XK_F32 / XK_BF16 / XK_I8
  const void* x;            // [M][K] activations
  float x_scale;            // multiplies the result (I8 s_x of a GEMV); 1 otherwise
  const float* x_scales;    // per-row result scales (small-M I8), or NULL
  int ykind;
  void* y;                  // [M][N]
  void* ws;                 // workspace (counters first)
};
// bytes of workspace the fused GEMV needs (counters included)
size_t gemv_workspace_bytes(int fmt, int64_t N, int64_t K, int64_t M, int xkind);
hipError_t launch_gemv_mfma(const GemvArgs& a, hipStream_t s);

// Persistent chain of batch-1 products (one cooperative launch runs them all;
// product i may wait for product i-1 to complete before reading its x)
struct ChainStage {
  int fmt;
  int64_t N, K;
  const void* pcodes;
  const uint16_t* pscales;
  const void* x;
  void* y;
  int wait_prev;
  int epi;  // 1: SiLU-mul epilogue (N fused gate/up rows -> N/2 outputs)
};
hipError_t chain_create(const ChainStage* st, int S, int64_t M, int xkind, int ykind, void** plan);
hipError_t chain_run(void* plan, hipStream_t s);
hipError_t chain_status(void* plan, int* failed_waits);
void chain_destroy(void* plan);

struct SignArgs {
  int64_t N, K, M;
  const void* pcodes;
  const uint16_t* pscales;
  const uint8_t* xbits;  // K sign bits (the kernel reorders them into the binary word order)
  float alpha;
  int ykind;
  void* y;
};
hipError_t launch_gemv_sign(const SignArgs& a, hipStream_t s);

// Large-M GEMM (activations staged into per-(row tile, group) tiles in the
// workspace, then MFMA over decoded weight registers)
struct GemmArgs {
  int fmt;
  int64_t M, N, K;
  const void* pcodes;
  const uint16_t* pscales;  // NULL only for the exact int32 product
  int xkind;                // XK_BF16, XK_I8 or XK_SIGN1
  const void* x;            // [M][K] (sign bits: [M][K/8])
  const float* x_scales;    // per-row scales of int8 / sign activations (scaled outputs)
  int ykind;
  void* y;                  // [M][N]
  void* ws;                 // workspace (counters first)
};
size_t gemm_workspace_bytes(int fmt, int xkind, int64_t M, int64_t N, int64_t K);
hipError_t launch_gemm(const GemmArgs& a, hipStream_t s);

// streaming read of `bytes` (a multiple of 16) at src; XOR of the data into *out
hipError_t launch_hbm_read(const void* src, int64_t bytes, uint32_t* out, hipStream_t s);

// data-free weight quantizer and the matching activation rotation
hipError_t launch_quantize_weights(int fmt, int64_t N, int64_t K, const uint16_t* W,
                                   const int8_t* signs, int8_t* codes, uint16_t* scales,
                                   hipStream_t s);
hipError_t launch_rotate_act(int64_t M, int64_t K, const uint16_t* X, const int8_t* signs,
                             float* Xr, hipStream_t s);

}  // namespace lowbit
