/*
 * oracle.h -- plain, slow, fp64 CPU reference for group-scaled binary and
 * ternary matrix products.  TEST INFRASTRUCTURE ONLY: the tests, the smoke
 * check and the benchmark's CPU-baseline leg may call it; the product
 * library never does, and it shares no code with the HIP path.
 *
 * Every function restates a definition from the pages (cited per function in
 * oracle.c) or the byte layout written in the layout specification of the
 * library header, re-implemented here from that text.
 */
#ifndef LOWBIT_ORACLE_H
#define LOWBIT_ORACLE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* format ids and activation kinds, numbered as in the layout specification */
#define ORC_BINARY 1
#define ORC_TERNARY_2BIT 2
#define ORC_TERNARY_BASE3 3

#define ORC_X_F32 1
#define ORC_X_BF16 2
#define ORC_X_I8 3
#define ORC_X_SIGN1 4

double orc_f16_to_f64(uint16_t h);
double orc_bf16_to_f64(uint16_t b);

/* 0 on success, -1 bad format, -2 bad shape */
int orc_packed_bytes(int fmt, int64_t N, int64_t K, size_t* code_bytes,
                     size_t* scale_bytes);

/* returns the number of codes outside the format's value set (they are
 * packed as 0 / +1), or a negative error */
int64_t orc_pack(int fmt, int64_t N, int64_t K, const int8_t* codes,
                 const uint16_t* scales, uint8_t* pcodes, uint16_t* pscales);

/* returns the number of reserved / out-of-range packed values met inside the
 * N x K region (decoded as 0), or a negative error */
int64_t orc_unpack(int fmt, int64_t N, int64_t K, const uint8_t* pcodes,
                   const uint16_t* pscales, int8_t* codes, uint16_t* scales);

/* Y[m][n] = sum_k scale[n][k/128] * code[n][k] * x(m, k) in fp64 and
 * absY[m][n] = sum_k |scale * code * x| (absY may be NULL).  scales may be
 * NULL (all 1).  xs: per-row s_x (I8) or alpha (SIGN1), NULL means 1. */
int orc_matmul(int64_t M, int64_t N, int64_t K, const int8_t* codes,
               const uint16_t* scales, int xkind, const void* X,
               const float* xs, double* Y, double* absY);

/* The same product without multiplications by codes: per group, the sum of
 * x over code +1 minus the sum over code -1, times the scale. */
int orc_matmul_addflip(int64_t M, int64_t N, int64_t K, const int8_t* codes,
                       const uint16_t* scales, int xkind, const void* X,
                       const float* xs, double* Y);

/* Exact per-group integer sums A[m][n][g] = sum_{k in g} code * q. */
int orc_group_int_sums(int64_t M, int64_t N, int64_t K, const int8_t* codes,
                       const int8_t* Q, int64_t* A);

/* Binary weights x sign activations by XOR + popcount: per group
 * d = 128 - 2 * popcount(wbits ^ xbits); Y = alpha * sum_g scale * d and
 * D[m][n] = sum_g d (either output may be NULL). */
int orc_xor_popcount(int64_t M, int64_t N, int64_t K, const int8_t* codes,
                     const uint16_t* scales, const uint8_t* xbits,
                     const float* alpha, double* Y, int64_t* D);

/* Per-row absmax int8 quantization in fp32, ties to even. */
int orc_quantize_act_i8(int64_t M, int64_t K, const uint16_t* X_bf16,
                        int8_t* Q, float* s_x);

/* fp64 -> binary16 bits, round to nearest even. */
uint16_t orc_f64_to_f16(double x);

/* Data-free weight quantizer: signed Hadamard rotation per 128-group (signs
 * may be NULL: no rotation), absmean fp16 scale, rounding to the format's
 * codes.  codes int8 [N][K], scales fp16 bits [N][K/128]. */
int orc_quantize_weights(int fmt, int64_t N, int64_t K, const uint16_t* W_bf16,
                         const int8_t* signs, int8_t* codes, uint16_t* scales);

/* The quantizer's rotation step: T [N][K] = per-group signed Hadamard
 * rotation (orthonormal) of W, fp64. */
int orc_rotate_rows(int64_t N, int64_t K, const uint16_t* W_bf16, const int8_t* signs,
                    double* T);

/* z[k] = silu(g[k]) * u[k], silu(v) = v / (1 + exp(-v)), fp64. */
int orc_silu_mul(int64_t K, const double* g, const double* u, double* z);

#ifdef __cplusplus
}
#endif

#endif
