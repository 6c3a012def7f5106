/*
 * oracle.c -- fp64 CPU reference for the group-scaled binary / ternary
 * matrix product.  TEST INFRASTRUCTURE: only the tests, the smoke check and
 * the benchmark's CPU-baseline leg load this file's library.  It shares no
 * code, header, table or constant generator with the HIP library.
 *
 * Sources for what is computed:
 *  [R1] richmindsetzone.com, "瀏覽器生圖技術內幕：1-bit diffusion 點樣將 3GB
 *       模型塞入 WebGPU？", section "1-bit 嘅數學：點解唔爆鑊？": every weight
 *       is a sign, a group of weights shares one FP16 scale, ternary adds a
 *       zero state; effective widths 1.125 and 1.71 bits; a binary GEMM can
 *       be computed with XOR + popcount.
 *  [R3] kongchang.com, "三值权重压缩：27B模型缩至6GB，可在浏览器本地运行", section
 *       "精度保留了多少": ternary values need about log2(3) bits and a
 *       product with -1/0/+1 reduces to additions and sign flips.
 *  [R4] ainewscove.com, "我开源了 OpenBonsai：把你自己的 BF16 模型与微调压缩
 *       成约 2 GB 的三值 GGUF", method list of the paragraph "工作原理": one FP16
 *       scale per 128 weights; a signed Hadamard rotation to reduce weight
 *       outliers before the weights are quantized.
 *  The byte layout is the one written in the layout specification of the
 *  library header (it is not on the pages); this file re-implements it from
 *  that text.
 *
 * Everything is plain loops in fp64 (int64 for integer sums); no blocking,
 * no reordering beyond the definitions.
 */
#include "oracle.h"

#include <math.h>
#include <string.h>

#define GROUP 128

/* ---------------------------------------------------------------- decoders */

/* IEEE binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double orc_f16_to_f64(uint16_t h) {
  int sign = (h >> 15) & 1;
  int e = (h >> 10) & 0x1f;
  int f = h & 0x3ff;
  double v;
  if (e == 0)
    v = ldexp((double)f, -24); /* subnormal: f * 2^-10 * 2^-14 */
  else if (e == 31)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1.0 + f / 1024.0, e - 15);
  return sign ? -v : v;
}

/* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits. */
double orc_bf16_to_f64(uint16_t b) {
  int sign = (b >> 15) & 1;
  int e = (b >> 7) & 0xff;
  int f = b & 0x7f;
  double v;
  if (e == 0)
    v = ldexp((double)f, -133); /* f * 2^-7 * 2^-126 */
  else if (e == 255)
    v = f ? NAN : INFINITY;
  else
    v = ldexp(1.0 + f / 128.0, e - 127);
  return sign ? -v : v;
}

/* ------------------------------------------------------------------ layout */

static int valid_fmt(int fmt) {
  return fmt == ORC_BINARY || fmt == ORC_TERNARY_2BIT || fmt == ORC_TERNARY_BASE3;
}

static int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

/* k offset inside a group of slot i of quarter q (layout specification) */
static int kmap(int q, int i) {
  return 64 * (q & 1) + 16 * (q >> 1) + 32 * (i >> 4) + (i & 15);
}

/* binary: slot held by bit b of a quarter's word */
static int binary_slot_of_bit(int b) { return 8 * (3 - (b & 3)) + (b >> 2); }

int orc_packed_bytes(int fmt, int64_t N, int64_t K, size_t* code_bytes,
                     size_t* scale_bytes) {
  if (!valid_fmt(fmt)) return -1;
  if (N < 1 || K < 1 || K % GROUP != 0) return -2;
  int64_t NB = cdiv(N, 16), G = K / GROUP;
  int64_t c;
  if (fmt == ORC_BINARY)
    c = NB * cdiv(G, 4) * 1024;
  else if (fmt == ORC_TERNARY_2BIT)
    c = NB * cdiv(G, 2) * 1024;
  else
    c = NB * cdiv(G, 8) * 3328;
  if (code_bytes) *code_bytes = (size_t)c;
  if (scale_bytes) *scale_bytes = (size_t)(NB * cdiv(G, 4) * 128);
  return 0;
}

/* code of the dense matrix at (n, k), 0 outside N x K (padding) */
static int dense_code(const int8_t* codes, int64_t N, int64_t K, int64_t n,
                      int64_t k) {
  if (n >= N || k >= K) return 0;
  return codes[n * K + k];
}

/* byte address of base-3 byte b (0..51) of lane L in octet block (rb, o) */
static int64_t base3_byte_addr(int64_t rb, int64_t GO, int64_t o, int L, int b) {
  int64_t blk = (rb * GO + o) * 3328;
  if (b < 48) return blk + 1024 * (b / 16) + 16 * L + (b % 16);
  return blk + 3072 + 4 * L + (b - 48);
}

/* byte index and digit of slot i of group j (0..7) inside a lane's 52 bytes */
static void base3_pos(int j, int i, int* byte, int* digit) {
  if (i < 30) {
    *byte = 6 * j + i / 5;
    *digit = i % 5;
  } else {
    *byte = 48 + j / 2;
    *digit = 2 * (j % 2) + (i - 30);
  }
}

int64_t orc_pack(int fmt, int64_t N, int64_t K, const int8_t* codes,
                 const uint16_t* scales, uint8_t* pcodes, uint16_t* pscales) {
  size_t cb, sb;
  int rc = orc_packed_bytes(fmt, N, K, &cb, &sb);
  if (rc) return rc;
  int64_t NB = cdiv(N, 16), G = K / GROUP;
  int64_t GQ = cdiv(G, 4), GP = cdiv(G, 2), GO = cdiv(G, 8);
  int64_t bad = 0;
  memset(pcodes, 0, cb);
  memset(pscales, 0, sb);

  /* validate the dense codes [R1]: binary is +-1, ternary is -1/0/+1 */
  for (int64_t n = 0; n < N; n++)
    for (int64_t k = 0; k < K; k++) {
      int c = codes[n * K + k];
      int ok = (fmt == ORC_BINARY) ? (c == 1 || c == -1) : (c >= -1 && c <= 1);
      if (!ok) bad++;
    }

  for (int64_t rb = 0; rb < NB; rb++)
    for (int r = 0; r < 16; r++) {
      int64_t n = rb * 16 + r;
      /* scales: 4 groups per row per block of 128 bytes */
      for (int64_t g = 0; g < G; g++)
        if (n < N) pscales[((rb * GQ + g / 4) * 16 + r) * 4 + (g % 4)] = scales[n * G + g];
      for (int q = 0; q < 4; q++) {
        int L = r + 16 * q;
        if (fmt == ORC_BINARY) {
          for (int64_t g = 0; g < GQ * 4; g++) {
            uint32_t w = 0;
            for (int b = 0; b < 32; b++) {
              int64_t k = g * GROUP + kmap(q, binary_slot_of_bit(b));
              int c = (g < G) ? dense_code(codes, N, K, n, k) : 0;
              if (c == -1) w |= 1u << b; /* bit 1 = -1, bit 0 = +1 */
            }
            int64_t wi = ((rb * GQ + g / 4) * 64 + L) * 4 + (g % 4);
            memcpy(pcodes + 4 * wi, &w, 4);
          }
        } else if (fmt == ORC_TERNARY_2BIT) {
          for (int64_t g = 0; g < GP * 2; g++) {
            uint32_t P[2] = {0, 0};
            for (int i = 0; i < 32; i++) {
              int j = i / 8, p = i % 8;
              int64_t k = g * GROUP + kmap(q, i);
              int c = (g < G) ? dense_code(codes, N, K, n, k) : 0;
              if (c < -1 || c > 1) c = 0;
              int z = c != 0, s = c < 0;
              int zb = 4 * p + 1 - (j & 1), sbit = 4 * p + 3 - (j & 1);
              P[j / 2] |= ((uint32_t)z << zb) | ((uint32_t)s << sbit);
            }
            for (int t = 0; t < 2; t++) {
              int64_t wi = ((rb * GP + g / 2) * 64 + L) * 4 + 2 * (g % 2) + t;
              memcpy(pcodes + 4 * wi, &P[t], 4);
            }
          }
        } else {
          for (int64_t o = 0; o < GO; o++) {
            int B[52];
            for (int b = 0; b < 52; b++) B[b] = 0;
            for (int j = 0; j < 8; j++) {
              int64_t g = 8 * o + j;
              for (int i = 0; i < 32; i++) {
                int64_t k = g * GROUP + kmap(q, i);
                int c = (g < G) ? dense_code(codes, N, K, n, k) : 0;
                if (c < -1 || c > 1) c = 0;
                int byte, digit;
                base3_pos(j, i, &byte, &digit);
                int p3 = 1;
                for (int d = 0; d < digit; d++) p3 *= 3;
                B[byte] += (c + 1) * p3; /* trit t = code + 1 */
              }
            }
            for (int b = 0; b < 52; b++)
              pcodes[base3_byte_addr(rb, GO, o, L, b)] = (uint8_t)B[b];
          }
        }
      }
    }
  return bad;
}

int64_t orc_unpack(int fmt, int64_t N, int64_t K, const uint8_t* pcodes,
                   const uint16_t* pscales, int8_t* codes, uint16_t* scales) {
  int rc = orc_packed_bytes(fmt, N, K, NULL, NULL);
  if (rc) return rc;
  int64_t G = K / GROUP;
  int64_t GQ = cdiv(G, 4), GP = cdiv(G, 2), GO = cdiv(G, 8);
  int64_t bad = 0;
  for (int64_t n = 0; n < N; n++) {
    int64_t rb = n / 16;
    int r = (int)(n % 16);
    for (int64_t g = 0; g < G; g++)
      scales[n * G + g] = pscales[((rb * GQ + g / 4) * 16 + r) * 4 + (g % 4)];
    for (int64_t g = 0; g < G; g++)
      for (int q = 0; q < 4; q++) {
        int L = r + 16 * q;
        if (fmt == ORC_BINARY) {
          uint32_t w;
          memcpy(&w, pcodes + 4 * (((rb * GQ + g / 4) * 64 + L) * 4 + (g % 4)), 4);
          for (int b = 0; b < 32; b++) {
            int64_t k = g * GROUP + kmap(q, binary_slot_of_bit(b));
            codes[n * K + k] = ((w >> b) & 1) ? -1 : 1;
          }
        } else if (fmt == ORC_TERNARY_2BIT) {
          uint32_t P[2];
          for (int t = 0; t < 2; t++)
            memcpy(&P[t], pcodes + 4 * (((rb * GP + g / 2) * 64 + L) * 4 + 2 * (g % 2) + t), 4);
          for (int i = 0; i < 32; i++) {
            int j = i / 8, p = i % 8;
            int z = (P[j / 2] >> (4 * p + 1 - (j & 1))) & 1;
            int s = (P[j / 2] >> (4 * p + 3 - (j & 1))) & 1;
            int64_t k = g * GROUP + kmap(q, i);
            if (!z && s) {
              bad++; /* reserved pattern */
              codes[n * K + k] = 0;
            } else {
              codes[n * K + k] = (int8_t)(z ? (s ? -1 : 1) : 0);
            }
          }
        } else {
          int64_t o = g / 8;
          int j = (int)(g % 8);
          for (int i = 0; i < 32; i++) {
            int byte, digit;
            base3_pos(j, i, &byte, &digit);
            int v = pcodes[base3_byte_addr(rb, GO, o, L, byte)];
            int limit = byte < 48 ? 243 : 81;
            int64_t k = g * GROUP + kmap(q, i);
            if (v >= limit) {
              bad++;
              codes[n * K + k] = 0;
              continue;
            }
            for (int d = 0; d < digit; d++) v /= 3;
            codes[n * K + k] = (int8_t)(v % 3 - 1);
          }
        }
      }
  }
  return bad;
}

/* ---------------------------------------------------------------- products */

/* activation x(m, k) as a real number */
static double x_value(int xkind, const void* X, const float* xs, int64_t K,
                      int64_t m, int64_t k) {
  double sc = xs ? (double)xs[m] : 1.0;
  switch (xkind) {
    case ORC_X_F32:
      return (double)((const float*)X)[m * K + k];
    case ORC_X_BF16:
      return orc_bf16_to_f64(((const uint16_t*)X)[m * K + k]);
    case ORC_X_I8:
      return sc * (double)((const int8_t*)X)[m * K + k];
    case ORC_X_SIGN1: {
      const uint8_t* bits = (const uint8_t*)X + m * (K / 8);
      int b = (bits[k / 8] >> (k % 8)) & 1;
      return b ? -sc : sc;
    }
  }
  return NAN;
}

static int valid_x(int xkind) { return xkind >= ORC_X_F32 && xkind <= ORC_X_SIGN1; }

/* Dequantize-then-multiply [R1]: W[n][k] = scale[n][k/128] * code[n][k]
 * (group of 128 from [R4]); Y = X W^T, all in fp64. */
int orc_matmul(int64_t M, int64_t N, int64_t K, const int8_t* codes,
               const uint16_t* scales, int xkind, const void* X,
               const float* xs, double* Y, double* absY) {
  if (M < 1 || N < 1 || K < 1 || K % GROUP || !valid_x(xkind)) return -2;
  int64_t G = K / GROUP;
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      double acc = 0.0, aacc = 0.0;
      for (int64_t k = 0; k < K; k++) {
        double s = scales ? orc_f16_to_f64(scales[n * G + k / GROUP]) : 1.0;
        double w = s * (double)codes[n * K + k];
        double t = w * x_value(xkind, X, xs, K, m, k);
        acc += t;
        aacc += fabs(t);
      }
      Y[m * N + n] = acc;
      if (absY) absY[m * N + n] = aacc;
    }
  return 0;
}

/* Multiply-free form [R3]: within a group, add x where the code is +1,
 * subtract it where the code is -1, skip it where the code is 0; then apply
 * the group's scale once. */
int orc_matmul_addflip(int64_t M, int64_t N, int64_t K, const int8_t* codes,
                       const uint16_t* scales, int xkind, const void* X,
                       const float* xs, double* Y) {
  if (M < 1 || N < 1 || K < 1 || K % GROUP || !valid_x(xkind)) return -2;
  int64_t G = K / GROUP;
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      double acc = 0.0;
      for (int64_t g = 0; g < G; g++) {
        double plus = 0.0, minus = 0.0;
        for (int64_t k = g * GROUP; k < (g + 1) * GROUP; k++) {
          int c = codes[n * K + k];
          if (c == 1) plus += x_value(xkind, X, xs, K, m, k);
          else if (c == -1) minus += x_value(xkind, X, xs, K, m, k);
        }
        double s = scales ? orc_f16_to_f64(scales[n * G + g]) : 1.0;
        acc += s * (plus - minus);
      }
      Y[m * N + n] = acc;
    }
  return 0;
}

int orc_group_int_sums(int64_t M, int64_t N, int64_t K, const int8_t* codes,
                       const int8_t* Q, int64_t* A) {
  if (M < 1 || N < 1 || K < 1 || K % GROUP) return -2;
  int64_t G = K / GROUP;
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++)
      for (int64_t g = 0; g < G; g++) {
        int64_t a = 0;
        for (int64_t k = g * GROUP; k < (g + 1) * GROUP; k++)
          a += (int64_t)codes[n * K + k] * (int64_t)Q[m * K + k];
        A[(m * N + n) * G + g] = a;
      }
  return 0;
}

static int popcount64(uint64_t v) {
  int c = 0;
  while (v) {
    v &= v - 1;
    c++;
  }
  return c;
}

/* XOR + popcount [R1]: for +-1 vectors a, b encoded as bits (1 = -1), the
 * dot product over L positions is L - 2 * popcount(a xor b). */
int orc_xor_popcount(int64_t M, int64_t N, int64_t K, const int8_t* codes,
                     const uint16_t* scales, const uint8_t* xbits,
                     const float* alpha, double* Y, int64_t* D) {
  if (M < 1 || N < 1 || K < 1 || K % GROUP) return -2;
  int64_t G = K / GROUP;
  for (int64_t m = 0; m < M; m++)
    for (int64_t n = 0; n < N; n++) {
      double acc = 0.0;
      int64_t dsum = 0;
      for (int64_t g = 0; g < G; g++) {
        uint64_t w[2] = {0, 0}, x[2] = {0, 0};
        for (int j = 0; j < GROUP; j++) {
          int64_t k = g * GROUP + j;
          if (codes[n * K + k] == -1) w[j / 64] |= 1ull << (j % 64);
          if ((xbits[m * (K / 8) + k / 8] >> (k % 8)) & 1) x[j / 64] |= 1ull << (j % 64);
        }
        int d = GROUP - 2 * (popcount64(w[0] ^ x[0]) + popcount64(w[1] ^ x[1]));
        double s = scales ? orc_f16_to_f64(scales[n * G + g]) : 1.0;
        acc += s * d;
        dsum += d;
      }
      if (Y) Y[m * N + n] = (alpha ? (double)alpha[m] : 1.0) * acc;
      if (D) D[m * N + n] = dsum;
    }
  return 0;
}

/* Per-row absmax int8 quantization in fp32 (the pages are silent on
 * activations; this is the reading written in the library header). */
int orc_quantize_act_i8(int64_t M, int64_t K, const uint16_t* X_bf16,
                        int8_t* Q, float* s_x) {
  if (M < 1 || K < 1) return -2;
  for (int64_t m = 0; m < M; m++) {
    float a = 0.0f;
    for (int64_t k = 0; k < K; k++) {
      float v = (float)orc_bf16_to_f64(X_bf16[m * K + k]);
      if (fabsf(v) > a) a = fabsf(v);
    }
    if (a == 0.0f) {
      for (int64_t k = 0; k < K; k++) Q[m * K + k] = 0;
      s_x[m] = 0.0f;
      continue;
    }
    volatile float inv = 127.0f / a;
    for (int64_t k = 0; k < K; k++) {
      volatile float v = (float)orc_bf16_to_f64(X_bf16[m * K + k]);
      volatile float p = v * inv;
      float r = rintf(p); /* default rounding mode: nearest, ties to even */
      if (r > 127.0f) r = 127.0f;
      if (r < -127.0f) r = -127.0f;
      Q[m * K + k] = (int8_t)r;
    }
    volatile float sx = a / 127.0f;
    s_x[m] = sx;
  }
  return 0;
}

/* ------------------------------------------------------- weight quantizer */

/* fp64 -> IEEE binary16 bits, round to nearest even (subnormals kept,
 * overflow to infinity). */
uint16_t orc_f64_to_f16(double x) {
  uint16_t sign = signbit(x) ? 0x8000 : 0;
  double a = fabs(x);
  if (isnan(x)) return 0x7E00;
  if (a >= 65520.0) return sign | 0x7C00; /* rounds past the largest finite */
  if (a < ldexp(1.0, -14)) {
    /* subnormal (or zero): a multiple of 2^-24 */
    double q = a * ldexp(1.0, 24); /* exact: a < 2^-14 */
    double r = nearbyint(q);       /* ties to even */
    return sign | (uint16_t)r;     /* r = 1024 becomes the smallest normal */
  }
  int e;
  double f = frexp(a, &e); /* a = f 2^e, f in [0.5, 1) */
  /* significand with 10 fraction bits: a = m 2^(e - 11), m in [1024, 2048) */
  double m = nearbyint(ldexp(f, 11));
  if (m == 2048.0) {
    m = 1024.0;
    e += 1;
  }
  int biased = e - 1 + 15;
  if (biased >= 31) return sign | 0x7C00;
  return sign | (uint16_t)(biased << 10) | (uint16_t)((int)m - 1024);
}

/* Data-free quantizer front end [R4] (the rotation and the per-128 FP16
 * scale of its method list; the calibrated GPTQ step needs data and is not
 * part of it).  Per row n and group g of 128 weights:
 *   v_i = W[n][128 g + i] * d[128 g + i]           (signs d in {-1, +1})
 *   u_i = sum_j H[i][j] v_j,  H[i][j] = (-1)^popcount(i & j)   (index order)
 *   t_i = u_i * r, r = 1/sqrt(128) as an fp64 number (orthonormal rotation)
 *   s   = (sum_i |u_i| / 128) * r                  (mean |t|)
 *   s16 = fp16(s) (round to nearest even); scales[n][g] = s16
 *   ternary: c_i = +1 if t_i > s16 / 2, -1 if t_i < -s16 / 2, else 0
 *            (t / s16 rounded to the nearest integer, ties to even, clamped
 *            to [-1, 1], decided by exact comparison)
 *   binary:  c_i = -1 if t_i < 0, else +1
 *   s16 == 0: every c_i = 0 (ternary) or +1 (binary).
 * signs == NULL: no rotation (u = t = v, s = sum |v| / 128), the plain
 * absmean rounding.  All in fp64. */
int orc_quantize_weights(int fmt, int64_t N, int64_t K, const uint16_t* W_bf16,
                         const int8_t* signs, int8_t* codes, uint16_t* scales) {
  if ((fmt != 1 && fmt != 2 && fmt != 3) || N < 1 || K < 1 || K % GROUP) return -2;
  const int64_t G = K / GROUP;
  const double r = 1.0 / sqrt(128.0);
  double v[GROUP], t[GROUP];
  for (int64_t n = 0; n < N; n++)
    for (int64_t g = 0; g < G; g++) {
      for (int i = 0; i < GROUP; i++) {
        double w = orc_bf16_to_f64(W_bf16[n * K + g * GROUP + i]);
        v[i] = signs ? w * (double)signs[g * GROUP + i] : w;
      }
      double S = 0.0;
      for (int i = 0; i < GROUP; i++) {
        double u = v[i];
        if (signs) {
          u = 0.0;
          for (int j = 0; j < GROUP; j++) {
            int par = __builtin_popcount((unsigned)(i & j)) & 1;
            u += par ? -v[j] : v[j];
          }
        }
        S += fabs(u);
        t[i] = signs ? u * r : u;
      }
      double sc = signs ? (S / 128.0) * r : S / 128.0;
      uint16_t s16 = orc_f64_to_f16(sc);
      double sd = orc_f16_to_f64(s16);
      scales[n * G + g] = s16;
      for (int i = 0; i < GROUP; i++) {
        int c;
        if (fmt == 1) {
          c = (sd == 0.0 || !(t[i] < 0.0)) ? 1 : -1;
        } else if (sd == 0.0) {
          c = 0;
        } else {
          double h = sd * 0.5; /* exact */
          c = t[i] > h ? 1 : (t[i] < -h ? -1 : 0);
        }
        codes[n * K + g * GROUP + i] = (int8_t)c;
      }
    }
  return 0;
}

/* The rotation step alone: T[n][k] = t of the quantizer above (fp64). */
int orc_rotate_rows(int64_t N, int64_t K, const uint16_t* W_bf16, const int8_t* signs,
                    double* T) {
  if (N < 1 || K < 1 || K % GROUP || !signs) return -2;
  const int64_t G = K / GROUP;
  const double r = 1.0 / sqrt(128.0);
  double v[GROUP];
  for (int64_t n = 0; n < N; n++)
    for (int64_t g = 0; g < G; g++) {
      for (int i = 0; i < GROUP; i++)
        v[i] = orc_bf16_to_f64(W_bf16[n * K + g * GROUP + i]) * (double)signs[g * GROUP + i];
      for (int i = 0; i < GROUP; i++) {
        double u = 0.0;
        for (int j = 0; j < GROUP; j++) {
          int par = __builtin_popcount((unsigned)(i & j)) & 1;
          u += par ? -v[j] : v[j];
        }
        T[n * K + g * GROUP + i] = u * r;
      }
    }
  return 0;
}

/* Gated FFN activation feeding the down projection: z[k] = silu(g[k]) u[k],
 * silu(v) = v / (1 + e^-v), in fp64.  The pages state that the compressed
 * models keep their base model's architecture and change only how weights
 * are stored ([R3] section "三值权重（Ternary）到底做了什么"; page
 * "PrismMLが27BモデルをiPhoneに押し込んだ。しかも頭の良さはほぼ落ちていない",
 * section "土台は依然Qwen3.6-27B。Bonsaiが網全体を極限ビットに押し込む"); the gated
 * SiLU FFN is that base family's, which the pages do not print. */
int orc_silu_mul(int64_t K, const double* g, const double* u, double* z) {
  if (K < 0 || (K && (!g || !u || !z))) return -2;
  for (int64_t k = 0; k < K; k++) z[k] = g[k] / (1.0 + exp(-g[k])) * u[k];
  return 0;
}
