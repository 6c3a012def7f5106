/*
 * lowbit.h -- C ABI of liblowbit: matrix products over group-scaled binary
 * {-1,+1} and ternary {-1,0,+1} weights on AMD Instinct MI355X (gfx950).
 *
 * Pages cited, by title (a citation names the page's tag and a section of it
 * in the page's own words):
 *   [RM] richmindsetzone.com: "瀏覽器生圖技術內幕：1-bit diffusion 點樣將 3GB
 *        模型塞入 WebGPU？"
 *   [KC] kongchang.com: "三值权重压缩：27B模型缩至6GB，可在浏览器本地运行"
 *   [OB] ainewscove.com: "我开源了 OpenBonsai：把你自己的 BF16 模型与微调压缩成约
 *        2 GB 的三值 GGUF"
 *   [XH] best.xiaohu.ai: "PrismMLが27BモデルをiPhoneに押し込んだ。しかも頭の良さは
 *        ほぼ落ちていない"
 *
 * What is computed:
 *   - Each weight is a sign (binary) or one of {-1,0,+1} (ternary), and every
 *     group of weights shares one FP16 scale ([RM] section "1-bit 嘅數學：
 *     點解唔爆鑊？"; effective widths 1.125 bits binary, 1.71 ternary).
 *   - The group holds 128 weights, one FP16 scale each ([OB], the method list
 *     of the paragraph "工作原理").
 *   - Multiplying by -1/0/+1 is an add or a sign flip ([KC] section
 *     "精度保留了多少"); a binary product can be done with XOR + popcount
 *     ([RM] section "1-bit 嘅數學：點解唔爆鑊？", the paragraph comparing
 *     binary and ternary).
 *   - Batch-1 decode streams every weight once per token and is bound by
 *     memory bandwidth; prefill is a dense contraction ([XH] sections
 *     "ローカル27Bを阻む第一の壁：「1語生成するたびに全身を運び直す」" and
 *     "速度は二層：低ビット搬送と、CUDA上の草稿加速").
 *
 * Dense (unpacked) meaning of the operands, shared by every entry point:
 *   W       [N][K] weights, row n = output feature, k = reduction index.
 *   codes   int8 [N][K] row-major: binary in {-1,+1}, ternary in {-1,0,+1}.
 *   scales  IEEE binary16 bits, uint16 [N][G], G = K/128; group g of row n
 *           covers k in [128g, 128g+128).  W[n][k] = scale[n][k/128]*code[n][k].
 *           There is no zero point.  Scales must be finite (any sign, 0 ok).
 *   X       [M][K] activations, row-major.  Y = X * W^T, Y is [M][N].
 *   K must be a positive multiple of 128; N, M >= 1.
 *
 * Every pointer is caller-owned device memory unless stated.  Every call is
 * asynchronous on `stream` (a hipStream_t passed as void*, NULL = the null
 * stream) on the current device.  Argument errors are returned synchronously
 * before any HIP call.  A launch failure returns LOWBIT_E_HIP.  No entry
 * point waits for the GPU except lowbit_chain_status, lowbit_chain_destroy
 * and lowbit_release_workspaces, which say so.
 *
 * Streams, workspaces and graphs.  lowbit_gemv and lowbit_gemm use a device
 * workspace that the library owns, one per (device, stream).  Calls on one
 * stream are ordered and share it; calls on different streams never share
 * one.  A call that needs more than its stream's workspace holds allocates a
 * larger one (hipMalloc, which may synchronize the device as HIP does) and
 * keeps the smaller one allocated until lowbit_release_workspaces, because
 * kernels already queued, and graphs captured earlier, may still use it; no
 * call waits on the stream.  A stream that is being captured into a HIP graph
 * cannot grow its workspace: such a call returns LOWBIT_E_NOMEM, so reserve
 * the workspace first (lowbit_workspace_bytes + lowbit_reserve_workspace, or
 * one eager call of the largest captured product on that stream).  A captured
 * graph keeps the workspace address it was captured with; replaying it is
 * valid until lowbit_release_workspaces.  Replays of graphs captured on one
 * stream must run in order on one stream (they share its workspace).  The
 * kernels leave the workspace's counters as they found them, so a replay
 * needs no reset.  No call records a memset into a capture.
 *
 * =====================  PACKED LAYOUT (gfx950)  ===========================
 * Rows are tiled in row-blocks of 16 (NB = ceil(N/16), rows >= N are padding
 * with code 0 / +1 and scale 0).  Inside a row-block, row r = n % 16 and the
 * 128 weights of a group are split over four quarters q = 0..3; the pair
 * (r, q) is the lane L = r + 16q of a 64-wide wavefront.  Quarter q of a
 * group holds 32 weights in slots i = 0..31; slot i of quarter q is the
 * weight at k = 128g + KMAP(q, i) with
 *     KMAP(q, i) = 64*(q & 1) + 16*(q >> 1) + 32*(i >> 4) + (i & 15).
 * (This is the order in which the fp4 B operand of the gfx950
 * 16x16x128 f8f6f4 MFMA consumes k, so one lane's 32 weights are one MFMA
 * fragment.)
 *
 * LOWBIT_BINARY (1 bit / weight).  One 32-bit word per (row, group, quarter);
 *   bit b of the word holds slot  i = 8*(3 - (b & 3)) + (b >> 2),  bit value
 *   1 means -1 and 0 means +1.  Words are stored as
 *     word[((rb * GQ + g/4) * 64 + L) * 4 + (g % 4)],   GQ = ceil(G/4),
 *   so a wavefront reading one 16-byte vector per lane reads 1 KiB contiguous
 *   (16 rows x 4 groups).  Code bytes: NB * GQ * 1024.
 *
 * LOWBIT_TERNARY_2BIT (2 bits / weight, bit-sliced).  Two words P0, P1 per
 *   (row, group, quarter).  Each weight has a "nonzero" bit z and a "negative"
 *   bit s (code = z * (1 - 2s); z = 0 with s = 1 is reserved and never
 *   written).  For slot i = 8j + p (j = 0..3, p = 0..7):
 *     j = 0: P0 bit 4p+1 = z, P0 bit 4p+3 = s      j = 1: P0 bit 4p = z, P0 bit 4p+2 = s
 *     j = 2: P1 bit 4p+1 = z, P1 bit 4p+3 = s      j = 3: P1 bit 4p = z, P1 bit 4p+2 = s
 *   Words are stored as
 *     word[((rb * GP + g/2) * 64 + L) * 4 + 2*(g % 2) + t],  t = 0 (P0), 1 (P1),
 *   GP = ceil(G/2).  Code bytes: NB * GP * 1024.
 *
 * LOWBIT_TERNARY_BASE3 (5 trits / byte, 1.625 bits / weight).  Trit
 *   t = code + 1 in {0,1,2}; a byte holding trits t_0..t_{d-1} has value
 *   sum t_e * 3^e (t_0 is the least-significant digit).  Groups are handled
 *   in octets o = g/8 (GO = ceil(G/8)).  Lane L of octet o owns 52 bytes
 *   B[0..51] covering the 8 groups j = 0..7 (g = 8o + j) of its quarter:
 *     slots 0..29 of group j -> bytes 6j .. 6j+5, slot i in byte 6j + i/5,
 *                                digit i % 5;
 *     slots 30, 31 of group j -> byte 48 + j/2, digits 2*(j%2) + (i-30).
 *   (Bytes 0..47 hold 5 trits, bytes 48..51 hold 4.)  An octet block of a
 *   row-block is 3328 bytes: for s = 0..2 the 1024 bytes at 1024s hold
 *   B[16s .. 16s+15] of lane L at offset 1024s + 16L, and the 256 bytes at
 *   3072 hold B[48..51] of lane L at 3072 + 4L.  Block (rb, o) starts at
 *   byte (rb * GO + o) * 3328.  Code bytes: NB * GO * 3328.  Byte values
 *   >= 243 (>= 81 in bytes 48..51) are invalid.
 *
 * Scales, all formats: fp16 bits stored as
 *     scale[((rb * GQ + g/4) * 16 + r) * 4 + (g % 4)],
 *   i.e. 128 bytes per (row-block, 4 groups).  Scale bytes: NB * GQ * 128.
 *   Padding groups (g >= G) and padding rows hold code 0 (+1 binary) and
 *   scale 0.
 *
 * Bits per weight when N % 16 == 0 and G % 8 == 0: binary 1 + 0.125 = 1.125,
 * ternary 2-bit 2.125, ternary base-3 1.625 + 0.125 = 1.75 (all at or above
 * the information bound log2(3) + 0.125 = 1.70996 for ternary).
 * ========================================================================= */
#ifndef LOWBIT_H
#define LOWBIT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LOWBIT_ABI_VERSION 3

enum lowbit_status {
  LOWBIT_OK = 0,
  LOWBIT_E_NULL = -1,        /* a required pointer is NULL                    */
  LOWBIT_E_SHAPE = -2,       /* K % 128 != 0, N/M/K < 1, or size overflow     */
  LOWBIT_E_ALIGN = -3,       /* pointer not aligned as documented             */
  LOWBIT_E_UNSUPPORTED = -4, /* format / dtype combination not provided       */
  LOWBIT_E_BADCODE = -5,     /* reserved for callers that check the flag     */
  LOWBIT_E_HIP = -6,         /* a HIP runtime call or launch failed           */
  LOWBIT_E_NOMEM = -7,       /* the library could not allocate its workspace  */
  LOWBIT_E_TOO_LARGE = -8    /* lowbit_gemv_noalloc: the product needs more
                                scratch than the library's static array       */
};

enum lowbit_format {
  LOWBIT_BINARY = 1,
  LOWBIT_TERNARY_2BIT = 2,
  LOWBIT_TERNARY_BASE3 = 3
};

enum lowbit_dtype {
  LOWBIT_F32 = 1,   /* IEEE binary32                                          */
  LOWBIT_BF16 = 2,  /* bfloat16 bits (uint16)                                 */
  LOWBIT_I8 = 3,    /* int8 with a float scale: value = scale * q             */
  LOWBIT_SIGN1 = 4, /* packed sign bits, K/8 bytes per row, bit k%8 of byte
                       k/8 (LSB first); bit 1 means -alpha, 0 means +alpha     */
  LOWBIT_I32 = 5    /* int32 output of the exact integer paths               */
};

/* ABI version of the loaded library (LOWBIT_ABI_VERSION).  Library
 * bookkeeping; no passage of the pages. */
int lowbit_abi_version(void);

/* Static text for a status code; never NULL.  Library bookkeeping. */
const char* lowbit_status_str(int status);

/* Bytes of the packed code and scale buffers for an N x K matrix in `fmt`
 * (layout above; storage of [RM] section "1-bit 嘅數學：點解唔爆鑊？" and
 * the ternary width of [KC] section "精度保留了多少").  Host-only, no HIP
 * call.  Errors: E_NULL, E_SHAPE, E_UNSUPPORTED. */
int lowbit_packed_bytes(int fmt, int64_t N, int64_t K, size_t* code_bytes,
                        size_t* scale_bytes);

/* Pack dense codes [N][K] (int8) and scales [N][G] (fp16 bits) into the
 * layout above, writing every byte of pcodes/pscales (padding included).
 * Group-scaled weights of [RM] section "1-bit 嘅數學：點解唔爆鑊？" with the
 * group of 128 of [OB] paragraph "工作原理".
 * pcodes and pscales must be 16-byte aligned.  Codes outside the format's
 * value set are counted into *bad_code_count (device int32, atomically
 * added; pass NULL to skip); their packed value is unspecified.  The count is
 * not cleared by the call. */
int lowbit_pack(int fmt, int64_t N, int64_t K, const int8_t* codes,
                const uint16_t* scales, void* pcodes, void* pscales,
                int32_t* bad_code_count, void* stream);

/* Inverse of lowbit_pack (same passages): writes codes [N][K] and scales
 * [N][G].  A weight
 * decoded from a reserved 2-bit pattern or an out-of-range base-3 byte is
 * written as 0 and counted (one per weight) into *bad_code_count (device
 * int32, atomically added, nullable). */
int lowbit_unpack(int fmt, int64_t N, int64_t K, const void* pcodes,
                  const void* pscales, int8_t* codes, uint16_t* scales,
                  int32_t* bad_code_count, void* stream);

/* Per-row absmax int8 quantization of bf16 X [M][K] (the pages fix no
 * activation format; an 8-bit activation is the plainest reading of the
 * integer product of [KC] section "精度保留了多少".  fp32 arithmetic, no
 * fused operations): a = max_k |x|; if a == 0 then q = 0 and s_x = 0, else
 * inv = 127.0f / a, q = clamp(rint(x * inv), -127, 127) with ties to even,
 * s_x = a / 127.0f.  Writes Q [M][K] and s_x [M]. */
int lowbit_quantize_act_i8(int64_t M, int64_t K, const uint16_t* X_bf16,
                           int8_t* Q, float* s_x, void* stream);

/* Batch-1 product y[n] = sum_k W[n][k] * x[k] for n < N: the per-token
 * product of decode ([XH] section "ローカル27Bを阻む第一の壁：「1語生成する
 * たびに全身を運び直す」") over the weights of [RM] section "1-bit 嘅數學：
 * 點解唔爆鑊？".
 *   x_dtype F32 / BF16: x holds K values.
 *   x_dtype I8: x holds K int8 q; the result is multiplied by x_scale.
 *   x_dtype SIGN1 (binary weights only, K <= 393216): x holds K/8 bytes of
 *     sign bits; the result is multiplied by x_scale (alpha).  Runs as one
 *     launch without the workspace.
 *   y_dtype F32 or BF16 (round to nearest even).  y_dtype I32 is allowed
 *   only for x_dtype I8 / SIGN1 with pscales == NULL: y = exact integer
 *   sum_k code * q (or the signed bit agreement count), x_scale ignored.
 * Alignment: pcodes, pscales, x 16 bytes; y 4 bytes.  Uses the stream's
 * workspace (see "Streams, workspaces and graphs" above; E_NOMEM if it must
 * grow during capture or cannot be allocated). */
int lowbit_gemv(int fmt, int64_t N, int64_t K, const void* pcodes,
                const void* pscales, int x_dtype, const void* x, float x_scale,
                int y_dtype, void* y, void* stream);

/* Allocation-free lowbit_gemv, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Arguments, results and errors as lowbit_gemv, which it
 * equals bit for bit (the same kernels), plus LOWBIT_E_TOO_LARGE.  Instead of
 * the per-stream workspace it uses a static device array of 4 MiB per GPU
 * (held until the process ends), enough for every product whose workspace
 * (lowbit_workspace_bytes with M = 1) is at most 4 MiB -- every N <= 65536
 * with K <= 65536, and the 27B-class layer shapes; larger products return
 * LOWBIT_E_TOO_LARGE before any launch.  It calls no hipMalloc or hipFree.
 * The first call on a device looks the array up and clears its counter
 * block with a small kernel on `stream`.  All calls on one GPU share the
 * array: calls that may overlap in time on one GPU (different streams, or
 * replays of graphs holding this call on different streams) race and give
 * wrong results; order them on one stream.  Sign activations (SIGN1) use no
 * scratch. */
int lowbit_gemv_noalloc(int fmt, int64_t N, int64_t K, const void* pcodes,
                        const void* pscales, int x_dtype, const void* x, float x_scale,
                        int y_dtype, void* y, void* stream);

/* Product Y[m][n] = sum_k W[n][k] * X[m][k] for m < M, n < N: the dense
 * contraction of prefill and of a denoising step ([XH] section "速度は二層：
 * 低ビット搬送と、CUDA上の草稿加速"; [RM] section "1-bit 嘅數學：點解唔爆鑊？").
 * M <= 16 / (activation split terms) runs the small-M GEMV path (8 rows for
 * binary bf16, 5 for ternary bf16, 8 for int8).
 *   x_dtype BF16: X bf16 [M][K], fp32 accumulation.
 *   x_dtype I8: X int8 [M][K] (e.g. from lowbit_quantize_act_i8) with
 *     x_scales[M] (device fp32); per 128-group integer sums are exact in int32
 *     and Y[m][n] = x_scales[m] * sum_g scale[n][g] * A[m][n][g].
 *     y_dtype I32 requires pscales == NULL and returns sum_g A[m][n][g].
 *   x_dtype SIGN1 (batched sign activations, any weight format): X holds
 *     K/8 bytes of sign bits per row (bit k%8 of byte k/8, 1 = negative) and
 *     x_scales[M] the per-row magnitude alpha_m (device fp32), so that
 *     x[m][k] = alpha_m (-1)^bit.  Per group D[m][n][g] = sum_k code * sign
 *     is an exact integer (for binary weights 128 - 2 popcount(w XOR x) per
 *     group, the XOR + popcount product of [RM] section "1-bit 嘅數學：點解唔爆鑊？") and Y = alpha_m sum_g scale[n][g] D[m][n][g];
 *     y_dtype I32 requires pscales == NULL and returns sum_g D (x_scales
 *     ignored).
 *   y_dtype F32 or BF16 (or I32 as above).
 * K <= 2^36 (E_SHAPE beyond).  Alignment: pcodes, pscales, X, Y 16 bytes.
 * Uses the stream's workspace as lowbit_gemv does. */
int lowbit_gemm(int fmt, int64_t M, int64_t N, int64_t K, const void* pcodes,
                const void* pscales, int x_dtype, const void* X,
                const float* x_scales, int y_dtype, void* Y, void* stream);

/* Workspace management (library bookkeeping, no passage of the pages).
 * lowbit_workspace_bytes: host-only; *bytes = the workspace a lowbit_gemm
 *   call with these arguments needs (M = 1: also bounds lowbit_gemv's).
 *   Errors: E_NULL, E_UNSUPPORTED, E_SHAPE.
 * lowbit_reserve_workspace: makes the stream's workspace on the current
 *   device hold at least `bytes` (grows it as a product call would; E_NOMEM
 *   during capture or when hipMalloc fails).  Call before capturing.
 * lowbit_release_workspaces: waits for each device that holds one, then frees
 *   every workspace, current and retired, of every stream and device.  Call
 *   it only when no queued kernel and no graph that will be replayed uses one;
 *   later calls allocate afresh.  Errors: E_HIP. */
int lowbit_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K, int x_dtype,
                           size_t* bytes);
int lowbit_reserve_workspace(size_t bytes, void* stream);
int lowbit_release_workspaces(void);

/* ---- chains of batch-1 products in one persistent launch ------------------
 * Batch-1 decode streams every weight of every layer once per token and is
 * bound by memory bandwidth, so the cost that matters is the one paid per
 * token ([XH] sections "ローカル27Bを阻む第一の壁：「1語生成するたびに全身を運び
 * 直す」" and "速度は二層：低ビット搬送と、CUDA上の草稿加速").
 * A chain runs a fixed list of batch-1 products of one weight format as one
 * cooperative launch whose workgroups stream the weights of later products
 * while earlier ones finish.  Stage i with wait_prev != 0 reads its x only
 * after every output of stage i-1 has been written (so x may be, or be
 * computed from, an earlier stage's y); its weights may be read earlier.
 * Outputs are written with device-coherent stores. */
typedef struct lowbit_gemv_stage {
  int fmt;              /* any lowbit_format, equal for all stages                */
  int64_t N, K;         /* W is N x K, K % 128 == 0                                */
  const void* pcodes;   /* packed codes (16-byte aligned)                          */
  const void* pscales;  /* packed fp16 scales (16-byte aligned)                    */
  const void* x;        /* rows x K activations of the chain's x_dtype (row-major,
                           16-byte aligned; rows = 1 unless created with rows)      */
  void* y;              /* rows x N outputs of the chain's y_dtype (4-byte aligned) */
  int wait_prev;        /* 1: read x only after stage i-1 is complete (then rows
                           times K times the x element size must stay below 2^31
                           bytes)                                                  */
  int epilogue;         /* LOWBIT_EPI_NONE or LOWBIT_EPI_SILU_MUL (see below)      */
} lowbit_gemv_stage;

/* Stage epilogues.  LOWBIT_EPI_SILU_MUL: the stage is a fused gate/up
 * product of a gated FFN (the compressed models keep their base model's
 * architecture: [KC] section "三值权重（Ternary）到底做了什么") whose N rows (N % 16 == 0) are ordered so that in every 16-row
 * block rows 0..7 are gate rows 8b..8b+7 and rows 8..15 the up rows
 * 8b..8b+7; y then receives N/2 values z[i] = silu(g[i]) u[i],
 * silu(v) = v / (1 + e^-v), computed in fp32 from the fp32 products and
 * stored in the chain's y_dtype -- the input of the down projection, which a
 * later stage (wait_prev = 1, K = N/2, x = this y when y_dtype equals
 * x_dtype) reads. */
#define LOWBIT_EPI_NONE 0
#define LOWBIT_EPI_SILU_MUL 1

typedef struct lowbit_chain lowbit_chain; /* opaque */

/* Plan a chain of n_stages products on the current device: copies the stage
 * list (pointers are used as given at every run), allocates the chain's
 * device descriptors, counters and split-K partial sums (owned by the chain
 * until lowbit_chain_destroy).  x_dtype F32 or BF16; y_dtype F32 or BF16.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_UNSUPPORTED, E_HIP, E_NOMEM. */
int lowbit_chain_create(int n_stages, const lowbit_gemv_stage* stages, int x_dtype,
                        int y_dtype, lowbit_chain** chain);

/* The same with `rows` activation rows per product (1 <= rows <= 8 for BF16 x,
 * <= 4 for F32 x; every stage takes rows x K activations and writes rows x N
 * outputs): a small-M chain such as one pass that verifies rows - 1 drafted
 * tokens and the next one through every product of a model ([XH] section
 * "速度は二層：低ビット搬送と、CUDA上の草稿加速": drafts are checked by the
 * target model in one pass).  The SiLU-mul epilogue needs rows == 1.  Errors as
 * lowbit_chain_create (E_SHAPE for rows out of range). */
int lowbit_chain_create_rows(int n_stages, const lowbit_gemv_stage* stages, int64_t rows,
                             int x_dtype, int y_dtype, lowbit_chain** chain);

/* Run every stage once, asynchronously on `stream`.  Runs of one chain must
 * not overlap (they share its counters); run it on one stream at a time. */
int lowbit_chain_run(lowbit_chain* chain, void* stream);

/* Synchronous: *failed_waits != 0 if a stage ever gave up waiting for its
 * predecessor (a bounded wait of about a second; its outputs are then not
 * meaningful).  Never expected when runs do not overlap. */
int lowbit_chain_status(lowbit_chain* chain, int* failed_waits);

/* Frees the chain's device memory (synchronizes the device first).  Library
 * bookkeeping. */
int lowbit_chain_destroy(lowbit_chain* chain);

/* Data-free quantizer front end (the signed Hadamard rotation and the
 * FP16 scale per 128 weights of the method list of [OB] paragraph
 * "工作原理"; its calibrated GPTQ step needs data and is
 * not part of it).  From bf16 weights W [N][K] writes dense codes [N][K]
 * (int8, the input of lowbit_pack) and fp16 scales [N][K/128].  Per row and
 * group of 128: v = W * d (signs d[K], int8 +-1; signs == NULL: no
 * rotation), u = H v with H[i][j] = (-1)^popcount(i & j), t = u r with
 * r = 1/sqrt(128) as an fp64 number, s16 = fp16((sum |u| / 128) r) (round to
 * nearest even); ternary formats: c = +1 if t > s16/2, -1 if t < -s16/2,
 * else 0; binary: c = -1 if t < 0 else +1; s16 = 0 gives codes 0 / +1.
 * Computed in fp64 (sums exact while a group's magnitudes span less than
 * 2^38, so the result does not depend on the summation order).  Rotated
 * weights expect rotated activations (lowbit_rotate_act with the same
 * signs).  Alignment: W, signs and codes 16 bytes, scales 2 bytes.
 * Errors: E_NULL, E_UNSUPPORTED, E_SHAPE, E_ALIGN, E_HIP. */
int lowbit_quantize_weights(int fmt, int64_t N, int64_t K, const uint16_t* W_bf16,
                            const int8_t* signs, int8_t* codes, uint16_t* scales,
                            void* stream);

/* Activations for rotated weights ([OB] paragraph "工作原理", the signed
 * Hadamard rotation): per row of bf16 X [M][K] and block of 128,
 * X_rot = H (d * x) / sqrt(128) in fp32 (signs as given to
 * lowbit_quantize_weights), so that products with the rotated weights
 * equal those with the original ones.  Output fp32 [M][K].
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_HIP. */
int lowbit_rotate_act(int64_t M, int64_t K, const uint16_t* X_bf16, const int8_t* signs,
                      float* X_rot, void* stream);

/* Measurement helper, not part of the matrix-product path (the bandwidth
 * bound of [XH] section "ローカル27Bを阻む第一の壁：「1語生成するたびに全身を
 * 運び直す」"): reads the
 * `bytes` (a positive multiple of 16) at src once with 16-byte streaming
 * loads spread over the whole device and XORs the data into *out (device
 * uint32, caller-initialised), so the sustained HBM read rate can be timed
 * beside the decode kernels.  src 16-byte aligned, out 4-byte aligned.
 * Errors: E_NULL, E_SHAPE, E_ALIGN, E_HIP. */
int lowbit_hbm_read_probe(const void* src, int64_t bytes, uint32_t* out, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* LOWBIT_H */
