/*
 * q4_oracle.h -- plain, slow CPU oracle for 4-bit group-wise weight quantization.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The product library
 * (bit_group_wise_amd/libq4.so) never links, loads or calls it, and the two
 * share no source: this file has its own codebook literal, its own fp16/bf16
 * conversions and its own packing loops.
 *
 * Everything is scalar C, one element at a time, in the order the pages state
 * the method.  Floating point follows IEEE binary32 / binary64 as written in C
 * (compile with -O2 -ffp-contract=off, never -ffast-math).
 *
 * Sources (web pages on 4-bit group-wise quantization):
 *   [n4n]   "What is 4-bit quantization and why does it matter?", section
 *           "How 4-bit quantization works": affine quantize/dequantize formula,
 *           INT4-symmetric levels -8..7 with scale max|w|/7, the printed
 *           16-value NF4 table, the packed-uint8 unpack expression (low nibble
 *           first) and the dequantize = table value times block scale step.
 *   [atlas] "INT4" (AI technologies atlas), sections "How it works" and
 *           "Components": asymmetric levels 0..15, integer zero-point, per-group
 *           scale usually stored in FP16, groups of 32/64/128.
 *   [hf4]   "Loading a model in 4-bit", section "Block-wise quantisation, stated
 *           exactly": contiguous blocks, absmax c = max|w| per block, nearest of
 *           the 16 codebook entries after dividing by c, dequantize c*Q[i].
 *   [hf4]   section "Where the accuracy goes" and [bnb] "INT4 Quantization >
 *           Practical Implementation with bitsandbytes": the matmul runs in the
 *           16-bit compute dtype on dequantized weights.
 *   [dq]    Double quantization of the NF4 block constants: "Loading a model
 *           in 4-bit", the configuration flag and the section "Where the
 *           accuracy goes" (the constants are compressed too, about 0.4 bits
 *           per parameter saved), and the closing section on NF4 (the
 *           per-block scales quantized again in blocks of 256 to 8 bits,
 *           0.5 -> about 0.127 bits per parameter).  The 8-bit code is not
 *           given: read as symmetric absmax int8 coding (scale = block
 *           max / 127, nearest level), with a binary32 second-level constant
 *           per 256 absmax values (8/64 + 32/(64*256) = 0.127 bits at g = 64).
 *           No mean is subtracted (none is described).
 *   [n4n]   section "QLoRA fine-tunes in 4-bit": in QLoRA the 4-bit base
 *           weights stay frozen and the gradient passes through the
 *           dequantized weights, i.e. dX = dY . What (orc_matmul_dx).
 */
#ifndef Q4_ORACLE_H
#define Q4_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Format and dtype ids (the same numbering as the product ABI, defined here
 * independently). */
enum { ORC_NF4 = 0, ORC_INT4_SYM = 1, ORC_INT4_ASYM = 2, ORC_NF4_DQ = 3, ORC_FP4 = 4 };

/* Double quantization ([dq]): absmax values per second-level block. */
enum { ORC_DQ_BLOCK = 256 };
enum { ORC_F16 = 0, ORC_BF16 = 1 };

/* The NF4 codebook as printed (16 binary32 values). */
extern const float orc_nf4_table[16];

/* IEEE conversions written from the format definitions: round to nearest,
 * ties to even; fp16 subnormals are produced and consumed (no flush);
 * overflow gives infinity. */
float    orc_f16_to_f32(uint16_t h);
uint16_t orc_f32_to_f16(float f);
float    orc_bf16_to_f32(uint16_t b);
uint16_t orc_f32_to_bf16(float f);

/* Element-wise array forms of the conversions (n values). */
void orc_f32_to_f16_array(const float *in, uint16_t *out, int64_t n);
void orc_f16_to_f32_array(const uint16_t *in, float *out, int64_t n);
void orc_f32_to_bf16_array(const float *in, uint16_t *out, int64_t n);

/* The FP4 codebook (a reading, PARITY UNPINNED against the pages: [hf4]
 * "Developer" names the fp4 quant type without a table): the E2M1 values
 * 0, 0.5, 1, 1.5, 2, 3, 4, 6 with a sign bit (bit 3), divided by 6, each the
 * nearest binary32; code = sign * 8 + 2 * e + m. */
extern const float orc_fp4_table[16];

/* Nearest NF4 index of a binary32 value x (ties to the lower index). */
int orc_nf4_nearest(float x);
/* Nearest FP4 index (ties to the lower index, so 0 codes as +0). */
int orc_fp4_nearest(float x);
void orc_nf4_nearest_array(const float *in, uint8_t *out, int64_t n);

/* Second-level quantization of n absmax values c[] ([dq]): per run of
 * ORC_DQ_BLOCK values, s2[b] = c2 / 127 (c2 the run's max) and
 * qc[i] = clamp(rint(c[i] / s2), 0, 127), 0 where s2 == 0. */
void orc_double_quant(const float *c, int64_t n, uint8_t *qc, float *s2);

/* Byte offset of the s2 array in an NF4_DQ scales buffer with n_groups
 * codes: the codes rounded up to a multiple of 16 bytes. */
int64_t orc_dq_s2_offset(int64_t n_groups);

/* Quantize a row-major fp16 weight W[N][K] (bit patterns) with groups of g
 * contiguous elements along K.
 *   codes  : uint8[N*K/2], byte t = nib[2t] | nib[2t+1] << 4 (flat order)
 *   scales : NF4, FP4 -> float[N*K/g] (absmax), INT4 -> uint16 fp16 bits [N*K/g],
 *            NF4_DQ -> bytes: uint8 qc[N*K/g] (zero-filled up to the next
 *            multiple of 16), then float s2[ceil(N*K/g / 256)]; the codes are
 *            those NF4 gives
 *   zeros  : INT4-asym only, uint8[ceil(N*K/g / 2)], zero-points packed two
 *            per byte in flat group order, low nibble first; NULL otherwise.
 * Returns 0, or -1 on a bad argument (K % g != 0, unknown format, ...). */
int orc_quantize(int fmt, int g, const uint16_t *w, int64_t N, int64_t K,
                 uint8_t *codes, void *scales, uint8_t *zeros);

/* Dequantize to fp16 (out_t = ORC_F16) or bf16 (ORC_BF16) bit patterns,
 * out[N*K]. Returns 0 or -1. */
int orc_dequantize(int fmt, int g, const uint8_t *codes, const void *scales,
                   const uint8_t *zeros, int64_t N, int64_t K, int out_t,
                   uint16_t *out);

/* Reference product y[m][j] = sum_k x[m][k] * what[rows[j]][k] in binary64,
 * summed in k order, where what is the dequantized weight rounded to the
 * activation dtype act_t (x is given as act_t bit patterns, [M][K]).
 * absdot[m][j] = sum_k |x[m][k] * what[rows[j]][k]| (the tolerance scale).
 * rows == NULL means rows 0..N-1 (nrows must then equal N).
 * Returns 0 or -1. */
int orc_matmul(int fmt, int g, int act_t, const uint16_t *x, int64_t M,
               const uint8_t *codes, const void *scales, const uint8_t *zeros,
               int64_t N, int64_t K, const int64_t *rows, int64_t nrows,
               double *y, double *absdot);

/* Backward product through the dequantized weights ([n4n] "QLoRA fine-tunes
 * in 4-bit": gradients flow through the dequantized weights, which do not
 * change): dx[m][j] = sum_n dy[m][n] * what[n][cols[j]] in binary64 (n
 * order), what rounded to act_t as in orc_matmul; dy is [M][N] act_t bits;
 * absdot as in orc_matmul.  cols == NULL means columns 0..K-1.  Returns 0 or
 * -1. */
int orc_matmul_dx(int fmt, int g, int act_t, const uint16_t *dy, int64_t M,
                  const uint8_t *codes, const void *scales, const uint8_t *zeros,
                  int64_t N, int64_t K, const int64_t *cols, int64_t ncols,
                  double *dx, double *absdot);

#ifdef __cplusplus
}
#endif
#endif
