/*
 * q4.h -- C ABI of libq4: 4-bit group-wise LLM weight quantization on AMD
 * Instinct MI355X (gfx950).
 *
 * Four operations: quantize fp16 weights to packed 4-bit codes plus per-group
 * metadata, dequantize them back to fp16/bf16, and multiply activations by
 * the quantized weights without materialising them (y = x . W^T), as a decode
 * GEMV (1 <= M <= 16) and a prefill GEMM (any M).
 *
 * Definitions this library implements (web pages on 4-bit group-wise
 * quantization, cited by title and section):
 *   - "What is 4-bit quantization and why does it matter?", "How 4-bit
 *     quantization works": quantized = round((w - zero_point) / scale),
 *     dequantized = quantized * scale + zero_point; INT4-symmetric levels
 *     -8..7 with an implicit zero and scale = max|w| / 7; NF4's 16 values
 *     (the printed table, used verbatim); weights stored as packed uint8 with
 *     the low nibble holding the earlier element; dequantize = table value
 *     times the block scale.
 *   - "INT4" (AI technologies atlas), "How it works" and "Components":
 *     asymmetric levels 0..15 with an integer zero-point; per-group scale
 *     usually stored in FP16; groups of 32, 64 or 128 weights.
 *   - "Loading a model in 4-bit", "Block-wise quantisation, stated exactly":
 *     contiguous blocks, absmax c = max|w| stored per block, each weight coded
 *     as the nearest of the 16 codebook entries after dividing by c,
 *     dequantized as c * Q[i]; "Where the accuracy goes": the layer
 *     dequantizes to the 16-bit compute dtype and runs an ordinary 16-bit
 *     matmul (fp32 accumulation here).
 *   - Double quantization of the NF4 absmax (Q4_NF4_DQ): the same page's
 *     double-quantization flag and "Where the accuracy goes" (the block
 *     constants are compressed as well), and its closing section on NF4 (the
 *     per-block scales quantized again in blocks of 256 to 8 bits, from 0.5
 *     to about 0.127 bits per parameter).  The 8-bit coding is not spelled
 *     out; it is read here as symmetric absmax int8 with a binary32 constant
 *     per run of 256 absmax values (rules below).
 *   - FP4 (Q4_FP4): "Loading a model in 4-bit", "Developer", names the fp4
 *     quant type beside nf4 without printing its codebook.  Read here as the
 *     E2M1 element values (bit 3 the sign, bits 2..1 an exponent e, bit 0 a
 *     mantissa bit m: m/2 for e = 0, else 2^(e-1) (1 + m/2), i.e. 0, 0.5, 1,
 *     1.5, 2, 3, 4, 6) divided by 6, each the nearest binary32, used exactly
 *     as NF4's table (block absmax, nearest entry).  Its agreement with any
 *     other fp4 implementation is not established by the pages.
 *
 * Data layout (all row-major, W is [N, K] like a Linear layer's weight):
 *   w       fp16 [N, K]
 *   codes   uint8 [N, K/2]; byte t of the flat array holds element 2t in its
 *           low nibble and element 2t+1 in its high nibble.
 *   scales  NF4, FP4: float32 [N, K/g] (the block absmax c)
 *           INT4-sym / INT4-asym: fp16 [N, K/g]
 *           NF4_DQ: bytes.  uint8 qc[N*K/g] (the 8-bit absmax codes in flat
 *           group order r*(K/g) + j), zero bytes up to the next multiple of
 *           16, then float32 s2[ceil(N*K/g / 256)] (one per run of 256
 *           groups in flat order; runs cross row boundaries).
 *   zeros   INT4-asym only: uint8 [ceil(N*K/g / 2)], the integer zero-points
 *           (0..15) of the groups in flat order r*(K/g) + j, two per byte,
 *           low nibble first.  NULL for the other formats.
 *   x       [M, K] fp16 or bf16 (act_t); y [M, N] in the same dtype.
 * A group is g contiguous elements of one row (K % g == 0).
 *
 * Coding rules (bit-exact, no fast-math; binary32 IEEE division by the
 * stored scale, round-half-even):
 *   NF4   c = max|w|; code = index of the nearest table entry to w / c, ties
 *         to the lower index; c == 0 gives code 7 (the entry 0.0).
 *   SYM   s = fp16(max|w| / 7); nibble = clamp(rint(w / s), -8, 7) + 8;
 *         s == 0 gives nibble 8.
 *   ASYM  lo = min(0, min w), hi = max(0, max w); s = fp16((hi - lo) / 15);
 *         z = clamp(rint(-lo / s), 0, 15); nibble = clamp(rint(w / s) + z,
 *         0, 15); s == 0 gives z = 0 and nibble 0.
 *   FP4   as NF4 with the FP4 table; ties to the lower index, so 0 codes as
 *         +0 (code 0); c == 0 gives code 0.
 *   NF4_DQ codes exactly as NF4 (with the exact absmax c); then per run of
 *         256 absmax values, s2 = c2 / 127 with c2 the run's max, and
 *         qc = clamp(rint(c / s2), 0, 127) (0 where s2 == 0).
 * Dequantize: NF4 and FP4 Q[i] * c, SYM (nibble - 8) * s, ASYM (nibble - z) * s, one
 * binary32 product rounded once (nearest-even) to fp16 or bf16.  NF4_DQ first
 * recovers c' = qc * s2 (one binary32 product), then Q[i] * c' as NF4.
 *
 * Conventions:
 *   - Ownership: every buffer is device memory owned by the caller.  The
 *     library never allocates, frees or retains memory, keeps no state
 *     between calls and never synchronises; it only enqueues kernels on
 *     `stream` (a hipStream_t; NULL selects the null stream).  Its globals
 *     are read-only constant tables, plus the per-GPU sync words of
 *     q4_gemv_chain_static (a static device array, and a host table of their
 *     addresses filled once per device under a lock); every other call is
 *     thread-safe, and overlapping q4_gemv_chain_static calls on one GPU
 *     race (see there).
 *   - Errors: every call validates its arguments on the host, before any HIP
 *     call, and returns a q4_status.  Nothing aborts and no C++ exception
 *     crosses the ABI.  Faults inside a kernel surface at the caller's next
 *     synchronisation.
 *   - Alignment: w, codes, x and out must be 16-byte aligned (the kernels
 *     move 16 bytes per lane); scales must be 4-byte (NF4, FP4), 2-byte (INT4) or
 *     16-byte (NF4_DQ) aligned, y 2-byte aligned.  There is no slow fallback path.
 *   - Preconditions not checked: inputs are finite; output buffers do not
 *     alias inputs; the buffers are at least the sizes q4_*_bytes report.
 */
#ifndef Q4_H
#define Q4_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { Q4_NF4 = 0, Q4_INT4_SYM = 1, Q4_INT4_ASYM = 2, Q4_NF4_DQ = 3, Q4_FP4 = 4 } q4_format;
typedef enum { Q4_F16 = 0, Q4_BF16 = 1 } q4_dtype;
typedef enum {
    Q4_OK = 0,
    Q4_EINVAL = 1,       /* null pointer, N/K/M <= 0, K % g != 0, zeros given
                            (or missing) for the format */
    Q4_EUNSUPPORTED = 2, /* unknown format or dtype, g not in {32, 64, 128},
                            M > 16 for q4_gemv, a size beyond an entry
                            point's stated limit */
    Q4_EALIGN = 3,       /* a pointer violates the alignment rules above */
    Q4_EHIP = 4          /* the HIP runtime refused a launch */
} q4_status;

/* Sizes in bytes of the caller-allocated buffers for an [N, K] weight with
 * groups of g (0 for invalid arguments).
 *   codes:  exactly N*K/2.
 *   scales: the meaningful size -- N*(K/g)*4 (NF4, FP4), N*(K/g)*2 (INT4), or
 *           for NF4_DQ the 8-bit codes padded to a multiple of 16 plus
 *           4*ceil(N*(K/g)/256) -- plus P bytes of trailing padding;
 *   zeros:  the meaningful size ceil(N*(K/g)/2) (INT4-asym; 0 otherwise)
 *           plus P bytes of trailing padding;
 * where P = 16 + (the meaningful size rounded up to a multiple of 16, minus
 * the meaningful size), i.e. the total is the meaningful size plus 16,
 * rounded up to a multiple of 16.  Every entry point reads the meaningful
 * bytes only as values; q4_gemm with M > 16 fetches a row's scales and
 * zero-points for 256 columns at a time with wide loads that may start at
 * the last meaningful bytes and run into the padding, so a caller must
 * allocate the padded size (the padding's contents are never used and may
 * be anything).  q4_quantize writes only the meaningful bytes. */
size_t q4_codes_bytes(int64_t N, int64_t K);                      /* N*K/2 */
size_t q4_scales_bytes(q4_format f, int64_t N, int64_t K, int g); /* N*K/g * (4 NF4/FP4, 2 INT4), padded;
                                                                      NF4_DQ: qc, s2 as above, padded */
size_t q4_zeros_bytes(q4_format f, int64_t N, int64_t K, int g);  /* asym: ceil(N*K/g / 2), padded; else 0 */

/* Quantize fp16 weights w[N, K] into codes, scales and (asym) zeros.
 * Sources: the coding rules above ("How 4-bit quantization works";
 * "How it works" / "Components"; "Block-wise quantisation, stated exactly"). */
q4_status q4_quantize(q4_format f, int g, const void *w_f16, int64_t N, int64_t K,
                      uint8_t *codes, void *scales, uint8_t *zeros, void *stream);

/* Dequantize into out[N, K] of dtype out_t (fp16 or bf16).
 * Source: the dequantize rule above ("How 4-bit quantization works":
 * table value times the block scale; the affine inverse). */
q4_status q4_dequantize(q4_format f, int g, const uint8_t *codes, const void *scales,
                        const uint8_t *zeros, int64_t N, int64_t K, q4_dtype out_t,
                        void *out, void *stream);

/* Decode-shape product y[M, N] = x[M, K] . What^T for 1 <= M <= 16, reading
 * the packed weights once and dequantizing them in registers; fp32
 * accumulation, one rounding of y to act_t.  Every weight enters as the
 * value q4_dequantize writes in act_t, so the result equals a 16-bit matmul
 * on the dequantized weights up to summation order ("Where the accuracy
 * goes").  M = 1, 2 dequantize and multiply on the vector ALUs (binary32
 * dot products of 16-bit pairs) with one row per wave; 3 <= M <= 16 run as
 * a skinny product over blocks of 16 rows on the matrix cores.  M > 16
 * returns Q4_EUNSUPPORTED (use q4_gemm); K > Q4_GEMV_MAX_K returns
 * Q4_EUNSUPPORTED. */
#define Q4_GEMV_MAX_K 33554432
q4_status q4_gemv(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                  const uint8_t *codes, const void *scales, const uint8_t *zeros,
                  int64_t N, int64_t K, void *y, void *stream);

/* Prefill-shape product y[M, N] = x[M, K] . What^T for any M >= 1: weight
 * tiles are dequantized to the activation dtype on the fly (each value as
 * q4_dequantize writes it) and multiplied on the matrix cores with fp32
 * accumulation; y is rounded once to act_t ("Where the accuracy goes").
 * M <= 96 runs as the skinny product q4_gemv uses for 3 <= M <= 16, with
 * one, two or four blocks of 16 activation rows per launch (up to 64 rows)
 * and, past 64 rows, consecutive launches over row slices of x and y, all on
 * the caller's stream; 97 <= M <= 512 runs in tiles of 256 activation rows
 * by 128 weight rows, larger M in 256 x 256 tiles (the same bits either way).
 * K > Q4_GEMM_MAX_K returns Q4_EUNSUPPORTED. */
#define Q4_GEMM_MAX_K 4194304
q4_status q4_gemm(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                  const uint8_t *codes, const void *scales, const uint8_t *zeros,
                  int64_t N, int64_t K, void *y, void *stream);

/* Backward product through the frozen 4-bit weight, dX[M, K] = dY[M, N] .
 * What[N, K]: the gradient with respect to the layer input when the base
 * weights are quantized and frozen and only adapters train ("What is 4-bit
 * quantization and why does it matter?", "QLoRA fine-tunes in 4-bit": the
 * gradient flows through the dequantized weights, which never change).  Each
 * weight value is the one q4_dequantize writes in act_t; the products run on
 * the matrix cores with fp32 accumulation and dX is rounded once to act_t.
 * dy is [M, N], dx is [M, K], both act_t, row-major, 16-byte aligned.
 * Requires N % 8 == 0 (16-byte aligned dY rows), N <= Q4_GEMM_DX_MAX_N and
 * codes N*K/2 <= Q4_GEMV_CHAIN_MAX_CODES bytes, else Q4_EUNSUPPORTED. */
#define Q4_GEMM_DX_MAX_N 4194303
q4_status q4_gemm_dx(q4_format f, int g, q4_dtype act_t, const void *dy, int64_t M,
                     const uint8_t *codes, const void *scales, const uint8_t *zeros,
                     int64_t N, int64_t K, void *dx, void *stream);

/* A chain of decode GEMVs in one launch.  Each task is one M = 1 product
 * y[1, N] = x[1, K] . What^T with the layout and alignment rules of q4_gemv;
 * all tasks share the format, group size and activation dtype.  The tasks run
 * in order with the semantics of consecutive q4_gemv calls on the stream (and
 * the same bits in y): unless its flags hold Q4_TASK_NO_WAIT, a task reads x
 * only after every earlier task of the chain has written its y, so x may be
 * an earlier task's output.  Weights are read ahead across task boundaries,
 * so no task may write another task's weights.  Used for the weight stream of
 * a decode step, whose GEMVs are otherwise dominated by per-launch cost when
 * launched one by one ("Why it matters for deployment": a decode step reads
 * every weight once).
 *
 * ntasks is 1..Q4_GEMV_CHAIN_MAX; each K must satisfy K <= Q4_GEMV_CHAIN_MAX_K
 * and each task's codes N*K/2 <= Q4_GEMV_CHAIN_MAX_CODES bytes (else
 * Q4_EUNSUPPORTED); N and K are checked as in q4_gemv.  `sync` is a
 * device buffer of Q4_GEMV_CHAIN_SYNC_BYTES, 128-byte aligned, zeroed by the
 * caller before its first use: the kernel returns every word but word 2 to
 * zero when it ends, so the buffer can be reused without clearing by later
 * chains on the same stream; chains that may overlap (other streams) need
 * their own.  Word 2 becomes nonzero if a wait between tasks gave up after
 * about a second (the grid could not make progress; y is then undefined) and
 * stays set until the caller clears it.  The chain is one launch of one workgroup per
 * compute unit, cooperative when a task waits (its grid barrier needs every
 * workgroup resident): a launch the runtime refuses returns Q4_EHIP. */
#define Q4_GEMV_CHAIN_MAX 64
#define Q4_GEMV_CHAIN_MAX_K 16384
#define Q4_GEMV_CHAIN_MAX_CODES 2147483519LL /* 2^31 - 129 */
#define Q4_GEMV_CHAIN_SYNC_BYTES 1280 /* 10 lines of 128 bytes */
#define Q4_TASK_NO_WAIT 1u /* x is not written by earlier tasks: no grid-wide wait */
typedef struct {
    const void *x;        /* [1, K] act_t */
    const uint8_t *codes; /* [N, K/2] */
    const void *scales;   /* [N, K/g] */
    const uint8_t *zeros; /* asym: packed zero-points; else NULL */
    void *y;              /* [1, N] act_t */
    int64_t N, K;
    uint32_t flags;       /* 0 or Q4_TASK_NO_WAIT */
} q4_gemv_task;
q4_status q4_gemv_chain(q4_format f, int g, q4_dtype act_t, const q4_gemv_task *tasks,
                        int ntasks, uint32_t *sync, void *stream);

/* q4_gemv_chain without the sync buffer, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * allocation): the sync words live in a static device array of
 * Q4_GEMV_CHAIN_SYNC_BYTES that the library holds on each GPU it runs on
 * until the process ends.  Same tasks, limits, status codes and results as
 * q4_gemv_chain (the chain's size limits bound everything the array holds,
 * so no larger input needs more of it).  It calls no allocating routine:
 * the array's device address is looked up once per device, on the first
 * call with that device current, and a failed lookup returns Q4_EHIP.  The
 * kernel leaves the barrier counters at zero for the next call; the timeout
 * flag (word 2 of the sync words) is not reported.  All calls on one GPU
 * share the array: chains that may overlap on one GPU (different streams,
 * or one call still running while another is enqueued elsewhere) race and
 * must use q4_gemv_chain with their own sync buffers instead. */
q4_status q4_gemv_chain_static(q4_format f, int g, q4_dtype act_t, const q4_gemv_task *tasks,
                               int ntasks, void *stream);

/* A static, human-readable name for a status code. */
const char *q4_status_str(q4_status s);

#ifdef __cplusplus
}
#endif

#endif /* Q4_H */
