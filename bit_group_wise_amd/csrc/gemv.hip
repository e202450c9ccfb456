// gemv.hip -- decode-shape fused dequant-GEMV, y[M, N] = x[M, K] . What^T,
// M = 1 or 2, with no matrix-core instructions (three or more rows run as
// the skinny matrix-core product of gemv_mfma.hip), and the chained M = 1
// kernel behind q4_gemv_chain.
//
// Method ("Loading a model in 4-bit", "Where the accuracy goes"; "INT4
// Quantization > Practical Implementation with bitsandbytes"): the layer
// multiplies 16-bit activations by the dequantized weights; "What is 4-bit
// quantization and why does it matter?", "Why it matters for deployment":
// a decode step reads every weight once, so the kernel is bound by the bytes
// of packed codes and scales it streams.
//
// gfx950 mapping:
//  * A wave owns one weight row at a time.  Along K it walks stages of
//    128 chunks of 32 weights: lane l reads chunks l and 64 + l (16 bytes of
//    codes each), so each load instruction of the wave covers 1 KB of
//    consecutive bytes.  Loads are buffer loads (tails past a row or past the
//    matrix read zeros) marked non-temporal, since every weight byte is used
//    once.  The loads of the next positions -- of the same or the next row --
//    are issued before the current stage is computed, so HBM reads stay in
//    flight.
//  * The scale is hoisted out of the inner product: a chunk lies inside one
//    group, so p = sum x * level is formed first and then acc += s * p
//    (INT4-asym: acc += s * (p - z * sum x)).
//  * Levels come from a per-workgroup LDS table indexed by a whole code byte:
//    an entry holds the two nibbles' levels as a packed 16-bit pair, so one
//    v_dot2_f32_{f16,bf16} multiplies two weights by two activations into an
//    fp32 accumulator.  The table is replicated per lane (a lane reads only
//    its own bank) and a byte's LDS address is one v_perm_b32 (code byte ->
//    address bits 8..15, lane slot -> bits 0..7).
//  * Level pairs: INT4 levels are small integers, exact in bf16 and fp16, so
//    the activations are used as they are.  NF4 levels are taken in fp16; for
//    bf16 activations with M <= 2 the activations are first converted to
//    fp16 after an exact power-of-two scaling per 32-value chunk (max |x|
//    mapped into [2^14, 2^15)), which is lossless over fp16's normal range.
//    For larger M with bf16 activations NF4 levels are split into bf16 hi +
//    lo parts (two dot2 per byte).
//  * Activations: for M = 1 and rows that fit one stage (K <= 4096) each lane
//    keeps its slices in registers; else, for M <= 2, they are staged once
//    per workgroup in LDS (rows padded to whole stages with zeros, 16 bytes
//    of skew per 64-byte chunk so the 16-byte reads of a wave do not collide
//    in banks); larger M reads them from L2 step by step.
//  * Lane partial sums are reduced across the wave with DPP; y is rounded
//    once to the activation dtype.
//  * NF4 with double-quantized absmax ("Loading a model in 4-bit", "Where
//    the accuracy goes"): a chunk's scale is read as its group's 8-bit code
//    (one byte) and its run's binary32 constant (a dword that the 8 to 32
//    groups of a row in the same run share, so it comes from cache), and
//    the absmax is recovered with one product; all else is NF4's path.
#include <type_traits>

#include "q4_common.hpp"
#include "q4_internal.hpp"

namespace q4 {
namespace {

// Steps (of 8 weights) between scheduling barriers in a stage; 0 = none.
#ifndef Q4_GEMV_SB
#define Q4_GEMV_SB 2
#endif
// Positions (stages) whose loads are kept in flight per wave, in the
// single-product and the chained kernels.
#ifndef Q4_GEMV_DEPTH
#define Q4_GEMV_DEPTH 2
#endif
#ifndef Q4_GEMV_CHAIN_DEPTH
#define Q4_GEMV_CHAIN_DEPTH 2
#endif

constexpr int kTableDwords = 256 * 64;  // 256 entries x 256 bytes = 64 KB
constexpr int kXBytes = 80 * 1024;      // LDS region for staged activations
constexpr int kStageChunks = 128;       // 16-byte chunks per row per stage
constexpr int kStageXBytes = kStageChunks * 64;  // activation bytes per row per stage

// Where a wave reads its activations from.
enum XSrc { X_GLOBAL = 0, X_LDS = 1, X_REG = 2 };

// Per-kernel arithmetic choices (see the header comment).
template <int FMT, int ACT, int XS>
struct Cfg {
    // bf16 activations converted to fp16 for NF4 when they are staged
    static constexpr bool conv_x = level_fmt(FMT) == Q4_NF4 && ACT == Q4_BF16 && XS != X_GLOBAL;
    // dot2 operand type
    static constexpr int ct = (ACT == Q4_F16 || conv_x) ? Q4_F16 : Q4_BF16;
    // NF4 in bf16: hi + lo level parts (two table dwords per byte)
    static constexpr bool pair = level_fmt(FMT) == Q4_NF4 && ct == Q4_BF16;
};

__constant__ uint32_t c_parts[3][16] = {
#define ROW(a) {a[0], a[1], a[2], a[3], a[4], a[5], a[6], a[7], a[8], a[9], a[10], a[11], a[12], a[13], a[14], a[15]}
    ROW(kPairParts.nf4_bf16_hi), ROW(kPairParts.nf4_bf16_lo), ROW(kPairParts.nf4_f16_hi),
#undef ROW
};

template <int CT>
__device__ __forceinline__ float dot2(uint32_t a, uint32_t b, float c)
{
    if constexpr (CT == Q4_BF16)
        return __builtin_amdgcn_fdot2_f32_bf16(std::bit_cast<bf16x2>(a), std::bit_cast<bf16x2>(b), c,
                                               false);
    else
        return __builtin_amdgcn_fdot2(std::bit_cast<f16x2>(a), std::bit_cast<f16x2>(b), c, false);
}

template <int CT>
__device__ __forceinline__ uint32_t level_bits(int v)
{
    return CT == Q4_BF16 ? f2bf_bits((float)v) : f2h_bits((float)v);
}

// The byte-indexed table.  Single layout: entry e, lane slot L (0..63) at
// byte e*256 + 4L.  Pair layout (NF4 in bf16): hi part at e*256 + 4L, lo
// part at e*256 + 128 + 4L, L in 0..31.  It is filled in 16-byte pieces:
// thread t writes pieces t, t + BLOCK, ..., so each store instruction covers
// consecutive addresses; a piece lies in one entry (half), so its dwords
// are equal.

template <int CTRL, int ROW_MASK>
__device__ __forceinline__ float dpp_f32(float x)
{
    return std::bit_cast<float>(
        __builtin_amdgcn_update_dpp(0, std::bit_cast<int>(x), CTRL, ROW_MASK, 0xf, false));
}

// Sum over the 64 lanes with DPP row operations; the total is returned to
// every lane (read from lane 63).
__device__ __forceinline__ float wave_sum(float v)
{
    v += dpp_f32<0xb1, 0xf>(v);   // quad_perm [1,0,3,2]
    v += dpp_f32<0x4e, 0xf>(v);   // quad_perm [2,3,0,1]
    v += dpp_f32<0x141, 0xf>(v);  // row_half_mirror
    v += dpp_f32<0x140, 0xf>(v);  // row_mirror: every lane holds its row's sum
    v += dpp_f32<0x142, 0xa>(v);  // row_bcast15 into rows 1 and 3
    v += dpp_f32<0x143, 0xc>(v);  // row_bcast31 into rows 2 and 3
    return std::bit_cast<float>(__builtin_amdgcn_readlane(std::bit_cast<int>(v), 63));
}

// Buffer resource over [base, base + bytes): loads past the end return zero
// (the hardware range check), so row and chunk tails need no branches.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int64_t bytes)
{
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0xffffffffll ? 0xffffffffu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             0x00020000);
}

// Buffer views of one weight row n0: its codes, scales and zero-point bytes
// (empty for n0 >= N, so a position past the last row loads zeros).  With
// double-quantized absmax, `scales` covers the row's 8-bit absmax codes and
// s2 points at the second-level constant of the run holding the row's first
// group (the kernels receive the constants' base in place of `zeros`).
struct RowViews {
    __amdgpu_buffer_rsrc_t codes, scales, zeros;
    int zpar;  // parity of the row's first flat group index (asym), or its
               // position in its run of kDqRun groups (double quantization)
    const float *s2;
};

template <int FMT>
__device__ __forceinline__ RowViews row_views(const uint8_t *codes, const void *scales,
                                              const uint8_t *zeros, int64_t n0, int64_t N,
                                              int64_t row_bytes, int64_t G)
{
    constexpr int ss = FMT == Q4_NF4 ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);
    const bool live = n0 < N;
    RowViews v;
    v.s2 = nullptr;
    v.codes = make_rsrc(codes + n0 * row_bytes, live ? row_bytes : 0);
    v.scales = make_rsrc((const char *)scales + n0 * G * ss, live ? G * ss : 0);
    const int64_t g0 = n0 * G;
    v.zpar = (int)(g0 & 1);
    if constexpr (FMT == Q4_INT4_ASYM) {
        v.zeros = make_rsrc(zeros + (g0 >> 1), live ? ((g0 + G - 1) >> 1) - (g0 >> 1) + 1 : 0);
    } else if constexpr (FMT == Q4_NF4_DQ) {
        // g0 >= 0: shifts instead of signed division; a row past the end
        // points at the first constant (read, never used: its codes are 0)
        const uint64_t ug0 = (uint64_t)g0;
        v.s2 = (const float *)zeros + (live ? ug0 >> 8 : 0);
        v.zpar = (int)(ug0 & (kDqRun - 1));
        v.zeros = v.codes;
    } else {
        v.zeros = v.codes;
    }
    return v;
}

// One pipeline stage of a wave: 128 chunks of 32 weights of one row; lane l
// holds chunks l and 64 + l of the stage (so each of the two 16-byte loads
// of the wave reads 1 KB of consecutive codes), with their scales and
// zero-points.
struct Stage {
    u32x4 cw[2];
    float sc[2];
    float zf[2];
    // double quantization: the constants of the (at most 3) runs of kDqRun
    // groups the row touches (scalar registers) and the row's first group's
    // position in the first of them
    float s2[3];
    int zpar;
};

// Chunk of half h of stage s for a lane.
__device__ __forceinline__ int stage_chunk(int s, int lane, int h) { return kStageChunks * s + 64 * h + lane; }

// Non-temporal loads: the weights are streamed once per product, so they are
// not kept in the caches (the "nt" cache-policy bit).
constexpr int kNT = 2;

// Chunks past the row end (C chunks per row) are sent out of the row's
// views, so they read zeros without touching memory (their activations are
// zero as well).
template <int FMT>
__device__ __forceinline__ void load_stage(Stage &st, const RowViews &v, int s, int lane, int gshift,
                                           int C)
{
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int ch = stage_chunk(s, lane, h);
        const bool in = ch < C;
        st.cw[h] = __builtin_amdgcn_raw_buffer_load_b128(v.codes, in ? 16 * ch : -16, 0, kNT);
        const int gl = (32 * ch) >> gshift;  // group index within the row
        if constexpr (FMT == Q4_NF4)
            st.sc[h] = std::bit_cast<float>(
                __builtin_amdgcn_raw_buffer_load_b32(v.scales, in ? 4 * gl : -16, 0, kNT));
        else if constexpr (FMT == Q4_NF4_DQ)  // the 8-bit code; the constant below
            st.sc[h] = std::bit_cast<float>((uint32_t)
                __builtin_amdgcn_raw_buffer_load_b8(v.scales, in ? gl : -16, 0, kNT));
        else
            st.sc[h] = h2f(__builtin_amdgcn_raw_buffer_load_b16(v.scales, in ? 2 * gl : -16, 0, kNT));
        if constexpr (FMT == Q4_INT4_ASYM) {
            const int gz = gl + v.zpar;
            const uint32_t b =
                __builtin_amdgcn_raw_buffer_load_b8(v.zeros, in ? gz >> 1 : -16, 0, kNT);
            st.zf[h] = (float)((b >> ((gz & 1) * 4)) & 0xf);
        } else {
            st.zf[h] = 0.0f;
        }
    }
    if constexpr (FMT == Q4_NF4_DQ) {
        // One scalar load of the constants of the row's runs (a row of at
        // most 16384 / 32 groups touches at most 3 runs; the last ones may
        // read the buffer's padding, never used), rather than a vector load
        // per stage: the vector memory instructions per stage are what the
        // loop's rate is most sensitive to.  The group's run is picked when
        // the stage is computed.
        typedef float f32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
        const f32x4a4 c = *(const __attribute__((address_space(4))) f32x4a4 *)v.s2;
        st.s2[0] = c[0];
        st.s2[1] = c[1];
        st.s2[2] = c[2];
        st.zpar = v.zpar;
    }
}

// LDS byte offset of activation byte o of the staged rows: 16 bytes of skew
// per 64-byte chunk, so the 16 lanes of a read pass (16-byte reads, one
// chunk apart) fall on 16 distinct groups of 4 banks (offsets 80 l mod 256).
__device__ __forceinline__ int xpad(int o) { return o + ((o >> 6) << 4); }

// Activations of step (chunk ch, dword j) for rows m < MT.
template <int MT, int XS>
__device__ __forceinline__ void load_x(u32x4 (&xv)[MT], const uint32_t *xs,
                                       __amdgpu_buffer_rsrc_t xr, int K, int xrow, int ch, int C,
                                       int j)
{
    if constexpr (XS == X_LDS) {
        // rows are zero past K, up to whole stages
#pragma unroll
        for (int m = 0; m < MT; ++m)
            xv[m] = *(const u32x4 *)((const char *)xs + xpad(m * xrow + 64 * ch + 16 * j));
    } else {
        // chunks past the row end are sent out of range, so they read zeros;
        // rows m >= M lie past the end of the x view and read zeros too
        const int base = ch < C ? 64 * ch + 16 * j : 0x7fffff00;
#pragma unroll
        for (int m = 0; m < MT; ++m)
            xv[m] = __builtin_amdgcn_raw_buffer_load_b128(xr, base + m * 2 * K, 0, 0);
    }
}

// Largest |value| of the two bf16 halves of a dword.
__device__ __forceinline__ float bf2_absmax(uint32_t u)
{
    return fmaxf(fabsf(std::bit_cast<float>(u << 16)), fabsf(std::bit_cast<float>(u & 0xffff0000u)));
}

// Maximum over aligned groups of 4 lanes (returned to each lane of the group).
__device__ __forceinline__ float max4(float v)
{
    v = fmaxf(v, dpp_f32<0xb1, 0xf>(v));  // lane ^ 1
    v = fmaxf(v, dpp_f32<0x4e, 0xf>(v));  // lane ^ 2
    return v;
}

// Powers of two f = 2^(14 - e) and 1/f, e the exponent of a >= 0, so that
// a * f lies in [2^14, 2^15) (clamped so both stay normal binary32).
__device__ __forceinline__ void x_scale(float a, float &f, float &inv)
{
    const uint32_t b = std::bit_cast<uint32_t>(a);
    int e = b ? (int)((b >> 23) & 0xff) - 127 : 14;
    e = e < -100 ? -100 : e;
    f = std::bit_cast<float>((uint32_t)(14 - e + 127) << 23);
    inv = std::bit_cast<float>((uint32_t)(e - 14 + 127) << 23);
}

// bf16 pair -> fp16 pair after multiplying by the power of two f (exact over
// fp16's normal range, nearest-even below it).
__device__ __forceinline__ uint32_t bf2_to_h2(uint32_t u, float f)
{
    const float a = std::bit_cast<float>(u << 16) * f;
    const float b = std::bit_cast<float>(u & 0xffff0000u) * f;
    return pack_h2(a, b);
}

// Products of one stage: 8 steps of 8 weights (two chunks x four dwords of
// codes).  Scheduling barriers every Q4_GEMV_SB steps keep the table reads of
// later steps from being hoisted (which would exhaust the register budget).
template <int FMT, int CT, bool PAIR, int MT, int XS>
__device__ __forceinline__ void compute_stage(const Stage &st, float (&acc)[MT],
                                              const uint32_t *__restrict__ tbl, const uint32_t *xs,
                                              const u32x4 (&xreg)[XS == X_REG ? 8 * MT : 1],
                                              const float (&xinv)[MT][2], __amdgpu_buffer_rsrc_t xr,
                                              int K, int xrow, int s, int lane, int C,
                                              uint32_t laneoff, int gshift)
{
    constexpr uint32_t kSel[4] = {0x0c0c0400u, 0x0c0c0500u, 0x0c0c0600u, 0x0c0c0700u};
    const uint32_t ones = CT == Q4_BF16 ? 0x3f803f80u : 0x3c003c00u;
    // two independent accumulator chains per output (and two more for the lo
    // parts), so consecutive dot2 do not wait on each other
    constexpr int NA = MT <= 2 ? 2 : 1;
    u32x4 xv[MT];
    if constexpr (XS == X_REG) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            xv[m] = xreg[m * 8];
    } else {
        load_x<MT, XS>(xv, xs, xr, K, xrow, stage_chunk(s, lane, 0), C, 0);
    }
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        float p[MT][NA], pl[MT][NA];
        float sx[MT];
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            sx[m] = 0.0f;
#pragma unroll
            for (int a = 0; a < NA; ++a)
                p[m][a] = pl[m][a] = 0.0f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            u32x4 xn[MT];
            if (h * 4 + j < 7) {
                if constexpr (XS == X_REG) {
#pragma unroll
                    for (int m = 0; m < MT; ++m)
                        xn[m] = xreg[m * 8 + h * 4 + j + 1];
                } else {
                    load_x<MT, XS>(xn, xs, xr, K, xrow, stage_chunk(s, lane, j == 3 ? h + 1 : h),
                                   C, (j + 1) & 3);
                }
            }
            if constexpr (FMT == Q4_INT4_ASYM) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        sx[m] = dot2<CT>(xv[m][k], ones, sx[m]);
            }
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t addr = __builtin_amdgcn_perm(st.cw[h][j], laneoff, kSel[k]);
                const uint32_t lv = *(const uint32_t *)((const char *)tbl + addr);
                uint32_t lo = 0;
                if constexpr (PAIR)
                    lo = *(const uint32_t *)((const char *)tbl + addr + 128);
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    p[m][k % NA] = dot2<CT>(xv[m][k], lv, p[m][k % NA]);
                    if constexpr (PAIR)
                        pl[m][k % NA] = dot2<CT>(xv[m][k], lo, pl[m][k % NA]);
                }
            }
            if (h * 4 + j < 7) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    xv[m] = xn[m];
            }
#if Q4_GEMV_SB > 0
            if ((j + 1) % Q4_GEMV_SB == 0)
                __builtin_amdgcn_sched_barrier(0);
#endif
        }
#pragma unroll
        for (int m = 0; m < MT; ++m) {
            float t = 0.0f;
#pragma unroll
            for (int a = 0; a < NA; ++a)
                t += PAIR ? p[m][a] + pl[m][a] : p[m][a];
            if constexpr (FMT == Q4_INT4_ASYM)
                t = __builtin_fmaf(-st.zf[h], sx[m], t);
            float sc = st.sc[h];
            if constexpr (FMT == Q4_NF4_DQ) {
                // The half's 64 chunks cover at most 64 groups, so at most
                // two runs: the run of its first group (ra) and the next
                // (rb), picked per half from wave-uniform values; a lane
                // takes rb when its group is at or past the run boundary.
                // Groups are counted from the start of the row's first run.
                const int u = st.zpar + ((kStageChunks * 32 * s + 64 * 32 * h) >> gshift);
                const int r0 = u >> 8;                         // 0..2
                const int thr = 256 * (r0 + 1) - u;            // first lane group in rb
                const uint32_t a0 = std::bit_cast<uint32_t>(st.s2[0]);
                const uint32_t a1 = std::bit_cast<uint32_t>(st.s2[1]);
                const uint32_t a2 = std::bit_cast<uint32_t>(st.s2[2]);
                const uint32_t ra = r0 == 0 ? a0 : (r0 == 1 ? a1 : a2);
                const uint32_t rb = r0 == 0 ? a1 : a2;
                const int lg = (32 * lane) >> gshift;          // the lane's group in the half
                const float s2 = std::bit_cast<float>(lg >= thr ? rb : ra);
                sc = keep_f32((float)std::bit_cast<uint32_t>(st.sc[h]) * s2);  // c' = qc * s2
            }
            acc[m] = __builtin_fmaf(t, sc * xinv[m][h], acc[m]);
        }
    }
}

// Workgroup shape: 16 waves (one workgroup per CU, sharing one table and the
// staged activations) when the activations are staged, else 8 waves (two
// workgroups per CU).
#ifndef Q4_GEMV_STAGED_WAVES
#define Q4_GEMV_STAGED_WAVES 16
#endif
template <int XS>
struct Shape {
    static constexpr int waves = XS != X_GLOBAL ? Q4_GEMV_STAGED_WAVES : 8;
    static constexpr int block = waves * 64;
    static constexpr int per_cu = XS != X_GLOBAL ? 1 : 2;
    // pieces of 16 bytes per thread that cover the staged-activation region
    static constexpr int x_pieces = (kXBytes / 16 + block - 1) / block;
};

// A wave's position in its walk: row and stage along K.
struct Pos {
    int row, s;
};

// Each wave walks its rows and, inside a row, the stages along K.  The
// loads of the next P positions are kept in flight in a ring of stage
// registers: position q is computed while q+1..q+P-1 are arriving, and its
// slot is refilled with position q+P right after.  The first P positions are
// issued before the LDS is filled.
template <int FMT, int ACT, int MT, int XS, int P>
__global__ __launch_bounds__(Shape<XS>::block)
__attribute__((amdgpu_waves_per_eu(XS != X_GLOBAL ? Shape<XS>::waves / 4 : (MT < 8 ? 4 : 2))))
void gemv_kernel(const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
                 const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int N, int K,
                 int gshift, uint16_t *__restrict__ y)
{
    using F = Cfg<FMT, ACT, XS>;
    constexpr int kWaves = Shape<XS>::waves;
    constexpr int kBlock = Shape<XS>::block;
    // One LDS block with the table first, at address 0, so that a lookup's
    // address is the v_perm result itself.
    struct Lds {
        uint32_t tbl[kTableDwords];
        uint32_t xs[XS != X_GLOBAL ? kXBytes / 4 : 4];
        // inverse activation scale of each staged 32-value chunk
        float xsinv[XS != X_GLOBAL && Cfg<FMT, ACT, XS>::conv_x ? kXBytes / 64 : 1];
    };
    __shared__ Lds lds;
    uint32_t *const tbl = lds.tbl;
    uint32_t *const xs = lds.xs;
    float *const xsinv = lds.xsinv;

    const int lane = threadIdx.x & 63;
    const uint32_t laneoff = (uint32_t)(F::pair ? (lane & 31) : lane) << 2;
    const int C = K >> 5;                                    // 16-byte chunks per row
    const int S = (C + kStageChunks - 1) / kStageChunks;    // stages per row
    const int G = K >> gshift;                               // groups per row
    const int row_bytes = K >> 1;
    const int xrow = S * kStageXBytes;                       // staged bytes per x row
    const int total_waves = gridDim.x * kWaves;
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(x, (int64_t)M * K * 2);

    auto advance = [&](Pos q) {
        if (++q.s == S) {
            q.s = 0;
            q.row += total_waves;
        }
        return q;
    };

    // Prologue, ordered so that nothing waits behind the weight stream
    // (vector-memory loads retire in order): activations first, then the
    // table's level values, then the first P weight positions.
    u32x4 xreg[XS == X_REG ? 8 * MT : 1];
    constexpr int XP = Shape<XS>::x_pieces;
    u32x4 xt[XP];
    int xp[XP];
    if constexpr (XS != X_GLOBAL) {
        // the workgroup stages x once in LDS: row m at m * xrow, zero from
        // byte 2K to the end of its last stage, in pieces of 16 bytes
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            const int p = threadIdx.x + kBlock * i;
            const int m = (16 * p) / xrow, o = 16 * p - m * xrow;
            xp[i] = p < M * xrow / 16 ? p : -1;
            xt[i] = u32x4{0, 0, 0, 0};
            if (xp[i] >= 0 && o < 2 * K)
                xt[i] = __builtin_amdgcn_raw_buffer_load_b128(xr, m * 2 * K + o, 0, 0);
        }
    }
    // NF4 level parts: lane i (mod 16) holds entry i; fetched by lane permutes
    uint32_t part_lo = 0, part_hi = 0;
    if constexpr (level_fmt(FMT) == Q4_NF4) {
        part_lo = c_parts[F::pair ? 0 : 2][lane & 15];
        if constexpr (F::pair)
            part_hi = c_parts[1][lane & 15];
    }

    // ring of P in-flight positions (a row past the end has an empty view,
    // so its loads return zeros and it is never computed)
    Pos pos[P];
    Stage st[P];
    pos[0] = Pos{(int)__builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6)), 0};
#pragma unroll
    for (int q = 0; q < P; ++q) {
        if (q > 0)
            pos[q] = advance(pos[q - 1]);
        const RowViews v = row_views<FMT>(codes, scales, zeros, pos[q].row, N, row_bytes, G);
        load_stage<FMT>(st[q], v, pos[q].s, lane, gshift, C);
    }

    // fp16 conversion of bf16 activations with a power-of-two scale per
    // 32-value chunk (half of a lane's share of a stage); the products are
    // scaled back exactly together with the group scale
    if constexpr (XS != X_GLOBAL) {
#pragma unroll
        for (int i = 0; i < XP; ++i) {
            if constexpr (F::conv_x) {
                // the 4 pieces of a chunk sit in 4 consecutive threads
                float mx = 0.0f;
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    mx = fmaxf(mx, bf2_absmax(xt[i][k]));
                mx = max4(mx);
                float f, inv;
                x_scale(mx, f, inv);
#pragma unroll
                for (int k = 0; k < 4; ++k)
                    xt[i][k] = bf2_to_h2(xt[i][k], f);
                if (xp[i] >= 0 && (xp[i] & 3) == 0)
                    xsinv[xp[i] >> 2] = inv;
            }
            if (xp[i] >= 0)
                *(u32x4 *)((char *)xs + xpad(16 * xp[i])) = xt[i];
        }
    }
    // table: level values by lane permutes (NF4) or arithmetic (INT4)
#pragma unroll
    for (int i = 0; i < kTableDwords / 4 / kBlock; ++i) {
        const int piece = threadIdx.x + kBlock * i;
        const int e = piece >> 4, h = (piece >> 3) & 1;
        const int n0 = e & 15, n1 = e >> 4;
        uint32_t v;
        if constexpr (level_fmt(FMT) == Q4_NF4) {
            // every lane holds the same part variable, so the permute reads
            // entry n of that part; the hi/lo choice is made afterwards
            uint32_t a = (uint32_t)__shfl((int)part_lo, n0), b = (uint32_t)__shfl((int)part_lo, n1);
            if constexpr (F::pair) {
                const uint32_t c = (uint32_t)__shfl((int)part_hi, n0);
                const uint32_t d = (uint32_t)__shfl((int)part_hi, n1);
                if (h) {
                    a = c;
                    b = d;
                }
            }
            v = a | (b << 16);
        } else {
            const int off = FMT == Q4_INT4_SYM ? 8 : 0;
            v = level_bits<F::ct>(n0 - off) | (level_bits<F::ct>(n1 - off) << 16);
        }
        ((u32x4 *)tbl)[piece] = u32x4{v, v, v, v};
    }
    __syncthreads();

    // one stage per row (M = 1): each lane keeps its activation slices
    // (chunks lane and 64 + lane) and their inverse scales in registers for
    // the whole kernel
    float xinv_reg[MT][2];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        xinv_reg[m][0] = xinv_reg[m][1] = 1.0f;
    if constexpr (XS == X_REG) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                xreg[m * 8 + t] = *(const u32x4 *)((const char *)xs +
                                                   xpad(m * xrow + 64 * stage_chunk(0, lane, t >> 2) +
                                                        16 * (t & 3)));
            if constexpr (F::conv_x) {
                xinv_reg[m][0] = xsinv[m * (xrow >> 6) + stage_chunk(0, lane, 0)];
                xinv_reg[m][1] = xsinv[m * (xrow >> 6) + stage_chunk(0, lane, 1)];
            }
        }
    }

    float acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        acc[m] = 0.0f;

    // A round of the ring is never left in the middle (the load waits stay
    // partial only if every path refills every slot): a position past the
    // last row has loaded zeros from an empty view; it is computed on them
    // and writes nothing.
    while (pos[0].row < N) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const Pos cp = pos[q];
            float xinv[MT][2];
#pragma unroll
            for (int m = 0; m < MT; ++m) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    if constexpr (F::conv_x && XS == X_LDS)
                        xinv[m][h] = xsinv[m * (xrow >> 6) + stage_chunk(cp.s, lane, h)];
                    else
                        xinv[m][h] = xinv_reg[m][h];
                }
            }
            compute_stage<FMT, F::ct, F::pair, MT, XS>(st[q], acc, tbl, xs, xreg, xinv, xr, K,
                                                      xrow, cp.s, lane, C, laneoff, gshift);
            // (double quantization: keep the refill after the compute, which
            // the scheduler otherwise hoists at the cost of registers)
            if constexpr (FMT == Q4_NF4_DQ)
                __builtin_amdgcn_sched_barrier(0);
            // refill this slot with the position P steps ahead
            pos[q] = advance(pos[(q + P - 1) % P]);
            {
                const RowViews v =
                    row_views<FMT>(codes, scales, zeros, pos[q].row, N, row_bytes, G);
                load_stage<FMT>(st[q], v, pos[q].s, lane, gshift, C);
            }
            if (cp.s == S - 1) {
                float out = 0.0f;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float t = wave_sum(acc[m]);
                    acc[m] = 0.0f;
                    if (lane == m)
                        out = t;
                }
                if (cp.row < N && lane < M && lane < MT)
                    y[(int64_t)lane * N + cp.row] =
                        (uint16_t)(ACT == Q4_BF16 ? f2bf_bits(out) : f2h_bits(out));
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Chained GEMVs: one persistent launch runs a list of M = 1 GEMVs in order.
//
// The weights never depend on earlier tasks, so each compute wave's ring of
// in-flight weight loads runs on across task boundaries.  Only x may depend
// on earlier tasks.  A workgroup is 15 compute waves and one loader wave.
// x sits in LDS in 8 slots of one stage each (8 KB); task t's stages take
// consecutive slots from slot base_t on (mod 8), tasks in turn, so a slot is
// reused only by a task at least two later.  The loader copies x of task t
// (by DMA, as early as the slots allow) once every compute wave has entered
// the task after the last one that used those slots (the gate, computed on
// the host) and publishes it; a compute wave entering task t waits only for
// that.  So waves may drift several tasks apart.  With no task waiting for
// earlier outputs, each workgroup works on one contiguous block of the
// tasks' rows and loads and enters only the block's tasks.  Otherwise every
// task's rows are spread over all waves, and for a task that reads earlier
// outputs the loader first waits until every compute wave has finished the
// earlier tasks, then for the whole grid (a grid barrier between loader
// waves).  The compute waves never wait for each other.  The table is
// filled once per launch.
struct ChainTask {
    const uint16_t *x;
    const uint8_t *codes;
    const void *scales;
    const uint8_t *zeros;
    uint16_t *y;
    int N, K;
    // bit 0: wait for every earlier task before reading x; bits 1-3: the
    // first x slot; bits 8-15: the gate (every compute wave must have
    // entered that task before x is copied)
    int ctl;
};
__device__ __forceinline__ bool ctl_wait(int ctl) { return ctl & 1; }
__device__ __forceinline__ int ctl_base(int ctl) { return (ctl >> 1) & 7; }
__device__ __forceinline__ int ctl_gate(int ctl) { return (ctl >> 8) & 0xff; }
constexpr int kChainSlots = 8;
constexpr int kChainMax = Q4_GEMV_CHAIN_MAX;
struct ChainArgs {
    ChainTask t[kChainMax];
    int ntasks;
    int gshift;
    // [0] barrier arrivals and [1] finished workgroups (zero on entry, left
    // zero on exit); [2] set to 1 when a barrier wait ran out
    uint32_t *sync;
};
constexpr uint32_t kSpinLimit = 1u << 20;  // bounded waits (of the order of a second)
constexpr int kChainMaxK = 16384;  // 4 stages: a task and the next fit the 8 slots

// A wave's position in the chain: task, row and stage along K; whether the
// stage is the row's last, where the row's output goes and the task's first
// x slot.
struct CPos {
    int t, row, s;
    bool last;
    uint16_t *yp;
    int xbase;
};

__host__ __device__ __forceinline__ int chain_stages(int K) { return ((K >> 5) + kStageChunks - 1) / kStageChunks; }

// The views of one task for the chained kernel: whole arrays (each under
// 2 GiB, checked on the host), with a row's and a stage's place added as a
// wave-uniform offset, so that moving to the next row costs a few scalar
// instructions and no reload of the task's arguments.  Lanes whose chunk is
// past the row end are sent past the view by kChainOob.
struct TaskViews {
    __amdgpu_buffer_rsrc_t codes, scales, zeros;
    const float *s2;  // double quantization: the second-level constants
    uint16_t *y;
    int N, S, C, row_bytes, G, xbase;
};
constexpr uint32_t kChainOob = 0x80000000u;

template <int FMT>
__device__ __forceinline__ TaskViews task_views(const ChainTask &T, int gshift)
{
    constexpr int ss = FMT == Q4_NF4 ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);
    TaskViews v;
    v.N = T.N;
    v.row_bytes = T.K >> 1;
    v.G = T.K >> gshift;
    v.C = T.K >> 5;
    v.S = chain_stages(T.K);
    v.codes = make_rsrc(T.codes, (int64_t)v.N * v.row_bytes);
    v.scales = make_rsrc(T.scales, (int64_t)v.N * v.G * ss);
    v.zeros = FMT == Q4_INT4_ASYM ? make_rsrc(T.zeros, ((int64_t)v.N * v.G + 1) / 2) : v.codes;
    v.s2 = (const float *)T.zeros;
    v.y = T.y;
    v.xbase = ctl_base(T.ctl);
    return v;
}

// The loads of stage s of row `row` (row == N: past the last row, every load
// is out of the views and returns zero), as load_stage does with row views.
template <int FMT>
__device__ __forceinline__ void load_stage_chain(Stage &st, const TaskViews &tv, int row, int s,
                                                 int lane, int gshift)
{
    constexpr int ss = FMT == Q4_NF4 ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);
    const int g0 = row * tv.G;                                // the row's first flat group
    const int gs = (kStageChunks * 32 * s) >> gshift;          // the stage's first group in the row
    const int cd_off = row * tv.row_bytes + 16 * kStageChunks * s;
    const int sc_off = (g0 + gs) * ss;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int lc = 64 * h + lane;                         // chunk within the stage
        const bool in = kStageChunks * s + lc < tv.C;
        st.cw[h] = __builtin_amdgcn_raw_buffer_load_b128(tv.codes, in ? 16 * lc : kChainOob, cd_off,
                                                         kNT);
        const int gl = (32 * lc) >> gshift;                    // group within the stage
        if constexpr (FMT == Q4_NF4)
            st.sc[h] = std::bit_cast<float>(
                __builtin_amdgcn_raw_buffer_load_b32(tv.scales, in ? 4 * gl : kChainOob, sc_off, kNT));
        else if constexpr (FMT == Q4_NF4_DQ)
            st.sc[h] = std::bit_cast<float>((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(
                tv.scales, in ? gl : kChainOob, sc_off, kNT));
        else
            st.sc[h] = h2f(
                __builtin_amdgcn_raw_buffer_load_b16(tv.scales, in ? 2 * gl : kChainOob, sc_off, kNT));
        if constexpr (FMT == Q4_INT4_ASYM) {
            // nibble g0 + gs + gl; gs is even, so the byte is
            // (g0 >> 1) + gs / 2 + ((g0 & 1) + gl) / 2
            const int gz = (g0 & 1) + gl;
            const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(
                tv.zeros, in ? gz >> 1 : kChainOob, (g0 >> 1) + (gs >> 1), kNT);
            st.zf[h] = (float)((b >> ((gz & 1) * 4)) & 0xf);
        } else {
            st.zf[h] = 0.0f;
        }
    }
    if constexpr (FMT == Q4_NF4_DQ) {
        // the constants of the row's runs, as load_stage reads them (a row
        // past the end reads the first ones, never used)
        typedef float f32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
        const float *p = tv.s2 + (row < tv.N ? (g0 >> 8) : 0);
        const f32x4a4 c = *(const __attribute__((address_space(4))) f32x4a4 *)p;
        st.s2[0] = c[0];
        st.s2[1] = c[1];
        st.s2[2] = c[2];
        st.zpar = g0 & (kDqRun - 1);
    }
}

// s_waitcnt on vector memory only (expcnt and lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vm()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// x of a chained task in LDS: stage s in slot (base + s) mod 8, piece-major
// within the stage (piece j of its local chunk c at 16-byte index
// 128 j + c of the slot), so that the 16 lanes of a read pass take 256
// consecutive bytes (no bank conflicts); the inverse scales of stage s at
// float index 128 slot + c.
__device__ __forceinline__ int chain_slot(int base, int s) { return (base + s) & (kChainSlots - 1); }
__device__ __forceinline__ int chain_x_index(int slot, int j, int c) { return 512 * slot + 128 * j + c; }

// A lane's x slice for stage s of a row: chunks l and 64 + l of the stage
// (the stored rows are zero past K up to whole stages), with the inverse
// scales of their conversion.
__device__ __forceinline__ void chain_x_slice(u32x4 (&xreg)[8], float (&xinv)[2], const u32x4 *xb,
                                              const float *inv, int base, int s, int lane)
{
    const int slot = chain_slot(base, s);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xreg[4 * h + j] = xb[chain_x_index(slot, j, 64 * h + lane)];
        xinv[h] = inv[kStageChunks * slot + 64 * h + lane];
    }
}

// A task's descriptor from the table's copy in LDS, in scalar registers.
__device__ __forceinline__ ChainTask lds_task(const ChainTask *tasks, int t)
{
    constexpr int W = sizeof(ChainTask) / 4;
    const uint32_t *p = reinterpret_cast<const uint32_t *>(tasks + t);
    uint32_t w[W];
#pragma unroll
    for (int i = 0; i < W; ++i)
        w[i] = __builtin_amdgcn_readfirstlane(p[i]);
    ChainTask T;
    __builtin_memcpy(&T, w, sizeof(T));
    return T;
}

// x DMA instructions per stage: 2 halves of 64 chunks, 4 pieces each.
constexpr int kChainDmaPerStage = 8;
// x DMA instructions of later tasks the loader keeps in flight at most (a
// multiple of kChainDmaPerStage, within the vector-memory counter's range).
constexpr int kChainDmaAhead = 40;

// The loader's copy of x[0, K) of a task into the task's slots, by the
// buffer unit straight into LDS (no registers, so the loader can have
// several tasks in flight): per stage, half and piece, one 16-byte load per
// lane, lane l's piece j of chunk c0 + l landing at 16-byte index
// 128 j + c0 + l of the slot, the piece-major order the compute waves read.
// Chunks past K read zeros: the stored rows are padded to whole stages.
__device__ __forceinline__ void chain_dma_x(const ChainTask &T, u32x4 *xb, int lane)
{
    const __amdgpu_buffer_rsrc_t xr = make_rsrc(T.x, (int64_t)T.K * 2);
    const int S = chain_stages(T.K);
    const int base = ctl_base(T.ctl);
    for (int s = 0; s < S; ++s) {
        const int slot = chain_slot(base, s);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    xr, (__attribute__((address_space(3))) void *)(xb + chain_x_index(slot, j, 64 * h)),
                    16, 64 * lane, 64 * (kStageChunks * s + 64 * h) + 16 * j, 0, 0);
    }
}

// Once a task's x is in its slots: converted in place where the arithmetic
// uses fp16 for bf16 activations (per 32-value chunk, max |x| scaled into
// [2^14, 2^15) by a power of two: the staged single-product conversion);
// inv receives the chunks' inverse scales (1 when nothing is converted).
template <int FMT, int ACT>
__device__ __forceinline__ void chain_convert_x(const ChainTask &T, u32x4 *xb, float *inv, int lane)
{
    using F = Cfg<FMT, ACT, X_LDS>;
    const int S = chain_stages(T.K);
    const int base = ctl_base(T.ctl);
    for (int s = 0; s < S; ++s) {
        const int slot = chain_slot(base, s);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int c = 64 * h + lane;
            float iv = 1.0f;
            if constexpr (F::conv_x) {
                u32x4 v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = xb[chain_x_index(slot, j, c)];
                float mx = 0.0f;
#pragma unroll
                for (int j = 0; j < 4; ++j)
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        mx = fmaxf(mx, bf2_absmax(v[j][k]));
                float f;
                x_scale(mx, f, iv);
#pragma unroll
                for (int j = 0; j < 4; ++j) {
#pragma unroll
                    for (int k = 0; k < 4; ++k)
                        v[j][k] = bf2_to_h2(v[j][k], f);
                    xb[chain_x_index(slot, j, c)] = v[j];
                }
            }
            inv[kStageChunks * slot + c] = iv;
        }
    }
}

// Waits until at most n vector-memory instructions (a multiple of
// kChainDmaPerStage, at most kChainDmaAhead) are in flight.
__device__ __forceinline__ void wait_vm_upto(int n)
{
    static_assert(kChainDmaAhead == 40 && kChainDmaPerStage == 8, "bins below");
    if (n >= 40)
        wait_vm<40>();
    else if (n >= 32)
        wait_vm<32>();
    else if (n >= 24)
        wait_vm<24>();
    else if (n >= 16)
        wait_vm<16>();
    else if (n >= 8)
        wait_vm<8>();
    else
        wait_vm<0>();
}

constexpr int kChainCompute = 15;  // compute waves per workgroup (wave 15 loads x)

// DEP: some task waits for earlier outputs (else the grid-barrier code is
// left out).
template <int FMT, int ACT, int P, bool DEP>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_chain_kernel(const ChainArgs a)
{
    using F = Cfg<FMT, ACT, X_LDS>;  // the arithmetic of the staged single-product kernels
    static_assert(Cfg<FMT, ACT, X_REG>::ct == F::ct && Cfg<FMT, ACT, X_REG>::pair == F::pair,
                  "x source must not change the arithmetic");
    // One LDS block with the table first, at address 0, so that a lookup's
    // address is the v_perm result itself.
    struct Lds {
        uint32_t tbl[kTableDwords];
        u32x4 xb[kChainSlots * 512];
        float xinv[kChainSlots * kStageChunks];
        int entered[kChainMax];  // compute waves that entered each task
        int ready[kChainMax];    // 1 once x of the task is in its slots
        ChainTask tasks[kChainMax];
    };
    __shared__ Lds lds;
    uint32_t *const tbl = lds.tbl;
    auto &xb = lds.xb;
    auto &xinv_lds = lds.xinv;
    auto &entered = lds.entered;
    auto &ready = lds.ready;

    const int lane = threadIdx.x & 63;
    const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t laneoff = (uint32_t)(F::pair ? (lane & 31) : lane) << 2;
    const int nt = a.ntasks;
    // every compute wave has entered task t
    auto all_entered = [&](int t) {
        return __hip_atomic_load(&entered[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >=
               kChainCompute;
    };
    auto fail = [&]() { __hip_atomic_store(&a.sync[2], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT); };

    // the level table, by every wave
    {
        uint32_t part_lo = 0, part_hi = 0;
        if constexpr (level_fmt(FMT) == Q4_NF4) {
            part_lo = c_parts[F::pair ? 0 : 2][lane & 15];
            if constexpr (F::pair)
                part_hi = c_parts[1][lane & 15];
        }
#pragma unroll
        for (int i = 0; i < kTableDwords / 4 / 1024; ++i) {
            const int piece = threadIdx.x + 1024 * i;
            const int e = piece >> 4, h = (piece >> 3) & 1;
            const int n0 = e & 15, n1 = e >> 4;
            uint32_t v;
            if constexpr (level_fmt(FMT) == Q4_NF4) {
                uint32_t x0 = (uint32_t)__shfl((int)part_lo, n0), x1 = (uint32_t)__shfl((int)part_lo, n1);
                if constexpr (F::pair) {
                    const uint32_t c0 = (uint32_t)__shfl((int)part_hi, n0);
                    const uint32_t c1 = (uint32_t)__shfl((int)part_hi, n1);
                    if (h) {
                        x0 = c0;
                        x1 = c1;
                    }
                }
                v = x0 | (x1 << 16);
            } else {
                const int off = FMT == Q4_INT4_SYM ? 8 : 0;
                v = level_bits<F::ct>(n0 - off) | (level_bits<F::ct>(n1 - off) << 16);
            }
            ((u32x4 *)tbl)[piece] = u32x4{v, v, v, v};
        }
    }
    // the task table into LDS, read there at every task switch: through the
    // scalar cache, a miss would stall the wave (and the loads of its next
    // rows) for a loaded memory system's latency once per task
    {
        constexpr int W = sizeof(ChainTask) / 4;
        const uint32_t *src = reinterpret_cast<const uint32_t *>(&a.t[0]);
        uint32_t *dst = reinterpret_cast<uint32_t *>(lds.tasks);
        static_assert(kChainMax * W <= 1024, "one word per thread");
        if ((int)threadIdx.x < nt * W)
            dst[threadIdx.x] = src[threadIdx.x];
    }
    __syncthreads();
    auto task = [&](int t) { return lds_task(lds.tasks, t); };

    // The rows this workgroup works on.  With no task waiting for earlier
    // outputs, each workgroup takes one contiguous block of the tasks' rows
    // laid end to end, [(tlo, rlo), (tend, rend)), balanced by stage count:
    // a wave then meets a new task once or twice per launch rather than at
    // almost every row of a short task (each switch reads the task's
    // descriptor and x slice and waits for its x, inside the ring).  A chain
    // with waits keeps the walk of every task over all waves, since the
    // whole grid finishes a task before a waiting one starts.
    int tlo = 0, rlo = 0, tend = nt, rend = 0;
    if constexpr (!DEP) {
        // first row whose start (in stages, rows laid end to end) is at or
        // after `target`
        auto locate = [&](int64_t target, int &u, int &r) {
            int64_t acc = 0;
            for (u = 0; u < nt; ++u) {
                const ChainTask U = task(u);
                const int S = chain_stages(U.K);
                const int64_t span = (int64_t)U.N * S;
                if (target < acc + span) {
                    const int64_t rr = (target - acc + S - 1) / S;
                    if (rr < U.N) {
                        r = (int)rr;
                    } else {
                        r = 0;
                        ++u;
                    }
                    return;
                }
                acc += span;
            }
            u = nt;
            r = 0;
        };
        int64_t total = 0;
        for (int u = 0; u < nt; ++u) {
            const ChainTask U = task(u);
            total += (int64_t)U.N * chain_stages(U.K);
        }
        locate(total * blockIdx.x / gridDim.x, tlo, rlo);
        locate(total * (blockIdx.x + 1) / gridDim.x, tend, rend);
    }
    const bool has_rows = tlo < tend || (tlo == tend && rlo < rend);
    // the tasks this workgroup loads and enters: tlo .. thi
    const int thi = !has_rows ? tlo - 1 : (rend == 0 ? tend - 1 : tend);

    if (wave == kChainCompute) {
        // ---------------------------------------------------------- loader
        // x goes in by DMA as early as the slots allow: a later task's as
        // soon as its gate is open (unless it reads earlier outputs), up to
        // kChainDmaAhead instructions ahead; the current task's is then
        // awaited, converted and published.
        int issued = 0;  // tasks whose x DMA is issued (in order)
        int ahead = 0;   // DMA instructions in flight for tasks after the current one
        auto dma_count = [&](const ChainTask &T) { return kChainDmaPerStage * chain_stages(T.K); };
        auto issue_ahead = [&]() {
            while (issued <= thi) {
                const ChainTask T = task(issued);
                const int n = dma_count(T);
                if ((DEP && ctl_wait(T.ctl)) || ahead + n > kChainDmaAhead || !all_entered(ctl_gate(T.ctl)))
                    break;
                chain_dma_x(T, xb, lane);
                ahead += n;
                ++issued;
            }
        };
        auto publish = [&](int t) {
            wait_vm_upto(ahead);  // task t's DMA is done (they complete in order)
            chain_convert_x<FMT, ACT>(task(t), xb, xinv_lds, lane);
            __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): x is in LDS
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __hip_atomic_store(&ready[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        // task tlo is entered by every compute wave in the prologue; the
        // tasks before it are never entered here (they count as entered,
        // for the gates of the slots they would have used)
        entered[lane] = lane <= tlo ? kChainCompute : 0;
        ready[lane] = 0;
        issued = tlo;
        if (has_rows) {
            chain_dma_x(task(tlo), xb, lane);
            issued = tlo + 1;
            issue_ahead();
            publish(tlo);
        }
        __syncthreads();  // the table, the counters and x of task tlo
        int nbar = 0;
        for (int t = tlo + 1; t <= thi; ++t) {
            const ChainTask T = task(t);
            if (issued > t) {
                ahead -= dma_count(T);  // in flight already: now the current task
            } else {
                // the slots of task t last held x of an earlier task: wait
                // until every compute wave has entered the task after it
                // (the gate); a task that reads earlier outputs waits until
                // they have finished t - 1 (entered t, stores complete).
                // Nothing is in flight here.
                const bool wait = DEP && ctl_wait(T.ctl);
                const int need = wait ? t : ctl_gate(T.ctl);
                uint32_t spins = 0;
                while (!all_entered(need)) {
                    if (++spins == kSpinLimit) {
                        fail();
                        break;
                    }
                    __builtin_amdgcn_s_sleep(1);
                }
                if (wait) {
                    // grid barrier between the loaders: this workgroup's
                    // outputs are released with the arrival, the others'
                    // acquired after it
                    ++nbar;
                    if (lane == 0) {
                        __hip_atomic_fetch_add(&a.sync[0], 1u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
                        const uint32_t target = (uint32_t)nbar * gridDim.x;
                        uint32_t gspins = 0;
                        while (__hip_atomic_load(&a.sync[0], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) <
                               target) {
                            if (++gspins == kSpinLimit) {
                                fail();
                                break;
                            }
                            __builtin_amdgcn_s_sleep(1);
                        }
                    }
                    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
                }
                chain_dma_x(T, xb, lane);
                issued = t + 1;
            }
            issue_ahead();
            publish(t);
        }
    } else {
        // ---------------------------------------------------------- compute
        // vector-memory instructions per ring refill
        const int wave_id = (int)__builtin_amdgcn_readfirstlane(blockIdx.x * kChainCompute + wave);
        const int total_waves = gridDim.x * kChainCompute;
        // A wave's walk: its rows in order and each row's stages.  With no
        // waiting task, the rows are those of the workgroup's block, dealt
        // to its waves in turn.  Otherwise the walk goes task by task: task
        // t's rows are dealt to all the grid's waves from a rotated start,
        // so that the waves holding one row more than the others differ
        // from task to task.
        // tv: the views of the newest position's task (positions are made
        // and loaded in order, so the newest is always the one loaded)
        TaskViews tv = task_views<FMT>(task(tlo < nt ? tlo : 0), a.gshift);
        // a position past this wave's rows: a row past the end of the
        // current views
        auto past = [&]() { return CPos{nt, tv.N, 0, false, tv.y, 0}; };
        // blocked walk: wave w takes rows w, w + 15, ... of the block
        auto in_block = [&](int u, int r) { return u < tend || (u == tend && r < rend); };
        auto block_pos = [&](int u, int r) {
            // row r of task u, or the first row after it when r >= N_u
            while (u < nt) {
                const int n = task(u).N;
                if (r < n)
                    break;
                r -= n;
                ++u;
            }
            if (!in_block(u, r))
                return past();
            tv = task_views<FMT>(task(u), a.gshift);
            return CPos{u, r, 0, tv.S == 1, tv.y + r, tv.xbase};
        };
        auto first_pos = [&](int t) {
            if constexpr (!DEP)
                return has_rows ? block_pos(tlo, rlo + wave) : past();
            for (; t < nt; ++t) {
                const int e =
                    (int)(((uint32_t)wave_id + (uint32_t)t * 1237u) % (uint32_t)total_waves);
                const ChainTask T = task(t);
                if (e < T.N) {
                    tv = task_views<FMT>(T, a.gshift);
                    return CPos{t, e, 0, tv.S == 1, tv.y + e, tv.xbase};
                }
            }
            // past the last task: a row past the end of the last views
            return past();
        };
        auto advance = [&](CPos q) {
            if (q.t >= nt)
                return q;
            if (++q.s == tv.S) {
                q.s = 0;
                if constexpr (!DEP) {
                    const int r = q.row + kChainCompute;
                    if (r >= tv.N || !in_block(q.t, r))
                        return block_pos(q.t, r);
                    q.row = r;
                    q.yp += kChainCompute;
                } else {
                    q.row += total_waves;
                    q.yp += total_waves;
                    if (q.row >= tv.N)
                        return first_pos(q.t + 1);
                }
            }
            q.last = q.s == tv.S - 1;
            return q;
        };
        // Refills are issued unconditionally (past the last task with every
        // load out of the views: they return zeros) so that the number of
        // loads in flight is the same on every path and the waits stay
        // partial.
        auto load_pos = [&](Stage &st, CPos q) {
            load_stage_chain<FMT>(st, tv, q.row, q.s, lane, a.gshift);
        };
        CPos pos[P];
        Stage st[P];
        pos[0] = first_pos(0);
#pragma unroll
        for (int q = 0; q < P; ++q) {
            if (q > 0)
                pos[q] = advance(pos[q - 1]);
            st[q] = Stage{};
            load_pos(st[q], pos[q]);
        }
        __syncthreads();  // the table, the counters and x of task tlo
        int cur = tlo;
        // Entering task cur + 1: count in, then wait for its x.  Before a
        // task that reads earlier outputs, this wave's own stores complete
        // first (the loader releases them to the grid).
        auto enter = [&]() {
            const int t = ++cur;
            if (DEP && ctl_wait(task(t).ctl))
                wait_vm<0>();
            if (lane == 0)
                __hip_atomic_fetch_add(&entered[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            uint32_t spins = 0;
            while (__hip_atomic_load(&ready[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) != 1) {
                if (++spins == kSpinLimit) {
                    fail();
                    break;
                }
                __builtin_amdgcn_s_sleep(1);
            }
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
        };

        // The ring: position q is computed while the next ones arrive, then
        // its slot is refilled with the position P ahead.  A position of a
        // later task first enters that task (and any task between without
        // rows for this wave).  Each lane keeps its x slice (chunks l and
        // 64 + l of the position's stage) in registers, read from LDS when
        // the task or the stage changes.
        //
        // A round of the ring is never left in the middle (the load waits
        // stay partial only if every path refills every slot): a position
        // past the last task has loaded zeros from an empty view; it is
        // computed on them and writes nothing.
        u32x4 xreg[8];
        float xinv_reg[2] = {1.0f, 1.0f};
        int xkey = -1;
        float acc[1] = {0.0f};
        while (pos[0].t < nt) {
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const CPos cp = pos[q];
                const bool live = cp.t < nt;
                if (live) {
                    while (cur < cp.t)
                        enter();
                }
                const int key = 8 * cp.t + cp.s;
                if (key != xkey) {
                    chain_x_slice(xreg, xinv_reg, xb, xinv_lds, cp.xbase, cp.s, lane);
                    xkey = key;
                }
                const float xinv[1][2] = {{xinv_reg[0], xinv_reg[1]}};
                // (x comes from registers: no x view, K or chunk count needed)
                compute_stage<FMT, F::ct, F::pair, 1, X_REG>(st[q], acc, tbl, nullptr, xreg, xinv,
                                                           make_rsrc(nullptr, 0), 0, 0, cp.s, lane,
                                                           0, laneoff, a.gshift);
                if (cp.last) {
                    const float out = wave_sum(acc[0]);
                    acc[0] = 0.0f;
                    if (live && lane == 0)
                        // through a global (not flat) pointer: a flat store may
                        // write LDS, so LDS reads after it would wait for it
                        *(__attribute__((address_space(1))) uint16_t *)cp.yp =
                            (uint16_t)(ACT == Q4_BF16 ? f2bf_bits(out) : f2h_bits(out));
                }
                pos[q] = advance(pos[(q + P - 1) % P]);
                load_pos(st[q], pos[q]);
            }
        }
        // waves with no rows in the last tasks still count into them
        while (cur < thi)
            enter();
    }
    wait_vm<0>();  // no LDS DMA may be in flight when the workgroup ends
    __syncthreads();
    if (threadIdx.x == 0) {
        // the last workgroup to finish leaves the counters at zero for the
        // next chain on this sync buffer (every workgroup is past its last
        // barrier by then)
        const uint32_t d =
            __hip_atomic_fetch_add(&a.sync[1], 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
        if (d == gridDim.x - 1) {
            __hip_atomic_store(&a.sync[0], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            __hip_atomic_store(&a.sync[1], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
    }
}

// Staged activations fit when M rows of whole stages, skewed, fit the region
// (the last 16-byte piece ends at xpad(bytes - 16) + 16).
bool x_fits_lds(int64_t M, int64_t K)
{
    const int64_t C = K / 32;
    const int64_t S = (C + kStageChunks - 1) / kStageChunks;
    const int64_t bytes = M * S * kStageXBytes;
    return bytes - 16 + ((bytes - 16) >> 6 << 4) + 16 <= kXBytes;
}

template <int FMT, int ACT, int MT, int XS>
hipError_t launch_one(const void *x, int M, const uint8_t *codes, const void *scales,
                      const uint8_t *zeros, int64_t N, int64_t K, int gshift, void *y,
                      hipStream_t s)
{
    constexpr int waves = Shape<XS>::waves;
    int64_t blocks = (N + waves - 1) / waves;
    const int64_t cap = (int64_t)device_cu_count() * Shape<XS>::per_cu;
    if (blocks > cap)
        blocks = cap;
    constexpr int depth = MT <= 2 ? Q4_GEMV_DEPTH : 2;
    // double-quantized absmax: the kernel takes the constants' base in
    // place of the (absent) zero-points
    if constexpr (FMT == Q4_NF4_DQ)
        zeros = (const uint8_t *)scales + dq_s2_offset(N * (K >> gshift));
    hipLaunchKernelGGL((gemv_kernel<FMT, ACT, MT, XS, depth>), dim3((unsigned)blocks),
                       dim3(Shape<XS>::block), 0, s, (const uint16_t *)x, M, codes, scales, zeros,
                       (int)N, (int)K, gshift, (uint16_t *)y);
    return hipGetLastError();
}

template <int FMT, int ACT>
hipError_t launch_m(const void *x, int M, const uint8_t *codes, const void *scales,
                    const uint8_t *zeros, int64_t N, int64_t K, int gshift, void *y, hipStream_t s)
{
    // M = 1 with one stage per row: activations live in registers; else
    // staged in LDS when they fit; else read from L2 (M <= 2 here)
    const bool one_stage = K <= 32 * kStageChunks;
    const bool xl = x_fits_lds(M <= 1 ? 1 : 2, K);
#define Q4_GEMV_LAUNCH(MT_, XS_) \
    launch_one<FMT, ACT, MT_, XS_>(x, M, codes, scales, zeros, N, K, gshift, y, s)
    if (M <= 1)
        return one_stage ? Q4_GEMV_LAUNCH(1, X_REG)
                         : (xl ? Q4_GEMV_LAUNCH(1, X_LDS) : Q4_GEMV_LAUNCH(1, X_GLOBAL));
    return xl ? Q4_GEMV_LAUNCH(2, X_LDS) : Q4_GEMV_LAUNCH(2, X_GLOBAL);
#undef Q4_GEMV_LAUNCH
}

template <int FMT>
hipError_t launch_act(q4_dtype act_t, const void *x, int M, const uint8_t *codes,
                      const void *scales, const uint8_t *zeros, int64_t N, int64_t K, int gshift,
                      void *y, hipStream_t s)
{
    if (act_t == Q4_BF16)
        return launch_m<FMT, Q4_BF16>(x, M, codes, scales, zeros, N, K, gshift, y, s);
    return launch_m<FMT, Q4_F16>(x, M, codes, scales, zeros, N, K, gshift, y, s);
}

template <int FMT, int ACT>
hipError_t launch_chain_t(const ChainArgs &args, hipStream_t s)
{
    constexpr int depth = Q4_GEMV_CHAIN_DEPTH;
    const int cus = device_cu_count();
    if (cus <= 0)
        return hipErrorInvalidDevice;
    bool dep = false;
    for (int i = 1; i < args.ntasks; ++i)
        dep = dep || (args.t[i].ctl & 1);
    void *kargs[] = {const_cast<ChainArgs *>(&args)};
    // Only the grid barrier of a waiting task needs every workgroup resident
    // at once (a cooperative launch); without one no workgroup ever waits
    // for another, and a plain launch saves the cooperative one's extra
    // dispatch cost (measured: 10-15 us per launch).
    if (!dep)
        return hipLaunchKernel((const void *)gemv_chain_kernel<FMT, ACT, depth, false>, dim3(cus),
                               dim3(1024), kargs, 0, s);
    return hipLaunchCooperativeKernel((const void *)gemv_chain_kernel<FMT, ACT, depth, true>,
                                      dim3(cus), dim3(1024), kargs, 0, s);
}

}  // namespace

bool gemv_chain_k_ok(int64_t K) { return K <= kChainMaxK; }

hipError_t launch_gemv_chain(q4_format f, int g, q4_dtype act_t, const q4_gemv_task *tasks,
                             int ntasks, uint32_t *sync, hipStream_t s)
{
    ChainArgs a = {};
    a.gshift = g == 32 ? 5 : (g == 64 ? 6 : 7);
    int base = 0, last_user[kChainSlots];
    for (int sl = 0; sl < kChainSlots; ++sl)
        last_user[sl] = -1;
    for (int i = 0; i < ntasks; ++i) {
        // double-quantized absmax: the constants' base in place of zeros
        const uint8_t *z = f == Q4_NF4_DQ ? (const uint8_t *)tasks[i].scales +
                                                dq_s2_offset(tasks[i].N * (tasks[i].K >> a.gshift))
                                          : tasks[i].zeros;
        // x slots: task i's stages take consecutive slots (mod 8) after task
        // i - 1's; the gate is the task after the last one that used any of
        // them (every task has at most 4 stages, so that is at most i - 1)
        const int S = chain_stages((int)tasks[i].K);
        int last = -1;
        for (int st = 0; st < S; ++st) {
            const int sl = (base + st) % kChainSlots;
            last = last_user[sl] > last ? last_user[sl] : last;
            last_user[sl] = i;
        }
        const int ctl = ((tasks[i].flags & Q4_TASK_NO_WAIT) ? 0 : 1) | (base << 1) | ((last + 1) << 8);
        base = (base + S) % kChainSlots;
        a.t[i] = ChainTask{(const uint16_t *)tasks[i].x, tasks[i].codes, tasks[i].scales, z,
                           (uint16_t *)tasks[i].y, (int)tasks[i].N, (int)tasks[i].K, ctl};
    }
    a.ntasks = ntasks;
    a.sync = sync;
    const bool bf = act_t == Q4_BF16;
    switch (f) {
    case Q4_NF4:
        return bf ? launch_chain_t<Q4_NF4, Q4_BF16>(a, s) : launch_chain_t<Q4_NF4, Q4_F16>(a, s);
    case Q4_NF4_DQ:
        return bf ? launch_chain_t<Q4_NF4_DQ, Q4_BF16>(a, s)
                  : launch_chain_t<Q4_NF4_DQ, Q4_F16>(a, s);
    case Q4_INT4_SYM:
        return bf ? launch_chain_t<Q4_INT4_SYM, Q4_BF16>(a, s)
                  : launch_chain_t<Q4_INT4_SYM, Q4_F16>(a, s);
    default:
        return bf ? launch_chain_t<Q4_INT4_ASYM, Q4_BF16>(a, s)
                  : launch_chain_t<Q4_INT4_ASYM, Q4_F16>(a, s);
    }
}

hipError_t launch_gemv(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                       const uint8_t *codes, const void *scales, const uint8_t *zeros, int64_t N,
                       int64_t K, void *y, hipStream_t s)
{
    // three or more activation rows: the skinny matrix-core product
    if (M >= 3)
        return launch_gemv_mfma(f, g, act_t, x, M, codes, scales, zeros, N, K, y, s);
    const int gshift = g == 32 ? 5 : (g == 64 ? 6 : 7);
    switch (f) {
    case Q4_NF4:
        return launch_act<Q4_NF4>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    case Q4_NF4_DQ:
        return launch_act<Q4_NF4_DQ>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    case Q4_INT4_SYM:
        return launch_act<Q4_INT4_SYM>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    default:
        return launch_act<Q4_INT4_ASYM>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    }
}

}  // namespace q4
