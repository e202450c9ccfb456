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
//  * Every weight enters the product as the value q4_dequantize writes: the
//    binary32 product level * scale (NF4: Q[i] * c; INT4-sym: (q - 8) * s;
//    INT4-asym: q * s + (-z * s), both terms exact), rounded once to the
//    activation dtype.  The levels come from a per-workgroup LDS table
//    indexed by a whole code byte: an entry holds the binary32 levels of its
//    two nibbles, so one 8-byte read, two fma and one packed conversion give
//    a pair of 16-bit weights.  The table is replicated per 32 lane slots (a
//    lane reads only its own banks) and a byte's LDS address is one
//    v_perm_b32 (code byte -> address bits 8..15, lane slot -> bits 3..7).
//  * Multiply-accumulate on the vector ALUs in binary32: v_dot2_f32_bf16 /
//    v_dot2_f32_f16 multiply a pair of 16-bit weights by a pair of 16-bit
//    activations (both products exact in binary32) and add them to a
//    binary32 accumulator.  Each activation row keeps two accumulators that
//    take alternate weight pairs, so consecutive dot2 do not wait on each
//    other.  (A lane-own form on the 4 x 4 x 4
//    matrix-core blocks, which takes the dot products off the vector ALUs,
//    measured the same speed on the decode token: 4503 against 4505 GB/s.)
//  * Activations: for M = 1 and rows that fit one stage (K <= 4096) each lane
//    keeps its slices in registers; else, for M <= 2, they are staged once
//    per workgroup in LDS (rows padded to whole stages with zeros, 16 bytes
//    of skew per 64-byte chunk so the 16-byte reads of a wave do not collide
//    in banks); larger K reads them from L2 step by step.
//  * At the end of a row each lane's two accumulators are added and summed
//    across the wave with DPP; y is rounded once to the activation dtype.
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

// The byte-indexed level table: entry e (a code byte), lane slot L (0..31)
// at byte 256 e + 8 L holds the binary32 levels of the byte's low and high
// nibble.  Lanes L and L + 32 read the same slot, in different halves of
// the wave's 8-byte read, so no read meets a bank conflict.  It is filled
// in 16-byte pieces (two slots of one entry): thread t writes pieces t,
// t + BLOCK, ..., so each store instruction covers consecutive addresses.
constexpr int kTablePieces = kTableDwords / 4;

// Binary32 level of nibble i: the NF4 table entry, i - 8 (INT4-sym, offset
// binary) or i (INT4-asym, whose zero-point enters as the bias -z * s).
// NF4 entries come from a per-lane constant (lane i % 16 holds entry i,
// built from immediates) by lane permute, so filling the table issues no
// memory load (which would queue behind the weight loads in flight).
template <int FMT>
__device__ __forceinline__ float nf4_lane_entry()
{
    const int i = threadIdx.x & 15;
    float v = level_entry<FMT>(0);
#pragma unroll
    for (int k = 1; k < 16; ++k)
        v = i == k ? level_entry<FMT>(k) : v;
    return v;
}
template <int FMT>
__device__ __forceinline__ float level_of(int i, float lane_entry)
{
    if constexpr (level_fmt(FMT) == Q4_NF4)
        return std::bit_cast<float>(__shfl(std::bit_cast<int>(lane_entry), i, 16));
    else
        return (float)(FMT == Q4_INT4_SYM ? i - 8 : i);
}

// Fill the table: `block` threads, thread t writes pieces t, t + block, ...
// Piece p holds entry p >> 4, so thread t's pieces share the entry's low
// nibble ((t >> 4) & 15: block is a multiple of 256) and their high nibbles
// ((t >> 8) + i block / 256) are the same across the wave: one lane
// permute for the low level, a read of one lane for each high level.
template <int FMT, int BLOCK>
__device__ __forceinline__ void fill_level_table(uint32_t *tbl)
{
    static_assert(kTablePieces % BLOCK == 0 && BLOCK % 256 == 0, "whole rounds of pieces");
    const float mine = level_fmt(FMT) == Q4_NF4 ? nf4_lane_entry<FMT>() : 0.0f;
    const uint32_t lo = std::bit_cast<uint32_t>(level_of<FMT>((threadIdx.x >> 4) & 15, mine));
    const int h0 = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 8);
#pragma unroll
    for (int i = 0; i < kTablePieces / BLOCK; ++i) {
        const int hn = h0 + (BLOCK >> 8) * i;  // wave-uniform
        uint32_t hi;
        if constexpr (level_fmt(FMT) == Q4_NF4)
            hi = (uint32_t)__builtin_amdgcn_readlane(std::bit_cast<int>(mine), hn);
        else
            hi = std::bit_cast<uint32_t>((float)(FMT == Q4_INT4_SYM ? hn - 8 : hn));
        ((u32x4 *)tbl)[threadIdx.x + BLOCK * i] = u32x4{lo, hi, lo, hi};
    }
}

// Scale and bias of a chunk's group: weight = fma(level, s, b).  The bias
// is -0 where there is no zero-point, so fma(level, s, -0) is the plain
// product level * s (sign of zero included).
template <int FMT>
__device__ __forceinline__ float chunk_bias(float s, float zf)
{
    if constexpr (FMT == Q4_INT4_ASYM)
        return -(zf * s);  // exact: z <= 15 and s has 11 significant bits
    else
        return -0.0f;
}

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

// One weight row: where its codes, scales and zero-points start (row `live`
// false: past the last row, every load reads zero).  With double-quantized
// absmax, `scales` points at the row's 8-bit absmax codes and s2 at the
// second-level constant of the run holding the row's first group (the
// kernels receive the constants' base in place of `zeros`).
struct RowRef {
    const uint8_t *codes;
    const char *scales;
    const uint8_t *zeros;  // asym: the byte holding the row's first zero-point nibble
    const float *s2;
    int zpar;  // parity of the row's first flat group index (asym), or its
               // position in its run of kDqRun groups (double quantization)
    bool live;
};

template <int FMT>
__device__ __forceinline__ RowRef row_ref(const uint8_t *codes, const void *scales,
                                          const uint8_t *zeros, int64_t n0, int64_t N,
                                          int64_t row_bytes, int64_t G)
{
    constexpr int ss = f32_absmax(FMT) ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);
    RowRef r;
    r.live = n0 < N;
    r.codes = codes + n0 * row_bytes;
    r.scales = (const char *)scales + n0 * G * ss;
    const uint64_t g0 = (uint64_t)(n0 * G);
    r.zeros = zeros + (g0 >> 1);
    r.zpar = (int)(g0 & 1);
    r.s2 = nullptr;
    if constexpr (FMT == Q4_NF4_DQ) {
        // a row past the end points at the first constant (read, never
        // used: its codes are 0)
        r.s2 = (const float *)zeros + (r.live ? g0 >> 8 : 0);
        r.zpar = (int)(g0 & (kDqRun - 1));
    }
    return r;
}

// One pipeline stage of a wave: 128 chunks of 32 weights of one row; lane l
// holds chunks l and 64 + l of the stage (so each of the two 16-byte loads
// of the wave reads 1 KB of consecutive codes), with their scales and
// zero-points.
struct Stage {
    u32x4 cw[2];
    float sc[2];
    float zf[2];
    // double quantization: the constants of the runs of kDqRun groups the
    // stage touches (at most 2, and the next; scalar registers) and the
    // stage's first group's position in the first of them
    float s2[3];
    int zpar;
};

// Chunk of half h of stage s for a lane.
__device__ __forceinline__ int stage_chunk(int s, int lane, int h) { return kStageChunks * s + 64 * h + lane; }

// A lane's offsets into the per-stage views (constant for the kernel): its
// chunk's codes and scale, and (asym) the byte and nibble of its group's
// zero-point for either parity of the row's first flat group.
struct LaneOffs {
    uint32_t cd[2], sc[2], zb[2][2], zsh[2][2];
};
template <int FMT>
__device__ __forceinline__ LaneOffs lane_offs(int lane, int gshift)
{
    constexpr int ss = f32_absmax(FMT) ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);
    LaneOffs o;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int lc = 64 * h + lane;      // chunk within the stage
        const int gl = (32 * lc) >> gshift;  // its group within the stage
        o.cd[h] = 16 * lc;
        o.sc[h] = ss * gl;
#pragma unroll
        for (int p = 0; p < 2; ++p) {
            o.zb[p][h] = (p + gl) >> 1;
            o.zsh[p][h] = 4 * ((p + gl) & 1);
        }
    }
    return o;
}

// Non-temporal loads: the weights are streamed once per product, so they are
// not kept in the caches (the "nt" cache-policy bit).
constexpr int kNT = 2;
// The device-scope cache policy (the "sc1" bit): the access is coherent
// across the device's L2 caches, as an agent-scope atomic load is.
constexpr int kCoherent = 16;

// The loads of stage s of a row.  Each array is read through a view that
// starts at the stage's first byte and ends at the row's last (built with
// scalar arithmetic), and every lane uses its constant offset: the buffer
// unit's range check then returns zeros for chunks past the row end and for
// a row past the last one (an empty view), without any per-lane arithmetic
// and without touching memory outside the row.
template <int FMT>
__device__ __forceinline__ void load_stage(Stage &st, const RowRef &r, int s, const LaneOffs &lo,
                                           int row_bytes, int G, int gshift)
{
    constexpr int ss = f32_absmax(FMT) ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);
    const int cs = 16 * kStageChunks * s;                 // the stage's first code byte
    const int gs = (kStageChunks * 32 * s) >> gshift;      // the stage's first group in the row
    const __amdgpu_buffer_rsrc_t cr = make_rsrc(r.codes + cs, r.live ? row_bytes - cs : 0);
    const __amdgpu_buffer_rsrc_t sr = make_rsrc(r.scales + gs * ss, r.live ? (G - gs) * ss : 0);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        st.cw[h] = __builtin_amdgcn_raw_buffer_load_b128(cr, lo.cd[h], 0, kNT);
        if constexpr (f32_absmax(FMT))
            st.sc[h] = std::bit_cast<float>(__builtin_amdgcn_raw_buffer_load_b32(sr, lo.sc[h], 0, kNT));
        else if constexpr (FMT == Q4_NF4_DQ)  // the 8-bit code; the constant below
            st.sc[h] = std::bit_cast<float>((uint32_t)__builtin_amdgcn_raw_buffer_load_b8(sr, lo.sc[h], 0, kNT));
        else
            st.sc[h] = h2f(__builtin_amdgcn_raw_buffer_load_b16(sr, lo.sc[h], 0, kNT));
        st.zf[h] = 0.0f;
    }
    if constexpr (FMT == Q4_INT4_ASYM) {
        // nibble zpar + gs + gl of the row's zero-point bytes; gs is even
        const __amdgpu_buffer_rsrc_t zr =
            make_rsrc(r.zeros + (gs >> 1), r.live ? (G - gs + r.zpar + 1) >> 1 : 0);
        const int p = r.zpar;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t b = __builtin_amdgcn_raw_buffer_load_b8(zr, p ? lo.zb[1][h] : lo.zb[0][h], 0, kNT);
            st.zf[h] = (float)((b >> (p ? lo.zsh[1][h] : lo.zsh[0][h])) & 0xf);
        }
    }
    if constexpr (FMT == Q4_NF4_DQ) {
        // One scalar load of the constants of the runs the stage touches,
        // from the run holding its first group (a stage of 4096 weights
        // holds at most 128 groups, so it touches at most 2 runs, whatever
        // the row's length; the last constants loaded may be the buffer's
        // padding, never used for a real group), rather than a vector load
        // per stage.  The group's run is picked when the stage is computed.
        // A row past the end reads the first constants (its codes are 0).
        const int u0 = r.zpar + gs;  // the stage's first group, from the start of the row's first run
        typedef float f32x4a4 __attribute__((ext_vector_type(4), aligned(4)));
        const f32x4a4 c =
            *(const __attribute__((address_space(4))) f32x4a4 *)(r.s2 + (r.live ? u0 / kDqRun : 0));
        st.s2[0] = c[0];
        st.s2[1] = c[1];
        st.s2[2] = c[2];
        st.zpar = u0 & (kDqRun - 1);
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

// acc += the dot product of 8 weights and 8 activations (16-bit values,
// packed in pairs): four v_dot2, alternating between the two accumulators.
template <int ACT>
__device__ __forceinline__ void dot8(const u32x4 &w, const u32x4 &x, float2 &acc)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        float &a = (k & 1) ? acc.y : acc.x;
        if constexpr (ACT == Q4_BF16)
            a = __builtin_amdgcn_fdot2_f32_bf16(std::bit_cast<bf16x2>(w[k]), std::bit_cast<bf16x2>(x[k]), a,
                                                false);
        else
            a = __builtin_amdgcn_fdot2(std::bit_cast<f16x2>(w[k]), std::bit_cast<f16x2>(x[k]), a, false);
    }
}

// Sum over the wave of the lanes' two accumulators; every lane gets the total.
__device__ __forceinline__ float row_sum(const float2 &a) { return wave_sum(a.x + a.y); }

// Table lookups of one code dword: the binary32 level pairs of its 4 bytes.
__device__ __forceinline__ void lookup4(uint32_t w, uint32_t laneoff, const uint32_t *__restrict__ tbl,
                                        float2 (&lv)[4])
{
    constexpr uint32_t kSel[4] = {0x0c0c0400u, 0x0c0c0500u, 0x0c0c0600u, 0x0c0c0700u};
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const uint32_t addr = __builtin_amdgcn_perm(w, laneoff, kSel[k]);
        lv[k] = *(const float2 *)((const char *)tbl + addr);
    }
}

// Products of one stage: 8 steps of 8 weights (two chunks x four dwords of
// codes).  Per code byte: its LDS address by one v_perm, one 8-byte table
// read (the two nibbles' binary32 levels), two fma with the chunk's scale
// and bias, one packed conversion to the activation dtype and one v_dot2
// per activation row.  The lookups of the next dword
// are issued before the current one is converted (scheduling barriers keep
// that order), so a table read's latency hides behind a dword of
// arithmetic.
template <int FMT, int ACT, int MT, int XS>
__device__ __forceinline__ void compute_stage(const Stage &st, float2 (&acc)[MT],
                                              const uint32_t *__restrict__ tbl, const uint32_t *xs,
                                              const u32x4 (&xreg)[XS == X_REG ? 8 * MT : 1],
                                              __amdgpu_buffer_rsrc_t xr, int K, int xrow, int s,
                                              int lane, int C, uint32_t laneoff, int gshift)
{
    constexpr bool nf4 = level_fmt(FMT) == Q4_NF4;
    // scale and bias of each half
    float sc[2], bias[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        sc[h] = st.sc[h];
        if constexpr (FMT == Q4_NF4_DQ) {
            // The half's 64 chunks cover at most 64 groups, so at most
            // two runs: the run of its first group (ra) and the next
            // (rb), picked per half from wave-uniform values; a lane
            // takes rb when its group is at or past the run boundary.
            // Groups are counted from the start of the run holding the
            // stage's first group.
            const int u = st.zpar + ((64 * 32 * h) >> gshift);
            const int r0 = u >> 8;                         // 0..1
            const int thr = 256 * (r0 + 1) - u;            // first lane group in rb
            const uint32_t a0 = std::bit_cast<uint32_t>(st.s2[0]);
            const uint32_t a1 = std::bit_cast<uint32_t>(st.s2[1]);
            const uint32_t a2 = std::bit_cast<uint32_t>(st.s2[2]);
            const uint32_t ra = r0 == 0 ? a0 : (r0 == 1 ? a1 : a2);
            const uint32_t rb = r0 == 0 ? a1 : a2;
            const int lg = (32 * lane) >> gshift;          // the lane's group in the half
            const float s2 = std::bit_cast<float>(lg >= thr ? rb : ra);
            // c' = qc * s2.  A chunk past the row end has qc = 0 (its load
            // is out of the view) and its run may lie past the last one,
            // where the constant is read from the buffer's padding (any
            // bits): c' = 0 there without the product.  For a real group
            // with qc = 0 this is the same +0 as the product.
            const uint32_t qc = std::bit_cast<uint32_t>(st.sc[h]);
            sc[h] = qc != 0 ? keep_f32((float)qc * s2) : 0.0f;
        }
        bias[h] = chunk_bias<FMT>(sc[h], st.zf[h]);
    }
    u32x4 xv[MT];
    if constexpr (XS == X_REG) {
#pragma unroll
        for (int m = 0; m < MT; ++m)
            xv[m] = xreg[m * 8];
    } else {
        load_x<MT, XS>(xv, xs, xr, K, xrow, stage_chunk(s, lane, 0), C, 0);
    }
    float2 lv[2][4];
    lookup4(st.cw[0][0], laneoff, tbl, lv[0]);
#pragma unroll
    for (int t = 0; t < 8; ++t) {  // step t: dword t & 3 of half t >> 2
        const int h = t >> 2;
        u32x4 xn[MT];
        if (t < 7) {
            lookup4(st.cw[(t + 1) >> 2][(t + 1) & 3], laneoff, tbl, lv[(t + 1) & 1]);
            if constexpr (XS == X_REG) {
#pragma unroll
                for (int m = 0; m < MT; ++m)
                    xn[m] = xreg[m * 8 + t + 1];
            } else {
                load_x<MT, XS>(xn, xs, xr, K, xrow, stage_chunk(s, lane, (t + 1) >> 2), C,
                               (t + 1) & 3);
            }
        }
        __builtin_amdgcn_sched_barrier(0);
        u32x4 wf;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float w0 = __builtin_fmaf(lv[t & 1][k].x, sc[h], bias[h]);
            float w1 = __builtin_fmaf(lv[t & 1][k].y, sc[h], bias[h]);
            if constexpr (nf4) {
                // rounded to binary32 first, then to the activation dtype
                // (no single-rounding mixed fma)
                w0 = keep_f32(w0);
                w1 = keep_f32(w1);
            }
            wf[k] = ACT == Q4_BF16 ? pack_bf2(w0, w1) : pack_h2(w0, w1);
        }
#pragma unroll
        for (int m = 0; m < MT; ++m)
            dot8<ACT>(wf, xv[m], acc[m]);
        if (t < 7) {
#pragma unroll
            for (int m = 0; m < MT; ++m)
                xv[m] = xn[m];
        }
        __builtin_amdgcn_sched_barrier(0);
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
// ... and in a chain's walk: task, row and stage.
struct ChainPos {
    int t, row, s;
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
    constexpr int kWaves = Shape<XS>::waves;
    constexpr int kBlock = Shape<XS>::block;
    // One LDS block with the table first, at address 0, so that a lookup's
    // address is the v_perm result itself.
    struct Lds {
        uint32_t tbl[kTableDwords];
        uint32_t xs[XS != X_GLOBAL ? kXBytes / 4 : 4];
    };
    __shared__ Lds lds;
    uint32_t *const tbl = lds.tbl;
    uint32_t *const xs = lds.xs;

    const int lane = threadIdx.x & 63;
    const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
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
    // first P weight positions, then the table.
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

    // ring of P in-flight positions (a row past the end has an empty view,
    // so its loads return zeros and it is never computed)
    const LaneOffs lo = lane_offs<FMT>(lane, gshift);
    Pos pos[P];
    Stage st[P];
    pos[0] = Pos{(int)__builtin_amdgcn_readfirstlane(blockIdx.x * kWaves + (threadIdx.x >> 6)), 0};
#pragma unroll
    for (int q = 0; q < P; ++q) {
        if (q > 0)
            pos[q] = advance(pos[q - 1]);
        load_stage<FMT>(st[q], row_ref<FMT>(codes, scales, zeros, pos[q].row, N, row_bytes, G),
                        pos[q].s, lo, row_bytes, G, gshift);
    }

    fill_level_table<FMT, kBlock>(tbl);
    if constexpr (XS != X_GLOBAL) {
#pragma unroll
        for (int i = 0; i < XP; ++i)
            if (xp[i] >= 0)
                *(u32x4 *)((char *)xs + xpad(16 * xp[i])) = xt[i];
    }
    __syncthreads();

    // one stage per row (M = 1): each lane keeps its activation slices
    // (chunks lane and 64 + lane) in registers for the whole kernel
    if constexpr (XS == X_REG) {
#pragma unroll
        for (int m = 0; m < MT; ++m) {
#pragma unroll
            for (int t = 0; t < 8; ++t)
                xreg[m * 8 + t] = *(const u32x4 *)((const char *)xs +
                                                   xpad(m * xrow + 64 * stage_chunk(0, lane, t >> 2) +
                                                        16 * (t & 3)));
        }
    }

    float2 acc[MT];
#pragma unroll
    for (int m = 0; m < MT; ++m)
        acc[m] = float2{0.0f, 0.0f};

    // A round of the ring is never left in the middle (the load waits stay
    // partial only if every path refills every slot): a position past the
    // last row has loaded zeros from an empty view; it is computed on them
    // and writes nothing.
    while (pos[0].row < N) {
#pragma unroll
        for (int q = 0; q < P; ++q) {
            const Pos cp = pos[q];
            // (a position past the last row is not computed: its slot is
            // still refilled below)
            if (cp.row < N)
                compute_stage<FMT, ACT, MT, XS>(st[q], acc, tbl, xs, xreg, xr, K, xrow, cp.s, lane,
                                               C, laneoff, gshift);
            // (double quantization: keep the refill after the compute, which
            // the scheduler otherwise hoists at the cost of registers)
            if constexpr (FMT == Q4_NF4_DQ)
                __builtin_amdgcn_sched_barrier(0);
            // refill this slot with the position P steps ahead
            pos[q] = advance(pos[(q + P - 1) % P]);
            {
                load_stage<FMT>(st[q], row_ref<FMT>(codes, scales, zeros, pos[q].row, N, row_bytes, G),
                                pos[q].s, lo, row_bytes, G, gshift);
            }
            if (cp.s == S - 1 && cp.row < N) {
                float out = 0.0f;
#pragma unroll
                for (int m = 0; m < MT; ++m) {
                    const float t = row_sum(acc[m]);
                    acc[m] = float2{0.0f, 0.0f};
                    if (lane == m)
                        out = t;
                }
                if (lane < M && lane < MT)
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
// on earlier tasks.  x sits in LDS in 8 slots of one stage each (8 KB);
// task t's stages take consecutive slots from slot base_t on (mod 8), tasks
// in turn, so a slot is reused only by a task at least two later.  x of
// task t is copied in (by DMA) once every compute wave has entered the task
// after the last one that used those slots (the gate, computed on the host)
// and then published; a compute wave entering task t waits only for that.
// All 16 waves of a workgroup compute; the last one also moves x, for each
// task in turn once it has no earlier positions left to compute, with its
// own weight loads for the task already out.  (A
// separate loader wave, which copied x as early as the gates allowed, left
// its SIMD a wave short of the others: 16 compute waves measured 1 % faster
// on the independent decode token and 8 % on the dependent one.)
//  * With no task waiting for earlier outputs, each workgroup works on one
//    contiguous block of the tasks' rows and loads and enters only the
//    block's tasks, so a workgroup meets a new task once or twice per
//    launch.
//  * Otherwise every task's rows are spread over all waves of the grid:
//    4096 waves on 256 units, so that the 4096-row products of a decode
//    layer give every wave one row (with 15 compute waves, 256 of the 3840
//    waves took a second row, and a task ended one row later).  For a task
//    that reads earlier outputs the last wave first waits until every wave
//    of the workgroup has finished the earlier tasks, then for the whole
//    grid (a grid barrier between these waves).
// The table is filled once per launch.
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
    // the sync words (layout below: zero on entry, left zero on exit except
    // the timeout flag, set to 1 when a wait ran out)
    uint32_t *sync;
};
constexpr uint32_t kSpinLimit = 1u << 20;  // bounded waits (of the order of a second)

// Layout of the sync buffer, in 32-bit words (one 128-byte line holds 32):
// line 0 the finished-workgroup count and the timeout flag; lines 1-8 the
// grid barrier's arrival counters, one per group, each on a line of its own
// so that the atomics of different groups do not contend; line 9 the
// groups' done flags, words 0-7 (polled, never the target of an atomic).
constexpr int kSyncLine = 32;
constexpr int kBarGroups = 8;
constexpr int kSyncDone = 0;
constexpr int kSyncTimeout = 2;
constexpr int kSyncArrive = kSyncLine;                    // + kSyncLine * group
constexpr int kSyncFlag = kSyncLine * (1 + kBarGroups);  // + group
static_assert(4 * (kSyncFlag + kSyncLine) == Q4_GEMV_CHAIN_SYNC_BYTES, "sync buffer layout");

// Grid barrier number `nbar` of a chain, run by one whole wave per
// workgroup.  Workgroup b arrives at group b % 8's counter; the group's last
// arrival raises the group's done flag to nbar; lane g of every waiting wave
// polls group g's flag until all are up.  Arrivals are spread over 8
// counters so that no counter takes more than a few dozen atomics per
// barrier, and the polls read a line no atomic targets.  The counters only
// grow during a chain (barrier n is complete at n times the arrivals), so no
// barrier resets them.
//
// Memory order without cache maintenance.  Every access that carries data
// from one workgroup to another -- the outputs of a task that a later task
// reads, and that read itself -- is an agent-scope coherent access (the
// device-scope cache policy, sc1, that agent-scope atomic loads and stores
// use), so no dirty or stale copy of it sits in any one XCD's L2.  What is
// left is order: a compute wave waits for its output stores to complete
// (s_waitcnt vmcnt(0)) before it counts into the next task in LDS; the
// workgroup's last wave, which moves x, arrives only after every compute
// wave has; the last arrival of a
// group and the flag store follow the counter's atomic return; the x
// loads go out after a flag poll has returned.  Each step starts after the
// previous one has completed, so the outputs are at the coherence point
// before any reader asks for them.  (A release/acquire fence pair at agent
// scope would write back and invalidate the L2 at every barrier: measured
// at about 4 us per barrier on the 7B token's chain.)
template <class Fail>
__device__ __forceinline__ void grid_barrier(uint32_t *sync, uint32_t nbar, int lane, Fail fail)
{
    const uint32_t ng = gridDim.x < kBarGroups ? gridDim.x : kBarGroups;
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
    if (lane == 0) {
        const uint32_t grp = blockIdx.x % kBarGroups;
        const uint32_t gsz = (gridDim.x - grp + kBarGroups - 1) / kBarGroups;  // its workgroups
        const uint32_t old = __hip_atomic_fetch_add(&sync[kSyncArrive + kSyncLine * grp], 1u,
                                                    __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if (old + 1 == nbar * gsz)
            __hip_atomic_store(&sync[kSyncFlag + grp], nbar, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    }
    const uint32_t g = (uint32_t)lane < ng ? (uint32_t)lane : 0u;
    uint32_t spins = 0;
    while (!__all(__hip_atomic_load(&sync[kSyncFlag + g], __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT) >= nbar)) {
        if (++spins == kSpinLimit) {
            fail();
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
constexpr int kChainMaxK = 16384;  // 4 stages: a task and the next fit the 8 slots

__host__ __device__ __forceinline__ int chain_stages(int K) { return ((K >> 5) + kStageChunks - 1) / kStageChunks; }

// One task's arrays and sizes, kept in scalar registers while a wave works
// on the task: a row's and a stage's views are built from them with a few
// scalar instructions, without reloading the task's arguments.
struct TaskViews {
    const uint8_t *codes;
    const void *scales;
    const uint8_t *zeros;  // asym: zero-points; double quantization: the constants
    uint16_t *y;
    int N, S, C, row_bytes, G, xbase;
};

template <int FMT>
__device__ __forceinline__ TaskViews task_views(const ChainTask &T, int gshift)
{
    TaskViews v;
    v.N = T.N;
    v.row_bytes = T.K >> 1;
    v.G = T.K >> gshift;
    v.C = T.K >> 5;
    v.S = chain_stages(T.K);
    v.codes = T.codes;
    v.scales = T.scales;
    v.zeros = T.zeros;
    v.y = T.y;
    v.xbase = ctl_base(T.ctl);
    return v;
}

// The loads of stage s of row `row` of a task (row == N: past the last row,
// every load returns zero).
template <int FMT>
__device__ __forceinline__ void load_stage_chain(Stage &st, const TaskViews &tv, int row, int s,
                                                 const LaneOffs &lo, int gshift)
{
    load_stage<FMT>(st, row_ref<FMT>(tv.codes, tv.scales, tv.zeros, row, tv.N, tv.row_bytes, tv.G),
                    s, lo, tv.row_bytes, tv.G, gshift);
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
// consecutive bytes (no bank conflicts).
__device__ __forceinline__ int chain_slot(int base, int s) { return (base + s) & (kChainSlots - 1); }
__device__ __forceinline__ int chain_x_index(int slot, int j, int c) { return 512 * slot + 128 * j + c; }

// A lane's x slice for stage s of a row: chunks l and 64 + l of the stage
// (the stored rows are zero past K up to whole stages).
__device__ __forceinline__ void chain_x_slice(u32x4 (&xreg)[8], const u32x4 *xb, int base, int s,
                                              int lane)
{
    const int slot = chain_slot(base, s);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
            xreg[4 * h + j] = xb[chain_x_index(slot, j, 64 * h + lane)];
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

// The copy of x[0, K) of a task into the task's slots (by the workgroup's
// last wave), by the buffer unit straight into LDS (no registers): per
// stage, half and piece, one 16-byte load per lane, lane l's piece j of
// chunk c0 + l landing at 16-byte index 128 j + c0 + l of the slot, the
// piece-major order the compute waves read.
// The whole offset is the lane's (voffset, range-checked against the x
// view), so pieces past K read zeros: the stored rows are padded to whole
// stages with zeros.
template <int CPOL = 0>
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
                    16, 64 * (kStageChunks * s + 64 * h + lane) + 16 * j, 0, 0, CPOL);
    }
}

constexpr int kChainCompute = 16;  // compute waves per workgroup (all of them)

// DEP: some task waits for earlier outputs (else the grid-barrier code is
// left out).
template <int FMT, int ACT, int P, bool DEP>
__global__ __launch_bounds__(1024) __attribute__((amdgpu_waves_per_eu(4)))
void gemv_chain_kernel(const ChainArgs a)
{
    // One LDS block with the table first, at address 0, so that a lookup's
    // address is the v_perm result itself.
    struct Lds {
        uint32_t tbl[kTableDwords];
        u32x4 xb[kChainSlots * 512];
        int entered[kChainMax];  // compute waves that entered each task
        int ready[kChainMax];    // 1 once x of the task is in its slots
        ChainTask tasks[kChainMax];
    };
    __shared__ Lds lds;
    uint32_t *const tbl = lds.tbl;
    auto &xb = lds.xb;
    auto &entered = lds.entered;
    auto &ready = lds.ready;

    const int lane = threadIdx.x & 63;
    const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const uint32_t laneoff = (uint32_t)(lane & 31) << 3;
    const int nt = a.ntasks;
    constexpr int NC = kChainCompute;
    // every compute wave has entered task t
    auto all_entered = [&](int t) {
        return __hip_atomic_load(&entered[t], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP) >= NC;
    };
    auto fail = [&]() {
        __hip_atomic_store(&a.sync[kSyncTimeout], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    };

    // the level table, by every wave
    fill_level_table<FMT, 1024>(tbl);
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

    {
        // ---------------------------------------------------------- compute
        // A wave's walk, task by task: in each task it takes rows first,
        // first + step, ... below end (a segment).  With no waiting task the
        // rows are those of the workgroup's block, dealt to its waves in
        // turn (continuing the turn across tasks); otherwise task t's rows
        // are dealt to all the grid's waves from a rotated start, so that
        // the waves holding one row more than the others differ from task
        // to task.  The ring is the single-product kernel's, with a position
        // a task, a row and a stage: it runs on from one segment into the
        // next (into the wave's next task with rows), so the loads of a
        // task's first rows are in flight while the wave finishes the
        // previous task and waits for the new task's x.
        const int wave_id = (int)__builtin_amdgcn_readfirstlane(blockIdx.x * NC + wave);
        const LaneOffs lo = lane_offs<FMT>(lane, a.gshift);
        const int total_waves = gridDim.x * NC;
        // the last wave also moves x: task tlo's here, every later task's
        // when it enters the task or passes it (lead_x)
        const bool lead = wave == NC - 1;
        if (lead) {
            // task tlo is entered by every compute wave in the prologue; the
            // tasks before it are never entered here (they count as entered,
            // for the gates of the slots they would have used)
            entered[lane] = lane <= tlo ? NC : 0;
            ready[lane] = 0;
            if (has_rows) {
                chain_dma_x(task(tlo), xb, lane);
                wait_vm<0>();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                __hip_atomic_store(&ready[tlo], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
            }
        }
        __syncthreads();  // the table, the counters and x of task tlo
        int cur = tlo;  // the last task this wave has counted into
        // Counting into task t (this wave is done with every earlier task).
        // Before a task that waits for the grid, this wave's own stores
        // complete first (the lead wave then passes them on to the grid; the
        // wait also covers the weight loads the ring already has in flight).
        auto arrive = [&](int t) {
            if (DEP && ctl_wait(task(t).ctl)) {
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
                wait_vm<0>();
                __atomic_signal_fence(__ATOMIC_SEQ_CST);
            }
            if (lane == 0)
                __hip_atomic_fetch_add(&entered[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };
        // Waiting for x of task t in its slots.
        auto await_x = [&](int t) {
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
        // (lead wave) x of task t into its slots, then published: once every
        // compute wave has entered the task's gate, or, for a task that reads
        // earlier outputs, has entered t (finished t - 1, stores complete)
        // and every workgroup has passed the grid barrier.  The lead wave's
        // own weight loads for t are out by then; the wait before publishing
        // covers them too.
        int nbar = 0;
        auto lead_x = [&](int t) {
            const ChainTask T = task(t);
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
                grid_barrier(a.sync, ++nbar, lane, fail);
                chain_dma_x<kCoherent>(T, xb, lane);  // earlier outputs
            } else {
                chain_dma_x(T, xb, lane);
            }
            wait_vm<0>();
            __atomic_signal_fence(__ATOMIC_SEQ_CST);
            __hip_atomic_store(&ready[t], 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
        };

        u32x4 xreg[8];
        float2 acc[1] = {float2{0.0f, 0.0f}};
        // The loader: the next position to load, in walk order across the
        // tasks (task lt, row lrow, stage ls), and the segment of task lt
        // (rows from its first, lstep apart, below lend); lt > thi once every
        // position is loaded.  The ring runs on across task boundaries, so a
        // task's first weights are in flight while the wave finishes the
        // previous task and waits for the new task's x.
        int lt = has_rows ? tlo - 1 : thi + 1, lrow = 0, ls = 0, lstep = 1, lend = 0;
        int turn = 0;  // blocked walk: the block's rows before task lt, mod NC
        TaskViews ltv = task_views<FMT>(task(0), a.gshift);
        auto next_task = [&]() {
            while (++lt <= thi) {
                const ChainTask T = task(lt);
                int first;
                if constexpr (!DEP) {
                    const int start = lt == tlo ? rlo : 0;
                    lend = lt == tend ? rend : T.N;
                    first = start + (wave - turn + NC) % NC;
                    lstep = NC;
                    turn = (turn + lend - start) % NC;
                } else {
                    first = (int)(((uint32_t)wave_id + (uint32_t)lt * 1237u) % (uint32_t)total_waves);
                    lstep = total_waves;
                    lend = T.N;
                }
                if (first < lend) {
                    ltv = task_views<FMT>(T, a.gshift);
                    lrow = first;
                    ls = 0;
                    return;
                }
            }
        };
        // Loads the loader's position into a ring slot (past the walk: an
        // empty row, whose loads return zeros) and moves the loader on.
        auto load_next = [&](Stage &st_, ChainPos &p) {
            const bool live = lt <= thi;
            p = ChainPos{live ? lt : nt, lrow, ls};
            load_stage_chain<FMT>(st_, ltv, live ? lrow : ltv.N, live ? ls : 0, lo, a.gshift);
            if (live && ++ls == ltv.S) {
                ls = 0;
                lrow += lstep;
                if (lrow >= lend)
                    next_task();
            }
        };
        // The compute side: task ct (views ctv) is the one being computed;
        // entering task t counts this wave into every task up to t, has the
        // lead wave copy x of every task up to t, and waits for x of t.
        int ct = -1, led = tlo;
        TaskViews ctv = ltv;
        auto enter = [&](int t) {
            while (cur < t)
                arrive(++cur);
            if (lead)
                while (led < t)
                    lead_x(++led);
            await_x(t);
            ctv = task_views<FMT>(task(t), a.gshift);
            ct = t;
            if (ctv.S == 1)
                chain_x_slice(xreg, xb, ctv.xbase, 0, lane);
        };

        if (has_rows)
            next_task();
        ChainPos pos[P];
        Stage st[P];
#pragma unroll
        for (int q = 0; q < P; ++q)
            load_next(st[q], pos[q]);
        // A round of the ring is never left in the middle (the load waits
        // stay partial only if every path refills every slot).
        while (pos[0].t <= thi) {
#pragma unroll
            for (int q = 0; q < P; ++q) {
                const ChainPos cp = pos[q];
                // (a position past the walk is not computed: its slot is
                // still refilled below)
                if (cp.t <= thi) {
                    if (cp.t != ct)
                        enter(cp.t);
                    if (ctv.S > 1)
                        chain_x_slice(xreg, xb, ctv.xbase, cp.s, lane);
                    // (x comes from registers: no x view, K or chunk count needed)
                    compute_stage<FMT, ACT, 1, X_REG>(st[q], acc, tbl, nullptr, xreg,
                                                      make_rsrc(nullptr, 0), 0, 0, cp.s, lane, 0,
                                                      laneoff, a.gshift);
                    if (cp.s == ctv.S - 1) {
                        const float out = row_sum(acc[0]);
                        acc[0] = float2{0.0f, 0.0f};
                        // through a global (not flat) pointer: a flat store
                        // may write LDS, so LDS reads after it would wait
                        auto *const yp = (__attribute__((address_space(1))) uint16_t *)(ctv.y + cp.row);
                        const uint16_t yb = (uint16_t)(ACT == Q4_BF16 ? f2bf_bits(out) : f2h_bits(out));
                        if (lane == 0) {
                            if constexpr (DEP)  // later tasks may read it (coherent store)
                                __hip_atomic_store(yp, yb, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                            else
                                *yp = yb;
                        }
                    }
                }
                load_next(st[q], pos[q]);
            }
        }
        // the tasks after this wave's last position: still counted into,
        // and (lead wave) their x copied for the other waves
        while (cur < thi)
            arrive(++cur);
        if (lead)
            while (led < thi)
                lead_x(++led);
    }
    wait_vm<0>();  // no LDS DMA may be in flight when the workgroup ends
    __syncthreads();
    if (threadIdx.x == 0) {
        // the last workgroup to finish leaves the counters at zero for the
        // next chain on this sync buffer (every workgroup is past its last
        // barrier by then)
        const uint32_t d = __hip_atomic_fetch_add(&a.sync[kSyncDone], 1u, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_AGENT);
        if (d == gridDim.x - 1) {
            for (int g = 0; g < kBarGroups; ++g) {
                __hip_atomic_store(&a.sync[kSyncArrive + kSyncLine * g], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(&a.sync[kSyncFlag + g], 0u, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
            }
            __hip_atomic_store(&a.sync[kSyncDone], 0u, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
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
    case Q4_FP4:
        return bf ? launch_chain_t<Q4_FP4, Q4_BF16>(a, s) : launch_chain_t<Q4_FP4, Q4_F16>(a, s);
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
    case Q4_FP4:
        return launch_act<Q4_FP4>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    case Q4_NF4_DQ:
        return launch_act<Q4_NF4_DQ>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    case Q4_INT4_SYM:
        return launch_act<Q4_INT4_SYM>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    default:
        return launch_act<Q4_INT4_ASYM>(act_t, x, (int)M, codes, scales, zeros, N, K, gshift, y, s);
    }
}

}  // namespace q4
