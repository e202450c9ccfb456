// gemm.hip -- prefill-shape fused dequant-GEMM on the matrix cores,
// y[M, N] = x[M, K] . What^T for any M.
//
// Method ("Loading a model in 4-bit", "Where the accuracy goes"; "INT4
// Quantization > Practical Implementation with bitsandbytes"): the weights
// are dequantized to the 16-bit compute dtype and multiplied in a standard
// 16-bit matmul with fp32 accumulation.  Every weight value fed to the
// matrix cores is exactly the one q4_dequantize writes (the activation
// dtype's nearest-even rounding of the binary32 product level * scale).
//
// gfx950 mapping (each choice measured on the part):
//  * A workgroup of 8 waves (two per SIMD) computes a 256 (x rows) by 256
//    (W rows) tile of y.  Wave w owns all 256 x rows against 32 W rows as
//    2 x 16 accumulators of v_mfma_f32_16x16x32_{bf16,f16} (128 fp32
//    registers, VGPR form; with 256 accumulators per wave the register
//    allocator shuffles them between register files around every MFMA).
//    The MFMA's first operand is a 16 x 32 block of dequantized W, the
//    second a 16 x 32 block of x, so a result lane holds 4 consecutive W
//    rows of one x row.  No wave dequantizes another wave's weights.
//  * K advances 64 per step.  x is staged in double-buffered LDS by the
//    buffer unit's direct-to-LDS loads (no registers, no LDS writes): each
//    wave moves 4 KB per step as 1 KB blocks of 8 rows x 128 bytes, the
//    16-byte chunks of a row XOR-swizzled.  One barrier per step.
//  * The contraction order over k inside a step is permuted identically for
//    both operands (lane quad f takes k-chunks 2f and 2f + 1 of the step), so
//    a lane's weights in a step are 16 contiguous codes of one group: one
//    8-byte code load per fragment and step, issued two steps ahead.
//  * Scales and zero-points are fetched once per 4 steps (256 k): one wide
//    load per fragment covering every group the row needs in that span, kept
//    in registers for the next span while the current one is used.  Loading
//    them per step (sub-dword loads from 16 rows at a time) held the texture
//    units up to a fifth of the run time.
//  * Dequantization runs in registers between the MFMAs: INT4 as one exact
//    fma per weight ((q - z) * s = q * s + (-z * s), both terms exact), NF4
//    as a byte-indexed LDS table of level pairs and one binary32 multiply.
//    With double-quantized NF4 absmax the span load brings the 8-bit codes
//    and the runs' binary32 constants, and each group's absmax is recovered
//    with one product before the NF4 path.
//  * W rows are assigned to fragment positions so that each lane's 8 output
//    values are 8 consecutive columns of y: one 16-byte store per lane per
//    x-row fragment.
//  * Tiles are numbered x-block fastest; workgroups are dealt round-robin to
//    the 8 XCDs, so with 8 x-blocks each XCD keeps one 256-row block of x
//    hot in its own L2.
#include "q4_common.hpp"
#include "q4_internal.hpp"
#include "q4_mfma.hpp"

namespace q4 {
namespace {

constexpr int BM = 256;                       // x rows per tile
#ifndef Q4_GEMM_BN
#define Q4_GEMM_BN 256
#endif
#ifndef Q4_GEMM_WAVES
#define Q4_GEMM_WAVES 8
#endif
constexpr int BN = Q4_GEMM_BN;                // W rows per tile
constexpr int BK = 64;                        // k per step
constexpr int kWaves = Q4_GEMM_WAVES;         // waves per workgroup (BN / 32)
constexpr int kBlock = 64 * kWaves;
constexpr int ROW_BYTES = BK * 2;             // one staged x row
constexpr int X_BYTES = BM * ROW_BYTES;
constexpr int kXBlocks = X_BYTES / 1024 / kWaves;  // 1 KB x DMA blocks per wave per step (4)
constexpr int kMF = BM / 16;                  // x fragments per wave (16)
constexpr int kNF = BN / 16 / kWaves;         // W fragments per wave (2)
constexpr int kWRows = 16 * kNF;              // W rows per wave (32)
constexpr int kSpan = 4;                      // steps per scale / zero-point span
constexpr int kSpanK = kSpan * BK;            // 256

// A buffer view: base and length in bytes (at most 2^32 - 1; the host
// bounds K so that every view of a tile fits).  Loads go through a resource
// over [base + off, base + bytes) for the load's wave-uniform offset `off`:
// the buffer unit range-checks only the lane's offset (voffset), not a
// load's soffset, so a uniform part that may pass the end of the view
// moves the view instead.  The range check is per dword: a dword not
// wholly inside the view reads as zero.
struct View {
    const char *base;
    uint32_t bytes;
};
__device__ __forceinline__ View make_view(const void *base, int64_t bytes)
{
    const int64_t cap = 0xffffffffll;
    return View{(const char *)base, (uint32_t)(bytes <= 0 ? 0 : (bytes > cap ? cap : bytes))};
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t at(const View &v, uint32_t off)
{
    // (read back as a wave-uniform value: the compiler forms this clamped
    // difference with a vector instruction, and a resource it cannot prove
    // uniform turns every load through it into a loop over lanes)
    const uint32_t n = __builtin_amdgcn_readfirstlane(off < v.bytes ? v.bytes - off : 0u);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<char *>(v.base + off), (short)0, (int)n,
                                             0x00020000);
}

// Position of 16-byte chunk c of staged x row r (and the chunk at position c):
// c XOR a 3-bit key from bits 1-3 of r.  A fragment read (lane l: row l & 15,
// chunk 2 (l >> 4) + h) then puts the rows that share a 128-bank line
// (r, r + 4, r + 8, r + 12) on distinct 16-byte positions for each pair of
// lane quads, and the 8 rows of one parity on 8 distinct positions: no bank
// conflicts.  (A key of (r >> 1) & 7 cost about 4 conflict cycles per read.)
__device__ __forceinline__ int swz_key(int r) { return ((r >> 2) & 1) | (r & 2) | (((r >> 3) & 1) << 2); }
__device__ __forceinline__ int swz(int r, int c) { return c ^ swz_key(r); }

// Scale / zero-point layout of one 256-k span of a row.
template <int FMT, int G>
struct Span {
    static constexpr int ng = kSpanK / G;                  // groups per span (8, 4, 2)
    // bytes per scale (double-quantized NF4: the 8-bit absmax code)
    static constexpr int ss = f32_absmax(FMT) ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);
    // scale dwords per span (1 .. 8)
    static constexpr int sdw = FMT == Q4_NF4_DQ ? (ng == 8 ? 2 : 1) : ng * ss / 4;
    // loads per fragment and span: scales (16 bytes each at most), then the
    // zero-points (asym) or the runs' second-level constants (NF4_DQ)
    static constexpr int nload =
        (sdw >= 4 ? sdw / 4 : 1) + (FMT == Q4_INT4_ASYM || FMT == Q4_NF4_DQ ? 1 : 0);
};

// Per-lane codes of one step: 16 codes per fragment, one dword per 32-deep
// half step.
struct WStep {
    u32x2 cw[kNF];
};

// Per-lane scales and zero-points of one span, as loaded: the scale dwords
// of the row's groups and the 64 bits holding its zero-point nibbles (for
// double-quantized NF4: the 8-bit absmax codes, and the second-level
// constants of the run holding the span's first group and of the next run).
template <int FMT, int G>
struct MSpan {
    uint32_t s[kNF][Span<FMT, G>::sdw];
    u32x2 z[kNF];
};

// Per-thread constants of the tile.  Every load address is a lane constant
// (voffset) plus a wave-uniform part that moves the view (scalar
// arithmetic), so the loads cost no vector arithmetic.
struct TileCtx {
    View xr, cr, sr, zr;
    int K, Gn;   // K and groups per row
    int xv[2];   // x DMA: voffset for even / odd blocks
    int rd[2];   // fragment reads: LDS byte offset of half step h (+2048 per fragment)
    int cv;      // codes: voffset of fragment 0 at k = 0
    int sv;      // scales: voffset of fragment 0's row
    int zv;      // zero-points: voffset of the byte holding fragment 0's row's first nibble;
                 // NF4_DQ: fragment 0's row's first group counted from the start of
                 // the run holding the tile's first group
    int zo;      // ... and that nibble's position in it (0 or 1)
    int fq;      // lane quad
};

// x of the step at k0 into LDS buffer xn: 32 blocks of 1 KB (8 rows each),
// kXBlocks per wave, written by the buffer unit straight into LDS (lane l
// of a block lands at 16 l).  Rows past M read zeros.
__device__ __forceinline__ void load_x1(const TileCtx &c, char *xn, int wave, int i, int k0)
{
    const int B = kXBlocks * wave + i;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        at(c.xr, (uint32_t)(B * 16 * c.K + 2 * k0)),
        (__attribute__((address_space(3))) void *)(xn + 1024 * B), 16, c.xv[i & 1], 0, 0, 0);
}

// Codes of fragment j at step k0 (fragment j's rows are 4 j below
// fragment 0's).
__device__ __forceinline__ void load_codes(WStep &ws, int j, const TileCtx &c, int k0)
{
    ws.cw[j] = __builtin_amdgcn_raw_buffer_load_b64(at(c.cr, (uint32_t)(4 * j * (c.K >> 1) + (k0 >> 1))),
                                                    c.cv, 0, 0);
}

// Scales and zero-points of fragment j for the span starting at k0.
template <int FMT, int G>
__device__ __forceinline__ void load_span(MSpan<FMT, G> &ms, int j, const TileCtx &c, int k0)
{
    using S = Span<FMT, G>;
    const int ug = 4 * j * c.Gn + k0 / G;  // uniform part of the group index (even)
    const int so = ug * S::ss;
    if constexpr (S::sdw >= 4) {
#pragma unroll
        for (int q = 0; q < S::sdw / 4; ++q) {
            const u32x4 v = __builtin_amdgcn_raw_buffer_load_b128(at(c.sr, (uint32_t)(so + 16 * q)), c.sv, 0, 0);
            ms.s[j][4 * q] = v[0];
            ms.s[j][4 * q + 1] = v[1];
            ms.s[j][4 * q + 2] = v[2];
            ms.s[j][4 * q + 3] = v[3];
        }
    } else if constexpr (S::sdw == 2) {
        const u32x2 v = __builtin_amdgcn_raw_buffer_load_b64(at(c.sr, (uint32_t)so), c.sv, 0, 0);
        ms.s[j][0] = v[0];
        ms.s[j][1] = v[1];
    } else {
        ms.s[j][0] = __builtin_amdgcn_raw_buffer_load_b32(at(c.sr, (uint32_t)so), c.sv, 0, 0);
    }
    if constexpr (FMT == Q4_INT4_ASYM) {
        // ng nibbles from nibble zo of the first byte: 9 nibbles (5 bytes) at
        // most
        if constexpr (S::ng == 8)
            ms.z[j] = __builtin_amdgcn_raw_buffer_load_b64(at(c.zr, (uint32_t)(ug >> 1)), c.zv, 0, 0);
        else
            ms.z[j] = u32x2{__builtin_amdgcn_raw_buffer_load_b32(at(c.zr, (uint32_t)(ug >> 1)), c.zv, 0, 0), 0u};
    }
    if constexpr (FMT == Q4_NF4_DQ) {
        // the span's groups (at most 8) lie in one run or straddle into the
        // next: both constants, from the run of the first group
        ms.z[j] = __builtin_amdgcn_raw_buffer_load_b64(at(c.zr, 0), 4 * ((c.zv + ug) / kDqRun), 0, 0);
    }
}

// Scale and exact bias -z * s of fragment j at step sp (0..3) of the span
// at k0; the lane's 16 weights are group (64 sp + 16 fq) / G of the span.
// Weights at k >= K (the tail of a step past the end of the row) get
// s = b = 0, so they contribute exact zeros whatever x holds there.
template <int FMT, int G>
__device__ __forceinline__ void wscale(const MSpan<FMT, G> &ms, int j, int sp, const TileCtx &c,
                                       int k0, float &s, float &b)
{
    if constexpr (f32_absmax(FMT)) {
        if constexpr (G == 32)
            s = std::bit_cast<float>(c.fq >= 2 ? ms.s[j][2 * sp + 1] : ms.s[j][2 * sp]);
        else
            s = std::bit_cast<float>(ms.s[j][(64 * sp) / G]);
        b = 0.0f;
    } else if constexpr (FMT == Q4_NF4_DQ) {
        const int e = G == 32 ? 2 * sp + (c.fq >> 1) : (64 * sp) / G;  // group in the span
        const uint32_t q = (ms.s[j][e >> 2] >> (8 * (e & 3))) & 0xffu;
        const int first = c.zv + 4 * j * c.Gn + k0 / G;                // span's first group
        const uint32_t s2 = ((first % kDqRun) + e >= kDqRun) ? ms.z[j][1] : ms.z[j][0];
        s = keep_f32((float)q * std::bit_cast<float>(s2));  // c' = qc * s2, one product
        b = 0.0f;
    } else {
        uint32_t h;
        if constexpr (G == 32)
            h = c.fq >= 2 ? ms.s[j][sp] >> 16 : ms.s[j][sp];
        else if constexpr (G == 64)
            h = (sp & 1) ? ms.s[j][sp >> 1] >> 16 : ms.s[j][sp >> 1];
        else
            h = (sp & 2) ? ms.s[j][0] >> 16 : ms.s[j][0];
        s = h2f(h & 0xffffu);
        if constexpr (FMT == Q4_INT4_SYM) {
            b = -8.0f * s;
        } else {
            int e;
            if constexpr (G == 32)
                e = 2 * sp + (c.fq >> 1);
            else
                e = (64 * sp) / G;
            const uint64_t zz = ((uint64_t)ms.z[j][1] << 32) | ms.z[j][0];
            const uint32_t z = (uint32_t)(zz >> (4 * (c.zo + e))) & 0xfu;
            b = -(float)z * s;
        }
    }
    const bool in = k0 + 64 * sp + 16 * c.fq < c.K;
    s = in ? s : 0.0f;
    b = in ? b : 0.0f;
}

// One K step: step SP (0..3) of the span at k0 (the step's first k is
// k0 + 64 SP).  On entry wf[0] holds this step's first-half W fragments,
// own the codes of this step, nxt those of the next, mo / mn the scales of
// this step's / the next step's span, and LDS buffer xb this step's x.  The
// step is 32 groups, one per x fragment g = 16 h + i (x rows 16 i .. + 15,
// k-chunk 2 fq + h).  Each group reads x fragment g + 2 from LDS, runs the
// two MFMAs of fragment g and carries a share of the side work: the DMA of
// the next step's x into LDS buffer xn (groups 0-3), the loads of the codes
// two steps ahead (16-17, into own, dequantized by then), in step 1 of a
// span the scales of the next span (18-19, into mload), and the
// dequantization of this step's second half into wf[1] (groups 0-15) and
// of the next step's first half into wf[0] (16-31), one fragment every
// eight groups.  Scheduling fences between groups keep this order, so LDS
// reads stay two groups ahead of their use and no load is waited for
// early.  The step ends once this wave's x DMA has landed (later loads may
// still be in flight) at a workgroup barrier.
template <int FMT, int ACT, int G, int SP, bool LOADSPAN>
__device__ __forceinline__ void kstep(f32x4 (&acc)[kNF][kMF], u32x4 (&wf)[2][kNF], WStep &own,
                                      const WStep &nxt, const MSpan<FMT, G> &mo,
                                      const MSpan<FMT, G> &mn, MSpan<FMT, G> &mload,
                                      const char *xb, char *xn, const TileCtx &c,
                                      const float2 *ptbl, int wave, int k0)
{
    constexpr int SPN = (SP + 1) % kSpan;             // next step's index in its span
    const int ks = k0 + BK * SP;                       // this step's first k
    const int kn = SP + 1 < kSpan ? k0 : k0 + kSpanK;  // next step's span
    auto xread = [&](int g) {
        return *(const u32x4 *)(xb + c.rd[g >> 4] + 2048 * (g & 15));
    };
    u32x4 xf[3];
    float2 lp[4];
    float s = 0.0f, b = 0.0f;
    xf[0] = xread(0);
    xf[1] = xread(1);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int g = 0; g < 2 * kMF; ++g) {
        if (g < kXBlocks)
            load_x1(c, xn, wave, g, ks + BK);
        if (g >= kMF && g < kMF + kNF)
            load_codes(own, g - kMF, c, ks + 2 * BK);
        if constexpr (LOADSPAN) {
            if (g >= kMF + kNF && g < kMF + 2 * kNF)
                load_span<FMT, G>(mload, g - kMF - kNF, c, k0 + kSpanK);
        }
        if (g + 2 < 2 * kMF)
            xf[(g + 2) % 3] = xread(g + 2);
#pragma unroll
        for (int j = 0; j < kNF; ++j)
            acc[j][g & 15] = mfma<ACT>(wf[g >> 4][j], xf[g % 3], acc[j][g & 15]);
        // dequantization: one fragment every kUS groups, its scale and
        // table reads first, the arithmetic kUS / 2 groups later
        constexpr int kUS = kMF / kNF;
        const bool first = g < kMF;
        const WStep &src = first ? own : nxt;
        const int dh = first ? 1 : 0, dj = (g & 15) / kUS;
        if (g % kUS == 0) {
            if (first)
                wscale<FMT, G>(mo, dj, SP, c, k0, s, b);
            else
                wscale<FMT, G>(mn, dj, SPN, c, kn, s, b);
            if constexpr (level_fmt(FMT) == Q4_NF4) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lp[i] = ptbl[(src.cw[dj][dh] >> (8 * i)) & 0xffu];
            }
        }
        if (g % kUS == kUS / 2)
            wf[dh][dj] = dequant8<FMT, ACT>(src.cw[dj][dh], s, b, lp);
        __builtin_amdgcn_sched_barrier(0);
    }
    // The x DMA was issued before the other loads, and loads complete in
    // order: waiting until at most those are outstanding means this wave's
    // x is in LDS.  (vmcnt is bits 3:0 and 15:14; expcnt and lgkmcnt are
    // left at their maxima.)
    constexpr int nw = kNF + (LOADSPAN ? kNF * Span<FMT, G>::nload : 0);
    static_assert(nw < 16, "vmcnt field");
    __builtin_amdgcn_s_waitcnt(0x0f70 | nw);
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_sched_barrier(0);
}

template <int FMT, int ACT, int G>
__global__ __launch_bounds__(kBlock) void gemm_kernel(const uint16_t *__restrict__ x, int M,
                                                      const uint8_t *__restrict__ codes,
                                                      const void *__restrict__ scales,
                                                      const uint8_t *__restrict__ zeros, int N,
                                                      int K, int mtiles, int vec_y,
                                                      uint16_t *__restrict__ y)
{
    using S = Span<FMT, G>;
    // two x buffers as separate objects, so the compiler can tell that the
    // reads of one never alias the DMA into the other
    __shared__ __attribute__((aligned(1024))) char xs0[X_BYTES];
    __shared__ __attribute__((aligned(1024))) char xs1[X_BYTES];
    __shared__ float2 ptbl[level_fmt(FMT) == Q4_NF4 ? 256 : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int fr = lane & 15;
    const int fq = lane >> 4;
    const int m0 = (int)(blockIdx.x % (unsigned)mtiles) * BM;
    const int n0 = (int)(blockIdx.x / (unsigned)mtiles) * BN;
    const int Gn = K / G;

    if constexpr (level_fmt(FMT) == Q4_NF4) {
        if (t < 256)
            ptbl[t] = float2{level_entry<FMT>(t & 15), level_entry<FMT>(t >> 4)};
    }

    TileCtx c;
    c.K = K;
    c.Gn = Gn;
    c.fq = fq;
    // x and codes: views over this tile's rows only (x rows past M and W
    // rows past N read zeros).  Reads past the end of a row fall into the
    // next row (or past the view): such weights are given zero scale, and
    // such x values meet them only.  Scales and zero-points: views from the
    // tile's first group to the end of the padded arrays, so a wide span
    // load that starts at a meaningful byte never meets a dword straddling
    // the end (such a dword would read as zero).
    const int64_t mrows = M - m0 < BM ? M - m0 : BM;
    const int64_t nrows = N - n0 < BN ? N - n0 : BN;
    c.xr = make_view(x + (int64_t)m0 * K, mrows * K * 2);
    c.cr = make_view(codes + (int64_t)n0 * (K >> 1), nrows * (K >> 1));
    const int64_t s_total = FMT == Q4_NF4_DQ ? padded_meta_bytes(dq_scales_bytes((int64_t)N * Gn))
                                             : padded_meta_bytes((int64_t)N * Gn * S::ss);
    c.sr = make_view((const char *)scales + (int64_t)n0 * Gn * S::ss,
                     s_total - (int64_t)n0 * Gn * S::ss);
    const int64_t zg0 = (int64_t)n0 * Gn;  // flat group index of the tile's first group
    if constexpr (FMT == Q4_INT4_ASYM) {
        const int64_t z_total = padded_meta_bytes(((int64_t)N * Gn + 1) / 2);
        c.zr = make_view(zeros + (zg0 >> 1), z_total - (zg0 >> 1));
    } else if constexpr (FMT == Q4_NF4_DQ) {
        // second-level constants from the run of the tile's first group to
        // the end of the padded buffer (the 8-byte load of the last run
        // reads into the padding)
        const int64_t o2 = dq_s2_offset((int64_t)N * Gn) + 4 * (zg0 / kDqRun);
        c.zr = make_view((const char *)scales + o2, s_total - o2);
    } else {
        c.zr = c.sr;
    }

    // Fragment row p = 4a + v of W fragment j holds tile W row
    // kWRows * wave + 4 kNF a + 4j + v, so the result lane quad a ends up
    // with the 4 kNF consecutive W rows from kWRows * wave + 4 kNF a.
    const int wrow = kWRows * wave + 4 * kNF * (fr >> 2) + (fr & 3);
    c.cv = wrow * (K >> 1) + 8 * fq;
    c.sv = wrow * Gn * S::ss;
    {
        // zero-point nibbles of the row start at nibble (zg0 & 1) + wrow Gn
        // of the view; the uniform part added per span (4 j Gn + k / G) is
        // even, so the byte is (lane part >> 1) + (uniform part >> 1)
        const int a = (int)(zg0 & 1) + wrow * Gn;
        c.zv = a >> 1;
        c.zo = a & 1;
        if constexpr (FMT == Q4_NF4_DQ) {
            c.zv = (int)(zg0 % kDqRun) + wrow * Gn;
            c.zo = 0;
        }
    }
    // x DMA: lane l of 1 KB block B is row 8 B + l / 8, position l % 8,
    // holding chunk swz(8 B + l / 8, l % 8); bits 0-3 of the row are
    // 8 (B & 1) + l / 8
    {
        const int rl = lane >> 3, p = lane & 7;
#pragma unroll
        for (int e = 0; e < 2; ++e)
            c.xv[e] = rl * 2 * K + 16 * swz(8 * e + rl, p);
    }
    // fragment reads: x row 16 i + fr, chunk 2 fq + h (the swizzle does not
    // depend on i)
    c.rd[0] = fr * ROW_BYTES + 16 * swz(fr, 2 * fq);
    c.rd[1] = fr * ROW_BYTES + 16 * swz(fr, 2 * fq + 1);

    f32x4 acc[kNF][kMF];
#pragma unroll
    for (int j = 0; j < kNF; ++j)
#pragma unroll
        for (int i = 0; i < kMF; ++i)
            acc[j][i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // prologue: x of step 0 into LDS buffer 0, codes of steps 0 and 1, the
    // scales of span 0, the first half of step 0 dequantized
    u32x4 wf[2][kNF];
    WStep wa, wb;
    MSpan<FMT, G> mc, mn;
#pragma unroll
    for (int i = 0; i < kXBlocks; ++i)
        load_x1(c, xs0, wave, i, 0);
#pragma unroll
    for (int j = 0; j < kNF; ++j) {
        load_codes(wa, j, c, 0);
        load_codes(wb, j, c, BK);
        load_span<FMT, G>(mc, j, c, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0f70);  // everything issued so far
    __syncthreads();                     // x step 0 and the NF4 level-pair table
#pragma unroll
    for (int j = 0; j < kNF; ++j) {
        float s, b;
        float2 lp[4];
        wscale<FMT, G>(mc, j, 0, c, 0, s, b);
        if constexpr (level_fmt(FMT) == Q4_NF4) {
#pragma unroll
            for (int i = 0; i < 4; ++i)
                lp[i] = ptbl[(wa.cw[j][0] >> (8 * i)) & 0xffu];
        }
        wf[0][j] = dequant8<FMT, ACT>(wa.cw[j][0], s, b, lp);
    }

    // Spans of 4 steps; the code registers alternate roles step by step,
    // the span registers span by span (mn is loaded in step 1 and becomes
    // mc after step 3).  When K is not a multiple of 256 the last span runs
    // past K, where every weight has zero scale, so it adds exact zeros.
    // (A loop exit inside the span would keep two copies of the
    // accumulators live.)
    for (int k0 = 0; k0 < K; k0 += kSpanK) {
        kstep<FMT, ACT, G, 0, false>(acc, wf, wa, wb, mc, mc, mn, xs0, xs1, c, ptbl, wave, k0);
        kstep<FMT, ACT, G, 1, true>(acc, wf, wb, wa, mc, mc, mn, xs1, xs0, c, ptbl, wave, k0);
        kstep<FMT, ACT, G, 2, false>(acc, wf, wa, wb, mc, mc, mn, xs0, xs1, c, ptbl, wave, k0);
        kstep<FMT, ACT, G, 3, false>(acc, wf, wb, wa, mc, mn, mn, xs1, xs0, c, ptbl, wave, k0);
        mc = mn;
    }

    // epilogue: acc[j][i][v] is y[m0 + 16 i + fr][n0 + kWRows wave + 4 kNF fq + 4j + v]
    const int nb = n0 + kWRows * wave + 4 * kNF * fq;
#pragma unroll
    for (int i = 0; i < kMF; ++i) {
        const int m = m0 + 16 * i + fr;
        if (m >= M)
            continue;
        uint32_t p[2 * kNF];
#pragma unroll
        for (int j = 0; j < kNF; ++j) {
            p[2 * j] = pack2<ACT>(acc[j][i][0], acc[j][i][1]);
            p[2 * j + 1] = pack2<ACT>(acc[j][i][2], acc[j][i][3]);
        }
        uint16_t *yr = y + (int64_t)m * N + nb;
        if (vec_y && nb + 4 * kNF <= N) {
#pragma unroll
            for (int q = 0; q < kNF / 2; ++q)
                *(u32x4 *)(yr + 8 * q) = u32x4{p[4 * q], p[4 * q + 1], p[4 * q + 2], p[4 * q + 3]};
        } else {
#pragma unroll
            for (int e = 0; e < 4 * kNF; ++e)
                if (nb + e < N)
                    yr[e] = (uint16_t)(p[e >> 1] >> (16 * (e & 1)));
        }
    }
}

template <int FMT, int G>
hipError_t launch_g(q4_dtype act_t, const void *x, int64_t M, const uint8_t *codes,
                    const void *scales, const uint8_t *zeros, int64_t N, int64_t K, void *y,
                    hipStream_t s)
{
    const int64_t mt = (M + BM - 1) / BM, nt = (N + BN - 1) / BN;
    if (mt * nt > 0x7fffffffll)
        return hipErrorInvalidValue;
    // 16-byte output stores need 16-byte rows
    const int vec_y = (N % 8 == 0 && ((uintptr_t)y & 15) == 0) ? 1 : 0;
    dim3 grid((unsigned)(mt * nt)), block(kBlock);
    if (act_t == Q4_BF16)
        hipLaunchKernelGGL((gemm_kernel<FMT, Q4_BF16, G>), grid, block, 0, s, (const uint16_t *)x,
                           (int)M, codes, scales, zeros, (int)N, (int)K, (int)mt, vec_y,
                           (uint16_t *)y);
    else
        hipLaunchKernelGGL((gemm_kernel<FMT, Q4_F16, G>), grid, block, 0, s, (const uint16_t *)x,
                           (int)M, codes, scales, zeros, (int)N, (int)K, (int)mt, vec_y,
                           (uint16_t *)y);
    return hipGetLastError();
}

template <int FMT>
hipError_t launch_fmt(int g, q4_dtype act_t, const void *x, int64_t M, const uint8_t *codes,
                      const void *scales, const uint8_t *zeros, int64_t N, int64_t K, void *y,
                      hipStream_t s)
{
    switch (g) {
    case 32:
        return launch_g<FMT, 32>(act_t, x, M, codes, scales, zeros, N, K, y, s);
    case 64:
        return launch_g<FMT, 64>(act_t, x, M, codes, scales, zeros, N, K, y, s);
    default:
        return launch_g<FMT, 128>(act_t, x, M, codes, scales, zeros, N, K, y, s);
    }
}

}  // namespace

hipError_t launch_gemm(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                       const uint8_t *codes, const void *scales, const uint8_t *zeros, int64_t N,
                       int64_t K, void *y, hipStream_t s)
{
    switch (f) {
    case Q4_NF4:
        return launch_fmt<Q4_NF4>(g, act_t, x, M, codes, scales, zeros, N, K, y, s);
    case Q4_FP4:
        return launch_fmt<Q4_FP4>(g, act_t, x, M, codes, scales, zeros, N, K, y, s);
    case Q4_NF4_DQ:
        return launch_fmt<Q4_NF4_DQ>(g, act_t, x, M, codes, scales, zeros, N, K, y, s);
    case Q4_INT4_SYM:
        return launch_fmt<Q4_INT4_SYM>(g, act_t, x, M, codes, scales, zeros, N, K, y, s);
    default:
        return launch_fmt<Q4_INT4_ASYM>(g, act_t, x, M, codes, scales, zeros, N, K, y, s);
    }
}

}  // namespace q4
