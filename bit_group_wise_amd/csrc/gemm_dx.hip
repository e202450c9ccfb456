// gemm_dx.hip -- the backward product through a 4-bit weight,
// dX[M, K] = dY[M, N] . What[N, K], on the matrix cores.
//
// Method ("What is 4-bit quantization and why does it matter?", "QLoRA
// fine-tunes in 4-bit": the 4-bit base weights stay frozen and the gradient
// reaches the layer input through the dequantized weights; "Loading a model
// in 4-bit", "Where the accuracy goes": the weights are dequantized to the
// 16-bit compute dtype): every weight value is exactly the one q4_dequantize
// writes, the products run on v_mfma_f32_16x16x32_{bf16,f16} with fp32
// accumulation and dX is rounded once to the activation dtype.
//
// gfx950 mapping:
//  * The contraction runs over the weight's rows (N), so a matrix-core lane
//    needs 8 consecutive rows of one column.  The weight tile of a step (64
//    rows x 128 columns) is dequantized into LDS in its own row order (a
//    thread: 16 columns of one row, from one 8-byte code load that 8 lanes
//    make together, written as two 16-byte pieces) and read back transposed
//    by gfx950's ds_read_b64_tr_b16: in each 16-lane group, result lane i
//    takes element i % 4 of the 4-element piece addressed by lane
//    4 e + i / 4 (e the result element; probed on the part).  Two such reads
//    give a lane its 8 rows.  Rows are 288 bytes apart and the halves of
//    rows with bit 3 set are swapped, which spreads a read's 4 rows and its
//    next 16-lane group over distinct banks.  (Transposing on the write
//    side instead, as pairs of rows, needs row-strided code loads in which
//    every lane touches its own cache line; that ran at half the speed.)
//  * dY (the other operand, contiguous along N) is staged per step like the
//    forward product's activations: 256 rows x 128 bytes with the 16-byte
//    chunks of a row XOR-swizzled.
//  * A workgroup of 8 waves computes a 256 x 128 tile of dX, as 4 (rows) x
//    2 (columns) waves of 64 x 64: per 32-row half step a wave reads 4
//    fragments of each operand for 16 MFMAs (with all 256 rows per wave it
//    read 17 for 16, and the LDS reads, not the matrix cores, set the pace).
//  * Software pipeline: both LDS tiles are double-buffered (one barrier per
//    step) and each thread keeps two steps of loads (dY, codes, scales) in
//    flight in registers, so HBM/L2 latency hides behind two steps of
//    matrix-core work.
//  * Tiles are numbered M-block fastest and dealt round-robin to the 8 XCDs,
//    so each XCD keeps its 256 rows of dY in its own L2.
#include "q4_common.hpp"
#include "q4_internal.hpp"
#include "q4_mfma.hpp"

namespace q4 {
namespace {

constexpr int TM = 256;                // dY / dX rows per tile
constexpr int TK = 128;                // dX columns per tile (16 per wave)
constexpr int TN = 64;                 // contraction (weight rows) per step
constexpr int kWaves = 8;
constexpr int kBlock = 64 * kWaves;
constexpr int kYRow = TN * 2;          // bytes of one staged dY row
constexpr int kWPitch = TK * 2 + 32;   // bytes of one staged weight row (128 columns)
constexpr int kKF = 4;                 // k fragments per wave (64 columns)
constexpr int kWMF = 4;                // m fragments per wave (64 rows)

static_assert(TK == 2 * 16 * kKF && TM == 4 * 16 * kWMF && kWaves == 8, "2 x 4 waves");
static_assert(TN * TK / 16 == kBlock, "16 columns of one row per thread");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dx_rsrc(const void *base, int64_t bytes)
{
    // (read back as a wave-uniform value: a resource the compiler cannot
    // prove uniform turns every load through it into a loop over lanes)
    const uint32_t n = __builtin_amdgcn_readfirstlane(
        bytes <= 0 ? 0u : (bytes >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)bytes));
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             0x00020000);
}

// Position of 16-byte chunk c of staged dY row r.
__device__ __forceinline__ int yswz(int r, int c) { return c ^ ((r >> 1) & 7); }

typedef short v4i16 __attribute__((ext_vector_type(4)));

// One thread's loads of a step: 4 x 16 bytes of dY (chunk t % 8 of rows
// t / 8 + 64 i), and for weight rows 2p, 2p + 1 of the step (p = t % 32)
// the code dword of columns 8 cq .. 8 cq + 7 (cq = t / 32) with its group's
// scale (NF4: fp32 bits, INT4: fp16 bits, NF4_DQ: the 8-bit code) and
// zero-point byte (asym) or run constant (NF4_DQ).
struct DxLoads {
    u32x4 y[4];
    u32x2 c;
    uint32_t s, z;
    int zsh;
};

struct DxCtx {
    // dY: the tile's rows, as base and length (a step's column offset moves
    // the view: the buffer unit range-checks the lane's offset only, not a
    // load's soffset)
    const char *yb;
    uint32_t ybytes;
    __amdgpu_buffer_rsrc_t cr, sr, zr;
    int N, K, G, gshift;
    int p, cq;
};

template <int FMT>
__device__ __forceinline__ void dx_load(DxLoads &ld, const DxCtx &c, int n0_, int k0)
{
    // (the step is wave-uniform; said so, or the compiler may wrap the loads
    // in a loop over the lanes' values of their scalar offset)
    const int n0 = __builtin_amdgcn_readfirstlane(n0_);
    const int t = threadIdx.x;
    // dY: elements n0 + 8 (t % 8) .. + 7 of rows t / 8 + 64 i of the tile,
    // 8 lanes to a row, so that each 16-byte LDS store instruction fills 8
    // whole rows (rows past M and elements past the buffer read zeros;
    // elements past N of a row read the next row, which meets zero weights)
    const uint32_t yoff = 2u * (uint32_t)n0;
    const __amdgpu_buffer_rsrc_t yr = dx_rsrc(c.yb + yoff, yoff < c.ybytes ? c.ybytes - yoff : 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int yrow = (t >> 3) + 64 * i;
        ld.y[i] = __builtin_amdgcn_raw_buffer_load_b128(yr, 2 * (yrow * c.N + 8 * (t & 7)), 0, 0);
    }
    // weights: row n0 + t / 8 of the step, columns k0 + 16 (t % 8) .. + 15
    // (8 lanes read a row's 64 bytes of the tile together).  Rows past N
    // are clamped to row N: every offset then lies at or past the end of its
    // view, so codes and scales read zero (no selects, which the compiler
    // would turn into branches and full load waits).
    const int n = min(n0 + (t >> 3), c.N);
    const int k = k0 + 16 * (t & 7);
    ld.c = __builtin_amdgcn_raw_buffer_load_b64(c.cr, n * (c.K >> 1) + (k >> 1), 0, 0);
    const int gi = n * c.G + (k >> c.gshift);  // flat group index of the 16 columns
    if constexpr (f32_absmax(FMT)) {
        ld.s = __builtin_amdgcn_raw_buffer_load_b32(c.sr, 4 * gi, 0, 0);
    } else if constexpr (FMT == Q4_NF4_DQ) {
        ld.s = __builtin_amdgcn_raw_buffer_load_b8(c.sr, gi, 0, 0);
        ld.z = __builtin_amdgcn_raw_buffer_load_b32(c.zr, 4 * (gi >> 8), 0, 0);
    } else {
        ld.s = __builtin_amdgcn_raw_buffer_load_b16(c.sr, 2 * gi, 0, 0);
    }
    if constexpr (FMT == Q4_INT4_ASYM) {
        // the byte as loaded (no arithmetic on a load in flight) and the
        // nibble's position
        ld.z = __builtin_amdgcn_raw_buffer_load_b8(c.zr, gi >> 1, 0, 0);
        ld.zsh = 4 * (gi & 1);
    }
}

// Byte offset in a staged weight tile of element (row nl, column kl): rows
// of 288 bytes (72 dwords: the 4 rows a transposed read takes fall in
// distinct banks), the two 128-byte halves swapped on rows with bit 3 set
// (so that the next group of 8 rows uses the other banks).
__device__ __forceinline__ int wofs(int nl, int kl) { return nl * kWPitch + ((2 * kl) ^ (((nl >> 3) & 1) << 7)); }

template <int FMT, int ACT>
__global__ __launch_bounds__(kBlock) void gemm_dx_kernel(const uint16_t *__restrict__ dy, int M,
                                                         const uint8_t *__restrict__ codes,
                                                         const void *__restrict__ scales,
                                                         const uint8_t *__restrict__ zeros, int N,
                                                         int K, int gshift, int mtiles,
                                                         uint16_t *__restrict__ dx)
{
    __shared__ __attribute__((aligned(16))) char ys[2][TM * kYRow];
    __shared__ __attribute__((aligned(16))) char wt[2][TN * kWPitch];
    __shared__ float2 ptbl[level_fmt(FMT) == Q4_NF4 ? 256 : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int fi = lane & 15, fq = lane >> 4;
    const int m0 = (int)(blockIdx.x % (unsigned)mtiles) * TM;
    const int k0 = (int)(blockIdx.x / (unsigned)mtiles) * TK;
    constexpr int ss = f32_absmax(FMT) ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);

    if constexpr (level_fmt(FMT) == Q4_NF4) {
        if (t < 256)
            ptbl[t] = float2{level_entry<FMT>(t & 15), level_entry<FMT>(t >> 4)};
    }

    DxCtx c;
    c.N = N;
    c.K = K;
    c.G = K >> gshift;
    c.gshift = gshift;
    c.p = t & 31;
    c.cq = t >> 5;
    const int64_t ngroups = (int64_t)N * c.G;
    const int mrows = M - m0 < TM ? M - m0 : TM;
    c.yb = (const char *)(dy + (int64_t)m0 * N);
    c.ybytes = (uint32_t)((int64_t)mrows * N * 2 > 0x7fffffffll ? 0x7fffffffll : (int64_t)mrows * N * 2);
    c.cr = dx_rsrc(codes, (int64_t)N * (K >> 1));
    // scales: exactly the meaningful entries (an index at or past the end
    // reads zero); NF4_DQ: the 8-bit codes, and zr the run constants
    c.sr = dx_rsrc(scales, ngroups * ss);
    if constexpr (FMT == Q4_NF4_DQ)
        c.zr = dx_rsrc((const char *)scales + dq_s2_offset(ngroups),
                       4 * ((ngroups + kDqRun - 1) / kDqRun));
    else
        c.zr = FMT == Q4_INT4_ASYM ? dx_rsrc(zeros, (ngroups + 1) / 2) : c.cr;

    // waves: 2 along k (64 columns each) x 4 along m (64 rows each)
    const int wk = wave & 1, wm = wave >> 1;
    f32x4 acc[kKF][kWMF];
#pragma unroll
    for (int j = 0; j < kKF; ++j)
#pragma unroll
        for (int f = 0; f < kWMF; ++f)
            acc[j][f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // One round: the products of the step in LDS buffer (ysc, wtc), with the
    // staging of the next step (register set ld -> buffer (ysn, wtn)) worked
    // in between the matrix-core instructions, then the loads of a later
    // step into ld.  Scheduling fences keep that order: the two waves of a
    // SIMD run in step (one barrier per round), so staging that is not
    // interleaved leaves the matrix cores idle.
    auto round = [&](const char *ysc, const char *wtc, char *ysn, char *wtn, DxLoads &ld,
                     int next_n0) {
        u32x4 fa[kKF], fb[kWMF];
        auto reads = [&](int h) {
            // A operand (8 rows n = 32 h + 8 fq + 0..7 at column k of the
            // fragment, for lane (k = fi, fq)) by two transposed reads: in
            // each 16-lane group, result lane i takes element i % 4 of the
            // 4-element row piece addressed by lane 4 e + i / 4 (e the
            // result element); so lane s addresses row 8 fq + 4 u + s / 4,
            // columns 4 (s % 4) .. + 3 of the fragment.
#pragma unroll
            for (int j = 0; j < kKF; ++j) {
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    const int nl = 32 * h + 8 * fq + 4 * u + (fi >> 2);
                    const int kl = 64 * wk + 16 * j + 4 * (fi & 3);
                    const v4i16 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                        (__attribute__((address_space(3))) v4i16 *)(wtc + wofs(nl, kl)));
                    fa[j][2 * u] = (uint32_t)(uint16_t)r[0] | ((uint32_t)(uint16_t)r[1] << 16);
                    fa[j][2 * u + 1] = (uint32_t)(uint16_t)r[2] | ((uint32_t)(uint16_t)r[3] << 16);
                }
            }
#pragma unroll
            for (int f = 0; f < kWMF; ++f) {
                const int r = 64 * wm + 16 * f + fi;
                fb[f] = *(const u32x4 *)(ysc + r * kYRow + 16 * yswz(r, 4 * h + fq));
            }
        };
        auto mfmas = [&](int j) {
#pragma unroll
            for (int f = 0; f < kWMF; ++f)
                acc[j][f] = mfma<ACT>(fa[j], fb[f], acc[j][f]);
        };
        // the weight row piece of the next step: 16 columns of row t / 8,
        // dequantized (pairs along k, as q4_dequantize writes them) and
        // written as two 16-byte pieces
        u32x4 wv[2];
        auto dequant = [&](int e) {
            float sc, bias = 0.0f;
            if constexpr (f32_absmax(FMT)) {
                sc = std::bit_cast<float>(ld.s);
            } else if constexpr (FMT == Q4_NF4_DQ) {
                sc = keep_f32((float)(ld.s & 0xffu) * std::bit_cast<float>(ld.z));
            } else {
                sc = h2f(ld.s & 0xffffu);
                bias = FMT == Q4_INT4_SYM ? -8.0f * sc : -(float)((ld.z >> ld.zsh) & 0xfu) * sc;
            }
            float2 lp[4];
            if constexpr (level_fmt(FMT) == Q4_NF4) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lp[i] = ptbl[(ld.c[e] >> (8 * i)) & 0xffu];
            }
            wv[e] = dequant8<FMT, ACT>(ld.c[e], sc, bias, lp);
        };
        auto wwrite = [&](int e) {
            *(u32x4 *)(wtn + wofs(t >> 3, 16 * (t & 7) + 8 * e)) = wv[e];
        };

        reads(0);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < kKF; ++j) {
            mfmas(j);
            // dY of the next step, one 16-byte piece per group of MFMAs
            const int yr = (t >> 3) + 64 * j;
            *(u32x4 *)(ysn + yr * kYRow + 16 * yswz(yr, t & 7)) = ld.y[j];
            __builtin_amdgcn_sched_barrier(0);
        }
        reads(1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(0);
        dequant(0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(1);
        dequant(1);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(2);
        wwrite(0);
        __builtin_amdgcn_sched_barrier(0);
        mfmas(3);
        wwrite(1);
        __builtin_amdgcn_sched_barrier(0);
        dx_load<FMT>(ld, c, next_n0, k0);
        __syncthreads();
    };

    // Software pipeline: LDS double-buffered (one barrier per step), and two
    // steps of loads in flight in registers.  On entry to the round of step
    // s, buffer s & 1 holds step s, one register set step s + 1 and the
    // other step s + 2.  Loads of steps past the end read zeros (rows
    // clamped) or unused data; the buffers they fill are never computed.
    const int nsteps = (N + TN - 1) / TN;
    DxLoads la, lb;
    dx_load<FMT>(la, c, 0, k0);
    dx_load<FMT>(lb, c, TN, k0);
    __syncthreads();  // the level-pair table
    {
        // step 0 into buffer 0 (no products yet)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int yr = (t >> 3) + 64 * i;
            *(u32x4 *)(ys[0] + yr * kYRow + 16 * yswz(yr, t & 7)) = la.y[i];
        }
        float sc, bias = 0.0f;
        if constexpr (f32_absmax(FMT)) {
            sc = std::bit_cast<float>(la.s);
        } else if constexpr (FMT == Q4_NF4_DQ) {
            sc = keep_f32((float)(la.s & 0xffu) * std::bit_cast<float>(la.z));
        } else {
            sc = h2f(la.s & 0xffffu);
            bias = FMT == Q4_INT4_SYM ? -8.0f * sc : -(float)((la.z >> la.zsh) & 0xfu) * sc;
        }
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            float2 lp[4];
            if constexpr (level_fmt(FMT) == Q4_NF4) {
#pragma unroll
                for (int i = 0; i < 4; ++i)
                    lp[i] = ptbl[(la.c[e] >> (8 * i)) & 0xffu];
            }
            *(u32x4 *)(wt[0] + wofs(t >> 3, 16 * (t & 7) + 8 * e)) = dequant8<FMT, ACT>(la.c[e], sc, bias, lp);
        }
    }
    dx_load<FMT>(la, c, 2 * TN, k0);
    __syncthreads();
    for (int st = 0; st < nsteps; st += 2) {
        round(ys[0], wt[0], ys[1], wt[1], lb, (st + 3) * TN);  // step st; stages st + 1
        if (st + 1 >= nsteps)
            break;
        round(ys[1], wt[1], ys[0], wt[0], la, (st + 4) * TN);  // step st + 1; stages st + 2
    }

    // lane (fi, fq) of fragment (j, f) holds
    // dX[m0 + 64 wm + 16 f + fi][k0 + 64 wk + 16 j + 4 fq + v]
#pragma unroll
    for (int j = 0; j < kKF; ++j) {
        const int k = k0 + 64 * wk + 16 * j + 4 * fq;
        if (k < K) {
#pragma unroll
            for (int f = 0; f < kWMF; ++f) {
                const int m = m0 + 64 * wm + 16 * f + fi;
                if (m < M)
                    *(u32x2 *)(dx + (int64_t)m * K + k) = u32x2{
                        pack2<ACT>(acc[j][f][0], acc[j][f][1]), pack2<ACT>(acc[j][f][2], acc[j][f][3])};
            }
        }
    }
}

template <int FMT>
hipError_t launch_dx_fmt(q4_dtype act_t, int gshift, const void *dy, int64_t M,
                         const uint8_t *codes, const void *scales, const uint8_t *zeros, int64_t N,
                         int64_t K, void *dx, hipStream_t s)
{
    const int mtiles = (int)((M + TM - 1) / TM);
    const int64_t ktiles = (K + TK - 1) / TK;
    const dim3 grid((unsigned)(mtiles * ktiles)), block(kBlock);
    if (act_t == Q4_BF16)
        hipLaunchKernelGGL((gemm_dx_kernel<FMT, Q4_BF16>), grid, block, 0, s, (const uint16_t *)dy,
                           (int)M, codes, scales, zeros, (int)N, (int)K, gshift, mtiles,
                           (uint16_t *)dx);
    else
        hipLaunchKernelGGL((gemm_dx_kernel<FMT, Q4_F16>), grid, block, 0, s, (const uint16_t *)dy,
                           (int)M, codes, scales, zeros, (int)N, (int)K, gshift, mtiles,
                           (uint16_t *)dx);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_dx(q4_format f, int g, q4_dtype act_t, const void *dy, int64_t M,
                          const uint8_t *codes, const void *scales, const uint8_t *zeros,
                          int64_t N, int64_t K, void *dx, hipStream_t s)
{
    const int gshift = g == 32 ? 5 : (g == 64 ? 6 : 7);
    switch (f) {
    case Q4_NF4:
        return launch_dx_fmt<Q4_NF4>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    case Q4_FP4:
        return launch_dx_fmt<Q4_FP4>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    case Q4_NF4_DQ:
        return launch_dx_fmt<Q4_NF4_DQ>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    case Q4_INT4_SYM:
        return launch_dx_fmt<Q4_INT4_SYM>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    default:
        return launch_dx_fmt<Q4_INT4_ASYM>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    }
}

}  // namespace q4
