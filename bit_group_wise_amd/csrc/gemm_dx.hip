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
//  * The contraction runs over the weight's rows (N), so a matrix-core lane,
//    which needs 8 consecutive contraction values, would need 8 rows of the
//    packed layout.  The weight tile of a step (64 rows x 128 columns) is
//    therefore dequantized into LDS transposed: entry (k, n) of a row of
//    What^T holds weights n and n + 1 as a 16-bit pair.  A thread
//    dequantizes one code dword (8 columns) of two adjacent rows and writes
//    8 pairs; with a 144-byte row pitch both these writes and the 16-byte
//    fragment reads are free of bank conflicts.
//  * dY (the other operand, contiguous along N) is staged per step like the
//    forward product's activations: 256 rows x 128 bytes with the 16-byte
//    chunks of a row XOR-swizzled.
//  * A workgroup of 8 waves computes a 256 x 128 tile of dX; wave w owns
//    columns 16 w .. 16 w + 15 against all 256 rows (16 accumulators).
//  * The next step's loads (dY, codes, scales) are issued before the current
//    step's matrix-core work and written to LDS after it, so HBM/L2 latency
//    hides behind the MFMAs.
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
constexpr int kWPitch = TN * 2 + 16;   // bytes of one staged What^T row
constexpr int kMF = TM / 16;           // m fragments per wave

static_assert(TK == 16 * kWaves, "one 16-column fragment per wave");
static_assert(TN * TK / 16 == kBlock, "one code dword of two rows per thread");

__device__ __forceinline__ __amdgpu_buffer_rsrc_t dx_rsrc(const void *base, int64_t bytes)
{
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             0x00020000);
}

// Position of 16-byte chunk c of staged dY row r.
__device__ __forceinline__ int yswz(int r, int c) { return c ^ ((r >> 1) & 7); }

// One thread's loads of a step: 4 x 16 bytes of dY (row t / 2, chunks
// 4 (t & 1) .. + 3), and for weight rows 2p, 2p + 1 of the step (p = t % 32)
// the code dword of columns 8 cq .. 8 cq + 7 (cq = t / 32) with its group's
// scale (NF4: fp32 bits, INT4: fp16 bits, NF4_DQ: the 8-bit code) and
// zero-point byte (asym) or run constant (NF4_DQ).
struct DxLoads {
    u32x4 y[4];
    uint32_t c[2], s[2], z[2];
};

struct DxCtx {
    __amdgpu_buffer_rsrc_t yr, cr, sr, zr;
    int N, K, G, gshift;
    int p, cq;
};

template <int FMT>
__device__ __forceinline__ void dx_load(DxLoads &ld, const DxCtx &c, int n0, int k0)
{
    const int t = threadIdx.x;
    // dY: elements n0 + 8 chunk .. of row t / 2 of the tile (rows past M and
    // elements past the buffer read zeros; elements past N of a row read the
    // next row, which meets zero weights)
    const int yrow = t >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ch = 4 * (t & 1) + i;
        ld.y[i] = __builtin_amdgcn_raw_buffer_load_b128(c.yr, 2 * (yrow * c.N + 8 * ch), 2 * n0, 0);
    }
#pragma unroll
    for (int e = 0; e < 2; ++e) {
        // rows past N are clamped to row N: every offset then lies at or
        // past the end of its view, so codes and scales read zero (no
        // selects, which the compiler would turn into branches and full
        // load waits)
        const int n = min(n0 + 2 * c.p + e, c.N);
        const int k = k0 + 8 * c.cq;
        ld.c[e] = __builtin_amdgcn_raw_buffer_load_b32(c.cr, n * (c.K >> 1) + (k >> 1), 0, 0);
        const int gi = n * c.G + (k >> c.gshift);  // flat group index
        if constexpr (FMT == Q4_NF4) {
            ld.s[e] = __builtin_amdgcn_raw_buffer_load_b32(c.sr, 4 * gi, 0, 0);
        } else if constexpr (FMT == Q4_NF4_DQ) {
            ld.s[e] = __builtin_amdgcn_raw_buffer_load_b8(c.sr, gi, 0, 0);
            ld.z[e] = __builtin_amdgcn_raw_buffer_load_b32(c.zr, 4 * (gi >> 8), 0, 0);
        } else {
            ld.s[e] = __builtin_amdgcn_raw_buffer_load_b16(c.sr, 2 * gi, 0, 0);
        }
        if constexpr (FMT == Q4_INT4_ASYM)
            ld.z[e] = __builtin_amdgcn_raw_buffer_load_b8(c.zr, gi >> 1, 0, 0) >> (4 * (gi & 1));
    }
}

template <int FMT, int ACT>
__global__ __launch_bounds__(kBlock) void gemm_dx_kernel(const uint16_t *__restrict__ dy, int M,
                                                         const uint8_t *__restrict__ codes,
                                                         const void *__restrict__ scales,
                                                         const uint8_t *__restrict__ zeros, int N,
                                                         int K, int gshift, int mtiles,
                                                         uint16_t *__restrict__ dx)
{
    __shared__ __attribute__((aligned(16))) char ys[TM * kYRow];
    __shared__ __attribute__((aligned(16))) char wt[TK * kWPitch];
    __shared__ float2 ptbl[level_fmt(FMT) == Q4_NF4 ? 256 : 1];

    const int t = threadIdx.x;
    const int lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int fi = lane & 15, fq = lane >> 4;
    const int m0 = (int)(blockIdx.x % (unsigned)mtiles) * TM;
    const int k0 = (int)(blockIdx.x / (unsigned)mtiles) * TK;
    constexpr int ss = FMT == Q4_NF4 ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);

    if constexpr (level_fmt(FMT) == Q4_NF4) {
        if (t < 256)
            ptbl[t] = float2{kNF4[t & 15], kNF4[t >> 4]};
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
    c.yr = dx_rsrc(dy + (int64_t)m0 * N, (int64_t)mrows * N * 2);
    c.cr = dx_rsrc(codes, (int64_t)N * (K >> 1));
    // scales: exactly the meaningful entries (an index at or past the end
    // reads zero); NF4_DQ: the 8-bit codes, and zr the run constants
    c.sr = dx_rsrc(scales, ngroups * ss);
    if constexpr (FMT == Q4_NF4_DQ)
        c.zr = dx_rsrc((const char *)scales + dq_s2_offset(ngroups),
                       4 * ((ngroups + kDqRun - 1) / kDqRun));
    else
        c.zr = FMT == Q4_INT4_ASYM ? dx_rsrc(zeros, (ngroups + 1) / 2) : c.cr;

    f32x4 acc[kMF];
#pragma unroll
    for (int f = 0; f < kMF; ++f)
        acc[f] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    DxLoads ld;
    dx_load<FMT>(ld, c, 0, k0);
    for (int n0 = 0; n0 < N; n0 += TN) {
        __syncthreads();  // the previous step's fragment reads are done (and the table is in)
        // dY of this step into LDS
        {
            const int r = t >> 1;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                *(u32x4 *)(ys + r * kYRow + 16 * yswz(r, 4 * (t & 1) + i)) = ld.y[i];
        }
        // the weight tile, dequantized and transposed: column 8 cq + i of
        // rows 2p, 2p + 1 -> the pair at What^T row 8 cq + i, entry p
        {
            float v[2][8];
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                float s, b = 0.0f;
                if constexpr (FMT == Q4_NF4) {
                    s = std::bit_cast<float>(ld.s[e]);
                } else if constexpr (FMT == Q4_NF4_DQ) {
                    s = keep_f32((float)(ld.s[e] & 0xffu) * std::bit_cast<float>(ld.z[e]));
                } else {
                    s = h2f(ld.s[e] & 0xffffu);
                    b = FMT == Q4_INT4_SYM ? -8.0f * s : -(float)(ld.z[e] & 0xfu) * s;
                }
                float2 lp[4];
                if constexpr (level_fmt(FMT) == Q4_NF4) {
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        lp[i] = ptbl[(ld.c[e] >> (8 * i)) & 0xffu];
                }
                dequant8_f32<FMT>(ld.c[e], s, b, lp, v[e]);
            }
#pragma unroll
            for (int i = 0; i < 8; ++i)
                *(uint32_t *)(wt + (8 * c.cq + i) * kWPitch + 4 * c.p) = pack2<ACT>(v[0][i], v[1][i]);
        }
        __syncthreads();
        // the next step's loads, in flight during this step's products
        if (n0 + TN < N)
            dx_load<FMT>(ld, c, n0 + TN, k0);
        // dX[16 f + fi][16 wave + 4 fq + v] += sum over the step's 64 rows
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const u32x4 a = *(const u32x4 *)(wt + (16 * wave + fi) * kWPitch + 64 * h + 16 * fq);
#pragma unroll
            for (int f = 0; f < kMF; ++f) {
                const int r = 16 * f + fi;
                const u32x4 bv = *(const u32x4 *)(ys + r * kYRow + 16 * yswz(r, 4 * h + fq));
                acc[f] = mfma<ACT>(a, bv, acc[f]);
            }
        }
    }

    // lane (fi, fq) of fragment f holds dX[m0 + 16 f + fi][k0 + 16 wave + 4 fq + v]
    const int k = k0 + 16 * wave + 4 * fq;
    if (k < K) {
#pragma unroll
        for (int f = 0; f < kMF; ++f) {
            const int m = m0 + 16 * f + fi;
            if (m < M)
                *(u32x2 *)(dx + (int64_t)m * K + k) =
                    u32x2{pack2<ACT>(acc[f][0], acc[f][1]), pack2<ACT>(acc[f][2], acc[f][3])};
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
    case Q4_NF4_DQ:
        return launch_dx_fmt<Q4_NF4_DQ>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    case Q4_INT4_SYM:
        return launch_dx_fmt<Q4_INT4_SYM>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    default:
        return launch_dx_fmt<Q4_INT4_ASYM>(act_t, gshift, dy, M, codes, scales, zeros, N, K, dx, s);
    }
}

}  // namespace q4
