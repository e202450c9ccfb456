// gemv_mfma.hip -- skinny product y[M, N] = x[M, K] . What^T for small M on
// the matrix cores (q4_gemv with 3 <= M <= 16, q4_gemm with M <= 96).
//
// Method ("Loading a model in 4-bit", "Where the accuracy goes"; "INT4
// Quantization > Practical Implementation with bitsandbytes"): the weights
// are dequantized to the 16-bit compute dtype (each value as q4_dequantize
// writes it) and multiplied with fp32 accumulation.  With a few activation
// rows the product still streams every weight byte once ("What is 4-bit
// quantization and why does it matter?", "Why it matters for deployment"),
// but the per-weight work grows with M, so from 3 rows on it runs here on
// v_mfma_f32_16x16x32 instead of the vector ALUs.
//
// gfx950 mapping:
//  * A workgroup owns RB blocks of 16 weight rows (one MFMA operand each)
//    and MT blocks of 16 activation rows (MT = 1, 2 or 4: up to 64 rows per
//    launch; each dequantized weight fragment feeds MT products); more rows
//    run as consecutive launches over row slices.  Its 8 waves split K into steps of
//    128, interleaved (wave w takes steps w, w + 8, ...).  A step's x
//    fragment serves all RB blocks, so each workgroup reads x once for RB
//    blocks; RB (1, 2 or 4) is the largest that still gives every compute
//    unit a workgroup.  (Without x loads at all, a timing-only variant ran
//    twice as fast at M = 16; halving them gained only 6 %: what the x loads
//    cost is mostly their latency in a pipeline of few steps per wave.)
//  * Lane (r, q) = (lane % 16, lane / 16) loads 16 bytes of codes: 32
//    weights of row r at k = k0 + 32 q.  Dword d of them is the lane's share
//    of MFMA d of the step, which therefore contracts over k0 + 32 q + 8 d
//    ... + 7 for lane quad q; the activation operand uses the same order, so
//    lane (m, q) loads x[m][k0 + 32 q ... + 31] as four 16-byte pieces.
//    Every load is contiguous; x rows past M and k past K are sent out of
//    range and read zeros.
//  * A 2-deep ring of steps keeps the next step's loads in flight.
//  * The 8 partial 16 x 16 tiles of each (row block, activation block) meet
//    in LDS and are summed in wave order (a fixed order, so the result does
//    not depend on timing).
//  * Double-quantized NF4 absmax: the lane loads its group's 8-bit code and
//    its run's binary32 constant and recovers the absmax with one product.
#include "q4_common.hpp"
#include "q4_internal.hpp"
#include "q4_mfma.hpp"

namespace q4 {
namespace {

constexpr int kSkWaves = 8;
constexpr int kSkBlock = 64 * kSkWaves;
constexpr int kSkStep = 128;  // k per step
constexpr int kSkMaxRows = 64;  // activation rows per launch (4 blocks of 16)
#ifndef Q4_SK_RING
#define Q4_SK_RING 2
#endif
constexpr int kSkRing = Q4_SK_RING;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t sk_rsrc(const void *base, int64_t bytes)
{
    const uint32_t n = bytes <= 0 ? 0u : (bytes >= 0x7fffffffll ? 0x7fffffffu : (uint32_t)bytes);
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, (int)n,
                                             0x00020000);
}

// One step's operands for a lane: for each of the RB row blocks, 32 codes
// and their group's scale (and asym zero-point, or NF4_DQ run constant);
// and 32 activations of one x row, shared by the blocks.
template <int FMT, int RB, int MT>
struct SkStep {
    u32x4 cw[RB];
    uint32_t sraw[RB];
    uint32_t zraw[RB];
    int zsh[RB];
    u32x4 xv[MT][4];
};

template <int FMT, int ACT, int RB, int MT>
__global__ __launch_bounds__(kSkBlock) void gemv_mfma_kernel(
    const uint16_t *__restrict__ x, int M, const uint8_t *__restrict__ codes,
    const void *__restrict__ scales, const uint8_t *__restrict__ zeros, int N, int K, int gshift,
    uint16_t *__restrict__ y)
{
    constexpr int LF = level_fmt(FMT);
    __shared__ float2 ptbl[LF == Q4_NF4 ? 256 : 1];
    __shared__ f32x4 part[kSkWaves][RB][MT][64];

    const int lane = threadIdx.x & 63;
    const int wave = (int)__builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int r = lane & 15, q = lane >> 4;
    const int n0 = blockIdx.x * 16 * RB;
    const int G = K >> gshift;
    const int row_bytes = K >> 1;
    constexpr int ss = f32_absmax(FMT) ? 4 : (FMT == Q4_NF4_DQ ? 1 : 2);

    if constexpr (LF == Q4_NF4) {
        if (threadIdx.x < 256)
            ptbl[threadIdx.x] = float2{level_entry<FMT>(threadIdx.x & 15), level_entry<FMT>(threadIdx.x >> 4)};
    }

    // views: this workgroup's 16 RB weight rows (rows past N read zeros) and
    // the M activation rows
    const int nrows = N - n0 < 16 * RB ? N - n0 : 16 * RB;
    const __amdgpu_buffer_rsrc_t cr = sk_rsrc(codes + (int64_t)n0 * row_bytes, (int64_t)nrows * row_bytes);
    const __amdgpu_buffer_rsrc_t sr =
        sk_rsrc((const char *)scales + (int64_t)n0 * G * ss, (int64_t)nrows * G * ss);
    const int64_t zg0 = (int64_t)n0 * G;  // flat group index of the first row's first group
    __amdgpu_buffer_rsrc_t zr = sr;
    if constexpr (FMT == Q4_INT4_ASYM)
        zr = sk_rsrc(zeros + (zg0 >> 1), (((int64_t)nrows * G + (zg0 & 1)) + 1) / 2);
    // double-quantized absmax: the runs' binary32 constants for the rows'
    // groups (zr then starts at the run holding the first group)
    if constexpr (FMT == Q4_NF4_DQ) {
        const float *s2 = (const float *)((const char *)scales + dq_s2_offset((int64_t)N * G));
        const int64_t r0 = zg0 / kDqRun, r1 = (zg0 + (int64_t)nrows * G - 1) / kDqRun;
        zr = sk_rsrc(s2 + r0, 4 * (r1 - r0 + 1));
    }
    const __amdgpu_buffer_rsrc_t xr = sk_rsrc(x, (int64_t)M * K * 2);

    const int nsteps = (K + kSkStep - 1) / kSkStep;
    auto load = [&](SkStep<FMT, RB, MT> &st, int step) {
        const int k = step * kSkStep + 32 * q;  // the lane's first k
        const bool in = step < nsteps && k < K;
#pragma unroll
        for (int b = 0; b < RB; ++b) {
            const int rr = 16 * b + r;  // the lane's weight row in the workgroup
            st.cw[b] = __builtin_amdgcn_raw_buffer_load_b128(cr, in ? rr * row_bytes + (k >> 1) : -16,
                                                             0, 0);
            const int gi = rr * G + (k >> gshift);  // group within the workgroup's rows
            if constexpr (f32_absmax(FMT))
                st.sraw[b] = __builtin_amdgcn_raw_buffer_load_b32(sr, in ? 4 * gi : -16, 0, 0);
            else if constexpr (FMT == Q4_NF4_DQ)
                st.sraw[b] = __builtin_amdgcn_raw_buffer_load_b8(sr, in ? gi : -16, 0, 0);
            else
                st.sraw[b] = __builtin_amdgcn_raw_buffer_load_b16(sr, in ? 2 * gi : -16, 0, 0);
            if constexpr (FMT == Q4_INT4_ASYM) {
                // the byte as loaded (no arithmetic on a load in flight) and
                // the nibble's position
                const int gz = (int)(zg0 & 1) + gi;
                st.zraw[b] = __builtin_amdgcn_raw_buffer_load_b8(zr, in ? gz >> 1 : -16, 0, 0);
                st.zsh[b] = 4 * (gz & 1);
            } else if constexpr (FMT == Q4_NF4_DQ) {
                const int gr = (int)(zg0 % kDqRun) + gi;  // group index from the first run's start
                st.zraw[b] =
                    __builtin_amdgcn_raw_buffer_load_b32(zr, in ? 4 * (gr / kDqRun) : -16, 0, 0);
            } else {
                st.zraw[b] = 0;
            }
        }
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = 16 * mt + r;  // the lane's activation row
            const bool xin = in && m < M;
#pragma unroll
            for (int d = 0; d < 4; ++d)
                st.xv[mt][d] = __builtin_amdgcn_raw_buffer_load_b128(
                    xr, xin ? 2 * (m * K + k + 8 * d) : -16, 0, 0);
        }
    };

    // the wave's steps: wave, wave + 8, ...
    SkStep<FMT, RB, MT> ring[kSkRing];
#pragma unroll
    for (int i = 0; i < kSkRing; ++i)
        load(ring[i], wave + kSkWaves * i);
    __syncthreads();  // the level-pair table

    f32x4 acc[RB][MT];
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            acc[b][mt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    for (int step = wave; step < nsteps; step += kSkWaves * kSkRing) {
#pragma unroll
        for (int i = 0; i < kSkRing; ++i) {
            SkStep<FMT, RB, MT> &st = ring[i];
            // a step past the end is not computed (its slot is still
            // refilled below, so the load waits stay partial)
#pragma unroll
            for (int b = 0; b < RB; ++b) {
                if (step + kSkWaves * i >= nsteps)
                    break;
                float s, bias;
                if constexpr (f32_absmax(FMT)) {
                    s = std::bit_cast<float>(st.sraw[b]);
                    bias = 0.0f;
                } else if constexpr (FMT == Q4_NF4_DQ) {  // c' = qc * s2, one product
                    s = keep_f32((float)st.sraw[b] * std::bit_cast<float>(st.zraw[b]));
                    bias = 0.0f;
                } else {
                    s = h2f(st.sraw[b] & 0xffffu);
                    bias = FMT == Q4_INT4_SYM ? -8.0f * s
                                              : -(float)((st.zraw[b] >> st.zsh[b]) & 0xfu) * s;
                }
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    float2 lp[4];
                    if constexpr (LF == Q4_NF4) {
#pragma unroll
                        for (int e = 0; e < 4; ++e)
                            lp[e] = ptbl[(st.cw[b][d] >> (8 * e)) & 0xffu];
                    }
                    const u32x4 wf = dequant8<FMT, ACT>(st.cw[b][d], s, bias, lp);
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        acc[b][mt] = mfma<ACT>(wf, st.xv[mt][d], acc[b][mt]);
                }
            }
            load(st, step + kSkWaves * (i + kSkRing));
        }
    }

    // sum the 8 partial tiles of each (row block, activation block) in wave
    // order; lane l holds rows 4 q + v of the row block against activation
    // row 16 mt + r
#pragma unroll
    for (int b = 0; b < RB; ++b)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
            part[wave][b][mt][lane] = acc[b][mt];
    __syncthreads();
    for (int t = wave; t < RB * MT; t += kSkWaves) {
        const int b = t / MT, mt = t % MT;
        f32x4 u0 = part[0][b][mt][lane];
#pragma unroll
        for (int w = 1; w < kSkWaves; ++w) {
            const f32x4 u = part[w][b][mt][lane];
            u0 = f32x4{u0[0] + u[0], u0[1] + u[1], u0[2] + u[2], u0[3] + u[3]};
        }
        const int m = 16 * mt + r;
        const int n = n0 + 16 * b + 4 * q;
        if (m < M) {
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                if (n + v < N)
                    y[(int64_t)m * N + n + v] =
                        (uint16_t)(ACT == Q4_BF16 ? f2bf_bits(u0[v]) : f2h_bits(u0[v]));
            }
        }
    }
}

template <int FMT, int RB, int MT>
hipError_t launch_sk_mt(q4_dtype act_t, const void *x, int M, const uint8_t *codes,
                        const void *scales, const uint8_t *zeros, int64_t N, int64_t K, int gshift,
                        void *y, hipStream_t s)
{
    const unsigned blocks = (unsigned)((N + 16 * RB - 1) / (16 * RB));
    if (act_t == Q4_BF16)
        hipLaunchKernelGGL((gemv_mfma_kernel<FMT, Q4_BF16, RB, MT>), dim3(blocks), dim3(kSkBlock),
                           0, s, (const uint16_t *)x, M, codes, scales, zeros, (int)N, (int)K,
                           gshift, (uint16_t *)y);
    else
        hipLaunchKernelGGL((gemv_mfma_kernel<FMT, Q4_F16, RB, MT>), dim3(blocks), dim3(kSkBlock),
                           0, s, (const uint16_t *)x, M, codes, scales, zeros, (int)N, (int)K,
                           gshift, (uint16_t *)y);
    return hipGetLastError();
}

// Activation blocks of 16 rows per launch: 1, 2 or 4 (M <= 16, 32, 64).
template <int FMT, int RB>
hipError_t launch_sk_rb(q4_dtype act_t, const void *x, int M, const uint8_t *codes,
                        const void *scales, const uint8_t *zeros, int64_t N, int64_t K, int gshift,
                        void *y, hipStream_t s)
{
    if (M <= 16)
        return launch_sk_mt<FMT, RB, 1>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    if (M <= 32)
        return launch_sk_mt<FMT, RB, 2>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    return launch_sk_mt<FMT, RB, 4>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
}

// Row blocks per workgroup: the blocks spread over the compute units
// (ceil(blocks / units), at most 4), so that no unit holds more than its
// share and x is read once for several blocks.  (With a number of
// workgroups between one and two per unit, the units holding two finish
// last: 688 blocks as 344 pairs ran a third longer than as 230 triples.)
template <int FMT>
hipError_t launch_sk_fmt(q4_dtype act_t, const void *x, int M, const uint8_t *codes,
                         const void *scales, const uint8_t *zeros, int64_t N, int64_t K,
                         int gshift, void *y, hipStream_t s)
{
    const int64_t nb = (N + 15) / 16;
    const int64_t cus = device_cu_count();
    const int64_t rb = (nb + cus - 1) / cus;
    if (rb >= 4)
        return launch_sk_rb<FMT, 4>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    if (rb == 3)
        return launch_sk_rb<FMT, 3>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    if (rb == 2)
        return launch_sk_rb<FMT, 2>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
    return launch_sk_rb<FMT, 1>(act_t, x, M, codes, scales, zeros, N, K, gshift, y, s);
}

}  // namespace

hipError_t launch_gemv_mfma(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                            const uint8_t *codes, const void *scales, const uint8_t *zeros,
                            int64_t N, int64_t K, void *y, hipStream_t s)
{
    const int gshift = g == 32 ? 5 : (g == 64 ? 6 : 7);
    // up to kSkMaxRows activation rows per launch; more run as consecutive
    // launches over row slices of x and y (each reads every weight once)
    for (int64_t m0 = 0; m0 < M; m0 += kSkMaxRows) {
        const int mc = (int)(M - m0 < kSkMaxRows ? M - m0 : kSkMaxRows);
        const void *xc = (const uint16_t *)x + m0 * K;
        void *yc = (uint16_t *)y + m0 * N;
        hipError_t e;
        switch (f) {
        case Q4_NF4:
            e = launch_sk_fmt<Q4_NF4>(act_t, xc, mc, codes, scales, zeros, N, K, gshift, yc, s);
            break;
        case Q4_FP4:
            e = launch_sk_fmt<Q4_FP4>(act_t, xc, mc, codes, scales, zeros, N, K, gshift, yc, s);
            break;
        case Q4_NF4_DQ:
            e = launch_sk_fmt<Q4_NF4_DQ>(act_t, xc, mc, codes, scales, zeros, N, K, gshift, yc, s);
            break;
        case Q4_INT4_SYM:
            e = launch_sk_fmt<Q4_INT4_SYM>(act_t, xc, mc, codes, scales, zeros, N, K, gshift, yc, s);
            break;
        default:
            e = launch_sk_fmt<Q4_INT4_ASYM>(act_t, xc, mc, codes, scales, zeros, N, K, gshift, yc, s);
            break;
        }
        if (e != hipSuccess)
            return e;
    }
    return hipSuccess;
}

}  // namespace q4
