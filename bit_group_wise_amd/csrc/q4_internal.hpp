// q4_internal.hpp -- launchers shared between the C-ABI front end
// (q4_api.hip) and the kernel files.  Arguments arrive validated.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

#include "q4.h"

namespace q4 {

// Number of compute units of the current device (queried per call).
int device_cu_count();

// Allocated size of a scale or zero-point array of n meaningful bytes: at
// least 16 bytes of padding, to a multiple of 16, so that loads of up to 16
// bytes starting at any meaningful byte stay inside the allocation.
__host__ __device__ constexpr int64_t padded_meta_bytes(int64_t n)
{
    return (n + 16 + 15) & ~(int64_t)15;
}

// NF4_DQ scales buffer: byte offset of the float32 second-level constants
// (one per kDqRun groups, flat order) after the n_groups 8-bit codes.
constexpr int kDqRun = 256;
__host__ __device__ constexpr int64_t dq_s2_offset(int64_t n_groups)
{
    return (n_groups + 15) & ~(int64_t)15;
}
__host__ __device__ constexpr int64_t dq_scales_bytes(int64_t n_groups)
{
    return dq_s2_offset(n_groups) + 4 * ((n_groups + kDqRun - 1) / kDqRun);
}

hipError_t launch_quantize(q4_format f, int g, const void *w, int64_t N, int64_t K,
                           uint8_t *codes, void *scales, uint8_t *zeros, hipStream_t s);
hipError_t launch_dequantize(q4_format f, int g, const uint8_t *codes, const void *scales,
                             const uint8_t *zeros, int64_t N, int64_t K, q4_dtype out_t,
                             void *out, hipStream_t s);
hipError_t launch_gemv(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                       const uint8_t *codes, const void *scales, const uint8_t *zeros,
                       int64_t N, int64_t K, void *y, hipStream_t s);
// Skinny product on the matrix cores: up to 64 activation rows per launch,
// more as consecutive launches over row slices.
hipError_t launch_gemv_mfma(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                            const uint8_t *codes, const void *scales, const uint8_t *zeros,
                            int64_t N, int64_t K, void *y, hipStream_t s);
// Chained M = 1 GEMVs (at most Q4_GEMV_CHAIN_MAX tasks per launch).
bool gemv_chain_k_ok(int64_t K);
hipError_t launch_gemv_chain(q4_format f, int g, q4_dtype act_t, const q4_gemv_task *tasks,
                             int ntasks, uint32_t *sync, hipStream_t s);
// Backward product dX = dY . What (QLoRA's gradient through the frozen weights).
hipError_t launch_gemm_dx(q4_format f, int g, q4_dtype act_t, const void *dy, int64_t M,
                          const uint8_t *codes, const void *scales, const uint8_t *zeros,
                          int64_t N, int64_t K, void *dx, hipStream_t s);
hipError_t launch_gemm(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                       const uint8_t *codes, const void *scales, const uint8_t *zeros,
                       int64_t N, int64_t K, void *y, hipStream_t s);
// The same with 128-row weight tiles (4 waves per workgroup), for middle M.
hipError_t launch_gemm_bn128(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                       const uint8_t *codes, const void *scales, const uint8_t *zeros,
                       int64_t N, int64_t K, void *y, hipStream_t s);

}  // namespace q4
