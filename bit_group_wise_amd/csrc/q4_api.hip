// q4_api.hip -- the C ABI of libq4 (declared in include/q4.h): host-side
// argument validation, status mapping and dispatch to the kernel launchers.
// Every check runs before the first HIP call, so a bad argument never reaches
// the runtime and the checks can be exercised on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>

#include "q4.h"
#include "q4_common.hpp"
#include "q4_internal.hpp"

#ifndef Q4_GEMM_BN128_MAX_M
#define Q4_GEMM_BN128_MAX_M 512
#endif
#ifndef Q4_GEMM_SKINNY_MAX_M
#define Q4_GEMM_SKINNY_MAX_M 96
#endif

// The sync words of q4_gemv_chain_static: one chain's finished-workgroup
// count, timeout flag and grid-barrier words (Q4_GEMV_CHAIN_SYNC_BYTES),
// in static device memory that each GPU holds for the life of the process.
// In host code this name is not a device address; the address of each
// device's copy comes from hipGetSymbolAddress.
static __device__ __align__(256) uint32_t scratch[Q4_GEMV_CHAIN_SYNC_BYTES / 4];

namespace {

// Device address of `scratch` on each device, looked up once per device
// with that device current (every GPU holds its own copy at its own
// address).
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint32_t *g_scratch_ptr[kMaxDevices] = {};

hipError_t scratch_for_current_device(uint32_t **out)
{
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return e;
    if (dev < 0 || dev >= kMaxDevices)
        return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return e;
        g_scratch_ptr[dev] = (uint32_t *)p;
    }
    *out = g_scratch_ptr[dev];
    return hipSuccess;
}

bool format_ok(q4_format f)
{
    return f == Q4_NF4 || f == Q4_INT4_SYM || f == Q4_INT4_ASYM || f == Q4_NF4_DQ || f == Q4_FP4;
}
bool dtype_ok(q4_dtype t) { return t == Q4_F16 || t == Q4_BF16; }
bool group_ok(int g) { return g == 32 || g == 64 || g == 128; }
bool aligned(const void *p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// Checks shared by every entry point that takes a quantized weight.
q4_status check_weight(q4_format f, int g, const void *codes, const void *scales,
                       const void *zeros, int64_t N, int64_t K)
{
    if (!format_ok(f) || !group_ok(g))
        return Q4_EUNSUPPORTED;
    if (!codes || !scales)
        return Q4_EINVAL;
    if (N <= 0 || K <= 0 || K % g != 0)
        return Q4_EINVAL;
    if ((f == Q4_INT4_ASYM) != (zeros != nullptr))
        return Q4_EINVAL;
    const uintptr_t sa = f == Q4_NF4_DQ ? 16 : (q4::f32_absmax(f) ? 4 : 2);
    if (!aligned(codes, 16) || !aligned(scales, sa))
        return Q4_EALIGN;
    return Q4_OK;
}

q4_status from_hip(hipError_t e) { return e == hipSuccess ? Q4_OK : Q4_EHIP; }

}  // namespace

extern "C" {

size_t q4_codes_bytes(int64_t N, int64_t K)
{
    if (N <= 0 || K <= 0 || K % 2 != 0)
        return 0;
    return (size_t)(N * K / 2);
}

// Scales and zero-points carry padding: the GEMM reads them with wide (up to
// 16-byte, unaligned) loads that may run past the last entry into it.
static size_t pad16(int64_t n) { return (size_t)q4::padded_meta_bytes(n); }

size_t q4_scales_bytes(q4_format f, int64_t N, int64_t K, int g)
{
    if (!format_ok(f) || !group_ok(g) || N <= 0 || K <= 0 || K % g != 0)
        return 0;
    if (f == Q4_NF4_DQ)
        return pad16(q4::dq_scales_bytes(N * (K / g)));
    return pad16(N * (K / g) * (q4::f32_absmax(f) ? 4 : 2));
}

size_t q4_zeros_bytes(q4_format f, int64_t N, int64_t K, int g)
{
    if (!format_ok(f) || !group_ok(g) || N <= 0 || K <= 0 || K % g != 0)
        return 0;
    if (f != Q4_INT4_ASYM)
        return 0;
    return pad16((N * (K / g) + 1) / 2);
}

const char *q4_status_str(q4_status s)
{
    switch (s) {
    case Q4_OK:
        return "ok";
    case Q4_EINVAL:
        return "invalid argument";
    case Q4_EUNSUPPORTED:
        return "unsupported format, dtype, group size or shape";
    case Q4_EALIGN:
        return "misaligned pointer";
    case Q4_EHIP:
        return "HIP runtime error";
    }
    return "unknown status";
}

q4_status q4_quantize(q4_format f, int g, const void *w_f16, int64_t N, int64_t K,
                      uint8_t *codes, void *scales, uint8_t *zeros, void *stream)
{
    q4_status st = check_weight(f, g, codes, scales, zeros, N, K);
    if (st != Q4_OK)
        return st;
    if (!w_f16)
        return Q4_EINVAL;
    if (!aligned(w_f16, 16))
        return Q4_EALIGN;
    return from_hip(q4::launch_quantize(f, g, w_f16, N, K, codes, scales, zeros,
                                        (hipStream_t)stream));
}

q4_status q4_dequantize(q4_format f, int g, const uint8_t *codes, const void *scales,
                        const uint8_t *zeros, int64_t N, int64_t K, q4_dtype out_t,
                        void *out, void *stream)
{
    q4_status st = check_weight(f, g, codes, scales, zeros, N, K);
    if (st != Q4_OK)
        return st;
    if (!dtype_ok(out_t))
        return Q4_EUNSUPPORTED;
    if (!out)
        return Q4_EINVAL;
    if (!aligned(out, 16))
        return Q4_EALIGN;
    return from_hip(q4::launch_dequantize(f, g, codes, scales, zeros, N, K, out_t, out,
                                          (hipStream_t)stream));
}

static q4_status check_product(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                               const uint8_t *codes, const void *scales, const uint8_t *zeros,
                               int64_t N, int64_t K, void *y)
{
    q4_status st = check_weight(f, g, codes, scales, zeros, N, K);
    if (st != Q4_OK)
        return st;
    if (!dtype_ok(act_t))
        return Q4_EUNSUPPORTED;
    if (!x || !y || M <= 0)
        return Q4_EINVAL;
    if (M > INT32_MAX || N > INT32_MAX || K > INT32_MAX)
        return Q4_EUNSUPPORTED;
    if (!aligned(x, 16) || !aligned(y, 2))
        return Q4_EALIGN;
    return Q4_OK;
}

q4_status q4_gemv(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                  const uint8_t *codes, const void *scales, const uint8_t *zeros,
                  int64_t N, int64_t K, void *y, void *stream)
{
    q4_status st = check_product(f, g, act_t, x, M, codes, scales, zeros, N, K, y);
    if (st != Q4_OK)
        return st;
    if (M > 16 || K > Q4_GEMV_MAX_K)
        return Q4_EUNSUPPORTED;
    return from_hip(q4::launch_gemv(f, g, act_t, x, M, codes, scales, zeros, N, K, y,
                                    (hipStream_t)stream));
}

q4_status q4_gemm(q4_format f, int g, q4_dtype act_t, const void *x, int64_t M,
                  const uint8_t *codes, const void *scales, const uint8_t *zeros,
                  int64_t N, int64_t K, void *y, void *stream)
{
    q4_status st = check_product(f, g, act_t, x, M, codes, scales, zeros, N, K, y);
    if (st != Q4_OK)
        return st;
    if (K > Q4_GEMM_MAX_K)
        return Q4_EUNSUPPORTED;
    // up to Q4_GEMM_SKINNY_MAX_M activation rows: the skinny product, 64
    // rows per launch (256-row tiles would leave most units idle)
    if (M <= Q4_GEMM_SKINNY_MAX_M)
        return from_hip(q4::launch_gemv_mfma(f, g, act_t, x, M, codes, scales, zeros, N, K, y,
                                             (hipStream_t)stream));
    // up to Q4_GEMM_BN128_MAX_M rows: tiles of 128 weight rows (twice the
    // workgroups of the 256-row tiles, which leave units idle below M = 1024)
    if (M <= Q4_GEMM_BN128_MAX_M)
        return from_hip(q4::launch_gemm_bn128(f, g, act_t, x, M, codes, scales, zeros, N, K, y,
                                              (hipStream_t)stream));
    return from_hip(q4::launch_gemm(f, g, act_t, x, M, codes, scales, zeros, N, K, y,
                                    (hipStream_t)stream));
}

q4_status q4_gemm_dx(q4_format f, int g, q4_dtype act_t, const void *dy, int64_t M,
                     const uint8_t *codes, const void *scales, const uint8_t *zeros,
                     int64_t N, int64_t K, void *dx, void *stream)
{
    q4_status st = check_product(f, g, act_t, dy, M, codes, scales, zeros, N, K, dx);
    if (st != Q4_OK)
        return st;
    if (N % 8 != 0 || N > Q4_GEMM_DX_MAX_N || N * (K / 2) > Q4_GEMV_CHAIN_MAX_CODES)
        return Q4_EUNSUPPORTED;
    if (!aligned(dx, 16))
        return Q4_EALIGN;
    return from_hip(q4::launch_gemm_dx(f, g, act_t, dy, M, codes, scales, zeros, N, K, dx,
                                       (hipStream_t)stream));
}

static q4_status check_chain(q4_format f, int g, q4_dtype act_t, const q4_gemv_task *tasks,
                             int ntasks)
{
    if (!format_ok(f) || !group_ok(g) || !dtype_ok(act_t))
        return Q4_EUNSUPPORTED;
    if (!tasks || ntasks <= 0)
        return Q4_EINVAL;
    if (ntasks > Q4_GEMV_CHAIN_MAX)
        return Q4_EUNSUPPORTED;
    for (int i = 0; i < ntasks; ++i) {
        const q4_gemv_task &t = tasks[i];
        q4_status st = check_product(f, g, act_t, t.x, 1, t.codes, t.scales, t.zeros, t.N, t.K,
                                     t.y);
        if (st != Q4_OK)
            return st;
        if ((t.flags & ~Q4_TASK_NO_WAIT) != 0)
            return Q4_EINVAL;
        if (t.K > Q4_GEMV_CHAIN_MAX_K || !q4::gemv_chain_k_ok(t.K))
            return Q4_EUNSUPPORTED;
        if (t.N * (t.K / 2) > Q4_GEMV_CHAIN_MAX_CODES)  // 32-bit offsets into one view
            return Q4_EUNSUPPORTED;
    }
    return Q4_OK;
}

q4_status q4_gemv_chain(q4_format f, int g, q4_dtype act_t, const q4_gemv_task *tasks,
                        int ntasks, uint32_t *sync, void *stream)
{
    if (!sync && format_ok(f) && group_ok(g) && dtype_ok(act_t))
        return Q4_EINVAL;
    q4_status st = check_chain(f, g, act_t, tasks, ntasks);
    if (st != Q4_OK)
        return st;
    if (!aligned(sync, 128))
        return Q4_EALIGN;
    return from_hip(q4::launch_gemv_chain(f, g, act_t, tasks, ntasks, sync, (hipStream_t)stream));
}

q4_status q4_gemv_chain_static(q4_format f, int g, q4_dtype act_t, const q4_gemv_task *tasks,
                               int ntasks, void *stream)
{
    q4_status st = check_chain(f, g, act_t, tasks, ntasks);
    if (st != Q4_OK)
        return st;
    uint32_t *sync = nullptr;
    if (scratch_for_current_device(&sync) != hipSuccess)
        return Q4_EHIP;
    // The kernel leaves every word but the timeout flag (word 2) at zero
    // when it ends, as static device memory starts; the timeout flag is
    // sticky and not reported here.
    return from_hip(q4::launch_gemv_chain(f, g, act_t, tasks, ntasks, sync, (hipStream_t)stream));
}

}  // extern "C"

int q4::device_cu_count()
{
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
        return 256;
    return cus;
}
