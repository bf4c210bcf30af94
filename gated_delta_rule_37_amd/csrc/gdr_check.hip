// gdr_check.hip -- the input checks of the debug mode (GDR_VALIDATE=1).
//
// The chunked kernels work with log2(alpha), so the gate must lie in (0, 1]
// (KDA blog, section 2.1, calls alpha a forget rate in [0, 1]; 0 has no
// logarithm).  For bf16 inputs the matrix-core operands are fp16 (the blog's
// section 2.2 only asks for "mixed precision"), so every value that becomes an
// fp16 operand or an fp16 snapshot must be below fp16's largest finite value,
// 65504, in magnitude.  NaN and Inf propagate silently in the normal mode.
//
// One launch per tensor: a grid-stride pass that records which rules failed
// (an OR of bits) and the smallest failing element index in a two-word result
// the host reads back.  Debug mode only; nothing here runs unless asked.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include "gdr_common.hpp"
#include "gdr_launch.hpp"

namespace gdr {

// [0]: OR of the failed rules' bits; [1]: smallest failing element index.
// Each GPU holds its own copy; the host takes its address per device with
// hipGetSymbolAddress and passes that address to the kernels.
__device__ __align__(16) unsigned long long check_result[2];

namespace {

__global__ void check_clear_kernel(unsigned long long* res) {
    if (threadIdx.x == 0) {
        res[0] = 0ull;
        res[1] = ~0ull;
    }
}

template <bool BF16>
__global__ void __launch_bounds__(256) check_kernel(const void* __restrict__ p, int64_t n, uint32_t rules,
                                                    unsigned long long* res) {
    uint32_t bad = 0;
    unsigned long long first = ~0ull;
    const int64_t stride = int64_t(gridDim.x) * blockDim.x;
    for (int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float x = BF16 ? bf16_to_f32(static_cast<const bf16_t*>(p)[i]) : static_cast<const float*>(p)[i];
        uint32_t b = 0;
        if ((rules & CHECK_FINITE) && !__builtin_isfinite(x)) b |= CHECK_FINITE;
        if ((rules & CHECK_FP16_RANGE) && !(__builtin_fabsf(x) < 65504.f)) b |= CHECK_FP16_RANGE;
        if ((rules & CHECK_ALPHA_OPEN) && !(x > 0.f && x <= 1.f)) b |= CHECK_ALPHA_OPEN;
        if ((rules & CHECK_ALPHA_CLOSED) && !(x >= 0.f && x <= 1.f)) b |= CHECK_ALPHA_CLOSED;
        if ((rules & CHECK_NONZERO) && x == 0.f) b |= CHECK_NONZERO;
        if (b) {
            bad |= b;
            if (static_cast<unsigned long long>(i) < first) first = static_cast<unsigned long long>(i);
        }
    }
    if (bad) {
        atomicOr(&res[0], static_cast<unsigned long long>(bad));
        atomicMin(&res[1], first);
    }
}

}  // namespace

hipError_t launch_check(const void* p, int64_t n, bool bf16, uint32_t rules, unsigned long long* res,
                        hipStream_t stream) {
    check_clear_kernel<<<1, 64, 0, stream>>>(res);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess || n <= 0) return e;
    int64_t blocks = (n + 255) / 256;
    if (blocks > 2048) blocks = 2048;
    if (bf16)
        check_kernel<true><<<dim3(uint32_t(blocks)), 256, 0, stream>>>(p, n, rules, res);
    else
        check_kernel<false><<<dim3(uint32_t(blocks)), 256, 0, stream>>>(p, n, rules, res);
    return hipGetLastError();
}

hipError_t check_result_address(unsigned long long** out) {
    return hipGetSymbolAddress(reinterpret_cast<void**>(out), HIP_SYMBOL(check_result));
}

}  // namespace gdr
