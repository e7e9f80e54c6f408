// Device self-test of the two exact division shortcuts the quantizers rely
// on (see make_params in kivi_device.h), run on the GPU they execute on:
//  1. scale = Markstein quotient by the constant L = 2^bits - 1, against the
//     IEEE quotient range / L, for L in {1, 3, 15, 255} and every range
//     significand at every exponent of the fast range [2^-56, 2^56];
//  2. y = hardware reciprocal + one Newton step, against the IEEE 1 / scale,
//     for every significand at every exponent of [2^-64, 2^64).
// Every thread owns one significand and walks the exponents, so the grid is
// exactly 2^23 threads; mismatches are summed into one counter.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

template <int BITS>
__device__ __forceinline__ uint32_t scale_mismatch(float range) {
    constexpr float L = (float)((1 << BITS) - 1);
    constexpr float inv_L = 1.0f / L;
    const float q0 = range * inv_L;
    const float r = __builtin_fmaf(-q0, L, range);
    const float s = __builtin_fmaf(r, inv_L, q0);
    return __float_as_uint(s) != __float_as_uint(range / L);
}

__global__ __launch_bounds__(256) void selftest_division_kernel(
    unsigned long long* __restrict__ mismatches) {
    const uint32_t m = blockIdx.x * 256u + threadIdx.x;   // < 2^23
    uint32_t bad = 0;
    for (int e = -56; e <= 55; ++e) {
        const float range = __uint_as_float(((uint32_t)(127 + e) << 23) | m);
        bad += scale_mismatch<1>(range) + scale_mismatch<2>(range) +
               scale_mismatch<4>(range) + scale_mismatch<8>(range);
    }
    for (int e = -64; e <= 63; ++e) {
        const float s = __uint_as_float(((uint32_t)(127 + e) << 23) | m);
        const float y0 = __builtin_amdgcn_rcpf(s);
        const float er = __builtin_fmaf(-s, y0, 1.0f);
        const float y = __builtin_fmaf(er, y0, y0);
        bad += __float_as_uint(y) != __float_as_uint(1.0f / s);
    }
    if (bad) atomicAdd(mismatches, (unsigned long long)bad);
}

hipError_t launch_selftest_division(unsigned long long* mismatches,
                                    hipStream_t stream) {
    return launch_kernel(selftest_division_kernel, dim3((1u << 23) / 256),
                       dim3(256), 0, stream, mismatches);
}

}  // namespace kivi
