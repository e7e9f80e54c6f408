// Internal interface between the C ABI (kivi_api.cpp) and the kernel
// launchers.  Arguments are validated by the caller; launchers only choose a
// kernel and a grid and enqueue it on the given stream.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kivi {

// Events armed by kivi_time_next_launch for the calling thread's next
// launch; take_launch_events hands them over once and disarms them.
void take_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Every kernel of the library is launched through here: with armed events
// the launch records them at the dispatch's start and end
// (hipExtLaunchKernel), so they time the kernel alone.
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block,
                         uint32_t shmem, hipStream_t stream, Args... args) {
    hipEvent_t start = nullptr, stop = nullptr;
    take_launch_events(&start, &stop);
    if (start != nullptr && stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start, stop,
                              0, static_cast<Params>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream,
                           static_cast<Params>(args)...);
    return hipGetLastError();
}

// Smallest l with 2^l >= n (host-side launch helper).
inline uint32_t log2_ceil(uint64_t n) {
    uint32_t l = 0;
    while ((1ull << l) < n) ++l;
    return l;
}

struct QuantJob {
    const void* x;        // [BH, S, D] 16-bit input
    int dtype;            // 0 fp16, 1 bf16
    int64_t BH, S, D;
    int bits;
    int64_t group;
    uint8_t* codes;       // may be null only when recon-only
    float* scale;
    float* zero;
    void* recon;          // null unless fused; same dtype as x
    hipStream_t stream;
};

struct DequantJob {
    const uint8_t* codes;
    const float* scale;
    const float* zero;
    int64_t BH, S, D;
    int bits;
    int64_t group;
    int out_dtype;
    void* out;
    hipStream_t stream;
};

hipError_t launch_quant_keys(const QuantJob& j);
hipError_t launch_quant_values(const QuantJob& j);
hipError_t launch_dequant_keys(const DequantJob& j);
hipError_t launch_dequant_values(const DequantJob& j);

// Fallback kernels for shapes the fast kernels do not cover (keys with
// D % 8 != 0 or group > 32; values with D % 8 != 0, D > 512 or a group that
// is not 8 times a power of two; dequant with D % 8 != 0 or, for values,
// group % 8 != 0).
hipError_t launch_generic_quant_keys(const QuantJob& j);
hipError_t launch_generic_quant_values(const QuantJob& j);
hipError_t launch_generic_dequant(const DequantJob& j, bool keys);

hipError_t launch_selftest_division(unsigned long long* mismatches,
                                    hipStream_t stream);

}  // namespace kivi
