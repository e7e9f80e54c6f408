// KIVI residual-window cache for gfx950: the ring store of an append.
//
// KIVI blog post on the fused Metal kernels, section "What we're actually
// optimizing", and the 0.8.0 release post, section "What KIVI is": the most
// recent tokens stay in 16-bit floats and are quantized as a batch (a
// flush) once they age out of the residual window.  The flush itself runs
// in the key and value quantizers (CacheRows layout), with the copy of the
// appended tokens that stay unquantized into their ring slots in the same
// launch where it can (quant_values.hip, cache_append_kernel); this file
// holds the copy as a launch of its own.
#include "kivi_device.h"
#include "kivi_launch.h"
#include "kivi_rows.h"

namespace kivi {

// The ring store alone (an append that flushes nothing, or one whose flush
// reads ring slots the new tokens overwrite): RingStore::lane over
// 2 * half lanes, keys and values in one launch.
__global__ __launch_bounds__(256) void ring_store_kernel(RingStore r) {
    ring_store_lane(r, blockIdx.x * 256u + threadIdx.x);
}

RingStore make_ring_store(const void* k_in, const void* v_in, void* k_ring,
                          void* v_ring, int64_t BH, int64_t D, int64_t n_in,
                          int64_t T, int64_t s_first, int64_t ring_len) {
    const int64_t ncopy = T + n_in - s_first;
    return RingStore{static_cast<const uint16_t*>(k_in),
                     static_cast<const uint16_t*>(v_in),
                     static_cast<uint16_t*>(k_ring),
                     static_cast<uint16_t*>(v_ring),
                     (uint32_t)((uint64_t)BH * ncopy * (D / 8)),
                     (uint32_t)(D / 8), (uint32_t)ncopy, (int32_t)s_first,
                     (int32_t)T, (int32_t)n_in, (int32_t)ring_len};
}

hipError_t launch_ring_store(const RingStore& r, hipStream_t stream) {
    return launch_kernel(ring_store_kernel,
                         dim3((uint32_t)((2ull * r.half + 255) / 256)), dim3(256),
                         0, stream, r);
}

}  // namespace kivi
