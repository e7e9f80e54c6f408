// KIVI residual-window cache for gfx950: the store half of an append.
//
// KIVI blog post on the fused Metal kernels, section "What we're actually
// optimizing", and the 0.8.0 release post, section "What KIVI is": the most
// recent tokens stay in 16-bit floats and are quantized as a batch (a
// flush) once they age out of the residual window.  The flush itself runs
// in the key and value quantizers (CacheRows layout); this file holds the
// copy of the appended tokens that stay unquantized into their ring slots.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

// One lane per 16-byte chunk of one appended token that stays unquantized,
// keys and values in one launch (a decode-time append is launch-bound):
// lanes are (tensor, bh, token j, chunk c) with c fastest, so a wave copies
// whole contiguous rows.  Token s = s_first + j is row s - T of the appended
// block and goes to slot s % ring_len.  The ring is read again by the next
// flush, so the stores are plain (cached) stores.
__global__ __launch_bounds__(256) void ring_store_kernel(
    const uint16_t* __restrict__ k_in, const uint16_t* __restrict__ v_in,
    uint16_t* __restrict__ k_ring, uint16_t* __restrict__ v_ring,
    uint32_t half, uint32_t D8, uint32_t ncopy, int32_t s_first, int32_t T,
    int32_t n_in, int32_t ring_len) {
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    if (gid >= 2u * half) return;
    const bool val = gid >= half;
    const uint32_t lid = val ? gid - half : gid;
    const uint32_t c = lid % D8;
    const uint32_t j = (lid / D8) % ncopy;
    const uint32_t bh = lid / (D8 * ncopy);
    const int32_t s = s_first + (int32_t)j;
    const int64_t D = (int64_t)D8 * 8;
    const uint16_t* in = val ? v_in : k_in;
    uint16_t* ring = val ? v_ring : k_ring;
    const uint4 v = load16_nt(in + ((int64_t)bh * n_in + (s - T)) * D + c * 8);
    *reinterpret_cast<uint4*>(ring + ((int64_t)bh * ring_len + s % ring_len) * D +
                              c * 8) = v;
}

hipError_t launch_ring_store(const void* k_in, const void* v_in, void* k_ring,
                             void* v_ring, int64_t BH, int64_t D, int64_t n_in,
                             int64_t T, int64_t s_first, int64_t ring_len,
                             hipStream_t stream) {
    const int64_t ncopy = T + n_in - s_first;
    const uint64_t half = (uint64_t)BH * ncopy * (D / 8);
    return launch_kernel(ring_store_kernel,
                         dim3((uint32_t)((2 * half + 255) / 256)), dim3(256), 0,
                         stream, static_cast<const uint16_t*>(k_in),
                         static_cast<const uint16_t*>(v_in),
                         static_cast<uint16_t*>(k_ring),
                         static_cast<uint16_t*>(v_ring), (uint32_t)half,
                         (uint32_t)(D / 8), (uint32_t)ncopy, (int32_t)s_first,
                         (int32_t)T, (int32_t)n_in, (int32_t)ring_len);
}

}  // namespace kivi
