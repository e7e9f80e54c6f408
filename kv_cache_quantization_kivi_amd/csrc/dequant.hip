// KIVI dequantization for gfx950: recon = RN(RN(code * scale) + zero),
// narrowed to fp16/bf16 with round to nearest even (KIVI blog post on the
// fused Metal kernels, section "What we're actually optimizing", and "Three
// ways to be off by one bit", item 1: the product is rounded before the add).
//
// Keys: one lane owns an 8-channel chunk of one (bh, token group) tile, so
// its 8 scales and 8 zeros are loaded once (four 128-bit loads) and reused
// for every token of the group; each token then costs one BITS-byte code
// load and one 128-bit store.
// Values: one lane owns an 8-channel chunk of one row; the chunk lies in one
// group (group % 8 == 0), so it needs one scale and one zero.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kDqTokUnroll = 8;   // code loads in flight per lane (keys)
constexpr int kDqValItems = 4;    // chunks per lane (values)

template <int DT, int BITS>
__global__ __launch_bounds__(256) void dequant_keys_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint32_t n_items, uint32_t D8,
    uint32_t NG, int32_t S, int32_t G, uint16_t* __restrict__ out) {
    const uint32_t item = blockIdx.x * 256u + threadIdx.x;
    if (item >= n_items) return;
    const uint32_t c = item % D8;
    const uint32_t tile = item / D8;
    const uint32_t g = tile % NG;
    const uint32_t bh = tile / NG;
    const int32_t s0 = (int32_t)g * G;
    const int32_t nt = min(G, S - s0);
    const int64_t D = (int64_t)D8 * 8;
    const int64_t row0 = (int64_t)bh * S + s0;

    const int64_t p = ((int64_t)bh * NG + g) * D + (int64_t)c * 8;
    const float4 s_a = reinterpret_cast<const float4*>(scale + p)[0];
    const float4 s_b = reinterpret_cast<const float4*>(scale + p)[1];
    const float4 z_a = reinterpret_cast<const float4*>(zero + p)[0];
    const float4 z_b = reinterpret_cast<const float4*>(zero + p)[1];
    const float sc[8] = {s_a.x, s_a.y, s_a.z, s_a.w, s_b.x, s_b.y, s_b.z, s_b.w};
    const float z[8] = {z_a.x, z_a.y, z_a.z, z_a.w, z_b.x, z_b.y, z_b.z, z_b.w};

    const int64_t row_bytes = (int64_t)D8 * BITS;
    const uint8_t* src = codes + row0 * row_bytes + (int64_t)c * BITS;
    uint16_t* dst = out + row0 * D + (int64_t)c * 8;
    for (int32_t t0 = 0; t0 < nt; t0 += kDqTokUnroll) {
        uint64_t q[kDqTokUnroll];
#pragma unroll
        for (int u = 0; u < kDqTokUnroll; ++u)
            if (t0 + u < nt) q[u] = load_codes<BITS>(src + (t0 + u) * row_bytes);
#pragma unroll
        for (int u = 0; u < kDqTokUnroll; ++u)
            if (t0 + u < nt)
                *reinterpret_cast<uint4*>(dst + (int64_t)(t0 + u) * D) =
                    dequant_chunk<DT, BITS>(q[u], sc, z);
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(256) void dequant_values_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint64_t n_items, uint32_t D8,
    uint32_t G8, uint32_t NGD, uint16_t* __restrict__ out) {
    // Items (row, chunk) with the chunk fastest; a block covers
    // kDqValItems * 256 consecutive items, 256 per step, so each wave-wide
    // load and store is contiguous.
    const uint64_t base = (uint64_t)blockIdx.x * (256u * kDqValItems) +
                          threadIdx.x;
    uint64_t q[kDqValItems];
    float sc[kDqValItems], z[kDqValItems];
#pragma unroll
    for (int i = 0; i < kDqValItems; ++i) {
        const uint64_t item = base + (uint64_t)i * 256u;
        if (item < n_items) {
            const uint64_t row = item / D8;
            const uint32_t c = (uint32_t)(item - row * D8);
            q[i] = load_codes<BITS>(codes + item * BITS);
            const uint64_t pi = row * NGD + c / G8;
            sc[i] = scale[pi];
            z[i] = zero[pi];
        }
    }
#pragma unroll
    for (int i = 0; i < kDqValItems; ++i) {
        const uint64_t item = base + (uint64_t)i * 256u;
        if (item < n_items) {
            const float s8[8] = {sc[i], sc[i], sc[i], sc[i],
                                 sc[i], sc[i], sc[i], sc[i]};
            const float z8[8] = {z[i], z[i], z[i], z[i], z[i], z[i], z[i], z[i]};
            *reinterpret_cast<uint4*>(out + item * 8) =
                dequant_chunk<DT, BITS>(q[i], s8, z8);
        }
    }
}

template <int DT, int BITS>
static hipError_t launch_dq_keys_t(const DequantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t NG = (uint32_t)((j.S + j.group - 1) / j.group);
    const uint64_t n_items = (uint64_t)j.BH * NG * D8;
    const uint32_t blocks = (uint32_t)((n_items + 255) / 256);
    hipLaunchKernelGGL((dequant_keys_kernel<DT, BITS>), dim3(blocks),
                       dim3(256), 0, j.stream, j.codes, j.scale, j.zero,
                       (uint32_t)n_items, D8, NG, (int32_t)j.S,
                       (int32_t)j.group, static_cast<uint16_t*>(j.out));
    return hipGetLastError();
}

template <int DT, int BITS>
static hipError_t launch_dq_values_t(const DequantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint64_t n_items = (uint64_t)j.BH * j.S * D8;
    const uint32_t NGD = (uint32_t)((j.D + j.group - 1) / j.group);
    const uint64_t per_block = 256u * kDqValItems;
    const uint32_t blocks = (uint32_t)((n_items + per_block - 1) / per_block);
    hipLaunchKernelGGL((dequant_values_kernel<DT, BITS>), dim3(blocks),
                       dim3(256), 0, j.stream, j.codes, j.scale, j.zero,
                       n_items, D8, (uint32_t)(j.group / 8), NGD,
                       static_cast<uint16_t*>(j.out));
    return hipGetLastError();
}

#define KIVI_DISPATCH_DQ(NAME, J)                                       \
    do {                                                                \
        if ((J).out_dtype == DT_F16) {                                  \
            switch ((J).bits) {                                         \
                case 1: return NAME<DT_F16, 1>(J);                      \
                case 2: return NAME<DT_F16, 2>(J);                      \
                case 4: return NAME<DT_F16, 4>(J);                      \
                default: return NAME<DT_F16, 8>(J);                     \
            }                                                           \
        } else {                                                        \
            switch ((J).bits) {                                         \
                case 1: return NAME<DT_BF16, 1>(J);                     \
                case 2: return NAME<DT_BF16, 2>(J);                     \
                case 4: return NAME<DT_BF16, 4>(J);                     \
                default: return NAME<DT_BF16, 8>(J);                    \
            }                                                           \
        }                                                               \
    } while (0)

hipError_t launch_dequant_keys(const DequantJob& j) {
    const int64_t NG = (j.S + j.group - 1) / j.group;
    const bool fits = (uint64_t)j.BH * NG * (j.D / 8) < (1ull << 31) &&
                      j.S < (1ll << 31) && j.group < (1ll << 31);
    if (j.D % 8 != 0 || !fits) return launch_generic_dequant(j, true);
    KIVI_DISPATCH_DQ(launch_dq_keys_t, j);
}

hipError_t launch_dequant_values(const DequantJob& j) {
    if (j.D % 8 != 0 || j.group % 8 != 0) return launch_generic_dequant(j, false);
    KIVI_DISPATCH_DQ(launch_dq_values_t, j);
}

}  // namespace kivi
