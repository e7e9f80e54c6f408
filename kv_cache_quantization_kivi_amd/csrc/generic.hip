// Fallback KIVI kernels for shapes outside the fast kernels' layouts:
// any D with D*bits % 8 == 0 and any group size.  They compute exactly the
// same results (true IEEE division for every code) with simple one-thread
// mappings; they re-read the input once more instead of keeping a group in
// registers and are not tuned.
//
// Keys: one thread per (bh, token group, byte column); a byte column holds
// 8/bits adjacent channels, so no two threads write the same code byte.
// Values: one thread per row (bh, s), walking its groups in order and
// assembling code bytes that may straddle two groups.
// Dequant: one thread per element.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

template <int DT>
__device__ __forceinline__ float widen1(uint16_t h) {
    if constexpr (DT == DT_F16) return (float)__builtin_bit_cast(_Float16, h);
    else return __uint_as_float((uint32_t)h << 16);
}

template <int DT>
__device__ __forceinline__ uint16_t narrow1(float f) {
    if constexpr (DT == DT_F16) return __builtin_bit_cast(uint16_t, (_Float16)f);
    else return __builtin_bit_cast(uint16_t, (__bf16)f);
}

template <int DT, int BITS, bool WQ, bool WR>
__global__ __launch_bounds__(256) void generic_quant_keys_kernel(
    const uint16_t* __restrict__ x, uint64_t n_items, int64_t S, int64_t D,
    int64_t G, int64_t NG, uint8_t* __restrict__ codes,
    float* __restrict__ scale, float* __restrict__ zero,
    uint16_t* __restrict__ recon) {
    constexpr int per = 8 / BITS;
    constexpr float levels = (float)((1 << BITS) - 1);
    const uint64_t item = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (item >= n_items) return;
    const int64_t nbc = D / per;
    const int64_t bc = (int64_t)(item % (uint64_t)nbc);
    const int64_t tile = (int64_t)(item / (uint64_t)nbc);
    const int64_t g = tile % NG;
    const int64_t bh = tile / NG;
    const int64_t s0 = g * G;
    const int64_t s1 = s0 + G < S ? s0 + G : S;
    const int64_t d0 = bc * per;

    float mn[per], mx[per];
#pragma unroll
    for (int k = 0; k < per; ++k)
        mn[k] = mx[k] = widen1<DT>(x[(bh * S + s0) * D + d0 + k]);
    for (int64_t s = s0 + 1; s < s1; ++s)
#pragma unroll
        for (int k = 0; k < per; ++k) {
            const float f = widen1<DT>(x[(bh * S + s) * D + d0 + k]);
            mn[k] = fminf(mn[k], f);
            mx[k] = fmaxf(mx[k], f);
        }
    Params p[per];
#pragma unroll
    for (int k = 0; k < per; ++k) {
        p[k] = make_params<BITS>(mn[k], mx[k]);
        if constexpr (WQ) {
            scale[(bh * NG + g) * D + d0 + k] = p[k].scale;
            zero[(bh * NG + g) * D + d0 + k] = p[k].zero;
        }
    }
    const int64_t row_bytes = D * BITS / 8;
    for (int64_t s = s0; s < s1; ++s) {
        uint32_t byte = 0;
#pragma unroll
        for (int k = 0; k < per; ++k) {
            const float f = widen1<DT>(x[(bh * S + s) * D + d0 + k]);
            const uint32_t c = code_slow(f, p[k], levels);
            byte |= c << (k * BITS);
            if constexpr (WR)
                recon[(bh * S + s) * D + d0 + k] =
                    narrow1<DT>(kivi::recon(c, p[k].scale, p[k].zero));
        }
        if constexpr (WQ) codes[(bh * S + s) * row_bytes + bc] = (uint8_t)byte;
    }
}

template <int DT, int BITS, bool WQ, bool WR>
__global__ __launch_bounds__(256) void generic_quant_values_kernel(
    const uint16_t* __restrict__ x, int64_t n_rows, int64_t D, int64_t G,
    int64_t NGD, uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, uint16_t* __restrict__ recon) {
    constexpr int per = 8 / BITS;
    constexpr float levels = (float)((1 << BITS) - 1);
    const int64_t row = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (row >= n_rows) return;
    const uint16_t* xr = x + row * D;
    const int64_t row_bytes = D * BITS / 8;
    uint32_t acc = 0;
    for (int64_t j = 0; j < NGD; ++j) {
        const int64_t d0 = j * G;
        const int64_t d1 = d0 + G < D ? d0 + G : D;
        float mn = widen1<DT>(xr[d0]);
        float mx = mn;
        for (int64_t d = d0 + 1; d < d1; ++d) {
            const float f = widen1<DT>(xr[d]);
            mn = fminf(mn, f);
            mx = fmaxf(mx, f);
        }
        const Params p = make_params<BITS>(mn, mx);
        if constexpr (WQ) {
            scale[row * NGD + j] = p.scale;
            zero[row * NGD + j] = p.zero;
        }
        for (int64_t d = d0; d < d1; ++d) {
            const uint32_t c = code_slow(widen1<DT>(xr[d]), p, levels);
            acc |= c << ((d % per) * BITS);
            if (d % per == per - 1) {
                if constexpr (WQ) codes[row * row_bytes + d / per] = (uint8_t)acc;
                acc = 0;
            }
            if constexpr (WR)
                recon[row * D + d] = narrow1<DT>(kivi::recon(c, p.scale, p.zero));
        }
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(256) void generic_dequant_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint64_t n, int64_t S, int64_t D,
    int64_t G, int64_t NG, int64_t NGD, int keys,
    uint16_t* __restrict__ out) {
    constexpr int per = 8 / BITS;
    const uint64_t e = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (e >= n) return;
    const int64_t row = (int64_t)(e / (uint64_t)D);
    const int64_t d = (int64_t)(e % (uint64_t)D);
    const uint32_t byte = codes[row * (D * BITS / 8) + d / per];
    const uint32_t c = (byte >> ((d % per) * BITS)) & ((1u << BITS) - 1u);
    int64_t pi;
    if (keys) {
        const int64_t bh = row / S;
        const int64_t s = row % S;
        pi = (bh * NG + s / G) * D + d;
    } else {
        pi = row * NGD + d / G;
    }
    out[e] = narrow1<DT>(recon(c, scale[pi], zero[pi]));
}

// ---------------------------------------------------------------------------

template <int DT, int BITS, bool WQ, bool WR>
static hipError_t gk_t(const QuantJob& j) {
    constexpr int per = 8 / BITS;
    const int64_t NG = (j.S + j.group - 1) / j.group;
    const uint64_t n = (uint64_t)j.BH * NG * (j.D / per);
    return launch_kernel((generic_quant_keys_kernel<DT, BITS, WQ, WR>),
                       dim3((uint32_t)((n + 255) / 256)), dim3(256), 0,
                       j.stream, static_cast<const uint16_t*>(j.x), n, j.S,
                       j.D, j.group, NG, j.codes, j.scale, j.zero,
                       static_cast<uint16_t*>(j.recon));
}

template <int DT, int BITS, bool WQ, bool WR>
static hipError_t gv_t(const QuantJob& j) {
    const int64_t NGD = (j.D + j.group - 1) / j.group;
    const int64_t n = j.BH * j.S;
    return launch_kernel((generic_quant_values_kernel<DT, BITS, WQ, WR>),
                       dim3((uint32_t)((n + 255) / 256)), dim3(256), 0,
                       j.stream, static_cast<const uint16_t*>(j.x), n, j.D,
                       j.group, NGD, j.codes, j.scale, j.zero,
                       static_cast<uint16_t*>(j.recon));
}

template <int DT, int BITS>
static hipError_t gdq_t(const DequantJob& j, bool keys) {
    const uint64_t n = (uint64_t)j.BH * j.S * j.D;
    const int64_t NG = (j.S + j.group - 1) / j.group;
    const int64_t NGD = (j.D + j.group - 1) / j.group;
    return launch_kernel((generic_dequant_kernel<DT, BITS>),
                       dim3((uint32_t)((n + 255) / 256)), dim3(256), 0,
                       j.stream, j.codes, j.scale, j.zero, n, j.S, j.D,
                       j.group, NG, NGD, keys ? 1 : 0,
                       static_cast<uint16_t*>(j.out));
}

template <int DT, int BITS>
static hipError_t gk_mode(const QuantJob& j) {
    const bool wq = j.codes != nullptr, wr = j.recon != nullptr;
    if (wq && wr) return gk_t<DT, BITS, true, true>(j);
    if (wq) return gk_t<DT, BITS, true, false>(j);
    return gk_t<DT, BITS, false, true>(j);
}

template <int DT, int BITS>
static hipError_t gv_mode(const QuantJob& j) {
    const bool wq = j.codes != nullptr, wr = j.recon != nullptr;
    if (wq && wr) return gv_t<DT, BITS, true, true>(j);
    if (wq) return gv_t<DT, BITS, true, false>(j);
    return gv_t<DT, BITS, false, true>(j);
}

template <int DT>
static hipError_t gk_bits(const QuantJob& j) {
    switch (j.bits) {
        case 1: return gk_mode<DT, 1>(j);
        case 2: return gk_mode<DT, 2>(j);
        case 4: return gk_mode<DT, 4>(j);
        default: return gk_mode<DT, 8>(j);
    }
}

template <int DT>
static hipError_t gv_bits(const QuantJob& j) {
    switch (j.bits) {
        case 1: return gv_mode<DT, 1>(j);
        case 2: return gv_mode<DT, 2>(j);
        case 4: return gv_mode<DT, 4>(j);
        default: return gv_mode<DT, 8>(j);
    }
}

template <int DT>
static hipError_t gdq_bits(const DequantJob& j, bool keys) {
    switch (j.bits) {
        case 1: return gdq_t<DT, 1>(j, keys);
        case 2: return gdq_t<DT, 2>(j, keys);
        case 4: return gdq_t<DT, 4>(j, keys);
        default: return gdq_t<DT, 8>(j, keys);
    }
}

hipError_t launch_generic_quant_keys(const QuantJob& j) {
    return j.dtype == DT_F16 ? gk_bits<DT_F16>(j) : gk_bits<DT_BF16>(j);
}

hipError_t launch_generic_quant_values(const QuantJob& j) {
    return j.dtype == DT_F16 ? gv_bits<DT_F16>(j) : gv_bits<DT_BF16>(j);
}

hipError_t launch_generic_dequant(const DequantJob& j, bool keys) {
    return j.out_dtype == DT_F16 ? gdq_bits<DT_F16>(j, keys)
                                 : gdq_bits<DT_BF16>(j, keys);
}

}  // namespace kivi
