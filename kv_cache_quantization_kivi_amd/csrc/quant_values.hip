// KIVI per-token value quantization for gfx950.
//
// KIVI blog post on the fused Metal kernels, section "Kernel B -- per-token
// values": the group runs along the contiguous channel axis, so lanes split
// a group and reduce across lanes.  Here a row of D channels is spread over
// P = next_pow2(D/8) lanes, 8 channels (one 128-bit load) per lane, so one
// wave covers 64/P rows per load and every load is a contiguous 1 KiB of the
// tensor.  A group of G = 8*2^k channels sits on an aligned block of 2^k
// lanes; its min/max is an xor-butterfly over those lanes using DPP row
// permutes (quad xor 1, quad xor 2, half-row mirror, row mirror) and, only
// for blocks wider than 16 lanes, a cross-row lane shuffle.  The post's rule
// carries over: every lane of the wave reaches the reduction (no lane exits
// early), so the permutes never read a retired lane.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kValRows = 4;   // rows per lane per launch slot

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(
        __builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// Min and max over aligned blocks of `red` lanes (red a power of two <= 64,
// uniform across the wave).
__device__ __forceinline__ void block_minmax(float& mn, float& mx,
                                             uint32_t red) {
    if (red > 1) {
        mn = fminf(mn, dpp_f<0xB1>(mn));   // quad_perm [1,0,3,2]
        mx = fmaxf(mx, dpp_f<0xB1>(mx));
    }
    if (red > 2) {
        mn = fminf(mn, dpp_f<0x4E>(mn));   // quad_perm [2,3,0,1]
        mx = fmaxf(mx, dpp_f<0x4E>(mx));
    }
    if (red > 4) {
        mn = fminf(mn, dpp_f<0x141>(mn));  // row_half_mirror
        mx = fmaxf(mx, dpp_f<0x141>(mx));
    }
    if (red > 8) {
        mn = fminf(mn, dpp_f<0x140>(mn));  // row_mirror
        mx = fmaxf(mx, dpp_f<0x140>(mx));
    }
    if (red > 16) {
        mn = fminf(mn, __shfl_xor(mn, 16));
        mx = fmaxf(mx, __shfl_xor(mx, 16));
    }
    if (red > 32) {
        mn = fminf(mn, __shfl_xor(mn, 32));
        mx = fmaxf(mx, __shfl_xor(mx, 32));
    }
}

// Min and max of the 8 elements of one chunk, as fp32.
template <int DT>
__device__ __forceinline__ void chunk_minmax(const uint4& v, float& mn,
                                             float& mx) {
    uint32_t w[4];
    words(v, w);
    if constexpr (DT == DT_F16) {
        const h2_t a = __builtin_elementwise_min(as_h2(w[0]), as_h2(w[1]));
        const h2_t b = __builtin_elementwise_min(as_h2(w[2]), as_h2(w[3]));
        const h2_t m = __builtin_elementwise_min(a, b);
        const h2_t A = __builtin_elementwise_max(as_h2(w[0]), as_h2(w[1]));
        const h2_t B = __builtin_elementwise_max(as_h2(w[2]), as_h2(w[3]));
        const h2_t M = __builtin_elementwise_max(A, B);
        mn = fminf((float)m.x, (float)m.y);
        mx = fmaxf((float)M.x, (float)M.y);
    } else {
        mn = mx = elem<DT>(w, 0);
#pragma unroll
        for (int k = 1; k < 8; ++k) {
            const float f = elem<DT>(w, k);
            mn = fminf(mn, f);
            mx = fmaxf(mx, f);
        }
    }
}

template <int DT, int BITS, bool WQ, bool WR>
__global__ __launch_bounds__(256) void quant_values_kernel(
    const uint16_t* __restrict__ x, int64_t n_rows, uint32_t D8,
    uint32_t lp, uint32_t red, uint32_t lcpg, uint32_t NGD,
    uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, uint16_t* __restrict__ recon) {
    const uint32_t lane = threadIdx.x & 63u;
    const int64_t wave = ((int64_t)blockIdx.x * 256 + threadIdx.x) >> 6;
    const uint32_t c = lane & ((1u << lp) - 1u);   // chunk within its row
    const uint32_t rw = lane >> lp;                // row within a pass
    const uint32_t rpp = 64u >> lp;                // rows per pass
    const int64_t row_base = wave * (int64_t)(rpp * kValRows) + rw;
    const int64_t D = (int64_t)D8 * 8;
    const bool cvalid = c < D8;

    uint4 v[kValRows];
    bool valid[kValRows];
#pragma unroll
    for (int i = 0; i < kValRows; ++i) {
        const int64_t row = row_base + (int64_t)i * rpp;
        valid[i] = cvalid && row < n_rows;
        v[i] = valid[i] ? load16_nt(x + row * D + (int64_t)c * 8)
                        : make_uint4(0, 0, 0, 0);
    }

    float mn[kValRows], mx[kValRows];
#pragma unroll
    for (int i = 0; i < kValRows; ++i) {
        chunk_minmax<DT>(v[i], mn[i], mx[i]);
        if (!valid[i]) {   // identity elements for lanes past the row end
            mn[i] = __builtin_inff();
            mx[i] = -__builtin_inff();
        }
    }
#pragma unroll
    for (int i = 0; i < kValRows; ++i) block_minmax(mn[i], mx[i], red);

    const int64_t row_bytes = (int64_t)D8 * BITS;
    const bool writes_params = (c & ((1u << lcpg) - 1u)) == 0;
#pragma unroll
    for (int i = 0; i < kValRows; ++i) {
        if (!valid[i]) continue;
        const int64_t row = row_base + (int64_t)i * rpp;
        Params p = make_params<BITS>(mn[i], mx[i]);
        if constexpr (WQ) {
            if (writes_params) {
                const int64_t pi = row * NGD + (c >> lcpg);
                scale[pi] = p.scale;
                zero[pi] = p.zero;
            }
        }
        Params pk[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) pk[k] = p;
        uint4 r;
        const uint64_t q = p.fast
            ? quant_chunk<DT, BITS, true, WR>(v[i], pk, &r)
            : quant_chunk<DT, BITS, false, WR>(v[i], pk, &r);
        if constexpr (WQ)
            store_codes<BITS>(codes + row * row_bytes + (int64_t)c * BITS, q);
        if constexpr (WR)
            *reinterpret_cast<uint4*>(recon + row * D + (int64_t)c * 8) = r;
    }
}

static uint32_t log2_ceil(uint64_t n) {
    uint32_t l = 0;
    while ((1ull << l) < n) ++l;
    return l;
}

template <int DT, int BITS, bool WQ, bool WR>
static hipError_t launch_values_t(const QuantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t lp = log2_ceil(D8);                 // lanes per row = 2^lp
    const uint32_t lcpg = log2_ceil((uint64_t)(j.group / 8));
    const uint32_t red = 1u << (lcpg < lp ? lcpg : lp);
    const uint32_t NGD = (uint32_t)((j.D + j.group - 1) / j.group);
    const int64_t n_rows = j.BH * j.S;
    const int64_t rows_per_wave = (int64_t)(64u >> lp) * kValRows;
    const int64_t waves = (n_rows + rows_per_wave - 1) / rows_per_wave;
    const uint32_t blocks = (uint32_t)((waves + 3) / 4);
    hipLaunchKernelGGL((quant_values_kernel<DT, BITS, WQ, WR>), dim3(blocks),
                       dim3(256), 0, j.stream,
                       static_cast<const uint16_t*>(j.x), n_rows, D8, lp, red,
                       lcpg, NGD, j.codes, j.scale, j.zero,
                       static_cast<uint16_t*>(j.recon));
    return hipGetLastError();
}

template <int DT, int BITS>
static hipError_t launch_values_mode(const QuantJob& j) {
    const bool wq = j.codes != nullptr;
    const bool wr = j.recon != nullptr;
    if (wq && wr) return launch_values_t<DT, BITS, true, true>(j);
    if (wq) return launch_values_t<DT, BITS, true, false>(j);
    return launch_values_t<DT, BITS, false, true>(j);
}

template <int DT>
static hipError_t launch_values_bits(const QuantJob& j) {
    switch (j.bits) {
        case 1: return launch_values_mode<DT, 1>(j);
        case 2: return launch_values_mode<DT, 2>(j);
        case 4: return launch_values_mode<DT, 4>(j);
        default: return launch_values_mode<DT, 8>(j);
    }
}

hipError_t launch_quant_values(const QuantJob& j) {
    // Fast path: whole 8-channel chunks, a row within one wave, and groups
    // of 8 * 2^k channels (each group then sits on an aligned lane block).
    const int64_t cpg = j.group / 8;
    const bool pow2 = cpg >= 1 && (cpg & (cpg - 1)) == 0 && j.group % 8 == 0;
    const int64_t n_rows = j.BH * j.S;
    const bool fits = n_rows < (1ll << 40) / 64;
    if (j.D % 8 != 0 || j.D > 512 || !pow2 || !fits)
        return launch_generic_quant_values(j);
    return j.dtype == DT_F16 ? launch_values_bits<DT_F16>(j)
                             : launch_values_bits<DT_BF16>(j);
}

}  // namespace kivi
