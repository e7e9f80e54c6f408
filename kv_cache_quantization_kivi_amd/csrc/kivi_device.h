// Device-side building blocks shared by the KIVI kernels (gfx950).
//
// Arithmetic contract: every step of the quantizer is one IEEE binary32
// operation rounded to nearest even, exactly as the KIVI blog post on the
// fused Metal kernels states it (sections "What we're actually optimizing"
// and "Three ways to be off by one bit"): zero = min, scale = (max - min) /
// (2^bits - 1), code = clip(round_half_even((x - zero) / scale)), recon =
// (code * scale) + zero with the product rounded first.  This file is built
// with -ffp-contract=off so no multiply-add is ever fused behind our back;
// the only fused operations are the explicit __builtin_fmaf calls of the
// division below.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kivi {

typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
typedef __bf16 b2_t __attribute__((ext_vector_type(2)));

enum { DT_F16 = 0, DT_BF16 = 1 };

__device__ __forceinline__ h2_t as_h2(uint32_t w) {
    return __builtin_bit_cast(h2_t, w);
}

// Element k (0..7) of an 8-element chunk held as 4 dwords, widened to fp32
// (exact for both 16-bit formats).
template <int DT>
__device__ __forceinline__ float elem(const uint32_t (&w)[4], int k) {
    const uint32_t word = w[k >> 1];
    if constexpr (DT == DT_F16) {
        const uint16_t h = (k & 1) ? (uint16_t)(word >> 16) : (uint16_t)word;
        return (float)__builtin_bit_cast(_Float16, h);
    } else {
        return __uint_as_float((k & 1) ? (word & 0xffff0000u) : (word << 16));
    }
}

// Two fp32 values -> one dword of two 16-bit values, round to nearest even.
template <int DT>
__device__ __forceinline__ uint32_t narrow2(float lo, float hi) {
    if constexpr (DT == DT_F16) {
        h2_t v = {(_Float16)lo, (_Float16)hi};
        return __builtin_bit_cast(uint32_t, v);
    } else {
        b2_t v = {(__bf16)lo, (__bf16)hi};
        return __builtin_bit_cast(uint32_t, v);
    }
}

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

// One 128-bit load (through a native vector type, so it is never split).
__device__ __forceinline__ uint4 load16(const void* p) {
    const u32x4_t q = *reinterpret_cast<const u32x4_t*>(p);
    return make_uint4(q.x, q.y, q.z, q.w);
}

// Streaming 128-bit load: the input of a flush is read exactly once, so it
// is marked non-temporal and does not displace reusable lines in the caches.
__device__ __forceinline__ uint4 load16_nt(const void* p) {
    const u32x4_t q =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_uint4(q.x, q.y, q.z, q.w);
}

// Streaming 128-bit store for whole 16-byte pieces of a fresh output
// (reconstructions): written once and not read back by this kernel, so it
// is marked non-temporal and does not leave dirty lines in the caches for
// the next kernel to evict.
__device__ __forceinline__ void store16_nt(void* p, const uint4& v) {
    const u32x4_t q = {v.x, v.y, v.z, v.w};
    __builtin_nontemporal_store(q, reinterpret_cast<u32x4_t*>(p));
}

// Make one wave's LDS writes visible to the other lanes of the same wave
// (the waits for its outstanding LDS operations plus a wave barrier).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ void words(const uint4& v, uint32_t (&w)[4]) {
    w[0] = v.x;
    w[1] = v.y;
    w[2] = v.z;
    w[3] = v.w;
}

// IEEE 754-2019 minimum/maximum.  On gfx950 these map to v_[pk_]minimum3 /
// v_[pk_]maximum3, which need no NaN-quieting of their inputs (minNum/maxNum
// under the IEEE mode bit do) and fold two new operands per instruction.
// They order -0 below +0; the group min/max is canonicalised afterwards.
__device__ __forceinline__ h2_t vmin(h2_t a, h2_t b) {
    return __builtin_elementwise_minimum(a, b);
}
__device__ __forceinline__ h2_t vmax(h2_t a, h2_t b) {
    return __builtin_elementwise_maximum(a, b);
}
__device__ __forceinline__ float vmin(float a, float b) {
    return __builtin_elementwise_minimum(a, b);
}
__device__ __forceinline__ float vmax(float a, float b) {
    return __builtin_elementwise_maximum(a, b);
}

// Running min/max of one 8-element chunk position across rows.
template <int DT>
struct MinMax8 {
    // fp16: packed pairs (exact: min/max only select).
    // bf16: each element is compared as a raw fp32 dword that holds it in
    // its high half: the dword itself for the high element, the dword
    // rotated by 16 bits for the low one.  The other element then sits in
    // the low 16 bits and perturbs the value by less than one bf16 ulp
    // toward larger magnitude, which keeps the order of distinct bf16
    // values, so the min/max dword carries the min/max bf16 in its high half
    // (zeros of either sign may come out as tiny values of either sign;
    // get() masks the low half and make_params canonicalises the zero).
    // The rotate is one instruction like the plain widening shift, but it
    // is not merged with the code pass's widening, which would keep every
    // token's widened low half live across both passes.
    h2_t mn2[4], mx2[4];
    float mn[8], mx[8];

    __device__ __forceinline__ void init(const uint4& v) {
        uint32_t w[4];
        words(v, w);
        if constexpr (DT == DT_F16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) mn2[j] = mx2[j] = as_h2(w[j]);
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mn[2 * j] = mx[2 * j] =
                    __uint_as_float(__builtin_amdgcn_alignbit(w[j], w[j], 16));
                mn[2 * j + 1] = mx[2 * j + 1] = __uint_as_float(w[j]);
            }
        }
    }

    __device__ __forceinline__ void add(const uint4& v) {
        uint32_t w[4];
        words(v, w);
        if constexpr (DT == DT_F16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                mn2[j] = vmin(mn2[j], as_h2(w[j]));
                mx2[j] = vmax(mx2[j], as_h2(w[j]));
            }
        } else {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const float lo =
                    __uint_as_float(__builtin_amdgcn_alignbit(w[j], w[j], 16));
                const float hi = __uint_as_float(w[j]);
                mn[2 * j] = vmin(mn[2 * j], lo);
                mx[2 * j] = vmax(mx[2 * j], lo);
                mn[2 * j + 1] = vmin(mn[2 * j + 1], hi);
                mx[2 * j + 1] = vmax(mx[2 * j + 1], hi);
            }
        }
    }

    // Fold in the running min/max of the lane `mask` lanes away (an xor
    // partner in the same wave; every lane of the wave must take part).
    __device__ __forceinline__ void combine_xor(int mask) {
        if constexpr (DT == DT_F16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                const int a = __shfl_xor(__builtin_bit_cast(int, mn2[j]), mask);
                const int b = __shfl_xor(__builtin_bit_cast(int, mx2[j]), mask);
                mn2[j] = vmin(mn2[j], __builtin_bit_cast(h2_t, a));
                mx2[j] = vmax(mx2[j], __builtin_bit_cast(h2_t, b));
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                mn[k] = vmin(mn[k], __shfl_xor(mn[k], mask));
                mx[k] = vmax(mx[k], __shfl_xor(mx[k], mask));
            }
        }
    }

    // Per-channel min and max as fp32.
    __device__ __forceinline__ void get(float (&lo)[8], float (&hi)[8]) const {
        if constexpr (DT == DT_F16) {
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                lo[2 * j] = (float)mn2[j].x;
                lo[2 * j + 1] = (float)mn2[j].y;
                hi[2 * j] = (float)mx2[j].x;
                hi[2 * j + 1] = (float)mx2[j].y;
            }
        } else {
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                lo[k] = __uint_as_float(__float_as_uint(mn[k]) & 0xffff0000u);
                hi[k] = __uint_as_float(__float_as_uint(mx[k]) & 0xffff0000u);
            }
        }
    }
};

// Group parameters from the group's fp32 min and max.
//   zero  = min (stored as +0 when it compares equal to 0)
//   scale = RN(RN(max - min) / (2^bits - 1))
//   y     = RN(1 / scale), used by the division below (0 when scale == 0)
//   fast  = whether the reciprocal-based division is exact for this scale
//
// Both divisions are computed exactly without the IEEE division sequence:
//  - x + 0.0 turns -0 into +0 and leaves every other value unchanged;
//  - scale: the quotient by the constant L = 2^bits - 1 with Markstein's
//    correction from c = RN(1/L): q0 = RN(range*c), r = range - q0*L (exact
//    in one FMA), scale = RN(q0 + r*c).  Checked against IEEE division for
//    every significand, L in {1, 3, 15, 255}, range in [2^-100, 2^101);
//  - y: the hardware reciprocal estimate (within one ulp) plus one Newton
//    step, y = RN(y0 + y0*(1 - scale*y0)), equals RN(1/scale) for every
//    significand at every exponent of the fast range on gfx950; the library
//    carries a self-test of exactly this (kivi_selftest_division).
// Groups whose range falls outside [2^-56, 2^56] (possible only for bf16
// inputs of extreme magnitude) are marked slow: their scale is recomputed
// with IEEE division and their codes take the IEEE-division path.
struct Params {
    float zero, scale, y;
    bool fast;
};

template <int BITS>
__device__ __forceinline__ Params make_params(float mn, float mx) {
    constexpr float L = (float)((1 << BITS) - 1);
    constexpr float inv_L = 1.0f / L;   // RN(1/L), folded at compile time
    Params p;
    mn = mn + 0.0f;
    mx = mx + 0.0f;
    const float range = mx - mn;
    p.zero = mn;
    const float q0 = range * inv_L;
    const float r = __builtin_fmaf(-q0, L, range);
    p.scale = __builtin_fmaf(r, inv_L, q0);
    const float y0 = __builtin_amdgcn_rcpf(p.scale);
    const float e = __builtin_fmaf(-p.scale, y0, 1.0f);
    const float y = __builtin_fmaf(e, y0, y0);
    p.y = (range == 0.0f) ? 0.0f : y;
    p.fast = (range == 0.0f) || (range >= 0x1p-56f && range <= 0x1p56f);
    // Ranges outside the fast window are rare; a wave-uniform branch keeps
    // the IEEE division sequence off the common path (a per-lane select
    // would execute it for every group).
    if (__any(!p.fast)) {
        if (!p.fast) p.scale = range / L;
    }
    return p;
}

// RN(a / scale) from y = RN(1 / scale) (Markstein, IBM J. Res. Dev. 34(1),
// 1990; Muller et al., Handbook of Floating-Point Arithmetic, "Newton-Raphson
// based division with an FMA"): q0 = RN(a*y) is within an ulp of a/scale,
// the residual a - q0*scale is exact in one fused multiply-add, and one more
// fused multiply-add gives the correctly rounded quotient.  With scale == 0
// (so y == 0 and a == 0) it returns 0.
__device__ __forceinline__ float div_fast(float a, float scale, float y) {
    const float q0 = a * y;
    const float r = __builtin_fmaf(-q0, scale, a);
    return __builtin_fmaf(r, y, q0);
}

// Code of quotient t = RN(a/scale): round half to even and clip to
// [0, maxc]; maxNum/minNum send a NaN quotient to 0.
__device__ __forceinline__ uint32_t code_exact(float t, float maxc) {
    float r = __builtin_rintf(t);
    r = fmaxf(r, 0.0f);
    r = fminf(r, maxc);
    return (uint32_t)r;
}

// The slow path: true IEEE division (scale == 0 gives code 0).
__device__ __forceinline__ uint32_t code_slow(float f, const Params& p,
                                              float maxc) {
    if (p.scale == 0.0f) return 0u;
    const float a = f - p.zero;
    return code_exact(a / p.scale, maxc);
}

// f - zero for element k of a chunk, rounded once to fp32.  For fp16 the
// widening is folded into the subtraction: v_fma_mix_f32 reads the 16-bit
// half selected by op_sel, and fma(h, 1.0, -zero) = RN(h - zero) exactly.
template <int DT>
__device__ __forceinline__ float sub_zero(const uint32_t (&w)[4], int k,
                                          float zero) {
    if constexpr (DT == DT_F16) {
        float r;
        if (k & 1)
            asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[1,0,0] op_sel_hi:[1,0,0]"
                : "=v"(r) : "v"(w[k >> 1]), "v"(zero));
        else
            asm("v_fma_mix_f32 %0, %1, 1.0, -%2 op_sel:[0,0,0] op_sel_hi:[1,0,0]"
                : "=v"(r) : "v"(w[k >> 1]), "v"(zero));
        return r;
    } else {
        return elem<DT>(w, k) - zero;
    }
}

// The fast path.  For an element of its own group, a = RN(f - zero) lies in
// [0, RN(max - min)], so t = RN(a / scale) lies in [0, maxc * (1 + 2^-23)]
// and round-half-even never leaves [0, maxc]: the clip cannot bind.  Adding
// 2^23 rounds t to an integer (ties to even) in the low mantissa bits.
// Returns the bits of t + 2^23: the code sits in the low mantissa bits and
// every mantissa bit above it is 0 (the exponent field holds 0x4b).
__device__ __forceinline__ uint32_t code_fast_bits(float a, const Params& p) {
    const float t = div_fast(a, p.scale, p.y);
    return __float_as_uint(t + 0x1p23f);
}

// Pack 8 codes: m[k] has code k in its low BITS bits, zeros above it up to
// bit 22 and garbage only from bit 23 on (bits of t + 2^23, or plain codes).
// Shifts and ORs keep the garbage above the packed field; v_perm_b32 picks
// bytes where it would not.
template <int BITS>
__device__ __forceinline__ uint64_t pack8(const uint32_t (&m)[8]) {
    if constexpr (BITS == 1 || BITS == 2) {
        const uint32_t n01 = (m[1] << BITS) | m[0], n23 = (m[3] << BITS) | m[2];
        const uint32_t n45 = (m[5] << BITS) | m[4], n67 = (m[7] << BITS) | m[6];
        const uint32_t q0 = (n23 << (2 * BITS)) | n01;
        const uint32_t q1 = (n67 << (2 * BITS)) | n45;
        return ((q1 << (4 * BITS)) | q0) & ((1u << (8 * BITS)) - 1u);
    } else if constexpr (BITS == 4) {
        const uint32_t n01 = (m[1] << 4) | m[0], n23 = (m[3] << 4) | m[2];
        const uint32_t n45 = (m[5] << 4) | m[4], n67 = (m[7] << 4) | m[6];
        const uint32_t p0 = (n23 << 8) | n01, p1 = (n67 << 8) | n45;
        return __builtin_amdgcn_perm(p1, p0, 0x05040100u);
    } else {
        const uint32_t p01 = __builtin_amdgcn_perm(m[1], m[0], 0x0c0c0400u);
        const uint32_t p23 = __builtin_amdgcn_perm(m[3], m[2], 0x04000c0cu);
        const uint32_t p45 = __builtin_amdgcn_perm(m[5], m[4], 0x0c0c0400u);
        const uint32_t p67 = __builtin_amdgcn_perm(m[7], m[6], 0x04000c0cu);
        return (uint64_t)(p01 | p23) | ((uint64_t)(p45 | p67) << 32);
    }
}

// recon = RN(RN(code * scale) + zero): two roundings, never fused.
__device__ __forceinline__ float recon(uint32_t code, float scale, float zero) {
    const float prod = (float)code * scale;
    return prod + zero;
}

// Store the 8*BITS bits of one chunk's codes (BITS bytes) at p.
// NT: a non-temporal store (streamed past the caches), for outputs that no
// later step of the same kernel reads.
template <int BITS, bool NT = false>
__device__ __forceinline__ void store_codes(uint8_t* p, uint64_t bits) {
    if constexpr (BITS == 1) {
        if constexpr (NT) __builtin_nontemporal_store((uint8_t)bits, p);
        else *p = (uint8_t)bits;
    } else if constexpr (BITS == 2) {
        if constexpr (NT)
            __builtin_nontemporal_store((uint16_t)bits, reinterpret_cast<uint16_t*>(p));
        else *reinterpret_cast<uint16_t*>(p) = (uint16_t)bits;
    } else if constexpr (BITS == 4) {
        if constexpr (NT)
            __builtin_nontemporal_store((uint32_t)bits, reinterpret_cast<uint32_t*>(p));
        else *reinterpret_cast<uint32_t*>(p) = (uint32_t)bits;
    } else {
        if constexpr (NT) {
            typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t w = {(uint32_t)bits, (uint32_t)(bits >> 32)};
            __builtin_nontemporal_store(w, reinterpret_cast<u32x2_t*>(p));
        } else {
            *reinterpret_cast<uint2*>(p) =
                make_uint2((uint32_t)bits, (uint32_t)(bits >> 32));
        }
    }
}

template <int BITS>
__device__ __forceinline__ uint64_t load_codes(const uint8_t* p) {
    if constexpr (BITS == 1) {
        return *p;
    } else if constexpr (BITS == 2) {
        return *reinterpret_cast<const uint16_t*>(p);
    } else if constexpr (BITS == 4) {
        return *reinterpret_cast<const uint32_t*>(p);
    } else {
        const uint2 v = *reinterpret_cast<const uint2*>(p);
        return (uint64_t)v.x | ((uint64_t)v.y << 32);
    }
}

// Quantize one 8-element chunk against 8 per-element parameter sets
// (pk[k] for element k).  Returns the packed codes (code k at bits
// [k*BITS, (k+1)*BITS)) and, if wanted, the reconstruction as 4 dwords.
template <int DT, int BITS, bool FAST, bool WR>
__device__ __forceinline__ uint64_t quant_chunk(const uint4& v,
                                                const Params* pk,
                                                uint4* rec) {
    constexpr float maxc = (float)((1 << BITS) - 1);
    uint32_t w[4];
    words(v, w);
    uint32_t m[8];
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        uint32_t c;
        if constexpr (FAST) {
            m[k] = code_fast_bits(sub_zero<DT>(w, k, pk[k].zero), pk[k]);
            c = m[k] - 0x4b000000u;
        } else {
            c = code_slow(elem<DT>(w, k), pk[k], maxc);
            m[k] = c;
        }
        if constexpr (WR) r[k] = recon(c, pk[k].scale, pk[k].zero);
    }
    if constexpr (WR) {
        rec->x = narrow2<DT>(r[0], r[1]);
        rec->y = narrow2<DT>(r[2], r[3]);
        rec->z = narrow2<DT>(r[4], r[5]);
        rec->w = narrow2<DT>(r[6], r[7]);
    }
    return pack8<BITS>(m);
}

// Dequantize one chunk of 8 packed codes.
template <int DT, int BITS>
__device__ __forceinline__ uint4 dequant_chunk(uint64_t packed,
                                               const float (&sc)[8],
                                               const float (&z)[8]) {
    constexpr uint32_t mask = (1u << BITS) - 1u;
    float r[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        const uint32_t c = (uint32_t)(packed >> (k * BITS)) & mask;
        r[k] = recon(c, sc[k], z[k]);
    }
    uint4 o;
    o.x = narrow2<DT>(r[0], r[1]);
    o.y = narrow2<DT>(r[2], r[3]);
    o.z = narrow2<DT>(r[4], r[5]);
    o.w = narrow2<DT>(r[6], r[7]);
    return o;
}

}  // namespace kivi
