// Per-token mixed precision for gfx950 (VeloxQuant-MLX 0.24.1 package page,
// section "ZipCache-adapted -- saliency-adaptive per-token mixed
// precision"): the tokens of highest key-norm score are quantized at
// hi_bits, the rest at lo_bits, both with the KIVI group quantizer.  The two
// token sets are lists of positions; the quantizers read a set's rows in
// place (the ListRows layout) and write it as its own compact tensor, so no
// gathered copy of the keys or values is ever made.  This file holds the
// partition of the positions and the dequantizers that write a set's rows
// back to their positions.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

// ---- partition ----------------------------------------------------------

constexpr int kPartThreads = 1024;
constexpr int kPartWaves = kPartThreads / 64;

// An unsigned key with the order of the float scores (-0 taken as +0, so
// that equal scores have equal keys).
__device__ __forceinline__ uint32_t order_key(float f) {
    uint32_t u = __float_as_uint(f);
    if (u == 0x80000000u) u = 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix count of `flag` over the block in thread order, plus the
// block's total.  Lanes of a wave count with their ballot mask; the waves'
// totals meet in LDS.
__device__ __forceinline__ uint32_t block_rank(bool flag, uint32_t* wsum,
                                               uint32_t* total) {
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint64_t m = __ballot(flag);
    const uint32_t below = (uint32_t)__popcll(m & ((1ull << lane) - 1ull));
    if (lane == 0) wsum[w] = (uint32_t)__popcll(m);
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < kPartWaves; ++i) {
        const uint32_t c = wsum[i];
        before += i < (int)w ? c : 0u;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + below;
}

// One block per sequence.  The n_hi-th largest key is found digit by digit
// (four 8-bit radix passes over the scores, counting only the scores that
// share the digits fixed so far); then one pass in position order marks the
// scores above it and, of the scores equal to it, the lowest positions still
// needed, and writes both lists in ascending position.
__global__ __launch_bounds__(kPartThreads) void partition_top_kernel(
    const float* __restrict__ score, int32_t S, int32_t n_hi,
    int32_t* __restrict__ pos_hi, int32_t* __restrict__ pos_lo) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wsum[kPartWaves];
    __shared__ uint32_t pick[2];
    const int32_t b = blockIdx.x, tid = threadIdx.x;
    const float* sc = score + (int64_t)b * S;
    uint32_t prefix = 0, need = (uint32_t)n_hi;   // keys above prefix still to take
    if (n_hi > 0 && n_hi < S) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kPartThreads) hist[i] = 0u;
            __syncthreads();
            const uint32_t hmask = shift == 24 ? 0u : ~0u << (shift + 8);
            for (int32_t s = tid; s < S; s += kPartThreads) {
                const uint32_t k = order_key(sc[s]);
                if ((k & hmask) == (prefix & hmask))
                    atomicAdd(&hist[(k >> shift) & 255u], 1u);
            }
            __syncthreads();
            // wave 0: lane l holds digits 255-4l .. 252-4l (descending), an
            // inclusive scan of the counts finds the digit where the running
            // count from the top reaches `need`
            if (tid < 64) {
                uint32_t c[4], own = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    c[i] = hist[255 - 4 * tid - i];
                    own += c[i];
                }
                uint32_t incl = own;
#pragma unroll
                for (int o = 1; o < 64; o <<= 1) {
                    const uint32_t y = __shfl_up(incl, o);
                    if (tid >= o) incl += y;
                }
                const uint64_t hit = __ballot(incl >= need);
                const int first = __ffsll((unsigned long long)hit) - 1;
                if (tid == first) {
                    uint32_t run = incl - own;     // count above this lane's digits
                    int i = 0;
                    while (run + c[i] < need) {
                        run += c[i];
                        ++i;
                    }
                    pick[0] = (uint32_t)(255 - 4 * tid - i);
                    pick[1] = need - run;
                }
            }
            __syncthreads();
            prefix |= pick[0] << shift;
            need = pick[1];
            __syncthreads();
        }
    }
    // keys above `prefix` are hi; of the keys equal to it the first `need`
    // in position order
    const bool all_hi = n_hi == S, none_hi = n_hi == 0;
    uint32_t eq_base = 0, hi_base = 0;
    for (int32_t s0 = 0; s0 < S; s0 += kPartThreads) {
        const int32_t s = s0 + tid;
        const bool real = s < S;
        const uint32_t k = real ? order_key(sc[s]) : 0u;
        const bool eq = real && !all_hi && !none_hi && k == prefix;
        uint32_t n_eq, n_h;
        const uint32_t eq_rank = eq_base + block_rank(eq, wsum, &n_eq);
        const bool hi = real && (all_hi || (!none_hi && (k > prefix ||
                                                         (eq && eq_rank < need))));
        const uint32_t hi_rank = hi_base + block_rank(hi, wsum, &n_h);
        if (hi) pos_hi[(int64_t)b * n_hi + hi_rank] = s;
        else if (real) pos_lo[(int64_t)b * (S - n_hi) + (s - (int32_t)hi_rank)] = s;
        eq_base += n_eq;
        hi_base += n_h;
    }
}

// ---- dequantize a set back to its positions ------------------------------

// Keys: one lane per (bh, group of the set, 8-channel chunk), chunk fastest;
// the chunk's 8 scales and zeros are loaded once for the group's tokens.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void list_dequant_keys_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint32_t n_items, uint32_t D8, uint32_t NG,
    int32_t S, int32_t n, int32_t H, int32_t G, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out) {
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    if (gid >= n_items) return;
    const uint32_t c = gid % D8;
    const uint32_t tile = gid / D8;
    const uint32_t g = tile % NG;
    const uint32_t bh = tile / NG;
    const int64_t D = (int64_t)D8 * 8;
    const int32_t j0 = (int32_t)g * G;
    const int32_t nt = min(G, n - j0);
    const int64_t p = ((int64_t)bh * NG + g) * D + (int64_t)c * 8;
    const float4 s_a = *reinterpret_cast<const float4*>(scale + p);
    const float4 s_b = *reinterpret_cast<const float4*>(scale + p + 4);
    const float4 z_a = *reinterpret_cast<const float4*>(zero + p);
    const float4 z_b = *reinterpret_cast<const float4*>(zero + p + 4);
    const float sc[8] = {s_a.x, s_a.y, s_a.z, s_a.w, s_b.x, s_b.y, s_b.z, s_b.w};
    const float z[8] = {z_a.x, z_a.y, z_a.z, z_a.w, z_b.x, z_b.y, z_b.z, z_b.w};
    const int64_t row_bytes = (int64_t)D8 * BITS;
    const uint8_t* src = codes + ((int64_t)bh * n + j0) * row_bytes + (int64_t)c * BITS;
    const int32_t* lp = pos + (int64_t)(bh / (uint32_t)H) * n + j0;
    uint16_t* dst = out + (int64_t)bh * S * D + (int64_t)c * 8;
    for (int32_t t = 0; t < nt; ++t) {
        const int32_t s = lp[t];
        const uint4 r = dequant_chunk<DT, BITS>(load_codes<BITS>(src + t * row_bytes), sc, z);
        if (s >= 0 && s < S) store16_nt(dst + (int64_t)s * D, r);
    }
}

// Values: one lane per (row of the set, 8-channel chunk); a chunk lies in
// one value group (groups are multiples of 8 channels).
template <int DT, int BITS>
__global__ __launch_bounds__(256) void list_dequant_values_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint64_t n_items, uint32_t D8,
    uint32_t NGD, int32_t S, int32_t n, int32_t H, int32_t G,
    const int32_t* __restrict__ pos, uint16_t* __restrict__ out) {
    const uint64_t gid = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    if (gid >= n_items) return;
    const uint32_t c = (uint32_t)(gid % D8);
    const uint32_t r = (uint32_t)(gid / D8);          // bh * n + j
    const uint32_t bh = r / (uint32_t)n;
    const int32_t j = (int32_t)(r - bh * (uint32_t)n);
    const int32_t s = pos[(int64_t)(bh / (uint32_t)H) * n + j];
    if (s < 0 || s >= S) return;
    const int64_t D = (int64_t)D8 * 8;
    const int64_t pi = (int64_t)r * NGD + (int64_t)(c * 8) / G;
    const float sv = scale[pi], zv = zero[pi];
    const float sc[8] = {sv, sv, sv, sv, sv, sv, sv, sv};
    const float z[8] = {zv, zv, zv, zv, zv, zv, zv, zv};
    const uint64_t q = load_codes<BITS>(codes + (int64_t)r * D8 * BITS + (int64_t)c * BITS);
    store16_nt(out + ((int64_t)bh * S + s) * D + (int64_t)c * 8,
               dequant_chunk<DT, BITS>(q, sc, z));
}

template <int DT, int BITS>
static hipError_t launch_list_dq_t(const ListJob& j, bool keys, void* out) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    uint16_t* o = static_cast<uint16_t*>(out);
    if (keys) {
        const uint32_t NG = (uint32_t)((j.n + j.group - 1) / j.group);
        const uint32_t n = (uint32_t)(j.B * j.H) * NG * D8;
        return launch_kernel((list_dequant_keys_kernel<DT, BITS>),
                             dim3((n + 255u) / 256u), dim3(256), 0, j.stream,
                             j.codes, j.scale, j.zero, n, D8, NG, (int32_t)j.S,
                             (int32_t)j.n, (int32_t)j.H, (int32_t)j.group,
                             j.pos, o);
    }
    const uint32_t NGD = (uint32_t)((j.D + j.group - 1) / j.group);
    const uint64_t n = (uint64_t)j.B * j.H * j.n * D8;
    return launch_kernel((list_dequant_values_kernel<DT, BITS>),
                         dim3((uint32_t)((n + 255u) / 256u)), dim3(256), 0,
                         j.stream, j.codes, j.scale, j.zero, n, D8, NGD,
                         (int32_t)j.S, (int32_t)j.n, (int32_t)j.H,
                         (int32_t)j.group, j.pos, o);
}

template <int DT>
static hipError_t launch_list_dq_dt(const ListJob& j, bool keys, void* out) {
    switch (j.bits) {
        case 1: return launch_list_dq_t<DT, 1>(j, keys, out);
        case 2: return launch_list_dq_t<DT, 2>(j, keys, out);
        case 4: return launch_list_dq_t<DT, 4>(j, keys, out);
        default: return launch_list_dq_t<DT, 8>(j, keys, out);
    }
}

hipError_t launch_list_dequant(const ListJob& j, bool keys, void* out) {
    return j.dtype == DT_F16 ? launch_list_dq_dt<DT_F16>(j, keys, out)
                             : launch_list_dq_dt<DT_BF16>(j, keys, out);
}

hipError_t launch_partition_top(const float* score, int64_t B, int64_t S,
                                int64_t n_hi, int32_t* pos_hi, int32_t* pos_lo,
                                hipStream_t stream) {
    return launch_kernel(partition_top_kernel, dim3((uint32_t)B),
                         dim3(kPartThreads), 0, stream, score, (int32_t)S,
                         (int32_t)n_hi, pos_hi, pos_lo);
}

}  // namespace kivi
