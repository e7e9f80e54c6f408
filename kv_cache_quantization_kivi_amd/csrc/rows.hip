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
    // tokens in batches of 8: every load of a batch is issued before its
    // first store
    for (int32_t t0 = 0; t0 < nt; t0 += 8) {
        uint64_t q[8];
        int32_t sp[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int32_t t = min(t0 + u, nt - 1);
            q[u] = load_codes<BITS>(src + t * row_bytes);
            sp[u] = lp[t];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const int32_t s = sp[u];
            if (t0 + u < nt && s >= 0 && s < S)
                store16_nt(dst + (int64_t)s * D, dequant_chunk<DT, BITS>(q[u], sc, z));
        }
    }
}

// Values: one lane per (row of the set, CPL consecutive 8-channel chunks):
// one CPL * BITS-byte code load and one (scale, zero) load per value group
// it touches (groups are multiples of 8 channels).  The reconstruction goes
// out through LDS: a wave's rows are parked there and stored with one lane
// per 16-byte chunk, so each store instruction writes whole rows.
constexpr int kLdvWaveRowsMax = 64;

template <int DT, int BITS, int CPL, int D8>
__global__ __launch_bounds__(256) void list_dequant_values_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint64_t n_items, uint32_t NGD, int32_t S,
    int32_t n, int32_t H, int32_t G, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out) {
    constexpr int UNITS = D8 / CPL;                  // lanes per row
    constexpr int WROWS = 64 / UNITS;                // rows per wave
    constexpr int RS = D8 * 16 + 16;                 // padded LDS row bytes
    constexpr int64_t D = D8 * 8;
    __shared__ __attribute__((aligned(16))) uint8_t rec_s[4][WROWS * RS];
    __shared__ int64_t row_s[4][WROWS];              // output row, or -1
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    const uint64_t gid = (uint64_t)blockIdx.x * 256u + threadIdx.x;
    const bool valid = gid < n_items;
    const uint64_t item = valid ? gid : n_items - 1u;
    const uint32_t u = (uint32_t)(item % UNITS);
    const uint32_t r = (uint32_t)(item / UNITS);     // bh * n + j
    const uint32_t bh = r / (uint32_t)n;
    const int32_t j = (int32_t)(r - bh * (uint32_t)n);
    const int32_t s = pos[(int64_t)(bh / (uint32_t)H) * n + j];
    const uint8_t* cp = codes + (int64_t)r * D8 * BITS + (int64_t)u * CPL * BITS;
    uint64_t q[CPL];
    if constexpr (CPL * BITS == 8) {
        const uint2 wd = *reinterpret_cast<const uint2*>(cp);
        const uint64_t all = (uint64_t)wd.x | ((uint64_t)wd.y << 32);
        if constexpr (CPL == 1) {
            q[0] = all;
        } else {
#pragma unroll
            for (int i = 0; i < CPL; ++i)
                q[i] = (all >> (i * 8 * BITS)) & ((1ull << (8 * BITS)) - 1ull);
        }
    } else {
#pragma unroll
        for (int i = 0; i < CPL; ++i) q[i] = load_codes<BITS>(cp + i * BITS);
    }
    const float* sr = scale + (int64_t)r * NGD;
    const float* zr = zero + (int64_t)r * NGD;
    // The LDS slot comes from the lane, not the item: a lane past the end
    // mirrors the last item, but its slot (and the row index its wave row
    // gets, -1) must still be its own, so that every wave row is written.
    const uint32_t wrow = lane / UNITS, ul = lane % UNITS;
    uint8_t* mine = rec_s[w] + wrow * RS + ul * CPL * 16;
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
        const int32_t gv = (int32_t)((u * CPL + i) * 8) / G;
        const float sv = sr[gv], zv = zr[gv];
        const float sc[8] = {sv, sv, sv, sv, sv, sv, sv, sv};
        const float z[8] = {zv, zv, zv, zv, zv, zv, zv, zv};
        *reinterpret_cast<uint4*>(mine + i * 16) = dequant_chunk<DT, BITS>(q[i], sc, z);
    }
    if (ul == 0)
        row_s[w][wrow] = (valid && s >= 0 && s < S) ? (int64_t)bh * S + s : -1;
    wave_lds_sync();
#pragma unroll
    for (int k = 0; k < CPL; ++k) {
        const uint32_t piece = k * 64u + lane;       // chunk of the wave's rows
        const uint32_t pr = piece / D8, pc = piece % D8;
        const int64_t orow = row_s[w][pr];
        if (orow >= 0)
            store16_nt(out + orow * D + pc * 8,
                       *reinterpret_cast<const uint4*>(rec_s[w] + pr * RS + pc * 16));
    }
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
    const uint32_t cpl = D8 < 4 ? D8 : 4;              // D8 is a power of two
    // whole waves of lanes: n_items rounded up to a multiple of 64 lanes is
    // not needed, lanes past the end mirror the last item and store nothing
    const uint64_t n = (uint64_t)j.B * j.H * j.n * (D8 / cpl);
    const dim3 grid((uint32_t)((n + 255u) / 256u)), block(256);
    const auto go = [&](auto kern) {
        return launch_kernel(kern, grid, block, 0, j.stream, j.codes, j.scale,
                             j.zero, n, NGD, (int32_t)j.S, (int32_t)j.n,
                             (int32_t)j.H, (int32_t)j.group, j.pos, o);
    };
    switch (D8) {
        case 1: return go(list_dequant_values_kernel<DT, BITS, 1, 1>);
        case 2: return go(list_dequant_values_kernel<DT, BITS, 2, 2>);
        case 4: return go(list_dequant_values_kernel<DT, BITS, 4, 4>);
        case 8: return go(list_dequant_values_kernel<DT, BITS, 4, 8>);
        case 16: return go(list_dequant_values_kernel<DT, BITS, 4, 16>);
        default: return go(list_dequant_values_kernel<DT, BITS, 4, 32>);
    }
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
