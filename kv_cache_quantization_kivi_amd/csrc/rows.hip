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

// Exclusive prefix sum of `v` over the block in thread order, plus the
// block's total: an inclusive scan inside each wave (shuffles), the waves'
// totals through LDS.
__device__ __forceinline__ uint32_t block_scan(uint32_t v, uint32_t* wsum,
                                               uint32_t* total) {
    const uint32_t lane = threadIdx.x & 63u, w = threadIdx.x >> 6;
    uint32_t incl = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const uint32_t y = __shfl_up(incl, o);
        if (lane >= (uint32_t)o) incl += y;
    }
    if (lane == 63) wsum[w] = incl;
    __syncthreads();
    uint32_t before = 0, all = 0;
    for (int i = 0; i < kPartWaves; ++i) {
        const uint32_t c = wsum[i];
        before += i < (int)w ? c : 0u;
        all += c;
    }
    __syncthreads();
    *total = all;
    return before + incl - v;
}

// Elements per thread per round: thread t owns positions
// [round * kPartThreads * kPartPer + t * kPartPer, + kPartPer).
constexpr int kPartPer = 32;
constexpr int kPartRound = kPartThreads * kPartPer;

// One block per sequence.  The n_hi-th largest key is found digit by digit
// (four 8-bit radix passes over the scores, counting only the scores that
// share the digits fixed so far; in the first pass, where most scores share
// their top byte, a wave adds each distinct digit once through a ballot).
// Then each thread walks its own run of positions in order: the scores above
// the threshold and, of those equal to it, the lowest positions still
// needed, are hi; block prefix sums of the per-thread counts give every
// thread its place in both lists, which stay in ascending position.
__global__ __launch_bounds__(kPartThreads) void partition_top_kernel(
    const float* __restrict__ score, int32_t S, int32_t n_hi,
    int32_t* __restrict__ pos_hi, int32_t* __restrict__ pos_lo) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wsum[kPartWaves];
    __shared__ uint32_t pick[2];
    // a round's keys, element p at p + p / 32: the block loads them with
    // coalesced reads, and the 64 lanes reading element i of their runs
    // (stride 33 words) hit 64 different banks
    __shared__ uint32_t stage_s[kPartRound + kPartRound / 32];
    const int32_t b = blockIdx.x, tid = threadIdx.x;
    const int lane = tid & 63;
    const float* sc = score + (int64_t)b * S;
    const int n_rounds = (S + kPartRound - 1) / kPartRound;
    // this thread's run of the round: in registers for the radix passes,
    // read from LDS in the final pass (with the 32 keys live there too the
    // kernel needed more than the 128 VGPRs of a 1024-thread block, and
    // spilled)
    const uint32_t* run_s = stage_s + tid * (kPartPer + 1);
    uint32_t key[kPartPer];
    const auto load_run = [&](int r, bool regs) {   // every thread, barriers inside
        __syncthreads();
#pragma unroll 8
        for (int i = tid; i < kPartRound; i += kPartThreads) {
            const int32_t p = r * kPartRound + i;
            stage_s[i + i / 32] = p < S ? order_key(sc[p]) : 0u;
        }
        __syncthreads();
        if (regs) {
#pragma unroll
            for (int i = 0; i < kPartPer; ++i) key[i] = run_s[i];
        }
    };
    if (n_rounds == 1) load_run(0, true);
    uint32_t prefix = 0, need = (uint32_t)n_hi;   // keys above prefix still to take
    if (n_hi > 0 && n_hi < S) {
        for (int shift = 24; shift >= 0; shift -= 8) {
            for (int i = tid; i < 256; i += kPartThreads) hist[i] = 0u;
            __syncthreads();
            const uint32_t hmask = shift == 24 ? 0u : ~0u << (shift + 8);
            for (int r = 0; r < n_rounds; ++r) {
                if (n_rounds > 1) load_run(r, true);
                const int32_t s0 = r * kPartRound + tid * kPartPer;
#pragma unroll
                for (int i = 0; i < kPartPer; ++i) {
                    const bool in = s0 + i < S && (key[i] & hmask) == (prefix & hmask);
                    const uint32_t d = (key[i] >> shift) & 255u;
                    if (shift == 24) {
                        // each distinct digit of the wave once
                        uint64_t left = __ballot(in);
                        while (left) {
                            const int ld = __ffsll((unsigned long long)left) - 1;
                            const uint32_t dd = __shfl(d, ld);
                            const uint64_t same = __ballot(in && d == dd) & left;
                            if (lane == ld) atomicAdd(&hist[dd], (uint32_t)__popcll(same));
                            left &= ~same;
                        }
                    } else if (in) {
                        atomicAdd(&hist[d], 1u);
                    }
                }
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
    for (int r = 0; r < n_rounds; ++r) {
        if (n_rounds > 1) load_run(r, false);
        const int32_t s0 = r * kPartRound + tid * kPartPer;
        uint32_t n_eq = 0;
#pragma unroll
        for (int i = 0; i < kPartPer; ++i)
            n_eq += (s0 + i < S && !all_hi && !none_hi && run_s[i] == prefix) ? 1u : 0u;
        uint32_t eq_all, hi_all;
        uint32_t eq_rank = eq_base + block_scan(n_eq, wsum, &eq_all);
        uint32_t hi_here = 0;
        uint32_t mark = 0;                     // bit i: position s0 + i is hi
#pragma unroll
        for (int i = 0; i < kPartPer; ++i) {
            const bool real = s0 + i < S;
            const bool eq = real && !all_hi && !none_hi && run_s[i] == prefix;
            const bool hi = real && (all_hi || (!none_hi && (run_s[i] > prefix ||
                                                             (eq && eq_rank < need))));
            eq_rank += eq ? 1u : 0u;
            hi_here += hi ? 1u : 0u;
            mark |= (hi ? 1u : 0u) << i;
        }
        uint32_t hi_rank = hi_base + block_scan(hi_here, wsum, &hi_all);
        if (n_rounds == 1) {
            // one round: both lists are assembled in LDS (the keys are
            // already in registers) and leave with coalesced stores
            // Lane L takes its run's elements in the order i = (t + L) mod
            // 32, so that the 64 lanes of a wave, whose runs start about 32
            // words apart, write distinct banks; an element's rank within
            // the run is the count of hi marks before it.
            __syncthreads();
#pragma unroll 4
            for (int t = 0; t < kPartPer; ++t) {
                const int i = (t + lane) & (kPartPer - 1);
                const int32_t s = s0 + i;
                const uint32_t before = (uint32_t)__builtin_popcount(mark & ((1u << i) - 1u));
                const uint32_t hr = hi_rank + before;
                if (s < S)
                    stage_s[((mark >> i) & 1u) ? hr : (uint32_t)n_hi + (uint32_t)s - hr] =
                        (uint32_t)s;
            }
            __syncthreads();
            for (int i = tid; i < S; i += kPartThreads) {
                const int32_t v = (int32_t)stage_s[i];
                if (i < n_hi) pos_hi[(int64_t)b * n_hi + i] = v;
                else pos_lo[(int64_t)b * (S - n_hi) + (i - n_hi)] = v;
            }
        } else {
#pragma unroll
            for (int i = 0; i < kPartPer; ++i) {
                const int32_t s = s0 + i;
                if (s < S) {                       // positions past S: none
                    if ((mark >> i) & 1u) {
                        pos_hi[(int64_t)b * n_hi + hi_rank] = s;
                        ++hi_rank;
                    } else {
                        pos_lo[(int64_t)b * (S - n_hi) + (s - (int32_t)hi_rank)] = s;
                    }
                }
            }
        }
        eq_base += eq_all;
        hi_base += hi_all;
    }
}

// ---- dequantize a set back to its positions ------------------------------

// Keys: one lane per (bh, group of the set, 8-channel chunk), chunk fastest;
// the chunk's 8 scales and zeros are loaded once for the group's tokens.
// stage: the host's verdict that a wave of full groups has one contiguous
// block of codes made of whole 16-byte pieces per lane (64 % D8 == 0,
// D8 >= 4, group <= 32, group * BITS % 16 == 0, BITS <= 4); the wave then
// loads the block with 16-byte loads into LDS (each group's codes padded
// apart), and its groups' positions beside it, so that the token loop is
// stores only.  A global load in that loop would make each batch wait for
// the stores before it, since one counter tracks a wave's outstanding
// loads and stores together.  The set's codes [BH, n, D*BITS/8] have the
// row order of the wave's groups, so the block starts at lane 0's first row.
template <int BITS>
struct ListDqKeyStage {
    static constexpr int kWaveBytes = BITS <= 4 ? 64 * 32 * BITS + 64 * 16 : 0;
    static constexpr int kWavePos = 16 * 32;   // positions: <= 16 groups of <= 32
};

template <int BITS>
__device__ __forceinline__ uint64_t lds_key_codes(const uint8_t* p) {
    if constexpr (BITS == 1) return *p;
    else if constexpr (BITS == 2) return *reinterpret_cast<const uint16_t*>(p);
    else return *reinterpret_cast<const uint32_t*>(p);
}

template <int DT, int BITS>
__global__ __launch_bounds__(256) void list_dequant_keys_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint32_t n_items, uint32_t D8, uint32_t NG,
    int32_t S, int32_t n, int32_t H, int32_t G, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out, int32_t stage) {
    constexpr int kWaveBytes = ListDqKeyStage<BITS>::kWaveBytes;
    constexpr int kWavePos = ListDqKeyStage<BITS>::kWavePos;
    __shared__ __attribute__((aligned(16)))
    uint8_t lds[BITS <= 4 ? 4 * kWaveBytes : 16];
    __shared__ int32_t pos_s[BITS <= 4 ? 4 * kWavePos : 1];
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const bool valid = gid < n_items;
    const uint32_t item = valid ? gid : n_items - 1u;
    const uint32_t c = item % D8;
    const uint32_t tile = item / D8;
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
    const int64_t crow0 = (int64_t)bh * n + j0;      // the group's first code row
    const int32_t* lp = pos + (int64_t)(bh / (uint32_t)H) * n + j0;
    uint16_t* dst = out + (int64_t)bh * S * D + (int64_t)c * 8;

    if constexpr (BITS <= 4) {
        if (stage && __all(valid && nt == G)) {
            const uint32_t lane = threadIdx.x & 63u;
            uint8_t* L = lds + (threadIdx.x >> 6) * kWaveBytes;
            const uint32_t tile_bytes = (uint32_t)G * D8 * BITS;
            const uint32_t ts = tile_bytes + ((D8 * BITS + 15u) & ~15u);
            const uint32_t r_lo = __builtin_amdgcn_readfirstlane(
                (uint32_t)((uint64_t)crow0 & 0xffffffffu));
            const uint32_t r_hi = __builtin_amdgcn_readfirstlane(
                (uint32_t)((uint64_t)crow0 >> 32));
            const uint8_t* wsrc =
                codes + (int64_t)(((uint64_t)r_hi << 32) | r_lo) * row_bytes;
            const uint32_t n16 = (uint32_t)G * BITS / 16;   // pieces per lane
            uint4 t4[8];
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k)
                if (k < n16) t4[k] = load16_nt(wsrc + (k * 64u + lane) * 16u);
            // the group's positions: lane c of the group loads t = c + m*D8
            // (D8 >= 4, so at most 8 each)
            int32_t pp[8];
#pragma unroll
            for (uint32_t m = 0; m < 8; ++m)   // wave-uniform bound, clamped index
                if (m * D8 < (uint32_t)G) pp[m] = lp[min(c + m * D8, (uint32_t)G - 1u)];
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) {
                if (k < n16) {
                    const uint32_t off = (k * 64u + lane) * 16u;
                    const uint32_t ti = off / tile_bytes;
                    *reinterpret_cast<uint4*>(L + ti * ts + (off - ti * tile_bytes)) = t4[k];
                }
            }
            int32_t* P = pos_s + (threadIdx.x >> 6) * kWavePos + (lane / D8) * 32;
#pragma unroll
            for (uint32_t m = 0; m < 8; ++m) {
                const uint32_t t = c + m * D8;
                if (m * D8 < (uint32_t)G && t < (uint32_t)G) P[t] = pp[m];
            }
            wave_lds_sync();
            const uint8_t* mine = L + (lane / D8) * ts + c * BITS;
            for (int32_t t0 = 0; t0 < G; t0 += 8) {
                int32_t sp[8];
                uint64_t q[8];
#pragma unroll
                for (int u = 0; u < 8; ++u) {   // every LDS read of a batch first
                    const int32_t t = min(t0 + u, G - 1);
                    sp[u] = P[t];
                    q[u] = lds_key_codes<BITS>(mine + t * row_bytes);
                }
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const int32_t s = sp[u];
                    if (t0 + u < G && s >= 0 && s < S)
                        store16_nt(dst + (int64_t)s * D, dequant_chunk<DT, BITS>(q[u], sc, z));
                }
            }
            return;
        }
    }
    if (!valid) return;
    const uint8_t* src = codes + crow0 * row_bytes + (int64_t)c * BITS;
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

// Keys at D = 128 (16 chunks), codes of at most 4 bits, groups of at most 32:
// one wave per (bh, group of the set), four lanes per chunk with
// interleaved tokens, so that every store instruction writes four
// consecutive entries of the list (mostly consecutive rows); the group's
// codes (at most 32 rows of 16 * BITS bytes, contiguous in the set's codes)
// and positions go through LDS first, so the token loop is stores only.
template <int DT, int BITS>
__global__ __launch_bounds__(64) void list_dequant_keys_split_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint32_t NG, int32_t S, int32_t n,
    int32_t H, int32_t G, const int32_t* __restrict__ pos,
    uint16_t* __restrict__ out) {
    static_assert(BITS <= 4, "a group's codes are at most 2 KiB");
    constexpr int64_t D = 128;
    constexpr int64_t row_bytes = 16 * BITS;
    __shared__ __attribute__((aligned(16))) uint8_t lds[32 * row_bytes];
    __shared__ int32_t pos_s[32];
    const uint32_t lane = threadIdx.x;
    const uint32_t tile = blockIdx.x;              // bh * NG + g
    const uint32_t c = lane % 16u, part = lane / 16u;
    const uint32_t g = tile % NG, bh = tile / NG;
    const int32_t j0 = (int32_t)g * G;
    const int32_t nt = min(G, n - j0);
    const int64_t crow0 = (int64_t)bh * n + j0;    // the group's first code row
    const uint32_t n16 = (uint32_t)nt * BITS;      // 16-byte pieces of its codes
    uint4 t4[2];
#pragma unroll
    for (uint32_t k = 0; k < 2; ++k)
        if (k * 64u + lane < n16)
            t4[k] = load16_nt(codes + crow0 * row_bytes + (k * 64u + lane) * 16u);
    const int32_t* lp = pos + (int64_t)(bh / (uint32_t)H) * n + j0;
    const int32_t my_pos = lane < (uint32_t)nt ? lp[lane] : -1;
    const int64_t p = (int64_t)tile * D + (int64_t)c * 8;
    const float4 s_a = *reinterpret_cast<const float4*>(scale + p);
    const float4 s_b = *reinterpret_cast<const float4*>(scale + p + 4);
    const float4 z_a = *reinterpret_cast<const float4*>(zero + p);
    const float4 z_b = *reinterpret_cast<const float4*>(zero + p + 4);
#pragma unroll
    for (uint32_t k = 0; k < 2; ++k)
        if (k * 64u + lane < n16)
            *reinterpret_cast<uint4*>(lds + (k * 64u + lane) * 16u) = t4[k];
    if (lane < 32u) pos_s[lane] = my_pos;
    wave_lds_sync();
    const float sc[8] = {s_a.x, s_a.y, s_a.z, s_a.w, s_b.x, s_b.y, s_b.z, s_b.w};
    const float z[8] = {z_a.x, z_a.y, z_a.z, z_a.w, z_b.x, z_b.y, z_b.z, z_b.w};
    uint16_t* dst = out + (int64_t)bh * S * D + (int64_t)c * 8;
#pragma unroll
    for (int32_t i = 0; i < 8; ++i) {
        const int32_t t = (int32_t)part + 4 * i;
        if (t < nt) {
            const int32_t s = pos_s[t];
            const uint64_t q = lds_key_codes<BITS>(lds + t * row_bytes + c * BITS);
            if (s >= 0 && s < S)
                store16_nt(dst + (int64_t)s * D, dequant_chunk<DT, BITS>(q, sc, z));
        }
    }
}

// Values: one lane per (row of the set, CPL consecutive 8-channel chunks):
// one CPL * BITS-byte code load and one (scale, zero) load per value group
// it touches (groups are multiples of 8 channels).  The reconstruction goes
// out through LDS: a wave's rows are parked there and stored with one lane
// per 16-byte chunk, so each store instruction writes whole rows.

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
        if constexpr (BITS <= 4) {
            if (D8 == 16 && j.group <= 32)
                return launch_kernel((list_dequant_keys_split_kernel<DT, BITS>),
                                     dim3((uint32_t)(j.B * j.H) * NG), dim3(64),
                                     0, j.stream, j.codes, j.scale, j.zero, NG,
                                     (int32_t)j.S, (int32_t)j.n, (int32_t)j.H,
                                     (int32_t)j.group, j.pos, o);
        }
        const uint32_t n = (uint32_t)(j.B * j.H) * NG * D8;
        const int32_t stage = BITS <= 4 && 64 % D8 == 0 && D8 >= 4 &&
                              j.group <= 32 && (j.group * BITS) % 16 == 0;
        return launch_kernel((list_dequant_keys_kernel<DT, BITS>),
                             dim3((n + 255u) / 256u), dim3(256), 0, j.stream,
                             j.codes, j.scale, j.zero, n, D8, NG, (int32_t)j.S,
                             (int32_t)j.n, (int32_t)j.H, (int32_t)j.group,
                             j.pos, o, stage);
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
