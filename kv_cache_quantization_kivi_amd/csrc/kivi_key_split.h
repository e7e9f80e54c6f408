// The split key quantizer's lane body (KIVI blog post on the fused Metal
// kernels, section "Kernel A -- per-channel keys"), shared by its own
// kernel and by the launch that quantizes keys and values together.
#pragma once
#include "kivi_device.h"
#include "kivi_rows.h"

namespace kivi {

// Lanes per group.  Below kKeySplitBelow (bh, group, chunk) items (a
// decode-time flush) one lane per item would leave most of the GPU's 256
// CUs idle, so each group takes 4 lanes; above it 2 lanes per group, which
// measured 3-13% faster than one lane per group on the large workloads (half
// the registers per lane, so more waves in flight, for one xor shuffle and
// one repeated parameter computation per group).
constexpr uint64_t kKeySplitBelow = 256ull * 256ull;
constexpr int kKeyGMaxPair = 32;   // key groups of the paired K+V launch: 17..32

// Small flushes (a decode-time flush of a few dozen tokens per head) have
// too few (bh, token group, chunk) items to fill the GPU, and one lane
// working through a whole group is then the latency.  This variant gives the
// chunk of a group to SPLIT lanes of one wave, TPL = GMAX / SPLIT tokens
// each, interleaved: lane part p takes tokens p, p + SPLIT, p + 2 SPLIT, ...
// Lanes are laid out channel chunk fastest, then part, so one load or store
// instruction covers SPLIT consecutive rows of a tile, and the SPLIT lanes
// of a group are D8 lanes apart, where their min/max meet through xor
// shuffles; then every lane codes its own tokens.  A lane's token index is
// clamped to the group's last token (the edge padding), so lanes of a
// ragged group load in bounds and store only real tokens.  Lanes past the
// end mirror the last lane; items come in whole groups of D8*SPLIT lanes
// aligned inside the wave, so they only ever meet each other.
// Code and store a lane's first n tokens; token t's code row is at
// dst + t * cstride bytes and its recon row at rdst + t * rstride elements.
// With SINKS, bit t of `sinks` marks the lane's token t as a sink: code 0,
// and its own row as the reconstruction.
template <int DT, int BITS, bool WQ, bool WR, bool FAST, int TPL, bool SINKS,
          bool TO_LDS = false>
__device__ __forceinline__ void emit_split(const uint4 (&v)[TPL],
                                           const Params (&pk)[8], int32_t n,
                                           uint8_t* dst, int64_t cstride,
                                           uint16_t* rdst, int64_t rstride,
                                           uint32_t sinks) {
#pragma unroll
    for (int t = 0; t < TPL; ++t) {
        if (t < n) {
            uint4 r;
            uint64_t q = quant_chunk<DT, BITS, FAST, WR>(v[t], pk, &r);
            if constexpr (SINKS) {
                if ((sinks >> t) & 1u) {
                    q = 0;
                    r = v[t];
                }
            }
            // quantize-only: codes streamed (measured faster for this
            // kernel and for the kernels after it); the fused form keeps
            // plain stores (streaming them beside the reconstruction was
            // slower).  TO_LDS: dst is the tile's code block in LDS.
            if constexpr (WQ && TO_LDS) store_codes<BITS, false>(dst + t * cstride, q);
            else if constexpr (WQ) store_codes<BITS, !WR>(dst + t * cstride, q);
            if constexpr (WR) store16_nt(rdst + t * rstride, r);
        }
    }
}

// IO: the row layout (DenseRows, CacheRows or ListRows, kivi_rows.h); NG here is the
// number of groups per bh that this launch quantizes.
// gid: the lane's index over all lanes of the launch (waves 64-aligned).
// STAGE (with D = 128): a tile's codes are gathered in LDS and stored as
// 16-byte pieces of its contiguous code block (a group's rows are
// consecutive in every row layout), instead of one BITS-byte store per
// lane and token; BLOCK is the launch's block size, whose lanes map to
// tiles from lane 0 (gid = block * BLOCK + thread).
template <int DT, int BITS, int TPL, int SPLIT, bool WQ, bool WR, bool ILV,
          typename IO, bool STAGE = false, int BLOCK = 64>
__device__ __forceinline__ void quant_keys_split_body(
    IO io, uint32_t gid, uint32_t n_lanes, uint32_t D8, uint32_t NG,
    uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, uint16_t* __restrict__ recon) {
    const bool valid = gid < n_lanes;
    const uint32_t lid = valid ? gid : n_lanes - 1u;
    const uint32_t c = lid % D8;
    const uint32_t part = (lid / D8) % SPLIT;
    const uint32_t tile = lid / (D8 * SPLIT);
    const uint32_t g = tile % NG;
    const uint32_t bh = tile / NG;
    const int32_t s0 = io.first(g);
    const int32_t nt = io.count(s0);
    const int64_t D = (int64_t)D8 * 8;

    const auto rows = io.tile(bh, s0, D);
    uint4 v[TPL];
    uint32_t lane_sinks = 0;   // bit t: this lane's token t is a sink
    uint32_t group_sinks = 0;  // bit t: token s0 + t is a sink
    if constexpr (IO::kSinks) group_sinks = io.sink_mask(bh, s0, nt);
    if constexpr (IO::kOff32) {
        // a 32-bit byte offset from the wave-uniform base: the loads take
        // the scalar-base form and the per-token address is one 32-bit add
        const char* xb = reinterpret_cast<const char*>(io.x);
        const uint32_t b0 =
            (uint32_t)((((uint64_t)bh * (uint32_t)io.S + (uint32_t)s0) * (uint64_t)D +
                        (uint64_t)c * 8u) * 2u);
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
            const int32_t tt = min(ILV ? (int32_t)part + SPLIT * t
                                       : (int32_t)part * TPL + t, nt - 1);
            v[t] = load16_nt(xb + (b0 + (uint32_t)tt * (uint32_t)D * 2u));
        }
    } else {
#pragma unroll
        for (int t = 0; t < TPL; ++t) {
            const int32_t tt = min(ILV ? (int32_t)part + SPLIT * t
                                       : (int32_t)part * TPL + t, nt - 1);
            v[t] = load16_nt(rows.row(tt, D) + (int64_t)c * 8);
            if constexpr (IO::kSinks) lane_sinks |= ((group_sinks >> tt) & 1u) << t;
        }
    }

    // A sink takes no part in the min/max: it is replaced there by the
    // group's first token that is not a sink (a duplicate changes neither).
    uint4 fill = v[0];
    bool no_tokens = false;    // every token of the group is a sink
    if constexpr (IO::kSinks) {
        const uint32_t live = ~group_sinks & (nt < 32 ? (1u << nt) - 1u : ~0u);
        no_tokens = live == 0u;
        if (lane_sinks != 0u && !no_tokens)
            fill = load16_nt(rows.row(__builtin_ctz(live), D) + (int64_t)c * 8);
    }
    const auto tok = [&](int t) -> uint4 {
        if constexpr (IO::kSinks) return ((lane_sinks >> t) & 1u) ? fill : v[t];
        return v[t];
    };
    MinMax8<DT> mm;
    mm.init(tok(0));
#pragma unroll
    for (int t = 1; t < TPL; ++t) mm.add(tok(t));
#pragma unroll
    for (int k = 1; k < SPLIT; k <<= 1) mm.combine_xor((int)D8 * k);
    float lo[8], hi[8];
    mm.get(lo, hi);

    Params pk[8];
    bool fast = true;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        pk[k] = make_params<BITS>(no_tokens ? 0.0f : lo[k], no_tokens ? 0.0f : hi[k]);
        fast = fast && pk[k].fast;
    }
    if (!valid) return;

    if (WQ && part == 0) {
        const int64_t p = io.out_group(bh, g) * D + (int64_t)c * 8;
        const uint4 s0 = make_uint4(__float_as_uint(pk[0].scale), __float_as_uint(pk[1].scale),
                                    __float_as_uint(pk[2].scale), __float_as_uint(pk[3].scale));
        const uint4 s1 = make_uint4(__float_as_uint(pk[4].scale), __float_as_uint(pk[5].scale),
                                    __float_as_uint(pk[6].scale), __float_as_uint(pk[7].scale));
        const uint4 z0 = make_uint4(__float_as_uint(pk[0].zero), __float_as_uint(pk[1].zero),
                                    __float_as_uint(pk[2].zero), __float_as_uint(pk[3].zero));
        const uint4 z1 = make_uint4(__float_as_uint(pk[4].zero), __float_as_uint(pk[5].zero),
                                    __float_as_uint(pk[6].zero), __float_as_uint(pk[7].zero));
        if constexpr (!WR) {   // params streamed like the codes
            store16_nt(scale + p, s0);
            store16_nt(scale + p + 4, s1);
            store16_nt(zero + p, z0);
            store16_nt(zero + p + 4, z1);
        } else {
            uint4* ps = reinterpret_cast<uint4*>(scale + p);
            uint4* pz = reinterpret_cast<uint4*>(zero + p);
            ps[0] = s0;
            ps[1] = s1;
            pz[0] = z0;
            pz[1] = z1;
        }
    }
    // real tokens of this lane: part + SPLIT * t < nt (interleaved), or
    // part * TPL + t < nt (blocked)
    const int32_t n = ILV ? ((int32_t)nt - (int32_t)part + SPLIT - 1) / SPLIT
                          : (int32_t)nt - (int32_t)part * TPL;
    const int32_t first = ILV ? (int32_t)part : (int32_t)part * TPL;
    const int32_t step = ILV ? SPLIT : 1;
    const int64_t row_bytes = (int64_t)D8 * BITS;
    const int64_t orow = io.out_row(bh, s0 + first);
    uint16_t* rdst = WR ? recon + orow * D + (int64_t)c * 8 : nullptr;
    if constexpr (STAGE && WQ) {
        constexpr int TL = 16 * SPLIT;                // a tile's lanes at D = 128
        constexpr int TB = TPL * SPLIT * 16 * BITS;   // a tile's code bytes, at most
        static_assert(BLOCK % TL == 0, "tiles whole inside a block");
        __shared__ __attribute__((aligned(16))) uint8_t code_s[BLOCK / TL][TB];
        if (D8 == 16) {                               // launch-uniform
            uint8_t* tl = code_s[threadIdx.x / TL];
            uint8_t* ldst = tl + (int64_t)first * row_bytes + (int64_t)c * BITS;
            if (fast)
                emit_split<DT, BITS, WQ, WR, true, TPL, IO::kSinks, true>(
                    v, pk, n, ldst, step * row_bytes, rdst, step * D, lane_sinks);
            else
                emit_split<DT, BITS, WQ, WR, false, TPL, IO::kSinks, true>(
                    v, pk, n, ldst, step * row_bytes, rdst, step * D, lane_sinks);
            wave_lds_sync();
            // nt rows of 16 * BITS bytes: a multiple of 16 bytes
            const int32_t bytes = nt * (int32_t)row_bytes;
            uint8_t* gdst = codes + io.out_row(bh, s0) * row_bytes;
            const int32_t lt = (int32_t)(threadIdx.x % TL);
#pragma unroll
            for (int k = 0; k < (TB + 16 * TL - 1) / (16 * TL); ++k) {
                const int32_t piece = lt + TL * k;
                if (piece * 16 < bytes) {
                    const uint4 w = *reinterpret_cast<const uint4*>(tl + piece * 16);
                    if constexpr (!WR) store16_nt(gdst + piece * 16, w);
                    else *reinterpret_cast<uint4*>(gdst + piece * 16) = w;
                }
            }
            return;
        }
    }
    uint8_t* dst = WQ ? codes + orow * row_bytes + (int64_t)c * BITS : nullptr;
    if (fast)
        emit_split<DT, BITS, WQ, WR, true, TPL, IO::kSinks>(
            v, pk, n, dst, step * row_bytes, rdst, step * D, lane_sinks);
    else
        emit_split<DT, BITS, WQ, WR, false, TPL, IO::kSinks>(
            v, pk, n, dst, step * row_bytes, rdst, step * D, lane_sinks);
}


}  // namespace kivi
