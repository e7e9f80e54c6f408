// KIVI per-channel key quantization for gfx950.
//
// KIVI blog post on the fused Metal kernels, section "Kernel A -- per-channel
// keys": the group of channel d runs along the strided token axis, so a
// thread owning whole groups needs no cross-thread reduction.  Here one lane
// owns a chunk of 8 adjacent channels of one (bh, token group) tile: every
// step of its token loop is one 128-bit load, and the 16 lanes covering a
// 128-channel row read 256 contiguous bytes, so a wave's loads stay fully
// coalesced without a transpose (the post's discarded transposing variant).
// The whole group (up to 32 tokens x 8 channels) stays in registers, so the
// input is read from HBM exactly once: min/max, then codes, from the same
// registers.
//
// Code stores: a lane's codes for one token are only BITS bytes, one per
// row of the tile.  When the wave holds whole tiles (64 % (D/8) == 0) of full
// groups, the tiles' codes form one contiguous block; the wave writes its
// codes into LDS and stores the block with 16-byte stores instead of 2-byte
// ones.  Other waves store directly from each lane.
#include "kivi_device.h"
#include "kivi_launch.h"
#include "kivi_rows.h"
#include "kivi_key_split.h"

namespace kivi {

constexpr int kKeyGMax = 32;   // largest group held in registers

// Quantize and store the GMAX tokens of a whole group from registers.
template <int DT, int BITS, bool WQ, bool WR, int GMAX>
__device__ __forceinline__ void emit_full(const uint4 (&v)[GMAX],
                                          const Params (&pk)[8], uint8_t* dst,
                                          int64_t row_bytes, uint16_t* rdst,
                                          int64_t D) {
#pragma unroll
    for (int t = 0; t < GMAX; ++t) {
        uint4 r;
        const uint64_t q = quant_chunk<DT, BITS, true, WR>(v[t], pk, &r);
        if constexpr (WQ) store_codes<BITS>(dst + t * row_bytes, q);
        if constexpr (WR) store16_nt(rdst + t * D, r);
    }
}

// The rare cases (a ragged last group, a group size below the register
// capacity, or a scale outside the fast division's range): a rolled loop
// that reloads each token (an L2 hit), so the unrolled register path is the
// only large code in the kernel.
template <int DT, int BITS, bool WQ, bool WR, bool FAST>
__device__ __forceinline__ void emit_rolled(const uint16_t* src,
                                            const Params (&pk)[8], int32_t n,
                                            uint8_t* dst, int64_t row_bytes,
                                            uint16_t* rdst, int64_t D) {
#pragma unroll 1
    for (int32_t t = 0; t < n; ++t) {
        const uint4 v = load16(src + (int64_t)t * D);
        uint4 r;
        const uint64_t q = quant_chunk<DT, BITS, FAST, WR>(v, pk, &r);
        if constexpr (WQ) store_codes<BITS>(dst + t * row_bytes, q);
        if constexpr (WR) store16_nt(rdst + t * D, r);
    }
}

// LDS bytes per wave for the staged code block: tiles of GMAX rows padded
// by up to 16 bytes each (bank spreading), at most 64 tiles.  Used when a
// lane's share of the block is whole 16-byte pieces.
template <int GMAX, int BITS>
struct KeyStage {
    static constexpr bool kUsed = BITS <= 4 && (GMAX * BITS) % 16 == 0;
    static constexpr int kWaveBytes = kUsed ? 64 * GMAX * BITS + 64 * 16 : 0;
};

// Work item = (bh, token group g, channel chunk c), flattened with c fastest
// so consecutive lanes take consecutive 16-byte chunks of the same rows.
// A lane past the last item mirrors the last item's loads (in bounds) and
// stores nothing, so every lane reaches the wave-wide steps.
// GMAX >= group size; a ragged last group loads its last token again in the
// missing slots, which is the pages' edge-replicate padding and leaves the
// min/max unchanged, so the min/max carries no guards.
// WQ: write codes + params.  WR: write the reconstruction (fused path).
// stage: the host's verdict that whole waves hold whole tiles (64 % D8 == 0,
// group == GMAX), so that a wave's codes are one contiguous block.
// (Staging the fused path's reconstruction the same way, so that each store
// instruction writes a contiguous KiB, measured 1-2% slower than the direct
// 16-byte stores below, and was left out.)
template <int DT, int BITS, int GMAX, bool WQ, bool WR>
__global__ __launch_bounds__(256) void quant_keys_kernel(
    const uint16_t* __restrict__ x, uint32_t n_items, uint32_t D8,
    uint32_t NG, int32_t S, int32_t G, uint8_t* __restrict__ codes,
    float* __restrict__ scale, float* __restrict__ zero,
    uint16_t* __restrict__ recon, int32_t stage) {
    using Stage = KeyStage<GMAX, BITS>;
    constexpr bool kStaged = WQ && Stage::kUsed;
    __shared__ __attribute__((aligned(16)))
    uint8_t lds[kStaged ? 4 * Stage::kWaveBytes : 16];

    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const bool valid = gid < n_items;
    const uint32_t item = valid ? gid : n_items - 1u;
    const uint32_t c = item % D8;
    const uint32_t tile = item / D8;
    const uint32_t g = tile % NG;
    const uint32_t bh = tile / NG;
    const int32_t s0 = (int32_t)g * G;
    const int32_t nt = min(G, S - s0);
    const int64_t D = (int64_t)D8 * 8;
    const int64_t row0 = (int64_t)bh * S + s0;
    const uint16_t* src = x + row0 * D + (int64_t)c * 8;
    const bool full = nt == GMAX;

    uint4 v[GMAX];
    if (full) {
#pragma unroll
        for (int t = 0; t < GMAX; ++t) v[t] = load16_nt(src + t * D);
    } else {
#pragma unroll
        for (int t = 0; t < GMAX; ++t) v[t] = load16_nt(src + min(t, nt - 1) * D);
    }

    MinMax8<DT> mm;
    mm.init(v[0]);
#pragma unroll
    for (int t = 1; t < GMAX; ++t) mm.add(v[t]);
    float lo[8], hi[8];
    mm.get(lo, hi);

    Params pk[8];
    bool fast = true;
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        pk[k] = make_params<BITS>(lo[k], hi[k]);
        fast = fast && pk[k].fast;
    }

    if (WQ && valid) {
        const int64_t p = ((int64_t)bh * NG + g) * D + (int64_t)c * 8;
        float4* ps = reinterpret_cast<float4*>(scale + p);
        float4* pz = reinterpret_cast<float4*>(zero + p);
        ps[0] = make_float4(pk[0].scale, pk[1].scale, pk[2].scale, pk[3].scale);
        ps[1] = make_float4(pk[4].scale, pk[5].scale, pk[6].scale, pk[7].scale);
        pz[0] = make_float4(pk[0].zero, pk[1].zero, pk[2].zero, pk[3].zero);
        pz[1] = make_float4(pk[4].zero, pk[5].zero, pk[6].zero, pk[7].zero);
    }

    const int64_t row_bytes = (int64_t)D8 * BITS;   // D * BITS / 8
    uint8_t* dst = WQ ? codes + row0 * row_bytes + (int64_t)c * BITS : nullptr;
    uint16_t* rdst = WR ? recon + row0 * D + (int64_t)c * 8 : nullptr;

    if constexpr (kStaged) {
        // Wave-uniform choice: every lane valid, full and fast.
        if (stage && __all(valid && full && fast)) {
            const uint32_t lane = threadIdx.x & 63u;
            uint8_t* L = lds + (threadIdx.x >> 6) * Stage::kWaveBytes;
            const uint32_t tile_bytes = GMAX * D8 * BITS;
            const uint32_t pad = (D8 * BITS + 15u) & ~15u;
            const uint32_t ts = tile_bytes + pad;   // padded tile stride
            uint8_t* mine = L + (lane / D8) * ts + c * BITS;
#pragma unroll
            for (int t = 0; t < GMAX; ++t) {
                uint4 r;
                const uint64_t q = quant_chunk<DT, BITS, true, WR>(v[t], pk, &r);
                if constexpr (BITS == 1) mine[t * row_bytes] = (uint8_t)q;
                else if constexpr (BITS == 2)
                    *reinterpret_cast<uint16_t*>(mine + t * row_bytes) = (uint16_t)q;
                else
                    *reinterpret_cast<uint32_t*>(mine + t * row_bytes) = (uint32_t)q;
                if constexpr (WR) store16_nt(rdst + t * D, r);
            }
            wave_lds_sync();
            // Lane 0 holds chunk 0 of the wave's first tile; the wave's
            // tiles are consecutive token groups, i.e. consecutive rows.
            const uint32_t b_lo = __builtin_amdgcn_readfirstlane(
                (uint32_t)((uint64_t)row0 & 0xffffffffu));
            const uint32_t b_hi = __builtin_amdgcn_readfirstlane(
                (uint32_t)((uint64_t)row0 >> 32));
            const int64_t wrow0 = (int64_t)(((uint64_t)b_hi << 32) | b_lo);
            uint8_t* wdst = codes + wrow0 * row_bytes;
            constexpr int kChunks = GMAX * BITS / 16;   // 16-byte chunks per lane
#pragma unroll
            for (int k = 0; k < kChunks; ++k) {
                const uint32_t off = (k * 64u + lane) * 16u;   // in the block
                const uint32_t t_idx = off / tile_bytes;
                const uint4 q = *reinterpret_cast<const uint4*>(
                    L + t_idx * ts + (off - t_idx * tile_bytes));
                *reinterpret_cast<uint4*>(wdst + off) = q;
            }
            return;
        }
    }
    if (!valid) return;
    if (fast && full)
        emit_full<DT, BITS, WQ, WR, GMAX>(v, pk, dst, row_bytes, rdst, D);
    else if (fast)
        emit_rolled<DT, BITS, WQ, WR, true>(src, pk, nt, dst, row_bytes, rdst, D);
    else
        emit_rolled<DT, BITS, WQ, WR, false>(src, pk, nt, dst, row_bytes, rdst, D);
}

// The split variant for small flushes (its lane body: kivi_key_split.h).
// Codes of at most 4 bits are staged through LDS at D = 128 (measured 2-3%
// faster on the large dense workloads than 2-byte code stores).
template <int DT, int BITS, int TPL, int SPLIT, bool WQ, bool WR, bool ILV,
          typename IO>
__global__ __launch_bounds__(64) void quant_keys_split_kernel(
    IO io, uint32_t n_lanes, uint32_t D8, uint32_t NG,
    uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, uint16_t* __restrict__ recon) {
    quant_keys_split_body<DT, BITS, TPL, SPLIT, WQ, WR, ILV, IO, (BITS <= 4), 64>(
        io, blockIdx.x * 64u + threadIdx.x, n_lanes, D8, NG, codes, scale, zero,
        recon);
}

// Lanes per group: 4 below kKeySplitBelow (bh, group, chunk) items, 2 above
// (kivi_key_split.h).

template <int DT, int BITS, int GMAX, int SPLIT, bool WQ, bool WR>
static hipError_t launch_keys_split_t(const QuantJob& j) {
    constexpr int TPL = GMAX / SPLIT;
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t NG = (uint32_t)((j.S + j.group - 1) / j.group);
    const uint64_t n_lanes = (uint64_t)j.BH * NG * D8 * SPLIT;
    const uint32_t blocks = (uint32_t)((n_lanes + 63) / 64);
    const DenseRows io{static_cast<const uint16_t*>(j.x), (int32_t)j.S, NG,
                       (int32_t)j.group};
    // a tensor under 4 GiB: row addresses as 32-bit offsets (measured 1-2%
    // faster on the roundtrip tensor)
    if ((uint64_t)j.BH * (uint64_t)j.S * (uint64_t)j.D * 2u < (1ull << 32)) {
        DenseRows32 io32;
        static_cast<DenseRows&>(io32) = io;
        return launch_kernel(
            (quant_keys_split_kernel<DT, BITS, TPL, SPLIT, WQ, WR, true, DenseRows32>),
            dim3(blocks), dim3(64), 0, j.stream, io32, (uint32_t)n_lanes, D8, NG,
            j.codes, j.scale, j.zero, static_cast<uint16_t*>(j.recon));
    }
    return launch_kernel(
        (quant_keys_split_kernel<DT, BITS, TPL, SPLIT, WQ, WR, true, DenseRows>),
        dim3(blocks), dim3(64), 0, j.stream, io, (uint32_t)n_lanes, D8, NG,
        j.codes, j.scale, j.zero, static_cast<uint16_t*>(j.recon));
}

template <int DT, int BITS, int GMAX, int SPLIT>
static hipError_t launch_keys_split_mode(const QuantJob& j) {
    const bool wq = j.codes != nullptr;
    const bool wr = j.recon != nullptr;
    if (wq && wr) return launch_keys_split_t<DT, BITS, GMAX, SPLIT, true, true>(j);
    if (wq) return launch_keys_split_t<DT, BITS, GMAX, SPLIT, true, false>(j);
    return launch_keys_split_t<DT, BITS, GMAX, SPLIT, false, true>(j);
}

template <int DT, int BITS, int GMAX, bool WQ, bool WR>
static hipError_t launch_keys_t(const QuantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t NG = (uint32_t)((j.S + j.group - 1) / j.group);
    const uint64_t n_items = (uint64_t)j.BH * NG * D8;
    const uint32_t blocks = (uint32_t)((n_items + 255) / 256);
    const int32_t stage = 64 % D8 == 0 && j.group == GMAX;
    return launch_kernel((quant_keys_kernel<DT, BITS, GMAX, WQ, WR>),
                       dim3(blocks), dim3(256), 0, j.stream,
                       static_cast<const uint16_t*>(j.x), (uint32_t)n_items,
                       D8, NG, (int32_t)j.S, (int32_t)j.group, j.codes,
                       j.scale, j.zero, static_cast<uint16_t*>(j.recon),
                       stage);
}

template <int DT, int BITS, int GMAX>
static hipError_t launch_keys_mode(const QuantJob& j) {
    const bool wq = j.codes != nullptr;
    const bool wr = j.recon != nullptr;
    const uint64_t D8 = (uint64_t)(j.D / 8);
    const uint64_t NG = (uint64_t)((j.S + j.group - 1) / j.group);
    const uint64_t items = (uint64_t)j.BH * NG * D8;
    // n_lanes = items * SPLIT must fit the kernel's 32-bit lane index.
    // With a reconstruction to write, 4 lanes per item at every size: each
    // reconstruction store instruction then covers 4 consecutive rows of a
    // tile (1 KiB at D = 128), and those stores are most of the kernel's
    // bytes.  A/B on the roundtrip tensor: the fused kernel 1-2% faster; the
    // quantize-only kernel 8-10% slower the same way, its loads dominating.
    if ((items < kKeySplitBelow || (wr && items < (1ull << 30))) && 64 % (D8 * 4) == 0)
        return launch_keys_split_mode<DT, BITS, GMAX, 4>(j);
    if (items < (1ull << 31) && 64 % (D8 * 2) == 0)
        return launch_keys_split_mode<DT, BITS, GMAX, 2>(j);
    if (wq && wr) return launch_keys_t<DT, BITS, GMAX, true, true>(j);
    if (wq) return launch_keys_t<DT, BITS, GMAX, true, false>(j);
    return launch_keys_t<DT, BITS, GMAX, false, true>(j);
}

template <int DT, int BITS>
static hipError_t launch_keys_gmax(const QuantJob& j) {
    if (j.group <= 8) return launch_keys_mode<DT, BITS, 8>(j);
    if (j.group <= 16) return launch_keys_mode<DT, BITS, 16>(j);
    return launch_keys_mode<DT, BITS, 32>(j);
}

template <int DT>
static hipError_t launch_keys_bits(const QuantJob& j) {
    switch (j.bits) {
        case 1: return launch_keys_gmax<DT, 1>(j);
        case 2: return launch_keys_gmax<DT, 2>(j);
        case 4: return launch_keys_gmax<DT, 4>(j);
        default: return launch_keys_gmax<DT, 8>(j);
    }
}

template <int DT, int BITS, int GMAX, int SPLIT>
static hipError_t launch_cache_keys_t(const CacheFlushJob& j) {
    constexpr int TPL = GMAX / SPLIT;
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t NG = (uint32_t)(j.F / j.G_k);      // groups flushed per bh
    const uint64_t n_lanes = (uint64_t)j.BH * NG * D8 * SPLIT;
    const uint32_t blocks = (uint32_t)((n_lanes + 63) / 64);
    const CacheRows io{static_cast<const uint16_t*>(j.ring),
                       static_cast<const uint16_t*>(j.in), (int32_t)j.ring_len,
                       (int32_t)j.n_in, (int32_t)j.T, (int32_t)j.Q,
                       (int32_t)j.F, (int32_t)j.S_max,
                       (uint32_t)((j.S_max + j.G_k - 1) / j.G_k),
                       (int32_t)j.G_k};
    return launch_kernel(
        (quant_keys_split_kernel<DT, BITS, TPL, SPLIT, true, false, true,
                                 CacheRows>),
        dim3(blocks), dim3(64), 0, j.stream, io, (uint32_t)n_lanes, D8, NG,
        j.codes, j.scale, j.zero, (uint16_t*)nullptr);
}

template <int DT, int BITS, int GMAX>
static hipError_t launch_cache_keys_gmax(const CacheFlushJob& j) {
    const uint64_t D8 = (uint64_t)(j.D / 8);
    const uint64_t items = (uint64_t)j.BH * (j.F / j.G_k) * D8;
    if (items < kKeySplitBelow && 64 % (D8 * 4) == 0)
        return launch_cache_keys_t<DT, BITS, GMAX, 4>(j);
    return launch_cache_keys_t<DT, BITS, GMAX, 2>(j);
}

template <int DT, int BITS>
static hipError_t launch_cache_keys_bits(const CacheFlushJob& j) {
    if (j.G_k <= 8) return launch_cache_keys_gmax<DT, BITS, 8>(j);
    if (j.G_k <= 16) return launch_cache_keys_gmax<DT, BITS, 16>(j);
    return launch_cache_keys_gmax<DT, BITS, 32>(j);
}

template <int DT>
static hipError_t launch_cache_keys_dt(const CacheFlushJob& j) {
    switch (j.bits) {
        case 1: return launch_cache_keys_bits<DT, 1>(j);
        case 2: return launch_cache_keys_bits<DT, 2>(j);
        case 4: return launch_cache_keys_bits<DT, 4>(j);
        default: return launch_cache_keys_bits<DT, 8>(j);
    }
}

template <int DT, int BITS, int GMAX, int SPLIT>
static hipError_t launch_list_keys_t(const ListJob& j) {
    constexpr int TPL = GMAX / SPLIT;
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t NG = (uint32_t)((j.n + j.group - 1) / j.group);
    const uint64_t n_lanes = (uint64_t)j.B * j.H * NG * D8 * SPLIT;
    const uint32_t blocks = (uint32_t)((n_lanes + 63) / 64);
    const ListRows io{static_cast<const uint16_t*>(j.x), j.pos, (int32_t)j.S,
                      (int32_t)j.n, (int32_t)j.H, NG, (int32_t)j.group};
    return launch_kernel(
        (quant_keys_split_kernel<DT, BITS, TPL, SPLIT, true, false, true,
                                 ListRows>),
        dim3(blocks), dim3(64), 0, j.stream, io, (uint32_t)n_lanes, D8, NG,
        j.codes, j.scale, j.zero, (uint16_t*)nullptr);
}

template <int DT, int BITS, int GMAX>
static hipError_t launch_list_keys_gmax(const ListJob& j) {
    const uint64_t D8 = (uint64_t)(j.D / 8);
    const uint64_t items = (uint64_t)j.B * j.H * ((j.n + j.group - 1) / j.group) * D8;
    if (items < kKeySplitBelow && 64 % (D8 * 4) == 0)
        return launch_list_keys_t<DT, BITS, GMAX, 4>(j);
    return launch_list_keys_t<DT, BITS, GMAX, 2>(j);
}

template <int DT, int BITS>
static hipError_t launch_list_keys_bits(const ListJob& j) {
    if (j.group <= 8) return launch_list_keys_gmax<DT, BITS, 8>(j);
    if (j.group <= 16) return launch_list_keys_gmax<DT, BITS, 16>(j);
    return launch_list_keys_gmax<DT, BITS, 32>(j);
}

template <int DT>
static hipError_t launch_list_keys_dt(const ListJob& j) {
    switch (j.bits) {
        case 1: return launch_list_keys_bits<DT, 1>(j);
        case 2: return launch_list_keys_bits<DT, 2>(j);
        case 4: return launch_list_keys_bits<DT, 4>(j);
        default: return launch_list_keys_bits<DT, 8>(j);
    }
}

template <int DT, int BITS, int GMAX, int SPLIT, bool WQ, bool WR>
static hipError_t launch_sink_keys_t(const SinkQuantJob& j) {
    constexpr int TPL = GMAX / SPLIT;
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t NG = (uint32_t)((j.S + j.group - 1) / j.group);
    const uint64_t n_lanes = (uint64_t)j.B * j.H * NG * D8 * SPLIT;
    const uint32_t blocks = (uint32_t)((n_lanes + 63) / 64);
    SinkRows io{};
    io.x = static_cast<const uint16_t*>(j.k);
    io.S = (int32_t)j.S;
    io.NG = NG;
    io.G = (int32_t)j.group;
    io.idx = j.idx;
    io.n_sink = (int32_t)j.n_sink;
    io.H = (int32_t)j.H;
    return launch_kernel(
        (quant_keys_split_kernel<DT, BITS, TPL, SPLIT, WQ, WR, true, SinkRows>),
        dim3(blocks), dim3(64), 0, j.stream, io, (uint32_t)n_lanes, D8, NG,
        j.codes, j.scale, j.zero, static_cast<uint16_t*>(j.recon));
}

template <int DT, int BITS, int GMAX, int SPLIT>
static hipError_t launch_sink_keys_mode(const SinkQuantJob& j) {
    const bool wq = j.codes != nullptr, wr = j.recon != nullptr;
    if (wq && wr) return launch_sink_keys_t<DT, BITS, GMAX, SPLIT, true, true>(j);
    if (wq) return launch_sink_keys_t<DT, BITS, GMAX, SPLIT, true, false>(j);
    return launch_sink_keys_t<DT, BITS, GMAX, SPLIT, false, true>(j);
}

template <int DT, int BITS, int GMAX>
static hipError_t launch_sink_keys_gmax(const SinkQuantJob& j) {
    const uint64_t D8 = (uint64_t)(j.D / 8);
    const uint64_t items = (uint64_t)j.B * j.H * ((j.S + j.group - 1) / j.group) * D8;
    if (items < kKeySplitBelow && 64 % (D8 * 4) == 0)
        return launch_sink_keys_mode<DT, BITS, GMAX, 4>(j);
    return launch_sink_keys_mode<DT, BITS, GMAX, 2>(j);
}

template <int DT, int BITS>
static hipError_t launch_sink_keys_bits(const SinkQuantJob& j) {
    if (j.group <= 8) return launch_sink_keys_gmax<DT, BITS, 8>(j);
    if (j.group <= 16) return launch_sink_keys_gmax<DT, BITS, 16>(j);
    return launch_sink_keys_gmax<DT, BITS, 32>(j);
}

template <int DT>
static hipError_t launch_sink_keys_dt(const SinkQuantJob& j) {
    switch (j.bits) {
        case 1: return launch_sink_keys_bits<DT, 1>(j);
        case 2: return launch_sink_keys_bits<DT, 2>(j);
        case 4: return launch_sink_keys_bits<DT, 4>(j);
        default: return launch_sink_keys_bits<DT, 8>(j);
    }
}

// KIVI-Sink keys on the split kernel; the caller guarantees D / 8 a power
// of two <= 32, group <= 32 and fewer than 2^31 lanes.
hipError_t launch_split_quant_keys_sink(const SinkQuantJob& j) {
    return j.dtype == DT_F16 ? launch_sink_keys_dt<DT_F16>(j)
                             : launch_sink_keys_dt<DT_BF16>(j);
}

hipError_t launch_list_quant_keys(const ListJob& j) {
    return j.dtype == DT_F16 ? launch_list_keys_dt<DT_F16>(j)
                             : launch_list_keys_dt<DT_BF16>(j);
}

// The caller guarantees: D / 8 a power of two <= 32, G_k <= 32, F a
// multiple of G_k, and fewer than 2^31 lanes.
hipError_t launch_cache_flush_keys(const CacheFlushJob& j) {
    return j.dtype == DT_F16 ? launch_cache_keys_dt<DT_F16>(j)
                             : launch_cache_keys_dt<DT_BF16>(j);
}

hipError_t launch_quant_keys(const QuantJob& j) {
    // Register-resident fast path: whole 8-channel chunks, groups <= 32
    // tokens, and an item count that fits 32-bit indexing.
    const int64_t NG = (j.S + j.group - 1) / j.group;
    const bool fits = (uint64_t)j.BH * NG * (j.D / 8) < (1ull << 31) &&
                      j.S < (1ll << 31) && j.D < (1ll << 28);
    if (j.D % 8 != 0 || j.group > kKeyGMax || !fits)
        return launch_generic_quant_keys(j);
    return j.dtype == DT_F16 ? launch_keys_bits<DT_F16>(j)
                             : launch_keys_bits<DT_BF16>(j);
}

}  // namespace kivi
