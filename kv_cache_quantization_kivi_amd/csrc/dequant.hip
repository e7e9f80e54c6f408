// KIVI dequantization for gfx950: recon = RN(RN(code * scale) + zero),
// narrowed to fp16/bf16 with round to nearest even (KIVI blog post on the
// fused Metal kernels, section "What we're actually optimizing", and "Three
// ways to be off by one bit", item 1: the product is rounded before the add).
//
// Both kernels move whole 16-byte pieces with non-temporal accesses: the
// codes and params are read once and the reconstruction is written once, so
// none of it should displace reusable lines or linger as dirty lines for the
// next kernel to evict.  Where the natural per-lane access would be narrow
// or strided, a wave moves its contiguous block through LDS instead.
//
// Keys: one lane owns an 8-channel chunk of one (bh, token group) tile, so
// its 8 scales and 8 zeros are loaded once (four 128-bit loads) and reused
// for every token of the group.  A lane's codes are BITS bytes per token
// (one per row); when the wave holds whole tiles of full groups, the tiles'
// codes are one contiguous block that the wave reads with 16-byte loads into
// LDS, and each lane then picks its codes from LDS.
// Values: one lane owns 32 consecutive channels of a row (as in the value
// quantizer): one 4*BITS-byte code load, one (scale, zero) per group it
// touches, and 64 bytes of recon, which go out through LDS as 1 KiB
// contiguous stores when rows tile the lanes exactly.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kDqTokUnroll = 8;   // tokens per step of the keys' token loop

__device__ __forceinline__ float4 load_f4_nt(const float* p) {
    const u32x4_t q =
        __builtin_nontemporal_load(reinterpret_cast<const u32x4_t*>(p));
    return make_float4(__uint_as_float(q.x), __uint_as_float(q.y),
                       __uint_as_float(q.z), __uint_as_float(q.w));
}

// Codes of one token of a chunk from LDS (BITS bytes).
template <int BITS>
__device__ __forceinline__ uint64_t lds_codes(const uint8_t* p) {
    if constexpr (BITS == 1) return *p;
    else if constexpr (BITS == 2) return *reinterpret_cast<const uint16_t*>(p);
    else return *reinterpret_cast<const uint32_t*>(p);
}

// Staged key codes: at most 32 tokens per group and BITS <= 4, so a wave's
// block is at most 64 * 32 * BITS bytes (plus up to 16 bytes of padding per
// tile, at most 64 tiles).
template <int BITS>
struct DqKeyStage {
    static constexpr int kWaveBytes = BITS <= 4 ? 64 * 32 * BITS + 64 * 16 : 0;
};

// stage: the host's verdict that a wave of full tiles has one contiguous
// code block of whole 16-byte pieces per lane (64 % D8 == 0, group <= 32,
// group * BITS % 16 == 0, BITS <= 4).
// (Gathering a few tokens of reconstruction in LDS so that every store
// instruction writes a contiguous KiB measured 3-4% slower than the direct
// 16-byte stores below, and was left out.)
template <int DT, int BITS>
__global__ __launch_bounds__(256) void dequant_keys_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint32_t n_items, uint32_t D8,
    uint32_t NG, int32_t S, int32_t G, uint16_t* __restrict__ out,
    int32_t stage) {
    constexpr int kWaveBytes = DqKeyStage<BITS>::kWaveBytes;
    __shared__ __attribute__((aligned(16)))
    uint8_t lds[BITS <= 4 ? 4 * kWaveBytes : 16];

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

    const int64_t p = ((int64_t)bh * NG + g) * D + (int64_t)c * 8;
    const float4 s_a = load_f4_nt(scale + p);
    const float4 s_b = load_f4_nt(scale + p + 4);
    const float4 z_a = load_f4_nt(zero + p);
    const float4 z_b = load_f4_nt(zero + p + 4);
    const float sc[8] = {s_a.x, s_a.y, s_a.z, s_a.w, s_b.x, s_b.y, s_b.z, s_b.w};
    const float z[8] = {z_a.x, z_a.y, z_a.z, z_a.w, z_b.x, z_b.y, z_b.z, z_b.w};

    const int64_t row_bytes = (int64_t)D8 * BITS;
    uint16_t* dst = out + row0 * D + (int64_t)c * 8;

    if constexpr (BITS <= 4) {
        if (stage && __all(valid && nt == G)) {
            const uint32_t lane = threadIdx.x & 63u;
            uint8_t* L = lds + (threadIdx.x >> 6) * kWaveBytes;
            const uint32_t tile_bytes = (uint32_t)G * D8 * BITS;
            const uint32_t ts = tile_bytes + ((D8 * BITS + 15u) & ~15u);
            // Lane 0 holds chunk 0 of the wave's first tile; the wave's
            // tiles are consecutive token groups, i.e. consecutive rows.
            const uint32_t b_lo = __builtin_amdgcn_readfirstlane(
                (uint32_t)((uint64_t)row0 & 0xffffffffu));
            const uint32_t b_hi = __builtin_amdgcn_readfirstlane(
                (uint32_t)((uint64_t)row0 >> 32));
            const int64_t wrow0 = (int64_t)(((uint64_t)b_hi << 32) | b_lo);
            const uint8_t* wsrc = codes + wrow0 * row_bytes;
            const uint32_t n16 = (uint32_t)G * BITS / 16;   // pieces per lane
            uint4 t4[8];
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k)
                if (k < n16) t4[k] = load16_nt(wsrc + (k * 64u + lane) * 16u);
#pragma unroll
            for (uint32_t k = 0; k < 8; ++k) {
                if (k < n16) {
                    const uint32_t off = (k * 64u + lane) * 16u;
                    const uint32_t ti = off / tile_bytes;
                    *reinterpret_cast<uint4*>(L + ti * ts + (off - ti * tile_bytes)) = t4[k];
                }
            }
            wave_lds_sync();
            const uint8_t* mine = L + (lane / D8) * ts + c * BITS;
#pragma unroll kDqTokUnroll
            for (int32_t t = 0; t < G; ++t)
                store16_nt(dst + (int64_t)t * D,
                           dequant_chunk<DT, BITS>(lds_codes<BITS>(mine + t * row_bytes), sc, z));
            return;
        }
    }
    if (!valid) return;
    const uint8_t* src = codes + row0 * row_bytes + (int64_t)c * BITS;
    for (int32_t t0 = 0; t0 < nt; t0 += kDqTokUnroll) {
        uint64_t q[kDqTokUnroll];
#pragma unroll
        for (int u = 0; u < kDqTokUnroll; ++u)
            if (t0 + u < nt) q[u] = load_codes<BITS>(src + (t0 + u) * row_bytes);
#pragma unroll
        for (int u = 0; u < kDqTokUnroll; ++u)
            if (t0 + u < nt)
                store16_nt(dst + (int64_t)(t0 + u) * D,
                           dequant_chunk<DT, BITS>(q[u], sc, z));
    }
}

// Recon staging layout, as in the value quantizer: chunk j of a wave's
// 4 KiB block at LDS byte (j + j/4) * 16 (lane stride 80 bytes).
constexpr int kDqRecLaneStride = 80;
constexpr int kDqRecWaveBytes = 64 * kDqRecLaneStride;

// GPL: groups per lane (4: G = 8, 2: G = 16, 1: G a multiple of 32, so a
// lane's 4 chunks, which start at a multiple of 4 chunks, share one group).
// lp: log2 of lanes per row P; vec: D % 32 == 0 (a lane's codes are one
// naturally aligned load); tile: D / 32 is a power of two (a wave's recon is
// one contiguous 4 KiB block).
// u: the lane's index over all lanes of the launch (blocks of 256 lanes);
// lds: the block's 4 * kDqRecWaveBytes staging bytes.
template <int DT, int BITS, int GPL>
__device__ __forceinline__ void dequant_values_body(
    uint64_t u, uint8_t* lds, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, const float* __restrict__ zero,
    int64_t n_rows, uint32_t D8, uint32_t lp, uint32_t G8, uint32_t NGD,
    int32_t vec, int32_t tile, uint16_t* __restrict__ out) {
    const uint32_t c = (uint32_t)(u & ((1u << lp) - 1u));
    const int64_t row = (int64_t)(u >> lp);
    const bool row_ok = row < n_rows;
    const int32_t ch0 = (int32_t)c * 4;
    const int32_t nch = min(4, (int32_t)D8 - ch0);
    const bool staged = tile && __all(row_ok);
    if (!staged && (!row_ok || nch <= 0)) return;

    const int64_t row_bytes = (int64_t)D8 * BITS;
    const uint8_t* csrc = codes + row * row_bytes + (int64_t)ch0 * BITS;
    uint64_t q[4];
    if (vec && nch == 4) {
        if constexpr (BITS == 1) {
            const uint32_t w = __builtin_nontemporal_load(
                reinterpret_cast<const uint32_t*>(csrc));
#pragma unroll
            for (int k = 0; k < 4; ++k) q[k] = (w >> (8 * k)) & 0xffu;
        } else if constexpr (BITS == 2) {
            typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
            const u32x2_t w = __builtin_nontemporal_load(
                reinterpret_cast<const u32x2_t*>(csrc));
            q[0] = w.x & 0xffffu;
            q[1] = w.x >> 16;
            q[2] = w.y & 0xffffu;
            q[3] = w.y >> 16;
        } else if constexpr (BITS == 4) {
            const uint4 w = load16_nt(csrc);
            q[0] = w.x;
            q[1] = w.y;
            q[2] = w.z;
            q[3] = w.w;
        } else {
            const uint4 a = load16_nt(csrc);
            const uint4 b = load16_nt(csrc + 16);
            q[0] = (uint64_t)a.x | ((uint64_t)a.y << 32);
            q[1] = (uint64_t)a.z | ((uint64_t)a.w << 32);
            q[2] = (uint64_t)b.x | ((uint64_t)b.y << 32);
            q[3] = (uint64_t)b.z | ((uint64_t)b.w << 32);
        }
    } else {
#pragma unroll
        for (int k = 0; k < 4; ++k)
            q[k] = k < nch ? load_codes<BITS>(csrc + k * BITS) : 0;
    }

    // Params: in-lane group t starts at chunk ch0 + t*CPG and lies in row
    // group (ch0 + t*CPG) / G8; a group past the row's end reads the lane's
    // first group instead (its result is never stored).
    constexpr int CPG = 4 / GPL;
    float gs[GPL], gz[GPL];
#pragma unroll
    for (int t = 0; t < GPL; ++t) {
        const int32_t ch = ch0 + t * CPG;
        const int64_t pi =
            row * NGD + (uint32_t)(ch < (int32_t)D8 ? ch : ch0) / G8;
        gs[t] = __builtin_nontemporal_load(scale + pi);
        gz[t] = __builtin_nontemporal_load(zero + pi);
    }

    uint4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const float s = gs[k / CPG], zz = gz[k / CPG];
        const float s8[8] = {s, s, s, s, s, s, s, s};
        const float z8[8] = {zz, zz, zz, zz, zz, zz, zz, zz};
        r[k] = dequant_chunk<DT, BITS>(q[k], s8, z8);
    }

    if (staged) {
        const uint32_t lane = threadIdx.x & 63u;
        uint8_t* L = lds + (threadIdx.x >> 6) * kDqRecWaveBytes;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            *reinterpret_cast<uint4*>(L + lane * kDqRecLaneStride + k * 16) = r[k];
        wave_lds_sync();
        uint8_t* wdst = reinterpret_cast<uint8_t*>(out + (u - lane) * 32);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t off = k * 1024u + lane * 16u;
            store16_nt(wdst + off, *reinterpret_cast<const uint4*>(
                                       L + (off >> 6) * kDqRecLaneStride + (off & 63u)));
        }
    } else {
        uint16_t* dst = out + row * ((int64_t)D8 * 8) + (int64_t)ch0 * 8;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            if (k < nch) store16_nt(dst + k * 8, r[k]);
    }
}

template <int DT, int BITS, int GPL>
__global__ __launch_bounds__(256) void dequant_values_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, int64_t n_rows, uint32_t D8, uint32_t lp,
    uint32_t G8, uint32_t NGD, int32_t vec, int32_t tile,
    uint16_t* __restrict__ out) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kDqRecWaveBytes];
    dequant_values_body<DT, BITS, GPL>((uint64_t)blockIdx.x * 256u + threadIdx.x,
                                       lds, codes, scale, zero, n_rows, D8, lp,
                                       G8, NGD, vec, tile, out);
}

// Small dequantizations (a decode-time flush) have too few (bh, group,
// chunk) items to fill the GPU, and one lane storing a whole group is then
// the latency.  Here each item is split over SPLIT lanes, interleaved: part
// p takes tokens p, p + SPLIT, ... (lanes: chunk fastest, then part, so one
// store instruction covers SPLIT consecutive rows); the lanes share the
// item's scale and zero and need no communication.
constexpr int kDqKeySplit = 4;
constexpr uint64_t kDqKeySplitBelow = 256ull * 256ull;

// lid: the lane's index over all lanes of the launch (waves 64-aligned).
template <int DT, int BITS>
__device__ __forceinline__ void dequant_keys_split_body(
    uint32_t lid, const uint8_t* __restrict__ codes,
    const float* __restrict__ scale, const float* __restrict__ zero,
    uint32_t n_lanes, uint32_t D8, uint32_t NG, int32_t S, int32_t G,
    uint16_t* __restrict__ out) {
    if (lid >= n_lanes) return;
    const uint32_t c = lid % D8;
    const uint32_t part = (lid / D8) % kDqKeySplit;
    const uint32_t tile = lid / (D8 * kDqKeySplit);
    const uint32_t g = tile % NG;
    const uint32_t bh = tile / NG;
    const int32_t s0 = (int32_t)g * G;
    const int32_t nt = min(G, S - s0);
    // tokens part + SPLIT * t < nt
    const int32_t n = (nt - (int32_t)part + kDqKeySplit - 1) / kDqKeySplit;
    if (n <= 0) return;
    const int64_t D = (int64_t)D8 * 8;
    const int64_t row0 = (int64_t)bh * S + s0;

    const int64_t p = ((int64_t)bh * NG + g) * D + (int64_t)c * 8;
    const float4 s_a = load_f4_nt(scale + p);
    const float4 s_b = load_f4_nt(scale + p + 4);
    const float4 z_a = load_f4_nt(zero + p);
    const float4 z_b = load_f4_nt(zero + p + 4);
    const float sc[8] = {s_a.x, s_a.y, s_a.z, s_a.w, s_b.x, s_b.y, s_b.z, s_b.w};
    const float z[8] = {z_a.x, z_a.y, z_a.z, z_a.w, z_b.x, z_b.y, z_b.z, z_b.w};

    const int64_t row_bytes = (int64_t)D8 * BITS;
    const int64_t cs = kDqKeySplit * row_bytes;   // code row stride
    const int64_t rs = kDqKeySplit * D;           // recon row stride
    const uint8_t* src = codes + (row0 + part) * row_bytes + (int64_t)c * BITS;
    uint16_t* dst = out + (row0 + part) * D + (int64_t)c * 8;
    for (int32_t t0 = 0; t0 < n; t0 += kDqTokUnroll) {
        uint64_t q[kDqTokUnroll];
#pragma unroll
        for (int u = 0; u < kDqTokUnroll; ++u)
            if (t0 + u < n) q[u] = load_codes<BITS>(src + (t0 + u) * cs);
#pragma unroll
        for (int u = 0; u < kDqTokUnroll; ++u)
            if (t0 + u < n)
                store16_nt(dst + (int64_t)(t0 + u) * rs,
                           dequant_chunk<DT, BITS>(q[u], sc, z));
    }
}

template <int DT, int BITS>
__global__ __launch_bounds__(64) void dequant_keys_split_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint32_t n_lanes, uint32_t D8,
    uint32_t NG, int32_t S, int32_t G, uint16_t* __restrict__ out) {
    dequant_keys_split_body<DT, BITS>(blockIdx.x * 64u + threadIdx.x, codes,
                                      scale, zero, n_lanes, D8, NG, S, G, out);
}

// Large calls of whole groups: the split layout above (four lanes per
// chunk with interleaved tokens, so that every store instruction writes four
// consecutive rows of a tile: 1 KiB at D = 128), with the codes read the way
// the one-lane kernel reads them: the wave's tiles are consecutive rows, so
// their codes are one contiguous block of 16 * G * BITS bytes, loaded once
// with 16-byte loads into LDS, from where each lane picks its own.  A wave
// with lanes past the end takes the unstaged split body.
template <int DT, int BITS>
__global__ __launch_bounds__(64) void dequant_keys_staged_kernel(
    const uint8_t* __restrict__ codes, const float* __restrict__ scale,
    const float* __restrict__ zero, uint32_t n_lanes, uint32_t D8,
    uint32_t NG, int32_t G, uint16_t* __restrict__ out) {
    static_assert(BITS <= 4, "a wave's block is at most 2 KiB");
    __shared__ __attribute__((aligned(16))) uint8_t lds[16 * 32 * BITS];
    const uint32_t lane = threadIdx.x;
    const uint32_t lid = blockIdx.x * 64u + lane;
    const int32_t S = (int32_t)NG * G;
    if (!__all(lid < n_lanes)) {
        dequant_keys_split_body<DT, BITS>(lid, codes, scale, zero, n_lanes, D8,
                                          NG, S, G, out);
        return;
    }
    const uint32_t c = lid % D8;
    const uint32_t part = (lid / D8) % kDqKeySplit;
    const uint32_t tile = lid / (D8 * kDqKeySplit);
    const uint32_t tile0 = (blockIdx.x * 64u) / (D8 * kDqKeySplit);
    const int64_t D = (int64_t)D8 * 8;
    const int64_t row_bytes = (int64_t)D8 * BITS;

    // the wave's code block: tiles tile0.. are rows tile0 * G.. (S = NG * G)
    const uint8_t* wsrc = codes + (int64_t)tile0 * G * row_bytes;
    const uint32_t n16 = (uint32_t)G * BITS;          // 16-byte pieces
    uint4 t4[2];
#pragma unroll
    for (uint32_t k = 0; k < 2; ++k)
        if (k * 64u + lane < n16) t4[k] = load16_nt(wsrc + (k * 64u + lane) * 16u);
    const int64_t p = (int64_t)tile * D + (int64_t)c * 8;   // tile = bh * NG + g
    const float4 s_a = load_f4_nt(scale + p);
    const float4 s_b = load_f4_nt(scale + p + 4);
    const float4 z_a = load_f4_nt(zero + p);
    const float4 z_b = load_f4_nt(zero + p + 4);
#pragma unroll
    for (uint32_t k = 0; k < 2; ++k)
        if (k * 64u + lane < n16)
            *reinterpret_cast<uint4*>(lds + (k * 64u + lane) * 16u) = t4[k];
    wave_lds_sync();
    const float sc[8] = {s_a.x, s_a.y, s_a.z, s_a.w, s_b.x, s_b.y, s_b.z, s_b.w};
    const float z[8] = {z_a.x, z_a.y, z_a.z, z_a.w, z_b.x, z_b.y, z_b.z, z_b.w};

    const uint8_t* mine = lds + ((tile - tile0) * G + part) * row_bytes + c * BITS;
    uint16_t* dst = out + ((int64_t)tile * G + part) * D + (int64_t)c * 8;
    const int32_t n = (G - (int32_t)part + kDqKeySplit - 1) / kDqKeySplit;
#pragma unroll
    for (int32_t i = 0; i < 32 / kDqKeySplit; ++i)
        if (i < n)
            store16_nt(dst + (int64_t)i * kDqKeySplit * D,
                       dequant_chunk<DT, BITS>(
                           lds_codes<BITS>(mine + i * kDqKeySplit * row_bytes), sc, z));
}

template <int DT, int BITS>
static hipError_t launch_dq_keys_t(const DequantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint64_t items = (uint64_t)j.BH * ((j.S + j.group - 1) / j.group) * D8;
    if constexpr (BITS <= 4) {
        if (items >= kDqKeySplitBelow && 64 % (D8 * kDqKeySplit) == 0 &&
            j.group <= 32 && j.S % j.group == 0 &&
            items * kDqKeySplit < (1ull << 32)) {
            const uint32_t NG = (uint32_t)(j.S / j.group);
            const uint64_t n_lanes = items * kDqKeySplit;
            return launch_kernel((dequant_keys_staged_kernel<DT, BITS>),
                                 dim3((uint32_t)((n_lanes + 63) / 64)), dim3(64),
                                 0, j.stream, j.codes, j.scale, j.zero,
                                 (uint32_t)n_lanes, D8, NG, (int32_t)j.group,
                                 static_cast<uint16_t*>(j.out));
        }
    }
    if (items < kDqKeySplitBelow) {
        const uint32_t NG = (uint32_t)((j.S + j.group - 1) / j.group);
        const uint64_t n_lanes = (uint64_t)j.BH * NG * D8 * kDqKeySplit;
        return launch_kernel((dequant_keys_split_kernel<DT, BITS>),
                             dim3((uint32_t)((n_lanes + 63) / 64)), dim3(64), 0,
                             j.stream, j.codes, j.scale, j.zero,
                             (uint32_t)n_lanes, D8, NG, (int32_t)j.S,
                             (int32_t)j.group, static_cast<uint16_t*>(j.out));
    }
    const uint32_t NG = (uint32_t)((j.S + j.group - 1) / j.group);
    const uint64_t n_items = (uint64_t)j.BH * NG * D8;
    const uint32_t blocks = (uint32_t)((n_items + 255) / 256);
    const int32_t stage = BITS <= 4 && 64 % D8 == 0 && j.group <= 32 &&
                          (j.group * BITS) % 16 == 0;
    return launch_kernel((dequant_keys_kernel<DT, BITS>), dim3(blocks),
                       dim3(256), 0, j.stream, j.codes, j.scale, j.zero,
                       (uint32_t)n_items, D8, NG, (int32_t)j.S,
                       (int32_t)j.group, static_cast<uint16_t*>(j.out), stage);
}

template <int DT, int BITS, int GPL>
static hipError_t launch_dq_values_gpl(const DequantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t lpr = (D8 + 3) / 4;
    const uint32_t lp = log2_ceil(lpr);
    const uint32_t NGD = (uint32_t)((j.D + j.group - 1) / j.group);
    const int64_t n_rows = j.BH * j.S;
    const uint64_t lanes = (uint64_t)n_rows << lp;
    const uint32_t blocks = (uint32_t)((lanes + 255) / 256);
    const int32_t vec = (D8 % 4) == 0;
    const int32_t tile = vec && (1u << lp) == lpr;
    return launch_kernel((dequant_values_kernel<DT, BITS, GPL>), dim3(blocks),
                       dim3(256), 0, j.stream, j.codes, j.scale, j.zero,
                       n_rows, D8, lp, (uint32_t)(j.group / 8), NGD, vec, tile,
                       static_cast<uint16_t*>(j.out));
}

template <int DT, int BITS>
static hipError_t launch_dq_values_t(const DequantJob& j) {
    if (j.group == 8) return launch_dq_values_gpl<DT, BITS, 4>(j);
    if (j.group == 16) return launch_dq_values_gpl<DT, BITS, 2>(j);
    return launch_dq_values_gpl<DT, BITS, 1>(j);
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
    // A lane's chunks map onto whole groups (group 8, 16 or a multiple of
    // 32); rows of at most 64 lanes (D <= 2048).
    const bool grp_ok = j.group == 8 || j.group == 16 || j.group % 32 == 0;
    if (j.D % 8 != 0 || !grp_ok || j.D > 2048 || j.BH * j.S >= (1ll << 40))
        return launch_generic_dequant(j, false);
    KIVI_DISPATCH_DQ(launch_dq_values_t, j);
}

// ---- keys and values of a small flush in one launch --------------------

// Blocks [0, v_blocks) run the value body (groups of 32 * k channels), the
// rest the 4-lane split key body on 256 lanes per block.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void dequant_kv_kernel(
    const uint8_t* __restrict__ kc, const float* __restrict__ ks,
    const float* __restrict__ kz, uint32_t k_lanes, uint32_t D8, uint32_t NG,
    int32_t S, int32_t G, uint16_t* __restrict__ kout,
    const uint8_t* __restrict__ vc, const float* __restrict__ vs,
    const float* __restrict__ vz, int64_t n_rows, uint32_t lp, uint32_t G8,
    uint32_t NGD, int32_t vec, int32_t tile, uint16_t* __restrict__ vout,
    uint32_t v_blocks) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kDqRecWaveBytes];
    if (blockIdx.x < v_blocks)
        dequant_values_body<DT, BITS, 1>((uint64_t)blockIdx.x * 256u + threadIdx.x,
                                         lds, vc, vs, vz, n_rows, D8, lp, G8, NGD,
                                         vec, tile, vout);
    else
        dequant_keys_split_body<DT, BITS>((blockIdx.x - v_blocks) * 256u + threadIdx.x,
                                          kc, ks, kz, k_lanes, D8, NG, S, G, kout);
}

template <int DT, int BITS>
static hipError_t launch_dq_kv_t(const DequantJob& k, const DequantJob& v) {
    const uint32_t D8 = (uint32_t)(k.D / 8);
    const uint32_t NG = (uint32_t)((k.S + k.group - 1) / k.group);
    const uint64_t k_lanes = (uint64_t)k.BH * NG * D8 * kDqKeySplit;
    const uint32_t lpr = (D8 + 3) / 4;
    const uint32_t lp = log2_ceil(lpr);
    const uint32_t NGD = (uint32_t)((v.D + v.group - 1) / v.group);
    const int64_t n_rows = v.BH * v.S;
    const uint64_t v_lanes = (uint64_t)n_rows << lp;
    const uint32_t v_blocks = (uint32_t)((v_lanes + 255) / 256);
    const int32_t vec = (D8 % 4) == 0;
    const int32_t tile = vec && (1u << lp) == lpr;
    const uint32_t blocks = v_blocks + (uint32_t)((k_lanes + 255) / 256);
    return launch_kernel((dequant_kv_kernel<DT, BITS>), dim3(blocks), dim3(256),
                         0, k.stream, k.codes, k.scale, k.zero, (uint32_t)k_lanes,
                         D8, NG, (int32_t)k.S, (int32_t)k.group,
                         static_cast<uint16_t*>(k.out), v.codes, v.scale, v.zero,
                         n_rows, lp, (uint32_t)(v.group / 8), NGD, vec, tile,
                         static_cast<uint16_t*>(v.out), v_blocks);
}

template <int DT, int BITS>
static hipError_t launch_dq_kv_pair(const DequantJob& k, const DequantJob& v) {
    return launch_dq_kv_t<DT, BITS>(k, v);
}

// The caller has validated both jobs (same shape, bits and output dtype).
// One launch when the keys take the split kernel and the value groups are
// multiples of 32 channels; otherwise the two single launches, keys first.
hipError_t launch_dequant_kv(const DequantJob& k, const DequantJob& v) {
    const uint64_t D8 = (uint64_t)(k.D / 8);
    const uint64_t items = (uint64_t)k.BH * ((k.S + k.group - 1) / k.group) * D8;
    const bool pair = k.D % 8 == 0 && k.D <= 2048 && items < kDqKeySplitBelow &&
                      k.S < (1ll << 31) && v.group % 32 == 0;
    if (!pair) {
        const hipError_t e = launch_dequant_keys(k);
        return e != hipSuccess ? e : launch_dequant_values(v);
    }
    if (k.out_dtype == DT_F16) {
        switch (k.bits) {
            case 1: return launch_dq_kv_pair<DT_F16, 1>(k, v);
            case 2: return launch_dq_kv_pair<DT_F16, 2>(k, v);
            case 4: return launch_dq_kv_pair<DT_F16, 4>(k, v);
            default: return launch_dq_kv_pair<DT_F16, 8>(k, v);
        }
    }
    switch (k.bits) {
        case 1: return launch_dq_kv_pair<DT_BF16, 1>(k, v);
        case 2: return launch_dq_kv_pair<DT_BF16, 2>(k, v);
        case 4: return launch_dq_kv_pair<DT_BF16, 4>(k, v);
        default: return launch_dq_kv_pair<DT_BF16, 8>(k, v);
    }
}

}  // namespace kivi
