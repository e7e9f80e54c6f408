// Where the quantizers find token rows and where they put a token's
// outputs.  Three layouts share the kernels:
//   DenseRows - one [BH, S, D] tensor, outputs at the same (bh, token);
//   CacheRows - a flush of tokens [Q, Q + F) of a residual-window cache:
//               token s < T is in its ring slot s % ring_len of
//               [BH, ring_len, D], token s >= T is row s - T of the appended
//               [BH, n_in, D]; outputs go to the cache's compressed store at
//               token s of [BH, S_max, ...] (key groups counted from 0);
//   ListRows  - a listed token set: row j of head bh is token
//               pos[bh / H][j] of [BH, S, D] (the H heads of a sequence share
//               one list); outputs are the set's own rows [BH, n, ...].
// Token indices are 32-bit: the launchers only use these layouts for
// tensors of fewer than 2^31 tokens per bh.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

// The rows of one key tile (the tokens s0, s0 + 1, ... of one bh): row t is
// at a + t * D for t < split, else at b + (t - split) * D.
struct TileRows {
    const uint16_t* a;
    const uint16_t* b;
    int32_t split;
    __device__ const uint16_t* row(int32_t t, int64_t D) const {
        return t < split ? a + t * D : b + (t - split) * D;
    }
};

struct DenseRows {
    const uint16_t* x;
    int32_t S;      // tokens per bh
    uint32_t NG;    // key groups per bh (input = output)
    int32_t G;      // key group size

    // key tiles: group g of bh
    __device__ int32_t first(uint32_t g) const { return (int32_t)g * G; }
    __device__ int32_t count(int32_t s0) const { return min(G, S - s0); }
    __device__ TileRows tile(uint32_t bh, int32_t s0, int64_t D) const {
        const uint16_t* a = x + ((int64_t)bh * S + s0) * D;
        return TileRows{a, a, 0x7fffffff};
    }
    __device__ int64_t out_row(uint32_t bh, int32_t s) const {
        return (int64_t)bh * S + s;
    }
    __device__ int64_t out_group(uint32_t bh, uint32_t g) const {
        return (int64_t)bh * NG + g;
    }
    // no sinks: every token takes part in its group's min/max
    static constexpr bool kSinks = false;
    static constexpr bool kOff32 = false;
    __device__ uint32_t sink_mask(uint32_t, int32_t, int32_t) const { return 0u; }
    // value rows: row r of the flattened [BH * S] rows
    static constexpr bool kContiguous = true;
    __device__ const uint16_t* vrow(int64_t r, int64_t D) const {
        return x + r * D;
    }
    __device__ int64_t vout(int64_t r) const { return r; }
};

// DenseRows of a tensor under 4 GiB: the key body forms each row's address
// as a 32-bit byte offset from x.
struct DenseRows32 : DenseRows {
    static constexpr bool kOff32 = true;
};

struct CacheRows {
    const uint16_t* ring;   // [BH, ring_len, D]
    const uint16_t* in;     // [BH, n_in, D]
    int32_t ring_len, n_in, T, Q, F, S_max;
    uint32_t NG_out;        // key groups per bh in the compressed store
    int32_t G;              // key group size (the flush unit)

    __device__ const uint16_t* token(uint32_t bh, int32_t s, int64_t D) const {
        return s < T ? ring + ((int64_t)bh * ring_len + s % ring_len) * D
                     : in + ((int64_t)bh * n_in + (s - T)) * D;
    }
    __device__ int32_t first(uint32_t g) const { return Q + (int32_t)g * G; }
    __device__ int32_t count(int32_t) const { return G; }
    // A group is G-aligned and the ring a multiple of G long, so the tile's
    // ring slots are consecutive; a tile may continue into the new tokens.
    __device__ TileRows tile(uint32_t bh, int32_t s0, int64_t D) const {
        const uint16_t* nb = in + ((int64_t)bh * n_in + (s0 - T)) * D;
        if (s0 >= T) return TileRows{nb, nb, 0x7fffffff};
        return TileRows{ring + ((int64_t)bh * ring_len + s0 % ring_len) * D,
                        in + (int64_t)bh * n_in * D, T - s0};
    }
    __device__ int64_t out_row(uint32_t bh, int32_t s) const {
        return (int64_t)bh * S_max + s;
    }
    __device__ int64_t out_group(uint32_t bh, uint32_t g) const {
        return (int64_t)bh * NG_out + (uint32_t)(Q / G) + g;
    }
    static constexpr bool kSinks = false;
    static constexpr bool kOff32 = false;
    __device__ uint32_t sink_mask(uint32_t, int32_t, int32_t) const { return 0u; }
    static constexpr bool kContiguous = false;
    __device__ const uint16_t* vrow(int64_t r, int64_t D) const {
        const uint32_t bh = (uint32_t)r / (uint32_t)F;
        return token(bh, Q + (int32_t)((uint32_t)r - bh * (uint32_t)F), D);
    }
    __device__ int64_t vout(int64_t r) const {
        const uint32_t bh = (uint32_t)r / (uint32_t)F;
        return (int64_t)bh * S_max + Q + ((uint32_t)r - bh * (uint32_t)F);
    }
};

// The ring store (RingStore, kivi_launch.h): lane gid of 2 * half, keys
// then values, (bh, token j, 16-byte chunk c) with c fastest, so a wave
// copies whole contiguous rows.  Token s = s_first + j is row s - T of the
// appended block and goes to slot s % ring_len; the ring is read again by
// the next flush, so the stores are plain (cached).
__device__ __forceinline__ void ring_store_lane(const RingStore& r,
                                                uint32_t gid) {
    if (gid >= 2u * r.half) return;
    const bool val = gid >= r.half;
    const uint32_t lid = val ? gid - r.half : gid;
    const uint32_t c = lid % r.D8;
    const uint32_t j = (lid / r.D8) % r.ncopy;
    const uint32_t bh = lid / (r.D8 * r.ncopy);
    const int32_t s = r.s_first + (int32_t)j;
    const int64_t D = (int64_t)r.D8 * 8;
    const uint16_t* in = val ? r.v_in : r.k_in;
    uint16_t* ring = val ? r.v_ring : r.k_ring;
    const uint4 v = load16_nt(in + ((int64_t)bh * r.n_in + (s - r.T)) * D + c * 8);
    *reinterpret_cast<uint4*>(ring + ((int64_t)bh * r.ring_len + s % r.ring_len) * D +
                              c * 8) = v;
}

// Rows of one key tile of a listed set: row t is token pos[t] of the bh's
// [S, D] rows.  A position outside [0, S) is clamped, so a bad list reads
// in bounds (its results are unspecified).
struct ListTile {
    const uint16_t* x;     // the bh's token 0
    const int32_t* pos;    // the tile's first list entry
    int32_t S;
    __device__ const uint16_t* row(int32_t t, int64_t D) const {
        const int32_t p = min(max(pos[t], 0), S - 1);
        return x + (int64_t)p * D;
    }
};

struct ListRows {
    const uint16_t* x;     // [BH, S, D]
    const int32_t* pos;    // [BH / H, n]
    int32_t S, n, H;
    uint32_t NG;           // key groups of the set per bh
    int32_t G;

    __device__ int32_t first(uint32_t g) const { return (int32_t)g * G; }
    __device__ int32_t count(int32_t s0) const { return min(G, n - s0); }
    __device__ ListTile tile(uint32_t bh, int32_t s0, int64_t D) const {
        return ListTile{x + (int64_t)bh * S * D,
                        pos + (int64_t)(bh / (uint32_t)H) * n + s0, S};
    }
    __device__ int64_t out_row(uint32_t bh, int32_t s) const {
        return (int64_t)bh * n + s;
    }
    __device__ int64_t out_group(uint32_t bh, uint32_t g) const {
        return (int64_t)bh * NG + g;
    }
    static constexpr bool kSinks = false;
    static constexpr bool kOff32 = false;
    __device__ uint32_t sink_mask(uint32_t, int32_t, int32_t) const { return 0u; }
    // value rows: row r of the flattened [BH * n] set rows (fewer than 2^31)
    static constexpr bool kContiguous = false;
    __device__ const uint16_t* vrow(int64_t r, int64_t D) const {
        const uint32_t bh = (uint32_t)r / (uint32_t)n;
        const int32_t j = (int32_t)((uint32_t)r - bh * (uint32_t)n);
        const int32_t p = min(max(pos[(int64_t)(bh / (uint32_t)H) * n + j], 0), S - 1);
        return x + ((int64_t)bh * S + p) * D;
    }
    __device__ int64_t vout(int64_t r) const { return r; }
};

// KIVI-Sink: dense [BH, S, D] keys whose sinks (a list of n_sink positions
// per sequence of H heads, [BH / H, n_sink]) take no part in their group's
// min/max.  sink_mask(bh, s0, nt): bit t set when token s0 + t is a sink
// (t < nt <= 32); positions outside [0, S) match nothing.
struct SinkRows : DenseRows {
    const int32_t* idx;
    int32_t n_sink, H;
    static constexpr bool kSinks = true;
    __device__ uint32_t sink_mask(uint32_t bh, int32_t s0, int32_t nt) const {
        const int32_t* l = idx + (int64_t)(bh / (uint32_t)H) * n_sink;
        uint32_t m = 0u;
        for (int32_t i = 0; i < n_sink; ++i) {
            const int32_t t = l[i] - s0;
            if ((uint32_t)t < (uint32_t)nt) m |= 1u << t;
        }
        return m;
    }
};

}  // namespace kivi
