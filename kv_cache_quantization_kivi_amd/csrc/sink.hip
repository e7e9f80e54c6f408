// KIVI-Sink for gfx950 (VeloxQuant-MLX 0.24.1 package page, section
// "KVSink-adapted sink protection"): per sequence, the n_sink token
// positions whose keys have the largest L2 norm, averaged over the KV heads,
// are sinks; they stay in 16-bit form and are left out of the min/max of
// their key groups, so a high-magnitude sink no longer stretches its
// neighbours' scale.
//
// Three steps, each one launch:
//   scores  - one lane per (sequence b, token s) walks the token's key row
//             in every head (rows staged through LDS by coalesced wave
//             loads) and forms the mean norm in a fixed order:
//             per head fma-accumulated squares in channel order, the
//             correctly rounded square root, the head-order sum, one division
//             by H;
//   select  - one block per sequence takes the n_sink best (score, position)
//             pairs in the order "higher score, then lower position", round
//             by round: round r keeps the best pair that comes after round
//             r - 1's pick in that order (a total order, so no list of taken
//             positions is needed);
//   keys    - per-channel key quantization, one lane per (bh, key group,
//             8-channel chunk) holding the group in registers, whose min/max
//             skips the group's sinks; a sink gets code 0 and, in the fused
//             form, reconstructs to itself.
// Value groups are single tokens, so sinks change nothing there: the plain
// value quantizer serves, and gather / restore keep and put back the sinks'
// 16-bit rows.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

// ---- scores -------------------------------------------------------------

// One wave per (sequence b, tile of 64 tokens).  The tile's rows of one
// head are contiguous, so the wave reads them with fully coalesced 16-byte
// loads (consecutive lanes on consecutive 16-byte pieces), parks them in
// LDS, and each lane then walks its own token's row from LDS in channel
// order.  The next head's rows are loaded into registers while the current
// head is summed.  Rows are padded by 16 bytes in LDS, so the 16 lanes that
// read at once hit 16 different 4-bank groups.
template <int DT, int D8>
__global__ __launch_bounds__(64) void sink_score_kernel(
    const uint16_t* __restrict__ k, int32_t H, int32_t S, int32_t n_tiles,
    float* __restrict__ score) {
    constexpr int RS = D8 * 16 + 16;          // padded LDS row bytes
    __shared__ __attribute__((aligned(16))) uint8_t rows_s[64 * RS];
    const int32_t tile = (int32_t)(blockIdx.x % (uint32_t)n_tiles);
    const int64_t b = blockIdx.x / (uint32_t)n_tiles;
    const int32_t s0 = tile * 64;
    const int32_t nv = min(64, S - s0);       // real tokens of the tile
    const int lane = threadIdx.x;
    constexpr int D = D8 * 8;
    uint4 pre[D8];                            // 64 * D8 pieces, D8 per lane
    const auto load_head = [&](int32_t h) {
        const uint16_t* base = k + ((b * H + h) * S + s0) * D;
#pragma unroll
        for (int q = 0; q < D8; ++q) {
            const int piece = q * 64 + lane;
            const int row = min(piece / D8, nv - 1);
            pre[q] = load16_nt(base + row * D + (piece % D8) * 8);
        }
    };
    load_head(0);
    float total = 0.0f;
    for (int32_t h = 0; h < H; ++h) {
#pragma unroll
        for (int q = 0; q < D8; ++q) {
            const int piece = q * 64 + lane;
            *reinterpret_cast<uint4*>(rows_s + (piece / D8) * RS + (piece % D8) * 16) = pre[q];
        }
        wave_lds_sync();
        if (h + 1 < H) load_head(h + 1);
        float ss = 0.0f;
#pragma unroll
        for (int c = 0; c < D8; ++c) {
            const uint4 x = *reinterpret_cast<const uint4*>(rows_s + lane * RS + c * 16);
            uint32_t w[4];
            words(x, w);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float f = elem<DT>(w, e);
                ss = __builtin_fmaf(f, f, ss);
            }
        }
        // correctly rounded (built with -fhip-fp32-correctly-rounded-divide-sqrt)
        total = total + __builtin_sqrtf(ss);
        wave_lds_sync();                      // every lane has read its row
    }
    if (lane < nv) score[b * S + s0 + lane] = total / (float)H;
}

template <int DT>
static hipError_t launch_scores_dt(const void* k, int64_t B, int64_t H,
                                   int64_t S, int64_t D, float* score,
                                   hipStream_t st) {
    const int32_t n_tiles = (int32_t)((S + 63) / 64);
    const dim3 grid((uint32_t)(B * n_tiles)), block(64);
    const uint16_t* x = static_cast<const uint16_t*>(k);
    const int32_t h = (int32_t)H, s = (int32_t)S;
    switch (D) {
        case 8: return launch_kernel(sink_score_kernel<DT, 1>, grid, block, 0, st, x, h, s, n_tiles, score);
        case 16: return launch_kernel(sink_score_kernel<DT, 2>, grid, block, 0, st, x, h, s, n_tiles, score);
        case 32: return launch_kernel(sink_score_kernel<DT, 4>, grid, block, 0, st, x, h, s, n_tiles, score);
        case 64: return launch_kernel(sink_score_kernel<DT, 8>, grid, block, 0, st, x, h, s, n_tiles, score);
        case 128: return launch_kernel(sink_score_kernel<DT, 16>, grid, block, 0, st, x, h, s, n_tiles, score);
        default: return launch_kernel(sink_score_kernel<DT, 32>, grid, block, 0, st, x, h, s, n_tiles, score);
    }
}

// ---- selection ----------------------------------------------------------

// (score, position) a ranks before b: higher score, then lower position.
__device__ __forceinline__ bool ranks_before(float sa, int32_t pa, float sb,
                                             int32_t pb) {
    return sa > sb || (sa == sb && pa < pb);
}

constexpr int kSelThreads = 1024;
constexpr int kSelPer = 32;   // scores per thread when a sequence fits in registers

// One pick: the best (score, position) that ranks after the previous pick.
// best starts as (-inf, INT_MAX), which every non-NaN score outranks and
// which itself outranks nothing, so it doubles as "nothing yet"; a NaN
// score ranks neither before nor after anything and is never picked.
__device__ __forceinline__ void consider(float prev_s, int32_t prev_p, float v,
                                         int32_t s, float& best_s,
                                         int32_t& best_p) {
    if (ranks_before(prev_s, prev_p, v, s) && ranks_before(v, s, best_s, best_p)) {
        best_s = v;
        best_p = s;
    }
}

// One block per sequence, n_sink rounds of a block-wide argmax in (score
// desc, position asc) order, each round restricted to what ranks after the
// previous round's pick.  RESIDENT: the sequence's scores (S <= 32768) are
// loaded once into registers, thread t holding positions t + 1024 i;
// otherwise every round streams them again.
template <bool RESIDENT>
__global__ __launch_bounds__(kSelThreads) void sink_select_kernel(
    const float* __restrict__ score, int32_t S, int32_t n_sink,
    int32_t* __restrict__ idx) {
    constexpr int NW = kSelThreads / 64;
    // two buffers, so one barrier per round suffices: a round writes the
    // buffer the round before it did not read
    __shared__ float red_s[2][NW];
    __shared__ int32_t red_p[2][NW];
    const int32_t b = blockIdx.x, tid = threadIdx.x;
    const float* sc = score + (int64_t)b * S;
    float v[RESIDENT ? kSelPer : 1];
    if constexpr (RESIDENT) {
#pragma unroll
        for (int i = 0; i < kSelPer; ++i) {
            const int32_t s = tid + i * kSelThreads;
            v[i] = s < S ? sc[s] : __builtin_nanf("");
        }
    }
    float prev_s = __builtin_huge_valf();   // the first round has no pick before it
    int32_t prev_p = -1;
    for (int32_t r = 0; r < n_sink; ++r) {
        float best_s = -__builtin_huge_valf();
        int32_t best_p = 0x7fffffff;
        if constexpr (RESIDENT) {
#pragma unroll
            for (int i = 0; i < kSelPer; ++i)
                consider(prev_s, prev_p, v[i], tid + i * kSelThreads, best_s, best_p);
        } else {
            // 64-bit positions: S may come within a batch of 2^31
            for (int64_t s0 = 0; s0 < S; s0 += 8 * kSelThreads) {
                float w[8];
#pragma unroll
                for (int i = 0; i < 8; ++i) {
                    const int64_t s = s0 + tid + i * kSelThreads;
                    w[i] = s < S ? sc[s] : __builtin_nanf("");
                }
#pragma unroll
                for (int i = 0; i < 8; ++i)
                    consider(prev_s, prev_p, w[i], (int32_t)(s0 + tid + i * kSelThreads),
                             best_s, best_p);
            }
        }
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) {
            const float os = __shfl_xor(best_s, o);
            const int32_t op = __shfl_xor(best_p, o);
            if (ranks_before(os, op, best_s, best_p)) {
                best_s = os;
                best_p = op;
            }
        }
        const int buf = r & 1;
        if ((tid & 63) == 0) {
            red_s[buf][tid >> 6] = best_s;
            red_p[buf][tid >> 6] = best_p;
        }
        __syncthreads();
        best_s = red_s[buf][0];
        best_p = red_p[buf][0];
#pragma unroll
        for (int w = 1; w < NW; ++w)
            if (ranks_before(red_s[buf][w], red_p[buf][w], best_s, best_p)) {
                best_s = red_s[buf][w];
                best_p = red_p[buf][w];
            }
        // only NaN scores can leave a round empty; such a round stores -1
        if (tid == 0) idx[(int64_t)b * n_sink + r] = best_p == 0x7fffffff ? -1 : best_p;
        prev_s = best_s;
        prev_p = best_p;
    }
}

// ---- keys with sinks ----------------------------------------------------

constexpr int kSinkGMax = 32;

// Codes (0 for a sink) and reconstructions (a sink's own row) of the
// group's nt tokens from registers.
template <int DT, int BITS, bool WQ, bool WR, bool FAST>
__device__ __forceinline__ void emit_sink(const uint4 (&v)[kSinkGMax],
                                          const Params (&pk)[8], uint32_t skip,
                                          int32_t nt, uint8_t* dst,
                                          int64_t row_bytes, uint16_t* rdst,
                                          int64_t D) {
#pragma unroll
    for (int t = 0; t < kSinkGMax; ++t) {
        if (t < nt) {
            uint4 r = v[t];
            uint64_t q = 0;
            if (!((skip >> t) & 1u)) q = quant_chunk<DT, BITS, FAST, WR>(v[t], pk, &r);
            if constexpr (WQ) store_codes<BITS>(dst + t * row_bytes, q);
            if constexpr (WR) store16_nt(rdst + t * D, r);
        }
    }
}

// One lane per item (bh, group g, chunk c), c fastest.  Bit t of `skip` is
// set for token s0 + t when it is a sink or past the group's end; the
// min/max runs over the other tokens.  A lane past the last item mirrors
// the last item's loads and stores nothing.
template <int DT, int BITS, bool WQ, bool WR>
__global__ __launch_bounds__(256) void quant_keys_sink_kernel(
    const uint16_t* __restrict__ x, uint32_t n_items, uint32_t D8, uint32_t NG,
    int32_t S, int32_t G, int32_t H, const int32_t* __restrict__ idx,
    int32_t n_sink, uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, uint16_t* __restrict__ recon) {
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    const bool valid = gid < n_items;
    const uint32_t item = valid ? gid : n_items - 1u;
    const uint32_t c = item % D8;
    const uint32_t tile = item / D8;
    const uint32_t g = tile % NG;
    const uint32_t bh = tile / NG;
    const int32_t b = (int32_t)bh / H;
    const int32_t s0 = (int32_t)g * G;
    const int32_t nt = min(G, S - s0);
    const int64_t D = (int64_t)D8 * 8;
    const int64_t row0 = (int64_t)bh * S + s0;
    const uint16_t* src = x + row0 * D + (int64_t)c * 8;

    uint32_t skip = nt < 32 ? ~((1u << nt) - 1u) : 0u;
    for (int32_t i = 0; i < n_sink; ++i) {
        const int32_t t = idx[(int64_t)b * n_sink + i] - s0;
        if ((uint32_t)t < (uint32_t)nt) skip |= 1u << t;
    }

    uint4 v[kSinkGMax];
#pragma unroll
    for (int t = 0; t < kSinkGMax; ++t) v[t] = load16_nt(src + min(t, nt - 1) * D);

    float lo[8], hi[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        lo[e] = __builtin_huge_valf();
        hi[e] = -__builtin_huge_valf();
    }
#pragma unroll
    for (int t = 0; t < kSinkGMax; ++t) {
        if ((skip >> t) & 1u) continue;
        uint32_t w[4];
        words(v[t], w);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float f = elem<DT>(w, e);
            lo[e] = fminf(lo[e], f);
            hi[e] = fmaxf(hi[e], f);
        }
    }
    const bool none = skip == 0xffffffffu;   // every token a sink
    Params pk[8];
    bool fast = true;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        pk[e] = make_params<BITS>(none ? 0.0f : lo[e], none ? 0.0f : hi[e]);
        fast = fast && pk[e].fast;
    }
    if (!valid) return;
    if (WQ) {
        const int64_t p = ((int64_t)bh * NG + g) * D + (int64_t)c * 8;
        float4* ps = reinterpret_cast<float4*>(scale + p);
        float4* pz = reinterpret_cast<float4*>(zero + p);
        ps[0] = make_float4(pk[0].scale, pk[1].scale, pk[2].scale, pk[3].scale);
        ps[1] = make_float4(pk[4].scale, pk[5].scale, pk[6].scale, pk[7].scale);
        pz[0] = make_float4(pk[0].zero, pk[1].zero, pk[2].zero, pk[3].zero);
        pz[1] = make_float4(pk[4].zero, pk[5].zero, pk[6].zero, pk[7].zero);
    }
    const int64_t row_bytes = (int64_t)D8 * BITS;
    uint8_t* dst = WQ ? codes + row0 * row_bytes + (int64_t)c * BITS : nullptr;
    uint16_t* rdst = WR ? recon + row0 * D + (int64_t)c * 8 : nullptr;
    if (fast)
        emit_sink<DT, BITS, WQ, WR, true>(v, pk, skip, nt, dst, row_bytes, rdst, D);
    else
        emit_sink<DT, BITS, WQ, WR, false>(v, pk, skip, nt, dst, row_bytes, rdst, D);
}

template <int DT, int BITS>
static hipError_t launch_keys_sink_t(const SinkQuantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t NG = (uint32_t)((j.S + j.group - 1) / j.group);
    const uint32_t n = (uint32_t)(j.B * j.H) * NG * D8;
    const dim3 grid((n + 255u) / 256u), block(256);
    const uint16_t* x = static_cast<const uint16_t*>(j.k);
    uint16_t* rec = static_cast<uint16_t*>(j.recon);
    const auto args = [&](auto kern) {
        return launch_kernel(kern, grid, block, 0, j.stream, x, n, D8, NG,
                             (int32_t)j.S, (int32_t)j.group, (int32_t)j.H,
                             j.idx, (int32_t)j.n_sink, j.codes, j.scale,
                             j.zero, rec);
    };
    if (j.codes && j.recon) return args(quant_keys_sink_kernel<DT, BITS, true, true>);
    if (j.codes) return args(quant_keys_sink_kernel<DT, BITS, true, false>);
    return args(quant_keys_sink_kernel<DT, BITS, false, true>);
}

template <int DT>
static hipError_t launch_keys_sink_dt(const SinkQuantJob& j) {
    switch (j.bits) {
        case 1: return launch_keys_sink_t<DT, 1>(j);
        case 2: return launch_keys_sink_t<DT, 2>(j);
        case 4: return launch_keys_sink_t<DT, 4>(j);
        default: return launch_keys_sink_t<DT, 8>(j);
    }
}

// ---- gather / restore ---------------------------------------------------

// One lane per (bh, sink i, 16-byte chunk c): GATHER copies row idx[b, i] of
// x [BH, S, D] to row i of the sink store [BH, n_sink, D]; otherwise the
// other way.  Positions outside [0, S) are skipped.
template <bool GATHER>
__global__ __launch_bounds__(256) void sink_copy_kernel(
    const uint16_t* __restrict__ src, uint16_t* __restrict__ dst,
    uint32_t n_items, uint32_t D8, int32_t S, int32_t H,
    const int32_t* __restrict__ idx, int32_t n_sink) {
    const uint32_t gid = blockIdx.x * 256u + threadIdx.x;
    if (gid >= n_items) return;
    const uint32_t c = gid % D8;
    const uint32_t row = gid / D8;               // bh * n_sink + i
    const uint32_t i = row % (uint32_t)n_sink;
    const uint32_t bh = row / (uint32_t)n_sink;
    const int32_t s = idx[(int64_t)(bh / (uint32_t)H) * n_sink + i];
    if (s < 0 || s >= S) return;
    const int64_t D = (int64_t)D8 * 8;
    const int64_t full = ((int64_t)bh * S + s) * D + (int64_t)c * 8;
    const int64_t kept = (int64_t)row * D + (int64_t)c * 8;
    if (GATHER)
        *reinterpret_cast<uint4*>(dst + kept) = load16(src + full);
    else
        *reinterpret_cast<uint4*>(dst + full) = load16(src + kept);
}

hipError_t launch_sink_scores(const void* k, int dtype, int64_t B, int64_t H,
                              int64_t S, int64_t D, float* score,
                              hipStream_t stream) {
    return dtype == DT_F16 ? launch_scores_dt<DT_F16>(k, B, H, S, D, score, stream)
                           : launch_scores_dt<DT_BF16>(k, B, H, S, D, score, stream);
}

hipError_t launch_sink_select(const float* score, int64_t B, int64_t S,
                              int64_t n_sink, int32_t* idx, hipStream_t stream) {
    if (S <= (int64_t)kSelThreads * kSelPer)
        return launch_kernel(sink_select_kernel<true>, dim3((uint32_t)B),
                             dim3(kSelThreads), 0, stream, score, (int32_t)S,
                             (int32_t)n_sink, idx);
    return launch_kernel(sink_select_kernel<false>, dim3((uint32_t)B),
                         dim3(kSelThreads), 0, stream, score, (int32_t)S,
                         (int32_t)n_sink, idx);
}

hipError_t launch_quant_keys_sink(const SinkQuantJob& j) {
    // Head dimensions whose 8-channel chunks tile a wave go to the split key
    // kernel (two or four lanes per group, the plain quantizer's fast path);
    // others to the one-lane kernel above.
    const int64_t D8 = j.D / 8;
    const int64_t lanes = j.B * j.H * ((j.S + j.group - 1) / j.group) * D8 * 4;
    if ((D8 & (D8 - 1)) == 0 && D8 <= 32 && lanes < (1ll << 31))
        return launch_split_quant_keys_sink(j);
    return j.dtype == DT_F16 ? launch_keys_sink_dt<DT_F16>(j)
                             : launch_keys_sink_dt<DT_BF16>(j);
}

hipError_t launch_sink_copy(bool gather, const void* src, void* dst, int64_t B,
                            int64_t H, int64_t S, int64_t D,
                            const int32_t* idx, int64_t n_sink,
                            hipStream_t stream) {
    const uint32_t D8 = (uint32_t)(D / 8);
    const uint32_t n = (uint32_t)(B * H * n_sink) * D8;
    const dim3 grid((n + 255u) / 256u), block(256);
    const uint16_t* s = static_cast<const uint16_t*>(src);
    uint16_t* d = static_cast<uint16_t*>(dst);
    if (gather)
        return launch_kernel(sink_copy_kernel<true>, grid, block, 0, stream, s,
                             d, n, D8, (int32_t)S, (int32_t)H, idx,
                             (int32_t)n_sink);
    return launch_kernel(sink_copy_kernel<false>, grid, block, 0, stream, s, d,
                         n, D8, (int32_t)S, (int32_t)H, idx, (int32_t)n_sink);
}

}  // namespace kivi
