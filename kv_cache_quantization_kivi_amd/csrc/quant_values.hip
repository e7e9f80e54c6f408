// KIVI per-token value quantization for gfx950.
//
// KIVI blog post on the fused Metal kernels, section "Kernel B -- per-token
// values": the group runs along the contiguous channel axis.  Here one lane
// owns 32 consecutive channels of a row (four 128-bit loads, 64 contiguous
// bytes), so
//   - a group of 8, 16 or 32 channels lies inside one lane: no cross-lane
//     step at all, one (scale, zero) computation per group, and the lane's
//     codes are one contiguous 4*BITS-byte store;
//   - a group of 32*2^k channels spans an aligned block of 2^k lanes: the
//     block's min/max is an xor-butterfly over DPP row permutes (quad xor 1,
//     quad xor 2, half-row mirror, row mirror) and, beyond 16 lanes, a
//     cross-row lane shuffle.
// A row of D channels takes ceil(D/32) lanes, padded to P = next_pow2 so
// rows start on aligned lane blocks.  The post's rule for its SIMD-group
// butterfly carries over: every lane reaches the reduction (no lane exits
// early); lanes past the row's end or past the last row load an in-bounds
// copy of a chunk of the same group, which leaves every min/max unchanged,
// and store nothing.
#include "kivi_device.h"
#include "kivi_launch.h"
#include "kivi_key_split.h"
#include "kivi_rows.h"

namespace kivi {

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
        mn = vmin(mn, dpp_f<0xB1>(mn));   // quad_perm [1,0,3,2]
        mx = vmax(mx, dpp_f<0xB1>(mx));
    }
    if (red > 2) {
        mn = vmin(mn, dpp_f<0x4E>(mn));   // quad_perm [2,3,0,1]
        mx = vmax(mx, dpp_f<0x4E>(mx));
    }
    if (red > 4) {
        mn = vmin(mn, dpp_f<0x141>(mn));  // row_half_mirror
        mx = vmax(mx, dpp_f<0x141>(mx));
    }
    if (red > 8) {
        mn = vmin(mn, dpp_f<0x140>(mn));  // row_mirror
        mx = vmax(mx, dpp_f<0x140>(mx));
    }
    if (red > 16) {
        mn = vmin(mn, __shfl_xor(mn, 16));
        mx = vmax(mx, __shfl_xor(mx, 16));
    }
    if (red > 32) {
        mn = vmin(mn, __shfl_xor(mn, 32));
        mx = vmax(mx, __shfl_xor(mx, 32));
    }
}

// Min and max over chunks [k0, k0 + n) of the lane's four, as fp32.
template <int DT, int N>
__device__ __forceinline__ void chunks_minmax(const uint4 (&v)[4], int k0,
                                              float& mn, float& mx) {
    MinMax8<DT> mm;
    mm.init(v[k0]);
#pragma unroll
    for (int k = 1; k < N; ++k) mm.add(v[k0 + k]);
    float lo[8], hi[8];
    mm.get(lo, hi);
    mn = lo[0];
    mx = hi[0];
#pragma unroll
    for (int k = 1; k < 8; ++k) {
        mn = vmin(mn, lo[k]);
        mx = vmax(mx, hi[k]);
    }
}

// A group parameter; NT: streamed (quantize-only outputs, which measured
// faster non-temporal, for this kernel and the ones after it).
template <bool NT>
__device__ __forceinline__ void put_param(float* p, float v) {
    if constexpr (NT) __builtin_nontemporal_store(v, p);
    else *p = v;
}

// LDS staging.  A lane's 64 bytes of input (and of recon) are contiguous
// but lanes are 64 bytes apart, so direct 16-byte accesses are strided:
// each 128-byte line is touched by four instructions, which defeats
// non-temporal loads (a streamed line is fetched again by every touch) and
// leaves plain loads allocating lines that evict the previous kernel's
// dirty output.  When rows tile the lanes exactly, a wave's input (and
// recon) is one contiguous 4 KiB block: the wave loads it with
// 1 KiB-contiguous non-temporal 16-byte loads, passes it through LDS so
// that every lane gets its own four consecutive chunks, and stores recon
// back the same way.  Chunk j of the block sits at LDS byte (j + j/4) * 16,
// i.e. lane stride 80 bytes, which spreads 8 consecutive lanes over
// distinct banks.
constexpr int kRecLaneStride = 80;
constexpr int kRecWaveBytes = 64 * kRecLaneStride;

// GPL: groups per lane (4: G = 8, 2: G = 16, 1: G >= 32).
// lp: log2 of lanes per row P; red: lanes per group block (GPL == 1);
// gl: log2 of lanes per group (GPL == 1, may exceed lp when G > D);
// vec: D % 32 == 0, so a lane's codes are one naturally aligned store;
// tile: D / 32 is a power of two, so lane unit u covers elements
// [32u, 32u + 32) of the tensor and a wave's input and recon are contiguous.
// IO: the row layout (DenseRows or CacheRows, kivi_rows.h); the staged
// (tiled) path needs contiguous rows.
// u: the lane's index over all lanes of the launch (blocks of 256 lanes);
// lds: the block's 4 * kRecWaveBytes staging bytes.
template <int DT, int BITS, int GPL, bool WQ, bool WR, typename IO>
__device__ __forceinline__ void quant_values_body(
    IO io, uint64_t u, uint8_t* lds, int64_t n_rows, uint32_t D8, uint32_t lp,
    uint32_t red, uint32_t gl, uint32_t NGD, int32_t vec, int32_t tile,
    uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, uint16_t* __restrict__ recon) {
    constexpr int CPG = 4 / GPL;   // chunks per in-lane group
    const uint32_t c = (uint32_t)(u & ((1u << lp) - 1u));   // lane in its row
    const int64_t row = (int64_t)(u >> lp);
    const bool row_ok = row < n_rows;
    const int64_t lrow = row_ok ? row : n_rows - 1;
    const int64_t D = (int64_t)D8 * 8;
    const int32_t ch0 = (int32_t)c * 4;                  // first chunk
    const int32_t nch = min(4, (int32_t)D8 - ch0);       // real chunks (<= 0: pad lane)
    const uint16_t* rsrc = io.vrow(lrow, D);

    // Wave-uniform: a whole wave of real rows in a tiled layout.
    const bool staged = IO::kContiguous && tile && __all(row_ok);
    const uint32_t lane = threadIdx.x & 63u;
    uint8_t* L = lds + (threadIdx.x >> 6) * kRecWaveBytes;
    uint4 v[4];
    if (staged) {
        const uint16_t* wsrc = io.vrow(0, D) + (u - lane) * 32;   // the wave's 4 KiB
        uint4 t[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) t[k] = load16_nt(wsrc + (k * 64 + lane) * 8);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const uint32_t j = k * 64u + lane;
            *reinterpret_cast<uint4*>(L + (j + (j >> 2)) * 16) = t[k];
        }
        wave_lds_sync();
#pragma unroll
        for (int m = 0; m < 4; ++m)
            v[m] = *reinterpret_cast<const uint4*>(L + lane * kRecLaneStride + m * 16);
    } else {
        // Chunk k of this lane; a missing chunk of a partial lane loads the
        // lane's last real chunk (same lane, so the same group, or a group
        // with no real chunk that is never stored); a pad lane loads the
        // row's last chunk, which belongs to the row's last group -- the
        // only group a pad lane's reduction block can share.
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int32_t ch = nch <= 0 ? (int32_t)D8 - 1
                                        : ch0 + (k < nch ? k : nch - 1);
            v[k] = load16(rsrc + (int64_t)ch * 8);
        }
    }

    float mn[GPL], mx[GPL];
#pragma unroll
    for (int t = 0; t < GPL; ++t) chunks_minmax<DT, CPG>(v, t * CPG, mn[t], mx[t]);
    if constexpr (GPL == 1) block_minmax(mn[0], mx[0], red);

    if (!staged && (!row_ok || nch <= 0)) return;
    const int64_t orow = io.vout(row);   // output row of this lane's row

    Params pg[GPL];
#pragma unroll
    for (int t = 0; t < GPL; ++t) pg[t] = make_params<BITS>(mn[t], mx[t]);

    if constexpr (WQ) {
        if constexpr (GPL == 1) {
            if ((c & ((1u << gl) - 1u)) == 0) {
                const int64_t pi = orow * NGD + (c >> gl);
                put_param<!WR>(scale + pi, pg[0].scale);
                put_param<!WR>(zero + pi, pg[0].zero);
            }
        } else {
#pragma unroll
            for (int t = 0; t < GPL; ++t) {
                if (t * CPG < nch) {
                    const int64_t pi = orow * NGD + (ch0 / CPG) + t;
                    put_param<!WR>(scale + pi, pg[t].scale);
                    put_param<!WR>(zero + pi, pg[t].zero);
                }
            }
        }
    }

    bool fast = true;
#pragma unroll
    for (int t = 0; t < GPL; ++t) fast = fast && pg[t].fast;
    const int64_t row_bytes = (int64_t)D8 * BITS;
    uint8_t* cdst = WQ ? codes + orow * row_bytes + (int64_t)ch0 * BITS : nullptr;
    uint16_t* rdst = WR ? recon + orow * D + (int64_t)ch0 * 8 : nullptr;
    uint64_t q[4];
    uint4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        Params pk[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) pk[e] = pg[k / CPG];
        q[k] = fast ? quant_chunk<DT, BITS, true, WR>(v[k], pk, &r[k])
                    : quant_chunk<DT, BITS, false, WR>(v[k], pk, &r[k]);
    }
    if constexpr (WR) {
        if (staged) {
            wave_lds_sync();   // every lane has read its input chunks
#pragma unroll
            for (int k = 0; k < 4; ++k)
                *reinterpret_cast<uint4*>(L + lane * kRecLaneStride + k * 16) = r[k];
            wave_lds_sync();
            uint8_t* wdst = reinterpret_cast<uint8_t*>(recon + (u - lane) * 32);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const uint32_t off = k * 1024u + lane * 16u;
                store16_nt(wdst + off, *reinterpret_cast<const uint4*>(
                                           L + (off >> 6) * kRecLaneStride + (off & 63u)));
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (k < nch) store16_nt(rdst + k * 8, r[k]);
        }
    }
    if constexpr (WQ) {
        if (vec && nch == 4) {
            // the lane's 4 chunks' codes as one store (BITS bytes per chunk)
            if constexpr (BITS == 1) {
                store_codes<4, !WR>(cdst, q[0] | (q[1] << 8) | (q[2] << 16) | (q[3] << 24));
            } else if constexpr (BITS == 2) {
                store_codes<8, !WR>(cdst, q[0] | (q[1] << 16) | (q[2] << 32) | (q[3] << 48));
            } else {   // 16 bytes (4-bit) or 32 bytes (8-bit) of codes
                constexpr int N = BITS / 4;
                uint4 w[2];
                if constexpr (BITS == 4) {
                    w[0] = make_uint4((uint32_t)q[0], (uint32_t)q[1], (uint32_t)q[2],
                                      (uint32_t)q[3]);
                } else {
                    w[0] = make_uint4((uint32_t)q[0], (uint32_t)(q[0] >> 32),
                                      (uint32_t)q[1], (uint32_t)(q[1] >> 32));
                    w[1] = make_uint4((uint32_t)q[2], (uint32_t)(q[2] >> 32),
                                      (uint32_t)q[3], (uint32_t)(q[3] >> 32));
                }
#pragma unroll
                for (int k = 0; k < N; ++k) {
                    if constexpr (!WR) store16_nt(cdst + 16 * k, w[k]);
                    else reinterpret_cast<uint4*>(cdst)[k] = w[k];
                }
            }
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k)
                if (k < nch) store_codes<BITS, !WR>(cdst + k * BITS, q[k]);
        }
    }
}

template <int DT, int BITS, int GPL, bool WQ, bool WR, typename IO>
__global__ __launch_bounds__(256) void quant_values_kernel(
    IO io, int64_t n_rows, uint32_t D8, uint32_t lp,
    uint32_t red, uint32_t gl, uint32_t NGD, int32_t vec, int32_t tile,
    uint8_t* __restrict__ codes, float* __restrict__ scale,
    float* __restrict__ zero, uint16_t* __restrict__ recon) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kRecWaveBytes];
    quant_values_body<DT, BITS, GPL, WQ, WR, IO>(
        io, (uint64_t)blockIdx.x * 256u + threadIdx.x, lds, n_rows, D8, lp, red,
        gl, NGD, vec, tile, codes, scale, zero, recon);
}

template <int DT, int BITS, int GPL, bool WQ, bool WR>
static hipError_t launch_values_t(const QuantJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t lpr = (D8 + 3) / 4;                 // real lanes per row
    const uint32_t lp = log2_ceil(lpr);                // P = 2^lp
    const uint32_t gl = GPL == 1 ? log2_ceil((uint64_t)(j.group / 32)) : 0;
    const uint32_t red = 1u << (gl < lp ? gl : lp);
    const uint32_t NGD = (uint32_t)((j.D + j.group - 1) / j.group);
    const int64_t n_rows = j.BH * j.S;
    const uint64_t lanes = (uint64_t)n_rows << lp;
    const uint32_t blocks = (uint32_t)((lanes + 255) / 256);
    const int32_t vec = (D8 % 4) == 0;
    const int32_t tile = vec && (1u << lp) == lpr;
    const DenseRows io{static_cast<const uint16_t*>(j.x), 0, 0, 1};   // rows only
    return launch_kernel((quant_values_kernel<DT, BITS, GPL, WQ, WR, DenseRows>),
                       dim3(blocks), dim3(256), 0, j.stream, io, n_rows, D8,
                       lp, red, gl, NGD, vec, tile, j.codes, j.scale, j.zero,
                       static_cast<uint16_t*>(j.recon));
}

template <int DT, int BITS, int GPL>
static hipError_t launch_values_mode(const QuantJob& j) {
    const bool wq = j.codes != nullptr;
    const bool wr = j.recon != nullptr;
    if (wq && wr) return launch_values_t<DT, BITS, GPL, true, true>(j);
    if (wq) return launch_values_t<DT, BITS, GPL, true, false>(j);
    return launch_values_t<DT, BITS, GPL, false, true>(j);
}

template <int DT, int BITS>
static hipError_t launch_values_gpl(const QuantJob& j) {
    if (j.group == 8) return launch_values_mode<DT, BITS, 4>(j);
    if (j.group == 16) return launch_values_mode<DT, BITS, 2>(j);
    return launch_values_mode<DT, BITS, 1>(j);
}

template <int DT>
static hipError_t launch_values_bits(const QuantJob& j) {
    switch (j.bits) {
        case 1: return launch_values_gpl<DT, 1>(j);
        case 2: return launch_values_gpl<DT, 2>(j);
        case 4: return launch_values_gpl<DT, 4>(j);
        default: return launch_values_gpl<DT, 8>(j);
    }
}

template <int DT, int BITS, int GPL>
static hipError_t launch_cache_values_t(const CacheFlushJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t lpr = (D8 + 3) / 4;
    const uint32_t lp = log2_ceil(lpr);
    const uint32_t gl = GPL == 1 ? log2_ceil((uint64_t)(j.group / 32)) : 0;
    const uint32_t red = 1u << (gl < lp ? gl : lp);
    const uint32_t NGD = (uint32_t)((j.D + j.group - 1) / j.group);
    const int64_t n_rows = j.BH * j.F;
    const uint64_t lanes = (uint64_t)n_rows << lp;
    const uint32_t blocks = (uint32_t)((lanes + 255) / 256);
    const int32_t vec = (D8 % 4) == 0;
    const CacheRows io{static_cast<const uint16_t*>(j.ring),
                       static_cast<const uint16_t*>(j.in), (int32_t)j.ring_len,
                       (int32_t)j.n_in, (int32_t)j.T, (int32_t)j.Q,
                       (int32_t)j.F, (int32_t)j.S_max,
                       (uint32_t)((j.S_max + j.G_k - 1) / j.G_k),
                       (int32_t)j.G_k};
    return launch_kernel(
        (quant_values_kernel<DT, BITS, GPL, true, false, CacheRows>),
        dim3(blocks), dim3(256), 0, j.stream, io, n_rows, D8, lp, red, gl, NGD,
        vec, (int32_t)0, j.codes, j.scale, j.zero, (uint16_t*)nullptr);
}

template <int DT, int BITS>
static hipError_t launch_cache_values_bits(const CacheFlushJob& j) {
    if (j.group == 8) return launch_cache_values_t<DT, BITS, 4>(j);
    if (j.group == 16) return launch_cache_values_t<DT, BITS, 2>(j);
    return launch_cache_values_t<DT, BITS, 1>(j);
}

template <int DT>
static hipError_t launch_cache_values_dt(const CacheFlushJob& j) {
    switch (j.bits) {
        case 1: return launch_cache_values_bits<DT, 1>(j);
        case 2: return launch_cache_values_bits<DT, 2>(j);
        case 4: return launch_cache_values_bits<DT, 4>(j);
        default: return launch_cache_values_bits<DT, 8>(j);
    }
}

template <int DT, int BITS, int GPL>
static hipError_t launch_list_values_t(const ListJob& j) {
    const uint32_t D8 = (uint32_t)(j.D / 8);
    const uint32_t lpr = (D8 + 3) / 4;
    const uint32_t lp = log2_ceil(lpr);
    const uint32_t gl = GPL == 1 ? log2_ceil((uint64_t)(j.group / 32)) : 0;
    const uint32_t red = 1u << (gl < lp ? gl : lp);
    const uint32_t NGD = (uint32_t)((j.D + j.group - 1) / j.group);
    const int64_t n_rows = j.B * j.H * j.n;
    const uint64_t lanes = (uint64_t)n_rows << lp;
    const uint32_t blocks = (uint32_t)((lanes + 255) / 256);
    const int32_t vec = (D8 % 4) == 0;
    const ListRows io{static_cast<const uint16_t*>(j.x), j.pos, (int32_t)j.S,
                      (int32_t)j.n, (int32_t)j.H, 0u, 1};
    return launch_kernel(
        (quant_values_kernel<DT, BITS, GPL, true, false, ListRows>),
        dim3(blocks), dim3(256), 0, j.stream, io, n_rows, D8, lp, red, gl, NGD,
        vec, (int32_t)0, j.codes, j.scale, j.zero, (uint16_t*)nullptr);
}

template <int DT, int BITS>
static hipError_t launch_list_values_bits(const ListJob& j) {
    if (j.group == 8) return launch_list_values_t<DT, BITS, 4>(j);
    if (j.group == 16) return launch_list_values_t<DT, BITS, 2>(j);
    return launch_list_values_t<DT, BITS, 1>(j);
}

template <int DT>
static hipError_t launch_list_values_dt(const ListJob& j) {
    switch (j.bits) {
        case 1: return launch_list_values_bits<DT, 1>(j);
        case 2: return launch_list_values_bits<DT, 2>(j);
        case 4: return launch_list_values_bits<DT, 4>(j);
        default: return launch_list_values_bits<DT, 8>(j);
    }
}

hipError_t launch_list_quant_values(const ListJob& j) {
    return j.dtype == DT_F16 ? launch_list_values_dt<DT_F16>(j)
                             : launch_list_values_dt<DT_BF16>(j);
}

// The caller guarantees: D / 8 a power of two <= 32 (so D <= 256), a value
// group of 8, 16 or a multiple of 32, and fewer than 2^31 rows.
hipError_t launch_cache_flush_values(const CacheFlushJob& j) {
    return j.dtype == DT_F16 ? launch_cache_values_dt<DT_F16>(j)
                             : launch_cache_values_dt<DT_BF16>(j);
}

// ---- keys and values of a small flush in one launch --------------------

// Blocks [0, v_blocks) run the value body, the rest the 4-lane split key
// body on 256 lanes per block (its lanes need no block-level step).  A
// decode-time flush of both tensors is then one launch instead of two:
// each is a few microseconds of fixed latency at these sizes.
template <int DT, int BITS, bool WQ, bool WR, typename IO>
__global__ __launch_bounds__(256) void quant_kv_kernel(
    IO kio, uint32_t k_lanes, uint32_t D8, uint32_t NG,
    uint8_t* __restrict__ kc, float* __restrict__ ks, float* __restrict__ kz,
    uint16_t* __restrict__ kr, IO vio, int64_t n_rows, uint32_t lp,
    uint32_t red, uint32_t gl, uint32_t NGD, int32_t vec, int32_t tile,
    uint8_t* __restrict__ vc, float* __restrict__ vs, float* __restrict__ vz,
    uint16_t* __restrict__ vr, uint32_t v_blocks) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kRecWaveBytes];
    if (blockIdx.x < v_blocks) {
        quant_values_body<DT, BITS, 1, WQ, WR, IO>(
            vio, (uint64_t)blockIdx.x * 256u + threadIdx.x, lds, n_rows, D8, lp,
            red, gl, NGD, vec, tile, vc, vs, vz, vr);
    } else {
        quant_keys_split_body<DT, BITS, kKeyGMaxPair / 4, 4, WQ, WR, true, IO,
                              (BITS <= 4), 256>(
            kio, (blockIdx.x - v_blocks) * 256u + threadIdx.x, k_lanes, D8, NG,
            kc, ks, kz, kr);
    }
}

template <int DT, int BITS, bool WQ, bool WR>
static hipError_t launch_kv_t(const QuantJob& k, const QuantJob& v) {
    const uint32_t D8 = (uint32_t)(k.D / 8);
    const uint32_t NG = (uint32_t)((k.S + k.group - 1) / k.group);
    const uint64_t k_lanes = (uint64_t)k.BH * NG * D8 * 4;
    const DenseRows kio{static_cast<const uint16_t*>(k.x), (int32_t)k.S, NG,
                        (int32_t)k.group};
    // value launch shape, as launch_values_t
    const uint32_t lpr = (D8 + 3) / 4;
    const uint32_t lp = log2_ceil(lpr);
    const uint32_t gl = log2_ceil((uint64_t)(v.group / 32));
    const uint32_t red = 1u << (gl < lp ? gl : lp);
    const uint32_t NGD = (uint32_t)((v.D + v.group - 1) / v.group);
    const int64_t n_rows = v.BH * v.S;
    const uint64_t v_lanes = (uint64_t)n_rows << lp;
    const uint32_t v_blocks = (uint32_t)((v_lanes + 255) / 256);
    const int32_t vec = (D8 % 4) == 0;
    const int32_t tile = vec && (1u << lp) == lpr;
    const DenseRows vio{static_cast<const uint16_t*>(v.x), 0, 0, 1};
    const uint32_t blocks = v_blocks + (uint32_t)((k_lanes + 255) / 256);
    return launch_kernel((quant_kv_kernel<DT, BITS, WQ, WR, DenseRows>), dim3(blocks),
                         dim3(256), 0, k.stream, kio, (uint32_t)k_lanes, D8, NG,
                         k.codes, k.scale, k.zero, static_cast<uint16_t*>(k.recon),
                         vio, n_rows, lp, red, gl, NGD, vec, tile, v.codes,
                         v.scale, v.zero, static_cast<uint16_t*>(v.recon),
                         v_blocks);
}

template <int DT, int BITS>
static hipError_t launch_kv_mode(const QuantJob& k, const QuantJob& v) {
    const bool wq = k.codes != nullptr;
    const bool wr = k.recon != nullptr;
    if (wq && wr) return launch_kv_t<DT, BITS, true, true>(k, v);
    if (wq) return launch_kv_t<DT, BITS, true, false>(k, v);
    return launch_kv_t<DT, BITS, false, true>(k, v);
}

template <int DT>
static hipError_t launch_kv_bits(const QuantJob& k, const QuantJob& v) {
    switch (k.bits) {
        case 1: return launch_kv_mode<DT, 1>(k, v);
        case 2: return launch_kv_mode<DT, 2>(k, v);
        case 4: return launch_kv_mode<DT, 4>(k, v);
        default: return launch_kv_mode<DT, 8>(k, v);
    }
}

// The caller has validated both jobs (same dtype, shape, bits and outputs
// present alike).  One launch when the keys take the 4-lane split kernel
// with groups of 17 to 32 tokens and the value groups are 32 * 2^k
// channels; otherwise the two single launches, keys first.
hipError_t launch_quant_kv(const QuantJob& k, const QuantJob& v) {
    const uint64_t D8 = (uint64_t)(k.D / 8);
    const uint64_t items = (uint64_t)k.BH * ((k.S + k.group - 1) / k.group) * D8;
    const int64_t g32 = v.group / 32;
    const bool pair = k.D % 8 == 0 && items < kKeySplitBelow &&
                      64 % (D8 * 4) == 0 && k.group > kKeyGMaxPair / 2 &&
                      k.group <= kKeyGMaxPair && v.group % 32 == 0 &&
                      (g32 & (g32 - 1)) == 0;
    if (!pair) {
        const hipError_t e = launch_quant_keys(k);
        return e != hipSuccess ? e : launch_quant_values(v);
    }
    return k.dtype == DT_F16 ? launch_kv_bits<DT_F16>(k, v)
                             : launch_kv_bits<DT_BF16>(k, v);
}

// A residual-window cache's flush of both tensors (CacheRows) in one
// launch, under the rule of launch_quant_kv with a larger item bound: up to
// kCacheKvPairBelow key items the one launch, with the 4-lane key body, is
// faster than the two (a 2016-token prefill flush of 112 heads, 112896
// items: the step 42.2 -> 37.5 us), since each launch's ramp and tail is
// a third of a key flush that size.
constexpr uint64_t kCacheKvPairBelow = 4 * kKeySplitBelow;

// A residual-window cache append in one launch: the flush of both tensors
// and, when the append has one, its ring store.  Blocks [0, k_blocks) run
// the 4-lane split key body, the next v_blocks the value body, the rest the
// ring store; the caller guarantees that the ring store writes no slot the
// flush reads, so the three need no ordering.  The key blocks come first:
// their waves run longest, and started first they do not trail the launch.
template <int DT, int BITS>
__global__ __launch_bounds__(256) void cache_append_kernel(
    CacheRows kio, uint32_t k_lanes, uint32_t D8, uint32_t NG,
    uint8_t* __restrict__ kc, float* __restrict__ ks, float* __restrict__ kz,
    CacheRows vio, int64_t n_rows, uint32_t lp, uint32_t red, uint32_t gl,
    uint32_t NGD, int32_t vec, uint8_t* __restrict__ vc,
    float* __restrict__ vs, float* __restrict__ vz, uint32_t k_blocks,
    uint32_t v_blocks, RingStore ring) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[4 * kRecWaveBytes];
    if (blockIdx.x < k_blocks) {
        quant_keys_split_body<DT, BITS, kKeyGMaxPair / 4, 4, true, false, true,
                              CacheRows, (BITS <= 4), 256>(
            kio, blockIdx.x * 256u + threadIdx.x, k_lanes, D8, NG, kc, ks, kz, nullptr);
    } else if (blockIdx.x < k_blocks + v_blocks) {
        quant_values_body<DT, BITS, 1, true, false, CacheRows>(
            vio, (uint64_t)(blockIdx.x - k_blocks) * 256u + threadIdx.x, lds,
            n_rows, D8, lp, red, gl, NGD, vec, 0, vc, vs, vz, nullptr);
    } else {
        ring_store_lane(ring, (blockIdx.x - k_blocks - v_blocks) * 256u + threadIdx.x);
    }
}

template <int DT, int BITS>
static hipError_t launch_cache_kv_t(const CacheFlushJob& k, const CacheFlushJob& v,
                                    const RingStore* ring) {
    const uint32_t D8 = (uint32_t)(k.D / 8);
    const uint32_t NG = (uint32_t)(k.F / k.G_k);          // groups flushed per bh
    const uint64_t k_lanes = (uint64_t)k.BH * NG * D8 * 4;
    const uint32_t NG_out = (uint32_t)((k.S_max + k.G_k - 1) / k.G_k);
    const auto rows = [&](const CacheFlushJob& j) {
        return CacheRows{static_cast<const uint16_t*>(j.ring),
                         static_cast<const uint16_t*>(j.in), (int32_t)j.ring_len,
                         (int32_t)j.n_in, (int32_t)j.T, (int32_t)j.Q,
                         (int32_t)j.F, (int32_t)j.S_max, NG_out, (int32_t)j.G_k};
    };
    const uint32_t lpr = (D8 + 3) / 4;
    const uint32_t lp = log2_ceil(lpr);
    const uint32_t gl = log2_ceil((uint64_t)(v.group / 32));
    const uint32_t red = 1u << (gl < lp ? gl : lp);
    const uint32_t NGD = (uint32_t)((v.D + v.group - 1) / v.group);
    const int64_t n_rows = v.BH * v.F;
    const uint32_t v_blocks = (uint32_t)((((uint64_t)n_rows << lp) + 255) / 256);
    const int32_t vec = (D8 % 4) == 0;
    const uint32_t k_blocks = (uint32_t)((k_lanes + 255) / 256);
    RingStore none{};
    const RingStore& r = ring != nullptr ? *ring : none;
    const uint32_t r_blocks = (uint32_t)((2ull * r.half + 255) / 256);
    return launch_kernel((cache_append_kernel<DT, BITS>),
                         dim3(k_blocks + v_blocks + r_blocks), dim3(256), 0,
                         k.stream, rows(k), (uint32_t)k_lanes, D8, NG, k.codes,
                         k.scale, k.zero, rows(v), n_rows, lp, red, gl, NGD, vec,
                         v.codes, v.scale, v.zero, k_blocks, v_blocks, r);
}

template <int DT>
static hipError_t launch_cache_kv_bits(const CacheFlushJob& k, const CacheFlushJob& v,
                                       const RingStore* ring) {
    switch (k.bits) {
        case 1: return launch_cache_kv_t<DT, 1>(k, v, ring);
        case 2: return launch_cache_kv_t<DT, 2>(k, v, ring);
        case 4: return launch_cache_kv_t<DT, 4>(k, v, ring);
        default: return launch_cache_kv_t<DT, 8>(k, v, ring);
    }
}

hipError_t launch_cache_flush_kv(const CacheFlushJob& k, const CacheFlushJob& v) {
    if (!cache_append_fits(k, v)) {
        const hipError_t e = launch_cache_flush_keys(k);
        return e != hipSuccess ? e : launch_cache_flush_values(v);
    }
    return launch_cache_append(k, v, nullptr);
}

bool cache_append_fits(const CacheFlushJob& k, const CacheFlushJob& v) {
    const uint64_t D8 = (uint64_t)(k.D / 8);
    const uint64_t items = (uint64_t)k.BH * (k.F / k.G_k) * D8;
    const int64_t g32 = v.group / 32;
    return items < kCacheKvPairBelow && 64 % (D8 * 4) == 0 &&
           k.G_k > kKeyGMaxPair / 2 && k.G_k <= kKeyGMaxPair &&
           v.group % 32 == 0 && (g32 & (g32 - 1)) == 0;
}

hipError_t launch_cache_append(const CacheFlushJob& k, const CacheFlushJob& v,
                               const RingStore* ring) {
    return k.dtype == DT_F16 ? launch_cache_kv_bits<DT_F16>(k, v, ring)
                             : launch_cache_kv_bits<DT_BF16>(k, v, ring);
}

hipError_t launch_quant_values(const QuantJob& j) {
    // Fast path: whole 8-channel chunks, rows of at most 64 lanes
    // (D <= 2048), and groups of 8, 16 or 32 * 2^k channels.
    const int64_t g32 = j.group / 32;
    const bool grp_ok = j.group == 8 || j.group == 16 ||
                        (j.group % 32 == 0 && (g32 & (g32 - 1)) == 0);
    const int64_t n_rows = j.BH * j.S;
    const bool fits = n_rows < (1ll << 40);
    if (j.D % 8 != 0 || j.D > 2048 || !grp_ok || !fits)
        return launch_generic_quant_values(j);
    return j.dtype == DT_F16 ? launch_values_bits<DT_F16>(j)
                             : launch_values_bits<DT_BF16>(j);
}

}  // namespace kivi
