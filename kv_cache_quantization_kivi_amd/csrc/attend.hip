// KIVI decode attention over a residual-window cache, reading the packed
// codes directly (KIVI blog post on the fused Metal kernels, section "So why
// does the kernel ship?": the memory and speed win needs packed storage and
// attention that expands the codes in registers, never in memory).
//
// One decode position per query head; n_q query heads share each KV head.
// For every bh the T cached tokens are split into chunks of kAttChunk
// tokens, one block per (chunk, bh) (flash-decoding): the block computes
// its chunk's scores, a softmax partial (max m, sum l) and the partial
// output o = sum_t exp(s_t - m) v_t, and writes (m, l, o) to the workspace;
// a second kernel merges the chunks of each bh.
//
// Tokens t < Q are used through their codes and params without being
// rounded to the 16-bit type: a key enters a score as
// sum_d (q_d scale_d) code_d + sum_d q_d zero_d, a value enters the output as
// (p scale) code + p zero, both in fp32; tokens t >= Q come from the ring as
// stored.  Scores, the softmax and all sums are fp32.
#include <mutex>

#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kAttChunk = 128;   // tokens per block (one per thread)
constexpr int kAttMaxGroups = kAttChunk / 8;   // key groups in a chunk (G_k >= 8)

// Max and sum over the block's two waves of N values at once (one pair of
// barriers for all N); red holds 2 * N floats.
template <int N>
__device__ __forceinline__ void block_max_n(float (&v)[N], float* red) {
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v[j] = fmaxf(v[j], __shfl_xor(v[j], o));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int j = 0; j < N; ++j) red[w * N + j] = v[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = fmaxf(red[j], red[N + j]);
    __syncthreads();
}

template <int N>
__device__ __forceinline__ void block_sum_n(float (&v)[N], float* red) {
#pragma unroll
    for (int j = 0; j < N; ++j)
#pragma unroll
        for (int o = 32; o >= 1; o >>= 1) v[j] += __shfl_xor(v[j], o);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0)
#pragma unroll
        for (int j = 0; j < N; ++j) red[w * N + j] = v[j];
    __syncthreads();
#pragma unroll
    for (int j = 0; j < N; ++j) v[j] = red[j] + red[N + j];
    __syncthreads();
}

template <int DT>
__device__ __forceinline__ float widen16(uint16_t h) {
    if constexpr (DT == DT_F16)
        return (float)__builtin_bit_cast(_Float16, h);
    else
        return __uint_as_float((uint32_t)h << 16);
}


// The 8 codes (8 * BITS bits) of channel chunk c8 from a token's code row
// held as 32-bit words.
template <int BITS>
__device__ __forceinline__ uint64_t row_chunk(const uint32_t* w, int c8) {
    if constexpr (BITS == 8) {
        return (uint64_t)w[2 * c8] | ((uint64_t)w[2 * c8 + 1] << 32);
    } else if constexpr (BITS == 4) {
        return w[c8];
    } else {   // 8 or 16 bits inside one word
        const int bit = c8 * BITS * 8;
        return (w[bit >> 5] >> (bit & 31)) & ((1u << (8 * BITS)) - 1u);
    }
}

// D: head dimension (64 or 128); NQ: query heads per KV head rounded up to
// 1, 2, 3, 4, 6 or 8 (rows past n_q are zeros and never stored).  One block of
// kAttChunk threads per (chunk, bh); the caller guarantees D * BITS >= 128
// (whole 16-byte code rows), G_k in {8, 16, 32} (chunks are group-aligned)
// and n_q <= NQ.
template <int DT, int BITS, int D, int NQ>
__global__ __launch_bounds__(kAttChunk) void attend_partial_kernel(AttendArgs a) {
    constexpr int D8 = D / 8;
    constexpr int kRowWords = D * BITS / 32;      // code row as 32-bit words
    constexpr int PARTS = kAttChunk / D8;         // token parts in phase 3
    __shared__ __attribute__((aligned(16))) float q_s[NQ][D];
    // Key params of the chunk's groups, as scale / zero rows (ks, kz) or,
    // when they fit (groups * NQ <= kQsRows), as the scaled queries
    // qs[g][j][d] = q[j][d] * scale[g][d] with bias[g][j] = sum_d q[j][d] *
    // zero[g][d], so that a score is sum_d qs * code + bias.
    constexpr int kKpStride = D + 4;
    constexpr int kQsRows = 16;
    static_assert(kQsRows * 8 == kAttChunk, "bias: eight lanes per row");
    __shared__ __attribute__((aligned(16))) float kp_s[2 * kAttMaxGroups * kKpStride];
    float (*ks_s)[kKpStride] = reinterpret_cast<float (*)[kKpStride]>(kp_s);
    float (*kz_s)[kKpStride] =
        reinterpret_cast<float (*)[kKpStride]>(kp_s + kAttMaxGroups * kKpStride);
    float (*qs_s)[D] = reinterpret_cast<float (*)[D]>(kp_s);
    float* bias_s = kp_s + kQsRows * D;
    __shared__ __attribute__((aligned(16))) float p_s[NQ][kAttChunk];
    __shared__ __attribute__((aligned(16))) float acc_s[NQ][D];
    __shared__ float red[2 * NQ];

    const int chunk = (int)blockIdx.x + a.chunk0;
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int nq = a.n_q;
    const int t0 = chunk * kAttChunk;
    const int nt = min(kAttChunk, a.T - t0);           // tokens in this chunk
    const int nq_tok = max(0, min(nt, a.Q - t0));      // of them quantized
    constexpr int64_t row_bytes = (int64_t)D8 * BITS;

    // query heads (widened once; padded rows are zero) and the key params
    // of the chunk's quantized groups
    for (int i = tid; i < NQ * D; i += kAttChunk)
        q_s[i / D][i % D] =
            i / D < nq ? widen16<DT>(a.q[((int64_t)bh * nq + i / D) * D + i % D])
                       : 0.0f;
    const int g0 = t0 / a.G_k;
    const int ng = (nq_tok + a.G_k - 1) / a.G_k;
    const bool scaled_q = ng * NQ <= kQsRows;     // block-uniform
    __syncthreads();                             // q_s complete
    if (scaled_q) {
        float* z_s = bias_s + kQsRows;   // the groups' zeros, [ng][D]
        for (int i = tid; i < ng * NQ * D; i += kAttChunk) {
            const int row = i / D, d = i % D;    // row = g * NQ + j
            const int64_t p = ((int64_t)bh * a.NG + g0 + row / NQ) * D + d;
            qs_s[row][d] = q_s[row % NQ][d] * a.k_scale[p];
        }
        for (int i = tid; i < ng * D; i += kAttChunk)
            z_s[i] = a.k_zero[((int64_t)bh * a.NG + g0 + i / D) * D + i % D];
        __syncthreads();
        // bias[g][j] = sum_d q[j][d] * zero[g][d]: eight lanes per (g, j)
        // (kQsRows * 8 == kAttChunk), each summing every eighth channel,
        // then three xor shuffles inside the eight
        {
            const int row = tid >> 3, part = tid & 7;
            float b = 0.0f;
            if (row < ng * NQ) {
                const int g = row / NQ, j = row % NQ;
#pragma unroll 4
                for (int d = part; d < D; d += 8)
                    b = __builtin_fmaf(q_s[j][d], z_s[g * D + d], b);
            }
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) b += __shfl_xor(b, o);
            if (part == 0 && row < ng * NQ) bias_s[row] = b;
        }
    } else {
        for (int i = tid; i < ng * D; i += kAttChunk) {
            const int64_t p = ((int64_t)bh * a.NG + g0 + i / D) * D + i % D;
            ks_s[i / D][i % D] = a.k_scale[p];
            kz_s[i / D][i % D] = a.k_zero[p];
        }
    }
    __syncthreads();

    // ---- scores: one token per thread, its whole row loaded up front ----
    float sc[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) sc[j] = 0.0f;
    const int t = t0 + tid;
    if (tid < nq_tok) {
        const uint8_t* crow = a.k_codes + ((int64_t)bh * a.S_max + t) * row_bytes;
        uint32_t w[kRowWords];
#pragma unroll
        for (int k = 0; k < kRowWords / 4; ++k) {
            const uint4 x = load16_nt(crow + k * 16);
            w[4 * k] = x.x;
            w[4 * k + 1] = x.y;
            w[4 * k + 2] = x.z;
            w[4 * k + 3] = x.w;
        }
        const int g = t / a.G_k - g0;   // this token's group in the chunk
        if (scaled_q) {
#pragma unroll
            for (int c8 = 0; c8 < D8; ++c8) {
                const uint64_t packed = row_chunk<BITS>(w, c8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = c8 * 8 + e;
                    const float code = (float)((uint32_t)(packed >> (e * BITS)) &
                                               ((1u << BITS) - 1u));
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        sc[j] = __builtin_fmaf(qs_s[g * NQ + j][d], code, sc[j]);
                }
            }
#pragma unroll
            for (int j = 0; j < NQ; ++j) sc[j] += bias_s[g * NQ + j];
        } else {
#pragma unroll
            for (int c8 = 0; c8 < D8; ++c8) {
                const uint64_t packed = row_chunk<BITS>(w, c8);
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int d = c8 * 8 + e;
                    const uint32_t code =
                        (uint32_t)(packed >> (e * BITS)) & ((1u << BITS) - 1u);
                    const float k = recon(code, ks_s[g][d], kz_s[g][d]);
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        sc[j] = __builtin_fmaf(q_s[j][d], k, sc[j]);
                }
            }
        }
    } else if (tid < nt) {
        const uint16_t* krow =
            a.k_ring + ((int64_t)bh * a.ring + t % a.ring) * D;
        uint4 x[D8];
#pragma unroll
        for (int k = 0; k < D8; ++k) x[k] = load16(krow + k * 8);
#pragma unroll
        for (int c8 = 0; c8 < D8; ++c8) {
            const uint32_t ws[4] = {x[c8].x, x[c8].y, x[c8].z, x[c8].w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = c8 * 8 + e;
                const uint16_t h = (uint16_t)(ws[e >> 1] >> ((e & 1) * 16));
                const float k = widen16<DT>(h);
#pragma unroll
                for (int j = 0; j < NQ; ++j)
                    sc[j] = __builtin_fmaf(q_s[j][d], k, sc[j]);
            }
        }
    }

    // ---- softmax partial of the chunk, every query head at once ----
    float m[NQ], l[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        sc[j] = tid < nt ? sc[j] * a.sm_scale : -__builtin_huge_valf();
        m[j] = sc[j];
    }
    block_max_n<NQ>(m, red);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        const float p = tid < nt ? __expf(sc[j] - m[j]) : 0.0f;
        p_s[j][tid] = p;
        l[j] = p;
    }
    block_sum_n<NQ>(l, red);

    // ---- partial outputs: thread (channel chunk c8, token part) reads its
    // tokens' value codes straight from memory (consecutive threads take
    // consecutive chunks of a row), reconstructs them exactly as the value
    // dequantizer does, and accumulates p * v; the parts are then summed
    // with lane shuffles (inside a wave) and LDS (across the two waves).
    const int c8 = tid % D8, part = tid / D8;
    float o[NQ][8];
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] = 0.0f;
    // A quantized value is code * scale + zero with one (scale, zero) per
    // (token, value group), so its share of the output is taken as
    // (p * scale) * code plus p * zero, summed separately (zb).
    const int gv = (c8 * 8) / a.G_v;
    float zb[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) zb[j] = 0.0f;
#pragma unroll 4
    for (int tt = part; tt < nq_tok; tt += PARTS) {
        const int64_t row = (int64_t)bh * a.S_max + t0 + tt;
        const uint64_t pc = load_codes<BITS>(a.v_codes + row * row_bytes + c8 * BITS);
        const int64_t p = row * a.NGD + gv;
        const float sv = a.v_scale[p], zv = a.v_zero[p];
        float ws[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            const float pj = p_s[j][tt];
            ws[j] = pj * sv;
            zb[j] = __builtin_fmaf(pj, zv, zb[j]);
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = (float)((uint32_t)(pc >> (e * BITS)) & ((1u << BITS) - 1u));
#pragma unroll
            for (int j = 0; j < NQ; ++j) o[j][e] = __builtin_fmaf(ws[j], x, o[j][e]);
        }
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j)
#pragma unroll
        for (int e = 0; e < 8; ++e) o[j][e] += zb[j];
    // the exact tokens of the ring
    for (int tt = max(part, nq_tok + ((part - nq_tok) % PARTS + PARTS) % PARTS);
         tt < nt; tt += PARTS) {
        const uint4 v = load16(a.v_ring + ((int64_t)bh * a.ring + (t0 + tt) % a.ring) * D +
                               c8 * 8);
        const uint32_t ws[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const float x = widen16<DT>((uint16_t)(ws[e >> 1] >> ((e & 1) * 16)));
#pragma unroll
            for (int j = 0; j < NQ; ++j) o[j][e] = __builtin_fmaf(p_s[j][tt], x, o[j][e]);
        }
    }
    // parts inside a wave: lanes D8, 2 D8, ... apart
#pragma unroll
    for (int msk = D8; msk < 64; msk <<= 1)
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) o[j][e] += __shfl_xor(o[j][e], msk);
    // the second wave's sum into LDS, the first wave adds it and stores
    const int lane = tid & 63, wave = tid >> 6;
    if (wave == 1 && lane < D8)
#pragma unroll
        for (int j = 0; j < NQ; ++j)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc_s[j][c8 * 8 + e] = o[j][e];
    __syncthreads();
    if (wave == 1 || lane >= D8) return;
    float* w = a.work + ((int64_t)bh * a.n_chunks + chunk) * nq * att_slot(D);
#pragma unroll
    for (int j = 0; j < NQ; ++j) {
        if (j >= nq) break;
        float* wj = w + j * att_slot(D);
        if (c8 == 0) {
            wj[0] = m[j];
            wj[1] = l[j];
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) wj[kAttData + c8 * 8 + e] = o[j][e] + acc_s[j][c8 * 8 + e];
    }
}

// Merge the chunks of each (bh, query head): out = sum_c e^{m_c - M} o_c /
// sum_c e^{m_c - M} l_c with M = max_c m_c.  One wave per (bh, head), four
// per block, over batches of 32 chunks: every load of a batch is issued at
// once (lane c takes chunk c's m and l, every lane its channels of each
// chunk's o); the batch's maximum and denominator are reduced over the
// first 32 lanes (two DPP rows, then a swizzle) and read back as
// wave-uniform values, and
// the running sums are rescaled when the maximum grows (online softmax).
template <int CTRL>
__device__ __forceinline__ float merge_dpp(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}

// The value of lane l ^ 16 (within each 32 lanes): ds_swizzle, bit mode
// with xor mask 16.
__device__ __forceinline__ float merge_xor16(float v) {
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}

template <int DT, int D>
__global__ __launch_bounds__(256) void attend_merge_kernel(AttendArgs a,
                                                           int32_t n_pairs) {
    const int32_t pair = (int32_t)blockIdx.x * 4 + (int32_t)(threadIdx.x >> 6);
    if (pair >= n_pairs) return;                 // the whole wave
    const int lane = threadIdx.x & 63;
    const int nq = a.n_q, nc = a.n_chunks;
    const int bh = pair / nq, j = pair - bh * nq;
    const int64_t cs = (int64_t)nq * att_slot(D);        // chunk stride
    const float* w = a.work + (int64_t)bh * nc * cs + (int64_t)j * att_slot(D);
    constexpr int PER = D / 64;                  // channels per lane
    constexpr int B = 32;                        // chunks per batch
    float mx = -__builtin_huge_valf(), ls = 0.0f;
    float O[PER];
#pragma unroll
    for (int i = 0; i < PER; ++i) O[i] = 0.0f;
    for (int c0 = 0; c0 < nc; c0 += B) {         // wave-uniform
        const int nb = min(B, nc - c0);
        float2 ml = make_float2(-__builtin_huge_valf(), 0.0f);
        if (lane < nb) ml = *reinterpret_cast<const float2*>(w + (c0 + lane) * cs);
        float ov[B][PER];
#pragma unroll
        for (int c = 0; c < B; ++c)
#pragma unroll
            for (int i = 0; i < PER; ++i)
                ov[c][i] = c < nb ? w[(c0 + c) * cs + kAttData + lane + 64 * i] : 0.0f;
        // the batch maximum over lanes 0..31: quad_perm [1,0,3,2],
        // quad_perm [2,3,0,1], row_half_mirror, row_mirror, then lane ^ 16
        // (an LDS-unit swizzle)
        float bm = ml.x;
        bm = fmaxf(bm, merge_dpp<0xB1>(bm));
        bm = fmaxf(bm, merge_dpp<0x4E>(bm));
        bm = fmaxf(bm, merge_dpp<0x141>(bm));
        bm = fmaxf(bm, merge_dpp<0x140>(bm));
        bm = fmaxf(bm, merge_xor16(bm));
        // lane 0 (the first active lane: the whole wave runs) holds the result
        const float mnew =
            fmaxf(mx, __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(bm))));
        const float scale = __expf(mx - mnew);   // 0 on the first batch
        const float e = lane < nb ? __expf(ml.x - mnew) : 0.0f;
        float el = e * ml.y;
        el += merge_dpp<0xB1>(el);
        el += merge_dpp<0x4E>(el);
        el += merge_dpp<0x141>(el);
        el += merge_dpp<0x140>(el);
        el += merge_xor16(el);
        ls = ls * scale + __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(el)));
#pragma unroll
        for (int i = 0; i < PER; ++i) O[i] *= scale;
#pragma unroll
        for (int c = 0; c < B; ++c) {
            if (c < nb) {                        // wave-uniform
                const float ec = __int_as_float(
                    __builtin_amdgcn_readlane(__float_as_int(e), c));
#pragma unroll
                for (int i = 0; i < PER; ++i) O[i] = __builtin_fmaf(ec, ov[c][i], O[i]);
            }
        }
        mx = mnew;
    }
#pragma unroll
    for (int i = 0; i < PER; ++i) {
        const float r = O[i] / ls;
        uint16_t h;
        if constexpr (DT == DT_F16)
            h = __builtin_bit_cast(uint16_t, (_Float16)r);
        else
            h = __builtin_bit_cast(uint16_t, (__bf16)r);
        a.out[((int64_t)bh * nq + j) * D + lane + 64 * i] = h;
    }
}

template <int DT, int BITS, int D, int NQ>
static hipError_t launch_partial(const AttendArgs& a, int64_t BH, int64_t nc,
                                 hipStream_t stream) {
    return launch_kernel((attend_partial_kernel<DT, BITS, D, NQ>),
                         dim3((uint32_t)nc, (uint32_t)BH),
                         dim3(kAttChunk), 0, stream, a);
}

template <int DT, int BITS, int D>
static hipError_t launch_partial_nq(const AttendArgs& a, int64_t BH,
                                    int64_t nc, hipStream_t stream) {
    switch (a.n_q) {
        case 1: return launch_partial<DT, BITS, D, 1>(a, BH, nc, stream);
        case 2: return launch_partial<DT, BITS, D, 2>(a, BH, nc, stream);
        case 3: return launch_partial<DT, BITS, D, 3>(a, BH, nc, stream);
        case 4: return launch_partial<DT, BITS, D, 4>(a, BH, nc, stream);
        case 5:
        case 6: return launch_partial<DT, BITS, D, 6>(a, BH, nc, stream);
        default: return launch_partial<DT, BITS, D, 8>(a, BH, nc, stream);
    }
}

template <int DT, int BITS>
static hipError_t launch_attend_t(const AttendArgs& a0, int64_t BH,
                                  hipStream_t stream) {
    // Every chunk goes to the matrix-core kernel when its shape rules hold
    // (it takes the ring's exact tokens too: their scores on the matrix
    // cores, their values on the vector units); otherwise all go to the
    // token-per-thread kernel.
    AttendArgs a = a0;
    a.chunk0 = 0;
    const bool mfma = BITS <= 4 && (a.G_k == 16 || a.G_k == 32) && a.G_v >= 16;
    const int n_full = mfma ? a.n_chunks : 0;
    if (n_full > 0) {
        hipError_t e = launch_attend_mfma(a, BH, n_full, DT, BITS, stream);
        if (e != hipSuccess) return e;
        a.chunk0 = n_full;
    }
    if (a.chunk0 < a.n_chunks) {
        const int64_t nc = a.n_chunks - a.chunk0;
        hipError_t e = a.D == 64 ? launch_partial_nq<DT, BITS, 64>(a, BH, nc, stream)
                                 : launch_partial_nq<DT, BITS, 128>(a, BH, nc, stream);
        if (e != hipSuccess) return e;
    }
    const int32_t pairs = (int32_t)(BH * a.n_q);
    const dim3 grid((uint32_t)((pairs + 3) / 4)), block(256);
    return a.D == 64
        ? launch_kernel((attend_merge_kernel<DT, 64>), grid, block, 0, stream, a, pairs)
        : launch_kernel((attend_merge_kernel<DT, 128>), grid, block, 0, stream, a, pairs);
}

// The workspace of kivi_cache_attend_noalloc: a file-scope device array,
// one copy per GPU.  Host code never passes the array's own name to a
// kernel (on the host it is only a stand-in for the symbol); it uses the
// device address that hipGetSymbolAddress returns for the current device.
constexpr int64_t kScratchBytes = 32ll << 20;
constexpr int kMaxDevices = 64;
__device__ __align__(256) float scratch[kScratchBytes / 4];

namespace {
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};
}  // namespace

int64_t attend_scratch_bytes() { return kScratchBytes; }

hipError_t attend_scratch(float** ptr) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (g_scratch[dev] == nullptr) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch[dev] = static_cast<float*>(p);
    }
    *ptr = g_scratch[dev];
    return hipSuccess;
}

int64_t attend_chunks(int64_t T) { return (T + kAttChunk - 1) / kAttChunk; }

int64_t attend_work_floats(int64_t BH, int64_t T, int64_t D, int64_t n_q) {
    return BH * attend_chunks(T) * n_q * att_slot(D);
}

hipError_t launch_attend(const AttendArgs& a, int64_t BH, int dtype, int bits,
                         hipStream_t stream) {
    if (dtype == DT_F16) {
        switch (bits) {
            case 1: return launch_attend_t<DT_F16, 1>(a, BH, stream);
            case 2: return launch_attend_t<DT_F16, 2>(a, BH, stream);
            case 4: return launch_attend_t<DT_F16, 4>(a, BH, stream);
            default: return launch_attend_t<DT_F16, 8>(a, BH, stream);
        }
    }
    switch (bits) {
        case 1: return launch_attend_t<DT_BF16, 1>(a, BH, stream);
        case 2: return launch_attend_t<DT_BF16, 2>(a, BH, stream);
        case 4: return launch_attend_t<DT_BF16, 4>(a, BH, stream);
        default: return launch_attend_t<DT_BF16, 8>(a, BH, stream);
    }
}

}  // namespace kivi
