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
// Keys of tokens t < Q are reconstructed from codes and their group's
// params as the dequantizer does, RN(RN(code * scale) + zero), in fp32 (no
// narrowing to 16 bits); values of tokens t < Q are reconstructed and
// narrowed exactly as kivi_dequant_values produces them; tokens t >= Q come
// from the ring as stored.  Scores and the softmax are fp32.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

constexpr int kAttChunk = 128;   // tokens per block (one per thread)
constexpr int kAttMaxQ = 8;      // query heads per KV head
constexpr int kAttMaxD = 128;    // head dimension
constexpr int kAttMaxGroups = kAttChunk / 8;   // key groups in a chunk (G_k >= 8)

__device__ __forceinline__ float block_reduce_max(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    v = fmaxf(red[0], red[1]);
    __syncthreads();
    return v;
}

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    const int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    v = red[0] + red[1];
    __syncthreads();
    return v;
}

template <int DT>
__device__ __forceinline__ float widen16(uint16_t h) {
    if constexpr (DT == DT_F16)
        return (float)__builtin_bit_cast(_Float16, h);
    else
        return __uint_as_float((uint32_t)h << 16);
}

// Workspace per (bh, chunk, query head): m, l, then D partial outputs.
__host__ __device__ inline int64_t att_slot(int64_t D) { return D + 2; }

template <int DT, int BITS>
__global__ __launch_bounds__(kAttChunk) void attend_partial_kernel(AttendArgs a) {
    __shared__ float q_s[kAttMaxQ][kAttMaxD];
    __shared__ float ks_s[kAttMaxGroups][kAttMaxD + 4];   // key scale, zero
    __shared__ float kz_s[kAttMaxGroups][kAttMaxD + 4];
    __shared__ float p_s[kAttMaxQ][kAttChunk];
    __shared__ __attribute__((aligned(16))) uint16_t v_s[kAttChunk][kAttMaxD];
    __shared__ float red[2];

    const int chunk = blockIdx.x;
    const int bh = blockIdx.y;
    const int tid = threadIdx.x;
    const int D = a.D, D8 = a.D / 8, nq = a.n_q;
    const int t0 = chunk * kAttChunk;
    const int nt = min(kAttChunk, a.T - t0);           // tokens in this chunk
    const int nq_tok = max(0, min(nt, a.Q - t0));      // of them quantized
    const int64_t row_bytes = (int64_t)D8 * BITS;

    // query heads (widened once)
    for (int i = tid; i < nq * D; i += kAttChunk)
        q_s[i / D][i % D] =
            widen16<DT>(a.q[((int64_t)bh * nq + i / D) * D + i % D]);
    // key params of the chunk's quantized groups (chunks are group-aligned)
    const int g0 = t0 / a.G_k;
    const int ng = (nq_tok + a.G_k - 1) / a.G_k;
    for (int i = tid; i < ng * D; i += kAttChunk) {
        const int64_t p = ((int64_t)bh * a.NG + g0 + i / D) * D + i % D;
        ks_s[i / D][i % D] = a.k_scale[p];
        kz_s[i / D][i % D] = a.k_zero[p];
    }
    __syncthreads();

    // ---- scores: one token per thread ----
    float sc[kAttMaxQ];
#pragma unroll
    for (int j = 0; j < kAttMaxQ; ++j) sc[j] = 0.0f;
    const int t = t0 + tid;
    if (tid < nq_tok) {
        const uint8_t* crow = a.k_codes + ((int64_t)bh * a.S_max + t) * row_bytes;
        const int g = t / a.G_k - g0;   // this token's group in ks_s / kz_s
        for (int c8 = 0; c8 < D8; ++c8) {
            const uint64_t packed = load_codes<BITS>(crow + c8 * BITS);
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = c8 * 8 + e;
                const uint32_t code =
                    (uint32_t)(packed >> (e * BITS)) & ((1u << BITS) - 1u);
                const float k = recon(code, ks_s[g][d], kz_s[g][d]);
#pragma unroll
                for (int j = 0; j < kAttMaxQ; ++j)
                    if (j < nq) sc[j] = __builtin_fmaf(q_s[j][d], k, sc[j]);
            }
        }
    } else if (tid < nt) {
        const uint16_t* krow =
            a.k_ring + ((int64_t)bh * a.ring + t % a.ring) * D;
        for (int c8 = 0; c8 < D8; ++c8) {
            const uint4 w = load16(krow + c8 * 8);
            const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int d = c8 * 8 + e;
                const uint16_t h = (uint16_t)(ws[e >> 1] >> ((e & 1) * 16));
                const float k = widen16<DT>(h);
#pragma unroll
                for (int j = 0; j < kAttMaxQ; ++j)
                    if (j < nq) sc[j] = __builtin_fmaf(q_s[j][d], k, sc[j]);
            }
        }
    }

    // ---- softmax partial of the chunk, per query head ----
    float m[kAttMaxQ], l[kAttMaxQ];
#pragma unroll
    for (int j = 0; j < kAttMaxQ; ++j) {
        if (j >= nq) break;
        const float s = tid < nt ? sc[j] * a.sm_scale : -__builtin_huge_valf();
        m[j] = block_reduce_max(s, red);
        const float p = tid < nt ? __expf(s - m[j]) : 0.0f;
        p_s[j][tid] = p;
        l[j] = block_reduce_sum(p, red);
    }

    // ---- the chunk's values, as 16-bit recon, into LDS ----
    for (int i = tid; i < nt * D8; i += kAttChunk) {
        const int tt = i / D8, c8 = i % D8;
        const int ts = t0 + tt;
        uint4 v;
        if (tt < nq_tok) {
            const int64_t r = (int64_t)bh * a.S_max + ts;
            const uint64_t packed = load_codes<BITS>(a.v_codes + r * row_bytes + c8 * BITS);
            const int64_t p = r * a.NGD + (c8 * 8) / a.G_v;
            const float s = a.v_scale[p], z = a.v_zero[p];
            const float sv[8] = {s, s, s, s, s, s, s, s};
            const float zv[8] = {z, z, z, z, z, z, z, z};
            v = dequant_chunk<DT, BITS>(packed, sv, zv);
        } else {
            v = load16(a.v_ring + ((int64_t)bh * a.ring + ts % a.ring) * D + c8 * 8);
        }
        *reinterpret_cast<uint4*>(&v_s[tt][c8 * 8]) = v;
    }
    __syncthreads();

    // ---- partial outputs: threads split (channel, token stride) ----
    const int per = kAttChunk / D;            // threads per channel (1 or 2)
    const int d = tid % D, part = tid / D;
    float o[kAttMaxQ];
#pragma unroll
    for (int j = 0; j < kAttMaxQ; ++j) o[j] = 0.0f;
    for (int tt = part; tt < nt; tt += per) {
        const float v = widen16<DT>(v_s[tt][d]);
#pragma unroll
        for (int j = 0; j < kAttMaxQ; ++j)
            if (j < nq) o[j] = __builtin_fmaf(p_s[j][tt], v, o[j]);
    }
    float* w = a.work + ((int64_t)bh * a.n_chunks + chunk) * nq * att_slot(D);
    if (per > 1) {
        // fold the second half of the threads into the first, through LDS
        __syncthreads();
        float* acc = reinterpret_cast<float*>(&v_s[0][0]);   // reuse
        if (part == 1)
#pragma unroll
            for (int j = 0; j < kAttMaxQ; ++j)
                if (j < nq) acc[j * D + d] = o[j];
        __syncthreads();
        if (part == 1) return;
#pragma unroll
        for (int j = 0; j < kAttMaxQ; ++j)
            if (j < nq) o[j] += acc[j * D + d];
    }
#pragma unroll
    for (int j = 0; j < kAttMaxQ; ++j) {
        if (j >= nq) break;
        float* wj = w + j * att_slot(D);
        if (d == 0) { wj[0] = m[j]; wj[1] = l[j]; }
        wj[2 + d] = o[j];
    }
}

// Merge the chunks of each bh: out = sum_c e^{m_c - M} o_c / sum_c e^{m_c - M} l_c.
template <int DT>
__global__ __launch_bounds__(128) void attend_merge_kernel(AttendArgs a) {
    const int bh = blockIdx.x;
    const int D = a.D, nq = a.n_q;
    for (int i = threadIdx.x; i < nq * D; i += 128) {
        const int j = i / D, d = i % D;
        const float* w = a.work + (int64_t)bh * a.n_chunks * nq * att_slot(D) +
                         j * att_slot(D);
        float M = -__builtin_huge_valf();
        for (int c = 0; c < a.n_chunks; ++c)
            M = fmaxf(M, w[(int64_t)c * nq * att_slot(D)]);
        float L = 0.0f, O = 0.0f;
        for (int c = 0; c < a.n_chunks; ++c) {
            const float* wc = w + (int64_t)c * nq * att_slot(D);
            const float f = __expf(wc[0] - M);
            L = __builtin_fmaf(f, wc[1], L);
            O = __builtin_fmaf(f, wc[2 + d], O);
        }
        const float r = O / L;
        uint16_t h;
        if constexpr (DT == DT_F16)
            h = __builtin_bit_cast(uint16_t, (_Float16)r);
        else
            h = __builtin_bit_cast(uint16_t, (__bf16)r);
        a.out[((int64_t)bh * nq + j) * D + d] = h;
    }
}

template <int DT, int BITS>
static hipError_t launch_attend_t(const AttendArgs& a, int64_t BH,
                                  hipStream_t stream) {
    hipError_t e = launch_kernel((attend_partial_kernel<DT, BITS>),
                                 dim3((uint32_t)a.n_chunks, (uint32_t)BH),
                                 dim3(kAttChunk), 0, stream, a);
    if (e != hipSuccess) return e;
    return launch_kernel((attend_merge_kernel<DT>), dim3((uint32_t)BH),
                         dim3(128), 0, stream, a);
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
