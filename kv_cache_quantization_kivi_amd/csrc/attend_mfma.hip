// Decode attention over the packed cache on the matrix cores (gfx950
// v_mfma_f32_16x16x32_f16) (KIVI blog post on the fused Metal kernels,
// section "So why does the kernel ship?": attention reads the packed codes
// and expands them in registers, never in memory).  Same chunking,
// workspace and merge as the token-per-thread kernel in attend.hip; this
// kernel computes the same quantities with the contractions over the
// quantized tokens moved to MFMA (the ring's exact tokens of the last
// chunks stay on the vector units):
//
//   scores  s[t][j] = sum_d (q[j][d] scale[g][d]) code[t][d] + sum_d q[j][d] zero[g][d]
//           A = codes (M = 16 tokens, K = 32 channels) as the f16
//               subnormals code * 2^-24, exact;
//           B = the scaled queries (K = channels, N = query heads), split in
//               two f16 parts hi + lo after scaling by a power of two 2^e
//               per (key group, head) that keeps them inside f16's range;
//   values  o[j][d] = sum_t (p[j][t] vscale[t][gv]) code[t][d] + sum_t p[j][t] vzero[t][gv]
//           A = codes transposed through LDS (M = 16 channels, K = 32 tokens),
//               as f16 subnormals too;
//           B = the weights p * vscale, hi + lo after a power-of-two scaling
//               per value group.
// f16 x f16 products are exact in fp32 and the matrix core accumulates in
// fp32; hi + lo carries about 22 bits of each scaled operand.  The bias and
// zero-point sums stay on the vector units in fp32.
//
// Operand layout of the 16x16x32 instruction (probed on gfx950): lane l
// holds A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16] for i < 8,
// and receives C[4 (l / 16) + i][l % 16] for i < 4.  The k index is free to
// map to any channel (or token) as long as A and B agree: lane block
// kb = l / 16 takes channels [kb D/4, (kb + 1) D/4), so a lane's codes of one
// token are one contiguous load.
#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2x_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kMChunk = 128;            // tokens per block, one per thread

// Sizes of one instantiation.  GK is the smallest key and value group the
// instantiation serves (16, or 32 when G_k = 32 and G_v >= 32): it bounds
// the key groups of a chunk and the value groups of a row, and so the LDS
// that holds their operands.  kWaves: the waves per SIMD that the LDS
// footprint allows (two waves per block, four SIMDs per CU, 160 KiB of LDS
// per CU), capped at 5 (4 for 4-bit codes); the launch bounds ask the
// compiler for registers that allow as many.
template <int BITS, int D, int NQ, int GK>
struct MfmaShape {
    static constexpr int D8 = D / 8;
    static constexpr int KS = D / 32;                 // k-steps over the channels
    static constexpr int CPL = D / 4;                 // channels of a lane block
    static constexpr int LB = CPL * BITS / 8;         // code bytes of a lane block
    static constexpr int DW = D * BITS / 32;          // code row in dwords
    static constexpr int MT = D / 16;                 // channel tiles (values)
    static constexpr int KGROUPS = kMChunk / GK;      // key groups of a chunk
    static constexpr int MAXGV = D / GK;              // value groups of a row
    static constexpr int VKS = kMChunk / 32;          // k-steps over the tokens
    static constexpr int kKOps = KGROUPS * 4 * NQ * KS * 2;   // uint4 key operands
    static constexpr int kVOps = MAXGV * 4 * NQ * VKS * 2;    // uint4 value operands
    static constexpr int kOps = kKOps > kVOps ? kKOps : kVOps;
    static constexpr int kZero = 2 * (KS > VKS ? KS : VKS);   // zero block (uint4)
    static constexpr int kLds =
        NQ * D * 4 + kOps * 16 + kZero * 16 + 2 * KGROUPS * NQ * 4 +
        NQ * kMChunk * 4 + DW * kMChunk * 4 + MAXGV * kMChunk * 4 +
        MAXGV * 4 + NQ * MAXGV * 4 + 2 * NQ * 4 + 256;       // + alignment
    static constexpr int kBlocks = (160 * 1024) / kLds;
    // 4-bit codes hold twice the key code registers: at most 4 waves there
    static constexpr int kCap = BITS == 4 ? 4 : 5;
    static constexpr int kWaves = kBlocks / 2 < 1 ? 1 : (kBlocks / 2 > kCap ? kCap : kBlocks / 2);
};

__device__ __forceinline__ h8_t as_h8(uint32_t a, uint32_t b, uint32_t c,
                                      uint32_t d) {
    return __builtin_bit_cast(h8_t, make_uint4(a, b, c, d));
}

// Codes enter the matrix cores as f16 subnormals: the bit pattern c (c <
// 1024) is exactly the f16 value c * 2^-24, so a code needs only to be
// masked into place; the products' 2^-24 is taken out again, exactly, with
// the operands' power-of-two scaling (kCodeExp).
constexpr int kCodeExp = 24;

// 8 codes held LSB-first in the low 8 * BITS bits of `bits` (higher bits
// zero) as 8 f16 values code * 2^-24, code 2k and 2k + 1 in dword k.
template <int BITS>
__device__ __forceinline__ h8_t codes8(uint32_t bits) {
    constexpr uint32_t M = (1u << BITS) - 1u;
    uint32_t d[4];
    if constexpr (BITS <= 2) {
        // a second copy 16 - BITS bits up puts code 2k + 1 at bit 16 + 2k BITS
        const uint32_t t = bits | (bits << (16 - BITS));
#pragma unroll
        for (int k = 0; k < 4; ++k) d[k] = (t >> (2 * k * BITS)) & (M | (M << 16));
    } else {
        // byte k holds codes 2k (low nibble) and 2k + 1: the low nibbles and
        // the high ones apart, then one byte permute per pair
        const uint32_t u = bits & 0x0f0f0f0fu, v = (bits >> 4) & 0x0f0f0f0fu;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            d[k] = __builtin_amdgcn_perm(v, u, (uint32_t)k | 0x0c00u |
                                                   ((uint32_t)(4 + k) << 16) | 0x0c000000u);
    }
    return as_h8(d[0], d[1], d[2], d[3]);
}

// Scaling exponent for operands bounded by P: P * 2^e < 2^14, so that hi
// and lo stay finite f16 values (0 when P is 0 or not finite).
__device__ __forceinline__ int op_exp(float P) {
    if (!(P > 0.0f) || !(P <= 3.0e38f)) return 0;
    // floor(log2 P) from the exponent field (a subnormal P counts as 2^-127,
    // which still keeps P * 2^e below 2^14)
    const int lg = (int)((__float_as_uint(P) >> 23) & 0xffu) - 127;
    return 13 - lg;
}

// x = hi + lo with hi = RN16(x) and lo = RN16(x - hi), for two values at
// once as packed pairs (x0 in the low halves): one paired conversion for the
// two hi parts and one for the two lo parts.
__device__ __forceinline__ void split16x2(float x0, float x1, uint32_t& hi,
                                          uint32_t& lo) {
    const h2x_t h = {(_Float16)x0, (_Float16)x1};
    const h2x_t l = {(_Float16)(x0 - (float)h.x), (_Float16)(x1 - (float)h.y)};
    hi = __builtin_bit_cast(uint32_t, h);
    lo = __builtin_bit_cast(uint32_t, l);
}

// An operand, or zeros when `keep` is false.
__device__ __forceinline__ h8_t pick_op(uint4 v, bool keep) {
    return as_h8(keep ? v.x : 0u, keep ? v.y : 0u, keep ? v.z : 0u, keep ? v.w : 0u);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o));
    return v;
}
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

template <int DT>
__device__ __forceinline__ float widen_h(uint16_t h) {
    if constexpr (DT == DT_F16)
        return (float)__builtin_bit_cast(_Float16, h);
    else
        return __uint_as_float((uint32_t)h << 16);
}

}  // namespace

// One 128-thread block (two waves) per (chunk, bh).  The chunk's quantized
// tokens (a whole number of key groups, since Q is G_k-aligned) go through
// the matrix cores; its ring tokens through the vector units.  The caller
// guarantees D in {64, 128}, BITS <= 4, G_k in {16, 32}, a value group of
// 16 * 2^k channels and n_q <= NQ.
//
// B operands live in LDS, each lane's operands of one group contiguous:
// keys [g][kb][j][k-step][hi, lo], values [gv][kb][j][k-step][hi, lo]
// (uint4 = 8 halves each).  Lanes past the query heads read a zero block
// instead (an LDS address select), so no operand needs masking.
template <int DT, int BITS, int D, int NQ, int GK>
__global__ __launch_bounds__(kMChunk, (MfmaShape<BITS, D, NQ, GK>::kWaves))
void attend_mfma_kernel(AttendArgs a) {
    using Sh = MfmaShape<BITS, D, NQ, GK>;
    constexpr int D8 = Sh::D8, KS = Sh::KS, CPL = Sh::CPL, LB = Sh::LB;
    constexpr int DW = Sh::DW, MT = Sh::MT, MAXGV = Sh::MAXGV, VKS = Sh::VKS;
    constexpr int kMaxKGroups = Sh::KGROUPS;
    constexpr int kOps = Sh::kOps, kZero = Sh::kZero;
    static_assert(NQ * MAXGV * kMChunk <= kOps * 4, "zero-point rows fit");

    __shared__ __attribute__((aligned(16))) float q_s[NQ][D];
    __shared__ __attribute__((aligned(16))) uint4 ops_s[kOps];
    __shared__ __attribute__((aligned(16))) uint4 zero_s[kZero];
    __shared__ float kbias_s[kMaxKGroups][NQ];
    __shared__ int kexp_s[kMaxKGroups][NQ];
    __shared__ __attribute__((aligned(16))) float p_s[NQ][kMChunk];
    // value codes by token pair: row q holds, for each pair of tokens
    // (2P, 2P + 1), the q-th 16 bits of each token's code row, the even
    // token's in the low half (rows padded to 68 dwords, which keeps the
    // two writers of a pair off one bank)
    constexpr int kVpStride = kMChunk / 2 + 4;
    __shared__ __attribute__((aligned(16))) uint32_t vp_s[2 * DW][kVpStride];
    __shared__ __attribute__((aligned(16))) float sv_s[MAXGV][kMChunk];
    __shared__ float vmax_s[MAXGV];
    __shared__ float zsum_s[NQ * MAXGV];
    __shared__ float ml_s[2][NQ];

    const int chunk = blockIdx.x, bh = blockIdx.y, tid = threadIdx.x;
    const int lane = tid & 63, wave = tid >> 6;
    const int m16 = lane & 15, kb = lane >> 4;
    const int nq = a.n_q;
    const int t0 = chunk * kMChunk;
    const int nt = min(kMChunk, a.T - t0);                 // tokens in the chunk
    const int nq_tok = max(0, min(nt, a.Q - t0));          // of them quantized
    const int gk_sh = a.G_k == 16 ? 4 : 5;     // G_k is 16 or 32
    const int ngk = nq_tok >> gk_sh;           // quantized key groups (Q is
                                               // G_k-aligned, so whole ones)
    const int g0 = t0 >> gk_sh;
    const int ngd = a.NGD;                     // value groups per token
    const int gv_sh = 31 - __builtin_clz((unsigned)a.G_v);   // G_v a power of two

    // ---- every load that depends on nothing, issued up front ----
    float qv[NQ];                              // query element d = tid
#pragma unroll
    for (int j = 0; j < NQ; ++j)
        qv[j] = (tid < D && j < nq) ? widen_h<DT>(a.q[((int64_t)bh * nq + j) * D + tid]) : 0.0f;
    // key params of this thread's item (key group g, 8-channel chunk c8)
    const bool kitem = tid < ngk * D8;
    const int kg = kitem ? tid / D8 : 0, kc8 = tid % D8;
    float ksc[8], kzr[8];
    {
        const int64_t p = ((int64_t)bh * a.NG + g0 + kg) * D + kc8 * 8;
        float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), s1 = s0, z0 = s0, z1 = s0;
        if (kitem) {
            s0 = *reinterpret_cast<const float4*>(a.k_scale + p);
            s1 = *reinterpret_cast<const float4*>(a.k_scale + p + 4);
            z0 = *reinterpret_cast<const float4*>(a.k_zero + p);
            z1 = *reinterpret_cast<const float4*>(a.k_zero + p + 4);
        }
        ksc[0] = s0.x; ksc[1] = s0.y; ksc[2] = s0.z; ksc[3] = s0.w;
        ksc[4] = s1.x; ksc[5] = s1.y; ksc[6] = s1.z; ksc[7] = s1.w;
        kzr[0] = z0.x; kzr[1] = z0.y; kzr[2] = z0.z; kzr[3] = z0.w;
        kzr[4] = z1.x; kzr[5] = z1.y; kzr[6] = z1.z; kzr[7] = z1.w;
    }
    // this lane's key code blocks of its four 16-token tiles
    constexpr int LBW = LB >= 4 ? LB / 4 : 1;
    uint32_t kw[4][LBW];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tok0 = (wave + 2 * tt) * 16;
        kw[tt][0] = 0u;
        if (tok0 >= nq_tok) continue;          // no codes past Q
        const uint8_t* crow = a.k_codes +
            ((int64_t)bh * a.S_max + t0 + tok0 + m16) * (D * BITS / 8) + kb * LB;
        if constexpr (LB == 16) {
            const uint4 v = *reinterpret_cast<const uint4*>(crow);
            kw[tt][0] = v.x; kw[tt][1] = v.y; kw[tt][2] = v.z; kw[tt][3] = v.w;
        } else if constexpr (LB == 8) {
            const uint2 v = *reinterpret_cast<const uint2*>(crow);
            kw[tt][0] = v.x; kw[tt][1] = v.y;
        } else if constexpr (LB == 4) {
            kw[tt][0] = *reinterpret_cast<const uint32_t*>(crow);
        } else {
            kw[tt][0] = *reinterpret_cast<const uint16_t*>(crow);
        }
    }
    // this thread's token: value code row and value params
    const int64_t vrow = (int64_t)bh * a.S_max + t0 + tid;
    uint32_t vw[DW];
#pragma unroll
    for (int k = 0; k < DW; ++k) vw[k] = 0u;
    const bool vq = tid < nq_tok;              // this token is quantized
    if (vq) {
        const uint8_t* vp = a.v_codes + vrow * (D * BITS / 8);
        if constexpr (DW >= 4) {
#pragma unroll
            for (int k = 0; k < DW / 4; ++k) {
                const uint4 v = *reinterpret_cast<const uint4*>(vp + 16 * k);
                vw[4 * k] = v.x; vw[4 * k + 1] = v.y; vw[4 * k + 2] = v.z; vw[4 * k + 3] = v.w;
            }
        } else {
            const uint2 v = *reinterpret_cast<const uint2*>(vp);
            vw[0] = v.x; vw[1] = v.y;
        }
    }
    float svv[MAXGV], zvv[MAXGV];
#pragma unroll
    for (int gv = 0; gv < MAXGV; ++gv) {
        svv[gv] = (vq && gv < ngd) ? a.v_scale[vrow * ngd + gv] : 0.0f;
        zvv[gv] = (vq && gv < ngd) ? a.v_zero[vrow * ngd + gv] : 0.0f;
    }

    // queries and the zero block into LDS
#pragma unroll
    for (int j = 0; j < NQ; ++j)
        if (tid < D) q_s[j][tid] = qv[j];
    if (tid < kZero) zero_s[tid] = make_uint4(0u, 0u, 0u, 0u);
    __syncthreads();

    // ---- key operands: q[j][d] scale[g][d] 2^e(g, j) as hi + lo and the
    // zero bias.  Thread = item (g, 8-channel chunk) for every head; the D8
    // items of a group sit in consecutive lanes (all items, or none), where
    // each head's maximum (for e) and bias sum meet in xor shuffles. ----
    if (kitem) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float pr[8], b = 0.0f, mxl = 0.0f;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float qd = q_s[j][kc8 * 8 + i];
                pr[i] = qd * ksc[i];
                mxl = fmaxf(mxl, fabsf(pr[i]));
                b = __builtin_fmaf(qd, kzr[i], b);
            }
#pragma unroll
            for (int o = 1; o < D8; o <<= 1) {
                b += __shfl_xor(b, o);
                mxl = fmaxf(mxl, __shfl_xor(mxl, o));
            }
            if (kitem) {
                const int e = op_exp(mxl);
                uint32_t hw[4], lw[4];
#pragma unroll
                for (int i = 0; i < 8; i += 2) {
                    split16x2(__builtin_ldexpf(pr[i], e), __builtin_ldexpf(pr[i + 1], e),
                              hw[i / 2], lw[i / 2]);
                }
                const int d = kc8 * 8, blk = d / CPL, s = (d % CPL) / 8;
                uint4* ob = ops_s + ((kg * 4 + blk) * NQ + j) * (2 * KS);
                ob[2 * s] = make_uint4(hw[0], hw[1], hw[2], hw[3]);
                ob[2 * s + 1] = make_uint4(lw[0], lw[1], lw[2], lw[3]);
                if (kc8 == 0) {
                    kbias_s[kg][j] = b;
                    kexp_s[kg][j] = e;
                }
            }
        }
    }
    __syncthreads();

    // ---- scores on the matrix cores: wave w takes 16-token tiles w, w+2, ...
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tok0 = (wave + 2 * tt) * 16;
        if (tok0 >= nq_tok) break;             // wave-uniform
        const int g = tok0 >> gk_sh;
        const uint4* bp = m16 < NQ ? ops_s + ((g * 4 + kb) * NQ + m16) * (2 * KS) : zero_s;
        f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < KS; ++s) {
            constexpr int SB = 8 * BITS;                    // bits per k-step
            const int bit = s * SB;
            uint32_t bits = kw[tt][bit / 32] >> (bit % 32);
            if constexpr (SB < 32) bits &= (1u << SB) - 1u;
            const h8_t A = codes8<BITS>(bits);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                A, __builtin_bit_cast(h8_t, bp[2 * s]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                A, __builtin_bit_cast(h8_t, bp[2 * s + 1]), acc, 0, 0, 0);
        }
        if (m16 < NQ) {
            const int e = kexp_s[g][m16];
            const float bias = kbias_s[g][m16];
#pragma unroll
            for (int i = 0; i < 4; ++i)
                p_s[m16][tok0 + kb * 4 + i] = __builtin_ldexpf(acc[i], kCodeExp - e) + bias;
        }
    }
    __syncthreads();

    // ---- the ring's exact keys (tokens nq_tok .. nt - 1): thread = token
    if (tid >= nq_tok && tid < nt) {
        const uint16_t* krow = a.k_ring + ((int64_t)bh * a.ring + (t0 + tid) % a.ring) * D;
        float sc[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) sc[j] = 0.0f;
#pragma unroll 4
        for (int c8 = 0; c8 < D8; ++c8) {
            const uint4 x = *reinterpret_cast<const uint4*>(krow + c8 * 8);
            const uint32_t wx[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const float k = widen_h<DT>((uint16_t)(wx[e >> 1] >> ((e & 1) * 16)));
#pragma unroll
                for (int j = 0; j < NQ; ++j) sc[j] = __builtin_fmaf(q_s[j][c8 * 8 + e], k, sc[j]);
            }
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) p_s[j][tid] = sc[j];
    }
    __syncthreads();

    // ---- softmax partial of the chunk: eight lanes per head find the max,
    // then every thread takes its token's p, then eight lanes per head sum
    // (rows are 512 bytes apart, so each row's lanes start at another eight
    // banks: lane i of row j reads t = i + 8 ((u + j) mod 16) at step u)
    if (tid < 8 * NQ) {
        const int j = tid >> 3;
        float v = -__builtin_huge_valf();
#pragma unroll 4
        for (int u = 0; u < kMChunk / 8; ++u) {
            const int t = (tid & 7) + 8 * ((u + j) & (kMChunk / 8 - 1));
            if (t < nt) v = fmaxf(v, p_s[j][t] * a.sm_scale);
        }
#pragma unroll
        for (int o = 1; o < 8; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
        if ((tid & 7) == 0) ml_s[0][j] = v;
    }
    // value codes (by token pair) and value scales of this thread's token
    // into LDS
    {
        // the even thread of a pair writes rows of words [0, DW/2), the odd
        // one rows of words [DW/2, DW); each first swaps with its partner
        // the words the partner needs (DW >= 4 on this path)
        const bool even = (tid & 1) == 0;
        const uint32_t sel_lo = even ? 0x05040100u : 0x01000504u;
        const uint32_t sel_hi = even ? 0x07060302u : 0x03020706u;
        uint32_t* row = &vp_s[even ? 0 : DW][tid >> 1];
#pragma unroll
        for (int k = 0; k < DW / 2; ++k) {
            const uint32_t lo_w = vw[k], hi_w = vw[k + DW / 2];   // static indices
            const uint32_t mine = even ? lo_w : hi_w;
            const uint32_t other = (uint32_t)__shfl_xor((int)(even ? hi_w : lo_w), 1);
            row[(2 * k) * kVpStride] = __builtin_amdgcn_perm(other, mine, sel_lo);
            row[(2 * k + 1) * kVpStride] = __builtin_amdgcn_perm(other, mine, sel_hi);
        }
    }
#pragma unroll
    for (int gv = 0; gv < MAXGV; ++gv)
        if (gv < ngd) sv_s[gv][tid] = svv[gv];
    __syncthreads();
    float pt[NQ];                              // this token's p per head
#pragma unroll
    for (int j = 0; j < NQ; ++j)
        pt[j] = tid < nt ? __expf(p_s[j][tid] * a.sm_scale - ml_s[0][j]) : 0.0f;
    // zero-point products into the (now free) operand region, [j*ngd+gv][t]
    float* zrows = reinterpret_cast<float*>(ops_s);
#pragma unroll
    for (int gv = 0; gv < MAXGV; ++gv) {
        if (gv < ngd) {
#pragma unroll
            for (int j = 0; j < NQ; ++j) zrows[(j * ngd + gv) * kMChunk + tid] = pt[j] * zvv[gv];
        }
    }
#pragma unroll
    for (int j = 0; j < NQ; ++j) p_s[j][tid] = pt[j];
    __syncthreads();
    // the ring's exact values: thread = channel, summed over the ring tokens
    // into the (now free) query rows
    const bool has_ring = nq_tok < nt;        // block-uniform
    if (has_ring && tid < D) {
        float o[NQ];
#pragma unroll
        for (int j = 0; j < NQ; ++j) o[j] = 0.0f;
        // eight tokens' loads in flight at a time
        for (int tb = nq_tok; tb < nt; tb += 8) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                const int t = min(tb + u, nt - 1);
                v[u] = widen_h<DT>(
                    a.v_ring[((int64_t)bh * a.ring + (t0 + t) % a.ring) * D + tid]);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
                if (tb + u < nt) {
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        o[j] = __builtin_fmaf(p_s[j][tb + u], v[u], o[j]);
                }
            }
        }
#pragma unroll
        for (int j = 0; j < NQ; ++j) q_s[j][tid] = o[j];
    }
    // eight lanes per row: the sums of p (per head) and of p * zero, and the
    // maxima of the value scales (rotated starts as above: the eight rows a
    // wave reads at once sit in distinct banks)
    const int n_sum = NQ + NQ * ngd;
    for (int k = tid >> 3; k < n_sum + ngd; k += kMChunk / 8) {
        if (k < n_sum) {
            const float* row = k < NQ ? p_s[k] : zrows + (k - NQ) * kMChunk;
            float v = 0.0f;
#pragma unroll 4
            for (int u = 0; u < kMChunk / 8; ++u)
                v += row[(tid & 7) + 8 * ((u + k) & (kMChunk / 8 - 1))];
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) v += __shfl_xor(v, o);
            if ((tid & 7) == 0) {
                if (k < NQ) ml_s[1][k] = v;
                else zsum_s[k - NQ] = v;
            }
        } else {
            const float* row = sv_s[k - n_sum];
            float v = 0.0f;
#pragma unroll 4
            for (int u = 0; u < kMChunk / 8; ++u)
                v = fmaxf(v, row[(tid & 7) + 8 * ((u + k) & (kMChunk / 8 - 1))]);
#pragma unroll
            for (int o = 1; o < 8; o <<= 1) v = fmaxf(v, __shfl_xor(v, o));
            if ((tid & 7) == 0) vmax_s[k - n_sum] = v;
        }
    }
    __syncthreads();
    // weights p * vscale * 2^e(gv) of this token, hi + lo, at k index
    // (token) k-step tid / 32, lane block (tid % 32) / 8, element tid % 8
    {
        _Float16* vops = reinterpret_cast<_Float16*>(ops_s);
        const int s4 = tid >> 5, blk = (tid >> 3) & 3, i = tid & 7;
        for (int gv = 0; gv < ngd; ++gv) {
            const int e = op_exp(vmax_s[gv]);
            const float sv = sv_s[gv][tid];   // this token's scale
            // heads in pairs: one paired conversion per pair for hi and lo
#pragma unroll
            for (int j = 0; j < NQ; j += 2) {
                const float w0 = __builtin_ldexpf(pt[j] * sv, e);
                const float w1 = j + 1 < NQ ? __builtin_ldexpf(pt[j + 1] * sv, e) : 0.0f;
                uint32_t hi, lo;
                split16x2(w0, w1, hi, lo);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (j + u < NQ) {
                        _Float16* vb = vops + ((gv * 4 + blk) * NQ + j + u) * (2 * VKS) * 8;
                        vb[(2 * s4) * 8 + i] = __builtin_bit_cast(_Float16, (uint16_t)(hi >> (16 * u)));
                        vb[(2 * s4 + 1) * 8 + i] = __builtin_bit_cast(_Float16, (uint16_t)(lo >> (16 * u)));
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- values on the matrix cores: wave w takes channel tiles w, w+2, ...
    float* wbase = a.work + ((int64_t)bh * a.n_chunks + chunk) * nq * (D + 2);
    for (int mt = wave; mt < MT; mt += 2) {
        const int gv = (mt * 16) >> gv_sh;
        const int ch = mt * 16 + m16;                   // this lane's A row
        const int q = (ch * BITS) / 16, sh = (ch * BITS) % 16;
        const uint32_t pmask = ((1u << BITS) - 1u) * 0x10001u;
        const uint4* bp = m16 < NQ ? ops_s + ((gv * 4 + kb) * NQ + m16) * (2 * VKS) : zero_s;
        f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s4 = 0; s4 < VKS; ++s4) {
            // tokens s4*32 + kb*8 + [0, 8) are pairs P0 .. P0 + 3, each dword
            // holding this channel's two codes sh bits up in its two halves
            const int P0 = s4 * 16 + kb * 4;
            const uint4 d = *reinterpret_cast<const uint4*>(&vp_s[q][P0]);
            const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
            constexpr uint32_t M = (1u << BITS) - 1u;
            uint32_t pr[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) pr[k] = (dw[k] >> sh) & pmask;   // codes * 2^-24
            const h8_t A = as_h8(pr[0], pr[1], pr[2], pr[3]);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                A, __builtin_bit_cast(h8_t, bp[2 * s4]), acc, 0, 0, 0);
            acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                A, __builtin_bit_cast(h8_t, bp[2 * s4 + 1]), acc, 0, 0, 0);
        }
        // C: lane (head m16, row block kb) holds channels mt*16 + 4 kb + i
        if (m16 < nq) {
            const int e = op_exp(vmax_s[gv]);
            const float zs = zsum_s[m16 * ngd + gv];
            float* wj = wbase + m16 * (D + 2);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int ch = mt * 16 + kb * 4 + i;
                wj[2 + ch] = __builtin_ldexpf(acc[i], kCodeExp - e) + zs +
                             (has_ring ? q_s[m16][ch] : 0.0f);
            }
        }
    }
    if (tid < nq) {
        wbase[tid * (D + 2)] = ml_s[0][tid];
        wbase[tid * (D + 2) + 1] = ml_s[1][tid];
    }
}

template <int DT, int BITS, int D, int NQ>
static hipError_t launch_mfma_t(const AttendArgs& a, int64_t BH, int n_full,
                                hipStream_t stream) {
    const dim3 grid((uint32_t)n_full, (uint32_t)BH), block(kMChunk);
    if (a.G_k == 32 && a.G_v >= 32)
        return launch_kernel((attend_mfma_kernel<DT, BITS, D, NQ, 32>), grid,
                             block, 0, stream, a);
    return launch_kernel((attend_mfma_kernel<DT, BITS, D, NQ, 16>), grid,
                         block, 0, stream, a);
}

template <int DT, int BITS, int D>
static hipError_t launch_mfma_nq(const AttendArgs& a, int64_t BH, int n_full,
                                 hipStream_t stream) {
    switch (a.n_q) {
        case 1: return launch_mfma_t<DT, BITS, D, 1>(a, BH, n_full, stream);
        case 2: return launch_mfma_t<DT, BITS, D, 2>(a, BH, n_full, stream);
        case 3: return launch_mfma_t<DT, BITS, D, 3>(a, BH, n_full, stream);
        case 4: return launch_mfma_t<DT, BITS, D, 4>(a, BH, n_full, stream);
        case 5:
        case 6: return launch_mfma_t<DT, BITS, D, 6>(a, BH, n_full, stream);
        default: return launch_mfma_t<DT, BITS, D, 8>(a, BH, n_full, stream);
    }
}

template <int DT, int BITS>
static hipError_t launch_mfma_d(const AttendArgs& a, int64_t BH, int n_full,
                                hipStream_t stream) {
    return a.D == 64 ? launch_mfma_nq<DT, BITS, 64>(a, BH, n_full, stream)
                     : launch_mfma_nq<DT, BITS, 128>(a, BH, n_full, stream);
}

template <int DT>
static hipError_t launch_mfma_bits(const AttendArgs& a, int64_t BH, int n_full,
                                   int bits, hipStream_t stream) {
    switch (bits) {
        case 1: return launch_mfma_d<DT, 1>(a, BH, n_full, stream);
        case 2: return launch_mfma_d<DT, 2>(a, BH, n_full, stream);
        default: return launch_mfma_d<DT, 4>(a, BH, n_full, stream);
    }
}

hipError_t launch_attend_mfma(const AttendArgs& a, int64_t BH, int n_full,
                              int dtype, int bits, hipStream_t stream) {
    return dtype == DT_F16 ? launch_mfma_bits<DT_F16>(a, BH, n_full, bits, stream)
                           : launch_mfma_bits<DT_BF16>(a, BH, n_full, bits, stream);
}

}  // namespace kivi
