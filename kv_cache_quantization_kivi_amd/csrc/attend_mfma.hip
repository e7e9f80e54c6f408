// Decode attention over the packed cache on the matrix cores (gfx950
// v_mfma_f32_16x16x32_f16) (KIVI blog post on the fused Metal kernels,
// section "So why does the kernel ship?": attention reads the packed codes
// and expands them in registers, never in memory).  Same chunking,
// workspace and merge as the token-per-thread kernel in attend.hip; this
// kernel computes the same quantities with the contractions over the
// quantized tokens moved to MFMA, and the scores of the ring's exact tokens
// too (their values stay on the vector units):
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
// The hi parts of head j are B's column j and the lo parts its column 8 + j
// (n_q <= 8), so one instruction takes both; the two columns of C meet in
// one add across lanes 8 apart (DPP row rotation).  f16 x f16 products are
// exact in fp32 and the matrix core accumulates in fp32; hi + lo carries
// about 22 bits of each scaled operand.  The bias and zero-point sums stay
// on the vector units in fp32.
//
// Operand layout of the 16x16x32 instruction (probed on gfx950): lane l
// holds A[l % 16][8 (l / 16) + i] and B[8 (l / 16) + i][l % 16] for i < 8,
// and receives C[4 (l / 16) + i][l % 16] for i < 4.  The k index is free to
// map to any channel (or token) as long as A and B agree: lane block
// kb = l / 16 takes channels [kb D/4, (kb + 1) D/4), so a lane's codes of one
// token are one contiguous load.
#include <algorithm>

#include "kivi_device.h"
#include "kivi_launch.h"

namespace kivi {

namespace {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef _Float16 h2x_t __attribute__((ext_vector_type(2)));
typedef float f4_t __attribute__((ext_vector_type(4)));

constexpr int kMChunk = 128;            // tokens per block, one per thread

// Sizes of one instantiation.  GK is the smallest key and value group the
// instantiation serves (16, or 32 when G_k = 32 and G_v >= 32): it bounds
// the key groups of a chunk and the value groups of a row, and so the LDS
// that holds their operands.  kMinBlocks: the launch bounds' second
// argument, the blocks per CU whose residency the compiler must allow with
// its register choice (k blocks of two waves on four SIMDs: registers for
// k / 2 waves per SIMD).  It is half the blocks the LDS footprint allows
// (160 KiB per CU), capped at 5 (4 for 4-bit codes, whose key code
// registers double), so it only limits the largest instantiations; the
// common ones compile well inside it (2-bit, D = 128, three query heads:
// 75 VGPRs, 6 waves per SIMD).
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
    static constexpr int kKOps = KGROUPS * 4 * 2 * NQ * KS;   // uint4 key operands
    static constexpr int kVOps = MAXGV * 4 * 2 * NQ * VKS;    // uint4 value operands
    static constexpr int kPRow = kMChunk + 4;   // score rows, padded by 16 bytes
    static constexpr int kVpStride = kMChunk / 2 + 4;   // value code rows, padded
    static constexpr int kEarly = NQ * D * 2 + 2 * KGROUPS * NQ * 4;
    static constexpr int kVp = 2 * DW * kVpStride * 4;
    static constexpr int kOps = kKOps > kVOps ? kKOps : kVOps;
    // half-items of the key operands (a key group's 4 channels) per thread
    static constexpr int KH = (KGROUPS * D8 * 2 + kMChunk - 1) / kMChunk;
    static constexpr int kLds =
        (kEarly > kVp ? kEarly : kVp) + kOps * 16 + NQ * kPRow * 4 +
        MAXGV * 16 + MAXGV * 4 + NQ * 8 * 4 + 2 * NQ * 4 + 256;   // + alignment
    static constexpr int kBlocks = (160 * 1024) / kLds;
    // 4-bit codes hold twice the key code registers: at most 4 waves there
    static constexpr int kCap = BITS == 4 ? 4 : 5;
    static constexpr int kMinBlocks =
        kBlocks / 2 < 1 ? 1 : (kBlocks / 2 > kCap ? kCap : kBlocks / 2);
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

// The 16 two-bit codes of a dword as the A operands of two k-steps (codes
// 0-7, codes 8-15), f16 subnormals as codes8 makes them: the four codes
// 4k + r of byte k sit in byte k of copy r (a shift and a mask each), and
// one byte permute per operand dword takes a code pair from two copies.
__device__ __forceinline__ void codes16_2bit(uint32_t w, h8_t& A0, h8_t& A1) {
    const uint32_t m = 0x03030303u;
    const uint32_t u0 = w & m, v0 = (w >> 2) & m, u1 = (w >> 4) & m, v1 = (w >> 6) & m;
    // byte 0 of the result from byte b of the first copy, byte 2 from byte b
    // of the second, bytes 1 and 3 zero
#define KIVI_PAIR(x, y, b) __builtin_amdgcn_perm((y), (x), 0x0c000c00u | (b) | ((4u + (b)) << 16))
    A0 = as_h8(KIVI_PAIR(u0, v0, 0u), KIVI_PAIR(u1, v1, 0u), KIVI_PAIR(u0, v0, 1u),
               KIVI_PAIR(u1, v1, 1u));
    A1 = as_h8(KIVI_PAIR(u0, v0, 2u), KIVI_PAIR(u1, v1, 2u), KIVI_PAIR(u0, v0, 3u),
               KIVI_PAIR(u1, v1, 3u));
#undef KIVI_PAIR
}

// Scaling exponent for operands bounded by a finite P >= 0: with
// P = m 2^x, m in [1/2, 1) (frexp, subnormals included), P * 2^(14 - x) lies
// in [2^13, 2^14), so that hi and lo stay finite f16 values with the most
// bits kept (P = 0 gives 14, and every operand is 0).
__device__ __forceinline__ int op_exp(float P) {
    return 14 - __builtin_amdgcn_frexp_expf(P);
}

// x = hi + lo with hi = RN16(x) and lo = RN16(x - hi), for two values at
// once as packed pairs (x0 in the low halves): one paired conversion for the
// two hi parts and one for the two lo parts.
__device__ __forceinline__ void split16x2(float x0, float x1, uint32_t& hi,
                                          uint32_t& lo) {
    const h2x_t h = {(_Float16)x0, (_Float16)x1};
    hi = __builtin_bit_cast(uint32_t, h);
    // the hi parts widened back from the packed pair
    const float h0 = (float)__builtin_bit_cast(_Float16, (uint16_t)hi);
    const float h1 = (float)__builtin_bit_cast(_Float16, (uint16_t)(hi >> 16));
    const h2x_t l = {(_Float16)(x0 - h0), (_Float16)(x1 - h1)};
    lo = __builtin_bit_cast(uint32_t, l);
}

// B column of this lane (m16 = lane % 16): head m16's hi parts in columns
// [0, NQ), its lo parts in [8, 8 + NQ); the other columns of C are never
// used, so their lanes read column 0's operands (the same addresses as the
// lanes of column 0).
template <int NQ>
__device__ __forceinline__ int b_col(int m16) {
    return m16 < NQ ? m16 : (m16 >= 8 && m16 < 8 + NQ ? NQ + m16 - 8 : 0);
}


// Lane permutations inside rows of 16 lanes (DPP) and across the halves of
// 32 lanes (an LDS-unit swizzle that touches no memory), for reductions
// over aligned blocks of lanes.
template <int CTRL>
__device__ __forceinline__ uint32_t dpp_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xF, 0xF, true);
}
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xF, 0xF, true));
}
__device__ __forceinline__ float xor16_f(float v) {   // lane l reads lane l ^ 16
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401F));
}
__device__ __forceinline__ uint32_t xor16_u(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x401F);
}

// Sum over aligned blocks of N lanes (N a power of two <= 32); every lane of
// a block receives the same value (each step adds a pair in both orders).
// quad_perm [1,0,3,2], quad_perm [2,3,0,1], row_half_mirror, row_mirror,
// then lane ^ 16.
template <int N>
__device__ __forceinline__ float block_sum(float v) {
    if constexpr (N > 1) v += dpp_f<0xB1>(v);
    if constexpr (N > 2) v += dpp_f<0x4E>(v);
    if constexpr (N > 4) v += dpp_f<0x141>(v);
    if constexpr (N > 8) v += dpp_f<0x140>(v);
    if constexpr (N > 16) v += xor16_f(v);
    return v;
}
// Maximum of non-negative floats over aligned blocks of N lanes, on their
// bit patterns (which order like the values).
template <int N>
__device__ __forceinline__ float block_max_nonneg(float x) {
    uint32_t v = __float_as_uint(x);
    if constexpr (N > 1) v = max(v, dpp_u<0xB1>(v));
    if constexpr (N > 2) v = max(v, dpp_u<0x4E>(v));
    if constexpr (N > 4) v = max(v, dpp_u<0x141>(v));
    if constexpr (N > 8) v = max(v, dpp_u<0x140>(v));
    if constexpr (N > 16) v = max(v, xor16_u(v));
    return __uint_as_float(v);
}

// x plus the value of the lane 8 up in its row of 16 (lane l + 8 for
// l % 16 < 8): a head's hi-part sum and its lo-part sum.
__device__ __forceinline__ float add_lo_half(float x) {
    return x + dpp_f<0x128>(x);   // row_ror:8
}

// One 16x16x32 product of 16-bit operands of the cache's type.
template <int DT>
__device__ __forceinline__ f4_t mfma16(uint4 A, uint4 B, f4_t C) {
    if constexpr (DT == DT_F16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, A),
                                                      __builtin_bit_cast(h8_t, B), C, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, A),
                                                       __builtin_bit_cast(b8_t, B), C, 0, 0, 0);
}

template <int DT>
__device__ __forceinline__ float widen_h(uint16_t h) {
    if constexpr (DT == DT_F16)
        return (float)__builtin_bit_cast(_Float16, h);
    else
        return __uint_as_float((uint32_t)h << 16);
}

}  // namespace

// One 128-thread block (two waves) per (chunk, bh).  The chunk's scores go
// through the matrix cores, its quantized tokens' values too (Q is
// G_k-aligned, so a 16-token tile is all quantized or all exact); the ring's
// exact values are summed on the vector units.  The caller
// guarantees D in {64, 128}, BITS <= 4, G_k in {16, 32}, a value group of
// 16 * 2^k channels and n_q <= NQ.
//
// B operands live in LDS, each lane's operands of one group contiguous:
// keys [g][kb][column][k-step], values [gv][kb][column][k-step] (uint4 = 8
// halves each; columns: the heads' hi parts, then their lo parts).  A wave
// loads one group's operands into registers and uses them for every tile
// of that group: its tiles are taken group by group (tiles 2w, 2w + 1,
// 2w + 4, 2w + 5 of wave w).
template <int DT, int BITS, int D, int NQ, int GK>
__global__ __launch_bounds__(kMChunk, (MfmaShape<BITS, D, NQ, GK>::kMinBlocks))
void attend_mfma_kernel(AttendArgs a, int chunk_top) {
    using Sh = MfmaShape<BITS, D, NQ, GK>;
    constexpr int D8 = Sh::D8, KS = Sh::KS, CPL = Sh::CPL, LB = Sh::LB;
    constexpr int DW = Sh::DW, MT = Sh::MT, MAXGV = Sh::MAXGV, VKS = Sh::VKS;
    constexpr int kMaxKGroups = Sh::KGROUPS;
    constexpr int kOps = Sh::kOps, KH = Sh::KH;
    static_assert(NQ * MAXGV * kMChunk <= kOps * 4, "zero-point rows fit");

    // the query, 16-bit patterns of the cache's type
    __shared__ __attribute__((aligned(16))) uint4 ops_s[kOps];
    // scores, then weights, per head (rows padded: the heads' lanes of a
    // matrix-core tile write their rows at once)
    __shared__ __attribute__((aligned(16))) float p_s[NQ][Sh::kPRow];
    // value codes by token pair: row q holds, for each pair of tokens
    // (2P, 2P + 1), the q-th 16 bits of each token's code row, the even
    // token's in the low half (rows padded to 68 dwords, which keeps the
    // two writers of a pair off one bank)
    constexpr int kVpStride = Sh::kVpStride;
    // The query (16-bit patterns of the cache's type) and each key group's
    // bias and scaling exponent are last read by the scores; the value codes
    // are first written after them.  One region holds both.
    union EarlyLate {
        struct {
            uint16_t q[NQ][D];
            float kbias[kMaxKGroups][NQ];
            int kexp[kMaxKGroups][NQ];
        } early;
        uint32_t vp[2 * DW][kVpStride];
    };
    __shared__ __attribute__((aligned(16))) EarlyLate el_s;
    auto& q_s = el_s.early.q;
    auto& kbias_s = el_s.early.kbias;
    auto& kexp_s = el_s.early.kexp;
    auto& vp_s = el_s.vp;
    // the largest value scale of each value group, per half wave
    __shared__ float vmx_s[MAXGV][4];
    __shared__ int vexp_s[MAXGV];          // scaling exponent of each value group
    __shared__ float ml_s[2][NQ];
    // the partial score maxima (per wave and lane block) are read before
    // the sums of p * zero per value group are written
    union MaxZero {
        float mxp[NQ][8];
        float zsum[NQ * MAXGV];
    };
    __shared__ __attribute__((aligned(16))) MaxZero mz_s;
    auto& mxp_s = mz_s.mxp;
    auto& zsum_s = mz_s.zsum;

    // Blocks run the chunks from the last one down (grid x = bh, y = chunk
    // counted down from chunk_top), every bh of a chunk before the next
    // chunk: the chunks that hold the ring's exact tokens, which take
    // longest, start first instead of closing the grid.
    const int bh = (int)blockIdx.x;
    const int chunk = chunk_top - (int)blockIdx.y;
    const int tid = threadIdx.x;
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

    // ---- the loads the key side needs, issued up front ----
    uint16_t qv[NQ];                           // query element d = tid
#pragma unroll
    for (int j = 0; j < NQ; ++j)
        qv[j] = (tid < D && j < nq) ? a.q[((int64_t)bh * nq + j) * D + tid] : (uint16_t)0;
    // key params of this thread's half-items: half-item h = tid + 128 r is
    // 4 channels (c4) of key group h / (2 D8), the group's half-items in
    // consecutive lanes
    float ksc[KH][4], kzr[KH][4];
#pragma unroll
    for (int r = 0; r < KH; ++r) {
        const int h = tid + kMChunk * r;
        const int kg = h / (2 * D8), c4 = h % (2 * D8);
        float4 s0 = make_float4(0.f, 0.f, 0.f, 0.f), z0 = s0;
        if (h < ngk * D8 * 2) {
            const int64_t p = ((int64_t)bh * a.NG + g0 + kg) * D + c4 * 4;
            s0 = *reinterpret_cast<const float4*>(a.k_scale + p);
            z0 = *reinterpret_cast<const float4*>(a.k_zero + p);
        }
        ksc[r][0] = s0.x; ksc[r][1] = s0.y; ksc[r][2] = s0.z; ksc[r][3] = s0.w;
        kzr[r][0] = z0.x; kzr[r][1] = z0.y; kzr[r][2] = z0.z; kzr[r][3] = z0.w;
    }
    // this lane's key code blocks of its four 16-token tiles
    constexpr int LBW = LB >= 4 ? LB / 4 : 1;
    uint32_t kw[4][LBW];
#pragma unroll
    for (int tt = 0; tt < 4; ++tt) {
        const int tok0 = ((tt >> 1) * 4 + 2 * wave + (tt & 1)) * 16;
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
    // queries and the zero block into LDS
#pragma unroll
    for (int j = 0; j < NQ; ++j)
        if (tid < D) q_s[j][tid] = qv[j];
    __syncthreads();

    // ---- key operands: q[j][d] scale[g][d] 2^e(g, j) as hi + lo and the
    // zero bias, on both waves.  Thread = half-item (g, 4 channels) for
    // every head; the 2 D8 half-items of a group sit in consecutive lanes
    // (all of them, or none), where each head's maximum (for e) and bias sum
    // meet in xor shuffles. ----
#pragma unroll
    for (int r = 0; r < KH; ++r) {
        const int h = tid + kMChunk * r;
        if (h >= ngk * D8 * 2) continue;
        const int kg = h / (2 * D8), c4 = h % (2 * D8);
        const int d = c4 * 4, blk = d / CPL, s = (d % CPL) / 8, half = (d % 8) / 4;
#pragma unroll
        for (int j = 0; j < NQ; ++j) {
            float pr[4], b = 0.0f, mxl = 0.0f;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float qd = widen_h<DT>(q_s[j][d + i]);
                pr[i] = qd * ksc[r][i];
                mxl = fmaxf(mxl, fabsf(pr[i]));
                b = __builtin_fmaf(qd, kzr[r][i], b);
            }
            b = block_sum<2 * D8>(b);
            mxl = block_max_nonneg<2 * D8>(mxl);
            const int e = op_exp(mxl);
            uint32_t h0, h1, l0, l1;
            split16x2(__builtin_ldexpf(pr[0], e), __builtin_ldexpf(pr[1], e), h0, l0);
            split16x2(__builtin_ldexpf(pr[2], e), __builtin_ldexpf(pr[3], e), h1, l1);
            uint2* hb = reinterpret_cast<uint2*>(
                ops_s + (((kg * 4 + blk) * 2 * NQ + j) * KS + s)) + half;
            uint2* lb = reinterpret_cast<uint2*>(
                ops_s + (((kg * 4 + blk) * 2 * NQ + NQ + j) * KS + s)) + half;
            *hb = make_uint2(h0, h1);
            *lb = make_uint2(l0, l1);
            if (c4 == 0) {
                kbias_s[kg][j] = b;
                kexp_s[kg][j] = e;
            }
        }
    }
    // This thread's token: value code row and value params.  Issued only
    // now, once the key side's data has arrived: when every resident block
    // asks for all its bytes at once, the key side's share arrives no sooner
    // than the rest, and the key operands and the scores then wait longer.
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

    __syncthreads();

    // ---- scores on the matrix cores: wave w takes 16-token tiles 2w,
    // 2w + 1, 2w + 4, 2w + 5 (two whole key groups of 32 tokens), with the
    // B operands of a group loaded once.  Tiles of the ring's exact tokens
    // (Q is a multiple of 16, so a tile is all quantized or all exact) take
    // the keys themselves as A and the 16-bit query as B, both exact in the
    // cache's type: their scores need no split, no scaling and no bias.
    // Scores go to LDS already times sm_scale; each lane keeps the largest
    // of its valid ones, one partial max per head, wave and lane block.
    float lmx = -__builtin_huge_valf();
    {
        const int col = b_col<NQ>(m16);
        int gcur = -1;
        uint4 bk[KS];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int tok0 = ((tt >> 1) * 4 + 2 * wave + (tt & 1)) * 16;
            if (tok0 >= nq_tok) continue;          // wave-uniform
            const int g = tok0 >> gk_sh;
            if (g != gcur) {                       // wave-uniform
                const uint4* bp = ops_s + ((g * 4 + kb) * 2 * NQ + col) * KS;
#pragma unroll
                for (int s = 0; s < KS; ++s) bk[s] = bp[s];
                gcur = g;
            }
            f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
            if constexpr (BITS == 2) {
#pragma unroll
                for (int s = 0; s < KS; s += 2) {         // a code dword per two k-steps
                    h8_t A0, A1;
                    codes16_2bit(kw[tt][s / 2], A0, A1);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A0, __builtin_bit_cast(h8_t, bk[s]), acc, 0, 0, 0);
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        A1, __builtin_bit_cast(h8_t, bk[s + 1]), acc, 0, 0, 0);
                }
            } else {
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    constexpr int SB = 8 * BITS;            // bits per k-step
                    const int bit = s * SB;
                    uint32_t bits = kw[tt][bit / 32] >> (bit % 32);
                    if constexpr (SB < 32) bits &= (1u << SB) - 1u;
                    acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                        codes8<BITS>(bits), __builtin_bit_cast(h8_t, bk[s]), acc, 0, 0, 0);
                }
            }
            float sc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) sc[i] = add_lo_half(acc[i]);
            if (m16 < NQ) {
                const int e = kexp_s[g][m16];
                const float bias = kbias_s[g][m16];
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = (__builtin_ldexpf(sc[i], kCodeExp - e) + bias) * a.sm_scale;
                    p_s[m16][tok0 + kb * 4 + i] = x;
                    lmx = fmaxf(lmx, x);
                }
            }
        }
    }
    if (nq_tok < nt) {                             // block-uniform: ring tiles
        bool have_q = false;
        uint4 bq[KS];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
            const int tok0 = ((tt >> 1) * 4 + 2 * wave + (tt & 1)) * 16;
            if (tok0 < nq_tok || tok0 >= nt) continue;   // wave-uniform
            if (!have_q) {
                // B = the query of head m16 (zeros in the other columns)
#pragma unroll
                for (int s = 0; s < KS; ++s) {
                    const int d0 = kb * CPL + s * 8;
                    bq[s] = m16 < NQ ? *reinterpret_cast<const uint4*>(&q_s[m16][d0])
                                     : make_uint4(0u, 0u, 0u, 0u);
                }
                have_q = true;
            }
            // A = the keys of tokens tok0 + m16, channels of lane block kb
            // (a row past T holds another ring token; its score is never read)
            const uint16_t* krow = a.k_ring +
                ((int64_t)bh * a.ring + (t0 + tok0 + m16) % a.ring) * D + kb * CPL;
            f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < KS; ++s)
                acc = mfma16<DT>(*reinterpret_cast<const uint4*>(krow + s * 8), bq[s], acc);
            if (m16 < NQ) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float x = acc[i] * a.sm_scale;
                    p_s[m16][tok0 + kb * 4 + i] = x;
                    if (tok0 + kb * 4 + i < nt) lmx = fmaxf(lmx, x);
                }
            }
        }
    }
    if (m16 < NQ) mxp_s[m16][wave * 4 + kb] = lmx;
    __syncthreads();

    // ---- softmax partial of the chunk: a thread per head takes the max of
    // the eight partial maxima, then every thread takes its token's p, then
    // eight lanes per row sum.
    // Eight lanes read a 128-token row as four 16-byte pieces each: lane i
    // takes tokens 4i .. 4i + 3 of each block of 32, the blocks in an order
    // rotated by one on odd rows, so that the two rows of a 16-lane LDS pass
    // sit in different banks (rows are 512 bytes apart).
    const int i8 = tid & 7;
    auto row4 = [&](const float* row, int k, int m) {
        return *reinterpret_cast<const float4*>(
            row + ((4 * i8 + 32 * (m + (k & 1))) & (kMChunk - 1)));
    };
    if (tid < NQ) {
        const float4 x = *reinterpret_cast<const float4*>(&mxp_s[tid][0]);
        const float4 y = *reinterpret_cast<const float4*>(&mxp_s[tid][4]);
        ml_s[0][tid] = fmaxf(fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)),
                             fmaxf(fmaxf(y.x, y.y), fmaxf(y.z, y.w)));
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
            const uint32_t other = dpp_u<0xB1>(even ? hi_w : lo_w);   // lane ^ 1
            row[(2 * k) * kVpStride] = __builtin_amdgcn_perm(other, mine, sel_lo);
            row[(2 * k + 1) * kVpStride] = __builtin_amdgcn_perm(other, mine, sel_hi);
        }
    }
#pragma unroll
    for (int gv = 0; gv < MAXGV; ++gv) {
        if (gv < ngd) {                        // block-uniform
            const float m = block_max_nonneg<32>(svv[gv]);
            if ((tid & 31) == 0) vmx_s[gv][tid >> 5] = m;
        }
    }
    __syncthreads();
    float pt[NQ];                              // this token's p per head
#pragma unroll
    for (int j = 0; j < NQ; ++j)
        pt[j] = tid < nt ? __expf(p_s[j][tid] - ml_s[0][j]) : 0.0f;
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
    // in registers (they go to the score rows once the reductions below have
    // read those).  The chunk's ring tokens are fewer
    // than the ring's slots (T - Q < R + G_k <= ring), so their slots follow
    // the first one with at most one wrap.  Sixteen tokens' loads are in
    // flight at a time, the next sixteen issued before this batch's sums.
    const bool has_ring = nq_tok < nt;        // block-uniform
    float o[NQ];
#pragma unroll
    for (int j = 0; j < NQ; ++j) o[j] = 0.0f;
    if (has_ring && tid < D) {
        const uint16_t* vcol = a.v_ring + (int64_t)bh * a.ring * D + tid;
        const int slot0 = (t0 + nq_tok) % a.ring;
        const int n_ring = nt - nq_tok;
        uint16_t v[16], vn[16] = {};
        auto load16 = [&](uint16_t* dst, int base) {
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                int sl = slot0 + min(base + u, n_ring - 1);
                if (sl >= a.ring) sl -= a.ring;
                dst[u] = vcol[(int64_t)sl * D];
            }
        };
        load16(v, 0);
        for (int tb = 0; tb < n_ring; tb += 16) {
            if (tb + 16 < n_ring) load16(vn, tb + 16);
#pragma unroll
            for (int u = 0; u < 16; ++u) {
                if (tb + u < n_ring) {
                    const float x = widen_h<DT>(v[u]);
#pragma unroll
                    for (int j = 0; j < NQ; ++j)
                        o[j] = __builtin_fmaf(p_s[j][nq_tok + tb + u], x, o[j]);
                }
            }
#pragma unroll
            for (int u = 0; u < 16; ++u) v[u] = vn[u];
        }
    }
    // eight lanes per row (read as above): the sums of p (per head) and of
    // p * zero; and each value group's scaling exponent from the largest
    // scale of its four half waves (non-negative)
    const int n_sum = NQ + NQ * ngd;
    for (int k = tid >> 3; k < n_sum; k += kMChunk / 8) {
        const float* row = k < NQ ? p_s[k] : zrows + (k - NQ) * kMChunk;
        float4 x[4];
#pragma unroll
        for (int m = 0; m < 4; ++m) x[m] = row4(row, k, m);
        float v = 0.0f;
#pragma unroll
        for (int m = 0; m < 4; ++m) v = ((v + x[m].x) + x[m].y) + (x[m].z + x[m].w);
        v = block_sum<8>(v);
        if (i8 == 0) {
            if (k < NQ) ml_s[1][k] = v;
            else zsum_s[k - NQ] = v;
        }
    }
    if (tid < ngd)
        vexp_s[tid] = op_exp(fmaxf(fmaxf(vmx_s[tid][0], vmx_s[tid][1]),
                                   fmaxf(vmx_s[tid][2], vmx_s[tid][3])));
    __syncthreads();
    // the ring values' sums (zeros without ring tokens) into the score rows
    // (free now, and read only after the barrier below)
    if (tid < D) {
#pragma unroll
        for (int j = 0; j < NQ; ++j) p_s[j][tid] = o[j];
    }
    // weights p * vscale * 2^e(gv) of this token, hi + lo, at k index
    // (token) k-step tid / 32, lane block (tid % 32) / 8, element tid % 8
    {
        _Float16* vops = reinterpret_cast<_Float16*>(ops_s);
        const int s4 = tid >> 5, blk = (tid >> 3) & 3, i = tid & 7;
#pragma unroll
        for (int gv = 0; gv < MAXGV; ++gv) {
            if (gv >= ngd) break;              // block-uniform
            // this token's scale times 2^e (exact unless it falls below
            // fp32's normal range; e keeps it below 2^14)
            const float sv = __builtin_ldexpf(svv[gv], vexp_s[gv]);
            // heads in pairs: one paired conversion per pair for hi and lo
#pragma unroll
            for (int j = 0; j < NQ; j += 2) {
                const float w0 = pt[j] * sv;
                const float w1 = j + 1 < NQ ? pt[j + 1] * sv : 0.0f;
                uint32_t hi, lo;
                split16x2(w0, w1, hi, lo);
#pragma unroll
                for (int u = 0; u < 2; ++u) {
                    if (j + u < NQ) {
                        _Float16* vh = vops + (((gv * 4 + blk) * 2 * NQ + j + u) * VKS + s4) * 8;
                        _Float16* vl = vops + (((gv * 4 + blk) * 2 * NQ + NQ + j + u) * VKS + s4) * 8;
                        vh[i] = __builtin_bit_cast(_Float16, (uint16_t)(hi >> (16 * u)));
                        vl[i] = __builtin_bit_cast(_Float16, (uint16_t)(lo >> (16 * u)));
                    }
                }
            }
        }
    }
    __syncthreads();

    // ---- values on the matrix cores: wave w takes channel tiles 2w, 2w + 1,
    // 2w + 4, 2w + 5 (pairs of tiles in one value group when groups have 32
    // channels or more), with the B operands of a group loaded once
    float* wbase = a.work + ((int64_t)bh * a.n_chunks + chunk) * nq * att_slot(D);
    {
        const int col = b_col<NQ>(m16);
        int gcur = -1;
        uint4 bv[VKS];
#pragma unroll
        for (int u = 0; u < MT / 2; ++u) {
            const int mt = (u >> 1) * 4 + 2 * wave + (u & 1);
            const int gv = (mt * 16) >> gv_sh;
            if (gv != gcur) {                      // wave-uniform
                const uint4* bp = ops_s + ((gv * 4 + kb) * 2 * NQ + col) * VKS;
#pragma unroll
                for (int s4 = 0; s4 < VKS; ++s4) bv[s4] = bp[s4];
                gcur = gv;
            }
            const int ch = mt * 16 + m16;                   // this lane's A row
            const int q = (ch * BITS) / 16, sh = (ch * BITS) % 16;
            const uint32_t pmask = ((1u << BITS) - 1u) * 0x10001u;
            f4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s4 = 0; s4 < VKS; ++s4) {
                // tokens s4*32 + kb*8 + [0, 8) are pairs P0 .. P0 + 3, each dword
                // holding this channel's two codes sh bits up in its two halves
                const int P0 = s4 * 16 + kb * 4;
                const uint4 d = *reinterpret_cast<const uint4*>(&vp_s[q][P0]);
                const uint32_t dw[4] = {d.x, d.y, d.z, d.w};
                uint32_t pr[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) pr[k] = (dw[k] >> sh) & pmask;   // codes * 2^-24
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                    as_h8(pr[0], pr[1], pr[2], pr[3]), __builtin_bit_cast(h8_t, bv[s4]),
                    acc, 0, 0, 0);
            }
            float ov[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) ov[i] = add_lo_half(acc[i]);
            // C: lane (head m16, row block kb) holds channels mt*16 + 4 kb + i
            if (m16 < nq) {
                const int e = vexp_s[gv];
                const float zs = zsum_s[m16 * ngd + gv];
                const int c0 = mt * 16 + kb * 4;
                // plus the ring values' sums (zeros in a chunk without ring
                // tokens); four channels, one 16-byte store
                const float4 rv = *reinterpret_cast<const float4*>(&p_s[m16][c0]);
                float4 r;
                r.x = __builtin_ldexpf(ov[0], kCodeExp - e) + zs + rv.x;
                r.y = __builtin_ldexpf(ov[1], kCodeExp - e) + zs + rv.y;
                r.z = __builtin_ldexpf(ov[2], kCodeExp - e) + zs + rv.z;
                r.w = __builtin_ldexpf(ov[3], kCodeExp - e) + zs + rv.w;
                *reinterpret_cast<float4*>(wbase + m16 * att_slot(D) + kAttData + c0) = r;
            }
        }
    }
    if (tid < nq) {
        wbase[tid * att_slot(D)] = ml_s[0][tid];
        wbase[tid * att_slot(D) + 1] = ml_s[1][tid];
    }
}

template <int DT, int BITS, int D, int NQ>
static hipError_t launch_mfma_t(const AttendArgs& a, int64_t BH, int n_full,
                                hipStream_t stream) {
    // one block per (chunk, bh), the chunks from n_full - 1 down, at most
    // 65535 chunks (the grid's y limit) per launch
    constexpr int kMaxY = 65535;
    for (int top = n_full - 1; top >= 0; top -= kMaxY) {
        const dim3 grid((uint32_t)BH, (uint32_t)std::min(top + 1, kMaxY)), block(kMChunk);
        const hipError_t e =
            a.G_k == 32 && a.G_v >= 32
                ? launch_kernel((attend_mfma_kernel<DT, BITS, D, NQ, 32>), grid, block, 0,
                                stream, a, top)
                : launch_kernel((attend_mfma_kernel<DT, BITS, D, NQ, 16>), grid, block, 0,
                                stream, a, top);
        if (e != hipSuccess) return e;
    }
    return hipSuccess;
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
