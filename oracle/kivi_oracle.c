/*
 * KIVI reference oracle (TEST INFRASTRUCTURE ONLY; see kivi_oracle.h).
 *
 * Plain loops in the order the VeloxQuant-MLX pages state the method.  No
 * blocking, no fusion, no vectorisation: every quantity is computed by the
 * obvious loop so a reader can check it against the pages by eye.
 *
 * Build: gcc -std=c11 -O2 -ffp-contract=off (no -ffast-math, no -march).
 * On x86-64 every float operation below is one SSE binary32 operation,
 * rounded to nearest even.
 */
#include "kivi_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}

static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* ------------------------------------------------------------------------ */
/* 16-bit formats.  IEEE-754 binary16: 1 sign, 5 exponent (bias 15), 10      */
/* fraction bits.  bfloat16: the top half of a binary32.                    */
/* ------------------------------------------------------------------------ */

float kivi_ref_half_to_float(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1f;
    int m = h & 0x3ff;
    float v;
    if (e == 0) {
        v = ldexpf((float)m, -24); /* subnormal: m * 2^-24, exact */
    } else if (e == 31) {
        v = (m == 0) ? INFINITY : NAN;
    } else {
        v = ldexpf((float)(1024 + m), e - 25); /* (1 + m/1024) * 2^(e-15) */
    }
    return sign ? -v : v;
}

uint16_t kivi_ref_float_to_half(float f) {
    uint32_t u = f32_bits(f);
    uint16_t sign = (uint16_t)((u >> 16) & 0x8000u);
    uint32_t a = u & 0x7fffffffu;
    if (a > 0x7f800000u) return (uint16_t)(sign | 0x7e00u); /* NaN */
    /* 65520 is the midpoint between 65504 (odd fraction) and 2^16: ties go
       to the even side, which overflows to infinity. */
    if (a >= 0x477ff000u) return (uint16_t)(sign | 0x7c00u);
    if (a >= 0x38800000u) { /* result is a normal binary16 (>= 2^-14) */
        uint32_t e16 = (a >> 23) - 127u + 15u;
        uint32_t mant = a & 0x7fffffu;
        uint32_t h = (e16 << 10) | (mant >> 13);
        uint32_t rem = mant & 0x1fffu; /* the 13 dropped bits */
        if (rem > 0x1000u || (rem == 0x1000u && (h & 1u))) h += 1u;
        return (uint16_t)(sign | h);
    }
    /* Subnormal or zero result: round a / 2^-24 to an integer, ties even. */
    if (a <= 0x33000000u) return sign; /* <= 2^-25: rounds to 0 */
    {
        uint32_t E = a >> 23; /* biased exponent, 102..112 here */
        uint32_t M = (a & 0x7fffffu) | 0x800000u;
        uint32_t shift = 126u - E; /* value / 2^-24 = M * 2^-shift */
        uint32_t q = M >> shift;
        uint32_t rem = M & ((1u << shift) - 1u);
        uint32_t half = 1u << (shift - 1u);
        if (rem > half || (rem == half && (q & 1u))) q += 1u;
        return (uint16_t)(sign | q);
    }
}

float kivi_ref_bf16_to_float(uint16_t h) { return bits_f32((uint32_t)h << 16); }

uint16_t kivi_ref_float_to_bf16(float f) {
    uint32_t u = f32_bits(f);
    if ((u & 0x7fffffffu) > 0x7f800000u)
        return (uint16_t)(((u >> 16) & 0x8000u) | 0x7fc0u); /* NaN */
    /* round to nearest even on the low 16 bits */
    uint32_t r = u + 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(r >> 16);
}

static float widen(uint16_t h, int dtype) {
    return dtype == 0 ? kivi_ref_half_to_float(h) : kivi_ref_bf16_to_float(h);
}

static uint16_t narrow(float f, int dtype) {
    return dtype == 0 ? kivi_ref_float_to_half(f) : kivi_ref_float_to_bf16(f);
}

int kivi_ref_widen_array(const uint16_t* in, int64_t n, int dtype, float* out) {
    if (n < 0 || (dtype != 0 && dtype != 1)) return 1;
    for (int64_t i = 0; i < n; ++i) out[i] = widen(in[i], dtype);
    return 0;
}

int kivi_ref_narrow_array(const float* in, int64_t n, int dtype, uint16_t* out) {
    if (n < 0 || (dtype != 0 && dtype != 1)) return 1;
    for (int64_t i = 0; i < n; ++i) out[i] = narrow(in[i], dtype);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* The quantizer on one group.                                              */
/* ------------------------------------------------------------------------ */

static int bits_ok(int bits) {
    return bits == 1 || bits == 2 || bits == 4 || bits == 8;
}

/*
 * KIVI blog post on the fused Metal kernels, section "What we're actually
 * optimizing": zero = min(group); scale = (max(group) - min(group)) /
 * (2^bits - 1).  Min and max are a sequential scan in fp32 as the pages'
 * kernels keep them (sections "Kernel A" and "Kernel B").  A min or max that
 * compares equal to zero is stored as +0 (reading: the pages are silent on
 * signed zero; this makes the result independent of scan order).
 */
int kivi_ref_group_params(const float* vals, int64_t n, int bits, float* scale,
                          float* zero) {
    if (n <= 0 || !bits_ok(bits)) return 1;
    float mn = vals[0];
    float mx = vals[0];
    for (int64_t i = 1; i < n; ++i) {
        if (vals[i] < mn) mn = vals[i];
        if (vals[i] > mx) mx = vals[i];
    }
    if (mn == 0.0f) mn = 0.0f;
    if (mx == 0.0f) mx = 0.0f;
    float range = mx - mn;
    float levels = (float)((1 << bits) - 1);
    *zero = mn;
    *scale = range / levels;
    return 0;
}

/*
 * Same section and the 0.8.0 release post, section "What KIVI is":
 * q = round((x - zero) / scale), an unsigned code in [0, 2^bits - 1].  The
 * op order is the MLX chain the post lists: subtract, divide, round, clip.
 * Rounding is half-to-even (section "Three ways to be off by one bit",
 * item 2).  Reading for the silent case scale == 0 (a constant group): code 0.
 * The clip is max-then-min with IEEE maxNum/minNum, so a NaN quotient (only
 * possible when a group's range overflows binary32) gives code 0.
 */
int kivi_ref_code(float f, float scale, float zero, int bits) {
    float maxc = (float)((1 << bits) - 1);
    if (scale == 0.0f) return 0;
    float a = f - zero;
    float t = a / scale;
    float r = rintf(t);
    r = fmaxf(r, 0.0f);
    r = fminf(r, maxc);
    return (int)r;
}

/*
 * Section "What we're actually optimizing": recon = q * scale + zero, and
 * section "Three ways to be off by one bit", item 1: the product is rounded
 * before the add (two roundings, never a fused multiply-add).
 */
float kivi_ref_recon(int code, float scale, float zero) {
    float p = (float)code * scale;
    float r = p + zero;
    return r;
}

/* ------------------------------------------------------------------------ */
/* Whole tensors.  Layout: section "The layout problem that shapes          */
/* everything": [BH, S, D] row-major.                                       */
/* ------------------------------------------------------------------------ */

static int shape_ok(int64_t BH, int64_t S, int64_t D, int bits, int64_t group) {
    if (BH < 0 || S < 0 || D < 0) return 0;
    if (!bits_ok(bits)) return 0;
    if (group < 1) return 0;
    if ((D * bits) % 8 != 0) return 0;
    return 1;
}

/*
 * Keys, per channel (section "Kernel A — per-channel keys"): for every
 * (bh, token group g, channel d) the group is tokens
 * s in [g*G, min(g*G + G, S)) of channel d.  Params are stored [BH, NG, D].
 * A ragged last group is taken over its real tokens only; the pages pad it
 * with copies of its last element (section "Three ways to be off by one bit",
 * item 3), which cannot change a min or a max.
 */
int kivi_ref_quant_keys_unpacked(const uint16_t* x, int dtype, int64_t BH,
                                 int64_t S, int64_t D, int bits, int64_t group,
                                 uint8_t* codes, float* scale, float* zero) {
    if (!shape_ok(BH, S, D, bits, group) || (dtype != 0 && dtype != 1)) return 1;
    int64_t NG = (S + group - 1) / group;
    float* vals = (float*)malloc((size_t)(group > 0 ? group : 1) * sizeof(float));
    if (!vals) return 1;
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t g = 0; g < NG; ++g) {
            int64_t s0 = g * group;
            int64_t s1 = s0 + group < S ? s0 + group : S;
            for (int64_t d = 0; d < D; ++d) {
                for (int64_t s = s0; s < s1; ++s)
                    vals[s - s0] = widen(x[(bh * S + s) * D + d], dtype);
                float sc, z;
                kivi_ref_group_params(vals, s1 - s0, bits, &sc, &z);
                scale[(bh * NG + g) * D + d] = sc;
                zero[(bh * NG + g) * D + d] = z;
                for (int64_t s = s0; s < s1; ++s)
                    codes[(bh * S + s) * D + d] =
                        (uint8_t)kivi_ref_code(vals[s - s0], sc, z, bits);
            }
        }
    }
    free(vals);
    return 0;
}

/*
 * Values, per token (section "Kernel B — per-token values"): for every
 * (bh, token s, channel group j) the group is channels
 * d in [j*G, min(j*G + G, D)) of token s.  Params are stored [BH, S, NGD].
 */
int kivi_ref_quant_values_unpacked(const uint16_t* x, int dtype, int64_t BH,
                                   int64_t S, int64_t D, int bits,
                                   int64_t group, uint8_t* codes, float* scale,
                                   float* zero) {
    if (!shape_ok(BH, S, D, bits, group) || (dtype != 0 && dtype != 1)) return 1;
    int64_t NGD = (D + group - 1) / group;
    float* vals = (float*)malloc((size_t)(group > 0 ? group : 1) * sizeof(float));
    if (!vals) return 1;
    for (int64_t bh = 0; bh < BH; ++bh) {
        for (int64_t s = 0; s < S; ++s) {
            for (int64_t j = 0; j < NGD; ++j) {
                int64_t d0 = j * group;
                int64_t d1 = d0 + group < D ? d0 + group : D;
                for (int64_t d = d0; d < d1; ++d)
                    vals[d - d0] = widen(x[(bh * S + s) * D + d], dtype);
                float sc, z;
                kivi_ref_group_params(vals, d1 - d0, bits, &sc, &z);
                scale[(bh * S + s) * NGD + j] = sc;
                zero[(bh * S + s) * NGD + j] = z;
                for (int64_t d = d0; d < d1; ++d)
                    codes[(bh * S + s) * D + d] =
                        (uint8_t)kivi_ref_code(vals[d - d0], sc, z, bits);
            }
        }
    }
    free(vals);
    return 0;
}

/*
 * Packing (TurboQuant Metal kernels post, section "Kernel 1: Bit-Packing";
 * TurboQuant port overview, section "The Bit-Packing Problem"): 8/bits codes
 * per byte, code i of a byte in bits [i*bits, (i+1)*bits).  Applied along D
 * for every row (bh, s); a row holds D*bits/8 bytes.
 */
int kivi_ref_pack(const uint8_t* codes, int64_t rows, int64_t D, int bits,
                  uint8_t* packed) {
    if (!bits_ok(bits) || rows < 0 || D < 0 || (D * bits) % 8 != 0) return 1;
    int64_t per = 8 / bits;
    int64_t row_bytes = D * bits / 8;
    uint32_t mask = (1u << bits) - 1u;
    for (int64_t r = 0; r < rows; ++r) {
        for (int64_t b = 0; b < row_bytes; ++b) {
            uint32_t byte = 0;
            for (int64_t i = 0; i < per; ++i) {
                uint32_t c = codes[r * D + b * per + i] & mask;
                byte |= c << (i * bits);
            }
            packed[r * row_bytes + b] = (uint8_t)byte;
        }
    }
    return 0;
}

int kivi_ref_unpack(const uint8_t* packed, int64_t rows, int64_t D, int bits,
                    uint8_t* codes) {
    if (!bits_ok(bits) || rows < 0 || D < 0 || (D * bits) % 8 != 0) return 1;
    int64_t per = 8 / bits;
    int64_t row_bytes = D * bits / 8;
    uint32_t mask = (1u << bits) - 1u;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t d = 0; d < D; ++d) {
            uint32_t byte = packed[r * row_bytes + d / per];
            codes[r * D + d] = (uint8_t)((byte >> ((d % per) * bits)) & mask);
        }
    return 0;
}

int kivi_ref_quant_keys(const uint16_t* x, int dtype, int64_t BH, int64_t S,
                        int64_t D, int bits, int64_t group, uint8_t* packed,
                        float* scale, float* zero) {
    if (!shape_ok(BH, S, D, bits, group)) return 1;
    size_t n = (size_t)(BH * S * D);
    uint8_t* codes = (uint8_t*)malloc(n ? n : 1);
    if (!codes) return 1;
    int st = kivi_ref_quant_keys_unpacked(x, dtype, BH, S, D, bits, group,
                                          codes, scale, zero);
    if (st == 0) st = kivi_ref_pack(codes, BH * S, D, bits, packed);
    free(codes);
    return st;
}

int kivi_ref_quant_values(const uint16_t* x, int dtype, int64_t BH, int64_t S,
                          int64_t D, int bits, int64_t group, uint8_t* packed,
                          float* scale, float* zero) {
    if (!shape_ok(BH, S, D, bits, group)) return 1;
    size_t n = (size_t)(BH * S * D);
    uint8_t* codes = (uint8_t*)malloc(n ? n : 1);
    if (!codes) return 1;
    int st = kivi_ref_quant_values_unpacked(x, dtype, BH, S, D, bits, group,
                                            codes, scale, zero);
    if (st == 0) st = kivi_ref_pack(codes, BH * S, D, bits, packed);
    free(codes);
    return st;
}

/* Dequantize: unpack, look up the element's group params, recon, narrow. */
int kivi_ref_dequant_keys(const uint8_t* packed, const float* scale,
                          const float* zero, int64_t BH, int64_t S, int64_t D,
                          int bits, int64_t group, int out_dtype,
                          uint16_t* out) {
    if (!shape_ok(BH, S, D, bits, group) || (out_dtype != 0 && out_dtype != 1))
        return 1;
    int64_t NG = (S + group - 1) / group;
    size_t n = (size_t)(BH * S * D);
    uint8_t* codes = (uint8_t*)malloc(n ? n : 1);
    if (!codes) return 1;
    kivi_ref_unpack(packed, BH * S, D, bits, codes);
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t d = 0; d < D; ++d) {
                int64_t p = (bh * NG + s / group) * D + d;
                float r = kivi_ref_recon(codes[(bh * S + s) * D + d], scale[p],
                                         zero[p]);
                out[(bh * S + s) * D + d] = narrow(r, out_dtype);
            }
    free(codes);
    return 0;
}

int kivi_ref_dequant_values(const uint8_t* packed, const float* scale,
                            const float* zero, int64_t BH, int64_t S,
                            int64_t D, int bits, int64_t group, int out_dtype,
                            uint16_t* out) {
    if (!shape_ok(BH, S, D, bits, group) || (out_dtype != 0 && out_dtype != 1))
        return 1;
    int64_t NGD = (D + group - 1) / group;
    size_t n = (size_t)(BH * S * D);
    uint8_t* codes = (uint8_t*)malloc(n ? n : 1);
    if (!codes) return 1;
    kivi_ref_unpack(packed, BH * S, D, bits, codes);
    for (int64_t bh = 0; bh < BH; ++bh)
        for (int64_t s = 0; s < S; ++s)
            for (int64_t d = 0; d < D; ++d) {
                int64_t p = (bh * S + s) * NGD + d / group;
                float r = kivi_ref_recon(codes[(bh * S + s) * D + d], scale[p],
                                         zero[p]);
                out[(bh * S + s) * D + d] = narrow(r, out_dtype);
            }
    free(codes);
    return 0;
}

/* One flush: the G_k oldest unquantized tokens [Q, Q + G_k) of every bh,
 * which form exactly one key group, go through the plain quantizers above,
 * writing straight into the compressed store at their own offsets. */
static int cache_flush_group(kivi_ref_cache* c) {
    const int64_t D = c->D, G = c->G_k, S = c->S_max;
    const int64_t row_bytes = D * c->bits / 8;
    const int64_t NG = (S + G - 1) / G;
    const int64_t NGD = (D + c->G_v - 1) / c->G_v;
    for (int64_t bh = 0; bh < c->BH; ++bh) {
        const int64_t row = bh * S + c->Q;
        int st = kivi_ref_quant_keys(c->k + row * D, c->dtype, 1, G, D,
                                     c->bits, G, c->k_codes + row * row_bytes,
                                     c->k_scale + (bh * NG + c->Q / G) * D,
                                     c->k_zero + (bh * NG + c->Q / G) * D);
        if (st == 0)
            st = kivi_ref_quant_values(c->v + row * D, c->dtype, 1, G, D,
                                       c->bits, c->G_v,
                                       c->v_codes + row * row_bytes,
                                       c->v_scale + row * NGD,
                                       c->v_zero + row * NGD);
        if (st != 0) return st;
    }
    c->Q += G;
    return 0;
}

int kivi_ref_cache_append(kivi_ref_cache* c, const uint16_t* k_new,
                          const uint16_t* v_new, int64_t n) {
    if (!c || n < 0 || c->R < 0 || c->G_k < 1 || c->G_v < 1 ||
        c->T < 0 || c->Q < 0 || c->Q > c->T ||
        !shape_ok(c->BH, c->S_max, c->D, c->bits, c->G_k) ||
        (c->dtype != 0 && c->dtype != 1) || n > c->S_max - c->T)
        return 1;
    if (n > 0 && (!k_new || !v_new)) return 1;
    const int64_t D = c->D;
    for (int64_t i = 0; i < n; ++i) {
        for (int64_t bh = 0; bh < c->BH; ++bh) {
            memcpy(c->k + (bh * c->S_max + c->T) * D, k_new + (bh * n + i) * D,
                   (size_t)D * sizeof(uint16_t));
            memcpy(c->v + (bh * c->S_max + c->T) * D, v_new + (bh * n + i) * D,
                   (size_t)D * sizeof(uint16_t));
        }
        c->T += 1;
        while (c->T - c->Q >= c->R + c->G_k) {
            int st = cache_flush_group(c);
            if (st != 0) return st;
        }
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* KIVI-Sink (VeloxQuant-MLX 0.24.1 package page, section "KVSink-adapted   */
/* sink protection"): per sequence, the n_sink token positions whose keys   */
/* have the largest L2 norm (averaged over the KV heads) are sinks.  Sinks  */
/* are kept in 16-bit floats and take no part in the min/max of their key   */
/* groups; every other token is quantized as plain KIVI.                    */
/* Tensors are [B*H, S, D] with the H heads of sequence b at rows           */
/* b*H .. b*H + H - 1; sink lists are [B, n_sink] token positions.          */
/* ------------------------------------------------------------------------ */

static int sink_shape_ok(int64_t B, int64_t H, int64_t S, int64_t D,
                         int64_t n_sink) {
    return B >= 0 && H >= 1 && S >= 0 && D >= 0 && n_sink >= 0 && n_sink <= S;
}

/*
 * Score of token s of sequence b: the mean over the H heads of the key's L2
 * norm.  Reading of the silent arithmetic: per head the squares are summed in
 * channel order with one rounding per step (ss = fma(x, x, ss)), the norm is
 * the correctly rounded square root, the H norms are summed in head order and
 * the sum is divided by H once.  (The square of a 16-bit float is exact in
 * fp32 unless a bf16 square underflows, so a separate multiply and add gives
 * the same sums.)
 */
int kivi_ref_sink_scores(const uint16_t* k, int dtype, int64_t B, int64_t H,
                         int64_t S, int64_t D, float* score) {
    if (!sink_shape_ok(B, H, S, D, 0) || (dtype != 0 && dtype != 1)) return 1;
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t s = 0; s < S; ++s) {
            float total = 0.0f;
            for (int64_t h = 0; h < H; ++h) {
                const uint16_t* row = k + ((b * H + h) * S + s) * D;
                float ss = 0.0f;
                for (int64_t d = 0; d < D; ++d) {
                    float x = widen(row[d], dtype);
                    ss = fmaf(x, x, ss);
                }
                total = total + sqrtf(ss);
            }
            score[b * S + s] = total / (float)H;
        }
    }
    return 0;
}

/*
 * The sinks of each sequence: the n_sink positions of highest score, taken
 * one at a time, highest first.  Reading where the pages are silent: of equal
 * scores the lower position is taken first.
 */
int kivi_ref_sink_select(const float* score, int64_t B, int64_t S,
                         int64_t n_sink, int32_t* idx) {
    if (!sink_shape_ok(B, 1, S, 0, n_sink)) return 1;
    unsigned char* taken = (unsigned char*)calloc((size_t)(S > 0 ? S : 1), 1);
    if (!taken) return 1;
    for (int64_t b = 0; b < B; ++b) {
        memset(taken, 0, (size_t)(S > 0 ? S : 1));
        for (int64_t r = 0; r < n_sink; ++r) {
            int64_t best = -1;
            for (int64_t s = 0; s < S; ++s) {
                if (taken[s]) continue;
                if (best < 0 || score[b * S + s] > score[b * S + best]) best = s;
            }
            taken[best] = 1;
            idx[b * n_sink + r] = (int32_t)best;
        }
    }
    free(taken);
    return 0;
}

/* Whether position s is one of the sinks of sequence b (positions outside
 * [0, S) in a list match nothing). */
static int is_sink(const int32_t* idx, int64_t n_sink, int64_t b, int64_t s) {
    for (int64_t i = 0; i < n_sink; ++i)
        if ((int64_t)idx[b * n_sink + i] == s) return 1;
    return 0;
}

/*
 * Keys with sinks: as kivi_ref_quant_keys_unpacked, except that a group's min
 * and max run over its tokens that are not sinks of the row's sequence
 * (b = bh / H), and a sink's code is 0 (the sink is kept in 16-bit form, so
 * it has no code).  Readings: a group made only of sinks has scale 0 and
 * zero 0; the per-token value groups need no change, since a value group
 * holds a single token and excluding a sink from calibration cannot touch
 * any other token.
 */
int kivi_ref_quant_keys_sink_unpacked(const uint16_t* x, int dtype, int64_t B,
                                      int64_t H, int64_t S, int64_t D,
                                      int bits, int64_t group,
                                      const int32_t* idx, int64_t n_sink,
                                      uint8_t* codes, float* scale,
                                      float* zero) {
    if (!sink_shape_ok(B, H, S, D, n_sink) ||
        !shape_ok(B * H, S, D, bits, group) || (dtype != 0 && dtype != 1))
        return 1;
    int64_t NG = (S + group - 1) / group;
    float* vals = (float*)malloc((size_t)group * sizeof(float));
    unsigned char* sink = (unsigned char*)malloc((size_t)group);
    if (!vals || !sink) {
        free(vals);
        free(sink);
        return 1;
    }
    for (int64_t bh = 0; bh < B * H; ++bh) {
        int64_t b = bh / H;
        for (int64_t g = 0; g < NG; ++g) {
            int64_t s0 = g * group;
            int64_t s_end = s0 + group < S ? s0 + group : S;
            for (int64_t s = s0; s < s_end; ++s) sink[s - s0] = (unsigned char)is_sink(idx, n_sink, b, s);
            for (int64_t d = 0; d < D; ++d) {
                int64_t n = 0;
                for (int64_t s = s0; s < s_end; ++s)
                    if (!sink[s - s0]) vals[n++] = widen(x[(bh * S + s) * D + d], dtype);
                float sc = 0.0f, z = 0.0f;
                if (n > 0) kivi_ref_group_params(vals, n, bits, &sc, &z);
                int64_t pi = (bh * NG + g) * D + d;
                scale[pi] = sc;
                zero[pi] = z;
                for (int64_t s = s0; s < s_end; ++s) {
                    float f = widen(x[(bh * S + s) * D + d], dtype);
                    codes[(bh * S + s) * D + d] =
                        sink[s - s0] ? 0 : (uint8_t)kivi_ref_code(f, sc, z, bits);
                }
            }
        }
    }
    free(vals);
    free(sink);
    return 0;
}

int kivi_ref_quant_keys_sink(const uint16_t* x, int dtype, int64_t B,
                             int64_t H, int64_t S, int64_t D, int bits,
                             int64_t group, const int32_t* idx, int64_t n_sink,
                             uint8_t* packed, float* scale, float* zero) {
    if (!sink_shape_ok(B, H, S, D, n_sink) || !shape_ok(B * H, S, D, bits, group))
        return 1;
    size_t n = (size_t)(B * H * S * D);
    uint8_t* codes = (uint8_t*)malloc(n ? n : 1);
    if (!codes) return 1;
    int st = kivi_ref_quant_keys_sink_unpacked(x, dtype, B, H, S, D, bits,
                                               group, idx, n_sink, codes,
                                               scale, zero);
    if (st == 0) st = kivi_ref_pack(codes, B * H * S, D, bits, packed);
    free(codes);
    return st;
}

/* The sinks' rows kept in 16-bit form: x_sink[bh, i, :] = x[bh, idx[b, i], :]
 * (a position outside [0, S) leaves its row of x_sink untouched). */
int kivi_ref_sink_gather(const uint16_t* x, int64_t B, int64_t H, int64_t S,
                         int64_t D, const int32_t* idx, int64_t n_sink,
                         uint16_t* x_sink) {
    if (!sink_shape_ok(B, H, S, D, n_sink)) return 1;
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t i = 0; i < n_sink; ++i) {
            int64_t s = idx[(bh / H) * n_sink + i];
            if (s < 0 || s >= S) continue;
            memcpy(x_sink + (bh * n_sink + i) * D, x + (bh * S + s) * D,
                   (size_t)D * sizeof(uint16_t));
        }
    return 0;
}

/* The reconstruction with sinks: each sink row copied back into the
 * dequantized tensor, out[bh, idx[b, i], :] = x_sink[bh, i, :]. */
int kivi_ref_sink_restore(const uint16_t* x_sink, int64_t B, int64_t H,
                          int64_t S, int64_t D, const int32_t* idx,
                          int64_t n_sink, uint16_t* out) {
    if (!sink_shape_ok(B, H, S, D, n_sink)) return 1;
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t i = 0; i < n_sink; ++i) {
            int64_t s = idx[(bh / H) * n_sink + i];
            if (s < 0 || s >= S) continue;
            memcpy(out + (bh * S + s) * D, x_sink + (bh * n_sink + i) * D,
                   (size_t)D * sizeof(uint16_t));
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Per-token mixed precision (VeloxQuant-MLX 0.24.1 package page, section   */
/* "ZipCache-adapted -- saliency-adaptive per-token mixed precision"): the  */
/* tokens with the highest key norm are quantized at hi_bits, the rest at   */
/* lo_bits, both with the KIVI group quantizer.  Reading: the two token     */
/* sets are quantized as two tensors -- the listed tokens of every head in  */
/* position order -- so a key group is `group` consecutive tokens of a set. */
/* ------------------------------------------------------------------------ */

static const float* g_part_score;   /* the scores being ranked by qsort */

/* Rank order: higher score first; of equal scores the lower position. */
static int rank_cmp(const void* a, const void* b) {
    int32_t i = *(const int32_t*)a, j = *(const int32_t*)b;
    float si = g_part_score[i], sj = g_part_score[j];
    if (si > sj) return -1;
    if (si < sj) return 1;
    return (i > j) - (i < j);
}

/* pos_hi [B, n_hi]: positions of the n_hi first tokens in rank order, listed
 * in ascending position; pos_lo [B, S - n_hi]: all other positions, ascending. */
int kivi_ref_partition_top(const float* score, int64_t B, int64_t S,
                           int64_t n_hi, int32_t* pos_hi, int32_t* pos_lo) {
    if (B < 0 || S < 0 || n_hi < 0 || n_hi > S) return 1;
    int32_t* order = (int32_t*)malloc((size_t)(S > 0 ? S : 1) * sizeof(int32_t));
    unsigned char* hi = (unsigned char*)malloc((size_t)(S > 0 ? S : 1));
    if (!order || !hi) {
        free(order);
        free(hi);
        return 1;
    }
    for (int64_t b = 0; b < B; ++b) {
        for (int64_t s = 0; s < S; ++s) order[s] = (int32_t)s;
        g_part_score = score + b * S;
        qsort(order, (size_t)S, sizeof(int32_t), rank_cmp);
        memset(hi, 0, (size_t)(S > 0 ? S : 1));
        for (int64_t r = 0; r < n_hi; ++r) hi[order[r]] = 1;
        int64_t nh = 0, nl = 0;
        for (int64_t s = 0; s < S; ++s) {
            if (hi[s]) pos_hi[b * n_hi + nh++] = (int32_t)s;
            else pos_lo[b * (S - n_hi) + nl++] = (int32_t)s;
        }
    }
    free(order);
    free(hi);
    return 0;
}

/* The listed tokens of every head as one tensor: out[bh, j, :] =
 * x[bh, pos[bh / H, j], :]. */
static uint16_t* gather_rows(const uint16_t* x, int64_t B, int64_t H,
                             int64_t S, int64_t D, const int32_t* pos,
                             int64_t n) {
    uint16_t* out = (uint16_t*)malloc((size_t)(B * H * n * D + 1) * sizeof(uint16_t));
    if (!out) return NULL;
    for (int64_t bh = 0; bh < B * H; ++bh)
        for (int64_t j = 0; j < n; ++j)
            memcpy(out + (bh * n + j) * D, x + (bh * S + pos[(bh / H) * n + j]) * D,
                   (size_t)D * sizeof(uint16_t));
    return out;
}

static int rows_ok(int64_t B, int64_t H, int64_t S, int64_t D,
                   const int32_t* pos, int64_t n) {
    if (B < 0 || H < 1 || S < 0 || D < 0 || n < 0 || n > S) return 0;
    for (int64_t i = 0; i < B * n; ++i)
        if (pos[i] < 0 || pos[i] >= S) return 0;
    return 1;
}

/* Keys of the listed tokens: kivi_ref_quant_keys of the gathered
 * [B*H, n, D] tensor (codes [B*H, n, D*bits/8], params [B*H, ceil(n/group), D]). */
int kivi_ref_quant_keys_rows(const uint16_t* x, int dtype, int64_t B,
                             int64_t H, int64_t S, int64_t D, int bits,
                             int64_t group, const int32_t* pos, int64_t n,
                             uint8_t* packed, float* scale, float* zero) {
    if (!rows_ok(B, H, S, D, pos, n)) return 1;
    uint16_t* g = gather_rows(x, B, H, S, D, pos, n);
    if (!g) return 1;
    int st = kivi_ref_quant_keys(g, dtype, B * H, n, D, bits, group, packed,
                                 scale, zero);
    free(g);
    return st;
}

/* Values of the listed tokens: kivi_ref_quant_values of the gathered tensor
 * (params [B*H, n, ceil(D/group)]). */
int kivi_ref_quant_values_rows(const uint16_t* x, int dtype, int64_t B,
                               int64_t H, int64_t S, int64_t D, int bits,
                               int64_t group, const int32_t* pos, int64_t n,
                               uint8_t* packed, float* scale, float* zero) {
    if (!rows_ok(B, H, S, D, pos, n)) return 1;
    uint16_t* g = gather_rows(x, B, H, S, D, pos, n);
    if (!g) return 1;
    int st = kivi_ref_quant_values(g, dtype, B * H, n, D, bits, group, packed,
                                   scale, zero);
    free(g);
    return st;
}

/* Dequantize a listed set and write its rows back to their positions:
 * out[bh, pos[bh / H, j], :] = recon[bh, j, :]; other rows are untouched. */
static int dequant_rows(int keys, const uint8_t* packed, const float* scale,
                        const float* zero, int64_t B, int64_t H, int64_t S,
                        int64_t D, int bits, int64_t group, const int32_t* pos,
                        int64_t n, int out_dtype, uint16_t* out) {
    if (!rows_ok(B, H, S, D, pos, n)) return 1;
    uint16_t* r = (uint16_t*)malloc((size_t)(B * H * n * D + 1) * sizeof(uint16_t));
    if (!r) return 1;
    int st = keys ? kivi_ref_dequant_keys(packed, scale, zero, B * H, n, D,
                                          bits, group, out_dtype, r)
                  : kivi_ref_dequant_values(packed, scale, zero, B * H, n, D,
                                            bits, group, out_dtype, r);
    if (st == 0)
        for (int64_t bh = 0; bh < B * H; ++bh)
            for (int64_t j = 0; j < n; ++j)
                memcpy(out + (bh * S + pos[(bh / H) * n + j]) * D, r + (bh * n + j) * D,
                       (size_t)D * sizeof(uint16_t));
    free(r);
    return st;
}

int kivi_ref_dequant_keys_rows(const uint8_t* packed, const float* scale,
                               const float* zero, int64_t B, int64_t H,
                               int64_t S, int64_t D, int bits, int64_t group,
                               const int32_t* pos, int64_t n, int out_dtype,
                               uint16_t* out) {
    return dequant_rows(1, packed, scale, zero, B, H, S, D, bits, group, pos,
                        n, out_dtype, out);
}

int kivi_ref_dequant_values_rows(const uint8_t* packed, const float* scale,
                                 const float* zero, int64_t B, int64_t H,
                                 int64_t S, int64_t D, int bits, int64_t group,
                                 const int32_t* pos, int64_t n, int out_dtype,
                                 uint16_t* out) {
    return dequant_rows(0, packed, scale, zero, B, H, S, D, bits, group, pos,
                        n, out_dtype, out);
}
