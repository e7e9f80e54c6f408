/*
 * KIVI reference oracle: plain, slow, obviously correct CPU implementation.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the GPU library (kivi.h / libkivi.so); the
 * product path never calls it.
 *
 * What it computes (sources are the VeloxQuant-MLX pages):
 *   - KIVI blog post on the fused Metal kernels, section "What we're actually
 *     optimizing": asymmetric min/max group quantization
 *       zero = min(group), scale = (max - min) / (2^bits - 1),
 *       q = round((x - zero) / scale), recon = q * scale + zero,
 *     keys grouped per channel along the token axis, values per token along
 *     the channel axis.
 *   - same post, section "The layout problem that shapes everything":
 *     tensors are [BH, S, D] row-major, element (bh, s, d) at bh*S*D + s*D + d.
 *   - same post, section "Three ways to be off by one bit": the dequant is a
 *     multiply then an add (two roundings, no FMA), rounding is half-to-even,
 *     and a ragged last group is padded by replicating the edge element.
 *   - VeloxQuant-MLX 0.8.0 release post, section "What KIVI is": codes are
 *     unsigned integers in [0, 2^bits - 1].
 *   - TurboQuant Metal kernels post, section "Kernel 1: Bit-Packing", and the
 *     TurboQuant port overview, section "The Bit-Packing Problem": 8/bits
 *     codes per byte, element i of a byte at bit offset i*bits (LSB first).
 *
 * Arithmetic: every step is one IEEE-754 binary32 operation rounded to nearest
 * even (the pages' kernels widen each element to float and keep min/max in
 * float).  The file must be compiled with floating-point contraction off.
 *
 * Readings where the pages are silent (each listed in the design notes):
 *   - a group whose computed scale is 0 gets code 0 and reconstructs to zero;
 *   - a min or max equal to zero is stored as +0 (signed-zero canonical form);
 *   - codes are packed along D, one layout for keys and values,
 *     [BH, S, D*bits/8] bytes; scale and zero are fp32, planar,
 *     keys [BH, ceil(S/G), D], values [BH, S, ceil(D/G)].
 *
 * dtype: 0 = IEEE binary16 (fp16), 1 = bfloat16.  Tensors are passed as raw
 * 16-bit patterns.
 */
#ifndef KIVI_ORACLE_H
#define KIVI_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status: 0 ok, 1 bad argument */

/* Exact widening and round-to-nearest-even narrowing of the 16-bit types. */
float    kivi_ref_half_to_float(uint16_t h);
uint16_t kivi_ref_float_to_half(float f);
float    kivi_ref_bf16_to_float(uint16_t h);
uint16_t kivi_ref_float_to_bf16(float f);

/* Array forms of the four conversions above (dtype 0 fp16, 1 bf16). */
int kivi_ref_widen_array(const uint16_t* in, int64_t n, int dtype, float* out);
int kivi_ref_narrow_array(const float* in, int64_t n, int dtype, uint16_t* out);

/* One group: n fp32 values -> (scale, zero). */
int   kivi_ref_group_params(const float* vals, int64_t n, int bits,
                            float* scale, float* zero);
/* One element -> its code, given its group's (scale, zero). */
int   kivi_ref_code(float f, float scale, float zero, int bits);
/* One code -> fp32 reconstruction (multiply, then add). */
float kivi_ref_recon(int code, float scale, float zero);

/* Unpacked codes (one per byte, [BH,S,D]) plus planar params. */
int kivi_ref_quant_keys_unpacked(const uint16_t* x, int dtype, int64_t BH,
                                 int64_t S, int64_t D, int bits, int64_t group,
                                 uint8_t* codes, float* scale, float* zero);
int kivi_ref_quant_values_unpacked(const uint16_t* x, int dtype, int64_t BH,
                                   int64_t S, int64_t D, int bits,
                                   int64_t group, uint8_t* codes, float* scale,
                                   float* zero);

/* Bit packing of [rows, D] codes into [rows, D*bits/8] bytes and back. */
int kivi_ref_pack(const uint8_t* codes, int64_t rows, int64_t D, int bits,
                  uint8_t* packed);
int kivi_ref_unpack(const uint8_t* packed, int64_t rows, int64_t D, int bits,
                    uint8_t* codes);

/* Full quantize: packed codes [BH,S,D*bits/8] plus params. */
int kivi_ref_quant_keys(const uint16_t* x, int dtype, int64_t BH, int64_t S,
                        int64_t D, int bits, int64_t group, uint8_t* packed,
                        float* scale, float* zero);
int kivi_ref_quant_values(const uint16_t* x, int dtype, int64_t BH, int64_t S,
                          int64_t D, int bits, int64_t group, uint8_t* packed,
                          float* scale, float* zero);

/* Dequantize packed codes + params into out_dtype 16-bit patterns [BH,S,D]. */
int kivi_ref_dequant_keys(const uint8_t* packed, const float* scale,
                          const float* zero, int64_t BH, int64_t S, int64_t D,
                          int bits, int64_t group, int out_dtype,
                          uint16_t* out);
int kivi_ref_dequant_values(const uint8_t* packed, const float* scale,
                            const float* zero, int64_t BH, int64_t S,
                            int64_t D, int bits, int64_t group, int out_dtype,
                            uint16_t* out);

/* Residual-window cache (KIVI blog post on the fused Metal kernels, section
 * "What we're actually optimizing": the most recent residual_length tokens
 * stay in 16-bit floats and, once enough fresh tokens have accumulated, are
 * quantized as a batch -- a flush; the 0.8.0 release post, section "What
 * KIVI is": the last R tokens are held exactly and tokens are quantized as
 * they age out of that window).  Reading: tokens arrive one at a time; after
 * each, while at least R + G_k tokens are unquantized, the oldest G_k of them
 * (one whole key group, group-aligned) are quantized -- keys per channel
 * over those G_k tokens, values per token -- into the compressed store at
 * their own token offset.  Every appended token is also kept in k / v, so a
 * test can read back the tokens [Q, T) that are still unquantized.
 * The caller allocates every array:
 *   k, v              [BH, S_max, D] 16-bit patterns
 *   k_codes, v_codes  [BH, S_max, D*bits/8]
 *   k_scale, k_zero   [BH, ceil(S_max/G_k), D]
 *   v_scale, v_zero   [BH, S_max, ceil(D/G_v)]
 * and sets T = Q = 0 before the first append. */
typedef struct {
    int64_t BH, D, S_max, R, G_k, G_v;
    int32_t bits, dtype;
    uint16_t* k;
    uint16_t* v;
    uint8_t* k_codes;
    uint8_t* v_codes;
    float* k_scale;
    float* k_zero;
    float* v_scale;
    float* v_zero;
    int64_t T, Q;   /* tokens appended, tokens quantized */
} kivi_ref_cache;

/* Append n tokens of every bh (k_new, v_new [BH, n, D]); flush as above.
 * Returns 1 (and appends nothing) if the cache would exceed S_max or an
 * argument is invalid. */
int kivi_ref_cache_append(kivi_ref_cache* c, const uint16_t* k_new,
                          const uint16_t* v_new, int64_t n);

/* KIVI-Sink (VeloxQuant-MLX 0.24.1 package page, section "KVSink-adapted
 * sink protection").  Keys are [B*H, S, D] with the H KV heads of sequence b
 * at rows b*H .. b*H + H - 1; a sink list is [B, n_sink] positions.
 *   sink_scores: score[b, s] = mean over heads of the key's L2 norm
 *                (per head fma-accumulated squares in channel order, fp32
 *                square root, head-order sum, one division by H);
 *   sink_select: the n_sink highest scores per sequence, highest first, the
 *                lower position first among equal scores (0 <= n_sink <= S);
 *   quant_keys_sink: per-channel key quantization whose group min/max skip
 *                the sinks; a sink's code is 0; an all-sink group has scale
 *                0 and zero 0;
 *   sink_gather / sink_restore: copy the sinks' rows to / from
 *                [B*H, n_sink, D] (positions outside [0, S) are skipped). */
int kivi_ref_sink_scores(const uint16_t* k, int dtype, int64_t B, int64_t H,
                         int64_t S, int64_t D, float* score);
int kivi_ref_sink_select(const float* score, int64_t B, int64_t S,
                         int64_t n_sink, int32_t* idx);
int kivi_ref_quant_keys_sink_unpacked(const uint16_t* x, int dtype, int64_t B,
                                      int64_t H, int64_t S, int64_t D,
                                      int bits, int64_t group,
                                      const int32_t* idx, int64_t n_sink,
                                      uint8_t* codes, float* scale,
                                      float* zero);
int kivi_ref_quant_keys_sink(const uint16_t* x, int dtype, int64_t B,
                             int64_t H, int64_t S, int64_t D, int bits,
                             int64_t group, const int32_t* idx, int64_t n_sink,
                             uint8_t* packed, float* scale, float* zero);
int kivi_ref_sink_gather(const uint16_t* x, int64_t B, int64_t H, int64_t S,
                         int64_t D, const int32_t* idx, int64_t n_sink,
                         uint16_t* x_sink);
int kivi_ref_sink_restore(const uint16_t* x_sink, int64_t B, int64_t H,
                          int64_t S, int64_t D, const int32_t* idx,
                          int64_t n_sink, uint16_t* out);

/* Per-token mixed precision (VeloxQuant-MLX 0.24.1 package page, section
 * "ZipCache-adapted -- saliency-adaptive per-token mixed precision"): the
 * n_hi tokens of highest key-norm score per sequence at hi_bits, the rest at
 * lo_bits.  The two sets are quantized as two tensors of the listed tokens.
 *   partition_top: pos_hi [B, n_hi] the n_hi first positions in the order
 *       (score descending, position ascending), listed ascending; pos_lo
 *       [B, S - n_hi] the others, ascending;
 *   quant_{keys,values}_rows: the plain quantizers applied to the tensor
 *       [B*H, n, D] of rows x[bh, pos[bh / H, j]] (positions in [0, S));
 *   dequant_{keys,values}_rows: the plain dequantizers, each row written
 *       back to out[bh, pos[bh / H, j]]. */
int kivi_ref_partition_top(const float* score, int64_t B, int64_t S,
                           int64_t n_hi, int32_t* pos_hi, int32_t* pos_lo);
int kivi_ref_quant_keys_rows(const uint16_t* x, int dtype, int64_t B,
                             int64_t H, int64_t S, int64_t D, int bits,
                             int64_t group, const int32_t* pos, int64_t n,
                             uint8_t* packed, float* scale, float* zero);
int kivi_ref_quant_values_rows(const uint16_t* x, int dtype, int64_t B,
                               int64_t H, int64_t S, int64_t D, int bits,
                               int64_t group, const int32_t* pos, int64_t n,
                               uint8_t* packed, float* scale, float* zero);
int kivi_ref_dequant_keys_rows(const uint8_t* packed, const float* scale,
                               const float* zero, int64_t B, int64_t H,
                               int64_t S, int64_t D, int bits, int64_t group,
                               const int32_t* pos, int64_t n, int out_dtype,
                               uint16_t* out);
int kivi_ref_dequant_values_rows(const uint8_t* packed, const float* scale,
                                 const float* zero, int64_t B, int64_t H,
                                 int64_t S, int64_t D, int bits, int64_t group,
                                 const int32_t* pos, int64_t n, int out_dtype,
                                 uint16_t* out);

#ifdef __cplusplus
}
#endif
#endif
