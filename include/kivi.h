/*
 * kivi.h -- C ABI of libkivi.so, the KIVI KV-cache flush for MI355X (gfx950).
 *
 * The method (VeloxQuant-MLX pages; KIVI blog post on the fused Metal
 * kernels, section "What we're actually optimizing", and the 0.8.0 release
 * post, section "What KIVI is"): asymmetric min/max group quantization,
 *     zero  = min(group)
 *     scale = (max(group) - min(group)) / (2^bits - 1)
 *     code  = clip(round_half_even((x - zero) / scale), 0, 2^bits - 1)
 *     recon = code * scale + zero          (multiply rounded, then add)
 * with keys grouped per channel over `group` consecutive tokens and values
 * grouped per token over `group` consecutive channels.  Every step is one
 * IEEE binary32 operation rounded to nearest even ("Three ways to be off by
 * one bit": two roundings in the dequant, half-to-even rounding; a ragged
 * last group behaves as if padded with its edge element, i.e. its min/max
 * are over its real elements).  A group whose scale is 0 (constant group)
 * gets code 0 and reconstructs to `zero`; a min or max equal to zero is
 * stored as +0.
 *
 * Layouts (section "The layout problem that shapes everything"):
 *   x, recon, out : [BH, S, D] row-major 16-bit floats, element (bh, s, d)
 *                   at bh*S*D + s*D + d (batch and heads flattened into BH).
 *   codes         : [BH, S, D*bits/8] bytes; along D, 8/bits codes per byte,
 *                   code i of a byte in bits [i*bits, (i+1)*bits) (the
 *                   TurboQuant Metal kernels post, section "Kernel 1:
 *                   Bit-Packing").  One layout for keys and values.
 *   key params    : scale, zero fp32 [BH, ceil(S/group), D] (planar).
 *   value params  : scale, zero fp32 [BH, S, ceil(D/group)] (planar).
 *
 * Ownership and execution: every pointer is caller-owned device memory
 * (e.g. allocated by PyTorch); the library never allocates, frees or
 * synchronises and keeps no state between calls (apart from the per-thread
 * profiling events of kivi_time_next_launch, the launch counter of
 * kivi_launch_count and the per-device workspace of
 * kivi_cache_attend_noalloc); calls are re-entrant.
 * Work is enqueued on `stream` (0 = the null stream) and runs
 * asynchronously; outputs are valid once the stream has reached the call.
 * Inputs and outputs must not overlap.
 *
 * Errors: every argument is checked before anything is launched; on an
 * error nothing is written and nothing is launched.  Rules:
 *   bits in {1, 2, 4, 8}                                   else KIVI_ERR_BITS
 *   group >= 1                                             else KIVI_ERR_GROUP
 *   BH, S, D >= 0, D*bits % 8 == 0, BH*S*D*2 fits int64    else KIVI_ERR_SHAPE
 *   dtype is KIVI_FP16 or KIVI_BF16                        else KIVI_ERR_DTYPE
 *   every pointer that must be written or read is non-NULL else KIVI_ERR_NULL
 *   every pointer is 16-byte aligned                       else KIVI_ERR_ALIGN
 * An empty tensor (BH, S or D equal to 0) is valid and launches nothing.
 * A failed launch returns KIVI_ERR_LAUNCH.  Results for NaN or infinite
 * inputs, or for groups whose max - min overflows binary32, are unspecified.
 */
#ifndef KIVI_H
#define KIVI_H

#include <stdint.h>

#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    KIVI_OK = 0,
    KIVI_ERR_NULL = 1,
    KIVI_ERR_SHAPE = 2,
    KIVI_ERR_BITS = 3,
    KIVI_ERR_GROUP = 4,
    KIVI_ERR_DTYPE = 5,
    KIVI_ERR_ALIGN = 6,
    KIVI_ERR_LAUNCH = 7,
    KIVI_ERR_SCRATCH = 8
} kivi_status;

typedef enum { KIVI_FP16 = 0, KIVI_BF16 = 1 } kivi_dtype;

/*
 * Quantize keys per channel (KIVI blog post on the fused Metal kernels,
 * section "Kernel A -- per-channel keys"): for every (bh, token group g,
 * channel d) the group is tokens [g*group, min(g*group + group, S)) of
 * channel d, read along the strided S axis.
 *   k      in : [BH, S, D] of dtype `dt`
 *   codes out : [BH, S, D*bits/8] bytes
 *   scale, zero out : fp32 [BH, ceil(S/group), D]
 */
kivi_status kivi_quant_keys(const void* k, kivi_dtype dt, int64_t BH,
                            int64_t S, int64_t D, int bits, int64_t group,
                            uint8_t* codes, float* scale, float* zero,
                            hipStream_t stream);

/*
 * Quantize values per token (same post, section "Kernel B -- per-token
 * values"): for every (bh, token s, channel group j) the group is channels
 * [j*group, min(j*group + group, D)) of token s, along the contiguous D axis.
 *   v      in : [BH, S, D] of dtype `dt`
 *   codes out : [BH, S, D*bits/8] bytes
 *   scale, zero out : fp32 [BH, S, ceil(D/group)]
 */
kivi_status kivi_quant_values(const void* v, kivi_dtype dt, int64_t BH,
                              int64_t S, int64_t D, int bits, int64_t group,
                              uint8_t* codes, float* scale, float* zero,
                              hipStream_t stream);

/*
 * Dequantize keys (section "What we're actually optimizing", recon =
 * code * scale + zero, and "Three ways to be off by one bit", item 1: the
 * product is rounded before the add): codes and key params as produced by
 * kivi_quant_keys with the same bits and group -> out [BH, S, D] of
 * `out_dt`, each recon rounded to nearest even in that type.
 */
kivi_status kivi_dequant_keys(const uint8_t* codes, const float* scale,
                              const float* zero, int64_t BH, int64_t S,
                              int64_t D, int bits, int64_t group,
                              kivi_dtype out_dt, void* out,
                              hipStream_t stream);

/* Dequantize values: as kivi_dequant_keys with value params
 * [BH, S, ceil(D/group)]. */
kivi_status kivi_dequant_values(const uint8_t* codes, const float* scale,
                                const float* zero, int64_t BH, int64_t S,
                                int64_t D, int bits, int64_t group,
                                kivi_dtype out_dt, void* out,
                                hipStream_t stream);

/*
 * Fused quantize -> dequantize of keys in one pass: the operation the
 * pages' own Metal kernels perform (section "Three ways to be off by one
 * bit", item 1, and "So why does the kernel ship?": the cache quantizes and
 * immediately expands back to the input type).  Writes recon [BH, S, D] in
 * dtype `dt`, bit-identical to kivi_quant_keys followed by
 * kivi_dequant_keys.  codes, scale and zero are either all non-NULL (they
 * are written as by kivi_quant_keys) or all NULL (recon only).
 */
kivi_status kivi_quant_dequant_keys(const void* k, kivi_dtype dt, int64_t BH,
                                    int64_t S, int64_t D, int bits,
                                    int64_t group, uint8_t* codes,
                                    float* scale, float* zero, void* recon,
                                    hipStream_t stream);

/* Fused quantize -> dequantize of values; as kivi_quant_dequant_keys. */
kivi_status kivi_quant_dequant_values(const void* v, kivi_dtype dt,
                                      int64_t BH, int64_t S, int64_t D,
                                      int bits, int64_t group, uint8_t* codes,
                                      float* scale, float* zero, void* recon,
                                      hipStream_t stream);

/*
 * Keys and values of one flush in one call (the 0.8.0 release post, section
 * "What KIVI is": a flush quantizes the aged-out keys per channel and the
 * values per token together; the KIVI blog post on the fused Metal kernels,
 * section "What we're actually optimizing": at decode sizes the flush is
 * launch-bound).  Each result is exactly that of the single call on that
 * tensor (kivi_quant_keys / kivi_quant_values, kivi_quant_dequant_*,
 * kivi_dequant_*), with group_k for keys and group_v for values.  K and V
 * share dtype, shape and bits; every argument of both halves is checked by
 * the single call's rules before anything is launched, and codes/params
 * must be given for both tensors or (kivi_quant_dequant_kv) for neither.
 * Small flushes run as one kernel launch: for the quantizing calls, D/8
 * dividing 16, key groups of 17 to 32 tokens, fewer than 65536 (bh, key
 * group, 8-channel) items and value groups of 32 * 2^k channels; for
 * kivi_dequant_kv, D a multiple of 8 up to 2048, fewer than 65536 key items
 * and value groups a multiple of 32.  Otherwise the two single launches
 * are issued, keys first (a caller timing one launch then sees the keys').
 */
kivi_status kivi_quant_kv(const void* k, const void* v, kivi_dtype dt,
                          int64_t BH, int64_t S, int64_t D, int bits,
                          int64_t group_k, int64_t group_v, uint8_t* k_codes,
                          float* k_scale, float* k_zero, uint8_t* v_codes,
                          float* v_scale, float* v_zero, hipStream_t stream);
kivi_status kivi_quant_dequant_kv(const void* k, const void* v, kivi_dtype dt,
                                  int64_t BH, int64_t S, int64_t D, int bits,
                                  int64_t group_k, int64_t group_v,
                                  uint8_t* k_codes, float* k_scale,
                                  float* k_zero, uint8_t* v_codes,
                                  float* v_scale, float* v_zero, void* k_recon,
                                  void* v_recon, hipStream_t stream);
kivi_status kivi_dequant_kv(const uint8_t* k_codes, const float* k_scale,
                            const float* k_zero, const uint8_t* v_codes,
                            const float* v_scale, const float* v_zero,
                            int64_t BH, int64_t S, int64_t D, int bits,
                            int64_t group_k, int64_t group_v, kivi_dtype out_dt,
                            void* k_out, void* v_out, hipStream_t stream);

/*
 * Residual-window cache (KIVI blog post on the fused Metal kernels, section
 * "What we're actually optimizing": the most recent residual_length tokens
 * stay in 16-bit floats and, once enough fresh tokens have accumulated, are
 * quantized as a batch -- a flush -- and folded into the compressed store;
 * the 0.8.0 release post, section "What KIVI is": the last R tokens are held
 * exactly and tokens are quantized as they age out of that window).
 *
 * After an append brings the cache to T tokens, the first
 *     Q = G_k * floor((T - R) / G_k)     (0 while T < R)
 * tokens are quantized, in whole key groups aligned at token 0, and tokens
 * [Q, T) -- at least min(T, R) and fewer than R + G_k of them -- are held
 * in 16-bit ring buffers.  The compressed store then equals kivi_quant_keys
 * / kivi_quant_values of tokens [0, Q) at their own offsets (keys grouped
 * per channel over G_k tokens, values per token over G_v channels).
 *
 * The struct carries the geometry, caller-owned device buffers and the two
 * counters:
 *   k_ring, v_ring    [BH, ring, D] 16-bit (dtype); token s in [Q, T) is
 *                     in slot s % ring.  ring: a multiple of G_k, >= R + G_k
 *   k_codes, v_codes  [BH, S_max, D*bits/8] bytes (layout as kivi_quant_*)
 *   k_scale, k_zero   fp32 [BH, ceil(S_max/G_k), D]
 *   v_scale, v_zero   fp32 [BH, S_max, ceil(D/G_v)]
 *   T, Q              tokens appended / quantized; 0 and 0 for an empty cache
 * Storage past Q (codes, params) and ring slots of other tokens are not
 * written.
 */
typedef struct {
    int64_t BH, D, S_max, R, G_k, G_v, ring;
    int32_t bits;
    int32_t dtype;            /* kivi_dtype */
    void* k_ring;
    void* v_ring;
    uint8_t* k_codes;
    uint8_t* v_codes;
    float* k_scale;
    float* k_zero;
    float* v_scale;
    float* v_zero;
    int64_t T, Q;
} kivi_cache;

/*
 * Append n tokens of every bh: k_new, v_new [BH, n, D] of the cache's dtype
 * (device memory, read before the call's work completes).  Enqueues on
 * `stream`: the flush of tokens [Q, Q_new) (from the ring and from the new
 * tokens) into the compressed store, then the copy of the new tokens that
 * stay unquantized into their ring slots; then sets cache->T and cache->Q
 * to their new values (they describe the state once the stream has reached
 * this call).  Calls on one cache must be ordered on one stream.
 * Errors (nothing is enqueued and the struct is unchanged):
 *   cache == NULL, a NULL buffer, or k_new/v_new NULL with n > 0 KIVI_ERR_NULL
 *   bits not 1, 2, 4, 8                                       KIVI_ERR_BITS
 *   G_k not in [1, 32], or G_v not 8, 16 or 32 * 2^k          KIVI_ERR_GROUP
 *   dtype invalid                                             KIVI_ERR_DTYPE
 *   D not 8, 16, 32, 64, 128 or 256; BH, R, S_max or n < 0; ring not a
 *   multiple of G_k or < R + G_k; S_max or ring >= 2^31; BH*S_max*D/2
 *   >= 2^32; an inconsistent state (not 0 <= Q <= T <= S_max,
 *   Q % G_k == 0, T - Q < ring); T + n > S_max                 KIVI_ERR_SHAPE
 *   a pointer not 16-byte aligned                             KIVI_ERR_ALIGN
 */
kivi_status kivi_cache_append(kivi_cache* cache, const void* k_new,
                              const void* v_new, int64_t n,
                              hipStream_t stream);

/*
 * Decode attention over a residual-window cache, reading the compressed
 * store directly (KIVI blog post on the fused Metal kernels, section "So
 * why does the kernel ship?": the memory and speed win needs packed storage
 * and attention that expands the codes in registers, never in memory).
 * For every bh and query head j < n_q (n_q query heads share each KV head):
 *     out[bh, j] = softmax_t(sm_scale * q[bh, j] . K[bh, t]) V[bh, t]
 * over the cache's T tokens, where K, V of tokens t < Q are the codes
 * reconstructed with their group's params, code * scale + zero, used in
 * fp32 without rounding to the 16-bit type (a key through
 * sum_d (q_d scale_d) code_d + sum_d q_d zero_d, a value through
 * (p scale) code + p zero), and tokens t >= Q are the exact tokens in the
 * rings.  fp32 scores, softmax and accumulation; out is rounded to the
 * cache's dtype.
 *   q    in  : [BH, n_q, D] of the cache's dtype
 *   out  out : [BH, n_q, D] of the cache's dtype
 *   work     : device scratch of at least kivi_cache_attend_work_bytes
 *              bytes (16-byte aligned); its contents are not used after
 *              the call
 * Uses the cache's counters at the time of the call; launches two kernels.
 * Errors (nothing is launched): any kivi_cache_append rule on the struct;
 * D not 64 or 128, D * bits < 128, G_k not 8, 16 or 32, T < 1 or
 * BH >= 65536
 * (KIVI_ERR_SHAPE / KIVI_ERR_GROUP); n_q not in [1, 8] (KIVI_ERR_SHAPE);
 * a NULL pointer (KIVI_ERR_NULL); a misaligned one (KIVI_ERR_ALIGN);
 * work_bytes too small (KIVI_ERR_SHAPE).
 */
kivi_status kivi_cache_attend(const kivi_cache* cache, const void* q,
                              int64_t n_q, float sm_scale, void* out,
                              void* work, int64_t work_bytes,
                              hipStream_t stream);

/* Workspace bytes kivi_cache_attend needs for this cache (at its current T)
 * and n_q; -1 if the arguments are invalid. */
int64_t kivi_cache_attend_work_bytes(const kivi_cache* cache, int64_t n_q);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * kivi_cache_attend with its chunk workspace in a buffer that the library
 * itself holds on each device, KIVI_ATTEND_SCRATCH_BYTES (32 MiB) per GPU,
 * kept until the process ends.  Same arguments, results and errors as
 * kivi_cache_attend, without work / work_bytes; a call whose workspace
 * (kivi_cache_attend_work_bytes) exceeds the buffer returns
 * KIVI_ERR_SCRATCH and launches nothing (e.g. 224 KV heads x 3 query heads
 * at D = 128 fit up to about 12 000 cached tokens).  The call allocates
 * nothing and does not synchronise; its first call on a device (the current
 * device) looks up that device's copy of the buffer.  Nothing in the buffer
 * needs clearing: every call writes each workspace slot it reads.  All
 * calls on one GPU share that GPU's buffer, so calls that may overlap in
 * time (on different streams, or from threads without ordering) race and
 * give undefined results; calls ordered on one stream are safe.
 */
#define KIVI_ATTEND_SCRATCH_BYTES (32ll << 20)
kivi_status kivi_cache_attend_noalloc(const kivi_cache* cache, const void* q,
                                      int64_t n_q, float sm_scale, void* out,
                                      hipStream_t stream);

/*
 * KIVI-Sink (VeloxQuant-MLX 0.24.1 package page, section "KVSink-adapted
 * sink protection"): per sequence, the n_sink token positions whose keys
 * have the largest L2 norm averaged over the KV heads are sinks; they are
 * kept in 16-bit form and left out of the min/max of their key groups, so a
 * high-magnitude sink does not stretch its neighbours' scale.
 *
 * Layout: keys and values [B*H, S, D] (the [BH, S, D] layout above with the
 * H KV heads of sequence b at rows b*H .. b*H + H - 1); a sink list is
 * int32 [B, n_sink] token positions; a sink store is [B*H, n_sink, D] of the
 * tensor's 16-bit type, row (bh, i) holding token idx[bh / H, i].
 * Common rules (else nothing is launched): B, H, S >= 1 and D >= 8
 * (KIVI_ERR_SHAPE), 0 <= n_sink <= min(S, 64) (KIVI_ERR_SHAPE), B*H*S*D
 * < 2^40 and B*S < 2^31 (KIVI_ERR_SHAPE), dtype as above, pointers non-NULL
 * (KIVI_ERR_NULL) and 16-byte aligned (KIVI_ERR_ALIGN; 4-byte for idx and
 * score).  Positions outside [0, S) in a list given by the caller are
 * ignored.  n_sink == 0 launches nothing (kivi_sink_select still writes the
 * scores).
 */

/* Scores and selection.  score[b, s] (fp32 [B, S], written) is the mean
 * over the H heads of the L2 norm of key row (b*H + h, s): per head the
 * squares summed in channel order with one rounding per step, the correctly
 * rounded square root, the head-order sum divided once by H.  idx (int32
 * [B, n_sink], written) gets each sequence's n_sink highest scores, highest
 * first; of equal scores the lower position comes first.  D must be a power
 * of two in [8, 256] (KIVI_ERR_SHAPE).  Launches two kernels (one when
 * n_sink == 0). */
kivi_status kivi_sink_select(const void* k, kivi_dtype dt, int64_t B,
                             int64_t H, int64_t S, int64_t D, int64_t n_sink,
                             float* score, int32_t* idx, hipStream_t stream);

/* Per-channel key quantization with sinks: as kivi_quant_keys (codes
 * [B*H, S, D*bits/8], params [B*H, ceil(S/group), D]), except that each
 * group's min and max run over its tokens that are not sinks of the row's
 * sequence; a sink's code is 0, and a group made only of sinks gets scale 0
 * and zero 0.  recon, if non-NULL ([B*H, S, D], the input's dtype), gets the
 * reconstruction with every sink row equal to its input row (the dequant of
 * the codes followed by kivi_sink_restore).  codes, scale and zero are all
 * given or all NULL; at least one output (KIVI_ERR_NULL).  D % 8 == 0
 * (KIVI_ERR_SHAPE); 1 <= group <= 32 (KIVI_ERR_GROUP).  One kernel. */
kivi_status kivi_quant_keys_sink(const void* k, kivi_dtype dt, int64_t B,
                                 int64_t H, int64_t S, int64_t D, int bits,
                                 int64_t group, const int32_t* idx,
                                 int64_t n_sink, uint8_t* codes, float* scale,
                                 float* zero, void* recon, hipStream_t stream);

/* Keep the sinks' rows: x_sink[bh, i, :] = x[bh, idx[bh / H, i], :].
 * Values need nothing more than this: a value group is one token, so the
 * plain kivi_quant_values already leaves every other token untouched by a
 * sink.  D % 8 == 0 (KIVI_ERR_SHAPE).  One kernel. */
kivi_status kivi_sink_gather(const void* x, int64_t B, int64_t H, int64_t S,
                             int64_t D, const int32_t* idx, int64_t n_sink,
                             void* x_sink, hipStream_t stream);

/* Put the sinks' rows back into a dequantized tensor:
 * out[bh, idx[bh / H, i], :] = x_sink[bh, i, :].  D % 8 == 0
 * (KIVI_ERR_SHAPE).  One kernel. */
kivi_status kivi_sink_restore(const void* x_sink, int64_t B, int64_t H,
                              int64_t S, int64_t D, const int32_t* idx,
                              int64_t n_sink, void* out, hipStream_t stream);

/*
 * Per-token mixed precision (VeloxQuant-MLX 0.24.1 package page, section
 * "ZipCache-adapted -- saliency-adaptive per-token mixed precision"): the
 * tokens of highest key-norm score (kivi_sink_select with n_sink = 0 gives
 * the scores) are quantized at hi_bits and the rest at lo_bits, both with
 * the KIVI group quantizer.  The two token sets are position lists shared
 * by the H heads of a sequence; each set is quantized as its own tensor of
 * the listed rows, so a key group is `group` consecutive tokens of a set.
 *
 * Layout: x and out [B*H, S, D] as for KIVI-Sink; a list is int32 [B, n]
 * positions in [0, S), distinct within a sequence (ascending, as
 * kivi_partition_top writes them, keeps a key group's tokens in order); a
 * set's codes [B*H, n, D*bits/8], key params [B*H, ceil(n/group), D],
 * value params [B*H, n, ceil(D/group)].  A position outside [0, S) is read
 * clamped into range by the quantizers (its results are unspecified) and
 * is never written by the dequantizers.
 * Rules (else nothing is launched): bits in {1, 2, 4, 8} (KIVI_ERR_BITS);
 * key group in [1, 32], value group 8, 16 or 32 * 2^k (KIVI_ERR_GROUP);
 * B, H, S >= 1, D in {8, 16, 32, 64, 128, 256}, 0 <= n <= S, B*H*n < 2^31,
 * B*H*S*D < 2^40, for keys B*H*ceil(n/group)*D < 2^33 (KIVI_ERR_SHAPE); dtype (KIVI_ERR_DTYPE); non-NULL
 * (KIVI_ERR_NULL) and 16-byte aligned pointers, 4-byte for lists
 * (KIVI_ERR_ALIGN).  n == 0 launches nothing.  One kernel per call.
 */

/* pos_hi [B, n_hi] gets the n_hi first positions of each sequence in the
 * order (score descending, position ascending), listed in ascending
 * position; pos_lo [B, S - n_hi] the other positions, ascending.  score is
 * fp32 [B, S] (NaN scores: unspecified).  0 <= n_hi <= S < 2^31, B >= 1;
 * pos_hi may be NULL when n_hi == 0 and pos_lo when n_hi == S. */
kivi_status kivi_partition_top(const float* score, int64_t B, int64_t S,
                               int64_t n_hi, int32_t* pos_hi, int32_t* pos_lo,
                               hipStream_t stream);

/* Quantize the listed rows as one [B*H, n, D] tensor: keys per channel over
 * groups of `group` consecutive listed tokens, values per token. */
kivi_status kivi_quant_keys_rows(const void* k, kivi_dtype dt, int64_t B,
                                 int64_t H, int64_t S, int64_t D, int bits,
                                 int64_t group, const int32_t* pos, int64_t n,
                                 uint8_t* codes, float* scale, float* zero,
                                 hipStream_t stream);
kivi_status kivi_quant_values_rows(const void* v, kivi_dtype dt, int64_t B,
                                   int64_t H, int64_t S, int64_t D, int bits,
                                   int64_t group, const int32_t* pos,
                                   int64_t n, uint8_t* codes, float* scale,
                                   float* zero, hipStream_t stream);

/* Dequantize a set and write each row j of head bh to
 * out[bh, pos[bh / H, j], :]; rows of out not listed are untouched. */
kivi_status kivi_dequant_keys_rows(const uint8_t* codes, const float* scale,
                                   const float* zero, int64_t B, int64_t H,
                                   int64_t S, int64_t D, int bits,
                                   int64_t group, const int32_t* pos,
                                   int64_t n, kivi_dtype out_dt, void* out,
                                   hipStream_t stream);
kivi_status kivi_dequant_values_rows(const uint8_t* codes, const float* scale,
                                     const float* zero, int64_t B, int64_t H,
                                     int64_t S, int64_t D, int bits,
                                     int64_t group, const int32_t* pos,
                                     int64_t n, kivi_dtype out_dt, void* out,
                                     hipStream_t stream);

/*
 * Profiling aid: the next kernel that a kivi_* call made by this thread
 * launches records `start` when it begins executing and `stop` when it ends
 * (hipExtLaunchKernel), so hipEventElapsedTime(start, stop) is that kernel's
 * duration alone, without the dispatch gap that events recorded between
 * launches include.  Both events must be created by the caller (e.g.
 * hipEventCreate) and outlive the launch.  The pair is consumed by the next
 * launch: every quantize or dequantize call launches exactly one kernel,
 * kivi_cache_append up to three, kivi_cache_attend and kivi_sink_select
 * two (the pair times the first), and calls that
 * launch nothing -- errors, empty tensors -- leave it armed.  Passing NULL
 * for either disarms it.
 */
void kivi_time_next_launch(hipEvent_t start, hipEvent_t stop);

/*
 * Profiling aid: the number of kernel launches the library has made in this
 * process (every thread, every device; a launch recorded into a graph under
 * capture counts once, however often the graph is replayed).  Lets a
 * profiler's dispatch trace be split into the phases of a benchmark.
 */
int64_t kivi_launch_count(void);

/*
 * Self-test of the division shortcuts the quantizers use on this GPU.  The
 * pages prescribe IEEE division for the scale and for every code's quotient
 * (section "What we're actually optimizing": subtract, divide, round, clip);
 * the kernels reach the same correctly rounded results with (1) Markstein's
 * quotient by the constant 2^bits - 1 and (2) the hardware reciprocal
 * refined by one Newton step.  This call checks both against IEEE division
 * for every significand at every exponent where the kernels use them, and
 * adds the number of mismatches to *mismatches (one device-memory
 * unsigned long long, 8-byte aligned, zeroed by the caller).  Zero
 * mismatches is what every quantizer result relies on.
 */
kivi_status kivi_selftest_division(unsigned long long* mismatches,
                                   hipStream_t stream);

/* Sizes: bytes of packed codes, and element counts of each params array
 * (scale and zero each), for a [BH, S, D] tensor.  Return -1 on invalid
 * arguments (same rules as above). */
int64_t kivi_codes_bytes(int64_t BH, int64_t S, int64_t D, int bits);
int64_t kivi_key_param_count(int64_t BH, int64_t S, int64_t D,
                             int64_t group);
int64_t kivi_value_param_count(int64_t BH, int64_t S, int64_t D,
                               int64_t group);

/* A static, human-readable name for a status code. */
const char* kivi_status_string(kivi_status status);

#ifdef __cplusplus
}
#endif

#endif /* KIVI_H */
