// C ABI of libkivi.so (declared in include/kivi.h): argument validation and
// dispatch to the HIP kernel launchers.  Everything is checked before any
// launch, so an invalid call writes nothing and enqueues nothing.
#include "kivi.h"

#include <stdint.h>

#include "kivi_launch.h"

#include <atomic>

namespace kivi {

namespace {
thread_local hipEvent_t g_start = nullptr;
thread_local hipEvent_t g_stop = nullptr;
std::atomic<int64_t> g_launches{0};
}  // namespace

void count_launch() { g_launches.fetch_add(1, std::memory_order_relaxed); }

void take_launch_events(hipEvent_t* start, hipEvent_t* stop) {
    *start = g_start;
    *stop = g_stop;
    g_start = nullptr;
    g_stop = nullptr;
}

}  // namespace kivi

namespace {

bool bits_ok(int bits) {
    return bits == 1 || bits == 2 || bits == 4 || bits == 8;
}

bool aligned16(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 15u) == 0;
}

// Shape rules shared by every entry point.
kivi_status check_shape(int64_t BH, int64_t S, int64_t D, int bits,
                        int64_t group) {
    if (!bits_ok(bits)) return KIVI_ERR_BITS;
    if (group < 1) return KIVI_ERR_GROUP;
    if (BH < 0 || S < 0 || D < 0) return KIVI_ERR_SHAPE;
    if (D > (INT64_MAX / 8)) return KIVI_ERR_SHAPE;
    if ((D * bits) % 8 != 0) return KIVI_ERR_SHAPE;
    int64_t n = 0;
    if (__builtin_mul_overflow(BH, S, &n)) return KIVI_ERR_SHAPE;
    if (__builtin_mul_overflow(n, D, &n)) return KIVI_ERR_SHAPE;
    if (__builtin_mul_overflow(n, (int64_t)2, &n)) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

bool empty(int64_t BH, int64_t S, int64_t D) {
    return BH == 0 || S == 0 || D == 0;
}

bool dtype_ok(int dt) { return dt == KIVI_FP16 || dt == KIVI_BF16; }

kivi_status launched(hipError_t e) {
    return e == hipSuccess ? KIVI_OK : KIVI_ERR_LAUNCH;
}

// Common checks of the quantize family.  need_q: codes/scale/zero must be
// given; need_r: recon must be given; q_optional: codes/scale/zero may be
// all NULL or all non-NULL.
kivi_status check_quant(const void* x, int dt, int64_t BH, int64_t S,
                        int64_t D, int bits, int64_t group,
                        const uint8_t* codes, const float* scale,
                        const float* zero, const void* recon, bool need_q,
                        bool need_r, bool q_optional, bool* is_empty) {
    kivi_status st = check_shape(BH, S, D, bits, group);
    if (st != KIVI_OK) return st;
    if (!dtype_ok(dt)) return KIVI_ERR_DTYPE;
    *is_empty = empty(BH, S, D);
    if (*is_empty) return KIVI_OK;
    const int nq = (codes != nullptr) + (scale != nullptr) + (zero != nullptr);
    if (x == nullptr) return KIVI_ERR_NULL;
    if (need_q && nq != 3) return KIVI_ERR_NULL;
    if (q_optional && nq != 0 && nq != 3) return KIVI_ERR_NULL;
    if (need_r && recon == nullptr) return KIVI_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scale) ||
        !aligned16(zero) || !aligned16(recon))
        return KIVI_ERR_ALIGN;
    return KIVI_OK;
}

kivi_status quant(bool keys, const void* x, kivi_dtype dt, int64_t BH,
                  int64_t S, int64_t D, int bits, int64_t group,
                  uint8_t* codes, float* scale, float* zero, void* recon,
                  bool fused, hipStream_t stream) {
    bool is_empty = false;
    kivi_status st = check_quant(x, dt, BH, S, D, bits, group, codes, scale,
                                 zero, recon, !fused, fused, fused, &is_empty);
    if (st != KIVI_OK || is_empty) return st;
    kivi::QuantJob j{x, (int)dt, BH, S, D, bits, group, codes, scale, zero,
                     fused ? recon : nullptr, stream};
    return launched(keys ? kivi::launch_quant_keys(j)
                         : kivi::launch_quant_values(j));
}

kivi_status dequant(bool keys, const uint8_t* codes, const float* scale,
                    const float* zero, int64_t BH, int64_t S, int64_t D,
                    int bits, int64_t group, kivi_dtype out_dt, void* out,
                    hipStream_t stream) {
    kivi_status st = check_shape(BH, S, D, bits, group);
    if (st != KIVI_OK) return st;
    if (!dtype_ok(out_dt)) return KIVI_ERR_DTYPE;
    if (empty(BH, S, D)) return KIVI_OK;
    if (!codes || !scale || !zero || !out) return KIVI_ERR_NULL;
    if (!aligned16(codes) || !aligned16(scale) || !aligned16(zero) ||
        !aligned16(out))
        return KIVI_ERR_ALIGN;
    kivi::DequantJob j{codes, scale, zero, BH, S, D, bits, group,
                       (int)out_dt, out, stream};
    return launched(keys ? kivi::launch_dequant_keys(j)
                         : kivi::launch_dequant_values(j));
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
    return !__builtin_mul_overflow(a, b, out);
}

// Value groups the register-resident value kernel handles: 8 or 16
// channels, or 32 * 2^k (whole lanes of 32 channels combined by butterflies).
bool value_group_ok(int64_t g) {
    if (g == 8 || g == 16) return true;
    if (g < 32 || g % 32 != 0) return false;
    const int64_t m = g / 32;
    return (m & (m - 1)) == 0;
}

bool pow2_d(int64_t D) {
    return D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256;
}

// Rules of the listed-set entry points (include/kivi.h).
kivi_status check_list(int64_t B, int64_t H, int64_t S, int64_t D, int bits,
                       int64_t group, int64_t n, bool keys) {
    if (!bits_ok(bits)) return KIVI_ERR_BITS;
    if (keys ? (group < 1 || group > 32) : !value_group_ok(group))
        return KIVI_ERR_GROUP;
    if (B < 1 || H < 1 || S < 1 || !pow2_d(D) || n < 0 || n > S)
        return KIVI_ERR_SHAPE;
    int64_t m = 0;
    if (!mul_ok(B, H, &m) || !mul_ok(m, n, &m) || m >= (1ll << 31))
        return KIVI_ERR_SHAPE;
    if (!mul_ok(B, H, &m) || !mul_ok(m, S, &m) || !mul_ok(m, D, &m) ||
        m >= (1ll << 40) || S >= (1ll << 31))
        return KIVI_ERR_SHAPE;
    // key kernels: up to 4 lanes per (bh, group, 8 channels), 32-bit counts
    if (keys && (!mul_ok(B * H, (n + group - 1) / group, &m) ||
                 !mul_ok(m, D, &m) || m >= (1ll << 33)))
        return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

// Every rule of kivi_cache_append's contract (include/kivi.h), checked
// before anything is enqueued.
kivi_status check_cache(const kivi_cache* c, const void* k_new,
                        const void* v_new, int64_t n) {
    if (c == nullptr) return KIVI_ERR_NULL;
    if (!bits_ok(c->bits)) return KIVI_ERR_BITS;
    if (c->G_k < 1 || c->G_k > 32) return KIVI_ERR_GROUP;
    if (!value_group_ok(c->G_v)) return KIVI_ERR_GROUP;
    if (!dtype_ok(c->dtype)) return KIVI_ERR_DTYPE;
    const int64_t D = c->D;
    if (!(D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256))
        return KIVI_ERR_SHAPE;
    if (c->BH < 0 || c->R < 0 || c->S_max < 0 || n < 0) return KIVI_ERR_SHAPE;
    if (c->S_max >= (1ll << 31) || c->ring >= (1ll << 31) ||
        c->ring % c->G_k != 0 || c->ring < c->R + c->G_k)
        return KIVI_ERR_SHAPE;
    int64_t cells = 0;   // bounds the kernels' 32-bit lane and row indices
    if (!mul_ok(c->BH, c->S_max, &cells) || !mul_ok(cells, D / 2, &cells) ||
        cells >= (1ll << 32))
        return KIVI_ERR_SHAPE;
    if (!mul_ok(c->BH, c->ring, &cells) || !mul_ok(cells, D, &cells))
        return KIVI_ERR_SHAPE;
    if (c->Q < 0 || c->Q > c->T || c->T > c->S_max || c->Q % c->G_k != 0 ||
        c->T - c->Q >= c->ring)
        return KIVI_ERR_SHAPE;
    if (n > c->S_max - c->T) return KIVI_ERR_SHAPE;
    const void* bufs[] = {c->k_ring, c->v_ring, c->k_codes, c->v_codes,
                          c->k_scale, c->k_zero, c->v_scale, c->v_zero};
    for (const void* b : bufs)
        if (b == nullptr) return KIVI_ERR_NULL;
    if (n > 0 && (k_new == nullptr || v_new == nullptr)) return KIVI_ERR_NULL;
    for (const void* b : bufs)
        if (!aligned16(b)) return KIVI_ERR_ALIGN;
    if (!aligned16(k_new) || !aligned16(v_new)) return KIVI_ERR_ALIGN;
    return KIVI_OK;
}

// kivi_cache_attend's extra rules on top of a valid cache struct.
kivi_status check_attend(const kivi_cache* c, int64_t n_q) {
    kivi_status st = check_cache(c, nullptr, nullptr, 0);
    if (st != KIVI_OK) return st;
    if (!(c->D == 64 || c->D == 128) || c->D * c->bits < 128)
        return KIVI_ERR_SHAPE;
    if (!(c->G_k == 8 || c->G_k == 16 || c->G_k == 32)) return KIVI_ERR_GROUP;
    if (n_q < 1 || n_q > 8 || c->T < 1 || c->BH >= 65536) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

// Rules shared by the KIVI-Sink entry points (include/kivi.h).
kivi_status check_sink(int64_t B, int64_t H, int64_t S, int64_t D,
                       int64_t n_sink) {
    if (B < 1 || H < 1 || S < 1 || D < 8) return KIVI_ERR_SHAPE;
    if (n_sink < 0 || n_sink > 64 || n_sink > S) return KIVI_ERR_SHAPE;
    int64_t n = 0;
    if (!mul_ok(B, H, &n) || !mul_ok(n, S, &n) || !mul_ok(n, D, &n) ||
        n >= (1ll << 40))
        return KIVI_ERR_SHAPE;
    if (!mul_ok(B, S, &n) || n >= (1ll << 31)) return KIVI_ERR_SHAPE;
    return KIVI_OK;
}

bool aligned4(const void* p) {
    return (reinterpret_cast<uintptr_t>(p) & 3u) == 0;
}

kivi_status sink_copy(bool gather, const void* src, int64_t B, int64_t H,
                      int64_t S, int64_t D, const int32_t* idx,
                      int64_t n_sink, void* dst, hipStream_t stream) {
    kivi_status st = check_sink(B, H, S, D, n_sink);
    if (st != KIVI_OK) return st;
    if (D % 8 != 0 || B * H * n_sink * (D / 8) >= (1ll << 32))
        return KIVI_ERR_SHAPE;
    if (n_sink == 0) return KIVI_OK;
    if (!src || !dst || !idx) return KIVI_ERR_NULL;
    if (!aligned16(src) || !aligned16(dst) || !aligned4(idx))
        return KIVI_ERR_ALIGN;
    return launched(kivi::launch_sink_copy(gather, src, dst, B, H, S, D, idx,
                                           n_sink, stream));
}

kivi_status quant_rows(bool keys, const void* x, kivi_dtype dt, int64_t B,
                       int64_t H, int64_t S, int64_t D, int bits,
                       int64_t group, const int32_t* pos, int64_t n,
                       uint8_t* codes, float* scale, float* zero,
                       hipStream_t stream) {
    kivi_status st = check_list(B, H, S, D, bits, group, n, keys);
    if (st != KIVI_OK) return st;
    if (!dtype_ok(dt)) return KIVI_ERR_DTYPE;
    if (n == 0) return KIVI_OK;
    if (!x || !pos || !codes || !scale || !zero) return KIVI_ERR_NULL;
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scale) ||
        !aligned16(zero) || !aligned4(pos))
        return KIVI_ERR_ALIGN;
    kivi::ListJob j{x, (int)dt, B, H, S, D, bits, group, pos, n, codes, scale,
                    zero, stream};
    return launched(keys ? kivi::launch_list_quant_keys(j)
                         : kivi::launch_list_quant_values(j));
}

kivi_status dequant_rows(bool keys, const uint8_t* codes, const float* scale,
                         const float* zero, int64_t B, int64_t H, int64_t S,
                         int64_t D, int bits, int64_t group,
                         const int32_t* pos, int64_t n, kivi_dtype out_dt,
                         void* out, hipStream_t stream) {
    kivi_status st = check_list(B, H, S, D, bits, group, n, keys);
    if (st != KIVI_OK) return st;
    if (!dtype_ok(out_dt)) return KIVI_ERR_DTYPE;
    if (n == 0) return KIVI_OK;
    if (!codes || !scale || !zero || !pos || !out) return KIVI_ERR_NULL;
    if (!aligned16(codes) || !aligned16(scale) || !aligned16(zero) ||
        !aligned16(out) || !aligned4(pos))
        return KIVI_ERR_ALIGN;
    kivi::ListJob j{nullptr, (int)out_dt, B, H, S, D, bits, group, pos, n,
                    const_cast<uint8_t*>(codes), const_cast<float*>(scale),
                    const_cast<float*>(zero), stream};
    return launched(kivi::launch_list_dequant(j, keys, out));
}

}  // namespace

extern "C" {

kivi_status kivi_partition_top(const float* score, int64_t B, int64_t S,
                               int64_t n_hi, int32_t* pos_hi, int32_t* pos_lo,
                               hipStream_t stream) {
    if (B < 1 || S < 1 || S >= (1ll << 31) || B >= (1ll << 31) || n_hi < 0 ||
        n_hi > S)
        return KIVI_ERR_SHAPE;
    if (!score || (n_hi > 0 && !pos_hi) || (n_hi < S && !pos_lo))
        return KIVI_ERR_NULL;
    if (!aligned4(score) || !aligned4(pos_hi) || !aligned4(pos_lo))
        return KIVI_ERR_ALIGN;
    return launched(kivi::launch_partition_top(score, B, S, n_hi, pos_hi,
                                               pos_lo, stream));
}

kivi_status kivi_quant_keys_rows(const void* k, kivi_dtype dt, int64_t B,
                                 int64_t H, int64_t S, int64_t D, int bits,
                                 int64_t group, const int32_t* pos, int64_t n,
                                 uint8_t* codes, float* scale, float* zero,
                                 hipStream_t stream) {
    return quant_rows(true, k, dt, B, H, S, D, bits, group, pos, n, codes,
                      scale, zero, stream);
}

kivi_status kivi_quant_values_rows(const void* v, kivi_dtype dt, int64_t B,
                                   int64_t H, int64_t S, int64_t D, int bits,
                                   int64_t group, const int32_t* pos,
                                   int64_t n, uint8_t* codes, float* scale,
                                   float* zero, hipStream_t stream) {
    return quant_rows(false, v, dt, B, H, S, D, bits, group, pos, n, codes,
                      scale, zero, stream);
}

kivi_status kivi_dequant_keys_rows(const uint8_t* codes, const float* scale,
                                   const float* zero, int64_t B, int64_t H,
                                   int64_t S, int64_t D, int bits,
                                   int64_t group, const int32_t* pos,
                                   int64_t n, kivi_dtype out_dt, void* out,
                                   hipStream_t stream) {
    return dequant_rows(true, codes, scale, zero, B, H, S, D, bits, group, pos,
                        n, out_dt, out, stream);
}

kivi_status kivi_dequant_values_rows(const uint8_t* codes, const float* scale,
                                     const float* zero, int64_t B, int64_t H,
                                     int64_t S, int64_t D, int bits,
                                     int64_t group, const int32_t* pos,
                                     int64_t n, kivi_dtype out_dt, void* out,
                                     hipStream_t stream) {
    return dequant_rows(false, codes, scale, zero, B, H, S, D, bits, group,
                        pos, n, out_dt, out, stream);
}

kivi_status kivi_sink_select(const void* k, kivi_dtype dt, int64_t B,
                             int64_t H, int64_t S, int64_t D, int64_t n_sink,
                             float* score, int32_t* idx, hipStream_t stream) {
    kivi_status st = check_sink(B, H, S, D, n_sink);
    if (st != KIVI_OK) return st;
    if (!(D == 8 || D == 16 || D == 32 || D == 64 || D == 128 || D == 256))
        return KIVI_ERR_SHAPE;
    if (!dtype_ok(dt)) return KIVI_ERR_DTYPE;
    if (!k || !score || (n_sink > 0 && !idx)) return KIVI_ERR_NULL;
    if (!aligned16(k) || !aligned4(score) || !aligned4(idx))
        return KIVI_ERR_ALIGN;
    if (kivi::launch_sink_scores(k, (int)dt, B, H, S, D, score, stream) !=
        hipSuccess)
        return KIVI_ERR_LAUNCH;
    if (n_sink == 0) return KIVI_OK;
    return launched(kivi::launch_sink_select(score, B, S, n_sink, idx, stream));
}

kivi_status kivi_quant_keys_sink(const void* k, kivi_dtype dt, int64_t B,
                                 int64_t H, int64_t S, int64_t D, int bits,
                                 int64_t group, const int32_t* idx,
                                 int64_t n_sink, uint8_t* codes, float* scale,
                                 float* zero, void* recon, hipStream_t stream) {
    if (!bits_ok(bits)) return KIVI_ERR_BITS;
    if (group < 1 || group > 32) return KIVI_ERR_GROUP;
    kivi_status st = check_sink(B, H, S, D, n_sink);
    if (st != KIVI_OK) return st;
    if (D % 8 != 0) return KIVI_ERR_SHAPE;
    if (B * H * ((S + group - 1) / group) * (D / 8) >= (1ll << 32))
        return KIVI_ERR_SHAPE;
    if (!dtype_ok(dt)) return KIVI_ERR_DTYPE;
    const int nq = (codes != nullptr) + (scale != nullptr) + (zero != nullptr);
    if (!k || (nq != 0 && nq != 3) || (nq == 0 && !recon) ||
        (n_sink > 0 && !idx))
        return KIVI_ERR_NULL;
    if (!aligned16(k) || !aligned16(codes) || !aligned16(scale) ||
        !aligned16(zero) || !aligned16(recon) || !aligned4(idx))
        return KIVI_ERR_ALIGN;
    kivi::SinkQuantJob j{k, (int)dt, B, H, S, D, bits, group, idx, n_sink,
                         codes, scale, zero, recon, stream};
    return launched(kivi::launch_quant_keys_sink(j));
}

kivi_status kivi_sink_gather(const void* x, int64_t B, int64_t H, int64_t S,
                             int64_t D, const int32_t* idx, int64_t n_sink,
                             void* x_sink, hipStream_t stream) {
    return sink_copy(true, x, B, H, S, D, idx, n_sink, x_sink, stream);
}

kivi_status kivi_sink_restore(const void* x_sink, int64_t B, int64_t H,
                              int64_t S, int64_t D, const int32_t* idx,
                              int64_t n_sink, void* out, hipStream_t stream) {
    return sink_copy(false, x_sink, B, H, S, D, idx, n_sink, out, stream);
}

kivi_status kivi_quant_keys(const void* k, kivi_dtype dt, int64_t BH,
                            int64_t S, int64_t D, int bits, int64_t group,
                            uint8_t* codes, float* scale, float* zero,
                            hipStream_t stream) {
    return quant(true, k, dt, BH, S, D, bits, group, codes, scale, zero,
                 nullptr, false, stream);
}

kivi_status kivi_quant_values(const void* v, kivi_dtype dt, int64_t BH,
                              int64_t S, int64_t D, int bits, int64_t group,
                              uint8_t* codes, float* scale, float* zero,
                              hipStream_t stream) {
    return quant(false, v, dt, BH, S, D, bits, group, codes, scale, zero,
                 nullptr, false, stream);
}

kivi_status kivi_quant_dequant_keys(const void* k, kivi_dtype dt, int64_t BH,
                                    int64_t S, int64_t D, int bits,
                                    int64_t group, uint8_t* codes,
                                    float* scale, float* zero, void* recon,
                                    hipStream_t stream) {
    return quant(true, k, dt, BH, S, D, bits, group, codes, scale, zero,
                 recon, true, stream);
}

kivi_status kivi_quant_dequant_values(const void* v, kivi_dtype dt,
                                      int64_t BH, int64_t S, int64_t D,
                                      int bits, int64_t group, uint8_t* codes,
                                      float* scale, float* zero, void* recon,
                                      hipStream_t stream) {
    return quant(false, v, dt, BH, S, D, bits, group, codes, scale, zero,
                 recon, true, stream);
}

// Both halves of a K+V call checked (each by the single call's rules)
// before anything is launched.
static kivi_status quant_kv(const void* k, const void* v, kivi_dtype dt,
                            int64_t BH, int64_t S, int64_t D, int bits,
                            int64_t group_k, int64_t group_v, uint8_t* kc,
                            float* ks, float* kz, uint8_t* vc, float* vs,
                            float* vz, void* kr, void* vr, bool fused,
                            hipStream_t stream) {
    bool ek = false, ev = false;
    kivi_status st = check_quant(k, dt, BH, S, D, bits, group_k, kc, ks, kz, kr,
                                 !fused, fused, fused, &ek);
    if (st != KIVI_OK) return st;
    st = check_quant(v, dt, BH, S, D, bits, group_v, vc, vs, vz, vr, !fused,
                     fused, fused, &ev);
    if (st != KIVI_OK) return st;
    if ((kc == nullptr) != (vc == nullptr)) return KIVI_ERR_NULL;
    if (ek) return KIVI_OK;   // same shape: both empty
    kivi::QuantJob jk{k, (int)dt, BH, S, D, bits, group_k, kc, ks, kz,
                      fused ? kr : nullptr, stream};
    kivi::QuantJob jv{v, (int)dt, BH, S, D, bits, group_v, vc, vs, vz,
                      fused ? vr : nullptr, stream};
    return launched(kivi::launch_quant_kv(jk, jv));
}

kivi_status kivi_quant_kv(const void* k, const void* v, kivi_dtype dt,
                          int64_t BH, int64_t S, int64_t D, int bits,
                          int64_t group_k, int64_t group_v, uint8_t* k_codes,
                          float* k_scale, float* k_zero, uint8_t* v_codes,
                          float* v_scale, float* v_zero, hipStream_t stream) {
    return quant_kv(k, v, dt, BH, S, D, bits, group_k, group_v, k_codes,
                    k_scale, k_zero, v_codes, v_scale, v_zero, nullptr, nullptr,
                    false, stream);
}

kivi_status kivi_quant_dequant_kv(const void* k, const void* v, kivi_dtype dt,
                                  int64_t BH, int64_t S, int64_t D, int bits,
                                  int64_t group_k, int64_t group_v,
                                  uint8_t* k_codes, float* k_scale,
                                  float* k_zero, uint8_t* v_codes,
                                  float* v_scale, float* v_zero, void* k_recon,
                                  void* v_recon, hipStream_t stream) {
    return quant_kv(k, v, dt, BH, S, D, bits, group_k, group_v, k_codes,
                    k_scale, k_zero, v_codes, v_scale, v_zero, k_recon, v_recon,
                    true, stream);
}

kivi_status kivi_dequant_kv(const uint8_t* k_codes, const float* k_scale,
                            const float* k_zero, const uint8_t* v_codes,
                            const float* v_scale, const float* v_zero,
                            int64_t BH, int64_t S, int64_t D, int bits,
                            int64_t group_k, int64_t group_v, kivi_dtype out_dt,
                            void* k_out, void* v_out, hipStream_t stream) {
    kivi_status st = check_shape(BH, S, D, bits, group_k);
    if (st != KIVI_OK) return st;
    st = check_shape(BH, S, D, bits, group_v);
    if (st != KIVI_OK) return st;
    if (!dtype_ok(out_dt)) return KIVI_ERR_DTYPE;
    if (empty(BH, S, D)) return KIVI_OK;
    if (!k_codes || !k_scale || !k_zero || !k_out || !v_codes || !v_scale ||
        !v_zero || !v_out)
        return KIVI_ERR_NULL;
    if (!aligned16(k_codes) || !aligned16(k_scale) || !aligned16(k_zero) ||
        !aligned16(k_out) || !aligned16(v_codes) || !aligned16(v_scale) ||
        !aligned16(v_zero) || !aligned16(v_out))
        return KIVI_ERR_ALIGN;
    kivi::DequantJob jk{k_codes, k_scale, k_zero, BH, S, D, bits, group_k,
                        (int)out_dt, k_out, stream};
    kivi::DequantJob jv{v_codes, v_scale, v_zero, BH, S, D, bits, group_v,
                        (int)out_dt, v_out, stream};
    return launched(kivi::launch_dequant_kv(jk, jv));
}

kivi_status kivi_dequant_keys(const uint8_t* codes, const float* scale,
                              const float* zero, int64_t BH, int64_t S,
                              int64_t D, int bits, int64_t group,
                              kivi_dtype out_dt, void* out,
                              hipStream_t stream) {
    return dequant(true, codes, scale, zero, BH, S, D, bits, group, out_dt,
                   out, stream);
}

kivi_status kivi_dequant_values(const uint8_t* codes, const float* scale,
                                const float* zero, int64_t BH, int64_t S,
                                int64_t D, int bits, int64_t group,
                                kivi_dtype out_dt, void* out,
                                hipStream_t stream) {
    return dequant(false, codes, scale, zero, BH, S, D, bits, group, out_dt,
                   out, stream);
}

kivi_status kivi_cache_append(kivi_cache* c, const void* k_new,
                              const void* v_new, int64_t n,
                              hipStream_t stream) {
    kivi_status st = check_cache(c, k_new, v_new, n);
    if (st != KIVI_OK) return st;
    const int64_t T_new = c->T + n;
    const int64_t Q_new =
        T_new >= c->R ? c->G_k * ((T_new - c->R) / c->G_k) : 0;
    const int64_t Q_to = Q_new > c->Q ? Q_new : c->Q;
    bool flush = false, one_launch = false;
    kivi::CacheFlushJob fk{}, fvv{};
    if (c->BH > 0 && Q_to > c->Q) {
        // flush tokens [Q, Q_to): keys per channel, values per token
        kivi::CacheFlushJob f{c->k_ring, k_new, (int)c->dtype, c->BH, c->D,
                              c->ring, n, c->T, c->Q, Q_to - c->Q, c->S_max,
                              (int)c->bits, c->G_k, c->G_k, c->k_codes,
                              c->k_scale, c->k_zero, stream};
        kivi::CacheFlushJob fv = f;
        fv.ring = c->v_ring;
        fv.in = v_new;
        fv.group = c->G_v;
        fv.codes = c->v_codes;
        fv.scale = c->v_scale;
        fv.zero = c->v_zero;
        flush = true;
        one_launch = kivi::cache_append_fits(f, fv);
        if (one_launch) {
            fk = f;
            fvv = fv;
        } else if (kivi::launch_cache_flush_kv(f, fv) != hipSuccess) {
            return KIVI_ERR_LAUNCH;
        }
    }
    // The new tokens that stay unquantized go to their ring slots.  The
    // flush reads the ring slots of tokens [Q, min(Q_to, T)); a new token s
    // shares a slot with one of them only if s - Q >= ring, so when
    // T_new - Q <= ring (every decode-time append) or no flushed token comes
    // from the ring (T == Q), the copy runs in the flush's own launch;
    // otherwise it is a launch of its own after the flush, on the same stream.
    const int64_t s_first = Q_to > c->T ? Q_to : c->T;
    const bool copy = c->BH > 0 && T_new > s_first;
    const kivi::RingStore rs =
        copy ? kivi::make_ring_store(k_new, v_new, c->k_ring, c->v_ring, c->BH,
                                     c->D, n, c->T, s_first, c->ring)
             : kivi::RingStore{};
    if (flush && one_launch) {
        const bool together = copy && (T_new - c->Q <= c->ring || c->T == c->Q);
        if (kivi::launch_cache_append(fk, fvv, together ? &rs : nullptr) !=
            hipSuccess)
            return KIVI_ERR_LAUNCH;
        if (copy && !together &&
            kivi::launch_ring_store(rs, stream) != hipSuccess)
            return KIVI_ERR_LAUNCH;
    } else if (copy && kivi::launch_ring_store(rs, stream) != hipSuccess) {
        return KIVI_ERR_LAUNCH;
    }
    c->T = T_new;
    c->Q = Q_to;
    return KIVI_OK;
}

int64_t kivi_cache_attend_work_bytes(const kivi_cache* c, int64_t n_q) {
    if (check_attend(c, n_q) != KIVI_OK) return -1;
    return kivi::attend_work_floats(c->BH, c->T, c->D, n_q) * 4;
}

namespace {

kivi_status attend_launch(const kivi_cache* c, const void* q, int64_t n_q,
                          float sm_scale, void* out, float* work,
                          hipStream_t stream) {
    kivi::AttendArgs a{
        c->k_codes, c->k_scale, c->k_zero, c->v_codes, c->v_scale, c->v_zero,
        static_cast<const uint16_t*>(c->k_ring),
        static_cast<const uint16_t*>(c->v_ring),
        static_cast<const uint16_t*>(q), static_cast<uint16_t*>(out),
        work, (int32_t)c->D, (int32_t)c->S_max,
        (int32_t)c->ring, (int32_t)c->G_k, (int32_t)c->G_v,
        (int32_t)((c->S_max + c->G_k - 1) / c->G_k),
        (int32_t)((c->D + c->G_v - 1) / c->G_v), (int32_t)c->T, (int32_t)c->Q,
        (int32_t)n_q, (int32_t)kivi::attend_chunks(c->T), sm_scale};
    return launched(kivi::launch_attend(a, c->BH, c->dtype, c->bits, stream));
}

}  // namespace

kivi_status kivi_cache_attend(const kivi_cache* c, const void* q, int64_t n_q,
                              float sm_scale, void* out, void* work,
                              int64_t work_bytes, hipStream_t stream) {
    kivi_status st = check_attend(c, n_q);
    if (st != KIVI_OK) return st;
    if (q == nullptr || out == nullptr || work == nullptr) return KIVI_ERR_NULL;
    if (!aligned16(q) || !aligned16(out) || !aligned16(work))
        return KIVI_ERR_ALIGN;
    if (work_bytes < kivi::attend_work_floats(c->BH, c->T, c->D, n_q) * 4)
        return KIVI_ERR_SHAPE;
    if (c->BH == 0) return KIVI_OK;
    return attend_launch(c, q, n_q, sm_scale, out, static_cast<float*>(work),
                         stream);
}

kivi_status kivi_cache_attend_noalloc(const kivi_cache* c, const void* q,
                                      int64_t n_q, float sm_scale, void* out,
                                      hipStream_t stream) {
    kivi_status st = check_attend(c, n_q);
    if (st != KIVI_OK) return st;
    if (q == nullptr || out == nullptr) return KIVI_ERR_NULL;
    if (!aligned16(q) || !aligned16(out)) return KIVI_ERR_ALIGN;
    if (kivi::attend_work_floats(c->BH, c->T, c->D, n_q) * 4 >
        kivi::attend_scratch_bytes())
        return KIVI_ERR_SCRATCH;
    if (c->BH == 0) return KIVI_OK;
    float* work = nullptr;
    if (kivi::attend_scratch(&work) != hipSuccess) return KIVI_ERR_LAUNCH;
    return attend_launch(c, q, n_q, sm_scale, out, work, stream);
}

int64_t kivi_launch_count(void) {
    return kivi::g_launches.load(std::memory_order_relaxed);
}

void kivi_time_next_launch(hipEvent_t start, hipEvent_t stop) {
    kivi::g_start = start;
    kivi::g_stop = stop;
}

kivi_status kivi_selftest_division(unsigned long long* mismatches,
                                   hipStream_t stream) {
    if (mismatches == nullptr) return KIVI_ERR_NULL;
    if ((reinterpret_cast<uintptr_t>(mismatches) & 7u) != 0)
        return KIVI_ERR_ALIGN;
    return launched(kivi::launch_selftest_division(mismatches, stream));
}

int64_t kivi_codes_bytes(int64_t BH, int64_t S, int64_t D, int bits) {
    if (check_shape(BH, S, D, bits, 1) != KIVI_OK) return -1;
    return BH * S * (D * bits / 8);
}

int64_t kivi_key_param_count(int64_t BH, int64_t S, int64_t D,
                             int64_t group) {
    if (check_shape(BH, S, D, 8, group) != KIVI_OK) return -1;
    return BH * ((S + group - 1) / group) * D;
}

int64_t kivi_value_param_count(int64_t BH, int64_t S, int64_t D,
                               int64_t group) {
    if (check_shape(BH, S, D, 8, group) != KIVI_OK) return -1;
    return BH * S * ((D + group - 1) / group);
}

const char* kivi_status_string(kivi_status status) {
    switch (status) {
        case KIVI_OK: return "ok";
        case KIVI_ERR_NULL: return "a required pointer is NULL";
        case KIVI_ERR_SHAPE: return "invalid shape (negative, overflowing, or D*bits not a multiple of 8)";
        case KIVI_ERR_BITS: return "bits must be 1, 2, 4 or 8";
        case KIVI_ERR_GROUP: return "group must be >= 1";
        case KIVI_ERR_DTYPE: return "dtype must be KIVI_FP16 or KIVI_BF16";
        case KIVI_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case KIVI_ERR_LAUNCH: return "kernel launch failed";
        case KIVI_ERR_SCRATCH: return "the call needs more workspace than the library's fixed per-device buffer (KIVI_ATTEND_SCRATCH_BYTES)";
    }
    return "unknown status";
}

}  // extern "C"
