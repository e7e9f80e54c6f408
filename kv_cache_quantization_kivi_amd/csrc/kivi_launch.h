// Internal interface between the C ABI (kivi_api.cpp) and the kernel
// launchers.  Arguments are validated by the caller; launchers only choose a
// kernel and a grid and enqueue it on the given stream.
#pragma once

#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kivi {

// Events armed by kivi_time_next_launch for the calling thread's next
// launch; take_launch_events hands them over once and disarms them.
void take_launch_events(hipEvent_t* start, hipEvent_t* stop);

// Counts every launch (kivi_launch_count).
void count_launch();

// Every kernel of the library is launched through here: with armed events
// the launch records them at the dispatch's start and end
// (hipExtLaunchKernel), so they time the kernel alone.
template <typename... Params, typename... Args>
hipError_t launch_kernel(void (*kernel)(Params...), dim3 grid, dim3 block,
                         uint32_t shmem, hipStream_t stream, Args... args) {
    count_launch();
    hipEvent_t start = nullptr, stop = nullptr;
    take_launch_events(&start, &stop);
    if (start != nullptr && stop != nullptr)
        hipExtLaunchKernelGGL(kernel, grid, block, shmem, stream, start, stop,
                              0, static_cast<Params>(args)...);
    else
        hipLaunchKernelGGL(kernel, grid, block, shmem, stream,
                           static_cast<Params>(args)...);
    return hipGetLastError();
}

// Smallest l with 2^l >= n (host-side launch helper).
inline uint32_t log2_ceil(uint64_t n) {
    uint32_t l = 0;
    while ((1ull << l) < n) ++l;
    return l;
}

struct QuantJob {
    const void* x;        // [BH, S, D] 16-bit input
    int dtype;            // 0 fp16, 1 bf16
    int64_t BH, S, D;
    int bits;
    int64_t group;
    uint8_t* codes;       // may be null only when recon-only
    float* scale;
    float* zero;
    void* recon;          // null unless fused; same dtype as x
    hipStream_t stream;
};

struct DequantJob {
    const uint8_t* codes;
    const float* scale;
    const float* zero;
    int64_t BH, S, D;
    int bits;
    int64_t group;
    int out_dtype;
    void* out;
    hipStream_t stream;
};

// One flush of a residual-window cache: tokens [Q, Q + F) of every bh, where
// token s < T sits in ring slot s % ring_len of [BH, ring_len, D] and token
// s >= T is row s - T of the appended [BH, n_in, D]; codes and params go to
// the compressed store ([BH, S_max, ...]) at the tokens' own offsets.  Q and
// F are multiples of the key group G_k; D / 8 is a power of two <= 32.
struct CacheFlushJob {
    const void* ring;
    const void* in;
    int dtype;
    int64_t BH, D, ring_len, n_in, T, Q, F, S_max;
    int bits;
    int64_t G_k;          // key group (the flush unit)
    int64_t group;        // this tensor's group: G_k for keys, G_v for values
    uint8_t* codes;
    float* scale;
    float* zero;
    hipStream_t stream;
};

// Decode attention over a residual-window cache (attend.hip); the caller has
// checked D in {64, 128}, D * bits >= 128, G_k in {8, 16, 32},
// 1 <= n_q <= 8, T >= 1, BH < 65536 and the workspace size
// (attend_work_floats floats).
struct AttendArgs {
    const uint8_t* k_codes;
    const float* k_scale;
    const float* k_zero;
    const uint8_t* v_codes;
    const float* v_scale;
    const float* v_zero;
    const uint16_t* k_ring;
    const uint16_t* v_ring;
    const uint16_t* q;     // [BH, n_q, D]
    uint16_t* out;         // [BH, n_q, D]
    float* work;
    int32_t D, S_max, ring, G_k, G_v, NG, NGD, T, Q, n_q, n_chunks;
    float sm_scale;
    int32_t chunk0;        // first chunk of the token-per-thread kernel
};
int64_t attend_chunks(int64_t T);
// Workspace slot per (bh, chunk, query head): m, l, two unused floats, then
// the D partial outputs (16-byte aligned for whole-vector stores).
constexpr int kAttData = 4;
__host__ __device__ inline int64_t att_slot(int64_t D) { return D + kAttData; }
int64_t attend_work_floats(int64_t BH, int64_t T, int64_t D, int64_t n_q);
// The library-held attention workspace of the current device
// (attend_scratch_bytes bytes): its device address, looked up on the
// device's first call.
hipError_t attend_scratch(float** ptr);
int64_t attend_scratch_bytes();
hipError_t launch_attend(const AttendArgs& a, int64_t BH, int dtype, int bits,
                         hipStream_t stream);
// The matrix-core kernel (attend_mfma.hip) over chunks [0, n_full) of every
// bh; the caller has checked D in {64, 128}, bits <= 4, G_k in {16, 32} and
// a value group of at least 16.
hipError_t launch_attend_mfma(const AttendArgs& a, int64_t BH, int n_full,
                              int dtype, int bits, hipStream_t stream);

// KIVI-Sink (sink.hip).  Keys are [B*H, S, D] with the H heads of
// sequence b at rows b*H .. b*H + H - 1; sink lists are [B, n_sink].  The
// caller has checked D in {8, ..., 256} (a power of two) for the scores,
// D % 8 == 0 and 1 <= group <= 32 for the keys, 1 <= n_sink <= 64 for the
// selection and the copies, and sizes that keep lane indices in 32 bits.
struct SinkQuantJob {
    const void* k;
    int dtype;
    int64_t B, H, S, D;
    int bits;
    int64_t group;
    const int32_t* idx;
    int64_t n_sink;
    uint8_t* codes;       // codes/scale/zero all null or all given
    float* scale;
    float* zero;
    void* recon;          // may be null
    hipStream_t stream;
};
hipError_t launch_sink_scores(const void* k, int dtype, int64_t B, int64_t H,
                              int64_t S, int64_t D, float* score,
                              hipStream_t stream);
hipError_t launch_sink_select(const float* score, int64_t B, int64_t S,
                              int64_t n_sink, int32_t* idx, hipStream_t stream);
hipError_t launch_quant_keys_sink(const SinkQuantJob& j);
// The same on the split key kernel (quant_keys.hip); D / 8 a power of two.
hipError_t launch_split_quant_keys_sink(const SinkQuantJob& j);
hipError_t launch_sink_copy(bool gather, const void* src, void* dst, int64_t B,
                            int64_t H, int64_t S, int64_t D,
                            const int32_t* idx, int64_t n_sink,
                            hipStream_t stream);

// Listed token sets (per-token mixed precision, rows.hip and the list
// launchers of the quantizers).  Keys/values [B*H, S, D]; a list is
// [B, n] positions shared by the H heads of a sequence; outputs are the
// set's rows [B*H, n, ...].  The caller has checked D / 8 a power of two
// <= 32, 1 <= n <= S, B*H*n < 2^31, key groups <= 32 and value groups of
// 8, 16 or a multiple of 32.
struct ListJob {
    const void* x;        // quantize: [B*H, S, D] input
    int dtype;
    int64_t B, H, S, D;
    int bits;
    int64_t group;
    const int32_t* pos;
    int64_t n;
    uint8_t* codes;       // [B*H, n, D*bits/8]
    float* scale;
    float* zero;
    hipStream_t stream;
};
hipError_t launch_list_quant_keys(const ListJob& j);
hipError_t launch_list_quant_values(const ListJob& j);
// Dequantize a set and write each row to its position of out [B*H, S, D]
// (rows listed outside [0, S) are not written).
hipError_t launch_list_dequant(const ListJob& j, bool keys, void* out);
// pos_hi [B, n_hi] and pos_lo [B, S - n_hi], each ascending: the n_hi first
// positions in the order (score descending, position ascending) and the rest.
hipError_t launch_partition_top(const float* score, int64_t B, int64_t S,
                                int64_t n_hi, int32_t* pos_hi, int32_t* pos_lo,
                                hipStream_t stream);

hipError_t launch_quant_keys(const QuantJob& j);
hipError_t launch_quant_values(const QuantJob& j);
hipError_t launch_dequant_keys(const DequantJob& j);
hipError_t launch_dequant_values(const DequantJob& j);
// Keys and values of one flush (validated, same shape, dtype and bits):
// one launch for small flushes, else the two single launches.
hipError_t launch_quant_kv(const QuantJob& k, const QuantJob& v);
hipError_t launch_dequant_kv(const DequantJob& k, const DequantJob& v);
hipError_t launch_cache_flush_keys(const CacheFlushJob& j);
hipError_t launch_cache_flush_values(const CacheFlushJob& j);
// Both tensors of a flush: one launch under the rule of launch_quant_kv
// with four times its item bound (kCacheKvPairBelow), else the key and
// value launches.
hipError_t launch_cache_flush_kv(const CacheFlushJob& k, const CacheFlushJob& v);
// The copy of tokens [s_first, T + n_in) of the appended keys and values
// into their ring slots (ring_store_lane, kivi_rows.h): 2 * half lanes of
// one 16-byte chunk each.
struct RingStore {
    const uint16_t* k_in;    // [BH, n_in, D] appended tokens
    const uint16_t* v_in;
    uint16_t* k_ring;        // [BH, ring_len, D]
    uint16_t* v_ring;
    uint32_t half;           // lanes per tensor: BH * ncopy * D8
    uint32_t D8, ncopy;
    int32_t s_first, T, n_in, ring_len;
};
RingStore make_ring_store(const void* k_in, const void* v_in, void* k_ring,
                          void* v_ring, int64_t BH, int64_t D, int64_t n_in,
                          int64_t T, int64_t s_first, int64_t ring_len);
// The ring store alone, both tensors in one launch.
hipError_t launch_ring_store(const RingStore& r, hipStream_t stream);
// The flush of both tensors and, when ring != nullptr, the ring store in one
// launch (the caller has checked that the ring store writes no slot the
// flush reads); false if the flush does not take the one-launch form
// (nothing is launched then).
bool cache_append_fits(const CacheFlushJob& k, const CacheFlushJob& v);
hipError_t launch_cache_append(const CacheFlushJob& k, const CacheFlushJob& v,
                               const RingStore* ring);

// Fallback kernels for shapes the fast kernels do not cover (keys with
// D % 8 != 0 or group > 32; values with D % 8 != 0, D > 2048 or a group
// other than 8, 16 or a multiple of 32; dequant with D % 8 != 0 or, for
// values, such a group).
hipError_t launch_generic_quant_keys(const QuantJob& j);
hipError_t launch_generic_quant_values(const QuantJob& j);
hipError_t launch_generic_dequant(const DequantJob& j, bool keys);

hipError_t launch_selftest_division(unsigned long long* mismatches,
                                    hipStream_t stream);

}  // namespace kivi
