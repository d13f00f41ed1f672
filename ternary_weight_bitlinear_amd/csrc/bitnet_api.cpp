// bitnet_api.cpp -- the C ABI declared in include/bitnet.h.
//
// Every entry point validates its arguments on the host before any launch and
// reports failures through a status code plus a thread-local message.  The
// device work itself lives in the .hip files behind kernels.h.
//
// The host packer (BITNET_MEM_HOST) is the same WeightQuant + layout-v1 pack
// as the device packer ("BitVLA -- 1.58-bit Vision-Language-Action on Core
// AI", s1 and s2; "BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference
// Optimization Guide", s3.3 "I2_S Ternary Packing"), for converting weights
// offline without a GPU.  It is chosen explicitly by the caller through
// `where`; nothing in the library falls back to it.
#include "../../include/bitnet.h"

#include <cmath>
#include <cstddef>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <vector>

#include "gemv.h"
#include "kernels.h"

namespace {

constexpr int64_t kMaxK = 1 << 20;
constexpr int64_t kMaxMN = 0x7FFFFFFF;
constexpr int64_t kBlockedMaxK = 8192;   // block scales of a 128-column tile staged in LDS
constexpr int64_t kGemvMaxM = 16;
constexpr int64_t kFusedLdsBytes = 32768;     // single call: M * Kp bytes of q in LDS
constexpr int64_t kGroupLdsBytes = 65536;     // grouped launch: M * max Kp
constexpr int64_t kPlanMagic = 0x62746E6770ll;   // "btngp"
static_assert(bitnet::kPackStaticMaxRows == BITNET_PACK_STATIC_MAX_ROWS &&
                  bitnet::kPackStaticMaxSegs == BITNET_PACK_STATIC_MAX_SEGS,
              "limits of the allocation-free pack");

thread_local std::string g_last_error;

bitnet_status_t fail(bitnet_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
bitnet_status_t fail(bitnet_status_t s, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return s;
}

bitnet_status_t ok() {
    g_last_error.clear();
    return BITNET_OK;
}

bitnet_status_t hip_fail(hipError_t e, const char* what) {
    return fail(BITNET_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t padded_k(int64_t K) {
    if (K <= 0 || K % 16 != 0 || K > kMaxK) return -1;
    return (K + 127) / 128 * 128;
}

bool aligned(const void* p, size_t a) { return reinterpret_cast<uintptr_t>(p) % a == 0; }

bitnet_status_t check_dims(const char* fn, int64_t M, int64_t N, int64_t K) {
    if (M <= 0 || M > kMaxMN) return fail(BITNET_ERR_INVALID_ARG, "%s: M=%lld out of range", fn, (long long)M);
    if (N <= 0 || N > kMaxMN) return fail(BITNET_ERR_INVALID_ARG, "%s: N=%lld out of range", fn, (long long)N);
    if (padded_k(K) < 0)
        return fail(BITNET_ERR_INVALID_ARG, "%s: K=%lld must be a positive multiple of 16 and <= %lld", fn,
                    (long long)K, (long long)kMaxK);
    return BITNET_OK;
}

bool valid_dtype(bitnet_dtype_t d) { return d == BITNET_F32 || d == BITNET_BF16; }

// ---------------------------------------------------------------- host packer

float host_load(const void* W, bitnet_dtype_t dt, int64_t idx) {
    if (dt == BITNET_BF16) {
        uint32_t bits = static_cast<uint32_t>(static_cast<const uint16_t*>(W)[idx]) << 16;
        float f;
        std::memcpy(&f, &bits, sizeof f);
        return f;
    }
    return static_cast<const float*>(W)[idx];
}

bitnet_status_t host_pack(const void* W, bitnet_dtype_t dt, int64_t N, int64_t K, int64_t ldw,
                          const std::vector<int64_t>& seg_start, uint8_t* packed, float* w_scale,
                          float* seg_mean, int64_t* zero_count) {
    const int64_t Kp = padded_k(K);
    const int n_segs = static_cast<int>(seg_start.size()) - 1;
    std::vector<double> row_sum(static_cast<size_t>(N));
    for (int64_t n = 0; n < N; ++n) {
        double acc = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            const float v = host_load(W, dt, n * ldw + k);
            if (!std::isfinite(v))
                return fail(BITNET_ERR_NONFINITE, "bitnet_pack_weights: W[%lld][%lld] is not finite",
                            (long long)n, (long long)k);
            acc += std::fabs(static_cast<double>(v));
        }
        row_sum[static_cast<size_t>(n)] = acc;
    }
    const int64_t words_per_row = Kp / 16;
    for (int s = 0; s < n_segs; ++s) {
        double total = 0.0;
        for (int64_t n = seg_start[s]; n < seg_start[s + 1]; ++n) total += row_sum[static_cast<size_t>(n)];
        const int64_t rows = seg_start[s + 1] - seg_start[s];
        const float mean = static_cast<float>(total / static_cast<double>(rows * K));
        const float scale = 1.0f / mean;
        int64_t zeros = 0;
        for (int64_t n = seg_start[s]; n < seg_start[s + 1]; ++n) {
            w_scale[n] = mean;
            for (int64_t j = 0; j < words_per_row; ++j) {
                uint32_t word = 0;
                for (int e = 0; e < 16; ++e) {
                    const int64_t k = 16 * j + e;
                    uint32_t u = 1u;
                    if (k < K) {
                        const float p = host_load(W, dt, n * ldw + k) * scale;
                        const int t = (p > 0.5f) - (p < -0.5f);
                        u = static_cast<uint32_t>(t + 1);
                        zeros += (t == 0);
                    }
                    word |= u << (8 * (e % 4) + 2 * (e / 4));
                }
                uint8_t* dst = packed + n * (Kp / 4) + 4 * j;
                for (int b = 0; b < 4; ++b) dst[b] = static_cast<uint8_t>(word >> (8 * b));
            }
        }
        if (seg_mean) seg_mean[s] = mean;
        if (zero_count) zero_count[s] = zeros;
    }
    return ok();
}

// -------------------------------------------------------------- device packer

struct DeviceTemps {
    hipStream_t stream = nullptr;
    void* p = nullptr;
    ~DeviceTemps() {
        if (p) {
            hipFreeAsync(p, stream);
            hipStreamSynchronize(stream);
        }
    }
};

// Device pack with its temporaries (pack_temp_layout(N, n_segs).bytes) at
// `temps`: upload the segment table, launch, read back the status, the means
// and the zero counts, and wait.
bitnet_status_t device_pack_into(hipStream_t stream, void* temps, const void* W, bitnet_dtype_t dt, int64_t N,
                                 int64_t K, int64_t ldw, const std::vector<int64_t>& seg_start, uint8_t* packed,
                                 float* w_scale, float* seg_mean, int64_t* zero_count, const char* fn) {
    const int64_t Kp = padded_k(K);
    const int n_segs = static_cast<int>(seg_start.size()) - 1;
    const bitnet::PackTemps lay = bitnet::pack_temp_layout(N, n_segs);
    char* base = static_cast<char*>(temps);
    auto* d_row_sum = reinterpret_cast<double*>(base);
    auto* d_start = reinterpret_cast<int64_t*>(base + lay.off_start);
    auto* d_mean = reinterpret_cast<float*>(base + lay.off_mean);
    auto* d_zero = reinterpret_cast<unsigned long long*>(base + lay.off_zero);
    auto* d_status = reinterpret_cast<unsigned int*>(base + lay.off_status);
    hipError_t e;
    char what[96];
    if ((e = hipMemcpyAsync(d_start, seg_start.data(), (n_segs + 1) * sizeof(int64_t), hipMemcpyHostToDevice,
                            stream)) != hipSuccess) {
        snprintf(what, sizeof what, "%s: segment table upload", fn);
        return hip_fail(e, what);
    }
    e = bitnet::launch_pack(W, dt == BITNET_BF16, N, K, ldw, Kp, d_start, n_segs, d_row_sum, d_mean, d_zero,
                            d_status, packed, w_scale, stream);
    if (e != hipSuccess) {
        snprintf(what, sizeof what, "%s: launch", fn);
        return hip_fail(e, what);
    }
    unsigned int status = 0;
    std::vector<float> means(static_cast<size_t>(n_segs));
    std::vector<unsigned long long> zeros(static_cast<size_t>(n_segs));
    if ((e = hipMemcpyAsync(&status, d_status, sizeof status, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
        (e = hipMemcpyAsync(means.data(), d_mean, n_segs * sizeof(float), hipMemcpyDeviceToHost, stream)) !=
            hipSuccess ||
        (e = hipMemcpyAsync(zeros.data(), d_zero, n_segs * sizeof(unsigned long long), hipMemcpyDeviceToHost,
                            stream)) != hipSuccess) {
        snprintf(what, sizeof what, "%s: read-back", fn);
        return hip_fail(e, what);
    }
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) {
        snprintf(what, sizeof what, "%s: sync", fn);
        return hip_fail(e, what);
    }
    if (status & 1u) return fail(BITNET_ERR_NONFINITE, "%s: a weight is not finite", fn);
    for (int s = 0; s < n_segs; ++s) {
        if (seg_mean) seg_mean[s] = means[static_cast<size_t>(s)];
        if (zero_count) zero_count[s] = static_cast<int64_t>(zeros[static_cast<size_t>(s)]);
    }
    return ok();
}

bitnet_status_t device_pack(hipStream_t stream, const void* W, bitnet_dtype_t dt, int64_t N, int64_t K,
                            int64_t ldw, const std::vector<int64_t>& seg_start, uint8_t* packed,
                            float* w_scale, float* seg_mean, int64_t* zero_count) {
    const int n_segs = static_cast<int>(seg_start.size()) - 1;
    DeviceTemps temps;
    temps.stream = stream;
    hipError_t e = hipMallocAsync(&temps.p, bitnet::pack_temp_layout(N, n_segs).bytes, stream);
    if (e != hipSuccess) {
        temps.p = nullptr;
        return hip_fail(e, "bitnet_pack_weights: temporary allocation");
    }
    return device_pack_into(stream, temps.p, W, dt, N, K, ldw, seg_start, packed, w_scale, seg_mean, zero_count,
                            "bitnet_pack_weights");
}

bitnet_status_t check_linear(const int8_t* q, const float* a_scale, const int32_t* q_rowsum, int64_t M,
                             int64_t K, const uint8_t* packed, const float* w_scale, int64_t N, void* y,
                             bitnet_dtype_t y_dtype, int64_t ldy, const char* fn) {
    bitnet_status_t s = check_dims(fn, M, N, K);
    if (s != BITNET_OK) return s;
    if (!q || !a_scale || !q_rowsum || !packed || !w_scale || !y)
        return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (!valid_dtype(y_dtype)) return fail(BITNET_ERR_INVALID_ARG, "%s: bad y dtype %d", fn, (int)y_dtype);
    if (ldy < N) return fail(BITNET_ERR_INVALID_ARG, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
    if (!aligned(q, 16) || !aligned(packed, 16))
        return fail(BITNET_ERR_INVALID_ARG, "%s: q and packed must be 16-byte aligned", fn);
    if (!aligned(y, y_dtype == BITNET_F32 ? 4 : 2) || !aligned(a_scale, 4) || !aligned(w_scale, 4) ||
        !aligned(q_rowsum, 4))
        return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned y or scale pointer", fn);
    return BITNET_OK;
}

bitnet_status_t check_act_quant(const void* x, bitnet_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                const int8_t* q, const float* a_scale, const int32_t* q_rowsum, const char* fn) {
    bitnet_status_t s = check_dims(fn, M, 1, K);
    if (s != BITNET_OK) return s;
    if (!x || !q || !a_scale || !q_rowsum) return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (!valid_dtype(x_dtype)) return fail(BITNET_ERR_INVALID_ARG, "%s: bad x dtype %d", fn, (int)x_dtype);
    if (ldx < K) return fail(BITNET_ERR_INVALID_ARG, "%s: ldx=%lld < K=%lld", fn, (long long)ldx, (long long)K);
    if (!aligned(x, x_dtype == BITNET_F32 ? 4 : 2) || !aligned(q, 16) || !aligned(a_scale, 4) ||
        !aligned(q_rowsum, 4))
        return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned pointer (q must be 16-byte aligned)", fn);
    return BITNET_OK;
}

bitnet_status_t run_linear(hipStream_t stream, const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                           int64_t M, int64_t K, const uint8_t* packed, const float* w_scale, int64_t N, void* y,
                           bitnet_dtype_t y_dtype, int64_t ldy, int32_t* acc_debug, const char* fn) {
    const int64_t Kp = padded_k(K);
    const bool bf16 = y_dtype == BITNET_BF16;
    hipError_t e = (M <= kGemvMaxM)
                       ? bitnet::launch_gemv(q, a_scale, q_rowsum, M, Kp, packed, w_scale, N, y, bf16, ldy,
                                             acc_debug, stream)
                       : bitnet::launch_gemm(q, a_scale, q_rowsum, M, Kp, packed, w_scale, N, y, bf16, ldy,
                                             acc_debug, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

}  // namespace

extern "C" {

int32_t bitnet_abi_version(void) { return BITNET_ABI_VERSION; }

int64_t bitnet_padded_k(int64_t K) { return padded_k(K); }

int64_t bitnet_packed_bytes(int64_t N, int64_t K) {
    const int64_t Kp = padded_k(K);
    if (Kp < 0 || N <= 0 || N > kMaxMN) return -1;
    return N * (Kp / 4);
}

static bitnet_status_t check_pack(const char* fn, const void* W, bitnet_dtype_t w_dtype, int64_t N, int64_t K,
                                  int64_t ldw, const int64_t* seg_rows, int32_t n_segs, const uint8_t* packed,
                                  const float* w_scale, std::vector<int64_t>& seg_start) {
    bitnet_status_t s = check_dims(fn, 1, N, K);
    if (s != BITNET_OK) return s;
    if (!W || !packed || !w_scale) return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (!valid_dtype(w_dtype)) return fail(BITNET_ERR_INVALID_ARG, "%s: bad W dtype %d", fn, (int)w_dtype);
    if (ldw < K) return fail(BITNET_ERR_INVALID_ARG, "%s: ldw=%lld < K=%lld", fn, (long long)ldw, (long long)K);
    if (!aligned(packed, 16) || !aligned(w_scale, 4) || !aligned(W, w_dtype == BITNET_F32 ? 4 : 2))
        return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned pointer (packed must be 16-byte aligned)", fn);
    if (n_segs < 0 || (n_segs > 0 && !seg_rows))
        return fail(BITNET_ERR_INVALID_ARG, "%s: bad segment table", fn);
    seg_start.assign(1, 0);
    if (n_segs == 0 || !seg_rows) {
        seg_start.push_back(N);
    } else {
        for (int32_t i = 0; i < n_segs; ++i) {
            if (seg_rows[i] <= 0)
                return fail(BITNET_ERR_INVALID_ARG, "%s: segment %d has %lld rows", fn, i, (long long)seg_rows[i]);
            seg_start.push_back(seg_start.back() + seg_rows[i]);
            if (seg_start.back() > N) break;
        }
        if (seg_start.back() != N || static_cast<int32_t>(seg_start.size()) != n_segs + 1)
            return fail(BITNET_ERR_INVALID_ARG, "%s: segment rows do not add up to N=%lld", fn, (long long)N);
    }
    return BITNET_OK;
}

bitnet_status_t bitnet_pack_weights(bitnet_mem_t where, hipStream_t stream, const void* W, bitnet_dtype_t w_dtype,
                                    int64_t N, int64_t K, int64_t ldw, const int64_t* seg_rows, int32_t n_segs,
                                    uint8_t* packed, float* w_scale, float* seg_mean, int64_t* zero_count) {
    const char* fn = "bitnet_pack_weights";
    if (where != BITNET_MEM_HOST && where != BITNET_MEM_DEVICE)
        return fail(BITNET_ERR_INVALID_ARG, "%s: bad memory kind %d", fn, (int)where);
    std::vector<int64_t> seg_start;
    bitnet_status_t s = check_pack(fn, W, w_dtype, N, K, ldw, seg_rows, n_segs, packed, w_scale, seg_start);
    if (s != BITNET_OK) return s;
    if (where == BITNET_MEM_HOST) return host_pack(W, w_dtype, N, K, ldw, seg_start, packed, w_scale, seg_mean, zero_count);
    return device_pack(stream, W, w_dtype, N, K, ldw, seg_start, packed, w_scale, seg_mean, zero_count);
}

bitnet_status_t bitnet_pack_weights_static(hipStream_t stream, const void* W, bitnet_dtype_t w_dtype, int64_t N,
                                           int64_t K, int64_t ldw, const int64_t* seg_rows, int32_t n_segs,
                                           uint8_t* packed, float* w_scale, float* seg_mean, int64_t* zero_count) {
    const char* fn = "bitnet_pack_weights_static";
    std::vector<int64_t> seg_start;
    bitnet_status_t s = check_pack(fn, W, w_dtype, N, K, ldw, seg_rows, n_segs, packed, w_scale, seg_start);
    if (s != BITNET_OK) return s;
    const int64_t segs = static_cast<int64_t>(seg_start.size()) - 1;
    if (N > BITNET_PACK_STATIC_MAX_ROWS || segs > BITNET_PACK_STATIC_MAX_SEGS)
        return fail(BITNET_ERR_UNSUPPORTED,
                    "%s: N=%lld rows and %lld segments exceed the fixed temporaries (at most %d rows, %d segments); "
                    "use bitnet_pack_weights",
                    fn, (long long)N, (long long)segs, BITNET_PACK_STATIC_MAX_ROWS, BITNET_PACK_STATIC_MAX_SEGS);
    void* temps = nullptr;
    size_t bytes = 0;
    hipError_t e = bitnet::pack_scratch(&temps, &bytes);
    if (e != hipSuccess) return hip_fail(e, "bitnet_pack_weights_static: scratch address");
    if (bitnet::pack_temp_layout(N, segs).bytes > bytes)
        return fail(BITNET_ERR_UNSUPPORTED, "%s: temporaries exceed the fixed array", fn);
    return device_pack_into(stream, temps, W, w_dtype, N, K, ldw, seg_start, packed, w_scale, seg_mean, zero_count,
                            fn);
}

bitnet_status_t bitnet_act_quant(hipStream_t stream, const void* x, bitnet_dtype_t x_dtype, int64_t M, int64_t K,
                                 int64_t ldx, int8_t* q, float* a_scale, int32_t* q_rowsum) {
    const char* fn = "bitnet_act_quant";
    bitnet_status_t s = check_act_quant(x, x_dtype, M, K, ldx, q, a_scale, q_rowsum, fn);
    if (s != BITNET_OK) return s;
    hipError_t e = bitnet::launch_act_quant(x, x_dtype == BITNET_BF16, M, K, ldx, q, a_scale, q_rowsum,
                                            padded_k(K), stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

static bitnet_status_t check_norm(const void* x, const void* up, bitnet_dtype_t x_dtype, const void* norm_w,
                                  bitnet_dtype_t norm_dtype, float eps, const char* fn) {
    if (!norm_w) return fail(BITNET_ERR_INVALID_ARG, "%s: norm_w is NULL", fn);
    if (!valid_dtype(norm_dtype)) return fail(BITNET_ERR_INVALID_ARG, "%s: bad norm_w dtype %d", fn, (int)norm_dtype);
    if (!aligned(norm_w, norm_dtype == BITNET_F32 ? 4 : 2))
        return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned norm_w", fn);
    if (up && !aligned(up, x_dtype == BITNET_F32 ? 4 : 2)) return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned up", fn);
    if (!(eps >= 0.0f) || !std::isfinite(eps))
        return fail(BITNET_ERR_INVALID_ARG, "%s: eps must be finite and >= 0", fn);
    (void)x;
    return BITNET_OK;
}

bitnet_status_t bitnet_rmsnorm_act_quant(hipStream_t stream, const void* x, const void* up, bitnet_dtype_t x_dtype,
                                         int64_t M, int64_t K, int64_t ldx, const void* norm_w,
                                         bitnet_dtype_t norm_dtype, float eps, int8_t* q, float* a_scale,
                                         int32_t* q_rowsum) {
    const char* fn = "bitnet_rmsnorm_act_quant";
    bitnet_status_t s = check_act_quant(x, x_dtype, M, K, ldx, q, a_scale, q_rowsum, fn);
    if (s != BITNET_OK) return s;
    if ((s = check_norm(x, up, x_dtype, norm_w, norm_dtype, eps, fn)) != BITNET_OK) return s;
    hipError_t e = bitnet::launch_norm_act_quant(x, up, x_dtype == BITNET_BF16, M, K, ldx, norm_w,
                                                 norm_dtype == BITNET_BF16, eps, q, a_scale, q_rowsum,
                                                 padded_k(K), stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

int64_t bitnet_block_count(int64_t K) {
    return padded_k(K) < 0 ? -1 : (K + 255) / 256;
}

bitnet_status_t bitnet_pack_weights_blocked(hipStream_t stream, const void* W, bitnet_dtype_t w_dtype, int64_t N,
                                            int64_t K, int64_t ldw, uint8_t* packed, float* block_scale) {
    const char* fn = "bitnet_pack_weights_blocked";
    bitnet_status_t s = check_dims(fn, 1, N, K);
    if (s != BITNET_OK) return s;
    if (K > kBlockedMaxK) return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld > %lld", fn, (long long)K, (long long)kBlockedMaxK);
    if (!W || !packed || !block_scale) return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (!valid_dtype(w_dtype)) return fail(BITNET_ERR_INVALID_ARG, "%s: bad W dtype %d", fn, (int)w_dtype);
    if (ldw < K) return fail(BITNET_ERR_INVALID_ARG, "%s: ldw=%lld < K=%lld", fn, (long long)ldw, (long long)K);
    if (!aligned(W, w_dtype == BITNET_F32 ? 4 : 2) || !aligned(packed, 16) || !aligned(block_scale, 4))
        return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned pointer (packed must be 16-byte aligned)", fn);
    DeviceTemps temps;
    temps.stream = stream;
    hipError_t e = hipMallocAsync(&temps.p, sizeof(unsigned int), stream);
    if (e != hipSuccess) {
        temps.p = nullptr;
        return hip_fail(e, "bitnet_pack_weights_blocked: temporary allocation");
    }
    auto* d_status = static_cast<unsigned int*>(temps.p);
    if ((e = hipMemsetAsync(d_status, 0, sizeof(unsigned int), stream)) != hipSuccess)
        return hip_fail(e, "bitnet_pack_weights_blocked: status clear");
    e = bitnet::launch_pack_blocked(W, w_dtype == BITNET_BF16, N, K, ldw, padded_k(K), d_status, packed, block_scale,
                                    stream);
    if (e != hipSuccess) return hip_fail(e, "bitnet_pack_weights_blocked: launch");
    unsigned int status = 0;
    if ((e = hipMemcpyAsync(&status, d_status, sizeof status, hipMemcpyDeviceToHost, stream)) != hipSuccess)
        return hip_fail(e, "bitnet_pack_weights_blocked: read-back");
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "bitnet_pack_weights_blocked: sync");
    if (status & 1u) return fail(BITNET_ERR_NONFINITE, "bitnet_pack_weights_blocked: a weight is not finite");
    return ok();
}

bitnet_status_t bitnet_linear_blocked_forward(hipStream_t stream, const int8_t* q, const float* a_scale, int64_t M,
                                              int64_t K, const uint8_t* packed, const float* block_scale, int64_t N,
                                              void* y, bitnet_dtype_t y_dtype, int64_t ldy) {
    const char* fn = "bitnet_linear_blocked_forward";
    bitnet_status_t s = check_dims(fn, M, N, K);
    if (s != BITNET_OK) return s;
    if (K > kBlockedMaxK) return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld > %lld", fn, (long long)K, (long long)kBlockedMaxK);
    if (!q || !a_scale || !packed || !block_scale || !y)
        return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (!valid_dtype(y_dtype)) return fail(BITNET_ERR_INVALID_ARG, "%s: bad y dtype %d", fn, (int)y_dtype);
    if (ldy < N) return fail(BITNET_ERR_INVALID_ARG, "%s: ldy=%lld < N=%lld", fn, (long long)ldy, (long long)N);
    if (!aligned(q, 16) || !aligned(packed, 16))
        return fail(BITNET_ERR_INVALID_ARG, "%s: q and packed must be 16-byte aligned", fn);
    if (!aligned(y, y_dtype == BITNET_F32 ? 4 : 2) || !aligned(a_scale, 4) || !aligned(block_scale, 4))
        return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned y or scale pointer", fn);
    hipError_t e = hipErrorInvalidValue;
    if (M <= kGemvMaxM) {
        // decode sizes: the streaming kernel, one pass over codes and scales
        bitnet::GemvProblem p{};
        p.q = q; p.a_scale = a_scale; p.packed = packed; p.w_scale = block_scale;
        p.y = y; p.ldy = ldy;
        p.M = (int)M; p.N = (int)N; p.K = (int)K; p.Kp = (int)padded_k(K);
        e = bitnet::launch_gemv_blocked(p, y_dtype == BITNET_BF16, stream);
    }
    if (e == hipErrorInvalidValue)          // larger M, or token rows beyond the streaming kernel's LDS
        e = bitnet::launch_gemm_blocked(q, a_scale, M, K, padded_k(K), packed, block_scale, N, y,
                                        y_dtype == BITNET_BF16, ldy, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

bitnet_status_t bitnet_linear_forward(hipStream_t stream, const int8_t* q, const float* a_scale,
                                      const int32_t* q_rowsum, int64_t M, int64_t K, const uint8_t* packed,
                                      const float* w_scale, int64_t N, void* y, bitnet_dtype_t y_dtype, int64_t ldy,
                                      int32_t* acc_debug) {
    const char* fn = "bitnet_linear_forward";
    bitnet_status_t s = check_linear(q, a_scale, q_rowsum, M, K, packed, w_scale, N, y, y_dtype, ldy, fn);
    if (s != BITNET_OK) return s;
    if (acc_debug && !aligned(acc_debug, 4)) return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned acc_debug", fn);
    return run_linear(stream, q, a_scale, q_rowsum, M, K, packed, w_scale, N, y, y_dtype, ldy, acc_debug, fn);
}

static bitnet_status_t bitlinear_impl(hipStream_t stream, const void* x, const void* up, bitnet_dtype_t x_dtype,
                                      int64_t M, int64_t K, int64_t ldx, const void* norm_w,
                                      bitnet_dtype_t norm_dtype, float eps, const uint8_t* packed,
                                      const float* w_scale, int64_t N, void* y, bitnet_dtype_t y_dtype, int64_t ldy,
                                      int8_t* q, float* a_scale, int32_t* q_rowsum, const char* fn) {
    bitnet_status_t s = check_act_quant(x, x_dtype, M, K, ldx, q, a_scale, q_rowsum, fn);
    if (s != BITNET_OK) return s;
    if (norm_w && (s = check_norm(x, up, x_dtype, norm_w, norm_dtype, eps, fn)) != BITNET_OK) return s;
    s = check_linear(q, a_scale, q_rowsum, M, K, packed, w_scale, N, y, y_dtype, ldy, fn);
    if (s != BITNET_OK) return s;
    const int64_t Kp = padded_k(K);
    const int64_t esize = x_dtype == BITNET_BF16 ? 2 : 4;
    const bool fuse = M <= kGemvMaxM && M * Kp <= kFusedLdsBytes && aligned(x, 16) && (ldx * esize) % 16 == 0 &&
                      (!up || aligned(up, 16)) && (!norm_w || aligned(norm_w, 16));
    hipError_t e;
    if (fuse) {
        bitnet::GemvProblem p{};
        p.x = x; p.ldx = ldx;
        p.up = norm_w ? up : nullptr;
        p.norm_w = norm_w; p.eps = eps; p.norm_bf16 = norm_dtype == BITNET_BF16;
        p.q_out = q; p.a_scale_out = a_scale; p.rowsum_out = q_rowsum;
        p.packed = packed; p.w_scale = w_scale; p.y = y; p.ldy = ldy;
        p.M = (int)M; p.N = (int)N; p.K = (int)K; p.Kp = (int)Kp;
        e = bitnet::launch_gemv_fused(p, x_dtype == BITNET_BF16, y_dtype == BITNET_BF16, stream);
        if (e != hipSuccess) return hip_fail(e, fn);
        return ok();
    }
    e = norm_w ? bitnet::launch_norm_act_quant(x, up, x_dtype == BITNET_BF16, M, K, ldx, norm_w,
                                               norm_dtype == BITNET_BF16, eps, q, a_scale, q_rowsum, Kp, stream)
               : bitnet::launch_act_quant(x, x_dtype == BITNET_BF16, M, K, ldx, q, a_scale, q_rowsum, Kp, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return run_linear(stream, q, a_scale, q_rowsum, M, K, packed, w_scale, N, y, y_dtype, ldy, nullptr, fn);
}

bitnet_status_t bitnet_bitlinear_forward(hipStream_t stream, const void* x, bitnet_dtype_t x_dtype, int64_t M,
                                         int64_t K, int64_t ldx, const uint8_t* packed, const float* w_scale,
                                         int64_t N, void* y, bitnet_dtype_t y_dtype, int64_t ldy, int8_t* q,
                                         float* a_scale, int32_t* q_rowsum) {
    return bitlinear_impl(stream, x, nullptr, x_dtype, M, K, ldx, nullptr, BITNET_F32, 0.0f, packed, w_scale, N, y,
                          y_dtype, ldy, q, a_scale, q_rowsum, "bitnet_bitlinear_forward");
}

bitnet_status_t bitnet_rmsnorm_bitlinear_forward(hipStream_t stream, const void* x, const void* up,
                                                 bitnet_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                                 const void* norm_w, bitnet_dtype_t norm_dtype, float eps,
                                                 const uint8_t* packed, const float* w_scale, int64_t N, void* y,
                                                 bitnet_dtype_t y_dtype, int64_t ldy, int8_t* q, float* a_scale,
                                                 int32_t* q_rowsum) {
    const char* fn = "bitnet_rmsnorm_bitlinear_forward";
    if (!norm_w) return fail(BITNET_ERR_INVALID_ARG, "%s: norm_w is NULL", fn);
    return bitlinear_impl(stream, x, up, x_dtype, M, K, ldx, norm_w, norm_dtype, eps, packed, w_scale, N, y,
                          y_dtype, ldy, q, a_scale, q_rowsum, fn);
}

// -------------------------------------------------------------- W1.58A16

bitnet_status_t bitnet_linear_a16(hipStream_t stream, const void* x, bitnet_dtype_t x_dtype, int64_t M, int64_t K,
                                  int64_t ldx, const uint8_t* packed, const float* w_scale, int64_t N, void* y,
                                  bitnet_dtype_t y_dtype, int64_t ldy) {
    const char* fn = "bitnet_linear_a16";
    bitnet_status_t s = check_dims(fn, M, N, K);
    if (s != BITNET_OK) return s;
    if (!x || !packed || !w_scale || !y) return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (x_dtype != BITNET_BF16 && x_dtype != BITNET_F16)
        return fail(BITNET_ERR_UNSUPPORTED, "%s: W1.58A16 takes bf16 or fp16 activations (x_dtype %d)", fn,
                    (int)x_dtype);
    if (!valid_dtype(y_dtype)) return fail(BITNET_ERR_INVALID_ARG, "%s: bad y dtype %d", fn, (int)y_dtype);
    if (ldx < K || ldy < N) return fail(BITNET_ERR_INVALID_ARG, "%s: ldx < K or ldy < N", fn);
    if (!aligned(x, 16) || (ldx * 2) % 16 != 0 || !aligned(packed, 16) || !aligned(w_scale, 4) ||
        !aligned(y, y_dtype == BITNET_F32 ? 4 : 2))
        return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned pointer (x rows and packed must be 16-byte aligned)", fn);
    hipError_t e = bitnet::launch_gemv_a16(static_cast<const uint16_t*>(x), ldx, M, K, padded_k(K), packed, w_scale,
                                           N, y, y_dtype == BITNET_BF16, ldy, stream, x_dtype == BITNET_F16);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

// ------------------------------------------------------------------ I2_S

int64_t bitnet_i2s_bytes(int64_t N, int64_t K) {
    if (N <= 0 || K <= 0 || K % 16 != 0 || K > kMaxK || N > kMaxMN || (N * K) % 128 != 0) return -1;
    return N * K / 4 + 4;
}

static int64_t i2s_byte_at(int64_t v, bool consecutive) { return consecutive ? v / 4 : v % 32; }
static int i2s_shift_at(int64_t v, bool consecutive) {
    return consecutive ? 6 - 2 * static_cast<int>(v % 4) : 6 - 2 * static_cast<int>(v / 32);
}

static bitnet_status_t check_i2s(bitnet_mem_t where, const void* a, const void* b, const void* c, int64_t N,
                                 int64_t K, bitnet_i2s_order_t order, const char* fn) {
    if (where != BITNET_MEM_HOST && where != BITNET_MEM_DEVICE)
        return fail(BITNET_ERR_INVALID_ARG, "%s: bad memory kind %d", fn, (int)where);
    if (order != BITNET_I2S_STRIDED && order != BITNET_I2S_CONSECUTIVE)
        return fail(BITNET_ERR_INVALID_ARG, "%s: bad I2_S order %d", fn, (int)order);
    if (!a || !b || !c) return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", fn);
    if (bitnet_i2s_bytes(N, K) < 0)
        return fail(BITNET_ERR_INVALID_ARG, "%s: N=%lld, K=%lld: need K %% 16 == 0 and N*K %% 128 == 0", fn,
                    (long long)N, (long long)K);
    return BITNET_OK;
}

static bitnet_status_t i2s_device(bool import, hipStream_t stream, const uint8_t* in, const float* ws_in,
                                  int64_t N, int64_t K, bool consecutive, uint8_t* out, float* ws_out,
                                  const char* fn) {
    DeviceTemps temps;
    temps.stream = stream;
    hipError_t e = hipMallocAsync(&temps.p, sizeof(unsigned int), stream);
    if (e != hipSuccess) {
        temps.p = nullptr;
        return hip_fail(e, fn);
    }
    auto* d_status = static_cast<unsigned int*>(temps.p);
    if ((e = hipMemsetAsync(d_status, 0, sizeof(unsigned int), stream)) != hipSuccess) return hip_fail(e, fn);
    const int64_t Kp = padded_k(K);
    e = import ? bitnet::launch_i2s_import(in, N, K, Kp, consecutive, out, ws_out, d_status, stream)
               : bitnet::launch_i2s_export(in, ws_in, N, K, Kp, consecutive, out, d_status, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    unsigned int status = 0;
    if ((e = hipMemcpyAsync(&status, d_status, sizeof status, hipMemcpyDeviceToHost, stream)) != hipSuccess ||
        (e = hipStreamSynchronize(stream)) != hipSuccess)
        return hip_fail(e, fn);
    if (status & 1u) return fail(BITNET_ERR_INVALID_ARG, "%s: a 2-bit field holds 3, which encodes no weight", fn);
    if (status & 2u) return fail(BITNET_ERR_INVALID_ARG, "%s: the I2_S scale is not positive", fn);
    if (status & 4u)
        return fail(BITNET_ERR_INVALID_ARG, "%s: w_scale differs between rows (export one source tensor at a time)",
                    fn);
    return ok();
}

bitnet_status_t bitnet_i2s_import(bitnet_mem_t where, hipStream_t stream, const uint8_t* i2s, int64_t N, int64_t K,
                                  bitnet_i2s_order_t order, uint8_t* packed, float* w_scale) {
    const char* fn = "bitnet_i2s_import";
    bitnet_status_t st = check_i2s(where, i2s, packed, w_scale, N, K, order, fn);
    if (st != BITNET_OK) return st;
    const bool consecutive = order == BITNET_I2S_CONSECUTIVE;
    if (where == BITNET_MEM_DEVICE) {
        if (!aligned(i2s, 4) || !aligned(w_scale, 4))
            return fail(BITNET_ERR_INVALID_ARG, "%s: i2s and w_scale must be 4-byte aligned", fn);
        return i2s_device(true, stream, i2s, nullptr, N, K, consecutive, packed, w_scale, fn);
    }
    const int64_t Kp = padded_k(K), row_bytes = Kp / 4;
    float s;
    memcpy(&s, i2s + N * K / 4, sizeof s);
    if (!(s > 0.0f)) return fail(BITNET_ERR_INVALID_ARG, "%s: the I2_S scale is not positive", fn);
    memset(packed, 0, static_cast<size_t>(N * row_bytes));
    for (int64_t n = 0; n < N; ++n) {
        uint8_t* row = packed + n * row_bytes;
        for (int64_t k = 0; k < Kp; ++k) {
            unsigned c = 1u;
            if (k < K) {
                const int64_t i = n * K + k, v = i % 128;
                c = (i2s[(i / 128) * 32 + i2s_byte_at(v, consecutive)] >> i2s_shift_at(v, consecutive)) & 3u;
                if (c == 3u) return fail(BITNET_ERR_INVALID_ARG, "%s: a 2-bit field holds 3, which encodes no weight", fn);
            }
            row[4 * (k / 16) + k % 4] |= static_cast<uint8_t>(c << (2 * ((k % 16) / 4)));
        }
        w_scale[n] = 1.0f / s;
    }
    return ok();
}

bitnet_status_t bitnet_i2s_export(bitnet_mem_t where, hipStream_t stream, const uint8_t* packed,
                                  const float* w_scale, int64_t N, int64_t K, bitnet_i2s_order_t order,
                                  uint8_t* i2s) {
    const char* fn = "bitnet_i2s_export";
    bitnet_status_t st = check_i2s(where, packed, w_scale, i2s, N, K, order, fn);
    if (st != BITNET_OK) return st;
    const bool consecutive = order == BITNET_I2S_CONSECUTIVE;
    if (where == BITNET_MEM_DEVICE) {
        if (!aligned(i2s, 4) || !aligned(w_scale, 4))
            return fail(BITNET_ERR_INVALID_ARG, "%s: i2s and w_scale must be 4-byte aligned", fn);
        return i2s_device(false, stream, packed, w_scale, N, K, consecutive, i2s, nullptr, fn);
    }
    for (int64_t n = 1; n < N; ++n)
        if (w_scale[n] != w_scale[0])
            return fail(BITNET_ERR_INVALID_ARG, "%s: w_scale differs between rows (export one source tensor at a time)",
                        fn);
    const int64_t Kp = padded_k(K), row_bytes = Kp / 4, total = N * K;
    memset(i2s, 0, static_cast<size_t>(total / 4));
    for (int64_t i = 0; i < total; ++i) {
        const int64_t n = i / K, k = i % K, v = i % 128;
        const unsigned c = (packed[n * row_bytes + 4 * (k / 16) + k % 4] >> (2 * ((k % 16) / 4))) & 3u;
        if (c == 3u) return fail(BITNET_ERR_INVALID_ARG, "%s: a 2-bit field holds 3, which encodes no weight", fn);
        i2s[(i / 128) * 32 + i2s_byte_at(v, consecutive)] |= static_cast<uint8_t>(c << i2s_shift_at(v, consecutive));
    }
    const float s = 1.0f / w_scale[0];
    memcpy(i2s + total / 4, &s, sizeof s);
    return ok();
}

// ------------------------------------------------------- packed-weight files

namespace {

constexpr char kFileMagic[8] = {'B', 'T', 'N', 'L', 'V', '1', 0, 0};
constexpr uint32_t kFileVersion = 1;
constexpr uint32_t kFileHeaderBytes = 64;

struct FileHeader {                 // little-endian, 64 bytes
    char magic[8];
    uint32_t version;
    uint32_t header_bytes;
    int64_t N, K, Kp;
    int32_t n_segs;
    uint32_t layout;                // 1: layout v1
    uint64_t fnv1a;                 // FNV-1a 64 over header bytes 0..47, then every byte after the header
    uint64_t reserved;              // 0
};
static_assert(sizeof(FileHeader) == kFileHeaderBytes, "file header layout");
constexpr size_t kHashedHeaderBytes = offsetof(FileHeader, fnv1a);
static_assert(kHashedHeaderBytes == 48, "the checksum covers the header fields before it");

uint64_t fnv1a(uint64_t h, const void* p, size_t n) {
    const auto* b = static_cast<const unsigned char*>(p);
    for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 0x100000001b3ull;
    return h;
}

struct File {
    FILE* f = nullptr;
    ~File() {
        if (f) fclose(f);
    }
};

}  // namespace

bitnet_status_t bitnet_save_packed(const char* path, const uint8_t* packed, const float* w_scale, int64_t N,
                                   int64_t K, const int64_t* seg_rows, const float* seg_mean, int32_t n_segs) {
    const char* fn = "bitnet_save_packed";
    bitnet_status_t s = check_dims(fn, 1, N, K);
    if (s != BITNET_OK) return s;
    if (!path || !packed || !w_scale || !seg_rows || !seg_mean || n_segs <= 0)
        return fail(BITNET_ERR_INVALID_ARG, "%s: need path, packed, w_scale, seg_rows, seg_mean and n_segs > 0", fn);
    int64_t rows = 0;
    for (int32_t i = 0; i < n_segs; ++i) {
        if (seg_rows[i] <= 0) return fail(BITNET_ERR_INVALID_ARG, "%s: segment %d is empty", fn, i);
        rows += seg_rows[i];
    }
    if (rows != N) return fail(BITNET_ERR_INVALID_ARG, "%s: segment rows sum to %lld, not N", fn, (long long)rows);
    const int64_t Kp = padded_k(K);
    const size_t nb_packed = static_cast<size_t>(N * (Kp / 4)), nb_scale = static_cast<size_t>(N) * 4;
    FileHeader h{};
    memcpy(h.magic, kFileMagic, sizeof h.magic);
    h.version = kFileVersion;
    h.header_bytes = kFileHeaderBytes;
    h.N = N; h.K = K; h.Kp = Kp; h.n_segs = n_segs; h.layout = 1;
    uint64_t c = fnv1a(0xcbf29ce484222325ull, &h, kHashedHeaderBytes);
    c = fnv1a(c, packed, nb_packed);
    c = fnv1a(c, w_scale, nb_scale);
    c = fnv1a(c, seg_rows, static_cast<size_t>(n_segs) * 8);
    c = fnv1a(c, seg_mean, static_cast<size_t>(n_segs) * 4);
    h.fnv1a = c;
    File f;
    f.f = fopen(path, "wb");
    if (!f.f) return fail(BITNET_ERR_INVALID_ARG, "%s: cannot open %s for writing", fn, path);
    if (fwrite(&h, sizeof h, 1, f.f) != 1 || fwrite(packed, 1, nb_packed, f.f) != nb_packed ||
        fwrite(w_scale, 1, nb_scale, f.f) != nb_scale ||
        fwrite(seg_rows, 8, static_cast<size_t>(n_segs), f.f) != static_cast<size_t>(n_segs) ||
        fwrite(seg_mean, 4, static_cast<size_t>(n_segs), f.f) != static_cast<size_t>(n_segs))
        return fail(BITNET_ERR_INVALID_ARG, "%s: short write to %s", fn, path);
    if (fclose(f.f) != 0) {
        f.f = nullptr;
        return fail(BITNET_ERR_INVALID_ARG, "%s: closing %s failed", fn, path);
    }
    f.f = nullptr;
    return ok();
}

bitnet_status_t bitnet_load_packed(const char* path, int64_t* N, int64_t* K, int32_t* n_segs, uint8_t* packed,
                                   float* w_scale, int64_t* seg_rows, float* seg_mean) {
    const char* fn = "bitnet_load_packed";
    if (!path || !N || !K || !n_segs) return fail(BITNET_ERR_INVALID_ARG, "%s: need path, N, K and n_segs", fn);
    File f;
    f.f = fopen(path, "rb");
    if (!f.f) return fail(BITNET_ERR_INVALID_ARG, "%s: cannot open %s", fn, path);
    FileHeader h{};
    if (fread(&h, sizeof h, 1, f.f) != 1 || memcmp(h.magic, kFileMagic, sizeof h.magic) != 0)
        return fail(BITNET_ERR_INVALID_ARG, "%s: %s is not a packed-weight file", fn, path);
    if (h.version != kFileVersion || h.header_bytes != kFileHeaderBytes || h.layout != 1)
        return fail(BITNET_ERR_UNSUPPORTED, "%s: file version %u, layout %u not supported (this library: %u, 1)", fn,
                    h.version, h.layout, kFileVersion);
    if (check_dims(fn, 1, h.N, h.K) != BITNET_OK || h.Kp != padded_k(h.K) || h.n_segs <= 0 || h.n_segs > h.N ||
        h.reserved != 0)
        return fail(BITNET_ERR_INVALID_ARG, "%s: %s has an inconsistent header", fn, path);
    *N = h.N;
    *K = h.K;
    *n_segs = h.n_segs;
    if (!packed) return ok();                       // header query
    if (!w_scale || !seg_rows || !seg_mean)
        return fail(BITNET_ERR_INVALID_ARG, "%s: need packed, w_scale, seg_rows and seg_mean", fn);
    const size_t nb_packed = static_cast<size_t>(h.N * (h.Kp / 4)), nb_scale = static_cast<size_t>(h.N) * 4;
    const size_t ns = static_cast<size_t>(h.n_segs);
    if (fread(packed, 1, nb_packed, f.f) != nb_packed || fread(w_scale, 1, nb_scale, f.f) != nb_scale ||
        fread(seg_rows, 8, ns, f.f) != ns || fread(seg_mean, 4, ns, f.f) != ns)
        return fail(BITNET_ERR_INVALID_ARG, "%s: %s is truncated", fn, path);
    uint64_t c = fnv1a(0xcbf29ce484222325ull, &h, kHashedHeaderBytes);
    c = fnv1a(c, packed, nb_packed);
    c = fnv1a(c, w_scale, nb_scale);
    c = fnv1a(c, seg_rows, ns * 8);
    c = fnv1a(c, seg_mean, ns * 4);
    if (c != h.fnv1a) return fail(BITNET_ERR_INVALID_ARG, "%s: %s fails its checksum", fn, path);
    return ok();
}

// Kernels of a grouped plan.  BITNET_GROUP_KERNEL=persistent, read when a
// plan is made, skips the streaming kernel (for comparisons; results are
// identical).
enum { kGroupPersistent = 0, kGroupStream = 1, kGroupA16 = 2, kGroupBlocked = 3 };
enum GroupMode { kModeA8 = 0, kModeA16 = 1, kModeBlocked = 2 };
static bool persistent_forced() {
    const char* v = getenv("BITNET_GROUP_KERNEL");
    return v && strcmp(v, "persistent") == 0;
}

int64_t bitnet_group_table_bytes(int32_t count) {
    if (count <= 0) return -1;
    // the problems, then a streaming launch's share bounds (grid + 1) and
    // per-workgroup records (4 each)
    return static_cast<int64_t>(count) * static_cast<int64_t>(sizeof(bitnet::GemvProblem)) +
           (bitnet::kMaxStreamGrid + 1 + 4 * static_cast<int64_t>(bitnet::kMaxStreamGrid)) *
               static_cast<int64_t>(sizeof(int32_t));
}

static bitnet_status_t group_plan_impl(hipStream_t stream, const bitnet_group_item_t* items,
                                       const bitnet_group_norm_t* norms, int32_t count, int64_t M,
                                       bitnet_dtype_t x_dtype, bitnet_dtype_t y_dtype, void* table_dev,
                                       int64_t table_bytes, bitnet_group_plan_t* plan, const char* fn,
                                       GroupMode mode = kModeA8) {
    const bool a16 = mode == kModeA16;
    if (count <= 0 || !items || !plan || !table_dev)
        return fail(BITNET_ERR_INVALID_ARG, "%s: need count > 0, items, table_dev and plan", fn);
    if (!aligned(table_dev, 16) || table_bytes < bitnet_group_table_bytes(count))
        return fail(BITNET_ERR_INVALID_ARG, "%s: table_dev must be 16-byte aligned and hold %lld bytes", fn,
                    (long long)bitnet_group_table_bytes(count));
    if (M <= 0 || M > kGemvMaxM) return fail(BITNET_ERR_INVALID_ARG, "%s: M=%lld must be in 1..16", fn, (long long)M);
    if (!(valid_dtype(x_dtype) || (a16 && x_dtype == BITNET_F16)) || !valid_dtype(y_dtype))
        return fail(BITNET_ERR_INVALID_ARG, "%s: bad dtype", fn);
    const int64_t esize = x_dtype == BITNET_F32 ? 4 : 2;
    std::vector<bitnet::GemvProblem> table(static_cast<size_t>(count));
    int64_t tiles = 0, steps = 0, max_kp = 0;
    for (int32_t i = 0; i < count; ++i) {
        const bitnet_group_item_t& it = items[i];
        char where[64];
        snprintf(where, sizeof where, "%s: item %d", fn, i);
        bitnet_status_t s = check_dims(where, M, it.N, it.K);
        if (s != BITNET_OK) return s;
        if (!it.x || !it.packed || !it.w_scale || !it.y)
            return fail(BITNET_ERR_INVALID_ARG, "%s: a required pointer is NULL", where);
        if (it.ldx < it.K || it.ldy < it.N) return fail(BITNET_ERR_INVALID_ARG, "%s: ldx < K or ldy < N", where);
        if (!aligned(it.x, 16) || (it.ldx * esize) % 16 != 0 || !aligned(it.packed, 16) ||
            !aligned(it.w_scale, 4) || !aligned(it.y, y_dtype == BITNET_F32 ? 4 : 2))
            return fail(BITNET_ERR_INVALID_ARG, "%s: misaligned pointer or x row stride", where);
        const int64_t Kp = padded_k(it.K);
        if (mode == kModeBlocked && it.K > kBlockedMaxK)
            return fail(BITNET_ERR_UNSUPPORTED, "%s: K=%lld > %lld", where, (long long)it.K, (long long)kBlockedMaxK);
        if (static_cast<int64_t>(bitnet::gemv_group_lds(M, Kp)) > kGroupLdsBytes)
            return fail(BITNET_ERR_UNSUPPORTED, "%s: M tokens of K=%lld need more than %lld bytes of LDS", where,
                        (long long)it.K, (long long)kGroupLdsBytes);
        const bitnet_group_norm_t* nm = norms && norms[i].norm_w ? &norms[i] : nullptr;
        if (nm) {
            if ((s = check_norm(it.x, nm->up, x_dtype, nm->norm_w, nm->norm_dtype, nm->eps, where)) != BITNET_OK)
                return s;
            if (!aligned(nm->norm_w, 16) || (nm->up && !aligned(nm->up, 16)))
                return fail(BITNET_ERR_INVALID_ARG, "%s: norm_w and up must be 16-byte aligned", where);
        }
        bitnet::GemvProblem& p = table[static_cast<size_t>(i)];
        p = bitnet::GemvProblem{};
        if (nm) {
            p.up = nm->up; p.norm_w = nm->norm_w; p.eps = nm->eps; p.norm_bf16 = nm->norm_dtype == BITNET_BF16;
        }
        p.x = it.x; p.ldx = it.ldx; p.packed = it.packed; p.w_scale = it.w_scale;
        p.y = it.y; p.ldy = it.ldy;
        p.M = (int)M; p.N = (int)it.N; p.K = (int)it.K; p.Kp = (int)Kp;
        p.tile0 = (int)tiles;
        p.ntiles = (int)bitnet::gemv_group_tiles(it.N);
        p.steps = (int)bitnet::gemv_group_steps(Kp);
        p.step0 = steps;
        tiles += p.ntiles;
        steps += static_cast<int64_t>(p.ntiles) * p.steps;
        if (tiles > kMaxMN) return fail(BITNET_ERR_INVALID_ARG, "%s: too many tiles in the group", fn);
        if (Kp > max_kp) max_kp = Kp;
    }
    // Kernel choice: the streaming kernel where every workgroup's problems
    // fit its LDS share, else the persistent one.
    int kind = kGroupPersistent, grid = 0;
    size_t lds = bitnet::gemv_group_lds(M, max_kp);
    std::vector<int32_t> bounds;
    if (mode == kModeBlocked) {
        if (!bitnet::gemv_stream_plan(table.data(), count, tiles, steps, &grid, &lds, 1, &bounds, true))
            return fail(BITNET_ERR_UNSUPPORTED,
                        "%s: a workgroup's share of the group needs more LDS than it has for M=%lld token rows", fn,
                        (long long)M);
        kind = kGroupBlocked;
    } else if (a16) {
        if (!bitnet::gemv_stream_plan(table.data(), count, tiles, steps, &grid, &lds, 2, &bounds))
            return fail(BITNET_ERR_UNSUPPORTED,
                        "%s: a workgroup's share of the group needs more LDS than it has for M=%lld bf16 token rows "
                        "(use bitnet_linear_a16 per item)",
                        fn, (long long)M);
        kind = kGroupA16;
    } else if (!persistent_forced() &&
               bitnet::gemv_stream_plan(table.data(), count, tiles, steps, &grid, &lds, 1, &bounds)) {
        kind = kGroupStream;
    } else {
        grid = 0;
        lds = bitnet::gemv_group_lds(M, max_kp);
        bounds.clear();
    }
    // one upload: the problems, then (streaming kernels) the share bounds
    std::vector<char> blob(table.size() * sizeof(bitnet::GemvProblem) + bounds.size() * sizeof(int32_t));
    memcpy(blob.data(), table.data(), table.size() * sizeof(bitnet::GemvProblem));
    if (!bounds.empty())
        memcpy(blob.data() + table.size() * sizeof(bitnet::GemvProblem), bounds.data(),
               bounds.size() * sizeof(int32_t));
    hipError_t e = hipMemcpyAsync(table_dev, blob.data(), blob.size(), hipMemcpyHostToDevice, stream);
    if (e != hipSuccess) return hip_fail(e, "bitnet_group_plan: table upload");
    if ((e = hipStreamSynchronize(stream)) != hipSuccess) return hip_fail(e, "bitnet_group_plan: sync");
    plan->opaque[0] = kPlanMagic;
    plan->opaque[1] = static_cast<int64_t>(reinterpret_cast<uintptr_t>(table_dev));
    plan->opaque[2] = count;
    plan->opaque[3] = M;
    plan->opaque[4] = tiles;
    plan->opaque[5] = static_cast<int64_t>(lds);
    plan->opaque[6] = static_cast<int64_t>(x_dtype) | (static_cast<int64_t>(y_dtype) << 8) |
                      (static_cast<int64_t>(kind) << 16) | (static_cast<int64_t>(grid) << 32);
    plan->opaque[7] = steps;
    return ok();
}

bitnet_status_t bitnet_group_plan(hipStream_t stream, const bitnet_group_item_t* items, int32_t count, int64_t M,
                                  bitnet_dtype_t x_dtype, bitnet_dtype_t y_dtype, void* table_dev,
                                  int64_t table_bytes, bitnet_group_plan_t* plan) {
    return group_plan_impl(stream, items, nullptr, count, M, x_dtype, y_dtype, table_dev, table_bytes, plan,
                           "bitnet_group_plan");
}

bitnet_status_t bitnet_group_plan_a16(hipStream_t stream, const bitnet_group_item_t* items, int32_t count, int64_t M,
                                      bitnet_dtype_t y_dtype, void* table_dev, int64_t table_bytes,
                                      bitnet_group_plan_t* plan) {
    return group_plan_impl(stream, items, nullptr, count, M, BITNET_BF16, y_dtype, table_dev, table_bytes, plan,
                           "bitnet_group_plan_a16", kModeA16);
}

bitnet_status_t bitnet_group_plan_a16_fp16(hipStream_t stream, const bitnet_group_item_t* items, int32_t count,
                                           int64_t M, bitnet_dtype_t y_dtype, void* table_dev, int64_t table_bytes,
                                           bitnet_group_plan_t* plan) {
    return group_plan_impl(stream, items, nullptr, count, M, BITNET_F16, y_dtype, table_dev, table_bytes, plan,
                           "bitnet_group_plan_a16_fp16", kModeA16);
}

bitnet_status_t bitnet_group_plan_blocked(hipStream_t stream, const bitnet_group_item_t* items, int32_t count,
                                          int64_t M, bitnet_dtype_t x_dtype, bitnet_dtype_t y_dtype, void* table_dev,
                                          int64_t table_bytes, bitnet_group_plan_t* plan) {
    return group_plan_impl(stream, items, nullptr, count, M, x_dtype, y_dtype, table_dev, table_bytes, plan,
                           "bitnet_group_plan_blocked", kModeBlocked);
}

bitnet_status_t bitnet_group_plan_rmsnorm(hipStream_t stream, const bitnet_group_item_t* items,
                                          const bitnet_group_norm_t* norms, int32_t count, int64_t M,
                                          bitnet_dtype_t x_dtype, bitnet_dtype_t y_dtype, void* table_dev,
                                          int64_t table_bytes, bitnet_group_plan_t* plan) {
    if (!norms) return fail(BITNET_ERR_INVALID_ARG, "bitnet_group_plan_rmsnorm: norms is NULL");
    return group_plan_impl(stream, items, norms, count, M, x_dtype, y_dtype, table_dev, table_bytes, plan,
                           "bitnet_group_plan_rmsnorm");
}

bitnet_status_t bitnet_bitlinear_grouped(hipStream_t stream, const bitnet_group_plan_t* plan) {
    const char* fn = "bitnet_bitlinear_grouped";
    if (!plan || plan->opaque[0] != kPlanMagic)
        return fail(BITNET_ERR_INVALID_ARG, "%s: plan was not made by bitnet_group_plan", fn);
    const auto* table = reinterpret_cast<const bitnet::GemvProblem*>(static_cast<uintptr_t>(plan->opaque[1]));
    const int count = static_cast<int>(plan->opaque[2]);
    const int kind = static_cast<int>((plan->opaque[6] >> 16) & 0xFF);
    const int grid = static_cast<int>(plan->opaque[6] >> 32);
    const bool x_bf16 = (plan->opaque[6] & 0xFF) == BITNET_BF16;
    const bool y_bf16 = ((plan->opaque[6] >> 8) & 0xFF) == BITNET_BF16;
    hipError_t e;
    if (kind == kGroupA16)
        e = bitnet::launch_gemv_a16_grouped(table, count, plan->opaque[4], plan->opaque[7], grid, y_bf16, stream,
                                            (plan->opaque[6] & 0xFF) == BITNET_F16);
    else if (kind == kGroupBlocked)
        e = bitnet::launch_gemv_blocked_grouped(table, count, plan->opaque[4], plan->opaque[7], grid, x_bf16, y_bf16,
                                                stream);
    else
        e = bitnet::launch_gemv_grouped(table, count, plan->opaque[4], plan->opaque[7],
                                        static_cast<size_t>(plan->opaque[5]), kind == kGroupStream ? grid : 0, x_bf16,
                                        y_bf16, stream);
    if (e != hipSuccess) return hip_fail(e, fn);
    return ok();
}

const char* bitnet_group_plan_kernel(const bitnet_group_plan_t* plan) {
    if (!plan || plan->opaque[0] != kPlanMagic) return "";
    const int kind = static_cast<int>((plan->opaque[6] >> 16) & 0xFF);
    return kind == kGroupStream    ? "stream"
           : kind == kGroupA16     ? "stream-a16"
           : kind == kGroupBlocked ? "stream-blocked"
                                   : "persistent";
}

const char* bitnet_status_string(bitnet_status_t s) {
    switch (s) {
        case BITNET_OK: return "ok";
        case BITNET_ERR_INVALID_ARG: return "invalid argument";
        case BITNET_ERR_UNSUPPORTED: return "unsupported";
        case BITNET_ERR_HIP: return "HIP error";
        case BITNET_ERR_NONFINITE: return "non-finite weight";
    }
    return "unknown status";
}

const char* bitnet_last_error(void) { return g_last_error.c_str(); }

}  // extern "C"
