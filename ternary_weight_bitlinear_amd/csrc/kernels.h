// kernels.h -- internal launchers behind the C ABI (not part of the public API).
// Each launcher enqueues on `stream` and returns the launch status.  Shapes and
// pointers are validated by the caller (bitnet_api.cpp) before any launch.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

// Per-token ActQuant of x [M, K] (row stride ldx) into q [M][Kp].
hipError_t launch_act_quant(const void* x, bool x_bf16, int64_t M, int64_t K, int64_t ldx,
                            int8_t* q, float* a_scale, int32_t* q_rowsum, int64_t Kp,
                            hipStream_t stream);

// ActQuant(RMSNorm(input, norm_w)) of M tokens: input = x, or silu(x) * up
// when up is given (same dtype and row stride as x); norm_w has K entries.
hipError_t launch_norm_act_quant(const void* x, const void* up, bool x_bf16, int64_t M, int64_t K, int64_t ldx,
                                 const void* norm_w, bool norm_bf16, float eps, int8_t* q, float* a_scale,
                                 int32_t* q_rowsum, int64_t Kp, hipStream_t stream);

// Linear on quantised operands, M <= 16: one streaming pass over packed.
hipError_t launch_gemv(const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                       int64_t M, int64_t Kp, const uint8_t* packed, const float* w_scale,
                       int64_t N, void* y, bool y_bf16, int64_t ldy, int32_t* acc_debug,
                       hipStream_t stream);

// Linear on quantised operands, any M: int8-MFMA GEMM.
hipError_t launch_gemm(const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                       int64_t M, int64_t Kp, const uint8_t* packed, const float* w_scale,
                       int64_t N, void* y, bool y_bf16, int64_t ldy, int32_t* acc_debug,
                       hipStream_t stream);

// Temporaries of one device pack, carved from one buffer: row_sum [N] f64,
// seg_start [n_segs + 1] i64, seg_mean [n_segs] f32 (padded to 8 bytes),
// seg_zero [n_segs] u64, status u32.
struct PackTemps {
    size_t off_start, off_mean, off_zero, off_status, bytes;
};
constexpr PackTemps pack_temp_layout(int64_t N, int64_t n_segs) {
    PackTemps t{};
    t.off_start = static_cast<size_t>(N) * sizeof(double);
    t.off_mean = t.off_start + static_cast<size_t>(n_segs + 1) * sizeof(int64_t);
    t.off_zero = (t.off_mean + static_cast<size_t>(n_segs) * sizeof(float) + 7) / 8 * 8;
    t.off_status = t.off_zero + static_cast<size_t>(n_segs) * sizeof(unsigned long long);
    t.bytes = t.off_status + sizeof(unsigned int);
    return t;
}

// Limits of the allocation-free device pack, whose temporaries live in a
// fixed device array of the library (one per GPU, held until the process ends).
constexpr int64_t kPackStaticMaxRows = 131072;
constexpr int64_t kPackStaticMaxSegs = 64;

// Device address of that array on the current device (looked up once per
// device with hipGetSymbolAddress); its size in bytes in *bytes.
hipError_t pack_scratch(void** ptr, size_t* bytes);

// Device WeightQuant + pack.  seg_start_dev [n_segs + 1] holds the first row of
// every segment and N at the end.  Temporaries: row_sum [N] doubles,
// seg_mean_dev / seg_zero_dev [n_segs], status_dev (bit 0: non-finite weight;
// cleared by the launch itself, seg_zero_dev too).
hipError_t launch_pack(const void* W, bool w_bf16, int64_t N, int64_t K, int64_t ldw,
                       int64_t Kp, const int64_t* seg_start_dev, int32_t n_segs,
                       double* row_sum, float* seg_mean_dev, unsigned long long* seg_zero_dev,
                       unsigned int* status_dev, uint8_t* packed, float* w_scale,
                       hipStream_t stream);

// WeightQuant with one scale per 256-weight block of a row: packed [N][Kp/4]
// (layout v1) and block_scale [ceil(K/256)][N]; status bit 0: a weight is not
// finite.
hipError_t launch_pack_blocked(const void* W, bool w_bf16, int64_t N, int64_t K, int64_t ldw, int64_t Kp,
                               unsigned int* status_dev, uint8_t* packed, float* block_scale, hipStream_t stream);

// Linear with per-block weight scales, any M: y = a_scale * sum_b (float)acc_b
// * block_scale[b][n] in block order (int8 MFMA GEMM, 128x128 tiles); K <= 8192.
hipError_t launch_gemm_blocked(const int8_t* q, const float* a_scale, int64_t M, int64_t K, int64_t Kp,
                               const uint8_t* packed, const float* block_scale, int64_t N, void* y, bool y_bf16,
                               int64_t ldy, hipStream_t stream);

// W1.58A16: y = w_scale * (x_bf16 . t), fp32 accumulation on bf16 MFMA; x rows
// 16-byte aligned (ldx * 2 % 16 == 0).
// x_f16: fp16 activations (fp16 matrix cores) instead of bf16.
hipError_t launch_gemv_a16(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, int64_t Kp, const uint8_t* packed,
                           const float* w_scale, int64_t N, void* y, bool y_bf16, int64_t ldy, hipStream_t stream,
                           bool x_f16 = false);

// I2_S <-> layout v1 (status bits: 1 a field holds 3, 2 a scale is not
// positive, 4 rows differ in scale on export).  The grid covers every output
// byte and every row.
hipError_t launch_i2s_import(const uint8_t* in, int64_t N, int64_t K, int64_t Kp, bool consecutive, uint8_t* packed,
                             float* w_scale, unsigned int* status, hipStream_t stream);
hipError_t launch_i2s_export(const uint8_t* packed, const float* w_scale, int64_t N, int64_t K, int64_t Kp,
                             bool consecutive, uint8_t* out, unsigned int* status, hipStream_t stream);

}  // namespace bitnet
