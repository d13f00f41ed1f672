// i2s.hip -- conversion between the I2_S interchange format and layout v1.
//
// I2_S ("BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference
// Optimization Guide", s3.3 "I2_S Ternary Packing"): a tensor's values,
// flattened row-major, form blocks of 128; each block is 32 bytes, a byte
// holding four stored codes as (c0 << 6) | (c1 << 4) | (c2 << 2) | c3 with
// -1 -> 0, 0 -> 1, +1 -> 2; the fp32 scale s = 1/mean|W| follows the codes.
// The page does not say which four values of a block share a byte: `strided`
// puts values j, j+32, j+64, j+96 in byte j, `consecutive` values 4j..4j+3.
// Layout v1 keeps the same code values, so conversion only moves 2-bit
// fields; w_scale (the dequantisation factor mean|W|) is 1/s.
//
// One thread per output byte (import: a layout-v1 byte; export: an I2_S
// byte), reading the four fields it needs; the conversion is offline and
// L2-resident per block, so no tiling.  Invalid input (a field holding 3, a
// scale that is not positive, rows of different scales on export) sets bits
// of a status word the caller reads back.
#include <algorithm>

#include "device_common.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ int64_t i2s_byte_of(int64_t v, bool consecutive) { return consecutive ? v / 4 : v % 32; }
__device__ __forceinline__ int i2s_shift_of(int64_t v, bool consecutive) {
    return consecutive ? 6 - 2 * static_cast<int>(v % 4) : 6 - 2 * static_cast<int>(v / 32);
}

// layout v1: element k of a row sits in byte 4*(k/16) + k%4 at bit 2*((k%16)/4)
__global__ __launch_bounds__(kThreads) void i2s_import_kernel(const uint8_t* __restrict__ in, int64_t N, int64_t K,
                                                              int64_t Kp, bool consecutive,
                                                              uint8_t* __restrict__ packed,
                                                              float* __restrict__ w_scale,
                                                              unsigned int* __restrict__ status) {
    const int64_t row_bytes = Kp / 4;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (idx < N) {                                      // the scale, one row per thread
        float s;
        __builtin_memcpy(&s, in + N * K / 4, sizeof s);
        if (!(s > 0.0f)) atomicOr(status, 2u);
        w_scale[idx] = 1.0f / s;
    }
    if (idx >= N * row_bytes) return;
    const int64_t n = idx / row_bytes, ob = idx % row_bytes;
    const int64_t j = ob / 4, b = ob % 4;
    unsigned out = 0, bad = 0;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
        const int64_t k = 16 * j + 4 * p + b;
        unsigned c = 1u;                                // padding: weight 0
        if (k < K) {
            const int64_t i = n * K + k, blk = i / 128, v = i % 128;
            c = (in[blk * 32 + i2s_byte_of(v, consecutive)] >> i2s_shift_of(v, consecutive)) & 3u;
            bad |= c == 3u;
        }
        out |= c << (2 * p);
    }
    packed[idx] = static_cast<uint8_t>(out);
    if (bad) atomicOr(status, 1u);
}

__global__ __launch_bounds__(kThreads) void i2s_export_kernel(const uint8_t* __restrict__ packed,
                                                              const float* __restrict__ w_scale, int64_t N,
                                                              int64_t K, int64_t Kp, bool consecutive,
                                                              uint8_t* __restrict__ out,
                                                              unsigned int* __restrict__ status) {
    const int64_t row_bytes = Kp / 4;
    const int64_t total = N * K;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x;
    if (idx < N && w_scale[idx] != w_scale[0]) atomicOr(status, 4u);
    if (idx == 0) {
        const float s = 1.0f / w_scale[0];
        __builtin_memcpy(out + total / 4, &s, sizeof s);
    }
    if (idx >= total / 4) return;
    const int64_t blk = idx / 32, jb = idx % 32;
    unsigned byte = 0, bad = 0;
#pragma unroll
    for (int f = 0; f < 4; ++f) {                       // c0 .. c3
        const int64_t v = consecutive ? 4 * jb + f : jb + 32 * f;
        const int64_t i = blk * 128 + v, n = i / K, k = i % K;
        const unsigned c = (packed[n * row_bytes + 4 * (k / 16) + k % 4] >> (2 * ((k % 16) / 4))) & 3u;
        bad |= c == 3u;
        byte |= c << i2s_shift_of(v, consecutive);
    }
    out[idx] = static_cast<uint8_t>(byte);
    if (bad) atomicOr(status, 1u);
}

}  // namespace

hipError_t launch_i2s_import(const uint8_t* in, int64_t N, int64_t K, int64_t Kp, bool consecutive, uint8_t* packed,
                             float* w_scale, unsigned int* status, hipStream_t stream) {
    const int64_t work = std::max<int64_t>(N * (Kp / 4), N);
    const dim3 grid(static_cast<unsigned>((work + kThreads - 1) / kThreads)), block(kThreads);
    i2s_import_kernel<<<grid, block, 0, stream>>>(in, N, K, Kp, consecutive, packed, w_scale, status);
    return hipGetLastError();
}

hipError_t launch_i2s_export(const uint8_t* packed, const float* w_scale, int64_t N, int64_t K, int64_t Kp,
                             bool consecutive, uint8_t* out, unsigned int* status, hipStream_t stream) {
    const int64_t work = std::max<int64_t>(N * K / 4, N);
    const dim3 grid(static_cast<unsigned>((work + kThreads - 1) / kThreads)), block(kThreads);
    i2s_export_kernel<<<grid, block, 0, stream>>>(packed, w_scale, N, K, Kp, consecutive, out, status);
    return hipGetLastError();
}

}  // namespace bitnet
