// pack.hip -- device WeightQuant + packing into layout v1 (gfx950).
//
// Method: per source tensor, s = 1/mean|W| and codes t = clamp(round(W*s),
// -1, 1) ("BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s1; the
// codes are built from the bf16 latent weights, s2), stored as u = t + 1, four
// per byte ("BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference
// Optimization Guide", s3.3 "I2_S Ternary Packing": -1 -> 0, 0 -> 1, +1 -> 2).
//
// The mean must come out bit-identical to the fixed-order definition
// (fp64, k ascending within a row, rows ascending within a tensor), so:
//  1. row_sum_kernel: one thread per row adds |W[n][k]| in fp64 in k order.
//     A 64-row workgroup stages 64 x 64 tiles in LDS so the global reads are
//     coalesced while each thread still walks its own row in order.
//  2. finalize_kernel: one thread per segment adds its row sums in row order,
//     divides once in fp64 and rounds to fp32; a non-finite sum (only possible
//     from an inf/NaN weight, since |W| >= 0 cannot cancel) sets a flag.
//  3. pack_kernel: one thread per 32-bit word (16 codes).  t = +1 iff
//     W*s > 0.5, t = -1 iff W*s < -0.5, else 0: for any non-NaN fp32 product
//     this is exactly clamp(rne(W*s), -1, 1) (rne(0.5) = 0), and a NaN product
//     gives 0.  Zero codes are counted per segment (wave sum, one atomic).
// Packing runs once per weight, offline; it is not on the timed path.
//
// Per-block scales ("BitVLA -- 1.58-bit Vision-Language-Action on Core AI",
// s2: the sibling matvec kernel keeps one scale per 256-weight block instead
// of one per tensor): pack_blocked_kernel, one thread per (row, block of 256
// k), adds |W| over the block's k in fp64 in k order, divides once by the
// block's weight count, rounds to fp32, and writes the block's code words
// (padding positions k >= K hold code 1) and its scale, block-major.
#include <mutex>

#include "device_common.h"
#include "kernels.h"

namespace bitnet {

// The allocation-free pack keeps its temporaries here: row sums of up to
// kPackStaticMaxRows rows and the fields of up to kPackStaticMaxSegs segments
// (about 1 MiB per GPU).  In host code this name is a stand-in for the symbol,
// not a device address: host code uses the address from pack_scratch() only.
constexpr size_t kPackScratchBytes =
    (pack_temp_layout(kPackStaticMaxRows, kPackStaticMaxSegs).bytes + 255) / 256 * 256;
static __device__ __align__(256) unsigned char scratch[kPackScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void* g_scratch_ptr[kMaxDevices];

__global__ void clear_status_kernel(unsigned int* status) { *status = 0u; }

template <typename T>
__device__ __forceinline__ float ld(const T* p);
template <>
__device__ __forceinline__ float ld<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }
template <>
__device__ __forceinline__ float ld<float>(const float* p) { return *p; }

constexpr int kRowTile = 64;   // rows per workgroup in row_sum_kernel
constexpr int kKTile = 64;     // k per LDS tile

template <typename T>
__global__ __launch_bounds__(256) void row_sum_kernel(const T* __restrict__ W, int64_t N, int64_t K,
                                                      int64_t ldw, double* __restrict__ row_sum) {
    __shared__ float tile[kRowTile][kKTile + 1];
    const int64_t r0 = static_cast<int64_t>(blockIdx.x) * kRowTile;
    const int tid = threadIdx.x;
    double acc = 0.0;   // used by threads tid < kRowTile
    for (int64_t k0 = 0; k0 < K; k0 += kKTile) {
        for (int i = tid; i < kRowTile * kKTile; i += 256) {
            const int r = i / kKTile, c = i % kKTile;
            const int64_t n = r0 + r, k = k0 + c;
            tile[r][c] = (n < N && k < K) ? ld<T>(W + n * ldw + k) : 0.0f;
        }
        __syncthreads();
        if (tid < kRowTile) {
            const int kmax = static_cast<int>(K - k0 < kKTile ? K - k0 : kKTile);
            for (int c = 0; c < kmax; ++c) acc += fabs(static_cast<double>(tile[tid][c]));
        }
        __syncthreads();
    }
    if (tid < kRowTile && r0 + tid < N) row_sum[r0 + tid] = acc;
}

__global__ void finalize_kernel(const double* __restrict__ row_sum, const int64_t* __restrict__ seg_start,
                                int n_segs, int64_t K, float* __restrict__ seg_mean,
                                unsigned long long* __restrict__ seg_zero, unsigned int* __restrict__ status) {
    const int s = blockIdx.x * blockDim.x + threadIdx.x;
    if (s >= n_segs) return;
    double total = 0.0;
    for (int64_t n = seg_start[s]; n < seg_start[s + 1]; ++n) total += row_sum[n];
    const int64_t rows = seg_start[s + 1] - seg_start[s];
    if (!isfinite(total)) atomicOr(status, 1u);
    seg_mean[s] = static_cast<float>(total / static_cast<double>(rows * K));
    seg_zero[s] = 0ull;
}

__device__ __forceinline__ int segment_of(int64_t n, const int64_t* seg_start, int n_segs) {
    int lo = 0, hi = n_segs - 1;          // last segment whose start <= n
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (seg_start[mid] <= n) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

template <typename T>
__global__ __launch_bounds__(256) void pack_kernel(const T* __restrict__ W, int64_t N, int64_t K,
                                                   int64_t ldw, int64_t Kp,
                                                   const int64_t* __restrict__ seg_start, int n_segs,
                                                   const float* __restrict__ seg_mean,
                                                   unsigned long long* __restrict__ seg_zero,
                                                   uint32_t* __restrict__ packed_words,
                                                   float* __restrict__ w_scale) {
    const int64_t words_per_row = Kp / 16;
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    const bool live = idx < N * words_per_row;
    int zeros = 0;
    int seg = 0;
    if (live) {
        const int64_t n = idx / words_per_row;
        const int64_t j = idx % words_per_row;
        seg = segment_of(n, seg_start, n_segs);
        const float mean = seg_mean[seg];
        const float s = 1.0f / mean;
        uint32_t word = 0;
        const T* wr = W + n * ldw;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t k = 16 * j + e;
            uint32_t u = 1u;                          // padding: weight 0
            if (k < K) {
                const float p = ld<T>(wr + k) * s;
                const int t = (p > 0.5f) - (p < -0.5f);
                u = static_cast<uint32_t>(t + 1);
                zeros += (t == 0);
            }
            const int pair = e / 4, byte = e % 4;     // element 16j+4*pair+byte
            word |= u << (8 * byte + 2 * pair);
        }
        packed_words[idx] = word;
        if (j == 0) w_scale[n] = mean;
    }
    // per-wave zero count; a wave spans at most a few segments
    const int lane = threadIdx.x % kWave;
    const int seg0 = __shfl(seg, 0, kWave);
    const bool same = __all(!live || seg == seg0);
    if (same) {
        const int total = wave_sum(zeros);
        if (lane == 0 && total) atomicAdd(&seg_zero[seg0], static_cast<unsigned long long>(total));
    } else if (live && zeros) {
        atomicAdd(&seg_zero[seg], static_cast<unsigned long long>(zeros));
    }
}


// One thread per (row n, block b): block b of row n covers k = 256b ..
// min(256b + 256, K) - 1 and the packed words 16b .. 16b + 15 that lie below
// Kp / 16.  block_scale is [nb][N].
template <typename T>
__global__ __launch_bounds__(256) void pack_blocked_kernel(const T* __restrict__ W, int64_t N, int64_t K,
                                                           int64_t ldw, int64_t Kp, int64_t nb,
                                                           uint32_t* __restrict__ packed_words,
                                                           float* __restrict__ block_scale,
                                                           unsigned int* __restrict__ status) {
    const int64_t idx = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    if (idx >= N * nb) return;
    const int64_t n = idx / nb, b = idx % nb;
    const int64_t k0 = 256 * b, k1 = k0 + 256 < K ? k0 + 256 : K;
    const T* wr = W + n * ldw;
    double sum = 0.0;
    for (int64_t k = k0; k < k1; ++k) sum += fabs(static_cast<double>(ld<T>(wr + k)));
    if (!isfinite(sum)) atomicOr(status, 1u);
    const float mean = static_cast<float>(sum / static_cast<double>(k1 - k0));
    const float s = 1.0f / mean;
    block_scale[b * N + n] = mean;
    const int64_t words_per_row = Kp / 16;
    for (int64_t j = 16 * b; j < 16 * b + 16 && j < words_per_row; ++j) {
        uint32_t word = 0;
#pragma unroll
        for (int e = 0; e < 16; ++e) {
            const int64_t k = 16 * j + e;
            uint32_t u = 1u;                          // padding: weight 0
            if (k < K) {
                const float p = ld<T>(wr + k) * s;
                u = static_cast<uint32_t>((p > 0.5f) - (p < -0.5f) + 1);
            }
            word |= u << (8 * (e % 4) + 2 * (e / 4));  // element 16j + 4*(e/4) + e%4
        }
        packed_words[n * words_per_row + j] = word;
    }
}

template <typename T>
hipError_t launch_t(const T* W, int64_t N, int64_t K, int64_t ldw, int64_t Kp,
                    const int64_t* seg_start, int n_segs, double* row_sum, float* seg_mean,
                    unsigned long long* seg_zero, unsigned int* status, uint8_t* packed,
                    float* w_scale, hipStream_t stream) {
    clear_status_kernel<<<1, 1, 0, stream>>>(status);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    row_sum_kernel<T><<<static_cast<unsigned>((N + kRowTile - 1) / kRowTile), 256, 0, stream>>>(W, N, K, ldw, row_sum);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    finalize_kernel<<<static_cast<unsigned>((n_segs + 63) / 64), 64, 0, stream>>>(row_sum, seg_start, n_segs, K,
                                                                                seg_mean, seg_zero, status);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    const int64_t words = N * (Kp / 16);
    pack_kernel<T><<<static_cast<unsigned>((words + 255) / 256), 256, 0, stream>>>(
        W, N, K, ldw, Kp, seg_start, n_segs, seg_mean, seg_zero, reinterpret_cast<uint32_t*>(packed), w_scale);
    return hipGetLastError();
}

}  // namespace

hipError_t pack_scratch(void** ptr, size_t* bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {                 // once per device, with that device current
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess) return e;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    *bytes = kPackScratchBytes;
    return hipSuccess;
}

hipError_t launch_pack(const void* W, bool w_bf16, int64_t N, int64_t K, int64_t ldw,
                       int64_t Kp, const int64_t* seg_start_dev, int32_t n_segs,
                       double* row_sum, float* seg_mean_dev, unsigned long long* seg_zero_dev,
                       unsigned int* status_dev, uint8_t* packed, float* w_scale,
                       hipStream_t stream) {
    if (w_bf16)
        return launch_t(static_cast<const uint16_t*>(W), N, K, ldw, Kp, seg_start_dev, n_segs, row_sum,
                        seg_mean_dev, seg_zero_dev, status_dev, packed, w_scale, stream);
    return launch_t(static_cast<const float*>(W), N, K, ldw, Kp, seg_start_dev, n_segs, row_sum,
                    seg_mean_dev, seg_zero_dev, status_dev, packed, w_scale, stream);
}

hipError_t launch_pack_blocked(const void* W, bool w_bf16, int64_t N, int64_t K, int64_t ldw, int64_t Kp,
                               unsigned int* status_dev, uint8_t* packed, float* block_scale, hipStream_t stream) {
    const int64_t nb = (K + 255) / 256;
    const unsigned grid = static_cast<unsigned>((N * nb + 255) / 256);
    if (w_bf16)
        pack_blocked_kernel<uint16_t><<<grid, 256, 0, stream>>>(static_cast<const uint16_t*>(W), N, K, ldw, Kp, nb,
                                                                reinterpret_cast<uint32_t*>(packed), block_scale,
                                                                status_dev);
    else
        pack_blocked_kernel<float><<<grid, 256, 0, stream>>>(static_cast<const float*>(W), N, K, ldw, Kp, nb,
                                                             reinterpret_cast<uint32_t*>(packed), block_scale,
                                                             status_dev);
    return hipGetLastError();
}

}  // namespace bitnet
