// act_quant.hip -- per-token absmax int8 activation quantisation on gfx950.
//
// Method: "BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s1 (ActQuant
// is per-token int8: round(x*127/max|x|) clamped to [-128, 127]) and
// "BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference Optimization
// Guide", s2 (8-bit absmax activations, per token).  Fixed here: one fp32
// factor sa = 127/amax, q = rne(x*sa), a_scale = amax/127, q = 0 and
// a_scale = 0 for an all-zero token.
//
// The same kernel also runs the step before the path, per-projection RMSNorm
// ("BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference Optimization
// Guide", s3.1: every projection normalises its input with its own weight g
// and rms_norm_eps before ActQuant), optionally on the gated product
// silu(gate) * up that feeds the down projection (same guide, s2: SiLU).
// RMSNorm scales a token by one positive factor r = 1/sqrt(mean(x^2) + eps),
// which ActQuant's codes do not see: the codes are those of z = x * g (fp32
// products) and r enters a_scale = amax(z) * r / 127, evaluated in fp64 with
// the squares summed in fp64.  silu(a) * u is evaluated in fp32 with
// silu_mul of device_common.h (within 4.3 fp32 ulps of the exact value).
//
// One wave per token up to K = 4096, one workgroup per token above (below).
// The kernels are HBM-bound: 2 B read + 1 B written per element for bf16
// input.
#include "device_common.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;

// 8 consecutive elements as fp32, from bf16 or fp32 storage.
template <typename T>
struct Vec8;

template <>
struct Vec8<uint16_t> {
    static __device__ __forceinline__ void load(const uint16_t* p, float (&v)[8]) {
        uint4 w = *reinterpret_cast<const uint4*>(p);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
    static __device__ __forceinline__ void load_scalar(const uint16_t* p, float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = bf16_to_f32(p[i]);
    }
};

template <>
struct Vec8<float> {
    static __device__ __forceinline__ void load(const float* p, float (&v)[8]) {
        float4 a = *reinterpret_cast<const float4*>(p);
        float4 b = *reinterpret_cast<const float4*>(p + 4);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
    static __device__ __forceinline__ void load_scalar(const float* p, float (&v)[8]) {
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = p[i];
    }
};

template <typename T, bool kAligned>
__device__ __forceinline__ void load8(const T* p, float (&v)[8]) {
    if constexpr (kAligned) Vec8<T>::load(p, v);
    else Vec8<T>::load_scalar(p, v);
}

// Quantise 8 values with factor sa; returns their sum, writes 8 int8 codes.
__device__ __forceinline__ int quant8(const float (&v)[8], float sa, uint2& out) {
    uint32_t lo, hi;
    const int sum = quant8_codes(v, sa, lo, hi);
    out = make_uint2(lo, hi);
    return sum;
}

// Input modes: the token itself; RMSNorm of it; RMSNorm of silu(x) * up.
enum { kPlain = 0, kNorm = 1, kGatedNorm = 2 };

// The 8 values whose codes are taken (x, or x * g, or silu(x) * up * g) of
// vector vi, and the fp64 sum of squares of the normalised input's 8 values.
template <typename T, bool kAligned, int kMode>
__device__ __forceinline__ void load_input8(const T* xr, const T* ur, const void* g, bool g_bf16, int vi,
                                            float (&z)[8], double& squares) {
    load8<T, kAligned>(xr + vi * 8, z);
    if constexpr (kMode == kGatedNorm) {
        float u[8];
        load8<T, kAligned>(ur + vi * 8, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = silu_mul(z[e], u[e]);
    }
    if constexpr (kMode != kPlain) {
        float gv[8];
        if (g_bf16) load8<uint16_t, kAligned>(static_cast<const uint16_t*>(g) + vi * 8, gv);
        else load8<float, kAligned>(static_cast<const float*>(g) + vi * 8, gv);
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            squares += static_cast<double>(z[e]) * static_cast<double>(z[e]);
            z[e] = z[e] * gv[e];
        }
    }
}

// One wave per token, four tokens per workgroup: the reductions (absmax, the
// code sum, the fp64 sum of squares) are wave butterflies with no barrier, and
// a lane keeps VPT vectors of 8 values in registers, so a token of up to
// 8 * 64 * VPT elements is read from HBM once with all of its loads in flight
// together.  VPT == 0: any K; the row is read twice (the second read hits L2).
constexpr int kTokensPerBlock = kThreads / kWave;

template <typename T, int VPT, bool kAligned, int kMode>
__global__ __launch_bounds__(kThreads) void act_quant_kernel(
    const T* __restrict__ x, const T* __restrict__ up, int64_t ldx, int M, int K, int Kp,
    const void* __restrict__ g, bool g_bf16, float eps,
    int8_t* __restrict__ q, float* __restrict__ a_scale, int32_t* __restrict__ q_rowsum) {
    const int lane = threadIdx.x % kWave;
    const int64_t m = static_cast<int64_t>(blockIdx.x) * kTokensPerBlock + threadIdx.x / kWave;
    if (m >= M) return;                                 // wave-uniform
    const T* xr = x + m * ldx;
    const T* ur = kMode == kGatedNorm ? up + m * ldx : nullptr;
    int8_t* qr = q + m * static_cast<int64_t>(Kp);
    const int nvec = K / 8;

    float amax = 0.0f;
    double squares = 0.0;
    float v[VPT > 0 ? VPT : 1][8];
    if constexpr (VPT > 0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int vi = lane + i * kWave;
            if (vi < nvec) load_input8<T, kAligned, kMode>(xr, ur, g, g_bf16, vi, v[i], squares);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i)
            if (lane + i * kWave < nvec)
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    } else {
        for (int vi = lane; vi < nvec; vi += kWave) {
            load_input8<T, kAligned, kMode>(xr, ur, g, g_bf16, vi, v[0], squares);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[0][e]));
        }
    }
    amax = wave_max(amax);
    if constexpr (kMode != kPlain) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) squares += __shfl_xor(squares, o, kWave);
    }
    // A zero token (amax == 0, or 127/amax not a finite fp32): sa = 0 gives
    // q = 0, and a_scale is 0.
    const bool zero_token = !(127.0f / amax <= __FLT_MAX__);
    const float sa = zero_token ? 0.0f : 127.0f / amax;

    int sum = 0;
    if constexpr (VPT > 0) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int vi = lane + i * kWave;
            if (vi < nvec) {
                uint2 out;
                sum += quant8(v[i], sa, out);
                *reinterpret_cast<uint2*>(qr + vi * 8) = out;
            }
        }
    } else {
        double unused = 0.0;
        for (int vi = lane; vi < nvec; vi += kWave) {
            load_input8<T, kAligned, kMode>(xr, ur, g, g_bf16, vi, v[0], unused);
            uint2 out;
            sum += quant8(v[0], sa, out);
            *reinterpret_cast<uint2*>(qr + vi * 8) = out;
        }
    }
    // zero tail K..Kp-1 (at most 112 bytes, 8-byte stores)
    for (int vi = nvec + lane; vi < Kp / 8; vi += kWave)
        *reinterpret_cast<uint2*>(qr + vi * 8) = make_uint2(0u, 0u);

    sum = wave_sum(sum);
    if (lane == 0) {
        q_rowsum[m] = sum;
        if (zero_token) {
            a_scale[m] = 0.0f;
        } else if constexpr (kMode == kPlain) {
            a_scale[m] = amax / 127.0f;
        } else {
            const double r = 1.0 / sqrt(squares / static_cast<double>(K) + static_cast<double>(eps));
            a_scale[m] = static_cast<float>(static_cast<double>(amax) * r / 127.0);
        }
    }
}

// One workgroup (four waves) per token for the longer rows, up to
// 8 * kThreads * kTokenVecs elements: a thread keeps at most kTokenVecs
// vectors of 8 values, a quarter of what one wave per token needs per lane
// at K = 8192, so more waves stay resident and a token's loads are all in
// flight at once.  The absmax, the code sum and the fp64 sum of squares are
// wave butterflies joined through LDS (the fp64 sum in another order than the
// one-wave kernel's; codes, absmax and code sums do not depend on the order).
constexpr int kTokenVecs = 4;

template <typename T, bool kAligned, int kMode>
__global__ __launch_bounds__(kThreads) void act_quant_token_kernel(
    const T* __restrict__ x, const T* __restrict__ up, int64_t ldx, int K, int Kp,
    const void* __restrict__ g, bool g_bf16, float eps,
    int8_t* __restrict__ q, float* __restrict__ a_scale, int32_t* __restrict__ q_rowsum) {
    __shared__ float red_f[kTokensPerBlock];
    __shared__ double red_d[kTokensPerBlock];
    __shared__ int red_i[kTokensPerBlock];
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    const int64_t m = blockIdx.x;
    const T* xr = x + m * ldx;
    const T* ur = kMode == kGatedNorm ? up + m * ldx : nullptr;
    int8_t* qr = q + m * static_cast<int64_t>(Kp);
    const int nvec = K / 8;

    float amax = 0.0f;
    double squares = 0.0;
    float v[kTokenVecs][8];
#pragma unroll
    for (int i = 0; i < kTokenVecs; ++i) {
        const int vi = tid + i * kThreads;
        if (vi < nvec) load_input8<T, kAligned, kMode>(xr, ur, g, g_bf16, vi, v[i], squares);
    }
#pragma unroll
    for (int i = 0; i < kTokenVecs; ++i)
        if (tid + i * kThreads < nvec)
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[i][e]));
    amax = wave_max(amax);
    if constexpr (kMode != kPlain) {
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) squares += __shfl_xor(squares, o, kWave);
    }
    if (lane == 0) {
        red_f[wave] = amax;
        red_d[wave] = squares;
    }
    __syncthreads();
    amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
    // A zero token (amax == 0, or 127/amax not a finite fp32): sa = 0 gives
    // q = 0, and a_scale is 0.
    const bool zero_token = !(127.0f / amax <= __FLT_MAX__);
    const float sa = zero_token ? 0.0f : 127.0f / amax;

    int sum = 0;
#pragma unroll
    for (int i = 0; i < kTokenVecs; ++i) {
        const int vi = tid + i * kThreads;
        if (vi < nvec) {
            uint2 out;
            sum += quant8(v[i], sa, out);
            *reinterpret_cast<uint2*>(qr + vi * 8) = out;
        }
    }
    // zero tail K..Kp-1 (at most 112 bytes, 8-byte stores)
    for (int vi = nvec + tid; vi < Kp / 8; vi += kThreads)
        *reinterpret_cast<uint2*>(qr + vi * 8) = make_uint2(0u, 0u);

    sum = wave_sum(sum);
    if (lane == 0) red_i[wave] = sum;
    __syncthreads();
    if (tid == 0) {
        q_rowsum[m] = (red_i[0] + red_i[1]) + (red_i[2] + red_i[3]);
        if (zero_token) {
            a_scale[m] = 0.0f;
        } else if constexpr (kMode == kPlain) {
            a_scale[m] = amax / 127.0f;
        } else {
            const double ss = (red_d[0] + red_d[1]) + (red_d[2] + red_d[3]);
            const double r = 1.0 / sqrt(ss / static_cast<double>(K) + static_cast<double>(eps));
            a_scale[m] = static_cast<float>(static_cast<double>(amax) * r / 127.0);
        }
    }
}

template <typename T, bool kAligned, int kMode>
hipError_t launch_t(const T* x, const T* up, int64_t M, int64_t K, int64_t ldx, const void* g, bool g_bf16,
                    float eps, int8_t* q, float* a_scale, int32_t* q_rowsum, int Kp, hipStream_t stream) {
    const int nvec = static_cast<int>(K / 8);
    const dim3 grid(static_cast<unsigned>((M + kTokensPerBlock - 1) / kTokensPerBlock)), block(kThreads);
    const int vpt = (nvec + kWave - 1) / kWave;
    const int m = static_cast<int>(M), k = static_cast<int>(K);
#define BITNET_AQ_LAUNCH(V)                                                                                    \
    act_quant_kernel<T, V, kAligned, kMode><<<grid, block, 0, stream>>>(x, up, ldx, m, k, Kp, g, g_bf16, eps, q, \
                                                                         a_scale, q_rowsum)
    // one wave per token up to 8 vectors per lane (measured faster at
    // K = 2560 than a workgroup per token: 6.0 against 6.5 us at M = 4096),
    // one workgroup per token above
    if (vpt <= 2) BITNET_AQ_LAUNCH(2);
    else if (vpt <= 4) BITNET_AQ_LAUNCH(4);
    else if (vpt <= 8) BITNET_AQ_LAUNCH(8);
    else if (nvec <= kThreads * kTokenVecs)
        act_quant_token_kernel<T, kAligned, kMode><<<dim3(static_cast<unsigned>(M)), block, 0, stream>>>(
            x, up, ldx, k, Kp, g, g_bf16, eps, q, a_scale, q_rowsum);
    else BITNET_AQ_LAUNCH(0);
#undef BITNET_AQ_LAUNCH
    return hipGetLastError();
}

template <int kMode>
hipError_t launch_mode(const void* x, const void* up, bool x_bf16, int64_t M, int64_t K, int64_t ldx,
                       const void* g, bool g_bf16, float eps, int8_t* q, float* a_scale, int32_t* q_rowsum,
                       int64_t Kp, hipStream_t stream) {
    const size_t esize = x_bf16 ? 2 : 4;
    // 16-byte vector loads of x, up and g, else element loads of all three
    const bool aligned = (reinterpret_cast<uintptr_t>(x) % 16 == 0) && (reinterpret_cast<uintptr_t>(up) % 16 == 0) &&
                         ((ldx * esize) % 16 == 0) && (reinterpret_cast<uintptr_t>(g) % 16 == 0);
    if (x_bf16) {
        auto* p = static_cast<const uint16_t*>(x);
        auto* u = static_cast<const uint16_t*>(up);
        return aligned ? launch_t<uint16_t, true, kMode>(p, u, M, K, ldx, g, g_bf16, eps, q, a_scale, q_rowsum,
                                                          (int)Kp, stream)
                       : launch_t<uint16_t, false, kMode>(p, u, M, K, ldx, g, g_bf16, eps, q, a_scale, q_rowsum,
                                                           (int)Kp, stream);
    }
    auto* p = static_cast<const float*>(x);
    auto* u = static_cast<const float*>(up);
    return aligned ? launch_t<float, true, kMode>(p, u, M, K, ldx, g, g_bf16, eps, q, a_scale, q_rowsum, (int)Kp,
                                                   stream)
                   : launch_t<float, false, kMode>(p, u, M, K, ldx, g, g_bf16, eps, q, a_scale, q_rowsum, (int)Kp,
                                                    stream);
}

}  // namespace

hipError_t launch_act_quant(const void* x, bool x_bf16, int64_t M, int64_t K, int64_t ldx,
                            int8_t* q, float* a_scale, int32_t* q_rowsum, int64_t Kp,
                            hipStream_t stream) {
    return launch_mode<kPlain>(x, nullptr, x_bf16, M, K, ldx, nullptr, false, 0.0f, q, a_scale, q_rowsum, Kp,
                               stream);
}

hipError_t launch_norm_act_quant(const void* x, const void* up, bool x_bf16, int64_t M, int64_t K, int64_t ldx,
                                 const void* norm_w, bool norm_bf16, float eps, int8_t* q, float* a_scale,
                                 int32_t* q_rowsum, int64_t Kp, hipStream_t stream) {
    if (up)
        return launch_mode<kGatedNorm>(x, up, x_bf16, M, K, ldx, norm_w, norm_bf16, eps, q, a_scale, q_rowsum,
                                       Kp, stream);
    return launch_mode<kNorm>(x, nullptr, x_bf16, M, K, ldx, norm_w, norm_bf16, eps, q, a_scale, q_rowsum, Kp,
                              stream);
}

}  // namespace bitnet
