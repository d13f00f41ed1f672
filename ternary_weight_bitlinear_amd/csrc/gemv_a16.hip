// gemv_a16.hip -- the W1.58A16 variant: bf16 or fp16 activations x ternary weights.
//
// "BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s5 (On-device
// gotchas): where the in-graph 8-bit activation quantiser stalled the GPU,
// the path ran with 16-bit activations and ternary weights.  Here
// y[m][n] = w_scale[n] * sum_k x[m][k] * t[n][k] with x in bf16 as given and
// the sum in fp32 on the matrix cores (v_mfma_f32_16x16x32_bf16); the order
// of that sum is the hardware's, so results are held to a bound derived from
// it rather than to exact bits.
//
// Layout as the A8 split-K decode kernel: a workgroup owns 16 output rows and
// 16 tokens; lane group g of wave w takes every 16th 64-code chunk of the row,
// starting at 4w + g, so the 4 waves read contiguous 256-byte runs; partial
// 16 x 16 tiles meet in LDS.  The packed codes go straight into MFMA operands:
// two 2-bit fields of a word (8 consecutive k) become 8 16-bit values, each
// pair by two byte permutes against a 3-entry table of high bytes (fp16 of t;
// bf16 of 2t, whose fp32 sums are exactly twice and are halved).  A operands are 8 consecutive bf16 of the token row,
// read from global memory (L1/L2-resident: every workgroup reads the same
// rows).  Token tiles beyond the first 16 re-read the packed rows, so this is
// a decode-size kernel.
#include "codes_bf16.h"
#include "device_common.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kUnroll = 4;

// kF16: fp16 activations (v_mfma_f32_16x16x32_f16, codes expanded to fp16).
template <bool kOutBf16, bool kF16 = false>
__global__ __launch_bounds__(kThreads) void gemv_a16_kernel(const uint16_t* __restrict__ x, int64_t ldx, int M,
                                                            int K, int Kp, const uint8_t* __restrict__ packed,
                                                            const float* __restrict__ w_scale, int N, void* y,
                                                            int64_t ldy) {
    __shared__ float part[kWaves][16][17];
    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int col = lane % 16;                          // token row (A) and output row (B) of this lane
    const int grp = lane / 16;
    const int n0 = blockIdx.x * 16;
    const int m0 = blockIdx.y * 16;
    const bool n_ok = n0 + col < N;
    const bool m_ok = m0 + col < M;
    const int chunks = Kp / 64;
    const uint8_t* brow = packed + static_cast<int64_t>(n_ok ? n0 + col : 0) * (Kp / 4);
    const uint16_t* xrow = x + static_cast<int64_t>(m_ok ? m0 + col : 0) * ldx;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    // w_scale of this thread's output (token m0 + threadIdx.x / 16, row
    // n0 + threadIdx.x % 16), loaded first so that no memory round trip
    // follows the reduction
    const int em = threadIdx.x / 16, en = n0 + threadIdx.x % 16;
    const bool e_ok = m0 + em < M && en < N;
    const float ws_e = e_ok ? gload<float>(w_scale + en) : 0.0f;

    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    // The loop and its exits are wave-uniform (an MFMA needs the whole wave);
    // a lane group past the last chunk multiplies zeros.
    for (int cw = 4 * wave; cw < chunks; cw += 16 * kUnroll) {
        u32x4 bw[kUnroll];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = cw + grp + 16 * u;
            bw[u] = (n_ok && c < chunks) ? gload<u32x4>(brow + 16 * c) : zero;
        }
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = cw + grp + 16 * u;
            if (cw + 16 * u >= chunks) break;           // wave-uniform: nothing left
#pragma unroll
            for (int j = 0; j < 4; ++j) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int k = 64 * c + 16 * j + 8 * h;       // 8 consecutive k; K % 8 == 0
                    const u32x4 a = (m_ok && c < chunks && k < K) ? gload<u32x4>(xrow + k) : zero;
                    if constexpr (kF16)
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a),
                                                                     __builtin_bit_cast(f16x8, expand_f16(bw[u][j], h)),
                                                                     acc, 0, 0, 0);
                    else
                        acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                                      __builtin_bit_cast(bf16x8, expand_bf16_twice(bw[u][j], h)),
                                                                      acc, 0, 0, 0);
                }
            }
        }
    }
    // lane holds C[m = 4*grp + r][n = col] of this wave's share of k
#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][4 * grp + r][col] = acc[r];
    __syncthreads();
    if (e_ok) {
        const int nc = threadIdx.x % 16;
        float s = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += part[w][em][nc];
        if constexpr (!kF16) s = s * 0.5f;             // the bf16 operand held 2t (exact)
        const float v = s * ws_e;
        if constexpr (kOutBf16)
            gstore<uint16_t>(static_cast<uint16_t*>(y) + (m0 + em) * ldy + en, f32_to_bf16(v));
        else
            gstore<float>(static_cast<float*>(y) + (m0 + em) * ldy + en, v);
    }
}

}  // namespace

hipError_t launch_gemv_a16(const uint16_t* x, int64_t ldx, int64_t M, int64_t K, int64_t Kp, const uint8_t* packed,
                           const float* w_scale, int64_t N, void* y, bool y_bf16, int64_t ldy, hipStream_t stream,
                           bool x_f16) {
    const dim3 grid(static_cast<unsigned>((N + 15) / 16), static_cast<unsigned>((M + 15) / 16)), block(kThreads);
    auto kern = x_f16 ? (y_bf16 ? gemv_a16_kernel<true, true> : gemv_a16_kernel<false, true>)
                      : (y_bf16 ? gemv_a16_kernel<true, false> : gemv_a16_kernel<false, false>);
    kern<<<grid, block, 0, stream>>>(x, ldx, (int)M, (int)K, (int)Kp, packed, w_scale, (int)N, y, ldy);
    return hipGetLastError();
}

}  // namespace bitnet
