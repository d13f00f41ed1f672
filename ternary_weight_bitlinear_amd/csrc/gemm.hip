// gemm.hip -- prefill-size ternary linear on gfx950 int8 MFMA.
//
// Method: acc[m][n] = sum_k q[m][k] * t[n][k], y = acc * (a_scale[m] *
// w_scale[n]) ("BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s1 and
// s2; "BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference
// Optimization Guide", s2: W1.58A8, no bias).  At prefill sizes this is a
// dense int8 contraction, so it runs on v_mfma_i32_16x16x64_i8.
//
// Design.
//  * Workgroup tile BM x BN over K in steps of BK = 128; 4 waves in a 2 x 2
//    grid, each wave owning (BM/2) x (BN/2) of the output as 16x16 MFMA tiles
//    held in int32 accumulators.
//  * Per k-step the workgroup stages the int8 activation tile [BM][BK] and the
//    packed code tile [BN][BK/4] (4x smaller than int8) in LDS, double
//    buffered: the global loads of step k+1 are in flight while step k runs.
//  * Codes stay packed in LDS.  Each lane reads one 32-bit word per 16x16x64
//    MFMA (16 codes of one output row) and expands it in registers with
//    (word >> 2p) & 0x03030303 (7 VALU ops) into the int8 B operand; this keeps
//    LDS traffic and capacity for B at a quarter of an int8 tile.
//  * Stored codes are u = t + 1 in {0,1,2}; the epilogue subtracts q_rowsum[m]
//    to get the exact sum of q*t (the padded tail has q = 0).
//  * Kp is a multiple of 128 = BK, so there is no K tail; ragged M and N are
//    handled by zero-filled loads and guarded stores.
#include "device_common.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int BK = 128;          // k elements per step
constexpr int kApad = 16;        // bytes of padding per LDS activation row
constexpr int kBpad = 4;         // bytes of padding per LDS code row

template <int BM, int BN, bool kOutBf16>
__global__ __launch_bounds__(kThreads) void gemm_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ a_scale,
    const int32_t* __restrict__ q_rowsum, int M, int Kp,
    const uint8_t* __restrict__ packed, const float* __restrict__ w_scale, int N,
    void* __restrict__ y, int64_t ldy, int32_t* __restrict__ acc_debug) {
    constexpr int WM = BM / 2, WN = BN / 2;      // per-wave tile
    constexpr int TM = WM / 16, TN = WN / 16;    // MFMA tiles per wave
    constexpr int A_ROW = BK + kApad;            // LDS bytes per activation row
    constexpr int B_ROW = BK / 4 + kBpad;        // LDS bytes per code row
    constexpr int A_LOADS = BM * BK / 16 / kThreads;   // 16-byte loads per thread
    constexpr int B_LOADS = BN * (BK / 4) / 16 / kThreads;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1, "tile too small for the workgroup");

    __shared__ __attribute__((aligned(16))) int8_t a_lds[2][BM * A_ROW];
    __shared__ __attribute__((aligned(16))) uint8_t b_lds[2][BN * B_ROW];

    const int tid = threadIdx.x;
    const int lane = tid % kWave;
    const int wave = tid / kWave;
    const int wm = wave / 2, wn = wave % 2;
    const int m0 = blockIdx.y * BM;
    const int n0 = blockIdx.x * BN;
    const int64_t brow_bytes = Kp / 4;

    // global -> register staging for one k-step
    uint4 a_reg[A_LOADS];
    uint4 b_reg[B_LOADS];
    auto load_tile = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int f = i * kThreads + tid;       // 16-byte piece index in the tile
            const int r = f / (BK / 16), s = f % (BK / 16);
            const int m = m0 + r;
            a_reg[i] = make_uint4(0u, 0u, 0u, 0u);
            if (m < M)
                a_reg[i] = *reinterpret_cast<const uint4*>(q + static_cast<int64_t>(m) * Kp + k0 + 16 * s);
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 64), s = f % (BK / 64);
            const int n = n0 + r;
            b_reg[i] = make_uint4(0u, 0u, 0u, 0u);   // code 0 rows contribute nothing
            if (n < N)
                b_reg[i] = *reinterpret_cast<const uint4*>(packed + static_cast<int64_t>(n) * brow_bytes +
                                                          k0 / 4 + 16 * s);
        }
    };
    auto store_tile = [&](int stage) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 16), s = f % (BK / 16);
            *reinterpret_cast<uint4*>(&a_lds[stage][r * A_ROW + 16 * s]) = a_reg[i];
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 64), s = f % (BK / 64);
            uint32_t* dst = reinterpret_cast<uint32_t*>(&b_lds[stage][r * B_ROW + 16 * s]);
            dst[0] = b_reg[i].x; dst[1] = b_reg[i].y; dst[2] = b_reg[i].z; dst[3] = b_reg[i].w;
        }
    };

    v4i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j) acc[i][j] = v4i{0, 0, 0, 0};

    const int ksteps = Kp / BK;
    load_tile(0);
    store_tile(0);
    __syncthreads();

    const int row_in = lane % 16;   // A row / B column of this lane inside a 16x16 tile
    const int kgrp = lane / 16;     // which 16 k values of the 64

    for (int ks = 0; ks < ksteps; ++ks) {
        const int stage = ks & 1;
        if (ks + 1 < ksteps) load_tile((ks + 1) * BK);

#pragma unroll
        for (int kk = 0; kk < BK; kk += 64) {
            v4i af[TM];
            v4i bf[TN];
#pragma unroll
            for (int i = 0; i < TM; ++i) {
                const int r = wm * WM + i * 16 + row_in;
                af[i] = *reinterpret_cast<const v4i*>(&a_lds[stage][r * A_ROW + kk + 16 * kgrp]);
            }
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int r = wn * WN + j * 16 + row_in;
                const uint32_t w =
                    *reinterpret_cast<const uint32_t*>(&b_lds[stage][r * B_ROW + kk / 4 + 4 * kgrp]);
                bf[j] = expand_word(w);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma16(af[i], bf[j], acc[i][j]);
        }

        if (ks + 1 < ksteps) {
            store_tile(stage ^ 1);
            __syncthreads();
        }
    }

    // epilogue: lane holds C[4*(lane/16)+r][lane%16] of each 16x16 tile
#pragma unroll
    for (int i = 0; i < TM; ++i) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int m = m0 + wm * WM + i * 16 + 4 * kgrp + r;
            if (m >= M) continue;
            const int32_t rs = q_rowsum[m];
            const float as = a_scale[m];
#pragma unroll
            for (int j = 0; j < TN; ++j) {
                const int n = n0 + wn * WN + j * 16 + row_in;
                if (n >= N) continue;
                const int32_t exact = acc[i][j][r] - rs;
                const float v = static_cast<float>(exact) * (as * w_scale[n]);
                if constexpr (kOutBf16)
                    static_cast<uint16_t*>(y)[m * ldy + n] = f32_to_bf16(v);
                else
                    static_cast<float*>(y)[m * ldy + n] = v;
                if (acc_debug) acc_debug[static_cast<int64_t>(m) * N + n] = exact;
            }
        }
    }
}

}  // namespace

hipError_t launch_gemm(const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                       int64_t M, int64_t Kp, const uint8_t* packed, const float* w_scale,
                       int64_t N, void* y, bool y_bf16, int64_t ldy, int32_t* acc_debug,
                       hipStream_t stream) {
    constexpr int BM = 128, BN = 128;
    const dim3 grid(static_cast<unsigned>((N + BN - 1) / BN), static_cast<unsigned>((M + BM - 1) / BM));
    const dim3 block(kThreads);
    if (y_bf16)
        gemm_kernel<BM, BN, true><<<grid, block, 0, stream>>>(q, a_scale, q_rowsum, (int)M, (int)Kp,
                                                               packed, w_scale, (int)N, y, ldy, acc_debug);
    else
        gemm_kernel<BM, BN, false><<<grid, block, 0, stream>>>(q, a_scale, q_rowsum, (int)M, (int)Kp,
                                                                packed, w_scale, (int)N, y, ldy, acc_debug);
    return hipGetLastError();
}

}  // namespace bitnet
