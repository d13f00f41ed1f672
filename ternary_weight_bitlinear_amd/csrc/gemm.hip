// gemm.hip -- prefill-size ternary linear on gfx950 int8 MFMA.
//
// Method: acc[m][n] = sum_k q[m][k] * t[n][k], y = acc * (a_scale[m] *
// w_scale[n]) ("BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s1 and
// s2; "BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference
// Optimization Guide", s2: W1.58A8, no bias).  At prefill sizes this is a
// dense int8 contraction, so it runs on the matrix cores.
//
// Design.
//  * v_mfma_i32_32x32x32_i8: on gfx950 it runs at about twice the rate of the
//    16x16x64 form (measured ~4.5 vs ~2.6 int8 POPS with registers only).
//    Lane l holds row l%32 of A, column l%32 of B and 16 k values of group
//    l/32; the accumulator's register r holds C[8(r/4) + 4(l/32) + r%4][l%32].
//  * Workgroup tile BM x BN, k stage BK = 128, double-buffered in LDS; waves
//    in a WGM x WGN grid, each owning (BM/WGM) x (BN/WGN) as 32x32 tiles held
//    in accumulation registers.  Global loads of stage k+1 go to registers
//    while stage k is computed, then to the other LDS buffer.
//  * Codes stay packed in LDS (a quarter of an int8 tile).  In one stage lane
//    group g takes the contiguous k range [64g, 64g + 64) of the stage, so its
//    B operand for the whole stage is one 16-byte LDS read (four packed words,
//    one per 32-k step); each word is expanded in registers with
//    (word >> 2p) & 0x03030303 (7 VALU ops per 16 codes).  A uses the same k
//    mapping, so the exact integer sum does not depend on the MFMA's internal
//    k order.
//  * Stored codes are u = t + 1 in {0,1,2}; the epilogue subtracts q_rowsum[m]
//    (the padded tail has q = 0) to get the exact sum of q*t.
//  * LDS rows are padded (A: 144 B, B: 48 B) so that the 16-byte reads of 16
//    consecutive rows fall in distinct bank groups.
//  * Tiles are ordered XCD-aware: consecutive workgroup ids go round-robin to
//    the 8 XCDs, so the id is remapped to give each XCD a contiguous band of
//    tiles that share activation rows in its own L2.
//  * Kp is a multiple of 128 = BK, so there is no K tail; ragged M and N are
//    handled by zero-filled loads and guarded stores.
#include "device_common.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int BK = 128;          // k elements per stage
constexpr int kApad = 16;        // bytes of padding per LDS activation row
constexpr int kBpad = 16;        // bytes of padding per LDS code row
constexpr int kXcds = 8;

__device__ __forceinline__ v16i mfma32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

template <int BM, int BN>
constexpr size_t lds_bytes() {
    return 2 * (static_cast<size_t>(BM) * (BK + kApad) + static_cast<size_t>(BN) * (BK / 4 + kBpad));
}

template <int BM, int BN, int WGM, int WGN, bool kOutBf16>
__global__ __launch_bounds__(WGM * WGN * 64) void gemm_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ a_scale,
    const int32_t* __restrict__ q_rowsum, int M, int Kp,
    const uint8_t* __restrict__ packed, const float* __restrict__ w_scale, int N,
    void* __restrict__ y, int64_t ldy, int32_t* __restrict__ acc_debug, int tiles_m, int tiles_n) {
    constexpr int kThreads = WGM * WGN * 64;
    constexpr int WM = BM / WGM, WN = BN / WGN;      // per-wave tile
    constexpr int TM = WM / 32, TN = WN / 32;        // 32x32 MFMA tiles per wave
    constexpr int A_ROW = BK + kApad;
    constexpr int B_ROW = BK / 4 + kBpad;
    constexpr int A_LOADS = BM * BK / 16 / kThreads; // 16-byte global loads per thread
    constexpr int B_LOADS = BN * (BK / 4) / 16 / kThreads;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1 && TM >= 1 && TN >= 1, "tile shape");
    static_assert(BM * BK / 16 % kThreads == 0 && BN * (BK / 4) / 16 % kThreads == 0, "tile shape");

    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    __shared__ __attribute__((aligned(16))) float as_s[BM];      // a_scale of the tile's rows
    __shared__ __attribute__((aligned(16))) int32_t rs_s[BM];    // q_rowsum of the tile's rows
    int8_t* a_lds = lds;                                           // [2][BM][A_ROW]
    uint8_t* b_lds = reinterpret_cast<uint8_t*>(lds + 2 * BM * A_ROW);   // [2][BN][B_ROW]

    // XCD-aware tile order: workgroup b runs on XCD b % 8; give XCD x the
    // contiguous tile range [x * T/8, (x+1) * T/8), walked n-fastest so the
    // workgroups of one XCD share activation rows.
    const int tiles = tiles_m * tiles_n;
    int tile = blockIdx.x;
    if (tiles % kXcds == 0) tile = (blockIdx.x % kXcds) * (tiles / kXcds) + blockIdx.x / kXcds;
    const int m0 = (tile / tiles_n) * BM;
    const int n0 = (tile % tiles_n) * BN;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = tid / 64;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r32 = lane % 32;     // A row / B column inside a 32x32 tile
    const int g = lane / 32;       // k group: bytes [64g, 64g + 64) of a stage
    const int64_t brow_bytes = Kp / 4;

    u32x4 a_reg[A_LOADS];
    u32x4 b_reg[B_LOADS];
    auto load_stage = [&](int k0) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 16), s = f % (BK / 16);
            const int m = m0 + r;
            a_reg[i] = u32x4{0u, 0u, 0u, 0u};
            if (m < M) a_reg[i] = gload<u32x4>(q + static_cast<int64_t>(m) * Kp + k0 + 16 * s);
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 64), s = f % (BK / 64);
            const int n = n0 + r;
            b_reg[i] = u32x4{0u, 0u, 0u, 0u};          // code 0 rows contribute nothing
            if (n < N) b_reg[i] = gload<u32x4>(packed + static_cast<int64_t>(n) * brow_bytes + k0 / 4 + 16 * s);
        }
    };
    auto store_stage = [&](int st) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 16), s = f % (BK / 16);
            *reinterpret_cast<u32x4*>(a_lds + st * BM * A_ROW + r * A_ROW + 16 * s) = a_reg[i];
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 64), s = f % (BK / 64);
            *reinterpret_cast<u32x4*>(b_lds + st * BN * B_ROW + r * B_ROW + 16 * s) = b_reg[i];
        }
    };

    v16i acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0;

    for (int i = tid; i < BM; i += kThreads) {
        const int m = m0 + i;
        as_s[i] = m < M ? a_scale[m] : 0.0f;
        rs_s[i] = m < M ? q_rowsum[m] : 0;
    }
    const int stages = Kp / BK;
    load_stage(0);
    store_stage(0);
    __syncthreads();

    for (int ks = 0; ks < stages; ++ks) {
        const int st = ks & 1;
        if (ks + 1 < stages) load_stage((ks + 1) * BK);

        const int8_t* a_base = a_lds + st * BM * A_ROW + (wm * WM + r32) * A_ROW + 64 * g;
        const uint8_t* b_base = b_lds + st * BN * B_ROW + (wn * WN + r32) * B_ROW + 16 * g;
        u32x4 bw[TN];
#pragma unroll
        for (int j = 0; j < TN; ++j) bw[j] = *reinterpret_cast<const u32x4*>(b_base + j * 32 * B_ROW);
#pragma unroll
        for (int s = 0; s < 4; ++s) {                  // 32-k steps of the stage
            v4i a[TM];
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = *reinterpret_cast<const v4i*>(a_base + i * 32 * A_ROW + 16 * s);
            v4i b[TN];
#pragma unroll
            for (int j = 0; j < TN; ++j) b[j] = expand_word(bw[j][s]);
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
        }

        if (ks + 1 < stages) {
            store_stage(st ^ 1);
            __syncthreads();
        }
    }

    // epilogue: register r of lane l holds C[8(r/4) + 4g + r%4][r32] of each
    // 32x32 tile; the per-row scale and sum come from LDS, four rows per read
#pragma unroll
    for (int j = 0; j < TN; ++j) {
        const int n = n0 + wn * WN + j * 32 + r32;
        if (n >= N) continue;
        const float ws = w_scale[n];
#pragma unroll
        for (int i = 0; i < TM; ++i) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int row = wm * WM + i * 32 + 8 * rb + 4 * g;          // local row of r = 4rb
                const f32x4 as4 = *reinterpret_cast<const f32x4*>(&as_s[row]);
                const v4i rs4 = *reinterpret_cast<const v4i*>(&rs_s[row]);
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    const int m = m0 + row + rr;
                    if (m >= M) continue;
                    const int32_t exact = acc[i][j][4 * rb + rr] - rs4[rr];
                    const float v = static_cast<float>(exact) * (as4[rr] * ws);
                    if constexpr (kOutBf16)
                        static_cast<__bf16*>(y)[m * ldy + n] = static_cast<__bf16>(v);   // v_cvt_pk_bf16_f32: RNE
                    else
                        static_cast<float*>(y)[m * ldy + n] = v;
                    if (acc_debug) acc_debug[static_cast<int64_t>(m) * N + n] = exact;
                }
            }
        }
    }
}

template <int BM, int BN, int WGM, int WGN>
hipError_t launch_tile(const int8_t* q, const float* a_scale, const int32_t* q_rowsum, int64_t M, int64_t Kp,
                       const uint8_t* packed, const float* w_scale, int64_t N, void* y, bool y_bf16,
                       int64_t ldy, int32_t* acc_debug, hipStream_t stream) {
    const int tiles_m = static_cast<int>((M + BM - 1) / BM);
    const int tiles_n = static_cast<int>((N + BN - 1) / BN);
    constexpr size_t lds = lds_bytes<BM, BN>();
    const dim3 grid(static_cast<unsigned>(tiles_m) * tiles_n), block(WGM * WGN * 64);
    auto kern = y_bf16 ? gemm_kernel<BM, BN, WGM, WGN, true> : gemm_kernel<BM, BN, WGM, WGN, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    kern<<<grid, block, lds, stream>>>(q, a_scale, q_rowsum, (int)M, (int)Kp, packed, w_scale, (int)N, y, ldy,
                                       acc_debug, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                       int64_t M, int64_t Kp, const uint8_t* packed, const float* w_scale,
                       int64_t N, void* y, bool y_bf16, int64_t ldy, int32_t* acc_debug,
                       hipStream_t stream) {
    // 128x128 tiles, 4 waves of 64x64: measured faster than 256x256 on every
    // prefill shape here (more workgroups per CU hide the load latency).
    return launch_tile<128, 128, 2, 2>(q, a_scale, q_rowsum, M, Kp, packed, w_scale, N, y, y_bf16, ldy, acc_debug,
                                       stream);
}

}  // namespace bitnet
