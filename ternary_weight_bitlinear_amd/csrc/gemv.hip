// gemv.hip -- decode-size ternary linear (M <= 16 tokens) on gfx950.
//
// Method: acc[m][n] = sum_k q[m][k] * t[n][k] on int8 activation codes and
// ternary weight codes, then y = acc * (a_scale[m] * w_scale[n])
// ("BitVLA -- 1.58-bit Vision-Language-Action on Core AI", s1 for the two
// quantisers, s2 for the per-row scale, the arbitrary K / ragged N the kernel
// must take, and ActQuant running right before the ternary kernel; s3 for
// decode feeding one position at a time, M = 1).
//
// Design (HBM-bound: every packed byte is read exactly once).
//  * A workgroup owns 16*TN output rows n and splits K over its 4 waves.  The
//    packed rows are cut into 16-byte chunks (64 codes); chunk c of every row
//    goes to wave (c/4)%4, lane group c%4, so the 4 waves of a workgroup read
//    256 contiguous bytes of each of its rows per step, 16 bytes per lane
//    (global_load_dwordx4).
//  * Codes are expanded in registers: (word >> 2p) & 0x03030303 gives four
//    stored codes u = t+1 in {0,1,2} as int8 lanes, 7 VALU ops per 16 codes,
//    and feed v_mfma_i32_16x16x64_i8 directly as the B operand.  The A operand
//    is the token rows (row m = lane%16, zero for m >= M).  One MFMA consumes
//    256 packed bytes, so the matrix core does the k-reduction that a dot4
//    kernel would do with 4 VALU dot products and a DPP tree per output.
//  * Because u = t + 1, the MFMA sums q*u; the epilogue subtracts q_rowsum[m]
//    (= sum_k q, zero on the padded tail) to get the exact sum of q*t.
//  * Fused variant: the workgroup first issues its first weight loads, then
//    quantises the M token rows itself (block absmax over K, then q into LDS)
//    while those loads are in flight, so ActQuant costs no extra launch and no
//    HBM round trip of q.  The first workgroup of a problem also stores q,
//    a_scale and q_rowsum when the caller asks for them.
//  * Grouped variant: one launch runs many independent problems (each with
//    its own x, packed weight, scales and y); a workgroup finds its problem by
//    a binary search over the problems' first-tile indices.  This streams a
//    whole set of weights (for example every projection of 30 decoder layers)
//    without paying a launch per matrix.
//  * The 4 per-wave 16x16 int32 partial tiles meet in LDS; the epilogue does
//    the fp32 rescale and writes fp32 or bf16 (and optionally the int32 acc).
#include "device_common.h"
#include "gemv.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

template <bool kXBf16>
__device__ __forceinline__ void load_x8(const void* xrow, int vi, float (&v)[8]) {
    if constexpr (kXBf16) {
        const uint4 w = reinterpret_cast<const uint4*>(xrow)[vi];
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    } else {
        const float4 a = reinterpret_cast<const float4*>(xrow)[2 * vi];
        const float4 b = reinterpret_cast<const float4*>(xrow)[2 * vi + 1];
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// ActQuant of the problem's M token rows into q_lds [M][Kp] (zero tail),
// with a_scale and q_rowsum of each token into as_lds / rs_lds.  Also stores
// them to global memory when `store` is set.  All 256 threads take part.
template <bool kXBf16>
__device__ void quantise_tokens(const GemvProblem& p, int8_t* q_lds, float* as_lds, int* rs_lds,
                                float* red_f, int* red_i, bool store) {
    const int tid = threadIdx.x;
    const int nvec = p.K / 8;
    const size_t esize = kXBf16 ? 2 : 4;
    for (int m = 0; m < p.M; ++m) {
        const void* xrow = static_cast<const char*>(p.x) + static_cast<int64_t>(m) * p.ldx * esize;
        float amax = 0.0f;
        for (int vi = tid; vi < nvec; vi += kThreads) {
            float v[8];
            load_x8<kXBf16>(xrow, vi, v);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
        }
        amax = wave_max(amax);
        if (tid % kWave == 0) red_f[tid / kWave] = amax;
        __syncthreads();
        amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
        const float sa = (amax == 0.0f) ? 0.0f : 127.0f / amax;
        int sum = 0;
        int8_t* qrow = q_lds + m * p.Kp;
        int8_t* qout = store ? p.q_out + static_cast<int64_t>(m) * p.Kp : nullptr;
        for (int vi = tid; vi < p.Kp / 8; vi += kThreads) {
            uint2 packed8 = make_uint2(0u, 0u);
            if (vi < nvec) {
                float v[8];
                load_x8<kXBf16>(xrow, vi, v);
                uint32_t lo = 0, hi = 0;
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const int c = static_cast<int>(fminf(fmaxf(rne(v[e] * sa), -128.0f), 127.0f));
                    sum += c;
                    const uint32_t byte = static_cast<uint32_t>(c) & 0xFFu;
                    if (e < 4) lo |= byte << (8 * e);
                    else hi |= byte << (8 * (e - 4));
                }
                packed8 = make_uint2(lo, hi);
            }
            *reinterpret_cast<uint2*>(qrow + 8 * vi) = packed8;
            if (qout) *reinterpret_cast<uint2*>(qout + 8 * vi) = packed8;
        }
        sum = wave_sum(sum);
        if (tid % kWave == 0) red_i[tid / kWave] = sum;
        __syncthreads();
        if (tid == 0) {
            const int total = red_i[0] + red_i[1] + red_i[2] + red_i[3];
            const float as = (amax == 0.0f) ? 0.0f : amax / 127.0f;
            as_lds[m] = as;
            rs_lds[m] = total;
            if (store) {
                p.a_scale_out[m] = as;
                p.rowsum_out[m] = total;
            }
        }
        __syncthreads();   // red_f / red_i are reused by the next token
    }
}

template <int TN, bool kFused, bool kGrouped, bool kXBf16, bool kOutBf16>
__global__ __launch_bounds__(kThreads) void gemv_kernel(GemvProblem single, const GemvProblem* __restrict__ table,
                                                        int count) {
    extern __shared__ __attribute__((aligned(16))) int8_t q_lds[];   // fused: [M][Kp]
    __shared__ int part[kWaves][TN][16][17];
    __shared__ float red_f[kWaves];
    __shared__ int red_i[kWaves];
    __shared__ float as_lds[16];
    __shared__ int rs_lds[16];

    int tile = blockIdx.x;
    GemvProblem p;
    if constexpr (kGrouped) {
        int lo = 0, hi = count - 1;                 // last problem with tile0 <= blockIdx.x
        while (lo < hi) {
            const int mid = (lo + hi + 1) / 2;
            if (table[mid].tile0 <= tile) lo = mid;
            else hi = mid - 1;
        }
        p = table[lo];
        tile -= p.tile0;
    } else {
        p = single;
    }

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int col = lane % 16;   // output row n (B column) and token m (A row) of this lane
    const int grp = lane / 16;   // chunk within a wave's 4-chunk step
    const int n0 = tile * 16 * TN;
    const bool m_ok = col < p.M;
    const int chunks = p.Kp / 64;  // 16-byte chunks per packed row
    const int steps = (chunks + 15) / 16;
    const int64_t row_bytes = p.Kp / 4;

    const uint8_t* brow[TN];
    bool n_ok[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) {
        const int n = n0 + 16 * t + col;
        n_ok[t] = n < p.N;
        brow[t] = p.packed + static_cast<int64_t>(n_ok[t] ? n : 0) * row_bytes;
    }

    constexpr int kUnroll = (TN >= 4) ? 1 : 4 / TN;
    uint4 bw[kUnroll][TN];
    auto load_b = [&](int s0) {
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = 16 * (s0 + u) + 4 * wave + grp;
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                bw[u][t] = make_uint4(0u, 0u, 0u, 0u);
                if (c < chunks && n_ok[t]) bw[u][t] = *reinterpret_cast<const uint4*>(brow[t] + 16 * c);
            }
        }
    };

    load_b(0);   // first weight loads are in flight during the fused quantisation

    const int8_t* arow;
    if constexpr (kFused) {
        quantise_tokens<kXBf16>(p, q_lds, as_lds, rs_lds, red_f, red_i, p.q_out != nullptr && tile == 0);
        arow = q_lds + (m_ok ? col : 0) * p.Kp;
    } else {
        arow = p.q + static_cast<int64_t>(m_ok ? col : 0) * p.Kp;
    }

    v4i acc[TN];
#pragma unroll
    for (int t = 0; t < TN; ++t) acc[t] = v4i{0, 0, 0, 0};

    for (int s0 = 0; s0 < steps; s0 += kUnroll) {
        v4i a[kUnroll][4];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = 16 * (s0 + u) + 4 * wave + grp;
#pragma unroll
            for (int j = 0; j < 4; ++j) a[u][j] = v4i{0, 0, 0, 0};
            if (c < chunks && m_ok) {
                const v4i* ap = reinterpret_cast<const v4i*>(arow + 64 * c);
#pragma unroll
                for (int j = 0; j < 4; ++j) a[u][j] = ap[j];
            }
        }
        uint4 cur[kUnroll][TN];
#pragma unroll
        for (int u = 0; u < kUnroll; ++u)
#pragma unroll
            for (int t = 0; t < TN; ++t) cur[u][t] = bw[u][t];
        if (s0 + kUnroll < steps) load_b(s0 + kUnroll);   // next weights in flight during the MFMAs
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            if (16 * (s0 + u) + 4 * wave >= chunks) break;  // wave-uniform: nothing left
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                acc[t] = mfma16(a[u][0], expand_word(cur[u][t].x), acc[t]);
                acc[t] = mfma16(a[u][1], expand_word(cur[u][t].y), acc[t]);
                acc[t] = mfma16(a[u][2], expand_word(cur[u][t].z), acc[t]);
                acc[t] = mfma16(a[u][3], expand_word(cur[u][t].w), acc[t]);
            }
        }
    }

#pragma unroll
    for (int t = 0; t < TN; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r) part[wave][t][4 * grp + r][col] = acc[t][r];
    __syncthreads();

    for (int e = threadIdx.x; e < TN * 256; e += kThreads) {
        const int t = e / 256, m = (e / 16) % 16, nc = e % 16;
        const int n = n0 + 16 * t + nc;
        if (m < p.M && n < p.N) {
            int s = 0;
#pragma unroll
            for (int w = 0; w < kWaves; ++w) s += part[w][t][m][nc];
            int32_t rs;
            float as;
            if constexpr (kFused) {
                rs = rs_lds[m];
                as = as_lds[m];
            } else {
                rs = p.q_rowsum[m];
                as = p.a_scale[m];
            }
            const int32_t exact = s - rs;
            const float v = static_cast<float>(exact) * (as * p.w_scale[n]);
            if constexpr (kOutBf16)
                static_cast<uint16_t*>(p.y)[m * p.ldy + n] = f32_to_bf16(v);
            else
                static_cast<float*>(p.y)[m * p.ldy + n] = v;
            if (p.acc_debug) p.acc_debug[static_cast<int64_t>(m) * p.N + n] = exact;
        }
    }
}

template <int TN, bool kFused, bool kGrouped>
hipError_t launch_variant(const GemvProblem& single, const GemvProblem* table, int count, unsigned tiles,
                          size_t lds, bool x_bf16, bool y_bf16, hipStream_t stream) {
    const dim3 grid(tiles), block(kThreads);
#define BITNET_GEMV_LAUNCH(XB, YB) \
    gemv_kernel<TN, kFused, kGrouped, XB, YB><<<grid, block, lds, stream>>>(single, table, count)
    if (x_bf16) {
        if (y_bf16) BITNET_GEMV_LAUNCH(true, true);
        else BITNET_GEMV_LAUNCH(true, false);
    } else {
        if (y_bf16) BITNET_GEMV_LAUNCH(false, true);
        else BITNET_GEMV_LAUNCH(false, false);
    }
#undef BITNET_GEMV_LAUNCH
    return hipGetLastError();
}

constexpr int kTN = 1;   // 16 output rows per workgroup

}  // namespace

int64_t gemv_tiles(int64_t N) { return (N + 16 * kTN - 1) / (16 * kTN); }

hipError_t launch_gemv(const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                       int64_t M, int64_t Kp, const uint8_t* packed, const float* w_scale,
                       int64_t N, void* y, bool y_bf16, int64_t ldy, int32_t* acc_debug,
                       hipStream_t stream) {
    GemvProblem p{};
    p.q = q; p.a_scale = a_scale; p.q_rowsum = q_rowsum;
    p.packed = packed; p.w_scale = w_scale; p.y = y; p.ldy = ldy; p.acc_debug = acc_debug;
    p.M = (int)M; p.N = (int)N; p.Kp = (int)Kp; p.K = (int)Kp;
    return launch_variant<kTN, false, false>(p, nullptr, 0, (unsigned)gemv_tiles(N), 0, true, y_bf16, stream);
}

hipError_t launch_gemv_fused(const GemvProblem& p, bool x_bf16, bool y_bf16, hipStream_t stream) {
    const size_t lds = static_cast<size_t>(p.M) * p.Kp;
    return launch_variant<kTN, true, false>(p, nullptr, 0, (unsigned)gemv_tiles(p.N), lds, x_bf16, y_bf16,
                                            stream);
}

hipError_t launch_gemv_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles, size_t lds,
                               bool fused, bool x_bf16, bool y_bf16, hipStream_t stream) {
    GemvProblem none{};
    if (fused)
        return launch_variant<kTN, true, true>(none, table_dev, count, (unsigned)total_tiles, lds, x_bf16, y_bf16,
                                               stream);
    return launch_variant<kTN, false, true>(none, table_dev, count, (unsigned)total_tiles, 0, x_bf16, y_bf16,
                                            stream);
}

}  // namespace bitnet
