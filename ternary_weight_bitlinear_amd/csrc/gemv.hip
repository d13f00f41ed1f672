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
//  * Codes are expanded in registers: (word >> 2p) & 0x03030303 gives four
//    stored codes u = t+1 in {0,1,2} as int8 lanes, 7 VALU ops per 16 codes,
//    and feed v_mfma_i32_16x16x64_i8 directly as the B operand.  The A operand
//    is the token rows (row m = lane%16, zero for m >= M).  One MFMA consumes
//    256 packed bytes, so the matrix core does the k-reduction that a dot4
//    kernel would do with 4 VALU dot products and a DPP tree per output, and
//    the VALU cost does not grow with M.
//  * Because u = t + 1, the MFMA sums q*u; the epilogue subtracts q_rowsum[m]
//    (= sum_k q, zero on the padded tail) to get the exact sum of q*t.
//  * Packed rows are read as 16-byte chunks (64 codes, global_load_dwordx4).
//  * Fused ActQuant: a workgroup quantises the M token rows itself (block
//    absmax over K, then q into LDS) while its first weight loads are in
//    flight, so ActQuant costs no extra launch and no HBM round trip of q.
//
// Kernels:
//  * split-K (small single calls): a workgroup owns 16 output rows and its 4
//    waves split K; partial 16x16 tiles meet in LDS.  Most workgroups for a
//    small matrix, which is what a latency-bound launch needs.
//  * streaming (grouped launches and large single calls): two workgroups per
//    CU, each owning the 64-row tiles of its share of all k steps; every wave
//    streams its 16 rows through a private LDS ring filled by buffer-to-LDS
//    loads, across tile and problem boundaries (see its section below).  A
//    W1.58A16 version of it takes bf16 token rows on bf16 MFMA.
//  * persistent (groups whose token rows do not fit the streaming kernel's
//    LDS share): the same work split with double-buffered register batches,
//    the ActQuant prologue running when the consumer enters a new problem.
//
// Every global access goes through gload / gstore (global address space), so
// the ring's loads are counted by vmcnt alone and are waited for one at a time.
#include <algorithm>
#include <type_traits>

#include "codes_bf16.h"
#include "device_common.h"
#include "gemv.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;
constexpr int kRsrcWord3 = 0x00020000;          // raw 32-bit buffer access on gfx9-family parts

// Workgroup barrier for data written to LDS by ds_write: waits for this
// wave's LDS operations only.  __syncthreads() would also wait for every
// LDS-bound DMA still in flight (its release fence covers them); callers use
// this one where no other wave reads DMA'd data after the barrier.
__device__ __forceinline__ void barrier_lds() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

// LDS accesses in inline asm.  Once LDS-bound DMAs are in flight, the
// compiler makes every plain LDS access it cannot prove disjoint from their
// targets wait for all of them; these do not (the kernels order them against
// the DMAs themselves, by vmcnt waits and barriers).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}
__device__ __forceinline__ u32x4 lds_read16(const void* p) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p)) : "memory");
    return v;
}
__device__ __forceinline__ float lds_read_f32(const void* p) {
    float v;
    asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_addr(p)) : "memory");
    return v;
}
__device__ __forceinline__ void lds_write_i32(void* p, int32_t v) {
    asm volatile("ds_write_b32 %0, %1" : : "v"(lds_addr(p)), "v"(v) : "memory");
}
// Four 32-bit words 16 bytes apart (one per wave of a [wave][4] array).
__device__ __forceinline__ u32x4 lds_read_4x16(const void* p) {
    u32x4 v;
    asm volatile("ds_read_b32 %0, %4\n\tds_read_b32 %1, %4 offset:16\n\tds_read_b32 %2, %4 offset:32\n\t"
                 "ds_read_b32 %3, %4 offset:48\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(v.x), "=&v"(v.y), "=&v"(v.z), "=&v"(v.w)
                 : "v"(lds_addr(p))
                 : "memory");
    return v;
}

// Tuning knobs (build-time): rows and batch size of the persistent kernel, its
// resident workgroups per CU, and the packed size from which a single call
// uses it instead of split-K.
#ifndef BITNET_PERSIST_TN             // row tiles of 16 rows per wave
#define BITNET_PERSIST_TN 1
#endif
#ifndef BITNET_PERSIST_BATCH          // k steps per double-buffered batch
#define BITNET_PERSIST_BATCH 2
#endif
#ifndef BITNET_PERSIST_PER_CU          // resident workgroups per CU (0: as many as fit)
#define BITNET_PERSIST_PER_CU 0
#endif
#ifndef BITNET_PERSIST_MIN_BYTES
#define BITNET_PERSIST_MIN_BYTES (8ll << 20)
#endif
constexpr int kTN = BITNET_PERSIST_TN;
constexpr int kBatch = BITNET_PERSIST_BATCH;
constexpr int64_t kPersistMinBytes = BITNET_PERSIST_MIN_BYTES;

template <bool kXBf16>
__device__ __forceinline__ void load_x8(const void* xrow, int vi, float (&v)[8]) {
    if constexpr (kXBf16) {
        const u32x4 w = gload<u32x4>(static_cast<const char*>(xrow) + 16 * vi);
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x); v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z); v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    } else {
        const f32x4 a = gload<f32x4>(static_cast<const char*>(xrow) + 32 * vi);
        const f32x4 b = gload<f32x4>(static_cast<const char*>(xrow) + 32 * vi + 16);
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w; v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
}

// ActQuant of the problem's M token rows into q_lds [M][Kp] (zero tail), with
// a_scale and q_rowsum of each token into as_lds / rs_lds; also stored to
// global memory when `store` is set.  All 256 threads take part; each keeps up
// to kCache vectors of 8 elements in registers between the absmax pass and
// the quantise pass (the rest are read again, from L2).
// Position of element k of a token row in the persistent kernel's LDS layout:
// inside every 64-element chunk the 4-byte groups are transposed, element
// 16j + 4p + b going to 16p + 4j + b, so that the 16 elements whose codes sit
// in field p of a lane's four packed words are one contiguous 16-byte read.
__device__ __forceinline__ int perm_pos(int k) {
    return (k & ~63) | (((k >> 2) & 3) << 4) | (((k >> 4) & 3) << 2) | (k & 3);
}

// Row length of a token in the persistent kernel's LDS: zero padded to whole
// batches of k steps, so padded steps read A = 0 and need no branch.
__host__ __device__ __forceinline__ int padded_q_row(int Kp) {
    return (Kp + 256 * kBatch - 1) / (256 * kBatch) * (256 * kBatch);
}

// 8 values whose codes are taken, of vector vi of token row m: x, or with a
// norm weight z = h * g where h = x or h = silu(x) * up (fp32, exp_f32 and
// rcp); `squares` gathers the fp64 sum of h^2 that RMSNorm needs.  The norm
// factor r > 0 is common to the token, so the codes of RMSNorm(h) are those of
// z and r enters a_scale only ("BitNet-Embeddings-0.6B/270M: I2_S Conversion
// and Inference Optimization Guide", s3.1: each projection normalises its
// input with its own weight before ActQuant).
template <bool kXBf16>
__device__ __forceinline__ void load_input8(const GemvProblem& p, const void* xrow, const void* urow, int vi,
                                            float (&z)[8], double& squares) {
    load_x8<kXBf16>(xrow, vi, z);
    if (!p.norm_w) return;
    if (urow) {
        float u[8];
        load_x8<kXBf16>(urow, vi, u);
#pragma unroll
        for (int e = 0; e < 8; ++e) z[e] = silu_mul(z[e], u[e]);
    }
    float g[8];
    if (p.norm_bf16) {
        const u32x4 w = gload<u32x4>(static_cast<const char*>(p.norm_w) + 16 * vi);
        g[0] = bf16_lo(w.x); g[1] = bf16_hi(w.x); g[2] = bf16_lo(w.y); g[3] = bf16_hi(w.y);
        g[4] = bf16_lo(w.z); g[5] = bf16_hi(w.z); g[6] = bf16_lo(w.w); g[7] = bf16_hi(w.w);
    } else {
        const f32x4 lo = gload<f32x4>(static_cast<const char*>(p.norm_w) + 32 * vi);
        const f32x4 hi = gload<f32x4>(static_cast<const char*>(p.norm_w) + 32 * vi + 16);
        g[0] = lo.x; g[1] = lo.y; g[2] = lo.z; g[3] = lo.w; g[4] = hi.x; g[5] = hi.y; g[6] = hi.z; g[7] = hi.w;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        squares += static_cast<double>(z[e]) * static_cast<double>(z[e]);
        z[e] = z[e] * g[e];
    }
}

template <bool kXBf16, int kCache, bool kPerm>
__device__ void quantise_tokens(const GemvProblem& p, int8_t* q_lds, float* as_lds, int* rs_lds,
                                float* red_f, int* red_i, double* red_d, bool store) {
    const int ldq = kPerm ? padded_q_row(p.Kp) : p.Kp;
    const int tid = threadIdx.x;
    const int nvec = p.K / 8;
    const size_t esize = kXBf16 ? 2 : 4;
    const bool norm = p.norm_w != nullptr;
    for (int m = 0; m < p.M; ++m) {
        const void* xrow = static_cast<const char*>(p.x) + static_cast<int64_t>(m) * p.ldx * esize;
        const void* urow = p.up ? static_cast<const char*>(p.up) + static_cast<int64_t>(m) * p.ldx * esize
                                : nullptr;
        float cache[kCache][8];
        float amax = 0.0f;
        double squares = 0.0;
#pragma unroll
        for (int i = 0; i < kCache; ++i) {
            const int vi = tid + i * kThreads;
            if (vi < nvec) {
                load_input8<kXBf16>(p, xrow, urow, vi, cache[i], squares);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(cache[i][e]));
            }
        }
        for (int vi = tid + kCache * kThreads; vi < nvec; vi += kThreads) {
            float v[8];
            load_input8<kXBf16>(p, xrow, urow, vi, v, squares);
#pragma unroll
            for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(v[e]));
        }
        amax = wave_max(amax);
        if (norm) {
#pragma unroll
            for (int o = 32; o > 0; o >>= 1) squares += __shfl_xor(squares, o, kWave);
        }
        if (tid % kWave == 0) {
            red_f[tid / kWave] = amax;
            red_d[tid / kWave] = squares;
        }
        __syncthreads();
        amax = fmaxf(fmaxf(red_f[0], red_f[1]), fmaxf(red_f[2], red_f[3]));
        // a zero token: amax == 0, or 127/amax not a finite fp32
        const bool zero_token = !(127.0f / amax <= __FLT_MAX__);
        const float sa = zero_token ? 0.0f : 127.0f / amax;
        int sum = 0;
        int8_t* qrow = q_lds + m * ldq;
        int8_t* qout = store ? p.q_out + static_cast<int64_t>(m) * p.Kp : nullptr;
        auto quant8 = [&](const float (&v)[8]) {
            uint32_t lo, hi;
            sum += quant8_codes(v, sa, lo, hi);
            return u32x2{lo, hi};
        };
        for (int vi = tid; vi < ldq / 8; vi += kThreads) {
            u32x2 packed8 = {0u, 0u};
            if (vi < nvec) {
                const int i = (vi - tid) / kThreads;
                if (i < kCache) {
#pragma unroll
                    for (int c = 0; c < kCache; ++c)
                        if (c == i) packed8 = quant8(cache[c]);
                } else {
                    float v[8];
                    double unused = 0.0;
                    load_input8<kXBf16>(p, xrow, urow, vi, v, unused);
                    packed8 = quant8(v);
                }
            }
            if constexpr (kPerm) {
                *reinterpret_cast<uint32_t*>(qrow + perm_pos(8 * vi)) = packed8.x;
                *reinterpret_cast<uint32_t*>(qrow + perm_pos(8 * vi + 4)) = packed8.y;
            } else {
                *reinterpret_cast<u32x2*>(qrow + 8 * vi) = packed8;
            }
            if (qout && vi < p.Kp / 8) gstore<u32x2>(qout + 8 * vi, packed8);
        }
        sum = wave_sum(sum);
        if (tid % kWave == 0) red_i[tid / kWave] = sum;
        __syncthreads();
        if (tid == 0) {
            const int total = red_i[0] + red_i[1] + red_i[2] + red_i[3];
            float as = 0.0f;
            if (!zero_token) {
                if (norm) {
                    const double ss = red_d[0] + red_d[1] + red_d[2] + red_d[3];
                    const double r = 1.0 / sqrt(ss / static_cast<double>(p.K) + static_cast<double>(p.eps));
                    as = static_cast<float>(static_cast<double>(amax) * r / 127.0);
                } else {
                    as = amax / 127.0f;
                }
            }
            as_lds[m] = as;
            rs_lds[m] = total;
            if (store) {
                gstore<float>(p.a_scale_out + m, as);
                gstore<int32_t>(p.rowsum_out + m, total);
            }
        }
        __syncthreads();   // red_f / red_i / red_d are reused by the next token
    }
}

// Unfused persistent path: copy the problem's quantised rows q [M][Kp] from
// global memory into the permuted, zero-padded LDS layout, with a_scale and
// q_rowsum into as_lds / rs_lds.
__device__ void stage_tokens(const GemvProblem& p, int8_t* q_lds, float* as_lds, int* rs_lds, bool rowsum = true) {
    const int ldq = padded_q_row(p.Kp);
    __syncthreads();   // every wave is done with the previous problem's rows and scales
    for (int i = threadIdx.x; i < p.M * (ldq / 8); i += kThreads) {
        const int m = i / (ldq / 8), vi = i % (ldq / 8);
        u32x2 v = {0u, 0u};
        if (vi < p.Kp / 8) v = gload<u32x2>(p.q + static_cast<int64_t>(m) * p.Kp + 8 * vi);
        int8_t* qrow = q_lds + m * ldq;
        *reinterpret_cast<uint32_t*>(qrow + perm_pos(8 * vi)) = v.x;
        *reinterpret_cast<uint32_t*>(qrow + perm_pos(8 * vi + 4)) = v.y;
    }
    if (threadIdx.x < p.M) {
        as_lds[threadIdx.x] = gload<float>(p.a_scale + threadIdx.x);
        rs_lds[threadIdx.x] = rowsum ? gload<int32_t>(p.q_rowsum + threadIdx.x) : 0;
    }
    __syncthreads();
}

// y (and optionally acc) of one output: token m, row n of problem p.
// kNt: a non-temporal store, for outputs written after a kernel's loop
// (measured on MI355X: c2 at M = 4 2.8% faster on the streaming kernel, M = 1
// alike); stores inside a loop stay ordinary (non-temporal ones there cost the
// persistent kernel 11% at M = 8).
template <bool kOutBf16, bool kNt = false>
__device__ __forceinline__ void store_output(const GemvProblem& p, int m, int n, int32_t exact, float as, float ws) {
    const float v = static_cast<float>(exact) * (as * ws);
    if constexpr (kOutBf16) {
        uint16_t* const dst = static_cast<uint16_t*>(p.y) + m * p.ldy + n;
        if constexpr (kNt) __builtin_nontemporal_store(static_cast<uint16_t>(f32_to_bf16(v)), dst);
        else gstore<uint16_t>(dst, f32_to_bf16(v));
    } else {
        float* const dst = static_cast<float*>(p.y) + m * p.ldy + n;
        if constexpr (kNt) __builtin_nontemporal_store(v, dst);
        else gstore<float>(dst, v);
    }
    if (p.acc_debug) gstore<int32_t>(p.acc_debug + static_cast<int64_t>(m) * p.N + n, exact);
}

// The four 16-byte A operands (64 k values) of chunk c for token row m.
template <bool kFused>
__device__ __forceinline__ void load_a(const GemvProblem& p, const int8_t* q_lds, int m, bool ok, int c, v4i (&a)[4]) {
#pragma unroll
    for (int j = 0; j < 4; ++j) a[j] = v4i{0, 0, 0, 0};
    if (!ok) return;
    if constexpr (kFused) {
        const v4i* ap = reinterpret_cast<const v4i*>(q_lds + m * p.Kp + 64 * c);
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = ap[j];
    } else {
        const int8_t* ap = p.q + static_cast<int64_t>(m) * p.Kp + 64 * c;
#pragma unroll
        for (int j = 0; j < 4; ++j) a[j] = gload<v4i>(ap + 16 * j);
    }
}

// ------------------------------------------------------------------ split-K

// A workgroup owns 16 output rows; chunk c of every row goes to wave (c/4)%4,
// lane group c%4, so the 4 waves read 256 contiguous bytes of each row per step.
template <bool kFused, bool kXBf16, bool kOutBf16>
__global__ __launch_bounds__(kThreads) void gemv_splitk_kernel(GemvProblem p) {
    extern __shared__ __attribute__((aligned(16))) int8_t q_lds[];   // fused: [M][Kp]
    __shared__ int part[kWaves][16][17];
    __shared__ float red_f[kWaves];
    __shared__ int red_i[kWaves];
    __shared__ double red_d[kWaves];
    __shared__ float as_lds[16];
    __shared__ int rs_lds[16];
    constexpr int kUnroll = 4;

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int col = lane % 16;   // output row n (B column) and token m (A row) of this lane
    const int grp = lane / 16;
    const int n0 = blockIdx.x * 16;
    const bool n_ok = (n0 + col) < p.N;
    const bool m_ok = col < p.M;
    const int chunks = p.Kp / 64;
    const int steps = (chunks + 15) / 16;
    const uint8_t* brow = p.packed + static_cast<int64_t>(n_ok ? n0 + col : 0) * (p.Kp / 4);

    u32x4 bw[kUnroll];
    bool bw_ok[kUnroll];
    auto load_b = [&](int s0) {   // one load per slot, always issued (dummy address when out of range)
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = 16 * (s0 + u) + 4 * wave + grp;
            bw_ok[u] = c < chunks && n_ok;
            bw[u] = gload<u32x4>(bw_ok[u] ? brow + 16 * c : p.packed);
        }
    };
    load_b(0);   // in flight during the fused quantisation
    // the epilogue's scales of this thread's output (token threadIdx.x / 16,
    // row n0 + threadIdx.x % 16), loaded now so that no memory round trip
    // follows the reduction
    const int em = threadIdx.x / 16, en = n0 + threadIdx.x % 16;
    const bool e_ok = em < p.M && en < p.N;
    const float ws_e = e_ok ? gload<float>(p.w_scale + en) : 0.0f;
    int32_t rs_e = 0;
    float as_e = 0.0f;
    if constexpr (!kFused) {
        if (e_ok) {
            rs_e = gload<int32_t>(p.q_rowsum + em);
            as_e = gload<float>(p.a_scale + em);
        }
    }
    if constexpr (kFused)
        quantise_tokens<kXBf16, 4, false>(p, q_lds, as_lds, rs_lds, red_f, red_i, red_d,
                                          p.q_out != nullptr && blockIdx.x == 0);

    v4i acc = {0, 0, 0, 0};
    for (int s0 = 0; s0 < steps; s0 += kUnroll) {
        u32x4 cur[kUnroll];
        const u32x4 zero = {0u, 0u, 0u, 0u};
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) cur[u] = bw_ok[u] ? bw[u] : zero;
        if (s0 + kUnroll < steps) load_b(s0 + kUnroll);
#pragma unroll
        for (int u = 0; u < kUnroll; ++u) {
            const int c = 16 * (s0 + u) + 4 * wave + grp;
            if (16 * (s0 + u) + 4 * wave >= chunks) break;   // wave-uniform: nothing left
            v4i a[4];
            load_a<kFused>(p, q_lds, col, m_ok && c < chunks, c, a);
            acc = mfma16(a[0], expand_word(cur[u].x), acc);
            acc = mfma16(a[1], expand_word(cur[u].y), acc);
            acc = mfma16(a[2], expand_word(cur[u].z), acc);
            acc = mfma16(a[3], expand_word(cur[u].w), acc);
        }
    }

#pragma unroll
    for (int r = 0; r < 4; ++r) part[wave][4 * grp + r][col] = acc[r];
    __syncthreads();

    if (e_ok) {
        const int nc = threadIdx.x % 16;
        int s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += part[w][em][nc];
        if constexpr (kFused) {
            rs_e = rs_lds[em];
            as_e = as_lds[em];
        }
        store_output<kOutBf16>(p, em, en, s - rs_e, as_e, ws_e);
    }
}

// --------------------------------------------------------------- persistent

// Descriptor access for the persistent kernel: a device table (grouped) or
// the single problem passed by value.
template <bool kGrouped>
struct Problems {
    const GemvProblem* table;
    const GemvProblem& single;
    int count;
    __device__ __forceinline__ GemvProblem get(int i) const {
        if constexpr (kGrouped) return table[i];
        else return single;
    }
};

template <bool kGrouped>
__device__ __forceinline__ int find_problem(const Problems<kGrouped>& ps, int tile) {
    int lo = 0, hi = ps.count - 1;              // last problem with tile0 <= tile
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (ps.get(mid).tile0 <= tile) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// The tile boundary nearest to batch `s`: the first tile of the workgroup
// whose share starts at s (total_tiles if none).  Rounding to the nearest
// boundary rather than the next one halves the largest excess of a share over
// its exact part.
template <bool kGrouped>
__device__ __forceinline__ int first_tile_from_step(const Problems<kGrouped>& ps, int64_t s, int total_tiles) {
    int lo = 0, hi = ps.count - 1;              // last problem with step0 <= s
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (ps.get(mid).step0 <= s) lo = mid;
        else hi = mid - 1;
    }
    const GemvProblem p = ps.get(lo);
    const int64_t t = (2 * (s - p.step0) + p.steps) / (2 * p.steps);   // nearest tile start, ties up
    if (t >= p.ntiles) return (lo + 1 < ps.count) ? ps.get(lo + 1).tile0 : total_tiles;
    return p.tile0 + static_cast<int>(t);
}

// Persistent kernel.  kGrouped: problems come from `table` (device memory);
// otherwise the single problem passed by value (tile0 = step0 = 0).
//
// Units: a tile is 64*TN output rows (each wave owns 16*TN of them); a batch
// is U consecutive k steps of a tile (a step is 64 bytes of each row: one
// 16-byte chunk per lane group).  A tile's k steps are padded up to whole
// batches; padding loads re-read an in-range chunk (L2-resident) and meet
// A = 0, so they change nothing.  Batches are double buffered: the loads of the next batch of the
// workgroup's (tile, batch) sequence are issued before the current batch is
// consumed, so U*TN loads per wave stay in flight through the MFMAs, through
// tile epilogues and through the ActQuant prologue of a new problem.  Every
// batch issues exactly U*TN loads and the cursors advance once per batch,
// which keeps the hot loop short.
//
// Code expansion without shifts: for a packed word w, (w & 0x03030303),
// (w & 0x0C0C0C0C), (w & 0x30303030) and ((w >> 1) & 0x60606060) hold the
// codes of fields p = 0..3 scaled by 1, 4, 16 and 32 (all below 128, so they
// are valid int8 MFMA operands): 5 VALU ops per 16 codes.  Each field has its
// own accumulator, divided back exactly in the epilogue.  The token rows sit
// in LDS with the matching permutation (perm_pos), zero padded to a multiple
// of 256, so the A operand of field p is one contiguous 16-byte LDS read and
// tail chunks read zeros.  Lanes whose token row is beyond M never load their
// A registers, which therefore stay zero; rows beyond N are never stored.
template <int TN, int U, bool kFused, bool kGrouped, bool kXBf16, bool kOutBf16>
__global__ __launch_bounds__(kThreads) void gemv_persistent_kernel(GemvProblem single,
                                                                   const GemvProblem* __restrict__ table,
                                                                   int count, int total_tiles,
                                                                   int64_t total_steps) {
    extern __shared__ __attribute__((aligned(16))) int8_t q_lds[];   // [M][padded_q_row(Kp)], permuted
    __shared__ float red_f[kWaves];
    __shared__ int red_i[kWaves];
    __shared__ double red_d[kWaves];
    __shared__ float as_lds[16];
    __shared__ int rs_lds[16];

    const Problems<kGrouped> ps{table, single, count};
    const int64_t s_lo = total_steps * blockIdx.x / gridDim.x;
    const int64_t s_hi = total_steps * (blockIdx.x + 1) / gridDim.x;
    const int t_begin = first_tile_from_step(ps, s_lo, total_tiles);
    const int t_end = first_tile_from_step(ps, s_hi, total_tiles);
    if (t_begin >= t_end) return;                       // workgroup-uniform

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int col = lane % 16;
    const int grp = lane / 16;
    const int p_start = find_problem(ps, t_begin);

    // The workgroup's tiles are walked one problem segment at a time: stage
    // the problem's tokens (ActQuant; every earlier load has landed by then),
    // issue its first two batches, then run a loop that only ever sees this
    // problem, so the loop entry and its back edge have the same loads in
    // flight and each wait is for one batch.
    int pc = p_start;
    GemvProblem P = ps.get(pc);
    const bool m_ok = col < P.M;                        // M is shared by the group
    v4i a[4];                                           // loop-carried; zero where the lane has no token
#pragma unroll
    for (int f = 0; f < 4; ++f) a[f] = v4i{0, 0, 0, 0};
    int seg_begin = t_begin;
    while (true) {
        const int seg_end = min(t_end, P.tile0 + P.ntiles);
        const int chunks = P.Kp / 64;
        const int row_bytes = P.Kp / 4;
        const int8_t* abase = nullptr;                  // token rows in LDS, set once staged

        // producer: next (tile, batch) of this segment; past its end it keeps
        // re-reading the last tile (exactly U*TN loads per batch, never used)
        int tp = seg_begin, bp = 0;
        const uint8_t* prow[TN];
        auto set_rows = [&]() {
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const int n = (tp - P.tile0) * 64 * TN + t * 64 + wave * 16 + col;
                prow[t] = P.packed + static_cast<int64_t>(n < P.N ? n : 0) * row_bytes;
            }
        };
        set_rows();
        auto load_batch = [&](u32x4 (&buf)[U][TN]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int c = 4 * (bp * U + u) + grp;
                const int cc = c < chunks ? c : chunks - 1;
#pragma unroll
                for (int t = 0; t < TN; ++t) buf[u][t] = gload<u32x4>(prow[t] + 16 * cc);
            }
            if (++bp == P.steps) {                      // P.steps = batches per tile
                bp = 0;
                if (tp + 1 < seg_end) {
                    ++tp;
                    set_rows();
                }
            }
        };

        // consumer
        int tc = seg_begin, bc = 0;
        float ws[TN];
        auto prefetch_epilogue = [&]() {                // used after the tile's last batch
#pragma unroll
            for (int t = 0; t < TN; ++t) {
                const int n = (tc - P.tile0) * 64 * TN + t * 64 + wave * 16 + col;
                ws[t] = gload<float>(P.w_scale + (n < P.N ? n : 0));
            }
        };
        v4i acc[TN][4];
#pragma unroll
        for (int t = 0; t < TN; ++t)
#pragma unroll
            for (int f = 0; f < 4; ++f) acc[t][f] = v4i{0, 0, 0, 0};

        auto consume = [&](const u32x4 (&buf)[U][TN]) {
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int s = bc * U + u;               // padding steps read A = 0 from LDS
                if (m_ok) {
                    const v4i* ap = reinterpret_cast<const v4i*>(abase + 256 * s);
#pragma unroll
                    for (int f = 0; f < 4; ++f) a[f] = ap[f];
                }
#pragma unroll
                for (int t = 0; t < TN; ++t) {
                    const u32x4 w = buf[u][t];
                    const v4i b0 = {int(w.x & 0x03030303u), int(w.y & 0x03030303u), int(w.z & 0x03030303u),
                                    int(w.w & 0x03030303u)};
                    const v4i b1 = {int(w.x & 0x0C0C0C0Cu), int(w.y & 0x0C0C0C0Cu), int(w.z & 0x0C0C0C0Cu),
                                    int(w.w & 0x0C0C0C0Cu)};
                    const v4i b2 = {int(w.x & 0x30303030u), int(w.y & 0x30303030u), int(w.z & 0x30303030u),
                                    int(w.w & 0x30303030u)};
                    const v4i b3 = {int((w.x >> 1) & 0x60606060u), int((w.y >> 1) & 0x60606060u),
                                    int((w.z >> 1) & 0x60606060u), int((w.w >> 1) & 0x60606060u)};
                    acc[t][0] = mfma16(a[0], b0, acc[t][0]);
                    acc[t][1] = mfma16(a[1], b1, acc[t][1]);
                    acc[t][2] = mfma16(a[2], b2, acc[t][2]);
                    acc[t][3] = mfma16(a[3], b3, acc[t][3]);
                }
            }
        };
        // after a batch: tile epilogue and cursor advance; true at the segment end
        auto advance = [&]() -> bool {
            if (++bc < P.steps) return false;
            bc = 0;
#pragma unroll
            for (int t = 0; t < TN; ++t) {              // lane holds token m = 4*grp + r of row n
                const int n = (tc - P.tile0) * 64 * TN + t * 64 + wave * 16 + col;
                if (n < P.N) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) {
                        const int m = 4 * grp + r;
                        if (m < P.M) {
                            const int32_t sum_qu = acc[t][0][r] + (acc[t][1][r] >> 2) + (acc[t][2][r] >> 4) +
                                                   (acc[t][3][r] >> 5);
                            store_output<kOutBf16>(P, m, n, sum_qu - rs_lds[m], as_lds[m], ws[t]);
                        }
                    }
                }
#pragma unroll
                for (int f = 0; f < 4; ++f) acc[t][f] = v4i{0, 0, 0, 0};
            }
            if (++tc == seg_end) return true;
            prefetch_epilogue();
            return false;
        };

        // The segment's first weight loads go out before its tokens are
        // staged, so their latency overlaps the ActQuant prologue (whose own
        // loads then wait behind them in the same queue).
        u32x4 bufA[U][TN], bufB[U][TN];
        load_batch(bufA);
        load_batch(bufB);
        prefetch_epilogue();
        if constexpr (kFused)
            quantise_tokens<kXBf16, 2, true>(P, q_lds, as_lds, rs_lds, red_f, red_i, red_d,
                                             P.q_out != nullptr && seg_begin == P.tile0);
        else
            stage_tokens(P, q_lds, as_lds, rs_lds);
        abase = q_lds + (m_ok ? col : 0) * padded_q_row(P.Kp) + 64 * grp;
        while (true) {
            consume(bufA);
            load_batch(bufA);
            if (advance()) break;
            consume(bufB);
            load_batch(bufB);
            if (advance()) break;
        }
        if (seg_end == t_end) break;
        seg_begin = seg_end;
        P = ps.get(++pc);
    }
}

// ActQuant of the token rows of a workgroup's problems, kQuantBatch rows at a
// time (bf16 x, no input norm, K <= 8192, M <= 4 shared by the group; row r
// is token r % M of problem p_first + r / M): every row of a batch is loaded
// into registers before any reduction (quantise_batch_load, which the
// streaming kernel issues ahead of its first weight DMAs so that the first
// batch returns first), and the absmax and row-sum reductions of the batch
// share one barrier each, so a batch pays one memory latency and two barriers
// instead of that per token.  Results are bit-identical to quantise_tokens
// (same fp32 operations per element).
constexpr int kQuantBatch = 4;
constexpr int kQuantVecs = 4;                   // 8-element vectors per thread and row
constexpr int kQuantBatchMaxK = 8 * kThreads * kQuantVecs;
constexpr int kQuantBatchMaxM = 4;

// Host and device test of one problem for the batched quantiser.
__host__ __device__ inline bool quantise_batch_fits(const GemvProblem& P) {
    return P.M <= kQuantBatchMaxM && P.norm_w == nullptr && P.K <= kQuantBatchMaxK;
}

// Position of row r of a batch series: its problem, token and the offset of
// its q row from the first problem's rows (q rows of a problem are [M][ldq]).
struct BatchRow {
    int p, m, qoff;
};

template <typename PS>
__device__ __forceinline__ void quantise_batch_load(const PS& ps, int p_first, int M, int r0, int nrows,
                                                    u32x4 (&raw)[kQuantBatch][kQuantVecs]) {
    // Buffer loads over the row's K bf16 (an empty range past the batch) read
    // zeros beyond it.  The loads are unconditional: straight-line code lets
    // the compiler count exactly how many later memory operations a wait for
    // them may leave in flight.
    const int tid = threadIdx.x;
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        const int r = r0 + (j < nrows ? j : 0);
        const GemvProblem P = ps.get(p_first + r / M);
        const char* xrow = static_cast<const char*>(P.x) + static_cast<int64_t>(r % M) * P.ldx * 2;
        const __amdgpu_buffer_rsrc_t rs =
            __builtin_amdgcn_make_buffer_rsrc(const_cast<char*>(xrow), 0, j < nrows ? 2 * P.K : 0, kRsrcWord3);
#pragma unroll
        for (int i = 0; i < kQuantVecs; ++i)
            raw[j][i] = __builtin_amdgcn_raw_buffer_load_b128(rs, 16 * (tid + i * kThreads), 0, 0);
    }
}

// The rest of a batch of rows from the loaded tokens; `at` is the position of
// its first row and is advanced past the batch.  Ends with a barrier, after
// which q, a_scale and the row sums are visible to the workgroup.
template <typename PS>
__device__ __forceinline__ void quantise_batch(const PS& ps, int p_first, int M, int nrows, BatchRow& at,
                                               const u32x4 (&raw)[kQuantBatch][kQuantVecs], int8_t* q_lds,
                                               float* as_lds, int* rs_lds, float* red_f, int* red_i, int t_begin) {
    const int tid = threadIdx.x, lane = tid % kWave, wave = tid / kWave;
    static_assert(kQuantBatch == 4 && kWaves == 4, "lds_read_4x16 reads one word per wave, 16 bytes apart");
    // problem and token of each row without branches (the loads' waits come
    // before the first barrier); the q offsets after it
    BatchRow rows[kQuantBatch];
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        rows[j].p = at.p + (at.m + j) / M;
        rows[j].m = (at.m + j) % M;
        rows[j].qoff = 0;
    }
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        if (j >= nrows) break;
        const int nvec = ps.get(rows[j].p).K / 8;
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kQuantVecs; ++i) {
            if (i * kThreads >= nvec) break;
            const u32x4 w = raw[j][i];
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_lo(w.x)), fabsf(bf16_hi(w.x))),
                                     fmaxf(fabsf(bf16_lo(w.y)), fabsf(bf16_hi(w.y)))));
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(bf16_lo(w.z)), fabsf(bf16_hi(w.z))),
                                     fmaxf(fabsf(bf16_lo(w.w)), fabsf(bf16_hi(w.w)))));
        }
        amax = wave_max(amax);
        if (lane == 0) lds_write_i32(red_f + wave * kQuantBatch + j, __float_as_int(amax));
    }
    // Every token register is read here, before the barrier, so the waits for
    // the loads all fall in the caller's straight-line code (where they count
    // exactly the loads ahead of the weight DMAs); later reads need none.
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j)
#pragma unroll
        for (int i = 0; i < kQuantVecs; ++i) asm volatile("" : : "v"(raw[j][i]));
    barrier_lds();
    {
        BatchRow c = at;
#pragma unroll
        for (int j = 0; j < kQuantBatch; ++j) {
            if (j >= nrows) break;                      // c stays on problems of the batch
            rows[j].qoff = c.qoff;
            if (++c.m == M) {
                c.qoff += M * padded_q_row(ps.get(c.p).Kp);
                c.m = 0;
                ++c.p;
            }
            if (j + 1 == nrows) at = c;
        }
    }
    int sums[kQuantBatch];
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        sums[j] = 0;
        if (j >= nrows) continue;
        const GemvProblem P = ps.get(rows[j].p);
        const u32x4 wm = lds_read_4x16(red_f + j);            // the waves' maxima
        const float amax = fmaxf(fmaxf(__uint_as_float(wm.x), __uint_as_float(wm.y)),
                                 fmaxf(__uint_as_float(wm.z), __uint_as_float(wm.w)));
        // a zero token: amax == 0, or 127/amax not a finite fp32
        const float sa = !(127.0f / amax <= __FLT_MAX__) ? 0.0f : 127.0f / amax;
        const int ldq = padded_q_row(P.Kp), nvec = P.K / 8;
        int8_t* qrow = q_lds + rows[j].qoff + rows[j].m * ldq;
        int8_t* qout = P.q_out != nullptr && t_begin <= P.tile0 ? P.q_out + static_cast<int64_t>(rows[j].m) * P.Kp
                                                                : nullptr;
#pragma unroll
        for (int i = 0; i < kQuantVecs; ++i) {
            const int vi = tid + i * kThreads;
            if (vi >= ldq / 8) continue;
            uint32_t lo = 0, hi = 0;
            if (vi < nvec) {
                const u32x4 w = raw[j][i];
                const float v[8] = {bf16_lo(w.x), bf16_hi(w.x), bf16_lo(w.y), bf16_hi(w.y),
                                    bf16_lo(w.z), bf16_hi(w.z), bf16_lo(w.w), bf16_hi(w.w)};
                sums[j] += quant8_codes(v, sa, lo, hi);
            }
            lds_write_i32(qrow + perm_pos(8 * vi), static_cast<int32_t>(lo));
            lds_write_i32(qrow + perm_pos(8 * vi + 4), static_cast<int32_t>(hi));
            if (qout && vi < P.Kp / 8) gstore<u32x2>(qout + 8 * vi, u32x2{lo, hi});
        }
    }
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        if (j >= nrows) break;
        const int total = wave_sum(sums[j]);
        if (lane == 0) lds_write_i32(red_i + wave * kQuantBatch + j, total);
    }
    barrier_lds();
    // thread j finishes row j; the problem's fields are read with a
    // workgroup-uniform index (a per-thread index would be a vector load,
    // queued behind every weight DMA already in flight)
#pragma unroll
    for (int j = 0; j < kQuantBatch; ++j) {
        if (j >= nrows) break;
        const GemvProblem P = ps.get(rows[j].p);
        if (tid == j) {
            const u32x4 wm = lds_read_4x16(red_f + j), ws = lds_read_4x16(red_i + j);
            const float amax = fmaxf(fmaxf(__uint_as_float(wm.x), __uint_as_float(wm.y)),
                                     fmaxf(__uint_as_float(wm.z), __uint_as_float(wm.w)));
            const int total = static_cast<int>(ws.x) + static_cast<int>(ws.y) + static_cast<int>(ws.z) +
                              static_cast<int>(ws.w);
            const float as = !(127.0f / amax <= __FLT_MAX__) ? 0.0f : amax / 127.0f;
            const int slot = 16 * (rows[j].p - p_first) + rows[j].m;
            lds_write_i32(as_lds + slot, __float_as_int(as));
            lds_write_i32(rs_lds + slot, total);
            if (P.q_out != nullptr && t_begin <= P.tile0) {
                gstore<float>(P.a_scale_out + rows[j].m, as);
                gstore<int32_t>(P.rowsum_out + rows[j].m, total);
            }
        }
    }
    barrier_lds();                    // red_f / red_i are reused by the next batch
}

// ---------------------------------------------------------------- streaming kernel
//
// Same work split, tiles and MFMA arithmetic as the persistent kernel, with a
// different memory pipeline.  Each wave streams its 16 rows x 64 bytes per k
// step through a private ring of kDepth LDS slots filled by buffer_load ... lds
// (the memory unit writes LDS directly, no registers involved), issued up to
// kDepth - 1 steps ahead of the steps being computed and running straight
// through tile and problem boundaries, so about kDepth KB per wave stay in
// flight at all times.  Lane l's 16 bytes land at slot offset 16*l and are read
// back by lane l alone, so waves never synchronise in the loop; a pass over
// two steps waits for their loads with vmcnt(kDepth - 2).  Every problem the workgroup touches
// is quantised into LDS once, before the loop (its token loads queue behind
// the first ring loads), so a problem boundary only moves the A pointer.
// Rows past N and k past Kp lie outside the buffer range and read as zero.
#ifndef BITNET_STREAM_DEPTH
#define BITNET_STREAM_DEPTH 8
#endif
#ifndef BITNET_STREAM_PER_CU
#define BITNET_STREAM_PER_CU 2
#endif
// Share of a CU's first workgroup relative to its second, in percent (see
// share_start).
#ifndef BITNET_STREAM_FIRST_WEIGHT
#define BITNET_STREAM_FIRST_WEIGHT 126
#endif
constexpr int kDepth = BITNET_STREAM_DEPTH;
constexpr int kStreamMaxProblems = 16;          // problems one workgroup may touch
// Groups of at most this many tokens keep the w_scale of their rows in LDS
// for the output phase; larger ones read it from memory there (one load per
// row after the loop), which leaves the LDS to the [M][rows] exact sums and
// token rows that bound their shares.  Measured on MI355X (c2 group): from
// memory, M = 4 streams 5% faster (4.32 -> 4.54 TB/s: larger shares fit), while
// M = 1 and 2 lose 1.7% to the load's latency at the end of every workgroup.
#ifndef BITNET_STREAM_WS_STAGE_MAX_M
#define BITNET_STREAM_WS_STAGE_MAX_M 2
#endif
// LDS bytes per row of a workgroup's tiles besides the token rows: the M exact
// sums and, when staged, w_scale (the block-scaled kernel keeps the w_scale
// slot unused).
__host__ __device__ inline bool stream_ws_staged(int M, bool blocked) {
    return blocked || M <= BITNET_STREAM_WS_STAGE_MAX_M;
}
constexpr uint32_t kStreamOutOfRange = 0x80000000u;
typedef __attribute__((address_space(3))) void* lds_ptr_t;

__shared__ __attribute__((aligned(1024))) int8_t g_stream_ring[kDepth * kThreads * 16];

// Token rows of the workgroup's problems, then the w_scale of its rows: a
// static array sized to the workgroup's LDS share.
constexpr int kStreamStaticOther = 2 * 4 * kStreamMaxProblems * 16 + 2 * 4 * kWaves + 8 * kWaves + 2 * 4 * kWaves * 4;
constexpr int kStreamQBytes = (160 * 1024 / BITNET_STREAM_PER_CU - kDepth * kThreads * 16 - kStreamStaticOther - 256) / 256 * 256;
static_assert(kStreamQBytes >= 8192, "streaming kernel: too little LDS left for token rows");
static_assert(kThreads * 16 == 4096 && kDepth % 2 == 0, "ring slot stride and pairs of steps");
static_assert(kBatch % 2 == 0, "token rows must be zero padded to whole pairs of k steps");
__shared__ __attribute__((aligned(16))) int8_t g_stream_q[kStreamQBytes];

// Per-256-block weight scales ride the ring too: per step each lane DMAs the
// 4-byte scale of its row into a second ring (kThreads floats per slot), so
// the block-scaled kernel keeps kDepth KB less for token rows.
constexpr int kStreamQBytesBlocked = kStreamQBytes - kDepth * kThreads * 4;
__shared__ __attribute__((aligned(1024))) float g_stream_bs_ring[kDepth * kThreads];
__shared__ __attribute__((aligned(16))) int8_t g_stream_q_blocked[kStreamQBytesBlocked];

template <int kVm>
__device__ __forceinline__ void wait_vm() {     // s_waitcnt vmcnt(kVm), other counters untouched
    static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8));
}

// LDS reads of the streaming loop, each with its completion wait in the same
// asm block.  The compiler does not see these reads, so it adds no wait for
// the ring's DMA loads in flight (it would otherwise order every LDS read
// after all of them); the loop's own vmcnt waits order the ring.
// Two 16-byte words 64 bytes apart.
__device__ __forceinline__ void lds_read_2x16_64(const void* p, u32x4& w0, u32x4& w1) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:64\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(w0), "=&v"(w1)
                 : "v"(lds_addr(p))
                 : "memory");
}
// Two consecutive ring slots of the lane (slot stride kThreads * 16 bytes).
__device__ __forceinline__ void lds_read_ring2(const void* p, u32x4& w0, u32x4& w1) {
    asm volatile("ds_read_b128 %0, %2\n\tds_read_b128 %1, %2 offset:4096\n\ts_waitcnt lgkmcnt(0)"
                 : "=&v"(w0), "=&v"(w1)
                 : "v"(lds_addr(p))
                 : "memory");
}
// A operands of two consecutive k steps (64 + 64 bytes, 256 bytes apart).
__device__ __forceinline__ void lds_read_a2(const void* p, v4i (&a)[2][4]) {
    asm volatile(
        "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:16\n\tds_read_b128 %2, %8 offset:32\n\t"
        "ds_read_b128 %3, %8 offset:48\n\tds_read_b128 %4, %8 offset:256\n\tds_read_b128 %5, %8 offset:272\n\t"
        "ds_read_b128 %6, %8 offset:288\n\tds_read_b128 %7, %8 offset:304\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(a[0][0]), "=&v"(a[0][1]), "=&v"(a[0][2]), "=&v"(a[0][3]), "=&v"(a[1][0]), "=&v"(a[1][1]),
          "=&v"(a[1][2]), "=&v"(a[1][3])
        : "v"(lds_addr(p))
        : "memory");
}
// The lane's ring words of two k steps and, for the lanes set in `rows` (the
// others keep their registers), the 16-bit token-row operands of the same two
// steps (2 x 128 bytes, 512 bytes apart), with one wait for all of them.
__device__ __forceinline__ void lds_read_ring2_x16(const void* ring, const void* x, uint64_t rows, u32x4& w0,
                                                   u32x4& w1, u32x4 (&a)[2][8]) {
    uint64_t save;
    asm volatile(
        "s_mov_b64 %[save], exec\n\t"
        "s_mov_b64 exec, %[rows]\n\t"
        "ds_read_b128 %[a0], %[x]\n\tds_read_b128 %[a1], %[x] offset:16\n\t"
        "ds_read_b128 %[a2], %[x] offset:32\n\tds_read_b128 %[a3], %[x] offset:48\n\t"
        "ds_read_b128 %[a4], %[x] offset:64\n\tds_read_b128 %[a5], %[x] offset:80\n\t"
        "ds_read_b128 %[a6], %[x] offset:96\n\tds_read_b128 %[a7], %[x] offset:112\n\t"
        "ds_read_b128 %[b0], %[x] offset:512\n\tds_read_b128 %[b1], %[x] offset:528\n\t"
        "ds_read_b128 %[b2], %[x] offset:544\n\tds_read_b128 %[b3], %[x] offset:560\n\t"
        "ds_read_b128 %[b4], %[x] offset:576\n\tds_read_b128 %[b5], %[x] offset:592\n\t"
        "ds_read_b128 %[b6], %[x] offset:608\n\tds_read_b128 %[b7], %[x] offset:624\n\t"
        "s_mov_b64 exec, %[save]\n\t"
        "ds_read_b128 %[w0], %[r]\n\tds_read_b128 %[w1], %[r] offset:4096\n\t"
        "s_waitcnt lgkmcnt(0)"
        : [save] "=&s"(save), [w0] "=&v"(w0), [w1] "=&v"(w1), [a0] "+v"(a[0][0]), [a1] "+v"(a[0][1]),
          [a2] "+v"(a[0][2]), [a3] "+v"(a[0][3]), [a4] "+v"(a[0][4]), [a5] "+v"(a[0][5]), [a6] "+v"(a[0][6]),
          [a7] "+v"(a[0][7]), [b0] "+v"(a[1][0]), [b1] "+v"(a[1][1]), [b2] "+v"(a[1][2]), [b3] "+v"(a[1][3]),
          [b4] "+v"(a[1][4]), [b5] "+v"(a[1][5]), [b6] "+v"(a[1][6]), [b7] "+v"(a[1][7])
        : [x] "v"(lds_addr(x)), [r] "v"(lds_addr(ring)), [rows] "s"(rows)
        : "memory");
}
__device__ __forceinline__ void lds_read64(const void* p, v4i (&a)[4]) {
    asm volatile(
        "ds_read_b128 %0, %4\n\tds_read_b128 %1, %4 offset:16\n\tds_read_b128 %2, %4 offset:32\n\t"
        "ds_read_b128 %3, %4 offset:48\n\ts_waitcnt lgkmcnt(0)"
        : "=&v"(a[0]), "=&v"(a[1]), "=&v"(a[2]), "=&v"(a[3])
        : "v"(lds_addr(p))
        : "memory");
}

// First batch of workgroup b's share of the launch's total_steps batches.
// With two workgroups per CU the first n_first workgroups of the grid go one
// to each CU and the rest second.  Measured on MI355X, the first workgroup on
// a CU wins the CU's arbitration and streams about 1.2 to 1.3 times as fast as
// the second, so it gets a share BITNET_STREAM_FIRST_WEIGHT percent of the
// second's and the two finish closer together.  n_first = grid: equal shares.
__host__ __device__ __forceinline__ int64_t share_start(int64_t total_steps, int b, int grid, int n_first) {
    const int64_t f = b < n_first ? b : n_first;
    const int64_t w = BITNET_STREAM_FIRST_WEIGHT * f + 100 * (b - f);
    const int64_t all = BITNET_STREAM_FIRST_WEIGHT * static_cast<int64_t>(n_first) + 100 * (grid - n_first);
    return total_steps * w / all;
}

// k steps of a tile, rounded up to whole pairs (the loop takes two per pass;
// the token rows are zero padded that far, see padded_q_row).
__host__ __device__ __forceinline__ int stream_steps(int Kp) { return ((Kp / 64 + 3) / 4 + 1) / 2 * 2; }

// Tiles [t_begin, t_end) of this workgroup, the first and last problem they
// touch, and whether all of those take the batched quantiser: for a grouped
// launch from the host's records stored after the problem table (the G + 1
// share bounds, then per workgroup {p_first, p_last, batch, 0}), all loaded
// at once; for a single problem its k-step share snapped to the nearest tile
// start.
template <bool kGrouped>
__device__ __forceinline__ void stream_share(const Problems<kGrouped>& ps, const int32_t* bounds, int total_tiles,
                                             int64_t total_steps, int n_first, int& t_begin, int& t_end,
                                             int& p_first, int& p_last, bool& batch) {
    const int G = static_cast<int>(gridDim.x), b = static_cast<int>(blockIdx.x);
    if constexpr (kGrouped) {
        t_begin = bounds[b];
        t_end = bounds[b + 1];
        const int32_t* span = bounds + G + 1 + 4 * b;
        p_first = span[0];
        p_last = span[1];
        batch = span[2] != 0;
        // The planner keeps every record within these bounds (the span indexes
        // kStreamMaxProblems-sized LDS arrays); a record outside them makes
        // the workgroup do nothing rather than touch memory outside its own.
        if (p_first < 0 || p_last < p_first || p_last >= ps.count || p_last - p_first >= kStreamMaxProblems ||
            t_begin < 0 || t_end > total_tiles)
            t_end = t_begin;
    } else {
        t_begin = first_tile_from_step(ps, share_start(total_steps, b, G, n_first), total_tiles);
        t_end = first_tile_from_step(ps, share_start(total_steps, b + 1, G, n_first), total_tiles);
        p_first = p_last = 0;
        batch = quantise_batch_fits(ps.single);
    }
}

__device__ __forceinline__ __amdgpu_buffer_rsrc_t packed_rsrc(const GemvProblem& p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<uint8_t*>(p.packed), 0, p.N * (p.Kp / 4), kRsrcWord3);
}

// Block scales [nb][N] of a block-scaled problem (held in w_scale).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t block_scale_rsrc(const GemvProblem& p) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<float*>(p.w_scale), 0,
                                             (p.K + 255) / 256 * p.N * static_cast<int>(sizeof(float)), kRsrcWord3);
}

//
// kBlocked: weights with one scale per 256-weight block of a row ("BitVLA --
// 1.58-bit Vision-Language-Action on Core AI", s2: the sibling matvec kernel's
// per-256-block scales); the problem's w_scale points to block_scale [nb][N].
// A k step is exactly one block.  Per step the unscaled fields of the codes u
// give sum q*u and an all-ones B operand gives sum q over the same k, so their
// difference is the exact int32 block sum of q*t; it is scaled by the block's
// scale (DMA'd with the codes) and added to fp32 totals in block order, and
// the outputs are y = total * a_scale.
template <bool kFused, bool kGrouped, bool kXBf16, bool kOutBf16, bool kBlocked = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BITNET_STREAM_PER_CU)))
void gemv_stream_kernel(GemvProblem single, const GemvProblem* __restrict__ table,
                        const int32_t* __restrict__ bounds, int count, int total_tiles, int64_t total_steps,
                        int n_first) {
    int8_t* const q_lds = kBlocked ? g_stream_q_blocked : g_stream_q;   // the problems' token rows
    __shared__ float red_f[kWaves];
    __shared__ int red_i[kWaves];
    __shared__ double red_d[kWaves];
    __shared__ float red_fb[kWaves * kQuantBatch];
    __shared__ int red_ib[kWaves * kQuantBatch];
    __shared__ __attribute__((aligned(16))) float as_lds[kStreamMaxProblems * 16];
    __shared__ __attribute__((aligned(16))) int rs_lds[kStreamMaxProblems * 16];

    const Problems<kGrouped> ps{table, single, count};
    int t_begin, t_end, p_first, p_last;                // the host keeps the span within kStreamMaxProblems
    bool batch;
    stream_share(ps, bounds, total_tiles, total_steps, n_first, t_begin, t_end, p_first, p_last, batch);
    if (t_begin >= t_end) return;                       // workgroup-uniform
    batch = batch && kFused && kXBf16;

    const int lane = threadIdx.x % kWave;
    const int wave = threadIdx.x / kWave;
    const int col = lane % 16;
    const int grp = lane / 16;
    int8_t* const ring = g_stream_ring + wave * 1024;   // slot j of this wave: ring + j * kThreads * 16

    // producer: the (tile, step) sequence of the workgroup, kDepth - 1 ahead
    int pp = p_first;
    GemvProblem PP = ps.get(pp);
    __amdgpu_buffer_rsrc_t rsrc = packed_rsrc(PP);
    int tp = t_begin, sp = 0, steps_p = stream_steps(PP.Kp), chunks_p = PP.Kp / 64, slot_p = 0;
    uint32_t rowoff = static_cast<uint32_t>(((tp - PP.tile0) * 64 + wave * 16 + col) * (PP.Kp / 4) + 16 * grp);
    // kBlocked: the lane's row and the buffer of the problem's block scales
    int row_p = (tp - PP.tile0) * 64 + wave * 16 + col, nb_p = (PP.K + 255) / 256;
    __amdgpu_buffer_rsrc_t bs_rsrc = kBlocked ? block_scale_rsrc(PP) : rsrc;
    float* const bs_ring = g_stream_bs_ring + wave * kWave;   // slot j of this wave: bs_ring + j * kThreads
    // the DMA(s) of k step `step` of the current tile into ring slot `slot`
    auto issue = [&](int slot, int step) {
        // chunks past the row (padding steps) read nothing
        const uint32_t off = tp < t_end && 4 * step + grp < chunks_p ? rowoff + 64u * static_cast<uint32_t>(step)
                                                                     : kStreamOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(ring + slot * kThreads * 16), 16, off, 0, 0, 0);
        if constexpr (kBlocked) {
            // block `step` of the lane's row (zero past the last block and past N)
            const uint32_t soff = tp < t_end && step < nb_p && row_p < PP.N
                                      ? static_cast<uint32_t>((step * PP.N + row_p) * 4)
                                      : kStreamOutOfRange;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(bs_rsrc, (lds_ptr_t)(bs_ring + slot * kThreads), 4, soff, 0, 0,
                                                     0);
        }
    };
    // move past the step just issued (to the next tile, the next problem)
    auto advance = [&]() {
        if (tp < t_end && ++sp == steps_p) {
            sp = 0;
            ++tp;
            rowoff += static_cast<uint32_t>(64 * (PP.Kp / 4));
            row_p += 64;
            if (tp < t_end && tp == PP.tile0 + PP.ntiles) {
                PP = ps.get(++pp);
                rsrc = packed_rsrc(PP);
                if constexpr (kBlocked) bs_rsrc = block_scale_rsrc(PP);
                steps_p = stream_steps(PP.Kp);
                chunks_p = PP.Kp / 64;
                rowoff = static_cast<uint32_t>((wave * 16 + col) * (PP.Kp / 4) + 16 * grp);
                row_p = wave * 16 + col;
                nb_p = (PP.K + 255) / 256;
            }
        }
    };
    auto produce = [&]() {
        issue(slot_p, sp);
        slot_p = slot_p + 1 == kDepth ? 0 : slot_p + 1;
        advance();
    };
    constexpr int kDmaPerStep = kBlocked ? 2 : 1;
    static_assert(kDepth >= 4 && kDepth % 2 == 0, "the ring takes two steps per pass");

    // The prologue: the ring's first kDepth - 2 steps (the ring holds kDepth
    // steps: before the pass over steps (k, k+1) the producer has issued up
    // to step k + kDepth - 3, and the pass issues k + kDepth - 2 and
    // k + kDepth - 1 into the slots of k - 2 and k - 1, which the previous
    // pass has read), then the tokens of every problem the workgroup touches
    // and the w_scale of every row of its tiles (one 64-float DMA per tile,
    // after the token rows) into LDS.
    //
    // Batched tokens (M <= 4, no norm): the first batch's token loads go out
    // before any weight DMA, so (loads completing in order) they wait behind
    // none of them.  The
    // prologue comes in two copies: where the ring's first steps all lie in
    // the workgroup's first tile (every K >= 64 * kDepth - 128), its DMAs are
    // straight-line code, and the compiler's waits for the tokens then leave
    // every DMA in flight; otherwise produce() issues them.
    u32x4 raw[kQuantBatch][kQuantVecs];
    const bool ws_staged = stream_ws_staged(PP.M, kBlocked);   // M is shared by the group
    auto prologue = [&](auto straight) __attribute__((always_inline)) {
        const int group_m = PP.M;                       // M is shared by the group
        const int batch_rows = (p_last - p_first + 1) * group_m;
        if (batch) quantise_batch_load(ps, p_first, group_m, 0, min(kQuantBatch, batch_rows), raw);
        if constexpr (decltype(straight)::value) {
#pragma unroll
            for (int i = 0; i < kDepth - 2; ++i) issue(i, i);
            slot_p = kDepth - 2;
            sp = kDepth - 3;
            advance();
        } else {
#pragma unroll
            for (int i = 0; i < kDepth - 2; ++i) produce();
        }
        int q_bytes = 0;
        for (int pi = p_first; pi <= p_last; ++pi) q_bytes += group_m * padded_q_row(ps.get(pi).Kp);
        int8_t* ws_lds = q_lds + q_bytes;
        auto stage_w_scale = [&]() {
            for (int pi = p_first; pi <= p_last && !kBlocked; ++pi) {
                const GemvProblem Pi = ps.get(pi);
                const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<float*>(Pi.w_scale), 0, Pi.N * static_cast<int>(sizeof(float)), kRsrcWord3);
                const int t0 = max(t_begin, Pi.tile0), t1 = min(t_end, Pi.tile0 + Pi.ntiles);
                for (int t = t0 + wave; t < t1; t += kWaves)   // rows past N read as zero
                    __builtin_amdgcn_raw_ptr_buffer_load_lds(
                        ws_rsrc, (lds_ptr_t)(ws_lds + (t - t_begin) * 64 * sizeof(float)), 4,
                        static_cast<uint32_t>(((t - Pi.tile0) * 64 + lane) * sizeof(float)), 0, 0, 0);
            }
        };
        if (batch) {
            // kQuantBatch token rows per pass; the batch ends with a barrier
            // that publishes q, a_scale and the row sums.
            // The ring needs no barrier (each wave reads only what its own
            // DMAs wrote, after its own vmcnt wait), and w_scale is read only
            // after the loop's final wait and barrier, so its DMAs go out last.
            // The first batch is kept out of the loop so that its waits count
            // only the token loads ahead of the ring's DMAs.
            BatchRow at{p_first, 0, 0};
            quantise_batch(ps, p_first, group_m, min(kQuantBatch, batch_rows), at, raw, q_lds, as_lds, rs_lds,
                           red_fb, red_ib, t_begin);
            for (int r = kQuantBatch; r < batch_rows; r += kQuantBatch) {
                const int nr = min(kQuantBatch, batch_rows - r);
                quantise_batch_load(ps, p_first, group_m, r, nr, raw);
                quantise_batch(ps, p_first, group_m, nr, at, raw, q_lds, as_lds, rs_lds, red_fb, red_ib, t_begin);
            }
            if (ws_staged) stage_w_scale();
        } else {
            // the DMAs go out first; the token loads queue behind them and
            // behind the ring's first loads, so one memory latency covers all
            if (ws_staged) stage_w_scale();
            int off = 0;
            for (int pi = p_first; pi <= p_last; ++pi) {
                const GemvProblem Pi = ps.get(pi);
                const int j = pi - p_first;
                if constexpr (kFused)
                    quantise_tokens<kXBf16, 2, true>(Pi, q_lds + off, as_lds + 16 * j, rs_lds + 16 * j, red_f, red_i,
                                                     red_d, Pi.q_out != nullptr && t_begin <= Pi.tile0);
                else
                    stage_tokens(Pi, q_lds + off, as_lds + 16 * j, rs_lds + 16 * j, !kBlocked);
                off += Pi.M * padded_q_row(Pi.Kp);
            }
            // Every wave's DMAs so far (ring, w_scale, staged tokens) have
            // landed once its own vmcnt drains; then the barrier makes them
            // visible to all waves.
            wait_vm<0>();
            __syncthreads();
        }
    };
    if (steps_p >= kDepth - 2) prologue(std::true_type{});
    else prologue(std::false_type{});

    // LDS after the token rows: w_scale of the workgroup's rows, the exact
    // sums [M][rows], and (kBlocked) the block sums [step][16] per problem
    int q_total = 0;
    for (int pi = p_first; pi <= p_last; ++pi) {
        const GemvProblem Pi = ps.get(pi);
        q_total += Pi.M * padded_q_row(Pi.Kp);
    }
    const int wg_rows = (t_end - t_begin) * 64;
    const float* ws_lds = reinterpret_cast<const float*>(q_lds + q_total);
    int32_t* out_lds = reinterpret_cast<int32_t*>(q_lds + q_total) + (ws_staged ? wg_rows : 0);   // [M][wg_rows] exact sums
    int32_t* const bsum_lds = out_lds + ps.get(p_first).M * wg_rows;

    // kBlocked: the exact sum of q over each 256-k block (one k step) per
    // problem, block and token -- the term sum q that turns sum q*u into
    // sum q*t, the same for every row of a problem, so taken once here rather
    // than by a second matrix product per step.  Tokens past M hold zero.
    // One (block, token) pair per thread; q rows are permuted only within
    // 64-byte groups, so a block is 256 consecutive bytes of its row.
    if constexpr (kBlocked) {
        int qo = 0, bo = 0;
        for (int pi = p_first; pi <= p_last; ++pi) {
            const GemvProblem Pi = ps.get(pi);
            const int nsteps = stream_steps(Pi.Kp), ldq = padded_q_row(Pi.Kp);
            for (int e = threadIdx.x; e < nsteps * 16; e += kThreads) {
                const int b = e / 16, m = e % 16;
                int v = 0;
                if (m < Pi.M) {
                    const int8_t* src = q_lds + qo + m * ldq + 256 * b;
#pragma unroll
                    for (int c = 0; c < 4; ++c) {
                        v4i x[4];
                        lds_read64(src + 64 * c, x);
#pragma unroll
                        for (int f = 0; f < 4; ++f)
#pragma unroll
                            for (int d = 0; d < 4; ++d) v = __builtin_amdgcn_sdot4(x[f][d], 0x01010101, v, false);
                    }
                }
                lds_write_i32(bsum_lds + bo + e, v);
            }
            qo += Pi.M * ldq;
            bo += nsteps * 16;
        }
        barrier_lds();
    }

    // consumer
    int pc = p_first, pj = 0, tc = t_begin, sc = 0, slot_c = 0;
    const int32_t* bsum_c = bsum_lds;                   // kBlocked: the current problem's block sums
    GemvProblem P = ps.get(pc);
    int steps_c = stream_steps(P.Kp);
    int qoff = 0;
    const bool m_ok = col < P.M;                        // M is shared by the group
    const int8_t* abase = q_lds + (m_ok ? col : 0) * padded_q_row(P.Kp) + 64 * grp;
    // q_rowsum of tokens 4*grp .. 4*grp+3 of the current problem
    u32x4 rs4 = lds_read16(rs_lds + 4 * grp);
    v4i acc[4];
#pragma unroll
    for (int f = 0; f < 4; ++f) acc[f] = v4i{0, 0, 0, 0};
    float total[4] = {0.0f, 0.0f, 0.0f, 0.0f};           // kBlocked: fp32 sums of scaled block sums
    v4i a[2][4];                                        // zero where the lane has no token
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int f = 0; f < 4; ++f) a[i][f] = v4i{0, 0, 0, 0};

    // two k steps per pass
    while (true) {
        produce();
        produce();
        wait_vm<kDmaPerStep * (kDepth - 2)>();          // both steps' ring loads have landed
        u32x4 w[2];
        lds_read_ring2(ring + slot_c * kThreads * 16 + 16 * lane, w[0], w[1]);
        float bsc[2] = {0.0f, 0.0f};
        if constexpr (kBlocked) {
            bsc[0] = lds_read_f32(bs_ring + slot_c * kThreads + lane);
            bsc[1] = lds_read_f32(bs_ring + (slot_c + 1) * kThreads + lane);
        }
        slot_c = slot_c + 2 == kDepth ? 0 : slot_c + 2;
        if (m_ok) lds_read_a2(abase + 256 * sc, a);
        u32x4 sq[2];                                    // kBlocked: sum q over the two blocks, tokens 4*grp + r
        if constexpr (kBlocked) lds_read_2x16_64(bsum_c + 16 * sc + 4 * grp, sq[0], sq[1]);
#pragma unroll
        for (int i = 0; i < 2 && kBlocked; ++i) {
            const u32x4 v = w[i];
            v4i su = {0, 0, 0, 0};
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const v4i bf = {int((v.x >> (2 * f)) & 0x03030303u), int((v.y >> (2 * f)) & 0x03030303u),
                                int((v.z >> (2 * f)) & 0x03030303u), int((v.w >> (2 * f)) & 0x03030303u)};
                su = mfma16(a[i][f], bf, su);          // sum q * u over the block
            }
            // block order, fp32: total = total + (float)(exact block sum) * scale
#pragma unroll
            for (int r = 0; r < 4; ++r)
                total[r] = total[r] + static_cast<float>(su[r] - static_cast<int32_t>(sq[i][r])) * bsc[i];
        }
#pragma unroll
        for (int i = 0; i < 2 && !kBlocked; ++i) {
            const u32x4 v = w[i];
            const v4i b0 = {int(v.x & 0x03030303u), int(v.y & 0x03030303u), int(v.z & 0x03030303u),
                            int(v.w & 0x03030303u)};
            const v4i b1 = {int(v.x & 0x0C0C0C0Cu), int(v.y & 0x0C0C0C0Cu), int(v.z & 0x0C0C0C0Cu),
                            int(v.w & 0x0C0C0C0Cu)};
            const v4i b2 = {int(v.x & 0x30303030u), int(v.y & 0x30303030u), int(v.z & 0x30303030u),
                            int(v.w & 0x30303030u)};
            const v4i b3 = {int((v.x >> 1) & 0x60606060u), int((v.y >> 1) & 0x60606060u),
                            int((v.z >> 1) & 0x60606060u), int((v.w >> 1) & 0x60606060u)};
            acc[0] = mfma16(a[i][0], b0, acc[0]);
            acc[1] = mfma16(a[i][1], b1, acc[1]);
            acc[2] = mfma16(a[i][2], b2, acc[2]);
            acc[3] = mfma16(a[i][3], b3, acc[3]);
        }
        sc += 2;
        if (sc < steps_c) continue;
        // tile epilogue: lane holds token m = 4*grp + r of row n; the exact sum
        // goes to LDS (a global store here would sit in the ring's in-order
        // queue); the scaled outputs are written after the loop
        sc = 0;
        {
            const int row = (tc - t_begin) * 64 + wave * 16 + col;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * grp + r;
                if (m < P.M) {
                    if constexpr (kBlocked) {
                        lds_write_i32(out_lds + m * wg_rows + row, __float_as_int(total[r]));
                    } else {
                        const int32_t sum_qu = acc[0][r] + (acc[1][r] >> 2) + (acc[2][r] >> 4) + (acc[3][r] >> 5);
                        lds_write_i32(out_lds + m * wg_rows + row, sum_qu - static_cast<int32_t>(rs4[r]));
                    }
                }
            }
        }
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[f] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int r = 0; r < 4; ++r) total[r] = 0.0f;
        if (++tc == t_end) break;
        if (tc == P.tile0 + P.ntiles) {
            qoff += P.M * padded_q_row(P.Kp);
            bsum_c += 16 * steps_c;
            P = ps.get(++pc);
            ++pj;
            steps_c = stream_steps(P.Kp);
            abase = q_lds + qoff + (m_ok ? col : 0) * padded_q_row(P.Kp) + 64 * grp;
            rs4 = lds_read16(rs_lds + 16 * pj + 4 * grp);
        }
    }
    wait_vm<0>();                                       // ring loads past the end land before the LDS is reused
    __syncthreads();

    // outputs of the workgroup's rows, problem by problem, consecutive threads
    // on consecutive rows
    for (int pi = p_first, j = 0; pi <= p_last; ++pi, ++j) {
        const GemvProblem Pi = ps.get(pi);
        const int t0 = max(t_begin, Pi.tile0), t1 = min(t_end, Pi.tile0 + Pi.ntiles);
        const int n0 = (t0 - Pi.tile0) * 64, lrow0 = (t0 - t_begin) * 64;
        const int rows = min((t1 - t0) * 64, Pi.N - n0);         // rows past N have no output
        if (!kBlocked && !ws_staged) {
            // w_scale from memory, once per row for all of its tokens
            for (int rr = threadIdx.x; rr < rows; rr += kThreads) {
                const float ws = gload<float>(Pi.w_scale + n0 + rr);
                for (int m = 0; m < Pi.M; ++m)
                    store_output<kOutBf16, true>(Pi, m, n0 + rr, out_lds[m * wg_rows + lrow0 + rr], as_lds[16 * j + m], ws);
            }
            continue;
        }
        for (int m = 0; m < Pi.M; ++m) {
            const float as = as_lds[16 * j + m];
            const int32_t* const sums = out_lds + m * wg_rows + lrow0;
#pragma unroll 4
            for (int rr = threadIdx.x; rr < rows; rr += kThreads) {
                if constexpr (kBlocked) {
                    const float v = __int_as_float(sums[rr]) * as;
                    if constexpr (kOutBf16)
                        gstore<uint16_t>(static_cast<uint16_t*>(Pi.y) + m * Pi.ldy + n0 + rr, f32_to_bf16(v));
                    else
                        gstore<float>(static_cast<float*>(Pi.y) + m * Pi.ldy + n0 + rr, v);
                } else {
                    store_output<kOutBf16, true>(Pi, m, n0 + rr, sums[rr], as, ws_lds[lrow0 + rr]);
                }
            }
        }
    }
}

// ------------------------------------------------------ W1.58A16 streaming kernel
//
// The grouped W1.58A16 decode ("BitVLA -- 1.58-bit Vision-Language-Action on
// Core AI", s5: 16-bit activations with the ternary weights): the streaming
// kernel's work split, tiles and memory pipeline, with the bf16 (or, kF16,
// fp16) token rows copied into LDS unquantised and each lane's 16 bytes of
// codes (64 k of one row) expanded into the B operands of eight
// v_mfma_f32_16x16x32_bf16 (v_mfma_f32_16x16x32_f16).  Lane group g of a
// wave takes the 16-byte chunk 4s + g of k step s, as in the int8 kernel;
// its A operands are the 64 token-row values at the same k (128 bytes of
// LDS).  The B operand is 2t, one packed 16-bit multiply-add per two values
// (expand_twice_interleaved), in the k order 0 2 1 3 within each 4, and the
// LDS copy of x is stored in that order, so each MFMA still pairs x[m][k]
// with t[n][k]; the fp32 sums, exactly twice those of t, are halved and
// scaled by w_scale.  Per pass (two k steps) one LDS wait covers the ring
// words and the token rows.

template <bool kGrouped, bool kOutBf16, bool kF16 = false>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(BITNET_STREAM_PER_CU)))
void gemv_stream_a16_kernel(GemvProblem single, const GemvProblem* __restrict__ table,
                            const int32_t* __restrict__ bounds, int count, int total_tiles, int64_t total_steps,
                            int n_first) {
    uint16_t* const x_lds = reinterpret_cast<uint16_t*>(g_stream_q);   // bf16 token rows of the problems

    const Problems<kGrouped> ps{table, single, count};
    int t_begin, t_end, p_first, p_last;                // the host keeps the span within kStreamMaxProblems
    bool batch;                                         // (no quantiser here)
    stream_share(ps, bounds, total_tiles, total_steps, n_first, t_begin, t_end, p_first, p_last, batch);
    if (t_begin >= t_end) return;                       // workgroup-uniform

    const int lane = threadIdx.x % kWave;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);   // scalar ring addresses
    const int col = lane % 16;
    const int grp = lane / 16;
    int8_t* const ring = g_stream_ring + wave * 1024;   // slot j of this wave: ring + j * kThreads * 16

    // producer: as in gemv_stream_kernel
    int pp = p_first;
    GemvProblem PP = ps.get(pp);
    __amdgpu_buffer_rsrc_t rsrc = packed_rsrc(PP);
    int tp = t_begin, sp = 0, steps_p = stream_steps(PP.Kp), chunks_p = PP.Kp / 64, slot_p = 0;
    uint32_t rowoff = static_cast<uint32_t>(((tp - PP.tile0) * 64 + wave * 16 + col) * (PP.Kp / 4) + 16 * grp);
    auto next_tile = [&]() {
        sp = 0;
        ++tp;
        rowoff += static_cast<uint32_t>(64 * (PP.Kp / 4));
        if (tp < t_end && tp == PP.tile0 + PP.ntiles) {
            PP = ps.get(++pp);
            rsrc = packed_rsrc(PP);
            steps_p = stream_steps(PP.Kp);
            chunks_p = PP.Kp / 64;
            rowoff = static_cast<uint32_t>((wave * 16 + col) * (PP.Kp / 4) + 16 * grp);
        }
    };
    auto produce = [&]() {
        const uint32_t off = tp < t_end && 4 * sp + grp < chunks_p ? rowoff + 64u * static_cast<uint32_t>(sp)
                                                                   : kStreamOutOfRange;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rsrc, (lds_ptr_t)(ring + slot_p * kThreads * 16), 16, off, 0, 0, 0);
        slot_p = slot_p + 1 == kDepth ? 0 : slot_p + 1;
        if (tp < t_end && ++sp == steps_p) next_tile();
    };
#pragma unroll
    for (int i = 0; i < kDepth - 2; ++i) produce();

    // w_scale of the workgroup's rows (DMA behind the ring's first loads), then
    // the token rows of its problems: x [M][K] bf16, zero padded to
    // padded_q_row(Kp) elements so padded k steps multiply zeros
    int x_elems = 0;
    for (int pi = p_first; pi <= p_last; ++pi) {
        const GemvProblem Pi = ps.get(pi);
        x_elems += Pi.M * padded_q_row(Pi.Kp);
    }
    float* const ws_lds = reinterpret_cast<float*>(x_lds + x_elems);
    {
        for (int pi = p_first; pi <= p_last; ++pi) {
            const GemvProblem Pi = ps.get(pi);
            const __amdgpu_buffer_rsrc_t ws_rsrc = __builtin_amdgcn_make_buffer_rsrc(
                const_cast<float*>(Pi.w_scale), 0, Pi.N * static_cast<int>(sizeof(float)), kRsrcWord3);
            const int t0 = max(t_begin, Pi.tile0), t1 = min(t_end, Pi.tile0 + Pi.ntiles);
            for (int t = t0 + wave; t < t1; t += kWaves)   // rows past N read as zero
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    ws_rsrc, (lds_ptr_t)(ws_lds + (t - t_begin) * 64), 4,
                    static_cast<uint32_t>(((t - Pi.tile0) * 64 + lane) * sizeof(float)), 0, 0, 0);
        }
        int off = 0;
        for (int pi = p_first; pi <= p_last; ++pi) {
            const GemvProblem Pi = ps.get(pi);
            const int ldq = padded_q_row(Pi.Kp);
            const uint16_t* xg = static_cast<const uint16_t*>(Pi.x);
            for (int i = threadIdx.x; i < Pi.M * (ldq / 8); i += kThreads) {
                const int m = i / (ldq / 8), k = 8 * (i % (ldq / 8));
                const u32x4 v = k < Pi.K ? gload<u32x4>(xg + static_cast<int64_t>(m) * Pi.ldx + k) : u32x4{0u, 0u, 0u, 0u};
                *reinterpret_cast<u32x4*>(x_lds + off + m * ldq + k) = interleave_x_pairs(v);
            }
            off += Pi.M * ldq;
        }
        wait_vm<0>();
        __syncthreads();
    }

    // consumer
    const int wg_rows = (t_end - t_begin) * 64;
    float* const out_lds = ws_lds + wg_rows;           // [M][wg_rows] fp32 sums
    int pc = p_first, tc = t_begin, sc = 0, slot_c = 0;
    GemvProblem P = ps.get(pc);
    int steps_c = stream_steps(P.Kp);
    int xoff = 0;
    const bool m_ok = col < P.M;                        // M is shared by the group
    const uint16_t* xbase = x_lds + (m_ok ? col : 0) * padded_q_row(P.Kp) + 64 * grp;
    f32x4 acc = {0.0f, 0.0f, 0.0f, 0.0f};
    u32x4 a2[2][8];                                     // zero where the lane has no token
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) a2[i][e] = u32x4{0u, 0u, 0u, 0u};
    const TwiceMultipliers mul;
    const uint64_t rows_mask = __builtin_amdgcn_ballot_w64(m_ok);
    while (true) {
        produce();
        produce();
        wait_vm<kDepth - 2>();                          // both steps' ring loads have landed
        u32x4 w[2];
        lds_read_ring2_x16(ring + slot_c * kThreads * 16 + 16 * lane, xbase + 256 * sc, rows_mask, w[0], w[1], a2);
        slot_c = slot_c + 2 == kDepth ? 0 : slot_c + 2;
        // MFMA t of the pass takes field pair t % 2 of word (t / 2) % 4 of step t / 8; its
        // B operand is built while MFMA t - 1 runs
        const uint32_t words[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
        u32x4 bn = expand_twice_interleaved(words[0], 0, mul);
#pragma unroll
        for (int t = 0; t < 16; ++t) {
            const u32x4 b = bn;
            if (t + 1 < 16) bn = expand_twice_interleaved(words[(t + 1) / 2], (t + 1) % 2, mul);
            if constexpr (kF16)
                acc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a2[t / 8][t % 8]),
                                                             __builtin_bit_cast(f16x8, b), acc, 0, 0, 0);
            else
                acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a2[t / 8][t % 8]),
                                                              __builtin_bit_cast(bf16x8, b), acc, 0, 0, 0);
        }
        sc += 2;
        if (sc >= steps_c) {
            // tile epilogue: lane holds C[m = 4*grp + r][row] of this wave's 16 rows
            sc = 0;
            const f32x4 sum = acc * 0.5f;               // the operand held 2t (exact)
            const int row = (tc - t_begin) * 64 + wave * 16 + col;
            const int32_t bits[4] = {__float_as_int(sum[0]), __float_as_int(sum[1]), __float_as_int(sum[2]),
                                     __float_as_int(sum[3])};
#pragma unroll
            for (int r = 0; r < 4; ++r) {
                const int m = 4 * grp + r;
                if (m < P.M) lds_write_i32(out_lds + m * wg_rows + row, bits[r]);
            }
            acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            if (++tc == t_end) break;
            if (tc == P.tile0 + P.ntiles) {
                xoff += P.M * padded_q_row(P.Kp);
                P = ps.get(++pc);
                steps_c = stream_steps(P.Kp);
                xbase = x_lds + xoff + (m_ok ? col : 0) * padded_q_row(P.Kp) + 64 * grp;
            }
        }
    }
    wait_vm<0>();                                       // ring loads past the end land before the LDS is reused
    __syncthreads();

    for (int pi = p_first; pi <= p_last; ++pi) {
        const GemvProblem Pi = ps.get(pi);
        const int t0 = max(t_begin, Pi.tile0), t1 = min(t_end, Pi.tile0 + Pi.ntiles);
        const int n0 = (t0 - Pi.tile0) * 64, lrow0 = (t0 - t_begin) * 64;
        const int rows = min((t1 - t0) * 64, Pi.N - n0);         // rows past N have no output
        for (int m = 0; m < Pi.M; ++m) {
            const float* const sums = out_lds + m * wg_rows + lrow0;
#pragma unroll 4
            for (int rr = threadIdx.x; rr < rows; rr += kThreads) {
                const float v = sums[rr] * ws_lds[lrow0 + rr];
                if constexpr (kOutBf16)
                    gstore<uint16_t>(static_cast<uint16_t*>(Pi.y) + m * Pi.ldy + n0 + rr, f32_to_bf16(v));
                else
                    gstore<float>(static_cast<float*>(Pi.y) + m * Pi.ldy + n0 + rr, v);
            }
        }
    }
}

// ---------------------------------------------------------------- launchers


int64_t splitk_tiles(int64_t N) { return (N + 15) / 16; }

template <bool kFused>
hipError_t launch_splitk(const GemvProblem& p, size_t lds, bool x_bf16, bool y_bf16, hipStream_t stream) {
    const dim3 grid(static_cast<unsigned>(splitk_tiles(p.N))), block(kThreads);
    if (x_bf16) {
        if (y_bf16) gemv_splitk_kernel<kFused, true, true><<<grid, block, lds, stream>>>(p);
        else gemv_splitk_kernel<kFused, true, false><<<grid, block, lds, stream>>>(p);
    } else {
        if (y_bf16) gemv_splitk_kernel<kFused, false, true><<<grid, block, lds, stream>>>(p);
        else gemv_splitk_kernel<kFused, false, false><<<grid, block, lds, stream>>>(p);
    }
    return hipGetLastError();
}

template <bool kFused, bool kGrouped, bool XB, bool YB>
hipError_t launch_persistent_t(const GemvProblem& single, const GemvProblem* table, int count,
                               int64_t total_tiles, int64_t total_steps, size_t lds, hipStream_t stream) {
    auto kern = gemv_persistent_kernel<kTN, kBatch, kFused, kGrouped, XB, YB>;
    int device = 0, cus = 0, per_cu = 0;
    hipError_t e = hipGetDevice(&device);
    if (e == hipSuccess) e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device);
    if (e == hipSuccess) e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, kThreads, lds);
    if (e != hipSuccess) return e;
    if (BITNET_PERSIST_PER_CU > 0 && per_cu > BITNET_PERSIST_PER_CU) per_cu = BITNET_PERSIST_PER_CU;
    int64_t grid = static_cast<int64_t>(cus) * (per_cu > 0 ? per_cu : 1);
    if (grid > total_tiles) grid = total_tiles;
    kern<<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), lds, stream>>>(single, table, count,
                                                                           static_cast<int>(total_tiles),
                                                                           total_steps);
    return hipGetLastError();
}

template <bool kFused, bool kGrouped>
hipError_t launch_persistent(const GemvProblem& single, const GemvProblem* table, int count, int64_t total_tiles,
                             int64_t total_steps, size_t lds, bool x_bf16, bool y_bf16, hipStream_t stream) {
    if (x_bf16) {
        if (y_bf16) return launch_persistent_t<kFused, kGrouped, true, true>(single, table, count, total_tiles,
                                                                            total_steps, lds, stream);
        return launch_persistent_t<kFused, kGrouped, true, false>(single, table, count, total_tiles, total_steps,
                                                                  lds, stream);
    }
    if (y_bf16) return launch_persistent_t<kFused, kGrouped, false, true>(single, table, count, total_tiles,
                                                                         total_steps, lds, stream);
    return launch_persistent_t<kFused, kGrouped, false, false>(single, table, count, total_tiles, total_steps, lds,
                                                               stream);
}

// CUs of the current device (0 on error).
int device_cus() {
    static int cached[64] = {0};
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cached[dev] == 0) {
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cached[dev] = cus;
    }
    return cached[dev];
}

// Workgroups of the streaming kernel resident at once on the current device.
int stream_grid() { return device_cus() * BITNET_STREAM_PER_CU; }

// Workgroups of a streaming grid that are the first on their CU.
int stream_first(int grid) { return std::min(grid, device_cus()); }

// Host copy of the kernel's first_tile_from_step.
int64_t host_first_tile(const GemvProblem* t, int count, int64_t s, int64_t total_tiles) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (t[mid].step0 <= s) lo = mid;
        else hi = mid - 1;
    }
    const int64_t k = (2 * (s - t[lo].step0) + t[lo].steps) / (2 * t[lo].steps);
    if (k >= t[lo].ntiles) return lo + 1 < count ? t[lo + 1].tile0 : total_tiles;
    return t[lo].tile0 + k;
}

int host_find_problem(const GemvProblem* t, int count, int64_t tile) {
    int lo = 0, hi = count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (t[mid].tile0 <= tile) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// A grouped launch's share bounds sit right after its problem table.
const int32_t* stream_bounds_of(const GemvProblem* table, int count) {
    return reinterpret_cast<const int32_t*>(table + count);
}

// Extra cost of each problem a workgroup touches beyond its first, in k steps
// of a CU's second workgroup per token row: the problem's token rows are
// quantised (or staged) into LDS before the loop and its outputs written
// after it, measured on MI355X (c2-sized groups) at ~2.4 us per problem and
// token while such a workgroup streams ~2.7 steps per us.
#ifndef BITNET_STREAM_PROBLEM_COST
#define BITNET_STREAM_PROBLEM_COST 6
#endif
// The same for a problem the batched quantiser does not take (an input norm,
// M > 4): its tokens are quantised one at a time (c2 with input norms ends
// soonest at 12 of 6, 12, 20, 30 measured on MI355X).
#ifndef BITNET_STREAM_PROBLEM_COST_SLOW
#define BITNET_STREAM_PROBLEM_COST_SLOW 12
#endif
double problem_cost(const GemvProblem& P) {
    return static_cast<double>(quantise_batch_fits(P) ? BITNET_STREAM_PROBLEM_COST : BITNET_STREAM_PROBLEM_COST_SLOW) *
           P.M;
}
// Start cost of a CU's second workgroup, in the same k steps: its prologue
// ends ~1.9 us after that of the CU's first workgroup (measured as above).
#ifndef BITNET_STREAM_SECOND_START
#define BITNET_STREAM_SECOND_START 5
#endif

// Relative speed of a CU's two workgroups, by kernel: the first workgroup on
// a CU (older waves) wins the arbitration for memory and for the SIMDs.  The
// int8 kernel is bound by memory (first ~1.22x the second; the c2 group ends
// soonest with shares weighted 1.26-1.30, start cost 5-8); the W1.58A16
// kernel by its VALU code expansion, where the older waves' issue priority
// gives the first 1.5x to 1.8x the second's rate while both run (the c2
// group ends soonest at 1.70 to 1.85; both measured on MI355X).
// first_weight in percent of the second's rate; second_start in k steps of
// the second workgroup.
struct StreamSlotCosts {
    int first_weight;
    int second_start;
};
constexpr StreamSlotCosts kSlotCostsA8{BITNET_STREAM_FIRST_WEIGHT, BITNET_STREAM_SECOND_START};
constexpr StreamSlotCosts kSlotCostsA16{175, 0};
constexpr StreamSlotCosts kSlotCostsBlocked{BITNET_STREAM_FIRST_WEIGHT, BITNET_STREAM_SECOND_START};

// Greedy share of one workgroup: the tiles from `i` on whose cost (the slot's
// start cost, k steps over the slot's relative rate, plus the cost of every
// further problem) stays within `cap` and whose token rows, w_scale and exact sums
// fit the LDS array.  Returns the end tile.
int64_t fill_share(const GemvProblem* t, int count, int64_t i, int64_t total_tiles, double cap, double rate,
                   double start, int token_bytes, int64_t step_bytes, int64_t q_limit, bool blocked) {
    if (i >= total_tiles) return i;
    int p = host_find_problem(t, count, i);
    double cost = start;
    int64_t bytes = 0;
    for (int np = 0; i < total_tiles && np < kStreamMaxProblems && p < count; ++np, ++p) {
        const GemvProblem& P = t[p];
        const double enter = np > 0 ? problem_cost(P) : 0.0;
        const int64_t enter_bytes =
            static_cast<int64_t>(P.M) * padded_q_row(P.Kp) * token_bytes + step_bytes * stream_steps(P.Kp);
        const double tile_cost = P.steps / rate;
        const int64_t tile_bytes =
            64 * static_cast<int64_t>(sizeof(float)) * ((token_bytes == 1 && !stream_ws_staged(P.M, blocked) ? 0 : 1) + P.M);
        const int64_t left = P.tile0 + P.ntiles - i;
        const double room = cap - cost - enter;
        const int64_t lds_room = q_limit - bytes - enter_bytes;
        if (room < tile_cost || lds_room < tile_bytes) break;
        const int64_t k = std::min<int64_t>(left, std::min<int64_t>(static_cast<int64_t>(room / tile_cost),
                                                                     lds_room / tile_bytes));
        cost += enter + static_cast<double>(k) * tile_cost;
        bytes += enter_bytes + k * tile_bytes;
        i += k;
        if (k < left) break;
    }
    return i;
}

// Share bounds of a grouped streaming launch (bounds[b] .. bounds[b + 1] are
// workgroup b's tiles, whole tiles in table order) that minimise the largest
// workgroup cost: a binary search on that cost, each candidate filled
// greedily.  The first n_first workgroups (the first on their CU) stream
// slots.first_weight percent as fast as the rest, which start
// slots.second_start steps later.  False if no cost covers every tile within
// the LDS limits.
bool stream_bounds(const GemvProblem* t, int count, int64_t total_tiles, int grid, int n_first, int token_bytes,
                   int64_t step_bytes, int64_t q_limit, const StreamSlotCosts& slots, bool blocked,
                   std::vector<int32_t>& bounds) {
    auto cover = [&](double cap, bool keep) {
        int64_t i = 0;
        for (int b = 0; b < grid; ++b) {
            if (keep) bounds[b] = static_cast<int32_t>(i);
            const double rate = b < n_first ? slots.first_weight / 100.0 : 1.0;
            const double start = b < n_first ? 0.0 : static_cast<double>(slots.second_start);
            i = fill_share(t, count, i, total_tiles, cap, rate, start, token_bytes, step_bytes, q_limit, blocked);
        }
        if (keep) bounds[grid] = static_cast<int32_t>(i);
        return i >= total_tiles;
    };
    double all = 0.0;
    for (int p = 0; p < count; ++p)
        all += static_cast<double>(t[p].ntiles) * t[p].steps + problem_cost(t[p]);
    double lo = 0.0, hi = all + 1.0;
    if (!cover(hi, false)) return false;
    for (int it = 0; it < 64 && hi - lo > 1e-3; ++it) {
        const double mid = 0.5 * (lo + hi);
        if (cover(mid, false)) hi = mid;
        else lo = mid;
    }
    bounds.assign(static_cast<size_t>(grid) + 1, 0);
    return cover(hi, true);
}

template <bool kFused, bool kGrouped, bool XB, bool YB, bool kBlocked = false>
hipError_t launch_stream_t(const GemvProblem& single, const GemvProblem* table, int count, int64_t total_tiles,
                           int64_t total_steps, int grid, size_t lds, hipStream_t stream) {
    auto kern = gemv_stream_kernel<kFused, kGrouped, XB, YB, kBlocked>;
    const int32_t* bounds = kGrouped ? stream_bounds_of(table, count) : nullptr;
    kern<<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), lds, stream>>>(
        single, table, bounds, count, static_cast<int>(total_tiles), total_steps, stream_first(grid));
    return hipGetLastError();
}

template <bool kFused, bool kGrouped>
hipError_t launch_stream(const GemvProblem& single, const GemvProblem* table, int count, int64_t total_tiles,
                         int64_t total_steps, int grid, size_t lds, bool x_bf16, bool y_bf16, hipStream_t stream) {
    if (x_bf16) {
        if (y_bf16) return launch_stream_t<kFused, kGrouped, true, true>(single, table, count, total_tiles,
                                                                        total_steps, grid, lds, stream);
        return launch_stream_t<kFused, kGrouped, true, false>(single, table, count, total_tiles, total_steps, grid,
                                                              lds, stream);
    }
    if (y_bf16) return launch_stream_t<kFused, kGrouped, false, true>(single, table, count, total_tiles,
                                                                     total_steps, grid, lds, stream);
    return launch_stream_t<kFused, kGrouped, false, false>(single, table, count, total_tiles, total_steps, grid,
                                                           lds, stream);
}

template <bool kOutBf16, bool kF16>
hipError_t launch_stream_a16_t(const GemvProblem* table, int count, int64_t total_tiles, int64_t total_steps,
                               int grid, hipStream_t stream) {
    GemvProblem none{};
    gemv_stream_a16_kernel<true, kOutBf16, kF16><<<dim3(static_cast<unsigned>(grid)), dim3(kThreads), 0, stream>>>(
        none, table, stream_bounds_of(table, count), count, static_cast<int>(total_tiles), total_steps,
        stream_first(grid));
    return hipGetLastError();
}

// A single problem laid out as a one-entry group.
GemvProblem as_group_of_one(GemvProblem p, int64_t& tiles, int64_t& steps) {
    p.tile0 = 0;
    p.ntiles = static_cast<int>(gemv_group_tiles(p.N));
    p.steps = static_cast<int>(gemv_group_steps(p.Kp));
    p.step0 = 0;
    tiles = p.ntiles;
    steps = static_cast<int64_t>(p.ntiles) * p.steps;
    return p;
}

}  // namespace

size_t gemv_group_lds(int64_t M, int64_t max_Kp) { return static_cast<size_t>(M) * padded_q_row((int)max_Kp); }

int64_t gemv_group_tiles(int64_t N) { return (N + 64 * kTN - 1) / (64 * kTN); }
int64_t gemv_group_steps(int64_t Kp) {          // batches of kBatch k steps per tile
    const int64_t steps = (Kp / 64 + 3) / 4;
    return (steps + kBatch - 1) / kBatch;
}

bool gemv_stream_plan(const GemvProblem* host_table, int count, int64_t total_tiles, int64_t total_steps,
                      int* grid_out, size_t* lds_out, int token_bytes, std::vector<int32_t>* bounds, bool blocked) {
    const int64_t q_limit = blocked ? kStreamQBytesBlocked : kStreamQBytes;
    const int grid = static_cast<int>(std::min<int64_t>(std::min(stream_grid(), kMaxStreamGrid), total_tiles));
    if (grid <= 0 || count <= 0) return false;
    // buffer offsets are 32-bit: every problem's padded rows must stay below 2 GiB
    for (int i = 0; i < count; ++i)
        if (static_cast<int64_t>(host_table[i].ntiles) * 64 * (host_table[i].Kp / 4) >= (int64_t(1) << 31))
            return false;
    const int n_first = stream_first(grid);
    // grouped: balanced shares (built to fit; the loop below checks them)
    const StreamSlotCosts& slots = token_bytes == 2 ? kSlotCostsA16 : blocked ? kSlotCostsBlocked : kSlotCostsA8;
    // LDS per k step of each problem beyond its token rows: the block sums
    const int64_t step_bytes = blocked ? 16 * static_cast<int64_t>(sizeof(int32_t)) : 0;
    if (bounds && !stream_bounds(host_table, count, total_tiles, grid, n_first, token_bytes, step_bytes, q_limit,
                                 slots, blocked, *bounds))
        return false;
    // the shares must tile [0, total_tiles) in order, and the token rows of
    // each workgroup's problems must fit the static array
    size_t need = 0;
    int64_t covered = 0;
    std::vector<int32_t> spans(bounds ? 4 * static_cast<size_t>(grid) : 0, 0);
    for (int b = 0; b < grid; ++b) {
        int64_t t0, t1;
        if (bounds) {
            t0 = (*bounds)[b];
            t1 = (*bounds)[b + 1];
        } else {
            t0 = host_first_tile(host_table, count, share_start(total_steps, b, grid, n_first), total_tiles);
            t1 = host_first_tile(host_table, count, share_start(total_steps, b + 1, grid, n_first), total_tiles);
        }
        if (t0 != covered || t1 < t0 || t1 > total_tiles) return false;
        covered = t1;
        if (t0 >= t1) continue;
        const int p0 = host_find_problem(host_table, count, t0), p1 = host_find_problem(host_table, count, t1 - 1);
        if (p1 - p0 + 1 > kStreamMaxProblems) return false;
        if (bounds) {
            bool fits = true;
            for (int i = p0; i <= p1; ++i) fits = fits && quantise_batch_fits(host_table[i]);
            spans[4 * static_cast<size_t>(b)] = p0;
            spans[4 * static_cast<size_t>(b) + 1] = p1;
            spans[4 * static_cast<size_t>(b) + 2] = fits ? 1 : 0;
        }
        // w_scale (when staged) and the M exact sums of each row
        const int M0 = host_table[p0].M;
        size_t bytes = static_cast<size_t>(t1 - t0) * 64 * sizeof(float) *
                       ((token_bytes == 1 && !stream_ws_staged(M0, blocked) ? 0 : 1) + M0);
        for (int i = p0; i <= p1; ++i)
            bytes += static_cast<size_t>(host_table[i].M) * padded_q_row(host_table[i].Kp) * token_bytes +
                     static_cast<size_t>(step_bytes) * stream_steps(host_table[i].Kp);
        need = std::max(need, bytes);
    }
    if (need > static_cast<size_t>(q_limit) || covered != total_tiles) return false;
    // the kernel's records: the grid + 1 share bounds, then {p_first, p_last,
    // batch, 0} per workgroup (a workgroup with no tiles keeps zeros)
    if (bounds) bounds->insert(bounds->end(), spans.begin(), spans.end());
    *grid_out = grid;
    *lds_out = 0;                                       // all of the kernel's LDS is static
    return true;
}

hipError_t launch_gemv(const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                       int64_t M, int64_t Kp, const uint8_t* packed, const float* w_scale,
                       int64_t N, void* y, bool y_bf16, int64_t ldy, int32_t* acc_debug,
                       hipStream_t stream) {
    GemvProblem p{};
    p.q = q; p.a_scale = a_scale; p.q_rowsum = q_rowsum;
    p.packed = packed; p.w_scale = w_scale; p.y = y; p.ldy = ldy; p.acc_debug = acc_debug;
    p.M = (int)M; p.N = (int)N; p.Kp = (int)Kp; p.K = (int)Kp;
    if (N * (Kp / 4) >= kPersistMinBytes) {
        int64_t tiles = 0, steps = 0;
        const GemvProblem g = as_group_of_one(p, tiles, steps);
        int grid = 0;
        size_t lds = 0;
        if (gemv_stream_plan(&g, 1, tiles, steps, &grid, &lds))
            return launch_stream<false, false>(g, nullptr, 1, tiles, steps, grid, lds, true, y_bf16, stream);
        return launch_persistent<false, false>(g, nullptr, 1, tiles, steps, gemv_group_lds(M, Kp), true, y_bf16,
                                               stream);
    }
    return launch_splitk<false>(p, 0, true, y_bf16, stream);
}

hipError_t launch_gemv_fused(const GemvProblem& p, bool x_bf16, bool y_bf16, hipStream_t stream) {
    if (static_cast<int64_t>(p.N) * (p.Kp / 4) >= kPersistMinBytes) {
        int64_t tiles = 0, steps = 0;
        const GemvProblem g = as_group_of_one(p, tiles, steps);
        int grid = 0;
        size_t lds = 0;
        if (gemv_stream_plan(&g, 1, tiles, steps, &grid, &lds))
            return launch_stream<true, false>(g, nullptr, 1, tiles, steps, grid, lds, x_bf16, y_bf16, stream);
        return launch_persistent<true, false>(g, nullptr, 1, tiles, steps, gemv_group_lds(p.M, p.Kp), x_bf16,
                                              y_bf16, stream);
    }
    return launch_splitk<true>(p, static_cast<size_t>(p.M) * p.Kp, x_bf16, y_bf16, stream);
}

hipError_t launch_gemv_blocked(const GemvProblem& p, bool y_bf16, hipStream_t stream) {
    int64_t tiles = 0, steps = 0;
    const GemvProblem g = as_group_of_one(p, tiles, steps);
    int grid = 0;
    size_t lds = 0;
    if (!gemv_stream_plan(&g, 1, tiles, steps, &grid, &lds, 1, nullptr, true)) return hipErrorInvalidValue;
    return y_bf16 ? launch_stream_t<false, false, true, true, true>(g, nullptr, 1, tiles, steps, grid, lds, stream)
                  : launch_stream_t<false, false, true, false, true>(g, nullptr, 1, tiles, steps, grid, lds, stream);
}

hipError_t launch_gemv_blocked_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles,
                                       int64_t total_steps, int grid, bool x_bf16, bool y_bf16, hipStream_t stream) {
    GemvProblem none{};
    if (x_bf16)
        return y_bf16 ? launch_stream_t<true, true, true, true, true>(none, table_dev, count, total_tiles, total_steps,
                                                                      grid, 0, stream)
                      : launch_stream_t<true, true, true, false, true>(none, table_dev, count, total_tiles,
                                                                       total_steps, grid, 0, stream);
    return y_bf16 ? launch_stream_t<true, true, false, true, true>(none, table_dev, count, total_tiles, total_steps,
                                                                   grid, 0, stream)
                  : launch_stream_t<true, true, false, false, true>(none, table_dev, count, total_tiles, total_steps,
                                                                    grid, 0, stream);
}

hipError_t launch_gemv_a16_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles,
                                   int64_t total_steps, int grid, bool y_bf16, hipStream_t stream, bool x_f16) {
    if (x_f16)
        return y_bf16 ? launch_stream_a16_t<true, true>(table_dev, count, total_tiles, total_steps, grid, stream)
                      : launch_stream_a16_t<false, true>(table_dev, count, total_tiles, total_steps, grid, stream);
    return y_bf16 ? launch_stream_a16_t<true, false>(table_dev, count, total_tiles, total_steps, grid, stream)
                  : launch_stream_a16_t<false, false>(table_dev, count, total_tiles, total_steps, grid, stream);
}

hipError_t launch_gemv_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles,
                               int64_t total_steps, size_t lds, int stream_grid_size, bool x_bf16, bool y_bf16,
                               hipStream_t stream) {
    GemvProblem none{};
    if (stream_grid_size > 0)
        return launch_stream<true, true>(none, table_dev, count, total_tiles, total_steps, stream_grid_size, lds,
                                         x_bf16, y_bf16, stream);
    return launch_persistent<true, true>(none, table_dev, count, total_tiles, total_steps, lds, x_bf16, y_bf16,
                                         stream);
}

}  // namespace bitnet
