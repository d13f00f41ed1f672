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
// Two kernels:
//  * split-K (small single calls): a workgroup owns 16 output rows and its 4
//    waves split K; partial 16x16 tiles meet in LDS.  Most workgroups for a
//    small matrix, which is what a latency-bound launch needs.
//  * persistent (grouped launches and large single calls): about one
//    workgroup per resident slot; workgroup w owns the 64-row tiles whose
//    first k step falls in its equal share of all k steps, so every workgroup
//    streams about the same number of bytes.  A ring of D prefetched 1 KB
//    steps per wave runs across tile and problem boundaries: the producer walks
//    the workgroup's (tile, step) sequence D steps ahead of the consumer, so
//    loads stay in flight through epilogues and through the ActQuant prologue,
//    which runs only when the consumer enters a new problem.
//
// Every global access goes through gload / gstore (global address space), so
// the ring's loads are counted by vmcnt alone and are waited for one at a time.
#include "device_common.h"
#include "gemv.h"
#include "kernels.h"

namespace bitnet {
namespace {

constexpr int kThreads = 256;
constexpr int kWaves = kThreads / kWave;

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

template <bool kXBf16, int kCache, bool kPerm>
__device__ void quantise_tokens(const GemvProblem& p, int8_t* q_lds, float* as_lds, int* rs_lds,
                                float* red_f, int* red_i, bool store) {
    const int ldq = kPerm ? padded_q_row(p.Kp) : p.Kp;
    const int tid = threadIdx.x;
    const int nvec = p.K / 8;
    const size_t esize = kXBf16 ? 2 : 4;
    for (int m = 0; m < p.M; ++m) {
        const void* xrow = static_cast<const char*>(p.x) + static_cast<int64_t>(m) * p.ldx * esize;
        float cache[kCache][8];
        float amax = 0.0f;
#pragma unroll
        for (int i = 0; i < kCache; ++i) {
            const int vi = tid + i * kThreads;
            if (vi < nvec) {
                load_x8<kXBf16>(xrow, vi, cache[i]);
#pragma unroll
                for (int e = 0; e < 8; ++e) amax = fmaxf(amax, fabsf(cache[i][e]));
            }
        }
        for (int vi = tid + kCache * kThreads; vi < nvec; vi += kThreads) {
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
        int8_t* qrow = q_lds + m * ldq;
        int8_t* qout = store ? p.q_out + static_cast<int64_t>(m) * p.Kp : nullptr;
        auto quant8 = [&](const float (&v)[8]) {
            uint32_t lo = 0, hi = 0;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
                const int c = static_cast<int>(fminf(fmaxf(rne(v[e] * sa), -128.0f), 127.0f));
                sum += c;
                const uint32_t byte = static_cast<uint32_t>(c) & 0xFFu;
                if (e < 4) lo |= byte << (8 * e);
                else hi |= byte << (8 * (e - 4));
            }
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
                    load_x8<kXBf16>(xrow, vi, v);
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
            const float as = (amax == 0.0f) ? 0.0f : amax / 127.0f;
            as_lds[m] = as;
            rs_lds[m] = total;
            if (store) {
                gstore<float>(p.a_scale_out + m, as);
                gstore<int32_t>(p.rowsum_out + m, total);
            }
        }
        __syncthreads();   // red_f / red_i are reused by the next token
    }
}

// Unfused persistent path: copy the problem's quantised rows q [M][Kp] from
// global memory into the permuted, zero-padded LDS layout, with a_scale and
// q_rowsum into as_lds / rs_lds.
__device__ void stage_tokens(const GemvProblem& p, int8_t* q_lds, float* as_lds, int* rs_lds) {
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
        rs_lds[threadIdx.x] = gload<int32_t>(p.q_rowsum + threadIdx.x);
    }
    __syncthreads();
}

// y (and optionally acc) of one output: token m, row n of problem p.
template <bool kOutBf16>
__device__ __forceinline__ void store_output(const GemvProblem& p, int m, int n, int32_t exact, float as, float ws) {
    const float v = static_cast<float>(exact) * (as * ws);
    if constexpr (kOutBf16)
        gstore<uint16_t>(static_cast<uint16_t*>(p.y) + m * p.ldy + n, f32_to_bf16(v));
    else
        gstore<float>(static_cast<float*>(p.y) + m * p.ldy + n, v);
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
    if constexpr (kFused)
        quantise_tokens<kXBf16, 4, false>(p, q_lds, as_lds, rs_lds, red_f, red_i,
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

    const int m = threadIdx.x / 16;
    const int nc = threadIdx.x % 16;
    const int n = n0 + nc;
    if (m < p.M && n < p.N) {
        int s = 0;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) s += part[w][m][nc];
        int32_t rs;
        float as;
        if constexpr (kFused) {
            rs = rs_lds[m];
            as = as_lds[m];
        } else {
            rs = gload<int32_t>(p.q_rowsum + m);
            as = gload<float>(p.a_scale + m);
        }
        store_output<kOutBf16>(p, m, n, s - rs, as, gload<float>(p.w_scale + n));
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

// First tile whose first k step is at or after `s` (total_tiles if none).
template <bool kGrouped>
__device__ __forceinline__ int first_tile_from_step(const Problems<kGrouped>& ps, int64_t s, int total_tiles) {
    int lo = 0, hi = ps.count - 1;              // last problem with step0 <= s
    while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (ps.get(mid).step0 <= s) lo = mid;
        else hi = mid - 1;
    }
    const GemvProblem p = ps.get(lo);
    const int64_t t = (s - p.step0 + p.steps - 1) / p.steps;   // tiles of p that start before s
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
        if constexpr (kFused)
            quantise_tokens<kXBf16, 2, true>(P, q_lds, as_lds, rs_lds, red_f, red_i,
                                             P.q_out != nullptr && seg_begin == P.tile0);
        else
            stage_tokens(P, q_lds, as_lds, rs_lds);
        const int8_t* abase = q_lds + (m_ok ? col : 0) * padded_q_row(P.Kp) + 64 * grp;
        const int chunks = P.Kp / 64;
        const int row_bytes = P.Kp / 4;

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

        u32x4 bufA[U][TN], bufB[U][TN];
        load_batch(bufA);
        load_batch(bufB);
        prefetch_epilogue();
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
        return launch_persistent<false, false>(g, nullptr, 1, tiles, steps, gemv_group_lds(M, Kp), true, y_bf16,
                                               stream);
    }
    return launch_splitk<false>(p, 0, true, y_bf16, stream);
}

hipError_t launch_gemv_fused(const GemvProblem& p, bool x_bf16, bool y_bf16, hipStream_t stream) {
    if (static_cast<int64_t>(p.N) * (p.Kp / 4) >= kPersistMinBytes) {
        int64_t tiles = 0, steps = 0;
        const GemvProblem g = as_group_of_one(p, tiles, steps);
        return launch_persistent<true, false>(g, nullptr, 1, tiles, steps, gemv_group_lds(p.M, p.Kp), x_bf16,
                                              y_bf16, stream);
    }
    return launch_splitk<true>(p, static_cast<size_t>(p.M) * p.Kp, x_bf16, y_bf16, stream);
}

hipError_t launch_gemv_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles,
                               int64_t total_steps, size_t lds, bool x_bf16, bool y_bf16,
                               hipStream_t stream) {
    GemvProblem none{};
    return launch_persistent<true, true>(none, table_dev, count, total_tiles, total_steps, lds, x_bf16, y_bf16,
                                         stream);
}

}  // namespace bitnet
