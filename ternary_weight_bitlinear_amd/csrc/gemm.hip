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
//    Lane l supplies row l%32 of the first operand, column l%32 of the second
//    and 16 k values of group l/32; register r of the result holds
//    D[8(r/4) + 4(l/32) + r%4][l%32].  The codes are the first operand and
//    the activations the second, so D is the transposed output tile and each
//    lane ends with four consecutive outputs of one row: the epilogue writes
//    them as one 8-byte (bf16) or 16-byte (fp32) store.
//  * Workgroup tile BM x BN, k stage BK = 128, double-buffered in LDS; waves
//    in a WGM x WGN grid, each owning (BM/WGM) x (BN/WGN) as 32x32 tiles held
//    in accumulation registers.
//  * Two kernels share tiles, operand roles and epilogue.  gemm_dma_kernel
//    (the default for the 128x128 and 128x256 tiles; its own comment block
//    below) fetches stages straight into an LDS ring.  gemm_kernel (the 64x64
//    tile, and the others under BITNET_GEMM_KERNEL=regs) runs global loads PF
//    stages ahead of the MFMAs through PF register sets, so a load has PF
//    stages of matrix work to land in; a stage is written to the free LDS
//    buffer one stage before it is used.  In both the loads are buffer loads:
//    rows past M or N and stages past the end lie outside the buffer's range
//    and read as zero, so every load is issued unconditionally and the
//    compiler can keep exact wait counts.
//  * Codes stay packed in LDS (a quarter of an int8 tile).  In one stage lane
//    group g takes the contiguous k range [64g, 64g + 64) of the stage, so its
//    B operand for the whole stage is one 16-byte LDS read (four packed words,
//    one per 32-k step); each word is expanded in registers with
//    (word >> 2p) & 0x03030303 (7 VALU ops per 16 codes).  A uses the same k
//    mapping, so the exact integer sum does not depend on the MFMA's internal
//    k order.
//  * Stored codes are u = t + 1 in {0,1,2}; the epilogue subtracts q_rowsum[m]
//    (the padded tail has q = 0) to get the exact sum of q*t.
//  * gemm_kernel pads LDS rows (A: 144 B, B: 48 B) so that the 16-byte reads
//    of 16 consecutive rows fall in distinct bank groups; gemm_dma_kernel
//    swizzles 16-byte chunks instead.
//  * Tile order: workgroup b runs on XCD b % 8, so ids are remapped to give
//    each XCD a contiguous range of the tile sequence, and the sequence walks
//    bands of GM tile rows column by column, so the workgroups that run
//    together on one XCD share both activation rows and code rows in its L2.
//  * Kp is a multiple of 128 = BK, so there is no K tail; ragged M and N are
//    handled by the buffer range and guarded stores.
#include <cstdlib>
#include <cstring>

#include "device_common.h"
#include "kernels.h"

namespace bitnet {
namespace {

// Output stores are non-temporal: the outputs are written once and not read
// again by the GEMM, so marking them streaming keeps them from evicting the
// activation and code tiles that other workgroups read again from L2 and the
// MALL (measured on MI355X: c5 GEMMs 1.3-4% faster, c4 5-20%).
template <typename T>
__device__ __forceinline__ void nt_store(T* p, T v) {
    __builtin_nontemporal_store(v, p);
}

constexpr int BK = 128;          // k elements per stage
constexpr int kApad = 16;        // bytes of padding per LDS activation row
constexpr int kBpad = 16;        // bytes of padding per LDS code row
constexpr int kXcds = 8;
constexpr uint32_t kOutOfRange = 0x80000000u;   // offset past any buffer range used here
constexpr int kRsrcWord3 = 0x00020000;          // raw 32-bit buffer access on gfx9-family parts

__device__ __forceinline__ v16i mfma32(v4i a, v4i b, v16i c) {
    return __builtin_amdgcn_mfma_i32_32x32x32_i8(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ u32x4 bload(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

template <int BM, int BN>
constexpr size_t lds_bytes() {
    return 2 * (static_cast<size_t>(BM) * (BK + kApad) + static_cast<size_t>(BN) * (BK / 4 + kBpad));
}

struct TileOrder {
    int tiles_m, tiles_n, group_m;
};

// Workgroup id -> (tile row, tile column).
__device__ __forceinline__ void tile_of(const TileOrder& o, int& tm, int& tn) {
    const int tiles = o.tiles_m * o.tiles_n;
    const int b = blockIdx.x;
    // ids with b % 8 == x form XCD x's queue; give it tiles [start_x, start_x + count_x)
    const int per = tiles / kXcds, rem = tiles % kXcds, x = b % kXcds;
    const int seq = x * per + min(x, rem) + b / kXcds;
    const int band = o.group_m * o.tiles_n;
    const int first_m = (seq / band) * o.group_m;
    const int rows = min(o.tiles_m - first_m, o.group_m);
    const int in_band = seq % band;
    tm = first_m + in_band % rows;
    tn = in_band / rows;
}

// Epilogue shared by both GEMM kernels: register 4rb + rr of lane l in
// acc[j][i] holds output row m = i*32 + l%32, column n = j*32 + 8rb + 4(l/32)
// + rr of the wave's tile; the stored codes are t + 1, so the exact sum of
// q*t is the register minus q_rowsum[m].
template <int BM, int BN, int WM, int WN, int TM, int TN, bool kOutBf16>
__device__ __forceinline__ void gemm_epilogue(const v16i (&acc)[TN][TM], const float* as_s, const int32_t* rs_s,
                                              const float* ws_s, int m0, int n0, int wm, int wn, int r32, int g,
                                              int M, int N, void* __restrict__ y, int64_t ldy,
                                              int32_t* __restrict__ acc_debug, int vec_store) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int ml = wm * WM + i * 32 + r32;
        const int m = m0 + ml;
        const float as = as_s[ml];
        const int32_t rs = rs_s[ml];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int nl = wn * WN + j * 32 + 8 * rb + 4 * g;
                const int n = n0 + nl;
                const f32x4 ws4 = *reinterpret_cast<const f32x4*>(&ws_s[nl]);
                int32_t e[4];
                f32x4 v;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) {
                    e[rr] = acc[j][i][4 * rb + rr] - rs;
                    v[rr] = static_cast<float>(e[rr]) * (as * ws4[rr]);
                }
                if (m >= M) continue;
                const int64_t off = static_cast<int64_t>(m) * ldy + n;
                if (vec_store && n + 3 < N) {
                    if constexpr (kOutBf16) {
                        bf16x4 h;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) h[rr] = static_cast<__bf16>(v[rr]);   // v_cvt_pk_bf16_f32: RNE
                        nt_store(reinterpret_cast<bf16x4*>(static_cast<__bf16*>(y) + off), h);
                    } else {
                        nt_store(reinterpret_cast<f32x4*>(static_cast<float*>(y) + off), v);
                    }
                } else {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        if (n + rr >= N) break;
                        if constexpr (kOutBf16)
                            nt_store(static_cast<__bf16*>(y) + off + rr, static_cast<__bf16>(v[rr]));
                        else
                            nt_store(static_cast<float*>(y) + off + rr, v[rr]);
                    }
                }
                if (acc_debug) {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr)
                        if (n + rr < N) acc_debug[static_cast<int64_t>(m) * N + n + rr] = e[rr];
                }
            }
        }
    }
}

template <int BM, int BN, int WGM, int WGN, int PF, int kWaves, bool kOutBf16>
__global__ __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(kWaves))) void gemm_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ a_scale,
    const int32_t* __restrict__ q_rowsum, int M, int Kp,
    const uint8_t* __restrict__ packed, const float* __restrict__ w_scale, int N,
    void* __restrict__ y, int64_t ldy, int32_t* __restrict__ acc_debug, TileOrder order, int vec_store) {
    constexpr int kThreads = WGM * WGN * 64;
    constexpr int WM = BM / WGM, WN = BN / WGN;      // per-wave tile
    constexpr int TM = WM / 32, TN = WN / 32;        // 32x32 MFMA tiles per wave
    constexpr int A_ROW = BK + kApad;
    constexpr int B_ROW = BK / 4 + kBpad;
    constexpr int A_LOADS = BM * BK / 16 / kThreads; // 16-byte loads per thread per stage
    constexpr int B_LOADS = BN * (BK / 4) / 16 / kThreads;
    static_assert(A_LOADS >= 1 && B_LOADS >= 1 && TM >= 1 && TN >= 1 && PF >= 1, "tile shape");
    static_assert(BM * BK / 16 % kThreads == 0 && BN * (BK / 4) / 16 % kThreads == 0, "tile shape");

    extern __shared__ __attribute__((aligned(16))) int8_t lds[];
    __shared__ __attribute__((aligned(16))) float as_s[BM];      // a_scale of the tile's rows
    __shared__ __attribute__((aligned(16))) int32_t rs_s[BM];    // q_rowsum of the tile's rows
    __shared__ __attribute__((aligned(16))) float ws_s[BN];      // w_scale of the tile's columns
    int8_t* a_lds = lds;                                           // [2][BM][A_ROW]
    uint8_t* b_lds = reinterpret_cast<uint8_t*>(lds + 2 * BM * A_ROW);   // [2][BN][B_ROW]

    int tm, tn;
    tile_of(order, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = tid / 64;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r32 = lane % 32;     // A row / B column inside a 32x32 tile
    const int g = lane / 32;       // k group: bytes [64g, 64g + 64) of a stage
    const int brow_bytes = Kp / 4;
    const int stages = Kp / BK;

    // Buffer ranges cover exactly the tile's valid rows.
    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(q + static_cast<int64_t>(m0) * Kp), 0, a_rows * Kp, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed + static_cast<int64_t>(n0) * brow_bytes), 0, b_rows * brow_bytes, kRsrcWord3);

    // Per-thread offsets of its pieces inside stage 0.
    uint32_t a_off[A_LOADS], b_off[B_LOADS];
#pragma unroll
    for (int i = 0; i < A_LOADS; ++i) {
        const int f = i * kThreads + tid;
        a_off[i] = static_cast<uint32_t>((f / (BK / 16)) * Kp + 16 * (f % (BK / 16)));
    }
#pragma unroll
    for (int i = 0; i < B_LOADS; ++i) {
        const int f = i * kThreads + tid;
        b_off[i] = static_cast<uint32_t>((f / (BK / 64)) * brow_bytes + 16 * (f % (BK / 64)));
    }

    u32x4 a_reg[PF][A_LOADS];
    u32x4 b_reg[PF][B_LOADS];
    auto load_stage = [&](u32x4 (&ar)[A_LOADS], u32x4 (&br)[B_LOADS], int ks) {
        const bool in = ks < stages;
        const uint32_t ka = in ? static_cast<uint32_t>(ks * BK) : kOutOfRange;
        const uint32_t kb = in ? static_cast<uint32_t>(ks * (BK / 4)) : kOutOfRange;
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) ar[i] = bload(a_rsrc, a_off[i] + ka);
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) br[i] = bload(b_rsrc, b_off[i] + kb);
    };
    auto store_stage = [&](const u32x4 (&ar)[A_LOADS], const u32x4 (&br)[B_LOADS], int st) {
#pragma unroll
        for (int i = 0; i < A_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 16), s = f % (BK / 16);
            *reinterpret_cast<u32x4*>(a_lds + st * BM * A_ROW + r * A_ROW + 16 * s) = ar[i];
        }
#pragma unroll
        for (int i = 0; i < B_LOADS; ++i) {
            const int f = i * kThreads + tid;
            const int r = f / (BK / 64), s = f % (BK / 64);
            *reinterpret_cast<u32x4*>(b_lds + st * BN * B_ROW + r * B_ROW + 16 * s) = br[i];
        }
    };

    v16i acc[TN][TM];              // acc[j][i]: transposed 32x32 output tile (n of j, m of i)
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;

    auto compute_stage = [&](int st) {
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
                for (int j = 0; j < TN; ++j) acc[j][i] = mfma32(b[j], a[i], acc[j][i]);
        }
    };

    for (int i = tid; i < BM; i += kThreads) {
        const int m = m0 + i;
        as_s[i] = m < M ? a_scale[m] : 0.0f;
        rs_s[i] = m < M ? q_rowsum[m] : 0;
    }
    for (int i = tid; i < BN; i += kThreads) ws_s[i] = n0 + i < N ? w_scale[n0 + i] : 0.0f;
#pragma unroll
    for (int u = 0; u < PF; ++u) load_stage(a_reg[u], b_reg[u], u);
    store_stage(a_reg[0], b_reg[0], 0);
    __syncthreads();

    // Stage k's data sits in register set k % PF from stage k - PF on; at the
    // end of stage k the set holding stage k + 1 goes to LDS buffer (k+1) % 2.
    // The main loop covers the groups of PF stages that are all followed by
    // another stage, so its stores and barriers are unconditional; the
    // scheduling barrier keeps the next loads ahead of the stage's MFMAs.
    int k = 0;
    for (; k + PF < stages; k += PF) {
#pragma unroll
        for (int u = 0; u < PF; ++u) {
            const int kk = k + u;
            load_stage(a_reg[u], b_reg[u], kk + PF);
            __builtin_amdgcn_sched_barrier(0);
            compute_stage(kk & 1);
            store_stage(a_reg[(u + 1) % PF], b_reg[(u + 1) % PF], (kk + 1) & 1);
            __syncthreads();
        }
    }
#pragma unroll
    for (int u = 0; u < PF; ++u) {
        const int kk = k + u;
        if (kk < stages) {
            compute_stage(kk & 1);
            if (kk + 1 < stages) {
                store_stage(a_reg[(u + 1) % PF], b_reg[(u + 1) % PF], (kk + 1) & 1);
                __syncthreads();
            }
        }
    }

    gemm_epilogue<BM, BN, WM, WN, TM, TN, kOutBf16>(acc, as_s, rs_s, ws_s, m0, n0, wm, wn, r32, g, M, N, y, ldy,
                                                   acc_debug, vec_store);
}

// ------------------------------------------------------------ LDS-DMA variant
//
// Same tiles, operand roles and epilogue as gemm_kernel, with a different
// memory pipeline:
//  * Global data goes straight to LDS with buffer_load_dwordx4 ... lds (the
//    memory unit writes LDS; no staging registers, no ds_write), into a ring
//    of NS stage buffers.  One such load of a wave fills 1 KB of LDS, lane l at
//    byte 16*l, so the LDS layout is set by choosing which 16 global bytes each
//    lane fetches: rows are unpadded (128 B of activations, 32 B of codes per
//    stage) and the 16-byte chunks of a row are XOR-swizzled so that the
//    16-byte fragment reads of 16 consecutive rows hit distinct bank groups.
//      activations: chunk c of row r at 16 * (c ^ sa(r)), sa(r) = (r&7) ^ ((r>>3)&1)
//      codes:       chunk c of row n at 16 * (c ^ sb(n)), sb(n) = ((n>>2) ^ (n>>3)) & 1
//    Both depend on the row's low 4 bits only, which are the lane's own in
//    every fragment read.
//  * Pipeline per stage k, four 32-k steps: each step issues the next step's
//    activation fragments (step 3: the next stage's code words and first
//    fragments) from asm, then runs its MFMAs interleaved with the next
//    step's code expansion (scheduling groups of one MFMA and up to four VALU
//    ops), then waits for the reads.  Before step 3 the wave waits for its
//    own loads of stage k+1 and one barrier makes every wave's loads visible
//    (and tells that stage k's buffer has been read by all); the loads of
//    stage k+NS then go into that buffer.  One barrier per stage; loads run
//    NS stages ahead.
//  * LDS reads are issued from asm: the compiler would otherwise order every
//    LDS read after all LDS DMA loads in flight.  The issuing asm names the
//    destination registers as outputs and a later waiting asm names them as
//    in-out operands, with scheduling barriers on both sides of the step's
//    MFMAs, so no use of the data precedes the wait and the reads' latency
//    hides behind the MFMAs.  The MFMAs are compiler builtins, so the
//    compiler's hazard handling covers them.
//  * Tail stages past the end are fetched from an offset outside the buffer
//    range, so every stage issues the same loads and the wait counts are
//    compile-time constants; those loads write zeros into buffers nobody
//    reads, and the wave drains them before the epilogue.
typedef __attribute__((address_space(3))) void* lds_ptr_t;

// VALU ops placed after each MFMA of a step (the next step's code expansion).
#ifndef BITNET_GEMM_VALU_GROUP
#define BITNET_GEMM_VALU_GROUP 4
#endif

template <int kVm>
__device__ __forceinline__ void wait_vm() {     // s_waitcnt vmcnt(kVm), other counters untouched
    static_assert(kVm >= 0 && kVm < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((kVm & 15) | ((kVm >> 4) << 14) | (7 << 4) | (15 << 8));
}

// 16 bytes per lane from buffer offset off to LDS at dst + 16 * lane (dst
// wave-uniform).
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, void* dst, uint32_t off) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)dst, 16, off, 0, 0, 0);
}

__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return static_cast<uint32_t>(reinterpret_cast<uintptr_t>((__attribute__((address_space(3))) const char*)(p)));
}

__host__ __device__ constexpr int swz_a(int r) { return (r & 7) ^ ((r >> 3) & 1); }
__host__ __device__ constexpr int swz_b(int n) { return ((n >> 2) ^ (n >> 3)) & 1; }

template <int BM, int BN>
constexpr int dma_stage_bytes() {
    return BM * BK + BN * (BK / 4);
}

// Split LDS reads: the issuing asm names the destination registers as
// outputs, the waiting asm names them again as in-out operands, so the
// compiler keeps them live and places no use of them before the wait.
__device__ __forceinline__ void lds_issue_a(v4i (&na)[2], uint32_t ad) {
    asm volatile("ds_read_b128 %[n0], %[ad]\n\tds_read_b128 %[n1], %[ad] offset:4096"
                 : [n0] "=&v"(na[0]), [n1] "=&v"(na[1])
                 : [ad] "v"(ad)
                 : "memory");
}
__device__ __forceinline__ void lds_wait_a(v4i (&na)[2]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(na[0]), "+v"(na[1]) : : "memory");
}
__device__ __forceinline__ void lds_issue_head(v4i (&na)[2], u32x4 (&nw)[4], uint32_t ad, uint32_t bd) {
    asm volatile(
        "ds_read_b128 %[w0], %[bd]\n\tds_read_b128 %[w1], %[bd] offset:1024\n\t"
        "ds_read_b128 %[w2], %[bd] offset:2048\n\tds_read_b128 %[w3], %[bd] offset:3072\n\t"
        "ds_read_b128 %[n0], %[ad]\n\tds_read_b128 %[n1], %[ad] offset:4096"
        : [n0] "=&v"(na[0]), [n1] "=&v"(na[1]), [w0] "=&v"(nw[0]), [w1] "=&v"(nw[1]), [w2] "=&v"(nw[2]),
          [w3] "=&v"(nw[3])
        : [ad] "v"(ad), [bd] "v"(bd)
        : "memory");
}
__device__ __forceinline__ void lds_wait_head(v4i (&na)[2], u32x4 (&nw)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(na[0]), "+v"(na[1]), "+v"(nw[0]), "+v"(nw[1]), "+v"(nw[2]), "+v"(nw[3])
                 :
                 : "memory");
}
__device__ __forceinline__ void lds_issue_head(v4i (&na)[2], u32x4 (&nw)[2], uint32_t ad, uint32_t bd) {
    asm volatile(
        "ds_read_b128 %[w0], %[bd]\n\tds_read_b128 %[w1], %[bd] offset:1024\n\t"
        "ds_read_b128 %[n0], %[ad]\n\tds_read_b128 %[n1], %[ad] offset:4096"
        : [n0] "=&v"(na[0]), [n1] "=&v"(na[1]), [w0] "=&v"(nw[0]), [w1] "=&v"(nw[1])
        : [ad] "v"(ad), [bd] "v"(bd)
        : "memory");
}
__device__ __forceinline__ void lds_wait_head(v4i (&na)[2], u32x4 (&nw)[2]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(na[0]), "+v"(na[1]), "+v"(nw[0]), "+v"(nw[1]) : : "memory");
}
// Four activation fragments (a wave tile of 128 rows: 32-row fragments 4 KB
// apart in the stage).
__device__ __forceinline__ void lds_issue_a(v4i (&na)[4], uint32_t ad) {
    asm volatile("ds_read_b128 %[n0], %[ad]\n\tds_read_b128 %[n1], %[ad] offset:4096\n\t"
                 "ds_read_b128 %[n2], %[ad] offset:8192\n\tds_read_b128 %[n3], %[ad] offset:12288"
                 : [n0] "=&v"(na[0]), [n1] "=&v"(na[1]), [n2] "=&v"(na[2]), [n3] "=&v"(na[3])
                 : [ad] "v"(ad)
                 : "memory");
}
__device__ __forceinline__ void lds_wait_a(v4i (&na)[4]) {
    asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(na[0]), "+v"(na[1]), "+v"(na[2]), "+v"(na[3]) : : "memory");
}
__device__ __forceinline__ void lds_issue_head(v4i (&na)[4], u32x4 (&nw)[2], uint32_t ad, uint32_t bd) {
    asm volatile(
        "ds_read_b128 %[w0], %[bd]\n\tds_read_b128 %[w1], %[bd] offset:1024\n\t"
        "ds_read_b128 %[n0], %[ad]\n\tds_read_b128 %[n1], %[ad] offset:4096\n\t"
        "ds_read_b128 %[n2], %[ad] offset:8192\n\tds_read_b128 %[n3], %[ad] offset:12288"
        : [n0] "=&v"(na[0]), [n1] "=&v"(na[1]), [n2] "=&v"(na[2]), [n3] "=&v"(na[3]), [w0] "=&v"(nw[0]),
          [w1] "=&v"(nw[1])
        : [ad] "v"(ad), [bd] "v"(bd)
        : "memory");
}
__device__ __forceinline__ void lds_wait_head(v4i (&na)[4], u32x4 (&nw)[2]) {
    asm volatile("s_waitcnt lgkmcnt(0)"
                 : "+v"(na[0]), "+v"(na[1]), "+v"(na[2]), "+v"(na[3]), "+v"(nw[0]), "+v"(nw[1])
                 :
                 : "memory");
}

typedef float f32x16 __attribute__((ext_vector_type(16)));

// Signed MFMA operand of one packed word: byte 4p+b is t = u - 1 of element
// 16j+4p+b, looked up from the stored code u in {0,1,2} with one byte
// permute per 4 codes (table bytes 0xFF, 0x00, 0x01).
__device__ __forceinline__ v4i expand_word_signed(uint32_t w) {
    constexpr uint32_t kSigned = 0x000100FFu;
    v4i r;
#pragma unroll
    for (int p = 0; p < 4; ++p)
        r[p] = static_cast<int>(__builtin_amdgcn_perm(0u, kSigned, (w >> (2 * p)) & 0x03030303u));
    return r;
}

// One 16-byte LDS read with its completion wait in the same asm block (see the
// LDS-read note above: a compiler-visible read would wait for the DMA loads).
__device__ __forceinline__ u32x4 lds_read_b128(const void* p) {
    u32x4 v;
    asm volatile("ds_read_b128 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=&v"(v) : "v"(lds_offset(p)) : "memory");
    return v;
}

// Epilogue of the block-scaled kernel: y = facc * a_scale[m] (fp32), with
// the register-to-output mapping of gemm_epilogue.
template <int BM, int BN, int WM, int WN, int TM, int TN, bool kOutBf16>
__device__ __forceinline__ void gemm_epilogue_blocked(const f32x16 (&facc)[TN][TM], const float* as_s, int m0,
                                                      int n0, int wm, int wn, int r32, int g, int M, int N,
                                                      void* __restrict__ y, int64_t ldy, int vec_store) {
    typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
#pragma unroll
    for (int i = 0; i < TM; ++i) {
        const int ml = wm * WM + i * 32 + r32;
        const int m = m0 + ml;
        if (m >= M) continue;
        const float as = as_s[ml];
#pragma unroll
        for (int j = 0; j < TN; ++j) {
#pragma unroll
            for (int rb = 0; rb < 4; ++rb) {
                const int n = n0 + wn * WN + j * 32 + 8 * rb + 4 * g;
                f32x4 v;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = facc[j][i][4 * rb + rr] * as;
                const int64_t off = static_cast<int64_t>(m) * ldy + n;
                if (vec_store && n + 3 < N) {
                    if constexpr (kOutBf16) {
                        bf16x4 h;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) h[rr] = static_cast<__bf16>(v[rr]);
                        nt_store(reinterpret_cast<bf16x4*>(static_cast<__bf16*>(y) + off), h);
                    } else {
                        nt_store(reinterpret_cast<f32x4*>(static_cast<float*>(y) + off), v);
                    }
                } else {
#pragma unroll
                    for (int rr = 0; rr < 4; ++rr) {
                        if (n + rr >= N) break;
                        if constexpr (kOutBf16)
                            nt_store(static_cast<__bf16*>(y) + off + rr, static_cast<__bf16>(v[rr]));
                        else
                            nt_store(static_cast<float*>(y) + off + rr, v[rr]);
                    }
                }
            }
        }
    }
}

// Bytes of one wave's staging region in gemm_epilogue_lds: the rows of one
// pass (all TM*32 rows for bf16, 32 rows per pass for fp32) at a row pitch of
// WN elements plus 8 bytes, so that the 8- or 16-byte writes of the 32 rows a
// fragment spans spread over the LDS banks.
template <int WN, int TM, bool kOutBf16>
constexpr int epi_pitch() { return WN * (kOutBf16 ? 2 : 4) + 8; }
template <int WN, int TM, bool kOutBf16>
constexpr int epi_wave_bytes() { return (kOutBf16 ? TM * 32 : 32) * epi_pitch<WN, TM, kOutBf16>(); }

// Epilogue through LDS (the stage ring is free by then): each wave writes its
// WM x WN outputs, y = (float)(acc - q_rowsum) * (a_scale * w_scale) rounded
// to the output type, into its own LDS region in the fragment layout, then
// reads them back as 16-byte row segments and stores whole rows, 16 bytes per
// lane.  A store instruction then covers 2-8 full rows instead of 16 bytes of
// 32 rows, a quarter of the cache lines per output byte.  The values and
// their roundings are those of gemm_epilogue.  Needs 16-byte aligned y rows
// (ldy * size % 16 == 0 and y 16-byte aligned).
//
// value(i, j, rb, ml, nl) returns the four fp32 outputs a lane holds in
// registers 4rb..4rb+3 of fragment (j, i): rows ml, columns nl..nl+3 of the
// workgroup tile.
template <int WM, int WN, int TM, int TN, bool kOutBf16, typename Value>
__device__ __forceinline__ void gemm_epilogue_lds(Value value, int8_t* region, int m0, int n0, int wm, int wn,
                                                  int lane, int M, int N, void* __restrict__ y, int64_t ldy) {
    constexpr int ESZ = kOutBf16 ? 2 : 4;
    constexpr int PITCH = epi_pitch<WN, TM, kOutBf16>();
    constexpr int PASS_TM = kOutBf16 ? TM : 1;             // 32-row fragments per pass
    constexpr int LANES_PER_ROW = WN * ESZ / 16;
    constexpr int ROWS_PER_READ = 64 / LANES_PER_ROW;
    static_assert(64 % LANES_PER_ROW == 0 && (PASS_TM * 32) % ROWS_PER_READ == 0, "epilogue shape");
    const int r32 = lane % 32, g = lane / 32;
#pragma unroll
    for (int pass = 0; pass < TM / PASS_TM; ++pass) {
#pragma unroll
        for (int ii = 0; ii < PASS_TM; ++ii) {
            const int i = pass * PASS_TM + ii;
            const int ml = wm * WM + i * 32 + r32;
            int8_t* row = region + (ii * 32 + r32) * PITCH;
#pragma unroll
            for (int j = 0; j < TN; ++j) {
#pragma unroll
                for (int rb = 0; rb < 4; ++rb) {
                    const int nl = j * 32 + 8 * rb + 4 * g;          // column inside the wave tile
                    const f32x4 v = value(i, j, rb, ml, wn * WN + nl);
                    if constexpr (kOutBf16) {
                        typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
                        bf16x4 h;
#pragma unroll
                        for (int rr = 0; rr < 4; ++rr) h[rr] = static_cast<__bf16>(v[rr]);   // RNE
                        *reinterpret_cast<bf16x4*>(row + nl * ESZ) = h;
                    } else {
                        *reinterpret_cast<f32x4*>(row + nl * ESZ) = v;
                    }
                }
            }
        }
        // the wave's own LDS writes are visible to its own reads after they complete
#pragma unroll
        for (int r0 = 0; r0 < PASS_TM * 32; r0 += ROWS_PER_READ) {
            const int rl = r0 + lane / LANES_PER_ROW;                 // row inside the pass
            const int cb = (lane % LANES_PER_ROW) * 16;               // byte inside the row
            const u32x4 v = *reinterpret_cast<const u32x4*>(region + rl * PITCH + cb);
            const int m = m0 + wm * WM + pass * PASS_TM * 32 + rl;
            const int n = n0 + wn * WN + cb / ESZ;
            if (m >= M) continue;
            char* dst = static_cast<char*>(y) + (static_cast<int64_t>(m) * ldy + n) * ESZ;
            if (n + 16 / ESZ <= N) {
                nt_store(reinterpret_cast<u32x4*>(dst), v);
            } else {
#pragma unroll
                for (int e = 0; e < 16 / ESZ; ++e) {
                    if (n + e >= N) break;
                    if constexpr (kOutBf16)
                        nt_store(reinterpret_cast<uint16_t*>(dst) + e, static_cast<uint16_t>(v[e / 2] >> (16 * (e % 2))));
                    else
                        nt_store(reinterpret_cast<uint32_t*>(dst) + e, static_cast<uint32_t>(v[e]));
                }
            }
        }
    }
}

// kBlocked: weights with one scale per 256-k block of a row ("BitVLA --
// 1.58-bit Vision-Language-Action on Core AI", s2: the sibling matvec
// kernel's per-256-block scales, against BitNet's one per tensor).  The codes are
// expanded to signed t (one byte permute per 4 codes), every 256 k (two
// stages, or the last stage) the exact int32 block sums are scaled by the
// block's scale and added to fp32 accumulators in block order, and the
// epilogue multiplies by a_scale; block_scale [nb][N] is staged in LDS after
// the ring and read from asm like the ring.
template <int BM, int BN, int WGM, int WGN, int NS, int kWaves, bool kOutBf16, bool kBlocked = false>
__global__ __launch_bounds__(WGM * WGN * 64) __attribute__((amdgpu_waves_per_eu(kWaves))) void gemm_dma_kernel(
    const int8_t* __restrict__ q, const float* __restrict__ a_scale,
    const int32_t* __restrict__ q_rowsum, int M, int Kp,
    const uint8_t* __restrict__ packed, const float* __restrict__ w_scale, int N,
    void* __restrict__ y, int64_t ldy, int32_t* __restrict__ acc_debug, TileOrder order, int vec_store,
    const float* __restrict__ block_scale, int nb) {
    constexpr int kNW = WGM * WGN;
    constexpr int kThreads = kNW * 64;
    constexpr int WM = BM / WGM, WN = BN / WGN;
    constexpr int TM = WM / 32, TN = WN / 32;
    constexpr int SA = BM * BK, SB = BN * (BK / 4), STAGE = SA + SB;
    constexpr int A_DMA = SA / 1024 / kNW, B_DMA = SB / 1024 / kNW, D = A_DMA + B_DMA;
    static_assert((TM == 2 && (TN == 2 || TN == 4)) || (TM == 4 && TN == 2),
                  "wave tile 64 x 64, 64 x 128 or 128 x 64");
    static_assert(SA % (1024 * kNW) == 0 && SB % (1024 * kNW) == 0 && A_DMA >= 1 && B_DMA >= 1, "tile shape");
    static_assert(NS >= 2 && (NS - 1) * D < 64, "stage ring");

    extern __shared__ __attribute__((aligned(16))) int8_t lds[];   // [NS][activations SA | codes SB]
    __shared__ __attribute__((aligned(16))) float as_s[BM];
    __shared__ __attribute__((aligned(16))) int32_t rs_s[BM];
    __shared__ __attribute__((aligned(16))) float ws_s[BN];

    int tm, tn;
    tile_of(order, tm, tn);
    const int m0 = tm * BM, n0 = tn * BN;
    const int tid = threadIdx.x;
    const int lane = tid % 64;
    const int wave = tid / 64;
    const int wm = wave / WGN, wn = wave % WGN;
    const int r32 = lane % 32;
    const int g = lane / 32;
    const int brow_bytes = Kp / 4;
    const int stages = Kp / BK;

    const int a_rows = min(BM, M - m0), b_rows = min(BN, N - n0);
    const __amdgpu_buffer_rsrc_t a_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<int8_t*>(q + static_cast<int64_t>(m0) * Kp), 0, a_rows * Kp, kRsrcWord3);
    const __amdgpu_buffer_rsrc_t b_rsrc = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint8_t*>(packed + static_cast<int64_t>(n0) * brow_bytes), 0, b_rows * brow_bytes, kRsrcWord3);

    // Global offsets (stage 0) of the lane's 16 bytes in each of its loads.
    uint32_t a_off[A_DMA], b_off[B_DMA];
#pragma unroll
    for (int i = 0; i < A_DMA; ++i) {
        const int r = (i * kNW + wave) * 8 + lane / 8;           // 8 rows of 128 B per load
        a_off[i] = static_cast<uint32_t>(r * Kp + 16 * ((lane % 8) ^ swz_a(r)));
    }
#pragma unroll
    for (int i = 0; i < B_DMA; ++i) {
        const int n = (i * kNW + wave) * 32 + lane / 2;          // 32 rows of 32 B per load
        b_off[i] = static_cast<uint32_t>(n * brow_bytes + 16 * ((lane % 2) ^ swz_b(n)));
    }
    auto issue = [&](int ks, int buf) {                           // stage ks -> buffer buf (= ks % NS)
        const bool in = ks < stages;
        const uint32_t ka = in ? static_cast<uint32_t>(ks * BK) : kOutOfRange;
        const uint32_t kb = in ? static_cast<uint32_t>(ks * (BK / 4)) : kOutOfRange;
        int8_t* base = lds + buf * STAGE + wave * 1024;
#pragma unroll
        for (int i = 0; i < A_DMA; ++i)
            dma16(a_rsrc, base + i * kNW * 1024, a_off[i] + ka);
#pragma unroll
        for (int i = 0; i < B_DMA; ++i)
            dma16(b_rsrc, base + SA + i * kNW * 1024, b_off[i] + kb);
    };

    // LDS byte addresses of the lane's fragment reads in buffer 0: activation
    // row wm*WM + r32 (+32 rows at +4096), k chunk 4g + s; code row wn*WN + r32
    // (+32 rows per code tile at +1024), chunk g.
    const uint32_t lds0 = lds_offset(lds);
    uint32_t a_rd[4];
    {
        const int r = wm * WM + r32;
#pragma unroll
        for (int s = 0; s < 4; ++s) a_rd[s] = lds0 + r * BK + 16 * ((4 * g + s) ^ swz_a(r));
    }
    const int bn = wn * WN + r32;
    const uint32_t b_rd = lds0 + SA + bn * (BK / 4) + 16 * (g ^ swz_b(bn));

    for (int i = tid; i < BM; i += kThreads) {
        const int m = m0 + i;
        as_s[i] = m < M ? a_scale[m] : 0.0f;
        if constexpr (!kBlocked) rs_s[i] = m < M ? q_rowsum[m] : 0;   // kBlocked: q_rowsum not passed
    }
    float* const bs_lds = reinterpret_cast<float*>(lds + NS * STAGE);   // kBlocked: [nb][BN]
    if constexpr (kBlocked) {
        for (int i = tid; i < nb * BN; i += kThreads) {
            const int b = i / BN, n = n0 + i % BN;
            bs_lds[i] = n < N ? block_scale[static_cast<int64_t>(b) * N + n] : 0.0f;
        }
    } else {
        for (int i = tid; i < BN; i += kThreads) ws_s[i] = n0 + i < N ? w_scale[n0 + i] : 0.0f;
    }
#pragma unroll
    for (int u = 0; u < NS; ++u) issue(u, u);
    wait_vm<(NS - 1) * D>();
    __syncthreads();

    v16i acc[TN][TM];
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[j][i][r] = 0;

    f32x16 facc[TN][TM];                                          // kBlocked: scaled block sums
#pragma unroll
    for (int j = 0; j < TN; ++j)
#pragma unroll
        for (int i = 0; i < TM; ++i)
#pragma unroll
            for (int r = 0; r < 16; ++r) facc[j][i][r] = 0.0f;
    v4i a[TM], na[TM];
    u32x4 bw[TN];
    lds_issue_head(a, bw, a_rd[0], b_rd);
    lds_wait_head(a, bw);
    int cur = 0;                                                  // buffer of stage k
    v4i b[TN], bx[TN];                                            // this and the next step's codes
    u32x4 nbw[TN];
    for (int k = 0; k < stages; ++k) {
        const int nxt = cur + 1 == NS ? 0 : cur + 1;
        const uint32_t co = static_cast<uint32_t>(cur * STAGE), no = static_cast<uint32_t>(nxt * STAGE);
#pragma unroll
        for (int j = 0; j < TN; ++j) b[j] = kBlocked ? expand_word_signed(bw[j][0]) : expand_word(bw[j][0]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s == 3) {
                // every wave: own loads of stage k+1 landed, stage k's buffer read
                wait_vm<(NS - 2) * D>();
                __builtin_amdgcn_s_barrier();
                issue(k + NS, cur);
                lds_issue_head(na, nbw, a_rd[0] + no, b_rd + no);
            } else {
                lds_issue_a(na, a_rd[s + 1] + co);
            }
            __builtin_amdgcn_sched_barrier(0);
            if (s < 3) {
#pragma unroll
                for (int j = 0; j < TN; ++j)
                    bx[j] = kBlocked ? expand_word_signed(bw[j][s + 1]) : expand_word(bw[j][s + 1]);
            }
#pragma unroll
            for (int i = 0; i < TM; ++i)
#pragma unroll
                for (int j = 0; j < TN; ++j) acc[j][i] = mfma32(b[j], a[i], acc[j][i]);
#pragma unroll
            for (int t = 0; t < TM * TN; ++t) {
                __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);   // one MFMA
                __builtin_amdgcn_sched_group_barrier(0x002, BITNET_GEMM_VALU_GROUP, 0);   // then VALU ops
            }
            __builtin_amdgcn_sched_barrier(0);
            if (s == 3) {
                lds_wait_head(na, nbw);
            } else {
                lds_wait_a(na);
#pragma unroll
                for (int j = 0; j < TN; ++j) b[j] = bx[j];
            }
#pragma unroll
            for (int i = 0; i < TM; ++i) a[i] = na[i];
        }
#pragma unroll
        for (int j = 0; j < TN; ++j) bw[j] = nbw[j];
        if constexpr (kBlocked) {
            if ((k & 1) || k + 1 == stages) {             // block k/2 complete
#pragma unroll
                for (int j = 0; j < TN; ++j)
#pragma unroll
                    for (int rb = 0; rb < 4; ++rb) {
                        const u32x4 w4 = lds_read_b128(bs_lds + (k >> 1) * BN + wn * WN + j * 32 + 8 * rb + 4 * g);
#pragma unroll
                        for (int i = 0; i < TM; ++i)
#pragma unroll
                            for (int rr = 0; rr < 4; ++rr) {
                                const float term = static_cast<float>(acc[j][i][4 * rb + rr]) * __uint_as_float(w4[rr]);
                                facc[j][i][4 * rb + rr] = facc[j][i][4 * rb + rr] + term;
                                acc[j][i][4 * rb + rr] = 0;
                            }
                    }
            }
        }
        cur = nxt;
    }
    // the loads past the last stage must land before the workgroup's LDS is released
    wait_vm<0>();

    static_assert(kNW * epi_wave_bytes<WN, TM, kOutBf16>() <= NS * STAGE, "epilogue staging fits the ring");
    int8_t* const region = lds + wave * epi_wave_bytes<WN, TM, kOutBf16>();
    if (kBlocked && vec_store == 2) {
        __syncthreads();          // every wave has read the ring for the last time
        gemm_epilogue_lds<WM, WN, TM, TN, kOutBf16>(
            [&](int i, int j, int rb, int ml, int) {
                const float as = as_s[ml];
                f32x4 v;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = facc[j][i][4 * rb + rr] * as;
                return v;
            },
            region, m0, n0, wm, wn, lane, M, N, y, ldy);
    } else if (kBlocked) {
        gemm_epilogue_blocked<BM, BN, WM, WN, TM, TN, kOutBf16>(facc, as_s, m0, n0, wm, wn, r32, g, M, N, y, ldy,
                                                               vec_store);
    } else if (vec_store == 2 && !acc_debug) {
        __syncthreads();          // every wave has read the ring for the last time
        gemm_epilogue_lds<WM, WN, TM, TN, kOutBf16>(
            [&](int i, int j, int rb, int ml, int nl) {
                const float as = as_s[ml];
                const int32_t rs = rs_s[ml];
                const f32x4 ws4 = *reinterpret_cast<const f32x4*>(&ws_s[nl]);
                f32x4 v;
#pragma unroll
                for (int rr = 0; rr < 4; ++rr) v[rr] = static_cast<float>(acc[j][i][4 * rb + rr] - rs) * (as * ws4[rr]);
                return v;
            },
            region, m0, n0, wm, wn, lane, M, N, y, ldy);
    } else {
        gemm_epilogue<BM, BN, WM, WN, TM, TN, kOutBf16>(acc, as_s, rs_s, ws_s, m0, n0, wm, wn, r32, g, M, N, y, ldy,
                                                       acc_debug, vec_store);
    }
}

// BITNET_GEMM_EPILOGUE=direct keeps the register-to-global epilogue in the
// LDS-DMA kernel (for comparisons; results are identical), read at each launch.
bool epilogue_direct() {
    const char* v = getenv("BITNET_GEMM_EPILOGUE");
    return v && strcmp(v, "direct") == 0;
}

template <int BM, int BN, int WGM, int WGN, int NS, int kWaves>
hipError_t launch_tile_dma(const int8_t* q, const float* a_scale, const int32_t* q_rowsum, int64_t M, int64_t Kp,
                           const uint8_t* packed, const float* w_scale, int64_t N, void* y, bool y_bf16,
                           int64_t ldy, int32_t* acc_debug, int group_m, hipStream_t stream) {
    TileOrder order;
    order.tiles_m = static_cast<int>((M + BM - 1) / BM);
    order.tiles_n = static_cast<int>((N + BN - 1) / BN);
    order.group_m = group_m > 0 ? group_m : order.tiles_m;
    constexpr size_t lds = static_cast<size_t>(NS) * dma_stage_bytes<BM, BN>();
    const dim3 grid(static_cast<unsigned>(order.tiles_m) * order.tiles_n), block(WGM * WGN * 64);
    auto kern = y_bf16 ? gemm_dma_kernel<BM, BN, WGM, WGN, NS, kWaves, true>
                       : gemm_dma_kernel<BM, BN, WGM, WGN, NS, kWaves, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    // 1: 4-element vector stores; 2: 16-byte rows, so the LDS-staged epilogue
    const bool rows16 = (ldy * (y_bf16 ? 2 : 4)) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
    const int vec_store = rows16 && !epilogue_direct() ? 2 : (ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
    kern<<<grid, block, lds, stream>>>(q, a_scale, q_rowsum, (int)M, (int)Kp, packed, w_scale, (int)N, y, ldy,
                                       acc_debug, order, vec_store, nullptr, 0);
    return hipGetLastError();
}

template <int BM, int BN, int WGM, int WGN, int PF, int kWaves>
hipError_t launch_tile(const int8_t* q, const float* a_scale, const int32_t* q_rowsum, int64_t M, int64_t Kp,
                       const uint8_t* packed, const float* w_scale, int64_t N, void* y, bool y_bf16,
                       int64_t ldy, int32_t* acc_debug, int group_m, hipStream_t stream) {
    TileOrder order;
    order.tiles_m = static_cast<int>((M + BM - 1) / BM);
    order.tiles_n = static_cast<int>((N + BN - 1) / BN);
    order.group_m = group_m > 0 ? group_m : order.tiles_m;
    constexpr size_t lds = lds_bytes<BM, BN>();
    const dim3 grid(static_cast<unsigned>(order.tiles_m) * order.tiles_n), block(WGM * WGN * 64);
    auto kern = y_bf16 ? gemm_kernel<BM, BN, WGM, WGN, PF, kWaves, true>
                       : gemm_kernel<BM, BN, WGM, WGN, PF, kWaves, false>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    // vector stores need every row start aligned to 4 elements
    const int vec_store = (ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
    kern<<<grid, block, lds, stream>>>(q, a_scale, q_rowsum, (int)M, (int)Kp, packed, w_scale, (int)N, y, ldy,
                                       acc_debug, order, vec_store);
    return hipGetLastError();
}

}  // namespace

// Build-time knobs: register prefetch distance and tile rows per band.
#ifndef BITNET_GEMM_PF
#define BITNET_GEMM_PF 2
#endif
#ifndef BITNET_GEMM_GM
#define BITNET_GEMM_GM 8
#endif

namespace {

// Workgroups of one kernel that are resident on the current device at once
// (CUs x blocks per CU), cached per device; 0 if the query fails.
template <typename Kern>
int resident_slots(Kern kern, int threads, size_t lds, int (&cache)[64]) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
    if (cache[dev] == 0) {
        int cus = 0, per_cu = 0;
        if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(kern), threads, lds) !=
            hipSuccess)
            return 0;
        cache[dev] = cus * (per_cu > 0 ? per_cu : 1);
    }
    return cache[dev];
}

// A third tile, 64x64 with 2 waves of 32x64, for shapes whose 128x128 tiles
// would leave most resident slots empty (e.g. 2048 x 1152: 144 tiles for 768
// slots): four times the tiles at a lower MFMA rate per tile.
#ifndef BITNET_GEMM_TINY_FILL
#define BITNET_GEMM_TINY_FILL 0.5
#endif
bool use_tiny(int64_t M, int64_t N, int slots_small) {
    if (slots_small <= 0) return false;
    const int64_t tiles = ((M + 127) / 128) * ((N + 127) / 128);
    return static_cast<double>(tiles) < BITNET_GEMM_TINY_FILL * slots_small;
}

// Share of the launched rounds' resident slots that hold a tile.
double round_fill(int64_t tiles, int slots) {
    if (slots <= 0) return 1.0;
    const int64_t rounds = (tiles + slots - 1) / slots;
    return static_cast<double>(tiles) / static_cast<double>(rounds * slots);
}

int g_slots_small[64], g_slots_wide[64], g_slots_tiny[64];

// BITNET_GEMM_TILE=small|wide|tiny forces a tile (for comparisons; results are
// identical), read at each launch.
int forced_tile() {
    const char* v = getenv("BITNET_GEMM_TILE");
    if (!v) return -1;
    if (strcmp(v, "small") == 0) return 0;
    if (strcmp(v, "wide") == 0) return 1;
    if (strcmp(v, "tiny") == 0) return 2;
    return -1;
}

// BITNET_GEMM_KERNEL=regs selects the register-staged kernel for the 128x128
// and 128x256 tiles instead of the LDS-DMA one (for comparisons; results are
// identical), read at each launch.
bool use_regs_kernel() {
    const char* v = getenv("BITNET_GEMM_KERNEL");
    return v && strcmp(v, "regs") == 0;
}

#ifndef BITNET_GEMM_NS_WIDE
#define BITNET_GEMM_NS_WIDE 3
#endif
// Wave grid of the wide LDS-DMA tile: 1 x 4 waves of 128x64 (each expanded
// code word feeds four 32-row activation fragments) or 2 x 2 of 64x128 (two).
#ifndef BITNET_GEMM_WIDE_WGM
#define BITNET_GEMM_WIDE_WGM 1
#endif
constexpr int kWideWGM = BITNET_GEMM_WIDE_WGM, kWideWGN = 4 / BITNET_GEMM_WIDE_WGM;
#ifndef BITNET_GEMM_NS_SMALL
#define BITNET_GEMM_NS_SMALL 2
#endif
int g_dslots_small[64], g_dslots_wide[64];

}  // namespace

hipError_t launch_gemm(const int8_t* q, const float* a_scale, const int32_t* q_rowsum,
                       int64_t M, int64_t Kp, const uint8_t* packed, const float* w_scale,
                       int64_t N, void* y, bool y_bf16, int64_t ldy, int32_t* acc_debug,
                       hipStream_t stream) {
    // Two tiles: 128x128 with 2x2 waves of 64x64 (3 workgroups per CU), and
    // 128x256 with 1x4 waves of 128x64 (2 per CU), which has 40% fewer global
    // bytes per MFMA and runs each tile faster.
    // The grid runs in rounds of resident workgroups, so the choice weighs
    // that gain against the share of the last round left empty (e.g. N=3840:
    // 960 small tiles fill 1.25 rounds of 768, 480 wide tiles 0.94 of 512).
    const bool regs = use_regs_kernel();
    const int slots_small =
        regs ? resident_slots(gemm_kernel<128, 128, 2, 2, BITNET_GEMM_PF, 3, true>, 256, lds_bytes<128, 128>(),
                              g_slots_small)
             : resident_slots(gemm_dma_kernel<128, 128, 2, 2, BITNET_GEMM_NS_SMALL, 3, true>, 256,
                              BITNET_GEMM_NS_SMALL * dma_stage_bytes<128, 128>(), g_dslots_small);
    const int slots_wide =
        regs ? resident_slots(gemm_kernel<128, 256, 2, 2, BITNET_GEMM_PF, 2, true>, 256, lds_bytes<128, 256>(),
                              g_slots_wide)
             : resident_slots(gemm_dma_kernel<128, 256, kWideWGM, kWideWGN, BITNET_GEMM_NS_WIDE, 2, true>, 256,
                              BITNET_GEMM_NS_WIDE * dma_stage_bytes<128, 256>(), g_dslots_wide);
    const int64_t tiles_m = (M + 127) / 128;
    const double small = round_fill(tiles_m * ((N + 127) / 128), slots_small);
    const int64_t tiles_wide = tiles_m * ((N + 255) / 256);
    const double wide = 1.07 * round_fill(tiles_wide, slots_wide);
    // Measured on the prefill shapes: the wide tile wins only with K >= 2048
    // (with 8-16 stages the per-tile prologue and epilogue favour three
    // resident 128x128 tiles) and at least ~a full round of wide tiles.
    const bool use_wide = wide > small && Kp >= 2048 && tiles_wide * 10 >= static_cast<int64_t>(slots_wide) * 9;
    const int forced = forced_tile();
    if (forced == 2 || (forced < 0 && use_tiny(M, N, slots_small)))
        return launch_tile<64, 64, 2, 1, BITNET_GEMM_PF, 4>(q, a_scale, q_rowsum, M, Kp, packed, w_scale, N, y, y_bf16,
                                                            ldy, acc_debug, BITNET_GEMM_GM, stream);
    if (forced == 1 || (forced < 0 && use_wide))
        return regs ? launch_tile<128, 256, 2, 2, BITNET_GEMM_PF, 2>(q, a_scale, q_rowsum, M, Kp, packed, w_scale, N,
                                                                     y, y_bf16, ldy, acc_debug, BITNET_GEMM_GM, stream)
                    : launch_tile_dma<128, 256, kWideWGM, kWideWGN, BITNET_GEMM_NS_WIDE, 2>(
                          q, a_scale, q_rowsum, M, Kp, packed, w_scale, N, y, y_bf16, ldy, acc_debug, BITNET_GEMM_GM,
                          stream);
    return regs ? launch_tile<128, 128, 2, 2, BITNET_GEMM_PF, 3>(q, a_scale, q_rowsum, M, Kp, packed, w_scale, N, y,
                                                                 y_bf16, ldy, acc_debug, BITNET_GEMM_GM, stream)
                : launch_tile_dma<128, 128, 2, 2, BITNET_GEMM_NS_SMALL, 3>(q, a_scale, q_rowsum, M, Kp, packed,
                                                                         w_scale, N, y, y_bf16, ldy, acc_debug,
                                                                         BITNET_GEMM_GM, stream);
}

hipError_t launch_gemm_blocked(const int8_t* q, const float* a_scale, int64_t M, int64_t K, int64_t Kp,
                               const uint8_t* packed, const float* block_scale, int64_t N, void* y, bool y_bf16,
                               int64_t ldy, hipStream_t stream) {
    // 128x128 tiles (2x2 waves of 64x64): the fp32 block accumulators double
    // the accumulator registers, which leaves two workgroups per CU.
    constexpr int BM = 128, BN = 128, NS = 2;
    const int nb = static_cast<int>((K + 255) / 256);
    TileOrder order;
    order.tiles_m = static_cast<int>((M + BM - 1) / BM);
    order.tiles_n = static_cast<int>((N + BN - 1) / BN);
    order.group_m = BITNET_GEMM_GM;
    const size_t lds = static_cast<size_t>(NS) * dma_stage_bytes<BM, BN>() + static_cast<size_t>(nb) * BN * sizeof(float);
    auto kern = y_bf16 ? gemm_dma_kernel<BM, BN, 2, 2, NS, 2, true, true>
                       : gemm_dma_kernel<BM, BN, 2, 2, NS, 2, false, true>;
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, static_cast<int>(lds));
    if (e != hipSuccess) return e;
    const bool rows16 = (ldy * (y_bf16 ? 2 : 4)) % 16 == 0 && reinterpret_cast<uintptr_t>(y) % 16 == 0;
    const int vec_store = rows16 && !epilogue_direct() ? 2 : (ldy % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0);
    const dim3 grid(static_cast<unsigned>(order.tiles_m) * order.tiles_n), block(256);
    kern<<<grid, block, lds, stream>>>(q, a_scale, nullptr, (int)M, (int)Kp, packed, nullptr, (int)N, y, ldy,
                                       nullptr, order, vec_store, block_scale, nb);
    return hipGetLastError();
}

}  // namespace bitnet
