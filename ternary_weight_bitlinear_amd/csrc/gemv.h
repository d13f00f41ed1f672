// gemv.h -- descriptor of one decode-size problem (internal; plain data shared
// by the host launcher and the gfx950 kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <vector>

namespace bitnet {

struct GemvProblem {
    const void* x;             // fused: activations [M, K], row stride ldx (elements)
    int64_t ldx;
    const int8_t* q;           // unfused: quantised activations [M][Kp]
    const float* a_scale;      // unfused: [M]
    const int32_t* q_rowsum;   // unfused: [M]
    int8_t* q_out;             // fused, optional: receives q [M][Kp]
    float* a_scale_out;        // fused, optional: receives a_scale [M]
    int32_t* rowsum_out;       // fused, optional: receives q_rowsum [M]
    const uint8_t* packed;     // [N][Kp/4], layout v1
    const float* w_scale;      // [N]
    void* y;                   // [M, N], row stride ldy
    int64_t ldy;
    int32_t* acc_debug;        // optional [M][N]
    const void* up;            // fused, optional: input is silu(x) * up (x's dtype and stride)
    const void* norm_w;        // fused, optional: RMSNorm weight [K] applied before ActQuant
    float eps;                 // fused: RMSNorm epsilon
    int32_t norm_bf16;         // fused: norm_w is bf16 (else fp32)
    int32_t M, N, K, Kp;
    int32_t tile0;             // grouped: global index of this problem's first 64-row tile
    int32_t ntiles;            // grouped: tiles of this problem
    int32_t steps;             // grouped: 256-element k steps per tile (Kp / 256, rounded up)
    int32_t reserved;
    int64_t step0;             // grouped: steps of all earlier problems (ntiles * steps each)
};

// LDS bytes the grouped kernel needs for M tokens of the longest row.
size_t gemv_group_lds(int64_t M, int64_t max_Kp);

// Tiles (64 output rows) and k steps per tile of a grouped problem.
int64_t gemv_group_tiles(int64_t N);
int64_t gemv_group_steps(int64_t Kp);

// Fused ActQuant + decode linear for one problem; LDS holds M*Kp bytes.
hipError_t launch_gemv_fused(const GemvProblem& p, bool x_bf16, bool y_bf16, hipStream_t stream);

// Largest grid of a grouped streaming launch: the device table holds this
// many + 1 share bounds after the problems.
constexpr int kMaxStreamGrid = 4096;

// Whether the streaming kernel (per-wave LDS ring of DMA weight loads) can
// run this table of problems (host copy, tile0 / ntiles / steps / step0 set):
// every workgroup's problems must fit its LDS share, with token rows of
// token_bytes per element (1: int8 codes; 2: the bf16 rows of the W1.58A16
// kernel).  On success gives the grid and the dynamic LDS bytes to launch with.
// `bounds` (grouped launches) receives grid + 1 share bounds, to be uploaded
// right after the problem table; without it the shares are k-step shares
// snapped to tile starts (single problems).
// `blocked`: the per-256-block scale version of the kernel, which keeps less
// LDS for token rows.
bool gemv_stream_plan(const GemvProblem* host_table, int count, int64_t total_tiles, int64_t total_steps,
                      int* grid, size_t* lds, int token_bytes = 1, std::vector<int32_t>* bounds = nullptr,
                      bool blocked = false);

// Per-256-block weight scales (w_scale holds block_scale [ceil(K/256)][N]):
// one problem on quantised tokens (q, a_scale; M <= 16) through the streaming
// kernel; hipErrorInvalidValue if its token rows do not fit.
hipError_t launch_gemv_blocked(const GemvProblem& p, bool y_bf16, hipStream_t stream);

// Grouped block-scaled launch (ActQuant fused), table and grid from
// gemv_stream_plan(..., blocked = true).
hipError_t launch_gemv_blocked_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles,
                                       int64_t total_steps, int grid, bool x_bf16, bool y_bf16, hipStream_t stream);

// W1.58A16 grouped launch of the streaming kernel (bf16 or fp16 x, no quantiser):
// table_dev and the grid as for launch_gemv_grouped's streaming case.
hipError_t launch_gemv_a16_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles,
                                   int64_t total_steps, int grid, bool y_bf16, hipStream_t stream,
                                   bool x_f16 = false);

// Many independent problems in one launch (ActQuant fused); table_dev is a
// device array of `count` descriptors with tile0 / ntiles / steps / step0 set.
// stream_grid > 0 runs the streaming kernel with that grid and `lds` from
// gemv_stream_plan, otherwise the persistent kernel with `lds` for the longest row.
hipError_t launch_gemv_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles,
                               int64_t total_steps, size_t lds, int stream_grid, bool x_bf16, bool y_bf16,
                               hipStream_t stream);

}  // namespace bitnet
