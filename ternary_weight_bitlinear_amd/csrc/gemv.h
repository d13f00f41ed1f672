// gemv.h -- descriptor of one decode-size problem (internal; plain data shared
// by the host launcher and the gfx950 kernel).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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
    int32_t M, N, K, Kp;
    int32_t tile0;             // grouped: index of this problem's first workgroup
    int32_t reserved;
};

// Workgroups (tiles of output rows) a problem with N rows needs.
int64_t gemv_tiles(int64_t N);

// Fused ActQuant + decode linear for one problem; LDS holds M*Kp bytes.
hipError_t launch_gemv_fused(const GemvProblem& p, bool x_bf16, bool y_bf16, hipStream_t stream);

// Many independent problems in one launch; table_dev is a device array of
// `count` descriptors ordered by tile0, total_tiles = sum of gemv_tiles(N).
hipError_t launch_gemv_grouped(const GemvProblem* table_dev, int count, int64_t total_tiles, size_t lds,
                               bool fused, bool x_bf16, bool y_bf16, hipStream_t stream);

}  // namespace bitnet
