// codes_bf16.h -- bf16 operands of t = u - 1 from layout-v1 packed codes, for
// the W1.58A16 kernels (bf16 matrix cores), internal.
#pragma once

#include "device_common.h"

namespace bitnet {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 bytes of t = u - 1 for stored codes u = 0, 1, 2 (-1.0, 0.0, +1.0):
// low bytes 0x80, 0x00, 0x80 and high bytes 0xBF, 0x00, 0x3F.
constexpr uint32_t kTableLo = 0x00800080u;
constexpr uint32_t kTableHi = 0x003F00BFu;

// Two bf16 values of t from the codes in bytes i0 and i1 of f (each 0..2):
// a byte permute spreads them to [u0, u0, u1, u1], +4 on the odd bytes picks
// the high-byte table, and a second permute looks both tables up.
template <uint32_t kSpread>
__device__ __forceinline__ uint32_t bf16_pair(uint32_t f) {
    const uint32_t sel = __builtin_amdgcn_perm(f, f, kSpread) + 0x04000400u;
    return __builtin_amdgcn_perm(kTableHi, kTableLo, sel);
}

// B operand (8 bf16 of t, k ascending) from fields 2h and 2h+1 of a packed
// word: field p holds k = 16j + 4p + b in byte b, so the two fields cover the
// 8 consecutive k from 16j + 8h.
__device__ __forceinline__ u32x4 expand_bf16(uint32_t w, int h) {
    const uint32_t f0 = (w >> (4 * h)) & 0x03030303u;
    const uint32_t f1 = (w >> (4 * h + 2)) & 0x03030303u;
    return u32x4{bf16_pair<0x01010000u>(f0), bf16_pair<0x03030202u>(f0), bf16_pair<0x01010000u>(f1),
                 bf16_pair<0x03030202u>(f1)};
}

}  // namespace bitnet
