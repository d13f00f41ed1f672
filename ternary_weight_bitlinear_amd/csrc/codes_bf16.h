// codes_bf16.h -- bf16 and fp16 operands of t = u - 1 from layout-v1 packed
// codes, for the W1.58A16 kernels (16-bit matrix cores), internal.
#pragma once

#include "device_common.h"

namespace bitnet {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

// bf16 bytes of t = u - 1 for stored codes u = 0, 1, 2 (-1.0, 0.0, +1.0):
// low bytes 0x80, 0x00, 0x80 and high bytes 0xBF, 0x00, 0x3F.
constexpr uint32_t kTableLo = 0x00800080u;
constexpr uint32_t kTableHi = 0x003F00BFu;

// Four bf16 values of t from the codes in the bytes of f (each 0..2), as two
// dwords of two: with g = f + 4 in every byte, one byte permute of (g, f)
// spreads two codes to [u0, u0 + 4, u1, u1 + 4] (the +4 picks the high-byte
// table) and a second looks both tables up: 5 VALU ops per 4 codes.
__device__ __forceinline__ u32x2 bf16_quad(uint32_t f) {
    const uint32_t g = f + 0x04040404u;
    return u32x2{__builtin_amdgcn_perm(kTableHi, kTableLo, __builtin_amdgcn_perm(g, f, 0x05010400u)),
                 __builtin_amdgcn_perm(kTableHi, kTableLo, __builtin_amdgcn_perm(g, f, 0x07030602u))};
}

// B operand (8 bf16 of t, k ascending) from fields 2h and 2h+1 of a packed
// word: field p holds k = 16j + 4p + b in byte b, so the two fields cover the
// 8 consecutive k from 16j + 8h.
__device__ __forceinline__ u32x4 expand_bf16(uint32_t w, int h) {
    const u32x2 a = bf16_quad((w >> (4 * h)) & 0x03030303u);
    const u32x2 b = bf16_quad((w >> (4 * h + 2)) & 0x03030303u);
    return u32x4{a.x, a.y, b.x, b.y};
}

// fp16 of t = u - 1 has a zero low byte for all three codes (-1.0 = 0xBC00,
// 0.0 = 0x0000, +1.0 = 0x3C00), so one byte permute against the high bytes
// 0xBC, 0x00, 0x3C -- with selector byte 12 giving the constant zero low
// bytes -- turns a selector [12, u0, 12, u1] into two fp16 values; the
// selector itself is one permute of the codes against the constant 12:
// 4 VALU ops per 4 codes (bf16 needs 5: its low bytes differ).
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
constexpr uint32_t kTableF16 = 0x003C00BCu;
constexpr uint32_t kSel12 = 0x0C0C0C0Cu;

__device__ __forceinline__ u32x2 f16_quad(uint32_t f) {
    return u32x2{__builtin_amdgcn_perm(0u, kTableF16, __builtin_amdgcn_perm(f, kSel12, 0x05000400u)),
                 __builtin_amdgcn_perm(0u, kTableF16, __builtin_amdgcn_perm(f, kSel12, 0x07000600u))};
}

// B operand (8 fp16 of t, k ascending) from fields 2h and 2h+1 of a packed word.
__device__ __forceinline__ u32x4 expand_f16(uint32_t w, int h) {
    const u32x2 a = f16_quad((w >> (4 * h)) & 0x03030303u);
    const u32x2 b = f16_quad((w >> (4 * h + 2)) & 0x03030303u);
    return u32x4{a.x, a.y, b.x, b.y};
}

}  // namespace bitnet
