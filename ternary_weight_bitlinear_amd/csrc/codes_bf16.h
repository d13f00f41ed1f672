// codes_bf16.h -- bf16 and fp16 operands of the ternary weights from layout-v1
// packed codes, for the W1.58A16 kernels (16-bit matrix cores), internal.
#pragma once

#include "device_common.h"

namespace bitnet {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

// fp16 of t = u - 1 has a zero low byte for all three codes (-1.0 = 0xBC00,
// 0.0 = 0x0000, +1.0 = 0x3C00), so one byte permute against the high bytes
// 0xBC, 0x00, 0x3C -- with selector byte 12 giving the constant zero low
// bytes -- turns a selector [12, u0, 12, u1] into two fp16 values; the
// selector itself is one permute of the codes against the constant 12:
// 4 VALU ops per 4 codes.
//
// bf16 of t itself has a non-zero low byte (-1.0 = 0xBF80), but bf16 of 2t
// does not (-2.0 = 0xC000, +2.0 = 0x4000), so the bf16 operand holds 2t and
// expands the same way.  Products x * 2t are exact, and an fp32 sum of
// values all scaled by 2 rounds exactly as the unscaled sum does, so the
// kernels' fp32 sums are exactly twice those of t (while below 2^127 in
// magnitude) and are halved before the epilogue: the same bits as with t.
constexpr uint32_t kTableF16 = 0x003C00BCu;
constexpr uint32_t kTableBf16Twice = 0x004000C0u;
constexpr uint32_t kSel12 = 0x0C0C0C0Cu;

// Two 16-bit values from the codes in bytes 0-1 and 2-3 of f (each 0..2):
// table holds the high bytes of the values for codes 0, 1, 2.
template <uint32_t kTable>
__device__ __forceinline__ u32x2 hi_byte_quad(uint32_t f) {
    return u32x2{__builtin_amdgcn_perm(0u, kTable, __builtin_amdgcn_perm(f, kSel12, 0x05000400u)),
                 __builtin_amdgcn_perm(0u, kTable, __builtin_amdgcn_perm(f, kSel12, 0x07000600u))};
}

// B operand (8 values, k ascending) from fields 2h and 2h+1 of a packed word:
// field p holds k = 16j + 4p + b in byte b, so the two fields cover the 8
// consecutive k from 16j + 8h.
template <uint32_t kTable>
__device__ __forceinline__ u32x4 expand_hi_bytes(uint32_t w, int h) {
    const u32x2 a = hi_byte_quad<kTable>((w >> (4 * h)) & 0x03030303u);
    const u32x2 b = hi_byte_quad<kTable>((w >> (4 * h + 2)) & 0x03030303u);
    return u32x4{a.x, a.y, b.x, b.y};
}

// 8 fp16 of t.
__device__ __forceinline__ u32x4 expand_f16(uint32_t w, int h) { return expand_hi_bytes<kTableF16>(w, h); }

// 8 bf16 of 2t (sums built from them are halved before use).
__device__ __forceinline__ u32x4 expand_bf16_twice(uint32_t w, int h) {
    return expand_hi_bytes<kTableBf16Twice>(w, h);
}

}  // namespace bitnet
