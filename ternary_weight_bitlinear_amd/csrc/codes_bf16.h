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

// ---- 2t by one packed 16-bit multiply-add per two values
//
// -2.0, 0 and +2.0 have the same 16-bit patterns in bf16 and in fp16 (0xC000,
// 0x0000, 0x4000), and these equal u * 0x4000 + 0xC000 modulo 2^16 for the
// code u = t + 1: linear in u.  So with one code alone at bit b of both
// 16-bit halves of a word (the others masked off), v_pk_mad_u16 by 2^(14 - b)
// plus 0xC000 gives two operands; for b = 0 no mask is needed, since every
// higher code is carried out of its half by the multiply.  A word's byte
// pairs (0, 2) and (1, 3) share a half-word position, so the two values of
// one result are k and k + 2 of a field: 15 VALU ops per 16 codes, against
// 24 with the table permutes above.  The operand's k order within each 8 is
// 0 2 1 3 4 6 5 7; the activations' copy is permuted to match
// (interleave_x_pairs).  Sums are twice those of t, as for the bf16 table.
typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));

// Multipliers in scalar registers: a multiply by a power of two the compiler
// can see becomes a shift and a separate add.
struct TwiceMultipliers {
    uint32_t m[8];   // [2p]: 2^(14 - 2p) for field p of bytes 0, 2; [2p + 1]: 2^(6 - 2p) for bytes 1, 3
    __device__ __forceinline__ TwiceMultipliers() {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
            uint32_t e = 0x00010001u << (14 - 2 * p), o = 0x00010001u << (6 - 2 * p);
            asm("" : "+s"(e));
            asm("" : "+s"(o));
            m[2 * p] = e;
            m[2 * p + 1] = o;
        }
    }
};

// Field p's codes of byte pair (0, 2) (kOdd false) or (1, 3) (kOdd true) of
// w as two 16-bit operands 2t.
template <bool kOdd>
__device__ __forceinline__ uint32_t twice_pair(uint32_t w, int p, const TwiceMultipliers& mul) {
    const int b = 2 * p + (kOdd ? 8 : 0);
    const uint32_t sel = (0x00030003u << b);
    const uint32_t v = b == 0 ? w : (w & sel);
    const u16x2 r = __builtin_bit_cast(u16x2, v) * __builtin_bit_cast(u16x2, mul.m[2 * p + (kOdd ? 1 : 0)]) +
                    u16x2{0xC000, 0xC000};
    return __builtin_bit_cast(uint32_t, r);
}

// 8 operands 2t from fields 2h and 2h + 1 of w (k = 16j + 8h + 0 2 1 3 4 6 5 7).
__device__ __forceinline__ u32x4 expand_twice_interleaved(uint32_t w, int h, const TwiceMultipliers& mul) {
    return u32x4{twice_pair<false>(w, 2 * h, mul), twice_pair<true>(w, 2 * h, mul),
                 twice_pair<false>(w, 2 * h + 1, mul), twice_pair<true>(w, 2 * h + 1, mul)};
}

// 8 consecutive 16-bit activations (k ascending, two per word) in the k order
// of expand_twice_interleaved.
__device__ __forceinline__ u32x4 interleave_x_pairs(u32x4 v) {
    return u32x4{__builtin_amdgcn_perm(v.y, v.x, 0x05040100u), __builtin_amdgcn_perm(v.y, v.x, 0x07060302u),
                 __builtin_amdgcn_perm(v.w, v.z, 0x05040100u), __builtin_amdgcn_perm(v.w, v.z, 0x07060302u)};
}

}  // namespace bitnet
