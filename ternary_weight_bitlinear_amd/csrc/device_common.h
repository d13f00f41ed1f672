// device_common.h -- small device helpers shared by the gfx950 kernels.
//
// Numerics: every kernel is compiled with -ffp-contract=off and correctly
// rounded fp32 division, so x*sa, 127/amax, a_scale*w_scale and (float)acc*f
// are single IEEE operations with round-to-nearest-even, the same operations
// in the same order as the definition in bitnet.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace bitnet {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// Loads and stores through pointers that the compiler cannot prove global (for
// example pointers read from a descriptor in memory) would otherwise become
// flat accesses, which count against both wait counters and force a full
// wait before every use; these casts make them global_load / global_store so
// independent loads can stay in flight.
#define BITNET_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ T gload(const void* p) {
    return *(const BITNET_GLOBAL T*)(p);
}
template <typename T>
__device__ __forceinline__ void gstore(void* p, T v) {
    *(BITNET_GLOBAL T*)(p) = v;
}

constexpr int kWave = 64;

// bf16 bit pattern -> fp32 (exact widening).
__device__ __forceinline__ float bf16_to_f32(uint16_t h) {
    return __uint_as_float(static_cast<uint32_t>(h) << 16);
}

// fp32 -> bf16, round to nearest even; NaN -> quiet NaN.
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return static_cast<uint16_t>(u >> 16);
}

// Two packed bf16 (low half = element 0) -> fp32 pair.
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// Round half to even (v_rndne_f32).
__device__ __forceinline__ float rne(float v) { return __builtin_rintf(v); }

// ActQuant codes of eight values: rne(fp32(v * sa)) as int8, packed little-
// endian into lo (values 0-3) and hi (4-7); returns their sum.  For |p| below
// 2^22, fp32(p + 1.5 * 2^23) equals 1.5 * 2^23 + rne(p) (its ulp is 1 and the
// constant is even, so ties go to the even integer exactly as rne does), and
// the low byte of its bits is rne(p) in two's complement.  Callers pass
// |v| <= amax with sa = fp32(127 / amax) (or sa = 0), so |v * sa| rounds to at
// most 127 and the [-128, 127] clamp of the definition never binds.  The
// product and the sum are rounded separately (fp contraction is off).
__device__ __forceinline__ int quant8_codes(const float (&v)[8], float sa, uint32_t& lo, uint32_t& hi) {
    constexpr float kRound = 12582912.0f;                  // 1.5 * 2^23
    uint32_t b[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) b[i] = __float_as_uint(__fadd_rn(__fmul_rn(v[i], sa), kRound));
    // low bytes of two values, then of four: byte selectors 0 and 4 pick
    // byte 0 of the second and the first operand, 12 gives zero
    lo = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[3], b[2], 0x0C0C0400u),
                               __builtin_amdgcn_perm(b[1], b[0], 0x0C0C0400u), 0x05040100u);
    hi = __builtin_amdgcn_perm(__builtin_amdgcn_perm(b[7], b[6], 0x0C0C0400u),
                               __builtin_amdgcn_perm(b[5], b[4], 0x0C0C0400u), 0x05040100u);
    return __builtin_amdgcn_sdot4(static_cast<int>(hi), 0x01010101,
                                  __builtin_amdgcn_sdot4(static_cast<int>(lo), 0x01010101, 0, false), false);
}

// Four stored codes of one 32-bit packed word, lane p = 0..3: the bytes hold
// elements 16j+4p+0..3 as unsigned values u in {0,1,2}.
__device__ __forceinline__ uint32_t codes_of(uint32_t word, int p) {
    return (word >> (2 * p)) & 0x03030303u;
}

// Expand one packed word (16 elements) into a 16-byte int8 MFMA operand whose
// byte 4p+b is element 16j+4p+b.
__device__ __forceinline__ v4i expand_word(uint32_t w) {
    v4i r;
    r[0] = static_cast<int>(w & 0x03030303u);
    r[1] = static_cast<int>((w >> 2) & 0x03030303u);
    r[2] = static_cast<int>((w >> 4) & 0x03030303u);
    r[3] = static_cast<int>((w >> 6) & 0x03030303u);
    return r;
}

// exp(t) in fp32 for the gated input silu(a) * u of the down projection:
// +inf above 88 and 0 below -104 (where e^t < 2^-150); else t * log2(e) is
// carried as hi + lo, with hi = fp32(t * L) and lo = fma(t, L, -hi) + t * L_lo,
// where L + L_lo is log2(e) to about 2^-52 (L = fp32(log2 e)); the fma gives
// the rounding error of t * L exactly, so hi + lo is t * log2(e) to ~2^-40
// relative.  With n = rint(hi) and f = hi - n (exact, |f| <= 1/2),
// e^t = 2^n * 2^(f + lo): 2^(f + lo) is the hardware exp2 (v_exp_f32) of a
// value within ~0.51 of zero, whose own rounding adds at most ln 2 * 2^-25
// relative, and 2^n is an ldexp (exact for normal results, one rounding for
// subnormal ones).  This is the usual two-constant reduction of an
// exponential to a power of two (as in Cody and Waite's method), with the
// polynomial replaced by the hardware's exp2.  Measured on MI355X: within
// 0.85 fp32 ulps of exp(t) over [-87, 88].
__device__ __forceinline__ float exp_f32(float t) {
    if (t > 88.0f) return __builtin_inff();
    if (t < -104.0f) return 0.0f;
    constexpr float kL = 1.44269502f;                   // fp32(log2 e), 0x3FB8AA3B
    constexpr float kLlo = 1.925963e-08f;               // log2 e - kL
    const float hi = t * kL;
    const float lo = __builtin_fmaf(t, kL, -hi) + t * kLlo;
    const float n = rne(hi);
    return __builtin_ldexpf(__builtin_amdgcn_exp2f((hi - n) + lo), static_cast<int>(n));
}

// silu(a) * u = a * sigmoid(a) * u in fp32, from e = exp(-|a|) in (0, 1]
// (never overflows): sigmoid(a) = 1 / (1 + e) for a >= 0 and e / (1 + e) for
// a < 0, the quotient taken with the hardware reciprocal (v_rcp_f32, 1 ulp).
// Relative error at most ~4.3 fp32 ulps where e is normal (|a| <= 87): 0.85
// from exp_f32, 0.5 for a * e (a < 0 only), 0.9 for 1 + e (its sum plus e's
// error at weight e / (1 + e) <= 1/2), 1 for rcp and 0.5 for each of the two
// remaining products.  For a < -87 the term a * e is subnormal-limited: its
// absolute error stays below |a * u| * 2^-149.
__device__ __forceinline__ float silu_mul(float a, float u) {
    const float e = exp_f32(-fabsf(a));
    const float s = a >= 0.0f ? a : a * e;
    return s * __builtin_amdgcn_rcpf(1.0f + e) * u;
}

// Wave reductions without LDS traffic: DPP moves within each 16-lane row
// (lane ^ 1, lane ^ 2, the other quad of the half row, the other half of the
// row), after which every lane of a row holds the row's result, then the four
// rows' results read out with v_readlane.  Max and integer sum do not depend
// on the order of combination; the result is wave-uniform.
template <int kCtrl>
__device__ __forceinline__ int dpp_move(int v) {
    return __builtin_amdgcn_update_dpp(0, v, kCtrl, 0xF, 0xF, false);
}
constexpr int kDppXor1 = 0xB1;          // quad_perm [1, 0, 3, 2]
constexpr int kDppXor2 = 0x4E;          // quad_perm [2, 3, 0, 1]
constexpr int kDppHalfMirror = 0x141;   // lane i <-> 7 - i within each half row
constexpr int kDppMirror = 0x140;       // lane i <-> 15 - i within each row

__device__ __forceinline__ float wave_max(float v) {
    v = fmaxf(v, __int_as_float(dpp_move<kDppXor1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<kDppXor2>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<kDppHalfMirror>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_move<kDppMirror>(__float_as_int(v))));
    const int b = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}

__device__ __forceinline__ int wave_sum(int v) {
    v += dpp_move<kDppXor1>(v);
    v += dpp_move<kDppXor2>(v);
    v += dpp_move<kDppHalfMirror>(v);
    v += dpp_move<kDppMirror>(v);
    return (__builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16)) +
           (__builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48));
}

// 16x16x64 int8 MFMA (gfx950): C[i][j] += sum_k A[i][k] B[k][j]; lane l holds
// row i = l%16 of A and column j = l%16 of B for one group of 16 k values
// (the same group for A and B), and C[4*(l/16)+r][l%16] in register r.
__device__ __forceinline__ v4i mfma16(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

}  // namespace bitnet
