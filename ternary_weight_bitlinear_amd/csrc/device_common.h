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

// exp(t) in fp32 by fixed IEEE steps (Cody and Waite's argument reduction
// with a Taylor polynomial), used for the gated input silu(a) * u of the down
// projection, where it stays within 2 fp32 ulps of exp and silu(a) * u within
// 4 ulps of the exact value, independent of any math library:
// +inf above 88 and 0 below -88; else n = rint(t * log2 e), reduced argument
// r = (t - n * ln2_hi) - n * ln2_lo with a 15-bit ln2_hi (n * ln2_hi exact),
// the degree-7 Taylor polynomial of exp at r in Horner form (|r| <= ln2/2),
// times 2^n.  Each line is one correctly rounded fp32 operation (contraction
// is off for these sources).
__device__ __forceinline__ float exp_f32_fixed(float t) {
    if (t > 88.0f) return __builtin_inff();
    if (t < -88.0f) return 0.0f;
    const float n = rne(t * 1.44269502f);
    const float r = (t - n * 0.693145752f) - n * 1.42860677e-06f;
    float p = 1.0f / 5040.0f;
    p = p * r + 1.0f / 720.0f;
    p = p * r + 1.0f / 120.0f;
    p = p * r + 1.0f / 24.0f;
    p = p * r + 1.0f / 6.0f;
    p = p * r + 0.5f;
    p = p * r + 1.0f;
    p = p * r + 1.0f;
    return __builtin_ldexpf(p, static_cast<int>(n));
}

// silu(a) * u = a / (1 + exp(-a)) * u, fp32.
__device__ __forceinline__ float silu_mul(float a, float u) { return a / (1.0f + exp_f32_fixed(-a)) * u; }

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
