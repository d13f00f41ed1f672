/*
 * bitnet_oracle.c -- plain, slow CPU oracle for the W1.58A8 BitLinear.
 *
 * TEST INFRASTRUCTURE ONLY.  The tests, the smoke check and the CPU-baseline
 * leg of the benchmark load this file's shared object; the product library
 * never includes, links or calls it, and it shares no code with the HIP path.
 *
 * Pages cited (title, then section):
 *   [BitVLA] "BitVLA -- 1.58-bit Vision-Language-Action on Core AI"
 *            (Core AI model zoo).
 *   [Guide]  "BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference
 *            Optimization Guide" (microsoft/BitNet docs).
 *   [BitMar] "BitMar: Low-Bit Multimodal Fusion with Episodic Memory for Edge
 *            Devices" (AI summary page).
 *
 * What is computed (y = linear(ActQuant(x), WeightQuant(W)), no bias):
 *   WeightQuant  [BitVLA s1; Guide s2 and s3.3 "I2_S Ternary Packing"]:
 *                one scale per source tensor, s = 1/mean|W|, codes
 *                t = clamp(round(W*s), -1, +1), dequantised value t/s.
 *   ActQuant     [BitVLA s1; Guide s2]: per token, int8 codes
 *                q = clamp(round(x*127/max|x|), -128, 127), dequantised by
 *                dividing by 127/max|x|.
 *   Encoding     [Guide s3.3; BitVLA s2]: stored code u = t + 1, i.e.
 *                -1 -> 0, 0 -> 1, +1 -> 2.
 *   Tails        [BitVLA s2]: K must be a multiple of 16; N is arbitrary.
 *
 * Readings taken where the pages leave a step open.  The numbers are the
 * same as in the design notes of the repository, which give the reasons;
 * R10 concerns the tests, not this file.
 *   R1  "round" is round-half-to-even, for weights and activations.
 *   R2  mean|W| is an fp64 sum of |W| over k ascending within a row, then
 *       over the tensor's rows ascending, one fp64 division by rows*K, then
 *       rounding to fp32.  (For bf16 weights of the workloads' magnitudes
 *       every partial sum is exact in fp64, so this is the correctly rounded
 *       fp32 value of the exact mean.)
 *   R3  s = 1/mean is an fp32 division; the code uses the fp32 product W*s.
 *   R4  ActQuant uses one fp32 factor sa = 127/amax, then the fp32 product
 *       x*sa; a_scale = amax/127 (fp32 division).
 *   R5  A token with amax == 0 gets q = 0 and a_scale = 0; so does a token
 *       whose scale 127/amax is not a finite fp32 (amax < 127/FLT_MAX, about
 *       2^-121), for which R4's factor cannot be formed.
 *   R6  A fused weight (q|k|v, gate|up) keeps one scale per source tensor
 *       ("segment"); w_scale[n] is the scale of row n's segment.
 *   R7  Where W*s is NaN (only 0 * inf, i.e. a zero weight in a tensor whose
 *       mean rounded to 0) the code is 0.
 *   R8  Epilogue: f = a_scale[m] * w_scale[n] in fp32, then y = (float)acc * f
 *       in fp32; a bf16 output is y rounded to nearest-even.
 *   R9  The activation clamp is [-128, 127] as written; it never binds, since
 *       the largest element maps to exactly +-127.
 *   R11 K must be a multiple of 16; rows are padded to Kp (R12) with weight-0
 *       codes; N is arbitrary, with no padding rows.
 *   R12 Storage layout ("layout v1", this library's own, not I2_S):
 *       Kp = K rounded up to a multiple of 128; row n occupies Kp/4 bytes;
 *       element k of a row is in byte 4*(k/16) + (k%4), bits
 *       2*((k%16)/4) .. +1; positions k >= K hold code 1 (weight 0).
 *
 * The step before the path [Guide s3.1 "Background"; s3.1 key parameters,
 * rms_norm_eps]: every projection normalises its input first,
 * y = ActQuant(RMSNorm(x, g)) with a per-projection weight g [K] and eps; for
 * the down projection the input is the gated product silu(gate) * up [Guide
 * s2, model table: SiLU activation].
 *   R13 RMSNorm(x, g)_k = x_k * g_k * r with r = 1/sqrt(mean_k(x_k^2) + eps)
 *       (the plain reading; no rounding of the normalised vector to bf16).
 *       r > 0 is one factor for the whole token, and ActQuant's codes do not
 *       change when a token is scaled by a positive factor, so the codes are
 *       taken from z = x*g (fp32 products, R4 on z) and r enters a_scale
 *       only: a_scale = amax(z) * r / 127, evaluated in fp64 with the sum of
 *       squares in fp64 (k ascending) and rounded once to fp32.
 *   R14 silu(a) * u is the definition a / (1 + exp(-a)) * u evaluated in
 *       fp64 (the C library's exp) and rounded once to fp32; that fp32 value
 *       is the input of R13.
 *
 * The I2_S interchange format [Guide s3.3 "I2_S Ternary Packing"]: the
 * tensor's values, flattened row-major, form blocks of 128; a block is 32
 * bytes; byte = (c0 << 6) | (c1 << 4) | (c2 << 2) | c3 with the stored codes
 * -1 -> 0, 0 -> 1, +1 -> 2; the fp32 scale 1/mean|W| follows the codes.
 *   R15 Which four values of a block share a byte is not stated.  Reading
 *       "strided" (the default): byte j of a block holds values j, j+32,
 *       j+64, j+96 as c0..c3 -- a block size only matters to a layout of
 *       this kind.  Reading "consecutive": byte j holds values 4j..4j+3.
 *       Both are provided.
 *   R16 The appended float is the quantisation scale s = 1/mean|W| as the
 *       page names it; the dequantisation factor is 1/s.
 *
 * The W1.58A16 variant [BitVLA s5 "On-device gotchas": where the in-graph
 * 8-bit activation quantiser stalled the GPU, the path kept the activations
 * in 16-bit and quantised only the weights]:
 *   R17 y[m][n] = w_scale[n] * sum_k x[m][k] * t[n][k] with the activations
 *       as given (bf16 or fp16, the two 16-bit formats the path may keep;
 *       both widen to fp32 exactly); the oracle evaluates it in fp64 (each product exact, one
 *       rounding per addition, k ascending) -- the reference value that a
 *       kernel summing in fp32, in its own order, is held to within a bound.
 *
 * Per-block weight scales [BitVLA s2: the sibling matvec kernel it grew from
 * keeps one scale per 256-weight block where BitNet keeps one per tensor,
 * i.e. a scale matrix of N x K/256 instead of N x 1]:
 *   R18 Blocks run along k within a row: block b of row n holds
 *       k = 256b .. min(256b + 256, K) - 1, nb = ceil(K / 256) blocks per
 *       row, the last one partial when 256 does not divide K.  Its scale is
 *       the absmean of its own weights, R2 restricted to the block: fp64 sum
 *       of |W| over its k ascending, one fp64 division by the number of
 *       weights in the block, rounding to fp32.  Codes follow R1, R3, R7 with
 *       the block's s = 1/mean.  Scales are stored block-major,
 *       block_scale[b][n].
 *   R19 y[m][n] = a_scale[m] * sum_b acc_b[m][n] * block_scale[b][n] with the
 *       exact int32 block sums acc_b = sum_{k in block b} q*t, evaluated in
 *       fp32 in this order: total = 0; for b ascending,
 *       total = total + (float)acc_b * block_scale[b][n]; y = total * a_scale.
 *
 * Everything here is a direct loop over the definition.  No blocking, no
 * fusion, no intrinsics.
 */
#include <float.h>
#include <math.h>
#include <stdint.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

enum { ORC_F32 = 0, ORC_BF16 = 1, ORC_F16 = 2 };

/* ---------------------------------------------------------------- scalars */

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
float orc_bf16_to_f32(uint16_t h)
{
    uint32_t bits = (uint32_t)h << 16;
    float f;
    memcpy(&f, &bits, sizeof f);
    return f;
}

/* IEEE binary16 -> fp32, exact: 1 sign bit, 5 exponent bits (bias 15), 10
 * fraction bits; exponent 0 holds zero and the subnormals f * 2^-24,
 * exponent 31 infinities (f = 0) and NaNs. */
float orc_f16_to_f32(uint16_t h)
{
    int sign = h >> 15, e = (h >> 10) & 0x1F, f = h & 0x3FF;
    float v;
    if (e == 0)
        v = ldexpf((float)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexpf((float)(1024 + f), e - 25);
    return sign ? -v : v;
}

/* fp32 -> bf16, round to nearest, ties to even; NaN stays a (quiet) NaN. */
uint16_t orc_f32_to_bf16(float f)
{
    uint32_t bits;
    memcpy(&bits, &f, sizeof bits);
    if (isnan(f))
        return (uint16_t)((bits >> 16) | 0x0040u);
    uint32_t upper = bits >> 16;        /* truncated candidate               */
    uint32_t rest = bits & 0xFFFFu;     /* the part that is dropped          */
    if (rest > 0x8000u)
        upper += 1;                     /* more than half: round up          */
    else if (rest == 0x8000u && (upper & 1u))
        upper += 1;                     /* exactly half: round to even       */
    return (uint16_t)upper;             /* carry into the exponent is right: */
                                        /* it yields the next binade or inf  */
}

/* The same rounding for n values. */
void orc_f32_to_bf16_array(const float* f, int64_t n, uint16_t* out)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = orc_f32_to_bf16(f[i]);
}

static float load_elem(const void* base, int dtype, int64_t idx)
{
    if (dtype == ORC_BF16)
        return orc_bf16_to_f32(((const uint16_t*)base)[idx]);
    if (dtype == ORC_F16)
        return orc_f16_to_f32(((const uint16_t*)base)[idx]);
    return ((const float*)base)[idx];
}

/* round half to even in the current (default: nearest-even) mode, R1 */
static float round_half_even(float v)
{
    return nearbyintf(v);
}

int64_t orc_padded_k(int64_t K)
{
    if (K <= 0 || K % 16 != 0)
        return -1;
    return (K + 127) / 128 * 128;
}

/* ------------------------------------------------------------ WeightQuant */

/* Sum of |W[n, k]| for k = 0..K-1, ascending, in fp64 (R2). */
double orc_row_abs_sum(const void* W, int dtype, int64_t n, int64_t K, int64_t ldw)
{
    double s = 0.0;
    for (int64_t k = 0; k < K; ++k)
        s += fabs((double)load_elem(W, dtype, n * ldw + k));
    return s;
}

/* mean|W| of rows [row0, row0 + rows): row sums added in row order (R2). */
float orc_segment_mean(const void* W, int dtype, int64_t row0, int64_t rows,
                       int64_t K, int64_t ldw)
{
    double total = 0.0;
    for (int64_t n = row0; n < row0 + rows; ++n)
        total += orc_row_abs_sum(W, dtype, n, K, ldw);
    return (float)(total / (double)(rows * K));
}

/* Ternary code of one weight given the tensor's fp32 factor s (R1, R3, R7). */
int8_t orc_ternary(float w, float s)
{
    float p = w * s;
    if (isnan(p))
        return 0;
    float r = round_half_even(p);
    if (r > 1.0f)
        r = 1.0f;
    if (r < -1.0f)
        r = -1.0f;
    return (int8_t)r;
}

/*
 * WeightQuant of an [N, K] tensor made of n_segs source tensors stacked by
 * rows (seg_rows[i] rows each; n_segs == 0 means one tensor of N rows).
 * Outputs: t [N][K] codes in {-1,0,1}; w_scale [N]; seg_mean [n_segs or 1];
 * zero_count [n_segs or 1] = number of zero codes among the real K columns.
 * Returns 0, or -1 if the segment rows do not add up to N, or -2 if a weight
 * is not finite.
 */
int orc_weight_quant(const void* W, int dtype, int64_t N, int64_t K, int64_t ldw,
                     const int64_t* seg_rows, int32_t n_segs,
                     int8_t* t, float* w_scale, float* seg_mean, int64_t* zero_count)
{
    int64_t one = N;
    if (n_segs <= 0) {
        seg_rows = &one;
        n_segs = 1;
    }
    int64_t total = 0;
    for (int32_t i = 0; i < n_segs; ++i)
        total += seg_rows[i];
    if (total != N)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            if (!isfinite(load_elem(W, dtype, n * ldw + k)))
                return -2;

    int64_t row0 = 0;
    for (int32_t i = 0; i < n_segs; ++i) {
        float mean = orc_segment_mean(W, dtype, row0, seg_rows[i], K, ldw);
        float s = 1.0f / mean;
        int64_t zeros = 0;
        for (int64_t n = row0; n < row0 + seg_rows[i]; ++n) {
            w_scale[n] = mean;
            for (int64_t k = 0; k < K; ++k) {
                int8_t c = orc_ternary(load_elem(W, dtype, n * ldw + k), s);
                t[n * K + k] = c;
                zeros += (c == 0);
            }
        }
        if (seg_mean)
            seg_mean[i] = mean;
        if (zero_count)
            zero_count[i] = zeros;
        row0 += seg_rows[i];
    }
    return 0;
}

/* ------------------------------------------------------------- layout v1 */

/* Byte index and bit offset of element k inside a row (R12). */
static int64_t v1_byte(int64_t k) { return 4 * (k / 16) + (k % 4); }
static int v1_shift(int64_t k) { return (int)(2 * ((k % 16) / 4)); }

/* Pack codes t [N][K] into packed [N][Kp/4]; stored code u = t + 1. */
int orc_pack(const int8_t* t, int64_t N, int64_t K, uint8_t* packed)
{
    int64_t Kp = orc_padded_k(K);
    if (Kp < 0)
        return -1;
    int64_t row_bytes = Kp / 4;
    memset(packed, 0, (size_t)(N * row_bytes));
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < Kp; ++k) {
            unsigned u = (k < K) ? (unsigned)(t[n * K + k] + 1) : 1u;
            packed[n * row_bytes + v1_byte(k)] |= (uint8_t)(u << v1_shift(k));
        }
    }
    return 0;
}

/* Inverse of orc_pack over the real columns.  Returns -1 on a bad K, or the
 * number of 2-bit fields that hold the unused value 3 (0 for a valid buffer). */
int64_t orc_unpack(const uint8_t* packed, int64_t N, int64_t K, int8_t* t)
{
    int64_t Kp = orc_padded_k(K);
    if (Kp < 0)
        return -1;
    int64_t row_bytes = Kp / 4, bad = 0;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t k = 0; k < K; ++k) {
            unsigned u = (packed[n * row_bytes + v1_byte(k)] >> v1_shift(k)) & 3u;
            bad += (u == 3u);
            t[n * K + k] = (int8_t)((int)u - 1);
        }
    }
    return bad;
}

/* ----------------------------------------------------------------- I2_S */

/* Byte index inside a block and shift of value v (0..127) of the block (R15). */
static int64_t i2s_byte(int64_t v, int consecutive) { return consecutive ? v / 4 : v % 32; }
static int i2s_shift(int64_t v, int consecutive) { return consecutive ? 6 - 2 * (int)(v % 4) : 6 - 2 * (int)(v / 32); }

/*
 * Codes t [N, K] (-1, 0, +1) and the scale s = 1/mean|W| as an I2_S buffer:
 * N*K/4 code bytes, then s as 4 little-endian bytes (R15, R16).  N*K must be
 * a multiple of 128.  Returns -1 otherwise.
 */
int orc_i2s_pack(const int8_t* t, int64_t N, int64_t K, float s, int consecutive, uint8_t* out)
{
    int64_t total = N * K;
    if (total <= 0 || total % 128 != 0)
        return -1;
    memset(out, 0, (size_t)(total / 4));
    for (int64_t i = 0; i < total; ++i) {
        int64_t block = i / 128, v = i % 128;
        unsigned c = (unsigned)(t[i] + 1);
        out[block * 32 + i2s_byte(v, consecutive)] |= (uint8_t)(c << i2s_shift(v, consecutive));
    }
    memcpy(out + total / 4, &s, sizeof s);
    return 0;
}

/* Inverse of orc_i2s_pack: codes t [N, K] and *s.  Returns -1 for a bad size,
 * else the number of fields holding the unused value 3. */
int64_t orc_i2s_unpack(const uint8_t* in, int64_t N, int64_t K, int consecutive, int8_t* t, float* s)
{
    int64_t total = N * K, bad = 0;
    if (total <= 0 || total % 128 != 0)
        return -1;
    for (int64_t i = 0; i < total; ++i) {
        int64_t block = i / 128, v = i % 128;
        unsigned c = (in[block * 32 + i2s_byte(v, consecutive)] >> i2s_shift(v, consecutive)) & 3u;
        bad += (c == 3u);
        t[i] = (int8_t)((int)c - 1);
    }
    memcpy(s, in + total / 4, sizeof *s);
    return bad;
}

/* -------------------------------------------------------------- ActQuant */

/*
 * Per-token ActQuant of x [M, K] (row stride ldx, fp32 or bf16).
 * q [M][Kp]: int8 codes, columns K..Kp-1 set to 0.  a_scale [M] = amax/127.
 * q_rowsum [M] = sum of q over the row.  (R1, R4, R5, R9.)
 */
int orc_act_quant(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx,
                  int8_t* q, float* a_scale, int32_t* q_rowsum)
{
    int64_t Kp = orc_padded_k(K);
    if (Kp < 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        float amax = 0.0f;
        for (int64_t k = 0; k < K; ++k) {
            float a = fabsf(load_elem(x, dtype, m * ldx + k));
            if (a > amax)
                amax = a;
        }
        int64_t sum = 0;
        float sa = 127.0f / amax;                  /* +inf for amax == 0 */
        if (!(sa <= FLT_MAX)) {                    /* R5 */
            for (int64_t k = 0; k < Kp; ++k)
                q[m * Kp + k] = 0;
            a_scale[m] = 0.0f;
        } else {
            for (int64_t k = 0; k < K; ++k) {
                float r = round_half_even(load_elem(x, dtype, m * ldx + k) * sa);
                if (r > 127.0f)
                    r = 127.0f;
                if (r < -128.0f)
                    r = -128.0f;
                q[m * Kp + k] = (int8_t)r;
                sum += (int8_t)r;
            }
            for (int64_t k = K; k < Kp; ++k)
                q[m * Kp + k] = 0;
            a_scale[m] = amax / 127.0f;
        }
        q_rowsum[m] = (int32_t)sum;
    }
    return 0;
}

/* ------------------------------------------------- RMSNorm -> ActQuant */

/*
 * q, a_scale and q_rowsum of ActQuant(RMSNorm(x, g)) for M tokens of K (R13):
 * codes of z = x*g exactly as orc_act_quant, a_scale = amax(z) * r / 127 with
 * r = 1/sqrt(sum_k x_k^2 / K + eps) in fp64.  x and g are bf16 or fp32; g has
 * K entries.  Returns -1 for a bad K.
 */
int orc_rms_act_quant(const void* x, int x_dtype, const void* g, int g_dtype, int64_t M, int64_t K,
                      int64_t ldx, float eps, int8_t* q, float* a_scale, int32_t* q_rowsum)
{
    int64_t Kp = orc_padded_k(K);
    if (Kp < 0)
        return -1;
    for (int64_t m = 0; m < M; ++m) {
        /* z = x * g, one fp32 product per element */
        float amax = 0.0f;
        double squares = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            float xv = load_elem(x, x_dtype, m * ldx + k);
            float z = xv * load_elem(g, g_dtype, k);
            float a = fabsf(z);
            if (a > amax)
                amax = a;
            squares += (double)xv * (double)xv;
        }
        double r = 1.0 / sqrt(squares / (double)K + (double)eps);
        int64_t sum = 0;
        memset(&q[m * Kp], 0, (size_t)Kp);         /* zero token and the tail k >= K */
        float sa = 127.0f / amax;                  /* +inf for amax == 0 */
        if (!(sa <= FLT_MAX)) {                    /* R5 */
            a_scale[m] = 0.0f;
        } else {
            for (int64_t k = 0; k < K; ++k) {
                float z = load_elem(x, x_dtype, m * ldx + k) * load_elem(g, g_dtype, k);
                float c = round_half_even(z * sa);
                if (c > 127.0f)
                    c = 127.0f;
                if (c < -128.0f)
                    c = -128.0f;
                q[m * Kp + k] = (int8_t)c;
                sum += (int8_t)c;
            }
            a_scale[m] = (float)((double)amax * r / 127.0);
        }
        q_rowsum[m] = (int32_t)sum;
    }
    return 0;
}

/* h = silu(gate) * up per element (R14): the definition in fp64, one
 * rounding to fp32; out [M][K] (row stride K). */
void orc_swiglu(const void* gate, const void* up, int dtype, int64_t M, int64_t K, int64_t ld, float* h)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t k = 0; k < K; ++k) {
            double a = (double)load_elem(gate, dtype, m * ld + k);
            double u = (double)load_elem(up, dtype, m * ld + k);
            h[m * K + k] = (float)(a / (1.0 + exp(-a)) * u);
        }
}

/* ------------------------------------------------------------- W1.58A16 */

/*
 * y [M][N] fp64 = w_scale[n] * sum_{k<K} x[m][k] * t[n][k] (R17); also the
 * magnitude sum_k |x[m][k] * t[n][k]| into mag [M][N] (for error bounds).
 * x is bf16 or fp32 with row stride ldx; t has row stride K.
 */
void orc_linear_a16(const void* x, int dtype, int64_t M, int64_t K, int64_t ldx, const int8_t* t, int64_t N,
                    const float* w_scale, double* y, double* mag)
{
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double s = 0.0, a = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = (double)load_elem(x, dtype, m * ldx + k) * (double)t[n * K + k];
                s += p;
                a += fabs(p);
            }
            y[m * N + n] = s * (double)w_scale[n];
            mag[m * N + n] = a;
        }
}

/* ----------------------------------------------------------- integer dot */

/*
 * acc[m][n] = sum_{k<K} q[m][k] * t[n][k], summed in int64 and stored as
 * int32.  q has row stride Kp, t has row stride K.  Rows n are split over
 * nthreads threads (results do not depend on it).  Returns -1 if a sum does
 * not fit in int32.
 */
int orc_int_dot(const int8_t* q, int64_t M, int64_t K, const int8_t* t, int64_t N,
                int32_t* acc, int nthreads)
{
    int64_t Kp = orc_padded_k(K);
    if (Kp < 0)
        return -1;
    int overflow = 0;
    if (nthreads < 1)
        nthreads = 1;
#pragma omp parallel for num_threads(nthreads) schedule(static) reduction(| : overflow)
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t m = 0; m < M; ++m) {
            int64_t s = 0;
            for (int64_t k = 0; k < K; ++k)
                s += (int64_t)q[m * Kp + k] * (int64_t)t[n * K + k];
            if (s > INT32_MAX || s < INT32_MIN)
                overflow = 1;
            acc[m * N + n] = (int32_t)s;
        }
    }
    return overflow ? -1 : 0;
}

/* The same sum for a list of (m, n) pairs only. */
int orc_int_dot_pairs(const int8_t* q, int64_t K, const int8_t* t,
                      int64_t n_pairs, const int64_t* m_idx, const int64_t* n_idx,
                      int32_t* acc)
{
    int64_t Kp = orc_padded_k(K);
    if (Kp < 0)
        return -1;
    for (int64_t i = 0; i < n_pairs; ++i) {
        int64_t s = 0;
        for (int64_t k = 0; k < K; ++k)
            s += (int64_t)q[m_idx[i] * Kp + k] * (int64_t)t[n_idx[i] * K + k];
        acc[i] = (int32_t)s;
    }
    return 0;
}

/* -------------------------------------------------------------- epilogue */

/* y[m][n] = (float)acc[m][n] * (a_scale[m] * w_scale[n]), all fp32 (R8). */
float orc_dequant_one(int32_t acc, float a_scale, float w_scale)
{
    float f = a_scale * w_scale;
    return (float)acc * f;
}

void orc_epilogue(const int32_t* acc, int64_t M, int64_t N, const float* a_scale,
                  const float* w_scale, int out_dtype, void* y, int64_t ldy)
{
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float v = orc_dequant_one(acc[m * N + n], a_scale[m], w_scale[n]);
            if (out_dtype == ORC_BF16)
                ((uint16_t*)y)[m * ldy + n] = orc_f32_to_bf16(v);
            else
                ((float*)y)[m * ldy + n] = v;
        }
    }
}

int orc_max_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* ------------------------------------------------ per-block weight scales */

/* Blocks of 256 weights per row (R18); -1 for a bad K. */
int64_t orc_block_count(int64_t K)
{
    if (K <= 0 || K % 16 != 0)
        return -1;
    return (K + 255) / 256;
}

/*
 * WeightQuant with one scale per 256-weight block of a row (R18): codes
 * t [N][K] and block_scale [nb][N].  Returns 0, -1 for a bad K, -2 if a
 * weight is not finite.
 */
int orc_weight_quant_blocked(const void* W, int dtype, int64_t N, int64_t K, int64_t ldw,
                             int8_t* t, float* block_scale)
{
    int64_t nb = orc_block_count(K);
    if (nb < 0)
        return -1;
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k)
            if (!isfinite(load_elem(W, dtype, n * ldw + k)))
                return -2;
    for (int64_t n = 0; n < N; ++n) {
        for (int64_t b = 0; b < nb; ++b) {
            int64_t k0 = 256 * b, k1 = (k0 + 256 < K) ? k0 + 256 : K;
            double sum = 0.0;
            for (int64_t k = k0; k < k1; ++k)
                sum += fabs((double)load_elem(W, dtype, n * ldw + k));
            float mean = (float)(sum / (double)(k1 - k0));
            float s = 1.0f / mean;
            block_scale[b * N + n] = mean;
            for (int64_t k = k0; k < k1; ++k)
                t[n * K + k] = orc_ternary(load_elem(W, dtype, n * ldw + k), s);
        }
    }
    return 0;
}

/*
 * Linear with block scales (R19): y [M][N] fp32 from q [M][Kp] (ActQuant
 * output), a_scale [M], codes t [N][K] and block_scale [nb][N].  acc_blocks
 * [M][nb][N] (or NULL) receives the exact block sums.  Returns -1 for a bad K.
 */
int orc_linear_blocked(const int8_t* q, const float* a_scale, int64_t M, int64_t K, const int8_t* t,
                       const float* block_scale, int64_t N, float* y, int32_t* acc_blocks)
{
    int64_t Kp = orc_padded_k(K), nb = orc_block_count(K);
    if (Kp < 0)
        return -1;
#pragma omp parallel for schedule(static)
    for (int64_t m = 0; m < M; ++m) {
        for (int64_t n = 0; n < N; ++n) {
            float total = 0.0f;
            for (int64_t b = 0; b < nb; ++b) {
                int64_t k0 = 256 * b, k1 = (k0 + 256 < K) ? k0 + 256 : K;
                int64_t s = 0;
                for (int64_t k = k0; k < k1; ++k)
                    s += (int64_t)t[n * K + k] * (int64_t)q[m * Kp + k];
                if (acc_blocks)
                    acc_blocks[(m * nb + b) * N + n] = (int32_t)s;
                float term = (float)s * block_scale[b * N + n];
                total = total + term;
            }
            y[m * N + n] = total * a_scale[m];
        }
    }
    return 0;
}
