/*
 * bitnet.h -- C ABI of libbitnet_hip.so, a W1.58A8 BitLinear for MI355X (gfx950).
 *
 *   y = linear(ActQuant(x), WeightQuant(W)),  no bias.
 *
 * Pages cited (title, then section):
 *   [BitVLA] "BitVLA -- 1.58-bit Vision-Language-Action on Core AI"
 *            (Core AI model zoo).
 *   [Guide]  "BitNet-Embeddings-0.6B/270M: I2_S Conversion and Inference
 *            Optimization Guide" (microsoft/BitNet docs).
 *
 * Method.  WeightQuant is per-tensor absmean: s = 1/mean|W|, ternary codes
 * t = clamp(round(W*s), -1, 1), dequantised as t/s [BitVLA s1; Guide s2,
 * s3.3 "I2_S Ternary Packing"].  ActQuant is per-token absmax int8:
 * q = clamp(round(x*127/max|x|), -128, 127), dequantised by 127/max|x|
 * [BitVLA s1; Guide s2].  The product is an exact int32 sum of q*t, rescaled by
 * (max|x|/127) * mean|W|.  ActQuant runs before the ternary product and the
 * codes are built from the bf16 latent weights [BitVLA s2].
 *
 * Numerics fixed by this library where the pages leave them open:
 *   - "round" is round-half-to-even (weights and activations);
 *   - mean|W| = fp64 sum over k ascending per row, rows ascending, one fp64
 *     division by rows*K, rounded to fp32; s = 1.0f/mean (fp32 division);
 *     t = clamp(rne(fp32(W*s)), -1, 1), and t = 0 where W*s is NaN;
 *   - sa = 127.0f/amax (fp32), q = clamp(rne(fp32(x*sa)), -128, 127),
 *     a_scale = amax/127.0f; a token with amax == 0 gets q = 0, a_scale = 0;
 *   - y = (float)acc * (a_scale[m] * w_scale[n]) in fp32; bf16 output is that
 *     value rounded to nearest-even.
 * Every integer result (codes, packed bytes, q, q_rowsum, acc) is exact and
 * independent of launch configuration.
 *
 * Packed weight layout v1 (this library's own; not I2_S).  Stored code
 * u = t + 1, so -1 -> 0, 0 -> 1, +1 -> 2 [Guide s3.3; BitVLA s2].  Rows are
 * padded to Kp = bitnet_padded_k(K) elements.  Row n occupies Kp/4 bytes at
 * offset n*Kp/4.  Element k of a row lives in byte 4*(k/16) + k%4 at bits
 * 2*((k%16)/4)..+1; equivalently, little-endian 32-bit word j holds elements
 * 16j..16j+15 and (word >> 2p) & 0x03030303 gives elements 16j+4p+0..3 in its
 * four bytes.  Elements K..Kp-1 hold code 1 (weight 0).  There are no padding
 * rows: N is arbitrary [BitVLA s2 asks for arbitrary N and K % 16 == 0].
 * w_scale[n] (fp32) is mean|W| of the source tensor that row n belongs to, one
 * value per output row, a 1-D array of N floats [BitVLA s2: per-tensor scale
 * stored per row].
 *
 * Conventions for every entry point:
 *   - Sizes are element counts; M, N, K > 0; K % 16 == 0; K <= 1048576;
 *     M, N <= 2^31 - 1.  Leading dimensions (ld*) are in elements.
 *   - The caller owns and allocates every buffer.  Device pointers are HIP
 *     device memory on the current device; the library allocates no memory
 *     that outlives a call (bitnet_pack_weights with BITNET_MEM_DEVICE uses
 *     stream-ordered temporaries of O(N) bytes that it frees before
 *     returning).
 *   - Device work is enqueued on `stream` (0 = the null stream) and is
 *     asynchronous unless stated otherwise.
 *   - Every argument check runs before any launch; a failed check launches
 *     nothing and returns BITNET_ERR_INVALID_ARG (detail in
 *     bitnet_last_error()).  A failed launch returns BITNET_ERR_HIP.
 *   - Pointers named "16-byte aligned" must be; strides keep rows aligned
 *     because Kp is a multiple of 128.
 *   - No exceptions and no printing cross this boundary; all functions are
 *     reentrant.  Calls that overlap on one stream are ordered by the stream.
 */
#ifndef BITNET_H
#define BITNET_H

#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BITNET_ABI_VERSION 1

typedef enum {
    BITNET_OK = 0,
    BITNET_ERR_INVALID_ARG = 1,  /* bad size, stride, pointer, alignment or dtype */
    BITNET_ERR_UNSUPPORTED = 2,  /* valid request this build does not handle      */
    BITNET_ERR_HIP = 3,          /* a HIP runtime call or kernel launch failed     */
    BITNET_ERR_NONFINITE = 4     /* a weight given to the packer is inf or NaN     */
} bitnet_status_t;

/* The last two enumerators of each input enum give it the range of int32, so
 * that a caller's out-of-range value is a checked argument error rather than
 * undefined behaviour in the library (they are not valid arguments). */
typedef enum {
    BITNET_F32 = 0,
    BITNET_BF16 = 1,
    BITNET_F16 = 2,              /* IEEE binary16: W1.58A16 activations only */
    BITNET_DTYPE_RANGE_MIN_ = -0x7FFFFFFF - 1,
    BITNET_DTYPE_RANGE_MAX_ = 0x7FFFFFFF
} bitnet_dtype_t;

typedef enum {
    BITNET_MEM_HOST = 0,
    BITNET_MEM_DEVICE = 1,
    BITNET_MEM_RANGE_MIN_ = -0x7FFFFFFF - 1,
    BITNET_MEM_RANGE_MAX_ = 0x7FFFFFFF
} bitnet_mem_t;

/* ABI version of the loaded library (BITNET_ABI_VERSION). */
int32_t bitnet_abi_version(void);

/* Padded row length Kp = K rounded up to a multiple of 128; -1 if K <= 0,
 * K % 16 != 0 or K is above the limit. */
int64_t bitnet_padded_k(int64_t K);

/* Bytes of a packed [N, K] weight: N * Kp / 4; -1 on a bad N or K. */
int64_t bitnet_packed_bytes(int64_t N, int64_t K);

/*
 * WeightQuant + pack [BitVLA s1, s2; Guide s3.3 "I2_S Ternary Packing"].
 *
 * W        [N, K] latent weights, row stride ldw >= K, dtype w_dtype
 *          (BITNET_BF16 or BITNET_F32).  Host memory if where == HOST,
 *          device memory if where == DEVICE.
 * seg_rows host array of n_segs row counts summing to N: the fused weight is
 *          n_segs source tensors stacked by rows (e.g. q|k|v), each with its
 *          own mean|W|.  seg_rows == NULL or n_segs == 0 means one tensor.
 * packed   out, [N][Kp/4] bytes in layout v1, same memory kind as W,
 *          16-byte aligned.
 * w_scale  out, [N] fp32, same memory kind as W.
 * seg_mean out, optional host array [max(n_segs,1)]: mean|W| per segment.
 * zero_count out, optional host array [max(n_segs,1)]: zero codes per
 *          segment over the real K columns (the zero-weight fraction).
 * stream   used for DEVICE only.  A DEVICE call is synchronous: it waits for
 *          its own work on `stream` before returning (it must read back the
 *          non-finite flag), and it needs O(N) bytes of temporary device
 *          memory, taken and returned on `stream`.
 * Errors:  INVALID_ARG for bad sizes/pointers/segments; NONFINITE if any
 *          weight is inf or NaN (outputs are then unspecified); HIP.
 */
bitnet_status_t bitnet_pack_weights(bitnet_mem_t where, hipStream_t stream,
                                    const void* W, bitnet_dtype_t w_dtype,
                                    int64_t N, int64_t K, int64_t ldw,
                                    const int64_t* seg_rows, int32_t n_segs,
                                    uint8_t* packed, float* w_scale,
                                    float* seg_mean, int64_t* zero_count);

/*
 * bitnet_pack_weights for device memory, for callers that cannot allocate
 * device memory (code that must not call hipMalloc: serving loops, harnesses
 * that forbid it).  Same arguments, results and errors as
 * bitnet_pack_weights(BITNET_MEM_DEVICE, ...), but its temporaries (the fp64
 * row sums and the per-segment fields) live in a fixed device array of the
 * library, about 1 MiB, held on each GPU the library runs on until the
 * process ends.  It allocates nothing and is synchronous on `stream` like the
 * device pack.  Limits: N <= BITNET_PACK_STATIC_MAX_ROWS and at most
 * BITNET_PACK_STATIC_MAX_SEGS segments; larger requests return
 * BITNET_ERR_UNSUPPORTED before any launch.  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (from several host threads or
 * streams) race and must be serialised by the caller.
 */
#define BITNET_PACK_STATIC_MAX_ROWS 131072
#define BITNET_PACK_STATIC_MAX_SEGS 64
bitnet_status_t bitnet_pack_weights_static(hipStream_t stream, const void* W, bitnet_dtype_t w_dtype,
                                           int64_t N, int64_t K, int64_t ldw,
                                           const int64_t* seg_rows, int32_t n_segs,
                                           uint8_t* packed, float* w_scale,
                                           float* seg_mean, int64_t* zero_count);

/*
 * ActQuant, per token [BitVLA s1; Guide s2].  Device memory throughout.
 *
 * x        [M, K] activations, row stride ldx >= K, dtype x_dtype (BF16 or
 *          F32).  Non-finite activations give unspecified results.
 * q        out, [M][Kp] int8, 16-byte aligned; columns K..Kp-1 are written 0.
 * a_scale  out, [M] fp32 = amax/127 (0 for an all-zero token).
 * q_rowsum out, [M] int32 = sum over k of q[m][k].
 */
bitnet_status_t bitnet_act_quant(hipStream_t stream, const void* x, bitnet_dtype_t x_dtype,
                                 int64_t M, int64_t K, int64_t ldx,
                                 int8_t* q, float* a_scale, int32_t* q_rowsum);

/*
 * ActQuant of the normalised input of a projection [Guide s3.1: every
 * projection applies RMSNorm with its own weight and rms_norm_eps (1e-6 in
 * the guide's models) before ActQuant; Guide s2: SiLU gating before the down
 * projection].  Device memory throughout; results as bitnet_act_quant's.
 *
 * x        [M, K], row stride ldx >= K, dtype x_dtype (BF16 or F32).
 * up       NULL, or [M, K] with x's dtype and row stride: the input is then
 *          h = silu(x) * up (x being the gate) = x * sigmoid(x) * up in
 *          fp32, with e = exp(-|x|) (t * log2(e) split into two fp32 parts,
 *          the hardware exp2 of the fraction, a scaling by 2^n) and
 *          sigmoid(x) = rcp(1 + e) for x >= 0, e * rcp(1 + e) below: h within
 *          4.3 fp32 ulps of the exact silu(x) * up for |x| <= 87, so int8
 *          codes whose unrounded value lies within 2e-4 of a .5 tie may
 *          differ by one from those of the exact h.
 * norm_w   [K] RMSNorm weight g, dtype norm_dtype (BF16 or F32).
 * eps      finite, >= 0.
 * RMSNorm(h)_k = h_k * g_k * r with r = 1/sqrt(mean_k(h_k^2) + eps).  r is
 * one positive factor per token, so the int8 codes are those of z = h * g
 * (fp32 products, then ActQuant exactly as bitnet_act_quant) and
 * a_scale = amax(z) * r / 127, with the sum of squares and r in fp64 and one
 * rounding to fp32 at the end (0 for a token whose z is all zero).
 */
bitnet_status_t bitnet_rmsnorm_act_quant(hipStream_t stream, const void* x, const void* up,
                                         bitnet_dtype_t x_dtype, int64_t M, int64_t K, int64_t ldx,
                                         const void* norm_w, bitnet_dtype_t norm_dtype, float eps,
                                         int8_t* q, float* a_scale, int32_t* q_rowsum);

/*
 * Ternary linear on quantised operands + dequant epilogue [BitVLA s1, s2;
 * Guide s2 (no bias)].  Device memory throughout.
 *
 * q, a_scale, q_rowsum  as produced by bitnet_act_quant for [M, K].
 * packed, w_scale       as produced by bitnet_pack_weights for [N, K].
 * y        out, [M, N] with row stride ldy >= N, dtype y_dtype (F32 or BF16):
 *          y[m][n] = (float)acc[m][n] * (a_scale[m] * w_scale[n]),
 *          acc[m][n] = sum_{k<K} q[m][k] * t[n][k] (exact int32).
 * acc_debug optional out, [M][N] int32 (row stride N): the exact acc.
 * M <= 16 runs the streaming decode kernel (one pass over the packed weight);
 * larger M runs the int8-MFMA GEMM.  Both give identical bits.
 */
bitnet_status_t bitnet_linear_forward(hipStream_t stream,
                                      const int8_t* q, const float* a_scale,
                                      const int32_t* q_rowsum, int64_t M, int64_t K,
                                      const uint8_t* packed, const float* w_scale, int64_t N,
                                      void* y, bitnet_dtype_t y_dtype, int64_t ldy,
                                      int32_t* acc_debug);

/*
 * Whole BitLinear from activations: bitnet_act_quant then
 * bitnet_linear_forward, enqueued back to back on `stream` [BitVLA s2: the
 * wrapper applies ActQuant before the ternary kernel].  q, a_scale and
 * q_rowsum are caller-provided buffers that receive the quantised activations
 * (same shapes as in bitnet_act_quant).  For M * Kp <= 32768 bytes with
 * 16-byte-aligned x rows this is a single launch: the decode kernel quantises
 * the tokens itself and its first workgroup also stores q, a_scale and
 * q_rowsum; otherwise it is two launches.
 */
bitnet_status_t bitnet_bitlinear_forward(hipStream_t stream,
                                         const void* x, bitnet_dtype_t x_dtype,
                                         int64_t M, int64_t K, int64_t ldx,
                                         const uint8_t* packed, const float* w_scale, int64_t N,
                                         void* y, bitnet_dtype_t y_dtype, int64_t ldy,
                                         int8_t* q, float* a_scale, int32_t* q_rowsum);

/*
 * bitnet_bitlinear_forward with the projection's input norm first:
 * y = linear(ActQuant(RMSNorm(h, norm_w)), WeightQuant(W)) where h = x, or
 * h = silu(x) * up when up is given [Guide s3.1, s2].  x, up, norm_w and eps
 * as in bitnet_rmsnorm_act_quant; every other argument as in
 * bitnet_bitlinear_forward, including the single-launch condition (for the
 * single launch, up and norm_w must also be 16-byte aligned).  q, a_scale
 * and q_rowsum receive bitnet_rmsnorm_act_quant's results.
 */
bitnet_status_t bitnet_rmsnorm_bitlinear_forward(hipStream_t stream,
                                                 const void* x, const void* up, bitnet_dtype_t x_dtype,
                                                 int64_t M, int64_t K, int64_t ldx,
                                                 const void* norm_w, bitnet_dtype_t norm_dtype, float eps,
                                                 const uint8_t* packed, const float* w_scale, int64_t N,
                                                 void* y, bitnet_dtype_t y_dtype, int64_t ldy,
                                                 int8_t* q, float* a_scale, int32_t* q_rowsum);

/*
 * Many independent decode-size BitLinears in one launch.  A decoder streams
 * the weights of many projections per token (one position at a time, M = 1:
 * [BitVLA s3]); each matrix alone moves only a few MB, far too little to
 * amortise a kernel launch, so a caller that holds several independent
 * problems can run them as one grouped launch.  Each item is
 * y_i = linear(ActQuant(x_i), WeightQuant(W_i)) with its own activations,
 * packed weight, scales and output; items may differ in N and K.
 */
typedef struct {
    const void* x;           /* [M, K] activations (device), row stride ldx    */
    int64_t ldx;             /* elements; x and ldx*size keep rows 16-B aligned */
    const uint8_t* packed;   /* [N][Kp/4] layout v1 (device), 16-byte aligned   */
    const float* w_scale;    /* [N] (device)                                    */
    void* y;                 /* [M, N] output (device), row stride ldy          */
    int64_t ldy;
    int64_t N;
    int64_t K;
} bitnet_group_item_t;

/* Host-side handle of a prepared group (contents private to the library). */
typedef struct {
    int64_t opaque[8];
} bitnet_group_plan_t;

/* Device bytes bitnet_group_plan needs for `count` items (-1 if count <= 0). */
int64_t bitnet_group_table_bytes(int32_t count);

/*
 * Validate `count` items (host array) that share M (1..16), the activation
 * dtype and the output dtype, and write their launch table into table_dev
 * (caller-owned device memory of at least bitnet_group_table_bytes(count)
 * bytes, 16-byte aligned).  Fills *plan.  Synchronous (uploads the table on
 * `stream` and waits).  The plan stays valid while table_dev and every buffer
 * the items name stay allocated; their contents may change between launches.
 * Errors: INVALID_ARG for any bad item (its index is in bitnet_last_error());
 * UNSUPPORTED if M * Kp exceeds 65536 bytes for some item; HIP.
 */
bitnet_status_t bitnet_group_plan(hipStream_t stream, const bitnet_group_item_t* items, int32_t count,
                                  int64_t M, bitnet_dtype_t x_dtype, bitnet_dtype_t y_dtype,
                                  void* table_dev, int64_t table_bytes, bitnet_group_plan_t* plan);

/* Input norm of one grouped item (see bitnet_rmsnorm_act_quant): norm_w NULL
 * means none; otherwise norm_w [K] (16-byte aligned), its dtype and eps, and
 * up NULL or [M, K] with the item's x dtype and row stride (16-byte aligned)
 * for the gated input silu(x) * up. */
typedef struct {
    const void* up;
    const void* norm_w;
    bitnet_dtype_t norm_dtype;
    float eps;
} bitnet_group_norm_t;

/* bitnet_group_plan with an input norm per item: norms[i] applies to items[i]
 * (count entries, host memory); the launch then quantises each item's
 * normalised input, with bitnet_rmsnorm_act_quant's results. */
bitnet_status_t bitnet_group_plan_rmsnorm(hipStream_t stream, const bitnet_group_item_t* items,
                                          const bitnet_group_norm_t* norms, int32_t count,
                                          int64_t M, bitnet_dtype_t x_dtype, bitnet_dtype_t y_dtype,
                                          void* table_dev, int64_t table_bytes, bitnet_group_plan_t* plan);

/*
 * W1.58A16 variant of bitnet_group_plan [BitVLA s5: 16-bit activations with
 * the ternary weights]: items as for bitnet_group_plan with bf16 x (M 1..16,
 * 16-byte aligned rows), launched by bitnet_bitlinear_grouped as one
 * streaming launch that computes y_i = w_scale_i * (x_i . t_i) with the sum in
 * fp32 on bf16 matrix cores, as bitnet_linear_a16 does per item (the fp32
 * order differs; both stay within bitnet_linear_a16's bound).  Errors as for
 * bitnet_group_plan, and UNSUPPORTED when one workgroup's share of the group
 * needs more LDS than it has for the bf16 token rows (2 * M * Kp bytes per
 * item it touches); then use bitnet_linear_a16 per item.
 */
bitnet_status_t bitnet_group_plan_a16(hipStream_t stream, const bitnet_group_item_t* items, int32_t count,
                                      int64_t M, bitnet_dtype_t y_dtype, void* table_dev, int64_t table_bytes,
                                      bitnet_group_plan_t* plan);

/* bitnet_group_plan_a16 with fp16 activations x (fp16 matrix cores; the same
 * bound as bitnet_linear_a16). */
bitnet_status_t bitnet_group_plan_a16_fp16(hipStream_t stream, const bitnet_group_item_t* items, int32_t count,
                                           int64_t M, bitnet_dtype_t y_dtype, void* table_dev, int64_t table_bytes,
                                           bitnet_group_plan_t* plan);

/*
 * Grouped decode with per-256-block weight scales [BitVLA s2]: items as for
 * bitnet_group_plan, except that each item's w_scale points to its
 * block_scale [ceil(K/256)][N] from bitnet_pack_weights_blocked (K <= 8192);
 * the launch quantises each item's tokens (as bitnet_act_quant) and computes
 * bitnet_linear_blocked_forward's y for every item, with the same bits.
 * Errors as for bitnet_group_plan; UNSUPPORTED for K > 8192 or when a
 * workgroup's token rows do not fit its LDS share.
 */
bitnet_status_t bitnet_group_plan_blocked(hipStream_t stream, const bitnet_group_item_t* items, int32_t count,
                                          int64_t M, bitnet_dtype_t x_dtype, bitnet_dtype_t y_dtype,
                                          void* table_dev, int64_t table_bytes, bitnet_group_plan_t* plan);

/*
 * Run every item of a plan in one kernel launch on `stream`: each workgroup
 * quantises its item's tokens (ActQuant, same numerics as bitnet_act_quant)
 * and streams its share of that item's packed weight once.  Results are
 * bit-identical to bitnet_bitlinear_forward on each item.  Makes no
 * allocation and no host-device copy, so it can be captured in a HIP graph.
 */
bitnet_status_t bitnet_bitlinear_grouped(hipStream_t stream, const bitnet_group_plan_t* plan);

/* Name of the kernel a plan launches: "stream" (each workgroup streams a
 * share of all packed bytes through per-wave LDS rings; chosen when every
 * workgroup's token rows fit its LDS share), "persistent" (the fallback) or
 * "stream-a16" (a bitnet_group_plan_a16 plan), "stream-blocked" (a
 * bitnet_group_plan_blocked plan); "" for a handle not made by
 * bitnet_group_plan*.  The environment
 * variable BITNET_GROUP_KERNEL=persistent, read by bitnet_group_plan, forces
 * the fallback (for comparisons; results are identical). */
const char* bitnet_group_plan_kernel(const bitnet_group_plan_t* plan);

/*
 * The W1.58A16 variant [BitVLA s5: where the 8-bit activation quantiser
 * stalled the GPU, activations stayed in 16 bits]:
 * y[m][n] = w_scale[n] * sum_k x[m][k] * t[n][k], x bf16 [M, K] (row stride
 * ldx, rows 16-byte aligned), packed / w_scale as for bitnet_linear_forward,
 * y fp32 or bf16 [M, N] (ldy).  x may also be fp16 (x_dtype BITNET_F16; the
 * path kept 16-bit activations, and both 16-bit formats widen exactly); the
 * sum then runs on fp16 matrix cores.  The sum runs in fp32 on the matrix
 * cores in the hardware's order: |y - exact| <= w_scale[n] * (K/32 + 64) *
 * 2^-24 * sum_k |x[m][k] * t[n][k]| (+ the bf16 rounding for bf16 y), for
 * partial sums below 2^127 in magnitude (bf16 x is summed as x * 2t and
 * halved: exact below that, infinite above).  A decode-size kernel: every 16
 * tokens re-read the packed weight.  Errors:
 * UNSUPPORTED for fp32 x; INVALID_ARG as bitnet_linear_forward; HIP.
 */
bitnet_status_t bitnet_linear_a16(hipStream_t stream, const void* x, bitnet_dtype_t x_dtype,
                                  int64_t M, int64_t K, int64_t ldx,
                                  const uint8_t* packed, const float* w_scale, int64_t N,
                                  void* y, bitnet_dtype_t y_dtype, int64_t ldy);

/*
 * Per-block weight scales [BitVLA s2: the sibling matvec kernel keeps one
 * scale per 256-weight block, a scale matrix of N x K/256, where BitNet keeps
 * one per tensor].  Block b of row n holds k = 256b .. min(256b + 256, K) - 1;
 * a row has bitnet_block_count(K) = ceil(K/256) blocks, the last one partial
 * when 256 does not divide K.
 *
 * bitnet_pack_weights_blocked (device memory, synchronous on `stream`):
 *   W [N, K] bf16 or fp32 (row stride ldw), packed [N][Kp/4] in layout v1
 *   (16-byte aligned), block_scale [nb][N] fp32, block-major.  Per block:
 *   mean = fp32(fp64 sum of |W| over the block, k ascending, / the block's
 *   weight count), s = 1/mean (fp32), t = clamp(rne(W*s), -1, 1); a zero
 *   block has scale 0 and codes 0.  K <= 8192.
 * bitnet_linear_blocked_forward (asynchronous on `stream`): q, a_scale from
 *   bitnet_act_quant ([M][Kp], 16-byte aligned), y fp32 or bf16 [M, N] (ldy):
 *   y[m][n] = a_scale[m] * sum_b acc_b * block_scale[b][n] with the exact
 *   int32 block sums acc_b = sum_{k in block b} q*t, evaluated in fp32 as
 *   total = 0; for b ascending: total = total + (float)acc_b * block_scale;
 *   y = total * a_scale (bf16 y: that value rounded to nearest even).
 *   M <= 16 runs the streaming decode kernel (one pass over codes and scales),
 *   larger M an int8-MFMA GEMM; both give identical bits.
 * Errors: INVALID_ARG (sizes, NULL or misaligned pointers, ld < K or N, bad
 * dtype); UNSUPPORTED for K > 8192; NONFINITE for a non-finite weight; HIP.
 */
int64_t bitnet_block_count(int64_t K);   /* ceil(K/256); -1 for a bad K */

bitnet_status_t bitnet_pack_weights_blocked(hipStream_t stream, const void* W, bitnet_dtype_t w_dtype,
                                            int64_t N, int64_t K, int64_t ldw,
                                            uint8_t* packed, float* block_scale);

bitnet_status_t bitnet_linear_blocked_forward(hipStream_t stream, const int8_t* q, const float* a_scale,
                                              int64_t M, int64_t K, const uint8_t* packed,
                                              const float* block_scale, int64_t N,
                                              void* y, bitnet_dtype_t y_dtype, int64_t ldy);

/*
 * I2_S interchange [Guide s3.3 "I2_S Ternary Packing"], for weights
 * converted by bitnet.cpp's tooling.  An I2_S buffer of one [N, K] tensor is
 * N*K/4 code bytes followed by one fp32 scale s = 1/mean|W| (little-endian),
 * bitnet_i2s_bytes(N, K) bytes in all.  The tensor's values, flattened
 * row-major, form blocks of 128; block b is bytes 32b..32b+31; a byte holds
 * four stored codes (-1 -> 0, 0 -> 1, +1 -> 2, the codes of layout v1) as
 * (c0 << 6) | (c1 << 4) | (c2 << 2) | c3.  The page does not say which four
 * values of a block share a byte:
 *   BITNET_I2S_STRIDED      byte j of a block holds values j, j+32, j+64,
 *                           j+96 as c0..c3 (a block size only matters to a
 *                           layout of this kind, so this is the default);
 *   BITNET_I2S_CONSECUTIVE  byte j holds values 4j, 4j+1, 4j+2, 4j+3.
 */
typedef enum {
    BITNET_I2S_STRIDED = 0,
    BITNET_I2S_CONSECUTIVE = 1,
    BITNET_I2S_RANGE_MIN_ = -0x7FFFFFFF - 1,
    BITNET_I2S_RANGE_MAX_ = 0x7FFFFFFF
} bitnet_i2s_order_t;

/* Bytes of the I2_S buffer of an [N, K] tensor; -1 unless K % 16 == 0 and
 * N*K % 128 == 0. */
int64_t bitnet_i2s_bytes(int64_t N, int64_t K);

/*
 * I2_S buffer -> layout v1 (packed [N][Kp/4], w_scale[n] = 1/s for every row,
 * codes k >= K set to 1).  `where` says whether all three buffers are host or
 * device memory (device: 4-byte aligned i2s and w_scale; synchronous on
 * `stream`).  Errors: INVALID_ARG for bad sizes, a field holding 3 or a scale
 * that is not positive (outputs then partly written); HIP.
 */
bitnet_status_t bitnet_i2s_import(bitnet_mem_t where, hipStream_t stream, const uint8_t* i2s,
                                  int64_t N, int64_t K, bitnet_i2s_order_t order,
                                  uint8_t* packed, float* w_scale);

/*
 * Layout v1 -> I2_S buffer of bitnet_i2s_bytes(N, K) bytes, with
 * s = 1/w_scale[0].  I2_S has one scale per tensor: every w_scale[n] must be
 * equal (export the segments of a fused tensor one at a time, by rows).
 * Same memory rules and errors as bitnet_i2s_import.
 */
bitnet_status_t bitnet_i2s_export(bitnet_mem_t where, hipStream_t stream, const uint8_t* packed,
                                  const float* w_scale, int64_t N, int64_t K, bitnet_i2s_order_t order,
                                  uint8_t* i2s);

/*
 * Packed-weight files: a versioned container for layout v1, so packing (an
 * offline conversion [Guide s3.3]) is done once.  Host memory, synchronous.
 * Format (little-endian): a 64-byte header -- magic "BTNLV1\0\0", u32
 * version (1), u32 header size (64), i64 N, K, Kp, i32 segment count, u32
 * layout (1 = layout v1), u64 FNV-1a-64 of the 48 header bytes before it and
 * then of every byte after the header, u64 reserved (0) -- then packed
 * [N][Kp/4], w_scale [N] fp32, the segments' row counts (i64) and means
 * (fp32).
 * bitnet_load_packed with packed == NULL only reads the header into N, K and
 * n_segs (to size the buffers); otherwise it fills all four arrays and checks
 * the checksum.  Errors: INVALID_ARG (I/O, bad or inconsistent file,
 * checksum), UNSUPPORTED (another version or layout).
 */
bitnet_status_t bitnet_save_packed(const char* path, const uint8_t* packed, const float* w_scale,
                                   int64_t N, int64_t K, const int64_t* seg_rows, const float* seg_mean,
                                   int32_t n_segs);
bitnet_status_t bitnet_load_packed(const char* path, int64_t* N, int64_t* K, int32_t* n_segs,
                                   uint8_t* packed, float* w_scale, int64_t* seg_rows, float* seg_mean);

/* Static text for a status code. */
const char* bitnet_status_string(bitnet_status_t s);

/* Detail of the calling thread's last failure ("" if none); valid until that
 * thread's next call into the library. */
const char* bitnet_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* BITNET_H */
