/*
 * fp4.h -- C ABI of the MI355X (gfx950) block-scaled FP4 library.
 *
 * The method (page citations; the pages print no formula, the reading taken
 * where they are silent is stated at each call):
 *   quant_prune_distill/486 "Метод": NVFP4 = E2M1 elements in groups of 16
 *     with an E4M3 scale (4.5 bit/param); MXFP = groups of 32 with an E8M0
 *     (power-of-two) scale (4.25 bit/param); small groups need efficient
 *     kernels for the scale handling.
 *   gonzo_ML/3986 "Форматы FP4": group 16; scale encodings swept from E1M6
 *     to E8M0.  "Стохастическая квантизация": round to nearest, or up/down
 *     with probability set by the distance; nearest for forward weights and
 *     activations, stochastic for backward gradients.
 *   ue5m3-fp4-pretraining "Что сделали": unsigned UE5M3 block scales; the
 *     tensor maximum is refreshed every 50 steps, stored in between; all
 *     suitable linear layers run in FP4.
 *   quant_prune_distill/574 "Эксперименты": weight-only NVFP4 with a
 *     memory-bound small-batch kernel for rollouts.
 *
 * Conventions for every call:
 *   - Data pointers are DEVICE pointers owned by the caller (e.g. torch
 *     tensors).  The library never allocates or frees caller memory and
 *     allocates nothing per call; an fp4_amax_state owns 17664 bytes of
 *     device memory allocated at creation.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Every launch is asynchronous on it; no call synchronizes the host
 *     except fp4_amax_state_get / fp4_amax_state_set.
 *   - Arguments are validated before any launch.  A negative status means
 *     nothing was launched and nothing was written.  FP4_ERR_HIP means a
 *     launch was attempted and the runtime reported an error.
 *   - No exceptions cross the ABI.
 *   - Element codes: row-major [rows, cols/2] bytes, the even-index element
 *     in the low nibble; nibble = sign << 3 | E2M1 magnitude code.  Scales:
 *     row-major [rows, cols/block] bytes.  (Reading: the pages fix the
 *     storage cost, not the layout.)
 */
#ifndef FP4_H
#define FP4_H

#include <stdint.h>

#if defined(__GNUC__)
#define FP4_API __attribute__((visibility("default")))
#else
#define FP4_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum fp4_status {
    FP4_OK = 0,
    FP4_ERR_INVALID_ARG = -1, /* null pointer, bad enum, bad block size     */
    FP4_ERR_UNSUPPORTED = -2, /* valid but unsupported combination          */
    FP4_ERR_SHAPE = -3,       /* cols % block != 0, K mismatch, ld < cols   */
    FP4_ERR_ALIGN = -4,       /* pointer or leading dimension misaligned    */
    FP4_ERR_HIP = -5          /* the HIP runtime reported an error          */
} fp4_status;

/* Block-scale encodings.  ExMy (sign + x exponent + y mantissa bits, x+y=7)
 * and UE5M3 (no sign bit): bias 2^(x-1)-1, exponent field 0 is subnormal,
 * no infinity, the code with every exponent and mantissa bit set is NaN
 * (reading; the pages name the formats only).  E8M0: value 2^(code-127). */
typedef enum fp4_scale_fmt {
    FP4_SCALE_E4M3 = 0,
    FP4_SCALE_UE5M3 = 1,
    FP4_SCALE_E3M4 = 2,
    FP4_SCALE_E1M6 = 3,
    FP4_SCALE_E8M0 = 4,
    FP4_SCALE_E2M5 = 5,
    FP4_SCALE_E5M2 = 6,
    FP4_SCALE_E6M1 = 7,
    FP4_SCALE_E7M0 = 8
} fp4_scale_fmt;

typedef enum fp4_rounding {
    FP4_ROUND_NEAREST_EVEN = 0, /* ties to the even code, saturate at 6      */
    FP4_ROUND_STOCHASTIC = 1    /* Philox4x32-10, 16 random bits per element */
} fp4_rounding;

typedef enum fp4_amax_policy {
    FP4_AMAX_NONE = 0,    /* no tensor scale (g = 1); required for E8M0      */
    FP4_AMAX_CURRENT = 1, /* g from max|x| of this call's tensor             */
    FP4_AMAX_DELAYED = 2  /* g from the stored max, refreshed every interval */
} fp4_amax_policy;

typedef enum fp4_dtype { FP4_DTYPE_F32 = 0, FP4_DTYPE_BF16 = 1 } fp4_dtype;

/* Transform applied to every block before quantization
 * (ue5m3-fp4-pretraining "Что сделали": a randomized Hadamard transform
 * spreads outliers over the block before quantization, and that scheme
 * leaves it out; quant_prune_distill/574 "Метод": Hadamard rotations bring
 * weights and activations closer to Gaussian).  The pages give no formula;
 * reading, for every block v of `block` consecutive elements along the
 * blocked dimension:
 *   y = c * H * D * v,  D = diag(-1 where bit j of transform_signs is set,
 *   else +1),  H the Sylvester Hadamard matrix ((H)_ij = (-1)^popcount(i&j)),
 *   c = 1/sqrt(block) rounded to binary32 (exactly 1/4 for block 16),
 * in binary32: H by butterfly stages h = 1, 2, 4, ... (each pair (i, i+h)
 * becomes (a + b, a - b)), then the product by c.  Block maxima, the tensor
 * maximum and the codes all see y.  Dequantization applies the inverse
 * v = D * (c * (H * y)) to the binary32 dequantized values.  H D / sqrt(B) is
 * orthogonal, so fp4_gemm of two operands transformed with the same
 * block and signs along K computes the same product. */
typedef enum fp4_transform {
    FP4_TRANSFORM_NONE = 0,
    FP4_TRANSFORM_RHT = 1      /* blockwise randomized Hadamard transform     */
} fp4_transform;

/* Element grid (quant_prune_distill/574 "Метод": the NV and MX block/scale
 * schemes paired with an FP or an INT element grid).  Reading for INT4: the
 * symmetric grid -7..7 as a two's-complement nibble (zero has no sign; the
 * code 0x8 is never produced); every rule that maps a maximum to the E2M1
 * maximum 6 maps it to 7 instead (g = amax_t / (7 Smax), u = amax_b /
 * RN(7 g)); the E8M0 exponent rule is unchanged (amax_b / s in [4, 8), the
 * MX convention for a sign + 3-bit fixed-point element); nearest rounding
 * ties to the even integer and saturates at 7; stochastic rounding as for
 * E2M1 with grid spacing 1.
 * The 8-bit grids (the same page's MXFP8 / MXINT8) store one byte per
 * element, codes [rows, cols] (reading): FP8 E4M3 elements, nearest-even
 * and saturating at 448, the sign bit kept (also for zero); INT8 on the
 * symmetric grid -127..127 (two's complement, zero unsigned).  448 or 127
 * takes the place of 6 in the tensor and block scales; the E8M0 rule uses
 * floor(log2 amax_b) - 8 (FP8) or - 6 (INT8) + 127, the OCP MX offsets.
 * Every call takes them.
 * The 6-bit grids (the same page's MXFP6 / MXINT6; reading: the OCP FP6
 * element formats E2M3 and E3M2, and INT6 on -31..31) pack six bits per
 * element as a little-endian bit stream: element c of a row at bits
 * 6c .. 6c + 5 of the row's cols*3/4 bytes.  FP6 E2M3: bias 1, largest 7.5;
 * E3M2: bias 3, largest 28; sign bit 5, subnormals, no reserved codes;
 * nearest-even, saturating.  INT6: six-bit two's complement, zero unsigned.
 * 7.5, 28 or 31 takes the place of 6; the E8M0 offsets are 2, 4 and 4.
 * Every call takes them (the column-wise and two-orientation calls with
 * R % 64 == 0, SHAPE otherwise). */
typedef enum fp4_element {
    FP4_ELEM_E2M1 = 0,
    FP4_ELEM_INT4 = 1,
    FP4_ELEM_FP8_E4M3 = 2,    /* MXFP8-style, one byte per element           */
    FP4_ELEM_INT8 = 3,        /* MXINT8-style, one byte per element          */
    FP4_ELEM_FP6_E2M3 = 4,    /* MXFP6-style, six bits per element           */
    FP4_ELEM_FP6_E3M2 = 5,    /* MXFP6-style, six bits per element           */
    FP4_ELEM_INT6 = 6         /* MXINT6-style, six bits per element          */
} fp4_element;

typedef struct fp4_format {
    int32_t block;            /* 16 or 32 elements per scale                  */
    int32_t scale;            /* fp4_scale_fmt                                */
    int32_t rounding;         /* fp4_rounding                                 */
    int32_t amax;             /* fp4_amax_policy                              */
    int32_t transform;        /* fp4_transform                                */
    uint32_t transform_signs; /* RHT: bit j negates element j of each block   */
    int32_t element;          /* fp4_element                                  */
} fp4_format;

/* A quantized tensor.  q: rows*cols/2 bytes (4-bit grids), rows*cols
 * bytes (8-bit grids) or rows*cols*3/4 bytes (6-bit grids); scales:
 * rows*cols/block bytes; tensor_scale: 2 floats {g, amax used} (g = 1 and
 * amax = 0 under NONE).  All three are device pointers; q must be 4-byte
 * aligned (8-byte for the 8- and 6-bit grids). */
typedef struct fp4_tensor {
    uint8_t* q;
    uint8_t* scales;
    float* tensor_scale;
    int64_t rows;
    int64_t cols;
    fp4_format fmt;
} fp4_tensor;

/* Per-tensor amax state (ue5m3-fp4-pretraining "Что сделали": the maximum
 * is refreshed every `interval` steps and the stored value used between).
 * Required by CURRENT (which refreshes on every call) and DELAYED.  Owns 17664
 * bytes of device memory on the device current at creation: the stored
 * amax, the per-workgroup partial maxima of the refresh and the exchange
 * words of the single-pass refresh.  Not thread-safe; calls that use one
 * state must be ordered (one stream, or synchronized). */
typedef struct fp4_amax_state fp4_amax_state;

/* interval >= 1.  Allocates the device workspace (zeroed, synchronously). */
FP4_API fp4_status fp4_amax_state_create(uint32_t interval, fp4_amax_state** out);
FP4_API fp4_status fp4_amax_state_destroy(fp4_amax_state* state);
/* Checkpoint: number of quantize calls seen and the stored amax.  Waits for
 * the device to finish outstanding work. */
FP4_API fp4_status fp4_amax_state_get(const fp4_amax_state* state, uint64_t* calls, float* amax);
/* Resume: overwrite the call count and stored amax (synchronous copy; also
 * clears the exchange words and the fallback count). */
FP4_API fp4_status fp4_amax_state_set(fp4_amax_state* state, uint64_t calls, float amax);

/* Single-pass refresh diagnostics.  In a single-pass refresh (see
 * fp4_quantize) the workgroups exchange their maxima through the state and
 * each waits a bounded time for all the others; a workgroup that gives up
 * (other work on the device kept some from being scheduled) reads the whole
 * tensor to take its maximum itself.  That maximum is the same value, so
 * codes, scales and tensor scale never depend on it; only the time does.
 * fp4_amax_state_fallbacks: the number of workgroups that took this path on
 * this state since its creation or last fp4_amax_state_set (waits for the
 * device).  fp4_set_exchange_wait: the process-wide wait bound in ticks of
 * the device's 100 MHz real-time counter (default 20000000, 0.2 s; 0 gives
 * up after one look at the other workgroups' words), for tests of the
 * fallback; the previous bound is returned in *previous if not null. */
FP4_API fp4_status fp4_amax_state_fallbacks(const fp4_amax_state* state, uint32_t* n);
FP4_API fp4_status fp4_set_exchange_wait(uint64_t ticks, uint64_t* previous);

/*
 * fp4_quantize -- quantize x[rows, cols] (row stride ld_x elements, f32 or
 * bf16) into out->q / out->scales / out->tensor_scale with out->fmt.
 * Pages: gonzo_ML/3986 "Форматы FP4" (E2M1 values, groups of 16, the swept
 * scale encodings) and "Стохастическая квантизация" (nearest rounding,
 * stochastic rounding for gradients); quant_prune_distill/486 "Метод" (NVFP4:
 * group 16 with an E4M3 scale under a tensor scale; MXFP4: group 32 with an
 * E8M0 scale); ue5m3-fp4-pretraining "Что сделали" (UE5M3 scales, the tensor
 * maximum refreshed every 50 steps).
 *
 * Per block of B elements (reading of the pages' "shared scale per small
 * group"; every step binary32 round-to-nearest-even):
 *   ExMy: g = amax_t / (6 * Smax) (g = 1 under NONE, or if the quotient is
 *         0 or not finite); u = RN(amax_b / RN(6 g)); code = nearest-even
 *         saturating ExMy encode of u; s = decode(code).
 *   E8M0: code = clamp(floor(log2 amax_b) - 2 + 127, 0, 254) (0 for an
 *         all-zero block); s = 2^(code-127); g = 1.
 *   S = RN(s g); inv = RN(1/S) clamped to FLT_MAX (inv = 0 when S = 0);
 *   v = RN(x inv); magnitude = nearest-even E2M1 code of |v| saturated at 6,
 *   or, for FP4_ROUND_STOCHASTIC, lo + [r16 / 2^16 < (|v|-lo)/(hi-lo)] with
 *   r16 the 16-bit half (i & 1) of word (i >> 1) & 3 of
 *   Philox4x32-10(key = seed, counter = {i >> 3 as 64 bits, offset as 64
 *   bits}), i = row * cols + col the logical element index.
 *
 * x: device, 16-byte aligned; ld_x * sizeof(elem) a multiple of 16; ld_x >=
 * cols.  cols % block == 0; block in {16, 32}; rows * cols / 8 < 2^31.  For an
 * empty tensor (rows or cols 0) x, q and scales may be null; tensor_scale
 * is still written ({1, 0} under CURRENT).
 * state: required for CURRENT and DELAYED (ignored for NONE).  CURRENT
 * recomputes amax_t on every call; DELAYED recomputes it when
 * state->calls % interval == 0 and otherwise reuses the stored value (a
 * tensor that outgrew it saturates at +-6).  Each call increments the
 * state's call count on the host (no device synchronization).  A refresh
 * reads x once when the tensor fits one workgroup per compute unit at 8192
 * units of 8 elements each (4096 x 4096 on a 256-CU device; the
 * workgroups agree on amax_t through the state), else twice (an amax pass,
 * then the quantize pass).
 * seed, offset: used only for FP4_ROUND_STOCHASTIC.
 * out->fmt.transform = FP4_TRANSFORM_RHT transforms every block first (see
 * fp4_transform); the tensor maximum is then that of the transformed tensor.
 * Errors: INVALID_ARG (null pointers, bad enums, missing state), SHAPE,
 * ALIGN, UNSUPPORTED (E8M0 with a tensor-scale policy).
 */
FP4_API fp4_status fp4_quantize(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* out,
                        fp4_amax_state* state, uint64_t seed, uint64_t offset, void* stream);

/*
 * fp4_quantize_noalloc -- for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): fp4_quantize with the policies NONE and CURRENT, the same
 * result bit for bit, but the current-amax workspace (17664 bytes) comes
 * from a static device array of the library, one per device, held until
 * the process ends, instead of an fp4_amax_state.  The workspace does not
 * grow with the tensor, so no size is refused on its account (fp4_quantize's
 * own limits apply).  The caller passes x and out as for fp4_quantize;
 * nothing is allocated or freed, on any call.  The first call on a device
 * looks up that device's array address (with the device current).
 * Every call on a device shares that one array: calls that overlap on one
 * device (different streams, or threads without ordering) race and must be
 * ordered by the caller.  Errors as fp4_quantize; UNSUPPORTED for DELAYED
 * (the stored maximum belongs to one tensor and needs an fp4_amax_state).
 */
FP4_API fp4_status fp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* out,
                                        uint64_t seed, uint64_t offset, void* stream);

/*
 * fp4_quantize_transposed -- column-wise quantization for the backward
 * pass: out describes x^T, where x is [out->cols, out->rows] (row stride
 * ld_x elements, f32 or bf16), so each block holds `block` consecutive rows
 * of one column of x.  The result is, bit for bit, fp4_quantize applied to
 * the materialized transpose of x: same scale, rounding and amax rules,
 * and the stochastic-rounding index is that of x^T (i = c * out->cols + r
 * for element x[r, c]).  (gonzo_ML/3986 "Стохастическая квантизация":
 * stochastic rounding for the backward gradients; ue5m3-fp4-pretraining
 * "Что сделали": every suitable linear layer in FP4, which needs the
 * weight-gradient operands blocked along the token dimension.  Reading:
 * the pages give no layout for them; the transpose's row-major layout is
 * the [N, K] operand fp4_gemm consumes.)
 * x: device, 16-byte aligned, ld_x * sizeof(elem) a multiple of 16, ld_x >=
 * out->rows; out->rows % 8 == 0; out->cols % block == 0; out->q 16-byte
 * aligned.  A refresh of the tensor maximum reads x twice (an amax pass,
 * then the quantize pass).  With out->fmt.transform = FP4_TRANSFORM_RHT the
 * transform runs down the columns of x (over each block of x^T), and a
 * refresh takes the maximum of the transformed tensor.  Errors as
 * fp4_quantize.
 */
FP4_API fp4_status fp4_quantize_transposed(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* out,
                                   fp4_amax_state* state, uint64_t seed, uint64_t offset, void* stream);

/*
 * fp4_quantize_both -- both orientations of x [R, C] from one read: rowwise
 * [R, C] receives exactly what fp4_quantize(x) writes, colwise [C, R]
 * exactly what fp4_quantize_transposed(x) writes, and both get the same
 * tensor scale (gonzo_ML/3986 "Стохастическая квантизация" and
 * ue5m3-fp4-pretraining "Что сделали": the backward pass quantizes the
 * same gradient and activation tensors along both dimensions, one for each
 * of its two products).  Both tensors must carry the same block size, scale
 * encoding, rounding, amax policy and element grid, and no transform
 * (UNSUPPORTED otherwise: a transform along each axis would give the two
 * outputs different maxima).  The amax state counts the pair as one call.
 * Requirements as for the two calls together: R % block == 0, C % block ==
 * 0 (R % 64 == 0 for the 6-bit grids), x 16-byte aligned with ld_x *
 * sizeof(elem) a multiple of 16, colwise->q 16-byte aligned.  A refresh of the tensor maximum reads x twice (an amax
 * pass, then this one); otherwise x is read once.
 */
FP4_API fp4_status fp4_quantize_both(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* rowwise,
                                     fp4_tensor* colwise, fp4_amax_state* state, uint64_t seed, uint64_t offset,
                                     void* stream);

/*
 * fp4_dequantize -- y[rows, cols] (row stride ld_y, f32 or bf16) =
 * RN(RN(e2m1(code) * s) * g), rounded once more to bf16 (RNE) for bf16
 * output (quant_prune_distill/486 "Метод": the element times its group's
 * scale).  With in->fmt.transform = FP4_TRANSFORM_RHT the inverse transform
 * is applied to the binary32 values before any bf16 rounding.
 * in->tensor_scale[0] is read on the device.  y: 16-byte aligned,
 * ld_y * sizeof(elem) a multiple of 16.
 */
FP4_API fp4_status fp4_dequantize(const fp4_tensor* in, void* y, int32_t y_dtype, int64_t ld_y, void* stream);

/*
 * fp4_gemm -- C[M, N] (bf16, row stride ldc) = bf16_RNE(ga * gb *
 * sum_k (e2m1(a_mk) s_a)(e2m1(b_nk) s_b)) with fp32 accumulation, for
 * A = a [M, K] and W = b [N, K] both blocked along K (C = A W^T)
 * (ue5m3-fp4-pretraining "Что сделали": the linear layers run in FP4;
 * quant_prune_distill/574 "Выводы": weight + activation FP4 for the
 * compute-bound regime).  Both operands must use the same block size, the
 * same element grid and the same transform (kind and signs; UNSUPPORTED
 * otherwise).  Every element times its block scale enters a matrix
 * instruction exactly, in a 16-bit type chosen per pairing: INT4 in bf16
 * when int * s fits it exactly for both scale formats, else f16; FP8 E4M3
 * elements in bf16 for scale formats with at most 3 mantissa bits (E8M0,
 * E7M0, E6M1, E5M2, E4M3, UE5M3); INT8 in bf16 for power-of-two scales
 * (E8M0, E7M0) and in f16 for E4M3 scales; FP6 E2M3 as FP8, FP6 E3M2 in
 * bf16 for scales with at most 4 mantissa bits, INT6 in bf16 for at most 2
 * (E8M0, E7M0, E6M1, E5M2) and in f16 for E4M3 / E3M4 / E2M5; other 8- and
 * 6-bit pairings return UNSUPPORTED.
 * Paths: E2M1 with E8M0 scales on both operands runs on the gfx950
 * block-scaled FP4 matrix instruction (at block 16 when K % 256 == 0 and
 * each operand's codes are below 4 GiB; else in LDS); E2M1 with the formats
 * exact in f16 (E4M3, E3M4, E2M5, E1M6) or in bf16 (UE5M3, E5M2, E6M1,
 * E7M0), MXFP8 (FP8 with E8M0 on both) and INT8 with E4M3 on both are
 * converted to f16 / bf16 in registers; every other pairing is dequantized
 * to bf16 / f16 in LDS.  Small products of E2M1 with f16-exact ExMy scales
 * on both operands, of MXFP8 and of INT8 with E4M3 scales (M * N at most
 * the bound of fp4_set_gemm_small_outputs, 2^21 by default), of E2M1 with
 * bf16-exact ExMy scales (1.5 times the bound) or with E8M0 scales (an
 * eighth of it) run one wave per 32 x 32 output tile with the same
 * conversions and instructions and no LDS.  Result within 1e-5 * sum_k
 * |a||b| of the exact product before the bf16 rounding.
 * K % 128 == 0 (K = 0 writes C = 0 and reads no operand), M and N
 * arbitrary; ldc >= N; c 2-byte aligned (rows that
 * are 8-byte aligned are written with vector stores); operand codes 16-byte
 * and scales 4-byte aligned.
 */
FP4_API fp4_status fp4_gemm(const fp4_tensor* a, const fp4_tensor* b, uint16_t* c, int64_t ldc, void* stream);

/*
 * fp4_set_gemm_small_outputs -- the process-wide bound on M * N (output
 * elements) up to which fp4_gemm takes the small-product path for the
 * pairings it covers (above; E2M1 with E8M0 an eighth of it, E2M1 with the
 * bf16-exact ExMy pairings 1.5 times it).  0 turns the
 * path off, so that tests can run the tiled kernels on small shapes.
 * Results on either path meet the same error bound.  The previous value is
 * returned in *previous if not null; a negative bound is
 * FP4_ERR_INVALID_ARG.
 */
FP4_API fp4_status fp4_set_gemm_small_outputs(int64_t outputs, int64_t* previous);

/*
 * fp4_wo_gemm -- Y[M, N] (bf16, row stride ldy) = bf16_RNE(gw *
 * sum_k x[m, k] (e2m1(w_nk) s_w)), fp32 accumulation, weights dequantized
 * in registers (quant_prune_distill/574 "Метод"/"Эксперименты":
 * weight-only NVFP4, memory-bound small-batch generation).
 * x: bf16 [M, K] (row stride ldx), w: [N, K] quantized along K.
 * 1 <= M <= 16; K % 256 == 0 (K = 0 writes Y = 0 and reads neither x nor w);
 * x 16-byte aligned, ldx % 8 == 0, ldy >= N;
 * w's codes 16-byte and scales 4-byte aligned; w's codes < 4 GiB and no
 * transform on w (UNSUPPORTED otherwise).  Every element grid: E2M1, INT4
 * and the 8- and 6-bit ones (quant_prune_distill/486 "Метод": the MX
 * family's 8- and 6-bit members); each product e(w_nk) s_w enters the bf16
 * matrix instruction exactly, as one bf16 value or as the sum of two.
 */
FP4_API fp4_status fp4_wo_gemm(const uint16_t* x, int64_t ldx, int64_t m, const fp4_tensor* w, uint16_t* y,
                       int64_t ldy, void* stream);

/* Static description of a status code. */
FP4_API const char* fp4_status_string(fp4_status status);

/* Library ABI version (major * 100 + minor). */
FP4_API int32_t fp4_version(void);

#ifdef __cplusplus
}
#endif

#endif /* FP4_H */
