/*
 * fp4_oracle.c -- CPU oracle for block-scaled FP4 (E2M1) quantization,
 * dequantization and the GEMMs that consume it.
 *
 * TEST INFRASTRUCTURE ONLY.  The test suite, the smoke check and the CPU
 * baseline leg of the benchmark are the only callers.  The HIP library is
 * the product; it never loads this file and the two share no code, header,
 * table or constant generator.
 *
 * Deliberately plain: sequential loops over rows and blocks, table decode,
 * brute-force nearest-value search for every encode.  Floating-point steps
 * that decide a code are IEEE binary32 with round-to-nearest-even and no
 * contraction (built with -ffp-contract=off); dequantized values for the GEMM
 * reference are exact in binary64.
 *
 * Sources.  The pages name the formats and the method but print no formula:
 *  [P-MXNV]  tgoop.com/quant_prune_distill/486, section "Метод": NVFP4 is
 *            E2M1 in groups of 16 with an E4M3 scale (4.5 bit/param); MXFP
 *            groups of 32 with a log-scale E8M0 scale (4.25 bit/param).
 *  [P-FP4]   nervesearch.ai/c/gonzo_ML/3986 (review of "FP4 all the way"),
 *            "Форматы FP4": group 16, scale formats swept from E1M6 to E8M0,
 *            E1M6 has the narrowest range; "Стохастическая квантизация":
 *            round to nearest, or up/down with a probability set by the
 *            distance to the neighbour.
 *  [P-UE5M3] rit.work/blog/ue5m3-fp4-pretraining, "Что сделали": blocks of
 *            16, the unsigned UE5M3 scale spends all bits on exponent and
 *            mantissa, the tensor maximum is refreshed every 50 steps and the
 *            stored value used in between, stochastic rounding on backward
 *            gradients.
 *  [P-INT]   news.1rj.ru/str/quant_prune_distill/574 (INT vs FP review),
 *            "Метод": Hadamard rotations make distributions more Gaussian.
 * Where the pages are silent the reading taken is stated at each function.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>
#include <float.h>

#define OR_EXPORT __attribute__((visibility("default")))

/* ------------------------------------------------------------------------ */
/* bit helpers                                                               */
/* ------------------------------------------------------------------------ */
static float f_from_bits(uint32_t u) { float f; memcpy(&f, &u, 4); return f; }
static uint32_t bits_of_f(float f) { uint32_t u; memcpy(&u, &f, 4); return u; }

/* bf16 -> fp32 is exact: the bf16 bits are the top half of the fp32 bits. */
static float bf16_to_f32(uint16_t h) { return f_from_bits((uint32_t)h << 16); }

/* ------------------------------------------------------------------------ */
/* E2M1 element codec.  E2M1 = 1 sign, 2 exponent, 1 mantissa bit, bias 1,  */
/* exponent field 0 is subnormal (0 and 0.5), no Inf/NaN.  [P-MXNV]          */
/* ------------------------------------------------------------------------ */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

/* Decode one 4-bit code (bit 3 = sign) to its value. */
OR_EXPORT double or_e2m1_decode(int code)
{
    /* derive the value from the bit fields rather than the table */
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = (e == 0) ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/* Round-to-nearest (reading: ties go to the even code, |v| beyond 6
 * saturates to 6 since E2M1 has no infinity).  Returns the magnitude code
 * 0..7 of |v|.  Plain nearest search over the eight grid magnitudes. */
OR_EXPORT int or_e2m1_rtn(float v)
{
    double a = fabs((double)v);
    if (a != a) return 0;              /* NaN: outside the contract */
    if (a >= 6.0) return 7;
    int best = 0;
    double bd = a;                      /* distance to magnitude 0 */
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - E2M1_MAG[c]);   /* exact: both dyadic, a < 8 */
        if (d < bd || (d == bd && (c & 1) == 0)) { best = c; bd = d; }
    }
    return best;
}

/* Stochastic rounding [P-FP4 "Стохастическая квантизация"]: |v| between the
 * adjacent grid magnitudes lo <= |v| < hi goes up with probability
 * frac = (|v|-lo)/(hi-lo).  Reading: the uniform variate is u = r16 / 2^16
 * from 16 random bits, and the value rounds up iff u < frac; |v| >= 6
 * saturates.  frac is exact (Sterbenz, power-of-two spacing). */
OR_EXPORT int or_e2m1_sr(float v, uint32_t r16)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    if (a >= 6.0) return 7;
    int lo = 0;
    while (lo < 7 && E2M1_MAG[lo + 1] <= a) ++lo;
    double frac = (a - E2M1_MAG[lo]) / (E2M1_MAG[lo + 1] - E2M1_MAG[lo]);
    double u = (double)(r16 & 0xFFFFu) / 65536.0;
    return (u < frac) ? lo + 1 : lo;
}

/* ------------------------------------------------------------------------ */
/* INT4 element grid.  [P-INT] quant_prune_distill/574 "Метод": the NV and   */
/* MX block/scale schemes are paired with an integer element grid (NVINT4:  */
/* groups of 16 with E4M3 scales, MXINT4: groups of 32 with E8M0 scales).    */
/* The page gives no encoding.  Reading: a 4-bit two's-complement integer on */
/* the symmetric grid -7..7 (the code 0x8 = -8 is never produced), the block */
/* maximum mapped to 7, round to nearest with ties to the even integer,      */
/* |v| beyond 7 saturating; stochastic rounding as for E2M1 with grid        */
/* spacing 1.  A zero result has no sign (code 0).                            */
/* ------------------------------------------------------------------------ */
OR_EXPORT double or_int4_decode(int code)
{
    code &= 0xF;
    return (double)(code >= 8 ? code - 16 : code);
}

/* Nearest integer magnitude 0..7 of |v|: plain search over the grid, ties
 * to the even integer, saturating at 7. */
OR_EXPORT int or_int4_rtn(float v)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    if (a >= 7.0) return 7;
    int best = 0;
    double bd = a;
    for (int c = 1; c < 8; ++c) {
        double d = fabs(a - (double)c);
        if (d < bd || (d == bd && (c & 1) == 0)) { best = c; bd = d; }
    }
    return best;
}

OR_EXPORT int or_int4_sr(float v, uint32_t r16)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    if (a >= 7.0) return 7;
    int lo = (int)floor(a);
    double frac = a - (double)lo;
    double u = (double)(r16 & 0xFFFFu) / 65536.0;
    return (u < frac) ? lo + 1 : lo;
}

/* two's-complement nibble of sign * magnitude (magnitude 0 -> code 0) */
static int int4_code(int negative, int mag) { return negative ? ((16 - mag) & 0xF) : mag; }

/* Element grids: 0 = E2M1, 1 = INT4 (4-bit codes, two per byte), 2 = FP8
 * E4M3, 3 = INT8 (one byte each).  [P-INT] quant_prune_distill/574 "Метод":
 * MXFP8/MXINT8 pair the MX groups of 32 with E8M0 scales with the FP8 and
 * INT8 grids.  Reading for the 8-bit grids: FP8 E4M3 elements take the E4M3
 * magnitudes (largest 448), nearest-even and saturating, the sign bit kept
 * (also for zero, as for E2M1); INT8 takes the symmetric grid -127..127 as
 * two's complement (0x80 never produced, zero unsigned). */
/* 6-bit grids: 4 = FP6 E2M3, 5 = FP6 E3M2, 6 = INT6.  [P-INT]
 * quant_prune_distill/574 "Метод" also pairs MXFP6 with MXINT6 (groups of
 * 32, E8M0 scales) and gives no element encoding.  Reading: the two FP6
 * element formats of the OCP MX family (sign bit on top, bias 1 / 3,
 * subnormals, every code finite: largest magnitudes 7.5 / 28), and INT6 on
 * the symmetric grid -31..31 as six-bit two's complement.  Codes are packed
 * little-endian as a bit stream: element c of a row occupies bits 6c ..
 * 6c + 5 of the row's cols * 3 / 4 bytes. */
static int elem_bits(int elem) { return elem >= 4 ? 6 : elem >= 2 ? 8 : 4; }

/* largest element magnitude of a grid */
static float elem_max(int elem)
{
    switch (elem) {
    case 0: return 6.0f;
    case 1: return 7.0f;
    case 2: return 448.0f;
    case 4: return 7.5f;
    case 5: return 28.0f;
    case 6: return 31.0f;
    default: return 127.0f;
    }
}

/* exponent of the grid's largest binade, the E8M0 rule's offset: the block
 * maximum lands in [2^emax, 2^(emax+1)) after scaling (OCP MX convention) */
static int elem_emax(int elem)
{
    switch (elem) {
    case 2: return 8;
    case 3: return 6;
    case 5: return 4;
    case 6: return 4;
    default: return 2;
    }
}

/* INT8: nearest integer magnitude of |v| (ties to even), saturating at 127 */
OR_EXPORT int or_int8_rtn(float v)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    if (a >= 127.0) return 127;
    double lo = floor(a), frac = a - lo;
    int m = (int)lo;
    if (frac > 0.5 || (frac == 0.5 && (m & 1))) m += 1;
    return m;
}

OR_EXPORT int or_int8_sr(float v, uint32_t r16)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    if (a >= 127.0) return 127;
    int lo = (int)floor(a);
    double frac = a - (double)lo;
    double u = (double)(r16 & 0xFFFFu) / 65536.0;
    return (u < frac) ? lo + 1 : lo;
}

OR_EXPORT double or_int8_decode(int code)
{
    code &= 0xFF;
    return (double)(code >= 128 ? code - 256 : code);
}

/* INT6 magnitude: nearest integer of |v| (ties to even), saturating at 31;
 * stochastic as INT8 with spacing 1. */
OR_EXPORT int or_int6_rtn(float v)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    if (a >= 31.0) return 31;
    double lo = floor(a), frac = a - lo;
    int m = (int)lo;
    if (frac > 0.5 || (frac == 0.5 && (m & 1))) m += 1;
    return m;
}

OR_EXPORT int or_int6_sr(float v, uint32_t r16)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    if (a >= 31.0) return 31;
    int lo = (int)floor(a);
    double frac = a - (double)lo;
    double u = (double)(r16 & 0xFFFFu) / 65536.0;
    return (u < frac) ? lo + 1 : lo;
}

OR_EXPORT double or_int6_decode(int code)
{
    code &= 0x3F;
    return (double)(code >= 32 ? code - 64 : code);
}

/* FP6 element value of a 6-bit code (sign bit 5): E2M3 (elem 4) has
 * exponent bias 1 and 3 mantissa bits, E3M2 (elem 5) bias 3 and 2; an
 * exponent field of 0 is subnormal; no code is reserved. */
OR_EXPORT double or_fp6_decode(int code, int elem)
{
    const int mb = elem == 4 ? 3 : 2, bias = elem == 4 ? 1 : 3;
    const int mag = code & 0x1F, e = mag >> mb, m = mag & ((1 << mb) - 1);
    const double frac = ldexp((double)m, -mb);
    const double v = e == 0 ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, e - bias);
    return (code & 0x20) ? -v : v;
}

/* ------------------------------------------------------------------------ */
/* Scale formats.                                                            */
/*   ExMy signed (x+y = 7, sign bit on top) and UE5M3 (unsigned, 8 bits):    */
/*   reading: bias 2^(x-1)-1, exponent field 0 is subnormal, no infinity,    */
/*   the single code with every exponent and mantissa bit set is NaN (the    */
/*   "FN" convention of E4M3).                                               */
/*   E8M0 [P-MXNV]: exponent only, value 2^(code-127), 0xFF is NaN, no zero. */
/* A format is given as (ebits, mbits, has_sign); (8, 0, 0) is E8M0.         */
/* ------------------------------------------------------------------------ */
static int is_e8m0(int eb, int mb, int sg) { return eb == 8 && mb == 0 && !sg; }

static int fmt_valid(int eb, int mb, int sg)
{
    if (is_e8m0(eb, mb, sg)) return 1;
    if (eb < 1 || mb < 0) return 0;
    return (eb + mb + (sg ? 1 : 0)) == 8;
}

/* Number of non-negative codes (sign bit clear). */
static int fmt_ncodes(int eb, int mb, int sg)
{
    (void)sg;
    return 1 << (eb + mb);
}

OR_EXPORT int or_scale_is_nan(int eb, int mb, int sg, int code)
{
    if (is_e8m0(eb, mb, sg)) return code == 0xFF;
    int mag = code & ((1 << (eb + mb)) - 1);
    return mag == (1 << (eb + mb)) - 1;
}

/* Decode a scale code (any of the 256 byte values) to a binary64 value. */
OR_EXPORT double or_scale_decode(int eb, int mb, int sg, int code)
{
    if (!fmt_valid(eb, mb, sg)) return NAN;
    code &= 0xFF;
    if (or_scale_is_nan(eb, mb, sg, code)) return NAN;
    if (is_e8m0(eb, mb, sg)) return ldexp(1.0, code - 127);
    int mag = code & ((1 << (eb + mb)) - 1);
    int neg = sg ? ((code >> (eb + mb)) & 1) : 0;
    int e = mag >> mb, m = mag & ((1 << mb) - 1);
    int bias = (1 << (eb - 1)) - 1;
    double frac = ldexp((double)m, -mb);
    double v = (e == 0) ? ldexp(frac, 1 - bias) : ldexp(1.0 + frac, e - bias);
    return neg ? -v : v;
}

/* Largest finite value of the format (binary64). */
OR_EXPORT double or_scale_max(int eb, int mb, int sg)
{
    double best = 0.0;
    int n = is_e8m0(eb, mb, sg) ? 256 : fmt_ncodes(eb, mb, sg);
    for (int c = 0; c < n; ++c) {
        double v = or_scale_decode(eb, mb, sg, c);
        if (v == v && v > best) best = v;
    }
    return best;
}

/* Encode a non-negative fp32 value to the nearest finite non-negative code
 * (reading: ties to the even code, values above the maximum saturate to
 * it).  Brute force over every code.  Not used for E8M0, whose block rule
 * is the exponent rule below. */
static int last_finite(const double* etab, int n);
static int encode_nearest(const double* tab, int n, float u)
{
    double a = (double)u;
    if (!(a > 0.0)) return 0;          /* 0, negative or NaN: outside contract */
    /* saturation, explicitly: far above the top the binary64 distances to
     * the two largest codes are equal and a tie rule would decide */
    const int top = last_finite(tab, n);
    if (a >= tab[top]) return top;
    int best = -1;
    double bd = INFINITY;
    for (int c = 0; c < n; ++c) {
        double v = tab[c];
        if (v != v) continue;
        double d = fabs(a - v);
        if (best < 0 || d < bd || (d == bd && (c & 1) == 0)) { best = c; bd = d; }
    }
    return best;
}

static void decode_table(int eb, int mb, int sg, double tab[256])
{
    for (int c = 0; c < 256; ++c) tab[c] = or_scale_decode(eb, mb, sg, c);
}

OR_EXPORT int or_scale_encode(int eb, int mb, int sg, float u)
{
    double tab[256];
    decode_table(eb, mb, sg, tab);
    return encode_nearest(tab, fmt_ncodes(eb, mb, sg), u);
}

/* E8M0 block scale (reading of the MX rule [P-MXNV]): the block maximum is
 * brought into the top binade of E2M1, e = floor(log2(amax_b)) - 2, so the
 * largest element lands in [4, 8) and anything above 6 saturates;
 * code = clamp(e + 127, 0, 254); amax_b = 0 gives code 0. */
OR_EXPORT int or_e8m0_block_code_emax(float amax_b, int emax);
OR_EXPORT int or_e8m0_block_code(float amax_b) { return or_e8m0_block_code_emax(amax_b, 2); }

/* As above with the element grid's offset emax (2 for E2M1 and INT4, 8 for
 * FP8 E4M3, 6 for INT8): floor(log2 amax_b) - emax + 127, clamped. */
OR_EXPORT int or_e8m0_block_code_emax(float amax_b, int emax)
{
    if (!(amax_b > 0.0f)) return 0;
    int ex;
    double m = frexp((double)amax_b, &ex);      /* amax_b = m * 2^ex, m in [0.5,1) */
    (void)m;
    int e = (ex - 1) - emax;                    /* floor(log2 amax_b) - emax, exact */
    int code = e + 127;
    if (code < 0) code = 0;
    if (code > 254) code = 254;
    return code;
}

/* Per-tensor scale (reading generalising the NVFP4 recipe amax/(6*448)):
 * g = amax_t / (6 * Smax) in binary32; a zero, underflowed or non-finite
 * quotient gives g = 1.  E8M0 carries no tensor scale (g = 1). */
OR_EXPORT float or_tensor_scale_elem(float amax_t, int eb, int mb, int sg, int elem);
OR_EXPORT float or_tensor_scale(float amax_t, int eb, int mb, int sg)
{
    return or_tensor_scale_elem(amax_t, eb, mb, sg, 0);
}

/* As above for the element grid `elem`: the grid's largest magnitude (6 for
 * E2M1, 7 for INT4) takes the place of 6. */
OR_EXPORT float or_tensor_scale_elem(float amax_t, int eb, int mb, int sg, int elem)
{
    if (is_e8m0(eb, mb, sg)) return 1.0f;
    float smax = (float)or_scale_max(eb, mb, sg);
    float den = elem_max(elem) * smax;
    float g = amax_t / den;
    if (!(g > 0.0f) || g > FLT_MAX) g = 1.0f;
    return g;
}

/* ------------------------------------------------------------------------ */
/* Philox4x32-10 (Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as  */
/* easy as 1, 2, 3", SC'11): ten rounds of two 32x32->64 multiplies with    */
/* the published multipliers and Weyl key increments.                        */
/* ------------------------------------------------------------------------ */
OR_EXPORT void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4])
{
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0; c1 = n1; c2 = n2; c3 = n3;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    out[0] = c0; out[1] = c1; out[2] = c2; out[3] = c3;
}

/* The 16 random bits of the element with logical row-major index i
 * (reading): one Philox call per 8 elements, key = seed, counter =
 * (i/8 as 64 bits, offset as 64 bits); the element takes half (i mod 2) of
 * word ((i/2) mod 4). */
OR_EXPORT uint32_t or_sr_bits(uint64_t seed, uint64_t offset, uint64_t i)
{
    uint64_t blk = i >> 3;
    uint32_t ctr[4] = {(uint32_t)blk, (uint32_t)(blk >> 32), (uint32_t)offset, (uint32_t)(offset >> 32)};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t w[4];
    or_philox4x32_10(ctr, key, w);
    uint32_t word = w[(i >> 1) & 3];
    return (word >> (16 * (i & 1))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------ */
/* Tensor amax: max |x| over a [rows, cols] tensor with row stride ld.       */
/* ------------------------------------------------------------------------ */
static float load_elem(const void* x, int is_bf16, int64_t idx)
{
    return is_bf16 ? bf16_to_f32(((const uint16_t*)x)[idx]) : ((const float*)x)[idx];
}

OR_EXPORT float or_amax(const void* x, int is_bf16, int64_t rows, int64_t cols, int64_t ld)
{
    float m = 0.0f;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            float a = fabsf(load_elem(x, is_bf16, r * ld + c));
            if (a > m) m = a;
        }
    return m;
}

/* ------------------------------------------------------------------------ */
/* Quantize.  For every block of B consecutive elements of a row:           */
/*   amax_b = max |x|                                                        */
/*   ExMy:  d = RN(6 g); u = RN(amax_b / d); code = nearest(u); s = dec(code)*/
/*   E8M0:  code = exponent rule above; s = 2^(code-127)                     */
/*   S = RN(s g); S == 0 -> every magnitude is 0                             */
/*   inv = RN(1 / S), clamped to the largest finite binary32 (reading)       */
/*   v = RN(x inv); magnitude = RTN(v) or SR(v, r16(i))                      */
/*   element code = signbit(x) << 3 | magnitude                              */
/*   byte j of a row = code[2j] | code[2j+1] << 4 (reading: low nibble =     */
/*   even element); scales are one byte per block, row-major.                */
/* Rows [row0, row1) are processed; q/scales point at row row0's output.     */
/* ------------------------------------------------------------------------ */
typedef struct {
    const void* x; int is_bf16; int64_t rows, cols, ld;
    int block, eb, mb, sg; float g;
    int stochastic; uint64_t seed, offset;
    int64_t row0, row1;
    uint8_t* q; uint8_t* scales;
    int elem;                        /* 0 = E2M1, 1 = INT4 */
} quant_job;

/* Index of the largest finite magnitude in a decoded element table: the
 * E4M3 table's last non-negative code (0x7F) is NaN, so its largest finite
 * magnitude (448) sits at 0x7E; every FP6 code is finite. */
static int last_finite(const double* etab, int n)
{
    int top = n - 1;
    while (top > 0 && etab[top] != etab[top]) --top;
    return top;
}

/* FP8 E4M3 / FP6 element, stochastic: |v| between adjacent grid magnitudes
 * lo <= |v| < hi rounds up iff u = r16 / 2^16 < (|v| - lo) / (hi - lo) (exact:
 * the spacing is a power of two); |v| at or beyond the largest finite
 * magnitude saturates to it. */
static int fp8_sr(const double* etab, int n, float v, uint32_t r16)
{
    double a = fabs((double)v);
    if (a != a) return 0;
    const int top = last_finite(etab, n);
    if (a >= etab[top]) return top;
    int lo = 0;
    while (lo + 1 < top && etab[lo + 1] <= a) ++lo;
    double frac = (a - etab[lo]) / (etab[lo + 1] - etab[lo]);
    double u = (double)(r16 & 0xFFFFu) / 65536.0;
    return (u < frac) ? lo + 1 : lo;
}

/* Element magnitude table of the FP8 E4M3 (elem 2) and FP6 (elem 4, 5)
 * grids; returns the number of non-negative codes. */
static int elem_table(int elem, double etab[256])
{
    if (elem == 4 || elem == 5) {
        for (int c = 0; c < 32; ++c) etab[c] = or_fp6_decode(c, elem);
        return 32;
    }
    decode_table(4, 3, 1, etab);
    return fmt_ncodes(4, 3, 1);
}

/* Magnitude code of the scaled value v on an element grid, nearest or
 * stochastic (r16 used only when stochastic). */
static int elem_mag(int elem, const double* etab, int encodes, float v, int stochastic, uint32_t r16)
{
    if (stochastic) {
        switch (elem) {
        case 0: return or_e2m1_sr(v, r16);
        case 1: return or_int4_sr(v, r16);
        case 2: case 4: case 5: return fp8_sr(etab, encodes, v, r16);
        case 6: return or_int6_sr(v, r16);
        default: return or_int8_sr(v, r16);
        }
    }
    switch (elem) {
    case 0: return or_e2m1_rtn(v);
    case 1: return or_int4_rtn(v);
    case 2: case 4: case 5: return encode_nearest(etab, encodes, fabsf(v));
    case 6: return or_int6_rtn(v);
    default: return or_int8_rtn(v);
    }
}

/* Array form of the element rounding on any grid, for exhaustive sweeps in
 * the tests: the magnitude code of each v[i] (r16 may be null for
 * nearest rounding). */
OR_EXPORT void or_elem_mag_array(const float* v, const uint32_t* r16, uint8_t* mag, int64_t n, int elem,
                                 int stochastic)
{
    double etab[256];
    const int encodes = elem_table(elem, etab);
    for (int64_t i = 0; i < n; ++i)
        mag[i] = (uint8_t)elem_mag(elem, etab, encodes, v[i], stochastic, stochastic ? r16[i] : 0u);
}

static void quantize_rows(const quant_job* J, int64_t ra, int64_t rb)
{
    const int64_t nb = J->cols / J->block;
    const int e8 = is_e8m0(J->eb, J->mb, J->sg);
    const float d = elem_max(J->elem) * J->g;
    double tab[256];
    decode_table(J->eb, J->mb, J->sg, tab);
    const int ncodes = fmt_ncodes(J->eb, J->mb, J->sg);
    double etab[256];                               /* FP8 E4M3 / FP6 element magnitudes */
    const int encodes = elem_table(J->elem, etab);
    const int64_t qstride = J->cols * elem_bits(J->elem) / 8;
    for (int64_t r = ra; r < rb; ++r) {
        uint8_t* qrow = J->q + (r - J->row0) * qstride;
        if (elem_bits(J->elem) == 6) memset(qrow, 0, (size_t)qstride);
        uint8_t* srow = J->scales + (r - J->row0) * nb;
        for (int64_t b = 0; b < nb; ++b) {
            const int64_t c0 = b * J->block;
            float amax_b = 0.0f;
            for (int k = 0; k < J->block; ++k) {
                float a = fabsf(load_elem(J->x, J->is_bf16, r * J->ld + c0 + k));
                if (a > amax_b) amax_b = a;
            }
            int scode;
            float s;
            if (e8) {
                scode = or_e8m0_block_code_emax(amax_b, elem_emax(J->elem));
                s = (float)ldexp(1.0, scode - 127);
            } else {
                float u = amax_b / d;
                scode = encode_nearest(tab, ncodes, u);
                s = (float)tab[scode];
            }
            srow[b] = (uint8_t)scode;
            float S = s * J->g;
            float inv = 0.0f;
            if (S != 0.0f) {
                inv = 1.0f / S;
                if (inv > FLT_MAX) inv = FLT_MAX;
            }
            for (int k = 0; k < J->block; ++k) {
                const int64_t col = c0 + k;
                float xv = load_elem(J->x, J->is_bf16, r * J->ld + col);
                int mag = 0;
                if (S != 0.0f) {
                    float v = xv * inv;
                    uint32_t r16 = 0;
                    if (J->stochastic) {
                        uint64_t i = (uint64_t)r * (uint64_t)J->cols + (uint64_t)col;
                        r16 = or_sr_bits(J->seed, J->offset, i);
                    }
                    mag = elem_mag(J->elem, etab, encodes, v, J->stochastic, r16);
                }
                const int neg = (int)(bits_of_f(xv) >> 31);
                int code;
                switch (J->elem) {
                case 0: code = (neg << 3) | mag; break;
                case 1: code = int4_code(neg, mag); break;
                case 2: code = (neg << 7) | mag; break;
                case 4: case 5: code = (neg << 5) | mag; break;
                case 6: code = neg ? ((64 - mag) & 0x3F) : mag; break;
                default: code = neg ? ((256 - mag) & 0xFF) : mag; break;
                }
                if (elem_bits(J->elem) == 6) {
                    const int64_t bit = 6 * col;
                    const int sh = (int)(bit & 7);
                    qrow[bit >> 3] |= (uint8_t)(code << sh);
                    if (sh > 2) qrow[(bit >> 3) + 1] |= (uint8_t)(code >> (8 - sh));
                } else if (elem_bits(J->elem) == 8) qrow[col] = (uint8_t)code;
                else if ((col & 1) == 0) qrow[col >> 1] = (uint8_t)code;
                else qrow[col >> 1] |= (uint8_t)(code << 4);
            }
        }
    }
}

typedef struct { const quant_job* J; int64_t ra, rb; } quant_slice;
static void* quant_thread(void* p)
{
    quant_slice* s = (quant_slice*)p;
    quantize_rows(s->J, s->ra, s->rb);
    return NULL;
}

/* Returns 0 on success, -1 on an argument outside the contract. */
OR_EXPORT int or_quantize_elem(const void* x, int is_bf16, int64_t rows, int64_t cols, int64_t ld,
                               int block, int eb, int mb, int sg, float g,
                               int stochastic, uint64_t seed, uint64_t offset,
                               int64_t row0, int64_t row1, uint8_t* q, uint8_t* scales, int nthreads, int elem);

OR_EXPORT int or_quantize(const void* x, int is_bf16, int64_t rows, int64_t cols, int64_t ld,
                          int block, int eb, int mb, int sg, float g,
                          int stochastic, uint64_t seed, uint64_t offset,
                          int64_t row0, int64_t row1, uint8_t* q, uint8_t* scales, int nthreads)
{
    return or_quantize_elem(x, is_bf16, rows, cols, ld, block, eb, mb, sg, g, stochastic, seed, offset, row0, row1,
                            q, scales, nthreads, 0);
}

/* As or_quantize, on the element grid `elem` (0 = E2M1, 1 = INT4). */
OR_EXPORT int or_quantize_elem(const void* x, int is_bf16, int64_t rows, int64_t cols, int64_t ld,
                               int block, int eb, int mb, int sg, float g,
                               int stochastic, uint64_t seed, uint64_t offset,
                               int64_t row0, int64_t row1, uint8_t* q, uint8_t* scales, int nthreads, int elem)
{
    if (elem < 0 || elem > 6) return -1;
    if (!x || !q || !scales || rows < 0 || cols < 0 || ld < cols) return -1;
    if (block != 16 && block != 32) return -1;
    if (cols % block) return -1;
    if (!fmt_valid(eb, mb, sg)) return -1;
    if (row0 < 0 || row1 > rows || row0 > row1) return -1;
    if (!(g > 0.0f)) return -1;
    quant_job J = {x, is_bf16, rows, cols, ld, block, eb, mb, sg, g, stochastic, seed, offset, row0, row1, q, scales,
                   elem};
    int64_t n = row1 - row0;
    if (nthreads <= 1 || n < 2 * nthreads) {
        quantize_rows(&J, row0, row1);
        return 0;
    }
    if (nthreads > 256) nthreads = 256;
    pthread_t th[256];
    quant_slice sl[256];
    for (int t = 0; t < nthreads; ++t) {
        sl[t].J = &J;
        sl[t].ra = row0 + n * t / nthreads;
        sl[t].rb = row0 + n * (t + 1) / nthreads;
        pthread_create(&th[t], NULL, quant_thread, &sl[t]);
    }
    for (int t = 0; t < nthreads; ++t) pthread_join(th[t], NULL);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Dequantize: x_hat = RN(RN(e2m1(code) * s) * g) in binary32 (the inner     */
/* product is exact), optionally rounded once more to bf16 (RNE).            */
/* ------------------------------------------------------------------------ */
OR_EXPORT uint16_t or_f32_to_bf16(float f)
{
    /* round to nearest even at bit 16 of the binary32 encoding */
    uint32_t u = bits_of_f(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (uint16_t)((u >> 16) | 0x40);   /* NaN stays NaN */
    uint32_t lsb = (u >> 16) & 1u;
    return (uint16_t)((u + 0x7FFFu + lsb) >> 16);
}

static double elem_decode(int code, int elem)
{
    switch (elem) {
    case 0: return or_e2m1_decode(code);
    case 1: return or_int4_decode(code);
    case 2: return or_scale_decode(4, 3, 1, code);
    case 4: case 5: return or_fp6_decode(code, elem);
    case 6: return or_int6_decode(code);
    default: return or_int8_decode(code);
    }
}

static int elem_code_at(const uint8_t* q, int64_t r, int64_t c, int64_t cols, int elem)
{
    if (elem_bits(elem) == 8) return q[r * cols + c];
    if (elem_bits(elem) == 6) {
        const uint8_t* row = q + r * (cols * 3 / 4);
        const int64_t bit = 6 * c;
        const int sh = (int)(bit & 7);
        int v = row[bit >> 3] >> sh;
        if (sh > 2) v |= row[(bit >> 3) + 1] << (8 - sh);
        return v & 0x3F;
    }
    uint8_t byte = q[r * (cols / 2) + c / 2];
    return (c & 1) ? (byte >> 4) : (byte & 0xF);
}

OR_EXPORT int or_dequantize_elem(const uint8_t* q, const uint8_t* scales, float g,
                                 int64_t rows, int64_t cols, int block, int eb, int mb, int sg,
                                 int out_bf16, void* y, int64_t ld_y, int elem);
OR_EXPORT int or_dequantize(const uint8_t* q, const uint8_t* scales, float g,
                            int64_t rows, int64_t cols, int block, int eb, int mb, int sg,
                            int out_bf16, void* y, int64_t ld_y)
{
    return or_dequantize_elem(q, scales, g, rows, cols, block, eb, mb, sg, out_bf16, y, ld_y, 0);
}

/* As or_dequantize on the element grid `elem` (0 = E2M1, 1 = INT4). */
OR_EXPORT int or_dequantize_elem(const uint8_t* q, const uint8_t* scales, float g,
                                 int64_t rows, int64_t cols, int block, int eb, int mb, int sg,
                                 int out_bf16, void* y, int64_t ld_y, int elem)
{
    if (!q || !scales || !y || (block != 16 && block != 32) || cols % block || ld_y < cols) return -1;
    if (!fmt_valid(eb, mb, sg) || elem < 0 || elem > 6) return -1;
    const int64_t nb = cols / block;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int code = elem_code_at(q, r, c, cols, elem);
            float s = (float)or_scale_decode(eb, mb, sg, scales[r * nb + c / block]);
            float e = (float)elem_decode(code, elem);
            float t = e * s;
            float xh = t * g;
            if (out_bf16) ((uint16_t*)y)[r * ld_y + c] = or_f32_to_bf16(xh);
            else ((float*)y)[r * ld_y + c] = xh;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Blockwise randomized Hadamard transform (RHT), applied before            */
/* quantization.  [P-UE5M3] "Что сделали": a randomized Hadamard transform   */
/* spreads outliers over the block before quantization (that scheme drops    */
/* it); [P-INT] quant_prune_distill/574 "Метод": Hadamard rotations make     */
/* weights and activations closer to Gaussian.  The pages give no formula.   */
/* Reading: for every block v of B consecutive elements of a row,            */
/*   y = c_B * (H_B (D v)),                                                  */
/*   D = diag(s_j), s_j = -1 where bit j of `signs` is set, else +1;         */
/*   H_B the Sylvester Hadamard matrix, (H_B)_ij = (-1)^popcount(i & j);     */
/*   c_B = 1/sqrt(B) rounded to binary32 (exactly 1/4 for B = 16).           */
/* H_B v is the in-place butterfly: stages h = 1, 2, 4, ..., B/2 in that     */
/* order, each pair (i, i + h) with bit h of i clear becoming (a + b, a - b),*/
/* every operation binary32 round-to-nearest-even.  The inverse is           */
/* v = D (c_B * (H_B y)) (H_B is symmetric and H_B H_B = B I), evaluated by  */
/* the same butterfly.  bf16 input is widened exactly to binary32 first.     */
/* ------------------------------------------------------------------------ */
OR_EXPORT float or_rht_norm(int block)
{
    return block == 16 ? 0.25f : (float)(1.0 / sqrt((double)block));
}

static void fwht_f32(float* v, int n)
{
    for (int h = 1; h < n; h <<= 1)
        for (int i = 0; i < n; ++i)
            if (!(i & h)) {
                float a = v[i], b = v[i + h];
                v[i] = a + b;
                v[i + h] = a - b;
            }
}

OR_EXPORT int or_rht_forward(const void* x, int is_bf16, int64_t rows, int64_t cols, int block, uint32_t signs,
                             float* y)
{
    if ((block != 16 && block != 32) || cols % block || !y) return -1;
    const float c = or_rht_norm(block);
    float v[32];
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b0 = 0; b0 < cols; b0 += block) {
            for (int j = 0; j < block; ++j) {
                float t = load_elem(x, is_bf16, r * cols + b0 + j);
                v[j] = ((signs >> j) & 1u) ? -t : t;
            }
            fwht_f32(v, block);
            for (int j = 0; j < block; ++j) y[r * cols + b0 + j] = v[j] * c;
        }
    return 0;
}

OR_EXPORT int or_rht_inverse(const float* y, int64_t rows, int64_t cols, int block, uint32_t signs, float* x)
{
    if ((block != 16 && block != 32) || cols % block || !y || !x) return -1;
    const float c = or_rht_norm(block);
    float v[32];
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t b0 = 0; b0 < cols; b0 += block) {
            for (int j = 0; j < block; ++j) v[j] = y[r * cols + b0 + j];
            fwht_f32(v, block);
            for (int j = 0; j < block; ++j) {
                float t = v[j] * c;
                x[r * cols + b0 + j] = ((signs >> j) & 1u) ? -t : t;
            }
        }
    return 0;
}

OR_EXPORT void or_f32_to_bf16_array(const float* x, uint16_t* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = or_f32_to_bf16(x[i]);
}

/* Exact binary64 dequantization for the GEMM reference: e2m1 * s * g. */
OR_EXPORT int or_dequantize_f64_elem(const uint8_t* q, const uint8_t* scales, float g, int64_t rows, int64_t cols,
                                     int block, int eb, int mb, int sg, double* y, int elem);
OR_EXPORT int or_dequantize_f64(const uint8_t* q, const uint8_t* scales, float g,
                                int64_t rows, int64_t cols, int block, int eb, int mb, int sg, double* y)
{
    return or_dequantize_f64_elem(q, scales, g, rows, cols, block, eb, mb, sg, y, 0);
}

OR_EXPORT int or_dequantize_f64_elem(const uint8_t* q, const uint8_t* scales, float g, int64_t rows, int64_t cols,
                                     int block, int eb, int mb, int sg, double* y, int elem)
{
    if (!q || !scales || !y || (block != 16 && block != 32) || cols % block) return -1;
    if (!fmt_valid(eb, mb, sg) || elem < 0 || elem > 6) return -1;
    const int64_t nb = cols / block;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            int code = elem_code_at(q, r, c, cols, elem);
            double s = or_scale_decode(eb, mb, sg, scales[r * nb + c / block]);
            y[r * cols + c] = elem_decode(code, elem) * s * (double)g;
        }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Correct rounding of a binary64 value to bf16 (8 significant bits, the    */
/* binary32 exponent range with subnormals down to 2^-133), RNE.  Used to   */
/* bracket a GEMM result: an output c passes iff c lies between the bf16    */
/* roundings of Cref - T and Cref + T.                                       */
/* ------------------------------------------------------------------------ */
OR_EXPORT double or_round_to_bf16(double x)
{
    if (x != x || x == 0.0 || isinf(x)) return x;
    int ex;
    frexp(x, &ex);                       /* |x| in [2^(ex-1), 2^ex) */
    int qe = ex - 8;                     /* quantum of an 8-bit significand */
    if (qe < -133) qe = -133;            /* subnormal spacing */
    double y = ldexp(nearbyint(ldexp(x, -qe)), qe);   /* default mode: nearest-even */
    const double bmax = ldexp(255.0, 120);           /* (2 - 2^-7) * 2^127 */
    if (fabs(y) > bmax) return x > 0 ? INFINITY : -INFINITY;
    return y;
}

OR_EXPORT void or_round_to_bf16_array(const double* x, double* y, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) y[i] = or_round_to_bf16(x[i]);
}

/* Array forms of the element rounding, for exhaustive sweeps in the tests. */
OR_EXPORT void or_e2m1_rtn_array(const float* v, uint8_t* mag, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) mag[i] = (uint8_t)or_e2m1_rtn(v[i]);
}

OR_EXPORT void or_e2m1_sr_array(const float* v, const uint32_t* r16, uint8_t* mag, int64_t n)
{
    for (int64_t i = 0; i < n; ++i) mag[i] = (uint8_t)or_e2m1_sr(v[i], r16[i]);
}

OR_EXPORT void or_sr_bits_array(uint64_t seed, uint64_t offset, uint64_t i0, int64_t n, uint32_t* out)
{
    for (int64_t k = 0; k < n; ++k) out[k] = or_sr_bits(seed, offset, i0 + (uint64_t)k);
}
