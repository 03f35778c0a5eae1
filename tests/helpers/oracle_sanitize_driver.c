/* Drives every entry point of the CPU oracle over small ragged inputs, for
 * a build with AddressSanitizer and UndefinedBehaviorSanitizer: every grid,
 * scale format, block size, rounding mode and input type, strided rows,
 * zeros, subnormals and values far above each grid's range.  Exit status 0
 * when every call succeeds; the sanitizers abort on the first finding. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

int or_quantize_elem(const void* x, int is_bf16, int64_t rows, int64_t cols, int64_t ld, int block, int eb, int mb,
                     int sg, float g, int stochastic, uint64_t seed, uint64_t offset, int64_t row0, int64_t row1,
                     uint8_t* q, uint8_t* scales, int nthreads, int elem);
int or_dequantize_elem(const uint8_t* q, const uint8_t* scales, float g, int64_t rows, int64_t cols, int block,
                       int eb, int mb, int sg, int out_bf16, void* y, int64_t ld_y, int elem);
int or_dequantize_f64_elem(const uint8_t* q, const uint8_t* scales, float g, int64_t rows, int64_t cols, int block,
                           int eb, int mb, int sg, double* y, int elem);
float or_tensor_scale_elem(float amax_t, int eb, int mb, int sg, int elem);
float or_amax(const void* x, int is_bf16, int64_t rows, int64_t cols, int64_t ld);
int or_rht_forward(const void* x, int is_bf16, int64_t rows, int64_t cols, int block, uint32_t signs, float* y);
int or_rht_inverse(const float* y, int64_t rows, int64_t cols, int block, uint32_t signs, float* x);
void or_elem_mag_array(const float* v, const uint32_t* r16, uint8_t* mag, int64_t n, int elem, int stochastic);
double or_scale_decode(int eb, int mb, int sg, int code);
int or_scale_encode(int eb, int mb, int sg, float u);
int or_scale_is_nan(int eb, int mb, int sg, int code);
double or_scale_max(int eb, int mb, int sg);
int or_e8m0_block_code_emax(float amax_b, int emax);
void or_philox4x32_10(const uint32_t ctr_in[4], const uint32_t key_in[2], uint32_t out[4]);
uint32_t or_sr_bits(uint64_t seed, uint64_t offset, uint64_t i);
uint16_t or_f32_to_bf16(float f);
void or_f32_to_bf16_array(const float* x, uint16_t* y, int64_t n);

static const int FMTS[][3] = {{4, 3, 1}, {5, 3, 0}, {3, 4, 1}, {1, 6, 1}, {2, 5, 1},
                              {5, 2, 1}, {6, 1, 1}, {7, 0, 1}, {8, 0, 0}};
static const int ELEM_BITS[7] = {4, 4, 8, 8, 6, 6, 6};

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static double uniform(void)
{
    rng_state = rng_state * 6364136223846793005ull + 1442695040888963407ull;
    return (double)(rng_state >> 11) * 0x1p-53;
}

static void* xmalloc(size_t n)
{
    void* p = malloc(n ? n : 1);
    if (!p) exit(3);
    return p;
}

static int fail(const char* what)
{
    fprintf(stderr, "oracle sanitize driver: %s\n", what);
    return 1;
}

int main(void)
{
    const int64_t rows = 5, cols = 96, ld = cols + 7;
    float* xf = xmalloc(sizeof(float) * rows * ld);
    uint16_t* xb = xmalloc(sizeof(uint16_t) * rows * ld);
    for (int64_t i = 0; i < rows * ld; ++i) {
        const double u = uniform();
        double v = (uniform() - 0.5) * 4.0;
        if (u < 0.05) v = 0.0;
        else if (u < 0.10) v = ldexp(v, -140);          /* binary32 subnormals */
        else if (u < 0.15) v = ldexp(v, 100);           /* far above every grid */
        else if (u < 0.30) v = ldexp(v, (int)(uniform() * 60) - 30);
        xf[i] = (float)v;
    }
    or_f32_to_bf16_array(xf, xb, rows * ld);

    for (int elem = 0; elem < 7; ++elem)
        for (size_t fi = 0; fi < sizeof(FMTS) / sizeof(FMTS[0]); ++fi)
            for (int block = 16; block <= 32; block += 16)
                for (int sr = 0; sr < 2; ++sr)
                    for (int bf = 0; bf < 2; ++bf) {
                        const int eb = FMTS[fi][0], mb = FMTS[fi][1], sg = FMTS[fi][2];
                        const void* x = bf ? (const void*)xb : (const void*)xf;
                        const int e8 = eb == 8 && mb == 0 && sg == 0;
                        const float amax = or_amax(x, bf, rows, cols, ld);
                        const float g = e8 ? 1.0f : or_tensor_scale_elem(amax, eb, mb, sg, elem);
                        const size_t qbytes = (size_t)(rows * cols * ELEM_BITS[elem] / 8);
                        uint8_t* q = xmalloc(qbytes);
                        uint8_t* s = xmalloc((size_t)(rows * cols / block));
                        if (or_quantize_elem(x, bf, rows, cols, ld, block, eb, mb, sg, g, sr, 0x5EEDull,
                                             (uint64_t)elem * 977u + fi, 0, rows, q, s, 2, elem) != 0)
                            return fail("quantize");
                        const int64_t ldy = cols + 3;
                        float* yf = xmalloc(sizeof(float) * rows * ldy);
                        uint16_t* yb = xmalloc(sizeof(uint16_t) * rows * ldy);
                        double* yd = xmalloc(sizeof(double) * rows * cols);
                        if (or_dequantize_elem(q, s, g, rows, cols, block, eb, mb, sg, 0, yf, ldy, elem) != 0 ||
                            or_dequantize_elem(q, s, g, rows, cols, block, eb, mb, sg, 1, yb, ldy, elem) != 0 ||
                            or_dequantize_f64_elem(q, s, g, rows, cols, block, eb, mb, sg, yd, elem) != 0)
                            return fail("dequantize");
                        free(q); free(s); free(yf); free(yb); free(yd);
                    }

    /* blockwise Hadamard transform and its inverse (dense rows) */
    for (int block = 16; block <= 32; block += 16) {
        float* y = xmalloc(sizeof(float) * rows * cols);
        float* z = xmalloc(sizeof(float) * rows * cols);
        if (or_rht_forward(xf, 0, rows, cols, block, 0xA5A5F00Fu, y) != 0) return fail("rht forward");
        if (or_rht_forward(xb, 1, rows, cols, block, 0x12345678u, y) != 0) return fail("rht forward bf16");
        if (or_rht_inverse(y, rows, cols, block, 0x12345678u, z) != 0) return fail("rht inverse");
        free(y); free(z);
    }

    /* element rounding arrays on every grid, nearest and stochastic */
    {
        const int64_t n = 4096;
        float* v = xmalloc(sizeof(float) * n);
        uint32_t* r = xmalloc(sizeof(uint32_t) * n);
        uint8_t* m = xmalloc((size_t)n);
        for (int64_t i = 0; i < n; ++i) {
            v[i] = (float)ldexp(uniform(), (int)(uniform() * 24) - 12);
            r[i] = (uint32_t)(uniform() * 65536.0) & 0xFFFFu;
        }
        for (int elem = 0; elem < 7; ++elem) {
            or_elem_mag_array(v, NULL, m, n, elem, 0);
            or_elem_mag_array(v, r, m, n, elem, 1);
        }
        free(v); free(r); free(m);
    }

    /* every code of every scale format, the encoder around each value */
    for (size_t fi = 0; fi < sizeof(FMTS) / sizeof(FMTS[0]); ++fi) {
        const int eb = FMTS[fi][0], mb = FMTS[fi][1], sg = FMTS[fi][2];
        const int ncodes = 1 << (eb + mb);
        volatile double acc = or_scale_max(eb, mb, sg);
        for (int c = 0; c < ncodes; ++c) {
            if (or_scale_is_nan(eb, mb, sg, c)) continue;
            const double d = or_scale_decode(eb, mb, sg, c);
            acc += d;
            if (!(eb == 8 && mb == 0 && sg == 0)) {
                acc += or_scale_encode(eb, mb, sg, (float)d);
                acc += or_scale_encode(eb, mb, sg, (float)(d * 1.0001));
            }
        }
        (void)acc;
    }
    for (int emax = 2; emax <= 8; ++emax)
        for (int e = -140; e <= 128; e += 3) (void)or_e8m0_block_code_emax((float)ldexp(1.3, e), emax);
    (void)or_e8m0_block_code_emax(0.0f, 2);

    /* counter-based generator across the 64-bit counter range */
    {
        const uint32_t ctr[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu}, key[2] = {1u, 2u};
        uint32_t out[4];
        or_philox4x32_10(ctr, key, out);
        volatile uint32_t t = out[0];
        for (uint64_t i = 0; i < 64; ++i) t ^= or_sr_bits(~0ull - i, ~0ull - 3 * i, ~0ull - 7 * i);
        (void)t;
    }
    free(xf);
    free(xb);
    printf("oracle sanitize driver: ok\n");
    return 0;
}
