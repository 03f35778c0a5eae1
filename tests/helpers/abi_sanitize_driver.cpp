// Drives the host side of the C-ABI library's argument checks, for a build
// with AddressSanitizer and UndefinedBehaviorSanitizer and no GPU: every
// call below is rejected before the library touches the HIP runtime, so the
// pointers it is given (host buffers standing in for device memory) are
// never dereferenced on a device.  Exit status: the number of calls that
// did not return the expected status; the sanitizers abort on a finding.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "fp4.h"

static int failures = 0;

static void expect(const char* what, fp4_status got, fp4_status want)
{
    if (got != want) {
        std::fprintf(stderr, "%s: got %d (%s), want %d\n", what, (int)got, fp4_status_string(got), (int)want);
        ++failures;
    }
}

alignas(64) static uint8_t q_buf[1 << 16];
alignas(64) static uint8_t s_buf[1 << 12];
alignas(64) static float g_buf[4];
alignas(64) static float x_buf[1 << 14];
alignas(64) static uint16_t y_buf[1 << 14];

static fp4_tensor tensor(int64_t rows, int64_t cols, int block, int scale, int amax, int elem = FP4_ELEM_E2M1)
{
    fp4_tensor t;
    std::memset(&t, 0, sizeof(t));
    t.q = q_buf;
    t.scales = s_buf;
    t.tensor_scale = g_buf;
    t.rows = rows;
    t.cols = cols;
    t.fmt.block = block;
    t.fmt.scale = scale;
    t.fmt.rounding = FP4_ROUND_NEAREST_EVEN;
    t.fmt.amax = amax;
    t.fmt.transform = FP4_TRANSFORM_NONE;
    t.fmt.element = elem;
    return t;
}

int main()
{
    (void)fp4_version();
    for (int s = -8; s <= 2; ++s)
        if (!fp4_status_string((fp4_status)s)) ++failures;
    uint64_t prev = 0;
    expect("set exchange wait", fp4_set_exchange_wait(123, &prev), FP4_OK);
    expect("restore exchange wait", fp4_set_exchange_wait(prev, nullptr), FP4_OK);
    int64_t prev_small = 0;
    expect("set small-product bound", fp4_set_gemm_small_outputs(7, &prev_small), FP4_OK);
    expect("negative small-product bound", fp4_set_gemm_small_outputs(-1, nullptr), FP4_ERR_INVALID_ARG);
    expect("restore small-product bound", fp4_set_gemm_small_outputs(prev_small, nullptr), FP4_OK);

    fp4_amax_state* st = nullptr;
    expect("state interval 0", fp4_amax_state_create(0, &st), FP4_ERR_INVALID_ARG);
    expect("state null out", fp4_amax_state_create(50, nullptr), FP4_ERR_INVALID_ARG);
    expect("destroy null", fp4_amax_state_destroy(nullptr), FP4_ERR_INVALID_ARG);
    uint64_t calls;
    float amax;
    uint32_t nfb;
    expect("get null", fp4_amax_state_get(nullptr, &calls, &amax), FP4_ERR_INVALID_ARG);
    expect("set null", fp4_amax_state_set(nullptr, 0, 1.0f), FP4_ERR_INVALID_ARG);
    expect("fallbacks null", fp4_amax_state_fallbacks(nullptr, &nfb), FP4_ERR_INVALID_ARG);

    // quantize: each rejected before any launch
    fp4_tensor t = tensor(64, 256, 16, FP4_SCALE_E4M3, FP4_AMAX_NONE);
    expect("quantize null out", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, nullptr, nullptr, 0, 0, nullptr),
           FP4_ERR_INVALID_ARG);
    expect("quantize null x", fp4_quantize(nullptr, FP4_DTYPE_F32, 256, &t, nullptr, 0, 0, nullptr),
           FP4_ERR_INVALID_ARG);
    expect("quantize bad dtype", fp4_quantize(x_buf, 7, 256, &t, nullptr, 0, 0, nullptr), FP4_ERR_INVALID_ARG);
    expect("quantize ld < cols", fp4_quantize(x_buf, FP4_DTYPE_F32, 255, &t, nullptr, 0, 0, nullptr),
           FP4_ERR_SHAPE);
    expect("quantize misaligned x", fp4_quantize(x_buf + 1, FP4_DTYPE_F32, 256, &t, nullptr, 0, 0, nullptr),
           FP4_ERR_ALIGN);
    expect("quantize misaligned ld", fp4_quantize(x_buf, FP4_DTYPE_BF16, 260, &t, nullptr, 0, 0, nullptr),
           FP4_ERR_ALIGN);
    {
        fp4_tensor u = t;
        u.fmt.block = 24;
        expect("quantize block 24", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_INVALID_ARG);
        u = t;
        u.fmt.scale = 99;
        expect("quantize scale 99", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_INVALID_ARG);
        u = t;
        u.fmt.element = 7;
        expect("quantize element 7", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_INVALID_ARG);
        u = t;
        u.fmt.rounding = 2;
        expect("quantize rounding 2", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_INVALID_ARG);
        u = t;
        u.fmt.transform = 5;
        expect("quantize transform 5", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_INVALID_ARG);
        u = t;
        u.cols = 250;
        expect("quantize cols % block", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_SHAPE);
        u = t;
        u.rows = -1;
        expect("quantize rows < 0", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_SHAPE);
        u = t;
        u.rows = int64_t(1) << 40;
        expect("quantize too large", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_SHAPE);
        u = t;
        u.q = q_buf + 2;
        expect("quantize misaligned q", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_ALIGN);
        u = t;
        u.tensor_scale = nullptr;
        expect("quantize null g", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_INVALID_ARG);
        u = tensor(64, 256, 32, FP4_SCALE_E8M0, FP4_AMAX_CURRENT);
        expect("quantize e8m0 current", fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr),
               FP4_ERR_UNSUPPORTED);
        u = tensor(64, 256, 16, FP4_SCALE_E4M3, FP4_AMAX_CURRENT);
        expect("quantize current without state",
               fp4_quantize(x_buf, FP4_DTYPE_F32, 256, &u, nullptr, 0, 0, nullptr), FP4_ERR_INVALID_ARG);
        u = tensor(64, 256, 16, FP4_SCALE_E4M3, FP4_AMAX_DELAYED);
        expect("noalloc delayed", fp4_quantize_noalloc(x_buf, FP4_DTYPE_F32, 256, &u, 0, 0, nullptr),
               FP4_ERR_UNSUPPORTED);
        expect("noalloc null x", fp4_quantize_noalloc(nullptr, FP4_DTYPE_F32, 256, &t, 0, 0, nullptr),
               FP4_ERR_INVALID_ARG);
    }
    // column-wise and two-orientation calls
    {
        fp4_tensor c = tensor(256, 64, 16, FP4_SCALE_E4M3, FP4_AMAX_NONE);
        expect("transposed ld < rows", fp4_quantize_transposed(x_buf, FP4_DTYPE_F32, 200, &c, nullptr, 0, 0, nullptr),
               FP4_ERR_SHAPE);
        fp4_tensor c6 = tensor(256, 64, 32, FP4_SCALE_E8M0, FP4_AMAX_NONE, FP4_ELEM_FP6_E2M3);
        c6.q = q_buf;
        c6.cols = 96;
        expect("transposed 6-bit cols % 64",
               fp4_quantize_transposed(x_buf, FP4_DTYPE_F32, 256, &c6, nullptr, 0, 0, nullptr), FP4_ERR_SHAPE);
        fp4_tensor r = tensor(64, 256, 16, FP4_SCALE_E4M3, FP4_AMAX_NONE);
        fp4_tensor bad = tensor(128, 64, 16, FP4_SCALE_E4M3, FP4_AMAX_NONE);
        expect("both shape mismatch", fp4_quantize_both(x_buf, FP4_DTYPE_F32, 256, &r, &bad, nullptr, 0, 0, nullptr),
               FP4_ERR_SHAPE);
        fp4_tensor c2 = c;
        c2.fmt.scale = FP4_SCALE_UE5M3;
        expect("both format mismatch", fp4_quantize_both(x_buf, FP4_DTYPE_F32, 256, &r, &c2, nullptr, 0, 0, nullptr),
               FP4_ERR_UNSUPPORTED);
        fp4_tensor r6 = tensor(96, 64, 32, FP4_SCALE_E8M0, FP4_AMAX_NONE, FP4_ELEM_FP6_E2M3);
        fp4_tensor c6b = tensor(64, 96, 32, FP4_SCALE_E8M0, FP4_AMAX_NONE, FP4_ELEM_FP6_E2M3);
        r6.q = q_buf;
        c6b.q = q_buf;
        expect("both 6-bit R % 64", fp4_quantize_both(x_buf, FP4_DTYPE_F32, 64, &r6, &c6b, nullptr, 0, 0, nullptr),
               FP4_ERR_SHAPE);
    }
    // dequantize, GEMM, weight-only GEMM
    {
        expect("dequantize bad dtype", fp4_dequantize(&t, y_buf, 9, 256, nullptr), FP4_ERR_INVALID_ARG);
        expect("dequantize null y", fp4_dequantize(&t, nullptr, FP4_DTYPE_BF16, 256, nullptr), FP4_ERR_INVALID_ARG);
        expect("dequantize ld < cols", fp4_dequantize(&t, y_buf, FP4_DTYPE_BF16, 128, nullptr), FP4_ERR_SHAPE);
        fp4_tensor a = tensor(64, 256, 16, FP4_SCALE_E4M3, FP4_AMAX_CURRENT);
        fp4_tensor b = tensor(32, 512, 16, FP4_SCALE_E4M3, FP4_AMAX_CURRENT);
        expect("gemm K mismatch", fp4_gemm(&a, &b, y_buf, 32, nullptr), FP4_ERR_SHAPE);
        fp4_tensor b2 = tensor(32, 256, 32, FP4_SCALE_E8M0, FP4_AMAX_NONE);
        expect("gemm block mismatch", fp4_gemm(&a, &b2, y_buf, 32, nullptr), FP4_ERR_UNSUPPORTED);
        fp4_tensor b3 = tensor(32, 256, 16, FP4_SCALE_E4M3, FP4_AMAX_CURRENT);
        expect("gemm ldc < N", fp4_gemm(&a, &b3, y_buf, 16, nullptr), FP4_ERR_SHAPE);
        expect("gemm null c", fp4_gemm(&a, &b3, nullptr, 32, nullptr), FP4_ERR_INVALID_ARG);
        expect("wo null w", fp4_wo_gemm(y_buf, 256, 4, nullptr, y_buf, 64, nullptr), FP4_ERR_INVALID_ARG);
        expect("wo m 17", fp4_wo_gemm(y_buf, 256, 17, &b3, y_buf, 64, nullptr), FP4_ERR_UNSUPPORTED);
    }
    if (failures) std::fprintf(stderr, "abi sanitize driver: %d unexpected statuses\n", failures);
    else std::printf("abi sanitize driver: ok\n");
    return failures;
}
