// api.cpp -- the C ABI declared in include/fp4.h: argument validation,
// amax-policy bookkeeping on the host and kernel launches on the caller's
// stream.  Nothing here computes on the host: every step of the quantize,
// dequantize and GEMM paths runs in the HIP kernels.
#include "fp4.h"

#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <new>

#include "fp4_internal.h"

namespace fp4 {

// ExMy (sign + x + y = 8 bits) and UE5M3: bias 2^(x-1)-1; the all-ones code
// is NaN, so the largest finite code is all ones minus one.  E8M0: 2^(c-127).
bool scale_fmt_params(int32_t fmt, ScaleFmtHost* out)
{
    int e = 0, m = 0, e8 = 0;
    switch (fmt) {
    case FP4_SCALE_E4M3: e = 4; m = 3; break;
    case FP4_SCALE_UE5M3: e = 5; m = 3; break;
    case FP4_SCALE_E3M4: e = 3; m = 4; break;
    case FP4_SCALE_E1M6: e = 1; m = 6; break;
    case FP4_SCALE_E2M5: e = 2; m = 5; break;
    case FP4_SCALE_E5M2: e = 5; m = 2; break;
    case FP4_SCALE_E6M1: e = 6; m = 1; break;
    case FP4_SCALE_E7M0: e = 7; m = 0; break;
    case FP4_SCALE_E8M0: e8 = 1; break;
    default: return false;
    }
    ScaleFmtHost f{};
    f.is_e8m0 = e8;
    if (e8) {
        f.ebits = 8; f.mbits = 0; f.bias = 127; f.maxcode = 254;
        f.smax = ldexpf(1.0f, 127);
    } else {
        f.ebits = e; f.mbits = m;
        f.bias = (1 << (e - 1)) - 1;
        f.maxcode = (1 << (e + m)) - 2;
        const int ecode = f.maxcode >> m, mcode = f.maxcode & ((1 << m) - 1);
        f.smax = ldexpf((float)(mcode | (1 << m)), ecode - f.bias - m);
    }
    *out = f;
    return true;
}

}  // namespace fp4

using namespace fp4;

struct fp4_amax_state {
    uint32_t interval;
    uint64_t calls;
    int device;
    AmaxDev* dev;
};

extern "C" {

int32_t fp4_version(void) { return 107; }

const char* fp4_status_string(fp4_status st)
{
    switch (st) {
    case FP4_OK: return "ok";
    case FP4_ERR_INVALID_ARG: return "invalid argument";
    case FP4_ERR_UNSUPPORTED: return "unsupported combination";
    case FP4_ERR_SHAPE: return "shape mismatch";
    case FP4_ERR_ALIGN: return "misaligned pointer or leading dimension";
    case FP4_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

fp4_status fp4_amax_state_create(uint32_t interval, fp4_amax_state** out)
{
    if (!out || interval == 0) return FP4_ERR_INVALID_ARG;
    fp4_amax_state* st = new (std::nothrow) fp4_amax_state;
    if (!st) return FP4_ERR_INVALID_ARG;
    st->interval = interval;
    st->calls = 0;
    if (hipGetDevice(&st->device) != hipSuccess) { delete st; return FP4_ERR_HIP; }
    if (hipMalloc((void**)&st->dev, sizeof(AmaxDev)) != hipSuccess) { delete st; return FP4_ERR_HIP; }
    AmaxDev zero{};
    if (hipMemcpy(st->dev, &zero, sizeof(zero), hipMemcpyHostToDevice) != hipSuccess) {
        (void)hipFree(st->dev);
        delete st;
        return FP4_ERR_HIP;
    }
    *out = st;
    return FP4_OK;
}

fp4_status fp4_amax_state_destroy(fp4_amax_state* st)
{
    if (!st) return FP4_ERR_INVALID_ARG;
    hipError_t e = hipFree(st->dev);
    delete st;
    return e == hipSuccess ? FP4_OK : FP4_ERR_HIP;
}

fp4_status fp4_amax_state_get(const fp4_amax_state* st, uint64_t* calls, float* amax)
{
    if (!st || !calls || !amax) return FP4_ERR_INVALID_ARG;
    if (hipDeviceSynchronize() != hipSuccess) return FP4_ERR_HIP;
    AmaxDev h;
    if (hipMemcpy(&h, st->dev, sizeof(h), hipMemcpyDeviceToHost) != hipSuccess) return FP4_ERR_HIP;
    *calls = st->calls;
    *amax = h.stored;
    return FP4_OK;
}

fp4_status fp4_amax_state_fallbacks(const fp4_amax_state* st, uint32_t* n)
{
    if (!st || !n) return FP4_ERR_INVALID_ARG;
    if (hipDeviceSynchronize() != hipSuccess) return FP4_ERR_HIP;
    if (hipMemcpy(n, &st->dev->fallbacks, sizeof(*n), hipMemcpyDeviceToHost) != hipSuccess) return FP4_ERR_HIP;
    return FP4_OK;
}

fp4_status fp4_set_exchange_wait(uint64_t ticks, uint64_t* previous)
{
    const uint64_t old = __atomic_exchange_n(&g_exchange_wait_ticks, ticks, __ATOMIC_RELAXED);
    if (previous) *previous = old;
    return FP4_OK;
}

fp4_status fp4_set_gemm_small_outputs(int64_t outputs, int64_t* previous)
{
    if (outputs < 0) return FP4_ERR_INVALID_ARG;
    const int64_t old = __atomic_exchange_n(&g_gemm_small_outputs, outputs, __ATOMIC_RELAXED);
    if (previous) *previous = old;
    return FP4_OK;
}

fp4_status fp4_amax_state_set(fp4_amax_state* st, uint64_t calls, float amax)
{
    if (!st || !(amax >= 0.0f) || !isfinite(amax)) return FP4_ERR_INVALID_ARG;
    if (hipDeviceSynchronize() != hipSuccess) return FP4_ERR_HIP;
    AmaxDev h{};
    h.stored = amax;
    if (hipMemcpy(st->dev, &h, sizeof(h), hipMemcpyHostToDevice) != hipSuccess) return FP4_ERR_HIP;
    st->calls = calls;
    return FP4_OK;
}

static bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
static bool elem_is_8bit(int32_t e) { return e == FP4_ELEM_FP8_E4M3 || e == FP4_ELEM_INT8; }
static bool elem_is_6bit(int32_t e) { return e >= FP4_ELEM_FP6_E2M3 && e <= FP4_ELEM_INT6; }
// the 8- and 6-bit grids: no two-orientation call and no weight-only GEMM
static bool elem_is_wide(int32_t e) { return elem_is_8bit(e) || elem_is_6bit(e); }

static fp4_status check_tensor(const fp4_tensor* t, ScaleFmtHost* f)
{
    if (!t || !t->tensor_scale) return FP4_ERR_INVALID_ARG;
    const bool empty = t->rows == 0 || t->cols == 0;
    if (!empty && (!t->q || !t->scales)) return FP4_ERR_INVALID_ARG;
    if (t->fmt.block != 16 && t->fmt.block != 32) return FP4_ERR_INVALID_ARG;
    if (t->fmt.rounding != FP4_ROUND_NEAREST_EVEN && t->fmt.rounding != FP4_ROUND_STOCHASTIC)
        return FP4_ERR_INVALID_ARG;
    if (t->fmt.amax != FP4_AMAX_NONE && t->fmt.amax != FP4_AMAX_CURRENT && t->fmt.amax != FP4_AMAX_DELAYED)
        return FP4_ERR_INVALID_ARG;
    if (!scale_fmt_params(t->fmt.scale, f)) return FP4_ERR_INVALID_ARG;
    if (t->fmt.transform != FP4_TRANSFORM_NONE && t->fmt.transform != FP4_TRANSFORM_RHT) return FP4_ERR_INVALID_ARG;
    if (t->fmt.element < FP4_ELEM_E2M1 || t->fmt.element > FP4_ELEM_INT6) return FP4_ERR_INVALID_ARG;
    if (t->rows < 0 || t->cols < 0) return FP4_ERR_SHAPE;
    if (t->cols % t->fmt.block) return FP4_ERR_SHAPE;
    // codes leave as 4-byte pieces (4-bit grids), 8-byte pieces (8-bit
    // grids) or 2-byte pieces at 6-byte steps (6-bit grids; 8-byte alignment
    // asked for as for 8 bits)
    if (((uintptr_t)t->q & (elem_is_wide(t->fmt.element) ? 7u : 3u)) != 0) return FP4_ERR_ALIGN;
    if ((t->rows * (t->cols / 8)) >= (int64_t(1) << 31)) return FP4_ERR_SHAPE;
    return FP4_OK;
}

static fp4_status hip_status(hipError_t e) { return e == hipSuccess ? FP4_OK : FP4_ERR_HIP; }

// Checks of fp4_quantize's arguments other than the amax state.
static fp4_status check_quantize_args(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* out,
                                      ScaleFmtHost* f)
{
    fp4_status st = check_tensor(out, f);
    if (st != FP4_OK) return st;
    if (!x && out->rows * out->cols != 0) return FP4_ERR_INVALID_ARG;
    if (x_dtype != FP4_DTYPE_F32 && x_dtype != FP4_DTYPE_BF16) return FP4_ERR_INVALID_ARG;
    const int64_t esz = x_dtype == FP4_DTYPE_BF16 ? 2 : 4;
    if (ld_x < out->cols) return FP4_ERR_SHAPE;
    // an empty x is never read (a [rows, 0] tensor may carry row stride 1)
    if (out->rows * out->cols != 0 && (!aligned16(x) || (ld_x * esz) % 16)) return FP4_ERR_ALIGN;
    if (f->is_e8m0 && out->fmt.amax != FP4_AMAX_NONE) return FP4_ERR_UNSUPPORTED;
    return FP4_OK;
}

// The row-wise quantize launch with the amax workspace `src` (null under
// NONE) and whether this call takes its own tensor maximum.
static fp4_status quantize_launch(const void* x, int32_t x_dtype, int64_t ld_x, const fp4_tensor* out,
                                  const ScaleFmtHost& f, AmaxDev* src, bool refresh, uint64_t seed, uint64_t offset,
                                  hipStream_t s)
{
    QuantLaunch p;
    p.x = x;
    p.x_bf16 = x_dtype == FP4_DTYPE_BF16;
    p.rows = out->rows;
    p.cols = out->cols;
    p.ld = ld_x;
    p.q = out->q;
    p.scales = out->scales;
    p.tensor_scale = out->tensor_scale;
    p.amax_src = src;
    p.refresh = refresh;
    p.block = out->fmt.block;
    p.stochastic = out->fmt.rounding == FP4_ROUND_STOCHASTIC;
    p.seed = seed;
    p.offset = offset;
    p.fmt = f;
    p.rht = out->fmt.transform == FP4_TRANSFORM_RHT;
    p.rht_signs = out->fmt.transform_signs;
    p.elem = out->fmt.element;
    return hip_status(launch_quantize(p, s));
}

fp4_status fp4_quantize(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* out, fp4_amax_state* state,
                        uint64_t seed, uint64_t offset, void* stream)
{
    ScaleFmtHost f;
    fp4_status st = check_quantize_args(x, x_dtype, ld_x, out, &f);
    if (st != FP4_OK) return st;
    const int32_t pol = out->fmt.amax;
    if (pol != FP4_AMAX_NONE && !state) return FP4_ERR_INVALID_ARG;
    AmaxDev* src = nullptr;
    bool refresh = false;
    if (pol != FP4_AMAX_NONE) {
        refresh = (pol == FP4_AMAX_CURRENT) || (state->calls % state->interval == 0);
        src = state->dev;
    }
    st = quantize_launch(x, x_dtype, ld_x, out, f, src, refresh, seed, offset, (hipStream_t)stream);
    if (st == FP4_OK && state && pol != FP4_AMAX_NONE) state->calls += 1;
    return st;
}

// ---------------------------------------------------------------------------
// fp4_quantize_noalloc: the amax workspace of a current-amax call lives in
// this static device array instead of an fp4_amax_state.  Its size does not
// depend on the tensor: the single-pass refresh uses at most kXchgSlots
// exchange words and the two-pass refresh exactly kAmaxParts partials.  It
// is zero at load; each single-pass launch publishes every slot with its
// epoch and the two-pass refresh overwrites every partial, so nothing needs
// clearing per call.  Host code uses the address hipGetSymbolAddress returns for the
// current device, never the array's own (host-side) name.
// ---------------------------------------------------------------------------
constexpr size_t kScratchBytes = sizeof(AmaxDev);
static __device__ __align__(256) uint8_t scratch[kScratchBytes];
constexpr int kMaxDevices = 64;
static std::atomic<AmaxDev*> g_scratch_ptr[kMaxDevices];

static fp4_status scratch_of_current_device(AmaxDev** out)
{
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) return FP4_ERR_HIP;
    if (dev < 0 || dev >= kMaxDevices) return FP4_ERR_UNSUPPORTED;
    AmaxDev* p = g_scratch_ptr[dev].load(std::memory_order_acquire);
    if (!p) {
        void* a = nullptr;
        if (hipGetSymbolAddress(&a, HIP_SYMBOL(scratch)) != hipSuccess || !a) return FP4_ERR_HIP;
        p = static_cast<AmaxDev*>(a);
        g_scratch_ptr[dev].store(p, std::memory_order_release);
    }
    *out = p;
    return FP4_OK;
}

fp4_status fp4_quantize_noalloc(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* out, uint64_t seed,
                                uint64_t offset, void* stream)
{
    ScaleFmtHost f;
    fp4_status st = check_quantize_args(x, x_dtype, ld_x, out, &f);
    if (st != FP4_OK) return st;
    const int32_t pol = out->fmt.amax;
    if (pol == FP4_AMAX_DELAYED) return FP4_ERR_UNSUPPORTED;   // the stored maximum belongs to one tensor
    AmaxDev* src = nullptr;
    if (pol == FP4_AMAX_CURRENT) {
        st = scratch_of_current_device(&src);
        if (st != FP4_OK) return st;
    }
    return quantize_launch(x, x_dtype, ld_x, out, f, src, pol == FP4_AMAX_CURRENT, seed, offset,
                           (hipStream_t)stream);
}

fp4_status fp4_quantize_transposed(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* out,
                                   fp4_amax_state* state, uint64_t seed, uint64_t offset, void* stream)
{
    ScaleFmtHost f;
    fp4_status st = check_tensor(out, &f);
    if (st != FP4_OK) return st;
    if (!x && out->rows * out->cols != 0) return FP4_ERR_INVALID_ARG;
    if (x_dtype != FP4_DTYPE_F32 && x_dtype != FP4_DTYPE_BF16) return FP4_ERR_INVALID_ARG;
    const int64_t esz = x_dtype == FP4_DTYPE_BF16 ? 2 : 4;
    // x is [out->cols, out->rows]: its rows are the blocked dimension
    // 6-bit codes: whole 16-byte output chunks need R % 64 == 0
    if (elem_is_6bit(out->fmt.element) && out->cols % 64) return FP4_ERR_SHAPE;
    if (out->rows % 8) return FP4_ERR_SHAPE;
    if (out->rows * out->cols != 0) {
        if (ld_x < out->rows) return FP4_ERR_SHAPE;
        if (!aligned16(x) || (ld_x * esz) % 16 || !aligned16(out->q)) return FP4_ERR_ALIGN;
    }
    const int32_t pol = out->fmt.amax;
    if (f.is_e8m0 && pol != FP4_AMAX_NONE) return FP4_ERR_UNSUPPORTED;
    if (pol != FP4_AMAX_NONE && !state) return FP4_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;

    AmaxDev* src = nullptr;
    bool refresh = false;
    if (pol != FP4_AMAX_NONE) {
        refresh = (pol == FP4_AMAX_CURRENT) || (state->calls % state->interval == 0);
        src = state->dev;
    }
    QuantLaunch p;
    p.x = x;
    p.x_bf16 = x_dtype == FP4_DTYPE_BF16;
    p.rows = out->rows;
    p.cols = out->cols;
    p.ld = ld_x;
    p.q = out->q;
    p.scales = out->scales;
    p.tensor_scale = out->tensor_scale;
    p.amax_src = src;
    p.refresh = refresh;
    p.block = out->fmt.block;
    p.stochastic = out->fmt.rounding == FP4_ROUND_STOCHASTIC;
    p.seed = seed;
    p.offset = offset;
    p.fmt = f;
    p.rht = out->fmt.transform == FP4_TRANSFORM_RHT;
    p.rht_signs = out->fmt.transform_signs;
    p.elem = out->fmt.element;
    st = hip_status(launch_quantize_t(p, s));
    if (st == FP4_OK && state && pol != FP4_AMAX_NONE) state->calls += 1;
    return st;
}

fp4_status fp4_quantize_both(const void* x, int32_t x_dtype, int64_t ld_x, fp4_tensor* rowwise,
                             fp4_tensor* colwise, fp4_amax_state* state, uint64_t seed, uint64_t offset,
                             void* stream)
{
    ScaleFmtHost f, fc;
    fp4_status st = check_tensor(rowwise, &f);
    if (st != FP4_OK) return st;
    st = check_tensor(colwise, &fc);
    if (st != FP4_OK) return st;
    if (rowwise->rows != colwise->cols || rowwise->cols != colwise->rows) return FP4_ERR_SHAPE;
    const fp4_format &fr = rowwise->fmt, &fl = colwise->fmt;
    if (fr.block != fl.block || fr.scale != fl.scale || fr.rounding != fl.rounding || fr.amax != fl.amax ||
        fr.element != fl.element)
        return FP4_ERR_UNSUPPORTED;
    // a transform would run along different axes, with different maxima
    if (fr.transform != FP4_TRANSFORM_NONE || fl.transform != FP4_TRANSFORM_NONE) return FP4_ERR_UNSUPPORTED;
    // 6-bit codes: whole 16-byte column-wise output chunks need R % 64 == 0
    if (elem_is_6bit(fr.element) && colwise->cols % 64) return FP4_ERR_SHAPE;
    if (!x && rowwise->rows * rowwise->cols != 0) return FP4_ERR_INVALID_ARG;
    if (x_dtype != FP4_DTYPE_F32 && x_dtype != FP4_DTYPE_BF16) return FP4_ERR_INVALID_ARG;
    const int64_t esz = x_dtype == FP4_DTYPE_BF16 ? 2 : 4;
    if (rowwise->rows * rowwise->cols != 0) {
        if (ld_x < rowwise->cols) return FP4_ERR_SHAPE;
        if (!aligned16(x) || (ld_x * esz) % 16 || !aligned16(colwise->q)) return FP4_ERR_ALIGN;
    }
    const int32_t pol = fr.amax;
    if (f.is_e8m0 && pol != FP4_AMAX_NONE) return FP4_ERR_UNSUPPORTED;
    if (pol != FP4_AMAX_NONE && !state) return FP4_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;

    AmaxDev* src = nullptr;
    bool refresh = false;
    if (pol != FP4_AMAX_NONE) {
        refresh = (pol == FP4_AMAX_CURRENT) || (state->calls % state->interval == 0);
        src = state->dev;
    }
    QuantLaunch p;
    p.x = x;
    p.x_bf16 = x_dtype == FP4_DTYPE_BF16;
    p.rows = colwise->rows;
    p.cols = colwise->cols;
    p.ld = ld_x;
    p.q = colwise->q;
    p.scales = colwise->scales;
    p.tensor_scale = colwise->tensor_scale;
    p.amax_src = src;
    p.refresh = refresh;
    p.block = fr.block;
    p.stochastic = fr.rounding == FP4_ROUND_STOCHASTIC;
    p.seed = seed;
    p.offset = offset;
    p.fmt = f;
    p.rht = 0;
    p.rht_signs = 0;
    p.elem = fr.element;
    const RowOut ro{rowwise->q, rowwise->scales, rowwise->tensor_scale};
    st = hip_status(launch_quantize_t(p, s, &ro));
    if (st == FP4_OK && state && pol != FP4_AMAX_NONE) state->calls += 1;
    return st;
}

fp4_status fp4_dequantize(const fp4_tensor* in, void* y, int32_t y_dtype, int64_t ld_y, void* stream)
{
    ScaleFmtHost f;
    fp4_status st = check_tensor(in, &f);
    if (st != FP4_OK) return st;
    if (y_dtype != FP4_DTYPE_F32 && y_dtype != FP4_DTYPE_BF16) return FP4_ERR_INVALID_ARG;
    if (in->rows * in->cols == 0) return FP4_OK;
    if (!y) return FP4_ERR_INVALID_ARG;
    const int64_t esz = y_dtype == FP4_DTYPE_BF16 ? 2 : 4;
    if (ld_y < in->cols) return FP4_ERR_SHAPE;
    if (!aligned16(y) || (ld_y * esz) % 16) return FP4_ERR_ALIGN;
    DequantLaunch p;
    p.q = in->q;
    p.scales = in->scales;
    p.tensor_scale = in->tensor_scale;
    p.rows = in->rows;
    p.cols = in->cols;
    p.block = in->fmt.block;
    p.fmt = f;
    p.y = y;
    p.y_bf16 = y_dtype == FP4_DTYPE_BF16;
    p.ld = ld_y;
    p.rht = in->fmt.transform == FP4_TRANSFORM_RHT;
    p.rht_signs = in->fmt.transform_signs;
    p.elem = in->fmt.element;
    return hip_status(launch_dequantize(p, (hipStream_t)stream));
}

fp4_status fp4_gemm(const fp4_tensor* a, const fp4_tensor* b, uint16_t* c, int64_t ldc, void* stream)
{
    ScaleFmtHost fa, fb;
    fp4_status st = check_tensor(a, &fa);
    if (st != FP4_OK) return st;
    st = check_tensor(b, &fb);
    if (st != FP4_OK) return st;
    if (!c) return FP4_ERR_INVALID_ARG;
    if (a->cols != b->cols) return FP4_ERR_SHAPE;
    if (a->fmt.block != b->fmt.block) return FP4_ERR_UNSUPPORTED;
    // transformed operands multiply to the same product only when both carry
    // the same transform along K
    if (a->fmt.element != b->fmt.element) return FP4_ERR_UNSUPPORTED;
    if (a->fmt.transform != b->fmt.transform) return FP4_ERR_UNSUPPORTED;
    if (a->fmt.transform != FP4_TRANSFORM_NONE && a->fmt.transform_signs != b->fmt.transform_signs)
        return FP4_ERR_UNSUPPORTED;
    if (a->cols % 128) return FP4_ERR_SHAPE;
    if (ldc < b->rows) return FP4_ERR_SHAPE;
    if (((uintptr_t)c & 1u) != 0) return FP4_ERR_ALIGN;
    if (a->rows == 0 || b->rows == 0) return FP4_OK;
    // an empty K: C is the empty sum, zero; no operand is read
    if (a->cols == 0) return hip_status(launch_fill_zero_bf16(c, ldc, a->rows, b->rows, (hipStream_t)stream));
    if (!aligned16(a->q) || !aligned16(b->q) || ((uintptr_t)a->scales & 3u) || ((uintptr_t)b->scales & 3u))
        return FP4_ERR_ALIGN;
    GemmLaunch p;
    p.qa = a->q; p.sa = a->scales; p.ga = a->tensor_scale;
    p.qb = b->q; p.sb = b->scales; p.gb = b->tensor_scale;
    p.m = a->rows; p.n = b->rows; p.k = a->cols;
    p.block = a->fmt.block;
    p.fa = fa; p.fb = fb;
    p.c = c; p.ldc = ldc;
    p.elem = a->fmt.element;
    hipStream_t s = (hipStream_t)stream;
    if (gemm_small_supported(p)) return hip_status(launch_gemm_small(p, s));
    if (p.elem == FP4_ELEM_E2M1 && fa.is_e8m0 && fb.is_e8m0 && p.block == 32) return hip_status(launch_gemm_mx(p, s));
    if (gemm_mx16_supported(p)) return hip_status(launch_gemm_mx16(p, s));
    if (!gemm_dq_supported(fa, fb, p.elem)) return FP4_ERR_UNSUPPORTED;
    return hip_status(launch_gemm_dq(p, s));
}

fp4_status fp4_wo_gemm(const uint16_t* x, int64_t ldx, int64_t m, const fp4_tensor* w, uint16_t* y, int64_t ldy,
                       void* stream)
{
    ScaleFmtHost fw;
    fp4_status st = check_tensor(w, &fw);
    if (st != FP4_OK) return st;
    if (!y || (!x && w->cols != 0)) return FP4_ERR_INVALID_ARG;
    if (m < 1 || m > 16) return FP4_ERR_UNSUPPORTED;
    if (w->fmt.transform != FP4_TRANSFORM_NONE) return FP4_ERR_UNSUPPORTED;   // x would need the same transform
    if (w->cols % 256) return FP4_ERR_SHAPE;
    if (ldx < w->cols || ldy < w->rows) return FP4_ERR_SHAPE;
    if (w->rows == 0) return FP4_OK;
    // an empty K: Y is the empty sum, zero; neither x nor W is read
    if (w->cols == 0) return hip_status(launch_fill_zero_bf16(y, ldy, m, w->rows, (hipStream_t)stream));
    // the kernel addresses W and x with 32-bit byte/element offsets
    const int64_t wbits = elem_is_8bit(w->fmt.element) ? 8 : elem_is_6bit(w->fmt.element) ? 6 : 4;
    if (w->rows * (w->cols * wbits / 8) >= (int64_t(1) << 32) || ldx * m >= (int64_t(1) << 31))
        return FP4_ERR_UNSUPPORTED;
    if (!aligned16(x) || ldx % 8) return FP4_ERR_ALIGN;
    if (!aligned16(w->q) || ((uintptr_t)w->scales & 3u)) return FP4_ERR_ALIGN;
    WoGemmLaunch p;
    p.x = x; p.ldx = ldx; p.m = m;
    p.qw = w->q; p.sw = w->scales; p.gw = w->tensor_scale;
    p.n = w->rows; p.k = w->cols;
    p.elem = w->fmt.element;
    p.block = w->fmt.block;
    p.fw = fw;
    p.y = y; p.ldy = ldy;
    return hip_status(launch_wo_gemm(p, (hipStream_t)stream));
}

}  // extern "C"
