// fp4_internal.h -- host-side launcher interface between the C ABI (api.cpp)
// and the kernel translation units.  Launchers assume validated arguments.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4 {

struct ScaleFmtHost {
    int32_t ebits, mbits, bias, maxcode;
    float smax;
    int32_t is_e8m0;
};

// Fill the parameters of a block-scale format (fp4_scale_fmt value).
bool scale_fmt_params(int32_t fmt, ScaleFmtHost* out);

// Device workspace of an amax state.
//  - partial/stored: the two-kernel refresh (tensors larger than the fused
//    path holds in registers) writes one partial maximum per workgroup of
//    the amax kernel; the quantize kernel of the same call reduces them and
//    stores the result in `stored`, which calls between refreshes read.
//  - slot: the single-pass refresh exchanges per-workgroup maxima through
//    `slot` (64-bit {epoch, max bits} words, one per 64-byte segment so that
//    stores of different workgroups never share a line) within one launch.
//    Every single-pass launch that exchanges runs the same grid and
//    publishes every slot (a grid of one writes none), so a workgroup's own
//    slot holds the previous exchanging launch's epoch, and that + 1 is
//    this launch's.
//  - fallbacks: number of workgroups that did not see every other
//    workgroup's maximum within the wait bound and read the whole tensor
//    themselves instead (the result is the same either way).
constexpr int kAmaxParts = 256;
constexpr int kXchgSlots = 256;
constexpr int kXchgStride = 8;          // 64-bit words between slots (64 bytes)
struct AmaxDev {
    float partial[kAmaxParts];
    float stored;
    uint32_t reserved;
    uint32_t fallbacks;
    uint32_t reserved2;
    uint32_t pad[60];
    uint64_t slot[kXchgSlots * kXchgStride];
};
static_assert(sizeof(AmaxDev) == 17664, "amax state layout");

struct QuantLaunch {
    const void* x;
    int32_t x_bf16;
    int64_t rows, cols, ld;
    uint8_t* q;
    uint8_t* scales;
    float* tensor_scale;       // out: {g, amax}
    AmaxDev* amax_src;         // null: no tensor scale (g = 1)
    int32_t refresh;           // compute this call's maximum (else read amax_src->stored)
    int32_t block;
    int32_t stochastic;
    uint64_t seed, offset;
    ScaleFmtHost fmt;
    int32_t rht;               // blockwise randomized Hadamard transform first
    uint32_t rht_signs;
    int32_t elem;              // element grid (fp4_element)
};

// Bound on a single-pass refresh's wait for the other workgroups' maxima, in
// ticks of the 100 MHz real-time counter (process-wide; 0.2 s by default).
extern uint64_t g_exchange_wait_ticks;

struct DequantLaunch {
    const uint8_t* q;
    const uint8_t* scales;
    const float* tensor_scale;
    int64_t rows, cols;
    int32_t block;
    ScaleFmtHost fmt;
    void* y;
    int32_t y_bf16;
    int64_t ld;
    int32_t rht;               // inverse blockwise Hadamard transform last
    uint32_t rht_signs;
    int32_t elem;              // element grid (fp4_element)
};

hipError_t launch_quantize(const QuantLaunch& p, hipStream_t s);
// The row-wise output of a two-orientation call.
struct RowOut {
    uint8_t* q;
    uint8_t* scales;
    float* tensor_scale;
};
// Column-wise: rows/cols describe the output (x^T); x is [cols, rows].  With
// `rows`, the row-wise quantization of x is written there too (one read).
hipError_t launch_quantize_t(const QuantLaunch& p, hipStream_t s, const RowOut* rows = nullptr);
hipError_t launch_dequantize(const DequantLaunch& p, hipStream_t s);

struct GemmLaunch {
    const uint8_t* qa; const uint8_t* sa; const float* ga;   // A [M, K]
    const uint8_t* qb; const uint8_t* sb; const float* gb;   // W [N, K]
    int64_t m, n, k;
    int32_t block;
    ScaleFmtHost fa, fb;
    uint16_t* c;
    int64_t ldc;
    int32_t elem;              // element grid of both operands (fp4_element)
};

// The exact dequantize path needs one 16-bit type (f16 or bf16) that holds
// every element * scale product of both operands exactly.
bool gemm_dq_supported(const ScaleFmtHost& fa, const ScaleFmtHost& fb, int elem);
hipError_t launch_gemm_mx(const GemmLaunch& p, hipStream_t s);
// E2M1 with E8M0 scales at block 16 on the scaled FP4 matrix instruction,
// when the stage shape fits.
bool gemm_mx16_supported(const GemmLaunch& p);
hipError_t launch_gemm_mx16(const GemmLaunch& p, hipStream_t s);
hipError_t launch_gemm_dq(const GemmLaunch& p, hipStream_t s);
// Small products on one wave per 32 x 32 output tile (no LDS): E2M1 with
// E8M0 or f16- / bf16-exact ExMy scales on both operands, MXFP8, INT8 with
// E4M3 scales; M * N at most g_gemm_small_outputs (E2M1 with E8M0: an
// eighth of it, the bf16 forms 1.5 times it; process-wide).
extern int64_t g_gemm_small_outputs;
bool gemm_small_supported(const GemmLaunch& p);
hipError_t launch_gemm_small(const GemmLaunch& p, hipStream_t s);

struct WoGemmLaunch {
    const uint16_t* x; int64_t ldx; int64_t m;
    const uint8_t* qw; const uint8_t* sw; const float* gw;
    int64_t n, k;
    int32_t block;
    ScaleFmtHost fw;
    uint16_t* y; int64_t ldy;
    int32_t elem;              // element grid of the weights (fp4_element)
};

hipError_t launch_wo_gemm(const WoGemmLaunch& p, hipStream_t s);
// C[rows, cols] (bf16, row stride ld) = 0: the product over an empty K.
hipError_t launch_fill_zero_bf16(uint16_t* c, int64_t ld, int64_t rows, int64_t cols, hipStream_t s);

}  // namespace fp4
