// quant.hip -- tensor amax, block-scaled FP4 quantization (round-to-nearest
// and stochastic) and dequantization for gfx950.
//
// Method (quant_prune_distill/486 "Метод"; gonzo_ML/3986 "Форматы FP4",
// "Стохастическая квантизация"; ue5m3-fp4-pretraining "Что сделали"): one
// scale per block of 16 or 32 E2M1 elements, the scale stored in a low
// precision encoding under an fp32 per-tensor scale derived from the tensor
// maximum; nearest or stochastic rounding of the elements.
//
// Work decomposition: the tensor is a flat sequence of 8-element "units"
// (one 16-byte bf16 load or two 16-byte fp32 loads, one 4-byte store of
// codes).  A block of B elements is B/8 adjacent lanes; its maximum is
// reduced with DPP quad permutations.  Each wave streams UNROLL*64
// consecutive units so every load instruction covers a contiguous 1 KiB
// (bf16) span.  All decisions are binary32 with round-to-nearest-even and no
// contraction, in the order the C ABI documents.
#include <float.h>

#include "fp4_device.hpp"
#include "fp4_internal.h"

namespace fp4 {

// ---------------------------------------------------------------------------
// exact unsigned division by a runtime constant (Granlund-Montgomery): for
// every 32-bit n, n / d = (umulhi(n, m) + n) >> s.
// ---------------------------------------------------------------------------
struct FastDiv {
    uint32_t d, m, s;
};

static FastDiv make_fastdiv(uint32_t d)
{
    FastDiv f;
    f.d = d;
    uint32_t s = 0;
    while ((1ull << s) < d) ++s;
    f.s = s;
    f.m = (uint32_t)((((1ull << s) - d) << 32) / d + 1);
    return f;
}

__device__ __forceinline__ uint32_t fdiv(uint32_t n, const FastDiv& f)
{
    uint64_t t = (uint64_t)__umulhi(n, f.m) + n;
    return (uint32_t)(t >> f.s);
}

// element offset of unit u (8 elements) in a row-strided tensor
__device__ __forceinline__ uint64_t unit_offset(uint32_t u, bool strided, const FastDiv& upr, int64_t ld)
{
    if (!strided) return (uint64_t)u * 8u;
    uint32_t row = fdiv(u, upr);
    uint32_t c8 = u - row * upr.d;
    return (uint64_t)row * (uint64_t)ld + (uint64_t)c8 * 8u;
}

template <typename InT>
struct Unit;

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

template <>
struct Unit<uint16_t> {                      // bf16
    u32x4 w;
    __device__ __forceinline__ void load(const void* x, uint64_t off)
    {
        w = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)x + off));
    }
    __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ void get(float v[8]) const
    {
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4] = bf16_lo(w.z); v[5] = bf16_hi(w.z);
        v[6] = bf16_lo(w.w); v[7] = bf16_hi(w.w);
    }
};

template <>
struct Unit<float> {
    f32x4 a, b;
    __device__ __forceinline__ void load(const void* x, uint64_t off)
    {
        const f32x4* p = (const f32x4*)((const float*)x + off);
        a = __builtin_nontemporal_load(p);
        b = __builtin_nontemporal_load(p + 1);
    }
    __device__ __forceinline__ void zero() { a = f32x4{0.f, 0.f, 0.f, 0.f}; b = a; }
    __device__ __forceinline__ void get(float v[8]) const
    {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};

__device__ __forceinline__ float absmax8(const float v[8])
{
    float m0 = __builtin_fmaxf(__builtin_fabsf(v[0]), __builtin_fabsf(v[1]));
    float m1 = __builtin_fmaxf(__builtin_fabsf(v[2]), __builtin_fabsf(v[3]));
    float m2 = __builtin_fmaxf(__builtin_fabsf(v[4]), __builtin_fabsf(v[5]));
    float m3 = __builtin_fmaxf(__builtin_fabsf(v[6]), __builtin_fabsf(v[7]));
    return __builtin_fmaxf(__builtin_fmaxf(m0, m1), __builtin_fmaxf(m2, m3));
}

// ---------------------------------------------------------------------------
// tensor amax: max |x| reduced to one value; the last workgroup to finish
// publishes it and clears the workspace for the next call.
// ---------------------------------------------------------------------------
constexpr int kAmaxThreads = 256;
constexpr int kAmaxUnroll = 4;

template <typename InT>
__global__ __launch_bounds__(kAmaxThreads) void k_amax(const void* __restrict__ x, uint32_t nunits, FastDiv upr,
                                                       int64_t ld, int strided, AmaxDev* __restrict__ dst)
{
    float m = 0.0f;
    const uint64_t stride = (uint64_t)gridDim.x * kAmaxThreads;
    uint64_t u = (uint64_t)blockIdx.x * kAmaxThreads + threadIdx.x;
    for (; u < nunits; u += stride * kAmaxUnroll) {
        Unit<InT> un[kAmaxUnroll];
#pragma unroll
        for (int j = 0; j < kAmaxUnroll; ++j) {
            uint64_t uj = u + j * stride;
            if (uj < nunits) un[j].load(x, unit_offset((uint32_t)uj, strided, upr, ld));
            else un[j].zero();
        }
#pragma unroll
        for (int j = 0; j < kAmaxUnroll; ++j) {
            float v[8];
            un[j].get(v);
            m = __builtin_fmaxf(m, absmax8(v));
        }
    }
    // wave reduction (non-negative floats: max of the bit patterns)
    for (int o = 32; o > 0; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
    __shared__ float wmax[kAmaxThreads / 64];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kAmaxThreads / 64; ++w) m = __builtin_fmaxf(m, wmax[w]);
        atomicMax(&dst->slot, __float_as_uint(m));
        __threadfence();
        uint32_t done = atomicAdd(&dst->count, 1u);
        if (done == gridDim.x - 1) {
            __threadfence();
            uint32_t v = atomicExch(&dst->slot, 0u);
            dst->amax = __uint_as_float(v);
            atomicExch(&dst->count, 0u);
        }
    }
}

hipError_t launch_amax(const void* x, int32_t x_bf16, int64_t rows, int64_t cols, int64_t ld, AmaxDev* dst,
                       hipStream_t s)
{
    const uint32_t upr = (uint32_t)(cols / 8);
    const uint32_t nunits = (uint32_t)(rows * (cols / 8));
    const int strided = (ld != cols);
    FastDiv fd = make_fastdiv(upr ? upr : 1);
    uint32_t blocks = (nunits + kAmaxThreads * kAmaxUnroll - 1) / (kAmaxThreads * kAmaxUnroll);
    if (blocks > 2048) blocks = 2048;
    if (blocks == 0) blocks = 1;
    if (x_bf16)
        hipLaunchKernelGGL(k_amax<uint16_t>, dim3(blocks), dim3(kAmaxThreads), 0, s, x, nunits, fd, ld, strided, dst);
    else
        hipLaunchKernelGGL(k_amax<float>, dim3(blocks), dim3(kAmaxThreads), 0, s, x, nunits, fd, ld, strided, dst);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// quantize
// ---------------------------------------------------------------------------
constexpr int kQThreads = 256;

struct QArgs {
    const void* x;
    uint32_t nunits;
    FastDiv upr;
    int64_t ld;
    int32_t strided;
    uint32_t* q;                 // one dword of codes per unit
    uint8_t* scales;
    float* tensor_scale;
    const AmaxDev* amax_src;
    ScaleFmt f;
    uint32_t key0, key1, off0, off1;
};

// Tensor scale g = amax_t / RN(6 Smax); 1 when there is no tensor scale or
// the quotient is zero or not finite.
__device__ __forceinline__ float tensor_scale_of(const QArgs& a, float* amax_out)
{
    float g = 1.0f, am = 0.0f;
    if (a.amax_src) {
        am = a.amax_src->amax;
        float den = 6.0f * a.f.smax;
        g = am / den;
        if (!(g > 0.0f) || !(g <= FLT_MAX)) g = 1.0f;
    }
    *amax_out = am;
    return g;
}

template <typename InT, int BLOCK, bool SR, bool E8M0, bool HWCVT>
__global__ __launch_bounds__(kQThreads) void k_quantize(QArgs a)
{
    constexpr int UNROLL = sizeof(InT) == 2 ? 4 : 2;
    constexpr int G = BLOCK / 8;                 // lanes per block
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x * (kQThreads / 64) + (threadIdx.x >> 6);
    const uint32_t base = wave * (64u * UNROLL);

    float amax_t;
    const float g = tensor_scale_of(a, &amax_t);
    const float d = 6.0f * g;
    if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.tensor_scale[0] = g;
        a.tensor_scale[1] = amax_t;
    }

    Unit<InT> un[UNROLL];
#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
        uint32_t u = base + j * 64 + lane;
        if (u < a.nunits) un[j].load(a.x, unit_offset(u, a.strided, a.upr, a.ld));
        else un[j].zero();
    }

#pragma unroll
    for (int j = 0; j < UNROLL; ++j) {
        const uint32_t u = base + j * 64 + lane;
        float v[8];
        un[j].get(v);
        float bmax = absmax8(v);
        bmax = dpp_max_xor1(bmax);
        if (G == 4) bmax = dpp_max_xor2(bmax);

        uint32_t scode;
        float inv;
        if (E8M0) {
            scode = scale_code_e8m0(bmax);
            inv = e8m0_inv(scode);
        } else {
            float us = bmax / d;
            scode = scale_encode_exmy(us, a.f);
            float s = scale_decode_exmy(scode, a.f);
            float S = s * g;
            inv = 0.0f;
            if (S != 0.0f) {
                inv = 1.0f / S;
                if (!(inv <= FLT_MAX)) inv = FLT_MAX;
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = v[k] * inv;

        uint32_t packed;
        if (SR) {
            U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
            const uint32_t w[4] = {r.x, r.y, r.z, r.w};
            packed = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                uint32_t r16 = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
                packed |= e2m1_sr(v[k], r16) << (4 * k);
            }
        } else if (HWCVT) {
            packed = FP4_CVT_PK(0u, v[0], v[1], 0);
            packed = FP4_CVT_PK(packed, v[2], v[3], 1);
            packed = FP4_CVT_PK(packed, v[4], v[5], 2);
            packed = FP4_CVT_PK(packed, v[6], v[7], 3);
        } else {
            packed = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) packed |= e2m1_rtn_sw(v[k]) << (4 * k);
        }
        if (u < a.nunits) {
            __builtin_nontemporal_store(packed, a.q + u);
            if ((lane & (G - 1)) == 0) a.scales[u / G] = (uint8_t)scode;
        }
    }
}

bool g_use_hw_cvt = true;    // hardware E2M1 pack for round-to-nearest

template <typename InT, int BLOCK, bool SR, bool E8M0>
static void launch_q4(const QArgs& a, uint32_t blocks, hipStream_t s)
{
    if (!SR && g_use_hw_cvt)
        hipLaunchKernelGGL((k_quantize<InT, BLOCK, SR, E8M0, true>), dim3(blocks), dim3(kQThreads), 0, s, a);
    else
        hipLaunchKernelGGL((k_quantize<InT, BLOCK, SR, E8M0, false>), dim3(blocks), dim3(kQThreads), 0, s, a);
}

template <typename InT, int BLOCK>
static void launch_q3(const QArgs& a, bool sr, bool e8, uint32_t blocks, hipStream_t s)
{
    if (sr) {
        if (e8) launch_q4<InT, BLOCK, true, true>(a, blocks, s);
        else launch_q4<InT, BLOCK, true, false>(a, blocks, s);
    } else {
        if (e8) launch_q4<InT, BLOCK, false, true>(a, blocks, s);
        else launch_q4<InT, BLOCK, false, false>(a, blocks, s);
    }
}

hipError_t launch_quantize(const QuantLaunch& p, hipStream_t s)
{
    QArgs a;
    a.x = p.x;
    a.nunits = (uint32_t)(p.rows * (p.cols / 8));
    a.upr = make_fastdiv((uint32_t)(p.cols / 8 ? p.cols / 8 : 1));
    a.ld = p.ld;
    a.strided = (p.ld != p.cols);
    a.q = (uint32_t*)p.q;
    a.scales = p.scales;
    a.tensor_scale = p.tensor_scale;
    a.amax_src = p.amax_src;
    a.f = ScaleFmt{p.fmt.ebits, p.fmt.mbits, p.fmt.bias, p.fmt.maxcode, p.fmt.smax, p.fmt.is_e8m0};
    a.key0 = (uint32_t)p.seed;
    a.key1 = (uint32_t)(p.seed >> 32);
    a.off0 = (uint32_t)p.offset;
    a.off1 = (uint32_t)(p.offset >> 32);
    const int unroll = p.x_bf16 ? 4 : 2;
    const uint32_t per_block = kQThreads * unroll;
    uint32_t blocks = (a.nunits + per_block - 1) / per_block;
    if (blocks == 0) blocks = 1;
    const bool sr = p.stochastic != 0, e8 = p.fmt.is_e8m0 != 0;
    if (p.x_bf16) {
        if (p.block == 16) launch_q3<uint16_t, 16>(a, sr, e8, blocks, s);
        else launch_q3<uint16_t, 32>(a, sr, e8, blocks, s);
    } else {
        if (p.block == 16) launch_q3<float, 16>(a, sr, e8, blocks, s);
        else launch_q3<float, 32>(a, sr, e8, blocks, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dequantize: y = RN(RN(e2m1 * s) * g), bf16 output rounded once more (RNE)
// ---------------------------------------------------------------------------
constexpr int kDQThreads = 256;

template <bool OUT_BF16, int BLOCK, bool E8M0>
__global__ __launch_bounds__(kDQThreads) void k_dequantize(const uint32_t* __restrict__ q,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ tensor_scale, uint32_t nunits,
                                                           FastDiv upr, int64_t ld, int strided, ScaleFmt f,
                                                           void* __restrict__ y)
{
    const uint32_t u = blockIdx.x * kDQThreads + threadIdx.x;
    if (u >= nunits) return;
    const float g = tensor_scale[0];
    const uint32_t w = q[u];
    const uint32_t sc = scales[u / (BLOCK / 8)];
    const float s = scale_decode_any(sc, f);
    float o[8];
#pragma unroll
    for (int k = 0; k < 8; ++k) {
        float t = e2m1_value((w >> (4 * k)) & 0xFu) * s;
        o[k] = t * g;
    }
    const uint64_t off = unit_offset(u, strided, upr, ld);
    if (OUT_BF16) {
        uint4 r;
        r.x = f32_to_bf16_rne(o[0]) | (f32_to_bf16_rne(o[1]) << 16);
        r.y = f32_to_bf16_rne(o[2]) | (f32_to_bf16_rne(o[3]) << 16);
        r.z = f32_to_bf16_rne(o[4]) | (f32_to_bf16_rne(o[5]) << 16);
        r.w = f32_to_bf16_rne(o[6]) | (f32_to_bf16_rne(o[7]) << 16);
        *(uint4*)((uint16_t*)y + off) = r;
    } else {
        float4* p = (float4*)((float*)y + off);
        p[0] = make_float4(o[0], o[1], o[2], o[3]);
        p[1] = make_float4(o[4], o[5], o[6], o[7]);
    }
}

template <bool OUT_BF16, int BLOCK>
static void launch_dq2(const DequantLaunch& p, uint32_t nunits, const FastDiv& fd, int strided, const ScaleFmt& f,
                       hipStream_t s)
{
    uint32_t blocks = (nunits + kDQThreads - 1) / kDQThreads;
    if (blocks == 0) blocks = 1;
    if (f.is_e8m0)
        hipLaunchKernelGGL((k_dequantize<OUT_BF16, BLOCK, true>), dim3(blocks), dim3(kDQThreads), 0, s,
                           (const uint32_t*)p.q, p.scales, p.tensor_scale, nunits, fd, p.ld, strided, f, p.y);
    else
        hipLaunchKernelGGL((k_dequantize<OUT_BF16, BLOCK, false>), dim3(blocks), dim3(kDQThreads), 0, s,
                           (const uint32_t*)p.q, p.scales, p.tensor_scale, nunits, fd, p.ld, strided, f, p.y);
}

hipError_t launch_dequantize(const DequantLaunch& p, hipStream_t s)
{
    const uint32_t nunits = (uint32_t)(p.rows * (p.cols / 8));
    FastDiv fd = make_fastdiv((uint32_t)(p.cols / 8 ? p.cols / 8 : 1));
    const int strided = (p.ld != p.cols);
    ScaleFmt f{p.fmt.ebits, p.fmt.mbits, p.fmt.bias, p.fmt.maxcode, p.fmt.smax, p.fmt.is_e8m0};
    if (p.y_bf16) {
        if (p.block == 16) launch_dq2<true, 16>(p, nunits, fd, strided, f, s);
        else launch_dq2<true, 32>(p, nunits, fd, strided, f, s);
    } else {
        if (p.block == 16) launch_dq2<false, 16>(p, nunits, fd, strided, f, s);
        else launch_dq2<false, 32>(p, nunits, fd, strided, f, s);
    }
    return hipGetLastError();
}

}  // namespace fp4
