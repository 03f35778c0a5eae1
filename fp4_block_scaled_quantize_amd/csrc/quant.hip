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

#include <atomic>

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
typedef uint16_t u16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// max |x| of 8 elements as binary32 bits.  Non-negative floats order like
// their bit patterns, so the maximum is taken on integers (no NaN
// canonicalization): bf16 pairs with packed 16-bit max, fp32 with 32-bit max.
__device__ __forceinline__ uint32_t absmax_bits_bf16(const u32x4& w)
{
    u16x2 a = __builtin_bit_cast(u16x2, w.x & 0x7FFF7FFFu), b = __builtin_bit_cast(u16x2, w.y & 0x7FFF7FFFu);
    u16x2 c = __builtin_bit_cast(u16x2, w.z & 0x7FFF7FFFu), d = __builtin_bit_cast(u16x2, w.w & 0x7FFF7FFFu);
    u16x2 m = __builtin_elementwise_max(__builtin_elementwise_max(a, b), __builtin_elementwise_max(c, d));
    uint32_t mm = __builtin_bit_cast(uint32_t, m);
    uint32_t lo = mm << 16, hi = mm & 0xFFFF0000u;
    return lo > hi ? lo : hi;
}

__device__ __forceinline__ uint32_t umax3(uint32_t a, uint32_t b, uint32_t c)
{
    uint32_t t = a > b ? a : b;
    return t > c ? t : c;
}

__device__ __forceinline__ uint32_t absmax_bits_f32(const f32x4& a, const f32x4& b)
{
    const uint32_t M = 0x7FFFFFFFu;
    uint32_t m0 = umax3(__float_as_uint(a.x) & M, __float_as_uint(a.y) & M, __float_as_uint(a.z) & M);
    uint32_t m1 = umax3(__float_as_uint(a.w) & M, __float_as_uint(b.x) & M, __float_as_uint(b.y) & M);
    uint32_t m2 = umax3(__float_as_uint(b.z) & M, __float_as_uint(b.w) & M, m0);
    return m1 > m2 ? m1 : m2;
}

template <>
struct Unit<uint16_t> {                      // bf16
    u32x4 w;
    __device__ __forceinline__ void load(const void* x, uint64_t off)
    {
        w = __builtin_nontemporal_load((const u32x4*)((const uint16_t*)x + off));
    }
    __device__ __forceinline__ void zero() { w = u32x4{0u, 0u, 0u, 0u}; }
    __device__ __forceinline__ uint32_t absmax() const { return absmax_bits_bf16(w); }
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
    __device__ __forceinline__ uint32_t absmax() const { return absmax_bits_f32(a, b); }
    __device__ __forceinline__ void get(float v[8]) const
    {
        v[0] = a.x; v[1] = a.y; v[2] = a.z; v[3] = a.w;
        v[4] = b.x; v[5] = b.y; v[6] = b.z; v[7] = b.w;
    }
};


// ---------------------------------------------------------------------------
// tensor amax: max |x| over the tensor.  Exactly kAmaxParts workgroups; each
// writes the maximum of its grid-stride share to its own partial slot, so
// the reduction needs neither atomics nor fences: the quantize kernel that
// follows on the stream reduces the partials.
// ---------------------------------------------------------------------------
constexpr int kAmaxThreads = 512;

// ROTG > 0: the maximum of the blockwise Hadamard-transformed tensor, blocks
// of 8*ROTG elements (adjacent units live in adjacent lanes, and a block's
// units are all in range or all out of it).
template <typename InT, bool STRIDED, int ROTG>
__global__ __launch_bounds__(kAmaxThreads) void k_amax(const void* __restrict__ x, uint32_t nunits, FastDiv upr,
                                                       int64_t ld, AmaxDev* __restrict__ dst, uint32_t signs)
{
    constexpr int U = sizeof(InT) == 2 ? 8 : 4;
    uint32_t m = 0u;
    const uint64_t stride = (uint64_t)kAmaxParts * kAmaxThreads;
    for (uint64_t u = (uint64_t)blockIdx.x * kAmaxThreads + threadIdx.x; u < nunits; u += stride * U) {
        Unit<InT> un[U];
#pragma unroll
        for (int j = 0; j < U; ++j) {
            uint64_t uj = u + j * stride;
            if (uj < nunits) un[j].load(x, unit_offset((uint32_t)uj, STRIDED, upr, ld));
            else un[j].zero();
        }
#pragma unroll
        for (int j = 0; j < U; ++j) {
            uint32_t t;
            if (ROTG) {
                float v[8];
                un[j].get(v);
                rht_forward<ROTG ? ROTG : 2>(v, threadIdx.x & (ROTG - 1), signs);
                t = absmax_bits8(v);
            } else {
                t = un[j].absmax();
            }
            m = m > t ? m : t;
        }
    }
    for (int o = 32; o > 0; o >>= 1) {
        uint32_t t = (uint32_t)__shfl_xor((int)m, o, 64);
        m = m > t ? m : t;
    }
    __shared__ uint32_t wmax[kAmaxThreads / 64];
    if ((threadIdx.x & 63) == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int w = 1; w < kAmaxThreads / 64; ++w) m = m > wmax[w] ? m : wmax[w];
        dst->partial[blockIdx.x] = __uint_as_float(m);
    }
}

template <typename InT, int ROTG>
static void launch_amax2(const void* x, uint32_t nunits, const FastDiv& fd, int64_t ld, bool strided, AmaxDev* dst,
                         uint32_t signs, hipStream_t s)
{
    const dim3 g(kAmaxParts), b(kAmaxThreads);
    if (strided) hipLaunchKernelGGL((k_amax<InT, true, ROTG>), g, b, 0, s, x, nunits, fd, ld, dst, signs);
    else hipLaunchKernelGGL((k_amax<InT, false, ROTG>), g, b, 0, s, x, nunits, fd, ld, dst, signs);
}

// rot_block: 0 (plain maximum) or the block size of the Hadamard transform
static hipError_t launch_amax(const void* x, int32_t x_bf16, int64_t rows, int64_t cols, int64_t ld, AmaxDev* dst,
                              hipStream_t s, int rot_block = 0, uint32_t signs = 0)
{
    const uint32_t upr = (uint32_t)(cols / 8);
    const uint32_t nunits = (uint32_t)(rows * (cols / 8));
    const bool strided = (ld != cols);
    FastDiv fd = make_fastdiv(upr ? upr : 1);
    if (x_bf16) {
        if (rot_block == 16) launch_amax2<uint16_t, 2>(x, nunits, fd, ld, strided, dst, signs, s);
        else if (rot_block == 32) launch_amax2<uint16_t, 4>(x, nunits, fd, ld, strided, dst, signs, s);
        else launch_amax2<uint16_t, 0>(x, nunits, fd, ld, strided, dst, signs, s);
    } else {
        if (rot_block == 16) launch_amax2<float, 2>(x, nunits, fd, ld, strided, dst, signs, s);
        else if (rot_block == 32) launch_amax2<float, 4>(x, nunits, fd, ld, strided, dst, signs, s);
        else launch_amax2<float, 0>(x, nunits, fd, ld, strided, dst, signs, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// quantize
// ---------------------------------------------------------------------------
constexpr int kQThreads = 256;
constexpr int kQUnroll = 4;                  // units per lane (one load each, all in flight)
// Single-pass refresh: one 1024-thread workgroup per CU holds up to
// kFUnroll units per lane in registers while the grid agrees on the tensor
// maximum, so the input is read once.
constexpr int kFThreads = 1024;
constexpr int kFUnroll = 8;
uint64_t g_exchange_wait_ticks = 20000000;   // 0.2 s of the 100 MHz real-time counter

struct QArgs {
    const void* x;
    uint32_t nunits;
    FastDiv upr;
    int64_t ld;
    uint32_t* q;                 // one dword of codes per unit
    uint8_t* scales;
    float* tensor_scale;
    AmaxDev* amax_src;
    int32_t refresh;
    ScaleFmt f;
    uint32_t key0, key1, off0, off1;
    uint32_t signs;              // blockwise Hadamard transform sign mask (ROT kernels)
    uint64_t wait_ticks;         // FUSED: bound on the wait for the other workgroups' maxima
};

// The tensor maximum of this call: the reduction of the amax kernel's
// partials on a refresh, the stored value otherwise.  Every wave reduces the
// partials itself (one 16-byte load per lane), so no barrier is needed.
template <typename A>
__device__ __forceinline__ float tensor_amax(const A& a)
{
    if (!a.refresh) return a.amax_src->stored;
    static_assert(kAmaxParts == 256, "one float4 of partials per lane");
    const uint32_t lane = threadIdx.x & 63;
    const float4 p = reinterpret_cast<const float4*>(a.amax_src->partial)[lane];
    float m = __builtin_fmaxf(__builtin_fmaxf(p.x, p.y), __builtin_fmaxf(p.z, p.w));
    for (int o = 32; o > 0; o >>= 1) m = __builtin_fmaxf(m, __shfl_xor(m, o, 64));
    return m;
}

__device__ __forceinline__ uint32_t wave_umax(uint32_t m)
{
    for (int o = 32; o > 0; o >>= 1) {
        const uint32_t t = (uint32_t)__shfl_xor((int)m, o, 64);
        m = m > t ? m : t;
    }
    return m;
}

// Tensor maximum (as binary32 bits) agreed by every workgroup of a
// single-pass launch.  Each workgroup publishes {epoch, its maximum} as one
// 64-bit word in its own slot with a relaxed agent-scope atomic store; wave
// 0 of every workgroup then polls all slots until each carries this
// launch's epoch.  Flag and value share a word, so single-location
// coherence suffices and no fence (L2 write-back or invalidate) is needed.
// The launch grid never exceeds one workgroup per CU, but other work on the
// device can still keep some of them from being scheduled, so the poll is
// bounded in time: a workgroup that gives up takes the maximum of the whole
// tensor itself (full_tensor_amax), which is the same value, so the result
// never depends on co-residency.
// Epochs: every single-pass launch that exchanges runs the same grid (one
// workgroup per CU, however small the tensor) and every workgroup publishes
// exactly once per launch, so at the start of a launch every slot carries
// the previous exchanging launch's epoch (0 in a fresh state); a tensor
// that fits one workgroup runs as a grid of one, which writes no slot.  Each workgroup reads
// its own slot -- written only by itself -- and uses that epoch + 1: the
// same fresh epoch for every workgroup of the launch (graph replays
// included), with no counter, no atomic read-modify-write and nothing left
// to do at the end of the kernel.  (Earlier schemes advanced a stored epoch
// from the last workgroup to leave; their departure counts cost 0.7-1.4 us
// per 4096 x 4096 launch in serialized same-address atomics.)
// The workgroup's own slot is loaded at the start of the kernel (before it
// publishes, so the load overlaps the data loads); launch_epoch turns it
// into this launch's epoch.
__device__ __forceinline__ uint32_t epoch_word(const AmaxDev* st)
{
    return (uint32_t)(__hip_atomic_load(&st->slot[blockIdx.x * kXchgStride], __ATOMIC_RELAXED,
                                        __HIP_MEMORY_SCOPE_AGENT) >> 32);
}
__device__ __forceinline__ uint32_t launch_epoch(uint32_t word)
{
    const uint32_t e = word + 1u;
    return e == 0 ? 1u : e;
}

// Publishes m and polls; returns true with *gm = the maximum over every
// workgroup, or false when the wait bound passed first.  A grid of one
// workgroup has the maximum at hand and publishes nothing.
template <int T>
__device__ bool grid_exchange(uint32_t m, uint32_t e, AmaxDev* st, uint64_t wait_ticks, uint32_t* gm)
{
    __shared__ uint32_t wmax[T / 64];
    __shared__ uint32_t gmax, gok;
    const uint32_t lane = threadIdx.x & 63, wv = threadIdx.x >> 6;
    m = wave_umax(m);
    if (lane == 0) wmax[wv] = m;
    __syncthreads();
    const uint32_t nwg = gridDim.x;
    if (wv == 0 && nwg == 1) {
        // the whole tensor is in this workgroup: its maximum is the tensor's,
        // and no slot is written (every slot keeps the epoch of the last
        // exchange, which is what the next one derives its epoch from)
        const uint32_t mm = wave_umax(lane < T / 64 ? wmax[lane] : 0u);
        if (lane == 0) {
            gmax = mm;
            gok = 1u;
        }
    } else if (wv == 0) {
        const uint32_t mm = wave_umax(lane < T / 64 ? wmax[lane] : 0u);
        if (lane == 0)
            __hip_atomic_store(&st->slot[blockIdx.x * kXchgStride], ((uint64_t)e << 32) | mm, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t t0 = __builtin_amdgcn_s_memrealtime();
        uint32_t tm = 0;
        bool done = false;
        // two poll rounds in flight: a round's answer takes about a
        // microsecond, and the next one is issued before it is examined, so
        // the last publication is seen half a round sooner (about 0.5 us of a
        // 4096 x 4096 launch).  Lanes past the grid reread the last slot.
        constexpr int SL = kXchgSlots / 64;
        auto poll = [&](uint64_t (&w)[SL]) {
#pragma unroll
            for (int k = 0; k < SL; ++k) {
                const uint32_t i = lane + 64 * k < nwg ? lane + 64 * k : nwg - 1;
                w[k] = __hip_atomic_load(&st->slot[i * kXchgStride], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        };
        // true once every slot holds this epoch (then tm is the maximum) or
        // the wait bound has passed
        auto check = [&](const uint64_t (&w)[SL]) {
            tm = 0;
            bool mine = true;
#pragma unroll
            for (int k = 0; k < SL; ++k) {
                const bool c = (uint32_t)(w[k] >> 32) == e;
                mine = mine && c;
                if (c) tm = tm > (uint32_t)w[k] ? tm : (uint32_t)w[k];
            }
            done = __all(mine);
            return done || __builtin_amdgcn_s_memrealtime() - t0 >= wait_ticks;
        };
        uint64_t b0[SL], b1[SL];
        poll(b0);
        for (;;) {
            poll(b1);
            if (check(b0)) break;
            poll(b0);
            if (check(b1)) break;
        }
        tm = wave_umax(tm);
        if (lane == 0) {
            gmax = tm;
            gok = done ? 1u : 0u;
        }
    }
    __syncthreads();
    *gm = gmax;
    return gok != 0;
}

// max |x| (of the blockwise-transformed x with ROT) over the whole tensor,
// by every thread of the workgroup: the fallback of a single-pass refresh
// whose exchange gave up.  Unit u = it * T + threadIdx.x, so a block's G
// units sit in adjacent lanes as in the quantize loop.
template <typename InT, int T, int G, bool STRIDED, bool ROT>
__device__ uint32_t full_tensor_amax(const void* x, uint32_t nunits, const FastDiv& upr, int64_t ld, uint32_t signs)
{
    __shared__ uint32_t wmax[T / 64];
    const uint32_t lane = threadIdx.x & 63;
    uint32_t m = 0;
    for (uint32_t u0 = 0; u0 < nunits; u0 += T) {
        const uint32_t u = u0 + threadIdx.x;
        Unit<InT> un;
        if (u < nunits) un.load(x, unit_offset(u, STRIDED, upr, ld));
        else un.zero();
        uint32_t t;
        if (ROT) {
            float v[8];
            un.get(v);
            rht_forward<G>(v, lane & (G - 1), signs);
            t = absmax_bits8(v);
        } else {
            t = un.absmax();
        }
        m = m > t ? m : t;
    }
    m = wave_umax(m);
    if (lane == 0) wmax[threadIdx.x >> 6] = m;
    __syncthreads();
    return wave_umax(lane < T / 64 ? wmax[lane] : 0u);
}

// Tensor scale g = amax_t / RN(qmax Smax), qmax the grid's largest
// magnitude (6 for E2M1, 7 for INT4); 1 when there is no tensor scale or the
// quotient is zero or not finite.
template <typename A>
__device__ __forceinline__ float tensor_scale_of(float am, const A& a, float qmax)
{
    if (!a.amax_src) return 1.0f;
    float den = qmax * a.f.smax;
    float g = am / den;
    if (!(g > 0.0f) || !(g <= FLT_MAX)) g = 1.0f;
    return g;
}

// Block scale of an ExMy format: returns the code and the reciprocal of the
// effective scale S = RN(s g) (clamped to FLT_MAX; 0 when S is 0).
__device__ __forceinline__ uint32_t exmy_scale(float bmax, float d, float g, const ScaleFmt& f, float* inv)
{
    float us = bmax / d;
    uint32_t code = scale_encode_exmy(us, f);
    float S = scale_decode_exmy(code, f) * g;
    float r = 0.0f;
    if (S != 0.0f) {
        r = 1.0f / S;
        if (!(r <= FLT_MAX)) r = FLT_MAX;
    }
    *inv = r;
    return code;
}

// Broadcast lane k of every quad to the whole quad.
template <int K>
__device__ __forceinline__ float quad_bcast(float v)
{
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), K | (K << 2) | (K << 4) | (K << 6), 0xF, 0xF,
                                                   false));
}

// FUSED: single-pass refresh (the tensor maximum of this call is agreed
// across the grid while the units stay in registers); otherwise the maximum
// comes from the amax kernel's partials (refresh) or the stored value.
// ROT: the blockwise randomized Hadamard transform is applied to every block
// right after the loads; block maxima, the tensor maximum and the codes all
// see the transformed values.
// INT: the INT4 element grid (-7..7) instead of E2M1.
// ELEM: the element grid (0 E2M1, 1 INT4, 2 FP8 E4M3, 3 INT8, 4 FP6 E2M3,
// 5 FP6 E3M2, 6 INT6; 2 and 3 one byte per element, 4..6 six bits).
template <typename InT, int BLOCK, bool SR, bool E8M0, bool STRIDED, bool FUSED, bool ROT, int ELEM>
__global__ __launch_bounds__(FUSED ? kFThreads : kQThreads) void k_quantize(QArgs a)
{
    constexpr bool INT = ELEM == 1;
    constexpr bool W8 = ELEM == 2 || ELEM == 3;
    constexpr bool W6 = ELEM >= 4;
    constexpr float QMAX = ELEM == 0 ? 6.0f : ELEM == 1 ? 7.0f : ELEM == 2 ? 448.0f : ELEM == 3 ? 127.0f
                         : ELEM == 4 ? 7.5f : ELEM == 5 ? 28.0f : 31.0f;   // grid maximum
    constexpr int T = FUSED ? kFThreads : kQThreads;
    constexpr int U = FUSED ? kFUnroll : kQUnroll;
    constexpr int G = BLOCK / 8;                 // lanes per block (2 or 4)
    constexpr int PER = U / G;                   // block scales computed per lane
    static_assert(U % G == 0, "every lane of a block group computes U/G scales");
    static_assert(!(FUSED && E8M0), "E8M0 has no tensor scale");
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t sub = lane & (G - 1);
    const uint32_t wave = blockIdx.x * (T / 64) + (threadIdx.x >> 6);
    const uint32_t base = wave * (64u * U);

    // issue every load first
    // (FUSED kernels always have a state; every wave loads the word so no
    // branch ties the wait for it to the load)
    const uint32_t eword = FUSED ? epoch_word(a.amax_src) : 0u;
    Unit<InT> un[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        uint32_t u = base + j * 64 + lane;
        if (u < a.nunits) un[j].load(a.x, unit_offset(u, STRIDED, a.upr, a.ld));
        else un[j].zero();
    }
    const uint32_t epoch = launch_epoch(eword);

    // the transformed values (ROT only; units past the end are zeros, and a
    // block's units are all in range or all out of it)
    float rv[ROT ? U : 1][8];
    if (ROT) {
#pragma unroll
        for (int j = 0; j < U; ++j) {
            un[j].get(rv[j]);
            rht_forward<G>(rv[j], sub, a.signs);
        }
    }

    // block maxima, reduced over the G lanes of each block (independent of
    // the tensor scale)
    float bm[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const uint32_t um = ROT ? absmax_bits8(rv[ROT ? j : 0]) : un[j].absmax();
        bm[j] = __uint_as_float(dpp_umax_xor1(um));
        if (G == 4) bm[j] = __uint_as_float(dpp_umax_xor2(__float_as_uint(bm[j])));
    }

    float g = 1.0f, d = QMAX;
    if (!E8M0 && a.amax_src) {
        float am;
        if (FUSED) {
            uint32_t m = 0;
#pragma unroll
            for (int j = 0; j < U; ++j) m = m > __float_as_uint(bm[j]) ? m : __float_as_uint(bm[j]);
            uint32_t gm;
            if (!grid_exchange<T>(m, epoch, a.amax_src, a.wait_ticks, &gm)) {
                gm = full_tensor_amax<InT, T, G, STRIDED, ROT>(a.x, a.nunits, a.upr, a.ld, a.signs);
                if (threadIdx.x == 0)
                    __hip_atomic_fetch_add(&a.amax_src->fallbacks, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
            am = __uint_as_float(gm);
        } else {
            am = tensor_amax(a);
        }
        g = tensor_scale_of(am, a, QMAX);
        d = QMAX * g;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.tensor_scale[0] = g;
            a.tensor_scale[1] = am;
            if (a.refresh) a.amax_src->stored = am;
        }
    } else if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.tensor_scale[0] = 1.0f;
        a.tensor_scale[1] = 0.0f;
    }

    // lane `sub` of a group computes the scales of blocks j = sub*PER + t
    float inv_own[PER];
#pragma unroll
    for (int t = 0; t < PER; ++t) {
        float x = bm[t];
#pragma unroll
        for (int k = 1; k < G; ++k) x = (sub == (uint32_t)k) ? bm[k * PER + t] : x;
        uint32_t code;
        if (E8M0) {
            code = ELEM == 2 ? scale_code_e8m0_emax<8>(x) : ELEM == 3 ? scale_code_e8m0_emax<6>(x)
                 : (ELEM == 5 || ELEM == 6) ? scale_code_e8m0_emax<4>(x) : scale_code_e8m0(x);
            inv_own[t] = e8m0_inv(code);
        } else {
            code = exmy_scale(x, d, g, a.f, &inv_own[t]);
        }
        const uint32_t j = sub * PER + t;
        const uint32_t u = base + j * 64 + lane;        // this lane's unit in block j
        if (u < a.nunits) a.scales[u / G] = (uint8_t)code;
    }

    // gather the reciprocal of block j from lane j / PER of the quad
    float inv[U];
#pragma unroll
    for (int t = 0; t < PER; ++t) {
        if (G == 2) {
            float mine = inv_own[t];
            float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mine), 0xB1, 0xF, 0xF, false));
            inv[t] = sub == 0 ? mine : other;             // block t lives in sub 0
            inv[PER + t] = sub == 1 ? mine : other;       // block PER+t lives in sub 1
        } else {
            inv[0 * PER + t] = quad_bcast<0>(inv_own[t]);
            inv[1 * PER + t] = quad_bcast<1>(inv_own[t]);
            inv[2 * PER + t] = quad_bcast<2>(inv_own[t]);
            inv[3 * PER + t] = quad_bcast<3>(inv_own[t]);
        }
    }

#pragma unroll
    for (int j = 0; j < U; ++j) {
        const uint32_t u = base + j * 64 + lane;
        float v[8];
        if (ROT) {
#pragma unroll
            for (int k = 0; k < 8; ++k) v[k] = rv[ROT ? j : 0][k];
        } else {
            un[j].get(v);
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) v[k] = v[k] * inv[j];
        uint32_t packed;
        if (W6) {
            // six bits per element: the unit's 48 bits leave as three
            // 16-bit stores at byte 6u
            uint64_t bits = 0;
            if (SR) {
                U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
                const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int k = 0; k < 8; ++k)
                    bits |= (uint64_t)w6_sr_code<ELEM>(v[k], (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu) << (6 * k);
            } else if (ELEM == 6) {
#pragma unroll
                for (int k = 0; k < 8; ++k) bits |= (uint64_t)w6_rtn_code<ELEM>(v[k]) << (6 * k);
            } else {
                bits = (uint64_t)fp6_rtn_pack4_hw<ELEM>(v[0], v[1], v[2], v[3]) |
                       ((uint64_t)fp6_rtn_pack4_hw<ELEM>(v[4], v[5], v[6], v[7]) << 24);
            }
            if (u < a.nunits) {
                uint16_t* dst = reinterpret_cast<uint16_t*>(a.q) + 3 * (uint64_t)u;
                __builtin_nontemporal_store((uint16_t)bits, dst);
                __builtin_nontemporal_store((uint16_t)(bits >> 16), dst + 1);
                __builtin_nontemporal_store((uint16_t)(bits >> 32), dst + 2);
            }
            continue;
        }
        if (W8) {
            // one byte per element: eight codes in two dwords
            uint32_t c[8];
            if (SR) {
                U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
                const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    const uint32_t r16 = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
                    c[k] = ELEM == 2 ? fp8_sr_code(v[k], r16) : int8_sr_code(v[k], r16);
                }
            } else if (ELEM == 2) {
                // the hardware OCP E4M3 conversion (nearest-even, sign kept)
                // after the saturating clamp to +-448
                const u32x2 pk{fp8_rtn_pack4(v[0], v[1], v[2], v[3]), fp8_rtn_pack4(v[4], v[5], v[6], v[7])};
                if (u < a.nunits) __builtin_nontemporal_store(pk, reinterpret_cast<u32x2*>(a.q) + u);
                continue;
            } else {
#pragma unroll
                for (int k = 0; k < 8; ++k) c[k] = int8_rtn_code(v[k]);
            }
            const u32x2 pk{c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24),
                           c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24)};
            if (u < a.nunits) __builtin_nontemporal_store(pk, reinterpret_cast<u32x2*>(a.q) + u);
            continue;
        }
        if (SR) {
            U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
            if (INT) {
                const uint32_t w[4] = {r.x, r.y, r.z, r.w};
                packed = 0;
#pragma unroll
                for (int k = 0; k < 8; ++k) {
                    uint32_t r16 = (w[k >> 1] >> (16 * (k & 1))) & 0xFFFFu;
                    packed |= int4_sr_code(v[k], r16) << (4 * k);
                }
            } else {
                packed = e2m1_sr_pack8(v, r.x, r.y, r.z, r.w);
            }
        } else if (INT) {
            packed = 0;
#pragma unroll
            for (int k = 0; k < 8; ++k) packed |= int4_rtn_code(v[k]) << (4 * k);
        } else {
            packed = FP4_CVT_PK(0u, v[0], v[1], 0);
            packed = FP4_CVT_PK(packed, v[2], v[3], 1);
            packed = FP4_CVT_PK(packed, v[4], v[5], 2);
            packed = FP4_CVT_PK(packed, v[6], v[7], 3);
        }
        if (u < a.nunits) __builtin_nontemporal_store(packed, a.q + u);
    }
}

template <typename InT, int BLOCK, bool SR, bool E8M0, bool FUSED, bool ROT, int ELEM>
static void launch_q6(const QArgs& a, bool strided, uint32_t blocks, hipStream_t s)
{
    const dim3 t(FUSED ? kFThreads : kQThreads);
    if (strided)
        hipLaunchKernelGGL((k_quantize<InT, BLOCK, SR, E8M0, true, FUSED, ROT, ELEM>), dim3(blocks), t, 0, s, a);
    else
        hipLaunchKernelGGL((k_quantize<InT, BLOCK, SR, E8M0, false, FUSED, ROT, ELEM>), dim3(blocks), t, 0, s, a);
}

template <typename InT, int BLOCK, bool ROT, int ELEM>
static void launch_q4(const QArgs& a, bool sr, bool e8, bool fused, bool strided, uint32_t blocks, hipStream_t s)
{
    if (sr) {
        if (fused) launch_q6<InT, BLOCK, true, false, true, ROT, ELEM>(a, strided, blocks, s);
        else if (e8) launch_q6<InT, BLOCK, true, true, false, ROT, ELEM>(a, strided, blocks, s);
        else launch_q6<InT, BLOCK, true, false, false, ROT, ELEM>(a, strided, blocks, s);
    } else {
        if (fused) launch_q6<InT, BLOCK, false, false, true, ROT, ELEM>(a, strided, blocks, s);
        else if (e8) launch_q6<InT, BLOCK, false, true, false, ROT, ELEM>(a, strided, blocks, s);
        else launch_q6<InT, BLOCK, false, false, false, ROT, ELEM>(a, strided, blocks, s);
    }
}

template <typename InT, int BLOCK, int ELEM>
static void launch_q35(const QArgs& a, bool sr, bool e8, bool fused, bool strided, bool rot, uint32_t blocks,
                       hipStream_t s)
{
    if (rot) launch_q4<InT, BLOCK, true, ELEM>(a, sr, e8, fused, strided, blocks, s);
    else launch_q4<InT, BLOCK, false, ELEM>(a, sr, e8, fused, strided, blocks, s);
}

template <typename InT, int BLOCK>
static void launch_q3(const QArgs& a, bool sr, bool e8, bool fused, bool strided, bool rot, int elem,
                      uint32_t blocks, hipStream_t s)
{
    switch (elem) {
    case 1: launch_q35<InT, BLOCK, 1>(a, sr, e8, fused, strided, rot, blocks, s); break;
    case 2: launch_q35<InT, BLOCK, 2>(a, sr, e8, fused, strided, rot, blocks, s); break;
    case 3: launch_q35<InT, BLOCK, 3>(a, sr, e8, fused, strided, rot, blocks, s); break;
    case 4: launch_q35<InT, BLOCK, 4>(a, sr, e8, fused, strided, rot, blocks, s); break;
    case 5: launch_q35<InT, BLOCK, 5>(a, sr, e8, fused, strided, rot, blocks, s); break;
    case 6: launch_q35<InT, BLOCK, 6>(a, sr, e8, fused, strided, rot, blocks, s); break;
    default: launch_q35<InT, BLOCK, 0>(a, sr, e8, fused, strided, rot, blocks, s); break;
    }
}

// Compute units of a device (cached; every thread computes the same value).
static int device_cus(int dev)
{
    static std::atomic<int> cache[64];
    if (dev < 0 || dev >= 64) return 0;
    int n = cache[dev].load(std::memory_order_relaxed);
    if (n == 0) {
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
        cache[dev].store(n, std::memory_order_relaxed);
    }
    return n;
}

hipError_t launch_quantize(const QuantLaunch& p, hipStream_t s)
{
    QArgs a;
    a.x = p.x;
    a.nunits = (uint32_t)(p.rows * (p.cols / 8));
    a.upr = make_fastdiv((uint32_t)(p.cols / 8 ? p.cols / 8 : 1));
    a.ld = p.ld;
    a.q = (uint32_t*)p.q;
    a.scales = p.scales;
    a.tensor_scale = p.tensor_scale;
    a.amax_src = p.amax_src;
    a.refresh = p.refresh;
    a.f = ScaleFmt{p.fmt.ebits, p.fmt.mbits, p.fmt.bias, p.fmt.maxcode, p.fmt.smax, p.fmt.is_e8m0};
    a.key0 = (uint32_t)p.seed;
    a.key1 = (uint32_t)(p.seed >> 32);
    a.off0 = (uint32_t)p.offset;
    a.off1 = (uint32_t)(p.offset >> 32);
    a.signs = p.rht_signs;
    a.wait_ticks = __atomic_load_n(&g_exchange_wait_ticks, __ATOMIC_RELAXED);
    const bool sr = p.stochastic != 0, e8 = p.fmt.is_e8m0 != 0, strided = p.ld != p.cols, rot = p.rht != 0;
    const int elem = p.elem;

    // A refresh reads the input once when the whole tensor fits the
    // single-pass grid (at most one workgroup per CU, kFUnroll units per
    // lane); larger tensors take the amax kernel and a second read.
    bool fused = false;
    uint32_t blocks;
    if (a.amax_src && a.refresh && !e8) {
        int dev = 0;
        if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
        const int cus = device_cus(dev);
        const uint32_t per_wg = kFThreads * kFUnroll;
        const uint32_t max_wg = (uint32_t)(cus < kXchgSlots ? cus : kXchgSlots);
        blocks = (a.nunits + per_wg - 1) / per_wg;
        if (blocks == 0) blocks = 1;
        fused = blocks <= max_wg;
        // every single-pass launch that exchanges runs the same grid (each
        // workgroup derives the launch's epoch from its own slot, so every
        // slot must be published by every such launch); workgroups past the
        // tensor publish a zero maximum and store nothing.  A tensor that
        // fits one workgroup runs alone and exchanges nothing.
        if (fused && blocks > 1) blocks = max_wg;
        if (!fused) {
            hipError_t e = launch_amax(p.x, p.x_bf16, p.rows, p.cols, p.ld, p.amax_src, s, rot ? p.block : 0,
                                       p.rht_signs);
            if (e != hipSuccess) return e;
        }
    }
    if (!fused) {
        const uint32_t per_block = kQThreads * kQUnroll;
        blocks = (a.nunits + per_block - 1) / per_block;
        if (blocks == 0) blocks = 1;
    }
    if (p.x_bf16) {
        if (p.block == 16) launch_q3<uint16_t, 16>(a, sr, e8, fused, strided, rot, elem, blocks, s);
        else launch_q3<uint16_t, 32>(a, sr, e8, fused, strided, rot, elem, blocks, s);
    } else {
        if (p.block == 16) launch_q3<float, 16>(a, sr, e8, fused, strided, rot, elem, blocks, s);
        else launch_q3<float, 32>(a, sr, e8, fused, strided, rot, elem, blocks, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// column-wise (transposed) quantize: the quantization of x^T for x [R, C],
// i.e. blocks of B consecutive rows of one column of x (the operands of the
// backward pass are blocked along the token dimension).  Output codes
// [C, R/2] and scales [C, R/B]; the stochastic-rounding index is that of
// x^T, i = c * R + r, so the result equals the row-wise quantization of the
// materialized transpose bit for bit.
//
// A workgroup owns a tile of kTR rows x kTC columns of x: coalesced 16-byte
// row loads into LDS, one barrier, then lane l of every wave takes column l
// and reads its kTR / 4 rows down the tile (consecutive lanes read
// consecutive LDS addresses, so the reads are free of bank conflicts).
// ---------------------------------------------------------------------------
constexpr int kTR = 256;
constexpr int kTC = 64;
constexpr int kTThreads = 256;
#ifndef FP4_T_SR_WAVES
#define FP4_T_SR_WAVES 3
#endif

struct QTArgs {
    const void* x;
    int64_t ld;
    uint32_t R, C;               // x is [R, C]
    uint32_t ntr;                // tiles along R
    uint32_t ntc;                // tiles along C
    uint32_t ntr_pad;            // ROWS kernels: ntr rounded up to a multiple of 8
    uint32_t xcd_chunk;          // consecutive tiles per XCD (0: plain order)
    uint8_t* q;                  // [C, R/2]
    uint8_t* scales;             // [C, R/B]
    float* tensor_scale;
    AmaxDev* amax_src;
    int32_t refresh;
    ScaleFmt f;
    uint32_t key0, key1, off0, off1;
    uint32_t signs;              // Hadamard transform sign mask (ROT kernels)
    uint8_t* q_row;              // ROWS kernels: the row-wise output too,
    uint8_t* s_row;              // codes [R, C/2], scales [R, C/B],
    float* ts_row;               // tensor scale {g, amax}
};

template <typename InT>
__device__ __forceinline__ float lds_elem(const InT* t, uint32_t i);
template <>
__device__ __forceinline__ float lds_elem<uint16_t>(const uint16_t* t, uint32_t i)
{
    return __uint_as_float((uint32_t)t[i] << 16);
}
template <>
__device__ __forceinline__ float lds_elem<float>(const float* t, uint32_t i)
{
    return t[i];
}

// Coalesced 16-byte loads of the tile at (r0, c0) into registers (zeros past
// the edges of x), then their store to the LDS tile.
template <typename InT>
struct TileLoad {
    static constexpr int EPP = 16 / (int)sizeof(InT);   // elements per 16-byte piece
    static constexpr int PPR = kTC / EPP;               // pieces per tile row
    static constexpr int RPR = kTThreads / PPR;         // tile rows per load round
    static constexpr int NLD = kTR / RPR;               // 16-byte loads per thread
    u32x4 v[NLD];
    __device__ __forceinline__ void load(const QTArgs& a, uint32_t r0, uint32_t c0)
    {
        const uint32_t piece = threadIdx.x % PPR, prow = threadIdx.x / PPR;
        const uint32_t gc = c0 + piece * EPP;
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            const uint32_t gr = r0 + prow + k * RPR;
            if (gr < a.R && gc < a.C)
                v[k] = __builtin_nontemporal_load(
                    (const u32x4*)((const InT*)a.x + (uint64_t)gr * (uint64_t)a.ld + gc));
            else
                v[k] = u32x4{0u, 0u, 0u, 0u};
        }
    }
    __device__ __forceinline__ void store(InT* tile) const
    {
        const uint32_t piece = threadIdx.x % PPR, prow = threadIdx.x / PPR;
#pragma unroll
        for (int k = 0; k < NLD; ++k) *(u32x4*)&tile[(prow + k * RPR) * kTC + piece * EPP] = v[k];
    }
};

// Tensor maximum of x transformed blockwise down its columns (the refresh
// of a transformed column-wise call): exactly kAmaxParts workgroups take the
// tiles in a grid stride, stage each through LDS as k_quantize_t does, and
// lane l transforms the blocks of column l; one partial maximum per
// workgroup, reduced by the quantize kernel.
template <typename InT, int BLOCK>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(sizeof(InT) == 4 ? 2 : 4))) void k_amax_t(
    QTArgs a, uint32_t ntiles)
{
    constexpr int RPW = kTR / (kTThreads / 64);
    constexpr int NB = RPW / BLOCK;
    __shared__ __align__(16) InT tile[kTR * kTC];
    const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    uint32_t m = 0;
    for (uint32_t t = blockIdx.x; t < ntiles; t += gridDim.x) {
        const uint32_t tc = t / a.ntr, tr = t - tc * a.ntr;
        TileLoad<InT> ld;
        ld.load(a, tr * kTR, tc * kTC);
        __syncthreads();                         // the previous tile has been read
        ld.store(tile);
        __syncthreads();
        const InT* tw = tile + w * RPW * kTC + lane;
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            float val[BLOCK];
#pragma unroll
            for (int j = 0; j < BLOCK; ++j) val[j] = lds_elem<InT>(tw, (b * BLOCK + j) * kTC);
            rht_forward_lane<BLOCK>(val, a.signs);
#pragma unroll
            for (int j = 0; j < BLOCK; ++j) {
                const uint32_t u = __float_as_uint(val[j]) & 0x7FFFFFFFu;
                m = m > u ? m : u;
            }
        }
    }
    m = wave_umax(m);
    __shared__ uint32_t wmax[kTThreads / 64];
    if (lane == 0) wmax[w] = m;
    __syncthreads();
    if (threadIdx.x == 0) {
        for (int i = 1; i < kTThreads / 64; ++i) m = m > wmax[i] ? m : wmax[i];
        a.amax_src->partial[blockIdx.x] = __uint_as_float(m);
    }
}

// Row-wise quantization of the tile's loaded 16-byte pieces (ROWS kernels):
// piece p of a tile row holds elements c0 + EPP p .. of row r, and the
// BLOCK / EPP pieces of a row block sit in adjacent lanes, so the block
// maximum is a shuffle reduction over those lanes; every rule (scale,
// nearest or stochastic rounding with the row-wise counter index r C + c,
// element grid and packing) is that of the row-wise kernel.
template <typename InT>
__device__ __forceinline__ void unpack_piece(const u32x4& w, float v[16 / sizeof(InT)])
{
    if (sizeof(InT) == 2) {
        v[0] = bf16_lo(w.x); v[1] = bf16_hi(w.x);
        v[2] = bf16_lo(w.y); v[3] = bf16_hi(w.y);
        v[4 % (16 / sizeof(InT))] = bf16_lo(w.z); v[5 % (16 / sizeof(InT))] = bf16_hi(w.z);
        v[6 % (16 / sizeof(InT))] = bf16_lo(w.w); v[7 % (16 / sizeof(InT))] = bf16_hi(w.w);
    } else {
        v[0] = __uint_as_float(w.x); v[1] = __uint_as_float(w.y);
        v[2] = __uint_as_float(w.z); v[3] = __uint_as_float(w.w);
    }
}

template <typename InT, int BLOCK, bool SR, bool E8M0, int ELEM>
__device__ __forceinline__ void rowwise_from_tile(const QTArgs& a, const TileLoad<InT>& ld, uint32_t r0, uint32_t c0,
                                                  float g, float d)
{
    constexpr int EPP = TileLoad<InT>::EPP;
    constexpr int NLD = TileLoad<InT>::NLD;
    constexpr int G = BLOCK / EPP;               // lanes per row block
    constexpr bool INT = ELEM == 1;
    constexpr bool W8 = ELEM == 2 || ELEM == 3;  // one byte per element
    constexpr bool W6 = ELEM >= 4;               // six bits per element
    const uint32_t piece = threadIdx.x % TileLoad<InT>::PPR, prow = threadIdx.x / TileLoad<InT>::PPR;
    const uint32_t gc = c0 + piece * EPP;
    const uint32_t sub = threadIdx.x & (G - 1);  // position of this lane's piece in its block

    // block maxima of every loaded piece, reduced over the block's lanes
    uint32_t bm[NLD];
#pragma unroll
    for (int k = 0; k < NLD; ++k) {
        float v[EPP];
        unpack_piece<InT>(ld.v[k], v);
        uint32_t m = dpp_umax_xor1(absmax_bits_n<EPP>(v));
        if (G >= 4) m = dpp_umax_xor2(m);
        if (G >= 8) {
            const uint32_t t = (uint32_t)__shfl_xor((int)m, 4, 64);
            m = m > t ? m : t;
        }
        bm[k] = m;
    }

    // scales: with G <= 4 lane `sub` computes those of pieces k = sub PER + t
    // and the block's lanes exchange them (DPP within the quad); with G = 8
    // every lane computes its own
    float inv[NLD];
    uint32_t code[NLD];
    auto scale_of = [&](uint32_t m, float* iv) -> uint32_t {
        if (E8M0) {
            const uint32_t c = ELEM == 2 ? scale_code_e8m0_emax<8>(__uint_as_float(m))
                             : ELEM == 3 ? scale_code_e8m0_emax<6>(__uint_as_float(m))
                             : (ELEM == 5 || ELEM == 6) ? scale_code_e8m0_emax<4>(__uint_as_float(m))
                             : scale_code_e8m0(__uint_as_float(m));
            *iv = e8m0_inv(c);
            return c;
        }
        return exmy_scale(__uint_as_float(m), d, g, a.f, iv);
    };
    constexpr bool SHARE = G <= 4;
    if (SHARE) {
        constexpr int PER = NLD / (SHARE ? G : 1);
        float inv_own[PER];
        uint32_t code_own[PER];
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            uint32_t m = bm[t];
#pragma unroll
            for (int j = 1; j < G; ++j) m = (sub == (uint32_t)j) ? bm[(j * PER + t) % NLD] : m;
            code_own[t] = scale_of(m, &inv_own[t]);
        }
#pragma unroll
        for (int t = 0; t < PER; ++t) {
            if (G == 2) {
                const float mine = inv_own[t];
                const float other = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(mine), 0xB1, 0xF, 0xF, false));
                inv[t] = sub == 0 ? mine : other;
                inv[(PER + t) % NLD] = sub == 1 ? mine : other;
            } else {
                inv[t] = quad_bcast<0>(inv_own[t]);
                inv[(PER + t) % NLD] = quad_bcast<1>(inv_own[t]);
                inv[(2 * PER + t) % NLD] = quad_bcast<2>(inv_own[t]);
                inv[(3 * PER + t) % NLD] = quad_bcast<3>(inv_own[t]);
            }
            // this lane stores the scale bytes it computed
            const uint32_t k = sub * PER + t;
            const uint32_t gr = r0 + prow + k * TileLoad<InT>::RPR;
            if (gr < a.R && gc < a.C) a.s_row[(uint64_t)gr * (a.C / BLOCK) + gc / BLOCK] = (uint8_t)code_own[t];
        }
    } else {
#pragma unroll
        for (int k = 0; k < NLD; ++k) {
            code[k] = scale_of(bm[k], &inv[k]);
            const uint32_t gr = r0 + prow + k * TileLoad<InT>::RPR;
            if (sub == 0 && gr < a.R && gc < a.C) a.s_row[(uint64_t)gr * (a.C / BLOCK) + gc / BLOCK] = (uint8_t)code[k];
        }
    }

#pragma unroll
    for (int k = 0; k < NLD; ++k) {
        const uint32_t gr = r0 + prow + k * TileLoad<InT>::RPR;
        float v[EPP];
        unpack_piece<InT>(ld.v[k], v);
#pragma unroll
        for (int i = 0; i < EPP; ++i) v[i] = v[i] * inv[k];
        const bool in = gr < a.R && gc < a.C;
        const uint32_t e0 = gc & 7u;                 // first element of the piece in its unit
        if constexpr (W8 || W6) {
            // the piece's random 16-bit halves (element e of a unit takes
            // half e % 2 of word e / 2), then one code per element
            uint32_t wd[4] = {0u, 0u, 0u, 0u};
            if (SR) {
                const uint32_t u = (uint32_t)(((uint64_t)gr * a.C + gc) >> 3);
                const U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
                wd[0] = r.x; wd[1] = r.y; wd[2] = r.z; wd[3] = r.w;
            }
            auto r16_of = [&](int i) { const uint32_t e = e0 + i; return (wd[e >> 1] >> (16 * (e & 1))) & 0xFFFFu; };
            if constexpr (W8) {
                // bytes of elements 0..3 and 4..7 of the piece
                uint32_t d0, d1 = 0;
                if (SR || ELEM == 3) {
                    uint32_t c[EPP];
#pragma unroll
                    for (int i = 0; i < EPP; ++i)
                        c[i] = SR ? (ELEM == 2 ? fp8_sr_code(v[i], r16_of(i)) : int8_sr_code(v[i], r16_of(i)))
                                  : int8_rtn_code(v[i]);
                    d0 = c[0] | (c[1] << 8) | (c[2 % EPP] << 16) | (c[3 % EPP] << 24);
                    if (EPP == 8) d1 = c[4 % EPP] | (c[5 % EPP] << 8) | (c[6 % EPP] << 16) | (c[7 % EPP] << 24);
                } else {
                    d0 = fp8_rtn_pack4(v[0], v[1], v[2 % EPP], v[3 % EPP]);
                    if (EPP == 8) d1 = fp8_rtn_pack4(v[4 % EPP], v[5 % EPP], v[6 % EPP], v[7 % EPP]);
                }
                if (in) {
                    uint8_t* qd = a.q_row + (uint64_t)gr * a.C + gc;
                    if (EPP == 8) *(u32x2*)qd = u32x2{d0, d1};
                    else *(uint32_t*)qd = d0;
                }
            } else {
                // element i of the piece at bit 6 i
                uint64_t bits = 0;
                if (SR || ELEM == 6) {
#pragma unroll
                    for (int i = 0; i < EPP; ++i)
                        bits |= (uint64_t)(SR ? w6_sr_code<ELEM>(v[i], r16_of(i)) : w6_rtn_code<ELEM>(v[i])) << (6 * i);
                } else {
                    bits = fp6_rtn_pack4_hw<ELEM>(v[0], v[1], v[2 % EPP], v[3 % EPP]);
                    if (EPP == 8) bits |= (uint64_t)fp6_rtn_pack4_hw<ELEM>(v[4 % EPP], v[5 % EPP], v[6 % EPP], v[7 % EPP]) << 24;
                }
                // unit u of the row-major stream at byte 6 u: a whole unit as
                // three 16-bit stores, a half unit (f32 pieces) as three bytes
                // at byte 3 of the unit for its second half
                if (in) {
                    const uint64_t u = ((uint64_t)gr * a.C + gc) >> 3;
                    if (EPP == 8) {
                        uint16_t* dst = reinterpret_cast<uint16_t*>(a.q_row) + 3 * u;
                        dst[0] = (uint16_t)bits;
                        dst[1] = (uint16_t)(bits >> 16);
                        dst[2] = (uint16_t)(bits >> 32);
                    } else {
                        uint8_t* dst = a.q_row + 6 * u + 3 * (e0 >> 2);
                        dst[0] = (uint8_t)bits;
                        dst[1] = (uint8_t)(bits >> 8);
                        dst[2] = (uint8_t)(bits >> 16);
                    }
                }
            }
            continue;
        }
        uint32_t packed = 0;
        if (SR) {
            const uint32_t u = (uint32_t)(((uint64_t)gr * a.C + gc) >> 3);   // unit (i >> 3), row-wise index
            const U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
            const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
            if (INT) {
#pragma unroll
                for (int i = 0; i < EPP; ++i) {
                    const uint32_t e = e0 + i;
                    const uint32_t r16 = (wd[e >> 1] >> (16 * (e & 1))) & 0xFFFFu;
                    packed |= int4_sr_code(v[i], r16) << (4 * i);
                }
            } else if (EPP == 8) {
                packed = e2m1_sr_pack8(v, r.x, r.y, r.z, r.w);
            } else {
                // a 4-element piece: the first or second half of its unit
                packed = e0 ? e2m1_sr_pack4(v[0], v[1], v[2 % EPP], v[3 % EPP], r.z, r.w)
                            : e2m1_sr_pack4(v[0], v[1], v[2 % EPP], v[3 % EPP], r.x, r.y);
            }
        } else if (INT) {
#pragma unroll
            for (int i = 0; i < EPP; ++i) packed |= int4_rtn_code(v[i]) << (4 * i);
        } else {
            packed = FP4_CVT_PK(0u, v[0], v[1], 0);
            packed = FP4_CVT_PK(packed, v[2 % EPP], v[3 % EPP], 1);
            if (EPP == 8) {
                packed = FP4_CVT_PK(packed, v[4 % EPP], v[5 % EPP], 2);
                packed = FP4_CVT_PK(packed, v[6 % EPP], v[7 % EPP], 3);
            }
        }
        // plain (not streaming) stores: each is a 32-byte piece of a line
        // that the neighbouring tiles of the super-tile complete in L2
        if (in) {
            uint8_t* qd = a.q_row + (uint64_t)gr * (a.C / 2) + gc / 2;
            if (EPP == 8) *(uint32_t*)qd = packed;
            else *(uint16_t*)qd = (uint16_t)packed;
        }
    }
}

// ROWS: also the row-wise quantization of the same tile from the loaded
// registers (x read once for both orientations; no transform).
// ELEM: the element grid (0 E2M1, 1 INT4, 2 FP8 E4M3, 3 INT8, 4 FP6 E2M3,
// 5 FP6 E3M2, 6 INT6; the 6-bit ones with R % 64 == 0 so that every
// column-wise output chunk is 16 whole bytes).
template <typename InT, int BLOCK, bool SR, bool E8M0, int ELEM, bool ROT, bool ROWS>
__global__ __launch_bounds__(kTThreads) __attribute__((amdgpu_waves_per_eu(sizeof(InT) == 4 ? 2 : (SR ? FP4_T_SR_WAVES : (ROWS && ELEM != 0 ? 4 : 5))))) void k_quantize_t(QTArgs a)
{
    constexpr bool INT = ELEM == 1;
    constexpr bool W8 = ELEM == 2 || ELEM == 3;
    constexpr bool W6 = ELEM >= 4;
    static_assert(!(ROWS && ROT), "the two orientations would need different transforms and maxima");
    constexpr float QMAX = ELEM == 1 ? 7.0f : ELEM == 2 ? 448.0f : ELEM == 3 ? 127.0f : ELEM == 4 ? 7.5f
                         : ELEM == 5 ? 28.0f : ELEM == 6 ? 31.0f : 6.0f;   // grid maximum
    constexpr int RPW = kTR / (kTThreads / 64);  // rows of every column per wave
    constexpr int NB = RPW / BLOCK;              // blocks per lane
    __shared__ __align__(16) InT tile[kTR * kTC];

    // XCD-aware order: consecutive tiles (down one column strip, which share
    // the lines of the scale rows) run on one XCD
    uint32_t t = blockIdx.x;
    if (a.xcd_chunk) t = (t & 7u) * a.xcd_chunk + (t >> 3);
    uint32_t tc, tr;
    if (ROWS) {
        // super-tiles of 8 (down) x 4 (across) tiles: the 128-byte lines of
        // the row-wise codes (4 tiles across) and of the column-wise scales
        // (8 tiles down) are written by tiles that run close together on
        // one XCD.  The grid is padded to whole super-tiles.
        const uint32_t st = t >> 5, wi = t & 31u, nsr = a.ntr_pad >> 3;
        tr = (st % nsr) * 8 + (wi & 7u);
        tc = (st / nsr) * 4 + (wi >> 3);
        // padding (whole workgroup); workgroup 0 always runs (it writes the
        // tensor scale, and every load and store below is bounds-checked)
        if ((tr >= a.ntr || tc >= a.ntc) && blockIdx.x != 0) return;
    } else {
        tc = t / a.ntr;
        tr = t - tc * a.ntr;
    }
    const uint32_t r0 = tr * kTR, c0 = tc * kTC;

    TileLoad<InT> ld;
    ld.load(a, r0, c0);

    float g = 1.0f, d = QMAX;
    if (!E8M0 && a.amax_src) {
        const float am = tensor_amax(a);
        g = tensor_scale_of(am, a, QMAX);
        d = QMAX * g;
        if (blockIdx.x == 0 && threadIdx.x == 0) {
            a.tensor_scale[0] = g;
            a.tensor_scale[1] = am;
            if (ROWS) {
                a.ts_row[0] = g;
                a.ts_row[1] = am;
            }
            if (a.refresh) a.amax_src->stored = am;
        }
    } else if (blockIdx.x == 0 && threadIdx.x == 0) {
        a.tensor_scale[0] = 1.0f;
        a.tensor_scale[1] = 0.0f;
        if (ROWS) {
            a.ts_row[0] = 1.0f;
            a.ts_row[1] = 0.0f;
        }
    }

    ld.store(tile);
    if (ROWS) rowwise_from_tile<InT, BLOCK, SR, E8M0, ELEM>(a, ld, r0, c0, g, d);
    __syncthreads();

    const uint32_t lane = threadIdx.x & 63, w = threadIdx.x >> 6;
    const uint32_t col = c0 + lane;
    const uint32_t rw = r0 + w * RPW;            // first row of x in this wave's blocks
    const InT* tw = tile + w * RPW * kTC + lane;

    // codes of this lane's NB blocks (column `col`, rows rw ..) and their
    // scale bytes; blocks past the end of x (R % BLOCK == 0, so blocks are
    // whole) compute on zeros and are never stored
    uint32_t packed[NB][W8 ? BLOCK / 4 : W6 ? BLOCK * 3 / 16 : BLOCK / 8];
    uint32_t sc = 0;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const uint32_t rb = rw + b * BLOCK;
        float val[BLOCK];
        uint32_t m = 0;
#pragma unroll
        for (int j = 0; j < BLOCK; ++j) val[j] = lds_elem<InT>(tw, (b * BLOCK + j) * kTC);
        if (ROT) rht_forward_lane<BLOCK>(val, a.signs);
#pragma unroll
        for (int j = 0; j < BLOCK; ++j) {
            const uint32_t u = __float_as_uint(val[j]) & 0x7FFFFFFFu;
            m = m > u ? m : u;
        }
        float inv;
        uint32_t code;
        if (E8M0) {
            code = ELEM == 2 ? scale_code_e8m0_emax<8>(__uint_as_float(m))
                 : ELEM == 3 ? scale_code_e8m0_emax<6>(__uint_as_float(m))
                 : (ELEM == 5 || ELEM == 6) ? scale_code_e8m0_emax<4>(__uint_as_float(m))
                 : scale_code_e8m0(__uint_as_float(m));
            inv = e8m0_inv(code);
        } else {
            code = exmy_scale(__uint_as_float(m), d, g, a.f, &inv);
        }
        sc |= code << (8 * b);
#pragma unroll
        for (int k = 0; k < BLOCK / 8; ++k) {
            float e[8];
#pragma unroll
            for (int i = 0; i < 8; ++i) e[i] = val[k * 8 + i] * inv;
            if constexpr (W6) {
                // six bits per element: unit k's 48 bits at bit 48 k of the block
                uint64_t bits = 0;
                if (SR) {
                    const uint32_t u = col * (a.R / 8u) + (rb >> 3) + k;  // unit (i >> 3) of x^T
                    U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
                    const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i)
                        bits |= (uint64_t)w6_sr_code<ELEM>(e[i], (wd[i >> 1] >> (16 * (i & 1))) & 0xFFFFu) << (6 * i);
                } else if (ELEM == 6) {
#pragma unroll
                    for (int i = 0; i < 8; ++i) bits |= (uint64_t)w6_rtn_code<ELEM>(e[i]) << (6 * i);
                } else {
                    bits = (uint64_t)fp6_rtn_pack4_hw<ELEM>(e[0], e[1], e[2], e[3]) |
                           ((uint64_t)fp6_rtn_pack4_hw<ELEM>(e[4], e[5], e[6], e[7]) << 24);
                }
                // units pair up into three dwords: even k fills dword 3k/2 and
                // the low half of the next, odd k the high half and the one after
                if ((k & 1) == 0) {
                    packed[b][3 * k / 2] = (uint32_t)bits;
                    packed[b][3 * k / 2 + 1] = (uint32_t)(bits >> 32);
                } else {
                    packed[b][3 * (k - 1) / 2 + 1] |= (uint32_t)bits << 16;
                    packed[b][3 * (k - 1) / 2 + 2] = (uint32_t)(bits >> 16);
                }
                continue;
            }
            if constexpr (W8) {
                // one byte per element: the unit's eight codes in two dwords
                if (SR) {
                    const uint32_t u = col * (a.R / 8u) + (rb >> 3) + k;  // unit (i >> 3) of x^T
                    U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
                    const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
                    uint32_t c[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t r16 = (wd[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                        c[i] = ELEM == 2 ? fp8_sr_code(e[i], r16) : int8_sr_code(e[i], r16);
                    }
                    packed[b][2 * k] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
                    packed[b][2 * k + 1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
                } else if (ELEM == 2) {
                    packed[b][2 * k] = fp8_rtn_pack4(e[0], e[1], e[2], e[3]);
                    packed[b][2 * k + 1] = fp8_rtn_pack4(e[4], e[5], e[6], e[7]);
                } else {
                    uint32_t c[8];
#pragma unroll
                    for (int i = 0; i < 8; ++i) c[i] = int8_rtn_code(e[i]);
                    packed[b][2 * k] = c[0] | (c[1] << 8) | (c[2] << 16) | (c[3] << 24);
                    packed[b][2 * k + 1] = c[4] | (c[5] << 8) | (c[6] << 16) | (c[7] << 24);
                }
                continue;
            }
            if (SR) {
                const uint32_t u = col * (a.R / 8u) + (rb >> 3) + k;      // unit (i >> 3) of x^T
                U4 r = philox10(U4{u, 0u, a.off0, a.off1}, a.key0, a.key1);
                uint32_t pk = 0;
                if (INT) {
                    const uint32_t wd[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const uint32_t r16 = (wd[i >> 1] >> (16 * (i & 1))) & 0xFFFFu;
                        pk |= int4_sr_code(e[i], r16) << (4 * i);
                    }
                } else {
                    pk = e2m1_sr_pack8(e, r.x, r.y, r.z, r.w);
                }
                packed[b][k] = pk;
            } else if (INT) {
                uint32_t pk = 0;
#pragma unroll
                for (int i = 0; i < 8; ++i) pk |= int4_rtn_code(e[i]) << (4 * i);
                packed[b][k] = pk;
            } else {
                uint32_t pk = FP4_CVT_PK(0u, e[0], e[1], 0);
                pk = FP4_CVT_PK(pk, e[2], e[3], 1);
                pk = FP4_CVT_PK(pk, e[4], e[5], 2);
                packed[b][k] = FP4_CVT_PK(pk, e[6], e[7], 3);
            }
        }
    }

    // Stage the tile's output in LDS ([kTC] output rows of kTR/2 code bytes
    // and kTR/BLOCK scale bytes), then store whole row pieces: each wave
    // store instruction covers full 128-byte lines of eight output rows,
    // instead of one 8- or 16-byte piece per lane in 64 different rows.
    constexpr int QB = W8 ? kTR : W6 ? kTR * 3 / 4 : kTR / 2;   // code bytes per output row and tile
    constexpr int QP = QB + 16;                  // padded LDS pitch
    constexpr int SB = kTR / BLOCK;              // scale bytes per output row and tile
    static_assert(kTC * (QP + SB) <= kTR * kTC * (int)sizeof(InT), "output stage fits the input tile");
    uint8_t* oq = reinterpret_cast<uint8_t*>(tile);
    uint8_t* os = oq + kTC * QP;
    __syncthreads();                             // every wave has read its rows of the tile
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if constexpr (W6) {
            uint32_t* dst = reinterpret_cast<uint32_t*>(oq + lane * QP + (w * RPW + b * BLOCK) * 3 / 4);
#pragma unroll
            for (int v = 0; v < BLOCK * 3 / 16; ++v) dst[v] = packed[b][v];
        } else if constexpr (W8) {
            uint8_t* dst = oq + lane * QP + (w * RPW + b * BLOCK);
#pragma unroll
            for (int v = 0; v < BLOCK / 16; ++v)
                *(u32x4*)(dst + 16 * v) =
                    u32x4{packed[b][4 * v], packed[b][4 * v + 1], packed[b][4 * v + 2], packed[b][4 * v + 3]};
        } else {
            uint8_t* dst = oq + lane * QP + (w * RPW + b * BLOCK) / 2;
            if (BLOCK == 16) *(u32x2*)dst = u32x2{packed[b][0], packed[b][1]};
            else *(u32x4*)dst = u32x4{packed[b][0], packed[b][1], packed[b][2], packed[b][3]};
        }
    }
    if (NB == 4) *(uint32_t*)(os + lane * SB + w * NB) = sc;
    else *(uint16_t*)(os + lane * SB + w * NB) = (uint16_t)sc;
    __syncthreads();

    const uint32_t rows_here = a.R - r0 < (uint32_t)kTR ? a.R - r0 : (uint32_t)kTR;   // multiple of BLOCK
    const uint32_t qbytes = W8 ? rows_here : W6 ? rows_here / 4 * 3 : rows_here / 2, sbytes = rows_here / BLOCK;
    const uint64_t qrow = W8 ? a.R : W6 ? a.R / 4 * 3 : a.R / 2, srow = a.R / BLOCK;
    const bool q16 = (qrow & 15u) == 0;          // 16-byte aligned output rows
    constexpr int QCH = QB / 16;                 // 16-byte chunks per output row
#pragma unroll
    for (int k = 0; k < kTC * QCH / kTThreads; ++k) {
        const uint32_t p = threadIdx.x + k * kTThreads;
        const uint32_t orow = p / QCH, ch = p % QCH;
        const uint32_t oc = c0 + orow;
        if (oc >= a.C || ch * 16 >= qbytes) continue;
        const u32x4 v4 = *(const u32x4*)(oq + orow * QP + ch * 16);
        uint8_t* g8 = a.q + (uint64_t)oc * qrow + (W8 ? r0 : W6 ? r0 / 4 * 3 : r0 / 2) + ch * 16;
        if (q16 && ch * 16 + 16 <= qbytes) {
            __builtin_nontemporal_store(v4, (u32x4*)g8);
        } else {
            __builtin_nontemporal_store(u32x2{v4.x, v4.y}, (u32x2*)g8);
            if (ch * 16 + 16 <= qbytes) __builtin_nontemporal_store(u32x2{v4.z, v4.w}, (u32x2*)(g8 + 8));
        }
    }
    if (threadIdx.x < kTC) {
        const uint32_t oc = c0 + threadIdx.x;
        if (oc < a.C) {
            const uint8_t* src = os + threadIdx.x * SB;
            uint8_t* g8 = a.scales + (uint64_t)oc * srow + r0 / BLOCK;
            if ((srow % SB) == 0 && sbytes == (uint32_t)SB && ((uintptr_t)a.scales % SB) == 0) {
                if (SB == 16) *(u32x4*)g8 = *(const u32x4*)src;
                else *(u32x2*)g8 = *(const u32x2*)src;
            } else {
                for (uint32_t i = 0; i < sbytes; ++i) g8[i] = src[i];
            }
        }
    }
}

template <typename InT, int BLOCK, int ELEM, bool ROT, bool ROWS>
static void launch_qt3(const QTArgs& a, bool sr, bool e8, uint32_t blocks, hipStream_t s)
{
    const dim3 g(blocks), t(kTThreads);
    if (sr) {
        if (e8) hipLaunchKernelGGL((k_quantize_t<InT, BLOCK, true, true, ELEM, ROT, ROWS>), g, t, 0, s, a);
        else hipLaunchKernelGGL((k_quantize_t<InT, BLOCK, true, false, ELEM, ROT, ROWS>), g, t, 0, s, a);
    } else {
        if (e8) hipLaunchKernelGGL((k_quantize_t<InT, BLOCK, false, true, ELEM, ROT, ROWS>), g, t, 0, s, a);
        else hipLaunchKernelGGL((k_quantize_t<InT, BLOCK, false, false, ELEM, ROT, ROWS>), g, t, 0, s, a);
    }
}

// rows: the two-orientation variant (never with a transform)
template <typename InT, int BLOCK>
static void launch_qt2(const QTArgs& a, bool sr, bool e8, int elem, bool rot, bool rows, uint32_t blocks,
                       hipStream_t s)
{
    if (rows) {
        switch (elem) {
        case 1: launch_qt3<InT, BLOCK, 1, false, true>(a, sr, e8, blocks, s); break;
        case 2: launch_qt3<InT, BLOCK, 2, false, true>(a, sr, e8, blocks, s); break;
        case 3: launch_qt3<InT, BLOCK, 3, false, true>(a, sr, e8, blocks, s); break;
        case 4: launch_qt3<InT, BLOCK, 4, false, true>(a, sr, e8, blocks, s); break;
        case 5: launch_qt3<InT, BLOCK, 5, false, true>(a, sr, e8, blocks, s); break;
        case 6: launch_qt3<InT, BLOCK, 6, false, true>(a, sr, e8, blocks, s); break;
        default: launch_qt3<InT, BLOCK, 0, false, true>(a, sr, e8, blocks, s); break;
        }
        return;
    }
    switch (elem) {
    case 1:
        if (rot) launch_qt3<InT, BLOCK, 1, true, false>(a, sr, e8, blocks, s);
        else launch_qt3<InT, BLOCK, 1, false, false>(a, sr, e8, blocks, s);
        break;
    case 2:
        if (rot) launch_qt3<InT, BLOCK, 2, true, false>(a, sr, e8, blocks, s);
        else launch_qt3<InT, BLOCK, 2, false, false>(a, sr, e8, blocks, s);
        break;
    case 3:
        if (rot) launch_qt3<InT, BLOCK, 3, true, false>(a, sr, e8, blocks, s);
        else launch_qt3<InT, BLOCK, 3, false, false>(a, sr, e8, blocks, s);
        break;
    case 4:
        if (rot) launch_qt3<InT, BLOCK, 4, true, false>(a, sr, e8, blocks, s);
        else launch_qt3<InT, BLOCK, 4, false, false>(a, sr, e8, blocks, s);
        break;
    case 5:
        if (rot) launch_qt3<InT, BLOCK, 5, true, false>(a, sr, e8, blocks, s);
        else launch_qt3<InT, BLOCK, 5, false, false>(a, sr, e8, blocks, s);
        break;
    case 6:
        if (rot) launch_qt3<InT, BLOCK, 6, true, false>(a, sr, e8, blocks, s);
        else launch_qt3<InT, BLOCK, 6, false, false>(a, sr, e8, blocks, s);
        break;
    default:
        if (rot) launch_qt3<InT, BLOCK, 0, true, false>(a, sr, e8, blocks, s);
        else launch_qt3<InT, BLOCK, 0, false, false>(a, sr, e8, blocks, s);
        break;
    }
}

template <typename InT>
static void launch_amax_t(const QTArgs& a, int block, uint32_t ntiles, hipStream_t s)
{
    const dim3 g(kAmaxParts), t(kTThreads);
    if (block == 16) hipLaunchKernelGGL((k_amax_t<InT, 16>), g, t, 0, s, a, ntiles);
    else hipLaunchKernelGGL((k_amax_t<InT, 32>), g, t, 0, s, a, ntiles);
}

// p.rows / p.cols are the output's shape (C, R); x is [R, C] with row stride
// p.ld.  A refresh takes an amax kernel first (x is read twice): the row-wise
// one, or the tiled one when the blocks are transformed.
hipError_t launch_quantize_t(const QuantLaunch& p, hipStream_t s, const RowOut* rows)
{
    QTArgs a;
    a.q_row = rows ? rows->q : nullptr;
    a.s_row = rows ? rows->scales : nullptr;
    a.ts_row = rows ? rows->tensor_scale : nullptr;
    a.x = p.x;
    a.ld = p.ld;
    a.R = (uint32_t)p.cols;
    a.C = (uint32_t)p.rows;
    const uint32_t ntr = (a.R + kTR - 1) / kTR, ntc = (a.C + kTC - 1) / kTC;
    const uint32_t ntiles = ntr * ntc;
    a.ntr = ntr ? ntr : 1;
    a.ntc = ntc;
    a.ntr_pad = (a.ntr + 7) & ~7u;
    const uint32_t grid_tiles = rows ? a.ntr_pad * ((ntc + 3) & ~3u) : ntiles;     // super-tile padding
    a.xcd_chunk = (grid_tiles % 8 == 0) ? grid_tiles / 8 : 0;
    a.q = p.q;
    a.scales = p.scales;
    a.tensor_scale = p.tensor_scale;
    a.amax_src = p.amax_src;
    a.refresh = p.refresh;
    a.f = ScaleFmt{p.fmt.ebits, p.fmt.mbits, p.fmt.bias, p.fmt.maxcode, p.fmt.smax, p.fmt.is_e8m0};
    a.key0 = (uint32_t)p.seed;
    a.key1 = (uint32_t)(p.seed >> 32);
    a.off0 = (uint32_t)p.offset;
    a.off1 = (uint32_t)(p.offset >> 32);
    a.signs = p.rht_signs;
    const bool sr = p.stochastic != 0, e8 = p.fmt.is_e8m0 != 0, rot = p.rht != 0;
    const int elem = p.elem;
    if (a.amax_src && a.refresh && !e8) {
        if (rot) {
            // the maximum of the column-transformed tensor
            if (p.x_bf16) launch_amax_t<uint16_t>(a, p.block, ntiles, s);
            else launch_amax_t<float>(a, p.block, ntiles, s);
            hipError_t e = hipGetLastError();
            if (e != hipSuccess) return e;
        } else {
            hipError_t e = launch_amax(p.x, p.x_bf16, a.R, a.C, p.ld, p.amax_src, s);
            if (e != hipSuccess) return e;
        }
    }
    const uint32_t blocks = grid_tiles ? grid_tiles : 1;
    if (p.x_bf16) {
        if (p.block == 16) launch_qt2<uint16_t, 16>(a, sr, e8, elem, rot, rows != nullptr, blocks, s);
        else launch_qt2<uint16_t, 32>(a, sr, e8, elem, rot, rows != nullptr, blocks, s);
    } else {
        if (p.block == 16) launch_qt2<float, 16>(a, sr, e8, elem, rot, rows != nullptr, blocks, s);
        else launch_qt2<float, 32>(a, sr, e8, elem, rot, rows != nullptr, blocks, s);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// dequantize: y = RN(RN(e2m1 * s) * g), bf16 output rounded once more (RNE)
// ---------------------------------------------------------------------------
constexpr int kDQThreads = 256;
constexpr int kDQUnroll = 4;                 // units per lane, loads issued together

// Each wave dequantizes kDQUnroll * 64 consecutive units; unit j of a lane
// is base + 64 j + lane, so every load and store instruction of a wave
// covers a contiguous span.
// ROT: the inverse blockwise Hadamard transform follows the binary32
// dequantization (the G units of a block are adjacent lanes and are all in
// range or all out of it).
typedef __bf16 dq_v2bf __attribute__((ext_vector_type(2)));
typedef float dq_v2f __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16_pair(float a, float b)
{
    return __builtin_bit_cast(uint32_t, dq_v2bf{(__bf16)a, (__bf16)b});
}

template <bool OUT_BF16, int BLOCK, bool E8M0, bool ROT, int ELEM>
__global__ __launch_bounds__(kDQThreads) void k_dequantize(const uint32_t* __restrict__ q,
                                                           const uint8_t* __restrict__ scales,
                                                           const float* __restrict__ tensor_scale, uint32_t nunits,
                                                           FastDiv upr, int64_t ld, int strided, ScaleFmt f,
                                                           void* __restrict__ y, uint32_t signs)
{
    constexpr int U = kDQUnroll;
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t wave = blockIdx.x * (kDQThreads / 64) + (threadIdx.x >> 6);
    const uint32_t base = wave * (64u * U);
    constexpr bool W8 = ELEM == 2 || ELEM == 3;  // one byte per element
    constexpr bool W6 = ELEM >= 4;               // six bits per element
    uint32_t w[U], w2[U], sc[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const uint32_t u = base + j * 64 + lane;
        const uint32_t uu = u < nunits ? u : nunits - 1;           // in bounds; not stored
        if (W6) {
            const uint16_t* src = reinterpret_cast<const uint16_t*>(q) + 3 * (uint64_t)uu;
            w[j] = (uint32_t)__builtin_nontemporal_load(src) | ((uint32_t)__builtin_nontemporal_load(src + 1) << 16);
            w2[j] = (uint32_t)__builtin_nontemporal_load(src + 2);
        } else if (W8) {
            const u32x2 p2 = __builtin_nontemporal_load(reinterpret_cast<const u32x2*>(q) + uu);
            w[j] = p2.x;
            w2[j] = p2.y;
        } else {
            w[j] = __builtin_nontemporal_load(q + uu);
            w2[j] = 0u;
        }
        sc[j] = scales[uu / (BLOCK / 8)];
    }
    const float g = tensor_scale[0];
#pragma unroll
    for (int j = 0; j < U; ++j) {
        const uint32_t u = base + j * 64 + lane;
        if (u >= nunits) continue;
        const float s = scale_decode_any(sc[j], f);
        float o[8];
        // E2M1 pairs by the hardware conversion (scale 1: the exact values)
        float e2[8];
        if (ELEM == 0) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const dq_v2f pe = b == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 0)
                                : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 1)
                                : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 2)
                                         : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[j], 1.0f, 3);
                e2[2 * b] = pe[0];
                e2[2 * b + 1] = pe[1];
            }
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float e;
            if (ELEM == 0) {
                e = e2[k];
            } else if (W6) {
                // bits 6k .. 6k + 5 of the 48-bit unit (w2 holds bits 32..47)
                const uint64_t bits = (uint64_t)w[j] | ((uint64_t)w2[j] << 32);
                e = w6_value<ELEM>((uint32_t)(bits >> (6 * k)) & 0x3Fu);
            } else if (W8) {
                const uint32_t b = ((k < 4 ? w[j] : w2[j]) >> (8 * (k & 3))) & 0xFFu;
                e = ELEM == 2 ? scale_decode_any(b, kFp8E4M3) : int8_value(b);
            } else {
                e = int4_value((w[j] >> (4 * k)) & 0xFu);
            }
            float t = e * s;
            o[k] = t * g;
        }
        if (ROT) rht_inverse<BLOCK / 8>(o, lane & (BLOCK / 8 - 1), signs);
        const uint64_t off = unit_offset(u, strided, upr, ld);
        if (OUT_BF16) {
            // the hardware pair conversion rounds to nearest even, as the
            // bit-level rounding does for every finite value
            u32x4 r;
            r.x = bf16_pair(o[0], o[1]);
            r.y = bf16_pair(o[2], o[3]);
            r.z = bf16_pair(o[4], o[5]);
            r.w = bf16_pair(o[6], o[7]);
            __builtin_nontemporal_store(r, reinterpret_cast<u32x4*>((uint16_t*)y + off));
        } else {
            f32x4* pp = reinterpret_cast<f32x4*>((float*)y + off);
            __builtin_nontemporal_store(f32x4{o[0], o[1], o[2], o[3]}, pp);
            __builtin_nontemporal_store(f32x4{o[4], o[5], o[6], o[7]}, pp + 1);
        }
    }
}

template <bool OUT_BF16, int BLOCK, bool ROT, int ELEM>
static void launch_dq4(const DequantLaunch& p, uint32_t nunits, const FastDiv& fd, int strided, const ScaleFmt& f,
                       hipStream_t s)
{
    const uint32_t per_block = kDQThreads * kDQUnroll;
    uint32_t blocks = (nunits + per_block - 1) / per_block;
    if (blocks == 0) blocks = 1;
    if (f.is_e8m0)
        hipLaunchKernelGGL((k_dequantize<OUT_BF16, BLOCK, true, ROT, ELEM>), dim3(blocks), dim3(kDQThreads), 0, s,
                           (const uint32_t*)p.q, p.scales, p.tensor_scale, nunits, fd, p.ld, strided, f, p.y,
                           p.rht_signs);
    else
        hipLaunchKernelGGL((k_dequantize<OUT_BF16, BLOCK, false, ROT, ELEM>), dim3(blocks), dim3(kDQThreads), 0, s,
                           (const uint32_t*)p.q, p.scales, p.tensor_scale, nunits, fd, p.ld, strided, f, p.y,
                           p.rht_signs);
}

template <bool OUT_BF16, int BLOCK>
static void launch_dq2(const DequantLaunch& p, uint32_t nunits, const FastDiv& fd, int strided, const ScaleFmt& f,
                       hipStream_t s)
{
    switch (p.elem) {
    case 1:
        if (p.rht) launch_dq4<OUT_BF16, BLOCK, true, 1>(p, nunits, fd, strided, f, s);
        else launch_dq4<OUT_BF16, BLOCK, false, 1>(p, nunits, fd, strided, f, s);
        break;
    case 2:
        if (p.rht) launch_dq4<OUT_BF16, BLOCK, true, 2>(p, nunits, fd, strided, f, s);
        else launch_dq4<OUT_BF16, BLOCK, false, 2>(p, nunits, fd, strided, f, s);
        break;
    case 3:
        if (p.rht) launch_dq4<OUT_BF16, BLOCK, true, 3>(p, nunits, fd, strided, f, s);
        else launch_dq4<OUT_BF16, BLOCK, false, 3>(p, nunits, fd, strided, f, s);
        break;
    case 4:
        if (p.rht) launch_dq4<OUT_BF16, BLOCK, true, 4>(p, nunits, fd, strided, f, s);
        else launch_dq4<OUT_BF16, BLOCK, false, 4>(p, nunits, fd, strided, f, s);
        break;
    case 5:
        if (p.rht) launch_dq4<OUT_BF16, BLOCK, true, 5>(p, nunits, fd, strided, f, s);
        else launch_dq4<OUT_BF16, BLOCK, false, 5>(p, nunits, fd, strided, f, s);
        break;
    case 6:
        if (p.rht) launch_dq4<OUT_BF16, BLOCK, true, 6>(p, nunits, fd, strided, f, s);
        else launch_dq4<OUT_BF16, BLOCK, false, 6>(p, nunits, fd, strided, f, s);
        break;
    default:
        if (p.rht) launch_dq4<OUT_BF16, BLOCK, true, 0>(p, nunits, fd, strided, f, s);
        else launch_dq4<OUT_BF16, BLOCK, false, 0>(p, nunits, fd, strided, f, s);
        break;
    }
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
