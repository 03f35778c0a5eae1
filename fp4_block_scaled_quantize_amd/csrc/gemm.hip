// gemm.hip -- block-scaled FP4 x FP4 -> bf16 GEMM for gfx950.
//
// C[M, N] = bf16_RNE(ga * gb * sum_k (e2m1(a_mk) s_a)(e2m1(w_nk) s_w)), fp32
// accumulation, both operands blocked along K and stored K-major (A [M, K],
// W [N, K]; C = A W^T).  ue5m3-fp4-pretraining "Что сделали": the linear
// layers run in FP4; quant_prune_distill/574 "Выводы": weight + activation
// FP4 for the compute-bound regime.
//
// Kernels (each computes the transposed tile D = W A^T, so that each lane
// owns consecutive output columns of C; workgroup tile 256 x 256; codes and
// scale bytes reach LDS by direct-to-LDS loads in multi-stage pipelines; the
// C tile leaves through LDS as whole 16-byte row pieces):
//  * k_gemm_mx: both operands E8M0 at block 32 (MXFP4).  The gfx950
//    block-scaled matrix instruction v_mfma_scale_f32_32x32x64_f8f6f4 takes
//    FP4 operands and one E8M0 scale per 32 K-elements per row directly: lane
//    l supplies row (l % 32), K-half (l / 32) as 16 contiguous bytes -- the
//    packed row-major layout of the quantizer -- and that K-half's scale
//    byte.  No dequantization.  Eight waves of 128 x 64.
//  * k_gemm_mx16: E8M0 at block 16 on the same instruction, each 64-element
//    step run twice with the other 16-element block of A zeroed.
//  * k_gemm_nv: scale formats whose e2m1 * s products are exact in f16
//    (E4M3 -- NVFP4 --, E3M4, E2M5, E1M6) or, with more exponent bits
//    (UE5M3, E5M2, E6M1, E7M0), in bf16: each wave converts its fragments in
//    registers right before the f16 / bf16 32x32x16 matrix instruction; the
//    same kernel takes MXFP8 (FP8 elements, E8M0 scales) to bf16 and INT8
//    with E4M3 scales to f16.
//  * k_gemm_dq: the remaining pairs (E8M0 with a non-power-of-two format)
//    and the INT4, other 8-bit and 6-bit pairings: FP4 / integer / FP8 / FP6
//    tiles are dequantized exactly to f16 or bf16 in LDS.
//  * k_gemm_small: small products (E2M1 with f16- / bf16-exact ExMy or E8M0
//    scales, MXFP8, INT8 with E4M3 scales; M * N up to a process-wide
//    bound): one wave per 32 x 32 output
//    tile, operands straight from global memory into registers, the same
//    conversions and matrix instructions, no LDS.
//  * k_wo_gemm: the weight-only GEMM (bf16 X times W on any element grid,
//    M <= 16).
#include <type_traits>

#include "fp4_device.hpp"
#include "fp4_internal.h"

namespace fp4 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 v8bf __attribute__((ext_vector_type(8)));
typedef __bf16 v2bf __attribute__((ext_vector_type(2)));
typedef _Float16 v8h __attribute__((ext_vector_type(8)));

constexpr int kTile = 256;        // workgroup tile (rows of W) x (rows of A)
constexpr int kGemmThreads = 256;

// ---------------------------------------------------------------------------
// epilogue: acc[i][j] holds D[n = 32 i + 8 q + 4 (l/32) + e][m = 32 j + l%32]
// for register r = 4 q + e; scale by g and store as bf16 into C[m][n].
// ---------------------------------------------------------------------------
__device__ __forceinline__ void store_tile(const v16f (&acc)[4][4], float g, uint16_t* __restrict__ c, int64_t ldc,
                                           int64_t m_base, int64_t n_base, int64_t M, int64_t N)
{
    // 8-byte stores need 8-byte aligned rows; otherwise store element-wise
    const bool vec = ((ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(c) & 7) == 0);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int64_t m = m_base + 32 * j + (lane & 31);
        if (m >= M) continue;
        uint16_t* crow = c + m * ldc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n_base + 32 * i + 8 * q + 4 * (lane >> 5);
                const uint32_t b0 = f32_to_bf16_rne(acc[i][j][4 * q + 0] * g);
                const uint32_t b1 = f32_to_bf16_rne(acc[i][j][4 * q + 1] * g);
                const uint32_t b2 = f32_to_bf16_rne(acc[i][j][4 * q + 2] * g);
                const uint32_t b3 = f32_to_bf16_rne(acc[i][j][4 * q + 3] * g);
                if (vec && n + 3 < N) {
                    uint2 v;
                    v.x = b0 | (b1 << 16);
                    v.y = b2 | (b3 << 16);
                    *reinterpret_cast<uint2*>(crow + n) = v;
                } else {
                    if (n + 0 < N) crow[n + 0] = (uint16_t)b0;
                    if (n + 1 < N) crow[n + 1] = (uint16_t)b1;
                    if (n + 2 < N) crow[n + 2] = (uint16_t)b2;
                    if (n + 3 < N) crow[n + 3] = (uint16_t)b3;
                }
            }
        }
    }
}

// ---------------------------------------------------------------------------
// MXFP4: native block-scaled FP4 matrix instruction
// ---------------------------------------------------------------------------
// Output tile order.  Workgroups are dispatched round-robin over the 8 XCDs
// (each with its own L2); remap so every XCD walks a contiguous band of
// tiles, ordered in groups of 4 tile-rows, so the A and W panels a band
// touches stay in that XCD's L2.
__device__ __forceinline__ void tile_coords(int tiles_n, int tiles_m, int* tn, int* tm)
{
    const int nt = tiles_n * tiles_m;
    int r = blockIdx.x;
    if ((nt % 8) == 0) r = (r % 8) * (nt / 8) + r / 8;
    constexpr int GM = 4;
    const int band = GM * tiles_n;
    const int g = r / band, in = r % band;
    const int rows_in = (g * GM + GM <= tiles_m) ? GM : tiles_m - g * GM;
    *tm = g * GM + in % rows_in;
    *tn = in / rows_in;
}

// ---------------------------------------------------------------------------
// MXFP4: operands go HBM -> LDS with the gfx950 direct-to-LDS loads
// (global_load_lds_dwordx4: each lane's 16 bytes land at LDS base + 16 *
// lane) through NS stages of BK K-elements, one barrier per stage, and from
// LDS straight into v_mfma_scale_f32_32x32x64_f8f6f4.  Eight waves, two per
// SIMD (each 128 x 64 of the 256 x 256 tile, 128 accumulator registers), so
// one wave's matrix instructions overlap the other's LDS reads and barrier
// waits.  The LDS image of a row is XOR-swizzled in 16-byte chunks so that
// the 32 rows one fragment read touches land on distinct banks; the swizzle
// is applied by choosing each lane's global source address.
// ---------------------------------------------------------------------------
constexpr int kMx4Threads = 512;
constexpr int kMx3BK = 128;                          // K elements per stage (f16 path)
constexpr int kMx3RB = kMx3BK / 2;                   // 64 bytes of codes per row
constexpr int kMx3Codes = kTile * kMx3RB;            // 16 KiB per operand per stage

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void dma16(const void* g, uint8_t* lds)
{
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 16, 0, 0);
}
__device__ __forceinline__ void dma4(const void* g, uint8_t* lds)
{
    __builtin_amdgcn_global_load_lds(g, (lds_ptr_t)lds, 4, 0, 0);
}

template <int BK>
struct MxStage {
    static constexpr int RB = BK / 2;                 // code bytes per row per stage
    static constexpr int CPR = RB / 16;               // 16-byte chunks per row
    static constexpr int RPI = 64 / CPR;              // rows per DMA instruction
    static constexpr int NI = kTile / (8 * RPI);      // DMA instructions per wave per operand
    static constexpr int Codes = kTile * RB;          // per operand
    static constexpr int SRow = BK / 32;              // E8M0 bytes per row per stage
    static constexpr int Scales = kTile * SRow;       // per operand
    static constexpr int SDma = 2 * Scales / (4 * kMx4Threads);   // dword DMAs per lane
    // 256-element stages keep the scales out of the stage: 32 bytes per row
    // (four stages) arrive at once, two lanes per row, into one of two
    // group buffers after the stages
    static constexpr bool Grouped = BK == 256;
    static constexpr int GroupStages = 4;
    static constexpr int GroupRow = GroupStages * SRow;               // 32 bytes
    static constexpr int GroupBytes = 2 * kTile * GroupRow;           // W then A: 16 KiB
    static constexpr int Bytes = 2 * Codes + (Grouped ? 0 : 2 * Scales);
};

// Position of 16-byte chunk c of row r: c ^ mx_swz(r).  64-byte rows:
// ((r >> 1) ^ (r >> 3)) & 3; 128-byte rows: (r >> 1) & 7.  Both keep the
// 8- and 16-lane phases of a fragment read (32 consecutive rows, one chunk)
// on distinct banks.
template <int BK>
__device__ __forceinline__ int mx_swz(int r)
{
    return BK == 128 ? (((r >> 1) ^ (r >> 3)) & 3) : ((r >> 1) & 7);
}

__device__ __forceinline__ void store_tile_4x2(const v16f (&acc)[4][2], float g, uint16_t* __restrict__ c,
                                               int64_t ldc, int64_t m_base, int64_t n_base, int64_t M, int64_t N)
{
    const bool vec = ((ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(c) & 7) == 0);
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
        const int64_t m = m_base + 32 * j + (lane & 31);
        if (m >= M) continue;
        uint16_t* crow = c + m * ldc;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int64_t n = n_base + 32 * i + 8 * q + 4 * (lane >> 5);
                const uint32_t b0 = f32_to_bf16_rne(acc[i][j][4 * q + 0] * g);
                const uint32_t b1 = f32_to_bf16_rne(acc[i][j][4 * q + 1] * g);
                const uint32_t b2 = f32_to_bf16_rne(acc[i][j][4 * q + 2] * g);
                const uint32_t b3 = f32_to_bf16_rne(acc[i][j][4 * q + 3] * g);
                if (vec && n + 3 < N) {
                    uint2 v;
                    v.x = b0 | (b1 << 16);
                    v.y = b2 | (b3 << 16);
                    *reinterpret_cast<uint2*>(crow + n) = v;
                } else {
                    if (n + 0 < N) crow[n + 0] = (uint16_t)b0;
                    if (n + 1 < N) crow[n + 1] = (uint16_t)b1;
                    if (n + 2 < N) crow[n + 2] = (uint16_t)b2;
                    if (n + 3 < N) crow[n + 3] = (uint16_t)b3;
                }
            }
        }
    }
}

// Epilogue of the 256 x 256 tiles through LDS (the stage buffers are free by
// then).  Each wave writes its scaled bf16 sub-tile, whose lanes each hold
// one column m and runs of four n, into a row-major image of the C tile
// (rows padded by 16 bytes); then every thread stores 16-byte pieces of C
// rows, so four consecutive lanes cover 64 contiguous bytes and a wave two
// whole 512-byte rows.  The caller has retired every load into LDS.
constexpr int kCTileRow = 2 * kTile + 16;           // bytes per LDS row of the C image
constexpr int kCTileBytes = kTile * kCTileRow;

template <int NJ>
__device__ __forceinline__ void store_tile_lds(const v16f (&acc)[4][NJ], float g, uint8_t* __restrict__ img,
                                               uint16_t* __restrict__ c, int64_t ldc, int wm_off, int wn_off,
                                               int64_t m_base, int64_t n_base, int64_t M, int64_t N)
{
    const int tid = threadIdx.x, lane = tid & 63;
    __syncthreads();                                 // every wave is done reading the stages
#pragma unroll
    for (int j = 0; j < NJ; ++j) {
        const int ml = wm_off + 32 * j + (lane & 31);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
#pragma unroll
            for (int q = 0; q < 4; ++q) {
                const int nl = wn_off + 32 * i + 8 * q + 4 * (lane >> 5);
                uint2 v;
                v.x = f32_to_bf16_rne(acc[i][j][4 * q + 0] * g) | (f32_to_bf16_rne(acc[i][j][4 * q + 1] * g) << 16);
                v.y = f32_to_bf16_rne(acc[i][j][4 * q + 2] * g) | (f32_to_bf16_rne(acc[i][j][4 * q + 3] * g) << 16);
                *reinterpret_cast<uint2*>(img + ml * kCTileRow + 2 * nl) = v;
            }
        }
    }
    __syncthreads();
    const bool vec = ((ldc & 7) == 0) && ((reinterpret_cast<uintptr_t>(c) & 15) == 0);
    for (int piece = tid; piece < kTile * (kTile / 8); piece += (int)blockDim.x) {
        const int ml = piece / (kTile / 8), cb = piece % (kTile / 8);
        const int64_t m = m_base + ml, n = n_base + 8 * cb;
        if (m >= M || n >= N) continue;
        const uint4 v = *reinterpret_cast<const uint4*>(img + ml * kCTileRow + 16 * cb);
        uint16_t* dst = c + m * ldc + n;
        if (vec && n + 7 < N) {
            *reinterpret_cast<uint4*>(dst) = v;
        } else {
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int e = 0; e < 8; ++e)
                if (n + e < N) dst[e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// The scaled matrix instruction taking byte SEL of each operand's scale
// dword (the instruction's own byte select).
template <int SEL>
__device__ __forceinline__ v16f mfma_fp4_sel(const v8i& w, const v8i& a, const v16f& c, uint32_t sw, uint32_t sa)
{
    return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w, a, c, 4, 4, SEL, (int)sw, SEL, (int)sa);
}
// The same with the byte select a run-time step index that unrolling
// makes constant.
__device__ __forceinline__ v16f mfma_fp4_step(int ks, const v8i& w, const v8i& a, const v16f& c, uint32_t sw,
                                              uint32_t sa)
{
    switch (ks) {
    case 0: return mfma_fp4_sel<0>(w, a, c, sw, sa);
    case 1: return mfma_fp4_sel<1>(w, a, c, sw, sa);
    case 2: return mfma_fp4_sel<2>(w, a, c, sw, sa);
    default: return mfma_fp4_sel<3>(w, a, c, sw, sa);
    }
}

template <int BK, int NS>
__global__ __launch_bounds__(kMx4Threads) void k_gemm_mx(GemmLaunch p)
{
    using L = MxStage<BK>;
    static_assert(NS >= 2 && (BK == 128 || BK == 256), "stage shape");
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;            // 2 x 4 waves: 128 (n) x 64 (m) each
    const int64_t M = p.m, N = p.n, K = p.k;
    int tn, tm;
    tile_coords((int)((N + kTile - 1) / kTile), (int)((M + kTile - 1) / kTile), &tn, &tm);
    const int64_t n_base = (int64_t)tn * kTile, m_base = (int64_t)tm * kTile;
    const int64_t rowb = K / 2, rows = K / 32;
    const int KT = (int)(K / BK);
    auto row_w = [&](int r) { return n_base + r < N ? n_base + r : N - 1; };   // rows past the matrix
    auto row_a = [&](int r) { return m_base + r < M ? m_base + r : M - 1; };   // re-read the last one

    // codes: DMA k of this wave fills rows RPI (NI wave + k) + lane / CPR,
    // physical chunk lane % CPR
    const uint8_t* srcw[L::NI];
    const uint8_t* srca[L::NI];
#pragma unroll
    for (int k = 0; k < L::NI; ++k) {
        const int r = L::RPI * (L::NI * wave + k) + lane / L::CPR;
        const int c = (lane % L::CPR) ^ mx_swz<BK>(r);
        srcw[k] = p.qb + row_w(r) * rowb + 16 * c;
        srca[k] = p.qa + row_a(r) * rowb + 16 * c;
    }
    // scales ([256][SRow] bytes per operand).  BK 128: waves 0-3 fill W's
    // rows 64 wave + lane, waves 4-7 A's.  BK 256: DMA j fills operand j
    // (0: W, 1: A), dword 64 wave + lane = (row, half).
    const uint8_t* srcs[L::SDma];
    int sdst[L::SDma];
    // grouped scales: DMA j fills operand j; LDS unit 2 r + u of row r holds
    // the row's 16-byte half u ^ b3(r) (rows with bit 3 set swap halves, so a
    // 16-lane read of one half over 16 consecutive rows meets every bank
    // once).  A half past the row end (the last, partial group) is read from
    // the row's last 16 bytes instead.
    const uint8_t* gsrc[2];
    int ghalf = 0;
    if (L::Grouped) {
        const int r = tid >> 1;
        ghalf = (tid & 1) ^ ((r >> 3) & 1);
        gsrc[0] = p.sb + row_w(r) * rows;
        gsrc[1] = p.sa + row_a(r) * rows;
    }
    if (BK == 128) {
        const int r = 64 * (wave & 3) + lane;
        srcs[0] = wave < 4 ? p.sb + row_w(r) * rows : p.sa + row_a(r) * rows;
        sdst[0] = 2 * L::Codes + (wave < 4 ? 0 : L::Scales) + 256 * (wave & 3);
    } else if (!L::Grouped) {
        const int q = 64 * wave + lane, r = q >> 1, d = q & 1;
        srcs[0] = p.sb + row_w(r) * rows + 4 * d;
        srcs[L::SDma - 1] = p.sa + row_a(r) * rows + 4 * d;
        sdst[0] = 2 * L::Codes + 256 * wave;
        sdst[L::SDma - 1] = 2 * L::Codes + L::Scales + 256 * wave;
    }
    uint8_t* const gbuf = smem + NS * L::Bytes;

    // stage kt into buffer buf; past the last stage the last one is loaded
    // again (into a buffer that is no longer read), so every wave always has
    // the same number of loads in flight
    auto issue = [&](int kt, int buf) {
        const int ks = kt < KT ? kt : KT - 1;
        uint8_t* st = smem + buf * L::Bytes;
#pragma unroll
        for (int k = 0; k < L::NI; ++k) {
            dma16(srcw[k] + (int64_t)ks * L::RB, st + 1024 * (L::NI * wave + k));
            dma16(srca[k] + (int64_t)ks * L::RB, st + L::Codes + 1024 * (L::NI * wave + k));
        }
        if (!L::Grouped) {
#pragma unroll
            for (int j = 0; j < L::SDma; ++j) dma4(srcs[j] + (int64_t)ks * L::SRow, st + sdst[j]);
        } else if (kt % L::GroupStages == 0 && kt < KT) {
            // group kt / 4 (stages kt .. kt + 3) with the codes of its first stage
            const int64_t off = (int64_t)(kt / L::GroupStages) * L::GroupRow + 16 * ghalf;
            const int64_t o = off + 16 <= rows ? off : rows - 16;
            uint8_t* const gb = gbuf + ((kt / L::GroupStages) & 1) * L::GroupBytes;
#pragma unroll
            for (int j = 0; j < 2; ++j) dma16(gsrc[j] + o, gb + j * (L::GroupBytes / 2) + 1024 * wave);
        }
    };
    static_assert(!L::Grouped || NS == 2, "grouped scales rely on waiting for every load each stage");
    // 256-element stages: the loads of the next stage are spread over the
    // first two 64-element steps of this one, between its matrix
    // instructions.  A load waits for the texture address unit, which the
    // eight waves' loads keep busy for thousands of cycles per stage; issued
    // all at once after the barrier, they held back the matrix instructions
    // behind them in every wave's program.  (Later steps leave too little
    // time for the loads to land before the next stage.)
    constexpr int kParts = L::Grouped ? 2 : 0;
    auto issue_part = [&](int kt, int buf, int part) {
        const int ks = kt < KT ? kt : KT - 1;
        uint8_t* st = smem + buf * L::Bytes;
        constexpr int kP = kParts > 0 ? kParts : 1;
#pragma unroll
        for (int k = part * L::NI / kP; k < (part + 1) * L::NI / kP; ++k) {
            dma16(srcw[k] + (int64_t)ks * L::RB, st + 1024 * (L::NI * wave + k));
            dma16(srca[k] + (int64_t)ks * L::RB, st + L::Codes + 1024 * (L::NI * wave + k));
        }
        if (part == 0 && kt % L::GroupStages == 0 && kt < KT) {
            const int64_t off = (int64_t)(kt / L::GroupStages) * L::GroupRow + 16 * ghalf;
            const int64_t o = off + 16 <= rows ? off : rows - 16;
            uint8_t* const gb = gbuf + ((kt / L::GroupStages) & 1) * L::GroupBytes;
#pragma unroll
            for (int j = 0; j < 2; ++j) dma16(gsrc[j] + o, gb + j * (L::GroupBytes / 2) + 1024 * wave);
        }
    };
    constexpr int kLoads = 2 * L::NI + (L::Grouped ? 0 : L::SDma);

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

#pragma unroll
    for (int s = 0; s < NS - 1; ++s) issue(s, s);

    const int frow = lane & 31, khalf = lane >> 5;
    uint4 swp[4], sap[2];                     // grouped scales: the pair of the current two stages
    for (int kt = 0; kt < KT; ++kt) {
        // this wave's loads of stage kt have landed; the barrier makes every
        // wave's visible and retires all reads of stage kt - 1
        asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 2) * kLoads) : "memory");
        __builtin_amdgcn_s_barrier();        // no fence: a fence would wait for every load in flight
        if (kParts == 0) issue(kt + NS - 1, (kt + NS - 1) % NS);
        const uint8_t* st = smem + (kt % NS) * L::Bytes;
        uint64_t swd[4], sad[2];
        if (L::Grouped) {
            // the 16-byte scale pair of stages kt, kt + 1 (kt even) is read once;
            // stage kt takes its low 8 bytes, kt + 1 the high ones, and so does
            // the last stage of an odd count (its half was read from the row end)
            if ((kt & 1) == 0) {
                const uint8_t* gb = gbuf + ((kt / L::GroupStages) & 1) * L::GroupBytes;
                const int h = (kt % L::GroupStages) >> 1;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = wn * 128 + 32 * i + frow;
                    swp[i] = *reinterpret_cast<const uint4*>(gb + L::GroupRow * r + 16 * (h ^ ((r >> 3) & 1)));
                }
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const int r = wm * 64 + 32 * j + frow;
                    sap[j] = *reinterpret_cast<const uint4*>(gb + L::GroupBytes / 2 + L::GroupRow * r +
                                                             16 * (h ^ ((r >> 3) & 1)));
                }
            }
            const bool hi = (kt & 1) || (kt == KT - 1 && (KT & 1));
#pragma unroll
            for (int i = 0; i < 4; ++i)
                swd[i] = hi ? ((uint64_t)swp[i].w << 32 | swp[i].z) : ((uint64_t)swp[i].y << 32 | swp[i].x);
#pragma unroll
            for (int j = 0; j < 2; ++j)
                sad[j] = hi ? ((uint64_t)sap[j].w << 32 | sap[j].z) : ((uint64_t)sap[j].y << 32 | sap[j].x);
        } else {
            const uint8_t* ssw = st + 2 * L::Codes;
            const uint8_t* ssa = ssw + L::Scales;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wn * 128 + 32 * i + frow;
                swd[i] = BK == 256 ? *reinterpret_cast<const uint64_t*>(ssw + 8 * r)
                                   : (uint64_t)*reinterpret_cast<const uint32_t*>(ssw + 4 * r);
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wm * 64 + 32 * j + frow;
                sad[j] = BK == 256 ? *reinterpret_cast<const uint64_t*>(ssa + 8 * r)
                                   : (uint64_t)*reinterpret_cast<const uint32_t*>(ssa + 4 * r);
            }
        }
        // 256-element stages: this stage's 8 scale bytes of a fragment row
        // gathered once, by one byte permute, into k-step order (byte ks =
        // block 2 ks + khalf), so each matrix instruction picks its byte
        // with its own byte select instead of a shift and mask per step
        uint32_t swb[4], sab[2];
        if (BK == 256) {
            const uint32_t psel = khalf ? 0x07050301u : 0x06040200u;
#pragma unroll
            for (int i = 0; i < 4; ++i) swb[i] = __builtin_amdgcn_perm((uint32_t)(swd[i] >> 32), (uint32_t)swd[i], psel);
#pragma unroll
            for (int j = 0; j < 2; ++j) sab[j] = __builtin_amdgcn_perm((uint32_t)(sad[j] >> 32), (uint32_t)sad[j], psel);
        }
        // fragments of chunk pair ks (16-byte chunk c = 2 ks + khalf of each
        // row) are read while the products of pair ks - 1 are issued
        auto read_frags = [&](int ks, v4i (&wf)[4], v4i (&af)[2]) {
            const int c = 2 * ks + khalf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wn * 128 + 32 * i + frow;
                wf[i] = *reinterpret_cast<const v4i*>(st + r * L::RB + 16 * (c ^ mx_swz<BK>(r)));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wm * 64 + 32 * j + frow;
                af[j] = *reinterpret_cast<const v4i*>(st + L::Codes + r * L::RB + 16 * (c ^ mx_swz<BK>(r)));
            }
        };
        v4i wf[2][4], af[2][2];
        read_frags(0, wf[0], af[0]);
#pragma unroll
        for (int ks = 0; ks < BK / 64; ++ks) {
            const int cur = ks & 1;
            if (ks + 1 < BK / 64) read_frags(ks + 1, wf[cur ^ 1], af[cur ^ 1]);
            if (kParts > 0 && ks < kParts) issue_part(kt + NS - 1, (kt + NS - 1) % NS, ks);
            const int sh = 8 * (2 * ks + khalf);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const v8i wv = {wf[cur][i][0], wf[cur][i][1], wf[cur][i][2], wf[cur][i][3], 0, 0, 0, 0};
#pragma unroll
                for (int j = 0; j < 2; ++j) {
                    const v8i av = {af[cur][j][0], af[cur][j][1], af[cur][j][2], af[cur][j][3], 0, 0, 0, 0};
                    if (BK == 256) {
                        acc[i][j] = mfma_fp4_step(ks, wv, av, acc[i][j], swb[i], sab[j]);
                    } else {
                        const int sw = (int)((swd[i] >> sh) & 0xFFu), sa = (int)((sad[j] >> sh) & 0xFFu);
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(wv, av, acc[i][j], 4, 4, 0, sw, 0,
                                                                                  sa);
                    }
                }
            }
            if (ks + 1 < BK / 64) {
#pragma unroll
                for (int q = 0; q < 6; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one matrix instruction
                    __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);     // one LDS read of the next pair
                }
            }
            if (kParts > 0 && ks < kParts) {
#pragma unroll
                for (int q = 0; q < 2 * L::NI / (kParts > 0 ? kParts : 1) + (ks == 0 ? 2 : 0); ++q) {   // codes (+ scales)
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one matrix instruction
                    __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);     // one load of the next stage
                }
            }
            __builtin_amdgcn_sched_barrier(0);
        }
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    static_assert(NS * L::Bytes + (L::Grouped ? 2 * L::GroupBytes : 0) >= kCTileBytes, "the C image fits the LDS");
    const float g = p.ga[0] * p.gb[0];
    store_tile_lds<2>(acc, g, smem, p.c, p.ldc, wm * 64, wn * 128, m_base, n_base, M, N);
}

// Kernels with more than 64 KiB of dynamic LDS must opt in once per device.
template <typename K>
static hipError_t allow_lds(K kernel, size_t bytes)
{
    return hipFuncSetAttribute(reinterpret_cast<const void*>(kernel), hipFuncAttributeMaxDynamicSharedMemorySize,
                               (int)bytes);
}

template <int BK, int NS>
static hipError_t launch_mx(const GemmLaunch& p, hipStream_t s)
{
    constexpr size_t sh = (size_t)NS * MxStage<BK>::Bytes + (MxStage<BK>::Grouped ? 2 * MxStage<BK>::GroupBytes : 0);
    static_assert(sh <= 160 * 1024, "LDS");
    hipError_t e = allow_lds(k_gemm_mx<BK, NS>, sh);
    if (e != hipSuccess) return e;
    const unsigned tiles = (unsigned)(((p.n + kTile - 1) / kTile) * ((p.m + kTile - 1) / kTile));
    hipLaunchKernelGGL((k_gemm_mx<BK, NS>), dim3(tiles), dim3(kMx4Threads), sh, s, p);
    return hipGetLastError();
}

// 256-element stages read whole 128-byte lines of every row (two stages fit
// in LDS); K that is only a multiple of 128 takes four 128-element stages.
hipError_t launch_gemm_mx(const GemmLaunch& p, hipStream_t s)
{
    if (p.k % 256 == 0 && p.k >= 512) return launch_mx<256, 2>(p, s);
    return launch_mx<128, 4>(p, s);
}

// ---------------------------------------------------------------------------
// E2M1 with E8M0 scales per 16 elements (gonzo_ML/3986 "Форматы FP4": groups
// of 16 with power-of-two scales) on the scaled FP4 matrix instruction.  The
// instruction takes one scale per 32-element K-half of each operand (lane l
// supplies row l % 32 and the 32 elements of K-half l / 32 in 4 dwords,
// scaled by its own scale byte), so every 64-element step runs twice: first
// with A's second 16-element block of every K-half zeroed, then its first,
// each time with both operands' scales of the block that remains.  W keeps
// all its elements: they meet zeros in the other block, so the products are
// exactly those of the block whose scales are applied.  Twice the matrix
// instructions of MXFP4, no dequantization.
//
// Same tile, waves, DMA and stage shape as k_gemm_mx: stages of 256
// elements (128 bytes per row), two stages, scale groups of 32 bytes per
// row (two stages each).
//
// (The instruction also takes FP8 E4M3 operands with E8M0 scales: there
// dwords 0-3 of both lane groups form the first 32-element block, scaled by
// the byte of lanes 0-31, and dwords 4-7 the second, scaled by the byte of
// lanes 32-63 -- measured on the device.  A GEMM of MXFP8 operands on it,
// checked against the exact product, missed the 1e-5 sum|a||b| bound on a
// few outputs in 10^4 whose operands spread over many binades, so FP8 stays
// on the exact dequantize path.)
// ---------------------------------------------------------------------------
struct Mx16Shape {
    static constexpr int EPS = 256;                   // elements per stage (128-byte rows)
    static constexpr int RB = 128;
    static constexpr int NI = 4;                      // code DMAs per wave per operand (8 rows each)
    static constexpr int Codes = kTile * RB;          // 32 KiB per operand
    static constexpr int Bytes = 2 * Codes;
    static constexpr int SRow = 16;                   // scale bytes per row per stage
    static constexpr int GS = 2;                      // stages per 32-byte scale group
    static constexpr int GroupBytes = 2 * kTile * 32; // W then A
    static constexpr int NKS = 4;                     // 64-element steps per stage
};


__global__ __launch_bounds__(kMx4Threads) void k_gemm_mx16(GemmLaunch p)
{
    using L = Mx16Shape;
    constexpr int NS = 2;
    extern __shared__ __align__(16) uint8_t smem[];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;            // 2 x 4 waves: 128 (n) x 64 (m) each
    const int64_t M = p.m, N = p.n, K = p.k;
    int tn, tm;
    tile_coords((int)((N + kTile - 1) / kTile), (int)((M + kTile - 1) / kTile), &tn, &tm);
    const int64_t n_base = (int64_t)tn * kTile, m_base = (int64_t)tm * kTile;
    const int64_t rowb = K / 2, rows = K / 16;
    const int KT = (int)(K / L::EPS);
    auto row_w = [&](int r) { return n_base + r < N ? n_base + r : N - 1; };
    auto row_a = [&](int r) { return m_base + r < M ? m_base + r : M - 1; };

    // 32-bit byte offsets of this lane's loads (the launch requires every
    // operand buffer below 4 GiB), so the loads take a uniform 64-bit base
    uint32_t offw[L::NI], offa[L::NI];
#pragma unroll
    for (int k = 0; k < L::NI; ++k) {
        const int r = 8 * (L::NI * wave + k) + lane / 8;
        const int c = (lane % 8) ^ mx_swz<256>(r);
        offw[k] = (uint32_t)(row_w(r) * rowb + 16 * c);
        offa[k] = (uint32_t)(row_a(r) * rowb + 16 * c);
    }
    // scale groups: two lanes per row, each 16 bytes; LDS unit 2 r + u of
    // row r holds the row's 16-byte half u ^ b3(r).  A half past the row end
    // (the last, partial group) is read from the row's last 16 bytes.
    const int grow = tid >> 1;
    const int ghalf = (tid & 1) ^ ((grow >> 3) & 1);
    const uint32_t goff[2] = {(uint32_t)(row_w(grow) * rows), (uint32_t)(row_a(grow) * rows)};
    uint8_t* const gbuf = smem + NS * L::Bytes;

    auto issue = [&](int kt, int buf, int part) {
        const int ks = kt < KT ? kt : KT - 1;
        uint8_t* st = smem + buf * L::Bytes;
        const uint8_t* bw = p.qb + (int64_t)ks * L::RB;
        const uint8_t* ba = p.qa + (int64_t)ks * L::RB;
#pragma unroll
        for (int k = part * L::NI / 2; k < (part + 1) * L::NI / 2; ++k) {
            dma16(bw + offw[k], st + 1024 * (L::NI * wave + k));
            dma16(ba + offa[k], st + L::Codes + 1024 * (L::NI * wave + k));
        }
        if (part == 0 && kt % L::GS == 0 && kt < KT) {
            const int64_t off = (int64_t)(kt / L::GS) * 32 + 16 * ghalf;
            const uint32_t o = (uint32_t)(off + 16 <= rows ? off : rows - 16);
            uint8_t* const gb = gbuf + ((kt / L::GS) & 1) * L::GroupBytes;
            dma16(p.sb + (goff[0] + o), gb + 1024 * wave);
            dma16(p.sa + (goff[1] + o), gb + L::GroupBytes / 2 + 1024 * wave);
        }
    };

    v16f acc[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = v16f{};

    issue(0, 0, 0);
    issue(0, 0, 1);

    const int frow = lane & 31, khalf = lane >> 5;
    // byte 2 (ks & 1) + run of gathered dword ks >> 1 is this lane's block
    // 2 (2 ks + khalf) + run of the stage: one byte permute per dword
    const uint32_t psel = khalf ? 0x07060302u : 0x05040100u;
    for (int kt = 0; kt < KT; ++kt) {
        asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
        __builtin_amdgcn_s_barrier();
        const uint8_t* st = smem + (kt % NS) * L::Bytes;
        // this stage's 16 scale bytes of each fragment row: half h of its
        // group, which starts at min(32 g + 16 h, rows - 16) of the row
        const int g = kt / L::GS, h = kt % L::GS;
        const uint8_t* gb = gbuf + (g & 1) * L::GroupBytes;
        uint32_t swg[4][2], sag[2][2];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wn * 128 + 32 * i + frow;
            const uint4 v = *reinterpret_cast<const uint4*>(gb + 32 * r + 16 * (h ^ ((r >> 3) & 1)));
            swg[i][0] = __builtin_amdgcn_perm(v.y, v.x, psel);
            swg[i][1] = __builtin_amdgcn_perm(v.w, v.z, psel);
        }
#pragma unroll
        for (int j = 0; j < 2; ++j) {
            const int r = wm * 64 + 32 * j + frow;
            const uint4 v = *reinterpret_cast<const uint4*>(gb + L::GroupBytes / 2 + 32 * r + 16 * (h ^ ((r >> 3) & 1)));
            sag[j][0] = __builtin_amdgcn_perm(v.y, v.x, psel);
            sag[j][1] = __builtin_amdgcn_perm(v.w, v.z, psel);
        }
        auto read_frags = [&](int ks, v4i (&wf)[4], v4i (&af)[2]) {
            const int c = 2 * ks + khalf;
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int r = wn * 128 + 32 * i + frow;
                wf[i] = *reinterpret_cast<const v4i*>(st + r * L::RB + 16 * (c ^ mx_swz<256>(r)));
            }
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const int r = wm * 64 + 32 * j + frow;
                af[j] = *reinterpret_cast<const v4i*>(st + L::Codes + r * L::RB + 16 * (c ^ mx_swz<256>(r)));
            }
        };
        v4i wf[2][4], af[2][2];
        read_frags(0, wf[0], af[0]);
        // one 64-element step; the step index is a template constant so the
        // matrix instructions' byte selects are immediates
        auto step = [&](auto ksc) {
            constexpr int ks = decltype(ksc)::value;
            constexpr int cur = ks & 1, dw = ks >> 1;
            if (ks + 1 < L::NKS) read_frags(ks + 1, wf[cur ^ 1], af[cur ^ 1]);
            if (ks < 2) issue(kt + 1, (kt + 1) % NS, ks);
#pragma unroll
            for (int j = 0; j < 2; ++j) {
                const v4i a = af[cur][j];
                const v8i a0 = {a[0], a[1], 0, 0, 0, 0, 0, 0}, a1 = {0, 0, a[2], a[3], 0, 0, 0, 0};
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const v4i w = wf[cur][i];
                    const v8i wv = {w[0], w[1], w[2], w[3], 0, 0, 0, 0};
                    acc[i][j] = mfma_fp4_sel<2 * (ks & 1)>(wv, a0, acc[i][j], swg[i][dw], sag[j][dw]);
                    acc[i][j] = mfma_fp4_sel<2 * (ks & 1) + 1>(wv, a1, acc[i][j], swg[i][dw], sag[j][dw]);
                }
            }
        };
        step(std::integral_constant<int, 0>{});
        step(std::integral_constant<int, 1>{});
        step(std::integral_constant<int, 2>{});
        step(std::integral_constant<int, 3>{});
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    static_assert(NS * L::Bytes + 2 * L::GroupBytes >= kCTileBytes, "the C image fits the LDS");
    const float gg = p.ga[0] * p.gb[0];
    store_tile_lds<2>(acc, gg, smem, p.c, p.ldc, wm * 64, wn * 128, m_base, n_base, M, N);
}

// E2M1 with E8M0 scales at block 16 on both operands, whole 256-element
// stages, at least 16 scale bytes per row and operands below 4 GiB.
bool gemm_mx16_supported(const GemmLaunch& p)
{
    if (p.elem != 0 || p.block != 16 || !p.fa.is_e8m0 || !p.fb.is_e8m0) return false;
    if (p.m * (p.k / 2) >= (int64_t(1) << 32) || p.n * (p.k / 2) >= (int64_t(1) << 32)) return false;
    return p.k % 256 == 0 && p.k / 16 >= 16;
}

hipError_t launch_gemm_mx16(const GemmLaunch& p, hipStream_t s)
{
    using L = Mx16Shape;
    constexpr size_t sh = (size_t)2 * L::Bytes + 2 * L::GroupBytes;
    static_assert(sh <= 160 * 1024, "LDS");
    hipError_t e = allow_lds(k_gemm_mx16, sh);
    if (e != hipSuccess) return e;
    const unsigned tiles = (unsigned)(((p.n + kTile - 1) / kTile) * ((p.m + kTile - 1) / kTile));
    hipLaunchKernelGGL(k_gemm_mx16, dim3(tiles), dim3(kMx4Threads), sh, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// exact dequantize path: FP4 tiles -> f16/bf16 in LDS -> 32x32x16 MFMA
// ---------------------------------------------------------------------------
constexpr int kDqBK = 64;                 // K elements per stage
constexpr int kDqRow = 144;               // LDS row stride in bytes: 64 x 2 B + 16 B pad

struct DqSmem {
    uint8_t w[2][kTile * kDqRow];
    uint8_t a[2][kTile * kDqRow];
};

// Largest power of two not above a positive normal g (1 for anything else):
// g / split_pow2(g) lies in [1, 2) and the division is exact.
__device__ __forceinline__ float split_pow2(float g)
{
    const uint32_t e = __float_as_uint(g) & 0x7F800000u;
    return (e == 0u || e == 0x7F800000u || g < 0.0f) ? 1.0f : __uint_as_float(e);
}

// Dequantize 32 E2M1 codes (16 bytes) with scale(s) into 32 16-bit values.
// The product e2m1 * s is exact in binary32 and, for the chosen element type,
// exact in f16 / bf16, so the narrowing is exact (truncation = rounding).
template <bool F16, bool INT = false>
__device__ __forceinline__ void dequant32(const v4i& codes, float s0, float s1, uint32_t out[16])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = (uint32_t)codes[d];
        const float s = d < 2 ? s0 : s1;    // elements 0..15 use s0, 16..31 use s1
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const uint32_t n0 = (w >> (8 * h)) & 0xFu, n1 = (w >> (8 * h + 4)) & 0xFu;
            const float v0 = (INT ? int4_value(n0) : e2m1_value(n0)) * s;
            const float v1 = (INT ? int4_value(n1) : e2m1_value(n1)) * s;
            uint32_t b0, b1;
            if (F16) {
                b0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0);
                b1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1);
            } else {
                b0 = __float_as_uint(v0) >> 16;
                b1 = __float_as_uint(v1) >> 16;
            }
            out[d * 4 + h] = b0 | (b1 << 16);
        }
    }
}

// As dequant32<false>, for scales whose products need up to 9 significant
// bits (E1M6): v = hi + lo with hi its bf16 truncation and lo the exact
// remainder, both exact bf16 values.
__device__ __forceinline__ void dequant32_split(const v4i& codes, float s0, float s1, uint32_t hi[16],
                                                uint32_t lo[16])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = (uint32_t)codes[d];
        const float s = d < 2 ? s0 : s1;
#pragma unroll
        for (int h = 0; h < 4; ++h) {
            const float v0 = e2m1_value((w >> (8 * h)) & 0xFu) * s;
            const float v1 = e2m1_value((w >> (8 * h + 4)) & 0xFu) * s;
            const uint32_t h0 = __float_as_uint(v0) & 0xFFFF0000u, h1 = __float_as_uint(v1) & 0xFFFF0000u;
            const float l0 = v0 - __uint_as_float(h0), l1 = v1 - __uint_as_float(h1);
            hi[d * 4 + h] = (h0 >> 16) | h1;
            lo[d * 4 + h] = (__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u);
        }
    }
}

typedef float v2f __attribute__((ext_vector_type(2)));

// Dequantize 16 one-byte elements (FP8 E4M3 codes for ELEM 2, INT8 for
// ELEM 3) with one scale into 16 16-bit values; out[j] holds elements 2j and
// 2j + 1.  As in dequant32 the launch only picks a 16-bit type that holds
// every product e * s exactly.
template <bool F16, int ELEM>
__device__ __forceinline__ void dequant16_w8(const v4i& codes, float s, uint32_t out[8])
{
#pragma unroll
    for (int d = 0; d < 4; ++d) {
        const uint32_t w = (uint32_t)codes[d];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            float v0, v1;
            if constexpr (ELEM == 2) {
                // the hardware OCP E4M3 -> f32 conversion of bytes 2h, 2h + 1
                // (exact; the NaN codes, which no quantizer writes, give NaN)
                const v2f e = h == 0 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false)
                                     : __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true);
                v0 = e[0] * s;
                v1 = e[1] * s;
            } else {
                v0 = int8_value((w >> (16 * h)) & 0xFFu) * s;
                v1 = int8_value((w >> (16 * h + 8)) & 0xFFu) * s;
            }
            uint32_t b0, b1;
            if (F16) {
                b0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0);
                b1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1);
            } else {
                b0 = __float_as_uint(v0) >> 16;
                b1 = __float_as_uint(v1) >> 16;
            }
            out[d * 2 + h] = b0 | (b1 << 16);
        }
    }
}

// Dequantize 32 six-bit codes (192 bits, element k at bit 6k of d[0..2])
// with scales s0 (elements 0..15) and s1 (16..31).  An FP6 code is the FP8
// byte of its value times 2^-6 (E2M3 -> E4M3) or 2^-12 (E3M2 -> E5M2): the
// hardware converts that exactly and one multiply by 2^6 / 2^12 restores
// the value.  INT6 codes are sign-extended.
template <bool F16, int ELEM>
__device__ __forceinline__ void dequant32_w6(const uint64_t d[3], float s0, float s1, uint32_t out[16])
{
    const uint32_t dw[6] = {(uint32_t)d[0], (uint32_t)(d[0] >> 32), (uint32_t)d[1],
                            (uint32_t)(d[1] >> 32), (uint32_t)d[2], (uint32_t)(d[2] >> 32)};
#pragma unroll
    for (int q = 0; q < 8; ++q) {                   // four elements 4q .. 4q + 3: bits 24q .. 24q + 23
        const int bit = 24 * q, i = bit >> 5, sh = bit & 31;
        const uint32_t x = sh == 0 ? dw[i] : sh <= 8 ? dw[i] >> sh : __builtin_amdgcn_alignbit(dw[i + 1], dw[i], sh);
        const float s = q < 4 ? s0 : s1;
        float e[4];
        if constexpr (ELEM == 6) {
#pragma unroll
            for (int t = 0; t < 4; ++t) e[t] = (float)(((int32_t)(x << (26 - 6 * t))) >> 26);
        } else {
            // the four codes to one byte each, then to FP8 bytes (sign bit 5 -> 7)
            const uint32_t y = (x & 0x3Fu) | ((x << 2) & 0x3F00u) | ((x << 4) & 0x3F0000u) | ((x << 6) & 0x3F000000u);
            const uint32_t w = (y & 0x1F1F1F1Fu) | ((y & 0x20202020u) << 2);
            const v2f lo2 = ELEM == 4 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false)
                                      : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
            const v2f hi2 = ELEM == 4 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, true)
                                      : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, true);
            constexpr float kFold = ELEM == 4 ? 64.0f : 4096.0f;      // exact: back to the FP6 value
            e[0] = lo2[0] * kFold; e[1] = lo2[1] * kFold; e[2] = hi2[0] * kFold; e[3] = hi2[1] * kFold;
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const float v0 = e[2 * h] * s, v1 = e[2 * h + 1] * s;
            uint32_t b0, b1;
            if (F16) {
                b0 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v0);
                b1 = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v1);
            } else {
                b0 = __float_as_uint(v0) >> 16;
                b1 = __float_as_uint(v1) >> 16;
            }
            out[2 * q + h] = b0 | (b1 << 16);
        }
    }
}

// ELEM: the element grid of both operands (fp4_element order: 0 E2M1, 1
// INT4, 2 FP8 E4M3, 3 INT8, 4 FP6 E2M3, 5 FP6 E3M2, 6 INT6).  The launch picks bf16 or f16 so that every
// dequantized value is exact: INT4 products carry at most 3 + 5 = 8
// significant bits in bf16 (3 + 7 in f16), FP8 ones 4 + 4 in bf16, INT8
// ones 7 + 1 in bf16 (power-of-two scales) or 7 + 4 in f16 (E4M3 scales,
// at most 127 * 448 < 65504).  The 8-bit grids stage 32 bytes per thread
// and row instead of 16, the 6-bit grids 24 (three 8-byte loads; FP6 E2M3
// products carry 4 + 4 bits, E3M2 3 + 5, INT6 5 + 3 in bf16 or 5 + 6 in
// f16); the LDS tiles and the matrix loop are the same.
template <bool F16, int BLOCK, int ELEM = 0>
__global__ __launch_bounds__(kGemmThreads) void k_gemm_dq(GemmLaunch p)
{
    constexpr bool INT = ELEM == 1;
    constexpr bool W8 = ELEM == 2 || ELEM == 3;
    constexpr bool W6 = ELEM >= 4;
    extern __shared__ __align__(16) uint8_t smem_raw[];
    DqSmem& sm = *reinterpret_cast<DqSmem*>(smem_raw);
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t n_base = (int64_t)blockIdx.x * kTile;
    const int64_t m_base = (int64_t)blockIdx.y * kTile;
    const int64_t M = p.m, N = p.n, K = p.k;
    const int64_t rowb = W8 ? K : W6 ? K / 4 * 3 : K / 2, rows = K / BLOCK;
    const int KT = (int)(K / kDqBK);
    const ScaleFmt fw{p.fb.ebits, p.fb.mbits, p.fb.bias, p.fb.maxcode, p.fb.smax, p.fb.is_e8m0};
    const ScaleFmt fa{p.fa.ebits, p.fa.mbits, p.fa.bias, p.fa.maxcode, p.fa.smax, p.fa.is_e8m0};
    // bf16 spans the binary32 range, so the power-of-two part of each tensor
    // scale is folded into the (still exact) dequantized values; this keeps
    // products of wide-range scales (E7M0 up to 2^63) inside binary32.  The
    // f16 formats have small scale ranges and keep g for the epilogue.
    float pw = 1.0f, pa = 1.0f, g = p.ga[0] * p.gb[0];
    if (!F16) {
        const float gw = p.gb[0], ga = p.ga[0];
        pw = split_pow2(gw);
        pa = split_pow2(ga);
        g = (gw / pw) * (ga / pa);
    }

    // staging: thread t owns chunk (t & 1) (32 elements: 16 B of FP4 / INT4
    // codes, 32 B of 8-bit ones) of rows (t >> 1) and (t >> 1) + 128 of
    // each operand, with their scales
    constexpr int kVec = W8 ? 2 : 1;                                  // 16-byte loads per chunk
    const int crow = tid >> 1, cchunk = tid & 1;
    v4i rw[2][kVec], ra[2][kVec];
    uint64_t r6w[2][W6 ? 3 : 1], r6a[2][W6 ? 3 : 1];                   // 6-bit chunks: 24 bytes
    uint32_t scw[2], sca[2];
    auto gload = [&](int kt) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            const int64_t nr = n_base + crow + 128 * r, mr = m_base + crow + 128 * r;
            const int64_t sb = ((int64_t)kt * kDqBK + cchunk * 32) / BLOCK; // first scale of the chunk
            if constexpr (W6) {
                const int64_t kb6 = (int64_t)kt * 48 + cchunk * 24;
#pragma unroll
                for (int v = 0; v < 3; ++v) {
                    r6w[r][v] = nr < N ? *reinterpret_cast<const uint64_t*>(p.qb + nr * rowb + kb6 + 8 * v) : 0ull;
                    r6a[r][v] = mr < M ? *reinterpret_cast<const uint64_t*>(p.qa + mr * rowb + kb6 + 8 * v) : 0ull;
                }
            }
            const int64_t kb = (int64_t)kt * (16 * kVec * 2) + cchunk * (16 * kVec);   // byte offset in the row
            if (nr < N) {
#pragma unroll
                for (int v = 0; v < kVec; ++v)
                    if (!W6) rw[r][v] = *reinterpret_cast<const v4i*>(p.qb + nr * rowb + kb + 16 * v);
                scw[r] = BLOCK == 16 ? (uint32_t)*reinterpret_cast<const uint16_t*>(p.sb + nr * rows + sb)
                                     : (uint32_t)p.sb[nr * rows + sb];
            } else {
#pragma unroll
                for (int v = 0; v < kVec; ++v) rw[r][v] = v4i{0, 0, 0, 0};
                scw[r] = 0;
            }
            if (mr < M) {
#pragma unroll
                for (int v = 0; v < kVec; ++v)
                    if (!W6) ra[r][v] = *reinterpret_cast<const v4i*>(p.qa + mr * rowb + kb + 16 * v);
                sca[r] = BLOCK == 16 ? (uint32_t)*reinterpret_cast<const uint16_t*>(p.sa + mr * rows + sb)
                                     : (uint32_t)p.sa[mr * rows + sb];
            } else {
#pragma unroll
                for (int v = 0; v < kVec; ++v) ra[r][v] = v4i{0, 0, 0, 0};
                sca[r] = 0;
            }
        }
    };
    // 32 elements -> 16 words of 16-bit pairs
    auto dq = [&](const v4i* c, float s0, float s1, uint32_t o[16]) {
        if constexpr (W8) {
            dequant16_w8<F16, ELEM>(c[0], s0, o);
            dequant16_w8<F16, ELEM>(c[kVec - 1], s1, o + 8);
        } else {
            dequant32<F16, INT>(c[0], s0, s1, o);
        }
    };
    auto sstore = [&](int buf) {
#pragma unroll
        for (int r = 0; r < 2; ++r) {
            uint32_t o[16];
            {
                const float s0 = scale_decode_any(scw[r] & 0xFFu, fw) * pw;
                const float s1 = BLOCK == 16 ? scale_decode_any((scw[r] >> 8) & 0xFFu, fw) * pw : s0;
                if constexpr (W6) dequant32_w6<F16, ELEM>(r6w[r], s0, s1, o);
                else dq(rw[r], s0, s1, o);
                uint8_t* dst = &sm.w[buf][(crow + 128 * r) * kDqRow + cchunk * 64];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    *reinterpret_cast<v4i*>(dst + 16 * v) = v4i{(int)o[4 * v], (int)o[4 * v + 1], (int)o[4 * v + 2],
                                                               (int)o[4 * v + 3]};
            }
            {
                const float s0 = scale_decode_any(sca[r] & 0xFFu, fa) * pa;
                const float s1 = BLOCK == 16 ? scale_decode_any((sca[r] >> 8) & 0xFFu, fa) * pa : s0;
                if constexpr (W6) dequant32_w6<F16, ELEM>(r6a[r], s0, s1, o);
                else dq(ra[r], s0, s1, o);
                uint8_t* dst = &sm.a[buf][(crow + 128 * r) * kDqRow + cchunk * 64];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    *reinterpret_cast<v4i*>(dst + 16 * v) = v4i{(int)o[4 * v], (int)o[4 * v + 1], (int)o[4 * v + 2],
                                                               (int)o[4 * v + 3]};
            }
        }
    };

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = v16f{};

    gload(0);
    sstore(0);
    __syncthreads();
    const int frow = lane & 31, khalf = lane >> 5;
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) gload(kt + 1);
#pragma unroll
        for (int ks = 0; ks < kDqBK / 16; ++ks) {
            v4i wf[4], af[4];
            const int off = ks * 32 + khalf * 16;        // 16 K = 32 bytes per step; lane half = 8 K
#pragma unroll
            for (int i = 0; i < 4; ++i)
                wf[i] = *reinterpret_cast<const v4i*>(&sm.w[buf][(wn * 128 + 32 * i + frow) * kDqRow + off]);
#pragma unroll
            for (int j = 0; j < 4; ++j)
                af[j] = *reinterpret_cast<const v4i*>(&sm.a[buf][(wm * 128 + 32 * j + frow) * kDqRow + off]);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    if (F16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(v8h, wf[i]),
                                                                          __builtin_bit_cast(v8h, af[j]), acc[i][j],
                                                                          0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(v8bf, wf[i]),
                                                                           __builtin_bit_cast(v8bf, af[j]), acc[i][j],
                                                                           0, 0, 0);
                }
        }
        if (kt + 1 < KT) sstore(buf ^ 1);
        __syncthreads();
    }
    store_tile(acc, g, p.c, p.ldc, m_base + wm * 128, n_base + wn * 128, M, N);
}

// ---------------------------------------------------------------------------
// In-register conversion path (scale formats whose e2m1 * s products are
// exact in f16: E4M3, E3M4, E2M5, E1M6 -- NVFP4 is E4M3 at block 16; and in
// bf16 the ExMy formats with 5+ exponent bits, UE5M3 among them).  The
// stages hold FP4 codes and raw scale bytes, loaded straight into LDS as in
// k_gemm_mx; each wave converts its own fragments right before the matrix
// instruction: for f16 the hardware FP4 -> f16 conversion (scale 1, exact)
// and one packed f16 multiply by the block scale per two elements.  The f16
// forms run eight waves (2 x 4, 128 x 64 each) so one wave's conversions
// overlap the other's matrix instructions on the same SIMD; the bf16 form
// four (2 x 2, 128 x 128 each), see launch_nv.
//
// K order inside a 128-element stage: lane half h of a 32x32x16 step (ks,
// t) supplies elements 32 (2 ks + h) + 8 t + 0..7 of its row -- one 16-byte
// fragment per lane and chunk.  The order is the same for both operands, so
// every product pairs equal k.
// ---------------------------------------------------------------------------
typedef _Float16 v2h __attribute__((ext_vector_type(2)));

// A 128-element stage: RB code bytes per row (64 for E2M1, 128 for FP8).
template <int BLOCK, int RB = kMx3RB>
struct NvStage {
    static constexpr int kRB = RB;
    static constexpr int kCodes = kTile * RB;                  // per operand
    static constexpr int kScaleRow = kMx3BK / BLOCK;           // scale bytes per row per stage
    static constexpr int kScales = kTile * kScaleRow;          // per operand
    static constexpr int kBytes = 2 * kCodes + 2 * kScales;
    static constexpr int kTable = 2 * 256 * 4;                 // decode tables of W and A (f16x2 or f32)
};

// How k_gemm_nv turns codes into matrix operands.
//  kNvTable: f16, block scales decoded through an LDS table;
//  kNvE4M3: f16, both scale formats E4M3, decoded by the hardware FP8 -> f16
//    conversion (exact) instead of the table;
//  kNvBf16: bf16 for the scale formats whose products leave f16's range
//    (UE5M3: e2m1 * s up to 6 * 2^15 * 1.875): each code pair is converted
//    to fp32 (scale 1), multiplied by the fp32 block scale from the table
//    (exact: at most 6 significant bits) and rounded to a bf16 pair, which
//    is exact.  gfx950 has no packed bf16 multiply, so this costs two VALU
//    per element where the f16 forms cost one.
//  kNvFp8: FP8 E4M3 elements with E8M0 scales on both operands (MXFP8):
//    one scaled FP8 -> bf16 conversion per element pair applies the
//    power-of-two scale exactly (4 significant bits fit bf16), bf16 matrix
//    instruction.  Rows are 128 code bytes per stage.
//  kNvInt8: INT8 elements with E4M3 scales on both operands (NVINT8-style),
//    f16: each byte in offset binary under the f16 exponent byte 0x64 is
//    1024 + (e + 128) exactly, one packed subtraction of 1152 leaves e, one
//    packed multiply by the E4M3 scale (at most 7 + 4 significant bits and
//    127 * 448 < 65504: exact).  Rows as kNvFp8.
enum { kNvTable = 0, kNvE4M3 = 1, kNvBf16 = 2, kNvFp8 = 3, kNvInt8 = 4 };

// 8 E2M1 codes (one dword, element 2b in the low nibble of byte b) times
// the f16 block scale s2 (replicated in both halves).
__device__ __forceinline__ v8h nv_convert8(uint32_t w, v2h s2)
{
    const v2h h0 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2;
    const v2h h1 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2;
    const v2h h2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2;
    const v2h h3 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2;
    return v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// 8 E2M1 codes times the fp32 block scale s, as bf16 (kNvBf16).
__device__ __forceinline__ v8bf nv_convert8_bf16(uint32_t w, float s)
{
    v8bf r;
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const v2f e = b == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
                    : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
                    : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                             : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
        r[2 * b] = (__bf16)(e[0] * s);
        r[2 * b + 1] = (__bf16)(e[1] * s);
    }
    return r;
}

// 8 FP8 E4M3 codes (two dwords, element 4 d + b in byte b of dword d)
// times the power-of-two scale s, as bf16 (kNvFp8; exact).
__device__ __forceinline__ v8bf nv_convert8_fp8(uint32_t d0, uint32_t d1, float s)
{
    const v2bf p0 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, s, false);
    const v2bf p1 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d0, s, true);
    const v2bf p2 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, s, false);
    const v2bf p3 = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8((int)d1, s, true);
    return v8bf{p0[0], p0[1], p1[0], p1[1], p2[0], p2[1], p3[0], p3[1]};
}

// 8 INT8 codes (two dwords, element 4 d + b in byte b of dword d) times the
// f16 scale s2 (replicated), as f16 (kNvInt8; exact).
__device__ __forceinline__ v8h nv_convert8_int8(uint32_t d0, uint32_t d1, v2h s2)
{
    const uint32_t x0 = d0 ^ 0x80808080u, x1 = d1 ^ 0x80808080u;      // offset binary
    const v2h k = {(_Float16)1152.0f, (_Float16)1152.0f};
    // bytes {x.b, 0x64} as f16: 1024 + x.b
    const v2h h0 = (__builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x0, 0x04010400u)) - k) * s2;
    const v2h h1 = (__builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x0, 0x04030402u)) - k) * s2;
    const v2h h2 = (__builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x1, 0x04010400u)) - k) * s2;
    const v2h h3 = (__builtin_bit_cast(v2h, __builtin_amdgcn_perm(0x64646464u, x1, 0x04030402u)) - k) * s2;
    return v8h{h0[0], h0[1], h1[0], h1[1], h2[0], h2[1], h3[0], h3[1]};
}

// Fragments of one half stage (chunk pair ks) for one lane: four W and JA
// A code fragments of P 16-byte pieces (32 E2M1 or FP8 elements) and their
// raw scale bytes (block 16: the two scales of the chunk in one u16; block
// 32: one byte).
template <int JA, int P = 1>
struct NvHalf {
    v4i w[4][P], a[JA][P];
    uint32_t sw[4], sa[JA];
};

// CVT: one of kNvTable, kNvE4M3, kNvBf16 (above).
//
// Schedule of one 128-element stage (per wave): the fragments of half 1 are
// read from LDS while half 0's products run; the workgroup barrier sits
// between the halves, and after it the first half of the next stage is
// read while half 1's products run.  The conversions of each 32x32x16 step
// are interleaved with the previous step's products.
template <int BLOCK, int NS, int CVT, int WM>
__global__ __launch_bounds__(128 * WM) void k_gemm_nv(GemmLaunch p)
{
    constexpr bool FP8 = CVT == kNvFp8, INT8 = CVT == kNvInt8;
    constexpr bool W8 = FP8 || INT8;            // one byte per element
    using L = NvStage<BLOCK, W8 ? 128 : kMx3RB>;
    constexpr int RB = L::kRB;                  // code bytes per row per stage
    constexpr int P = RB / 64;                  // 16-byte pieces per lane fragment
    constexpr int CPR = RB / 16;                // 16-byte chunks per row
    constexpr int NWV = 2 * WM;                 // waves: 2 along n (128 rows of W each) x WM along m
    constexpr int JA = 8 / WM;                  // 32-row A fragments per wave (its 32 JA rows of A)
    constexpr int CK = kTile * CPR / 64 / NWV;  // 16-byte code DMAs per lane per operand and stage
    constexpr bool HW_E4M3 = CVT == kNvE4M3 || INT8, BF16 = CVT == kNvBf16 || FP8;
    using V8 = std::conditional_t<BF16, v8bf, v8h>;
    static_assert(NS >= 2, "at least two stages");
    extern __shared__ __align__(16) uint8_t smem[];
    uint32_t* tab = reinterpret_cast<uint32_t*>(smem + NS * L::kBytes);   // [2][256] f16x2
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int wn = wave & 1, wm = wave >> 1;
    const int64_t M = p.m, N = p.n, K = p.k;
    int tn, tm;
    tile_coords((int)((N + kTile - 1) / kTile), (int)((M + kTile - 1) / kTile), &tn, &tm);
    const int64_t n_base = (int64_t)tn * kTile, m_base = (int64_t)tm * kTile;
    const int64_t rowb = W8 ? K : K / 2, rows = K / BLOCK;
    const int KT = (int)(K / kMx3BK);
    // 16-byte chunk c of row r sits at c ^ swz(r) (64- or 128-byte rows)
    auto swz = [&](int r) { return W8 ? mx_swz<256>(r) : mx_swz<128>(r); };

    // scale code -> f16 (exact for these formats), replicated for packed
    // math; or -> fp32 for the bf16 form, which (as the dequantize path)
    // folds the power-of-two part of each tensor scale into the operand's
    // scales so that products of wide-range scales (E7M0: up to 2^63) stay
    // inside binary32
    const float pw = BF16 ? split_pow2(p.gb[0]) : 1.0f, pa = BF16 ? split_pow2(p.ga[0]) : 1.0f;
    if (!HW_E4M3) {
        for (int e = tid; e < 512; e += 64 * NWV) {
            const int t = e & 255;
            const ScaleFmtHost& fh = e < 256 ? p.fb : p.fa;
            const ScaleFmt f{fh.ebits, fh.mbits, fh.bias, fh.maxcode, fh.smax, fh.is_e8m0};
            const float sv = BF16 ? scale_decode_any((uint32_t)t, f) * (e < 256 ? pw : pa)
                                  : scale_decode_any((uint32_t)t, f);
            const uint32_t h = (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)sv);
            tab[e] = BF16 ? __float_as_uint(sv) : h | (h << 16);
        }
        __syncthreads();
    }

    const uint8_t* srcw[CK];
    const uint8_t* srca[CK];
#pragma unroll
    for (int k = 0; k < CK; ++k) {
        const int r = (64 / CPR) * (CK * wave + k) + lane / CPR;
        const int c = (lane % CPR) ^ swz(r);
        const int64_t nr = n_base + r < N ? n_base + r : N - 1;
        const int64_t mr = m_base + r < M ? m_base + r : M - 1;
        srcw[k] = p.qb + nr * rowb + 16 * c;
        srca[k] = p.qa + mr * rowb + 16 * c;
    }
    // scales: the stage's dwords of both operands, W's then A's (block 16:
    // two per row, block 32: one), dword q of them by lane q % (64 NWV) in
    // DMA q / (64 NWV)
    constexpr int kSDw = BLOCK == 16 ? 512 : 256;                      // dwords per operand
    constexpr int kSDma = 2 * kSDw / (64 * NWV);
    const uint8_t* srcs[kSDma];
    int sdst[kSDma];
#pragma unroll
    for (int j = 0; j < kSDma; ++j) {
        const int q = 64 * wave + lane + 64 * NWV * j;
        const bool is_a = q >= kSDw;
        const int qq = q - (is_a ? kSDw : 0);
        const int r = BLOCK == 16 ? qq >> 1 : qq, d = BLOCK == 16 ? qq & 1 : 0;
        srcs[j] = is_a ? p.sa + (m_base + r < M ? m_base + r : M - 1) * rows + 4 * d
                       : p.sb + (n_base + r < N ? n_base + r : N - 1) * rows + 4 * d;
        sdst[j] = 2 * L::kCodes + (is_a ? L::kScales : 0) + 4 * (qq - lane);
    }

    // DMA of stage kt into buffer kt % NS; past the last stage the last one
    // is loaded again (into a buffer that is no longer read) so every wave
    // always has the same number of loads in flight
    auto issue = [&](int kt) {
        const int ks = kt < KT ? kt : KT - 1;
        uint8_t* st = smem + (kt % NS) * L::kBytes;
#pragma unroll
        for (int k = 0; k < CK; ++k) {
            dma16(srcw[k] + (int64_t)ks * RB, st + 1024 * (CK * wave + k));
            dma16(srca[k] + (int64_t)ks * RB, st + L::kCodes + 1024 * (CK * wave + k));
        }
#pragma unroll
        for (int j = 0; j < kSDma; ++j) dma4(srcs[j] + (int64_t)ks * L::kScaleRow, st + sdst[j]);
    };
    constexpr int kLoads = 2 * CK + kSDma;

    const int frow = lane & 31, khalf = lane >> 5;
    // chunk c = 2 ks + khalf of the row's 32 P-byte chunks: pieces P c ..
    auto load_half = [&](NvHalf<JA, P>& h, int kt, int ks) {
        const uint8_t* st = smem + (kt % NS) * L::kBytes;
        const uint8_t* ssw = st + 2 * L::kCodes;
        const uint8_t* ssa = ssw + L::kScales;
        const int c = 2 * ks + khalf;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = wn * 128 + 32 * i + frow;
#pragma unroll
            for (int q = 0; q < P; ++q)
                h.w[i][q] = *reinterpret_cast<const v4i*>(st + r * RB + 16 * ((P * c + q) ^ swz(r)));
            h.sw[i] = BLOCK == 16 ? (uint32_t)*reinterpret_cast<const uint16_t*>(ssw + r * L::kScaleRow + 2 * c)
                                  : (uint32_t)ssw[r * L::kScaleRow + c];
        }
#pragma unroll
        for (int j = 0; j < JA; ++j) {
            const int r = wm * 32 * JA + 32 * j + frow;
#pragma unroll
            for (int q = 0; q < P; ++q)
                h.a[j][q] = *reinterpret_cast<const v4i*>(st + L::kCodes + r * RB + 16 * ((P * c + q) ^ swz(r)));
            h.sa[j] = BLOCK == 16 ? (uint32_t)*reinterpret_cast<const uint16_t*>(ssa + r * L::kScaleRow + 2 * c)
                                  : (uint32_t)ssa[r * L::kScaleRow + c];
        }
    };
    // f16 scale of dword t (elements 8 t .. 8 t + 7) of a chunk, broadcast
    auto scale_of = [&](uint32_t code, int t, const uint32_t* tb) -> v2h {
        if (HW_E4M3) {
            const v2h s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(code, 1.0f, false);
            return (BLOCK == 16 && t >= 2) ? v2h{s2[1], s2[1]} : v2h{s2[0], s2[0]};
        }
        const uint32_t b = BLOCK == 16 ? (t >= 2 ? code >> 8 : code & 0xFFu) : code;
        return __builtin_bit_cast(v2h, tb[b]);
    };
    // fp32 scale of dword t of a chunk (kNvBf16)
    auto scale_f32 = [&](uint32_t code, int t, const uint32_t* tb) -> float {
        const uint32_t b = BLOCK == 16 ? (t >= 2 ? code >> 8 : code & 0xFFu) : code;
        return __uint_as_float(tb[b]);
    };
    auto convert = [&](const NvHalf<JA, P>& h, int t, V8 (&cw)[4], V8 (&ca)[JA]) {
        if constexpr (INT8) {
            // elements 8 t .. 8 t + 7: dwords 2 t, 2 t + 1 of the 32 bytes
            const int q = (2 * t) >> 2, d = (2 * t) & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cw[i] = nv_convert8_int8((uint32_t)h.w[i][q % P][d], (uint32_t)h.w[i][q % P][d + 1], scale_of(h.sw[i], t, tab));
#pragma unroll
            for (int j = 0; j < JA; ++j)
                ca[j] = nv_convert8_int8((uint32_t)h.a[j][q % P][d], (uint32_t)h.a[j][q % P][d + 1],
                                         scale_of(h.sa[j], t, tab + 256));
        } else if constexpr (FP8) {
            // elements 8 t .. 8 t + 7: dwords 2 t, 2 t + 1 of the 32 bytes
            const int q = (2 * t) >> 2, d = (2 * t) & 3;
#pragma unroll
            for (int i = 0; i < 4; ++i)
                cw[i] = nv_convert8_fp8((uint32_t)h.w[i][q % P][d], (uint32_t)h.w[i][q % P][d + 1], scale_f32(h.sw[i], t, tab));
#pragma unroll
            for (int j = 0; j < JA; ++j)
                ca[j] = nv_convert8_fp8((uint32_t)h.a[j][q % P][d], (uint32_t)h.a[j][q % P][d + 1],
                                        scale_f32(h.sa[j], t, tab + 256));
        } else if constexpr (BF16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) cw[i] = nv_convert8_bf16((uint32_t)h.w[i][0][t], scale_f32(h.sw[i], t, tab));
#pragma unroll
            for (int j = 0; j < JA; ++j)
                ca[j] = nv_convert8_bf16((uint32_t)h.a[j][0][t], scale_f32(h.sa[j], t, tab + 256));
        } else {
#pragma unroll
            for (int i = 0; i < 4; ++i) cw[i] = nv_convert8((uint32_t)h.w[i][0][t], scale_of(h.sw[i], t, tab));
#pragma unroll
            for (int j = 0; j < JA; ++j) ca[j] = nv_convert8((uint32_t)h.a[j][0][t], scale_of(h.sa[j], t, tab + 256));
        }
    };

    v16f acc[4][JA];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < JA; ++j) acc[i][j] = v16f{};

    // four steps of one half: products of step t with the conversions of
    // step t + 1 (the last step converts step 0 of `next`, if any)
    auto run_half = [&](const NvHalf<JA, P>& h, const NvHalf<JA, P>& next, bool has_next, V8 (&cw)[4], V8 (&ca)[JA]) {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
            V8 nw[4], na[JA];
            const bool conv = t < 3 || has_next;
            if (t < 3) convert(h, t + 1, nw, na);
            else if (has_next) convert(next, 0, nw, na);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < JA; ++j)
                    if constexpr (BF16)
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(cw[i], ca[j], acc[i][j], 0, 0, 0);
                    else
                        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_f16(cw[i], ca[j], acc[i][j], 0, 0, 0);
            if (conv) {
                // one matrix instruction, then its share of the next step's
                // conversions ((4 + JA) fragments, 8 or 16 VALU each)
                constexpr int kVpm = (4 + JA) * (FP8 ? 4 : INT8 ? 14 : BF16 ? 16 : 8) / (4 * JA);
#pragma unroll
                for (int q = 0; q < 4 * JA; ++q) {
                    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                    __builtin_amdgcn_sched_group_barrier(0x002, kVpm, 0);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (conv) {
#pragma unroll
                for (int i = 0; i < 4; ++i) cw[i] = nw[i];
#pragma unroll
                for (int j = 0; j < JA; ++j) ca[j] = na[j];
            }
        }
    };

#pragma unroll
    for (int s = 0; s < NS; ++s) issue(s);
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"((NS - 1) * kLoads) : "memory");
    __builtin_amdgcn_s_barrier();
    NvHalf<JA, P> f, g;
    load_half(f, 0, 0);
    V8 cw[4], ca[JA];
    convert(f, 0, cw, ca);
    // The loop body is uniform: after the last stage the prefetch reads a
    // buffer whose contents are never used (a re-loaded copy of the last
    // stage), which keeps one copy of the body and every barrier uniform.
    for (int kt = 0; kt < KT; ++kt) {
        load_half(g, kt, 1);
        __builtin_amdgcn_sched_barrier(0);
        run_half(f, g, true, cw, ca);
        // stage kt + 1 has landed for every wave, and every wave has
        // finished reading stage kt, whose buffer is refilled next
        asm volatile("s_waitcnt vmcnt(%0) lgkmcnt(0)" ::"n"((NS - 2) * kLoads) : "memory");
        __builtin_amdgcn_s_barrier();
        issue(kt + NS);
        load_half(f, kt + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
        run_half(g, f, true, cw, ca);
    }
    asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
    static_assert(NS * L::kBytes >= kCTileBytes, "the C image fits the stage buffers");
    const float gg = BF16 ? (p.ga[0] / pa) * (p.gb[0] / pw) : p.ga[0] * p.gb[0];
    store_tile_lds<JA>(acc, gg, smem, p.c, p.ldc, wm * 32 * JA, wn * 128, m_base, n_base, M, N);
}

#ifndef FP4_NV_NS
#define FP4_NV_NS 4
#endif

// Formats whose e2m1 * s products are exact in f16 (normal range) and those
// exact in bf16 (at most 8 significant bits).
static bool exact_in_f16(const ScaleFmtHost& f) { return !f.is_e8m0 && f.ebits <= 4 && (f.ebits + f.mbits == 7); }
static bool exact_in_bf16(const ScaleFmtHost& f) { return f.is_e8m0 || f.mbits <= 5; }

static bool is_e4m3(const ScaleFmtHost& f) { return !f.is_e8m0 && f.ebits == 4 && f.mbits == 3; }

// Waves along m: the f16 forms run eight waves (2 x 4, 128 x 64 each), two
// per SIMD, one converting while the other multiplies; the bf16 form, with
// twice the conversion work per product, four waves of 128 x 128 (its
// accumulators in the AGPRs, one wave per SIMD), which convert each A
// fragment for twice the products (measured: UE5M3 600 -> 743 TFLOP/s at
// the Llama-2 7B up projection; the f16 forms gain nothing from it).
// bf16 and 8-bit forms: four waves (one per SIMD); 8-bit rows (128 bytes
// per stage) leave room for two stages.
template <int BLOCK, int CVT>
static hipError_t launch_nv(const GemmLaunch& p, hipStream_t s)
{
    constexpr bool W8 = CVT == kNvFp8 || CVT == kNvInt8;
    constexpr int WM = CVT == kNvBf16 || W8 ? 2 : 4;
    constexpr int NS = W8 ? 2 : FP4_NV_NS;
    using L = NvStage<BLOCK, W8 ? 128 : kMx3RB>;
    constexpr size_t sh = (size_t)NS * L::kBytes + L::kTable;
    static_assert(sh <= 160 * 1024, "LDS");
    hipError_t e = allow_lds(k_gemm_nv<BLOCK, NS, CVT, WM>, sh);
    if (e != hipSuccess) return e;
    const unsigned tiles = (unsigned)(((p.n + kTile - 1) / kTile) * ((p.m + kTile - 1) / kTile));
    hipLaunchKernelGGL((k_gemm_nv<BLOCK, NS, CVT, WM>), dim3(tiles), dim3(128 * WM), sh, s, p);
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Small products (few 256 x 256 tiles, so the tiled kernels would leave most
// CUs idle or multiply mostly padding): one wave per 32 x 32 output tile,
// four waves per workgroup along n, or (KSPLIT, for fewer tiles than
// SIMDs) the four waves of a workgroup splitting K of one tile (chunk c to
// wave c mod 4) with the partial tiles summed once in LDS at the end in a
// fixed order; operands straight from global memory into registers.  Lane
// l takes row l % 32 of each
// operand and, of every 64-element chunk, the 16 bytes (32 E2M1 codes) of
// K-half l / 32: exactly one lane fragment of the scaled FP4 instruction
// (E8M0 scales, with the lane's own scale byte), or four 8-element
// fragments of the f16 / bf16 instruction after the in-register conversion
// of the ExMy forms (the K order inside a chunk permuted identically for
// both operands, which leaves every dot product unchanged).  Eight chunks
// are in flight per lane.
// MODE: 0 E2M1 with E4M3 scales (hardware scale decode), 1 other f16-exact
// scale formats (decoded in registers), 2 MXFP4, 3 the bf16-exact ExMy
// formats (UE5M3, E5M2, E6M1, E7M0, and pairs of them with the f16 ones):
// codes to fp32, times the fp32 scale with the power-of-two part of the
// tensor scale folded in (as the tiled bf16 form), to bf16, bf16 matrix
// instruction; 4 E8M0 at block 16: the scaled FP4 instruction twice per
// chunk, A's other 16-element block of each K-half zeroed, with the scale
// bytes of the block that remains (as k_gemm_mx16); 5 FP8 E4M3 elements
// with E8M0 scales (MXFP8: bytes to bf16 with the scale applied, bf16
// instruction) and 6 INT8 elements with E4M3 scales (to f16, f16
// instruction), as k_gemm_nv's 8-bit forms, 32 bytes per lane per chunk
// and four chunks in flight.
// ---------------------------------------------------------------------------
constexpr int kSmallWaves = 4;
constexpr int kSmallAhead = 8;
int64_t g_gemm_small_outputs = (int64_t)1 << 21;

template <int MODE, int BLOCK, bool KSPLIT>
__global__ __launch_bounds__(64 * kSmallWaves) void k_gemm_small(GemmLaunch p)
{
    static_assert(MODE != 2 || BLOCK == 32, "MXFP4 scales cover 32 elements");
    static_assert(MODE != 4 || BLOCK == 16, "two runs per K-half for blocks of 16");
    constexpr bool W8 = MODE >= 5;                 // one byte per element: 32 bytes per lane per chunk
    constexpr int AH = W8 ? kSmallAhead / 2 : kSmallAhead;
    constexpr int NQ = W8 ? 2 : 1;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t n0 = ((int64_t)blockIdx.x * (KSPLIT ? 1 : kSmallWaves) + (KSPLIT ? 0 : wave)) * 32;
    const int64_t m0 = (int64_t)blockIdx.y * 32;
    if (!KSPLIT && n0 >= p.n) return;         // whole waves; this form has no barrier
    const int r = lane & 31, h = lane >> 5;
    const int64_t nr = n0 + r < p.n ? n0 + r : p.n - 1;
    const int64_t mr = m0 + r < p.m ? m0 + r : p.m - 1;
    const int64_t rowb = W8 ? p.k : p.k / 2, srow = p.k / BLOCK;
    const int nc = (int)(p.k / 64);
    // this wave's chunks: KSPLIT wave, wave + W, wave + 2 W, ... (W waves),
    // else all of them
    constexpr int STEP = KSPLIT ? kSmallWaves : 1;
    const int first = KSPLIT ? wave : 0;
    const int mine = nc > first ? (nc - first + STEP - 1) / STEP : 0;
    // chunk c of this lane: codes at 32 c + 16 h of the row (one byte per
    // element: 64 c + 32 h, two 16-byte pieces); scales (block 16) the dword
    // at 4 c holding both K-halves' two bytes, (block 32) the u16 at 2 c
    // holding both K-halves' byte
    constexpr int CB = W8 ? 64 : 32;               // code bytes of a row per chunk
    const uint8_t* qw = p.qb + nr * rowb + (CB / 2) * h;
    const uint8_t* qa = p.qa + mr * rowb + (CB / 2) * h;
    const uint8_t* sw = p.sb + nr * srow;
    const uint8_t* sa = p.sa + mr * srow;
    auto scales_at = [&](const uint8_t* row, int c) -> uint32_t {
        if (BLOCK == 16) return *reinterpret_cast<const uint32_t*>(row + 4 * c) >> (16 * h);   // 2 bytes
        return (uint32_t)*reinterpret_cast<const uint16_t*>(row + 2 * c) >> (8 * h);         // 1 byte
    };
    ScaleFmt fw{}, fa{};
    constexpr bool FOLD = MODE == 3 || MODE == 5;   // fp32 scales with the tensor scale's power of two
    const float pw = FOLD ? split_pow2(p.gb[0]) : 1.0f, pa = FOLD ? split_pow2(p.ga[0]) : 1.0f;
    if (MODE == 1 || FOLD) {
        fw = ScaleFmt{p.fb.ebits, p.fb.mbits, p.fb.bias, p.fb.maxcode, p.fb.smax, p.fb.is_e8m0};
        fa = ScaleFmt{p.fa.ebits, p.fa.mbits, p.fa.bias, p.fa.maxcode, p.fa.smax, p.fa.is_e8m0};
    }
    // f16 scale of dword t (elements 8 t .. 8 t + 7 of the lane's 32)
    auto scale_h = [&](uint32_t code, int t, const ScaleFmt& f) -> v2h {
        const uint32_t b = BLOCK == 16 && t >= 2 ? (code >> 8) & 0xFFu : code & 0xFFu;
        if (MODE == 0 || MODE == 6) {
            const v2h s2 = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(b, 1.0f, false);
            return v2h{s2[0], s2[0]};
        }
        const _Float16 v = (_Float16)scale_decode_any(b, f);
        return v2h{v, v};
    };
    // fp32 scale of dword t times the power-of-two part p of the tensor scale
    auto scale_f = [&](uint32_t code, int t, const ScaleFmt& f, float pp) -> float {
        const uint32_t b = BLOCK == 16 && t >= 2 ? (code >> 8) & 0xFFu : code & 0xFFu;
        return scale_decode_any(b, f) * pp;
    };

    v4i cw[AH][NQ], ca[AH][NQ];
    uint32_t cs[AH], ct[AH];
    // the wave's j-th chunk into buffer i (past its last: the last again, or
    // chunk 0 for a wave with none; never used)
    auto load = [&](int i, int j) {
        const int cc = mine == 0 ? 0 : first + STEP * (j < mine ? j : mine - 1);
#pragma unroll
        for (int q = 0; q < NQ; ++q) {
            cw[i][q] = *reinterpret_cast<const v4i*>(qw + CB * (int64_t)cc + 16 * q);
            ca[i][q] = *reinterpret_cast<const v4i*>(qa + CB * (int64_t)cc + 16 * q);
        }
        cs[i] = scales_at(sw, cc);
        ct[i] = scales_at(sa, cc);
    };
#pragma unroll
    for (int i = 0; i < AH; ++i) load(i, i);
    v16f acc = {};
    for (int j0 = 0; j0 < mine; j0 += AH) {
#pragma unroll
        for (int i = 0; i < AH; ++i) {
            if (j0 + i < mine) {
                if constexpr (MODE == 2) {
                    const v8i w8{cw[i][0][0], cw[i][0][1], cw[i][0][2], cw[i][0][3], 0, 0, 0, 0};
                    const v8i a8{ca[i][0][0], ca[i][0][1], ca[i][0][2], ca[i][0][3], 0, 0, 0, 0};
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, a8, acc, 4, 4, 0, (int)(cs[i] & 0xFFu),
                                                                           0, (int)(ct[i] & 0xFFu));
                } else if constexpr (MODE == 4) {
                    // elements 0..15 of the lane's 32 are dwords 0, 1 (the
                    // K-half's first block), 16..31 dwords 2, 3
                    const v8i w8{cw[i][0][0], cw[i][0][1], cw[i][0][2], cw[i][0][3], 0, 0, 0, 0};
                    const v8i a0{ca[i][0][0], ca[i][0][1], 0, 0, 0, 0, 0, 0};
                    const v8i a1{0, 0, ca[i][0][2], ca[i][0][3], 0, 0, 0, 0};
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, a0, acc, 4, 4, 0, (int)(cs[i] & 0xFFu), 0,
                                                                           (int)(ct[i] & 0xFFu));
                    acc = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(w8, a1, acc, 4, 4, 0,
                                                                           (int)((cs[i] >> 8) & 0xFFu), 0,
                                                                           (int)((ct[i] >> 8) & 0xFFu));
                } else if constexpr (MODE == 3) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const v8bf xw = nv_convert8_bf16((uint32_t)cw[i][0][t], scale_f(cs[i], t, fw, pw));
                        const v8bf xa = nv_convert8_bf16((uint32_t)ca[i][0][t], scale_f(ct[i], t, fa, pa));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xw, xa, acc, 0, 0, 0);
                    }
                } else if constexpr (MODE == 5) {
                    // elements 8 t .. 8 t + 7: bytes 8 t .. 8 t + 7 of the 32
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int q = t >> 1, d = (2 * t) & 3;
                        const v8bf xw = nv_convert8_fp8((uint32_t)cw[i][q][d], (uint32_t)cw[i][q][d + 1],
                                                        scale_f(cs[i], t, fw, pw));
                        const v8bf xa = nv_convert8_fp8((uint32_t)ca[i][q][d], (uint32_t)ca[i][q][d + 1],
                                                        scale_f(ct[i], t, fa, pa));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(xw, xa, acc, 0, 0, 0);
                    }
                } else if constexpr (MODE == 6) {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const int q = t >> 1, d = (2 * t) & 3;
                        const v8h xw = nv_convert8_int8((uint32_t)cw[i][q][d], (uint32_t)cw[i][q][d + 1],
                                                        scale_h(cs[i], t, fw));
                        const v8h xa = nv_convert8_int8((uint32_t)ca[i][q][d], (uint32_t)ca[i][q][d + 1],
                                                        scale_h(ct[i], t, fa));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xw, xa, acc, 0, 0, 0);
                    }
                } else {
#pragma unroll
                    for (int t = 0; t < 4; ++t) {
                        const v8h xw = nv_convert8((uint32_t)cw[i][0][t], scale_h(cs[i], t, fw));
                        const v8h xa = nv_convert8((uint32_t)ca[i][0][t], scale_h(ct[i], t, fa));
                        acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(xw, xa, acc, 0, 0, 0);
                    }
                }
            }
            load(i, j0 + AH + i);
        }
    }

    // KSPLIT: the waves' partial tiles summed in LDS in wave order
    // (deterministic); wave w then owns registers 4 w .. 4 w + 3 of the sum
    constexpr int NQS = KSPLIT ? 1 : 4;           // register quads this wave stores
    float v[4 * NQS];
    if constexpr (KSPLIT) {
        __shared__ float part[kSmallWaves][16][64];
#pragma unroll
        for (int e = 0; e < 16; ++e) part[wave][e][lane] = acc[e];
        __syncthreads();
#pragma unroll
        for (int e = 0; e < 4; ++e) {
            float sum = part[0][4 * wave + e][lane];
#pragma unroll
            for (int u = 1; u < kSmallWaves; ++u) sum += part[u][4 * wave + e][lane];
            v[e] = sum;
        }
    } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) v[e] = acc[e];
    }

    // register 4 q + e of the tile is D[n0 + 8 q + 4 h + e][m0 + r]: C[m][n ..
    // n + 3] as bf16 (KSPLIT: this wave's q = w)
    const int64_t m = m0 + r;
    if (m >= p.m) return;
    const float g = FOLD ? (p.ga[0] / pa) * (p.gb[0] / pw) : p.ga[0] * p.gb[0];
    uint16_t* crow = p.c + m * p.ldc;
    const bool vec = ((p.ldc & 3) == 0) && ((reinterpret_cast<uintptr_t>(p.c) & 7) == 0);
#pragma unroll
    for (int qi = 0; qi < NQS; ++qi) {
        const int q = KSPLIT ? wave : qi;
        const int64_t n = n0 + 8 * q + 4 * h;
        const uint32_t b0 = f32_to_bf16_rne(v[4 * qi + 0] * g), b1 = f32_to_bf16_rne(v[4 * qi + 1] * g);
        const uint32_t b2 = f32_to_bf16_rne(v[4 * qi + 2] * g), b3 = f32_to_bf16_rne(v[4 * qi + 3] * g);
        if (vec && n + 3 < p.n) {
            *reinterpret_cast<uint2*>(crow + n) = uint2{b0 | (b1 << 16), b2 | (b3 << 16)};
        } else {
            if (n + 0 < p.n) crow[n + 0] = (uint16_t)b0;
            if (n + 1 < p.n) crow[n + 1] = (uint16_t)b1;
            if (n + 2 < p.n) crow[n + 2] = (uint16_t)b2;
            if (n + 3 < p.n) crow[n + 3] = (uint16_t)b3;
        }
    }
}

// The small path takes E2M1 operands with E8M0 scales (block 32 or 16), or with
// f16- or bf16-exact ExMy scale formats on both sides, and the 8-bit
// pairings of the tiled register-conversion kernel (MXFP8, INT8 with E4M3
// scales), when M * N is at most
// g_gemm_small_outputs (E8M0: an eighth of it; the bf16 forms, whose tiled
// kernel is slower, one and a half times it).  Measured on the MI355X at
// K = 4096, the small path runs at about 0.27 PFLOP/s whatever the shape,
// while a 256 x 256 tile of the f16 form takes about 90 us and one of MXFP4
// about 30 us however few tiles there are: NVFP4 64 x 11008 37 us against
// 91, 512 x 4096 68 against 89, 256 x 11008 111 against 92 (tiled), and
// MXFP4 64 x 11008 37 against 31 (tiled); UE5M3 (bf16 form) 64 x 11008 63
// against 156, 256 x 11008 126 against 160, 512 x 4096 90 against 159.
bool gemm_small_supported(const GemmLaunch& p)
{
    if ((p.m + 31) / 32 > 65535) return false;
    const int64_t bound = __atomic_load_n(&g_gemm_small_outputs, __ATOMIC_RELAXED);
    const double mn = (double)p.m * (double)p.n;
    if (p.elem == 2) return p.fa.is_e8m0 && p.fb.is_e8m0 && mn <= (double)bound;   // MXFP8
    if (p.elem == 3) return is_e4m3(p.fa) && is_e4m3(p.fb) && mn <= (double)bound; // INT8 with E4M3 scales
    if (p.elem != 0) return false;
    if (p.fa.is_e8m0 && p.fb.is_e8m0) return mn <= (double)bound / 8.0;
    if (p.fa.is_e8m0 || p.fb.is_e8m0) return false;
    if (exact_in_f16(p.fa) && exact_in_f16(p.fb)) return mn <= (double)bound;
    return exact_in_bf16(p.fa) && exact_in_bf16(p.fb) && mn <= 1.5 * (double)bound;
}

// Fewer 32 x 32 output tiles than SIMDs: the four waves of a workgroup split
// K of one tile (more waves in flight, each a quarter of the chunks);
// otherwise each wave takes a tile of its own.  Measured on the MI355X
// (graph replays, us, whole-K waves -> K split): NVFP4 64 x 11008 x 4096
// 37.1 -> 34.7, UE5M3 62.7 -> 41.6, MXFP8 48 -> 42, 64 x 256 x 256 UE5M3
// 9.5 -> 7.5 and MXFP4 6.8 -> 5.9; but NVFP4 512 x 4096 x 4096 (2048
// tiles) 68 -> 85.
template <int MODE, int BLOCK>
static void launch_small_mode(const GemmLaunch& p, hipStream_t s)
{
    const int64_t tm = (p.m + 31) / 32, tn = (p.n + 31) / 32;
    const dim3 t(64 * kSmallWaves);
    if (tm * tn < 1024)
        hipLaunchKernelGGL((k_gemm_small<MODE, BLOCK, true>), dim3((unsigned)tn, (unsigned)tm), t, 0, s, p);
    else
        hipLaunchKernelGGL((k_gemm_small<MODE, BLOCK, false>), dim3((unsigned)((tn + kSmallWaves - 1) / kSmallWaves),
                           (unsigned)tm), t, 0, s, p);
}

hipError_t launch_gemm_small(const GemmLaunch& p, hipStream_t s)
{
    if (p.elem == 2) {
        if (p.block == 16) launch_small_mode<5, 16>(p, s);
        else launch_small_mode<5, 32>(p, s);
    } else if (p.elem == 3) {
        if (p.block == 16) launch_small_mode<6, 16>(p, s);
        else launch_small_mode<6, 32>(p, s);
    } else if (p.fa.is_e8m0) {
        if (p.block == 32) launch_small_mode<2, 32>(p, s);
        else launch_small_mode<4, 16>(p, s);
    } else if (!(exact_in_f16(p.fa) && exact_in_f16(p.fb))) {
        if (p.block == 16) launch_small_mode<3, 16>(p, s);
        else launch_small_mode<3, 32>(p, s);
    } else if (is_e4m3(p.fa) && is_e4m3(p.fb)) {
        if (p.block == 16) launch_small_mode<0, 16>(p, s);
        else launch_small_mode<0, 32>(p, s);
    } else {
        if (p.block == 16) launch_small_mode<1, 16>(p, s);
        else launch_small_mode<1, 32>(p, s);
    }
    return hipGetLastError();
}

// INT4 elements carry 3 significant bits (E2M1: 2), so bf16 holds int * s
// exactly for scale formats with at most 4 mantissa bits.
static bool int4_exact_in_bf16(const ScaleFmtHost& f) { return f.is_e8m0 || f.mbits <= 4; }
// FP8 E4M3 elements carry 4 significant bits: bf16 holds e * s for scales
// with at most 3 mantissa bits.  f16 is never used for them: 448 times a
// scale above 146 overflows it.
static bool fp8_exact_in_bf16(const ScaleFmtHost& f) { return f.is_e8m0 || f.mbits <= 3; }
// INT8 elements carry 7 significant bits: bf16 needs power-of-two scales,
// f16 holds them times E4M3 scales (11 bits, at most 127 * 448 = 56896).
static bool int8_exact_in_bf16(const ScaleFmtHost& f) { return f.is_e8m0 || f.mbits == 0; }
// INT6 elements carry 5 significant bits: bf16 for scales with at most 2
// mantissa bits, f16 for the f16-ranged scale formats with at most 5
// (E4M3, E3M4, E2M5: 31 * 448 = 13888 < 65504).
static bool int6_exact_in_bf16(const ScaleFmtHost& f) { return f.is_e8m0 || f.mbits <= 2; }
static bool int6_exact_in_f16(const ScaleFmtHost& f) { return exact_in_f16(f) && f.mbits <= 5; }

// The 16-bit type of the exact dequantize path for element grid elem and
// scale formats fa, fb: 1 bf16, 2 f16, 0 none exact.
static int dq_type(const ScaleFmtHost& fa, const ScaleFmtHost& fb, int elem)
{
    switch (elem) {
    case 1:
        if (int4_exact_in_bf16(fa) && int4_exact_in_bf16(fb)) return 1;
        return exact_in_f16(fa) && exact_in_f16(fb) ? 2 : 0;
    case 2:
        return fp8_exact_in_bf16(fa) && fp8_exact_in_bf16(fb) ? 1 : 0;
    case 3:
        if (int8_exact_in_bf16(fa) && int8_exact_in_bf16(fb)) return 1;
        return is_e4m3(fa) && is_e4m3(fb) ? 2 : 0;
    case 4:                                         // FP6 E2M3: 4 significant bits, as FP8
        return fp8_exact_in_bf16(fa) && fp8_exact_in_bf16(fb) ? 1 : 0;
    case 5:                                         // FP6 E3M2: 3 significant bits, as INT4
        return int4_exact_in_bf16(fa) && int4_exact_in_bf16(fb) ? 1 : 0;
    case 6:                                         // INT6: 5 significant bits
        if (int6_exact_in_bf16(fa) && int6_exact_in_bf16(fb)) return 1;
        return int6_exact_in_f16(fa) && int6_exact_in_f16(fb) ? 2 : 0;
    default:
        if (exact_in_f16(fa) && exact_in_f16(fb)) return 2;
        return exact_in_bf16(fa) && exact_in_bf16(fb) ? 1 : 0;
    }
}

bool gemm_dq_supported(const ScaleFmtHost& fa, const ScaleFmtHost& fb, int elem)
{
    return dq_type(fa, fb, elem) != 0;
}

// Operands on the INT4 or an 8-bit grid: the exact dequantize path with the
// grid's decode, in the 16-bit type dq_type picks.
template <int BLOCK, int ELEM>
static hipError_t launch_dq_elem(const GemmLaunch& p, bool f16, hipStream_t s)
{
    dim3 grid((unsigned)((p.n + kTile - 1) / kTile), (unsigned)((p.m + kTile - 1) / kTile));
    const size_t sh = sizeof(DqSmem);
    if constexpr (ELEM != 2 && ELEM != 4 && ELEM != 5) {      // FP8 / FP6 elements have no f16 variant
        if (f16) {
            hipError_t e = allow_lds(k_gemm_dq<true, BLOCK, ELEM>, sh);
            if (e != hipSuccess) return e;
            hipLaunchKernelGGL((k_gemm_dq<true, BLOCK, ELEM>), grid, dim3(kGemmThreads), sh, s, p);
            return hipGetLastError();
        }
    }
    hipError_t e = allow_lds(k_gemm_dq<false, BLOCK, ELEM>, sh);
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemm_dq<false, BLOCK, ELEM>), grid, dim3(kGemmThreads), sh, s, p);
    return hipGetLastError();
}

template <int ELEM>
static hipError_t launch_dq_grid(const GemmLaunch& p, bool f16, hipStream_t s)
{
    return p.block == 16 ? launch_dq_elem<16, ELEM>(p, f16, s) : launch_dq_elem<32, ELEM>(p, f16, s);
}

hipError_t launch_gemm_dq(const GemmLaunch& p, hipStream_t s)
{
    if (p.elem != 0) {
        const int t = dq_type(p.fa, p.fb, p.elem);
        if (t == 0) return hipErrorNotSupported;
        // MXFP8: FP8 converted in registers with the E8M0 scale applied;
        // INT8 with E4M3 scales: converted in registers to f16
        if (p.elem == 2 && p.fa.is_e8m0 && p.fb.is_e8m0)
            return p.block == 16 ? launch_nv<16, kNvFp8>(p, s) : launch_nv<32, kNvFp8>(p, s);
        if (p.elem == 3 && is_e4m3(p.fa) && is_e4m3(p.fb))
            return p.block == 16 ? launch_nv<16, kNvInt8>(p, s) : launch_nv<32, kNvInt8>(p, s);
        if (p.elem == 1) return launch_dq_grid<1>(p, t == 2, s);
        if (p.elem == 2) return launch_dq_grid<2>(p, false, s);   // bf16 only
        if (p.elem == 3) return launch_dq_grid<3>(p, t == 2, s);
        if (p.elem == 4) return launch_dq_grid<4>(p, false, s);   // bf16 only
        if (p.elem == 5) return launch_dq_grid<5>(p, false, s);   // bf16 only
        return launch_dq_grid<6>(p, t == 2, s);
    }
    const bool f16 = exact_in_f16(p.fa) && exact_in_f16(p.fb);
    const bool bf16 = exact_in_bf16(p.fa) && exact_in_bf16(p.fb);
    if (!f16 && !bf16) return hipErrorNotSupported;
    if (f16) {
        const bool hw = is_e4m3(p.fa) && is_e4m3(p.fb);
        if (p.block == 16) {
            if (hw) return launch_nv<16, kNvE4M3>(p, s);
            return launch_nv<16, kNvTable>(p, s);
        }
        if (hw) return launch_nv<32, kNvE4M3>(p, s);
        return launch_nv<32, kNvTable>(p, s);
    }
    // bf16 in registers for ExMy scales; E8M0 in a pair (whose smallest
    // products are bf16 subnormals) keeps the LDS dequantize path
    if (!p.fa.is_e8m0 && !p.fb.is_e8m0)
        return p.block == 16 ? launch_nv<16, kNvBf16>(p, s) : launch_nv<32, kNvBf16>(p, s);
    dim3 grid((unsigned)((p.n + kTile - 1) / kTile), (unsigned)((p.m + kTile - 1) / kTile));
    const size_t sh = sizeof(DqSmem);
    hipError_t e = hipSuccess;
    if (f16) e = p.block == 16 ? allow_lds(k_gemm_dq<true, 16>, sh) : allow_lds(k_gemm_dq<true, 32>, sh);
    else e = p.block == 16 ? allow_lds(k_gemm_dq<false, 16>, sh) : allow_lds(k_gemm_dq<false, 32>, sh);
    if (e != hipSuccess) return e;
    if (f16) {
        if (p.block == 16) hipLaunchKernelGGL((k_gemm_dq<true, 16>), grid, dim3(kGemmThreads), sh, s, p);
        else hipLaunchKernelGGL((k_gemm_dq<true, 32>), grid, dim3(kGemmThreads), sh, s, p);
    } else {
        if (p.block == 16) hipLaunchKernelGGL((k_gemm_dq<false, 16>), grid, dim3(kGemmThreads), sh, s, p);
        else hipLaunchKernelGGL((k_gemm_dq<false, 32>), grid, dim3(kGemmThreads), sh, s, p);
    }
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// weight-only GEMM: Y[M, N] = bf16(gw * X[M, K] W[N, K]^T), 1 <= M <= 16
// (quant_prune_distill/574 "Эксперименты": weight-only NVFP4 with a
// memory-bound kernel for small-batch generation; quant_prune_distill/486
// "Метод": the same blocking with 8- and 6-bit elements).
//
// A workgroup owns RG groups of 16 rows of W; its NW waves split K in
// 128-element chunks (wave w takes chunks w, w + NW, ...), and every byte of
// W is read once.  Each chunk is dequantized exactly to bf16 in registers
// and multiplied on the 16x16x32 bf16 matrix cores against X (M padded to 16
// by repeating row M - 1, whose outputs are dropped).  The dot product is a
// sum, so the K order inside a chunk is free: lane group g (lane / 16) takes
// the 32 contiguous elements [32 g, 32 g + 32) of the chunk and feeds 8 of
// them to each of the chunk's four MFMAs, with X read in the same order.
//
// The operands reach the registers through LDS.  In the fragment layout
// every four consecutive lanes hold four different rows, and the texture
// address unit takes such a load one lane per cycle: 64 cycles per KiB of W,
// as many again for the chunk's 2-byte scales and up to four times that for
// X, against the ~13 bytes per cycle per CU that HBM delivers.  So each wave
// streams its chunks with direct-to-LDS loads in an order that keeps every
// four lanes on one 64-byte run of a row (four lanes per cycle) into a
// private ring of D slots (W, its scales, the chunk's M rows of X), and reads
// the fragments from there.  A chunk row of W is 64 bytes for the 4-bit
// grids, 128 for the 8-bit ones and 96 for the 6-bit ones; the wide rows sit
// at a 128-byte pitch (two loads per 16-row group, the 6-bit rows with the
// lanes of the two pieces past their 96 bytes masked off).  A wave reads only what it loaded itself, after
// the load counter says it has landed, so the ring needs no barrier.  The
// 16-byte pieces of a row are XOR-swizzled so that the fragment reads are
// free of bank conflicts.  The waves' partial tiles are summed in LDS in a
// fixed order (deterministic).
// ---------------------------------------------------------------------------
typedef float v4f __attribute__((ext_vector_type(4)));

// Exact bf16 dequantization of one dword of 8 E2M1 codes with scale s.  The
// gfx950 converts apply only the exponent of their scale operand, so:
//  POW2 (E8M0 scales): v_cvt_scalef32_pk_bf16_fp4 with s does everything;
//  otherwise: convert with scale 1 to fp32, multiply by s (exact: at most
//  9 significant bits), keep the top half (exact when the value fits bf16).
// Elements 2b and 2b + 1 of a dword of codes as binary32: the hardware
// E2M1 conversion (scale 1), or for INT4 the sign-extended nibbles.
template <bool INT>
__device__ __forceinline__ v2f elem_pair_f32(uint32_t w, int b)
{
    if (INT)
        return v2f{(float)((int32_t)(w << (28 - 8 * b)) >> 28), (float)((int32_t)(w << (24 - 8 * b)) >> 28)};
    return b == 0 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 0)
         : b == 1 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 1)
         : b == 2 ? __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 2)
                  : __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w, 1.0f, 3);
}

// Elements k and k + 1 (k even) of the codes dw of one chunk row piece (the
// grid's packing: 4-bit nibbles, bytes, or the six-bit stream) as binary32:
// E2M1 and FP8 E4M3 by the hardware conversions (scale 1, exact), INT4 /
// INT8 / INT6 sign-extended, FP6 E2M3 / E3M2 through the FP8 E4M3 / E5M2
// byte of the value times 2^-6 / 2^-12 (exact) and one multiply back.  k is
// a compile-time constant after unrolling.
template <int ELEM>
__device__ __forceinline__ v2f elem_pair_any(const uint32_t* dw, int k)
{
    if constexpr (ELEM <= 1) {
        return elem_pair_f32<ELEM == 1>(dw[k >> 3], (k & 7) >> 1);
    } else if constexpr (ELEM == 2) {
        return (k & 3) ? __builtin_amdgcn_cvt_pk_f32_fp8((int)dw[k >> 2], true)
                       : __builtin_amdgcn_cvt_pk_f32_fp8((int)dw[k >> 2], false);
    } else if constexpr (ELEM == 3) {
        const uint32_t w = dw[k >> 2] >> (8 * (k & 3));
        return v2f{int8_value(w), int8_value(w >> 8)};
    } else {
        const int bit = 6 * k, i = bit >> 5, sh = bit & 31;
        const uint32_t x = sh + 12 <= 32 ? dw[i] >> sh : __builtin_amdgcn_alignbit(dw[i + 1], dw[i], sh);
        if constexpr (ELEM == 6) {
            return v2f{(float)((int32_t)(x << 26) >> 26), (float)((int32_t)(x << 20) >> 26)};
        } else {
            // the two codes to one byte each, sign bit 5 -> 7: the FP8 byte
            const uint32_t y = (x & 0x3Fu) | ((x << 2) & 0x3F00u);
            const uint32_t w = (y & 0x1F1Fu) | ((y & 0x2020u) << 2);
            const v2f e = ELEM == 4 ? __builtin_amdgcn_cvt_pk_f32_fp8((int)w, false)
                                    : __builtin_amdgcn_cvt_pk_f32_bf8((int)w, false);
            constexpr float kFold = ELEM == 4 ? 64.0f : 4096.0f;
            return v2f{e[0] * kFold, e[1] * kFold};
        }
    }
}

// Elements 8t .. 8t + 7 of dw times s as bf16 pairs: hi the truncation of
// each binary32 product (exact when it fits bf16), with SPLIT lo the exact
// remainder (products of up to 16 significant bits).
template <int ELEM, bool SPLIT>
__device__ __forceinline__ void dq8_any(const uint32_t* dw, int t, float s, v4i& hi, v4i& lo)
{
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const v2f f = elem_pair_any<ELEM>(dw, 8 * t + 2 * b);
        const float v0 = f[0] * s, v1 = f[1] * s;
        if (SPLIT) {
            const uint32_t h0 = __float_as_uint(v0) & 0xFFFF0000u, h1 = __float_as_uint(v1) & 0xFFFF0000u;
            const float l0 = v0 - __uint_as_float(h0), l1 = v1 - __uint_as_float(h1);
            hi[b] = (int)((h0 >> 16) | h1);
            lo[b] = (int)((__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u));
        } else {
            hi[b] = (int)__builtin_amdgcn_perm(__float_as_uint(v1), __float_as_uint(v0), 0x07060302u);
        }
    }
}

// INT: INT4 elements (never POW2: the multiply by s is exact for E8M0 too).
template <bool POW2, bool INT = false>
__device__ __forceinline__ v4i dq8_bf16(uint32_t w, float s)
{
    v4i r;
    if (POW2 && !INT) {
        r[0] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 0));
        r[1] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 1));
        r[2] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 2));
        r[3] = __builtin_bit_cast(int, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(w, s, 3));
    } else {
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            const v2f f = elem_pair_f32<INT>(w, b);
            const uint32_t lo = __float_as_uint(f[0] * s), hi = __float_as_uint(f[1] * s);
            r[b] = (int)__builtin_amdgcn_perm(hi, lo, 0x07060302u);     // {hi[31:16], lo[31:16]}
        }
    }
    return r;
}

// Products wider than bf16 (E1M6 with E2M1: 9 significant bits; INT4 with
// 5- or 6-bit mantissas: up to 10): split v = hi + lo, both exact bf16.
template <bool INT = false>
__device__ __forceinline__ void dq8_bf16_split(uint32_t w, float s, v4i& hi, v4i& lo)
{
#pragma unroll
    for (int b = 0; b < 4; ++b) {
        const v2f f = elem_pair_f32<INT>(w, b);
        const float v0 = f[0] * s, v1 = f[1] * s;
        const uint32_t h0 = __float_as_uint(v0) & 0xFFFF0000u, h1 = __float_as_uint(v1) & 0xFFFF0000u;
        const float l0 = v0 - __uint_as_float(h0), l1 = v1 - __uint_as_float(h1);
        hi[b] = (int)((h0 >> 16) | h1);
        lo[b] = (int)((__float_as_uint(l0) >> 16) | (__float_as_uint(l1) & 0xFFFF0000u));
    }
}

// One ring slot of the weight-only GEMM (byte offsets).  A chunk is SUB
// runs of 128 K-elements.  XQ = 0: M == 1, the single X row arrives by
// 4-byte loads (SUB of them); else XQ * SUB loads of four 256-byte X row
// pieces each.  WP: LDS pitch of a W chunk row (64 bytes, or 128 for the
// wider rows); SCB: scale bytes of a row per chunk.
template <int RG, int XQ, int WP, int SUB, int SCB>
struct WoSlot {
    static constexpr int WD = WP / 64;                 // W loads per 16-row group
    static constexpr int W = 0;                        // row r of group g at 16 WP g + WP r
    static constexpr int SC = RG * 16 * WP;            // row r of the slot's 16 RG rows at SC + SCB r
    static constexpr int SCBytes = (RG * 16 * SCB + 255) / 256 * 256;
    static constexpr int NSC = (RG * 16 * SCB / 4 + 63) / 64;      // 4-byte scale loads (64 lanes each)
    static constexpr int X = SC + SCBytes;             // piece h of row m at X + 1024 (SUB (m / 4) + h) + 256 (m % 4)
    static constexpr int XRows = XQ == 0 ? 1 : 4 * XQ;
    static constexpr int Bytes = X + 256 * SUB * XRows;
    static constexpr int Loads = RG * WD + NSC + SUB * (XQ == 0 ? 1 : XQ);   // direct-to-LDS loads per chunk
};

// 16-byte piece c of row r sits at c ^ swz(r): 64-byte rows (r >> 1) & 3,
// 128-byte rows (r >> 1) & 7 (16 consecutive rows, one piece each, on
// distinct banks)
__device__ __forceinline__ int wo_swz(int r) { return (r >> 1) & 3; }
__device__ __forceinline__ int wo_swz8(int r) { return (r >> 1) & 7; }

template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

// Code bytes of a W row per 128 K-elements and the LDS pitch of a chunk row.
template <int ELEM, int SUB>
struct WoRow {
    static constexpr int Bytes128 = ELEM <= 1 ? 64 : ELEM <= 3 ? 128 : 96;
    static constexpr int WB = SUB * Bytes128;
    static constexpr int WP = WB <= 64 ? 64 : 128;
};

template <int NW, int D, int RG, int XQ, int BLOCK, bool SPLIT, bool POW2, int ELEM = 0, int SUB = 1>
__global__ __launch_bounds__(64 * NW) void k_wo_gemm(WoGemmLaunch p)
{
    constexpr bool WIDE = ELEM >= 2;
    static_assert(SUB == 1 || (SUB == 2 && !WIDE), "two runs per chunk for the 4-bit grids");
    constexpr int WP = WoRow<ELEM, SUB>::WP;                   // LDS pitch of a W chunk row
    constexpr int WB = WoRow<ELEM, SUB>::WB;                   // code bytes of a W chunk row
    constexpr int SCB = 128 * SUB / BLOCK;                     // scale bytes of a row per chunk
    constexpr int SDW = SCB / 4;                               // ... in dwords
    using S = WoSlot<RG, XQ, WP, SUB, SCB>;
    static_assert((D - 1) * S::Loads < 64, "loads in flight exceed the counter");
    extern __shared__ __align__(16) uint8_t wo_ring[];
    __shared__ float sdec[256];               // decoded scale times the power-of-two part of g
    const int tid = threadIdx.x, lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);       // wave-uniform (scalar)
    const int r16 = lane & 15, grp = lane >> 4;
    const int64_t n0 = (int64_t)blockIdx.x * (16 * RG);
    const int64_t N = p.n, K = p.k, M = p.m;
    const int64_t rowb = K * (ELEM <= 1 ? 4 : ELEM <= 3 ? 8 : 6) / 8, rows = K / BLOCK;
    const ScaleFmt fw{p.fw.ebits, p.fw.mbits, p.fw.bias, p.fw.maxcode, p.fw.smax, p.fw.is_e8m0};
    const float gw = p.gw[0];
    const float pw = split_pow2(gw);
    const float gres = gw / pw;
    for (int c = tid; c < 256; c += 64 * NW) sdec[c] = scale_decode_any((uint32_t)c, fw) * pw;
    uint8_t* const ring = wo_ring + wave * (D * S::Bytes);
    const int nchunks = (int)(K / (128 * SUB));
    const int mine = nchunks > wave ? (nchunks - wave + NW - 1) / NW : 0;   // chunks wave, wave + NW, ...

    // Global sources of this lane's direct-to-LDS loads for chunk 0, as
    // 32-bit offsets (the ABI bounds W below 4 GiB); rows past N re-read row
    // N - 1, rows of X past M re-read row M - 1 (in bounds, never stored).
    //  W: 64-byte rows: lane l -> row l / 4 of each group, 16-byte piece
    //     (l % 4) ^ swz(row), landing at 64 row + 16 (l % 4); 128-byte pitch:
    //     load k lane l -> row 8 k + l / 8, piece (l % 8) ^ swz8(row), landing
    //     at 128 row + 16 (l % 8) (6-bit: only pieces 0..5 exist; the other
    //     lanes stay idle);
    //  scales: SCB bytes per row; load j lane l -> dword f % SDW of row
    //     f / SDW, f = 64 j + l, landing at 4 f;
    //  X: XQ = 0: load h lane l -> dword l of piece h of row 0; else load
    //     (q, h), lane l -> row m = 4 q + l / 16, 16 bytes (l % 16) ^ (m % 8)
    //     of its piece h, landing at 1024 (SUB q + h) + 16 l.
    uint32_t wsrc[RG][S::WD];
    bool wact[S::WD];
#pragma unroll
    for (int k = 0; k < S::WD; ++k) {
        const int r = WP == 128 ? 8 * k + (lane >> 3) : lane >> 2;
        const int pc = WP == 128 ? (lane & 7) ^ wo_swz8(r) : (lane & 3) ^ wo_swz(r);
        wact[k] = 16 * pc < WB;
#pragma unroll
        for (int g = 0; g < RG; ++g) {
            const int64_t n = n0 + 16 * g + r < N ? n0 + 16 * g + r : N - 1;
            wsrc[g][k] = (uint32_t)(n * rowb) + 16u * (uint32_t)pc;
        }
    }
    uint32_t ssrc[S::NSC];
    bool sact[S::NSC];
#pragma unroll
    for (int j = 0; j < S::NSC; ++j) {
        const int f = 64 * j + lane, R = f / SDW;
        sact[j] = R < 16 * RG;
        const int64_t rr = R < 16 * RG ? R : 16 * RG - 1;
        const int64_t n = n0 + rr < N ? n0 + rr : N - 1;
        ssrc[j] = (uint32_t)(n * rows) + 4u * (uint32_t)(f % SDW);
    }
    constexpr int XL = XQ == 0 ? 1 : XQ;
    const uint16_t* xsrc[XL];
#pragma unroll
    for (int q = 0; q < XL; ++q) {
        if (XQ == 0) {
            xsrc[q] = p.x + 2 * lane;
        } else {
            const int m = 4 * q + (lane >> 4);
            const int64_t mr = m < M ? m : M - 1;
            xsrc[q] = p.x + mr * p.ldx + 8 * ((lane & 15) ^ (m & 7));
        }
    }
    // chunk min(i, mine - 1) of this wave into slot d.  Every load is issued
    // unconditionally (a prefetch past the end re-reads the last chunk), so
    // the number in flight per slot is fixed.
    auto issue = [&](int i, int d) {
        const uint32_t kc = (uint32_t)(wave + (i < mine ? i : mine - 1) * NW);
        uint8_t* const sl = ring + d * S::Bytes;
#pragma unroll
        for (int g = 0; g < RG; ++g)
#pragma unroll
            for (int k = 0; k < S::WD; ++k)
                if (ELEM < 4 || wact[k]) dma16(p.qw + wsrc[g][k] + kc * (uint32_t)WB, sl + S::W + 16 * WP * g + 1024 * k);
#pragma unroll
        for (int j = 0; j < S::NSC; ++j)
            if (sact[j]) dma4(p.sw + ssrc[j] + kc * (uint32_t)SCB, sl + S::SC + 256 * j);
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            if (XQ == 0) {
                dma4(xsrc[0] + kc * (128u * SUB) + 128 * h, sl + S::X + 256 * h);
            } else {
#pragma unroll
                for (int q = 0; q < XL; ++q)
                    dma16(xsrc[q] + kc * (128u * SUB) + 128 * h, sl + S::X + 1024 * (SUB * q + h));
            }
        }
    };

    // this lane's fragment addresses inside a slot, run h of the chunk
    const int mr = r16 < M ? r16 : (int)M - 1;
    auto xoff = [&](int h, int t) {
        return S::X + (XQ == 0 ? 256 * h + 16 * (4 * grp + t)
                               : 1024 * (SUB * (mr >> 2) + h) + 256 * (mr & 3) + 16 * ((4 * grp + t) ^ (mr & 7)));
    };
    // this lane's 32 elements [128 h + 32 grp, + 32) of its row: one 16-byte
    // piece (4-bit), two (8-bit), or bytes 24 grp .. 24 grp + 23 (6-bit)
    auto woff = [&](int h, int j) {
        if (WP == 64) return S::W + 64 * r16 + 16 * (grp ^ wo_swz(r16));
        const int byte = ELEM >= 4 ? 24 * grp + 8 * j : ELEM >= 2 ? 32 * grp + 16 * j : 64 * h + 16 * grp;
        return S::W + WP * r16 + 16 * ((byte >> 4) ^ wo_swz8(r16)) + (byte & 15);
    };
    // the scale bytes of run h: block 16 two (elements 0..15, 16..31), block 32 one
    auto soff = [&](int h) { return S::SC + SCB * r16 + (BLOCK == 16 ? 8 * h + 2 * grp : 4 * h + grp); };

    v4f acc[RG];
#pragma unroll
    for (int g = 0; g < RG; ++g) acc[g] = v4f{0.f, 0.f, 0.f, 0.f};
    auto consume = [&](int d) {
        const uint8_t* const sl = ring + d * S::Bytes;
#pragma unroll
        for (int h = 0; h < SUB; ++h) {
            v4i xf[4];
#pragma unroll
            for (int t = 0; t < 4; ++t) xf[t] = *reinterpret_cast<const v4i*>(sl + xoff(h, t));
#pragma unroll
            for (int g = 0; g < RG; ++g) {
                v4i wv;
                uint32_t dw[8];
                if constexpr (!WIDE) {
                    wv = *reinterpret_cast<const v4i*>(sl + woff(h, 0) + 16 * WP * g);
                } else if constexpr (ELEM <= 3) {
                    const v4i w0 = *reinterpret_cast<const v4i*>(sl + woff(h, 0) + 16 * WP * g);
                    const v4i w1 = *reinterpret_cast<const v4i*>(sl + woff(h, 1) + 16 * WP * g);
#pragma unroll
                    for (int i = 0; i < 4; ++i) { dw[i] = (uint32_t)w0[i]; dw[4 + i] = (uint32_t)w1[i]; }
                } else {
#pragma unroll
                    for (int j = 0; j < 3; ++j) {
                        const uint64_t v = *reinterpret_cast<const uint64_t*>(sl + woff(h, j) + 16 * WP * g);
                        dw[2 * j] = (uint32_t)v;
                        dw[2 * j + 1] = (uint32_t)(v >> 32);
                    }
                    dw[6] = dw[7] = 0u;
                }
                const uint32_t sc = BLOCK == 16 ? (uint32_t)*reinterpret_cast<const uint16_t*>(sl + soff(h) + 16 * SCB * g)
                                                : (uint32_t)sl[soff(h) + 16 * SCB * g];
                const float s0 = sdec[sc & 0xFFu];
                const float s1 = BLOCK == 16 ? sdec[(sc >> 8) & 0xFFu] : s0;
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                    const float st = t < 2 ? s0 : s1;                   // elements 0..15: the first block
                    if constexpr (WIDE) {
                        v4i hi, lo;
                        dq8_any<ELEM, SPLIT>(dw, t, st, hi, lo);
                        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xf[t]),
                                                                         __builtin_bit_cast(v8bf, hi), acc[g], 0, 0, 0);
                        if (SPLIT)
                            acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xf[t]),
                                                                             __builtin_bit_cast(v8bf, lo), acc[g], 0, 0, 0);
                    } else if (SPLIT) {
                        v4i hi, lo;
                        dq8_bf16_split<ELEM == 1>((uint32_t)wv[t], st, hi, lo);
                        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xf[t]),
                                                                         __builtin_bit_cast(v8bf, hi), acc[g], 0, 0, 0);
                        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xf[t]),
                                                                         __builtin_bit_cast(v8bf, lo), acc[g], 0, 0, 0);
                    } else {
                        const v4i wt = dq8_bf16<POW2, ELEM == 1>((uint32_t)wv[t], st);
                        acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(v8bf, xf[t]),
                                                                         __builtin_bit_cast(v8bf, wt), acc[g], 0, 0, 0);
                    }
                }
            }
        }
        // the slot's reads have returned before a load may overwrite it
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    };

    if (mine > 0) {
#pragma unroll
        for (int d = 0; d < D; ++d) issue(d, d);
    }
    // sdec is complete once every wave's LDS writes are; a plain barrier (no
    // fence) leaves the ring's loads in flight
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    __builtin_amdgcn_s_barrier();
    if (mine > 0) {
        int i0 = 0;
        for (; i0 + D <= mine; i0 += D) {        // whole groups: no conditions inside
#pragma unroll
            for (int d = 0; d < D; ++d) {
                wait_vmcnt<(D - 1) * S::Loads>();
                consume(d);
                issue(i0 + d + D, d);
            }
        }
        // the last mine % D chunks: slot d has the loads of slots d + 1 .. D - 1 behind it
        if (i0 + 0 < mine) { wait_vmcnt<(D - 1) * S::Loads>(); consume(0); }
        if (D > 2 && i0 + 1 < mine) { wait_vmcnt<(D > 2 ? (D - 2) * S::Loads : 0)>(); consume(1); }
        if (D > 3 && i0 + 2 < mine) { wait_vmcnt<(D > 3 ? (D - 3) * S::Loads : 0)>(); consume(2); }
        if (D > 4 && i0 + 3 < mine) { wait_vmcnt<(D > 4 ? (D - 4) * S::Loads : 0)>(); consume(3); }
        if (D > 5 && i0 + 4 < mine) { wait_vmcnt<(D > 5 ? (D - 5) * S::Loads : 0)>(); consume(4); }
        if (D > 6 && i0 + 5 < mine) { wait_vmcnt<(D > 6 ? (D - 6) * S::Loads : 0)>(); consume(5); }
        if (D > 7 && i0 + 6 < mine) { wait_vmcnt<(D > 7 ? (D - 7) * S::Loads : 0)>(); consume(6); }
    }
    // every wave's loads have landed and its reads returned before the ring
    // is reused for the partial tiles
    wait_vmcnt<0>();
    __syncthreads();
    // acc[g][r] = D[m = 4 grp + r][n = 16 g + r16]; fixed-order sum over the waves
    float (*red)[RG][256] = reinterpret_cast<float (*)[RG][256]>(wo_ring);
#pragma unroll
    for (int g = 0; g < RG; ++g)
#pragma unroll
        for (int r = 0; r < 4; ++r) red[wave][g][lane * 4 + r] = acc[g][r];
    __syncthreads();
    for (int e = tid; e < 256 * RG; e += 64 * NW) {
        const int g = e >> 8, t = e & 255;
        float sum = 0.0f;
#pragma unroll
        for (int w = 0; w < NW; ++w) sum += red[w][g][t];
        const int l = t >> 2, r = t & 3;
        const int64_t m = 4 * (l >> 4) + r, nn = n0 + 16 * g + (l & 15);
        if (m < M && nn < N) p.y[m * p.ldy + nn] = (uint16_t)f32_to_bf16_rne(sum * gres);
    }
}

template <int RG, int XQ, int ELEM, int SUB, int BLOCK>
using WoSlotOf = WoSlot<RG, XQ, WoRow<ELEM, SUB>::WP, SUB, 128 * SUB / BLOCK>;

// A ring of NW waves x D slots when it fits the LDS next to the scale
// table, else four waves x two slots.
template <int NW, int D, int RG, int XQ, int BLOCK, bool SPLIT, bool POW2, int ELEM, int SUB>
static hipError_t launch_wo_k(const WoGemmLaunch& p, hipStream_t s)
{
    constexpr size_t sh = (size_t)NW * D * WoSlotOf<RG, XQ, ELEM, SUB, BLOCK>::Bytes;   // the ring, later the partial tiles
    if constexpr (sh + sizeof(float) * 256 > 160 * 1024) {
        static_assert(NW != 4 || D != 2, "the smallest ring fits");
        return launch_wo_k<4, 2, RG, XQ, BLOCK, SPLIT, POW2, ELEM, SUB>(p, s);
    }
    static_assert(sh >= sizeof(float) * NW * RG * 256, "partial tiles fit the ring");
    if (sh > 64 * 1024) {
        const hipError_t e = allow_lds(k_wo_gemm<NW, D, RG, XQ, BLOCK, SPLIT, POW2, ELEM, SUB>, sh);
        if (e != hipSuccess) return e;
    }
    const dim3 grid((unsigned)((p.n + 16 * RG - 1) / (16 * RG))), block(64 * NW);
    hipLaunchKernelGGL((k_wo_gemm<NW, D, RG, XQ, BLOCK, SPLIT, POW2, ELEM, SUB>), grid, block, sh, s, p);
    return hipGetLastError();
}

// Significant bits of the largest element of each grid (E2M1 2, INT4 3,
// FP8 E4M3 4, INT8 7, FP6 E2M3 4, FP6 E3M2 3, INT6 5) plus those of the
// scale: products with at most 8 are exact in bf16, the others (at most 14)
// take the hi + lo split.
static bool wo_exact_in_bf16(int elem, const ScaleFmtHost& f)
{
    static const int ebits[7] = {2, 3, 4, 7, 4, 3, 5};
    const int sbits = f.is_e8m0 ? 1 : f.mbits + 1;
    return ebits[elem] + sbits <= 8;
}

// SUB: 128-element runs per chunk of the 4-bit grids (the wider grids
// take one).
template <int NW, int D, int RG, int XQ, int ELEM, int SUB>
static hipError_t launch_wo_w(const WoGemmLaunch& p, hipStream_t s)
{
    constexpr int U = ELEM >= 2 ? 1 : SUB;
    const bool split = !wo_exact_in_bf16(ELEM, p.fw);
    if (p.block == 16) {
        if (split) return launch_wo_k<NW, D, RG, XQ, 16, true, false, ELEM, U>(p, s);
        return launch_wo_k<NW, D, RG, XQ, 16, false, false, ELEM, U>(p, s);
    }
    if (split) return launch_wo_k<NW, D, RG, XQ, 32, true, false, ELEM, U>(p, s);
    return launch_wo_k<NW, D, RG, XQ, 32, false, false, ELEM, U>(p, s);
}

template <int NW, int D, int RG, int XQ, int SUB>
static hipError_t launch_wo_x(const WoGemmLaunch& p, hipStream_t s)
{
    switch (p.elem) {
    case 1: return launch_wo_w<NW, D, RG, XQ, 1, SUB>(p, s);
    case 2: return launch_wo_w<NW, D, RG, XQ, 2, SUB>(p, s);
    case 3: return launch_wo_w<NW, D, RG, XQ, 3, SUB>(p, s);
    case 4: return launch_wo_w<NW, D, RG, XQ, 4, SUB>(p, s);
    case 5: return launch_wo_w<NW, D, RG, XQ, 5, SUB>(p, s);
    case 6: return launch_wo_w<NW, D, RG, XQ, 6, SUB>(p, s);
    default: break;
    }
    const bool split = !exact_in_bf16(p.fw), pow2 = p.fw.is_e8m0 != 0;
    if (p.block == 16) {
        if (split) return launch_wo_k<NW, D, RG, XQ, 16, true, false, 0, SUB>(p, s);
        if (pow2) return launch_wo_k<NW, D, RG, XQ, 16, false, true, 0, SUB>(p, s);
        return launch_wo_k<NW, D, RG, XQ, 16, false, false, 0, SUB>(p, s);
    }
    if (split) return launch_wo_k<NW, D, RG, XQ, 32, true, false, 0, SUB>(p, s);
    if (pow2) return launch_wo_k<NW, D, RG, XQ, 32, false, true, 0, SUB>(p, s);
    return launch_wo_k<NW, D, RG, XQ, 32, false, false, 0, SUB>(p, s);
}



constexpr int64_t kWoManyGroups = 512;   // 16-row groups that fill the device on their own

// Zero fill of a bf16 matrix with row stride ld, one 2-byte store per
// element (a kernel rather than a memset, so graph capture records a kernel
// node).
__global__ __launch_bounds__(256) void k_fill_zero_bf16(uint16_t* __restrict__ c, int64_t ld, int64_t rows,
                                                        int64_t cols)
{
    const int64_t n = rows * cols;
    for (int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (int64_t)gridDim.x * 256)
        c[(i / cols) * ld + i % cols] = 0;
}

hipError_t launch_fill_zero_bf16(uint16_t* c, int64_t ld, int64_t rows, int64_t cols, hipStream_t s)
{
    const int64_t n = rows * cols;
    if (n == 0) return hipSuccess;
    const int64_t want = (n + 255) / 256;
    const unsigned blocks = (unsigned)(want < 4096 ? want : 4096);
    hipLaunchKernelGGL(k_fill_zero_bf16, dim3(blocks), dim3(256), 0, s, c, ld, rows, cols);
    return hipGetLastError();
}

// Per problem class (measured on the Qwen-2.5 7B MLP decode shapes):
//  M = 1: four waves with four slots each; with fewer than 512 row groups
//   eight waves, so that the single workgroup per CU still keeps 32 chunks
//   in flight.
//  M > 1 with many row groups: two row groups share every X chunk; for
//   M > 8 the slot is 6.4 KB and two slots per wave keep three workgroups
//   per CU resident.
//  M > 4 with few row groups (one workgroup per CU): chunks of two
//   128-element runs for the 4-bit grids, so each wave's X, scale and W
//   loads and waits cover twice the weight bytes (down projection, M = 16:
//   19.1 -> 17.3 us, where the 10.5 KB slot leaves room for two per wave;
//   with many row groups the larger ring costs resident workgroups and is
//   slower, and at M = 1 the single run per chunk is faster).
//  Each grid takes the ring asked for when its slot fits the LDS, else
//  four waves x two slots.
hipError_t launch_wo_gemm(const WoGemmLaunch& p, hipStream_t s)
{
    const bool many = (p.n + 15) / 16 >= kWoManyGroups;
    if (p.m == 1) return many ? launch_wo_x<4, 4, 1, 0, 1>(p, s) : launch_wo_x<8, 4, 1, 0, 1>(p, s);
    if (p.m <= 4) return many ? launch_wo_x<4, 4, 2, 1, 1>(p, s) : launch_wo_x<4, 4, 1, 1, 1>(p, s);
    if (p.m <= 8) return many ? launch_wo_x<4, 4, 2, 2, 1>(p, s) : launch_wo_x<4, 4, 1, 2, 2>(p, s);
    return many ? launch_wo_x<4, 2, 2, 4, 1>(p, s) : launch_wo_x<4, 4, 1, 4, 2>(p, s);
}

}  // namespace fp4
