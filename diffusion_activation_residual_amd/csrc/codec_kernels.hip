// codec_kernels.hip -- HIP kernels of the residual codec for gfx950 (CDNA4).
//
// Method (paper "Accelerating Parallel Diffusion Model Serving with Residual
// Compression"): per exchanged tensor and denoising step, send only a
// compressed step-wise residual, with error feedback (abstract); the first,
// uncompressed step initialises the base (reproducibility table, "Dataset
// Splits").  The quantizer is group-wise symmetric absmax, low-bit
// (4 and 2 bit), fp32 scales, round to nearest even.
//
// Layout of the work: the tensor is a flat array of N = rows*cols elements
// (groups never straddle rows because cols % group == 0).  One lane owns a
// chunk of 8 consecutive elements: a 16-byte bf16 load, 32 bytes of fp32
// state, and exactly one packed code word (32 bits at 4 bit, 16 bits at 2 bit).
// A group of G elements is G/8 adjacent lanes of one wavefront, so its absmax
// is a DPP butterfly inside a row of 16 lanes -- no LDS, no barrier.
// Every kernel is a pure stream: each element is read once and written once.
//
// Bit-exactness: fp32 IEEE division for the scale and for r/s, rint (ties to
// even), and explicit fma for the error and base updates; the library is
// compiled with -ffp-contract=off so the compiler adds no other fusion.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cfz_internal.h"

namespace cfz {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kBlock = 256;  // 4 wavefronts of 64

// ---------------------------------------------------------------- helpers

__device__ __forceinline__ u32x4 ld_nt(const u32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ f32x4 ld_nt(const f32x4 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x4 v, u32x4 *p) { __builtin_nontemporal_store(v, p); }
__device__ __forceinline__ void st_nt(f32x4 v, f32x4 *p) { __builtin_nontemporal_store(v, p); }

// element k (0..7) of 8 bf16 values held in a u32x4, widened to fp32 exactly
__device__ __forceinline__ float bf16_at(const u32x4 &v, int k)
{
    uint32_t w = v[k >> 1];
    return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// max over the LANES adjacent lanes that hold one group (LANES = G/8, a power of two <= 16)
template <int LANES>
__device__ __forceinline__ float group_max(float v)
{
    if constexpr (LANES >= 2) v = fmaxf(v, dpp_f32<0xb1>(v));   // quad_perm(1,0,3,2): lane ^ 1
    if constexpr (LANES >= 4) v = fmaxf(v, dpp_f32<0x4e>(v));   // quad_perm(2,3,0,1): lane ^ 2
    if constexpr (LANES >= 8) v = fmaxf(v, dpp_f32<0x141>(v));  // row_half_mirror: joins quads
    if constexpr (LANES >= 16) v = fmaxf(v, dpp_f32<0x140>(v)); // row_mirror: joins half rows
    return v;
}

// fp32 -> bf16, round to nearest even (hardware conversion on gfx950)
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// ---------------------------------------------------------------- compress

// One chunk of 8 elements per lane per unrolled slot; UNROLL slots per lane,
// strided by the block size so that every load instruction is fully coalesced.
template <int BITS, int G, int MODE, int UNROLL>
__global__ void __launch_bounds__(kBlock)
cfz_compress_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ prev,
                    float *__restrict__ base, float *__restrict__ err,
                    uint8_t *__restrict__ codes, float *__restrict__ scales, int64_t nchunks)
{
    constexpr int LANES = G / 8;
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    constexpr bool USE_PREV = (MODE == kDelta);
    constexpr bool USE_BASE = (MODE == kLiteral || MODE == kOff);
    constexpr bool USE_ERR = (MODE == kDelta || MODE == kLiteral);

    const int64_t c0 = (int64_t)blockIdx.x * (kBlock * UNROLL) + threadIdx.x;

    u32x4 xv[UNROLL], pv[UNROLL];
    f32x4 s0[UNROLL], s1[UNROLL], e0[UNROLL], e1[UNROLL];

#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t c = c0 + (int64_t)u * kBlock;
        const bool live = c < nchunks;
        xv[u] = live ? ld_nt((const u32x4 *)(x + 8 * c)) : u32x4{0, 0, 0, 0};
        if constexpr (USE_PREV)
            pv[u] = live ? ld_nt((const u32x4 *)(prev + 8 * c)) : u32x4{0, 0, 0, 0};
        if constexpr (USE_BASE) {
            s0[u] = live ? ld_nt((const f32x4 *)(base + 8 * c)) : f32x4{0, 0, 0, 0};
            s1[u] = live ? ld_nt((const f32x4 *)(base + 8 * c + 4)) : f32x4{0, 0, 0, 0};
        }
        if constexpr (USE_ERR) {
            e0[u] = live ? ld_nt((const f32x4 *)(err + 8 * c)) : f32x4{0, 0, 0, 0};
            e1[u] = live ? ld_nt((const f32x4 *)(err + 8 * c + 4)) : f32x4{0, 0, 0, 0};
        }
    }

#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t c = c0 + (int64_t)u * kBlock;
        const bool live = c < nchunks;

        float r[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const float xk = bf16_at(xv[u], k);
            if constexpr (MODE == kDelta)
                r[k] = (xk - bf16_at(pv[u], k)) + (k < 4 ? e0[u][k] : e1[u][k - 4]);
            else if constexpr (MODE == kLiteral)
                r[k] = (xk - (k < 4 ? s0[u][k] : s1[u][k - 4])) + (k < 4 ? e0[u][k] : e1[u][k - 4]);
            else
                r[k] = xk - (k < 4 ? s0[u][k] : s1[u][k - 4]);
        }

        float a = 0.0f;
#pragma unroll
        for (int k = 0; k < 8; ++k)
            a = fmaxf(a, fabsf(r[k]));
        a = group_max<LANES>(a);
        const float s = a / QMAX;        // IEEE fp32 division
        const bool zero = (s == 0.0f);

        uint32_t word = 0;
        float qf[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            float t = __builtin_rintf(r[k] / s);   // IEEE division, ties to even
            t = fminf(fmaxf(t, -QMAX), QMAX);
            t = zero ? 0.0f : t;
            qf[k] = t;
            word |= ((uint32_t)(int)t & MASK) << (BITS * k);
        }

        if (!live)
            continue;
        if constexpr (BITS == 4)
            ((uint32_t *)codes)[c] = word;
        else
            ((uint16_t *)codes)[c] = (uint16_t)word;
        if ((threadIdx.x & (LANES - 1)) == 0)
            scales[c / LANES] = s;

        if constexpr (USE_ERR) {
            f32x4 n0, n1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                n0[k] = __builtin_fmaf(-qf[k], s, r[k]);
                n1[k] = __builtin_fmaf(-qf[k + 4], s, r[k + 4]);
            }
            st_nt(n0, (f32x4 *)(err + 8 * c));
            st_nt(n1, (f32x4 *)(err + 8 * c + 4));
        }
        if constexpr (USE_PREV)
            st_nt(xv[u], (u32x4 *)(prev + 8 * c));
        if constexpr (USE_BASE) {
            f32x4 n0 = s0[u], n1 = s1[u];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                if (qf[k] != 0.0f) n0[k] = __builtin_fmaf(qf[k], s, n0[k]);
                if (qf[k + 4] != 0.0f) n1[k] = __builtin_fmaf(qf[k + 4], s, n1[k]);
            }
            st_nt(n0, (f32x4 *)(base + 8 * c));
            st_nt(n1, (f32x4 *)(base + 8 * c + 4));
        }
    }
}

// ---------------------------------------------------------------- decode

template <int BITS, int G, bool XHAT, int UNROLL>
__global__ void __launch_bounds__(kBlock)
cfz_decode_kernel(const uint8_t *__restrict__ codes, const float *__restrict__ scales,
                  float *__restrict__ base, uint16_t *__restrict__ xhat, int64_t nchunks)
{
    constexpr int LANES = G / 8;
    const int64_t c0 = (int64_t)blockIdx.x * (kBlock * UNROLL) + threadIdx.x;

    uint32_t word[UNROLL];
    float sc[UNROLL];
    f32x4 b0[UNROLL], b1[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t c = c0 + (int64_t)u * kBlock;
        const bool live = c < nchunks;
        if constexpr (BITS == 4)
            word[u] = live ? __builtin_nontemporal_load((const uint32_t *)codes + c) : 0u;
        else
            word[u] = live ? (uint32_t)__builtin_nontemporal_load((const uint16_t *)codes + c) : 0u;
        sc[u] = live ? scales[c / LANES] : 0.0f;
        b0[u] = live ? ld_nt((const f32x4 *)(base + 8 * c)) : f32x4{0, 0, 0, 0};
        b1[u] = live ? ld_nt((const f32x4 *)(base + 8 * c + 4)) : f32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t c = c0 + (int64_t)u * kBlock;
        if (c >= nchunks)
            continue;
        float b[8];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            b[k] = b0[u][k];
            b[k + 4] = b1[u][k];
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int q = __builtin_amdgcn_sbfe(word[u], BITS * k, BITS);  // sign-extended field
            if (q != 0)
                b[k] = __builtin_fmaf((float)q, sc[u], b[k]);
        }
        st_nt(f32x4{b[0], b[1], b[2], b[3]}, (f32x4 *)(base + 8 * c));
        st_nt(f32x4{b[4], b[5], b[6], b[7]}, (f32x4 *)(base + 8 * c + 4));
        if constexpr (XHAT) {
            u32x4 h = {pack_bf16x2(b[0], b[1]), pack_bf16x2(b[2], b[3]), pack_bf16x2(b[4], b[5]),
                       pack_bf16x2(b[6], b[7])};
            st_nt(h, (u32x4 *)(xhat + 8 * c));
        }
    }
}

// ---------------------------------------------------------------- warm-up

// x0 == nullptr means zeros.  Each of prev/base/err may be nullptr (not written).
__global__ void __launch_bounds__(kBlock)
cfz_warmup_kernel(const uint16_t *__restrict__ x0, uint16_t *__restrict__ prev,
                  float *__restrict__ base, float *__restrict__ err, int64_t nchunks)
{
    const int64_t c = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (c >= nchunks)
        return;
    const u32x4 xv = x0 ? *(const u32x4 *)(x0 + 8 * c) : u32x4{0, 0, 0, 0};
    if (prev)
        *(u32x4 *)(prev + 8 * c) = xv;
    if (base) {
        f32x4 b0, b1;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            b0[k] = bf16_at(xv, k);
            b1[k] = bf16_at(xv, k + 4);
        }
        *(f32x4 *)(base + 8 * c) = b0;
        *(f32x4 *)(base + 8 * c + 4) = b1;
    }
    if (err) {
        const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
        *(f32x4 *)(err + 8 * c) = z;
        *(f32x4 *)(err + 8 * c + 4) = z;
    }
}

// ---------------------------------------------------------------- calibration copy

template <int UNROLL>
__global__ void __launch_bounds__(kBlock)
cfz_stream_copy_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t nvec)
{
    const int64_t i0 = (int64_t)blockIdx.x * (kBlock * UNROLL) + threadIdx.x;
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        v[u] = i < nvec ? ld_nt(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        if (i < nvec)
            st_nt(v[u], dst + i);
    }
}

// ---------------------------------------------------------------- launchers

static inline unsigned grid_for(int64_t items, int64_t per_block)
{
    return (unsigned)((items + per_block - 1) / per_block);
}

template <int BITS, int G, int MODE>
static hipError_t launch_compress_t(const CompressArgs &a, hipStream_t st)
{
    constexpr int UNROLL = 2;
    const unsigned grid = grid_for(a.nchunks, (int64_t)kBlock * UNROLL);
    hipLaunchKernelGGL((cfz_compress_kernel<BITS, G, MODE, UNROLL>), dim3(grid), dim3(kBlock), 0,
                       st, a.x, a.prev, a.base, a.err, a.codes, a.scales, a.nchunks);
    return hipGetLastError();
}

template <int BITS, int G>
static hipError_t launch_compress_g(const CompressArgs &a, hipStream_t st)
{
    switch (a.mode) {
    case kDelta: return launch_compress_t<BITS, G, kDelta>(a, st);
    case kLiteral: return launch_compress_t<BITS, G, kLiteral>(a, st);
    default: return launch_compress_t<BITS, G, kOff>(a, st);
    }
}

template <int BITS>
static hipError_t launch_compress_b(const CompressArgs &a, hipStream_t st)
{
    switch (a.group) {
    case 8: return launch_compress_g<BITS, 8>(a, st);
    case 16: return launch_compress_g<BITS, 16>(a, st);
    case 32: return launch_compress_g<BITS, 32>(a, st);
    case 64: return launch_compress_g<BITS, 64>(a, st);
    default: return launch_compress_g<BITS, 128>(a, st);
    }
}

hipError_t launch_compress(const CompressArgs &a, hipStream_t st)
{
    if (a.nchunks == 0)
        return hipSuccess;
    return a.bits == 4 ? launch_compress_b<4>(a, st) : launch_compress_b<2>(a, st);
}

template <int BITS, int G>
static hipError_t launch_decode_g(const DecodeArgs &a, hipStream_t st)
{
    constexpr int UNROLL = 2;
    const unsigned grid = grid_for(a.nchunks, (int64_t)kBlock * UNROLL);
    if (a.xhat)
        hipLaunchKernelGGL((cfz_decode_kernel<BITS, G, true, UNROLL>), dim3(grid), dim3(kBlock), 0,
                           st, a.codes, a.scales, a.base, a.xhat, a.nchunks);
    else
        hipLaunchKernelGGL((cfz_decode_kernel<BITS, G, false, UNROLL>), dim3(grid), dim3(kBlock),
                           0, st, a.codes, a.scales, a.base, a.xhat, a.nchunks);
    return hipGetLastError();
}

template <int BITS>
static hipError_t launch_decode_b(const DecodeArgs &a, hipStream_t st)
{
    switch (a.group) {
    case 8: return launch_decode_g<BITS, 8>(a, st);
    case 16: return launch_decode_g<BITS, 16>(a, st);
    case 32: return launch_decode_g<BITS, 32>(a, st);
    case 64: return launch_decode_g<BITS, 64>(a, st);
    default: return launch_decode_g<BITS, 128>(a, st);
    }
}

hipError_t launch_decode(const DecodeArgs &a, hipStream_t st)
{
    if (a.nchunks == 0)
        return hipSuccess;
    return a.bits == 4 ? launch_decode_b<4>(a, st) : launch_decode_b<2>(a, st);
}

hipError_t launch_warmup(const uint16_t *x0, uint16_t *prev, float *base, float *err,
                         int64_t nchunks, hipStream_t st)
{
    if (nchunks == 0)
        return hipSuccess;
    hipLaunchKernelGGL(cfz_warmup_kernel, dim3(grid_for(nchunks, kBlock)), dim3(kBlock), 0, st,
                       x0, prev, base, err, nchunks);
    return hipGetLastError();
}

hipError_t launch_stream_copy(const void *src, void *dst, int64_t nvec, hipStream_t st)
{
    if (nvec == 0)
        return hipSuccess;
    constexpr int UNROLL = 4;
    hipLaunchKernelGGL((cfz_stream_copy_kernel<UNROLL>), dim3(grid_for(nvec, kBlock * UNROLL)),
                       dim3(kBlock), 0, st, (const u32x4 *)src, (u32x4 *)dst, nvec);
    return hipGetLastError();
}

}  // namespace cfz
