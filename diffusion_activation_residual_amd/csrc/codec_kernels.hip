// codec_kernels.hip -- HIP kernels of the residual codec for gfx950 (CDNA4).
//
// Method (paper "Accelerating Parallel Diffusion Model Serving with Residual
// Compression"): per exchanged tensor and denoising step, send only a
// compressed step-wise residual, with error feedback (abstract); the first,
// uncompressed step initialises the base (reproducibility table, "Dataset
// Splits").  The quantizer is group-wise symmetric absmax, low-bit
// (4 and 2 bit), fp32 scales, round to nearest even.
//
// Layout of the work: a tensor is a flat array of N = rows*cols elements
// (groups never straddle rows because cols % group == 0).  One lane owns a
// quad of 4 consecutive elements: an 8-byte bf16 load, 16 bytes of fp32 state
// and one packed code field of 16 bits (int4) or 8 bits (int2).  Every load and
// store instruction of a wavefront therefore covers one contiguous span, which
// is what keeps the mixed read/write stream near the copy ceiling.  A group of
// G elements is G/4 adjacent lanes, so its absmax is a DPP butterfly inside a
// row of 16 lanes (plus one swizzle across rows for G = 128) -- no LDS, no
// barrier.  Every kernel is a pure stream: each byte is read or written once.
//
// One launch may cover up to kMaxGroup separately allocated tensors of the same
// bits/group/mode: a table of per-tensor records in the kernel arguments, one
// grid row per tensor, so the K and V of a layer (or any set of tensors
// available at once) cost one launch ramp instead of several.
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
__device__ __forceinline__ float bf16_at8(const u32x4 &v, int k)
{
    uint32_t w = v[k >> 1];
    return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
}

template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v)
{
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xf, 0xf, false));
}

// max over LANES adjacent lanes (a power of two <= 16), inside one row of 16 lanes
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

// ---------------------------------------------------------------- tensor tables

// One 64-byte record per tensor: a work-group reads its tensor's record with a
// single scalar load (blockIdx.y is the tensor, blockIdx.x the block within it;
// work-groups past a smaller tensor's last block have nothing to do).
struct CompressRec {
    const uint16_t *x;
    uint16_t *prev;
    void *base;  // fp32 or bf16 state
    void *err;
    uint8_t *codes;
    float *scales;
    int64_t nquads;
    int64_t pad;
};

struct DecodeRec {
    const uint8_t *codes;
    const float *scales;
    void *base;
    uint16_t *xhat;
    int64_t nquads;
    int64_t pad[3];
};

template <int MAXT>
struct CompressTable {
    CompressRec t[MAXT];
};

template <int MAXT>
struct DecodeTable {
    DecodeRec t[MAXT];
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ u32x2 ld_nt(const u32x2 *p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void st_nt(u32x2 v, u32x2 *p) { __builtin_nontemporal_store(v, p); }

// element k (0..3) of 4 bf16 values held in a u32x2, widened to fp32 exactly
__device__ __forceinline__ float bf16_at(const u32x2 &v, int k)
{
    uint32_t w = v[k >> 1];
    return __uint_as_float((k & 1) ? (w & 0xffff0000u) : (w << 16));
}

// Four consecutive state values (E or X-hat) of one quad, fp32 (16 bytes) or
// bf16 (8 bytes).  `raw` keeps the loaded bf16 bits so that a base element with
// a zero code is stored back bit for bit.
template <bool SB>
struct Quad;

template <>
struct Quad<false> {
    f32x4 v;
    __device__ __forceinline__ void load(const void *p, int64_t q, bool live)
    {
        v = live ? __builtin_nontemporal_load((const f32x4 *)p + q) : f32x4{0, 0, 0, 0};
    }
    __device__ __forceinline__ float get(int k) const { return v[k]; }
    // stores new[k] where keep[k] is false, the loaded value where it is true
    __device__ __forceinline__ void store(void *p, int64_t q, const float (&nv)[4],
                                          const bool (&keep)[4]) const
    {
        f32x4 o;
#pragma unroll
        for (int k = 0; k < 4; ++k)
            o[k] = keep[k] ? v[k] : nv[k];
        __builtin_nontemporal_store(o, (f32x4 *)p + q);
    }
};

template <>
struct Quad<true> {
    u32x2 raw;
    __device__ __forceinline__ void load(const void *p, int64_t q, bool live)
    {
        raw = live ? __builtin_nontemporal_load((const u32x2 *)p + q) : u32x2{0, 0};
    }
    __device__ __forceinline__ float get(int k) const { return bf16_at(raw, k); }
    __device__ __forceinline__ void store(void *p, int64_t q, const float (&nv)[4],
                                          const bool (&keep)[4]) const
    {
        u32x2 o = {pack_bf16x2(nv[0], nv[1]), pack_bf16x2(nv[2], nv[3])};
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t m = (keep[2 * h] ? 0x0000ffffu : 0u) | (keep[2 * h + 1] ? 0xffff0000u : 0u);
            o[h] = (raw[h] & m) | (o[h] & ~m);
        }
        __builtin_nontemporal_store(o, (u32x2 *)p + q);
    }
};

// lane ^ 16 inside each half of the wavefront (ds_swizzle bit mode: and 0x1f, xor 0x10)
__device__ __forceinline__ float swizzle_xor16(float v)
{
    return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x401f));
}

// max over the LANES adjacent lanes of one group (LANES = G/4, a power of two <= 32)
template <int LANES>
__device__ __forceinline__ float group_max4(float v)
{
    v = group_max<(LANES < 16 ? LANES : 16)>(v);
    if constexpr (LANES >= 32) v = fmaxf(v, swizzle_xor16(v));
    return v;
}

// ---------------------------------------------------------------- compress

// Block `blk` (< the tensor's block count) of one tensor's compress: quads
// blk * kBlock * UNROLL + threadIdx.x + u * kBlock, u < UNROLL, those below nquads.
template <int BITS, int G, int MODE, bool SB, int UNROLL>
__device__ __forceinline__ void compress_block(const CompressRec &rec, int64_t blk)
{
    constexpr int LANES = G / 4;
    constexpr float QMAX = (float)((1 << (BITS - 1)) - 1);
    constexpr uint32_t MASK = (1u << BITS) - 1u;
    constexpr bool USE_PREV = (MODE == kDelta);
    constexpr bool USE_BASE = (MODE == kLiteral || MODE == kOff);
    constexpr bool USE_ERR = (MODE == kDelta || MODE == kLiteral);

    const int64_t nq = rec.nquads;
    const uint16_t *__restrict__ x = rec.x;
    uint16_t *__restrict__ prev = rec.prev;
    void *__restrict__ base = rec.base;
    void *__restrict__ err = rec.err;
    uint8_t *__restrict__ codes = rec.codes;
    float *__restrict__ scales = rec.scales;
    const int64_t q0 = blk * (kBlock * UNROLL) + threadIdx.x;

    u32x2 xv[UNROLL], pv[UNROLL];
    Quad<SB> sv[UNROLL], ev[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t q = q0 + (int64_t)u * kBlock;
        const bool live = q < nq;
        xv[u] = live ? ld_nt((const u32x2 *)(x + 4 * q)) : u32x2{0, 0};
        if constexpr (USE_PREV)
            pv[u] = live ? ld_nt((const u32x2 *)(prev + 4 * q)) : u32x2{0, 0};
        if constexpr (USE_BASE)
            sv[u].load(base, q, live);
        if constexpr (USE_ERR)
            ev[u].load(err, q, live);
    }

#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t q = q0 + (int64_t)u * kBlock;
        const bool live = q < nq;

        float r[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const float xk = bf16_at(xv[u], k);
            if constexpr (MODE == kDelta)
                r[k] = (xk - bf16_at(pv[u], k)) + ev[u].get(k);
            else if constexpr (MODE == kLiteral)
                r[k] = (xk - sv[u].get(k)) + ev[u].get(k);
            else
                r[k] = xk - sv[u].get(k);
        }

        float a = fmaxf(fmaxf(fabsf(r[0]), fabsf(r[1])), fmaxf(fabsf(r[2]), fabsf(r[3])));
        a = group_max4<LANES>(a);
        const float s = a / QMAX;        // IEEE fp32 division
        const bool zero = (s == 0.0f);

        uint32_t word = 0;
        float qf[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            float v = __builtin_rintf(r[k] / s);   // IEEE division, ties to even
            v = fminf(fmaxf(v, -QMAX), QMAX);
            v = zero ? 0.0f : v;
            qf[k] = v;
            word |= ((uint32_t)(int)v & MASK) << (BITS * k);
        }

        if (!live)
            continue;
        if constexpr (BITS == 4)
            __builtin_nontemporal_store((uint16_t)word, (uint16_t *)codes + q);
        else
            __builtin_nontemporal_store((uint8_t)word, codes + q);
        if ((threadIdx.x & (LANES - 1)) == 0)
            scales[q / LANES] = s;
        if constexpr (USE_ERR) {
            float n[4];
            const bool none[4] = {false, false, false, false};
#pragma unroll
            for (int k = 0; k < 4; ++k)
                n[k] = __builtin_fmaf(-qf[k], s, r[k]);
            ev[u].store(err, q, n, none);
        }
        if constexpr (USE_PREV)
            st_nt(xv[u], (u32x2 *)(prev + 4 * q));
        if constexpr (USE_BASE) {
            float n[4];
            bool keep[4];
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                keep[k] = (qf[k] == 0.0f);
                n[k] = __builtin_fmaf(qf[k], s, sv[u].get(k));
            }
            sv[u].store(base, q, n, keep);
        }
    }
}

// Grid (gx, tensors, gz): work-group (x, y, z) takes block x + gx * z of tensor y;
// gz > 1 only for a tensor with more blocks than one grid row holds.
__device__ __forceinline__ int64_t grid_block() { return blockIdx.x + (int64_t)gridDim.x * blockIdx.z; }

template <int BITS, int G, int MODE, bool SB, int UNROLL, int MAXT>
__global__ void __launch_bounds__(kBlock) cfz_compress_kernel(const CompressTable<MAXT> tab)
{
    const CompressRec &rec = tab.t[MAXT == 1 ? 0 : blockIdx.y];
    const int64_t blk = grid_block();
    if (blk * (kBlock * UNROLL) < rec.nquads)  // else past a smaller tensor's last block
        compress_block<BITS, G, MODE, SB, UNROLL>(rec, blk);
}

// ---------------------------------------------------------------- decode

template <int BITS, int G, bool SB, int UNROLL>
__device__ __forceinline__ void decode_block(const DecodeRec &rec, int64_t blk)
{
    constexpr int LANES = G / 4;
    const int64_t nq = rec.nquads;
    const uint8_t *__restrict__ codes = rec.codes;
    const float *__restrict__ scales = rec.scales;
    void *__restrict__ base = rec.base;
    uint16_t *__restrict__ xhat = rec.xhat;
    const int64_t q0 = blk * (kBlock * UNROLL) + threadIdx.x;

    uint32_t word[UNROLL];
    float sc[UNROLL];
    Quad<SB> bv[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t q = q0 + (int64_t)u * kBlock;
        const bool live = q < nq;
        if constexpr (BITS == 4)
            word[u] = live ? (uint32_t)__builtin_nontemporal_load((const uint16_t *)codes + q) : 0u;
        else
            word[u] = live ? (uint32_t)__builtin_nontemporal_load(codes + q) : 0u;
        sc[u] = live ? scales[q / LANES] : 0.0f;
        bv[u].load(base, q, live);
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t q = q0 + (int64_t)u * kBlock;
        if (q >= nq)
            continue;
        float n[4];
        bool keep[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int c = __builtin_amdgcn_sbfe(word[u], BITS * k, BITS);  // sign-extended field
            keep[k] = (c == 0);
            n[k] = __builtin_fmaf((float)c, sc[u], bv[u].get(k));
        }
        bv[u].store(base, q, n, keep);
        if (xhat) {
            float o[4];
#pragma unroll
            for (int k = 0; k < 4; ++k)
                o[k] = keep[k] ? bv[u].get(k) : n[k];
            st_nt(u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])}, (u32x2 *)(xhat + 4 * q));
        }
    }
}

template <int BITS, int G, bool SB, int UNROLL, int MAXT>
__global__ void __launch_bounds__(kBlock) cfz_decode_kernel(const DecodeTable<MAXT> tab)
{
    const DecodeRec &rec = tab.t[MAXT == 1 ? 0 : blockIdx.y];
    const int64_t blk = grid_block();
    if (blk * (kBlock * UNROLL) < rec.nquads)
        decode_block<BITS, G, SB, UNROLL>(rec, blk);
}

// ---------------------------------------------------------------- warm-up

// x0 == nullptr means zeros.  Each of prev/base/err may be nullptr (not written).
// With bf16 state the base is a copy of x0 and the error buffer bf16 zeros.
template <bool SB>
__global__ void __launch_bounds__(kBlock)
cfz_warmup_kernel(const uint16_t *__restrict__ x0, uint16_t *__restrict__ prev,
                  void *__restrict__ base, void *__restrict__ err, int64_t nchunks)
{
    const int64_t c = (int64_t)blockIdx.x * kBlock + threadIdx.x;
    if (c >= nchunks)
        return;
    const u32x4 xv = x0 ? *(const u32x4 *)(x0 + 8 * c) : u32x4{0, 0, 0, 0};
    if (prev)
        *(u32x4 *)(prev + 8 * c) = xv;
    if constexpr (SB) {
        if (base)
            *((u32x4 *)base + c) = xv;
        if (err)
            *((u32x4 *)err + c) = u32x4{0, 0, 0, 0};
    } else {
        if (base) {
            f32x4 b0, b1;
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                b0[k] = bf16_at8(xv, k);
                b1[k] = bf16_at8(xv, k + 4);
            }
            *((f32x4 *)base + 2 * c) = b0;
            *((f32x4 *)base + 2 * c + 1) = b1;
        }
        if (err) {
            const f32x4 z = {0.0f, 0.0f, 0.0f, 0.0f};
            *((f32x4 *)err + 2 * c) = z;
            *((f32x4 *)err + 2 * c + 1) = z;
        }
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

// Reads nr 16-byte vectors and writes nw <= nr of them: vector i of src goes to
// dst[i * nw / nr] exactly when that index steps, so the writes are spread evenly
// through the read stream and the traffic keeps one read:write ratio throughout.
// One vector per lane, UNROLL per lane, all loads issued before the stores.
template <int UNROLL>
__global__ void __launch_bounds__(kBlock)
cfz_stream_mix_kernel(const u32x4 *__restrict__ src, u32x4 *__restrict__ dst, int64_t nr,
                      int64_t nw)
{
    const int64_t i0 = (int64_t)blockIdx.x * (kBlock * UNROLL) + threadIdx.x;
    u32x4 v[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        v[u] = i < nr ? ld_nt(src + i) : u32x4{0, 0, 0, 0};
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const int64_t i = i0 + (int64_t)u * kBlock;
        const int64_t j = i * nw / nr;
        if (i < nr && j != (i + 1) * nw / nr)
            st_nt(v[u], dst + j);
    }
}

// ---------------------------------------------------------------- launchers

static inline unsigned grid_for(int64_t items, int64_t per_block)
{
    return (unsigned)((items + per_block - 1) / per_block);
}

// Launches over fewer quads than this ramp up too briefly for one quad per lane
// to keep enough bytes in flight; they take four quads per lane instead.
constexpr int64_t kBigLaunchQuads = (int64_t)4 << 20;
// The grid's x dimension times kBlock threads must stay below 2^32.
constexpr int64_t kMaxGridX = (int64_t)1 << 23;

// Grid for tensors of at most `widest` quads: one work-group per block, in rows of
// at most kMaxGridX work-groups (z) when one row cannot hold them.
static bool plain_grid(int64_t widest, int unroll, int count, dim3 *grid)
{
    const int64_t nblk = (widest + kBlock * unroll - 1) / (kBlock * unroll);
    const int64_t gx = nblk < kMaxGridX ? nblk : kMaxGridX;
    const int64_t gz = (nblk + gx - 1) / gx;
    if (gz > 65535)
        return false;
    *grid = dim3((unsigned)gx, (unsigned)count, (unsigned)gz);
    return true;
}

template <int BITS, int G, int MODE, bool SB, int UNROLL, int MAXT>
static hipError_t compress_chunk(const CompressItem *it, int count, hipStream_t st)
{
    CompressTable<MAXT> tab{};
    int64_t widest = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t nq = it[i].n / 4;
        tab.t[i] = CompressRec{it[i].x, it[i].prev, it[i].base, it[i].err, it[i].codes,
                               it[i].scales, nq, 0};
        widest = nq > widest ? nq : widest;
    }
    dim3 grid;
    if (widest == 0 || !plain_grid(widest, UNROLL, count, &grid))
        return widest == 0 ? hipSuccess : hipErrorInvalidValue;
    hipLaunchKernelGGL((cfz_compress_kernel<BITS, G, MODE, SB, UNROLL, MAXT>), grid, dim3(kBlock),
                       0, st, tab);
    return hipGetLastError();
}

template <int BITS, int G, int MODE, bool SB>
static hipError_t compress_g(const CompressItem *it, int count, int64_t total_quads, hipStream_t st)
{
    const bool big = total_quads >= kBigLaunchQuads;
    if (count == 1)
        return big ? compress_chunk<BITS, G, MODE, SB, 1, 1>(it, 1, st)
                   : compress_chunk<BITS, G, MODE, SB, 4, 1>(it, 1, st);
    if (count == 2)  // a layer's K and V: a 128-byte table (about 0.2% faster than 1 KB)
        return big ? compress_chunk<BITS, G, MODE, SB, 1, 2>(it, 2, st)
                   : compress_chunk<BITS, G, MODE, SB, 4, 2>(it, 2, st);
    return big ? compress_chunk<BITS, G, MODE, SB, 1, kMaxGroup>(it, count, st)
               : compress_chunk<BITS, G, MODE, SB, 4, kMaxGroup>(it, count, st);
}

template <int BITS, int G, bool SB>
static hipError_t compress_m(const CompressItem *it, int count, int mode, int64_t tq, hipStream_t st)
{
    switch (mode) {
    case kDelta: return compress_g<BITS, G, kDelta, SB>(it, count, tq, st);
    case kLiteral: return compress_g<BITS, G, kLiteral, SB>(it, count, tq, st);
    default: return compress_g<BITS, G, kOff, SB>(it, count, tq, st);
    }
}

template <int BITS, bool SB>
static hipError_t compress_b(const CompressItem *it, int count, int group, int mode, int64_t tq,
                             hipStream_t st)
{
    switch (group) {
    case 8: return compress_m<BITS, 8, SB>(it, count, mode, tq, st);
    case 16: return compress_m<BITS, 16, SB>(it, count, mode, tq, st);
    case 32: return compress_m<BITS, 32, SB>(it, count, mode, tq, st);
    case 64: return compress_m<BITS, 64, SB>(it, count, mode, tq, st);
    default: return compress_m<BITS, 128, SB>(it, count, mode, tq, st);
    }
}

hipError_t launch_compress(const CompressItem *items, int count, int bits, int group, int mode,
                           bool state_bf16, hipStream_t st)
{
    CompressItem chunk[kMaxGroup];
    int k = 0;
    int64_t tq = 0;
    for (int i = 0; i <= count; ++i) {
        if (i < count && items[i].n > 0) {
            chunk[k++] = items[i];
            tq += items[i].n / 4;
        }
        if ((k == kMaxGroup || i == count) && k > 0) {
            hipError_t e;
            if (state_bf16)
                e = bits == 4 ? compress_b<4, true>(chunk, k, group, mode, tq, st)
                              : compress_b<2, true>(chunk, k, group, mode, tq, st);
            else
                e = bits == 4 ? compress_b<4, false>(chunk, k, group, mode, tq, st)
                              : compress_b<2, false>(chunk, k, group, mode, tq, st);
            if (e != hipSuccess)
                return e;
            k = 0;
            tq = 0;
        }
    }
    return hipSuccess;
}

template <int BITS, int G, bool SB, int UNROLL, int MAXT>
static hipError_t decode_chunk(const DecodeItem *it, int count, hipStream_t st)
{
    DecodeTable<MAXT> tab{};
    int64_t widest = 0;
    for (int i = 0; i < count; ++i) {
        const int64_t nq = it[i].n / 4;
        tab.t[i] = DecodeRec{it[i].codes, it[i].scales, it[i].base, it[i].xhat, nq, {0, 0, 0}};
        widest = nq > widest ? nq : widest;
    }
    dim3 grid;
    if (widest == 0 || !plain_grid(widest, UNROLL, count, &grid))
        return widest == 0 ? hipSuccess : hipErrorInvalidValue;
    hipLaunchKernelGGL((cfz_decode_kernel<BITS, G, SB, UNROLL, MAXT>), grid, dim3(kBlock), 0, st,
                       tab);
    return hipGetLastError();
}

template <int BITS, int G, bool SB>
static hipError_t decode_g(const DecodeItem *it, int count, int64_t tq, hipStream_t st)
{
    const bool big = tq >= kBigLaunchQuads;
    if (count == 1)
        return big ? decode_chunk<BITS, G, SB, 1, 1>(it, 1, st)
                   : decode_chunk<BITS, G, SB, 4, 1>(it, 1, st);
    if (count == 2)
        return big ? decode_chunk<BITS, G, SB, 1, 2>(it, 2, st)
                   : decode_chunk<BITS, G, SB, 4, 2>(it, 2, st);
    return big ? decode_chunk<BITS, G, SB, 1, kMaxGroup>(it, count, st)
               : decode_chunk<BITS, G, SB, 4, kMaxGroup>(it, count, st);
}

template <int BITS, bool SB>
static hipError_t decode_b(const DecodeItem *it, int count, int group, int64_t tq, hipStream_t st)
{
    switch (group) {
    case 8: return decode_g<BITS, 8, SB>(it, count, tq, st);
    case 16: return decode_g<BITS, 16, SB>(it, count, tq, st);
    case 32: return decode_g<BITS, 32, SB>(it, count, tq, st);
    case 64: return decode_g<BITS, 64, SB>(it, count, tq, st);
    default: return decode_g<BITS, 128, SB>(it, count, tq, st);
    }
}

hipError_t launch_decode(const DecodeItem *items, int count, int bits, int group, bool state_bf16,
                         hipStream_t st)
{
    DecodeItem chunk[kMaxGroup];
    int k = 0;
    int64_t tq = 0;
    for (int i = 0; i <= count; ++i) {
        if (i < count && items[i].n > 0) {
            chunk[k++] = items[i];
            tq += items[i].n / 4;
        }
        if ((k == kMaxGroup || i == count) && k > 0) {
            hipError_t e;
            if (state_bf16)
                e = bits == 4 ? decode_b<4, true>(chunk, k, group, tq, st)
                              : decode_b<2, true>(chunk, k, group, tq, st);
            else
                e = bits == 4 ? decode_b<4, false>(chunk, k, group, tq, st)
                              : decode_b<2, false>(chunk, k, group, tq, st);
            if (e != hipSuccess)
                return e;
            k = 0;
            tq = 0;
        }
    }
    return hipSuccess;
}

hipError_t launch_warmup(const uint16_t *x0, uint16_t *prev, void *base, void *err,
                         bool state_bf16, int64_t nchunks, hipStream_t st)
{
    if (nchunks == 0)
        return hipSuccess;
    if (state_bf16)
        hipLaunchKernelGGL(cfz_warmup_kernel<true>, dim3(grid_for(nchunks, kBlock)), dim3(kBlock),
                           0, st, x0, prev, base, err, nchunks);
    else
        hipLaunchKernelGGL(cfz_warmup_kernel<false>, dim3(grid_for(nchunks, kBlock)), dim3(kBlock),
                           0, st, x0, prev, base, err, nchunks);
    return hipGetLastError();
}

hipError_t launch_stream_mix(const void *src, void *dst, int64_t nr, int64_t nw, hipStream_t st)
{
    if (nr == 0)
        return hipSuccess;
    constexpr int UNROLL = 4;
    hipLaunchKernelGGL((cfz_stream_mix_kernel<UNROLL>), dim3(grid_for(nr, kBlock * UNROLL)),
                       dim3(kBlock), 0, st, (const u32x4 *)src, (u32x4 *)dst, nr, nw);
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
