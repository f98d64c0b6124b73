// lowrank_ef_kernels.hip -- the rank-r compressor inside the error-feedback loop.
//
// Paper: "Accelerating Parallel Diffusion Model Serving with Residual
// Compression" (Luo et al., NeurIPS 2025).  The method sends step-wise
// residuals with error feedback (abstract); the reproducibility table's
// "Pseudocode" entry gives the subspace iteration (Algorithm 3) as a
// compressor.  Combined like the quantizer's DELTA mode:
//
//   sender:   r = (x - prev) + err;  A = bf16(r);  (U, R_U, V) = Algorithm 3 (A)
//             err' = r - (U R_U) V^T;  prev' = x
//   receiver: base' = base + (U R_U) V^T;  xhat = bf16(base')
//
// Two kernels here; Algorithm 3 itself is the low-rank path's.
//   lr_ef_residual_kernel   one pass over x, prev, err: writes r into err, x into prev and
//                           bf16(r) into A (16 bytes per element, HBM bound).
//   lr_ef_update_kernel<RP> Y = Y +- (U R_U) V^T for an m x n fp32 Y, optionally writing
//                           bf16(Y') too (8 or 10 bytes per element, HBM bound).  The
//                           rank-r product is a contraction over r <= 32, evaluated as
//                           U (V R_U^T)^T on v_mfma_f32_16x16x4_f32: a work-group owns
//                           256 columns of 64 rows (128 at r > 16), forms its columns'
//                           rows of V R_U^T once on MFMA, in registers, and streams the
//                           block's rows of Y and U.  Its RESID form is the sender's
//                           update deferred into the next step's residual pass
//                           (24 -> 16 bytes per element over the two passes).
//                           Sender and receiver run the same kernel on the same factors,
//                           so their reconstructions agree bit for bit.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "cfz_internal.h"

namespace cfz {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;
constexpr int kUpdRows = 64;   // rows of Y per work-group of the update at r <= 16
constexpr int kUpdCols = 256;  // columns per work-group (each wave: 64 = 4 tiles of 16)

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi)
{
    typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
    bf16x2 v = {(__bf16)lo, (__bf16)hi};
    return __builtin_bit_cast(uint32_t, v);
}

// Work-groups of one matrix go to one XCD (blocks are dealt to the 8 XCDs
// round-robin), so the matrix's U and V are read into one L2.
__device__ __forceinline__ int xcd_remap(int id, int n)
{
    const int per = n / 8, rem = n % 8, x = id % 8, s = id / 8;
    return x < rem ? x * (per + 1) + s : rem * (per + 1) + (x - rem) * per + s;
}

// ---------------------------------------------------------------- residual

__global__ void __launch_bounds__(kThreads)
lr_ef_residual_kernel(const uint16_t *__restrict__ x, uint16_t *__restrict__ prev,
                      float *__restrict__ err, uint16_t *__restrict__ A, int64_t nquads)
{
    const int64_t q = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (q >= nquads)
        return;
    const u32x2 xv = __builtin_nontemporal_load((const u32x2 *)x + q);
    const u32x2 pv = __builtin_nontemporal_load((const u32x2 *)prev + q);
    const f32x4 ev = __builtin_nontemporal_load((const f32x4 *)err + q);
    f32x4 r;
    r[0] = (bf16_lo(xv[0]) - bf16_lo(pv[0])) + ev[0];
    r[1] = (bf16_hi(xv[0]) - bf16_hi(pv[0])) + ev[1];
    r[2] = (bf16_lo(xv[1]) - bf16_lo(pv[1])) + ev[2];
    r[3] = (bf16_hi(xv[1]) - bf16_hi(pv[1])) + ev[3];
    __builtin_nontemporal_store(r, (f32x4 *)err + q);
    __builtin_nontemporal_store(xv, (u32x2 *)prev + q);
    // A is read again at once by the subspace iteration: a normal store keeps it in cache
    *((u32x2 *)A + q) = u32x2{pack_bf16x2(r[0], r[1]), pack_bf16x2(r[2], r[3])};
}

// ---------------------------------------------------------------- reconstruct and update

// D(16 x 16) += A(16 x 4) B(4 x 16) in fp32: lane l gives A[l % 16][l / 16] and
// B[l / 16][l % 16] and holds D[4 (l / 16) + v][l % 16] in item v.
__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// n floats from p into o[0..N), zero past `valid`; `vec` means all N are valid and p is
// aligned to the vector width used.
template <int N>
__device__ __forceinline__ void load_floats(const float *p, int valid, bool vec, float (&o)[N])
{
    if (vec) {
        if constexpr (N % 4 == 0) {
#pragma unroll
            for (int q = 0; q < N / 4; ++q) {
                const f32x4 t = *((const f32x4 *)p + q);
                o[4 * q] = t[0], o[4 * q + 1] = t[1], o[4 * q + 2] = t[2], o[4 * q + 3] = t[3];
            }
        } else {
            typedef float f32x2 __attribute__((ext_vector_type(2)));
#pragma unroll
            for (int q = 0; q < N / 2; ++q) {
                const f32x2 t = *((const f32x2 *)p + q);
                o[2 * q] = t[0], o[2 * q + 1] = t[1];
            }
        }
    } else {
#pragma unroll
        for (int i = 0; i < N; ++i)
            o[i] = i < valid ? p[i] : 0.0f;
    }
}

// Y = Y +- U (V R_U^T)^T for one ROWS x 256 block of one matrix; the same product as
// (U R_U) V^T.  Wave w owns columns 64 w .. 64 w + 63 of the block (4 tiles of 16).
//   prologue: the wave forms V R_U^T for its tiles on MFMA as R_U V^T (16 k x 16 columns
//             per tile, K = r over l), lane group g holding l = g S + s in step s
//             (S = RP / 4).  The result leaves lane (c, g) with W[column c][k = 16 kt + 4 g
//             + v] in item v of k-tile kt -- exactly the A operand of the main product when
//             its step j gives lane group g the index k = 16 (j / 4) + 4 g + j % 4, so no
//             layout change is needed, and U's operands are 4 consecutive floats of a row.
//   main loop: 32 rows per step; the MFMA result holds 16 rows x 4 columns per lane
//             group, so each lane would touch 64-byte pieces of 16 rows; instead the wave
//             passes its 32 x 64 result through its own LDS region and reads and writes Y as
//             4 rows x 256 bytes per instruction.  The next step's loads are issued before
//             this step's stores (vector memory counters retire in order, so waiting for a
//             step's loads never waits for the stores queued behind them), and the first
//             step's loads before the prologue.
// Short blocks (64 rows at r <= 16, 128 at r = 32) keep many work-groups in the grid; the
// MFMA prologue is what makes them affordable (see the launcher).
// RESID: the sender's pending update fused into the next step's residual pass -- Y is
// the carried error's buffer holding the previous residual r0; each element becomes
// e = r0 - D (the value the update alone would store), then the new residual
// r = (x - prev) + e is stored into Y, x into prev and bf16(r) into A (x, prev and A
// as in the residual kernel; sign and xhat unused).
template <int RP, int ROWS, bool RESID>
__global__ void __launch_bounds__(kThreads)
lr_ef_update_kernel(int64_t m, int64_t n, int r, const float *__restrict__ U,
                    const float *__restrict__ V, const float *__restrict__ RU, float sign,
                    float *__restrict__ Y, uint16_t *__restrict__ xhat, int row_groups,
                    int col_groups, const uint16_t *__restrict__ x, uint16_t *__restrict__ prev,
                    uint16_t *__restrict__ A)
{
    static_assert(RP == 16 || RP == 32, "rank padded to 16 or 32");
    static_assert(ROWS % 32 == 0, "whole 32-row steps");
    constexpr int J = RP / 4, KT = RP / 16, S = RP / 4;
    constexpr int SD = 64 + 4;  // padded row of a wave's result tile (floats)
    __shared__ f32x4 sD[4][32][SD / 4];

    const int groups = row_groups * col_groups;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int64_t b = lid / groups;
    const int t = lid % groups;
    const int64_t row0 = (int64_t)(t / col_groups) * ROWS;
    const int64_t col0 = (int64_t)(t % col_groups) * kUpdCols;
    const float *Ub = U + b * m * r;
    const float *Vb = V + b * n * r;
    const float *Rb = RU + b * r * r;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    float *Yb = Y + b * m * n;
    uint16_t *Xb = xhat ? xhat + b * m * n : nullptr;
    // streaming layout: instruction k of row tile h covers rows 16 h + 4 k + lane / 16,
    // this lane's 4 columns being 4 (lane % 16) of the wave's 64
    const int64_t col = col0 + 64 * wave + 4 * li;
    const bool col_ok = col < n;  // n % 8 == 0: all four or none
    const bool vec = r == RP;     // rows of U, V and R_U 16-byte aligned, no tail

    f32x4 yv[2][4];
    u32x2 xv[2][4], pv[2][4];
    auto load_step = [&](int rb) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t row = row0 + 16 * (rb + h) + 4 * k + g;
                const bool ok = col_ok && row < m;
                yv[h][k] = ok ? __builtin_nontemporal_load((const f32x4 *)(Yb + row * n + col))
                              : f32x4{0, 0, 0, 0};
                if constexpr (RESID) {
                    const int64_t o = b * m * n + row * n + col;
                    xv[h][k] = ok ? __builtin_nontemporal_load((const u32x2 *)(x + o)) : u32x2{0, 0};
                    pv[h][k] = ok ? __builtin_nontemporal_load((const u32x2 *)(prev + o)) : u32x2{0, 0};
                }
            }
    };
    load_step(0);

    float vop[4][J];
    {
        float ra[KT][S];
        const int lv = r - g * S;  // valid l of this lane group
#pragma unroll
        for (int kt = 0; kt < KT; ++kt) {
            const int kr = 16 * kt + li;
            if (kr < r && lv > 0)
                load_floats<S>(Rb + kr * r + g * S, lv, vec, ra[kt]);
            else
#pragma unroll
                for (int s = 0; s < S; ++s)
                    ra[kt][s] = 0.0f;
        }
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) {
            const int64_t c = col0 + 64 * wave + 16 * ct + li;
            float vb[S];
            if (c < n && lv > 0)
                load_floats<S>(Vb + c * r + g * S, lv, vec, vb);
            else
#pragma unroll
                for (int s = 0; s < S; ++s)
                    vb[s] = 0.0f;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                f32x4 w = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int s = 0; s < S; ++s)
                    w = mfma4(ra[kt][s], vb[s], w);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    vop[ct][4 * kt + v] = w[v];
            }
        }
    }

    for (int rb = 0; rb < ROWS / 16; rb += 2) {
        if (row0 + 16 * rb >= m)
            break;  // uniform over the work-group
        float uop[2][J];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t row = row0 + 16 * (rb + h) + li;
#pragma unroll
            for (int kt = 0; kt < KT; ++kt) {
                const int kv = r - (16 * kt + 4 * g);
                float u4[4];
                if (row < m && kv > 0)
                    load_floats<4>(Ub + row * r + 16 * kt + 4 * g, kv, vec, u4);
                else
                    u4[0] = u4[1] = u4[2] = u4[3] = 0.0f;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    uop[h][4 * kt + v] = u4[v];
            }
        }
        // D tiles (row li, columns 16 ct + 4 g) into the wave's LDS tile
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int ct = 0; ct < 4; ++ct) {
                f32x4 d = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
                for (int j = 0; j < J; ++j)
                    d = mfma4(vop[ct][j], uop[h][j], d);
                sD[wave][16 * h + li][4 * ct + g] = d;
            }
        // the tile is private to this wave: order its LDS writes before its reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        f32x4 yc[2][4];
        u32x2 xc[2][4], pc[2][4];
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                yc[h][k] = yv[h][k];
                if constexpr (RESID) {
                    xc[h][k] = xv[h][k];
                    pc[h][k] = pv[h][k];
                }
            }
        if (rb + 2 < ROWS / 16 && row0 + 16 * (rb + 2) < m)
            load_step(rb + 2);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int64_t row = row0 + 16 * (rb + h) + 4 * k + g;
                const f32x4 d = sD[wave][16 * h + 4 * k + g][li];
                if (!col_ok || row >= m)
                    continue;
                f32x4 o;
                if constexpr (RESID) {
                    // e = r0 - D exactly as the sender's update stores it, then the residual
                    // exactly as the residual kernel forms it
                    f32x4 ev;
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        ev[v] = yc[h][k][v] - d[v];
                    const u32x2 xq = xc[h][k], pq = pc[h][k];
                    o[0] = (bf16_lo(xq[0]) - bf16_lo(pq[0])) + ev[0];
                    o[1] = (bf16_hi(xq[0]) - bf16_hi(pq[0])) + ev[1];
                    o[2] = (bf16_lo(xq[1]) - bf16_lo(pq[1])) + ev[2];
                    o[3] = (bf16_hi(xq[1]) - bf16_hi(pq[1])) + ev[3];
                    const int64_t oo = b * m * n + row * n + col;
                    __builtin_nontemporal_store(o, (f32x4 *)(Yb + row * n + col));
                    __builtin_nontemporal_store(xq, (u32x2 *)(prev + oo));
                    // A is read again at once by the subspace iteration: a normal store
                    *(u32x2 *)(A + oo) = u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])};
                } else {
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        o[v] = sign > 0.0f ? yc[h][k][v] + d[v] : yc[h][k][v] - d[v];
                    __builtin_nontemporal_store(o, (f32x4 *)(Yb + row * n + col));
                    if (Xb)
                        __builtin_nontemporal_store(
                            u32x2{pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3])},
                            (u32x2 *)(Xb + row * n + col));
                }
            }
        // the next step's writes to the tile come after these reads
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// Rows per work-group.  At 57 x 1024 x 3072, per sender / receiver / fused call: r = 16
// with 64 rows 249 / 321 / 530 us against 264 / 342 / 568 with 256; r = 32 with 128 rows
// 285 / 353 / 563 us.  Short blocks pay when the prologue is cheap: with V R_U^T formed by
// per-lane fma chains from an LDS copy of R_U, 64-row blocks took 316 us against 271 with
// 256 (sender, r = 16), and the old 256-row kernel 276 / 355 / 578 us.
template <int RP>
constexpr int upd_rows() { return RP == 32 ? 2 * kUpdRows : kUpdRows; }

template <int RP>
hipError_t update_rp(int64_t batch, int64_t m, int64_t n, int r, const float *U, const float *V,
                     const float *RU, float sign, float *Y, uint16_t *xhat, const uint16_t *x,
                     uint16_t *prev, uint16_t *A, hipStream_t st)
{
    constexpr int ROWS = upd_rows<RP>();
    const int rg = (int)((m + ROWS - 1) / ROWS);
    const int cg = (int)((n + kUpdCols - 1) / kUpdCols);
    const int64_t blocks = batch * rg * cg;
    if (x)
        hipLaunchKernelGGL((lr_ef_update_kernel<RP, ROWS, true>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, st, m, n, r, U, V, RU, -1.0f, Y, nullptr, rg, cg, x,
                           prev, A);
    else
        hipLaunchKernelGGL((lr_ef_update_kernel<RP, ROWS, false>), dim3((unsigned)blocks),
                           dim3(kThreads), 0, st, m, n, r, U, V, RU, sign, Y, xhat, rg, cg,
                           nullptr, nullptr, nullptr);
    return hipGetLastError();
}

}  // namespace

// The largest grid any rank class launches (the shortest blocks).
int64_t lowrank_ef_update_blocks(int64_t batch, int64_t m, int64_t n)
{
    return batch * ((m + kUpdRows - 1) / kUpdRows) * ((n + kUpdCols - 1) / kUpdCols);
}

hipError_t launch_lowrank_ef_residual(const uint16_t *x, uint16_t *prev, float *err, uint16_t *A,
                                      int64_t count, hipStream_t st)
{
    const int64_t nq = count / 4;
    if (nq == 0)
        return hipSuccess;
    hipLaunchKernelGGL(lr_ef_residual_kernel, dim3((unsigned)((nq + kThreads - 1) / kThreads)),
                       dim3(kThreads), 0, st, x, prev, err, A, nq);
    return hipGetLastError();
}

hipError_t launch_lowrank_ef_update(int64_t batch, int64_t m, int64_t n, int r, const float *U,
                                    const float *V, const float *RU, float sign, float *Y,
                                    uint16_t *xhat, hipStream_t st)
{
    if (batch == 0)
        return hipSuccess;
    if (r <= 16)
        return update_rp<16>(batch, m, n, r, U, V, RU, sign, Y, xhat, nullptr, nullptr, nullptr, st);
    return update_rp<32>(batch, m, n, r, U, V, RU, sign, Y, xhat, nullptr, nullptr, nullptr, st);
}

hipError_t launch_lowrank_ef_residual_update(int64_t batch, int64_t m, int64_t n, int r,
                                             const float *U, const float *V, const float *RU,
                                             const uint16_t *x, uint16_t *prev, float *err,
                                             uint16_t *A, hipStream_t st)
{
    if (batch == 0)
        return hipSuccess;
    if (r <= 16)
        return update_rp<16>(batch, m, n, r, U, V, RU, -1.0f, err, nullptr, x, prev, A, st);
    return update_rp<32>(batch, m, n, r, U, V, RU, -1.0f, err, nullptr, x, prev, A, st);
}

}  // namespace cfz
