// lowrank_kernels.hip -- rank-r subspace iteration (paper "Accelerating Parallel
// Diffusion Model Serving with Residual Compression", reproducibility table,
// "Pseudocode", Algorithm 3) for gfx950, batched over independent matrices.
//
//   Q = orth(Q0);  T times { Y = A Q;  Z = A^T Y;  Q = orth(Z) };
//   P = A Q;  (U, R_U) = orth(P);  V = Q.
//
// Tall-skinny products on bf16 MFMA (v_mfma_f32_16x16x32_bf16, fp32 accumulate).
// A is bf16 and exact; the skinny operand (Q or Y, fp32) is split into
// hi = bf16(x) and lo = bf16(x - hi) and both halves are multiplied, so the
// product carries about 16 bits of the skinny operand instead of 8.
//
// orth() is Cholesky-QR applied twice: Gram matrix G = M^T M accumulated in
// fp64 from fp32 rows, r x r Cholesky and triangular inverse in fp64 in LDS,
// then M R^-1 row by row.  A pivot <= 1e-13 * trace(G) / r (or not finite)
// drops the column: zero Q column, zero R row and column.
//
// Skinny operands live in the workspace in "operand layout": hi and lo bf16
// planes of shape [L/8][RP][8], where RP = 16 or 32 is r padded to the MFMA
// width.  One 16-byte load then gives a lane the 8 consecutive k values of one
// column that an MFMA operand slot holds.  A and the skinny operand use the same
// k assignment per (lane / 16, slot), so the sum over k is exact regardless of
// how the instruction orders k internally.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include "cfz_internal.h"

namespace cfz {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kGramRows = 64;     // rows of M per Gram work-group
constexpr int kApplyRows = 256;   // rows of M per apply work-group
constexpr int kAqRows = 64;       // rows of A per A*Q work-group (4 waves x 16)
constexpr int kAtyCols = 64;      // columns of A per A^T*Y work-group (4 waves x 16)

__host__ __device__ inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

// Work-groups are dispatched to the 8 XCDs round-robin by linear id.  Remap so
// that consecutive logical ids (the blocks of one matrix, which share its
// skinny operand) run on one XCD and share its L2.
__device__ __forceinline__ int xcd_remap(int id, int n)
{
    const int per = n / 8, rem = n % 8, x = id % 8, s = id / 8;
    return x < rem ? x * (per + 1) + s : rem * (per + 1) + (x - rem) * per + s;
}

__device__ __forceinline__ f32x4 mfma(bf16x8 a, bf16x8 b, f32x4 c)
{
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ workspace layout

struct Layout {
    int rp;
    int64_t mp, np;             // m, n padded to 64
    int64_t gram_blocks;        // max over (m, n) of row blocks of the Gram kernel
    size_t off_qops, off_yops, off_mf, off_gram, off_r1, off_r1inv, off_rinv;
    size_t layer_bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

Layout make_layout(int64_t m, int64_t n, int r)
{
    Layout L;
    L.rp = r <= 16 ? 16 : 32;
    L.mp = round_up(m, 64);
    L.np = round_up(n, 64);
    const int64_t lmax = m > n ? m : n;
    L.gram_blocks = (lmax + kGramRows - 1) / kGramRows;
    size_t off = 0;
    L.off_qops = off; off = align256(off + (size_t)L.np * L.rp * 2 * 2);
    L.off_yops = off; off = align256(off + (size_t)L.mp * L.rp * 2 * 2);
    L.off_mf = off;   off = align256(off + (size_t)lmax * r * 4);
    L.off_gram = off; off = align256(off + (size_t)L.gram_blocks * L.rp * L.rp * 8);
    L.off_r1 = off;   off = align256(off + (size_t)L.rp * L.rp * 8);
    L.off_r1inv = off; off = align256(off + (size_t)L.rp * L.rp * 8);
    L.off_rinv = off; off = align256(off + (size_t)L.rp * L.rp * 8);
    L.layer_bytes = off;
    return L;
}

// ------------------------------------------------------------------ Y = A Q

// One work-group: 64 rows of A (wave w owns rows 16w..16w+15) against all of Q.
// OUT_OPS: write Y in operand layout (hi/lo planes, rows up to mp, zero beyond m).
// Otherwise write Y as fp32 [m][r].
template <int RP, bool OUT_OPS>
__global__ void __launch_bounds__(kThreads)
lr_aq_kernel(const uint16_t *__restrict__ A, int64_t m, int64_t n, int r, uint8_t *__restrict__ ws,
             size_t layer_bytes, size_t off_qops, size_t off_out, int64_t mp, int64_t np, int blocks_per_mat)
{
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    const uint16_t *Ab = A + (int64_t)b * m * n;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const bf16x8 *qhi = (const bf16x8 *)(wsb + off_qops);
    const bf16x8 *qlo = qhi + (np / 8) * RP;

    __shared__ bf16x8 sq[2][8][RP];
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    const int64_t row = (int64_t)blk * kAqRows + wave * 16 + li;
    const bool row_ok = row < m;
    const uint16_t *arow = Ab + (row_ok ? row : 0) * n;

    constexpr int QE = 2 * 8 * RP;                 // 16-byte entries of one Q tile
    constexpr int QPT = (QE + kThreads - 1) / kThreads;

    auto load_a = [&](int64_t k0, bf16x8 &a0, bf16x8 &a1) {
        const int64_t c0 = k0 + 8 * g, c1 = k0 + 32 + 8 * g;
        a0 = (row_ok && c0 < n) ? __builtin_nontemporal_load((const bf16x8 *)(arow + c0)) : bf16x8{};
        a1 = (row_ok && c1 < n) ? __builtin_nontemporal_load((const bf16x8 *)(arow + c1)) : bf16x8{};
    };
    auto load_q = [&](int64_t k0, bf16x8 *qv) {
#pragma unroll
        for (int p = 0; p < QPT; ++p) {
            const int e = threadIdx.x + p * kThreads;
            if (e < QE) {
                const int hl = e / (8 * RP), rem = e % (8 * RP), kb = rem / RP, c = rem % RP;
                qv[p] = (hl ? qlo : qhi)[(k0 / 8 + kb) * RP + c];
            }
        }
    };

    f32x4 acc[RP / 16];
#pragma unroll
    for (int j = 0; j < RP / 16; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    bf16x8 a0, a1, qv[QPT];
    load_a(0, a0, a1);
    load_q(0, qv);
    for (int64_t k0 = 0; k0 < n; k0 += 64) {
        __syncthreads();  // previous tile's readers are done
#pragma unroll
        for (int p = 0; p < QPT; ++p) {
            const int e = threadIdx.x + p * kThreads;
            if (e < QE)
                (&sq[0][0][0])[e] = qv[p];
        }
        __syncthreads();
        const bf16x8 c0 = a0, c1 = a1;
        if (k0 + 64 < n) {  // prefetch the next tile while this one is multiplied
            load_a(k0 + 64, a0, a1);
            load_q(k0 + 64, qv);
        }
#pragma unroll
        for (int jt = 0; jt < RP / 16; ++jt) {
            acc[jt] = mfma(c0, sq[0][g][jt * 16 + li], acc[jt]);
            acc[jt] = mfma(c0, sq[1][g][jt * 16 + li], acc[jt]);
            acc[jt] = mfma(c1, sq[0][4 + g][jt * 16 + li], acc[jt]);
            acc[jt] = mfma(c1, sq[1][4 + g][jt * 16 + li], acc[jt]);
        }
    }

    // D layout: lane holds rows 4g..4g+3 of the 16-row tile, column li
    const int64_t i0 = (int64_t)blk * kAqRows + wave * 16 + 4 * g;
    if constexpr (OUT_OPS) {
        bf16x4 *yhi = (bf16x4 *)(wsb + off_out);
        bf16x4 *ylo = yhi + (mp / 8) * RP * 2;  // bf16x4 units: plane = mp/8 * RP * 8 bf16
        if (i0 < mp) {
#pragma unroll
            for (int jt = 0; jt < RP / 16; ++jt) {
                bf16x4 h, l;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float y = acc[jt][v];
                    h[v] = (__bf16)y;
                    l[v] = (__bf16)(y - (float)h[v]);
                }
                const int64_t idx = ((i0 / 8) * RP + jt * 16 + li) * 2 + ((i0 % 8) / 4);
                yhi[idx] = h;
                ylo[idx] = l;
            }
        }
    } else {
        float *out = (float *)(wsb + off_out);
#pragma unroll
        for (int jt = 0; jt < RP / 16; ++jt) {
            const int c = jt * 16 + li;
#pragma unroll
            for (int v = 0; v < 4; ++v)
                if (i0 + v < m && c < r)
                    out[(i0 + v) * r + c] = acc[jt][v];
        }
    }
}

// ------------------------------------------------------------------ Z = A^T Y

// One work-group: 64 columns of A (wave w owns columns 16w..16w+15) against all
// rows.  Each 32-row slab of A is loaded with coalesced 16-byte loads and stored
// transposed in LDS, so that a lane's MFMA operand (8 consecutive rows of one
// column) is one 16-byte LDS read.
template <int RP>
__global__ void __launch_bounds__(kThreads)
lr_aty_kernel(const uint16_t *__restrict__ A, int64_t m, int64_t n, int r, uint8_t *__restrict__ ws,
              size_t layer_bytes, size_t off_yops, size_t off_out, int64_t mp, int blocks_per_mat)
{
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    const uint16_t *Ab = A + (int64_t)b * m * n;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const bf16x8 *yhi = (const bf16x8 *)(wsb + off_yops);
    const bf16x8 *ylo = yhi + (mp / 8) * RP;

    constexpr int SROW = 32 + 8;                  // padded row of the transposed tile (80 B)
    __shared__ __attribute__((aligned(16))) uint16_t sa[kAtyCols][SROW];
    __shared__ bf16x8 sy[2][4][RP];

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    // loader role: thread t loads row t/8 of the slab, columns 8*(t%8) .. +7
    const int trow = threadIdx.x / 8, tcc = threadIdx.x % 8;
    const int64_t tcol = (int64_t)blk * kAtyCols + 8 * tcc;
    constexpr int YE = 2 * 4 * RP;

    auto load_a = [&](int64_t i0) -> u32x4 {
        const int64_t i = i0 + trow;
        return (i < m && tcol < n) ? __builtin_nontemporal_load((const u32x4 *)(Ab + i * n + tcol))
                                   : u32x4{0, 0, 0, 0};
    };
    auto load_y = [&](int64_t i0) -> bf16x8 {
        const int e = threadIdx.x;
        if (e >= YE)
            return bf16x8{};
        const int hl = e / (4 * RP), rem = e % (4 * RP), kb = rem / RP, c = rem % RP;
        return (hl ? ylo : yhi)[(i0 / 8 + kb) * RP + c];
    };

    f32x4 acc[RP / 16];
#pragma unroll
    for (int j = 0; j < RP / 16; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};

    u32x4 av = load_a(0);
    bf16x8 yv = load_y(0);
    for (int64_t i0 = 0; i0 < m; i0 += 32) {
        __syncthreads();
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const uint32_t w = av[s >> 1];
            sa[8 * tcc + s][trow] = (uint16_t)((s & 1) ? (w >> 16) : (w & 0xffffu));
        }
        if (threadIdx.x < YE)
            (&sy[0][0][0])[threadIdx.x] = yv;
        __syncthreads();
        if (i0 + 32 < m) {
            av = load_a(i0 + 32);
            yv = load_y(i0 + 32);
        }
        const bf16x8 aop = *(const bf16x8 *)&sa[wave * 16 + li][8 * g];
#pragma unroll
        for (int jt = 0; jt < RP / 16; ++jt) {
            acc[jt] = mfma(aop, sy[0][g][jt * 16 + li], acc[jt]);
            acc[jt] = mfma(aop, sy[1][g][jt * 16 + li], acc[jt]);
        }
    }

    float *out = (float *)(wsb + off_out);
    const int64_t j0 = (int64_t)blk * kAtyCols + wave * 16 + 4 * g;
#pragma unroll
    for (int jt = 0; jt < RP / 16; ++jt) {
        const int c = jt * 16 + li;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            if (j0 + v < n && c < r)
                out[(j0 + v) * r + c] = acc[jt][v];
    }
}

// ------------------------------------------------------------------ Gram partials

// Partial G = M'^T M' over kGramRows rows, in fp64, where M' = M (fp32 [L][r]) or,
// with `rinv` given, M' = M Rinv (Rinv upper triangular fp64 [RP][RP]).
template <int RP>
__global__ void __launch_bounds__(kThreads)
lr_gram_kernel(const float *__restrict__ M, int64_t m_stride, int64_t L, int r,
               uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_rinv, bool transform,
               size_t off_gram, int blocks_per_mat)
{
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    const float *Mb = M + (int64_t)b * m_stride;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;

    __shared__ double srow[kGramRows][RP + 1];
    __shared__ double sR[RP][RP];
    constexpr int NB = (RP / 4) * (RP / 4);  // 4x4 blocks of G
    constexpr int RG = kThreads / NB;        // row groups
    __shared__ double sacc[RG][RP * RP];

    // stage the rows as fp64 (zero beyond L and beyond r)
    for (int e = threadIdx.x; e < kGramRows * RP; e += kThreads) {
        const int rr = e / RP, c = e % RP;
        const int64_t row = (int64_t)blk * kGramRows + rr;
        srow[rr][c] = (row < L && c < r) ? (double)Mb[row * r + c] : 0.0;
    }
    if (transform) {
        const double *rinv = (const double *)(wsb + off_rinv);
        for (int e = threadIdx.x; e < RP * RP; e += kThreads)
            (&sR[0][0])[e] = rinv[e];
        __syncthreads();
        // TPR threads per row, each producing RP / TPR entries of the transformed row
        constexpr int TPR = kThreads / kGramRows, PER = RP / TPR;
        const int rr = threadIdx.x / TPR, part = threadIdx.x % TPR;
        double outv[PER];
#pragma unroll
        for (int cc = 0; cc < PER; ++cc) {
            const int c = part * PER + cc;
            double s = 0.0;
            for (int k = 0; k <= c; ++k)
                s = fma(srow[rr][k], sR[k][c], s);
            outv[cc] = s;
        }
        __syncthreads();
#pragma unroll
        for (int cc = 0; cc < PER; ++cc)
            srow[rr][part * PER + cc] = outv[cc];
    }
    __syncthreads();

    const int pb = threadIdx.x % NB, rg = threadIdx.x / NB;
    const int bi = pb / (RP / 4), bj = pb % (RP / 4);
    double acc[4][4] = {};
    for (int rr = rg; rr < kGramRows; rr += RG) {
        double xi[4], xj[4];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
            xi[a] = srow[rr][4 * bi + a];
            xj[a] = srow[rr][4 * bj + a];
        }
#pragma unroll
        for (int a = 0; a < 4; ++a)
#pragma unroll
            for (int c = 0; c < 4; ++c)
                acc[a][c] = fma(xi[a], xj[c], acc[a][c]);
    }
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int c = 0; c < 4; ++c)
            sacc[rg][(4 * bi + a) * RP + 4 * bj + c] = acc[a][c];
    __syncthreads();
    double *part = (double *)(wsb + off_gram) + (size_t)blk * RP * RP;
    for (int e = threadIdx.x; e < RP * RP; e += kThreads) {
        double s = 0.0;
        for (int q = 0; q < RG; ++q)
            s += sacc[q][e];
        part[e] = s;
    }
}

// ------------------------------------------------------------------ Cholesky + inverse

// One work-group per matrix.  Sums the Gram partials in a fixed order, factors
// G = R^T R (R upper, positive diagonal) in fp64, inverts R.
// pass 1: store R1 and R1^-1.  pass 2: R = R2 R1, store (R1^-1 R2^-1); write R
// as fp32 [r][r] into ru_out when it is given.
template <int RP>
__global__ void __launch_bounds__(kThreads)
lr_chol_kernel(uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_gram, int gram_blocks,
               int r, int pass, size_t off_r1, size_t off_r1inv, size_t off_rinv,
               float *__restrict__ ru_out)
{
    const int b = blockIdx.x;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    __shared__ double G[RP][RP], R[RP][RP], X[RP][RP], W[RP][RP];
    __shared__ int dead[RP];
    __shared__ double tol;
    const int t = threadIdx.x;

    const double *part = (const double *)(wsb + off_gram);
    for (int e = t; e < RP * RP; e += kThreads) {
        double s = 0.0;
        for (int q = 0; q < gram_blocks; ++q)
            s += part[(size_t)q * RP * RP + e];
        (&G[0][0])[e] = s;
        (&R[0][0])[e] = 0.0;
        (&X[0][0])[e] = 0.0;
    }
    __syncthreads();
    if (t == 0) {
        double tr = 0.0;
        for (int k = 0; k < r; ++k)
            tr += G[k][k];
        tol = 1e-13 * tr / r;
    }
    __syncthreads();

    // right-looking Cholesky on the upper triangle
    for (int k = 0; k < r; ++k) {
        if (t == 0) {
            const double d = G[k][k];
            const bool bad = !(d > tol) || !isfinite(d);
            dead[k] = bad;
            R[k][k] = bad ? 0.0 : sqrt(d);
        }
        __syncthreads();
        if (t > k && t < r)
            R[k][t] = dead[k] ? 0.0 : G[k][t] / R[k][k];
        __syncthreads();
        for (int e = t; e < RP * RP; e += kThreads) {
            const int i = e / RP, j = e % RP;
            if (i > k && j >= i && j < r)
                G[i][j] -= R[k][i] * R[k][j];
        }
        __syncthreads();
    }
    // a dropped column has a zero R column as well
    for (int e = t; e < RP * RP; e += kThreads) {
        const int i = e / RP, j = e % RP;
        if (j < r && dead[j])
            R[i][j] = 0.0;
    }
    __syncthreads();
    // X = R^-1 by back substitution, one column per thread
    if (t < r && !dead[t]) {
        const int c = t;
        X[c][c] = 1.0 / R[c][c];
        for (int i = c - 1; i >= 0; --i) {
            if (dead[i])
                continue;
            double s = 0.0;
            for (int k = i + 1; k <= c; ++k)
                s += R[i][k] * X[k][c];
            X[i][c] = -s / R[i][i];
        }
    }
    __syncthreads();

    double *r1 = (double *)(wsb + off_r1), *r1inv = (double *)(wsb + off_r1inv);
    double *rinv = (double *)(wsb + off_rinv);
    if (pass == 1) {
        for (int e = t; e < RP * RP; e += kThreads) {
            r1[e] = (&R[0][0])[e];
            r1inv[e] = (&X[0][0])[e];
        }
        return;
    }
    // pass 2: combined factor R2 R1 and inverse R1^-1 R2^-1 (both upper triangular)
    for (int e = t; e < RP * RP; e += kThreads) {
        const int i = e / RP, j = e % RP;
        double s = 0.0, si = 0.0;
        for (int k = i; k <= j; ++k) {
            s += R[i][k] * r1[k * RP + j];
            si += r1inv[i * RP + k] * X[k][j];
        }
        W[i][j] = (j >= i) ? s : 0.0;
        rinv[e] = (j >= i) ? si : 0.0;
    }
    __syncthreads();
    if (ru_out) {
        float *ru = ru_out + (size_t)b * r * r;
        for (int e = t; e < r * r; e += kThreads)
            ru[e] = (float)W[e / r][e % r];
    }
}

// ------------------------------------------------------------------ apply M Rinv

// Q = M Rinv row by row (fp64 arithmetic).  Writes Q as fp32 [L][r] into `out`
// when given, and the operand layout (hi/lo, rows up to Lp, zero beyond L and
// beyond r) at off_ops when ops is set.
template <int RP>
__global__ void __launch_bounds__(kThreads)
lr_apply_kernel(const float *__restrict__ M, int64_t m_stride, int64_t L, int64_t Lp, int r,
                uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_rinv, bool ops,
                size_t off_ops, float *__restrict__ out, int64_t out_stride, int blocks_per_mat)
{
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    const float *Mb = M + (int64_t)b * m_stride;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    __shared__ double sR[RP][RP];
    const double *rinv = (const double *)(wsb + off_rinv);
    for (int e = threadIdx.x; e < RP * RP; e += kThreads)
        (&sR[0][0])[e] = rinv[e];
    __syncthreads();

    const int64_t row = (int64_t)blk * kApplyRows + threadIdx.x;
    if (row >= Lp)
        return;
    const bool live = row < L;
    float in[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k)
        in[k] = (live && k < r) ? Mb[row * r + k] : 0.0f;
    float q[RP];
#pragma unroll
    for (int c = 0; c < RP; ++c) {
        double s = 0.0;
#pragma unroll
        for (int k = 0; k <= c; ++k)
            s = fma((double)in[k], sR[k][c], s);
        q[c] = (c < r) ? (float)s : 0.0f;
    }
    if (out && live) {
        float *ob = out + (int64_t)b * out_stride + row * r;
        for (int c = 0; c < r; ++c)
            ob[c] = q[c];
    }
    if (ops) {
        __bf16 *hi = (__bf16 *)(wsb + off_ops);
        __bf16 *lo = hi + Lp * RP;
        const int64_t base = (row / 8) * RP * 8 + (row % 8);
#pragma unroll
        for (int c = 0; c < RP; ++c) {
            const __bf16 h = (__bf16)q[c];
            hi[base + c * 8] = h;
            lo[base + c * 8] = (__bf16)(q[c] - (float)h);
        }
    }
}

// ------------------------------------------------------------------ host orchestration

template <int RP>
hipError_t run_orth(const Layout &Ly, int64_t batch, const float *M, int64_t m_stride, int64_t L,
                    int r, uint8_t *ws, float *out, int64_t out_stride, bool ops, float *ru,
                    hipStream_t st)
{
    const int gblocks = (int)((L + kGramRows - 1) / kGramRows);
    const int Lp_ops = (int)round_up(L, 64);
    const int ablocks = (Lp_ops + kApplyRows - 1) / kApplyRows;
    const unsigned ggrid = (unsigned)(gblocks * batch), agrid = (unsigned)(ablocks * batch);
    hipLaunchKernelGGL((lr_gram_kernel<RP>), dim3(ggrid), dim3(kThreads), 0, st, M, m_stride, L,
                       r, ws, Ly.layer_bytes, Ly.off_r1inv, false, Ly.off_gram, gblocks);
    hipLaunchKernelGGL((lr_chol_kernel<RP>), dim3((unsigned)batch), dim3(kThreads), 0, st, ws,
                       Ly.layer_bytes, Ly.off_gram, gblocks, r, 1, Ly.off_r1, Ly.off_r1inv,
                       Ly.off_rinv, (float *)nullptr);
    hipLaunchKernelGGL((lr_gram_kernel<RP>), dim3(ggrid), dim3(kThreads), 0, st, M, m_stride, L,
                       r, ws, Ly.layer_bytes, Ly.off_r1inv, true, Ly.off_gram, gblocks);
    hipLaunchKernelGGL((lr_chol_kernel<RP>), dim3((unsigned)batch), dim3(kThreads), 0, st, ws,
                       Ly.layer_bytes, Ly.off_gram, gblocks, r, 2, Ly.off_r1, Ly.off_r1inv,
                       Ly.off_rinv, ru);
    hipLaunchKernelGGL((lr_apply_kernel<RP>), dim3(agrid), dim3(kThreads), 0, st, M, m_stride, L,
                       (int64_t)Lp_ops, r, ws, Ly.layer_bytes, Ly.off_rinv, ops, Ly.off_qops, out,
                       out_stride, ablocks);
    return hipGetLastError();
}

template <int RP>
hipError_t run_lowrank(const LowrankArgs &a, hipStream_t st)
{
    const Layout Ly = make_layout(a.m, a.n, a.r);
    uint8_t *ws = (uint8_t *)a.ws;
    const float *mf = (const float *)(ws + Ly.off_mf);
    const int64_t mf_stride = (int64_t)(Ly.layer_bytes / 4);
    hipError_t e;
    const int aq_blocks = (int)(Ly.mp / kAqRows);
    const int aty_blocks = (int)((a.n + kAtyCols - 1) / kAtyCols);

    // step 1: orthonormalise the random sample
    if ((e = run_orth<RP>(Ly, a.batch, a.Q0, a.n * a.r, a.n, a.r, ws, a.V, a.n * a.r, true,
                          nullptr, st)) != hipSuccess)
        return e;
    for (int t = 0; t < a.T; ++t) {
        hipLaunchKernelGGL((lr_aq_kernel<RP, true>), dim3((unsigned)(aq_blocks * a.batch)),
                           dim3(kThreads), 0, st, a.A, a.m, a.n, a.r, ws, Ly.layer_bytes,
                           Ly.off_qops, Ly.off_yops, Ly.mp, Ly.np, aq_blocks);
        hipLaunchKernelGGL((lr_aty_kernel<RP>), dim3((unsigned)(aty_blocks * a.batch)),
                           dim3(kThreads), 0, st, a.A, a.m, a.n, a.r, ws, Ly.layer_bytes,
                           Ly.off_yops, Ly.off_mf, Ly.mp, aty_blocks);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        if ((e = run_orth<RP>(Ly, a.batch, mf, mf_stride, a.n, a.r, ws, a.V, a.n * a.r, true,
                              nullptr, st)) != hipSuccess)
            return e;
    }
    // final: P = A Q, (U, R_U) = orth(P), V = Q (already written)
    hipLaunchKernelGGL((lr_aq_kernel<RP, false>), dim3((unsigned)(aq_blocks * a.batch)),
                       dim3(kThreads), 0, st, a.A, a.m, a.n, a.r, ws, Ly.layer_bytes, Ly.off_qops,
                       Ly.off_mf, Ly.mp, Ly.np, aq_blocks);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    return run_orth<RP>(Ly, a.batch, mf, mf_stride, a.m, a.r, ws, a.U, a.m * a.r, false, a.RU,
                        st);
}

}  // namespace

size_t lowrank_workspace_bytes(int64_t batch, int64_t m, int64_t n, int r)
{
    return make_layout(m, n, r).layer_bytes * (size_t)batch;
}

hipError_t launch_lowrank(const LowrankArgs &a, hipStream_t st)
{
    if (a.batch == 0)
        return hipSuccess;
    return a.r <= 16 ? run_lowrank<16>(a, st) : run_lowrank<32>(a, st);
}

}  // namespace cfz
