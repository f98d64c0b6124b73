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
// product carries about 16 bits of the skinny operand instead of 8.  For
// r <= 16 and n <= 3072, Y = A Q and Z = A^T Y run as one pass over A
// (lr_ata_kernel, lr_ata8_kernel for r <= 8); otherwise as two (lr_aq_kernel,
// lr_aty_kernel).  With T >= 1 the sample Q0 enters the first product as it is
// (see run_lowrank); at r <= 8 the first one-pass product also splits it into
// its hi / lo operands itself.
//
// orth() is Cholesky-QR: Gram matrix G = M^T M accumulated in fp64 from fp32
// rows, r x r Cholesky and triangular inverse in fp64, then M R^-1 row by row.
// A second pass (CholQR2) runs for a matrix only when the first cannot deliver
// fp32 orthogonality: its loss of orthogonality is about kappa(M)^2 u_fp64, so
// the second pass is taken when the estimate ||R1||_F ||R1^-1||_F >= kappa(M)
// exceeds 2^14.5 (kappa^2 u_fp64 > u_fp32).  For r <= 16 this is two launches
// (Gram partials, then factorisations and apply in lr_cholapply_kernel; for P
// the final A Q leaves the Gram partials, so one); for r > 16 five, the second
// pass's two leaving at once for the matrices that do not need it.  A pivot
// <= 1e-13 * trace(G) / r (or not finite) drops the column: zero Q column, zero
// R row and column.
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
constexpr int kGramRows = 256;    // rows of M per Gram work-group (64 per wave)
constexpr int kApplyRows = 256;   // rows of M per apply work-group (64 per wave)
constexpr int kCholThreads = 64;  // the r x r factorisation runs on one wavefront
constexpr int kMaxPartials = 8;   // partial sums of Z the Gram kernel adds up
constexpr int kGramHalf = 2;      // 16-row tiles per wave whose loads are in flight together
// Second Cholesky-QR pass when ||R1||_F^2 ||R1^-1||_F^2 exceeds 2^29: the first
// pass's loss of orthogonality, about kappa^2 u_fp64 = kappa^2 2^-53, could then
// exceed the fp32 output's own rounding, 2^-24.
constexpr double kTwoPassKappa2 = 536870912.0;  // 2^29

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

// ------------------------------------------------------------------ fp64 MFMA helpers

typedef double f64x4 __attribute__((ext_vector_type(4)));

// v_mfma_f64_16x16x4_f64: A[i][k] at lane i + 16 k, B[k][j] at lane j + 16 k,
// D[i][j] at lane j + 16 (i % 4), item i / 4.
__device__ __forceinline__ f64x4 mfma64(double a, double b, f64x4 c)
{
    return __builtin_amdgcn_mfma_f64_16x16x4f64(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ double readlane_f64(double v, int l)
{
    const uint64_t u = __builtin_bit_cast(uint64_t, v);
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)u, l);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(u >> 32), l);
    return __builtin_bit_cast(double, ((uint64_t)hi << 32) | lo);
}

// ------------------------------------------------------------------ workspace layout

struct Layout {
    int rp;
    int64_t mp, np;             // m, n padded to 64
    int64_t gram_blocks;        // max over (m, n) of row blocks of the Gram kernel
    int splits;                 // row ranges of the one-pass A^T (A Q); 0: two passes
    int64_t split_rows;         // rows per range, a multiple of the 16-row panel
    size_t off_qops, off_yops, off_mf, off_gram, off_r1, off_r1inv, off_rinv, off_flag;
    size_t layer_bytes;
};

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

constexpr int64_t kComputeUnits = 256;  // MI355X

// Row ranges per matrix for the one-pass A^T (A Q) (declared with its kernel
// below): about one 1024-thread work-group per compute unit over the batch, at
// most kAtaMaxSplits partial sums per matrix.  0 where the pass does not apply
// (r > 16 or n > 3072): then A Q and A^T Y run as two passes.
int ata_splits(int64_t batch, int64_t m, int64_t n, int r);

Layout make_layout(int64_t batch, int64_t m, int64_t n, int r)
{
    Layout L;
    L.rp = r <= 16 ? 16 : 32;
    L.mp = round_up(m, 128);
    L.np = round_up(n, 64);
    const int64_t lmax = m > n ? m : n;
    L.gram_blocks = (lmax + kGramRows - 1) / kGramRows;
    L.splits = ata_splits(batch, m, n, r);
    L.split_rows = L.splits ? round_up((m + L.splits - 1) / L.splits, 16) : 0;
    if (L.gram_blocks < L.splits)  // the final A Q leaves one Gram partial per row range
        L.gram_blocks = L.splits;
    // Z or P in fp32 [L][r]; with the one-pass product, Z's partial sums side by side
    const int64_t mf_rows = L.splits * n > lmax ? L.splits * n : lmax;
    size_t off = 0;
    L.off_qops = off; off = align256(off + (size_t)L.np * L.rp * 2 * 2);
    L.off_yops = off; off = align256(off + (size_t)L.mp * L.rp * 2 * 2);
    L.off_mf = off;   off = align256(off + (size_t)mf_rows * r * 4);
    L.off_gram = off; off = align256(off + (size_t)L.gram_blocks * L.rp * L.rp * 8);
    L.off_r1 = off;   off = align256(off + (size_t)L.rp * L.rp * 8);
    L.off_r1inv = off; off = align256(off + (size_t)L.rp * L.rp * 8);
    L.off_rinv = off; off = align256(off + (size_t)L.rp * L.rp * 8);
    L.off_flag = off; off = align256(off + sizeof(int32_t));
    L.layer_bytes = off;
    return L;
}

// ------------------------------------------------------------------ buffer loads

// Raw buffer loads: the hardware returns zeros for offsets at or beyond
// num_records, so masked lanes and tiles past the end need no branch (which
// keeps the loads of the software pipelines below in flight across steps).
constexpr uint32_t kBufWord3 = 0x00020000u;  // gfx9 raw buffer: 32-bit data format
constexpr uint32_t kOOB = 0x80000000u;        // any offset >= num_records

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes)
{
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), 0, (int)bytes, kBufWord3);
}

__device__ __forceinline__ bf16x8 buf_load16(__amdgpu_buffer_rsrc_t rs, uint32_t off)
{
    return __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 2 /*nt*/));
}

// Rows 8 kb .. 8 kb + 7 of column c of an fp32 [L][r] matrix as one operand slot, split
// into bf16 hi (lo = false) or the bf16 rounding of what hi misses (lo = true); rows past
// L and columns past r are zeros.  The same values the operand-layout kernel stores.
__device__ __forceinline__ bf16x8 slot_from_f32(const float *M, int64_t L, int r, int64_t kb,
                                                int c, bool lo)
{
    bf16x8 o;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = 8 * kb + i;
        const float q = (row < L && c < r) ? M[row * r + c] : 0.0f;
        const __bf16 h = (__bf16)q;
        o[i] = lo ? (__bf16)(q - (float)h) : h;
    }
    return o;
}

// ------------------------------------------------------------------ Y = A Q

constexpr int kPipe = 4;                        // register stages of the A-streaming pipelines
constexpr int kAqTiles = 2;                     // 16-row MFMA tiles per wave
constexpr int kAqRows = 4 * 16 * kAqTiles;      // rows of A per work-group
static_assert(128 % kAqRows == 0, "A Q blocks must tile m padded to 128 (Layout::mp)");

// One work-group: kAqRows rows of A against all of Q, 64 columns of A per step.
// A is loaded 8 rows x 128 bytes per wave instruction (whole cache lines) and
// passed through a wave-private LDS tile into MFMA operand layout (16 rows x 8
// columns per lane group), which read straight from memory would split every
// instruction into 16 half lines.  Pipeline: A tiles kPipe steps ahead in
// statically named register stages, Q tiles one step ahead in registers and
// double-buffered in LDS, one work-group barrier per step.
// OUT_OPS: write Y in operand layout (hi/lo planes, rows up to mp, zero beyond
// m); otherwise write Y as fp32 [m][r].
template <int RP, bool OUT_OPS>
__global__ void __launch_bounds__(kThreads)
lr_aq_kernel(const uint16_t *__restrict__ A, int64_t m, int64_t n, int r, uint8_t *__restrict__ ws,
             size_t layer_bytes, size_t off_qops, size_t off_out, int64_t mp, int64_t np, int blocks_per_mat)
{
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const bf16x8 *qhi = (const bf16x8 *)(wsb + off_qops);
    const bf16x8 *qlo = qhi + (np / 8) * RP;

    __shared__ bf16x8 sq[2][2][8][RP];  // [buffer][hi, lo][k block][column]
    __shared__ bf16x8 sa[4][16 * kAqTiles][9];  // [wave][row][8 column chunks + pad]
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    const int64_t row0 = (int64_t)blk * kAqRows;
    // rows of A this work-group owns; 0 for a block wholly in the padding past m (its
    // loads then all return zeros: a negative count would make the buffer size wrap)
    const int64_t rows_here = m - row0 <= 0 ? 0 : (m - row0 < kAqRows ? m - row0 : kAqRows);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(A + (int64_t)b * m * n + row0 * n, (uint32_t)(rows_here * n * 2));

    constexpr int QE = 2 * 8 * RP;                 // 16-byte entries of one Q tile
    constexpr int QPT = (QE + kThreads - 1) / kThreads;
    const int64_t last_tile = np - 64;             // Q loads past the end re-read a valid tile

    // load instruction p: rows 8 p + lane / 8 of the wave's rows, column chunk lane % 8
    auto load_a = [&](int64_t k0, bf16x8 (&av)[kAqTiles][2]) {
#pragma unroll
        for (int p = 0; p < 2 * kAqTiles; ++p) {
            const int64_t rr = wave * 16 * kAqTiles + 8 * p + (lane >> 3);
            const int64_t col = k0 + 8 * (lane & 7);
            av[p / 2][p % 2] = buf_load16(
                ra, (rr < rows_here && col < n) ? (uint32_t)((rr * n + col) * 2) : kOOB);
        }
    };
    auto load_q = [&](int64_t k0, bf16x8 (&qv)[QPT]) {
        const int64_t kt = (k0 < last_tile ? k0 : last_tile) / 8;
#pragma unroll
        for (int p = 0; p < QPT; ++p) {
            const int e = threadIdx.x + p * kThreads;
            const int ee = e < QE ? e : 0;
            const int hl = ee / (8 * RP), rem = ee % (8 * RP), kb = rem / RP, c = rem % RP;
            qv[p] = (hl ? qlo : qhi)[(kt + kb) * RP + c];
        }
    };
    auto store_q = [&](int buf, const bf16x8 (&qv)[QPT]) {
#pragma unroll
        for (int p = 0; p < QPT; ++p) {
            const int e = threadIdx.x + p * kThreads;
            if (e < QE)
                (&sq[buf][0][0][0])[e] = qv[p];
        }
    };

    f32x4 acc[kAqTiles][RP / 16];
#pragma unroll
    for (int t = 0; t < kAqTiles; ++t)
#pragma unroll
        for (int j = 0; j < RP / 16; ++j)
            acc[t][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int buf, const bf16x8 (&ld)[kAqTiles][2]) {
        // the loaded rows into the wave's tile, then the operands out of it
#pragma unroll
        for (int p = 0; p < 2 * kAqTiles; ++p)
            sa[wave][8 * p + (lane >> 3)][lane & 7] = ld[p / 2][p % 2];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        bf16x8 av[kAqTiles][2];
#pragma unroll
        for (int t = 0; t < kAqTiles; ++t) {
            av[t][0] = sa[wave][16 * t + li][g];
            av[t][1] = sa[wave][16 * t + li][4 + g];
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll
        for (int t = 0; t < kAqTiles; ++t)
#pragma unroll
            for (int jt = 0; jt < RP / 16; ++jt) {
                acc[t][jt] = mfma(av[t][0], sq[buf][0][g][jt * 16 + li], acc[t][jt]);
                acc[t][jt] = mfma(av[t][0], sq[buf][1][g][jt * 16 + li], acc[t][jt]);
                acc[t][jt] = mfma(av[t][1], sq[buf][0][4 + g][jt * 16 + li], acc[t][jt]);
                acc[t][jt] = mfma(av[t][1], sq[buf][1][4 + g][jt * 16 + li], acc[t][jt]);
            }
    };

    // Step i multiplies tile i (A stage i % S, LDS buffer i % 2), refills that A
    // stage with tile i + S, stages Q tile i + 1 into the other LDS buffer and
    // refills its Q stage with tile i + 1 + S.  What a step waits for was issued
    // S - 1 steps earlier, so the in-order load counter keeps the loads of the
    // last S - 1 steps in flight.  The loop is unrolled by S so that every stage
    // is a fixed set of registers.
    constexpr int S = kPipe;
    bf16x8 a[S][kAqTiles][2], q[S][QPT];
#pragma unroll
    for (int j = 0; j < S; ++j) {
        load_q(64 * j, q[j]);
        load_a(64 * j, a[j]);
    }
    store_q(0, q[0]);
    load_q(64 * S, q[0]);
    __syncthreads();
    for (int64_t k0 = 0; k0 < n; k0 += 64 * S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            compute(j % 2, a[j]);  // zeros past the end of A
            load_a(k0 + 64 * (j + S), a[j]);
            store_q((j + 1) % 2, q[(j + 1) % S]);
            load_q(k0 + 64 * (j + 1 + S), q[(j + 1) % S]);
            __syncthreads();
        }
    }

    // D layout: lane holds rows 4g..4g+3 of each 16-row tile, column li
#pragma unroll
    for (int t = 0; t < kAqTiles; ++t) {
        const int64_t i0 = row0 + wave * 16 * kAqTiles + t * 16 + 4 * g;
        if constexpr (OUT_OPS) {
            bf16x4 *yhi = (bf16x4 *)(wsb + off_out);
            bf16x4 *ylo = yhi + (mp / 8) * RP * 2;  // bf16x4 units: plane = mp/8 * RP * 8 bf16
            if (i0 < mp) {
#pragma unroll
                for (int jt = 0; jt < RP / 16; ++jt) {
                    bf16x4 h, l;
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float y = acc[t][jt][v];
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
                        out[(i0 + v) * r + c] = acc[t][jt][v];
            }
        }
    }
}

// ------------------------------------------------------------------ Z = A^T Y

constexpr int kAtyWaves = 8;                 // waves per work-group, 16 columns each
constexpr int kAtyThreads = 64 * kAtyWaves;
constexpr int kAtyCols = 16 * kAtyWaves;     // columns of A per work-group

constexpr int kAtyRows = 64;  // rows of A per pipeline step (two 32-row MFMA k steps)

typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));

// ds_read_b64_tr_b16: within each group of 16 lanes, lane j receives element
// j % 4 of the 4-element chunks addressed by lanes j / 4, 4 + j / 4, 8 + j / 4
// and 12 + j / 4 (measured on gfx950).  So if lane i of a group addresses row
// base + i / 4, columns c0 + 4 (i % 4) .. + 3 of a row-major slab, lane j gets
// rows base .. base + 3 of column c0 + j: half an MFMA operand.
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t *p)
{
    return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
        (__attribute__((address_space(3))) i16x4 *)(p));
}

// One work-group: kAtyCols = 128 columns of A (wave w owns columns 16w..16w+15)
// against all rows; each row of a slab is then one 256-byte piece (64-column
// work-groups, reading 128-byte pieces 6 KB apart, took 2-4% longer per call).
// Each 64-row slab of A is loaded with coalesced 16-byte loads, stored in
// LDS as it is (one 16-byte store per load) and read back with the transposing
// LDS load, so that a lane's MFMA operand (8 consecutive rows of one column) is
// two 8-byte reads.  Same pipeline as A Q: slabs kPipe steps ahead in static
// register stages, Y tiles one step ahead, double-buffered LDS.
template <int RP>
__global__ void __launch_bounds__(kAtyThreads)
lr_aty_kernel(const uint16_t *__restrict__ A, int64_t m, int64_t n, int r, uint8_t *__restrict__ ws,
              size_t layer_bytes, size_t off_yops, size_t off_out, int64_t mp, int blocks_per_mat)
{
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const bf16x8 *yhi = (const bf16x8 *)(wsb + off_yops);
    const bf16x8 *ylo = yhi + (mp / 8) * RP;
    const __amdgpu_buffer_rsrc_t ra = make_rsrc(A + (int64_t)b * m * n, (uint32_t)(m * n * 2));

    constexpr int SCOL = kAtyCols + 8;             // padded slab row: rows 4 banks apart
    __shared__ __attribute__((aligned(16))) uint16_t sa[2][kAtyRows][SCOL];
    __shared__ bf16x8 sy[2][2][kAtyRows / 8][RP];  // [buffer][hi, lo][k block][column]

    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    // loader role: thread t loads rows t/C and t/C + 32 of the slab, columns 8*(t%C) .. +7
    // (C = kAtyCols / 8 chunks of 16 bytes per slab row)
    constexpr int C = kAtyCols / 8;
    static_assert(kAtyThreads / C == 32, "two loads per thread cover the 64-row slab");
    const int trow = threadIdx.x / C, tcc = threadIdx.x % C;
    const int64_t tcol = (int64_t)blk * kAtyCols + 8 * tcc;
    constexpr int YE = 2 * (kAtyRows / 8) * RP;
    constexpr int YPT = (YE + kAtyThreads - 1) / kAtyThreads;
    const int64_t last_slab = mp - kAtyRows;       // Y loads past the end re-read a valid slab

    auto load_a = [&](int64_t i0, u32x4 (&av)[2]) {
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t i = i0 + trow + 32 * h;
            const uint32_t off = (i < m && tcol < n) ? (uint32_t)((i * n + tcol) * 2) : kOOB;
            av[h] = __builtin_amdgcn_raw_buffer_load_b128(ra, off, 0, 2 /*nt*/);
        }
    };
    auto load_y = [&](int64_t i0, bf16x8 (&yv)[YPT]) {
        const int64_t kt = (i0 < last_slab ? i0 : last_slab) / 8;
#pragma unroll
        for (int p = 0; p < YPT; ++p) {
            const int e = threadIdx.x + p * kAtyThreads;
            const int ee = e < YE ? e : 0;
            const int hl = ee / ((kAtyRows / 8) * RP), rem = ee % ((kAtyRows / 8) * RP);
            const int kb = rem / RP, c = rem % RP;
            yv[p] = (hl ? ylo : yhi)[(kt + kb) * RP + c];
        }
    };
    auto store = [&](int buf, const u32x4 (&av)[2], const bf16x8 (&yv)[YPT]) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *(u32x4 *)&sa[buf][trow + 32 * h][8 * tcc] = av[h];
#pragma unroll
        for (int p = 0; p < YPT; ++p) {
            const int e = threadIdx.x + p * kAtyThreads;
            if (e < YE)
                (&sy[buf][0][0][0])[e] = yv[p];
        }
    };

    f32x4 acc[RP / 16];
#pragma unroll
    for (int j = 0; j < RP / 16; ++j)
        acc[j] = f32x4{0.f, 0.f, 0.f, 0.f};
    auto compute = [&](int buf) {
#pragma unroll
        for (int ks = 0; ks < kAtyRows / 32; ++ks) {
            // rows 32 ks + 8 g .. + 7 of column 16 wave + li
            const uint16_t *p = &sa[buf][32 * ks + 8 * g + (li >> 2)][wave * 16 + 4 * (li & 3)];
            const i16x4 lo = lds_read_tr16(p), hi = lds_read_tr16(p + 4 * SCOL);
            const i16x8 both = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            const bf16x8 aop = __builtin_bit_cast(bf16x8, both);
#pragma unroll
            for (int jt = 0; jt < RP / 16; ++jt) {
                acc[jt] = mfma(aop, sy[buf][0][4 * ks + g][jt * 16 + li], acc[jt]);
                acc[jt] = mfma(aop, sy[buf][1][4 * ks + g][jt * 16 + li], acc[jt]);
            }
        }
    };

    // Step i multiplies slab i from LDS buffer i % 2, then stages slab i + 1
    // (issued S - 1 steps earlier) into the other buffer and refills that
    // register stage with slab i + 1 + S; unrolled by S as in A Q.
    constexpr int S = kPipe;
    u32x4 a[S][2];
    bf16x8 y[S][YPT];
#pragma unroll
    for (int j = 0; j < S; ++j) {
        load_a(kAtyRows * j, a[j]);
        load_y(kAtyRows * j, y[j]);
    }
    store(0, a[0], y[0]);
    load_a(kAtyRows * S, a[0]);
    load_y(kAtyRows * S, y[0]);
    __syncthreads();
    for (int64_t i0 = 0; i0 < m; i0 += kAtyRows * S) {
#pragma unroll
        for (int j = 0; j < S; ++j) {
            compute(j % 2);
            store((j + 1) % 2, a[(j + 1) % S], y[(j + 1) % S]);
            load_a(i0 + kAtyRows * (j + 1 + S), a[(j + 1) % S]);
            load_y(i0 + kAtyRows * (j + 1 + S), y[(j + 1) % S]);
            __syncthreads();
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

// ------------------------------------------------------------------ Z = A^T (A Q), one pass

// Step 3 of the iteration with each row panel of A read from HBM once.  A
// work-group owns a contiguous range of rows of one matrix (one of `splits`
// ranges) and walks it in 8-row panels; a panel (8 full rows, contiguous in
// memory) goes through LDS, where
//   phase 1: each wave multiplies the panel's columns of its own 32-column
//            blocks by Q (hi + lo) into a partial Y (8 rows in a 16-row MFMA
//            tile), and the 16 partials are summed in wave order and split
//            into bf16 hi + lo;
//   phase 2: each wave adds panel^T Y to its blocks' rows of Z, read back with
//            the transposing LDS load; hi and lo ride in one K = 16 MFMA
//            (k = 0..7 the panel's rows against Y hi, 8..15 against Y lo).
// Each wave holds its blocks' Q hi (24 registers; Q lo sits in wave-private
// LDS slots) and its rows of Z (48) for the whole kernel, so the only memory
// loads in the loop are the panels: every wave keeps its share of the next
// panel (3 x 16 bytes per lane) in flight from the moment the current one is
// in LDS.  Vector loads return in issue order, so any other load issued
// behind a panel would wait for it.  Z is written once per work-group as one
// fp32 [n][r] partial; the Gram kernel sums the `splits` partials in a fixed
// order.  RP = 16 only.
constexpr int kAtaWaves = 16;
constexpr int kAtaThreads = 64 * kAtaWaves;
constexpr int kAtaPanel = 8;                           // rows per panel
constexpr int kAtaMaxBlocks = 6;                       // 32-column blocks per wave
constexpr int64_t kAtaMaxN = (int64_t)kAtaWaves * kAtaMaxBlocks * 32;  // 3072
constexpr int kAtaChunks = (int)(kAtaMaxN / 8 / 128);  // 16-byte loads per lane: half a row per wave
constexpr int kAtaMaxSplits = 8;
// LDS row stride: the row padded to 128 columns plus 24, so that consecutive rows
// start 12 banks apart -- the rows of a phase 1 read and the 4 rows of a
// transposing read then touch distinct banks.
constexpr int kAtaSrowMax = (int)kAtaMaxN + 24;
static_assert(kAtaWaves == 2 * kAtaPanel && kAtaMaxN == 2 * 8 * 64 * kAtaChunks,
              "two waves load each panel row, kAtaChunks 16-byte loads per lane each");

typedef short i16x4k __attribute__((ext_vector_type(4)));

template <int RP>
__global__ void __launch_bounds__(kAtaThreads)
lr_ata_kernel(const uint16_t *__restrict__ A, int64_t m, int64_t n, int r, uint8_t *__restrict__ ws,
              size_t layer_bytes, size_t off_qops, size_t off_z, int64_t np, int splits,
              int64_t split_rows, const float *__restrict__ /* q0: the r <= 8 kernel's only */)
{
    static_assert(RP == 16, "the one-pass product keeps Z in registers only for RP = 16");
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / splits, s = lid % splits;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const bf16x8 *qhi = (const bf16x8 *)(wsb + off_qops);
    const bf16x8 *qlo = qhi + (np / 8) * RP;
    float *zpart = (float *)(wsb + off_z) + (size_t)s * n * r;

    const int64_t row0 = (int64_t)s * split_rows;
    const int64_t rows_here = m - row0 <= 0 ? 0 : (m - row0 < split_rows ? m - row0 : split_rows);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(A + (int64_t)b * m * n + row0 * n, (uint32_t)(rows_here * n * 2));

    __shared__ __attribute__((aligned(16))) uint16_t sp[kAtaPanel * kAtaSrowMax];
    __shared__ float sy[kAtaWaves][kAtaPanel * 16];
    __shared__ i16x4k syo[2][2][16];  // [hi, lo][rows 0..3, 4..7][column of Y]
    __shared__ bf16x8 sql[kAtaWaves][kAtaMaxBlocks][64];  // each wave's Q lo operands

    // the wave index in a scalar register, so that every per-wave offset below is too
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    const int nb = (int)((n + 31) / 32);                   // 32-column blocks
    const int nbw = (nb + kAtaWaves - 1) / kAtaWaves;      // blocks per wave (<= kAtaMaxBlocks)
    const int kb0 = wave * nbw;
    const int kbn = nb - kb0 < nbw ? nb - kb0 : nbw;       // this wave's blocks (may be <= 0)
    const int srow = (int)round_up(32 * nb, 128) + 24;
    const int cpr = (int)(n / 8);                          // 16-byte chunks per row
    const int prow = wave >> 1;                            // the panel row this wave loads
    const int chalf = (wave & 1) * (64 * kAtaChunks);      // and its first chunk

    auto load_panel = [&](int64_t p, u32x4 (&v)[kAtaChunks]) {
        const uint32_t base = (uint32_t)((p * kAtaPanel + prow) * n * 2);
#pragma unroll
        for (int k = 0; k < kAtaChunks; ++k) {
            const int cc = chalf + lane + 64 * k;
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(
                ra, cc < cpr ? base + (uint32_t)cc * 16 : kOOB, 0, 2 /*nt*/);
        }
    };
    auto store_panel = [&](const u32x4 (&v)[kAtaChunks]) {
#pragma unroll
        for (int k = 0; k < kAtaChunks; ++k) {
            const int cc = chalf + lane + 64 * k;
            if (cc < cpr)
                *(u32x4 *)&sp[prow * srow + 8 * cc] = v[k];
        }
    };

    u32x4 pf[kAtaChunks];
    load_panel(0, pf);

    // Q operands of this wave's blocks: slot (4 (kb0 + j) + g, li) of each plane; hi
    // in registers, lo in the wave's own LDS slots (read back only by the same lane)
    bf16x8 qh[kAtaMaxBlocks];
#pragma unroll
    for (int j = 0; j < kAtaMaxBlocks; ++j) {
        const int64_t slot = (int64_t)(4 * (kb0 + (j < kbn ? j : 0)) + g) * RP + li;
        qh[j] = j < kbn ? qhi[slot] : bf16x8{};
        sql[wave][j][lane] = j < kbn ? qlo[slot] : bf16x8{};
    }

    // columns n .. 32 nb - 1 of every panel row stay zero (phase 1 multiplies them)
    const int tailc = (32 * nb - (int)n) / 8;
    if ((int)threadIdx.x < kAtaPanel * tailc) {
        const int row = threadIdx.x / tailc, cc = threadIdx.x % tailc;
        *(u32x4 *)&sp[row * srow + (int)n + 8 * cc] = u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 zacc[kAtaMaxBlocks][2];
#pragma unroll
    for (int j = 0; j < kAtaMaxBlocks; ++j)
        zacc[j][0] = zacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t npanels = (rows_here + kAtaPanel - 1) / kAtaPanel;
    for (int64_t p = 0; p < npanels; ++p) {
        store_panel(pf);
        load_panel(p + 1, pf);  // past the last panel: all out of range, zeros, unused
        __syncthreads();        // the panel is in LDS (and the previous one fully used)

        // phase 1: this wave's share of Y = panel Q; lanes of tile rows 8..15 hold zeros
        f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kAtaMaxBlocks; ++j) {
            if (j < kbn) {
                const bf16x8 a = *(const bf16x8 *)&sp[(li & 7) * srow + 32 * (kb0 + j) + 8 * g];
                const bf16x8 az = li < kAtaPanel ? a : bf16x8{};
                y = mfma(az, qh[j], y);
                y = mfma(az, sql[wave][j][lane], y);
            }
        }
        // D layout: lane (li, g) holds rows 4g..4g+3 of column li; rows 0..7 are g < 2
        if (g < 2)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                sy[wave][(4 * g + v) * 16 + li] = y[v];
        __syncthreads();  // partial Y written
        if (threadIdx.x < kAtaPanel * 16) {
            const int e = threadIdx.x, row = e / 16, col = e % 16;
            float t = sy[0][e];
#pragma unroll
            for (int w = 1; w < kAtaWaves; ++w)
                t += sy[w][e];
            const __bf16 h = (__bf16)t, l = (__bf16)(t - (float)h);
            syo[0][row / 4][col][row % 4] = __builtin_bit_cast(short, h);
            syo[1][row / 4][col][row % 4] = __builtin_bit_cast(short, l);
        }
        __syncthreads();  // Y operand written

        // phase 2: Z rows of this wave's blocks += panel^T (Y hi, Y lo)
        const i16x4k bop = syo[g >> 1][g & 1][li];
#pragma unroll
        for (int j = 0; j < kAtaMaxBlocks; ++j) {
            if (j < kbn) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c0 = 32 * (kb0 + j) + 16 * h;
                    const i16x4 aop =
                        lds_read_tr16(&sp[(4 * (g & 1) + (li >> 2)) * srow + c0 + 4 * (li & 3)]);
                    zacc[j][h] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, bop, zacc[j][h],
                                                                           0, 0, 0);
                }
            }
        }
        __syncthreads();  // every wave is done with the panel and with Y
    }

    // D layout: lane (li, g) holds rows c0 + 4g .. + 3 of Z, column li
#pragma unroll
    for (int j = 0; j < kAtaMaxBlocks; ++j) {
        if (j < kbn) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t c0 = 32 * (kb0 + j) + 16 * h + 4 * g;
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    if (c0 + v < n && li < r)
                        zpart[(c0 + v) * r + li] = zacc[j][h][v];
            }
        }
    }
}

// The one-pass A^T (A Q) for r <= 8.  Only 8 of the 16 MFMA columns would carry
// data, so they carry Q hi (columns 0..7) and Q lo (8..15) at once: a lane
// of column li >= 8 loads column li - 8 of the lo plane.  Phase 1 then needs
// one MFMA per block, Q lo leaves LDS, and the panel can be 16 rows (one full
// row per wave to load, 6 x 16 bytes per lane in flight); phase 2 likewise
// carries Y hi and Y lo as columns 0..7 and 8..15 of one K = 16 MFMA.  The two
// halves of each product are added across lanes li and li + 8 (Y before the
// cross-wave sum, Z once at the end).  q0 non-null (the first iteration): the
// lanes split the fp32 sample into its hi and lo operands themselves, the values
// the operand-layout kernel would have stored, and that launch is skipped.
constexpr int kAta8Panel = 16;
static_assert(kAtaWaves == kAta8Panel && kAtaMaxN == 8 * 64 * 6,
              "each wave loads one full-width panel row in 6 16-byte loads per lane");

template <int RP>
__global__ void __launch_bounds__(kAtaThreads)
lr_ata8_kernel(const uint16_t *__restrict__ A, int64_t m, int64_t n, int r, uint8_t *__restrict__ ws,
               size_t layer_bytes, size_t off_qops, size_t off_z, int64_t np, int splits,
               int64_t split_rows, const float *__restrict__ q0)
{
    static_assert(RP == 16, "columns 0..7 and 8..15 of the padded width carry hi and lo");
    constexpr int kChunks = 6;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / splits, s = lid % splits;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const bf16x8 *qhi = (const bf16x8 *)(wsb + off_qops);
    const bf16x8 *qlo = qhi + (np / 8) * RP;
    float *zpart = (float *)(wsb + off_z) + (size_t)s * n * r;

    const int64_t row0 = (int64_t)s * split_rows;
    const int64_t rows_here = m - row0 <= 0 ? 0 : (m - row0 < split_rows ? m - row0 : split_rows);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(A + (int64_t)b * m * n + row0 * n, (uint32_t)(rows_here * n * 2));

    __shared__ __attribute__((aligned(16))) uint16_t sp[kAta8Panel * kAtaSrowMax];
    __shared__ float sy[kAtaWaves][kAta8Panel * 8];  // each wave's Y (hi + lo products added)
    __shared__ i16x4k syo[16][4];  // [column: Y hi 0..7, Y lo 8..15][rows 4g..4g+3]

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    const int nb = (int)((n + 31) / 32);
    const int nbw = (nb + kAtaWaves - 1) / kAtaWaves;
    const int kb0 = wave * nbw;
    const int kbn = nb - kb0 < nbw ? nb - kb0 : nbw;
    const int srow = (int)round_up(32 * nb, 128) + 24;
    const int cpr = (int)(n / 8);

    // wave w loads row w of a panel: chunk k of a lane is columns 8 (lane + 64 k) .. + 7
    auto load_panel = [&](int64_t p, u32x4 (&v)[kChunks]) {
        const uint32_t base = (uint32_t)((p * kAta8Panel + wave) * n * 2);
#pragma unroll
        for (int k = 0; k < kChunks; ++k) {
            const int cc = lane + 64 * k;
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(
                ra, cc < cpr ? base + (uint32_t)cc * 16 : kOOB, 0, 2 /*nt*/);
        }
    };
    auto store_panel = [&](const u32x4 (&v)[kChunks]) {
#pragma unroll
        for (int k = 0; k < kChunks; ++k) {
            const int cc = lane + 64 * k;
            if (cc < cpr)
                *(u32x4 *)&sp[wave * srow + 8 * cc] = v[k];
        }
    };

    u32x4 pf[kChunks];
    load_panel(0, pf);

    // packed Q operands of this wave's blocks: slot (4 (kb0 + j) + g, li & 7) of the hi
    // plane in lanes li < 8, of the lo plane in lanes li >= 8
    bf16x8 qp[kAtaMaxBlocks];
#pragma unroll
    for (int j = 0; j < kAtaMaxBlocks; ++j) {
        const int64_t kb = 4 * (kb0 + (j < kbn ? j : 0)) + g, slot = kb * RP + (li & 7);
        if (q0)  // the first iteration reads the fp32 sample itself
            qp[j] = j < kbn ? slot_from_f32(q0 + (int64_t)b * n * r, n, r, kb, li & 7, li >= 8)
                            : bf16x8{};
        else
            qp[j] = j < kbn ? (li < 8 ? qhi[slot] : qlo[slot]) : bf16x8{};
    }

    const int tailc = (32 * nb - (int)n) / 8;
    if ((int)threadIdx.x < kAta8Panel * tailc) {
        const int row = threadIdx.x / tailc, cc = threadIdx.x % tailc;
        *(u32x4 *)&sp[row * srow + (int)n + 8 * cc] = u32x4{0u, 0u, 0u, 0u};
    }

    f32x4 zacc[kAtaMaxBlocks][2];
#pragma unroll
    for (int j = 0; j < kAtaMaxBlocks; ++j)
        zacc[j][0] = zacc[j][1] = f32x4{0.f, 0.f, 0.f, 0.f};

    const int64_t npanels = (rows_here + kAta8Panel - 1) / kAta8Panel;
    for (int64_t p = 0; p < npanels; ++p) {
        store_panel(pf);
        load_panel(p + 1, pf);  // past the last panel: all out of range, zeros, unused
        __syncthreads();        // the panel is in LDS (and the previous one fully used)

        // phase 1: D[row][c] = (panel Q hi)[row][c] for c < 8, (panel Q lo)[row][c - 8] above
        f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kAtaMaxBlocks; ++j) {
            if (j < kbn) {
                const bf16x8 a = *(const bf16x8 *)&sp[li * srow + 32 * (kb0 + j) + 8 * g];
                y = mfma(a, qp[j], y);
            }
        }
        // D layout: lane (li, g) holds rows 4g..4g+3 of column li; hi + lo across li ^ 8
        float ys[4];
#pragma unroll
        for (int v = 0; v < 4; ++v)
            ys[v] = y[v] + __shfl_xor(y[v], 8);
        if (li < 8)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                sy[wave][(4 * g + v) * 8 + li] = ys[v];
        __syncthreads();  // partial Y written
        if (threadIdx.x < kAta8Panel * 8) {
            const int e = threadIdx.x, row = e / 8, col = e % 8;
            float t = sy[0][e];
#pragma unroll
            for (int w = 1; w < kAtaWaves; ++w)
                t += sy[w][e];
            const __bf16 h = (__bf16)t, l = (__bf16)(t - (float)h);
            syo[col][row / 4][row % 4] = __builtin_bit_cast(short, h);
            syo[col + 8][row / 4][row % 4] = __builtin_bit_cast(short, l);
        }
        __syncthreads();  // Y operand written

        // phase 2: D[c][j] = (panel^T Y hi)[c][j] for j < 8, (panel^T Y lo)[c][j - 8] above
        const i16x4k bop = syo[li][g];
#pragma unroll
        for (int j = 0; j < kAtaMaxBlocks; ++j) {
            if (j < kbn) {
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int c0 = 32 * (kb0 + j) + 16 * h;
                    const i16x4 aop =
                        lds_read_tr16(&sp[(4 * g + (li >> 2)) * srow + c0 + 4 * (li & 3)]);
                    zacc[j][h] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(aop, bop, zacc[j][h],
                                                                           0, 0, 0);
                }
            }
        }
        __syncthreads();  // every wave is done with the panel and with Y
    }

    // D layout: lane (li, g) holds rows c0 + 4g .. + 3 of Z, column li; hi + lo across li ^ 8
#pragma unroll
    for (int j = 0; j < kAtaMaxBlocks; ++j) {
        if (j < kbn) {
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int64_t c0 = 32 * (kb0 + j) + 16 * h + 4 * g;
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float zs = zacc[j][h][v] + __shfl_xor(zacc[j][h][v], 8);
                    if (c0 + v < n && li < r)
                        zpart[(c0 + v) * r + li] = zs;
                }
            }
        }
    }
}

// P = A Q (fp32 [m][r]) for r <= 16 and n <= 3072, the final product of the
// iteration, built like the one-pass product's first phase: 16 waves, 16-row panels
// of A through LDS (wave w loads row w of the next panel into registers while the
// current one is used), and each wave holding the Q hi and Q lo operands of its
// 32-column blocks in registers for the whole kernel, so the panels are the only
// memory loads in the loop.  Per panel each wave multiplies its blocks by Q hi and
// Q lo into a 16 x 16 partial, and the 16 partials are added in wave order for the
// panel's rows of P.  No partial sums cross work-groups: each owns whole rows.
template <int RP>
__global__ void __launch_bounds__(kAtaThreads)
lr_aqp_kernel(const uint16_t *__restrict__ A, int64_t m, int64_t n, int r,
              uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_qops, size_t off_out,
              int64_t np, int splits, int64_t split_rows, size_t off_gram)
{
    static_assert(RP == 16, "Q hi and lo of 16 columns stay in registers");
    constexpr int kChunks = 6;
    constexpr int kPanel = 16;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / splits, s = lid % splits;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const bf16x8 *qhi = (const bf16x8 *)(wsb + off_qops);
    const bf16x8 *qlo = qhi + (np / 8) * RP;
    float *out = (float *)(wsb + off_out);

    const int64_t row0 = (int64_t)s * split_rows;
    const int64_t rows_here = m - row0 <= 0 ? 0 : (m - row0 < split_rows ? m - row0 : split_rows);
    const __amdgpu_buffer_rsrc_t ra =
        make_rsrc(A + (int64_t)b * m * n + row0 * n, (uint32_t)(rows_here * n * 2));

    __shared__ __attribute__((aligned(16))) uint16_t sp[kPanel * kAtaSrowMax];
    __shared__ f32x4 sy[kAtaWaves][64];  // each wave's 16 x 16 partial, in its D layout

    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, g = lane >> 4, li = lane & 15;
    const int nb = (int)((n + 31) / 32);
    const int nbw = (nb + kAtaWaves - 1) / kAtaWaves;
    const int kb0 = wave * nbw;
    const int kbn = nb - kb0 < nbw ? nb - kb0 : nbw;
    const int srow = (int)round_up(32 * nb, 128) + 24;
    const int cpr = (int)(n / 8);

    // wave w loads row w of a panel: chunk k of a lane is columns 8 (lane + 64 k) .. + 7
    auto load_panel = [&](int64_t p, u32x4 (&v)[kChunks]) {
        const uint32_t base = (uint32_t)((p * kPanel + wave) * n * 2);
#pragma unroll
        for (int k = 0; k < kChunks; ++k) {
            const int cc = lane + 64 * k;
            v[k] = __builtin_amdgcn_raw_buffer_load_b128(
                ra, cc < cpr ? base + (uint32_t)cc * 16 : kOOB, 0, 2 /*nt*/);
        }
    };
    auto store_panel = [&](const u32x4 (&v)[kChunks]) {
#pragma unroll
        for (int k = 0; k < kChunks; ++k) {
            const int cc = lane + 64 * k;
            if (cc < cpr)
                *(u32x4 *)&sp[wave * srow + 8 * cc] = v[k];
        }
    };

    u32x4 pf[kChunks];
    load_panel(0, pf);

    // Q operands of this wave's blocks: slot (4 (kb0 + j) + g, li) of each plane
    bf16x8 qh[kAtaMaxBlocks], ql[kAtaMaxBlocks];
#pragma unroll
    for (int j = 0; j < kAtaMaxBlocks; ++j) {
        const int64_t slot = (int64_t)(4 * (kb0 + (j < kbn ? j : 0)) + g) * RP + li;
        qh[j] = j < kbn ? qhi[slot] : bf16x8{};
        ql[j] = j < kbn ? qlo[slot] : bf16x8{};
    }

    // columns n .. 32 nb - 1 of every panel row stay zero (they are multiplied)
    const int tailc = (32 * nb - (int)n) / 8;
    if ((int)threadIdx.x < kPanel * tailc) {
        const int row = threadIdx.x / tailc, cc = threadIdx.x % tailc;
        *(u32x4 *)&sp[row * srow + (int)n + 8 * cc] = u32x4{0u, 0u, 0u, 0u};
    }

    // wave 0: this work-group's part of G = P^T P, from the panel's rows of P as it
    // writes them (rows past m are zero and add nothing)
    f64x4 gacc = f64x4{0.0, 0.0, 0.0, 0.0};
    const int64_t npanels = (rows_here + kPanel - 1) / kPanel;
    for (int64_t p = 0; p < npanels; ++p) {
        store_panel(pf);
        load_panel(p + 1, pf);  // past the last panel: all out of range, zeros, unused
        __syncthreads();        // the panel is in LDS (and the previous one's partials read)

        f32x4 y = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int j = 0; j < kAtaMaxBlocks; ++j) {
            if (j < kbn) {
                const bf16x8 a = *(const bf16x8 *)&sp[li * srow + 32 * (kb0 + j) + 8 * g];
                y = mfma(a, qh[j], y);
                y = mfma(a, ql[j], y);
            }
        }
        sy[wave][lane] = y;  // D layout: rows 4g..4g+3 of column li
        __syncthreads();     // every partial written, every wave done with the panel
        if (threadIdx.x < 64) {
            // the lane's four values: rows 4g + v, column li, summed over the waves in order
            f32x4 t = sy[0][threadIdx.x];
#pragma unroll 3
            for (int w = 1; w < kAtaWaves; ++w) {
                const f32x4 u = sy[w][threadIdx.x];
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    t[v] += u[v];
            }
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t row = row0 + p * kPanel + 4 * g + v;
                if (row < row0 + rows_here && li < r)
                    out[row * r + li] = t[v];
            }
            // A[i][k] = P[row k][i] and B[k][j] = P[row k][j] at lane (i or j, k): the
            // lane's value of row 4 k + v
#pragma unroll
            for (int v = 0; v < 4; ++v)
                gacc = mfma64((double)t[v], (double)t[v], gacc);
        }
    }
    if (threadIdx.x < 64) {  // the partial in the Gram kernel's layout: G[i][j] at i RP + j
        double *part = (double *)(wsb + off_gram) + (size_t)s * RP * RP;
#pragma unroll
        for (int v = 0; v < 4; ++v)
            part[(4 * v + g) * RP + li] = gacc[v];
    }
}

int ata_splits(int64_t batch, int64_t m, int64_t n, int r)
{
    if (r > 16 || n > kAtaMaxN || batch <= 0)
        return 0;
    int64_t s = kComputeUnits / batch;
    s = s < 1 ? 1 : (s > kAtaMaxSplits ? kAtaMaxSplits : s);
    const int64_t panels = (m + kAtaPanel - 1) / kAtaPanel;
    return (int)(s < panels ? s : panels);
}

// Loads the B operands of M Rinv for every k step and column tile (Rinv upper
// triangular fp64 [RP][RP]): rb[ks][ct] = Rinv[4 ks + g][16 ct + c].
template <int RP>
__device__ __forceinline__ void load_rinv_ops(const double *rinv, int g, int c, double (&rb)[RP / 4][RP / 16])
{
#pragma unroll
    for (int ks = 0; ks < RP / 4; ++ks)
#pragma unroll
        for (int ct = 0; ct < RP / 16; ++ct)
            rb[ks][ct] = rinv[(4 * ks + g) * RP + 16 * ct + c];
}

// Rows t0..t0+15 of M Rinv (fp64 products of the fp32 rows) in the D layout:
// item v of lane (c, g) holds row t0 + 4 v + g, column 16 ct + c.
template <int RP>
__device__ __forceinline__ void tile_times_rinv(const float *Mb, int64_t L, int r, int64_t t0, int g,
                                                int c, const double (&rb)[RP / 4][RP / 16],
                                                f64x4 (&tile)[RP / 16])
{
#pragma unroll
    for (int ct = 0; ct < RP / 16; ++ct)
        tile[ct] = f64x4{0.0, 0.0, 0.0, 0.0};
    const int64_t row = t0 + c;
#pragma unroll
    for (int ks = 0; ks < RP / 4; ++ks) {
        const int k = 4 * ks + g;
        const double av = (row < L && k < r) ? (double)Mb[row * r + k] : 0.0;
#pragma unroll
        for (int ct = 0; ct < RP / 16; ++ct)
            if (4 * ks < 16 * ct + 16)  // Rinv is upper triangular: rows past the tile are zero
                tile[ct] = mfma64(av, rb[ks][ct], tile[ct]);
    }
}

// ------------------------------------------------------------------ Gram partials

// Partial G = M'^T M' over kGramRows rows in fp64 on MFMA, M' = M (fp32 [L][r])
// or, with TRANSFORM, M' = M Rinv.  Each wave takes 16-row tiles; tiles in the
// D layout feed the Gram MFMA directly (A and B hold the same rows per lane
// group and item, so the k order is consistent).  Only the upper tile pairs are
// formed; the partial's lower off-diagonal tiles are written as zero.
// nsum > 1 (without TRANSFORM): M is the first of nsum partial sums, pstride
// floats apart; each element is their sum in order 0, 1, ..., written back
// over the first (Msum, the same buffer) for the kernels after this one.  M and
// Msum alias, so neither is declared restrict; each element is read by the one
// thread that then writes it.
// With TRANSFORM (the second pass) the work-groups of a matrix whose first pass
// sufficed (flag 0 at off_flag) return at once.
template <int RP, bool TRANSFORM>
__global__ void __launch_bounds__(kThreads)
lr_gram_kernel(const float *M, int64_t m_stride, int64_t L, int r,
               uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_rinv, size_t off_gram,
               int blocks_per_mat, float *Msum, int nsum, int64_t pstride, size_t off_flag)
{
    constexpr int CT = RP / 16, NP = CT * (CT + 1) / 2;
    constexpr int WROWS = kGramRows / 4;  // rows per wave
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    const float *Mb = M + (int64_t)b * m_stride;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    if constexpr (TRANSFORM) {
        if (*(const int32_t *)(wsb + off_flag) == 0)
            return;
    }
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, g = lane >> 4, c = lane & 15;
    __shared__ double sacc[4][RP * RP];

    double rb[RP / 4][RP / 16];
    if constexpr (TRANSFORM)
        load_rinv_ops<RP>((const double *)(wsb + off_rinv), g, c, rb);

    f64x4 acc[NP];
#pragma unroll
    for (int p = 0; p < NP; ++p)
        acc[p] = f64x4{0.0, 0.0, 0.0, 0.0};
    const int64_t w0 = (int64_t)blk * kGramRows + wave * WROWS;
    if constexpr (!TRANSFORM && RP == 16) {
        // the wave's rows in two halves of kGramHalf 16-row tiles; per half, every element
        // x[tt][v] = M[t0 + 16 tt + 4 v + g][c] summed over the partials with all loads
        // in flight together, and every store (Msum aliases M) after every load.  Raw
        // buffer loads: one 32-bit offset per element, the partial's in a scalar
        // register; an element past the matrix gets an offset past the end and reads 0.
        constexpr int NH = kGramHalf;
        static_assert(WROWS == 2 * 16 * NH, "two halves per wave");
        const __amdgpu_buffer_rsrc_t rsm =
            make_rsrc(Mb, (uint32_t)((nsum > 1 ? nsum * pstride : L * r) * 4));
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int64_t t0 = w0 + 16 * NH * h;
            float x[NH][4], pv[kMaxPartials - 1][NH][4];
            uint32_t off[NH][4];
#pragma unroll
            for (int tt = 0; tt < NH; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const int64_t row = t0 + 16 * tt + 4 * v + g;
                    off[tt][v] = (row < L && c < r) ? (uint32_t)((row * r + c) * 4) : kOOB;
                    x[tt][v] = __builtin_bit_cast(
                        float, __builtin_amdgcn_raw_buffer_load_b32(rsm, off[tt][v], 0, 0));
#pragma unroll
                    for (int q = 1; q < kMaxPartials; ++q)
                        pv[q - 1][tt][v] =
                            q < nsum ? __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(
                                                                    rsm, off[tt][v], (int)(q * pstride * 4), 0))
                                     : 0.0f;
                }
#pragma unroll
            for (int q = 1; q < kMaxPartials; ++q)
                if (q < nsum)
#pragma unroll
                    for (int tt = 0; tt < NH; ++tt)
#pragma unroll
                        for (int v = 0; v < 4; ++v)
                            x[tt][v] += pv[q - 1][tt][v];
            if (nsum > 1) {
                const __amdgpu_buffer_rsrc_t rso =
                    make_rsrc(Msum + (int64_t)b * m_stride, (uint32_t)(L * r * 4));
#pragma unroll
                for (int tt = 0; tt < NH; ++tt)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        __builtin_amdgcn_raw_buffer_store_b32(__builtin_bit_cast(uint32_t, x[tt][v]),
                                                              rso, off[tt][v], 0, 0);
            }
#pragma unroll
            for (int tt = 0; tt < NH; ++tt)
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[0] = mfma64((double)x[tt][v], (double)x[tt][v], acc[0]);
        }
    } else {
        for (int tt = 0; tt < WROWS / 16; ++tt) {
            const int64_t t0 = w0 + 16 * tt;
            if (t0 >= L)
                break;  // per wave; no barrier inside this loop
            f64x4 tile[CT];
            if constexpr (TRANSFORM) {
                tile_times_rinv<RP>(Mb, L, r, t0, g, c, rb, tile);
            } else {
#pragma unroll
                for (int ct = 0; ct < CT; ++ct)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const int64_t row = t0 + 4 * v + g;
                        const int col = 16 * ct + c;
                        float x = 0.0f;
                        if (row < L && col < r) {
                            const int64_t o = row * r + col;
                            x = Mb[o];
                            if (nsum > 1) {
                                float pv[kMaxPartials];
#pragma unroll
                                for (int q = 1; q < kMaxPartials; ++q)
                                    pv[q] = q < nsum ? Mb[o + q * pstride] : 0.0f;
#pragma unroll
                                for (int q = 1; q < kMaxPartials; ++q)
                                    if (q < nsum)
                                        x += pv[q];
                                Msum[(int64_t)b * m_stride + o] = x;
                            }
                        }
                        tile[ct][v] = (double)x;
                    }
            }
            int p = 0;
#pragma unroll
            for (int ta = 0; ta < CT; ++ta)
#pragma unroll
                for (int tb = ta; tb < CT; ++tb, ++p)
#pragma unroll
                    for (int v = 0; v < 4; ++v)
                        acc[p] = mfma64(tile[ta][v], tile[tb][v], acc[p]);
        }
    }
    int p = 0;
#pragma unroll
    for (int ta = 0; ta < CT; ++ta)
#pragma unroll
        for (int tb = ta; tb < CT; ++tb, ++p)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                sacc[wave][(16 * ta + 4 * v + g) * RP + 16 * tb + c] = acc[p][v];
    __syncthreads();
    double *part = (double *)(wsb + off_gram) + (size_t)blk * RP * RP;
    for (int e = threadIdx.x; e < RP * RP; e += kThreads) {
        const int i = e / RP, j = e % RP;
        part[e] = (i / 16 <= j / 16) ? (sacc[0][e] + sacc[1][e]) + (sacc[2][e] + sacc[3][e]) : 0.0;
    }
}

// ------------------------------------------------------------------ Cholesky + inverse

// Orders one wavefront's LDS accesses (write, then other lanes read) without a
// work-group barrier: the factorisation below runs on one wave of a larger
// work-group too.
__device__ __forceinline__ void wave_sync()
{
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

template <int RP>
struct CholShared {
    double G[RP][RP + 1];   // the Gram matrix (entries i <= j are used)
    double Rs[RP][RP + 1];  // R
    double S1[RP][RP + 1];  // pass 2: R1^-1
    double rdiag[RP];
};

// On one wavefront: factors G = R^T R (R upper, positive diagonal) in fp64 with
// lane j holding column j in registers (pivots and multipliers broadcast with
// readlane), stores R in cs.Rs (zero below the diagonal and in dropped and pad
// columns), and inverts R by back substitution, again one column per lane:
// x[i] = (R^-1)[i][lane], sx = sum_i x[i]^2.  A pivot <= 1e-13 trace(G) / r, or
// not finite, drops its column.
template <int RP>
__device__ __forceinline__ void chol_factor_invert(CholShared<RP> &cs, int r, int lane,
                                                   double (&x)[RP], double &sx)
{
    const bool col = lane < RP;
    const int lc = col ? lane : 0;
    double tr = 0.0;
#pragma unroll
    for (int k = 0; k < RP; ++k)
        tr += k < r ? cs.G[k][k] : 0.0;
    const double tol = 1e-13 * tr / r;

    // gc[i] = G[i][lane] for i <= lane, overwritten by R[i][lane].  Steps k >= r
    // only see zero padding; they run with a zero pivot and change nothing.
    uint32_t dead = 0;
    {
        double gc[RP];
#pragma unroll
        for (int i = 0; i < RP; ++i)
            gc[i] = (col && i <= lane) ? cs.G[i][lc] : 0.0;
#pragma unroll
        for (int k = 0; k < RP; ++k) {
            const double dkk = readlane_f64(gc[k], k);
            const bool bad = k >= r || !(dkk > tol) || !isfinite(dkk);
            // 1 / sqrt(pivot): the hardware estimate and two Newton steps (within
            // about an ulp), a third of the latency of a rounded sqrt and divide on
            // the one chain every step waits for
            const double d = bad ? 1.0 : dkk;
            double y = __builtin_amdgcn_rsq(d);
#pragma unroll
            for (int it = 0; it < 2; ++it)
                y = fma(0.5 * y, fma(-d * y, y, 1.0), y);
            const double inv = bad ? 0.0 : y;
            dead |= bad ? (1u << k) : 0u;
            // R[k][lane] = G[k][lane] / R[k][k]; on the diagonal that is the pivot
            // times its inverse square root, R[k][k] itself
            const double rk = gc[k] * (lane >= k ? inv : 0.0);
            gc[k] = rk;
            // every lane updates: below the diagonal (i > lane) the values stay
            // finite and are only ever multiplied by zero or dropped, so no lane
            // mask is needed
#pragma unroll
            for (int i = k + 1; i < RP; ++i)
                gc[i] = fma(-readlane_f64(rk, i), rk, gc[i]);
        }
        // a dropped column has a zero R column as well; pad columns (>= r) are zero
        const bool zero_col = !col || ((dead >> lc) & 1u);
#pragma unroll
        for (int i = 0; i < RP; ++i)
            if (col)
                cs.Rs[i][lc] = (zero_col || i > lane) ? 0.0 : gc[i];
    }
    wave_sync();
    if (col)
        cs.rdiag[lc] = ((dead >> lc) & 1u) ? 0.0 : 1.0 / cs.Rs[lc][lc];
    wave_sync();

    // x[i] = (R^-1)[i][lane], bottom row first.  Each sum runs from the far end,
    // so x[i + 1], the value just computed, enters last and the rows' sums overlap.
    sx = 0.0;
#pragma unroll
    for (int i = RP - 1; i >= 0; --i) {
        double s = 0.0;
#pragma unroll
        for (int k = RP - 1; k > i; --k)
            s = fma(cs.Rs[i][k], x[k], s);
        // (delta - s) / R[i][i]: below the diagonal every x[k] in s is zero, so
        // one expression covers all three cases without a branch
        x[i] = ((i == lane ? 1.0 : 0.0) - s) * cs.rdiag[i];
        sx = fma(x[i], x[i], sx);
    }
}

// On the same wavefront after a first-pass factorisation: whether the matrix
// needs the second pass.  Condition estimate ||R1||_F^2 ||R1^-1||_F^2
// (>= kappa_2(M)^2) from the columns' sums of squares, added through LDS in the
// same order by every lane so that all lanes (and runs) decide alike; a NaN
// estimate takes the second pass.  Overwrites rows 0 and 1 of cs.G.
template <int RP>
__device__ __forceinline__ bool chol_needs_second_pass(CholShared<RP> &cs, int lane, double sx)
{
    if (lane < RP) {
        double sr = 0.0;
#pragma unroll
        for (int i = 0; i < RP; ++i)
            sr = fma(cs.Rs[i][lane], cs.Rs[i][lane], sr);
        cs.G[0][lane] = sr;
        cs.G[1][lane] = sx;
    }
    wave_sync();
    double tr2 = 0.0, tx2 = 0.0;
#pragma unroll
    for (int j = 0; j < RP; ++j) {
        tr2 += cs.G[0][j];
        tx2 += cs.G[1][j];
    }
    return !(tr2 * tx2 <= kTwoPassKappa2);
}

// One wavefront per matrix.  Sums the Gram partials in a fixed order, then the
// factorisation and inverse above.
// pass 1: store R1 and R1^-1, R1^-1 also as the final R^-1, and decide whether
// the matrix needs the second pass (flag at off_flag).  pass 2: for a flagged
// matrix, overwrite the final R^-1 with (R1^-1 R2^-1) and, when ru_out is
// given, store R = R2 R1 as fp32 [r][r]; for the others only R = R1.
template <int RP>
__global__ void __launch_bounds__(kCholThreads)
lr_chol_kernel(uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_gram, int gram_blocks,
               int r, int pass, size_t off_r1, size_t off_r1inv, size_t off_rinv,
               float *__restrict__ ru_out, size_t off_flag)
{
    const int b = blockIdx.x;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    int32_t *flag = (int32_t *)(wsb + off_flag);
    if (pass == 2 && *flag == 0) {
        // the first pass sufficed: R = R1, already final in the workspace
        if (ru_out && (int)threadIdx.x < r) {
            const double *r1 = (const double *)(wsb + off_r1);
            float *ru = ru_out + (size_t)b * r * r;
            for (int i = 0; i < r; ++i)
                ru[i * r + threadIdx.x] = (float)r1[i * RP + threadIdx.x];
        }
        return;
    }
    __shared__ CholShared<RP> cs;
    const int lane = threadIdx.x;
    constexpr int PER = RP * RP / kCholThreads;

    // 1. sum the partials in a fixed order.  Every load is issued before the
    //    first add waits: QU partials per round (all the lane's entries of each),
    //    and in pass 2 R1^-1 alongside.
    const double *part = (const double *)(wsb + off_gram);
    double s1v[PER];
    if (pass == 2) {
        const double *r1inv = (const double *)(wsb + off_r1inv);
#pragma unroll
        for (int e = 0; e < PER; ++e)
            s1v[e] = r1inv[lane + kCholThreads * e];
    }
    constexpr int QU = PER >= 16 ? 2 : 32 / PER;
    double sum[PER];
#pragma unroll
    for (int e = 0; e < PER; ++e)
        sum[e] = 0.0;
    for (int q0 = 0; q0 < gram_blocks; q0 += QU) {
        double v[QU][PER];
#pragma unroll
        for (int j = 0; j < QU; ++j) {  // past the last partial: re-read it, add nothing
            const int q = q0 + j < gram_blocks ? q0 + j : gram_blocks - 1;
#pragma unroll
            for (int e = 0; e < PER; ++e)
                v[j][e] = part[(size_t)q * RP * RP + lane + kCholThreads * e];
        }
#pragma unroll
        for (int j = 0; j < QU; ++j)
#pragma unroll
            for (int e = 0; e < PER; ++e)
                sum[e] += q0 + j < gram_blocks ? v[j][e] : 0.0;
    }
#pragma unroll
    for (int e = 0; e < PER; ++e) {
        const int idx = lane + kCholThreads * e;
        cs.G[idx / RP][idx % RP] = sum[e];
    }
    if (pass == 2)
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = lane + kCholThreads * e;
            cs.S1[idx / RP][idx % RP] = s1v[e];
        }
    wave_sync();

    // 2.-3. factorisation and inverse
    double x[RP], sx;
    chol_factor_invert<RP>(cs, r, lane, x, sx);

    double *r1 = (double *)(wsb + off_r1), *r1inv = (double *)(wsb + off_r1inv);
    double *rinv = (double *)(wsb + off_rinv);
    if (lane >= RP)
        return;
    if (pass == 1) {
        // R1 and R1^-1; R1^-1 is the final R^-1 unless the second pass runs
#pragma unroll
        for (int i = 0; i < RP; ++i) {
            r1[i * RP + lane] = cs.Rs[i][lane];
            r1inv[i * RP + lane] = x[i];
            rinv[i * RP + lane] = x[i];
        }
        // 4. whether the second pass runs
        const bool two = chol_needs_second_pass<RP>(cs, lane, sx);
        if (lane == 0)
            *flag = two ? 1 : 0;
        return;
    }
    // 5. pass 2: column lane of R2 R1 and of R1^-1 R2^-1, four rows at a time
    //    (their sums interleave), the group's stores after its sums
    float *ru = ru_out ? ru_out + (size_t)b * r * r : nullptr;
    const bool ru_col = ru != nullptr && lane < r;
    double r1c[RP];
#pragma unroll
    for (int k = 0; k < RP; ++k)
        r1c[k] = r1[k * RP + lane];
    constexpr int IG = 4;
#pragma unroll
    for (int i0 = 0; i0 < RP; i0 += IG) {
        double sw[IG], si[IG];
#pragma unroll
        for (int ii = 0; ii < IG; ++ii) {
            const int i = i0 + ii;
            sw[ii] = 0.0;
            si[ii] = 0.0;
#pragma unroll
            for (int k = i; k < RP; ++k) {
                sw[ii] = fma(cs.Rs[i][k], r1c[k], sw[ii]);
                si[ii] = fma(cs.S1[i][k], x[k], si[ii]);
            }
        }
#pragma unroll
        for (int ii = 0; ii < IG; ++ii)
            rinv[(i0 + ii) * RP + lane] = si[ii];
        if (ru_col)
#pragma unroll
            for (int ii = 0; ii < IG; ++ii)
                if (i0 + ii < r)
                    ru[(i0 + ii) * r + lane] = (float)sw[ii];
    }
}

// ------------------------------------------------------------------ apply M Rinv

// Q = M Rinv on fp64 MFMA, 16-row tiles per wave, then through LDS so that the
// fp32 output is written row by row and every operand slot (8 rows of one
// column) is one 16-byte store per plane.  Rows L..Lp-1 of the operand layout
// are written as zeros; columns r..RP-1 are zero.  M and out may be the same
// buffer (Q0 passed as V at T = 0), so neither is restrict: a wave reads its
// 16-row tile in full before it writes that tile's rows, and no other wave
// touches them.
template <int RP>
__global__ void __launch_bounds__(kThreads)
lr_apply_kernel(const float *M, int64_t m_stride, int64_t L, int64_t Lp, int r,
                uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_rinv, bool ops,
                size_t off_ops, float *out, int64_t out_stride, int blocks_per_mat)
{
    constexpr int CT = RP / 16;
    constexpr int WROWS = kApplyRows / 4;
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    const float *Mb = M + (int64_t)b * m_stride;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const int wave = threadIdx.x / 64, lane = threadIdx.x % 64, g = lane >> 4, c = lane & 15;
    __shared__ float sq[4][16][RP + 1];

    double rb[RP / 4][RP / 16];
    load_rinv_ops<RP>((const double *)(wsb + off_rinv), g, c, rb);
    bf16x8 *hi = (bf16x8 *)(wsb + off_ops);
    bf16x8 *lo = hi + (Lp / 8) * RP;
    float *ob = out ? out + (int64_t)b * out_stride : nullptr;

    const int64_t w0 = (int64_t)blk * kApplyRows + wave * WROWS;
    for (int tt = 0; tt < WROWS / 16; ++tt) {
        const int64_t t0 = w0 + 16 * tt;
        if (t0 >= Lp)
            break;  // per wave; only wave-local LDS below
        f64x4 tile[CT];
        tile_times_rinv<RP>(Mb, L, r, t0, g, c, rb, tile);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                sq[wave][4 * v + g][16 * ct + c] = (float)tile[ct][v];
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        if (ob) {  // 4 lanes per row, RP/4 consecutive columns each
            const int i = lane >> 2, c0 = (lane & 3) * (RP / 4);
            const int64_t row = t0 + i;
            if (row < L)
#pragma unroll
                for (int cc = 0; cc < RP / 4; ++cc)
                    if (c0 + cc < r)
                        ob[row * r + c0 + cc] = sq[wave][i][c0 + cc];
        }
        if (ops && lane < 2 * RP) {  // one operand slot per lane
            const int kb = lane / RP, cc = lane % RP;
            bf16x8 h, l;
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const float q = sq[wave][8 * kb + i][cc];
                h[i] = (__bf16)q;
                l[i] = (__bf16)(q - (float)h[i]);
            }
            const int64_t slot = ((t0 >> 3) + kb) * RP + cc;
            hi[slot] = h;
            lo[slot] = l;
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    }
}

// ------------------------------------------------------------------ factor and apply

// Second half of the orthogonalisation for RP = 16 in one launch, after the
// Gram kernel: each work-group takes kCaRows rows of one matrix and
//   1. while its apply tiles load, wave 0 adds up the Gram partials in a fixed
//      order and factors them (the Cholesky, inverse and condition estimate
//      above) -- every work-group of the matrix repeats this small step, so
//      that no launch or cross-work-group wait separates it from the apply;
//   2. only for a matrix the estimate flags: G2 = (M R1^-1)^T (M R1^-1) over
//      all rows of the matrix, again in every work-group, and wave 0 factors
//      G2 and forms R1^-1 R2^-1 and R2 R1;
//   3. Q = M R^-1 on its rows, written as fp32 rows (out) and in the operand
//      layout (ops); the matrix's first work-group writes R as fp32 (ru_out).
// This replaces the launches of the first factorisation, of the gated second
// pass (Gram and factorisation, which matrices whose first pass suffices leave
// at once) and of the apply.  M's tiles are read with the rows in the low lane
// bits (the fp64 MFMA's A operand); the D layout result goes through LDS for
// the row-major and operand-layout stores.  out must not overlap M: the second
// pass of one work-group reads rows that another may already be writing.
constexpr int kCaWaves = 4;
constexpr int kCaThreads = 64 * kCaWaves;
constexpr int kCaRows = 768;                          // apply rows per work-group
constexpr int kCaTiles = kCaRows / 16 / kCaWaves;    // 16-row tiles per wave
constexpr int kCaPass2Tiles = 8;                      // tiles in flight in the second pass
constexpr int kCaGroup = 4;                           // tiles per LDS round trip of the apply

// A operands (rows in the low lane bits) of NT 16-row tiles from row t0 on, one
// 16-byte load per lane and tile: av[u][ks] = M[t0 + 16 u + c][4 g + ks], zero
// past row L or column r.  The MFMA's k index k' = g of chunk ks then stands for
// column 4 k' + ks; the B operand uses the same assignment (R^-1[4 g + ks][c]).
template <int NT>
__device__ __forceinline__ void load_a_tiles(__amdgpu_buffer_rsrc_t rs, int64_t L, int r, int64_t t0,
                                             int g, int c, float (&av)[NT][4])
{
    const bool vec = r % 4 == 0;  // rows of whole 16-byte pieces: one 16-byte load per lane
#pragma unroll
    for (int u = 0; u < NT; ++u) {
        const int64_t row = t0 + 16 * u + c;
        if (vec) {
            const uint32_t off = (row < L && 4 * g < r) ? (uint32_t)((row * r + 4 * g) * 4) : kOOB;
            // cast as a whole: subscripting the builtin's integer vector result
            // compiles into one dword load splat over the four elements
            const f32x4 v =
                __builtin_bit_cast(f32x4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                av[u][ks] = v[ks];
        } else {
#pragma unroll
            for (int ks = 0; ks < 4; ++ks) {
                const int k = 4 * g + ks;
                const uint32_t off = (k < r && row < L) ? (uint32_t)((row * r + k) * 4) : kOOB;
                av[u][ks] = __builtin_bit_cast(
                    float, __builtin_amdgcn_raw_buffer_load_b32(rs, off, 0, 0));
            }
        }
    }
}

template <int RP>
__global__ void __launch_bounds__(kCaThreads)
lr_cholapply_kernel(const float *M, int64_t m_stride, int64_t L, int r, uint8_t *__restrict__ ws,
                    size_t layer_bytes, size_t off_gram, int gram_blocks, size_t off_ops,
                    int64_t Lp_ops, bool ops, float *out, int64_t out_stride,
                    float *__restrict__ ru_out, int blocks_per_mat)
{
    static_assert(RP == 16, "one 16 x 16 fp64 tile per product");
    const int lid = xcd_remap(blockIdx.x, gridDim.x);
    const int b = lid / blocks_per_mat, blk = lid % blocks_per_mat;
    const float *Mb = M + (int64_t)b * m_stride;
    uint8_t *wsb = ws + (size_t)b * layer_bytes;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / 64);
    const int lane = threadIdx.x % 64, g = lane >> 4, c = lane & 15;
    const int64_t Lp = round_up(L, 64);
    const int64_t w0 = (int64_t)blk * kCaRows + wave * (kCaRows / kCaWaves);
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(Mb, (uint32_t)(L * r * 4));

    __shared__ double sg[kCaWaves][RP * RP];
    __shared__ float sq[kCaWaves][16 * kCaGroup][RP + 1];
    __shared__ CholShared<RP> cs;
    __shared__ double r1s[RP][RP + 1];   // R1
    __shared__ double rfin[RP][RP + 1];  // the final R^-1
    __shared__ int two_s;

    // 1. the Gram partials in order, then the first factorisation, on wave 0.
    //    Every wave's apply tiles load meanwhile; wave 0 issues its own after the
    //    partials, since a wave's loads return in issue order.
    float av[kCaTiles][4];
    if (wave != 0)
        load_a_tiles<kCaTiles>(rs, L, r, w0, g, c, av);
    if (wave == 0) {
        const double *part = (const double *)(wsb + off_gram);
        constexpr int PER = RP * RP / 64;
        constexpr int QU = 16;  // partials whose loads are in flight together
        double sum[PER];
#pragma unroll
        for (int e = 0; e < PER; ++e)
            sum[e] = 0.0;
        for (int q0 = 0; q0 < gram_blocks; q0 += QU) {
            double v[QU][PER];
#pragma unroll
            for (int j = 0; j < QU; ++j)
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    v[j][e] = q0 + j < gram_blocks
                                  ? part[(size_t)(q0 + j) * RP * RP + lane + 64 * e] : 0.0;
#pragma unroll
            for (int j = 0; j < QU; ++j)
#pragma unroll
                for (int e = 0; e < PER; ++e)
                    if (q0 + j < gram_blocks)
                        sum[e] += v[j][e];
        }
#pragma unroll
        for (int e = 0; e < PER; ++e) {
            const int idx = lane + 64 * e;
            cs.G[idx / RP][idx % RP] = sum[e];
        }
        wave_sync();
        __builtin_amdgcn_sched_barrier(0);  // the partials' loads stay ahead of the tiles'
        load_a_tiles<kCaTiles>(rs, L, r, w0, g, c, av);
        double x[RP], sx;
        chol_factor_invert<RP>(cs, r, lane, x, sx);
        if (lane < RP) {
#pragma unroll
            for (int i = 0; i < RP; ++i) {
                r1s[i][lane] = cs.Rs[i][lane];
                cs.S1[i][lane] = x[i];
                rfin[i][lane] = x[i];
            }
            const bool two = chol_needs_second_pass<RP>(cs, lane, sx);
            if (lane == 0)
                two_s = two ? 1 : 0;
        }
    }
    __syncthreads();

    float *ru = (ru_out && blk == 0) ? ru_out + (size_t)b * r * r : nullptr;
    // 2. the second pass, for a flagged matrix only: G2 over all rows of the matrix
    if (two_s != 0) {
        double rb[4];
#pragma unroll
        for (int ks = 0; ks < 4; ++ks)
            rb[ks] = cs.S1[4 * g + ks][c];
        f64x4 acc[2] = {f64x4{0.0, 0.0, 0.0, 0.0}, f64x4{0.0, 0.0, 0.0, 0.0}};
        const int64_t ntile = Lp / 16;
        for (int64_t t0 = (int64_t)wave * kCaPass2Tiles; t0 < ntile; t0 += (int64_t)kCaWaves * kCaPass2Tiles) {
            float pv[kCaPass2Tiles][4];
            load_a_tiles<kCaPass2Tiles>(rs, L, r, 16 * t0, g, c, pv);
#pragma unroll
            for (int u = 0; u < kCaPass2Tiles; ++u) {
                f64x4 w = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
                for (int ks = 0; ks < 4; ++ks)
                    w = mfma64((double)pv[u][ks], rb[ks], w);
#pragma unroll
                for (int v = 0; v < 4; ++v)
                    acc[u % 2] = mfma64(w[v], w[v], acc[u % 2]);
            }
        }
#pragma unroll
        for (int v = 0; v < 4; ++v)
            sg[wave][(4 * v + g) * RP + c] = acc[0][v] + acc[1][v];
        __syncthreads();
        if (wave == 0) {
#pragma unroll
            for (int e = 0; e < RP * RP / 64; ++e) {
                const int idx = lane + 64 * e;
                double t = sg[0][idx];
#pragma unroll
                for (int w = 1; w < kCaWaves; ++w)
                    t += sg[w][idx];
                cs.G[idx / RP][idx % RP] = t;
            }
            wave_sync();
            double x[RP], sx;
            chol_factor_invert<RP>(cs, r, lane, x, sx);
            if (lane < RP) {
                // column lane of R2 R1 and of R1^-1 R2^-1, four rows at a time (their
                // sums interleave), the group's stores after its sums
                const bool ru_col = ru != nullptr && lane < r;
                double r1c[RP];
#pragma unroll
                for (int k = 0; k < RP; ++k)
                    r1c[k] = r1s[k][lane];
                constexpr int IG = 4;
#pragma unroll
                for (int i0 = 0; i0 < RP; i0 += IG) {
                    double sw[IG], si[IG];
#pragma unroll
                    for (int ii = 0; ii < IG; ++ii) {
                        const int i = i0 + ii;
                        sw[ii] = 0.0;
                        si[ii] = 0.0;
#pragma unroll
                        for (int k = i; k < RP; ++k) {
                            sw[ii] = fma(cs.Rs[i][k], r1c[k], sw[ii]);
                            si[ii] = fma(cs.S1[i][k], x[k], si[ii]);
                        }
                    }
#pragma unroll
                    for (int ii = 0; ii < IG; ++ii)
                        rfin[i0 + ii][lane] = si[ii];
                    if (ru_col)
#pragma unroll
                        for (int ii = 0; ii < IG; ++ii)
                            if (i0 + ii < r)
                                ru[(i0 + ii) * r + lane] = (float)sw[ii];
                }
            }
        }
    } else if (wave == 0 && ru && lane < r) {  // R = R1
        for (int i = 0; i < r; ++i)
            ru[i * r + lane] = (float)r1s[i][lane];
    }
    __syncthreads();

    // 3. Q = M R^-1 on this work-group's rows
    double rb[4];
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
        rb[ks] = rfin[4 * g + ks][c];
    float *ob = out ? out + (int64_t)b * out_stride : nullptr;
    bf16x8 *hi = (bf16x8 *)(wsb + off_ops);
    bf16x8 *lo = hi + (Lp_ops / 8) * RP;
    static_assert(kCaTiles % kCaGroup == 0, "whole groups of tiles");
#pragma unroll
    for (int u0 = 0; u0 < kCaTiles; u0 += kCaGroup) {
        const int64_t g0 = w0 + 16 * u0;  // first row of the group
        if (g0 >= Lp)
            break;  // per wave; only wave-local LDS below
        f64x4 q[kCaGroup];
#pragma unroll
        for (int u = 0; u < kCaGroup; ++u) {
            q[u] = f64x4{0.0, 0.0, 0.0, 0.0};
#pragma unroll
            for (int ks = 0; ks < 4; ++ks)
                q[u] = mfma64((double)av[u0 + u][ks], rb[ks], q[u]);
        }
#pragma unroll
        for (int u = 0; u < kCaGroup; ++u)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                sq[wave][16 * u + 4 * v + g][c] = (float)q[u][v];
        wave_sync();
        if (ob) {  // 4 lanes per row, 4 consecutive columns each
            const int i = lane >> 2, c0 = (lane & 3) * 4;
#pragma unroll
            for (int u = 0; u < kCaGroup; ++u) {
                const int64_t row = g0 + 16 * u + i;
                const float *qs = &sq[wave][16 * u + i][c0];
                if (row < L) {
                    if (r % 4 == 0) {
                        if (c0 < r)
                            *(float4 *)&ob[row * r + c0] = make_float4(qs[0], qs[1], qs[2], qs[3]);
                    } else
#pragma unroll
                        for (int cc = 0; cc < 4; ++cc)
                            if (c0 + cc < r)
                                ob[row * r + c0 + cc] = qs[cc];
                }
            }
        }
        if (ops) {  // one operand slot (8 rows of one column) per lane and half group
            const int kb = lane / RP, cc = lane % RP;  // kb 0..3: 8-row blocks of 32 rows
#pragma unroll
            for (int h2 = 0; h2 < kCaGroup / 2; ++h2) {
                const int rr = 32 * h2 + 8 * kb;  // first row of the slot in the group
                if (g0 + rr < Lp) {
                    bf16x8 h, l;
#pragma unroll
                    for (int i = 0; i < 8; ++i) {
                        const float qv = sq[wave][rr + i][cc];
                        h[i] = (__bf16)qv;
                        l[i] = (__bf16)(qv - (float)h[i]);
                    }
                    const int64_t slot = ((g0 + rr) >> 3) * RP + cc;
                    hi[slot] = h;
                    lo[slot] = l;
                }
            }
        }
        wave_sync();
    }
}

// ------------------------------------------------------------------ operand layout

// M (fp32 [L][r]) into the operand layout of A Q: one thread per slot (8 rows of
// one column), split into bf16 hi and lo planes; rows L..Lp-1 and columns r..RP-1
// are zeros.
template <int RP>
__global__ void __launch_bounds__(kThreads)
lr_ops_kernel(const float *__restrict__ M, int64_t m_stride, int64_t L, int64_t Lp, int r,
              uint8_t *__restrict__ ws, size_t layer_bytes, size_t off_ops, int64_t slots_per_mat,
              int64_t batch)
{
    const int64_t id = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t b = id / slots_per_mat, slot = id % slots_per_mat;
    if (b >= batch)
        return;
    const int64_t kb = slot / RP;
    const int c = (int)(slot % RP);
    const float *Mb = M + b * m_stride;
    bf16x8 *hi = (bf16x8 *)(ws + (size_t)b * layer_bytes + off_ops);
    bf16x8 *lo = hi + (Lp / 8) * RP;
    bf16x8 h, l;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t row = 8 * kb + i;
        const float q = (row < L && c < r) ? Mb[row * r + c] : 0.0f;
        h[i] = (__bf16)q;
        l[i] = (__bf16)(q - (float)h[i]);
    }
    hi[slot] = h;
    lo[slot] = l;
}

// ------------------------------------------------------------------ host orchestration

// nsum > 1: M (in the workspace) holds nsum partial sums of the matrix, L * r
// floats apart; the first Gram kernel adds them up in place.
// pre_gram > 0: the Gram partials of M (pre_gram of them) are already in the
// workspace; only the r <= 16 path without overlap takes them.
template <int RP>
hipError_t run_orth(const Layout &Ly, int64_t batch, const float *M, int64_t m_stride, int64_t L,
                    int r, uint8_t *ws, float *out, int64_t out_stride, bool ops, float *ru,
                    hipStream_t st, int nsum = 1, int pre_gram = 0)
{
    const int64_t Lp_ops = round_up(L, 64);
    const int gblocks = (int)((L + kGramRows - 1) / kGramRows);
    const int ablocks = (int)((Lp_ops + kApplyRows - 1) / kApplyRows);
    const unsigned ggrid = (unsigned)(gblocks * batch), agrid = (unsigned)(ablocks * batch);
    // factorisations and apply in one launch, unless out overlaps M (Q0 passed as V)
    const char *m0 = (const char *)M, *m1 = (const char *)(M + (batch - 1) * m_stride + L * r);
    const char *o0 = (const char *)out, *o1 = out ? (const char *)(out + (batch - 1) * out_stride + L * r) : o0;
    const bool overlap = out != nullptr && o0 < m1 && m0 < o1;
    if (pre_gram > 0 && (RP != 16 || overlap))
        return hipErrorInvalidValue;
    if (pre_gram == 0)
        hipLaunchKernelGGL((lr_gram_kernel<RP, false>), dim3(ggrid), dim3(kThreads), 0, st, M,
                           m_stride, L, r, ws, Ly.layer_bytes, Ly.off_r1inv, Ly.off_gram, gblocks,
                           nsum > 1 ? const_cast<float *>(M) : (float *)nullptr, nsum, L * r,
                           Ly.off_flag);
    if constexpr (RP == 16) {
        if (!overlap) {
            const int cblocks = (int)((Lp_ops + kCaRows - 1) / kCaRows);
            hipLaunchKernelGGL((lr_cholapply_kernel<RP>), dim3((unsigned)(cblocks * batch)),
                               dim3(kCaThreads), 0, st, M, m_stride, L, r, ws, Ly.layer_bytes,
                               Ly.off_gram, pre_gram > 0 ? pre_gram : gblocks, Ly.off_qops,
                               Lp_ops, ops, out, out_stride, ru, cblocks);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((lr_chol_kernel<RP>), dim3((unsigned)batch), dim3(kCholThreads), 0, st, ws,
                       Ly.layer_bytes, Ly.off_gram, gblocks, r, 1, Ly.off_r1, Ly.off_r1inv,
                       Ly.off_rinv, ru, Ly.off_flag);
    // the second pass: work-groups of matrices whose first pass sufficed return at once
    hipLaunchKernelGGL((lr_gram_kernel<RP, true>), dim3(ggrid), dim3(kThreads), 0, st, M,
                       m_stride, L, r, ws, Ly.layer_bytes, Ly.off_r1inv, Ly.off_gram, gblocks,
                       (float *)nullptr, 1, (int64_t)0, Ly.off_flag);
    hipLaunchKernelGGL((lr_chol_kernel<RP>), dim3((unsigned)batch), dim3(kCholThreads), 0, st, ws,
                       Ly.layer_bytes, Ly.off_gram, gblocks, r, 2, Ly.off_r1, Ly.off_r1inv,
                       Ly.off_rinv, ru, Ly.off_flag);
    hipLaunchKernelGGL((lr_apply_kernel<RP>), dim3(agrid), dim3(kThreads), 0, st, M, m_stride, L,
                       Lp_ops, r, ws, Ly.layer_bytes, Ly.off_rinv, ops, Ly.off_qops, out,
                       out_stride, ablocks);
    return hipGetLastError();
}

template <int RP>
hipError_t run_lowrank(const LowrankArgs &a, hipStream_t st)
{
    const Layout Ly = make_layout(a.batch, a.m, a.n, a.r);
    uint8_t *ws = (uint8_t *)a.ws;
    const float *mf = (const float *)(ws + Ly.off_mf);
    const int64_t mf_stride = (int64_t)(Ly.layer_bytes / 4);
    hipError_t e;
    const int aq_blocks = (int)(Ly.mp / kAqRows);
    const int aty_blocks = (int)((a.n + kAtyCols - 1) / kAtyCols);

    // step 1: orthonormalise the random sample.  With T >= 1 the sample only enters
    // through qf(A^T A Q0) = qf(A^T A orth(Q0)) (Q0 = orth(Q0) R0 with R0 upper
    // triangular, positive diagonal), so Q0 goes into the first product as it is; only
    // T = 0 returns orth(Q0) itself as V.
    if (a.T == 0) {
        if ((e = run_orth<RP>(Ly, a.batch, a.Q0, a.n * a.r, a.n, a.r, ws, a.V, a.n * a.r, true,
                              nullptr, st)) != hipSuccess)
            return e;
    } else if (!(RP == 16 && Ly.splits > 0 && a.r <= 8)) {
        // (at r <= 8 the one-pass product reads Q0 itself: 8 us less per call; at r = 9..16
        // the same conversion in that kernel's prologue cost it more than the launch saves)
        const int64_t slots = (Ly.np / 8) * RP, total = slots * a.batch;
        hipLaunchKernelGGL((lr_ops_kernel<RP>), dim3((unsigned)((total + kThreads - 1) / kThreads)),
                           dim3(kThreads), 0, st, a.Q0, a.n * a.r, a.n, Ly.np, a.r, ws,
                           Ly.layer_bytes, Ly.off_qops, slots, a.batch);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
    }
    for (int t = 0; t < a.T; ++t) {
        // Z = A^T (A Q): one pass over A with partial sums (r <= 16, n <= 3072), else two
        if constexpr (RP == 16) {
            if (Ly.splits > 0)
                hipLaunchKernelGGL((a.r <= 8 ? lr_ata8_kernel<RP> : lr_ata_kernel<RP>),
                                   dim3((unsigned)(Ly.splits * a.batch)), dim3(kAtaThreads), 0, st,
                                   a.A, a.m, a.n, a.r, ws, Ly.layer_bytes, Ly.off_qops,
                                   Ly.off_mf, Ly.np, Ly.splits, Ly.split_rows,
                                   t == 0 && a.r <= 8 ? a.Q0 : nullptr);
        }
        if (Ly.splits == 0) {
            hipLaunchKernelGGL((lr_aq_kernel<RP, true>), dim3((unsigned)(aq_blocks * a.batch)),
                               dim3(kThreads), 0, st, a.A, a.m, a.n, a.r, ws, Ly.layer_bytes,
                               Ly.off_qops, Ly.off_yops, Ly.mp, Ly.np, aq_blocks);
            hipLaunchKernelGGL((lr_aty_kernel<RP>), dim3((unsigned)(aty_blocks * a.batch)),
                               dim3(kAtyThreads), 0, st, a.A, a.m, a.n, a.r, ws, Ly.layer_bytes,
                               Ly.off_yops, Ly.off_mf, Ly.mp, aty_blocks);
        }
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        if ((e = run_orth<RP>(Ly, a.batch, mf, mf_stride, a.n, a.r, ws, a.V, a.n * a.r, true,
                              nullptr, st, Ly.splits > 1 ? Ly.splits : 1)) != hipSuccess)
            return e;
    }
    // final: P = A Q, (U, R_U) = orth(P), V = Q (already written)
    bool aq_done = false;
    if constexpr (RP == 16) {
        if (Ly.splits > 0) {
            hipLaunchKernelGGL((lr_aqp_kernel<RP>), dim3((unsigned)(Ly.splits * a.batch)),
                               dim3(kAtaThreads), 0, st, a.A, a.m, a.n, a.r, ws, Ly.layer_bytes,
                               Ly.off_qops, Ly.off_mf, Ly.np, Ly.splits, Ly.split_rows,
                               Ly.off_gram);
            aq_done = true;
        }
    }
    if (!aq_done)
        hipLaunchKernelGGL((lr_aq_kernel<RP, false>), dim3((unsigned)(aq_blocks * a.batch)),
                           dim3(kThreads), 0, st, a.A, a.m, a.n, a.r, ws, Ly.layer_bytes,
                           Ly.off_qops, Ly.off_mf, Ly.mp, Ly.np, aq_blocks);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    // after lr_aqp_kernel the Gram partials of P (one per row range) are in the workspace
    return run_orth<RP>(Ly, a.batch, mf, mf_stride, a.m, a.r, ws, a.U, a.m * a.r, false, a.RU,
                        st, 1, aq_done ? Ly.splits : 0);
}

}  // namespace

size_t lowrank_workspace_bytes(int64_t batch, int64_t m, int64_t n, int r)
{
    return make_layout(batch, m, n, r).layer_bytes * (size_t)batch;
}

hipError_t launch_lowrank(const LowrankArgs &a, hipStream_t st)
{
    if (a.batch == 0)
        return hipSuccess;
    return a.r <= 16 ? run_lowrank<16>(a, st) : run_lowrank<32>(a, st);
}

}  // namespace cfz
