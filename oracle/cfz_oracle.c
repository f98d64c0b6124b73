/*
 * cfz_oracle.c -- plain, slow CPU oracle for the CompactFusion residual codec
 * and the rank-r subspace iteration.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  It shares no code,
 * header, table or helper with the HIP library; it is written from the
 * definitions alone, one element and one group at a time, with no blocking,
 * fusion or reordering.
 *
 * Sources (paper: "Accelerating Parallel Diffusion Model Serving with
 * Residual Compression", Luo et al., NeurIPS 2025):
 *   - abstract: what travels between devices is the compressed change of an
 *     activation from one denoising step to the next, and an error-feedback
 *     term keeps the compression error from building up;
 *   - reproducibility table, "Dataset Splits": at least one uncompressed
 *     warm-up step initialises the base tensor used for later residuals;
 *   - reproducibility table, "Pseudocode", Algorithm 3 (Subspace Iteration):
 *     random orthonormal Q; T times Z = A^T A Q, Q = orth(Z); U = orth(AQ); V = Q.
 *   - xDiT issue #573 (proposal to integrate CompactFusion): the residual
 *     scheme with error feedback reduces communication by a factor of 8 to 16.
 *
 * Readings taken where the pages are silent (each one is also listed with the
 * design notes of the library):
 *   - quantizer: symmetric group-wise absmax, qmax = 2^(b-1) - 1, s = a / qmax
 *     (IEEE fp32 division), q = clamp(rint(r / s), -qmax, qmax), q = 0 when s == 0;
 *   - error feedback on step-wise differences (mode DELTA): the residual is
 *     taken against the previous activation, the carried error is added, and
 *     the receiver's base advances by the decoded payload.  LITERAL (residual
 *     against the base plus carried error) and OFF (closed loop, no error
 *     buffer) are the two other modes; OPENLOOP (differences without error
 *     feedback) exists here only as an ablation;
 *   - all codec arithmetic in IEEE fp32, round to nearest even, the only fused
 *     operations being the two explicit fmaf calls; build with
 *     -fno-fast-math -ffp-contract=off;
 *   - codes: b-bit two's complement fields, element j of the flat array in
 *     byte floor(j*b/8) at bit (j*b) mod 8;
 *   - orthogonalize(): thin QR with positive diagonal, by Householder
 *     reflections in fp64; a column whose remaining squared norm is
 *     <= 1e-13 * ||M||_F^2 / r (or not finite) is dropped: its Q column and its
 *     R row and column are zero;
 *   - the step-7 triangular factor R_U is returned beside U and V, so that the
 *     reconstruction is U R_U V^T = (A Q) Q^T;
 *   - optional bf16 state: the carried error and the base are stored in bf16;
 *     each update is the same fp32 fmaf, rounded once to bf16 (nearest even),
 *     and a zero code still leaves the base untouched;
 *   - the rank-r compressor inside the error-feedback loop: the DELTA residual
 *     rounded to bf16 goes through Algorithm 3, and the carried error and the
 *     receiver's base are updated with the fp64 reconstruction U R_U V^T.
 *
 * Parity of every function here is pinned by the CPU tests (closed forms,
 * hand-derived fixtures, brute force, invariants, exact-rank recovery and the
 * Eckart-Young bound); none is "parity unpinned".
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { MODE_DELTA = 0, MODE_LITERAL = 1, MODE_OFF = 2, MODE_OPENLOOP = 3 };
enum { ROLE_SENDER = 0, ROLE_RECEIVER = 1 };

/* ------------------------------------------------------------------ */
/* bf16 <-> fp32 from the format's definition (bf16 = upper half of fp32). */

static float bf16_to_float(uint16_t h)
{
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return f;
}

/* Round to nearest, ties to even, on the 16 dropped bits; NaN stays NaN. */
static uint16_t float_to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, sizeof u);
    if ((u & 0x7f800000u) == 0x7f800000u && (u & 0x007fffffu) != 0)
        return (uint16_t)((u >> 16) | 0x0040u);
    uint32_t lower = u & 0xffffu;
    uint32_t upper = u >> 16;
    if (lower > 0x8000u || (lower == 0x8000u && (upper & 1u)))
        upper += 1u;
    return (uint16_t)upper;
}

int oracle_qmax(int bits) { return (1 << (bits - 1)) - 1; }

/* ------------------------------------------------------------------ */
/* Code packing: two's complement b-bit fields, little-endian bit order. */

/* Both loops run over blocks of 8 elements, which fill whole bytes, so that the
 * blocks are independent (the OpenMP build splits them among threads; the
 * serial build ignores the pragmas). */
void oracle_pack_codes(int64_t n, int bits, const int8_t *q, uint8_t *codes)
{
    int64_t nbytes = n * bits / 8;
    uint8_t mask = (uint8_t)((1u << bits) - 1u);
    memset(codes, 0, (size_t)nbytes);
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < (n + 7) / 8; ++blk)
        for (int64_t j = 8 * blk; j < 8 * blk + 8 && j < n; ++j) {
            int64_t bit = j * bits;
            codes[bit / 8] |= (uint8_t)(((uint8_t)q[j] & mask) << (bit % 8));
        }
}

void oracle_unpack_codes(int64_t n, int bits, const uint8_t *codes, int8_t *q)
{
    uint32_t mask = (1u << bits) - 1u;
#pragma omp parallel for schedule(static)
    for (int64_t blk = 0; blk < (n + 7) / 8; ++blk)
        for (int64_t j = 8 * blk; j < 8 * blk + 8 && j < n; ++j) {
            int64_t bit = j * bits;
            int v = (int)((codes[bit / 8] >> (bit % 8)) & mask);
            if (v >= (1 << (bits - 1)))       /* sign bit set */
                v -= (1 << bits);
            q[j] = (int8_t)v;
        }
}

/* ------------------------------------------------------------------ */
/* Group-wise absmax quantizer for one group of `group` fp32 residuals.  */

static float quantize_group(const float *r, int group, int qmax, int8_t *q)
{
    float a = 0.0f;
    for (int i = 0; i < group; ++i) {
        float v = fabsf(r[i]);
        if (v > a)
            a = v;
    }
    float s = a / (float)qmax;
    for (int i = 0; i < group; ++i) {
        if (s == 0.0f) {
            q[i] = 0;
            continue;
        }
        float t = rintf(r[i] / s);
        if (t > (float)qmax)
            t = (float)qmax;
        if (t < (float)-qmax)
            t = (float)-qmax;
        q[i] = (int8_t)t;
    }
    return s;
}

/* Quantize an arbitrary fp32 array group by group (no state, no feedback). */
void oracle_quantize(int64_t n, int bits, int group, const float *r,
                     uint8_t *codes, float *scales)
{
    int qmax = oracle_qmax(bits);
    int8_t *q = (int8_t *)malloc((size_t)n);
    for (int64_t g = 0; g < n / group; ++g)
        scales[g] = quantize_group(r + g * group, group, qmax, q + g * group);
    oracle_pack_codes(n, bits, q, codes);
    free(q);
}

/* ------------------------------------------------------------------ */
/* State element access: fp32 arrays, or bf16 bit patterns when state_bf16. */

static float state_get(const void *p, int64_t j, int state_bf16)
{
    return state_bf16 ? bf16_to_float(((const uint16_t *)p)[j]) : ((const float *)p)[j];
}

static void state_set(void *p, int64_t j, float v, int state_bf16)
{
    if (state_bf16)
        ((uint16_t *)p)[j] = float_to_bf16(v);
    else
        ((float *)p)[j] = v;
}

/* ------------------------------------------------------------------ */
/* Warm-up (step 0): the uncompressed activation initialises the state.
 * x0 may be NULL, meaning an all-zero activation. */

void oracle_warmup(int64_t n, int mode, int role, int state_bf16, const uint16_t *x0,
                   uint16_t *prev, void *base, void *err)
{
    for (int64_t j = 0; j < n; ++j) {
        uint16_t h = x0 ? x0[j] : 0;
        if (role == ROLE_RECEIVER) {
            state_set(base, j, bf16_to_float(h), state_bf16);
            continue;
        }
        if (mode == MODE_DELTA || mode == MODE_OPENLOOP)
            prev[j] = h;
        if (mode == MODE_LITERAL || mode == MODE_OFF)
            state_set(base, j, bf16_to_float(h), state_bf16);
        if (mode == MODE_DELTA || mode == MODE_LITERAL)
            state_set(err, j, 0.0f, state_bf16);
    }
}

/* One compressed step at the sender.  Buffers not used by `mode` may be NULL. */
void oracle_compress(int64_t n, int bits, int group, int mode, int state_bf16,
                     const uint16_t *x, uint16_t *prev, void *base, void *err,
                     uint8_t *codes, float *scales)
{
    int qmax = oracle_qmax(bits);
    int8_t *q = (int8_t *)malloc((size_t)n);
#pragma omp parallel
    {
    float *r = (float *)malloc(sizeof(float) * (size_t)group);
#pragma omp for schedule(static)
    for (int64_t g = 0; g < n / group; ++g) {
        int64_t j0 = g * group;
        for (int i = 0; i < group; ++i) {
            int64_t j = j0 + i;
            float xj = bf16_to_float(x[j]);
            if (mode == MODE_DELTA)
                r[i] = (xj - bf16_to_float(prev[j])) + state_get(err, j, state_bf16);
            else if (mode == MODE_LITERAL)
                r[i] = (xj - state_get(base, j, state_bf16)) + state_get(err, j, state_bf16);
            else if (mode == MODE_OFF)
                r[i] = xj - state_get(base, j, state_bf16);
            else /* MODE_OPENLOOP */
                r[i] = xj - bf16_to_float(prev[j]);
        }
        float s = quantize_group(r, group, qmax, q + j0);
        scales[g] = s;
        for (int i = 0; i < group; ++i) {
            int64_t j = j0 + i;
            float qf = (float)q[j];
            if (mode == MODE_DELTA || mode == MODE_LITERAL)
                state_set(err, j, fmaf(-qf, s, r[i]), state_bf16);
            if (mode == MODE_DELTA || mode == MODE_OPENLOOP)
                prev[j] = x[j];
            if ((mode == MODE_LITERAL || mode == MODE_OFF) && q[j] != 0)
                state_set(base, j, fmaf(qf, s, state_get(base, j, state_bf16)), state_bf16);
        }
    }
    free(r);
    }
    oracle_pack_codes(n, bits, q, codes);
    free(q);
}

/* One step at the receiver: decode the payload and advance the base.
 * xhat (bf16 copy of the new base) may be NULL. */
void oracle_decompress(int64_t n, int bits, int group, int state_bf16, const uint8_t *codes,
                       const float *scales, void *base, uint16_t *xhat)
{
    int8_t *q = (int8_t *)malloc((size_t)n);
    oracle_unpack_codes(n, bits, codes, q);
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j) {
        if (q[j] != 0)
            state_set(base, j, fmaf((float)q[j], scales[j / group], state_get(base, j, state_bf16)),
                      state_bf16);
        if (xhat)
            xhat[j] = float_to_bf16(state_get(base, j, state_bf16));
    }
    free(q);
}

/* bf16 <-> fp32 conversions exposed for tests of the conversion itself. */
void oracle_bf16_to_f32(int64_t n, const uint16_t *h, float *f)
{
    for (int64_t j = 0; j < n; ++j)
        f[j] = bf16_to_float(h[j]);
}

void oracle_f32_to_bf16(int64_t n, const float *f, uint16_t *h)
{
    for (int64_t j = 0; j < n; ++j)
        h[j] = float_to_bf16(f[j]);
}

/* ------------------------------------------------------------------ */
/* Thin QR by Householder reflections (fp64), positive diagonal.
 * M: rows x cols, row-major.  Q: rows x cols.  R: cols x cols (upper).
 * Dropped columns (remaining squared norm <= 1e-13 ||M||_F^2 / cols, or not
 * finite) give a zero Q column and a zero R row and column. */

int oracle_qr(int64_t rows, int cols, const double *M, double *Q, double *R)
{
    double *W = (double *)malloc(sizeof(double) * (size_t)(rows * cols));
    double *V = (double *)calloc((size_t)(rows * cols), sizeof(double));
    int *prow = (int *)malloc(sizeof(int) * (size_t)cols);
    memcpy(W, M, sizeof(double) * (size_t)(rows * cols));

    double fro2 = 0.0;
    for (int64_t i = 0; i < rows * cols; ++i)
        fro2 += M[i] * M[i];
    double tol = 1e-13 * fro2 / cols;

    int p = 0; /* next reflection row */
    for (int k = 0; k < cols; ++k) {
        double norm2 = 0.0;
        for (int64_t i = p; i < rows; ++i)
            norm2 += W[i * cols + k] * W[i * cols + k];
        if (p >= rows || !(norm2 > tol) || !isfinite(norm2)) {
            prow[k] = -1;
            continue;
        }
        double x0 = W[(int64_t)p * cols + k];
        double alpha = -copysign(sqrt(norm2), x0);
        /* v = x - alpha e_p, stored in column p of V (rows p..) */
        double vnorm2 = 0.0;
        for (int64_t i = p; i < rows; ++i) {
            double vi = W[i * cols + k] - (i == p ? alpha : 0.0);
            V[i * cols + p] = vi;
            vnorm2 += vi * vi;
        }
        /* apply H = I - 2 v v^T / (v^T v) to columns k..cols-1 */
#pragma omp parallel for schedule(static)
        for (int j = k; j < cols; ++j) {
            double dot = 0.0;
            for (int64_t i = p; i < rows; ++i)
                dot += V[i * cols + p] * W[i * cols + j];
            double f = 2.0 * dot / vnorm2;
            for (int64_t i = p; i < rows; ++i)
                W[i * cols + j] -= f * V[i * cols + p];
        }
        prow[k] = p;
        ++p;
    }
    int nref = p;

    /* R: entry (i, j) is row prow[i] of the reflected column j, for live i and j >= i */
    for (int i = 0; i < cols; ++i)
        for (int j = 0; j < cols; ++j) {
            double v = 0.0;
            if (prow[i] >= 0 && prow[j] >= 0 && j >= i)
                v = W[(int64_t)prow[i] * cols + j];
            R[i * cols + j] = v;
        }

    /* Q column k = H_0 H_1 ... H_{nref-1} e_{prow[k]} */
#pragma omp parallel
    {
    double *e = (double *)malloc(sizeof(double) * (size_t)rows);
#pragma omp for schedule(static)
    for (int k = 0; k < cols; ++k) {
        if (prow[k] < 0) {
            for (int64_t i = 0; i < rows; ++i)
                Q[i * cols + k] = 0.0;
            continue;
        }
        for (int64_t i = 0; i < rows; ++i)
            e[i] = (i == prow[k]) ? 1.0 : 0.0;
        for (int h = nref - 1; h >= 0; --h) {
            double dot = 0.0, vn = 0.0;
            for (int64_t i = h; i < rows; ++i) {
                dot += V[i * cols + h] * e[i];
                vn += V[i * cols + h] * V[i * cols + h];
            }
            double f = 2.0 * dot / vn;
            for (int64_t i = h; i < rows; ++i)
                e[i] -= f * V[i * cols + h];
        }
        for (int64_t i = 0; i < rows; ++i)
            Q[i * cols + k] = e[i];
    }
    free(e);
    }

    /* sign convention: diag(R) > 0 */
    for (int k = 0; k < cols; ++k) {
        if (R[k * cols + k] < 0.0) {
            for (int j = 0; j < cols; ++j)
                R[k * cols + j] = -R[k * cols + j];
            for (int64_t i = 0; i < rows; ++i)
                Q[i * cols + k] = -Q[i * cols + k];
        }
    }
    free(prow);
    free(V);
    free(W);
    return cols - nref; /* number of dropped columns */
}

/* ------------------------------------------------------------------ */
/* Algorithm 3, rank r, T iterations, for one m x n bf16 matrix A.
 * Q0: n x r fp32 random sample.  Outputs (fp64): U m x r, V n x r, RU r x r. */

static void mat_AQ(int64_t m, int64_t n, int r, const double *A, const double *Q, double *Y)
{
#pragma omp parallel for schedule(static)
    for (int64_t i = 0; i < m; ++i)
        for (int c = 0; c < r; ++c) {
            double acc = 0.0;
            for (int64_t j = 0; j < n; ++j)
                acc += A[i * n + j] * Q[j * r + c];
            Y[i * r + c] = acc;
        }
}

static void mat_AtY(int64_t m, int64_t n, int r, const double *A, const double *Y, double *Z)
{
#pragma omp parallel for schedule(static)
    for (int64_t j = 0; j < n; ++j)
        for (int c = 0; c < r; ++c) {
            double acc = 0.0;
            for (int64_t i = 0; i < m; ++i)
                acc += A[i * n + j] * Y[i * r + c];
            Z[j * r + c] = acc;
        }
}

void oracle_lowrank(int64_t m, int64_t n, int r, int T, const uint16_t *A_bf16,
                    const float *Q0, double *U, double *V, double *RU)
{
    double *A = (double *)malloc(sizeof(double) * (size_t)(m * n));
    double *Q = (double *)malloc(sizeof(double) * (size_t)(n * r));
    double *Z = (double *)malloc(sizeof(double) * (size_t)(n * r));
    double *Y = (double *)malloc(sizeof(double) * (size_t)(m * r));
    double *Rt = (double *)malloc(sizeof(double) * (size_t)(r * r));
    for (int64_t i = 0; i < m * n; ++i)
        A[i] = (double)bf16_to_float(A_bf16[i]);
    for (int64_t i = 0; i < n * r; ++i)
        Z[i] = (double)Q0[i];

    /* step 1: orthonormalise the random sample */
    oracle_qr(n, r, Z, Q, Rt);
    /* steps 2-5: Z = A^T (A Q), Q = orth(Z) */
    for (int t = 0; t < T; ++t) {
        mat_AQ(m, n, r, A, Q, Y);
        mat_AtY(m, n, r, A, Y, Z);
        oracle_qr(n, r, Z, Q, Rt);
    }
    /* steps 6-8: U = orth(A Q) with its triangular factor, V = Q */
    mat_AQ(m, n, r, A, Q, Y);
    oracle_qr(m, r, Y, U, RU);
    memcpy(V, Q, sizeof(double) * (size_t)(n * r));

    free(Rt);
    free(Y);
    free(Z);
    free(Q);
    free(A);
}

/* ------------------------------------------------------------------ */
/* The rank-r compressor inside the error-feedback loop.  The pages give
 * error feedback on step-wise differences as the method and the subspace
 * iteration (Algorithm 3) as a compressor; they are combined here the way the
 * quantizer is used: the DELTA-mode residual is rounded to bf16 (the input
 * type of the subspace iteration), compressed to (U, R_U, V), and what the
 * reconstruction misses is carried to the next step.
 *
 * Sender, one step, for one m x n tensor:
 *   r = (x - prev) + err          fp32, as in the quantizer's DELTA mode
 *   A = bf16(r)                   round to nearest even
 *   (U, V, R_U) = Algorithm 3 on A with the random sample Q0
 *   D = (U R_U) V^T               fp64
 *   err' = fp32(r - D), prev' = x
 * Receiver: base' = fp32(base + D), xhat = bf16(base').
 * The warm-up is the quantizer's DELTA warm-up (prev = x0, err = 0; base = x0).
 * Plain additions: a zero D leaves every value unchanged (a -0 base may become
 * +0). */

/* Y = fp32(Y + sign * (U R_U) V^T), every element from its fp64 sum. */
void oracle_lowrank_ef_update(int64_t m, int64_t n, int r, const double *U, const double *V,
                              const double *RU, double sign, float *Y)
{
    double *W = (double *)malloc(sizeof(double) * (size_t)(m * r));
    for (int64_t i = 0; i < m; ++i)
        for (int k = 0; k < r; ++k) {
            double acc = 0.0;
            for (int l = 0; l < r; ++l)
                acc += U[i * r + l] * RU[l * r + k];
            W[i * r + k] = acc;
        }
    for (int64_t i = 0; i < m; ++i)
        for (int64_t j = 0; j < n; ++j) {
            double d = 0.0;
            for (int k = 0; k < r; ++k)
                d += W[i * r + k] * V[j * r + k];
            Y[i * n + j] = (float)((double)Y[i * n + j] + sign * d);
        }
    free(W);
}

/* Sender step.  A (m x n bf16, the compressed residual) may be NULL. */
void oracle_lowrank_ef_compress(int64_t m, int64_t n, int r, int T, const uint16_t *x,
                                uint16_t *prev, float *err, const float *Q0, uint16_t *A,
                                double *U, double *V, double *RU)
{
    uint16_t *a = A ? A : (uint16_t *)calloc((size_t)(m * n), sizeof(uint16_t));
    for (int64_t j = 0; j < m * n; ++j) {
        float rj = (bf16_to_float(x[j]) - bf16_to_float(prev[j])) + err[j];
        err[j] = rj;
        a[j] = float_to_bf16(rj);
        prev[j] = x[j];
    }
    oracle_lowrank(m, n, r, T, a, Q0, U, V, RU);
    oracle_lowrank_ef_update(m, n, r, U, V, RU, -1.0, err);
    if (!A)
        free(a);
}

/* Receiver step.  xhat (bf16 copy of the new base) may be NULL. */
void oracle_lowrank_ef_decompress(int64_t m, int64_t n, int r, const double *U, const double *V,
                                  const double *RU, float *base, uint16_t *xhat)
{
    oracle_lowrank_ef_update(m, n, r, U, V, RU, 1.0, base);
    if (xhat)
        for (int64_t j = 0; j < m * n; ++j)
            xhat[j] = float_to_bf16(base[j]);
}

int oracle_abi_version(void) { return 2; }

/* Threads the loops above may use: 1 in the serial build, OpenMP's count (all
 * cores unless OMP_NUM_THREADS says otherwise) in the OpenMP build. */
#ifdef _OPENMP
#include <omp.h>
int oracle_threads(void) { return omp_get_max_threads(); }
#else
int oracle_threads(void) { return 1; }
#endif
