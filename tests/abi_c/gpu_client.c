/*
 * Plain C11 client of include/cfz.h that runs the codec on the GPU: device
 * memory from the HIP runtime API, every call through the C ABI of libcfz.so,
 * no Python and no torch.  Each step's codes, scales, sender state, receiver
 * base and bf16 output are copied back and compared byte for byte with the CPU
 * oracle (oracle/libcfz_oracle.so, test infrastructure) run on the same inputs;
 * cfz_lowrank's reconstruction is compared with the oracle's fp64 one, and the
 * deferred low-rank error-feedback sender with the plain one.  Prints
 * one line per case before its GPU work, and "OK" at the end.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "cfz.h"

/* the oracle's entry points (oracle/cfz_oracle.c) */
void oracle_warmup(int64_t n, int mode, int role, int state_bf16, const uint16_t *x0,
                   uint16_t *prev, void *base, void *err);
void oracle_compress(int64_t n, int bits, int group, int mode, int state_bf16, const uint16_t *x,
                     uint16_t *prev, void *base, void *err, uint8_t *codes, float *scales);
void oracle_decompress(int64_t n, int bits, int group, int state_bf16, const uint8_t *codes,
                       const float *scales, void *base, uint16_t *xhat);
void oracle_lowrank(int64_t m, int64_t n, int r, int T, const uint16_t *A_bf16, const float *Q0,
                    double *U, double *V, double *RU);

#define FAIL(...)                                                        \
    do {                                                                 \
        fprintf(stderr, "%s:%d: ", __FILE__, __LINE__);                  \
        fprintf(stderr, __VA_ARGS__);                                    \
        fprintf(stderr, "\n");                                           \
        return 1;                                                        \
    } while (0)
#define HIP(call)                                                        \
    do {                                                                 \
        hipError_t e_ = (call);                                          \
        if (e_ != hipSuccess)                                            \
            FAIL("%s: %s", #call, hipGetErrorString(e_));                \
    } while (0)
#define CFZ(call)                                                        \
    do {                                                                 \
        cfz_status s_ = (call);                                          \
        if (s_ != CFZ_OK)                                                \
            FAIL("%s: %s (%s)", #call, cfz_status_string(s_), cfz_last_error()); \
    } while (0)

enum { ROWS = 48, COLS = 384, N = ROWS * COLS, STEPS = 4 };  /* COLS: a multiple of every group size used */

static uint32_t lcg(uint32_t *s)
{
    *s = *s * 1664525u + 1013904223u;
    return *s;
}

/* fp32 -> bf16, round to nearest even (finite inputs) */
static uint16_t to_bf16(float f)
{
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

/* STEPS + 1 activations, each a small random walk step from the last */
static void make_inputs(uint16_t *x, uint32_t seed)
{
    float cur[N];
    for (int j = 0; j < N; ++j)
        cur[j] = ((float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f) * 4.0f;
    for (int t = 0; t <= STEPS; ++t) {
        for (int j = 0; j < N; ++j) {
            if (t > 0)
                cur[j] += ((float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f) * 0.25f;
            x[t * N + j] = to_bf16(cur[j]);
        }
    }
}

static int run_case(int bits, int group, int mode, int state_bf16, const uint16_t *x)
{
    printf("case bits=%d group=%d mode=%d state_bf16=%d\n", bits, group, mode, state_bf16);
    fflush(stdout);
    const size_t w = state_bf16 ? 2 : 4, nc = (size_t)N * bits / 8, ns = N / group;
    cfz_desc sd, rd;
    memset(&sd, 0, sizeof sd);
    sd.rows = ROWS;
    sd.cols = COLS;
    sd.bits = bits;
    sd.group = group;
    sd.ef_mode = mode;
    sd.role = CFZ_SENDER;
    sd.state_dtype = state_bf16 ? CFZ_STATE_BF16 : CFZ_STATE_F32;
    rd = sd;
    rd.ef_mode = CFZ_EF_DELTA;
    rd.role = CFZ_RECEIVER;
    if (cfz_codes_bytes(&sd) != nc || cfz_scales_bytes(&sd) != ns * 4)
        FAIL("payload sizes");

    void *d_x, *d_prev, *d_base, *d_err, *d_codes, *d_scales, *d_rbase, *d_xhat;
    HIP(hipMalloc(&d_x, 2 * N));
    HIP(hipMalloc(&d_prev, 2 * N));
    HIP(hipMalloc(&d_base, w * N));
    HIP(hipMalloc(&d_err, w * N));
    HIP(hipMalloc(&d_codes, nc));
    HIP(hipMalloc(&d_scales, ns * 4));
    HIP(hipMalloc(&d_rbase, w * N));
    HIP(hipMalloc(&d_xhat, 2 * N));

    /* host copies: oracle state and what comes back from the device */
    static uint16_t o_prev[N], o_xhat[N], g_prev[N], g_xhat[N];
    static uint8_t o_base[4 * N], o_err[4 * N], o_rbase[4 * N], g_base[4 * N], g_err[4 * N],
        g_rbase[4 * N], o_codes[N], g_codes[N];
    static float o_scales[N], g_scales[N];

    cfz_buffers sb, rb;
    sb.prev_bf16 = (uint16_t *)d_prev;
    sb.base = d_base;
    sb.err = d_err;
    rb.prev_bf16 = NULL;
    rb.base = d_rbase;
    rb.err = NULL;
    HIP(hipMemcpy(d_x, x, 2 * N, hipMemcpyHostToDevice));
    cfz_state *snd = NULL, *rcv = NULL;
    CFZ(cfz_state_create(&sd, &sb, (const uint16_t *)d_x, NULL, &snd));
    CFZ(cfz_state_create(&rd, &rb, (const uint16_t *)d_x, NULL, &rcv));
    oracle_warmup(N, mode, CFZ_SENDER, state_bf16, x, o_prev, o_base, o_err);
    oracle_warmup(N, CFZ_EF_DELTA, CFZ_RECEIVER, state_bf16, x, NULL, o_rbase, NULL);

    for (int t = 1; t <= STEPS; ++t) {
        const uint16_t *xt = x + (size_t)t * N;
        HIP(hipMemcpy(d_x, xt, 2 * N, hipMemcpyHostToDevice));
        CFZ(cfz_compress(snd, (const uint16_t *)d_x, (uint8_t *)d_codes, (float *)d_scales, NULL));
        CFZ(cfz_decompress(rcv, (const uint8_t *)d_codes, (const float *)d_scales,
                           (uint16_t *)d_xhat, NULL));
        HIP(hipDeviceSynchronize());
        oracle_compress(N, bits, group, mode, state_bf16, xt, o_prev, o_base, o_err, o_codes,
                        o_scales);
        oracle_decompress(N, bits, group, state_bf16, o_codes, o_scales, o_rbase, o_xhat);

        HIP(hipMemcpy(g_codes, d_codes, nc, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g_scales, d_scales, ns * 4, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g_rbase, d_rbase, w * N, hipMemcpyDeviceToHost));
        HIP(hipMemcpy(g_xhat, d_xhat, 2 * N, hipMemcpyDeviceToHost));
        if (memcmp(g_codes, o_codes, nc) || memcmp(g_scales, o_scales, ns * 4))
            FAIL("step %d: payload differs from the oracle", t);
        if (memcmp(g_rbase, o_rbase, w * N) || memcmp(g_xhat, o_xhat, 2 * N))
            FAIL("step %d: receiver base or bf16 output differs from the oracle", t);
        if (mode == CFZ_EF_DELTA) {
            HIP(hipMemcpy(g_prev, d_prev, 2 * N, hipMemcpyDeviceToHost));
            if (memcmp(g_prev, o_prev, 2 * N))
                FAIL("step %d: prev differs", t);
        } else {
            HIP(hipMemcpy(g_base, d_base, w * N, hipMemcpyDeviceToHost));
            if (memcmp(g_base, o_base, w * N))
                FAIL("step %d: sender base differs", t);
        }
        if (mode != CFZ_EF_OFF) {
            HIP(hipMemcpy(g_err, d_err, w * N, hipMemcpyDeviceToHost));
            if (memcmp(g_err, o_err, w * N))
                FAIL("step %d: carried error differs", t);
        }
    }
    if (cfz_state_steps(snd) != STEPS || cfz_state_steps(rcv) != STEPS)
        FAIL("step counters");
    CFZ(cfz_state_destroy(snd));
    CFZ(cfz_state_destroy(rcv));
    HIP(hipFree(d_x));
    HIP(hipFree(d_prev));
    HIP(hipFree(d_base));
    HIP(hipFree(d_err));
    HIP(hipFree(d_codes));
    HIP(hipFree(d_scales));
    HIP(hipFree(d_rbase));
    HIP(hipFree(d_xhat));
    return 0;
}

/* (U R_U) V^T of one matrix, fp64, from fp32 or fp64 factors */
static void reconstruct(int m, int n, int r, const double *U, const double *V, const double *RU,
                        double *D)
{
    for (int i = 0; i < m; ++i)
        for (int j = 0; j < n; ++j) {
            double acc = 0.0;
            for (int k = 0; k < r; ++k) {
                double ur = 0.0;
                for (int l = 0; l < r; ++l)
                    ur += U[i * r + l] * RU[l * r + k];
                acc += ur * V[j * r + k];
            }
            D[i * n + j] = acc;
        }
}

/* cfz_lowrank on a batch of rank-r + noise matrices (r = 8, so the subspace is well defined): the reconstruction U R_U V^T of every
 * matrix within 1e-3 (relative Frobenius) of the oracle's fp64 one */
static int run_lowrank(void)
{
    enum { B = 3, M = 64, NN = 128, R = 8, T = 2 };
    printf("case lowrank batch=%d m=%d n=%d r=%d T=%d\n", B, M, NN, R, T);
    fflush(stdout);
    static uint16_t A[B * M * NN];
    static float Q0[B * NN * R], U[B * M * R], V[B * NN * R], RU[B * R * R];
    static double Uo[M * R], Vo[NN * R], RUo[R * R], Ug[M * R], Vg[NN * R], RUg[R * R];
    static double Do[M * NN], Dg[M * NN];
    uint32_t seed = 77u;
    for (int b = 0; b < B; ++b) {
        float f[M * R], g[NN * R];
        for (int i = 0; i < M * R; ++i)
            f[i] = (float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f;
        for (int i = 0; i < NN * R; ++i)
            g[i] = (float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f;
        for (int i = 0; i < M; ++i)
            for (int j = 0; j < NN; ++j) {
                float a = 0.01f * ((float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f);
                for (int k = 0; k < R; ++k)
                    a += f[i * R + k] * g[j * R + k];
                A[(b * M + i) * NN + j] = to_bf16(a);
            }
    }
    for (int i = 0; i < B * NN * R; ++i)
        Q0[i] = (float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f;

    const size_t ws_bytes = cfz_lowrank_workspace_bytes(B, M, NN, R);
    if (ws_bytes == 0)
        FAIL("workspace size");
    void *dA, *dQ0, *dU, *dV, *dRU, *dws;
    HIP(hipMalloc(&dA, sizeof A));
    HIP(hipMalloc(&dQ0, sizeof Q0));
    HIP(hipMalloc(&dU, sizeof U));
    HIP(hipMalloc(&dV, sizeof V));
    HIP(hipMalloc(&dRU, sizeof RU));
    HIP(hipMalloc(&dws, ws_bytes));
    HIP(hipMemcpy(dA, A, sizeof A, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dQ0, Q0, sizeof Q0, hipMemcpyHostToDevice));
    if (cfz_lowrank(B, M, NN, R, T, (const uint16_t *)dA, (const float *)dQ0, (float *)dU,
                    (float *)dV, (float *)dRU, dws, ws_bytes - 1, NULL) != CFZ_ERR_WORKSPACE)
        FAIL("a short workspace must be refused");
    CFZ(cfz_lowrank(B, M, NN, R, T, (const uint16_t *)dA, (const float *)dQ0, (float *)dU,
                    (float *)dV, (float *)dRU, dws, ws_bytes, NULL));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(U, dU, sizeof U, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(V, dV, sizeof V, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(RU, dRU, sizeof RU, hipMemcpyDeviceToHost));
    for (int b = 0; b < B; ++b) {
        oracle_lowrank(M, NN, R, T, A + (size_t)b * M * NN, Q0 + (size_t)b * NN * R, Uo, Vo, RUo);
        for (int i = 0; i < M * R; ++i)
            Ug[i] = U[b * M * R + i];
        for (int i = 0; i < NN * R; ++i)
            Vg[i] = V[b * NN * R + i];
        for (int i = 0; i < R * R; ++i)
            RUg[i] = RU[b * R * R + i];
        reconstruct(M, NN, R, Uo, Vo, RUo, Do);
        reconstruct(M, NN, R, Ug, Vg, RUg, Dg);
        double num = 0.0, den = 0.0;
        for (int i = 0; i < M * NN; ++i) {
            num += (Dg[i] - Do[i]) * (Dg[i] - Do[i]);
            den += Do[i] * Do[i];
        }
        const double rel = sqrt(num / den);
        printf("  matrix %d: reconstruction within %.2e of the oracle\n", b, rel);
        if (!(rel <= 1e-3))
            FAIL("matrix %d: reconstruction differs from the oracle by %.3e", b, rel);
    }
    HIP(hipFree(dA));
    HIP(hipFree(dQ0));
    HIP(hipFree(dU));
    HIP(hipFree(dV));
    HIP(hipFree(dRU));
    HIP(hipFree(dws));
    return 0;
}

/* The rank-r compressor inside error feedback from C: a plain sender
 * (cfz_lowrank_ef_compress) and a deferred one (cfz_lowrank_ef_compress_deferred,
 * then cfz_lowrank_ef_flush) on the same inputs, each with its receiver, the
 * previous step's V as Q0 from the second step on.  After every step the factors,
 * prev and the receivers' base and bf16 output agree bit for bit; after the flush
 * so does err. */
static int run_lowrank_ef(void)
{
    enum { B = 2, M = 64, NN = 128, R = 8, T = 2, S = 4, E = B * M * NN };
    printf("case lowrank-ef batch=%d m=%d n=%d r=%d T=%d steps=%d, plain and deferred\n", B, M, NN,
           R, T, S);
    fflush(stdout);
    static uint16_t x[(S + 1) * E];
    static float Q0[B * NN * R];
    uint32_t seed = 91u;
    float drift[M * R], dir[NN * R];
    for (int i = 0; i < M * R; ++i)
        drift[i] = (float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f;
    for (int t = 0; t <= S; ++t) {
        for (int i = 0; i < NN * R; ++i)
            dir[i] = (float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f;
        for (int b = 0; b < B; ++b)
            for (int i = 0; i < M; ++i)
                for (int j = 0; j < NN; ++j) {
                    float a = 0.05f * ((float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f);
                    for (int k = 0; k < R; ++k)
                        a += 0.1f * (float)t * drift[i * R + k] * dir[j * R + k];
                    x[(size_t)t * E + (b * M + i) * NN + j] = to_bf16(a + (float)(b + 1));
                }
    }
    for (int i = 0; i < B * NN * R; ++i)
        Q0[i] = (float)(lcg(&seed) >> 8) / 16777216.0f - 0.5f;

    const size_t ws_bytes = cfz_lowrank_ef_workspace_bytes(B, M, NN, R);
    if (ws_bytes == 0)
        FAIL("workspace size");
    /* [0]: plain sender and its receiver, [1]: deferred */
    void *dx, *dQ0, *prev[2], *err[2], *U[2], *V[2], *RU[2], *ws[2], *base[2], *xhat[2];
    HIP(hipMalloc(&dx, sizeof x));
    HIP(hipMalloc(&dQ0, sizeof Q0));
    HIP(hipMemcpy(dx, x, sizeof x, hipMemcpyHostToDevice));
    HIP(hipMemcpy(dQ0, Q0, sizeof Q0, hipMemcpyHostToDevice));
    for (int k = 0; k < 2; ++k) {
        HIP(hipMalloc(&prev[k], 2 * E));
        HIP(hipMalloc(&err[k], 4 * E));
        HIP(hipMalloc(&U[k], 4 * B * M * R));
        HIP(hipMalloc(&V[k], 4 * B * NN * R));
        HIP(hipMalloc(&RU[k], 4 * B * R * R));
        HIP(hipMalloc(&ws[k], ws_bytes));
        HIP(hipMalloc(&base[k], 4 * E));
        HIP(hipMalloc(&xhat[k], 2 * E));
        CFZ(cfz_lowrank_ef_warmup(E, (const uint16_t *)dx, (uint16_t *)prev[k], (float *)err[k],
                                  (float *)base[k], NULL));
    }
    if (cfz_lowrank_ef_compress_deferred(B, M, NN, R, T, 2, (const uint16_t *)dx,
                                         (uint16_t *)prev[1], (float *)err[1],
                                         (const float *)dQ0, (float *)U[1], (float *)V[1],
                                         (float *)RU[1], ws[1], ws_bytes, NULL) != CFZ_ERR_SHAPE)
        FAIL("pending = 2 must be refused");
    if (cfz_lowrank_ef_flush(B, M, NN, R, (const float *)U[1], (const float *)V[1],
                             (const float *)RU[1], NULL, NULL) != CFZ_ERR_NULL)
        FAIL("a flush without err must be refused");
    static unsigned char h0[4 * E], h1[4 * E];
    for (int t = 1; t <= S; ++t) {
        const uint16_t *xt = (const uint16_t *)dx + (size_t)t * E;
        for (int k = 0; k < 2; ++k) {
            const float *q0 = t == 1 ? (const float *)dQ0 : (const float *)V[k];
            if (k == 0)
                CFZ(cfz_lowrank_ef_compress(B, M, NN, R, T, xt, (uint16_t *)prev[k],
                                            (float *)err[k], q0, (float *)U[k], (float *)V[k],
                                            (float *)RU[k], ws[k], ws_bytes, NULL));
            else
                CFZ(cfz_lowrank_ef_compress_deferred(B, M, NN, R, T, t > 1, xt,
                                                     (uint16_t *)prev[k], (float *)err[k], q0,
                                                     (float *)U[k], (float *)V[k], (float *)RU[k],
                                                     ws[k], ws_bytes, NULL));
            CFZ(cfz_lowrank_ef_decompress(B, M, NN, R, (const float *)U[k], (const float *)V[k],
                                          (const float *)RU[k], (float *)base[k],
                                          (uint16_t *)xhat[k], NULL));
        }
        HIP(hipDeviceSynchronize());
        const struct { void **p; size_t bytes; const char *name; } cmp[] = {
            {U, 4 * B * M * R, "U"}, {V, 4 * B * NN * R, "V"}, {RU, 4 * B * R * R, "RU"},
            {prev, 2 * E, "prev"}, {base, 4 * E, "base"}, {xhat, 2 * E, "xhat"}};
        for (size_t c = 0; c < sizeof cmp / sizeof cmp[0]; ++c) {
            HIP(hipMemcpy(h0, cmp[c].p[0], cmp[c].bytes, hipMemcpyDeviceToHost));
            HIP(hipMemcpy(h1, cmp[c].p[1], cmp[c].bytes, hipMemcpyDeviceToHost));
            if (memcmp(h0, h1, cmp[c].bytes) != 0)
                FAIL("step %d: %s of the deferred sender differs from the plain one", t,
                     cmp[c].name);
        }
    }
    CFZ(cfz_lowrank_ef_flush(B, M, NN, R, (const float *)U[1], (const float *)V[1],
                             (const float *)RU[1], (float *)err[1], NULL));
    HIP(hipDeviceSynchronize());
    HIP(hipMemcpy(h0, err[0], 4 * E, hipMemcpyDeviceToHost));
    HIP(hipMemcpy(h1, err[1], 4 * E, hipMemcpyDeviceToHost));
    if (memcmp(h0, h1, 4 * E) != 0)
        FAIL("err after the flush differs from the plain sender's");
    printf("  %d steps bit-identical, err after the flush too\n", S);
    for (int k = 0; k < 2; ++k) {
        HIP(hipFree(prev[k]));
        HIP(hipFree(err[k]));
        HIP(hipFree(U[k]));
        HIP(hipFree(V[k]));
        HIP(hipFree(RU[k]));
        HIP(hipFree(ws[k]));
        HIP(hipFree(base[k]));
        HIP(hipFree(xhat[k]));
    }
    HIP(hipFree(dx));
    HIP(hipFree(dQ0));
    return 0;
}

int main(void)
{
    static uint16_t x[(STEPS + 1) * N];
    make_inputs(x, 2024u);
    if (cfz_abi_version() != CFZ_ABI_VERSION) {
        fprintf(stderr, "ABI version mismatch\n");
        return 1;
    }
    const int cases[][4] = {
        {4, 64, CFZ_EF_DELTA, 0}, {2, 32, CFZ_EF_DELTA, 0}, {4, 64, CFZ_EF_DELTA, 1},
        {4, 32, CFZ_EF_LITERAL, 0}, {2, 64, CFZ_EF_OFF, 0}, {4, 128, CFZ_EF_OFF, 1},
    };
    for (size_t i = 0; i < sizeof cases / sizeof cases[0]; ++i)
        if (run_case(cases[i][0], cases[i][1], cases[i][2], cases[i][3], x))
            return 1;
    if (run_lowrank())
        return 1;
    if (run_lowrank_ef())
        return 1;
    printf("OK\n");
    return 0;
}
