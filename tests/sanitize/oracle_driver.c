/*
 * Drives every entry point of the CPU oracle (oracle/cfz_oracle.c) on small,
 * ragged inputs so that a build with AddressSanitizer and
 * UndefinedBehaviorSanitizer sees each code path: packing, the quantizer, all
 * error-feedback modes with fp32 and bf16 state, the QR, the subspace
 * iteration (including a zero matrix and T = 0) and the low-rank
 * error-feedback steps.  Test infrastructure only.  Prints "OK" on success;
 * a sanitizer report aborts the process with a non-zero status.
 */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

void oracle_pack_codes(int64_t n, int bits, const int8_t *q, uint8_t *codes);
void oracle_unpack_codes(int64_t n, int bits, const uint8_t *codes, int8_t *q);
void oracle_quantize(int64_t n, int bits, int group, const float *r, uint8_t *codes, float *scales);
void oracle_warmup(int64_t n, int mode, int role, int state_bf16, const uint16_t *x0,
                   uint16_t *prev, void *base, void *err);
void oracle_compress(int64_t n, int bits, int group, int mode, int state_bf16, const uint16_t *x,
                     uint16_t *prev, void *base, void *err, uint8_t *codes, float *scales);
void oracle_decompress(int64_t n, int bits, int group, int state_bf16, const uint8_t *codes,
                       const float *scales, void *base, uint16_t *xhat);
void oracle_f32_to_bf16(int64_t n, const float *f, uint16_t *h);
int oracle_qr(int64_t rows, int cols, const double *M, double *Q, double *R);
void oracle_lowrank(int64_t m, int64_t n, int r, int T, const uint16_t *A_bf16, const float *Q0,
                    double *U, double *V, double *RU);
void oracle_lowrank_ef_compress(int64_t m, int64_t n, int r, int T, const uint16_t *x,
                                uint16_t *prev, float *err, const float *Q0, uint16_t *A,
                                double *U, double *V, double *RU);
void oracle_lowrank_ef_decompress(int64_t m, int64_t n, int r, const double *U, const double *V,
                                  const double *RU, float *base, uint16_t *xhat);

static uint64_t rng_state = 0x9e3779b97f4a7c15ull;

static float uniform(void) /* splitmix64 -> [-1, 1) */
{
    uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
    z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
    z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
    z ^= z >> 31;
    return (float)((double)(z >> 11) / 9007199254740992.0 * 2.0 - 1.0);
}

static void fill_bf16(int64_t n, uint16_t *h, float scale)
{
    float *f = malloc(sizeof(float) * (size_t)n);
    for (int64_t i = 0; i < n; ++i)
        f[i] = uniform() * scale;
    oracle_f32_to_bf16(n, f, h);
    free(f);
}

static int codec_paths(void)
{
    const int64_t n = 8 * 40; /* 320 elements: ragged for G = 64 */
    const int bits_list[2] = {4, 2};
    const int groups[3] = {8, 32, 64};
    int8_t q[320], q2[320];
    uint8_t codes[160];
    float scales[40], r[320];
    for (int b = 0; b < 2; ++b) {
        const int bits = bits_list[b], qmax = (1 << (bits - 1)) - 1;
        for (int64_t i = 0; i < n; ++i)
            q[i] = (int8_t)((i % (2 * qmax + 1)) - qmax);
        oracle_pack_codes(n, bits, q, codes);
        oracle_unpack_codes(n, bits, codes, q2);
        if (memcmp(q, q2, (size_t)n) != 0)
            return 1;
        for (int g = 0; g < 3; ++g) {
            if (n % groups[g])
                continue;
            for (int64_t i = 0; i < n; ++i)
                r[i] = uniform();
            oracle_quantize(n, bits, groups[g], r, codes, scales);
        }
    }
    for (int sb = 0; sb < 2; ++sb)
        for (int mode = 0; mode < 4; ++mode)
            for (int b = 0; b < 2; ++b) {
                const int bits = bits_list[b], group = 32;
                const size_t w = sb ? 2 : 4;
                uint16_t *x = malloc(2 * (size_t)n), *prev = malloc(2 * (size_t)n);
                void *base = malloc(w * (size_t)n), *err = malloc(w * (size_t)n);
                void *rbase = malloc(w * (size_t)n);
                uint16_t *xhat = malloc(2 * (size_t)n);
                fill_bf16(n, x, 3.0f);
                oracle_warmup(n, mode, 0, sb, x, prev, base, err);
                oracle_warmup(n, 0, 1, sb, x, NULL, rbase, NULL);
                for (int t = 0; t < 3; ++t) {
                    fill_bf16(n, x, 3.0f);
                    oracle_compress(n, bits, group, mode, sb, x, prev, base, err, codes, scales);
                    oracle_decompress(n, bits, group, sb, codes, scales, rbase, xhat);
                }
                oracle_warmup(n, mode, 0, sb, NULL, prev, base, err); /* x0 == NULL: zeros */
                free(x), free(prev), free(base), free(err), free(rbase), free(xhat);
            }
    return 0;
}

static int lowrank_paths(void)
{
    const int64_t m = 24, n = 40;
    const int r = 5;
    uint16_t *A = malloc(2 * (size_t)(m * n)), *x = malloc(2 * (size_t)(m * n));
    uint16_t *prev = calloc((size_t)(m * n), 2), *Ares = malloc(2 * (size_t)(m * n));
    uint16_t *xhat = malloc(2 * (size_t)(m * n));
    float *Q0 = malloc(sizeof(float) * (size_t)(n * r)), *err = calloc((size_t)(m * n), 4);
    float *base = calloc((size_t)(m * n), 4);
    double *U = malloc(sizeof(double) * (size_t)(m * r)), *V = malloc(sizeof(double) * (size_t)(n * r));
    double *RU = malloc(sizeof(double) * (size_t)(r * r));
    double *M = malloc(sizeof(double) * (size_t)(n * r)), *Q = malloc(sizeof(double) * (size_t)(n * r));
    double *R = malloc(sizeof(double) * (size_t)(r * r));
    for (int64_t i = 0; i < n * r; ++i)
        Q0[i] = uniform();
    for (int64_t i = 0; i < n * r; ++i)
        M[i] = (i % r == 2) ? 0.0 : (double)uniform(); /* one zero column: dropped */
    if (oracle_qr(n, r, M, Q, R) != 1)
        return 1;
    fill_bf16(m * n, A, 2.0f);
    for (int T = 0; T < 3; ++T)
        oracle_lowrank(m, n, r, T, A, Q0, U, V, RU);
    memset(A, 0, 2 * (size_t)(m * n)); /* zero matrix: every column dropped */
    oracle_lowrank(m, n, r, 2, A, Q0, U, V, RU);
    for (int t = 0; t < 3; ++t) {
        fill_bf16(m * n, x, 2.0f);
        oracle_lowrank_ef_compress(m, n, r, 1, x, prev, err, Q0, t ? Ares : NULL, U, V, RU);
        oracle_lowrank_ef_decompress(m, n, r, U, V, RU, base, t ? xhat : NULL);
    }
    free(A), free(x), free(prev), free(Ares), free(xhat), free(Q0), free(err), free(base);
    free(U), free(V), free(RU), free(M), free(Q), free(R);
    return 0;
}

int main(void)
{
    if (codec_paths() != 0) {
        fprintf(stderr, "codec round trip failed\n");
        return 2;
    }
    if (lowrank_paths() != 0) {
        fprintf(stderr, "low-rank checks failed\n");
        return 3;
    }
    printf("OK\n");
    return 0;
}
