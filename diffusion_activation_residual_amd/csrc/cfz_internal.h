// cfz_internal.h -- declarations shared by the sources of libcfz only.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace cfz {

enum { kDelta = 0, kLiteral = 1, kOff = 2 };

constexpr int kMaxGroup = 16;  // tensors per codec launch

struct CompressItem {
    const uint16_t *x;
    uint16_t *prev;
    void *base;  // fp32 or bf16 per the state precision
    void *err;
    uint8_t *codes;
    float *scales;
    int64_t n;  // elements, a multiple of the group size
};

struct DecodeItem {
    const uint8_t *codes;
    const float *scales;
    void *base;
    uint16_t *xhat;  // may be null
    int64_t n;
};

// Any count: tensors are launched kMaxGroup at a time; empty tensors are skipped.
hipError_t launch_compress(const CompressItem *items, int count, int bits, int group, int mode,
                           bool state_bf16, hipStream_t st);
hipError_t launch_decode(const DecodeItem *items, int count, int bits, int group, bool state_bf16,
                         hipStream_t st);
hipError_t launch_warmup(const uint16_t *x0, uint16_t *prev, void *base, void *err,
                         bool state_bf16, int64_t nchunks, hipStream_t st);
hipError_t launch_stream_copy(const void *src, void *dst, int64_t nvec, hipStream_t st);
hipError_t launch_stream_mix(const void *src, void *dst, int64_t nr, int64_t nw, hipStream_t st);

struct LowrankArgs {
    int64_t batch, m, n;
    int r, T;
    const uint16_t *A;
    const float *Q0;
    float *U, *V, *RU;
    void *ws;
};
size_t lowrank_workspace_bytes(int64_t batch, int64_t m, int64_t n, int r);
hipError_t launch_lowrank(const LowrankArgs &a, hipStream_t st);

// rank-r compressor inside the error-feedback loop
hipError_t launch_lowrank_ef_residual(const uint16_t *x, uint16_t *prev, float *err, uint16_t *A,
                                      int64_t count, hipStream_t st);
hipError_t launch_lowrank_ef_update(int64_t batch, int64_t m, int64_t n, int r, const float *U,
                                    const float *V, const float *RU, float sign, float *Y,
                                    uint16_t *xhat, hipStream_t st);
// the sender's pending update e = r0 - (U R_U) V^T fused into the next residual pass:
// err (holding r0) becomes (x - prev) + e, prev becomes x, A bf16 of the new residual
hipError_t launch_lowrank_ef_residual_update(int64_t batch, int64_t m, int64_t n, int r,
                                             const float *U, const float *V, const float *RU,
                                             const uint16_t *x, uint16_t *prev, float *err,
                                             uint16_t *A, hipStream_t st);
int64_t lowrank_ef_update_blocks(int64_t batch, int64_t m, int64_t n);

}  // namespace cfz
