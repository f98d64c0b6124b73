// cfz_api.hip -- the C ABI of libcfz: argument validation, state handles,
// status strings and kernel dispatch.  Nothing here touches the device until
// every argument has been checked; a non-OK status means nothing was enqueued.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <mutex>
#include <new>

#include "cfz.h"
#include "cfz_internal.h"

namespace {

constexpr uint32_t kMagic = 0x43465a31u;  // "CFZ1"

thread_local char g_last_error[512] = "";

cfz_status fail(cfz_status st, const char *fmt, ...) __attribute__((format(printf, 2, 3)));
cfz_status fail(cfz_status st, const char *fmt, ...)
{
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
    va_end(ap);
    return st;
}

// Re-labels the current error text with the group entry it came from.
cfz_status fail_entry(cfz_status st, int32_t i)
{
    char detail[sizeof g_last_error];
    memcpy(detail, g_last_error, sizeof detail);
    return fail(st, "entry %d: %s", i, detail);
}

cfz_status hip_fail(hipError_t e, const char *what)
{
    return fail(CFZ_ERR_HIP, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }

cfz_status check_desc(const cfz_desc *d)
{
    if (!d)
        return fail(CFZ_ERR_NULL, "descriptor is NULL");
    if (d->rows < 0 || d->cols < 0)
        return fail(CFZ_ERR_SHAPE, "negative shape %lld x %lld", (long long)d->rows,
                    (long long)d->cols);
    if (d->bits != 2 && d->bits != 4)
        return fail(CFZ_ERR_UNSUPPORTED, "bits = %d (supported: 2, 4)", d->bits);
    if (d->group != 8 && d->group != 16 && d->group != 32 && d->group != 64 && d->group != 128)
        return fail(CFZ_ERR_UNSUPPORTED, "group = %d (supported: 8, 16, 32, 64, 128)", d->group);
    if (d->cols % d->group != 0)
        return fail(CFZ_ERR_SHAPE, "cols = %lld is not a multiple of group = %d",
                    (long long)d->cols, d->group);
    if (d->cols != 0 && d->rows > INT64_MAX / 16 / d->cols)
        return fail(CFZ_ERR_SHAPE, "tensor too large");
    if (d->ef_mode < CFZ_EF_DELTA || d->ef_mode > CFZ_EF_OFF)
        return fail(CFZ_ERR_MODE, "ef_mode = %d", d->ef_mode);
    if (d->role != CFZ_SENDER && d->role != CFZ_RECEIVER)
        return fail(CFZ_ERR_MODE, "role = %d", d->role);
    if (d->state_dtype != CFZ_STATE_F32 && d->state_dtype != CFZ_STATE_BF16)
        return fail(CFZ_ERR_UNSUPPORTED, "state_dtype = %d", d->state_dtype);
    if (d->reserved != 0)
        return fail(CFZ_ERR_SHAPE, "reserved field must be 0");
    return CFZ_OK;
}

bool needs_prev(const cfz_desc &d) { return d.role == CFZ_SENDER && d.ef_mode == CFZ_EF_DELTA; }
bool needs_base(const cfz_desc &d)
{
    return d.role == CFZ_RECEIVER || d.ef_mode == CFZ_EF_LITERAL || d.ef_mode == CFZ_EF_OFF;
}
bool needs_err(const cfz_desc &d)
{
    return d.role == CFZ_SENDER && (d.ef_mode == CFZ_EF_DELTA || d.ef_mode == CFZ_EF_LITERAL);
}

cfz_status check_buffers(const cfz_desc &d, const cfz_buffers *b, cfz_buffers *used)
{
    if (!b)
        return fail(CFZ_ERR_NULL, "buffers is NULL");
    const bool empty = d.rows * d.cols == 0;
    *used = cfz_buffers{needs_prev(d) ? b->prev_bf16 : nullptr, needs_base(d) ? b->base : nullptr,
                        needs_err(d) ? b->err : nullptr};
    if (needs_prev(d) && !b->prev_bf16 && !empty)
        return fail(CFZ_ERR_NULL, "prev_bf16 is required by a DELTA sender");
    if (needs_base(d) && !b->base && !empty)
        return fail(CFZ_ERR_NULL, "base is required by this role/mode");
    if (needs_err(d) && !b->err && !empty)
        return fail(CFZ_ERR_NULL, "err is required by this mode");
    if (!aligned16(used->prev_bf16) || !aligned16(used->base) || !aligned16(used->err))
        return fail(CFZ_ERR_ALIGN, "state buffers must be 16-byte aligned");
    return CFZ_OK;
}

}  // namespace

struct cfz_state {
    uint32_t magic;
    cfz_desc desc;
    cfz_buffers bufs;
    int64_t steps;
};

static cfz_status check_state(const cfz_state *s)
{
    if (!s)
        return fail(CFZ_ERR_NULL, "state is NULL");
    if (s->magic != kMagic)
        return fail(CFZ_ERR_NULL, "not a live cfz_state handle");
    return CFZ_OK;
}

extern "C" {

int cfz_abi_version(void) { return CFZ_ABI_VERSION; }

const char *cfz_last_error(void) { return g_last_error; }

const char *cfz_status_string(cfz_status st)
{
    switch (st) {
    case CFZ_OK: return "ok";
    case CFZ_ERR_NULL: return "required pointer is NULL";
    case CFZ_ERR_SHAPE: return "invalid shape";
    case CFZ_ERR_UNSUPPORTED: return "unsupported bits or group";
    case CFZ_ERR_ALIGN: return "pointer not 16-byte aligned";
    case CFZ_ERR_MODE: return "invalid mode or role for this call";
    case CFZ_ERR_WORKSPACE: return "workspace missing or too small";
    case CFZ_ERR_HIP: return "HIP runtime error";
    }
    return "unknown status";
}

size_t cfz_codes_bytes(const cfz_desc *d)
{
    if (check_desc(d) != CFZ_OK)
        return 0;
    return (size_t)(d->rows * d->cols * d->bits / 8);
}

size_t cfz_scales_bytes(const cfz_desc *d)
{
    if (check_desc(d) != CFZ_OK)
        return 0;
    return (size_t)(d->rows * d->cols / d->group) * sizeof(float);
}

cfz_status cfz_state_resume(const cfz_desc *desc, const cfz_buffers *bufs, int64_t steps,
                            cfz_state **out)
{
    cfz_status st = check_desc(desc);
    if (st != CFZ_OK)
        return st;
    if (!out)
        return fail(CFZ_ERR_NULL, "out is NULL");
    if (steps < 0)
        return fail(CFZ_ERR_SHAPE, "steps = %lld", (long long)steps);
    cfz_buffers used;
    if ((st = check_buffers(*desc, bufs, &used)) != CFZ_OK)
        return st;
    cfz_state *s = new (std::nothrow) cfz_state{kMagic, *desc, used, steps};
    if (!s)
        return fail(CFZ_ERR_NULL, "out of host memory");
    *out = s;
    return CFZ_OK;
}

cfz_status cfz_state_create(const cfz_desc *desc, const cfz_buffers *bufs, const uint16_t *x0,
                            void *stream, cfz_state **out)
{
    cfz_status st = check_desc(desc);
    if (st != CFZ_OK)
        return st;
    if (!out)
        return fail(CFZ_ERR_NULL, "out is NULL");
    cfz_buffers used;
    if ((st = check_buffers(*desc, bufs, &used)) != CFZ_OK)
        return st;
    if (!aligned16(x0))
        return fail(CFZ_ERR_ALIGN, "x0 must be 16-byte aligned");
    cfz_state *s = new (std::nothrow) cfz_state{kMagic, *desc, used, 0};
    if (!s)
        return fail(CFZ_ERR_NULL, "out of host memory");
    const int64_t nchunks = desc->rows * desc->cols / 8;
    hipError_t e = cfz::launch_warmup(x0, used.prev_bf16, used.base, used.err,
                                      desc->state_dtype == CFZ_STATE_BF16, nchunks,
                                      (hipStream_t)stream);
    if (e != hipSuccess) {
        s->magic = 0;
        delete s;
        return hip_fail(e, "warm-up launch");
    }
    *out = s;
    return CFZ_OK;
}

cfz_status cfz_state_destroy(cfz_state *s)
{
    if (!s)
        return CFZ_OK;
    cfz_status st = check_state(s);
    if (st != CFZ_OK)
        return st;
    s->magic = 0;
    delete s;
    return CFZ_OK;
}

int64_t cfz_state_steps(const cfz_state *s)
{
    if (check_state(s) != CFZ_OK)
        return -1;
    return s->steps;
}

// Per-tensor checks shared by the single and grouped entry points.
static cfz_status check_compress_one(cfz_state *s, const uint16_t *x, uint8_t *codes, float *scales,
                                     cfz::CompressItem *item)
{
    cfz_status st = check_state(s);
    if (st != CFZ_OK)
        return st;
    const cfz_desc &d = s->desc;
    if (d.role != CFZ_SENDER)
        return fail(CFZ_ERR_MODE, "cfz_compress needs a sender state");
    const int64_t n = d.rows * d.cols;
    if (n != 0 && (!x || !codes || !scales))
        return fail(CFZ_ERR_NULL, "x, codes and scales are required");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales))
        return fail(CFZ_ERR_ALIGN, "x, codes and scales must be 16-byte aligned");
    *item = cfz::CompressItem{x, s->bufs.prev_bf16, s->bufs.base, s->bufs.err, codes, scales, n};
    return CFZ_OK;
}

static cfz_status check_decode_one(cfz_state *s, const uint8_t *codes, const float *scales,
                                   uint16_t *xhat, cfz::DecodeItem *item)
{
    cfz_status st = check_state(s);
    if (st != CFZ_OK)
        return st;
    const cfz_desc &d = s->desc;
    if (d.role != CFZ_RECEIVER)
        return fail(CFZ_ERR_MODE, "cfz_decompress needs a receiver state");
    const int64_t n = d.rows * d.cols;
    if (n != 0 && (!codes || !scales))
        return fail(CFZ_ERR_NULL, "codes and scales are required");
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(xhat))
        return fail(CFZ_ERR_ALIGN, "codes, scales and xhat must be 16-byte aligned");
    *item = cfz::DecodeItem{codes, scales, s->bufs.base, xhat, n};
    return CFZ_OK;
}

static bool same_codec(const cfz_desc &a, const cfz_desc &b)
{
    return a.bits == b.bits && a.group == b.group && a.ef_mode == b.ef_mode && a.role == b.role &&
           a.state_dtype == b.state_dtype;
}

cfz_status cfz_compress(cfz_state *s, const uint16_t *x, uint8_t *codes, float *scales,
                        void *stream)
{
    cfz::CompressItem item;
    cfz_status st = check_compress_one(s, x, codes, scales, &item);
    if (st != CFZ_OK)
        return st;
    const cfz_desc &d = s->desc;
    hipError_t e = cfz::launch_compress(&item, 1, d.bits, d.group, d.ef_mode,
                                        d.state_dtype == CFZ_STATE_BF16, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "compress launch");
    ++s->steps;
    return CFZ_OK;
}

cfz_status cfz_decompress(cfz_state *s, const uint8_t *codes, const float *scales,
                          uint16_t *xhat, void *stream)
{
    cfz::DecodeItem item;
    cfz_status st = check_decode_one(s, codes, scales, xhat, &item);
    if (st != CFZ_OK)
        return st;
    const cfz_desc &d = s->desc;
    hipError_t e = cfz::launch_decode(&item, 1, d.bits, d.group, d.state_dtype == CFZ_STATE_BF16,
                                      (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "decode launch");
    ++s->steps;
    return CFZ_OK;
}

// Group checks common to both directions: array presence, one codec setting, no repeats.
static cfz_status check_group(int32_t count, cfz_state *const *states, const void *a, const void *b,
                              const void *c)
{
    if (count < 0)
        return fail(CFZ_ERR_SHAPE, "count = %d", count);
    if (count == 0)
        return CFZ_OK;
    if (!states || !a || !b || !c)
        return fail(CFZ_ERR_NULL, "state and buffer arrays are required");
    for (int32_t i = 0; i < count; ++i) {
        cfz_status st = check_state(states[i]);
        if (st != CFZ_OK)
            return fail_entry(st, i);
        if (!same_codec(states[i]->desc, states[0]->desc))
            return fail(CFZ_ERR_MODE, "entry %d: bits, group, mode, role and state must match entry 0",
                        i);
        for (int32_t j = 0; j < i; ++j)
            if (states[j] == states[i])
                return fail(CFZ_ERR_MODE, "entries %d and %d are the same state", j, i);
    }
    return CFZ_OK;
}

cfz_status cfz_compress_group(int32_t count, cfz_state *const *senders, const uint16_t *const *xs,
                              uint8_t *const *codes, float *const *scales, void *stream)
{
    cfz_status st = check_group(count, senders, xs, codes, scales);
    if (st != CFZ_OK || count == 0)
        return st;
    cfz::CompressItem *items = new (std::nothrow) cfz::CompressItem[count];
    if (!items)
        return fail(CFZ_ERR_NULL, "out of host memory");
    for (int32_t i = 0; i < count && st == CFZ_OK; ++i)
        if ((st = check_compress_one(senders[i], xs[i], codes[i], scales[i], &items[i])) != CFZ_OK)
            st = fail_entry(st, i);
    if (st == CFZ_OK) {
        const cfz_desc &d = senders[0]->desc;
        hipError_t e = cfz::launch_compress(items, count, d.bits, d.group, d.ef_mode,
                                            d.state_dtype == CFZ_STATE_BF16, (hipStream_t)stream);
        if (e != hipSuccess)
            st = hip_fail(e, "grouped compress launch");
        else
            for (int32_t i = 0; i < count; ++i)
                ++senders[i]->steps;
    }
    delete[] items;
    return st;
}

cfz_status cfz_decompress_group(int32_t count, cfz_state *const *receivers,
                                const uint8_t *const *codes, const float *const *scales,
                                uint16_t *const *xhat, void *stream)
{
    cfz_status st = check_group(count, receivers, codes, scales, codes);
    if (st != CFZ_OK || count == 0)
        return st;
    cfz::DecodeItem *items = new (std::nothrow) cfz::DecodeItem[count];
    if (!items)
        return fail(CFZ_ERR_NULL, "out of host memory");
    for (int32_t i = 0; i < count && st == CFZ_OK; ++i)
        if ((st = check_decode_one(receivers[i], codes[i], scales[i], xhat ? xhat[i] : nullptr,
                                   &items[i])) != CFZ_OK)
            st = fail_entry(st, i);
    if (st == CFZ_OK) {
        const cfz_desc &d = receivers[0]->desc;
        hipError_t e = cfz::launch_decode(items, count, d.bits, d.group,
                                          d.state_dtype == CFZ_STATE_BF16, (hipStream_t)stream);
        if (e != hipSuccess)
            st = hip_fail(e, "grouped decode launch");
        else
            for (int32_t i = 0; i < count; ++i)
                ++receivers[i]->steps;
    }
    delete[] items;
    return st;
}

size_t cfz_lowrank_workspace_bytes(int64_t batch, int64_t m, int64_t n, int32_t r)
{
    if (batch < 0 || m <= 0 || n <= 0 || r < 1 || r > 32 || r > m || r > n || n % 8 != 0 ||
        m > (1 << 20) || n > (1 << 20) || batch > (1 << 20) || m * n > ((int64_t)1 << 30))
        return 0;
    return cfz::lowrank_workspace_bytes(batch, m, n, r);
}

}  // extern "C"

namespace {

// Shape rules shared by the low-rank entry points (T < 0 is checked where T is taken).
cfz_status check_lowrank_shape(int64_t batch, int64_t m, int64_t n, int32_t r)
{
    if (batch < 0 || m <= 0 || n <= 0)
        return fail(CFZ_ERR_SHAPE, "batch = %lld, m = %lld, n = %lld", (long long)batch,
                    (long long)m, (long long)n);
    if (r < 1 || r > 32 || r > m || r > n)
        return fail(CFZ_ERR_SHAPE, "rank r = %d must be in [1, min(32, m, n)]", r);
    if (n % 8 != 0)
        return fail(CFZ_ERR_SHAPE, "n = %lld must be a multiple of 8 (16-byte rows)", (long long)n);
    if (m * n > ((int64_t)1 << 30))
        return fail(CFZ_ERR_SHAPE, "m * n = %lld exceeds 2^30 elements per matrix", (long long)(m * n));
    if (m > (1 << 20) || n > (1 << 20) || batch > (1 << 20))
        return fail(CFZ_ERR_SHAPE, "sizes too large");
    return CFZ_OK;
}

cfz_status check_lowrank_ef_shape(int64_t batch, int64_t m, int64_t n, int32_t r)
{
    cfz_status st = check_lowrank_shape(batch, m, n, r);
    if (st != CFZ_OK)
        return st;
    if (cfz::lowrank_ef_update_blocks(batch, m, n) >= ((int64_t)1 << 31) ||
        batch * m * n / 4 / 256 >= ((int64_t)1 << 31))
        return fail(CFZ_ERR_SHAPE, "batch * m * n too large for one launch");
    return CFZ_OK;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

extern "C" {

cfz_status cfz_lowrank(int64_t batch, int64_t m, int64_t n, int32_t r, int32_t T,
                       const uint16_t *A, const float *Q0, float *U, float *V, float *RU,
                       void *ws, size_t ws_bytes, void *stream)
{
    cfz_status st = check_lowrank_shape(batch, m, n, r);
    if (st != CFZ_OK)
        return st;
    if (T < 0)
        return fail(CFZ_ERR_SHAPE, "iterations T = %d", T);
    if (batch == 0)
        return CFZ_OK;
    if (!A || !Q0 || !U || !V || !RU)
        return fail(CFZ_ERR_NULL, "A, Q0, U, V and RU are required");
    if (!aligned16(A) || !aligned16(Q0) || !aligned16(U) || !aligned16(V) || !aligned16(RU))
        return fail(CFZ_ERR_ALIGN, "A, Q0, U, V and RU must be 16-byte aligned");
    const size_t need = cfz::lowrank_workspace_bytes(batch, m, n, r);
    if (!ws || ws_bytes < need)
        return fail(CFZ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : (size_t)0);
    if (((uintptr_t)ws & 255u) != 0)
        return fail(CFZ_ERR_ALIGN, "workspace must be 256-byte aligned");
    cfz::LowrankArgs a{batch, m, n, r, T, A, Q0, U, V, RU, ws};
    hipError_t e = cfz::launch_lowrank(a, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "low-rank launch");
    return CFZ_OK;
}

}  // extern "C"

// ---- the subspace iteration without a caller workspace ---------------------
//
// For callers that cannot allocate device memory (code under graph capture, tight
// serving loops): the workspace is this file-scope device array, one copy per GPU,
// held until the process ends.  In host code `scratch` names a host-side stand-in,
// not a device address, so every use goes through the address hipGetSymbolAddress
// returns for the current device, looked up once per device.

namespace {

constexpr size_t kScratchBytes = (size_t)64 << 20;  // covers 57 x 1024 x 3072 at any r
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
void *g_scratch_ptr[kMaxDevices];  // per device, filled on first use

// The current device's copy of `scratch`, or an error status.
cfz_status scratch_for_current_device(void **out)
{
    int dev = -1;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess)
        return hip_fail(e, "hipGetDevice");
    if (dev < 0 || dev >= kMaxDevices)
        return fail(CFZ_ERR_HIP, "device %d beyond the %d this library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_scratch_mutex);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess)
            return hip_fail(e, "hipGetSymbolAddress(scratch)");
        if (!p || ((uintptr_t)p & 255u) != 0)
            return fail(CFZ_ERR_HIP, "scratch array at an unusable address");
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return CFZ_OK;
}

}  // namespace

extern "C" {

size_t cfz_lowrank_noalloc_max_bytes(void) { return kScratchBytes; }

cfz_status cfz_lowrank_noalloc(int64_t batch, int64_t m, int64_t n, int32_t r, int32_t T,
                               const uint16_t *A, const float *Q0, float *U, float *V, float *RU,
                               void *stream)
{
    cfz_status st = check_lowrank_shape(batch, m, n, r);
    if (st != CFZ_OK)
        return st;
    if (T < 0)
        return fail(CFZ_ERR_SHAPE, "iterations T = %d", T);
    if (batch == 0)
        return CFZ_OK;
    if (!A || !Q0 || !U || !V || !RU)
        return fail(CFZ_ERR_NULL, "A, Q0, U, V and RU are required");
    if (!aligned16(A) || !aligned16(Q0) || !aligned16(U) || !aligned16(V) || !aligned16(RU))
        return fail(CFZ_ERR_ALIGN, "A, Q0, U, V and RU must be 16-byte aligned");
    const size_t need = cfz::lowrank_workspace_bytes(batch, m, n, r);
    if (need > kScratchBytes)
        return fail(CFZ_ERR_WORKSPACE,
                    "these sizes need %zu bytes of workspace, beyond the %zu-byte built-in "
                    "scratch; use cfz_lowrank with a caller workspace", need, kScratchBytes);
    void *ws = nullptr;
    if ((st = scratch_for_current_device(&ws)) != CFZ_OK)
        return st;
    cfz::LowrankArgs a{batch, m, n, r, T, A, Q0, U, V, RU, ws};
    hipError_t e = cfz::launch_lowrank(a, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "low-rank launch");
    return CFZ_OK;
}

size_t cfz_lowrank_ef_workspace_bytes(int64_t batch, int64_t m, int64_t n, int32_t r)
{
    if (batch < 0 || m <= 0 || n <= 0 || r < 1 || r > 32 || r > m || r > n || n % 8 != 0 ||
        m > (1 << 20) || n > (1 << 20) || batch > (1 << 20) || m * n > ((int64_t)1 << 30))
        return 0;
    return align256((size_t)(batch * m * n) * 2) + cfz::lowrank_workspace_bytes(batch, m, n, r);
}

cfz_status cfz_lowrank_ef_warmup(int64_t count, const uint16_t *x0, uint16_t *prev, float *err,
                                 float *base, void *stream)
{
    if (count < 0 || count % 8 != 0)
        return fail(CFZ_ERR_SHAPE, "count = %lld must be a non-negative multiple of 8",
                    (long long)count);
    if (!aligned16(x0) || !aligned16(prev) || !aligned16(err) || !aligned16(base))
        return fail(CFZ_ERR_ALIGN, "buffers must be 16-byte aligned");
    if (count == 0 || (!prev && !err && !base))
        return CFZ_OK;
    hipError_t e = cfz::launch_warmup(x0, prev, base, err, false, count / 8, (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "warm-up launch");
    return CFZ_OK;
}

namespace {

// The sender's three forms: kPlain updates err at the end of the call; kDeferred leaves the
// residual in err; kDeferredPending also first applies the previous deferred call's update
// (with the factors still in U, V, RU) inside the residual pass.
enum EfSend { kPlain, kDeferred, kDeferredPending };

cfz_status ef_send(EfSend mode, int64_t batch, int64_t m, int64_t n, int32_t r, int32_t T,
                   const uint16_t *x, uint16_t *prev, float *err, const float *Q0, float *U,
                   float *V, float *RU, void *ws, size_t ws_bytes, void *stream)
{
    cfz_status st = check_lowrank_ef_shape(batch, m, n, r);
    if (st != CFZ_OK)
        return st;
    if (T < 0)
        return fail(CFZ_ERR_SHAPE, "iterations T = %d", T);
    if (batch == 0)
        return CFZ_OK;
    if (!x || !prev || !err || !Q0 || !U || !V || !RU)
        return fail(CFZ_ERR_NULL, "x, prev, err, Q0, U, V and RU are required");
    if (!aligned16(x) || !aligned16(prev) || !aligned16(err) || !aligned16(Q0) || !aligned16(U) ||
        !aligned16(V) || !aligned16(RU))
        return fail(CFZ_ERR_ALIGN, "every buffer must be 16-byte aligned");
    const size_t a_bytes = align256((size_t)(batch * m * n) * 2);
    const size_t need = a_bytes + cfz::lowrank_workspace_bytes(batch, m, n, r);
    if (!ws || ws_bytes < need)
        return fail(CFZ_ERR_WORKSPACE, "workspace of %zu bytes needed, %zu given", need,
                    ws ? ws_bytes : (size_t)0);
    if (((uintptr_t)ws & 255u) != 0)
        return fail(CFZ_ERR_ALIGN, "workspace must be 256-byte aligned");
    hipStream_t hs = (hipStream_t)stream;
    uint16_t *A = (uint16_t *)ws;
    hipError_t e = mode == kDeferredPending
                       ? cfz::launch_lowrank_ef_residual_update(batch, m, n, r, U, V, RU, x, prev,
                                                                err, A, hs)
                       : cfz::launch_lowrank_ef_residual(x, prev, err, A, batch * m * n, hs);
    if (e != hipSuccess)
        return hip_fail(e, "residual launch");
    cfz::LowrankArgs a{batch, m, n, r, T, A, Q0, U, V, RU, (uint8_t *)ws + a_bytes};
    e = cfz::launch_lowrank(a, hs);
    if (e != hipSuccess)
        return hip_fail(e, "low-rank launch");
    if (mode == kPlain) {
        e = cfz::launch_lowrank_ef_update(batch, m, n, r, U, V, RU, -1.0f, err, nullptr, hs);
        if (e != hipSuccess)
            return hip_fail(e, "update launch");
    }
    return CFZ_OK;
}

}  // namespace

cfz_status cfz_lowrank_ef_compress(int64_t batch, int64_t m, int64_t n, int32_t r, int32_t T,
                                   const uint16_t *x, uint16_t *prev, float *err, const float *Q0,
                                   float *U, float *V, float *RU, void *ws, size_t ws_bytes,
                                   void *stream)
{
    return ef_send(kPlain, batch, m, n, r, T, x, prev, err, Q0, U, V, RU, ws, ws_bytes, stream);
}

cfz_status cfz_lowrank_ef_compress_deferred(int64_t batch, int64_t m, int64_t n, int32_t r,
                                            int32_t T, int32_t pending, const uint16_t *x,
                                            uint16_t *prev, float *err, const float *Q0, float *U,
                                            float *V, float *RU, void *ws, size_t ws_bytes,
                                            void *stream)
{
    if (pending != 0 && pending != 1)
        return fail(CFZ_ERR_SHAPE, "pending = %d must be 0 or 1", pending);
    return ef_send(pending ? kDeferredPending : kDeferred, batch, m, n, r, T, x, prev, err, Q0, U,
                   V, RU, ws, ws_bytes, stream);
}

cfz_status cfz_lowrank_ef_flush(int64_t batch, int64_t m, int64_t n, int32_t r, const float *U,
                                const float *V, const float *RU, float *err, void *stream)
{
    cfz_status st = check_lowrank_ef_shape(batch, m, n, r);
    if (st != CFZ_OK)
        return st;
    if (batch == 0)
        return CFZ_OK;
    if (!U || !V || !RU || !err)
        return fail(CFZ_ERR_NULL, "U, V, RU and err are required");
    if (!aligned16(U) || !aligned16(V) || !aligned16(RU) || !aligned16(err))
        return fail(CFZ_ERR_ALIGN, "every buffer must be 16-byte aligned");
    hipError_t e = cfz::launch_lowrank_ef_update(batch, m, n, r, U, V, RU, -1.0f, err, nullptr,
                                                 (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "update launch");
    return CFZ_OK;
}

cfz_status cfz_lowrank_ef_decompress(int64_t batch, int64_t m, int64_t n, int32_t r,
                                     const float *U, const float *V, const float *RU, float *base,
                                     uint16_t *xhat, void *stream)
{
    cfz_status st = check_lowrank_ef_shape(batch, m, n, r);
    if (st != CFZ_OK)
        return st;
    if (batch == 0)
        return CFZ_OK;
    if (!U || !V || !RU || !base)
        return fail(CFZ_ERR_NULL, "U, V, RU and base are required");
    if (!aligned16(U) || !aligned16(V) || !aligned16(RU) || !aligned16(base) || !aligned16(xhat))
        return fail(CFZ_ERR_ALIGN, "every buffer must be 16-byte aligned");
    hipError_t e = cfz::launch_lowrank_ef_update(batch, m, n, r, U, V, RU, 1.0f, base, xhat,
                                                 (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "update launch");
    return CFZ_OK;
}

cfz_status cfz_stream_mix(const void *src, size_t src_bytes, void *dst, size_t dst_bytes,
                          void *stream)
{
    if (src_bytes == 0)
        return dst_bytes == 0 ? CFZ_OK : fail(CFZ_ERR_SHAPE, "dst_bytes > src_bytes");
    if (!src || (dst_bytes && !dst))
        return fail(CFZ_ERR_NULL, "src and dst are required");
    if ((src_bytes & 15u) != 0 || (dst_bytes & 15u) != 0)
        return fail(CFZ_ERR_SHAPE, "byte counts must be multiples of 16");
    if (dst_bytes > src_bytes)
        return fail(CFZ_ERR_SHAPE, "dst_bytes > src_bytes");
    if (src_bytes / 16 > ((size_t)1 << 31))
        return fail(CFZ_ERR_SHAPE, "src_bytes too large");
    if (!aligned16(src) || !aligned16(dst))
        return fail(CFZ_ERR_ALIGN, "src and dst must be 16-byte aligned");
    hipError_t e = cfz::launch_stream_mix(src, dst, (int64_t)(src_bytes / 16),
                                          (int64_t)(dst_bytes / 16), (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "mixed stream launch");
    return CFZ_OK;
}

cfz_status cfz_stream_copy(const void *src, void *dst, size_t bytes, void *stream)
{
    if (bytes == 0)
        return CFZ_OK;
    if (!src || !dst)
        return fail(CFZ_ERR_NULL, "src and dst are required");
    if ((bytes & 15u) != 0)
        return fail(CFZ_ERR_SHAPE, "bytes must be a multiple of 16");
    if (!aligned16(src) || !aligned16(dst))
        return fail(CFZ_ERR_ALIGN, "src and dst must be 16-byte aligned");
    hipError_t e = cfz::launch_stream_copy(src, dst, (int64_t)(bytes / 16), (hipStream_t)stream);
    if (e != hipSuccess)
        return hip_fail(e, "copy launch");
    return CFZ_OK;
}

}  // extern "C"
