/*
 * cfz.h -- C ABI of libcfz, the CompactFusion residual-compression codec and
 * rank-r subspace-iteration compressor for one AMD Instinct MI355X (gfx950).
 *
 * Method: "Accelerating Parallel Diffusion Model Serving with Residual
 * Compression" (Luo et al., NeurIPS 2025).  Parallel diffusion serving
 * exchanges large activations (K/V or patch features) between devices at every
 * denoising step; adjacent steps are nearly identical, so only a compressed
 * step-wise residual is sent, with error feedback so that compression error
 * does not accumulate (abstract; xDiT issue #573).  One uncompressed warm-up
 * step initialises the base tensor that later residuals are taken against
 * (reproducibility table, "Dataset Splits").  A rank-r compressor by subspace
 * iteration is given as Algorithm 3 (reproducibility table, "Pseudocode").
 *
 * Conventions for every entry point:
 *   - Device pointers are caller-owned, contiguous, row-major and 16-byte
 *     aligned.  The library never allocates device memory.
 *   - bf16 values travel as raw uint16_t bit patterns.
 *   - Work is enqueued asynchronously on `hip_stream` (a hipStream_t; NULL is
 *     the default stream).  No call synchronises.  Buffers must stay alive
 *     until the enqueued work has finished.
 *   - All arguments are validated before anything is enqueued: a non-OK
 *     status means no device work was queued and no buffer was written.
 *     A failed launch returns CFZ_ERR_HIP.  No C++ exception crosses the ABI.
 *     cfz_last_error() gives a thread-local description of the last failure.
 *   - A cfz_state is a small host object.  It must not be used on two
 *     streams at once; the caller's stream order is the step order.
 */
#ifndef CFZ_H
#define CFZ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define CFZ_ABI_VERSION 4

typedef enum {
    CFZ_OK = 0,
    CFZ_ERR_NULL = 1,        /* a required pointer is NULL                          */
    CFZ_ERR_SHAPE = 2,       /* negative size, cols % group != 0, m/n/r/T out of range */
    CFZ_ERR_UNSUPPORTED = 3, /* bits not in {2, 4}, group not in {8,16,32,64,128}  */
    CFZ_ERR_ALIGN = 4,       /* a device pointer is not 16-byte aligned             */
    CFZ_ERR_MODE = 5,        /* bad ef_mode/role, or the call does not fit the role */
    CFZ_ERR_WORKSPACE = 6,   /* low-rank workspace missing or too small             */
    CFZ_ERR_HIP = 7          /* the HIP runtime reported an error                   */
} cfz_status;

/* How the sender forms the residual and carries the compression error.
 *   DELTA   (default): r = (x - prev) + err; prev' = x; err' = r - q s.
 *           Error feedback on the change between consecutive steps: the
 *           receiver's base then equals x - err' after every step.
 *   LITERAL: r = (x - base) + err; err' = r - q s; base' = base + q s.
 *           The carried error is added on top of a base that already absorbs
 *           it; kept to reproduce that reading, which is unstable at 2 bits.
 *   OFF:     r = x - base; base' = base + q s (closed loop, no error buffer).
 * The receiver always does base' = base + q s. */
typedef enum { CFZ_EF_DELTA = 0, CFZ_EF_LITERAL = 1, CFZ_EF_OFF = 2 } cfz_ef_mode;

typedef enum { CFZ_SENDER = 0, CFZ_RECEIVER = 1 } cfz_role;

/* Precision of the carried error E and of the base X-hat.
 *   F32:  fp32 state (default).
 *   BF16: bf16 state, half the state traffic.  Every update is the same fp32
 *         fma as with F32, rounded once to bf16 (nearest even); a zero code
 *         leaves the base's bits untouched.  In OFF mode sender and receiver
 *         then hold bit-identical bf16 bases and the closed loop absorbs the
 *         rounding; the receiver's base is directly a bf16 activation. */
typedef enum { CFZ_STATE_F32 = 0, CFZ_STATE_BF16 = 1 } cfz_state_dtype;

/* One exchanged tensor: rows (tokens) x cols (channels), quantized in groups of
 * `group` consecutive channels of one row with `bits`-bit codes.
 * Requirements: rows >= 0, cols >= 0, bits in {2, 4}, group in {8,16,32,64,128},
 * cols % group == 0, state_dtype a cfz_state_dtype, reserved == 0.
 * rows * cols == 0 is allowed (every call is then a no-op). */
typedef struct {
    int64_t rows;
    int64_t cols;
    int32_t bits;
    int32_t group;
    int32_t ef_mode;     /* cfz_ef_mode     */
    int32_t role;        /* cfz_role        */
    int32_t state_dtype; /* cfz_state_dtype */
    int32_t reserved;    /* must be 0       */
} cfz_desc;

/* Caller-owned state buffers, rows*cols elements each, on the device.
 *   prev_bf16: sender in DELTA mode (previous activation, bf16).
 *   base:      receiver; sender in LITERAL and OFF modes (running reconstruction).
 *   err:       sender in DELTA and LITERAL modes (carried error).
 * base and err hold fp32 or bf16 values according to desc.state_dtype.
 * Buffers the role/mode does not use are ignored and may be NULL. */
typedef struct {
    uint16_t *prev_bf16;
    void *base;
    void *err;
} cfz_buffers;

typedef struct cfz_state cfz_state;

/* Warm-up (step 0): the uncompressed activation x0 initialises the state.
 * Receiver: base = x0.  Sender: prev = x0 (DELTA), base = x0 (LITERAL, OFF),
 * err = 0 (DELTA, LITERAL) -- in the state's precision (bf16 to fp32 is exact).  x0 == NULL means all zeros.
 * Enqueues one initialisation kernel on hip_stream, then returns the handle.
 * On error *out is left unchanged.  (paper: reproducibility table,
 * "Dataset Splits" -- warm-up initialises the base tensor.) */
cfz_status cfz_state_create(const cfz_desc *desc, const cfz_buffers *bufs,
                            const uint16_t *x0_bf16, void *hip_stream, cfz_state **out);

/* Rebuild a handle around buffers that already hold a state (checkpoint/resume).
 * Enqueues nothing.  `steps` is the number of compressed steps already taken. */
cfz_status cfz_state_resume(const cfz_desc *desc, const cfz_buffers *bufs, int64_t steps,
                            cfz_state **out);

/* Frees the host handle only; the caller owns and frees the device buffers.
 * NULL is accepted. */
cfz_status cfz_state_destroy(cfz_state *state);

/* Number of compressed steps enqueued on this state so far (-1 for NULL). */
int64_t cfz_state_steps(const cfz_state *state);

/* Payload sizes for one step: codes rows*cols*bits/8 bytes, scales
 * rows*cols/group fp32 values (bytes returned).  0 for an invalid descriptor. */
size_t cfz_codes_bytes(const cfz_desc *desc);
size_t cfz_scales_bytes(const cfz_desc *desc);

/* One compressed step at the sender, fused in one kernel: residual with error
 * feedback, group absmax scale s = max|r| / qmax (qmax = 2^(bits-1) - 1, IEEE
 * fp32 division), q = clamp(rint(r / s), -qmax, qmax) (0 when s == 0), packing
 * of q into bits-bit two's complement fields (element j in byte j*bits/8 at
 * bit (j*bits) % 8), and the state update of the sender's ef_mode.
 * x: rows*cols bf16.  codes: cfz_codes_bytes.  scales: rows*cols/group fp32,
 * scale k covering elements [k*group, (k+1)*group).
 * (paper: abstract -- compressed step-wise residuals with error feedback.)
 * NaN and +-Inf in x lie outside the method: the call still writes only its own
 * buffers, and only the groups that hold such values get unspecified codes,
 * scales and state (their error and base elements can stay non-finite until the
 * state is warmed again with cfz_state_create); every other group is unaffected.
 * Errors: CFZ_ERR_NULL, CFZ_ERR_ALIGN, CFZ_ERR_MODE (receiver state), CFZ_ERR_HIP. */
cfz_status cfz_compress(cfz_state *sender, const uint16_t *x_bf16, uint8_t *codes,
                        float *scales, void *hip_stream);

/* One step at the receiver: unpack, sign-extend, base' = fma(q, s, base) where
 * q != 0 (a zero code leaves the base bit-identical; with bf16 state the fma
 * result is rounded once to bf16), and optionally write the new base rounded to
 * bf16 (nearest even) into xhat_bf16 (may be NULL).
 * (paper: abstract -- only compressed residuals are transmitted, so the receiver
 * rebuilds the activation by adding each decoded residual to its base;
 * reproducibility table, "Dataset Splits" -- that base starts from the
 * uncompressed warm-up activation.)
 * Errors: CFZ_ERR_NULL, CFZ_ERR_ALIGN, CFZ_ERR_MODE (sender state), CFZ_ERR_HIP. */
cfz_status cfz_decompress(cfz_state *receiver, const uint8_t *codes, const float *scales,
                          uint16_t *xhat_bf16, void *hip_stream);

/* The same steps for `count` separately allocated tensors in as few launches as
 * possible (up to 16 tensors per launch): e.g. the K and V of one layer, which
 * the sender has at the same time.  Entry i uses senders[i] / receivers[i] with
 * x_bf16[i], codes[i], scales[i] (and xhat_bf16[i]; xhat_bf16 itself or any of
 * its entries may be NULL).  All states must share bits, group, ef_mode and
 * role, and no state may appear twice; the tensors' buffers must not overlap.
 * Results are bit-identical to `count` single calls.  All entries are validated
 * before anything is enqueued; on a validation error nothing is enqueued and
 * cfz_last_error() names the entry.  count == 0 is a no-op.
 * Errors: as the single calls, plus CFZ_ERR_SHAPE (count < 0) and CFZ_ERR_MODE
 * (mixed settings or a repeated state).  CFZ_ERR_HIP may leave the launches
 * before the failing one enqueued. */
cfz_status cfz_compress_group(int32_t count, cfz_state *const *senders,
                              const uint16_t *const *x_bf16, uint8_t *const *codes,
                              float *const *scales, void *hip_stream);
cfz_status cfz_decompress_group(int32_t count, cfz_state *const *receivers,
                                const uint8_t *const *codes, const float *const *scales,
                                uint16_t *const *xhat_bf16, void *hip_stream);

/* Workspace for cfz_lowrank, in bytes, or 0 if the sizes are invalid.  Not
 * monotone in batch (a small batch splits each matrix into more row ranges, each
 * with its own partial sums), so query it with each call's own sizes; a call
 * given less returns CFZ_ERR_WORKSPACE and enqueues nothing. */
size_t cfz_lowrank_workspace_bytes(int64_t batch, int64_t m, int64_t n, int32_t r);

/* Algorithm 3 (Subspace Iteration, rank r) on `batch` independent matrices
 * (paper: reproducibility table, "Pseudocode", Algorithm 3):
 *   Q = orth(Q0); T times { Z = A^T (A Q); Q = orth(Z) }; (U, R_U) = orth(A Q); V = Q.
 * orth() is a thin QR with positive diagonal: Cholesky-QR with the Gram
 * matrix and r x r Cholesky in fp64, repeated once (CholQR2) for the matrices
 * whose condition estimate ||R||_F ||R^-1||_F from the first pass exceeds 2^14.5,
 * where one pass could lose more orthogonality than fp32 output keeps; a column
 * whose pivot is <= 1e-13 of the mean squared column norm is dropped (zero
 * column of Q, zero row and column of R).  The reconstruction of A is U R_U V^T = (A Q) Q^T.
 * A: [batch][m][n] bf16.  Q0: [batch][n][r] fp32 random sample (caller-drawn); it
 * may be the V buffer itself (a warm start from the previous call's V): Q0 is
 * read in full before V is written.
 * U: [batch][m][r], V: [batch][n][r], RU: [batch][r][r], fp32 outputs.
 * Requires 1 <= r <= 32, r <= m, r <= n, T >= 0, n a multiple of 8 (rows of A
 * are 16-byte aligned), m, n, batch <= 2^20, m * n <= 2^30, batch >= 0 (0 is a no-op); a
 * workspace of cfz_lowrank_workspace_bytes(batch, m, n, r) bytes, 256-byte
 * aligned, that the call overwrites.  Products use bf16 MFMA with fp32
 * accumulation; Q and A Q enter them split into two bf16 halves (about 16
 * significant bits), so U R_U V^T agrees with an fp64 evaluation to about 1e-5
 * relative Frobenius error on well-conditioned inputs.
 * Errors: CFZ_ERR_NULL, CFZ_ERR_SHAPE, CFZ_ERR_ALIGN, CFZ_ERR_WORKSPACE, CFZ_ERR_HIP. */
cfz_status cfz_lowrank(int64_t batch, int64_t m, int64_t n, int32_t r, int32_t T,
                       const uint16_t *A_bf16, const float *Q0, float *U, float *V, float *RU,
                       void *workspace, size_t ws_bytes, void *hip_stream);

/* cfz_lowrank without a workspace argument, for callers that cannot allocate
 * device memory (code under HIP graph capture, serving loops that forbid
 * hipMalloc).  Same arguments, results and errors as cfz_lowrank, bit for bit;
 * the workspace is a device array built into the library, one copy per GPU,
 * cfz_lowrank_noalloc_max_bytes() bytes (64 MiB: enough for 57 matrices of
 * 1024 x 3072 at any r), held until the process ends.  Sizes whose
 * cfz_lowrank_workspace_bytes exceeds it return CFZ_ERR_WORKSPACE before any
 * device work.  The call itself allocates nothing; its first call on a device
 * looks up that device's copy (hipGetSymbolAddress).  Every call on one GPU
 * uses the same array and leaves its contents behind (nothing in it needs to
 * start at zero), so calls that may run at the same time on one GPU -- on two
 * streams, or from two threads -- race and must be serialised by the caller. */
cfz_status cfz_lowrank_noalloc(int64_t batch, int64_t m, int64_t n, int32_t r, int32_t T,
                               const uint16_t *A_bf16, const float *Q0, float *U, float *V,
                               float *RU, void *hip_stream);
size_t cfz_lowrank_noalloc_max_bytes(void);

/* ---- The rank-r compressor inside the error-feedback loop ----------------
 * The pages send step-wise residuals with error feedback (abstract) and give
 * the subspace iteration as a compressor (Algorithm 3).  Combined like the
 * DELTA mode of the quantizer, on `batch` independent m x n tensors:
 *   sender:   r = (x - prev) + err (fp32);  A = bf16(r), round to nearest even;
 *             (U, R_U, V) = Algorithm 3 on A;  err' = r - (U R_U) V^T;  prev' = x
 *   receiver: base' = base + (U R_U) V^T;  xhat = bf16(base')
 * The payload is (U, R_U, V) in fp32.  Sender and receiver form (U R_U) V^T
 * with the same kernel (fp32, v_mfma_f32_16x16x4_f32), so with the same
 * factors their reconstructions agree bit for bit.
 * Layouts: x, prev, xhat bf16 and err, base fp32, all [batch][m][n]; U, V, RU
 * as for cfz_lowrank.  Sizes as for cfz_lowrank, plus two launch-size limits:
 * batch * ceil(m / 64) * ceil(n / 256) < 2^31 and batch * m * n / 1024 < 2^31
 * (integer division).  Every pointer 16-byte aligned; the caller owns all
 * memory.  Calls are asynchronous on hip_stream; tensors of one state must not
 * be used on two streams at once. */

/* Workspace for cfz_lowrank_ef_compress in bytes (0 if the sizes are
 * invalid): A, the bf16 residual [batch][m][n], at offset 0 -- left there by
 * the call, for inspection -- then, from the next 256-byte boundary, the
 * workspace of cfz_lowrank. */
size_t cfz_lowrank_ef_workspace_bytes(int64_t batch, int64_t m, int64_t n, int32_t r);

/* Warm-up (t = 0, the uncompressed step; reproducibility table, "Dataset
 * Splits"): prev = x0 and err = 0 at the sender, base = fp32(x0) at the
 * receiver, over `count` elements (a multiple of 8).  prev, err and base may
 * each be NULL (not written); x0 NULL means zeros.
 * Errors: CFZ_ERR_SHAPE, CFZ_ERR_ALIGN, CFZ_ERR_HIP. */
cfz_status cfz_lowrank_ef_warmup(int64_t count, const uint16_t *x0_bf16, uint16_t *prev_bf16,
                                 float *err, float *base, void *hip_stream);

/* One sender step (above).  Q0: [batch][n][r] fp32 random sample of the
 * subspace iteration; passing the previous step's V warm-starts it (Q0 may be
 * the V buffer itself: it is read in full before V is written).  Outputs
 * U, V, RU; updates prev and err in place.  Workspace: at least
 * cfz_lowrank_ef_workspace_bytes(batch, m, n, r) bytes, 256-byte aligned.
 * Errors: CFZ_ERR_NULL, CFZ_ERR_SHAPE, CFZ_ERR_ALIGN, CFZ_ERR_WORKSPACE,
 * CFZ_ERR_HIP; on error nothing is enqueued. */
cfz_status cfz_lowrank_ef_compress(int64_t batch, int64_t m, int64_t n, int32_t r, int32_t T,
                                   const uint16_t *x_bf16, uint16_t *prev_bf16, float *err,
                                   const float *Q0, float *U, float *V, float *RU,
                                   void *workspace, size_t ws_bytes, void *hip_stream);

/* The sender step with its last pass deferred: the call stops after the
 * subspace iteration and leaves the residual r in err; the update
 * err' = r - (U R_U) V^T is applied by the next deferred call, inside its own
 * residual pass (pending = 1), which reads each element of err once instead of
 * twice, or by cfz_lowrank_ef_flush.  pending = 0: err holds the carried error
 * (as after cfz_lowrank_ef_warmup or cfz_lowrank_ef_compress); pending = 1: the
 * previous call was deferred and U, V, RU still hold its factors, with the same
 * batch, m, n and r.  For the same inputs a run of deferred calls followed by
 * cfz_lowrank_ef_flush leaves prev, err, U, V and RU bit for bit as the same run
 * of cfz_lowrank_ef_compress calls; the factors of each call are those of the
 * plain call, so the receiver is unchanged.  Other arguments, workspace and
 * errors as cfz_lowrank_ef_compress (Q0 may be the V buffer, the pending
 * update only reads it), plus CFZ_ERR_SHAPE for pending not 0 or 1. */
cfz_status cfz_lowrank_ef_compress_deferred(int64_t batch, int64_t m, int64_t n, int32_t r,
                                            int32_t T, int32_t pending, const uint16_t *x_bf16,
                                            uint16_t *prev_bf16, float *err, const float *Q0,
                                            float *U, float *V, float *RU, void *workspace,
                                            size_t ws_bytes, void *hip_stream);

/* Applies a deferred call's pending update: err -= (U R_U) V^T, with the
 * factors that call wrote (the same kernel and rounding as the plain sender).
 * Errors: CFZ_ERR_NULL, CFZ_ERR_SHAPE, CFZ_ERR_ALIGN, CFZ_ERR_HIP. */
cfz_status cfz_lowrank_ef_flush(int64_t batch, int64_t m, int64_t n, int32_t r, const float *U,
                                const float *V, const float *RU, float *err, void *hip_stream);

/* One receiver step (above): base += (U R_U) V^T; xhat_bf16 (nullable)
 * receives bf16(base') rounded to nearest even.
 * Errors: CFZ_ERR_NULL, CFZ_ERR_SHAPE, CFZ_ERR_ALIGN, CFZ_ERR_HIP. */
cfz_status cfz_lowrank_ef_decompress(int64_t batch, int64_t m, int64_t n, int32_t r,
                                     const float *U, const float *V, const float *RU, float *base,
                                     uint16_t *xhat_bf16, void *hip_stream);

/* Measurement aid: a plain streaming copy of `bytes` bytes (multiple of 16,
 * both pointers 16-byte aligned) on hip_stream, used to calibrate HBM
 * traffic counters and the achievable copy bandwidth.  Not part of the codec. */
cfz_status cfz_stream_copy(const void *src, void *dst, size_t bytes, void *hip_stream);

/* Measurement aid: reads src_bytes and writes dst_bytes (<= src_bytes; both
 * multiples of 16, pointers 16-byte aligned, src_bytes <= 2^35): 16-byte
 * vector i of src is stored to vector floor(i * nw / nr) of dst when that index
 * steps (nr, nw: the vector counts), so the writes are spread evenly through the
 * reads.  With the codec's own ratio (compress 8 : 6.5625 bytes per element) it
 * measures what a plain stream of that read:write mix reaches.  Not part of the
 * codec. */
cfz_status cfz_stream_mix(const void *src, size_t src_bytes, void *dst, size_t dst_bytes,
                          void *hip_stream);

const char *cfz_status_string(cfz_status status);
const char *cfz_last_error(void);
int cfz_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CFZ_H */
