"""Pins of the oracle's rank-r compressor inside the error-feedback loop (CPU only).

What fixes it without reference to the oracle's own code: the residual and its
bf16 rounding recomputed with numpy's IEEE float32 and integer operations; a
zero residual; an exactly low-rank residual that must be transmitted exactly;
the telescoping identity sum of reconstructions + carried error = X_T - X_0
(with the reconstructions U R_U V^T formed by numpy); the receiver tracking
X_t - E_t; and the update formula against numpy's matmul."""
import numpy as np
import pytest
import torch

import oracle
from synth import LowrankDrift, exact_rank_batch, gaussian_q0


def bits16(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def widen(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rne_bf16(f32):
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def recon(U, V, RU):
    return (U @ RU) @ V.T


def test_residual_rounding_and_prev():
    m, n, r = 24, 40, 4
    rng = np.random.default_rng(0)
    x = rne_bf16(rng.standard_normal(m * n).astype(np.float32))
    p = rne_bf16(rng.standard_normal(m * n).astype(np.float32))
    e = (rng.standard_normal(m * n) * 0.1).astype(np.float32)
    s = oracle.LowrankSender(m, n)
    s.prev[:] = p
    s.err[:] = e
    q0 = gaussian_q0(1, n, r, seed=1)[0].numpy()
    U, V, RU, A = s.compress(x, q0, 1)
    res = (widen(x) - widen(p)) + e           # numpy float32: IEEE, no contraction
    assert np.array_equal(A, rne_bf16(res))
    assert np.array_equal(s.prev, x)
    # the carried error is what the reconstruction of A's factors misses of the fp32 residual
    want = res.astype(np.float64) - recon(U, V, RU).reshape(-1)
    assert np.allclose(s.err, want, rtol=2 ** -23, atol=1e-12)


def test_zero_residual_sends_nothing_and_keeps_state():
    m, n, r = 32, 48, 8
    x = bits16(torch.randn(m, n).to(torch.bfloat16))
    s = oracle.LowrankSender(m, n, x0=x)
    rc = oracle.LowrankReceiver(m, n, x0=x)
    base0 = rc.base.copy()
    U, V, RU, A = s.compress(x, gaussian_q0(1, n, r, seed=2)[0].numpy(), 2)
    assert not A.any() and not U.any() and not V.any() and not RU.any()
    assert not s.err.any()
    rc.decompress(U, V, RU)
    assert np.array_equal(rc.base, base0)


@pytest.mark.parametrize("rank,r", [(4, 4), (8, 16), (16, 16)])
def test_exact_low_rank_residual_is_transmitted_exactly(rank, r):
    """x - prev = F G^T with ternary F, G (integers, exact in bf16) and rank <= r: the receiver
    reproduces x and the carried error vanishes, both to fp64 rounding (every nonzero entry
    of x, an integer, comes out exact in fp32)."""
    m, n = 64, 96
    x = bits16(exact_rank_batch(1, m, n, rank, seed=rank)[0])
    s = oracle.LowrankSender(m, n)            # prev = 0, err = 0
    rc = oracle.LowrankReceiver(m, n)         # base = 0
    U, V, RU, A = s.compress(x, gaussian_q0(1, n, r, seed=3)[0].numpy(), 2)
    assert np.array_equal(A, x)
    xh = rc.decompress(U, V, RU, want_xhat=True)
    xf = widen(x)
    tol = 1e-12 * np.max(np.abs(xf))
    assert np.max(np.abs(rc.base - xf)) <= tol
    nz = xf != 0
    assert np.array_equal(rc.base[nz], xf[nz]) and np.array_equal(xh[nz], x[nz])
    assert np.max(np.abs(widen(xh) - xf)) <= tol
    assert np.max(np.abs(s.err)) <= tol


def test_telescoping_and_receiver_tracks_x_minus_e():
    m, n, r, T, steps = 48, 80, 8, 2, 8
    st = LowrankDrift(1, m, n, rank=6, sigma=0.05, seed=4)
    xs = [bits16(st.next()[0]) for _ in range(steps)]
    s = oracle.LowrankSender(m, n, x0=xs[0])
    rc = oracle.LowrankReceiver(m, n, x0=xs[0])
    dsum = np.zeros(m * n)
    for t in range(1, steps):
        q0 = gaussian_q0(1, n, r, seed=10 + t)[0].numpy()
        U, V, RU, _ = s.compress(xs[t], q0, T)
        rc.decompress(U, V, RU)
        dsum += recon(U, V, RU).reshape(-1)
        xt = widen(xs[t]).astype(np.float64)
        scale = np.max(np.abs(xt))
        # sum of reconstructions + carried error = X_t - X_0 (fp32 rounding per step)
        lhs = dsum + s.err
        assert np.max(np.abs(lhs - (xt - widen(xs[0])))) <= 8 * t * 2 ** -24 * scale
        # the receiver holds X_t - E_t up to the same rounding
        assert np.max(np.abs(rc.base - (xt - s.err))) <= 8 * t * 2 ** -24 * scale


def test_error_feedback_keeps_the_drift_bounded():
    """With the error carried, the receiver's error stays at the level of one step's residual
    that the rank-r reconstruction misses; dropping the carried error each step (open loop)
    lets the misses add up."""
    m, n, r, steps = 64, 96, 8, 12
    st = LowrankDrift(1, m, n, rank=12, sigma=0.05, seed=5)
    xs = [bits16(st.next()[0]) for _ in range(steps)]

    def run(carry):
        s = oracle.LowrankSender(m, n, x0=xs[0])
        rc = oracle.LowrankReceiver(m, n, x0=xs[0])
        for t in range(1, steps):
            if not carry:
                s.err[:] = 0
            U, V, RU, _ = s.compress(xs[t], gaussian_q0(1, n, r, seed=20 + t)[0].numpy(), 2)
            rc.decompress(U, V, RU)
        xt = widen(xs[-1])
        return np.linalg.norm(rc.base - xt) / np.linalg.norm(xt)

    assert run(True) < 0.7 * run(False)


def test_update_formula_against_numpy():
    rng = np.random.default_rng(6)
    m, n, r = 20, 36, 5
    U, V = rng.standard_normal((m, r)), rng.standard_normal((n, r))
    RU = np.triu(rng.standard_normal((r, r)))
    for sign in (1.0, -1.0):
        Y0 = rng.standard_normal(m * n).astype(np.float32)
        Y = Y0.copy()
        oracle.lowrank_ef_update(U, V, RU, sign, Y)
        want = Y0.astype(np.float64) + sign * recon(U, V, RU).reshape(-1)
        assert np.allclose(Y, want, rtol=2 ** -23, atol=1e-12)
        assert np.array_equal(Y, want.astype(np.float32)) or \
            np.max(np.abs(Y - want.astype(np.float32))) <= 2 ** -23 * np.max(np.abs(want))
