"""Pins of the CPU oracle's subspace iteration (paper "Accelerating Parallel
Diffusion Model Serving with Residual Compression", reproducibility table,
"Pseudocode", Algorithm 3) against facts that do not come from the oracle:
the defining properties of a thin QR, numpy's LAPACK QR and SVD as third-party
routines, the closed form of the iteration, exact-rank recovery and the
Eckart-Young bound."""
import numpy as np
import pytest
import torch

import oracle
from synth import exact_rank_batch, gaussian_q0, lowrank_batch


def bf16_np(t):
    return t.contiguous().view(torch.int16).numpy().view(np.uint16)


def bf16_to_f64(h):
    return (np.asarray(h, np.uint32) << 16).view(np.float32).astype(np.float64)


def lapack_qf(M):
    """Thin QR from LAPACK with the positive-diagonal convention (a third-party check)."""
    q, r = np.linalg.qr(M)
    d = np.sign(np.diag(r))
    d[d == 0] = 1
    return q * d, (r.T * d).T


@pytest.mark.parametrize("rows,cols", [(8, 8), (64, 5), (3072, 32), (1024, 16), (10, 1)])
def test_qr_defining_properties(rows, cols):
    rng = np.random.default_rng(rows * 131 + cols)
    M = rng.standard_normal((rows, cols))
    Q, R, dropped = oracle.qr(M)
    assert dropped == 0
    assert np.allclose(np.tril(R, -1), 0, atol=0)
    assert np.all(np.diag(R) > 0)
    assert np.linalg.norm(Q.T @ Q - np.eye(cols)) <= 1e-13 * cols
    assert np.linalg.norm(Q @ R - M) <= 1e-13 * np.linalg.norm(M)
    q2, r2 = lapack_qf(M)
    assert np.linalg.norm(Q - q2) <= 1e-11 * cols
    assert np.linalg.norm(R - r2) <= 1e-11 * np.linalg.norm(M)


def test_qr_drops_zero_columns_only():
    rng = np.random.default_rng(5)
    M = rng.standard_normal((50, 6))
    M[:, 2] = 0.0
    Q, R, dropped = oracle.qr(M)
    assert dropped == 1
    assert not Q[:, 2].any() and not R[2, :].any() and not R[:, 2].any()
    keep = [0, 1, 3, 4, 5]
    q2, r2 = lapack_qf(M[:, keep])
    assert np.linalg.norm(Q[:, keep] - q2) <= 1e-12
    assert np.linalg.norm(R[np.ix_(keep, keep)] - r2) <= 1e-12 * np.linalg.norm(M)
    Q, R, dropped = oracle.qr(np.zeros((20, 4)))
    assert dropped == 4 and not Q.any() and not R.any()


@pytest.mark.parametrize("m,n,r,T", [(8, 8, 3, 1), (8, 8, 8, 2), (40, 24, 4, 2), (64, 96, 6, 0),
                                     (64, 96, 6, 3)])
def test_algorithm3_closed_form(m, n, r, T):
    """Q_T = orth((A^T A)^T Q0): the triangular factors of successive QRs compose."""
    A = bf16_np(lowrank_batch(1, m, n, rank=min(m, n), sigma=0.3, seed=m + n + r)[0])
    Q0 = gaussian_q0(1, n, r, seed=r + T)[0].numpy()
    U, V, RU = oracle.lowrank(A, Q0, T)
    Af = bf16_to_f64(A)
    Qt, _ = lapack_qf(np.linalg.matrix_power(Af.T @ Af, T) @ Q0.astype(np.float64))
    assert np.linalg.norm(V - Qt) <= 1e-9 * r
    Ut, Rt = lapack_qf(Af @ Qt)
    assert np.linalg.norm(U - Ut) <= 1e-9 * r
    assert np.linalg.norm(RU - Rt) <= 1e-9 * np.linalg.norm(Rt)
    # reconstruction U R_U V^T equals (A Q) Q^T
    assert np.linalg.norm(U @ RU @ V.T - (Af @ V) @ V.T) <= 1e-12 * np.linalg.norm(Af)


@pytest.mark.parametrize("r", [8, 16, 32])
def test_exact_rank_recovery(r):
    m, n = 256, 384
    A = bf16_np(exact_rank_batch(1, m, n, r, seed=r)[0])
    Af = bf16_to_f64(A)
    assert np.linalg.matrix_rank(Af) == r
    Q0 = gaussian_q0(1, n, r, seed=3)[0].numpy()
    U, V, RU = oracle.lowrank(A, Q0, 2)
    rel = np.linalg.norm(Af - U @ RU @ V.T) / np.linalg.norm(Af)
    assert rel <= 1e-4
    assert rel <= 1e-12  # in fp64 the recovery is exact up to rounding


@pytest.mark.slow
def test_exact_rank_recovery_full_layer_shape():
    m, n, r = 1024, 3072, 16
    A = bf16_np(exact_rank_batch(1, m, n, r, seed=11)[0])
    Af = bf16_to_f64(A)
    Q0 = gaussian_q0(1, n, r, seed=4)[0].numpy()
    U, V, RU = oracle.lowrank(A, Q0, 2)
    assert np.linalg.norm(Af - U @ RU @ V.T) / np.linalg.norm(Af) <= 1e-12


@pytest.mark.parametrize("r,T", [(4, 2), (8, 2), (8, 6), (16, 2)])
def test_eckart_young_bound_and_orthonormality(r, T):
    m, n = 128, 192
    A = bf16_np(lowrank_batch(1, m, n, rank=8, sigma=0.05, seed=r * 10 + T)[0])
    Af = bf16_to_f64(A)
    Q0 = gaussian_q0(1, n, r, seed=T)[0].numpy()
    U, V, RU = oracle.lowrank(A, Q0, T)
    sv = np.linalg.svd(Af, compute_uv=False)
    floor = np.sqrt(np.sum(sv[r:] ** 2))
    err = np.linalg.norm(Af - U @ RU @ V.T)
    assert err >= floor * (1 - 1e-12)
    assert np.linalg.norm(U.T @ U - np.eye(r)) <= 1e-12
    assert np.linalg.norm(V.T @ V - np.eye(r)) <= 1e-12
    if r == 8:  # a clear spectral gap after the rank-8 signal: the iteration reaches the floor
        assert err <= floor * (1 + 1e-3)


def test_converges_to_truncated_svd_with_gap():
    """Many iterations on a matrix with a spectral gap give the best rank-r approximation."""
    rng = np.random.default_rng(9)
    m, n, r = 48, 40, 3
    u, _ = np.linalg.qr(rng.standard_normal((m, m)))
    v, _ = np.linalg.qr(rng.standard_normal((n, n)))
    s = np.concatenate([[64.0, 32.0, 16.0], np.linspace(1.0, 0.5, n - 3)])
    Af = (u[:, :n] * s) @ v.T
    A = oracle.f32_to_bf16(Af.astype(np.float32)).reshape(m, n)
    Af = bf16_to_f64(A)
    uu, ss, vv = np.linalg.svd(Af)
    best = (uu[:, :r] * ss[:r]) @ vv[:r]
    Q0 = rng.standard_normal((n, r)).astype(np.float32)
    U, V, RU = oracle.lowrank(A, Q0, 30)
    assert np.linalg.norm(U @ RU @ V.T - best) <= 1e-9 * np.linalg.norm(best)


def test_zero_matrix_gives_zero_factors():
    A = np.zeros((32, 48), np.uint16)
    Q0 = gaussian_q0(1, 48, 4)[0].numpy()
    U, V, RU = oracle.lowrank(A, Q0, 2)
    assert not U.any() and not V.any() and not RU.any()


def test_lowrank_deterministic():
    A = bf16_np(lowrank_batch(1, 64, 96, seed=1)[0])
    Q0 = gaussian_q0(1, 96, 8)[0].numpy()
    a = oracle.lowrank(A, Q0, 2)
    b = oracle.lowrank(A, Q0, 2)
    for x, y in zip(a, b):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64))
