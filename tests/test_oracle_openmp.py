"""The OpenMP build of the oracle (the one the benchmark times on all host cores) is the
same C source with its independent outer loops split among threads; every output is
computed by one thread in the serial build's order.  Its results must therefore be the
serial build's bit for bit: codec steps in every mode and state precision (ragged group
counts, more groups than threads), and the subspace iteration (every r class, T = 0..2)."""
import numpy as np
import pytest

import oracle
from synth import AR1Stream, gaussian_q0, lowrank_batch


def _u16(t):
    import torch
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def test_openmp_build_uses_several_threads():
    assert oracle.threads() == 1
    with oracle.parallel():
        assert oracle.threads() >= 1
    assert oracle.threads() == 1


@pytest.mark.parametrize("bits,group,mode,sb", [(4, 64, oracle.DELTA, False),
                                                (2, 32, oracle.DELTA, False),
                                                (4, 8, oracle.LITERAL, False),
                                                (2, 128, oracle.OFF, False),
                                                (4, 64, oracle.DELTA, True),
                                                (2, 16, oracle.OFF, True)])
def test_codec_steps_bit_identical(bits, group, mode, sb):
    rows, cols = 301, 512   # 301 rows: group counts that do not split evenly among threads
    st = AR1Stream(1, rows, cols, 0.98, 0.199, 0.01, seed=bits + group, key="omp")
    xs = [_u16(st.next()[0]) for _ in range(4)]
    n = rows * cols
    s1 = oracle.Sender(n, bits, group, mode, x0=xs[0], state_bf16=sb)
    r1 = oracle.Receiver(n, bits, group, x0=xs[0], state_bf16=sb)
    with oracle.parallel():
        s2 = oracle.Sender(n, bits, group, mode, x0=xs[0], state_bf16=sb)
        r2 = oracle.Receiver(n, bits, group, x0=xs[0], state_bf16=sb)
    for t in range(1, 4):
        c1, sc1 = s1.compress(xs[t])
        x1 = r1.decompress(c1, sc1, want_xhat=True)
        with oracle.parallel():
            c2, sc2 = s2.compress(xs[t])
            x2 = r2.decompress(c2, sc2, want_xhat=True)
        assert np.array_equal(c1, c2), f"step {t}: codes"
        assert np.array_equal(sc1.view(np.uint32), sc2.view(np.uint32)), f"step {t}: scales"
        for name in ("prev", "err", "base"):
            a, b = getattr(s1, name), getattr(s2, name)
            if a is not None:
                assert np.array_equal(a.view(np.uint8), b.view(np.uint8)), f"step {t}: {name}"
        assert np.array_equal(r1.base.view(np.uint8), r2.base.view(np.uint8)), f"step {t}: base"
        assert np.array_equal(x1, x2), f"step {t}: xhat"


def test_packing_bit_identical():
    rng = np.random.default_rng(5)
    for bits in (2, 4):
        qmax = (1 << (bits - 1)) - 1
        q = rng.integers(-qmax, qmax + 1, size=8 * 1001).astype(np.int8)
        p1 = oracle.pack_codes(q, bits)
        with oracle.parallel():
            p2 = oracle.pack_codes(q, bits)
            u2 = oracle.unpack_codes(p2, q.size, bits)
        assert np.array_equal(p1, p2) and np.array_equal(u2, q)


@pytest.mark.parametrize("r,T", [(1, 2), (8, 0), (8, 2), (16, 1), (32, 2)])
def test_lowrank_bit_identical(r, T):
    m, n = 96, 160
    A = _u16(lowrank_batch(1, m, n, rank=12, sigma=0.05, seed=r + T)[0]).reshape(m, n)
    Q0 = gaussian_q0(1, n, r, seed=T)[0].numpy()
    a = oracle.lowrank(A, Q0, T)
    with oracle.parallel():
        b = oracle.lowrank(A, Q0, T)
    for name, x, y in zip(("U", "V", "R_U"), a, b):
        assert np.array_equal(x.view(np.uint64), y.view(np.uint64)), name
