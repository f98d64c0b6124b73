"""Pins of the CPU oracle's codec against facts that do not come from the oracle:
hand-derived fixtures, brute force on 8x8 tiles, closed-form bounds and the
invariants the method implies (paper "Accelerating Parallel Diffusion Model
Serving with Residual Compression": abstract -- compressed step-wise residuals
with error feedback that prevents error accumulation; reproducibility table,
"Dataset Splits" -- one uncompressed warm-up step initialises the base)."""
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from synth import AR1Stream, SPECS
from tests._fixtures import (MODES, bits32, floats, hexbytes, hexwords, ints, load_ini,
                             to_bf16_bits)

U32 = 2.0 ** -24


def bf16_np(t: torch.Tensor) -> np.ndarray:
    return t.contiguous().view(torch.int16).numpy().view(np.uint16).reshape(-1)


def bf16_bits_to_f64(h):
    return (np.asarray(h, np.uint32) << 16).view(np.float32).astype(np.float64)


# ---------------------------------------------------------------- fixtures

@pytest.mark.parametrize("case", sorted(load_ini("packing.ini")))
def test_packing_fixture(case):
    c = load_ini("packing.ini")[case]
    if case == "bf16_rne":
        f = hexwords(c["f32"], np.uint32).view(np.float32)
        want = hexwords(c["bf16"], np.uint16)
        assert np.array_equal(oracle.f32_to_bf16(f), want)
        return
    bits = int(c["bits"])
    q = ints(c["q"])
    codes = oracle.pack_codes(q, bits)
    assert np.array_equal(codes, hexbytes(c["codes"]))
    assert np.array_equal(oracle.unpack_codes(codes, q.size, bits), q)


@pytest.mark.parametrize("bits", [2, 4])
def test_pack_unpack_roundtrip_every_value(bits):
    lo, hi = -(1 << (bits - 1)), (1 << (bits - 1)) - 1
    rng = np.random.default_rng(1)
    q = rng.integers(lo, hi + 1, size=4096).astype(np.int8)
    q[: hi - lo + 1] = np.arange(lo, hi + 1)
    assert np.array_equal(oracle.unpack_codes(oracle.pack_codes(q, bits), q.size, bits), q)


@pytest.mark.parametrize("case", sorted(load_ini("compress_steps.ini")))
def test_compress_fixture(case):
    c = load_ini("compress_steps.ini")[case]
    bits, group, mode = int(c["bits"]), int(c["group"]), MODES[c["mode"]]
    x = to_bf16_bits(floats(c["x"]))
    n = x.size
    s = oracle.Sender(n, bits, group, mode)
    if s.prev is not None:
        s.prev[:] = to_bf16_bits(floats(c["prev"]))
    if s.err is not None:
        s.err[:] = floats(c["err"])
    if s.base is not None:
        s.base[:] = floats(c["base"])
    codes, scales = s.compress(x)
    assert np.array_equal(codes, hexbytes(c["codes"]))
    assert np.array_equal(bits32(scales), bits32(floats(c["scales"])))
    if "err_out" in c:
        assert np.array_equal(bits32(s.err), bits32(floats(c["err_out"])))
    if "base_out" in c:
        assert np.array_equal(bits32(s.base), bits32(floats(c["base_out"])))
    if s.prev is not None:
        assert np.array_equal(s.prev, x)


@pytest.mark.parametrize("case", sorted(load_ini("decode_steps.ini")))
def test_decode_fixture(case):
    c = load_ini("decode_steps.ini")[case]
    bits, group = int(c["bits"]), int(c["group"])
    base = floats(c["base"])
    r = oracle.Receiver(base.size, bits, group)
    r.base[:] = base
    xhat = r.decompress(hexbytes(c["codes"]), floats(c["scales"]), want_xhat=True)
    assert np.array_equal(bits32(r.base), bits32(floats(c["base_out"])))
    assert np.array_equal(xhat, to_bf16_bits(floats(c["xhat"])))


# ---------------------------------------------------------------- brute force (8x8 tiles)

def _frac_to_f32(fr: Fraction) -> np.float32:
    """Exact rational -> nearest fp32, ties to even (used for brute-force expectations)."""
    c = np.float32(float(fr))
    best = None
    for cand in (np.nextafter(c, np.float32(-np.inf)), c, np.nextafter(c, np.float32(np.inf))):
        d = abs(Fraction(float(cand)) - fr)
        key = (d, int(np.array(cand, np.float32).view(np.uint32)) & 1)
        if best is None or key < best[0]:
            best = (key, cand)
    return np.float32(best[1])


def _brute_group(r32, bits):
    """Exhaustive argmin over all 2^b codes of |r - c s|, exact rationals, ties to even c."""
    qmax = (1 << (bits - 1)) - 1
    a = max(abs(float(v)) for v in r32)
    s = np.float32(np.float32(a) / np.float32(qmax))  # the one IEEE division of the scale
    out, ambiguous = [], []
    for v in r32:
        if s == 0:
            out.append(0)
            ambiguous.append(False)
            continue
        rv, sv = Fraction(float(v)), Fraction(float(s))
        cands = range(-(1 << (bits - 1)), 1 << (bits - 1))
        dists = sorted((abs(rv - c * sv), c % 2, c) for c in cands)
        out.append(dists[0][2])
        # a near-tie that fp32 division could resolve either way
        t = rv / sv
        frac = t - (t.numerator // t.denominator)
        ambiguous.append(abs(frac - Fraction(1, 2)) <= Fraction(1, 1 << 20) * abs(t))
    return s, out, ambiguous


@pytest.mark.parametrize("bits,group", [(4, 8), (4, 64), (2, 8), (2, 64)])
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_brute_force_8x8_tiles(bits, group, seed):
    rng = np.random.default_rng(100 + seed)
    n = 64
    sc = np.exp(0.5 * rng.standard_normal(8)).repeat(8)
    x = to_bf16_bits(oracle.bf16_to_f32(oracle.f32_to_bf16(
        (rng.standard_normal(n) * sc).astype(np.float32))))
    prev = oracle.f32_to_bf16((rng.standard_normal(n) * sc).astype(np.float32))
    err = (rng.standard_normal(n) * 0.05).astype(np.float32)
    if seed == 2:  # exact ties: residuals on a half-integer lattice of the scale
        x = to_bf16_bits(np.round(rng.uniform(-7, 7, n) * 2) / 2)
        prev[:] = 0
        err[:] = 0
        x[0] = to_bf16_bits(np.float32([7.0]))[0]
    s = oracle.Sender(n, bits, group, oracle.DELTA)
    s.prev[:] = prev
    s.err[:] = err
    codes, scales = s.compress(x)
    q = oracle.unpack_codes(codes, n, bits)

    xf = bf16_bits_to_f64(x)
    pf = bf16_bits_to_f64(prev)
    for g in range(n // group):
        sl = slice(g * group, (g + 1) * group)
        # residual with one rounding per fp32 operation, as the definition states
        r32 = [_frac_to_f32(_frac_to_f32(Fraction(xv) - Fraction(pv)) + Fraction(float(ev)))
               for xv, pv, ev in zip(xf[sl], pf[sl], err[sl])]
        s_bf, q_bf, amb = _brute_group(r32, bits)
        assert bits32(scales[g]) == bits32(s_bf)
        for i, (qo, qb, am) in enumerate(zip(q[sl], q_bf, amb)):
            if not am:
                assert qo == qb, (g, i, qo, qb)
            else:
                assert abs(int(qo) - qb) <= 1
            # err' = r - q s with a single rounding
            e_bf = _frac_to_f32(Fraction(float(r32[i])) - int(qo) * Fraction(float(s_bf)))
            assert bits32(s.err[g * group + i]) == bits32(e_bf)
    assert np.array_equal(s.prev, x)


# ---------------------------------------------------------------- closed-form bounds

@pytest.mark.parametrize("bits,group", [(4, 64), (2, 32), (4, 8), (2, 128)])
def test_error_at_most_half_scale(bits, group):
    rng = np.random.default_rng(7)
    n = 256 * 512
    sc = np.exp(0.5 * rng.standard_normal(512))
    r = (rng.standard_normal((256, 512)) * sc).astype(np.float32).reshape(-1)
    r[:group] = 0.0                      # an all-zero group
    r[group:2 * group] = 1e-42           # subnormal residuals
    codes, scales = oracle.quantize(r, bits, group)
    q = oracle.unpack_codes(codes, n, bits).astype(np.float64)
    qmax = (1 << (bits - 1)) - 1
    assert np.all(np.abs(q) <= qmax)
    s = np.repeat(scales.astype(np.float64), group)
    err = np.abs(r.astype(np.float64) - q * s)
    assert np.all(err <= s / 2 * (1 + 2.0 ** -20) + 1e-45)
    # the scale is the group's absmax over qmax, rounded once
    a = np.abs(r.astype(np.float64)).reshape(-1, group).max(axis=1)
    assert np.all(np.abs(scales.astype(np.float64) * qmax - a) <= a * 2.0 ** -23)
    assert scales[0] == 0 and np.all(q[:group] == 0)
    # the largest element of every nonzero group is coded as +-qmax
    big = np.abs(r).reshape(-1, group).argmax(axis=1)
    qg = q.reshape(-1, group)[np.arange(n // group), big]
    nz = scales > 0
    assert np.all(np.abs(qg[nz]) == qmax)


def test_zero_residual_gives_zero_codes_and_unchanged_state():
    for mode in (oracle.DELTA, oracle.LITERAL, oracle.OFF):
        rng = np.random.default_rng(3)
        n = 4096
        x0 = oracle.f32_to_bf16(rng.standard_normal(n).astype(np.float32))
        s = oracle.Sender(n, 4, 64, mode, x0=x0)
        r = oracle.Receiver(n, 4, 64, x0=x0)
        before = [None if b is None else b.copy() for b in (s.prev, s.err, s.base)]
        codes, scales = s.compress(x0)
        assert not codes.any() and not scales.any()
        for b, a in zip(before, (s.prev, s.err, s.base)):
            if b is not None:
                assert np.array_equal(b.view(np.uint8), a.view(np.uint8))
        base0 = r.base.copy()
        r.decompress(codes, scales)
        assert np.array_equal(base0.view(np.uint32), r.base.view(np.uint32))


# ---------------------------------------------------------------- invariants over time

def _run(mode, bits, group, steps, spec="tiny", seed=0):
    sp = SPECS[spec]
    stream = AR1Stream(1, 256, 512, sp.alpha, sp.noise, 0.01 if spec != "tiny" else 0.0,
                       seed=seed, key=spec)
    xs = [bf16_np(stream.next()) for _ in range(steps)]
    n = xs[0].size
    snd = oracle.Sender(n, bits, group, mode, x0=xs[0])
    rcv = oracle.Receiver(n, bits, group, x0=xs[0])
    return xs, snd, rcv


@pytest.mark.parametrize("bits,group", [(4, 64), (2, 32)])
def test_delta_telescoping(bits, group):
    """sum of decoded payloads + E_T = X_T - Xhat_0, and the receiver tracks X_t - E_t."""
    steps = 28
    xs, snd, rcv = _run(oracle.DELTA, bits, group, steps)
    n = xs[0].size
    dsum = np.zeros(n)
    xh0 = rcv.base.astype(np.float64).copy()
    for t in range(1, steps):
        codes, scales = snd.compress(xs[t])
        q = oracle.unpack_codes(codes, n, bits).astype(np.float64)
        dsum += q * np.repeat(scales.astype(np.float64), group)
        rcv.decompress(codes, scales)
        xt = bf16_bits_to_f64(xs[t])
        mag = max(np.abs(xt).max(), np.abs(rcv.base).max())
        # receiver's base equals X_t - E_t up to fp32 rounding of each update
        assert np.abs(rcv.base - (xt - snd.err)).max() <= 4 * t * U32 * mag
        lhs = dsum + snd.err.astype(np.float64)
        assert np.abs(lhs - (xt - xh0)).max() <= 4 * t * U32 * mag
        assert np.all(np.abs(snd.err) <= np.repeat(scales, group) / 2 * (1 + 2.0 ** -20) + 1e-45)


def test_literal_derived_invariant_and_sync():
    """LITERAL: Xhat_t + E_t - E_{t-1} = X_t per step; sender and receiver bases agree bitwise."""
    steps = 12
    xs, snd, rcv = _run(oracle.LITERAL, 4, 64, steps)
    for t in range(1, steps):
        e_prev = snd.err.astype(np.float64).copy()
        codes, scales = snd.compress(xs[t])
        rcv.decompress(codes, scales)
        assert np.array_equal(snd.base.view(np.uint32), rcv.base.view(np.uint32))
        xt = bf16_bits_to_f64(xs[t])
        mag = max(np.abs(xt).max(), np.abs(snd.base).max(), np.abs(snd.err).max())
        resid = snd.base.astype(np.float64) + snd.err - e_prev - xt
        assert np.abs(resid).max() <= 4 * U32 * mag


@pytest.mark.parametrize("bits,group", [(4, 64), (2, 32)])
def test_off_mode_sync_and_bound(bits, group):
    steps = 12
    xs, snd, rcv = _run(oracle.OFF, bits, group, steps)
    for t in range(1, steps):
        codes, scales = snd.compress(xs[t])
        rcv.decompress(codes, scales)
        assert np.array_equal(snd.base.view(np.uint32), rcv.base.view(np.uint32))
        err = np.abs(bf16_bits_to_f64(xs[t]) - rcv.base)
        s = np.repeat(scales.astype(np.float64), group)
        assert np.all(err <= s / 2 * (1 + 2.0 ** -20) + 2 * U32 * np.abs(rcv.base))


def _final_rel_err(mode, bits, group, steps=28, spec="flux"):
    xs, snd, rcv = _run(mode, bits, group, steps, spec=spec)
    errs = []
    for t in range(1, steps):
        codes, scales = snd.compress(xs[t])
        rcv.decompress(codes, scales)
        xt = bf16_bits_to_f64(xs[t])
        errs.append(np.linalg.norm(xt - rcv.base) / np.linalg.norm(xt))
    return errs


def _direct_rel_err(bits, group, steps=28, spec="flux"):
    sp = SPECS[spec]
    stream = AR1Stream(1, 256, 512, sp.alpha, sp.noise, 0.01, seed=0, key=spec)
    xs = [bf16_np(stream.next()) for _ in range(steps)]
    xt = oracle.bf16_to_f32(xs[-1])
    codes, scales = oracle.quantize(xt, bits, group)
    q = oracle.unpack_codes(codes, xt.size, bits).astype(np.float64)
    rec = q * np.repeat(scales.astype(np.float64), group)
    return np.linalg.norm(xt - rec) / np.linalg.norm(xt)


def test_ar1_workload_redundancy():
    """The workload's step-to-step change is about sqrt(2 (1 - alpha)) of the signal."""
    sp = SPECS["flux"]
    stream = AR1Stream(1, 256, 512, sp.alpha, sp.noise, 0.01, seed=0, key="flux")
    xs = [stream.next().double() for _ in range(12)]
    ratio = np.mean([float((xs[t] - xs[t - 1]).norm() / xs[t].norm()) for t in range(1, 12)])
    assert abs(ratio - np.sqrt(2 * (1 - sp.alpha))) < 0.02


@pytest.mark.parametrize("bits,group", [(4, 64), (2, 32)])
def test_residual_beats_direct_and_feedback_prevents_accumulation(bits, group):
    delta = _final_rel_err(oracle.DELTA, bits, group)
    off = _final_rel_err(oracle.OFF, bits, group)
    openloop = _final_rel_err(oracle.OPENLOOP, bits, group)
    direct = _direct_rel_err(bits, group)
    # closed-loop DELTA and OFF agree to rounding (they are equal in real arithmetic)
    assert abs(delta[-1] - off[-1]) <= 1e-3 * delta[-1]
    # residual compression with feedback is far more accurate than quantizing X directly
    assert direct / delta[-1] > 2.5
    # without feedback the error accumulates: rising, and well above the closed loop
    assert openloop[-1] > 2.5 * delta[-1]
    assert openloop[-1] > 1.5 * openloop[3]
    # with feedback it stays bounded
    assert max(delta) < 1.2 * max(delta[:5]) + 1e-3


def test_literal_reading_diverges_at_two_bits():
    """The literal 'R = X_t - Xhat_{t-1} + E' reading feeds the error back twice; with the
    ternary quantizer the loop is unstable (kept as a mode to show exactly that)."""
    lit = _final_rel_err(oracle.LITERAL, 2, 32, steps=28)
    delta = _final_rel_err(oracle.DELTA, 2, 32, steps=28)
    assert lit[-1] > 10 * delta[-1]
    assert delta[-1] < 0.3


def test_checkpoint_resume_and_determinism():
    steps, k = 10, 4
    xs, snd, rcv = _run(oracle.DELTA, 4, 64, steps)
    n = xs[0].size
    outs = []
    for t in range(1, steps):
        outs.append(snd.compress(xs[t]))
        rcv.decompress(*outs[-1])
    # second run: stop after k steps, copy the state out, restore it into fresh objects
    xs2, snd2, rcv2 = _run(oracle.DELTA, 4, 64, steps)
    for t in range(1, k + 1):
        c, s = snd2.compress(xs2[t])
        rcv2.decompress(c, s)
    saved = (snd2.prev.copy(), snd2.err.copy(), rcv2.base.copy())
    snd3 = oracle.Sender(n, 4, 64, oracle.DELTA)
    rcv3 = oracle.Receiver(n, 4, 64)
    snd3.prev[:], snd3.err[:], rcv3.base[:] = saved
    for t in range(k + 1, steps):
        c, s = snd3.compress(xs2[t])
        assert np.array_equal(c, outs[t - 1][0])
        assert np.array_equal(s.view(np.uint32), outs[t - 1][1].view(np.uint32))
        rcv3.decompress(c, s)
    assert np.array_equal(rcv3.base.view(np.uint32), rcv.base.view(np.uint32))
    assert np.array_equal(snd3.err.view(np.uint32), snd.err.view(np.uint32))
