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


def _state_values(c, key, bf16):
    v = floats(c[key])
    return to_bf16_bits(v) if bf16 else v


def _state_bits(a, bf16):
    return a if bf16 else bits32(a)


@pytest.mark.parametrize("case", sorted(load_ini("compress_steps.ini")))
def test_compress_fixture(case):
    c = load_ini("compress_steps.ini")[case]
    bits, group, mode = int(c["bits"]), int(c["group"]), MODES[c["mode"]]
    sb = c.get("state", "f32") == "bf16"
    x = to_bf16_bits(floats(c["x"]))
    n = x.size
    s = oracle.Sender(n, bits, group, mode, state_bf16=sb)
    if s.prev is not None:
        s.prev[:] = to_bf16_bits(floats(c["prev"]))
    if s.err is not None:
        s.err[:] = _state_values(c, "err", sb)
    if s.base is not None:
        s.base[:] = _state_values(c, "base", sb)
    codes, scales = s.compress(x)
    assert np.array_equal(codes, hexbytes(c["codes"]))
    assert np.array_equal(bits32(scales), bits32(floats(c["scales"])))
    if "err_out" in c:
        assert np.array_equal(_state_bits(s.err, sb), _state_bits(_state_values(c, "err_out", sb), sb))
    if "base_out" in c:
        assert np.array_equal(_state_bits(s.base, sb), _state_bits(_state_values(c, "base_out", sb), sb))
    if s.prev is not None:
        assert np.array_equal(s.prev, x)


@pytest.mark.parametrize("case", sorted(load_ini("decode_steps.ini")))
def test_decode_fixture(case):
    c = load_ini("decode_steps.ini")[case]
    bits, group = int(c["bits"]), int(c["group"])
    sb = c.get("state", "f32") == "bf16"
    base = _state_values(c, "base", sb)
    r = oracle.Receiver(base.size, bits, group, state_bf16=sb)
    r.base[:] = base
    xhat = r.decompress(hexbytes(c["codes"]), floats(c["scales"]), want_xhat=True)
    assert np.array_equal(_state_bits(r.base, sb), _state_bits(_state_values(c, "base_out", sb), sb))
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


# ---------------------------------------------------------------- bf16 state

def _bf16_ulp_half(v):
    """Half a bf16 ulp at |v| (for normal numbers; at least the smallest subnormal step)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0 ** -126)))
    return np.maximum(2.0 ** (e - 8), 2.0 ** -134)


@pytest.mark.parametrize("bits,group", [(4, 64), (2, 32)])
def test_bf16_state_closed_loop_sync_and_bound(bits, group):
    """OFF mode with bf16 bases: sender and receiver stay bit-identical, and the receiver is
    within half a quantization step plus half a bf16 ulp of every activation."""
    steps = 12
    sp = SPECS["tiny"]
    stream = AR1Stream(1, 256, 512, sp.alpha, sp.noise, 0.0, seed=3, key="tiny")
    xs = [bf16_np(stream.next()) for _ in range(steps)]
    n = xs[0].size
    snd = oracle.Sender(n, bits, group, oracle.OFF, x0=xs[0], state_bf16=True)
    rcv = oracle.Receiver(n, bits, group, x0=xs[0], state_bf16=True)
    for t in range(1, steps):
        codes, scales = snd.compress(xs[t])
        rcv.decompress(codes, scales)
        assert np.array_equal(snd.base, rcv.base)
        b = bf16_bits_to_f64(rcv.base)
        s = np.repeat(scales.astype(np.float64), group)
        err = np.abs(bf16_bits_to_f64(xs[t]) - b)
        assert np.all(err <= s / 2 * (1 + 2.0 ** -20) + _bf16_ulp_half(b) * 1.0001)


def test_bf16_state_zero_residual_and_error_bound():
    rng = np.random.default_rng(4)
    n = 4096
    x0 = oracle.f32_to_bf16(rng.standard_normal(n).astype(np.float32))
    for mode in (oracle.DELTA, oracle.LITERAL, oracle.OFF):
        s = oracle.Sender(n, 4, 64, mode, x0=x0, state_bf16=True)
        before = [None if b is None else b.copy() for b in (s.prev, s.err, s.base)]
        codes, scales = s.compress(x0)
        assert not codes.any() and not scales.any()
        for b, a in zip(before, (s.prev, s.err, s.base)):
            if b is not None:
                assert np.array_equal(b, a)
    # DELTA with a bf16 error buffer: |E| <= s/2 up to its bf16 rounding
    sp = SPECS["flux"]
    stream = AR1Stream(1, 256, 512, sp.alpha, sp.noise, 0.01, seed=0, key="flux")
    xs = [bf16_np(stream.next()) for _ in range(6)]
    snd = oracle.Sender(xs[0].size, 4, 64, oracle.DELTA, x0=xs[0], state_bf16=True)
    for t in range(1, 6):
        codes, scales = snd.compress(xs[t])
        e = np.abs(bf16_bits_to_f64(snd.err))
        s = np.repeat(scales.astype(np.float64), 64)
        assert np.all(e <= s / 2 * (1 + 2.0 ** -8) + 2.0 ** -133)


@pytest.mark.parametrize("mode", [oracle.DELTA, oracle.OFF])
def test_bf16_state_accuracy_matches_fp32_state(mode):
    """Keeping the state in bf16 changes the reconstruction error by well under 5% here."""
    def final_err(sb):
        sp = SPECS["flux"]
        stream = AR1Stream(1, 256, 512, sp.alpha, sp.noise, 0.01, seed=0, key="flux")
        xs = [bf16_np(stream.next()) for _ in range(28)]
        snd = oracle.Sender(xs[0].size, 4, 64, mode, x0=xs[0], state_bf16=sb)
        rcv = oracle.Receiver(xs[0].size, 4, 64, x0=xs[0], state_bf16=sb)
        for t in range(1, 28):
            rcv.decompress(*snd.compress(xs[t]))
        b = bf16_bits_to_f64(rcv.base) if sb else rcv.base.astype(np.float64)
        xt = bf16_bits_to_f64(xs[-1])
        return np.linalg.norm(xt - b) / np.linalg.norm(xt)
    e32, e16 = final_err(False), final_err(True)
    assert abs(e16 - e32) <= 0.05 * e32


def _rne_bf16_numpy(f32):
    """fp32 -> bf16 bits, round to nearest even, written with integer ops (finite inputs)."""
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("mode", [oracle.DELTA, oracle.LITERAL, oracle.OFF])
@pytest.mark.parametrize("bits,group", [(4, 64), (2, 8)])
def test_bf16_state_step_is_fp32_step_rounded(mode, bits, group):
    """From a state that is exact in bf16, one bf16-state step gives the same codes and scales
    as the fp32-state step, and each state array equals the fp32 result rounded to bf16."""
    rng = np.random.default_rng(11 + mode + bits)
    n = 2048
    x = oracle.f32_to_bf16(rng.standard_normal(n).astype(np.float32))
    p = oracle.f32_to_bf16(rng.standard_normal(n).astype(np.float32))
    e16 = _rne_bf16_numpy((rng.standard_normal(n) * 0.05).astype(np.float32))
    b16 = _rne_bf16_numpy(rng.standard_normal(n).astype(np.float32))
    b16[::7] = x[::7]                       # some zero residuals in OFF mode
    widen = lambda h: (h.astype(np.uint32) << 16).view(np.float32)
    s32 = oracle.Sender(n, bits, group, mode)
    s16 = oracle.Sender(n, bits, group, mode, state_bf16=True)
    for s_, e_, b_ in ((s32, widen(e16), widen(b16)), (s16, e16, b16)):
        if s_.prev is not None:
            s_.prev[:] = p
        if s_.err is not None:
            s_.err[:] = e_
        if s_.base is not None:
            s_.base[:] = b_
    c32, sc32 = s32.compress(x)
    c16, sc16 = s16.compress(x)
    assert np.array_equal(c32, c16) and np.array_equal(sc32.view(np.uint32), sc16.view(np.uint32))
    for a32, a16 in ((s32.err, s16.err), (s32.base, s16.base)):
        if a32 is not None:
            assert np.array_equal(_rne_bf16_numpy(a32), a16)
    # receiver: one decode from the same bf16-exact base
    r32 = oracle.Receiver(n, bits, group)
    r16 = oracle.Receiver(n, bits, group, state_bf16=True)
    r32.base[:] = widen(b16)
    r16.base[:] = b16
    r32.decompress(c32, sc32)
    r16.decompress(c32, sc32)
    assert np.array_equal(_rne_bf16_numpy(r32.base), r16.base)


# ---------------------------------------------------------------- lost payload and recovery

def _stream_xs(steps, seed=21):
    sp = SPECS["flux"]
    st = AR1Stream(1, 128, 512, sp.alpha, sp.noise, 0.01, seed=seed, key="flux")
    return [bf16_np(st.next()) for _ in range(steps)]


def test_lost_payload_is_detected_and_rewarm_recovers():
    """Closed loop (OFF): the sender's and receiver's bases are bit-identical after every
    step, so one skipped decode shows up as a mismatch and stays.  Re-warming both sides from
    an uncompressed activation (the warm-up step) gives exactly the states of a fresh run
    started there."""
    xs = _stream_xs(10)
    n = xs[0].size
    snd = oracle.Sender(n, 4, 64, oracle.OFF, x0=xs[0])
    rcv = oracle.Receiver(n, 4, 64, x0=xs[0])
    for t in range(1, 6):
        codes, scales = snd.compress(xs[t])
        if t != 3:  # the payload of step 3 is lost
            rcv.decompress(codes, scales)
        assert np.array_equal(snd.base, rcv.base) == (t < 3), f"step {t}"
    # re-warm both from x_5, next to a fresh pair started at x_5
    snd = oracle.Sender(n, 4, 64, oracle.OFF, x0=xs[5])
    rcv = oracle.Receiver(n, 4, 64, x0=xs[5])
    fs = oracle.Sender(n, 4, 64, oracle.OFF, x0=xs[5])
    fr = oracle.Receiver(n, 4, 64, x0=xs[5])
    for t in range(6, 10):
        c1, s1 = snd.compress(xs[t])
        c2, s2 = fs.compress(xs[t])
        rcv.decompress(c1, s1)
        fr.decompress(c2, s2)
        assert np.array_equal(c1, c2) and np.array_equal(s1.view(np.uint32), s2.view(np.uint32))
        assert np.array_equal(snd.base, rcv.base) and np.array_equal(rcv.base, fr.base)


def test_lost_payload_in_delta_mode_shows_in_the_error():
    """DELTA: the receiver tracks X - E, so its error stays at the quantizer's level; a lost
    payload leaves it behind by that step's whole residual, which never comes back."""
    xs = _stream_xs(10, seed=22)
    n = xs[0].size

    def errs(skip):
        snd = oracle.Sender(n, 4, 64, oracle.DELTA, x0=xs[0])
        rcv = oracle.Receiver(n, 4, 64, x0=xs[0])
        out = []
        for t in range(1, 10):
            codes, scales = snd.compress(xs[t])
            if t != skip:
                rcv.decompress(codes, scales)
            xt = bf16_bits_to_f64(xs[t])
            out.append(np.linalg.norm(xt - rcv.base) / np.linalg.norm(xt))
        return out

    clean, lost = errs(None), errs(4)
    assert lost[:3] == clean[:3]
    assert all(l > 3 * c for l, c in zip(lost[3:], clean[3:]))
