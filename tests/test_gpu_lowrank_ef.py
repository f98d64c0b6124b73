"""GPU parity of the rank-r compressor inside the error-feedback loop
(cfz_lowrank_ef_* through the C ABI) against the CPU oracle.

Each step is teacher-forced: the oracle starts from the GPU's state (prev, err
and base copied to the host), so the comparison is of one step, not of two
runs drifting apart through fp32 versus fp64 factors.  Bar:
- prev and the bf16 residual A bit-exact (plain fp32 arithmetic and one
  rounding on both sides);
- the reconstruction U R_U V^T and the new carried error within 1e-3 of the
  oracle's, relative to the residual's Frobenius norm (the subspace iteration
  runs in bf16 MFMA against fp64 Householder);
- the update itself -- err' = r - (U R_U) V^T at the sender, base' = base +
  (U R_U) V^T at the receiver -- checked on the GPU's own factors against an
  fp64 evaluation, to 1e-5 of the reconstruction's largest entry;
- xhat equal to the GPU's new base rounded to bf16.
Inputs: seeded activations whose step-to-step change is rank 16 plus noise."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import LowrankDrift, exact_rank_batch, gaussian_q0

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from diffusion_activation_residual_amd import cfz
DEV = "cuda:0"


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def widen(h):
    return (np.asarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def rne_bf16(f32):
    u = np.ascontiguousarray(f32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def f64(t):
    return t.detach().cpu().numpy().astype(np.float64)


def recon(U, V, RU):
    return (U @ RU) @ V.T


def _check_step(tag, b_idx, m, n, r, T, x_host, prev0, err0, base0, q0, snd, rcv, xhat,
                lead=None):
    """Compare matrix b_idx of one teacher-forced GPU step with the oracle.  The factors
    U, V and R_U are compared on their leading `lead` columns (all by default): past the
    rank of the drift the columns span noise and their basis depends on rounding."""
    sl = slice(b_idx * m * n, (b_idx + 1) * m * n)
    # oracle sender from the GPU's pre-step state
    os_ = oracle.LowrankSender(m, n)
    os_.prev[:] = prev0[sl]
    os_.err[:] = err0[sl]
    Uo, Vo, RUo, Ao = os_.compress(x_host[sl], q0, T)
    res = (widen(x_host[sl]) - widen(prev0[sl])) + err0[sl]   # fp32, as both sides compute it
    scale = np.linalg.norm(res.astype(np.float64)) + 1e-30

    A = u16(snd.residual_bf16()[sl])
    assert np.array_equal(A, Ao), f"{tag}: bf16 residual"
    assert np.array_equal(A, rne_bf16(res)), f"{tag}: bf16 residual vs numpy rounding"
    assert np.array_equal(u16(snd.prev[sl]), x_host[sl]), f"{tag}: prev"

    U, V, RU = f64(snd.U[b_idx]), f64(snd.V[b_idx]), f64(snd.RU[b_idx])
    D = recon(U, V, RU)
    Do = recon(Uo, Vo, RUo)
    rel = np.linalg.norm(D - Do) / scale
    assert rel <= 1e-3, f"{tag}: reconstruction differs from the oracle by {rel:.2e}"
    nd = np.linalg.norm(Do)
    if nd > 1e-6 * scale:  # a (near) zero reconstruction has no relative error to speak of
        rel_d = np.linalg.norm(D - Do) / nd
        assert rel_d <= 1e-3, f"{tag}: reconstruction {rel_d:.2e} from the oracle's, of |D|"
        k = r if lead is None else min(lead, r)
        for name, g, o in (("U", U[:, :k], Uo[:, :k]), ("V", V[:, :k], Vo[:, :k]),
                           ("R_U", RU[:k, :k], RUo[:k, :k])):
            e = np.linalg.norm(g - o) / (np.linalg.norm(o) + 1e-30)
            assert e <= 1e-3, f"{tag}: {name} differs from the oracle by {e:.2e}"

    err = snd.err[sl].cpu().numpy().astype(np.float64)
    rel_e = np.linalg.norm(err - os_.err.astype(np.float64)) / scale
    assert rel_e <= 1e-3, f"{tag}: carried error differs from the oracle by {rel_e:.2e}"
    say(f"  {tag}: reconstruction {rel:.1e}, carried error {rel_e:.1e} (relative to |r|)")
    # the update on the GPU's own factors, against fp64
    dmax = np.max(np.abs(D)) + 1e-30
    want = res.astype(np.float64) - D.reshape(-1)
    assert np.max(np.abs(err - want)) <= 1e-5 * dmax + 2 ** -23 * np.max(np.abs(res)), \
        f"{tag}: err' != r - U R_U V^T"

    base = rcv.base[sl].cpu().numpy()
    want_b = base0[sl].astype(np.float64) + D.reshape(-1)
    assert np.max(np.abs(base - want_b)) <= 1e-5 * dmax + 2 ** -23 * np.max(np.abs(want_b)), \
        f"{tag}: base' != base + U R_U V^T"
    # the oracle's receiver on the GPU's factors lands on the same values
    orc = oracle.LowrankReceiver(m, n)
    orc.base[:] = base0[sl]
    orc.decompress(U, V, RU)
    assert np.max(np.abs(base - orc.base)) <= 1e-5 * dmax + 2 ** -23 * np.max(np.abs(want_b))
    if xhat is not None:
        assert np.array_equal(u16(xhat[sl]), rne_bf16(base)), f"{tag}: xhat"


def _run(batch, m, n, r, T, steps, check, seed=0, warm_start=False, rank=16):
    say(f"[gpu] lowrank-ef batch={batch} m={m} n={n} r={r} T={T} steps={steps} "
        f"warm_start={warm_start} checked={list(check)}")
    st = LowrankDrift(batch, m, n, rank=rank, seed=seed, device=DEV)
    x0 = st.next()
    snd = cfz.LowrankSender(batch, m, n, r, x0=x0)
    rcv = cfz.LowrankReceiver(batch, m, n, r, x0=x0)
    xhat = torch.empty(batch * m * n, dtype=torch.bfloat16, device=DEV)
    q0 = gaussian_q0(batch, n, r, seed=seed, device=DEV)
    for t in range(1, steps):
        x = st.next()
        torch.cuda.synchronize()
        prev0, err0, base0 = u16(snd.prev), snd.err.cpu().numpy(), rcv.base.cpu().numpy()
        if warm_start and t > 1:
            q0 = snd.V.clone()
        elif not warm_start:
            q0 = gaussian_q0(batch, n, r, seed=seed * 100 + t, device=DEV)
        q0_host = q0.cpu().numpy()
        snd.compress(x, q0, T)
        rcv.decompress(snd.U, snd.V, snd.RU, xhat)
        torch.cuda.synchronize()
        xh = u16(x)
        for b in check:
            _check_step(f"step {t} matrix {b}", b, m, n, r, T, xh, prev0, err0, base0,
                        q0_host[b], snd, rcv, xhat, lead=rank)
    return snd, rcv, st


@pytest.mark.parametrize("batch,m,n,r,T", [(1, 256, 384, 8, 2), (3, 200, 328, 5, 1),
                                           (2, 130, 264, 16, 2), (1, 64, 512, 32, 0),
                                           (2, 96, 136, 1, 3), (1, 1100, 264, 32, 1)])
def test_teacher_forced_steps(batch, m, n, r, T):
    """Several tiles and ragged edges of the update's blocks (256 columns of 64 rows, or
    128 rows at r > 16); every rank class, r not a multiple of 4 (scalar operand loads)."""
    _run(batch, m, n, r, T, 4, range(batch), seed=batch * 7 + r)


def test_warm_start_from_previous_v():
    _run(2, 192, 256, 8, 1, 5, range(2), seed=3, warm_start=True)


def test_zero_residual_sends_nothing():
    say("[gpu] lowrank-ef zero residual")
    m, n, r = 128, 256, 8
    x0 = LowrankDrift(1, m, n, seed=9, device=DEV).next()
    snd = cfz.LowrankSender(1, m, n, r, x0=x0)
    rcv = cfz.LowrankReceiver(1, m, n, r, x0=x0)
    b0 = rcv.base.clone()
    snd.compress(x0, gaussian_q0(1, n, r, seed=1, device=DEV), 2)
    rcv.decompress(snd.U, snd.V, snd.RU)
    torch.cuda.synchronize()
    for t in (snd.U, snd.V, snd.RU, snd.err):
        assert not t.any()
    assert torch.equal(rcv.base, b0)


def test_exact_low_rank_residual_arrives():
    """x - prev = F G^T with ternary factors (exact in bf16), rank 8 <= r: the receiver's base
    equals x to the subspace iteration's precision and the carried error is near zero."""
    say("[gpu] lowrank-ef exact rank")
    b, m, n, r = 2, 256, 384, 8
    x = exact_rank_batch(b, m, n, 8, seed=5).to(DEV)
    snd = cfz.LowrankSender(b, m, n, r)     # prev = 0, err = 0
    rcv = cfz.LowrankReceiver(b, m, n, r)   # base = 0
    snd.compress(x, gaussian_q0(b, n, r, seed=2, device=DEV), 2)
    rcv.decompress(snd.U, snd.V, snd.RU)
    torch.cuda.synchronize()
    xf = x.float().reshape(-1)
    scale = xf.abs().max().item()
    assert (rcv.base - xf).abs().max().item() <= 1e-4 * scale
    assert snd.err.abs().max().item() <= 1e-4 * scale


def test_sender_and_receiver_telescope_over_steps():
    """base_T + err_T = X_T: the receiver adds exactly the reconstruction the sender removed
    (same kernel, same factors), so only fp32 rounding per step separates the two sides."""
    b, m, n, r, steps = 2, 256, 512, 16, 10
    say("[gpu] lowrank-ef telescoping")
    st = LowrankDrift(b, m, n, seed=11, device=DEV)
    x = st.next()
    snd = cfz.LowrankSender(b, m, n, r, x0=x)
    rcv = cfz.LowrankReceiver(b, m, n, r, x0=x)
    for t in range(1, steps):
        x = st.next()
        snd.compress(x, gaussian_q0(b, n, r, seed=t, device=DEV), 2)
        rcv.decompress(snd.U, snd.V, snd.RU)
    torch.cuda.synchronize()
    xt = x.float().reshape(-1).double()
    gap = (rcv.base.double() + snd.err.double() - xt).abs().max().item()
    assert gap <= 16 * steps * 2 ** -24 * xt.abs().max().item()


def test_full_size_flux_share_sampled_layers():
    """57 layers of 1024 x 3072 in one call per step (r = 16, T = 2), the benchmark's launch
    configuration; layers 0, 28 and 56 compared with the oracle on two steps."""
    _run(57, 1024, 3072, 16, 2, 3, [0, 28, 56], seed=1)


def test_graph_replay_matches_eager_every_replay():
    """A sender and receiver step of the low-rank EF path captured once in a HIP graph and
    replayed step after step (inputs copied into static buffers, eager work and
    synchronisations between replays) gives, after every replay, the bits of the same steps
    run eagerly: every kernel of the path is graph-safe (no memset nodes, no host work)."""
    b, m, n, r, T, steps = 2, 192, 256, 8, 2, 5
    say("[gpu] lowrank-ef graph replay")
    st = LowrankDrift(b, m, n, seed=21, device=DEV)
    xs = [st.next() for _ in range(steps + 1)]
    q0s = [gaussian_q0(b, n, r, seed=40 + t, device=DEV) for t in range(steps + 1)]
    xhat_e = torch.empty(b * m * n, dtype=torch.bfloat16, device=DEV)
    es, er = cfz.LowrankSender(b, m, n, r, x0=xs[0]), cfz.LowrankReceiver(b, m, n, r, x0=xs[0])
    gs, gr = cfz.LowrankSender(b, m, n, r, x0=xs[0]), cfz.LowrankReceiver(b, m, n, r, x0=xs[0])
    xin, qin = torch.empty_like(xs[0]), torch.empty_like(q0s[0])
    xhat_g = torch.empty_like(xhat_e)
    torch.cuda.synchronize()
    # capture records the launches without running them; the states stay at the warm-up
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        gs.compress(xin, qin, T)
        gr.decompress(gs.U, gs.V, gs.RU, xhat_g)
    torch.cuda.synchronize()
    for t in range(1, steps + 1):
        es.compress(xs[t], q0s[t], T)
        er.decompress(es.U, es.V, es.RU, xhat_e)
        xin.copy_(xs[t])
        qin.copy_(q0s[t])
        g.replay()
        torch.cuda.synchronize()
        for name, a_, b_ in (("U", gs.U, es.U), ("V", gs.V, es.V), ("RU", gs.RU, es.RU),
                             ("err", gs.err, es.err), ("prev", gs.prev, es.prev),
                             ("base", gr.base, er.base), ("xhat", xhat_g, xhat_e)):
            assert torch.equal(a_.view(torch.int16) if a_.dtype == torch.bfloat16 else a_,
                               b_.view(torch.int16) if b_.dtype == torch.bfloat16 else b_), \
                f"replay {t}: {name} differs from the eager step"
    say(f"  {steps} replays bit-identical to eager steps")


@pytest.mark.parametrize("batch,m,n,r,T,warm", [(2, 130, 264, 16, 2, False),
                                                (1, 1100, 264, 32, 1, True),
                                                (3, 96, 136, 5, 2, True),
                                                (2, 100, 136, 12, 0, False),
                                                (57, 1024, 3072, 16, 2, True)])
def test_deferred_sender_matches_plain_bit_for_bit(batch, m, n, r, T, warm):
    """The deferred sender (each step's update applied inside the next step's residual pass)
    against the plain sender on the same inputs: the factors, prev and the bf16 residual after
    every step, and err after each flush, equal bit for bit.  One flush in the middle of the
    run, so that steps after it start with nothing pending."""
    steps = 6
    say(f"[gpu] lowrank-ef deferred batch={batch} m={m} n={n} r={r} T={T} warm={warm}")
    st = LowrankDrift(batch, m, n, seed=31 + r, device=DEV)
    x = st.next()
    plain = cfz.LowrankSender(batch, m, n, r, x0=x)
    dfr = cfz.LowrankSender(batch, m, n, r, x0=x, deferred=True)
    for t in range(1, steps):
        x = st.next()
        q0 = gaussian_q0(batch, n, r, seed=60 + t, device=DEV)
        plain.compress(x, plain.V if warm and t > 1 else q0, T)
        dfr.compress(x, dfr.V if warm and t > 1 else q0, T)
        if t == 3:
            dfr.flush()
            assert not dfr.pending
        torch.cuda.synchronize()
        for name, a_, b_ in (("U", dfr.U, plain.U), ("V", dfr.V, plain.V),
                             ("RU", dfr.RU, plain.RU),
                             ("prev", dfr.prev.view(torch.int16), plain.prev.view(torch.int16)),
                             ("A", dfr.residual_bf16().view(torch.int16),
                              plain.residual_bf16().view(torch.int16))):
            assert torch.equal(a_, b_), f"step {t}: {name} differs from the plain sender"
        if t == 3:
            assert torch.equal(dfr.err, plain.err), f"step {t}: err after the flush"
    dfr.flush()
    torch.cuda.synchronize()
    assert torch.equal(dfr.err, plain.err), "err after the final flush"


def test_deferred_sender_graph_replay_matches_eager():
    """The deferred sender's steady-state call (the pending update fused into the residual
    pass, then the subspace iteration) captured once in a HIP graph and replayed step after
    step gives the bits of the same deferred steps run eagerly, and after a final flush the
    carried error of the plain sender."""
    b, m, n, r, T, steps = 2, 192, 256, 16, 2, 5
    say("[gpu] lowrank-ef deferred graph replay")
    st = LowrankDrift(b, m, n, seed=23, device=DEV)
    xs = [st.next() for _ in range(steps + 2)]
    q0s = [gaussian_q0(b, n, r, seed=70 + t, device=DEV) for t in range(steps + 2)]
    es = cfz.LowrankSender(b, m, n, r, x0=xs[0], deferred=True)
    gs = cfz.LowrankSender(b, m, n, r, x0=xs[0], deferred=True)
    ps = cfz.LowrankSender(b, m, n, r, x0=xs[0])
    # the first step leaves an update pending on every deferred sender
    for s_ in (es, gs, ps):
        s_.compress(xs[1], q0s[1], T)
    xin, qin = torch.empty_like(xs[0]), torch.empty_like(q0s[0])
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        cfz.cfz_lowrank_ef_compress_deferred(b, m, n, r, T, 1, xin, gs.prev, gs.err, qin, gs.U,
                                             gs.V, gs.RU, gs.ws)
    torch.cuda.synchronize()
    for t in range(2, steps + 2):
        es.compress(xs[t], q0s[t], T)
        ps.compress(xs[t], q0s[t], T)
        xin.copy_(xs[t])
        qin.copy_(q0s[t])
        g.replay()
        torch.cuda.synchronize()
        for name, a_, b_ in (("U", gs.U, es.U), ("V", gs.V, es.V), ("RU", gs.RU, es.RU),
                             ("err", gs.err, es.err),
                             ("prev", gs.prev.view(torch.int16), es.prev.view(torch.int16))):
            assert torch.equal(a_, b_), f"replay {t}: {name} differs from the eager deferred step"
    cfz.cfz_lowrank_ef_flush(b, m, n, r, gs.U, gs.V, gs.RU, gs.err)
    torch.cuda.synchronize()
    assert torch.equal(gs.err, ps.err), "flushed err differs from the plain sender's"
    say(f"  {steps} deferred replays bit-identical to eager steps")
