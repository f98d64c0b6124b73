"""GPU parity of the HIP codec (through the C ABI) against the CPU oracle.

Bar: packed codes and fp32 scales bit-exact; error buffer, previous activation,
bases and bf16 reconstructions bit-exact as well (both sides use IEEE fp32
division, ties-to-even rounding and the same two explicit fma operations; with
bf16 state each fma result is rounded once to bf16, ties to even).
Inputs: seeded AR(1) activations at the workload shapes (synth module)."""
import ctypes as C
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import SPECS, AR1Stream

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from diffusion_activation_residual_amd import cfz
DEV = "cuda:0"

MODE_PAIRS = {0: oracle.DELTA, 1: oracle.LITERAL, 2: oracle.OFF}


def say(*a):
    print(*a, file=sys.stderr, flush=True)


def raw_bytes(t):
    """The bytes of a device tensor (any element type, bf16 included) as a numpy uint8 array."""
    return t.contiguous().view(torch.uint8).cpu().numpy()


def u16(t):
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(-1)


def u32(t):
    return t.contiguous().cpu().numpy().view(np.uint32).reshape(-1)


def sbits(t):
    """Bit patterns of a state tensor, fp32 or bf16."""
    return u16(t) if t.element_size() == 2 else u32(t)


def obits(a):
    """Bit patterns of an oracle state array (uint16 for bf16 state, else fp32)."""
    return a if a.dtype == np.uint16 else a.view(np.uint32)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _compare_step(tag, gs, gr, codes, scales, os_, or_, ocodes, oscales, xhat=None, oxhat=None):
    assert np.array_equal(codes.cpu().numpy(), ocodes), f"{tag}: codes"
    assert np.array_equal(u32(scales), oscales.view(np.uint32)), f"{tag}: scales"
    if os_.err is not None:
        assert np.array_equal(sbits(gs.err), obits(os_.err)), f"{tag}: err"
    if os_.prev is not None:
        assert np.array_equal(u16(gs.prev), os_.prev), f"{tag}: prev"
    if os_.base is not None:
        assert np.array_equal(sbits(gs.base), obits(os_.base)), f"{tag}: sender base"
    assert np.array_equal(sbits(gr.base), obits(or_.base)), f"{tag}: receiver base"
    if xhat is not None:
        assert np.array_equal(u16(xhat), oxhat), f"{tag}: xhat"


def _run_parity(xs, rows, cols, bits, group, mode, tag, want_xhat=True, state_bf16=False):
    """xs: list of bf16 CPU tensors [rows, cols]; step 0 is the warm-up."""
    n = rows * cols
    say(f"[gpu] {tag}: rows={rows} cols={cols} bits={bits} group={group} mode={mode} "
        f"bf16 state={state_bf16}")
    sb = state_bf16
    gs = cfz.Sender(rows, cols, bits, group, mode, x0=xs[0].to(DEV), state_bf16=sb)
    gr = cfz.Receiver(rows, cols, bits, group, x0=xs[0].to(DEV), state_bf16=sb)
    os_ = oracle.Sender(n, bits, group, MODE_PAIRS[mode], x0=u16(xs[0]), state_bf16=sb)
    or_ = oracle.Receiver(n, bits, group, x0=u16(xs[0]), state_bf16=sb)
    xhat = torch.empty(n, dtype=torch.bfloat16, device=DEV) if want_xhat else None
    for t in range(1, len(xs)):
        codes, scales = gs.compress(xs[t].to(DEV))
        gr.decompress(codes, scales, xhat)
        ocodes, oscales = os_.compress(u16(xs[t]))
        oxhat = or_.decompress(ocodes, oscales, want_xhat=want_xhat)
        torch.cuda.synchronize()
        _compare_step(f"{tag} step {t}", gs, gr, codes, scales, os_, or_, ocodes, oscales,
                      xhat, oxhat)
    assert cfz.cfz_state_steps(gs.handle) == len(xs) - 1
    gs.close()
    gr.close()


def _ar1(rows, cols, steps, spec="flux", seed=0, n_tensors=1):
    sp = SPECS[spec]
    st = AR1Stream(n_tensors, rows, cols, sp.alpha, sp.noise, sp.outlier_frac, seed=seed,
                   key=f"{spec}-test")
    return [st.next() for _ in range(steps)]


def test_tiny_config_every_step():
    sp = SPECS["tiny"]
    st = AR1Stream.from_spec(sp, seed=0)
    xs = [st.next()[0] for _ in range(sp.steps)]
    _run_parity(xs, sp.rows, sp.cols, 4, 64, cfz.CFZ_EF_DELTA, "tiny int4 g64")


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("group", [8, 16, 32, 64, 128])
@pytest.mark.parametrize("bits", [4, 2])
def test_every_variant_several_tiles_and_ragged_tail(bits, group, mode):
    # 300 x 256 = 9600 chunks of 8: 18.75 blocks of 512 chunks, so a ragged last block
    xs = [x[0] for x in _ar1(300, 256, 4, seed=bits * 100 + group + mode)]
    _run_parity(xs, 300, 256, bits, group, mode, f"variant b{bits} g{group} m{mode}")


@pytest.mark.parametrize("rows,cols,group", [(1, 8, 8), (1, 64, 64), (3, 128, 128), (5, 24, 8),
                                             (513, 64, 32), (2, 4096, 64)])
def test_odd_shapes(rows, cols, group):
    xs = [x[0] for x in _ar1(rows, cols, 3, seed=rows + cols)]
    for bits in (4, 2):
        _run_parity(xs, rows, cols, bits, group, cfz.CFZ_EF_DELTA, f"shape {rows}x{cols}")


def test_empty_tensor_is_a_noop():
    say("[gpu] empty tensor")
    s = cfz.Sender(0, 64, 4, 64)
    r = cfz.Receiver(0, 64, 4, 64)
    x = torch.empty(0, dtype=torch.bfloat16, device=DEV)
    codes, scales = s.compress(x)
    r.decompress(codes, scales)
    torch.cuda.synchronize()
    assert codes.numel() == 0 and scales.numel() == 0


def _extreme_inputs(rows=64, cols=512):
    rng = np.random.default_rng(5)
    mags = np.array([1e-38, 1e-30, 3e-39, 1.0, 1e20, 1e30, 0.0, 1e-3], np.float32)
    sc = np.repeat(mags, cols // len(mags))
    xs = []
    for t in range(4):
        v = (rng.standard_normal((rows, cols)) * sc).astype(np.float32)
        if t == 2:
            v[:8] = np.round(rng.uniform(-7, 7, (8, cols)) * 2) / 2  # half-integer lattice
        xs.append(torch.from_numpy(v).to(torch.bfloat16))
    xs[3][10:20] = xs[2][10:20]  # unchanged rows: zero residual in DELTA
    return xs


@pytest.mark.parametrize("state_bf16", [False, True])
def test_extreme_magnitudes(state_bf16):
    """Subnormal, tiny and huge groups, all-zero groups and exact ties."""
    xs = _extreme_inputs()
    for bits, group in ((4, 64), (2, 32), (4, 8)):
        for mode in (0, 1, 2):
            _run_parity(xs, 64, 512, bits, group, mode, f"extreme b{bits} g{group} m{mode}",
                        state_bf16=state_bf16)


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("bits,group,sb", [(4, 64, False), (2, 32, True)])
def test_non_finite_values_stay_in_their_group(bits, group, mode, sb):
    """NaN and +-Inf activations lie outside the method's domain; what the library promises
    is that they touch only the groups that hold them.  A NaN, a +Inf and a -Inf go into three
    groups of step 1 (the oracle gets the clean values there); over that step and two clean
    steps after it, every other group's codes, scales, error, previous activation, bases and
    reconstruction equal the oracle's bits -- the residual, the scale, the codes and the state
    updates never mix groups."""
    rows, cols = 64, 512
    n = rows * cols
    xs = [x[0] for x in _ar1(rows, cols, 4, seed=41 + mode)]
    spots = [(3, 7, float("nan")), (20, 300, float("inf")), (63, 511, float("-inf"))]
    bad = np.zeros(n // group, bool)
    dirty = xs[1].clone()
    for r, c, v in spots:
        dirty[r, c] = v
        bad[(r * cols + c) // group] = True
    ok_elem = np.repeat(~bad, group)
    ok_byte = np.repeat(~bad, group * bits // 8)
    say(f"[gpu] non-finite inputs b{bits} g{group} m{mode} bf16 state={sb}")
    gs = cfz.Sender(rows, cols, bits, group, mode, x0=xs[0].to(DEV), state_bf16=sb)
    gr = cfz.Receiver(rows, cols, bits, group, x0=xs[0].to(DEV), state_bf16=sb)
    os_ = oracle.Sender(n, bits, group, MODE_PAIRS[mode], x0=u16(xs[0]), state_bf16=sb)
    or_ = oracle.Receiver(n, bits, group, x0=u16(xs[0]), state_bf16=sb)
    xhat = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    for t in (1, 2, 3):
        codes, scales = gs.compress((dirty if t == 1 else xs[t]).to(DEV))
        gr.decompress(codes, scales, xhat)
        oc, osc = os_.compress(u16(xs[t]))
        ox = or_.decompress(oc, osc, want_xhat=True)
        torch.cuda.synchronize()
        tag = f"step {t}"
        sc = scales.cpu().numpy()
        if t == 1:  # the injected values reached the kernel: |+-Inf| makes its group's scale Inf
            for r, c, v in spots[1:]:
                assert np.isinf(sc[(r * cols + c) // group]), tag
        assert np.array_equal(codes.cpu().numpy()[ok_byte], oc[ok_byte]), f"{tag}: codes"
        assert np.array_equal(sc.view(np.uint32)[~bad], osc.view(np.uint32)[~bad]), \
            f"{tag}: scales"
        if os_.err is not None:
            assert np.array_equal(sbits(gs.err)[ok_elem], obits(os_.err)[ok_elem]), f"{tag}: err"
        if os_.prev is not None:
            assert np.array_equal(u16(gs.prev)[ok_elem], os_.prev[ok_elem]), f"{tag}: prev"
        if os_.base is not None:
            assert np.array_equal(sbits(gs.base)[ok_elem], obits(os_.base)[ok_elem]), \
                f"{tag}: sender base"
        assert np.array_equal(sbits(gr.base)[ok_elem], obits(or_.base)[ok_elem]), \
            f"{tag}: receiver base"
        assert np.array_equal(u16(xhat)[ok_elem], ox[ok_elem]), f"{tag}: xhat"
    gs.close()
    gr.close()


@pytest.mark.parametrize("mode", [0, 1, 2])
@pytest.mark.parametrize("group", [8, 32, 128])
@pytest.mark.parametrize("bits", [4, 2])
def test_bf16_state_several_tiles_and_ragged_tail(bits, group, mode):
    """Carried error and base kept in bf16: every state update rounded once to bf16."""
    xs = [x[0] for x in _ar1(300, 256, 5, seed=7 * bits + group + mode)]
    _run_parity(xs, 300, 256, bits, group, mode, f"bf16 state b{bits} g{group} m{mode}",
                state_bf16=True)


def test_bf16_state_odd_shapes_and_empty():
    for rows, cols, group in ((1, 8, 8), (5, 24, 8), (513, 64, 32)):
        xs = [x[0] for x in _ar1(rows, cols, 3, seed=rows * cols)]
        _run_parity(xs, rows, cols, 4, group, cfz.CFZ_EF_DELTA, f"bf16 state {rows}x{cols}",
                    state_bf16=True)
    s = cfz.Sender(0, 64, 4, 64, state_bf16=True)
    r = cfz.Receiver(0, 64, 4, 64, state_bf16=True)
    codes, scales = s.compress(torch.empty(0, dtype=torch.bfloat16, device=DEV))
    r.decompress(codes, scales)
    torch.cuda.synchronize()


@pytest.mark.parametrize("state_bf16", [False, True])
def test_zero_residual_leaves_state_bitwise(state_bf16):
    say(f"[gpu] zero residual, bf16 state={state_bf16}")
    x0 = _ar1(64, 256, 1)[0][0].to(DEV)
    s = cfz.Sender(64, 256, 4, 64, cfz.CFZ_EF_DELTA, x0=x0, state_bf16=state_bf16)
    r = cfz.Receiver(64, 256, 4, 64, x0=x0, state_bf16=state_bf16)
    base0 = r.base.clone()
    codes, scales = s.compress(x0)
    r.decompress(codes, scales)
    torch.cuda.synchronize()
    assert not codes.any() and not scales.any()
    assert not s.err.view(torch.int16 if state_bf16 else torch.int32).any()
    assert torch.equal(sbits_t(r.base), sbits_t(base0))
    if state_bf16:  # the warm-up base of a bf16 receiver is x0 itself
        assert torch.equal(r.base.view(torch.int16), x0.reshape(-1).view(torch.int16))


def sbits_t(t):
    return t.view(torch.int16 if t.element_size() == 2 else torch.int32)


def test_checkpoint_resume_and_determinism():
    rows, cols, steps, k = 128, 512, 8, 3
    xs = [x[0].to(DEV) for x in _ar1(rows, cols, steps, seed=9)]
    say("[gpu] checkpoint/resume")

    def run_all():
        s = cfz.Sender(rows, cols, 4, 64, cfz.CFZ_EF_DELTA, x0=xs[0])
        outs = []
        for t in range(1, steps):
            c, sc = s.compress(xs[t])
            outs.append((c.clone(), sc.clone()))
        torch.cuda.synchronize()
        return s, outs

    s1, outs1 = run_all()
    s2, outs2 = run_all()
    for (a, b), (c, d) in zip(outs1, outs2):
        assert torch.equal(a, c) and torch.equal(b.view(torch.int32), d.view(torch.int32))
    # resume from a copy of the state after k steps
    s3 = cfz.Sender(rows, cols, 4, 64, cfz.CFZ_EF_DELTA, x0=xs[0])
    for t in range(1, k + 1):
        s3.compress(xs[t])
    prev, err = s3.prev.clone(), s3.err.clone()
    h = cfz.cfz_state_resume(s3.desc, prev=prev, err=err, steps=k)
    codes = torch.empty_like(s3.codes)
    scales = torch.empty_like(s3.scales)
    for t in range(k + 1, steps):
        cfz.cfz_compress(h, xs[t], codes, scales)
        torch.cuda.synchronize()
        assert torch.equal(codes, outs1[t - 1][0])
        assert torch.equal(scales.view(torch.int32), outs1[t - 1][1].view(torch.int32))
    assert cfz.cfz_state_steps(h) == steps - 1
    assert torch.equal(err.view(torch.int32), s1.err.view(torch.int32))
    cfz.cfz_state_destroy(h)


def test_error_paths_have_no_side_effects():
    say("[gpu] error paths")
    x0 = _ar1(32, 256, 1)[0][0].to(DEV)
    s = cfz.Sender(32, 256, 4, 64, cfz.CFZ_EF_DELTA, x0=x0)
    codes = torch.full((32 * 256 // 2 + 16,), 0x5a, dtype=torch.uint8, device=DEV)
    scales = torch.full((32 * 256 // 64,), 3.0, device=DEV)
    err0 = s.err.clone()
    with pytest.raises(cfz.CfzError) as ei:
        cfz.cfz_compress(s.handle, x0, codes[1:].data_ptr(), scales)
    assert ei.value.status == cfz.CFZ_ERR_ALIGN
    torch.cuda.synchronize()
    assert bool((codes == 0x5a).all()) and bool((scales == 3.0).all())
    assert torch.equal(s.err, err0)
    assert cfz.cfz_state_steps(s.handle) == 0


@pytest.mark.parametrize("nr,nw", [(1000, 1000), (1000, 820), (4096 * 3 + 5, 3001), (64, 1),
                                   (7, 0)])
def test_stream_mix_writes_the_spread_vectors(nr, nw):
    """Vector i of src lands at floor(i nw / nr) of dst when that index steps: every dst
    vector is written once, by the last src vector that maps to it."""
    src = torch.randint(0, 2**31 - 1, (nr * 4,), dtype=torch.int32, device=DEV)
    dst = torch.full((max(nw, 1) * 4 + 4,), -1, dtype=torch.int32, device=DEV)
    cfz.cfz_stream_mix(src, nr * 16, dst, nw * 16)
    torch.cuda.synchronize()
    i = np.arange(nr, dtype=np.int64)
    j = i * nw // nr
    last = j != (i + 1) * nw // nr
    expect = np.full(((max(nw, 1) + 1) * 4,), -1, dtype=np.int32)
    s = src.cpu().numpy().reshape(nr, 4)
    expect.reshape(-1, 4)[j[last]] = s[i[last]]
    assert np.array_equal(dst.cpu().numpy(), expect)


def test_stream_copy_matches():
    say("[gpu] stream copy")
    a = torch.randint(0, 255, (1 << 20,), dtype=torch.uint8, device=DEV)
    b = torch.zeros_like(a)
    cfz.cfz_stream_copy(a, b)
    torch.cuda.synchronize()
    assert torch.equal(a, b)


def test_runs_on_a_side_stream():
    rows, cols = 256, 512
    xs = [x[0].to(DEV) for x in _ar1(rows, cols, 3, seed=4)]
    say("[gpu] side stream")
    st = torch.cuda.Stream()
    with torch.cuda.stream(st):
        s = cfz.Sender(rows, cols, 4, 64, x0=xs[0])
        for t in (1, 2):
            c, sc = s.compress(xs[t])
    st.synchronize()
    os_ = oracle.Sender(rows * cols, 4, 64, oracle.DELTA, x0=u16(xs[0]))
    for t in (1, 2):
        oc, osc = os_.compress(u16(xs[t]))
    assert np.array_equal(c.cpu().numpy(), oc)


# ------------------------------------------------------------------ full workload sizes

@pytest.mark.parametrize("state_bf16", [False, True])
def test_flux_int4_full_size_sampled_tensors(state_bf16):
    """FLUX.1-dev share, 57 layers x {K, V} of 1024 x 3072, int4 g64, DELTA, 28 steps, in the
    launch configuration of the benchmark (one grouped launch per layer for its K and V);
    layers 0, 28 and 56 are compared every step."""
    sp = SPECS["flux"]
    st = AR1Stream.from_spec(sp, seed=0, device=DEV)
    picks = [0, 1, 56, 57, 112, 113]
    say(f"[gpu] flux int4 full size, tensors {picks}, bf16 state={state_bf16}")
    x = st.next()
    n = sp.rows * sp.cols
    sb = state_bf16
    gs = [cfz.Sender(sp.rows, sp.cols, 4, 64, x0=x[i].contiguous(), state_bf16=sb) for i in picks]
    gr = [cfz.Receiver(sp.rows, sp.cols, 4, 64, x0=x[i].contiguous(), state_bf16=sb)
          for i in picks]
    os_ = [oracle.Sender(n, 4, 64, oracle.DELTA, x0=u16(x[i]), state_bf16=sb) for i in picks]
    or_ = [oracle.Receiver(n, 4, 64, x0=u16(x[i]), state_bf16=sb) for i in picks]
    for t in range(1, sp.steps):
        x = st.next()
        for j in range(0, len(picks), 2):  # K and V of one layer per grouped call
            pair = (j, j + 1)
            cfz.cfz_compress_group([gs[k].handle for k in pair],
                                   [x[picks[k]].contiguous() for k in pair],
                                   [gs[k].codes for k in pair], [gs[k].scales for k in pair])
            cfz.cfz_decompress_group([gr[k].handle for k in pair], [gs[k].codes for k in pair],
                                     [gs[k].scales for k in pair])
        torch.cuda.synchronize()
        for j, i in enumerate(picks):
            oc, osc = os_[j].compress(u16(x[i]))
            or_[j].decompress(oc, osc)
            _compare_step(f"flux t{t} tensor {i}", gs[j], gr[j], gs[j].codes, gs[j].scales,
                          os_[j], or_[j], oc, osc)


def test_flux_int4_layer_streams_graph_every_step():
    """The benchmark's overlapped schedule: all 57 layers' K and V of the FLUX.1-dev share
    (114 tensors of 1024 x 3072), int4 g64, DELTA, each layer's grouped compress and decode on
    one of 3 streams round-robin, captured into one HIP graph per step and replayed for all 27
    compressed steps.  Layers 0, 28 and 56 (with the bf16 output) are compared with the oracle
    every step; every tensor's codes and states are compared at the end with a run of the same
    launches eagerly on one stream."""
    from diffusion_activation_residual_amd import cadence
    sp = SPECS["flux"]
    T, n = sp.tensors, sp.rows * sp.cols
    layers = [[2 * l, 2 * l + 1] for l in range(T // 2)]
    picks = [0, 1, 56, 57, 112, 113]
    say(f"[gpu] flux int4, 3-stream graph schedule, {sp.steps - 1} steps, tensors {picks}")
    st = AR1Stream.from_spec(sp, seed=9, device=DEV)
    x0 = st.next().reshape(T, n)
    xs = torch.empty((T, n), dtype=torch.bfloat16, device=DEV)  # the graph's input buffer
    xhat = torch.empty((T, n), dtype=torch.bfloat16, device=DEV)
    gs = [cfz.Sender(sp.rows, sp.cols, 4, 64, x0=x0[i]) for i in range(T)]
    gr = [cfz.Receiver(sp.rows, sp.cols, 4, 64, x0=x0[i]) for i in range(T)]
    es = [cfz.Sender(sp.rows, sp.cols, 4, 64, x0=x0[i]) for i in range(T)]  # one-stream run
    er = [cfz.Receiver(sp.rows, sp.cols, 4, 64, x0=x0[i]) for i in range(T)]
    eh = torch.empty((T, n), dtype=torch.bfloat16, device=DEV)
    os_ = [oracle.Sender(n, 4, 64, oracle.DELTA, x0=u16(x0[i])) for i in picks]
    or_ = [oracle.Receiver(n, 4, 64, x0=u16(x0[i])) for i in picks]
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    streams = [cap, torch.cuda.Stream(), torch.cuda.Stream()]
    cap.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=cap):  # records the launches; runs nothing
        cadence.enqueue_layer_step(layers, [g.handle for g in gs], [g.handle for g in gr], xs,
                                   [g.codes for g in gs], [g.scales for g in gs], streams,
                                   xhat=xhat)
    torch.cuda.synchronize()
    one = [torch.cuda.current_stream()]
    for t in range(1, sp.steps):
        x = st.next().reshape(T, n)
        xs.copy_(x)
        graph.replay()
        cadence.enqueue_layer_step(layers, [g.handle for g in es], [g.handle for g in er], x,
                                   [g.codes for g in es], [g.scales for g in es], one, xhat=eh)
        torch.cuda.synchronize()
        for j, i in enumerate(picks):
            oc, osc = os_[j].compress(u16(x[i]))
            oh = or_[j].decompress(oc, osc, want_xhat=True)
            _compare_step(f"3-stream graph t{t} tensor {i}", gs[i], gr[i], gs[i].codes,
                          gs[i].scales, os_[j], or_[j], oc, osc, xhat[i], oh)
    for i in range(T):
        assert torch.equal(gs[i].codes, es[i].codes), f"tensor {i} codes"
        assert torch.equal(gs[i].scales.view(torch.int32), es[i].scales.view(torch.int32))
        assert torch.equal(gs[i].err.view(torch.int32), es[i].err.view(torch.int32))
        assert torch.equal(gs[i].prev.view(torch.int16), es[i].prev.view(torch.int16))
        assert torch.equal(gr[i].base.view(torch.int32), er[i].base.view(torch.int32))
    assert torch.equal(xhat.view(torch.int16), eh.view(torch.int16))
    del graph
    for h in gs + gr + es + er:
        h.close()


def _batched_rows_parity(spec_name, bits, group, steps, row_slices, tag):
    sp = SPECS[spec_name]
    rows = sp.tensors * sp.rows
    st = AR1Stream.from_spec(sp, seed=1, device=DEV)
    say(f"[gpu] {tag}: one launch over {rows} x {sp.cols}, {steps} steps")
    x = st.next().reshape(rows, sp.cols)
    gs = cfz.Sender(rows, sp.cols, bits, group, x0=x)
    gr = cfz.Receiver(rows, sp.cols, bits, group, x0=x)
    os_, or_ = [], []
    for a, b in row_slices:
        xs = u16(x[a:b])
        os_.append(oracle.Sender(xs.size, bits, group, oracle.DELTA, x0=xs))
        or_.append(oracle.Receiver(xs.size, bits, group, x0=xs))
    cpr = sp.cols * bits // 8   # code bytes per row
    spr = sp.cols // group      # scales per row
    for t in range(1, steps):
        x = st.next().reshape(rows, sp.cols)
        codes, scales = gs.compress(x)
        gr.decompress(codes, scales)
        torch.cuda.synchronize()
        for j, (a, b) in enumerate(row_slices):
            oc, osc = os_[j].compress(u16(x[a:b]))
            or_[j].decompress(oc, osc)
            assert np.array_equal(codes[a * cpr:b * cpr].cpu().numpy(), oc), f"{tag} t{t} codes"
            assert np.array_equal(u32(scales[a * spr:b * spr]), osc.view(np.uint32))
            n0, n1 = a * sp.cols, b * sp.cols
            assert np.array_equal(u32(gs.err[n0:n1]), os_[j].err.view(np.uint32))
            assert np.array_equal(u16(gs.prev[n0:n1]), os_[j].prev)
            assert np.array_equal(u32(gr.base[n0:n1]), or_[j].base.view(np.uint32))


def test_flux_int2_batched_full_size_sampled_rows():
    """All 57 layers' K/V (116736 x 3072 bf16, about 717 MB) in one launch per step,
    2-bit group 32; first, middle and last rows compared every step."""
    rows = SPECS["flux"].tensors * SPECS["flux"].rows
    sl = [(0, 64), (rows // 2 - 32, rows // 2 + 32), (rows - 64, rows)]
    _batched_rows_parity("flux", 2, 32, SPECS["flux"].steps, sl, "flux int2 batched")


def test_flux_int2_batched_whole_batch_first_steps():
    """All 57 layers' K/V as one 116736 x 3072 tensor, int2 g32, one launch per step: every
    code, scale and state value of the whole batch compared with the oracle (its OpenMP
    build, identical bits to the serial one) for compressed steps 1 to 3."""
    sp = SPECS["flux"]
    rows = sp.tensors * sp.rows
    n = rows * sp.cols
    st = AR1Stream.from_spec(sp, seed=5, device=DEV)
    say(f"[gpu] flux int2 whole batch: {rows} x {sp.cols}, steps 1-3")
    x = st.next().reshape(rows, sp.cols)
    gs = cfz.Sender(rows, sp.cols, 2, 32, x0=x)
    gr = cfz.Receiver(rows, sp.cols, 2, 32, x0=x)
    with oracle.parallel():
        os_ = oracle.Sender(n, 2, 32, oracle.DELTA, x0=u16(x))
        or_ = oracle.Receiver(n, 2, 32, x0=u16(x))
    for t in range(1, 4):
        x = st.next().reshape(rows, sp.cols)
        codes, scales = gs.compress(x)
        gr.decompress(codes, scales)
        torch.cuda.synchronize()
        with oracle.parallel():
            oc, osc = os_.compress(u16(x))
            or_.decompress(oc, osc)
        _compare_step(f"flux int2 whole batch t{t}", gs, gr, codes, scales, os_, or_, oc, osc)
    gs.close()
    gr.close()


@pytest.mark.parametrize("mode", [1, 2])
def test_flux_literal_and_off_full_layer_every_step(mode):
    """The LITERAL and OFF readings at full size: one FLUX.1-dev layer (its K and V, 1024 x
    3072 each) in the benchmark's grouped per-layer launches, int4 g64, all 27 compressed
    steps, every value compared with the oracle."""
    sp = SPECS["flux"]
    st = AR1Stream(2, sp.rows, sp.cols, sp.alpha, sp.noise, sp.outlier_frac, seed=6 + mode,
                   key="flux-layer")
    n = sp.rows * sp.cols
    say(f"[gpu] flux one layer, mode {mode}, {sp.steps - 1} steps")
    x = st.next()
    gs = [cfz.Sender(sp.rows, sp.cols, 4, 64, mode, x0=x[i].to(DEV).contiguous()) for i in (0, 1)]
    gr = [cfz.Receiver(sp.rows, sp.cols, 4, 64, x0=x[i].to(DEV).contiguous()) for i in (0, 1)]
    os_ = [oracle.Sender(n, 4, 64, MODE_PAIRS[mode], x0=u16(x[i])) for i in (0, 1)]
    or_ = [oracle.Receiver(n, 4, 64, x0=u16(x[i])) for i in (0, 1)]
    for t in range(1, sp.steps):
        x = st.next()
        xd = [x[i].to(DEV).contiguous() for i in (0, 1)]
        cfz.cfz_compress_group([g.handle for g in gs], xd, [g.codes for g in gs],
                               [g.scales for g in gs])
        cfz.cfz_decompress_group([g.handle for g in gr], [g.codes for g in gs],
                                 [g.scales for g in gs])
        torch.cuda.synchronize()
        for i in (0, 1):
            oc, osc = os_[i].compress(u16(x[i]))
            or_[i].decompress(oc, osc)
            _compare_step(f"mode {mode} t{t} tensor {i}", gs[i], gr[i], gs[i].codes,
                          gs[i].scales, os_[i], or_[i], oc, osc)


@pytest.mark.parametrize("bits,group", [(4, 64), (2, 32)])
def test_cogvideox_full_size_sampled_rows(bits, group):
    """CogVideoX-2b share, 30 layers x {K, V} of 4388 x 1920 in one launch per step, 50 steps."""
    sp = SPECS["cogvideox"]
    rows = sp.tensors * sp.rows
    sl = [(0, 96), (29 * sp.rows, 29 * sp.rows + 96), (rows - 96, rows)]
    _batched_rows_parity("cogvideox", bits, group, sp.steps, sl, f"cogvideox b{bits}")


@pytest.mark.parametrize("bits,group,sb,steps", [(4, 64, False, 50), (2, 32, False, 50),
                                                  (4, 64, True, 12)])
def test_cogvideox_full_size_per_layer_launches(bits, group, sb, steps):
    """CogVideoX-2b share in the benchmark's launch configuration: 30 layers x {K, V} of
    4388 x 1920, one grouped compress and one grouped decode launch per layer, 49 compressed
    steps (11 with bf16 state); layers 0 and 29 (tensors 0, 1, 58, 59) compared with the
    oracle every step."""
    sp = SPECS["cogvideox"]
    st = AR1Stream.from_spec(sp, seed=2, device=DEV)
    picks = [0, 1, 58, 59]
    say(f"[gpu] cogvideox per-layer launches int{bits} g{group} bf16 state={sb}, tensors {picks}")
    x = st.next()
    n = sp.rows * sp.cols
    gs = [cfz.Sender(sp.rows, sp.cols, bits, group, x0=x[i].contiguous(), state_bf16=sb)
          for i in range(sp.tensors)]
    gr = [cfz.Receiver(sp.rows, sp.cols, bits, group, x0=x[i].contiguous(), state_bf16=sb)
          for i in range(sp.tensors)]
    os_ = {i: oracle.Sender(n, bits, group, oracle.DELTA, x0=u16(x[i]), state_bf16=sb)
           for i in picks}
    or_ = {i: oracle.Receiver(n, bits, group, x0=u16(x[i]), state_bf16=sb) for i in picks}
    for t in range(1, steps):
        x = st.next()
        for l in range(sp.tensors // 2):
            pair = (2 * l, 2 * l + 1)
            cfz.cfz_compress_group([gs[k].handle for k in pair], [x[k].contiguous() for k in pair],
                                   [gs[k].codes for k in pair], [gs[k].scales for k in pair])
            cfz.cfz_decompress_group([gr[k].handle for k in pair], [gs[k].codes for k in pair],
                                     [gs[k].scales for k in pair])
        torch.cuda.synchronize()
        for i in picks:
            oc, osc = os_[i].compress(u16(x[i]))
            or_[i].decompress(oc, osc)
            _compare_step(f"cogvideox t{t} tensor {i}", gs[i], gr[i], gs[i].codes, gs[i].scales,
                          os_[i], or_[i], oc, osc)
    for h in gs + gr:
        h.close()


def test_graph_replay_matches_oracle_every_replay():
    """The benchmark replays captured per-tensor launches; every replay must advance the state
    exactly like an eager step (checked against the oracle after each replay, with eager
    work and synchronisations between replays)."""
    rows, cols, steps = 256, 1024, 6
    xs = [x[0].to(DEV) for x in _ar1(rows, cols, steps + 1, seed=12)]
    say("[gpu] graph replay")
    xin = torch.empty_like(xs[0])
    gs = cfz.Sender(rows, cols, 4, 64, x0=xs[0])
    gr = cfz.Receiver(rows, cols, 4, 64, x0=xs[0])
    torch.cuda.synchronize()
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        gs.compress(xin)
        gr.decompress(gs.codes, gs.scales)
    torch.cuda.synchronize()
    n = rows * cols
    os_ = oracle.Sender(n, 4, 64, oracle.DELTA, x0=u16(xs[0]))
    or_ = oracle.Receiver(n, 4, 64, x0=u16(xs[0]))
    for t in range(1, steps + 1):
        xin.copy_(xs[t])                       # eager work between replays
        g.replay()
        torch.cuda.synchronize()
        oc, osc = os_.compress(u16(xs[t]))
        or_.decompress(oc, osc)
        _compare_step(f"graph replay {t}", gs, gr, gs.codes, gs.scales, os_, or_, oc, osc)


@pytest.mark.parametrize("bits,group,mode,sb", [(4, 64, 0, False), (2, 32, 0, False),
                                                (4, 128, 1, False), (2, 8, 2, False),
                                                (4, 64, 0, True), (2, 16, 2, True)])
def test_grouped_launch_matches_oracle(bits, group, mode, sb):
    """Separately allocated tensors of different sizes (one empty) in grouped calls: more than
    16 tensors, so the call spans several launches, and both launch shapes (big and small)."""
    shapes = [(1024, 1024)] * 17 + [(300, 256), (0, 256), (17, 128), (64, 1024)]
    say(f"[gpu] grouped b{bits} g{group} m{mode} bf16 state={sb}: {len(shapes)} tensors")
    seqs = [[x[0] for x in _ar1(r, c, 4, seed=100 + i)] if r else None
            for i, (r, c) in enumerate(shapes)]
    snd, rcv, osnd, orcv, xh = [], [], [], [], []
    for i, (r, c) in enumerate(shapes):
        x0 = seqs[i][0].to(DEV) if r else None
        snd.append(cfz.Sender(r, c, bits, group, mode, x0=x0, state_bf16=sb))
        rcv.append(cfz.Receiver(r, c, bits, group, x0=x0, state_bf16=sb))
        osnd.append(oracle.Sender(r * c, bits, group, MODE_PAIRS[mode],
                                  x0=u16(seqs[i][0]) if r else None, state_bf16=sb))
        orcv.append(oracle.Receiver(r * c, bits, group, x0=u16(seqs[i][0]) if r else None,
                                    state_bf16=sb))
        xh.append(torch.empty(r * c, dtype=torch.bfloat16, device=DEV))
    for t in range(1, 4):
        xs = [seqs[i][t].to(DEV) if r else torch.empty(0, dtype=torch.bfloat16, device=DEV)
              for i, (r, c) in enumerate(shapes)]
        cfz.cfz_compress_group([s.handle for s in snd], xs, [s.codes for s in snd],
                               [s.scales for s in snd])
        cfz.cfz_decompress_group([r_.handle for r_ in rcv], [s.codes for s in snd],
                                 [s.scales for s in snd], xh)
        torch.cuda.synchronize()
        for i, (r, c) in enumerate(shapes):
            if r == 0:
                continue
            oc, osc = osnd[i].compress(u16(seqs[i][t]))
            ox = orcv[i].decompress(oc, osc, want_xhat=True)
            _compare_step(f"group t{t} entry {i}", snd[i], rcv[i], snd[i].codes, snd[i].scales,
                          osnd[i], orcv[i], oc, osc, xh[i], ox)
    assert all(cfz.cfz_state_steps(s.handle) == 3 for s in snd)


def test_lost_payload_then_rewarm_in_place():
    """OFF mode on the GPU: a skipped decode makes the sender's and receiver's bases differ;
    re-warming both states in place (cfz_state_create on the same buffers with an
    uncompressed activation) gives the bits of a fresh run from there, step by step, and the
    oracle's."""
    rows, cols = 128, 512
    xs = [x[0] for x in _ar1(rows, cols, 9, seed=31)]
    say("[gpu] lost payload and re-warm")
    gs = cfz.Sender(rows, cols, 4, 64, cfz.CFZ_EF_OFF, x0=xs[0].to(DEV))
    gr = cfz.Receiver(rows, cols, 4, 64, x0=xs[0].to(DEV))
    for t in range(1, 5):
        codes, scales = gs.compress(xs[t].to(DEV))
        if t != 2:
            gr.decompress(codes, scales)
        torch.cuda.synchronize()
        assert torch.equal(sbits_t(gs.base), sbits_t(gr.base)) == (t < 2), f"step {t}"
    # in place: new handles on the same buffers, warmed from x_4
    x4 = xs[4].to(DEV)
    cfz.cfz_state_destroy(gs.handle)
    cfz.cfz_state_destroy(gr.handle)
    gs.handle = cfz.cfz_state_create(gs.desc, None, gs.base, None, x4)
    gr.handle = cfz.cfz_state_create(gr.desc, None, gr.base, None, x4)
    fs = cfz.Sender(rows, cols, 4, 64, cfz.CFZ_EF_OFF, x0=x4)
    fr = cfz.Receiver(rows, cols, 4, 64, x0=x4)
    n = rows * cols
    os_ = oracle.Sender(n, 4, 64, oracle.OFF, x0=u16(xs[4]))
    or_ = oracle.Receiver(n, 4, 64, x0=u16(xs[4]))
    for t in range(5, 9):
        c1, s1 = gs.compress(xs[t].to(DEV))
        gr.decompress(c1, s1)
        c2, s2 = fs.compress(xs[t].to(DEV))
        fr.decompress(c2, s2)
        oc, osc = os_.compress(u16(xs[t]))
        or_.decompress(oc, osc)
        torch.cuda.synchronize()
        assert torch.equal(c1, c2) and torch.equal(sbits_t(gr.base), sbits_t(fr.base))
        assert torch.equal(sbits_t(gs.base), sbits_t(gr.base))
        _compare_step(f"re-warmed step {t}", gs, gr, c1, s1, os_, or_, oc, osc)
    for h in (gs, gr, fs, fr):
        h.close()


@pytest.mark.parametrize("bits,group,sb", [(4, 64, False), (2, 32, True)])
def test_beyond_2_pow_31_elements_sampled_groups(bits, group, sb):
    """One tensor of 524,544 x 4096 = 2,148,532,224 elements (past 2^31: 64-bit indexing of
    elements, quads, codes and scales), one warm-up and one compressed step at the sender and
    the receiver; 24 groups spread over the tensor -- including those around element 2^31 and
    the last one -- compared bit for bit with the oracle run on those groups alone."""
    rows, cols = 524544, 4096
    n = rows * cols
    assert n > 2 ** 31
    say(f"[gpu] beyond 2^31 elements: {rows} x {cols}, int{bits} g{group}, bf16 state={sb}")
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    x0 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    x1 = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    chunk = 1 << 28
    for o in range(0, n, chunk):  # fp32 draws a chunk at a time, kept as bf16
        k = min(chunk, n - o)
        a = torch.randn(k, generator=g, device=DEV)
        x0[o:o + k] = a.bfloat16()
        x1[o:o + k] = (0.98 * a + 0.2 * torch.randn(k, generator=g, device=DEV)).bfloat16()
        del a
    snd = cfz.Sender(rows, cols, bits, group, x0=x0, state_bf16=sb)
    rcv = cfz.Receiver(rows, cols, bits, group, x0=x0, state_bf16=sb)
    xhat = torch.empty(n, dtype=torch.bfloat16, device=DEV)
    snd.compress(x1)
    rcv.decompress(snd.codes, snd.scales, xhat)
    torch.cuda.synchronize()
    ngroups = n // group
    edge = 2 ** 31 // group
    picks = sorted({0, 1, ngroups // 3, ngroups // 2, edge - 2, edge - 1, edge, edge + 1,
                    ngroups - 2, ngroups - 1} |
                   {int(v) for v in np.linspace(2, ngroups - 3, 14)})
    per_code = group * bits // 8
    for gi in picks:
        lo, hi = gi * group, (gi + 1) * group
        os_ = oracle.Sender(group, bits, group, oracle.DELTA, x0=u16(x0[lo:hi]), state_bf16=sb)
        or_ = oracle.Receiver(group, bits, group, x0=u16(x0[lo:hi]), state_bf16=sb)
        oc, osc = os_.compress(u16(x1[lo:hi]))
        oxh = or_.decompress(oc, osc, want_xhat=True)
        tag = f"group {gi} (elements {lo}..{hi - 1})"
        assert np.array_equal(snd.codes[gi * per_code:(gi + 1) * per_code].cpu().numpy(), oc), \
            f"{tag}: codes"
        assert snd.scales[gi:gi + 1].cpu().numpy().view(np.uint32)[0] == \
            osc.view(np.uint32)[0], f"{tag}: scale"
        assert np.array_equal(u16(snd.prev[lo:hi]), os_.prev), f"{tag}: prev"
        assert np.array_equal(raw_bytes(snd.err[lo:hi]), os_.err.view(np.uint8)), f"{tag}: err"
        assert np.array_equal(raw_bytes(rcv.base[lo:hi]), or_.base.view(np.uint8)), \
            f"{tag}: receiver base"
        assert np.array_equal(u16(xhat[lo:hi]), oxh[1] if isinstance(oxh, tuple) else oxh), \
            f"{tag}: xhat"
    say(f"  {len(picks)} groups bit-exact, including groups {edge - 1} and {edge} at 2^31")
