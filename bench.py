"""Throughput of the residual codec on one MI355X.

One step = one denoising step of the FLUX.1-dev share at patch degree 4: the
57 layers' K and V (114 tensors of 1024 tokens x 3072 channels, bf16), each
layer's pair in one grouped compress launch (residual + error feedback + int4
group-64 quantization + state update, DELTA mode) and one grouped decode launch
(unpack + base update).  Inputs are seeded AR(1) activations, generated into
HBM before the timed region.  A layer's compress and decode stay in order on
one stream; the layers are spread round-robin over --streams streams (3 by
default) so that one layer's launches overlap another's, and the launches of
one step are captured once into a HIP graph and replayed.

value = bf16 activation bytes coded per second: 2 bytes x elements per step x
steps / elapsed (compress + decode).  The roofline entry is for the compress
kernel: algorithmic bytes per launch over its average launch duration, timed
with HIP events on the stream the kernels run on, in a second timed pass of
the same launches on one stream (events around the compress and the decode
phase of each step; overlapped launches have no duration of their own).

Further legs in the same JSON line: the tiny configuration's per-call latency, other
launch granularities (per tensor,
16 tensors), the three error-feedback readings with their receiver error,
bf16 state, int2 group-32 over all tensors in one launch, the CogVideoX-2b
share, the subspace iteration at r = 8/16/32, the rank-r compressor inside
error feedback (plain and deferred sender; random or warm-started Q0), and the
CPU oracle on a bounded sample of the same workload.

Usage: python bench.py [--gpus 1] [--steps 27] [--warmup 1] [--streams 3] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0  # MI355X HBM3E, published


def algorithmic_bytes(bits, group, mode="delta", state_bf16=False):
    """Bytes per element each kernel must move with the state layout of the library
    (carried error and base 4 bytes each in fp32 state, 2 in bf16 state)."""
    payload = bits / 8 + 4 / group
    w = 2 if state_bf16 else 4
    state = {"delta": 2 + 2 + w + w, "literal": 4 * w, "off": 2 * w}[mode]
    compress = 2 + state + payload           # read x, read+write state, write payload
    decode = payload + 2 * w                 # read payload, read+write base
    return compress, decode


def kernel_source_hash():
    p = os.path.join(ROOT, "diffusion_activation_residual_amd", "csrc", "codec_kernels.hip")
    with open(p, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()[:16]


def load_traffic(kernel, workload):
    """HBM traffic per launch from the committed rocprofv3 counter summary, if it was taken
    on the current kernel source; else None."""
    p = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        with open(p) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    e = rec.get(kernel, {})
    if e.get("source_hash") != kernel_source_hash() or e.get("workload") != workload:
        return None
    return e.get("bytes_per_launch")


def host_cpu():
    """The host's CPU model name and the cores this process may run on."""
    model = None
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {"cpu_model": model, "nproc": os.cpu_count(),
            "cores_available": len(os.sched_getaffinity(0))}


def _cpu_codec_rate(xs_host, bits, group, budget_s):
    import oracle

    n_tensors = len(xs_host[0])
    n = xs_host[0][0].size
    done, t_total = 0, 0.0
    snd = [oracle.Sender(n, bits, group, oracle.DELTA, x0=xs_host[0][i]) for i in range(n_tensors)]
    rcv = [oracle.Receiver(n, bits, group, x0=xs_host[0][i]) for i in range(n_tensors)]
    for t in range(1, len(xs_host)):
        for i in range(n_tensors):
            t0 = time.perf_counter()
            c, s = snd[i].compress(xs_host[t][i])
            rcv[i].decompress(c, s)
            t_total += time.perf_counter() - t0
            done += 1
            if t_total > budget_s:
                break
        if t_total > budget_s:
            break
    return done, t_total, 2 * done * n / t_total / 1e9


def cpu_baseline(xs_host, bits, group, budget_s=20.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload: its OpenMP
    build on all the host's cores (same source, bit-identical results), and beside it the
    single-threaded build."""
    import oracle

    with oracle.parallel():
        cores = oracle.threads()
        done_p, t_p, rate_p = _cpu_codec_rate(xs_host, bits, group, budget_s / 2)
    done_1, t_1, rate_1 = _cpu_codec_rate(xs_host, bits, group, budget_s)
    what = f"1024x3072 (compress+decode, int{bits} g{group}, DELTA)"
    out = {"value": round(rate_p, 4), "unit": "GB/s", "cores": cores, "kind": "oracle",
           "sample": f"{done_p} tensor-steps of {what}, C oracle built with OpenMP on {cores} "
                     f"threads, {t_p:.1f} s",
           **host_cpu(),
           "single_core": {"value": round(rate_1, 4), "unit": "GB/s", "cores": 1,
                           "sample": f"{done_1} tensor-steps of {what}, single-threaded C "
                                     f"oracle, {t_1:.1f} s"}}
    return out


def bench_batched(cfz, torch, X, slots, rows, cols, bits, group, steps, label=None):
    """All tensors of a step in one compress and one decode launch (rows = tensors x tokens)."""
    n = rows * cols
    dev = X.device
    prev = torch.empty(n, dtype=torch.bfloat16, device=dev)
    err = torch.empty(n, dtype=torch.float32, device=dev)
    base = torch.empty(n, dtype=torch.float32, device=dev)
    codes = torch.empty(n * bits // 8, dtype=torch.uint8, device=dev)
    scales = torch.empty(n // group, dtype=torch.float32, device=dev)
    sd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_SENDER)
    rd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_RECEIVER)
    snd = cfz.cfz_state_create(sd, prev=prev, err=err, x0=X[0])
    rcv = cfz.cfz_state_create(rd, base=base, x0=X[0])
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps + 1)]
    for k in range(steps + 1):  # the first step is an untimed warm-up
        s = 1 + k % (slots - 1)
        ev[k][0].record()
        cfz.cfz_compress(snd, X[s], codes, scales)
        ev[k][1].record()
        cfz.cfz_decompress(rcv, codes, scales, None)
        ev[k][2].record()
    torch.cuda.synchronize()
    tc = sum(e[0].elapsed_time(e[1]) for e in ev[1:]) / 1e3 / steps
    td = sum(e[1].elapsed_time(e[2]) for e in ev[1:]) / 1e3 / steps
    cfz.cfz_state_destroy(snd)
    cfz.cfz_state_destroy(rcv)
    bc, bd = algorithmic_bytes(bits, group)
    if label is None:
        label = f"flux-share all 114 tensors in one launch ({rows}x{cols})"
    return {"workload": f"{label}, int{bits} g{group}, delta", "steps": steps,
            "activation_GB/s": round(2 * n / (tc + td) / 1e9, 2),
            "compress": {"us": round(tc * 1e6, 2), "GB/s": round(bc * n / tc / 1e9, 1),
                         "frac_hbm_peak": round(bc * n / tc / 1e9 / HBM_PEAK_GBS, 4)},
            "decode": {"us": round(td * 1e6, 2), "GB/s": round(bd * n / td / 1e9, 1),
                       "frac_hbm_peak": round(bd * n / td / 1e9 / HBM_PEAK_GBS, 4)}}


def bench_tiny(cfz, torch, dev, reps=200):
    """The tiny configuration (one 256 x 512 tensor, int4 g64, DELTA, its 4 seeded steps): a
    latency figure, not a bandwidth one -- the tensor sits in cache.  Each compress and decode
    call launched back to back reps times, eagerly and from a HIP graph of reps launches."""
    from synth import SPECS, AR1Stream

    sp = SPECS["tiny"]
    st = AR1Stream.from_spec(sp, seed=0, device=dev)
    xs = [st.next()[0].contiguous() for _ in range(sp.steps)]
    snd = cfz.Sender(sp.rows, sp.cols, 4, 64, x0=xs[0])
    rcv = cfz.Receiver(sp.rows, sp.cols, 4, 64, x0=xs[0])
    out = {"workload": f"tiny {sp.rows}x{sp.cols} int4 g64 delta, {sp.steps} steps"}

    def calls(k):
        x = xs[1 + k % (sp.steps - 1)]
        cfz.cfz_compress(snd.handle, x, snd.codes, snd.scales)
        cfz.cfz_decompress(rcv.handle, snd.codes, snd.scales)

    for k in range(reps // 10):
        calls(k)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(reps):
        calls(k)
    e1.record()
    torch.cuda.synchronize()
    out["eager_us_per_compress_plus_decode"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=cap):
        for k in range(reps):
            calls(k)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    out["graph_us_per_compress_plus_decode"] = round(e0.elapsed_time(e1) * 1e3 / reps, 2)
    snd.close()
    rcv.close()
    return out


def bench_lowrank(cfz, torch, dev, batch=57, m=1024, n=3072, T=2, reps=5):
    """Algorithm 3 on 57 layer residuals of 1024 x 3072 (rank-16 signal + 0.05 noise)."""
    from synth import gaussian_q0, lowrank_batch

    A = lowrank_batch(batch, m, n, rank=16, sigma=0.05, seed=7, device=dev)
    out = {"workload": f"{batch} x {m}x{n} bf16, rank-16 + 0.05 noise, T={T}", "per_rank": {},
           "A_layer0": A[0]}
    for r in (8, 16, 32):
        Q0 = gaussian_q0(batch, n, r, seed=r, device=dev)
        U = torch.empty(batch, m, r, device=dev)
        V = torch.empty(batch, n, r, device=dev)
        RU = torch.empty(batch, r, r, device=dev)
        ws = torch.empty(cfz.cfz_lowrank_workspace_bytes(batch, m, n, r), dtype=torch.uint8,
                         device=dev)
        def timed(iters):
            cfz.cfz_lowrank(batch, m, n, r, iters, A, Q0, U, V, RU, ws)
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                cfz.cfz_lowrank(batch, m, n, r, iters, A, Q0, U, V, RU, ws)
            e1.record()
            torch.cuda.synchronize()
            return e0.elapsed_time(e1) / 1e3 / reps

        t1 = timed(T - 1) if T >= 2 else None
        t = timed(T)  # last, so that U, V, R_U hold the T-iteration result
        # algorithmic bytes: A read once, Q0 read, U, V, R_U written
        alg = batch * (2 * m * n + 4 * n * r + 4 * (m + n) * r + 4 * r * r)
        useful_flop = batch * 2 * m * n * r * (2 * T + 1)
        # A^T (A Q) reads A once per iteration for r <= 16 and n <= 3072 (the library's
        # one-pass product), twice otherwise; the final A Q reads it once more
        passes = (T if r <= 16 and n <= 3072 else 2 * T) + 1
        out["per_rank"][str(r)] = {
            "ms_per_call": round(t * 1e3, 4), "us_per_layer": round(t * 1e6 / batch, 2),
            "achieved_GB/s_single_read": round(alg / t / 1e9, 1),
            "frac_hbm_peak_single_read": round(alg / t / 1e9 / HBM_PEAK_GBS, 4),
            "A_passes": passes,
            "achieved_GB/s_all_passes": round(passes * batch * 2 * m * n / t / 1e9, 1),
            "useful_TFLOP/s": round(useful_flop / t / 1e12, 2)}
        if t1 is not None:
            # one iteration (A^T (A Q) and the orthogonalisation of Z) = the difference
            # between T and T - 1 iterations
            it, reads = t - t1, (passes - 1) // T
            out["per_rank"][str(r)].update({
                "us_per_iteration": round(it * 1e6, 1),
                "A_reads_per_iteration": reads,
                "A_GB/s_in_iteration": round(reads * batch * 2 * m * n / it / 1e9, 1)})
        del ws
    return out


def bench_lowrank_ef(cfz, torch, dev, batch=57, m=1024, n=3072, r=16, T=2, steps=6):
    """The rank-r compressor inside error feedback on 57 layers of 1024 x 3072 per step:
    activations drift by rank 16 + noise per step.  One step = one sender call (residual,
    subspace iteration, error update) and one receiver call (base update + bf16 output);
    timed again with the deferred sender (each step's error update applied inside the next
    step's residual pass; the last one flushed after the timed steps).
    Timed with a fresh random Q0 per step; then, over the same consecutive steps, the
    receiver's relative error ||base - x|| / ||x|| with random or warm-started Q0 (the
    previous step's V) at T = 1 and T = 2."""
    from synth import LowrankDrift, gaussian_q0

    st = LowrankDrift(batch, m, n, rank=16, seed=3, device=dev)
    X = [st.next() for _ in range(steps + 2)]  # consecutive steps: warm-up + steps + 1
    del st
    Q0 = [gaussian_q0(batch, n, r, seed=s, device=dev) for s in range(steps + 1)]
    xhat = torch.empty(batch * m * n, dtype=torch.bfloat16, device=dev)

    def run(T_, warm, timed, deferred=False):
        snd = cfz.LowrankSender(batch, m, n, r, x0=X[0], deferred=deferred)
        rcv = cfz.LowrankReceiver(batch, m, n, r, x0=X[0])
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps + 1)]
        for k in range(steps + 1):  # the first step is an untimed warm-up
            q = snd.V.clone() if (warm and k > 0) else Q0[k]
            ev[k][0].record()
            snd.compress(X[1 + k], q, T_)
            ev[k][1].record()
            rcv.decompress(snd.U, snd.V, snd.RU, xhat)
            ev[k][2].record()
        snd.flush()
        torch.cuda.synchronize()
        tc = sum(e[0].elapsed_time(e[1]) for e in ev[1:]) / 1e3 / steps
        td = sum(e[1].elapsed_time(e[2]) for e in ev[1:]) / 1e3 / steps
        x_last = X[steps + 1].float().reshape(-1)
        rel = (torch.linalg.vector_norm(rcv.base - x_last) / torch.linalg.vector_norm(x_last)).item()
        del snd, rcv
        return tc, td, rel

    tc, td, rel = run(T, False, True)
    tcd, tdd, reld = run(T, False, True, deferred=True)
    accuracy = {}
    for T_, warm in ((1, False), (2, False), (1, True), (2, True)):
        c, _, e = run(T_, warm, False)
        accuracy[f"{'warm' if warm else 'random'}_Q0_T{T_}"] = {
            "compress_ms": round(c * 1e3, 4), "receiver_rel_error_last_step": float(f"{e:.4g}")}
    elems = batch * m * n
    payload = batch * 4 * (m * r + r * r + n * r)
    upd_bytes = 10 * elems  # read + write fp32 base, write bf16 xhat
    del X, Q0, xhat
    return {"workload": f"{batch} x {m}x{n}, activations drifting by rank 16 + 0.05 noise, "
                        f"r={r}, T={T}, random Q0 each step", "steps": steps,
            "activation_GB/s": round(2 * elems / (tc + td) / 1e9, 2),
            "compress_ms": round(tc * 1e3, 4), "decompress_ms": round(td * 1e3, 4),
            "receiver_rel_error_last_step": float(f"{rel:.4g}"),
            "compression_ratio_vs_bf16": round(2 * elems / payload, 1),
            "deferred_sender": {
                "note": "each step's error update applied inside the next step's residual pass "
                        "(bit-identical factors and states)",
                "activation_GB/s": round(2 * elems / (tcd + tdd) / 1e9, 2),
                "compress_ms": round(tcd * 1e3, 4),
                "receiver_rel_error_last_step": float(f"{reld:.4g}")},
            "decompress_update_kernel": {
                "GB/s": round(upd_bytes / td / 1e9, 1),
                "frac_hbm_peak": round(upd_bytes / td / 1e9 / HBM_PEAK_GBS, 4),
                "bytes_per_elem": 10},
            "q0_and_T": accuracy}


def bench_ef_modes(cfz, torch, X, slots, rows, cols, steps=10):
    """The three error-feedback readings on the FLUX share at int4 g64 and int2 g32, one
    grouped compress and one grouped decode launch per layer from HIP graphs, steps
    1..steps+1 in order (the first untimed): kernel rates against each mode's algorithmic
    bytes, and the receiver's relative error ||base - x|| / ||x|| after the last step."""
    T = X.shape[1]
    out = {"workload": f"flux-share {T} tensors of {rows}x{cols}, one grouped launch per layer "
                       "(K and V), replayed from HIP graphs", "steps": steps}
    for bits, group in ((4, 64), (2, 32)):
        out[f"int{bits}_g{group}"] = _ef_modes_one(cfz, torch, X, slots, rows, cols, bits, group,
                                                   steps)
        torch.cuda.empty_cache()
    return out


def _ef_modes_one(cfz, torch, X, slots, rows, cols, bits, group, steps):
    T, n = X.shape[1], X.shape[2]
    dev = X.device
    codes = torch.empty((T, n * bits // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, n // group), dtype=torch.float32, device=dev)
    rbase = torch.empty((T, n), dtype=torch.float32, device=dev)
    layers = [(2 * l, 2 * l + 1) for l in range(T // 2)]
    names = {cfz.CFZ_EF_DELTA: "delta", cfz.CFZ_EF_LITERAL: "literal", cfz.CFZ_EF_OFF: "off"}
    out = {}
    for mode in (cfz.CFZ_EF_DELTA, cfz.CFZ_EF_LITERAL, cfz.CFZ_EF_OFF):
        sd = cfz.make_desc(rows, cols, bits, group, mode, cfz.CFZ_SENDER)
        rd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_RECEIVER)
        prev = torch.empty((T, n), dtype=torch.bfloat16, device=dev) if mode == cfz.CFZ_EF_DELTA else None
        sbase = torch.empty((T, n), dtype=torch.float32, device=dev) if mode != cfz.CFZ_EF_DELTA else None
        err = torch.empty((T, n), dtype=torch.float32, device=dev) if mode != cfz.CFZ_EF_OFF else None

        def states():
            return ([cfz.cfz_state_create(sd, prev=None if prev is None else prev[i],
                                          base=None if sbase is None else sbase[i],
                                          err=None if err is None else err[i], x0=X[0, i])
                     for i in range(T)],
                    [cfz.cfz_state_create(rd, base=rbase[i], x0=X[0, i]) for i in range(T)])

        snd, rcv = states()
        slot_of = [1 + k % (slots - 1) for k in range(steps + 1)]
        cap = torch.cuda.Stream()
        cap.wait_stream(torch.cuda.current_stream())
        gc = {}
        for s_ in sorted(set(slot_of)):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=cap):
                for c in layers:
                    cfz.cfz_compress_group([snd[i] for i in c], [X[s_, i] for i in c],
                                           [codes[i] for i in c], [scales[i] for i in c])
            gc[s_] = g
        gd = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gd, stream=cap):
            for c in layers:
                cfz.cfz_decompress_group([rcv[i] for i in c], [codes[i] for i in c],
                                         [scales[i] for i in c])
        torch.cuda.synchronize()
        for h in snd + rcv:  # capture only recorded the launches; start from a fresh warm-up
            cfz.cfz_state_destroy(h)
        snd[:], rcv[:] = states()
        ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps + 1)]
        for k in range(steps + 1):
            ev[k][0].record()
            gc[slot_of[k]].replay()
            ev[k][1].record()
            gd.replay()
            ev[k][2].record()
        torch.cuda.synchronize()
        tc = sum(e[0].elapsed_time(e[1]) for e in ev[1:]) / 1e3 / (steps * len(layers))
        td = sum(e[1].elapsed_time(e[2]) for e in ev[1:]) / 1e3 / (steps * len(layers))
        x_last = X[slot_of[-1]].float()
        rel = (torch.linalg.vector_norm(rbase - x_last) / torch.linalg.vector_norm(x_last)).item()
        for h in snd + rcv:
            cfz.cfz_state_destroy(h)
        del gc, gd
        bc, bd = algorithmic_bytes(bits, group, names[mode])
        out[names[mode]] = {
            "compress": {"avg_launch_us": round(tc * 1e6, 3),
                         "GB/s": round(bc * 2 * n / tc / 1e9, 1),
                         "frac_hbm_peak": round(bc * 2 * n / tc / 1e9 / HBM_PEAK_GBS, 4),
                         "bytes_per_elem": bc},
            "decode": {"avg_launch_us": round(td * 1e6, 3),
                       "GB/s": round(bd * 2 * n / td / 1e9, 1),
                       "frac_hbm_peak": round(bd * 2 * n / td / 1e9 / HBM_PEAK_GBS, 4)},
            "activation_GB/s": round(2 * n * T / ((tc + td) * len(layers)) / 1e9, 2),
            "receiver_rel_error_last_step": float(f"{rel:.4g}")}
    return out


def bench_error_trajectory(cfz, torch, X, slots, rows, cols, bits=4, group=64):
    """Receiver error ||X_t - base_t|| / ||X_t|| over all tensors after every compressed step
    (steps 1 .. slots - 1 of the pre-generated, consecutive AR(1) steps, DELTA, grouped per
    layer), beside the error of quantizing each X_t directly with the same quantizer (a
    closed loop from a zero base, re-warmed every step): the residual scheme's gain is their
    ratio.  The abstract claims temporal redundancy and error feedback that keeps the error
    from accumulating: the trajectory should stay flat."""
    T, n = X.shape[1], X.shape[2]
    dev = X.device
    prev = torch.empty((T, n), dtype=torch.bfloat16, device=dev)
    err = torch.empty((T, n), dtype=torch.float32, device=dev)
    base = torch.empty((T, n), dtype=torch.float32, device=dev)
    dbase_s = torch.empty((T, n), dtype=torch.float32, device=dev)
    dbase_r = torch.empty((T, n), dtype=torch.float32, device=dev)
    codes = torch.empty((T, n * bits // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, n // group), dtype=torch.float32, device=dev)
    sd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_SENDER)
    rd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_RECEIVER)
    od = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_OFF, cfz.CFZ_SENDER)
    snd = [cfz.cfz_state_create(sd, prev=prev[i], err=err[i], x0=X[0, i]) for i in range(T)]
    rcv = [cfz.cfz_state_create(rd, base=base[i], x0=X[0, i]) for i in range(T)]
    layers = [(2 * l, 2 * l + 1) for l in range(T // 2)]
    res, direct = [], []
    for t in range(1, slots):
        for c in layers:
            cfz.cfz_compress_group([snd[i] for i in c], [X[t, i] for i in c],
                                   [codes[i] for i in c], [scales[i] for i in c])
            cfz.cfz_decompress_group([rcv[i] for i in c], [codes[i] for i in c],
                                     [scales[i] for i in c])
        xt = X[t].float()
        res.append((torch.linalg.vector_norm(base - xt) / torch.linalg.vector_norm(xt)).item())
        # direct: quantize X_t itself (zero base, re-warmed), decode into a zero base
        ds = [cfz.cfz_state_create(od, base=dbase_s[i]) for i in range(T)]
        dr = [cfz.cfz_state_create(rd, base=dbase_r[i]) for i in range(T)]
        for c in layers:
            cfz.cfz_compress_group([ds[i] for i in c], [X[t, i] for i in c],
                                   [codes[i] for i in c], [scales[i] for i in c])
            cfz.cfz_decompress_group([dr[i] for i in c], [codes[i] for i in c],
                                     [scales[i] for i in c])
        direct.append((torch.linalg.vector_norm(dbase_r - xt) / torch.linalg.vector_norm(xt)).item())
        for h in ds + dr:
            cfz.cfz_state_destroy(h)
    for h in snd + rcv:
        cfz.cfz_state_destroy(h)
    return {"workload": f"flux-share {T} tensors of {rows}x{cols}, int{bits} g{group}, delta, "
                        f"steps 1..{slots - 1}",
            "receiver_rel_error_by_step": [float(f"{e:.4g}") for e in res],
            "direct_quantization_rel_error_by_step": [float(f"{e:.4g}") for e in direct],
            "direct_over_residual_error_ratio_last_step": round(direct[-1] / res[-1], 3),
            "direct_over_residual_error_ratio_min": round(min(d / r for d, r in zip(direct, res)), 3)}


def bench_cogvideox(cfz, torch, dev, bits, group, steps=10, pool=4):
    """CogVideoX-2b share at sequence-parallel degree 4: 30 layers x {K, V} of 4388 x 1920
    bf16 (AR(1), alpha 0.97), DELTA, one grouped compress and one grouped decode launch per
    layer (its K and V), replayed from HIP graphs; then the same tensors as one contiguous
    batch, one compress and one decode launch per step."""
    from synth import SPECS, AR1Stream

    sp = SPECS["cogvideox"]
    T, rows, cols = sp.tensors, sp.rows, sp.cols
    n = rows * cols
    gen = AR1Stream.from_spec(sp, seed=0, device=dev)
    X = torch.empty((pool + 1, T, n), dtype=torch.bfloat16, device=dev)
    for s_ in range(pool + 1):
        X[s_] = gen.next().reshape(T, n)
    del gen
    prev = torch.empty((T, n), dtype=torch.bfloat16, device=dev)
    err = torch.empty((T, n), dtype=torch.float32, device=dev)
    base = torch.empty((T, n), dtype=torch.float32, device=dev)
    codes = torch.empty((T, n * bits // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, n // group), dtype=torch.float32, device=dev)
    sd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_SENDER)
    rd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_RECEIVER)
    layers = [(2 * l, 2 * l + 1) for l in range(T // 2)]

    def states():
        return ([cfz.cfz_state_create(sd, prev=prev[i], err=err[i], x0=X[0, i]) for i in range(T)],
                [cfz.cfz_state_create(rd, base=base[i], x0=X[0, i]) for i in range(T)])

    snd, rcv = states()

    def compress_phase(slot):
        for c in layers:
            cfz.cfz_compress_group([snd[i] for i in c], [X[slot, i] for i in c],
                                   [codes[i] for i in c], [scales[i] for i in c])

    def decode_phase():
        for c in layers:
            cfz.cfz_decompress_group([rcv[i] for i in c], [codes[i] for i in c],
                                     [scales[i] for i in c])

    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    gc = {}
    for s_ in range(1, pool + 1):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=cap):
            compress_phase(s_)
        gc[s_] = g
    gd = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gd, stream=cap):
        decode_phase()
    torch.cuda.synchronize()
    for h in snd + rcv:  # capture only recorded the launches; start from a fresh warm-up
        cfz.cfz_state_destroy(h)
    snd[:], rcv[:] = states()
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(steps + 1)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for k in range(steps + 1):  # the first step is an untimed warm-up
        if k == 1:
            torch.cuda.synchronize()
            t0 = time.perf_counter()
        ev[k][0].record()
        gc[1 + k % pool].replay()
        ev[k][1].record()
        gd.replay()
        ev[k][2].record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    tc = sum(e[0].elapsed_time(e[1]) for e in ev[1:]) / 1e3 / (steps * len(layers))
    td = sum(e[1].elapsed_time(e[2]) for e in ev[1:]) / 1e3 / (steps * len(layers))
    for h in snd + rcv:
        cfz.cfz_state_destroy(h)
    bc, bd = algorithmic_bytes(bits, group)
    per = 2 * n  # elements per launch
    del prev, err, base, codes, scales
    # the same tensors as one contiguous batch: one compress and one decode launch per step
    batched = bench_batched(cfz, torch, X.view(pool + 1, T * n), pool + 1, T * rows, cols, bits,
                            group, steps, label=f"cogvideox-2b-share all {T} tensors in one "
                                                f"launch ({T * rows}x{cols})")
    return {"workload": f"cogvideox-2b-share {T} tensors of {rows}x{cols}, int{bits} g{group}, "
                        "delta, one grouped launch per layer (K and V), replayed from HIP graphs",
            "steps": steps,
            "activation_GB/s": round(2 * n * T * steps / elapsed / 1e9, 2),
            "compress": {"avg_launch_us": round(tc * 1e6, 3), "GB/s": round(bc * per / tc / 1e9, 1),
                         "frac_hbm_peak": round(bc * per / tc / 1e9 / HBM_PEAK_GBS, 4)},
            "decode": {"avg_launch_us": round(td * 1e6, 3), "GB/s": round(bd * per / td / 1e9, 1),
                       "frac_hbm_peak": round(bd * per / td / 1e9 / HBM_PEAK_GBS, 4)},
            "one_launch_per_step": batched}


def lowrank_cpu_baseline(A_layer, batch, T=2, ranks=(8, 16, 32)):
    """The fp64 CPU oracle on one layer per rank, single-threaded and with OpenMP on all host
    cores; per-call figures scale the per-layer time by the batch."""
    import numpy as np

    import oracle
    from synth import gaussian_q0

    a = A_layer.contiguous().view(__import__("torch").int16).cpu().numpy().view(np.uint16)
    m, n = a.shape
    with oracle.parallel():
        cores = oracle.threads()
    res = {"kind": "oracle", "cores": cores, "unit": "ms per call", **host_cpu(),
           "sample": f"one {m}x{n} layer per rank, fp64 oracle with OpenMP on {cores} threads "
                     f"and single-threaded; per-call time = per-layer time x {batch} "
                     "(extrapolated)", "per_rank": {}}
    for r in ranks:
        q0 = gaussian_q0(1, n, r, seed=r)[0].numpy()
        with oracle.parallel():
            t0 = time.perf_counter()
            oracle.lowrank(a, q0, T)
            dp = time.perf_counter() - t0
        t0 = time.perf_counter()
        oracle.lowrank(a, q0, T)
        d1 = time.perf_counter() - t0
        res["per_rank"][str(r)] = {"ms_per_layer": round(dp * 1e3, 1),
                                   "ms_per_call": round(dp * 1e3 * batch, 1),
                                   "single_core_ms_per_layer": round(d1 * 1e3, 1),
                                   "single_core_ms_per_call": round(d1 * 1e3 * batch, 1)}
    return res


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=27)
    ap.add_argument("--warmup", type=int, default=1)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--streams", type=int, default=3,
                    help="streams the per-layer launches are spread over (1 = one stream)")
    ap.add_argument("--no-graph", action="store_true", help="launch eagerly instead of replaying graphs")
    ap.add_argument("--no-batched", action="store_true", help="skip the one-launch-per-step int2 leg")
    ap.add_argument("--no-lowrank", action="store_true", help="skip the subspace-iteration leg")
    ap.add_argument("--no-cogvideox", action="store_true",
                    help="skip the CogVideoX-2b-share legs (int4 g64 and int2 g32)")
    ap.add_argument("--launch", choices=("layer", "tensor", "step"), default="layer",
                    help="tensors per launch: K+V of a layer (default), one, or the whole step")
    ap.add_argument("--no-modes", action="store_true", help="skip the other launch granularities")
    ap.add_argument("--no-ef-modes", action="store_true",
                    help="skip the LITERAL / OFF error-feedback readings leg")
    ap.add_argument("--no-bf16-state", action="store_true",
                    help="skip the leg with the carried error and base held in bf16")
    ap.add_argument("--pool", type=int, default=29,
                    help="distinct pre-generated steps kept in HBM (inputs cycle through them)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU's share on one GPU; --gpus {args.gpus} is not "
              "supported (the codec shards per tensor with no cross-GPU work).", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from diffusion_activation_residual_amd import cadence, cfz
    from synth import SPECS, AR1Stream

    sp = SPECS["flux"]
    bits, group = 4, 64
    T, rows, cols = sp.tensors, sp.rows, sp.cols
    n = rows * cols
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    slots = max(2, min(K + W + 1, args.pool))
    print(f"[bench] generating {slots} steps of {T} x {rows} x {cols} bf16", file=sys.stderr,
          flush=True)
    gen = AR1Stream.from_spec(sp, seed=0, device=dev)
    X = torch.empty((slots, T, n), dtype=torch.bfloat16, device=dev)
    for s in range(slots):
        X[s] = gen.next().reshape(T, n)
    del gen
    torch.cuda.synchronize()

    prev = torch.empty((T, n), dtype=torch.bfloat16, device=dev)
    err = torch.empty((T, n), dtype=torch.float32, device=dev)
    base = torch.empty((T, n), dtype=torch.float32, device=dev)
    codes = torch.empty((T, n * bits // 8), dtype=torch.uint8, device=dev)
    scales = torch.empty((T, n // group), dtype=torch.float32, device=dev)
    half = {}  # bf16 carried error and base, allocated on first use

    def fresh_states(sb=False):
        sdt = cfz.CFZ_STATE_BF16 if sb else cfz.CFZ_STATE_F32
        if sb and not half:
            half["err"] = torch.empty((T, n), dtype=torch.bfloat16, device=dev)
            half["base"] = torch.empty((T, n), dtype=torch.bfloat16, device=dev)
        e_, b_ = (half["err"], half["base"]) if sb else (err, base)
        sd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_SENDER, sdt)
        rd = cfz.make_desc(rows, cols, bits, group, cfz.CFZ_EF_DELTA, cfz.CFZ_RECEIVER, sdt)
        s_ = [cfz.cfz_state_create(sd, prev=prev[i], err=e_[i], x0=X[0, i]) for i in range(T)]
        r_ = [cfz.cfz_state_create(rd, base=b_[i], x0=X[0, i]) for i in range(T)]
        return s_, r_

    def slot_of(step):  # step >= 1; wraps around the pre-generated pool
        return 1 + (step - 1) % (slots - 1)

    # tensors per call: 2 = the K and V of one layer, 1 = each tensor alone, T = the whole step
    per_call = {"layer": 2, "tensor": 1, "step": T}

    def run_mode(mode, K, W, use_graph, sb=False, streams=1):
        """K timed steps after W warm-up steps.  streams == 1: each step is a compress graph
        then a decode graph on one stream, with HIP events around each phase (per-launch
        kernel times).  streams > 1 (per-layer launches from graphs only): each step is one
        graph of the layers spread round-robin over the streams (the overlapped schedule),
        with events only at step boundaries."""
        g = per_call[mode]
        calls = [list(range(i, min(i + g, T))) for i in range(0, T, g)]
        launches = sum((len(c) + 15) // 16 for c in calls)
        if streams > 1 and not (mode == "layer" and use_graph):
            raise ValueError("several streams only for per-layer launches from graphs")
        snd, rcv = fresh_states(sb)

        def compress_phase(slot):
            for c in calls:
                if len(c) == 1:
                    cfz.cfz_compress(snd[c[0]], X[slot, c[0]], codes[c[0]], scales[c[0]])
                else:
                    cfz.cfz_compress_group([snd[i] for i in c], [X[slot, i] for i in c],
                                           [codes[i] for i in c], [scales[i] for i in c])

        def decode_phase():
            for c in calls:
                if len(c) == 1:
                    cfz.cfz_decompress(rcv[c[0]], codes[c[0]], scales[c[0]], None)
                else:
                    cfz.cfz_decompress_group([rcv[i] for i in c], [codes[i] for i in c],
                                             [scales[i] for i in c])

        graphs = None
        if use_graph:
            # capture advances the host-side step counters but enqueues no work; the states
            # are re-warmed afterwards, so replays start from step 0 like eager launches
            graphs = {}
            cap = torch.cuda.Stream()
            cap.wait_stream(torch.cuda.current_stream())
            if streams > 1:
                sts = [cap] + [torch.cuda.Stream() for _ in range(streams - 1)]
                for s_ in range(1, slots):
                    gs_ = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gs_, stream=cap):
                        cadence.enqueue_layer_step(calls, snd, rcv, X[s_], codes, scales, sts)
                    graphs[s_] = gs_
            else:
                gd = torch.cuda.CUDAGraph()
                with torch.cuda.graph(gd, stream=cap):
                    decode_phase()
                for s_ in range(1, slots):
                    gc = torch.cuda.CUDAGraph()
                    with torch.cuda.graph(gc, stream=cap):
                        compress_phase(s_)
                    graphs[s_] = gc
                graphs["dec"] = gd
            torch.cuda.synchronize()
            for h in snd + rcv:
                cfz.cfz_state_destroy(h)
            snd[:], rcv[:] = fresh_states(sb)
            torch.cuda.synchronize()

        def run_step(step, ev=None):
            s_ = slot_of(step)
            if streams > 1:
                graphs[s_].replay()
                if ev is not None:
                    ev.record()
                return
            if ev is not None:
                ev[0].record()
            graphs[s_].replay() if graphs else compress_phase(s_)
            if ev is not None:
                ev[1].record()
            graphs["dec"].replay() if graphs else decode_phase()
            if ev is not None:
                ev[2].record()

        for step in range(1, W + 1):
            run_step(step)
        torch.cuda.synchronize()
        if streams > 1:  # one event per step boundary
            evs = [torch.cuda.Event(enable_timing=True) for _ in range(K + 1)]
        else:
            evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(K)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        if streams > 1:
            evs[0].record()
        for k in range(K):
            run_step(W + 1 + k, evs[k + 1] if streams > 1 else evs[k])
        torch.cuda.synchronize()
        elapsed = time.perf_counter() - t0
        for h in snd + rcv:
            cfz.cfz_state_destroy(h)
        if streams > 1:
            t_comp = t_dec = None
            per_step_ms = sorted(evs[k].elapsed_time(evs[k + 1]) for k in range(K))
        else:
            t_comp = sum(e[0].elapsed_time(e[1]) for e in evs) / 1e3
            t_dec = sum(e[1].elapsed_time(e[2]) for e in evs) / 1e3
            per_step_ms = sorted(e[0].elapsed_time(e[2]) for e in evs)
        return {"elapsed": elapsed, "t_comp": t_comp, "t_dec": t_dec, "launches": launches,
                "tensors_per_launch": T / launches, "per_step_ms": per_step_ms}

    overlap = args.launch == "layer" and not args.no_graph and args.streams > 1
    nstreams = args.streams if overlap else 1
    print(f"[bench] timing {K} steps ({args.launch} launches, {nstreams} stream(s))",
          file=sys.stderr, flush=True)
    res = run_mode(args.launch, K, W, not args.no_graph, streams=nstreams)
    elapsed = res["elapsed"]
    # per-launch kernel times: the same launches on one stream, events around each phase
    if overlap:
        print(f"[bench] timing {K} steps on one stream (per-launch kernel times)",
              file=sys.stderr, flush=True)
        kres = run_mode(args.launch, K, W, True, streams=1)
    else:
        kres = res
    t_comp, t_dec = kres["t_comp"], kres["t_dec"]
    bc, bd = algorithmic_bytes(bits, group)
    n_launch = K * kres["launches"]
    per_launch_elems = n * T / res["launches"]
    avg_comp = t_comp / n_launch
    avg_dec = t_dec / n_launch
    comp_gbs = bc * per_launch_elems / avg_comp / 1e9
    dec_gbs = bd * per_launch_elems / avg_dec / 1e9
    act_bytes = 2 * n * T * K
    value = act_bytes / elapsed / 1e9

    other_modes = {}
    for mode in ("layer", "tensor", "step"):
        if mode == args.launch or args.no_modes:
            continue
        print(f"[bench] {mode} launches", file=sys.stderr, flush=True)
        r_ = run_mode(mode, min(K, 10), 1, not args.no_graph)
        nl = min(K, 10) * r_["launches"]
        pe = n * T / r_["launches"]
        other_modes[mode] = {
            "tensors_per_launch": round(r_["tensors_per_launch"], 2),
            "activation_GB/s": round(2 * n * T * min(K, 10) / r_["elapsed"] / 1e9, 2),
            "compress_GB/s": round(bc * pe / (r_["t_comp"] / nl) / 1e9, 1),
            "decode_GB/s": round(bd * pe / (r_["t_dec"] / nl) / 1e9, 1)}

    # the same per-layer launches with the carried error and the base held in bf16
    bf16_state = None
    if not args.no_bf16_state:
        print("[bench] bf16-state leg", file=sys.stderr, flush=True)
        kb = min(K, 10)
        r_ = run_mode(args.launch, kb, 1, not args.no_graph, sb=True)
        r_ov = run_mode(args.launch, kb, 1, True, sb=True, streams=nstreams) if overlap else r_
        bc16, bd16 = algorithmic_bytes(bits, group, state_bf16=True)
        nl = kb * r_["launches"]
        pe = n * T / r_["launches"]
        c16 = bc16 * pe / (r_["t_comp"] / nl) / 1e9
        d16 = bd16 * pe / (r_["t_dec"] / nl) / 1e9
        wl16 = f"flux-share-57x2x1024x3072-int4-g64-delta-bf16state/{args.launch}"
        bf16_state = {
            "workload": f"{T} tensors of {rows}x{cols}, int{bits} g{group}, delta, carried "
                        "error and base in bf16", "steps": kb,
            "traffic_bytes_per_launch": {"compress": load_traffic("compress_bf16_state", wl16),
                                         "decode": load_traffic("decode_bf16_state", wl16)},
            "activation_GB/s": round(2 * n * T * kb / r_ov["elapsed"] / 1e9, 2),
            "activation_GB/s_one_stream": round(2 * n * T * kb / r_["elapsed"] / 1e9, 2),
            "step_hbm": {"GB/s": round((bc16 + bd16) * n * T * kb / r_ov["elapsed"] / 1e9, 1),
                         "frac_hbm_peak": round((bc16 + bd16) * n * T * kb / r_ov["elapsed"] / 1e9
                                                / HBM_PEAK_GBS, 4),
                         "bytes_per_elem": bc16 + bd16},
            "compress": {"avg_launch_us": round(r_["t_comp"] / nl * 1e6, 3),
                         "GB/s": round(c16, 1), "frac_hbm_peak": round(c16 / HBM_PEAK_GBS, 4),
                         "bytes_per_elem": bc16},
            "decode": {"avg_launch_us": round(r_["t_dec"] / nl * 1e6, 3),
                       "GB/s": round(d16, 1), "frac_hbm_peak": round(d16 / HBM_PEAK_GBS, 4),
                       "bytes_per_elem": bd16}}
        half.clear()

    # achievable copy ceiling on a buffer as large as two steps of activations
    src = X[1:3].reshape(-1)
    dst = torch.empty_like(src)
    cfz.cfz_stream_copy(src, dst)
    torch.cuda.synchronize()
    ce = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
    ce[0].record()
    for _ in range(3):
        cfz.cfz_stream_copy(src, dst)
    ce[1].record()
    torch.cuda.synchronize()
    copy_gbs = 3 * 2 * src.numel() * 2 / (ce[0].elapsed_time(ce[1]) / 1e3) / 1e9
    del dst
    # the same copy kernel at the compress launch's traffic (read + write = its algorithmic
    # bytes), 57 launches replayed from a graph: what a launch of that size can reach
    lay_elems = int(bc * n * 2) // 4  # 2-byte elements: half the bytes read, half written
    lay_elems -= lay_elems % 8
    flat = X.reshape(-1)
    srcs = torch.empty(57 * lay_elems, dtype=torch.bfloat16, device=dev)
    for o in range(0, srcs.numel(), flat.numel()):  # activation data, not an empty buffer
        k = min(flat.numel(), srcs.numel() - o)
        srcs[o:o + k].copy_(flat[:k])
    srcs = srcs.view(57, lay_elems)
    dsts = torch.empty_like(srcs)
    cap = torch.cuda.Stream()
    cap.wait_stream(torch.cuda.current_stream())
    gcopy = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gcopy, stream=cap):
        for i in range(57):
            cfz.cfz_stream_copy(srcs[i], dsts[i], stream=cap)
    torch.cuda.synchronize()
    gcopy.replay()
    torch.cuda.synchronize()
    ce[0].record()
    for _ in range(3):
        gcopy.replay()
    ce[1].record()
    torch.cuda.synchronize()
    layer_copy_gbs = 3 * 57 * 2 * lay_elems * 2 / (ce[0].elapsed_time(ce[1]) / 1e3) / 1e9
    del dsts, gcopy
    # the same streams at the codec's own read:write ratios (compress 8 : 6.5625, decode
    # 4.5625 : 4 bytes per element): a large launch, and 57 launches of the per-layer size
    mix = {}
    big = src.numel() * 2 // 16 * 16
    dst_big = torch.empty(big // 2, dtype=torch.bfloat16, device=dev)
    # compress reads x, prev and err (8 B) and writes the rest; decode reads the payload and
    # the base and writes the base (4 B)
    for name, rd, wr in (("compress", 8.0, bc - 8.0), ("decode", bd - 4.0, 4.0)):
        wbig = int(big * wr / rd) // 16 * 16
        cfz.cfz_stream_mix(src, big, dst_big, wbig)
        torch.cuda.synchronize()
        ce[0].record()
        for _ in range(3):
            cfz.cfz_stream_mix(src, big, dst_big, wbig)
        ce[1].record()
        torch.cuda.synchronize()
        big_gbs = 3 * (big + wbig) / (ce[0].elapsed_time(ce[1]) / 1e3) / 1e9
        lr_ = int(rd * n * 2) // 16 * 16   # one layer's K and V: 2 n elements
        lw_ = int(wr * n * 2) // 16 * 16
        flat_src = srcs.view(-1).view(torch.uint8)
        msrc = flat_src[: 57 * lr_].view(57, lr_) if flat_src.numel() >= 57 * lr_ else None
        if msrc is None:
            msrc = torch.empty((57, lr_), dtype=torch.uint8, device=dev)
            msrc.view(-1)[: flat_src.numel()].copy_(flat_src[: msrc.numel()])
        mdst = torch.empty((57, max(lw_, 16)), dtype=torch.uint8, device=dev)
        gmix = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gmix, stream=cap):
            for i in range(57):
                cfz.cfz_stream_mix(msrc[i], lr_, mdst[i], lw_, stream=cap)
        torch.cuda.synchronize()
        gmix.replay()
        torch.cuda.synchronize()
        ce[0].record()
        for _ in range(3):
            gmix.replay()
        ce[1].record()
        torch.cuda.synchronize()
        lay_gbs = 3 * 57 * (lr_ + lw_) / (ce[0].elapsed_time(ce[1]) / 1e3) / 1e9
        mix[name] = {"read_to_write": f"{rd:g}:{wr:g}", "large_launch_GB/s": round(big_gbs, 1),
                     "per_layer_launch_GB/s": round(lay_gbs, 1)}
        del mdst, gmix
    del dst_big, srcs

    workload = "flux-share-57x2x1024x3072-int4-g64-delta"
    traffic = load_traffic("compress", f"{workload}/{args.launch}")
    line = {
        "metric": "codec GB/s of bf16 activation (compress+decode) and % of HBM peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(elapsed / K * 1e3, 4),
        "step_ms_events": {  # compress + decode of one step, HIP events at step boundaries
            "median": round(res["per_step_ms"][len(res["per_step_ms"]) // 2], 4),
            "min": round(res["per_step_ms"][0], 4),
            "max": round(res["per_step_ms"][-1], 4)},
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",  # the codec's arithmetic: residual, scale division and updates in fp32
        "activation_dtype": "bf16",  # what the metric counts: bf16 activation bytes
        "state_dtype": "f32",  # carried error and base (the bf16_state leg holds them in bf16)
        "data": "synthetic (seeded AR(1) bf16 activations, alpha 0.98, LogNormal(0,0.5) channel "
                "scales, 1% outlier channels x20)",
        "config": {"workload": workload, "tensors": T, "rows": rows, "cols": cols, "bits": bits,
                   "group": group, "ef_mode": "delta",
                   "launch": {"layer": "one grouped compress and decode launch per layer (K and V)",
                              "tensor": "one compress and decode launch per tensor",
                              "step": "grouped launches of 16 tensors over the whole step"}[
                       args.launch] + (f", layers round-robin over {nstreams} streams, one HIP "
                                       "graph per step" if overlap else
                                       ", replayed from HIP graphs" if not args.no_graph else
                                       ", eager"),
                   "streams": nstreams},
        "roofline": {"bound": "hbm", "achieved": round(comp_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(comp_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "cfz_compress_kernel<bits=4, G=64, DELTA>",
                     "bytes_per_launch": int(bc * per_launch_elems),
                     "avg_launch_us": round(avg_comp * 1e6, 3)},
        "kernels": {
            "compress": {"avg_launch_us": round(avg_comp * 1e6, 3), "GB/s": round(comp_gbs, 1),
                         "frac_hbm_peak": round(comp_gbs / HBM_PEAK_GBS, 4),
                         "bytes_per_elem": bc},
            "decode": {"avg_launch_us": round(avg_dec * 1e6, 3), "GB/s": round(dec_gbs, 1),
                       "frac_hbm_peak": round(dec_gbs / HBM_PEAK_GBS, 4), "bytes_per_elem": bd},
            "stream_copy_ceiling_GB/s": round(copy_gbs, 1),
            "stream_copy_at_compress_launch_size_GB/s": round(layer_copy_gbs, 1),
            "stream_mix_at_codec_ratios": mix,
        },
        "schedules": {  # activation GB/s of the same per-layer launches
            f"{nstreams}_streams": round(value, 2),
            "1_stream": round(2 * n * T * K / kres["elapsed"] / 1e9, 2)},
        # the whole step's algorithmic bytes (compress + decode of every tensor) over its time
        "step_hbm": {"GB/s": round((bc + bd) * n * T * K / elapsed / 1e9, 1),
                     "frac_hbm_peak": round((bc + bd) * n * T * K / elapsed / 1e9 / HBM_PEAK_GBS, 4),
                     "bytes_per_elem": bc + bd},
        "other_launch_granularities": other_modes,
        "bf16_state": bf16_state,
        "compression_ratio_vs_bf16": round(2 / (bits / 8 + 4 / group), 3),
    }
    print("[bench] error trajectory leg", file=sys.stderr, flush=True)
    line["error_trajectory"] = bench_error_trajectory(cfz, torch, X, slots, rows, cols)
    torch.cuda.empty_cache()
    if not args.no_ef_modes:
        print("[bench] error-feedback readings leg", file=sys.stderr, flush=True)
        line["ef_modes"] = bench_ef_modes(cfz, torch, X, slots, rows, cols, steps=min(K, 10))
        torch.cuda.empty_cache()
    if not args.no_batched:
        print("[bench] batched int2 leg", file=sys.stderr, flush=True)
        line["batched_int2_g32"] = bench_batched(cfz, torch, X, slots, T * rows, cols, 2, 32,
                                                 steps=min(K, 10))
    print("[bench] tiny-configuration latency leg", file=sys.stderr, flush=True)
    line["tiny_latency"] = bench_tiny(cfz, torch, dev)
    if not args.no_cogvideox:
        for cb, cg in ((4, 64), (2, 32)):
            print(f"[bench] CogVideoX-share leg, int{cb} g{cg}", file=sys.stderr, flush=True)
            line[f"cogvideox_int{cb}_g{cg}"] = bench_cogvideox(cfz, torch, dev, cb, cg)
            torch.cuda.empty_cache()
    if not args.no_lowrank:
        print("[bench] subspace-iteration leg", file=sys.stderr, flush=True)
        lr = bench_lowrank(cfz, torch, dev)
        a0 = lr.pop("A_layer0")
        if not args.no_cpu_baseline:
            print("[bench] CPU oracle baseline (subspace iteration)", file=sys.stderr, flush=True)
            lr["cpu_baseline"] = lowrank_cpu_baseline(a0, 57)
        line["lowrank"] = lr
        print("[bench] low-rank inside error feedback leg", file=sys.stderr, flush=True)
        line["lowrank_ef"] = bench_lowrank_ef(cfz, torch, dev)
    if not args.no_cpu_baseline:
        print("[bench] CPU oracle baseline", file=sys.stderr, flush=True)
        sample_tensors = 114  # every tensor of a step; four steps, about 13 s on one core
        xs_host = []
        for s in range(min(5, X.shape[0])):
            xh = X[s, :sample_tensors].contiguous().view(torch.int16).cpu().numpy().view(np.uint16)
            xs_host.append([xh[i] for i in range(sample_tensors)])
        line["cpu_baseline"] = cpu_baseline(xs_host, bits, group)
    else:
        line["cpu_baseline"] = None
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
