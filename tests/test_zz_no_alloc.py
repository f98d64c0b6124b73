"""cfz_lowrank_noalloc: the subspace iteration on the library's built-in device
scratch instead of a caller workspace.  Two calls in a row through the C ABI --
the 57 x 1024 x 3072 batch, then a smaller ragged one that finds the first
call's data still in the scratch -- each bit-identical to cfz_lowrank on a
caller workspace filled with 0xff bytes beforehand (so neither path may depend
on what the workspace held), and the small one within 1e-3 of the oracle."""
import sys

import numpy as np
import pytest
import torch

import oracle
from synth import gaussian_q0, lowrank_batch

pytestmark = pytest.mark.gpu

if torch.cuda.is_available():
    from diffusion_activation_residual_amd import cfz
DEV = "cuda:0"


def say(*a):
    print(*a, file=sys.stderr, flush=True)


@pytest.fixture(autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def _both(batch, m, n, r, T, seed):
    A = lowrank_batch(batch, m, n, rank=16, sigma=0.05, seed=seed, device=DEV)
    Q0 = gaussian_q0(batch, n, r, seed=seed + 1, device=DEV)
    out = {}
    for kind in ("workspace", "noalloc"):
        U = torch.full((batch, m, r), float("nan"), device=DEV)
        V = torch.full((batch, n, r), float("nan"), device=DEV)
        RU = torch.full((batch, r, r), float("nan"), device=DEV)
        if kind == "workspace":
            ws = torch.full((cfz.cfz_lowrank_workspace_bytes(batch, m, n, r),), 255,
                            dtype=torch.uint8, device=DEV)
            cfz.cfz_lowrank(batch, m, n, r, T, A, Q0, U, V, RU, ws)
        else:
            cfz.cfz_lowrank_noalloc(batch, m, n, r, T, A, Q0, U, V, RU)
        torch.cuda.synchronize()
        out[kind] = (U, V, RU)
    return A, Q0, out


def test_noalloc_two_calls_match_workspace_entry_point():
    assert cfz.cfz_lowrank_noalloc_max_bytes() == 64 << 20
    cases = [(57, 1024, 3072, 16, 2, 11), (3, 300, 520, 5, 1, 12)]
    for batch, m, n, r, T, seed in cases:
        say(f"[gpu] noalloc batch={batch} m={m} n={n} r={r} T={T}")
        assert cfz.cfz_lowrank_workspace_bytes(batch, m, n, r) <= cfz.cfz_lowrank_noalloc_max_bytes()
        A, Q0, out = _both(batch, m, n, r, T, seed)
        for name, a, b in zip(("U", "V", "RU"), out["workspace"], out["noalloc"]):
            assert torch.isfinite(b).all(), f"{name}: not written"
            assert torch.equal(a.view(torch.int32), b.view(torch.int32)), f"{name} differs"
    # the second (small) call against the fp64 oracle, every matrix
    U, V, RU = out["noalloc"]
    for b in range(batch):
        a16 = A[b].contiguous().view(torch.int16).cpu().numpy().view(np.uint16).reshape(m, n)
        ou, ov, oru = oracle.lowrank(a16, Q0[b].cpu().numpy(), T)
        rec = (U[b].double() @ RU[b].double() @ V[b].double().T).cpu().numpy()
        orec = ou @ oru @ ov.T
        rel = np.linalg.norm(rec - orec) / np.linalg.norm(orec)
        assert rel <= 1e-3, f"matrix {b}: reconstruction {rel:.2e} from the oracle"
