"""Seeded random shapes through the megabatch entry point: ragged n, m, k,
k > m (the transposed Gram), one row or one column, small batches; both
the fused and the tiled Gram iteration (the automatic choice).  Every matrix
is checked against the fp64 oracle with the acceptance rules of the step."""
import sys

import numpy as np
import pytest

from tests.parity import check_step
from workloads import host_gaussian

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"


def _cases(count=40, seed=2026):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        n = int(rng.integers(1, 700))
        m = int(rng.integers(1, 700))
        k = int(rng.integers(1, n + 1))
        B = int(rng.integers(1, 4))
        out.append((i, n, m, k, B))
    return out


@pytest.mark.parametrize("i,n,m,k,B", _cases())
def test_random_shape_step(i, n, m, k, B):
    print(f"[case] fuzz {i}: {B} x {n}x{m}, k={k}", flush=True)
    sys.stdout.flush()
    Ws = [host_gaussian((n, m), [70, i, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [71, i, b]) for b in range(B)]
    Wd = [torch.from_numpy(w).to(DEV) for w in Ws]
    Md = [torch.from_numpy(x).to(DEV) for x in Ms]
    idx, O = d3.step_megabatch(Wd, Md, k, 0.04, 0.95, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    for b in range(B):
        check_step(Ws[b], Ms[b], Wd[b].cpu().numpy(), Md[b].cpu().numpy(), idx[b].cpu().numpy(),
                   O[b].cpu().numpy(), k, 0.04, 0.95)


def _small_cases(count=24, seed=2027):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(count):
        n = int(rng.integers(1, 300))
        m = int(rng.integers(1, 2000))
        side = int(rng.integers(1, 65))
        k = min(n, side) if rng.random() < 0.5 else n   # k <= 64, or k = n (then m may be the side)
        if k > 64 and m > 64:
            m = int(rng.integers(1, 65))
        B = int(rng.integers(1, 5))
        out.append((i, n, m, k, B))
    return out


@pytest.mark.parametrize("i,n,m,k,B", _small_cases())
def test_random_small_side_fused_equals_tiled(i, n, m, k, B):
    """Random shapes with a Gram side of at most 64 (the one-wave fused
    kernel and, for n <= 256, the one-thread-per-row top-k): the fused and
    the tiled Gram iteration must give the same bits, and the first matrix
    must pass the step's acceptance rules against the fp64 oracle."""
    print(f"[case] small fuzz {i}: {B} x {n}x{m}, k={k}", flush=True)
    sys.stdout.flush()
    Ws = [host_gaussian((n, m), [72, i, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [73, i, b]) for b in range(B)]
    outs = []
    for path in (d3.PATH_FUSED, d3.PATH_TILED):
        Wd = [torch.from_numpy(w).to(DEV) for w in Ws]
        Md = [torch.from_numpy(x).to(DEV) for x in Ms]
        idx, O = d3.step_megabatch(Wd, Md, k, 0.04, 0.95, d3.ns_cfg(path=path), return_idx=True,
                                   return_O=True)
        torch.cuda.synchronize()
        outs.append(([w.cpu().numpy() for w in Wd], [x.cpu().numpy() for x in Md],
                     idx.cpu().numpy(), O.cpu().numpy()))
    (Wf, Mf, If, Of), (Wt, Mt, It, Ot) = outs
    assert If.tobytes() == It.tobytes() and Of.tobytes() == Ot.tobytes()
    for b in range(B):
        assert Wf[b].tobytes() == Wt[b].tobytes() and Mf[b].tobytes() == Mt[b].tobytes(), b
    check_step(Ws[0], Ms[0], Wf[0], Mf[0], If[0], Of[0], k, 0.04, 0.95)
