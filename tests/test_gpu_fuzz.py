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
