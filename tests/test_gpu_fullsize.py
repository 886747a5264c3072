"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: one megabatched call over a whole shape group of the 1B,
7B (f = 1/4 and f = 1/2) and 14B ill-conditioned weight sets.  The oracle
checks the first and the last matrix of the group (the oracle runs one fp64
matrix at a time)."""
import sys

import numpy as np
import pytest

from tests.parity import check_step
from workloads import MU, WORKLOADS, device_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"

CASES = [("c3", 0), ("c3", 1), ("c3", 2), ("c4", 0), ("c4", 1), ("c4", 2), ("c4h", 1),
         ("c5", 0), ("c5", 1), ("c5", 2)]


@pytest.mark.parametrize("wl_name,group", CASES)
def test_fullsize_group(wl_name, group):
    wl = WORKLOADS[wl_name]
    g = wl.groups[group]
    print(f"[case] {wl.name} group {group}: {g.count} x {g.n}x{g.m}", flush=True)
    sys.stdout.flush()
    (_, Ws, Ms), = device_workload(wl, DEV, groups=[group])
    picks = sorted({0, g.count - 1})
    W0 = {j: Ws[j].cpu().numpy() for j in picks}
    M0 = {j: Ms[j].cpu().numpy() for j in picks}
    k = d3.k_from_fraction(float(wl.fraction), g.n)
    idx, O = d3.step_megabatch(Ws, Ms, k, wl.lr, MU, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    for j in picks:
        err = check_step(W0[j], M0[j], Ws[j].cpu().numpy(), Ms[j].cpu().numpy(),
                         idx[j].cpu().numpy(), O[j].cpu().numpy(), k, wl.lr, MU)
        print(f"{wl.name} group {group} matrix {j}: k={k}, O rel err {err:.3e}", flush=True)
    del Ws, Ms, idx, O
    torch.cuda.empty_cache()
