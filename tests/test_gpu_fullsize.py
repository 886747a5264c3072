"""GPU parity at the workloads' full sizes, in the launch configuration the
benchmark times: one megabatched call over a whole shape group of the 1B,
7B (f = 1/4 and f = 1/2) and 14B ill-conditioned weight sets.  The oracle
runs one fp64 matrix at a time, so it checks a sample of each group: its
first and last matrix ("ends") and two more drawn with a seeded generator
("random"), each pair in a test of its own."""
import sys

import numpy as np
import pytest

from oracle import dion3_oracle as orc
from tests.parity import check_step, rel
from workloads import MU, WORKLOADS, device_workload

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"

GROUPS = [("c3", 0), ("c3", 1), ("c3", 2), ("c4", 0), ("c4", 1), ("c4", 2),
          ("c4h", 0), ("c4h", 1), ("c4h", 2), ("c5", 0), ("c5", 1), ("c5", 2)]
CASES = [(w, g, s) for (w, g) in GROUPS for s in ("ends", "random")]


def sample(wl, group, which):
    """Matrix indices of a group checked by the oracle: the first and last, or
    two others drawn from a generator seeded by the workload and group."""
    count = wl.groups[group].count
    if which == "ends":
        return sorted({0, count - 1})
    inner = np.arange(1, count - 1)
    rng = np.random.default_rng([wl.seed_base, group, 2])
    return sorted(int(j) for j in rng.choice(inner, size=min(2, len(inner)), replace=False))


@pytest.mark.parametrize("wl_name,group,which", CASES)
def test_fullsize_group(wl_name, group, which):
    wl = WORKLOADS[wl_name]
    g = wl.groups[group]
    picks = sample(wl, group, which)
    print(f"[case] {wl.name} group {group}: {g.count} x {g.n}x{g.m}, matrices {picks}", flush=True)
    sys.stdout.flush()
    (_, Ws, Ms), = device_workload(wl, DEV, groups=[group])
    W0 = {j: Ws[j].cpu().numpy() for j in picks}
    M0 = {j: Ms[j].cpu().numpy() for j in picks}
    k = d3.k_from_fraction(float(wl.fraction), g.n)
    idx, O = d3.step_megabatch(Ws, Ms, k, wl.lr, MU, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    for j in picks:
        S, Oj = idx[j].cpu().numpy(), O[j].cpu().numpy()
        err = check_step(W0[j], M0[j], Ws[j].cpu().numpy(), Ms[j].cpu().numpy(), S, Oj, k,
                         wl.lr, MU)
        # the kernel's own share of the error: the oracle on the fp16 X the
        # gather writes (fp32 rows times fp32(1 / (||X|| + eps)), rounded)
        Xs = M0[j][S]
        scale = 1.0 / (np.sqrt(np.sum(Xs.astype(np.float64) ** 2)) + 1e-7)
        X16 = (Xs * np.float32(scale)).astype(np.float16).astype(np.float64)
        e16 = rel(Oj, orc.ns_gram(X16, orc.default_coeffs(), (3,)))
        print(f"{wl.name} group {group} matrix {j}: k={k}, O rel err {err:.3e} against the "
              f"fp64 oracle, {e16:.3e} against the oracle on the fp16-rounded input", flush=True)
    del Ws, Ms, idx, O
    torch.cuda.empty_cache()
