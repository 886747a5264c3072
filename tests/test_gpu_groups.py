"""GPU checks of the grouped step (dion3_step_groups): several shape groups
in one call, where groups with equal Gram sides share the launches of their
s x s products.  Each matrix's arithmetic is the same as in a megabatched
call of its own group, so the results must equal per-group calls bit for
bit; one matrix per group is also checked against the fp64 oracle."""
import sys

import numpy as np
import pytest

from tests.parity import check_step
from workloads import host_gaussian

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"
MU = 0.95


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def make(specs, seed, scale=1.0):
    """Host fp32 (W, M) lists per group from (batch, n, m) specs."""
    out = []
    for gi, (b, n, m) in enumerate(specs):
        Ws = [host_gaussian((n, m), [seed, gi, j, 1], std=0.02) for j in range(b)]
        Ms = [host_gaussian((n, m), [seed, gi, j, 2]) * np.float32(scale * (1 + j % 3))
              for j in range(b)]
        out.append((Ws, Ms))
    return out


def to_dev(arrs):
    return [torch.from_numpy(a).to(DEV) for a in arrs]


def run_grouped(host, ks, lr, cfg, grads=None, norm=None):
    groups, tensors = [], []
    for gi, ((Ws, Ms), k) in enumerate(zip(host, ks)):
        Wd, Md = to_dev(Ws), to_dev(Ms)
        Gd = to_dev(grads[gi]) if grads is not None else None
        Vd = [torch.zeros(Ms[0].shape[0], dtype=torch.float32, device=DEV) for _ in Ms] if norm \
            else None
        groups.append(d3.Group(Wd, Md, k, lr, Gs=Gd, Vs=Vd))
        tensors.append((Wd, Md, Vd))
    outs = d3.step_groups(groups, MU, cfg, norm=norm, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    return tensors, outs


def run_per_group(host, ks, lr, cfg, grads=None, norm=None):
    tensors, outs = [], []
    for gi, ((Ws, Ms), k) in enumerate(zip(host, ks)):
        Wd, Md = to_dev(Ws), to_dev(Ms)
        Gd = to_dev(grads[gi]) if grads is not None else None
        Vd = [torch.zeros(Ms[0].shape[0], dtype=torch.float32, device=DEV) for _ in Ms] if norm \
            else None
        nrm = (Vd, norm[0], norm[1]) if norm else None
        outs.append(d3.step_megabatch(Wd, Md, k, lr, MU, cfg, return_idx=True, return_O=True,
                                      Gs=Gd, norm=nrm))
        tensors.append((Wd, Md, Vd))
    torch.cuda.synchronize()
    return tensors, outs


def assert_bitwise(ta, oa, tb, ob):
    for (Wa, Ma, Va), (Wb, Mb, Vb), (ia, Oa), (ib, Ob) in zip(ta, tb, oa, ob):
        assert torch.equal(ia, ib)
        assert Oa.cpu().numpy().tobytes() == Ob.cpu().numpy().tobytes()
        for x, y in zip(Wa + Ma + (Va or []), Wb + Mb + (Vb or [])):
            assert x.cpu().numpy().tobytes() == y.cpu().numpy().tobytes()


# (batch, n, m) per group at f = 1/4: groups 0, 2 and 3 share the Gram side
# 256 (group 3 has k > m, so its Gram is X^T X with s = m = 256); group 1 has
# its own (k = 688); group 4's side (k = 32) pads to one 128 tile
MIXED = [(4, 1024, 1536), (3, 2752, 1024), (2, 1024, 2752), (3, 1200, 256), (5, 128, 512)]
KS_MIXED = [256, 688, 256, 300, 32]


@pytest.mark.parametrize("path", [d3.PATH_AUTO, d3.PATH_TILED])
def test_groups_equal_per_group_calls_bitwise(path):
    say("groups vs per-group calls, path", path)
    host = make(MIXED, 71)
    cfg = d3.ns_cfg(path=path)
    ta, oa = run_grouped(host, KS_MIXED, 0.04, cfg)
    tb, ob = run_per_group(host, KS_MIXED, 0.04, cfg)
    assert_bitwise(ta, oa, tb, ob)


def test_groups_against_oracle():
    say("groups vs oracle")
    host = make(MIXED, 72, scale=0.5)
    cfg = d3.default_cfg()
    ta, oa = run_grouped(host, KS_MIXED, 0.04, cfg)
    for gi, ((Ws, Ms), k) in enumerate(zip(host, KS_MIXED)):
        Wd, Md, _ = ta[gi]
        idx, O = oa[gi]
        j = len(Ws) - 1
        check_step(Ws[j], Ms[j], Wd[j].cpu().numpy(), Md[j].cpu().numpy(), idx[j].cpu().numpy(),
                   O[j].cpu().numpy(), k, 0.04, MU)


def test_groups_standard_method_bitwise():
    say("groups, standard NS")
    host = make(MIXED[:3], 73)
    cfg = d3.ns_cfg(method=d3.NS_STANDARD)
    ta, oa = run_grouped(host, KS_MIXED[:3], 0.04, cfg)
    tb, ob = run_per_group(host, KS_MIXED[:3], 0.04, cfg)
    assert_bitwise(ta, oa, tb, ob)


@pytest.mark.parametrize("restarts", [(), (2, 4), (3,)])
def test_groups_accumulate_and_normalize_bitwise(restarts):
    say("groups with gradients and normalization, restarts", restarts)
    host = make(MIXED, 74)
    grads = [[host_gaussian(Ms[0].shape, [75, gi, j]) * np.float32(0.1) for j in range(len(Ms))]
             for gi, (_, Ms) in enumerate(host)]
    cfg = d3.ns_cfg(restart_at=restarts)
    for norm in (None, (0.9, 1e-8)):
        ta, oa = run_grouped(host, KS_MIXED, 0.04, cfg, grads=grads, norm=norm)
        tb, ob = run_per_group(host, KS_MIXED, 0.04, cfg, grads=grads, norm=norm)
        assert_bitwise(ta, oa, tb, ob)


def test_many_groups_one_call():
    """DION3_MAX_GROUPS groups of seeded random shapes (several sharing each
    Gram side) in one call, bitwise against per-group calls."""
    rng = np.random.default_rng(76)
    specs, ks = [], []
    for _ in range(d3.MAX_GROUPS):
        n = int(rng.choice([64, 200, 256, 384, 520]))
        m = int(rng.choice([96, 256, 300, 640]))
        specs.append((int(rng.integers(1, 4)), n, m))
        ks.append(int(rng.choice([n // 4, n // 2, n])) or 1)
    say("max groups", specs[:4], "...")
    host = make(specs, 77)
    cfg = d3.default_cfg()
    ta, oa = run_grouped(host, ks, 0.02, cfg)
    tb, ob = run_per_group(host, ks, 0.02, cfg)
    assert_bitwise(ta, oa, tb, ob)


def test_groups_trace_shares_the_side_products():
    """Groups 0 and 2 share a Gram side, and the two side sets run their
    schedule in step: every polynomial and symmetric product is one launch
    over both sets, and every Gram one launch over the three groups."""
    say("groups trace")
    host = make(MIXED[:3], 78)
    cfg = d3.ns_cfg(path=d3.PATH_TILED)
    run_grouped(host, KS_MIXED[:3], 0.04, cfg)          # warm
    d3.trace_enable(512)
    try:
        run_grouped(host, KS_MIXED[:3], 0.04, cfg)
        recs = d3.trace_records()
    finally:
        d3.trace_disable()
    names = [r[0] for r in recs]
    assert sum(n.startswith("gemm_poly") for n in names) == 5
    assert sum(n.startswith("gemm_symm") for n in names) == 8   # iteration 4: Z Q and Z R together
    assert sum(n.startswith("gemm_gram") for n in names) == 2
    assert sum(n.startswith("gemm_back") for n in names) == 3


def test_groups_trace_times_every_kernel_within_the_call():
    """The trace times each kernel from the previous kernel's end inside one
    call, and restarts after the untimed copies of idx and O (here between
    the groups' normalization passes): every record is positive, one record
    per launch, and together they fit in the call's own time."""
    say("groups trace chain")
    host = make(MIXED[:3], 79)
    cfg = d3.ns_cfg(path=d3.PATH_TILED)
    norm = (0.95, 1e-8)
    run_grouped(host, KS_MIXED[:3], 0.04, cfg, norm=norm)          # warm
    d3.trace_enable(512)
    try:
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        run_grouped(host, KS_MIXED[:3], 0.04, cfg, norm=norm)
        e1.record()
        torch.cuda.synchronize()
        recs = d3.trace_records()
    finally:
        d3.trace_disable()
    names = [r[0] for r in recs]
    # per group: scoring, top-k, gather, the final product, norm stats and update
    for kind in ("row_score", "topk", "norm_stats", "norm_update"):
        assert sum(n == kind for n in names) == 3, kind
    assert sum(n in ("gather", "gather_rows") for n in names) == 3
    assert all(r[1] > 0.0 for r in recs)
    assert sum(r[1] for r in recs) <= e0.elapsed_time(e1) * 1.02


def test_groups_more_side_sets_than_one_launch_holds():
    """Six Gram sides, more than the four products one launch holds: every
    s x s product is split over two launches (four sets, then two), and each
    Gram over two as well; results stay bitwise those of per-group calls."""
    say("six side sets")
    specs = [(2, 700, 160), (2, 600, 200), (2, 520, 256), (1, 900, 300), (2, 384, 420), (1, 1000, 520)]
    ks = [350, 300, 260, 450, 384, 1000]    # Gram sides 160, 200, 256, 300, 384, 520
    host = make(specs, 80)
    cfg = d3.ns_cfg(path=d3.PATH_TILED)
    ta, oa = run_grouped(host, ks, 0.03, cfg)
    tb, ob = run_per_group(host, ks, 0.03, cfg)
    assert_bitwise(ta, oa, tb, ob)
    d3.trace_enable(1024)
    try:
        run_grouped(host, ks, 0.03, cfg)
        recs = d3.trace_records()
    finally:
        d3.trace_disable()
    names = [r[0] for r in recs]
    assert sum(n.startswith("gemm_poly") for n in names) == 2 * 5
    # two launches per product, but iteration 4's Z Q and Z R together (12
    # products) take three
    assert sum(n.startswith("gemm_symm") for n in names) == 2 * 9 - 1
    assert sum(n.startswith("gemm_gram") for n in names) == 2 * 2
    assert sum(n.startswith("gemm_back") for n in names) == 6


@pytest.mark.parametrize("path,norm,acc", [(d3.PATH_AUTO, None, False), (d3.PATH_TILED, None, False),
                                           (d3.PATH_AUTO, (0.95, 1e-8), False),
                                           (d3.PATH_AUTO, None, True)])
def test_grouped_step_graph_capture(path, norm, acc):
    """The grouped call (shared side-set launches, several products per
    launch, the fused small group on the automatic path) captured in a HIP
    graph: every replay equals an eager grouped step bit for bit, with eager
    work and synchronizations between replays."""
    say("grouped step graph capture, path", path, "norm", norm, "accumulate", acc)
    host = make(MIXED, 73)
    cfg = d3.ns_cfg(path=path)

    def build():
        groups, tensors = [], []
        for (Ws, Ms), k in zip(host, KS_MIXED):
            Wd, Md = to_dev(Ws), to_dev(Ms)
            Vd = [torch.zeros(Ms[0].shape[0], dtype=torch.float32, device=DEV) for _ in Ms] \
                if norm else None
            Gd = [g * 0.1 for g in to_dev(Ms)] if acc else None    # fixed gradients
            groups.append(d3.Group(Wd, Md, k, 0.04, Gs=Gd, Vs=Vd))
            tensors += Wd + Md + (Vd or [])
        return groups, tensors

    (ge, te), (gg, tg) = build(), build()
    ws_e, ws_g = d3.Workspace(), d3.Workspace()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):           # sizes the workspace outside the capture
        d3.step_groups(gg, MU, cfg, norm=norm, ws=ws_g)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    d3.step_groups(ge, MU, cfg, norm=norm, ws=ws_e)    # the eager copy takes the same first step
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        d3.step_groups(gg, MU, cfg, norm=norm, ws=ws_g)
    for rep in range(3):
        graph.replay()
        d3.step_groups(ge, MU, cfg, norm=norm, ws=ws_e)
        junk = torch.randn(1000, device=DEV).sum()      # eager work between replays
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for j, (a, b) in enumerate(zip(te, tg)):
            assert a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes(), (rep, j)
