"""GPU parity of the HIP path (called through the C ABI) against the fp64
oracle, on seeded inputs spanning several tiles, ragged tails and the
degenerate cases of the method."""
import math
import sys

import numpy as np
import pytest

from oracle import dion3_oracle as orc
from tests.parity import O_TOL, check_selection, check_step, rel
from workloads import c1_inputs, c2_inputs, host_gaussian, host_lowrank, host_tied

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_step(W, M, k, lr, mu, cfg=None):
    Wd, Md = dev(W), dev(M)
    idx, O = d3.step(Wd, Md, k, lr, mu, cfg, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    return Wd.cpu().numpy(), Md.cpu().numpy(), idx.cpu().numpy(), O.cpu().numpy()


# ------------------------------------------------------------ selection

SELECT_CASES = [
    ("gauss", 128, 512, 32), ("gauss", 1000, 77, 250), ("gauss", 1, 5, 1), ("gauss", 300, 300, 300),
    ("gauss", 13824, 8, 1728), ("tied", 37, 11, 5), ("tied", 4096, 64, 1024), ("tied", 999, 3, 998),
    ("gauss", 2049, 130, 2048), ("tied", 256, 9, 100), ("tied", 200, 5, 199), ("gauss", 255, 33, 64),
    ("tied", 257, 9, 100),
]


@pytest.mark.parametrize("kind,n,m,k", SELECT_CASES)
def test_row_select_exact(kind, n, m, k):
    say("row_select", kind, n, m, k)
    M = host_gaussian((n, m), [1, n, m]) if kind == "gauss" else host_tied(n, m, n, n_distinct=7)
    idx, scores = d3.row_select(dev(M), k, return_scores=True)
    torch.cuda.synchronize()
    l1, _ = orc.row_scores(M)
    assert rel(scores.cpu().numpy(), l1) <= 1e-12
    S = idx.cpu().numpy()
    if kind == "tied":        # exact ties: the lowest-index rule decides, no band
        assert np.array_equal(S, orc.select_rows(l1, k))
    else:
        check_selection(S, M, k)


def test_row_select_batched():
    say("row_select batched")
    M = np.stack([host_tied(500, 40, b, 9) for b in range(3)])
    idx = d3.row_select(dev(M), 123).cpu().numpy()
    for b in range(3):
        l1, _ = orc.row_scores(M[b])
        assert np.array_equal(idx[b], orc.select_rows(l1, 123))


@pytest.mark.parametrize("n,m,k", [(200, 96, 50), (256, 130, 256), (37, 300, 5), (129, 64, 128)])
def test_small_topk_matches_radix_topk_bitwise(n, m, k):
    """Matrices of at most 256 rows take the one-thread-per-row top-k.  With
    zero momentum rows appended (300 rows in all: the radix top-k; zero rows
    score 0 and are never taken) the step must give the same selection, the
    same Frobenius scale and so the same outputs, bit for bit."""
    say("small top-k", n, m, k)
    W = host_gaussian((n, m), [60, n, m], std=0.02)
    M = host_gaussian((n, m), [61, n, m])
    pad = 300 - n
    Wp = np.vstack([W, host_gaussian((pad, m), [62, n, m], std=0.02)])
    Mp = np.vstack([M, np.zeros((pad, m), np.float32)])
    W1, M1, S1, O1 = run_step(W, M, k, 0.04, 0.95)
    W2, M2, S2, O2 = run_step(Wp, Mp, k, 0.04, 0.95)
    assert np.array_equal(S1, S2)
    assert O1.tobytes() == O2.tobytes()
    assert W1.tobytes() == W2[:n].tobytes() and M1.tobytes() == M2[:n].tobytes()
    assert W2[n:].tobytes() == Wp[n:].tobytes() and M2[n:].tobytes() == Mp[n:].tobytes()


# ------------------------------------------------------------ symmetric kernels

@pytest.mark.parametrize("B,rows,cols", [(1, 128, 128), (3, 256, 384), (2, 384, 1024)])
def test_syrk_f16(B, rows, cols):
    say("syrk", B, rows, cols)
    A = (host_gaussian((B, rows, cols), [2, rows, cols]) * 0.05).astype(np.float16)
    R = d3.syrk_f16(dev(A)).cpu().numpy()
    for b in range(B):
        ref = A[b].astype(np.float64) @ A[b].astype(np.float64).T
        assert rel(R[b], ref) <= 2e-3
        assert np.array_equal(R[b], R[b].T)


@pytest.mark.parametrize("s", [128, 384])
def test_symm_f16_poly(s):
    say("symm poly", s)
    G = host_gaussian((s, s), [3, s]).astype(np.float64)
    A64 = G @ G.T
    A64 /= np.linalg.norm(A64, 2)                      # symmetric, spectrum in [0, 1]
    A = A64.astype(np.float16)
    a, b, c = 3.4445, -4.7750, 2.0315
    C = d3.symm_f16(dev(A), dev(A), dev(A), alpha=c, beta=b, gamma=a).cpu().numpy()
    Af = A.astype(np.float64)
    ref = c * Af @ Af + b * Af + a * np.eye(s)
    assert rel(C, ref) <= 2e-3
    assert np.array_equal(C, C.T)
    # plain product of two commuting symmetric matrices
    B2 = (Af @ Af).astype(np.float16)
    P = d3.symm_f16(dev(A), dev(B2)).cpu().numpy()
    assert rel(P, Af @ B2.astype(np.float64)) <= 2e-3
    assert np.array_equal(P, P.T)


# ------------------------------------------------------------ Gram Newton-Schulz

GRAM_CASES = [(1, 32, 512), (2, 100, 300), (1, 300, 100), (1, 1, 1), (1, 1, 7), (1, 7, 1),
              (2, 128, 128), (1, 257, 1000), (1, 1000, 257), (4, 64, 4096)]


@pytest.mark.parametrize("B,k,m", GRAM_CASES)
def test_gram_ns(B, k, m):
    say("gram_ns", B, k, m)
    X = host_gaussian((B, k, m), [4, k, m]).astype(np.float16)
    O = d3.gram_ns(dev(X)).cpu().numpy()
    co = orc.default_coeffs()
    for b in range(B):
        ref = orc.ns_gram(X[b].astype(np.float64), co, (3,))
        assert rel(O[b], ref) <= O_TOL, (b, rel(O[b], ref))


@pytest.mark.parametrize("iters,restarts", [(5, ()), (5, (2, 4)), (3, (2,)), (7, (3, 6)), (1, ())])
def test_gram_ns_schedules(iters, restarts):
    say("gram_ns schedule", iters, restarts)
    X = host_gaussian((2, 96, 333), [5, iters]).astype(np.float16)
    co = [orc.MUON_COEFFS] * iters
    cfg = d3.ns_cfg(iters=iters, restart_at=restarts, coeffs=co)
    O = d3.gram_ns(dev(X), cfg).cpu().numpy()
    for b in range(2):
        ref = orc.ns_gram(X[b].astype(np.float64), co, restarts)
        assert rel(O[b], ref) <= O_TOL


# A coefficient table that changes from iteration to iteration (Muon's
# quintic, the convergent (15/8, -10/8, 3/8) one, a third), on inputs and a
# schedule for which the result depends strongly on which set each iteration
# uses: the table reversed gives an oracle result far outside the tolerance,
# so reading a set at the wrong iteration would fail.
VARIED = [orc.MUON_COEFFS, (15 / 8, -10 / 8, 3 / 8), (3.0, -3.2, 1.2)]


@pytest.mark.parametrize("method,path", [(d3.NS_GRAM, d3.PATH_TILED), (d3.NS_GRAM, d3.PATH_FUSED),
                                         (d3.NS_STANDARD, d3.PATH_AUTO)])
@pytest.mark.parametrize("k,m", [(96, 333), (24, 256), (300, 100)])
def test_per_iteration_coefficients(method, path, k, m):
    say("per-iteration coefficients", method, path, k, m)
    # ill-conditioned rows (singular values spread as i^-1.5), far from the
    # quintic's fixed point after three iterations
    X = np.stack([host_lowrank(k, m, 53 + b) for b in range(2)]).astype(np.float16)
    restarts = (2,) if method == d3.NS_GRAM else ()
    cfg = d3.ns_cfg(iters=3, restart_at=restarts, coeffs=VARIED, method=method, path=path)
    O = d3.gram_ns(dev(X), cfg).cpu().numpy()
    for b in range(2):
        Xb = X[b].astype(np.float64)
        if method == d3.NS_GRAM:
            ref, rev = orc.ns_gram(Xb, VARIED, restarts), orc.ns_gram(Xb, VARIED[::-1], restarts)
        else:
            ref, rev = orc.ns_standard(Xb, VARIED), orc.ns_standard(Xb, VARIED[::-1])
        assert rel(rev, ref) > 5 * O_TOL      # the test can tell the tables apart
        err = rel(O[b], ref)
        print(f"{k}x{m} matrix {b}: O rel err {err:.3e} (reversed table {rel(rev, ref):.3e})",
              flush=True)
        assert err <= O_TOL, (b, err)


@pytest.mark.parametrize("B,k,m", [(2, 100, 300), (1, 300, 100), (1, 257, 1000), (3, 64, 64)])
def test_standard_ns(B, k, m):
    """The standard iteration on X (the Muon baseline) on the same kernels."""
    say("standard ns", B, k, m)
    X = host_gaussian((B, k, m), [22, k, m]).astype(np.float16)
    O = d3.gram_ns(dev(X), d3.ns_cfg(method=d3.NS_STANDARD)).cpu().numpy()
    co = orc.default_coeffs()
    for b in range(B):
        ref = orc.ns_standard(X[b].astype(np.float64), co)
        assert rel(O[b], ref) <= O_TOL, (b, rel(O[b], ref))


@pytest.mark.parametrize("n,m,k", [(256, 512, 256), (400, 160, 400), (300, 200, 75)])
def test_step_standard_method(n, m, k):
    say("step standard", n, m, k)
    W = host_gaussian((n, m), [23, n], std=0.02)
    M = host_gaussian((n, m), [24, n])
    W1, M1, S, O = run_step(W, M, k, 0.02, 0.95, d3.ns_cfg(method=d3.NS_STANDARD))
    ref = orc.dion3_step(W, M, k, 0.02, 0.95, method="standard")
    assert np.array_equal(S, ref["S"])
    assert rel(O, ref["O"]) <= O_TOL
    mask = np.zeros(n, bool)
    mask[S] = True
    assert W1[~mask].tobytes() == W[~mask].tobytes() and M1[~mask].tobytes() == M[~mask].tobytes()
    assert M1[mask].tobytes() == ref["M"][mask].tobytes()


def test_default_workspaces_are_per_stream():
    """Calls on two streams without an explicit workspace must not share
    scratch memory: results equal the sequential ones bit for bit."""
    say("default workspace per stream")
    X1 = dev(host_gaussian((3, 200, 700), 60).astype(np.float16))
    X2 = dev(host_gaussian((3, 200, 700), 61).astype(np.float16))
    ref1, ref2 = d3.gram_ns(X1).cpu().numpy(), d3.gram_ns(X2).cpu().numpy()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    torch.cuda.synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            o1 = d3.gram_ns(X1)
        with torch.cuda.stream(s2):
            o2 = d3.gram_ns(X2)
        outs.append((o1, o2))
    torch.cuda.synchronize()
    for o1, o2 in outs:
        assert o1.cpu().numpy().tobytes() == ref1.tobytes()
        assert o2.cpu().numpy().tobytes() == ref2.tobytes()


def test_gram_ns_deterministic():
    say("gram_ns twice")
    X = dev(host_gaussian((3, 200, 700), 6).astype(np.float16))
    a = d3.gram_ns(X).cpu().numpy()
    b = d3.gram_ns(X).cpu().numpy()
    assert a.tobytes() == b.tobytes()


def test_restart_diagnostic_lowrank():
    """Ill-conditioned input (rank 64, singular values i^-1.5, 1e-3 noise):
    without the restart the fp16 Gram iteration drifts (spurious negative
    eigenvalues grow); with it the error against the oracle on the same fp16
    bytes must meet the tolerance."""
    say("restart diagnostic")
    M = host_lowrank(640, 2048, 11)
    Xn = (M.astype(np.float64) / np.linalg.norm(M.astype(np.float64))).astype(np.float16)
    co = orc.default_coeffs()
    ref = orc.ns_gram(Xn.astype(np.float64), co, (3,))
    ref_exact = orc.ns_gram(M.astype(np.float64), co, (3,))
    with_r = d3.gram_ns(dev(Xn)).cpu().numpy()
    no_r = d3.gram_ns(dev(Xn), d3.ns_cfg(iters=5, restart_at=())).cpu().numpy()
    e1, e0 = rel(with_r, ref), rel(no_r, ref)
    print(f"lowrank 640x2048: kernel rel err with restart {e1:.3e}, without {e0:.3e}; "
          f"fp16 input rounding alone {rel(ref, ref_exact):.3e}", flush=True)
    assert e1 <= O_TOL
    assert e0 > 5 * e1


# ------------------------------------------------------------ the step

def test_step_single_128x512():
    say("step 128x512 k=32")
    W, M = c1_inputs()
    k, lr, mu = 32, 0.02 / math.sqrt(0.25), 0.95
    assert d3.k_from_fraction(0.25, 128) == k
    W1, M1, S, O = run_step(W, M, k, lr, mu)
    err = check_step(W, M, W1, M1, S, O, k, lr, mu)
    print(f"128x512 k=32: O rel err {err:.3e}", flush=True)


STEP_CASES = [(256, 64, 100), (300, 200, 75), (64, 64, 64), (1, 16, 1), (17, 1, 5), (2048, 512, 1),
              (130, 130, 129), (700, 1300, 350), (1500, 260, 1100)]


@pytest.mark.parametrize("n,m,k", STEP_CASES)
def test_step_shapes(n, m, k):
    say("step", n, m, k)
    W = host_gaussian((n, m), [7, n, m], std=0.02)
    M = host_gaussian((n, m), [8, n, m])
    W1, M1, S, O = run_step(W, M, k, 0.04, 0.95)
    check_step(W, M, W1, M1, S, O, k, 0.04, 0.95)


def test_step_ties_take_lowest_index():
    say("step ties")
    M = host_tied(200, 48, 3, n_distinct=4)
    W = host_gaussian((200, 48), 9, std=0.02)
    W1, M1, S, O = run_step(W, M, 50, 0.04, 0.95)
    l1, _ = orc.row_scores(M)
    assert np.array_equal(S, orc.select_rows(l1, 50))
    check_step(W, M, W1, M1, S, O, 50, 0.04, 0.95)


def test_step_strided_rows():
    """Row stride larger than m (a column slice of a wider buffer)."""
    say("step strided")
    n, m, ldm, k = 96, 40, 64, 24
    Wb = dev(host_gaussian((n, ldm), 10, std=0.02))
    Mb = dev(host_gaussian((n, ldm), 11))
    W0, M0 = Wb.cpu().numpy().copy(), Mb.cpu().numpy().copy()
    idx, O = d3.step(Wb[:, :m], Mb[:, :m], k, 0.04, 0.95, return_idx=True, return_O=True)
    W1, M1 = Wb.cpu().numpy(), Mb.cpu().numpy()
    assert W1[:, m:].tobytes() == W0[:, m:].tobytes() and M1[:, m:].tobytes() == M0[:, m:].tobytes()
    check_step(np.ascontiguousarray(W0[:, :m]), np.ascontiguousarray(M0[:, :m]),
               np.ascontiguousarray(W1[:, :m]), np.ascontiguousarray(M1[:, :m]),
               idx.cpu().numpy(), O.cpu().numpy(), k, 0.04, 0.95)


def test_megabatch_equals_single_calls_bitwise():
    say("megabatch vs single")
    B, n, m, k = 5, 200, 300, 50
    Ws = [host_gaussian((n, m), [12, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [13, b]) for b in range(B)]
    Wd, Md = [dev(w) for w in Ws], [dev(x) for x in Ms]
    idx, O = d3.step_megabatch(Wd, Md, k, 0.04, 0.95, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    for b in range(B):
        W1, M1, S, Ob = run_step(Ws[b], Ms[b], k, 0.04, 0.95)
        assert np.array_equal(idx[b].cpu().numpy(), S)
        assert O[b].cpu().numpy().tobytes() == Ob.tobytes()
        assert Wd[b].cpu().numpy().tobytes() == W1.tobytes()
        assert Md[b].cpu().numpy().tobytes() == M1.tobytes()


def test_megabatch_16x1024x4096_f1():
    """16 matrices of 1024x4096, f = 1 (every row, the Muon-equivalent path), one call."""
    say("megabatch 16x1024x4096 f=1")
    Ws, Ms = c2_inputs()
    Wd, Md = [dev(w) for w in Ws], [dev(x) for x in Ms]
    k = d3.k_from_fraction(1.0, 1024)
    idx, O = d3.step_megabatch(Wd, Md, k, 0.02, 0.95, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    for b in (0, 7, 15):
        S = idx[b].cpu().numpy()
        assert np.array_equal(S, np.arange(1024))
        err = check_step(Ws[b], Ms[b], Wd[b].cpu().numpy(), Md[b].cpu().numpy(), S,
                         O[b].cpu().numpy(), k, 0.02, 0.95)
        print(f"16x1024x4096 f=1 matrix {b}: O rel err {err:.3e}", flush=True)


@pytest.mark.parametrize("n,m,k", [(300, 200, 75), (128, 512, 32), (250, 40, 200)])
def test_step_accumulates_gradient(n, m, k):
    """M <- M + G fused into the scoring, then the step on the updated M."""
    say("step accum", n, m, k)
    W = host_gaussian((n, m), [16, n], std=0.02)
    M = host_gaussian((n, m), [17, n])
    G = host_gaussian((n, m), [18, n], std=0.3)
    Wd, Md, Gd = dev(W), dev(M), dev(G)
    idx, O = d3.step(Wd, Md, k, 0.04, 0.95, return_idx=True, return_O=True, G=Gd)
    torch.cuda.synchronize()
    check_step(W, M, Wd.cpu().numpy(), Md.cpu().numpy(), idx.cpu().numpy(), O.cpu().numpy(),
               k, 0.04, 0.95, G=G)
    assert Gd.cpu().numpy().tobytes() == G.tobytes()          # G is read only


def test_megabatch_accum_equals_add_then_step_bitwise():
    say("megabatch accum vs add + step")
    B, n, m, k = 4, 180, 260, 45
    Ws = [host_gaussian((n, m), [19, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [20, b]) for b in range(B)]
    Gs = [host_gaussian((n, m), [21, b], std=0.5) for b in range(B)]
    Wa, Ma, Ga = [dev(w) for w in Ws], [dev(x) for x in Ms], [dev(g) for g in Gs]
    ia, Oa = d3.step_megabatch(Wa, Ma, k, 0.04, 0.95, return_idx=True, return_O=True, Gs=Ga)
    Wb, Mb = [dev(w) for w in Ws], [dev(x + g) for x, g in zip(Ms, Gs)]
    ib, Ob = d3.step_megabatch(Wb, Mb, k, 0.04, 0.95, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    assert ia.cpu().numpy().tobytes() == ib.cpu().numpy().tobytes()
    assert Oa.cpu().numpy().tobytes() == Ob.cpu().numpy().tobytes()
    for b in range(B):
        assert Wa[b].cpu().numpy().tobytes() == Wb[b].cpu().numpy().tobytes()
        assert Ma[b].cpu().numpy().tobytes() == Mb[b].cpu().numpy().tobytes()


# the fused one-launch iteration (automatic path at this Gram side) and the
# tiled products
@pytest.mark.parametrize("path", [d3.PATH_AUTO, d3.PATH_TILED])
def test_graph_capture_replays_match_eager(path):
    """The step's launch sequence (no allocation, no memset) captured in a HIP
    graph: every replay, with eager work and synchronizations in between,
    equals the same number of eager steps bit for bit."""
    say("graph capture", path)
    cfg = d3.ns_cfg(path=path)
    B, n, m, k = 3, 160, 288, 40
    Ws = [host_gaussian((n, m), [25, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [26, b]) for b in range(B)]
    We, Me = [dev(w) for w in Ws], [dev(x) for x in Ms]
    Wg, Mg = [dev(w) for w in Ws], [dev(x) for x in Ms]
    ws_e, ws_g = d3.Workspace(), d3.Workspace()
    pg = (d3.pointer_array(Wg, DEV), d3.pointer_array(Mg, DEV))
    ws_g.get(d3.workspace_size(B, n, m, k), DEV)
    torch.cuda.synchronize()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):          # warm the path outside the capture
        d3.step_megabatch(Wg, Mg, k, 0.04, 0.95, cfg, ws=ws_g, ptrs=pg)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    d3.step_megabatch(We, Me, k, 0.04, 0.95, cfg, ws=ws_e)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        d3.step_megabatch(Wg, Mg, k, 0.04, 0.95, cfg, ws=ws_g, ptrs=pg)
    for rep in range(3):
        graph.replay()
        d3.step_megabatch(We, Me, k, 0.04, 0.95, cfg, ws=ws_e)
        junk = torch.randn(1000, device=DEV).sum()        # eager work between replays
        torch.cuda.synchronize()
        assert float(junk) == float(junk)
        for b in range(B):
            assert Wg[b].cpu().numpy().tobytes() == We[b].cpu().numpy().tobytes(), (rep, b)
            assert Mg[b].cpu().numpy().tobytes() == Me[b].cpu().numpy().tobytes(), (rep, b)


def test_timing_trace_records_every_kernel():
    say("trace")
    W = dev(host_gaussian((300, 500), 27, std=0.02))
    M = dev(host_gaussian((300, 500), 28))
    tiled = d3.ns_cfg(path=d3.PATH_TILED)
    d3.step(W, M, 75, 0.04, 0.95, tiled)          # warm
    torch.cuda.synchronize()
    d3.trace_enable(256)
    try:
        d3.step(W, M, 75, 0.04, 0.95, tiled)
        recs = d3.trace_records()
    finally:
        d3.trace_disable()
    names = [r[0] for r in recs]
    assert names[:3] == ["row_score", "topk", "gather_rows"]   # k <= m: rows layout only
    gemms = [r for r in recs if r[0].startswith("gemm_")]
    # 5 iterations with a restart at 3: 2 Grams, 5 polynomials, 2 multiply-backs
    # and 9 symmetric products (iterations 1-2: R <- Z R Z, Q <- Z Q; iterations
    # 3-5: R <- Z R Z twice, Q <- Z Q twice) in 8 launches: iteration 4's
    # Q <- Z Q and Z R, which both read Z, share one
    assert sum(1 for r in gemms if r[0].startswith("gemm_gram")) == 2
    assert sum(1 for r in gemms if r[0].startswith("gemm_poly")) == 5
    assert sum(1 for r in gemms if r[0].startswith("gemm_symm")) == 8
    # the restart's X <- Q X, then the final multiply-back with the fused update
    assert sum(1 for r in gemms if r[0].startswith("gemm_rect")) == 1
    assert sum(1 for r in gemms if r[0].startswith("gemm_back")) == 1
    assert all(r[1] > 0 for r in recs)
    s_, L_ = 75.0, 500.0
    flops = sum(r[2] for r in gemms)
    assert flops == pytest.approx(6 * s_ * s_ * L_ + 14 * s_ ** 3)
    # algorithmic bytes of the final product: Q and X read, W[S] read and written
    back = [r for r in gemms if r[0].startswith("gemm_back")][0]
    assert back[3] == pytest.approx(2 * s_ * s_ + 10 * s_ * L_)


def test_dion3step_groups_by_shape():
    say("Dion3Step grouping")
    shapes = [(64, 96), (96, 64), (64, 96), (64, 96), (96, 64)]
    Ws = [dev(host_gaussian(s, [14, i], std=0.02)) for i, s in enumerate(shapes)]
    Ms = [dev(host_gaussian(s, [15, i])) for i, s in enumerate(shapes)]
    W0 = [w.cpu().numpy() for w in Ws]
    M0 = [x.cpu().numpy() for x in Ms]
    opt = d3.Dion3Step(Ws, Ms, lr=0.02, fraction=0.25, mu=0.9)
    assert len(opt.groups) == 2
    opt.step()
    torch.cuda.synchronize()
    for i, s in enumerate(shapes):
        k = orc.k_from_fraction(0.25, s[0])
        ref = orc.dion3_step(W0[i], M0[i], k, 0.04, 0.9)
        assert rel(Ws[i].cpu().numpy() - W0[i], ref["W"] - W0[i]) <= O_TOL
        assert Ms[i].cpu().numpy().tobytes() == ref["M"].tobytes()


def test_dion3_optimizer_two_steps():
    """torch.optim-style Dion3: momentum accumulates the gradient (M <- M + G),
    then the step; two steps on two shapes against the oracle."""
    say("Dion3 optimizer")
    shapes = [(96, 64), (64, 96), (96, 64)]
    params = [torch.nn.Parameter(dev(host_gaussian(sh, [80, i], std=0.02)))
              for i, sh in enumerate(shapes)]
    opt = d3.Dion3(params, lr=0.02, fraction=0.25, mu=0.9)
    W = [p.detach().cpu().numpy().copy() for p in params]
    M = [np.zeros(sh, np.float32) for sh in shapes]
    for it in range(2):
        G = [host_gaussian(sh, [81, it, i]) for i, sh in enumerate(shapes)]
        for p, g in zip(params, G):
            p.grad = dev(g)
        opt.step()
        torch.cuda.synchronize()
        for i, (p, sh) in enumerate(zip(params, shapes)):
            k = orc.k_from_fraction(0.25, sh[0])
            ref = orc.dion3_step(W[i], M[i] + G[i], k, 0.04, 0.9)
            W1 = p.detach().cpu().numpy()
            M1 = opt.state[p]["momentum"].cpu().numpy()
            changed = np.nonzero(np.any(W1 != W[i], axis=1))[0]
            assert np.array_equal(changed, ref["S"]), (it, i)
            assert M1.tobytes() == ref["M"].tobytes(), (it, i)
            assert rel(W1 - W[i], ref["W"] - W[i]) <= O_TOL, (it, i)
            W[i], M[i] = W1, M1



# (n, m, ld, k) through the tiled path: the fused update's element path for
# rows that are not 16-byte aligned (odd ld) and ragged last chunks (m % 8),
# its vector path (ld % 4 == 0), with the output rows as the tile's rows
# (k <= m) and as its columns (k > m)
TILED_UPDATE_CASES = [(300, 203, 207, 150), (400, 77, 81, 250), (512, 520, 520, 200),
                      (333, 1000, 1003, 300), (260, 96, 100, 100)]


@pytest.mark.parametrize("n,m,ld,k", TILED_UPDATE_CASES)
def test_tiled_update_alignment_and_layouts(n, m, ld, k):
    say("tiled update", n, m, ld, k)
    Wb = dev(host_gaussian((n, ld), [70, n, m], std=0.02))
    Mb = dev(host_gaussian((n, ld), [71, n, m]))
    W0, M0 = Wb.cpu().numpy().copy(), Mb.cpu().numpy().copy()
    cfg = d3.ns_cfg(path=d3.PATH_TILED)
    idx, O = d3.step(Wb[:, :m], Mb[:, :m], k, 0.04, 0.95, cfg, return_idx=True, return_O=True)
    W1, M1 = Wb.cpu().numpy(), Mb.cpu().numpy()
    assert W1[:, m:].tobytes() == W0[:, m:].tobytes() and M1[:, m:].tobytes() == M0[:, m:].tobytes()
    check_step(np.ascontiguousarray(W0[:, :m]), np.ascontiguousarray(M0[:, :m]),
               np.ascontiguousarray(W1[:, :m]), np.ascontiguousarray(M1[:, :m]),
               idx.cpu().numpy(), O.cpu().numpy(), k, 0.04, 0.95)
    if min(k, m) <= 128:   # the fused kernel covers this Gram side: same bits
        Wf, Mf = dev(W0), dev(M0)
        idf, Of = d3.step(Wf[:, :m], Mf[:, :m], k, 0.04, 0.95, d3.ns_cfg(path=d3.PATH_FUSED),
                          return_idx=True, return_O=True)
        assert Wf.cpu().numpy().tobytes() == W1.tobytes()
        assert Of.cpu().numpy().tobytes() == O.cpu().numpy().tobytes()
