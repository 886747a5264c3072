"""Per-neuron normalization of the update (dion3_step_megabatch_norm)
against the oracle: the normalization arithmetic tightly, on the GPU's own
orthogonalized rows, and the whole step against the fp64 oracle at the
step's tolerance; fused and tiled Gram paths, k > m, gradient accumulation,
and the torch.optim-style optimizer."""
import sys

import numpy as np
import pytest

from oracle import dion3_oracle as orc
from tests.parity import O_TOL, check_selection, rel
from workloads import host_gaussian

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"
BETA2, EPS, LR, MU = 0.9, 1e-8, 0.04, 0.95


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


# (n, m, k): fused path (Gram side <= 128), tiled, k > m (transposed Gram), ragged
CASES = [(200, 300, 50), (700, 520, 300), (500, 96, 300), (130, 257, 129), (64, 64, 64)]


@pytest.mark.parametrize("n,m,k", CASES)
@pytest.mark.parametrize("accumulate", [False, True])
def test_norm_step(n, m, k, accumulate):
    say("norm step", n, m, k, accumulate)
    B = 3
    Ws = [host_gaussian((n, m), [100, n, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [101, n, b]) for b in range(B)]
    Gs = [host_gaussian((n, m), [102, n, b]) for b in range(B)] if accumulate else None
    rng = np.random.default_rng(n + m)
    Vs = [rng.uniform(0.0, 0.01, n).astype(np.float32) for _ in range(B)]
    Wd, Md, Vd = [dev(w) for w in Ws], [dev(x) for x in Ms], [dev(v) for v in Vs]
    Gd = [dev(g) for g in Gs] if accumulate else None
    idx, O = d3.step_megabatch(Wd, Md, k, LR, MU, Gs=Gd, norm=(Vd, BETA2, EPS), return_idx=True,
                               return_O=True)
    torch.cuda.synchronize()
    for b in range(B):
        M0 = Ms[b] + Gs[b] if accumulate else Ms[b]
        S, Ob = idx[b].cpu().numpy(), O[b].cpu().numpy().astype(np.float64)
        W1, M1, V1 = Wd[b].cpu().numpy(), Md[b].cpu().numpy(), Vd[b].cpu().numpy()
        assert np.array_equal(S, check_selection(S, M0, k))
        # the normalization on the GPU's own O: tight
        U_ref, V_ref = orc.normalize_neurons(Ob, S, Vs[b], BETA2, EPS)
        rest = np.setdiff1d(np.arange(n), S)
        assert V1[rest].tobytes() == Vs[b][rest].tobytes()
        assert np.max(np.abs(V1[S] - V_ref[S]) / V_ref[S]) <= 1e-5
        assert W1[rest].tobytes() == Ws[b][rest].tobytes()
        assert rel(W1[S] - Ws[b][S], -LR * U_ref) <= 1e-5
        # the whole step against the fp64 oracle
        ref = orc.dion3_step(Ws[b], M0, k, LR, MU, norm=(Vs[b], BETA2, EPS))
        assert M1.tobytes() == ref["M"].tobytes()
        assert rel(Ob, ref["O"]) <= O_TOL
        assert rel(W1[S] - Ws[b][S], ref["W"][S] - Ws[b][S]) <= O_TOL


def test_norm_step_equal_across_paths():
    """The fused and tiled Gram paths give the same O bit for bit, so the
    normalized step is bitwise the same too."""
    say("norm paths")
    n, m, k = 300, 200, 75
    W = host_gaussian((n, m), 103, std=0.02)
    M = host_gaussian((n, m), 104)
    outs = []
    for p in (d3.PATH_FUSED, d3.PATH_TILED):
        Wd, Md, Vd = [dev(W)], [dev(M)], [torch.zeros(n, device=DEV)]
        d3.step_megabatch(Wd, Md, k, LR, MU, d3.ns_cfg(path=p), norm=(Vd, BETA2, EPS))
        torch.cuda.synchronize()
        outs.append((Wd[0].cpu().numpy(), Vd[0].cpu().numpy()))
    assert outs[0][0].tobytes() == outs[1][0].tobytes()
    assert outs[0][1].tobytes() == outs[1][1].tobytes()


def test_dion3_optimizer_normalized_two_steps():
    say("Dion3 optimizer, normalized")
    shapes = [(96, 64), (64, 96)]
    params = [torch.nn.Parameter(dev(host_gaussian(sh, [105, i], std=0.02)))
              for i, sh in enumerate(shapes)]
    opt = d3.Dion3(params, lr=0.02, fraction=0.25, mu=0.9, normalize=True, beta2=BETA2, eps=EPS)
    W = [p.detach().cpu().numpy().copy() for p in params]
    M = [np.zeros(sh, np.float32) for sh in shapes]
    V = [np.zeros(sh[0], np.float32) for sh in shapes]
    for it in range(2):
        G = [host_gaussian(sh, [106, it, i]) for i, sh in enumerate(shapes)]
        for p, g in zip(params, G):
            p.grad = dev(g)
        opt.step()
        torch.cuda.synchronize()
        for i, (p, sh) in enumerate(zip(params, shapes)):
            k = orc.k_from_fraction(0.25, sh[0])
            ref = orc.dion3_step(W[i], M[i] + G[i], k, 0.04, 0.9, norm=(V[i], BETA2, EPS))
            W1 = p.detach().cpu().numpy()
            M1 = opt.state[p]["momentum"].cpu().numpy()
            V1 = opt.state[p]["second_moment"].cpu().numpy()
            assert M1.tobytes() == ref["M"].tobytes(), (it, i)
            assert rel(W1 - W[i], ref["W"] - W[i]) <= O_TOL, (it, i)
            assert rel(V1, ref["V"]) <= 2e-2, (it, i)
            W[i], M[i], V[i] = W1, M1, V1


def test_norm_fused_many_matrices_equals_tiled():
    """600 matrices (more than one wave of workgroups) through the one-launch
    fused path with normalization: each matrix's O goes inside that matrix's
    own padded block, so results equal the tiled path's bit for bit."""
    say("norm fused 600 matrices")
    B, n, m, k = 600, 40, 100, 30
    rng = np.random.default_rng(107)
    Wh = (rng.standard_normal((B, n, m)) * 0.02).astype(np.float32)
    Mh = rng.standard_normal((B, n, m)).astype(np.float32)
    outs = []
    for p in (d3.PATH_FUSED, d3.PATH_TILED):
        Wd, Md = dev(Wh), dev(Mh)
        Vd = torch.zeros((B, n), device=DEV)
        _, O = d3.step_megabatch(list(Wd.unbind(0)), list(Md.unbind(0)), k, LR, MU,
                                 d3.ns_cfg(path=p), norm=(list(Vd.unbind(0)), BETA2, EPS),
                                 return_O=True)
        torch.cuda.synchronize()
        outs.append((Wd.cpu().numpy(), Vd.cpu().numpy(), O.cpu().numpy()))
    for a, b in zip(outs[0], outs[1]):
        assert a.tobytes() == b.tobytes()


def test_norm_single_matrix_equals_megabatch():
    say("norm single vs megabatch")
    n, m, k = 300, 200, 75
    W = host_gaussian((n, m), 108, std=0.02)
    M = host_gaussian((n, m), 109)
    Wa, Ma, Va = dev(W), dev(M), torch.zeros(n, device=DEV)
    idx_a, O_a = d3.step(Wa, Ma, k, LR, MU, norm=(Va, BETA2, EPS), return_idx=True, return_O=True)
    Wb, Mb, Vb = dev(W), dev(M), torch.zeros(n, device=DEV)
    idx_b, O_b = d3.step_megabatch([Wb], [Mb], k, LR, MU, norm=([Vb], BETA2, EPS),
                                   return_idx=True, return_O=True)
    torch.cuda.synchronize()
    assert np.array_equal(idx_a.cpu().numpy(), idx_b[0].cpu().numpy())
    assert O_a.cpu().numpy().tobytes() == O_b[0].cpu().numpy().tobytes()
    for x, y in ((Wa, Wb), (Ma, Mb), (Va, Vb)):
        assert x.cpu().numpy().tobytes() == y.cpu().numpy().tobytes()


@pytest.mark.parametrize("iters,restarts,method,path", [
    (5, (), d3.NS_GRAM, d3.PATH_TILED), (5, (3,), d3.NS_GRAM, d3.PATH_TILED),
    (7, (3, 6), d3.NS_GRAM, d3.PATH_TILED), (7, (3, 6), d3.NS_GRAM, d3.PATH_FUSED),
    (5, (), d3.NS_GRAM, d3.PATH_FUSED), (5, (), d3.NS_STANDARD, d3.PATH_AUTO),
    (4, (), d3.NS_STANDARD, d3.PATH_AUTO)])
def test_norm_o_buffer_never_aliases_the_iteration(iters, restarts, method, path):
    """O goes to the X pair the iteration no longer reads; which pair that is
    depends on the parity of restarts (Gram) or iterations (standard).  For
    every parity the normalized path's O equals the plain path's bit for bit."""
    say("norm O buffer", iters, restarts, method, path)
    n, m, k = 300, 200, 75 if path != d3.PATH_TILED else 150
    W = host_gaussian((n, m), [110, iters], std=0.02)
    M = host_gaussian((n, m), [111, iters])
    cfg = d3.ns_cfg(iters=iters, restart_at=restarts, coeffs=[orc.MUON_COEFFS] * iters,
                    method=method, path=path)
    _, O_plain = d3.step(dev(W), dev(M), k, LR, MU, cfg, return_O=True)
    _, O_norm = d3.step(dev(W), dev(M), k, LR, MU, cfg, return_O=True,
                        norm=(torch.zeros(n, device=DEV), BETA2, EPS))
    torch.cuda.synchronize()
    assert O_norm.cpu().numpy().tobytes() == O_plain.cpu().numpy().tobytes()


def test_norm_step_large_tile_block_sums():
    """16 matrices with k = 1024 take the 256-wide tiles, whose output rows
    each hold two 128-column blocks of the row sums the final product writes
    for the normalization; the normalization of the GPU's own O matches the
    oracle's tightly, on the first and last matrix."""
    say("norm 256 tile")
    B, n, m, k = 16, 1100, 2048, 1024
    Ws = [host_gaussian((n, m), [112, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [113, b]) for b in range(B)]
    Vs = [np.random.default_rng([114, b]).uniform(0.0, 0.01, n).astype(np.float32)
          for b in range(B)]
    Wd, Md, Vd = [dev(w) for w in Ws], [dev(x) for x in Ms], [dev(v) for v in Vs]
    idx, O = d3.step_megabatch(Wd, Md, k, LR, MU, norm=(Vd, BETA2, EPS), return_idx=True,
                               return_O=True)
    torch.cuda.synchronize()
    for b in (0, B - 1):
        S, Ob = idx[b].cpu().numpy(), O[b].cpu().numpy().astype(np.float64)
        U_ref, V_ref = orc.normalize_neurons(Ob, S, Vs[b], BETA2, EPS)
        V1, W1 = Vd[b].cpu().numpy(), Wd[b].cpu().numpy()
        assert np.max(np.abs(V1[S] - V_ref[S]) / V_ref[S]) <= 1e-5
        assert rel(W1[S] - Ws[b][S], -LR * U_ref) <= 1e-5
        rest = np.setdiff1d(np.arange(n), S)
        assert W1[rest].tobytes() == Ws[b][rest].tobytes()
