"""Pins of the fp64 oracle against facts that do not come from the oracle:
the SVD polar factor, the scalar Newton-Schulz map applied to singular values,
brute-force selection, exact fp32 rounding, the pages' printed FLOP figures
and k = ceil(f n) examples.  CPU only."""
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import dion3_oracle as orc
from workloads import host_gaussian, host_lowrank, host_tied

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
CONVERGENT = (15 / 8, -10 / 8, 3 / 8)   # cubic-convergent quintic: fixed point 1


def rel(a, b):
    return np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300)


def scalar_ns_map(sig, coeffs):
    """Apply the quintic iteration to each singular value on its own:
    sigma <- a sigma + b sigma^3 + c sigma^5 (a different route than any
    matrix product)."""
    out = []
    for s in sig:
        x = float(s)
        for (a, b, c) in coeffs:
            x = a * x + b * x ** 3 + c * x ** 5
        out.append(x)
    return np.array(out)


def svd_route(X, coeffs, eps=orc.DEFAULT_EPS):
    X = np.asarray(X, np.float64)
    Xn = X / (np.linalg.norm(X) + eps)
    U, S, Vt = np.linalg.svd(Xn, full_matrices=False)
    return (U * scalar_ns_map(S, coeffs)) @ Vt


SHAPES = [(8, 32), (32, 128), (16, 16), (48, 20), (1, 7), (7, 1), (5, 5), (33, 65)]
RESTARTS = [(), (2,), (3,), (2, 4), (3, 5)]


@pytest.mark.parametrize("shape", SHAPES)
@pytest.mark.parametrize("restart", RESTARTS)
def test_gram_equals_standard(shape, restart):
    X = host_gaussian(shape, [7, shape[0], shape[1]])
    co = orc.default_coeffs()
    g = orc.ns_gram(X, co, restart)
    s = orc.ns_standard(X, co)
    assert g.shape == X.shape
    assert rel(g, s) <= 1e-10


@pytest.mark.parametrize("shape", [(32, 128), (128, 32), (16, 16), (1, 9), (40, 41)])
@pytest.mark.parametrize("method", ["gram", "standard"])
def test_scalar_map_on_singular_values(shape, method):
    X = host_gaussian(shape, [11, shape[0]])
    co = orc.default_coeffs()
    out = orc.ns_gram(X, co, (3,)) if method == "gram" else orc.ns_standard(X, co)
    assert rel(out, svd_route(X, co)) <= 1e-10


@pytest.mark.parametrize("shape", [(24, 64), (64, 24), (20, 20)])
def test_polar_factor(shape):
    """With the convergent coefficients the iteration reaches U V^T."""
    rng = np.random.default_rng(5)
    r = min(shape)
    U, _ = np.linalg.qr(rng.standard_normal((shape[0], r)))
    V, _ = np.linalg.qr(rng.standard_normal((shape[1], r)))
    sig = np.linspace(0.2, 1.0, r)
    X = (U * sig) @ V.T
    co = [CONVERGENT] * 40
    out = orc.ns_gram(X, co, (10, 20, 30))
    assert rel(out, U @ V.T) <= 1e-10
    assert rel(orc.ns_standard(X, co), U @ V.T) <= 1e-10


def test_muon_coefficient_band():
    X = host_gaussian((128, 512), 0)
    out = orc.ns_gram(X, orc.default_coeffs(), (3,))
    sv = np.linalg.svd(out, compute_uv=False)
    assert sv.min() > 0.6 and sv.max() < 1.2
    # same singular subspaces as X: out = U f(S) V^T (near-equal singular
    # values make the SVD basis itself ill-defined, hence the loose bound)
    U, S, Vt = np.linalg.svd(X, full_matrices=False)
    core = U.T @ out @ Vt.T
    assert np.abs(core - np.diag(np.diag(core))).max() < 1e-6


def test_permutation_equivariance():
    X = host_gaussian((24, 40), 3)
    rng = np.random.default_rng(9)
    p, q = rng.permutation(24), rng.permutation(40)
    co = orc.default_coeffs()
    a = orc.ns_gram(X[p][:, q], co, (3,))
    b = orc.ns_gram(X, co, (3,))[p][:, q]
    assert rel(a, b) <= 1e-12


@pytest.mark.parametrize("c", [3.7, 1e-3, 250.0])
def test_scale_invariance(c):
    X = host_gaussian((16, 48), 4).astype(np.float64)
    co = orc.default_coeffs()
    assert rel(orc.ns_gram(c * X, co, (3,), eps=0.0), orc.ns_gram(X, co, (3,), eps=0.0)) <= 1e-12


def test_zero_padding_is_exact():
    """Zero rows/columns appended to X leave the real block unchanged and
    produce zero output there (the padded-tile layout of the kernels relies
    on this)."""
    X = host_gaussian((10, 23), 8)
    co = orc.default_coeffs()
    Xp = np.zeros((16, 32))
    Xp[:10, :23] = X
    out = orc.ns_gram(Xp, co, (3,))
    ref = orc.ns_gram(X, co, (3,))
    assert rel(out[:10, :23], ref) <= 1e-12
    assert np.all(out[10:, :] == 0) and np.all(out[:, 23:] == 0)


def test_restart_schedule_matters_only_numerically():
    X = host_gaussian((12, 30), 2)
    co = orc.default_coeffs()
    outs = [orc.ns_gram(X, co, r) for r in RESTARTS]
    for o in outs[1:]:
        assert rel(o, outs[0]) <= 1e-11


# -------------------------------------------------------------- selection

def brute_topk(scores, k):
    """Repeated first-maximum scan: k passes, each taking the lowest index
    among the largest remaining scores."""
    taken = [False] * len(scores)
    out = []
    for _ in range(k):
        best = -1
        for i, s in enumerate(scores):
            if taken[i]:
                continue
            if best < 0 or s > scores[best]:
                best = i
        taken[best] = True
        out.append(best)
    return sorted(out)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_select_bruteforce_with_ties(seed):
    M = host_tied(37, 11, seed, n_distinct=5)
    l1, _ = orc.row_scores(M)
    assert len(set(l1.tolist())) <= 5          # planted exact ties
    for k in range(1, 38):
        assert orc.select_rows(l1, k).tolist() == brute_topk(l1.tolist(), k)


def test_select_bruteforce_random():
    M = host_gaussian((61, 7), 13)
    l1, _ = orc.row_scores(M)
    for k in (1, 2, 15, 30, 60, 61):
        assert orc.select_rows(l1, k).tolist() == brute_topk(l1.tolist(), k)


def test_select_closed_form_scores():
    """Rows of +-c_i entries have l1 = c_i m exactly."""
    rng = np.random.default_rng(3)
    n, m = 50, 16
    c = rng.permutation(np.arange(1, n + 1)).astype(np.float32)
    M = (rng.choice([-1.0, 1.0], size=(n, m)) * c[:, None]).astype(np.float32)
    l1, sq = orc.row_scores(M)
    assert np.array_equal(l1, c.astype(np.float64) * m)
    assert np.array_equal(sq, c.astype(np.float64) ** 2 * m)
    k = 12
    want = sorted(np.argsort(-c)[:k].tolist())
    assert orc.select_rows(l1, k).tolist() == want


def test_k_from_fraction_golden():
    d = json.load(open(os.path.join(GOLDEN, "k_examples.json")))
    for case in d["cases"]:
        f = Fraction(case["f"]) if "/" in case["f"] else float(case["f"])
        assert orc.k_from_fraction(f, case["n"]) == case["k"], case


# -------------------------------------------------------------- the step

def test_step_unselected_rows_bitwise_and_decay_exact():
    W = host_gaussian((64, 48), 21, std=0.02)
    M = host_gaussian((64, 48), 22)
    k, lr, mu = 16, 0.04, 0.95
    r = orc.dion3_step(W, M, k, lr, mu)
    S = r["S"]
    mask = np.zeros(64, bool)
    mask[S] = True
    assert r["M"][~mask].tobytes() == M[~mask].tobytes()
    assert r["W"][~mask].astype(np.float32).tobytes() == W[~mask].tobytes()
    # decay: numpy's own fp32 multiply is the correctly rounded product
    assert r["M"][mask].tobytes() == (np.float32(mu) * M[mask]).tobytes()


def test_step_update_matches_svd_route():
    W = host_gaussian((40, 24), 31, std=0.02)
    M = host_gaussian((40, 24), 32)
    k, lr, mu = 10, 0.04, 0.9
    r = orc.dion3_step(W, M, k, lr, mu)
    S = r["S"]
    O = svd_route(M[S], orc.default_coeffs())
    assert rel(r["O"], O) <= 1e-10
    assert rel(r["W"][S], W[S].astype(np.float64) - lr * O) <= 1e-12
    # a negative step: the weights move against O
    assert np.sum((r["W"][S] - W[S]) * O) < 0


def test_step_f1_reduces_to_muon():
    """k = n selects every row; the step is W - lr * NS(M), M <- mu M, and with
    the convergent coefficients NS(M) is the polar factor U V^T."""
    W = host_gaussian((24, 56), 41, std=0.02)
    M = host_gaussian((24, 56), 42)
    co = [CONVERGENT] * 30
    r = orc.dion3_step(W, M, 24, 0.02, 0.95, coeffs=co, restart_at=(10, 20))
    assert r["S"].tolist() == list(range(24))
    U, _, Vt = np.linalg.svd(M.astype(np.float64), full_matrices=False)
    assert rel(r["W"], W.astype(np.float64) - 0.02 * (U @ Vt)) <= 1e-12
    assert r["M"].tobytes() == (np.float32(0.95) * M).tobytes()


def test_step_transposed_side():
    """k > m: the Gram is taken on the column side; result is unchanged."""
    W = host_gaussian((48, 12), 51, std=0.02)
    M = host_gaussian((48, 12), 52)
    r = orc.dion3_step(W, M, 30, 0.04, 0.95)
    assert r["O"].shape == (30, 12)
    assert rel(r["O"], svd_route(M[r["S"]], orc.default_coeffs())) <= 1e-10


def test_step_lowrank_restart_runs():
    M = host_lowrank(96, 80, 7)
    W = host_gaussian((96, 80), 8, std=0.02)
    r = orc.dion3_step(W, M, 12, 0.0566, 0.95)
    assert np.all(np.isfinite(r["O"]))
    assert rel(r["O"], svd_route(M[r["S"]], orc.default_coeffs())) <= 1e-9


def test_step_rejects_bad_input():
    W = host_gaussian((8, 8), 1)
    M = host_gaussian((8, 8), 2)
    with pytest.raises(ValueError):
        orc.dion3_step(W, M, 0, 0.1, 0.9)
    with pytest.raises(ValueError):
        orc.dion3_step(W, M, 9, 0.1, 0.9)
    M2 = M.copy()
    M2[3, 3] = np.nan
    with pytest.raises(ValueError):
        orc.dion3_step(W, M2, 2, 0.1, 0.9)


def test_step_accumulates_gradient_exactly():
    """M <- M + G is one correctly rounded fp32 add (numpy's own fp32 add is
    that), every row of the buffer keeps it, and the selection and update
    follow the accumulated buffer."""
    W = host_gaussian((50, 30), 71, std=0.02)
    M = host_gaussian((50, 30), 72)
    G = host_gaussian((50, 30), 73, std=0.1)
    r = orc.dion3_step(W, M, 12, 0.04, 0.95, G=G)
    acc = M + G                                  # numpy float32 add
    mask = np.zeros(50, bool)
    mask[r["S"]] = True
    assert r["M"][~mask].tobytes() == acc[~mask].tobytes()
    assert r["M"][mask].tobytes() == (np.float32(0.95) * acc[mask]).tobytes()
    ref = orc.dion3_step(W, acc, 12, 0.04, 0.95)
    assert np.array_equal(r["S"], ref["S"]) and rel(r["W"], ref["W"]) == 0.0


def test_step_standard_and_gram_agree():
    W = host_gaussian((30, 50), 61, std=0.02)
    M = host_gaussian((30, 50), 62)
    a = orc.dion3_step(W, M, 9, 0.04, 0.95, method="gram")
    b = orc.dion3_step(W, M, 9, 0.04, 0.95, method="standard")
    assert rel(a["O"], b["O"]) <= 1e-10


# --------------------------------------------------------------- FLOP model

def _flops(s, L, restart, symmetric=True, method="gram"):
    log = orc.ProductLog()
    X = np.ones((s, L)) + np.eye(s, L)
    if method == "gram":
        orc.ns_gram(X, orc.default_coeffs(), restart, log=log)
    else:
        orc.ns_standard(X, orc.default_coeffs(), log=log)
    if symmetric:
        return log.flops(), log
    full = sum(2.0 * it[1] * it[1] * it[2] if it[0] == "sym" else 2.0 * it[1] * it[2] * it[3]
               for it in log.items)
    return full, log


def test_flop_figures_of_the_pages():
    d = json.load(open(os.path.join(GOLDEN, "pages_figures.json")))
    s = 16
    L = d["alpha"] * s
    fg, lg = _flops(s, L, ())
    fs, ls = _flops(s, L, (), method="standard")
    fp, _ = _flops(s, L, (), symmetric=False, method="standard")
    touching_L = lambda log: sum(1 for it in log.items if L in it[1:])
    assert touching_L(lg) == d["rectangular_products_gram"]
    assert touching_L(ls) == d["rectangular_products_standard"]
    assert round(100 * (1 - fg / fs)) == d["saving_pct_vs_standard_symmetric"]
    assert round(100 * (1 - fg / fp)) == d["saving_pct_vs_standard_plain"]
    # restart at iteration 3 costs exactly 3 (alpha - 1) s^3 more
    fr, _ = _flops(s, L, (3,))
    assert fr - fg == d["restart_extra_flops_coeff"] * (d["alpha"] - 1) * s ** 3


# ------------------------------------------------------------- per-neuron normalization
# (no formula on the pages: the reading is stated in normalize_neurons; these
# pins fix its invariants and one example worked by hand)

def _norm_case(seed, k=6, m=10, n=9):
    rng = np.random.default_rng(seed)
    O = rng.standard_normal((k, m))
    S = np.sort(rng.choice(n, size=k, replace=False))
    V = rng.uniform(0.01, 1.0, n).astype(np.float32)
    return O, S, V


def test_normalize_keeps_frobenius_norm():
    for seed in range(5):
        O, S, V = _norm_case(seed)
        U, _ = orc.normalize_neurons(O, S, V, 0.9, 1e-8)
        assert abs(np.linalg.norm(U) - np.linalg.norm(O)) <= 1e-12 * np.linalg.norm(O)


def test_normalize_beta0_equalizes_rows():
    """beta2 = 0 and eps = 0: every row is divided by its own RMS, so after the
    norm-preserving rescale all rows have norm ||O||_F / sqrt(k)."""
    O, S, V = _norm_case(11)
    U, _ = orc.normalize_neurons(O, S, V, 0.0, 0.0)
    want = np.linalg.norm(O) / np.sqrt(O.shape[0])
    assert np.allclose(np.linalg.norm(U, axis=1), want, rtol=1e-7)   # V is stored as fp32


def test_normalize_is_identity_on_equal_rows_at_steady_state():
    """Rows of equal mean square whose state already equals that mean square:
    the division is one common factor, which the rescale removes."""
    rng = np.random.default_rng(12)
    Q, _ = np.linalg.qr(rng.standard_normal((16, 5)))
    O = Q.T                                   # 5 orthonormal rows of length 16
    S = np.array([1, 3, 4, 7, 8])
    V = np.full(10, 1.0 / 16, np.float32)     # mean square of a unit row of 16
    U, V1 = orc.normalize_neurons(O, S, V, 0.95, 0.0)
    assert np.allclose(U, O, atol=1e-6)
    assert np.allclose(V1, V, rtol=1e-6)


def test_normalize_worked_example():
    """O = [[3, 4], [0, 5]] (m = 2), rows S = {0, 1}, V = [1, 2, 9], beta2 = 1/2,
    eps = 0, worked by hand:
      q = [25/2, 25/2];  v = [1/2 + 25/4, 1 + 25/4] = [6.75, 7.25];
      U_hat = [[3, 4] / sqrt(6.75), [0, 5] / sqrt(7.25)];
      ||U_hat||^2 = 25/6.75 + 25/7.25 = 7.15197956577...;
      U = U_hat * sqrt(50 / 7.15197956577...), i.e.
      U = [[3.05310147, 4.07080196], [0, 4.90990253]]; V' = [6.75, 7.25, 9]."""
    O = np.array([[3.0, 4.0], [0.0, 5.0]])
    U, V1 = orc.normalize_neurons(O, np.array([0, 1]), np.array([1, 2, 9], np.float32), 0.5, 0.0)
    assert np.allclose(U, [[3.05310147, 4.07080196], [0.0, 4.90990253]], atol=5e-8)
    assert V1.tolist() == [6.75, 7.25, 9.0]


def test_normalize_state_of_unselected_rows_untouched():
    O, S, V = _norm_case(13)
    _, V1 = orc.normalize_neurons(O, S, V, 0.9, 1e-8)
    rest = np.setdiff1d(np.arange(V.size), S)
    assert V1[rest].tobytes() == V[rest].tobytes()
    assert V1.dtype == np.float32


def test_normalize_permutation_equivariant():
    O, S, V = _norm_case(14)
    p = np.random.default_rng(15).permutation(O.shape[0])
    U, V1 = orc.normalize_neurons(O, S, V, 0.8, 1e-6)
    Up, V1p = orc.normalize_neurons(O[p], S[p], V, 0.8, 1e-6)
    assert np.allclose(Up, U[p], atol=1e-12)
    assert V1p.tobytes() == V1.tobytes()


def test_normalize_homogeneous_at_beta0():
    O, S, V = _norm_case(16)
    U, _ = orc.normalize_neurons(O, S, V, 0.0, 0.0)
    U3, _ = orc.normalize_neurons(3.0 * O, S, V, 0.0, 0.0)
    assert np.allclose(U3, 3.0 * U, rtol=1e-6)


def test_normalize_rejects_bad_input():
    O, S, V = _norm_case(17)
    with pytest.raises(TypeError):
        orc.normalize_neurons(O, S, V.astype(np.float64), 0.9, 1e-8)
    with pytest.raises(ValueError):
        orc.normalize_neurons(O, S, V, 1.0, 1e-8)
    with pytest.raises(ValueError):
        orc.normalize_neurons(O, S, V, 0.9, -1.0)


def test_step_with_normalization_updates_by_u():
    rng = np.random.default_rng(18)
    W = (rng.standard_normal((40, 24)) * 0.02).astype(np.float32)
    M = rng.standard_normal((40, 24)).astype(np.float32)
    V = np.zeros(40, np.float32)
    ref = orc.dion3_step(W, M, 10, 0.04, 0.95, norm=(V, 0.95, 1e-8))
    S = ref["S"]
    assert np.allclose(ref["W"][S] - W[S], -0.04 * ref["U"], atol=1e-12)
    assert abs(np.linalg.norm(ref["U"]) - np.linalg.norm(ref["O"])) <= 1e-10
    assert ref["V"][np.setdiff1d(np.arange(40), S)].tobytes() == bytes(4 * 30)
    # a zero momentum gives a zero update (and a decayed, still zero, state)
    ref0 = orc.dion3_step(W, np.zeros_like(M), 10, 0.04, 0.95, norm=(V, 0.95, 1e-8))
    assert not np.any(ref0["U"])


def test_normalize_worked_example_ema_weights_and_eps():
    """The example above with beta2 = 0.9: v = [0.9 + 1.25, 1.8 + 1.25] =
    [2.15, 3.05] (a swapped weighting would give 11.35); and with beta2 = 1/2,
    eps = 1: U_hat = O / (sqrt(v) + 1) = [[3, 4] / 3.598076, [0, 5] / 3.692582],
    rescaled to norm sqrt(50): [[3.038633, 4.051510], [0, 4.934772]]."""
    O = np.array([[3.0, 4.0], [0.0, 5.0]])
    V = np.array([1, 2, 9], np.float32)
    _, V1 = orc.normalize_neurons(O, np.array([0, 1]), V, 0.9, 0.0)
    assert V1.tolist() == np.array([2.15, 3.05, 9.0], np.float32).tolist()
    U, _ = orc.normalize_neurons(O, np.array([0, 1]), V, 0.5, 1.0)
    assert np.allclose(U, [[3.038633, 4.051510], [0.0, 4.934772]], rtol=0, atol=1e-6)


def test_normalize_zero_row_with_zero_state_and_eps():
    O = np.array([[0.0, 0.0], [0.0, 5.0]])
    U, V1 = orc.normalize_neurons(O, np.array([0, 1]), np.zeros(2, np.float32), 0.5, 0.0)
    assert np.all(np.isfinite(U)) and not np.any(U[0])
    assert np.allclose(U[1], [0.0, 5.0])
