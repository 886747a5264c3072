"""Comparison helpers shared by the GPU parity tests: run the HIP path
through the binding, run the oracle on the same fp32 bytes, and apply the
acceptance rules (exact row sets up to the tie band, bit-exact untouched and
decayed rows, relative Frobenius error of the orthogonalized update)."""
import numpy as np

from oracle import dion3_oracle as orc

O_TOL = 2e-2          # relative Frobenius error of O against the fp64 oracle
TIE_BAND = 1e-6       # rows whose l1 is this close (relative) to the k-th score may differ


def rel(a, b):
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    return float(np.linalg.norm(a - b) / max(np.linalg.norm(b), 1e-300))


def check_selection(S_gpu, M, k):
    """S_gpu must equal the oracle's set except for rows inside the tie band
    around the k-th largest l1 score.  Returns the oracle set."""
    l1, _ = orc.row_scores(M)
    S_ref = orc.select_rows(l1, k)
    S_gpu = np.asarray(S_gpu, np.int64)
    assert S_gpu.shape == (k,)
    assert np.all(np.diff(S_gpu) > 0), "indices must be strictly ascending"
    assert S_gpu.min() >= 0 and S_gpu.max() < M.shape[0]
    if not np.array_equal(S_gpu, S_ref):
        b = np.sort(l1)[::-1][k - 1]
        diff = np.setxor1d(S_gpu, S_ref)
        assert np.all(np.abs(l1[diff] - b) <= TIE_BAND * b), (
            f"selection differs outside the tie band: {diff[:10]}")
    return S_ref


def oracle_for(W, M, k, lr, mu, S_gpu, coeffs=None, restart_at=(3,)):
    """The oracle's step, re-run on the GPU's set when the two differ only in
    the tie band (any set that is correct gives its own O)."""
    S_ref = check_selection(S_gpu, M, k)
    override = None if np.array_equal(S_ref, S_gpu) else S_gpu
    return orc.dion3_step(W, M, k, lr, mu, coeffs=coeffs, restart_at=restart_at,
                          S_override=override)


def check_step(W0, M0, W1, M1, S_gpu, O_gpu, k, lr, mu, coeffs=None, restart_at=(3,), G=None):
    """Full acceptance of one matrix's step.  Returns the O error.  With a
    gradient G, the buffer the step starts from is fl32(M0 + G)."""
    if G is not None:
        M0 = M0 + G          # numpy float32 add: the correctly rounded sum
    ref = oracle_for(W0, M0, k, lr, mu, S_gpu, coeffs, restart_at)
    S = ref["S"]
    n = M0.shape[0]
    mask = np.zeros(n, bool)
    mask[S] = True
    # untouched rows: bit-exact
    assert W1[~mask].tobytes() == W0[~mask].tobytes()
    assert M1[~mask].tobytes() == M0[~mask].tobytes()
    # decayed rows: the correctly rounded fp32 product
    assert M1[mask].tobytes() == ref["M"][mask].tobytes()
    # orthogonalized update
    err = rel(O_gpu.astype(np.float64), ref["O"])
    assert err <= O_TOL, f"O relative error {err:.3e} > {O_TOL}"
    # weights: W - lr * O_gpu with one fp32 rounding (an fma).  fp32(lr) times
    # an fp16 value is exact in fp64, so `exact` carries one fp64 rounding;
    # rounded to fp32 it is the correctly rounded result except where the two
    # roundings meet at a tie, so every element must lie within 1 fp32 ulp of
    # it and almost all must equal it
    exact = W0[S].astype(np.float64) - np.float64(np.float32(lr)) * O_gpu.astype(np.float64)
    want = exact.astype(np.float32)
    ulp = np.spacing(np.abs(want)).astype(np.float64)
    off = np.abs(W1[S].astype(np.float64) - want.astype(np.float64))
    assert np.all(off <= ulp), f"W[S] off by {np.max(off / ulp):.2f} ulp"
    assert np.mean(W1[S] == want) >= 0.999
    # and against the oracle's fp64 weights, to the O tolerance scaled by lr
    assert rel(W1[S] - W0[S], ref["W"][S] - W0[S]) <= O_TOL
    return err
