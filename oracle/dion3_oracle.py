"""Plain fp64 CPU oracle of the Dion3 optimizer step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product (the HIP library, its
Python binding) imports, calls or links this file; only the tests, the smoke
check and the benchmark's CPU-baseline leg do.  It shares no code with the
HIP path: it is written from the pages' description of the method and
uses NumPy float64 matrix products as its only primitive.

Sources (the pages are cited by title and paragraph):

* [AGI] "Dion3: Full-Stack Orthogonal Updates", agihunt.info/papers/2608.11612
  (summary in Chinese):
    - level-1 paragraph: Newton-Schulz run on the small symmetric Gram matrix
      X X^T instead of X, multiplied back onto X at the end; output identical
      to standard Newton-Schulz; one restart at the 3rd iteration against
      spurious negative eigenvalues; float16 compute.
    - level-3 paragraph: pick k = ceil(f n) rows by l1 norm, orthogonalize
      only that submatrix, update only those weight rows, decay only the
      selected momentum rows by mu, leave the rest untouched; f = 1 reduces to
      Muon; eta proportional to 1/sqrt(f).
    - limitations paragraph: the restart costs an extra 3(alpha-1) n^3 FLOP.
* [QSA] "Dion3 Cuts Muon Optimizer Time by Up to 6x - With Parallelism
  Limits", quasa.io: section "Dion3's fastest path is a combined systems
  stack" (error feedback; a full fraction reduces to Muon in exact
  arithmetic).
* [ABS] the paper abstract ("Dion3: Full-Stack Orthogonal Updates", as
  reproduced on arxivlens.com and scholarbro.com): the step orthogonalizes a
  subset of the momentum rows rather than the whole matrix.

Readings where the pages are silent (each is also a row of the design notes):

* quintic coefficients: Muon's published (3.4445, -4.7750, 2.0315) for every
  iteration, passed in as a per-iteration table;
* the submatrix is divided by (||X||_F + eps), eps = 1e-7, before iterating;
* "restart at the 3rd iteration": iteration 3 (1-based) starts from
  X <- Q X, R <- X X^T, Q <- I;
* the Gram is taken on the smaller side: if k > m the oracle works on X^T;
* "rows" are dim 0 of the row-major n x m matrix;
* k = ceil(f n) is computed in exact rationals and clamped to [1, n];
* ties in the l1 score go to the lowest row index;
* X is built from the undecayed momentum rows, then those rows are decayed;
* when a gradient G is given, it is first accumulated into the buffer,
  M <- M + G (one fp32 addition): error feedback keeps every row of the
  buffer and only the selected ones are decayed after use ([AGI] level-3
  paragraph), so the buffer is a running sum.

* per-neuron normalization (no formula on the pages): see
  normalize_neurons.

Parity pins for every function live in tests/test_oracle.py (SVD polar
factor, the scalar Newton-Schulz map on singular values, Gram NS against
standard NS, brute-force selection, the pages' FLOP figures, and for the
normalization its invariants and a hand-worked example).
"""
from __future__ import annotations

from fractions import Fraction
from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

MUON_COEFFS: Tuple[float, float, float] = (3.4445, -4.7750, 2.0315)
DEFAULT_ITERS = 5
DEFAULT_RESTART_AT: Tuple[int, ...] = (3,)
DEFAULT_EPS = 1e-7


def default_coeffs(iters: int = DEFAULT_ITERS) -> List[Tuple[float, float, float]]:
    return [MUON_COEFFS] * iters


# --------------------------------------------------------------- selection

def k_from_fraction(f, n: int) -> int:
    """k = ceil(f n) ([AGI] level-3 paragraph), exact: f is read as the nearest
    fraction with denominator <= 2^20, so 0.1 * 30 gives 3, not 4."""
    if n < 1:
        raise ValueError("n must be >= 1")
    fr = Fraction(f).limit_denominator(1 << 20) if not isinstance(f, Fraction) else f
    k = -((-fr.numerator * n) // fr.denominator)
    return int(max(1, min(n, k)))


def row_scores(M: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Per-row l1 norm ([AGI] level-3: rows are picked by l1 norm) and, for
    the Frobenius normalization, per-row sum of squares; both in fp64 over
    exact upcasts of the fp32 entries."""
    X = np.asarray(M, dtype=np.float64)
    return np.abs(X).sum(axis=1), (X * X).sum(axis=1)


def select_rows(l1: np.ndarray, k: int) -> np.ndarray:
    """Indices of the k largest scores, ties to the lowest index, returned in
    ascending index order ([AGI] level-3 paragraph)."""
    n = l1.shape[0]
    if not 1 <= k <= n:
        raise ValueError("k out of range")
    order = np.lexsort((np.arange(n), -l1))      # primary: -score, secondary: index
    return np.sort(order[:k]).astype(np.int64)


# ---------------------------------------------------------- Newton-Schulz

class ProductLog:
    """Records every matrix product the Gram iteration performs, so the
    operation count can be checked against the pages' FLOP figures.
    Symmetric products (the result is symmetric, only one triangle is
    needed: [AGI] level-2 paragraph) are logged as ("sym", rows, inner);
    others as ("rect", rows, cols, inner)."""

    def __init__(self):
        self.items: List[tuple] = []

    def sym(self, rows: int, inner: int):
        self.items.append(("sym", rows, inner))

    def rect(self, rows: int, cols: int, inner: int):
        self.items.append(("rect", rows, cols, inner))

    def flops(self) -> float:
        """Multiply-add counted as 2 flops; a symmetric product counts half
        of the full product (one triangle)."""
        tot = 0.0
        for it in self.items:
            if it[0] == "sym":
                tot += it[1] * it[1] * it[2]
            else:
                tot += 2.0 * it[1] * it[2] * it[3]
        return tot

    def count(self, kind: str) -> int:
        return sum(1 for it in self.items if it[0] == kind)


def _orient(X: np.ndarray) -> Tuple[np.ndarray, bool]:
    """Work on the wide orientation (rows <= cols) so the Gram is the small side."""
    X = np.asarray(X, dtype=np.float64)
    if X.ndim != 2:
        raise ValueError("expected a matrix")
    if X.shape[0] > X.shape[1]:
        return X.T.copy(), True
    return X.copy(), False


def _normalize(X: np.ndarray, eps: float) -> np.ndarray:
    return X / (np.linalg.norm(X) + eps)


def ns_standard(X, coeffs: Sequence[Tuple[float, float, float]], eps: float = DEFAULT_EPS,
                log: Optional[ProductLog] = None) -> np.ndarray:
    """Standard quintic Newton-Schulz on X itself (the iteration the Gram form
    replaces, [AGI] level-1 paragraph): X <- a X + (b A + c A^2) X, A = X X^T.
    Restarts have no meaning here."""
    X, tr = _orient(X)
    X = _normalize(X, eps)
    s, L = X.shape
    for (a, b, c) in coeffs:
        A = X @ X.T
        A2 = A @ A
        B = b * A + c * A2
        X = a * X + B @ X
        if log is not None:
            log.sym(s, L)
            log.sym(s, s)
            log.rect(s, L, s)
    return X.T if tr else X


def ns_gram(X, coeffs: Sequence[Tuple[float, float, float]],
            restart_at: Iterable[int] = DEFAULT_RESTART_AT, eps: float = DEFAULT_EPS,
            log: Optional[ProductLog] = None) -> np.ndarray:
    """Gram Newton-Schulz ([AGI] level-1 paragraph).

    The iteration runs on R = X X^T and accumulates the product of the
    quintic polynomials Z_t = a_t I + b_t R + c_t R^2 in Q; only at the end is
    Q multiplied back onto X.  Because X_{t+1} = Z_t X_t, the Gram of the next
    iterate is Z_t R_t Z_t, and every matrix involved is a polynomial in the
    first Gram, so all of them commute and are symmetric.

    Restart ([AGI] level-1 paragraph, cost stated in the limitations
    paragraph): an iteration listed in ``restart_at`` (1-based) first
    materializes X <- Q X, recomputes R <- X X^T and resets Q <- I.

    Products that the algorithm does not need are not performed: Q <- Z Q
    when Q is the identity, and the Gram update after the last iteration or
    right before a restart (which recomputes it).
    """
    restarts = set(int(r) for r in restart_at)
    T = len(coeffs)
    X, tr = _orient(X)
    X = _normalize(X, eps)
    s, L = X.shape
    R = X @ X.T
    if log is not None:
        log.sym(s, L)
    Q = np.eye(s)
    q_identity = True
    for t in range(1, T + 1):
        if t in restarts:
            if not q_identity:
                X = Q @ X
                if log is not None:
                    log.rect(s, L, s)
            R = X @ X.T
            if log is not None:
                log.sym(s, L)
            Q = np.eye(s)
            q_identity = True
        a, b, c = coeffs[t - 1]
        R2 = R @ R
        if log is not None:
            log.sym(s, s)
        Z = a * np.eye(s) + b * R + c * R2
        if q_identity:
            Q = Z
            q_identity = False
        else:
            Q = Z @ Q
            if log is not None:
                log.sym(s, s)
        if t < T and (t + 1) not in restarts:
            R = Z @ R @ Z
            if log is not None:
                log.sym(s, s)
                log.sym(s, s)
    O = Q @ X
    if log is not None and not q_identity:
        log.rect(s, L, s)
    return O.T if tr else O


# ------------------------------------------------------------- per-neuron normalization

def normalize_neurons(O: np.ndarray, S: np.ndarray, V: np.ndarray, beta2: float,
                      eps: float) -> Tuple[np.ndarray, np.ndarray]:
    """Per-neuron normalization of the orthogonalized update.

    The pages say only that Dion3 inherits NorMuon's per-neuron normalization
    ([QSA] section "Dion3's fastest path is a combined systems stack") and
    that it runs in float32 ([AGI] limitations paragraph); they give no
    formula.  Reading taken here, for the rows S of one matrix with the
    orthogonalized rows O (k x m) and a float32 second-moment state V (one
    entry per row of the matrix):

      q_i = mean_j O_ij^2                       (mean square of row i)
      V[S_i] <- beta2 V[S_i] + (1 - beta2) q_i  (stored as float32; rows
                                                 outside S keep their state)
      U_i = O_i / (sqrt(V[S_i]) + eps)          (0 when that is 0 / 0: a zero
                                                 row with a zero state)
      U  <- U ||O||_F / ||U||_F                 (the update keeps O's norm, so
                                                 the step size keeps its
                                                 meaning, eta ~ 1/sqrt(f))

    Returns (U, V') with U the update that takes O's place.
    """
    O = np.asarray(O, np.float64)
    S = np.asarray(S, np.int64)
    V = np.asarray(V)
    if V.dtype != np.float32 or V.ndim != 1:
        raise TypeError("V must be a float32 vector")
    if not (0.0 <= beta2 < 1.0) or not eps >= 0.0:
        raise ValueError("need 0 <= beta2 < 1 and eps >= 0")
    k, m = O.shape
    if S.shape != (k,):
        raise ValueError("one state row per row of O")
    sq = (O * O).sum(axis=1)
    v = (beta2 * V[S].astype(np.float64) + (1.0 - beta2) * (sq / m)).astype(np.float32)
    V_new = V.copy()
    V_new[S] = v
    d = np.sqrt(v.astype(np.float64)) + eps
    # d = 0 needs v = 0 and eps = 0, so the row of O is zero: its update is zero
    U = np.divide(O, d[:, None], out=np.zeros_like(O), where=d[:, None] > 0)
    nU = np.linalg.norm(U)
    U = U * (np.sqrt(sq.sum()) / nU) if nU > 0 else np.zeros_like(O)
    return U, V_new


# ------------------------------------------------------------- the step

def dion3_step(W: np.ndarray, M: np.ndarray, k: int, lr: float, mu: float,
               coeffs: Optional[Sequence[Tuple[float, float, float]]] = None,
               restart_at: Iterable[int] = DEFAULT_RESTART_AT, eps: float = DEFAULT_EPS,
               S_override: Optional[np.ndarray] = None, method: str = "gram",
               G: Optional[np.ndarray] = None,
               norm: Optional[Tuple[np.ndarray, float, float]] = None) -> dict:
    """One Dion3 step on one matrix ([AGI] level-3 paragraph, [ABS]).

    1. score rows by l1 and keep the k best (ties: lowest index);
    2. orthogonalize the selected k x m submatrix by Gram Newton-Schulz;
    3. W[S] <- W[S] - lr * O (lr is the final step size; the caller applies
       the 1/sqrt(f) scaling), other weight rows untouched;
    4. M[S] <- mu * M[S] as one correctly rounded fp32 product, other momentum
       rows untouched (error feedback keeps them for later steps).

    With a gradient G, the buffer first accumulates it: M <- fl32(M + G).
    With norm = (V, beta2, eps) the update is the per-neuron normalized U of
    normalize_neurons in place of O, and the new state is returned as "V".

    Returns W' (fp64 on S, the input bytes elsewhere), M' (fp32), S, O and
    the normalized fp64 submatrix that entered the iteration.
    """
    W = np.asarray(W)
    M = np.asarray(M)
    if G is not None:
        G = np.asarray(G)
        if G.dtype != np.float32 or G.shape != M.shape:
            raise TypeError("G must be float32 with the shape of M")
        # exact sum in fp64, one rounding to fp32: the correctly rounded fp32 add
        M = (M.astype(np.float64) + G.astype(np.float64)).astype(np.float32)
    if M.dtype != np.float32 or W.dtype != np.float32:
        raise TypeError("W and M must be float32")
    n, m = M.shape
    if W.shape != (n, m):
        raise ValueError("W and M shapes differ")
    if not 1 <= k <= n:
        raise ValueError("k out of range")
    if not np.all(np.isfinite(M)):
        raise ValueError("non-finite momentum")
    coeffs = default_coeffs() if coeffs is None else list(coeffs)

    l1, sq = row_scores(M)
    if S_override is None:
        S = select_rows(l1, k)
    else:
        S = np.sort(np.asarray(S_override, dtype=np.int64))
        if S.shape != (k,) or len(set(S.tolist())) != k:
            raise ValueError("S_override must hold k distinct rows")
    X = M[S].astype(np.float64)
    if method == "gram":
        O = ns_gram(X, coeffs, restart_at, eps)
    elif method == "standard":
        O = ns_standard(X, coeffs, eps)
    else:
        raise ValueError(method)

    out = {}
    U = O
    if norm is not None:
        V, beta2, neps = norm
        U, out["V"] = normalize_neurons(O, S, V, beta2, neps)
        out["U"] = U
    W_new = W.astype(np.float64)
    W_new[S] = W_new[S] - float(lr) * U
    M_new = M.copy()
    mu32 = np.float64(np.float32(mu))
    M_new[S] = (mu32 * M[S].astype(np.float64)).astype(np.float32)
    out.update({"W": W_new, "M": M_new, "S": S, "O": O, "l1": l1, "sq": sq,
                "X": _normalize(X, eps)})
    return out

