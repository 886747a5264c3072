"""The fused one-launch Gram iteration (Gram side min(k, m) <= 128, one
workgroup per matrix): bitwise equal to the tiled launches on the same
inputs, within the oracle tolerance, and under every schedule shape."""
import sys

import numpy as np
import pytest

from oracle import dion3_oracle as orc
from tests.parity import O_TOL, check_step, rel
from workloads import host_gaussian, host_lowrank

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def run_step(W, M, k, lr, mu, cfg):
    Wd, Md = dev(W), dev(M)
    idx, O = d3.step(Wd, Md, k, lr, mu, cfg, return_idx=True, return_O=True)
    torch.cuda.synchronize()
    return Wd.cpu().numpy(), Md.cpu().numpy(), idx.cpu().numpy(), O.cpu().numpy()


def same(a, b):
    return np.asarray(a).tobytes() == np.asarray(b).tobytes()


# (n, m, k): k <= m with the Gram on X X^T, k > m with X^T X (m <= 128),
# ragged sides, one row, one column, long rows (L = 4096)
# (sides up to 32 and up to 64 take the one-wave kernel, larger sides the
# 128-padded one)
FUSED_STEP_CASES = [(128, 512, 32), (300, 200, 75), (512, 512, 128), (1024, 96, 512),
                    (200, 128, 200), (64, 4096, 16), (130, 1, 5), (1, 16, 1), (129, 129, 128),
                    (300, 200, 40), (300, 200, 64), (120, 40, 100), (100, 30, 90), (65, 700, 33),
                    (20, 6, 3), (64, 13, 8),
                    # rows that end in a partial chunk of the Gram's LDS staging
                    # (512 columns at sides up to 32, 256 up to 64), both orientations
                    (100, 600, 20), (100, 300, 50), (2000, 20, 600), (1000, 50, 300)]


@pytest.mark.parametrize("n,m,k", FUSED_STEP_CASES)
def test_fused_step_equals_tiled_bitwise(n, m, k):
    say("fused step", n, m, k)
    W = host_gaussian((n, m), [40, n, m], std=0.02)
    M = host_gaussian((n, m), [41, n, m])
    ft = run_step(W, M, k, 0.04, 0.95, d3.ns_cfg(path=d3.PATH_FUSED))
    tt = run_step(W, M, k, 0.04, 0.95, d3.ns_cfg(path=d3.PATH_TILED))
    for a, b, what in zip(ft, tt, ("W", "M", "idx", "O")):
        assert same(a, b), what
    err = check_step(W, M, *ft, k, 0.04, 0.95)
    print(f"{n}x{m} k={k}: fused O rel err {err:.3e}", flush=True)


# W and M as column slices of wider buffers: row stride ld, first column off
# (off > 0 or an odd ld leaves the rows without 16-byte alignment, so the
# update takes its element path)
@pytest.mark.parametrize("n,m,k,ld,off", [(96, 40, 24, 64, 0), (96, 40, 24, 65, 1),
                                          (80, 200, 40, 203, 3), (300, 520, 60, 528, 4)])
def test_fused_step_strided_equals_tiled_bitwise(n, m, k, ld, off):
    say("fused step strided", n, m, k, ld, off)
    W = host_gaussian((n, ld), [47, n, ld], std=0.02)
    M = host_gaussian((n, ld), [48, n, ld])
    outs = []
    for path in (d3.PATH_FUSED, d3.PATH_TILED):
        Wb, Mb = dev(W), dev(M)
        idx, O = d3.step(Wb[:, off:off + m], Mb[:, off:off + m], k, 0.04, 0.95,
                         d3.ns_cfg(path=path), return_idx=True, return_O=True)
        torch.cuda.synchronize()
        outs.append((Wb.cpu().numpy(), Mb.cpu().numpy(), idx.cpu().numpy(), O.cpu().numpy()))
    for a, b, what in zip(outs[0], outs[1], ("W", "M", "idx", "O")):
        assert same(a, b), what
    W1, M1, S, O = outs[0]
    for X0, X1 in ((W, W1), (M, M1)):   # columns outside the slice untouched
        assert same(X0[:, :off], X1[:, :off]) and same(X0[:, off + m:], X1[:, off + m:])
    sl = slice(off, off + m)
    check_step(np.ascontiguousarray(W[:, sl]), np.ascontiguousarray(M[:, sl]),
               np.ascontiguousarray(W1[:, sl]), np.ascontiguousarray(M1[:, sl]), S, O, k, 0.04, 0.95)


@pytest.mark.parametrize("k,m", [(96, 333), (40, 333), (24, 256)])
@pytest.mark.parametrize("iters,restarts", [(5, ()), (5, (2, 4)), (3, (2,)), (7, (3, 6)), (1, ()),
                                            (16, (4, 8, 12, 16))])
def test_fused_schedules(iters, restarts, k, m):
    say("fused schedule", iters, restarts, k, m)
    X = dev(host_gaussian((3, k, m), [42, iters]).astype(np.float16))
    co = [orc.MUON_COEFFS] * iters
    fused = d3.gram_ns(X, d3.ns_cfg(iters=iters, restart_at=restarts, coeffs=co,
                                    path=d3.PATH_FUSED)).cpu().numpy()
    tiled = d3.gram_ns(X, d3.ns_cfg(iters=iters, restart_at=restarts, coeffs=co,
                                    path=d3.PATH_TILED)).cpu().numpy()
    assert same(fused, tiled)
    Xh = X.cpu().numpy()
    if iters <= 7:    # the quintic's fixed point: longer schedules only stay near it
        for b in range(3):
            ref = orc.ns_gram(Xh[b].astype(np.float64), co, restarts)
            assert rel(fused[b], ref) <= O_TOL


def _polar(a):
    u, _, vt = np.linalg.svd(np.asarray(a, np.float64), full_matrices=False)
    return u @ vt


@pytest.mark.parametrize("k,m", [(96, 333), (100, 300), (300, 100)])
def test_long_schedule_without_restart_stays_finite(k, m):
    """Twelve Muon iterations with no restart on a Gram side that pads to
    128: the identity term of the polynomial goes on the real diagonal only,
    so the zero padding block stays zero.  (Added on the padded diagonal too,
    it grew as 3.4445^t, overflowed fp16 after nine iterations and turned the
    cross terms, and then O, into NaN.)  Both paths must agree bit for bit,
    keep the singular values in the band the quintic holds them in (the
    oracle's are in [0.68, 1.14] for these inputs), and keep the polar factor
    of X."""
    say("long schedule", k, m)
    iters = 12
    X = host_gaussian((2, k, m), [43, k, m]).astype(np.float16)
    co = [orc.MUON_COEFFS] * iters
    outs = [d3.gram_ns(dev(X), d3.ns_cfg(iters=iters, restart_at=(), coeffs=co, path=path))
            .cpu().numpy() for path in (d3.PATH_FUSED, d3.PATH_TILED)]
    assert same(outs[0], outs[1])
    O = outs[0].astype(np.float64)
    assert np.isfinite(O).all()
    for b in range(2):
        sv = np.linalg.svd(O[b], compute_uv=False)
        assert 0.6 <= sv.min() and sv.max() <= 1.25, (sv.min(), sv.max())
        assert rel(_polar(O[b]), _polar(X[b])) <= O_TOL


@pytest.mark.parametrize("m", [100, 50, 20])
def test_fused_transposed_gram_ns(m):
    """k > m: the Gram is X^T X and the multiply-back runs along k."""
    say("fused gram_ns k>m", m)
    X = dev(host_gaussian((2, 700, m), 43).astype(np.float16))
    fused = d3.gram_ns(X, d3.ns_cfg(path=d3.PATH_FUSED)).cpu().numpy()
    tiled = d3.gram_ns(X, d3.ns_cfg(path=d3.PATH_TILED)).cpu().numpy()
    assert same(fused, tiled)
    Xh = X.cpu().numpy()
    for b in range(2):
        assert rel(fused[b], orc.ns_gram(Xh[b].astype(np.float64), orc.default_coeffs(), (3,))) <= O_TOL


@pytest.mark.parametrize("k", [100, 60])
def test_fused_restart_on_lowrank(k):
    """Ill-conditioned input: the restart lives inside the fused kernels too."""
    say("fused lowrank", k)
    M = host_lowrank(k, 2048, 44)
    Xn = (M.astype(np.float64) / np.linalg.norm(M.astype(np.float64))).astype(np.float16)
    ref = orc.ns_gram(Xn.astype(np.float64), orc.default_coeffs(), (3,))
    fused = d3.gram_ns(dev(Xn), d3.ns_cfg(path=d3.PATH_FUSED)).cpu().numpy()
    tiled = d3.gram_ns(dev(Xn), d3.ns_cfg(path=d3.PATH_TILED)).cpu().numpy()
    assert same(fused, tiled)
    print(f"lowrank {k}x2048 fused rel err {rel(fused, ref):.3e}", flush=True)
    assert rel(fused, ref) <= O_TOL


def test_fused_megabatch_equals_tiled_bitwise():
    """Many matrices in one launch (one workgroup each)."""
    say("fused megabatch")
    B, n, m, k = 40, 256, 384, 64
    Ws = [host_gaussian((n, m), [45, b], std=0.02) for b in range(B)]
    Ms = [host_gaussian((n, m), [46, b]) for b in range(B)]
    outs = []
    for path in (d3.PATH_FUSED, d3.PATH_TILED):
        Wd, Md = [dev(w) for w in Ws], [dev(x) for x in Ms]
        idx, O = d3.step_megabatch(Wd, Md, k, 0.04, 0.95, d3.ns_cfg(path=path),
                                   return_idx=True, return_O=True)
        torch.cuda.synchronize()
        outs.append(([w.cpu().numpy() for w in Wd], [x.cpu().numpy() for x in Md],
                     idx.cpu().numpy(), O.cpu().numpy()))
    (Wf, Mf, If, Of), (Wt, Mt, It, Ot) = outs
    assert same(If, It) and same(Of, Ot)
    for b in range(B):
        assert same(Wf[b], Wt[b]) and same(Mf[b], Mt[b]), b
    for b in (0, B - 1):
        check_step(Ws[b], Ms[b], Wf[b], Mf[b], If[b], Of[b], k, 0.04, 0.95)


# the 128-padded kernel reads both layouts of X (gather), the one-wave
# kernel only the rows layout (gather_rows)
@pytest.mark.parametrize("k,gather,name", [(75, "gather", "gram_ns_fused_128"),
                                           (64, "gather_rows", "gram_ns_fused_64"),
                                           (32, "gather_rows", "gram_ns_fused_32")])
def test_fused_trace_records_one_launch(k, gather, name):
    say("fused trace", k)
    W = dev(host_gaussian((300, 500), 47, std=0.02))
    M = dev(host_gaussian((300, 500), 48))
    cfg = d3.ns_cfg(path=d3.PATH_FUSED)
    d3.step(W, M, k, 0.04, 0.95, cfg)
    torch.cuda.synchronize()
    d3.trace_enable(64)
    try:
        d3.step(W, M, k, 0.04, 0.95, cfg)
        recs = d3.trace_records()
    finally:
        d3.trace_disable()
    assert [r[0] for r in recs] == ["row_score", "topk", gather, name]
    s_, L_ = float(k), 500.0
    assert recs[3][2] == pytest.approx(6 * s_ * s_ * L_ + 14 * s_ ** 3)
    assert recs[3][1] > 0


@pytest.mark.parametrize("B,k,m", [(512, 32, 256), (256, 64, 512), (2, 32, 8192), (33, 64, 4096)])
def test_auto_path_small_sides_equal_tiled_bitwise(B, k, m):
    """Shapes the automatic rule now sends to the one-wave kernel (many small
    matrices; Gram side 32 with rows up to 8192): bitwise the tiled result."""
    say("auto small sides", B, k, m)
    X = dev(host_gaussian((B, k, m), [49, B, k, m]).astype(np.float16))
    auto = d3.gram_ns(X, d3.ns_cfg()).cpu().numpy()
    tiled = d3.gram_ns(X, d3.ns_cfg(path=d3.PATH_TILED)).cpu().numpy()
    assert same(auto, tiled)
    Xh = X.cpu().numpy()
    for b in (0, B - 1):
        ref = orc.ns_gram(Xh[b].astype(np.float64), orc.default_coeffs(), (3,))
        assert rel(auto[b], ref) <= O_TOL
