"""GPU: the symmetric GEMM entry points on every code path their launches
can take: the 256 tile (at least 512 lower 256-tiles per launch) and the
128 tile; a ragged last tile row (a side that is a multiple of 128 but not
of 256); K below 2048 (columns read from the row-major staging) and from
2048 up (columns restaged column-major); diagonal and off-diagonal tiles.
Each case checks sampled matrices against the fp64 product and every
matrix for exact symmetry (the upper triangle is the mirror of the lower)."""
import sys

import numpy as np
import pytest

from tests.parity import rel
from workloads import host_gaussian

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def dev(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def lower_tiles(side, tile):
    t = (side + tile - 1) // tile
    return t * (t + 1) // 2


def large_tile(tiles, k):
    """The library's tile rule: the 256 tile from 512 tiles of it, or from
    128 when the inner dimension is at least 2048."""
    return tiles >= 512 or (tiles >= 128 and k >= 2048)


# (batch, rows, cols) and the path each case takes:
#   52 x 1024 x 2304: 256 tile (520 lower tiles), K >= 2048
#   35 x 1152 x 1024: 256 tile (525), ragged last tile row, K < 2048
#   2 x 384 x 2560:   128 tile, ragged for the 256 rule, K >= 2048
#   3 x 640 x 640:    128 tile, K < 2048
#   13 x 1024 x 2560: 256 tile by the long-K rule (130 lower tiles, K >= 2048)
SYRK_CASES = [(52, 1024, 2304), (35, 1152, 1024), (2, 384, 2560), (3, 640, 640),
              (13, 1024, 2560)]


@pytest.mark.parametrize("B,rows,cols", SYRK_CASES)
def test_syrk_every_tile_path(B, rows, cols):
    big = large_tile(lower_tiles(rows, 256) * B, cols)
    say("syrk paths", B, rows, cols, "256 tile" if big else "128 tile",
        "K >= 2048" if cols >= 2048 else "K < 2048")
    A = (host_gaussian((B, rows, cols), [60, B, rows, cols]) * 0.03).astype(np.float16)
    R = d3.syrk_f16(dev(A)).cpu().numpy()
    for b in range(B):
        assert np.array_equal(R[b], R[b].T), b
    for b in sorted({0, B // 2, B - 1}):
        A64 = A[b].astype(np.float64)
        assert rel(R[b], A64 @ A64.T) <= 2e-3, b


# (batch, side): 15 x 2048 takes the 256 tile (540 lower tiles) with K = 2048;
# 3 x 2048 the 128 tile with K = 2048 (108 large tiles); 35 x 1152 the 256
# tile, ragged, K < 2048
SYMM_CASES = [(15, 2048), (3, 2048), (35, 1152)]


@pytest.mark.parametrize("B,s", SYMM_CASES)
def test_symm_poly_every_tile_path(B, s):
    big = large_tile(lower_tiles(s, 256) * B, s)
    say("symm poly paths", B, s, "256 tile" if big else "128 tile")
    G = host_gaussian((B, s, s), [61, B, s])
    A = ((G + G.transpose(0, 2, 1)) * (0.5 / np.sqrt(s))).astype(np.float16)   # symmetric
    a, b_, c = 3.4445, -4.7750, 2.0315
    Ad = dev(A)
    C = d3.symm_f16(Ad, Ad, Ad, alpha=c, beta=b_, gamma=a).cpu().numpy()
    P = d3.symm_f16(Ad, Ad).cpu().numpy()
    for i in range(B):
        assert np.array_equal(C[i], C[i].T), i
        assert np.array_equal(P[i], P[i].T), i
    for i in sorted({0, B - 1}):
        Af = A[i].astype(np.float64)
        A2 = Af @ Af
        assert rel(P[i], A2) <= 2e-3, i
        assert rel(C[i], c * A2 + b_ * Af + a * np.eye(s)) <= 2e-3, i


# Gram-NS on the large tile where the Gram side is not a multiple of 256,
# so the last tile row (and, for the multiply-back of a transposed Gram,
# the last tile column) lies partly in the zero padding, whose 32 x 32
# blocks the large tile does not compute.  The same matrices in a launch
# small enough for the 128 tile (which computes every block) must give the
# same bits, and both must match the fp64 oracle.
#   90 x 700 x 1024:  side 700 (6 lower tiles of 256 per matrix, 540 in all)
#   90 x 1100 x 600:  k > m, side 600, rows of length 1100 (multiply-back
#                     N = 1152: a last tile column with 76 real columns)
PAD_CASES = [(90, 700, 1024), (90, 1100, 600)]


@pytest.mark.parametrize("B,k,m", PAD_CASES)
def test_gram_ns_large_tile_padding_blocks(B, k, m):
    from oracle import dion3_oracle as orc
    side = min(k, m)
    assert lower_tiles(side, 256) * B >= 512
    say("gram-ns padding blocks", B, k, m, "side", side)
    X = (host_gaussian((B, k, m), [62, B, k, m]) * 0.05).astype(np.float16)
    tiled = d3.ns_cfg(path=d3.PATH_TILED)
    O = d3.gram_ns(dev(X), tiled).cpu().numpy()
    pick = [0, B // 2, B - 1]
    assert lower_tiles(side, 256) * len(pick) < 512   # the small tile
    O_small = d3.gram_ns(dev(X[pick]), tiled).cpu().numpy()
    for j, b in enumerate(pick):
        assert np.array_equal(O[b].view(np.uint16), O_small[j].view(np.uint16)), b
    co = orc.default_coeffs()
    want = orc.ns_gram(X[0].astype(np.float64), co, (3,))
    assert rel(O[0], want) <= 5e-3
