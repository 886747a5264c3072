"""The allocation-free megabatched step (dion3_step_megabatch_noalloc),
called through the C ABI, against dion3_step_megabatch with a caller
workspace: bitwise equal on two calls in a row, the second on a smaller
input (so the static scratch holds the first call's data when the second
starts); a call that needs more than the static scratch is refused before
any launch."""
import ctypes
import sys

import numpy as np
import pytest

from workloads import host_gaussian

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
import orthogonalizing_optimizer_amd as d3  # noqa: E402

DEV = "cuda:0"


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def inputs(B, n, m, seed):
    Ws = [torch.from_numpy(host_gaussian((n, m), [seed, b, 1], std=0.02)).to(DEV) for b in range(B)]
    Ms = [torch.from_numpy(host_gaussian((n, m), [seed, b, 2])).to(DEV) for b in range(B)]
    return Ws, Ms


def noalloc(Ws, Ms, k, lr, mu, cfg):
    B = len(Ws)
    n, m = Ws[0].shape
    pw, pm = d3.pointer_array(Ws, DEV), d3.pointer_array(Ms, DEV)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    O = torch.empty((B, k, m), dtype=torch.float16, device=DEV)
    st = d3.lib().dion3_step_megabatch_noalloc(pw.data_ptr(), pm.data_ptr(), B, n, m, m, k, lr, mu,
                                               ctypes.byref(cfg), idx.data_ptr(), O.data_ptr(),
                                               torch.cuda.current_stream().cuda_stream)
    assert st == 0, d3.status_string(st)
    return idx, O


def same(a, b):
    return a.cpu().numpy().tobytes() == b.cpu().numpy().tobytes()


# (batch, n, m, k): a tiled Gram side of 300 with the restart, then a smaller
# input whose Gram side takes the fused one-launch path
CASES = [(3, 600, 700, 300), (2, 128, 200, 40)]


def test_noalloc_equals_workspace_call_on_two_calls():
    cfg = d3.default_cfg()
    for i, (B, n, m, k) in enumerate(CASES):
        say("noalloc", B, n, m, k)
        Wa, Ma = inputs(B, n, m, 90 + i)
        Wb, Mb = [w.clone() for w in Wa], [x.clone() for x in Ma]
        ia, Oa = noalloc(Wa, Ma, k, 0.04, 0.95, cfg)
        ib, Ob = d3.step_megabatch(Wb, Mb, k, 0.04, 0.95, cfg, return_idx=True, return_O=True,
                                   ws=d3.Workspace())
        torch.cuda.synchronize()
        assert same(ia, ib) and same(Oa, Ob)
        for x, y in zip(Wa + Ma, Wb + Mb):
            assert same(x, y)


def test_noalloc_refuses_a_call_beyond_the_static_scratch():
    say("noalloc too large")
    Ws, Ms = inputs(1, 64, 96, 95)
    W0, M0 = Ws[0].clone(), Ms[0].clone()
    pw, pm = d3.pointer_array(Ws, DEV), d3.pointer_array(Ms, DEV)
    cfg = d3.default_cfg()
    # 16 x 2048 x 4096 at k = 1024 needs about 600 MB of scratch: refused with
    # DION3_ERR_WORKSPACE before anything runs (the pointers are never read)
    st = d3.lib().dion3_step_megabatch_noalloc(pw.data_ptr(), pm.data_ptr(), 16, 2048, 4096, 4096,
                                               1024, 0.04, 0.95, ctypes.byref(cfg), None, None,
                                               torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert st == -2
    assert same(Ws[0], W0) and same(Ms[0], M0)
