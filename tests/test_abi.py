"""Host-side checks of the C ABI: the library loads, exports every symbol the
header declares, and its host logic (k from f, workspace sizes, argument and
workspace validation) behaves as documented.  No kernel is launched: every
call here fails its checks before the first launch.  CPU only."""
import ctypes
import json
import os
import re
from fractions import Fraction

import pytest

import orthogonalizing_optimizer_amd as d3
from orthogonalizing_optimizer_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dion3.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

ERR_ARG, ERR_WS, ERR_UNSUP = -1, -2, -3
FAKE = 1 << 20           # a non-null, 256-aligned address that is never dereferenced


def declared_symbols():
    txt = open(HEADER).read()
    return sorted(set(re.findall(r"DION3_API\s+[\w\s\*]+?\b(dion3_\w+)\s*\(", txt)))


def test_library_exports_every_declared_symbol():
    lib = d3.lib()
    names = declared_symbols()
    assert len(names) >= 12
    for name in names:
        assert hasattr(lib, name), name
    assert set(names) == set(_lib.EXPORTED)
    assert lib.dion3_version() >= 1


def test_k_from_fraction_golden():
    d = json.load(open(os.path.join(GOLDEN, "k_examples.json")))
    for case in d["cases"]:
        f = float(Fraction(case["f"]))
        assert d3.k_from_fraction(f, case["n"]) == case["k"], case


def test_k_from_fraction_edges():
    lib = d3.lib()
    assert lib.dion3_k_from_fraction(0.25, 0) == -1
    assert lib.dion3_k_from_fraction(0.0, 10) == -1
    assert lib.dion3_k_from_fraction(float("nan"), 10) == -1
    assert lib.dion3_k_from_fraction(1e-30, 10) == 1
    assert lib.dion3_k_from_fraction(2.5, 10) == 10
    assert lib.dion3_k_from_fraction(1 / 3, 3) == 1
    assert lib.dion3_k_from_fraction(1 / 3, 4) == 2
    for n in (1, 7, 100, 13824, 1 << 20):
        for num, den in ((1, 8), (1, 4), (1, 2), (3, 7), (5, 16)):
            want = max(1, min(n, -((-num * n) // den)))
            assert lib.dion3_k_from_fraction(num / den, n) == want


def test_default_cfg():
    cfg = d3.default_cfg()
    assert cfg.iters == 5 and cfg.n_restart == 1 and cfg.restart_at[0] == 3
    assert cfg.method == d3.NS_GRAM and cfg.path == d3.PATH_AUTO
    assert abs(cfg.abc[0][0] - 3.4445) < 1e-6 and abs(cfg.abc[4][2] - 2.0315) < 1e-6
    assert abs(cfg.eps - 1e-7) < 1e-12


def test_workspace_size_layout():
    # padded: kp = mp = 128 and sp = 128; 2 X blocks + 5 Gram-side blocks
    b = d3.workspace_size(1, 128, 100, 32)
    assert b >= 7 * 128 * 128 * 2
    assert d3.workspace_size(4, 128, 100, 32) > 3 * b
    # transposed side (k > m) pads the Gram to m
    assert d3.workspace_size(1, 1000, 64, 900) < d3.workspace_size(1, 1000, 1000, 900)
    with pytest.raises(d3.Dion3Error):
        d3.workspace_size(1, 10, 10, 11)
    with pytest.raises(d3.Dion3Error):
        d3.workspace_size(0, 10, 10, 1)
    out = ctypes.c_size_t()
    assert d3.lib().dion3_workspace_size(1, (1 << 20) + 1, 4, 1, ctypes.byref(out)) == ERR_UNSUP
    assert d3.lib().dion3_workspace_size(1, 10, 10, 0, ctypes.byref(out)) == ERR_ARG
    assert d3.lib().dion3_workspace_size(1, 10, 0, 1, ctypes.byref(out)) == ERR_ARG
    assert d3.lib().dion3_workspace_size(1, (1 << 20) + 1, 4, 0, ctypes.byref(out)) == ERR_ARG
    # padded selected block of 2^31 bytes or more: rejected (32-bit buffer offsets)
    assert d3.lib().dion3_workspace_size(1, 1 << 16, 1 << 15, 1 << 15, ctypes.byref(out)) == ERR_UNSUP
    assert d3.lib().dion3_workspace_size(1, 1 << 16, 1 << 14, 1 << 15, ctypes.byref(out)) == 0
    # a product grid beyond 2^31 - 1 blocks (65408 128-tiles per matrix times 65535 matrices):
    # refused up front, before any kernel could run
    assert d3.lib().dion3_workspace_size(65535, 16384, 65408, 16384, ctypes.byref(out)) == ERR_UNSUP
    assert d3.lib().dion3_workspace_size(1, 16384, 65408, 16384, ctypes.byref(out)) == 0


def _cfg(**kw):
    cfg = d3.default_cfg()
    for k, v in kw.items():
        setattr(cfg, k, v)
    return cfg


def _step(lib, W=FAKE, M=FAKE, n=64, m=32, ld=32, k=16, lr=0.04, mu=0.95, cfg=None, ws=FAKE,
          nbytes=None):
    if nbytes is None:
        nbytes = d3.workspace_size(1, n, m, min(k, n)) if 1 <= k <= n else 1 << 30
    return lib.dion3_step(W, M, n, m, ld, k, lr, mu, ctypes.byref(cfg) if cfg else None, None,
                          None, ws, nbytes, None)


def test_step_rejects_bad_arguments_before_launch():
    lib = d3.lib()
    assert _step(lib, W=None) == ERR_ARG
    assert _step(lib, M=None) == ERR_ARG
    assert _step(lib, k=0) == ERR_ARG
    assert _step(lib, k=-3) == ERR_ARG
    assert _step(lib, k=65) == ERR_ARG
    assert _step(lib, n=0, k=1, nbytes=1 << 30) == ERR_ARG
    assert _step(lib, m=0, ld=8, nbytes=1 << 30) == ERR_ARG
    # a size below 1 or k > n is an argument error even when another size is
    # beyond the library's limit
    assert _step(lib, n=(1 << 20) + 1, k=0) == ERR_ARG
    assert _step(lib, n=(1 << 20) + 1, k=(1 << 20) + 2) == ERR_ARG
    assert _step(lib, n=(1 << 20) + 1, k=4, nbytes=1 << 30) == ERR_UNSUP
    assert _step(lib, ld=31) == ERR_ARG
    assert _step(lib, lr=float("inf")) == ERR_ARG
    assert _step(lib, cfg=_cfg(iters=0)) == ERR_ARG
    assert _step(lib, cfg=_cfg(iters=17)) == ERR_ARG
    bad = _cfg()
    bad.restart_at[0] = 1
    assert _step(lib, cfg=bad) == ERR_ARG
    bad = _cfg()
    bad.restart_at[0] = 6
    assert _step(lib, cfg=bad) == ERR_ARG
    bad = _cfg(n_restart=2)
    bad.restart_at[0], bad.restart_at[1] = 3, 3
    assert _step(lib, cfg=bad) == ERR_ARG
    assert _step(lib, cfg=_cfg(eps=-1.0)) == ERR_ARG
    assert _step(lib, cfg=_cfg(method=2)) == ERR_ARG
    assert _step(lib, cfg=_cfg(path=3)) == ERR_ARG
    assert _step(lib, cfg=_cfg(path=-1)) == ERR_ARG


def test_fused_path_needs_gram_side_of_at_most_128():
    lib = d3.lib()
    fused = _cfg(path=d3.PATH_FUSED)
    # Gram side min(k, m) = 200 pads to 256: refused before any launch
    assert _step(lib, n=400, m=300, ld=300, k=200, cfg=fused) == ERR_UNSUP
    assert _step(lib, n=400, m=200, ld=200, k=300, cfg=fused) == ERR_UNSUP
    # the standard method ignores the path
    std = _cfg(path=d3.PATH_FUSED, method=d3.NS_STANDARD)
    assert _step(lib, n=400, m=300, ld=300, k=200, cfg=std, ws=FAKE + 16) == ERR_WS
    # min(k, m) <= 128 passes the path check and fails later on the workspace
    assert _step(lib, n=400, m=300, ld=300, k=128, cfg=fused, ws=FAKE + 16) == ERR_WS
    assert _step(lib, n=400, m=100, ld=100, k=300, cfg=fused, ws=FAKE + 16) == ERR_WS
    X = FAKE
    assert lib.dion3_gram_ns(X, X, 1, 129, 129, ctypes.byref(fused), FAKE, 1 << 30, None) == ERR_UNSUP


def test_step_rejects_bad_workspace_before_launch():
    lib = d3.lib()
    need = d3.workspace_size(1, 64, 32, 16)
    assert _step(lib, ws=None) == ERR_WS
    assert _step(lib, ws=FAKE + 16) == ERR_WS
    assert _step(lib, nbytes=need - 1) == ERR_WS


def test_other_entry_points_validate():
    lib = d3.lib()
    cfg = None
    assert lib.dion3_step_megabatch(None, FAKE, 2, 8, 8, 8, 2, 0.1, 0.9, cfg, None, None, FAKE,
                                    1 << 30, None) == ERR_ARG
    assert lib.dion3_step_megabatch(FAKE, FAKE, 0, 8, 8, 8, 2, 0.1, 0.9, cfg, None, None, FAKE,
                                    1 << 30, None) == ERR_ARG
    assert lib.dion3_step_accum(FAKE, FAKE, None, 8, 8, 8, 2, 0.1, 0.9, cfg, None, None, FAKE,
                                1 << 30, None) == ERR_ARG
    assert lib.dion3_step_megabatch_accum(FAKE, FAKE, None, 2, 8, 8, 8, 2, 0.1, 0.9, cfg, None,
                                          None, FAKE, 1 << 30, None) == ERR_ARG
    assert lib.dion3_row_select(None, 1, 8, 8, 8, 2, FAKE, None, FAKE, 1 << 30, None) == ERR_ARG
    assert lib.dion3_row_select(FAKE, 1, 8, 8, 8, 9, FAKE, None, FAKE, 1 << 30, None) == ERR_ARG
    assert lib.dion3_row_select(FAKE, 1, 8, 8, 8, 0, FAKE, None, FAKE, 1 << 30, None) == ERR_ARG
    assert lib.dion3_gram_ns(FAKE, FAKE, 1, 0, 8, cfg, FAKE, 1 << 30, None) == ERR_ARG
    assert lib.dion3_gram_ns(FAKE, FAKE, 1, 8, 0, cfg, FAKE, 1 << 30, None) == ERR_ARG
    assert lib.dion3_syrk_f16(FAKE, FAKE, 1, 0, 128, 128, 128, None) == ERR_ARG
    assert lib.dion3_symm_f16(FAKE, FAKE, None, FAKE + 512, 1, 0, 128, 1.0, 0.0, 0.0,
                              None) == ERR_ARG
    assert lib.dion3_row_select(FAKE, 1, 8, 8, 8, 2, FAKE, None, FAKE, 0, None) == ERR_WS
    assert lib.dion3_gram_ns(None, FAKE, 1, 8, 8, cfg, FAKE, 1 << 30, None) == ERR_ARG
    assert lib.dion3_gram_ns(FAKE, FAKE, 1, 8, 8, cfg, FAKE, 16, None) == ERR_WS
    assert lib.dion3_syrk_f16(FAKE, FAKE, 1, 100, 128, 128, 128, None) == ERR_ARG
    assert lib.dion3_syrk_f16(FAKE, FAKE, 1, 128, 128, 120, 128, None) == ERR_ARG
    assert lib.dion3_symm_f16(FAKE, FAKE, None, FAKE + 256, 1, 128, 128, 1.0, 0.5, 0.0,
                              None) == ERR_ARG          # beta != 0 needs D
    assert lib.dion3_symm_f16(FAKE, FAKE + 256, None, FAKE, 1, 128, 128, 1.0, 0.0, 0.0,
                              None) == ERR_ARG          # C aliases A


def test_status_strings():
    for st in (0, -1, -2, -3, -4):
        assert d3.status_string(st)
    assert d3.status_string(7) == "unknown status"


def test_binding_refuses_cpu_tensors():
    import torch
    with pytest.raises(TypeError):
        d3.step(torch.zeros(4, 4), torch.zeros(4, 4), 2, 0.1, 0.9)
    with pytest.raises(TypeError):
        d3.gram_ns(torch.zeros(4, 4, dtype=torch.float16))


def test_binding_struct_matches_library():
    assert d3.lib().dion3_ns_cfg_size() == ctypes.sizeof(d3.NsCfg)


def test_dion3step_rejects_mismatched_strides_before_any_device_work():
    torch = pytest.importorskip("torch")
    W = torch.zeros(4, 6)
    M = torch.zeros(6, 4).t()          # same shape, column-major strides
    with pytest.raises(ValueError):
        d3.Dion3Step([W], [M])


def test_dion3_optimizer_refuses_what_it_cannot_step():
    torch = pytest.importorskip("torch")
    with pytest.raises(ValueError):
        d3.Dion3([torch.nn.Parameter(torch.zeros(4))])              # not a matrix
    with pytest.raises(ValueError):
        d3.Dion3([torch.nn.Parameter(torch.zeros(4, 6, dtype=torch.float64))])
    with pytest.raises(ValueError):
        d3.Dion3([torch.nn.Parameter(torch.zeros(6, 4).t())])       # columns contiguous
    with pytest.raises(ValueError):
        d3.Dion3([torch.nn.Parameter(torch.zeros(4, 6))], fraction=0.0)
    p = torch.nn.Parameter(torch.zeros(4, 6))
    opt = d3.Dion3([p])
    p.grad = torch.ones(4, 6)
    with pytest.raises(TypeError):                                  # host tensors: no CPU path
        opt.step()


def test_norm_step_rejects_bad_arguments_before_launch():
    lib = d3.lib()
    nb = d3.workspace_size(1, 64, 32, 16)
    good = d3.NormCfg(0.95, 1e-8)

    def call(V=FAKE, norm=good):
        return lib.dion3_step_megabatch_norm(FAKE, FAKE, None, V, 1, 64, 32, 32, 16, 0.04, 0.95,
                                             None, ctypes.byref(norm) if norm else None, None,
                                             None, FAKE, nb, None)
    assert call(V=None) == ERR_ARG
    assert call(norm=None) == ERR_ARG
    assert call(norm=d3.NormCfg(1.0, 1e-8)) == ERR_ARG
    assert call(norm=d3.NormCfg(-0.1, 1e-8)) == ERR_ARG
    assert call(norm=d3.NormCfg(0.9, -1.0)) == ERR_ARG
    assert call(norm=d3.NormCfg(0.9, float("nan"))) == ERR_ARG
    # valid normalization arguments pass on to the workspace check
    assert lib.dion3_step_megabatch_norm(FAKE, FAKE, None, FAKE, 1, 64, 32, 32, 16, 0.04, 0.95,
                                         None, ctypes.byref(good), None, None, FAKE + 16, nb,
                                         None) == ERR_WS


def test_header_compiles_as_c99_and_host_calls_work_from_c(tmp_path):
    """The ABI from plain C: gcc -std=c99 -Wall -Werror against include/dion3.h,
    linked to the built library, host-only calls (no device work)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    pkg = os.path.join(ROOT, "orthogonalizing_optimizer_amd")
    exe = str(tmp_path / "abi_check")
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_check.c"), "-o", exe, "-L", pkg, "-ldion3",
           "-Wl,-rpath," + pkg, "-lm"]
    subprocess.run(cmd, check=True)
    out = subprocess.run([exe], check=True, capture_output=True, text=True)
    assert "c abi ok" in out.stdout


def _groups(*specs, W=FAKE, M=FAKE, G=None, V=None, ld=None, lr=0.04):
    """dion3_group array from (batch, n, m, k) tuples; pointers are fake."""
    arr = (_lib.GroupDesc * len(specs))()
    for i, (b, n, m, k) in enumerate(specs):
        arr[i] = _lib.GroupDesc(W, M, G, V, n, m, ld if ld is not None else m, k, b, lr, None, None)
    return arr


def _ws_groups(arr, cfg=None):
    out = ctypes.c_size_t(0)
    st = d3.lib().dion3_workspace_size_groups(arr, len(arr), ctypes.byref(cfg) if cfg else None,
                                              ctypes.byref(out))
    return st, out.value


def test_group_workspace_shares_gram_sides():
    lib = d3.lib()
    tiled = _cfg(path=d3.PATH_TILED)
    # 7B-like shapes at f = 1/4: the attention (k = 1024) and down-projection
    # (k = 1024) groups share the Gram side 1024, the up-projection (k = 2752)
    # has its own
    spec = [(128, 4096, 4096, 1024), (64, 11008, 4096, 2752), (32, 4096, 11008, 1024)]
    st, grouped = _ws_groups(_groups(*spec), tiled)
    assert st == 0
    singles = sum(d3.workspace_size(*s) for s in spec)
    # one side set per Gram side: the same Gram-side bytes, only alignment differs
    assert abs(grouped - singles) <= 64 * 1024
    # a group whose Gram side pads to 128 takes the fused path under AUTO and
    # needs no Gram-side buffers at all
    st, fused = _ws_groups(_groups((64, 512, 1024, 128)), _cfg())
    st2, tiled_one = _ws_groups(_groups((64, 512, 1024, 128)), tiled)
    assert st == 0 and st2 == 0
    assert tiled_one - fused >= 5 * 64 * 128 * 128 * 2
    assert tiled_one == d3.workspace_size(64, 512, 1024, 128)


def test_step_groups_rejects_bad_arguments_before_launch():
    lib = d3.lib()
    ok = _groups((2, 64, 32, 16), (3, 96, 32, 16))
    st, need = _ws_groups(ok)
    assert st == 0 and need > 0

    def call(arr, n=None, mu=0.95, cfg=None, norm=None, ws=FAKE, nbytes=None):
        return lib.dion3_step_groups(arr, len(arr) if n is None else n, mu,
                                     ctypes.byref(cfg) if cfg else None,
                                     ctypes.byref(norm) if norm else None, ws,
                                     need if nbytes is None else nbytes, None)

    assert lib.dion3_step_groups(None, 1, 0.95, None, None, FAKE, need, None) == ERR_ARG
    assert call(ok, n=0) == ERR_ARG
    assert call(ok, n=65) == ERR_ARG
    assert call(ok, mu=float("nan")) == ERR_ARG
    assert call(_groups((2, 64, 32, 16), W=None)) == ERR_ARG
    assert call(_groups((2, 64, 32, 16), M=None)) == ERR_ARG
    assert call(_groups((2, 64, 32, 16), lr=float("inf"))) == ERR_ARG
    assert call(_groups((0, 64, 32, 16))) == ERR_ARG
    assert call(_groups((2, 64, 32, 0), (2, 64, 32, 16))) == ERR_ARG
    assert call(_groups((2, 64, 32, 16), (2, 64, 32, 65))) == ERR_ARG
    assert call(_groups((2, 64, 32, 16), ld=31)) == ERR_ARG
    # an argument error in a later group wins over an unsupported size in an
    # earlier one
    assert call(_groups((2, (1 << 20) + 1, 4, 1), (2, 8, 8, 0)), nbytes=1 << 30) == ERR_ARG
    assert call(_groups((2, (1 << 20) + 1, 4, 1)), nbytes=1 << 30) == ERR_UNSUP
    assert call(ok, cfg=_cfg(iters=0)) == ERR_ARG
    assert call(ok, norm=d3.NormCfg(0.9, 1e-8)) == ERR_ARG          # no states V
    assert call(_groups((2, 64, 32, 16), V=FAKE), norm=d3.NormCfg(1.0, 1e-8)) == ERR_ARG
    fused = _cfg(path=d3.PATH_FUSED)
    assert call(_groups((2, 400, 300, 200)), cfg=fused, nbytes=1 << 30) == ERR_UNSUP
    assert call(ok, ws=None) == ERR_WS
    assert call(ok, ws=FAKE + 16) == ERR_WS
    assert call(ok, nbytes=need - 1) == ERR_WS
    st, _ = _ws_groups(_groups((2, 64, 32, 16), (2, 64, 32, 0)))
    assert st == ERR_ARG
    assert lib.dion3_workspace_size_groups(ok, len(ok), None, None) == ERR_ARG


def test_group_struct_matches_binding():
    assert d3.lib().dion3_group_size() == ctypes.sizeof(_lib.GroupDesc)


def test_noalloc_refuses_before_any_device_work():
    lib = d3.lib()
    assert lib.dion3_step_megabatch_noalloc(None, FAKE, 1, 64, 32, 32, 16, 0.04, 0.95, None, None,
                                            None, None) == ERR_ARG
    assert lib.dion3_step_megabatch_noalloc(FAKE, FAKE, 1, 64, 32, 32, 0, 0.04, 0.95, None, None,
                                            None, None) == ERR_ARG
    # more than DION3_STATIC_SCRATCH_BYTES of workspace
    need = d3.workspace_size(16, 2048, 4096, 1024)
    assert need > (64 << 20)
    assert lib.dion3_step_megabatch_noalloc(FAKE, FAKE, 16, 2048, 4096, 4096, 1024, 0.04, 0.95,
                                            None, None, None, None) == ERR_WS
