"""ctypes binding of libdion3.so: argument marshalling only.

Every step of the optimizer runs in the library's HIP kernels; this module
turns torch tensors into device pointers, picks torch's current stream and
keeps a workspace tensor.  If the library is missing it raises: there is no
fallback path.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional, Sequence, Tuple

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libdion3.so")

DION3_OK = 0
MAX_ITERS = 16
MAX_RESTARTS = 4
STATUS = {0: "ok", -1: "invalid argument", -2: "workspace missing, misaligned or too small",
          -3: "shape beyond the library's limits", -4: "HIP call or kernel launch failed"}

MUON_ABC = (3.4445, -4.7750, 2.0315)


class Dion3Error(RuntimeError):
    def __init__(self, status: int, where: str, hip_error: int = 0):
        msg = f"{where}: {STATUS.get(status, 'unknown status')} (status {status}"
        if status == -4:
            msg += f", hipError {hip_error}"
        super().__init__(msg + ")")
        self.status = status
        self.hip_error = hip_error


class NsCfg(ctypes.Structure):
    """Mirror of dion3_ns_cfg."""
    _fields_ = [("iters", ctypes.c_int32), ("n_restart", ctypes.c_int32),
                ("restart_at", ctypes.c_int32 * MAX_RESTARTS),
                ("abc", (ctypes.c_float * 3) * MAX_ITERS), ("eps", ctypes.c_float),
                ("method", ctypes.c_int32), ("path", ctypes.c_int32)]


class NormCfg(ctypes.Structure):
    """Mirror of dion3_norm_cfg (per-neuron normalization of the update)."""
    _fields_ = [("beta2", ctypes.c_float), ("eps", ctypes.c_float)]


class GroupDesc(ctypes.Structure):
    """Mirror of dion3_group (one shape group of a grouped step)."""
    _fields_ = [("W", ctypes.c_void_p), ("M", ctypes.c_void_p), ("G", ctypes.c_void_p),
                ("V", ctypes.c_void_p), ("n", ctypes.c_int64), ("m", ctypes.c_int64),
                ("ld", ctypes.c_int64), ("k", ctypes.c_int64), ("batch", ctypes.c_int32),
                ("lr", ctypes.c_float), ("idx_out", ctypes.c_void_p), ("O_out", ctypes.c_void_p)]


MAX_GROUPS = 64
NS_GRAM = 0
NS_STANDARD = 1
PATH_AUTO = 0
PATH_TILED = 1
PATH_FUSED = 2


_lib = None


def _declare(lib):
    c = ctypes
    vp, i32, i64, f32, f64, sz = c.c_void_p, c.c_int32, c.c_int64, c.c_float, c.c_double, c.c_size_t
    sig = {
        "dion3_version": (c.c_int, []),
        "dion3_ns_cfg_size": (sz, []),
        "dion3_ns_cfg_default": (None, [c.POINTER(NsCfg)]),
        "dion3_k_from_fraction": (i64, [f64, i64]),
        "dion3_workspace_size": (c.c_int, [i32, i64, i64, i64, c.POINTER(sz)]),
        "dion3_row_select": (c.c_int, [vp, i32, i64, i64, i64, i64, vp, vp, vp, sz, vp]),
        "dion3_gram_ns": (c.c_int, [vp, vp, i32, i64, i64, c.POINTER(NsCfg), vp, sz, vp]),
        "dion3_step": (c.c_int, [vp, vp, i64, i64, i64, i64, f32, f32, c.POINTER(NsCfg), vp, vp,
                                 vp, sz, vp]),
        "dion3_step_megabatch": (c.c_int, [vp, vp, i32, i64, i64, i64, i64, f32, f32,
                                           c.POINTER(NsCfg), vp, vp, vp, sz, vp]),
        "dion3_step_accum": (c.c_int, [vp, vp, vp, i64, i64, i64, i64, f32, f32,
                                       c.POINTER(NsCfg), vp, vp, vp, sz, vp]),
        "dion3_step_megabatch_accum": (c.c_int, [vp, vp, vp, i32, i64, i64, i64, i64, f32, f32,
                                                 c.POINTER(NsCfg), vp, vp, vp, sz, vp]),
        "dion3_step_megabatch_norm": (c.c_int, [vp, vp, vp, vp, i32, i64, i64, i64, i64, f32, f32,
                                                c.POINTER(NsCfg), c.POINTER(NormCfg), vp, vp, vp,
                                                sz, vp]),
        "dion3_group_size": (sz, []),
        "dion3_workspace_size_groups": (c.c_int, [c.POINTER(GroupDesc), i32, c.POINTER(NsCfg),
                                                  c.POINTER(sz)]),
        "dion3_step_groups": (c.c_int, [c.POINTER(GroupDesc), i32, f32, c.POINTER(NsCfg),
                                        c.POINTER(NormCfg), vp, sz, vp]),
        "dion3_step_megabatch_noalloc": (c.c_int, [vp, vp, i32, i64, i64, i64, i64, f32, f32,
                                                   c.POINTER(NsCfg), vp, vp, vp]),
        "dion3_syrk_f16": (c.c_int, [vp, vp, i32, i64, i64, i64, i64, vp]),
        "dion3_symm_f16": (c.c_int, [vp, vp, vp, vp, i32, i64, i64, f32, f32, f32, vp]),
        "dion3_trace_enable": (c.c_int, [i32]),
        "dion3_trace_count": (i32, []),
        "dion3_trace_reset": (None, []),
        "dion3_trace_record": (c.c_int, [i32, c.POINTER(c.c_char_p), c.POINTER(f64),
                                         c.POINTER(f64), c.POINTER(f64)]),
        "dion3_status_string": (c.c_char_p, [c.c_int]),
        "dion3_last_hip_error": (c.c_int, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


EXPORTED = ("dion3_version", "dion3_ns_cfg_size", "dion3_ns_cfg_default", "dion3_k_from_fraction",
            "dion3_workspace_size", "dion3_row_select", "dion3_gram_ns", "dion3_step",
            "dion3_step_megabatch", "dion3_step_accum", "dion3_step_megabatch_accum",
            "dion3_step_megabatch_norm", "dion3_group_size", "dion3_workspace_size_groups",
            "dion3_step_groups", "dion3_step_megabatch_noalloc",
            "dion3_syrk_f16", "dion3_symm_f16", "dion3_trace_enable",
            "dion3_trace_count", "dion3_trace_reset", "dion3_trace_record", "dion3_status_string",
            "dion3_last_hip_error")


def lib():
    """Load libdion3.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it with "
                              "`python -m orthogonalizing_optimizer_amd.build`")
        loaded = _declare(ctypes.CDLL(LIB_PATH))
        if loaded.dion3_ns_cfg_size() != ctypes.sizeof(NsCfg):
            raise ImportError(f"{LIB_PATH}: dion3_ns_cfg is {loaded.dion3_ns_cfg_size()} bytes, "
                              f"the binding's NsCfg {ctypes.sizeof(NsCfg)}: rebuild the library")
        if loaded.dion3_group_size() != ctypes.sizeof(GroupDesc):
            raise ImportError(f"{LIB_PATH}: dion3_group is {loaded.dion3_group_size()} bytes, "
                              f"the binding's GroupDesc {ctypes.sizeof(GroupDesc)}: rebuild the "
                              "library")
        _lib = loaded
    return _lib


def _check(status: int, where: str):
    if status != DION3_OK:
        raise Dion3Error(status, where, lib().dion3_last_hip_error() if status == -4 else 0)


# ------------------------------------------------------------- host-only API

def ns_cfg(iters: int = 5, restart_at: Sequence[int] = (3,),
           coeffs: Optional[Sequence[Tuple[float, float, float]]] = None,
           eps: float = 1e-7, method: int = NS_GRAM, path: int = PATH_AUTO) -> NsCfg:
    """Build a dion3_ns_cfg (validated by the library at call time).
    method: NS_GRAM (Gram Newton-Schulz) or NS_STANDARD (iteration on X).
    path: PATH_AUTO, PATH_TILED (one product per launch) or PATH_FUSED (the
    whole iteration in one launch; Gram side min(k, m) <= 128 only)."""
    cfg = NsCfg()
    lib().dion3_ns_cfg_default(ctypes.byref(cfg))
    cfg.method = method
    cfg.path = path
    if len(restart_at) > MAX_RESTARTS or iters > MAX_ITERS:
        raise ValueError("too many restarts or iterations")
    cfg.iters = iters
    cfg.n_restart = len(restart_at)
    for i, r in enumerate(restart_at):
        cfg.restart_at[i] = int(r)
    if coeffs is not None:
        if len(coeffs) != iters:
            raise ValueError("need one (a, b, c) per iteration")
        for t, (a, b, c) in enumerate(coeffs):
            cfg.abc[t][0], cfg.abc[t][1], cfg.abc[t][2] = a, b, c
    cfg.eps = eps
    return cfg


def default_cfg() -> NsCfg:
    cfg = NsCfg()
    lib().dion3_ns_cfg_default(ctypes.byref(cfg))
    return cfg


def k_from_fraction(f: float, n: int) -> int:
    k = lib().dion3_k_from_fraction(float(f), int(n))
    if k < 0:
        raise ValueError("invalid fraction or n")
    return int(k)


def workspace_size(batch: int, n: int, m: int, k: int) -> int:
    out = ctypes.c_size_t(0)
    _check(lib().dion3_workspace_size(batch, n, m, k, ctypes.byref(out)), "dion3_workspace_size")
    return int(out.value)


def status_string(status: int) -> str:
    return lib().dion3_status_string(status).decode()


# ------------------------------------------------------------- device API

def _torch():
    import torch
    return torch


def _stream(device) -> int:
    torch = _torch()
    return torch.cuda.current_stream(device).cuda_stream


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


class Workspace:
    """A reusable device workspace (a uint8 torch tensor, 256-byte aligned)."""

    def __init__(self):
        self.buf = None

    def get(self, nbytes: int, device):
        torch = _torch()
        if self.buf is None or self.buf.numel() < nbytes or self.buf.device != torch.device(device):
            self.buf = torch.empty(max(nbytes, 256) + 256, dtype=torch.uint8, device=device)
        base = self.buf.data_ptr()
        off = (-base) % 256
        return base + off, self.buf.numel() - off


# Default workspaces, one per (device, stream): calls on different streams
# never share scratch memory.  Each is kept (and grown as needed) until the
# process ends; pass ``ws`` to manage the memory yourself.
_default_ws: dict = {}


def _ws_for(ws: Optional[Workspace], device) -> Workspace:
    if ws is not None:
        return ws
    torch = _torch()
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    w = _default_ws.get(key)
    if w is None:
        w = _default_ws[key] = Workspace()
    return w


def _req(t, dtype, name):
    torch = _torch()
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")


def row_select(M, k: int, return_scores: bool = False, ws: Optional[Workspace] = None):
    """Top-k l1 rows of M ([n, m] or [batch, n, m] fp32, rows contiguous)."""
    torch = _torch()
    _req(M, torch.float32, "M")
    Mb = M.unsqueeze(0) if M.dim() == 2 else M
    if Mb.dim() != 3 or Mb.stride(2) != 1 or Mb.stride(0) != Mb.shape[1] * Mb.stride(1):
        raise ValueError("M must be [n, m] or [batch, n, m] with contiguous rows")
    B, n, m = Mb.shape
    ld = Mb.stride(1)
    idx = torch.empty((B, k), dtype=torch.int32, device=M.device)
    scores = torch.empty((B, n), dtype=torch.float64, device=M.device) if return_scores else None
    p, nb = _ws_for(ws, M.device).get(workspace_size(B, n, m, k), M.device)
    _check(lib().dion3_row_select(Mb.data_ptr(), B, n, m, ld, k, idx.data_ptr(), _ptr(scores), p,
                                  nb, _stream(M.device)), "dion3_row_select")
    if M.dim() == 2:
        idx = idx[0]
        scores = scores[0] if scores is not None else None
    return (idx, scores) if return_scores else idx


def gram_ns(X, cfg: Optional[NsCfg] = None, ws: Optional[Workspace] = None):
    """Gram Newton-Schulz of X ([k, m] or [batch, k, m] fp16, contiguous)."""
    torch = _torch()
    _req(X, torch.float16, "X")
    if not X.is_contiguous():
        raise ValueError("X must be contiguous")
    Xb = X.unsqueeze(0) if X.dim() == 2 else X
    B, k, m = Xb.shape
    O = torch.empty_like(Xb)
    p, nb = _ws_for(ws, X.device).get(workspace_size(B, k, m, k), X.device)
    _check(lib().dion3_gram_ns(Xb.data_ptr(), O.data_ptr(), B, k, m,
                               ctypes.byref(cfg) if cfg is not None else None, p, nb,
                               _stream(X.device)), "dion3_gram_ns")
    return O[0] if X.dim() == 2 else O


def step(W, M, k: int, lr: float, mu: float, cfg: Optional[NsCfg] = None,
         return_idx: bool = False, return_O: bool = False, ws: Optional[Workspace] = None,
         G=None, norm=None):
    """One Dion3 step on one matrix, in place on W and M (fp32, [n, m]).
    With G (same shape and strides as M), M <- M + G first, fused into the
    row scoring.  With norm = (V, beta2, eps) (V: fp32 [n] state, updated in
    place) the update is normalized per neuron, through the megabatch entry
    point with one matrix."""
    torch = _torch()
    if norm is not None:
        V, beta2, eps = norm
        idx, O = step_megabatch([W], [M], k, lr, mu, cfg, return_idx, return_O, ws,
                                Gs=None if G is None else [G], norm=([V], beta2, eps))
        return (idx[0] if idx is not None else None), (O[0] if O is not None else None)
    _req(W, torch.float32, "W")
    _req(M, torch.float32, "M")
    if W.shape != M.shape or W.dim() != 2 or W.stride() != M.stride() or W.stride(1) != 1:
        raise ValueError("W and M must be [n, m] with equal strides and contiguous rows")
    if G is not None:
        _req(G, torch.float32, "G")
        if G.shape != M.shape or G.stride() != M.stride():
            raise ValueError("G must have the shape and strides of M")
    n, m = M.shape
    idx = torch.empty(k, dtype=torch.int32, device=M.device) if return_idx else None
    O = torch.empty((k, m), dtype=torch.float16, device=M.device) if return_O else None
    p, nb = _ws_for(ws, M.device).get(workspace_size(1, n, m, k), M.device)
    c = ctypes.byref(cfg) if cfg is not None else None
    if G is None:
        _check(lib().dion3_step(W.data_ptr(), M.data_ptr(), n, m, M.stride(0), k, lr, mu, c,
                                _ptr(idx), _ptr(O), p, nb, _stream(M.device)), "dion3_step")
    else:
        _check(lib().dion3_step_accum(W.data_ptr(), M.data_ptr(), G.data_ptr(), n, m, M.stride(0),
                                      k, lr, mu, c, _ptr(idx), _ptr(O), p, nb,
                                      _stream(M.device)), "dion3_step_accum")
    return idx, O


def pointer_array(tensors, device):
    """Device array of the tensors' data pointers (int64)."""
    torch = _torch()
    return torch.tensor([t.data_ptr() for t in tensors], dtype=torch.int64).to(device)


def step_megabatch(Ws, Ms, k: int, lr: float, mu: float, cfg: Optional[NsCfg] = None,
                   return_idx: bool = False, return_O: bool = False,
                   ws: Optional[Workspace] = None, ptrs=None, Gs=None, gptrs=None, norm=None,
                   vptrs=None):
    """One Dion3 step on a group of same-shape matrices in one call.
    ``ptrs`` may carry cached (W pointer array, M pointer array).  With
    gradients ``Gs`` (or their cached pointer array ``gptrs``), each M <- M + G
    first, fused into the row scoring.  With ``norm = (Vs, beta2, eps)`` the
    update is normalized per neuron (Vs: one fp32 [n] state per matrix,
    updated in place; ``vptrs`` may carry their cached pointer array)."""
    torch = _torch()
    if len(Ws) != len(Ms) or not Ws:
        raise ValueError("need equally many W and M matrices")
    if Gs is not None and len(Gs) != len(Ms):
        raise ValueError("need one gradient per matrix")
    shape, stride = Ms[0].shape, Ms[0].stride()
    for t in list(Ws) + list(Ms) + list(Gs or []):
        _req(t, torch.float32, "W/M")
        if t.shape != shape or t.stride() != stride or t.dim() != 2 or t.stride(1) != 1:
            raise ValueError("all matrices must share shape and strides with contiguous rows")
    dev = Ms[0].device
    B = len(Ms)
    n, m = shape
    if ptrs is None:
        ptrs = (pointer_array(Ws, dev), pointer_array(Ms, dev))
    idx = torch.empty((B, k), dtype=torch.int32, device=dev) if return_idx else None
    O = torch.empty((B, k, m), dtype=torch.float16, device=dev) if return_O else None
    p, nb = _ws_for(ws, dev).get(workspace_size(B, n, m, k), dev)
    c = ctypes.byref(cfg) if cfg is not None else None
    if norm is not None:
        Vs, beta2, eps = norm
        if len(Vs) != B:
            raise ValueError("need one state vector per matrix")
        for v in Vs:
            _req(v, torch.float32, "V")
            if v.dim() != 1 or v.shape[0] != n or v.stride(0) != 1:
                raise ValueError("each state must be a contiguous fp32 vector of n entries")
        if vptrs is None:
            vptrs = pointer_array(Vs, dev)
        if Gs is not None and gptrs is None:
            gptrs = pointer_array(Gs, dev)
        nc = NormCfg(float(beta2), float(eps))
        _check(lib().dion3_step_megabatch_norm(
            ptrs[0].data_ptr(), ptrs[1].data_ptr(), gptrs.data_ptr() if gptrs is not None else None,
            vptrs.data_ptr(), B, n, m, stride[0], k, lr, mu, c, ctypes.byref(nc), _ptr(idx), _ptr(O),
            p, nb, _stream(dev)), "dion3_step_megabatch_norm")
    elif Gs is None and gptrs is None:
        _check(lib().dion3_step_megabatch(ptrs[0].data_ptr(), ptrs[1].data_ptr(), B, n, m, stride[0],
                                          k, lr, mu, c, _ptr(idx), _ptr(O), p, nb, _stream(dev)),
               "dion3_step_megabatch")
    else:
        if gptrs is None:
            gptrs = pointer_array(Gs, dev)
        _check(lib().dion3_step_megabatch_accum(ptrs[0].data_ptr(), ptrs[1].data_ptr(),
                                                gptrs.data_ptr(), B, n, m, stride[0], k, lr, mu, c,
                                                _ptr(idx), _ptr(O), p, nb, _stream(dev)),
               "dion3_step_megabatch_accum")
    return idx, O


class Group:
    """One shape group of a grouped step: same-shape fp32 matrices W and M
    (contiguous rows, equal strides), k selected rows each, step size lr.
    Optional: gradients Gs (accumulated first) and per-neuron states Vs (fp32
    [n] each).  The device pointer arrays are built once and kept; build a
    new Group if the tensors change."""

    def __init__(self, Ws, Ms, k: int, lr: float, Gs=None, Vs=None):
        torch = _torch()
        if len(Ws) != len(Ms) or not Ws:
            raise ValueError("need equally many W and M matrices")
        if Gs is not None and len(Gs) != len(Ms):
            raise ValueError("need one gradient per matrix")
        if Vs is not None and len(Vs) != len(Ms):
            raise ValueError("need one state vector per matrix")
        shape, stride = Ms[0].shape, Ms[0].stride()
        for t in list(Ws) + list(Ms) + list(Gs or []):
            _req(t, torch.float32, "W/M/G")
            if t.shape != shape or t.stride() != stride or t.dim() != 2 or t.stride(1) != 1:
                raise ValueError("all matrices must share shape and strides with contiguous rows")
        self.n, self.m = shape
        for v in Vs or []:
            _req(v, torch.float32, "V")
            if v.dim() != 1 or v.shape[0] != self.n or v.stride(0) != 1:
                raise ValueError("each state must be a contiguous fp32 vector of n entries")
        self.device = Ms[0].device
        self.Ws, self.Ms, self.Gs, self.Vs = list(Ws), list(Ms), Gs, Vs
        self.k, self.lr, self.ld, self.batch = int(k), float(lr), stride[0], len(Ms)
        self.ptrs = (pointer_array(Ws, self.device), pointer_array(Ms, self.device))
        self.gptrs = pointer_array(Gs, self.device) if Gs is not None else None
        self.vptrs = pointer_array(Vs, self.device) if Vs is not None else None

    def desc(self, idx=None, O=None) -> GroupDesc:
        return GroupDesc(self.ptrs[0].data_ptr(), self.ptrs[1].data_ptr(),
                         self.gptrs.data_ptr() if self.gptrs is not None else None,
                         self.vptrs.data_ptr() if self.vptrs is not None else None,
                         self.n, self.m, self.ld, self.k, self.batch, self.lr, _ptr(idx), _ptr(O))


def workspace_size_groups(groups: Sequence[Group], cfg: Optional[NsCfg] = None) -> int:
    arr = (GroupDesc * len(groups))(*[g.desc() for g in groups])
    out = ctypes.c_size_t(0)
    _check(lib().dion3_workspace_size_groups(arr, len(groups),
                                             ctypes.byref(cfg) if cfg is not None else None,
                                             ctypes.byref(out)), "dion3_workspace_size_groups")
    return int(out.value)


def step_groups(groups: Sequence[Group], mu: float, cfg: Optional[NsCfg] = None, norm=None,
                return_idx: bool = False, return_O: bool = False,
                ws: Optional[Workspace] = None):
    """One Dion3 step over several shape groups in one call (each s x s
    product is one launch over all groups' Gram-side sets, each Gram one
    launch over all groups).  norm: None or
    (beta2, eps), with every group carrying its states Vs.  Returns one
    (idx, O) pair per group (None unless asked for)."""
    torch = _torch()
    if not groups:
        raise ValueError("need at least one group")
    dev = groups[0].device
    if any(g.device != dev for g in groups):
        raise ValueError("all groups must be on one device")
    if norm is not None and any(g.vptrs is None for g in groups):
        raise ValueError("the normalized step needs the states Vs of every group")
    outs = []
    for g in groups:
        idx = torch.empty((g.batch, g.k), dtype=torch.int32, device=dev) if return_idx else None
        O = torch.empty((g.batch, g.k, g.m), dtype=torch.float16, device=dev) if return_O else None
        outs.append((idx, O))
    arr = (GroupDesc * len(groups))(*[g.desc(i, o) for g, (i, o) in zip(groups, outs)])
    c = ctypes.byref(cfg) if cfg is not None else None
    need = ctypes.c_size_t(0)
    _check(lib().dion3_workspace_size_groups(arr, len(groups), c, ctypes.byref(need)),
           "dion3_workspace_size_groups")
    p, nb = _ws_for(ws, dev).get(int(need.value), dev)
    nc = NormCfg(float(norm[0]), float(norm[1])) if norm is not None else None
    _check(lib().dion3_step_groups(arr, len(groups), float(mu), c,
                                   ctypes.byref(nc) if nc is not None else None, p, nb,
                                   _stream(dev)), "dion3_step_groups")
    return outs


def syrk_f16(A):
    """R = A A^T for fp16 A ([rows, cols] or [batch, rows, cols], both multiples of 128)."""
    torch = _torch()
    _req(A, torch.float16, "A")
    Ab = A.unsqueeze(0) if A.dim() == 2 else A
    if not Ab.is_contiguous():
        raise ValueError("A must be contiguous")
    B, r, c = Ab.shape
    R = torch.empty((B, r, r), dtype=torch.float16, device=A.device)
    _check(lib().dion3_syrk_f16(Ab.data_ptr(), R.data_ptr(), B, r, c, c, r, _stream(A.device)),
           "dion3_syrk_f16")
    return R[0] if A.dim() == 2 else R


def symm_f16(A, B, D=None, alpha: float = 1.0, beta: float = 0.0, gamma: float = 0.0):
    """C = alpha A B + beta D + gamma I for symmetric commuting fp16 A, B."""
    torch = _torch()
    for t, nm in ((A, "A"), (B, "B")):
        _req(t, torch.float16, nm)
    Ab = A.unsqueeze(0) if A.dim() == 2 else A
    Bb = B.unsqueeze(0) if B.dim() == 2 else B
    Db = None if D is None else (D.unsqueeze(0) if D.dim() == 2 else D)
    for t in (Ab, Bb) + ((Db,) if Db is not None else ()):
        if not t.is_contiguous() or t.shape != Ab.shape:
            raise ValueError("A, B, D must be contiguous and of one shape")
    nb, s, _ = Ab.shape
    C = torch.empty_like(Ab)
    _check(lib().dion3_symm_f16(Ab.data_ptr(), Bb.data_ptr(), _ptr(Db), C.data_ptr(), nb, s, s,
                                alpha, beta, gamma, _stream(A.device)), "dion3_symm_f16")
    return C[0] if A.dim() == 2 else C


# ------------------------------------------------------------- timing trace

def trace_enable(capacity: int):
    """Start recording an event pair around every kernel the library launches."""
    _check(lib().dion3_trace_enable(int(capacity)), "dion3_trace_enable")


def trace_disable():
    _check(lib().dion3_trace_enable(0), "dion3_trace_enable")


def trace_reset():
    lib().dion3_trace_reset()


def trace_records():
    """[(kernel name, ms, algorithmic flops, algorithmic bytes)] in launch order
    (waits for the recorded kernels to finish)."""
    out = []
    name = ctypes.c_char_p()
    ms, fl, by = ctypes.c_double(), ctypes.c_double(), ctypes.c_double()
    for i in range(lib().dion3_trace_count()):
        _check(lib().dion3_trace_record(i, ctypes.byref(name), ctypes.byref(ms), ctypes.byref(fl),
                                        ctypes.byref(by)), "dion3_trace_record")
        out.append((name.value.decode(), ms.value, fl.value, by.value))
    return out
