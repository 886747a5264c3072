"""Shape-grouped Dion3 step over a set of weight matrices.

Transformers hold only a few distinct weight shapes; the matrices of one
shape are stepped together ("Dion3: Full-Stack Orthogonal Updates",
agihunt.info, level-4 paragraph: megabatching; here on one GPU, where it
turns one launch sequence per matrix into one per shape), and all shape
groups of a device go to the library in one call, which runs the s x s
products of groups with equal Gram sides as one launch.
"""
from __future__ import annotations

import math
from collections import OrderedDict
from fractions import Fraction
from typing import Dict, List, Optional, Sequence, Tuple

from . import _lib


class Dion3Step:
    """Holds (W, M) pairs, grouped by (shape, row stride).

    ``step()`` runs, per group, l1 row scoring, top-k selection with
    k = ceil(f n), Gram Newton-Schulz on the selected rows, the row-sparse
    update W[S] -= lr_eff * O with lr_eff = lr / sqrt(f) (level-3 paragraph:
    eta proportional to 1/sqrt(f)) and the decay M[S] *= mu.  The momentum M
    is the optimizer state.  ``step(grads)`` first accumulates one gradient
    per weight into it (M <- M + G, fused into the row scoring); ``step()``
    starts from M as it is.
    """

    def __init__(self, weights: Sequence, momenta: Sequence, lr: float = 0.02,
                 fraction=Fraction(1, 4), mu: float = 0.95, cfg: Optional[_lib.NsCfg] = None):
        if len(weights) != len(momenta):
            raise ValueError("need one momentum per weight")
        self.lr = float(lr)
        self.fraction = fraction
        self.mu = float(mu)
        self.cfg = cfg
        self.groups: "OrderedDict[Tuple, Dict]" = OrderedDict()
        self._order = list(weights)
        for w, m in zip(weights, momenta):
            if w.dim() != 2 or w.shape != m.shape:
                raise ValueError("Dion3 steps 2-D matrices with same-shape momentum")
            if w.stride() != m.stride() or w.stride(1) != 1 or w.device != m.device:
                raise ValueError("W and M must share strides and device, with contiguous rows")
            key = (tuple(w.shape), w.stride(0), str(w.device))
            self.groups.setdefault(key, {"W": [], "M": []})
            self.groups[key]["W"].append(w)
            self.groups[key]["M"].append(m)
        self.ws: Dict[str, _lib.Workspace] = {}     # one per device, shared by its groups
        for key, g in self.groups.items():
            dev = g["M"][0].device
            self.ws.setdefault(str(dev), _lib.Workspace())
            g["k"] = _lib.k_from_fraction(float(self.fraction), key[0][0])
            g["group"] = _lib.Group(g["W"], g["M"], g["k"], self.lr_eff)

    @property
    def lr_eff(self) -> float:
        return self.lr / math.sqrt(float(self.fraction))

    def step(self, grads: Optional[Sequence] = None):
        """One step over every group.  With ``grads`` (one per weight, in the
        order the weights were given), each momentum first accumulates its
        gradient, M <- M + G, fused into the row scoring."""
        gmap = None
        if grads is not None:
            if len(grads) != sum(len(g["W"]) for g in self.groups.values()):
                raise ValueError("need one gradient per weight")
            gmap = {id(w): gr for w, gr in zip(self._order, grads)}
        by_dev: "OrderedDict[str, List]" = OrderedDict()
        for key, g in self.groups.items():
            grp = g["group"]
            if gmap is not None:
                grp = _lib.Group(g["W"], g["M"], g["k"], self.lr_eff,
                                 Gs=[gmap[id(w)] for w in g["W"]])
            by_dev.setdefault(key[2], []).append(grp)
        for dev, grps in by_dev.items():
            for i in range(0, len(grps), _lib.MAX_GROUPS):
                _lib.step_groups(grps[i:i + _lib.MAX_GROUPS], self.mu, self.cfg, ws=self.ws[dev])


def _optimizer_base():
    import torch
    return torch.optim.Optimizer


class Dion3(_optimizer_base()):
    """torch.optim-style Dion3 for 2-D fp32 parameters.

    Each parameter p with a gradient keeps a momentum buffer M (fp32, zero at
    first).  ``step()`` runs, per parameter group and per (shape, strides,
    device), one megabatched library call: M <- M + grad (fused into the row
    scoring), top-k row selection with k = ceil(f n), Gram Newton-Schulz on
    the selected rows, p[S] -= lr / sqrt(f) * O and M[S] *= mu ("Dion3:
    Full-Stack Orthogonal Updates", agihunt.info, level-3 paragraph: error
    feedback keeps the unselected rows of M for a later step; level-4:
    megabatching by shape).  Parameters that are not 2-D fp32 matrices with
    contiguous rows are refused: route them to another optimizer.

    With ``normalize=True`` the update is normalized per neuron (row) with a
    float32 second-moment state per row (``beta2``, ``eps``), the reading of
    the pages' "per-neuron normalization inherited from NorMuon" stated in
    include/dion3.h at dion3_norm_cfg.
    """

    def __init__(self, params, lr: float = 0.02, fraction=Fraction(1, 4), mu: float = 0.95,
                 cfg: Optional[_lib.NsCfg] = None, normalize: bool = False,
                 beta2: float = 0.95, eps: float = 1e-8):
        if lr <= 0 or not (0 < float(fraction) <= 1) or not (0 <= mu <= 1):
            raise ValueError("need lr > 0, 0 < fraction <= 1 and 0 <= mu <= 1")
        if normalize and not (0 <= beta2 < 1 and eps >= 0):
            raise ValueError("need 0 <= beta2 < 1 and eps >= 0")
        super().__init__(params, dict(lr=lr, fraction=fraction, mu=mu, normalize=normalize,
                                      beta2=beta2, eps=eps))
        import torch
        for group in self.param_groups:
            for p in group["params"]:
                if p.dim() != 2 or p.dtype != torch.float32 or p.stride(1) != 1:
                    raise ValueError("Dion3 steps 2-D fp32 matrices with contiguous rows")
        self.cfg = cfg
        self._ws: Dict[str, _lib.Workspace] = {}

    def step(self, closure=None):
        import torch
        loss = None
        if closure is not None:
            with torch.enable_grad():
                loss = closure()
        with torch.no_grad():
            for group in self.param_groups:
                f = float(group["fraction"])
                buckets: "OrderedDict[Tuple, List]" = OrderedDict()
                for p in group["params"]:
                    if p.grad is None:
                        continue
                    if p.grad.stride() != p.stride():
                        raise ValueError("a gradient must have its parameter's strides")
                    st = self.state[p]
                    if "momentum" not in st:   # the parameter's own strides
                        st["momentum"] = torch.empty_strided(p.shape, p.stride(), dtype=p.dtype,
                                                             device=p.device).zero_()
                    if group["normalize"] and "second_moment" not in st:
                        st["second_moment"] = torch.zeros(p.shape[0], dtype=torch.float32,
                                                          device=p.device)
                    buckets.setdefault((tuple(p.shape), p.stride(), str(p.device)), []).append(p)
                # one library call per device over all of its shape buckets
                by_dev: "OrderedDict[str, List]" = OrderedDict()
                for (shape, _, dev), ps in buckets.items():
                    k = _lib.k_from_fraction(f, shape[0])
                    Vs = ([self.state[p]["second_moment"] for p in ps] if group["normalize"]
                          else None)
                    by_dev.setdefault(dev, []).append(
                        _lib.Group(ps, [self.state[p]["momentum"] for p in ps], k,
                                   group["lr"] / math.sqrt(f), Gs=[p.grad for p in ps], Vs=Vs))
                norm = (group["beta2"], group["eps"]) if group["normalize"] else None
                for dev, grps in by_dev.items():
                    ws = self._ws.setdefault(dev, _lib.Workspace())
                    for i in range(0, len(grps), _lib.MAX_GROUPS):
                        _lib.step_groups(grps[i:i + _lib.MAX_GROUPS], group["mu"], self.cfg,
                                         norm=norm, ws=ws)
        return loss
