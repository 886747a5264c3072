"""Shape-grouped Dion3 step over a set of weight matrices.

Transformers hold only a few distinct weight shapes; the matrices of one
shape are stepped together by one library call ("Dion3: Full-Stack
Orthogonal Updates", agihunt.info, level-4 paragraph: megabatching; here on
one GPU, where it turns one launch sequence per matrix into one per shape).
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
    is the optimizer state; accumulating gradients into it is left to the
    caller.
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
            g["ws"] = self.ws.setdefault(str(dev), _lib.Workspace())
            g["ptrs"] = (_lib.pointer_array(g["W"], dev), _lib.pointer_array(g["M"], dev))
            g["k"] = _lib.k_from_fraction(float(self.fraction), key[0][0])

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
        for key, g in self.groups.items():
            Gs = [gmap[id(w)] for w in g["W"]] if gmap is not None else None
            _lib.step_megabatch(g["W"], g["M"], g["k"], self.lr_eff, self.mu, self.cfg,
                                ws=g["ws"], ptrs=g["ptrs"], Gs=Gs)
