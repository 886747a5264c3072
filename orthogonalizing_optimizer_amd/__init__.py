"""Dion3 optimizer step for AMD MI355X (gfx950).

The hot path is libdion3.so (hand-written HIP kernels behind a C ABI, see
include/dion3.h); this package is its thin Python binding.
"""
from ._lib import (MAX_GROUPS, NS_GRAM, NS_STANDARD, PATH_AUTO, PATH_FUSED, PATH_TILED,
                   Dion3Error, Group, NormCfg, NsCfg, Workspace, default_cfg, gram_ns,
                   k_from_fraction, lib, ns_cfg, pointer_array, row_select, status_string, step,
                   step_groups, step_megabatch, symm_f16, syrk_f16, trace_disable, trace_enable,
                   trace_records, trace_reset, workspace_size, workspace_size_groups)
from .optim import Dion3, Dion3Step

__all__ = ["MAX_GROUPS", "NS_GRAM", "NS_STANDARD", "PATH_AUTO", "PATH_FUSED", "PATH_TILED",
           "Dion3Error", "Group", "NormCfg", "NsCfg", "Workspace", "default_cfg", "gram_ns",
           "k_from_fraction", "lib", "ns_cfg", "pointer_array", "row_select", "status_string",
           "step", "step_groups", "step_megabatch", "symm_f16", "syrk_f16", "trace_disable",
           "trace_enable", "trace_records", "trace_reset", "workspace_size",
           "workspace_size_groups", "Dion3", "Dion3Step"]
