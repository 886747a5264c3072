"""fp64 CPU oracle of the Dion3 optimizer step (test infrastructure only:
imported by tests, the smoke check and the benchmark's CPU-baseline leg,
never by the product path)."""
from .dion3_oracle import (MUON_COEFFS, DEFAULT_EPS, DEFAULT_ITERS, DEFAULT_RESTART_AT,
                           ProductLog, default_coeffs, dion3_step, k_from_fraction,
                           normalize_neurons, ns_gram, ns_standard, row_scores,
                           select_rows)

__all__ = ["MUON_COEFFS", "DEFAULT_EPS", "DEFAULT_ITERS", "DEFAULT_RESTART_AT", "ProductLog",
           "default_coeffs", "dion3_step", "k_from_fraction", "normalize_neurons", "ns_gram",
           "ns_standard",
           "row_scores", "select_rows"]
