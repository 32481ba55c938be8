"""Independent float64 CPU oracle (test infrastructure only; see am.py)."""
from .am import *  # noqa: F401,F403
from .am import (row_lse, attention_stats, select_topt, compact_probs, nnls_normal,
                 fit_bias, compacted_weights, fit_values, fit, compact, compact_chunked,
                 omp_dictionary, omp_select, compact_omp,
                 compact_ragged, compact_protected, attend,
                 attend_appended, rel_l2, W_FLOOR, DEFAULT_RIDGE_REL)
