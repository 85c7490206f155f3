"""CPU float64 oracle of the low-rank draft LM head, and the comparison rule.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library. It shares
no code with the HIP path.
"""
from .lowrank_head import (  # noqa: F401
    to_f64, round_fp32, round_bf16, round_weight_dtype, down_projection,
    vocab_scores, topk_order, selection_stats, exact_logits, lowrank_head,
    full_head,
)
from .branching import draft_distribution, branch_order, branches  # noqa: F401
from .compare import (  # noqa: F401
    check_candidates, check_logits, check_scores, band_counts, ulp_bf16,
    z_step_allowance, LOGIT_RTOL, SCORE_TOL,
)
from . import recall  # noqa: F401,E402
