"""Plain float64 CPU oracle of the speculative-sampling verifier.

TEST INFRASTRUCTURE ONLY: imported by the tests, the smoke check and the benchmark's CPU-baseline leg, never by the
HIP library or its binding. It shares no code with them.
"""
from .verify import (FLAG_EMPTY_RESIDUAL, FLAG_ID_RANGE, FLAG_NONFINITE, FLAG_Q_ZERO, FATAL, accept_test,
                     accept_test_exact, inverse_cdf,
                     log_softmax_at, residual, softmax, verify_dense, verify_onehot, verify_sparse, verify_windows,
                     widen)
from .support import build_support, topk_order
from .greedy import first_argmax, verify_greedy
from .commit import confidence_commit, slot_confidence
from .tree import tree_children, tree_is_valid, verify_tree

__all__ = ["FLAG_EMPTY_RESIDUAL", "FLAG_ID_RANGE", "FLAG_NONFINITE", "FLAG_Q_ZERO", "FATAL", "accept_test",
           "accept_test_exact",
           "inverse_cdf", "log_softmax_at", "residual", "softmax", "verify_dense", "verify_onehot", "verify_sparse",
           "verify_windows", "widen", "build_support", "topk_order", "first_argmax", "verify_greedy",
           "confidence_commit", "slot_confidence", "tree_children", "tree_is_valid", "verify_tree"]
