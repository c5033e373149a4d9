"""Planted mistakes: plausible errors written into copies of the oracle's sources, each of which some CPU pin must
catch. A mutation is an exact text edit of one oracle module (the text must occur exactly once); ``plant`` loads the
edited source as a fresh module of the ``oracle`` package and points the package's names (and the original
submodule's) at the edited functions, so that every pin that calls the oracle calls the mistaken version.

The tests/conftest.py hook applies the mutation named by the ORACLE_PLANT environment variable when a pytest session
starts; tests/test_planted_mistakes.py runs the pins of each mutation in such a session and requires a failure.
"""
from __future__ import annotations

import importlib
import os
import sys
import types

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# name -> (oracle module, text, replacement, pin files and pytest -k expression, what the mistake is)
MUTATIONS = {
    # masked-diffusion windows (Self-Speculative Masked Diffusions, 关键设计 2 and 4)
    "window_round0_uniforms": (
        "verify", "u_accept_rounds[r], u_sample_rounds[r]", "u_accept_rounds[0], u_sample_rounds[0]",
        ("tests/test_oracle_pins.py", "window"), "every round reuses round 0's uniforms"),
    "window_start_at_reject": (
        "verify", "np.where(live, np.minimum(G, k + 1), st)", "np.where(live, np.minimum(G, k), st)",
        ("tests/test_oracle_pins.py", "window"), "the next round starts at the rejected slot instead of after it"),
    "window_order_ignored": (
        "verify", "order = np.tile(np.arange(G), (B, 1)) if order is None else np.asarray(order, dtype=np.int64)",
        "order = np.tile(np.arange(G), (B, 1))",
        ("tests/test_oracle_pins.py", "window"), "slots verified in storage order instead of sigma"),
    # confidence-threshold commit (block diffusion page, section 5)
    "commit_strict_threshold": (
        "commit", "keep = conf >= tau", "keep = conf > tau",
        ("tests/test_commit_pins.py", None), "a confidence equal to tau is not committed"),
    "commit_forced_highest_slot": (
        "commit", "keep[int(np.argmax(conf))] = True", "keep[len(conf) - 1 - int(np.argmax(conf[::-1]))] = True",
        ("tests/test_commit_pins.py", None), "the forced commit breaks ties towards the highest slot"),
    "commit_no_forced_slot": (
        "commit", "keep[int(np.argmax(conf))] = True", "pass",
        ("tests/test_commit_pins.py", None), "no slot is committed when none reaches tau"),
    "commit_wrong_confidence": (
        "commit", "return a, 1.0 / s", "return a, 1.0 / (s + 1.0)",
        ("tests/test_commit_pins.py", None), "the confidence counts the maximum twice"),
    # top-k / top-p support builder (Uno, "The speedup, without the 'up to'"; DFlash guide section 9 Q3)
    "support_le_for_lt": (
        "support", "np.count_nonzero(C[:-1] < p_cut)", "np.count_nonzero(C[:-1] <= p_cut)",
        ("tests/test_support_pins.py", None), "a prefix whose mass equals top_p does not stop the support"),
    "support_no_temperature": (
        "support", "a = z[order] / T", "a = z[order] / 1.0",
        ("tests/test_support_pins.py", None), "the temperature is ignored"),
    "support_topp_over_full_row": (
        "support", "C = cum / cum[-1]", "C = cum / np.exp(z / T - a[0]).sum()",
        ("tests/test_support_pins.py", None), "top-p measured on the full distribution, not the top-k one"),
    "support_reverse_ties": (
        "support", "np.lexsort((ids, -z))", "np.lexsort((-ids, -z))",
        ("tests/test_support_pins.py", None), "equal logits ordered by descending id"),
    "support_drop_crossing_slot": (
        "support", "m = 1 + int(np.count_nonzero(C[:-1] < p_cut))", "m = max(1, int(np.count_nonzero(C < p_cut)))",
        ("tests/test_support_pins.py", None), "the slot that crosses top_p is dropped"),
    "support_renorm_over_all_k": (
        "support", "out[:m] = e[:m] / cum[m - 1]", "out[:m] = e[:m] / cum[-1]",
        ("tests/test_support_pins.py", None), "kept probabilities renormalised over all k slots"),
    # tree verification (SpecInfer's multi-step speculative sampling with one-hot q per candidate)
    "tree_no_renormalisation": (
        "tree", "P = p[x] / np.sum(p[~excluded])", "P = p[x]",
        ("tests/test_tree_pins.py", "golden or exact_law"), "a later candidate is tested against p, not p without the "
        "rejected tokens"),
    "tree_draw_keeps_rejected": (
        "tree", "r = np.where(excluded, 0.0, p)", "r = p",
        ("tests/test_tree_pins.py", "golden or exact_law"), "the final draw can return a rejected candidate"),
    "tree_children_descending": (
        "tree", "kids[int(parent[i])].append(i)", "kids[int(parent[i])].insert(0, i)",
        ("tests/test_tree_pins.py", "golden or exact_law"), "siblings tested from the highest node index"),
    "tree_non_strict_test": (
        "tree", "if ua[b, c] < min(1.0, P):", "if ua[b, c] <= min(1.0, P):",
        ("tests/test_tree_pins.py", "golden or exact_law"), "u equal to p'(x) accepts (a repeated token passes at "
        "u = 0)"),
    "tree_exclusions_kept_after_accept": (
        "tree", """        cur, path, fault = 0, [], False
        while True:
            p = row_p(cur)
            if p is None:
                fault = True
                break
            excluded = np.zeros(V, bool)
""", """        cur, path, fault = 0, [], False
        excluded = np.zeros(V, bool)
        while True:
            p = row_p(cur)
            if p is None:
                fault = True
                break
""", ("tests/test_tree_pins.py", "golden or exact_law"), "tokens rejected at one node stay excluded at the next"),
}


def source_of(module: str) -> str:
    with open(os.path.join(ROOT, "oracle", module + ".py"), encoding="utf-8") as f:
        return f.read()


def mutated_source(name: str) -> str:
    module, old, new, _, _ = MUTATIONS[name]
    src = source_of(module)
    if src.count(old) != 1:
        raise ValueError(f"mutation {name}: the text to replace occurs {src.count(old)} times in oracle/{module}.py")
    return src.replace(old, new)


def plant(name: str) -> None:
    """Replace the oracle's functions from one module by those of its mutated source."""
    import oracle
    module = MUTATIONS[name][0]
    real = importlib.import_module(f"oracle.{module}")
    mod = types.ModuleType(f"oracle.{module}_planted")
    mod.__package__ = "oracle"
    mod.__file__ = real.__file__
    exec(compile(mutated_source(name), real.__file__, "exec"), mod.__dict__)
    for attr, val in mod.__dict__.items():
        if isinstance(val, types.FunctionType) and val.__module__ == mod.__name__:
            setattr(real, attr, val)
            if hasattr(oracle, attr):
                setattr(oracle, attr, val)
    sys.modules["oracle"].__planted__ = name
