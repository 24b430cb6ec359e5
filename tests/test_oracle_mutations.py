"""The oracle's pins catch plausible mistakes. Each case plants one mistake in a copy of the
oracle's source (a dropped term, a wrong sign or index, a swapped operand, a wrong exponent), loads
that copy as the module the pins call, and runs the pins written for the function it touches: at
least one of them must fail. The unmutated copy must pass the same pins."""
import itertools
import sys
import types

import pytest

import oracle.ssd_oracle as real
import test_oracle_pins as pins

SRC = open(real.__file__, encoding="utf-8").read()

# (name, text in the oracle, planted replacement, pins that must catch it)
MUTATIONS = [
    ("temperature ignored", "y = np.asarray(z, dtype=np.float64) / T", "y = np.asarray(z, dtype=np.float64)",
     ["test_softmax_is_scipy_softmax_of_scaled_logits"]),
    ("Saguaro normaliser with C in place of 1 - C", "N = 1.0 - (1.0 - C) * sigma", "N = 1.0 - C * sigma",
     ["test_saguaro_is_softmax_with_log_c_added_on_the_set", "test_saguaro_identity_conditional_and_set_hygiene"]),
    ("Saguaro weight on the complement", "w[idx] = C", "w[:] = C\n    w[idx] = 1.0",
     ["test_saguaro_is_softmax_with_log_c_added_on_the_set"]),
    ("acceptance test against q instead of p", "if k == K and not (float(u[i]) * qx < px):",
     "if k == K and not (float(u[i]) * px < qx):",
     ["test_accept_rule_cases_from_the_blog", "test_lossless_first_token_exact_enumeration"]),
    ("residual not clipped at zero", "r = np.maximum(p[k] - qd[k], 0.0)", "r = np.abs(p[k] - qd[k])",
     ["test_lossless_first_token_exact_enumeration", "test_residual_mass_is_one_minus_acceptance_rate"]),
    ("residual with the rows swapped", "r = np.maximum(p[k] - qd[k], 0.0)", "r = np.maximum(qd[k] - p[k], 0.0)",
     ["test_lossless_first_token_exact_enumeration"]),
    ("bonus after full acceptance from the last drafted row", "r, R, R_out = p[K], 1.0, 1.0",
     "r, R, R_out = p[K - 1], 1.0, 1.0", ["test_lossless_two_positions_and_bonus_after_full_acceptance"]),
    ("inverse CDF taking the first token at or above the target", 'side="right"))  # first index with cum > target',
     'side="left"))  # first index with cum > target', ["test_bonus_never_lands_on_zero_mass_tokens",
                                                        "test_bonus_inverse_cdf_closed_forms"]),
    ("top-F ties to the larger index", "order = np.lexsort((np.arange(V), -z))", "order = np.lexsort((-np.arange(V), -z))",
     ["test_topf_matches_python_sort_with_ties_and_masking"]),
    ("top-F keeps the excluded token", "keep = order[(order != exclude) & (z[order] > -np.inf)]",
     "keep = order[z[order] > -np.inf]", ["test_topf_matches_python_sort_with_ties_and_masking",
                                          "test_ssd_round_keys_outcome_k_with_the_guesses_of_draft_row_k"]),
    ("fan-out exponent 1/r", "ratio = (P / P[0]) ** (1.0 / (1.0 + r))", "ratio = (P / P[0]) ** (1.0 / r)",
     ["test_fanout_continuous_is_the_lagrange_stationary_point", "test_fanout_twelve_branch_case_and_edges"]),
    ("geometric law without the stop term", "P = np.array([(1.0 - a) * a ** k for k in range(K)] + [a ** K]",
     "P = np.array([(1.0 - a) * a ** k for k in range(K + 1)]", ["test_fanout_twelve_branch_case_and_edges",
                                                                  "test_accepted_length_is_geometric_with_identical_rows"]),
    ("cache keyed one position late", "kk.append(k if t >= 0 else -1)", "kk.append(k + 1 if t >= 0 else -1)",
     ["test_cache_keys_layout_and_lookup_against_a_dict", "test_ssd_round_keys_outcome_k_with_the_guesses_of_draft_row_k"]),
    ("round guesses from the next draft row", "guesses = [topf(zq[i], int(F[i]), int(x[b, i])) for i in range(K)]",
     "guesses = [topf(zq[min(i + 1, K)], int(F[i]), int(x[b, i])) for i in range(K)]",
     ["test_ssd_round_keys_outcome_k_with_the_guesses_of_draft_row_k"]),
    ("all-hit probability linear in B", "return float(h) ** int(B)", "return max(0.0, 1.0 - (1.0 - float(h)) * int(B))",
     ["test_all_hit_fraction_decays_as_h_to_the_b", "test_ninety_two_percent_example"]),
    ("speedup adds the primary's time to the verification", "return A / (max(1.0, T_p) + (1.0 - h ** b) * T_b)",
     "return A / (1.0 + T_p + (1.0 - h ** b) * T_b)", ["test_batch_speedup_matches_a_simulated_two_gpu_schedule",
                                                       "test_batch_speedup_hand_values_and_limits"]),
    ("sampling draws from q instead of q'", "cum = np.cumsum(qs)", "cum = np.cumsum(q)",
     ["test_saguaro_sample_is_the_library_inverse_cdf"]),
]


def _load(src):
    mod = types.ModuleType("mutated_oracle")
    mod.__file__ = real.__file__
    sys.modules["mutated_oracle"] = mod  # dataclasses look their module up while the class is made
    try:
        exec(compile(src, real.__file__, "exec"), mod.__dict__)
    finally:
        del sys.modules["mutated_oracle"]
    return mod


def _run(fn):
    """Run one pin over every parameter combination its parametrize marks give."""
    marks = [m for m in getattr(fn, "pytestmark", []) if m.name == "parametrize"]
    if not marks:
        fn()
        return
    axes = []
    for m in marks:
        names = [n.strip() for n in m.args[0].split(",")] if isinstance(m.args[0], str) else list(m.args[0])
        vals = [v if len(names) > 1 else (v,) for v in m.args[1]]
        axes.append([dict(zip(names, v)) for v in vals])
    for combo in itertools.product(*axes):
        kw = {}
        for d in combo:
            kw.update(d)
        fn(**kw)


def _caught(mod, names, monkeypatch):
    monkeypatch.setattr(pins, "O", mod)
    for n in names:
        try:
            _run(getattr(pins, n))
        except Exception:  # a failed assertion, or an error the mistake provokes
            return True
    return False


def test_the_unmutated_copy_passes_the_pins(monkeypatch):
    mod = _load(SRC)
    names = sorted({n for *_, ns in MUTATIONS for n in ns})
    assert not _caught(mod, names, monkeypatch)


@pytest.mark.parametrize("name,old,new,names", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_a_planted_mistake_fails_a_pin(name, old, new, names, monkeypatch):
    assert SRC.count(old) == 1, f"the text to mutate is not unique in the oracle: {old!r}"
    mod = _load(SRC.replace(old, new))
    assert _caught(mod, names, monkeypatch), f"no pin caught: {name}"
