"""Planted mistakes: each copy of the oracle source with one plausible error must
fail at least one pin of tests/test_oracle.py (CPU only).

This checks the pins, not the oracle: a pin set that every mutant passes would
not be evidence of anything.
"""
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "moda_oracle.c")

MUTANTS = {
    # causal diagonal dropped: key j = t no longer visible
    "diagonal_excluded": ("return (s->flags & 1) ? s->T - 1 : t;",
                          "return (s->flags & 1) ? s->T - 1 : t - 1;"),
    # KV head chosen by modulo instead of adjacent grouping
    "head_mapping_modulo": ("kv = h / G, L = s->L", "kv = h % s->Hk, L = s->L"),
    # depth rows read layer-major instead of token-major
    "depth_layer_major": (
        "scores[nseq + l] = s->scale * dot(s, Q, qo, Kd, dep_off(s, b, kv, t * L + l));",
        "scores[nseq + l] = s->scale * dot(s, Q, qo, Kd, dep_off(s, b, kv, l * s->T + t));"),
    # depth weights left out of the softmax denominator
    "depth_not_in_denominator": (
        "        Z += w;\n        for (int64_t e = 0; e < d; ++e) o[e] += w * elem(Vd,",
        "        for (int64_t e = 0; e < d; ++e) o[e] += w * elem(Vd,"),
    # depth scores not scaled
    "depth_unscaled": ("scores[nseq + l] = s->scale * dot(", "scores[nseq + l] = dot("),
    # log-sum-exp in base 2
    "lse_base2": ("*lse = m + log(Z);", "*lse = m + log2(Z);"),
    # sign error in the softmax backward
    "ds_sign": ("const double ds = p * (dot(s, dO, qo, V, ko) - D[i]);\n"
                "                for (int64_t e = 0; e < d; ++e) dq[e]",
                "const double ds = p * (dot(s, dO, qo, V, ko) + D[i]);\n"
                "                for (int64_t e = 0; e < d; ++e) dq[e]"),
    # dV accumulates the score gradient instead of the probability
    "dV_uses_ds": ("dv[e] += p * elem(dO,", "dv[e] += ds * elem(dO,"),
    # depth key gradient missing the score scale
    "dKd_unscaled": ("dkd[e] += s->scale * du * elem(Q,", "dkd[e] += du * elem(Q,"),
    # transposed operand: key gradient built from keys instead of queries
    "dK_wrong_operand": ("dk[e] += s->scale * ds * elem(Q, s->dtype, qo + e);",
                         "dk[e] += s->scale * ds * elem(K, s->dtype, ko + e);"),
    # depth value gradient attributed to the wrong token's rows
    "dVd_wrong_row": ("double* dvd = dVd + (tt * L + l) * d;",
                      "double* dvd = dVd + (((tt + 1) % n) * L + l) * d;"),
    # non-causal flag ignored: the sequence causal mask stays on
    "noncausal_keeps_mask": ("return (s->flags & 1) ? s->T - 1 : t;", "return t;"),
    # depth window ignored: every slot stays visible
    "window_ignored": ("return s->window > 0 ? s->L - s->window : 0;", "return 0;"),
    # depth window one slot short
    "window_off_by_one": ("return s->window > 0 ? s->L - s->window : 0;",
                          "return s->window > 0 ? s->L - s->window + 1 : 0;"),
    # key gradients of the token-set backward keep the causal test in non-causal mode
    "dK_causal_in_noncausal": ("if (j > last_key(s, t)) continue;", "if (j > t) continue;"),
}

PINS = [
    pins.test_forward_matches_dense_transcription_grid,
    pins.test_variants_match_dense_transcription_grid,
    pins.test_zero_query_gives_uniform_weights,
    pins.test_hand_worked_two_token_example,
    pins.test_sequence_pushed_to_minus_infinity_gives_depth_attention,
    pins.test_backward_matches_central_finite_differences,
    pins.test_backward_invariants,
]


def run_pins():
    """Names of the pins that fail on the currently loaded oracle build."""
    failed = []
    calls = [(f.__name__, f, ()) for f in PINS]
    calls.append(("library_causal_G2", pins.test_no_depth_equals_library_causal_attention, (2,)))
    calls.append(("library_autograd_G2", pins.test_backward_no_depth_equals_library_autograd,
                  (2,)))
    calls.append(("library_noncausal_G4", pins.test_noncausal_no_depth_equals_library_attention,
                  (4,)))
    calls.append(("window_truncated_W3", pins.test_window_equals_operator_on_truncated_depth_cache,
                  (True, 3)))
    calls.append(("sparse_dO_noncausal",
                  pins.test_sparse_upstream_gradient_token_set_backward_is_complete, (False,)))
    for name, f, args in calls:
        try:
            f(*args)
        except AssertionError:
            failed.append(name)
    return failed


def test_unmutated_source_passes_every_pin():
    assert run_pins() == []


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(name, tmp_path):
    old, new = MUTANTS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not unique"
    path = tmp_path / f"{name}.c"
    path.write_text(src.replace(old, new))
    lib = oracle.build(str(path), str(tmp_path / f"lib_{name}.so"))
    with oracle.use_library(lib):
        failed = run_pins()
    assert failed, f"no pin caught the planted mistake {name}"
