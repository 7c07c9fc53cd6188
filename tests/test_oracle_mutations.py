"""The pins have teeth: each test here plants one plausible mistake in a copy of the
oracle's source (a dropped term, a wrong sign or index, a misplaced bias, a swapped
order), points the package at the mutated copy, and checks that at least one of the
pins in test_oracle_pins.py then fails. Everything runs on the CPU; the oracle itself
is never modified."""
import inspect
import sys
import types

import pytest

import oracle
import oracle.hstu_oracle as ho
import test_oracle_pins as pins

SOURCE = inspect.getsource(ho)
PATCHED = ["encode", "attention_user", "layer_user", "pack_uih", "score_head", "sigmoid", "round_bf16",
           "silu", "normalize_rows", "user_positions"]


def mutated(old: str, new: str) -> types.ModuleType:
    assert SOURCE.count(old) == 1, f"mutation site not unique: {old!r}"
    name = "oracle_with_planted_mistake"
    mod = types.ModuleType(name)
    sys.modules[name] = mod          # dataclasses look their module up while the source runs
    try:
        exec(compile(SOURCE.replace(old, new), name, "exec"), mod.__dict__)
    finally:
        del sys.modules[name]
    return mod


MUTATIONS = [
    ("diagonal excluded from the history mask",
     "allowed = key_pos[None, :] <= (m + rb)[:, None]", "allowed = key_pos[None, :] < (m + rb)[:, None]",
     [(pins.test_oracle_matches_brute_force, ("f64",)), (pins.test_attention_two_tokens_causal_closed_form, ())]),
    ("candidate's own key dropped",
     "a @ vh + a_self[:, None] * v_c[s:s + block, cols]", "a @ vh",
     [(pins.test_oracle_matches_brute_force, ("f64",)), (pins.test_attention_candidate_with_empty_history, ())]),
    ("1/max_len scale dropped on history rows",
     "o_u[s:s + block, cols] = R(inv * (a @ vh))", "o_u[s:s + block, cols] = R(a @ vh)",
     [(pins.test_attention_single_history_token, (False,)), (pins.test_oracle_matches_brute_force, ("f64",))]),
    ("position bias also added to U",
     "u = R(s[:, 0:D])", "u = R(s[:, 0:D] + bias[:, 0:D])",
     [(pins.test_oracle_matches_brute_force, ("f64",)), (pins.test_oracle_matches_brute_force_no_cache_four_heads, ())]),
    ("gate formed as U + O",
     "gate = R(u * o)", "gate = R(u + o)",
     [(pins.test_oracle_matches_brute_force, ("f64",))]),
    ("residual dropped",
     "return R(x + z)", "return R(z)",
     [(pins.test_oracle_matches_brute_force, ("f64",))]),
    ("bfloat16 rounding truncates instead of rounding to nearest even",
     "y = np.ldexp(np.rint(np.ldexp(x, -q)), q)", "y = np.ldexp(np.floor(np.ldexp(x, -q)), q)",
     [(pins.test_round_bf16_hand_built_cases, ()), (pins.test_round_bf16_matches_library_on_float32_values, ())]),
    ("variance taken about zero instead of the mean",
     "var = np.mean((x - mu) ** 2, axis=1, keepdims=True)", "var = np.mean(x ** 2, axis=1, keepdims=True)",
     [(pins.test_normalize_rows_closed_forms, ())]),
    ("relative position taken as pos_j - pos_i",
     "rel[h][np.maximum((m + rb)[:, None] - key_pos[None, :], 0)]",
     "rel[h][np.maximum(key_pos[None, :] - (m + rb)[:, None], 0)]",
     [(pins.test_relative_bias_two_tokens_with_cache_and_candidate, ()),
      (pins.test_relative_bias_zero_query_is_a_causal_convolution, ())]),
    ("interleaving puts the action first",
     "t[0::2] = c\n            t[1::2] = a", "t[0::2] = a\n            t[1::2] = c",
     [(pins.test_interleave_doubles_the_history, ()), (pins.test_pack_matches_brute_force, ("interleave",))]),
    ("merged tokens not rounded in the bfloat16 mirror",
     "            if bf16:\n                t = round_bf16(t)\n", "",
     [(pins.test_pack_sum_closed_forms, ()), (pins.test_pack_matches_brute_force, ("sum",))]),
    ("no ReLU between head layers",
     "h = np.maximum(z, 0.0)", "h = z",
     [(pins.test_score_head_relu_between_layers, ()), (pins.test_score_head_matches_brute_force, (False,))]),
    ("sigmoid of the negated logit",
     "return np.where(z >= 0, 1.0 / (1.0 + e), e / (1.0 + e))",
     "return np.where(z >= 0, e / (1.0 + e), 1.0 / (1.0 + e))",
     [(pins.test_sigmoid_closed_forms_and_library, ()), (pins.test_score_head_single_layer_is_logistic_regression, ())]),
]


@pytest.mark.parametrize("label,old,new,catchers", MUTATIONS, ids=[m[0] for m in MUTATIONS])
def test_a_pin_catches_the_planted_mistake(monkeypatch, label, old, new, catchers):
    mod = mutated(old, new)
    for name in PATCHED:
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    caught = []
    for fn, args in catchers:
        try:
            fn(*args)
        except AssertionError:
            caught.append(fn.__name__)
    assert caught, f"no pin failed with the planted mistake: {label}"


def test_the_unmutated_copy_passes_the_same_pins(monkeypatch):
    """Control: the copying itself changes nothing, so every catcher passes on a clean copy."""
    mod = mutated("def silu(x) -> np.ndarray:", "def silu(x) -> np.ndarray:")
    for name in PATCHED:
        monkeypatch.setattr(oracle, name, getattr(mod, name))
    for _, _, _, catchers in MUTATIONS:
        for fn, args in catchers:
            fn(*args)
