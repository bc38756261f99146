"""Plant plausible mistakes in a copy of the oracle and check that the pins catch each one.

Every mutant is the oracle's own source with one textual edit, executed as a
fresh module on the CPU.  A mutant survives only if every check in
tests/oracle_checks.py still passes, which would mean the pins cannot tell that
slip from the correct oracle.  (Running NS on the long side instead of the short
side is not listed: it gives the same result in exact arithmetic.)
"""

import inspect
import types

import pytest

import oracle.adamw as oa
import oracle.muon as om
from tests import oracle_checks as oc

MUTANTS = {
    "nesterov_uses_old_buffer": ("u = grad + mu * buf_new", "u = grad + mu * buf"),
    "momentum_as_lerp": ("buf_new = mu * buf + grad", "buf_new = mu * buf + (1.0 - mu) * grad"),
    "nesterov_flag_ignored": ("if nesterov:", "if True:"),
    "row_norm_over_columns": ("axis=1, keepdims=True", "axis=0, keepdims=True"),
    "row_norm_without_eps": ("return u / (norms + eps)", "return u / norms"),
    "row_norm_squared_norm": ("np.sqrt(np.sum(u * u, axis=1, keepdims=True))",
                              "np.sum(u * u, axis=1, keepdims=True)"),
    "frobenius_without_sqrt": ("x / (math.sqrt(float(np.sum(x * x))) + eps)",
                               "x / (float(np.sum(x * x)) + eps)"),
    "gram_transposed": ("gram = x @ x.T", "gram = x.T @ x"),
    "dropped_quintic_term": ("poly = b * gram + c * (gram @ gram)", "poly = b * gram + c * gram"),
    "dropped_cubic_term": ("poly = b * gram + c * (gram @ gram)", "poly = c * (gram @ gram)"),
    "update_right_multiplied": ("x = a * x + poly @ x", "x = a * x + x @ poly"),
    "update_sign": ("x = a * x + poly @ x", "x = a * x - poly @ x"),
    "dropped_linear_term": ("x = a * x + poly @ x", "x = x + poly @ x"),
    "table_reversed": ("for a, b, c in coeffs:", "for a, b, c in list(coeffs)[::-1]:"),
    "table_a_c_swapped": ("for a, b, c in coeffs:", "for c, b, a in coeffs:"),
    "table_first_row_skipped": ("for a, b, c in coeffs:", "for a, b, c in list(coeffs)[1:]:"),
    "table_first_row_repeated": ("for a, b, c in coeffs:", "for a, b, c in [coeffs[0]] * len(coeffs):"),
    "row_norm_skipped": ("r = row_normalize(u, eps) if row_norm else _f64(u)", "r = _f64(u)"),
    "row_norm_after_frobenius": (
        "r = row_normalize(u, eps) if row_norm else _f64(u)\n    x0 = frobenius_normalize(r, eps)",
        "r = frobenius_normalize(u, eps)\n    x0 = row_normalize(r, eps) if row_norm else r"),
    "not_transposed_back": ("return x.T if transposed else x", "return x"),
    "shape_scale_inverted": ("math.sqrt(max(1.0, rows / cols))", "math.sqrt(max(1.0, cols / rows))"),
    "shape_scale_without_sqrt": ("math.sqrt(max(1.0, rows / cols))", "max(1.0, rows / cols)"),
    "wd_without_lr": ("(1.0 - lr * wd) * w - lr * scale * o", "(1.0 - wd) * w - lr * scale * o"),
    "wd_after_update": ("(1.0 - lr * wd) * w - lr * scale * o", "(1.0 - lr * wd) * (w - lr * scale * o)"),
    "update_sign_in_apply": ("(1.0 - lr * wd) * w - lr * scale * o", "(1.0 - lr * wd) * w + lr * scale * o"),
    "shape_scale_dropped": ("(1.0 - lr * wd) * w - lr * scale * o", "(1.0 - lr * wd) * w - lr * o"),
    "ema_weights_swapped": ("d * e + (1.0 - d) * p", "(1.0 - d) * e + d * p"),
    "ema_dropped_param": ("d * e + (1.0 - d) * p", "d * e + (1.0 - d) * e"),
    "eps_too_large": ("EPS = 1e-7", "EPS = 1e-3"),
}


# The AdamW oracle (non-matrix parameters), checked by its own pins.
ADAMW_MUTANTS = {
    "adamw_no_bias_correction_m": ("m_hat = m_new / (1.0 - beta1 ** step)", "m_hat = m_new"),
    "adamw_no_bias_correction_v": ("v_hat = v_new / (1.0 - beta2 ** step)", "v_hat = v_new"),
    "adamw_step_counted_from_zero": ("(1.0 - beta1 ** step)", "(1.0 - beta1 ** (step + 1))"),
    "adamw_eps_inside_sqrt": ("(np.sqrt(v_hat) + eps)", "np.sqrt(v_hat + eps)"),
    "adamw_coupled_weight_decay": ("decayed = (1.0 - lr * wd) * p", "decayed = p\n    g = g + wd * p"),
    "adamw_wd_without_lr": ("decayed = (1.0 - lr * wd) * p", "decayed = (1.0 - wd) * p"),
    "adamw_wd_after_update": ("p_new = decayed - lr * m_hat / (np.sqrt(v_hat) + eps)",
                              "p_new = (1.0 - lr * wd) * (p - lr * m_hat / (np.sqrt(v_hat) + eps))"),
    "adamw_second_moment_not_squared": ("(1.0 - beta2) * (g * g)", "(1.0 - beta2) * g"),
    "adamw_betas_swapped": ("m_new = beta1 * m + (1.0 - beta1) * g", "m_new = beta2 * m + (1.0 - beta2) * g"),
    "adamw_update_sign": ("p_new = decayed - lr * m_hat", "p_new = decayed + lr * m_hat"),
}


def _mutant_module(old: str, new: str, base=om) -> types.ModuleType:
    src = inspect.getsource(base)
    assert src.count(old) >= 1, f"mutation site not found: {old!r}"
    mod = types.ModuleType("oracle_mutant")
    exec(compile(src.replace(old, new), "oracle_mutant", "exec"), mod.__dict__)
    return mod


def _caught(mod, checks=oc.ALL_ORACLE_CHECKS) -> bool:
    for check in checks:
        try:
            check(mod)
        except Exception:
            return True
    return False


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name):
    old, new = MUTANTS[name]
    assert _caught(_mutant_module(old, new)), f"mutant {name} survived every pin"


def test_unmutated_copy_passes():
    src = inspect.getsource(om)
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    assert not _caught(mod)


@pytest.mark.parametrize("name", sorted(ADAMW_MUTANTS))
def test_adamw_mutant_is_caught(name):
    old, new = ADAMW_MUTANTS[name]
    assert _caught(_mutant_module(old, new, oa), oc.ADAMW_CHECKS), f"mutant {name} survived every pin"


def test_unmutated_adamw_copy_passes():
    src = inspect.getsource(oa)
    mod = types.ModuleType("oracle_copy")
    exec(compile(src, "oracle_copy", "exec"), mod.__dict__)
    assert not _caught(mod, oc.ADAMW_CHECKS)
