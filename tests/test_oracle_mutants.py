"""Each plausible mistake planted in a copy of the oracle is caught by a pin.

The mistakes are planted on the CPU only, in a temporary copy of oracle.cpp
built into its own library; the real oracle is untouched.
"""
import os
import subprocess
import tempfile

import pytest

import oracle
import oracle.build as ob
from tests import pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.cpp")

# (name, text in oracle.cpp, replacement)
MUTANTS = [
    ("drop_rank_1", "for (int32_t r = 1; r < N; ++r)", "for (int32_t r = 2; r < N; ++r)"),
    ("inclusive_bound_divisor", "return s / (float)N;", "return s / (float)(N + 1);"),
    ("sum_not_averaged", "return s / (float)N;", "return s;"),
    ("reverse_rank_order", "s = s + widen(G[r][i]);", "s = s + widen(G[N - r][i]);"),
    ("wrong_index", "s = s + widen(G[r][i]);", "s = s + widen(G[r][i > 0 ? i - 1 : i]);"),
    ("swap_beta1_terms", "f.b1 * M[i] + f.c1 * g", "f.c1 * M[i] + f.b1 * g"),
    ("v_uses_g_not_g2", "f.c2 * (g * g)", "f.c2 * g"),
    ("v_from_m", "f.b2 * V[i]", "f.b2 * M[i]"),
    ("eps_inside_sqrt", "std::sqrt(v1) * f.rb + f.e", "std::sqrt(v1 + f.e) * f.rb"),
    ("rb_not_applied", "std::sqrt(v1) * f.rb + f.e", "std::sqrt(v1) + f.e"),
    ("multiply_not_divide", "float u = m1 / d;", "float u = m1 * d;"),
    ("ascent_sign", "f.dk * P[i] - f.ss * u", "f.dk * P[i] + f.ss * u"),
    ("decay_on_update", "f.dk * P[i] - f.ss * u", "P[i] - f.ss * u * f.dk"),
    ("bias1_off_by_one", "std::pow(hp.beta1, (double)t)", "std::pow(hp.beta1, (double)(t + 1))"),
    ("no_bias1", "f.ss = (float)(hp.lr / (1.0 - std::pow(hp.beta1, (double)t)));", "f.ss = (float)hp.lr;"),
    ("bias2_uses_beta1", "std::pow(hp.beta2, (double)t)", "std::pow(hp.beta1, (double)t)"),
    ("decay_not_lr_scaled", "(1.0 - hp.lr * hp.weight_decay)", "(1.0 - hp.weight_decay)"),
    ("fold_in_fp32", "f.c1 = (float)(1.0 - hp.beta1);", "f.c1 = 1.0f - (float)hp.beta1;"),
    ("bf16_truncates", "return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)(u >> 16);"),
    ("bf16_ties_up", "return (uint16_t)((u + 0x7FFFu + lsb) >> 16);", "return (uint16_t)((u + 0x8000u) >> 16);"),
    ("bf16_nan_to_inf", "return 0x7FC0;  // NaN", "return (uint16_t)(u >> 16) & 0xFF80;  // NaN"),
    ("copy_from_wrong_value", "B[i] = to_bf16(p1);", "B[i] = to_bf16(m1);"),
    ("state_bytes_fp32_grad", "return 4 + 2 + 2 + 4 + 4;", "return 4 + 2 + 4 + 4 + 4;"),
    # two-pass form
    ("f16_truncates", "const uint32_t r = (a + 0xFFFu + lsb) >> 13;", "const uint32_t r = a >> 13;"),
    ("f16_subnormal_scale", "const float q = f * 0x1p24f;", "const float q = f * 0x1p23f;"),
    ("f16_decode_bias", "u = sign | ((uint32_t)(exp - 15 + 127) << 23) | (man << 13);",
     "u = sign | ((uint32_t)(exp - 16 + 127) << 23) | (man << 13);"),
    ("unscale_multiplies", "gbar[i] = (s / (float)N) * inv;", "gbar[i] = (s / (float)N) * (float)loss_scale;"),
    ("norm_not_squared", "acc += (double)gbar[i] * (double)gbar[i];", "acc += std::fabs((double)gbar[i]);"),
    ("clip_no_min", "return (float)(c < 1.0 ? c : 1.0);", "return (float)c;"),
    ("clip_no_eps", "const double c = max_norm / (std::sqrt(total_sq) + 1e-6);", "const double c = max_norm / total_sq;"),
    ("overflow_not_skipped", "if (skip_nonfinite && !std::isfinite(total_sq)) return 2;", ""),
    ("clip_coef_unused", "const float g = gbar[i] * k;", "const float g = gbar[i];"),
    ("scaler_no_hysteresis", "if (s->overflows >= s->hysteresis) {", "if (s->overflows >= 1) {"),
    ("scaler_window_off_by_one", "if (s->clean >= s->window) {", "if (s->clean > s->window) {"),
    ("scaler_no_floor", "s->scale = s->scale / 2.0 < s->min_scale ? s->min_scale : s->scale / 2.0;",
     "s->scale = s->scale / 2.0;"),
    # the other readings of hysteresis: the budget restored at every halving, by any clean step, or never
    ("scaler_budget_restored_on_halving",
     "s->scale = s->scale / 2.0 < s->min_scale ? s->min_scale : s->scale / 2.0;",
     "s->scale = s->scale / 2.0 < s->min_scale ? s->min_scale : s->scale / 2.0; s->overflows = 0;"),
    ("scaler_budget_restored_on_clean", "  s->clean += 1;\n", "  s->clean += 1;\n  s->overflows = 0;\n"),
    ("scaler_budget_never_restored", "    s->overflows = 0;  // growth restores the budget", ""),
    ("scaler_overflow_keeps_clean_run", "    s->clean = 0;\n    if (s->overflows < s->hysteresis)",
     "    if (s->overflows < s->hysteresis)"),
]


def test_mutations_apply_once():
    src = open(SRC, encoding="utf-8").read()
    for name, old, _new in MUTANTS:
        assert src.count(old) >= 1, f"mutant {name}: text not found in oracle.cpp"


@pytest.mark.parametrize("name,old,new", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_mutant_is_caught(name, old, new):
    src = open(SRC, encoding="utf-8").read()
    mutated = src.replace(old, new)
    assert mutated != src
    with tempfile.TemporaryDirectory() as d:
        cpp = os.path.join(d, "oracle_mutant.cpp")
        with open(cpp, "w", encoding="utf-8") as f:
            f.write(mutated)
        lib = ob.build(src=cpp, out=os.path.join(d, "liboracle_mutant.so"))
        o = oracle.Oracle(lib)
        caught = None
        for pin in pins.ALL:
            try:
                pin(o)
            except AssertionError as e:
                caught = f"{pin.__name__}: {str(e)[:80]}"
            except (ValueError, FloatingPointError, ZeroDivisionError) as e:
                caught = f"{pin.__name__}: {type(e).__name__}"
            if caught:
                break
        assert caught, f"mutant {name} passed every pin"
