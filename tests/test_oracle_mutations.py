"""The pins are strong enough: plausible mistakes planted in the oracle (on the
CPU, in throw-away copies) each make at least one pin fail.

C mistakes are planted in a copy of zero_oracle.c, built to a temporary
library and swapped in; Python mistakes replace one function of the oracle
module for the duration of a check.
"""
import inspect
import os
import textwrap

import numpy as np
import pytest

import oracle
import test_oracle_arith as A
import test_oracle_layout as L
import test_oracle_pages as PG
import test_oracle_state_bytes as SB

SRC = os.path.join(os.path.dirname(oracle.__file__), "zero_oracle.c")

# Cheap probes first: a mutant usually fails within the first few.
C_PROBES = [
    A.test_sum_order_is_rank_order_in_fp32, A.test_negative_zero_sum_starts_at_plus_zero,
    A.test_accumulate_starts_from_out, A.test_overflow_and_nan_propagate,
    A.test_division_is_correctly_rounded_for_any_divisor, lambda: A.test_dyadic_inputs_are_exact(4),
    A.test_single_rank_divisor_one_is_widening, A.test_gradient_accumulation_is_rank_reduce_with_divisor_one,
    A.test_grad_check_closed_forms, lambda: A.test_grad_check_flags_non_finite(7, np.nan),
    A.test_grad_check_sum_matches_fsum, PG.test_first_step_python_and_c,
    A.test_first_step_closed_form_any_betas, A.test_zero_betas_any_step_and_pure_decay,
    lambda: A.test_adam_matches_torch_float64(True, 0.01), lambda: A.test_adam_matches_torch_float64(False, 0.05),
    A.test_clip_coefficient_scales_the_gradient, PG.test_resume_lab_printed_values,
    A.test_owner_step_is_reduce_then_adam_then_cast_over_real_elements,
    A.test_decoders_are_exact, A.test_f16_encoder_matches_numpy, A.test_bf16_encoder_matches_torch,
    A.test_reduce_add_rounds_the_mean_before_adding, A.test_reduce_add_dyadic_microsteps_are_exact,
]

C_MUTANTS = {
    "first moment uses beta2": ("(1.0 - h->beta1) * grad", "(1.0 - h->beta2) * grad"),
    "second moment not bias-corrected": ("second / (1.0 - pow(h->beta2, (double)h->step))", "second"),
    "eps inside the square root": ("(sqrt(vhat) + h->eps)", "sqrt(vhat + h->eps)"),
    "decoupled decay sign": ("(1.0 - h->lr * h->weight_decay)", "(1.0 + h->lr * h->weight_decay)"),
    "L2 term sign": ("grad = grad + h->weight_decay * weight", "grad = grad - h->weight_decay * weight"),
    "clip factor dropped": ("double grad = g * h->clip_coef;", "double grad = g;"),
    "reduce starts at -0": ("accumulate ? out[i] : 0.0f", "accumulate ? out[i] : -0.0f"),
    "ranks summed in reverse": ("for (uint32_t r = 0; r < R; ++r) s = s + widen(grads[r], dtype, i);",
                                "for (uint32_t r = R; r-- > 0;) s = s + widen(grads[r], dtype, i);"),
    "sum kept in double": ("  float s = start;\n", "  double s = start;\n"),
    "division by reciprocal": ("return s / divisor;", "return s * (1.0f / divisor);"),
    "ties away from zero": ("rem == 0.5 && fmod(kr, 2.0) != 0.0", "rem == 0.5"),
    "subnormals not handled": ("if (e < 1 - bias) e = 1 - bias;", ""),
    "NaN not flagged": ("if (!isfinite(x)) flag = 1;", "if (isinf(x)) flag = 1;"),
    "accumulator not reset": ("const float base = first ? 0.0f : acc[i];", "const float base = acc[i];"),
    "norm sums |g|": ("const double sq = x * x;", "const double sq = fabs(x);"),
    "bf16 bias off by one": ("decode16(b, 10, 15) : decode16(b, 7, 127)", "decode16(b, 10, 15) : decode16(b, 7, 126)"),
    "rank index uses the owner base": (
        "g = reduce_one(R, gdtype, grads, (uint64_t)f - grad_base, 0.0f, divisor);",
        "g = reduce_one(R, gdtype, grads, (uint64_t)f - local_base, 0.0f, divisor);"),
    "write-back always bf16": ("pdtype == OR_F16 ? oracle_f32_to_f16(wf) : oracle_f32_to_bf16(wf)",
                               "oracle_f32_to_bf16(wf)"),
    "per-backward add before the division": (
        "const float reduced = reduce_one(R, dtype, grads, (uint64_t)i, 0.0f, divisor);\n    out[i] = out[i] + reduced;",
        "out[i] = reduce_one(R, dtype, grads, (uint64_t)i, out[i], divisor);"),
}


def _fails(probes):
    for p in probes:
        try:
            p()
        except (AssertionError, ValueError):
            return True
    return False


@pytest.mark.parametrize("name", list(C_MUTANTS))
def test_c_mutant_is_caught(name, tmp_path, monkeypatch):
    old, new = C_MUTANTS[name]
    text = open(SRC).read()
    assert text.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    src = tmp_path / "mutant.c"
    src.write_text(text.replace(old, new))
    path = oracle.build(str(src), str(tmp_path / "libmutant.so"))
    monkeypatch.setattr(oracle, "_lib", oracle.load(path))
    assert _fails(C_PROBES), f"no pin catches the planted mistake: {name}"


PY_PROBES = [
    L.test_eleven_over_four, L.test_tiny_brute_force_all_P_R, L.test_padded_layout_against_slots,
    SB.test_printed_table_1p5e9_4_ranks, SB.test_printed_asserts, SB.test_memory_matrix_identity,
    SB.test_parameter_storage_printed, PG.test_first_step_python_and_c, PG.test_sharded_equals_unsharded_lab,
    PG.test_resume_lab_printed_values, PG.test_mean_of_squares_is_not_square_of_mean,
    A.test_grad_check_closed_forms, SB.test_stage3_gather_sizes_match_parameter_storage_and_rebuild_tensors,
]

PY_MUTANTS = {
    "ceil ownership": ("owner_ranges", "parameters * r // ranks", "(parameters * r + ranks - 1) // ranks"),
    "last tensor unpadded": ("layout", "total += -(-n // align) * align", "total += n if n == numels[-1] else -(-n // align) * align"),
    "no padding": ("layout", "total += -(-n // align) * align", "total += n"),
    "ZeRO-2 keeps full grads": ("state_bytes", '"grad": 2', '"grad": 3'),
    "ZeRO-1 shards params": ("state_bytes", '"param": 3', '"param": 1'),
    "DP shards the optimizer state": ("state_bytes", '"optimizer": 1', '"optimizer": 0'),
    "bias correction with beta1": ("adam_step", "vhat = second / (1.0 - beta2 ** step)",
                                   "vhat = second / (1.0 - beta1 ** step)"),
    "floor shards in stage 3": ("parameter_storage", "shard = n // ranks + (1 if n % ranks else 0)",
                                "shard = n // ranks"),
    "gather buffer aliases the shard": ("parameter_storage", "gathered += ranks * shard",
                                        "gathered += (ranks - 1) * shard"),
    "owner updates from one rank's gradient": ("compare_owned_updates",
                                               "states[k] = adam_step(*states[k], rank_mean(g, i), t)",
                                               "states[k] = adam_step(*states[k], g[0][i], t)"),
    "rank mean over one rank too many": ("compare_owned_updates", "return total / ranks",
                                         "return total / (ranks + 1)"),
    "clip never clamps": ("clip_coef", "return min(1.0, max_norm / (math.sqrt(sumsq) + eps))",
                          "return max_norm / (math.sqrt(sumsq) + eps)"),
    "stage-3 shard starts at the floor split": ("stage3_shards", "e = r * s + j", "e = r * n // ranks + j"),
    "stage-3 gather in tensor order": ("stage3_gather", "for k in live:", "for k in sorted(live):"),
}


@pytest.mark.parametrize("name", list(PY_MUTANTS))
def test_python_mutant_is_caught(name, monkeypatch):
    fn, old, new = PY_MUTANTS[name]
    src = textwrap.dedent(inspect.getsource(getattr(oracle, fn)))
    assert src.count(old) == 1, f"mutation site for '{name}' not found exactly once"
    ns = {}
    exec(compile(src.replace(old, new), f"<mutant {name}>", "exec"), oracle.__dict__, ns)
    monkeypatch.setattr(oracle, fn, ns[fn])
    assert _fails(PY_PROBES), f"no pin catches the planted mistake: {name}"
