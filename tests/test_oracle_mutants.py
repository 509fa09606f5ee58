"""The pins must reject plausible mistakes in the oracle.

Each case compiles a copy of oracle/onebit_oracle.c with one deliberate mistake
(a wrong sign, a dropped term, a transposed operand, a wrong index or bit order),
routes the oracle through it, and requires at least one pin to fail.  Mistakes are
planted only in CPU copies of the oracle.
"""
import os
import tempfile

import pytest

import oracle
from oracle import build as obuild

import test_oracle_average as TA
import test_oracle_compress as TC  # noqa: E402
import test_oracle_qsdp as TQ
import test_oracle_loco as TL
import test_oracle_qsgd as TG
import test_oracle_server as TS
import test_oracle_warmup as TW

SRC = open(os.path.join(os.path.dirname(obuild.__file__), "onebit_oracle.c")).read()


def _warm():
    TW.test_constant_gradient_closed_form(False)
    TW.test_constant_gradient_closed_form(True)
    TW.test_matches_torch(TW.torch.optim.AdamW, 0.01)


def _comp():
    TC.test_compressor_against_library_routines_and_invariants()
    TC.test_zero_and_extreme_chunks()
    TC.test_identity_compressor_is_momentum_sgd_closed_form()
    TC.test_error_feedback_telescopes(0.9)
    TC.test_mask_pins_masked_tensors_and_leaves_others_alone()
    TC.test_mask_inside_shared_chunks_with_nonzero_gradient()
    TC.test_bf16_copy_matches_torch_rounding()
    TC.test_bf16_rounding_special_values_match_torch()


def _serv():
    TS.test_server_brute_force(3)
    TS.test_single_worker_server_reproduces_worker_stream()
    TS.test_decompress_matches_unpackbits()


def _qsdp():
    TQ.test_lattice_values_are_exact_for_every_seed(4)
    TQ.test_degenerate_buckets_and_ragged_tail()
    TQ.test_philox_known_answers()
    TQ.test_philox_element_stream_matches_independent_implementations("torch")
    TQ.test_unbiased_and_variance_closed_form_brute_force(8)


def _qsgd():
    TG.test_integer_ratio_buckets_are_exact(False)
    TG.test_lone_value_zero_bucket_signed_zero_and_padding()
    TG.test_norm_is_the_rounded_exact_norm()
    TG.test_unbiased_and_variance_closed_form(4)
    TG.test_average_of_workers()
    TG.test_decode_is_exact_average_rounded_once(8, 1, 0)
    TG.test_decode_is_exact_average_rounded_once(4, 3, 18)
    TG.test_lone_value_decodes_to_itself_over_the_whole_range()


def _loco():
    TL.test_zero_average_is_plain_qsgd_and_error(4)
    TL.test_beta_zero_is_error_feedback(8)
    TL.test_moving_average_closed_form(0.9)


def _avg():
    TA.test_one_row_copies_and_negation()
    TA.test_exact_mean_rounded_once(3, False)
    TA.test_exact_mean_rounded_once(5, True)


def _finish():
    TS.test_worker_server_finish_composition_equals_fused_step()
    TS.test_momentum_update_mask_and_closed_form()


MUTANTS = [
    # (name, original text, mistaken text, pins expected to catch it)
    ("warmup g^2 dropped", "ob2 * (gi * gi)", "ob2 * gi", _warm),
    ("warmup eps inside sqrt", "mhat / (sqrtf(vhat) + eps)", "mhat / sqrtf(vhat + eps)", _warm),
    ("warmup bias correction inverted", "mi / bc1 : mi", "mi * bc1 : mi", _warm),
    ("warmup weight decay sign", "+ weight_decay * x[i];\n        x[i] = x[i] - lr * update;\n    }\n    return",
     "- weight_decay * x[i];\n        x[i] = x[i] - lr * update;\n    }\n    return", _warm),
    ("momentum operands transposed", "beta1 * m[i] + ob1 * g[i]", "beta1 * g[i] + ob1 * m[i]", _comp),
    ("error added with wrong sign", "c[k] = m1 + e[i];", "c[k] = m1 - e[i];", _comp),
    ("sign of zero", "q = (c[k] < 0.0f) ? -scale : scale;", "q = (c[k] <= 0.0f) ? -scale : scale;", _comp),
    ("bit order reversed", "                bits[wbase + (k >> 5)] |= 1u << (k & 31);",
     "                bits[wbase + (k >> 5)] |= 1u << (31 - (k & 31));", _comp),
    ("scale normalisation", "sqrt(s) / sqrt((double)n)", "sqrt(s) / (double)n", _comp),
    ("error residual sign", "float e_new = c[k] - q;", "float e_new = q - c[k];", _comp),
    ("mask forgets e", "                m_new = 0.0f;\n                e_new = 0.0f;", "                m_new = 0.0f;", _comp),
    ("update ignores weight decay", "m_new / (sqrtf(v[i]) + eps) + weight_decay * x[i]",
     "m_new / (sqrtf(v[i]) + eps)", _comp),
    ("bf16 ties away", "lower > 0x8000u ||", "lower >= 0x8000u ||", _comp),
    ("server average not divided", "(float)(sum / (double)W)", "(float)(sum)", _serv),
    ("server sign flipped", "sum += ((word >> (k & 31)) & 1u) ? -s : s;", "sum += ((word >> (k & 31)) & 1u) ? s : -s;",
     _serv),
    ("server error sign", "server_error[o + k] = c[k] - q;", "server_error[o + k] = q - c[k];", _serv),
    ("qsdp rounds the wrong way", "(uint64_t)u < thr ? 1u : 0u", "(uint64_t)u >= thr ? 1u : 0u", _qsdp),
    ("qsdp nibble order", "codes[i >> 1] |= (uint8_t)(code << ((i & 1) ? 4 : 0));",
     "codes[i >> 1] |= (uint8_t)(code << ((i & 1) ? 0 : 4));", _qsdp),
    ("qsdp levels off by one", "const float delta = (mx - mn) / (float)L;", "const float delta = (mx - mn) / (float)(L + 1);",
     _qsdp),
    ("philox wrong high half", "const uint32_t y0 = hi1 ^ x1 ^ k0;", "const uint32_t y0 = hi0 ^ x1 ^ k0;", _qsdp),
    ("philox word index", "return out[i & 3];", "return out[0];", _qsdp),
    ("qsgd rounds the wrong way", "first_index + lo + k) < thr ? 1u : 0u", "first_index + lo + k) >= thr ? 1u : 0u", _qsgd),
    ("qsgd sign of zero", "(v[k] < 0.0f ? 1u << (nbits - 1) : 0u)", "(v[k] <= 0.0f ? 1u << (nbits - 1) : 0u)", _qsgd),
    ("qsgd s + 1 levels", "const float u = t * (float)s;", "const float u = t * (float)(s + 1);", _qsgd),
    ("qsgd norm not square-rooted", "const float norm = (float)sqrt(bucket_sum_squares(v, len));",
     "const float norm = (float)bucket_sum_squares(v, len);", _qsgd),
    ("qsgd decode scale", "const double sW = (double)((1u << (nbits - 1)) - 1u) * (double)W;",
     "const double sW = (double)(1u << (nbits - 1)) * (double)W;", _qsgd),
    ("qsgd level spacing rounded to fp32 first", "(double)level * (double)norms[i / bucket];",
     "(double)level * (double)(norms[i / bucket] / (float)s) * (double)s;", _qsgd),
    ("qsgd level times norm rounded to fp32", "            acc += qsgd_value_times_s(",
     "            acc += (double)(float)qsgd_value_times_s(", _qsgd),
    ("qsgd pack nibble order", "codes[i >> 1] |= (uint8_t)((i & 1) ? code << 4 : code);",
     "codes[i >> 1] |= (uint8_t)((i & 1) ? code : code << 4);", _qsgd),
    ("qsgd decode nibble order", "(uint32_t)((codes[i >> 1] >> ((i & 1) ? 4 : 0)) & 0xfu)",
     "(uint32_t)((codes[i >> 1] >> ((i & 1) ? 0 : 4)) & 0xfu)", _qsgd),
    ("qsgd average not divided", "const float y = (float)(acc / sW);", "const float y = (float)(acc / (sW / (double)W));",
     _qsgd),
    ("loco compensation sign", "h[i] = gi + err_avg[i];", "h[i] = gi - err_avg[i];", _loco),
    ("loco weights swapped", "err_avg[i] = beta * err_avg[i] + one_minus_beta * (h[i] - y[i]);",
     "err_avg[i] = one_minus_beta * err_avg[i] + beta * (h[i] - y[i]);", _loco),
    ("loco error sign", "err_avg[i] = beta * err_avg[i] + one_minus_beta * (h[i] - y[i]);",
     "err_avg[i] = beta * err_avg[i] + one_minus_beta * (y[i] - h[i]);", _loco),
    ("average summed in fp32", "            sum += (double)g[(int64_t)w * row_stride + i];",
     "            sum = (double)((float)sum + g[(int64_t)w * row_stride + i]);", _avg),
    ("average not divided", "        const double mean = sum / (double)W;", "        const double mean = sum;", _avg),
    ("average skips the last row", "        for (int w = 0; w < W; ++w)\n            sum +=",
     "        for (int w = 0; w + 1 < W; ++w)\n            sum +=", _avg),
    ("finish ignores the mask", "m[i] = m[i] * (mask[i] ? 1.0f : 0.0f);", "m[i] = m[i];", _finish),
    ("finish weight decay sign", "const float update = m[i] / (sqrtf(v[i]) + eps) + weight_decay * x[i];",
     "const float update = m[i] / (sqrtf(v[i]) + eps) - weight_decay * x[i];", _finish),
]


@pytest.mark.parametrize("name,old,new,pins", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_pins_reject_mutant(name, old, new, pins):
    assert SRC.count(old) == 1, f"mutation anchor for '{name}' must occur exactly once"
    with tempfile.TemporaryDirectory() as d:
        lib = obuild.build_from_text(SRC.replace(old, new), os.path.join(d, "liboracle_mutant.so"))
        with oracle.use_library(lib):
            with pytest.raises((AssertionError, RuntimeError)):
                pins()
