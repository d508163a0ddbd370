"""The oracle's pins have teeth: each plausible mistake, planted in a copy of
oracle.c (compiled with gcc on the CPU, the same flags), makes at least one
pin of tests/test_oracle.py fail.  The library under test is not involved.

Every mutant keeps every memory access in bounds (a skipped row, a permuted
in-range index, a changed constant), so a failing pin is a wrong value, never
a crash."""
import contextlib
import ctypes
import os
import subprocess

import pytest

import oracle
import test_oracle as pins

SRC = os.path.join(os.path.dirname(oracle.__file__), "oracle.c")


def _function_span(text, signature):
    start = text.index(signature)
    end = text.index("\n}\n", start) + 3
    return start, end


# (name, function it lives in, [(text, replacement), ...])
MUTANTS = [
    ("side step unfused (two roundings)", "void oracle_epilogue_i8_ex(",
     [("        if (use_side)                    /* (2) side input, single rounding */\n"
       "          t = fmaf((float)side[i], side_input_scale, t);",
       "        if (use_side)\n"
       "          t = (float)side[i] * side_input_scale + t;")]),
    ("scale and bias contracted into one fma", "void oracle_epilogue_i8_ex(",
     [("        t = t * cis;                     /* (1) scale */",
       "        t = use_side ? t * cis : fmaf(t, cis, bias[k]);"),
      ("        t = t + bias[k];                 /* (3) bias */",
       "        if (use_side) t = t + bias[k];")]),
    ("round half away from zero", "void oracle_epilogue_i8_ex(",
     [("      t = nearbyintf(t);", "      t = roundf(t);")]),
    ("int32 -> fp32 conversion truncates toward zero", "void oracle_epilogue_i8_ex(",
     [("      float t = (float)acc[i];          /* int32 -> fp32, round to nearest even */",
       "      float t = (float)(double)(acc[i] / (1 << (acc[i] > 16777216 || acc[i] < -16777216))"
       " * (1 << (acc[i] > 16777216 || acc[i] < -16777216)));")]),
    ("int32 -> fp32 conversion rounds ties up", "void oracle_epilogue_i8_ex(",
     [("      float t = (float)acc[i];          /* int32 -> fp32, round to nearest even */",
       "      float t = (float)((acc[i] > 16777216 && (acc[i] & 1)) ? (long)acc[i] + 1 : acc[i]);")]),
    ("clip lower bound -127", "void oracle_epilogue_i8_ex(",
     [("  const float lo = relu ? 0.0f : -128.0f;", "  const float lo = relu ? 0.0f : -127.0f;")]),
    ("SAME padding: the odd pixel before", "int oracle_geometry(",
     [("    pt = prow / 2;", "    pt = prow - prow / 2;")]),
    ("filter flipped (direct form)", "int oracle_conv_i8_direct(",
     [("int64_t wv = w[((r * s.S + q) * s.C + c) * s.K + k];",
       "int64_t wv = w[(((s.R - 1 - r) * s.S + (s.S - 1 - q)) * s.C + c) * s.K + k];")]),
    ("filter read transposed (im2col form)", "int oracle_conv_i8_im2col(",
     [("(int64_t)w[j * s.K + k];", "(int64_t)w[(j % s.K) * depth + (j / s.K) + k * 0];")]),
    ("first input row skipped", "int oracle_conv_i8_direct(",
     [("if (hi < 0 || hi >= s.H) continue; /* zero padding */",
       "if (hi < 1 || hi >= s.H) continue; /* zero padding */")]),
    ("batch norm without the mean", "void oracle_epilogue_float_ex(",
     [("(t - (double)mean[k])", "(t)")]),
    ("leaky ReLU drops the input", "void oracle_epilogue_float_ex(",
     [("if (!(t > 0.0)) t = (double)alpha * t;", "if (!(t > 0.0)) t = (double)alpha;")]),
    ("weight gradient ignores the left pad", "int oracle_wgrad_direct(",
     [("long wi = wo * s.sw - s.pl + q;", "long wi = wo * s.sw + q;")]),
    ("weight gradient taps transposed", "int oracle_wgrad_direct(",
     [("double* out = dw + ((r * s.S + q) * s.C + c) * s.K;",
       "double* out = dw + ((q * s.R + r) * s.C + c) * s.K;")]),
]

# Pins tried for every mutant, cheapest first; the first failure settles it.
PINS = [
    pins.test_size_formulas_grid,
    pins.test_epilogue_hand_values,
    pins.test_epilogue_crafted_fma_and_contraction_cases,
    pins.test_epilogue_variant_hand_values,
    pins.test_tie_dense_rounding_is_half_even,
    pins.test_delta_filter_strided_asymmetric_pad,
    pins.test_identity_filter_passes_through,
    pins.test_constant_closed_form,
    pins.test_1x1_stride1_is_gemm,
    pins.test_full_size_valid_is_gemm,
    pins.test_float_epilogue_against_torch_batch_norm,
    lambda: pins.test_float_activations_against_torch("leaky_relu", 0.1, 0.0),
    pins.test_wgrad_of_a_delta_gradient_is_the_patch,
    lambda: [pins.test_wgrad_against_torch(seed) for seed in range(12)],
    pins.test_brute_force_tiny_shapes_both_forms,
    pins.test_brute_force_float_paths,
]


@contextlib.contextmanager
def _mutant(text, tmp_path):
    src = tmp_path / "oracle_mutant.c"
    lib_path = tmp_path / "liboracle_mutant.so"
    src.write_text(text)
    subprocess.run(["gcc", *oracle.CFLAGS, str(src), "-o", str(lib_path), "-lm"], check=True)
    saved = oracle._lib
    oracle._lib = oracle._bind(ctypes.CDLL(str(lib_path)))
    try:
        yield
    finally:
        oracle._lib = saved


def test_mutation_sites_exist_once():
    text = open(SRC).read()
    for name, func, edits in MUTANTS:
        a, b = _function_span(text, func)
        for old, _new in edits:
            assert text[a:b].count(old) == 1, name


@pytest.mark.parametrize("name,func,edits", MUTANTS, ids=[m[0] for m in MUTANTS])
def test_planted_mistake_fails_a_pin(name, func, edits, tmp_path):
    text = open(SRC).read()
    a, b = _function_span(text, func)
    body = text[a:b]
    for old, new in edits:
        body = body.replace(old, new)
    mutated = text[:a] + body + text[b:]
    assert mutated != text
    with _mutant(mutated, tmp_path):
        for pin in PINS:
            try:
                pin()
            except AssertionError:
                return  # caught
    pytest.fail("no pin caught the planted mistake: %s" % name)
