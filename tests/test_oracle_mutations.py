"""Planted mistakes in the oracle must each fail at least one pin (CPU only).

Mutated copies of ``oracle/q8_oracle.c`` are built with gcc in a temporary
directory and loaded in place of the real library; mutated bound functions
are swapped into the ``oracle`` module. Each mutant is one plausible slip
(a wrong block index, unsigned quants, a flushed subnormal, a wrong
exponent bias, fp32 accumulation, swapped scale bytes, a wrong token
stride, a transposed output, a dropped term, a lost sign, a bound made
looser). The pins run against it; a mutant that no pin notices fails this
test. The real oracle is restored afterwards.
"""
import contextlib
import os
import shutil
import subprocess

import numpy as np
import pytest

import oracle
from tests import test_oracle_bounds as B
from tests import test_oracle_pins as P
from tests.golden_io import load_handbuilt

SRC = os.path.join(os.path.dirname(oracle.__file__), "q8_oracle.c")

# (name, text in q8_oracle.c, replacement); each text occurs exactly once
C_MUTANTS = [
    ("wrong block index", "or_half_to_double(drow[k / OR_QK])", "or_half_to_double(drow[(k + 1) / OR_QK])"),
    ("unsigned quants", "* (double)qrow[k];", "* (double)(uint8_t)qrow[k];"),
    ("flushed subnormals", "v = ldexp((double)f, -24);", "v = 0.0;"),
    ("wrong exponent bias", "ldexp((double)(1024 + f), e - 25)", "ldexp((double)(1024 + f), e - 24)"),
    ("fp32 accumulation", "double s = 0.0, t = 0.0;", "float s = 0.0f; double t = 0.0;"),
    ("swapped scale bytes", "(uint16_t)(p[0] | (p[1] << 8))", "(uint16_t)(p[1] | (p[0] << 8))"),
    ("wrong token stride", "j->ldx = K;", "j->ldx = M;"),
    ("transposed output", "&j->y[n * j->R + i], &j->a[n * j->R + i]",
     "&j->y[i * j->N + n], &j->a[i * j->N + n]"),
    ("dropped last term", "        s = s + p;", "        if (k != K - 1) s = s + p;"),
    ("lost sign", "return sign ? -v : v;", "return v;"),
    ("signed magnitude sum", "t = t + fabs(p);", "t = t + p;"),
]


def _c_pins():
    """The pins that exercise q8_oracle.c, as plain calls."""
    pins = [P.test_half_decoder_all_finite_patterns, P.test_half_decoder_specials,
            P.test_block_decoder_roundtrip_random, P.test_subnormal_scale_and_activation,
            P.test_zero_blocks_contribute_exactly_zero, P.test_per_block_scales_equal_block_decomposition,
            P.test_matches_float64_matmul_of_dequantized_weights,
            P.test_fp32_emulation_inside_higham_bound, P.test_threads_and_sampled_rows_agree,
            P.test_bruteforce_fraction_fp32_x]
    pins += [lambda c=c: P.test_golden_handbuilt(c) for c in load_handbuilt()]
    pins += [lambda s=s, k=k: P.test_bruteforce_fraction(s, k) for s in (0, 1) for k in (32, 96)]
    pins += [lambda j=j: P.test_unit_vector_recovers_each_int8(j) for j in (0, 31, 32, 95)]
    pins += [lambda s=s: P.test_power_of_two_scaling_is_exact(s) for s in (-4, 3)]
    pins += [lambda a=a: P.test_integer_exact_equals_int64_matmul(*a)
             for a in ((24, 640, 3), (640, 96, 2))]
    return pins


def _failures(pins):
    bad = 0
    for pin in pins:
        try:
            pin()
        except Exception:  # an assertion, or a mutant that breaks a call outright
            bad += 1
    return bad


@contextlib.contextmanager
def _oracle_library(path):
    saved_lib, saved_path = oracle._lib, oracle._LIB
    oracle._lib, oracle._LIB = None, path
    try:
        oracle._get()
        yield
    finally:
        oracle._lib, oracle._LIB = saved_lib, saved_path


def _build(src_text, out_dir, name):
    c = os.path.join(out_dir, name + ".c")
    so = os.path.join(out_dir, name + ".so")
    with open(c, "w") as f:
        f.write(src_text)
    subprocess.run(["gcc", "-O1", "-std=c99", "-ffp-contract=off", "-fno-fast-math", "-fPIC",
                    "-shared", "-o", so, c, "-lpthread", "-lm"], check=True)
    return so


@pytest.fixture(scope="module")
def src_text():
    with open(SRC) as f:
        return f.read()


def test_unmutated_copy_passes_every_pin(src_text, tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    so = _build(src_text, str(tmp_path), "clean")
    with _oracle_library(so):
        assert _failures(_c_pins()) == 0


@pytest.mark.parametrize("name,old,new", C_MUTANTS, ids=[m[0] for m in C_MUTANTS])
def test_c_mutant_fails_a_pin(src_text, tmp_path, name, old, new):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not available")
    assert src_text.count(old) == 1, f"mutation site for {name!r} not found exactly once"
    so = _build(src_text.replace(old, new), str(tmp_path), "mutant")
    with _oracle_library(so):
        assert _failures(_c_pins()) >= 1, f"no pin notices: {name}"


def _scaled(fn, k):
    return lambda *a, **kw: k * fn(*a, **kw)


# (name, attribute, replacement factory, pins that should notice)
PY_MUTANTS = [
    ("router bound 8x looser", "topk_softmax_bound", lambda f: _scaled(f, 8.0),
     [B.test_router_bound_contains_fp32_emulation, B.test_router_bound_rejects_precision_mistakes]),
    ("silu*mul bound 2x looser", "silu_mul_bound", lambda f: _scaled(f, 2.0),
     [B.test_silu_mul_bound_is_reached_near_the_steepest_point]),
    ("silu*mul bound halved", "silu_mul_bound", lambda f: _scaled(f, 0.5),
     [B.test_silu_mul_bound_contains_fp32_emulation, B.test_silu_mul_bound_is_reached_near_the_steepest_point]),
    ("sigmoid bound 2x looser", "sigmoid_bound", lambda f: _scaled(f, 2.0),
     [B.test_sigmoid_bound_contains_fp32_emulation_and_is_reached_at_zero]),
    ("down bound 2x looser", "down_bound", lambda f: _scaled(f, 2.0),
     [B.test_down_bound_adversarial_input_reaches_it, B.test_moe_ffn_bound_reached_by_stagewise_worst_case]),
    ("combine bound 2x looser", "combine_bound", lambda f: _scaled(f, 2.0),
     [B.test_combine_bound_reached_and_contains_fp32_sum, B.test_moe_ffn_bound_reached_by_stagewise_worst_case]),
    ("gated add bound 2x looser", "gated_add_bound", lambda f: _scaled(f, 2.0),
     [B.test_gated_add_bound_reached_and_contains_fp32_fma, B.test_shared_expert_bound_reached_by_worst_case]),
    ("fp16 half-ulp doubled", "fp16_ulp", lambda f: _scaled(f, 2.0),
     [B.test_fp16_output_bound_half_ulp_is_tight_for_subnormal_outputs]),
    ("silu sign lost", "silu", lambda f: (lambda z: np.abs(f(z))),
     [P.test_silu_closed_forms, P.test_gate_up_silu_closed_forms]),
    ("sigmoid mirrored", "sigmoid", lambda f: (lambda z: f(-np.asarray(z))),
     [P.test_sigmoid_closed_forms]),
]


@pytest.mark.parametrize("name,attr,make,pins", PY_MUTANTS, ids=[m[0] for m in PY_MUTANTS])
def test_bound_mutant_fails_a_pin(monkeypatch, name, attr, make, pins):
    monkeypatch.setattr(oracle, attr, make(getattr(oracle, attr)))
    assert _failures(pins) >= 1, f"no pin notices: {name}"
