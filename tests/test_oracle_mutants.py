"""The oracle's pins must reject plausible mistakes.

Each case copies oracle/ssd_oracle.c to a temporary directory, plants one
mistake with a textual substitution (the committed source is never touched),
compiles the copy with gcc and runs every pin of test_oracle.py against it.
At least one pin must fail for every mutant.  The step-size preparation
(oracle/dt.py) is treated the same way: a mutated copy of its text is
executed in a fresh namespace and run against the step-size pins.
"""
import os
import subprocess

import pytest

import oracle
from test_oracle import ALL_PINS, DT_PINS

SRC = os.path.join(os.path.dirname(oracle.__file__), "ssd_oracle.c")

MUTANTS = {
    # output read from the state before token t is absorbed
    "output_before_update": (
        "row[n] = alpha * row[n] + u * (double)bt[n];\n                    acc += row[n] * (double)ct[n];",
        "acc += row[n] * (double)ct[n];\n                    row[n] = alpha * row[n] + u * (double)bt[n];"),
    "skip_term_dropped": ("yt[p] = acc + d_h * (double)xt[p];", "yt[p] = acc;"),
    "decay_sign_flipped": ("exp(dtv * a_h)", "exp(-dtv * a_h)"),
    "decay_without_dt": ("exp(dtv * a_h)", "exp(a_h)"),
    "input_without_dt": ("const double u = dtv * (double)xt[p];", "const double u = (double)xt[p];"),
    "B_and_C_swapped": ("const float* bt = Bm +", "const float* bt = Cm +"),
    "wrong_group_mapping": ("g = h / heads_per_group;", "g = h % G;"),
    "init_state_ignored": ("if (init_state) {", "if (0) {"),
    "head_zero_decay": ("const double a_h = (double)A[h];", "const double a_h = (double)A[0];"),
    "dt_of_wrong_head": ("dt[(b * L + t) * H + h]", "dt[(b * L + t) * H + 0]"),
    "chunk_state_after_token": (
        "if (chunk_states && t % chunk_size == 0) {",
        "if (chunk_states && t % chunk_size == 1 % chunk_size) {"),
}


def _build_mutant(tmp_path, name, old, new):
    text = open(SRC).read()
    assert text.count(old) >= 1, "mutation anchor not found: %s" % name
    mutated = text.replace(old, new)
    c_path = tmp_path / ("%s.c" % name)
    so_path = tmp_path / ("%s.so" % name)
    c_path.write_text(mutated)
    subprocess.run(["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-std=c99", str(c_path), "-o",
                    str(so_path), "-lm"], check=True)
    return oracle.load_library(str(so_path))


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_pins_reject_mutant(tmp_path, name):
    old, new = MUTANTS[name]
    lib = _build_mutant(tmp_path, name, old, new)
    failed = []
    for pin in ALL_PINS:
        try:
            pin(lib=lib)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no pin rejects the mutant %s" % name


def test_unmodified_copy_passes_all_pins(tmp_path):
    lib = _build_mutant(tmp_path, "identity", "int ssd_oracle_fwd(", "int ssd_oracle_fwd(")
    for pin in ALL_PINS:
        pin(lib=lib)


DT_SRC = os.path.join(os.path.dirname(oracle.__file__), "dt.py")

DT_MUTANTS = {
    "softplus_drops_max": ("return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))",
                           "return np.log1p(np.exp(-np.abs(v)))"),
    "softplus_exp_sign": ("np.log1p(np.exp(-np.abs(v)))", "np.log1p(np.exp(np.abs(v)))"),
    "softplus_log_not_log1p": ("np.log1p(np.exp(-np.abs(v)))", "np.log(np.exp(-np.abs(v)))"),
    "bias_dropped": ("v = v + _f64(dt_bias)[None, None, :]", "v = v"),
    "bias_subtracted": ("v = v + _f64(dt_bias)[None, None, :]", "v = v - _f64(dt_bias)[None, None, :]"),
    "clamp_swapped": ("np.minimum(np.maximum(v, dt_min), dt_max)",
                      "np.maximum(np.minimum(v, dt_min), dt_max)"),
    "softplus_flag_ignored": ("if use_softplus:", "if True:"),
}


def _dt_mutant(old, new):
    text = open(DT_SRC).read()
    assert text.count(old) == 1, "mutation anchor not found: %r" % old
    ns = {"__name__": "dt_mutant"}
    exec(compile(text.replace(old, new), "dt_mutant.py", "exec"), ns)
    return ns["softplus"], ns["dt_transform"]


@pytest.mark.parametrize("name", sorted(DT_MUTANTS))
def test_dt_pins_reject_mutant(name):
    sp, xf = _dt_mutant(*DT_MUTANTS[name])
    failed = []
    for pin in DT_PINS:
        try:
            pin(sp=sp, xf=xf)
        except (AssertionError, FloatingPointError):
            failed.append(pin.__name__)
    assert failed, "no step-size pin rejects the mutant %s" % name


def test_dt_unmodified_copy_passes():
    sp, xf = _dt_mutant("def softplus(v):", "def softplus(v):")
    for pin in DT_PINS:
        pin(sp=sp, xf=xf)
