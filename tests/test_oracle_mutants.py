"""The oracle's pins must reject plausible mistakes.

Each case copies oracle/ssd_oracle.c to a temporary directory, plants one
mistake with a textual substitution (the committed source is never touched),
compiles the copy with gcc and runs every pin of test_oracle.py against it.
At least one pin must fail for every mutant.  The step-size preparation
(oracle/dt.py) is treated the same way: a mutated copy of its text is
executed in a fresh namespace and run against the step-size pins, and the
backward oracle (oracle/bwd.py) the same way against the backward pins.
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


BWD_SRC = os.path.join(os.path.dirname(oracle.__file__), "bwd.py")

BWD_MUTANTS = {
    "dC_from_previous_state": ("dC[t] = s_t.T @ dy[t]", "dC[t] = s_prev.T @ dy[t]"),
    "skip_gradient_dropped": ("dx[t] = Dh * dy[t] + dt[t] * lam_b", "dx[t] = dt[t] * lam_b"),
    "dx_without_dt": ("dx[t] = Dh * dy[t] + dt[t] * lam_b", "dx[t] = Dh * dy[t] + lam_b"),
    "dB_without_dt": ("dB[t] = dt[t] * (lam.T @ x[t])", "dB[t] = (lam.T @ x[t])"),
    "dl_from_new_state": ("dl = alpha * np.sum(lam * s_prev)", "dl = alpha * np.sum(lam * s_t)"),
    "dl_without_decay": ("dl = alpha * np.sum(lam * s_prev)", "dl = np.sum(lam * s_prev)"),
    "ddt_direct_term_dropped": ("ddt[t] = x[t] @ lam_b + a_coef * dl", "ddt[t] = a_coef * dl"),
    "ddt_decay_term_dropped": ("ddt[t] = x[t] @ lam_b + a_coef * dl", "ddt[t] = x[t] @ lam_b"),
    "dA_without_dt": ("dA += dt[t] * dl", "dA += dl"),
    "adjoint_not_decayed": ("lam = alpha * lam", "lam = lam"),
    "output_adjoint_uses_B": ("lam = lam + np.outer(dy[t], Cg[t])",
                              "lam = lam + np.outer(dy[t], Bg[t])"),
    "group_sum_overwritten": ('out["dB"][b, :, g] += dB', 'out["dB"][b, :, g] = dB'),
    "final_gradient_ignored": ("lam = dS.copy()", "lam = np.zeros_like(dS)"),
    "recompute_from_first_mark": ("s = marks[start].copy()", "s = marks[0].copy()"),
    "logistic_wrong": ("g = g * np.exp(v - w)", "g = g * np.exp(-w)"),
    "clamp_gradient_kept": ("g = g * ((w >= dt_min) & (w <= dt_max))", "g = g"),
}


def _bwd_mutant(old, new):
    text = open(BWD_SRC).read()
    assert text.count(old) == 1, "mutation anchor not found: %r" % old
    text = text.replace(old, new).replace("from .dt import softplus", "from oracle.dt import softplus")
    ns = {"__name__": "bwd_mutant"}
    exec(compile(text, "bwd_mutant.py", "exec"), ns)
    return ns["recurrence_bwd"], ns["dt_transform_bwd"]


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_bwd_pins_reject_mutant(name):
    from test_oracle_bwd import BWD_PINS
    rb, tb = _bwd_mutant(*BWD_MUTANTS[name])
    failed = []
    for pin in BWD_PINS:
        try:
            pin(rb=rb, tb=tb)
        except AssertionError:
            failed.append(pin.__name__)
    assert failed, "no backward pin rejects the mutant %s" % name


def test_bwd_unmodified_copy_passes():
    from test_oracle_bwd import BWD_PINS
    rb, tb = _bwd_mutant("def head_bwd(", "def head_bwd(")
    for pin in BWD_PINS:
        pin(rb=rb, tb=tb)
