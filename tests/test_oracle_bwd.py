"""Pins for the backward oracle (oracle.recurrence_bwd, oracle.dt_transform_bwd).

The gradients are checked against things other than the backward code: central
finite differences of the (separately pinned) C forward oracle, element by
element over every input of small problems, and the first-degree homogeneity
of the loss (Euler's theorem) in (x, init_state), in B, in C and in D.
test_oracle_mutants.py checks that altered copies of the backward oracle fail
at least one of these pins.
"""
import numpy as np
import pytest

import oracle
import ssd_synth


def _problem(**kw):
    base = dict(batch=1, seqlen=7, nheads=4, headdim=2, dstate=3, ngroups=2, chunk_size=16,
                io_dtype="fp32", init_std=0.3)
    base.update(kw)
    return ssd_synth.Problem(**base)


def _arrays(p, seed):
    inp = ssd_synth.make_inputs(p, seed)
    arr = {k: oracle.as_f32(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state")}
    rng = np.random.default_rng(seed + 1000)
    arr["dy"] = rng.standard_normal(arr["x"].shape).astype(np.float32)
    arr["dfinal"] = rng.standard_normal(arr["init_state"].shape).astype(np.float32)
    return arr


def _loss(a):
    """<dy, y> + <dfinal, final_state> through the C forward oracle."""
    y, fin, _ = oracle.recurrence(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init_state"])
    return float(np.sum(a["dy"].astype(np.float64) * y) +
                 np.sum(a["dfinal"].astype(np.float64) * fin))


def _grads(a, rb, seg=64):
    return rb(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init_state"], a["dy"],
              a["dfinal"], seg=seg)


NAMES = {"x": "dx", "dt": "ddt", "A": "dA", "B": "dB", "C": "dC", "D": "dD", "init_state": "dinit"}


def check_finite_differences(rb=None, tb=None):
    """Every gradient element against a central difference of the forward oracle."""
    rb = rb or oracle.recurrence_bwd
    a = _arrays(_problem(), seed=5)
    g = _grads(a, rb, seg=3)        # several checkpoint segments
    for name, gname in NAMES.items():
        base = a[name]
        flat = base.reshape(-1)
        for i in range(flat.size):
            v = flat[i]
            eps = 1e-4 * max(1.0, abs(float(v)))
            hi = np.float32(v + eps)
            lo = np.float32(v - eps)
            flat[i] = hi
            f_hi = _loss(a)
            flat[i] = lo
            f_lo = _loss(a)
            flat[i] = v
            fd = (f_hi - f_lo) / (float(hi) - float(lo))
            an = float(g[gname].reshape(-1)[i])
            assert abs(fd - an) <= 2e-5 * max(1.0, abs(fd)), (name, i, fd, an)


def check_homogeneity(rb=None, tb=None):
    """Euler's theorem: the loss is of degree one in (x, init), in B, in C, in D."""
    rb = rb or oracle.recurrence_bwd
    p = _problem(batch=2, seqlen=37, nheads=4, headdim=8, dstate=5, ngroups=2)
    a = _arrays(p, seed=6)
    g = _grads(a, rb)
    f = lambda k: np.asarray(a[k], dtype=np.float64)
    Ld = _loss(a)
    y, _, _ = oracle.recurrence(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init_state"])
    dy = f("dy")
    dx_skip = dy * f("D")[None, None, :, None] * f("x")          # dy . D x, elementwise
    # (x, init) jointly
    lhs = np.sum(f("x") * g["dx"]) + np.sum(f("init_state") * g["dinit"])
    assert abs(lhs - Ld) <= 1e-9 * max(1.0, abs(Ld)), (lhs, Ld)
    # B: the part of the loss that B drives (all but the initial state's part and the skip)
    a0 = dict(a, B=np.zeros_like(a["B"]))
    assert abs(np.sum(f("B") * g["dB"]) - (Ld - _loss(a0))) <= 1e-9 * max(1.0, abs(Ld))
    # C: y without the skip term
    want = np.sum(dy * y) - np.sum(dx_skip)
    assert abs(np.sum(f("C") * g["dC"]) - want) <= 1e-9 * max(1.0, abs(want))
    # D, per head
    np.testing.assert_allclose(f("D") * g["dD"], dx_skip.sum(axis=(0, 1, 3)), rtol=1e-10, atol=1e-12)


def check_checkpoint_invariance(rb=None, tb=None):
    """The segment length of the recomputation changes no value."""
    rb = rb or oracle.recurrence_bwd
    a = _arrays(_problem(seqlen=11), seed=7)
    g1 = _grads(a, rb, seg=1)
    g2 = _grads(a, rb, seg=64)
    for k in g1:
        np.testing.assert_allclose(g1[k], g2[k], rtol=1e-12, atol=1e-14)


def check_dt_transform_finite_differences(rb=None, tb=None):
    """Gradients through bias, softplus and clamp against central differences."""
    tb = tb or oracle.dt_transform_bwd
    rng = np.random.default_rng(8)
    raw = rng.standard_normal((2, 9, 3)) * 2.0
    bias = rng.standard_normal(3)
    up = rng.standard_normal(raw.shape)
    for use_sp, lo, hi in ((True, 0.0, np.inf), (True, 0.3, 1.5), (False, -1.0, 1.0)):
        # keep every point away from the clamp's ends (the derivative jumps there)
        v = raw + bias[None, None, :]
        w = oracle.softplus(v) if use_sp else v
        ok = (np.abs(w - lo) > 1e-3) & (np.abs(w - hi) > 1e-3)
        r = np.where(ok, raw, raw + 0.1)
        d_raw, d_bias = tb(r, up, bias, use_sp, lo, hi)
        eps = 1e-6
        f = lambda rr, bb: np.sum(up * oracle.dt_transform(rr, bb, use_sp, lo, hi))
        fd_raw = np.zeros_like(r)
        for i in np.ndindex(r.shape):
            e = np.zeros_like(r)
            e[i] = eps
            fd_raw[i] = (f(r + e, bias) - f(r - e, bias)) / (2 * eps)
        fd_bias = np.array([(f(r, bias + eps * (np.arange(3) == h)) -
                             f(r, bias - eps * (np.arange(3) == h))) / (2 * eps) for h in range(3)])
        np.testing.assert_allclose(d_raw, fd_raw, rtol=1e-6, atol=1e-8)
        np.testing.assert_allclose(d_bias, fd_bias, rtol=1e-6, atol=1e-8)


BWD_PINS = [check_finite_differences, check_homogeneity, check_checkpoint_invariance,
            check_dt_transform_finite_differences]


@pytest.mark.parametrize("pin", BWD_PINS, ids=lambda f: f.__name__)
def test_bwd_pin(pin):
    pin()


def test_heads_subset_matches_full():
    a = _arrays(_problem(batch=2, seqlen=20, nheads=4, ngroups=2), seed=9)
    full = _grads(a, oracle.recurrence_bwd)
    part = oracle.recurrence_bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"],
                                 a["init_state"], a["dy"], a["dfinal"], heads=[(1, 2), (0, 3)])
    for (b, h) in ((1, 2), (0, 3)):
        np.testing.assert_array_equal(part["dx"][b, :, h], full["dx"][b, :, h])
        np.testing.assert_array_equal(part["ddt"][b, :, h], full["ddt"][b, :, h])
        np.testing.assert_array_equal(part["dinit"][b, h], full["dinit"][b, h])


def test_no_final_gradient_and_no_init():
    # dfinal = None and init = None behave as zeros
    a = _arrays(_problem(), seed=10)
    g0 = oracle.recurrence_bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], None, a["dy"], None)
    g1 = oracle.recurrence_bwd(a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"],
                               np.zeros_like(a["init_state"]), a["dy"],
                               np.zeros_like(a["dfinal"]))
    for k in g0:
        np.testing.assert_array_equal(g0[k], g1[k])
