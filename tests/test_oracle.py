"""Pins for the CPU oracle: checks against things other than the oracle itself.

Each test compares the fp64 token recurrence (oracle.recurrence) with an
independent statement of what the scan must produce: a hand-worked example,
closed forms, the materialised SSD matrix, the chunked log-space form at many
chunk sizes, the zero-decay (causal linear attention) limit, the memoryless
limit, continuation, group expansion and linearity.  test_oracle_mutants.py
checks that altered copies of the oracle fail at least one of these pins.
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle
import ssd_synth

HERE = os.path.dirname(os.path.abspath(__file__))


def small_problem(**kw):
    base = dict(batch=2, seqlen=37, nheads=4, headdim=8, dstate=5, ngroups=2, chunk_size=16,
                io_dtype="fp32", init_std=0.3)
    base.update(kw)
    return ssd_synth.Problem(**base)


def inputs_of(prob, seed=0):
    return ssd_synth.make_inputs(prob, seed)


def run_rec(inp, lib=None, **kw):
    return oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                             inp["init_state"], lib=lib, **kw)


def rel(a, b):
    return np.linalg.norm(np.asarray(a) - np.asarray(b)) / max(np.linalg.norm(np.asarray(b)), 1e-300)


# ---------------------------------------------------------------- pin checks
# Each check takes a recurrence callable so the mutant test can reuse it.

def check_hand_worked(lib=None):
    fx = json.load(open(os.path.join(HERE, "golden", "hand_worked_3tok.json")))
    inp = {k: torch.tensor(v, dtype=torch.float32) for k, v in fx["inputs"].items()}
    y, fin, _ = run_rec(inp, lib=lib)
    np.testing.assert_allclose(y, np.array(fx["expected"]["y"]), rtol=1e-7, atol=1e-7)
    np.testing.assert_allclose(fin, np.array(fx["expected"]["final_state"]), rtol=1e-7, atol=1e-7)


def check_dense_matrix(lib=None):
    inp = inputs_of(small_problem(), seed=1)
    y, fin, _ = run_rec(inp, lib=lib)
    y2, fin2 = oracle.dense_matrix(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                   inp["init_state"])
    assert rel(y, y2) < 1e-12 and rel(fin, fin2) < 1e-12, (rel(y, y2), rel(fin, fin2))


def check_chunk_invariance(lib=None):
    prob = small_problem(seqlen=100, nheads=2, ngroups=1, headdim=6, dstate=7, batch=1)
    inp = inputs_of(prob, seed=2)
    y, fin, _ = run_rec(inp, lib=lib)
    for Q in (1, 2, 5, 16, 64, 100, 128):
        yq, fq, _ = oracle.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                   inp["init_state"], chunk_size=Q)
        assert rel(y, yq) < 1e-12 and rel(fin, fq) < 1e-12, (Q, rel(y, yq), rel(fin, fq))


def check_chunk_states(lib=None):
    prob = small_problem(seqlen=70, nheads=2, ngroups=1, headdim=4, dstate=6, batch=1)
    inp = inputs_of(prob, seed=3)
    for Q in (16, 32):
        _, _, cs = run_rec(inp, lib=lib, chunk_size=Q, want_chunk_states=True)
        _, _, cs2 = oracle.chunked(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                   inp["init_state"], chunk_size=Q, want_chunk_states=True)
        assert rel(cs, cs2) < 1e-12, (Q, rel(cs, cs2))
        # the first chunk starts from the initial state itself
        np.testing.assert_array_equal(cs[:, :, 0], inp["init_state"].double().numpy())


def check_linear_attention_limit(lib=None):
    inp = inputs_of(small_problem(), seed=4)
    inp["A"] = torch.zeros_like(inp["A"])
    y, fin, _ = run_rec(inp, lib=lib)
    y2, fin2 = oracle.linear_attention(inp["x"], inp["dt"], inp["B"], inp["C"], inp["D"],
                                       inp["init_state"])
    assert rel(y, y2) < 1e-12 and rel(fin, fin2) < 1e-12, (rel(y, y2), rel(fin, fin2))


def check_memoryless_limit(lib=None):
    inp = inputs_of(small_problem(), seed=5)
    inp["A"] = torch.full_like(inp["A"], -1e30)
    y, fin, _ = run_rec(inp, lib=lib)
    x, dt = inp["x"].double().numpy(), inp["dt"].double().numpy()
    Bm, Cm, D = inp["B"].double().numpy(), inp["C"].double().numpy(), inp["D"].double().numpy()
    H, G = x.shape[2], Bm.shape[2]
    g = np.arange(H) // (H // G)
    cb = np.einsum("blgn,blgn->blg", Cm, Bm)[:, :, g]           # (c_t . b_t) per head
    y_ref = (dt * cb)[..., None] * x + D[None, None, :, None] * x
    fin_ref = dt[:, -1, :, None, None] * x[:, -1, :, :, None] * Bm[:, -1][:, g][:, :, None, :]
    assert rel(y, y_ref) < 1e-13 and rel(fin, fin_ref) < 1e-13


def check_single_token(lib=None):
    inp = inputs_of(small_problem(seqlen=1), seed=6)
    y, fin, _ = run_rec(inp, lib=lib)
    x, dt, A = (inp[k].double().numpy() for k in ("x", "dt", "A"))
    Bm, Cm, D, s0 = (inp[k].double().numpy() for k in ("B", "C", "D", "init_state"))
    H, G = x.shape[2], Bm.shape[2]
    g = np.arange(H) // (H // G)
    alpha = np.exp(dt[:, 0, :] * A[None, :])                    # [b, h]
    s = alpha[:, :, None, None] * s0 + dt[:, 0, :, None, None] * x[:, 0, :, :, None] \
        * Bm[:, 0][:, g][:, :, None, :]
    y_ref = np.einsum("bhpn,bhn->bhp", s, Cm[:, 0][:, g]) + D[None, :, None] * x[:, 0]
    assert rel(y[:, 0], y_ref) < 1e-14 and rel(fin, s) < 1e-14


def check_continuation(lib=None):
    inp = inputs_of(small_problem(seqlen=60), seed=7)
    y, fin, _ = run_rec(inp, lib=lib)
    L1 = 23
    head = {k: (v[:, :L1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    _, fin1, _ = run_rec(head, lib=lib)
    tail = {k: (v[:, L1:] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
    tail["init_state"] = torch.from_numpy(fin1.astype(np.float32))
    y2, fin2, _ = run_rec(tail, lib=lib)
    # the hand-off state is rounded to fp32 by the interface: compare loosely
    assert rel(y[:, L1:], y2) < 1e-6 and rel(fin, fin2) < 1e-6


def check_groups(lib=None):
    prob = small_problem(nheads=6, ngroups=3)
    inp = inputs_of(prob, seed=8)
    y, fin, _ = run_rec(inp, lib=lib)
    rep = prob.nheads // prob.ngroups
    wide = dict(inp)
    wide["B"] = inp["B"].repeat_interleave(rep, dim=2).contiguous()
    wide["C"] = inp["C"].repeat_interleave(rep, dim=2).contiguous()
    y2, fin2, _ = run_rec(wide, lib=lib)
    np.testing.assert_array_equal(y, y2)
    np.testing.assert_array_equal(fin, fin2)


def check_linearity(lib=None):
    inp = inputs_of(small_problem(), seed=9)
    y, fin, _ = run_rec(inp, lib=lib)
    for lam in (2.0, -0.5):
        scaled = dict(inp)
        scaled["x"] = inp["x"] * lam
        scaled["init_state"] = inp["init_state"] * lam
        y2, fin2, _ = run_rec(scaled, lib=lib)
        assert rel(y2, lam * y) < 1e-14 and rel(fin2, lam * fin) < 1e-14


def check_no_skip(lib=None):
    """D = None means no skip term: the difference is exactly D x."""
    inp = inputs_of(small_problem(), seed=10)
    y, _, _ = run_rec(inp, lib=lib)
    no_d = dict(inp)
    no_d["D"] = None
    y2, _, _ = run_rec(no_d, lib=lib)
    x = inp["x"].double().numpy()
    diff_ref = inp["D"].double().numpy()[None, None, :, None] * x
    assert rel(y - y2, diff_ref) < 1e-12


ALL_PINS = [check_hand_worked, check_dense_matrix, check_chunk_invariance, check_chunk_states,
            check_linear_attention_limit, check_memoryless_limit, check_single_token,
            check_continuation, check_groups, check_linearity, check_no_skip]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda f: f.__name__)
def test_pin(pin):
    pin()


# ---------------------------------------------------------- chunk cumsum pins

def test_cumsum_constant_dt_closed_form():
    # constant dt: G_i = (i + 1) dt A log2(e), restarting at every chunk
    L, H, Q = 100, 3, 32
    dt = torch.full((2, L, H), 0.0625)
    A = torch.tensor([-1.0, -2.5, -0.125])
    G = oracle.chunk_cumsum(dt, A, Q)
    i = np.arange(L) % Q
    ref = (i + 1)[None, None, :] * 0.0625 * A.double().numpy()[None, :, None] / math.log(2.0)
    np.testing.assert_allclose(G, np.broadcast_to(ref, G.shape), rtol=1e-14)


def test_cumsum_zero_decay():
    dt = torch.rand(1, 50, 4) + 0.1
    G = oracle.chunk_cumsum(dt, torch.zeros(4), 16)
    assert np.all(G == 0.0)


def test_cumsum_matches_chunked_stage_and_resets():
    prob = small_problem(seqlen=90)
    inp = inputs_of(prob, seed=11)
    Q = 32
    G = oracle.chunk_cumsum(inp["dt"], inp["A"], Q)
    dt, A = inp["dt"].double().numpy(), inp["A"].double().numpy()
    # at each chunk start the running sum holds exactly one term
    for c in range(0, 90, Q):
        np.testing.assert_allclose(G[:, :, c], dt[:, c, :] * A[None, :] / math.log(2.0), rtol=1e-15)
    # consecutive differences inside a chunk are the per-token terms
    d = np.diff(G, axis=2)
    inside = (np.arange(1, 90) % Q) != 0
    np.testing.assert_allclose(d[:, :, inside], (dt[:, 1:, :] * A / math.log(2.0)).transpose(0, 2, 1)[:, :, inside],
                               rtol=1e-9, atol=1e-14)
    # decays are negative, so G is non-increasing within a chunk
    assert np.all(d[:, :, inside] <= 0)


def test_recurrence_heads_matches_full():
    prob = small_problem(nheads=6, ngroups=2)
    inp = inputs_of(prob, seed=12)
    y, fin, _ = run_rec(inp)
    got = oracle.recurrence_heads(inp, [(0, 0), (1, 5), (1, 2)])
    for (b, h), (yh, fh) in got.items():
        np.testing.assert_array_equal(yh, y[b, :, h])
        np.testing.assert_array_equal(fh, fin[b, h])


@pytest.mark.parametrize("heads_per_range", [1, 2, 3, 4, 6, 100])
def test_recurrence_head_ranges_cover_every_head(heads_per_range):
    # ranges of whole groups: every head exactly once, equal to the full call
    prob = small_problem(nheads=6, ngroups=2)
    inp = inputs_of(prob, seed=13)
    y, fin, _ = run_rec(inp)
    seen = np.zeros(6, dtype=int)
    for h0, h1, yr, fr in oracle.recurrence_head_ranges(inp, heads_per_range):
        assert h0 % 3 == 0 and h1 % 3 == 0      # 3 heads per group
        seen[h0:h1] += 1
        np.testing.assert_array_equal(yr, y[:, :, h0:h1])
        np.testing.assert_array_equal(fr, fin[:, h0:h1])
    assert np.all(seen == 1)


def test_inputs_are_seeded_and_shaped():
    prob = ssd_synth.CONFIGS["tiny_fp32"]
    a, b = ssd_synth.make_inputs(prob, 0), ssd_synth.make_inputs(prob, 0)
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k])
    assert a["x"].shape == (1, 256, 2, 16) and a["B"].shape == (1, 256, 1, 16)
    assert torch.all(a["dt"] > 0) and torch.all(a["A"] < 0)
    c2 = ssd_synth.CONFIGS["mamba2_2p7b"]
    assert c2.init_std == 0.1 and c2.nchunks == 32


# ------------------------------------------------- step-size preparation pins
# Each check takes the (softplus, dt_transform) pair so the mutant test can
# run it against altered copies of oracle/dt.py.

def check_softplus_closed_forms(sp=None, xf=None):
    sp = sp or oracle.softplus
    assert abs(sp(0.0) - math.log(2.0)) < 1e-16
    v = np.linspace(-30.0, 30.0, 601)
    # softplus(v) - softplus(-v) = v  (log(1+e^v) - log(1+e^-v) = log e^v)
    np.testing.assert_allclose(sp(v) - sp(-v), v, rtol=0, atol=1e-13)
    # inverse of the generator's inv_softplus: softplus(log(e^y - 1)) = y
    y = np.exp(np.linspace(math.log(1e-4), math.log(20.0), 200))
    np.testing.assert_allclose(sp(np.log(np.expm1(y))), y, rtol=1e-13)
    # asymptotes: ~v for large v (difference e^-v), ~e^v for very negative v
    assert sp(50.0) == 50.0 and abs(sp(800.0) - 800.0) == 0.0
    np.testing.assert_allclose(sp(-40.0), math.exp(-40.0), rtol=1e-15)
    assert np.all(sp(v) > 0) and np.all(np.diff(sp(v)) > 0)


def check_dt_transform_bias_and_clamp(sp=None, xf=None):
    xf = xf or oracle.dt_transform
    raw = torch.tensor([[[-3.0, 0.0], [2.0, 40.0]]])           # [1, 2, 2]
    bias = torch.tensor([1.0, -0.5])
    got = xf(raw, bias, use_softplus=True)
    v = raw.double().numpy() + bias.double().numpy()
    np.testing.assert_allclose(got, np.log1p(np.exp(np.minimum(v, 30))) + np.maximum(v - 30, 0),
                               rtol=1e-14)
    # without softplus the bias is just added; the clamp bounds from both sides
    np.testing.assert_array_equal(xf(raw, bias, use_softplus=False, dt_min=-np.inf), v)
    # the default lower limit 0 removes negative values
    assert xf(raw, bias, use_softplus=False).min() == 0.0
    cl = xf(raw, bias, use_softplus=False, dt_min=0.25, dt_max=2.0)
    np.testing.assert_array_equal(cl, np.clip(v, 0.25, 2.0))
    assert cl.min() == 0.25 and cl.max() == 2.0
    # values inside the limits are fixed points of the clamp
    np.testing.assert_array_equal(xf(raw, bias, dt_min=1e-9, dt_max=1e9), got)


def check_dt_transform_reproduces_generated(sp=None, xf=None):
    # the generator draws dt = softplus(dt_raw + dt_bias) in fp32 (a separate
    # implementation); the fp64 preparation agrees to fp32 rounding
    xf = xf or oracle.dt_transform
    inp = inputs_of(small_problem(seqlen=200, nheads=6, ngroups=2), seed=21)
    got = xf(inp["dt_raw"], inp["dt_bias"], use_softplus=True)
    np.testing.assert_allclose(got, inp["dt"].double().numpy(), rtol=2e-6)


DT_PINS = [check_softplus_closed_forms, check_dt_transform_bias_and_clamp,
           check_dt_transform_reproduces_generated]


@pytest.mark.parametrize("pin", DT_PINS, ids=lambda f: f.__name__)
def test_dt_pin(pin):
    pin()


def test_token_at_a_time_equals_whole_sequence():
    # the decode mode's reference: L calls of one token each, the state handed
    # from call to call, against one call over the whole sequence
    inp = inputs_of(small_problem(seqlen=12), seed=22)
    y, fin, _ = run_rec(inp)
    state = inp["init_state"]
    ys = []
    for t in range(12):
        one = {k: (v[:, t:t + 1] if k in ("x", "dt", "B", "C") else v) for k, v in inp.items()}
        one["init_state"] = state
        yt, ft, _ = run_rec(one)
        ys.append(yt)
        state = torch.from_numpy(ft.astype(np.float32))
    assert rel(np.concatenate(ys, 1), y) < 1e-6 and rel(ft, fin) < 1e-6
