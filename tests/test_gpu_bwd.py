"""GPU parity of the backward pass (ssd_bwd) against the fp64 backward oracle.

Every gradient (dx, ddt, dA, dB, dC, dD, dinit and the bias gradient) is
compared element by element with oracle.recurrence_bwd on the same seeded
inputs and upstream gradients, at sizes that span several chunks and token
blocks with a ragged tail, for both io dtypes, dstate up to 256, chunk sizes
16 to 256, grouped and ungrouped B/C, with and without D, init_state and
dfinal, and with the step-size preparation.  At the 2.7B layer shape the
per-head gradients of two (batch, head) pairs are checked against the oracle
run for those heads alone, and at the large-state layer shape one whole group
of one batch row (its dB and dC included).

Tolerances (relative L2 over the tensor; max-abs relative to max|ref|).
Every gradient is computed in fp32 from the (exact) io values, with fp32
chunk-boundary states; only dx, dB and dC are then stored in the io dtype.
  dx, dB, dC, bf16 io: 5e-3 / 2e-2 -- the bf16 store alone is up to 2^-9
      relative per element (about 1.7e-3 rel-L2 measured), as for y.
  dx, dB, dC, fp32 io: 1e-5 / 1e-4 -- fp32 sums over a chunk of tokens and a
      state row, and the hardware exp2 (about 1 ulp).
  ddt, dA, dD, dinit, bias gradient (fp32 outputs, either io dtype): 1e-4 /
      1e-3 -- as above, plus the running sum of P - dt Qr over the whole
      sequence: accumulated in fp64, but fed by fp32 terms that largely
      cancel (up to 2e-5 measured).
"""
import numpy as np
import pytest
import torch

import oracle
import ssd_synth
from bwd_layout import balanced, bwd_layout, part_heads, parts
from parity_util import errors

pytestmark = pytest.mark.gpu

lib = pytest.importorskip("state_space_sequence_03_amd")

TOL = {"bf16": (5e-3, 2e-2), "fp32": (1e-5, 1e-4), "f32out": (1e-4, 1e-3)}
IO_OUTPUTS = ("dx", "dB", "dC")


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu-case] %s" % request.node.name, flush=True)
    yield
    torch.cuda.synchronize()


def check(got, ref, io, what):
    rl2, mabs = errors(got, ref)
    tl2, tabs = TOL[io]
    print("  %-8s rel-L2 %.2e  max-abs %.2e" % (what, rl2, mabs), flush=True)
    assert rl2 <= tl2 and mabs <= tabs, "%s: rel-L2 %.3e (limit %.1e), max-abs %.3e (limit %.1e)" % (
        what, rl2, tl2, mabs, tabs)


CASES = {
    # name: (Problem kwargs, use D, use dfinal, dt transform)
    "bf16_q64_g2_ragged": (dict(batch=2, seqlen=300, nheads=4, headdim=32, dstate=64, ngroups=2,
                                chunk_size=64, io_dtype="bf16", init_std=0.1), True, True, None),
    "fp32_q128_g1": (dict(batch=1, seqlen=333, nheads=4, headdim=64, dstate=128, ngroups=1,
                          chunk_size=128, io_dtype="fp32", init_std=0.1), True, True, None),
    "bf16_q256_n256": (dict(batch=1, seqlen=520, nheads=2, headdim=64, dstate=256, ngroups=1,
                            chunk_size=256, io_dtype="bf16", init_std=0.1), True, True, None),
    # chunk 16 runs as 32 (the gradients do not depend on the chunk size)
    "fp32_q16": (dict(batch=1, seqlen=90, nheads=2, headdim=32, dstate=32, ngroups=1,
                      chunk_size=16, io_dtype="fp32", init_std=0.1), True, True, None),
    "fp32_q32_no_D_init_dfinal": (dict(batch=2, seqlen=70, nheads=2, headdim=16, dstate=16,
                                       ngroups=2, chunk_size=32, io_dtype="fp32"), False, False,
                                  None),
    "fp32_q64_raw_dt": (dict(batch=2, seqlen=150, nheads=4, headdim=32, dstate=32, ngroups=1,
                             chunk_size=64, io_dtype="fp32", init_std=0.1), True, True,
                        (True, (0.0, float("inf")))),
    "bf16_q128_raw_dt_clamped": (dict(batch=1, seqlen=260, nheads=4, headdim=64, dstate=128,
                                      ngroups=2, chunk_size=128, io_dtype="bf16", init_std=0.1),
                                 True, True, (True, (0.01, 0.08))),
    # headdim / dstate not multiples of 32: zero-padded MFMA K-steps and a
    # half-empty last state pass
    "bf16_p48_n48": (dict(batch=1, seqlen=100, nheads=2, headdim=48, dstate=48, ngroups=1,
                          chunk_size=64, io_dtype="bf16", init_std=0.1), True, True, None),
    "fp32_p80_n80_g2": (dict(batch=2, seqlen=90, nheads=4, headdim=80, dstate=80, ngroups=2,
                             chunk_size=32, io_dtype="fp32", init_std=0.1), True, True, None),
    # fewer tokens than one 32-token block
    "bf16_seq5": (dict(batch=3, seqlen=5, nheads=2, headdim=16, dstate=16, ngroups=1,
                       chunk_size=64, io_dtype="bf16", init_std=0.1), True, True, None),
    # enough workgroups (2 x 64 chunks x 8 parts) for parts of four heads:
    # each workgroup sums four heads' dB and dC before writing them
    "bf16_q32_parts4_ragged": (dict(batch=2, seqlen=2030, nheads=32, headdim=16, dstate=32,
                                    ngroups=2, chunk_size=32, io_dtype="bf16", init_std=0.1),
                               True, True, None),
    "fp32_q32_parts4_raw_dt": (dict(batch=2, seqlen=2030, nheads=32, headdim=16, dstate=32,
                                    ngroups=2, chunk_size=32, io_dtype="fp32", init_std=0.1),
                               True, True, (True, (0.0, float("inf")))),
}


def run_case(p, inp, grads, use_D, use_dfinal, xform):
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    dy = grads["dy"].cuda()
    dfinal = grads["dfinal"].cuda() if use_dfinal else None
    D = d["D"] if use_D else None
    kw = {}
    dt_arg = d["dt"]
    if xform is not None:
        sp, lim = xform
        kw = dict(dt_bias=d["dt_bias"], dt_softplus=sp, dt_limit=lim)
        dt_arg = d["dt_raw"]
    out = lib.ssd_bwd(d["x"], dt_arg, d["A"], d["B"], d["C"], D, p.chunk_size, d["init_state"],
                      dy, dfinal, want_ddt_bias=True, **kw)
    torch.cuda.synchronize()
    return out


def oracle_case(p, inp, grads, use_D, use_dfinal, xform):
    dt = inp["dt"]
    if xform is not None:
        sp, (lo, hi) = xform
        dt = oracle.dt_transform(inp["dt_raw"], inp["dt_bias"], sp, lo, hi)
    ref = oracle.recurrence_bwd(inp["x"], dt, inp["A"], inp["B"], inp["C"],
                                inp["D"] if use_D else None, inp["init_state"], grads["dy"],
                                grads["dfinal"] if use_dfinal else None)
    if xform is not None:
        sp, (lo, hi) = xform
        ref["ddt"], ref["ddt_bias"] = oracle.dt_transform_bwd(inp["dt_raw"], ref["ddt"],
                                                              inp["dt_bias"], sp, lo, hi)
    else:
        ref["ddt_bias"] = ref["ddt"].sum(axis=(0, 1))
    return ref


@pytest.mark.parametrize("name", sorted(CASES))
def test_bwd_matches_oracle(name):
    kw, use_D, use_dfinal, xform = CASES[name]
    p = ssd_synth.Problem(**kw)
    inp = ssd_synth.make_inputs(p, seed=51)
    grads = ssd_synth.make_grads(p, seed=51)
    got = run_case(p, inp, grads, use_D, use_dfinal, xform)
    ref = oracle_case(p, inp, grads, use_D, use_dfinal, xform)
    for k in ("dx", "ddt", "dA", "dB", "dC", "dD", "dinit", "ddt_bias"):
        check(got[k], ref[k], p.io_dtype if k in IO_OUTPUTS else "f32out", k)


def test_bwd_repeatable_and_workspace_reuse():
    # same call twice on one caller workspace: bitwise the same results
    kw, use_D, use_dfinal, xform = CASES["bf16_q64_g2_ragged"]
    p = ssd_synth.Problem(**kw)
    inp = {k: (None if v is None else v.cuda()) for k, v in ssd_synth.make_inputs(p, 52).items()}
    g = ssd_synth.make_grads(p, 52)
    prob = lib.make_problem(p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups,
                            p.chunk_size, lib.SSD_BF16)
    ws = torch.empty(lib.ssd_bwd_workspace_size(prob), dtype=torch.uint8, device="cuda")
    args = (inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], p.chunk_size,
            inp["init_state"], g["dy"].cuda(), g["dfinal"].cuda())
    a = lib.ssd_bwd(*args, workspace=ws)
    ws.fill_(0x7f)
    b = lib.ssd_bwd(*args, workspace=ws)
    torch.cuda.synchronize()
    for k in a:
        if a[k] is not None:
            assert torch.equal(a[k], b[k]), k


def bwd_outputs(p, inp, grads, ws_bytes):
    prob = lib.make_problem(p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups,
                            p.chunk_size, lib.SSD_BF16 if p.io_dtype == "bf16" else lib.SSD_F32)
    if ws_bytes is None:
        ws_bytes = lib.ssd_bwd_workspace_size(prob)
    ws = torch.empty(ws_bytes, dtype=torch.uint8, device="cuda")
    ws.fill_(0x7f)
    out = lib.ssd_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"], p.chunk_size,
                      inp["init_state"], grads["dy"], grads["dfinal"], want_ddt_bias=True,
                      workspace=ws)
    torch.cuda.synchronize()
    return prob, out


@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_bwd_head_batches_bitwise_equal(io):
    # dB and dC are summed over each group's heads in ascending head order
    # whatever the batches of heads the workspace allows, so every output is
    # bitwise the same for one head per batch (the minimum workspace), two
    # heads per batch (batches that cut the groups of three heads: a group's
    # first, middle and last heads in different batches), the default, and
    # all heads in one batch
    p = ssd_synth.Problem(batch=2, seqlen=300, nheads=6, headdim=32, dstate=64, ngroups=2,
                          chunk_size=64, io_dtype=io, init_std=0.1)
    inp = {k: (None if v is None else v.cuda()) for k, v in ssd_synth.make_inputs(p, 53).items()}
    grads = {k: v.cuda() for k, v in ssd_synth.make_grads(p, 53).items()}
    prob, ref = bwd_outputs(p, inp, grads, None)
    big = bwd_layout(prob, p.nheads)
    sizes = {"min": lib.ssd_bwd_workspace_min_size(prob), "hb2": bwd_layout(prob, 2),
             "hb1": bwd_layout(prob, 1), "one_batch": big}
    assert sizes["min"] == min(bwd_layout(prob, balanced(p.nheads, c)) for c in range(1, 7))
    for name, n in sizes.items():
        _, got = bwd_outputs(p, inp, grads, n)
        for k in ref:
            if ref[k] is not None:
                assert torch.equal(got[k], ref[k]), (name, k)
    cpu = {k: (None if v is None else v.cpu()) for k, v in inp.items()}
    ref64 = oracle.recurrence_bwd(cpu["x"], cpu["dt"], cpu["A"], cpu["B"], cpu["C"], cpu["D"],
                                  cpu["init_state"], grads["dy"].cpu(), grads["dfinal"].cpu())
    for k in ("dB", "dC"):
        check(ref[k], ref64[k], io, k)


def test_bwd_part_batches_bitwise_equal():
    # parts of four heads (two groups of four parts): the part sums and their
    # ascending per-group sum are the same for one part per batch (the
    # minimum workspace), three parts per batch (batches that cut the
    # groups), and all eight parts in one batch (the default)
    p = ssd_synth.Problem(batch=2, seqlen=2030, nheads=32, headdim=16, dstate=32, ngroups=2,
                          chunk_size=32, io_dtype="bf16", init_std=0.1)
    inp = {k: (None if v is None else v.cuda()) for k, v in ssd_synth.make_inputs(p, 54).items()}
    grads = {k: v.cuda() for k, v in ssd_synth.make_grads(p, 54).items()}
    prob, ref = bwd_outputs(p, inp, grads, None)
    assert part_heads(prob) == 4 and parts(prob) == 8
    assert lib.ssd_bwd_workspace_size(prob) == bwd_layout(prob, 8)
    sizes = {"min": lib.ssd_bwd_workspace_min_size(prob), "three": bwd_layout(prob, 3)}
    assert sizes["min"] == bwd_layout(prob, 1)
    for name, n in sizes.items():
        _, got = bwd_outputs(p, inp, grads, n)
        for k in ref:
            if ref[k] is not None:
                assert torch.equal(got[k], ref[k]), (name, k)


def test_bwd_2p7b_part_batches_equal_one_batch():
    # at the 2.7B layer shape the default workspace holds the dB/dC sums of
    # all 16 parts (five heads each) at once; a workspace for four parts at a
    # time (four batches) must give bitwise the same gradients
    p = ssd_synth.CONFIGS["mamba2_2p7b"]
    inp = {k: (None if v is None else v.cuda()) for k, v in ssd_synth.make_inputs(p, 6).items()}
    grads = {k: v.cuda() for k, v in ssd_synth.make_grads(p, 6).items()}
    prob, ref = bwd_outputs(p, inp, grads, None)
    assert part_heads(prob) == 5
    assert lib.ssd_bwd_workspace_size(prob) == bwd_layout(prob, 16) < 650 * 10 ** 6
    _, got = bwd_outputs(p, inp, grads, bwd_layout(prob, 4))
    for k in ref:
        if ref[k] is not None:
            assert torch.equal(got[k], ref[k]), k
    del inp, grads, ref, got
    torch.cuda.empty_cache()


def test_bwd_2p7b_sampled_heads():
    # the 2.7B layer shape (batch 2, 8192 tokens, 80 heads, headdim 64, dstate
    # 128, one group, chunk 256): per-head gradients of head 37 in both batch
    # rows against the oracle run for those heads alone
    p = ssd_synth.CONFIGS["mamba2_2p7b"]
    inp = ssd_synth.make_inputs(p, seed=3)
    grads = ssd_synth.make_grads(p, seed=3)
    got = run_case(p, inp, grads, True, True, None)
    h = 37
    heads = [(0, h), (1, h)]
    ref = oracle.recurrence_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                inp["init_state"], grads["dy"], grads["dfinal"], heads=heads)
    for b, hh in heads:
        check(got["dx"][b, :, hh], ref["dx"][b, :, hh], "bf16", "dx[%d]" % b)
        check(got["ddt"][b, :, hh], ref["ddt"][b, :, hh], "f32out", "ddt[%d]" % b)
        check(got["dinit"][b, hh], ref["dinit"][b, hh], "f32out", "dinit[%d]" % b)
    check(got["dA"][h:h + 1], ref["dA"][h:h + 1], "f32out", "dA[h]")
    check(got["dD"][h:h + 1], ref["dD"][h:h + 1], "f32out", "dD[h]")
    for k in ("dB", "dC"):
        assert torch.isfinite(got[k].float()).all(), k


def test_bwd_2p7b_dC_dB_properties():
    # dB and dC sum over all 80 heads of the group, too many for the oracle at
    # this size; instead two properties that hold at any size.  The loss
    # <dy, y> + <dfinal, final> is of degree one in C, so <C, dC> equals
    # <dy, y - D x> (y from the fp64 forward oracle); and of degree one in
    # (x, init) jointly, so <x, dx> + <init, dinit> equals the loss itself.
    p = ssd_synth.CONFIGS["mamba2_2p7b"]
    inp = ssd_synth.make_inputs(p, seed=4)
    grads = ssd_synth.make_grads(p, seed=4)
    got = run_case(p, inp, grads, True, True, None)
    y, fin, _ = oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                  inp["init_state"])
    f64 = lambda t: t.detach().double().cpu().numpy() if isinstance(t, torch.Tensor) else t
    x, dy = f64(inp["x"]), f64(grads["dy"])
    skip = float(np.sum(dy * f64(inp["D"])[None, None, :, None] * x))
    loss = float(np.sum(dy * y) + np.sum(f64(grads["dfinal"]) * fin))

    def bound(terms):
        # dC and dx are stored in bf16: each element carries a rounding error
        # of at most 2^-8 of itself, roughly uniform and independent, so the sum
        # of the terms moves by about 2^-8 / sqrt(3) * ||terms||_2; allow six
        # of those, plus fp32 accumulation (1e-5 of the absolute sum)
        return 6 * 2.0 ** -8 / np.sqrt(3) * np.linalg.norm(terms) + 1e-5 * np.abs(terms).sum()

    tc = f64(inp["C"]) * f64(got["dC"])
    lhs_c, want_c = float(tc.sum()), float(np.sum(dy * y)) - skip
    print("  <C,dC> %.6e  want %.6e  bound %.3e" % (lhs_c, want_c, bound(tc)), flush=True)
    assert abs(lhs_c - want_c) <= bound(tc)
    tx = x * f64(got["dx"])
    lhs_x = float(tx.sum() + np.sum(f64(inp["init_state"]) * f64(got["dinit"])))
    print("  <x,dx>+<init,dinit> %.6e  loss %.6e  bound %.3e" % (lhs_x, loss, bound(tx)),
          flush=True)
    assert abs(lhs_x - loss) <= bound(tx)


def test_bwd_large_state_one_whole_group():
    # the large-state layer shape (batch 8, 4096 tokens, 64 heads in 8 groups,
    # headdim 64, dstate 256, chunk 128): the oracle for all 8 heads of group 0
    # in batch row 0 gives their per-head gradients and, summed over the
    # group, dB and dC of that (batch, group) exactly
    p = ssd_synth.CONFIGS["large_state"]
    inp = ssd_synth.make_inputs(p, seed=5)
    grads = ssd_synth.make_grads(p, seed=5)
    got = run_case(p, inp, grads, True, True, None)
    hpg = p.nheads // p.ngroups
    heads = [(0, h) for h in range(hpg)]
    ref = oracle.recurrence_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                inp["init_state"], grads["dy"], grads["dfinal"], heads=heads)
    check(got["dx"][0, :, :hpg], ref["dx"][0, :, :hpg], "bf16", "dx[0,:,g0]")
    check(got["ddt"][0, :, :hpg], ref["ddt"][0, :, :hpg], "f32out", "ddt[0,:,g0]")
    check(got["dinit"][0, :hpg], ref["dinit"][0, :hpg], "f32out", "dinit[0,g0]")
    check(got["dB"][0, :, 0], ref["dB"][0, :, 0], "bf16", "dB[0,:,0]")
    check(got["dC"][0, :, 0], ref["dC"][0, :, 0], "bf16", "dC[0,:,0]")
