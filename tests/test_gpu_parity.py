"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Element-by-element comparisons on seeded inputs, at sizes the oracle finishes
in seconds that still span several tiles and a ragged tail, plus the five
workload shapes at full size, every (batch, head) of them compared with the
oracle (the two largest a range of heads at a time, so only one range of the
fp64 reference is held at once).  Tolerances: bf16 operands -- rel-L2 <= 5e-3
and max-abs <= 2e-2 * max|ref| on y and final_state; fp32 operands -- rel-L2
<= 1e-5; chunk cumsum -- |G - G_ref| <= 1e-5 |G_ref| + 1e-6 elementwise.
"""
import math

import numpy as np
import pytest
import torch

import oracle
import ssd_synth
from parity_util import WholeTensorError, assert_close, errors

pytestmark = pytest.mark.gpu

lib = pytest.importorskip("state_space_sequence_03_amd")


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu-case] %s" % request.node.name, flush=True)
    yield
    torch.cuda.synchronize()


def to_dev(inp):
    return {k: (None if v is None else v.cuda()) for k, v in inp.items()}


def gpu_fwd(dinp, Q, use_D=True, use_init=True):
    return lib.ssd_fwd(dinp["x"], dinp["dt"], dinp["A"], dinp["B"], dinp["C"],
                       dinp["D"] if use_D else None, Q,
                       dinp["init_state"] if use_init else None)


def oracle_fwd(inp, use_D=True, use_init=True, **kw):
    return oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                             inp["D"] if use_D else None,
                             inp["init_state"] if use_init else None, **kw)


def prob(**kw):
    base = dict(batch=1, seqlen=300, nheads=3, headdim=64, dstate=64, ngroups=1,
                chunk_size=64, io_dtype="bf16", init_std=0.1)
    base.update(kw)
    return ssd_synth.Problem(**base)


# ------------------------------------------------------------ stage 1 alone

@pytest.mark.parametrize("L,H,Q", [(256, 2, 64), (300, 5, 32), (1000, 17, 128), (2048, 48, 256),
                                   (777, 80, 256), (1, 3, 32), (300, 5, 16), (1, 3, 16)])
def test_chunk_cumsum(L, H, Q):
    p = prob(seqlen=L, nheads=H, chunk_size=Q)
    inp = ssd_synth.make_inputs(p, seed=L + H)
    G, dtt = lib.ssd_chunk_cumsum(inp["dt"].cuda(), inp["A"].cuda(), Q)
    Gref = oracle.chunk_cumsum(inp["dt"], inp["A"], Q)
    Gg = G.cpu().double().numpy()
    assert np.all(np.abs(Gg - Gref) <= 1e-5 * np.abs(Gref) + 1e-6)
    np.testing.assert_array_equal(dtt.cpu().numpy(), inp["dt"].permute(0, 2, 1).numpy())


@pytest.mark.parametrize("io", ["bf16", "fp32"])
def test_fwd_chunk_16(io):
    # chunk 16 runs as 32: the same kernels, so the same bits as chunk 32,
    # and the recurrence's result (the oracle does not chunk)
    p = prob(batch=2, seqlen=333, nheads=4, headdim=64, dstate=64, ngroups=2, chunk_size=16,
             io_dtype=io, init_std=0.1)
    inp = ssd_synth.make_inputs(p, seed=16)
    d = to_dev(inp)
    y16, f16 = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 16, d["init_state"])
    y32, f32 = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 32, d["init_state"])
    assert torch.equal(y16, y32) and torch.equal(f16, f32)
    y_ref, f_ref, _ = oracle_fwd(inp)
    assert_close(y16, y_ref, io, "y")
    assert_close(f16, f_ref, io, "final_state")


def test_chunk_cumsum_closed_forms():
    L, H, Q = 512, 4, 128
    dt = torch.full((2, L, H), 0.03125)
    A = torch.tensor([-1.0, -0.5, -8.0, 0.0])
    G, _ = lib.ssd_chunk_cumsum(dt.cuda(), A.cuda(), Q)
    i = np.arange(L) % Q
    ref = (i + 1)[None, None, :] * 0.03125 * A.double().numpy()[None, :, None] / math.log(2.0)
    Gg = G.cpu().double().numpy()
    assert np.all(np.abs(Gg - ref) <= 1e-5 * np.abs(ref) + 1e-6)
    assert np.all(Gg[:, 3] == 0.0)          # A = 0: no decay at all


# ------------------------------------------------------------ stages 1 + 2

@pytest.mark.parametrize("io", ["bf16", "fp32"])
@pytest.mark.parametrize("L,Q,P,N,G,H", [(300, 64, 64, 64, 1, 3), (1000, 128, 64, 128, 2, 4),
                                         (513, 256, 32, 48, 1, 2), (96, 32, 128, 256, 1, 1)])
def test_chunk_states(io, L, Q, P, N, G, H):
    p = prob(seqlen=L, chunk_size=Q, headdim=P, dstate=N, ngroups=G, nheads=H, io_dtype=io)
    inp = ssd_synth.make_inputs(p, seed=7)
    d = to_dev(inp)
    fin, cs = lib.ssd_fwd_states(d["x"], d["dt"], d["A"], d["B"], Q, d["init_state"])
    _, fin_ref, cs_ref = oracle_fwd(inp, chunk_size=Q, want_chunk_states=True)
    assert_close(fin, fin_ref, io, "final_state")
    assert_close(cs, cs_ref, io, "chunk_states")


# ------------------------------------------------------------ full pass, small

SMALL = [
    # (L, Q, P, N, G, H, batch)
    (300, 64, 64, 64, 1, 3, 1),
    (1000, 128, 64, 128, 2, 4, 2),
    (513, 256, 64, 128, 1, 2, 1),
    (777, 256, 128, 256, 2, 2, 1),
    (200, 32, 16, 16, 1, 2, 3),
    (130, 64, 32, 48, 3, 3, 1),
    (64, 64, 80, 96, 1, 1, 1),
    (1, 32, 64, 64, 1, 2, 1),
    (257, 256, 64, 128, 1, 1, 1),
]


@pytest.mark.parametrize("io", ["bf16", "fp32"])
@pytest.mark.parametrize("case", SMALL, ids=lambda c: "L%d_Q%d_P%d_N%d_G%d_H%d_B%d" % c)
def test_fwd_small(io, case):
    L, Q, P, N, G, H, bsz = case
    p = prob(seqlen=L, chunk_size=Q, headdim=P, dstate=N, ngroups=G, nheads=H, batch=bsz, io_dtype=io)
    inp = ssd_synth.make_inputs(p, seed=L)
    y, fin = gpu_fwd(to_dev(inp), Q)
    y_ref, fin_ref, _ = oracle_fwd(inp)
    assert_close(y, y_ref, io, "y")
    assert_close(fin, fin_ref, io, "final_state")


@pytest.mark.parametrize("use_D,use_init", [(False, True), (True, False), (False, False)])
def test_fwd_optional_inputs(use_D, use_init):
    p = prob(seqlen=400, chunk_size=128, nheads=2)
    inp = ssd_synth.make_inputs(p, seed=3)
    y, fin = gpu_fwd(to_dev(inp), 128, use_D, use_init)
    y_ref, fin_ref, _ = oracle_fwd(inp, use_D, use_init)
    assert_close(y, y_ref, "bf16", "y")
    assert_close(fin, fin_ref, "bf16", "final_state")


# ------------------------------------------------------------ the five workloads

def _full_check(name, heads_per_range=None):
    """The workload's whole y and final_state against the oracle.

    heads_per_range=None runs the oracle on the whole problem at once;
    otherwise on ranges of whole groups of about that many heads, with the
    whole-tensor rel-L2 and max-abs accumulated over the ranges."""
    p = ssd_synth.CONFIGS[name]
    idx = ssd_synth.CONFIG_ORDER.index(name)
    inp = ssd_synth.make_inputs(p, seed=idx)
    d = to_dev(inp)
    y, fin = gpu_fwd(d, p.chunk_size)
    torch.cuda.synchronize()
    del d
    if heads_per_range is None:
        y_ref, fin_ref, _ = oracle_fwd(inp)
        ry = assert_close(y, y_ref, p.io_dtype, name + " y")
        rf = assert_close(fin, fin_ref, p.io_dtype, name + " final_state")
    else:
        ey, ef = WholeTensorError(), WholeTensorError()
        for h0, h1, y_ref, fin_ref in oracle.recurrence_head_ranges(inp, heads_per_range):
            ey.add(y[:, :, h0:h1], y_ref)
            ef.add(fin[:, h0:h1], fin_ref)
            print("  heads %d..%d compared" % (h0, h1 - 1), flush=True)
        ry = ey.check(p.io_dtype, name + " y")
        rf = ef.check(p.io_dtype, name + " final_state")
    print("%s: y rel-L2 %.3e max-abs %.3e; final rel-L2 %.3e max-abs %.3e"
          % (name, ry[0], ry[1], rf[0], rf[1]), flush=True)
    return y, fin


def test_workload_tiny_fp32():
    _full_check("tiny_fp32")


def test_workload_780m():
    _full_check("mamba2_780m")


def test_workload_2p7b():
    _full_check("mamba2_2p7b")


def test_workload_long_prefill():
    # 131072 tokens x 80 heads: the fp64 reference of all heads would take 5.4 GB
    _full_check("long_prefill", heads_per_range=10)


def test_workload_large_state():
    _full_check("large_state", heads_per_range=16)


# ------------------------------------------------------------ invariants

def test_chunk_size_invariance():
    p = prob(seqlen=1000, nheads=4, dstate=128)
    inp = ssd_synth.make_inputs(p, seed=5)
    d = to_dev(inp)
    y_ref, fin_ref, _ = oracle_fwd(inp)
    outs = []
    for Q in (32, 64, 128, 256):
        y, fin = gpu_fwd(d, Q)
        assert_close(y, y_ref, "bf16", "y Q=%d" % Q)
        assert_close(fin, fin_ref, "bf16", "final Q=%d" % Q)
        outs.append(y.float())
    for o in outs[1:]:
        rl2, _ = errors(o, outs[0])
        assert rl2 < 5e-3


def test_deterministic():
    p = prob(seqlen=2048, nheads=8, dstate=128, chunk_size=256)
    d = to_dev(ssd_synth.make_inputs(p, seed=9))
    y1, f1 = gpu_fwd(d, 256)
    y2, f2 = gpu_fwd(d, 256)
    assert torch.equal(y1, y2) and torch.equal(f1, f2)


def test_continuation_two_calls():
    p = prob(seqlen=1536, nheads=4, dstate=128, chunk_size=256)
    inp = ssd_synth.make_inputs(p, seed=11)
    d = to_dev(inp)
    y, fin = gpu_fwd(d, 256)
    L1 = 768
    head = {k: (v[:, :L1].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    tail = {k: (v[:, L1:].contiguous() if k in ("x", "dt", "B", "C") else v) for k, v in d.items()}
    y1, f1 = gpu_fwd(head, 256)
    tail["init_state"] = f1
    y2, f2 = gpu_fwd(tail, 256)
    assert_close(torch.cat([y1, y2], 1), y, "bf16", "chained y")
    assert_close(f2, fin, "bf16", "chained final")


def test_final_state_aliases_init_state():
    p = prob(seqlen=700, nheads=3, dstate=128, chunk_size=128)
    inp = ssd_synth.make_inputs(p, seed=13)
    d = to_dev(inp)
    y_ref, fin_ref, _ = oracle_fwd(inp)
    state = d["init_state"].clone()
    y, fin = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 128, state,
                         final_out=state)
    assert fin.data_ptr() == state.data_ptr()
    assert_close(y, y_ref, "bf16", "y")
    assert_close(state, fin_ref, "bf16", "final (in place)")


def test_zero_decay_is_linear_attention():
    p = prob(seqlen=500, nheads=2, dstate=64, chunk_size=128)
    inp = ssd_synth.make_inputs(p, seed=17)
    inp["A"] = torch.zeros_like(inp["A"])
    y, fin = gpu_fwd(to_dev(inp), 128)
    y_ref, fin_ref = oracle.linear_attention(inp["x"], inp["dt"], inp["B"], inp["C"], inp["D"],
                                             inp["init_state"])
    assert_close(y, y_ref, "bf16", "y")
    assert_close(fin, fin_ref, "bf16", "final")


def test_strong_decay_stays_finite():
    # whole-chunk decays far below fp32 range: exp2 underflows, nothing overflows
    p = prob(seqlen=1024, nheads=4, dstate=128, chunk_size=256)
    inp = ssd_synth.make_inputs(p, seed=19)
    inp["A"] = torch.tensor([-32.0, -500.0, -1e4, -0.001])
    inp["dt"] = inp["dt"] * 10.0
    y, fin = gpu_fwd(to_dev(inp), 256)
    assert torch.isfinite(y.float()).all() and torch.isfinite(fin).all()
    y_ref, fin_ref, _ = oracle_fwd(inp)
    assert_close(y, y_ref, "bf16", "y")
    assert_close(fin, fin_ref, "bf16", "final")


def test_errors_enqueue_nothing():
    p = prob(seqlen=128, nheads=2)
    d = to_dev(ssd_synth.make_inputs(p, seed=1))
    with pytest.raises(lib.SsdArgumentError):
        lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 48)
    ws = torch.empty(16, dtype=torch.uint8, device="cuda")
    with pytest.raises(lib.SsdArgumentError):
        lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], 64, workspace=ws)


@pytest.mark.parametrize("kw", [dict(seqlen=300, nheads=3, dstate=64, chunk_size=64),
                                dict(seqlen=2048, nheads=8, dstate=128, chunk_size=256),
                                dict(seqlen=1000, nheads=4, dstate=128, chunk_size=128,
                                     io_dtype="fp32")],
                         ids=["L300_Q64", "L2048_Q256", "L1000_Q128_fp32"])
@pytest.mark.parametrize("fused", [0, 1], ids=["staged", "fused"])
def test_status_reports_no_timeout(kw, fused):
    # the kernels hand data between waves (compute_out) or between workgroups
    # (the fused kernel) through bounded waits; a wait past its bound would
    # mark the call in the workspace header.  Every call here must be clear,
    # on a workspace that starts with arbitrary contents.
    p = prob(**kw)
    inp = ssd_synth.make_inputs(p, seed=11)
    d = to_dev(inp)
    pr = lib.make_problem(p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups,
                          p.chunk_size, lib.SSD_BF16 if p.io_dtype == "bf16" else lib.SSD_F32)
    cfg = lib.ssd_default_config(pr)
    built = (p.io_dtype == "bf16" and p.headdim == 64 and p.dstate == 128 and p.chunk_size == 256
             and (p.nheads // p.ngroups) % 2 == 0)
    if fused and not built:
        pytest.skip("the fused kernel is not built for this shape")
    cfg["fused"] = fused
    ws = torch.randint(0, 256, (lib.ssd_fwd_workspace_size(pr),), dtype=torch.uint8, device="cuda")
    y, fin = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                         d["init_state"], workspace=ws, config=cfg)
    assert lib.ssd_fwd_status(ws) is False
    y_ref, fin_ref, _ = oracle_fwd(inp)
    assert_close(y, y_ref, p.io_dtype, "y")
    assert_close(fin, fin_ref, p.io_dtype, "final_state")
