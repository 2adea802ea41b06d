"""The forward pass under HIP graph capture.

The library enqueues kernels only (no allocation, memset or synchronisation
on the forward path), so a whole ssd_fwd can be captured once and replayed.
The graph is replayed several times, with the program's own eager work and
synchronisations between replays, and every replay is checked against the
eager result (bitwise: the path is deterministic) and the CPU oracle.
"""
import pytest
import torch

import oracle
import ssd_synth
from parity_util import assert_close

pytestmark = pytest.mark.gpu

lib = pytest.importorskip("state_space_sequence_03_amd")


@pytest.fixture(autouse=True)
def _announce(request):
    print("\n[gpu-case] %s" % request.node.name, flush=True)
    yield
    torch.cuda.synchronize()


@pytest.mark.parametrize("kw", [
    dict(batch=2, seqlen=700, nheads=4, headdim=64, dstate=128, ngroups=2, chunk_size=256,
         io_dtype="bf16", init_std=0.1),
    dict(batch=1, seqlen=256, nheads=2, headdim=16, dstate=16, ngroups=1, chunk_size=64,
         io_dtype="fp32", init_std=None),
], ids=["bf16_q256", "fp32_tiny"])
def test_forward_pass_replays_from_a_graph(kw):
    p = ssd_synth.Problem(**kw)
    inp = ssd_synth.make_inputs(p, seed=51)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    pr = lib.make_problem(p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups,
                          p.chunk_size, lib.SSD_BF16 if p.io_dtype == "bf16" else lib.SSD_F32)
    ws = torch.empty(lib.ssd_fwd_workspace_size(pr), dtype=torch.uint8, device="cuda")
    y = torch.empty_like(d["x"])
    fin = torch.empty((p.batch, p.nheads, p.headdim, p.dstate), dtype=torch.float32, device="cuda")

    def fwd():
        lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                    d["init_state"], out=y, final_out=fin, workspace=ws)

    fwd()                                   # eager (also sets per-device kernel attributes)
    torch.cuda.synchronize()
    y_eager, fin_eager = y.clone(), fin.clone()
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fwd()                               # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    with torch.cuda.graph(g):
        fwd()
    y_ref, fin_ref, _ = oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                                          inp["D"], inp["init_state"])
    for rep in range(4):
        y.zero_()
        fin.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y_eager) and torch.equal(fin, fin_eager), "replay %d" % rep
        assert_close(y, y_ref, p.io_dtype, "y (replay %d)" % rep)
        # eager work of the program's own between replays
        _ = (d["x"].float() * 2.0).sum().item()


def test_decode_step_replays_from_a_graph():
    # a captured decode step advances the resident state on every replay:
    # two replays equal two eager steps, bitwise
    p = ssd_synth.Problem(batch=4, seqlen=1, nheads=8, headdim=64, dstate=128, ngroups=1,
                          chunk_size=256, init_std=0.1)
    d = {k: (None if v is None else v.cuda()) for k, v in ssd_synth.make_inputs(p, seed=52).items()}
    y = torch.empty_like(d["x"])

    def step(state):
        lib.ssd_step(state, d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], out=y)

    eager = d["init_state"].clone()
    step(eager)
    step(eager)
    torch.cuda.synchronize()
    y_eager = y.clone()

    state = d["init_state"].clone()
    warm = d["init_state"].clone()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(warm)
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(state)
    # capture recorded the launch without running it: the state is unchanged
    torch.cuda.synchronize()
    assert torch.equal(state, d["init_state"])
    g.replay()
    _ = (d["x"].float() + 1.0).sum().item()
    g.replay()
    torch.cuda.synchronize()
    assert torch.equal(state, eager) and torch.equal(y, y_eager)


def test_backward_pass_replays_from_a_graph():
    # ssd_bwd enqueues kernels only as well: captured once (outputs and
    # workspace from the graph's pool), every replay equals the eager call
    p = ssd_synth.Problem(batch=2, seqlen=300, nheads=4, headdim=32, dstate=64, ngroups=2,
                          chunk_size=64, io_dtype="bf16", init_std=0.1)
    inp = ssd_synth.make_inputs(p, seed=53)
    gr = ssd_synth.make_grads(p, seed=53)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    dy, dfinal = gr["dy"].cuda(), gr["dfinal"].cuda()

    def bwd():
        return lib.ssd_bwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                           d["init_state"], dy, dfinal, want_ddt_bias=True)

    eager = bwd()
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        bwd()
    torch.cuda.current_stream().wait_stream(s)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        out = bwd()
    ref = oracle.recurrence_bwd(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"], inp["D"],
                                inp["init_state"], gr["dy"], gr["dfinal"])
    for rep in range(3):
        for t in out.values():
            t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for k in eager:
            assert torch.equal(out[k], eager[k]), "%s (replay %d)" % (k, rep)
        assert_close(out["dx"], ref["dx"], "bf16", "dx (replay %d)" % rep)
        _ = (d["x"].float() * 2.0).sum().item()
