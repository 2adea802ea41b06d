"""GPU check of the running sums formed inside chunk_state.

ssd_config.cumsum_heads = 0 (the default) forms the within-chunk running sums
G and the prepared step sizes inside the chunk_state kernel, with the same
scan as the stand-alone chunk_cumsum kernel (cumsum_heads = 4 or 16), and
writes the same rows for the later stages.  Every later stage reads only
those rows, so y and the final state must be bitwise the same with either
choice; and within the bf16/fp32 tolerance of the oracle.  The cases span
every chunk size the kernels run (16 runs as 32), ragged tails and a single
token, both io dtypes, 1, 2 and 4 heads per chunk_state workgroup, dstate
slices, and the step-size preparation (bias, softplus, clamp).
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


CASES = {
    # name: (Problem kwargs, state_heads, dt preparation)
    "bf16_q256_kh4": (dict(batch=2, seqlen=700, nheads=8, headdim=64, dstate=128, ngroups=2,
                           chunk_size=256, io_dtype="bf16", init_std=0.1), 4, None),
    "bf16_q128_kh2_xf": (dict(batch=1, seqlen=333, nheads=4, headdim=64, dstate=64, ngroups=1,
                              chunk_size=128, io_dtype="bf16", init_std=0.1), 2,
                         (True, (0.001, 0.1))),
    "fp32_q64_kh1": (dict(batch=2, seqlen=130, nheads=3, headdim=32, dstate=32, ngroups=3,
                          chunk_size=64, io_dtype="fp32", init_std=0.1), 1, None),
    "fp32_q32_kh2_xf": (dict(batch=1, seqlen=75, nheads=4, headdim=16, dstate=16, ngroups=2,
                             chunk_size=32, io_dtype="fp32", init_std=0.1), 2,
                        (True, (0.0, float("inf")))),
    "fp32_q16_kh4": (dict(batch=1, seqlen=50, nheads=4, headdim=16, dstate=16, ngroups=1,
                          chunk_size=16, io_dtype="fp32"), 4, None),
    "bf16_q256_one_token": (dict(batch=2, seqlen=1, nheads=4, headdim=64, dstate=128, ngroups=1,
                                 chunk_size=256, io_dtype="bf16", init_std=0.1), 4, None),
    "bf16_q256_n256_kh4_xf": (dict(batch=1, seqlen=600, nheads=8, headdim=64, dstate=256,
                                   ngroups=2, chunk_size=256, io_dtype="bf16", init_std=0.1), 4,
                              (False, (0.002, 0.2))),
}


@pytest.mark.parametrize("name", sorted(CASES))
def test_folded_running_sums_equal_chunk_cumsum(name):
    kw, sh, xform = CASES[name]
    p = ssd_synth.Problem(**kw)
    inp = ssd_synth.make_inputs(p, seed=61)
    d = {k: (None if v is None else v.cuda()) for k, v in inp.items()}
    prob = lib.make_problem(p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups,
                            p.chunk_size, lib.SSD_BF16 if p.io_dtype == "bf16" else lib.SSD_F32)
    base = lib.ssd_default_config(prob)
    assert base["cumsum_heads"] == 0
    xkw, dt_arg, dt_ref = {}, d["dt"], inp["dt"]
    if xform is not None:
        sp, lim = xform
        xkw = dict(dt_bias=d["dt_bias"], dt_softplus=sp, dt_limit=lim)
        dt_arg = d["dt_raw"]
        dt_ref = oracle.dt_transform(inp["dt_raw"], inp["dt_bias"], sp, lim[0], lim[1])
    outs = {}
    for ch in (0, 4, 16):
        cfg = dict(base, cumsum_heads=ch, state_heads=sh, fused=0)
        outs[ch] = lib.ssd_fwd(d["x"], dt_arg, d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                               d["init_state"], config=cfg, **xkw)
    for ch in (4, 16):
        assert torch.equal(outs[0][0], outs[ch][0]), ("y", ch)
        assert torch.equal(outs[0][1], outs[ch][1]), ("final_state", ch)
    y_ref, fin_ref, _ = oracle.recurrence(inp["x"], dt_ref, inp["A"], inp["B"], inp["C"], inp["D"],
                                          inp["init_state"])
    assert_close(outs[0][0], y_ref, p.io_dtype, "y")
    assert_close(outs[0][1], fin_ref, p.io_dtype, "final_state")


def test_folded_running_sums_2p7b_shape():
    # the 2.7B layer shape, default choices against a chunk_cumsum launch
    p = ssd_synth.CONFIGS["mamba2_2p7b"]
    d = {k: (None if v is None else v.cuda()) for k, v in ssd_synth.make_inputs(p, 62).items()}
    prob = lib.make_problem(p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups,
                            p.chunk_size, lib.SSD_BF16)
    base = lib.ssd_default_config(prob)
    y0, f0 = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                         d["init_state"], config=base)
    y4, f4 = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                         d["init_state"], config=dict(base, cumsum_heads=4))
    assert torch.equal(y0, y4) and torch.equal(f0, f4)
    del d, y0, y4
    torch.cuda.empty_cache()
