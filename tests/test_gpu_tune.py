"""GPU parity of every tile choice (ssd_config) and the shape tuner.

Each valid combination of chunk_cumsum head tile, chunk_state heads per
workgroup and compute_out heads per workgroup must reproduce the CPU oracle
within the forward-pass tolerances (bf16: rel-L2 <= 5e-3, max-abs <= 2e-2
max|ref|; fp32: rel-L2 <= 1e-5); ssd_tune must measure every valid choice and
leave a correct result in its outputs.
"""
import itertools

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


def to_dev(inp):
    return {k: (None if v is None else v.cuda()) for k, v in inp.items()}


PROBLEMS = {
    # name: Problem kwargs (chunk sizes and group layouts the choices depend on)
    "q256_n128_g1": dict(batch=1, seqlen=600, nheads=8, headdim=64, dstate=128, ngroups=1,
                         chunk_size=256, io_dtype="bf16", init_std=0.1),
    "q128_n256_g2": dict(batch=2, seqlen=300, nheads=8, headdim=64, dstate=256, ngroups=2,
                         chunk_size=128, io_dtype="bf16", init_std=0.1),
    "q64_n64_fp32": dict(batch=1, seqlen=200, nheads=4, headdim=32, dstate=64, ngroups=1,
                         chunk_size=64, io_dtype="fp32", init_std=0.1),
}


def fused_built(p):
    hg = p.nheads // p.ngroups
    return (p.io_dtype == "bf16" and p.headdim == 64 and p.dstate == 128 and p.chunk_size == 256
            and hg % 2 == 0)


def resident_built(p):
    return (p.io_dtype == "bf16" and p.headdim == 64 and p.dstate <= 128 and p.chunk_size == 256
            and p.nheads * p.headdim <= 1 << 22)


def valid_configs(p):
    """The choices ssd_tune tries: the fused kernel where it is built (with
    the default staged fields), then every staged combination -- stage 3 as
    the head-pair kernel with 2 or 1 heads, or as the resident-tile kernel
    where that is built (out_heads then at its default)."""
    hg = p.nheads // p.ngroups
    pair2 = p.io_dtype == "bf16" and p.dstate <= 128 and hg % 2 == 0
    out = []
    if fused_built(p):
        d = lib.ssd_default_config(lib.make_problem(
            p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.ngroups, p.chunk_size,
            lib.SSD_BF16))
        d["fused"] = 1
        out.append(d)
    for ch, sh in itertools.product((0, 4, 16), (1, 2, 4)):
        if hg % sh:
            continue
        for oh in (1, 2):
            if oh == 2 and not pair2:
                continue
            out.append(dict(cumsum_heads=ch, state_heads=sh, out_heads=oh, fused=0,
                            out_resident=0))
        if resident_built(p):
            out.append(dict(cumsum_heads=ch, state_heads=sh, out_heads=2 if pair2 else 1,
                            fused=0, out_resident=1))
    return out


@pytest.mark.parametrize("name", sorted(PROBLEMS))
def test_every_tile_choice_matches_oracle(name):
    p = ssd_synth.Problem(**PROBLEMS[name])
    inp = ssd_synth.make_inputs(p, seed=41)
    d = to_dev(inp)
    y_ref, fin_ref, _ = oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                                          inp["D"], inp["init_state"])
    cfgs = valid_configs(p)
    assert len(cfgs) >= 2
    for cfg in cfgs:
        y, fin = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                             d["init_state"], config=cfg)
        assert_close(y, y_ref, p.io_dtype, "y %s" % cfg)
        assert_close(fin, fin_ref, p.io_dtype, "final %s" % cfg)


def test_tune_measures_every_choice():
    p = ssd_synth.Problem(**PROBLEMS["q256_n128_g1"])
    inp = ssd_synth.make_inputs(p, seed=42)
    d = to_dev(inp)
    best, best_ms, rows = lib.ssd_tune(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"],
                                       p.chunk_size, d["init_state"], reps=3)
    want = valid_configs(p)
    assert sorted(map(str, (c for c, _ in rows))) == sorted(map(str, want))
    assert all(ms > 0 for _, ms in rows)
    assert best in [c for c, _ in rows]
    assert best_ms == min(ms for _, ms in rows)
    # the chosen configuration computes the same result
    y, fin = lib.ssd_fwd(d["x"], d["dt"], d["A"], d["B"], d["C"], d["D"], p.chunk_size,
                         d["init_state"], config=best)
    y_ref, fin_ref, _ = oracle.recurrence(inp["x"], inp["dt"], inp["A"], inp["B"], inp["C"],
                                          inp["D"], inp["init_state"])
    assert_close(y, y_ref, "bf16", "y (tuned)")
    assert_close(fin, fin_ref, "bf16", "final (tuned)")


def test_tune_with_raw_step_size():
    p = ssd_synth.Problem(**PROBLEMS["q128_n256_g2"])
    inp = ssd_synth.make_inputs(p, seed=43)
    d = to_dev(inp)
    best, _, rows = lib.ssd_tune(d["x"], d["dt_raw"], d["A"], d["B"], d["C"], d["D"],
                                 p.chunk_size, d["init_state"], reps=1, dt_bias=d["dt_bias"],
                                 dt_softplus=True)
    assert len(rows) == len(valid_configs(p)) and best in [c for c, _ in rows]
