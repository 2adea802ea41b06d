"""Property tests of the host-side validation (no GPU): for random problems
the workspace size follows the documented layout, and for random bad fields
the first failing check in the documented order is the one reported."""
import ctypes

from hypothesis import given, settings, strategies as st

import state_space_sequence_03_amd as lib

OK, NULLP, SHAPE, CHUNK, DTYPE, MISAL, WS, UNSUP, BADVAL = 0, 1, 2, 3, 4, 5, 6, 7, 10
FAKE = 1 << 20


def r256(v):
    return (v + 255) // 256 * 256


HEADER = 256


def expected_staged(b, L, H, P, N, Q, bf16):
    Q = max(Q, 32)                                  # chunk 16 runs as 32
    T = -(-L // Q)
    Lp = T * Q
    g = b * H * Lp * 4
    nk = -(-N // 32)
    ksw = 1 if nk <= 1 else 2 if nk <= 2 else 4 if nk <= 4 else 8
    pb = -(-P // 64)
    state = pb * 4 * ksw * 512                      # fragment-major, padded tiles
    hc = b * H * T * state * (2 if bf16 else 4)
    return HEADER + r256(g) + r256(g) + r256(hc)


def fused_built(H, G, P, N, Q, bf16):
    return bf16 and P == 64 and N == 128 and Q == 256 and (H // G) % 2 == 0


def expected_fused(b, H, P, N):
    return HEADER + r256(b * H * (N // 32) * (P // 32) * 8) + r256(b * H * P * N * 4)


def expected_ws(b, L, H, G, P, N, Q, bf16):
    staged = expected_staged(b, L, H, P, N, Q, bf16)
    if fused_built(H, G, P, N, Q, bf16):
        return max(staged, expected_fused(b, H, P, N))
    return staged


valid = st.fixed_dictionaries({
    "batch": st.integers(1, 8), "seqlen": st.integers(1, 5000),
    "hpg": st.integers(1, 8), "ngroups": st.integers(1, 4),
    "headdim": st.sampled_from([16, 32, 64, 80, 128]),
    "dstate": st.sampled_from([16, 32, 48, 64, 128, 256]),
    "chunk_size": st.sampled_from([16, 32, 64, 128, 256]),
    "io_dtype": st.sampled_from([0, 1]),
})


def prob_of(d):
    return lib.make_problem(d["batch"], d["seqlen"], d["hpg"] * d["ngroups"], d["headdim"],
                            d["dstate"], d["ngroups"], d["chunk_size"], d["io_dtype"])


@settings(max_examples=300, deadline=None)
@given(valid)
def test_workspace_size_follows_the_layout(d):
    so = lib.load_library()
    n = ctypes.c_size_t(0)
    st_ = so.ssd_fwd_workspace_size(ctypes.byref(prob_of(d)), ctypes.byref(n))
    if st_ == UNSUP:
        # only fp32 chunks whose compute_out tiles exceed the LDS are refused
        assert d["io_dtype"] == 0
        return
    assert st_ == OK, lib.ssd_last_error_message()
    H = d["hpg"] * d["ngroups"]
    args = (d["batch"], d["seqlen"], H, d["ngroups"], d["headdim"], d["dstate"], d["chunk_size"],
            d["io_dtype"] == 1)
    assert n.value == expected_ws(*args)
    # the default configuration's own layout (the staged kernels'), and the
    # fused kernel's where it is built
    m = ctypes.c_size_t(0)
    assert so.ssd_fwd_config_workspace_size(ctypes.byref(prob_of(d)), None, ctypes.byref(m)) == OK
    assert m.value == expected_staged(d["batch"], d["seqlen"], H, d["headdim"], d["dstate"],
                                      d["chunk_size"], d["io_dtype"] == 1)
    if fused_built(H, d["ngroups"], d["headdim"], d["dstate"], d["chunk_size"], d["io_dtype"] == 1):
        cfg = lib.ssd_config(4, 1, 1, 1)
        assert so.ssd_fwd_config_workspace_size(ctypes.byref(prob_of(d)), ctypes.byref(cfg),
                                                ctypes.byref(m)) == OK
        assert m.value == expected_fused(d["batch"], H, d["headdim"], d["dstate"])


@settings(max_examples=50, deadline=None)
@given(valid)
def test_fused_layout_where_built(d):
    # the fused kernel's shapes drawn directly (rare among the examples above)
    d = dict(d, headdim=64, dstate=128, chunk_size=256, io_dtype=1, hpg=2 * (d["hpg"] % 4 + 1))
    so = lib.load_library()
    cfg = lib.ssd_config(4, 1, 1, 1)
    m = ctypes.c_size_t(0)
    assert so.ssd_fwd_config_workspace_size(ctypes.byref(prob_of(d)), ctypes.byref(cfg),
                                            ctypes.byref(m)) == OK, lib.ssd_last_error_message()
    assert m.value == expected_fused(d["batch"], d["hpg"] * d["ngroups"], 64, 128)


@settings(max_examples=300, deadline=None)
@given(valid, st.booleans(), st.booleans(), st.booleans(), st.booleans(), st.booleans())
def test_first_failing_check_is_reported(d, bad_shape, bad_chunk, bad_dtype, misaligned, unsup):
    so = lib.load_library()
    p = prob_of(d)
    if bad_shape:
        p.batch = 0
    if bad_chunk:
        p.chunk_size = 48
    if bad_dtype:
        p.io_dtype = 5
    if unsup:
        p.headdim = 72
    x = FAKE + 4 if misaligned else FAKE
    got = so.ssd_fwd(ctypes.byref(p), x, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, 0,
                     None)
    if bad_shape:
        want = SHAPE
    elif bad_chunk:
        want = CHUNK
    elif bad_dtype:
        want = DTYPE
    elif misaligned:
        want = MISAL
    elif unsup:
        want = UNSUP
    else:
        want = None                   # workspace (0 bytes) or an fp32 LDS limit
    if want is None:
        assert got in (WS, UNSUP)
        if got == UNSUP:
            assert d["io_dtype"] == 0
    else:
        assert got == want, (got, want, lib.ssd_last_error_message())
