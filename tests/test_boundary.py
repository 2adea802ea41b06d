"""The C-ABI library: it loads, exports what include/ssd.h declares, and
rejects bad arguments on the host with the documented codes, in the
documented order, before any HIP call (none of these calls reaches a kernel
launch, so they run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

from bwd_layout import balanced, bwd_layout, part_heads, parts
import state_space_sequence_03_amd as lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ssd.h")

OK, NULLP, SHAPE, CHUNK, DTYPE, MISAL, WS, UNSUP, BADVAL = 0, 1, 2, 3, 4, 5, 6, 7, 10


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(ssd_[a-z_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def so():
    if not os.path.exists(lib.lib_path()):
        from state_space_sequence_03_amd import build
        build.build()
    return lib.load_library()


def test_exports_every_declared_symbol(so):
    names = declared_functions()
    assert set(names) == {"ssd_abi_version", "ssd_status_string", "ssd_last_error_message",
                          "ssd_fwd_workspace_size", "ssd_fwd", "ssd_chunk_cumsum",
                          "ssd_fwd_states", "ssd_compute_out", "ssd_fwd_ex",
                          "ssd_chunk_cumsum_ex", "ssd_step", "ssd_fwd_states_ex",
                          "ssd_default_config", "ssd_fwd_config", "ssd_tune",
                          "ssd_bwd_workspace_size", "ssd_bwd_workspace_min_size", "ssd_bwd",
                          "ssd_fwd_config_workspace_size",
                          "ssd_fwd_status", "ssd_fwd_noalloc"}
    out = subprocess.run(["nm", "-D", "--defined-only", lib.lib_path()], capture_output=True,
                         text=True, check=True).stdout
    exported = set(line.split()[-1] for line in out.splitlines() if line.strip())
    for n in names:
        assert n in exported, n
        assert hasattr(so, n)


def test_version_and_strings(so):
    assert lib.ssd_abi_version() == 6
    for code in range(11):
        assert lib.ssd_status_string(code) and lib.ssd_status_string(code) != "unknown status"
    assert lib.ssd_status_string(77) == "unknown status"


def P(**kw):
    base = dict(batch=2, seqlen=1000, nheads=8, headdim=64, dstate=128, ngroups=2,
                chunk_size=256, io_dtype=1)
    base.update(kw)
    return lib.make_problem(**base)


def ws_status(prob):
    n = ctypes.c_size_t(0)
    return lib.load_library().ssd_fwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)), n.value


def cfg_ws(prob, cfg):
    n = ctypes.c_size_t(0)
    st = lib.load_library().ssd_fwd_config_workspace_size(
        ctypes.byref(prob), None if cfg is None else ctypes.byref(cfg), ctypes.byref(n))
    return st, n.value


def test_workspace_size_formula(so):
    # a 256-byte header, then the staged layout (running sums, step sizes,
    # chunk-start states) or the fused one (flags per 32x32 state tile, an
    # fp32 state); the plain size covers both
    r = lambda v: (v + 255) // 256 * 256
    hdr = 256
    T, Lp = 4, 1024
    g = 2 * 8 * Lp * 4
    hc = 2 * 8 * T * 64 * 128 * 2
    staged = hdr + r(g) + r(g) + r(hc)
    fused = hdr + r(2 * 8 * 4 * 2 * 8) + r(2 * 8 * 64 * 128 * 4)
    st, n = ws_status(P())
    assert st == OK and n == max(staged, fused)
    assert cfg_ws(P(), CFG(fused=0)) == (OK, staged)
    assert cfg_ws(P(), CFG(fused=1)) == (OK, fused)
    assert cfg_ws(P(), None) == (OK, staged)             # the default is the staged kernels
    # a shape the fused kernel is not built for: the staged layout only
    st, n32 = ws_status(P(io_dtype=0, dstate=64))
    staged32 = hdr + r(g) + r(g) + r(2 * 8 * T * 64 * 64 * 4)
    assert st == OK and n32 == staged32
    assert cfg_ws(P(io_dtype=0, dstate=64), None) == (OK, staged32)


def test_config_workspace_size_errors(so):
    f = lib.load_library().ssd_fwd_config_workspace_size
    n = ctypes.c_size_t(0)
    assert f(None, None, ctypes.byref(n)) == NULLP
    assert f(ctypes.byref(P()), None, None) == NULLP
    assert cfg_ws(P(batch=0), None)[0] == SHAPE
    assert cfg_ws(P(), CFG(fused=2))[0] == BADVAL
    assert cfg_ws(P(dstate=64), CFG(fused=1))[0] == BADVAL   # not built for dstate 64
    assert cfg_ws(P(dstate=272), None)[0] == UNSUP


def test_status_errors(so):
    f = lib.load_library().ssd_fwd_status
    t = ctypes.c_int32(7)
    assert f(ctypes.c_void_p(FAKE), 256, None, None) == NULLP
    assert f(ctypes.c_void_p(FAKE + 4), 256, None, ctypes.byref(t)) == MISAL
    assert f(ctypes.c_void_p(FAKE), 15, None, ctypes.byref(t)) == WS
    assert t.value == 7          # nothing written on an error


@pytest.mark.parametrize("kw,code", [
    (dict(batch=0), SHAPE), (dict(seqlen=-1), SHAPE), (dict(nheads=6, ngroups=4), SHAPE),
    (dict(headdim=0), SHAPE), (dict(seqlen=2 ** 40, nheads=2 ** 20), SHAPE),
    (dict(chunk_size=8), CHUNK), (dict(chunk_size=100), CHUNK), (dict(chunk_size=512), CHUNK),
    (dict(chunk_size=16), OK),
    (dict(io_dtype=7), DTYPE), (dict(headdim=72), UNSUP), (dict(dstate=40), UNSUP),
    (dict(dstate=272), UNSUP),
    (dict(chunk_size=32), OK), (dict(io_dtype=0, dstate=128), OK), (dict(io_dtype=0, dstate=256), OK),
])
def test_workspace_size_validation(so, kw, code):
    st, _ = ws_status(P(**kw))
    assert st == code, (st, lib.ssd_last_error_message())
    if code != OK:
        assert lib.ssd_last_error_message()


FAKE = 1 << 20          # 16-byte aligned, never dereferenced: validation fails first


def call_fwd(prob, x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, init=None, y=FAKE,
             fin=None, ws=FAKE, ws_bytes=0):
    so = lib.load_library()
    return so.ssd_fwd(ctypes.byref(prob), x, dt, A, B, C, D, init, y, fin, ws, ws_bytes, None)


def test_fwd_null_pointers(so):
    for k in ("x", "dt", "A", "B", "C", "y", "ws"):
        assert call_fwd(P(), **{k: None}) == NULLP
    assert so.ssd_fwd(None, FAKE, FAKE, FAKE, FAKE, FAKE, None, None, FAKE, None, FAKE, 0, None) == NULLP


def test_fwd_check_order(so):
    # NULL beats shape, shape beats chunk, chunk beats dtype, dtype beats alignment,
    # alignment beats unsupported, unsupported beats workspace
    assert call_fwd(P(batch=0), x=None) == NULLP
    assert call_fwd(P(batch=0, chunk_size=7)) == SHAPE
    assert call_fwd(P(chunk_size=7, io_dtype=9)) == CHUNK
    assert call_fwd(P(io_dtype=9), x=FAKE + 4) == DTYPE
    assert call_fwd(P(headdim=72), x=FAKE + 4) == MISAL
    assert call_fwd(P(headdim=72)) == UNSUP
    assert call_fwd(P()) == WS


@pytest.mark.parametrize("arg", ["x", "dt", "A", "B", "C", "D", "init", "y", "fin", "ws"])
def test_fwd_misaligned(so, arg):
    assert call_fwd(P(), **{arg: FAKE + 8}) == MISAL


def test_fwd_workspace_too_small(so):
    # ssd_fwd needs the default configuration's layout (the staged kernels')
    _, need = cfg_ws(P(), None)
    assert call_fwd(P(), ws_bytes=need - 1) == WS
    assert "needs" in lib.ssd_last_error_message()
    _, need = cfg_ws(P(chunk_size=128), None)
    assert call_fwd(P(chunk_size=128), ws_bytes=need - 1) == WS


def test_noalloc_validation(so):
    # argument errors and a problem beyond the built-in 64 MiB scratch are
    # reported before the scratch is looked up or anything is enqueued
    def call(prob, x=FAKE, y=FAKE):
        return so.ssd_fwd_noalloc(ctypes.byref(prob), None, x, FAKE, FAKE, FAKE, FAKE, None, None,
                                  y, None, None)
    assert call(P(), x=None) == NULLP
    assert call(P(), y=None) == NULLP
    assert call(P(batch=0)) == SHAPE
    assert call(P(), x=FAKE + 4) == MISAL
    assert call(P(headdim=72)) == UNSUP
    big = P(batch=8, seqlen=4096, nheads=64, dstate=256, ngroups=8, chunk_size=128)
    assert cfg_ws(big, None)[1] > 64 << 20
    assert call(big) == WS
    assert "scratch" in lib.ssd_last_error_message()


def test_states_and_cumsum_validation(so):
    prob = P()
    assert so.ssd_fwd_states(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, None, None, None, FAKE, 0,
                             None) == NULLP
    assert so.ssd_fwd_states(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 0,
                             None) == WS
    bad = P(chunk_size=48)
    assert so.ssd_fwd_states(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE, 0,
                             None) == CHUNK
    assert so.ssd_chunk_cumsum(ctypes.byref(prob), None, FAKE, FAKE, FAKE, None) == NULLP
    assert so.ssd_chunk_cumsum(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None) == CHUNK
    assert so.ssd_chunk_cumsum(ctypes.byref(prob), FAKE, FAKE + 4, FAKE, FAKE, None) == MISAL


def test_chunk_16_runs_as_32(so):
    # y, the final state and the gradients do not depend on the chunk size:
    # the forward and backward entry points run chunk 16 as 32 (same
    # workspace), the entry points that return per-chunk states refuse it
    assert ws_status(P(chunk_size=16)) == ws_status(P(chunk_size=32))
    assert cfg_ws(P(chunk_size=16), None) == cfg_ws(P(chunk_size=32), None)
    prob = P(chunk_size=16)
    assert so.ssd_fwd_states(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE, None, FAKE, None, FAKE,
                             1 << 30, None) == UNSUP
    assert "chunk_size 16" in lib.ssd_last_error_message()
    assert so.ssd_compute_out(ctypes.byref(prob), FAKE, FAKE, FAKE, None, FAKE, FAKE, 1 << 30,
                              None) == UNSUP
    # ssd_fwd with chunk 16 passes validation up to the workspace check
    assert call_fwd(P(chunk_size=16)) == WS


def test_reserved_field_must_be_zero(so):
    prob = P()
    prob.reserved = 1
    assert call_fwd(prob) == DTYPE


def test_python_binding_rejects_cpu_tensors(so):
    import torch
    x = torch.zeros(1, 64, 2, 16, dtype=torch.bfloat16)
    B = torch.zeros(1, 64, 1, 16, dtype=torch.bfloat16)
    with pytest.raises(lib.SsdArgumentError):
        lib.ssd_fwd(x, torch.ones(1, 64, 2), -torch.ones(2), B, B, None, 64)


def test_compute_out_validation(so):
    prob = P()
    assert so.ssd_compute_out(ctypes.byref(prob), FAKE, FAKE, None, None, FAKE, FAKE, 0, None) == NULLP
    assert so.ssd_compute_out(ctypes.byref(prob), FAKE, FAKE, FAKE, FAKE + 4, FAKE, FAKE, 0, None) == MISAL
    assert so.ssd_compute_out(ctypes.byref(prob), FAKE, FAKE, FAKE, None, FAKE, FAKE, 0, None) == WS
    bad = P(io_dtype=3)
    assert so.ssd_compute_out(ctypes.byref(bad), FAKE, FAKE, FAKE, None, FAKE, FAKE, 0, None) == DTYPE


# ------------------------------------------- raw step size and the decode step

def XF(bias=None, softplus=1, reserved=0, lo=0.0, hi=float("inf")):
    return lib.ssd_dt_transform(bias, softplus, reserved, lo, hi)


def call_fwd_ex(prob, xf, **kw):
    so = lib.load_library()
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, init=None, y=FAKE, fin=None,
             ws=FAKE, ws_bytes=0)
    a.update(kw)
    return so.ssd_fwd_ex(ctypes.byref(prob), None if xf is None else ctypes.byref(xf), a["x"],
                         a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"], a["y"], a["fin"],
                         a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("xf", [XF(softplus=2), XF(reserved=1), XF(lo=float("nan")),
                                XF(hi=float("nan")), XF(lo=1.0, hi=0.5)],
                         ids=["softplus2", "reserved", "nan_lo", "nan_hi", "lo_gt_hi"])
def test_fwd_ex_rejects_bad_transform(so, xf):
    assert call_fwd_ex(P(), xf) == BADVAL
    assert "dt transform" in lib.ssd_last_error_message()
    assert so.ssd_chunk_cumsum_ex(ctypes.byref(P()), ctypes.byref(xf), FAKE, FAKE, FAKE, FAKE,
                                  None) == BADVAL
    assert so.ssd_fwd_states_ex(ctypes.byref(P()), ctypes.byref(xf), FAKE, FAKE, FAKE, FAKE, None,
                                FAKE, None, FAKE, 0, None) == BADVAL


def test_fwd_ex_check_order(so):
    # dtype beats the transform's values, the transform beats alignment
    assert call_fwd_ex(P(io_dtype=9), XF(softplus=5)) == DTYPE
    assert call_fwd_ex(P(), XF(softplus=5), x=FAKE + 4) == BADVAL
    assert call_fwd_ex(P(), XF(bias=FAKE + 4)) == MISAL
    assert call_fwd_ex(P(), XF(bias=FAKE)) == WS          # a good transform reaches the size check
    assert call_fwd_ex(P(), None) == WS                     # NULL transform = ssd_fwd
    assert call_fwd_ex(P(), XF(), x=None) == NULLP


def call_step(prob, xf=None, state=FAKE, x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, y=FAKE):
    so = lib.load_library()
    return so.ssd_step(ctypes.byref(prob) if prob is not None else None,
                       None if xf is None else ctypes.byref(xf), state, x, dt, A, B, C, D, y, None)


def test_step_validation(so):
    for k in ("state", "x", "dt", "A", "B", "C", "y"):
        assert call_step(P(batch=0), **{k: None}) == NULLP
    assert call_step(None) == NULLP
    assert call_step(P(batch=0)) == SHAPE
    assert call_step(P(nheads=6, ngroups=4)) == SHAPE
    assert call_step(P(io_dtype=3, batch=0)) == SHAPE
    assert call_step(P(io_dtype=3)) == DTYPE
    assert call_step(P(), XF(lo=3.0, hi=2.0)) == BADVAL
    for k in ("state", "x", "dt", "A", "B", "C", "D", "y"):
        assert call_step(P(), **{k: FAKE + 8}) == MISAL
    assert call_step(P(), XF(bias=FAKE + 8)) == MISAL
    assert call_step(P(headdim=72)) == UNSUP
    assert call_step(P(dstate=40)) == UNSUP
    assert call_step(P(dstate=272)) == UNSUP


def test_step_ignores_chunk_size(so):
    # the decode step does not chunk: an invalid chunk size is not an error
    # (the call stops at the first later check, here the dtype)
    assert call_step(P(chunk_size=48, io_dtype=5)) == DTYPE
    assert call_step(P(chunk_size=0, io_dtype=5)) == DTYPE


# ------------------------------------------------------------ tile choices

def CFG(ch=4, sh=4, oh=2, fused=0, res=0):
    return lib.ssd_config(ch, sh, oh, fused, res)


def call_fwd_config(prob, cfg, **kw):
    so = lib.load_library()
    a = dict(x=FAKE, dt=FAKE, A=FAKE, B=FAKE, C=FAKE, D=None, init=None, y=FAKE, fin=None,
             ws=FAKE, ws_bytes=0)
    a.update(kw)
    return so.ssd_fwd_config(ctypes.byref(prob), None if cfg is None else ctypes.byref(cfg), None,
                             a["x"], a["dt"], a["A"], a["B"], a["C"], a["D"], a["init"], a["y"],
                             a["fin"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,cfg", [
    (dict(), CFG(ch=8)), (dict(), CFG(sh=3)), (dict(), CFG(oh=3)), (dict(), CFG(fused=2)),
    (dict(chunk_size=128), CFG(fused=1)),              # the fused kernel is built for chunk 256
    (dict(nheads=6, ngroups=2), CFG(sh=1, oh=1, fused=1)),   # 3 heads per group: odd
    (dict(nheads=4, ngroups=2), CFG(sh=4)),            # 2 heads per group: 4 does not divide
    (dict(io_dtype=0), CFG(oh=2)),                     # fp32: one head per compute_out workgroup
    (dict(dstate=256), CFG(oh=2)),                     # dstate 256: accumulators do not fit twice
    (dict(nheads=6, ngroups=2), CFG(sh=1, oh=2)),      # 3 heads per group: odd
    (dict(), CFG(res=2)),
    (dict(chunk_size=128), CFG(res=1)),                # the resident tile is built for chunk 256
    (dict(io_dtype=0), CFG(oh=1, res=1)),              # ... for bf16 io
    (dict(dstate=144), CFG(oh=1, res=1)),              # ... for dstate <= 128
    (dict(headdim=128), CFG(res=1)),                   # ... for headdim 64
], ids=["cumsum8", "state3", "out3", "fused2", "fused_q128", "fused_odd", "state4_hg2", "out2_fp32",
        "out2_n256", "out2_odd", "resident2", "resident_q128", "resident_fp32", "resident_n144",
        "resident_p128"])
def test_fwd_config_rejects_bad_choice(so, kw, cfg):
    assert call_fwd_config(P(**kw), cfg) == BADVAL
    assert "config" in lib.ssd_last_error_message()


def test_fwd_config_check_order_and_default(so):
    assert call_fwd_config(P(io_dtype=9), CFG(ch=8)) == DTYPE          # dtype first
    assert call_fwd_config(P(), CFG(ch=8), x=FAKE + 4) == BADVAL       # then the choice
    assert call_fwd_config(P(), CFG(ch=16, sh=2, oh=1)) == WS           # a valid one passes on
    assert call_fwd_config(P(), None) == WS                             # NULL = the default


@pytest.mark.parametrize("kw,want", [
    (dict(batch=2, seqlen=8192, nheads=80, headdim=64, dstate=128, ngroups=1, chunk_size=256),
     dict(cumsum_heads=0, state_heads=4, out_heads=2, fused=0, out_resident=1)),
    (dict(batch=8, seqlen=4096, nheads=64, headdim=64, dstate=256, ngroups=8, chunk_size=128),
     dict(cumsum_heads=0, state_heads=4, out_heads=1, fused=0, out_resident=0)),
    (dict(nheads=6, ngroups=3), dict(cumsum_heads=0, state_heads=2, out_heads=2, fused=0, out_resident=1)),
    (dict(nheads=6, ngroups=2), dict(cumsum_heads=0, state_heads=1, out_heads=1, fused=0, out_resident=1)),
    (dict(nheads=3, ngroups=3, io_dtype=0), dict(cumsum_heads=0, state_heads=1, out_heads=1, fused=0, out_resident=0)),
])
def test_default_config_is_the_static_table(so, kw, want):
    assert lib.ssd_default_config(P(**kw)) == want


def test_tune_validation(so):
    so_ = lib.load_library()
    prob = P()
    _, need = ws_status(prob)
    best, n, ms = lib.ssd_config(), ctypes.c_int32(0), ctypes.c_float(0)

    def tune(reps=3, init=None, fin=FAKE, tried=None, tried_ms=None, max_tried=0, best_p=True,
             ws_bytes=need):
        return so_.ssd_tune(ctypes.byref(prob), None, FAKE, FAKE, FAKE, FAKE, FAKE, None, init, FAKE,
                            fin, FAKE, ws_bytes, None, reps, tried, tried_ms, max_tried,
                            ctypes.byref(n), ctypes.byref(best) if best_p else None, ctypes.byref(ms))
    assert tune(best_p=False) == NULLP
    assert tune(ws_bytes=0) == WS
    assert tune(reps=0) == BADVAL
    assert tune(reps=1001) == BADVAL
    assert tune(max_tried=2) == BADVAL                 # arrays missing
    assert tune(max_tried=-1) == BADVAL
    assert tune(init=FAKE, fin=FAKE) == BADVAL         # init_state aliases final_state


# ------------------------------------------------------------ built device code

LLVM = "/opt/rocm/llvm/bin"
BUILD_DIR = os.path.join(ROOT, "state_space_sequence_03_amd", "_build")
KERNEL_OBJECTS = ["chunk_cumsum.o", "chunk_state.o", "state_pass.o", "compute_out.o", "step.o",
                  "bwd.o", "fused_fwd.o", "out_resident.o"]


def device_disassembly(obj, tmp_path):
    """gfx950 disassembly of the device code object built into `obj`."""
    fat = tmp_path / (obj + ".fatbin")
    dev = tmp_path / (obj + ".co")
    subprocess.run([f"{LLVM}/llvm-objcopy", "--dump-section", f".hip_fatbin={fat}",
                    os.path.join(BUILD_DIR, obj), str(tmp_path / (obj + ".host"))], check=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fat}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"], check=True)
    out = subprocess.run([f"{LLVM}/llvm-objdump", "-d", str(dev)], check=True,
                         capture_output=True, text=True).stdout
    return [l.split("//")[0].strip() for l in out.splitlines() if l.startswith("\t")]


def device_functions(obj, tmp_path):
    """The disassembly of `obj`'s device code split by function symbol."""
    fat = tmp_path / (obj + ".fatbin2")
    dev = tmp_path / (obj + ".co2")
    subprocess.run([f"{LLVM}/llvm-objcopy", "--dump-section", f".hip_fatbin={fat}",
                    os.path.join(BUILD_DIR, obj), str(tmp_path / (obj + ".host2"))], check=True)
    subprocess.run([f"{LLVM}/clang-offload-bundler", "--unbundle", "--type=o", f"--input={fat}",
                    "--targets=hipv4-amdgcn-amd-amdhsa--gfx950", f"--output={dev}"], check=True)
    out = subprocess.run([f"{LLVM}/llvm-objdump", "-d", str(dev)], check=True,
                         capture_output=True, text=True).stdout
    funcs, cur = {}, None
    for line in out.splitlines():
        m = re.match(r"^[0-9a-f]+ <(.+)>:$", line)
        if m:
            cur = funcs.setdefault(m.group(1), [])
        elif line.startswith("\t") and cur is not None:
            cur.append(line.split("//")[0].strip())
    return funcs


@pytest.mark.skipif(not os.path.exists(f"{LLVM}/llvm-objdump"), reason="ROCm LLVM tools not installed")
@pytest.mark.parametrize("obj", KERNEL_OBJECTS)
def test_device_code_m0_and_scalar_stores(so, obj, tmp_path):
    # The direct-to-LDS load helper sets M0 in inline assembly; the compiler is
    # told M0 is clobbered there but may not honour that, so the built code
    # must write M0 nowhere else: every M0 write is followed (after at most an
    # s_nop) by the global_load_lds it configures.  No kernel writes memory
    # through the scalar data cache either.
    insts = device_disassembly(obj, tmp_path)
    assert insts, "no device code found"
    for k, ins in enumerate(insts):
        op = ins.split()[0] if ins else ""
        assert not re.match(r"s_(store|atomic|buffer_store|buffer_atomic|scratch_store|dcache_wb|dcache_discard)", op), ins
        fields = [f.strip() for f in ins[len(op):].split(",")]
        if fields and fields[0] == "m0" and op.startswith("s_"):
            nxt = [i for i in insts[k + 1:k + 3] if not i.startswith("s_nop")]
            assert nxt and nxt[0].startswith("global_load_lds"), (obj, ins, insts[k + 1:k + 3])
    if obj in ("chunk_state.o", "compute_out.o"):
        assert any(i.startswith("global_load_lds_dwordx4") for i in insts)
    # The saddr form of those loads takes a 64-bit SGPR base assembled from two
    # readfirstlane results.  The builtin returns a signed int, so widening it
    # directly sign-extends the low word (s_bfe_i64 ..., 0x200000) and the base
    # is invalid whenever bit 31 of the address is set; no kernel here needs a
    # signed 64-bit bitfield extract otherwise.
    if any(re.match(r"global_load_lds_dwordx4 v\d+, s\[", i) for i in insts):
        assert not any(i.startswith("s_bfe_i64") for i in insts), obj


def test_missing_library_fails_loudly(tmp_path, monkeypatch):
    # no fallback path: without libssd.so every entry point raises
    monkeypatch.setattr(lib, "_LIB_PATH", str(tmp_path / "libssd.so"))
    monkeypatch.setattr(lib, "_lib", None)
    with pytest.raises(ImportError):
        lib.load_library()
    with pytest.raises(ImportError):
        lib.ssd_abi_version()


# ---------------------------------------------------------------- backward

BWD_REQUIRED = ("x", "dt", "A", "B", "C", "dy", "dx", "ddt", "dA", "dB", "dC", "ws")
BWD_OPTIONAL = ("D", "init", "dfinal", "dD", "dinit", "dbias")


def call_bwd(prob, xf=None, ws_bytes=0, **kw):
    so = lib.load_library()
    a = {k: FAKE for k in BWD_REQUIRED}
    a.update({k: None for k in BWD_OPTIONAL})
    a.update(kw)
    return so.ssd_bwd(ctypes.byref(prob) if prob is not None else None,
                      None if xf is None else ctypes.byref(xf), a["x"], a["dt"], a["A"], a["B"],
                      a["C"], a["D"], a["init"], a["dy"], a["dfinal"], a["dx"], a["ddt"], a["dA"],
                      a["dB"], a["dC"], a["dD"], a["dinit"], a["dbias"], a["ws"], ws_bytes, None)


def bwd_ws(prob, fn="ssd_bwd_workspace_size"):
    n = ctypes.c_size_t(0)
    st = getattr(lib.load_library(), fn)(None if prob is None else ctypes.byref(prob),
                                         ctypes.byref(n))
    return st, n.value


def bwd_ws_min(prob):
    return bwd_ws(prob, "ssd_bwd_workspace_min_size")


def test_bwd_validation_order(so):
    for k in BWD_REQUIRED:
        assert call_bwd(P(batch=0), **{k: None}) == NULLP, k
    assert call_bwd(None) == NULLP
    assert call_bwd(P(batch=0)) == SHAPE
    assert call_bwd(P(nheads=6, ngroups=4)) == SHAPE
    assert call_bwd(P(chunk_size=48)) == CHUNK
    assert call_bwd(P(io_dtype=3)) == DTYPE
    assert call_bwd(P(), XF(lo=3.0, hi=2.0)) == BADVAL
    assert call_bwd(P(io_dtype=3), XF(lo=3.0, hi=2.0)) == DTYPE
    for k in BWD_REQUIRED + BWD_OPTIONAL:
        assert call_bwd(P(), **{k: FAKE + 8}) == MISAL, k
    assert call_bwd(P(), XF(bias=FAKE + 8)) == MISAL
    assert call_bwd(P(headdim=72)) == UNSUP
    assert call_bwd(P(dstate=272)) == UNSUP
    assert call_bwd(P(headdim=72), ws=FAKE + 8) == MISAL      # alignment before limits
    st, need = bwd_ws_min(P())
    assert st == OK and need > 0
    assert call_bwd(P(), ws_bytes=need - 1) == WS
    assert call_bwd(P(nheads=6, ngroups=4), ws_bytes=0) == SHAPE
    assert bwd_ws_min(None)[0] == NULLP
    assert bwd_ws_min(P(headdim=272))[0] == UNSUP


def test_bwd_limits(so):
    # headdim beyond 256 (dstate beyond 256 is the forward pass's limit too);
    # every headdim x dstate up to 256 x 256 fits the per-chunk kernels' LDS
    assert bwd_ws(P(headdim=272))[0] == UNSUP
    assert bwd_ws(P(dstate=272))[0] == UNSUP
    for pd in (dict(), dict(dstate=256), dict(headdim=128), dict(chunk_size=32),
               dict(io_dtype=0, chunk_size=128), dict(headdim=256, dstate=256),
               dict(io_dtype=0, headdim=256, dstate=256)):
        assert bwd_ws(P(**pd))[0] == OK, pd


def test_bwd_workspace_formula(so):
    # parts of kh heads (part_heads); default: all parts in one batch when
    # 2 dstate parts <= nheads headdim, else the parts whose sums fit one fp32
    # copy of x, at least 1024 / (batch * chunks), in balanced batches;
    # minimum: the smallest layout over the part counts
    cases = (dict(), dict(io_dtype=0, seqlen=77, chunk_size=64, ngroups=1),
             dict(headdim=128, dstate=64), dict(batch=2, seqlen=8192, nheads=80, headdim=64,
                                                dstate=128, ngroups=1, chunk_size=256),
             dict(batch=8, seqlen=4096, nheads=64, headdim=64, dstate=256, ngroups=8,
                  chunk_size=128),
             dict(batch=2, seqlen=2030, nheads=32, headdim=16, dstate=32, ngroups=2, chunk_size=32))
    for pd in cases:
        p = P(**pd)
        H, N, Pd = p.nheads, p.dstate, p.headdim
        T = -(-p.seqlen // p.chunk_size)
        npart = parts(p)
        hb = npart
        if 2 * N * npart > H * Pd:
            fit = max(1, H * Pd // (2 * N))
            hb = balanced(npart, min(npart, max(fit, -(-1024 // (p.batch * T)))))
        assert bwd_ws(p) == (OK, bwd_layout(p, hb)), pd
        want_min = min(bwd_layout(p, balanced(npart, c)) for c in range(1, npart + 1))
        assert bwd_ws_min(p) == (OK, want_min), pd
    # the 2.7B layer shape: 16 parts of five heads, all in one batch, under 650 MB
    p = P(**cases[3])
    assert part_heads(p) == 5
    assert bwd_ws(p)[1] == bwd_layout(p, 16) < 650 * 10 ** 6
    # four-head parts in two groups at the last case's shape
    assert part_heads(P(**cases[5])) == 4


@pytest.mark.skipif(not os.path.exists(f"{LLVM}/llvm-objdump"), reason="ROCm LLVM tools not installed")
def test_resident_kernel_memory_operation_counts(so, tmp_path):
    # The resident-tile kernel waits for one head's loads with a vmcnt target
    # that counts the stores issued after them: 4 stores of 16 bytes per wave
    # and head (whole y rows out of the wave's LDS staging; never merged,
    # never branched around), after 8 direct loads of the next head (4 x
    # blocks, 2 state blocks, the G and dt rows).  The built code must have
    # exactly that shape: 4 buffer_store_dwordx4; the only other
    # stores write the status word (the call record before the first load,
    # and a bounded wait's timeout report, a path that only a bug takes); and
    # every vector load of the head loop a direct-to-LDS one.
    funcs = device_functions("out_resident.o", tmp_path)
    kernels = [f for f in funcs if "out_resident_kernel" in f]
    assert len(kernels) == 3, list(funcs)             # dstate steps 1, 2 and 4
    for f in kernels:
        insts = funcs[f]
        stores = [i for i in insts if re.match(r"buffer_store", i)]
        assert len(stores) == 4 and all(i.startswith("buffer_store_dwordx4") for i in stores), (f, stores)
        first_load = min(k for k, i in enumerate(insts) if i.startswith("global_load"))
        others = [k for k, i in enumerate(insts) if re.match(r"(global|flat)_store", i)]
        assert others and others[0] < first_load, (f, [insts[k] for k in others])
        assert all(re.match(r"global_store_dwordx2 .* sc1$", insts[k]) for k in others), \
            (f, [insts[k] for k in others])
        loads = [i.split()[0] for i in insts if re.match(r"(buffer|global|flat)_load", i)]
        assert set(loads) <= {"global_load_lds_dwordx4", "global_load_dwordx4"}, (f, set(loads))
        # no register spills either: their scratch traffic would be vector
        # memory operations the per-head counts do not include
        assert not any(i.startswith("scratch_") for i in insts), f
