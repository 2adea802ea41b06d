"""libssd Python binding: the Mamba-2 chunked SSD scan on MI355X (forward pass,
decode step and backward pass).

Argument marshalling only.  Every step of the computation runs in the HIP
kernels of ``libssd.so`` (built in-tree by ``state_space_sequence_03_amd.build``);
PyTorch provides device memory and the current stream.  There is no CPU or
PyTorch fallback: importing works without the library, but every call raises
if ``libssd.so`` is missing or the tensors are not on a GPU.  The environment
variable SSD_LIBRARY names another build of the library to load instead
(the host sanitizer tests use it).

Names match the C ABI in include/ssd.h:
    ssd_fwd, ssd_fwd_ex, ssd_fwd_states, ssd_fwd_states_ex, ssd_compute_out, ssd_chunk_cumsum,
    ssd_chunk_cumsum_ex, ssd_step, ssd_default_config, ssd_tune, ssd_fwd_workspace_size,
    ssd_fwd_config_workspace_size, ssd_fwd_status, ssd_fwd_noalloc, ssd_bwd,
    ssd_bwd_workspace_size, ssd_bwd_workspace_min_size, ssd_status_string,
    ssd_last_error_message, ssd_abi_version
(ssd_fwd_config is reached through ssd_fwd(..., config=...).)
"""
from __future__ import annotations

import ctypes
import os
import threading
from typing import Optional, Tuple

import torch

__all__ = ["SsdError", "SsdArgumentError", "lib_path", "load_library", "make_problem",
           "ssd_abi_version", "ssd_status_string", "ssd_last_error_message",
           "ssd_fwd_workspace_size", "ssd_fwd", "ssd_fwd_states", "ssd_compute_out",
           "ssd_chunk_cumsum", "ssd_fwd_ex", "ssd_fwd_states_ex", "ssd_chunk_cumsum_ex",
           "ssd_step", "ssd_default_config", "ssd_tune", "ssd_bwd_workspace_size",
           "ssd_bwd_workspace_min_size", "ssd_bwd",
           "ssd_fwd_config_workspace_size", "staged_workspace_size", "ssd_fwd_status",
           "ssd_fwd_noalloc", "SSD_F32", "SSD_BF16"]

SSD_F32, SSD_BF16 = 0, 1
_STATUS_NAMES = {0: "SSD_OK", 1: "SSD_ERR_NULL_POINTER", 2: "SSD_ERR_BAD_SHAPE",
                 3: "SSD_ERR_BAD_CHUNK", 4: "SSD_ERR_BAD_DTYPE", 5: "SSD_ERR_MISALIGNED",
                 6: "SSD_ERR_WORKSPACE", 7: "SSD_ERR_UNSUPPORTED", 8: "SSD_ERR_HIP",
                 9: "SSD_ERR_INTERNAL", 10: "SSD_ERR_BAD_VALUE"}
_ARG_ERRORS = {1, 2, 3, 4, 5, 6, 7, 10}

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.environ.get("SSD_LIBRARY") or os.path.join(_HERE, "libssd.so")
ABI_VERSION = 6   # SSD_ABI_VERSION of include/ssd.h: the struct layouts declared below
_lock = threading.Lock()
_lib = None


class SsdError(RuntimeError):
    """A libssd call failed at run time (HIP or internal error)."""

    def __init__(self, status: int, message: str):
        self.status = status
        super().__init__("%s: %s" % (_STATUS_NAMES.get(status, str(status)), message))


class SsdArgumentError(SsdError, ValueError):
    """A libssd call rejected its arguments (nothing was enqueued)."""


class ssd_problem(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int64), ("seqlen", ctypes.c_int64),
                ("nheads", ctypes.c_int64), ("headdim", ctypes.c_int64),
                ("dstate", ctypes.c_int64), ("ngroups", ctypes.c_int64),
                ("chunk_size", ctypes.c_int64), ("io_dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ssd_dt_transform(ctypes.Structure):
    _fields_ = [("dt_bias", ctypes.c_void_p), ("softplus", ctypes.c_int32),
                ("reserved", ctypes.c_int32), ("dt_min", ctypes.c_float),
                ("dt_max", ctypes.c_float)]


class ssd_config(ctypes.Structure):
    _fields_ = [("cumsum_heads", ctypes.c_int32), ("state_heads", ctypes.c_int32),
                ("out_heads", ctypes.c_int32), ("fused", ctypes.c_int32),
                ("out_resident", ctypes.c_int32)]

    def as_dict(self):
        return {"cumsum_heads": self.cumsum_heads, "state_heads": self.state_heads,
                "out_heads": self.out_heads, "fused": self.fused,
                "out_resident": self.out_resident}


def _config_of(cfg) -> Optional["ssd_config"]:
    if cfg is None or isinstance(cfg, ssd_config):
        return cfg
    return ssd_config(int(cfg["cumsum_heads"]), int(cfg["state_heads"]), int(cfg["out_heads"]),
                      int(cfg.get("fused", 0)), int(cfg.get("out_resident", 0)))


def lib_path() -> str:
    return _LIB_PATH


def load_library():
    """Open libssd.so and declare its entry points (raises if not built)."""
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libssd.so is not built (run python -m state_space_sequence_03_amd.build)")
        lib = ctypes.CDLL(_LIB_PATH)
        lib.ssd_abi_version.restype = ctypes.c_int
        if lib.ssd_abi_version() != ABI_VERSION:
            raise ImportError("%s has ABI version %d, this binding needs %d (rebuild it)"
                              % (_LIB_PATH, lib.ssd_abi_version(), ABI_VERSION))
        P, vp, sz = ctypes.POINTER(ssd_problem), ctypes.c_void_p, ctypes.c_size_t
        lib.ssd_abi_version.restype = ctypes.c_int
        lib.ssd_abi_version.argtypes = []
        lib.ssd_status_string.restype = ctypes.c_char_p
        lib.ssd_status_string.argtypes = [ctypes.c_int]
        lib.ssd_last_error_message.restype = ctypes.c_char_p
        lib.ssd_last_error_message.argtypes = []
        lib.ssd_fwd_workspace_size.restype = ctypes.c_int
        lib.ssd_fwd_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
        lib.ssd_fwd.restype = ctypes.c_int
        lib.ssd_fwd.argtypes = [P] + [vp] * 10 + [sz, vp]
        lib.ssd_chunk_cumsum.restype = ctypes.c_int
        lib.ssd_chunk_cumsum.argtypes = [P] + [vp] * 5
        lib.ssd_fwd_states.restype = ctypes.c_int
        lib.ssd_fwd_states.argtypes = [P] + [vp] * 8 + [sz, vp]
        lib.ssd_compute_out.restype = ctypes.c_int
        lib.ssd_compute_out.argtypes = [P] + [vp] * 6 + [sz, vp]
        X = ctypes.POINTER(ssd_dt_transform)
        lib.ssd_fwd_ex.restype = ctypes.c_int
        lib.ssd_fwd_ex.argtypes = [P, X] + [vp] * 10 + [sz, vp]
        lib.ssd_fwd_states_ex.restype = ctypes.c_int
        lib.ssd_fwd_states_ex.argtypes = [P, X] + [vp] * 8 + [sz, vp]
        lib.ssd_chunk_cumsum_ex.restype = ctypes.c_int
        lib.ssd_chunk_cumsum_ex.argtypes = [P, X] + [vp] * 5
        lib.ssd_step.restype = ctypes.c_int
        lib.ssd_step.argtypes = [P, X] + [vp] * 9
        CF = ctypes.POINTER(ssd_config)
        lib.ssd_default_config.restype = ctypes.c_int
        lib.ssd_default_config.argtypes = [P, CF]
        lib.ssd_fwd_config.restype = ctypes.c_int
        lib.ssd_fwd_config.argtypes = [P, CF, X] + [vp] * 10 + [sz, vp]
        i32, pi32, pf = ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.POINTER(ctypes.c_float)
        lib.ssd_tune.restype = ctypes.c_int
        lib.ssd_tune.argtypes = [P, X] + [vp] * 10 + [sz, vp, i32, CF, pf, i32, pi32, CF, pf]
        lib.ssd_fwd_config_workspace_size.restype = ctypes.c_int
        lib.ssd_fwd_config_workspace_size.argtypes = [P, CF, ctypes.POINTER(sz)]
        lib.ssd_fwd_status.restype = ctypes.c_int
        lib.ssd_fwd_status.argtypes = [vp, sz, vp, pi32]
        lib.ssd_fwd_noalloc.restype = ctypes.c_int
        lib.ssd_fwd_noalloc.argtypes = [P, X] + [vp] * 10
        lib.ssd_bwd_workspace_size.restype = ctypes.c_int
        lib.ssd_bwd_workspace_size.argtypes = [P, ctypes.POINTER(sz)]
        lib.ssd_bwd_workspace_min_size.restype = ctypes.c_int
        lib.ssd_bwd_workspace_min_size.argtypes = [P, ctypes.POINTER(sz)]
        lib.ssd_bwd.restype = ctypes.c_int
        lib.ssd_bwd.argtypes = [P, X] + [vp] * 18 + [sz, vp]
        _lib = lib
        return lib


def ssd_abi_version() -> int:
    return int(load_library().ssd_abi_version())


def ssd_status_string(status: int) -> str:
    return load_library().ssd_status_string(int(status)).decode()


def ssd_last_error_message() -> str:
    return load_library().ssd_last_error_message().decode()


def _check(status: int) -> None:
    if status != 0:
        msg = ssd_last_error_message()
        if status in _ARG_ERRORS:
            raise SsdArgumentError(status, msg)
        raise SsdError(status, msg)


def make_problem(batch, seqlen, nheads, headdim, dstate, ngroups, chunk_size, io_dtype) -> ssd_problem:
    return ssd_problem(int(batch), int(seqlen), int(nheads), int(headdim), int(dstate),
                       int(ngroups), int(chunk_size), int(io_dtype), 0)


def ssd_fwd_workspace_size(prob: ssd_problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_fwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return int(n.value)


def _io_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return SSD_BF16
    if t.dtype == torch.float32:
        return SSD_F32
    raise SsdArgumentError(4, "x, B and C must be bfloat16 or float32, got %s" % t.dtype)


def _dev(t: Optional[torch.Tensor], name: str, dtype=None) -> int:
    if t is None:
        return None
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise SsdArgumentError(1, "%s must be a GPU tensor" % name)
    if not t.is_contiguous():
        raise SsdArgumentError(2, "%s must be contiguous" % name)
    if dtype is not None and t.dtype != dtype:
        raise SsdArgumentError(4, "%s must be %s, got %s" % (name, dtype, t.dtype))
    return t.data_ptr()


def _stream(device: torch.device) -> int:
    return torch.cuda.current_stream(device).cuda_stream


def _problem_of(x, B, chunk_size) -> ssd_problem:
    if x.dim() != 4 or B.dim() != 4:
        raise SsdArgumentError(2, "x must be [batch, seqlen, nheads, headdim] and B/C "
                                  "[batch, seqlen, ngroups, dstate]")
    bsz, L, H, P = x.shape
    if B.shape[0] != bsz or B.shape[1] != L:
        raise SsdArgumentError(2, "B/C batch and seqlen must match x")
    return make_problem(bsz, L, H, P, B.shape[3], B.shape[2], chunk_size, _io_code(x))


def ssd_fwd_config_workspace_size(prob: ssd_problem, config=None) -> int:
    """Workspace bytes of ssd_fwd_config with ``config`` (None = the default)."""
    n = ctypes.c_size_t(0)
    cfg = _config_of(config)
    _check(load_library().ssd_fwd_config_workspace_size(
        ctypes.byref(prob), None if cfg is None else ctypes.byref(cfg), ctypes.byref(n)))
    return int(n.value)


def staged_workspace_size(prob: ssd_problem) -> int:
    """Workspace bytes of the staged kernels (ssd_fwd_states, ssd_compute_out)."""
    cfg = ssd_default_config(prob)
    cfg["fused"] = 0
    return ssd_fwd_config_workspace_size(prob, cfg)


def ssd_fwd_status(workspace: Optional[torch.Tensor] = None, device=None) -> bool:
    """True if the latest forward call on ``workspace`` gave up a bounded wait
    (its outputs are then undefined).  Synchronises the current stream.
    ``workspace=None`` asks about the scratch of ssd_fwd_noalloc."""
    t = ctypes.c_int32(0)
    if workspace is None:
        dev = torch.device(device) if device is not None else torch.device("cuda", torch.cuda.current_device())
        st = load_library().ssd_fwd_status(None, 0, _stream(dev), ctypes.byref(t))
    else:
        st = load_library().ssd_fwd_status(_dev(workspace, "workspace"),
                                           workspace.numel() * workspace.element_size(),
                                           _stream(workspace.device), ctypes.byref(t))
    _check(st)
    return bool(t.value)


def _workspace(prob, device, workspace, need=None):
    if need is None:
        need = ssd_fwd_workspace_size(prob)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=device)
    return workspace, workspace.numel() * workspace.element_size()


def _dt_transform(H, dt_bias, dt_softplus, dt_limit):
    """ssd_dt_transform for the given options (None when none is asked for)."""
    if dt_bias is None and not dt_softplus and dt_limit is None:
        return None, None
    if dt_bias is not None and tuple(dt_bias.shape) != (H,):
        raise SsdArgumentError(2, "dt_bias must be [nheads]")
    lo, hi = dt_limit if dt_limit is not None else (0.0, float("inf"))
    xf = ssd_dt_transform(_dev(dt_bias, "dt_bias", torch.float32), 1 if dt_softplus else 0, 0,
                          float(lo), float(hi))
    return xf, ctypes.byref(xf)


def ssd_fwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
            C: torch.Tensor, D: Optional[torch.Tensor] = None, chunk_size: int = 256,
            init_state: Optional[torch.Tensor] = None, *, want_final_state: bool = True,
            out: Optional[torch.Tensor] = None, final_out: Optional[torch.Tensor] = None,
            workspace: Optional[torch.Tensor] = None, dt_bias: Optional[torch.Tensor] = None,
            dt_softplus: bool = False, dt_limit: Optional[Tuple[float, float]] = None,
            config=None) -> Tuple[torch.Tensor, Optional[torch.Tensor]]:
    """Full forward pass on the current stream.  Returns (y, final_state).

    With dt_bias, dt_softplus or dt_limit given, ``dt`` is the raw step size and
    is prepared inside the first stage as clamp(softplus(dt + dt_bias)) (the C
    entry point ssd_fwd_ex); otherwise ``dt`` is used as given (ssd_fwd).
    ``config`` (a dict with cumsum_heads, state_heads, out_heads, or an
    ssd_config) selects the kernels' tile choices (ssd_fwd_config)."""
    lib = load_library()
    prob = _problem_of(x, B, chunk_size)
    if x.dtype != B.dtype or x.dtype != C.dtype:
        raise SsdArgumentError(4, "x, B and C must share one dtype")
    if tuple(dt.shape) != tuple(x.shape[:3]) or A.shape != (x.shape[2],):
        raise SsdArgumentError(2, "dt must be [batch, seqlen, nheads] and A [nheads]")
    if tuple(C.shape) != tuple(B.shape):
        raise SsdArgumentError(2, "C must have the shape of B")
    if D is not None and D.shape != (x.shape[2],):
        raise SsdArgumentError(2, "D must be [nheads]")
    state_shape = (x.shape[0], x.shape[2], x.shape[3], B.shape[3])
    if init_state is not None and tuple(init_state.shape) != state_shape:
        raise SsdArgumentError(2, "init_state must be [batch, nheads, headdim, dstate]")
    y = out if out is not None else torch.empty_like(x)
    if tuple(y.shape) != tuple(x.shape) or y.dtype != x.dtype:
        raise SsdArgumentError(2, "out must match x")
    fin = None
    if want_final_state:
        fin = final_out if final_out is not None else torch.empty(
            state_shape, dtype=torch.float32, device=x.device)
    ws, ws_bytes = _workspace(prob, x.device, workspace,
                              ssd_fwd_config_workspace_size(prob, config))
    args = (_dev(x, "x"), _dev(dt, "dt", torch.float32),
            _dev(A, "A", torch.float32), _dev(B, "B"), _dev(C, "C"),
            _dev(D, "D", torch.float32), _dev(init_state, "init_state", torch.float32),
            _dev(y, "y"), _dev(fin, "final_state", torch.float32), _dev(ws, "workspace"),
            ws_bytes, _stream(x.device))
    xf, xfp = _dt_transform(x.shape[2], dt_bias, dt_softplus, dt_limit)
    cfg = _config_of(config)
    if cfg is not None:
        st = lib.ssd_fwd_config(ctypes.byref(prob), ctypes.byref(cfg), xfp, *args)
    elif xf is None:
        st = lib.ssd_fwd(ctypes.byref(prob), *args)
    else:
        st = lib.ssd_fwd_ex(ctypes.byref(prob), xfp, *args)
    _check(st)
    return y, fin


def ssd_default_config(prob) -> dict:
    """The tile choices ssd_fwd makes for an ssd_problem (make_problem)."""
    c = ssd_config()
    _check(load_library().ssd_default_config(ctypes.byref(prob), ctypes.byref(c)))
    return c.as_dict()


def ssd_tune(x, dt, A, B, C, D=None, chunk_size=256, init_state=None, *, reps: int = 5,
             dt_bias=None, dt_softplus=False, dt_limit=None, workspace=None):
    """Time the forward pass with every valid tile choice (synchronises the
    current stream).  Returns (best config dict, best mean ms,
    [(config dict, mean ms), ...] in the order measured)."""
    lib = load_library()
    prob = _problem_of(x, B, chunk_size)
    state_shape = (x.shape[0], x.shape[2], x.shape[3], B.shape[3])
    y = torch.empty_like(x)
    fin = torch.empty(state_shape, dtype=torch.float32, device=x.device)
    ws, ws_bytes = _workspace(prob, x.device, workspace)
    xf, xfp = _dt_transform(x.shape[2], dt_bias, dt_softplus, dt_limit)
    cap = 32
    tried = (ssd_config * cap)()
    tried_ms = (ctypes.c_float * cap)()
    n = ctypes.c_int32(0)
    best = ssd_config()
    best_ms = ctypes.c_float(0.0)
    st = lib.ssd_tune(ctypes.byref(prob), xfp, _dev(x, "x"), _dev(dt, "dt", torch.float32),
                      _dev(A, "A", torch.float32), _dev(B, "B"), _dev(C, "C"),
                      _dev(D, "D", torch.float32), _dev(init_state, "init_state", torch.float32),
                      _dev(y, "y"), _dev(fin, "final_state", torch.float32), _dev(ws, "workspace"),
                      ws_bytes, _stream(x.device), int(reps), tried, tried_ms, cap,
                      ctypes.byref(n), ctypes.byref(best), ctypes.byref(best_ms))
    _check(st)
    rows = [(tried[i].as_dict(), float(tried_ms[i])) for i in range(min(n.value, cap))]
    return best.as_dict(), float(best_ms.value), rows


def ssd_fwd_ex(x, dt, A, B, C, D=None, chunk_size=256, init_state=None, *, dt_bias=None,
               dt_softplus=True, dt_limit=(0.0, float("inf")), **kw):
    """ssd_fwd from a raw step size: dt' = clamp(softplus(dt + dt_bias), *dt_limit)."""
    return ssd_fwd(x, dt, A, B, C, D, chunk_size, init_state, dt_bias=dt_bias,
                   dt_softplus=dt_softplus, dt_limit=dt_limit, **kw)


def ssd_fwd_noalloc(x, dt, A, B, C, D=None, chunk_size=256, init_state=None, *,
                    want_final_state: bool = True, out=None, final_out=None, dt_bias=None,
                    dt_softplus: bool = False, dt_limit=None):
    """ssd_fwd on the library's built-in scratch (no workspace is allocated or
    passed; for callers that cannot allocate).  Calls that overlap on one GPU
    share that scratch and race.  Returns (y, final_state)."""
    lib = load_library()
    prob = _problem_of(x, B, chunk_size)
    if x.dtype != B.dtype or x.dtype != C.dtype:
        raise SsdArgumentError(4, "x, B and C must share one dtype")
    state_shape = (x.shape[0], x.shape[2], x.shape[3], B.shape[3])
    y = out if out is not None else torch.empty_like(x)
    fin = None
    if want_final_state:
        fin = final_out if final_out is not None else torch.empty(
            state_shape, dtype=torch.float32, device=x.device)
    xf, xfp = _dt_transform(x.shape[2], dt_bias, dt_softplus, dt_limit)
    st = lib.ssd_fwd_noalloc(ctypes.byref(prob), xfp, _dev(x, "x"), _dev(dt, "dt", torch.float32),
                             _dev(A, "A", torch.float32), _dev(B, "B"), _dev(C, "C"),
                             _dev(D, "D", torch.float32),
                             _dev(init_state, "init_state", torch.float32), _dev(y, "y"),
                             _dev(fin, "final_state", torch.float32), _stream(x.device))
    _check(st)
    return y, fin


def ssd_fwd_states(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
                   chunk_size: int = 256, init_state: Optional[torch.Tensor] = None, *,
                   want_chunk_states: bool = True,
                   workspace: Optional[torch.Tensor] = None,
                   final_out: Optional[torch.Tensor] = None,
                   dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False,
                   dt_limit: Optional[Tuple[float, float]] = None):
    """Stages 1-2 only.  Returns (final_state fp32, chunk_states [B,H,T,P,N] or None).
    dt_bias / dt_softplus / dt_limit: raw step size, as in ssd_fwd (ssd_fwd_states_ex)."""
    lib = load_library()
    prob = _problem_of(x, B, chunk_size)
    if x.dtype != B.dtype:
        raise SsdArgumentError(4, "x and B must share one dtype")
    bsz, L, H, P = x.shape
    N = B.shape[3]
    T = -(-L // int(chunk_size)) if chunk_size > 0 else 0
    fin = final_out if final_out is not None else torch.empty((bsz, H, P, N), dtype=torch.float32,
                                                              device=x.device)
    cs = torch.empty((bsz, H, T, P, N), dtype=x.dtype, device=x.device) if want_chunk_states else None
    ws, ws_bytes = _workspace(prob, x.device, workspace, staged_workspace_size(prob))
    args = (_dev(x, "x"), _dev(dt, "dt", torch.float32),
            _dev(A, "A", torch.float32), _dev(B, "B"),
            _dev(init_state, "init_state", torch.float32),
            _dev(fin, "final_state", torch.float32), _dev(cs, "chunk_states"),
            _dev(ws, "workspace"), ws_bytes, _stream(x.device))
    xf, xfp = _dt_transform(H, dt_bias, dt_softplus, dt_limit)
    if xf is None:
        st = lib.ssd_fwd_states(ctypes.byref(prob), *args)
    else:
        st = lib.ssd_fwd_states_ex(ctypes.byref(prob), xfp, *args)
    _check(st)
    return fin, cs


def ssd_fwd_states_ex(x, dt, A, B, chunk_size=256, init_state=None, *, dt_bias=None,
                      dt_softplus=True, dt_limit=(0.0, float("inf")), **kw):
    """ssd_fwd_states from a raw step size (prepared as in ssd_fwd_ex)."""
    return ssd_fwd_states(x, dt, A, B, chunk_size, init_state, dt_bias=dt_bias,
                          dt_softplus=dt_softplus, dt_limit=dt_limit, **kw)


def ssd_compute_out(x: torch.Tensor, B: torch.Tensor, C: torch.Tensor,
                    D: Optional[torch.Tensor], chunk_size: int, workspace: torch.Tensor, *,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Stage 3 only, from a workspace filled by ssd_fwd_states(..., workspace=ws,
    want_chunk_states=False) on the same stream.  Returns y."""
    lib = load_library()
    prob = _problem_of(x, B, chunk_size)
    if x.dtype != B.dtype or x.dtype != C.dtype:
        raise SsdArgumentError(4, "x, B and C must share one dtype")
    y = out if out is not None else torch.empty_like(x)
    st = lib.ssd_compute_out(ctypes.byref(prob), _dev(x, "x"), _dev(B, "B"), _dev(C, "C"),
                             _dev(D, "D", torch.float32), _dev(y, "y"), _dev(workspace, "workspace"),
                             workspace.numel() * workspace.element_size(), _stream(x.device))
    _check(st)
    return y


def ssd_chunk_cumsum(dt: torch.Tensor, A: torch.Tensor, chunk_size: int = 256, *,
                     dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False,
                     dt_limit: Optional[Tuple[float, float]] = None):
    """Stage 1 only.  Returns (G, dt_t), both [batch, nheads, seqlen] fp32.
    With dt_bias, dt_softplus or dt_limit, dt is prepared first (ssd_chunk_cumsum_ex)
    and dt_t holds the prepared values."""
    lib = load_library()
    if dt.dim() != 3:
        raise SsdArgumentError(2, "dt must be [batch, seqlen, nheads]")
    bsz, L, H = dt.shape
    prob = make_problem(bsz, L, H, 16, 16, 1, chunk_size, SSD_F32)
    G = torch.empty((bsz, H, L), dtype=torch.float32, device=dt.device)
    dtt = torch.empty_like(G)
    args = (_dev(dt, "dt", torch.float32), _dev(A, "A", torch.float32), _dev(G, "G_out"),
            _dev(dtt, "dt_out"), _stream(dt.device))
    xf, xfp = _dt_transform(H, dt_bias, dt_softplus, dt_limit)
    if xf is None:
        st = lib.ssd_chunk_cumsum(ctypes.byref(prob), *args)
    else:
        st = lib.ssd_chunk_cumsum_ex(ctypes.byref(prob), xfp, *args)
    _check(st)
    return G, dtt


def ssd_chunk_cumsum_ex(dt, A, chunk_size=256, *, dt_bias=None, dt_softplus=True,
                        dt_limit=(0.0, float("inf"))):
    """ssd_chunk_cumsum from a raw step size (prepared as in ssd_fwd_ex)."""
    return ssd_chunk_cumsum(dt, A, chunk_size, dt_bias=dt_bias, dt_softplus=dt_softplus,
                            dt_limit=dt_limit)


def ssd_step(state: torch.Tensor, x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor,
             B: torch.Tensor, C: torch.Tensor, D: Optional[torch.Tensor] = None, *,
             dt_bias: Optional[torch.Tensor] = None, dt_softplus: bool = False,
             dt_limit: Optional[Tuple[float, float]] = None,
             out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Token-sequential mode: advance ``state`` [batch, nheads, headdim, dstate]
    (fp32, updated in place) through the seqlen tokens of x [batch, seqlen,
    nheads, headdim] one at a time.  Returns y (shape and dtype of x)."""
    lib = load_library()
    prob = _problem_of(x, B, 256)
    if x.dtype != B.dtype or x.dtype != C.dtype:
        raise SsdArgumentError(4, "x, B and C must share one dtype")
    if tuple(dt.shape) != tuple(x.shape[:3]) or A.shape != (x.shape[2],):
        raise SsdArgumentError(2, "dt must be [batch, seqlen, nheads] and A [nheads]")
    if tuple(C.shape) != tuple(B.shape):
        raise SsdArgumentError(2, "C must have the shape of B")
    if D is not None and D.shape != (x.shape[2],):
        raise SsdArgumentError(2, "D must be [nheads]")
    if tuple(state.shape) != (x.shape[0], x.shape[2], x.shape[3], B.shape[3]):
        raise SsdArgumentError(2, "state must be [batch, nheads, headdim, dstate]")
    y = out if out is not None else torch.empty_like(x)
    if tuple(y.shape) != tuple(x.shape) or y.dtype != x.dtype:
        raise SsdArgumentError(2, "out must match x")
    xf, xfp = _dt_transform(x.shape[2], dt_bias, dt_softplus, dt_limit)
    st = lib.ssd_step(ctypes.byref(prob), xfp, _dev(state, "state", torch.float32), _dev(x, "x"),
                      _dev(dt, "dt", torch.float32), _dev(A, "A", torch.float32), _dev(B, "B"),
                      _dev(C, "C"), _dev(D, "D", torch.float32), _dev(y, "y"),
                      _stream(x.device))
    _check(st)
    return y


def ssd_bwd_workspace_size(prob: ssd_problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_bwd_workspace_size(ctypes.byref(prob), ctypes.byref(n)))
    return int(n.value)


def ssd_bwd_workspace_min_size(prob: ssd_problem) -> int:
    n = ctypes.c_size_t(0)
    _check(load_library().ssd_bwd_workspace_min_size(ctypes.byref(prob), ctypes.byref(n)))
    return int(n.value)


def ssd_bwd(x: torch.Tensor, dt: torch.Tensor, A: torch.Tensor, B: torch.Tensor,
            C: torch.Tensor, D: Optional[torch.Tensor], chunk_size: int,
            init_state: Optional[torch.Tensor], dy: torch.Tensor,
            dfinal: Optional[torch.Tensor] = None, *, dt_bias: Optional[torch.Tensor] = None,
            dt_softplus: bool = False, dt_limit: Optional[Tuple[float, float]] = None,
            want_dD: bool = True, want_dinit: bool = True, want_ddt_bias: bool = False,
            workspace: Optional[torch.Tensor] = None) -> dict:
    """Backward pass on the current stream (C entry point ssd_bwd).

    Given dy = dLoss/dy and optionally dfinal = dLoss/d(final state), returns a
    dict with dx, ddt, dA, dB, dC and, when asked, dD, dinit and ddt_bias.  The
    dt options mean what they mean for ssd_fwd; ddt is then the gradient with
    respect to the raw ``dt`` argument."""
    lib = load_library()
    prob = _problem_of(x, B, chunk_size)
    if x.dtype != B.dtype or x.dtype != C.dtype or dy.dtype != x.dtype:
        raise SsdArgumentError(4, "x, B, C and dy must share one dtype")
    if tuple(dt.shape) != tuple(x.shape[:3]) or A.shape != (x.shape[2],):
        raise SsdArgumentError(2, "dt must be [batch, seqlen, nheads] and A [nheads]")
    if tuple(C.shape) != tuple(B.shape) or tuple(dy.shape) != tuple(x.shape):
        raise SsdArgumentError(2, "C must have the shape of B and dy that of x")
    if D is not None and D.shape != (x.shape[2],):
        raise SsdArgumentError(2, "D must be [nheads]")
    state_shape = (x.shape[0], x.shape[2], x.shape[3], B.shape[3])
    for name, t in (("init_state", init_state), ("dfinal", dfinal)):
        if t is not None and tuple(t.shape) != state_shape:
            raise SsdArgumentError(2, "%s must be [batch, nheads, headdim, dstate]" % name)
    H = x.shape[2]
    f32 = dict(dtype=torch.float32, device=x.device)
    out = {"dx": torch.empty_like(x), "ddt": torch.empty(tuple(dt.shape), **f32),
           "dA": torch.empty(H, **f32), "dB": torch.empty_like(B), "dC": torch.empty_like(C),
           "dD": torch.empty(H, **f32) if want_dD else None,
           "dinit": torch.empty(state_shape, **f32) if want_dinit else None,
           "ddt_bias": torch.empty(H, **f32) if want_ddt_bias else None}
    if workspace is None:
        need = ssd_bwd_workspace_size(prob)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=x.device)
    xf, xfp = _dt_transform(H, dt_bias, dt_softplus, dt_limit)
    st = lib.ssd_bwd(ctypes.byref(prob), xfp, _dev(x, "x"), _dev(dt, "dt", torch.float32),
                     _dev(A, "A", torch.float32), _dev(B, "B"), _dev(C, "C"),
                     _dev(D, "D", torch.float32), _dev(init_state, "init_state", torch.float32),
                     _dev(dy, "dy"), _dev(dfinal, "dfinal", torch.float32),
                     _dev(out["dx"], "dx"), _dev(out["ddt"], "ddt"), _dev(out["dA"], "dA"),
                     _dev(out["dB"], "dB"), _dev(out["dC"], "dC"), _dev(out["dD"], "dD"),
                     _dev(out["dinit"], "dinit"), _dev(out["ddt_bias"], "ddt_bias"),
                     _dev(workspace, "workspace"),
                     workspace.numel() * workspace.element_size(), _stream(x.device))
    _check(st)
    return out
