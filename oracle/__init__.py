"""CPU oracle for the Mamba-2 chunked SSD forward pass.

TEST INFRASTRUCTURE.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  It shares no code
with the HIP library and never imports it.

Contents
  recurrence(...)     fp64 token-by-token scan, in C (``ssd_oracle.c``).
  chunk_cumsum(...)   fp64 within-chunk running sum of a_t = dt_t A, base-2 log.
  dense_matrix(...)   fp64 materialised SSD matrix form (numpy, tiny inputs).
  chunked(...)        fp64 chunked log-space form (numpy, small inputs).
  dt_transform(...)   fp64 step-size preparation (bias, softplus, clamp) of a
                      Mamba-2 layer, for the raw-dt entry points.
  recurrence_bwd(...) fp64 gradients of the scan (reverse-mode, token by token).
  dt_transform_bwd(...) fp64 gradients through the step-size preparation.

The token-sequential (decode) mode needs no function of its own: it is the
recurrence itself, started from a given state (``recurrence`` with
``init_state``).

All functions take CPU tensors or numpy arrays in the layouts documented in
``ssd_synth`` and return numpy float64 arrays.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

from .dense import dense_matrix, linear_attention
from .chunked import chunked
from .dt import dt_transform, softplus
from .bwd import dt_transform_bwd, recurrence_bwd

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "ssd_oracle.c")
_LIB = os.path.join(_HERE, "libssd_oracle.so")
_lock = threading.Lock()
_lib = None

__all__ = ["build", "load_library", "recurrence", "recurrence_heads", "recurrence_head_ranges",
           "chunk_cumsum", "dense_matrix",
           "linear_attention", "chunked", "as_f32", "dt_transform", "softplus",
           "recurrence_bwd", "dt_transform_bwd"]


def build(force: bool = True) -> str:
    """Compile the C oracle with gcc (-O2, OpenMP, no fast-math, no FMA)."""
    if force or not os.path.exists(_LIB):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = ["gcc", "-O2", "-fPIC", "-shared", "-fopenmp", "-ffp-contract=off",
               "-std=c99", "-Wall", "-Wextra", _SRC, "-o", tmp, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


def load_library(path):
    """Open a compiled oracle library (the default one, or a test's variant)."""
    lib = ctypes.CDLL(path)
    i64, ptr = ctypes.c_int64, ctypes.c_void_p
    lib.ssd_oracle_fwd.restype = ctypes.c_int
    lib.ssd_oracle_fwd.argtypes = [i64] * 6 + [ptr] * 9 + [i64, ptr, ctypes.c_int]
    lib.ssd_oracle_chunk_cumsum.restype = ctypes.c_int
    lib.ssd_oracle_chunk_cumsum.argtypes = [i64] * 4 + [ptr] * 3
    return lib


def _load():
    """The default build, or the one SSD_ORACLE_LIBRARY names (the host
    sanitizer tests load an instrumented build that way)."""
    global _lib
    with _lock:
        if _lib is None:
            other = os.environ.get("SSD_ORACLE_LIBRARY")
            if other:
                _lib = load_library(other)
            else:
                if not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
                    build(force=True)
                _lib = load_library(_LIB)
    return _lib


def as_f32(t) -> np.ndarray:
    """Exact fp32 numpy copy of a CPU tensor / array (bf16 widens exactly)."""
    if t is None:
        return None
    if hasattr(t, "detach"):
        t = t.detach().cpu()
        if t.dtype != __import__("torch").float32:
            t = t.float()
        return np.ascontiguousarray(t.numpy())
    return np.ascontiguousarray(np.asarray(t, dtype=np.float32))


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def recurrence(x, dt, A, B, C, D=None, init_state=None, chunk_size=0,
               want_chunk_states=False, nthreads=None, lib=None):
    """fp64 token recurrence.  Returns (y, final_state, chunk_states or None).

    y [batch, seqlen, nheads, headdim], final_state [batch, nheads, headdim, dstate],
    chunk_states [batch, nheads, nchunks, headdim, dstate] = state at the start of
    each chunk of ``chunk_size`` tokens.  ``lib`` selects another build of the
    C source (tests use it to check that the pins reject altered copies).
    """
    lib = lib or _load()
    x, dt, A, B, C = (as_f32(v) for v in (x, dt, A, B, C))
    D = as_f32(D)
    init_state = as_f32(init_state)
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    assert dt.shape == (bsz, L, H) and A.shape == (H,)
    assert B.shape == (bsz, L, G, N) and C.shape == B.shape
    y = np.empty((bsz, L, H, P), dtype=np.float64)
    fin = np.empty((bsz, H, P, N), dtype=np.float64)
    cs = None
    if want_chunk_states:
        assert chunk_size > 0
        T = -(-L // chunk_size)
        cs = np.empty((bsz, H, T, P, N), dtype=np.float64)
    if nthreads is None:
        nthreads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    rc = lib.ssd_oracle_fwd(bsz, L, H, P, N, G, _p(x), _p(dt), _p(A), _p(B), _p(C), _p(D),
                            _p(init_state), _p(y), _p(fin), int(chunk_size), _p(cs),
                            int(nthreads))
    if rc != 0:
        raise ValueError("ssd_oracle_fwd rejected its arguments (rc=%d)" % rc)
    return y, fin, cs


def recurrence_heads(inputs, heads, nthreads=None):
    """Run the recurrence for a few (batch, head) pairs only.

    ``inputs`` is the dict made by ``ssd_synth.make_inputs``; ``heads`` is a list
    of (b, h).  Returns {(b, h): (y [L, P], final [P, N])}.  Used to check
    outputs of problems too large for the full oracle.
    """
    x, dt, A, B, C, D, init = (inputs[k] for k in ("x", "dt", "A", "B", "C", "D", "init_state"))
    H, G = x.shape[2], B.shape[2]
    hpg = H // G
    out = {}
    for (b, h) in heads:
        g = h // hpg
        sl = lambda t, idx: t[b:b + 1, :, idx:idx + 1]
        init_bh = None if init is None else init[b:b + 1, h:h + 1]
        Dh = None if D is None else D[h:h + 1]
        y, fin, _ = recurrence(sl(x, h), sl(dt, h), A[h:h + 1], sl(B, g), sl(C, g), Dh,
                               init_bh, nthreads=nthreads)
        out[(b, h)] = (y[0, :, 0], fin[0, 0])
    return out


def recurrence_head_ranges(inputs, heads_per_range, nthreads=None):
    """The recurrence over every head, a range of whole groups at a time.

    Yields (h0, h1, y [batch, seqlen, h1-h0, headdim], final [batch, h1-h0,
    headdim, dstate]) for consecutive head ranges covering all heads, each
    range holding whole groups (heads_per_range is rounded up to a multiple
    of the heads per group).  Every (batch, head) is computed, so a caller
    can compare a whole output tensor while holding only one range of the
    fp64 result at a time.  The arithmetic is ``recurrence`` itself: a range
    of whole groups is the same problem restricted to those heads and
    groups.
    """
    x, dt, A, B, C, D, init = (inputs[k] for k in ("x", "dt", "A", "B", "C", "D", "init_state"))
    H, G = x.shape[2], B.shape[2]
    hpg = H // G
    step = max(hpg, -(-int(heads_per_range) // hpg) * hpg)
    for h0 in range(0, H, step):
        h1 = min(H, h0 + step)
        g0, g1 = h0 // hpg, h1 // hpg
        y, fin, _ = recurrence(x[:, :, h0:h1], dt[:, :, h0:h1], A[h0:h1], B[:, :, g0:g1],
                               C[:, :, g0:g1], None if D is None else D[h0:h1],
                               None if init is None else init[:, h0:h1], nthreads=nthreads)
        yield h0, h1, y, fin


def chunk_cumsum(dt, A, chunk_size):
    """G[b,h,t] = (1/ln 2) * sum of dt[b,k,h]*A[h] over k from the chunk start to t."""
    lib = _load()
    dt, A = as_f32(dt), as_f32(A)
    bsz, L, H = dt.shape
    G = np.empty((bsz, H, L), dtype=np.float64)
    rc = lib.ssd_oracle_chunk_cumsum(bsz, L, H, int(chunk_size), _p(dt), _p(A), _p(G))
    if rc != 0:
        raise ValueError("ssd_oracle_chunk_cumsum rejected its arguments")
    return G
