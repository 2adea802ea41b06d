"""Seeded synthetic inputs for the Mamba-2 chunked SSD forward pass.

This module is the only code shared by the HIP path's callers (bench, tests)
and the CPU oracle.  It draws input tensors and nothing else: it holds none of
the scan's arithmetic.  ``dt`` is produced the way a Mamba-2 layer produces it
(softplus of a biased pre-activation), because the scan consumes an already
positive step size; that transform is input preparation, not part of the scan.

Shapes and layouts (all contiguous, row-major):
    x   [batch, seqlen, nheads, headdim]   io dtype (bf16 or fp32)
    dt  [batch, seqlen, nheads]            fp32, > 0
    A   [nheads]                           fp32, < 0
    B   [batch, seqlen, ngroups, dstate]   io dtype
    C   [batch, seqlen, ngroups, dstate]   io dtype
    D   [nheads]                           fp32
    init_state [batch, nheads, headdim, dstate] fp32 or None
    dt_raw  [batch, seqlen, nheads]        fp32, the pre-activation 0.5 * N(0, 1)
    dt_bias [nheads]                       fp32
(dt is softplus(dt_raw + dt_bias); dt_raw and dt_bias are returned as well, for
the entry points that prepare a raw step size themselves.)

Draw order for one problem (CPU ``torch.Generator`` seeded once):
    1. dt_bias[H] = inv_softplus(exp(U(log 1e-3, log 1e-1)))
    2. A[H]       = -exp(U(a_lo, a_hi))     (default U(0, log 16))
    3. D[H]       ~ N(0, 1)
    4. x          ~ N(0, 1)
    5. dt         = softplus(0.5 * N(0, 1) + dt_bias)
    6. B          ~ N(0, 1) / sqrt(N)
    7. C          ~ N(0, 1) / sqrt(N)
    8. init_state ~ 0.1 * N(0, 1)           (only when requested)
Values are drawn in fp32; x, B and C are then rounded to the io dtype (bf16
rounding is round-to-nearest-even, done by ``Tensor.to``).
"""
from __future__ import annotations

import dataclasses
import hashlib
import math
from typing import Dict, Optional

import torch

__all__ = ["Problem", "CONFIGS", "make_inputs", "make_grads", "tensor_digest"]


@dataclasses.dataclass(frozen=True)
class Problem:
    """Shape, io dtype and input distribution of one SSD forward problem."""

    batch: int
    seqlen: int
    nheads: int
    headdim: int          # P
    dstate: int           # N
    ngroups: int          # G
    chunk_size: int       # Q
    io_dtype: str = "bf16"            # "bf16" or "fp32": dtype of x, B, C, y
    a_log_range: tuple = (0.0, math.log(16.0))   # A = -exp(U(lo, hi))
    init_std: Optional[float] = None             # None -> zero initial state
    name: str = ""

    @property
    def torch_io_dtype(self) -> torch.dtype:
        return {"bf16": torch.bfloat16, "fp32": torch.float32}[self.io_dtype]

    @property
    def nchunks(self) -> int:
        return -(-self.seqlen // self.chunk_size)

    def replace(self, **kw) -> "Problem":
        return dataclasses.replace(self, **kw)


# The five workloads: a tiny fp32 case and four Mamba-2 layer shapes.
CONFIGS: Dict[str, Problem] = {
    "tiny_fp32": Problem(1, 256, 2, 16, 16, 1, 64, io_dtype="fp32", name="tiny_fp32"),
    "mamba2_780m": Problem(4, 2048, 48, 64, 128, 1, 256, name="mamba2_780m"),
    "mamba2_2p7b": Problem(2, 8192, 80, 64, 128, 1, 256, init_std=0.1, name="mamba2_2p7b"),
    "long_prefill": Problem(1, 131072, 80, 64, 128, 1, 256, name="long_prefill"),
    "large_state": Problem(8, 4096, 64, 64, 256, 8, 128,
                           a_log_range=(math.log(0.5), math.log(32.0)), name="large_state"),
}
CONFIG_ORDER = ["tiny_fp32", "mamba2_780m", "mamba2_2p7b", "long_prefill", "large_state"]


def _uniform(g: torch.Generator, shape, lo: float, hi: float) -> torch.Tensor:
    return torch.rand(shape, generator=g, dtype=torch.float32) * (hi - lo) + lo


def make_inputs(prob: Problem, seed: int) -> Dict[str, Optional[torch.Tensor]]:
    """Draw one problem's inputs on the CPU, in the documented order.

    Returns a dict with keys x, dt, A, B, C, D, init_state (CPU tensors; x, B, C
    in the io dtype, everything else fp32; init_state None when the problem has
    a zero initial state).
    """
    Bsz, L, H, P, N, G = (prob.batch, prob.seqlen, prob.nheads, prob.headdim,
                          prob.dstate, prob.ngroups)
    if H % G != 0:
        raise ValueError("nheads must be a multiple of ngroups")
    g = torch.Generator().manual_seed(int(seed))
    # 1. dt bias: inverse softplus of a log-uniform target in [1e-3, 1e-1]
    target = torch.exp(_uniform(g, (H,), math.log(1e-3), math.log(1e-1)))
    dt_bias = torch.log(torch.expm1(target))
    # 2. A = -exp(U(lo, hi)) per head
    lo, hi = prob.a_log_range
    A = -torch.exp(_uniform(g, (H,), lo, hi))
    # 3. D ~ N(0, 1) per head
    D = torch.randn((H,), generator=g, dtype=torch.float32)
    # 4. x ~ N(0, 1)
    x = torch.randn((Bsz, L, H, P), generator=g, dtype=torch.float32)
    # 5. dt = softplus(0.5 * N(0,1) + dt_bias)
    dt_raw = 0.5 * torch.randn((Bsz, L, H), generator=g, dtype=torch.float32)
    dt = torch.nn.functional.softplus(dt_raw + dt_bias)
    # 6, 7. B, C ~ N(0, 1) / sqrt(N)
    scale = 1.0 / math.sqrt(N)
    Bm = torch.randn((Bsz, L, G, N), generator=g, dtype=torch.float32) * scale
    Cm = torch.randn((Bsz, L, G, N), generator=g, dtype=torch.float32) * scale
    # 8. optional initial state
    init = None
    if prob.init_std is not None:
        init = prob.init_std * torch.randn((Bsz, H, P, N), generator=g, dtype=torch.float32)
    io = prob.torch_io_dtype
    return {
        "x": x.to(io).contiguous(),
        "dt": dt.contiguous(),
        "A": A.contiguous(),
        "B": Bm.to(io).contiguous(),
        "C": Cm.to(io).contiguous(),
        "D": D.contiguous(),
        "init_state": init,
        "dt_raw": dt_raw.contiguous(),
        "dt_bias": dt_bias.contiguous(),
    }


def make_grads(prob: Problem, seed: int) -> Dict[str, torch.Tensor]:
    """Upstream gradients for the backward pass, drawn on the CPU from their own
    generator (seeded with seed + 7919, so the forward inputs of the same seed
    are unchanged): dy ~ N(0, 1) [batch, seqlen, nheads, headdim] in the io
    dtype, then dfinal ~ N(0, 1) [batch, nheads, headdim, dstate] fp32."""
    g = torch.Generator().manual_seed(int(seed) + 7919)
    Bsz, L, H, P, N = prob.batch, prob.seqlen, prob.nheads, prob.headdim, prob.dstate
    dy = torch.randn((Bsz, L, H, P), generator=g, dtype=torch.float32)
    dfinal = torch.randn((Bsz, H, P, N), generator=g, dtype=torch.float32)
    return {"dy": dy.to(prob.torch_io_dtype).contiguous(), "dfinal": dfinal.contiguous()}


def tensor_digest(t: Optional[torch.Tensor]) -> Optional[str]:
    """SHA-256 of a CPU tensor's bytes (None for None)."""
    if t is None:
        return None
    t = t.contiguous()
    if t.dtype == torch.bfloat16:
        t = t.view(torch.int16)
    return hashlib.sha256(t.numpy().tobytes()).hexdigest()
