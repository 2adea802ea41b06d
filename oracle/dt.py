"""Step-size preparation of a Mamba-2 layer, fp64 (numpy).

TEST INFRASTRUCTURE (see the package docstring).

The pages feed the scan an already positive step size dt and say nothing of
where it comes from.  A Mamba-2 layer makes it from a projection: it adds a
per-head bias, applies softplus(v) = log(1 + e^v) and optionally clamps the
result to [dt_min, dt_max].  This is that definition written out:

    v   = dt_raw[b, t, h] + dt_bias[h]          (bias optional)
    v   = log(1 + exp(v))                       (softplus optional)
    dt' = min(max(v, dt_min), dt_max)

log(1 + e^v) is evaluated as max(v, 0) + log1p(exp(-|v|)), the same value
written so that exp never overflows.  The scan then consumes dt' exactly as
it consumes a given dt.

Pinned (tests/test_oracle.py) by closed forms: softplus(0) = ln 2,
softplus(v) - softplus(-v) = v, softplus(log(e^y - 1)) = y, softplus(v) -> v
for large v and -> e^v for very negative v, and the clamp's fixed points.
"""
from __future__ import annotations

import numpy as np


def _f64(t):
    if t is None:
        return None
    if hasattr(t, "detach"):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def softplus(v):
    """log(1 + e^v) in fp64, elementwise."""
    v = np.asarray(v, dtype=np.float64)
    return np.maximum(v, 0.0) + np.log1p(np.exp(-np.abs(v)))


def dt_transform(dt_raw, dt_bias=None, use_softplus=True, dt_min=0.0, dt_max=np.inf):
    """Prepared step size dt' [batch, seqlen, nheads] (fp64) from the raw one."""
    v = _f64(dt_raw)
    if dt_bias is not None:
        v = v + _f64(dt_bias)[None, None, :]
    if use_softplus:
        v = softplus(v)
    return np.minimum(np.maximum(v, dt_min), dt_max)
