"""Gradients of the SSD scan, fp64 (numpy): the backward pass.

TEST INFRASTRUCTURE (see the package docstring).

The pages present the forward pass only and name the backward pass as the
piece still missing for end-to-end training (devin.kr "NVIDIA CUDA Tile로
Mamba-2 순방향 전달 커널 가속화", closing remarks on the measured gains;
brifing.si "Accelerating Mamba-2 ...", limitations).  There is therefore no
algorithm on the pages to follow; the gradient has a plain definition, and
this module is that definition written out: reverse-mode differentiation of
the token recurrence, one token at a time.

For one (b, h) with group g, token t = 1..L (a_t = exp(dt_t A_h)):

    s_t = a_t s_{t-1} + dt_t x_t B_t^T            (P x N)
    y_t = s_t C_t + D_h x_t

and a scalar loss whose gradients with respect to y_t and s_L are dy_t and
dfinal.  Walking t = L .. 1 with lam the gradient with respect to s_t
(lam = dfinal before token L):

    lam    += dy_t C_t^T                           (y_t reads s_t)
    dC_t   += s_t^T dy_t                           (summed over heads of group g)
    dx_t    = D_h dy_t + dt_t lam B_t
    dB_t   += dt_t lam^T x_t                       (summed over heads of group g)
    dl      = a_t <lam, s_{t-1}>                   (gradient of log a_t)
    ddt_t   = x_t^T lam B_t + A_h dl
    dA_h   += dt_t dl
    dD_h   += <dy_t, x_t>
    lam     = a_t lam                              (now the gradient of s_{t-1})

and the gradient of the initial state is the final lam.  The states s_t are
recomputed from checkpoints every ``seg`` tokens (checkpointing changes only
memory use, not a value).

Pinned (tests/test_oracle_bwd.py) by central finite differences of the C
forward oracle on small inputs (every element of every input), by the
first-degree homogeneity of the loss in (x, init_state), in B, in C and in D,
and by finite differences of the step-size preparation.
"""
from __future__ import annotations

import numpy as np

from .dt import softplus


def _f64(t):
    if t is None:
        return None
    if hasattr(t, "detach"):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def head_bwd(x, dt, a_coef, Bg, Cg, Dh, s0, dy, dS, seg=64):
    """Gradients for one (batch, head) sequence.

    x, dy [L, P]; dt [L]; a_coef = A_h; Bg, Cg [L, N] (the head's group);
    Dh scalar; s0, dS [P, N] (initial state, gradient of the final state).
    Returns dx [L, P], ddt [L], dA (scalar), dB [L, N], dC [L, N],
    dD (scalar), ds0 [P, N].
    """
    L, P = x.shape
    N = Bg.shape[1]
    # forward, keeping the state at the start of every segment of `seg` tokens
    marks = {}
    s = s0.copy()
    for t in range(L):
        if t % seg == 0:
            marks[t] = s.copy()
        s = np.exp(dt[t] * a_coef) * s + dt[t] * np.outer(x[t], Bg[t])

    dx = np.zeros((L, P))
    ddt = np.zeros(L)
    dB = np.zeros((L, N))
    dC = np.zeros((L, N))
    dA = 0.0
    dD = 0.0
    lam = dS.copy()
    for start in range(((L - 1) // seg) * seg, -1, -seg):
        stop = min(start + seg, L)
        # states s_{t-1} (before token t) for the tokens of this segment
        before = []
        s = marks[start].copy()
        for t in range(start, stop):
            before.append(s)
            s = np.exp(dt[t] * a_coef) * s + dt[t] * np.outer(x[t], Bg[t])
        after = s
        for t in range(stop - 1, start - 1, -1):
            s_prev = before[t - start]
            s_t = after
            alpha = np.exp(dt[t] * a_coef)
            lam = lam + np.outer(dy[t], Cg[t])
            dC[t] = s_t.T @ dy[t]
            lam_b = lam @ Bg[t]                       # lam B_t, [P]
            dx[t] = Dh * dy[t] + dt[t] * lam_b
            dB[t] = dt[t] * (lam.T @ x[t])
            dl = alpha * np.sum(lam * s_prev)
            ddt[t] = x[t] @ lam_b + a_coef * dl
            dA += dt[t] * dl
            dD += dy[t] @ x[t]
            lam = alpha * lam
            after = s_prev
    return dx, ddt, dA, dB, dC, dD, lam


def recurrence_bwd(x, dt, A, B, C, D=None, init_state=None, dy=None, dfinal=None, seg=64,
                   heads=None):
    """Gradients of <dy, y> + <dfinal, final_state> for the whole problem.

    Layouts as for ``recurrence``; dy [batch, seqlen, nheads, headdim], dfinal
    [batch, nheads, headdim, dstate] or None (zero).  Returns a dict with dx,
    ddt, dA, dB, dC, dD and dinit (dD and dinit also when D or init_state is
    None: the gradient with respect to a zero value).  ``heads`` = a list of
    (b, h) computes only those heads; then dA and dD hold only their
    contributions and dB/dC only the sum over the listed heads.
    """
    x, dt, A, B, C, dy = (_f64(v) for v in (x, dt, A, B, C, dy))
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    D = np.zeros(H) if D is None else _f64(D)
    init = np.zeros((bsz, H, P, N)) if init_state is None else _f64(init_state)
    dS = np.zeros((bsz, H, P, N)) if dfinal is None else _f64(dfinal)
    out = {
        "dx": np.zeros((bsz, L, H, P)), "ddt": np.zeros((bsz, L, H)), "dA": np.zeros(H),
        "dB": np.zeros((bsz, L, G, N)), "dC": np.zeros((bsz, L, G, N)), "dD": np.zeros(H),
        "dinit": np.zeros((bsz, H, P, N)),
    }
    todo = heads if heads is not None else [(b, h) for b in range(bsz) for h in range(H)]
    for (b, h) in todo:
        g = h // hpg
        dx, ddt, dA, dB, dC, dD, ds0 = head_bwd(x[b, :, h], dt[b, :, h], A[h], B[b, :, g],
                                                C[b, :, g], D[h], init[b, h], dy[b, :, h],
                                                dS[b, h], seg=seg)
        out["dx"][b, :, h] = dx
        out["ddt"][b, :, h] = ddt
        out["dA"][h] += dA
        out["dB"][b, :, g] += dB
        out["dC"][b, :, g] += dC
        out["dD"][h] += dD
        out["dinit"][b, h] = ds0
    return out


def dt_transform_bwd(dt_raw, ddt, dt_bias=None, use_softplus=True, dt_min=0.0, dt_max=np.inf):
    """Gradients through the step-size preparation (chain rule of dt_transform).

    Returns (d dt_raw [batch, seqlen, nheads], d dt_bias [nheads]).  The
    clamp passes the gradient where dt_min <= value <= dt_max (ends included)
    and stops it elsewhere; softplus' derivative is the logistic function
    e^v / (1 + e^v).
    """
    v = _f64(dt_raw)
    if dt_bias is not None:
        v = v + _f64(dt_bias)[None, None, :]
    g = _f64(ddt)
    if use_softplus:
        w = softplus(v)
        g = g * np.exp(v - w)               # e^v / (1 + e^v), without overflow
    else:
        w = v
    g = g * ((w >= dt_min) & (w <= dt_max))
    return g, g.sum(axis=(0, 1))
