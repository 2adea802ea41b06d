"""Materialised SSD matrix form of the scan (fp64, numpy, tiny inputs only).

TEST INFRASTRUCTURE (see the package docstring).

Unrolling the recurrence s_t = exp(a_t) s_{t-1} + dt_t x_t b_t^T,
y_t = s_t c_t + D x_t gives, for every (b, h), an L x L lower-triangular
matrix acting on the token axis:

    M[t, u] = (c_t . b_u) * dt_u * exp(a_{u+1} + ... + a_t)      for u <= t
    y_t     = sum_u M[t, u] x_u + D x_t + exp(a_0 + ... + a_t) * (s_init c_t)
    s_final = exp(a_0 + ... + a_{L-1}) s_init
              + sum_u exp(a_{u+1} + ... + a_{L-1}) dt_u x_u b_u^T

This is the whole interaction matrix that a fused kernel avoids writing to
HBM (devin.kr "NVIDIA CUDA Tile로 Mamba-2 순방향 전달 커널 가속화", section
"세 가지 핵심 커널 구현", compute_out paragraph: a naive implementation
materialises it in global memory).  Here it is materialised on purpose as an
independent check of the token recurrence.
"""
from __future__ import annotations

import numpy as np


def _f64(t):
    if t is None:
        return None
    if hasattr(t, "detach"):
        return t.detach().cpu().double().numpy()
    return np.asarray(t, dtype=np.float64)


def dense_matrix(x, dt, A, B, C, D=None, init_state=None):
    """y and final state through the explicit L x L matrix (fp64)."""
    x, dt, A, B, C, D, s0 = (_f64(v) for v in (x, dt, A, B, C, D, init_state))
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros((bsz, L, H, P))
    fin = np.zeros((bsz, H, P, N))
    for b in range(bsz):
        for h in range(H):
            g = h // hpg
            a = dt[b, :, h] * A[h]                      # a_t
            S = np.concatenate([[0.0], np.cumsum(a)])   # S[t+1] = a_0 + ... + a_t
            # seg[t, u] = a_{u+1} + ... + a_t = S[t+1] - S[u+1]
            seg = S[1:, None] - S[None, 1:]
            causal = np.tril(np.ones((L, L), dtype=bool))
            decay = np.where(causal, np.exp(np.where(causal, seg, 0.0)), 0.0)
            CB = C[b, :, g, :] @ B[b, :, g, :].T          # (c_t . b_u)
            M = CB * decay * dt[b, None, :, h]
            yb = M @ x[b, :, h, :]
            if D is not None:
                yb += D[h] * x[b, :, h, :]
            if s0 is not None:
                yb += np.exp(S[1:])[:, None] * (C[b, :, g, :] @ s0[b, h].T)
                fin[b, h] = np.exp(S[L]) * s0[b, h]
            y[b, :, h, :] = yb
            w = np.exp(S[L] - S[1:]) * dt[b, :, h]        # exp(a_{u+1}+...+a_{L-1}) dt_u
            fin[b, h] += (x[b, :, h, :] * w[:, None]).T @ B[b, :, g, :]
    return y, fin


def linear_attention(x, dt, B, C, D=None, init_state=None):
    """The scan with zero decay (A = 0): causal linear attention, textbook form.

    y = tril(C B^T) (dt * X) + D X + C s_init^T,  s_final = s_init + X^T diag(dt) B,
    with C acting as queries, B as keys and dt-weighted X as values.
    """
    x, dt, B, C, D, s0 = (_f64(v) for v in (x, dt, B, C, D, init_state))
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    y = np.zeros((bsz, L, H, P))
    fin = np.zeros((bsz, H, P, N))
    for b in range(bsz):
        for h in range(H):
            g = h // hpg
            scores = np.tril(C[b, :, g, :] @ B[b, :, g, :].T)
            v = dt[b, :, h, None] * x[b, :, h, :]
            y[b, :, h, :] = scores @ v
            if D is not None:
                y[b, :, h, :] += D[h] * x[b, :, h, :]
            fin[b, h] = v.T @ B[b, :, g, :]
            if s0 is not None:
                y[b, :, h, :] += C[b, :, g, :] @ s0[b, h].T
                fin[b, h] += s0[b, h]
    return y, fin
