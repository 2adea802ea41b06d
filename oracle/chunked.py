"""Chunked, base-2 log-space form of the scan (fp64, numpy, small inputs).

TEST INFRASTRUCTURE (see the package docstring).

This restates, in plain fp64 numpy, the three stages the pages describe for the
fast method, so that the token recurrence can be checked against it at many
chunk sizes (the result must not depend on the chunk size):

1. chunk cumsum -- G_i = log2(e) * (a_{cQ} + ... + a_{cQ+i}), a running sum of
   a_t = dt_t A inside each chunk, restarting at every chunk, kept in base-2 log
   space so that later stages use exp2 (devin.kr "NVIDIA CUDA Tile로 Mamba-2
   순방향 전달 커널 가속화", section "세 가지 핵심 커널 구현", chunk_cumsum;
   brifing.si "Accelerating Mamba-2 with High-Performance Forward Pass Kernels in
   NVIDIA CUDA Tile", section 7).
2. chunk states -- the jump formula: a chunk's contribution to the state after
   it is one matrix product over the chunk's stacked x and B rows, each row
   pre-multiplied by its decay to the chunk end, exp2(G_last - G_j) dt_j
   (brifing.si, sections 4 and 5).  States pass between chunks sequentially:
   H_{c+1} = exp2(G_last) H_c + S_c (devin.kr, same section, fwd_pass_state;
   brifing.si, section 8).
3. chunk output -- for token i of a chunk: the causal-masked, decayed
   interaction sum_{j<=i} (C_i . B_j) exp2(G_i - G_j) dt_j x_j, plus the carried
   state term exp2(G_i) H_c C_i, plus D x_i (devin.kr, same section,
   compute_out; brifing.si, sections 9 and 11).  The mask is applied to the
   exponent before exponentiating, so no positive exponent is ever evaluated.

A partial last chunk (seqlen not a multiple of the chunk size) is handled by
using only its valid tokens; its G_last is the running sum at its last token.
"""
from __future__ import annotations

import math

import numpy as np

from .dense import _f64

LOG2E = 1.0 / math.log(2.0)


def chunked(x, dt, A, B, C, D=None, init_state=None, chunk_size=64, want_chunk_states=False):
    """Chunked fp64 evaluation.  Returns (y, final_state, chunk_states or None)."""
    x, dt, A, B, C, D, s0 = (_f64(v) for v in (x, dt, A, B, C, D, init_state))
    bsz, L, H, P = x.shape
    G, N = B.shape[2], B.shape[3]
    hpg = H // G
    Q = int(chunk_size)
    T = -(-L // Q)
    y = np.zeros((bsz, L, H, P))
    fin = np.zeros((bsz, H, P, N))
    states = np.zeros((bsz, H, T, P, N)) if want_chunk_states else None
    for b in range(bsz):
        for h in range(H):
            g = h // hpg
            state = np.zeros((P, N)) if s0 is None else s0[b, h].copy()
            for c in range(T):
                lo, hi = c * Q, min(L, (c + 1) * Q)
                a = dt[b, lo:hi, h] * A[h]
                Gc = LOG2E * np.cumsum(a)                 # stage 1
                Xc, Bc, Cc = x[b, lo:hi, h, :], B[b, lo:hi, g, :], C[b, lo:hi, g, :]
                dtc = dt[b, lo:hi, h]
                if states is not None:
                    states[b, h, c] = state
                # stage 3 (uses the state at the chunk start)
                q = hi - lo
                ii, jj = np.meshgrid(np.arange(q), np.arange(q), indexing="ij")
                expo = np.where(jj <= ii, Gc[:, None] - Gc[None, :], -np.inf)
                Lmat = np.exp2(expo) * dtc[None, :]
                Yc = ((Cc @ Bc.T) * Lmat) @ Xc
                Yc += np.exp2(Gc)[:, None] * (Cc @ state.T)
                if D is not None:
                    Yc += D[h] * Xc
                y[b, lo:hi, h, :] = Yc
                # stage 2 (advance the state across the chunk)
                w = np.exp2(Gc[-1] - Gc) * dtc
                Sc = (Xc * w[:, None]).T @ Bc
                state = np.exp2(Gc[-1]) * state + Sc
            fin[b, h] = state
    return y, fin, states
