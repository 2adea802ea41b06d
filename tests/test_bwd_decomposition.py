"""The chunked decomposition of the backward pass, checked on the CPU.

The GPU backward evaluates the gradients per chunk (the forward pass's chunk
states, the state gradients L_c by the same recurrence run backwards, the
in-chunk terms with the decay matrix a_ij = exp(G_i - G_j)) and gets the
step-size gradient from the identity

    dl_k = <dfinal, s_L> + sum_{t >= k} (P_t - dt_t Qr_t),
    P_t = <dy_t, y_t - D x_t>,  Qr_t = <x_t, lam_t B_t>.

This test writes that decomposition out in numpy fp64 (natural-log decays, no
blocking) and compares every gradient with the token-by-token backward oracle,
on a ragged problem with groups, an initial state and dfinal.  It tests the
derivation the kernels follow, not the kernels (the GPU parity tests do that).
"""
import numpy as np
import pytest

import oracle
import ssd_synth


def chunked_bwd(x, dt, A, B, C, D, s0, dy, dS, Q):
    bsz, L, H, P = x.shape
    G, N = B.shape[2:]
    hpg = H // G
    T = -(-L // Q)
    out = {"dx": np.zeros_like(x), "ddt": np.zeros_like(dt), "dA": np.zeros(H),
           "dB": np.zeros_like(B), "dC": np.zeros_like(C), "dD": np.zeros(H),
           "dinit": np.zeros_like(s0)}
    for b in range(bsz):
        for h in range(H):
            g = h // hpg
            Gc = np.zeros(L)
            st = np.zeros((T + 1, P, N))
            st[0] = s0[b, h]
            for c in range(T):                    # chunk-start states
                t0, t1 = c * Q, min(L, c * Q + Q)
                Gc[t0:t1] = np.cumsum(dt[b, t0:t1, h] * A[h])
                w = np.exp(Gc[t1 - 1] - Gc[t0:t1]) * dt[b, t0:t1, h]
                st[c + 1] = np.exp(Gc[t1 - 1]) * st[c] + (x[b, t0:t1, h] * w[:, None]).T @ B[b, t0:t1, g]
            lam = np.zeros((T + 1, P, N))         # gradients of the chunk-end states
            lam[T] = dS[b, h]
            for c in range(T - 1, -1, -1):
                t0, t1 = c * Q, min(L, c * Q + Q)
                own = (dy[b, t0:t1, h] * np.exp(Gc[t0:t1])[:, None]).T @ C[b, t0:t1, g]
                lam[c] = np.exp(Gc[t1 - 1]) * lam[c + 1] + own
            out["dinit"][b, h] = lam[0]
            Pt, Qr = np.zeros(L), np.zeros(L)
            for c in range(T):
                t0, t1 = c * Q, min(L, c * Q + Q)
                Gq, d = Gc[t0:t1], dt[b, t0:t1, h]
                xs, gs, Bs, Cs = x[b, t0:t1, h], dy[b, t0:t1, h], B[b, t0:t1, g], C[b, t0:t1, g]
                n = t1 - t0
                a = np.where(np.tril(np.ones((n, n))) > 0, np.exp(Gq[:, None] - Gq[None, :]), 0.0)
                CB, GX = Cs @ Bs.T, gs @ xs.T
                W = a * GX * d[None, :]
                out["dC"][b, t0:t1, g] += W @ Bs + np.exp(Gq)[:, None] * (gs @ st[c])
                Pt[t0:t1] = (W * CB).sum(1) + np.exp(Gq) * np.einsum("ip,pn,in->i", gs, st[c], Cs)
                U, V, e = a * CB, a * GX, np.exp(Gq[-1] - Gq)
                cj = e[:, None] * (Bs @ lam[c + 1].T)
                out["dx"][b, t0:t1, h] = d[:, None] * (U.T @ gs + cj) + D[h] * gs
                out["dB"][b, t0:t1, g] += d[:, None] * (V.T @ Cs + e[:, None] * (xs @ lam[c + 1]))
                Qr[t0:t1] = (U * GX).sum(0) + (xs * cj).sum(1)
                out["dD"][h] += (gs * xs).sum()
            K = (dS[b, h] * st[T]).sum()
            dl = K + np.cumsum((Pt - dt[b, :, h] * Qr)[::-1])[::-1]
            out["ddt"][b, :, h] = A[h] * dl + Qr
            out["dA"][h] += (dt[b, :, h] * dl).sum()
    return out


@pytest.mark.parametrize("Q", [16, 32, 64])
def test_chunked_decomposition_matches_oracle(Q):
    p = ssd_synth.Problem(batch=2, seqlen=150, nheads=4, headdim=8, dstate=6, ngroups=2,
                          chunk_size=Q, io_dtype="fp32", init_std=0.1)
    inp = ssd_synth.make_inputs(p, 1)
    gr = ssd_synth.make_grads(p, 1)
    f = lambda t: t.double().numpy()
    x, dt, A, B, C, D, s0 = (f(inp[k]) for k in ("x", "dt", "A", "B", "C", "D", "init_state"))
    dy, dS = f(gr["dy"]), f(gr["dfinal"])
    ref = oracle.recurrence_bwd(x, dt, A, B, C, D, s0, dy, dS)
    got = chunked_bwd(x, dt, A, B, C, D, s0, dy, dS, Q)
    for k in ref:
        err = np.linalg.norm(got[k] - ref[k]) / np.linalg.norm(ref[k])
        assert err < 1e-12, (k, err)
