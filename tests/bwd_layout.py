"""Expected workspace layouts of ssd_bwd, written from its documentation.

bwd_layout(p, hb) is the byte count ssd_bwd's workspace takes when it forms
the per-head dB/dC partial gradients for batches of hb heads: token rows (6
fp32 [batch, H, T*Q] arrays), two fp32 state sets, the final state, the
scalar parts, (more than one batch of heads) two fp32 [batch, L, G, N]
running sums, and the dB/dC parts of hb heads; each piece 256-byte aligned.
`p` is an ssd_problem (io_dtype 1 = bf16).
"""


def _a(v):
    return (v + 255) // 256 * 256


def bwd_layout(p, hb):
    Bt, L, H, Pd, N, Q, G = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.chunk_size, p.ngroups
    T = -(-L // Q)
    fixed = (6 * _a(Bt * H * T * Q * 4) + 2 * _a(Bt * H * T * Pd * N * 4) + _a(Bt * H * Pd * N * 4) +
             2 * _a(Bt * H * 8) + _a(Bt * T * H * 4))
    acc = 2 * _a(Bt * L * G * N * 4) if hb < H else 0
    return fixed + acc + 2 * _a(Bt * L * hb * N * 4)


def balanced(H, cap):
    """Heads per batch when at most `cap` fit: ceil(H / cap) equal batches."""
    nbat = -(-H // cap)
    return -(-H // nbat)
