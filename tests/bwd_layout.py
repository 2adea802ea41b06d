"""Expected workspace layouts of ssd_bwd, written from its documentation.

The per-chunk kernels sum the dB/dC contributions of kh consecutive heads of
a group (a "part") before writing them: part_heads(p) is kh, the largest
divisor of the heads per group up to 8 that leaves batch * chunks * (H / kh)
>= 1024 workgroups, else 1.  bwd_layout(p, hb) is the byte count ssd_bwd's
workspace takes when it forms the fp32 dB/dC sums for batches of hb parts:
token rows (6 fp32 [batch, H, T*Q] arrays), two fp32 state sets, the final
state, the scalar parts, (more than one batch of parts) two fp32
[batch, L, G, N] running sums, and the dB/dC sums of hb parts; each piece
256-byte aligned.  `p` is an ssd_problem (io_dtype 1 = bf16).
"""


def _a(v):
    return (v + 255) // 256 * 256


def part_heads(p):
    T = -(-p.seqlen // p.chunk_size)
    hpg, wg = p.nheads // p.ngroups, p.batch * T
    kh = 1
    for k in range(2, min(8, hpg) + 1):
        if hpg % k == 0 and wg * (p.nheads // k) >= 1024:
            kh = k
    return kh


def parts(p):
    return p.nheads // part_heads(p)


def bwd_layout(p, hb):
    Bt, L, H, Pd, N, Q, G = p.batch, p.seqlen, p.nheads, p.headdim, p.dstate, p.chunk_size, p.ngroups
    T = -(-L // Q)
    fixed = (6 * _a(Bt * H * T * Q * 4) + 2 * _a(Bt * H * T * Pd * N * 4) + _a(Bt * H * Pd * N * 4) +
             2 * _a(Bt * H * 8) + _a(Bt * T * H * 4))
    acc = 2 * _a(Bt * L * G * N * 4) if hb < parts(p) else 0
    return fixed + acc + 2 * _a(Bt * L * hb * N * 4)


def balanced(n, cap):
    """Parts per batch when at most `cap` fit: ceil(n / cap) equal batches."""
    nbat = -(-n // cap)
    return -(-n // nbat)
