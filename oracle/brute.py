"""Brute-force attention in pure Python (no numpy), for tiny shapes.

Test infrastructure only (see the package docstring).

Same definition as ``attention.attend`` (the header there cites the pages),
written with nested loops, ``math.exp`` and ``math.fsum`` over Python lists,
so that an indexing or orientation mistake in the numpy version shows up as
a disagreement.
"""

from __future__ import annotations

import math


def brute_attend(q, k_seqs, v_seqs, scale):
    """q: nested lists [B][T][N][H]; k_seqs/v_seqs: [B][L_b][K][H].

    Returns (out [B][T][N][H], lse [B][T][N]) as nested lists of floats.
    """
    B = len(q)
    out, lse = [], []
    for b in range(B):
        T = len(q[b])
        N = len(q[b][0])
        H = len(q[b][0][0])
        L = len(k_seqs[b])
        K = len(k_seqs[b][0])
        G = N // K
        P = L - T
        out_b, lse_b = [], []
        for t in range(T):
            out_t, lse_t = [], []
            for n in range(N):
                kh = n // G
                scores = []
                for j in range(P + t + 1):
                    scores.append(scale * math.fsum(q[b][t][n][h] * k_seqs[b][j][kh][h] for h in range(H)))
                m = max(scores)
                w = [math.exp(s - m) for s in scores]
                z = math.fsum(w)
                o = [math.fsum(w[j] * v_seqs[b][j][kh][h] for j in range(len(w))) / z for h in range(H)]
                out_t.append(o)
                lse_t.append(m + math.log(z))
            out_b.append(out_t)
            lse_b.append(lse_t)
        out.append(out_b)
        lse.append(lse_b)
    return out, lse
