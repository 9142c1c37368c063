"""Independent pure-Python brute force for tiny shapes (math.fsum / math.exp).

A second implementation of the attention definition written without NumPy or
the C oracle: nested lists, exactly rounded sums.  Used only to pin the oracle.
"""
import math


def attention(q, k, v, scale):
    """q: nested list [B][Sq][H][d]; k, v: [B][Skv][H][d] (python floats).
    Returns (o [B][Sq][H][d], lse [B][H][Sq])."""
    B, Sq, H, d = len(q), len(q[0]), len(q[0][0]), len(q[0][0][0])
    Skv = len(k[0])
    o = [[[[0.0] * d for _ in range(H)] for _ in range(Sq)] for _ in range(B)]
    lse = [[[0.0] * Sq for _ in range(H)] for _ in range(B)]
    for b in range(B):
        for h in range(H):
            for i in range(Sq):
                logits = [scale * math.fsum(q[b][i][h][c] * k[b][j][h][c] for c in range(d))
                          for j in range(Skv)]
                mx = max(logits)
                w = [math.exp(s - mx) for s in logits]
                den = math.fsum(w)
                for c in range(d):
                    o[b][i][h][c] = math.fsum(w[j] * v[b][j][h][c] for j in range(Skv)) / den
                lse[b][h][i] = mx + math.log(den)
    return o, lse
