"""Pure-Python scalar brute force for tiny decode-attention cases.

TEST INFRASTRUCTURE ONLY: an independent second implementation used to pin
``oracle.reference`` on tiny shapes.  It uses only the ``math`` module and
Python floats (IEEE float64), explicit loops, and a two-pass softmax; it
shares no code with ``oracle.reference`` or with the HIP path.

Definitions follow the fusedtok 1.0.1 README ("Operators": RMSNorm, RoPE
NeoX layout, attention_decode with GQA and per-sequence lengths) and the
cutileGPT README ("Why tiles" RMSNorm figure; sliding-window attention).
"""
from __future__ import annotations

import math


def rmsnorm(x, w, eps):
    """List in, list out: x_i / sqrt(sum x^2 / n + eps) * w_i."""
    n = len(x)
    ss = 0.0
    for v in x:
        ss += v * v
    r = 1.0 / math.sqrt(ss / n + eps)
    return [x[i] * r * w[i] for i in range(n)]


def rope_neox(x, pos, theta):
    """Rotate element i with element i + D/2 by pos * theta**(-2i/D)."""
    D = len(x)
    h = D // 2
    y = list(x)
    for i in range(h):
        a = pos * theta ** (-2.0 * i / D)
        c, s = math.cos(a), math.sin(a)
        y[i] = x[i] * c - x[i + h] * s
        y[i + h] = x[i + h] * c + x[i] * s
    return y


def attend(q, K, V, lens, window=0, scale=0.0):
    """Nested lists: q[b][h][d], K/V[b][g][t][d], lens[b] -> (out[b][h][d], lse[b][h]).

    Two passes per (b, h): first the maximum score, then exponentials, the
    normaliser and the weighted sum of V rows.
    """
    B, Hq, D = len(q), len(q[0]), len(q[0][0])
    Hkv, T = len(K[0]), len(K[0][0])
    G = Hq // Hkv
    if scale <= 0:
        scale = 1.0 / math.sqrt(D)
    out, lse = [], []
    for b in range(B):
        n = min(max(lens[b], 0), T)
        lo = max(0, n - window) if window > 0 else 0
        ob, lb = [], []
        for h in range(Hq):
            g = h // G
            scores = []
            for t in range(lo, n):
                acc = 0.0
                for d in range(D):
                    acc += q[b][h][d] * K[b][g][t][d]
                scores.append(acc * scale)
            if not scores:
                ob.append([0.0] * D)
                lb.append(-math.inf)
                continue
            m = -math.inf
            for s in scores:
                if s > m:
                    m = s
            den = 0.0
            num = [0.0] * D
            for j, t in enumerate(range(lo, n)):
                p = math.exp(scores[j] - m)
                den += p
                for d in range(D):
                    num[d] += p * V[b][g][t][d]
            ob.append([v / den for v in num])
            lb.append(m + math.log(den))
        out.append(ob)
        lse.append(lb)
    return out, lse


def rope_pairs(x, pos, inv_freq, layout="neox", mscale=1.0):
    """Rotate pair i by pos * inv_freq[i] and scale by mscale, scalar loops.

    Pair i is (i, i + D/2) for "neox" and (2i, 2i + 1) for "interleaved"
    (the two layouts the fusedtok README's RoPE row names).
    """
    D = len(x)
    h = D // 2
    y = list(x)
    for i in range(h):
        u, v = (i, i + h) if layout == "neox" else (2 * i, 2 * i + 1)
        a = pos * inv_freq[i]
        c, s = math.cos(a), math.sin(a)
        y[u] = mscale * (x[u] * c - x[v] * s)
        y[v] = mscale * (x[v] * c + x[u] * s)
    return y


def linear(x, w):
    """Lists x[m][k], w[n][k] -> y[m][n] = sum_k x[m][k] * w[n][k], loops."""
    y = []
    for row in x:
        out = []
        for wr in w:
            acc = 0.0
            for a, b in zip(row, wr):
                acc += a * b
            out.append(acc)
        y.append(out)
    return y
