"""Brute-force scalar version of sliding-window GQA attention for tiny inputs.

TEST INFRASTRUCTURE ONLY (see swa_oracle).  Pure-Python loops with math.exp
and math.fsum, written independently of swa_oracle's NumPy code so that the
two can pin each other: the key set is enumerated per query straight from the
SWA equation of "Mistral 7B: Engineering Extreme Efficiency in LLMs" (How It
Works 2, read as i - W < j <= i) plus the sink prefix of the aionda page, and
the softmax is taken over that list one score at a time.
"""
from __future__ import annotations

import math

__all__ = ["attend_brute", "rope_brute"]


def rope_brute(vec, p, theta):
    """Rotate one head vector (a list of D floats) to position p, pairwise."""
    if theta == 0:
        return list(vec)
    D = len(vec)
    out = [0.0] * D
    for kk in range(D // 2):
        a = p * theta ** (-(2.0 * kk) / D)
        x0, x1 = vec[2 * kk], vec[2 * kk + 1]
        out[2 * kk] = x0 * math.cos(a) - x1 * math.sin(a)
        out[2 * kk + 1] = x0 * math.sin(a) + x1 * math.cos(a)
    return out


def _keys_of(i, window, n_sink, dilation):
    """Positions a query at i attends, built by walking back from i in steps
    of `dilation` while inside the window, then adding the sink positions not
    already listed."""
    keys = []
    j = i
    while j >= 0 and j > i - window:
        keys.append(j)
        j -= dilation
    for s in range(min(n_sink, i + 1)):
        if s not in keys:
            keys.append(s)
    return sorted(keys)


def attend_brute(q, k, v, window, n_sink=0, scale=None, dilation=1):
    """q: [N][Hq][D], k, v: [N][Hkv][D] nested lists for positions 0..N-1
    (already rotated).  Returns (out [N][Hq][D], lse [Hq][N])."""
    N = len(q)
    Hq = len(q[0])
    Hkv = len(k[0])
    D = len(q[0][0])
    G = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(N)]
    lse = [[0.0] * N for _ in range(Hq)]
    for i in range(N):
        keys = _keys_of(i, window, n_sink, dilation)
        for h in range(Hq):
            g = h // G
            scores = [scale * math.fsum(q[i][h][d] * k[j][g][d] for d in range(D)) for j in keys]
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            z = math.fsum(w)
            for d in range(D):
                out[i][h][d] = math.fsum(w[t] * v[j][g][d] for t, j in enumerate(keys)) / z
            lse[h][i] = m + math.log(z)
    return out, lse
