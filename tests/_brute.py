"""Scalar pure-Python brute force of the bifocal score, for tiny inputs.

Written independently of the oracle (no NumPy, no shared helpers): every
rotation, dot product and softmax term is a Python float loop, straight from
the definition. [Digest/Method, Eq. 1 and the "Dynamic group size"
paragraph; RoFormer rotation with pairs (i, i + d/2).]
"""
import math


def _rotate(vec, p, theta):
    d = len(vec)
    h = d // 2
    out = [0.0] * d
    for i in range(h):
        w = theta ** (-(2.0 * i) / d)
        c, s = math.cos(p * w), math.sin(p * w)
        a, b = vec[i], vec[i + h]
        out[i] = a * c - b * s
        out[i + h] = a * s + b * c
    return out


def brute_attention(xq, xk, v, w0, w_pre, theta, scale=None, positions=None, continuous=False):
    """xq: list[L][Hq][d], xk / v: list[L][Hkv][d] (nested Python lists).
    Returns (O list[L][Hq][d], LSE list[Hq][L]). continuous: remote pairs
    rotate at the real positions q / G and k / G instead of floor(. / G)."""
    L = len(xq)
    Hq = len(xq[0])
    Hkv = len(xk[0])
    d = len(xq[0][0])
    r = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    # G: smallest positive integer g with ceil(L / g) <= w_pre, found by search.
    G = 1
    while -(-L // G) > w_pre:
        G += 1
    O = [[[0.0] * d for _ in range(Hq)] for _ in range(L)]
    LSE = [[0.0] * L for _ in range(Hq)]
    for h in range(Hq):
        g = h // r
        for q in range(L):
            scores = []
            for k in range(q + 1):
                if q - k <= w0:
                    pq, pk = q, k
                elif continuous:
                    pq, pk = q / G, k / G
                else:
                    pq, pk = q // G, k // G
                a = _rotate(xq[q][h], pq, theta)
                b = _rotate(xk[k][g], pk, theta)
                scores.append(scale * sum(a[i] * b[i] for i in range(d)))
            m = max(scores)
            ws = [math.exp(s - m) for s in scores]
            tot = sum(ws)
            for i in range(d):
                O[q][h][i] = sum(ws[k] * v[k][g][i] for k in range(q + 1)) / tot
            LSE[h][q] = m + math.log(tot)
    return O, LSE


def brute_score(xq_row, q, xk_row, k, w0, G, theta, continuous=False):
    """Unscaled score of Eq. 1 for ONE query vector at position q and ONE key
    vector at position k (flat Python lists): the local route rotates at
    (q, k) when q - k <= w0, the remote route at floor(q / G), floor(k / G)
    (or q / G, k / G with continuous)."""
    if q - k <= w0:
        pq, pk = q, k
    elif continuous:
        pq, pk = q / G, k / G
    else:
        pq, pk = q // G, k // G
    a = _rotate(list(xq_row), pq, theta)
    b = _rotate(list(xk_row), pk, theta)
    return sum(a[i] * b[i] for i in range(len(a)))
