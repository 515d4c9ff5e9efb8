"""Plain fp64 CPU oracle for dynamic bifocal RoPE attention.

TEST INFRASTRUCTURE ONLY. This module is the checker, not the product: only
the test suite, the smoke check and the benchmark's CPU-baseline leg may
import it. The HIP library and its Python binding never import, call or link
anything here, and nothing here imports them.

Every routine is the plain definition from the pages, evaluated directly in
float64 with NumPy; no blocking, fusion or reordering beyond what the
definition states.

Citations (page title, then the part of the page):
  [Digest/Method]  r9-hu paper digest of "Jet-Long: Efficient Long-Context
                   Extension with Dynamic Bifocal RoPE", section Method.
                   Eq. 1 (the piecewise bifocal score), the "Dynamic group
                   size" paragraph (G and f), the "KV cache invariant"
                   paragraph (offsets and R_a R_b = R_{a+b}) and the
                   "Inclusion-exclusion prefill" paragraph (the merge).
  [Pith/Ledger]    pith.science review of arXiv 2607.07740, Axiom &
                   Free-Parameter Ledger: Sec. 3.1 Eq. 2 (G), Sec. 3.2
                   Eqs. 5-6 (correction rotation), Sec. 3.3 Eq. 7 (merge).
  [Pith/Review]    the same page's Referee Report, major comment 2 (Sec. 3.1
                   Eqs. 2-3 and Table 6) and the ledger's axiom on the
                   discrete angle grid (Sec. 4.5 / Table 6): the comparison
                   arm with continuous frequency interpolation in place of
                   floor-division aliasing.
  [RoFormer]       the rotary embedding the pages build on (their reference
                   list: Su et al., RoFormer). The pages print no frequency
                   formula; the reading used here is stated in rope().

Readings of points the pages leave open (each also listed in the design
notes): positions are 0-based per sequence; q - k == w0 is local; the
softmax scale is 1/sqrt(d) in both branches; RoPE pairs element i with
i + d/2 and uses omega_i = theta^(-2i/d); query head h reads KV head
h // (Hq/Hkv); decode at position p uses L = p + 1. The continuous remote
map (the Table 6 comparison arm, whose formula the pages do not print) is
read as f(x) = x / G, a real number, with the same G and the same local
window: positional interpolation of the remote branch by the factor G.

Status of the pins (tests/test_oracle_pins.py): every public function here is
pinned against closed forms, library routines, brute force or invariants.
"""
from __future__ import annotations

import math

import numpy as np

__all__ = [
    "group_size", "remap", "rope_frequencies", "rope", "bifocal_scores",
    "bifocal_attention", "bifocal_varlen", "decode_row", "decode_batch", "ie_pass",
    "ie_merge", "tile_class", "tile_class_map",
]


# ---------------------------------------------------------------------------
# Eq. 2 and the remote map
# ---------------------------------------------------------------------------
def group_size(L: int, w_pre: int) -> int:
    """G = max(1, ceil(L / w_pretrained)).

    [Digest/Method, "Dynamic group size"; Pith/Ledger Sec. 3.1 Eq. 2]. The
    ceiling is taken in exact integer arithmetic.
    """
    L = int(L)
    w_pre = int(w_pre)
    if L < 1 or w_pre < 1:
        raise ValueError("group_size needs L >= 1 and w_pre >= 1")
    return max(1, -(-L // w_pre))


def remap(p, G: int, continuous: bool = False):
    """f(x) = floor(x / G) for non-negative integer positions
    [Digest/Method, "Dynamic group size"].

    continuous=True: f(x) = x / G as a float64 real number, the continuous
    frequency-interpolation arm [Pith/Review, Table 6]: a rotation by
    (x / G) * omega_i is a rotation by x at the frequency omega_i / G.
    """
    if continuous:
        return np.asarray(p, dtype=np.int64).astype(np.float64) / float(G)
    return np.asarray(p, dtype=np.int64) // int(G)


# ---------------------------------------------------------------------------
# RoPE
# ---------------------------------------------------------------------------
def rope_frequencies(d: int, theta: float) -> np.ndarray:
    """omega_i = theta^(-2i/d), i = 0 .. d/2-1, in float64.

    [RoFormer]; the pages do not print it. This is the standard rotary
    frequency ladder used by the Qwen3-shaped workloads.
    """
    if d % 2:
        raise ValueError("head dim must be even")
    i = np.arange(d // 2, dtype=np.float64)
    return np.power(np.float64(theta), -2.0 * i / d)


def rope(x, pos, theta: float) -> np.ndarray:
    """RoPE(x, p): rotate each pair (x_i, x_{i+d/2}) by the angle p * omega_i.

    x: [n, H, d] (or [n, d]); pos: [n] positions (integers; any real value is
    accepted so that the rotation of a rotated vector can be written). The
    rotation is (a, b) -> (a cos t - b sin t, a sin t + b cos t).
    [Digest/Method, Eq. 1 uses RoPE(x, p); RoFormer for the rotation.]
    """
    x = np.asarray(x, dtype=np.float64)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    d = x.shape[-1]
    half = d // 2
    ang = np.asarray(pos, dtype=np.float64).reshape(-1, 1) * rope_frequencies(d, theta)[None, :]
    c = np.cos(ang)[:, None, :]
    s = np.sin(ang)[:, None, :]
    a = x[..., :half]
    b = x[..., half:]
    out = np.concatenate([a * c - b * s, a * s + b * c], axis=-1)
    return out[:, 0, :] if squeeze else out


# ---------------------------------------------------------------------------
# Eq. 1: the bifocal score
# ---------------------------------------------------------------------------
def bifocal_scores(xq_rows, q_pos, xk, k_pos, w0: int, G: int, theta: float,
                   continuous: bool = False) -> np.ndarray:
    """S(q, k) for one head: [len(q_pos), len(k_pos)] before scaling/masking.

    S = RoPE(x_q, q) . RoPE(x_k, k)          if q - k <= w0
      = RoPE(x_q, f(q)) . RoPE(x_k, f(k))    otherwise,   f(x) = floor(x/G).
    [Digest/Method, Eq. 1]. Both branches are computed in full from the raw
    vectors and the result is selected element by element on the distance.
    xq_rows: [nq, d], xk: [nk, d] raw (pre-RoPE) vectors. continuous: remote
    branch at f(x) = x / G (see remap).
    """
    q_pos = np.asarray(q_pos, dtype=np.int64)
    k_pos = np.asarray(k_pos, dtype=np.int64)
    qa = rope(xq_rows, q_pos, theta)
    qr = rope(xq_rows, remap(q_pos, G, continuous), theta)
    ka = rope(xk, k_pos, theta)
    kr = rope(xk, remap(k_pos, G, continuous), theta)
    s_local = qa @ ka.T
    s_remote = qr @ kr.T
    dist = q_pos[:, None] - k_pos[None, :]
    return np.where(dist <= w0, s_local, s_remote)


def _softmax_rows(S: np.ndarray, vals: np.ndarray):
    """Full softmax over the last axis with the max subtracted; returns
    (S-weighted average of vals, natural-log LSE). Rows must hold at least
    one finite score."""
    m = S.max(axis=1, keepdims=True)
    P = np.exp(S - m)
    l = P.sum(axis=1, keepdims=True)
    O = (P @ vals) / l
    lse = (m + np.log(l))[:, 0]
    return O, lse


def bifocal_attention(xq, xk, v, w0: int, w_pre: int, theta: float, scale=None,
                      rows=None, heads=None, G=None, row_chunk: int = 128,
                      continuous: bool = False):
    """Causal bifocal attention for ONE sequence (positions 0 .. L-1).

    xq: [L, Hq, d], xk / v: [L, Hkv, d] raw float arrays (upcast to fp64).
    Returns (O [len(rows), Hq, d], LSE [Hq, len(rows)]) in float64 for the
    query rows `rows` (default: all) and heads `heads` (default: all; other
    heads are left zero). G defaults to Eq. 2 with L = number of keys.

    Per row q: scores S(q, k) of Eq. 1 for keys k <= q, times scale
    (default 1/sqrt(d)), full softmax, weighted sum of v. GQA: query head h
    reads KV head h // (Hq / Hkv). [Digest/Method, Eq. 1 and "Dynamic group
    size".] Rotations are applied directly to the raw vectors at the absolute
    and the remapped positions, never through correction offsets.
    continuous: remote branch at f(x) = x / G (see remap).
    """
    xq = np.asarray(xq)
    xk = np.asarray(xk)
    v = np.asarray(v)
    L, Hq, d = xq.shape
    Lk, Hkv, dk = xk.shape
    if Lk != L or dk != d or v.shape != xk.shape or Hq % Hkv:
        raise ValueError("shape mismatch")
    r = Hq // Hkv
    if G is None:
        G = group_size(L, w_pre)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(L, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    heads = range(Hq) if heads is None else heads
    order = np.argsort(rows, kind="stable")
    O = np.zeros((len(rows), Hq, d), dtype=np.float64)
    LSE = np.zeros((Hq, len(rows)), dtype=np.float64)
    kpos = np.arange(L, dtype=np.int64)
    # Keys rotated once per KV head at absolute and remapped positions.
    ka_all = rope(xk, kpos, theta)
    kr_all = rope(xk, remap(kpos, G, continuous), theta)
    v64 = v.astype(np.float64)
    qa_all = rope(xq[rows], rows, theta)
    qr_all = rope(xq[rows], remap(rows, G, continuous), theta)
    for h in heads:
        g = h // r
        for c0 in range(0, len(rows), row_chunk):
            idx = order[c0:c0 + row_chunk]
            qrows = rows[idx]
            nk = int(qrows.max()) + 1  # keys beyond the last row are all masked
            s_local = qa_all[idx, h] @ ka_all[:nk, g].T
            s_remote = qr_all[idx, h] @ kr_all[:nk, g].T
            dist = qrows[:, None] - kpos[None, :nk]
            S = np.where(dist <= w0, s_local, s_remote) * scale
            S = np.where(dist >= 0, S, -np.inf)
            o, lse = _softmax_rows(S, v64[:nk, g])
            O[idx, h] = o
            LSE[h, idx] = lse
    return O, LSE


def bifocal_varlen(xq, xk, v, cu_seqlens, w0, w_pre, theta, scale=None, rows_per_seq=None,
                   heads=None, continuous: bool = False):
    """Packed batch: sequence b owns tokens cu_seqlens[b] .. cu_seqlens[b+1]-1.

    Each sequence is independent: positions restart at 0 and G comes from
    that sequence's own length. rows_per_seq: optional list of per-sequence
    row arrays (sequence-relative). Returns a list of (rows, O, LSE).
    [Digest/Method, "Dynamic group size": G depends on the current length.]
    """
    out = []
    cu = [int(c) for c in cu_seqlens]
    for b in range(len(cu) - 1):
        s, e = cu[b], cu[b + 1]
        rows = None if rows_per_seq is None else rows_per_seq[b]
        if e == s:  # an empty sequence has no query rows
            Hq, d = np.asarray(xq).shape[1:]
            out.append((np.zeros(0, dtype=np.int64), np.zeros((0, Hq, d)), np.zeros((Hq, 0))))
            continue
        O, LSE = bifocal_attention(xq[s:e], xk[s:e], v[s:e], w0, w_pre, theta, scale=scale,
                                   rows=rows, heads=heads, continuous=continuous)
        out.append((np.arange(e - s) if rows is None else np.asarray(rows), O, LSE))
    return out


# ---------------------------------------------------------------------------
# Decode: one query at position p against the absolute cache
# ---------------------------------------------------------------------------
def decode_row(xq_row, xk_cache, v_cache, pos: int, w0: int, w_pre: int, theta: float,
               scale=None, continuous: bool = False):
    """Single-token step at position `pos`, keys 0 .. pos, L = pos + 1.

    xq_row: [Hq, d] raw query; xk_cache / v_cache: [>= pos+1, Hkv, d] raw keys
    and values (the cache rows beyond pos are never read). For each key the
    route is chosen on pos - k <= w0 and the score is computed from vectors
    rotated directly at (pos, k) or (f(pos), f(k)). Returns (o [Hq, d],
    lse [Hq]) in float64. [Digest/Method, Eq. 1 and "KV cache invariant":
    the cache holds absolute keys and is never rewritten when G changes.]
    Written independently of bifocal_attention so that the two can be
    compared. continuous: remote route at pos / G and k / G (real numbers).
    """
    xq_row = np.asarray(xq_row, dtype=np.float64)
    Hq, d = xq_row.shape
    Hkv = xk_cache.shape[1]
    r = Hq // Hkv
    L = pos + 1
    G = group_size(L, w_pre)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    keys = np.arange(L, dtype=np.int64)
    xk = np.asarray(xk_cache[:L], dtype=np.float64)
    vv = np.asarray(v_cache[:L], dtype=np.float64)
    local = (pos - keys) <= w0
    if continuous:
        k_rem_pos, q_rem_pos = keys / float(G), pos / float(G)
    else:
        k_rem_pos, q_rem_pos = keys // G, pos // G
    k_at = rope(xk, np.where(local, keys, k_rem_pos), theta)  # [L, Hkv, d]
    q_abs = rope(xq_row[None], [pos], theta)[0]
    q_rem = rope(xq_row[None], [q_rem_pos], theta)[0]
    o = np.zeros((Hq, d))
    lse = np.zeros(Hq)
    for h in range(Hq):
        g = h // r
        s = np.where(local, k_at[:, g] @ q_abs[h], k_at[:, g] @ q_rem[h]) * scale
        m = s.max()
        p = np.exp(s - m)
        o[h] = (p @ vv[:, g]) / p.sum()
        lse[h] = m + math.log(p.sum())
    return o, lse


def decode_batch(xq, k_rows, v_rows, positions, starts, w0: int, w_pre: int, theta: float,
                 max_keys=None, scale=None, continuous: bool = False):
    """One decode step for each of B independent sequences sharing a cache
    buffer: sequence b's key k is row starts[b] + k of k_rows / v_rows (raw
    keys and values, [rows, Hkv, d]); its query xq[b] sits at positions[b]
    and takes G from its own L = positions[b] + 1 [Digest/Method, "Dynamic
    group size": G follows the current length of each sequence].

    An entry whose keys would fall outside the buffer (position < 0, start <
    0, start + position >= rows) or at or past max_keys (when given) has no
    defined result: its outputs are NaN. Returns (o [B, Hq, d], lse [B, Hq]).
    """
    xq = np.asarray(xq, dtype=np.float64)
    B, Hq, d = xq.shape
    rows = np.asarray(k_rows).shape[0]
    o = np.full((B, Hq, d), np.nan)
    lse = np.full((B, Hq), np.nan)
    for b in range(B):
        p, s0 = int(positions[b]), int(starts[b])
        if p < 0 or s0 < 0 or s0 + p >= rows or (max_keys is not None and p >= max_keys):
            continue
        o[b], lse[b] = decode_row(xq[b], k_rows[s0:s0 + p + 1], v_rows[s0:s0 + p + 1], p, w0,
                                  w_pre, theta, scale=scale, continuous=continuous)
    return o, lse


# ---------------------------------------------------------------------------
# Eq. 7: inclusion-exclusion over three attention passes
# ---------------------------------------------------------------------------
def ie_pass(xq, xk, v, which: str, w0: int, G: int, theta: float, scale=None,
            continuous: bool = False):
    """One of the three plain attention passes, one sequence, all rows/heads.

    'A': keys with 0 <= q-k <= w0, RoPE at absolute positions;
    'B': all keys with k <= q, RoPE at remapped positions f(.);
    'C': keys with 0 <= q-k <= w0, RoPE at remapped positions.
    B minus C is exactly the remote key set, so A + B - C covers every key
    once with the right rotation. [Digest/Method, "Inclusion-exclusion
    prefill"; ResearchPod dialogue: local view, remapped distant view and
    corrected local view.] Returns (O [L,Hq,d], LSE [Hq,L]) float64.
    continuous: passes B and C rotate at x / G (real numbers).
    """
    xq = np.asarray(xq, dtype=np.float64)
    xk = np.asarray(xk, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    L, Hq, d = xq.shape
    Hkv = xk.shape[1]
    r = Hq // Hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    pos = np.arange(L, dtype=np.int64)
    if which == "A":
        p_rot = pos
    else:
        p_rot = pos / float(G) if continuous else pos // G
    q = rope(xq, p_rot, theta)
    k = rope(xk, p_rot, theta)
    dist = pos[:, None] - pos[None, :]
    keep = dist >= 0 if which == "B" else (dist >= 0) & (dist <= w0)
    O = np.zeros((L, Hq, d))
    LSE = np.zeros((Hq, L))
    for h in range(Hq):
        g = h // r
        S = np.where(keep, (q[:, h] @ k[:, g].T) * scale, -np.inf)
        O[:, h], LSE[h] = _softmax_rows(S, v[:, g])
    return O, LSE


def ie_merge(OA, lA, OB, lB, OC, lC):
    """O = (W_A O_A + W_B O_B - W_C O_C) / (W_A + W_B - W_C),
    W_X = exp(l_X - M), M = max(l_A, l_B, l_C), natural log.

    [Digest/Method, "Inclusion-exclusion prefill"; Pith/Ledger Sec. 3.3
    Eq. 7.] O_X: [L, Hq, d]; l_X: [Hq, L]. Returns (O, LSE) where
    LSE = M + log(W_A + W_B - W_C) (the LSE of the union key set).
    """
    M = np.maximum(np.maximum(lA, lB), lC)
    WA, WB, WC = np.exp(lA - M), np.exp(lB - M), np.exp(lC - M)
    den = WA + WB - WC
    num = (WA.T[..., None] * OA + WB.T[..., None] * OB - WC.T[..., None] * OC)
    return num / den.T[..., None], M + np.log(den)


# ---------------------------------------------------------------------------
# Tile classification (the definition over query/key pairs)
# ---------------------------------------------------------------------------
def tile_class(q0: int, q1: int, k0: int, k1: int, w0: int) -> int:
    """Class of the tile of query positions q0..q1 and key positions k0..k1.

    Enumerates every pair. 0 = masked (no pair has k <= q); 1 = local (every
    causal pair has q-k <= w0); 2 = remote (every causal pair has q-k > w0);
    3 = boundary (both kinds). 4 is added when some pair has k > q (the
    causal diagonal crosses the tile). Follows Eq. 1's routing condition
    [Digest/Method, Eq. 1]; depends on distances only, never on G.
    """
    q = np.arange(q0, q1 + 1, dtype=np.int64)[:, None]
    k = np.arange(k0, k1 + 1, dtype=np.int64)[None, :]
    causal = k <= q
    if not causal.any():
        return 0
    near = causal & (q - k <= w0)
    far = causal & (q - k > w0)
    cls = 1 if not far.any() else (2 if not near.any() else 3)
    if (~causal).any():
        cls += 4
    return cls


def tile_class_map(L: int, BM: int, BN: int, w0: int) -> np.ndarray:
    """[ceil(L/BM), ceil(L/BN)] int8 map of tile_class over a length-L
    sequence cut into BM-row query tiles and BN-key tiles (the last tile of
    each axis is clipped at L-1)."""
    nq = -(-L // BM)
    nk = -(-L // BN)
    out = np.zeros((nq, nk), dtype=np.int8)
    for i in range(nq):
        q0, q1 = i * BM, min(L, (i + 1) * BM) - 1
        for j in range(nk):
            k0, k1 = j * BN, min(L, (j + 1) * BN) - 1
            out[i, j] = tile_class(q0, q1, k0, k1, w0)
    return out
