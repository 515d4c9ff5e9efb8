"""Pins for the fp64 oracle: closed forms, library routines, brute force and
invariants that the pages and the mathematics fix. CPU only.

Each test names the passage it pins. A plausible slip in the oracle (a
dropped branch, a wrong sign, a swapped index, a wrong group size, an
off-by-one in the window or the causal mask, the wrong GQA map) fails at
least one of them.
"""
import math
import os

import numpy as np
import pytest
import torch

from oracle import (bifocal_attention, bifocal_scores, bifocal_varlen, decode_batch, decode_row,
                    group_size, ie_merge, ie_pass, remap, rope, rope_frequencies, tile_class,
                    tile_class_map)
from tests._brute import brute_attention, brute_score

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, *shape):
    return np.random.default_rng(seed).standard_normal(shape)


# ---------------------------------------------------------------- Eq. 2 / G
def test_group_size_golden_table():
    """Hand-derived integer ceilings of Eq. 2 [Digest/Method, "Dynamic group
    size"; Pith/Ledger Sec. 3.1 Eq. 2], stored with their citation."""
    path = os.path.join(GOLDEN, "group_size_cases.txt")
    n = 0
    with open(path) as fh:
        for line in fh:
            line = line.split("#")[0].strip()
            if not line:
                continue
            L, w_pre, G = (int(t) for t in line.split())
            assert group_size(L, w_pre) == G, (L, w_pre)
            n += 1
    assert n >= 20


def test_group_size_minimal_bruteforce_small():
    """G is the smallest integer g >= 1 keeping every remapped position
    floor(p/g), p < L, inside the pretrained grid 0..w_pre-1 (the minimality
    stated with Eq. 2). Exhaustive search for L <= 2048."""
    for w_pre in (1, 7, 64, 32768):
        for L in range(1, 2049):
            g = 1
            while (L - 1) // g > w_pre - 1:
                g += 1
            assert group_size(L, w_pre) == g


def test_group_size_minimal_vectorized_large():
    """Same minimality for every L in [1, 2^20]: the condition holds at G and
    fails at G-1 (the condition is monotone in g)."""
    L = np.arange(1, 2 ** 20 + 1, dtype=np.int64)
    for w_pre in (1, 7, 64, 32768):
        G = np.array([group_size(int(x), w_pre) for x in L[:: 997]] +
                     [group_size(int(L[-1]), w_pre)], dtype=np.int64)
        Ls = np.concatenate([L[:: 997], L[-1:]])
        assert np.all((Ls - 1) // G <= w_pre - 1)
        prev = G - 1
        ok = prev >= 1
        assert np.all((Ls[ok] - 1) // prev[ok] > w_pre - 1)


def test_group_size_rejects_bad_args():
    with pytest.raises(ValueError):
        group_size(0, 4)
    with pytest.raises(ValueError):
        group_size(4, 0)


def test_remap_floor():
    assert list(remap(np.arange(9), 3)) == [0, 0, 0, 1, 1, 1, 2, 2, 2]
    assert list(remap(np.arange(4), 1)) == [0, 1, 2, 3]


# ---------------------------------------------------------------- RoPE
def test_rope_frequency_ladder_closed_form():
    """theta^(-2i/d) by hand: d=8, theta=1e4 -> 1, 0.1, 0.01, 0.001."""
    np.testing.assert_allclose(rope_frequencies(8, 1e4), [1.0, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(rope_frequencies(4, 1e6), [1.0, 1e-3], rtol=1e-15)


def test_rope_rotation_closed_form_d2():
    """d = 2, omega = 1: e1 -> (cos p, sin p), e2 -> (-sin p, cos p)."""
    p = np.array([0, 1, 5, 131071])
    e1 = np.tile([1.0, 0.0], (4, 1))
    e2 = np.tile([0.0, 1.0], (4, 1))
    np.testing.assert_allclose(rope(e1, p, 1e4), np.stack([np.cos(p), np.sin(p)], 1), atol=1e-15)
    np.testing.assert_allclose(rope(e2, p, 1e4), np.stack([-np.sin(p), np.cos(p)], 1), atol=1e-15)


def test_rope_matches_complex_multiplication():
    """Pair (x_i, x_{i+d/2}) as a complex number times exp(1j * p * omega_i)
    with omega_i = theta^(-2i/d) [RoFormer], via numpy's complex exp."""
    d, theta = 16, 1e4
    x = _rand(1, 7, 3, d)
    p = np.array([0, 1, 2, 100, 4097, 65535, 131071])
    z = x[..., : d // 2] + 1j * x[..., d // 2:]
    om = np.array([theta ** (-(2.0 * i) / d) for i in range(d // 2)])
    zr = z * np.exp(1j * p[:, None, None] * om[None, None, :])
    y = rope(x, p, theta)
    np.testing.assert_allclose(y[..., : d // 2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[..., d // 2:], zr.imag, atol=1e-12)


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("theta", [1e4, 1e6])
def test_correction_rotation_composition(d, theta):
    """R_{Delta k} RoPE(x, k) == RoPE(x, f(k)) with Delta k = f(k) - k, for all
    k < 2^17 and G in 1..8 [Digest/Method, "KV cache invariant"; Pith/Ledger
    Sec. 3.2 Eqs. 5-6: R_a R_b = R_{a+b}]."""
    k = np.arange(2 ** 17, dtype=np.int64)
    x = _rand(2, 1, 1, d)[0]                       # one raw key vector [1, d]
    xs = np.broadcast_to(x, (k.size, d))
    k_abs = rope(xs, k, theta)
    for G in range(1, 9):
        f = remap(k, G)
        direct = rope(xs, f, theta)
        corrected = rope(k_abs, f - k, theta)
        err = np.abs(corrected - direct).max() / np.abs(direct).max()
        assert err <= 1e-9, (G, err)


def test_rope_preserves_norm_and_relative_angle():
    """Rotation is orthogonal and RoPE(q,m).RoPE(k,n) depends on m - n only."""
    d, theta = 32, 1e6
    q, k = _rand(3, 1, d), _rand(4, 1, d)
    np.testing.assert_allclose(np.linalg.norm(rope(q, [12345], theta)), np.linalg.norm(q),
                               rtol=1e-13)
    a = (rope(q, [1000], theta) * rope(k, [400], theta)).sum()
    b = (rope(q, [600], theta) * rope(k, [0], theta)).sum()
    c = (rope(q, [700], theta) * rope(k, [100], theta)).sum()
    assert abs(a - b) < 1e-10 and abs(b - c) < 1e-10


# ---------------------------------------------------------------- Eq. 1 closed forms
def test_closed_form_three_tokens():
    """d = 2 (omega = 1), unit vectors, L = 3, w0 = 0, G = 2 (w_pre = 2).
    f = (0, 0, 1). By hand: S(q,q) = 1 (local, same angle); S(1,0) = cos(0);
    S(2,0) = S(2,1) = cos(f(2) - f(0)) = cos(1). Scale 1/sqrt(2).
    [Digest/Method, Eq. 1 and "Dynamic group size"]"""
    xq = np.tile([1.0, 0.0], (3, 1, 1))
    xk = xq.copy()
    v = np.array([[[1.0, 0.0]], [[0.0, 1.0]], [[2.0, 3.0]]])
    O, LSE = bifocal_attention(xq, xk, v, w0=0, w_pre=2, theta=1e4)
    sc = 1 / math.sqrt(2)
    s2 = [math.cos(1) * sc, math.cos(1) * sc, 1.0 * sc]
    m = max(s2)
    w = [math.exp(s - m) for s in s2]
    o2 = [sum(w[k] * v[k, 0, i] for k in range(3)) / sum(w) for i in range(2)]
    np.testing.assert_allclose(O[2, 0], o2, atol=1e-14)
    assert abs(LSE[0, 2] - (m + math.log(sum(w)))) < 1e-14
    # row 1: both scores equal 1*sc -> uniform over keys 0, 1
    np.testing.assert_allclose(O[1, 0], [0.5, 0.5], atol=1e-14)
    assert abs(LSE[0, 1] - (sc + math.log(2))) < 1e-14
    # row 0: single key
    np.testing.assert_allclose(O[0, 0], v[0, 0], atol=1e-15)
    assert abs(LSE[0, 0] - sc) < 1e-14


def test_zero_query_gives_causal_mean_and_log_count():
    """x_q = 0 makes every score 0: O[q] = mean(v[0..q]) and LSE = ln(q+1),
    whatever G and w0 are. Pins the causal mask and the softmax sums."""
    L, d = 23, 8
    xq = np.zeros((L, 2, d))
    xk = _rand(5, L, 1, d)
    v = _rand(6, L, 1, d)
    O, LSE = bifocal_attention(xq, xk, v, w0=3, w_pre=4, theta=1e4)
    for q in range(L):
        np.testing.assert_allclose(O[q, 0], v[: q + 1, 0].mean(0), atol=1e-13)
        assert abs(LSE[1, q] - math.log(q + 1)) < 1e-13


# ---------------------------------------------------------------- library reductions
def _sdpa_causal(q, k, v, scale):
    """torch SDPA (fp64, CPU, causal). q: [L,H,d], k/v: [L,H,d] numpy."""
    t = lambda a: torch.from_numpy(np.ascontiguousarray(a.transpose(1, 0, 2)))[None]
    o = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True,
                                                         scale=scale)
    return o[0].numpy().transpose(1, 0, 2)


@pytest.mark.parametrize("L,w_pre,w0", [(48, 64, 5), (64, 64, 0), (40, 8, 39), (40, 3, 100)])
def test_reduces_to_plain_rope_attention(L, w_pre, w0):
    """G = 1 (L <= w_pre) or w0 >= L-1 (every pair local, any G) reduces to
    plain causal RoPE attention [Digest/Method, "Dynamic group size": the base
    model is recovered exactly; Pith review, circularity check]. Compared
    with torch's scaled_dot_product_attention in fp64."""
    Hq, Hkv, d, theta = 4, 2, 16, 1e4
    xq, xk, v = _rand(7, L, Hq, d), _rand(8, L, Hkv, d), _rand(9, L, Hkv, d)
    assert group_size(L, w_pre) == 1 or w0 >= L - 1
    O, _ = bifocal_attention(xq, xk, v, w0, w_pre, theta)
    p = np.arange(L)
    qa, ka = rope(xq, p, theta), rope(xk, p, theta)
    ref = _sdpa_causal(qa, np.repeat(ka, 2, axis=1), np.repeat(v, 2, axis=1), 1 / math.sqrt(d))
    np.testing.assert_allclose(O, ref, atol=1e-12)


def test_remote_only_branch_is_remapped_rope_attention():
    """With w0 = -1 no pair is local: the result is plain causal attention on
    vectors rotated at f(p) = floor(p/G) [Digest/Method, Eq. 1, second
    branch]."""
    L, Hq, Hkv, d, theta, w_pre = 50, 2, 1, 16, 1e4, 16
    G = group_size(L, w_pre)
    assert G == 4
    xq, xk, v = _rand(10, L, Hq, d), _rand(11, L, Hkv, d), _rand(12, L, Hkv, d)
    O, _ = bifocal_attention(xq, xk, v, -1, w_pre, theta)
    f = np.arange(L) // G
    ref = _sdpa_causal(rope(xq, f, theta), np.repeat(rope(xk, f, theta), 2, 1),
                       np.repeat(v, 2, 1), 1 / math.sqrt(d))
    np.testing.assert_allclose(O, ref, atol=1e-12)


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("w0", [0, 1, 3, 7, 16])
@pytest.mark.parametrize("w_pre", [1, 4, 8, 16, 64])
def test_brute_force_agrees(w0, w_pre):
    """Scalar triple loop vs the vectorized oracle, L <= 64, G up to 64."""
    L = 64 if w0 in (0, 16) else 37
    Hq, Hkv, d, theta = 2, 1, 8, 1e4
    xq, xk, v = _rand(13, L, Hq, d), _rand(14, L, Hkv, d), _rand(15, L, Hkv, d)
    O, LSE = bifocal_attention(xq, xk, v, w0, w_pre, theta)
    Ob, Lb = brute_attention(xq.tolist(), xk.tolist(), v.tolist(), w0, w_pre, theta)
    np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)
    np.testing.assert_allclose(LSE, np.array(Lb), atol=1e-12)


def test_varlen_agrees_with_brute_force_per_sequence():
    """Packed sequences restart positions at 0 and take their own G."""
    lens = [5, 19, 33]
    cu = np.cumsum([0] + lens)
    Hq, Hkv, d, theta, w0, w_pre = 2, 1, 8, 1e4, 3, 8
    T = cu[-1]
    xq, xk, v = _rand(16, T, Hq, d), _rand(17, T, Hkv, d), _rand(18, T, Hkv, d)
    res = bifocal_varlen(xq, xk, v, cu, w0, w_pre, theta)
    for b, (rows, O, LSE) in enumerate(res):
        s, e = cu[b], cu[b + 1]
        Ob, Lb = brute_attention(xq[s:e].tolist(), xk[s:e].tolist(), v[s:e].tolist(), w0, w_pre,
                                 theta)
        np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)
        np.testing.assert_allclose(LSE, np.array(Lb), atol=1e-12)


def test_gqa_head_map():
    """Query head h reads KV head h // (Hq/Hkv): heads 2,3 of a 4/2 layout
    equal a 2/1 run on KV head 1 alone (h % Hkv would read KV head 0)."""
    L, d, theta = 30, 8, 1e4
    xq, xk, v = _rand(19, L, 4, d), _rand(20, L, 2, d), _rand(21, L, 2, d)
    O, LSE = bifocal_attention(xq, xk, v, 2, 8, theta)
    O1, L1 = bifocal_attention(xq[:, 2:4], xk[:, 1:2], v[:, 1:2], 2, 8, theta)
    np.testing.assert_allclose(O[:, 2:4], O1, atol=1e-14)
    np.testing.assert_allclose(LSE[2:4], L1, atol=1e-14)


def test_sampled_rows_match_full():
    L, d, theta = 70, 8, 1e6
    xq, xk, v = _rand(22, L, 2, d), _rand(23, L, 1, d), _rand(24, L, 1, d)
    O, LSE = bifocal_attention(xq, xk, v, 5, 16, theta)
    rows = np.array([69, 0, 33, 5, 6, 68])
    Os, Ls = bifocal_attention(xq, xk, v, 5, 16, theta, rows=rows, row_chunk=4)
    np.testing.assert_allclose(Os, O[rows], atol=1e-14)
    np.testing.assert_allclose(Ls, LSE[:, rows], atol=1e-14)


# ---------------------------------------------------------------- Eq. 7
@pytest.mark.parametrize("L,w0,w_pre", [(40, 6, 10), (64, 0, 16), (33, 40, 8), (57, 9, 7)])
def test_inclusion_exclusion_merge_equals_masked(L, w0, w_pre):
    """Eq. 7 applied to passes A (window, absolute), B (causal, remapped) and
    C (window, remapped) equals the direct masked result [Digest/Method,
    "Inclusion-exclusion prefill"; Pith/Ledger Sec. 3.3 Eq. 7]."""
    Hq, Hkv, d, theta = 2, 1, 8, 1e4
    G = group_size(L, w_pre)
    xq, xk, v = _rand(25, L, Hq, d), _rand(26, L, Hkv, d), _rand(27, L, Hkv, d)
    OA, lA = ie_pass(xq, xk, v, "A", w0, G, theta)
    OB, lB = ie_pass(xq, xk, v, "B", w0, G, theta)
    OC, lC = ie_pass(xq, xk, v, "C", w0, G, theta)
    O, LSE = ie_merge(OA, lA, OB, lB, OC, lC)
    Od, Ld = bifocal_attention(xq, xk, v, w0, w_pre, theta)
    np.testing.assert_allclose(O, Od, atol=1e-10)
    np.testing.assert_allclose(LSE, Ld, atol=1e-10)


def test_ie_merge_weights_closed_form():
    """Scalar check of Eq. 7's weights: with O_X constant per pass the merge
    is (wA a + wB b - wC c)/(wA + wB - wC), W = exp(l - max l)."""
    OA, OB, OC = (np.full((1, 1, 1), x) for x in (1.0, 2.0, 3.0))
    lA, lB, lC = (np.full((1, 1), x) for x in (0.5, 1.5, 0.25))
    O, LSE = ie_merge(OA, lA, OB, lB, OC, lC)
    wa, wb, wc = math.exp(-1.0), 1.0, math.exp(-1.25)
    assert abs(O[0, 0, 0] - (wa + 2 * wb - 3 * wc) / (wa + wb - wc)) < 1e-15
    assert abs(LSE[0, 0] - (1.5 + math.log(wa + wb - wc))) < 1e-15


# ---------------------------------------------------------------- decode
@pytest.mark.parametrize("pos", [6, 7, 8, 9, 16, 17, 30])
def test_decode_row_equals_prefill_last_row(pos):
    """decode(p) equals row p of a prefill of length p+1 (L = p+1 during
    decode), across the G flips of w_pre = 8 [Digest/Method, "KV cache
    invariant"]."""
    Hq, Hkv, d, theta, w0, w_pre = 4, 2, 8, 1e4, 3, 8
    C = 40
    xq, xk, v = _rand(28, C, Hq, d), _rand(29, C, Hkv, d), _rand(30, C, Hkv, d)
    o, lse = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta)
    O, LSE = bifocal_attention(xq[: pos + 1], xk[: pos + 1], v[: pos + 1], w0, w_pre, theta,
                               rows=[pos])
    np.testing.assert_allclose(o, O[0], atol=1e-13)
    np.testing.assert_allclose(lse, LSE[:, 0], atol=1e-13)


def test_decode_group_flip_positions():
    """With w_pre = 32768 the step at position 32767 has G = 1 (L = 32768)
    and the step at 32768 has G = 2 (L = 32769); 65537 -> 3; 131071 -> 4."""
    assert [group_size(p + 1, 32768) for p in (32767, 32768, 32769, 65537, 131071)] == \
        [1, 2, 2, 3, 4]


# ---------------------------------------------------------------- invariants
def test_shift_invariance_local_and_remote():
    """Local scores depend on q - k only; remote scores are unchanged when
    every position shifts by a multiple of G (f(p + cG) = f(p) + c) and, for
    G > 1, generally change under a shift of 1."""
    d, theta, G = 16, 1e4, 4
    xq, xk = _rand(31, 6, d), _rand(32, 6, d)
    qp = np.array([100, 101, 102, 103, 104, 105])
    kp = np.array([10, 11, 12, 13, 14, 15])
    big = 10 ** 6
    for c in (1, 7, 64):
        s0 = bifocal_scores(xq, qp, xk, kp, big, G, theta)
        s1 = bifocal_scores(xq, qp + c, xk, kp + c, big, G, theta)
        np.testing.assert_allclose(s0, s1, atol=1e-10)
    r0 = bifocal_scores(xq, qp, xk, kp, -1, G, theta)
    for c in (1, 3, 25):
        r1 = bifocal_scores(xq, qp + c * G, xk, kp + c * G, -1, G, theta)
        np.testing.assert_allclose(r0, r1, atol=1e-10)
    r2 = bifocal_scores(xq, qp + 1, xk, kp + 1, -1, G, theta)
    assert np.abs(r2 - r0).max() > 1e-3


@pytest.mark.parametrize("continuous", [False, True])
def test_scores_match_scalar_brute_force(continuous):
    """bifocal_scores element by element against the scalar definition of
    Eq. 1 [Digest/Method, Eq. 1: local when q - k <= w0, else both vectors at
    f(.)], on positions that put pairs at distances w0 - 1, w0, w0 + 1 and
    far beyond, with G = 1, 2, 3 and keys after queries (the routing is
    defined for any pair; the causal mask is applied elsewhere)."""
    d, theta = 8, 1e4
    xq, xk = _rand(41, 7, d), _rand(42, 9, d)
    qp = np.array([0, 5, 6, 7, 12, 40, 41])
    kp = np.array([0, 1, 2, 3, 4, 5, 6, 11, 39])
    for G in (1, 2, 3):
        for w0 in (0, 1, 3, 5):
            s = bifocal_scores(xq, qp, xk, kp, w0, G, theta, continuous=continuous)
            for i, q in enumerate(qp):
                for j, k in enumerate(kp):
                    ref = brute_score(xq[i], int(q), xk[j], int(k), w0, G, theta, continuous)
                    assert abs(s[i, j] - ref) <= 1e-12 * max(1.0, abs(ref)), (G, w0, q, k)


# ---------------------------------------------------------------- tile classes
def test_tile_class_hand_cases():
    """Hand-checked classes [Digest/Method, Eq. 1 routing condition]."""
    assert tile_class(0, 3, 4, 7, 0) == 0            # all keys after all queries
    assert tile_class(4, 7, 0, 3, 10) == 1           # distances 1..7 <= 10
    assert tile_class(100, 107, 0, 7, 10) == 2       # distances 93..107 > 10
    assert tile_class(10, 13, 0, 3, 10) == 3         # distances 7..13 straddle 10
    assert tile_class(0, 3, 0, 3, 5) == 1 + 4        # diagonal, local
    assert tile_class(0, 7, 0, 7, 2) == 3 + 4        # diagonal, boundary
    assert tile_class(11, 11, 0, 0, 10) == 2         # single pair, distance 11
    assert tile_class(10, 10, 0, 0, 10) == 1         # distance == w0 is local


def test_tile_class_map_ragged():
    m = tile_class_map(10, 4, 3, 2)
    assert m.shape == (3, 4)
    assert m[0, 0] == 3 + 4 and m[0, 2] == 0 and m[2, 0] == 2  # q-k up to 3 > 2 on tile (0,0)
    # last tiles clipped at L-1 = 9: query tile [8, 9], key tile [9, 9] is diagonal+local
    assert m[2, 3] == 1 + 4


# ---------------------------------------------------------------- continuous remote map
# The comparison arm of Table 6 [Pith/Review, major comment 2; ledger axiom
# on the discrete grid]: continuous frequency interpolation in place of
# floor-division aliasing, read as f(x) = x / G with the same G and window.
def test_continuous_remap_values():
    """f(x) = x / G exactly, as a real number, against hand values."""
    np.testing.assert_array_equal(remap([0, 1, 2, 3, 5, 8, 9], 4, continuous=True),
                                  [0.0, 0.25, 0.5, 0.75, 1.25, 2.0, 2.25])
    np.testing.assert_array_equal(remap([0, 7, 131071], 1, continuous=True), [0.0, 7.0, 131071.0])
    assert remap([7], 3, continuous=True).dtype == np.float64


def _freq_scaled_rope(x, pos, theta, factor):
    """Rotation of pair (i, i + d/2) by pos * omega_i / factor, written with
    complex numbers: the frequency-interpolation form (every frequency
    divided by the factor) rather than a remapped position."""
    d = x.shape[-1]
    h = d // 2
    w = theta ** (-(2.0 * np.arange(h)) / d) / factor
    z = (x[..., :h] + 1j * x[..., h:]) * np.exp(1j * np.asarray(pos, float)[:, None, None] * w)
    return np.concatenate([z.real, z.imag], axis=-1)


@pytest.mark.parametrize("w0", [0, -1])
def test_continuous_no_window_is_frequency_interpolation(w0):
    """With no key outside the diagonal in the window (w0 = 0; the diagonal
    has relative angle 0 on both routes) or none at all (w0 = -1), the
    continuous arm is plain causal RoPE attention with every frequency
    divided by G (positional interpolation), checked with torch SDPA."""
    L, Hq, Hkv, d, theta, w_pre = 50, 2, 1, 16, 1e4, 16
    G = group_size(L, w_pre)
    assert G == 4
    xq, xk, v = _rand(40, L, Hq, d), _rand(41, L, Hkv, d), _rand(42, L, Hkv, d)
    O, _ = bifocal_attention(xq, xk, v, w0, w_pre, theta, continuous=True)
    p = np.arange(L)
    ref = _sdpa_causal(_freq_scaled_rope(xq, p, theta, G),
                       np.repeat(_freq_scaled_rope(xk, p, theta, G), 2, 1),
                       np.repeat(v, 2, 1), 1 / math.sqrt(d))
    np.testing.assert_allclose(O, ref, atol=1e-12)


@pytest.mark.parametrize("L,w_pre,w0", [(48, 64, 5), (40, 3, 100)])
def test_continuous_reduces_like_discrete(L, w_pre, w0):
    """G = 1 or an all-local window: both maps give the same result (the
    base model inside the pretrained window)."""
    Hq, Hkv, d, theta = 2, 1, 16, 1e4
    xq, xk, v = _rand(43, L, Hq, d), _rand(44, L, Hkv, d), _rand(45, L, Hkv, d)
    Oc, Lc = bifocal_attention(xq, xk, v, w0, w_pre, theta, continuous=True)
    Od, Ld = bifocal_attention(xq, xk, v, w0, w_pre, theta)
    np.testing.assert_allclose(Oc, Od, atol=1e-13)
    np.testing.assert_allclose(Lc, Ld, atol=1e-13)


@pytest.mark.parametrize("w0,w_pre", [(0, 4), (3, 8), (7, 5), (2, 1)])
def test_continuous_brute_force_agrees(w0, w_pre):
    """Scalar loops with remote pairs at q / G, k / G vs the vectorized oracle;
    and the two maps differ once G > 1 and some pair is remote."""
    L, Hq, Hkv, d, theta = 37, 2, 1, 8, 1e4
    xq, xk, v = _rand(46, L, Hq, d), _rand(47, L, Hkv, d), _rand(48, L, Hkv, d)
    O, LSE = bifocal_attention(xq, xk, v, w0, w_pre, theta, continuous=True)
    Ob, Lb = brute_attention(xq.tolist(), xk.tolist(), v.tolist(), w0, w_pre, theta,
                             continuous=True)
    np.testing.assert_allclose(O, np.array(Ob), atol=1e-12)
    np.testing.assert_allclose(LSE, np.array(Lb), atol=1e-12)
    Od, _ = bifocal_attention(xq, xk, v, w0, w_pre, theta)
    assert np.abs(O - Od).max() > 1e-3


def test_continuous_remote_scores_shift_invariant_by_any_step():
    """Remote scores of the continuous map depend on (q - k) / G only, so any
    integer shift of both positions leaves them unchanged (the floor map
    needs multiples of G)."""
    d, theta, G = 16, 1e4, 4
    xq, xk = _rand(49, 6, d), _rand(50, 6, d)
    qp = np.array([100, 101, 102, 103, 104, 105])
    kp = np.array([10, 11, 12, 13, 14, 15])
    r0 = bifocal_scores(xq, qp, xk, kp, -1, G, theta, continuous=True)
    for c in (1, 3, 17):
        r1 = bifocal_scores(xq, qp + c, xk, kp + c, -1, G, theta, continuous=True)
        np.testing.assert_allclose(r0, r1, atol=1e-10)
    rf0 = bifocal_scores(xq, qp, xk, kp, -1, G, theta)
    rf1 = bifocal_scores(xq, qp + 1, xk, kp + 1, -1, G, theta)
    assert np.abs(rf1 - rf0).max() > 1e-3


@pytest.mark.parametrize("pos", [6, 8, 9, 17, 30])
def test_continuous_decode_row_equals_prefill_last_row(pos):
    """The decode form (keys rotated at their own route, real positions)
    equals row p of the continuous prefill of length p + 1."""
    Hq, Hkv, d, theta, w0, w_pre = 4, 2, 8, 1e4, 3, 8
    C = 40
    xq, xk, v = _rand(51, C, Hq, d), _rand(52, C, Hkv, d), _rand(53, C, Hkv, d)
    o, lse = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta, continuous=True)
    O, LSE = bifocal_attention(xq[: pos + 1], xk[: pos + 1], v[: pos + 1], w0, w_pre, theta,
                               rows=[pos], continuous=True)
    np.testing.assert_allclose(o, O[0], atol=1e-13)
    np.testing.assert_allclose(lse, LSE[:, 0], atol=1e-13)


def test_continuous_correction_rotation_of_cached_keys():
    """R_{k/G - k} applied to a key rotated at k gives the key rotated at
    k / G: the cache stays valid for the continuous map too (rotations by
    real angles compose additively) [Digest/Method, "KV cache invariant"]."""
    d, theta, G = 32, 1e6, 3
    k = np.arange(0, 5000, 7)
    x = _rand(54, len(k), 1, d)
    corr = rope(rope(x, k, theta), k / G - k, theta)
    np.testing.assert_allclose(corr, rope(x, k / G, theta), atol=1e-9)


@pytest.mark.parametrize("L,w0,w_pre", [(40, 6, 10), (57, 9, 7)])
def test_continuous_inclusion_exclusion_equals_masked(L, w0, w_pre):
    """Eq. 7 over the three passes with B and C at x / G equals the direct
    continuous result."""
    Hq, Hkv, d, theta = 2, 1, 8, 1e4
    G = group_size(L, w_pre)
    xq, xk, v = _rand(55, L, Hq, d), _rand(56, L, Hkv, d), _rand(57, L, Hkv, d)
    parts = [ie_pass(xq, xk, v, w, w0, G, theta, continuous=True) for w in "ABC"]
    O, LSE = ie_merge(*parts[0], *parts[1], *parts[2])
    Od, Ld = bifocal_attention(xq, xk, v, w0, w_pre, theta, continuous=True)
    np.testing.assert_allclose(O, Od, atol=1e-10)
    np.testing.assert_allclose(LSE, Ld, atol=1e-10)


# ---------------------------------------------------------------- batched decode
def test_decode_batch_equals_varlen_prefill_last_rows():
    """A batch of packed sequences (gaps between them, G = 1..5 with
    w_pre = 8) decoded at their last positions equals the last row of each
    sequence in a packed varlen prefill (an independent code path); two
    entries share one cache region at different positions (a shared prefix)."""
    Hq, Hkv, d, theta, w0, w_pre = 4, 2, 8, 1e4, 3, 8
    lens = [1, 9, 17, 33, 40]
    gaps = [2, 0, 5, 1, 3]
    starts, rows = [], 0
    for n, g in zip(lens, gaps):
        rows += g
        starts.append(rows)
        rows += n
    xk, v = _rand(60, rows, Hkv, d), _rand(61, rows, Hkv, d)
    xq_rows = _rand(62, rows, Hq, d)
    positions = [n - 1 for n in lens] + [20]
    starts = starts + [starts[-1]]
    xq = np.stack([xq_rows[s0 + p] for s0, p in zip(starts, positions)])
    o, lse = decode_batch(xq, xk, v, positions, starts, w0, w_pre, theta)
    for b, (s0, p) in enumerate(zip(starts, positions)):
        n = p + 1
        O, LSE = bifocal_attention(xq_rows[s0:s0 + n], xk[s0:s0 + n], v[s0:s0 + n], w0, w_pre,
                                   theta, rows=[p])
        np.testing.assert_allclose(o[b], O[0], atol=1e-13)
        np.testing.assert_allclose(lse[b], LSE[:, 0], atol=1e-13)
    assert [group_size(p + 1, w_pre) for p in positions] == [1, 2, 3, 5, 5, 3]


def test_decode_batch_invalid_entries_are_nan():
    """Entries whose keys leave the buffer or pass max_keys get NaN; the
    others are unaffected."""
    Hq, Hkv, d, theta = 2, 1, 8, 1e4
    xk, v = _rand(63, 30, Hkv, d), _rand(64, 30, Hkv, d)
    xq = _rand(65, 5, Hq, d)
    positions, starts = [5, -1, 10, 25, 3], [0, 0, 20, 4, -2]
    o, lse = decode_batch(xq, xk, v, positions, starts, 2, 4, theta, max_keys=20)
    assert np.isnan(o[1]).all() and np.isnan(o[2]).all() and np.isnan(o[3]).all()
    assert np.isnan(o[4]).all() and np.isnan(lse[[1, 2, 3, 4]]).all()
    ref, rl = decode_row(xq[0], xk, v, 5, 2, 4, theta)
    np.testing.assert_allclose(o[0], ref, atol=1e-14)
    np.testing.assert_allclose(lse[0], rl, atol=1e-14)
