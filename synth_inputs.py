"""Seeded synthetic inputs shared by the tests, the smoke check and the bench.

This module holds no attention or RoPE arithmetic: it draws Gaussian arrays,
rounds them to bfloat16 (the values the GPU consumes; the oracle upcasts the
very same values) and picks sampled query rows. Both the oracle and the HIP
path receive what these functions return.

Recipe: numpy.random.default_rng(seed) draws float32 standard normals in the
order x_q, x_k, v, then (for the peaked workload) the permutation choosing
the amplified key rows, then the permutation choosing sampled rows. Workload
c in 1..5 uses seed 1000 + c. The batched-decode workload (seed 1006) draws
each sequence b from its own generator default_rng([seed, b]): its query
row, then its pos_b + 1 key rows and value rows; sequences are packed back to
back in one cache buffer.
"""
from __future__ import annotations

import numpy as np

WORKLOADS = {
    # name: (seed, lengths, Hq, Hkv, d, w_pre, w0, theta, value scale, dtype)
    "tiny_fp32": dict(seed=1001, lengths=[256], Hq=1, Hkv=1, d=64, w_pre=64, w0=16,
                      theta=1e4, std=1.0, dtype="fp32"),
    "prefill_64k": dict(seed=1002, lengths=[65536], Hq=16, Hkv=8, d=128, w_pre=32768, w0=4096,
                        theta=1e6, std=2 ** -0.5, dtype="bf16"),
    "prefill_128k": dict(seed=1003, lengths=[131072], Hq=32, Hkv=8, d=128, w_pre=32768, w0=4096,
                         theta=1e6, std=1.0, dtype="bf16", peaked_frac=0.01, peaked_gain=8.0),
    "decode_128k": dict(seed=1004, lengths=[131072], Hq=32, Hkv=8, d=128, w_pre=32768, w0=4096,
                        theta=1e6, std=1.0, dtype="bf16",
                        decode_positions=[32767, 32768, 32769, 65537, 131071]),
    "varlen_4seq": dict(seed=1005, lengths=[8192, 40960, 73728, 106496], Hq=32, Hkv=8, d=128,
                        w_pre=32768, w0=2048, theta=1e6, std=1.0, dtype="bf16"),
    # 16 sequences decoding at once, positions spread over G = 1..4 (with the
    # G edges 32767 / 32768 and the longest 131071): 906,870 cached keys
    "decode_batch_16": dict(seed=1006, positions=[131071, 4095, 32767, 32768, 98303, 65537, 16383,
                                                  120000, 8191, 49151, 81920, 24575, 110000,
                                                  57343, 73727, 1023],
                            Hq=32, Hkv=8, d=128, w_pre=32768, w0=4096, theta=1e6, std=1.0,
                            dtype="bf16"),
}


def round_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """float32 -> bfloat16 bit patterns (uint16), round to nearest even.
    Inputs are finite Gaussian draws, so NaN handling is not needed."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    bias = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + bias) >> 16).astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns -> the exact float32 values they encode."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def quantize_bf16(x: np.ndarray) -> np.ndarray:
    """Round float32 to the nearest bfloat16 value, returned as float32."""
    return bf16_bits_to_f32(round_to_bf16_bits(x))


def gaussian(rng, shape, std=1.0) -> np.ndarray:
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        a *= np.float32(std)
    return a


def make_qkv(seed, T, Hq, Hkv, d, std=1.0, dtype="bf16", peaked_frac=0.0, peaked_gain=1.0):
    """Draw raw (pre-RoPE) x_q [T,Hq,d], x_k [T,Hkv,d], v [T,Hkv,d].

    dtype 'bf16' rounds every array to bfloat16 values (held as float32 here).
    With peaked_frac > 0, for each KV head a seeded permutation picks
    round(peaked_frac * T) distinct token rows of x_k, which are multiplied
    by peaked_gain (a power of two, so the product stays exactly
    representable). Returns (xq, xk, v, rng) with the generator advanced past
    these draws, for the caller's row sampling.
    """
    rng = np.random.default_rng(seed)
    xq = gaussian(rng, (T, Hq, d), std)
    xk = gaussian(rng, (T, Hkv, d), std)
    v = gaussian(rng, (T, Hkv, d), std)
    if dtype == "bf16":
        xq, xk, v = quantize_bf16(xq), quantize_bf16(xk), quantize_bf16(v)
    if peaked_frac > 0:
        n = int(round(peaked_frac * T))
        for g in range(Hkv):
            idx = rng.permutation(T)[:n]
            xk[idx, g, :] *= np.float32(peaked_gain)
    return xq, xk, v, rng


def make_decode_seq(seed, b, n_keys, Hq, Hkv, d, std=1.0, dtype="bf16"):
    """Sequence b of a batched-decode workload: (xq [Hq, d], xk [n_keys, Hkv, d],
    v [n_keys, Hkv, d]) raw, from default_rng([seed, b]) in that order."""
    rng = np.random.default_rng([seed, b])
    xq = gaussian(rng, (Hq, d), std)
    xk = gaussian(rng, (n_keys, Hkv, d), std)
    v = gaussian(rng, (n_keys, Hkv, d), std)
    if dtype == "bf16":
        xq, xk, v = quantize_bf16(xq), quantize_bf16(xk), quantize_bf16(v)
    return xq, xk, v


def packed_starts(positions, gaps=None):
    """First cache row of each sequence when sequence b's pos_b + 1 rows follow
    the previous sequence's rows (after gaps[b] unused rows, if given);
    returns (starts, total rows)."""
    starts, row = [], 0
    for b, p in enumerate(positions):
        row += 0 if gaps is None else int(gaps[b])
        starts.append(row)
        row += int(p) + 1
    return starts, row


def sample_rows(rng, L, n, must_include):
    """n distinct sequence-relative rows in [0, L): every valid entry of
    must_include first, then a seeded uniform sample of the rest."""
    fixed = sorted({int(r) for r in must_include if 0 <= int(r) < L})
    if len(fixed) >= n or L <= n:
        return np.array(sorted(set(fixed) | set(range(min(L, n)))) if L <= n else fixed[:n],
                        dtype=np.int64)
    pool = np.setdiff1d(np.arange(L, dtype=np.int64), np.array(fixed, dtype=np.int64))
    extra = rng.choice(pool, size=n - len(fixed), replace=False)
    return np.sort(np.concatenate([np.array(fixed, dtype=np.int64), extra]))


def edge_rows(L, w0, w_pre, G, BM, BN):
    """Rows that sit on the edges the method and the kernel tiling create:
    the first rows, the window edge, the pretrained-window edge, the last
    rows, and +-1 around every query-tile, key-tile and G-group boundary
    within the first few tiles and at the end."""
    cand = {0, 1, w0 - 1, w0, w0 + 1, w0 + 2, w_pre - 1, w_pre, w_pre + 1, L - 2, L - 1}
    for step in (BM, BN, G):
        for m in list(range(1, 4)) + [L // step - 1, L // step]:
            e = m * step
            cand.update({e - 1, e, e + 1})
    return sorted(c for c in cand if 0 <= c < L)
