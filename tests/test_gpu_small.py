"""GPU parity at sizes the oracle finishes in seconds: several tiles, ragged
tails, and the degenerate cases (one token, w0 = 0, w0 beyond L, G = 1, an
empty sequence in a packed batch). Every comparison is element by element
against the float64 oracle on the same seeded inputs."""
import math

import numpy as np
import pytest
import torch

import rope_context_extension_jl_amd as jl
from oracle import (bifocal_attention, bifocal_varlen, decode_row, group_size, rope,
                    tile_class, tile_class_map)
from synth_inputs import make_qkv
from tests._gpu_common import (BF16_LSE_ABS, FP32_LSE_ABS, assert_bf16_close, assert_f32_close,
                               errs, note, to_dev, to_host)

pytestmark = pytest.mark.gpu
BIG = 10 ** 9  # a window wider than any sequence: plain causal RoPE attention


# ------------------------------------------------------------------ RoPE
@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("T,H,d,pos_offset,lens", [
    (1000, 3, 128, 0, None), (777, 2, 64, 12345, None), (1300, 4, 128, 0, [5, 0, 700, 595]),
    (64, 1, 256, 131000, None), (500, 6, 128, 7, None)])
def test_rope_apply(dtype, T, H, d, pos_offset, lens):
    theta = 1e6
    x, _, _, _ = make_qkv(7, T, H, 1, d, dtype=dtype)
    cu = None
    pos = np.arange(T) + pos_offset
    if lens is not None:
        cuv = np.cumsum([0] + lens)
        cu = torch.tensor(cuv, dtype=torch.int32, device="cuda")
        pos = np.concatenate([np.arange(n) for n in lens]) + pos_offset
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    note(f"rope_apply {dtype} T={T} H={H} d={d} off={pos_offset} varlen={lens is not None}")
    xt = to_dev(x, tdt)
    jl.rope_apply(xt, theta, cu_seqlens=cu, pos_offset=pos_offset)
    torch.cuda.synchronize()
    ref = rope(x, pos, theta)
    got = to_host(xt)
    if dtype == "bf16":  # one rounding of an fp32 result to bf16
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-6)
    else:
        assert np.abs(got - ref).max() <= 2e-6 * max(1.0, np.abs(ref).max())


# ------------------------------------------------------------------ tile classes
@pytest.mark.parametrize("L", [1, 63, 64, 65, 127, 128, 129, 1000, 4113])
@pytest.mark.parametrize("w0", [0, 1, 63, 64, 100, 4096])
def test_device_tile_classes_bitexact(L, w0):
    bm, bn = jl.prefill_tile_shape()
    note(f"tile dump L={L} w0={w0}")
    dev = jl.debug_tile_classes(L, w0).cpu().numpy()
    ref = tile_class_map(L, bm, bn, w0)
    assert dev.shape == ref.shape
    np.testing.assert_array_equal(dev, ref)


def test_device_tile_classes_128k_sampled():
    L, w0 = 131072, 4096
    bm, bn = jl.prefill_tile_shape()
    note("tile dump 128K")
    dev = jl.debug_tile_classes(L, w0).cpu().numpy()
    rng = np.random.default_rng(3)
    nq = dev.shape[0]
    rows = sorted({0, 1, nq // 32, nq // 32 + 1, nq // 2, nq - 2, nq - 1} |
                  set(rng.integers(0, nq, 24).tolist()))
    for i in rows:
        q0, q1 = i * bm, min(L, (i + 1) * bm) - 1
        cols = set(range(max(0, (q0 - w0) // bn - 3), min(dev.shape[1], q1 // bn + 3)))
        cols |= set(rng.integers(0, dev.shape[1], 40).tolist()) | {0, dev.shape[1] - 1}
        for j in sorted(cols):
            k0, k1 = j * bn, min(L, (j + 1) * bn) - 1
            assert dev[i, j] == tile_class(q0, q1, k0, k1, w0), (i, j)
    # class mix of the 128K workload (causal tiles only)
    live = dev[dev > 0] & 3
    frac = {c: float(np.mean(live == c)) for c in (1, 2, 3)}
    note(f"128K tile mix local {frac[1]:.4f} remote {frac[2]:.4f} boundary {frac[3]:.4f}")
    assert frac[2] > 0.9 and frac[3] < 0.01


# ------------------------------------------------------------------ prefill, fp32
def _oracle(xq, xk, v, w0, w_pre, theta, rows=None):
    return bifocal_attention(xq, xk, v, w0, w_pre, theta, rows=rows)


@pytest.mark.parametrize("L", [256, 64])
@pytest.mark.parametrize("mode", ["fused", "ie", "plain"])
def test_prefill_fp32_tiny(L, mode):
    """Tiny fp32 workload: 1/1 heads, d = 64, w_pre = 64 (G = 4 at L = 256,
    G = 1 at L = 64), w0 = 16, theta = 1e4, N(0,1)."""
    xq, xk, v, _ = make_qkv(1001, 256, 1, 1, 64, dtype="fp32")
    xq, xk, v = xq[:L], xk[:L], v[:L]
    w0, w_pre, theta = 16, 64, 1e4
    note(f"prefill fp32 L={L} mode={mode}")
    o, lse = jl.bifocal_prefill(to_dev(xq, torch.float32), to_dev(xk, torch.float32),
                                to_dev(v, torch.float32), w0, w_pre, theta, mode=mode)
    torch.cuda.synchronize()
    O, LSE = _oracle(xq, xk, v, BIG if mode == "plain" else w0, w_pre, theta)
    assert_f32_close(to_host(o), O, f"fp32 L={L} {mode} O")
    assert_f32_close(to_host(lse), LSE, f"fp32 L={L} {mode} LSE", tol=FP32_LSE_ABS)


def test_prefill_fp32_short_context_is_plain_rope_attention():
    """L <= w_pre gives G = 1 and the bifocal result equals plain RoPE attention."""
    xq, xk, v, _ = make_qkv(1001, 256, 1, 1, 64, dtype="fp32")
    xq, xk, v = (to_dev(a[:64], torch.float32) for a in (xq, xk, v))
    o1, l1 = jl.bifocal_prefill(xq, xk, v, 16, 64, 1e4, mode="fused")
    o2, l2 = jl.bifocal_prefill(xq, xk, v, 16, 64, 1e4, mode="plain")
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)


# ------------------------------------------------------------------ prefill, bf16
SMALL_CASES = [
    # L, Hq, Hkv, w0, w_pre
    (1, 4, 2, 0, 1),
    (37, 4, 2, 5, 8),          # G = 5, one partial tile
    (200, 8, 2, 16, 64),       # G = 4, ragged second query tile
    (777, 4, 4, 100, 256),     # G = 4
    (1500, 8, 2, 300, 1000),   # G = 2
    (1024, 4, 1, 0, 128),      # w0 = 0, G = 8
    (640, 4, 2, 63, 64),       # window edge one short of a key tile
    (640, 4, 2, 64, 64),       # window edge on a key tile
    (2048, 2, 2, 4096, 512),   # w0 beyond L: every pair local
    (513, 16, 2, 127, 100),    # GQA 8:1, G = 6
    (300, 6, 2, 40, 128),      # GQA 3:1 (odd: one head per workgroup), G = 3
    (130, 3, 1, 20, 64),       # odd head count, G = 3
]


@pytest.mark.parametrize("case", SMALL_CASES, ids=[f"L{c[0]}-h{c[1]}x{c[2]}-w{c[3]}-p{c[4]}"
                                                    for c in SMALL_CASES])
@pytest.mark.parametrize("mode", ["fused", "ie", "plain"])
def test_prefill_bf16_small(case, mode):
    L, Hq, Hkv, w0, w_pre = case
    theta = 1e6
    xq, xk, v, _ = make_qkv(2000 + L, L, Hq, Hkv, 128)
    note(f"prefill bf16 L={L} Hq={Hq} Hkv={Hkv} w0={w0} w_pre={w_pre} G={group_size(L, w_pre)} "
         f"mode={mode}")
    o, lse = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), w0, w_pre, theta, mode=mode)
    torch.cuda.synchronize()
    O, LSE = _oracle(xq, xk, v, BIG if mode == "plain" else w0, w_pre, theta)
    assert_bf16_close(to_host(o), O, f"{case} {mode} O")
    mx, _ = errs(to_host(lse), LSE)
    assert mx <= BF16_LSE_ABS, ("LSE", mx)


def _reference_move_inputs(L, Hq, Hkv, d, seed):
    """Inputs whose softmax reference must move inside the walk, not only on
    its first tile: queries are close to one vector u placed on the lowest
    frequency pairs (RoPE turns them by < 0.01 rad over L, at absolute and at
    remapped positions alike), keys 0..63 lie along -u (scores about -64 in
    the log2 domain, the first reference), keys 64..95 score about 57.4 above
    it and keys 96..127 about 65 above it (a lane's 16-key block sum then
    stays below the 2^64 bound in the first block and exceeds it in the
    second), later keys are N(0, 1). After the move at keys 96..127 the keys
    64..95 keep about 0.5% of the weight, so a wrong rescale of the products
    already accumulated shows in every row past them."""
    rng = np.random.default_rng(seed)
    u = np.zeros(d, np.float32)
    u[d // 2 - 4:d // 2] = 5.0  # |u| = 10, on the four lowest-frequency pairs
    uh = u / 10.0
    xq = (u[None, None, :] + 0.05 * rng.standard_normal((L, Hq, d))).astype(np.float32)
    xk = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    b = np.zeros(L, np.float32)
    b[:64], b[64:96], b[96:128] = -5.0, -0.5, 0.1
    xk[:128] = b[:128, None, None] * 10.0 * uh[None, None, :] + 0.01 * xk[:128]
    v = rng.standard_normal((L, Hkv, d)).astype(np.float32)
    q16 = lambda a: torch.from_numpy(a).to(torch.bfloat16).float().numpy()
    return q16(xq), q16(xk), q16(v)


@pytest.mark.parametrize("heads", [(8, 2), (6, 2)], ids=["pair", "one-head"])
@pytest.mark.parametrize("mode", ["fused", "plain"])
def test_prefill_bf16_reference_moves_inside_the_walk(heads, mode):
    """The lazy softmax reference moves on a mask-free tile after the first
    one (rare branch of both mask-free steps, including a move at the second
    32-key block after the first block's products): parity with the oracle."""
    Hq, Hkv = heads
    L, w0, w_pre, theta = 1024, 16, 256, 1e6
    xq, xk, v = _reference_move_inputs(L, Hq, Hkv, 128, 4242)
    note(f"prefill bf16 reference moves L={L} Hq={Hq} Hkv={Hkv} mode={mode}")
    o, lse = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), w0, w_pre, theta, mode=mode)
    torch.cuda.synchronize()
    O, LSE = _oracle(xq, xk, v, BIG if mode == "plain" else w0, w_pre, theta)
    assert_bf16_close(to_host(o), O, f"reference moves {heads} {mode} O")
    mx, _ = errs(to_host(lse), LSE)
    assert mx <= BF16_LSE_ABS, ("LSE", mx)


# Eq. 7 subtracts pass C from pass B. On a row where the window's remapped
# mass (W_C) dwarfs the final mass (W_A + W_B - W_C), the passes' fp32
# rounding is amplified by ratio = (W_B + W_C) / (W_A + W_B - W_C). Rows up
# to RATIO_OK must meet the tolerance (max and mean); the others are checked
# on their own below.
RATIO_OK = 1e3
_PEAKED = {}


def _peaked_small():
    """1% of key rows x8 (peaked softmax), G = 4, every third row: inputs,
    oracle, and the GPU's fused and Eq. 7 outputs (computed once)."""
    if not _PEAKED:
        L, Hq, Hkv, w0, w_pre, theta = 4096, 8, 2, 256, 1024, 1e6
        xq, xk, v, _ = make_qkv(3001, L, Hq, Hkv, 128, peaked_frac=0.01, peaked_gain=8.0)
        rows = np.arange(0, L, 3)
        O, LSE = _oracle(xq, xk, v, w0, w_pre, theta, rows=rows)
        note("peaked prefill mode=fused")
        o, lse = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), w0, w_pre, theta)
        torch.cuda.synchronize()
        note("peaked prefill mode=ie")
        ws = torch.empty(jl.prefill_workspace_size(L, 1, Hq, Hkv, 128, mode="ie"),
                         dtype=torch.uint8, device="cuda")
        oi, _ = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), w0, w_pre, theta,
                                   mode="ie", workspace=ws)
        torch.cuda.synchronize()
        ratio = to_host(jl.ie_ratio_view(ws, L, 1, Hq, Hkv, 128))[:, rows].T  # [rows, Hq]
        _PEAKED.update(rows=rows, O=O, LSE=LSE, o=to_host(o)[rows], lse=to_host(lse)[:, rows],
                       oi=to_host(oi)[rows], ratio=ratio)
    return _PEAKED


def test_prefill_bf16_peaked_small():
    """The fused pass on every sampled row; Eq. 7 on the rows whose
    cancellation ratio is at most RATIO_OK."""
    p = _peaked_small()
    assert_bf16_close(p["o"], p["O"], "peaked fused O")
    assert errs(p["lse"], p["LSE"])[0] <= BF16_LSE_ABS
    diff = np.abs(p["oi"] - p["O"])   # [rows, Hq, d]
    ok = p["ratio"] <= RATIO_OK       # [rows, Hq]
    note(f"ie: worst ratio {p['ratio'].max():.3e}, pairs over {RATIO_OK:g}: {int((~ok).sum())}, "
         f"max-abs where ratio<=bound {diff[ok].max():.3e}, mean {diff[ok].mean():.3e}")
    assert diff[ok].max() <= 2e-2 and diff[ok].mean() <= 2e-3


@pytest.mark.xfail(strict=True, reason="Eq. 7 cancels catastrophically on rows whose "
                   "cancellation ratio exceeds 1e3 (errors up to ~2.4 on this peaked case); "
                   "the fused pass is the production path")
def test_prefill_bf16_peaked_small_ie_cancelling_rows():
    """Eq. 7 on the rows whose cancellation ratio exceeds RATIO_OK, at the
    same tolerance."""
    p = _peaked_small()
    bad = p["ratio"] > RATIO_OK
    err = np.abs(p["oi"] - p["O"]).max(axis=2)
    worst = float(err[bad].max()) if bad.any() else 0.0
    note(f"ie, ratio > {RATIO_OK:g}: {int(bad.sum())} (row, head) pairs, worst max-abs "
         f"{worst:.3e}, worst ratio {p['ratio'].max():.3e}")
    assert worst <= 2e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_prefill_varlen_small(dtype):
    lens = [5, 0, 300, 129, 1000, 64]
    Hq, Hkv, w0, w_pre, theta = 4, 2, 40, 128, 1e6
    d = 128 if dtype == "bf16" else 64
    T = sum(lens)
    xq, xk, v, _ = make_qkv(4001, T, Hq, Hkv, d, dtype=dtype)
    cu = torch.tensor(np.cumsum([0] + lens), dtype=torch.int32, device="cuda")
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    ref = bifocal_varlen(xq, xk, v, np.cumsum([0] + lens), w0, w_pre, theta)
    for mode in ("fused", "ie", "plain"):
        note(f"varlen {dtype} mode={mode} lens={lens}")
        o, lse = jl.bifocal_prefill(to_dev(xq, tdt), to_dev(xk, tdt), to_dev(v, tdt), w0, w_pre,
                                    theta, mode=mode, cu_seqlens=cu)
        torch.cuda.synchronize()
        oh, lh = to_host(o), to_host(lse)
        if mode == "plain":
            ref = bifocal_varlen(xq, xk, v, np.cumsum([0] + lens), BIG, w_pre, theta)
        s = 0
        for b, (rows, O, LSE) in enumerate(ref):
            n = lens[b]
            if n:
                if dtype == "bf16":
                    assert_bf16_close(oh[s:s + n], O, f"varlen seq {b} {mode}")
                else:
                    assert_f32_close(oh[s:s + n], O, f"varlen seq {b} {mode}")
                assert errs(lh[:, s:s + n], LSE)[0] <= (BF16_LSE_ABS if dtype == "bf16"
                                                         else FP32_LSE_ABS)
            s += n


def test_prefill_varlen_max_sequences():
    """The largest packed batch the boundary accepts: 4096 sequences of 0..48
    tokens (every 97th empty), each with its own G (1..6). The plan kernel's
    per-sequence arrays and its sort are full. Compared over all rows."""
    rng = np.random.default_rng(4096)
    lens = rng.integers(0, 49, 4096)
    lens[::97] = 0
    Hq, Hkv, w0, w_pre, theta = 4, 2, 5, 8, 1e6
    T = int(lens.sum())
    cu_h = np.cumsum([0] + list(lens))
    xq, xk, v, _ = make_qkv(4097, T, Hq, Hkv, 128, dtype="bf16")
    cu = torch.tensor(cu_h, dtype=torch.int32, device="cuda")
    for mode in ("fused", "plain"):
        note(f"varlen 4096 sequences mode={mode} T={T}")
        ref = bifocal_varlen(xq, xk, v, cu_h, BIG if mode == "plain" else w0, w_pre, theta)
        o_ref = np.concatenate([O for _, O, _ in ref if O.shape[0]], axis=0)
        l_ref = np.concatenate([L for _, _, L in ref if L.shape[-1]], axis=1)
        o, lse = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), w0, w_pre, theta,
                                    mode=mode, cu_seqlens=cu)
        torch.cuda.synchronize()
        assert_bf16_close(to_host(o), o_ref, f"4096 sequences {mode}")
        assert errs(to_host(lse), l_ref)[0] <= BF16_LSE_ABS


def test_kcache_out_equals_rope_apply_and_inputs_untouched():
    L, Hq, Hkv, theta = 1000, 4, 2, 1e6
    xq, xk, v, _ = make_qkv(5001, L, Hq, Hkv, 128)
    q, k, vv = to_dev(xq), to_dev(xk), to_dev(v)
    k0, q0, v0 = k.clone(), q.clone(), vv.clone()
    kc = torch.empty_like(k)
    note("kcache_out")
    jl.bifocal_prefill(q, k, vv, 64, 256, theta, kcache_out=kc)
    k2 = k.clone()
    jl.rope_apply(k2, theta)
    torch.cuda.synchronize()
    assert torch.equal(kc, k2)
    assert torch.equal(k, k0) and torch.equal(q, q0) and torch.equal(vv, v0)


def test_prefill_is_deterministic():
    L, Hq, Hkv = 3000, 8, 2
    xq, xk, v, _ = make_qkv(6001, L, Hq, Hkv, 128)
    q, k, vv = to_dev(xq), to_dev(xk), to_dev(v)
    note("determinism")
    a = jl.bifocal_prefill(q, k, vv, 100, 512, 1e6)
    b = jl.bifocal_prefill(q, k, vv, 100, 512, 1e6)
    torch.cuda.synchronize()
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])


# ------------------------------------------------------------------ decode
def _decode_setup(dtype, C=3000, Hq=8, Hkv=2, d=128, seed=7001):
    xq, xk, v, _ = make_qkv(seed, C, Hq, Hkv, d, dtype=dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    kc = to_dev(xk, tdt)
    jl.rope_apply(kc, 1e6)  # the absolute cache
    return xq, xk, v, kc, to_dev(v, tdt), tdt


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_small_positions(dtype):
    w0, w_pre, theta = 100, 512, 1e6
    d = 128 if dtype == "bf16" else 64
    xq, xk, v, kc, vc, tdt = _decode_setup(dtype, d=d)
    k_before = kc.clone()
    for pos in (0, 1, 100, 101, 511, 512, 513, 1023, 1024, 1500, 2999):
        for mode in ("fused", "plain"):
            note(f"decode {dtype} pos={pos} G={group_size(pos + 1, w_pre)} mode={mode}")
            o, lse = jl.bifocal_decode(to_dev(xq[pos], tdt), kc, vc, pos, w0, w_pre, theta,
                                       mode=mode)
            torch.cuda.synchronize()
            ro, rl = decode_row(xq[pos], xk, v, pos, BIG if mode == "plain" else w0, w_pre, theta)
            if dtype == "bf16":
                assert_bf16_close(to_host(o), ro, f"decode pos={pos} {mode}")
                assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS
            else:
                assert_f32_close(to_host(o), ro, f"decode pos={pos} {mode}")
                assert errs(to_host(lse), rl)[0] <= FP32_LSE_ABS
    torch.cuda.synchronize()
    assert torch.equal(kc, k_before), "decode wrote the cache"


@pytest.mark.parametrize("cont", [False, True])
def test_decode_bf16_group_sizes_past_16(cont):
    """G from 15 to 47 (w_pretrained = 64): for G above 16 every 16-key step of
    f(k) - k is -16 or -15 (floor(16 / G) = 0, a carry whenever (k mod G) + 16
    >= G), for G = 16 it is exactly -15, for G = 15 -15 or -14; most keys are
    remote (w0 = 50). Split counts 1 and 7 change which chunk starts a split."""
    w0, w_pre, theta = 50, 64, 1e6
    xq, xk, v, kc, vc, tdt = _decode_setup("bf16")
    for pos in (959, 1023, 1024, 1087, 1100, 2047, 2999):
        G = group_size(pos + 1, w_pre)
        for splits in (0, 1, 7):
            note(f"decode bf16 pos={pos} G={G} splits={splits} continuous={cont}")
            o, lse = jl.bifocal_decode(to_dev(xq[pos], tdt), kc, vc, pos, w0, w_pre, theta,
                                       mode="fused", num_splits=splits,
                                       remap="continuous" if cont else "floor")
            torch.cuda.synchronize()
            ro, rl = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta, continuous=cont)
            assert_bf16_close(to_host(o), ro, f"decode pos={pos} G={G} splits={splits}")
            assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


@pytest.mark.parametrize("Hq,Hkv,d", [(2, 2, 128), (4, 2, 128), (16, 2, 128), (8, 2, 64),
                                       (8, 8, 64), (12, 6, 128)])
def test_decode_bf16_head_ratios_and_dims(Hq, Hkv, d):
    """Every GQA ratio the boundary accepts and both head dims, remote and
    local keys, a ragged last chunk (pos + 1 not a multiple of 64)."""
    w0, w_pre, theta = 100, 512, 1e6
    xq, xk, v, _ = make_qkv(7100 + Hq + d, 1400, Hq, Hkv, d)
    kc = to_dev(xk)
    jl.rope_apply(kc, theta)
    vc = to_dev(v)
    for pos in (0, 63, 64, 150, 1023, 1399):
        for mode in ("fused", "plain"):
            note(f"decode bf16 Hq={Hq} Hkv={Hkv} d={d} pos={pos} {mode}")
            o, lse = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta, mode=mode)
            torch.cuda.synchronize()
            ro, rl = decode_row(xq[pos], xk, v, pos, BIG if mode == "plain" else w0, w_pre, theta)
            assert_bf16_close(to_host(o), ro, f"decode pos={pos} {mode}")
            assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


def test_decode_split_count_invariance():
    w0, w_pre, theta, pos = 100, 512, 1e6, 2500
    xq, xk, v, kc, vc, tdt = _decode_setup("bf16")
    ro, _ = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta)
    outs = []
    for s in (1, 2, 7, 40, 47):
        note(f"decode splits={s}")
        o, _ = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta, num_splits=s)
        torch.cuda.synchronize()
        outs.append(to_host(o))
        assert_bf16_close(outs[-1], ro, f"splits={s}")
    for o in outs[1:]:
        assert np.abs(o - outs[0]).max() <= 8e-3


def test_decode_matches_prefill_last_row():
    """decode(p) equals row p of a prefill of length p + 1 (both on the GPU)."""
    w0, w_pre, theta = 100, 512, 1e6
    xq, xk, v, kc, vc, tdt = _decode_setup("bf16")
    for pos in (700, 1024, 2047):
        note(f"decode vs prefill pos={pos}")
        L = pos + 1
        o_p, l_p = jl.bifocal_prefill(to_dev(xq[:L]), to_dev(xk[:L]), to_dev(v[:L]), w0, w_pre,
                                      theta)
        o_d, l_d = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta)
        torch.cuda.synchronize()
        assert np.abs(to_host(o_p)[pos] - to_host(o_d)).max() <= 1.6e-2
        assert np.abs(to_host(l_p)[:, pos] - to_host(l_d)).max() <= 1.6e-2


# ------------------------------------------------- prefill continued on a cache
def _cache(seed, C, Hq, Hkv, theta, d=128):
    """Raw inputs of a C-row sequence and its absolute bf16 key cache."""
    xq, xk, v, _ = make_qkv(seed, C, Hq, Hkv, d)
    kc = to_dev(xk)
    jl.rope_apply(kc, theta)
    return xq, xk, v, kc, to_dev(v)


@pytest.mark.parametrize("q_off,Tq,w0,w_pre", [
    (0, 700, 100, 512),      # a whole sequence read from the cache (G = 2)
    (1000, 300, 100, 512),   # a chunk in the middle, L = 1300 (G = 3)
    (1024, 1, 100, 512),     # one row: a decode step at pos 1024
    (900, 124, 64, 512),     # L = 1024 exactly (G = 2)
    (1000, 50, 100, 512),    # L = 1050: the chunk moves G from 2 to 3
    (1537, 263, 0, 600),     # w0 = 0, ragged chunk, G = 3
])
def test_prefill_cached_matches_oracle(q_off, Tq, w0, w_pre):
    theta, Hq, Hkv = 1e6, 8, 2
    L = q_off + Tq
    C = L + 37  # rows past L hold other keys: they must not be read
    xq, xk, v, kc, vc = _cache(7300 + L, C, Hq, Hkv, theta)
    k_before = kc.clone()
    for mode in ("fused", "plain"):
        note(f"prefill_cached q_off={q_off} Tq={Tq} w0={w0} G={group_size(L, w_pre)} {mode}")
        o, lse = jl.bifocal_prefill_cached(to_dev(xq[q_off:L]), kc, vc, q_off, w0, w_pre, theta,
                                           mode=mode)
        torch.cuda.synchronize()
        O, LSE = bifocal_attention(xq[:L], xk[:L], v[:L], BIG if mode == "plain" else w0, w_pre,
                                   theta, rows=np.arange(q_off, L))
        assert_bf16_close(to_host(o), O, f"cached q_off={q_off} Tq={Tq} {mode}")
        assert errs(to_host(lse), LSE)[0] <= BF16_LSE_ABS
    torch.cuda.synchronize()
    assert torch.equal(kc, k_before), "prefill_cached wrote the cache"


def test_prefill_cached_agrees_with_prefill_and_decode():
    """GPU against GPU: a cached chunk covering the whole sequence equals the
    ordinary prefill, and a one-row chunk equals the decode step, within the
    rounding of the bf16 cache."""
    theta, w0, w_pre, L = 1e6, 100, 512, 1500
    xq, xk, v, kc, vc = _cache(7400, L, 8, 2, theta)
    note("prefill_cached vs prefill, whole sequence")
    o_c, l_c = jl.bifocal_prefill_cached(to_dev(xq), kc, vc, 0, w0, w_pre, theta)
    o_p, l_p = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), w0, w_pre, theta)
    torch.cuda.synchronize()
    assert np.abs(to_host(o_c) - to_host(o_p)).max() <= 1.6e-2
    assert np.abs(to_host(l_c) - to_host(l_p)).max() <= 1.6e-2
    for pos in (1023, 1024, 1499):
        note(f"prefill_cached one row vs decode pos={pos}")
        o_1, l_1 = jl.bifocal_prefill_cached(to_dev(xq[pos:pos + 1]), kc, vc, pos, w0, w_pre, theta)
        o_d, l_d = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta)
        torch.cuda.synchronize()
        assert np.abs(to_host(o_1)[0] - to_host(o_d)).max() <= 1.6e-2
        assert np.abs(to_host(l_1)[:, 0] - to_host(l_d)).max() <= 1.6e-2


# ------------------------------------------------------------------ fp16 range
@pytest.mark.parametrize("where", ["none", "query", "key", "both"])
def test_prefill_range_flags(where):
    """Operands outside the fp16 range are reported, not faulted on: a raw
    query row of 2e5 (rotated components reach ~2.8e5 > 65504) sets
    FLAG_Q_RANGE, a key row of 1e6 (times the score scale log2(e)/sqrt(128),
    1.3e5 > 65504) sets FLAG_K_RANGE; in-range inputs leave both clear. The
    same holds for the prefill continued on a cache (keys taken from it)."""
    L, Hq, Hkv, w0, w_pre, theta = 300, 4, 2, 40, 128, 1e6
    xq, xk, v, _ = make_qkv(5001, L, Hq, Hkv, 128)
    if where in ("query", "both"):
        xq[200, 1, :] = 2e5
    if where in ("key", "both"):
        xk[17, 0, :] = 1e6
    want = {"none": 0, "query": jl.FLAG_Q_RANGE, "key": jl.FLAG_K_RANGE,
            "both": jl.FLAG_Q_RANGE | jl.FLAG_K_RANGE}[where]
    q, k, vv = to_dev(xq), to_dev(xk), to_dev(v)
    ws = torch.empty(jl.prefill_workspace_size(L, 1, Hq, Hkv, 128), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0xff)  # stale contents: every call clears the flags first
    kc = torch.empty_like(k)
    note(f"prefill range flags, out-of-range {where}")
    o, _ = jl.bifocal_prefill(q, k, vv, w0, w_pre, theta, workspace=ws, kcache_out=kc)
    torch.cuda.synchronize()
    assert jl.prefill_flags(ws) == want
    if where == "none":
        assert torch.isfinite(o.float()).all()
    note(f"cached prefill range flags, out-of-range {where}")
    wsc = torch.empty(jl.prefill_cached_workspace_size(100, L - 100, Hq, Hkv, 128),
                      dtype=torch.uint8, device="cuda")
    wsc.fill_(0xff)
    jl.bifocal_prefill_cached(q[100:].contiguous(), kc, vv, 100, w0, w_pre, theta, workspace=wsc)
    torch.cuda.synchronize()
    assert jl.prefill_flags(wsc) == want


# ------------------------------------------------------------------ decode workspace, fp16 range
def test_decode_workspace_reuse():
    """One workspace with stale contents serves any number of calls, at any
    position and split count; each result equals a call with a fresh
    workspace, bit for bit, and the oracle within the tolerance."""
    w0, w_pre, theta = 100, 512, 1e6
    xq, xk, v, kc, vc, tdt = _decode_setup("bf16")
    Hq = xq.shape[1]
    ws = torch.empty(jl.decode_workspace_size(kc.shape[0], Hq, 128), dtype=torch.uint8,
                     device="cuda")
    ws.fill_(0x5a)
    for pos, splits in ((2999, 0), (700, 3), (1500, 0), (2999, 40), (40, 0), (2999, 0)):
        note(f"decode workspace reuse pos={pos} splits={splits}")
        o1, l1 = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta,
                                   num_splits=splits, workspace=ws)
        o2, l2 = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta,
                                   num_splits=splits)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)
        ro, _ = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta)
        assert_bf16_close(to_host(o1), ro, f"reuse pos={pos}")


def test_workspace_of_any_dtype():
    """The binding passes a workspace's size in bytes (numel times element
    size): a float32 workspace of just enough elements serves decode and
    prefill, with the same results bit for bit as a uint8 workspace."""
    w0, w_pre, theta = 100, 512, 1e6
    xq, xk, v, kc, vc, tdt = _decode_setup("bf16")
    Hq = xq.shape[1]
    pos = 2999
    need = jl.decode_workspace_size(kc.shape[0], Hq, 128)
    ws32 = torch.empty((need + 3) // 4, dtype=torch.float32, device="cuda")
    note(f"decode with a float32 workspace of {ws32.numel()} elements ({need} bytes needed)")
    o1, l1 = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta, workspace=ws32)
    o2, l2 = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2) and torch.equal(l1, l2)
    T, Hkv = 300, kc.shape[1]
    q, k, vv = to_dev(xq[:T]), to_dev(xk[:T]), to_dev(v[:T])
    needp = jl.prefill_workspace_size(T, 1, Hq, Hkv, 128)
    wsp = torch.empty((needp + 1) // 2, dtype=torch.bfloat16, device="cuda")
    note(f"prefill with a bfloat16 workspace of {wsp.numel()} elements ({needp} bytes needed)")
    p1, s1 = jl.bifocal_prefill(q, k, vv, w0, w_pre, theta, workspace=wsp)
    p2, s2 = jl.bifocal_prefill(q, k, vv, w0, w_pre, theta)
    torch.cuda.synchronize()
    assert torch.equal(p1, p2) and torch.equal(s1, s2)


@pytest.mark.parametrize("where", ["key", "query"])
def test_decode_out_of_fp16_range_gives_nan(where):
    """A cached key beyond the fp16 range (1e6), or a query whose scaled
    rotation exceeds it (4e6 x scale log2 e), makes the outputs and LSE of
    the query heads of that KV head NaN; the other heads are unaffected and
    nothing faults. Single and batched decode."""
    w0, w_pre, theta, pos = 100, 512, 1e6, 1200
    Hq, Hkv = 8, 4
    xq, xk, v, _ = make_qkv(7301, 1400, Hq, Hkv, 128)
    bad = 1  # KV head 1 (query heads 2 and 3)
    if where == "key":
        xk[300, bad, :] = 1e6
    else:
        xq[pos, 2, :] = 4e6
    kc = to_dev(xk)
    jl.rope_apply(kc, theta)
    vc = to_dev(v)
    note(f"decode out-of-range {where}")
    o, lse = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta)
    torch.cuda.synchronize()
    oh, lh = to_host(o), to_host(lse)
    assert np.isnan(oh[2:4]).all() and np.isnan(lh[2:4]).all()
    good = [h for h in range(Hq) if h not in (2, 3)]
    ro, _ = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta)
    assert_bf16_close(oh[good], ro[good], f"decode out-of-range {where}, other heads")
    note(f"batched decode out-of-range {where}")
    pos_t = torch.tensor([pos, 900], dtype=torch.int32, device="cuda")
    st_t = torch.tensor([0, 0], dtype=torch.int32, device="cuda")
    xb = to_dev(np.stack([xq[pos], xq[900]]))
    ob, lb = jl.bifocal_decode_batch(xb, kc, vc, pos_t, st_t, pos + 1, w0, w_pre, theta)
    torch.cuda.synchronize()
    obh = to_host(ob)
    assert np.isnan(obh[0, 2:4]).all()
    assert np.isfinite(obh[0, good]).all()
    if where == "key":  # the second sequence reads the same key 300
        assert np.isnan(obh[1, 2:4]).all()
    else:
        assert np.isfinite(obh[1]).all()
