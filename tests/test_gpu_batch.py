"""GPU parity of batched decode (B sequences in one launch, each with its own
position, L = pos + 1 and G, on one shared cache buffer) against the float64
oracle, at sizes the oracle finishes in seconds: mixed positions across the G
edges, gaps between the packed sequences filled with large values (a misread
row shows), a shared prefix, every GQA ratio class, both head dims, fp32,
invalid entries, the split count, and agreement with the single-sequence
entry point."""
import numpy as np
import pytest
import torch

import rope_context_extension_jl_amd as jl
from oracle import decode_batch, group_size
from synth_inputs import make_decode_seq, make_qkv, packed_starts
from tests._gpu_common import (BF16_LSE_ABS, FP32_LSE_ABS, assert_bf16_close, assert_f32_close,
                               errs, note, to_dev, to_host)

pytestmark = pytest.mark.gpu
BIG = 10 ** 9


def _batch(seed, positions, Hq, Hkv, d, theta, dtype="bf16", gaps=None, share=()):
    """Raw per-sequence inputs packed into one buffer, the device cache (keys
    rotated at their absolute positions by jl_rope_apply per sequence) and
    the int32 index arrays. `share`: (b, b2) pairs where entry b reads the
    rows of entry b2 (a shared prefix) instead of rows of its own."""
    starts, rows = packed_starts(positions, gaps)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    k_rows = np.full((rows, Hkv, d), 300.0, dtype=np.float32)  # gap rows: never read
    v_rows = np.full((rows, Hkv, d), 300.0, dtype=np.float32)
    xq = np.zeros((len(positions), Hq, d), dtype=np.float32)
    for b, (p, s0) in enumerate(zip(positions, starts)):
        q, k, v = make_decode_seq(seed, b, p + 1, Hq, Hkv, d, dtype=dtype)
        xq[b] = q
        k_rows[s0:s0 + p + 1] = k
        v_rows[s0:s0 + p + 1] = v
    kc = to_dev(k_rows, tdt)
    for p, s0 in zip(positions, starts):
        jl.rope_apply(kc[s0:s0 + p + 1], theta)
    for b, b2 in share:
        starts[b] = starts[b2]
    pos_t = torch.tensor(positions, dtype=torch.int32, device="cuda")
    st_t = torch.tensor(starts, dtype=torch.int32, device="cuda")
    return xq, k_rows, v_rows, starts, kc, to_dev(v_rows, tdt), pos_t, st_t, tdt


POS = [0, 1, 100, 511, 512, 513, 1023, 1500, 64, 2047]


@pytest.mark.parametrize("mode,remap", [("fused", "floor"), ("plain", "floor"),
                                        ("fused", "continuous")])
def test_decode_batch_bf16(mode, remap):
    w0, w_pre, theta, Hq, Hkv, d = 100, 512, 1e6, 8, 2, 128
    gaps = [3, 0, 17, 1, 0, 64, 5, 0, 2, 9]
    xq, k_rows, v_rows, starts, kc, vc, pos_t, st_t, tdt = _batch(8100, POS, Hq, Hkv, d, theta,
                                                                 gaps=gaps)
    note(f"decode_batch bf16 B={len(POS)} mode={mode} remap={remap} "
         f"G={[group_size(p + 1, w_pre) for p in POS]}")
    o, lse = jl.bifocal_decode_batch(to_dev(xq), kc, vc, pos_t, st_t, max(POS) + 1, w0, w_pre,
                                     theta, mode=mode, remap=remap)
    torch.cuda.synchronize()
    ro, rl = decode_batch(xq, k_rows, v_rows, POS, starts, BIG if mode == "plain" else w0, w_pre,
                          theta, continuous=remap == "continuous")
    assert_bf16_close(to_host(o), ro, f"decode_batch {mode} {remap}")
    assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


def test_decode_batch_bf16_group_sizes_past_16():
    """w_pretrained = 64: entries with G = 1 .. 47 in one launch (for G above 16
    every 16-key step of f(k) - k is -16 or -15), most keys remote (w0 = 50)."""
    w0, w_pre, theta, Hq, Hkv, d = 50, 64, 1e6, 8, 2, 128
    positions = [30, 959, 1023, 1024, 1100, 2047, 2999, 600]
    xq, k_rows, v_rows, starts, kc, vc, pos_t, st_t, tdt = _batch(8150, positions, Hq, Hkv, d,
                                                                 theta, gaps=[2] * 8)
    note(f"decode_batch bf16 G={[group_size(p + 1, w_pre) for p in positions]}")
    o, lse = jl.bifocal_decode_batch(to_dev(xq), kc, vc, pos_t, st_t, max(positions) + 1, w0,
                                     w_pre, theta)
    torch.cuda.synchronize()
    ro, rl = decode_batch(xq, k_rows, v_rows, positions, starts, w0, w_pre, theta)
    assert_bf16_close(to_host(o), ro, "decode_batch G past 16")
    assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


@pytest.mark.parametrize("Hq,Hkv,d", [(2, 2, 128), (4, 2, 128), (16, 2, 128), (8, 2, 64),
                                       (8, 8, 64), (12, 6, 128)])
def test_decode_batch_heads_and_dims(Hq, Hkv, d):
    w0, w_pre, theta = 64, 256, 1e6
    pos = [63, 1299, 255, 256, 700]
    xq, k_rows, v_rows, starts, kc, vc, pos_t, st_t, _ = _batch(8200 + Hq + d, pos, Hq, Hkv, d,
                                                               theta, gaps=[1, 2, 3, 4, 5])
    note(f"decode_batch bf16 Hq={Hq} Hkv={Hkv} d={d}")
    o, lse = jl.bifocal_decode_batch(to_dev(xq), kc, vc, pos_t, st_t, 1300, w0, w_pre, theta)
    torch.cuda.synchronize()
    ro, rl = decode_batch(xq, k_rows, v_rows, pos, starts, w0, w_pre, theta)
    assert_bf16_close(to_host(o), ro, f"decode_batch Hq={Hq} Hkv={Hkv} d={d}")
    assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


@pytest.mark.parametrize("d", [64, 128])
def test_decode_batch_fp32(d):
    w0, w_pre, theta = 100, 512, 1e6
    pos = [0, 511, 512, 1400, 77]
    xq, k_rows, v_rows, starts, kc, vc, pos_t, st_t, tdt = _batch(8300 + d, pos, 4, 2, d, theta,
                                                                 dtype="fp32", gaps=[0, 4, 0, 8, 1])
    for remap in ("floor", "continuous"):
        note(f"decode_batch fp32 d={d} remap={remap}")
        o, lse = jl.bifocal_decode_batch(to_dev(xq, tdt), kc, vc, pos_t, st_t, 1401, w0, w_pre,
                                         theta, remap=remap)
        torch.cuda.synchronize()
        ro, rl = decode_batch(xq, k_rows, v_rows, pos, starts, w0, w_pre, theta,
                              continuous=remap == "continuous")
        assert_f32_close(to_host(o), ro, f"decode_batch fp32 d={d} {remap}")
        assert errs(to_host(lse), rl)[0] <= FP32_LSE_ABS


def test_decode_batch_shared_prefix_and_invalid_entries():
    """Entry 3 reads the rows of entry 1 at a shorter position (a shared
    prefix); entries whose keys would leave the buffer or pass max_keys come
    back NaN and leave the others intact."""
    w0, w_pre, theta, Hq, Hkv, d = 50, 256, 1e6, 4, 2, 128
    pos = [300, 900, 40, 600]
    xq, k_rows, v_rows, starts, kc, vc, pos_t, st_t, _ = _batch(8400, pos, Hq, Hkv, d, theta,
                                                               share=[(3, 1)])
    note("decode_batch shared prefix")
    o, lse = jl.bifocal_decode_batch(to_dev(xq), kc, vc, pos_t, st_t, 901, w0, w_pre, theta,
                                     num_splits=8)
    torch.cuda.synchronize()
    ro, rl = decode_batch(xq, k_rows, v_rows, pos, starts, w0, w_pre, theta)
    assert_bf16_close(to_host(o), ro, "decode_batch shared prefix")
    rows = k_rows.shape[0]
    bad_pos = pos + [-1, 10, 901, 5]
    bad_st = starts + [0, rows - 5, 0, -3]
    xq2 = np.concatenate([xq, xq[:4]])
    note("decode_batch with invalid entries")
    o2, l2 = jl.bifocal_decode_batch(to_dev(xq2), kc, vc,
                                     torch.tensor(bad_pos, dtype=torch.int32, device="cuda"),
                                     torch.tensor(bad_st, dtype=torch.int32, device="cuda"), 901,
                                     w0, w_pre, theta, num_splits=8)
    torch.cuda.synchronize()
    oh, lh = to_host(o2), to_host(l2)
    assert np.isnan(oh[4:]).all() and np.isnan(lh[4:]).all()
    ro2, _ = decode_batch(xq2, k_rows, v_rows, bad_pos, bad_st, w0, w_pre, theta, max_keys=901)
    assert np.isnan(ro2[4:]).all()
    assert_bf16_close(oh[:4], ro2[:4], "valid entries beside invalid ones")
    assert np.array_equal(oh[:4], to_host(o)), "invalid entries changed the valid ones"


def test_decode_batch_split_invariance_and_single_agreement():
    """num_splits changes only the LSE merge order; each entry agrees with the
    single-sequence entry point on its own cache slice: bitwise when the
    plans match (one sequence whose max_keys is its own pos + 1) and both
    evaluate every correction angle directly; to rounding when G divides 16,
    where the single-sequence kernel derives a chunk's second 16-key block of
    angles from its first by a fixed rotation."""
    w0, w_pre, theta, Hq, Hkv, d = 100, 512, 1e6, 8, 2, 128
    pos = [2500, 1023, 1024, 7]
    xq, k_rows, v_rows, starts, kc, vc, pos_t, st_t, _ = _batch(8500, pos, Hq, Hkv, d, theta,
                                                               gaps=[0, 3, 3, 3])
    ro, _ = decode_batch(xq, k_rows, v_rows, pos, starts, w0, w_pre, theta)
    ref = None
    for s in (0, 1, 3, 17, 40):
        note(f"decode_batch splits={s}")
        o, _ = jl.bifocal_decode_batch(to_dev(xq), kc, vc, pos_t, st_t, 2501, w0, w_pre, theta,
                                       num_splits=s)
        torch.cuda.synchronize()
        oh = to_host(o)
        assert_bf16_close(oh, ro, f"splits={s}")
        ref = oh if ref is None else ref
        assert np.abs(oh - ref).max() <= 8e-3
    for b, (p, s0) in enumerate(zip(pos, starts)):
        note(f"decode_batch B=1 vs decode pos={p}")
        one, l1 = jl.bifocal_decode_batch(to_dev(xq[b:b + 1]), kc, vc, pos_t[b:b + 1],
                                          st_t[b:b + 1], p + 1, w0, w_pre, theta)
        single, ls = jl.bifocal_decode(to_dev(xq[b]), kc[s0:s0 + p + 1], vc[s0:s0 + p + 1], p,
                                       w0, w_pre, theta)
        torch.cuda.synchronize()
        G = group_size(p + 1, w_pre)
        if G == 1 or 16 % G:
            assert torch.equal(one[0], single) and torch.equal(l1[0], ls)
        else:
            d_o = np.abs(to_host(one[0]) - to_host(single)).max()
            d_l = np.abs(to_host(l1[0]) - to_host(ls)).max()
            note(f"B=1 vs single pos={p} G={G}: |dO| {d_o:.3e} |dLSE| {d_l:.3e}")
            assert d_o <= 4e-3 and d_l <= 1e-3


def test_decode_batch_many_sequences():
    """B = 2500 short sequences (more entries than the plan kernel's 1024
    threads, so each thread scans several), positions 0 .. 300 drawn at
    random, every 97th entry invalid; checked on a sample of entries plus
    all invalid ones."""
    w0, w_pre, theta, Hq, Hkv, d = 20, 64, 1e6, 4, 2, 64
    rng = np.random.default_rng(8600)
    B = 2500
    pos = [int(p) for p in rng.integers(0, 301, B)]
    xq, k_rows, v_rows, starts, kc, vc, pos_t, st_t, _ = _batch(8600, pos, Hq, Hkv, d, theta)
    rows = k_rows.shape[0]
    bad = list(range(0, B, 97))
    pos_b, st_b = list(pos), list(starts)
    for i in bad:
        st_b[i] = rows - 1 if i % 2 else -1  # past the buffer, or a negative start
    note(f"decode_batch B={B} rows={rows}")
    o, lse = jl.bifocal_decode_batch(to_dev(xq), kc, vc,
                                     torch.tensor(pos_b, dtype=torch.int32, device="cuda"),
                                     torch.tensor(st_b, dtype=torch.int32, device="cuda"), 301,
                                     w0, w_pre, theta)
    torch.cuda.synchronize()
    oh, lh = to_host(o), to_host(lse)
    for i in bad:
        if pos_b[i] + st_b[i] >= rows or st_b[i] < 0:
            assert np.isnan(oh[i]).all() and np.isnan(lh[i]).all(), i
    sample = sorted(set(rng.choice([i for i in range(B) if i not in bad], 120, replace=False)))
    ro, rl = decode_batch(xq[sample], k_rows, v_rows, [pos[i] for i in sample],
                          [starts[i] for i in sample], w0, w_pre, theta)
    assert_bf16_close(oh[sample], ro, f"decode_batch B={B} sample")
    assert errs(lh[sample], rl)[0] <= BF16_LSE_ABS


def test_decode_batch_max_sequences():
    """The largest batch the boundary accepts: B = 65535 sequences with caches
    of 1 .. 16 keys packed back to back, every 997th entry invalid (its start
    past the buffer); all invalid entries and a sample of the rest checked."""
    w0, w_pre, theta, Hq, Hkv, d = 3, 4, 1e6, 2, 1, 64
    rng = np.random.default_rng(65535)
    B = 65535
    pos = [int(p) for p in rng.integers(0, 16, B)]
    starts, rows = packed_starts(pos)
    _, k_rows, v_rows, _ = make_qkv(65536, rows, 1, Hkv, d, dtype="bf16")
    xq, _, _, _ = make_qkv(65537, B, Hq, 1, d, dtype="bf16")
    kc = to_dev(k_rows)
    jl.rope_apply(kc, theta, cu_seqlens=torch.tensor(starts + [rows], dtype=torch.int32,
                                                     device="cuda"))
    bad = list(range(0, B, 997))
    st_b = list(starts)
    for i in bad:
        st_b[i] = rows  # past the buffer
    note(f"decode_batch B={B} rows={rows}")
    o, lse = jl.bifocal_decode_batch(to_dev(xq), kc, to_dev(v_rows),
                                     torch.tensor(pos, dtype=torch.int32, device="cuda"),
                                     torch.tensor(st_b, dtype=torch.int32, device="cuda"), 16,
                                     w0, w_pre, theta)
    torch.cuda.synchronize()
    oh, lh = to_host(o), to_host(lse)
    for i in bad:
        assert np.isnan(oh[i]).all() and np.isnan(lh[i]).all(), i
    good = np.setdiff1d(np.arange(B), bad)
    sample = sorted(set(rng.choice(good, 200, replace=False).tolist()) | {int(good[0]),
                                                                         int(good[-1])})
    ro, rl = decode_batch(xq[sample], k_rows, v_rows, [pos[i] for i in sample],
                          [starts[i] for i in sample], w0, w_pre, theta)
    assert_bf16_close(oh[sample], ro, f"decode_batch B={B} sample")
    assert errs(lh[sample], rl)[0] <= BF16_LSE_ABS
