"""GPU parity at the full workload sizes, in the launch configuration the
benchmark times (default tiles, automatic decode splits), on sampled rows
the float64 oracle computes one by one.

Workloads (synthetic stand-ins for the Qwen3-shaped long-context setting the
pages measure on; seeds 1002..1005, see synth_inputs.WORKLOADS):
  prefill_64k  : L=65536, Hq/Hkv=16/8, d=128, w_pre=32768 (G=2), w0=4096
  prefill_128k : L=131072, Hq/Hkv=32/8, G=4, w0=4096, 1% of key rows x8
  decode_128k  : 131072-key absolute cache, steps at 32767..131071
  decode_batch_16 : 16 sequences decoding together, positions 1023..131071
                 (G = 1..4), 906,870 keys packed in one cache buffer
  varlen_4seq  : 8192/40960/73728/106496 packed, G = 1..4, w0=2048
Rows: 512 per head (per sequence for varlen), always including the window,
pretrained-window, tile and G-group edges; the rest a seeded uniform draw.
"""
import gc

import numpy as np
import pytest
import torch

import rope_context_extension_jl_amd as jl
from oracle import bifocal_attention, decode_batch, decode_row, group_size, rope
from synth_inputs import (WORKLOADS, edge_rows, make_decode_seq, make_qkv, packed_starts,
                          quantize_bf16, sample_rows)
from tests._gpu_common import BF16_LSE_ABS, assert_bf16_close, errs, note, to_dev, to_host

pytestmark = pytest.mark.gpu
NROWS = 512


def _rows(rng, L, w0, w_pre):
    bm, bn = jl.prefill_tile_shape()
    return sample_rows(rng, L, NROWS, edge_rows(L, w0, w_pre, group_size(L, w_pre), bm, bn))


class _Prefill:
    """Inputs, sampled rows and GPU outputs (fused and IE) of one workload."""

    def __init__(self, name, modes=("fused",)):
        cfg = WORKLOADS[name]
        L = cfg["lengths"][0]
        self.cfg, self.L = cfg, L
        self._oracle = {}
        self.xq, self.xk, self.v, rng = make_qkv(
            cfg["seed"], L, cfg["Hq"], cfg["Hkv"], cfg["d"], cfg["std"], cfg["dtype"],
            cfg.get("peaked_frac", 0.0), cfg.get("peaked_gain", 1.0))
        self.rows = _rows(rng, L, cfg["w0"], cfg["w_pre"])
        q, k, v = to_dev(self.xq), to_dev(self.xk), to_dev(self.v)
        self.out = {}
        for key in modes:
            # "<mode>" or "<mode>-continuous" (remote positions x / G, real)
            mode, _, remap = key.partition("-")
            note(f"{name}: GPU prefill mode={mode} remap={remap or 'floor'}")
            ws = torch.empty(jl.prefill_workspace_size(L, 1, cfg["Hq"], cfg["Hkv"], cfg["d"],
                                                       mode=mode), dtype=torch.uint8,
                             device="cuda")
            o, lse = jl.bifocal_prefill(q, k, v, cfg["w0"], cfg["w_pre"], cfg["theta"], mode=mode,
                                        workspace=ws, remap=remap or "floor")
            torch.cuda.synchronize()
            ratio = None
            if mode == "ie":
                ratio = to_host(jl.ie_ratio_view(ws, L, 1, cfg["Hq"], cfg["Hkv"], cfg["d"]))
                ratio = ratio[:, self.rows]
            self.out[key] = (to_host(o[self.rows]), to_host(lse)[:, self.rows], ratio)
            del o, lse, ws
        del q, k, v
        torch.cuda.empty_cache()

    def oracle(self, g, continuous=False):
        """fp64 oracle for the query heads of KV group g on the sampled rows
        (computed once per group and map)."""
        key = (g, continuous)
        if key not in self._oracle:
            c = self.cfg
            r = c["Hq"] // c["Hkv"]
            hs = slice(g * r, (g + 1) * r)
            self._oracle[key] = bifocal_attention(
                self.xq[:, hs], self.xk[:, g:g + 1], self.v[:, g:g + 1], c["w0"], c["w_pre"],
                c["theta"], rows=self.rows, continuous=continuous)
        return self._oracle[key]


@pytest.fixture(scope="module")
def p64k():
    d = _Prefill("prefill_64k", modes=("fused", "ie"))
    yield d
    del d
    gc.collect()


@pytest.fixture(scope="module")
def p128k():
    d = _Prefill("prefill_128k", modes=("fused", "ie", "fused-continuous"))
    yield d
    del d
    gc.collect()


@pytest.mark.parametrize("g", range(8))
def test_prefill_64k(p64k, g):
    r = p64k.cfg["Hq"] // p64k.cfg["Hkv"]
    O, LSE = p64k.oracle(g)
    for mode in ("fused", "ie"):
        o, lse, _ = p64k.out[mode]
        assert_bf16_close(o[:, g * r:(g + 1) * r], O, f"64K kv{g} {mode}")
        assert errs(lse[g * r:(g + 1) * r], LSE)[0] <= BF16_LSE_ABS


@pytest.mark.parametrize("g", range(8))
def test_prefill_128k(p128k, g):
    r = p128k.cfg["Hq"] // p128k.cfg["Hkv"]
    O, LSE = p128k.oracle(g)
    o, lse, _ = p128k.out["fused"]
    assert_bf16_close(o[:, g * r:(g + 1) * r], O, f"128K kv{g} fused")
    assert errs(lse[g * r:(g + 1) * r], LSE)[0] <= BF16_LSE_ABS
    # Eq. 7 alternative on the rows whose cancellation ratio
    # (W_B + W_C) / (W_A + W_B - W_C) is at most 1e3: the same tolerance,
    # max and mean. The other rows are checked (and fail) in
    # test_prefill_128k_ie_cancelling_rows.
    o_ie, _, ratio = p128k.out["ie"]
    diff = np.abs(o_ie[:, g * r:(g + 1) * r] - O)  # [rows, r, d]
    ok = ratio[g * r:(g + 1) * r].T <= RATIO_OK    # [rows, r]
    note(f"128K kv{g} ie, ratio <= {RATIO_OK:g}: {ok.sum()} (row, head) pairs, max-abs "
         f"{diff[ok].max():.3e} mean-abs {diff[ok].mean():.3e}")
    assert diff[ok].max() <= 2e-2 and diff[ok].mean() <= 2e-3


# Eq. 7 subtracts the window's remapped pass C from the remapped pass B. On a
# row where a window key's remapped score dominates, W_B and W_C are nearly
# equal and much larger than the result's mass W_A + W_B - W_C; the passes'
# fp32 rounding is then amplified by that ratio. About 0.9% of the 128K rows
# (1% of the keys x8) exceed 1e3, with errors up to ~1e5 on some of them: the
# formula, evaluated in floating point as the pages give it, does not meet
# the tolerance there. The fused pass has no subtraction and meets it on
# every row.
RATIO_OK = 1e3


@pytest.mark.xfail(strict=True, reason="Eq. 7 cancels catastrophically on rows whose "
                   "cancellation ratio exceeds 1e3 (peaked 128K workload); the fused pass is "
                   "the production path")
def test_prefill_128k_ie_cancelling_rows(p128k):
    r = p128k.cfg["Hq"] // p128k.cfg["Hkv"]
    o_ie, _, ratio = p128k.out["ie"]
    worst, count = 0.0, 0
    for g in range(p128k.cfg["Hkv"]):
        O, _ = p128k.oracle(g)
        err = np.abs(o_ie[:, g * r:(g + 1) * r] - O).max(axis=2)  # [rows, r]
        bad = ratio[g * r:(g + 1) * r].T > RATIO_OK
        count += int(bad.sum())
        if bad.any():
            worst = max(worst, float(err[bad].max()))
    note(f"128K ie, ratio > {RATIO_OK:g}: {count} (row, head) pairs of "
         f"{ratio.size}, worst max-abs {worst:.3e}")
    assert worst <= 2e-2, f"{count} pairs with ratio > {RATIO_OK:g}, worst error {worst:.3e}"


@pytest.mark.parametrize("g", [0, 3, 7])
def test_prefill_128k_continuous(p128k, g):
    """The continuous remote map (x / G, real) at 128K, G = 4, three KV groups."""
    r = p128k.cfg["Hq"] // p128k.cfg["Hkv"]
    O, LSE = p128k.oracle(g, continuous=True)
    o, lse, _ = p128k.out["fused-continuous"]
    assert_bf16_close(o[:, g * r:(g + 1) * r], O, f"128K kv{g} fused continuous")
    assert errs(lse[g * r:(g + 1) * r], LSE)[0] <= BF16_LSE_ABS


# ------------------------------------------------------------------ varlen
@pytest.fixture(scope="module")
def pvar():
    c = WORKLOADS["varlen_4seq"]
    lens = c["lengths"]
    T = sum(lens)
    xq, xk, v, rng = make_qkv(c["seed"], T, c["Hq"], c["Hkv"], c["d"], c["std"], c["dtype"])
    cu_np = np.cumsum([0] + lens)
    rows = [_rows(rng, n, c["w0"], c["w_pre"]) for n in lens]
    cu = torch.tensor(cu_np, dtype=torch.int32, device="cuda")
    note("varlen_4seq: GPU prefill")
    o, lse = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), c["w0"], c["w_pre"],
                                c["theta"], cu_seqlens=cu)
    torch.cuda.synchronize()
    oh, lh = o.float().cpu(), lse.cpu()
    picked = [(to_host(oh[cu_np[b] + rows[b]]), lh[:, cu_np[b] + rows[b]].double().numpy())
              for b in range(len(lens))]
    del o, lse, oh, lh
    torch.cuda.empty_cache()
    yield dict(c=c, xq=xq, xk=xk, v=v, cu=cu_np, rows=rows, out=picked)


@pytest.mark.parametrize("b", range(4))
def test_prefill_varlen(pvar, b):
    c, cu = pvar["c"], pvar["cu"]
    s, e = cu[b], cu[b + 1]
    note(f"varlen seq {b}: L={e - s} G={group_size(e - s, c['w_pre'])}")
    O, LSE = bifocal_attention(pvar["xq"][s:e], pvar["xk"][s:e], pvar["v"][s:e], c["w0"],
                               c["w_pre"], c["theta"], rows=pvar["rows"][b])
    o, lse = pvar["out"][b]
    assert_bf16_close(o, O, f"varlen seq {b}")
    assert errs(lse, LSE)[0] <= BF16_LSE_ABS


# ------------------------------------------------------------------ decode
@pytest.fixture(scope="module")
def dec():
    c = WORKLOADS["decode_128k"]
    C = c["lengths"][0]
    xq, xk, v, _ = make_qkv(c["seed"], C, c["Hq"], c["Hkv"], c["d"], c["std"], c["dtype"])
    kc = to_dev(xk)
    note("decode_128k: building the absolute cache")
    jl.rope_apply(kc, c["theta"])
    vc = to_dev(v)
    torch.cuda.synchronize()
    yield dict(c=c, xq=xq, xk=xk, v=v, kc=kc, vc=vc, ksum=float(kc.float().sum()))
    del kc, vc
    torch.cuda.empty_cache()


@pytest.mark.parametrize("pos", WORKLOADS["decode_128k"]["decode_positions"])
def test_decode_128k(dec, pos):
    c = dec["c"]
    note(f"decode pos={pos} G={group_size(pos + 1, c['w_pre'])}")
    o, lse = jl.bifocal_decode(to_dev(dec["xq"][pos]), dec["kc"], dec["vc"], pos, c["w0"],
                               c["w_pre"], c["theta"])
    torch.cuda.synchronize()
    ro, rl = decode_row(dec["xq"][pos], dec["xk"], dec["v"], pos, c["w0"], c["w_pre"], c["theta"])
    assert_bf16_close(to_host(o), ro, f"decode pos={pos}")
    assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


@pytest.mark.parametrize("pos", [32768, 65537, 131071])
def test_decode_128k_continuous(dec, pos):
    c = dec["c"]
    note(f"decode continuous pos={pos} G={group_size(pos + 1, c['w_pre'])}")
    o, lse = jl.bifocal_decode(to_dev(dec["xq"][pos]), dec["kc"], dec["vc"], pos, c["w0"],
                               c["w_pre"], c["theta"], remap="continuous")
    torch.cuda.synchronize()
    ro, rl = decode_row(dec["xq"][pos], dec["xk"], dec["v"], pos, c["w0"], c["w_pre"], c["theta"],
                        continuous=True)
    assert_bf16_close(to_host(o), ro, f"decode continuous pos={pos}")
    assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


def test_decode_128k_plain_and_splits(dec):
    c, pos = dec["c"], 131071
    q = to_dev(dec["xq"][pos])
    note("decode plain pos=131071")
    o, _ = jl.bifocal_decode(q, dec["kc"], dec["vc"], pos, c["w0"], c["w_pre"], c["theta"],
                             mode="plain")
    torch.cuda.synchronize()
    ro, _ = decode_row(dec["xq"][pos], dec["xk"], dec["v"], pos, 10 ** 9, c["w_pre"], c["theta"])
    assert_bf16_close(to_host(o), ro, "decode plain 131071")
    ref = None
    for s in (1, 33, 128, 1024):
        note(f"decode splits={s}")
        o, _ = jl.bifocal_decode(q, dec["kc"], dec["vc"], pos, c["w0"], c["w_pre"], c["theta"],
                                 num_splits=s)
        torch.cuda.synchronize()
        oh = to_host(o)
        ref = oh if ref is None else ref
        assert np.abs(oh - ref).max() <= 8e-3
    assert float(dec["kc"].float().sum()) == dec["ksum"], "decode wrote the cache"


# ------------------------------------------------- prefill continued on a cache
def test_prefill_cached_128k_last_chunk(p128k):
    """The last 8192 rows of the 128K workload as one chunk on an absolute
    cache of all 131072 keys (G = 4), in the launch configuration bench.py
    times, against the oracle on sampled rows of the chunk.

    For this path the cache is the input: it holds the keys rotated at their
    absolute positions and rounded to bf16, a rounding the raw-key oracle
    does not see (on this workload's x8 key rows it alone moves outputs by
    several 1e-2). The cache is therefore built here on the CPU, with the
    oracle's rotation, and the oracle is evaluated on the keys it holds:
    R_{-k} applied in float64 to each cached row (exact up to float64)."""
    c = p128k.cfg
    L, Tq = p128k.L, 8192
    q_off = L - Tq
    pos = np.arange(L)
    cache = quantize_bf16(rope(p128k.xk, pos, c["theta"]).astype(np.float32))
    xk_eff = rope(cache, -pos, c["theta"])
    kc, vc = to_dev(cache), to_dev(p128k.v)
    note("prefill_cached 128K last 8192 rows")
    o, lse = jl.bifocal_prefill_cached(to_dev(p128k.xq[q_off:]), kc, vc, q_off, c["w0"],
                                       c["w_pre"], c["theta"])
    torch.cuda.synchronize()
    rng = np.random.default_rng(77)
    rows = np.unique(np.concatenate([[q_off, q_off + 1, L - 1],
                                     q_off + rng.choice(Tq, 61, replace=False)]))
    oh, lh = to_host(o[rows - q_off]), to_host(lse)[:, rows - q_off]
    del o, lse, kc, vc
    torch.cuda.empty_cache()
    O, LSE = bifocal_attention(p128k.xq, xk_eff, p128k.v, c["w0"], c["w_pre"], c["theta"],
                               rows=rows)
    assert_bf16_close(oh, O, "128K cached chunk")
    assert errs(lh, LSE)[0] <= BF16_LSE_ABS


# ------------------------------------------------------------------ batched decode
def test_decode_batch_16_workload():
    """All 16 sequences of the batched-decode workload in one launch (the
    configuration the benchmark times), every entry against the oracle."""
    c = WORKLOADS["decode_batch_16"]
    pos = c["positions"]
    starts, rows = packed_starts(pos)
    Hq, Hkv, d = c["Hq"], c["Hkv"], c["d"]
    k_rows = np.empty((rows, Hkv, d), dtype=np.float32)
    v_rows = np.empty((rows, Hkv, d), dtype=np.float32)
    xq = np.empty((len(pos), Hq, d), dtype=np.float32)
    for b, (p, s0) in enumerate(zip(pos, starts)):
        xq[b], k_rows[s0:s0 + p + 1], v_rows[s0:s0 + p + 1] = make_decode_seq(
            c["seed"], b, p + 1, Hq, Hkv, d, c["std"], c["dtype"])
    kc = to_dev(k_rows)
    for p, s0 in zip(pos, starts):
        jl.rope_apply(kc[s0:s0 + p + 1], c["theta"])
    vc = to_dev(v_rows)
    note(f"decode_batch_16: B={len(pos)} rows={rows}")
    o, lse = jl.bifocal_decode_batch(
        to_dev(xq), kc, vc, torch.tensor(pos, dtype=torch.int32, device="cuda"),
        torch.tensor(starts, dtype=torch.int32, device="cuda"), max(pos) + 1, c["w0"], c["w_pre"],
        c["theta"])
    torch.cuda.synchronize()
    oh, lh = to_host(o), to_host(lse)
    del kc, vc, o, lse
    torch.cuda.empty_cache()
    ro, rl = decode_batch(xq, k_rows, v_rows, pos, starts, c["w0"], c["w_pre"], c["theta"])
    assert_bf16_close(oh, ro, "decode_batch_16")
    assert errs(lh, rl)[0] <= BF16_LSE_ABS
