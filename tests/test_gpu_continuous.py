"""GPU parity of the continuous remote map (remote positions x / G as real
numbers, the frequency-interpolation arm the aliasing map is compared with
in the Table 6 discussion of the pith.science review) against the float64
oracle with continuous=True, for every path that has a remote branch:
prefill (fused and Eq. 7, bf16 and fp32), decode (bf16 and fp32) and
prefill continued on a cache. Sizes span several tiles and ragged tails."""
import numpy as np
import pytest
import torch

import rope_context_extension_jl_amd as jl
from oracle import bifocal_attention, decode_row, group_size
from synth_inputs import make_qkv
from tests._gpu_common import (BF16_LSE_ABS, FP32_LSE_ABS, assert_bf16_close, assert_f32_close,
                               errs, note, to_dev, to_host)

pytestmark = pytest.mark.gpu

CASES = [
    # L, Hq, Hkv, w0, w_pre
    (37, 4, 2, 5, 8),          # G = 5, one partial tile
    (777, 4, 4, 100, 256),     # G = 4
    (1500, 8, 2, 300, 1000),   # G = 2
    (1024, 4, 1, 0, 128),      # w0 = 0, G = 8
    (640, 4, 2, 64, 64),       # window edge on a key tile, G = 10
    (513, 16, 2, 127, 100),    # GQA 8:1, G = 6
]


@pytest.mark.parametrize("case", CASES, ids=[f"L{c[0]}-h{c[1]}x{c[2]}-w{c[3]}-p{c[4]}"
                                              for c in CASES])
@pytest.mark.parametrize("mode", ["fused", "ie"])
def test_prefill_bf16_continuous(case, mode):
    L, Hq, Hkv, w0, w_pre = case
    theta = 1e6
    xq, xk, v, _ = make_qkv(2500 + L, L, Hq, Hkv, 128)
    note(f"prefill bf16 continuous L={L} Hq={Hq} Hkv={Hkv} w0={w0} G={group_size(L, w_pre)} "
         f"mode={mode}")
    o, lse = jl.bifocal_prefill(to_dev(xq), to_dev(xk), to_dev(v), w0, w_pre, theta, mode=mode,
                                remap="continuous")
    torch.cuda.synchronize()
    O, LSE = bifocal_attention(xq, xk, v, w0, w_pre, theta, continuous=True)
    assert_bf16_close(to_host(o), O, f"{case} {mode} continuous O")
    assert errs(to_host(lse), LSE)[0] <= BF16_LSE_ABS


@pytest.mark.parametrize("mode", ["fused", "ie"])
def test_prefill_fp32_continuous(mode):
    """fp32 path, d = 64 and 128, G = 4 and 3."""
    for L, d, w_pre in ((256, 64, 64), (300, 128, 100)):
        xq, xk, v, _ = make_qkv(2600 + L, L, 2, 1, d, dtype="fp32")
        note(f"prefill fp32 continuous L={L} d={d} mode={mode}")
        o, lse = jl.bifocal_prefill(to_dev(xq, torch.float32), to_dev(xk, torch.float32),
                                    to_dev(v, torch.float32), 16, w_pre, 1e4, mode=mode,
                                    remap="continuous")
        torch.cuda.synchronize()
        O, LSE = bifocal_attention(xq, xk, v, 16, w_pre, 1e4, continuous=True)
        assert_f32_close(to_host(o), O, f"fp32 L={L} {mode} continuous O")
        assert_f32_close(to_host(lse), LSE, f"fp32 L={L} {mode} continuous LSE", tol=FP32_LSE_ABS)


def test_continuous_equals_floor_at_g1_and_differs_beyond():
    """G = 1: x / 1 and floor(x / 1) are the same positions, so the two maps
    give bitwise the same output; with G > 1 they must differ."""
    xq, xk, v, _ = make_qkv(2700, 900, 4, 2, 128)
    q, k, vv = to_dev(xq), to_dev(xk), to_dev(v)
    note("continuous vs floor, G = 1 and G = 3")
    a, la = jl.bifocal_prefill(q, k, vv, 50, 1024, 1e6)
    b, lb = jl.bifocal_prefill(q, k, vv, 50, 1024, 1e6, remap="continuous")
    c, _ = jl.bifocal_prefill(q, k, vv, 50, 300, 1e6)
    e, _ = jl.bifocal_prefill(q, k, vv, 50, 300, 1e6, remap="continuous")
    torch.cuda.synchronize()
    assert torch.equal(a, b) and torch.equal(la, lb)
    assert (c.float() - e.float()).abs().max().item() > 1e-2


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_decode_continuous(dtype):
    w0, w_pre, theta = 100, 512, 1e6
    d = 128 if dtype == "bf16" else 64
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    xq, xk, v, _ = make_qkv(7600, 2000, 8, 2, d, dtype=dtype)
    kc = to_dev(xk, tdt)
    jl.rope_apply(kc, theta)
    vc = to_dev(v, tdt)
    for pos in (0, 100, 101, 511, 512, 513, 1025, 1999):
        note(f"decode {dtype} continuous pos={pos} G={group_size(pos + 1, w_pre)}")
        o, lse = jl.bifocal_decode(to_dev(xq[pos], tdt), kc, vc, pos, w0, w_pre, theta,
                                   remap="continuous")
        torch.cuda.synchronize()
        ro, rl = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta, continuous=True)
        if dtype == "bf16":
            assert_bf16_close(to_host(o), ro, f"decode continuous pos={pos}")
            assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS
        else:
            assert_f32_close(to_host(o), ro, f"decode continuous pos={pos}")
            assert errs(to_host(lse), rl)[0] <= FP32_LSE_ABS


@pytest.mark.parametrize("Hq,Hkv,d", [(4, 2, 128), (8, 8, 64)])
def test_decode_bf16_continuous_heads_and_dims(Hq, Hkv, d):
    w0, w_pre, theta = 64, 256, 1e6
    xq, xk, v, _ = make_qkv(7700 + Hq + d, 1300, Hq, Hkv, d)
    kc = to_dev(xk)
    jl.rope_apply(kc, theta)
    vc = to_dev(v)
    for pos in (63, 300, 1299):
        note(f"decode bf16 continuous Hq={Hq} Hkv={Hkv} d={d} pos={pos}")
        o, lse = jl.bifocal_decode(to_dev(xq[pos]), kc, vc, pos, w0, w_pre, theta,
                                   remap="continuous")
        torch.cuda.synchronize()
        ro, rl = decode_row(xq[pos], xk, v, pos, w0, w_pre, theta, continuous=True)
        assert_bf16_close(to_host(o), ro, f"decode continuous pos={pos}")
        assert errs(to_host(lse), rl)[0] <= BF16_LSE_ABS


@pytest.mark.parametrize("q_off,Tq,w0,w_pre", [(1000, 300, 100, 512), (1537, 263, 0, 600),
                                              (1024, 1, 100, 512)])
def test_prefill_cached_continuous(q_off, Tq, w0, w_pre):
    theta, Hq, Hkv = 1e6, 8, 2
    L = q_off + Tq
    xq, xk, v, _ = make_qkv(7800 + L, L + 11, Hq, Hkv, 128)
    kc = to_dev(xk)
    jl.rope_apply(kc, theta)
    vc = to_dev(v)
    note(f"prefill_cached continuous q_off={q_off} Tq={Tq} G={group_size(L, w_pre)}")
    o, lse = jl.bifocal_prefill_cached(to_dev(xq[q_off:L]), kc, vc, q_off, w0, w_pre, theta,
                                       remap="continuous")
    torch.cuda.synchronize()
    O, LSE = bifocal_attention(xq[:L], xk[:L], v[:L], w0, w_pre, theta,
                               rows=np.arange(q_off, L), continuous=True)
    assert_bf16_close(to_host(o), O, f"cached continuous q_off={q_off} Tq={Tq}")
    assert errs(to_host(lse), LSE)[0] <= BF16_LSE_ABS
