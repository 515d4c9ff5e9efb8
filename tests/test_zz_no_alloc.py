"""The decode entry point that allocates nothing (jl_bifocal_decode_noalloc,
for callers that cannot allocate device memory) against the workspace entry
point jl_bifocal_decode: two calls in a row through the C ABI, the second at
a smaller position, each equal to the workspace call bit for bit and to the
float64 oracle within the bf16 tolerance."""
import ctypes

import numpy as np
import pytest
import torch

import rope_context_extension_jl_amd as jl
from oracle import decode_row
from synth_inputs import make_qkv
from tests._gpu_common import assert_bf16_close, note, to_dev, to_host

pytestmark = pytest.mark.gpu


def _noalloc(xq, kc, vc, pos, w0, w_pre, theta, mode="fused"):
    Hq, d = xq.shape
    C, Hkv, _ = kc.shape
    o = torch.empty_like(xq)
    lse = torch.empty((Hq,), dtype=torch.float32, device=xq.device)
    st = jl.lib().jl_bifocal_decode_noalloc(
        ctypes.c_void_p(xq.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
        ctypes.c_void_p(vc.data_ptr()), ctypes.c_void_p(o.data_ptr()),
        ctypes.c_void_p(lse.data_ptr()), int(pos), C, Hq, Hkv, d, int(w0), int(w_pre),
        float(theta), 0.0, 0, jl.MODES[mode], 0,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0, jl.status_string(st)
    return o, lse


def test_decode_noalloc_matches_workspace_entry():
    w0, w_pre, theta = 4096, 32768, 1e6
    Hq, Hkv, d, C = 32, 8, 128, 70000
    xq, xk, v, _ = make_qkv(7401, C, Hq, Hkv, d)
    kc = to_dev(xk)
    jl.rope_apply(kc, theta)
    vc = to_dev(v)
    for pos in (65537, 40000):  # the second call smaller (fewer splits)
        for mode in ("fused", "plain"):
            note(f"decode noalloc pos={pos} mode={mode}")
            q = to_dev(xq[pos])
            o1, l1 = _noalloc(q, kc, vc, pos, w0, w_pre, theta, mode)
            o2, l2 = jl.bifocal_decode(q, kc, vc, pos, w0, w_pre, theta, mode=mode)
            torch.cuda.synchronize()
            assert torch.equal(o1, o2) and torch.equal(l1, l2), (pos, mode)
            ro, _ = decode_row(xq[pos], xk, v, pos, 10 ** 9 if mode == "plain" else w0, w_pre,
                               theta)
            assert_bf16_close(to_host(o1), ro, f"noalloc pos={pos} {mode}")


def test_decode_noalloc_rejects_oversized_plan():
    """A caller-chosen split count whose partials exceed the array is refused
    before any launch (JL_EWORKSPACE)."""
    Hq, Hkv, d, C = 64, 8, 128, 70000
    q = torch.zeros((Hq, d), dtype=torch.bfloat16, device="cuda")
    kc = torch.zeros((C, Hkv, d), dtype=torch.bfloat16, device="cuda")
    o = torch.empty_like(q)
    st = jl.lib().jl_bifocal_decode_noalloc(
        ctypes.c_void_p(q.data_ptr()), ctypes.c_void_p(kc.data_ptr()),
        ctypes.c_void_p(kc.data_ptr()), ctypes.c_void_p(o.data_ptr()), None, C - 1, C, Hq, Hkv,
        d, 4096, 32768, 1e6, 0.0, 0, 0, 1000,
        ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == -4
