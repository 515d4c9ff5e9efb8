"""CPU tests of the C-ABI library: it loads, exports every symbol the header
declares, its host-side logic (Eq. 2 group size, tile classes) is bit-exact
against the oracle's independent definitions, and bad arguments come back as
status codes before any launch. No kernel runs here."""
import ctypes
import os
import re

import numpy as np
import pytest

import rope_context_extension_jl_amd as jl
from oracle import group_size as oracle_group_size
from oracle import tile_class as oracle_tile_class

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "bifocal.h")

pytestmark = pytest.mark.skipif(not os.path.exists(jl.LIB_PATH),
                                reason="libbifocal.so not built (run __graft_entry__.build())")


def _declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jl_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    syms = _declared_symbols()
    for name in ("jl_group_size", "jl_rope_apply", "jl_bifocal_prefill", "jl_bifocal_decode",
                 "jl_tile_class", "jl_debug_tile_classes"):
        assert name in syms


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(jl.LIB_PATH)
    missing = [s for s in _declared_symbols() if not hasattr(lib, s)]
    assert not missing, missing
    # and the binding declares a signature for each of them
    assert set(_declared_symbols()) == set(jl._SIGS)


def test_group_size_matches_oracle_exhaustive_small():
    for w_pre in (1, 2, 3, 7, 64, 32768):
        for L in range(1, 3000):
            assert jl.group_size(L, w_pre) == oracle_group_size(L, w_pre)


def test_group_size_matches_oracle_large():
    rng = np.random.default_rng(0)
    for L in list(rng.integers(1, 2 ** 40, 2000)) + [2 ** 31 - 1, 2 ** 31, 2 ** 40]:
        for w_pre in (1, 4096, 32768, 131072, 2 ** 31 - 1):
            assert jl.group_size(int(L), w_pre) == oracle_group_size(int(L), w_pre)


def test_group_size_rejects_bad_arguments():
    assert jl.lib().jl_group_size(0, 4) == -1
    assert jl.lib().jl_group_size(5, 0) == -1
    assert jl.lib().jl_group_size(-3, 4) == -1


def test_tile_class_matches_oracle_bruteforce_exhaustive():
    """Every tile of every small shape against the pairwise definition."""
    for w0 in (0, 1, 2, 5, 9):
        for q0 in range(0, 14):
            for q1 in range(q0, min(q0 + 6, 14)):
                for k0 in range(0, 14):
                    for k1 in range(k0, min(k0 + 6, 14)):
                        assert jl.tile_class(q0, q1, k0, k1, w0) == \
                            oracle_tile_class(q0, q1, k0, k1, w0), (q0, q1, k0, k1, w0)


def test_tile_class_matches_oracle_at_kernel_tile_shape():
    bm, bn = jl.prefill_tile_shape()
    rng = np.random.default_rng(1)
    for _ in range(300):
        w0 = int(rng.choice([0, 1, 63, 64, 65, 127, 2048, 4096]))
        i = int(rng.integers(0, 70))
        j = int(rng.integers(0, 2 * i + 3))
        L = int(rng.integers(max(1, i * bm + 1), (i + 1) * bm + 300))
        q0, q1 = i * bm, min(L, (i + 1) * bm) - 1
        k0 = j * bn
        if k0 > L - 1:
            continue
        k1 = min(L, k0 + bn) - 1
        assert jl.tile_class(q0, q1, k0, k1, w0) == oracle_tile_class(q0, q1, k0, k1, w0)


def test_tile_class_rejects_bad_arguments():
    f = jl.lib().jl_tile_class
    assert f(5, 4, 0, 0, 1) == -1
    assert f(0, 0, 3, 2, 1) == -1
    assert f(-1, 0, 0, 0, 1) == -1
    assert f(0, 0, 0, 0, -1) == -1


def test_tile_shapes():
    assert jl.prefill_tile_shape() == (128, 64)
    with pytest.raises(jl.BifocalError):
        jl.prefill_tile_shape(d=96)


def test_status_strings():
    for code in (0, -1, -2, -3, -4, -99):
        assert jl.status_string(code)


def test_workspace_sizes_are_monotone_and_positive():
    a = jl.prefill_workspace_size(1000, 1, 8, 2, 128)
    b = jl.prefill_workspace_size(2000, 1, 8, 2, 128)
    c = jl.prefill_workspace_size(2000, 1, 8, 2, 128, mode="ie")
    assert 0 < a < b < c
    assert jl.decode_workspace_size(131072, 32, 128) >= 32 * 1024 * 130 * 4


# --- argument validation: every failing call returns before any HIP call ----
P = ctypes.c_void_p(16)  # non-null dummy: validation fails before it is touched


def _prefill(**kw):
    args = dict(xq=P, xk=P, v=P, o=P, lse=None, kc=None, cu=None, B=1, T=256, Hq=4, Hkv=2, d=128,
                w0=16, w_pre=64, theta=1e4, scale=0.0, dt=0, mode=0, ws=P, ws_bytes=1 << 40,
                stream=None)
    args.update(kw)
    return jl.lib().jl_bifocal_prefill(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(Hq=3, Hkv=2), -1), (dict(Hkv=0), -1), (dict(T=-1), -1), (dict(w0=-1), -1),
    (dict(w_pre=0), -1), (dict(theta=1.0), -1), (dict(B=2), -1), (dict(d=96), -2),
    (dict(d=64), -2), (dict(dt=1, d=96), -2), (dict(mode=7), -1), (dict(xq=None), -1),
    (dict(ws=None), -4), (dict(ws_bytes=10), -4), (dict(ws=ctypes.c_void_p(16 + 8)), -1),
    (dict(B=5000, cu=P), -1), (dict(dt=5), -1),
])
def test_prefill_argument_errors(kw, code):
    assert _prefill(**kw) == code


def test_prefill_empty_is_noop():
    assert _prefill(T=0, xq=None, xk=None, v=None, o=None, ws=None, ws_bytes=0) == 0


def _decode(**kw):
    args = dict(xq=P, kc=P, vc=P, o=P, lse=None, pos=100, cap=1000, Hq=8, Hkv=2, d=128, w0=16,
                w_pre=64, theta=1e4, scale=0.0, dt=0, mode=0, splits=0, ws=P, ws_bytes=1 << 40,
                stream=None)
    args.update(kw)
    return jl.lib().jl_bifocal_decode(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(pos=-1), -1), (dict(pos=1000), -1), (dict(cap=0), -1), (dict(Hq=6, Hkv=4), -1),
    (dict(w0=-2), -1), (dict(w_pre=0), -1), (dict(splits=-1), -1), (dict(mode=1), -2),
    (dict(mode=9), -1), (dict(d=96), -2), (dict(Hq=12, Hkv=4), -2), (dict(Hq=32, Hkv=2), -2),
    (dict(kc=None), -1), (dict(ws=None), -4), (dict(ws_bytes=100), -4),
    (dict(splits=5000), -1), (dict(theta=0.5), -1),
])
def test_decode_argument_errors(kw, code):
    assert _decode(**kw) == code


@pytest.mark.parametrize("kw,code", [
    (dict(T=-1), -1), (dict(H=0), -1), (dict(d=7), -1), (dict(d=40), -2), (dict(d=512), -1),
    (dict(pos=-1), -1), (dict(theta=1.0), -1), (dict(x=None), -1), (dict(B=0, cu=P), -1),
])
def test_rope_argument_errors(kw, code):
    args = dict(x=P, T=10, H=2, d=128, cu=None, B=1, pos=0, theta=1e4, dt=0, stream=None)
    args.update(kw)
    assert jl.lib().jl_rope_apply(*args.values()) == code


def test_rope_empty_is_noop():
    assert jl.lib().jl_rope_apply(None, 0, 2, 128, None, 1, 0, 1e4, 0, None) == 0


def test_debug_dump_argument_errors():
    f = jl.lib().jl_debug_tile_classes
    assert f(0, 0, P, None) == -1
    assert f(10, -1, P, None) == -1
    assert f(10, 0, None, None) == -1


def test_python_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 2, 128, dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        jl.rope_apply(x, 1e4)
    with pytest.raises(ValueError):
        jl.bifocal_prefill(x, x[:, :1].contiguous(), x[:, :1].contiguous(), 1, 4, 1e4,
                           workspace=torch.zeros(1, dtype=torch.uint8))


def test_python_binding_checks_shapes_and_dtypes():
    """Mismatches the C ABI cannot see (bare pointers) raise ValueError in the
    binding before anything is launched: a key or value tensor of another
    dtype or shape than the queries, outputs of the wrong shape, an int64
    cu_seqlens."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    T, Hq, Hkv, d = 8, 4, 2, 128
    q = torch.zeros(T, Hq, d, dtype=bf)
    k = torch.zeros(T, Hkv, d, dtype=bf)
    ws = torch.zeros(1, dtype=torch.uint8)
    args = (1, 4, 1e4)
    cases = [
        (dict(xk=k.float()), "xk must be"),
        (dict(v=torch.zeros(T, Hkv + 1, d, dtype=bf)), "v must have shape"),
        (dict(out=torch.zeros(T, Hq, d, dtype=f32)), "out must be"),
        (dict(lse=torch.zeros(T, Hq, dtype=f32)), "lse must have shape"),
        (dict(kcache_out=torch.zeros(T, Hkv, d // 2, dtype=bf)), "kcache_out must have shape"),
        (dict(cu_seqlens=torch.tensor([0, 3, 8], dtype=torch.int64)), "cu_seqlens must be"),
        (dict(cu_seqlens=torch.tensor([8], dtype=torch.int32)), "cu_seqlens must be a 1-D"),
    ]
    for kw, msg in cases:
        xk = kw.pop("xk", k)
        v = kw.pop("v", k)
        with pytest.raises(ValueError, match=msg):
            jl.bifocal_prefill(q, xk, v, *args, workspace=ws, **kw)
    with pytest.raises(ValueError, match="cu_seqlens must be"):
        jl.rope_apply(k, 1e4, cu_seqlens=torch.tensor([0, 8], dtype=torch.int64))
    C = 16
    kc = torch.zeros(C, Hkv, d, dtype=bf)
    with pytest.raises(ValueError, match="vcache must have shape"):
        jl.bifocal_decode(q[0], kc, kc[:8], 3, *args)
    with pytest.raises(ValueError, match="kcache must be"):
        jl.bifocal_decode(q[0], kc.float(), kc, 3, *args)
    with pytest.raises(ValueError, match="out must have shape"):
        jl.bifocal_decode(q[0], kc, kc, 3, *args, out=torch.zeros(Hq + 1, d, dtype=bf))
    with pytest.raises(ValueError, match="lse must have shape"):
        jl.bifocal_decode(q[0], kc, kc, 3, *args, lse=torch.zeros(Hq, 1, dtype=f32))
    with pytest.raises(ValueError, match="vcache must be"):
        jl.bifocal_prefill_cached(q, kc, kc.float(), 0, *args)
    with pytest.raises(ValueError, match="lse must have shape"):
        jl.bifocal_prefill_cached(q, kc, kc, 0, *args, lse=torch.zeros(T, Hq, dtype=f32))
    pos = torch.zeros(2, dtype=torch.int32)
    qb = torch.zeros(2, Hq, d, dtype=bf)
    with pytest.raises(ValueError, match="out must have shape"):
        jl.bifocal_decode_batch(qb, kc, kc, pos, pos, 4, *args, out=torch.zeros(3, Hq, d, dtype=bf))
    with pytest.raises(ValueError, match="kcache must be"):
        jl.bifocal_decode_batch(qb, kc.float(), kc, pos, pos, 4, *args)
    with pytest.raises(ValueError, match="positions must be"):
        jl.bifocal_decode_batch(qb, kc, kc, pos.long(), pos, 4, *args)


def test_python_binding_checks_workspace_device():
    """A workspace on another device than the call's tensors raises before any
    launch (the C ABI sees a bare pointer); its byte count is numel times the
    element size for any dtype."""
    import torch
    bf = torch.bfloat16
    T, Hq, Hkv, d = 8, 4, 2, 128
    q = torch.zeros(T, Hq, d, dtype=bf)
    k = torch.zeros(T, Hkv, d, dtype=bf)
    kc = torch.zeros(16, Hkv, d, dtype=bf)
    other = torch.empty(64, dtype=torch.uint8, device="meta")
    args = (1, 4, 1e4)
    with pytest.raises(ValueError, match="workspace must be on"):
        jl.bifocal_prefill(q, k, k, *args, workspace=other)
    with pytest.raises(ValueError, match="workspace must be on"):
        jl.bifocal_prefill_cached(q, kc, kc, 0, *args, workspace=other)
    with pytest.raises(ValueError, match="workspace must be on"):
        jl.bifocal_decode(q[0], kc, kc, 3, *args, workspace=other)
    pos = torch.zeros(2, dtype=torch.int32)
    with pytest.raises(ValueError, match="workspace must be on"):
        jl.bifocal_decode_batch(torch.zeros(2, Hq, d, dtype=bf), kc, kc, pos, pos, 4, *args,
                                workspace=other)
    assert jl._ws_bytes(torch.zeros(10, dtype=torch.float32), torch.device("cpu")) == 40


def test_calibration_argument_errors():
    f, g = jl.lib().jl_calib_stream_read, jl.lib().jl_calib_mfma_bf16
    assert f(None, 1024, P, 16, None) == -1
    assert f(P, 1000, P, 16, None) == -1          # not a multiple of 16 bytes
    assert f(ctypes.c_void_p(24), 1024, P, 16, None) == -1  # not 16-byte aligned
    assert f(P, 1024, None, 16, None) == -1
    assert f(P, 1024, P, 0, None) == -1
    assert g(None, 4, 10, None) == -1
    assert g(P, 0, 10, None) == -1
    assert g(P, 4, 0, None) == -1


def _cached(**kw):
    args = dict(xq=P, kc=P, vc=P, o=P, lse=None, q_off=100, Tq=50, cap=1000, Hq=8, Hkv=2, d=128,
                w0=16, w_pre=64, theta=1e4, scale=0.0, dt=0, mode=0, ws=P, ws_bytes=1 << 40,
                stream=None)
    args.update(kw)
    return jl.lib().jl_bifocal_prefill_cached(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(q_off=-1), -1), (dict(Tq=-1), -1), (dict(q_off=960), -1), (dict(cap=0), -1),
    (dict(Hq=6, Hkv=4), -1), (dict(w0=-1), -1), (dict(w_pre=0), -1), (dict(theta=1.0), -1),
    (dict(mode=1), -2), (dict(mode=9), -1), (dict(dt=1), -2), (dict(d=64), -2), (dict(dt=4), -1),
    (dict(xq=None), -1), (dict(kc=None), -1), (dict(ws=None), -4), (dict(ws_bytes=64), -4),
    (dict(ws=ctypes.c_void_p(16 + 8)), -1),
])
def test_prefill_cached_argument_errors(kw, code):
    assert _cached(**kw) == code


def test_prefill_cached_empty_is_noop_and_sizes():
    assert _cached(Tq=0, xq=None, kc=None, vc=None, o=None, ws=None, ws_bytes=0) == 0
    a = jl.prefill_cached_workspace_size(0, 1000, 8, 2, 128)
    b = jl.prefill_cached_workspace_size(1000, 1000, 8, 2, 128)
    assert 0 < a < b
    assert b == jl.prefill_workspace_size(2000, 1, 8, 2, 128)
    assert jl.prefill_cached_workspace_size(0, 10, 8, 2, 64) == 0
    assert jl.prefill_cached_workspace_size(0, 10, 8, 2, 128, mode="ie") == 0


CONT = 16  # JL_REMAP_CONTINUOUS


def test_continuous_flag_is_declared_and_sizes_unchanged():
    text = open(HEADER).read()
    assert re.search(r"#define\s+JL_REMAP_CONTINUOUS\s+16\b", text)
    assert jl.REMAPS == {"floor": 0, "continuous": CONT}
    f = jl.lib()
    for m in (0, 1, 2):
        assert f.jl_prefill_workspace_size(3000, 2, 8, 2, 128, 0, m | CONT) == \
            f.jl_prefill_workspace_size(3000, 2, 8, 2, 128, 0, m)
    for m in (0, 2):
        assert f.jl_prefill_cached_workspace_size(100, 50, 8, 2, 128, m | CONT) == \
            f.jl_prefill_cached_workspace_size(100, 50, 8, 2, 128, m)


@pytest.mark.parametrize("mode,code", [(1 | CONT, -2), (7 | CONT, -1), (32, -1)])
def test_continuous_flag_argument_errors(mode, code):
    assert _decode(mode=mode) == code
    assert _cached(mode=mode) == code
    if mode != (1 | CONT):
        assert _prefill(mode=mode) == code


def test_continuous_flag_empty_calls_are_noops():
    assert _prefill(T=0, xq=None, xk=None, v=None, o=None, ws=None, ws_bytes=0, mode=CONT) == 0
    assert _cached(Tq=0, xq=None, kc=None, vc=None, o=None, ws=None, ws_bytes=0,
                   mode=CONT) == 0


def _batch(**kw):
    args = dict(xq=P, kc=P, vc=P, o=P, lse=None, pos=P, st=P, B=4, max_keys=1000, rows=5000,
                Hq=8, Hkv=2, d=128, w0=16, w_pre=64, theta=1e4, scale=0.0, dt=0, mode=0, splits=0,
                ws=P, ws_bytes=1 << 40, stream=None)
    args.update(kw)
    return jl.lib().jl_bifocal_decode_batch(*args.values())


@pytest.mark.parametrize("kw,code", [
    (dict(B=-1), -1), (dict(B=70000), -1), (dict(max_keys=0), -1), (dict(max_keys=2 ** 31), -1),
    (dict(rows=0), -1), (dict(Hq=6, Hkv=4), -1), (dict(w0=-1), -1), (dict(w_pre=0), -1),
    (dict(theta=1.0), -1), (dict(splits=-1), -1), (dict(splits=5000), -1), (dict(mode=1), -2),
    (dict(mode=9), -1), (dict(d=96), -2), (dict(Hq=32, Hkv=2), -2), (dict(dt=4), -1),
    (dict(pos=None), -1), (dict(st=None), -1), (dict(kc=None), -1), (dict(ws=None), -4),
    (dict(ws_bytes=100), -4), (dict(ws=ctypes.c_void_p(16 + 8)), -1),
])
def test_decode_batch_argument_errors(kw, code):
    assert _batch(**kw) == code


def test_decode_batch_empty_and_sizes():
    assert _batch(B=0, xq=None, kc=None, vc=None, o=None, pos=None, st=None, ws=None,
                  ws_bytes=0) == 0
    a = jl.decode_batch_workspace_size(1, 131072, 32, 128)
    assert a == jl.decode_workspace_size(131072, 32, 128) + 256  # + the work list
    assert jl.decode_batch_workspace_size(16, 131072, 32, 128) >= 16 * 32 * 1024 * 130 * 4
    assert jl.decode_batch_workspace_size(0, 10, 8, 128) == 0
    assert jl.decode_batch_workspace_size(2, 0, 8, 128) == 0
