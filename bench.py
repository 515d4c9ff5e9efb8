#!/usr/bin/env python3
"""Benchmark of the bifocal RoPE attention hot path on one MI355X.

Timed step (the whole prefill hot path of the 128K workload): one
jl_bifocal_prefill call in fused mode on raw bf16 Q/K/V, L = 131072,
Hq/Hkv = 32/8, d = 128, w_pretrained = 32768 (G = 4), w0 = 4096, 1% of key
rows x8; it rotates the keys, writes the absolute bf16 key cache, rotates the
queries and runs the fused attention pass. Inputs are resident in HBM before
the timed region. value = causal-attention FLOPs 2 L^2 d Hq per step / step
time (effective TFLOP/s).

Also reported (not part of the timed step): the attention kernel alone (live
HIP events around it, for the roofline), the library's plain causal RoPE
attention at the same shape (overhead ratio), the Eq. 7 inclusion-exclusion
alternative, the 64K and packed-varlen workloads, prefill continued on the cache for the
last 8192 rows, absolute RoPE (jl_rope_apply) of the query and key tensors, a
window-size sweep, the continuous remote map x/G (prefill
kernel and decode), decode latency at positions 32767 .. 131071 of a
131072-key cache with L2 / MALL evicted before every step, a batch of 16
sequences decoding in one launch, calibrated HBM-read and MFMA ceilings, and the float64 CPU
oracle on a bounded sample of rows.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W]
"""
import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = ("bifocal prefill TFLOP/s + tok/s at 128K (% MFMA peak); decode µs/token "
          "(% HBM BW)")
PEAK_BF16_TFLOPS = 2500.0   # MI355X dense bf16/fp16 MFMA
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "prefill_128k_fused_traffic.json")


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def _code_lines(text):
    """Source lines without // comments and blank lines (a line holding a
    string literal is kept whole), so that comment edits keep the hash."""
    out = []
    for line in text.splitlines():
        if '"' not in line and "//" in line:
            line = line[:line.index("//")]
        line = line.rstrip()
        if line:
            out.append(line)
    return "\n".join(out)


def kernel_source_hash():
    """Hash of the code (comments aside) the fused attention kernel is
    compiled from."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "rope_context_extension_jl_amd", "csrc")
    for name in ("jl_internal.hpp", "prefill_bf16.hip"):
        with open(os.path.join(csrc, name), encoding="utf-8") as fh:
            h.update(name.encode() + _code_lines(fh.read()).encode())
    return h.hexdigest()[:16]


def pct(xs, q):
    return float(np.percentile(np.asarray(xs), q))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=5)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--decode-iters", type=int, default=100)
    ap.add_argument("--cpu-rows", type=int, default=512, help="oracle rows for the CPU baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-extras", action="store_true", help="only the timed prefill steps")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run one 1 GiB device copy (counter calibration runs)")
    ap.add_argument("--legs", default="all",
                    help="comma list of the extra legs to run (plain, ie, cached, rope, sweep, "
                         "cont, decode, batch, others; default all)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: libbifocal has no multi-GPU path "
              "(--gpus must be 1)", file=sys.stderr)
        sys.exit(1)

    import torch

    import rope_context_extension_jl_amd as jl
    from synth_inputs import WORKLOADS, make_decode_seq, make_qkv, packed_starts

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    jl.lib()  # fail loudly if the library is missing

    def up(a):
        return torch.from_numpy(a).to(torch.bfloat16).to(dev).contiguous()

    # ------------------------------------------------- calibrated ceilings
    log("calibration: streaming HBM read and pure bf16 MFMA rate")
    cev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    # 4 GiB read: large enough that launch and tail costs stay under 1% of the
    # run (a 1 GiB read reports ~10% lower). Three read kernels at a few grid
    # sizes; the best median is the ceiling the decode figures are set against.
    rbuf = torch.ones(1 << 30, dtype=torch.float32, device=dev)  # 4 GiB
    read_variants = {}
    for variant, name in ((0, "grid_stride_x4"), (1, "chunk_nontemporal_x8"),
                          (2, "chunk_global_to_lds"), (3, "chunk_x8"),
                          (4, "chunk_global_to_lds_nontemporal")):
        best = 0.0
        for blocks in (2048, 8192, 16384):
            rts = []
            for _ in range(6):
                jl.calib_stream_read(rbuf, events=cev, blocks=blocks, variant=variant)
                torch.cuda.synchronize()
                rts.append(cev[0].elapsed_time(cev[1]))
            gbs = rbuf.numel() * 4 / (float(np.median(rts[1:])) * 1e-3) / 1e9
            read_variants[f"{name}_{blocks}wg"] = round(gbs, 1)
            best = max(best, gbs)
        log(f"calibration read {name}: best {best:.0f} GB/s")
    read_gbs = max(read_variants.values())
    del rbuf
    mts = []
    for _ in range(4):
        mfl = jl.calib_mfma_bf16(512, 20000, events=cev)
        torch.cuda.synchronize()
        mts.append(cev[0].elapsed_time(cev[1]))
    mfma_tflops = mfl / (float(np.median(mts[1:])) * 1e-3) / 1e12
    calib = {"hbm_read_GBps": round(read_gbs, 1), "mfma_bf16_TFLOPs": round(mfma_tflops, 1),
             "hbm_read_variants_GBps": read_variants,
             "method": "jl_calib_stream_read_ex over 4 GiB: the best median of 5 over five "
                       "read kernels (grid-stride; 32 KiB chunks with and without the "
                       "nontemporal hint; global->LDS chunks with and without it) "
                       "at 2048/8192/16384 workgroups; jl_calib_mfma_bf16, "
                       "2048 waves x 20000 rounds of 4 independent 32x32x16 MFMAs (median of 3)"}
    log(f"calibrated ceilings: HBM read {read_gbs:.0f} GB/s, bf16 MFMA {mfma_tflops:.0f} TFLOP/s")

    c = WORKLOADS["prefill_128k"]
    L, Hq, Hkv, d = c["lengths"][0], c["Hq"], c["Hkv"], c["d"]
    w0, w_pre, theta = c["w0"], c["w_pre"], c["theta"]
    G = jl.group_size(L, w_pre)
    flops = 2.0 * L * L * d * Hq
    log(f"generating prefill_128k inputs (L={L}, Hq={Hq}, Hkv={Hkv}, G={G})")
    xq, xk, v, _ = make_qkv(c["seed"], L, Hq, Hkv, d, c["std"], c["dtype"], c["peaked_frac"],
                            c["peaked_gain"])
    q, k, vv = up(xq), up(xk), up(v)
    o = torch.empty_like(q)
    lse = torch.empty((Hq, L), dtype=torch.float32, device=dev)
    kcache = torch.empty_like(k)
    ws = torch.empty(jl.prefill_workspace_size(L, 1, Hq, Hkv, d, mode="fused"), dtype=torch.uint8,
                     device=dev)
    stream = torch.cuda.current_stream()
    # the seeded rows the CPU oracle evaluates; GPU outputs are kept on them
    rows = np.sort(np.random.default_rng(99).choice(L, args.cpu_rows, replace=False))
    rows_t = torch.from_numpy(rows).to(dev)
    kept = {}

    def prefill(mode="fused", events=None, workspace=ws):
        jl.bifocal_prefill(q, k, vv, w0, w_pre, theta, mode=mode, out=o, lse=lse,
                           kcache_out=kcache, workspace=workspace, events=events)

    # ---------------------------------------------------------- timed steps
    log(f"warmup {args.warmup} step(s)")
    for _ in range(args.warmup):
        prefill()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.steps)]
    t_begin = torch.cuda.Event(enable_timing=True)
    t_end = torch.cuda.Event(enable_timing=True)
    log(f"timing {args.steps} step(s)")
    torch.cuda.synchronize()
    t_begin.record(stream)
    for i in range(args.steps):
        prefill(events=ev[i])
    t_end.record(stream)
    torch.cuda.synchronize()
    kept["fused"] = o.index_select(0, rows_t).float().cpu().numpy()
    total_ms = t_begin.elapsed_time(t_end)
    ms_per_step = total_ms / args.steps
    kern_ms = [b.elapsed_time(e) for b, e in ev]
    kern_avg = float(np.mean(kern_ms))
    value = flops / (ms_per_step * 1e-3) / 1e12
    achieved = flops / (kern_avg * 1e-3) / 1e12
    log(f"prefill_128k fused: {ms_per_step:.3f} ms/step ({value:.1f} TFLOP/s), attention kernel "
        f"{kern_avg:.3f} ms ({achieved:.1f} TFLOP/s, {100 * achieved / PEAK_BF16_TFLOPS:.1f}% of "
        "peak)")

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as fh:
            tr = json.load(fh)
        if tr.get("kernel_source_hash") == kernel_source_hash():
            traffic = tr.get("bytes_per_launch")
    result = {
        "metric": METRIC,
        "value": round(value, 3),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "prefill_128k", "seq_len": L, "batch": 1, "q_heads": Hq,
                   "kv_heads": Hkv, "head_dim": d, "w_pretrained": w_pre, "G": G, "w0": w0,
                   "theta": theta, "peaked_key_rows": c["peaked_frac"]},
        "tok_per_s": round(L / (ms_per_step * 1e-3), 1),
        "pct_mfma_peak": round(100.0 * value / PEAK_BF16_TFLOPS, 2),
        "roofline": {"bound": "mfma", "kernel": ("prefill_pair_kernel<FUSED>"
                                                  if (Hq // Hkv) % 2 == 0
                                                  else "prefill_bf16_kernel<FUSED>"),
                     "achieved": round(achieved, 3), "peak": PEAK_BF16_TFLOPS,
                     "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                     "traffic": traffic, "kernel_ms": round(kern_avg, 4),
                     "kernel_ms_min": round(min(kern_ms), 4),
                     "calibrated_peak": calib["mfma_bf16_TFLOPs"],
                     "frac_of_calibrated": round(achieved / calib["mfma_bf16_TFLOPs"], 4)},
        "calibration": calib,
    }
    del ev

    cpu_per = {}  # CPU oracle per workload (filled where the host inputs exist)
    legs = None if args.legs == "all" else set(args.legs.split(","))

    def want(name):
        return legs is None or name in legs
    if not args.no_extras:
        extras = {}
        plain_ms = None
        pe = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        call = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        # ---------------------------------------------------- plain baseline
        if want("plain"):
            log("plain causal RoPE attention at the same shape")
            ws_plain = torch.empty(jl.prefill_workspace_size(L, 1, Hq, Hkv, d, mode="plain"),
                                   dtype=torch.uint8, device=dev)
            pe = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            prefill("plain", workspace=ws_plain)
            torch.cuda.synchronize()
            pk = []
            for _ in range(3):
                prefill("plain", events=pe, workspace=ws_plain)
                torch.cuda.synchronize()
                pk.append(pe[0].elapsed_time(pe[1]))
            del ws_plain
            plain_ms = float(np.median(pk))
            extras["plain_128k"] = {"kernel_ms": round(plain_ms, 4),
                                    "tflops": round(flops / plain_ms / 1e9, 2),
                                    "overhead_ratio_kernel": round(kern_avg / plain_ms, 4)}
        # ---------------------------------------------------- IE alternative
        if want("ie"):
            log("inclusion-exclusion alternative")
            ws_ie = torch.empty(jl.prefill_workspace_size(L, 1, Hq, Hkv, d, mode="ie"),
                                dtype=torch.uint8, device=dev)
            prefill("ie", workspace=ws_ie)
            torch.cuda.synchronize()
            ik = []
            for _ in range(2):
                prefill("ie", events=pe, workspace=ws_ie)
                torch.cuda.synchronize()
                ik.append(pe[0].elapsed_time(pe[1]))
            ratio = jl.ie_ratio_view(ws_ie, L, 1, Hq, Hkv, d)
            kept["ie"] = o.index_select(0, rows_t).float().cpu().numpy()
            kept["ie_ratio"] = ratio[:, rows_t].cpu().numpy().T  # [rows, Hq]
            extras["ie_128k"] = {"kernels_ms": round(float(np.median(ik)), 4),
                                 "vs_fused": round(float(np.median(ik)) / kern_avg, 4),
                                 "worst_cancellation_ratio": float(ratio.max()),
                                 "rows_ratio_over_1e3": float((ratio > 1e3).float().mean())}
            del ws_ie, ratio
            prefill()  # restore the fused output and cache for the legs below
            torch.cuda.empty_cache()

        # ---------------------------------------------------- chunked prefill
        if want("cached"):
            log("prefill continued on the cache: last 8192 rows of the 128K sequence")
            Tq = 8192
            q_off = L - Tq
            qc = q[q_off:].contiguous()
            ws_c = torch.empty(jl.prefill_cached_workspace_size(q_off, Tq, Hq, Hkv, d),
                               dtype=torch.uint8, device=dev)
            oc = torch.empty_like(qc)
            lc = torch.empty((Hq, Tq), dtype=torch.float32, device=dev)
            fl_c = sum(4.0 * (p + 1) * d * Hq for p in range(q_off, L))
            call = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
            jl.bifocal_prefill_cached(qc, kcache, vv, q_off, w0, w_pre, theta, out=oc, lse=lc,
                                      workspace=ws_c)
            torch.cuda.synchronize()
            ck, cc_ = [], []
            for _ in range(5):
                call[0].record(stream)
                jl.bifocal_prefill_cached(qc, kcache, vv, q_off, w0, w_pre, theta, out=oc, lse=lc,
                                          workspace=ws_c, events=pe)
                call[1].record(stream)
                torch.cuda.synchronize()
                ck.append(pe[0].elapsed_time(pe[1]))
                cc_.append(call[0].elapsed_time(call[1]))
            extras["prefill_cached_128k_last8k"] = {
                "q_off": q_off, "rows": Tq, "kernel_ms": round(float(np.median(ck)), 4),
                "tflops": round(fl_c / float(np.median(ck)) / 1e9, 2),
                "call_ms": round(float(np.median(cc_)), 4),
                "note": "call_ms adds the plan and the pre-pass that rotates all 131072 cached keys"}
            del ws_c, oc, lc, qc
            torch.cuda.empty_cache()

        # ---------------------------------------------------- absolute RoPE
        if want("rope"):
            log("absolute RoPE (jl_rope_apply) of the 128K query and key tensors, in place")
            rope_x = {"queries": q.clone(), "keys": k.clone()}
            rope_res = {}
            for nm, xt in rope_x.items():
                jl.rope_apply(xt, theta)
                torch.cuda.synchronize()
                rt = []
                for _ in range(5):
                    call[0].record(stream)
                    jl.rope_apply(xt, theta)
                    call[1].record(stream)
                    torch.cuda.synchronize()
                    rt.append(call[0].elapsed_time(call[1]))
                rm = float(np.median(rt))
                nb = 2.0 * xt.numel() * xt.element_size()  # read and written once
                rope_res[nm] = {"shape": list(xt.shape), "ms": round(rm, 4),
                                "GBps": round(nb / (rm * 1e-3) / 1e9, 1),
                                "pct_hbm_peak": round(100 * nb / (rm * 1e-3) / 1e9 / PEAK_HBM_GBS, 2)}
            extras["rope_apply_128k"] = rope_res
            del rope_x
            torch.cuda.empty_cache()

        # ---------------------------------------------------- w0 sweep
        if want("sweep"):
            log("window sweep at 128K (fused attention kernel)")
            sweep = {}
            for w in (0, 512, 1024, 2048, 4096):
                jl.bifocal_prefill(q, k, vv, w, w_pre, theta, out=o, lse=lse, workspace=ws)
                torch.cuda.synchronize()
                wt = []
                for _ in range(2):
                    jl.bifocal_prefill(q, k, vv, w, w_pre, theta, out=o, lse=lse, workspace=ws,
                                       events=pe)
                    torch.cuda.synchronize()
                    wt.append(pe[0].elapsed_time(pe[1]))
                wm = float(np.median(wt))
                sweep[str(w)] = {"kernel_ms": round(wm, 4), "tflops": round(flops / wm / 1e9, 2),
                                 "vs_plain": round(wm / plain_ms, 4) if plain_ms else None}
            extras["w0_sweep_128k"] = sweep

        # ---------------------------------------------------- continuous remote map
        if want("cont"):
            log("continuous remote map x/G at 128K (fused attention kernel)")
            jl.bifocal_prefill(q, k, vv, w0, w_pre, theta, out=o, lse=lse, workspace=ws,
                               remap="continuous")
            torch.cuda.synchronize()
            ct = []
            for _ in range(3):
                jl.bifocal_prefill(q, k, vv, w0, w_pre, theta, out=o, lse=lse, workspace=ws,
                                   events=pe, remap="continuous")
                torch.cuda.synchronize()
                ct.append(pe[0].elapsed_time(pe[1]))
            cm = float(np.median(ct))
            extras["continuous_map_128k"] = {"kernel_ms": round(cm, 4),
                                             "tflops": round(flops / cm / 1e9, 2),
                                             "vs_floor_map": round(cm / kern_avg, 4),
                                             "vs_plain": round(cm / plain_ms, 4) if plain_ms else None}

        # evicts L2 and the memory-side cache between decode steps
        flush = torch.ones(1 << 28, dtype=torch.float32, device=dev)
        de = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
        # ---------------------------------------------------- decode
        if want("decode"):
            log("decode on the 131072-key absolute cache (L2/MALL evicted by a clean read per step)")
            cdec = WORKLOADS["decode_128k"]
            # Two cache states between steps: a clean 1 GiB read (evicts L2 and the
            # memory-side cache and leaves no dirty lines) and a 1 GiB zero-fill
            # (evicts too, but leaves dirty lines whose write-back the timed step
            # then pays for). The clean read is the headline state.
            wsd = jl.decode_workspace(L, Hq, d, dev)
            od = torch.empty((Hq, d), dtype=torch.bfloat16, device=dev)
            ld = torch.empty((Hq,), dtype=torch.float32, device=dev)
            dec = {}
            for pos in cdec["decode_positions"]:
                qd = q[pos].contiguous()
                row = {}
                # the five (mode, cache state) variants take turns step by step,
                # so a drift of the clock during the run affects them alike
                variants = [(m, e) for m in ("fused", "plain", "continuous")
                            for e in (("read",) if m == "continuous" else ("read", "write"))]
                times = {v: [] for v in variants}
                for it in range(args.decode_iters + 3):
                    for mode, evict in variants:
                        if evict == "read":
                            flush.sum()
                        else:
                            flush.zero_()
                        jl.bifocal_decode(qd, kcache, vv, pos, w0, w_pre, theta,
                                          mode="fused" if mode == "continuous" else mode,
                                          remap="continuous" if mode == "continuous" else "floor",
                                          out=od, lse=ld, workspace=wsd, events=de)
                        torch.cuda.synchronize()
                        if it >= 3:
                            times[(mode, evict)].append(de[0].elapsed_time(de[1]) * 1e3)  # us
                for (mode, evict), ts in times.items():
                    nbytes = 4.0 * (pos + 1) * Hkv * d
                    med = float(np.median(ts))
                    key = mode if evict == "read" else mode + "_after_zero_fill"
                    row[key] = {"us_median": round(med, 2), "us_p10": round(pct(ts, 10), 2),
                                "us_p90": round(pct(ts, 90), 2),
                                "GBps": round(nbytes / (med * 1e-6) / 1e9, 1),
                                "pct_hbm_peak": round(100 * nbytes / (med * 1e-6) / 1e9 /
                                                      PEAK_HBM_GBS, 2),
                                "pct_calibrated_read": round(100 * nbytes / (med * 1e-6) / 1e9 /
                                                             read_gbs, 2)}
                row["G"] = jl.group_size(pos + 1, w_pre)
                row["overhead_ratio"] = round(row["fused"]["us_median"] / row["plain"]["us_median"],
                                              4)
                dec[str(pos)] = row
                log(f"decode pos={pos}: {row['fused']['us_median']} us "
                    f"({row['fused']['pct_hbm_peak']}% HBM, {row['fused']['pct_calibrated_read']}% "
                    f"of the calibrated read rate), plain {row['plain']['us_median']} us")
            result["decode"] = dec
            del wsd

        # ---------------------------------------------------- batched decode
        if want("batch"):
            cb = WORKLOADS["decode_batch_16"]
            bpos = cb["positions"]
            log(f"batched decode: {len(bpos)} sequences in one launch (L2/MALL evicted per step)")
            bst, brows = packed_starts(bpos)
            kb = torch.empty((brows, Hkv, d), dtype=torch.bfloat16, device=dev)
            vb = torch.empty_like(kb)
            xb = torch.empty((len(bpos), Hq, d), dtype=torch.bfloat16, device=dev)
            for b, (p, s0) in enumerate(zip(bpos, bst)):
                qn, kn, vn = make_decode_seq(cb["seed"], b, p + 1, Hq, Hkv, d, cb["std"], cb["dtype"])
                xb[b] = up(qn)
                kb[s0:s0 + p + 1] = up(kn)
                vb[s0:s0 + p + 1] = up(vn)
                jl.rope_apply(kb[s0:s0 + p + 1], cb["theta"])
                del qn, kn, vn
            pos_t = torch.tensor(bpos, dtype=torch.int32, device=dev)
            st_t = torch.tensor(bst, dtype=torch.int32, device=dev)
            mk = max(bpos) + 1
            wsb = jl.decode_batch_workspace(len(bpos), mk, Hq, d, dev)
            ob = torch.empty_like(xb)
            lb = torch.empty((len(bpos), Hq), dtype=torch.float32, device=dev)
            bbytes = sum(4.0 * (p + 1) * Hkv * d for p in bpos)
            brow = {"B": len(bpos), "keys": int(sum(p + 1 for p in bpos)), "max_keys": mk}
            btimes = {"fused": [], "plain": []}
            for it in range(args.decode_iters + 3):  # the two modes take turns
                for mode in ("fused", "plain"):
                    flush.sum()
                    jl.bifocal_decode_batch(xb, kb, vb, pos_t, st_t, mk, cb["w0"], cb["w_pre"],
                                            cb["theta"], mode=mode, out=ob, lse=lb, workspace=wsb,
                                            events=de)
                    torch.cuda.synchronize()
                    if it >= 3:
                        btimes[mode].append(de[0].elapsed_time(de[1]) * 1e3)
            for mode, ts in btimes.items():
                med = float(np.median(ts))
                brow[mode] = {"us_median": round(med, 2), "us_p10": round(pct(ts, 10), 2),
                              "us_p90": round(pct(ts, 90), 2),
                              "tokens_per_s": round(len(bpos) / (med * 1e-6), 1),
                              "GBps": round(bbytes / (med * 1e-6) / 1e9, 1),
                              "pct_hbm_peak": round(100 * bbytes / (med * 1e-6) / 1e9 / PEAK_HBM_GBS,
                                                    2),
                              "pct_calibrated_read": round(100 * bbytes / (med * 1e-6) / 1e9 /
                                                           read_gbs, 2)}
            brow["overhead_ratio"] = round(brow["fused"]["us_median"] / brow["plain"]["us_median"], 4)
            extras["decode_batch_16"] = brow
            log(f"batched decode: {brow['fused']['us_median']} us per step "
                f"({brow['fused']['pct_calibrated_read']}% of the calibrated read rate)")
            del kb, vb, xb, wsb, ob, lb
            torch.cuda.empty_cache()

        del flush
        torch.cuda.empty_cache()
        # ---------------------------------------------------- other workloads
        if want("others"):
            for name in ("prefill_64k", "varlen_4seq"):
                cw = WORKLOADS[name]
                lens = cw["lengths"]
                T = sum(lens)
                log(f"{name}")
                a, b_, cc, _ = make_qkv(cw["seed"], T, cw["Hq"], cw["Hkv"], cw["d"], cw["std"],
                                        cw["dtype"])
                qa, ka, va = up(a), up(b_), up(cc)
                cu = None
                if len(lens) > 1:
                    cu = torch.tensor(np.cumsum([0] + lens), dtype=torch.int32, device=dev)
                wsw = torch.empty(jl.prefill_workspace_size(T, len(lens), cw["Hq"], cw["Hkv"], cw["d"]),
                                  dtype=torch.uint8, device=dev)
                ow = torch.empty_like(qa)
                fw = sum(2.0 * n * n * cw["d"] * cw["Hq"] for n in lens)
                jl.bifocal_prefill(qa, ka, va, cw["w0"], cw["w_pre"], cw["theta"], cu_seqlens=cu,
                                   out=ow, workspace=wsw, want_lse=False)
                torch.cuda.synchronize()
                ks = []
                for _ in range(3):
                    jl.bifocal_prefill(qa, ka, va, cw["w0"], cw["w_pre"], cw["theta"], cu_seqlens=cu,
                                       out=ow, workspace=wsw, want_lse=False, events=pe)
                    torch.cuda.synchronize()
                    ks.append(pe[0].elapsed_time(pe[1]))
                km = float(np.median(ks))
                extras[name] = {"kernel_ms": round(km, 4), "tflops": round(fw / km / 1e9, 2),
                                "pct_mfma_peak": round(100 * fw / km / 1e9 / PEAK_BF16_TFLOPS, 2)}
                if not args.no_cpu_baseline:
                    # the oracle on this workload's parity subset: 512 seeded rows
                    # per sequence, every head
                    from oracle import bifocal_varlen
                    rr = np.random.default_rng(7)
                    rps = [np.sort(rr.choice(n, min(n, args.cpu_rows), replace=False)) for n in lens]
                    log(f"CPU oracle on {name}: {sum(len(r) for r in rps)} rows x {cw['Hq']} heads")
                    t0 = time.perf_counter()
                    bifocal_varlen(a, b_, cc, np.cumsum([0] + lens), cw["w0"], cw["w_pre"],
                                   cw["theta"], rows_per_seq=rps)
                    dt = time.perf_counter() - t0
                    nrh = sum(len(r) for r in rps) * cw["Hq"]
                    flc = float(sum(4.0 * (int(x) + 1) * cw["d"] * cw["Hq"] for r in rps for x in r))
                    cpu_per[name] = {"seconds": round(dt, 3), "rows_per_s": round(nrh / dt, 2),
                                     "TFLOPs": round(flc / dt / 1e12, 6),
                                     "sample": f"{args.cpu_rows} seeded rows per sequence x "
                                               f"{cw['Hq']} heads, all keys of each row"}
                del qa, ka, va, wsw, ow, a, b_, cc
                torch.cuda.empty_cache()
        result["extras"] = extras

    if args.copy_calibration:
        log("1 GiB device copy (counter calibration)")
        src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        dst = torch.empty_like(src)
        src.fill_(1)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---------------------------------------------------------- CPU oracle
    if not args.no_cpu_baseline:
        from oracle import bifocal_attention, decode_row
        try:
            from threadpoolctl import threadpool_info
            blas_threads = max([p.get("num_threads", 0) for p in threadpool_info()] or [0])
        except Exception:  # noqa: BLE001
            blas_threads = None
        cores = len(os.sched_getaffinity(0))
        log(f"CPU oracle on {len(rows)} rows x {Hq} heads of prefill_128k")
        t0 = time.perf_counter()
        O_ref, _ = bifocal_attention(xq, xk, v, w0, w_pre, theta, rows=rows)
        dt = time.perf_counter() - t0
        fl = float(sum(4.0 * (int(r) + 1) * d * Hq for r in rows))
        result["cpu_baseline"] = {
            "value": round(fl / dt / 1e12, 6), "unit": "TFLOP/s",
            "cores": cores, "blas_threads": blas_threads,
            "kind": "oracle", "seconds": round(dt, 3),
            "rows_per_s": round(len(rows) * Hq / dt, 2),
            "sample": f"{len(rows)} seeded query rows x {Hq} heads of prefill_128k (all keys "
                      "of each row, float64 NumPy), FLOPs 4 (q+1) d per row and head; "
                      "rows_per_s counts (row, head) pairs"}
        log(f"CPU oracle: {dt:.2f} s")
        # GPU outputs on the same rows against the oracle
        acc = {}
        for key in ("fused", "ie"):
            if key in kept:
                e = np.abs(kept[key].astype(np.float64) - O_ref)
                acc[key] = {"max_abs": float(e.max()), "mean_abs": float(e.mean())}
        if "ie" in kept:
            e = np.abs(kept["ie"].astype(np.float64) - O_ref).max(axis=2)  # [rows, Hq]
            ok = kept["ie_ratio"] <= 1e3
            e3 = np.abs(kept["ie"].astype(np.float64) - O_ref)
            acc["ie"].update({
                "rows_ratio_le_1e3": {"max_abs": float(e[ok].max()) if ok.any() else None,
                                      "mean_abs": float(e3[ok].mean()) if ok.any() else None},
                "rows_ratio_gt_1e3": {"count": int((~ok).sum()),
                                      "max_abs": float(e[~ok].max()) if (~ok).any() else None},
                "worst_ratio_sampled": float(kept["ie_ratio"].max())})
            if "extras" in result and "ie_128k" in result["extras"]:
                result["extras"]["ie_128k"]["vs_oracle_sampled_rows"] = acc["ie"]
        result["accuracy_128k_sampled_rows"] = acc
        # the other configs' parity subsets
        tiny = WORKLOADS["tiny_fp32"]
        t0 = time.perf_counter()
        for Lt in (256, 64):
            a1, b1, c1, _ = make_qkv(tiny["seed"], Lt, tiny["Hq"], tiny["Hkv"], tiny["d"],
                                     tiny["std"], tiny["dtype"])
            bifocal_attention(a1, b1, c1, tiny["w0"], tiny["w_pre"], tiny["theta"])
        dt = time.perf_counter() - t0
        cpu_per["tiny_fp32"] = {"seconds": round(dt, 4), "rows_per_s": round(320 / dt, 2),
                                "sample": "all rows of L = 256 and L = 64 (1 head)"}
        cdec = WORKLOADS["decode_128k"]
        dsteps = {}
        for pos in cdec["decode_positions"]:
            t0 = time.perf_counter()
            decode_row(xq[pos], xk, v, pos, w0, w_pre, theta)
            dsteps[str(pos)] = round(time.perf_counter() - t0, 4)
        cpu_per["decode_128k"] = {
            "seconds_per_step": dsteps,
            "sample": "every step in full (all heads, keys 0..pos) on the prefill_128k cache"}
        cpu_per["prefill_128k"] = {k2: result["cpu_baseline"][k2]
                                   for k2 in ("seconds", "rows_per_s", "sample")}
        result["cpu_baseline"]["per_config"] = cpu_per
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
