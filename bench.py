"""Benchmark of the FlashAttention forward hot path on one MI355X.

One step = one pass of the whole hot path on resident synthetic inputs:
  * prefill: fa_forward on the causal GQA long-context workload
    (bf16, B=1, Hq=64, Hkv=8, N=32768, d=128) — one kernel launch;
  * decode:  fa_decode_splitkv on the GQA decode workload (bf16, B=16, Hq=64,
    Hkv=8, d=128, per-sequence key counts ~U[4096, 32768], chunk=256: key work
    split over the waves in runs of at least 256 keys) — the split kernel and
    the merge kernel.  The K and V caches come from the library's allocation helper
    (kv_cache_empty: one buffer, V 256 bytes off K's 1 KiB congruence class); the same
    decode on two separate allocations is timed as well and reported beside it.
`value` is the prefill's algorithmic TFLOP/s (4*B*Hq*Nq*Nk*d / 2 for causal) over
its measured kernel time; the decode's HBM GB/s (compulsory K/V/q/O/LSE bytes)
is reported alongside, and so are the paged-KV decode, the packed variable-length
prefill (16 causal GQA sequences, lengths ~U[512, 16384], one launch), the FP8 forward,
the backward pass on the prefill workload's shape, and the two other prefill workloads (the
peaky causal MHA one, B=1 H=32 N=8192 d=128 with Q, K x1.5, and the short causal MHA one,
B=2 H=12 N=2048 d=64, each with its own roofline fraction), each timed on its own after the
step.  The decode's reported rate is that of back-to-back decode calls; the same call timed
inside the step (right after each 15 ms prefill) is reported beside it as `in_step`.  Kernel times come from HIP events recorded on the
stream the kernels are launched on (torch's current stream), around every
launch of the timed region.

Prints ONE JSON line.  `python bench.py --gpus N` with N > 1 exits: the library
runs on one GPU only.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6   # MI355X dense bf16 MFMA (256 CU x 2.4 GHz x 4096 FLOP/clk)
PEAK_HBM_GBS = 8000.0       # MI355X HBM3E
PEAK_FP8_TFLOPS = 5033.2    # MI355X dense fp8 MFMA (twice the bf16 rate)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--prefill", default="c4", choices=["c2", "c3", "c4"],
                    help="prefill workload (default: the long-context GQA one)")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--no-legs", action="store_true",
                    help="skip the other prefill workloads (short MHA and peaky 8K MHA), each "
                         "timed on its own after the step")
    ap.add_argument("--no-paged", action="store_true",
                    help="skip the paged-KV decode measurement (reported beside the step)")
    ap.add_argument("--no-varlen", action="store_true",
                    help="skip the packed variable-length prefill measurement (reported beside "
                         "the step)")
    ap.add_argument("--no-fp8", action="store_true",
                    help="skip the FP8 forward measurement (reported beside the step)")
    ap.add_argument("--no-backward", action="store_true",
                    help="skip the backward-pass measurement (reported beside the step)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-power", action="store_true",
                    help="skip the board power / clock sampling (under the prefill and the "
                         "other compute legs) and the ceiling legs (matrix cores, HBM "
                         "streaming read)")
    ap.add_argument("--cpu-seconds", type=float, default=15.0,
                    help="target CPU time of the oracle sample")
    ap.add_argument("--copy-calib", action="store_true",
                    help="only run a plain 1 GiB device copy (HBM counter calibration)")
    return ap.parse_args()


def profiled_traffic(kernel: str):
    """HBM bytes per dispatch of `kernel` from profiles/hbm_traffic.json (rocprofv3 FETCH_SIZE
    and WRITE_SIZE, copy-calibrated), or None when the kernel's sources changed since then."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "hbm_traffic.json")
    try:
        with open(path) as f:
            rec = json.load(f)[kernel]
        h = hashlib.sha256()
        for src in rec["sources"]:
            with open(os.path.join(ROOT, src), "rb") as f:
                h.update(f.read())
        if h.hexdigest() != rec["sources_sha256"]:
            return None
        return rec["traffic_bytes"]
    except (OSError, KeyError, ValueError):
        return None


def copy_calib():
    import torch
    n = 1 << 30
    a = torch.empty(n, dtype=torch.uint8, device="cuda")
    a.fill_(1)
    b = torch.empty_like(a)
    torch.cuda.synchronize()
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"copy_calib_bytes_each_way": n, "launches": 3}))


def cpu_baseline_prefill(cfg, target_s):
    """The fp64 oracle on a bounded sample of the prefill workload: the last R query
    rows (each sees ~all keys) of the first H query heads, R grown to the whole
    sequence first, then H, until the sample takes ~target_s."""
    import torch
    import oracle
    import workloads as W
    q, k, v = W.prefill_inputs_for(cfg)
    N, d = cfg.Nq, cfg.d
    R, H = 64, 1
    while True:
        r0 = N - R
        t0 = time.perf_counter()
        oracle.attention(q, k, v, cfg.scale, cfg.causal, heads=list(range(H)), rows=(r0, N),
                         row_block=256)
        dt = time.perf_counter() - t0
        if dt * 2 > target_s or (R >= N and H >= cfg.Hq):
            break
        if R < N:
            R = min(N, R * 2)
        else:
            H = min(cfg.Hq, H * 2)
    if cfg.causal:
        keys = sum(min(cfg.Nk, i + (cfg.Nk - cfg.Nq) + 1) for i in range(r0, N))
    else:
        keys = R * cfg.Nk
    keys *= H
    flops = 4.0 * d * keys
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{cfg.name}: query heads 0..{H - 1}, query rows {r0}..{N - 1} ({R} rows "
                      f"per head, {keys} visible (row,key) pairs), fp64 torch CPU standard "
                      f"attention"}


def cpu_baseline_backward(cfg, target_s):
    """The fp64 oracle backward on a bounded sample of the same shape: dQ of the last R
    query rows of the query heads of K/V head 0, R doubled until the sample takes
    ~target_s.  FLOP counted for what the sample computes: the S, dP and dQ products
    (3 of the backward's 5), 6 d per visible (row, key) pair."""
    import torch
    import oracle
    import workloads as W
    q, k, v, do = W.backward_inputs(cfg.B, cfg.Hq, cfg.Hkv, cfg.Nq, cfg.Nk, cfg.d, seed=0,
                                    qk_gain=cfg.qk_gain)
    N, d, G = cfg.Nq, cfg.d, cfg.Hq // cfg.Hkv
    R = 16
    while True:
        r0 = N - R
        t0 = time.perf_counter()
        oracle.attention_backward(q, k, v, do, cfg.scale, cfg.causal, kv_heads=[0], rows=(r0, N),
                                  keys=(0, 0), row_block=64)
        dt = time.perf_counter() - t0
        if dt * 2 > target_s or R >= N:
            break
        R = min(N, R * 2)
    if cfg.causal:
        keys = sum(min(cfg.Nk, i + (cfg.Nk - cfg.Nq) + 1) for i in range(r0, N))
    else:
        keys = R * cfg.Nk
    keys *= G
    flops = 6.0 * d * keys
    return {"value": flops / dt / 1e12, "unit": "TFLOP/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "seconds": round(dt, 3),
            "sample": f"{cfg.name}: dQ of query rows {r0}..{N - 1} of the {G} query heads of K/V "
                      f"head 0 ({keys} visible (row,key) pairs; S, dP, dQ products = 6 d FLOP "
                      f"per pair), fp64 torch CPU (P, dP, dS materialised)"}


def bench_paged(fa, W, dcfg, dec, dev, K, page_size=256):
    """The same decode step with the KV cache scattered over a permuted pool of
    `page_size`-key pages (paged KV cache), timed on its own after the step."""
    import torch
    print("[bench] paged decode", file=sys.stderr, flush=True)
    kp_h, vp_h, table = W.paged_from_contiguous(dec["kc"], dec["vc"], dec["lengths"], page_size,
                                                seed=7, spare_pages=9)
    kp, vp = fa.kv_cache_empty(kp_h.shape, device=dev)  # page pools laid out as the caches
    kp.copy_(kp_h.to(dev))
    vp.copy_(vp_h.to(dev))
    table = table.to(dev)
    o = torch.empty_like(dec["o"])
    lse = torch.empty_like(dec["lse"])
    nbytes = fa.fa_decode_splitkv_workspace_bytes(dcfg.B, dcfg.Hq, table.shape[1] * page_size,
                                                  dcfg.d, dcfg.chunk)
    ws = torch.empty((nbytes,), dtype=torch.uint8, device=dev)

    def call():
        fa.fa_decode_paged(dec["dq"], kp, vp, table, dec["dl"], scale=dcfg.scale,
                           chunk=dcfg.chunk, o=o, lse=lse, workspace=ws)
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / K
    dbytes = W.decode_bytes(dec["lengths"].tolist(), dcfg.Hq, dcfg.Hkv, dcfg.d)
    gbs = dbytes / (avg * 1e-3) / 1e9
    return {"value": round(gbs, 1), "unit": "GB/s", "bound": "hbm", "peak": PEAK_HBM_GBS,
            "frac": round(gbs / PEAK_HBM_GBS, 4), "avg_call_ms": round(avg, 4),
            "median_call_ms": round(sorted(ms)[K // 2], 4), "page_size": page_size,
            "pool_pages": int(kp.shape[0]),
            "layout": "c5 keys in a seeded permutation of a page pool, block table per sequence"}


def bench_decode_separate(fa, W, dcfg, dec, dev, K):
    """The decode step with the K and V caches as two separate allocations (each 2 MiB
    aligned, so their starts are congruent modulo 1 KiB), timed on its own: the layout
    kv_cache_empty avoids, reported for comparison."""
    import torch
    print("[bench] decode, separate K/V allocations", file=sys.stderr, flush=True)
    kc2, vc2 = dec["kc"].to(dev), dec["vc"].to(dev)
    o = torch.empty_like(dec["o"])
    lse = torch.empty_like(dec["lse"])

    def call():
        fa.fa_decode_splitkv(dec["dq"], kc2, vc2, dec["dl"], scale=dcfg.scale,
                             chunk=dcfg.chunk, o=o, lse=lse, workspace=dec["ws"])
    for _ in range(5):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / K
    dbytes = W.decode_bytes(dec["lengths"].tolist(), dcfg.Hq, dcfg.Hkv, dcfg.d)
    gbs = dbytes / (avg * 1e-3) / 1e9
    rel = (vc2.data_ptr() - kc2.data_ptr()) % 1024
    del kc2, vc2
    torch.cuda.empty_cache()
    return {"value": round(gbs, 1), "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
            "avg_call_ms": round(avg, 4), "v_minus_k_mod_1KiB": int(rel)}


def bench_varlen(fa, W, dev, K):
    """The packed variable-length prefill (16 causal GQA sequences of U[512, 16384] tokens in
    one launch), timed on its own after the step; algorithmic TFLOP/s summed per sequence."""
    import torch
    cfg = W.VARLEN["v1"]
    print(f"[bench] generating {cfg.name} inputs", file=sys.stderr, flush=True)
    lengths, cu_q, cu_k, q, k, v = W.varlen_inputs_for(cfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    del q, k, v
    cqd, ckd = cu_q.to(dev), cu_k.to(dev)
    tq = int(cu_q[-1])
    o = torch.empty((tq, cfg.Hq, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.Hq, tq), dtype=torch.float32, device=dev)
    max_q = int(lengths.max())

    def call():
        fa.fa_forward_varlen(qd, kd, vd, cqd, ckd, max_q, max_q, scale=cfg.scale,
                             causal=cfg.causal, o=o, lse=lse)
    print("[bench] packed varlen prefill", file=sys.stderr, flush=True)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item(), "non-finite output"
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / K
    flops = W.varlen_flops(lengths, lengths, cfg.Hq, cfg.d, cfg.causal)
    tf = flops / (avg * 1e-3) / 1e12
    return {"value": round(tf, 2), "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
            "frac": round(tf / PEAK_BF16_TFLOPS, 4), "avg_launch_ms": round(avg, 4),
            "median_launch_ms": round(sorted(ms)[K // 2], 4), "flop_per_launch": flops,
            "workload": cfg.workload, "total_tokens": tq, "max_seqlen": max_q,
            "kernel": "prefill_bf16_kernel<128, causal, varlen>"}


def bench_fp8(fa, W, pcfg, dev, K, power=False):
    """fa_forward_fp8 on the prefill workload's shape (E4M3 codes of the same seeded draws,
    per-tensor descales), timed on its own after the step; FLOP as the bf16 prefill.  With
    `power`, board power and clocks are then sampled while the launch repeats."""
    import torch
    print(f"[bench] fp8 forward on {pcfg.name}", file=sys.stderr, flush=True)
    q8, k8, v8, qd, kd, vd = W.fp8_inputs(pcfg.B, pcfg.Hq, pcfg.Hkv, pcfg.Nq, pcfg.Nk, pcfg.d,
                                          seed=0, qk_gain=pcfg.qk_gain)
    q8, k8, v8 = q8.to(dev), k8.to(dev), v8.to(dev)
    o = torch.empty((pcfg.B, pcfg.Nq, pcfg.Hq, pcfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((pcfg.B, pcfg.Hq, pcfg.Nq), dtype=torch.float32, device=dev)

    def call():
        fa.fa_forward_fp8(q8, k8, v8, qd, kd, vd, scale=pcfg.scale, causal=pcfg.causal, o=o,
                          lse=lse)
    for _ in range(3):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item(), "non-finite output"
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / K
    flops = pcfg.flops()
    tf = flops / (avg * 1e-3) / 1e12
    res = {"value": round(tf, 2), "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_FP8_TFLOPS,
           "frac": round(tf / PEAK_FP8_TFLOPS, 4), "frac_of_bf16_peak": round(tf / PEAK_BF16_TFLOPS, 4),
           "avg_launch_ms": round(avg, 4), "median_launch_ms": round(sorted(ms)[K // 2], 4),
           "flop_per_launch": flops, "workload": pcfg.workload + " as E4M3 codes",
           "kernel": "prefill_fp8_kernel<128, causal>"}
    if power:
        pw = power_leg(call, torch.cuda.synchronize, seconds=3.0)
        if pw is not None:
            pw["pj_per_flop"] = round(pw["socket_power_w_median"] / (tf * 1e12) * 1e12, 3)
        res["power"] = pw
    return res


def bench_backward(fa, W, pcfg, dev, K, power=False):
    """fa_backward on the prefill workload's shape (seeded Q, K, V, dO; O and LSE from the
    GPU forward, outside the timed region), timed on its own after the step.  Algorithmic
    FLOP: the usual 2.5x the forward's (five products per visible pair: S, dP, dV, dK,
    dQ); the kernels execute seven (S and dP are formed on both the dK/dV and the dQ
    side), reported as executed_tflops.  With `power`, board power and clocks are then
    sampled while the call repeats."""
    import torch
    print(f"[bench] backward on {pcfg.name}", file=sys.stderr, flush=True)
    q, k, v, do = W.backward_inputs(pcfg.B, pcfg.Hq, pcfg.Hkv, pcfg.Nq, pcfg.Nk, pcfg.d, seed=0,
                                    qk_gain=pcfg.qk_gain)
    qd, kd, vd, dod = q.to(dev), k.to(dev), v.to(dev), do.to(dev)
    del q, k, v, do
    o, lse = fa.fa_forward(qd, kd, vd, scale=pcfg.scale, causal=pcfg.causal)
    dq = torch.empty_like(o)
    dk = torch.empty(kd.shape, dtype=torch.float32, device=dev)
    dv = torch.empty_like(dk)
    ws = torch.empty((fa.fa_backward_workspace_bytes(pcfg.B, pcfg.Hq, pcfg.Nq),),
                     dtype=torch.uint8, device=dev)

    def call():
        fa.fa_backward(qd, kd, vd, o, lse, dod, scale=pcfg.scale, causal=pcfg.causal, dq=dq,
                       dk=dk, dv=dv, workspace=ws)
    for _ in range(2):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    for t in (dq, dk, dv):
        assert torch.isfinite(t).all().item(), "non-finite gradient"
    ms = [a.elapsed_time(b) for a, b in ev]
    avg = sum(ms) / K
    flops = 2.5 * pcfg.flops()
    tf = flops / (avg * 1e-3) / 1e12
    res = {"value": round(tf, 2), "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
           "frac": round(tf / PEAK_BF16_TFLOPS, 4), "avg_call_ms": round(avg, 4),
           "median_call_ms": round(sorted(ms)[K // 2], 4), "flop_per_call": flops,
           "executed_tflops": round(tf * 7 / 5, 2), "workload": pcfg.workload,
           "kernels": "prep (D, lse2) + dK/dV per 256 keys + dQ per 128 rows (one call)"}
    if power:
        pw = power_leg(call, torch.cuda.synchronize, seconds=3.0)
        if pw is not None:
            pw["pj_per_flop"] = round(pw["socket_power_w_median"] / (tf * 1e12) * 1e12, 3)
        res["power"] = pw
    return res


def bench_prefill_leg(fa, W, name, dev, launches, min_seconds=0.3, power=False):
    """Another prefill workload of the same kernel (the short MHA one, or the peaky 8K MHA
    one), timed on its own after the step: `launches` back-to-back launches in ten groups,
    each group between two HIP events on the stream the kernel runs on, so the figure is the
    kernels' own rate (an event pair around every launch of a 25 us kernel adds the events'
    own few microseconds to each; that per-launch figure is reported beside it);
    algorithmic TFLOP/s as for the step.  With `power`, board power and clocks are then
    sampled while the launch repeats."""
    import torch
    cfg = W.CONFIGS[name]
    print(f"[bench] prefill leg {name}", file=sys.stderr, flush=True)
    q, k, v = W.prefill_inputs_for(cfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty((cfg.B, cfg.Nq, cfg.Hq, cfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((cfg.B, cfg.Hq, cfg.Nq), dtype=torch.float32, device=dev)

    def call():
        fa.fa_forward(qd, kd, vd, scale=cfg.scale, causal=cfg.causal, o=o, lse=lse)
    t0 = time.perf_counter()
    n = 0
    while n < 10 or time.perf_counter() - t0 < min_seconds:
        call()
        n += 1
        if n % 16 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    groups = 10
    per_group = max(1, launches // groups)
    launches = groups * per_group
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(groups)]
    for a, b in ev:
        a.record()
        for _ in range(per_group):
            call()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) / per_group for a, b in ev]
    avg = sum(ms) / groups
    # the same launches, each between its own pair of events
    ev1 = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(min(launches, 200))]
    for a, b in ev1:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item(), "non-finite output"
    ms1 = sorted(a.elapsed_time(b) for a, b in ev1)
    flops = cfg.flops()
    tf = flops / (avg * 1e-3) / 1e12
    res = {"value": round(tf, 2), "unit": "TFLOP/s", "bound": "mfma", "peak": PEAK_BF16_TFLOPS,
           "frac": round(tf / PEAK_BF16_TFLOPS, 4), "avg_launch_ms": round(avg, 4),
           "median_launch_ms": round(sorted(ms)[groups // 2], 4), "launches": launches,
           "timing": f"{groups} groups of {per_group} back-to-back launches, one event pair "
                     "per group",
           "per_launch_event_median_ms": round(ms1[len(ms1) // 2], 4),
           "flop_per_launch": flops, "workload": cfg.workload,
           "kernel": f"prefill_bf16_kernel<{cfg.d}, causal>"}
    if power:
        # launches grouped so that a group lasts at least ~0.5 ms between host syncs
        group = max(1, int(math.ceil(0.5 / max(avg, 1e-3))))

        def run_group():
            for _ in range(group):
                call()
        pw = power_leg(run_group, torch.cuda.synchronize, seconds=3.0)
        if pw is not None:
            pw["pj_per_flop"] = round(pw["socket_power_w_median"] / (tf * 1e12) * 1e12, 3)
        res["power"] = pw
    return res


def parse_smi_metric(text):
    """(socket power in W, [GFX clock of each XCD in MHz]) from `amd-smi metric -p -c` text,
    or None when either is missing."""
    import re
    pw = re.search(r"SOCKET_POWER:\s*([0-9.]+)\s*W", text)
    clks = [float(x) for x in re.findall(r"GFX_\d+:\s*\n\s*CLK:\s*([0-9.]+)\s*MHz", text)]
    if not pw or not clks:
        return None
    return float(pw.group(1)), clks


def power_sampled(workload):
    """Runs `workload()` while a child process samples `amd-smi metric -g 0 -p -c` (socket
    power, per-XCD GFX clocks) every ~0.3 s; returns (workload's result, power summary).
    The first two samples (clock ramp) are dropped; the summary is None when amd-smi is
    not available."""
    import shutil
    import subprocess
    import threading
    smi = shutil.which("amd-smi") or "/opt/rocm/bin/amd-smi"
    if not os.path.exists(smi):
        return workload(), None
    samples = []
    stop = threading.Event()

    def sampler():
        while not stop.is_set():
            try:
                r = subprocess.run([smi, "metric", "-g", "0", "-p", "-c"], capture_output=True,
                                   text=True, timeout=20)
            except (OSError, subprocess.SubprocessError):
                return
            got = parse_smi_metric(r.stdout)
            if got is not None:
                samples.append(got)
            stop.wait(0.3)

    th = threading.Thread(target=sampler, daemon=True)
    th.start()
    try:
        res = workload()
    finally:
        stop.set()
        th.join(timeout=30)
    use = samples[2:] if len(samples) > 4 else samples
    if not use:
        return res, None
    med = lambda xs: sorted(xs)[len(xs) // 2]
    watts = [w for w, _ in use]
    clk_mean = [sum(c) / len(c) for _, c in use]
    return res, {"socket_power_w_median": med(watts), "socket_power_w_max": max(watts),
                 "gfx_clock_mhz_median": round(med(clk_mean), 1),
                 "gfx_clock_mhz_range": [min(min(c) for _, c in use),
                                         max(max(c) for _, c in use)],
                 "board_power_limit_w": 1400, "samples": len(use),
                 "source": "amd-smi metric -g 0 -p -c every ~0.3 s while the launch repeats "
                           "back to back (board limit: the published MI355X total board power)"}


def power_leg(run, sync, seconds=4.0):
    """Board power and engine clocks while `run` (one prefill launch) repeats back to back
    for `seconds`."""
    def work():
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < seconds:
            run()
            n += 1
            if n % 4 == 0:
                sync()
        sync()
        return n
    n, pw = power_sampled(work)
    if pw is not None:
        pw["launches"] = n
    return pw


def mfma_ceiling_leg(fa, dev, seconds=4.0):
    """The bf16 matrix cores' sustained rate under the same power limit (fa_probe_mfma_bf16:
    independent 32x32x16 MFMAs on random bf16 register operands, no memory traffic, two
    waves per SIMD like the prefill), timed with HIP events over back-to-back launches of
    ~15 ms while power and clocks are sampled."""
    import torch
    print("[bench] matrix-core ceiling", file=sys.stderr, flush=True)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    blocks = 2 * cus
    g = torch.Generator(device="cpu").manual_seed(7)
    nb = fa.fa_probe_mfma_bf16_operand_bytes(blocks)
    ops = torch.randn(nb // 2, generator=g).to(torch.bfloat16).to(dev)
    out = torch.empty(blocks * 256, dtype=torch.float32, device=dev)
    iters = 100000
    flop = fa.fa_probe_mfma_bf16(ops, out, blocks, iters)  # warm
    torch.cuda.synchronize()

    def work():
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        n = 0
        e0.record()
        while time.perf_counter() - t0 < seconds:
            for _ in range(4):
                fa.fa_probe_mfma_bf16(ops, out, blocks, iters)
            n += 4
            torch.cuda.synchronize()
        e1.record()
        e1.synchronize()
        return n, e0.elapsed_time(e1)

    (n, ms), pw = power_sampled(work)
    assert torch.isfinite(out).all().item()
    tflops = flop * n / (ms * 1e-3) / 1e12
    return {"value": round(tflops, 1), "unit": "TFLOP/s", "peak": PEAK_BF16_TFLOPS,
            "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4), "launches": n,
            "avg_launch_ms": round(ms / n, 3), "power": pw,
            "method": "fa_probe_mfma_bf16: per thread four independent v_mfma_f32_32x32x16_bf16 "
                      "accumulators (VGPR form), every instruction on a different pair of random "
                      "bf16 register operands, no memory traffic; "
                      f"{blocks} workgroups of 256 threads (two waves per SIMD), {iters} "
                      "iterations per launch"}


def stream_ceiling_leg(fa, dev, nbytes, launches=40):
    """The HBM streaming-read rate on the same board (fa_probe_stream_read: every byte of a
    buffer as large as the decode's K/V stream read once, 16 bytes per lane per load, the
    decode's non-temporal cache policy, eight loads in flight per lane), over a few grid
    sizes, each timed with HIP events over back-to-back launches; the best is reported."""
    import torch
    print("[bench] streaming-read ceiling", file=sys.stderr, flush=True)
    cus = torch.cuda.get_device_properties(dev).multi_processor_count
    nbytes = min(int(nbytes) // 16 * 16, 1 << 31)
    g = torch.Generator(device="cpu").manual_seed(11)
    buf = torch.randint(-2**31, 2**31 - 1, (nbytes // 4,), generator=g,
                        dtype=torch.int32).to(dev)
    per = {}
    for mult in (4, 8, 16):
        blocks = mult * cus
        out = torch.empty(blocks * 256, dtype=torch.int32, device=dev)
        for _ in range(3):
            fa.fa_probe_stream_read(buf, out, blocks)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(launches):
            fa.fa_probe_stream_read(buf, out, blocks)
        e1.record()
        e1.synchronize()
        ms = e0.elapsed_time(e1) / launches
        per[f"{blocks}x256"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
        del out
    del buf
    torch.cuda.empty_cache()
    best = max(per.values())
    return {"value": best, "unit": "GB/s", "peak": PEAK_HBM_GBS,
            "frac_of_peak": round(best / PEAK_HBM_GBS, 4), "bytes": nbytes,
            "launches_per_grid": launches, "by_grid": per,
            "method": "fa_probe_stream_read: one pass over a buffer of the decode's byte count, "
                      "16-byte non-temporal buffer loads, each wave instruction 1 KB "
                      "contiguous, 32 KB chunks per workgroup, grid sizes as listed"}


def decode_piece_steps(lengths, dcfg, cus):
    """The decode's real split: all (batch, K/V head, head group) segments laid end to end
    in 64-key steps, T steps in all, cut into equal runs of R = max(ceil(T / W), chunk / 64)
    steps over the W = 4 * CUs persistent waves (the rule the split kernel applies)."""
    G = dcfg.Hq // dcfg.Hkv
    QG = (G + 15) // 16
    T = sum((int(L) + 63) // 64 for L in lengths) * dcfg.Hkv * QG
    Wv = 4 * cus
    R = max((T + Wv - 1) // Wv, dcfg.chunk // 64)
    return T, Wv, R


def bench_decode_isolated(fa, W, dcfg, dec, K):
    """The step's decode call (caches from kv_cache_empty) timed on its own: K back-to-back
    calls, each between two HIP events, with no prefill launched in between."""
    import torch

    def call():
        fa.fa_decode_splitkv(dec["dq"], dec["dkc"], dec["dvc"], dec["dl"], scale=dcfg.scale,
                             chunk=dcfg.chunk, o=dec["o"], lse=dec["lse"], workspace=dec["ws"])
    print("[bench] decode, isolated", file=sys.stderr, flush=True)
    for _ in range(20):
        call()
    torch.cuda.synchronize()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(K)]
    for a, b in ev:
        a.record()
        call()
        b.record()
    torch.cuda.synchronize()
    ms = [a.elapsed_time(b) for a, b in ev]
    return sum(ms) / K, sorted(ms)[K // 2]


def cpu_baseline_decode(cfg, lengths, q, kc, vc, target_s):
    import torch
    import oracle
    import workloads as W
    bs = []
    t_total = 0.0
    byts = 0.0
    for b in range(cfg.B):
        t0 = time.perf_counter()
        oracle.decode_attention(q, kc, vc, lengths, cfg.scale, batches=[b])
        t_total += time.perf_counter() - t0
        bs.append(b)
        byts += W.decode_bytes([int(lengths[b])], cfg.Hq, cfg.Hkv, cfg.d)
        if t_total > target_s:
            break
    return {"value": byts / t_total / 1e9, "unit": "GB/s", "cores": torch.get_num_threads(),
            "kind": "oracle", "seconds": round(t_total, 3),
            "sample": f"{cfg.name}: sequences {bs} (all {cfg.Hq} query heads), fp64 torch CPU"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: the library runs on exactly one GPU; --gpus {args.gpus} is not supported "
              f"(no collectives or sharding are implemented).", file=sys.stderr)
        sys.exit(2)
    import torch
    if args.copy_calib:
        copy_calib()
        return
    import io_aware_attention_attn_amd as fa
    import workloads as W

    dev = torch.device("cuda", 0)
    pcfg = W.CONFIGS[args.prefill]
    dcfg = W.CONFIGS["c5"]

    print(f"[bench] generating {pcfg.name} inputs", file=sys.stderr, flush=True)
    q, k, v = W.prefill_inputs_for(pcfg)
    qd, kd, vd = q.to(dev), k.to(dev), v.to(dev)
    o = torch.empty((pcfg.B, pcfg.Nq, pcfg.Hq, pcfg.d), dtype=torch.float32, device=dev)
    lse = torch.empty((pcfg.B, pcfg.Hq, pcfg.Nq), dtype=torch.float32, device=dev)

    dec = None
    if not args.no_decode:
        print(f"[bench] generating {dcfg.name} inputs", file=sys.stderr, flush=True)
        lengths, dq, kc, vc = W.decode_inputs_for(dcfg)
        # K and V caches from the library's allocation helper (one buffer, V 256 bytes off
        # the K cache's 1 KiB congruence class); the two-allocation layout is timed too
        dkc, dvc = fa.kv_cache_empty(kc.shape, device=dev)
        dkc.copy_(kc.to(dev))
        dvc.copy_(vc.to(dev))
        dec = dict(lengths=lengths, q=dq, kc=kc, vc=vc,
                   dq=dq.to(dev), dkc=dkc, dvc=dvc, dl=lengths.to(dev))
        dec["o"] = torch.empty((dcfg.B, dcfg.Hq, dcfg.d), dtype=torch.float32, device=dev)
        dec["lse"] = torch.empty((dcfg.B, dcfg.Hq), dtype=torch.float32, device=dev)
        nbytes = fa.fa_decode_splitkv_workspace_bytes(dcfg.B, dcfg.Hq, dcfg.Nk_max, dcfg.d,
                                                      dcfg.chunk)
        dec["ws"] = torch.empty((nbytes,), dtype=torch.uint8, device=dev)
    torch.cuda.synchronize()

    def prefill():
        fa.fa_forward(qd, kd, vd, scale=pcfg.scale, causal=pcfg.causal, o=o, lse=lse)

    def decode():
        fa.fa_decode_splitkv(dec["dq"], dec["dkc"], dec["dvc"], dec["dl"], scale=dcfg.scale,
                             chunk=dcfg.chunk, o=dec["o"], lse=dec["lse"], workspace=dec["ws"])

    print("[bench] warmup", file=sys.stderr, flush=True)
    # At least `warmup` steps and at least half a second of GPU work, so clocks have
    # ramped up before the timed region even when one step is short.
    t_w = time.perf_counter()
    done = 0
    while done < args.warmup or time.perf_counter() - t_w < 0.5:
        prefill()
        if dec:
            decode()
        done += 1
        if done % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()

    K = args.steps
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(K)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    print("[bench] timed region", file=sys.stderr, flush=True)
    torch.cuda.synchronize()
    t_wall = time.perf_counter()
    start.record()
    for i in range(K):
        ev[i][0].record()
        prefill()
        ev[i][1].record()
        if dec:
            ev[i][2].record()
            decode()
            ev[i][3].record()
    end.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t_wall
    total_ms = start.elapsed_time(end)
    pre_ms = [e[0].elapsed_time(e[1]) for e in ev]
    avg_pre = sum(pre_ms) / K
    flops = pcfg.flops()
    tflops = flops / (avg_pre * 1e-3) / 1e12
    assert torch.isfinite(o).all().item() and torch.isfinite(lse).all().item(), "non-finite output"

    result = {
        "metric": "attn fwd TFLOP/s and % bf16 MFMA peak (prefill); decode HBM GB/s and % peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": round(total_ms / K, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) inputs rounded to bf16; no dataset or weights)",
        "config": {"workload": pcfg.workload, "B": pcfg.B, "Hq": pcfg.Hq, "Hkv": pcfg.Hkv,
                   "seq_len": pcfg.Nq, "head_dim": pcfg.d, "causal": pcfg.causal,
                   "decode_workload": None if not dec else dcfg.workload + " (minimum run; "
                                     "real runs in decode.piece_keys)",
                   "parallelism": "single GPU"},
        "roofline": {"bound": "mfma", "kernel": "prefill_bf16_kernel<128, causal>",
                     "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": (profiled_traffic("prefill_bf16_kernel<128, 4, true, false, false>")
                                 if pcfg.d == 128 and pcfg.causal else None),
                     "traffic_unit": "bytes per launch (HBM, rocprofv3 FETCH_SIZE+WRITE_SIZE)",
                     "avg_launch_ms": round(avg_pre, 4),
                     "median_launch_ms": round(sorted(pre_ms)[K // 2], 4),
                     "flop_per_launch": flops},
        "wall_s_timed_region": round(wall, 3),
    }
    if not args.no_power:
        print("[bench] power and clocks under the prefill", file=sys.stderr, flush=True)
        pw = power_leg(prefill, torch.cuda.synchronize)
        if pw is not None:
            pw["pj_per_flop"] = round(pw["socket_power_w_median"] / (tflops * 1e12) * 1e12, 3)
        result["roofline"]["power"] = pw
        ceil = mfma_ceiling_leg(fa, dev)
        ceil["kernel_frac_of_ceiling"] = round(tflops / ceil["value"], 4)
        result["roofline"]["mfma_ceiling"] = ceil
    if dec:
        dbytes = W.decode_bytes(dec["lengths"].tolist(), dcfg.Hq, dcfg.Hkv, dcfg.d)
        dec_ms = [e[2].elapsed_time(e[3]) for e in ev]
        step_avg = sum(dec_ms) / K
        step_gbs = dbytes / (step_avg * 1e-3) / 1e9
        iso_avg, iso_med = bench_decode_isolated(fa, W, dcfg, dec, max(K, 50))
        gbs = dbytes / (iso_avg * 1e-3) / 1e9
        cus = torch.cuda.get_device_properties(dev).multi_processor_count
        T, Wv, R = decode_piece_steps(dec["lengths"].tolist(), dcfg, cus)
        result["decode"] = {"value": round(gbs, 1), "unit": "GB/s", "bound": "hbm",
                            "peak": PEAK_HBM_GBS, "frac": round(gbs / PEAK_HBM_GBS, 4),
                            "timing": f"{max(K, 50)} back-to-back decode calls, each between "
                                      f"HIP events (in_step: the same call timed inside the "
                                      f"step, right after each prefill)",
                            "avg_call_ms": round(iso_avg, 4), "median_call_ms": round(iso_med, 4),
                            "in_step": {"value": round(step_gbs, 1), "unit": "GB/s",
                                        "frac": round(step_gbs / PEAK_HBM_GBS, 4),
                                        "avg_call_ms": round(step_avg, 4),
                                        "median_call_ms": round(sorted(dec_ms)[K // 2], 4)},
                            "kernels": "split + merge (one call)",
                            "split": f"key work of all (batch, K/V head) segments laid end to end "
                                     f"in 64-key steps ({T} steps) and cut into equal runs of "
                                     f"R = max(ceil(T / W), chunk / 64) = {R} steps ({64 * R} "
                                     f"keys) over W = {Wv} persistent waves; a piece is a run's "
                                     f"part inside one segment (>= chunk keys unless the segment "
                                     f"is shorter); LSE merge of the pieces",
                            "piece_steps": R, "piece_keys": 64 * R, "waves": Wv,
                            "bytes_per_call": dbytes,
                            "sum_seqlens": int(dec["lengths"].sum().item()),
                            "traffic_split": profiled_traffic("decode_split_kernel<128, false>"),
                            "traffic_merge": profiled_traffic("decode_merge_kernel<128>"),
                            "cache_layout": "K and V caches in one allocation with V starting "
                                            "256 B past K's 1 KiB congruence class "
                                            "(kv_cache_empty)"}
        result["decode"]["separate_allocations"] = bench_decode_separate(fa, W, dcfg, dec, dev, K)
        if not args.no_power:
            def decode_group():
                for _ in range(8):
                    decode()
            pw = power_leg(decode_group, torch.cuda.synchronize, seconds=3.0)
            result["decode"]["power"] = pw
            sc = stream_ceiling_leg(fa, dev, dbytes)
            sc["kernel_frac_of_ceiling"] = round(gbs / sc["value"], 4)
            result["decode"]["stream_ceiling"] = sc
    if dec and not args.no_paged:
        result["decode_paged"] = bench_paged(fa, W, dcfg, dec, dev, K)
    if not args.no_varlen or not args.no_backward or not args.no_fp8 or not args.no_legs:
        del qd, kd, vd, o, lse
        torch.cuda.empty_cache()
    if not args.no_legs:
        # the other prefill workloads of the same kernel: the peaky 8K MHA one (N >= 8192,
        # d = 128, the roofline target applies) and the short MHA one
        legs = {}
        for name, launches in (("c3", max(100, 5 * K)), ("c2", 1000)):
            if name != pcfg.name:
                legs[name] = bench_prefill_leg(fa, W, name, dev, launches,
                                               power=not args.no_power)
                torch.cuda.empty_cache()
        result["prefill_legs"] = legs
    if not args.no_varlen:
        result["prefill_varlen"] = bench_varlen(fa, W, dev, K)
        torch.cuda.empty_cache()
    if not args.no_fp8:
        result["prefill_fp8"] = bench_fp8(fa, W, pcfg, dev, K, power=not args.no_power)
        torch.cuda.empty_cache()
    if not args.no_backward:
        result["backward"] = bench_backward(fa, W, pcfg, dev, max(2, K // 4),
                                            power=not args.no_power)
    if not args.no_cpu_baseline:
        print("[bench] cpu baseline (oracle)", file=sys.stderr, flush=True)
        result["cpu_baseline"] = cpu_baseline_prefill(pcfg, args.cpu_seconds)
        if "backward" in result:
            result["backward"]["cpu_baseline"] = cpu_baseline_backward(pcfg, args.cpu_seconds / 3)
        if dec:
            result["decode"]["cpu_baseline"] = cpu_baseline_decode(
                dcfg, dec["lengths"], dec["q"], dec["kc"], dec["vc"], args.cpu_seconds / 3)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
