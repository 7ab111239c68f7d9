"""Throughput of one compressed-KV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the LLaVA-7B-like layer (batch 32, 32 heads of 128, 2880 visual tokens
factored at rank 64 with 64 dense text tokens, r_lo = 16, 25% of tokens at full
rank, bf16 factors).  One step = one ap_decode_attn call over the batch (latent
query, low-rank scores, per-head top-k, mixed-rank flash-decode, dense text,
combine).  The factored caches are built on the device before timing; R copies
are rotated so that the 256 MB MALL cannot hold the working set.

Timed regions, in order:
  1. the headline: K steps with nothing else on the stream (wall clock around
     synchronisations, and HIP events on the launch stream as a cross-check);
  2. K more steps with the library's per-kernel HIP events (ap_timing_*) for the
     kernel breakdown and the dominant kernel's roofline;
  3. max(K, 100) single calls, each bracketed by its own pair of HIP events on the
     launch stream: median and p10 / p90 per call;
  4. the compressor: ap_recompress of the same batch's K and V (randomized
     subspace iteration), which runs once per cache, not per step;
  5. end to end (--e2e, on by default): ap_compress of the batch-256 4096 x 4096
     layer's 512 K and V matrices followed by 16 decode steps with fresh queries;
  6. the CPU oracle's decode step on a bounded sample of the same sequences.

Prints one JSON line.  `--calib-copy` instead runs only a plain device copy of a
known size (the calibration run for the HBM byte counters).
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0
MALL_BYTES = 256 << 20
METRIC = "compressed-KV decode attention: tokens attended/s + HBM GB/s (% of peak), batch 32"


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cfg", type=int, default=2, help="workload id (2 = the batch-32 LLaVA layer)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--select", default="logit", choices=["logit", "ema_token", "ema_head"],
                    help="which tokens get full rank: the current low-rank logit (default), or "
                         "the moving average of past attention per token or per (head, token)")
    ap.add_argument("--ema-alpha", type=float, default=0.9)
    ap.add_argument("--text-rank", type=int, default=0,
                    help="factor the workload's text tokens apart at this rank (a second segment; "
                         "rank/4 components and a quarter of the text tokens at full rank)")
    ap.add_argument("--storage", default=None, choices=["int4"],
                    help="int4: the workload with 4-bit token factors (U codes + block scales; B, "
                         "K, V and text in bf16)")
    ap.add_argument("--no-compress", action="store_true")
    ap.add_argument("--no-e2e", action="store_true",
                    help="skip the end-to-end leg (compress the batch-256 layer + 16 decode steps)")
    ap.add_argument("--compress-reps", type=int, default=5)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--leg", choices=["compress", "e2e"], default=None,
                    help="run only this leg (for profiling) and print its JSON")
    ap.add_argument("--calib-copy", action="store_true",
                    help="only run a plain 1 GiB device copy 10 times (counter calibration)")
    ap.add_argument("--write-traffic", nargs=4, metavar=("FETCH", "WRITE", "CFETCH", "CWRITE"),
                    help="no GPU: turn rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter CSVs of this "
                         "bench and of --calib-copy into profiles/traffic_<workload>.json")
    return ap.parse_args()


def kernel_bytes(w, select="logit", text_rank=0):
    """Algorithmic bytes per sequence read/written by each decode kernel.  With a
    moving-average selector the importance state (fp32, per token or per (head, token))
    is read by the selection and read + written by the update; the per-step logits the
    update consumes are an intermediate and are not counted."""
    s = 4 if w.storage == "f32" else 2
    W, r, N, T = w.width, w.rank, w.n_tokens, w.n_text
    qb = 4 * w.n_q_heads * w.head_dim
    # one token factor: 4-bit codes plus a bf16 scale per (32-token block, column)
    u = N * r // 2 + (N + 31) // 32 * r * 2 if w.storage == "int4" else s * N * r
    k = {
        "select": s * r * W + qb,                 # B_k, q   (U_k's low panels are re-read, not counted)
        "attn": 2 * u,                            # U_k, U_v
        "combine": s * r * W + s * 2 * T * W + qb,  # B_v, text K/V, out
    }
    if text_rank:
        # the text tokens factored apart: their U (same storage as the visual one) and B
        # replace the dense text rows
        k["combine"] -= s * 2 * T * W
        ut = T * text_rank // 2 + (T + 31) // 32 * text_rank * 2 if w.storage == "int4" else s * T * text_rank
        k["text"] = 2 * ut + 2 * s * text_rank * W + qb
    if select != "logit":
        state = 4 * N * (w.n_q_heads if select == "ema_head" else 1)
        k["select"] += state
        k["ema"] = 2 * state
    k["decode"] = sum(k.values())   # every byte of the step, whichever path runs
    return k


def compress_bytes(w):
    """Algorithmic bytes of one ap_compress/ap_recompress over the batch: 2q + 2
    passes over every K and V matrix (A Omega, q times A^T Q and A Q~, A^T Q)."""
    s = 4 if w.storage == "f32" else 2
    return (2 * w.power_iters + 2) * 2 * w.batch * w.n_tokens * w.width * s


# Sources whose change invalidates measured decode traffic.
DECODE_SOURCES = ["rank_compressed_kv_ap_amd/csrc/select_kernel.hip",
                  "rank_compressed_kv_ap_amd/csrc/decode_kernels.hip",
                  "rank_compressed_kv_ap_amd/csrc/device_common.h",
                  "rank_compressed_kv_ap_amd/csrc/tiles.h",
                  "rank_compressed_kv_ap_amd/csrc/ap_internal.h",
                  "rank_compressed_kv_ap_amd/csrc/api.hip"]
KERNEL_SYMBOL = {"select": "k_select", "attn": "k_attn", "combine": "k_combine", "decode": "k_decode"}


def write_traffic(cfg, fetch_csv, write_csv, cfetch_csv, cwrite_csv):
    """HBM bytes per launch of each decode kernel from two counter runs (FETCH_SIZE,
    WRITE_SIZE, KiB per dispatch), each scaled by what the same counter reads for a
    plain device copy of 1 GiB (the copy reads and writes exactly 2^30 bytes)."""
    import csv

    from rank_compressed_kv_ap_amd import workloads as wl

    def per_kernel(path, counter):
        acc = {}
        for r in csv.DictReader(open(path)):
            if r["Counter_Name"] != counter:
                continue
            acc.setdefault(r["Kernel_Name"], []).append(float(r["Counter_Value"]))
        return acc

    def copy_kib(path, counter):
        vals = [v for name, vs in per_kernel(path, counter).items() if "copyBuffer" in name for v in vs]
        return sum(vals) / len(vals)

    f_scale = (1 << 30) / 1024 / copy_kib(cfetch_csv, "FETCH_SIZE")
    w_scale = (1 << 30) / 1024 / copy_kib(cwrite_csv, "WRITE_SIZE")
    fetch, write = per_kernel(fetch_csv, "FETCH_SIZE"), per_kernel(write_csv, "WRITE_SIZE")
    w = wl.WORKLOADS[cfg]
    kb = kernel_bytes(w)
    kernels = {}
    for k, sym in KERNEL_SYMBOL.items():
        fv = [v for name, vs in fetch.items() if f"ap::{sym}<" in name for v in vs]
        wv = [v for name, vs in write.items() if f"ap::{sym}<" in name for v in vs]
        if not fv or not wv:
            continue
        fb = 1024 * f_scale * sum(fv) / len(fv)
        wb = 1024 * w_scale * sum(wv) / len(wv)
        kernels[k] = {"fetch_bytes": fb, "write_bytes": wb, "bytes_per_launch": fb + wb,
                      "algorithmic_bytes_per_launch": w.batch * kb[k], "dispatches": len(fv)}
    out = {"workload": w.name, "kernels": kernels,
           "calibration": {"fetch_scale": f_scale, "write_scale": w_scale,
                           "copy_bytes": 1 << 30},
           "sources": DECODE_SOURCES, "source_digest": source_digest(DECODE_SOURCES)}
    path = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    with open(path, "w") as fh:
        json.dump(out, fh, indent=1)
    print(json.dumps(out))


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def calib_copy():
    import torch
    n = 1 << 30
    src = torch.ones(n // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(10):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes_read": n, "calib_copy_bytes_written": n, "launches": 10}))


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "the library runs on one GPU; --gpus must be 1"}))
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return
    if args.write_traffic:
        write_traffic(args.cfg, *args.write_traffic)
        return

    import numpy as np
    import torch

    from rank_compressed_kv_ap_amd import binding
    from rank_compressed_kv_ap_amd import workloads as wl

    w = wl.WORKLOADS[args.cfg]
    if args.storage:
        w = w.replace(storage=args.storage)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    if args.leg == "compress":
        print(json.dumps({"compress": compress_leg(w, args.compress_reps, binding, wl, np, torch)}))
        return
    if args.leg == "e2e":
        print(json.dumps({"e2e": e2e_leg(binding, wl, np, torch)}))
        return
    dt = torch.float32 if w.storage == "f32" else torch.bfloat16      # B, text
    du = torch.bfloat16 if w.storage == "bf16" else torch.float32     # U handed to set_factors
    st_arg = "int4" if w.storage == "int4" else dt
    B = w.batch

    # ---- inputs: S distinct seeded sequences tiled over the batch
    S = min(B, 4)
    seqs = [wl.gen_decode_inputs(w, b) for b in range(S)]

    def stack(key, dtype):
        return torch.from_numpy(np.stack([seqs[b % S][key] for b in range(B)])).to(dtype).to(dev)

    kb = kernel_bytes(w, args.select, args.text_rank)
    step_bytes = B * kb["decode"]   # every byte of one step, whichever path runs
    # rotated cache copies: together at least twice the 256 MB last-level cache, and never
    # fewer than two, so that no step finds its factors left in that cache by the step
    # before (a single copy larger than the cache still leaves part of it resident)
    R = max(2, math.ceil(2 * MALL_BYTES / step_bytes))
    caches, qs, texts, tcaches = [], [], [], []
    Rt = args.text_rank
    tr_lo, tk_top = max(1, Rt // 4), (w.n_text + 3) // 4
    if Rt and not (w.n_text and Rt <= w.n_text):
        sys.exit("--text-rank needs a workload with at least that many text tokens")
    for _ in range(R):
        c = binding.compress(None, None, batch=B, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                             n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank, storage=st_arg)
        c.set_factors(stack("U_k", du), stack("B_k", dt), stack("U_v", du), stack("B_v", dt))
        caches.append(c)
        qs.append(stack("q", torch.float32))
        if Rt:
            # the text segment factored on the GPU (ap_compress), no dense text left
            tc = binding.compress(stack("text_k", dt).contiguous(), stack("text_v", dt).contiguous(),
                                  batch=B, n_tokens=w.n_text, n_kv_heads=w.n_kv_heads,
                                  n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=Rt,
                                  storage=st_arg, seed=3)
            tcaches.append(tc)
            texts.append((None, None))
        else:
            tcaches.append(None)
            texts.append((stack("text_k", dt), stack("text_v", dt)) if w.n_text else (None, None))
    out = torch.empty(B, w.n_q_heads * w.head_dim, dtype=torch.float32, device=dev)
    ema = args.select != "logit"
    # moving-average selector: one importance state per cache copy (the first call of
    # each copy has no history), one shared logit workspace
    imps = [torch.zeros((B, w.n_q_heads, w.n_tokens) if args.select == "ema_head" else (B, w.n_tokens),
                        dtype=torch.float32, device=dev) for _ in range(R)] if ema else [None] * R
    scratch = torch.empty(B, w.n_q_heads, w.n_tokens, dtype=torch.float32, device=dev) if ema else None
    first = [True] * R
    torch.cuda.synchronize()

    def step(i):
        j = i % R
        tk, tv = texts[j]
        binding.decode(caches[j], qs[j], r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk,
                       text_v=tv, out=out, splits=args.splits, select=args.select,
                       ema_alpha=args.ema_alpha, ema_first=first[j], importance=imps[j],
                       ema_scratch=scratch, text_cache=tcaches[j], text_r_lo=tr_lo,
                       text_top_k=tk_top)
        first[j] = False

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- 1. headline: K steps, nothing else on the stream
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record()
    for i in range(args.steps):
        step(i)
    ev1.record()
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    event_ms = ev0.elapsed_time(ev1) / args.steps

    # ---- 2. per-kernel breakdown: K steps with HIP events around every kernel
    for c in caches:
        c.timing_enable(math.ceil(args.steps / R) + 1)
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    kms = {k: 0.0 for k in binding.KERNEL_NAMES}
    ncalls = 0
    for c in caches:
        ms, n = c.timing_read()
        ncalls += n
        for k in kms:
            kms[k] += ms[k]
        c.timing_enable(0)
    kernel_avg_ms = {k: v / max(ncalls, 1) for k, v in kms.items() if v > 0}

    # ---- 3. per-call distribution: each call between its own two events
    ncall = max(args.steps, 100)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(ncall)]
    torch.cuda.synchronize()
    for i in range(ncall):
        evs[i][0].record()
        step(i)
        evs[i][1].record()
    torch.cuda.synchronize()
    per_call = sorted(a.elapsed_time(b) for a, b in evs)

    def pct(x):
        return per_call[min(len(per_call) - 1, int(round(x * (len(per_call) - 1))))]

    ms_per_step = 1e3 * elapsed / args.steps
    tokens_per_step = B * (w.n_tokens + w.n_text)
    value = tokens_per_step / (elapsed / args.steps)
    dom = max(kernel_avg_ms, key=kernel_avg_ms.get)
    dom_bytes = B * kb[dom]
    achieved = dom_bytes / (kernel_avg_ms[dom] * 1e-3) / 1e9

    traffic = None
    tfile = os.path.join(ROOT, "profiles", f"traffic_{w.name}.json")
    if os.path.exists(tfile):
        t = json.load(open(tfile))
        k = t.get("kernels", {}).get(dom)
        if k is not None and t.get("source_digest") == source_digest(t.get("sources", [])):
            traffic = k.get("bytes_per_launch")

    result = {
        "metric": METRIC,
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32" if w.storage == "f32" else "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_tokens": w.n_tokens, "n_text": w.n_text,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "rank": w.rank, "r_lo": w.r_lo, "top_k": w.top_k, "storage": w.storage,
                   "cache_copies_rotated": R, "distinct_sequences": S, "select": args.select,
                   **({"ema_alpha": args.ema_alpha} if ema else {}),
                   **({"text_rank": Rt, "text_r_lo": tr_lo, "text_top_k": tk_top} if Rt else {})},
        "ms_per_step_hip_events": event_ms,
        "per_call_ms": {"calls": ncall, "median": pct(0.5), "p10": pct(0.1), "p90": pct(0.9),
                        "min": per_call[0], "max": per_call[-1]},
        "hbm": {"algorithmic_bytes_per_step": step_bytes,
                "GB/s": step_bytes / (elapsed / args.steps) / 1e9,
                "frac_of_peak": step_bytes / (elapsed / args.steps) / 1e9 / HBM_PEAK_GBPS},
        "kernels_ms": kernel_avg_ms,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes},
    }

    for c in caches + [t for t in tcaches if t is not None]:
        c.free()
    del caches, qs, texts, tcaches

    # the device's streaming-read ceiling (a plain read kernel over 1 GiB, beyond the
    # 256 MB last-level cache), next to the datasheet peak: measured after the timed
    # steps, outside them
    rbuf = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    read_gbps = binding.read_bandwidth(rbuf, passes=10)
    del rbuf
    result["hbm"]["read_ceiling_GB/s"] = read_gbps
    result["hbm"]["frac_of_read_ceiling"] = result["hbm"]["GB/s"] / read_gbps
    result["roofline"]["frac_of_read_ceiling"] = achieved / read_gbps

    if not args.no_compress:
        result["compress"] = compress_leg(w, args.compress_reps, binding, wl, np, torch)
    if not args.no_e2e:
        result["e2e"] = e2e_leg(binding, wl, np, torch)

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, seqs, args.cpu_seconds)
    print(json.dumps(result))


def compress_leg(w, reps, binding, wl, np, torch):
    """ap_recompress of the whole batch (2 distinct sequences tiled), HIP events on
    the launch stream; the first call (workspace pool warm-up) is not timed."""
    dt = torch.float32 if w.storage == "f32" else torch.bfloat16
    S = min(w.batch, 2)
    idx = torch.tensor([b % S for b in range(w.batch)], device="cuda")
    k = torch.from_numpy(np.stack([wl.gen_kv(w, b, 0) for b in range(S)])).to(dt).cuda()[idx].contiguous()
    v = torch.from_numpy(np.stack([wl.gen_kv(w, b, 1) for b in range(S)])).to(dt).cuda()[idx].contiguous()
    c = binding.compress(k, v, batch=w.batch, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                         n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank,
                         storage="int4" if w.storage == "int4" else dt,
                         oversample=w.oversample, power_iters=w.power_iters, seed=1)
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ev0.record()
    for i in range(reps):
        c.recompress(k, v, seed=2 + i)
    ev1.record()
    torch.cuda.synchronize()
    ms = ev0.elapsed_time(ev1) / reps
    c.free()
    nbytes = compress_bytes(w)
    return {"ms": ms, "reps": reps, "matrices": 2 * w.batch, "ell": w.ell,
            "power_iters": w.power_iters, "algorithmic_bytes": nbytes,
            "GB/s": nbytes / (ms * 1e-3) / 1e9, "frac_of_hbm_peak": nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS}


def e2e_leg(binding, wl, np, torch):
    """The batch-256 layer end to end: the factorisation of its 256 K and 256 V matrices
    (4096 x 4096 bf16, p = 16, q = 2; two distinct sequences tiled over the batch) into
    an allocated cache (ap_recompress, the serving-slot form of ap_compress), then 16
    decode steps with fresh queries on the new factors, timed with HIP events on the
    launch stream.  A warm-up run of the same sequence comes first."""
    w = wl.WORKLOADS[5]
    S = 2
    idx = torch.tensor([b % S for b in range(w.batch)], device="cuda")
    k = torch.from_numpy(np.stack([wl.gen_kv(w, b, 0) for b in range(S)])).to(torch.bfloat16).cuda()[idx].contiguous()
    v = torch.from_numpy(np.stack([wl.gen_kv(w, b, 1) for b in range(S)])).to(torch.bfloat16).cuda()[idx].contiguous()
    qs = [torch.from_numpy(np.stack([wl.gen_q(w, b % S, step=t) for b in range(w.batch)])).cuda()
          for t in range(w.decode_steps)]
    out = torch.empty(w.batch, w.n_q_heads * w.head_dim, dtype=torch.float32, device="cuda")
    c = binding.compress(None, None, batch=w.batch, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                         n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank,
                         storage=torch.bfloat16, oversample=w.oversample, power_iters=w.power_iters)
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))

    def run(seed):
        e0.record()
        c.recompress(k, v, seed=seed)
        e1.record()
        for t in range(w.decode_steps):
            binding.decode(c, qs[t], r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, out=out)
        e2.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e2), e0.elapsed_time(e1)

    run(1)
    total, comp = run(2)
    c.free()
    s = 2
    cbytes = (2 * w.power_iters + 2) * 2 * w.batch * w.n_tokens * w.width * s
    dbytes = w.decode_steps * w.batch * kernel_bytes(w)["decode"]
    ideal = (cbytes + dbytes) / (HBM_PEAK_GBPS * 1e9) * 1e3
    return {"workload": w.name, "ms": total, "compress_ms": comp, "decode_ms": total - comp,
            "decode_steps": w.decode_steps, "matrices": 2 * w.batch, "ell": w.ell,
            "algorithmic_bytes": cbytes + dbytes, "ideal_ms_at_hbm_peak": ideal,
            "frac_of_hbm_peak": ideal / total}


def cpu_baseline(w, seqs, budget_s):
    """The oracle's decode step (explicit decompression + dense softmax, float64) on
    this host, on as many of the distinct sequences as fit the time budget."""
    from threadpoolctl import threadpool_info

    from oracle.decode import decode_ref
    from oracle.quant import quantize_dequant_u4
    if w.storage == "int4":   # the oracle attends over the values a 4-bit cache stores
        seqs = [dict(s, U_k=quantize_dequant_u4(s["U_k"]), U_v=quantize_dequant_u4(s["U_v"])) for s in seqs]
    threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    done, t0 = 0, time.perf_counter()
    while done == 0 or (time.perf_counter() - t0 < budget_s and done < 4096):
        s = seqs[done % len(seqs)]
        decode_ref(s["U_k"], s["B_k"], s["U_v"], s["B_v"], s["q"], w.n_kv_heads, w.head_dim,
                   w.r_lo, w.top_k, w.scale, s["text_k"] if w.n_text else None,
                   s["text_v"] if w.n_text else None)
        done += 1
    el = time.perf_counter() - t0
    return {"value": done * (w.n_tokens + w.n_text) / el, "unit": "tokens/s", "cores": threads,
            "kind": "oracle",
            "sample": f"{done} sequences of the {w.name} workload (one decode step each), "
                      f"{el:.1f} s on {os.cpu_count()} visible host CPUs"}


if __name__ == "__main__":
    main()
