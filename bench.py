"""Throughput of one compressed-KV decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

Workload: the LLaVA-7B-like layer (batch 32, 32 heads of 128, 2880 visual tokens
factored at rank 64 with 64 dense text tokens, r_lo = 16, 25% of tokens at full
rank, bf16 factors).  One step = one ap_decode_attn call over the batch (latent
query, low-rank scores, per-head top-k, mixed-rank flash-decode, combine).  The
factored caches are built on the device before timing; R copies are rotated so
the 256 MB MALL cannot hold the working set.

Prints one JSON line: tokens attended/s for the whole GPU, the per-kernel HIP-event
breakdown, the dominant kernel's roofline, and the CPU oracle timed on a bounded
sample on this host.
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


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--cfg", type=int, default=2, help="workload id (2 = the batch-32 LLaVA layer)")
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    return ap.parse_args()


def kernel_bytes(w):
    """Algorithmic bytes per sequence read/written by each kernel of one step."""
    s = 2 if w.storage == "bf16" else 4
    W, r, N, T = w.width, w.rank, w.n_tokens, w.n_text
    qb = 4 * w.n_q_heads * w.head_dim
    return {
        "select": s * r * W + qb,                 # B_k, q   (U_k's low panels are re-read, not counted)
        "attn": s * 2 * N * r,                    # U_k, U_v
        "combine": s * r * W + s * 2 * T * W + qb,  # B_v, text K/V, out
    }


def source_digest(paths):
    h = hashlib.sha256()
    for p in paths:
        h.update(open(os.path.join(ROOT, p), "rb").read())
    return h.hexdigest()[:16]


def main():
    args = parse()
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)

    import numpy as np
    import torch

    from rank_compressed_kv_ap_amd import binding
    from rank_compressed_kv_ap_amd import workloads as wl

    w = wl.WORKLOADS[args.cfg]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    dt = torch.bfloat16 if w.storage == "bf16" else torch.float32
    B = w.batch

    # ---- inputs: S distinct seeded sequences tiled over the batch
    S = min(B, 4)
    seqs = [wl.gen_decode_inputs(w, b) for b in range(S)]

    def stack(key, dtype):
        return torch.from_numpy(np.stack([seqs[b % S][key] for b in range(B)])).to(dtype).to(dev)

    kb = kernel_bytes(w)
    step_bytes = B * sum(kb.values())
    R = max(1, math.ceil(2 * MALL_BYTES / step_bytes))
    caches, qs, texts = [], [], []
    for _ in range(R):
        c = binding.compress(None, None, batch=B, n_tokens=w.n_tokens, n_kv_heads=w.n_kv_heads,
                             n_q_heads=w.n_q_heads, head_dim=w.head_dim, rank=w.rank, storage=dt)
        c.set_factors(stack("U_k", dt), stack("B_k", dt), stack("U_v", dt), stack("B_v", dt))
        caches.append(c)
        qs.append(stack("q", torch.float32))
        texts.append((stack("text_k", dt), stack("text_v", dt)) if w.n_text else (None, None))
    out = torch.empty(B, w.n_q_heads * w.head_dim, dtype=torch.float32, device=dev)
    torch.cuda.synchronize()

    def step(i):
        j = i % R
        tk, tv = texts[j]
        binding.decode(caches[j], qs[j], r_lo=w.r_lo, top_k=w.top_k, scale=w.scale, text_k=tk,
                       text_v=tv, out=out, splits=args.splits)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps, HIP events around every kernel on the launch stream
    for c in caches:
        c.timing_enable(math.ceil(args.steps / R) + 1)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kms = {k: 0.0 for k in binding.KERNEL_NAMES}
    ncalls = 0
    for c in caches:
        ms, n = c.timing_read()
        ncalls += n
        for k in kms:
            kms[k] += ms[k]
    kernel_avg_ms = {k: v / max(ncalls, 1) for k, v in kms.items()}

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
        if t.get("kernel") == dom and t.get("source_digest") == source_digest(t.get("sources", [])):
            traffic = t.get("bytes_per_launch")

    result = {
        "metric": "compressed-KV decode attention: tokens attended/s + HBM GB/s (% of peak), batch 32",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16" if w.storage == "bf16" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "batch": B, "n_tokens": w.n_tokens, "n_text": w.n_text,
                   "n_q_heads": w.n_q_heads, "n_kv_heads": w.n_kv_heads, "head_dim": w.head_dim,
                   "rank": w.rank, "r_lo": w.r_lo, "top_k": w.top_k, "storage": w.storage,
                   "cache_copies_rotated": R, "distinct_sequences": S},
        "hbm": {"algorithmic_bytes_per_step": step_bytes,
                "GB/s": step_bytes / (elapsed / args.steps) / 1e9,
                "frac_of_peak": step_bytes / (elapsed / args.steps) / 1e9 / HBM_PEAK_GBPS},
        "kernels_ms": kernel_avg_ms,
        "roofline": {"bound": "hbm", "kernel": dom, "achieved": achieved, "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": achieved / HBM_PEAK_GBPS, "traffic": traffic,
                     "algorithmic_bytes_per_launch": dom_bytes},
    }

    for c in caches:
        c.free()

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, seqs, args.cpu_seconds)
    print(json.dumps(result))


def cpu_baseline(w, seqs, budget_s):
    """The oracle's decode step (explicit decompression + dense softmax, float64) on
    this host, on as many of the distinct sequences as fit the time budget."""
    import os as _os
    from threadpoolctl import threadpool_info

    from oracle.decode import decode_ref
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
                      f"{el:.1f} s on {_os.cpu_count()} visible host CPUs"}


if __name__ == "__main__":
    main()
