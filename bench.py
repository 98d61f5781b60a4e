"""Benchmark of the CSA / HCA hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]

A step is one pass of the CSA prefill path over a 32768-token bf16 sequence
(64 query heads, one shared compressed KV entry of 512 + 64 dims, m = 4
overlapped compression, 16 x 64 lightning indexer, top-1024): compress the KV
entries and the indexer keys, score + select, sparse attention.  Inputs are
seeded synthetic tensors already resident in HBM.  Prints one JSON line.

The dominant kernel (sparse attention) is timed live with HIP events on the
stream it runs on; its algorithmic flop count (2 * pairs * heads * (576 +
512), pairs = sum over queries of min(k, visible entries)) over that time
gives the roofline fraction against the 2.5 PFLOP/s dense BF16 MFMA peak.
The CPU baseline times the fp64 oracle on a bounded row sample of the same
workload.
"""
import argparse
import json
import os
import sys
import time

import numpy as np
import torch

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

from compressed_sparse_amd import binding as cb  # noqa: E402
from compressed_sparse_amd import path, synth  # noqa: E402

PEAK_BF16_TFLOPS = 2500.0
PEAK_HBM_GBS = 8000.0


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def attention_pairs(w):
    n = (np.arange(w.tokens) + 1) // w.m
    return int(np.minimum(n, w.topk).sum())


def cpu_baseline(w, st, budget_s=15.0):
    """The fp64 oracle on this host: full compression of KV entries and
    indexer keys, then indexer + top-k + sparse attention for a seeded random
    sample of query rows until the time budget is spent; extrapolated to all
    rows."""
    from oracle import csa
    import threadpoolctl
    cpu = lambda x: x[0].to("cpu", torch.float64).numpy()
    t = {k: cpu(v) for k, v in st.tok.items()}
    p = {k: v.to("cpu", torch.float64).numpy() for k, v in st.prm.items()}
    t0 = time.perf_counter()
    ent = csa.compress(t["a"], t["za"], p["Ba"], w.m, t["b"], t["zb"], p["Bb"])
    cache = csa.finalize_kv(ent, 0, w.m, w.d_nope, w.rope_base, "bf16", "bf16")
    keys = csa.finalize_keys(csa.compress(t["ka"], t["kza"], p["kBa"], w.m, t["kb"], t["kzb"], p["kBb"]), "bf16")
    t_comp = time.perf_counter() - t0
    order = np.random.default_rng(0).permutation(w.tokens)
    rows_done, t_rows = 0, 0.0
    chunk = 64
    while t_rows < budget_s and rows_done < w.tokens:
        rows = np.sort(order[rows_done:rows_done + chunk])
        q = st.q[0, rows].to("cpu", torch.float64).numpy()
        qI = st.qI[0, rows].to("cpu", torch.float64).numpy()
        wt = st.wt[0, rows].to("cpu", torch.float64).numpy()
        t1 = time.perf_counter()
        csa.csa_rows(rows, rows, q, qI, wt, cache, keys, w.m, w.topk, w.d_nope, w.rope_base, w.tau)
        t_rows += time.perf_counter() - t1
        rows_done += len(rows)
    total = t_comp + t_rows / rows_done * w.tokens
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    return {"value": w.tokens / total, "unit": "tokens/s", "cores": int(threads), "kind": "oracle",
            "sample": f"full fp64 compression of {w.tokens} tokens ({t_comp:.1f} s) + {rows_done} random query rows "
                      f"of indexer/top-k/attention ({t_rows:.1f} s), extrapolated linearly to {w.tokens} rows"}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X; "
              "multi-GPU sharding is not built (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    w = synth.CSA_PREFILL_BF16_32K
    log(f"setup {w.name}")
    st = path.CsaPrefill(w)
    torch.cuda.synchronize()
    for i in range(args.warmup):
        st.step()
    torch.cuda.synchronize()
    log("warmup done")
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(args.steps)]
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for i in range(args.steps):
        st.step(evs[i])
    end.record()
    torch.cuda.synchronize()
    ms = start.elapsed_time(end) / args.steps
    attn_ms = float(np.mean([a.elapsed_time(b) for a, b in evs]))
    log(f"timed {args.steps} steps: {ms:.3f} ms/step, attention {attn_ms:.3f} ms")
    flops = 2.0 * attention_pairs(w) * w.heads * (w.c + w.d_nope)
    achieved = flops / (attn_ms * 1e-3) / 1e12
    out = {
        "metric": "CSA prefill tokens/s (L=32768, bf16, top-1024, 64 heads)",
        "value": w.tokens / (ms * 1e-3),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) projections, queries and indexer inputs; B ~ N(0, 1/sqrt(d)))",
        "config": {"workload": w.name, "batch": 1, "seq_len": w.tokens, "heads": w.heads,
                   "kv_dims": [w.d_nope, w.d_rope], "m": w.m, "topk": w.topk,
                   "indexer": [w.idx_heads, w.idx_dim]},
        "roofline": {"bound": "mfma", "kernel": "attn_mfma_kernel (sparse attention prefill)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": None,
                     "algorithmic_flop_per_launch": flops, "avg_launch_ms": attn_ms},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, st, args.cpu_budget)
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
