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

The decode workloads (CSA decode at batch 32 / 131072 context, HCA decode at
batch 16 / 2^20 context, the CSA + HCA pair at batch 4 / 2^20 context) are
reported under "secondary": consecutive decode steps captured in one HIP
graph, timed over replays, with their algorithmic HBM bytes per step against
the 8 TB/s HBM peak.  So is HCA prefill at 2^20 context: its last (hardest)
8192-token chunk, compressor + dense attention over all 8192 entries, with
the attention's algorithmic flops against the BF16 MFMA peak.
"""
import argparse
import dataclasses
import hashlib
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


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_bf16_csa_prefill_L32768_traffic.txt")
ATTN_SRC = os.path.join(ROOT, "compressed_sparse_amd", "csrc", "attention_bf16.hip")


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter
    summary, or None when the kernel source has changed since it was taken."""
    if not os.path.exists(TRAFFIC_FILE):
        return None
    kv = dict(line.split(":", 1) for line in open(TRAFFIC_FILE).read().splitlines() if ":" in line)
    src = hashlib.sha256(open(ATTN_SRC, "rb").read()).hexdigest()
    if kv.get("source_sha256", "").strip() != src:
        return None
    return float(kv["fetch_bytes_per_launch"]) + float(kv["write_bytes_per_launch"])


def copy_calibration():
    """A plain device copy of 1 GiB (read 1 GiB, write 1 GiB) whose FETCH_SIZE
    / WRITE_SIZE readings calibrate the counters."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


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


def decode_bytes_csa(w, n, B):
    """Algorithmic HBM bytes of one CSA decode step: every visible indexer key
    once, the k selected split entries, q / qI / w in, o / lse out, the
    index list written and read, one token into each compressor."""
    key_b = {"fp8": w.idx_dim + 4, "mxfp4": w.idx_dim // 2 + w.idx_dim // 32, "bf16": 2 * w.idx_dim}[w.key_fmt]
    ent_b = w.d_nope * (1 if w.nope_fmt == "fp8" else 2) + (4 if w.nope_fmt == "fp8" else 0) + 2 * w.d_rope
    tok_b = 2 * (4 * w.c + 4 * w.idx_dim)
    return B * (n * key_b + w.topk * ent_b + 2 * w.heads * w.c + 2 * w.idx_heads * w.idx_dim + 4 * w.idx_heads
                + 2 * w.heads * w.d_nope + 4 * w.heads + 8 * w.topk + tok_b)


def decode_bytes_hca(w, n, B):
    ent_b = w.d_nope * (1 if w.nope_fmt == "fp8" else 2) + (4 if w.nope_fmt == "fp8" else 0) + 2 * w.d_rope
    return B * (n * ent_b + 2 * w.heads * w.c + 2 * w.heads * w.d_nope + 4 * w.heads + 2 * 2 * w.c)


def time_graph(step_fn, n_steps, replays=20, warmup=3):
    """Captures n_steps consecutive decode steps in one HIP graph; returns
    the average ms per step over `replays` replays."""
    g = torch.cuda.CUDAGraph()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        for i in range(n_steps):  # eager run also fills caches for the positions
            step_fn(i)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        for i in range(n_steps):
            step_fn(i)
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(replays):
        g.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (replays * n_steps)


def csa_decode_line(n_steps=8):
    w = synth.CSA_DECODE_B32_128K
    log(f"setup {w.name}")
    lay = path.CsaLayer(w, w.batch, w.tokens // w.m + n_steps)
    lay.prefill_context(w.tokens)
    o = lay.alloc_decode_outputs()
    xs = [lay.decode_inputs([w.tokens + i] * w.batch) for i in range(n_steps)]
    ms = time_graph(lambda i: lay.decode_step(xs[i], o), n_steps)
    by = decode_bytes_csa(w, w.tokens // w.m, w.batch)
    return {"workload": w.name, "metric": "decode us/step (whole batch)", "value": ms * 1e3, "unit": "us",
            "tokens_per_s": w.batch / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "algorithmic_bytes_per_step": by}}


def hca_decode_line(n_steps=8):
    w = synth.HCA_DECODE_B16_1M
    log(f"setup {w.name}")
    lay = path.HcaLayer(w, w.batch, w.tokens // w.m + n_steps)
    lay.prefill_context(w.tokens)
    o = lay.alloc_decode_outputs()
    xs = [lay.decode_inputs([w.tokens + i] * w.batch) for i in range(n_steps)]
    ms = time_graph(lambda i: lay.decode_step(xs[i], o), n_steps)
    by = decode_bytes_hca(w, w.tokens // w.m, w.batch)
    return {"workload": w.name, "metric": "decode us/step (whole batch)", "value": ms * 1e3, "unit": "us",
            "tokens_per_s": w.batch / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "algorithmic_bytes_per_step": by}}


def pair_decode_lines(n_steps=8):
    wc, wh = synth.PAIR_CSA_DECODE_B4_1M, synth.PAIR_HCA_DECODE_B4_1M
    log(f"setup {wc.name} + {wh.name}")
    lc = path.CsaLayer(wc, wc.batch, wc.tokens // wc.m + n_steps)
    lh = path.HcaLayer(wh, wh.batch, wh.tokens // wh.m + n_steps, seed=1)
    lc.prefill_context(wc.tokens)
    lh.prefill_context(wh.tokens)
    oc, oh = lc.alloc_decode_outputs(), lh.alloc_decode_outputs()
    xc = [lc.decode_inputs([wc.tokens + i] * wc.batch) for i in range(n_steps)]
    xh = [lh.decode_inputs([wh.tokens + i] * wh.batch) for i in range(n_steps)]
    ms_c = time_graph(lambda i: lc.decode_step(xc[i], oc), n_steps)

    def pair(i):
        lc.decode_step(xc[i], oc)
        lh.decode_step(xh[i], oh)
    ms = time_graph(pair, n_steps)
    by_c = decode_bytes_csa(wc, wc.tokens // wc.m, wc.batch)
    by = by_c + decode_bytes_hca(wh, wh.tokens // wh.m, wh.batch)
    return [{"workload": wc.name, "metric": "CSA layer decode us/step (whole batch)", "value": ms_c * 1e3,
             "unit": "us", "roofline": {"bound": "hbm", "achieved": by_c / (ms_c * 1e-3) / 1e9,
                                        "peak": PEAK_HBM_GBS, "unit": "GB/s",
                                        "frac": by_c / (ms_c * 1e-3) / 1e9 / PEAK_HBM_GBS,
                                        "algorithmic_bytes_per_step": by_c}},
            {"workload": wc.name + " + " + wh.name, "metric": "CSA+HCA layer pair decode us/step",
             "value": ms * 1e3, "unit": "us",
             "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                          "unit": "GB/s", "frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                          "algorithmic_bytes_per_step": by}}]


def secondary_lines():
    out = [csa_decode_line()]
    torch.cuda.empty_cache()
    out.append(hca_decode_line())
    torch.cuda.empty_cache()
    out.extend(pair_decode_lines())
    torch.cuda.empty_cache()
    out.append(secondary_hca_prefill())
    torch.cuda.empty_cache()
    out.append(secondary_mxfp4_prefill_indexer())
    return out

def secondary_hca_prefill(steps=5):
    """The last 8192-token chunk of a 2^20-token HCA prefill: compress the
    chunk's tokens and run dense attention for its 8192 queries over the
    8192 entries of the whole context (inputs resident in HBM)."""
    w = synth.HCA_PREFILL_1M
    chunk = w.chunk
    c = w.tokens // chunk - 1
    log(f"setup {w.name}")
    lay = path.HcaLayer(w, 1, w.tokens // w.m)
    lay.prefill_context(w.tokens)
    tok = synth.token_chunk(w, 0, c, chunk, 0, "cuda")
    x = {k: v[None].contiguous() for k, v in tok.items()}
    q = synth.query_chunk(w, 0, c, chunk, 0, "cuda", with_index=False)["q"][None].contiguous()
    o = torch.empty((1, chunk, w.heads, w.d_nope), dtype=synth.TORCH_DTYPE[w.out_dtype], device="cuda")
    pos0 = c * chunk

    def step(ev=None):
        cb.compress_prefill(lay.kv, pos0, x["a"], x["za"], lay.prm["Ba"])
        if ev is not None:
            ev[0].record()
        cb.dense_attn_prefill(lay.adesc, lay.kv, pos0, q, w.tau, o)
        if ev is not None:
            ev[1].record()
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for i in range(steps):
        step(evs[i])
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    attn_ms = float(np.mean([e0.elapsed_time(e1) for e0, e1 in evs]))
    pairs = int(np.minimum((np.arange(pos0, pos0 + chunk) + 1) // w.m, w.tokens // w.m).sum())
    flops = 2.0 * pairs * w.heads * (w.c + w.d_nope)
    ach = flops / (attn_ms * 1e-3) / 1e12
    return {"workload": w.name + " (last chunk)", "metric": "HCA prefill tokens/s (chunk of 8192 at 2^20 context)",
            "value": chunk / (ms * 1e-3), "unit": "tokens/s", "ms_per_chunk": ms,
            "roofline": {"bound": "mfma", "kernel": "dense attention prefill", "achieved": ach,
                         "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                         "algorithmic_flop_per_launch": flops, "avg_launch_ms": attn_ms}}


def secondary_mxfp4_prefill_indexer(steps=5):
    """Lightning indexer + top-k of the 32768-token prefill with MXFP4 keys
    and query and BF16 scores (the 2^20-context pair's precision): the
    scaled-MFMA scan over every query row writes the score rows, the per-row
    select reads them back.  Keys from the MXFP4 compressor, inputs resident."""
    w = dataclasses.replace(synth.CSA_PREFILL_BF16_32K, name="csa_prefill_L32768_mxfp4_indexer",
                            key_fmt="mxfp4", qk_fmt="mxfp4", score_fmt="bf16")
    log(f"setup {w.name}")
    st = path.CsaPrefill(w)
    st.step()

    def run():
        cb.index_topk_prefill(st.idesc, st.keys, 0, st.qI, st.wt, w.topk, st.idx, ws=st.iws)
    for _ in range(2):
        run()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(steps):
        run()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / steps
    visible = int(((np.arange(w.tokens) + 1) // w.m).sum())
    by = 2.0 * visible * 4  # score rows written by the scan and read by the select
    return {"workload": w.name, "metric": "MXFP4 prefill indexer + top-k tokens/s (L=32768, k=1024)",
            "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_launch": ms,
            "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS, "unit": "GB/s",
                         "frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS, "algorithmic_bytes_per_launch": by}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--no-secondary", action="store_true", help="skip the decode workloads")
    ap.add_argument("--copy-calib", action="store_true", help="run a 1 GiB copy first (counter calibration)")
    ap.add_argument("--only", choices=["csa-decode", "hca-decode", "pair-decode", "hca-prefill", "mxfp4-indexer"],
                    help="run just this secondary workload and print its line(s) (for profiling)")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py measures one GPU only: the path runs on a single MI355X; "
              "multi-GPU sharding is not built (run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calib:
        copy_calibration()
    if args.only:
        fn = {"csa-decode": csa_decode_line, "hca-decode": hca_decode_line, "pair-decode": pair_decode_lines,
              "hca-prefill": secondary_hca_prefill, "mxfp4-indexer": secondary_mxfp4_prefill_indexer}[args.only]
        print(json.dumps(fn()), flush=True)
        return
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
        "roofline": {"bound": "mfma", "kernel": "attn_bf16_kernel (sparse attention prefill)",
                     "achieved": achieved, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": achieved / PEAK_BF16_TFLOPS, "traffic": measured_traffic(),
                     "algorithmic_flop_per_launch": flops, "avg_launch_ms": attn_ms},
    }
    if not args.no_cpu_baseline:
        log("cpu baseline (oracle)")
        out["cpu_baseline"] = cpu_baseline(w, st, args.cpu_budget)
    if not args.no_secondary:
        del st
        torch.cuda.empty_cache()
        out["secondary"] = secondary_lines()
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
