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
PEAK_FP8_TFLOPS = 5000.0
PEAK_FP4_TFLOPS = 10100.0
PEAK_HBM_GBS = 8000.0
CPU_BASELINE = True     # the oracle timings (cleared by --no-cpu-baseline)
REPLAYS = 12            # timed replays of each decode graph (--replays)
DECODE_EAGER = 0        # > 0: that many eager decode steps instead of graphs (--decode-eager, counter runs)


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def context_progress(done, total):
    log(f"  context chunks {done}/{total}")


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
    return {"value": w.tokens / total, "unit": "tokens/s", "cores": int(threads), "cpu": host_cpu()[0],
            "kind": "oracle",
            "sample": f"full fp64 compression of {w.tokens} tokens ({t_comp:.1f} s) + {rows_done} random query rows "
                      f"of indexer/top-k/attention ({t_rows:.1f} s), extrapolated linearly to {w.tokens} rows"}


def host_cpu():
    """The host's CPU model and the threads the oracle's BLAS uses."""
    import platform
    import threadpoolctl
    model = platform.processor() or ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    threads = max([i.get("num_threads", 1) for i in threadpoolctl.threadpool_info()] + [1])
    return model, int(threads), os.cpu_count()


def oracle_entries(w, seq, T, prefix="", seed=0, overlap=True):
    """Exact (fp64) entries of tokens [0, T) of sequence `seq`, computed by
    the oracle's compressor chunk by chunk (the previous chunk's last m rows
    carry the C^b side).  CPU-baseline setup: the cache a decode step reads."""
    from oracle import csa
    m, chunk = w.m, w.chunk
    names = [prefix + n for n in (("a", "za", "b", "zb") if overlap else ("a", "za"))]
    prm = {k: v.to("cpu", torch.float64).numpy() for k, v in synth.compressor_params(w, seed, "cuda").items()}
    outs, tail = [], None
    for c in range((T + chunk - 1) // chunk):
        n = min(chunk, T - c * chunk)
        x = synth.token_chunk(w, seq, c, chunk, seed, "cuda", names=names)
        x = {k: v[:n].to("cpu", torch.float64).numpy() for k, v in x.items()}
        tok0 = c * chunk
        if overlap and tail is not None:
            x = {k: np.concatenate([tail[k], x[k]], 0) for k in x}
            tok0 -= m
        i0, i1 = (c * chunk + m) // m - 1, (c * chunk + n) // m
        if i1 > i0:
            extra = (x[names[2]], x[names[3]], prm[prefix + "Bb"]) if overlap else ()
            outs.append(csa.compress(x[names[0]], x[names[1]], prm[prefix + "Ba"], m, *extra, i0=i0, i1=i1, tok0=tok0))
        if overlap:
            tail = {k: v[-m:] for k, v in x.items()}
    return np.concatenate(outs, 0)


def cpu_baseline_csa_decode(w, lay, x, gpu_idx, seqs, recall=False):
    """The oracle's CSA decode step (indexer over every visible key, top-k,
    attention over the selected entries) timed for the sampled sequences of
    the batch and extrapolated to the whole batch; its caches are built by the
    oracle's own compressor (untimed setup).  With recall=True also the
    indexer recall against the fp32 indexer on the exact keys, for the
    oracle's own selection and for the GPU's."""
    from oracle import csa
    pos = int(x["pos"][0])
    n = (pos + 1) // w.m
    t_step, rec_o, rec_g = 0.0, [], []
    for b in seqs:
        sid = lay.seq_ids[b]
        kexact = oracle_entries(w, sid, n * w.m, prefix="k")[:n]
        keys = csa.finalize_keys(kexact, w.key_fmt)
        q, qI, wt = (x[k][b].to("cpu", torch.float64).numpy() for k in ("q", "qI", "w"))
        t0 = time.perf_counter()
        I = csa.index_scores(csa.quantize_query(qI, w.qk_fmt), wt, keys["k"], n, w.score_fmt)
        sel = csa.topk(I, n, w.topk)
        t1 = time.perf_counter()
        ids = sel[sel >= 0]
        ex = csa.rope(oracle_selected_entries(w, sid, ids), csa.entry_position(ids, w.m), w.d_nope, w.rope_base)
        K = np.zeros((n, w.c))
        K[ids] = np.concatenate([csa.store_format(ex[:, :w.d_nope], w.nope_fmt)[0],
                                 csa.store_format(ex[:, w.d_nope:], w.rope_fmt)[0]], 1)
        t2 = time.perf_counter()
        csa.sparse_attention_row(q, pos, {"k": K, "v": K[:, :w.d_nope]}, sel, w.d_nope, w.rope_base, w.tau)
        t3 = time.perf_counter()
        t_step += (t1 - t0) + (t3 - t2)
        if recall:
            full = set(csa.topk(csa.index_scores(qI, wt, kexact, n, "f32"), n, w.topk).tolist())
            rec_o.append(len(full & set(sel.tolist())) / w.topk)
            rec_g.append(len(full & set(gpu_idx[b].tolist())) / w.topk)
    model, threads, _ = host_cpu()
    us = t_step / len(seqs) * w.batch * 1e6
    out = {"value": us, "unit": "us/step", "cores": threads, "cpu": model, "kind": "oracle",
           "sample": f"decode step at position {pos} of {len(seqs)} of {w.batch} sequences (indexer over {n} keys, "
                     f"top-{w.topk}, attention), extrapolated to the batch; caches from the oracle's compressor"}
    if recall:
        out["indexer_recall"] = {"gpu_vs_fp32": float(np.mean(rec_g)), "oracle_vs_fp32": float(np.mean(rec_o)),
                                 "sequences": len(seqs), "target_pages_trained_model": 0.997}
    return out


def oracle_selected_entries(w, seq, ids, seed=0):
    """Exact pre-RoPE CSA entries `ids` of sequence `seq`, each from its own
    2m tokens (windows i-1 and i), by the oracle's compressor."""
    from oracle import csa
    m, chunk = w.m, w.chunk
    ids = np.asarray(ids, dtype=np.int64)
    rows = np.maximum((ids[:, None] - 1) * m + np.arange(2 * m)[None, :], 0).ravel()
    names = ("a", "za", "b", "zb")
    got = {nm: np.zeros((len(rows), w.c)) for nm in names}
    for c in np.unique(rows // chunk):
        sel = np.nonzero(rows // chunk == c)[0]
        xc = synth.token_chunk(w, seq, int(c), chunk, seed, "cuda", names=list(names))
        r = torch.as_tensor(rows[sel] % chunk, device="cuda")
        for nm in names:
            got[nm][sel] = xc[nm][r].to("cpu", torch.float64).numpy()
    prm = {k: v.to("cpu", torch.float64).numpy() for k, v in synth.compressor_params(w, seed, "cuda").items()}
    out = np.zeros((len(ids), w.c))
    for j, i in enumerate(ids):
        sl = slice(j * 2 * m, (j + 1) * 2 * m)
        out[j] = csa.compress(got["a"][sl], got["za"][sl], prm["Ba"], m, got["b"][sl], got["zb"][sl], prm["Bb"],
                              i0=int(i), i1=int(i) + 1, tok0=(int(i) - 1) * m)[0]
    return out


def cpu_baseline_hca_decode(w, lay, x, seqs, seed=0):
    """The oracle's HCA decode step (dense attention over every visible
    entry) timed for the sampled sequences, extrapolated to the batch."""
    from oracle import csa
    pos = int(x["pos"][0])
    n = (pos + 1) // w.m
    t = 0.0
    for b in seqs:
        cache = csa.finalize_kv(oracle_entries(w, lay.seq_ids[b], n * w.m, seed=seed, overlap=False)[:n], 0, w.m,
                                w.d_nope, w.rope_base, w.nope_fmt, w.rope_fmt)
        q = x["q"][b].to("cpu", torch.float64).numpy()
        t0 = time.perf_counter()
        csa.dense_attention_row(q, pos, cache, w.m, w.d_nope, w.rope_base, w.tau)
        t += time.perf_counter() - t0
    model, threads, _ = host_cpu()
    return {"value": t / len(seqs) * w.batch * 1e6, "unit": "us/step", "cores": threads, "cpu": model,
            "kind": "oracle", "sample": f"dense attention of {len(seqs)} of {w.batch} sequences at position {pos} "
                                        f"over {n} entries, extrapolated to the batch; cache from the oracle's compressor"}


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


DECODE_STEPS = 128


def time_graph(layers, step_fn, n_steps=DECODE_STEPS, replays=None, warmup=2):
    """Captures n_steps consecutive decode steps in one HIP graph (each replay
    restores the layers' staging rings first, so every replay computes the
    same steps); returns (median, p10, p90) ms per step over the replays."""
    replays = replays or REPLAYS
    if DECODE_EAGER:  # counter collection: a few plain launches, no graph
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for i in range(DECODE_EAGER):
            step_fn(i % n_steps)
        e1.record()
        torch.cuda.synchronize()
        ms = e0.elapsed_time(e1) / DECODE_EAGER
        return ms, ms, ms
    dg = path.DecodeGraph(layers, step_fn, n_steps)
    for _ in range(warmup):
        dg.replay()
    torch.cuda.synchronize()
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(replays)]
    for a, b in evs:
        a.record()
        dg.replay()
        b.record()
    torch.cuda.synchronize()
    per = np.array([a.elapsed_time(b) / n_steps for a, b in evs])
    return float(np.median(per)), float(np.percentile(per, 10)), float(np.percentile(per, 90))


def decode_line(name, metric, ms3, by, B):
    ms, p10, p90 = ms3
    return {"workload": name, "metric": metric, "value": ms * 1e3, "unit": "us", "p10_us": p10 * 1e3,
            "p90_us": p90 * 1e3, "steps_per_graph": DECODE_STEPS, "tokens_per_s": B / (ms * 1e-3),
            "roofline": {"bound": "hbm", "achieved": by / (ms * 1e-3) / 1e9, "peak": PEAK_HBM_GBS,
                         "unit": "GB/s", "frac": by / (ms * 1e-3) / 1e9 / PEAK_HBM_GBS,
                         "algorithmic_bytes_per_step": by}}


def csa_decode_line(n_steps=DECODE_STEPS):
    w = synth.CSA_DECODE_B32_128K
    log(f"setup {w.name}")
    lay = path.CsaLayer(w, w.batch, w.tokens // w.m + n_steps)
    lay.prefill_context(w.tokens, progress=context_progress)
    o = lay.alloc_decode_outputs()
    xs = lay.decode_input_steps([[w.tokens + i] * w.batch for i in range(n_steps)])
    ms3 = time_graph([lay], lambda i: lay.decode_step(xs[i], o), n_steps)
    by = decode_bytes_csa(w, w.tokens // w.m, w.batch)
    line = decode_line(w.name, "decode us/step (whole batch)", ms3, by, w.batch)
    if CPU_BASELINE:
        log("cpu baseline (oracle) " + w.name)
        line["cpu_baseline"] = cpu_baseline_csa_decode(w, lay, xs[-1], o["idx"].cpu().numpy(), seqs=[0, 17])
    return line


def hca_decode_line(n_steps=DECODE_STEPS, qk="bf16"):
    """qk="fp8": the FP8 QK product (MXFP8 query against the FP8 codes)."""
    w = synth.HCA_DECODE_B16_1M
    log(f"setup {w.name}")
    lay = path.HcaLayer(w, w.batch, w.tokens // w.m + n_steps, qk=qk)
    lay.prefill_context(w.tokens, progress=context_progress)
    o = lay.alloc_decode_outputs()
    xs = lay.decode_input_steps([[w.tokens + i] * w.batch for i in range(n_steps)])
    ms3 = time_graph([lay], lambda i: lay.decode_step(xs[i], o), n_steps)
    by = decode_bytes_hca(w, w.tokens // w.m, w.batch)
    line = decode_line(w.name + (", FP8 QK" if qk == "fp8" else ""), "decode us/step (whole batch)", ms3, by,
                       w.batch)
    if qk == "fp8":
        return line
    if CPU_BASELINE:
        log("cpu baseline (oracle) " + w.name)
        line["cpu_baseline"] = cpu_baseline_hca_decode(w, lay, xs[-1], seqs=[9])
    return line


def pair_decode_lines(n_steps=DECODE_STEPS):
    wc, wh = synth.PAIR_CSA_DECODE_B4_1M, synth.PAIR_HCA_DECODE_B4_1M
    log(f"setup {wc.name} + {wh.name}")
    lc = path.CsaLayer(wc, wc.batch, wc.tokens // wc.m + n_steps)
    lh = path.HcaLayer(wh, wh.batch, wh.tokens // wh.m + n_steps, seed=1)
    lc.prefill_context(wc.tokens, progress=context_progress)
    lh.prefill_context(wh.tokens, progress=context_progress)
    oc, oh = lc.alloc_decode_outputs(), lh.alloc_decode_outputs()
    xc = lc.decode_input_steps([[wc.tokens + i] * wc.batch for i in range(n_steps)])
    xh = lh.decode_input_steps([[wh.tokens + i] * wh.batch for i in range(n_steps)])
    ms_c = time_graph([lc], lambda i: lc.decode_step(xc[i], oc), n_steps)

    def pair(i):
        lc.decode_step(xc[i], oc)
        lh.decode_step(xh[i], oh)
    ms = time_graph([lc, lh], pair, n_steps)
    by_c = decode_bytes_csa(wc, wc.tokens // wc.m, wc.batch)
    by = by_c + decode_bytes_hca(wh, wh.tokens // wh.m, wh.batch)
    lines = [decode_line(wc.name, "CSA layer decode us/step (whole batch)", ms_c, by_c, wc.batch),
             decode_line(wc.name + " + " + wh.name, "CSA+HCA layer pair decode us/step", ms, by, wc.batch)]
    if CPU_BASELINE:
        # the oracle on every sequence of the CSA layer: its time, and the
        # indexer recall (GPU and oracle MXFP4 / BF16-score selections against
        # the fp32 indexer on the exact keys) at the last timed step
        log("cpu baseline (oracle) + indexer recall " + wc.name)
        lines[0]["cpu_baseline"] = cpu_baseline_csa_decode(wc, lc, xc[-1], oc["idx"].cpu().numpy(),
                                                           seqs=range(wc.batch), recall=True)
        lines[0]["indexer_recall"] = lines[0]["cpu_baseline"].pop("indexer_recall")
    return lines


def swa_decode_lines(n_steps=DECODE_STEPS, window=128):
    """The 2^20-context CSA layer of the pair (B = 4, MXFP4 indexer) with its
    sliding-window branch over the last 128 tokens: per step the CSA decode,
    then the new token into the per-token cache, window attention and the
    log-sum-exp merge into the layer's output."""
    w = synth.PAIR_CSA_DECODE_B4_1M
    log(f"setup {w.name} + sliding window {window}")
    lc = path.CsaLayer(w, w.batch, w.tokens // w.m + n_steps)
    sw = path.SwaBranch(w, w.batch, w.tokens + n_steps, window)
    lc.prefill_context(w.tokens, progress=context_progress)
    sw.prefill_context(w.tokens, progress=context_progress)
    oc, osw = lc.alloc_decode_outputs(), sw.alloc_decode_outputs()
    xs = lc.decode_input_steps([[w.tokens + i] * w.batch for i in range(n_steps)])

    def step(i):
        lc.decode_step(xs[i], oc)
        sw.decode_step(xs[i], osw, oc)
    ms3 = time_graph([lc, sw], step, n_steps)
    ent_b = w.d_nope + 4 + 2 * w.d_rope
    by = decode_bytes_csa(w, w.tokens // w.m, w.batch) + w.batch * (window * ent_b + 2 * 2 * w.c + 2 * 2 * w.heads *
                                                                     w.d_nope)
    return decode_line(w.name + f" + sliding window {window}", "CSA layer + sliding-window branch decode us/step",
                       ms3, by, w.batch)


def paged_decode_lines(n_steps=DECODE_STEPS, page=64, layouts=("paged", "contiguous")):
    """Paged, variable-length CSA decode: 32 sequences with context lengths
    log-uniform over 8K..256K tokens, KV and indexer-key caches in 64-entry
    pages of one pool handed out in a seeded random order; the same batch in
    contiguous per-sequence caches (capacity of the longest) beside it."""
    w = synth.PAGED_CSA_DECODE_B32_MIXED
    lengths = synth.mixed_lengths(w.batch, 13, 18)
    need = [(L + n_steps) // w.m + 1 for L in lengths]
    cap = -(-max(need) // page) * page
    table, pool = path.block_tables(need, page, cap)
    by = sum(decode_bytes_csa(w, L // w.m, 1) for L in lengths)
    lines = []
    for paged in [lt == "paged" for lt in layouts]:
        log(f"setup {w.name} ({'paged' if paged else 'contiguous'})")
        kw = dict(page_size=page, block_table=table, pool_pages=pool) if paged else {}
        lay = path.CsaLayer(w, w.batch, cap, **kw)
        lay.prefill_contexts(lengths)
        o = lay.alloc_decode_outputs()
        xs = lay.decode_input_steps([[L + i for L in lengths] for i in range(n_steps)])
        ms3 = time_graph([lay], lambda i: lay.decode_step(xs[i], o), n_steps)
        name = w.name if paged else w.name.replace("paged", "contiguous").replace("_page64", "")
        line = decode_line(name, "decode us/step (whole batch, mixed contexts)", ms3, by, w.batch)
        line["contexts"] = {"min": min(lengths), "max": max(lengths), "mean": float(np.mean(lengths))}
        if paged:
            line["pages"] = {"entries_per_page": page, "pool_pages": pool, "capacity_per_seq": cap}
        lines.append(line)
        del lay, o, xs
        torch.cuda.empty_cache()
    return lines


def secondary_project_prefill(steps=5):
    """The 32K prefill's two compressors fed from hidden states (d_model =
    4096): projections fused with the compression (csa_compress_project_prefill)
    for the KV entries (4 x 576 projected columns) and the indexer keys (4 x 64).
    Priced as the GEMM it is: 2 * T * d_model * 2560 flop per step."""
    w, d = synth.PROJECT_PREFILL_32K, synth.PROJECT_D_MODEL
    T, m = w.tokens, w.m
    log(f"setup {w.name}")
    X = synth.hidden_chunk(0, 0, T, d, 0, "cuda")[None].contiguous()
    Wkv = cb.pack_projection_weights(synth.projection_weights(w.c, d, True, "", 0, "cuda"))
    Wk = cb.pack_projection_weights(synth.projection_weights(w.idx_dim, d, True, "k", 0, "cuda"))
    prm = synth.compressor_params(w, 0, "cuda")
    kv = cb.KVCache(cb.cache_desc(m, True, w.d_nope, w.d_rope, "bf16", w.nope_fmt, w.rope_fmt, T // m), 1)
    keys = cb.KVCache(cb.cache_desc(m, True, w.idx_dim, 0, "bf16", w.key_fmt, "f32", T // m), 1)
    ws = cb.workspace(max(cb.project_workspace_bytes(kv.desc, 1, T), cb.project_workspace_bytes(keys.desc, 1, T)))

    def step():
        cb.compress_project_prefill(kv, 0, X, Wkv, prm["Ba"], prm["Bb"], ws=ws)
        cb.compress_project_prefill(keys, 0, X, Wk, prm["kBa"], prm["kBb"], ws=ws)
    for _ in range(2):
        step()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        step()
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    flops = 2.0 * T * d * 4 * (w.c + w.idx_dim)
    ach = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "metric": "compressor prefill from hidden states tokens/s (L=32768, d_model=4096)",
            "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms,
            "roofline": {"bound": "mfma", "kernel": "project_gemm_kernel (projection GEMM + compressor epilogue)",
                         "achieved": ach, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s", "frac": ach / PEAK_BF16_TFLOPS,
                         "algorithmic_flop_per_step": flops}}


def planted_recall_line(rhos=(0.5, 0.6, 0.7, 0.8)):
    """planted_recall at several separations rho (the value reported is the
    recall at rho = 0.6, where the planted and the other keys still overlap
    near the k-th score)."""
    by = {rho: planted_recall(rho) for rho in rhos}
    main = by[0.6] if 0.6 in by else by[rhos[0]]
    out = dict(main)
    out["by_rho"] = {str(r): {"gpu": v["value"], "oracle_mxfp4": v["oracle_mxfp4_recall"],
                              "planted_share_of_fp32_top": v["planted_share_of_fp32_top"]} for r, v in by.items()}
    return out


def planted_recall(rho):
    """MXFP4 indexer recall on the labelled "planted" variant of the pair's
    CSA layer (B = 4 at 2^20 context: 262144 keys, 1024 of them planted along
    the query direction; synth.planted_index_inputs).  The keys reach the
    MXFP4 key cache through the library's own compressor (one-token windows
    with zero logits store each row as it is); the decode indexer (MXFP4 QK,
    BF16 scores) selects 1024; recall = overlap with the fp32 top-1024 on the
    exact keys, for the GPU and for the oracle's MXFP4 path."""
    from oracle import csa
    w = synth.PAIR_CSA_DECODE_B4_1M
    n, d, H, k, B = w.tokens // w.m, w.idx_dim, w.idx_heads, w.topk, w.batch
    log(f"setup planted recall ({B} x {n} keys, rho {rho})")
    desc = cb.cache_desc(1, False, d, 0, "f32", "mxfp4", "f32", n)
    keys = cb.KVCache(desc, B)
    zero = torch.zeros((1, d), dtype=torch.float32, device="cuda")
    inp = [synth.planted_index_inputs(n, d, H, k, rho, b) for b in range(B)]
    for b, (kk, _, _, _) in enumerate(inp):
        x = kk[None].cuda().contiguous()
        cb.compress_prefill(keys.seq_view(b), 0, x, torch.zeros_like(x), zero)
    idesc = cb.index_desc(H, d, "bf16", "mxfp4", "mxfp4", "bf16", w.m, n)
    qI = torch.stack([q for _, q, _, _ in inp]).to(torch.bfloat16).cuda().contiguous()
    wt = torch.stack([ww for _, _, ww, _ in inp]).cuda().contiguous()
    pos = torch.full((B,), w.tokens, dtype=torch.int64, device="cuda")
    idx = torch.empty((B, k), dtype=torch.int32, device="cuda")
    cb.index_topk_decode(idesc, keys, pos, qI, wt, k, idx)
    torch.cuda.synchronize()
    gidx = idx.cpu().numpy()
    rec_g, rec_o, planted_in = [], [], []
    for b, (kk, q, ww, pl) in enumerate(inp):
        kx = kk.double().numpy()
        qb = qI[b].float().cpu().double().numpy()
        full = set(csa.topk(csa.index_scores(qb, ww.double().numpy(), kx, n, "f32"), n, k).tolist())
        Kq = csa.finalize_keys(kx, "mxfp4")["k"]
        sel = csa.topk(csa.index_scores(csa.quantize_query(qb, "mxfp4"), ww.double().numpy(), Kq, n, "bf16"), n, k)
        rec_g.append(len(full & set(gidx[b].tolist())) / k)
        rec_o.append(len(full & set(sel.tolist())) / k)
        planted_in.append(len(full & set(pl.tolist())) / k)
    return {"workload": w.name + " (planted keys, labelled variant)",
            "metric": "MXFP4 indexer recall vs fp32 top-1024 (planted keys)",
            "value": float(np.mean(rec_g)), "unit": "fraction",
            "oracle_mxfp4_recall": float(np.mean(rec_o)), "planted_share_of_fp32_top": float(np.mean(planted_in)),
            "rho": rho, "sequences": B, "pages_value": 0.997}


def secondary_lines():
    out = []
    for fn in (csa_decode_line, hca_decode_line, pair_decode_lines, swa_decode_lines, paged_decode_lines,
               planted_recall_line, secondary_project_prefill, secondary_hca_prefill,
               lambda: secondary_hca_prefill(qk="fp8"),
               secondary_hca_prefill_whole, secondary_mxfp4_prefill_indexer, secondary_tiny):
        r = fn()
        out.extend(r if isinstance(r, list) else [r])
        torch.cuda.empty_cache()
    return out


def measured_peaks():
    """Microbenchmarks beside the datasheet peaks: a 4 GiB device copy (HBM
    read + write bytes over its time) and a 8192^3 BF16 GEMM (torch.matmul,
    the vendor BLAS) on this GPU."""
    a = torch.empty(4 << 30, dtype=torch.uint8, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        b.copy_(a)
    e1.record()
    torch.cuda.synchronize()
    hbm = 5 * 2 * a.numel() / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del a, b
    n = 8192
    x = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    y = torch.randn(n, n, device="cuda", dtype=torch.bfloat16)
    z = x @ y
    e0.record()
    for _ in range(10):
        z = x @ y
    e1.record()
    torch.cuda.synchronize()
    tf = 10 * 2.0 * n ** 3 / (e0.elapsed_time(e1) * 1e-3) / 1e12
    del x, y, z
    torch.cuda.empty_cache()
    return {"hbm_copy_GBs": hbm, "bf16_gemm_TFLOPs": tf,
            "note": "4 GiB device copy (2 x bytes / time); torch.matmul 8192^3 bf16"}


def secondary_hca_prefill_whole(reps=2):
    """The whole 2^20-token HCA prefill: all 128 chunks, each compressing its
    8192 tokens and running dense attention for its 8192 queries over the
    entries visible to them.  Token projections, all 128 query chunks and
    all 128 output chunks are resident in HBM (about 150 GB)."""
    w = synth.HCA_PREFILL_1M
    chunk, nch = w.chunk, w.tokens // w.chunk
    log(f"setup {w.name} (whole sequence)")
    lay = path.HcaLayer(w, 1, w.tokens // w.m)
    toks = [{k: v[None].contiguous() for k, v in synth.token_chunk(w, 0, c, chunk, 0, "cuda").items()}
            for c in range(nch)]
    qs = [synth.query_chunk(w, 0, c, chunk, 0, "cuda", with_index=False)["q"][None].contiguous() for c in range(nch)]
    odt = synth.TORCH_DTYPE[w.out_dtype]
    outs = [torch.empty((1, chunk, w.heads, w.d_nope), dtype=odt, device="cuda") for _ in range(nch)]
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(nch)]

    def whole(time_attn=False):
        for c in range(nch):
            cb.compress_prefill(lay.kv, c * chunk, toks[c]["a"], toks[c]["za"], lay.prm["Ba"])
            if time_attn:
                evs[c][0].record()
            cb.dense_attn_prefill(lay.adesc, lay.kv, c * chunk, qs[c], w.tau, outs[c])
            if time_attn:
                evs[c][1].record()
    whole()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        whole()
    b.record()
    torch.cuda.synchronize()
    s_total = a.elapsed_time(b) / reps * 1e-3
    whole(time_attn=True)
    torch.cuda.synchronize()
    s_attn = sum(e0.elapsed_time(e1) for e0, e1 in evs) * 1e-3
    t = np.arange(w.tokens, dtype=np.int64)
    flops = 2.0 * float(np.minimum((t + 1) // w.m, w.tokens // w.m).sum()) * w.heads * (w.c + w.d_nope)
    del toks, qs, outs
    return {"workload": w.name + " (whole sequence)", "metric": "HCA prefill tokens/s (2^20 tokens, 128 chunks)",
            "value": w.tokens / s_total, "unit": "tokens/s", "s_per_prefill": s_total,
            "roofline": {"bound": "mfma", "kernel": "dense attention prefill (128 launches)",
                         "achieved": flops / s_attn / 1e12, "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                         "frac": flops / s_attn / 1e12 / PEAK_BF16_TFLOPS, "algorithmic_flop": flops,
                         "attention_s": s_attn, "whole_step_frac": flops / s_total / 1e12 / PEAK_BF16_TFLOPS}}


def secondary_tiny(reps=20):
    """The tiny fp32 CSA prefill (2048 tokens, 8 heads, 32 + 32 dims, k = 64;
    the parity workload) end to end on the GPU, and the oracle on the host."""
    w = synth.TINY_CSA_PREFILL_FP32
    pr = {k: v.to("cuda") for k, v in synth.tiny_projections(w).items()}
    T, m, k = w.tokens, w.m, w.topk
    N = T // m
    kv = cb.KVCache(cb.cache_desc(m, True, w.d_nope, w.d_rope, "f32", "f32", "f32", N), 1)
    keys = cb.KVCache(cb.cache_desc(m, True, w.idx_dim, 0, "f32", "f32", "f32", N), 1)
    u = lambda t: t[None].contiguous()
    x = {kk: u(v) for kk, v in pr.items() if v.dim() > 1 and v.shape[0] == T}
    idesc = cb.index_desc(w.idx_heads, w.idx_dim, "f32", "f32", "f32", "f32", m, N)
    adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, "f32", "f32", "f32", "f32", m, N)
    idx = torch.empty((1, T, k), dtype=torch.int32, device="cuda")
    o = torch.empty((1, T, w.heads, w.d_nope), dtype=torch.float32, device="cuda")
    iws = cb.workspace(cb.workspace_bytes(cb.OP_INDEX_TOPK_PREFILL, idesc, 1, T, 0, k))

    def step():
        cb.compress_prefill(kv, 0, x["a"], x["za"], pr["Ba"], x["b"], x["zb"], pr["Bb"])
        cb.compress_prefill(keys, 0, x["ka"], x["kza"], pr["kBa"], x["kb"], x["kzb"], pr["kBb"])
        cb.index_topk_prefill(idesc, keys, 0, x["qI"], x["w"], k, idx, ws=iws)
        cb.sparse_attn_prefill(adesc, kv, 0, x["q"], idx, w.tau, o)
    step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        step()
    b.record()
    torch.cuda.synchronize()
    ms = a.elapsed_time(b) / reps
    line = {"workload": w.name, "metric": "tiny fp32 CSA prefill tokens/s (parity workload, generic fp32 kernels)",
            "value": T / (ms * 1e-3), "unit": "tokens/s", "ms_per_step": ms}
    if CPU_BASELINE:
        from oracle import csa
        h = {kk: v.cpu().double().numpy() for kk, v in pr.items()}
        t0 = time.perf_counter()
        cache = csa.finalize_kv(csa.compress(h["a"], h["za"], h["Ba"], m, h["b"], h["zb"], h["Bb"]), 0, m,
                                w.d_nope, w.rope_base, "f32", "f32")
        kk_ = csa.finalize_keys(csa.compress(h["ka"], h["kza"], h["kBa"], m, h["kb"], h["kzb"], h["kBb"]), "f32")
        rows = np.arange(T)
        csa.csa_rows(rows, rows, h["q"], h["qI"], h["w"], cache, kk_, m, k, w.d_nope, w.rope_base, w.tau)
        dt = time.perf_counter() - t0
        model, threads, _ = host_cpu()
        line["cpu_baseline"] = {"value": T / dt, "unit": "tokens/s", "cores": threads, "cpu": model, "kind": "oracle",
                                "sample": f"the whole workload ({T} tokens: compression, indexer, top-k, attention)"}
    return line

def secondary_hca_prefill(steps=5, qk="bf16"):
    """The last 8192-token chunk of a 2^20-token HCA prefill: compress the
    chunk's tokens and run dense attention for its 8192 queries over the
    8192 entries of the whole context (inputs resident in HBM).  qk="fp8":
    the attention's non-RoPE QK product in FP8 (MXFP8 query against the FP8
    codes); its roofline peak is the time-weighted mix of the FP8 (QK
    non-RoPE) and BF16 (QK RoPE, PV) MFMA peaks."""
    w = synth.HCA_PREFILL_1M
    chunk = w.chunk
    c = w.tokens // chunk - 1
    log(f"setup {w.name}")
    lay = path.HcaLayer(w, 1, w.tokens // w.m)
    lay.prefill_context(w.tokens, progress=context_progress)
    tok = synth.token_chunk(w, 0, c, chunk, 0, "cuda")
    x = {k: v[None].contiguous() for k, v in tok.items()}
    q = synth.query_chunk(w, 0, c, chunk, 0, "cuda", with_index=False)["q"][None].contiguous()
    o = torch.empty((1, chunk, w.heads, w.d_nope), dtype=synth.TORCH_DTYPE[w.out_dtype], device="cuda")
    pos0 = c * chunk
    adesc = type(lay.adesc).from_buffer_copy(lay.adesc)
    adesc.qk_mode = cb.FP8E4M3 if qk == "fp8" else 0

    def step(ev=None):
        cb.compress_prefill(lay.kv, pos0, x["a"], x["za"], lay.prm["Ba"])
        if ev is not None:
            ev[0].record()
        cb.dense_attn_prefill(adesc, lay.kv, pos0, q, w.tau, o)
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
    peak = PEAK_BF16_TFLOPS
    if qk == "fp8":  # FP8 share: 2 * 64 * d_nope flop per pair of the 2 * 64 * (c + d_nope)
        f8 = w.d_nope / (w.c + w.d_nope)
        peak = 1.0 / (f8 / PEAK_FP8_TFLOPS + (1.0 - f8) / PEAK_BF16_TFLOPS)
    return {"workload": w.name + " (last chunk)" + (", FP8 QK" if qk == "fp8" else ""),
            "metric": "HCA prefill tokens/s (chunk of 8192 at 2^20 context)",
            "value": chunk / (ms * 1e-3), "unit": "tokens/s", "ms_per_chunk": ms,
            "roofline": {"bound": "mfma", "kernel": "dense attention prefill", "achieved": ach,
                         "peak": peak, "unit": "TFLOP/s", "frac": ach / peak,
                         "algorithmic_flop_per_launch": flops, "avg_launch_ms": attn_ms}}


def secondary_mxfp4_prefill_indexer(steps=5):
    """Lightning indexer + top-k of the 32768-token prefill with MXFP4 keys
    and query and BF16 scores (the 2^20-context pair's precision): the query
    operands are formed once per row, then the fused kernel scores 4 query
    rows per workgroup with the scaled FP4 MFMA straight into LDS and selects
    from there (no score row reaches HBM).  Keys from the MXFP4 compressor,
    inputs resident.  Roofline: the scoring flops against the dense FP4 MFMA
    peak; the kernel's time is mostly its select."""
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
    flops = 2.0 * visible * w.idx_heads * w.idx_dim
    ach = flops / (ms * 1e-3) / 1e12
    return {"workload": w.name, "metric": "MXFP4 prefill indexer + top-k tokens/s (L=32768, k=1024)",
            "value": w.tokens / (ms * 1e-3), "unit": "tokens/s", "ms_per_launch": ms,
            "roofline": {"bound": "mfma", "achieved": ach, "peak": PEAK_FP4_TFLOPS, "unit": "TFLOP/s",
                         "frac": ach / PEAK_FP4_TFLOPS, "algorithmic_flop_per_launch": flops}}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=2)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=15.0)
    ap.add_argument("--replays", type=int, default=12, help="timed replays of each 128-step decode graph")
    ap.add_argument("--decode-eager", type=int, default=0,
                    help="run this many eager decode steps instead of the graphs (for counter collection)")
    ap.add_argument("--no-secondary", action="store_true", help="skip the decode workloads")
    ap.add_argument("--copy-calib", action="store_true", help="run a 1 GiB copy first (counter calibration)")
    ap.add_argument("--only", choices=["csa-decode", "hca-decode", "pair-decode", "swa-decode", "paged-decode",
                                       "project-prefill", "planted-recall", "hca-prefill", "hca-prefill-fp8qk",
                                       "hca-decode-fp8qk",
                                       "hca-prefill-whole",
                                       "mxfp4-indexer", "tiny", "peaks"],
                    help="run just this secondary workload and print its line(s) (for profiling)")
    args = ap.parse_args()
    global CPU_BASELINE, REPLAYS, DECODE_EAGER
    CPU_BASELINE = not args.no_cpu_baseline
    REPLAYS = args.replays
    DECODE_EAGER = args.decode_eager
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
              "swa-decode": swa_decode_lines, "paged-decode": paged_decode_lines,
              "project-prefill": secondary_project_prefill, "planted-recall": planted_recall_line,
              "hca-prefill": secondary_hca_prefill, "hca-prefill-whole": secondary_hca_prefill_whole,
              "hca-prefill-fp8qk": lambda: secondary_hca_prefill(qk="fp8"),
              "hca-decode-fp8qk": lambda: hca_decode_line(qk="fp8"),
              "mxfp4-indexer": secondary_mxfp4_prefill_indexer, "tiny": secondary_tiny,
              "peaks": measured_peaks}[args.only]
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
        log("measured peaks")
        pk = measured_peaks()
        out["measured_peaks"] = pk
        out["roofline"]["frac_vs_measured_gemm"] = achieved / pk["bf16_gemm_TFLOPs"]
        out["secondary"] = secondary_lines()
        for line in out["secondary"]:
            r = line.get("roofline", {})
            if r.get("unit") == "GB/s":
                r["frac_vs_measured_copy"] = r["achieved"] / pk["hbm_copy_GBs"]
            elif r.get("unit") == "TFLOP/s":
                r["frac_vs_measured_gemm"] = r["achieved"] / pk["bf16_gemm_TFLOPs"]
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
