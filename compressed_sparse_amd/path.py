"""Whole CSA / HCA steps built from the C-ABI entry points.

A layer object owns the compressed caches of B sequences and chains the
library calls of one step; every computation runs in libcsa's kernels, this
module only allocates buffers and orders the calls:

* CSA ([CSA/HCA 混注意力] §1.1): compress the KV entries and the indexer keys
  (two instances of the overlapped compressor), lightning indexer + top-k,
  sparse attention.
* HCA (§1.2): compress with m' = 128 (single window), dense attention.

Context tokens of sequence b at positions [c*chunk, (c+1)*chunk) are the
seeded tensors synth.token_chunk(w, b, c, ...), so a decode step at position
p reads the same token a longer prefill would.
"""
import math

import torch

from . import binding as cb
from . import synth


def _stack(tensors):
    return torch.stack(tensors, 0).contiguous()


def block_tables(entries, page_size, capacity, seed=0, device="cuda", share=None):
    """Block tables of B sequences over one page pool: sequence b gets
    ceil(entries[b] / page_size) pages, in a seeded random order of the pool;
    its other logical pages are -1.  share = (b0, b1, n): sequence b1's first
    n pages are sequence b0's (a shared prefix).  Returns (int32 table
    [B][capacity / page_size], pool_pages)."""
    assert capacity % page_size == 0
    tps = capacity // page_size
    need = [min(tps, -(-int(e) // page_size)) for e in entries]
    own = list(need)
    if share is not None:
        b0, b1, n = share
        assert n <= min(need[b0], need[b1])
        own[b1] -= n
    pool = max(1, sum(own))
    g = torch.Generator().manual_seed(1000 + seed)
    perm = torch.randperm(pool, generator=g).to(torch.int32)
    table = torch.full((len(entries), tps), -1, dtype=torch.int32)
    at = 0
    for b, nb in enumerate(need):
        if share is not None and b == share[1]:
            n = share[2]
            table[b, :n] = table[share[0], :n]
            table[b, n:nb] = perm[at:at + nb - n]
            at += nb - n
        else:
            table[b, :nb] = perm[at:at + nb]
            at += nb
    return table.to(device), pool


def _caches(desc_fn, B, device, page_size, block_table, pool_pages, capacity):
    """cache_desc arguments -> KVCache, contiguous or paged."""
    if page_size:
        return cb.KVCache(desc_fn(page_size=page_size, pool_pages=pool_pages), B, device, block_table)
    return cb.KVCache(desc_fn(), B, device)


class CsaLayer:
    """seq_ids: the seeded sequence held in each batch slot (default 0..B-1).
    page_size > 0: paged KV and indexer-key caches over pools of pool_pages
    pages, both addressed by block_table (the same logical entries)."""

    def __init__(self, w: synth.Workload, B, capacity, device="cuda", seed=0, seq_ids=None, page_size=0,
                 block_table=None, pool_pages=0):
        self.w, self.B, self.cap, self.device, self.seed = w, B, capacity, device, seed
        self.seq_ids = list(seq_ids) if seq_ids is not None else list(range(B))
        assert len(self.seq_ids) == B
        act = w.act_dtype
        pg = dict(page_size=page_size, pool_pages=pool_pages) if page_size else {}
        self.kv = _caches(lambda **k: cb.cache_desc(w.m, w.overlap, w.d_nope, w.d_rope, act, w.nope_fmt, w.rope_fmt,
                                                    capacity, w.rope_base, **k),
                          B, device, page_size, block_table, pool_pages, capacity)
        self.keys = _caches(lambda **k: cb.cache_desc(w.m, w.overlap, w.idx_dim, 0, act, w.key_fmt, "f32", capacity,
                                                      **k),
                            B, device, page_size, block_table, pool_pages, capacity)
        self.idesc = cb.index_desc(w.idx_heads, w.idx_dim, act, w.qk_fmt, w.key_fmt, w.score_fmt, w.m, capacity, **pg)
        self.adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, act, w.out_dtype, w.nope_fmt, w.rope_fmt, w.m,
                                  capacity, w.rope_base, **pg)
        self.prm = synth.compressor_params(w, seed, device)
        self.iws = None
        self.aws = None

    def caches(self):
        return [self.kv, self.keys]

    # -- context ----------------------------------------------------------
    def prefill_context(self, T, chunk=None, progress=None):
        """Compresses tokens [0, T) of every sequence into the caches
        (progress(done, total) after every 16 chunks, when given)."""
        chunk = chunk or self.w.chunk or T
        p = self.prm
        nc = math.ceil(T / chunk)
        for c in range(nc):
            if progress and c % 16 == 15:
                progress(c + 1, nc)
            n = min(chunk, T - c * chunk)
            toks = [synth.token_chunk(self.w, sid, c, chunk, self.seed, self.device) for sid in self.seq_ids]
            x = {k: _stack([t[k][:n] for t in toks]) for k in toks[0]}
            cb.compress_prefill(self.kv, c * chunk, x["a"], x["za"], p["Ba"], x.get("b"), x.get("zb"), p.get("Bb"))
            cb.compress_prefill(self.keys, c * chunk, x["ka"], x["kza"], p["kBa"], x.get("kb"), x.get("kzb"),
                                p.get("kBb"))

    def prefill_contexts(self, lengths, chunk=None):
        """Mixed contexts: tokens [0, lengths[b]) of sequence b, one sequence
        per call (its ring and block-table row)."""
        chunk = chunk or self.w.chunk
        p = self.prm
        for b, (sid, T) in enumerate(zip(self.seq_ids, lengths)):
            kv, keys = self.kv.seq_view(b), self.keys.seq_view(b)
            for c in range(math.ceil(T / chunk)):
                n = min(chunk, T - c * chunk)
                t = synth.token_chunk(self.w, sid, c, chunk, self.seed, self.device)
                x = {k: v[:n][None].contiguous() for k, v in t.items()}
                cb.compress_prefill(kv, c * chunk, x["a"], x["za"], p["Ba"], x.get("b"), x.get("zb"), p.get("Bb"))
                cb.compress_prefill(keys, c * chunk, x["ka"], x["kza"], p["kBa"], x.get("kb"), x.get("kzb"),
                                    p.get("kBb"))

    # -- decode -----------------------------------------------------------
    def decode_inputs(self, positions, chunk=None):
        """Token projections and queries of each sequence at its position."""
        return self.decode_input_steps([positions], chunk)[0]

    def decode_input_steps(self, steps, chunk=None):
        """decode_inputs for a list of steps (each a list of positions, one per
        sequence); every seeded chunk is drawn once."""
        chunk = chunk or self.w.chunk
        per = [[None] * self.B for _ in steps]
        for b, sid in enumerate(self.seq_ids):  # one sequence's chunks alive at a time
            by_chunk = {}
            for i, positions in enumerate(steps):
                by_chunk.setdefault(int(positions[b]) // chunk, []).append(i)
            for c, its in by_chunk.items():
                d = synth.token_chunk(self.w, sid, c, chunk, self.seed, self.device)
                d.update(synth.query_chunk(self.w, sid, c, chunk, self.seed, self.device))
                rows = torch.tensor([int(steps[i][b]) % chunk for i in its], device=self.device)
                # the rows gathered into new tensors (an index kernel), so the chunk is freed
                got = {k: v.index_select(0, rows) for k, v in d.items()}
                for j, i in enumerate(its):
                    per[i][b] = {k: v[j] for k, v in got.items()}
                del d
        out = []
        for i, positions in enumerate(steps):
            x = {k: _stack([p[k] for p in per[i]]) for k in per[i][0]}
            x["pos"] = torch.tensor([int(p) for p in positions], dtype=torch.int64, device=self.device)
            out.append(x)
        return out

    def alloc_decode_outputs(self):
        w = self.w
        odt = synth.TORCH_DTYPE[w.out_dtype]
        out = {"idx": torch.empty((self.B, w.topk), dtype=torch.int32, device=self.device),
               "o": torch.empty((self.B, w.heads, w.d_nope), dtype=odt, device=self.device),
               "lse": torch.empty((self.B, w.heads), dtype=torch.float32, device=self.device)}
        self.iws = cb.workspace(cb.workspace_bytes(cb.OP_INDEX_TOPK_DECODE, self.idesc, self.B, 1, 0, w.topk),
                                self.device)
        self.aws = cb.workspace(cb.workspace_bytes(cb.OP_SPARSE_ATTN_DECODE, self.adesc, self.B, 1, 0, w.topk),
                                self.device)
        self.sws = cb.workspace(cb.decode_step_workspace_bytes(self.idesc, self.adesc, self.B, w.topk), self.device)
        return out

    def decode_step(self, x, out, scores=None):
        """One CSA decode step through the fused entry point: the new token
        enters both compressors (an entry completed at this position is
        visible to it), then indexer + top-k and sparse attention."""
        cb.decode_step(self.kv, self.keys, self.idesc, self.adesc, x["pos"], x, self.prm, self.w.topk, self.w.tau,
                       out["idx"], out["o"], out["lse"], scores, ws=self.sws)

    def decode_step_separate(self, x, out, scores=None):
        """The same step as the four separate entry points."""
        p, w = self.prm, self.w
        cb.compress_decode(self.kv, x["pos"], x["a"], x["za"], p["Ba"], x.get("b"), x.get("zb"), p.get("Bb"))
        cb.compress_decode(self.keys, x["pos"], x["ka"], x["kza"], p["kBa"], x.get("kb"), x.get("kzb"), p.get("kBb"))
        cb.index_topk_decode(self.idesc, self.keys, x["pos"], x["qI"], x["w"], w.topk, out["idx"], scores,
                             ws=self.iws)
        cb.sparse_attn_decode(self.adesc, self.kv, x["pos"], x["q"], out["idx"], w.tau, out["o"], out["lse"],
                              ws=self.aws)


class HcaLayer:
    """seq_ids: the seeded sequence held in each batch slot (default 0..B-1)."""

    def __init__(self, w: synth.Workload, B, capacity, device="cuda", seed=0, seq_ids=None, page_size=0,
                 block_table=None, pool_pages=0, qk="bf16"):
        """qk: "bf16", or "fp8" for the FP8 QK product (MXFP8 query against the
        FP8 cache codes)."""
        self.w, self.B, self.cap, self.device, self.seed = w, B, capacity, device, seed
        self.seq_ids = list(seq_ids) if seq_ids is not None else list(range(B))
        assert len(self.seq_ids) == B
        pg = dict(page_size=page_size, pool_pages=pool_pages) if page_size else {}
        self.kv = _caches(lambda **k: cb.cache_desc(w.m, False, w.d_nope, w.d_rope, w.act_dtype, w.nope_fmt,
                                                    w.rope_fmt, capacity, w.rope_base, **k),
                          B, device, page_size, block_table, pool_pages, capacity)
        self.adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, w.act_dtype, w.out_dtype, w.nope_fmt, w.rope_fmt,
                                  w.m, capacity, w.rope_base, qk=qk, **pg)
        self.prm = synth.compressor_params(w, seed, device)
        self.aws = None

    def caches(self):
        return [self.kv]

    def compress_chunk(self, c, chunk, n=None):
        n = n or chunk
        toks = [synth.token_chunk(self.w, sid, c, chunk, self.seed, self.device) for sid in self.seq_ids]
        x = {k: _stack([t[k][:n] for t in toks]) for k in toks[0]}
        cb.compress_prefill(self.kv, c * chunk, x["a"], x["za"], self.prm["Ba"])

    def prefill_context(self, T, chunk=None, progress=None):
        chunk = chunk or self.w.chunk or T
        nc = math.ceil(T / chunk)
        for c in range(nc):
            if progress and c % 16 == 15:
                progress(c + 1, nc)
            self.compress_chunk(c, chunk, min(chunk, T - c * chunk))

    def prefill_contexts(self, lengths, chunk=None):
        """Mixed contexts: tokens [0, lengths[b]) of sequence b, one sequence per call."""
        chunk = chunk or self.w.chunk
        for b, (sid, T) in enumerate(zip(self.seq_ids, lengths)):
            kv = self.kv.seq_view(b)
            for c in range(math.ceil(T / chunk)):
                n = min(chunk, T - c * chunk)
                t = synth.token_chunk(self.w, sid, c, chunk, self.seed, self.device)
                cb.compress_prefill(kv, c * chunk, t["a"][:n][None].contiguous(), t["za"][:n][None].contiguous(),
                                    self.prm["Ba"])

    def prefill_chunk_attention(self, c, chunk, q, o, lse=None):
        """Dense attention of the queries at positions [c*chunk, c*chunk + T)."""
        cb.dense_attn_prefill(self.adesc, self.kv, c * chunk, q, self.w.tau, o, lse)

    def decode_inputs(self, positions, chunk=None):
        return self.decode_input_steps([positions], chunk)[0]

    def decode_input_steps(self, steps, chunk=None):
        """decode_inputs for a list of steps; every seeded chunk is drawn once."""
        chunk = chunk or self.w.chunk
        per = [[None] * self.B for _ in steps]
        for b, sid in enumerate(self.seq_ids):  # one sequence's chunks alive at a time
            by_chunk = {}
            for i, positions in enumerate(steps):
                by_chunk.setdefault(int(positions[b]) // chunk, []).append(i)
            for c, its in by_chunk.items():
                d = synth.token_chunk(self.w, sid, c, chunk, self.seed, self.device)
                d["q"] = synth.query_chunk(self.w, sid, c, chunk, self.seed, self.device, with_index=False)["q"]
                rows = torch.tensor([int(steps[i][b]) % chunk for i in its], device=self.device)
                # the rows gathered into new tensors (an index kernel), so the chunk is freed
                got = {k: v.index_select(0, rows) for k, v in d.items()}
                for j, i in enumerate(its):
                    per[i][b] = {k: v[j] for k, v in got.items()}
                del d
        out = []
        for i, positions in enumerate(steps):
            x = {k: _stack([p[k] for p in per[i]]) for k in per[i][0]}
            x["pos"] = torch.tensor([int(p) for p in positions], dtype=torch.int64, device=self.device)
            out.append(x)
        return out

    def alloc_decode_outputs(self):
        w = self.w
        out = {"o": torch.empty((self.B, w.heads, w.d_nope), dtype=synth.TORCH_DTYPE[w.out_dtype], device=self.device),
               "lse": torch.empty((self.B, w.heads), dtype=torch.float32, device=self.device)}
        self.aws = cb.workspace(cb.workspace_bytes(cb.OP_DENSE_ATTN_DECODE, self.adesc, self.B, 1, 0, 0), self.device)
        return out

    def decode_step(self, x, out):
        cb.compress_decode(self.kv, x["pos"], x["a"], x["za"], self.prm["Ba"])
        cb.dense_attn_decode(self.adesc, self.kv, x["pos"], x["q"], self.w.tau, out["o"], out["lse"], ws=self.aws)


class SwaBranch:
    """The sliding-window branch of a layer: per-token entries of the layer's
    C^a rows (the compressor with m = 1: a window of one token passes its row
    through, turned by RoPE at the token's position and stored like the
    layer's entries) and dense attention over the last `window` of them,
    joined to the layer's (o, lse) by csa_lse_merge: one softmax over the
    union of the layer's keys and the window's tokens."""

    def __init__(self, w: synth.Workload, B, capacity, window, device="cuda", seed=0, seq_ids=None):
        self.w, self.B, self.cap, self.window, self.device, self.seed = w, B, capacity, window, device, seed
        self.seq_ids = list(seq_ids) if seq_ids is not None else list(range(B))
        act = w.act_dtype
        self.kv = cb.KVCache(cb.cache_desc(1, False, w.d_nope, w.d_rope, act, w.nope_fmt, w.rope_fmt, capacity,
                                           w.rope_base), B, device)
        self.adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, act, w.out_dtype, w.nope_fmt, w.rope_fmt, 1, capacity,
                                  w.rope_base, window=window)
        self.Ba = torch.zeros((1, w.c), dtype=torch.float32, device=device)  # one row: weight 1 whatever the bias
        self.aws = None

    def caches(self):
        return [self.kv]

    def prefill_context(self, T, chunk=None, progress=None):
        chunk = chunk or self.w.chunk or T
        nc = math.ceil(T / chunk)
        for c in range(nc):
            if progress and c % 16 == 15:
                progress(c + 1, nc)
            n = min(chunk, T - c * chunk)
            toks = [synth.token_chunk(self.w, sid, c, chunk, self.seed, self.device, names=["a", "za"])
                    for sid in self.seq_ids]
            x = {k: _stack([t[k][:n] for t in toks]) for k in toks[0]}
            cb.compress_prefill(self.kv, c * chunk, x["a"], x["za"], self.Ba)

    def alloc_decode_outputs(self):
        w = self.w
        self.aws = cb.workspace(cb.workspace_bytes(cb.OP_DENSE_ATTN_DECODE, self.adesc, self.B, 1, 0, 0), self.device)
        return {"o": torch.empty((self.B, w.heads, w.d_nope), dtype=synth.TORCH_DTYPE[w.out_dtype], device=self.device),
                "lse": torch.empty((self.B, w.heads), dtype=torch.float32, device=self.device)}

    def decode_step(self, x, own, layer_out):
        """The new token enters the window; window attention into `own`, then
        merged into the layer's outputs in place."""
        cb.compress_decode(self.kv, x["pos"], x["a"], x["za"], self.Ba)
        cb.dense_attn_decode(self.adesc, self.kv, x["pos"], x["q"], self.w.tau, own["o"], own["lse"], ws=self.aws)
        cb.lse_merge(layer_out["o"], layer_out["lse"], own["o"], own["lse"], layer_out["o"], layer_out["lse"])


class DecodeGraph:
    """n consecutive decode steps of one or more layers captured in one HIP
    graph.  Every run starts from the same state: the graph first restores
    the staging rings of the layers' caches from a snapshot taken before
    capture (a device copy, no memset), so each replay recomputes the same
    steps from the same inputs; entries the steps complete are rewritten with
    the same values before any later step reads them.  An eager run of the
    same steps (warm-up) precedes capture."""

    def __init__(self, layers, step_fn, n_steps):
        self.rings = [c.ring for lay in layers for c in lay.caches()]
        self.snaps = [r.clone() for r in self.rings]
        self.step_fn, self.n = step_fn, n_steps
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(s):
            self.run_eager()
        torch.cuda.current_stream().wait_stream(s)
        torch.cuda.synchronize()
        self.graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(self.graph):
            self.run_eager()

    def run_eager(self):
        for r, sn in zip(self.rings, self.snaps):
            r.copy_(sn)
        for i in range(self.n):
            self.step_fn(i)

    def replay(self):
        self.graph.replay()


class CsaPrefill:
    """One sequence's CSA prefill over `tokens` positions starting at 0:
    seeded inputs resident on the device, caches, outputs and workspaces."""

    def __init__(self, w: synth.Workload, device="cuda", seed=0, tokens=None):
        T = tokens or w.tokens
        self.w, self.T, self.device = w, T, device
        m = w.m
        N = T // m
        tok = synth.token_chunk(w, 0, 0, T, seed, device)
        qs = synth.query_chunk(w, 0, 0, T, seed, device)
        self.prm = synth.compressor_params(w, seed, device)
        u = lambda t: t[None].contiguous()
        self.tok = {k: u(v) for k, v in tok.items()}
        self.q, self.qI, self.wt = u(qs["q"]), u(qs["qI"]), u(qs["w"])
        act = w.act_dtype
        self.kv = cb.KVCache(cb.cache_desc(m, True, w.d_nope, w.d_rope, act, w.nope_fmt, w.rope_fmt, N,
                                           w.rope_base), 1, device)
        self.keys = cb.KVCache(cb.cache_desc(m, True, w.idx_dim, 0, act, w.key_fmt, "f32", N), 1, device)
        self.idesc = cb.index_desc(w.idx_heads, w.idx_dim, act, w.qk_fmt, w.key_fmt, w.score_fmt, m, N)
        self.adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, act, w.out_dtype, w.nope_fmt, w.rope_fmt, m, N,
                                  w.rope_base)
        odt = synth.TORCH_DTYPE[w.out_dtype]
        self.idx = torch.empty((1, T, w.topk), dtype=torch.int32, device=device)
        self.o = torch.empty((1, T, w.heads, w.d_nope), dtype=odt, device=device)
        self.lse = torch.empty((1, T, w.heads), dtype=torch.float32, device=device)
        self.iws = cb.workspace(cb.workspace_bytes(cb.OP_INDEX_TOPK_PREFILL, self.idesc, 1, T, 0, w.topk), device)
        self.aws = cb.workspace(cb.workspace_bytes(cb.OP_SPARSE_ATTN_PREFILL, self.adesc, 1, T, 0, w.topk), device)

    def step(self, attn_events=None):
        """Compress KV entries and indexer keys, select, attend.  When given,
        attn_events = (start, end) bracket the attention launch."""
        t, p, w = self.tok, self.prm, self.w
        cb.compress_prefill(self.kv, 0, t["a"], t["za"], p["Ba"], t["b"], t["zb"], p["Bb"])
        cb.compress_prefill(self.keys, 0, t["ka"], t["kza"], p["kBa"], t["kb"], t["kzb"], p["kBb"])
        cb.index_topk_prefill(self.idesc, self.keys, 0, self.qI, self.wt, w.topk, self.idx, ws=self.iws)
        if attn_events is not None:
            attn_events[0].record()
        cb.sparse_attn_prefill(self.adesc, self.kv, 0, self.q, self.idx, w.tau, self.o, self.lse, ws=self.aws)
        if attn_events is not None:
            attn_events[1].record()
