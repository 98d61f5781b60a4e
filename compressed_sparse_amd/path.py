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


class CsaLayer:
    def __init__(self, w: synth.Workload, B, capacity, device="cuda", seed=0):
        self.w, self.B, self.cap, self.device, self.seed = w, B, capacity, device, seed
        act = w.act_dtype
        self.kv = cb.KVCache(cb.cache_desc(w.m, w.overlap, w.d_nope, w.d_rope, act, w.nope_fmt, w.rope_fmt,
                                           capacity, w.rope_base), B, device)
        self.keys = cb.KVCache(cb.cache_desc(w.m, w.overlap, w.idx_dim, 0, act, w.key_fmt, "f32", capacity), B,
                               device)
        self.idesc = cb.index_desc(w.idx_heads, w.idx_dim, act, w.qk_fmt, w.key_fmt, w.score_fmt, w.m, capacity)
        self.adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, act, w.out_dtype, w.nope_fmt, w.rope_fmt, w.m,
                                  capacity, w.rope_base)
        self.prm = synth.compressor_params(w, seed, device)
        self.iws = None
        self.aws = None

    # -- context ----------------------------------------------------------
    def prefill_context(self, T, chunk=None):
        """Compresses tokens [0, T) of every sequence into the caches."""
        chunk = chunk or self.w.chunk or T
        p = self.prm
        for c in range(math.ceil(T / chunk)):
            n = min(chunk, T - c * chunk)
            toks = [synth.token_chunk(self.w, b, c, chunk, self.seed, self.device) for b in range(self.B)]
            x = {k: _stack([t[k][:n] for t in toks]) for k in toks[0]}
            cb.compress_prefill(self.kv, c * chunk, x["a"], x["za"], p["Ba"], x.get("b"), x.get("zb"), p.get("Bb"))
            cb.compress_prefill(self.keys, c * chunk, x["ka"], x["kza"], p["kBa"], x.get("kb"), x.get("kzb"),
                                p.get("kBb"))

    # -- decode -----------------------------------------------------------
    def decode_inputs(self, positions, chunk=None):
        """Token projections and queries of each sequence at its position."""
        chunk = chunk or self.w.chunk
        toks, qs = [], []
        for b, pos in enumerate(positions):
            c, r = divmod(int(pos), chunk)
            toks.append({k: v[r] for k, v in synth.token_chunk(self.w, b, c, chunk, self.seed, self.device).items()})
            qs.append({k: v[r] for k, v in synth.query_chunk(self.w, b, c, chunk, self.seed, self.device).items()})
        x = {k: _stack([t[k] for t in toks]) for k in toks[0]}
        x.update({k: _stack([q[k] for q in qs]) for k in qs[0]})
        x["pos"] = torch.tensor([int(p) for p in positions], dtype=torch.int64, device=self.device)
        return x

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
        return out

    def decode_step(self, x, out, scores=None):
        """One CSA decode step: the new token enters both compressors (an
        entry completed at this position is visible to it), then indexer +
        top-k and sparse attention."""
        p, w = self.prm, self.w
        cb.compress_decode(self.kv, x["pos"], x["a"], x["za"], p["Ba"], x.get("b"), x.get("zb"), p.get("Bb"))
        cb.compress_decode(self.keys, x["pos"], x["ka"], x["kza"], p["kBa"], x.get("kb"), x.get("kzb"), p.get("kBb"))
        cb.index_topk_decode(self.idesc, self.keys, x["pos"], x["qI"], x["w"], w.topk, out["idx"], scores,
                             ws=self.iws)
        cb.sparse_attn_decode(self.adesc, self.kv, x["pos"], x["q"], out["idx"], w.tau, out["o"], out["lse"],
                              ws=self.aws)


class HcaLayer:
    def __init__(self, w: synth.Workload, B, capacity, device="cuda", seed=0):
        self.w, self.B, self.cap, self.device, self.seed = w, B, capacity, device, seed
        self.kv = cb.KVCache(cb.cache_desc(w.m, False, w.d_nope, w.d_rope, w.act_dtype, w.nope_fmt, w.rope_fmt,
                                           capacity, w.rope_base), B, device)
        self.adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, w.act_dtype, w.out_dtype, w.nope_fmt, w.rope_fmt,
                                  w.m, capacity, w.rope_base)
        self.prm = synth.compressor_params(w, seed, device)
        self.aws = None

    def compress_chunk(self, c, chunk, n=None):
        n = n or chunk
        toks = [synth.token_chunk(self.w, b, c, chunk, self.seed, self.device) for b in range(self.B)]
        x = {k: _stack([t[k][:n] for t in toks]) for k in toks[0]}
        cb.compress_prefill(self.kv, c * chunk, x["a"], x["za"], self.prm["Ba"])

    def prefill_context(self, T, chunk=None):
        chunk = chunk or self.w.chunk or T
        for c in range(math.ceil(T / chunk)):
            self.compress_chunk(c, chunk, min(chunk, T - c * chunk))

    def prefill_chunk_attention(self, c, chunk, q, o, lse=None):
        """Dense attention of the queries at positions [c*chunk, c*chunk + T)."""
        cb.dense_attn_prefill(self.adesc, self.kv, c * chunk, q, self.w.tau, o, lse)

    def decode_inputs(self, positions, chunk=None):
        chunk = chunk or self.w.chunk
        toks, qs = [], []
        for b, pos in enumerate(positions):
            c, r = divmod(int(pos), chunk)
            toks.append({k: v[r] for k, v in synth.token_chunk(self.w, b, c, chunk, self.seed, self.device).items()})
            qs.append(synth.query_chunk(self.w, b, c, chunk, self.seed, self.device, with_index=False)["q"][r])
        x = {k: _stack([t[k] for t in toks]) for k in toks[0]}
        x["q"] = _stack(qs)
        x["pos"] = torch.tensor([int(p) for p in positions], dtype=torch.int64, device=self.device)
        return x

    def alloc_decode_outputs(self):
        w = self.w
        out = {"o": torch.empty((self.B, w.heads, w.d_nope), dtype=synth.TORCH_DTYPE[w.out_dtype], device=self.device),
               "lse": torch.empty((self.B, w.heads), dtype=torch.float32, device=self.device)}
        self.aws = cb.workspace(cb.workspace_bytes(cb.OP_DENSE_ATTN_DECODE, self.adesc, self.B, 1, 0, 0), self.device)
        return out

    def decode_step(self, x, out):
        cb.compress_decode(self.kv, x["pos"], x["a"], x["za"], self.prm["Ba"])
        cb.dense_attn_decode(self.adesc, self.kv, x["pos"], x["q"], self.w.tau, out["o"], out["lse"], ws=self.aws)


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
