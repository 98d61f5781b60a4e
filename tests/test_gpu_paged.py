"""Paged, variable-length decode: compressed caches in a page pool shared by
the batch and addressed through per-sequence block tables, sequences of
mixed context lengths decoding together ("百万令牌的智慧觉醒…" §🏗️: the
serving framework's heterogeneous KV cache; "从论文出发…" 共享前缀场景的理复用:
compressed entries reused across a shared prefix).

Paging moves rows, never values, so each paged run must give the bits of the
same sequences in contiguous caches: every decode output, the indexer scores
and every visible cache entry.  Against the oracle, both legs on every
sequence: (A) the fp64 compressor from the seeded tokens, (B) the oracle's
indexer, top-k and attention over the GPU-written pages decoded exactly.
Pages are handed out in a seeded random order; mixed lengths include a
sequence with no visible entry yet and ones whose entries complete during
the steps; the dense case adds a sliding window whose first entry falls
inside a page.
"""
import dataclasses

import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import path, synth
from oracle import csa
from tests import fullsize_ref as R
from tests import gpu_cache as G
from tests.test_gpu_fullsize import csa_decode_reference, hca_reference_cache, leg_b_topk

pytestmark = pytest.mark.gpu

STEPS = 6


def layers(cls, w, lengths, page, steps, share=None, seq_ids=None):
    """(paged, contiguous) layers over the same sequences, contexts prefilled."""
    need = [(L + steps) // w.m + 1 for L in lengths]
    cap = -(-max(need) // page) * page
    table, pool = path.block_tables(need, page, cap, seed=len(lengths), share=share)
    paged = cls(w, len(lengths), cap, page_size=page, block_table=table, pool_pages=pool, seq_ids=seq_ids)
    contig = cls(w, len(lengths), cap, seq_ids=seq_ids)
    for lay in (paged, contig):
        lay.prefill_contexts(lengths)
    return paged, contig


def same_visible_entries(paged, contig, n):
    """Every cache tensor of the paged layer, gathered into sequence order,
    equals the contiguous layer's on each sequence's visible entries."""
    for cp, cc in zip(paged.caches(), contig.caches()):
        for name in ("nope", "scale", "rope"):
            tp, tc = getattr(cp, name), getattr(cc, name)
            if tp is None:
                continue
            lp = cp.logical(tp)
            for b, nb in enumerate(n):
                assert torch.equal(lp[b, :nb], tc[b, :nb]), f"{name}: sequence {b} differs"
        assert torch.equal(cp.ring, cc.ring)


CSA_CASES = {
    # FP8 keys, fp32 scores, 64-entry pages; lengths: no entry yet, ragged,
    # entries completing at different steps
    "fp8_page64": (dataclasses.replace(synth.CSA_DECODE_B32_128K, batch=5), [1, 517, 4098, 9000, 16383], 64),
    # MXFP4 keys, BF16 scores, 256-entry pages
    "mxfp4_page256": (dataclasses.replace(synth.PAIR_CSA_DECODE_B4_1M, batch=4), [6001, 2, 12289, 4095], 256),
}


@pytest.mark.parametrize("case", list(CSA_CASES))
def test_paged_csa_decode_equals_contiguous_and_oracle(case):
    w, lengths, page = CSA_CASES[case]
    B = len(lengths)
    print(f"paged csa {case}: lengths {lengths}, page {page}", flush=True)
    paged, contig = layers(path.CsaLayer, w, lengths, page, STEPS)
    op, oc = paged.alloc_decode_outputs(), contig.alloc_decode_outputs()
    xs = paged.decode_input_steps([[L + i for L in lengths] for i in range(STEPS)])
    for i, x in enumerate(xs):
        sp = torch.zeros((B, paged.cap), dtype=torch.float32, device="cuda")
        sc = torch.zeros_like(sp)
        if i % 2:  # the separate entry points (the attention turns its list into pool rows itself)
            paged.decode_step_separate(x, op, sp)
        else:
            paged.decode_step(x, op, sp)
        contig.decode_step(x, oc, sc)
        torch.cuda.synchronize()
        for k in oc:
            assert torch.equal(op[k], oc[k]), f"step {i}: {k} differs"
        assert torch.equal(sp, sc), f"step {i}: scores differ"
    pos = [L + STEPS - 1 for L in lengths]
    n = [(p + 1) // w.m for p in pos]
    same_visible_entries(paged, contig, n)
    # oracle, both legs, every sequence
    idx = op["idx"].cpu().numpy()
    o, lse = R.host(op["o"]), R.host(op["lse"])
    swaps = []
    for b in range(B):
        assert (idx[b] >= 0).sum() == min(w.topk, n[b])
        ref = csa_decode_reference(w, paged.seq_ids[b], pos[b], w.chunk, idx[b])
        G.check_attention(f"{case} seq {b} [A]", o[b], lse[b], ref["o"], ref["lse"])
        Kk = G.decode_nope(paged.keys, b, np.arange(n[b]))
        I = csa.index_scores(ref["qq"], ref["wt"], Kk, n[b], w.score_fmt)
        leg_b_topk(f"{case} seq {b}", idx[b], I, n[b], w.topk, w.score_fmt, swaps)
        ob, lb = G.attend_gpu_idx(ref["q"], pos[b], paged.kv, b, idx[b], w.d_nope, w.rope_base, w.tau)
        G.check_attention(f"{case} seq {b} [B]", o[b], lse[b], ob, lb)
    print(f"paged csa {case}: {B} sequences, tie swaps (B) {sum(swaps)}", flush=True)


def window_desc(lay, window):
    """The layer's dense-attention descriptor restricted to the last `window` entries."""
    w = lay.w
    return cb.attn_desc(w.heads, w.d_nope, w.d_rope, w.act_dtype, w.out_dtype, w.nope_fmt, w.rope_fmt, w.m, lay.cap,
                        w.rope_base, window=window, page_size=lay.kv.desc.page_size,
                        pool_pages=lay.kv.desc.pool_pages)


def test_paged_hca_decode_and_window():
    w = dataclasses.replace(synth.HCA_DECODE_B16_1M, batch=4)
    lengths = [127, 128 * 5 + 3, 128 * 71 - 1, 65536 + 9]   # 0, 5, 70 (71 after step 0), 512 entries
    steps, window = 3, 37
    print(f"paged hca: lengths {lengths}, window {window}", flush=True)
    paged, contig = layers(path.HcaLayer, w, lengths, 64, steps)
    op, oc = paged.alloc_decode_outputs(), contig.alloc_decode_outputs()
    wdesc = {lay: window_desc(lay, window) for lay in (paged, contig)}
    ow = {lay: {k: torch.empty_like(v) for k, v in op.items()} for lay in (paged, contig)}
    xs = paged.decode_input_steps([[L + i for L in lengths] for i in range(steps)])
    for i, x in enumerate(xs):
        for lay, out in ((paged, op), (contig, oc)):
            lay.decode_step(x, out)
            cb.dense_attn_decode(wdesc[lay], lay.kv, x["pos"], x["q"], w.tau, ow[lay]["o"], ow[lay]["lse"])
        torch.cuda.synchronize()
        for k in oc:
            assert torch.equal(op[k], oc[k]), f"step {i}: {k} differs"
            assert torch.equal(ow[paged][k], ow[contig][k]), f"step {i}: windowed {k} differs"
    pos = [L + steps - 1 for L in lengths]
    n = [(p + 1) // w.m for p in pos]
    same_visible_entries(paged, contig, n)
    x = xs[-1]
    for b in range(len(lengths)):
        q = R.host(x["q"][b])
        ex = hca_reference_cache(w, paged.seq_ids[b], pos[b] + 1, w.chunk) if n[b] else None
        Kb = G.decode_kv(paged.kv, b, np.arange(n[b]))
        gc = {"k": Kb, "v": Kb[:, :w.d_nope]}
        for win, out in ((0, op), (window, ow[paged])):
            for leg, cc in (("A", ex), ("B", gc)):
                if cc is None:
                    cc = gc
                oref, lref = csa.dense_attention_row(q, pos[b], cc, w.m, w.d_nope, w.rope_base, w.tau, window=win)
                G.check_attention(f"paged hca seq {b} window {win} [{leg}]", R.host(out["o"][b]),
                                  R.host(out["lse"][b]), oref, lref)


def test_paged_prefill_attention_equals_contiguous():
    # dense: the last 8192-token chunk of a 65536-token HCA context (512
    # entries in 8 pages), all visible entries and a 37-entry window
    w = dataclasses.replace(synth.HCA_DECODE_B16_1M, batch=2)
    T, chunk = 65536, 8192
    c = T // chunk - 1
    paged, contig = layers(path.HcaLayer, w, [T, T], 64, 0)
    for win in (0, 37):
        res = []
        for lay in (paged, contig):
            q = torch.stack([synth.query_chunk(w, sid, c, chunk, 0, "cuda", with_index=False)["q"]
                             for sid in lay.seq_ids]).contiguous()
            o = torch.empty((2, chunk, w.heads, w.d_nope), dtype=torch.bfloat16, device="cuda")
            lse = torch.empty((2, chunk, w.heads), dtype=torch.float32, device="cuda")
            cb.dense_attn_prefill(window_desc(lay, win), lay.kv, c * chunk, q, w.tau, o, lse)
            res.append((o, lse))
        torch.cuda.synchronize()
        assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1]), f"window {win}"
        # oracle on sampled rows of sequence 1 (GPU-written pages)
        rows = np.array([0, 1, 1000, 4095, chunk - 1])
        pos = c * chunk + rows
        Kb = G.decode_kv(paged.kv, 1, np.arange(T // w.m))
        q1 = R.host(q[1])[rows]
        for j, r in enumerate(rows):
            oref, lref = csa.dense_attention_row(q1[j], pos[j], {"k": Kb, "v": Kb[:, :w.d_nope]}, w.m, w.d_nope,
                                                 w.rope_base, w.tau, window=win)
            G.check_attention(f"paged hca prefill row {r} window {win}", R.host(res[0][0][1, r]),
                              R.host(res[0][1][1, r]), oref, lref)
    # sparse: CSA prefill lists from the contiguous indexer, attended over both caches
    wc = dataclasses.replace(synth.CSA_DECODE_B32_128K, batch=1)
    T = 2048
    paged, contig = layers(path.CsaLayer, wc, [T], 64, 0)
    qs = synth.query_chunk(wc, 0, 0, T, 0, "cuda")
    q, qI, wt = (qs[k][None].contiguous() for k in ("q", "qI", "w"))
    idx = torch.empty((1, T, wc.topk), dtype=torch.int32, device="cuda")
    cb.index_topk_prefill(contig.idesc, contig.keys, 0, qI, wt, wc.topk, idx)
    with pytest.raises(cb.CsaError):  # the prefill indexer reads contiguous keys only
        cb.index_topk_prefill(paged.idesc, paged.keys, 0, qI, wt, wc.topk, idx.clone())
    res = []
    for lay in (paged, contig):
        o = torch.empty((1, T, wc.heads, wc.d_nope), dtype=torch.bfloat16, device="cuda")
        lse = torch.empty((1, T, wc.heads), dtype=torch.float32, device="cuda")
        cb.sparse_attn_prefill(lay.adesc, lay.kv, 0, q, idx, wc.tau, o, lse)
        res.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(res[0][0], res[1][0]) and torch.equal(res[0][1], res[1][1])


def test_shared_prefix_pages():
    """Slots 0 and 1 hold the same sequence; slot 1's table names slot 0's
    pages for their common complete prefix (two pages of 64 entries), slot
    2 is another sequence.  Decoding at different positions reads the shared
    pages from both slots."""
    w = dataclasses.replace(synth.CSA_DECODE_B32_128K, batch=3)
    lengths = [700, 3001, 1500]
    paged, contig = layers(path.CsaLayer, w, lengths, 64, STEPS, share=(0, 1, 2), seq_ids=[0, 0, 1])
    assert torch.equal(paged.kv.block_table[0, :2], paged.kv.block_table[1, :2])
    op, oc = paged.alloc_decode_outputs(), contig.alloc_decode_outputs()
    xs = paged.decode_input_steps([[L + i for L in lengths] for i in range(STEPS)])
    for i, x in enumerate(xs):
        paged.decode_step(x, op)
        contig.decode_step(x, oc)
        torch.cuda.synchronize()
        for k in oc:
            assert torch.equal(op[k], oc[k]), f"step {i}: {k} differs"
    same_visible_entries(paged, contig, [(L + STEPS) // w.m for L in lengths])
