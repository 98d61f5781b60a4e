"""The tiny fp32 CSA prefill workload end to end on the GPU (compress KV and
indexer keys -> indexer + top-k -> sparse attention) against the oracle's
whole path from the same projected inputs: top-k sets equal except at score
ties closer than 1e-6 (relative to max(1, max|I|)); outputs within max-rel
1e-5 on every row, against the oracle's attention over the GPU's index list
where the two sets differ."""
import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import synth
from oracle import csa
from tests.helpers import compare_topk, lse_err, max_rel_rows, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def test_tiny_csa_prefill_end_to_end():
    w = synth.TINY_CSA_PREFILL_FP32
    pr = {k: v.to(DEV) for k, v in synth.tiny_projections(w).items()}
    T, m, k = w.tokens, w.m, w.topk
    N = T // m
    kv = cb.KVCache(cb.cache_desc(m, True, w.d_nope, w.d_rope, "f32", "f32", "f32", N), 1)
    keys = cb.KVCache(cb.cache_desc(m, True, w.idx_dim, 0, "f32", "f32", "f32", N), 1)
    u = lambda t: t[None].contiguous()
    cb.compress_prefill(kv, 0, u(pr["a"]), u(pr["za"]), pr["Ba"], u(pr["b"]), u(pr["zb"]), pr["Bb"])
    cb.compress_prefill(keys, 0, u(pr["ka"]), u(pr["kza"]), pr["kBa"], u(pr["kb"]), u(pr["kzb"]), pr["kBb"])
    idesc = cb.index_desc(w.idx_heads, w.idx_dim, "f32", "f32", "f32", "f32", m, N)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    cb.index_topk_prefill(idesc, keys, 0, u(pr["qI"]), u(pr["w"]), k, idx)
    adesc = cb.attn_desc(w.heads, w.d_nope, w.d_rope, "f32", "f32", "f32", "f32", m, N)
    o = torch.empty((1, T, w.heads, w.d_nope), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, T, w.heads), dtype=torch.float32, device=DEV)
    cb.sparse_attn_prefill(adesc, kv, 0, u(pr["q"]), idx, w.tau, o, lse)
    torch.cuda.synchronize()

    x = {kk: np64(v) for kk, v in pr.items()}
    cache = csa.finalize_kv(csa.compress(x["a"], x["za"], x["Ba"], m, x["b"], x["zb"], x["Bb"]),
                            0, m, w.d_nope, w.rope_base, "f32", "f32")
    kk = csa.finalize_keys(csa.compress(x["ka"], x["kza"], x["kBa"], m, x["kb"], x["kzb"], x["kBb"]), "f32")
    rows = np.arange(T)
    ref = csa.csa_rows(rows, rows, x["q"], x["qI"], x["w"], cache, kk, m, k, w.d_nope, w.rope_base, w.tau)
    got_idx = idx[0].cpu().numpy()
    differing, bad = compare_topk(got_idx, ref["idx"], ref["scores"], 1e-6)
    assert not bad, f"rows {bad[:5]}"
    same = np.array([set(got_idx[t][got_idx[t] >= 0]) == set(ref["idx"][t][ref["idx"][t] >= 0]) for t in rows])
    assert same.mean() > 0.99
    o_ref, l_ref = ref["o"].copy(), ref["lse"].copy()
    for t in np.nonzero(~same)[0]:
        o_ref[t], l_ref[t] = csa.sparse_attention_row(x["q"][t], int(t), cache, got_idx[t], w.d_nope, w.rope_base,
                                                      w.tau)
    og, lg = np64(o[0]), np64(lse[0])
    assert max_rel_rows(og.reshape(-1, w.d_nope), o_ref.reshape(-1, w.d_nope)) <= 1e-5
    inf_ok, err = lse_err(lg, l_ref)
    assert inf_ok and err <= 1e-5
