"""The sliding-window branch: dense attention over the last `window`
per-token entries (m = 1) on the GPU against the oracle, prefill and decode,
MFMA (64 heads, 512 + 64 dims, FP8 / BF16 caches) and generic (fp32) paths;
the log-sum-exp merge against the oracle's formula; and a whole tiny CSA
layer with its window branch against one oracle softmax over the union of
the selected entries and the window's tokens."""
import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import synth
from oracle import csa
from tests.helpers import compare_topk, lse_err, max_rel_rows, np64
from tests.test_gpu_attn import check, kv_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"


@pytest.mark.parametrize("nope_fmt", ["bf16", "fp8"])
def test_window_prefill_mfma(nope_fmt):
    """Queries at positions pos0.. over per-token entries, window 128: rows
    near the start see fewer than 128 tokens."""
    T, H, dn, dr, w = 300, 64, 512, 64, 128
    for pos0 in (0, 5000):
        cap = pos0 + T + 4
        kv, cache = kv_cache(nope_fmt, "bf16", 1, cap, dn, dr, 1, seed=40)
        q = synth.normal((1, T, H, dn + dr), "swa.q", 40, device=DEV, dtype=torch.bfloat16)
        o = torch.empty((1, T, H, dn), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
        desc = cb.attn_desc(H, dn, dr, "bf16", "bf16", nope_fmt, "bf16", 1, cap, window=w)
        tau = 576 ** -0.5
        cb.dense_attn_prefill(desc, kv, pos0, q, tau, o, lse)
        torch.cuda.synchronize()
        qn = np64(q[0])
        c0 = {"k": cache["k"][0], "v": cache["v"][0]}
        ref = [csa.dense_attention_row(qn[t], pos0 + t, c0, 1, dn, 1e4, tau, window=w) for t in range(T)]
        check(o, lse, np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), 1e-2, 1e-2)


def test_window_decode_mfma():
    B, H, dn, dr, cap = 5, 64, 512, 64, 20000
    kv, cache = kv_cache("fp8", "bf16", B, cap, dn, dr, 1, seed=41)
    positions = [cap - 1, 9000, 200, 127, 3]
    for w in (128, 1000):
        pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
        q = synth.normal((B, H, dn + dr), "swa.qd", 41, device=DEV, dtype=torch.bfloat16)
        o = torch.empty((B, H, dn), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
        desc = cb.attn_desc(H, dn, dr, "bf16", "bf16", "fp8", "bf16", 1, cap, window=w)
        tau = 576 ** -0.5
        cb.dense_attn_decode(desc, kv, pos, q, tau, o, lse)
        torch.cuda.synchronize()
        qn = np64(q)
        ref = [csa.dense_attention_row(qn[b], positions[b], {"k": cache["k"][b], "v": cache["v"][b]}, 1, dn, 1e4, tau,
                                       window=w) for b in range(B)]
        check(o, lse, np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), 1e-2, 1e-2)


def test_window_generic_fp32():
    T, H, dn, dr, w, cap = 200, 8, 32, 32, 16, 256
    kv, cache = kv_cache("f32", "f32", 1, cap, dn, dr, 1, seed=42)
    q = synth.normal((1, T, H, dn + dr), "swa.qg", 42, device=DEV)
    o = torch.empty((1, T, H, dn), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
    desc = cb.attn_desc(H, dn, dr, "f32", "f32", "f32", "f32", 1, cap, window=w)
    cb.dense_attn_prefill(desc, kv, 0, q, 0.125, o, lse)
    torch.cuda.synchronize()
    qn = np64(q[0])
    c0 = {"k": cache["k"][0], "v": cache["v"][0]}
    ref = [csa.dense_attention_row(qn[t], t, c0, 1, dn, 1e4, 0.125, window=w) for t in range(T)]
    check(o, lse, np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), 1e-5, 1e-5)


@pytest.mark.parametrize("dtype", [torch.float32, torch.bfloat16])
def test_lse_merge_matches_formula(dtype):
    R, H, dv = 37, 64, 512
    o1 = synth.normal((R, H, dv), "mg.o1", 43, device=DEV, dtype=dtype)
    o2 = synth.normal((R, H, dv), "mg.o2", 43, device=DEV, dtype=dtype)
    l1 = synth.normal((R, H), "mg.l1", 43, device=DEV) * 3
    l2 = synth.normal((R, H), "mg.l2", 43, device=DEV) * 3
    l1[0] = -float("inf")              # compressed branch empty (no entry visible yet)
    l1[1], l2[1] = -float("inf"), -float("inf")
    l2[2] = -float("inf")
    o = torch.empty_like(o1)
    lse = torch.empty_like(l1)
    cb.lse_merge(o1, l1, o2, l2, o, lse)
    torch.cuda.synchronize()
    oref, lref = csa.lse_merge(np64(o1), np64(l1), np64(o2), np64(l2))
    tol = 1e-6 if dtype == torch.float32 else 1e-2
    assert max_rel_rows(np64(o).reshape(-1, dv), oref.reshape(-1, dv)) <= tol
    inf_ok, err = lse_err(np64(lse), lref)
    assert inf_ok and err <= 1e-5
    assert not np64(o)[1].any()
    cb.lse_merge(o1, l1, o2, l2, o1)   # in place
    torch.cuda.synchronize()
    assert torch.equal(o1, o)


def test_tiny_csa_layer_with_window_branch():
    """Tiny fp32 workload: the CSA branch (compress, indexer + top-k, sparse
    attention) and the window branch (per-token entries from the compressor
    with m = 1, window 16) merged; against the oracle's single softmax over
    the selected compressed entries and the window's tokens."""
    w = synth.TINY_CSA_PREFILL_FP32
    pr = {k: v.to(DEV) for k, v in synth.tiny_projections(w).items()}
    T, m, k, win = w.tokens, w.m, w.topk, 16
    N = T // m
    u = lambda t: t[None].contiguous()
    kv = cb.KVCache(cb.cache_desc(m, True, w.d_nope, w.d_rope, "f32", "f32", "f32", N), 1)
    keys = cb.KVCache(cb.cache_desc(m, True, w.idx_dim, 0, "f32", "f32", "f32", N), 1)
    tok = cb.KVCache(cb.cache_desc(1, False, w.d_nope, w.d_rope, "f32", "f32", "f32", T), 1)
    cb.compress_prefill(kv, 0, u(pr["a"]), u(pr["za"]), pr["Ba"], u(pr["b"]), u(pr["zb"]), pr["Bb"])
    cb.compress_prefill(keys, 0, u(pr["ka"]), u(pr["kza"]), pr["kBa"], u(pr["kb"]), u(pr["kzb"]), pr["kBb"])
    cb.compress_prefill(tok, 0, u(pr["a"]), u(pr["za"]), pr["Ba"][:1].contiguous())
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    cb.index_topk_prefill(cb.index_desc(w.idx_heads, w.idx_dim, "f32", "f32", "f32", "f32", m, N), keys, 0,
                          u(pr["qI"]), u(pr["w"]), k, idx)
    shape = (1, T, w.heads, w.d_nope)
    o1, o2 = torch.empty(shape, device=DEV), torch.empty(shape, device=DEV)
    l1, l2 = torch.empty(shape[:3], device=DEV), torch.empty(shape[:3], device=DEV)
    cb.sparse_attn_prefill(cb.attn_desc(w.heads, w.d_nope, w.d_rope, "f32", "f32", "f32", "f32", m, N), kv, 0,
                           u(pr["q"]), idx, w.tau, o1, l1)
    cb.dense_attn_prefill(cb.attn_desc(w.heads, w.d_nope, w.d_rope, "f32", "f32", "f32", "f32", 1, T, window=win),
                          tok, 0, u(pr["q"]), w.tau, o2, l2)
    o, lse = torch.empty_like(o1), torch.empty_like(l1)
    cb.lse_merge(o1, l1, o2, l2, o, lse)
    torch.cuda.synchronize()
    x = {kk: np64(v) for kk, v in pr.items()}
    cache = csa.finalize_kv(csa.compress(x["a"], x["za"], x["Ba"], m, x["b"], x["zb"], x["Bb"]), 0, m, w.d_nope,
                            w.rope_base, "f32", "f32")
    kk_ = csa.finalize_keys(csa.compress(x["ka"], x["kza"], x["kBa"], m, x["kb"], x["kzb"], x["kBb"]), "f32")
    tcache = csa.finalize_kv(csa.compress(x["a"], x["za"], x["Ba"][:1], 1), 0, 1, w.d_nope, w.rope_base, "f32", "f32")
    rows = np.arange(T)
    ref = csa.csa_rows(rows, rows, x["q"], x["qI"], x["w"], cache, kk_, m, k, w.d_nope, w.rope_base, w.tau)
    gi = idx[0].cpu().numpy()
    _, bad = compare_topk(gi, ref["idx"], ref["scores"], 1e-6)
    assert not bad
    ou, lu = np.zeros((T, w.heads, w.d_nope)), np.zeros((T, w.heads))
    for t in rows:   # one softmax over the GPU's selected entries and the window's tokens
        sel = gi[t][gi[t] >= 0]
        lo = max(0, t + 1 - win)
        Ku = np.concatenate([cache["k"][sel], tcache["k"][lo:t + 1]], 0)
        ou[t], lu[t] = csa.attend(csa.rope_query(x["q"][t], t, w.d_nope, w.rope_base), Ku, Ku[:, :w.d_nope],
                                  np.arange(len(Ku)), w.tau)
    assert max_rel_rows(np64(o[0]).reshape(-1, w.d_nope), ou.reshape(-1, w.d_nope)) <= 1e-5
    inf_ok, err = lse_err(np64(lse[0]), lu)
    assert inf_ok and err <= 1e-5
