"""GPU parity of CSA sparse attention and HCA dense attention (prefill and
decode) against the CPU oracle, through the C ABI.  Caches and index lists
are filled directly with seeded synthetic values."""
import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import synth
from oracle import csa
from oracle import formats as F
from tests.helpers import lse_err, max_rel_rows, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def kv_cache(nope_fmt, rope_fmt, B, cap, d_nope, d_rope, m, seed):
    desc = cb.cache_desc(m, True, d_nope, d_rope, "f32", nope_fmt, rope_fmt, cap)
    kv = cb.KVCache(desc, B)
    if nope_fmt == "fp8":
        kv.nope.copy_(synth.random_fp8_codes((B, cap, d_nope), "kv", seed, device=DEV))
        kv.scale.copy_(synth.normal((B, cap), "kvscale", seed, device=DEV).abs() * 0.01 + 2e-3)
        V = F.fp8_decode(kv.nope.cpu().numpy()) * kv.scale.cpu().double().numpy()[..., None]
    else:
        kv.nope.copy_(synth.normal((B, cap, d_nope), "kv", seed, device=DEV, dtype=synth.TORCH_DTYPE[nope_fmt]))
        V = np64(kv.nope)
    if d_rope:
        kv.rope.copy_(synth.normal((B, cap, d_rope), "kvrope", seed, device=DEV, dtype=synth.TORCH_DTYPE[rope_fmt]))
        K = np.concatenate([V, np64(kv.rope)], -1)
    else:
        K = V
    return kv, {"k": K, "v": V}


def check(o_gpu, lse_gpu, o_ref, lse_ref, tol, lse_tol):
    assert max_rel_rows(np64(o_gpu).reshape(-1, o_ref.shape[-1]), o_ref.reshape(-1, o_ref.shape[-1])) <= tol
    inf_ok, err = lse_err(np64(lse_gpu).ravel(), lse_ref.ravel())
    assert inf_ok and err <= lse_tol


def test_sparse_prefill_fp32_tiny_workload_shapes():
    T, H, dn, dr, m, k = 2048, 8, 32, 32, 4, 64
    cap = T // m
    kv, cache = kv_cache("f32", "f32", 1, cap, dn, dr, m, seed=31)
    n_vis = [(t + 1) // m for t in range(T)]
    idx = synth.random_sorted_subsets(T, n_vis, k, "idx", 31, device=DEV)[None]
    q = synth.normal((1, T, H, dn + dr), "q", 31, device=DEV)
    o = torch.empty((1, T, H, dn), dtype=torch.float32, device=DEV)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
    desc = cb.attn_desc(H, dn, dr, "f32", "f32", "f32", "f32", m, cap)
    cb.sparse_attn_prefill(desc, kv, 0, q, idx, 0.125, o, lse)
    torch.cuda.synchronize()
    qn, ix = np64(q[0]), idx[0].cpu().numpy()
    ref = [csa.sparse_attention_row(qn[t], t, {"k": cache["k"][0], "v": cache["v"][0]}, ix[t], dn, 1e4, 0.125)
           for t in range(T)]
    check(o, lse, np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), 1e-5, 1e-5)


@pytest.mark.parametrize("nope_fmt", ["bf16", "fp8"])
def test_sparse_prefill_64_heads(nope_fmt):
    """64 heads, 512 + 64 dims, queries at positions 8192.., k = 1024 with
    padding and out-of-range indices that must be skipped."""
    T, H, dn, dr, m, k, pos0 = 192, 64, 512, 64, 4, 1024, 8192
    cap = (pos0 + T) // m + 8
    kv, cache = kv_cache(nope_fmt, "bf16", 1, cap, dn, dr, m, seed=32)
    n_vis = [(pos0 + t + 1) // m for t in range(T)]
    sub = [n - 40 if t % 3 == 0 else n for t, n in enumerate(n_vis)]  # some rows padded with -1
    idx = synth.random_sorted_subsets(T, sub, k, "idx", 32)
    idx[5, -1] = cap - 1          # beyond n(t): skipped
    idx = idx[None].to(DEV)
    q = synth.normal((1, T, H, dn + dr), "q", 32, device=DEV, dtype=torch.bfloat16)
    o = torch.empty((1, T, H, dn), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
    desc = cb.attn_desc(H, dn, dr, "bf16", "bf16", nope_fmt, "bf16", m, cap)
    tau = 1 / 24.0
    cb.sparse_attn_prefill(desc, kv, pos0, q, idx, tau, o, lse)
    torch.cuda.synchronize()
    qn, ix = np64(q[0]), idx[0].cpu().numpy()
    c0 = {"k": cache["k"][0], "v": cache["v"][0]}
    ref = [csa.sparse_attention_row(qn[t], pos0 + t, c0, ix[t][ix[t] < n_vis[t]], dn, 1e4, tau) for t in range(T)]
    check(o, lse, np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), 1e-2, 1e-2)


def test_sparse_decode_fp8_split_cache():
    B, H, dn, dr, m, k, cap = 3, 64, 512, 64, 4, 1024, 4096
    kv, cache = kv_cache("fp8", "bf16", B, cap, dn, dr, m, seed=33)
    positions = [4 * cap - 1, 5000, 1500]
    n_vis = [(p + 1) // m for p in positions]
    idx = synth.random_sorted_subsets(B, n_vis, k, "idx", 33).to(DEV)
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    q = synth.normal((B, H, dn + dr), "q", 33, device=DEV, dtype=torch.bfloat16)
    o = torch.empty((B, H, dn), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    desc = cb.attn_desc(H, dn, dr, "bf16", "bf16", "fp8", "bf16", m, cap)
    tau = 576 ** -0.5
    cb.sparse_attn_decode(desc, kv, pos, q, idx, tau, o, lse)
    torch.cuda.synchronize()
    qn, ix = np64(q), idx.cpu().numpy()
    ref = [csa.sparse_attention_row(qn[b], positions[b], {"k": cache["k"][b], "v": cache["v"][b]}, ix[b], dn, 1e4, tau)
           for b in range(B)]
    check(o, lse, np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), 1e-2, 1e-2)


@pytest.mark.parametrize("pos0,T", [(0, 300), (128 * 500 - 37, 300)])
def test_dense_prefill_hca(pos0, T):
    """HCA dense attention over m' = 128 entries, FP8 + BF16 cache; the first
    rows of a sequence see no entry (o = 0, lse = -inf)."""
    H, dn, dr, m = 64, 512, 64, 128
    cap = (pos0 + T) // m + 2
    kv, cache = kv_cache("fp8", "bf16", 1, cap, dn, dr, m, seed=34)
    q = synth.normal((1, T, H, dn + dr), "q", 34, device=DEV, dtype=torch.bfloat16)
    o = torch.empty((1, T, H, dn), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
    desc = cb.attn_desc(H, dn, dr, "bf16", "bf16", "fp8", "bf16", m, cap)
    tau = 576 ** -0.5
    cb.dense_attn_prefill(desc, kv, pos0, q, tau, o, lse)
    torch.cuda.synchronize()
    qn = np64(q[0])
    oref, lref = csa.hca_rows(pos0 + np.arange(T), qn, {"k": cache["k"][0], "v": cache["v"][0]}, m, dn, 1e4, tau)
    check(o, lse, oref, lref, 1e-2, 1e-2)


def test_dense_decode_hca():
    B, H, dn, dr, m, cap = 4, 64, 512, 64, 128, 1024
    kv, cache = kv_cache("fp8", "bf16", B, cap, dn, dr, m, seed=35)
    positions = [128 * cap - 1, 128 * 700 + 5, 127, 100]
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    q = synth.normal((B, H, dn + dr), "q", 35, device=DEV, dtype=torch.bfloat16)
    o = torch.empty((B, H, dn), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
    desc = cb.attn_desc(H, dn, dr, "bf16", "bf16", "fp8", "bf16", m, cap)
    tau = 576 ** -0.5
    cb.dense_attn_decode(desc, kv, pos, q, tau, o, lse)
    torch.cuda.synchronize()
    qn = np64(q)
    ref = [csa.dense_attention_row(qn[b], positions[b], {"k": cache["k"][b], "v": cache["v"][b]}, m, dn, 1e4, tau)
           for b in range(B)]
    check(o, lse, np.stack([r[0] for r in ref]), np.stack([r[1] for r in ref]), 1e-2, 1e-2)
