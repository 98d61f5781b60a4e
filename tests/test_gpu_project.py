"""GPU parity of the compressor fed from hidden states
(csa_compress_project_prefill: the four projections fused with the
compression) against the oracle's fp64 projections and compressor.

The GPU's projected rows carry fp32 accumulation error, so an entry value is
compared within the bound that error implies: per row the dot product's
error is at most d_model * 2^-23 * sum_k |x_k w_k|; a value row moves the
entry by its own error, a logit row by at most 2 max|dz| max|value| through
the softmax weights, and the compressor's own fp32 sum adds 2m * 2^-23
max|value|.  Stored codes must equal the oracle's except where the exact
value lies within that bound of a rounding boundary (as for the compressor).
"""
import dataclasses

import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import path, synth
from oracle import csa
from oracle import formats as F
from tests.helpers import bf16_codes_match, near_boundary, near_midpoint, np64

pytestmark = pytest.mark.gpu
DEV = "cuda"


def inputs(B, T, d, c, m, overlap, seed, prefix=""):
    X = torch.stack([synth.hidden_chunk(b, 0, T, d, seed, DEV) for b in range(B)]).contiguous()
    W = synth.projection_weights(c, d, overlap, prefix, seed, DEV)
    Ba = synth.normal((m, c), "prj.Ba" + prefix, seed, device=DEV, std=c ** -0.5)
    Bb = synth.normal((m, c), "prj.Bb" + prefix, seed, device=DEV, std=c ** -0.5) if overlap else None
    return X, W, Ba, Bb


def run(cache, X, W, Ba, Bb, pos0=0, lo=0, hi=None):
    hi = X.shape[1] if hi is None else hi
    cb.compress_project_prefill(cache, pos0, X[:, lo:hi].contiguous(), cb.pack_projection_weights(W), Ba, Bb)


def oracle(X, W, Ba, Bb, m, d_nope, b=0):
    """fp64 entries (before RoPE) of sequence b and their error bound [N, c]."""
    x = np64(X[b])
    Wn = {k: np64(v) for k, v in W.items()}
    ent = csa.compress_from_hidden(x, Wn, np64(Ba), m, None if Bb is None else np64(Bb))
    d = x.shape[1]
    N, c = ent.shape
    dY = {k: d * 2.0 ** -23 * (np.abs(x) @ np.abs(v)) for k, v in Wn.items()}
    Y = {k: x @ v for k, v in Wn.items()}
    win = lambda a: a[:N * m].reshape(N, m, c).max(1)
    dv, dz, vmax = win(dY["aKV"]), win(dY["aZ"]), win(np.abs(Y["aKV"]))
    if "bKV" in Wn:
        prev = lambda a: np.concatenate([np.zeros((1, c)), win(a)[:-1]], 0)
        dv = np.maximum(dv, prev(dY["bKV"]))
        dz = np.maximum(dz, prev(dY["bZ"]))
        vmax = np.maximum(vmax, prev(np.abs(Y["bKV"])))
    rows = 2 * m if "bKV" in Wn else m
    bound = dv + 2.0 * dz * vmax + rows * 2.0 ** -23 * vmax
    if c > d_nope:  # RoPE mixes the pairs
        r = bound[:, d_nope:].reshape(N, -1, 2).max(-1)
        bound[:, d_nope:] = np.repeat(r, 2, axis=1)
    return ent, bound, Y


@pytest.mark.parametrize("m,overlap", [(4, True), (128, False)])
def test_project_f32_values(m, overlap):
    """fp32 cache: every stored value within the bound of the oracle's."""
    B, T, d, c, d_nope = 2, 700 if m == 4 else 1100, 256, 576, 512
    X, W, Ba, Bb = inputs(B, T, d, c, m, overlap, seed=1)
    desc = cb.cache_desc(m, overlap, d_nope, 64, "bf16", "f32", "f32", T // m + 1)
    cache = cb.KVCache(desc, B)
    run(cache, X, W, Ba, Bb)
    torch.cuda.synchronize()
    N = T // m
    for b in range(B):
        ent, bound, _ = oracle(X, W, Ba, Bb, m, d_nope, b)
        exact = csa.finalize_kv(ent, 0, m, d_nope, 10000.0, "f32", "f32")["exact"]
        got = np.concatenate([np64(cache.nope[b, :N]), np64(cache.rope[b, :N])], 1)
        err = np.abs(got - exact)
        assert (err <= bound + 2.0 ** -23 * np.abs(exact)).all(), f"seq {b}: {(err / bound).max()} x the bound"
        print(f"project f32 m={m} seq {b}: max err / bound {(err / bound).max():.3f}", flush=True)


@pytest.mark.parametrize("m,overlap", [(4, True), (128, False)])
def test_project_fp8_codes(m, overlap):
    """FP8 codes + per-entry scale, BF16 RoPE dims, against the oracle."""
    B, T, d, c, d_nope = 1, 1536 + 20 if m == 4 else 2048 + 64, 512, 576, 512
    X, W, Ba, Bb = inputs(B, T, d, c, m, overlap, seed=2)
    desc = cb.cache_desc(m, overlap, d_nope, 64, "bf16", "fp8", "bf16", T // m + 1)
    cache = cb.KVCache(desc, B)
    run(cache, X, W, Ba, Bb)
    torch.cuda.synchronize()
    N = T // m
    ent, bound, _ = oracle(X, W, Ba, Bb, m, d_nope)
    fin = csa.finalize_kv(ent, 0, m, d_nope, 10000.0, "fp8", "bf16")
    exact = fin["exact"]
    s_gpu = cache.scale[0, :N].cpu().double().numpy()
    # the scale follows the entry's amax, itself within the bound
    ds = bound[:, :d_nope].max(1) / 448.0
    assert (np.abs(s_gpu - fin["scale"]) <= ds + 1e-6 * fin["scale"]).all()
    y = exact[:, :d_nope] / s_gpu[:, None]
    dy = bound[:, :d_nope] / s_gpu[:, None] + 2e-6 * np.abs(y)
    codes = cache.nope[0, :N].cpu().numpy()
    same = F.fp8_decode(codes) == F.fp8_round(y)
    assert (same | near_boundary(y, F.fp8_round, dy)).all()
    assert (~same).sum() <= 2e-3 * same.size
    ok, _ = bf16_codes_match(np64(cache.rope[0, :N]), exact[:, d_nope:], bound[:, d_nope:])
    assert ok.all()
    print(f"project fp8 m={m}: {N} entries, {(~same).sum()} codes at a boundary", flush=True)


def test_project_mxfp4_keys():
    """The indexer-key instance (64 dims, no RoPE) stored as MXFP4."""
    B, T, d, c, m = 1, 2048 + 8, 256, 64, 4
    X, W, Ba, Bb = inputs(B, T, d, c, m, True, seed=3, prefix="k")
    desc = cb.cache_desc(m, True, c, 0, "bf16", "mxfp4", "f32", T // m)
    cache = cb.KVCache(desc, B)
    run(cache, X, W, Ba, Bb)
    torch.cuda.synchronize()
    N = T // m
    ent, bound, _ = oracle(X, W, Ba, Bb, m, c)
    g_sc = cache.scale[0, :N].cpu().numpy()
    amax = np.abs(ent).reshape(N, 2, 32).max(-1)
    _, _, sc = F.mxfp4_quantize(ent)
    bmax = bound.reshape(N, 2, 32).max(-1)
    sc_ok = (g_sc == sc) | (np.floor(np.log2(amax - bmax)) != np.floor(np.log2(amax + bmax)))
    assert sc_ok.all()
    packed = cache.nope[0, :N].cpu().numpy().astype(np.int64)
    g_codes = np.stack([packed & 15, packed >> 4], -1).reshape(N, c)
    Xs = np.ldexp(1.0, g_sc.astype(np.int64) - 127).repeat(32, axis=1)
    y = ent / Xs
    same = F.e2m1_decode(g_codes) == F.e2m1_round(y)
    assert (same | near_boundary(y, F.e2m1_round, bound / Xs)).all()


def test_project_chunked_equals_single_call_and_ring():
    """Calls over consecutive token ranges (pos0 multiples of m; the ring
    carries the previous window) give the bits of one call; the ring then
    holds the projected rows of the last 2m tokens."""
    B, T, d, c, m = 2, 1000, 256, 576, 4
    X, W, Ba, Bb = inputs(B, T, d, c, m, True, seed=4)
    desc = cb.cache_desc(m, True, 512, 64, "bf16", "fp8", "bf16", T // m)
    one, parts = cb.KVCache(desc, B), cb.KVCache(desc, B)
    run(one, X, W, Ba, Bb)
    for lo, hi in ((0, 4), (4, 132), (132, 136), (136, 640), (640, 998), (996, T)):
        run(parts, X, W, Ba, Bb, pos0=lo, lo=lo, hi=hi)   # the last call repeats a partial window
    torch.cuda.synchronize()
    assert torch.equal(one.nope, parts.nope) and torch.equal(one.rope, parts.rope)
    assert torch.equal(one.scale, parts.scale) and torch.equal(one.ring, parts.ring)
    # ring: slot t mod 2m holds token t's rows a, za, b, zb
    _, _, Y = oracle(X, W, Ba, Bb, m, 512, b=1)
    x = np64(X[1])
    ring = np64(one.ring[1])                            # [2m][4][c]
    for t in range(T - 2 * m, T):
        for u, nm in enumerate(("aKV", "aZ", "bKV", "bZ")):
            dY = d * 2.0 ** -23 * (np.abs(x[t]) @ np.abs(np64(W[nm])))
            assert (np.abs(ring[t % (2 * m), u] - Y[nm][t]) <= dY).all(), (t, nm)


def test_project_paged_equals_contiguous():
    B, T, d, c, m, page = 3, 900, 256, 576, 4, 64
    X, W, Ba, Bb = inputs(B, T, d, c, m, True, seed=5)
    cap = -(-(T // m) // page) * page
    table, pool = path.block_tables([T // m] * B, page, cap, seed=2)
    flat = cb.KVCache(cb.cache_desc(m, True, 512, 64, "bf16", "fp8", "bf16", cap), B)
    paged = cb.KVCache(cb.cache_desc(m, True, 512, 64, "bf16", "fp8", "bf16", cap, page_size=page, pool_pages=pool),
                       B, block_table=table)
    run(flat, X, W, Ba, Bb)
    run(paged, X, W, Ba, Bb)
    torch.cuda.synchronize()
    N = T // m
    for name in ("nope", "scale", "rope"):
        assert torch.equal(paged.logical(getattr(paged, name))[:, :N], getattr(flat, name)[:, :N]), name
