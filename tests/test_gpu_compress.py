"""GPU parity of the compressor (csa_compress_prefill / csa_compress_decode)
against the CPU oracle, through the C ABI."""
import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import synth
from oracle import csa
from oracle import formats as F
from tests.helpers import (bf16_codes_match, compressor_error_bound, max_rel_rows, near_boundary,
                           near_midpoint, np64)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def make_inputs(T, c, m, overlap, dt, seed, B=1):
    dtype = synth.TORCH_DTYPE[dt]
    x = {nm: synth.normal((B, T, c), "cmp." + nm, seed, device=DEV, dtype=dtype)
         for nm in (["a", "za", "b", "zb"] if overlap else ["a", "za"])}
    x["Ba"] = synth.normal((m, c), "cmp.Ba", seed, device=DEV, std=c ** -0.5)
    if overlap:
        x["Bb"] = synth.normal((m, c), "cmp.Bb", seed, device=DEV, std=c ** -0.5)
    return x


def run_prefill(cache, x, pos0, lo, hi):
    sl = lambda t: None if t is None else t[:, lo:hi].contiguous()
    cb.compress_prefill(cache, pos0, sl(x["a"]), sl(x["za"]), x["Ba"], sl(x.get("b")), sl(x.get("zb")),
                        x.get("Bb"))


def err_bound(x, m, overlap, d_nope, seq=0):
    return compressor_error_bound({nm: np64(x[nm][seq]) for nm in ("a", "b") if nm in x}, m, overlap, d_nope)


def oracle_entries(x, m, overlap, seq=0):
    g = lambda nm: np64(x[nm][seq]) if nm in x else None
    return csa.compress(g("a"), g("za"), np64(x["Ba"]), m, g("b"), g("zb"),
                        np64(x["Bb"]) if overlap else None)


def test_compress_fp32_tiny_workload():
    """fp32 compressor of the tiny workload (m = 4, overlapped, 32 + 32 dims,
    and the 32-dim indexer-key instance) within 1e-5 per entry."""
    w = synth.TINY_CSA_PREFILL_FP32
    pr = synth.tiny_projections(w)
    T = w.tokens
    N = T // w.m
    for names, c, d_nope, d_rope in ((("a", "za", "b", "zb", "Ba", "Bb"), w.c, w.d_nope, w.d_rope),
                                      (("ka", "kza", "kb", "kzb", "kBa", "kBb"), w.idx_dim, w.idx_dim, 0)):
        desc = cb.cache_desc(w.m, True, d_nope, d_rope, "f32", "f32", "f32", N)
        cache = cb.KVCache(desc, 1)
        x = {k: pr[n][None].to(DEV) for k, n in zip(("a", "za", "b", "zb"), names[:4])}
        x["Ba"], x["Bb"] = pr[names[4]].to(DEV), pr[names[5]].to(DEV)
        run_prefill(cache, x, 0, 0, T)
        torch.cuda.synchronize()
        ent = oracle_entries(x, w.m, True)
        ref = csa.finalize_kv(ent, 0, w.m, d_nope, w.rope_base, "f32", "f32")["exact"]
        got = np64(cache.nope[0])
        if d_rope:
            got = np.concatenate([got, np64(cache.rope[0])], 1)
        assert max_rel_rows(got, ref) < 1e-5


@pytest.mark.parametrize("m,overlap", [(4, True), (1, False), (128, False)])
def test_compress_bf16_codes(m, overlap):
    T, c, d_nope = 2048 + 37, 576, 512
    x = make_inputs(T, c, m, overlap, "bf16", seed=11)
    N = T // m
    desc = cb.cache_desc(m, overlap, d_nope, 64, "bf16", "bf16", "bf16", N)
    cache = cb.KVCache(desc, 1)
    run_prefill(cache, x, 0, 0, T)
    torch.cuda.synchronize()
    exact = csa.finalize_kv(oracle_entries(x, m, overlap), 0, m, d_nope, 10000.0, "bf16", "bf16")["exact"]
    got = np.concatenate([np64(cache.nope[0]), np64(cache.rope[0])], 1)
    ok, nmis = bf16_codes_match(got, exact, err_bound(x, m, overlap, d_nope))
    assert ok.all(), f"{(~ok).sum()} BF16 codes differ away from a midpoint"
    assert nmis <= 1e-3 * got.size


@pytest.mark.parametrize("m,overlap", [(4, True), (128, False)])
def test_compress_fp8_split_cache(m, overlap):
    """FP8 codes with a per-entry fp32 scale (amax / 448) + BF16 RoPE dims."""
    T, c, d_nope = 4096 + 5, 576, 512
    x = make_inputs(T, c, m, overlap, "bf16", seed=12)
    N = T // m
    desc = cb.cache_desc(m, overlap, d_nope, 64, "bf16", "fp8", "bf16", N)
    cache = cb.KVCache(desc, 1)
    run_prefill(cache, x, 0, 0, T)
    torch.cuda.synchronize()
    fin = csa.finalize_kv(oracle_entries(x, m, overlap), 0, m, d_nope, 10000.0, "fp8", "bf16")
    exact = fin["exact"]
    s_gpu = cache.scale[0].cpu().double().numpy()
    assert np.allclose(s_gpu, fin["scale"], rtol=1e-6, atol=0)
    y = exact[:, :d_nope] / fin["scale"][:, None]
    bound = err_bound(x, m, overlap, d_nope)
    # the GPU divides its own fp32 value by its own fp32 scale (within 1e-6)
    dy = bound[:, :d_nope] / fin["scale"][:, None] + 2e-6 * np.abs(y)
    gpu_codes = cache.nope[0].cpu().numpy()
    same = F.fp8_decode(gpu_codes) == F.fp8_round(y)
    assert (same | near_boundary(y, F.fp8_round, dy)).all()
    assert (~same).sum() <= 1e-3 * same.size
    ok, _ = bf16_codes_match(np64(cache.rope[0]), exact[:, d_nope:], bound[:, d_nope:])
    assert ok.all()


def test_compress_mxfp4_keys():
    T, d, m = 4096 + 3, 64, 4
    x = make_inputs(T, d, m, True, "bf16", seed=13)
    N = T // m
    desc = cb.cache_desc(m, True, d, 0, "bf16", "mxfp4", "f32", N)
    cache = cb.KVCache(desc, 1)
    run_prefill(cache, x, 0, 0, T)
    torch.cuda.synchronize()
    exact = oracle_entries(x, m, True)
    _, codes, sc = F.mxfp4_quantize(exact)
    g_sc = cache.scale[0].cpu().numpy()
    amax = np.abs(exact).reshape(N, 2, 32).max(-1)
    sc_ok = (g_sc == sc) | near_midpoint(amax, lambda v: np.floor(np.log2(v)), 1e-6)
    assert sc_ok.all()
    packed = cache.nope[0].cpu().numpy().astype(np.int64)
    g_codes = np.stack([packed & 15, packed >> 4], -1).reshape(N, d)
    X = np.ldexp(1.0, g_sc.astype(np.int64) - 127).repeat(32, axis=1)
    y = exact / X
    dy = err_bound(x, m, True, d) / X
    same = F.e2m1_decode(g_codes) == F.e2m1_round(y)
    assert (same | near_boundary(y, F.e2m1_round, dy)).all()


@pytest.mark.parametrize("m,overlap,fmt", [(4, True, "fp8"), (128, False, "fp8"), (4, True, "f32")])
def test_chunked_prefill_equals_single_call(m, overlap, fmt):
    """Prefill split at arbitrary token boundaries (the ring carries the
    previous tokens) writes bitwise the same cache as one call."""
    T, c = 1000, 576
    dt = "f32" if fmt == "f32" else "bf16"
    x = make_inputs(T, c, m, overlap, dt, seed=14, B=2)
    desc = cb.cache_desc(m, overlap, 512, 64, dt, fmt, dt, T // m)
    one, parts = cb.KVCache(desc, 2), cb.KVCache(desc, 2)
    run_prefill(one, x, 0, 0, T)
    for lo, hi in ((0, 3), (3, 130), (130, 131), (131, 600), (600, T)):
        run_prefill(parts, x, lo, lo, hi)
    torch.cuda.synchronize()
    assert torch.equal(one.nope, parts.nope) and torch.equal(one.rope, parts.rope)
    if one.scale is not None:
        assert torch.equal(one.scale, parts.scale)


@pytest.mark.parametrize("m,overlap", [(4, True), (128, False)])
def test_decode_equals_prefill(m, overlap):
    """Token-by-token decode after a prefill equals one prefill over all
    tokens (bitwise), and matches the oracle."""
    T0, T1, c, B = 3 * m + 1, 3 * m + 2 * m + 3, 576, 3
    x = make_inputs(T1, c, m, overlap, "bf16", seed=15, B=B)
    desc = cb.cache_desc(m, overlap, 512, 64, "bf16", "fp8", "bf16", T1 // m + 2)
    full, dec = cb.KVCache(desc, B), cb.KVCache(desc, B)
    run_prefill(full, x, 0, 0, T1)
    run_prefill(dec, x, 0, 0, T0)
    for t in range(T0, T1):
        pos = torch.full((B,), t, dtype=torch.int64, device=DEV)
        tok = lambda nm: None if nm not in x else x[nm][:, t].contiguous()
        cb.compress_decode(dec, pos, tok("a"), tok("za"), x["Ba"], tok("b"), tok("zb"), x.get("Bb"))
    torch.cuda.synchronize()
    N = T1 // m
    assert torch.equal(full.nope[:, :N], dec.nope[:, :N])
    assert torch.equal(full.scale[:, :N], dec.scale[:, :N])
    assert torch.equal(full.rope[:, :N], dec.rope[:, :N])
    fin = csa.finalize_kv(oracle_entries(x, m, overlap, seq=2), 0, m, 512, 10000.0, "fp8", "bf16")
    assert np.allclose(dec.scale[2, :N].cpu().double().numpy(), fin["scale"], rtol=1e-6)
