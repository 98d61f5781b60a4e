"""The allocation-free sparse decode entry point (split partials in the
library's own device scratch) gives bit for bit the outputs of
csa_sparse_attn_decode with a caller workspace, on two calls in a row, the
second with a smaller batch; sizes past the scratch are rejected."""
import ctypes

import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import synth

pytestmark = pytest.mark.gpu
DEV = "cuda"
H, DN, DR, M, K = 64, 512, 64, 4, 1024


def fp8_cache(B, cap, seed):
    kv = cb.KVCache(cb.cache_desc(M, True, DN, DR, "bf16", "fp8", "bf16", cap), B)
    kv.nope.copy_(synth.random_fp8_codes((B, cap, DN), "na.kv", seed, device=DEV))
    kv.scale.copy_(synth.normal((B, cap), "na.sc", seed, device=DEV).abs() * 0.01 + 2e-3)
    kv.rope.copy_(synth.normal((B, cap, DR), "na.rope", seed, device=DEV, dtype=torch.bfloat16))
    return kv


def run_both(B, cap, seed):
    kv = fp8_cache(B, cap, seed)
    desc = cb.attn_desc(H, DN, DR, "bf16", "bf16", "fp8", "bf16", M, cap)
    pos = synth.uniform_int((B,), 4 * K, 4 * cap - 1, "na.pos", seed, device=DEV)
    n_vis = ((pos + 1) // M).clamp(max=cap).cpu().tolist()
    idx = synth.random_sorted_subsets(B, n_vis, K, "na.idx", seed, device=DEV)
    q = synth.normal((B, H, DN + DR), "na.q", seed, device=DEV, dtype=torch.bfloat16)
    o_ws = torch.empty((B, H, DN), dtype=torch.bfloat16, device=DEV)
    l_ws = torch.empty((B, H), dtype=torch.float32, device=DEV)
    cb.sparse_attn_decode(desc, kv, pos, q, idx, 1 / 24.0, o_ws, l_ws)
    o_na = torch.full_like(o_ws, float("nan"))
    l_na = torch.full_like(l_ws, float("nan"))
    cb.sparse_attn_decode_noalloc(desc, kv, pos, q, idx, 1 / 24.0, o_na, l_na)
    torch.cuda.synchronize()
    return (o_ws, l_ws), (o_na, l_na)


def test_noalloc_decode_matches_workspace_entry_point():
    for B, cap, seed in ((24, 65536, 1), (5, 16384, 2)):   # second call: a smaller input
        print(f"noalloc: B={B} cap={cap}", flush=True)
        (o_ws, l_ws), (o_na, l_na) = run_both(B, cap, seed)
        assert torch.equal(o_na, o_ws), f"B={B}: outputs differ"
        assert torch.equal(l_na, l_ws), f"B={B}: lse differs"


def test_noalloc_decode_rejects_sizes_past_scratch():
    desc = cb.attn_desc(H, DN, DR, "bf16", "bf16", "fp8", "bf16", M, 8192)
    per_seq = cb.workspace_bytes(cb.OP_SPARSE_ATTN_DECODE, desc, 1, 1, 0, K)
    B = cb.NOALLOC_SCRATCH_BYTES // per_seq + 1
    P = ctypes.c_void_p(0x4000)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    st = cb.lib().csa_sparse_attn_decode_noalloc(ctypes.byref(desc), B, P, P, ctypes.byref(kv), P, K, 0.1, P, None,
                                                 None)
    assert st == 4 and b"scratch" in cb.lib().csa_last_error()
