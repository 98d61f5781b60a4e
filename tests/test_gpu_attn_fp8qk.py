"""GPU parity of the FP8 QK product (attention descriptor qk_mode =
CSA_FP8E4M3): the query's non-RoPE dims rounded to MXFP8 inside the kernel
and multiplied with the FP8 cache codes by the scaled FP8 MFMA, against the
oracle's "mxfp8" query format.

The kernel rounds the same BF16 query values with the same rule, so the
codes agree exactly and the results differ from the oracle only by fp32
summation order and the BF16 rounding of P and of the output: the tolerances
of the BF16-QK tests apply.  Each test also checks that the GPU result sits
much closer to the oracle's FP8-QK result than to its BF16-QK result, so the
query is seen to be quantised.  Synthetic queries include blocks that take
each branch of the rounding: an all-zero block, blocks whose maximum rounds
up past 448 (saturating), tiny blocks (scale 2^-127)."""
import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import path, synth
from oracle import csa
from tests.helpers import lse_err, max_rel_rows, np64
from tests.test_gpu_attn import kv_cache

pytestmark = pytest.mark.gpu
DEV = "cuda"
H, DN, DR = 64, 512, 64


def query(shape, seed, scale=2.0):
    """BF16 queries [..., H, 576] with special blocks in the first rows."""
    q = synth.normal(shape + (H, DN + DR), "q8", seed, device=DEV) * scale
    flat = q.view(-1, H, DN + DR)
    flat[0, 0, :32] = 0.0                         # zero block
    flat[0, 1, 32:64] = 1e-37                     # below 2^-118: scale 2^-127
    flat[0, 2, 64:96] *= 0.1
    flat[0, 2, 70] = 1.95 * 4.0                   # 499 before rounding: saturates to 448
    flat[0, 3, 96:128] = 3.0                      # 1.5 * 2^1: 384, exact
    if flat.shape[0] > 1:
        flat[1, :, :DN] = 0.0                     # the RoPE dims alone
    return q.to(torch.bfloat16).contiguous()


def check(o, lse, ref8, ref16, tol=1e-2):
    """o / lse against the FP8-QK oracle; and at least 4x closer to it than
    the BF16-QK oracle is."""
    o8, l8 = ref8
    o16, l16 = ref16
    g_o = np64(o).reshape(-1, DN)
    err_o = max_rel_rows(g_o, o8.reshape(-1, DN))
    inf_ok, err_l = lse_err(np64(lse).ravel(), l8.ravel())
    assert inf_ok and err_o <= tol and err_l <= tol, (err_o, err_l)
    sep_l = lse_err(l16.ravel(), l8.ravel())[1]
    _, err16 = lse_err(np64(lse).ravel(), l16.ravel())
    assert err_l * 4 <= sep_l <= err16 * 1.5, (err_l, sep_l, err16)
    return err_o, err_l, sep_l


@pytest.mark.parametrize("pos0,T", [(0, 300), (128 * 500 - 37, 300)])
def test_dense_prefill_fp8qk(pos0, T):
    m = 128
    cap = (pos0 + T) // m + 2
    kv, cache = kv_cache("fp8", "bf16", 1, cap, DN, DR, m, seed=41)
    q = query((1, T), 41)
    o = torch.empty((1, T, H, DN), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
    tau = 576 ** -0.5
    cb.dense_attn_prefill(cb.attn_desc(H, DN, DR, "bf16", "bf16", "fp8", "bf16", m, cap, qk="fp8"), kv, pos0, q, tau,
                          o, lse)
    torch.cuda.synchronize()
    qn, c0 = np64(q[0]), {"k": cache["k"][0], "v": cache["v"][0]}
    pos = pos0 + np.arange(T)
    r8 = csa.hca_rows(pos, qn, c0, m, DN, 1e4, tau, qk_fmt="mxfp8")
    r16 = csa.hca_rows(pos, qn, c0, m, DN, 1e4, tau)
    print("dense prefill fp8qk pos0", pos0, "err o / lse / separation", check(o, lse, r8, r16), flush=True)


def test_dense_decode_fp8qk_splits_and_window():
    B, m, cap = 4, 128, 1024
    kv, cache = kv_cache("fp8", "bf16", B, cap, DN, DR, m, seed=42)
    positions = [128 * cap - 1, 128 * 700 + 5, 127, 100]
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    q = query((B,), 42)
    tau = 576 ** -0.5
    for window in (0, 300):
        o = torch.empty((B, H, DN), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
        desc = cb.attn_desc(H, DN, DR, "bf16", "bf16", "fp8", "bf16", m, cap, window=window, qk="fp8")
        cb.dense_attn_decode(desc, kv, pos, q, tau, o, lse)
        torch.cuda.synchronize()
        qn = np64(q)
        refs = {}
        for fmt in ("mxfp8", "bf16"):
            rr = [csa.dense_attention_row(qn[b], positions[b], {"k": cache["k"][b], "v": cache["v"][b]}, m, DN, 1e4,
                                          tau, window, qk_fmt=fmt) for b in range(B)]
            refs[fmt] = (np.stack([r[0] for r in rr]), np.stack([r[1] for r in rr]))
        print("dense decode fp8qk window", window, check(o, lse, refs["mxfp8"], refs["bf16"]), flush=True)


def test_sparse_prefill_and_decode_fp8qk():
    T, m, k, pos0 = 160, 4, 1024, 8192
    cap = (pos0 + T) // m + 8
    kv, cache = kv_cache("fp8", "bf16", 1, cap, DN, DR, m, seed=43)
    n_vis = [(pos0 + t + 1) // m for t in range(T)]
    sub = [n - 40 if t % 3 == 0 else n for t, n in enumerate(n_vis)]
    idx = synth.random_sorted_subsets(T, sub, k, "idx", 43)[None].to(DEV)
    q = query((1, T), 43)
    tau = 1 / 24.0
    desc = cb.attn_desc(H, DN, DR, "bf16", "bf16", "fp8", "bf16", m, cap, qk="fp8")
    o = torch.empty((1, T, H, DN), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((1, T, H), dtype=torch.float32, device=DEV)
    cb.sparse_attn_prefill(desc, kv, pos0, q, idx, tau, o, lse)
    # decode: rows 0, 7, 100 as three sequences over the same cache
    rows = [0, 7, 100]
    kv3, _ = kv_cache("fp8", "bf16", 3, cap, DN, DR, m, seed=43)
    for b in range(3):
        kv3.nope[b].copy_(kv.nope[0]); kv3.scale[b].copy_(kv.scale[0]); kv3.rope[b].copy_(kv.rope[0])
    od = torch.empty((3, H, DN), dtype=torch.bfloat16, device=DEV)
    ld = torch.empty((3, H), dtype=torch.float32, device=DEV)
    posd = torch.tensor([pos0 + r for r in rows], dtype=torch.int64, device=DEV)
    cb.sparse_attn_decode(desc, kv3, posd, q[0, rows].contiguous(), idx[0, rows].contiguous(), tau, od, ld)
    torch.cuda.synchronize()
    qn, ix, c0 = np64(q[0]), idx[0].cpu().numpy(), {"k": cache["k"][0], "v": cache["v"][0]}
    refs = {}
    for fmt in ("mxfp8", "bf16"):
        rr = [csa.sparse_attention_row(qn[t], pos0 + t, c0, ix[t][ix[t] < n_vis[t]], DN, 1e4, tau, qk_fmt=fmt)
              for t in range(T)]
        refs[fmt] = (np.stack([r[0] for r in rr]), np.stack([r[1] for r in rr]))
    print("sparse prefill fp8qk", check(o, lse, refs["mxfp8"], refs["bf16"]), flush=True)
    sel = lambda r: (r[0][rows], r[1][rows])
    print("sparse decode fp8qk", check(od, ld, sel(refs["mxfp8"]), sel(refs["bf16"])), flush=True)


def test_paged_dense_fp8qk_equals_contiguous():
    B, m, page, cap = 3, 128, 64, 1024
    kv, _ = kv_cache("fp8", "bf16", B, cap, DN, DR, m, seed=44)
    positions = [128 * cap - 1, 128 * 333 + 64, 128 * 90]
    table, pool = path.block_tables([(p + 1) // m for p in positions], page, cap, seed=4)
    pdesc = cb.cache_desc(m, True, DN, DR, "f32", "fp8", "bf16", cap, page_size=page, pool_pages=pool)
    pkv = cb.KVCache(pdesc, B, block_table=table)
    tab = table.cpu().numpy()
    for name in ("nope", "scale", "rope"):
        dst, src = getattr(pkv, name), getattr(kv, name)
        for b in range(B):
            for lp, pp in enumerate(tab[b]):
                if pp >= 0:
                    dst[pp] = src[b, lp * page:(lp + 1) * page]
    assert torch.equal(pkv.logical(pkv.nope)[0], kv.nope[0])
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    q = query((B,), 44)
    tau = 576 ** -0.5
    outs = []
    for cache_, kw in ((kv, {}), (pkv, dict(page_size=page, pool_pages=pool))):
        o = torch.empty((B, H, DN), dtype=torch.bfloat16, device=DEV)
        lse = torch.empty((B, H), dtype=torch.float32, device=DEV)
        cb.dense_attn_decode(cb.attn_desc(H, DN, DR, "bf16", "bf16", "fp8", "bf16", m, cap, qk="fp8", **kw), cache_,
                             pos, q, tau, o, lse)
        outs.append((o, lse))
    torch.cuda.synchronize()
    assert torch.equal(outs[0][0], outs[1][0]) and torch.equal(outs[0][1], outs[1][1])
