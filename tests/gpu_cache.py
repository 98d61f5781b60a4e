"""Exact host decoding of caches the GPU wrote, and the checks that run the
oracle on them (the second parity leg: the oracle's indexer, top-k and
attention over the very codes the kernels read, so that the tie rule can be
exact and attention is judged with the GPU's own index lists).

Decoding uses the format definitions in oracle/formats.py only (OFP8 E4M3
codes times the per-entry fp32 scale; BF16 / fp32 as stored; MXFP4 packed
E2M1 pairs, low nibble = even element, times 2^(E8M0 - 127)).
"""
import numpy as np
import torch

from oracle import csa
from oracle import formats as F
from tests.helpers import lse_err, max_rel_rows


def _rows(kv, t, b, ids):
    """Rows `ids` of sequence b of one cache tensor: rows b*cap + id of a
    contiguous cache; for a paged one the pool rows its block table names
    (table[b][id / page] * page + id mod page)."""
    ids = np.asarray(ids, dtype=np.int64)
    if kv.desc.page_size:
        P = kv.desc.page_size
        tab = kv.block_table[b].cpu().numpy().astype(np.int64)
        phys = tab[ids // P] * P + ids % P
        flat = t.reshape((-1,) + tuple(t.shape[2:]))
        return flat.index_select(0, torch.as_tensor(phys, device=t.device))
    return t[b].index_select(0, torch.as_tensor(ids, device=t.device))


def decode_nope(kv, b, ids):
    """Decoded non-RoPE (or indexer-key) rows `ids` of sequence b, fp64."""
    fmt = kv.desc.nope_dtype
    if fmt == 2:  # FP8 E4M3 + per-entry scale
        codes = _rows(kv, kv.nope, b, ids).cpu().numpy()
        sc = _rows(kv, kv.scale, b, ids).cpu().double().numpy()
        return F.fp8_decode(codes) * sc[:, None]
    if fmt == 3:  # MXFP4
        packed = _rows(kv, kv.nope, b, ids).cpu().numpy().astype(np.int64)
        codes = np.stack([packed & 0xF, packed >> 4], -1).reshape(packed.shape[0], -1)
        return F.mxfp4_decode(codes, _rows(kv, kv.scale, b, ids).cpu().numpy())
    return _rows(kv, kv.nope, b, ids).to("cpu", torch.float64).numpy()


def decode_kv(kv, b, ids):
    """Decoded KV rows `ids` of sequence b: K (the whole entry) [len, c]."""
    V = decode_nope(kv, b, ids)
    if kv.rope is None:
        return V
    R = _rows(kv, kv.rope, b, ids).to("cpu", torch.float64).numpy()
    return np.concatenate([V, R], 1)


def bf16_step(x):
    """Spacing of the BF16 grid at |x| (one unit in the last place)."""
    a = np.maximum(np.abs(np.asarray(x, np.float64)), 2.0 ** -126)
    return np.ldexp(1.0, np.floor(np.log2(a)).astype(np.int64) - 7)


def topk_exact_rule(gpu_row, I, n, k, score_fmt):
    """North-star rule on identical inputs: the GPU's set equals the oracle's
    top-k except for indices whose score lies within 1e-6 * max(1, max|I|)
    of the oracle's k-th score (plus one BF16 step in BF16-score mode, where
    the GPU's fp32 sum and the oracle's exact one may round to neighbouring
    BF16 values).  Returns (ok, number of swapped indices, oracle list)."""
    ref = csa.topk(I, n, k)
    g = set(int(x) for x in gpu_row if x >= 0)
    o = set(int(x) for x in ref if x >= 0)
    if g == o:
        return True, 0, ref
    if len(g) != len(o) or any(s >= n for s in g):
        return False, len(g ^ o), ref
    tau = float(np.min(I[sorted(o)]))
    win = 1e-6 * max(1.0, float(np.abs(I[:n]).max()))
    if score_fmt == "bf16":
        win += float(bf16_step(tau))
    ok = all(abs(float(I[s]) - tau) <= win for s in g ^ o)
    return ok, len(g ^ o) // 2, ref


def attend_gpu_idx(q, pos, kv, b, gpu_row, d_nope, base, tau):
    """Oracle attention of one query over the GPU's index list, reading the
    GPU-written cache rows."""
    ids = np.asarray([int(x) for x in gpu_row if x >= 0], dtype=np.int64)
    K = decode_kv(kv, b, ids) if len(ids) else np.zeros((0, q.shape[-1]))
    loc = np.arange(len(ids))
    return csa.attend(csa.rope_query(q, pos, d_nope, base), K, K[:, :d_nope], loc, tau)


def check_attention(name, o_gpu, lse_gpu, o_ref, lse_ref, tol=1e-2, lse_tol=1e-2):
    """Per-row max-rel of o (rows = (query, head)) and the absolute lse error."""
    err = max_rel_rows(np.asarray(o_gpu).reshape(-1, o_ref.shape[-1]), o_ref.reshape(-1, o_ref.shape[-1]))
    inf_ok, lerr = lse_err(np.asarray(lse_gpu).ravel(), np.asarray(lse_ref).ravel())
    assert inf_ok, f"{name}: empty rows differ"
    assert err <= tol, f"{name}: max-rel {err}"
    assert lerr <= lse_tol, f"{name}: lse error {lerr}"
    return err, lerr
