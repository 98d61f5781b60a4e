"""Oracle-side reconstruction of the full-size workloads for the GPU parity
tests.  Inputs come from the seeded generators only (regenerated on the GPU
and copied to the host); every value here is computed by oracle/ from them.
"""
import numpy as np
import torch

from compressed_sparse_amd import synth
from oracle import csa
from oracle import formats as F
from tests.helpers import near_boundary


def host(t):
    return t.detach().to("cpu", torch.float64).numpy()


def token_rows(w, b, chunk, positions, names, seed=0, device="cuda"):
    """Rows of the named token tensors at the given positions (fp64 host)."""
    positions = np.asarray(positions, dtype=np.int64)
    out = {nm: np.zeros((len(positions), w.idx_dim if nm.startswith("k") else w.c)) for nm in names}
    for c in np.unique(positions // chunk):
        sel = np.nonzero(positions // chunk == c)[0]
        x = synth.token_chunk(w, b, int(c), chunk, seed, device, names=list(names))
        r = torch.as_tensor(positions[sel] % chunk, device=device)
        for nm in names:
            out[nm][sel] = host(x[nm][r])
    return out


def params(w, seed=0):
    return {k: host(v) for k, v in synth.compressor_params(w, seed, "cuda").items()}


def csa_entries(w, b, ids, chunk, prefix="", seed=0):
    """Exact (fp64, pre-RoPE) CSA entries `ids` of sequence b, each from its
    2m-token window; prefix "k" selects the indexer-key compressor."""
    ids = np.asarray(ids, dtype=np.int64)
    m = w.m
    rows = (ids[:, None] - 1) * m + np.arange(2 * m)[None, :]     # window i-1 then i
    rows_c = np.maximum(rows, 0)
    names = [prefix + n for n in ("a", "za", "b", "zb")]
    tr = token_rows(w, b, chunk, rows_c.ravel(), names, seed)
    p = params(w, seed)
    Ba, Bb = p[prefix + "Ba"], p[prefix + "Bb"]
    out = np.zeros((len(ids), tr[names[0]].shape[1]))
    for j, i in enumerate(ids):
        sl = slice(j * 2 * m, (j + 1) * 2 * m)
        a, za, bb, zb = (tr[nm][sl] for nm in names)
        # the rows cover tokens [(i-1)m, (i+1)m); entry 0 ignores its C^b rows
        out[j] = csa.compress(a, za, Ba, m, bb, zb, Bb, i0=int(i), i1=int(i) + 1, tok0=(int(i) - 1) * m)[0]
    return out


def chunked_entries(w, b, T, chunk, prefix="", seed=0, overlap=True):
    """All entries of tokens [0, T) of sequence b, computed chunk by chunk
    (the previous chunk's last m rows carry the C^b side)."""
    m = w.m
    names = [prefix + n for n in (("a", "za", "b", "zb") if overlap else ("a", "za"))]
    p = params(w, seed)
    Ba = p[prefix + "Ba"]
    Bb = p.get(prefix + "Bb")
    outs, tail = [], None
    for c in range((T + chunk - 1) // chunk):
        n = min(chunk, T - c * chunk)
        x = synth.token_chunk(w, b, c, chunk, seed, "cuda", names=names)
        x = {k: host(v[:n]) for k, v in x.items()}
        tok0 = c * chunk
        if overlap and tail is not None:
            x = {k: np.concatenate([tail[k], x[k]], 0) for k in x}
            tok0 -= m
        i0 = (c * chunk + m) // m - 1
        i1 = (c * chunk + n) // m
        if i1 > i0:
            if overlap:
                outs.append(csa.compress(x[names[0]], x[names[1]], Ba, m, x[names[2]], x[names[3]], Bb,
                                         i0=i0, i1=i1, tok0=tok0))
            else:
                outs.append(csa.compress(x[names[0]], x[names[1]], Ba, m, i0=i0, i1=i1, tok0=tok0))
        if overlap:
            tail = {k: v[-m:] for k, v in x.items()}
    return np.concatenate(outs, 0)


def compressor_bound_rows(w, b, ids, chunk, prefix="", seed=0):
    """The GPU compressor's fp32 error bound per channel of entries `ids`
    (2m rows times 2^-23 times the largest value magnitude in the window)."""
    ids = np.asarray(ids, dtype=np.int64)
    m = w.m
    rows = np.maximum((ids[:, None] - 1) * m + np.arange(2 * m)[None, :], 0)
    tr = token_rows(w, b, chunk, rows.ravel(), [prefix + "a", prefix + "b"], seed)
    c = tr[prefix + "a"].shape[1]
    va = np.abs(tr[prefix + "a"]).reshape(len(ids), 2 * m, c)
    vb = np.abs(tr[prefix + "b"]).reshape(len(ids), 2 * m, c)
    mx = np.maximum(va[:, m:].max(1), vb[:, :m].max(1))
    return 2 * m * 2.0 ** -23 * mx


def key_flip_delta(exact, fmt, bound):
    """Per key element, the largest change the stored (decoded) key can show
    when the GPU's value rounds to the other side of a nearby boundary.
    exact: [N, d] fp64 keys; bound: [N, d] absolute fp32 error bound."""
    if fmt == "fp8":
        amax = np.abs(exact).max(1)
        s = F.to_f32(np.where(amax > 0, amax / 448, 1.0))
        y = exact / s[:, None]
        dy = bound / s[:, None] + 4e-6 * np.abs(y)
        near = near_boundary(y, F.fp8_round, dy)
        alt = np.maximum(np.abs(F.fp8_round(y - dy) - F.fp8_round(y)), np.abs(F.fp8_round(y + dy) - F.fp8_round(y)))
        return np.where(near, alt, 0.0) * s[:, None] + 4e-6 * np.abs(exact)
    if fmt == "mxfp4":
        N, d = exact.shape
        blk = np.abs(exact).reshape(N, d // 32, 32)
        amax = blk.max(-1)
        bmax = bound.reshape(N, d // 32, 32).max(-1)
        # a block scale can move one binade when amax sits near a power of two
        e_lo = F.mx_scale_exponent(np.maximum(amax - bmax, 0))
        e_hi = F.mx_scale_exponent(amax + bmax)
        X = np.ldexp(1.0, F.mx_scale_exponent(amax))
        Xs = np.repeat(X, 32, axis=1)
        y = exact / Xs
        dy = bound / Xs
        near = near_boundary(y, F.e2m1_round, dy)
        alt = np.maximum(np.abs(F.e2m1_round(y - dy) - F.e2m1_round(y)),
                         np.abs(F.e2m1_round(y + dy) - F.e2m1_round(y))) * Xs
        delta = np.where(near, alt, 0.0)
        moved = np.repeat(e_lo != e_hi, 32, axis=1)
        # re-scaled block: bound by the larger of the two roundings' errors
        return np.where(moved, np.abs(exact) * 0.5 + 2 * Xs, delta)
    if fmt == "bf16":
        near = near_boundary(exact, F.to_bf16, bound)
        ulp = np.abs(F.to_bf16(exact + bound) - F.to_bf16(exact - bound))
        return np.where(near, ulp, 0.0) + 1e-7 * np.abs(exact)
    return bound


def score_delta(qI, w_row, dk):
    """Upper bound of |I_gpu - I_oracle| for one query given per-element key
    changes dk [N, d]: sum_h |w_h| * sum_d |q_hd| * dk_d."""
    return (np.abs(qI) @ dk.T).T @ np.abs(w_row)
