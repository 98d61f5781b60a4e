"""Comparison helpers shared by the GPU parity tests."""
import numpy as np
import torch

from oracle import formats as F


def np64(t):
    """A torch tensor (any device, f32/bf16) as an fp64 numpy array."""
    return t.detach().to("cpu", torch.float64).numpy()


def max_rel_rows(got, ref):
    """max over rows of ||got - ref||_inf / ||ref||_inf (rows = last axis)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(got - ref).max(-1)
    den = np.abs(ref).max(-1)
    den = np.where(den > 0, den, 1.0)
    return float((num / den).max()) if num.size else 0.0


def lse_err(got, ref):
    """Absolute error of lse values (-inf must match -inf)."""
    got = np.asarray(got, np.float64)
    ref = np.asarray(ref, np.float64)
    inf_ok = np.array_equal(np.isneginf(got), np.isneginf(ref))
    fin = np.isfinite(ref)
    err = float(np.abs(got[fin] - ref[fin]).max()) if fin.any() else 0.0
    return inf_ok, err


def compare_topk(gpu_idx, ref_idx, ref_scores, rel_window, kth_rel_window=0.0):
    """Top-k index sets: equal, or every index in the symmetric difference
    has an oracle score within rel_window * max(1, max|I|) (plus
    kth_rel_window * |k-th score|) of the oracle's k-th score.
    Returns (n_rows_differing, list of unexplained rows)."""
    bad, differing = [], 0
    for r in range(len(ref_idx)):
        g = set(int(x) for x in gpu_idx[r] if x >= 0)
        o = set(int(x) for x in ref_idx[r] if x >= 0)
        if g == o:
            continue
        differing += 1
        I = np.asarray(ref_scores[r], np.float64)
        if len(g) != len(o):
            bad.append(r)
            continue
        kth = np.min(I[sorted(o)])
        win = rel_window * max(1.0, float(np.abs(I).max())) + kth_rel_window * abs(kth)
        for s in g ^ o:
            if s >= len(I) or abs(I[s] - kth) > win:
                bad.append(r)
                break
    return differing, bad


def ascending_padded(idx):
    """Each row lists distinct ascending indices then only -1."""
    for row in np.asarray(idx):
        v = row[row >= 0]
        n = v.size
        if not np.all(row[n:] == -1) or not np.all(np.diff(v) > 0):
            return False
    return True


def near_midpoint(y, grid_round, rel):
    """True where y (fp64) lies within rel*|y| of a rounding boundary of the
    format implemented by grid_round: rounding y*(1-rel) and y*(1+rel)
    disagree."""
    y = np.asarray(y, np.float64)
    lo = grid_round(y * (1 - rel))
    hi = grid_round(y * (1 + rel))
    return lo != hi


def near_boundary(y, grid_round, delta):
    """True where rounding y - delta and y + delta disagree, i.e. a value
    computed with an absolute error up to delta may round either way."""
    y = np.asarray(y, np.float64)
    return grid_round(y - delta) != grid_round(y + delta)


def bf16_codes_match(gpu_vals, exact, delta):
    """GPU BF16 values equal the oracle's RNE rounding of the exact fp64
    value, except where the exact value lies within delta (the GPU's fp32
    error bound) of a rounding boundary."""
    ref = F.to_bf16(exact)
    ok = (gpu_vals == ref) | near_boundary(exact, F.to_bf16, delta)
    return ok, int((gpu_vals != ref).sum())


def compressor_error_bound(x, m, overlap, d_nope):
    """Absolute fp32 error bound of each compressed channel: the GPU sums
    2m (or m) softmax-weighted rows in fp32, so its error is at most about
    rows * 2^-23 * max|value row|; the RoPE turn mixes channel pairs, so the
    RoPE dims take the larger bound of their pair.  x: dict of [T, c] fp64
    arrays a (and b).  Returns [N, c]."""
    a = np.abs(np.asarray(x["a"], np.float64))
    T, c = a.shape
    N = T // m
    mx = a[:N * m].reshape(N, m, c).max(1)
    rows = m
    if overlap:
        b = np.abs(np.asarray(x["b"], np.float64))[:N * m].reshape(N, m, c).max(1)
        prev = np.concatenate([np.zeros((1, c)), b[:-1]], 0)
        mx = np.maximum(mx, prev)
        rows = 2 * m
    bound = rows * 2.0 ** -23 * mx
    if c > d_nope:
        r = bound[:, d_nope:].reshape(N, -1, 2).max(-1)
        bound[:, d_nope:] = np.repeat(r, 2, axis=1)
    return bound


def topk_explained(gpu_row, ref_row, I, delta, eps):
    """True when the GPU's top-k set equals the oracle's, or every index in
    the symmetric difference has an oracle score within delta[s] +
    max(delta) near the threshold + eps of the oracle's k-th score: a swap
    that the bounded differences between the two sides' inputs can cause."""
    g = set(int(x) for x in gpu_row if x >= 0)
    o = set(int(x) for x in ref_row if x >= 0)
    if g == o:
        return True
    if len(g) != len(o):
        return False
    kth = np.min(I[sorted(o)])
    near = np.abs(I - kth) <= 2 * float(delta.max()) + eps
    d_thr = float(delta[near].max()) if near.any() else 0.0
    return all(s < len(I) and abs(I[s] - kth) <= delta[s] + d_thr + eps for s in g ^ o)


def fp32_score_bound(qq, w_row, K, n, gamma=2.0 ** -17):
    """Bound on the fp32 accumulation error of the indexer scores of one
    query: the standard summation bound (a constant times the unit roundoff
    times the sum of the absolute terms), gamma * sum_h |w_h| * sum_d
    |qq_hd K_sd| for s < n.  gamma = 2^-17 covers the 16 x 64 products of a
    score (u = 2^-24) with room for the order of the sums."""
    mag = np.abs(np.asarray(K[:n], np.float64)) @ np.abs(np.asarray(qq, np.float64)).T
    return gamma * (mag @ np.abs(np.asarray(w_row, np.float64)))
