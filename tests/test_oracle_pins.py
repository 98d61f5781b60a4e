"""Pins of the CSA / HCA oracle against things other than itself (CPU only):
closed forms, invariants, textbook special cases evaluated with torch's own
attention routine, and pure-Python brute force on tiny inputs."""
import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import brute, csa
from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_values.json")


def rnd(shape, seed, scale=1.0):
    return np.random.default_rng(seed).standard_normal(shape) * scale


def complex_rope(x, pos, d_nope, base):
    """RoPE written independently as complex multiplication by e^{i pos theta}."""
    t = torch.as_tensor(x, dtype=torch.float64)
    d_rope = t.shape[-1] - d_nope
    theta = base ** (-torch.arange(0, d_rope, 2, dtype=torch.float64) / d_rope)
    ang = torch.as_tensor(pos, dtype=torch.float64)[..., None] * theta
    z = torch.view_as_complex(t[..., d_nope:].reshape(*t.shape[:-1], d_rope // 2, 2).contiguous())
    zr = z * torch.polar(torch.ones_like(ang), ang)
    return torch.cat([t[..., :d_nope], torch.view_as_real(zr).reshape(*t.shape[:-1], d_rope)], -1).numpy()


# ---------------------------------------------------------------- compressor

def test_compress_matches_bruteforce_overlapped():
    T, c, m = 24, 5, 4
    a, b, za, zb = (rnd((T, c), s) for s in range(4))
    Ba, Bb = rnd((m, c), 10), rnd((m, c), 11)
    got = csa.compress(a, za, Ba, m, b, zb, Bb)
    ref = np.array(brute.compress(a.tolist(), za.tolist(), Ba.tolist(), m, b.tolist(), zb.tolist(), Bb.tolist()))
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("m", [1, 2, 4, 8])
def test_compress_matches_bruteforce_single_window(m):
    T, c = 32, 3
    a, za = rnd((T, c), 20), rnd((T, c), 21)
    Ba = rnd((m, c), 22)
    got = csa.compress(a, za, Ba, m)
    ref = np.array(brute.compress(a.tolist(), za.tolist(), Ba.tolist(), m))
    assert np.allclose(got, ref, rtol=0, atol=1e-13)


@pytest.mark.parametrize("m,overlap", [(4, True), (8, False)])
def test_compress_from_hidden_matches_bruteforce(m, overlap):
    """Projections from hidden states then compression, against explicit
    Python dot products and the brute-force compressor."""
    T, d, c = 16, 7, 3
    X = rnd((T, d), 60)
    names = ("aKV", "aZ", "bKV", "bZ") if overlap else ("aKV", "aZ")
    W = {n: rnd((d, c), 61 + i, 0.5) for i, n in enumerate(names)}
    Ba, Bb = rnd((m, c), 70), (rnd((m, c), 71) if overlap else None)
    got = csa.compress_from_hidden(X, W, Ba, m, Bb)
    ref = np.array(brute.compress_from_hidden(X.tolist(), {k: v.tolist() for k, v in W.items()}, Ba.tolist(), m,
                                              None if Bb is None else Bb.tolist()))
    assert np.allclose(got, ref, rtol=0, atol=1e-12)


def test_compress_from_hidden_closed_forms():
    """(1) Z-projections and biases zero: every overlapped entry i >= 1 is
    the mean of its 2m hidden rows times the value projections, (mean of
    window i) W^{aKV} / 2 + (mean of window i-1) W^{bKV} / 2 (entry 0: the mean
    of its window times W^{aKV}).  (2) d_model = c and identity projections:
    the entries are those of compress() on X itself."""
    T, d, c, m = 24, 5, 4, 4
    X = rnd((T, d), 80)
    W = {"aKV": rnd((d, c), 81), "bKV": rnd((d, c), 82), "aZ": np.zeros((d, c)), "bZ": np.zeros((d, c))}
    zero = np.zeros((m, c))
    got = csa.compress_from_hidden(X, W, zero, m, zero)
    win = X.reshape(T // m, m, d).mean(1)
    ref = np.concatenate([win[:1] @ W["aKV"], 0.5 * (win[1:] @ W["aKV"]) + 0.5 * (win[:-1] @ W["bKV"])], 0)
    assert np.allclose(got, ref, rtol=0, atol=1e-12)
    Xc = rnd((T, c), 83)
    eye = {"aKV": np.eye(c), "aZ": np.eye(c), "bKV": np.eye(c), "bZ": np.eye(c)}
    Ba, Bb = rnd((m, c), 84), rnd((m, c), 85)
    assert np.allclose(csa.compress_from_hidden(Xc, eye, Ba, m, Bb), csa.compress(Xc, Xc, Ba, m, Xc, Xc, Bb),
                       rtol=0, atol=1e-14)


def test_compress_zero_logits_is_mean():
    """Z = B = 0: an overlapped entry is the plain mean of its 2m rows (of m
    rows for entry 0); an HCA entry is the mean of its m' rows."""
    T, c, m = 40, 6, 4
    a, b = rnd((T, c), 30), rnd((T, c), 31)
    z = np.zeros((T, c))
    Bz = np.zeros((m, c))
    got = csa.compress(a, z, Bz, m, b, z, Bz)
    assert np.allclose(got[0], a[:m].mean(0), atol=1e-14)
    for i in range(1, T // m):
        ref = (a[i * m:(i + 1) * m].sum(0) + b[(i - 1) * m:i * m].sum(0)) / (2 * m)
        assert np.allclose(got[i], ref, atol=1e-14)
    mh = 8
    got = csa.compress(a, z, np.zeros((mh, c)), mh)
    assert np.allclose(got, a[:T // mh * mh].reshape(-1, mh, c).mean(1), atol=1e-14)


def test_compress_softmax_rows_sum_to_one():
    T, c, m = 16, 7, 4
    za, zb = rnd((T, c), 40, 3.0), rnd((T, c), 41, 3.0)
    Ba, Bb = rnd((m, c), 42), rnd((m, c), 43)
    for i in range(T // m):
        w = csa.compress_weights(za, Ba, m, zb, Bb, i)
        assert w.shape[0] == (m if i == 0 else 2 * m)
        assert np.allclose(w.sum(0), 1.0, atol=1e-12)


def test_compress_shift_invariance_and_dominant_logit():
    T, c, m = 16, 4, 4
    a, b, za, zb = (rnd((T, c), s) for s in range(50, 54))
    Ba, Bb = rnd((m, c), 54), rnd((m, c), 55)
    base = csa.compress(a, za, Ba, m, b, zb, Bb)
    shift = rnd((1, c), 56) * 5
    shifted = csa.compress(a, za + shift, Ba, m, b, zb + shift, Bb)
    assert np.allclose(base, shifted, atol=1e-12)
    # one logit far above the rest selects that row's value (entry 2: C^b row 1)
    zb2 = zb.copy()
    zb2[1 * m + 1, :] += 1e3
    sel = csa.compress(a, za, Ba, m, b, zb2, Bb)
    assert np.allclose(sel[2], b[1 * m + 1], atol=1e-12)


@pytest.mark.parametrize("overlap", [True, False])
def test_compress_locality(overlap):
    """Perturbing token group g changes only entries g and g+1 (overlapped:
    each group is covered by two entries) or entry g (single window)."""
    T, c, m, g = 32, 4, 4, 3
    a, b, za, zb = (rnd((T, c), s) for s in range(60, 64))
    Ba, Bb = rnd((m, c), 64), rnd((m, c), 65)
    args = (b, zb, Bb) if overlap else (None, None, None)
    base = csa.compress(a, za, Ba, m, *args)
    a2, b2 = a.copy(), b.copy()
    a2[g * m:(g + 1) * m] += 1.0
    b2[g * m:(g + 1) * m] += 1.0
    args2 = (b2, zb, Bb) if overlap else (None, None, None)
    pert = csa.compress(a2, za, Ba, m, *args2)
    changed = set(np.nonzero(np.abs(pert - base).max(1) > 0)[0])
    assert changed == ({g, g + 1} if overlap else {g})


def test_compress_chunk_offsets():
    """Entries computed from a token slice (tok0 > 0) equal the full run."""
    T, c, m = 64, 3, 4
    a, b, za, zb = (rnd((T, c), s) for s in range(70, 74))
    Ba, Bb = rnd((m, c), 74), rnd((m, c), 75)
    full = csa.compress(a, za, Ba, m, b, zb, Bb)
    tok0 = 20          # window 5 starts at 20; entry 6 needs window 5 for C^b
    part = csa.compress(a[tok0:], za[tok0:], Ba, m, b[tok0:], zb[tok0:], Bb, i0=6, i1=16, tok0=tok0)
    assert np.allclose(part, full[6:16], atol=0)


# ---------------------------------------------------------------- RoPE

def test_rope_matches_complex_form_and_preserves_norms():
    x = rnd((10, 12), 80)
    pos = np.arange(10) * 37 + 5
    got = csa.rope(x, pos, 4, 10000.0)
    assert np.allclose(got, complex_rope(x, pos, 4, 10000.0), atol=1e-13)
    assert np.array_equal(got[:, :4], x[:, :4])
    pairs = lambda v: np.hypot(v[:, 4::2], v[:, 5::2])
    assert np.allclose(pairs(got), pairs(x), atol=1e-13)


def test_rope_relative_position():
    q, k = rnd((1, 16), 81), rnd((1, 16), 82)
    d = lambda p, s: float((csa.rope(q, p, 8, 10000.0) @ csa.rope(k, s, 8, 10000.0).T)[0, 0])
    assert abs(d(100, 37) - d(100 + 5000, 37 + 5000)) < 1e-10


def test_rope_entry_position():
    assert list(csa.entry_position(np.arange(3), 4)) == [3, 7, 11]
    assert list(csa.entry_position(np.arange(3), 1)) == [0, 1, 2]


# ---------------------------------------------------------------- indexer / top-k

def test_scores_match_bruteforce():
    HI, d, n = 3, 8, 20
    qI, w, K = rnd((HI, d), 90), rnd(HI, 91), rnd((n, d), 92)
    got = csa.index_scores(qI, w, K, n)
    ref = brute.scores(qI.tolist(), w.tolist(), K.tolist(), n)
    assert np.allclose(got, ref, atol=1e-12)


def test_topk_matches_full_sort_and_tie_rule():
    rng = np.random.default_rng(93)
    for trial in range(50):
        n = int(rng.integers(1, 60))
        k = int(rng.integers(1, 40))
        I = np.round(rng.standard_normal(n), 1)       # many exact ties
        got = csa.topk(I, n, k)
        assert list(got) == brute.topk(list(I), k)
    I = np.array([0.0, -0.0, 0.0, -0.0, 1.0])
    assert list(csa.topk(I, 5, 3)) == [0, 1, 4]       # -0 == +0, lower index wins
    assert list(csa.topk(np.ones(4), 4, 6)) == [0, 1, 2, 3, -1, -1]


def test_topk_invariant_to_positive_weight_scaling():
    HI, d, n, k = 4, 8, 200, 17
    qI, w, K = rnd((HI, d), 94), rnd(HI, 95), rnd((n, d), 96)
    a = csa.topk(csa.index_scores(qI, w, K, n), n, k)
    b = csa.topk(csa.index_scores(qI, 3.7 * w, K, n), n, k)
    assert np.array_equal(a, b)
    # one head with w = 1: order is that of ReLU(q.k) (checked by torch.topk on distinct values)
    I1 = csa.index_scores(qI[:1], np.ones(1), K, n)
    dots = torch.relu(torch.as_tensor(K) @ torch.as_tensor(qI[0]))
    pos = dots > 0
    assert np.allclose(I1, dots.numpy(), atol=1e-14)
    if pos.sum() >= k:
        ref = torch.topk(dots, k).indices.sort().values.numpy()
        assert np.array_equal(csa.topk(I1, n, k), ref)


def test_visibility():
    assert list(csa.n_visible(np.array([0, 2, 3, 4, 7, 8]), 4)) == [0, 0, 1, 1, 2, 2]
    assert int(csa.n_visible((1 << 20) - 1, 4)) == 262144
    assert int(csa.n_visible((1 << 20) - 1, 128)) == 8192


def test_mxfp4_scores_exact_in_fp32():
    """Products of E2M1 values with E8M0 scales are exact; the per-head dot
    product of MXFP4 vectors is reproduced exactly in fp32 arithmetic."""
    rng = np.random.default_rng(97)
    q = F.mxfp4_quantize(rng.standard_normal((16, 64)))[0]
    K = F.mxfp4_quantize(rng.standard_normal((100, 64)))[0]
    d64 = K @ q.T
    d32 = (K.astype(np.float32) @ q.T.astype(np.float32)).astype(np.float64)
    assert np.array_equal(d64, d32)


# ---------------------------------------------------------------- attention

def test_attend_matches_bruteforce():
    H, c, dv, n = 3, 6, 4, 9
    q, K = rnd((H, c), 100), rnd((n, c), 101)
    V = K[:, :dv]
    sel = [0, 2, 3, 7]
    o, lse = csa.attend(q, K, V, sel, 0.3)
    ob, lb = brute.attend(q.tolist(), K.tolist(), V.tolist(), sel, 0.3)
    assert np.allclose(o, ob, atol=1e-13) and np.allclose(lse, lb, atol=1e-13)
    p = csa.attention_probs(q, K, sel, 0.3)
    assert np.allclose(p.sum(1), 1.0, atol=1e-13)


def test_attend_single_entry_and_empty_and_permutation():
    H, c, dv = 2, 6, 4
    q, K = rnd((H, c), 102), rnd((10, c), 103)
    V = K[:, :dv]
    o, lse = csa.attend(q, K, V, [4], 0.5)
    assert np.allclose(o, np.broadcast_to(V[4], o.shape), atol=1e-15)
    assert np.allclose(lse, 0.5 * q @ K[4], atol=1e-14)
    o, lse = csa.attend(q, K, V, [-1, -1], 0.5)
    assert not o.any() and np.all(np.isneginf(lse))
    o1, l1 = csa.attend(q, K, V, [1, 5, 8, -1], 0.5)
    o2, l2 = csa.attend(q, K, V, [8, 1, -1, 5], 0.5)
    assert np.allclose(o1, o2, atol=1e-14) and np.allclose(l1, l2, atol=1e-14)


def test_query_rescaling_keeps_topk_and_changes_temperature():
    """Rescaling the query by c > 0: the indexer's top-k is unchanged (ReLU
    and the head weights are positively homogeneous), while attention sees
    the logits scaled by c, i.e. the temperature tau -> c tau.  The two limits
    pin where tau enters: tau -> 0 gives the plain mean of the selected values
    with lse = log(count); a large tau gives the value of the best entry."""
    HI, dI, H, c, dv, n, k = 4, 8, 3, 10, 6, 300, 20
    qI, w, Ki = rnd((HI, dI), 110), rnd(HI, 111), rnd((n, dI), 112)
    for cc in (0.25, 3.0, 1e3):
        assert np.array_equal(csa.topk(csa.index_scores(qI, w, Ki, n), n, k),
                              csa.topk(csa.index_scores(cc * qI, w, Ki, n), n, k))
    q, K = rnd((H, c), 113), rnd((n, c), 114)
    V = K[:, :dv]
    sel = csa.topk(csa.index_scores(qI, w, Ki, n), n, k)
    tau = 1 / math.sqrt(c)
    o1, l1 = csa.attend(q, K, V, sel, tau)
    o2, l2 = csa.attend(2.0 * q, K, V, sel, tau)
    o3, l3 = csa.attend(q, K, V, sel, 2.0 * tau)
    assert np.allclose(o2, o3, atol=1e-13) and np.allclose(l2, l3, atol=1e-12)
    assert np.abs(o2 - o1).max() > 1e-2          # a different temperature
    # tau -> 0: uniform weights
    o0, l0 = csa.attend(q, K, V, sel, 1e-13)
    assert np.allclose(o0, np.broadcast_to(V[sel].mean(0), o0.shape), atol=1e-9)
    assert np.allclose(l0, math.log(k), atol=1e-9)
    # large tau: the arg-max entry of each head
    oi, li = csa.attend(q, K, V, sel, 1e4)
    best = sel[np.argmax(q @ K[sel].T, axis=1)]
    assert np.allclose(oi, V[best], atol=1e-9)
    assert np.allclose(li, 1e4 * np.max(q @ K[sel].T, axis=1), rtol=1e-12)


def _mxfp8_brute(x):
    """MXFP8 of one 32-element block by plain search: the e with
    2^(e+8) <= amax < 2^(e+9), then each element the nearest of the 127 E4M3
    magnitudes times 2^e (ties to the even code, saturating)."""
    amax = max(abs(v) for v in x)
    if amax == 0:
        return [0.0] * len(x)
    e = -130
    while 2.0 ** (e + 9) <= amax:
        e += 1
    mags = F.fp8_decode(np.arange(0x7F))
    out = []
    for v in x:
        d = np.abs(mags - min(abs(v) / 2.0 ** e, 448.0))
        best = np.nonzero(d == d.min())[0]
        pick = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        out.append(math.copysign(mags[pick] * 2.0 ** e, v))
    return out


def test_fp8_qk_attention_matches_bruteforce():
    """FP8 QK product: each head's non-RoPE query dims rounded to MXFP8 in
    32-dim blocks, RoPE dims untouched, then the plain attention (brute
    force end to end)."""
    H, d_nope, d_rope, n, m, pos = 2, 64, 4, 7, 4, 29
    c = d_nope + d_rope
    q = rnd((H, c), 120) * np.array([0.3] * 32 + [3.0] * 32 + [1.0] * d_rope)
    K = rnd((n, c), 121)
    cache = {"k": K, "v": K[:, :d_nope]}
    o, lse = csa.dense_attention_row(q, pos, cache, m, d_nope, 100.0, 0.3, qk_fmt="mxfp8")
    qq = [_mxfp8_brute(q[h, :32].tolist()) + _mxfp8_brute(q[h, 32:64].tolist()) + q[h, d_nope:].tolist()
          for h in range(H)]
    qr = complex_rope(np.array(qq), pos, d_nope, 100.0)
    ob, lb = brute.attend(qr.tolist(), K.tolist(), K[:, :d_nope].tolist(), list(range(n)), 0.3)
    assert np.allclose(o, ob, atol=1e-12) and np.allclose(lse, lb, atol=1e-12)
    # quantisation changes the result (the two formats are told apart)
    o16, _ = csa.dense_attention_row(q, pos, cache, m, d_nope, 100.0, 0.3)
    assert np.abs(o16 - o).max() > 1e-4


def test_fp8_qk_special_cases():
    H, d_nope, d_rope, n, m, pos = 3, 64, 8, 9, 1, 8
    c = d_nope + d_rope
    K = rnd((n, c), 122)
    cache = {"k": K, "v": K[:, :d_nope]}
    # a query already on the MXFP8 grid: both QK formats give the same bits
    codes = np.random.default_rng(123).integers(0, 0x7F, (H, d_nope)) | (np.random.default_rng(124).integers(0, 2, (H, d_nope)) << 7)
    codes[:, ::32] = 0x78                        # each block's maximum is 256 * 2^e
    codes = codes.astype(np.uint8)
    onm = (F.fp8_decode(codes) * 2.0 ** -9).clip(-0.5, 0.5)
    onm[:, ::32] = 0.5
    q = np.concatenate([F.mxfp8_quantize(onm)[0], rnd((H, d_rope), 125)], 1)
    a = csa.dense_attention_row(q, pos, cache, m, d_nope, 1e4, 0.2, qk_fmt="mxfp8")
    b = csa.dense_attention_row(q, pos, cache, m, d_nope, 1e4, 0.2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])
    # zero non-RoPE dims: the RoPE dims alone, untouched by the FP8 mode
    q0 = np.concatenate([np.zeros((H, d_nope)), rnd((H, d_rope), 126)], 1)
    a = csa.sparse_attention_row(q0, pos, cache, [0, 3, 5], d_nope, 1e4, 0.2, qk_fmt="mxfp8")
    b = csa.sparse_attention_row(q0, pos, cache, [0, 3, 5], d_nope, 1e4, 0.2)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_lse_merge_of_partitions():
    """Splitting the entry set and merging (o, lse) partials by LSE gives the
    unsplit result (the identity the split-K GPU kernels rely on)."""
    H, c, dv = 4, 8, 5
    q, K = rnd((H, c), 104), rnd((30, c), 105)
    V = K[:, :dv]
    full_o, full_l = csa.attend(q, K, V, np.arange(30), 0.4)
    parts = [csa.attend(q, K, V, np.arange(s, s + 10), 0.4) for s in (0, 10, 20)]
    L = np.logaddexp.reduce(np.stack([p[1] for p in parts]), axis=0)
    o = sum(np.exp(p[1] - L)[:, None] * p[0] for p in parts)
    assert np.allclose(o, full_o, atol=1e-13) and np.allclose(L, full_l, atol=1e-13)


def _tiny_inputs(T, c, d_nope, H, HI, dI, m, seed):
    g = np.random.default_rng(seed)
    return dict(a=g.standard_normal((T, c)), b=g.standard_normal((T, c)),
                za=g.standard_normal((T, c)), zb=g.standard_normal((T, c)),
                Ba=g.standard_normal((m, c)) * 0.3, Bb=g.standard_normal((m, c)) * 0.3,
                ka=g.standard_normal((T, dI)), kb=g.standard_normal((T, dI)),
                kza=g.standard_normal((T, dI)), kzb=g.standard_normal((T, dI)),
                kBa=g.standard_normal((m, dI)), kBb=g.standard_normal((m, dI)),
                q=g.standard_normal((T, H, c)), qI=g.standard_normal((T, HI, dI)),
                w=g.standard_normal((T, HI)))


def _run_csa(x, m, k, d_nope, base, tau, overlap=True, rows=None):
    T = x["a"].shape[0]
    ov = (x["b"], x["zb"], x["Bb"]) if overlap else (None, None, None)
    ent = csa.compress(x["a"], x["za"], x["Ba"], m, *ov)
    cache = csa.finalize_kv(ent, 0, m, d_nope, base, "f32", "f32")
    kov = (x["kb"], x["kzb"], x["kBb"]) if overlap else (None, None, None)
    keys = csa.finalize_keys(csa.compress(x["ka"], x["kza"], x["kBa"], m, *kov), "f32")
    rows = np.arange(T) if rows is None else rows
    return csa.csa_rows(rows, rows, x["q"][rows], x["qI"][rows], x["w"][rows], cache, keys,
                        m, k, d_nope, base, tau), cache


def test_m1_full_topk_is_causal_attention_sdpa():
    """m = 1, no overlap, k >= T: CSA is textbook causal MQA attention with
    K_t = RoPE_t(a_t), V_t = a_t[:d_nope], checked with torch's
    scaled_dot_product_attention (fp64, CPU) and complex-form RoPE."""
    T, c, d_nope, H = 40, 16, 8, 3
    x = _tiny_inputs(T, c, d_nope, H, 2, 8, 1, 110)
    x["Ba"] = np.zeros((1, c))
    res, _ = _run_csa(x, 1, T, d_nope, 10000.0, 0.25, overlap=False)
    # the cache stores fp32: round K and V as stored
    Kt = torch.as_tensor(complex_rope(x["a"], np.arange(T), d_nope, 10000.0)).float().double()
    Vt = Kt[:, :d_nope]
    Q = torch.as_tensor(complex_rope(x["q"], np.arange(T)[:, None], d_nope, 10000.0))
    ref = torch.nn.functional.scaled_dot_product_attention(
        Q.permute(1, 0, 2), Kt[None].expand(H, T, c), Vt[None].expand(H, T, d_nope),
        is_causal=True, scale=0.25).permute(1, 0, 2).numpy()
    assert np.allclose(res["o"], ref, atol=1e-12)


def test_full_topk_equals_dense_attention():
    """k >= number of entries: CSA equals dense (HCA-form) attention over the
    same compressed cache with block-granular causality."""
    T, c, d_nope, H, m = 64, 8, 4, 2, 4
    x = _tiny_inputs(T, c, d_nope, H, 2, 4, m, 111)
    res, cache = _run_csa(x, m, T // m, d_nope, 10000.0, 0.35)
    o, lse = csa.hca_rows(np.arange(T), x["q"], cache, m, d_nope, 10000.0, 0.35)
    assert np.allclose(res["o"], o, atol=1e-13)
    assert np.allclose(res["lse"][m - 1:], lse[m - 1:], atol=1e-13)


def test_whole_path_matches_bruteforce():
    T, c, d_nope, H, HI, dI, m, k = 36, 6, 2, 2, 2, 3, 4, 3
    x = _tiny_inputs(T, c, d_nope, H, HI, dI, m, 112)
    res, _ = _run_csa(x, m, k, d_nope, 100.0, 0.4)
    L = lambda v: v.tolist()
    ent = brute.compress(L(x["a"]), L(x["za"]), L(x["Ba"]), m, L(x["b"]), L(x["zb"]), L(x["Bb"]))
    kv = [brute.rotate(e, i * m + m - 1, d_nope, 100.0) for i, e in enumerate(ent)]
    kv = [list(np.float32(v).astype(np.float64)) for v in kv]
    keys = brute.compress(L(x["ka"]), L(x["kza"]), L(x["kBa"]), m, L(x["kb"]), L(x["kzb"]), L(x["kBb"]))
    keys = [list(np.float32(v).astype(np.float64)) for v in keys]
    for t in range(T):
        n = (t + 1) // m
        I = brute.scores(L(x["qI"][t]), L(x["w"][t]), keys, n)
        sel = brute.topk(I, k)
        assert list(res["idx"][t]) == sel
        qr = [brute.rotate(qh, t, d_nope, 100.0) for qh in L(x["q"][t])]
        o, lse = brute.attend(qr, kv, [e[:d_nope] for e in kv], sel, 0.4)
        assert np.allclose(res["o"][t], o, atol=1e-12)
        if n:
            assert np.allclose(res["lse"][t], lse, atol=1e-12)
        else:
            assert np.all(np.isneginf(res["lse"][t]))


def test_causality():
    """Perturbing tokens after t leaves every output at positions <= t."""
    T, c, d_nope, H, m, k, t = 48, 8, 4, 2, 4, 3, 27
    x = _tiny_inputs(T, c, d_nope, H, 2, 4, m, 113)
    base, _ = _run_csa(x, m, k, d_nope, 10000.0, 0.35)
    y = {kk: v.copy() for kk, v in x.items()}
    for kk in ("a", "b", "za", "zb", "ka", "kb", "kza", "kzb", "q", "qI", "w"):
        y[kk][t + 1:] += 1.0
    pert, _ = _run_csa(y, m, k, d_nope, 10000.0, 0.35)
    assert np.array_equal(base["idx"][:t + 1], pert["idx"][:t + 1])
    assert np.allclose(base["o"][:t + 1], pert["o"][:t + 1], atol=0)


def test_hca_zero_logits_is_mean_pool_attention():
    """HCA with Z = B = 0: entries are 128-token means; attention over them is
    reproduced by an independent mean-pool + torch softmax formula."""
    m, T, c, d_nope, H = 128, 640, 8, 4, 2
    a = rnd((T, c), 120)
    z = np.zeros((T, c))
    ent = csa.compress(a, z, np.zeros((m, c)), m)
    cache = csa.finalize_kv(ent, 0, m, d_nope, 10000.0, "f32", "f32")
    q = rnd((1, H, c), 121)
    t = T - 1
    o, lse = csa.dense_attention_row(q[0], t, cache, m, d_nope, 10000.0, 0.3)
    pooled = torch.as_tensor(a.reshape(-1, m, c).mean(1))
    Kr = torch.as_tensor(complex_rope(pooled.numpy(), np.arange(T // m) * m + m - 1, d_nope, 10000.0))
    Kr = Kr.to(torch.float32).to(torch.float64)
    qr = torch.as_tensor(complex_rope(q[0], t, d_nope, 10000.0))
    p = torch.softmax(0.3 * qr @ Kr.T, dim=-1)
    assert np.allclose(o, (p @ Kr[:, :d_nope]).numpy(), atol=1e-12)


# ---------------------------------------------------------------- page values

def test_page_values():
    g = json.load(open(GOLDEN))
    m, k, mh = g["csa_m"]["value"], g["csa_topk"]["value"], g["hca_m"]["value"]
    n_csa = int(csa.n_visible((1 << 20) - 1, m))
    assert abs(n_csa - g["csa_entries_at_1M_approx"]["value"]) / n_csa < 0.05
    assert int(csa.n_visible((1 << 20) - 1, mh)) == (1 << 20) // 128
    # entry i sees 2m tokens
    w = csa.compress_weights(np.zeros((3 * m, 1)), np.zeros((m, 1)), m, np.zeros((3 * m, 1)), np.zeros((m, 1)), i=2)
    assert w.shape[0] == g["csa_window_rows"]["value"]
    # split KV bytes: FP8 codes + fp32 scale + BF16 RoPE vs all-BF16
    x = rnd((1, 576), 130)
    cache = csa.finalize_kv(x, 0, m, 512, 10000.0, "fp8", "bf16")
    split_bytes = cache["nope_codes"].nbytes + 4 + 64 * 2
    assert split_bytes == 644
    ratio = split_bytes / (576 * 2)
    assert abs(ratio - g["split_kv_vs_bf16_approx"]["value"]) < 0.1
    assert k == 1024 and m == 4 and mh == 128


# ---------------------------------------------------------------- sliding-window branch

def test_sliding_window_is_banded_causal_attention_sdpa():
    """m = 1 per-token entries (the compressor with one row per window passes
    the token row through), window w: each query attends tokens
    t - w < s <= t; torch's attention with that band as the mask agrees."""
    T, H, dn, dr, w, base, tau = 40, 3, 6, 4, 7, 1e4, 0.3
    c = dn + dr
    a, za = rnd((T, c), 120), rnd((T, c), 121)
    Ba = rnd((1, c), 122, 0.1)
    ent = csa.compress(a, za, Ba, 1)                 # m = 1: the token rows themselves
    assert np.allclose(ent, a, atol=1e-15)
    cache = csa.finalize_kv(ent, 0, 1, dn, base, "f32", "f32")
    q = rnd((T, H, c), 123)
    o = np.zeros((T, H, dn))
    lse = np.zeros((T, H))
    for t in range(T):
        o[t], lse[t] = csa.dense_attention_row(q[t], t, cache, 1, dn, base, tau, window=w)
    qr = np.stack([csa.rope_query(q[t], t, dn, base) for t in range(T)])      # [T, H, c]
    K = torch.as_tensor(cache["k"])[None, None]                                # [1, 1, T, c]
    V = torch.as_tensor(cache["v"])[None, None]
    i, j = np.arange(T)[:, None], np.arange(T)[None, :]
    band = torch.as_tensor((j <= i) & (j > i - w))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.as_tensor(qr).permute(1, 0, 2)[None], K.expand(1, H, T, c), V.expand(1, H, T, dn),
        attn_mask=band, scale=tau)[0].permute(1, 0, 2).numpy()
    assert np.allclose(o, ref, atol=1e-12)
    # a window at least as long as the prefix is plain dense attention
    for t in (0, 5, T - 1):
        od, ld = csa.dense_attention_row(q[t], t, cache, 1, dn, base, tau)
        ow, lw = csa.dense_attention_row(q[t], t, cache, 1, dn, base, tau, window=T)
        assert np.allclose(od, ow, atol=1e-15) and np.allclose(ld, lw, atol=1e-15)


def test_lse_merge_is_one_softmax_over_the_union():
    """The merge of a compressed branch (selected entries) and a window branch
    (recent tokens) equals attention over both key sets at once (written out
    by brute force over the concatenated keys)."""
    H, c, dv, tau = 4, 9, 5, 0.35
    q = rnd((H, c), 130)
    K1, K2 = rnd((20, c), 131), rnd((11, c), 132)
    sel1, sel2 = np.array([0, 3, 4, 9, 15, 19]), np.arange(11)
    o1, l1 = csa.attend(q, K1, K1[:, :dv], sel1, tau)
    o2, l2 = csa.attend(q, K2, K2[:, :dv], sel2, tau)
    om, lm = csa.lse_merge(o1, l1, o2, l2)
    Ku = np.concatenate([K1[sel1], K2[sel2]], 0)
    ob, lb = brute.attend(q.tolist(), Ku.tolist(), Ku[:, :dv].tolist(), list(range(len(Ku))), tau)
    assert np.allclose(om, ob, atol=1e-13) and np.allclose(lm, lb, atol=1e-13)
    # one branch empty (no visible entry yet): the other branch unchanged
    oe, le = csa.attend(q, K1, K1[:, :dv], [-1], tau)
    o, lse = csa.lse_merge(oe, le, o2, l2)
    assert np.array_equal(o, o2) and np.allclose(lse, l2, atol=0)
    o, lse = csa.lse_merge(oe, le, oe, le)
    assert not o.any() and np.isneginf(lse).all()
