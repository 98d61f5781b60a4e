"""Plain fp64 CPU oracle of the CSA / HCA hybrid-attention hot path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the smoke check and the benchmark's
CPU-baseline leg may import this package; the product path never does.

Every function is the plain definition from the pages, evaluated in fp64 with
numpy (a matmul, a sort and elementwise ops are the only library steps), with
no blocking, fusion or reordering beyond what the definition states.  Page
short names used in the citations:

* [CSA/HCA 混注意力]  "从论文出发，逐层剖析 CSA / HCA 混注意力、mHC 残差连接与 Muon
  优化器" (dxhjj.kegongbw.com)
* [三大核心架构创新]  "DeepSeek-V4 技术解析：三大核心架构创新如何突破百万Token上下文
  瓶颈" (chousei-blog.pages.dev)
* [读完这篇]          "读完这篇你就搞懂 DeepSeek v4 了" (ai-engineering-6yk.pages.dev)

Readings where the pages leave a step open are stated at each function; the
full list is kept with the design notes.
"""
import numpy as np

from . import formats as F


# ---------------------------------------------------------------------------
# a1 / a2: compressor
# ---------------------------------------------------------------------------

def compress(a, za, Ba, m, b=None, zb=None, Bb=None, i0=0, i1=None, tok0=0):
    """Compressed KV entries i in [i0, i1), fp64, before RoPE.

    [CSA/HCA 混注意力] §1.1 工程细节: entry i is formed from the m tokens of the
    current window (C^a) and the m tokens of the previous window (C^b), so it
    sees 2m tokens.  [三大核心架构创新] §2.2 step 1: learned compression weights
    Z.  [读完这篇] §三 (CSA 步骤一): each dimension is weighted on its own, two
    consecutive groups are joined, parameters are 4 W matrices and 2 B bias
    matrices.  HCA ([CSA/HCA 混注意力] §1.2; [读完这篇] §三 HCA 步骤简化) uses a
    single window of m' tokens and no C^b (call with b = zb = Bb = None).

    Reading: for channel j, one softmax runs jointly over the 2m logits
    za[im+r, j] + Ba[r, j] and zb[(i-1)m+r, j] + Bb[r, j] (r < m); the entry is
    the softmax-weighted sum of the matching a and b rows.  Entry 0 has no
    previous window: its softmax covers the m C^a rows only.

    a, za, b, zb: [n_tok, c] rows of tokens tok0 .. tok0+n_tok-1.
    Ba, Bb: [m, c].  Returns [i1 - i0, c]."""
    a = np.asarray(a, np.float64)
    za = np.asarray(za, np.float64)
    Ba = np.asarray(Ba, np.float64)
    overlap = b is not None
    if i1 is None:
        i1 = (tok0 + a.shape[0]) // m
    ii = np.arange(i0, i1)
    r = np.arange(m)
    rows_a = ii[:, None] * m + r[None, :] - tok0                 # [n, m]
    vals = a[rows_a]                                             # [n, m, c]
    logits = za[rows_a] + Ba[None]                               # [n, m, c]
    if overlap:
        b = np.asarray(b, np.float64)
        zb = np.asarray(zb, np.float64)
        Bb = np.asarray(Bb, np.float64)
        has_prev = ii >= 1
        rows_b = (ii[:, None] - 1) * m + r[None, :] - tok0
        rows_b = np.where(has_prev[:, None], rows_b, 0)
        vb = b[rows_b]
        lb = zb[rows_b] + Bb[None]
        # entry 0: the C^b terms are absent (weight exactly zero)
        lb = np.where(has_prev[:, None, None], lb, -np.inf)
        vb = np.where(has_prev[:, None, None], vb, 0.0)
        vals = np.concatenate([vals, vb], axis=1)
        logits = np.concatenate([logits, lb], axis=1)
    mx = np.max(logits, axis=1, keepdims=True)
    wts = np.exp(logits - mx)
    wts = wts / np.sum(wts, axis=1, keepdims=True)
    return np.sum(wts * vals, axis=1)


def project(X, W):
    """One of the compressor's input projections from hidden states, fp64:
    X [n_tok, d_model] times W [d_model, c].  [读完这篇] §三 压缩机制 names the
    compressor's learnable parameters: four projection matrices W^{aKV},
    W^{bKV}, W^{aZ}, W^{bZ} (C^a = H W^{aKV}, C^b = H W^{bKV}, Z^a = H W^{aZ},
    Z^b = H W^{bZ}) and the two biases B^a, B^b."""
    return np.asarray(X, np.float64) @ np.asarray(W, np.float64)


def compress_from_hidden(X, W, Ba, m, Bb=None, i0=0, i1=None, tok0=0):
    """Entries from hidden states: the four projections (W: dict with keys
    aKV, aZ and, overlapped, bKV, bZ; each [d_model, c]) in fp64, then
    compress() on them.  The projections are not rounded to any storage
    format between the two steps (reading: they never leave the kernel)."""
    a, za = project(X, W["aKV"]), project(X, W["aZ"])
    b = project(X, W["bKV"]) if "bKV" in W else None
    zb = project(X, W["bZ"]) if "bZ" in W else None
    return compress(a, za, Ba, m, b, zb, Bb, i0=i0, i1=i1, tok0=tok0)


def compress_weights(za, Ba, m, zb=None, Bb=None, i=0, tok0=0):
    """The per-channel softmax weights of entry i, shape [rows, c] (rows = m,
    or 2m for an overlapped entry with i >= 1); exposed for the row-sum pin."""
    za = np.asarray(za, np.float64)
    rows = np.arange(m) + i * m - tok0
    logits = [za[rows] + np.asarray(Ba, np.float64)]
    if zb is not None and i >= 1:
        logits.append(np.asarray(zb, np.float64)[rows - m] + np.asarray(Bb, np.float64))
    L = np.concatenate(logits, axis=0)
    w = np.exp(L - L.max(axis=0, keepdims=True))
    return w / w.sum(axis=0, keepdims=True)


# ---------------------------------------------------------------------------
# a3: entry finalisation (RoPE + storage formats)
# ---------------------------------------------------------------------------

def rope(x, pos, d_nope, base):
    """Rotate the last (c - d_nope) dims of x by position `pos`.

    [CSA/HCA 混注意力] §1.4 存储格式混 names RoPE dims inside each entry.
    Reading: the RoPE dims are the last d_rope dims; adjacent pairs
    (d_nope+2p, d_nope+2p+1) turn by pos * base^(-2p/d_rope) (the original
    rotary definition).  x: [..., c]; pos broadcasts against x.shape[:-1]."""
    x = np.array(x, dtype=np.float64, copy=True)
    d_rope = x.shape[-1] - d_nope
    if d_rope == 0:
        return x
    p = np.arange(d_rope // 2, dtype=np.float64)
    theta = base ** (-2.0 * p / d_rope)
    ang = np.asarray(pos, dtype=np.float64)[..., None] * theta
    c, s = np.cos(ang), np.sin(ang)
    x0 = x[..., d_nope::2].copy()
    x1 = x[..., d_nope + 1::2].copy()
    x[..., d_nope::2] = x0 * c - x1 * s
    x[..., d_nope + 1::2] = x0 * s + x1 * c
    return x


def entry_position(i, m):
    """Reading: entry i is rotated at the position of the last token it
    covers, im + m - 1 (the step at which it becomes visible)."""
    return np.asarray(i) * m + m - 1


def store_format(x, fmt):
    """Round to a storage format; returns (decoded fp64, extra) where extra
    holds codes/scales for the quantised formats."""
    if fmt == "f32":
        return F.to_f32(x), None
    if fmt == "bf16":
        return F.to_bf16(x), None
    if fmt == "fp8":
        v, codes, s = F.fp8_entry_quantize(x)
        return v, (codes, s)
    if fmt == "mxfp4":
        v, codes, sc = F.mxfp4_quantize(x)
        return v, (codes, sc)
    raise ValueError(fmt)


def finalize_kv(entries, i0, m, d_nope, base, nope_fmt, rope_fmt):
    """Entries [n, c] (pre-RoPE, first index i0) -> the cache as stored.

    [CSA/HCA 混注意力] §1.4 存储格式混: RoPE dims in BF16, the rest in FP8.
    Reading: FP8 uses one fp32 scale per entry over its non-RoPE dims
    (amax / 448), RNE with saturation; RoPE dims are rotated, then rounded.
    Returns dict(k=[n, c] decoded key, v=[n, d_nope] decoded value part,
    nope_codes, scale, rope) with codes only for the quantised formats."""
    pos = entry_position(np.arange(i0, i0 + entries.shape[0]), m)
    x = rope(entries, pos, d_nope, base)
    nope, extra = store_format(x[:, :d_nope], nope_fmt)
    rp, _ = store_format(x[:, d_nope:], rope_fmt)
    out = dict(k=np.concatenate([nope, rp], axis=1), v=nope, rope=rp,
               exact=x)
    if extra is not None:
        out["nope_codes"], out["scale"] = extra
    return out


def finalize_keys(entries, fmt):
    """Indexer keys (no RoPE) in their storage format: f32, bf16, fp8 (one
    fp32 scale per key) or mxfp4 (block-32 E8M0 scales along d_I)."""
    v, extra = store_format(entries, fmt)
    out = dict(k=v, exact=np.asarray(entries, np.float64))
    if extra is not None:
        out["codes"], out["scale"] = extra
    return out


# ---------------------------------------------------------------------------
# a4 / a5: lightning indexer and top-k
# ---------------------------------------------------------------------------

def n_visible(pos, m):
    """Reading (block-granular causality): an entry is visible to the query
    at absolute position pos once its window is complete, i.e. entry i is
    visible iff im + m - 1 <= pos; so n(pos) = floor((pos + 1) / m)."""
    return (np.asarray(pos, dtype=np.int64) + 1) // m


def quantize_query(qI, fmt):
    """Indexer query in the QK format: f32/bf16 pass through the input
    values; mxfp4 quantises each head's d_I vector in blocks of 32."""
    if fmt == "mxfp4":
        return F.mxfp4_quantize(qI)[0]
    return np.asarray(qI, np.float64)


def index_scores(qI, w, K, n, score_fmt="f32"):
    """I[s] = sum_h w[h] * ReLU(qI[h] . K[s]) for s < n.

    [CSA/HCA 混注意力] §LIGHTNING INDEXER: the indexer scores each entry;
    [读完这篇] §三 (CSA 步骤二): same as V3.2 DSA, every token against all
    summaries, weighted per head.  Reading: no scale, no RoPE in the indexer.
    In BF16-score mode the fp64 score is first rounded to fp32 and then to
    BF16 ("scores quantised from FP32 to BF16", §1.4).
    qI: [H_I, d_I] (already in QK format), w: [H_I], K: [N, d_I] decoded."""
    dots = np.asarray(K[:n], np.float64) @ np.asarray(qI, np.float64).T
    I = np.maximum(dots, 0.0) @ np.asarray(w, np.float64)
    if score_fmt == "bf16":
        I = F.to_bf16(F.to_f32(I))
    return I


def topk(I, n, k):
    """Top-k selection over the n visible scores ([CSA/HCA 混注意力] §1.1:
    each query keeps the k most relevant entries).  Readings: equal scores go
    to the lower entry index; the result is listed in ascending index order
    and padded with -1 when n < k."""
    I = np.asarray(I[:n], np.float64)
    order = np.lexsort((np.arange(n), -I))
    sel = np.sort(order[:min(k, n)])
    out = np.full(k, -1, dtype=np.int64)
    out[:sel.size] = sel
    return out


# ---------------------------------------------------------------------------
# a6 / a7: attention over compressed entries
# ---------------------------------------------------------------------------

def attend(q_rot, K, V, sel, tau):
    """Softmax attention of one query's H heads over the entries `sel`.

    All heads share one compressed KV (MQA, [读完这篇] §三 CSA 步骤三: KV
    shared).  Readings: the key is the full entry (RoPE dims rotated), the
    value is its non-RoPE part; logits are tau * q.k.  With no entries the
    output is 0 and lse = -inf.  Returns (o [H, d_v], lse [H])."""
    H = q_rot.shape[0]
    sel = np.asarray(sel, dtype=np.int64)
    sel = sel[sel >= 0]
    if sel.size == 0:
        return np.zeros((H, V.shape[1])), np.full(H, -np.inf)
    logits = tau * (np.asarray(q_rot, np.float64) @ np.asarray(K[sel], np.float64).T)
    mx = np.max(logits, axis=1, keepdims=True)
    p = np.exp(logits - mx)
    Z = np.sum(p, axis=1, keepdims=True)
    o = (p / Z) @ np.asarray(V[sel], np.float64)
    lse = mx[:, 0] + np.log(Z[:, 0])
    return o, lse


def attention_probs(q_rot, K, sel, tau):
    """The softmax row of each head over `sel` (for the row-sum pin)."""
    logits = tau * (np.asarray(q_rot, np.float64) @ np.asarray(K[sel], np.float64).T)
    p = np.exp(logits - logits.max(axis=1, keepdims=True))
    return p / p.sum(axis=1, keepdims=True)


def rope_query(q, pos, d_nope, base):
    """The query's RoPE dims turn at its own absolute position."""
    return rope(q, pos, d_nope, base)


def quantize_attn_query(q, d_nope, qk_fmt="bf16"):
    """The attention query in the format of the QK product.

    "bf16": the query as given.  "mxfp8": each head's d_nope non-RoPE dims
    become MXFP8 (blocks of 32 consecutive dims, E4M3 elements, one E8M0
    scale each), so that they meet the FP8 cache codes in FP8; the RoPE dims
    stay as given, like the cache's BF16 RoPE dims.  Reading of
    [CSA/HCA 混注意力] §1.4 存储格式混 (non-RoPE dims in FP8, RoPE dims in
    BF16 for precision): the pages name no query format; MXFP8 is the block
    form that keeps a 32-dim block's dynamic range.  q: [..., H, c]."""
    q = np.asarray(q, np.float64)
    if qk_fmt == "bf16":
        return q
    assert qk_fmt == "mxfp8"
    out = q.copy()
    out[..., :d_nope] = F.mxfp8_quantize(q[..., :d_nope])[0]
    return out


def sparse_attention_row(q, pos, cache, sel, d_nope, base, tau, qk_fmt="bf16"):
    """CSA attention for one query at absolute position `pos` over the
    selected entries (indices outside [0, n) are not used)."""
    q = quantize_attn_query(q, d_nope, qk_fmt)
    return attend(rope_query(q, pos, d_nope, base), cache["k"], cache["v"], sel, tau)


def dense_attention_row(q, pos, cache, m, d_nope, base, tau, window=0, qk_fmt="bf16"):
    """HCA attention for one query: every visible entry, s < n(pos)
    ([CSA/HCA 混注意力] §1.2: dense attention over the 128x shorter
    sequence).  With window w > 0 only the last w visible entries,
    max(0, n - w) <= s < n: with m = 1 over per-token entries this is the
    sliding-window branch over the most recent uncompressed tokens
    ([CSA/HCA 混注意力] §1.3: V4-Flash's sliding-window layers; the
    uncompressed SWA KV of the prefix-cache paragraph)."""
    n = min(int(n_visible(pos, m)), cache["k"].shape[0])
    lo = n - window if 0 < window < n else 0
    q = quantize_attn_query(q, d_nope, qk_fmt)
    return attend(rope_query(q, pos, d_nope, base), cache["k"], cache["v"], np.arange(lo, n), tau)


def lse_merge(o1, lse1, o2, lse2):
    """One softmax over the union of two disjoint key sets, from the two
    partial results: o = (e^lse1 o1 + e^lse2 o2) / (e^lse1 + e^lse2) and
    lse = log(e^lse1 + e^lse2) per head; both empty gives o = 0, lse = -inf.
    Reading: the sliding-window branch and the compressed branch of a layer
    are joined this way (the pages name both branches, not how they join).
    o: [..., H, d_v], lse: [..., H]."""
    lse1 = np.asarray(lse1, np.float64)
    lse2 = np.asarray(lse2, np.float64)
    mx = np.maximum(lse1, lse2)
    safe = np.where(np.isneginf(mx), 0.0, mx)
    w1 = np.exp(lse1 - safe)
    w2 = np.exp(lse2 - safe)
    tot = w1 + w2
    den = np.where(tot > 0, tot, 1.0)
    o = (w1[..., None] * np.asarray(o1, np.float64) + w2[..., None] * np.asarray(o2, np.float64)) / den[..., None]
    lse = np.where(tot > 0, safe + np.log(den), -np.inf)
    return o, lse


# ---------------------------------------------------------------------------
# whole-path helpers (row loops, as plain as the definitions)
# ---------------------------------------------------------------------------

def csa_rows(rows, pos_of_row, q, qI, w, cache, keys, m, k, d_nope, base, tau,
             q_fmt="f32", score_fmt="f32"):
    """For each listed query row: indexer scores -> top-k -> sparse attention.

    q: [R, H, c], qI: [R, H_I, d_I], w: [R, H_I] for the listed rows.
    Returns dict(idx [R, k], o [R, H, d_v], lse [R, H], scores list)."""
    R = len(rows)
    H = q.shape[1]
    dv = cache["v"].shape[1]
    idx = np.full((R, k), -1, dtype=np.int64)
    o = np.zeros((R, H, dv))
    lse = np.zeros((R, H))
    scores = []
    N = keys["k"].shape[0]
    for r in range(R):
        pos = int(pos_of_row[r])
        n = min(int(n_visible(pos, m)), N)
        I = index_scores(quantize_query(qI[r], q_fmt), w[r], keys["k"], n, score_fmt)
        scores.append(I)
        idx[r] = topk(I, n, k)
        o[r], lse[r] = sparse_attention_row(q[r], pos, cache, idx[r], d_nope, base, tau)
    return dict(idx=idx, o=o, lse=lse, scores=scores)


def hca_rows(pos_of_row, q, cache, m, d_nope, base, tau, window=0, qk_fmt="bf16"):
    """Dense HCA attention for a list of query rows."""
    R, H = q.shape[0], q.shape[1]
    dv = cache["v"].shape[1]
    o = np.zeros((R, H, dv))
    lse = np.zeros((R, H))
    for r in range(R):
        o[r], lse[r] = dense_attention_row(q[r], int(pos_of_row[r]), cache, m, d_nope, base, tau, window, qk_fmt)
    return o, lse
