"""Pure-Python brute-force versions of the hot-path definitions, for tiny
inputs only (a second, loop-by-loop evaluation that the vectorised oracle is
pinned against).

TEST INFRASTRUCTURE ONLY.

Each function follows the same definition as its counterpart in
oracle/csa.py but is written with Python floats and explicit loops; top-k is
a full sort of (score, index) pairs.  Nothing here is shared with csa.py.
"""
import math


def compress(a, za, Ba, m, b=None, zb=None, Bb=None):
    """a, za, b, zb: lists of token rows (lists of floats); returns the list
    of entries for every complete window."""
    T = len(a)
    c = len(a[0])
    out = []
    for i in range(T // m):
        ent = []
        for j in range(c):
            terms = []                       # (logit, value)
            for r in range(m):
                t = i * m + r
                terms.append((za[t][j] + Ba[r][j], a[t][j]))
            if b is not None and i > 0:
                for r in range(m):
                    t = (i - 1) * m + r
                    terms.append((zb[t][j] + Bb[r][j], b[t][j]))
            mx = max(l for l, _ in terms)
            num = sum(math.exp(l - mx) * v for l, v in terms)
            den = sum(math.exp(l - mx) for l, _ in terms)
            ent.append(num / den)
        out.append(ent)
    return out


def matvec_rows(X, W):
    """Rows of X (lists) times W (d_model x c, lists): explicit dot products."""
    d, c = len(W), len(W[0])
    return [[sum(x[k] * W[k][j] for k in range(d)) for j in range(c)] for x in X]


def compress_from_hidden(X, W, Ba, m, Bb=None):
    """The four projections as explicit dot products, then compress()."""
    a, za = matvec_rows(X, W["aKV"]), matvec_rows(X, W["aZ"])
    if "bKV" in W:
        return compress(a, za, Ba, m, matvec_rows(X, W["bKV"]), matvec_rows(X, W["bZ"]), Bb)
    return compress(a, za, Ba, m)


def rotate(vec, pos, d_nope, base):
    c = len(vec)
    d_rope = c - d_nope
    out = list(vec)
    for p in range(d_rope // 2):
        th = pos * base ** (-2.0 * p / d_rope)
        x0 = vec[d_nope + 2 * p]
        x1 = vec[d_nope + 2 * p + 1]
        out[d_nope + 2 * p] = x0 * math.cos(th) - x1 * math.sin(th)
        out[d_nope + 2 * p + 1] = x0 * math.sin(th) + x1 * math.cos(th)
    return out


def scores(qI, w, K, n):
    res = []
    for s in range(n):
        tot = 0.0
        for h in range(len(qI)):
            d = sum(qI[h][x] * K[s][x] for x in range(len(K[s])))
            tot += w[h] * (d if d > 0 else 0.0)
        res.append(tot)
    return res


def topk(I, k):
    pairs = sorted(((-I[s], s) for s in range(len(I))))
    sel = sorted(s for _, s in pairs[:k])
    return sel + [-1] * (k - len(sel))


def attend(q, K, V, sel, tau):
    """q: H lists (already rotated); returns (o, lse) as nested lists."""
    o, lse = [], []
    sel = [s for s in sel if s >= 0]
    for h in range(len(q)):
        if not sel:
            o.append([0.0] * len(V[0]))
            lse.append(-math.inf)
            continue
        ls = [tau * sum(q[h][x] * K[s][x] for x in range(len(q[h]))) for s in sel]
        mx = max(ls)
        ex = [math.exp(l - mx) for l in ls]
        Z = sum(ex)
        o.append([sum(ex[i] * V[s][d] for i, s in enumerate(sel)) / Z for d in range(len(V[0]))])
        lse.append(mx + math.log(Z))
    return o, lse
