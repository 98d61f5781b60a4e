"""Thin ctypes binding of libcsa.so (the C ABI in include/csa.h).

Argument marshalling only: torch tensors supply device memory and the
current HIP stream; every step of the path runs in the library's HIP
kernels.  Loading fails loudly when the library is missing; there is no
fallback implementation.
"""
import ctypes
import os

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libcsa.so")

F32, BF16, FP8E4M3, MXFP4 = 0, 1, 2, 3
FMT = {"f32": F32, "bf16": BF16, "fp8": FP8E4M3, "mxfp4": MXFP4}
STATUS = {0: "CSA_OK", 1: "CSA_ERR_INVALID_ARG", 2: "CSA_ERR_ALIGNMENT", 3: "CSA_ERR_UNSUPPORTED",
          4: "CSA_ERR_WORKSPACE", 5: "CSA_ERR_CAPACITY", 6: "CSA_ERR_HIP"}
OP_INDEX_TOPK_PREFILL, OP_INDEX_TOPK_DECODE = 1, 2
OP_SPARSE_ATTN_PREFILL, OP_SPARSE_ATTN_DECODE = 3, 4
OP_DENSE_ATTN_PREFILL, OP_DENSE_ATTN_DECODE = 5, 6


class CacheDesc(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("overlap", ctypes.c_int32), ("d_nope", ctypes.c_int32),
                ("d_rope", ctypes.c_int32), ("in_dtype", ctypes.c_int32), ("nope_dtype", ctypes.c_int32),
                ("rope_dtype", ctypes.c_int32), ("page_size", ctypes.c_int32), ("rope_base", ctypes.c_double),
                ("capacity", ctypes.c_int64), ("pool_pages", ctypes.c_int64)]


class Cache(ctypes.Structure):
    _fields_ = [("nope", ctypes.c_void_p), ("scale", ctypes.c_void_p), ("rope", ctypes.c_void_p),
                ("ring", ctypes.c_void_p), ("block_table", ctypes.c_void_p)]


class IndexDesc(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("dim", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("qk_dtype", ctypes.c_int32), ("key_dtype", ctypes.c_int32), ("score_dtype", ctypes.c_int32),
                ("m", ctypes.c_int32), ("page_size", ctypes.c_int32), ("capacity", ctypes.c_int64),
                ("pool_pages", ctypes.c_int64)]


class AttnDesc(ctypes.Structure):
    _fields_ = [("n_heads", ctypes.c_int32), ("d_nope", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("q_dtype", ctypes.c_int32), ("o_dtype", ctypes.c_int32), ("nope_dtype", ctypes.c_int32),
                ("rope_dtype", ctypes.c_int32), ("m", ctypes.c_int32), ("window", ctypes.c_int32),
                ("qk_mode", ctypes.c_int32), ("rope_base", ctypes.c_double), ("capacity", ctypes.c_int64),
                ("page_size", ctypes.c_int32), ("reserved", ctypes.c_int32), ("pool_pages", ctypes.c_int64)]


class DecodeInputs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("a", "b", "za", "zb", "Ba", "Bb", "ka", "kb", "kza", "kzb", "kBa", "kBb",
                                               "q", "qI", "w")]


EXPORTS = ["csa_compress_prefill", "csa_compress_decode", "csa_index_topk_prefill", "csa_index_topk_decode",
           "csa_sparse_attn_prefill", "csa_sparse_attn_decode", "csa_sparse_attn_decode_noalloc",
           "hca_dense_attn_prefill", "hca_dense_attn_decode", "csa_decode_step", "csa_decode_step_workspace_bytes", "csa_lse_merge",
           "csa_compress_project_prefill", "csa_compress_project_workspace_bytes",
           "csa_workspace_bytes", "csa_status_string", "csa_last_error", "csa_version"]
NOALLOC_SCRATCH_BYTES = 64 << 20

_lib = None


def lib():
    """The loaded library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: run `python -m compressed_sparse_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        P, I, I64, F, SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
        sig = {
            "csa_compress_prefill": [P, I, I, I64, P, P, P, P, P, P, P, P],
            "csa_compress_decode": [P, I, P, P, P, P, P, P, P, P, P],
            "csa_index_topk_prefill": [P, I, I, I64, P, P, P, I, P, P, P, SZ, P],
            "csa_index_topk_decode": [P, I, P, P, P, P, I, P, P, P, SZ, P],
            "csa_sparse_attn_prefill": [P, I, I, I64, P, P, P, I, F, P, P, P, SZ, P],
            "csa_sparse_attn_decode": [P, I, P, P, P, P, I, F, P, P, P, SZ, P],
            "csa_sparse_attn_decode_noalloc": [P, I, P, P, P, P, I, F, P, P, P],
            "hca_dense_attn_prefill": [P, I, I, I64, P, P, F, P, P, P, SZ, P],
            "hca_dense_attn_decode": [P, I, P, P, P, F, P, P, P, SZ, P],
            "csa_workspace_bytes": [I, P, I, I, I64, I],
            "csa_decode_step": [P, P, P, P, P, P, I, P, P, I, F, P, P, P, P, P, SZ, P],
            "csa_decode_step_workspace_bytes": [P, P, I, I],
            "csa_lse_merge": [I, I, I, I, P, P, P, P, P, P, P],
            "csa_compress_project_prefill": [P, I, I, I64, P, I, P, P, P, P, P, SZ, P],
            "csa_compress_project_workspace_bytes": [P, I, I, I64],
        }
        for name, args in sig.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = SZ if name.endswith("workspace_bytes") else I
        L.csa_status_string.restype = ctypes.c_char_p
        L.csa_status_string.argtypes = [I]
        L.csa_last_error.restype = ctypes.c_char_p
        L.csa_version.restype = I
        _lib = L
    return _lib


class CsaError(RuntimeError):
    def __init__(self, status, msg):
        super().__init__(f"{STATUS.get(status, status)}: {msg}")
        self.status = status


def _check(st):
    if st != 0:
        raise CsaError(st, lib().csa_last_error().decode())


def ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def stream_ptr(stream=None):
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


# ---------------------------------------------------------------------------
# descriptors and caches
# ---------------------------------------------------------------------------

def cache_desc(m, overlap, d_nope, d_rope, in_fmt, nope_fmt, rope_fmt, capacity, base=10000.0, page_size=0,
               pool_pages=0):
    return CacheDesc(m, int(overlap), d_nope, d_rope, FMT[in_fmt], FMT[nope_fmt],
                     FMT.get(rope_fmt, F32), page_size, base, capacity, pool_pages)


class KVCache:
    """Device buffers of a compressed cache for B sequences (torch tensors).

    Contiguous (desc.page_size == 0): nope [B][cap][..], scale [B][cap](..),
    rope [B][cap][d_rope].  Paged: the same per row of a pool, [pool_pages]
    [page_size][..], and block_table int32 [B][cap / page_size] (the caller's
    mapping; identity-free: any page order)."""

    def __init__(self, desc: CacheDesc, B, device="cuda", block_table=None):
        self.desc, self.B = desc, B
        cap, dn, dr = desc.capacity, desc.d_nope, desc.d_rope
        c = dn + dr
        nf = desc.nope_dtype
        paged = desc.page_size > 0
        lead = (desc.pool_pages, desc.page_size) if paged else (B, cap)
        if paged:
            if block_table is None or tuple(block_table.shape) != (B, cap // desc.page_size) \
                    or block_table.dtype != torch.int32:
                raise ValueError("a paged cache needs an int32 block_table [B][capacity / page_size]")
        elif block_table is not None:
            raise ValueError("block_table given for a contiguous cache")
        self.block_table = block_table
        if nf == MXFP4:
            self.nope = torch.zeros(lead + (dn // 2,), dtype=torch.uint8, device=device)
            self.scale = torch.zeros(lead + (dn // 32,), dtype=torch.uint8, device=device)
        else:
            dt = {F32: torch.float32, BF16: torch.bfloat16, FP8E4M3: torch.uint8}[nf]
            self.nope = torch.zeros(lead + (dn,), dtype=dt, device=device)
            self.scale = torch.zeros(lead, dtype=torch.float32, device=device) if nf == FP8E4M3 else None
        rdt = torch.float32 if desc.rope_dtype == F32 else torch.bfloat16
        self.rope = torch.zeros(lead + (dr,), dtype=rdt, device=device) if dr else None
        R = 2 * desc.m if desc.overlap else desc.m
        NT = 4 if desc.overlap else 2
        self.ring = torch.zeros((B, R, NT, c), dtype=torch.float32, device=device)

    def struct(self):
        return Cache(self.nope.data_ptr(), None if self.scale is None else self.scale.data_ptr(),
                     None if self.rope is None else self.rope.data_ptr(), self.ring.data_ptr(),
                     None if self.block_table is None else self.block_table.data_ptr())

    def seq_view(self, b):
        """Sequence b alone, as a one-sequence cache over the same memory (its
        ring and block-table row; for a contiguous cache its rows)."""
        v = object.__new__(KVCache)
        v.desc, v.B = self.desc, 1
        v.ring = self.ring[b:b + 1]
        if self.desc.page_size:
            v.nope, v.scale, v.rope = self.nope, self.scale, self.rope
            v.block_table = self.block_table[b:b + 1]
        else:
            v.nope = self.nope[b:b + 1]
            v.scale = None if self.scale is None else self.scale[b:b + 1]
            v.rope = None if self.rope is None else self.rope[b:b + 1]
            v.block_table = None
        return v

    def logical(self, t):
        """One of nope / scale / rope in sequence order, [B][cap][..] (a gather of
        the pages for a paged cache; the tensor itself when contiguous)."""
        if self.desc.page_size == 0 or t is None:
            return t
        pages = t[self.block_table.long()]  # [B][cap / page][page][..]
        return pages.reshape((self.B, self.desc.capacity) + tuple(t.shape[2:]))


# ---------------------------------------------------------------------------
# entry points
# ---------------------------------------------------------------------------

def compress_prefill(cache: KVCache, pos0, a, za, Ba, b=None, zb=None, Bb=None, stream=None):
    B, T = a.shape[0], a.shape[1]
    cs = cache.struct()
    _check(lib().csa_compress_prefill(ctypes.byref(cache.desc), B, T, pos0, ptr(a), ptr(b), ptr(za), ptr(zb),
                                      ptr(Ba), ptr(Bb), ctypes.byref(cs), stream_ptr(stream)))


def compress_decode(cache: KVCache, pos, a, za, Ba, b=None, zb=None, Bb=None, stream=None):
    cs = cache.struct()
    _check(lib().csa_compress_decode(ctypes.byref(cache.desc), a.shape[0], ptr(pos), ptr(a), ptr(b), ptr(za),
                                     ptr(zb), ptr(Ba), ptr(Bb), ctypes.byref(cs), stream_ptr(stream)))


def pack_projection_weights(W):
    """The library's weight layout for compress_project_prefill: W is a dict of
    [d_model, c] matrices aKV, aZ (and bKV, bZ); row j*NT + u of the result
    is column j of matrix u in the order aKV, aZ, bKV, bZ."""
    names = [n for n in ("aKV", "aZ", "bKV", "bZ") if n in W]
    return torch.stack([W[n].t() for n in names], 1).reshape(-1, W[names[0]].shape[0]).contiguous()


def project_workspace_bytes(desc, B, T, pos0=0):
    return lib().csa_compress_project_workspace_bytes(ctypes.byref(desc), B, T, pos0)


def compress_project_prefill(cache: KVCache, pos0, X, W, Ba, Bb=None, ws=None, stream=None):
    """X [B][T][d_model] BF16 hidden states, W [NT * c][d_model] BF16 packed
    projection rows (row j*NT + u: column j of W^{aKV}, W^{aZ}, W^{bKV}, W^{bZ})."""
    B, T, d = X.shape
    if ws is None:
        ws = workspace(project_workspace_bytes(cache.desc, B, T, pos0), X.device)
    cs = cache.struct()
    _check(lib().csa_compress_project_prefill(ctypes.byref(cache.desc), B, T, pos0, ptr(X), d, ptr(W), ptr(Ba),
                                              ptr(Bb), ctypes.byref(cs), ptr(ws), ws.numel(), stream_ptr(stream)))


def index_desc(n_heads, dim, q_fmt, qk_fmt, key_fmt, score_fmt, m, capacity, page_size=0, pool_pages=0):
    return IndexDesc(n_heads, dim, FMT[q_fmt], FMT[qk_fmt], FMT[key_fmt], FMT[score_fmt], m, page_size, capacity,
                     pool_pages)


def workspace_bytes(op, desc, B, T, pos0=0, k=0):
    return lib().csa_workspace_bytes(op, ctypes.byref(desc), B, T, pos0, k)


def workspace(nbytes, device="cuda"):
    return torch.empty(max(int(nbytes), 256), dtype=torch.uint8, device=device)


def index_topk_prefill(desc, keys: KVCache, pos0, qI, w, k, idx, scores=None, ws=None, stream=None):
    B, T = qI.shape[0], qI.shape[1]
    need = workspace_bytes(OP_INDEX_TOPK_PREFILL, desc, B, T, pos0, k)
    if ws is None:
        ws = workspace(need, qI.device)
    cs = keys.struct()
    _check(lib().csa_index_topk_prefill(ctypes.byref(desc), B, T, pos0, ptr(qI), ptr(w), ctypes.byref(cs), k,
                                        ptr(idx), ptr(scores), ptr(ws), ws.numel(), stream_ptr(stream)))


def index_topk_decode(desc, keys: KVCache, pos, qI, w, k, idx, scores=None, ws=None, stream=None):
    B = qI.shape[0]
    need = workspace_bytes(OP_INDEX_TOPK_DECODE, desc, B, 1, 0, k)
    if ws is None:
        ws = workspace(need, qI.device)
    cs = keys.struct()
    _check(lib().csa_index_topk_decode(ctypes.byref(desc), B, ptr(pos), ptr(qI), ptr(w), ctypes.byref(cs), k,
                                       ptr(idx), ptr(scores), ptr(ws), ws.numel(), stream_ptr(stream)))


def attn_desc(n_heads, d_nope, d_rope, q_fmt, o_fmt, nope_fmt, rope_fmt, m, capacity, base=10000.0, window=0,
              page_size=0, pool_pages=0, qk="bf16"):
    """qk: "bf16" (the query's own format) or "fp8" (the non-RoPE query dims
    rounded to MXFP8 and multiplied with the FP8 cache codes in FP8)."""
    qk_mode = {"bf16": 0, "fp8": FP8E4M3}[qk]
    return AttnDesc(n_heads, d_nope, d_rope, FMT[q_fmt], FMT[o_fmt], FMT[nope_fmt], FMT.get(rope_fmt, F32),
                    m, window, qk_mode, base, capacity, page_size, 0, pool_pages)


def _ws(op, desc, B, T, pos0, k, ws, device):
    need = workspace_bytes(op, desc, B, T, pos0, k)
    if ws is None:
        ws = workspace(need, device)
    return ws


def sparse_attn_prefill(desc, kv: KVCache, pos0, q, idx, scale, o, lse=None, ws=None, stream=None):
    B, T = q.shape[0], q.shape[1]
    k = idx.shape[-1]
    ws = _ws(OP_SPARSE_ATTN_PREFILL, desc, B, T, pos0, k, ws, q.device)
    cs = kv.struct()
    _check(lib().csa_sparse_attn_prefill(ctypes.byref(desc), B, T, pos0, ptr(q), ctypes.byref(cs), ptr(idx), k,
                                         scale, ptr(o), ptr(lse), ptr(ws), ws.numel(), stream_ptr(stream)))


def sparse_attn_decode(desc, kv: KVCache, pos, q, idx, scale, o, lse=None, ws=None, stream=None):
    B = q.shape[0]
    k = idx.shape[-1]
    ws = _ws(OP_SPARSE_ATTN_DECODE, desc, B, 1, 0, k, ws, q.device)
    cs = kv.struct()
    _check(lib().csa_sparse_attn_decode(ctypes.byref(desc), B, ptr(pos), ptr(q), ctypes.byref(cs), ptr(idx), k,
                                        scale, ptr(o), ptr(lse), ptr(ws), ws.numel(), stream_ptr(stream)))


def sparse_attn_decode_noalloc(desc, kv: KVCache, pos, q, idx, scale, o, lse=None, stream=None):
    """csa_sparse_attn_decode with the split partials in the library's own
    device scratch (no workspace argument)."""
    cs = kv.struct()
    _check(lib().csa_sparse_attn_decode_noalloc(ctypes.byref(desc), q.shape[0], ptr(pos), ptr(q), ctypes.byref(cs),
                                                ptr(idx), idx.shape[-1], scale, ptr(o), ptr(lse), stream_ptr(stream)))


def decode_step_workspace_bytes(idesc, adesc, B, k):
    return lib().csa_decode_step_workspace_bytes(ctypes.byref(idesc), ctypes.byref(adesc), B, k)


def decode_step(kv: KVCache, keys: KVCache, idesc, adesc, pos, x, prm, k, scale, idx, o, lse=None, scores=None,
                ws=None, stream=None):
    """csa_decode_step: both compressors, indexer + top-k and sparse
    attention of one CSA decode step.  x: the step's rows (a, za, b, zb, ka,
    kza, kb, kzb, q, qI, w); prm: Ba, Bb, kBa, kBb."""
    B = x["q"].shape[0]
    if ws is None:
        ws = workspace(decode_step_workspace_bytes(idesc, adesc, B, k), x["q"].device)
    g = lambda d, n: None if d.get(n) is None else d[n].data_ptr()
    inp = DecodeInputs(g(x, "a"), g(x, "b"), g(x, "za"), g(x, "zb"), g(prm, "Ba"), g(prm, "Bb"), g(x, "ka"), g(x, "kb"),
                       g(x, "kza"), g(x, "kzb"), g(prm, "kBa"), g(prm, "kBb"), g(x, "q"), g(x, "qI"), g(x, "w"))
    kvs, ks = kv.struct(), keys.struct()
    _check(lib().csa_decode_step(ctypes.byref(kv.desc), ctypes.byref(kvs), ctypes.byref(keys.desc), ctypes.byref(ks),
                                 ctypes.byref(idesc), ctypes.byref(adesc), B, ptr(pos), ctypes.byref(inp), k, scale,
                                 ptr(idx), ptr(scores), ptr(o), ptr(lse), ptr(ws), ws.numel(), stream_ptr(stream)))


def lse_merge(o1, lse1, o2, lse2, o, lse=None, stream=None):
    """csa_lse_merge: one softmax over the union of two attention results'
    keys from their (o, lse) pairs; o [..., H, d_v] (may alias o1 or o2)."""
    H, dv = o1.shape[-2], o1.shape[-1]
    rows = o1.numel() // (H * dv)
    fmt = F32 if o1.dtype == torch.float32 else BF16
    _check(lib().csa_lse_merge(rows, H, dv, fmt, ptr(o1), ptr(lse1), ptr(o2), ptr(lse2), ptr(o), ptr(lse),
                               stream_ptr(stream)))


def dense_attn_prefill(desc, kv: KVCache, pos0, q, scale, o, lse=None, ws=None, stream=None):
    B, T = q.shape[0], q.shape[1]
    ws = _ws(OP_DENSE_ATTN_PREFILL, desc, B, T, pos0, 0, ws, q.device)
    cs = kv.struct()
    _check(lib().hca_dense_attn_prefill(ctypes.byref(desc), B, T, pos0, ptr(q), ctypes.byref(cs), scale,
                                        ptr(o), ptr(lse), ptr(ws), ws.numel(), stream_ptr(stream)))


def dense_attn_decode(desc, kv: KVCache, pos, q, scale, o, lse=None, ws=None, stream=None):
    B = q.shape[0]
    ws = _ws(OP_DENSE_ATTN_DECODE, desc, B, 1, 0, 0, ws, q.device)
    cs = kv.struct()
    _check(lib().hca_dense_attn_decode(ctypes.byref(desc), B, ptr(pos), ptr(q), ctypes.byref(cs), scale,
                                       ptr(o), ptr(lse), ptr(ws), ws.numel(), stream_ptr(stream)))
