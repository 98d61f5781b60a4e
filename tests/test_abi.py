"""The C ABI: the library loads, exports every function include/csa.h
declares, and rejects bad arguments on the host before touching the GPU."""
import ctypes
import os
import re

import pytest

from compressed_sparse_amd import binding as cb

HEADER = os.path.join(os.path.dirname(os.path.dirname(__file__)), "include", "csa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?(?:int|size_t|char\s*\*|void)\s*\**\s*(\w+)\s*\(",
                                 text, flags=re.M)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for fn in ("csa_compress_prefill", "csa_compress_decode", "csa_index_topk_prefill", "csa_index_topk_decode",
               "csa_sparse_attn_prefill", "csa_sparse_attn_decode", "hca_dense_attn_prefill",
               "hca_dense_attn_decode", "csa_workspace_bytes"):
        assert fn in names


def test_library_exports_every_declared_symbol():
    L = cb.lib()
    for name in declared_functions():
        assert hasattr(L, name), name
    assert L.csa_version() == 3
    assert L.csa_status_string(0) == b"CSA_OK"
    assert L.csa_status_string(5) == b"CSA_ERR_CAPACITY"


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(cb.CacheDesc) == 56
    assert ctypes.sizeof(cb.Cache) == 40
    assert ctypes.sizeof(cb.IndexDesc) == 48
    assert ctypes.sizeof(cb.AttnDesc) == 72


def fake(addr):
    return ctypes.c_void_p(addr)


def test_host_validation_rejects_before_launch():
    L = cb.lib()
    d = cb.cache_desc(4, True, 32, 32, "f32", "f32", "f32", 100)
    c = cb.Cache(0x1000, 0, 0x2000, 0x3000)
    P = fake(0x4000)
    assert L.csa_compress_prefill(None, 1, 4, 0, P, P, P, P, P, P, ctypes.byref(c), None) == 1
    bad = cb.cache_desc(0, True, 32, 32, "f32", "f32", "f32", 100)
    assert L.csa_compress_prefill(ctypes.byref(bad), 1, 4, 0, P, P, P, P, P, P, ctypes.byref(c), None) == 1
    odd = cb.cache_desc(4, True, 32, 31, "f32", "f32", "f32", 100)
    assert L.csa_compress_prefill(ctypes.byref(odd), 1, 4, 0, P, P, P, P, P, P, ctypes.byref(c), None) == 1
    # misaligned input
    assert L.csa_compress_prefill(ctypes.byref(d), 1, 4, 0, fake(0x4004), P, P, P, P, P, ctypes.byref(c), None) == 2
    # missing overlap tensors
    assert L.csa_compress_prefill(ctypes.byref(d), 1, 4, 0, P, None, P, None, P, None, ctypes.byref(c), None) == 1
    # capacity: 404 tokens -> 101 entries > 100
    assert L.csa_compress_prefill(ctypes.byref(d), 1, 404, 0, P, P, P, P, P, P, ctypes.byref(c), None) == 5
    assert b"capacity" in L.csa_last_error()
    # MXFP4 with RoPE dims is unsupported
    mx = cb.cache_desc(4, True, 64, 2, "f32", "mxfp4", "f32", 100)
    assert L.csa_compress_prefill(ctypes.byref(mx), 1, 4, 0, P, P, P, P, P, P, ctypes.byref(c), None) == 3
    # B == 0 / T == 0 are no-ops
    assert L.csa_compress_prefill(ctypes.byref(d), 0, 4, 0, P, P, P, P, P, P, ctypes.byref(c), None) == 0
    assert L.csa_compress_prefill(ctypes.byref(d), 1, 0, 0, P, P, P, P, P, P, ctypes.byref(c), None) == 0


def test_index_and_attention_validation():
    L = cb.lib()
    idesc = cb.index_desc(16, 64, "bf16", "bf16", "bf16", "f32", 4, 8192)
    keys = cb.Cache(0x1000, 0, 0, 0x2000)
    P = fake(0x4000)
    need = cb.workspace_bytes(cb.OP_INDEX_TOPK_PREFILL, idesc, 1, 32768, 0, 1024)
    assert need >= 32768 * 8192 * 4
    # k out of range, workspace too small
    assert L.csa_index_topk_prefill(ctypes.byref(idesc), 1, 16, 0, P, P, ctypes.byref(keys), 0, P, None, P, need, None) == 1
    assert L.csa_index_topk_prefill(ctypes.byref(idesc), 1, 32768, 0, P, P, ctypes.byref(keys), 1024, P, None, P, 16, None) == 4
    mx = cb.index_desc(16, 48, "bf16", "mxfp4", "mxfp4", "bf16", 4, 8192)
    assert L.csa_index_topk_decode(ctypes.byref(mx), 1, P, P, P, ctypes.byref(keys), 1024, P, None, P, 1 << 30, None) == 3
    adesc = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192)
    kv = cb.Cache(0x1000, 0, 0x2000, 0x3000)   # FP8 without a scale buffer
    assert L.csa_sparse_attn_decode(ctypes.byref(adesc), 1, P, P, ctypes.byref(kv), P, 1024, 0.1, P, None, P, 1 << 30, None) == 1
    assert L.csa_workspace_bytes(99, ctypes.byref(adesc), 1, 1, 0, 0) == 0


@pytest.mark.parametrize("scale", [0.0, -0.125, float("inf"), float("nan")])
def test_attention_rejects_nonpositive_scale(scale):
    # the kernels take the running maximum over unscaled scores, which is
    # only order-preserving for a positive, finite scale
    L = cb.lib()
    adesc = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    P = fake(0x4000)
    args = (P, P, ctypes.byref(kv))
    assert L.csa_sparse_attn_prefill(ctypes.byref(adesc), 1, 16, 0, P, ctypes.byref(kv), P, 1024, scale, P, None,
                                     P, 1 << 30, None) == 1
    assert b"softmax_scale" in L.csa_last_error()
    assert L.csa_sparse_attn_decode(ctypes.byref(adesc), 1, *args, P, 1024, scale, P, None, P, 1 << 30, None) == 1
    assert L.hca_dense_attn_prefill(ctypes.byref(adesc), 1, 16, 0, P, ctypes.byref(kv), scale, P, None, P, 1 << 30,
                                    None) == 1
    assert L.hca_dense_attn_decode(ctypes.byref(adesc), 1, *args, scale, P, None, P, 1 << 30, None) == 1


def test_mxfp4_workspace_holds_query_operands():
    # MXFP4 QK: per query row 64 lanes x 16 bytes of codes + 64 int32 scales
    # for the scaled-MFMA scan, on top of the BF16-QK workspace
    mx = cb.index_desc(16, 64, "bf16", "mxfp4", "mxfp4", "bf16", 4, 262144)
    bf = cb.index_desc(16, 64, "bf16", "bf16", "mxfp4", "bf16", 4, 262144)
    for op, B, T in ((cb.OP_INDEX_TOPK_DECODE, 4, 1), (cb.OP_INDEX_TOPK_PREFILL, 2, 48)):
        a = cb.workspace_bytes(op, mx, B, T, 4 * 8000, 1024)
        b = cb.workspace_bytes(op, bf, B, T, 4 * 8000, 1024)
        assert a - b >= B * T * (64 * 16 + 64 * 4)


@pytest.mark.parametrize("nope", ["bf16", "fp8"])
def test_attention_rejects_capacity_past_32bit_row_offsets(nope):
    # the MFMA kernels gather rows by 32-bit byte offsets within a sequence:
    # 2^21 BF16 (1 KB) or 2^22 FP8 (512 B) non-RoPE rows is the largest cache
    # they can address; one entry more is rejected before any launch
    L = cb.lib()
    lim = (1 << 31) // (1024 if nope == "bf16" else 512)
    P = fake(0x4000)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    over = cb.attn_desc(64, 512, 64, "bf16", "bf16", nope, "bf16", 4, lim + 1)
    ws = 1 << 40
    assert L.csa_sparse_attn_prefill(ctypes.byref(over), 1, 16, 0, P, ctypes.byref(kv), P, 1024, 0.1, P, None,
                                     P, ws, None) == 3
    assert b"2^31" in L.csa_last_error()
    assert L.csa_sparse_attn_decode(ctypes.byref(over), 1, P, P, ctypes.byref(kv), P, 1024, 0.1, P, None, P, ws,
                                    None) == 3
    assert L.hca_dense_attn_prefill(ctypes.byref(over), 1, 16, 0, P, ctypes.byref(kv), 0.1, P, None, P, ws, None) == 3
    assert L.hca_dense_attn_decode(ctypes.byref(over), 1, P, P, ctypes.byref(kv), 0.1, P, None, P, ws, None) == 3


def test_decode_attention_workspace_is_per_sequence():
    # the decode split count depends on the entry count only, never on the
    # batch size, so the workspace grows linearly with B
    for op, k, cap in ((cb.OP_SPARSE_ATTN_DECODE, 1024, 32776), (cb.OP_DENSE_ATTN_DECODE, 0, 8194)):
        d = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4 if k else 128, cap)
        one = cb.workspace_bytes(op, d, 1, 1, 0, k)
        assert one > 0
        for B in (4, 16, 32):
            assert cb.workspace_bytes(op, d, B, 1, 0, k) == B * one


def test_noalloc_decode_rejects_past_its_scratch_on_the_host():
    # the allocation-free decode holds its split partials in a fixed device
    # array; a batch whose partials would not fit is rejected before launch
    L = cb.lib()
    desc = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192)
    per_seq = cb.workspace_bytes(cb.OP_SPARSE_ATTN_DECODE, desc, 1, 1, 0, 1024)
    B = cb.NOALLOC_SCRATCH_BYTES // per_seq + 1
    P = fake(0x4000)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    assert L.csa_sparse_attn_decode_noalloc(ctypes.byref(desc), B, P, P, ctypes.byref(kv), P, 1024, 0.1, P, None,
                                            None) == 4
    assert b"scratch" in L.csa_last_error()
    assert L.csa_sparse_attn_decode_noalloc(ctypes.byref(desc), 1, P, P, ctypes.byref(kv), P, 0, 0.1, P, None,
                                            None) == 1


def test_decode_step_validates_everything_before_launch():
    L = cb.lib()
    assert ctypes.sizeof(cb.DecodeInputs) == 15 * 8
    cap = 8192
    kvd = cb.cache_desc(4, True, 512, 64, "bf16", "fp8", "bf16", cap)
    kd = cb.cache_desc(4, True, 64, 0, "bf16", "fp8", "f32", cap)
    idesc = cb.index_desc(16, 64, "bf16", "bf16", "fp8", "f32", 4, cap)
    adesc = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, cap)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    ks = cb.Cache(0x6000, 0x7000, 0, 0x8000)
    P = 0x4000
    inp = cb.DecodeInputs(*([P] * 15))
    need = L.csa_decode_step_workspace_bytes(ctypes.byref(idesc), ctypes.byref(adesc), 4, 1024)
    assert need >= cb.workspace_bytes(cb.OP_INDEX_TOPK_DECODE, idesc, 4, 1, 0, 1024) + \
        cb.workspace_bytes(cb.OP_SPARSE_ATTN_DECODE, adesc, 4, 1, 0, 1024)
    args = lambda d1, d2, d3, d4, i, ws_bytes: (ctypes.byref(d1), ctypes.byref(kv), ctypes.byref(d2), ctypes.byref(ks),
                                                ctypes.byref(d3), ctypes.byref(d4), 4, fake(P), i, 1024, 0.1,
                                                fake(P), None, fake(P), None, fake(P), ws_bytes, None)
    assert L.csa_decode_step(*args(kvd, kd, idesc, adesc, None, need)) == 1          # no inputs
    bad_m = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 8, cap)
    assert L.csa_decode_step(*args(kvd, kd, idesc, bad_m, ctypes.byref(inp), need)) == 1
    assert b"share m" in L.csa_last_error()
    bad_key = cb.index_desc(16, 64, "bf16", "bf16", "bf16", "f32", 4, cap)       # keys stored FP8
    assert L.csa_decode_step(*args(kvd, kd, bad_key, adesc, ctypes.byref(inp), need)) == 1
    assert L.csa_decode_step(*args(kvd, kd, idesc, adesc, ctypes.byref(inp), need - 256)) == 4
    no_b = cb.DecodeInputs(P, None, P, None, P, None, P, P, P, P, P, P, P, P, P)    # overlap needs b, zb, Bb
    assert L.csa_decode_step(*args(kvd, kd, idesc, adesc, ctypes.byref(no_b), need)) == 1


def test_window_and_merge_validation():
    L = cb.lib()
    P = fake(0x4000)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    # a window is for dense attention only
    win = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192, window=128)
    assert L.csa_sparse_attn_prefill(ctypes.byref(win), 1, 16, 0, P, ctypes.byref(kv), P, 1024, 0.1, P, None, P,
                                     1 << 30, None) == 1
    assert b"window" in L.csa_last_error()
    neg = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192, window=-1)
    assert L.hca_dense_attn_prefill(ctypes.byref(neg), 1, 16, 0, P, ctypes.byref(kv), 0.1, P, None, P, 1 << 30,
                                    None) == 1
    # the dense decode workspace covers the window's splits only
    full = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 1, 1 << 20)
    w128 = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 1, 1 << 20, window=128)
    assert cb.workspace_bytes(cb.OP_DENSE_ATTN_DECODE, w128, 1, 1, 0, 0) < \
        cb.workspace_bytes(cb.OP_DENSE_ATTN_DECODE, full, 1, 1, 0, 0)
    # merge: shapes and formats
    assert L.csa_lse_merge(4, 64, 510, 1, P, P, P, P, P, None, None) == 1
    assert L.csa_lse_merge(4, 64, 512, 2, P, P, P, P, P, None, None) == 3
    assert L.csa_lse_merge(4, 64, 512, 1, fake(0x4004), P, P, P, P, None, None) == 2
    assert L.csa_lse_merge(0, 64, 512, 1, P, P, P, P, P, None, None) == 0


def test_fp8_qk_mode_validation():
    """qk_mode: 0 or FP8E4M3; the FP8 QK product needs an FP8 cache and the
    64-head 512 + 64 shape (rejected on the host, before any launch)."""
    L = cb.lib()
    P = fake(0x4000)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    bad = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 128, 8192)
    bad.qk_mode = 3
    assert L.hca_dense_attn_prefill(ctypes.byref(bad), 1, 16, 0, P, ctypes.byref(kv), 0.1, P, None, P, 1 << 30,
                                    None) == 1
    for d in (cb.attn_desc(64, 512, 64, "bf16", "bf16", "bf16", "bf16", 128, 8192, qk="fp8"),
              cb.attn_desc(32, 512, 64, "bf16", "bf16", "fp8", "bf16", 128, 8192, qk="fp8"),
              cb.attn_desc(64, 512, 64, "f32", "bf16", "fp8", "bf16", 128, 8192, qk="fp8")):
        assert L.hca_dense_attn_prefill(ctypes.byref(d), 1, 16, 0, P, ctypes.byref(kv), 0.1, P, None, P, 1 << 30,
                                        None) == 3
        assert b"qk_mode" in L.csa_last_error()
    # sparse prefill lists beyond 1024 entries have no FP8 QK kernel
    d = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192, qk="fp8")
    assert L.csa_sparse_attn_prefill(ctypes.byref(d), 1, 16, 0, P, ctypes.byref(kv), P, 2048, 0.1, P, None, P,
                                     1 << 30, None) == 3


def test_paging_fields_are_validated_before_launch():
    # paged caches: page_size a power of two in 64..65536, capacity a multiple
    # of it, pool_pages >= 1, a block table exactly when paged (4-byte aligned)
    L = cb.lib()
    P = fake(0x4000)
    T = 0x9000
    cases = [(48, 640, 10, T, 1), (64, 100, 10, T, 1), (64, 640, 0, T, 1), (64, 640, 10, None, 1),
             (0, 640, 0, T, 1), (0, 640, 5, None, 1), (64, 640, 10, 0x9002, 2), (1 << 17, 1 << 17, 1, T, 1)]
    for ps, cap, pool, table, want in cases:
        d = cb.cache_desc(4, True, 32, 32, "f32", "f32", "f32", cap, page_size=ps, pool_pages=pool)
        c = cb.Cache(0x1000, 0, 0x2000, 0x3000, table)
        assert L.csa_compress_prefill(ctypes.byref(d), 1, 4, 0, P, P, P, P, P, P, ctypes.byref(c), None) == want, \
            (ps, cap, pool, table)
        a = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, cap, page_size=ps, pool_pages=pool)
        kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000, table)
        assert L.hca_dense_attn_decode(ctypes.byref(a), 1, P, P, ctypes.byref(kv), 0.1, P, None, P, 1 << 30,
                                       None) == want
        i = cb.index_desc(16, 64, "bf16", "bf16", "fp8", "f32", 4, cap, page_size=ps, pool_pages=pool)
        ks = cb.Cache(0x1000, 0x5000, 0, 0x3000, table)
        assert L.csa_index_topk_decode(ctypes.byref(i), 1, P, P, P, ctypes.byref(ks), 16, P, None, P, 1 << 30,
                                       None) == want
    # the attention descriptor's reserved field
    bad = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 640)
    bad.reserved = 1
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    assert L.hca_dense_attn_decode(ctypes.byref(bad), 1, P, P, ctypes.byref(kv), 0.1, P, None, P, 1 << 30, None) == 1
    # the prefill indexer reads contiguous keys only
    i = cb.index_desc(16, 64, "bf16", "bf16", "fp8", "f32", 4, 640, page_size=64, pool_pages=10)
    ks = cb.Cache(0x1000, 0x5000, 0, 0x3000, T)
    assert L.csa_index_topk_prefill(ctypes.byref(i), 1, 16, 0, P, P, ctypes.byref(ks), 16, P, None, P, 1 << 30,
                                    None) == 3
    assert b"paged" in L.csa_last_error()
    # the pool's rows must be addressable by the attention's 32-bit offsets
    big = cb.attn_desc(64, 512, 64, "bf16", "bf16", "bf16", "bf16", 4, 1024, page_size=1024, pool_pages=2049)
    kvp = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000, T)
    assert L.hca_dense_attn_decode(ctypes.byref(big), 1, P, P, ctypes.byref(kvp), 0.1, P, None, P, 1 << 40,
                                   None) == 3


def test_paged_workspaces():
    # paged sparse attention turns its lists into pool rows in the workspace
    # (B*T*k int32 after the split partials); dense attention and the
    # indexer need nothing more
    for op, T in ((cb.OP_SPARSE_ATTN_DECODE, 1), (cb.OP_SPARSE_ATTN_PREFILL, 64)):
        flat = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192)
        paged = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, 8192, page_size=64, pool_pages=512)
        for B in (1, 4):
            extra = cb.workspace_bytes(op, paged, B, T, 0, 1024) - cb.workspace_bytes(op, flat, B, T, 0, 1024)
            assert extra == -(-B * T * 1024 * 4 // 256) * 256
    flat = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 128, 8192)
    paged = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 128, 8192, page_size=64, pool_pages=512)
    assert cb.workspace_bytes(cb.OP_DENSE_ATTN_DECODE, paged, 4, 1, 0, 0) == \
        cb.workspace_bytes(cb.OP_DENSE_ATTN_DECODE, flat, 4, 1, 0, 0)


def test_decode_step_rejects_mixed_paging():
    L = cb.lib()
    cap = 8192
    kvd = cb.cache_desc(4, True, 512, 64, "bf16", "fp8", "bf16", cap, page_size=64, pool_pages=256)
    kd = cb.cache_desc(4, True, 64, 0, "bf16", "fp8", "f32", cap, page_size=64, pool_pages=256)
    idesc = cb.index_desc(16, 64, "bf16", "bf16", "fp8", "f32", 4, cap, page_size=64, pool_pages=256)
    adesc = cb.attn_desc(64, 512, 64, "bf16", "bf16", "fp8", "bf16", 4, cap)   # not paged
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000, 0x9000)
    ks = cb.Cache(0x6000, 0x7000, 0, 0x8000, 0x9000)
    inp = cb.DecodeInputs(*([0x4000] * 15))
    P = fake(0x4000)
    assert L.csa_decode_step(ctypes.byref(kvd), ctypes.byref(kv), ctypes.byref(kd), ctypes.byref(ks),
                             ctypes.byref(idesc), ctypes.byref(adesc), 4, P, ctypes.byref(inp), 1024, 0.1, P, None,
                             P, None, P, 1 << 30, None) == 1
    assert b"paging" in L.csa_last_error()


def test_project_prefill_validation():
    # the compressor fed from hidden states: shapes it does not take are
    # rejected before any launch
    L = cb.lib()
    desc = cb.cache_desc(4, True, 512, 64, "bf16", "fp8", "bf16", 1000)
    kv = cb.Cache(0x1000, 0x5000, 0x2000, 0x3000)
    P = fake(0x4000)
    args = lambda d, T, pos0, dm: (ctypes.byref(d), 1, T, pos0, P, dm, P, P, P, ctypes.byref(kv), P, 1 << 30, None)
    assert L.csa_compress_project_prefill(*args(desc, 16, 2, 256)) == 3      # pos0 not a multiple of m
    assert L.csa_compress_project_prefill(*args(desc, 16, 0, 100)) == 1      # d_model not a multiple of 64
    f32 = cb.cache_desc(4, True, 512, 64, "f32", "fp8", "bf16", 1000)
    assert L.csa_compress_project_prefill(*args(f32, 16, 0, 256)) == 3       # hidden states must be BF16
    m3 = cb.cache_desc(3, True, 512, 64, "bf16", "fp8", "bf16", 1000)
    assert L.csa_compress_project_prefill(*args(m3, 16, 0, 256)) == 3        # m must divide 128
    assert L.csa_compress_project_prefill(*args(desc, 4004, 0, 256)) == 5    # capacity
    assert b"capacity" in L.csa_last_error()
    assert L.csa_compress_project_prefill(*args(desc, 16, 0, 256)[:10], P, 16, None) == 4   # workspace
    assert L.csa_compress_project_prefill(ctypes.byref(desc), 1, 0, 0, P, 256, P, P, P, ctypes.byref(kv), P, 0,
                                          None) == 0                      # T == 0: nothing to do
