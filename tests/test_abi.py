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
    assert L.csa_version() == 1
    assert L.csa_status_string(0) == b"CSA_OK"
    assert L.csa_status_string(5) == b"CSA_ERR_CAPACITY"


def test_struct_sizes_match_header_layout():
    assert ctypes.sizeof(cb.CacheDesc) == 48
    assert ctypes.sizeof(cb.Cache) == 32
    assert ctypes.sizeof(cb.IndexDesc) == 40
    assert ctypes.sizeof(cb.AttnDesc) == 48


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
