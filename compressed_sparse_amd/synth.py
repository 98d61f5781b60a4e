"""Seeded synthetic inputs for the CSA / HCA hot path, and the workload shapes.

This module holds no step of the method: it only draws random tensors (with
torch's counter-based Philox generator on the GPU, or its CPU generator) and
states the sizes of each workload.  Both the HIP path and the CPU oracle read
the same tensors from here.

Every tensor is identified by (seed, name, sequence, chunk); the same key
always yields the same values on the same device type, so a test can draw a
large context chunk by chunk on the GPU and fetch only the chunks the oracle
needs to the host.
"""
import dataclasses
import math
import zlib

import torch

MASK63 = (1 << 63) - 1


def stream_key(seed, name, seq=0, chunk=0):
    """A 63-bit generator seed derived from the tensor's identity."""
    h = zlib.crc32(name.encode())
    return ((seed * 0x9E3779B97F4A7C15) ^ (h << 20) ^ (seq << 44) ^ (chunk * 0x632BE59BD9B4E019)) & MASK63


def normal(shape, name, seed=0, seq=0, chunk=0, device="cpu", dtype=torch.float32, std=1.0):
    """N(0, std^2) samples drawn in fp32 and cast (RNE) to `dtype`."""
    g = torch.Generator(device=device)
    g.manual_seed(stream_key(seed, name, seq, chunk))
    x = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


def uniform_int(shape, low, high, name, seed=0, seq=0, chunk=0, device="cpu"):
    g = torch.Generator(device=device)
    g.manual_seed(stream_key(seed, name, seq, chunk))
    return torch.randint(low, high, shape, generator=g, device=device, dtype=torch.int64)


def random_fp8_codes(shape, name, seed=0, seq=0, device="cpu"):
    """Random OFP8 E4M3 bytes over every exponent field 0..15 (subnormals and
    the top binades included; the NaN code S.1111.111 is replaced by the
    largest finite S.1111.110), used to fill a cache directly when a kernel is
    tested on its own."""
    e = uniform_int(shape, 0, 16, name + ".e", seed, seq, device=device)
    mnt = uniform_int(shape, 0, 8, name + ".m", seed, seq, device=device)
    s = uniform_int(shape, 0, 2, name + ".s", seed, seq, device=device)
    mnt = torch.where((e == 15) & (mnt == 7), torch.full_like(mnt, 6), mnt)
    return ((s << 7) | (e << 3) | mnt).to(torch.uint8)


def random_e2m1_bytes(shape, name, seed=0, seq=0, device="cpu"):
    """Random packed FP4 E2M1 pairs (two 4-bit codes per byte)."""
    return uniform_int(shape, 0, 256, name, seed, seq, device=device).to(torch.uint8)


def random_e8m0(shape, name, lo=104, hi=141, seed=0, seq=0, device="cpu"):
    """Random E8M0 scale bytes in [lo, hi) (2^-23 .. 2^13 by default)."""
    return uniform_int(shape, lo, hi, name, seed, seq, device=device).to(torch.uint8)


def random_sorted_subsets(n_rows, n_visible, k, name, seed=0, device="cpu"):
    """Per row r, a random ascending subset of [0, n_visible[r]) of size
    min(k, n_visible[r]), padded with -1 (an index list of the form the
    top-k step emits)."""
    out = torch.full((n_rows, k), -1, dtype=torch.int32)
    g = torch.Generator()
    g.manual_seed(stream_key(seed, name))
    for r in range(n_rows):
        n = int(n_visible[r])
        kk = min(k, n)
        if kk > 0:
            sel = torch.randperm(n, generator=g)[:kk].sort().values
            out[r, :kk] = sel.to(torch.int32)
    return out.to(device)


# ---------------------------------------------------------------------------
# workload shapes
# ---------------------------------------------------------------------------

@dataclasses.dataclass
class Workload:
    name: str
    batch: int
    tokens: int              # prefill: query tokens per sequence; decode: context length
    heads: int
    d_nope: int
    d_rope: int
    m: int
    overlap: bool
    topk: int                # 0 for HCA (dense)
    idx_heads: int
    idx_dim: int
    act_dtype: str           # projections, q, qI: "f32" | "bf16"
    nope_fmt: str            # KV cache non-RoPE part: "f32" | "bf16" | "fp8"
    rope_fmt: str            # KV cache RoPE part: "f32" | "bf16"
    key_fmt: str             # indexer keys: "f32" | "bf16" | "fp8" | "mxfp4"
    score_fmt: str           # "f32" | "bf16"
    qk_fmt: str              # indexer query format: "f32" | "bf16" | "mxfp4"
    out_dtype: str           # "f32" | "bf16"
    rope_base: float = 10000.0
    mode: str = "prefill"    # "prefill" | "decode"
    chunk: int = 0           # prefill query chunk (HCA 1M) / context generation chunk

    @property
    def c(self):
        return self.d_nope + self.d_rope

    @property
    def tau(self):
        return 1.0 / math.sqrt(self.c)


TINY_CSA_PREFILL_FP32 = Workload(
    "tiny_csa_prefill_fp32_L2048", batch=1, tokens=2048, heads=8, d_nope=32, d_rope=32, m=4,
    overlap=True, topk=64, idx_heads=4, idx_dim=32, act_dtype="f32", nope_fmt="f32",
    rope_fmt="f32", key_fmt="f32", score_fmt="f32", qk_fmt="f32", out_dtype="f32")

CSA_PREFILL_BF16_32K = Workload(
    "csa_prefill_bf16_L32768_H64_k1024", batch=1, tokens=32768, heads=64, d_nope=512, d_rope=64,
    m=4, overlap=True, topk=1024, idx_heads=16, idx_dim=64, act_dtype="bf16", nope_fmt="bf16",
    rope_fmt="bf16", key_fmt="bf16", score_fmt="f32", qk_fmt="bf16", out_dtype="bf16")

CSA_DECODE_B32_128K = Workload(
    "csa_decode_b32_ctx131072_fp8kv", batch=32, tokens=131072, heads=64, d_nope=512, d_rope=64,
    m=4, overlap=True, topk=1024, idx_heads=16, idx_dim=64, act_dtype="bf16", nope_fmt="fp8",
    rope_fmt="bf16", key_fmt="fp8", score_fmt="f32", qk_fmt="bf16", out_dtype="bf16",
    mode="decode", chunk=8192)

HCA_PREFILL_1M = Workload(
    "hca_prefill_1M_chunk8192", batch=1, tokens=1 << 20, heads=64, d_nope=512, d_rope=64,
    m=128, overlap=False, topk=0, idx_heads=0, idx_dim=0, act_dtype="bf16", nope_fmt="fp8",
    rope_fmt="bf16", key_fmt="none", score_fmt="none", qk_fmt="none", out_dtype="bf16",
    chunk=8192)

HCA_DECODE_B16_1M = Workload(
    "hca_decode_b16_ctx1M", batch=16, tokens=1 << 20, heads=64, d_nope=512, d_rope=64,
    m=128, overlap=False, topk=0, idx_heads=0, idx_dim=0, act_dtype="bf16", nope_fmt="fp8",
    rope_fmt="bf16", key_fmt="none", score_fmt="none", qk_fmt="none", out_dtype="bf16",
    mode="decode", chunk=8192)

PAIR_CSA_DECODE_B4_1M = Workload(
    "pair_csa_decode_b4_ctx1M_mxfp4idx", batch=4, tokens=1 << 20, heads=64, d_nope=512,
    d_rope=64, m=4, overlap=True, topk=1024, idx_heads=16, idx_dim=64, act_dtype="bf16",
    nope_fmt="fp8", rope_fmt="bf16", key_fmt="mxfp4", score_fmt="bf16", qk_fmt="mxfp4",
    out_dtype="bf16", mode="decode", chunk=8192)

PAIR_HCA_DECODE_B4_1M = dataclasses.replace(
    HCA_DECODE_B16_1M, name="pair_hca_decode_b4_ctx1M", batch=4)

# Paged, variable-length CSA decode (the serving shape): the B = 32 FP8
# workload's formats, each sequence with its own context length (mixed_lengths:
# log-uniform over 8K..256K tokens), caches in 64-entry pages of one pool.
PAGED_CSA_DECODE_B32_MIXED = dataclasses.replace(
    CSA_DECODE_B32_128K, name="paged_csa_decode_b32_ctx8K-256K_page64")

# Compressor inputs projected from hidden states for the 32K prefill: the
# pages give no model width; d_model = 4096 is this workload's reading.
PROJECT_PREFILL_32K = dataclasses.replace(CSA_PREFILL_BF16_32K, name="csa_compress_from_hidden_L32768_d4096")
PROJECT_D_MODEL = 4096

WORKLOADS = {w.name: w for w in (TINY_CSA_PREFILL_FP32, CSA_PREFILL_BF16_32K, CSA_DECODE_B32_128K,
                                 HCA_PREFILL_1M, HCA_DECODE_B16_1M, PAIR_CSA_DECODE_B4_1M,
                                 PAIR_HCA_DECODE_B4_1M, PAGED_CSA_DECODE_B32_MIXED)}


def mixed_lengths(B, lo_log2, hi_log2, seed=0):
    """B context lengths log-uniform over [2^lo_log2, 2^hi_log2) tokens, seeded."""
    g = torch.Generator().manual_seed(stream_key(seed, "ctx.len"))
    u = torch.rand(B, generator=g, dtype=torch.float64)
    return [int(2.0 ** (lo_log2 + (hi_log2 - lo_log2) * float(x))) for x in u]

TORCH_DTYPE = {"f32": torch.float32, "bf16": torch.bfloat16}


def tiny_projections(w: Workload, seed=0, T=None, d_model=512):
    """The tiny fp32 workload's projected tensors, formed from hidden states
    H ~ N(0,1) [T, d_model] and weights ~ N(0, (1/sqrt(d_model))^2), with the
    products taken in fp64 and rounded to fp32.  Returns a dict of fp32 CPU
    tensors: a, b, za, zb [T, c]; ka, kb, kza, kzb [T, d_I] (indexer-key
    compressor); q [T, H, c]; qI [T, H_I, d_I]; w [T, H_I]; Ba, Bb [m, c];
    kBa, kBb [m, d_I]."""
    T = T or w.tokens
    std = 1.0 / math.sqrt(d_model)
    Hs = normal((T, d_model), "hidden", seed, dtype=torch.float64)
    out = {}

    def proj(name, cols):
        W = normal((d_model, cols), "W." + name, seed, dtype=torch.float64, std=std)
        return (Hs @ W).to(torch.float32)

    for nm in ("a", "b", "za", "zb"):
        out[nm] = proj(nm, w.c)
    for nm in ("ka", "kb", "kza", "kzb"):
        out[nm] = proj(nm, w.idx_dim)
    out["q"] = proj("q", w.heads * w.c).reshape(T, w.heads, w.c)
    out["qI"] = proj("qI", w.idx_heads * w.idx_dim).reshape(T, w.idx_heads, w.idx_dim)
    out["w"] = proj("w", w.idx_heads)
    for nm, cols in (("Ba", w.c), ("Bb", w.c), ("kBa", w.idx_dim), ("kBb", w.idx_dim)):
        out[nm] = normal((w.m, cols), nm, seed, dtype=torch.float32, std=std)
    return out


def compressor_params(w: Workload, seed=0, device="cpu"):
    """Bias matrices B^a, B^b [m, c] (and the indexer-key instance's) drawn
    N(0, (1/sqrt(c))^2) in fp32."""
    out = {"Ba": normal((w.m, w.c), "Ba", seed, device=device, std=1 / math.sqrt(w.c))}
    if w.overlap:
        out["Bb"] = normal((w.m, w.c), "Bb", seed, device=device, std=1 / math.sqrt(w.c))
    if w.idx_dim:
        out["kBa"] = normal((w.m, w.idx_dim), "kBa", seed, device=device, std=1 / math.sqrt(w.idx_dim))
        out["kBb"] = normal((w.m, w.idx_dim), "kBb", seed, device=device, std=1 / math.sqrt(w.idx_dim))
    return out


def token_chunk(w: Workload, seq, chunk, n_tok, seed=0, device="cpu", names=None):
    """Projected per-token compressor inputs for tokens [chunk*w.chunk, +n_tok)
    of sequence `seq`, N(0,1) in the activation dtype: a, za (+ b, zb when
    overlapped) [n_tok, c] and ka, kza, kb, kzb [n_tok, d_I]."""
    dt = TORCH_DTYPE[w.act_dtype]
    names = names or (["a", "za"] + (["b", "zb"] if w.overlap else [])
                      + (["ka", "kza", "kb", "kzb"] if w.idx_dim else []))
    out = {}
    for nm in names:
        cols = w.idx_dim if nm.startswith("k") else w.c
        out[nm] = normal((n_tok, cols), "tok." + nm, seed, seq, chunk, device=device, dtype=dt)
    return out


def query_chunk(w: Workload, seq, chunk, n_tok, seed=0, device="cpu", with_index=True):
    """Queries for tokens of one chunk: q [n, H, c], and for CSA qI [n, H_I,
    d_I] and w [n, H_I] (fp32).  All N(0,1)."""
    dt = TORCH_DTYPE[w.act_dtype]
    out = {"q": normal((n_tok, w.heads, w.c), "q", seed, seq, chunk, device=device, dtype=dt)}
    if with_index and w.idx_dim:
        out["qI"] = normal((n_tok, w.idx_heads, w.idx_dim), "qI", seed, seq, chunk, device=device, dtype=dt)
        out["w"] = normal((n_tok, w.idx_heads), "w", seed, seq, chunk, device=device, dtype=torch.float32)
    return out


# ---------------------------------------------------------------------------
# hidden states and the compressor's projection weights (prefill from hidden
# states): X ~ N(0, 1) and each projection W ~ N(0, 1 / d_model) in BF16, so
# the projected rows are again about N(0, 1) like the other workloads'
# ---------------------------------------------------------------------------

def hidden_chunk(seq, chunk, n_tok, d_model, seed=0, device="cpu"):
    """Hidden states [n_tok, d_model] BF16 of tokens [chunk*n_tok, +n_tok) of `seq`."""
    return normal((n_tok, d_model), "hid.x", seed, seq, chunk, device=device, dtype=torch.bfloat16)


def projection_weights(c, d_model, overlap, prefix="", seed=0, device="cpu"):
    """The compressor's projections W^{aKV}, W^{aZ} (and W^{bKV}, W^{bZ}), each
    [d_model, c] BF16, std 1/sqrt(d_model)."""
    names = ("aKV", "aZ", "bKV", "bZ") if overlap else ("aKV", "aZ")
    return {n: normal((d_model, c), "W." + prefix + n, seed, device=device, dtype=torch.bfloat16,
                      std=d_model ** -0.5) for n in names}


# ---------------------------------------------------------------------------
# "planted" indexer inputs (a labelled variant for the MXFP4 recall, never a
# headline): the isotropic workloads give near-uniform scores, so MXFP4
# rounding reorders the many keys near the k-th score.  Here a sequence's
# query heads share a unit direction u and `n_plant` keys are drawn as
# rho * sqrt(d) * u + sqrt(1 - rho^2) * eps (the other keys eps ~ N(0, I)), so
# the top set stands apart as it does for a trained model's peaked scores.
# ---------------------------------------------------------------------------

def planted_index_inputs(n, d, heads, n_plant, rho, seq, seed=0):
    """fp32 keys [n, d], query heads [heads, d], positive head weights
    [heads] and the planted key indices, for one sequence (CPU tensors)."""
    u = normal((d,), "pl.u", seed, seq, dtype=torch.float64)
    u = u / u.norm()
    keys = normal((n, d), "pl.k", seed, seq, dtype=torch.float64)
    g = torch.Generator().manual_seed(stream_key(seed, "pl.idx", seq))
    idx = torch.randperm(n, generator=g)[:n_plant].sort().values
    keys[idx] = rho * d ** 0.5 * u + (1.0 - rho * rho) ** 0.5 * keys[idx]
    q = d ** 0.5 * u + 0.3 * normal((heads, d), "pl.q", seed, seq, dtype=torch.float64)
    w = normal((heads,), "pl.w", seed, seq, dtype=torch.float64).abs() + 0.1
    return keys.float(), q.float(), w.float(), idx
