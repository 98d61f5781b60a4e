"""GPU parity of the lightning indexer + top-k (csa_index_topk_prefill /
csa_index_topk_decode) against the CPU oracle, through the C ABI.  Key
caches are filled directly with seeded synthetic values of each storage
format, so the step is checked on its own."""
import numpy as np
import pytest
import torch

from compressed_sparse_amd import binding as cb
from compressed_sparse_amd import synth
from oracle import csa
from oracle import formats as F
from tests.helpers import ascending_padded, compare_topk, fp32_score_bound, np64, topk_explained

pytestmark = pytest.mark.gpu
DEV = "cuda"


def key_cache(fmt, B, cap, d, m, seed):
    desc = cb.cache_desc(m, True, d, 0, "f32", fmt, "f32", cap)
    kc = cb.KVCache(desc, B)
    if fmt in ("f32", "bf16"):
        kc.nope.copy_(synth.normal((B, cap, d), "keys", seed, device=DEV, dtype=synth.TORCH_DTYPE[fmt]))
        dec = np64(kc.nope)
    elif fmt == "fp8":
        kc.nope.copy_(synth.random_fp8_codes((B, cap, d), "keys", seed, device=DEV))
        kc.scale.copy_(synth.normal((B, cap), "kscale", seed, device=DEV).abs() * 0.01 + 1e-3)
        dec = F.fp8_decode(kc.nope.cpu().numpy()) * kc.scale.cpu().double().numpy()[..., None]
    else:
        kc.nope.copy_(synth.random_e2m1_bytes((B, cap, d // 2), "keys", seed, device=DEV))
        kc.scale.copy_(synth.random_e8m0((B, cap, d // 32), "kscale", seed=seed, device=DEV))
        packed = kc.nope.cpu().numpy().astype(np.int64)
        codes = np.stack([packed & 15, packed >> 4], -1).reshape(B, cap, d)
        dec = F.mxfp4_decode(codes, kc.scale.cpu().numpy())
    return kc, dec


def oracle_rows(qI, w, K, positions, m, k, qk_fmt, score_fmt):
    idx, scores = [], []
    for r, pos in enumerate(positions):
        n = min(int(csa.n_visible(pos, m)), K.shape[0])
        I = csa.index_scores(csa.quantize_query(qI[r], qk_fmt), w[r], K, n, score_fmt)
        scores.append(I)
        idx.append(csa.topk(I, n, k))
    return np.array(idx), scores


def test_prefill_fp32_tiny_workload_shapes():
    """fp32 indexer: 4 heads x 32 dims, m = 4, k = 64, 2048 queries."""
    T, H, d, m, k = 2048, 4, 32, 4, 64
    cap = T // m
    kc, K = key_cache("f32", 1, cap, d, m, seed=21)
    qI = synth.normal((1, T, H, d), "qI", 21, device=DEV)
    w = synth.normal((1, T, H), "w", 21, device=DEV)
    desc = cb.index_desc(H, d, "f32", "f32", "f32", "f32", m, cap)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    scores = torch.zeros((1, T, cap), dtype=torch.float32, device=DEV)
    cb.index_topk_prefill(desc, kc, 0, qI, w, k, idx, scores)
    torch.cuda.synchronize()
    ref_idx, ref_sc = oracle_rows(np64(qI[0]), np64(w[0]), K[0], np.arange(T), m, k, "f32", "f32")
    got = idx[0].cpu().numpy()
    assert ascending_padded(got)
    differing, bad = compare_topk(got, ref_idx, ref_sc, 1e-6)
    assert not bad, f"rows {bad[:5]} differ beyond the 1e-6 tie window"
    assert differing <= 0.01 * T
    gs = scores[0].cpu().double().numpy()
    for t in range(0, T, 97):
        n = len(ref_sc[t])
        assert np.allclose(gs[t, :n], ref_sc[t], rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("key_fmt,with_scores", [("bf16", False), ("fp8", False), ("bf16", True)])
def test_prefill_16x64_chunk_at_offset(key_fmt, with_scores):
    """16 heads x 64 dims, BF16 queries, BF16 or FP8 keys, queries at
    positions 3072..4072 of a longer prefill (a ragged last group of 4),
    k = 256.  Without a score output the scores stay on chip (fused
    kernel); with one the streaming scan writes them and the fused kernel's
    select reads them back."""
    T, H, d, m, k, pos0 = 1001, 16, 64, 4, 256, 3072
    cap = (pos0 + T) // m + 3
    kc, K = key_cache(key_fmt, 1, cap, d, m, seed=22)
    qI = synth.normal((1, T, H, d), "qI", 22, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((1, T, H), "w", 22, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "bf16", key_fmt, "f32", m, cap)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    scores = torch.zeros((1, T, cap), dtype=torch.float32, device=DEV) if with_scores else None
    cb.index_topk_prefill(desc, kc, pos0, qI, w, k, idx, scores)
    torch.cuda.synchronize()
    ref_idx, ref_sc = oracle_rows(np64(qI[0]), np64(w[0]), K[0], pos0 + np.arange(T), m, k, "bf16", "f32")
    got = idx[0].cpu().numpy()
    assert ascending_padded(got)
    differing, bad = compare_topk(got, ref_idx, ref_sc, 1e-6)
    assert not bad and differing <= 0.01 * T
    if with_scores:
        gs = scores[0].cpu().double().numpy()
        for t in range(0, T, 37):
            n = len(ref_sc[t])
            assert np.allclose(gs[t, :n], ref_sc[t], rtol=1e-5, atol=1e-5 * np.abs(ref_sc[t]).max())


def test_decode_fp8_keys_mixed_positions():
    """FP8 keys with per-entry scale, BF16 queries, fp32 scores; sequences at
    different positions, including one with a single visible entry and one
    with none."""
    B, H, d, m, k, cap = 4, 16, 64, 4, 1024, 8192
    kc, K = key_cache("fp8", B, cap, d, m, seed=23)
    positions = [4 * cap - 1, 20000, 5, 2]
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    qI = synth.normal((B, H, d), "qI", 23, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((B, H), "w", 23, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "bf16", "fp8", "f32", m, cap)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    cb.index_topk_decode(desc, kc, pos, qI, w, k, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert ascending_padded(got)
    for b in range(B):
        ri, rs = oracle_rows(np64(qI[b])[None], np64(w[b])[None], K[b], [positions[b]], m, k, "bf16", "f32")
        differing, bad = compare_topk(got[b:b + 1], ri, rs, 1e-6)
        assert not bad, f"sequence {b}"
    assert list(got[2]) == [0] + [-1] * (k - 1)
    assert (got[3] == -1).all()


def test_decode_mxfp4_bf16_scores():
    """MXFP4 keys and queries (the query is quantised inside the call), fp32
    accumulation, scores rounded to BF16 before selection.  The GPU's fp32
    sum and the oracle's fp64 sum may round to neighbouring BF16 values, so
    indices within one BF16 step of the threshold may differ."""
    B, H, d, m, k, cap = 2, 16, 64, 4, 1024, 16384
    kc, K = key_cache("mxfp4", B, cap, d, m, seed=24)
    positions = [4 * cap - 1, 30001]
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    qI = synth.normal((B, H, d), "qI", 24, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((B, H), "w", 24, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "mxfp4", "mxfp4", "bf16", m, cap)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    scores = torch.zeros((B, cap), dtype=torch.float32, device=DEV)
    cb.index_topk_decode(desc, kc, pos, qI, w, k, idx, scores)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert ascending_padded(got)
    for b in range(B):
        ri, rs = oracle_rows(np64(qI[b])[None], np64(w[b])[None], K[b], [positions[b]], m, k, "mxfp4", "bf16")
        # scores equal, or one BF16 step apart beyond the fp32 accumulation bound
        qq = csa.quantize_query(np64(qI[b]), "mxfp4")
        delta = 2.0 ** -7 * np.abs(rs[0]) + fp32_score_bound(qq, np64(w[b]), K[b], len(rs[0]))
        assert topk_explained(got[b], ri[0], rs[0], delta, 0.0), f"sequence {b}"
        gs = scores[b].cpu().double().numpy()[:len(rs[0])]
        assert (np.abs(gs - rs[0]) <= delta).all()
        assert (gs == rs[0]).mean() > 0.99


def test_k_larger_than_visible():
    B, H, d, m, k, cap = 2, 4, 32, 4, 64, 100
    kc, K = key_cache("f32", B, cap, d, m, seed=25)
    pos = torch.tensor([4 * 50 - 1, 4 * 63], dtype=torch.int64, device=DEV)
    qI = synth.normal((B, H, d), "qI", 25, device=DEV)
    w = synth.normal((B, H), "w", 25, device=DEV)
    desc = cb.index_desc(H, d, "f32", "f32", "f32", "f32", m, cap)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    cb.index_topk_decode(desc, kc, pos, qI, w, k, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert list(got[0]) == list(range(50)) + [-1] * 14
    assert list(got[1]) == list(range(63)) + [-1]


@pytest.mark.parametrize("n_entries", [6000, 20000])
def test_decode_all_ties_lowest_indices(n_entries):
    """Every key equal, so every score ties: the k lowest indices are kept.
    6000 entries fit the candidate list of the multi-workgroup decode top-k;
    20000 overflow it and take the whole-row select."""
    B, H, d, m, k = 2, 16, 64, 4, 1024
    cap = n_entries
    kc, K = key_cache("fp8", B, cap, d, m, seed=26)
    kc.nope.copy_(kc.nope[:, :1].expand(-1, cap, -1))
    kc.scale.fill_(0.01)
    pos = torch.tensor([4 * n_entries - 1, 4 * (n_entries // 2)], dtype=torch.int64, device=DEV)
    qI = synth.normal((B, H, d), "qI", 26, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((B, H), "w", 26, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "bf16", "fp8", "f32", m, cap)
    idx = torch.empty((B, k), dtype=torch.int32, device=DEV)
    cb.index_topk_decode(desc, kc, pos, qI, w, k, idx)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    assert list(got[0]) == list(range(k))
    assert list(got[1]) == list(range(k))


def test_decode_topk_many_chunks_repeatable():
    """Rows of up to 64 candidate chunks (4096 entries each) and of different
    lengths, the same call made several times: each row's last chunk
    workgroup to finish selects among the candidates its row's other chunk
    workgroups stored in the same launch, so every call must return the same
    sets, and those are the oracle's (exact except ties within 1e-6)."""
    B, H, d, m, k, cap = 6, 16, 64, 4, 1024, 262144
    kc, K = key_cache("fp8", B, cap, d, m, seed=27)
    positions = [4 * cap - 1, 4 * cap - 5, 600000, 131071, 20000, 4 * 4097]
    pos = torch.tensor(positions, dtype=torch.int64, device=DEV)
    qI = synth.normal((B, H, d), "qI", 27, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((B, H), "w", 27, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "bf16", "fp8", "f32", m, cap)
    ws = cb.workspace(cb.workspace_bytes(cb.OP_INDEX_TOPK_DECODE, desc, B, 1, 0, k))  # reused: state cleared per call
    runs = []
    for _ in range(6):
        idx = torch.full((B, k), -7, dtype=torch.int32, device=DEV)
        cb.index_topk_decode(desc, kc, pos, qI, w, k, idx, ws=ws)
        runs.append(idx)
    torch.cuda.synchronize()
    got = runs[0].cpu().numpy()
    for r in runs[1:]:
        assert np.array_equal(r.cpu().numpy(), got)
    assert ascending_padded(got)
    for b in range(B):
        ri, rs = oracle_rows(np64(qI[b])[None], np64(w[b])[None], K[b], [positions[b]], m, k, "bf16", "f32")
        differing, bad = compare_topk(got[b:b + 1], ri, rs, 1e-6)
        assert not bad, f"sequence {b}"


@pytest.mark.parametrize("pattern", ["all_equal", "three_values", "bf16_ties"])
def test_prefill_fused_ties(pattern):
    """Fused prefill select under ties, against the oracle (ties to the
    lower index): every score equal (one value between the extremes), keys
    of three values (a threshold bin far larger than the candidate list:
    radix fallback), and BF16-rounded scores of random keys (many exact
    ties inside the threshold bin)."""
    T, H, d, m, k, pos0 = 67, 16, 64, 4, 256, 4096
    cap = (pos0 + T) // m
    kc, K = key_cache("bf16", 1, cap, d, m, seed=27)
    score_fmt = "f32"
    if pattern == "all_equal":
        kc.nope.zero_()
    elif pattern == "three_values":
        r = torch.arange(cap, device=DEV) % 3
        row = synth.normal((1, 1, d), "krow", 27, device=DEV, dtype=torch.bfloat16)
        kc.nope.copy_(row * (r.to(torch.bfloat16) - 1)[None, :, None])
    else:
        score_fmt = "bf16"
    K = np64(kc.nope)[0]
    qI = synth.normal((1, T, H, d), "qI", 27, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((1, T, H), "w", 27, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "bf16", "bf16", score_fmt, m, cap)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    cb.index_topk_prefill(desc, kc, pos0, qI, w, k, idx)
    torch.cuda.synchronize()
    ref_idx, ref_sc = oracle_rows(np64(qI[0]), np64(w[0]), K, pos0 + np.arange(T), m, k, "bf16", score_fmt)
    got = idx[0].cpu().numpy()
    assert ascending_padded(got)
    if pattern == "bf16_ties":
        # the two sides round to BF16 from different fp32 / fp64 sums: an
        # entry may land one BF16 step apart, so differences must sit within
        # a few BF16 steps of the k-th score
        _, bad = compare_topk(got, ref_idx, ref_sc, 1e-6, kth_rel_window=2.0 ** -6)
        assert not bad
    else:
        # scores are exact here (products of zeros or of one key row), so
        # the sets, ties included, match exactly
        assert (got == ref_idx).all(), np.nonzero((got != ref_idx).any(1))[0][:5]


@pytest.mark.parametrize("T", [48, 47])
def test_prefill_mxfp4_bf16_scores(T):
    """MXFP4 keys and queries in prefill (the scaled-MFMA scan, two query
    rows per MFMA; an odd T leaves the last workgroup one row), then the
    select, same tolerance as decode."""
    B, H, d, m, k, cap = 2, 16, 64, 4, 1024, 8192
    pos0 = 4 * 8000 + 1
    kc, K = key_cache("mxfp4", B, cap, d, m, seed=26)
    qI = synth.normal((B, T, H, d), "qI", 26, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((B, T, H), "w", 26, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "mxfp4", "mxfp4", "bf16", m, cap)
    idx = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.zeros((B, T, cap), dtype=torch.float32, device=DEV)
    cb.index_topk_prefill(desc, kc, pos0, qI, w, k, idx, scores)
    torch.cuda.synchronize()
    got = idx.cpu().numpy()
    for b in range(B):
        assert ascending_padded(got[b])
        ri, rs = oracle_rows(np64(qI[b]), np64(w[b]), K[b], pos0 + np.arange(T), m, k, "mxfp4", "bf16")
        for t in range(T):
            # one BF16 step of the score plus the fp32 accumulation bound (key
            # blocks of very different scales meet in one sum)
            qq = csa.quantize_query(np64(qI[b, t]), "mxfp4")
            delta = 2.0 ** -7 * np.abs(rs[t]) + fp32_score_bound(qq, np64(w[b, t]), K[b], len(rs[t]))
            assert topk_explained(got[b, t], ri[t], rs[t], delta, 0.0), f"sequence {b}: row {t}"
            gs = scores[b, t].cpu().double().numpy()[:len(rs[t])]
            assert (np.abs(gs - rs[t]) <= delta).all()
            assert (gs == rs[t]).mean() > 0.99


@pytest.mark.parametrize("T,pos0", [(203, 4 * 8000 + 1), (6, 4 * 1030), (37, 4 * 200)])
def test_prefill_mxfp4_fused_equals_scan(T, pos0):
    """MXFP4 prefill with no scores requested runs the fused kernel (scores
    scored by the scaled FP4 MFMA straight into LDS, then the select); it
    must give the bits of the scan + select path (the same MFMA, head sum
    and select), and the oracle's sets within the BF16-score allowance.  Rows
    near n = k and an odd T (a partial last workgroup) included."""
    B, H, d, m, k = 2, 16, 64, 4, 1024
    cap = (pos0 + T) // m + 4
    kc, K = key_cache("mxfp4", B, cap, d, m, seed=28)
    qI = synth.normal((B, T, H, d), "qI", 28, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((B, T, H), "w", 28, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "mxfp4", "mxfp4", "bf16", m, cap)
    fused = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    scan = torch.empty((B, T, k), dtype=torch.int32, device=DEV)
    scores = torch.zeros((B, T, cap), dtype=torch.float32, device=DEV)
    cb.index_topk_prefill(desc, kc, pos0, qI, w, k, fused)
    cb.index_topk_prefill(desc, kc, pos0, qI, w, k, scan, scores)
    torch.cuda.synchronize()
    assert torch.equal(fused, scan)
    got = fused.cpu().numpy()
    for b in range(B):
        assert ascending_padded(got[b])
        ri, rs = oracle_rows(np64(qI[b]), np64(w[b]), K[b], pos0 + np.arange(T), m, k, "mxfp4", "bf16")
        for t in range(0, T, 5):
            qq = csa.quantize_query(np64(qI[b, t]), "mxfp4")
            delta = 2.0 ** -7 * np.abs(rs[t]) + fp32_score_bound(qq, np64(w[b, t]), K[b], len(rs[t]))
            assert topk_explained(got[b, t], ri[t], rs[t], delta, 0.0), f"sequence {b}: row {t}"


def test_prefill_rows_longer_than_fused_limit():
    """Rows with more than 8192 visible entries: streaming scan, then the
    one-workgroup-per-row radix select."""
    T, H, d, m, k, pos0 = 40, 16, 64, 4, 1024, 4 * 9000
    cap = (pos0 + T) // m + 1
    kc, K = key_cache("bf16", 1, cap, d, m, seed=27)
    qI = synth.normal((1, T, H, d), "qI", 27, device=DEV, dtype=torch.bfloat16)
    w = synth.normal((1, T, H), "w", 27, device=DEV)
    desc = cb.index_desc(H, d, "bf16", "bf16", "bf16", "f32", m, cap)
    idx = torch.empty((1, T, k), dtype=torch.int32, device=DEV)
    cb.index_topk_prefill(desc, kc, pos0, qI, w, k, idx)
    torch.cuda.synchronize()
    ref_idx, ref_sc = oracle_rows(np64(qI[0]), np64(w[0]), K[0], pos0 + np.arange(T), m, k, "bf16", "f32")
    got = idx[0].cpu().numpy()
    assert ascending_padded(got)
    differing, bad = compare_topk(got, ref_idx, ref_sc, 1e-6)
    assert not bad and differing <= 0.05 * T
