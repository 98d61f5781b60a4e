"""Pins of the oracle's number formats (CPU only).

BF16 and FP8 E4M3 rounding are pinned to torch's own casts (library
routines); the FP8 decode table to torch's float8_e4m3fn view and to values
fixed by the OFP8 specification; E2M1 and the MX scale rule (MXFP4 and
MXFP8) to the OCP MX v1.0 definitions checked by exhaustive enumeration /
brute-force nearest search."""
import numpy as np
import pytest
import torch

from oracle import formats as F


def test_fp8_decode_all_codes_match_torch():
    codes = np.arange(256, dtype=np.uint8)
    ours = F.fp8_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # OFP8: only S.1111.111 is NaN; max 448; min subnormal 2^-9; min normal 2^-6
    assert list(np.nonzero(nan)[0]) == [0x7F, 0xFF]
    assert ours[0x7E] == 448.0 and ours[0x01] == 2.0 ** -9 and ours[0x08] == 2.0 ** -6


def test_fp8_encode_roundtrip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF, 0x80)], dtype=np.uint8)
    assert np.array_equal(F.fp8_encode(F.fp8_decode(codes)), codes)


def test_fp8_round_matches_torch_including_midpoints():
    pos = F.fp8_decode(np.arange(0, 0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    rng = np.random.default_rng(1)
    rnd = rng.uniform(-448, 448, 20000).astype(np.float32).astype(np.float64)
    small = (rng.standard_normal(20000) * 0.05).astype(np.float32).astype(np.float64)
    x = np.concatenate([mids, -mids, rnd, small, pos, -pos])
    ours = F.fp8_round(x)
    ref = torch.from_numpy(x).to(torch.float32).to(torch.float8_e4m3fn).to(torch.float64).numpy()
    assert np.array_equal(ours, ref)


def test_fp8_saturates():
    x = np.array([448.0, 463.9, 464.0, 500.0, 1e6, -1e6])
    assert np.array_equal(F.fp8_round(x), [448, 448, 448, 448, 448, -448])


def test_bf16_matches_torch_including_midpoints():
    rng = np.random.default_rng(2)
    x = (rng.standard_normal(50000) * np.exp(rng.uniform(-20, 20, 50000))).astype(np.float32)
    bits = x.view(np.uint32)
    mids = ((bits & 0xFFFF0000) | 0x8000).view(np.float32)   # exact BF16 midpoints
    xx = np.concatenate([x, mids]).astype(np.float64)
    ref = torch.from_numpy(xx.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(F.to_bf16(xx), ref)


def test_e2m1_table_and_rne():
    vals = F.e2m1_decode(np.arange(16))
    assert list(vals[:8]) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert list(vals[9:]) == [-0.5, -1, -1.5, -2, -3, -4, -6]
    # brute force: nearest representable value, ties to the even code
    grid = np.arange(-8, 8.0001, 1 / 64)
    table = F.E2M1_VALUES
    for x in grid:
        a = min(abs(x), 6.0)
        d = np.abs(table - a)
        best = np.nonzero(d == d.min())[0]
        pick = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert F.e2m1_round(np.array([x]))[0] == np.copysign(table[pick], x) or table[pick] == 0


def test_mx_scale_rule():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((200, 64)) * np.exp(rng.uniform(-5, 5, (200, 1)))
    vals, codes, sc = F.mxfp4_quantize(x)
    blocks = np.abs(x).reshape(200, 2, 32).max(-1)
    expect = np.floor(np.log2(blocks)).astype(int) - 2 + 127
    assert np.array_equal(sc.astype(int), expect)
    # the largest element of each block lands in [4, 6] after scaling
    Xs = np.ldexp(1.0, sc.astype(int) - 127)
    scaled_max = np.abs(vals).reshape(200, 2, 32).max(-1) / Xs
    assert np.all((scaled_max >= 4) & (scaled_max <= 6))
    assert np.array_equal(F.mxfp4_decode(codes, sc), vals)
    # a zero block gets the smallest scale and all-zero codes
    v0, c0, s0 = F.mxfp4_quantize(np.zeros((1, 32)))
    assert s0[0, 0] == 0 and not c0.any() and not v0.any()


def _e4m3_nearest_brute(v):
    """Nearest E4M3 value to v by scanning all 127 finite magnitudes (ties to
    the even code), saturating at 448; independent of round_rne."""
    mags = F.fp8_decode(np.arange(0x7F))
    d = np.abs(mags - min(abs(v), 448.0))
    best = np.nonzero(d == d.min())[0]
    pick = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
    return np.copysign(mags[pick], v), pick


def test_mxfp8_brute_force():
    """MXFP8 (OCP MX v1.0, E4M3 elements): shared exponent by a plain search
    (the e with 2^(e+8) <= amax < 2^(e+9)), then each element the nearest E4M3
    value of x / 2^e by enumeration."""
    rng = np.random.default_rng(11)
    x = rng.standard_normal((40, 64)) * np.exp(rng.uniform(-6, 6, (40, 1)))
    x[3, :32] = 0.0                                          # a zero block
    x[5, 7] = 1.9375 * 2.0 ** 3                              # scales to 496: saturates
    x[5, :7] = x[5, 8:32] = 0.01
    vals, codes, sc = F.mxfp8_quantize(x)
    for r in range(x.shape[0]):
        for blk in range(2):
            xb = x[r, 32 * blk:32 * blk + 32]
            amax = np.abs(xb).max()
            if amax == 0:
                assert sc[r, blk] == 0 and not codes[r, 32 * blk:32 * blk + 32].any()
                continue
            e = -130
            while 2.0 ** (e + 1 + 8) <= amax:
                e += 1
            assert sc[r, blk] == e + 127
            for i, v in enumerate(xb):
                q, c = _e4m3_nearest_brute(v / 2.0 ** e)
                assert vals[r, 32 * blk + i] == q * 2.0 ** e
                assert codes[r, 32 * blk + i] & 0x7F == c
    assert codes[5, 7] == 0x7E and vals[5, 7] == 448.0 * 2.0 ** (3 - 8)


def test_mxfp8_closed_forms():
    # a block of 2^k: every element scales to 256 = 2^8 (code 0x78), exact
    for k in (-20, 0, 7):
        v, c, s = F.mxfp8_quantize(np.full((1, 32), 2.0 ** k))
        assert (c == 0x78).all() and s[0, 0] == k - 8 + 127 and (v == 2.0 ** k).all()
    # scaling a block by 2^j shifts the scale byte by j and keeps the codes
    x = np.random.default_rng(12).standard_normal((8, 96))
    v0, c0, s0 = F.mxfp8_quantize(x)
    v1, c1, s1 = F.mxfp8_quantize(x * 2.0 ** 9)
    assert np.array_equal(c0, c1) and np.array_equal(s1.astype(int), s0.astype(int) + 9)
    assert np.array_equal(v1, v0 * 2.0 ** 9)
    # error: half an E4M3 ulp (relative 2^-4) in the normal range, the
    # subnormal quantum 2^(e-10) below it; a saturated element at most 1/8
    Xs = np.ldexp(1.0, np.repeat(s0.astype(int) - 127, 32, axis=1))
    sat = np.abs(x / Xs) > 448.0
    err = np.abs(v0 - x)
    assert np.all(err[~sat] <= np.maximum(np.abs(x) * 2.0 ** -4, Xs * 2.0 ** -10)[~sat] * (1 + 1e-12))
    assert sat.any() and np.all(err[sat] <= np.abs(x[sat]) / 8) and np.all(np.abs(v0[sat]) == 448.0 * Xs[sat])
    assert np.array_equal(F.fp8_decode(c0) * Xs, v0)


def test_fp8_entry_scale():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((50, 512)) * 3
    v, codes, s = F.fp8_entry_quantize(x)
    amax = np.abs(x).max(1)
    assert np.allclose(s, amax / 448, rtol=1e-7)
    assert np.all(np.abs(v).max(1) <= 448 * s)
    # every element within half an E4M3 ulp (relative 2^-4) or the subnormal quantum
    err = np.abs(v - x)
    bound = np.maximum(np.abs(x) * 2.0 ** -4, s[:, None] * 2.0 ** -10)
    assert np.all(err <= bound * (1 + 1e-12))
    assert np.array_equal(F.fp8_decode(codes) * s[:, None], v)
    v0, c0, s0 = F.fp8_entry_quantize(np.zeros((1, 8)))
    assert s0[0] == 1.0 and not c0.any()


@pytest.mark.parametrize("fmt", ["f32", "bf16"])
def test_plain_formats_idempotent(fmt):
    from oracle import csa
    x = np.random.default_rng(5).standard_normal(1000)
    y, _ = csa.store_format(x, fmt)
    z, _ = csa.store_format(y, fmt)
    assert np.array_equal(y, z)
