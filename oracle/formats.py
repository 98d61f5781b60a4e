"""Number formats used by the compressed KV cache and the indexer, in fp64.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module.

Written from the public format definitions, not from any GPU code:

* BF16: IEEE-754 binary32 with the low 16 mantissa bits dropped (8 significant
  bits, 8 exponent bits), round-to-nearest-even.
* FP8 E4M3 as defined by the OCP 8-bit Floating Point Specification (OFP8):
  bias 7, 3 mantissa bits, no infinities, S.1111.111 is NaN, largest finite
  magnitude 448, smallest subnormal 2^-9.  Conversion here is RNE with
  saturation to +-448.
* MXFP4 as defined by the OCP Microscaling Formats (MX) v1.0 specification:
  blocks of 32 FP4 E2M1 elements (values 0, 0.5, 1, 1.5, 2, 3, 4, 6 and
  their negatives) sharing one E8M0 scale 2^(e-127).  The shared exponent is
  floor(log2(amax)) - emax_elem with emax_elem = 2 for E2M1; elements are
  rounded RNE and clamped to +-6.
* MXFP8 (same specification): blocks of 32 E4M3 elements sharing one E8M0
  scale; shared exponent floor(log2(amax)) - 8, elements RNE saturating to
  +-448.

The pages fix only the format names: the KV cache keeps the RoPE dims in BF16
and the rest in FP8, and the indexer runs its QK product in FP4 with scores
cast from FP32 to BF16 ("逐层剖析 CSA / HCA 混注意力" page, §1.4 精度优化叠加,
sub-sections 存储格式混 and LIGHTNING INDEXER 的 FP4 计).  MXFP8 serves the
attention's optional FP8 QK product (the query's non-RoPE dims against the
FP8 cache), a reading of the same sub-section.
"""
import numpy as np

FP8_MAX = 448.0
E2M1_MAX = 6.0
MX_BLOCK = 32


def round_rne(x, mant_bits, emin, max_val=None, saturate=False):
    """Round fp64 values to a binary format with `mant_bits` stored mantissa
    bits and minimum normal exponent `emin`, round-to-nearest-even.

    The quantum of a value in binade [2^E, 2^(E+1)) is 2^(max(E, emin) -
    mant_bits); below 2^emin the format is subnormal with the fixed quantum
    2^(emin - mant_bits).  Every step is exact in fp64 (scaling by powers of
    two and np.rint, which rounds halves to even)."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros_like(x)
    nz = x != 0
    xm = x[nz]
    _, e = np.frexp(np.abs(xm))          # |x| = f * 2^e, f in [0.5, 1)
    E = e.astype(np.int64) - 1           # |x| in [2^E, 2^(E+1))
    E = np.maximum(E, emin)
    quantum = np.ldexp(1.0, (E - mant_bits).astype(np.int64))
    q = np.rint(xm / quantum) * quantum
    if max_val is not None:
        over = np.abs(q) > max_val
        if saturate:
            q = np.where(over, np.sign(q) * max_val, q)
        elif np.any(over):
            raise OverflowError("value out of range of the target format")
    out[nz] = q
    return out


def to_bf16(x):
    """fp64 -> nearest BF16 value (RNE), returned as fp64."""
    return round_rne(x, 7, -126)


def to_f32(x):
    """fp64 -> nearest binary32 value (RNE), returned as fp64."""
    return np.asarray(x, dtype=np.float64).astype(np.float32).astype(np.float64)


def fp8_round(x):
    """fp64 -> nearest OFP8 E4M3 value (RNE, saturating), as fp64."""
    return round_rne(x, 3, -6, FP8_MAX, saturate=True)


def fp8_decode(code):
    """Decode OFP8 E4M3 bytes to fp64 (NaN for S.1111.111)."""
    c = np.asarray(code, dtype=np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    mnt = c & 0x7
    sub = mnt.astype(np.float64) * 2.0 ** -9
    nrm = (1.0 + mnt / 8.0) * np.ldexp(1.0, (e - 7))
    v = s * np.where(e == 0, sub, nrm)
    return np.where((e == 15) & (mnt == 7), np.nan, v)


def fp8_encode(v):
    """Encode fp64 values that are exactly E4M3-representable into bytes."""
    v = np.asarray(v, dtype=np.float64)
    sign = (np.signbit(v)).astype(np.int64) << 7
    a = np.abs(v)
    code = np.zeros(v.shape, dtype=np.int64)
    nz = a > 0
    an = a[nz]
    _, e = np.frexp(an)
    E = e.astype(np.int64) - 1
    normal = E >= -6
    mnt = np.where(normal, an / np.ldexp(1.0, E) * 8.0 - 8.0, an / 2.0 ** -9)
    mi = np.rint(mnt).astype(np.int64)
    if np.any(np.abs(mnt - mi) > 0):
        raise ValueError("fp8_encode: value not representable")
    ebits = np.where(normal, E + 7, 0)
    code[nz] = (ebits << 3) | mi
    return (code | sign).astype(np.uint8)


def e2m1_round(x):
    """fp64 -> nearest FP4 E2M1 value (RNE, clamped to +-6), as fp64."""
    return round_rne(x, 1, 0, E2M1_MAX, saturate=True)


E2M1_VALUES = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def e2m1_decode(code):
    """Decode 4-bit E2M1 codes (bit 3 = sign) to fp64."""
    c = np.asarray(code, dtype=np.int64)
    return np.where(c & 0x8, -1.0, 1.0) * E2M1_VALUES[c & 0x7]


def e2m1_encode(v):
    """Encode exactly-representable E2M1 values into 4-bit codes."""
    v = np.asarray(v, dtype=np.float64)
    mag = np.abs(v)
    idx = np.searchsorted(E2M1_VALUES, mag)
    idx = np.minimum(idx, 7)
    if np.any(E2M1_VALUES[idx] != mag):
        raise ValueError("e2m1_encode: value not representable")
    sign = np.signbit(v) & (mag > 0)
    return (idx | (sign.astype(np.int64) << 3)).astype(np.uint8)


def mx_scale_exponent(block_amax, emax_elem=2):
    """OCP MX v1.0 shared exponent: floor(log2 amax) - emax_elem, where
    emax_elem is the exponent of the element format's largest normal (2 for
    E2M1: 6 = 1.5 * 2^2; 8 for E4M3: 448 = 1.75 * 2^8), clamped to the E8M0
    range [-127, 127].  A block of zeros gets -127."""
    a = np.asarray(block_amax, dtype=np.float64)
    out = np.full(a.shape, -127, dtype=np.int64)
    nz = a > 0
    _, e = np.frexp(a[nz])
    out[nz] = np.clip(e.astype(np.int64) - 1 - emax_elem, -127, 127)
    return out


def mxfp4_quantize(x):
    """Quantise the last axis (a multiple of 32) to MXFP4.

    Returns (values, element_codes, scale_codes): `values` is the decoded
    fp64 tensor, element codes are 4-bit ints with the shape of x, scale
    codes are E8M0 bytes (exponent + 127) of shape [..., d/32]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    ex = mx_scale_exponent(np.max(np.abs(xb), axis=-1))
    X = np.ldexp(1.0, ex)[..., None]
    elems = e2m1_round(xb / X)
    vals = (elems * X).reshape(x.shape)
    codes = e2m1_encode(elems).reshape(x.shape)
    return vals, codes, (ex + 127).astype(np.uint8)


def mxfp8_quantize(x):
    """Quantise the last axis (a multiple of 32) to MXFP8 (OCP MX v1.0):
    blocks of 32 E4M3 elements sharing one E8M0 scale 2^e with
    e = floor(log2 amax) - 8; each element becomes RNE(x / 2^e) on the E4M3
    grid, saturating to +-448 (the block maximum lands in [256, 512) before
    rounding, so only it can saturate).

    Returns (values, element_codes, scale_codes): decoded fp64 values, E4M3
    bytes with the shape of x, E8M0 bytes (e + 127) of shape [..., d/32]."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    xb = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    ex = mx_scale_exponent(np.max(np.abs(xb), axis=-1), emax_elem=8)
    X = np.ldexp(1.0, ex)[..., None]
    elems = fp8_round(xb / X)
    vals = (elems * X).reshape(x.shape)
    codes = fp8_encode(elems).reshape(x.shape)
    return vals, codes, (ex + 127).astype(np.uint8)


def mxfp4_decode(codes, scale_codes):
    """Decode element codes [..., d] and E8M0 scale bytes [..., d/32]."""
    codes = np.asarray(codes)
    d = codes.shape[-1]
    v = e2m1_decode(codes).reshape(codes.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    X = np.ldexp(1.0, np.asarray(scale_codes, dtype=np.int64) - 127)[..., None]
    return (v * X).reshape(codes.shape)


def fp8_entry_quantize(x):
    """Per-entry scaled FP8 for the non-RoPE part of a KV entry (last axis).

    The scale is the fp32 value nearest to amax/448 (1 when the entry is all
    zeros); each element becomes RNE_sat(x / scale).  Returns (values, codes,
    scale) with values = decoded codes times scale, in fp64."""
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    s = to_f32(np.where(amax > 0, amax / FP8_MAX, 1.0))
    q = fp8_round(x / s[..., None])
    return q * s[..., None], fp8_encode(q), s
