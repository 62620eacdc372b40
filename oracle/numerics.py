"""Storage formats used at the boundary of the CSA path: bfloat16 and OCP FP8 E4M3 ("e4m3fn").

TEST INFRASTRUCTURE ONLY (see the package docstring).

The pages fix the storage precisions but not their bit layouts: compressed KV entries are BF16
and the indexer path runs in FP8/FP4 ("DeepSeek V4 模型技术大全", chapter "Attention", section
"注意力实现细节": mixed BF16/FP8 KV storage and a low-precision Lightning Indexer).  The layouts
below are the public format definitions, written out from the bit fields:

* bfloat16: 1 sign bit, 8 exponent bits (bias 127), 7 fraction bits; the upper half of an
  IEEE-754 binary32.  Rounding from a wider value is round-to-nearest, ties-to-even (RNE).
* E4M3 (OCP 8-bit floating point, "fn" variant): 1 sign bit, 4 exponent bits (bias 7), 3
  mantissa bits; no infinities; S.1111.111 is NaN; largest finite magnitude 448; exponent
  field 0 encodes subnormals m/8 * 2^-6.
* MXFP4 (OCP Microscaling Formats v1.0): blocks of 32 consecutive elements share one E8M0
  scale (an 8-bit biased exponent, value 2^(byte-127), byte 255 = NaN); each element is E2M1
  (1 sign bit, 2 exponent bits with bias 1, 1 mantissa bit: magnitudes 0, 0.5, 1, 1.5, 2, 3, 4,
  6, exponent field 0 = subnormal 0/0.5).  The shared exponent of a block is
  floor(log2(max|v|)) - 2, 2 being the largest E2M1 exponent, and each element is v / 2^exp
  rounded to E2M1 with ties to the even code and saturation at 6.
"""
import numpy as np

# ----------------------------------------------------------------------------- bfloat16

def bf16_bits_to_f64(bits):
    """Decode bf16 bit patterns (uint16) to float64: the bits are the top half of a binary32."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return b.view(np.float32).astype(np.float64)


def f64_to_bf16_bits(x):
    """Round float64 values to bf16 with round-to-nearest-even, returning uint16 bit patterns.

    Done directly from float64 (no intermediate binary32 rounding): for a value with binary
    exponent E (x = f * 2^E, 0.5 <= |f| < 1) the bf16 quantum is 2^(E-8) for normals and 2^-133
    for subnormals; np.round rounds half to even.  Overflow past the largest finite bf16 goes to
    infinity (IEEE behaviour of RNE); NaN maps to the canonical quiet NaN 0x7FC0.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    flat_x = x.reshape(-1)
    flat_o = out.reshape(-1)
    nan = np.isnan(flat_x)
    fin = np.isfinite(flat_x)
    _, e = np.frexp(flat_x)
    qexp = np.maximum(e - 8, -133).astype(np.float64)
    quantum = np.exp2(qexp)
    q = np.where(fin, np.round(flat_x / np.where(fin, quantum, 1.0)) * quantum, flat_x)
    max_bf16 = (2.0 - 2.0 ** -7) * 2.0 ** 127
    q = np.where(fin & (np.abs(q) > max_bf16), np.copysign(np.inf, flat_x), q)
    with np.errstate(over="ignore", invalid="ignore"):
        as32 = q.astype(np.float32)  # exact: q is representable in bf16 (or is +-inf)
    bits = (as32.view(np.uint32) >> np.uint32(16)).astype(np.uint16)
    flat_o[:] = np.where(nan, np.uint16(0x7FC0), bits)
    return out


# ----------------------------------------------------------------------------- E4M3

def _e4m3_value(code):
    s = (code >> 7) & 1
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return float("nan")
    if e == 0:
        v = (m / 8.0) * 2.0 ** -6
    else:
        v = (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return -v if s else v


_E4M3 = np.array([_e4m3_value(c) for c in range(256)], dtype=np.float64)


def e4m3_table():
    """The 256-entry decode table (float64), index = code byte."""
    return _E4M3.copy()


def e4m3_decode(codes):
    """Decode E4M3 code bytes (uint8) to float64."""
    return _E4M3[np.asarray(codes, dtype=np.uint8)]


# non-negative finite codes 0x00..0x7E in increasing value order
_POS_VALS = _E4M3[:0x7F]


def e4m3_encode(x):
    """Round float64 values to E4M3 codes: nearest representable value, ties to the even code
    (even mantissa), magnitudes beyond 448 saturate to +-448 (the 'fn' format has no infinity).
    The sign bit follows the sign of x (so -0.0 and small negatives that round to zero give
    0x80).  NaN input gives 0x7F.
    """
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 448.0)
    # candidate codes: the largest non-negative code whose value <= a, and the next one up
    lo = np.searchsorted(_POS_VALS, a, side="right") - 1
    lo = np.clip(lo, 0, 0x7E)
    hi = np.clip(lo + 1, 0, 0x7E)
    dlo = a - _POS_VALS[lo]
    dhi = _POS_VALS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    neg = np.signbit(x)
    code = np.where(neg, code | np.uint8(0x80), code).astype(np.uint8)
    code = np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)
    return code


def quantize_rows_e4m3(x):
    """Per-row E4M3 quantization with one float32 scale per row.

    Reading R5 (the pages say only that the indexer runs in low precision): scale = max|row| /
    448 stored as float32 (1.0 for an all-zero row), codes = e4m3_encode(row / scale), so the
    row's largest magnitude maps to the largest finite code.  Returns (codes uint8, scale f32).
    """
    x = np.asarray(x, dtype=np.float64)
    amax = np.max(np.abs(x), axis=-1)
    scale = np.where(amax > 0, amax / 448.0, 1.0).astype(np.float32)
    codes = e4m3_encode(x / scale.astype(np.float64)[..., None])
    return codes, scale


# ----------------------------------------------------------------------------- MXFP4

# E2M1 magnitudes of codes 0..7 (code bit 3 is the sign)
_E2M1_POS = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)
_E2M1 = np.concatenate([_E2M1_POS, -_E2M1_POS])
MX_BLOCK = 32


def e2m1_decode(codes):
    """Decode E2M1 codes (0..15, sign in bit 3) to float64."""
    return _E2M1[np.asarray(codes, dtype=np.uint8) & np.uint8(0xF)]


def e2m1_encode(x):
    """Round float64 values to E2M1 codes: nearest magnitude, ties to the even code (mantissa
    bit 0), magnitudes beyond 6 saturate to 6.  The sign bit follows the sign of x, so values
    that round to zero keep their sign (code 8 for negatives)."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), 6.0)
    lo = np.clip(np.searchsorted(_E2M1_POS, a, side="right") - 1, 0, 7)
    hi = np.clip(lo + 1, 0, 7)
    dlo = a - _E2M1_POS[lo]
    dhi = _E2M1_POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi != lo) & ((hi & 1) == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    return np.where(np.signbit(x), code | np.uint8(8), code).astype(np.uint8)


def mx_shared_exponent(amax):
    """Shared exponent of an MXFP4 block with largest magnitude amax: floor(log2(amax)) - 2,
    clamped to the E8M0 range [-127, 127]; an all-zero block takes -127.  floor(log2) comes
    from the binary exponent of frexp (amax = f * 2^e, 0.5 <= f < 1), so it is exact."""
    amax = np.asarray(amax, dtype=np.float64)
    _, e = np.frexp(amax)
    se = (e.astype(np.int64) - 1) - 2
    se = np.where(amax > 0, se, -127)
    return np.clip(se, -127, 127)


def quantize_rows_mxfp4(x):
    """MXFP4 quantization of rows whose length is a multiple of 32 (reading: the indexer keys'
    FP4 format is OCP MXFP4 with blocks of 32 consecutive dims).  Returns (packed uint8
    [..., d/2]: element 2i in the low nibble of byte i, element 2i+1 in the high nibble;
    scales uint8 [..., d/32]: E8M0 byte = shared exponent + 127)."""
    x = np.asarray(x, dtype=np.float64)
    d = x.shape[-1]
    assert d % MX_BLOCK == 0
    blocks = x.reshape(x.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    se = mx_shared_exponent(np.max(np.abs(blocks), axis=-1))
    codes = e2m1_encode(blocks / np.exp2(se.astype(np.float64))[..., None]).reshape(x.shape)
    packed = (codes[..., 0::2] | (codes[..., 1::2] << np.uint8(4))).astype(np.uint8)
    return packed, (se + 127).astype(np.uint8)


def mxfp4_decode(packed, scales):
    """Real values of MXFP4 rows: packed uint8 [..., d/2], scales uint8 [..., d/32]."""
    packed = np.asarray(packed, dtype=np.uint8)
    scales = np.asarray(scales, dtype=np.uint8)
    codes = np.empty(packed.shape[:-1] + (2 * packed.shape[-1],), dtype=np.uint8)
    codes[..., 0::2] = packed & np.uint8(0xF)
    codes[..., 1::2] = packed >> np.uint8(4)
    vals = e2m1_decode(codes)
    d = vals.shape[-1]
    blocks = vals.reshape(vals.shape[:-1] + (d // MX_BLOCK, MX_BLOCK))
    mult = np.exp2(scales.astype(np.float64) - 127.0)
    return (blocks * mult[..., None]).reshape(vals.shape)
