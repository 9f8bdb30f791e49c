"""KV page formats with fewer bytes per value: q8_0, q4_0 and FP8 (E4M3).

TEST INFRASTRUCTURE ONLY -- imported by tests, never by the product path.
Shares no code with the HIP library.

What the pages fix
------------------
The inference-optimisation chapter, section 8.4.2 ("KV compression and read
cost", Fig. 8-23): values are quantised in groups; each group keeps low-bit
codes plus a scale from which approximate values are recovered.  q8_0 gives
every 32 values one 2-byte scale and 32 one-byte codes (34 bytes where bf16
needs 64); q4_0 uses the same grouping with 4-bit codes (18 bytes).  Section
8.4.4: an FP8 KV cache with the query kept in bf16 (changing only the query's
precision changed answers, so the query stays bf16 here).

Readings (where the pages leave the encoding open)
--------------------------------------------------
* groups are 32 consecutive dimensions of one token row of one KV head (a
  128-dim row has 4 groups); the scale is an IEEE binary16 value;
* q8_0: d = max|x| / 127 in fp32, stored as fp16 (round to nearest even);
  code = x / d_stored in fp32, rounded half away from zero, clamped to
  [-127, 127]; value = code * d_stored;
* q4_0: m = the group's value of largest magnitude (the first one on ties),
  d = m / -8 stored as fp16; code = x / d_stored rounded half away from zero,
  clamped to [-8, 7], stored as code + 8 in a nibble; value = (nibble - 8) *
  d_stored.  The extreme value maps to code -8 exactly;
* a stored scale of zero gives codes 0 (values 0) and is stored as +0 (the
  sign of a zero scale changes no value, so it is fixed to one pattern);
* FP8 is the OCP E4M3 format (sign, 4 exponent bits with bias 7, 3 mantissa
  bits; no infinities; S.1111.111 is NaN; largest finite 448); code = the
  E4M3 value nearest to x / s (fp32 division), ties to the even code,
  saturating at +-448; value = decode(code) * s, with s one fp32 scale per
  cache (K and V each) chosen by the caller;
* divisions are fp32 and correctly rounded, the precision the kernels use,
  so both sides take every integer decision the same way.

Everything a test compares is computed here in float64 from those codes.
"""

from __future__ import annotations

import numpy as np

GROUP = 32


def fp16_bits(x32: np.ndarray) -> np.ndarray:
    """fp32 -> IEEE binary16 bit patterns, round to nearest even."""
    return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)


def fp16_value(bits: np.ndarray) -> np.ndarray:
    return np.asarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def _round_half_away(x64: np.ndarray) -> np.ndarray:
    """Round to the nearest integer, halves away from zero (exact in float64
    for any float32 input: |x| + 0.5 is exact there)."""
    return np.sign(x64) * np.floor(np.abs(x64) + 0.5)


def _groups(x: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float32)
    if x.shape[-1] % GROUP:
        raise ValueError("last dimension must be a multiple of 32")
    return x.reshape(*x.shape[:-1], x.shape[-1] // GROUP, GROUP)


# -- q8_0 ---------------------------------------------------------------------

def q8_0_encode(x):
    """x: float32 [..., D] -> (codes int8 [..., D], scale bits uint16 [..., D/32])."""
    g = _groups(x)
    amax = np.abs(g).max(axis=-1)
    d = (amax / np.float32(127)).astype(np.float32)          # fp32, correctly rounded
    d_bits = fp16_bits(d)
    d_bits = np.where(fp16_value(d_bits) == 0, np.uint16(0), d_bits)   # +0, not -0
    d_st = fp16_value(d_bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g / d_st[..., None]).astype(np.float32)      # fp32 division
    q = _round_half_away(ratio.astype(np.float64))
    q = np.where(d_st[..., None] == 0, 0, np.clip(q, -127, 127))
    return q.astype(np.int8).reshape(np.shape(x)), d_bits


def q8_0_decode(codes, scale_bits):
    c = np.asarray(codes, dtype=np.int8)
    g = c.reshape(*c.shape[:-1], c.shape[-1] // GROUP, GROUP).astype(np.float64)
    return (g * fp16_value(scale_bits)[..., None]).reshape(c.shape)


# -- q4_0 ---------------------------------------------------------------------

def q4_0_encode(x):
    """x: float32 [..., D] -> (packed nibbles uint8 [..., D/2], scale bits
    uint16 [..., D/32]).  Byte b holds dim 2b in its low nibble and dim 2b+1
    in its high nibble."""
    g = _groups(x)
    idx = np.abs(g).argmax(axis=-1)                             # first on ties
    m = np.take_along_axis(g, idx[..., None], axis=-1)[..., 0]
    d = (m / np.float32(-8)).astype(np.float32)
    d_bits = fp16_bits(d)
    d_bits = np.where(fp16_value(d_bits) == 0, np.uint16(0), d_bits)   # +0, not -0
    d_st = fp16_value(d_bits).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        ratio = (g / d_st[..., None]).astype(np.float32)
    q = _round_half_away(ratio.astype(np.float64))
    q = np.where(d_st[..., None] == 0, 0, np.clip(q, -8, 7)) + 8
    nib = q.astype(np.uint8).reshape(np.shape(x))
    packed = (nib[..., 0::2] | (nib[..., 1::2] << 4)).astype(np.uint8)
    return packed, d_bits


def q4_0_decode(packed, scale_bits):
    p = np.asarray(packed, dtype=np.uint8)
    nib = np.empty(p.shape[:-1] + (p.shape[-1] * 2,), dtype=np.int64)
    nib[..., 0::2] = p & 0xF
    nib[..., 1::2] = p >> 4
    g = nib.reshape(*nib.shape[:-1], nib.shape[-1] // GROUP, GROUP).astype(np.float64) - 8.0
    return (g * fp16_value(scale_bits)[..., None]).reshape(nib.shape)


# -- FP8 E4M3 -----------------------------------------------------------------

def e4m3_table() -> np.ndarray:
    """Value of each of the 256 E4M3 codes (float64; NaN for S.1111.111)."""
    out = np.empty(256, dtype=np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 0xF
        mant = c & 0x7
        if e == 0xF and mant == 0x7:
            out[c] = np.nan
        elif e == 0:
            out[c] = s * mant / 8.0 * 2.0 ** -6            # subnormal
        else:
            out[c] = s * (1.0 + mant / 8.0) * 2.0 ** (e - 7)
    return out


def e4m3_encode(y32) -> np.ndarray:
    """Nearest E4M3 code of each float32 value (ties to the even code,
    saturating at +-448; NaN -> 0x7F).

    The finite non-negative codes 0x00 .. 0x7E increase with their value, so
    the two candidates around |y| are found by bisection and the nearer one
    is kept (the even one on an exact tie)."""
    y = np.asarray(y32, dtype=np.float32).astype(np.float64)
    vals = e4m3_table()[:0x7F]                                # +0 .. 448
    a = np.minimum(np.abs(y), 448.0)
    a = np.where(np.isnan(a), 0.0, a)
    hi = np.clip(np.searchsorted(vals, a, side="left"), 0, 0x7E)
    lo = np.clip(hi - 1, 0, 0x7E)
    d_lo = a - vals[lo]
    d_hi = vals[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(y), code | np.uint8(0x80), code)
    return np.where(np.isnan(y), np.uint8(0x7F), code).astype(np.uint8)


def fp8_encode(x, scale: float) -> np.ndarray:
    with np.errstate(invalid="ignore"):
        y = (np.asarray(x, dtype=np.float32) / np.float32(scale)).astype(np.float32)
    return e4m3_encode(y)


def fp8_decode(codes, scale: float) -> np.ndarray:
    return e4m3_table()[np.asarray(codes, dtype=np.uint8)] * float(np.float32(scale))


# -- whole caches ---------------------------------------------------------------

def encode_cache(values_f32: np.ndarray, fmt: str, scale: float = 1.0):
    """Encode a [num_blocks][Hkv][16][D] float32 cache.  Returns (codes, scale
    bits or None)."""
    if fmt == "q8_0":
        return q8_0_encode(values_f32)
    if fmt == "q4_0":
        return q4_0_encode(values_f32)
    if fmt == "fp8":
        return fp8_encode(values_f32, scale), None
    raise ValueError(fmt)


def decode_cache(codes, scales, fmt: str, scale: float = 1.0) -> np.ndarray:
    if fmt == "q8_0":
        return q8_0_decode(codes, scales)
    if fmt == "q4_0":
        return q4_0_decode(codes, scales)
    if fmt == "fp8":
        return fp8_decode(codes, scale)
    raise ValueError(fmt)


def bytes_per_group(fmt: str) -> int:
    """Bytes that hold 32 values (section 8.4.2, Fig. 8-23)."""
    return {"bf16": 64, "q8_0": 34, "q4_0": 18, "fp8": 32}[fmt]
