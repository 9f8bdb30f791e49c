"""Pins of the quantised-KV oracle (q8_0, q4_0, FP8 E4M3) to the pages and
to brute force.

The byte counts and capacities are the ones the inference-optimisation
chapter prints in section 8.4.2 (Fig. 8-23); the codes are checked against
an exhaustive search over every code of the format; the E4M3 table against
the format's definition at a few printed points; and attention over
dequantised pages against bf16 attention where quantisation is exact.
"""

from __future__ import annotations

import numpy as np
import pytest

import oracle
from oracle import quant


def test_bytes_per_group_and_capacities():
    # Fig. 8-23: 32 values take 64 B in bf16, 34 B in q8_0, 18 B in q4_0.
    assert quant.bytes_per_group("bf16") == 64
    assert quant.bytes_per_group("q8_0") == 34 == 32 + 2
    assert quant.bytes_per_group("q4_0") == 18 == 16 + 2
    # 8.5 and 4.5 bits per value with the scale
    assert quant.bytes_per_group("q8_0") * 8 / 32 == 8.5
    assert quant.bytes_per_group("q4_0") * 8 / 32 == 4.5
    # An 8K context of BF16 KV is 1152 MiB: 612 MiB in q8_0, 324 MiB in q4_0
    # (saving 540 and 828 MiB); a finished long request, 1188 MiB, becomes
    # 631.125 MiB, and 16 of them about 9.86 GiB.
    kv_8k = 8192 * 36 * 8 * 128 * 2 * 2 / 2**20
    assert kv_8k == 1152
    assert kv_8k * 34 / 64 == 612 and kv_8k * 18 / 64 == 324
    assert kv_8k - 612 == 540 and kv_8k - 324 == 828
    assert 1188 * 34 / 64 == 631.125
    assert round(16 * 631.125 / 1024, 2) == 9.86
    # The encoders produce exactly those sizes.
    x = np.zeros((3, 128), dtype=np.float32)
    c8, s8 = quant.q8_0_encode(x)
    c4, s4 = quant.q4_0_encode(x)
    assert c8.nbytes + s8.nbytes == 3 * 4 * 34
    assert c4.nbytes + s4.nbytes == 3 * 4 * 18


def _nearest_code(x32, d_stored, codes):
    """Brute force: the code whose value code * d is nearest to x (fp32
    division semantics aside, ties away from zero)."""
    vals = codes.astype(np.float64) * float(d_stored)
    err = np.abs(vals - float(x32))
    best = err.min()
    cand = codes[err == best]
    return int(cand[np.argmax(np.abs(cand))]) if len(cand) > 1 else int(cand[0])


@pytest.mark.parametrize("seed", [0, 1])
def test_q8_0_codes_are_the_nearest(seed):
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((6, 128)) * rng.uniform(0.01, 40, (6, 1))).astype(np.float32)
    x[0, :32] = 0.0                      # an all-zero group
    x[1, 32:64] = 0.0
    x[1, 40] = -3.0                      # one non-zero value
    codes, sb = quant.q8_0_encode(x)
    d = quant.fp16_value(sb)
    allc = np.arange(-127, 128)
    for r in range(x.shape[0]):
        for g in range(4):
            dd = d[r, g]
            for i in range(32):
                xv = x[r, 32 * g + i]
                want = 0 if dd == 0 else _nearest_code(np.float32(xv), np.float32(dd), allc)
                assert codes[r, 32 * g + i] == want, (r, g, i)
    assert (codes[0, :32] == 0).all() and sb[0, 0] == 0
    assert codes[1, 40] == -127
    # the scale is max|x| / 127 rounded to fp16
    amax = np.abs(x.reshape(6, 4, 32)).max(-1)
    assert np.array_equal(sb, (amax / np.float32(127)).astype(np.float32).astype(np.float16).view(np.uint16))


def test_q4_0_codes_are_the_nearest():
    rng = np.random.default_rng(3)
    x = (rng.standard_normal((6, 128)) * 5).astype(np.float32)
    x[2, 0:32] = np.linspace(-1, 1, 32, dtype=np.float32)
    x[4, 64:96] = 0.0                    # a zero group: scale stored as +0, codes 8
    packed, sb = quant.q4_0_encode(x)
    d = quant.fp16_value(sb)
    nib = np.empty((6, 128), dtype=np.int64)
    nib[:, 0::2] = packed & 0xF
    nib[:, 1::2] = packed >> 4
    allc = np.arange(-8, 8)
    for r in range(6):
        for g in range(4):
            grp = x[r, 32 * g:32 * g + 32]
            m = grp[np.argmax(np.abs(grp))]
            want_bits = np.float32(m / np.float32(-8)).astype(np.float16).view(np.uint16)
            assert sb[r, g] == (0 if m == 0 else want_bits)
            if d[r, g] == 0:
                assert (nib[r, 32 * g:32 * g + 32] == 8).all()   # zero scale: code 0
                continue
            for i in range(32):
                want = _nearest_code(np.float32(grp[i]), np.float32(d[r, g]), allc) + 8
                assert nib[r, 32 * g + i] == want, (r, g, i)
            # the value of largest magnitude maps to code -8 exactly
            assert nib[r, 32 * g + np.argmax(np.abs(grp))] == 0


def test_dequantisation_error_bounds():
    rng = np.random.default_rng(5)
    x = (rng.standard_normal((64, 128)) * 2).astype(np.float32)
    c8, s8 = quant.q8_0_encode(x)
    d8 = np.repeat(quant.fp16_value(s8), 32, axis=-1)
    amax = np.repeat(np.abs(x.reshape(64, 4, 32)).max(-1), 32, axis=-1)
    err = np.abs(quant.q8_0_decode(c8, s8) - x)
    # within half a step, plus the clamp at +-127 steps when fp16 rounded d down
    assert (err <= d8 / 2 + np.maximum(0, amax - 127 * d8) + 1e-12).all()
    c4, s4 = quant.q4_0_encode(x)
    d4 = np.abs(np.repeat(quant.fp16_value(s4), 32, axis=-1))
    err4 = np.abs(quant.q4_0_decode(c4, s4) - x)
    # values on the far side of zero from the extreme can clamp at 7 steps
    assert (err4 <= np.maximum(d4 / 2, np.abs(x) - 7 * d4) + 1e-12).all()


def test_e4m3_table_points():
    t = quant.e4m3_table()
    assert t[0x00] == 0.0 and np.signbit(t[0x80])
    assert t[0x01] == 2.0 ** -9          # smallest subnormal
    assert t[0x07] == 7 * 2.0 ** -9      # largest subnormal
    assert t[0x08] == 2.0 ** -6          # smallest normal
    assert t[0x38] == 1.0
    assert t[0x7E] == 448.0 and t[0xFE] == -448.0
    assert np.isnan(t[0x7F]) and np.isnan(t[0xFF])
    assert np.isfinite(t[0x78]) and t[0x78] == 256.0   # exponent 15 is finite except S.1111.111
    finite = t[np.isfinite(t)]
    assert len(finite) == 254
    pos = t[:0x7F]
    assert (np.diff(pos) > 0).all()


def test_e4m3_encode_nearest_even_and_saturation():
    t = quant.e4m3_table()
    # halfway between 1.0 (0x38) and 1.125 (0x39): the even code wins
    assert quant.e4m3_encode(np.float32(1.0625)) == 0x38
    assert quant.e4m3_encode(np.float32(1.1875)) == 0x3A    # between 0x39 and 0x3A
    assert quant.e4m3_encode(np.float32(500.0)) == 0x7E
    assert quant.e4m3_encode(np.float32(-1e9)) == 0xFE
    assert quant.e4m3_encode(np.float32(2.0 ** -11)) == 0x00  # a quarter step rounds to 0
    assert quant.e4m3_encode(np.float32(-2.0 ** -11)) == 0x80
    assert quant.e4m3_encode(np.float32(3 * 2.0 ** -10)) == 0x02  # halfway 1 and 2 steps: even
    # brute force over a sweep
    rng = np.random.default_rng(11)
    y = (rng.standard_normal(5000) * np.exp(rng.uniform(-8, 6, 5000))).astype(np.float32)
    c = quant.e4m3_encode(y)
    a = np.minimum(np.abs(y.astype(np.float64)), 448.0)
    pos = t[:0x7F]
    err = np.abs(a[:, None] - pos[None, :])
    best = err.min(axis=1)
    assert np.allclose(np.abs(np.abs(t[c]) - a), best, rtol=0, atol=0)


def test_attention_over_exact_quantisation_equals_bf16_attention():
    # When every value is exactly representable (small integers times the
    # cache's power-of-two scale), FP8 pages decode to the bf16 values
    # themselves, so attention over them is attention over bf16.
    rng = np.random.default_rng(2)
    nb, hkv, hq = 6, 2, 8
    ints = rng.integers(-15, 16, (nb, hkv, 16, 128)).astype(np.float32)
    vals = ints * np.float32(0.25)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    q = (rng.standard_normal((3, hq, 128)).astype(np.float32).view(np.uint32) >> 16).astype(np.uint16)
    table = np.array([[0, 1], [2, 3], [4, 5]])
    ctx, ql = np.array([20, 32, 9]), np.array([1, 1, 1])
    ref = oracle.attend_fp64(q, bits, bits, table, ctx, ql, 0.088388, hkv)
    codes = quant.fp8_encode(vals, 0.25)   # integers up to 15 are exact in E4M3
    deq = quant.fp8_decode(codes, 0.25)
    assert np.array_equal(deq, vals.astype(np.float64))
    got = oracle.attend_fp64(q, deq, deq, table, ctx, ql, 0.088388, hkv)
    assert np.array_equal(got[0], ref[0]) and np.array_equal(got[1], ref[1])
