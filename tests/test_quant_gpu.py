"""GPU parity of the quantised-KV path (FP8 E4M3, q8_0, q4_0).

* pa_attend_kv decodes random codes and scales (drawn directly by the input
  generator, never produced by an encoder) and must match FP64 attention over
  the oracle's decoding of the same codes, within the bf16 tolerances.  Page
  tails hold NaN codes or scales that must never be read.
* pa_write_kv_cache must produce, bit for bit, the codes and scales the
  oracle's encoder gives for the same new rows at the same positions.
* Appending with the library and attending with the library must match the
  oracle encoding, decoding and attending on its own.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_attend_amd as pk
from oracle import quant
from oracle.paging import write_kv as ref_scatter
from paged_kv_cache_attend_amd import inputs

from gpu_util import DEV, LSE_SENTINEL, OUT_SENTINEL, compare, out_bound, say

pytestmark = pytest.mark.gpu

FMT = {"fp8": pk.KV_FP8_E4M3, "q8_0": pk.KV_Q8_0, "q4_0": pk.KV_Q4_0}


def _t(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:  # fp16 scale bits
        return torch.from_numpy(a.view(np.int16).copy()).to(DEV).view(torch.float16)
    return torch.from_numpy(a.copy()).to(DEV)


def _cache(fmt, kc, vc, ks, vs, k_scale, v_scale):
    return pk.QuantCache(FMT[fmt], _t(kc), _t(vc), None if ks is None else _t(ks),
                         None if vs is None else _t(vs), k_scale, v_scale)


def _run(p, cache, q_bits, partition_size=0):
    t = inputs.to_device(p, q_bits, np.zeros((1, 1, 1, 1), np.uint16), np.zeros((1, 1, 1, 1), np.uint16), DEV)
    out = torch.full(q_bits.shape, OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.full(q_bits.shape[:2], LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
    pk.attend_kv(t["q"], cache, t["block_table"], t["ctx_lens"], t["q_lens"], float(p.scale), out, lse,
                 max_q_len=1, max_ctx_len=p.max_ctx_len, partition_size=partition_size)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


def _oracle(p, fmt, pages, q_bits, seqs=None):
    kc, vc, ks, vs, k_scale, v_scale = pages
    kd = quant.decode_cache(kc, ks, fmt, k_scale)
    vd = quant.decode_cache(vc, vs, fmt, v_scale)
    return oracle.attend_fp64(q_bits, kd, vd, p.block_table, p.ctx_lens, p.q_lens, p.scale,
                              p.num_kv_heads, p.block_size, seqs=seqs)


CASES = [
    ("tiny", dict(ctx=[37, 100], hq=8, hkv=2), [0, 32]),
    ("ragged", dict(ctx=[1, 15, 16, 17, 300, 0, 2303, 64], hq=32, hkv=8), [0, 128, 512]),
    ("mha", dict(ctx=[200, 31, 999], hq=4, hkv=4), [0, 64]),
    ("gqa2", dict(ctx=[500, 7, 1000], hq=8, hkv=4), [0, 256]),
]


@pytest.mark.parametrize("fmt", list(FMT))
@pytest.mark.parametrize("name,case,parts", CASES, ids=[c[0] for c in CASES])
def test_attend_kv_matches_oracle(fmt, name, case, parts):
    ctx = case["ctx"]
    ql = [1 if n > 0 else 0 for n in ctx]
    p = inputs.make_problem(f"q_{name}", 90 + len(name), ctx, ql, case["hq"], case["hkv"])
    pages = inputs.quant_pages(p, fmt)
    q_bits, _, _ = p.layer(0)
    ref = _oracle(p, fmt, pages, q_bits)
    cache = _cache(fmt, *pages)
    for ps in parts:
        say(f"attend_kv {fmt} {name} partition_size={ps}")
        got = _run(p, cache, q_bits, ps)
        compare(p, got, ref, label=f"{fmt} {name} ps={ps}")


@pytest.mark.parametrize("fmt", list(FMT))
def test_attend_kv_zombie_slots_write_nothing(fmt):
    p = inputs.make_problem("q_zombie", 17, [50, 0, 80, 40], [1, 1, 0, 1], 8, 2)
    pages = inputs.quant_pages(p, fmt)
    q_bits, _, _ = p.layer(0)
    got = _run(p, _cache(fmt, *pages), q_bits, 32)
    compare(p, got, _oracle(p, fmt, pages, q_bits), label=f"{fmt} zombies")


@pytest.mark.parametrize("fmt", list(FMT))
def test_attend_kv_full_size_qwen3_short_decode(fmt):
    # 16 slots x 2303 keys, 32/8 heads, the automatic partition; the oracle
    # checks four slots.
    p = inputs.qwen3_short_decode(num_layers=1)
    pages = inputs.quant_pages(p, fmt)
    q_bits, _, _ = p.layer(0)
    say(f"attend_kv {fmt} full size")
    ob, lb = _run(p, _cache(fmt, *pages), q_bits)
    seqs = [0, 5, 10, 15]
    out, lse, written = _oracle(p, fmt, pages, q_bits, seqs=seqs)
    rows = np.zeros(p.total_q, dtype=bool)
    rows[seqs] = True
    o = oracle.bf16_bits_to_f64(ob[rows])
    err = np.abs(o - out[rows])
    assert (err <= out_bound(out[rows])).all() and err.mean() <= 1e-3, (err.max(), err.mean())
    assert np.abs(lb[rows] - lse[rows]).max() <= 1e-3
    assert np.isfinite(oracle.bf16_bits_to_f64(ob)).all()


def _encode_rows(fmt, rows_bits, scale):
    vals = oracle.bf16_bits_to_f64(rows_bits).astype(np.float32)
    return quant.encode_cache(vals, fmt, scale)


@pytest.mark.parametrize("fmt", list(FMT))
def test_write_kv_cache_bit_exact(fmt):
    ss = np.random.SeedSequence(inputs.SEED_BASE + 700 + list(FMT).index(fmt))
    rng = np.random.default_rng(ss)
    nb, hkv, mb = 48, 2, 8
    ctx = np.array([37, 0, 128, 5, 90, 17], dtype=np.int32)
    ql = np.array([1, 3, 40, 0, 33, 17], dtype=np.int32)
    table = rng.permutation(nb)[: len(ctx) * mb].reshape(len(ctx), mb).astype(np.int32)
    total = int(ql.sum())
    kn = inputs.normal_bf16(inputs.child_seed(ss, 0), (total, hkv, 128))
    vn = inputs.normal_bf16(inputs.child_seed(ss, 1), (total, hkv, 128))
    kn[0, 0, :32] = 0                        # an all-zero group
    vn[1, 1, 5] = 0x4780                     # 65536: one large value in a group
    p = inputs.make_problem("w", 1, [16] * 3, [1] * 3, 8, hkv, num_blocks=nb)
    base = inputs.quant_pages(p, fmt)
    kc0, vc0, ks0, vs0, k_scale, v_scale = base
    cache = _cache(fmt, *base)
    say(f"write_kv_cache {fmt} rows={total}")
    pk.write_kv_cache(_t(kn).view(torch.bfloat16), _t(vn).view(torch.bfloat16), _t(table), _t(ctx), _t(ql),
                      cache, max_q_len=int(ql.max()))
    torch.cuda.synchronize()
    kc, vc = kc0.copy(), vc0.copy()
    kcode, kscl = _encode_rows(fmt, kn, k_scale)
    vcode, vscl = _encode_rows(fmt, vn, v_scale)
    ref_scatter(kc, vc, kcode, vcode, table, ctx, ql)
    assert np.array_equal(cache.k_codes.cpu().numpy(), kc)
    assert np.array_equal(cache.v_codes.cpu().numpy(), vc)
    if ks0 is not None:
        ks, vs = ks0.copy(), vs0.copy()
        ref_scatter(ks, vs, kscl, vscl, table, ctx, ql)
        got_ks = cache.k_scales.cpu().numpy().view(np.uint16)
        got_vs = cache.v_scales.cpu().numpy().view(np.uint16)
        for got, want, name in ((got_ks, ks, "K"), (got_vs, vs, "V")):
            bad = np.argwhere(got != want)
            assert bad.size == 0, f"{name} scales differ at {bad[:6].tolist()}: " \
                f"{[hex(int(got[tuple(i)])) for i in bad[:6]]} vs {[hex(int(want[tuple(i)])) for i in bad[:6]]}"


@pytest.mark.parametrize("fmt", list(FMT))
def test_append_then_attend_matches_oracle(fmt):
    # Prompt rows written by the library's encoder, then a decode step; the
    # oracle encodes the same rows itself, decodes and attends.
    p = inputs.make_problem("qa", 23, [70, 129, 16], [70, 129, 16], 8, 2)
    ss = np.random.SeedSequence(inputs.SEED_BASE + 760)
    total = int(p.q_lens.sum())
    kn = inputs.normal_bf16(inputs.child_seed(ss, 0), (total, 2, 128))
    vn = inputs.normal_bf16(inputs.child_seed(ss, 1), (total, 2, 128))
    k_scale, v_scale = 1.0 / 16, 1.0 / 16
    cache = pk.QuantCache.empty(FMT[fmt], p.num_blocks, 2, DEV, k_scale, v_scale)
    table, ctx, ql = _t(p.block_table), _t(p.ctx_lens), _t(p.q_lens)
    pk.write_kv_cache(_t(kn).view(torch.bfloat16), _t(vn).view(torch.bfloat16), table, ctx, ql, cache,
                      max_q_len=int(p.q_lens.max()))
    q_bits = inputs.normal_bf16(inputs.child_seed(ss, 2), (3, 8, 128))
    one = _t(np.ones(3, dtype=np.int32))
    out = torch.empty((3, 8, 128), dtype=torch.bfloat16, device=DEV)
    lse = torch.empty((3, 8), dtype=torch.float32, device=DEV)
    pk.attend_kv(_t(q_bits).view(torch.bfloat16), cache, table, ctx, one, float(p.scale), out, lse,
                 max_q_len=1, max_ctx_len=p.max_ctx_len, partition_size=32)
    torch.cuda.synchronize()
    # oracle: encode the rows, scatter, decode, attend
    shape = (p.num_blocks, 2, 16, 64 if fmt == "q4_0" else 128)
    kc = np.zeros(shape, dtype=np.int8 if fmt == "q8_0" else np.uint8)
    vc = np.zeros_like(kc)
    kcode, kscl = _encode_rows(fmt, kn, k_scale)
    vcode, vscl = _encode_rows(fmt, vn, v_scale)
    ref_scatter(kc, vc, kcode, vcode, p.block_table, p.ctx_lens, p.q_lens)
    ks = vs = None
    if kscl is not None:
        ks = np.zeros((p.num_blocks, 2, 16, 4), dtype=np.uint16)
        vs = np.zeros_like(ks)
        ref_scatter(ks, vs, kscl, vscl, p.block_table, p.ctx_lens, p.q_lens)
    kd = quant.decode_cache(kc, ks, fmt, k_scale)
    vd = quant.decode_cache(vc, vs, fmt, v_scale)
    ref = oracle.attend_fp64(q_bits, kd, vd, p.block_table, p.ctx_lens, np.ones(3, np.int32), p.scale, 2)
    compare(p, (out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()), ref,
            label=f"append+attend {fmt}")
