"""GPU tests of the K/V append (pa_write_kv), the copy-on-write block copy
(pa_copy_blocks) and a decode loop driven by the block pool.

The byte-moving kernels must match the oracle's scatter and copy bit for bit.
The decode loop runs the library's pool and kernels on one side and the
oracle's allocator, cache and FP64 attention on the other, fed the same
operations and the same seeded rows; attention depends only on each slot's
logical sequence, so the two must agree although their block ids differ.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_attend_amd as pk
from oracle.paging import BlockPool, copy_blocks as ref_copy_blocks, write_kv as ref_write_kv
from paged_kv_cache_attend_amd import inputs

from gpu_util import DEV, LSE_SENTINEL, OUT_SENTINEL, compare, say

pytestmark = pytest.mark.gpu

D = 128


def _bits(ss, i, shape):
    return inputs.normal_bf16(inputs.child_seed(ss, i), shape)


def _dev_bf16(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).to(DEV).view(torch.bfloat16)


def _host_bits(t):
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


@pytest.mark.parametrize("hkv", [1, 2, 8])
def test_write_kv_bit_exact(hkv):
    # Slots with 1..40 new rows (several 16-row groups), a zombie without
    # keys, one without new rows, and new rows crossing page boundaries.
    ss = np.random.SeedSequence(inputs.SEED_BASE + 500 + hkv)
    rng = np.random.default_rng(ss)
    nb, mb = 64, 8
    ctx = np.array([37, 0, 128, 5, 90, 17], dtype=np.int32)
    ql = np.array([1, 3, 40, 0, 33, 17], dtype=np.int32)
    table = rng.permutation(nb)[: len(ctx) * mb].reshape(len(ctx), mb).astype(np.int32)
    total = int(ql.sum())
    k = _bits(ss, 0, (nb, hkv, 16, D))
    v = _bits(ss, 1, (nb, hkv, 16, D))
    kn = _bits(ss, 2, (total, hkv, D))
    vn = _bits(ss, 3, (total, hkv, D))
    say(f"write_kv hkv={hkv} rows={total}")
    kd, vd = _dev_bf16(k), _dev_bf16(v)
    pk.write_kv(_dev_bf16(kn), _dev_bf16(vn), _i32(table), _i32(ctx), _i32(ql), kd, vd,
                max_q_len=int(ql.max()))
    torch.cuda.synchronize()
    ref_write_kv(k, v, kn, vn, table, ctx, ql)
    assert np.array_equal(_host_bits(kd), k)
    assert np.array_equal(_host_bits(vd), v)


def test_write_kv_skips_out_of_range_targets():
    # A table entry outside the pool and a position beyond the table are
    # skipped; everything else is written.
    ss = np.random.SeedSequence(inputs.SEED_BASE + 520)
    nb, mb = 8, 2
    table = np.array([[3, 99], [-1, 4], [5, 6]], dtype=np.int32)
    ctx = np.array([20, 16, 40], dtype=np.int32)   # slot 2 claims 40 > 2 x 16 positions
    ql = np.array([8, 2, 12], dtype=np.int32)
    k = _bits(ss, 0, (nb, 2, 16, D))
    v = _bits(ss, 1, (nb, 2, 16, D))
    kn = _bits(ss, 2, (22, 2, D))
    vn = _bits(ss, 3, (22, 2, D))
    kd, vd = _dev_bf16(k), _dev_bf16(v)
    pk.write_kv(_dev_bf16(kn), _dev_bf16(vn), _i32(table), _i32(ctx), _i32(ql), kd, vd, max_q_len=12)
    torch.cuda.synchronize()
    want_k, want_v = k.copy(), v.copy()
    # slot 0: positions 12..19 -> block 3 slots 12..15 (rows 0..3), then block 99 (skipped)
    # slot 1: positions 14, 15 -> block -1 (skipped)
    # slot 2: positions 28..39 -> block 6 slots 12..15 (rows 10..13), rest beyond the table
    want_k[6, :, 12:16] = kn[10:14].transpose(1, 0, 2)
    want_v[6, :, 12:16] = vn[10:14].transpose(1, 0, 2)
    want_k[3, :, 12:16] = kn[0:4].transpose(1, 0, 2)
    want_v[3, :, 12:16] = vn[0:4].transpose(1, 0, 2)
    assert np.array_equal(_host_bits(kd), want_k)
    assert np.array_equal(_host_bits(vd), want_v)


def test_copy_blocks_bit_exact():
    ss = np.random.SeedSequence(inputs.SEED_BASE + 530)
    nb, hkv = 32, 4
    k = _bits(ss, 0, (nb, hkv, 16, D))
    v = _bits(ss, 1, (nb, hkv, 16, D))
    pairs = [(3, 17), (17, 4), (30, 0), (5, 99)]   # the last is outside the pool: skipped
    kd, vd = _dev_bf16(k), _dev_bf16(v)
    # (3 -> 17) and (17 -> 4) in one call would read a block another copy
    # writes; the contract forbids it, so they go in two calls.
    for chunk in (pairs[:1], pairs[1:]):
        src = _i32([s for s, _ in chunk])
        dst = _i32([d for _, d in chunk])
        pk.copy_blocks(src, dst, kd, vd)
    torch.cuda.synchronize()
    ref_copy_blocks(k, v, pairs[:1])
    ref_copy_blocks(k, v, pairs[1:3])
    assert np.array_equal(_host_bits(kd), k)
    assert np.array_equal(_host_bits(vd), v)


def test_decode_loop_through_the_pool():
    # Prompts, a fork sharing a partly filled tail (copy-on-write on both
    # branches' next tokens), decode steps with one new token per live slot,
    # a release with its fence retired after the stream has passed, and a
    # new request reusing the freed blocks.
    ss = np.random.SeedSequence(inputs.SEED_BASE + 540)
    NB, p, S, MB, HQ, HKV = 40, 16, 4, 8, 8, 2
    scale = 1.0 / np.sqrt(D)
    lib_pool, ref_pool = pk.Pool(NB, p, S, MB), BlockPool(NB, p, S, MB)
    kc = torch.zeros((NB, HKV, p, D), dtype=torch.bfloat16, device=DEV)
    vc = torch.zeros_like(kc)
    ref_k = np.zeros((NB, HKV, p, D), dtype=np.uint16)
    ref_v = np.zeros_like(ref_k)
    draw = [0]

    def fresh(shape):
        draw[0] += 1
        return _bits(ss, draw[0], shape)

    def append(new_rows):
        """new_rows: {slot: m}.  Grow both pools, copy, then write the rows."""
        for slot, m in new_rows.items():
            a, b = lib_pool.append(slot, m), ref_pool.append(slot, m)
            assert a is not None and b is not None and len(a) == len(b)
            if a:
                pk.copy_blocks(_i32([s for s, _ in a]), _i32([d for _, d in a]), kc, vc)
            ref_copy_blocks(ref_k, ref_v, b)
        ql = np.array([new_rows.get(s, 0) for s in range(S)], dtype=np.int32)
        ctx = np.array([ref_pool.lengths[s] for s in range(S)], dtype=np.int32)
        assert list(ctx) == [lib_pool.length(s) for s in range(S)]
        total = int(ql.sum())
        kn, vn = fresh((total, HKV, D)), fresh((total, HKV, D))
        pk.write_kv(_dev_bf16(kn), _dev_bf16(vn), _i32(lib_pool.table()), _i32(ctx), _i32(ql), kc, vc,
                    max_q_len=int(ql.max()))
        ref_tab = np.zeros((S, MB), dtype=np.int32)
        for s, t in enumerate(ref_pool.tables):
            ref_tab[s, :len(t)] = t
        ref_write_kv(ref_k, ref_v, kn, vn, ref_tab, ctx, ql)
        return ctx, ql, ref_tab

    def step(label, live):
        ctx, ql, ref_tab = append({s: 1 for s in live})
        q = fresh((len(live), HQ, D))
        out = torch.full((len(live), HQ, D), OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        lse = torch.full((len(live), HQ), LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
        pk.attend(_dev_bf16(q), kc, vc, _i32(lib_pool.table()), _i32(ctx), _i32(ql), scale, out, lse,
                  max_q_len=1, max_ctx_len=MB * p, partition_size=32)
        torch.cuda.synchronize()
        ref = oracle.attend_fp64(q, ref_k, ref_v, ref_tab, ctx, ql, scale, HKV, p)
        compare(None, (_host_bits(out), lse.cpu().numpy()), ref, label=label)

    say("decode loop: prompts")
    append({0: 40, 2: 17})
    lib_pool.fork(0, 1)
    ref_pool.fork(0, 1)
    for i in range(4):
        step(f"step {i}", [0, 1, 2])
    # slot 2 finishes; its blocks come back once the work that read them is done
    lib_pool.release(2, 4)
    ref_pool.release(2, 4)
    torch.cuda.synchronize()
    lib_pool.retire(4)
    ref_pool.retire(4)
    append({2: 50, 3: 9})
    for i in range(4, 8):
        step(f"step {i}", [0, 1, 2, 3])
    assert lib_pool.stats().used_blocks == ref_pool.physical_in_use()
