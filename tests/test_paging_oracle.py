"""Pins of the paging oracle (allocator model and K/V append) to the pages.

Each test reproduces a figure the inference-optimisation chapter prints for
paged allocation, prefix sharing, copy-on-write or release, or checks the
model against a brute-force statement of what a block table means.
"""

from __future__ import annotations

import numpy as np
import pytest

from oracle import closed_forms
from oracle.paging import BlockPool, copy_blocks, write_kv


def test_worked_example_paged_capacity():
    # Section 8.3.1, Figs. 8-11/8-12: lengths 9, 13, 5, 15 with 4-token
    # blocks get 12, 16, 8 and 16 token slots, 52 in all (64 if each had
    # reserved its 16-token maximum); 42 tokens are stored, 10 slots unused.
    pool = BlockPool(num_blocks=64, block_size=4, num_slots=4, max_blocks_per_seq=4)
    for slot, n in enumerate([9, 13, 5, 15]):
        assert pool.append(slot, n) == []
    assert [len(t) * 4 for t in pool.tables] == [12, 16, 8, 16]
    assert pool.capacity_tokens() == 52
    assert pool.capacity_tokens() - sum(pool.lengths) == 10
    assert 4 * 16 == 64


def test_worked_example_shared_prefix_capacity():
    # Section 8.3.1, Fig. 8-13: when A and B share their first 8 tokens (two
    # full blocks), the four requests hold 44 token slots.
    pool = BlockPool(num_blocks=64, block_size=4, num_slots=4, max_blocks_per_seq=4)
    pool.append(0, 8)
    pool.fork(0, 1)
    assert pool.append(0, 1) == [] and pool.append(1, 5) == []
    pool.append(2, 5)
    pool.append(3, 15)
    assert pool.lengths == [9, 13, 5, 15]
    assert pool.tables[0][:2] == pool.tables[1][:2]
    assert pool.capacity_tokens() == 44


def test_four_branch_sharing_counts():
    # Section 8.3.2: four branches over a 95-block common prefix with 9 private
    # blocks each: 4 x (95 + 9) = 416 references, 95 + 4 x 9 = 131 blocks.
    p = 16
    pool = BlockPool(num_blocks=600, block_size=p, num_slots=4, max_blocks_per_seq=104)
    pool.append(0, 95 * p)
    for b in (1, 2, 3):
        pool.fork(0, b)
    for b in range(4):
        assert pool.append(b, 9 * p) == []
    assert pool.references() == 416 == closed_forms.block_references(95, 9, 4)
    assert pool.physical_in_use() == 131 == closed_forms.shared_physical_blocks(95, 9, 4)


@pytest.mark.parametrize("b", [1, 10, 16, 35])
def test_shared_prefix_capacity_864_plus_324b(b):
    # Section 8.3.2: b long requests sharing 6144 prompt tokens, each with a
    # private 8192 - 6144 + 255 = 2303 tokens in 16-token blocks, hold
    # 864 + 324 b MiB of KV (Qwen3-8B: 147,456 B per token).
    pool = BlockPool(num_blocks=384 + 144 * b, block_size=16, num_slots=b, max_blocks_per_seq=528)
    pool.append(0, 6144)
    for r in range(1, b):
        pool.fork(0, r)
    for r in range(b):
        assert pool.append(r, 2303) == []
    mib = pool.physical_in_use() * 16 * closed_forms.kv_bytes_per_token(36, 8, 128, 2) / 2**20
    assert mib == 864 + 324 * b


def test_copy_on_write_of_a_shared_tail():
    # Section 8.3.2, Fig. 8-15: a 4-token block holds the common a, b, c; two
    # branches append x and y.  They end with different tail blocks holding
    # a b c x and a b c y, while the earlier full block stays shared.
    pool = BlockPool(num_blocks=8, block_size=4, num_slots=2, max_blocks_per_seq=4)
    cache = np.zeros((8, 4), dtype="<U1")
    pool.append(0, 7)
    for j, ch in enumerate("pqrsabc"):
        cache[pool.tables[0][j // 4], j % 4] = ch
    pool.fork(0, 1)
    for slot, ch in ((0, "x"), (1, "y")):
        for s, d in pool.append(slot, 1):
            cache[d] = cache[s]
        j = pool.lengths[slot] - 1
        cache[pool.tables[slot][j // 4], j % 4] = ch
    seq = ["".join(cache[t[j // 4], j % 4] for j in range(8)) for t in pool.tables]
    assert seq == ["pqrsabcx", "pqrsabcy"]
    assert pool.tables[0][0] == pool.tables[1][0]
    assert pool.tables[0][1] != pool.tables[1][1]
    assert pool.physical_in_use() == 3


def test_release_waits_for_last_reference_and_the_fence():
    # Section 8.3.2, Fig. 8-14: A ends, the shared blocks stay for B; only
    # when B's reference goes too, and the accelerator is done, are they free.
    pool = BlockPool(num_blocks=4, block_size=4, num_slots=2, max_blocks_per_seq=4)
    pool.append(0, 8)
    pool.fork(0, 1)
    shared = list(pool.tables[0])
    pool.release(0, fence=5)
    assert [pool.refs[b] for b in shared] == [1, 1] and len(pool.free) == 2
    pool.release(1, fence=7)
    assert pool.physical_in_use() == 0 and len(pool.free) == 2 and len(pool.pending) == 2
    pool.retire(6)
    assert len(pool.free) == 2
    pool.retire(7)
    assert len(pool.free) == 4 and not pool.pending


def test_out_of_blocks_changes_nothing():
    pool = BlockPool(num_blocks=3, block_size=4, num_slots=2, max_blocks_per_seq=8)
    pool.append(0, 6)
    before = ([list(t) for t in pool.tables], list(pool.lengths), set(pool.free))
    assert pool.append(1, 9) is None
    assert ([list(t) for t in pool.tables], list(pool.lengths), set(pool.free)) == before


def _history_check(pool, cache, history):
    for slot, toks in enumerate(history):
        t = pool.tables[slot]
        got = [int(cache[t[j // pool.block_size], j % pool.block_size]) for j in range(pool.lengths[slot])]
        assert got == toks, slot


def test_random_operations_keep_every_history_intact():
    # Brute force: token ids written through the tables (copying first where
    # the model asks) must read back, for every slot, as exactly that slot's
    # own history -- a write into a block another slot still uses would
    # show up here -- and the reference counts must equal the table entries.
    rng = np.random.default_rng(5)
    p, S = 4, 6
    pool = BlockPool(num_blocks=40, block_size=p, num_slots=S, max_blocks_per_seq=12)
    cache = np.full((40, p), -1, dtype=np.int64)
    history = [[] for _ in range(S)]
    next_tok, fence = 0, 0
    for _ in range(400):
        op = rng.integers(0, 4)
        slot = int(rng.integers(0, S))
        if op <= 1:
            t = int(rng.integers(0, 7))
            if pool.lengths[slot] + t > 12 * p:
                continue
            copies = pool.append(slot, t)
            if copies is None:
                continue
            for s, d in copies:
                cache[d] = cache[s]
            for _k in range(t):
                j = len(history[slot])
                cache[pool.tables[slot][j // p], j % p] = next_tok
                history[slot].append(next_tok)
                next_tok += 1
        elif op == 2:
            dst = int(rng.integers(0, S))
            if dst == slot or pool.lengths[dst] or pool.tables[dst]:
                continue
            n = int(rng.integers(0, pool.lengths[slot] + 1))
            pool.fork(slot, dst, n)
            history[dst] = history[slot][:n]
        else:
            fence += 1
            pool.release(slot, fence)
            history[slot] = []
            pool.retire(fence - int(rng.integers(0, 3)))
        _history_check(pool, cache, history)
        counts = np.zeros(40, dtype=int)
        for t in pool.tables:
            for b in t:
                counts[b] += 1
        assert list(counts) == pool.refs
        assert all(pool.refs[b] == 0 for b in pool.free)


def test_write_kv_matches_flat_addressing():
    # The scatter against an independent statement of the layout: position j
    # of a slot is flat row table[j // p] * p + j % p of the cache viewed as
    # [num_blocks * p] rows per KV head.
    rng = np.random.default_rng(9)
    nb, hkv, p, d = 12, 2, 4, 3
    k = rng.integers(0, 1000, (nb, hkv, p, d))
    v = rng.integers(0, 1000, (nb, hkv, p, d))
    table = np.array([[5, 2, 9], [0, 11, 3], [7, 7, 7]])
    ctx = np.array([10, 5, 0])
    ql = np.array([3, 5, 2])   # the third slot has no keys: writes nothing
    k_new = rng.integers(0, 1000, (10, hkv, d))
    v_new = rng.integers(0, 1000, (10, hkv, d))
    k2, v2 = k.copy(), v.copy()
    write_kv(k2, v2, k_new, v_new, table, ctx, ql)
    kf = k.transpose(1, 0, 2, 3).reshape(hkv, nb * p, d).copy()
    vf = v.transpose(1, 0, 2, 3).reshape(hkv, nb * p, d).copy()
    rows = [(0, j) for j in range(7, 10)] + [(1, j) for j in range(0, 5)]
    for row, (r, j) in enumerate(rows):
        flat = table[r][j // p] * p + j % p
        kf[:, flat] = k_new[row]
        vf[:, flat] = v_new[row]
    assert np.array_equal(k2.transpose(1, 0, 2, 3).reshape(hkv, nb * p, d), kf)
    assert np.array_equal(v2.transpose(1, 0, 2, 3).reshape(hkv, nb * p, d), vf)


def test_copy_blocks_copies_every_head():
    k = np.arange(4 * 2 * 4 * 3).reshape(4, 2, 4, 3)
    v = -k
    k2, v2 = k.copy(), v.copy()
    copy_blocks(k2, v2, [(1, 3)])
    assert np.array_equal(k2[3], k[1]) and np.array_equal(v2[3], v[1])
    assert np.array_equal(k2[:3], k[:3]) and np.array_equal(v2[:3], v[:3])
