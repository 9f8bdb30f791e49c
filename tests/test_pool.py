"""The C-ABI block pool (host side, no GPU) against the paging oracle.

Which physical block a request receives is the allocator's choice, so the two
are compared on what does not depend on it: the sharing structure of the
tables (block ids relabelled in order of first appearance), lengths,
reference counts, and the free / pending / used / reference totals.  A
token-content simulation driven by the library's own tables and copy lists
checks that no slot ever sees another slot's writes.
"""

from __future__ import annotations

import numpy as np
import pytest

import paged_kv_cache_attend_amd as pk
from oracle import closed_forms
from oracle.paging import BlockPool


@pytest.fixture(scope="module", autouse=True)
def _lib():
    import os
    from paged_kv_cache_attend_amd import _lib as L
    if not os.path.exists(L.lib_path()):
        from paged_kv_cache_attend_amd import build
        build.build()
    pk.load()


def _canon(tables, lengths, p):
    ids = {}
    return [tuple(ids.setdefault(int(b), len(ids)) for b in t[: -(-n // p)]) for t, n in zip(tables, lengths)]


def _state(pool: pk.Pool):
    lengths = [pool.length(s) for s in range(pool.num_slots)]
    tab = pool.table()
    canon = _canon(tab, lengths, pool.block_size)
    refs = {}
    for row, n in zip(tab, lengths):
        for b in row[: -(-n // pool.block_size)]:
            refs[int(b)] = pool.refcount(int(b))
    st = pool.stats()
    return canon, lengths, sorted(refs.values()), (st.free_blocks, st.pending_blocks, st.used_blocks,
                                                    st.references)


def _oracle_state(o: BlockPool):
    canon = _canon(o.tables, o.lengths, o.block_size)
    refs = sorted(o.refs[b] for b in {b for t in o.tables for b in t})
    return canon, list(o.lengths), refs, (len(o.free), len(o.pending), o.physical_in_use(), o.references())


def test_pages_figures_on_the_library_pool():
    # Section 8.3.1 (9/13/5/15 -> 52, and 44 with a shared 8-token prefix)
    # and section 8.3.2 (four branches: 416 references, 131 blocks).
    pool = pk.Pool(64, 4, 4, 4)
    for slot, n in enumerate([9, 13, 5, 15]):
        assert pool.append(slot, n) == []
    assert pool.stats().used_blocks * 4 == 52
    pool = pk.Pool(64, 4, 4, 4)
    pool.append(0, 8)
    pool.fork(0, 1)
    pool.append(0, 1), pool.append(1, 5), pool.append(2, 5), pool.append(3, 15)
    assert pool.stats().used_blocks * 4 == 44
    pool = pk.Pool(600, 16, 4, 104)
    pool.append(0, 95 * 16)
    for b in (1, 2, 3):
        pool.fork(0, b)
    for b in range(4):
        pool.append(b, 9 * 16)
    st = pool.stats()
    assert st.references == 416 == closed_forms.block_references(95, 9, 4)
    assert st.used_blocks == 131 == closed_forms.shared_physical_blocks(95, 9, 4)


def test_copy_on_write_tail_on_the_library_pool():
    # Section 8.3.2, Fig. 8-15: the first branch to write the shared, partly
    # filled tail gets a copy; the other then owns the original alone.
    pool = pk.Pool(8, 4, 2, 4)
    pool.append(0, 7)
    pool.fork(0, 1)
    tail = int(pool.table()[0][1])
    assert pool.refcount(tail) == 2
    copies = pool.append(0, 1)
    assert len(copies) == 1 and copies[0][0] == tail
    assert int(pool.table()[0][1]) == copies[0][1] != tail
    assert pool.refcount(tail) == 1 and pool.refcount(copies[0][1]) == 1
    assert pool.append(1, 1) == []                     # now private: written in place
    assert int(pool.table()[1][1]) == tail
    assert pool.table()[0][0] == pool.table()[1][0]    # the full block stays shared
    assert pool.stats().used_blocks == 3


def test_fenced_release_on_the_library_pool():
    pool = pk.Pool(4, 4, 2, 4)
    pool.append(0, 8)
    pool.fork(0, 1)
    pool.release(0, 5)
    st = pool.stats()
    assert (st.free_blocks, st.pending_blocks, st.used_blocks) == (2, 0, 2)
    pool.release(1, 7)
    st = pool.stats()
    assert (st.free_blocks, st.pending_blocks, st.used_blocks) == (2, 2, 0)
    assert pool.append(0, 12) is None                  # released blocks not reusable yet
    pool.retire(6)
    assert pool.stats().free_blocks == 2
    pool.retire(7)
    assert pool.stats().free_blocks == 4
    assert pool.append(0, 16) == []


def test_errors_change_nothing():
    pool = pk.Pool(3, 4, 2, 3)
    pool.append(0, 6)
    before = _state(pool)
    assert pool.append(1, 9) is None                   # needs 3 blocks, 1 free
    with pytest.raises(pk.PaError):
        pool.append(0, 7)                              # beyond 3 blocks of 4
    with pytest.raises(pk.PaError):
        pool.append(2, 1)                              # no such slot
    with pytest.raises(pk.PaError):
        pool.append(0, -1)
    with pytest.raises(pk.PaError):
        pool.fork(0, 0)
    with pytest.raises(pk.PaError):
        pool.fork(1, 0)                                # destination holds tokens
    with pytest.raises(pk.PaError):
        pool.fork(0, 1, 7)                             # beyond the source
    with pytest.raises(pk.PaError):
        pool.release(5, 0)
    assert _state(pool) == before
    with pytest.raises(pk.PaError):
        pk.Pool(0, 4, 1, 1)
    with pytest.raises(pk.PaError):
        pk.Pool(4, 0, 1, 1)
    lib = pk.load()
    assert lib.pa_pool_length(None, 0) == -1 and lib.pa_pool_refcount(None, 0) == -1
    assert not lib.pa_pool_block_table(None)


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_operations_match_the_oracle(seed):
    rng = np.random.default_rng(seed)
    p, S, NB, MB = 4, 7, 48, 10
    pool, o = pk.Pool(NB, p, S, MB), BlockPool(NB, p, S, MB)
    cache = np.full((NB, p), -1, dtype=np.int64)
    history = [[] for _ in range(S)]
    next_tok, fence = 0, 0
    for step in range(500):
        op = int(rng.integers(0, 4))
        slot = int(rng.integers(0, S))
        if op <= 1:
            t = int(rng.integers(0, 8))
            if o.lengths[slot] + t > MB * p:
                continue
            a, b = pool.append(slot, t), o.append(slot, t)
            assert (a is None) == (b is None), step
            if a is None:
                continue
            assert len(a) == len(b), step
            for s, d in a:
                cache[d] = cache[s]
            tab = pool.table()
            for _k in range(t):
                j = len(history[slot])
                cache[tab[slot][j // p], j % p] = next_tok
                history[slot].append(next_tok)
                next_tok += 1
        elif op == 2:
            dst = int(rng.integers(0, S))
            if dst == slot or o.lengths[dst] or o.tables[dst]:
                continue
            n = int(rng.integers(0, o.lengths[slot] + 1))
            pool.fork(slot, dst, n)
            o.fork(slot, dst, n)
            history[dst] = history[slot][:n]
        else:
            fence += 1
            pool.release(slot, fence)
            o.release(slot, fence)
            history[slot] = []
            back = int(rng.integers(0, 3))
            pool.retire(fence - back)
            o.retire(fence - back)
        assert _state(pool) == _oracle_state(o), step
        tab = pool.table()
        for s in range(S):
            got = [int(cache[tab[s][j // p], j % p]) for j in range(pool.length(s))]
            assert got == history[s], (step, s)
