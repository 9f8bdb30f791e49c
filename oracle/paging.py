"""Plain model of the paged KV allocator and of appending new K/V rows.

TEST INFRASTRUCTURE ONLY -- imported by tests, never by the product path.
Shares no code with the HIP library.

What is modelled, and where it is stated
----------------------------------------
The inference-optimisation chapter ("Chapter 8: Inference optimisation"):

* section 8.3.1, Fig. 8-10: a sequence is cut into fixed-size logical
  blocks; each request's block table maps logical block i to a physical
  block; when a sequence grows into a new block the engine takes a physical
  block from the free pool and records the mapping.  A request of L tokens
  holds ceil(L / p) blocks; only the last one can have unused slots.
* section 8.3.2, Fig. 8-14: every table entry pointing at a block is one
  reference; a block shared by several tables keeps a reference count, and it
  returns to the free pool only after its last reference is dropped *and*
  the accelerator has finished the work that reads it.
* section 8.3.2, Fig. 8-15: before writing into a shared block that is only
  partly filled, a branch takes a private copy of it (copy-on-write); the
  blocks that were already full stay shared.

Readings (where the pages leave the mechanics open):

* "the accelerator has finished" is a caller-supplied fence number: a block
  released under fence f is reusable once the caller retires a fence >= f;
* a fork shares the first ``num_tokens`` tokens of the source (all of it by
  default); the shared tail block, if partly filled, is copied by whichever
  holder writes into it next while it is still shared;
* which free block is handed out is not fixed by the pages; this model takes
  the lowest-numbered one, and tests compare allocators only on what does
  not depend on that choice.

``write_kv`` states where new rows go: the m new tokens of a request with n
visible tokens are positions n - m .. n - 1, and position j lives in block
``table[j // p]`` at slot ``j % p``.
"""

from __future__ import annotations

import numpy as np


class BlockPool:
    """Reference model: block tables, reference counts, free and pending blocks."""

    def __init__(self, num_blocks: int, block_size: int, num_slots: int, max_blocks_per_seq: int):
        self.num_blocks = num_blocks
        self.block_size = block_size
        self.max_blocks = max_blocks_per_seq
        self.free = set(range(num_blocks))
        self.refs = [0] * num_blocks
        self.pending: list[tuple[int, int]] = []  # (fence, block)
        self.tables: list[list[int]] = [[] for _ in range(num_slots)]
        self.lengths = [0] * num_slots

    # -- section 8.3.1: grow a sequence block by block --------------------
    def _take(self) -> int:
        b = min(self.free)
        self.free.remove(b)
        self.refs[b] = 1
        return b

    def append(self, slot: int, num_tokens: int):
        """Make room for num_tokens more tokens.  Returns the list of
        (source, destination) block copies the caller must make first, or
        None (and changes nothing) when the free pool is too small."""
        p = self.block_size
        length, table = self.lengths[slot], self.tables[slot]
        new_len = length + num_tokens
        if -(-new_len // p) > self.max_blocks:
            raise ValueError("sequence longer than its block table")
        grow = -(-new_len // p) - len(table)
        # Section 8.3.2: writing into a shared, partly filled tail needs a copy.
        cow = num_tokens > 0 and length % p != 0 and self.refs[table[-1]] > 1
        if grow + (1 if cow else 0) > len(self.free):
            return None
        copies = []
        if cow:
            old = table[-1]
            new = self._take()
            self.refs[old] -= 1
            table[-1] = new
            copies.append((old, new))
        for _ in range(grow):
            table.append(self._take())
        self.lengths[slot] = new_len
        return copies

    # -- section 8.3.2: share a prefix ------------------------------------
    def fork(self, src: int, dst: int, num_tokens: int | None = None):
        if self.lengths[dst] or self.tables[dst]:
            raise ValueError("fork into a slot that holds tokens")
        n = self.lengths[src] if num_tokens is None else num_tokens
        if not 0 <= n <= self.lengths[src]:
            raise ValueError("fork beyond the source's length")
        shared = self.tables[src][: -(-n // self.block_size)]
        for b in shared:
            self.refs[b] += 1
        self.tables[dst] = list(shared)
        self.lengths[dst] = n

    # -- section 8.3.2, Fig. 8-14: release, then reuse after the fence ----
    def release(self, slot: int, fence: int):
        for b in self.tables[slot]:
            self.refs[b] -= 1
            if self.refs[b] == 0:
                self.pending.append((fence, b))
        self.tables[slot] = []
        self.lengths[slot] = 0

    def retire(self, fence: int):
        done = [b for f, b in self.pending if f <= fence]
        self.pending = [(f, b) for f, b in self.pending if f > fence]
        self.free.update(done)

    # -- what the pages count ----------------------------------------------
    def physical_in_use(self) -> int:
        return sum(1 for r in self.refs if r > 0)

    def references(self) -> int:
        return sum(len(t) for t in self.tables)

    def capacity_tokens(self) -> int:
        """Token slots held by the blocks in use (section 8.3.1 example)."""
        return self.physical_in_use() * self.block_size


def write_kv(k_cache: np.ndarray, v_cache: np.ndarray, k_new: np.ndarray, v_new: np.ndarray,
             block_table: np.ndarray, ctx_lens: np.ndarray, q_lens: np.ndarray) -> None:
    """Scatter new rows into their pages, in place.

    k_cache, v_cache: [num_blocks][Hkv][p][D] (any dtype); k_new, v_new:
    [total_q][Hkv][D], rows packed by slot in slot order.  Slots with no new
    tokens or no tokens at all write nothing.
    """
    p = k_cache.shape[2]
    row = 0
    for r in range(len(ctx_lens)):
        n, m = int(ctx_lens[r]), int(q_lens[r])
        if m <= 0:
            continue
        if n > 0:
            for i in range(m):
                j = n - m + i
                b = int(block_table[r][j // p])
                k_cache[b, :, j % p, :] = k_new[row + i]
                v_cache[b, :, j % p, :] = v_new[row + i]
        row += m


def copy_blocks(k_cache: np.ndarray, v_cache: np.ndarray, pairs) -> None:
    """Copy whole blocks (every KV head) src -> dst, in place."""
    for s, d in pairs:
        k_cache[d] = k_cache[s]
        v_cache[d] = v_cache[s]
