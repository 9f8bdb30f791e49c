"""Seeded random batches against the FP64 oracle.

Each case draws a batch the hand-written cases do not pin down: 1 to 6 slots
with ragged context lengths, zombies (no keys, a query row kept) and empty
slots, 0 to 130 new tokens per slot (so one call can mix one-token decode,
several-token decode and the chunk path's row tiles), query / KV head ratios
1 to 8 (including 3, which only the chunk path serves), with and without the
causal flag, and several partition sizes.  Every written row is compared with
the oracle within the stated tolerances, every other row must keep its
sentinel bits.  The draws are fixed by the case index.
"""

from __future__ import annotations

import numpy as np
import pytest

from paged_kv_cache_attend_amd import inputs

from gpu_util import compare, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu

HEADS = [(8, 8), (8, 2), (16, 2), (32, 8), (4, 1), (64, 8), (12, 4), (6, 2)]
NEW_TOKENS = [0, 1, 1, 1, 2, 3, 5, 8, 9, 17, 64, 130]
PARTITIONS = [0, 16, 64, 256]


def draw(i: int):
    rng = np.random.default_rng(91000 + i)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    ns = int(rng.integers(1, 7))
    q_lens = [int(rng.choice(NEW_TOKENS)) for _ in range(ns)]
    if hq > 16:  # keep the oracle's work small
        q_lens = [min(m, 17) for m in q_lens]
    ctx = []
    for m in q_lens:
        u = rng.random()
        if u < 0.1:
            ctx.append(0)  # zombie (its query row stays) or empty slot
        else:
            ctx.append(int(rng.integers(max(m, 1), max(m, 1) + 700)))
    if all(n == 0 or m == 0 for n, m in zip(ctx, q_lens)):
        q_lens[0], ctx[0] = max(q_lens[0], 1), max(ctx[0], q_lens[0], 1)
    causal = bool(rng.integers(2))
    ps = PARTITIONS[int(rng.integers(len(PARTITIONS)))]
    return dict(hq=hq, hkv=hkv, ctx=ctx, q_lens=q_lens, causal=causal, ps=ps)


@pytest.mark.parametrize("i", range(48))
def test_random_batch_matches_oracle(i):
    c = draw(i)
    p = inputs.make_problem(f"random_{i}", inputs.SEED_BASE + 900 + i, c["ctx"], c["q_lens"], c["hq"], c["hkv"],
                            partition_size=c["ps"], causal=c["causal"])
    say(f"random case {i}: heads {c['hq']}/{c['hkv']} ctx {c['ctx']} new {c['q_lens']} "
        f"causal={c['causal']} partition_size={c['ps']}")
    got = run_gpu(p)
    ref = run_oracle(p)
    compare(p, got, ref, label=f"random {i}")
