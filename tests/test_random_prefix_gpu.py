"""Seeded random prefix-grouped batches against the FP64 oracle.

pa_attend_prefix computes pa_attend's result, so the oracle is the same one.
Each case draws what the hand-written cases do not pin down together: 1 to 5
groups of 1 to 20 members with prefixes of 1 to 40 pages, members with no
keys of their own (context = prefix) and members without a new token,
slots in no group, 1, 2, 4 or 8 query heads per KV head, a max_members below
the largest group (its other members read their prefix as ordinary keys),
the min_prefix_len hint, and several partition sizes -- so one launch (prefix
items beside the slots' partitions, the slots' own group lookup or the set-up
workgroup) and two launches (prefix pass, then the decode pass) both run.
The draws are fixed by the case index.
"""

from __future__ import annotations

import numpy as np
import pytest

from paged_kv_cache_attend_amd import inputs

from gpu_util import compare, run_oracle, say
from test_prefix_gpu import run_prefix

pytestmark = pytest.mark.gpu

HEADS = [(32, 8), (8, 8), (16, 8), (64, 8), (8, 2), (4, 1), (16, 4)]
PARTITIONS = [0, 0, 32, 64, 128]


def draw(i: int):
    rng = np.random.default_rng(73000 + i)
    hq, hkv = HEADS[int(rng.integers(len(HEADS)))]
    # a quarter of the cases give every group the same prefix length, so that
    # with the hint below the first page-id requests assume it
    same = 16 * int(rng.integers(1, 41)) if rng.random() < 0.25 else 0
    groups = []
    for _ in range(int(rng.integers(1, 6))):
        prefix = same or 16 * int(rng.integers(1, 41))
        members = []
        for _ in range(int(rng.integers(1, 21))):
            u = rng.random()
            members.append(prefix if u < 0.15 else prefix + int(rng.integers(1, 300)))
        groups.append((prefix, members))
    n_singles = 0 if rng.random() < 0.4 else int(rng.integers(1, 4))
    singles = [int(rng.integers(0, 500)) for _ in range(n_singles)]
    ctx = [n for _, m in groups for n in m] + singles
    q_lens = [1 if n > 0 and rng.random() > 0.1 else 0 for n in ctx]
    largest = max(len(m) for _, m in groups)
    # min_prefix_len may exceed 0 only when every slot with a new token reads
    # a prefix: the singles then get none, and every member shares its prefix
    hinted = rng.random() < 0.4
    n_members = len(ctx) - len(singles)
    if hinted:
        q_lens[n_members:] = [0] * len(singles)
        max_members = largest
        hint = 16 * int(rng.integers(1, min(pl for pl, _ in groups) // 16 + 1))
        if rng.random() < 0.6:
            hint = min(pl for pl, _ in groups)
    else:
        max_members = largest if rng.random() < 0.7 else int(rng.integers(1, largest + 1))
        hint = 0
    if not any(q_lens):
        q_lens[0] = 1
    ps = PARTITIONS[int(rng.integers(len(PARTITIONS)))]
    return dict(hq=hq, hkv=hkv, groups=groups, singles=singles, q_lens=q_lens, max_members=max_members,
                hint=hint, ps=ps)


@pytest.mark.parametrize("i", range(24))
def test_random_prefix_batch_matches_oracle(i):
    c = draw(i)
    p, gs, pl = inputs.make_grouped_problem(f"random_prefix_{i}", inputs.SEED_BASE + 1700 + i, c["groups"],
                                            c["singles"], c["hq"], c["hkv"], q_lens=c["q_lens"])
    say(f"random prefix case {i}: heads {c['hq']}/{c['hkv']} groups "
        f"{[(pfx, len(m)) for pfx, m in c['groups']]} singles {len(c['singles'])} "
        f"max_members {c['max_members']} min_prefix_len {c['hint']} partition_size {c['ps']}")
    got = run_prefix(p, gs, pl, partition_size=c["ps"], min_prefix_len=c["hint"], max_members=c["max_members"])
    compare(p, got, run_oracle(p), label=f"random prefix {i}")
