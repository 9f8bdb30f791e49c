"""GPU parity of prefix-grouped (cascade) decode, pa_attend_prefix.

The call computes exactly pa_attend's definition, so the FP64 oracle is the
same one; the prefix pass only changes the order of the arithmetic (the
shared keys' partials are merged by log-sum-exp with the suffix's), so the
result must match the oracle within the same tolerances and pa_attend within
twice them.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_attend_amd as pk
from paged_kv_cache_attend_amd import inputs

from gpu_util import DEV, LSE_SENTINEL, OUT_SENTINEL, compare, out_bound, run_gpu, run_oracle, say

pytestmark = pytest.mark.gpu


def _i32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(DEV)


def run_prefix(p, group_start, prefix_len, *, partition_size=0, min_prefix_len=0, layer=0, repeats=1,
               max_members=None, max_prefix_len=None):
    q, k, v = p.layer(layer)
    t = inputs.to_device(p, q, k, v, DEV)
    out = torch.full(q.shape, OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.full(q.shape[:2], LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
    members = int(np.diff(group_start).max(initial=0)) if max_members is None else max_members
    mpl = int(prefix_len.max(initial=0)) if max_prefix_len is None else max_prefix_len
    for _ in range(repeats):
        pk.attend_prefix(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"], float(p.scale),
                         out, lse, group_start=_i32(group_start), prefix_len=_i32(prefix_len),
                         max_members=members, max_prefix_len=mpl,
                         min_prefix_len=min_prefix_len, max_ctx_len=p.max_ctx_len, partition_size=partition_size)
    torch.cuda.synchronize()
    return out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()


CASES = [
    ("one_group", dict(groups=[(96, [96 + 13 * i for i in range(10)])], singles=[], hq=32, hkv=8)),
    ("mixed", dict(groups=[(64, [100, 0, 64, 300]), (32, [32, 77])], singles=[50, 0, 1000], hq=32, hkv=8,
                   q_lens=[1, 1, 0, 1, 1, 1, 1, 0, 1])),
    ("two_row_tiles", dict(groups=[(48, [48 + 7 * i for i in range(20)])], singles=[], hq=32, hkv=8)),
    ("mha", dict(groups=[(80, [80, 90, 200])], singles=[33], hq=4, hkv=4)),
    ("gqa2", dict(groups=[(16, [17, 100]), (160, [160, 170, 400])], singles=[], hq=8, hkv=4)),
    # eight query heads per KV head: 8 members x 8 heads = 64 rows, one full row tile
    ("gqa8", dict(groups=[(64, [64, 100, 300, 65, 80, 64, 200, 129])], singles=[40], hq=64, hkv=8)),
    ("long_prefix", dict(groups=[(2048, [2048, 2100, 2600])], singles=[700], hq=32, hkv=8)),
    # 60 prefix pages over 20 partitions of 3 pages: a partition's second
    # tile reaches into the next partition's first page (masked).
    ("odd_partition_pages", dict(groups=[(960, [960 + 5 * i for i in range(6)])], singles=[200], hq=32, hkv=8)),
    # 512 prefix pages need 32 partitions of 16 (eight tiles each): the
    # suffix merge folds its own partials and the prefix's in two batches.
    ("very_long_prefix", dict(groups=[(8192, [8192, 8200, 8500])], singles=[], hq=32, hkv=8)),
    # 63 groups: the slots find their group themselves; 70: the set-up
    # workgroup writes the slots' prefix lengths first.
    ("63_groups", dict(groups=[(16, [20, 50 + i]) for i in range(63)], singles=[30], hq=32, hkv=8)),
    ("70_groups", dict(groups=[(32, [40 + i, 90, 33]) for i in range(70)], singles=[20], hq=32, hkv=8)),
    # 40 members at four query heads per KV head: three prefix items of 16,
    # 16 and 8 members per (partition, KV head).
    ("40_members", dict(groups=[(160, [161 + 3 * i for i in range(40)])], singles=[], hq=32, hkv=8)),
]


@pytest.mark.parametrize("name,case", CASES, ids=[c[0] for c in CASES])
def test_prefix_matches_oracle(name, case):
    p, gs, pl = inputs.make_grouped_problem(f"pre_{name}", 300 + len(name), case["groups"], case["singles"],
                                            case["hq"], case["hkv"], q_lens=case.get("q_lens"))
    ref = run_oracle(p)
    for ps in (0, 32):
        say(f"attend_prefix {name} partition_size={ps}")
        got = run_prefix(p, gs, pl, partition_size=ps)
        compare(p, got, ref, label=f"{name} ps={ps}")


def test_prefix_min_prefix_hint_and_repeats():
    # The suffix split sized by min_prefix_len, and repeated calls on one
    # workspace (the counters come back to zero) give the same bits.
    p, gs, pl = inputs.make_grouped_problem("pre_hint", 41, [(128, [130, 300, 1000, 128])], [], 32, 8)
    a = run_prefix(p, gs, pl, min_prefix_len=128)
    b = run_prefix(p, gs, pl, min_prefix_len=128, repeats=3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    compare(p, a, run_oracle(p), label="hint")


def test_prefix_guessed_prefix_length_mismatch():
    # With min_prefix_len == max_prefix_len the partitions request their
    # first page ids for that prefix length before knowing their own; slots
    # outside the group and a member past max_members have none and reload.
    p, gs, pl = inputs.make_grouped_problem("pre_guess", 59, [(64, [70, 300, 65, 100])], [40, 90], 32, 8)
    ref = run_oracle(p)
    for ps in (0, 32):
        say(f"attend_prefix guessed prefix length, partition_size={ps}")
        got = run_prefix(p, gs, pl, partition_size=ps, min_prefix_len=64, max_members=3)
        compare(p, got, ref, label=f"guess ps={ps}")


def test_prefix_members_past_max_members_are_decoded_whole():
    # Slots past a group's first max_members get no prefix: the decode pass
    # attends them to all their keys, and the result is still exact.
    p, gs, pl = inputs.make_grouped_problem("pre_maxm", 47, [(64, [70, 300, 65, 100, 64])], [40], 32, 8)
    ref = run_oracle(p)
    for mm in (1, 3):
        say(f"attend_prefix max_members={mm}")
        compare(p, run_prefix(p, gs, pl, max_members=mm), ref, label=f"max_members={mm}")


def test_prefix_length_rounded_down_to_pages():
    # A prefix length that is not a whole number of pages is read as the
    # pages it covers whole by both passes (the rest are ordinary keys).
    p, gs, pl = inputs.make_grouped_problem("pre_round", 53, [(64, [70, 300, 65])], [], 32, 8)
    ref = run_oracle(p)
    say("attend_prefix prefix_len not a multiple of 16")
    compare(p, run_prefix(p, gs, pl + 6, max_prefix_len=80, partition_size=32), ref, label="rounded")


def test_prefix_graph_replay():
    p, gs, pl = inputs.make_grouped_problem("pre_graph", 43, [(64, [70, 300, 65])], [90], 32, 8)
    q, k, v = p.layer(0)
    t = inputs.to_device(p, q, k, v, DEV)
    out = torch.empty(q.shape, dtype=torch.bfloat16, device=DEV)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=DEV)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call = pk.attend_prefix(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                                float(p.scale), out, lse, group_start=_i32(gs), prefix_len=_i32(pl),
                                max_members=3, max_prefix_len=64, max_ctx_len=p.max_ctx_len, prepared=True)
        call.launch(s)
        torch.cuda.synchronize()
        eager = (out.clone(), lse.clone())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call.launch(s)
        for i in range(4):
            out.zero_()
            lse.zero_()
            g.replay()
            torch.cuda.synchronize()
            assert torch.equal(out.view(torch.int16), eager[0].view(torch.int16)), i
            assert torch.equal(lse.view(torch.int32), eager[1].view(torch.int32)), i


def test_prefix_full_size_shared_prefix_decode():
    # 10 slots x 8447 keys sharing 6144 (384 pages), 32/8 heads: the oracle
    # checks three slots; every row also agrees with pa_attend.
    p = inputs.qwen3_shared_prefix_decode(num_layers=1)
    gs = np.array([0, p.num_seqs], dtype=np.int32)
    pl = np.array([p.shared_prefix_blocks * 16], dtype=np.int32)
    say("attend_prefix full size")
    ob, lb = run_prefix(p, gs, pl, min_prefix_len=int(pl[0]))
    seqs = [0, 4, 9]
    out, lse, _ = run_oracle(p, seqs=seqs)
    rows = np.zeros(p.total_q, dtype=bool)
    rows[seqs] = True
    o = inputs_bf16(ob[rows])
    err = np.abs(o - out[rows])
    assert (err <= out_bound(out[rows])).all() and err.mean() <= 1e-3, (err.max(), err.mean())
    assert np.abs(lb[rows] - lse[rows]).max() <= 1e-3
    base = run_gpu(p)
    d = np.abs(inputs_bf16(ob) - inputs_bf16(base[0]))
    # two results each within out_bound of the exact one
    assert (d <= 2 * out_bound(inputs_bf16(base[0]))).all() and d.mean() <= 2e-3, (d.max(), d.mean())
    assert np.abs(lb - base[1]).max() <= 2e-3


def inputs_bf16(bits):
    import oracle
    return oracle.bf16_bits_to_f64(bits)
