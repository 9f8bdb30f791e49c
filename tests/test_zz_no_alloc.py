"""pa_attend_noalloc (the library's built-in scratch buffer instead of a
caller workspace) against pa_attend on the same inputs: bit-identical
outputs and LSE, both within the oracle tolerances, on two calls in a row
whose second input is smaller; the chunk path (no scratch) likewise; a
shape that needs more scratch than the buffer holds is refused on the host."""

from __future__ import annotations

import numpy as np
import pytest
import torch

import paged_kv_cache_attend_amd as pk
from paged_kv_cache_attend_amd import inputs

from gpu_util import DEV, LSE_SENTINEL, OUT_SENTINEL, compare, run_oracle, say

pytestmark = pytest.mark.gpu


def _bufs(q):
    out = torch.full(q.shape, OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.full(q.shape[:2], LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
    return out, lse


def _both(p, ps=0):
    t = inputs.to_device(p, *p.layer(0), DEV)
    args = (t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"], float(p.scale))
    kw = dict(max_q_len=p.max_q_len, max_ctx_len=p.max_ctx_len, partition_size=ps, causal=p.causal)
    o1, l1 = _bufs(t["q"])
    o2, l2 = _bufs(t["q"])
    torch.cuda.synchronize()
    pk.attend(*args, o1, l1, **kw)
    pk.attend_noalloc(*args, o2, l2, **kw)
    torch.cuda.synchronize()
    a = (o1.view(torch.int16).cpu().numpy().view(np.uint16), l1.cpu().numpy())
    b = (o2.view(torch.int16).cpu().numpy().view(np.uint16), l2.cpu().numpy())
    return a, b


def test_noalloc_matches_attend_on_two_calls_second_smaller():
    big = inputs.make_problem("noalloc_big", 71, [2303] * 12 + [0, 700, 1, 4000], [1] * 16, 32, 8)
    small = inputs.make_problem("noalloc_small", 72, [37, 100, 520], [1, 1, 1], 8, 2)
    for p, ps in ((big, 0), (small, 32)):
        shape = pk.make_shape(p.num_seqs, p.total_q, p.num_q_heads, p.num_kv_heads, p.max_blocks_per_seq,
                              p.max_q_len, p.max_ctx_len, p.num_blocks, ps)
        assert pk.plan(shape)[1] > 1, "the case must use the split (scratch) path"
        say(f"noalloc {p.name}: {pk.plan(shape)[1]} partitions, {pk.workspace_size(shape)} scratch bytes")
        a, b = _both(p, ps)
        assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
        compare(p, b, run_oracle(p), label=f"noalloc {p.name}")


def test_noalloc_chunk_path_needs_no_scratch():
    p = inputs.make_problem("noalloc_chunk", 73, [300, 64], [40, 64], 8, 2)
    a, b = _both(p)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    compare(p, b, run_oracle(p), label="noalloc chunk")


def test_noalloc_refuses_shapes_beyond_its_buffer():
    # 4096 slots x 8 KV heads x 17 partitions of partials need ~290 MB: refused
    # on the host before anything is launched (the pointers are never used).
    lib = pk.load()
    import ctypes
    shape = pk.make_shape(4096, 4096, 32, 8, 528, 1, 8447, 1 << 20, 512)
    assert pk.workspace_size(shape) > pk.NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(0x1000)
    st = lib.pa_attend_noalloc(ctypes.byref(shape), fake, fake, fake, fake, fake, fake, ctypes.c_float(0.088),
                               fake, None, None)
    assert st == pk.Status.ERR_SCRATCH_LIMIT
