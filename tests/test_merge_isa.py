"""The fused split-KV merge of the decode kernel, pinned on its gfx950 assembly.

The partitions of one (slot, KV head) exchange their partial results through
the workspace with relaxed device-scope atomics: each workgroup stores its
partial, waits until those stores are acknowledged, passes a barrier, and
only then bumps the counter; the workgroup that sees the counter reach P - 1
loads every partial and merges.  Relaxed atomics alone give no happens-before
in the C++ model, so correctness rests on what the compiler emits for gfx950:

* the partial stores carry the device-scope cache policy (``sc1``): they are
  written through to the point where every XCD sees them;
* ``s_waitcnt vmcnt(0)`` follows them (on gfx9 the vector-memory counter also
  counts stores, so this waits for their acknowledgement) and an ``s_barrier``
  follows that, before the counter's ``global_atomic_add`` is issued;
* every load of the merge (after the atomic) carries ``sc1``: it reads from
  that same point, never from a non-coherent cache.

This test compiles ``decode.hip`` to assembly with the library's own flags and
checks those three facts in every instance of the kernel, so that a compiler
change that would break the merge fails here instead of corrupting outputs.
"""

from __future__ import annotations

import os
import re
import shutil
import subprocess

import pytest

from paged_kv_cache_attend_amd import build as B


@pytest.fixture(scope="module")
def decode_asm(tmp_path_factory):
    if not os.path.exists(B.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("isa") / "decode.s"
    # the same options as the shipped object (argument preloading included)
    cmd = [B.HIPCC, *[a for a in B.COMMON if a != "-fPIC"], *B.EXTRA.get("decode.hip", []),
           "--cuda-device-only", "-S", os.path.join(B.CSRC, "decode.hip"), "-o", str(out)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return out.read_text()


def _kernels(asm: str):
    names = re.findall(r"^(_ZN2pa\w*decode_kernel\w*):", asm, re.M)
    assert names, "no decode_kernel in the assembly"
    for name in names:
        i = asm.index(name + ":")
        j = asm.index(".Lfunc_end", i)
        yield name, [l.strip() for l in asm[i:j].split("\n")]


_BRANCH = re.compile(r"^s_(c?branch\w*)\s+(\.LBB\w+)")


def _blocks(body):
    """Basic blocks of a function body: (first line, last line) per block and
    the successor edges (fall-through and branch targets)."""
    starts = {0}
    for n, l in enumerate(body):
        if re.match(r"^\.LBB\w+:", l):
            starts.add(n)
        if _BRANCH.match(l) or l.startswith("s_endpgm"):
            starts.add(n + 1)
    starts = sorted(x for x in starts if x < len(body))
    ends = [b - 1 for b in starts[1:]] + [len(body) - 1]
    label_block = {}
    for i, b in enumerate(starts):
        m = re.match(r"^(\.LBB\w+):", body[b])
        if m:
            label_block[m.group(1)] = i
    succ = []
    for i, (b, e) in enumerate(zip(starts, ends)):
        out = []
        last = body[e]
        m = _BRANCH.match(last)
        if m:
            out.append(label_block[m.group(2)])
        if not (last.startswith("s_endpgm") or (m and m.group(1) == "branch")) and i + 1 < len(starts):
            out.append(i + 1)
        succ.append(out)
    return starts, ends, succ


def _dominated_loads(body, line):
    """Vector-memory loads after `line` in its block and in every block that
    block dominates: code that only runs after `line` has run."""
    starts, ends, succ = _blocks(body)
    nb = len(starts)
    preds = [[] for _ in range(nb)]
    for i, out in enumerate(succ):
        for j in out:
            preds[j].append(i)
    # iterative dominators over the blocks reachable from the entry
    reach, todo = {0}, [0]
    while todo:
        for j in succ[todo.pop()]:
            if j not in reach:
                reach.add(j)
                todo.append(j)
    dom = {i: set(reach) for i in reach}
    dom[0] = {0}
    changed = True
    while changed:
        changed = False
        for i in sorted(reach):
            if i == 0:
                continue
            ps = [dom[j] for j in preds[i] if j in reach]
            new = (set.intersection(*ps) if ps else set()) | {i}
            if new != dom[i]:
                dom[i], changed = new, True
    home = max(i for i, b in enumerate(starts) if b <= line)
    loads = []
    for i in sorted(reach):
        if home not in dom[i]:
            continue
        lo = line + 1 if i == home else starts[i]
        loads += [body[n] for n in range(lo, ends[i] + 1)
                  if body[n].startswith("global_load") or body[n].startswith("buffer_load")]
    return loads


def test_every_decode_instance_publishes_before_counting_and_merges_coherently(decode_asm):
    count = 0
    for name, body in _kernels(decode_asm):
        count += 1
        atomics = [n for n, l in enumerate(body) if l.startswith("global_atomic_add")]
        # one counter per path: the slots' partitions, and in the instances
        # that also run prefix items, theirs
        assert 1 <= len(atomics) <= 2, (name, "expected one counter atomic per path")
        for a in atomics:
            # the partial stores just before the counter
            stores = [n for n in range(max(0, a - 150), a) if body[n].startswith("global_store")]
            assert stores, (name, "no partial store before the counter")
            for n in stores:
                assert "sc1" in body[n], (name, body[n])
            last = stores[-1]
            between = body[last + 1:a]
            w = [k for k, l in enumerate(between) if l.startswith("s_waitcnt") and "vmcnt(0)" in l]
            assert w, (name, "no vmcnt(0) between the partial stores and the counter")
            assert any(l.startswith("s_barrier") for l in between[w[0]:]), (name, "no barrier after the wait")
            # every load that only runs after the counter (the merge: after
            # the barrier that publishes the counter's answer through LDS)
            # reads coherently
            bar = [n for n in range(a + 1, min(a + 400, len(body))) if body[n].startswith("s_barrier")]
            assert bar, (name, "no barrier after the counter")
            loads = _dominated_loads(body, bar[0])
            assert loads, (name, "no merge loads after the counter")
            bad = [l for l in loads if "sc1" not in l]
            assert not bad, (name, bad[:3])
    assert count >= 12  # 3 group sizes x 4 page formats
