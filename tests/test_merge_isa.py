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
    cmd = [B.HIPCC, *[a for a in B.COMMON if a != "-fPIC"], "--cuda-device-only", "-S",
           os.path.join(B.CSRC, "decode.hip"), "-o", str(out)]
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


def test_every_decode_instance_publishes_before_counting_and_merges_coherently(decode_asm):
    count = 0
    for name, body in _kernels(decode_asm):
        count += 1
        atomics = [n for n, l in enumerate(body) if l.startswith("global_atomic_add")]
        assert len(atomics) == 1, (name, "expected one counter atomic")
        a = atomics[0]
        # the partial stores just before the counter
        stores = [n for n in range(max(0, a - 120), a) if body[n].startswith("global_store")]
        assert stores, (name, "no partial store before the counter")
        for n in stores:
            assert "sc1" in body[n], (name, body[n])
        last = stores[-1]
        between = body[last + 1:a]
        w = [k for k, l in enumerate(between) if l.startswith("s_waitcnt") and "vmcnt(0)" in l]
        assert w, (name, "no vmcnt(0) between the partial stores and the counter")
        assert any(l.startswith("s_barrier") for l in between[w[0]:]), (name, "no barrier after the wait")
        # every load after the counter (the merge) reads coherently
        loads = [l for l in body[a + 1:] if l.startswith("global_load")]
        assert loads, (name, "no merge loads after the counter")
        bad = [l for l in loads if "sc1" not in l]
        assert not bad, (name, bad[:3])
    assert count >= 12  # 3 group sizes x 4 page formats
