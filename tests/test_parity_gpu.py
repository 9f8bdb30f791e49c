"""GPU parity: the HIP path (through the C ABI) against the FP64 oracle.

Tolerances: output max |d| <= 1e-2 (where the exact output is 4 or more in
magnitude, half its bf16 spacing plus 1e-2: half an ulp alone exceeds 1e-2
there), mean |d| <= 1e-3, LSE max |d| <= 1e-3 on every written row; rows of
inactive slots keep their sentinel bytes exactly.
Bit-exact checks: page gather, page placement, shared-versus-copied prefix,
single-key output, repeat determinism.
"""

from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_attend_amd as pk
from paged_kv_cache_attend_amd import inputs

from gpu_util import (DEV, LSE_SENTINEL, OUT_SENTINEL, TOL_MEAN, bf16_to_f64, compare, half_ulp_bf16, out_bound,
                      run_gpu, run_oracle, say)

pytestmark = pytest.mark.gpu


def _case(ctx, ql=None, hq=8, hkv=2, seed=3, **kw):
    ql = [1] * len(ctx) if ql is None else ql
    return inputs.make_problem("case", seed, ctx, ql, hq, hkv, **kw)


# ---------------------------------------------------------------------------
# decode path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ps", [0, 16, 32, 64, 112])
def test_tiny_decode(ps):
    p = inputs.tiny_decode()
    say(f"tiny_decode partition_size={ps}")
    compare(p, run_gpu(p, partition_size=ps), run_oracle(p), label=f"tiny ps={ps}")


def test_fig_8_10_and_worked_example():
    for p in (inputs.fig_8_10_case(), inputs.worked_example_9_13_5_15()):
        say(p.name)
        compare(p, run_gpu(p), run_oracle(p), label=p.name)


@pytest.mark.parametrize("hq,hkv", [(8, 2), (32, 8), (4, 4), (8, 4), (2, 1)])
@pytest.mark.parametrize("ps", [0, 16, 64, 4096])
def test_decode_ragged_lengths(hq, hkv, ps):
    ctx = [1, 2, 15, 16, 17, 31, 32, 33, 100, 257, 1000, 1023, 1024, 1025, 3001]
    p = _case(ctx, hq=hq, hkv=hkv, seed=hq * 31 + hkv)
    say(f"decode ragged hq={hq} hkv={hkv} ps={ps}")
    compare(p, run_gpu(p, partition_size=ps), run_oracle(p), label=f"ragged {hq}/{hkv} ps={ps}")


@pytest.mark.parametrize("ps", [0, 32, 4096])
def test_zombies_and_empty_slots_untouched(ps):
    # zombies keep a query row (q_len 1, ctx_len 0); q_len 0 slots own no row
    p = _case([0, 37, 0, 100, 5, 0, 64], ql=[1, 1, 1, 1, 0, 0, 1], seed=17)
    say(f"zombies ps={ps}")
    ref = run_oracle(p)
    assert ref[2].tolist() == [False, True, False, True, True]
    compare(p, run_gpu(p, partition_size=ps), ref, label=f"zombies ps={ps}")


def test_all_zombies_write_nothing():
    p = _case([0, 0, 0], seed=19)
    p.ctx_lens[:] = 0
    ob, lb = run_gpu(p, partition_size=32)
    assert (ob == OUT_SENTINEL).all() and (lb.view(np.uint32) == LSE_SENTINEL).all()


def test_single_key_is_bit_exact():
    p = _case([1, 1, 1], hq=32, hkv=8, seed=23)
    q, k, v = p.layer(0)
    ob, lb = run_gpu(p, q=q, k=k, v=v)
    for r in range(3):
        phys = p.block_table[r, 0]
        for h in range(32):
            assert np.array_equal(ob[r, h], v[phys, h // 4, 0]), (r, h)


def test_page_placement_is_bit_exact():
    p = _case([37, 100, 300, 1000, 5], hq=32, hkv=8, seed=29)
    base = run_gpu(p, partition_size=64)
    for seed in (1, 2):
        q, table2, k2, v2 = inputs.relocate(p, 0, seed)
        other = run_gpu(p, q=q, k=k2, v=v2, table=table2, partition_size=64)
        assert np.array_equal(base[0], other[0])
        assert np.array_equal(base[1].view(np.uint32), other[1].view(np.uint32))


def test_shared_prefix_equals_private_copies_bit_exact():
    p = _case([600, 700, 512, 800], hq=32, hkv=8, seed=31, shared_prefix_tokens=512)
    q, k, v = p.layer(0)
    a = run_gpu(p, q=q, k=k, v=v, partition_size=128)
    # give slots 1..3 their own copies of the 32 shared blocks
    extra = 3 * 32
    k2 = np.concatenate([k, np.zeros((extra,) + k.shape[1:], k.dtype)])
    v2 = np.concatenate([v, np.zeros((extra,) + v.shape[1:], v.dtype)])
    table = p.block_table.copy()
    nxt = p.num_blocks
    for r in (1, 2, 3):
        for j in range(32):
            k2[nxt] = k[table[r, j]]
            v2[nxt] = v[table[r, j]]
            table[r, j] = nxt
            nxt += 1
    p2 = inputs.with_block_table(p, table, np.zeros(nxt, np.int32), num_blocks=nxt)
    b = run_gpu(p2, q=q, k=k2, v=v2, table=table, partition_size=128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_repeat_calls_are_deterministic():
    p = _case([2303] * 4, hq=32, hkv=8, seed=37)
    q, k, v = p.layer(0)
    a = run_gpu(p, q=q, k=k, v=v)
    b = run_gpu(p, q=q, k=k, v=v, repeats=3)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))


def test_graph_replay_matches_eager():
    # capture one split call in a graph; replay it several times with eager work
    # in between and check every replay (the workspace must stay consistent)
    p = _case([2303, 700, 0, 1500], hq=32, hkv=8, seed=61)
    q, k, v = p.layer(0)
    eager = run_gpu(p, q=q, k=k, v=v, partition_size=256)
    t = inputs.to_device(p, q, k, v, DEV)
    out = torch.full(q.shape, OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.full(q.shape[:2], LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        call = pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                                 float(p.scale), out, lse, max_q_len=1, max_ctx_len=p.max_ctx_len,
                                 partition_size=256)
        assert call.num_partitions == 9
        call.launch(s)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            call.launch(s)
        for i in range(4):
            out.view(torch.int16).fill_(OUT_SENTINEL)
            lse.view(torch.int32).fill_(LSE_SENTINEL)
            g.replay()
            torch.cuda.synchronize()
            ob = out.view(torch.int16).cpu().numpy().view(np.uint16)
            assert np.array_equal(ob, eager[0]), f"replay {i}"
            assert np.array_equal(lse.cpu().numpy().view(np.uint32), eager[1].view(np.uint32)), f"replay {i}"


def test_back_to_back_calls_never_read_stale_partials():
    # Two batches of one shape share a workspace and alternate: every call's
    # merge must use that call's partials only, never the previous call's.
    ctx = [2303, 700, 1500, 64]
    a = _case(ctx, hq=32, hkv=8, seed=73)
    b = _case(ctx, hq=32, hkv=8, seed=79)
    ref = {}
    dev = {}
    for name, prob in (("a", a), ("b", b)):
        q, k, v = prob.layer(0)
        ref[name] = run_gpu(prob, q=q, k=k, v=v, partition_size=128)
        dev[name] = inputs.to_device(prob, q, k, v, DEV)
    shape = pk.make_shape(a.num_seqs, a.total_q, 32, 8, a.max_blocks_per_seq, 1, a.max_ctx_len,
                          a.num_blocks, 128)
    ws = torch.empty(pk.workspace_size(shape), dtype=torch.uint8, device=DEV)
    pk.workspace_init(shape, ws)
    outs = []
    for i in range(12):
        name = "ab"[i % 2]
        t = dev[name]
        out = torch.full(t["q"].shape, OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        lse = torch.full(t["q"].shape[:2], LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
        pk.attend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"], float(a.scale),
                  out, lse, max_q_len=1, max_ctx_len=a.max_ctx_len, partition_size=128, workspace=ws)
        outs.append((name, out, lse))
    torch.cuda.synchronize()
    for i, (name, out, lse) in enumerate(outs):
        ob = out.view(torch.int16).cpu().numpy().view(np.uint16)
        assert np.array_equal(ob, ref[name][0]), f"call {i} ({name})"
        assert np.array_equal(lse.cpu().numpy().view(np.uint32), ref[name][1].view(np.uint32)), f"call {i}"


def test_workspace_reused_across_shapes():
    # one workspace, re-initialised for each new shape, serves different batches
    a = _case([3000, 40, 900], hq=32, hkv=8, seed=67)
    b = _case([100, 2000, 2000, 64, 5000, 1], hq=32, hkv=8, seed=71)
    ws = torch.empty(64 << 20, dtype=torch.uint8, device=DEV)
    for prob in (a, b, a):
        q, k, v = prob.layer(0)
        t = inputs.to_device(prob, q, k, v, DEV)
        out = torch.zeros(q.shape, dtype=torch.bfloat16, device=DEV)
        lse = torch.zeros(q.shape[:2], dtype=torch.float32, device=DEV)
        shape = pk.make_shape(prob.num_seqs, prob.total_q, 32, 8, prob.max_blocks_per_seq, 1,
                              prob.max_ctx_len, prob.num_blocks, 128)
        pk.workspace_init(shape, ws)
        pk.attend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"], float(prob.scale),
                  out, lse, max_q_len=1, max_ctx_len=prob.max_ctx_len, partition_size=128, workspace=ws)
        torch.cuda.synchronize()
        ob = out.view(torch.int16).cpu().numpy().view(np.uint16)
        ref = run_oracle(prob)
        compare(prob, (ob, lse.cpu().numpy()), ref, label=f"reuse {prob.ctx_lens.tolist()}")


def test_lse_optional():
    p = _case([37, 100], seed=41)
    ob, lb = run_gpu(p, with_lse=False, partition_size=32)
    assert lb is None
    compare(p, (ob, None), run_oracle(p), label="no lse")


def test_long_contexts_many_partitions():
    # 2 slots x 65536 keys on 8 KV heads: the automatic plan, then 64
    # partitions of 64 pages, so the merge folds its partials in three
    # batches (28 + 28 + 8); plus a batch of 600 short slots (4800 (slot, KV
    # head) pairs, several rounds of workgroups).
    p = _case([65536, 61000], hq=32, hkv=8, seed=91)
    shape = pk.make_shape(p.num_seqs, p.total_q, 32, 8, p.max_blocks_per_seq, 1, p.max_ctx_len, p.num_blocks)
    assert pk.plan(shape)[1] >= 16
    shape64 = pk.make_shape(p.num_seqs, p.total_q, 32, 8, p.max_blocks_per_seq, 1, p.max_ctx_len, p.num_blocks,
                            partition_size=1024)
    assert pk.plan(shape64)[1] == 64
    ref = run_oracle(p)
    say("decode 2 x 65536 keys, automatic partitions")
    compare(p, run_gpu(p), ref, label="long contexts")
    say("decode 2 x 65536 keys, 64 partitions")
    compare(p, run_gpu(p, partition_size=1024), ref, label="long contexts, 64 partitions")
    rng = np.random.default_rng(92)
    q = _case([int(x) for x in rng.integers(1, 300, 600)], hq=32, hkv=8, seed=93)
    say("decode 600 short slots")
    compare(q, run_gpu(q), run_oracle(q), label="600 slots")


# ---------------------------------------------------------------------------
# the reference workloads at full size (sampled layers)
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("layer", [0, 35])
def test_qwen3_short_decode_full_size(layer):
    p = inputs.qwen3_short_decode(num_layers=36)
    say(f"qwen3 short decode layer {layer}")
    compare(p, run_gpu(p, layer), run_oracle(p, layer), label=f"cfg2 layer {layer}")


def test_qwen3_shared_prefix_decode_full_size():
    p = inputs.qwen3_shared_prefix_decode(num_layers=36)
    say("qwen3 shared-prefix decode layer 7")
    compare(p, run_gpu(p, 7), run_oracle(p, 7), label="cfg3 layer 7")


def test_ragged_mixed_decode_full_size():
    p = inputs.ragged_mixed_decode()
    say("ragged mixed decode")
    assert pk.plan(pk.make_shape(p.num_seqs, p.total_q, 32, 8, 528, 1, p.max_ctx_len, p.num_blocks,
                                 partition_size=512))[1] == -(-p.max_ctx_len // 512)
    compare(p, run_gpu(p), run_oracle(p), label="cfg4")


def test_chunked_denoise_full_size():
    p = inputs.chunked_denoise()
    say("chunked denoise")
    compare(p, run_gpu(p), run_oracle(p), label="cfg5")


# ---------------------------------------------------------------------------
# chunk (MFMA) path
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("ctx,ql,hq,hkv", [
    ([64, 40], [8, 3], 4, 4),
    ([20, 50, 31], [20, 7, 1], 6, 2),
    ([300, 1024, 17], [129, 256, 17], 24, 24),
    ([1000, 77], [200, 2], 32, 8),
    ([33, 0, 65], [2, 1, 65], 8, 8),
])
@pytest.mark.parametrize("causal", [False, True])
def test_chunk_path(ctx, ql, hq, hkv, causal):
    p = _case(ctx, ql, hq=hq, hkv=hkv, seed=sum(ctx) + hq, causal=causal)
    say(f"chunk ctx={ctx} ql={ql} {hq}/{hkv} causal={causal}")
    compare(p, run_gpu(p), run_oracle(p), label=f"chunk {ctx} {ql} causal={causal}")


@pytest.mark.parametrize("num_seqs", [37, 70])
def test_chunk_path_many_slots(num_seqs):
    # the row offset of a slot sums the query lengths of all earlier slots
    # (in batches of 16 in the kernel): slots past 16, 32 and 64, some with
    # no query rows
    rng = np.random.default_rng(num_seqs)
    ctx = rng.integers(1, 120, size=num_seqs)
    ql = np.minimum(ctx, rng.integers(0, 6, size=num_seqs))
    p = _case(ctx.tolist(), ql.tolist(), hq=4, hkv=2, seed=num_seqs, causal=True)
    say(f"chunk many slots: {num_seqs}")
    compare(p, run_gpu(p), run_oracle(p), label=f"chunk {num_seqs} slots")


# Rows that see few keys: on the paths that feed PV single bf16 weights (the
# chunk kernel, decode with several tokens per slot where the score tile has
# no room for the lo copies), such rows cannot average the weights' rounding
# down, so there the weights go in as hi + lo halves.  Their outputs then
# carry the output rounding and fp32-level error only: half a bf16 ulp plus
# 2.5e-4, where single bf16 weights leave up to ~4e-3 on top of the half ulp
# (a CPU emulation of both on 2 - 40 keys: 3.3e-3 - 4.3e-3 against 1.5e-5).
FEW_KEY_CASES = [
    # decode, 8 tokens x 4 heads = 32 columns (two score tiles)
    ("decode_m8", dict(ctx=list(range(2, 42)), ql=[min(n, 1 + n % 8) for n in range(2, 42)], hq=32, hkv=8)),
    # decode, 2 tokens x 8 heads = 16 columns
    ("decode_g8_m2", dict(ctx=list(range(2, 40)), ql=[1 + n % 2 for n in range(2, 40)], hq=64, hkv=8)),
    # chunk path: a first prefill chunk (row t sees t + 1 keys), causal
    ("chunk_first_chunk", dict(ctx=[200, 130, 64], ql=[200, 130, 64], hq=8, hkv=8)),
    # chunk path, four heads per KV head, a tail with few keys in the second key half
    ("chunk_g4", dict(ctx=[300, 97, 40], ql=[40, 33, 40], hq=32, hkv=8)),
]


@pytest.mark.parametrize("name,case", FEW_KEY_CASES, ids=[c[0] for c in FEW_KEY_CASES])
def test_few_key_rows_within_output_rounding(name, case):
    p = _case(case["ctx"], ql=case["ql"], hq=case["hq"], hkv=case["hkv"], seed=67, causal=True)
    got = run_gpu(p)
    ref = run_oracle(p)
    compare(p, got, ref, label=name)
    out, _, written = ref
    o = bf16_to_f64(got[0])
    # keys each row sees (token t of a slot's m sees n - m + t + 1)
    vis = np.concatenate([np.arange(int(n) - int(m) + 1, int(n) + 1) for n, m in zip(p.ctx_lens, p.q_lens)])
    few = written & (vis < 64)
    assert few.any()
    err = np.abs(o[few] - out[few])
    over = err - half_ulp_bf16(out[few])
    say(f"  {name}: {int(few.sum())} rows with < 64 keys, max |dout| beyond half an ulp {over.max():.2e}")
    assert over.max() <= 2.5e-4, float(over.max())


def test_chunked_prefill_page_example_full_size():
    # section 8.2.3: the last 512-token chunk of an 8192-token prompt, causal,
    # Qwen3-8B heads; 4,063,488 visible (query, key) pairs per head
    p = inputs.chunked_prefill()
    m, n = int(p.q_lens[0]), int(p.ctx_lens[0])
    assert m * (n - m) + m * (m + 1) // 2 == 4_063_488
    say("chunked prefill c=512 h=7680")
    compare(p, run_gpu(p), run_oracle(p), label="chunked prefill c512 h7680")


@pytest.mark.parametrize("num_tokens", [5, 8])
def test_speculative_verification(num_tokens):
    # 16 requests x 2303 keys, 5 or 8 new tokens each, causal over them, 32/8
    # heads: (token, query head) rows of a KV head packed into one tile
    p = inputs.speculative_verify(num_tokens)
    say(f"speculative verification m={num_tokens}")
    compare(p, run_gpu(p), run_oracle(p), label=f"spec verify m={num_tokens}")


def test_decode_with_eight_query_heads_per_kv_head():
    # G = 8: eight hi and eight lo columns fill the decode kernel's tile
    p = _case([37, 100, 1000], hq=64, hkv=8, seed=43)
    assert pk.plan(pk.make_shape(p.num_seqs, p.total_q, 64, 8, p.max_blocks_per_seq, 1, p.max_ctx_len,
                                 p.num_blocks))[0] >= 0
    compare(p, run_gpu(p), run_oracle(p), label="G=8 decode")


@pytest.mark.parametrize("hq,hkv", [(8, 8), (4, 2), (8, 2), (32, 8), (16, 2)])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("ps", [0, 16, 4096])
def test_multi_token_decode(hq, hkv, causal, ps):
    # several new tokens per slot on the page-streaming decode path (tokens
    # x group <= 32): ragged lengths, token counts below the slot maximum,
    # a zombie, a slot without new tokens, the last page partly filled
    G = hq // hkv
    mmax = max(1, min(8, 32 // G))
    ctx = [37, 100, 1000, 17, 2303, 0, 64, 500]
    ql = [min(mmax, x) for x in (1, 3, mmax, 2, mmax, 1, 0, max(1, mmax - 1))]
    p = _case(ctx, ql, hq=hq, hkv=hkv, seed=hq * 7 + hkv + mmax, causal=causal)
    say(f"multi-token decode {hq}/{hkv} m<={mmax} causal={causal} ps={ps}")
    compare(p, run_gpu(p, partition_size=ps), run_oracle(p),
            label=f"multi-token {hq}/{hkv} m<={mmax} causal={causal} ps={ps}")


# ---------------------------------------------------------------------------
# gather, combine, validate
# ---------------------------------------------------------------------------

def test_gather_is_bit_exact():
    p = _case([37, 100, 0, 16, 1000], hq=8, hkv=2, seed=47)
    q, k, v = p.layer(0)
    t = inputs.to_device(p, q, k, v, DEV)
    dst = torch.full((p.num_seqs, p.max_ctx_len, 2, 128), 0x1234, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    pk.gather_kv(t["k"], t["block_table"], t["ctx_lens"], dst, max_ctx_len=p.max_ctx_len)
    torch.cuda.synchronize()
    got = dst.view(torch.int16).cpu().numpy().view(np.uint16)
    for r in range(p.num_seqs):
        n = int(p.ctx_lens[r])
        j = np.arange(n)
        expect = k[p.block_table[r][j // 16], :, j % 16, :]  # [n][Hkv][D]
        assert np.array_equal(got[r, :n], expect)
        assert (got[r, n:] == 0x1234).all()


def test_combine_matches_oracle_merge():
    rng = np.random.default_rng(53)
    P, rows, D = 7, 300, 128
    po = rng.standard_normal((P, rows, D)).astype(np.float32)
    pl = (rng.standard_normal((P, rows)) * 4).astype(np.float32)
    dead = rng.random((P, rows)) < 0.3
    pl[dead] = -np.inf
    po[dead] = np.nan
    pl[:, 5] = -np.inf   # a row with no live partial stays untouched
    po[:, 5] = np.nan
    out = torch.full((rows, D), OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.full((rows,), LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
    pk.combine(torch.from_numpy(po).to(DEV), torch.from_numpy(pl).to(DEV), out, lse)
    torch.cuda.synchronize()
    ref_o, ref_l, touched = oracle.combine_fp64(po, pl)
    ob = out.view(torch.int16).cpu().numpy().view(np.uint16)
    lb = lse.cpu().numpy()
    o = bf16_to_f64(ob)
    assert not touched[5] and (ob[5] == OUT_SENTINEL).all() and lb[5:6].view(np.uint32)[0] == LSE_SENTINEL
    err = np.abs(o[touched] - ref_o[touched])
    say(f"combine: max |dout| {err.max():.3e}, mean {err.mean():.3e}")
    assert (err <= out_bound(ref_o[touched])).all(), float((err / out_bound(ref_o[touched])).max())
    assert err.mean() <= TOL_MEAN
    assert np.abs(lb[touched] - ref_l[touched]).max() <= 1e-4


def test_validate_flags_bad_data():
    p = _case([37, 100, 0], ql=[1, 1, 1], seed=59)
    bt = torch.from_numpy(p.block_table).to(DEV)
    cl = torch.from_numpy(p.ctx_lens).to(DEV)
    ql = torch.from_numpy(p.q_lens).to(DEV)
    word = torch.full((1,), -1, dtype=torch.int32, device=DEV)

    def check(bt_, cl_, ql_, **kw):
        args = dict(num_blocks=p.num_blocks, total_q=3, max_q_len=1, max_ctx_len=100)
        args.update(kw)
        pk.validate(bt_, cl_, ql_, word, **args)
        torch.cuda.synchronize()
        return int(word.item())

    assert check(bt, cl, ql) == 0
    bad = bt.clone()
    bad[1, 3] = p.num_blocks
    assert check(bad, cl, ql) == pk._lib.PA_BAD_BLOCK_ID
    assert check(bt, cl, ql, max_ctx_len=99) == pk._lib.PA_BAD_CTX_LEN
    assert check(bt, cl, ql, total_q=2) == pk._lib.PA_BAD_TOTAL_Q
    ql2 = ql.clone()
    ql2[0] = 40
    assert check(bt, cl, ql2, max_q_len=64, total_q=64) == pk._lib.PA_BAD_Q_LEN


def test_validate_flags_unzeroed_workspace_counters():
    # A split shape (3 slots x 2 KV heads, 16-token partitions): the counters
    # are zero after pa_workspace_init and after a completed call, and a
    # non-zero one (a workspace not initialised for the shape) is flagged.
    p = _case([37, 100, 0], ql=[1, 1, 1], seed=59)
    t = inputs.to_device(p, *p.layer(0), DEV)
    kw = dict(num_blocks=p.num_blocks, total_q=p.total_q, max_q_len=1, max_ctx_len=p.max_ctx_len,
              num_q_heads=p.num_q_heads, num_kv_heads=p.num_kv_heads, partition_size=16)
    shape = pk.make_shape(p.num_seqs, p.total_q, p.num_q_heads, p.num_kv_heads, p.max_blocks_per_seq, 1,
                          p.max_ctx_len, p.num_blocks, 16)
    ws = torch.full((pk.workspace_size(shape),), 0x5A, dtype=torch.uint8, device=DEV)
    word = torch.full((1,), -1, dtype=torch.int32, device=DEV)

    def check():
        pk.validate(t["block_table"], t["ctx_lens"], t["q_lens"], word, workspace=ws, **kw)
        torch.cuda.synchronize()
        return int(word.item())

    assert check() == pk._lib.PA_BAD_WORKSPACE
    pk.workspace_init(shape, ws)
    assert check() == 0
    out = torch.empty_like(t["q"])
    pk.attend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"], float(p.scale), out,
              max_q_len=1, max_ctx_len=p.max_ctx_len, partition_size=16, workspace=ws)
    assert check() == 0
    ws[:4].view(torch.int32).fill_(1)
    assert check() == pk._lib.PA_BAD_WORKSPACE


def test_binding_on_a_non_current_stream():
    # attend() allocates its workspace from the launch stream's pool and zeroes
    # its counters there; PreparedAttend zeroes on its construction stream
    # and waits, so a launch on any other stream sees zeroed counters.
    p = _case([300, 1000, 37, 2000], hq=32, hkv=8, seed=61)
    ref = run_oracle(p)
    t = inputs.to_device(p, *p.layer(0), DEV)
    side = torch.cuda.Stream(device=DEV)
    for _ in range(3):
        out = torch.full(t["q"].shape, OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        lse = torch.full(t["q"].shape[:2], LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
        torch.cuda.synchronize()
        pk.attend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"], float(p.scale), out, lse,
                  max_q_len=1, max_ctx_len=p.max_ctx_len, partition_size=64, stream=side)
        side.synchronize()
        compare(p, (out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()), ref,
                label="attend on a side stream")
    out = torch.full(t["q"].shape, OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = torch.full(t["q"].shape[:2], LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
    torch.cuda.synchronize()
    call = pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                             float(p.scale), out, lse, max_q_len=1, max_ctx_len=p.max_ctx_len, partition_size=64)
    assert call.num_partitions > 1
    call.launch(side)
    side.synchronize()
    compare(p, (out.view(torch.int16).cpu().numpy().view(np.uint16), lse.cpu().numpy()), ref,
            label="prepared call launched on a side stream")
