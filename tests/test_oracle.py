"""Pins of the FP64 oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible slip in the oracle (a dropped term, a
wrong sign, index or head mapping, a transposed operand, log2 for ln, reading
past a request's keys) fails at least one of them:

* integer facts printed on the inference-optimisation page (golden file);
* special cases with closed forms (one key, two keys, zero query, constant V);
* invariances the definition implies (page placement, key order, scale
  factoring, GQA as repeated-head MHA, shared versus copied prefix);
* a library routine on an independently built contiguous layout
  (torch's scaled-dot-product attention and logsumexp in float64);
* the split-KV identity for the log-sum-exp merge.
"""

from __future__ import annotations

import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import closed_forms as cf
from paged_kv_cache_attend_amd import inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "kv_closed_forms.txt")
MIB = 1 << 20
GIB = 1 << 30


def _golden():
    facts = {}
    with open(GOLDEN) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            name, rest = line.split(None, 1)
            value = int(rest.split("|")[0].strip())
            facts[name] = value
    return facts


# --------------------------------------------------------------------------
# closed forms vs the page
# --------------------------------------------------------------------------

def test_golden_kv_closed_forms():
    g = _golden()
    k = cf.kv_bytes_per_token(36, 8, 128, 2)
    assert k == g["kv_bytes_per_token"]
    assert k == g["kv_bytes_per_token_kib"] * 1024
    assert 2048 * k == g["kv_mib_prefill_2048"] * MIB
    assert 8192 * k == g["kv_mib_prefill_8192"] * MIB
    assert 8192 * k * 1000 == g["kv_gib_x1000_per_long_request"] * GIB
    assert 16 * 8192 * k == g["kv_gib_16_long_inputs"] * GIB
    assert 2048 + 255 == g["tokens_computed_short"]
    assert 8192 + 255 == g["tokens_computed_long"]
    assert 16 * cf.blocks_needed(2303, 16) == g["slots_allocated_short"]
    assert 16 * cf.blocks_needed(8447, 16) == g["slots_allocated_long"]
    assert cf.kv_alloc_bytes(2303, 16, k) == g["kv_mib_after_256_short"] * MIB
    assert cf.kv_alloc_bytes(8447, 16, k) == g["kv_mib_after_256_long"] * MIB
    assert (12 * GIB) // cf.kv_alloc_bytes(2303, 16, k) == g["requests_in_12gib_short"]
    assert (12 * GIB) // cf.kv_alloc_bytes(8447, 16, k) == g["requests_in_12gib_long"]


def test_golden_paging_worked_example():
    g = _golden()
    lens = [9, 13, 5, 15]
    assert 4 * 16 == g["worked_reserved_whole"]
    assert [4 * cf.blocks_needed(L, 4) for L in lens] == [12, 16, 8, 16]
    assert cf.allocated_token_slots(lens, 4) == g["worked_paged_p4"]
    assert sum(lens) == g["worked_used"]
    assert 64 - sum(lens) == g["worked_unused_whole"]
    assert sum(cf.tail_waste(L, 4) for L in lens) == g["worked_unused_paged"]
    assert all(cf.tail_waste(L, 4) <= 3 for L in range(1, 200))
    # A and B share their first 8 tokens = two whole 4-token blocks.
    shared_blocks = 8 // 4
    assert cf.allocated_token_slots(lens, 4) - 4 * shared_blocks == g["worked_paged_shared_ab8"]


def test_golden_branch_sharing():
    g = _golden()
    assert cf.block_references(95, 9, 4) == g["branch_references"]
    assert cf.shared_physical_blocks(95, 9, 4) == g["branch_physical_blocks"]
    saving = 1 - cf.shared_physical_blocks(95, 9, 4) / cf.block_references(95, 9, 4)
    assert round(100 * saving) == g["branch_saving_percent"]


def test_golden_shared_prefix_capacity():
    g = _golden()
    k = cf.kv_bytes_per_token(36, 8, 128, 2)
    assert cf.kv_alloc_bytes(6144, 16, k) == g["shared_prefix_mib"] * MIB
    assert 8192 - 6144 + 255 == g["shared_private_tokens"]
    assert cf.kv_alloc_bytes(2303, 16, k) == g["shared_private_mib"] * MIB
    assert cf.shared_prefix_alloc_bytes(6144, 2303, 16, 16, k) == g["shared_16_total_mib"] * MIB
    assert 16 * cf.kv_alloc_bytes(8447, 16, k) == g["unshared_16_total_mib"] * MIB
    cap = max(b for b in range(1, 100) if cf.shared_prefix_alloc_bytes(6144, 2303, b, 16, k) <= 12 * GIB)
    assert cap == g["shared_capacity_requests_12g"]


def test_golden_chunk_pairs():
    g = _golden()
    assert cf.causal_pairs(0, 512) == g["pairs_c512_h0"]
    assert cf.causal_pairs(7680, 512) == g["pairs_c512_h7680"]
    assert cf.causal_pairs(0, 4) == g["pairs_fig8_8"]
    assert cf.causal_pairs(8, 4) == g["pairs_fig8_9"]


def test_reference_workload_pools_match_closed_forms():
    k = cf.kv_bytes_per_token(36, 8, 128, 2)
    p2 = inputs.qwen3_short_decode(num_layers=1)
    live = int((p2.block_fill > 0).sum())
    assert live == 16 * 144 == 2304
    assert live * 16 * k == 16 * cf.kv_alloc_bytes(2303, 16, k)
    p3 = inputs.qwen3_shared_prefix_decode(num_layers=1)
    live3 = int((p3.block_fill > 0).sum())
    assert live3 == 384 + 10 * 144
    assert live3 * 16 * k == cf.shared_prefix_alloc_bytes(6144, 2303, 10, 16, k)
    assert (p3.block_table[:, :384] == p3.block_table[0, :384]).all()
    # the shared-prefix workload's unique KV bytes per layer
    assert p3.kv_bytes_unique() == 119_496_704
    assert p2.kv_bytes_read() == 150_929_408
    p5 = inputs.chunked_denoise()
    pairs = int((p5.q_lens * p5.ctx_lens).sum())
    assert cf.chunk_attention_flops(pairs, 24, 128) == 12_884_901_888


# --------------------------------------------------------------------------
# helpers for small problems
# --------------------------------------------------------------------------

def _small(ctx, ql=None, hq=8, hkv=2, d=128, seed=7, **kw):
    ql = [1] * len(ctx) if ql is None else ql
    return inputs.make_problem("t", seed, ctx, ql, hq, hkv, head_dim=d, **kw)


def _run(p, layer=0, q=None, k=None, v=None, table=None, causal=False):
    q0, k0, v0 = p.layer(layer)
    q = q0 if q is None else q
    k = k0 if k is None else k
    v = v0 if v is None else v
    table = p.block_table if table is None else table
    return oracle.attend_fp64(q, k, v, table, p.ctx_lens, p.q_lens, p.scale,
                              p.num_kv_heads, p.block_size, causal=causal)


def _bits(x: np.ndarray) -> np.ndarray:
    """Exact float -> bf16 bits for values that bf16 represents exactly."""
    f = np.asarray(x, dtype=np.float32)
    b = (f.view(np.uint32) >> 16).astype(np.uint16)
    assert np.array_equal(oracle.bf16_bits_to_f64(b), f.astype(np.float64))
    return b


def _contiguous(pool_bits, p, r, g):
    """Contiguous keys of request r / KV head g built with one fancy-index
    over a flattened (block*slot) axis -- a second statement of the layout."""
    nb, hkv, bs, d = pool_bits.shape
    flat = np.transpose(pool_bits, (1, 0, 2, 3)).reshape(hkv, nb * bs, d)
    n = int(p.ctx_lens[r])
    j = np.arange(n)
    idx = p.block_table[r][j // bs].astype(np.int64) * bs + (j % bs)
    return oracle.bf16_bits_to_f64(flat[g][idx])


# --------------------------------------------------------------------------
# special cases with closed forms
# --------------------------------------------------------------------------

def test_bf16_widening_exact():
    vals = np.array([1.0, -2.5, 0.15625, 3.0e38, -1.0e-30, 0.0], dtype=np.float32)
    bits = (vals.view(np.uint32) >> 16).astype(np.uint16)
    trunc = (bits.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(oracle.bf16_bits_to_f64(bits), trunc.astype(np.float64))
    assert oracle.bf16_bits_to_f64(np.uint16(0x3F80)) == 1.0
    assert oracle.bf16_bits_to_f64(np.uint16(0xC000)) == -2.0


def test_single_key_returns_its_value():
    p = _small([1, 1], hq=8, hkv=2)
    q, k, v = p.layer(0)
    out, lse, wr = _run(p)
    assert wr.all()
    G = 4
    for r in range(2):
        phys = p.block_table[r, 0]
        for h in range(8):
            vrow = oracle.bf16_bits_to_f64(v[phys, h // G, 0])
            assert np.array_equal(out[r, h], vrow)
            krow = oracle.bf16_bits_to_f64(k[phys, h // G, 0])
            qrow = oracle.bf16_bits_to_f64(q[r, h])
            assert lse[r, h] == pytest.approx(float(p.scale) * float(qrow @ krow), abs=1e-12)


def test_zero_query_gives_uniform_weights():
    p = _small([37, 100, 16])
    q, k, v = p.layer(0)
    q = np.zeros_like(q)
    out, lse, _ = _run(p, q=q)
    for r in range(3):
        n = int(p.ctx_lens[r])
        for h in range(8):
            assert lse[r, h] == pytest.approx(math.log(n), abs=1e-12)
            V = _contiguous(v, p, r, h // 4)
            np.testing.assert_allclose(out[r, h], V.mean(axis=0), atol=1e-12, rtol=0)


def test_two_keys_logistic():
    p = _small([2, 2, 2], hq=4, hkv=4)
    q, k, v = p.layer(0)
    out, lse, _ = _run(p)
    for r in range(3):
        for h in range(4):
            K = _contiguous(k, p, r, h)
            V = _contiguous(v, p, r, h)
            qv = oracle.bf16_bits_to_f64(q[r, h])
            s0, s1 = float(p.scale) * (K @ qv)
            w0 = 1.0 / (1.0 + math.exp(-(s0 - s1)))
            np.testing.assert_allclose(out[r, h], w0 * V[0] + (1 - w0) * V[1], atol=1e-12, rtol=0)
            assert lse[r, h] == pytest.approx(max(s0, s1) + math.log1p(math.exp(-abs(s0 - s1))), abs=1e-12)


def test_constant_values_give_constant_output():
    p = _small([37, 100, 5, 64])
    q, k, v = p.layer(0)
    c = np.array([0.75, -1.5], dtype=np.float32)
    v2 = v.copy()
    # a distinct constant per KV head, exact in bf16, for every live slot
    for g in range(p.num_kv_heads):
        v2[:, g, :, :] = _bits(np.full(1, c[g]))[0]
    out, _, _ = _run(p, v=v2)
    for r in range(4):
        for h in range(8):
            assert np.abs(out[r, h] - float(c[h // 4])).max() <= 1e-15


# --------------------------------------------------------------------------
# invariances
# --------------------------------------------------------------------------

def test_physical_placement_does_not_matter():
    p = _small([37, 100, 5, 64, 129])
    out, lse, _ = _run(p)
    for seed in (1, 2):
        q, table2, k2, v2 = inputs.relocate(p, 0, seed)
        out2, lse2, _ = oracle.attend_fp64(q, k2, v2, table2, p.ctx_lens, p.q_lens, p.scale,
                                           p.num_kv_heads, p.block_size)
        assert np.array_equal(out, out2, equal_nan=True)
        assert np.array_equal(lse, lse2, equal_nan=True)


def test_key_order_does_not_matter_with_full_mask():
    # whole blocks only, so permuting table columns permutes keys
    p = _small([64, 128, 48])
    out, lse, _ = _run(p)
    rng = np.random.default_rng(3)
    table = p.block_table.copy()
    for r in range(3):
        nb = int(p.ctx_lens[r]) // 16
        table[r, :nb] = table[r, rng.permutation(nb)]
    out2, lse2, _ = _run(p, table=table)
    np.testing.assert_allclose(out2, out, atol=1e-13, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-13, rtol=0)


def test_scale_factoring_by_power_of_two():
    p = _small([37, 100])
    q, k, v = p.layer(0)
    out, lse, _ = _run(p)
    # q * 2 is exact in bf16 (exponent bump) -- scale / 2 is exact in fp32
    qf = oracle.bf16_bits_to_f64(q).astype(np.float32) * np.float32(2.0)
    q2 = _bits(qf)
    out2, lse2, _ = oracle.attend_fp64(q2, k, v, p.block_table, p.ctx_lens, p.q_lens,
                                       np.float32(p.scale) / np.float32(2.0), p.num_kv_heads)
    np.testing.assert_allclose(out2, out, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-14, rtol=0)


def test_gqa_equals_mha_with_repeated_kv_heads():
    p = _small([37, 100, 17], hq=8, hkv=2)
    q, k, v = p.layer(0)
    out, lse, _ = _run(p)
    k_rep = np.repeat(k, 4, axis=1)
    v_rep = np.repeat(v, 4, axis=1)
    out2, lse2, _ = oracle.attend_fp64(q, k_rep, v_rep, p.block_table, p.ctx_lens, p.q_lens,
                                       p.scale, 8)
    np.testing.assert_allclose(out2, out, atol=1e-14, rtol=0)
    np.testing.assert_allclose(lse2, lse, atol=1e-14, rtol=0)


def test_shared_prefix_equals_private_copies():
    p = _small([80, 96, 70], shared_prefix_tokens=64)
    q, k, v = p.layer(0)
    out, lse, _ = _run(p)
    # copy the shared blocks into fresh private blocks for slots 1 and 2
    nb = p.num_blocks
    extra = 2 * 4
    k2 = np.concatenate([k, np.zeros((extra,) + k.shape[1:], k.dtype)])
    v2 = np.concatenate([v, np.zeros((extra,) + v.shape[1:], v.dtype)])
    table = p.block_table.copy()
    nxt = nb
    for r in (1, 2):
        for j in range(4):
            k2[nxt] = k[table[r, j]]
            v2[nxt] = v[table[r, j]]
            table[r, j] = nxt
            nxt += 1
    assert len({int(table[r, 0]) for r in range(3)}) == 3
    out2, lse2, _ = oracle.attend_fp64(q, k2, v2, table, p.ctx_lens, p.q_lens, p.scale,
                                       p.num_kv_heads)
    assert np.array_equal(out, out2, equal_nan=True)
    assert np.array_equal(lse, lse2, equal_nan=True)


# --------------------------------------------------------------------------
# library routine on an independently gathered contiguous layout
# --------------------------------------------------------------------------

@pytest.mark.parametrize("ctx,ql,hq,hkv", [
    ([37, 100], [1, 1], 8, 2),
    ([1, 16, 17, 33, 95], [1, 1, 1, 1, 1], 32, 8),
    ([64, 40], [8, 3], 4, 4),
    ([20, 50, 31], [20, 7, 1], 6, 2),
])
def test_paged_matches_torch_sdpa_on_contiguous_layout(ctx, ql, hq, hkv):
    p = _small(ctx, ql, hq=hq, hkv=hkv, seed=11)
    q, k, v = p.layer(0)
    out, lse, wr = _run(p)
    assert wr.all()
    G = hq // hkv
    row = 0
    for r in range(len(ctx)):
        m = int(p.q_lens[r])
        Q = torch.from_numpy(oracle.bf16_bits_to_f64(q[row:row + m])).permute(1, 0, 2)  # [Hq][m][D]
        K = torch.stack([torch.from_numpy(_contiguous(k, p, r, g)) for g in range(hkv)])
        V = torch.stack([torch.from_numpy(_contiguous(v, p, r, g)) for g in range(hkv)])
        K = K.repeat_interleave(G, dim=0)
        V = V.repeat_interleave(G, dim=0)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, scale=float(p.scale)).permute(1, 0, 2).numpy()
        ref_lse = torch.logsumexp(float(p.scale) * (Q @ K.transpose(1, 2)), dim=-1).T.numpy()
        np.testing.assert_allclose(out[row:row + m], ref, atol=1e-12, rtol=0)
        np.testing.assert_allclose(lse[row:row + m], ref_lse, atol=1e-12, rtol=0)
        row += m


def test_causal_matches_torch_sdpa_with_bottom_right_mask():
    p = _small([40, 33], [8, 5], hq=4, hkv=2, seed=5)
    q, k, v = p.layer(0)
    out, lse, _ = _run(p, causal=True)
    row = 0
    for r in range(2):
        n, m = int(p.ctx_lens[r]), int(p.q_lens[r])
        Q = torch.from_numpy(oracle.bf16_bits_to_f64(q[row:row + m])).permute(1, 0, 2)
        K = torch.stack([torch.from_numpy(_contiguous(k, p, r, g)) for g in range(2)]).repeat_interleave(2, 0)
        V = torch.stack([torch.from_numpy(_contiguous(v, p, r, g)) for g in range(2)]).repeat_interleave(2, 0)
        allowed = torch.ones(m, n, dtype=torch.bool).tril(diagonal=n - m)
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K, V, attn_mask=allowed, scale=float(p.scale)).permute(1, 0, 2).numpy()
        np.testing.assert_allclose(out[row:row + m], ref, atol=1e-12, rtol=0)
        assert int(allowed.sum()) == cf.causal_pairs(n - m, m)
        row += m


def test_causal_single_row_is_full():
    p = _small([37, 100, 1])
    a = _run(p)
    b = _run(p, causal=True)
    assert np.array_equal(a[0], b[0], equal_nan=True)
    assert np.array_equal(a[1], b[1], equal_nan=True)


# --------------------------------------------------------------------------
# paging edge cases, zombies, poison
# --------------------------------------------------------------------------

def test_fig_8_10_hand_case():
    p = inputs.fig_8_10_case()
    q, k, v = p.layer(0)
    assert np.isnan(oracle.bf16_bits_to_f64(k[1])).all()
    out, lse, wr = _run(p)
    assert wr.all() and np.isfinite(out).all() and np.isfinite(lse).all()
    # contiguous statement: logical block i is physical [2, 0, 3][i]
    Kc = np.concatenate([k[2], k[0], k[3]], axis=1)  # [Hkv][48][D]
    Vc = np.concatenate([v[2], v[0], v[3]], axis=1)
    Q = torch.from_numpy(oracle.bf16_bits_to_f64(q[0]))[:, None, :]
    K = torch.from_numpy(oracle.bf16_bits_to_f64(Kc)).repeat_interleave(4, 0)
    V = torch.from_numpy(oracle.bf16_bits_to_f64(Vc)).repeat_interleave(4, 0)
    ref = torch.nn.functional.scaled_dot_product_attention(Q, K, V, scale=float(p.scale))[:, 0].numpy()
    np.testing.assert_allclose(out[0], ref, atol=1e-12, rtol=0)


def test_nan_tails_and_spare_blocks_never_leak():
    p = _small([37, 100, 5, 1, 33])
    q, k, v = p.layer(0)
    # every unused slot is NaN, and the table padding points at a NaN block
    assert (p.block_fill < 16).any()
    out, lse, wr = _run(p)
    assert np.isfinite(out[wr]).all() and np.isfinite(lse[wr]).all()


def test_zombie_and_empty_slots_write_nothing():
    p = _small([37, 0, 100, 0, 5], [1, 1, 1, 0, 0])
    out, lse, wr = _run(p)
    # rows: r0 -> 0, r1 (zombie, keeps its row) -> 1, r2 -> 2; r3, r4 have none
    assert wr.tolist() == [True, False, True]
    assert np.isnan(out[1]).all() and np.isnan(lse[1]).all()
    assert np.isfinite(out[[0, 2]]).all()


def test_tiny_decode_layout():
    p = inputs.tiny_decode()
    assert p.num_blocks == 16 and p.block_table.shape == (2, 7)
    assert list(p.ctx_lens) == [37, 100]
    assert sorted(p.block_fill.tolist()) == [0] * 6 + [4, 5] + [16] * 8
    assert float(p.scale) == float(np.float32(1 / math.sqrt(128)))
    assert np.float32(p.scale).view(np.uint32) == 0x3DB504F3


def test_ragged_layout():
    p = inputs.ragged_mixed_decode()
    assert p.num_seqs == 68 and (p.ctx_lens == 0).sum() == 4
    assert p.ctx_lens.max() <= 8447 and p.ctx_lens[p.ctx_lens > 0].min() >= 1
    assert p.partition_size == 512 and p.block_table.shape == (68, 528)


# --------------------------------------------------------------------------
# split-KV partials and the log-sum-exp merge
# --------------------------------------------------------------------------

@pytest.mark.parametrize("S", [16, 64, 512])
def test_split_then_merge_equals_unsplit(S):
    p = _small([37, 100, 700, 16, 0], [1, 1, 1, 1, 1], hq=8, hkv=2, seed=13)
    q, k, v = p.layer(0)
    out, lse, wr = _run(p)
    P = -(-p.max_ctx_len // S)
    parts_o, parts_l = [], []
    for i in range(P):
        o, l, w = oracle.attend_key_range_fp64(q, k, v, p.block_table, p.ctx_lens, p.q_lens,
                                               p.scale, p.num_kv_heads, i * S, (i + 1) * S)
        parts_o.append(o.reshape(-1, 128))
        parts_l.append(l.reshape(-1))
    po = np.stack(parts_o)
    pl = np.stack(parts_l)
    mo, ml, touched = oracle.combine_fp64(po, pl)
    rows_written = np.repeat(wr, 8)
    assert np.array_equal(touched, rows_written)
    np.testing.assert_allclose(mo[touched], out.reshape(-1, 128)[touched], atol=1e-12, rtol=0)
    np.testing.assert_allclose(ml[touched], lse.reshape(-1)[touched], atol=1e-12, rtol=0)
    # ln sum_p exp(lse_p) over live partitions equals the unsplit lse
    for r in np.nonzero(touched)[0]:
        live = pl[:, r][np.isfinite(pl[:, r])]
        assert math.log(np.exp(live).sum()) == pytest.approx(lse.reshape(-1)[r], abs=1e-12)


def test_merge_all_empty_row_untouched_and_ignores_dead_outputs():
    po = np.full((3, 2, 4), np.nan)
    pl = np.full((3, 2), -np.inf)
    po[1, 1] = [1.0, 2.0, 3.0, 4.0]
    pl[1, 1] = 0.5
    out, lse, touched = oracle.combine_fp64(po, pl)
    assert touched.tolist() == [False, True]
    assert np.isnan(out[0]).all()
    np.testing.assert_array_equal(out[1], [1.0, 2.0, 3.0, 4.0])
    assert lse[1] == 0.5


def test_merge_two_equal_halves():
    # two partials of equal lse weigh 1/2 each and add ln 2
    po = np.array([[[1.0, 0.0]], [[0.0, 1.0]]])
    pl = np.array([[0.25], [0.25]])
    out, lse, _ = oracle.combine_fp64(po, pl)
    np.testing.assert_allclose(out[0], [0.5, 0.5], atol=1e-15)
    assert lse[0] == pytest.approx(0.25 + math.log(2), abs=1e-15)
