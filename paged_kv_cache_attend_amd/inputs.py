"""Seeded synthetic inputs for paged attention: page pools, block tables, lengths.

This module only *lays out and draws* inputs; it holds none of the attention
arithmetic.  Both the HIP path (through the tests and the benchmark) and the
FP64 oracle consume what it returns.

Structure follows the paged-allocation model of the inference-optimisation
page ("Chapter 8: Inference optimisation", sections 8.1.2, 8.3.1 and 8.3.2):
16-token blocks, a per-request block table whose entries may point anywhere
in the pool, shared-prefix blocks referenced by several tables, and unused
tail slots in each request's last block.  Finished ("zombie") slots of the
Photon pipelined-decoding page (section 5) appear as slots with no keys.

Conventions
-----------
* Values are drawn float32 N(0, 1) and rounded once to bf16
  (round-to-nearest-even); arrays hold the bf16 bit patterns as uint16.
* Every pool has spare blocks (at least one, about one per eight live
  blocks).  Spare blocks and the unused tail slots of partially filled blocks
  hold bf16 NaN (0x7FC0), and block-table columns past a request's last
  block point at a spare block, so that any read outside a request's keys
  would poison the result.
* Seeds: ``SeedSequence(seed)`` has ``1 + num_layers`` children; child 0
  draws the structure (placements, lengths, zombies), child ``1 + l`` draws
  layer l's values in the order q, K pool, V pool.  Large arrays are drawn in
  fixed-size chunks, each from its own spawned child, so the values do not
  depend on the number of threads.
"""

from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 20261202
BF16_NAN = np.uint16(0x7FC0)
_CHUNK = 1 << 22


def child_seed(ss: np.random.SeedSequence, i: int) -> np.random.SeedSequence:
    """The i-th child of ``ss``, derived without advancing ``ss`` (unlike
    ``SeedSequence.spawn``, which is stateful)."""
    return np.random.SeedSequence(ss.entropy, spawn_key=tuple(ss.spawn_key) + (int(i),),
                                  pool_size=ss.pool_size)


def _round_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest, ties to even (finite inputs)."""
    u = x.view(np.uint32)
    r = u >> np.uint32(16)
    r &= np.uint32(1)
    r += np.uint32(0x7FFF)
    r += u
    r >>= np.uint32(16)
    return r.astype(np.uint16)


def _draw_chunk(args):
    child, count = args
    rng = np.random.default_rng(child)
    return _round_bf16(rng.standard_normal(count, dtype=np.float32))


def normal_bf16(seed_seq: np.random.SeedSequence, shape, threads: int | None = None) -> np.ndarray:
    """N(0, 1) values rounded to bf16, deterministic for a given seed sequence."""
    total = int(np.prod(shape))
    nchunks = max(1, -(-total // _CHUNK))
    children = [child_seed(seed_seq, i) for i in range(nchunks)]
    counts = [min(_CHUNK, total - i * _CHUNK) for i in range(nchunks)]
    if threads is None:
        threads = min(16, len(os.sched_getaffinity(0)))
    out = np.empty(total, dtype=np.uint16)
    if nchunks == 1:
        out[:] = _draw_chunk((children[0], counts[0]))
    else:
        with ThreadPoolExecutor(max_workers=max(1, threads)) as ex:
            for i, part in enumerate(ex.map(_draw_chunk, zip(children, counts))):
                out[i * _CHUNK:i * _CHUNK + counts[i]] = part
    return out.reshape(shape)


def _blocks(n: int, bs: int) -> int:
    return -(-int(n) // bs)


@dataclass
class PagedProblem:
    """One paged-attention workload (all layers share the block table)."""

    name: str
    num_layers: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int
    block_table: np.ndarray          # int32 [num_seqs][max_blocks_per_seq]
    ctx_lens: np.ndarray             # int32 [num_seqs]
    q_lens: np.ndarray               # int32 [num_seqs]
    scale: np.float32
    block_fill: np.ndarray           # int32 [num_blocks]: valid slots per physical block
    partition_size: int = 0          # 0 = let the library choose
    causal: bool = False
    shared_prefix_blocks: int = 0
    _value_seeds: list = field(default_factory=list, repr=False)

    @property
    def num_seqs(self) -> int:
        return int(self.ctx_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.q_lens.sum())

    @property
    def max_q_len(self) -> int:
        return int(self.q_lens.max()) if self.num_seqs else 0

    @property
    def max_ctx_len(self) -> int:
        return int(self.ctx_lens.max()) if self.num_seqs else 0

    @property
    def max_blocks_per_seq(self) -> int:
        return int(self.block_table.shape[1])

    def active(self) -> np.ndarray:
        """Slots that have both keys and new tokens."""
        return (self.ctx_lens > 0) & (self.q_lens > 0)

    def kv_bytes_read(self) -> int:
        """K+V bytes a single pass over every active slot's keys must read
        (per layer), counting a shared block once per referencing request."""
        a = self.active()
        return int(self.ctx_lens[a].astype(np.int64).sum()) * self.num_kv_heads * self.head_dim * 2 * 2

    def kv_bytes_unique(self) -> int:
        """K+V bytes of distinct (physical block, slot) pairs the pass reads."""
        seen = set()
        slots = 0
        bs = self.block_size
        for r in np.nonzero(self.active())[0]:
            n = int(self.ctx_lens[r])
            for j in range(_blocks(n, bs)):
                phys = int(self.block_table[r, j])
                cnt = min(bs, n - j * bs)
                if phys in seen:
                    continue
                seen.add(phys)
                slots += cnt
        return slots * self.num_kv_heads * self.head_dim * 2 * 2

    def layer(self, l: int, threads: int | None = None):
        """(q, k_pool, v_pool) bf16 bit arrays of layer l."""
        if not 0 <= l < self.num_layers:
            raise IndexError(l)
        sq, sk, sv = (child_seed(self._value_seeds[l], i) for i in range(3))
        D = self.head_dim
        q = normal_bf16(sq, (self.total_q, self.num_q_heads, D), threads)
        shape = (self.num_blocks, self.num_kv_heads, self.block_size, D)
        k = normal_bf16(sk, shape, threads)
        v = normal_bf16(sv, shape, threads)
        self._poison(k)
        self._poison(v)
        return q, k, v

    def _poison(self, pool: np.ndarray) -> None:
        for phys in np.nonzero(self.block_fill < self.block_size)[0]:
            pool[phys, :, self.block_fill[phys]:, :] = BF16_NAN


# Quantised pages: random codes and scales drawn directly (not encoded from
# values), so a test of the decoding side does not depend on any encoder.
QUANT_FORMATS = ("fp8", "q8_0", "q4_0")
FP16_NAN = np.uint16(0x7E00)
E4M3_NAN = np.uint8(0x7F)


def quant_pages(problem: PagedProblem, fmt: str, layer: int = 0):
    """Random K and V pages of one layer in a quantised format.

    Returns (k_codes, v_codes, k_scales, v_scales, k_scale, v_scale):
    fp8 codes are uint8 E4M3 patterns (never NaN) with per-cache scales
    1/64 (K, values up to 7) and 1/256 (V, values up to 1.75, so outputs stay
    in the range the bf16 tolerances are derived for); q8_0 codes int8 in [-127, 127] with fp16 group scales in
    [0.004, 0.0157]; q4_0 packed nibbles with fp16 group scales of either sign,
    |scale| in [0.05, 0.25] -- every decoded value within +-2, like the bf16
    inputs.  Past each block's valid slots (and in spare
    blocks) FP8 codes are E4M3 NaN and group scales fp16 NaN: no kernel may
    read them.
    """
    if fmt not in QUANT_FORMATS:
        raise ValueError(fmt)
    ss = child_seed(np.random.SeedSequence(SEED_BASE + 4000 + QUANT_FORMATS.index(fmt)),
                    int(problem._value_seeds[layer].entropy % (1 << 31)) + layer)
    rng = np.random.default_rng(ss)
    nb, hkv, bs = problem.num_blocks, problem.num_kv_heads, problem.block_size
    out = []
    for _kv in range(2):
        if fmt == "fp8":
            c = rng.integers(0, 256, (nb, hkv, bs, 128), dtype=np.uint8)
            c[(c & 0x7F) == 0x7F] &= np.uint8(0xF7)          # no NaN codes in live slots
            sc = None
        elif fmt == "q8_0":
            c = rng.integers(-127, 128, (nb, hkv, bs, 128), dtype=np.int8)
            sc = rng.uniform(0.004, 0.0157, (nb, hkv, bs, 4)).astype(np.float16).view(np.uint16)
        else:
            c = rng.integers(0, 256, (nb, hkv, bs, 64), dtype=np.uint8)
            mag = rng.uniform(0.05, 0.25, (nb, hkv, bs, 4))
            sign = np.where(rng.integers(0, 2, (nb, hkv, bs, 4)) == 0, -1.0, 1.0)
            sc = (mag * sign).astype(np.float16).view(np.uint16)
        for phys in np.nonzero(problem.block_fill < bs)[0]:
            f = problem.block_fill[phys]
            if fmt == "fp8":
                c[phys, :, f:, :] = E4M3_NAN
            else:
                sc[phys, :, f:, :] = FP16_NAN
        out.append((c, sc))
    (kc, ks), (vc, vs) = out
    return kc, vc, ks, vs, 1.0 / 64, 1.0 / 256


def make_problem(name: str, seed: int, ctx_lens, q_lens, num_q_heads: int, num_kv_heads: int,
                 head_dim: int = 128, block_size: int = 16, num_layers: int = 1,
                 shared_prefix_tokens: int = 0, max_blocks_per_seq: int | None = None,
                 num_blocks: int | None = None, partition_size: int = 0,
                 scale=None, causal: bool = False, structure_rng=None,
                 seed_seq: np.random.SeedSequence | None = None) -> PagedProblem:
    """Lay out a paged pool for the given per-slot lengths.

    Live blocks (the shared prefix once, then each active slot's private
    blocks in slot order) and spare blocks are placed at one seeded random
    permutation of the whole pool.  ``shared_prefix_tokens`` (a multiple of
    the block size) are one physical copy referenced by every active slot.
    """
    ctx = np.asarray(ctx_lens, dtype=np.int32).copy()
    ql = np.asarray(q_lens, dtype=np.int32).copy()
    if ctx.shape != ql.shape:
        raise ValueError("ctx_lens and q_lens differ in length")
    bs = int(block_size)
    if shared_prefix_tokens % bs:
        raise ValueError("shared prefix must be whole blocks")
    ss = seed_seq if seed_seq is not None else np.random.SeedSequence(seed)
    children = [child_seed(ss, i) for i in range(1 + num_layers)]
    rng = structure_rng if structure_rng is not None else np.random.default_rng(children[0])

    shared = shared_prefix_tokens // bs
    need = [_blocks(n, bs) if n > 0 else 0 for n in ctx]
    for r, n in enumerate(ctx):
        if n > 0 and need[r] < shared:
            raise ValueError("an active slot is shorter than the shared prefix")
    private = [max(0, b - shared) if b > 0 else 0 for b in need]
    live = (shared if any(b > 0 for b in need) else 0) + sum(private)
    spare = max(1, -(-live // 8))
    pool = live + spare if num_blocks is None else int(num_blocks)
    if pool < live + 1:
        raise ValueError("pool too small")
    perm = rng.permutation(pool).astype(np.int32)
    shared_ids = perm[:shared]
    cursor = shared
    spare_ids = perm[live:]

    maxb = max(need) if max_blocks_per_seq is None else int(max_blocks_per_seq)
    maxb = max(maxb, 1)
    table = np.full((len(ctx), maxb), spare_ids[0], dtype=np.int32)
    fill = np.zeros(pool, dtype=np.int32)
    for r, n in enumerate(ctx):
        if need[r] == 0:
            continue
        ids = list(shared_ids) + list(perm[cursor:cursor + private[r]])
        cursor += private[r]
        table[r, :need[r]] = ids
        for j, phys in enumerate(ids):
            fill[phys] = min(bs, int(n) - j * bs)
    if scale is None:
        scale = np.float32(1.0) / np.sqrt(np.float32(head_dim))
    return PagedProblem(
        name=name, num_layers=num_layers, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=bs, num_blocks=pool, block_table=table,
        ctx_lens=ctx, q_lens=ql, scale=np.float32(scale), block_fill=fill,
        partition_size=partition_size, causal=causal, shared_prefix_blocks=shared,
        _value_seeds=list(children[1:]),
    )


def make_grouped_problem(name: str, seed: int, groups, singles, num_q_heads: int, num_kv_heads: int,
                         q_lens=None, num_layers: int = 1, block_size: int = 16):
    """Slots in groups that share a prefix, then slots in no group.

    ``groups`` is a list of (prefix_tokens, [ctx_len of each member]); the
    members are consecutive slots, and every member's table row starts with
    the group's shared blocks (one physical copy) -- also for members without
    new tokens.  ``singles`` are the ctx_lens of the slots after the groups.
    ``q_lens`` defaults to 1 for every slot with keys.  Placement is one
    seeded random permutation of live and spare blocks, as in make_problem.
    Returns (problem, group_start int32 [num_groups + 1], prefix_len int32
    [num_groups]).
    """
    bs = int(block_size)
    ctx = [n for _, members in groups for n in members] + list(singles)
    ql = np.asarray([1 if n > 0 else 0 for n in ctx] if q_lens is None else q_lens, dtype=np.int32)
    ctx = np.asarray(ctx, dtype=np.int32)
    ss = np.random.SeedSequence(seed)
    children = [child_seed(ss, i) for i in range(1 + num_layers)]
    rng = np.random.default_rng(children[0])
    # logical blocks: (owner list, fill) in order
    blocks = []
    rows = []              # per slot: list of logical block indices
    starts, plens = [0], []
    for prefix, members in groups:
        if prefix % bs:
            raise ValueError("prefix must be whole blocks")
        shared = list(range(len(blocks), len(blocks) + prefix // bs))
        blocks += [bs] * (prefix // bs)
        for n in members:
            if n > 0 and n < prefix:
                raise ValueError("a member is shorter than its prefix")
            own = []
            for t in range(prefix, max(int(n), prefix), bs):
                own.append(len(blocks))
                blocks.append(min(bs, int(n) - t))
            rows.append(shared + own)
        starts.append(starts[-1] + len(members))
        plens.append(prefix)
    for n in singles:
        own = []
        for t in range(0, int(n), bs):
            own.append(len(blocks))
            blocks.append(min(bs, int(n) - t))
        rows.append(own)
    live = len(blocks)
    spare = max(1, -(-live // 8))
    pool = live + spare
    perm = rng.permutation(pool).astype(np.int32)
    maxb = max([len(r) for r in rows] + [1])
    table = np.full((len(ctx), maxb), perm[live], dtype=np.int32)
    fill = np.zeros(pool, dtype=np.int32)
    for i, f in enumerate(blocks):
        fill[perm[i]] = f
    for r, lb in enumerate(rows):
        table[r, :len(lb)] = perm[lb]
    problem = PagedProblem(
        name=name, num_layers=num_layers, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=128, block_size=bs, num_blocks=pool, block_table=table, ctx_lens=ctx, q_lens=ql,
        scale=np.float32(1.0) / np.sqrt(np.float32(128)), block_fill=fill, _value_seeds=list(children[1:]))
    return problem, np.asarray(starts, dtype=np.int32), np.asarray(plens, dtype=np.int32)


# ---------------------------------------------------------------------------
# The five reference workloads.  Sizes restate the Qwen3-8B serving design of
# the inference-optimisation page (36 layers, 8 KV heads of 128, 2048- and
# 8192-token prompts with 256 outputs, a 6144-token shared prefix, 16-token
# blocks) and the chunk-versus-history attention of the PhysisServe page.
# ---------------------------------------------------------------------------

def tiny_decode() -> PagedProblem:
    """1 layer, 2 slots of 37 and 100 keys, 8 query / 2 KV heads, 16-block pool."""
    return make_problem("tiny_decode", SEED_BASE + 1, [37, 100], [1, 1], 8, 2,
                        num_blocks=16, max_blocks_per_seq=7)


def qwen3_short_decode(num_layers: int = 36) -> PagedProblem:
    """16 slots x 2303 keys (2048 prompt + 255 generated), 32/8 heads."""
    return make_problem("qwen3_8b_short_decode", SEED_BASE + 2, [2303] * 16, [1] * 16, 32, 8,
                        num_layers=num_layers)


def qwen3_shared_prefix_decode(num_layers: int = 36) -> PagedProblem:
    """10 slots x 8447 keys; the first 6144 (384 blocks) are one shared copy."""
    return make_problem("qwen3_8b_shared_prefix_decode", SEED_BASE + 3, [8447] * 10, [1] * 10, 32, 8,
                        num_layers=num_layers, shared_prefix_tokens=6144)


def ragged_mixed_decode() -> PagedProblem:
    """68 slots: 4 zombies (no keys) and 64 with lengths uniform on [1, 8447];
    split over 512-token partitions."""
    ss = np.random.SeedSequence(SEED_BASE + 4)
    children = [child_seed(ss, i) for i in range(2)]
    rng = np.random.default_rng(children[0])
    zombies = rng.choice(68, 4, replace=False)
    lens = rng.integers(1, 8448, size=68).astype(np.int32)
    lens[zombies] = 0
    return make_problem("ragged_mixed_decode", SEED_BASE + 4, lens, [1] * 68, 32, 8,
                        max_blocks_per_seq=528, partition_size=512, structure_rng=rng,
                        seed_seq=children[1])


def chunked_denoise() -> PagedProblem:
    """4 streams, 24 heads (MHA), a 256-token chunk over 3 earlier chunks
    (768 cached tokens) plus itself: 1024 keys, full mask."""
    return make_problem("chunked_denoise", SEED_BASE + 5, [1024] * 4, [256] * 4, 24, 24)


def chunked_prefill(num_seqs: int = 1) -> PagedProblem:
    """The last 512-token chunk of an 8192-token prompt (7680 tokens already
    cached), Qwen3-8B heads (32 query / 8 KV), causal: the chunked-prefill
    example of the inference-optimisation chapter (section 8.2.3), whose last
    chunk covers 512 x 7680 + 512 x 513 / 2 = 4,063,488 query-key pairs."""
    return make_problem("chunked_prefill_c512_h7680", SEED_BASE + 6, [8192] * num_seqs, [512] * num_seqs,
                        32, 8, causal=True)


def speculative_verify(num_tokens: int = 8) -> PagedProblem:
    """Verification of `num_tokens` proposed tokens per request at once
    (section 8.5 of the same chapter: a draft proposes several tokens, the
    target model checks them in one step): the Qwen3-8B short decode batch
    (16 requests, 2303 keys each including the new tokens, 32/8 heads),
    causal over the new tokens."""
    return make_problem(f"speculative_verify_m{num_tokens}", SEED_BASE + 7 + num_tokens, [2303] * 16,
                        [num_tokens] * 16, 32, 8, causal=True)


CONFIGS = {
    "tiny_decode": tiny_decode,
    "qwen3_8b_short_decode": qwen3_short_decode,
    "qwen3_8b_shared_prefix_decode": qwen3_shared_prefix_decode,
    "ragged_mixed_decode": ragged_mixed_decode,
    "chunked_denoise": chunked_denoise,
}


def fig_8_10_case(num_q_heads: int = 8, num_kv_heads: int = 2, head_dim: int = 128) -> PagedProblem:
    """Fig. 8-10 of the paging section: logical blocks 0, 1, 2 of one request
    sit in physical blocks 2, 0, 3 of a 4-block pool; block 1 is free (NaN)."""
    bs = 16
    n = 3 * bs
    table = np.array([[2, 0, 3]], dtype=np.int32)
    fill = np.array([bs, 0, bs, bs], dtype=np.int32)
    ss = np.random.SeedSequence(SEED_BASE + 810)
    children = [child_seed(ss, i) for i in range(2)]
    return PagedProblem(
        name="fig_8_10", num_layers=1, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads,
        head_dim=head_dim, block_size=bs, num_blocks=4, block_table=table,
        ctx_lens=np.array([n], dtype=np.int32), q_lens=np.array([1], dtype=np.int32),
        scale=np.float32(1.0) / np.sqrt(np.float32(head_dim)), block_fill=fill,
        _value_seeds=[children[1]],
    )


def worked_example_9_13_5_15(num_q_heads: int = 8, num_kv_heads: int = 2) -> PagedProblem:
    """The four requests of the paging worked example (9, 13, 5 and 15
    tokens), here with 16-token blocks, one new token each."""
    return make_problem("worked_9_13_5_15", SEED_BASE + 913, [9, 13, 5, 15], [1, 1, 1, 1],
                        num_q_heads, num_kv_heads)


def with_block_table(problem: PagedProblem, table: np.ndarray, fill: np.ndarray,
                     num_blocks: int | None = None) -> PagedProblem:
    """Same values seeds and lengths, different physical placement."""
    import copy
    p = copy.copy(problem)
    p.block_table = np.asarray(table, dtype=np.int32)
    p.block_fill = np.asarray(fill, dtype=np.int32)
    if num_blocks is not None:
        p.num_blocks = int(num_blocks)
    return p


def relocate(problem: PagedProblem, layer: int, seed: int):
    """Move every physical block of ``problem`` to a new seeded position.

    Returns (table, k, v) for ``layer`` where block ``b`` of the original
    pool now lives at ``perm[b]``: the logical content of every request is
    unchanged, only its placement differs.
    """
    q, k, v = problem.layer(layer)
    perm = np.random.default_rng(seed).permutation(problem.num_blocks).astype(np.int32)
    k2 = np.empty_like(k)
    v2 = np.empty_like(v)
    k2[perm] = k
    v2[perm] = v
    table2 = perm[problem.block_table]
    return q, table2, k2, v2


# ---------------------------------------------------------------------------
# Host-side precondition check and upload (harness plumbing).
# ---------------------------------------------------------------------------

def check_preconditions(problem: PagedProblem, table=None) -> None:
    """Raise if the problem breaks a device-side precondition of pa_attend
    (so that no kernel is ever launched on out-of-range data)."""
    t = problem.block_table if table is None else np.asarray(table)
    bs = problem.block_size
    if (problem.ctx_lens < 0).any() or (problem.q_lens < 0).any():
        raise ValueError("negative length")
    if int(problem.ctx_lens.max(initial=0)) > bs * t.shape[1]:
        raise ValueError("ctx_len beyond the block table")
    if int(problem.q_lens.sum()) != problem.total_q:
        raise ValueError("q_lens do not sum to total_q")
    live = (problem.ctx_lens > 0)
    if ((problem.q_lens > problem.ctx_lens) & live).any():
        raise ValueError("more new rows than keys")
    for r in np.nonzero(live)[0]:
        ids = t[r, :_blocks(int(problem.ctx_lens[r]), bs)]
        if (ids < 0).any() or (ids >= problem.num_blocks).any():
            raise ValueError(f"slot {r}: block id outside the pool")


def bits_to_torch_bf16(bits: np.ndarray, device):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_device(problem: PagedProblem, q, k, v, device, table=None):
    """Upload one layer's arrays plus the shared index arrays as torch tensors."""
    import torch
    check_preconditions(problem, table)
    t = problem.block_table if table is None else table
    return dict(
        q=bits_to_torch_bf16(q, device),
        k=bits_to_torch_bf16(k, device),
        v=bits_to_torch_bf16(v, device),
        block_table=torch.from_numpy(np.ascontiguousarray(t, dtype=np.int32)).to(device),
        ctx_lens=torch.from_numpy(problem.ctx_lens.astype(np.int32)).to(device),
        q_lens=torch.from_numpy(problem.q_lens.astype(np.int32)).to(device),
    )
