"""C-ABI checks that need no GPU: the library loads, exports what include/pa.h
declares, and rejects bad arguments on the host before launching anything."""

from __future__ import annotations

import ctypes
import math
import os
import re
import subprocess

import pytest

import paged_kv_cache_attend_amd as pk
from paged_kv_cache_attend_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(os.path.join(ROOT, "include", f) for f in os.listdir(os.path.join(ROOT, "include"))
                 if f.endswith(".h"))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(_lib.lib_path()):
        from paged_kv_cache_attend_amd import build
        build.build()
    return pk.load()


def _declared():
    text = "\n".join(open(h).read() for h in HEADERS)
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_binding_names():
    assert _declared() == sorted(_lib.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", _lib.lib_path()], capture_output=True, text=True,
                         check=True).stdout
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    for name in _declared():
        assert name in exported, name
        assert getattr(lib, name) is not None


def test_shape_struct_layout():
    # int32 x 10, int64, uint32 x 2 -> 10*4 + 8 + 8 = 56 bytes, int64 at offset 40
    assert ctypes.sizeof(pk.Shape) == 56
    assert pk.Shape.num_blocks.offset == 40


def _align(x):
    return (x + 255) // 256 * 256


def _ws_bytes(num_seqs, hkv, parts, rows):
    """counters | partial LSE | partial out, each region 256-byte aligned."""
    return _align(num_seqs * hkv * 4) + _align(parts * rows * 4) + parts * rows * 128 * 4


def _shape(**kw):
    base = dict(num_seqs=4, total_q=4, num_q_heads=32, num_kv_heads=8, max_blocks_per_seq=10,
                max_q_len=1, max_ctx_len=160, num_blocks=64)
    base.update(kw)
    return pk.make_shape(**base)


FAKE = ctypes.c_void_p(0x1000)  # never dereferenced: every case below fails on the host


def _attend(lib, shape, scale=0.088, ws=None, ws_bytes=0, q=FAKE, out=FAKE, null_shape=False):
    sp = None if null_shape else ctypes.byref(shape)
    return lib.pa_attend(sp, q, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(scale), out, None, ws,
                         ctypes.c_size_t(ws_bytes), None)


def test_status_strings(lib):
    for s in pk.Status:
        assert pk.status_string(s)
    assert pk.status_string(99) == "unknown status"


@pytest.mark.parametrize("kw,expected", [
    (dict(num_q_heads=30), pk.Status.ERR_BAD_SHAPE),       # not a multiple of Hkv
    (dict(head_dim=64), pk.Status.ERR_UNSUPPORTED),
    (dict(block_size=32), pk.Status.ERR_UNSUPPORTED),
    (dict(partition_size=24), pk.Status.ERR_BAD_SHAPE),    # not whole blocks
    (dict(partition_size=-16), pk.Status.ERR_BAD_SHAPE),
    (dict(max_ctx_len=161), pk.Status.ERR_BAD_SHAPE),      # beyond 16 * max_blocks
    (dict(num_seqs=-1), pk.Status.ERR_BAD_SHAPE),
    (dict(num_kv_heads=0), pk.Status.ERR_BAD_SHAPE),
    (dict(max_q_len=5), pk.Status.ERR_BAD_SHAPE),          # above total_q
    (dict(num_blocks=0), pk.Status.ERR_BAD_SHAPE),
    (dict(flags=0x100), pk.Status.ERR_UNSUPPORTED),
])
def test_bad_shapes_rejected(lib, kw, expected):
    s = _shape(**kw)
    assert _attend(lib, s) == expected
    assert lib.pa_workspace_size(ctypes.byref(s)) == 0
    assert lib.pa_num_partitions(ctypes.byref(s)) == 0


def test_reserved_field_must_be_zero(lib):
    s = _shape()
    s.reserved = 1
    assert _attend(lib, s) == pk.Status.ERR_BAD_SHAPE


def test_null_arguments(lib):
    s = _shape()
    assert _attend(lib, s, null_shape=True) == pk.Status.ERR_NULL_ARG
    assert _attend(lib, s, q=None) == pk.Status.ERR_NULL_ARG
    assert _attend(lib, s, out=None) == pk.Status.ERR_NULL_ARG


def test_non_finite_scale(lib):
    s = _shape()
    assert _attend(lib, s, scale=math.nan) == pk.Status.ERR_BAD_SHAPE
    assert _attend(lib, s, scale=math.inf) == pk.Status.ERR_BAD_SHAPE


def test_workspace_checks(lib):
    s = _shape(num_seqs=68, total_q=68, max_blocks_per_seq=528, max_ctx_len=8447, num_blocks=20000,
               partition_size=512)
    need, parts = pk.plan(s)
    assert parts == 17
    rows = 68 * 32
    assert need == _ws_bytes(68, 8, parts, rows)
    assert need - _align(68 * 8 * 4) - (_align(parts * rows * 4) - parts * rows * 4) == 19_087_872
    assert _attend(lib, s, ws=None, ws_bytes=0) == pk.Status.ERR_NULL_ARG
    assert _attend(lib, s, ws=FAKE, ws_bytes=need - 1) == pk.Status.ERR_WORKSPACE_TOO_SMALL


def test_single_partition_needs_no_workspace(lib):
    s = _shape(partition_size=160)
    assert pk.plan(s) == (0, 1)


def test_auto_partitions_cover_the_chip(lib):
    # 16 slots x 8 KV heads x 2303 keys: two 72-page partitions per pair fill
    # the 256 CUs exactly once (four 36-page ones would too, with more fixed
    # cost per page).
    s = _shape(num_seqs=16, total_q=16, max_blocks_per_seq=144, max_ctx_len=2303, num_blocks=2592)
    ws, parts = pk.plan(s)
    assert parts == 2
    # q8_0 / q4_0 pages prefer the four-way split, FP8 the bf16 one; the
    # workspace covers both
    lib = pk.load()
    assert lib.pa_num_partitions_kv(ctypes.byref(s), pk.KV_BF16) == 2
    assert lib.pa_num_partitions_kv(ctypes.byref(s), pk.KV_FP8_E4M3) == 2
    for fmt in (pk.KV_Q8_0, pk.KV_Q4_0):
        assert lib.pa_num_partitions_kv(ctypes.byref(s), fmt) == 4
    assert lib.pa_num_partitions_kv(ctypes.byref(s), 9) == 0
    assert ws == _ws_bytes(16, 8, 4, 16 * 32)


@pytest.mark.parametrize("num_seqs,ctx,parts", [
    (10, 8447, 3),    # 80 pairs: 240 workgroups of 176 pages (6 x 88 fills the CUs as well: fewer wins)
    (10, 2303, 3),    # 80 pairs: 240 workgroups of 48 pages rather than 480 of 24
    (68, 8355, 5),    # 544 pairs, more than resident: long contexts cut to <= 128 pages
    (1, 32768, 32),   # one request: 32 x 64 pages, one workgroup per CU
    (2, 100, 1),      # 7 pages: never below 8 pages per partition
])
def test_auto_partition_counts(lib, num_seqs, ctx, parts):
    mb = (ctx + 15) // 16
    s = _shape(num_seqs=num_seqs, total_q=num_seqs, max_blocks_per_seq=mb, max_ctx_len=ctx,
               num_blocks=mb * num_seqs)
    assert pk.plan(s)[1] == parts


def test_chunk_path_needs_no_workspace(lib):
    s = _shape(num_seqs=4, total_q=1024, num_q_heads=24, num_kv_heads=24, max_blocks_per_seq=64,
               max_q_len=256, max_ctx_len=1024, num_blocks=288)
    assert pk.plan(s) == (0, 1)


def test_empty_batches_launch_nothing(lib):
    # nothing to write: returns OK without touching the (fake) pointers
    for kw in (dict(num_seqs=0), dict(total_q=0, max_q_len=0), dict(max_ctx_len=0), dict(max_q_len=0)):
        s = _shape(**kw)
        assert _attend(lib, s) == pk.Status.OK, kw


def test_combine_argument_checks(lib):
    f = lib.pa_combine
    assert f(0, 4, 128, FAKE, FAKE, FAKE, None, None) == pk.Status.ERR_BAD_SHAPE
    assert f(2, -1, 128, FAKE, FAKE, FAKE, None, None) == pk.Status.ERR_BAD_SHAPE
    assert f(2, 4, 126, FAKE, FAKE, FAKE, None, None) == pk.Status.ERR_BAD_SHAPE
    assert f(2, 4, 2048, FAKE, FAKE, FAKE, None, None) == pk.Status.ERR_BAD_SHAPE
    assert f(2, 4, 128, None, FAKE, FAKE, None, None) == pk.Status.ERR_NULL_ARG
    assert f(2, 4, 128, FAKE, FAKE, None, None, None) == pk.Status.ERR_NULL_ARG
    assert f(2, 0, 128, None, None, None, None, None) == pk.Status.OK


def test_workspace_init_argument_checks(lib):
    s = _shape(partition_size=32)
    need, parts = pk.plan(s)
    assert parts == 5 and need > 0
    assert lib.pa_workspace_init(ctypes.byref(s), None, need, None) == pk.Status.ERR_NULL_ARG
    assert lib.pa_workspace_init(ctypes.byref(s), FAKE, need - 1, None) == pk.Status.ERR_WORKSPACE_TOO_SMALL
    one = _shape(partition_size=160)
    assert lib.pa_workspace_init(ctypes.byref(one), None, 0, None) == pk.Status.OK  # nothing to prepare
    bad = _shape(head_dim=64)
    assert lib.pa_workspace_init(ctypes.byref(bad), FAKE, need, None) == pk.Status.ERR_UNSUPPORTED


def test_gather_and_validate_argument_checks(lib):
    s = _shape()
    assert lib.pa_gather_kv(ctypes.byref(s), None, FAKE, FAKE, FAKE, None) == pk.Status.ERR_NULL_ARG
    assert lib.pa_gather_kv(None, FAKE, FAKE, FAKE, FAKE, None) == pk.Status.ERR_NULL_ARG
    assert lib.pa_validate(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, None, None) == pk.Status.ERR_NULL_ARG
    bad = _shape(head_dim=96)
    assert lib.pa_gather_kv(ctypes.byref(bad), FAKE, FAKE, FAKE, FAKE, None) == pk.Status.ERR_UNSUPPORTED


def test_validate_workspace_counter_region_checked_on_host(lib):
    # 4 slots x 8 KV heads with a split: 32 counters (128 bytes) at the
    # workspace start.  A workspace too small for them is rejected before any
    # launch; NULL skips the counter check (and, here, fails on the NULL word).
    s = _shape(max_ctx_len=160, partition_size=16)
    assert pk.workspace_size(s) > 0
    assert lib.pa_validate(ctypes.byref(s), FAKE, FAKE, FAKE, FAKE, 127, FAKE, None) \
        == pk.Status.ERR_WORKSPACE_TOO_SMALL
    assert lib.pa_validate(ctypes.byref(s), FAKE, FAKE, FAKE, None, 0, None, None) == pk.Status.ERR_NULL_ARG
    assert _lib.PA_BAD_WORKSPACE == 0x10


def test_measure_entry_points_check_arguments_on_the_host(lib):
    assert lib.pa_measure_read_tiles(FAKE, FAKE, FAKE, -1, 4, FAKE, None) == pk.Status.ERR_BAD_SHAPE
    assert lib.pa_measure_read_tiles(FAKE, FAKE, FAKE, 10, 0, FAKE, None) == pk.Status.ERR_BAD_SHAPE
    assert lib.pa_measure_read_tiles(None, FAKE, FAKE, 10, 4, FAKE, None) == pk.Status.ERR_NULL_ARG
    assert lib.pa_measure_read_tiles(FAKE, FAKE, FAKE, 0, 4, FAKE, None) == pk.Status.OK  # nothing to do
    assert lib.pa_measure_mfma_bf16(0, 10, FAKE, None) == pk.Status.ERR_BAD_SHAPE
    assert lib.pa_measure_mfma_bf16(4, 0, FAKE, None) == pk.Status.ERR_BAD_SHAPE
    assert lib.pa_measure_mfma_bf16(4, 10, None, None) == pk.Status.ERR_NULL_ARG


def test_binding_fails_loudly_without_library(monkeypatch, tmp_path):
    monkeypatch.setattr(_lib, "_lib", None)
    monkeypatch.setattr(_lib, "_LIB_PATH", str(tmp_path / "missing.so"))
    with pytest.raises(RuntimeError, match="not built"):
        _lib.load()


def test_single_hip_runtime_in_process():
    # libpa.so must share torch's HIP runtime even when the library is loaded
    # before anything else imports torch (two runtimes break stream handles).
    code = ("import paged_kv_cache_attend_amd as pk; pk.load(); import torch; "
            "paths = {l.split()[-1] for l in open('/proc/self/maps') if 'libamdhip64' in l}; "
            "print(len(paths))")
    out = subprocess.run(["python", "-c", code], capture_output=True, text=True, cwd=ROOT, check=True).stdout
    assert out.strip() == "1"


def test_write_kv_and_copy_blocks_host_errors(lib):
    s = _shape()
    args = [FAKE] * 8
    assert lib.pa_write_kv(None, *args[:7], None) == pk.Status.ERR_NULL_ARG
    for i in range(7):
        a = list(args[:7])
        a[i] = None
        assert lib.pa_write_kv(ctypes.byref(s), *a, None) == pk.Status.ERR_NULL_ARG, i
    bad = _shape(head_dim=64)
    assert lib.pa_write_kv(ctypes.byref(bad), *args[:7], None) == pk.Status.ERR_UNSUPPORTED
    empty = _shape(num_seqs=0)
    assert lib.pa_write_kv(ctypes.byref(empty), *args[:7], None) == pk.Status.OK
    assert lib.pa_copy_blocks(-1, FAKE, FAKE, 8, 64, FAKE, FAKE, None) == pk.Status.ERR_BAD_SHAPE
    assert lib.pa_copy_blocks(1, FAKE, FAKE, 0, 64, FAKE, FAKE, None) == pk.Status.ERR_BAD_SHAPE
    assert lib.pa_copy_blocks(1, None, FAKE, 8, 64, FAKE, FAKE, None) == pk.Status.ERR_NULL_ARG
    assert lib.pa_copy_blocks(0, None, None, 8, 64, None, None, None) == pk.Status.OK


def test_pool_null_handles(lib):
    st = pk.PoolStats()
    i = ctypes.c_int32()
    assert lib.pa_pool_create(4, 16, 1, 1, None) == pk.Status.ERR_NULL_ARG
    assert lib.pa_pool_append(None, 0, 1, ctypes.byref(i), ctypes.byref(i), ctypes.byref(i)) == pk.Status.ERR_NULL_ARG
    assert lib.pa_pool_fork(None, 0, 1, -1) == pk.Status.ERR_NULL_ARG
    assert lib.pa_pool_release(None, 0, 0) == pk.Status.ERR_NULL_ARG
    assert lib.pa_pool_retire(None, 0) == pk.Status.ERR_NULL_ARG
    assert lib.pa_pool_get_stats(None, ctypes.byref(st)) == pk.Status.ERR_NULL_ARG
    lib.pa_pool_destroy(None)


def _kv(fmt, scales=True, k_scale=1.0, v_scale=1.0, reserved=0):
    s = FAKE.value if scales else None
    return pk.KVCache(fmt, reserved, FAKE.value, FAKE.value, s, s, k_scale, v_scale)


def test_attend_kv_host_errors(lib):
    s = _shape()
    args = (FAKE, FAKE, FAKE, FAKE, ctypes.c_float(0.1), FAKE, None, FAKE, ctypes.c_size_t(1 << 30), None)
    f = lib.pa_attend_kv
    assert f(ctypes.byref(s), None, *args) == pk.Status.ERR_NULL_ARG
    assert f(ctypes.byref(s), ctypes.byref(_kv(7)), *args) == pk.Status.ERR_BAD_SHAPE
    assert f(ctypes.byref(s), ctypes.byref(_kv(pk.KV_Q8_0, reserved=1)), *args) == pk.Status.ERR_BAD_SHAPE
    for ks in (0.0, -1.0, math.inf, math.nan):
        assert f(ctypes.byref(s), ctypes.byref(_kv(pk.KV_FP8_E4M3, k_scale=ks)), *args) == pk.Status.ERR_BAD_SHAPE
    for fmt in (pk.KV_Q8_0, pk.KV_Q4_0):
        assert f(ctypes.byref(s), ctypes.byref(_kv(fmt, scales=False)), *args) == pk.Status.ERR_NULL_ARG
    # quantised pages take the decode path only
    chunk = _shape(total_q=8, max_q_len=2)
    assert f(ctypes.byref(chunk), ctypes.byref(_kv(pk.KV_Q8_0)), *args) == pk.Status.ERR_UNSUPPORTED
    # a bad shape is reported as for pa_attend
    assert f(ctypes.byref(_shape(head_dim=64)), ctypes.byref(_kv(pk.KV_Q8_0)), *args) == pk.Status.ERR_UNSUPPORTED


def test_write_kv_cache_host_errors(lib):
    s = _shape()
    args = (FAKE, FAKE, FAKE, FAKE, FAKE, None)
    f = lib.pa_write_kv_cache
    assert f(ctypes.byref(s), None, *args) == pk.Status.ERR_NULL_ARG
    assert f(ctypes.byref(s), ctypes.byref(_kv(4)), *args) == pk.Status.ERR_BAD_SHAPE
    assert f(ctypes.byref(s), ctypes.byref(_kv(pk.KV_Q4_0, scales=False)), *args) == pk.Status.ERR_NULL_ARG
    assert f(ctypes.byref(s), ctypes.byref(_kv(pk.KV_FP8_E4M3, v_scale=0.0)), *args) == pk.Status.ERR_BAD_SHAPE
    assert f(ctypes.byref(s), ctypes.byref(_kv(pk.KV_Q8_0)), None, FAKE, FAKE, FAKE, FAKE, None) == \
        pk.Status.ERR_NULL_ARG
    empty = _shape(num_seqs=0)
    assert f(ctypes.byref(empty), ctypes.byref(_kv(pk.KV_Q8_0)), *args) == pk.Status.OK


def test_kv_cache_struct_layout():
    # int32 x 2, four pointers, two floats: 8 + 32 + 8 = 48 bytes
    assert ctypes.sizeof(pk.KVCache) == 48
    assert pk.KVCache.k_codes.offset == 8 and pk.KVCache.k_scale.offset == 40


def _groups(num_groups=1, max_members=4, max_prefix_len=64, min_prefix_len=0, reserved=0, ptrs=True):
    p = FAKE.value if ptrs else None
    return pk.PrefixGroups(num_groups, max_members, max_prefix_len, min_prefix_len, reserved, 0, p, p)


def test_prefix_groups_struct_layout():
    # int32 x 6, two pointers: 24 + 16 = 40 bytes
    assert ctypes.sizeof(pk.PrefixGroups) == 40
    assert pk.PrefixGroups.group_start.offset == 24 and pk.PrefixGroups.prefix_len.offset == 32


def test_prefix_workspace_size(lib):
    size = lambda s, g: lib.pa_prefix_workspace_size(ctypes.byref(s), ctypes.byref(g))
    s = _shape()
    ws = size(s, _groups())
    # suffix workspace | slot prefix lengths | prefix LSEs | prefix partials: 4 slots x 32 heads = 128
    # rows, one group of 4 x 4 rows on 8 KV heads with 4 prefix pages -> 2 prefix partitions
    suffix = size(s, _groups(num_groups=0, max_members=0, max_prefix_len=0))
    assert suffix > 0
    base = suffix - (_align(4 * 4) + _align(1 * 128 * 4) + 1 * 128 * 128 * 4)
    assert base >= 0 and base % 256 == 0   # 10 pages: one suffix partition, no suffix workspace
    assert ws == base + _align(4 * 4) + _align(2 * 128 * 4) + 2 * 128 * 128 * 4
    for bad in (_groups(reserved=1), _groups(max_prefix_len=40), _groups(min_prefix_len=80),
                _groups(max_prefix_len=176), _groups(max_members=5), _groups(num_groups=5),
                _groups(num_groups=-1), _groups(min_prefix_len=-16)):
        assert size(s, bad) == 0
    assert lib.pa_prefix_workspace_size(ctypes.byref(s), None) == 0
    assert size(_shape(num_q_heads=128), _groups()) == 0      # 16 query heads per KV head
    assert size(_shape(total_q=8, max_q_len=2), _groups()) == 0


def test_attend_prefix_host_errors(lib):
    s = _shape()
    g = _groups()
    need = lib.pa_prefix_workspace_size(ctypes.byref(s), ctypes.byref(g))
    f = lib.pa_attend_prefix

    def call(shape=s, groups=g, scale=0.088, ws=FAKE, ws_bytes=need, q=FAKE):
        gp = None if groups is None else ctypes.byref(groups)
        return f(ctypes.byref(shape), gp, q, FAKE, FAKE, FAKE, FAKE, FAKE, ctypes.c_float(scale), FAKE, None, ws,
                 ctypes.c_size_t(ws_bytes), None)

    assert call(groups=None) == pk.Status.ERR_NULL_ARG
    assert call(groups=_groups(ptrs=False)) == pk.Status.ERR_NULL_ARG
    assert call(q=None) == pk.Status.ERR_NULL_ARG
    assert call(ws=None) == pk.Status.ERR_NULL_ARG
    assert call(ws_bytes=need - 1) == pk.Status.ERR_WORKSPACE_TOO_SMALL
    assert call(scale=math.nan) == pk.Status.ERR_BAD_SHAPE
    assert call(groups=_groups(reserved=1)) == pk.Status.ERR_BAD_SHAPE
    assert call(groups=_groups(max_prefix_len=24)) == pk.Status.ERR_BAD_SHAPE
    assert call(shape=_shape(num_q_heads=128)) == pk.Status.ERR_UNSUPPORTED
    assert call(shape=_shape(total_q=8, max_q_len=2)) == pk.Status.ERR_UNSUPPORTED
    empty = _shape(num_seqs=0, total_q=0)
    assert call(shape=empty, groups=_groups(num_groups=0, max_members=0), ws=None, ws_bytes=0) == pk.Status.OK
    init = lib.pa_prefix_workspace_init
    assert init(ctypes.byref(s), ctypes.byref(g), None, ctypes.c_size_t(need), None) == pk.Status.ERR_NULL_ARG
    assert init(ctypes.byref(s), ctypes.byref(g), FAKE, ctypes.c_size_t(need - 1), None) == \
        pk.Status.ERR_WORKSPACE_TOO_SMALL


def test_prefix_partition_plan():
    # The prefix pass splits the longest prefix into partitions of at most
    # eight 32-key tiles (16 pages), more when CUs would sit idle (up to 24
    # per (group, KV head, row tile)), never under one tile: read back from
    # the workspace size, whose last region holds one fp32 partial per
    # partition and row.
    lib = pk.load()
    s = _shape(num_seqs=10, total_q=10, max_blocks_per_seq=528, max_ctx_len=8447, num_blocks=6000)
    rows = 10 * 32
    size = lambda g: lib.pa_prefix_workspace_size(ctypes.byref(s), ctypes.byref(g))
    none = size(_groups(num_groups=0, max_members=0, max_prefix_len=0))
    base = none - (_align(10 * 4) + _align(rows * 4) + rows * 128 * 4)

    def parts(max_prefix_len):
        ws = size(_groups(num_groups=1, max_members=10, max_prefix_len=max_prefix_len))
        for p in range(1, 200):
            if ws == base + _align(10 * 4) + _align(p * rows * 4) + p * rows * 128 * 4:
                return p
        raise AssertionError(f"workspace {ws} matches no partition count")

    assert parts(6144) == 24    # 384 pages: 24 partitions of 16 (one group x 8 KV heads = 8 of 256 CUs each)
    assert parts(8192) == 32    # 512 pages: 16 pages per partition at most
    assert parts(64) == 2       # 4 pages: one 32-key tile each
    assert parts(16) == 1
