"""ctypes binding over libpa.so, with the names of the C ABI in include/pa.h.

Argument marshalling only: tensors are checked for dtype, device, layout and
size, then their device pointers and the current HIP stream are passed to the
library.  Every step of the computation runs in the library's HIP kernels.
If libpa.so has not been built, loading raises -- there is no other path.
"""

from __future__ import annotations

import ctypes
import enum
import os

PKG = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(PKG, "libpa.so")
_lib = None

PA_FLAG_CAUSAL = 0x1
PA_BAD_BLOCK_ID = 0x1
PA_BAD_CTX_LEN = 0x2
PA_BAD_Q_LEN = 0x4
PA_BAD_TOTAL_Q = 0x8
PA_BAD_WORKSPACE = 0x10

EXPORTS = ("pa_workspace_size", "pa_workspace_init", "pa_num_partitions", "pa_attend", "pa_combine",
           "pa_gather_kv", "pa_validate", "pa_write_kv", "pa_copy_blocks", "pa_pool_create",
           "pa_pool_destroy", "pa_pool_append", "pa_pool_fork", "pa_pool_release", "pa_pool_retire",
           "pa_pool_length", "pa_pool_block_table", "pa_pool_refcount", "pa_pool_get_stats",
           "pa_attend_kv", "pa_write_kv_cache", "pa_num_partitions_kv", "pa_prefix_workspace_size",
           "pa_prefix_workspace_init", "pa_attend_prefix", "pa_attend_noalloc", "pa_status_string",
           "pa_measure_read_tiles", "pa_measure_mfma_bf16")

NOALLOC_SCRATCH_BYTES = 32 << 20   # PA_NOALLOC_SCRATCH_BYTES

# pa_kv_format
KV_BF16 = 0
KV_FP8_E4M3 = 1
KV_Q8_0 = 2
KV_Q4_0 = 3


class Status(enum.IntEnum):
    OK = 0
    ERR_NULL_ARG = 1
    ERR_BAD_SHAPE = 2
    ERR_UNSUPPORTED = 3
    ERR_WORKSPACE_TOO_SMALL = 4
    ERR_LAUNCH = 5
    ERR_OUT_OF_BLOCKS = 6
    ERR_SCRATCH_LIMIT = 7


class PaError(RuntimeError):
    def __init__(self, status, where: str = ""):
        self.status = Status(status) if status in Status._value2member_map_ else status
        msg = status_string(status) if _lib is not None else str(status)
        super().__init__(f"{where}: {msg} ({self.status!r})" if where else msg)


class PoolStats(ctypes.Structure):
    """Mirror of ``pa_pool_stats``."""

    _fields_ = [
        ("free_blocks", ctypes.c_int32),
        ("pending_blocks", ctypes.c_int32),
        ("used_blocks", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("references", ctypes.c_int64),
    ]


class PrefixGroups(ctypes.Structure):
    """Mirror of ``pa_prefix_groups``."""

    _fields_ = [
        ("num_groups", ctypes.c_int32),
        ("max_members", ctypes.c_int32),
        ("max_prefix_len", ctypes.c_int32),
        ("min_prefix_len", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("reserved2", ctypes.c_int32),
        ("group_start", ctypes.c_void_p),
        ("prefix_len", ctypes.c_void_p),
    ]


class KVCache(ctypes.Structure):
    """Mirror of ``pa_kv_cache``."""

    _fields_ = [
        ("format", ctypes.c_int32),
        ("reserved", ctypes.c_int32),
        ("k_codes", ctypes.c_void_p),
        ("v_codes", ctypes.c_void_p),
        ("k_scales", ctypes.c_void_p),
        ("v_scales", ctypes.c_void_p),
        ("k_scale", ctypes.c_float),
        ("v_scale", ctypes.c_float),
    ]


class Shape(ctypes.Structure):
    """Mirror of ``pa_shape``."""

    _fields_ = [
        ("num_seqs", ctypes.c_int32),
        ("total_q", ctypes.c_int32),
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("block_size", ctypes.c_int32),
        ("max_blocks_per_seq", ctypes.c_int32),
        ("max_q_len", ctypes.c_int32),
        ("max_ctx_len", ctypes.c_int32),
        ("partition_size", ctypes.c_int32),
        ("num_blocks", ctypes.c_int64),
        ("flags", ctypes.c_uint32),
        ("reserved", ctypes.c_uint32),
    ]


def lib_path() -> str:
    return _LIB_PATH


def load():
    """Load libpa.so (once).  Raises PaError-compatible RuntimeError if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH):
        raise RuntimeError(f"libpa.so not built at {_LIB_PATH}; run paged_kv_cache_attend_amd.build")
    # torch carries its own copy of the HIP runtime.  Loading torch first lets
    # libpa.so bind to that same copy (same SONAME), so device pointers and
    # stream handles from torch are valid in the library; loading libpa.so
    # first would put two HIP runtimes in the process.
    import torch  # noqa: F401
    lib = ctypes.CDLL(_LIB_PATH)
    P = ctypes.c_void_p
    shp = ctypes.POINTER(Shape)
    lib.pa_workspace_size.argtypes = [shp]
    lib.pa_workspace_size.restype = ctypes.c_size_t
    lib.pa_workspace_init.argtypes = [shp, P, ctypes.c_size_t, P]
    lib.pa_workspace_init.restype = ctypes.c_int
    lib.pa_num_partitions.argtypes = [shp]
    lib.pa_num_partitions.restype = ctypes.c_int32
    lib.pa_num_partitions_kv.argtypes = [shp, ctypes.c_int32]
    lib.pa_num_partitions_kv.restype = ctypes.c_int32
    lib.pa_attend.argtypes = [shp, P, P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
    lib.pa_attend.restype = ctypes.c_int
    lib.pa_measure_read_tiles.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int32, P, P]
    lib.pa_measure_read_tiles.restype = ctypes.c_int
    lib.pa_measure_mfma_bf16.argtypes = [ctypes.c_int32, ctypes.c_int32, P, P]
    lib.pa_measure_mfma_bf16.restype = ctypes.c_int
    lib.pa_attend_noalloc.argtypes = [shp, P, P, P, P, P, P, ctypes.c_float, P, P, P]
    lib.pa_attend_noalloc.restype = ctypes.c_int
    lib.pa_combine.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, P, P, P, P, P]
    lib.pa_combine.restype = ctypes.c_int
    lib.pa_gather_kv.argtypes = [shp, P, P, P, P, P]
    lib.pa_gather_kv.restype = ctypes.c_int
    lib.pa_validate.argtypes = [shp, P, P, P, P, ctypes.c_size_t, P, P]
    lib.pa_validate.restype = ctypes.c_int
    lib.pa_write_kv.argtypes = [shp, P, P, P, P, P, P, P, P]
    lib.pa_write_kv.restype = ctypes.c_int
    lib.pa_copy_blocks.argtypes = [ctypes.c_int32, P, P, ctypes.c_int32, ctypes.c_int64, P, P, P]
    lib.pa_copy_blocks.restype = ctypes.c_int
    i32, pi32 = ctypes.c_int32, ctypes.POINTER(ctypes.c_int32)
    lib.pa_pool_create.argtypes = [i32, i32, i32, i32, ctypes.POINTER(P)]
    lib.pa_pool_create.restype = ctypes.c_int
    lib.pa_pool_destroy.argtypes = [P]
    lib.pa_pool_destroy.restype = None
    lib.pa_pool_append.argtypes = [P, i32, i32, pi32, pi32, pi32]
    lib.pa_pool_append.restype = ctypes.c_int
    lib.pa_pool_fork.argtypes = [P, i32, i32, i32]
    lib.pa_pool_fork.restype = ctypes.c_int
    lib.pa_pool_release.argtypes = [P, i32, ctypes.c_uint64]
    lib.pa_pool_release.restype = ctypes.c_int
    lib.pa_pool_retire.argtypes = [P, ctypes.c_uint64]
    lib.pa_pool_retire.restype = ctypes.c_int
    lib.pa_pool_length.argtypes = [P, i32]
    lib.pa_pool_length.restype = i32
    lib.pa_pool_block_table.argtypes = [P]
    lib.pa_pool_block_table.restype = pi32
    lib.pa_pool_refcount.argtypes = [P, i32]
    lib.pa_pool_refcount.restype = i32
    lib.pa_pool_get_stats.argtypes = [P, ctypes.POINTER(PoolStats)]
    lib.pa_pool_get_stats.restype = ctypes.c_int
    kvp = ctypes.POINTER(KVCache)
    lib.pa_attend_kv.argtypes = [shp, kvp, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
    lib.pa_attend_kv.restype = ctypes.c_int
    lib.pa_write_kv_cache.argtypes = [shp, kvp, P, P, P, P, P, P]
    lib.pa_write_kv_cache.restype = ctypes.c_int
    pgp = ctypes.POINTER(PrefixGroups)
    lib.pa_prefix_workspace_size.argtypes = [shp, pgp]
    lib.pa_prefix_workspace_size.restype = ctypes.c_size_t
    lib.pa_prefix_workspace_init.argtypes = [shp, pgp, P, ctypes.c_size_t, P]
    lib.pa_prefix_workspace_init.restype = ctypes.c_int
    lib.pa_attend_prefix.argtypes = [shp, pgp, P, P, P, P, P, P, ctypes.c_float, P, P, P, ctypes.c_size_t, P]
    lib.pa_attend_prefix.restype = ctypes.c_int
    lib.pa_status_string.argtypes = [ctypes.c_int]
    lib.pa_status_string.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_string(status: int) -> str:
    return load().pa_status_string(int(status)).decode()


def _check(status: int, where: str):
    if status != Status.OK:
        raise PaError(status, where)


def make_shape(num_seqs, total_q, num_q_heads, num_kv_heads, max_blocks_per_seq, max_q_len,
               max_ctx_len, num_blocks, partition_size=0, causal=False, head_dim=128,
               block_size=16, flags=None) -> Shape:
    f = (PA_FLAG_CAUSAL if causal else 0) if flags is None else flags
    return Shape(int(num_seqs), int(total_q), int(num_q_heads), int(num_kv_heads), int(head_dim),
                 int(block_size), int(max_blocks_per_seq), int(max_q_len), int(max_ctx_len),
                 int(partition_size), int(num_blocks), int(f), 0)


def workspace_size(shape: Shape) -> int:
    return int(load().pa_workspace_size(ctypes.byref(shape)))


def workspace_init(shape: Shape, workspace, *, stream=None):
    """``pa_workspace_init``: zero the workspace's counters for this shape."""
    ws_bytes = workspace.numel() * workspace.element_size()
    st = load().pa_workspace_init(ctypes.byref(shape), _ptr(workspace), ctypes.c_size_t(ws_bytes),
                                  _stream_handle(workspace.device, stream))
    _check(st, "pa_workspace_init")


def plan(shape: Shape):
    """(workspace bytes, number of split-KV partitions) for a shape."""
    lib = load()
    return int(lib.pa_workspace_size(ctypes.byref(shape))), int(lib.pa_num_partitions(ctypes.byref(shape)))


# ---------------------------------------------------------------------------
# torch-tensor wrappers
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(device, stream):
    torch = _torch()
    return torch.cuda.current_stream(device) if stream is None else stream


def _stream_handle(device, stream):
    return ctypes.c_void_p(_stream(device, stream).cuda_stream)


def _new_workspace(shape: Shape, nbytes: int, device, stream, init=None, wait=False):
    """A workspace for calls launched on `stream`: allocated from that
    stream's pool (so the caching allocator reuses it only after the stream
    has passed the work queued on it) and initialised on that same stream.
    With ``wait`` the host waits for the initialisation (set-up of prepared
    calls, which may later be launched on other streams)."""
    torch = _torch()
    s = _stream(device, stream)
    with torch.cuda.stream(s):
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if init is None:
        workspace_init(shape, ws, stream=s)
    else:
        init(ws, s)
    if wait:
        done = torch.cuda.Event()
        done.record(s)
        done.synchronize()
    return ws


def _need(t, name, dtype, device, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")


def attend(q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, out, lse=None, *,
           max_q_len: int, max_ctx_len: int, partition_size: int = 0, causal: bool = False,
           workspace=None, stream=None):
    """``pa_attend`` on torch tensors (all on one GPU).

    q, out: bf16 [total_q, Hq, 128]; k_cache, v_cache: bf16 [num_blocks, Hkv, 16, 128];
    block_table: int32 [num_seqs, max_blocks]; ctx_lens, q_lens: int32 [num_seqs];
    lse: fp32 [total_q, Hq] or None.  ``max_q_len`` / ``max_ctx_len`` are the
    caller's known upper bounds (no device read happens here).  If the shape
    needs a workspace and none is given, one is allocated with torch.
    """
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(out, "out", torch.bfloat16, dev, 3)
    _need(k_cache, "k_cache", torch.bfloat16, dev, 4)
    _need(v_cache, "v_cache", torch.bfloat16, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, dev, 1)
    _need(q_lens, "q_lens", torch.int32, dev, 1)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    total_q, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if tuple(out.shape) != tuple(q.shape) or tuple(v_cache.shape) != tuple(k_cache.shape) or d2 != d:
        raise ValueError("shape mismatch between q/out or k_cache/v_cache")
    if lse is not None and tuple(lse.shape) != (total_q, hq):
        raise ValueError("lse must be [total_q, Hq]")
    num_seqs = block_table.shape[0]
    if ctx_lens.shape[0] != num_seqs or q_lens.shape[0] != num_seqs:
        raise ValueError("ctx_lens / q_lens must have one entry per block-table row")
    shape = make_shape(num_seqs, total_q, hq, hkv, block_table.shape[1], max_q_len, max_ctx_len,
                       nb, partition_size, causal, head_dim=d, block_size=bs)
    need = workspace_size(shape)
    if need and workspace is None:
        workspace = _new_workspace(shape, need, dev, stream)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().pa_attend(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                          _ptr(ctx_lens), _ptr(q_lens), ctypes.c_float(float(scale)), _ptr(out), _ptr(lse),
                          _ptr(workspace), ctypes.c_size_t(ws_bytes), _stream_handle(dev, stream))
    _check(st, "pa_attend")
    return out, lse


def attend_noalloc(q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, out, lse=None, *,
                   max_q_len: int, max_ctx_len: int, partition_size: int = 0, causal: bool = False,
                   stream=None):
    """``pa_attend_noalloc``: ``attend`` without a workspace; the library's
    built-in scratch buffer holds the split-KV partials (no allocation here
    or in the library)."""
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(out, "out", torch.bfloat16, dev, 3)
    _need(k_cache, "k_cache", torch.bfloat16, dev, 4)
    _need(v_cache, "v_cache", torch.bfloat16, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, dev, 1)
    _need(q_lens, "q_lens", torch.int32, dev, 1)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    total_q, hq, d = q.shape
    nb, hkv, bs, d2 = k_cache.shape
    if tuple(out.shape) != tuple(q.shape) or tuple(v_cache.shape) != tuple(k_cache.shape) or d2 != d:
        raise ValueError("shape mismatch between q/out or k_cache/v_cache")
    if lse is not None and tuple(lse.shape) != (total_q, hq):
        raise ValueError("lse must be [total_q, Hq]")
    num_seqs = block_table.shape[0]
    if ctx_lens.shape[0] != num_seqs or q_lens.shape[0] != num_seqs:
        raise ValueError("ctx_lens / q_lens must have one entry per block-table row")
    shape = make_shape(num_seqs, total_q, hq, hkv, block_table.shape[1], max_q_len, max_ctx_len,
                       nb, partition_size, causal, head_dim=d, block_size=bs)
    st = load().pa_attend_noalloc(ctypes.byref(shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                                  _ptr(ctx_lens), _ptr(q_lens), ctypes.c_float(float(scale)), _ptr(out),
                                  _ptr(lse), _stream_handle(dev, stream))
    _check(st, "pa_attend_noalloc")
    return out, lse


def measure_read_tiles(k_cache, v_cache, tiles, sink, *, tiles_per_wg: int, stream=None):
    """``pa_measure_read_tiles``: stream tiles (int32 tile indices) of both
    caches; sink uint32 [ceil(len(tiles) / tiles_per_wg)]."""
    torch = _torch()
    dev = k_cache.device
    _need(tiles, "tiles", torch.int32, dev, 1)
    _need(sink, "sink", torch.int32, dev, 1)
    n = int(tiles.shape[0])
    if sink.shape[0] < -(-n // tiles_per_wg):
        raise ValueError("sink too small")
    st = load().pa_measure_read_tiles(_ptr(k_cache), _ptr(v_cache), _ptr(tiles), ctypes.c_int64(n),
                                      ctypes.c_int32(tiles_per_wg), _ptr(sink), _stream_handle(dev, stream))
    _check(st, "pa_measure_read_tiles")


def measure_mfma_bf16(workgroups: int, iters: int, sink, *, stream=None):
    """``pa_measure_mfma_bf16``: sink float32 [workgroups * 4]; returns FLOP per call."""
    torch = _torch()
    _need(sink, "sink", torch.float32, sink.device, 1)
    if sink.shape[0] < workgroups * 4:
        raise ValueError("sink too small")
    st = load().pa_measure_mfma_bf16(int(workgroups), int(iters), _ptr(sink), _stream_handle(sink.device, stream))
    _check(st, "pa_measure_mfma_bf16")
    return workgroups * 4 * iters * 4 * 32768


def combine(partial_out, partial_lse, out, lse=None, *, stream=None):
    """``pa_combine``: partial_out fp32 [P, rows, D], partial_lse fp32 [P, rows],
    out bf16 [rows, D], lse fp32 [rows] or None."""
    torch = _torch()
    dev = partial_out.device
    _need(partial_out, "partial_out", torch.float32, dev, 3)
    _need(partial_lse, "partial_lse", torch.float32, dev, 2)
    _need(out, "out", torch.bfloat16, dev, 2)
    P, rows, D = partial_out.shape
    if tuple(partial_lse.shape) != (P, rows) or tuple(out.shape) != (rows, D):
        raise ValueError("shape mismatch")
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 1)
    st = load().pa_combine(P, rows, D, _ptr(partial_out), _ptr(partial_lse), _ptr(out), _ptr(lse),
                           _stream_handle(dev, stream))
    _check(st, "pa_combine")
    return out, lse


def gather_kv(cache, block_table, ctx_lens, dst, *, max_ctx_len: int, stream=None):
    """``pa_gather_kv``: dst bf16 [num_seqs, max_ctx_len, Hkv, 128]."""
    torch = _torch()
    dev = cache.device
    _need(cache, "cache", torch.bfloat16, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, dev, 1)
    _need(dst, "dst", torch.bfloat16, dev, 4)
    nb, hkv, bs, d = cache.shape
    num_seqs = block_table.shape[0]
    if tuple(dst.shape) != (num_seqs, max_ctx_len, hkv, d):
        raise ValueError("dst must be [num_seqs, max_ctx_len, Hkv, D]")
    shape = make_shape(num_seqs, 1, hkv, hkv, block_table.shape[1], 1, max_ctx_len, nb,
                       head_dim=d, block_size=bs)
    st = load().pa_gather_kv(ctypes.byref(shape), _ptr(cache), _ptr(block_table), _ptr(ctx_lens),
                             _ptr(dst), _stream_handle(dev, stream))
    _check(st, "pa_gather_kv")
    return dst


def validate(block_table, ctx_lens, q_lens, error_word, *, num_blocks: int, total_q: int,
             max_q_len: int, max_ctx_len: int, num_q_heads: int = 1, num_kv_heads: int = 1,
             partition_size: int = 0, workspace=None, stream=None):
    """``pa_validate``: writes the PA_BAD_* mask into error_word (int32 [1]);
    with ``workspace``, also checks its split-KV counters for this shape."""
    torch = _torch()
    dev = block_table.device
    _need(error_word, "error_word", torch.int32, dev, 1)
    shape = make_shape(block_table.shape[0], total_q, num_q_heads, num_kv_heads, block_table.shape[1],
                       max_q_len, max_ctx_len, num_blocks, partition_size)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    st = load().pa_validate(ctypes.byref(shape), _ptr(block_table), _ptr(ctx_lens), _ptr(q_lens),
                            _ptr(workspace), ctypes.c_size_t(ws_bytes), _ptr(error_word),
                            _stream_handle(dev, stream))
    _check(st, "pa_validate")
    return error_word


def write_kv(k_new, v_new, block_table, ctx_lens, q_lens, k_cache, v_cache, *, max_q_len: int,
             stream=None):
    """``pa_write_kv``: k_new, v_new bf16 [total_q, Hkv, 128] into the caches
    (bf16 [num_blocks, Hkv, 16, 128]) at positions n - m .. n - 1 of each slot."""
    torch = _torch()
    dev = k_cache.device
    _need(k_new, "k_new", torch.bfloat16, dev, 3)
    _need(v_new, "v_new", torch.bfloat16, dev, 3)
    _need(k_cache, "k_cache", torch.bfloat16, dev, 4)
    _need(v_cache, "v_cache", torch.bfloat16, dev, 4)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, dev, 1)
    _need(q_lens, "q_lens", torch.int32, dev, 1)
    total_q, hkv, d = k_new.shape
    nb, hkv2, bs, d2 = k_cache.shape
    if tuple(v_new.shape) != tuple(k_new.shape) or tuple(v_cache.shape) != tuple(k_cache.shape):
        raise ValueError("k_new/v_new or k_cache/v_cache shapes differ")
    if hkv != hkv2 or d != d2:
        raise ValueError("new rows and caches disagree on KV heads or head_dim")
    num_seqs = block_table.shape[0]
    if ctx_lens.shape[0] != num_seqs or q_lens.shape[0] != num_seqs:
        raise ValueError("ctx_lens / q_lens must have one entry per block-table row")
    shape = make_shape(num_seqs, total_q, hkv, hkv, block_table.shape[1], max_q_len,
                       bs * block_table.shape[1], nb, head_dim=d, block_size=bs)
    st = load().pa_write_kv(ctypes.byref(shape), _ptr(k_new), _ptr(v_new), _ptr(block_table),
                            _ptr(ctx_lens), _ptr(q_lens), _ptr(k_cache), _ptr(v_cache),
                            _stream_handle(dev, stream))
    _check(st, "pa_write_kv")


def copy_blocks(src, dst, k_cache, v_cache, *, stream=None):
    """``pa_copy_blocks``: src, dst int32 [num_copies] on the caches' device."""
    torch = _torch()
    dev = k_cache.device
    _need(src, "src", torch.int32, dev, 1)
    _need(dst, "dst", torch.int32, dev, 1)
    _need(k_cache, "k_cache", torch.bfloat16, dev, 4)
    _need(v_cache, "v_cache", torch.bfloat16, dev, 4)
    if src.shape != dst.shape:
        raise ValueError("src and dst differ in length")
    nb, hkv, _, _ = k_cache.shape
    st = load().pa_copy_blocks(int(src.shape[0]), _ptr(src), _ptr(dst), hkv, nb, _ptr(k_cache),
                               _ptr(v_cache), _stream_handle(dev, stream))
    _check(st, "pa_copy_blocks")


def attend_prefix(q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, out, lse=None, *,
                  group_start, prefix_len, max_members: int, max_prefix_len: int, min_prefix_len: int = 0,
                  max_ctx_len: int, partition_size: int = 0, workspace=None, stream=None,
                  prepared: bool = False):
    """``pa_attend_prefix``: pa_attend with groups of consecutive slots that
    share a prefix (group_start int32 [num_groups + 1], prefix_len int32
    [num_groups], on the device).  With ``prepared=True`` returns a
    launchable object instead of launching once."""
    torch = _torch()
    dev = q.device
    for t, name, dt, nd in ((q, "q", torch.bfloat16, 3), (out, "out", torch.bfloat16, 3),
                            (k_cache, "k_cache", torch.bfloat16, 4), (v_cache, "v_cache", torch.bfloat16, 4),
                            (block_table, "block_table", torch.int32, 2), (ctx_lens, "ctx_lens", torch.int32, 1),
                            (q_lens, "q_lens", torch.int32, 1), (group_start, "group_start", torch.int32, 1),
                            (prefix_len, "prefix_len", torch.int32, 1)):
        _need(t, name, dt, dev, nd)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    if group_start.shape[0] != prefix_len.shape[0] + 1:
        raise ValueError("group_start must have one entry more than prefix_len")
    total_q, hq, d = q.shape
    nb, hkv, bs, _ = k_cache.shape
    shape = make_shape(block_table.shape[0], total_q, hq, hkv, block_table.shape[1], 1, max_ctx_len, nb,
                       partition_size, head_dim=d, block_size=bs)
    groups = PrefixGroups(int(prefix_len.shape[0]), int(max_members), int(max_prefix_len), int(min_prefix_len),
                          0, 0, _ptr(group_start).value, _ptr(prefix_len).value)
    lib = load()
    need = int(lib.pa_prefix_workspace_size(ctypes.byref(shape), ctypes.byref(groups)))
    if need == 0:
        raise PaError(Status.ERR_BAD_SHAPE, "pa_prefix_workspace_size")
    if workspace is None:
        def init(ws, s):
            _check(lib.pa_prefix_workspace_init(ctypes.byref(shape), ctypes.byref(groups), _ptr(ws),
                                                ctypes.c_size_t(need), ctypes.c_void_p(s.cuda_stream)),
                   "pa_prefix_workspace_init")
        workspace = _new_workspace(shape, need, dev, stream, init, wait=prepared)
    ws_bytes = workspace.numel() * workspace.element_size()
    args = [ctypes.byref(shape), ctypes.byref(groups), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
            _ptr(ctx_lens), _ptr(q_lens), ctypes.c_float(float(scale)), _ptr(out), _ptr(lse), _ptr(workspace),
            ctypes.c_size_t(ws_bytes)]
    fn = lib.pa_attend_prefix

    class _Call:
        keep = (shape, groups, q, k_cache, v_cache, block_table, ctx_lens, q_lens, group_start, prefix_len,
                out, lse, workspace)

        def launch(self, s=None):
            st = fn(*args, _stream_handle(dev, s))
            if st:
                raise PaError(st, "pa_attend_prefix")

    call = _Call()
    if prepared:
        return call
    call.launch(stream)
    return out, lse


class QuantCache:
    """One layer's K/V pages in a ``pa_kv_format`` (torch tensors on one GPU).

    bf16: k_codes, v_codes bf16 [num_blocks, Hkv, 16, 128].
    FP8:  uint8 codes [num_blocks, Hkv, 16, 128] and one fp32 scale per cache.
    q8_0: int8 codes [num_blocks, Hkv, 16, 128], fp16 scales [num_blocks, Hkv, 16, 4].
    q4_0: uint8 codes [num_blocks, Hkv, 16, 64], fp16 scales as q8_0.
    """

    def __init__(self, fmt: int, k_codes, v_codes, k_scales=None, v_scales=None, k_scale: float = 1.0,
                 v_scale: float = 1.0):
        self.format = int(fmt)
        self.k_codes, self.v_codes = k_codes, v_codes
        self.k_scales, self.v_scales = k_scales, v_scales
        self.k_scale, self.v_scale = float(k_scale), float(v_scale)
        self.num_blocks, self.num_kv_heads = int(k_codes.shape[0]), int(k_codes.shape[1])

    @classmethod
    def empty(cls, fmt: int, num_blocks: int, num_kv_heads: int, device, k_scale: float = 1.0,
              v_scale: float = 1.0):
        torch = _torch()
        dims = {KV_BF16: (128, torch.bfloat16), KV_FP8_E4M3: (128, torch.uint8), KV_Q8_0: (128, torch.int8),
                KV_Q4_0: (64, torch.uint8)}
        if fmt not in dims:
            raise ValueError(f"unknown KV format {fmt}")
        d, dt = dims[fmt]
        shape = (num_blocks, num_kv_heads, 16, d)
        k = torch.zeros(shape, dtype=dt, device=device)
        v = torch.zeros(shape, dtype=dt, device=device)
        ks = vs = None
        if fmt in (KV_Q8_0, KV_Q4_0):
            ks = torch.zeros((num_blocks, num_kv_heads, 16, 4), dtype=torch.float16, device=device)
            vs = torch.zeros_like(ks)
        return cls(fmt, k, v, ks, vs, k_scale, v_scale)

    def struct(self) -> KVCache:
        return KVCache(self.format, 0, _ptr(self.k_codes).value, _ptr(self.v_codes).value,
                       None if self.k_scales is None else _ptr(self.k_scales).value,
                       None if self.v_scales is None else _ptr(self.v_scales).value,
                       self.k_scale, self.v_scale)

    def check(self, device):
        torch = _torch()
        want = {KV_BF16: torch.bfloat16, KV_FP8_E4M3: torch.uint8, KV_Q8_0: torch.int8, KV_Q4_0: torch.uint8}
        dim = 64 if self.format == KV_Q4_0 else 128
        for t, name in ((self.k_codes, "k_codes"), (self.v_codes, "v_codes")):
            _need(t, name, want[self.format], device, 4)
            if t.shape[2:] != (16, dim):
                raise ValueError(f"{name} must be [num_blocks, Hkv, 16, {dim}]")
        if self.k_codes.shape != self.v_codes.shape:
            raise ValueError("k_codes and v_codes differ in shape")
        if self.format in (KV_Q8_0, KV_Q4_0):
            for t, name in ((self.k_scales, "k_scales"), (self.v_scales, "v_scales")):
                _need(t, name, torch.float16, device, 4)
                if tuple(t.shape) != (self.num_blocks, self.num_kv_heads, 16, 4):
                    raise ValueError(f"{name} must be [num_blocks, Hkv, 16, 4]")


def attend_kv(q, cache: QuantCache, block_table, ctx_lens, q_lens, scale, out, lse=None, *,
              max_q_len: int, max_ctx_len: int, partition_size: int = 0, workspace=None, stream=None,
              prepared: bool = False):
    """``pa_attend_kv`` on torch tensors; with ``prepared=True`` returns a
    launchable object (for graphs and timing) instead of launching once."""
    torch = _torch()
    dev = q.device
    _need(q, "q", torch.bfloat16, dev, 3)
    _need(out, "out", torch.bfloat16, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, dev, 1)
    _need(q_lens, "q_lens", torch.int32, dev, 1)
    cache.check(dev)
    if lse is not None:
        _need(lse, "lse", torch.float32, dev, 2)
    total_q, hq, d = q.shape
    if tuple(out.shape) != tuple(q.shape):
        raise ValueError("out must match q")
    num_seqs = block_table.shape[0]
    shape = make_shape(num_seqs, total_q, hq, cache.num_kv_heads, block_table.shape[1], max_q_len,
                       max_ctx_len, cache.num_blocks, partition_size, head_dim=d)
    need = workspace_size(shape)
    if need and workspace is None:
        workspace = _new_workspace(shape, need, dev, stream, wait=prepared)
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    kv = cache.struct()
    args = [ctypes.byref(shape), ctypes.byref(kv), _ptr(q), _ptr(block_table), _ptr(ctx_lens), _ptr(q_lens),
            ctypes.c_float(float(scale)), _ptr(out), _ptr(lse), _ptr(workspace), ctypes.c_size_t(ws_bytes)]
    fn = load().pa_attend_kv

    class _Call:
        keep = (shape, kv, q, cache, block_table, ctx_lens, q_lens, out, lse, workspace)
        num_partitions = int(load().pa_num_partitions_kv(ctypes.byref(shape), cache.format))

        def launch(self, s=None):
            st = fn(*args, _stream_handle(dev, s))
            if st:
                raise PaError(st, "pa_attend_kv")

    call = _Call()
    if prepared:
        return call
    call.launch(stream)
    return out, lse


def write_kv_cache(k_new, v_new, block_table, ctx_lens, q_lens, cache: QuantCache, *, max_q_len: int,
                   stream=None):
    """``pa_write_kv_cache``: encode new bf16 rows [total_q, Hkv, 128] into the cache."""
    torch = _torch()
    dev = k_new.device
    _need(k_new, "k_new", torch.bfloat16, dev, 3)
    _need(v_new, "v_new", torch.bfloat16, dev, 3)
    _need(block_table, "block_table", torch.int32, dev, 2)
    _need(ctx_lens, "ctx_lens", torch.int32, dev, 1)
    _need(q_lens, "q_lens", torch.int32, dev, 1)
    cache.check(dev)
    total_q, hkv, d = k_new.shape
    if tuple(v_new.shape) != tuple(k_new.shape) or hkv != cache.num_kv_heads:
        raise ValueError("new rows disagree with each other or with the cache")
    num_seqs = block_table.shape[0]
    shape = make_shape(num_seqs, total_q, hkv, hkv, block_table.shape[1], max_q_len,
                       16 * block_table.shape[1], cache.num_blocks, head_dim=d)
    kv = cache.struct()
    st = load().pa_write_kv_cache(ctypes.byref(shape), ctypes.byref(kv), _ptr(k_new), _ptr(v_new),
                                  _ptr(block_table), _ptr(ctx_lens), _ptr(q_lens), _stream_handle(dev, stream))
    _check(st, "pa_write_kv_cache")


class Pool:
    """``pa_pool``: block tables, reference counts, copy-on-write, fenced release.

    Host-side only.  ``append`` returns the (src, dst) block copies the caller
    must make (``copy_blocks`` on every layer's caches) before writing.
    """

    def __init__(self, num_blocks: int, block_size: int, num_slots: int, max_blocks_per_seq: int):
        lib = load()
        h = ctypes.c_void_p()
        _check(lib.pa_pool_create(num_blocks, block_size, num_slots, max_blocks_per_seq, ctypes.byref(h)),
               "pa_pool_create")
        self._h = h
        self._lib = lib
        self.num_blocks, self.block_size = num_blocks, block_size
        self.num_slots, self.max_blocks = num_slots, max_blocks_per_seq

    def close(self):
        if self._h:
            self._lib.pa_pool_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, slot: int, num_tokens: int):
        """Copies to make (list of (src, dst)), or None if the pool is too small."""
        src, dst, n = ctypes.c_int32(), ctypes.c_int32(), ctypes.c_int32()
        st = self._lib.pa_pool_append(self._h, slot, num_tokens, ctypes.byref(src), ctypes.byref(dst),
                                      ctypes.byref(n))
        if st == Status.ERR_OUT_OF_BLOCKS:
            return None
        _check(st, "pa_pool_append")
        return [(src.value, dst.value)] if n.value else []

    def fork(self, src: int, dst: int, num_tokens: int = -1):
        _check(self._lib.pa_pool_fork(self._h, src, dst, num_tokens), "pa_pool_fork")

    def release(self, slot: int, fence: int):
        _check(self._lib.pa_pool_release(self._h, slot, ctypes.c_uint64(fence)), "pa_pool_release")

    def retire(self, fence: int):
        _check(self._lib.pa_pool_retire(self._h, ctypes.c_uint64(fence)), "pa_pool_retire")

    def length(self, slot: int) -> int:
        return int(self._lib.pa_pool_length(self._h, slot))

    def refcount(self, block: int) -> int:
        return int(self._lib.pa_pool_refcount(self._h, block))

    def stats(self) -> PoolStats:
        s = PoolStats()
        _check(self._lib.pa_pool_get_stats(self._h, ctypes.byref(s)), "pa_pool_get_stats")
        return s

    def table(self):
        """A numpy copy of the block tables, int32 [num_slots, max_blocks_per_seq]."""
        import numpy as np
        n = self.num_slots * self.max_blocks
        ptr = self._lib.pa_pool_block_table(self._h)
        if n == 0:
            return np.zeros((self.num_slots, self.max_blocks), dtype=np.int32)
        return np.ctypeslib.as_array(ptr, shape=(n,)).reshape(self.num_slots, self.max_blocks).copy()


class PreparedAttend:
    """A ``pa_attend`` call with its arguments marshalled once.

    For launch loops (benchmarks, graph capture): ``launch()`` makes the bare
    C call and checks the status.  The workspace is initialised on ``stream``
    (default: the current stream at construction), and construction waits for
    that initialisation, so the first launch may go to any stream.  The
    tensors must stay alive and in place for as long as the object is used.
    """

    def __init__(self, q, k_cache, v_cache, block_table, ctx_lens, q_lens, scale, out, lse=None, *,
                 max_q_len: int, max_ctx_len: int, partition_size: int = 0, causal: bool = False,
                 workspace=None, stream=None):
        torch = _torch()
        dev = q.device
        for t, name, dt, nd in ((q, "q", torch.bfloat16, 3), (out, "out", torch.bfloat16, 3),
                                (k_cache, "k_cache", torch.bfloat16, 4), (v_cache, "v_cache", torch.bfloat16, 4),
                                (block_table, "block_table", torch.int32, 2), (ctx_lens, "ctx_lens", torch.int32, 1),
                                (q_lens, "q_lens", torch.int32, 1)):
            _need(t, name, dt, dev, nd)
        if lse is not None:
            _need(lse, "lse", torch.float32, dev, 2)
        total_q, hq, d = q.shape
        nb, hkv, bs, _ = k_cache.shape
        self.shape = make_shape(block_table.shape[0], total_q, hq, hkv, block_table.shape[1], max_q_len,
                                max_ctx_len, nb, partition_size, causal, head_dim=d, block_size=bs)
        need, self.num_partitions = plan(self.shape)
        self.stream = _stream(dev, stream)
        if need:
            if workspace is None:
                workspace = _new_workspace(self.shape, need, dev, self.stream)
            else:
                if workspace.numel() * workspace.element_size() < need:
                    raise PaError(Status.ERR_WORKSPACE_TOO_SMALL, "PreparedAttend")
                workspace_init(self.shape, workspace, stream=self.stream)
            done = torch.cuda.Event()
            done.record(self.stream)
            done.synchronize()  # set-up only: launches on any stream see zeroed counters
        self.workspace = workspace
        ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
        self._keep = (q, k_cache, v_cache, block_table, ctx_lens, q_lens, out, lse, workspace)
        self._fn = load().pa_attend
        self._args = [ctypes.byref(self.shape), _ptr(q), _ptr(k_cache), _ptr(v_cache), _ptr(block_table),
                      _ptr(ctx_lens), _ptr(q_lens), ctypes.c_float(float(scale)), _ptr(out), _ptr(lse),
                      _ptr(workspace), ctypes.c_size_t(ws_bytes)]
        self.device = dev

    def launch(self, stream=None):
        """Launch on `stream` (default: the stream given at construction)."""
        s = self.stream if stream is None else stream
        st = self._fn(*self._args, ctypes.c_void_p(s.cuda_stream))
        if st:
            raise PaError(st, "pa_attend")
