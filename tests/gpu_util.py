"""Shared helpers for the GPU tests: run the HIP path through the C ABI on a
seeded problem and compare it with the FP64 oracle."""

from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import paged_kv_cache_attend_amd as pk
from paged_kv_cache_attend_amd import inputs

DEV = torch.device("cuda:0")

# Tolerances on the output and the LSE (natural log), from the accuracy
# budget of bf16 storage with fp32 accumulation: absolute bounds max |dout|
# <= 1e-2, mean |dout| <= 1e-3, max |dlse| <= 1e-3.  Below
# |o| = 4 half a bf16 ulp of the output is at most 2^-8 ~ 0.0039 and the max
# bound is the absolute 1e-2.  From |o| = 4 on, half an ulp alone is 2^-6 =
# 0.0156 or more, above 1e-2 before any arithmetic, so there the bound is that
# half ulp plus the same 1e-2 as the margin for the arithmetic.
TOL_MAX = 1e-2
TOL_MEAN = 1e-3
TOL_LSE = 1e-3


def half_ulp_bf16(x: np.ndarray) -> np.ndarray:
    """Half the bf16 spacing at |x| (8 significant bits): 2^(floor(log2|x|) - 8)."""
    a = np.maximum(np.abs(np.asarray(x, dtype=np.float64)), np.finfo(np.float64).tiny)
    return np.exp2(np.floor(np.log2(a)) - 8.0)


def out_bound(exact: np.ndarray) -> np.ndarray:
    """Per-element bound on |out - exact| for exact outputs `exact`."""
    a = np.abs(exact)
    return np.where(a < 4.0, TOL_MAX, half_ulp_bf16(a) + TOL_MAX)

OUT_SENTINEL = 0x7F81         # a bf16 NaN pattern no kernel produces
LSE_SENTINEL = 0x7FC12345     # an fp32 NaN pattern no kernel produces


def say(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return oracle.bf16_bits_to_f64(bits)


def run_gpu(problem, layer=0, *, q=None, k=None, v=None, table=None, partition_size=None,
            causal=None, with_lse=True, repeats=1):
    """One pa_attend call; returns (out bits uint16 [total_q, Hq, D], lse float32 [total_q, Hq])."""
    if q is None:
        q, k, v = problem.layer(layer)
    t = inputs.to_device(problem, q, k, v, DEV, table)
    total_q, hq, d = q.shape
    out = torch.full((total_q, hq, d), OUT_SENTINEL, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    lse = None
    if with_lse:
        lse = torch.full((total_q, hq), LSE_SENTINEL, dtype=torch.int32, device=DEV).view(torch.float32)
    ps = problem.partition_size if partition_size is None else partition_size
    cz = problem.causal if causal is None else causal
    for _ in range(repeats):
        pk.attend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                  float(problem.scale), out, lse, max_q_len=max(problem.max_q_len, 0),
                  max_ctx_len=problem.max_ctx_len, partition_size=ps, causal=cz)
    torch.cuda.synchronize()
    ob = out.view(torch.int16).cpu().numpy().view(np.uint16)
    lb = None if lse is None else lse.cpu().numpy()
    return ob, lb


def run_oracle(problem, layer=0, *, q=None, k=None, v=None, table=None, causal=None, seqs=None):
    if q is None:
        q, k, v = problem.layer(layer)
    t = problem.block_table if table is None else table
    cz = problem.causal if causal is None else causal
    return oracle.attend_fp64(q, k, v, t, problem.ctx_lens, problem.q_lens, problem.scale,
                              problem.num_kv_heads, problem.block_size, causal=cz, seqs=seqs)


def compare(problem, gpu, ref, *, label=""):
    """Assert tolerances on written rows and untouched sentinels elsewhere."""
    ob, lb = gpu
    out, lse, written = ref
    o = bf16_to_f64(ob)
    err = np.abs(o[written] - out[written])
    assert np.isfinite(o[written]).all(), f"{label}: non-finite output"
    emax = float(err.max()) if err.size else 0.0
    emean = float(err.mean()) if err.size else 0.0
    ratio = float((err / out_bound(out[written])).max()) if err.size else 0.0
    lmax = None
    if lb is not None:
        el = np.abs(lb[written].astype(np.float64) - lse[written])
        lmax = float(el.max()) if el.size else 0.0
    say(f"  {label}: max |dout| {emax:.3e} ({ratio:.3f} of its bound), mean |dout| {emean:.3e}, "
        f"max |dlse| {lmax if lmax is None else f'{lmax:.3e}'}")
    assert ratio <= 1.0, f"{label}: max |dout| {emax:.3e} ({ratio:.3f} of its bound)"
    assert emean <= TOL_MEAN, f"{label}: mean |dout| {emean:.3e}"
    if lb is not None:
        assert lmax <= TOL_LSE, f"{label}: max |dlse| {lmax:.3e}"
        assert (lb[~written].view(np.uint32) == np.uint32(LSE_SENTINEL)).all(), f"{label}: lse of an inactive row written"
    assert (ob[~written] == OUT_SENTINEL).all(), f"{label}: out of an inactive row written"
    return emax, emean
