#!/usr/bin/env python3
"""Paged KV-cache attention benchmark on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config NAME]

A step is one pass of the hot path over one batch: for the decode workloads,
``pa_attend`` on every layer in turn (each layer has its own K/V pool, so the
pass streams all layers' KV from HBM; a single layer would fit the 256 MB
Infinity Cache), for the chunk workload one ``pa_attend`` call.  Inputs are
seeded synthetic N(0, 1) bf16 values with the shapes of the named workload,
uploaded before timing.  Prints ONE JSON line.

Default workload: 36 layers x 16 slots x 2303 keys, 32 query / 8 KV heads of
128 (the Qwen3-8B-shaped decode batch), split-KV with an automatic partition.
"""

from __future__ import annotations

import argparse
import json
import os
import platform
import sys
import time

import numpy as np

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA
METRIC = "paged decode attention KV-read GB/s (% of HBM peak) + chunk-attn TFLOP/s"


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="qwen3_8b_short_decode")
    ap.add_argument("--partition-size", type=int, default=None,
                    help="split-KV partition in tokens (default: the workload's own, 0 = automatic)")
    ap.add_argument("--launch", choices=["graph", "eager"], default="graph")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chunk", action="store_true", help="skip the secondary chunk-path measurement")
    ap.add_argument("--no-append", action="store_true", help="skip the secondary K/V-append measurement")
    ap.add_argument("--no-quant", action="store_true", help="skip the secondary quantised-KV decode measurement")
    ap.add_argument("--no-prefix", action="store_true", help="skip the shared-prefix workload (pa_attend and pa_attend_prefix)")
    ap.add_argument("--no-ragged", action="store_true", help="skip the ragged mixed decode workload")
    ap.add_argument("--no-causal", action="store_true", help="skip chunked prefill and speculative verification")
    ap.add_argument("--cpu-budget-s", type=float, default=25.0)
    ap.add_argument("--mode", choices=["bench", "copy"], default="bench",
                    help="copy: time a plain 1 GiB device copy (counter calibration for rocprofv3)")
    ap.add_argument("--quick", action="store_true", help="skip the eager and per-launch re-timings and the ceilings")
    return ap.parse_args()


ROOT = os.path.dirname(os.path.abspath(__file__))
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")


def kernel_source_hash() -> str:
    """Hash of the HIP sources; counter-derived traffic is only reported for
    the exact sources it was measured on."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "paged_kv_cache_attend_amd", "csrc")
    for name in sorted(os.listdir(csrc)):
        with open(os.path.join(csrc, name), "rb") as f:
            h.update(name.encode())
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_entry(workload: str, kernel: str):
    """The committed counter summary of one kernel on one workload, or None
    if it is missing or was taken on other sources."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    if rec.get("source_hash") != kernel_source_hash():
        return None
    return rec.get("workloads", {}).get(workload, {}).get(kernel) or None


def measured_traffic(workload: str, kernel: str):
    """(fetch, write) HBM bytes per launch from the committed counter summary,
    or None if it is missing or was taken on other sources."""
    ent = traffic_entry(workload, kernel)
    if not ent:
        return None
    return ent["fetch_bytes_per_launch"], ent["write_bytes_per_launch"]


def copy_mode(steps: int):
    """A plain 1 GiB device-to-device copy, for calibrating FETCH_SIZE /
    WRITE_SIZE against a known byte count."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(steps):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    print(json.dumps({"mode": "copy", "bytes_read_per_copy": n, "bytes_written_per_copy": n, "ms_per_copy": ms,
                      "copy_gbs_read_plus_write": 2 * n / (ms * 1e-3) / 1e9}), flush=True)


def copy_ceiling(dev, steps: int = 20):
    """Read+write GB/s of a plain 1 GiB device-to-device copy on the launch
    stream: the rate a streaming kernel can hope for on this device."""
    import torch
    n = 1 << 30
    src = torch.ones(n, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    stream = torch.cuda.current_stream()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        dst.copy_(src)
    e1.record(stream)
    torch.cuda.synchronize()
    ms = e0.elapsed_time(e1) / steps
    del src, dst
    torch.cuda.empty_cache()
    return 2 * n / (ms * 1e-3) / 1e9


def build_decode(problem, dev, want_oracle: bool, cpu_budget_s: float):
    """Upload every layer; run the oracle on layers while the CPU budget lasts."""
    import torch
    from paged_kv_cache_attend_amd import inputs
    layers = []
    ref = {}
    cpu_time = 0.0
    cpu_bytes = 0
    if want_oracle:
        import oracle
        from threadpoolctl import threadpool_limits
    for l in range(problem.num_layers):
        q, k, v = problem.layer(l)
        t = inputs.to_device(problem, q, k, v, dev)
        layers.append(t)
        if want_oracle and cpu_time < cpu_budget_s:
            with threadpool_limits(1):
                t0 = time.perf_counter()
                ref[l] = oracle.attend_fp64(q, k, v, problem.block_table, problem.ctx_lens, problem.q_lens,
                                            problem.scale, problem.num_kv_heads, problem.block_size,
                                            causal=problem.causal)
                cpu_time += time.perf_counter() - t0
            cpu_bytes += problem.kv_bytes_read()
        del q, k, v
        if l % 6 == 5 or l == problem.num_layers - 1:
            log(f"uploaded {l + 1}/{problem.num_layers} layers; oracle {len(ref)} layers in {cpu_time:.1f}s")
    torch.cuda.synchronize()
    return layers, ref, cpu_time, cpu_bytes


def prepare_calls(problem, layers, partition_size):
    import torch
    import paged_kv_cache_attend_amd as pk
    calls, outs, lses = [], [], []
    workspace = None
    for t in layers:
        out = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device=t["q"].device)
        c = pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                              float(problem.scale), out, lse, max_q_len=problem.max_q_len,
                              max_ctx_len=problem.max_ctx_len, partition_size=partition_size,
                              causal=problem.causal, workspace=workspace)
        workspace = c.workspace  # one workspace serves every layer (stream-ordered)
        calls.append(c)
        outs.append(out)
        lses.append(lse)
    return calls, outs, lses


def time_pass(calls, steps, warmup, launch, trials=5):
    """Time `trials` runs of exactly `steps` passes each (a pass = every call
    once, in order), each bracketed by a synchronisation on both sides.
    Returns (median ms per pass, best ms per pass, wall ms per pass of the
    median trial, per-trial ms list)."""
    import torch
    stream = torch.cuda.current_stream()

    def one_pass():
        for c in calls:
            c.launch(stream)

    graph = None
    if launch == "graph":
        one_pass()  # make sure everything is loaded before capture
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=stream):
            one_pass()
        run = graph.replay
    else:
        run = one_pass
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    per, walls = [], []
    for _ in range(trials):
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        e0.record(stream)
        for _ in range(steps):
            run()
        e1.record(stream)
        torch.cuda.synchronize()
        walls.append((time.perf_counter() - t0) * 1e3 / steps)
        per.append(e0.elapsed_time(e1) / steps)
    order = sorted(range(trials), key=lambda i: per[i])
    med = order[trials // 2]
    return per[med], per[order[0]], walls[med], per


def time_kernel_launches(calls, reps):
    """Average duration of one pa_attend call (all of its launches), measured
    with HIP events on the launch stream around `reps` back-to-back passes."""
    import torch
    stream = torch.cuda.current_stream()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        for c in calls:
            c.launch(stream)
    e1.record(stream)
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / (reps * len(calls))


def parity(problem, outs, lses, ref):
    import torch
    import oracle
    emax = emean = lmax = worst = 0.0
    n = 0
    for l, (o_ref, l_ref, written) in ref.items():
        ob = outs[l].view(torch.int16).cpu().numpy().view(np.uint16)
        lb = lses[l].cpu().numpy().astype(np.float64)
        o = oracle.bf16_bits_to_f64(ob)
        err = np.abs(o[written] - o_ref[written])
        # 1e-2; where |o| >= 4, half its bf16 spacing (alone above 1e-2
        # there) plus 1e-2
        a = np.abs(o_ref[written])
        bound = np.where(a < 4, 1e-2, np.exp2(np.floor(np.log2(np.maximum(a, 1e-300))) - 8) + 1e-2)
        worst = max(worst, float((err / bound).max()))
        emax = max(emax, float(err.max()))
        emean = max(emean, float(err.mean()))
        lmax = max(lmax, float(np.abs(lb[written] - l_ref[written]).max()))
        n += 1
    return {"layers_checked": n, "max_abs_out": emax, "mean_abs_out": emean, "max_abs_lse": lmax,
            "pass": bool(worst <= 1.0 and emean <= 1e-3 and lmax <= 1e-3)}


def device_layers(problem, dev, num_layers, seed):
    """Per-layer device tensors for a workload's structure, with values drawn
    on the device (N(0, 1) rounded to bf16): for timing runs whose parity the
    GPU tests check on the host-drawn inputs."""
    import torch
    g = torch.Generator(device=dev)
    g.manual_seed(seed)
    bt = torch.from_numpy(problem.block_table.astype(np.int32)).to(dev)
    cl = torch.from_numpy(problem.ctx_lens.astype(np.int32)).to(dev)
    ql = torch.from_numpy(problem.q_lens.astype(np.int32)).to(dev)
    hd = problem.head_dim
    layers = []
    for _ in range(num_layers):
        shape = (problem.num_blocks, problem.num_kv_heads, problem.block_size, hd)
        layers.append(dict(
            q=torch.randn((problem.total_q, problem.num_q_heads, hd), generator=g, device=dev).bfloat16(),
            k=torch.randn(shape, generator=g, device=dev).bfloat16(),
            v=torch.randn(shape, generator=g, device=dev).bfloat16(),
            block_table=bt, ctx_lens=cl, q_lens=ql))
    return layers


def hbm_roofline(bytes_per_launch, us, kernel, ceiling_gbs=None, **extra):
    gbs = bytes_per_launch / (us * 1e-6) / 1e9
    r = {"bound": "hbm", "achieved": gbs, "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": gbs / HBM_PEAK_GBS,
         "algorithmic_bytes_per_launch": bytes_per_launch, "avg_launch_us": us, "kernel": kernel}
    if ceiling_gbs:
        r["frac_of_measured_read_ceiling"] = gbs / ceiling_gbs
    r.update(extra)
    return r


def read_ceiling(problem, layers, steps, launch):
    """The measured streaming ceiling for a decode workload: the same K/V
    tiles (each (slot, page, KV head) once) of every layer, read with the
    decode kernel's loads and nothing else, one launch per layer as the
    decode pass does; for 72 tiles per workgroup (the decode grid at two
    partitions) and for finer grids.  GB/s over the same algorithmic bytes."""
    import torch
    import paged_kv_cache_attend_amd as pk
    dev = layers[0]["k"].device
    tl = []
    hkv = problem.num_kv_heads
    for r in range(problem.num_seqs):
        n = int(problem.ctx_lens[r])
        for j in range(-(-n // problem.block_size)):
            phys = int(problem.block_table[r][j])
            tl.extend(phys * hkv + g for g in range(hkv))
    tiles = torch.tensor(tl, dtype=torch.int32, device=dev)
    bytes_per_launch = len(tl) * 2 * problem.block_size * problem.head_dim * 2
    res = {}
    for tpw in (72, 36, 18):
        sink = torch.zeros(-(-len(tl) // tpw), dtype=torch.int32, device=dev)

        class _C:
            def __init__(self, t):
                self.t = t

            def launch(self, s):
                pk.measure_read_tiles(self.t["k"], self.t["v"], tiles, sink, tiles_per_wg=tpw, stream=s)

        calls = [_C(t) for t in layers]
        ms, best, _, _ = time_pass(calls, max(steps // 4, 20), 3, launch)
        us = ms * 1e3 / len(calls)
        res[f"tiles_per_workgroup_{tpw}"] = {"us_per_launch": us, "gbs": bytes_per_launch / (us * 1e-6) / 1e9}
    best_gbs = max(v["gbs"] for v in res.values())
    return {"gbs": best_gbs, "frac_of_hbm_peak": best_gbs / HBM_PEAK_GBS, "bytes_per_launch": bytes_per_launch,
            "kernel": "pa_measure_read_tiles (same tiles and loads as the decode kernel, no arithmetic), "
                      "one launch per layer in a graph", "variants": res}


def mfma_ceiling():
    """Measured bf16 matrix-core throughput (v_mfma_f32_32x32x16_bf16, four
    independent chains per wave, 2 and 4 workgroups of 4 waves per CU)."""
    import torch
    import paged_kv_cache_attend_amd as pk
    best = 0.0
    res = {}
    for wgs in (512, 1024):
        sink = torch.zeros(wgs * 4, dtype=torch.float32, device="cuda:0")
        iters = 4000
        flop = pk.measure_mfma_bf16(wgs, iters, sink)  # warm-up
        torch.cuda.synchronize()
        stream = torch.cuda.current_stream()
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(5):
            pk.measure_mfma_bf16(wgs, iters, sink)
        e1.record(stream)
        torch.cuda.synchronize()
        tf = flop * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e12
        res[f"workgroups_{wgs}"] = tf
        best = max(best, tf)
    return {"tflops": best, "frac_of_spec": best / BF16_PEAK_TFLOPS,
            "kernel": "pa_measure_mfma_bf16 (v_mfma_f32_32x32x16_bf16, 4 chains per wave)", "variants": res}


def chunk_secondary(dev, steps, launch="graph", mfma_tflops=None):
    """TFLOP/s of the chunked-denoising workload (4 x 24 heads x 256 rows x 1024 keys)."""
    import torch
    import paged_kv_cache_attend_amd as pk
    from paged_kv_cache_attend_amd import inputs
    p = inputs.chunked_denoise()
    q, k, v = p.layer(0)
    sets = []
    for _ in range(16):  # 16 resident copies (~1 GB) so a rotation misses the Infinity Cache
        t = inputs.to_device(p, q, k, v, dev)
        out = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device=dev)
        sets.append(pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                                      float(p.scale), out, lse, max_q_len=p.max_q_len,
                                      max_ctx_len=p.max_ctx_len))
    flops = 4 * int((p.q_lens.astype(np.int64) * p.ctx_lens).sum()) * p.num_q_heads * p.head_dim
    passes = max(steps, 640) // 16  # 16 launches per pass; ~20 ms of GPU time per figure
    cold_ms, cold_best, _, _ = time_pass(sets, passes, 10, launch)
    cold_ms /= len(sets)
    cold_best /= len(sets)
    warm_ms, warm_best, _, _ = time_pass(sets[:1] * 16, passes, 10, launch)
    warm_ms /= 16
    warm_best /= 16
    warm_tf = flops / (warm_ms * 1e-3) / 1e12
    cold_tf = flops / (cold_ms * 1e-3) / 1e12
    moved = 63012864  # q + K/V pages + out + lse of one call
    roof = {"bound": "mfma", "achieved": warm_tf, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
            "frac": warm_tf / BF16_PEAK_TFLOPS, "algorithmic_flops_per_launch": flops,
            "avg_launch_us": warm_ms * 1e3, "kernel": "chunk_kernel (warm: inputs resident in the Infinity Cache)",
            "traffic": None}
    ent = traffic_entry("chunked_denoise", "chunk_kernel")
    if ent:
        roof["traffic"] = ent["fetch_bytes_per_launch"] + ent["write_bytes_per_launch"]
        roof["traffic_fetch"] = ent["fetch_bytes_per_launch"]
        roof["traffic_write"] = ent["write_bytes_per_launch"]
        if ent.get("mfma_flop_per_launch"):
            # SQ_INSTS_VALU_MFMA_MOPS_BF16 x 512 of the profiled dispatches
            roof["counted_mfma_flop_per_launch"] = ent["mfma_flop_per_launch"]
    if mfma_tflops:
        roof["measured_peak_tflops"] = mfma_tflops
        roof["frac_of_measured_peak"] = warm_tf / mfma_tflops
    return {"workload": "chunked_denoise", "flop_per_call": flops,
            "tflops_cold": cold_tf, "tflops_warm": warm_tf, "ms_cold": cold_ms, "ms_warm": warm_ms,
            "ms_cold_best": cold_best, "ms_warm_best": warm_best,
            "frac_of_bf16_peak_warm": warm_tf / BF16_PEAK_TFLOPS,
            # the call reads and writes 63,012,864 B: AI = 204.5 FLOP/B, so cold
            # it is capped at min(peak, AI x 8 TB/s) = 1,636 TFLOP/s
            "frac_of_roofline_cold": cold_tf / min(BF16_PEAK_TFLOPS, flops / moved * HBM_PEAK_GBS / 1e3),
            "roofline": roof}


class _WriteCall:
    """One pa_write_kv call with fixed tensors, launchable like PreparedAttend."""

    def __init__(self, k_new, v_new, table, ctx, q_lens, k_cache, v_cache, max_q_len):
        self.args = (k_new, v_new, table, ctx, q_lens, k_cache, v_cache)
        self.max_q_len = max_q_len

    def launch(self, stream):
        import paged_kv_cache_attend_amd as pk
        pk.write_kv(*self.args, max_q_len=self.max_q_len, stream=stream)


def append_secondary(dev, steps, launch="graph"):
    """pa_write_kv on the Qwen3-8B-shaped batch (16 slots x 2303 tokens, 8 KV
    heads): a whole-prompt append (every token new; bytes = new rows read +
    cache rows written) and a one-token-per-slot decode append (latency)."""
    import torch
    from paged_kv_cache_attend_amd import inputs
    p = inputs.qwen3_short_decode(num_layers=1)
    hkv, d = p.num_kv_heads, p.head_dim
    rows = int(p.ctx_lens.sum())
    ss = np.random.SeedSequence(inputs.SEED_BASE + 900)
    kn = inputs.bits_to_torch_bf16(inputs.normal_bf16(inputs.child_seed(ss, 0), (rows, hkv, d)), dev)
    vn = inputs.bits_to_torch_bf16(inputs.normal_bf16(inputs.child_seed(ss, 1), (rows, hkv, d)), dev)
    kc = torch.zeros((p.num_blocks, hkv, p.block_size, d), dtype=torch.bfloat16, device=dev)
    vc = torch.zeros_like(kc)
    table = torch.from_numpy(p.block_table.astype(np.int32)).to(dev)
    ctx = torch.from_numpy(p.ctx_lens.astype(np.int32)).to(dev)
    ones = torch.ones_like(ctx)
    prefill = _WriteCall(kn, vn, table, ctx, ctx, kc, vc, int(p.ctx_lens.max()))
    decode = _WriteCall(kn[:p.num_seqs], vn[:p.num_seqs], table, ctx, ones, kc, vc, 1)
    reps = max(steps // 4, 20)
    pre_ms, _, _, _ = time_pass([prefill], reps, 2, launch)
    dec_ms, _, _, _ = time_pass([decode] * 36, reps, 2, launch)
    moved = 4 * rows * hkv * d * 2  # K and V: read the new row, write the page slot
    return {"workload": "qwen3_8b_short_decode prompt and decode appends (one layer per call)",
            "prompt_rows": rows, "prompt_bytes_moved": moved, "prompt_us": pre_ms * 1e3,
            "prompt_gbs": moved / (pre_ms * 1e-3) / 1e9,
            "prompt_frac_of_hbm_peak": moved / (pre_ms * 1e-3) / 1e9 / HBM_PEAK_GBS,
            "decode_append_us_per_layer": dec_ms * 1e3 / 36,
            "parity": "bit-exact against the oracle scatter in the GPU tests"}


def quant_secondary(dev, steps, launch, bf16_us_per_layer):
    """Decode of the Qwen3-8B-shaped batch (16 x 2303 keys, 32/8 heads) over
    FP8, q8_0 and q4_0 pages, 36 distinct layers of random codes: microseconds
    per layer, GB/s over the bytes the format reads (codes + group scales),
    and the trade of section 8.4.2, Delta T = Delta D / beta - T_c, against the
    bf16 time measured above."""
    import torch
    import paged_kv_cache_attend_amd as pk
    from paged_kv_cache_attend_amd import inputs
    p = inputs.qwen3_short_decode(num_layers=1)
    nb, hkv = p.num_blocks, p.num_kv_heads
    q = inputs.bits_to_torch_bf16(inputs.normal_bf16(np.random.SeedSequence(inputs.SEED_BASE + 4200),
                                                     (p.total_q, p.num_q_heads, p.head_dim)), dev)
    table = torch.from_numpy(p.block_table.astype(np.int32)).to(dev)
    ctx = torch.from_numpy(p.ctx_lens.astype(np.int32)).to(dev)
    ql = torch.from_numpy(p.q_lens.astype(np.int32)).to(dev)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:2], dtype=torch.float32, device=dev)
    shape = pk.make_shape(p.num_seqs, p.total_q, p.num_q_heads, hkv, p.max_blocks_per_seq, 1,
                          p.max_ctx_len, nb)
    ws = torch.empty(max(pk.workspace_size(shape), 1), dtype=torch.uint8, device=dev)
    pk.workspace_init(shape, ws)
    tokens = int(p.ctx_lens.sum())
    bf16_bytes = tokens * hkv * 512
    distinct = 36
    res = {}
    for name, fmt, per_tok in (("fp8", pk.KV_FP8_E4M3, 256), ("q8_0", pk.KV_Q8_0, 272),
                               ("q4_0", pk.KV_Q4_0, 144)):
        gen = torch.Generator(device=dev)
        gen.manual_seed(inputs.SEED_BASE + 4100 + fmt)
        calls = []
        keep = []
        for _ in range(distinct):
            c = pk.QuantCache.empty(fmt, nb, hkv, dev, 1.0 / 64, 1.0 / 256)
            for codes in (c.k_codes, c.v_codes):
                if fmt == pk.KV_Q8_0:
                    codes.copy_(torch.randint(-127, 128, codes.shape, generator=gen, device=dev, dtype=torch.int8))
                else:
                    r = torch.randint(0, 256, codes.shape, generator=gen, device=dev, dtype=torch.int32)
                    if fmt == pk.KV_FP8_E4M3:
                        r = torch.where((r & 0x7F) == 0x7F, r & 0xF7, r)   # no NaN codes
                    codes.copy_(r.to(torch.uint8))
            for sc in (c.k_scales, c.v_scales):
                if sc is not None:
                    lo, hi = (0.004, 0.0157) if fmt == pk.KV_Q8_0 else (0.05, 0.25)
                    sc.copy_((torch.rand(sc.shape, generator=gen, device=dev) * (hi - lo) + lo).half())
            keep.append(c)
            calls.append(pk.attend_kv(q, c, table, ctx, ql, float(p.scale), out, lse, max_q_len=1,
                                      max_ctx_len=p.max_ctx_len, workspace=ws, prepared=True))
        ms, best, _, _ = time_pass(calls, max(steps // 4, 20), 3, launch)
        us = ms * 1e3 / distinct
        moved = tokens * hkv * per_tok
        beta = bf16_bytes / (bf16_us_per_layer * 1e-6)          # bf16's achieved read rate
        saved_read_us = (bf16_bytes - moved) / beta * 1e6       # Delta D / beta
        res[name] = {"us_per_layer": us, "us_per_layer_best": best * 1e3 / distinct, "bytes_per_layer": moved,
                     "gbs": moved / (us * 1e-6) / 1e9, "frac_of_hbm_peak": moved / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
                     "speedup_vs_bf16": bf16_us_per_layer / us,
                     "delta_T_us": bf16_us_per_layer - us, "delta_D_over_beta_us": saved_read_us,
                     "T_c_us": saved_read_us - (bf16_us_per_layer - us),
                     "partitions": calls[0].num_partitions}
        del calls, keep
        torch.cuda.empty_cache()
    res["workload"] = "qwen3_8b_short_decode, 36 distinct layers of random codes (drawn on the device)"
    res["parity"] = "against the FP64 oracle over decoded pages in the GPU tests"
    return res


def shared_prefix_config(dev, steps, launch, ceiling_gbs=None):
    """The shared-prefix long decode (10 slots x 8447 keys, the first 6144
    one physical copy, 32/8 heads), 36 distinct layers, through pa_attend and
    through prefix-grouped decode (pa_attend_prefix).  The headline figure is
    GB/s over the distinct bytes a layer must read (shared pages once)."""
    import torch
    import paged_kv_cache_attend_amd as pk
    from paged_kv_cache_attend_amd import inputs
    nl = 36
    p = inputs.qwen3_shared_prefix_decode(num_layers=nl)
    layers = device_layers(p, dev, nl, inputs.SEED_BASE + 3300)
    plen = p.shared_prefix_blocks * p.block_size
    gs = torch.tensor([0, p.num_seqs], dtype=torch.int32, device=dev)
    pl = torch.tensor([plen], dtype=torch.int32, device=dev)
    base, grouped = [], []
    ws_b = ws_g = None
    for t in layers:
        out = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device=dev)
        c = pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                              float(p.scale), out, lse, max_q_len=1, max_ctx_len=p.max_ctx_len, workspace=ws_b)
        ws_b = c.workspace
        base.append(c)
        g = pk.attend_prefix(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                             float(p.scale), out, lse, group_start=gs, prefix_len=pl, max_members=p.num_seqs,
                             max_prefix_len=plen, min_prefix_len=plen, max_ctx_len=p.max_ctx_len,
                             workspace=ws_g, prepared=True)
        ws_g = g.keep[-1]
        grouped.append(g)
    reps = max(steps // 4, 20)
    b_ms, b_best, _, _ = time_pass(base, reps, 3, launch)
    g_ms, g_best, _, _ = time_pass(grouped, reps, 3, launch)
    b_us, g_us = b_ms * 1e3 / nl, g_ms * 1e3 / nl
    unique = p.kv_bytes_unique()
    logical = p.kv_bytes_read()
    best = min(b_us, g_us)
    return {"workload": "qwen3_8b_shared_prefix_decode: 36 distinct layers (values drawn on the device), "
                        "10 slots x 8447 keys, 6144 shared, 32/8 heads",
            "unique_bytes_per_layer": unique, "logical_bytes_per_layer": logical,
            "pa_attend_us_per_layer": b_us, "pa_attend_us_per_layer_best": b_best * 1e3 / nl,
            "pa_attend_prefix_us_per_layer": g_us, "pa_attend_prefix_us_per_layer_best": g_best * 1e3 / nl,
            "pa_attend_gbs_unique": unique / (b_us * 1e-6) / 1e9,
            "pa_attend_prefix_gbs_unique": unique / (g_us * 1e-6) / 1e9,
            "pa_attend_effective_gbs": logical / (b_us * 1e-6) / 1e9,
            "speedup_prefix_vs_attend": b_us / g_us,
            "partitions": base[0].num_partitions,
            "roofline": hbm_roofline(unique, best, "the faster of pa_attend and pa_attend_prefix per layer "
                                     "(graph replay of 36 layers), on unique bytes", ceiling_gbs,
                                     path="pa_attend_prefix" if g_us < b_us else "pa_attend"),
            "parity": "against the FP64 oracle (layer 7 and sampled slots) and pa_attend in the GPU tests"}


def ragged_config(dev, steps, launch, ceiling_gbs=None):
    """The ragged mixed decode batch (64 slots of U[1, 8447] keys + 4 zombie
    slots, 32/8 heads, 512-token partitions): one layer (about 1.2 GB of
    pages, far beyond the Infinity Cache) per launch.  The split and its
    merge run in one launch (the last partition of each (slot, KV head)
    merges); the merge alone is also timed as the stand-alone pa_combine over
    the same partials, which is what a separate merge pass would cost."""
    import torch
    import paged_kv_cache_attend_amd as pk
    from paged_kv_cache_attend_amd import inputs
    p = inputs.ragged_mixed_decode()
    t = device_layers(p, dev, 1, inputs.SEED_BASE + 4400)[0]
    out = torch.empty_like(t["q"])
    lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device=dev)
    c = pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                          float(p.scale), out, lse, max_q_len=1, max_ctx_len=p.max_ctx_len,
                          partition_size=p.partition_size)
    reps = max(steps // 2, 40)
    ms, best, _, _ = time_pass([c], reps, 3, launch)
    c_auto = pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                               float(p.scale), out, lse, max_q_len=1, max_ctx_len=p.max_ctx_len)
    ms_auto, _, _, _ = time_pass([c_auto], reps, 3, launch)
    P = c.num_partitions
    rows = p.total_q * p.num_q_heads
    po = torch.zeros((P, rows, p.head_dim), dtype=torch.float32, device=dev)
    plse = torch.randn((P, rows), dtype=torch.float32, device=dev)
    cout = torch.empty((rows, p.head_dim), dtype=torch.bfloat16, device=dev)
    clse = torch.empty(rows, dtype=torch.float32, device=dev)

    class _Comb:
        def launch(self, s):
            pk.combine(po, plse, cout, clse, stream=s)

    comb_ms, _, _, _ = time_pass([_Comb()], reps, 3, launch)
    kv = p.kv_bytes_read()
    us = ms * 1e3
    return {"workload": "ragged_mixed_decode: 64 slots U[1, 8447] + 4 zombies, 32/8 heads, "
                        "512-token partitions (values drawn on the device)",
            "kv_bytes": kv, "partitions": P, "split_and_merge_us": us, "split_and_merge_us_best": best * 1e3,
            "gbs": kv / (us * 1e-6) / 1e9, "auto_partition_us": ms_auto * 1e3,
            "auto_partitions": c_auto.num_partitions,
            "merge_alone_us": comb_ms * 1e3,
            "merge_alone_note": f"pa_combine over {P} partials x {rows} rows x 128 (the same partials the fused "
                                "merge reads), launched by itself",
            "partial_bytes": P * rows * (p.head_dim + 1) * 4,
            "roofline": hbm_roofline(kv, us, "decode_kernel<4> with the fused merge, one launch", ceiling_gbs),
            "parity": "against the FP64 oracle in full in the GPU tests (test_ragged_mixed_decode_full_size)"}


def causal_secondary(dev, steps, launch, bf16_decode_us=None):
    """Causal multi-token queries (section 8.2.3 and 8.5 of the chapter):
    - the page's chunked-prefill example, the last 512-token chunk of an
      8192-token prompt, 32/8 heads: TFLOP/s on the visible (query, key)
      pairs (4 D FLOP per pair and query head), 16 resident copies rotated;
    - speculative verification of 5 and 8 tokens per request on the
      Qwen3-8B short-decode batch (16 x 2303 keys), 36 distinct layers:
      microseconds per layer and GB/s over the pages read."""
    import torch
    import paged_kv_cache_attend_amd as pk
    from paged_kv_cache_attend_amd import inputs
    res = {}
    p = inputs.chunked_prefill()
    m, n = int(p.q_lens[0]), int(p.ctx_lens[0])
    pairs = m * (n - m) + m * (m + 1) // 2
    flops = 4 * p.head_dim * p.num_q_heads * pairs
    sets = []
    for t in device_layers(p, dev, 16, inputs.SEED_BASE + 6600):
        out = torch.empty_like(t["q"])
        lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device=dev)
        sets.append(pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                                      float(p.scale), out, lse, max_q_len=m, max_ctx_len=n, causal=True))
    ms, best, _, _ = time_pass(sets, max(steps // 8, 20), 3, launch)
    us = ms * 1e3 / len(sets)
    res["chunked_prefill"] = {"workload": "chunked_prefill_c512_h7680: 1 request, 512 new tokens after 7680 "
                                          "cached, 32/8 heads, causal (values drawn on the device)",
                              "pairs": pairs, "flop_per_call": flops, "us_per_call": us,
                              "us_per_call_best": best * 1e3 / len(sets),
                              "tflops": flops / (us * 1e-6) / 1e12,
                              "frac_of_bf16_peak": flops / (us * 1e-6) / 1e12 / BF16_PEAK_TFLOPS}
    del sets
    torch.cuda.empty_cache()
    for mt in (5, 8):
        p = inputs.speculative_verify(mt)
        calls = []
        for t in device_layers(p, dev, 36, inputs.SEED_BASE + 6700 + mt):
            out = torch.empty_like(t["q"])
            lse = torch.empty(t["q"].shape[:2], dtype=torch.float32, device=dev)
            calls.append(pk.PreparedAttend(t["q"], t["k"], t["v"], t["block_table"], t["ctx_lens"], t["q_lens"],
                                           float(p.scale), out, lse, max_q_len=mt, max_ctx_len=p.max_ctx_len,
                                           causal=True))
        ms, best, _, _ = time_pass(calls, max(steps // 4, 20), 3, launch)
        us = ms * 1e3 / len(calls)
        kv = p.kv_bytes_read()
        res[f"speculative_verify_m{mt}"] = {
            "workload": f"16 requests x 2303 keys, {mt} new tokens each, 32/8 heads, causal, 36 distinct layers",
            "us_per_layer": us, "us_per_layer_best": best * 1e3 / len(calls),
            "kv_gbs": kv / (us * 1e-6) / 1e9, "frac_of_hbm_peak": kv / (us * 1e-6) / 1e9 / HBM_PEAK_GBS,
            "vs_one_token_decode": (us / bf16_decode_us) if bf16_decode_us else None}
        del calls
        torch.cuda.empty_cache()
    res["parity"] = "against the FP64 oracle in the GPU tests (test_chunked_prefill_page_example_full_size, " \
                    "test_speculative_verification)"
    return res


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on exactly one GPU (asked for {args.gpus}); multi-GPU runs are not part "
              "of this build", file=sys.stderr)
        sys.exit(2)
    if args.mode == "copy":
        copy_mode(args.steps)
        return
    import torch
    from paged_kv_cache_attend_amd import inputs
    import paged_kv_cache_attend_amd as pk
    pk.load()  # fail loudly if the HIP library is missing
    dev = torch.device("cuda:0")
    # All work runs on one non-default stream (graph capture needs one).
    torch.cuda.set_stream(torch.cuda.Stream(device=dev))
    if args.config not in inputs.CONFIGS or args.config in ("tiny_decode",):
        raise SystemExit(f"unknown or untimeable config {args.config}")
    problem = inputs.CONFIGS[args.config]()
    ps = problem.partition_size if args.partition_size is None else args.partition_size
    log(f"config {problem.name}: {problem.num_layers} layers, {problem.num_seqs} slots, "
        f"Hq {problem.num_q_heads} / Hkv {problem.num_kv_heads}, max ctx {problem.max_ctx_len}")

    t_setup = time.perf_counter()
    layers, ref, cpu_s, cpu_bytes = build_decode(problem, dev, not args.no_cpu_baseline, args.cpu_budget_s)
    calls, outs, lses = prepare_calls(problem, layers, ps)
    log(f"setup {time.perf_counter() - t_setup:.1f}s; partitions per slot {calls[0].num_partitions}")

    decode = problem.max_q_len == 1
    ms, best_ms, wall_ms, trials = time_pass(calls, args.steps, args.warmup, args.launch)
    log(f"timed: {ms * 1e3 / len(calls):.2f} us per layer (median of {len(trials)} trials)")
    eager_ms = None
    if args.launch == "graph" and not args.quick:
        eager_ms, _, _, _ = time_pass(calls, max(10, args.steps // 4), 2, "eager", trials=1)
    per_call_ms = ms / len(calls) if args.quick else time_kernel_launches(calls, max(5, args.steps // 10))

    kv_read = problem.kv_bytes_read() * problem.num_layers
    kv_unique = problem.kv_bytes_unique() * problem.num_layers
    flops = 4 * int((problem.q_lens.astype(np.int64) * problem.ctx_lens).sum()) * problem.num_q_heads \
        * problem.head_dim * problem.num_layers
    ceiling = mfma = None
    if not args.quick:
        mfma = mfma_ceiling()
        if decode:
            ceiling = read_ceiling(problem, layers, args.steps, args.launch)
            log(f"read ceiling {ceiling['gbs']:.0f} GB/s; MFMA {mfma['tflops']:.0f} TFLOP/s")
    if decode:
        headline_bytes = kv_unique  # each distinct byte read once (equals kv_read without sharing)
        value = headline_bytes / (ms * 1e-3) / 1e9
        unit = "GB/s"
        per_launch_bytes = headline_bytes / len(calls)
        achieved = per_launch_bytes / (per_call_ms * 1e-3) / 1e9
        kname = f"decode_kernel<{problem.num_q_heads // problem.num_kv_heads}>"
        tr = measured_traffic(problem.name, kname)
        roofline = {"bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                    "frac": achieved / HBM_PEAK_GBS,
                    "traffic": None if tr is None else tr[0] + tr[1],
                    "traffic_fetch": None if tr is None else tr[0],
                    "traffic_write": None if tr is None else tr[1],
                    "algorithmic_bytes_per_launch": per_launch_bytes,
                    "kernel": kname + " (split-KV decode with the LSE merge fused), one launch per layer",
                    "avg_launch_us": per_call_ms * 1e3,
                    "timing": "HIP events around back-to-back launches on the launch stream"}
        if ceiling:
            roofline["measured_read_ceiling_gbs"] = ceiling["gbs"]
            roofline["frac_of_measured_read_ceiling"] = achieved / ceiling["gbs"]
    else:
        value = flops / (ms * 1e-3) / 1e12
        unit = "TFLOP/s"
        achieved = (flops / len(calls)) / (per_call_ms * 1e-3) / 1e12
        tr = measured_traffic(problem.name, "chunk_kernel")
        roofline = {"bound": "mfma", "achieved": achieved, "peak": BF16_PEAK_TFLOPS, "unit": "TFLOP/s",
                    "frac": achieved / BF16_PEAK_TFLOPS,
                    "traffic": None if tr is None else tr[0] + tr[1],
                    "algorithmic_flops_per_launch": flops / len(calls), "kernel": "chunk_kernel",
                    "avg_launch_us": per_call_ms * 1e3}
        if mfma:
            roofline["measured_peak_tflops"] = mfma["tflops"]
            roofline["frac_of_measured_peak"] = achieved / mfma["tflops"]

    par = parity(problem, outs, lses, ref) if ref else None
    cpu = None
    if ref and cpu_s > 0:
        ncores = 1
        if decode:
            cpu = {"value": cpu_bytes / cpu_s / 1e9, "unit": "GB/s", "cores": ncores, "kind": "oracle",
                   "sample": f"{len(ref)} of {problem.num_layers} layers, all {problem.num_seqs} slots, "
                             f"FP64 NumPy oracle, 1 BLAS thread, {cpu_s:.1f}s"}
        else:
            cpu = {"value": flops / problem.num_layers * len(ref) / cpu_s / 1e12, "unit": "TFLOP/s",
                   "cores": ncores, "kind": "oracle", "sample": f"{len(ref)} call(s), 1 BLAS thread, {cpu_s:.1f}s"}
        cpu["cpu_model"] = cpu_model()
        cpu["host_cpus_available"] = len(os.sched_getaffinity(0))

    main_workload = decode and problem.name == "qwen3_8b_short_decode"
    del layers
    calls_keep = calls
    secondary = None
    if main_workload and not args.no_chunk:
        log("chunk workload")
        secondary = chunk_secondary(dev, args.steps, args.launch, mfma["tflops"] if mfma else None)
    configs = {}
    if main_workload and not args.no_prefix:
        log("shared-prefix workload")
        configs["shared_prefix"] = shared_prefix_config(dev, args.steps, args.launch,
                                                        ceiling["gbs"] if ceiling else None)
        torch.cuda.empty_cache()
    if main_workload and not args.no_ragged:
        log("ragged workload")
        configs["ragged"] = ragged_config(dev, args.steps, args.launch, ceiling["gbs"] if ceiling else None)
        torch.cuda.empty_cache()
    causal = None
    if main_workload and not args.no_causal:
        log("causal multi-token workloads")
        causal = causal_secondary(dev, args.steps, args.launch, ms / len(calls_keep) * 1e3)
    append = None
    if main_workload and not args.no_append:
        append = append_secondary(dev, args.steps, args.launch)
    quant = None
    if main_workload and not args.no_quant:
        log("quantised pages")
        quant = quant_secondary(dev, args.steps, args.launch, ms / len(calls_keep) * 1e3)

    line = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": problem.name,
            "layers": problem.num_layers,
            "batch": problem.num_seqs,
            "ctx_len_max": problem.max_ctx_len,
            "q_heads": problem.num_q_heads,
            "kv_heads": problem.num_kv_heads,
            "head_dim": problem.head_dim,
            "block_size": problem.block_size,
            "partition_size": ps,
            "partitions": calls_keep[0].num_partitions,
            "launch": args.launch,
            "accumulate": "fp32",
            "pv_weights": ("bf16 hi + lo pair per softmax weight (the fp32 weight to 2^-15)" if decode
                           else "bf16 softmax weights, output divided by their sum"),
        },
        "timing": {"trials": len(trials), "steps_per_trial": args.steps, "ms_per_step_median": ms,
                   "ms_per_step_best": best_ms, "ms_per_step_trials": trials},
        "frac_of_hbm_peak": (value / HBM_PEAK_GBS) if decode else None,
        "measured_read_ceiling": ceiling,
        "measured_mfma_ceiling": mfma,
        "kv_bytes_per_step": kv_read if decode else None,
        "kv_unique_bytes_per_step": kv_unique if decode else None,
        "effective_gbs": (kv_read / (ms * 1e-3) / 1e9) if decode else None,
        "eager_ms_per_step": eager_ms,
        "wall_ms_per_step": wall_ms,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": par,
        "chunk": secondary,
        "configs": configs or None,
        "causal": causal,
        "append": append,
        "quantised": quant,
        "source_hash": kernel_source_hash(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
