"""Plain float64 softmax attention of new query tokens against a block-paged KV cache.

TEST INFRASTRUCTURE ONLY -- imported by tests, the smoke check and the CPU
baseline of the benchmark, never by the product path.  Shares no code with the
HIP library.

What is computed, and where it is stated
----------------------------------------
* Paging is pure re-addressing.  The inference-optimisation chapter
  ("Chapter 8: Inference optimisation", section 8.3.1 "reservation,
  fragmentation and paged allocation", Fig. 8-10) splits a sequence into
  fixed-size logical blocks; a per-request block table maps each logical
  block to a physical block anywhere in the pool, and attention recovers the
  logical order through that table.  So the oracle first gathers each
  request's keys and values in logical order, one block at a time, and then
  applies the textbook definition of softmax attention to the gathered rows.
* Decode: a new token attends to every cached token of its own request
  (same chapter, sections 8.1.1 and 8.2.1: each request still reads its own
  KV even when weights are shared across the batch).
* Chunked denoising: a chunk at noise level d attends to the KV that earlier
  chunks left at the same level d (PhysisServe teardown page, section "why
  autoregressive denoising can be pipelined", the update
  z_c^(d-1) = Phi_d(z_c^(d), K_<c^(d), cond_c)).  Within the chunk the
  reading adopted is a full (bidirectional) mask over all ctx_len keys.
* Finished ("zombie") slots ride along in an in-flight batch but their
  results are never used (Photon pipelined-decoding page, section 5,
  "zombies: finalise early, release late"); a slot with ctx_len == 0 or
  q_len == 0 therefore produces nothing here.

Readings where the pages are silent (layout, head grouping, whether ctx_len
includes the new tokens, the LSE convention) are listed in the design notes;
in short:

* cache layout ``[num_blocks][num_kv_heads][block_size][head_dim]`` of bf16
  bit patterns, one array for K and one for V;
* query head h reads KV head ``h // (Hq // Hkv)``;
* ``ctx_lens[r]`` counts every visible key, including the new tokens' own;
* ``lse = M + ln(sum_j exp(s_j - M))`` in natural log over the *scaled*
  scores;
* the causal variant lets row i of a request with m new tokens see keys
  ``[0, n - m + i]`` (chunked prefill, section 8.2.3, Figs. 8-8 and 8-9).

Everything is float64.  bf16 -> float64 widening is exact, so the only
rounding is the float64 arithmetic itself.
"""

from __future__ import annotations

import math

import numpy as np


def bf16_bits_to_f64(bits) -> np.ndarray:
    """Widen bf16 bit patterns (uint16) to float64 exactly.

    A bf16 value is the top half of an IEEE binary32 word, so placing the
    16 bits in the high half of a 32-bit word gives the same number as fp32,
    which float64 then represents exactly.
    """
    b = np.asarray(bits, dtype=np.uint16)
    with np.errstate(invalid="ignore"):  # NaN payloads widen to NaN
        return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def gather_request_kv(cache_bits, table_row, n: int, kv_head: int, block_size: int = 16) -> np.ndarray:
    """Keys (or values) of one request and one KV head, in logical order.

    Logical position j lives in logical block ``j // block_size`` at slot
    ``j % block_size``; the block table row names the physical block that
    holds each logical block (Fig. 8-10: logical blocks 0, 1, 2 may sit in
    physical blocks 2, 0, 3).  Only the first ``n`` positions exist; the
    rest of the last block is unused tail (section 8.3.1: at most
    ``block_size - 1`` wasted slots) and is never read.

    The cache holds bf16 bit patterns (uint16), or values already widened
    to float64 (pages decoded from a quantised format), which pass through
    unchanged.

    Returns float64 ``[n][head_dim]``.
    """
    rows = []
    remaining = int(n)
    logical = 0
    while remaining > 0:
        phys = int(table_row[logical])
        take = min(block_size, remaining)
        rows.append(np.asarray(cache_bits[phys, kv_head, :take, :]))
        remaining -= take
        logical += 1
    if not rows:
        return np.zeros((0, cache_bits.shape[-1]), dtype=np.float64)
    block = np.concatenate(rows, axis=0)
    if block.dtype == np.float64:
        return block
    return bf16_bits_to_f64(block)


def _query_offsets(q_lens) -> list[int]:
    """Row of each request's first new token: exclusive running sum of q_lens."""
    offs = []
    acc = 0
    for m in q_lens:
        offs.append(acc)
        acc += int(m)
    return offs


def _softmax_attend(scores: np.ndarray, values: np.ndarray):
    """Textbook softmax attention of each score row over its keys.

    ``scores`` is ``[rows][keys]`` (masked entries are -inf), ``values`` is
    ``[keys][dim]``.  Returns (normalised output ``[rows][dim]``, natural-log
    LSE ``[rows]``).  The maximum is subtracted before ``exp`` purely to
    keep float64 in range; it cancels exactly in the ratio.
    """
    M = scores.max(axis=1)
    W = np.exp(scores - M[:, None])
    Z = W.sum(axis=1)
    out = (W @ values) / Z[:, None]
    lse = M + np.log(Z)
    return out, lse


def attend_fp64(q_bits, k_bits, v_bits, block_table, ctx_lens, q_lens, scale,
                num_kv_heads: int, block_size: int = 16, causal: bool = False,
                seqs=None):
    """Attention of every new query row against its request's paged KV.

    Parameters
    ----------
    q_bits : uint16 ``[total_q][Hq][D]`` bf16 bit patterns, rows packed by
        request in slot order.
    k_bits, v_bits : uint16 ``[num_blocks][Hkv][block_size][D]``.
    block_table : int ``[num_seqs][max_blocks_per_seq]``.
    ctx_lens, q_lens : int ``[num_seqs]``.
    scale : the fp32 softmax scale; widened to float64 unchanged.
    causal : if True, row i of a request with m new tokens and n keys sees
        keys ``[0, n - m + i]`` only.
    seqs : optional iterable of request indices to evaluate (others are left
        as NaN and not marked written) -- used to sample large problems.

    Returns
    -------
    out : float64 ``[total_q][Hq][D]`` (NaN where nothing is written)
    lse : float64 ``[total_q][Hq]``   (NaN where nothing is written)
    written : bool ``[total_q]`` -- rows that belong to an active request
    """
    q_bits = np.asarray(q_bits)
    total_q, Hq, D = q_bits.shape
    Hkv = int(num_kv_heads)
    if Hq % Hkv != 0:
        raise ValueError("query heads must be a multiple of KV heads")
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    offs = _query_offsets(q_lens)

    out = np.full((total_q, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((total_q, Hq), np.nan, dtype=np.float64)
    written = np.zeros(total_q, dtype=bool)

    which = range(len(ctx_lens)) if seqs is None else seqs
    for r in which:
        n = int(ctx_lens[r])
        m = int(q_lens[r])
        if n <= 0 or m <= 0:
            continue  # finished / empty slot: produces nothing
        row0 = offs[r]
        mask = None
        if causal:
            i = np.arange(m)[:, None]
            j = np.arange(n)[None, :]
            mask = j > (n - m + i)
        for g in range(Hkv):
            K = gather_request_kv(k_bits, block_table[r], n, g, block_size)
            V = gather_request_kv(v_bits, block_table[r], n, g, block_size)
            for h in range(g * G, (g + 1) * G):
                Q = bf16_bits_to_f64(q_bits[row0:row0 + m, h, :])
                S = scale64 * (Q @ K.T)
                if mask is not None:
                    S = np.where(mask, -np.inf, S)
                o, l = _softmax_attend(S, V)
                out[row0:row0 + m, h, :] = o
                lse[row0:row0 + m, h] = l
        written[row0:row0 + m] = True
    return out, lse, written


def attend_key_range_fp64(q_bits, k_bits, v_bits, block_table, ctx_lens, q_lens, scale,
                          num_kv_heads: int, key_lo: int, key_hi: int,
                          block_size: int = 16):
    """Partial attention restricted to logical keys ``[key_lo, min(key_hi, n))``.

    This is one split-KV partition: the normalised output and LSE of the
    softmax over that key range alone.  An empty range -- including every
    range of a request with no keys -- gives ``lse = -inf`` and an output of
    NaN (its weight in a merge is zero, so its output must never be read).
    ``written`` marks rows of requests that have keys.
    """
    q_bits = np.asarray(q_bits)
    total_q, Hq, D = q_bits.shape
    Hkv = int(num_kv_heads)
    G = Hq // Hkv
    scale64 = float(np.float32(scale))
    offs = _query_offsets(q_lens)
    out = np.full((total_q, Hq, D), np.nan, dtype=np.float64)
    lse = np.full((total_q, Hq), np.nan, dtype=np.float64)
    written = np.zeros(total_q, dtype=bool)
    for r in range(len(ctx_lens)):
        n = int(ctx_lens[r])
        m = int(q_lens[r])
        row0 = offs[r]
        if m <= 0:
            continue
        if n <= 0:
            lse[row0:row0 + m, :] = -np.inf
            continue
        lo, hi = int(key_lo), min(int(key_hi), n)
        written[row0:row0 + m] = True
        if hi <= lo:
            lse[row0:row0 + m, :] = -np.inf
            continue
        for g in range(Hkv):
            K = gather_request_kv(k_bits, block_table[r], n, g, block_size)[lo:hi]
            V = gather_request_kv(v_bits, block_table[r], n, g, block_size)[lo:hi]
            for h in range(g * G, (g + 1) * G):
                Q = bf16_bits_to_f64(q_bits[row0:row0 + m, h, :])
                o, l = _softmax_attend(scale64 * (Q @ K.T), V)
                out[row0:row0 + m, h, :] = o
                lse[row0:row0 + m, h] = l
    return out, lse, written


def combine_fp64(partial_out, partial_lse):
    """Merge split-KV partials by their log-sum-exp weights.

    For one row with partials (o_p, lse_p): the softmax over the union of
    disjoint key ranges weighs partition p by exp(lse_p) relative to the
    others, so with M = max_p lse_p,
        lse = M + ln(sum_p exp(lse_p - M)),
        o   = sum_p exp(lse_p - M) o_p / sum_p exp(lse_p - M).
    Partials with lse_p = -inf weigh zero and their outputs are not read.
    A row whose partials are all -inf is left untouched (returned as NaN,
    ``touched`` False).

    ``partial_out`` is ``[P][rows][D]``, ``partial_lse`` is ``[P][rows]``.
    Returns (out ``[rows][D]``, lse ``[rows]``, touched ``[rows]``).
    """
    po = np.asarray(partial_out, dtype=np.float64)
    pl = np.asarray(partial_lse, dtype=np.float64)
    P, rows, D = po.shape
    out = np.full((rows, D), np.nan, dtype=np.float64)
    lse = np.full(rows, np.nan, dtype=np.float64)
    touched = np.zeros(rows, dtype=bool)
    for r in range(rows):
        live = [p for p in range(P) if pl[p, r] != -math.inf]
        if not live:
            continue
        M = max(pl[p, r] for p in live)
        wsum = 0.0
        acc = np.zeros(D, dtype=np.float64)
        for p in live:
            w = math.exp(pl[p, r] - M)
            wsum += w
            acc += w * po[p, r]
        out[r] = acc / wsum
        lse[r] = M + math.log(wsum)
        touched[r] = True
    return out, lse, touched
