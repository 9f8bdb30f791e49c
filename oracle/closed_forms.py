"""Integer identities of paged KV storage stated on the inference-optimisation page.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources, all on the page "Chapter 8: Inference optimisation":
* section 8.1.2 (storage needs of weights, KV and runtime buffers): KV per
  token is 2 (K and V) x layers x KV heads x head dim x bytes per element;
  for Qwen3-8B that is 2 x 36 x 8 x 128 x 2 = 147,456 bytes = 144 KiB,
  and with 16-token blocks a 2048 + 255 token request occupies 2304 slots;
* section 8.3.1 (paged allocation): a length-L sequence needs ceil(L/p)
  blocks of p tokens and wastes p*ceil(L/p) - L <= p - 1 slots;
* section 8.3.2 (branch sharing, copy-on-write): b requests sharing a
  prefix hold one copy of the prefix blocks plus their own private blocks;
  references count every table entry, physical blocks count each block once;
* section 8.2.3 (chunked prefill): a new chunk of c tokens after h cached
  tokens forms c*h + c(c+1)/2 causal query-key pairs.
"""

from __future__ import annotations


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, elem_bytes: int) -> int:
    """K and V bytes one token adds across all layers."""
    return 2 * layers * kv_heads * head_dim * elem_bytes


def blocks_needed(length: int, block_size: int) -> int:
    """Number of p-token blocks that hold a length-L sequence: ceil(L / p)."""
    return -(-int(length) // int(block_size))


def tail_waste(length: int, block_size: int) -> int:
    """Unused slots in the last block: p * ceil(L / p) - L."""
    return block_size * blocks_needed(length, block_size) - int(length)


def allocated_token_slots(lengths, block_size: int) -> int:
    """Token slots allocated for independent requests of the given lengths."""
    return sum(block_size * blocks_needed(L, block_size) for L in lengths)


def kv_alloc_bytes(length: int, block_size: int, bytes_per_token: int) -> int:
    """KV bytes allocated for one request: whole blocks of per-token KV."""
    return block_size * blocks_needed(length, block_size) * bytes_per_token


def shared_prefix_alloc_bytes(prefix_len: int, private_len: int, requests: int,
                              block_size: int, bytes_per_token: int) -> int:
    """KV bytes for b requests that share one prefix copy and own their suffix.

    The prefix is assumed to end on a block boundary (otherwise its tail
    block would be copied on write and become private).
    """
    if prefix_len % block_size:
        raise ValueError("shared prefix must end on a block boundary")
    return (kv_alloc_bytes(prefix_len, block_size, bytes_per_token)
            + requests * kv_alloc_bytes(private_len, block_size, bytes_per_token))


def shared_physical_blocks(shared_blocks: int, private_blocks: int, branches: int) -> int:
    """Physical blocks when ``branches`` tables share ``shared_blocks``."""
    return shared_blocks + branches * private_blocks


def block_references(shared_blocks: int, private_blocks: int, branches: int) -> int:
    """Table entries (references) across all branches."""
    return branches * (shared_blocks + private_blocks)


def causal_pairs(cached: int, chunk: int) -> int:
    """Causal query-key pairs of a c-token chunk after h cached tokens."""
    return chunk * cached + chunk * (chunk + 1) // 2


def full_pairs(cached: int, chunk: int) -> int:
    """Query-key pairs when every chunk row sees all h + c keys."""
    return chunk * (cached + chunk)


def chunk_attention_flops(pairs: int, q_heads: int, head_dim: int) -> int:
    """FLOPs of QK^T plus PV over the given pairs: 2 products x 2 FLOP/MAC."""
    return 4 * pairs * q_heads * head_dim
