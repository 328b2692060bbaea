"""Byte accounting for paged decode attention and the cache append.

These are the algorithmic byte counts the roofline is priced on: every byte the
operation must move at least once, nothing for the pool's free blocks or the
unused tail of a last block, nothing for partial-result workspace traffic.

Formulas follow the KV-size arithmetic on the pages:

* per token and layer, K and V each hold heads x head_dim values
  ("PagedAttention 完全拆解", 背景 / KV Cache 有多大: 2 x hidden x layers x
  bytes per element; "PagedAttention 与 vLLM 推理加速", section 1:
  2 x L x H x D x S x dtype size);
* one int32 table entry per logical block (iaim.asia block-table article,
  section 块表自身的显存);
* at most B - 1 empty slots in a sequence's last block (same article, section
  末尾块的内部碎片).
"""

from __future__ import annotations

import numpy as np

TABLE_ENTRY_BYTES = 4
CONTEXT_LEN_BYTES = 4
SLOT_BYTES = 8


def kv_bytes_per_token(layers: int, kv_heads: int, head_dim: int, dtype_bytes: int) -> int:
    """K and V bytes one token occupies across ``layers`` layers."""
    return 2 * layers * kv_heads * head_dim * dtype_bytes


def kv_bytes_per_token_hidden(layers: int, hidden: int, dtype_bytes: int) -> int:
    """Same, written with the model's hidden size (= heads x head_dim)."""
    return 2 * layers * hidden * dtype_bytes


def max_tail_waste_tokens(block_size: int) -> int:
    """Largest number of empty slots a single append-only sequence can leave."""
    return block_size - 1


def num_blocks_for(tokens: int, block_size: int) -> int:
    return -(-int(tokens) // int(block_size))


def table_bytes(max_len: int, block_size: int, requests: int = 1) -> int:
    """Bytes of a full-width int32 block table for ``requests`` rows."""
    return num_blocks_for(max_len, block_size) * TABLE_ENTRY_BYTES * requests


def decode_bytes(context_lens, num_heads: int, head_dim: int, dtype_bytes: int, block_size: int,
                 kv_dtype_bytes: int = None) -> dict:
    """Algorithmic bytes of one decode call.

    K and V of every live token for every head, q read once, the output written
    once, the table entries actually needed and the context lengths.  The pools
    may hold a narrower type than q and out (``kv_dtype_bytes``, 1 for e4m3).
    """
    kvb = dtype_bytes if kv_dtype_bytes is None else kv_dtype_bytes
    L = np.asarray(context_lens, dtype=np.int64)
    L = np.maximum(L, 0)
    S = int(L.shape[0])
    kv = int(L.sum()) * num_heads * head_dim * 2 * kvb
    q = S * num_heads * head_dim * dtype_bytes
    out = q
    table = int(sum(num_blocks_for(x, block_size) for x in L)) * TABLE_ENTRY_BYTES
    lens = S * CONTEXT_LEN_BYTES
    return {"kv": kv, "q": q, "out": out, "table": table, "context_lens": lens,
            "total": kv + q + out + table + lens, "kv_tokens": int(L.sum())}


def append_bytes(num_valid_tokens: int, num_tokens: int, num_heads: int, head_dim: int, dtype_bytes: int,
                 pool_dtype_bytes: int = None) -> dict:
    """Algorithmic bytes of one cache append: read k and v of the valid tokens,
    write them into the pools (``pool_dtype_bytes`` per element, 1 for e4m3),
    read every slot number."""
    row = num_heads * head_dim * dtype_bytes
    prow = num_heads * head_dim * (dtype_bytes if pool_dtype_bytes is None else pool_dtype_bytes)
    read = 2 * num_valid_tokens * row
    write = 2 * num_valid_tokens * prow
    slots = num_tokens * SLOT_BYTES
    return {"read": read, "write": write, "slots": slots, "total": read + write + slots}


def slot_mapping_bytes(num_tokens: int) -> int:
    """Slot translation: read (sequence, position) and one table entry, write
    one int64 slot per token."""
    return int(num_tokens) * (4 + 4 + TABLE_ENTRY_BYTES + SLOT_BYTES)


def shared_prefix_bytes(context_lens, prefix_lens, group_size: int, num_heads: int, head_dim: int,
                        dtype_bytes: int, block_size: int) -> dict:
    """Algorithmic bytes of a decode over groups of ``group_size`` sequences
    that share their first ``prefix_lens[g]`` tokens, when each group's
    prefix is read once: the prefix K/V once per group, every sequence's own
    tokens, q, out, the table entries read (the first sequence's prefix
    entries once per group, every sequence's own), the lengths and the
    prefix lengths.  ``logical`` is the same batch counted by the plain
    decode formula (every sequence's whole context)."""
    L = np.maximum(np.asarray(context_lens, dtype=np.int64), 0)
    P = np.asarray(prefix_lens, dtype=np.int64)
    S = int(L.shape[0])
    own = np.maximum(L - np.repeat(P, group_size), 0)
    row = num_heads * head_dim * 2 * dtype_bytes
    kv = int(P.sum()) * row + int(own.sum()) * row
    q = S * num_heads * head_dim * dtype_bytes
    # the prefix pass reads a group's prefix entries once; a sequence's own
    # tokens need the entries from the block holding token prefix_len on
    pre_entries = int(sum(num_blocks_for(x, block_size) for x in P))
    own_entries = int(sum(num_blocks_for(l, block_size) - p // block_size
                          for l, p in zip(L, np.repeat(P, group_size)) if l > p))
    table = (pre_entries + own_entries) * TABLE_ENTRY_BYTES
    small = S * CONTEXT_LEN_BYTES + int(P.shape[0]) * CONTEXT_LEN_BYTES
    total = kv + 2 * q + table + small
    logical = decode_bytes(L, num_heads, head_dim, dtype_bytes, block_size)["total"]
    return {"kv": kv, "q": q, "out": q, "table": table, "total": total, "logical": logical,
            "kv_tokens": int(L.sum()), "unique_kv_tokens": int(P.sum() + own.sum())}
