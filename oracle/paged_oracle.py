"""Float64 CPU oracle for paged decode attention and the paged cache append.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module.  The library in
``paged_kv_cache_119_amd`` never imports it, and this module imports nothing
from the library: the two share no code.

Everything here is written straight from the definitions on the pages, in
float64, with plain loops and numpy primitives (a dot product, a max, an exp,
a sum).  There is no blocking, fusion or reordering beyond what those
definitions state.

Pages cited (titles as printed on each page):

* [PA] "PagedAttention 完全拆解：操作系统分页思想如何拯救 LLM 推理的内存利用率"
  (pinghaoyang.com.cn).
* [GA] the iaim.asia ai-infra article on the PagedAttention block table and
  gather (sections "KV Cache 如何按块分配", "“逐个 block 做 gather”具体执行什么",
  "vLLM 内核里的缓解写法").
* [LP] "PagedAttention 与 vLLM 推理加速" (lpnh.cn), section 2.3.
* [CB] the wiblog.cn article on vLLM paged attention and continuous batching,
  section 局限与未解决的问题.

Readings taken where the pages are silent or garbled:

* The softmax denominator of the blockwise equation in [PA] 原理详解（二） is
  printed as the exp of a block's summed score; it is read as the ordinary
  softmax sum over every visible token, the only reading under which the
  blockwise form equals the per-token definition in [PA] 背景, as that section
  states it must.
* The max is subtracted before exponentiating (a numerically stable softmax);
  in exact arithmetic this changes nothing.
* ``context_len`` counts the token appended in the same step; the new query
  attends to itself ([PA] 背景: the sum runs to t = i).
* The scale is passed as a float32 value; the oracle uses float64(float32(s)).
* Slots of the last block at or past ``context_len`` carry no data; they enter
  neither the max, the sum nor the weighted V sum.
* ``context_len == 0`` gives an all-zero output row.
* A partition's partial result is (m, l, o~) with m the max score, l the sum of
  exp(z - m) and o~ the exp(z - m)-weighted V sum; partitions are merged by the
  log-sum-exp rule (the pages name the segment reduction but print no formula).
* FP8 cache ([PA] 总结 item 6 names it, [CB] 局限与未解决的问题 leaves the
  quantisation choices open; no page fixes a format): OCP e4m3 codes, one
  float32 scale per pool, code = nearest e4m3 value of x * float32(1 / scale)
  (the product rounded to float32; ties to the even code; saturating at 448;
  NaN kept); a code c stands for e4m3(c) * scale.

Parity status: every function below is pinned by ``tests/test_oracle_pins.py``
against brute force, closed forms, library special cases or the pages' worked
examples.  No function here is "parity unpinned".

Array conventions: 16-bit floating point data is carried as ``np.uint16`` bit
patterns with a dtype tag (``"f16"`` or ``"bf16"``).  Pools have the layout
``[num_blocks, num_heads, block_size, head_dim]``; ``q``, ``k``, ``v`` and the
output have ``[tokens_or_seqs, num_heads, head_dim]``.
"""

from __future__ import annotations

import math

import numpy as np

__all__ = [
    "bits_to_f64",
    "f64_to_bits",
    "slot_of",
    "slot_mapping",
    "reshape_and_cache",
    "copy_blocks",
    "gather",
    "attend",
    "decode",
    "decode_one",
    "decode_rows",
    "partials",
    "lse_merge",
    "decode_partitioned",
    "dense_causal",
    "dense_causal_last_row",
    "e4m3_to_f64",
    "f64_to_e4m3",
    "quantize_e4m3",
    "reshape_and_cache_fp8",
    "decode_rows_fp8",
]


# ----------------------------------------------------------------------------
# 16-bit float bit patterns <-> float64
# ----------------------------------------------------------------------------

def bits_to_f64(bits: np.ndarray, dtype: str) -> np.ndarray:
    """Decode IEEE binary16 or bfloat16 bit patterns exactly into float64."""
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "f16":
        return bits.view(np.float16).astype(np.float64)
    if dtype == "bf16":
        # bfloat16 is the top half of a binary32 pattern.
        return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    raise ValueError(f"unknown dtype {dtype!r}")


def f64_to_bits(x: np.ndarray, dtype: str) -> np.ndarray:
    """Round float64 values to the nearest binary16 / bfloat16 (ties to even).

    Used only to build expected outputs for the exact special cases (a context
    of one token returns v itself).
    """
    x = np.asarray(x, dtype=np.float64)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    if dtype == "bf16":
        # Round from float64 directly (no detour through float32, which could
        # round twice): take the two bfloat16 neighbours of x and keep the
        # nearer one, the even one on a tie.
        out = np.empty(x.shape, dtype=np.uint16)
        flat_in, flat_out = x.reshape(-1), out.reshape(-1)
        for i, xi in enumerate(flat_in):
            if np.isnan(xi):
                flat_out[i] = 0x7FC0
                continue
            u = int(np.float32(xi).view(np.uint32))  # sign + a nearby pattern
            lo = (u >> 16) & 0xFFFF
            cands = [(lo - 1) & 0xFFFF, lo, (lo + 1) & 0xFFFF]
            best, best_err = None, None
            for c in cands:
                val = float(bits_to_f64(np.array([c], dtype=np.uint16), "bf16")[0])
                if np.isnan(val):
                    continue
                err = abs(val - xi) if np.isfinite(val) else float("inf")
                if best is None or err < best_err or (err == best_err and c % 2 == 0):
                    best, best_err = c, err
            flat_out[i] = best
        return out
    raise ValueError(f"unknown dtype {dtype!r}")


# ----------------------------------------------------------------------------
# 8-bit floating point (OCP e4m3) codes <-> float64
# ----------------------------------------------------------------------------
#
# [PA] 总结 item 6 names an FP8-quantised KV cache as a later layer on top of
# the paged cache; none of the pages fixes its format.  The reading taken: the
# OCP 8-bit "e4m3" format (1 sign bit, 4 exponent bits with bias 7, 3 mantissa
# bits, no infinities, one NaN pattern per sign: exponent and mantissa all
# ones; largest finite magnitude 448) and one float32 scale per pool, a code c
# standing for e4m3(c) * scale.


def e4m3_to_f64(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3 code, exactly, as float64 (NaN for 0x7F / 0xFF)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    normal = (1.0 + m / 8.0) * np.exp2(e.astype(np.float64) - 7.0)
    subnormal = (m / 8.0) * 2.0 ** -6
    val = sign * np.where(e == 0, subnormal, normal)
    return np.where((e == 15) & ((c & 7) == 7), np.nan, val)


# Magnitudes of the 127 non-negative finite codes 0x00 .. 0x7E, increasing.
_E4M3_MAGS = None


def _e4m3_mags() -> np.ndarray:
    global _E4M3_MAGS
    if _E4M3_MAGS is None:
        _E4M3_MAGS = e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    return _E4M3_MAGS


def f64_to_e4m3(x: np.ndarray) -> np.ndarray:
    """The e4m3 code nearest to each value: round to nearest, ties to the code
    with an even mantissa (the even code), saturating (a magnitude past 448,
    infinities included, takes the largest finite code), NaN to 0x7F.  The
    sign is kept, also for values that round to zero.

    Written as the definition: the nearest of the 127 finite magnitudes found
    by comparing against every one of them.
    """
    x = np.asarray(x, dtype=np.float64)
    flat = x.reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    mags = _e4m3_mags()
    codes = np.arange(0x7F)
    step = 1 << 16
    for i0 in range(0, flat.size, step):
        xs = flat[i0:i0 + step]
        a = np.abs(xs)
        finite = np.isfinite(a)
        a_f = np.where(finite, a, 0.0)
        dist = np.abs(a_f[:, None] - mags[None, :])
        best = dist.min(axis=1, keepdims=True)
        cand = dist == best  # one code, or two on a tie
        # on a tie prefer the even code: rank odd codes after every even one
        rank = np.where(cand, (codes[None, :] & 1) * 256 + codes[None, :], 1 << 20)
        c = rank.argmin(axis=1).astype(np.uint8)
        c = np.where(finite, c, np.uint8(0x7E))  # +-inf saturate
        c = np.where(np.signbit(xs), c | np.uint8(0x80), c)
        c = np.where(np.isnan(xs), np.uint8(0x7F), c)
        out[i0:i0 + step] = c
    return out.reshape(x.shape)


def quantize_e4m3(bits, dtype: str, scale: float) -> np.ndarray:
    """Codes of 16-bit values under a per-pool scale: code = e4m3(x * r) with
    r = 1 / scale rounded to float32 and the product rounded to float32 before
    the rounding to e4m3 (the decision is taken in float32, the precision the
    cache append computes in)."""
    x32 = bits_to_f64(bits, dtype).astype(np.float32)
    r = np.float32(1.0) / np.float32(scale)
    return f64_to_e4m3((x32 * r).astype(np.float64))


def reshape_and_cache_fp8(k_bits, v_bits, k_pool_codes, v_pool_codes, slots, block_size: int,
                          dtype: str, k_scale: float, v_scale: float) -> None:
    """The cache append of ``reshape_and_cache`` into e4m3 pools: each new row
    is quantised (``quantize_e4m3`` with the K or V scale) and written to its
    slot; negative slots and slots past the pool are skipped."""
    kq = quantize_e4m3(k_bits, dtype, k_scale)
    vq = quantize_e4m3(v_bits, dtype, v_scale)
    num_blocks = k_pool_codes.shape[0]
    for t in range(len(slots)):
        slot = int(slots[t])
        if slot < 0 or slot >= num_blocks * block_size:
            continue
        blk, off = divmod(slot, block_size)
        k_pool_codes[blk, :, off, :] = kq[t]
        v_pool_codes[blk, :, off, :] = vq[t]


# ----------------------------------------------------------------------------
# Translation: logical position -> pool slot
# ----------------------------------------------------------------------------

def slot_of(block_table_row, pos: int, block_size: int) -> int:
    """Pool slot of logical token ``pos`` of one sequence.

    [GA] "KV Cache 如何按块分配", BLOCK_SIZE=16 table: logical block n holds the
    tokens n*B .. n*B+B-1 and lives in pool block ``block_table[n]``; the token
    sits at offset pos mod B inside it ([PA] 原理详解（一）, Figure 6 walk-through).
    The slot number is block * B + offset.
    """
    logical_block = pos // block_size
    offset = pos % block_size
    return int(block_table_row[logical_block]) * block_size + offset


def slot_mapping(block_tables, token_seq, token_pos, block_size: int) -> np.ndarray:
    """Slots for a list of (sequence, position) tokens; -1 for padding tokens.

    A token whose sequence index or position is negative is padding and maps to
    slot -1 (the append then skips it).
    """
    block_tables = np.asarray(block_tables)
    out = np.full(len(token_seq), -1, dtype=np.int64)
    for t in range(len(token_seq)):
        s = int(token_seq[t])
        pos = int(token_pos[t])
        if s < 0 or pos < 0:
            continue
        out[t] = slot_of(block_tables[s], pos, block_size)
    return out


# ----------------------------------------------------------------------------
# Cache append ("fused reshape and block write")
# ----------------------------------------------------------------------------

def reshape_and_cache(k_bits, v_bits, k_pool_bits, v_pool_bits, slots, block_size: int) -> None:
    """Write each new token's K and V rows into its pool slot, in place.

    [PA] 原理详解（三） item 1: new keys and values are rearranged into the block
    layout and written through the block table.  For token t with slot
    ``slots[t] >= 0``: ``pool[slot // B, h, slot % B, :] = k[t, h, :]`` for every
    head h (same for v).  A negative slot or one past the pool is skipped.  The
    copy moves bit patterns, so it is exact.
    """
    num_blocks = k_pool_bits.shape[0]
    for t in range(len(slots)):
        slot = int(slots[t])
        if slot < 0 or slot >= num_blocks * block_size:
            continue
        blk, off = divmod(slot, block_size)
        for h in range(k_bits.shape[1]):
            k_pool_bits[blk, h, off, :] = k_bits[t, h, :]
            v_pool_bits[blk, h, off, :] = v_bits[t, h, :]


def copy_blocks(k_pool_bits, v_pool_bits, pairs) -> None:
    """Copy whole pool blocks, in place: ``pool[dst] = pool[src]`` for every
    (src, dst) pair, every head and every slot, in both pools.

    [PA] 内存共享 (Figure 8) and the fork / append primitives: before a
    sequence writes into a partly filled block it shares, that block is copied
    to a private block and the writer's table is redirected to the copy.  The
    sources are read as they were before the call (no destination is also a
    source).  Pairs with an index outside the pool are skipped.  Bit patterns
    are moved, so the copy is exact.
    """
    num_blocks = k_pool_bits.shape[0]
    k_src = k_pool_bits.copy()
    v_src = v_pool_bits.copy()
    for src, dst in pairs:
        src, dst = int(src), int(dst)
        if not (0 <= src < num_blocks and 0 <= dst < num_blocks):
            continue
        k_pool_bits[dst] = k_src[src]
        v_pool_bits[dst] = v_src[src]


# ----------------------------------------------------------------------------
# Gather + attention
# ----------------------------------------------------------------------------

def gather(pool_bits, block_table_row, context_len: int, block_size: int, head: int) -> np.ndarray:
    """Copy one head's K (or V) rows of logical tokens 0..L-1 into a contiguous
    ``[L, D]`` array of bit patterns, walking the block table token by token.

    [GA] "“逐个 block 做 gather”具体执行什么": look up the logical block's pool
    block, form the in-block address, read the row.
    """
    slots = [slot_of(block_table_row, pos, block_size) for pos in range(context_len)]
    blk = np.array([x // block_size for x in slots], dtype=np.int64)
    off = np.array([x % block_size for x in slots], dtype=np.int64)
    return pool_bits[blk, head, off, :].copy()


def attend(q64: np.ndarray, K64: np.ndarray, V64: np.ndarray, scale64: float):
    """Single-query softmax attention over contiguous float64 rows.

    [PA] 背景 (attention equation): a_j = exp(q.k_j * s) / sum_t exp(q.k_t * s),
    o = sum_j a_j v_j, with s = 1/sqrt(d) normally.  The max score is
    subtracted first (stable form; identical in exact arithmetic).

    Returns (o, a, m, l): output [D], weights [L], max score, sum of exp(z - m).
    """
    L = K64.shape[0]
    if L == 0:
        return np.zeros(V64.shape[1]), np.zeros(0), -math.inf, 0.0
    z = (K64 @ q64) * scale64
    m = float(np.max(z))
    e = np.exp(z - m)
    l = float(np.sum(e))
    a = e / l
    o = a @ V64
    return o, a, m, l


def decode_one(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
               scale: float, block_size: int, dtype: str, s: int, h: int) -> np.ndarray:
    """Float64 decode output of one (sequence, head): walk the table, gather K
    and V into contiguous arrays, convert to float64, attend."""
    L = int(context_lens[s])
    row = np.asarray(block_tables)[s]
    K = bits_to_f64(gather(k_pool_bits, row, L, block_size, h), dtype)
    V = bits_to_f64(gather(v_pool_bits, row, L, block_size, h), dtype)
    q = bits_to_f64(q_bits[s, h], dtype)
    scale64 = float(np.float32(scale))
    o, _, _, _ = attend(q, K, V, scale64)
    return o


def decode(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
           scale: float, block_size: int, dtype: str) -> np.ndarray:
    """Float64 paged decode attention for every (sequence, head): ``[S, H, D]``.

    [PA] 原理详解（二）: the blockwise form reaches exactly the per-token result,
    so the oracle computes the per-token definition over the gathered rows.
    """
    S, H, D = q_bits.shape
    out = np.zeros((S, H, D), dtype=np.float64)
    for s in range(S):
        for h in range(H):
            out[s, h] = decode_one(q_bits, k_pool_bits, v_pool_bits, block_tables,
                                   context_lens, scale, block_size, dtype, s, h)
    return out


def decode_rows(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
                scale: float, block_size: int, dtype: str) -> np.ndarray:
    """Float64 attention of several query rows per sequence: ``q_bits`` is
    ``[S, Q, H, D]`` over pools ``[N, Hkv, B, D]``; returns ``[S, Q, H, D]``.

    * Query head h reads KV head ``h // (H // Hkv)``: grouped-query attention,
      where a group of query heads shares one KV head (the Llama-2-70B shape of
      [GA] "末尾块的内部碎片", 8 KV heads).
    * Query i of sequence s is the token at position ``L - Q + i`` (the last Q
      tokens of the context) and attends over tokens ``0 .. L - Q + i``: the
      per-token equation of [PA] 背景, whose sum runs up to the query's own
      position.  With Q = 1 and H = Hkv this is ``decode``.

    Each row walks the table, gathers its visible K and V rows and attends.
    """
    S, Q, H, D = q_bits.shape
    Hkv = k_pool_bits.shape[1]
    G = H // Hkv
    out = np.zeros((S, Q, H, D), dtype=np.float64)
    scale64 = float(np.float32(scale))
    for s in range(S):
        L = int(context_lens[s])
        row = np.asarray(block_tables)[s]
        for i in range(Q):
            visible = L - Q + 1 + i if L > 0 else 0
            for h in range(H):
                kvh = h // G
                K = bits_to_f64(gather(k_pool_bits, row, visible, block_size, kvh), dtype)
                V = bits_to_f64(gather(v_pool_bits, row, visible, block_size, kvh), dtype)
                o, _, _, _ = attend(bits_to_f64(q_bits[s, i, h], dtype), K, V, scale64)
                out[s, i, h] = o
    return out


def decode_rows_fp8(q_bits, k_pool_codes, v_pool_codes, block_tables, context_lens,
                    scale: float, block_size: int, dtype: str, k_scale: float,
                    v_scale: float) -> np.ndarray:
    """``decode_rows`` over e4m3 pools: every gathered K row is
    ``e4m3(code) * k_scale`` and every V row ``e4m3(code) * v_scale`` (the
    scales taken as float32 values), exactly in float64; then the same
    attention.  ``q_bits`` is ``[S, Q, H, D]`` 16-bit, the output float64."""
    S, Q, H, D = q_bits.shape
    Hkv = k_pool_codes.shape[1]
    G = H // Hkv
    out = np.zeros((S, Q, H, D), dtype=np.float64)
    scale64 = float(np.float32(scale))
    ks = float(np.float32(k_scale))
    vs = float(np.float32(v_scale))
    for s in range(S):
        L = int(context_lens[s])
        row = np.asarray(block_tables)[s]
        for i in range(Q):
            visible = L - Q + 1 + i if L > 0 else 0
            for h in range(H):
                kvh = h // G
                K = e4m3_to_f64(gather(k_pool_codes, row, visible, block_size, kvh)) * ks
                V = e4m3_to_f64(gather(v_pool_codes, row, visible, block_size, kvh)) * vs
                o, _, _, _ = attend(bits_to_f64(q_bits[s, i, h], dtype), K, V, scale64)
                out[s, i, h] = o
    return out


# ----------------------------------------------------------------------------
# Split context: partial results and the log-sum-exp merge
# ----------------------------------------------------------------------------

def partials(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
             scale: float, block_size: int, dtype: str, partition_size: int, s: int, h: int):
    """Partial results of one (sequence, head) over partitions of P tokens.

    [GA] "vLLM 内核里的缓解写法": a long sequence is cut into segments processed
    independently and reduced afterwards.  Partition p covers logical tokens
    [p*P, min((p+1)*P, L)).  For each: m_p = max score, l_p = sum exp(z - m_p),
    o~_p = sum exp(z - m_p) v (unnormalised).  Returns arrays m [n], l [n],
    o [n, D] with n = ceil(L / P).
    """
    L = int(context_lens[s])
    row = np.asarray(block_tables)[s]
    D = q_bits.shape[2]
    n = -(-L // partition_size)
    K = bits_to_f64(gather(k_pool_bits, row, L, block_size, h), dtype)
    V = bits_to_f64(gather(v_pool_bits, row, L, block_size, h), dtype)
    q = bits_to_f64(q_bits[s, h], dtype)
    scale64 = float(np.float32(scale))
    m = np.zeros(n)
    l = np.zeros(n)
    o = np.zeros((n, D))
    for p in range(n):
        lo, hi = p * partition_size, min((p + 1) * partition_size, L)
        z = (K[lo:hi] @ q) * scale64
        m[p] = np.max(z)
        e = np.exp(z - m[p])
        l[p] = np.sum(e)
        o[p] = e @ V[lo:hi]
    return m, l, o


def lse_merge(m: np.ndarray, l: np.ndarray, o: np.ndarray) -> np.ndarray:
    """Merge partition partials into the normalised output.

    M = max_p m_p;  out = sum_p exp(m_p - M) o~_p / sum_p exp(m_p - M) l_p.
    Exact in real arithmetic because each partition's terms are its tokens'
    exp(z - M) terms rescaled by the common factor exp(m_p - M) ([PA]
    原理详解（二）: the softmax sum is associative over blocks).  Zero partials
    give a zero row (context length 0).
    """
    if len(m) == 0:
        return np.zeros(o.shape[1] if o.ndim == 2 else 0)
    M = float(np.max(m))
    w = np.exp(m - M)
    return (w @ o) / float(np.sum(w * l))


def decode_partitioned(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
                       scale: float, block_size: int, dtype: str, partition_size: int) -> np.ndarray:
    """Decode via partials + merge; equals ``decode`` up to float64 rounding."""
    S, H, D = q_bits.shape
    out = np.zeros((S, H, D))
    for s in range(S):
        for h in range(H):
            m, l, o = partials(q_bits, k_pool_bits, v_pool_bits, block_tables, context_lens,
                               scale, block_size, dtype, partition_size, s, h)
            if len(m):
                out[s, h] = lse_merge(m, l, o)
    return out


# ----------------------------------------------------------------------------
# Brute force: dense causal attention over an unpaged sequence
# ----------------------------------------------------------------------------

def dense_causal(Q64: np.ndarray, K64: np.ndarray, V64: np.ndarray, scale64: float) -> np.ndarray:
    """Full T x T causal attention for one head, every row: ``[T, D]``.

    [PA] 背景: position i attends to positions 1..i.  Scores above the diagonal
    are set to -inf before a row softmax; written with explicit loops so it
    shares nothing with ``attend``.
    """
    T = Q64.shape[0]
    D = V64.shape[1]
    out = np.zeros((T, D))
    for i in range(T):
        row = [-math.inf] * T
        for j in range(T):
            if j <= i:
                acc = 0.0
                for d in range(Q64.shape[1]):
                    acc += Q64[i, d] * K64[j, d]
                row[j] = acc * scale64
        mx = max(row)
        ex = [math.exp(r - mx) if r != -math.inf else 0.0 for r in row]
        tot = math.fsum(ex)
        for j in range(T):
            if ex[j] != 0.0:
                out[i] += (ex[j] / tot) * V64[j]
    return out


def dense_causal_last_row(Q64: np.ndarray, K64: np.ndarray, V64: np.ndarray, scale64: float) -> np.ndarray:
    """Row T-1 of ``dense_causal``: what a decode step of the last token sees."""
    return dense_causal(Q64, K64, V64, scale64)[Q64.shape[0] - 1]
