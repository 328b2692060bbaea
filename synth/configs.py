"""Seeded synthetic workloads for paged decode attention.

Shared by the tests, the benchmark and the smoke check as the single source of
inputs.  It draws context lengths, builds block tables with the host allocator,
and fills q and the two pools with N(0, 1) values rounded to the 16-bit type.
Pool slots that hold no token (free blocks, the unused tail of a sequence's
last block) are filled with a NaN pattern, so any read of them that reaches an
output shows up.  It contains none of the attention arithmetic and never
translates a position into a slot.

The five workloads stand in for the traces the pages evaluate on (ShareGPT,
Alpaca, WMT16), which are not used: only their shapes are taken from the pages
(sequences up to 2048 tokens, block size 16, shared prefixes and parallel
samples, a fragmented pool).

* ``tiny``      4 heads x 64, f16, B=16, pool of 128 blocks, 8 sequences,
                context_len ~ U{1..200}; tables from a random permutation of
                the pool.  Exercised through the append path end to end.
* ``opt13b``    40 heads x 128 (hidden 5120), f16, B=16, 64 sequences,
                context_len = clip(rint(lognormal(ln 300, 1.0)), 1, 2048);
                pool = 1.2 x the blocks needed, blocks scattered at random.
* ``llama13b``  40 x 128, bf16, B=16, 256 sequences, context_len ~ U{1..2048};
                the pool is first churned by 10,000 single-block allocations,
                each followed with probability 1/2 by freeing a random live
                churn block, then the rest freed in random order.  Includes the
                append of 256 new tokens.
* ``shared``    40 x 128, f16, B=16, 32 prompts x 512-token prefix forked into
                6 siblings (prefix blocks at refcount 6), each sibling with
                U{1..256} private tokens.  A control variant duplicates the
                prefix blocks per sibling with identical contents.
* ``longctx``   96 x 128, f16, 16 sequences, context_len ~ U{8192..32768},
                B in {8, 16, 32, 64}.

Seeds: numpy PCG64 ``default_rng(119000 + index)`` for lengths and tables;
torch generators seeded from the same number for values.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np

from .allocator import BlockAllocator

F16_NAN = 0x7E55   # quiet NaN with a payload: poison for empty f16 slots
BF16_NAN = 0x7FD5  # quiet NaN with a payload: poison for empty bf16 slots

CONFIGS = {
    "tiny": dict(index=1, num_heads=4, head_dim=64, dtype="f16", block_size=16, num_seqs=8,
                 lengths=("uniform", 1, 200), pool=("fixed", 128), tables="permute"),
    "opt13b": dict(index=2, num_heads=40, head_dim=128, dtype="f16", block_size=16, num_seqs=64,
                   lengths=("lognormal", 300.0, 1.0, 1, 2048), pool=("slack", 1.2), tables="permute",
                   max_len=2048),
    "llama13b": dict(index=3, num_heads=40, head_dim=128, dtype="bf16", block_size=16, num_seqs=256,
                     lengths=("uniform", 1, 2048), pool=("slack", 1.2), tables="churn", churn=10000,
                     max_len=2048),
    "shared": dict(index=4, num_heads=40, head_dim=128, dtype="f16", block_size=16,
                   prompts=32, prefix=512, siblings=6, private=(1, 256), pool=("slack", 1.2),
                   tables="fork"),
    "longctx": dict(index=5, num_heads=96, head_dim=128, dtype="f16", block_size=16, num_seqs=16,
                    lengths=("uniform", 8192, 32768), pool=("slack", 1.2), tables="permute",
                    max_len=32768, partition_size=512),
    # grouped-query layer of the Llama-2-70B shape: the pool holds 8 KV heads,
    # 64 query heads read them in groups of 8
    "llama70b": dict(index=6, num_heads=8, head_dim=128, dtype="bf16", block_size=16, num_seqs=256,
                     lengths=("uniform", 1, 2048), pool=("slack", 1.2), tables="permute", max_len=2048,
                     query_heads=64),
}


@dataclass
class Tables:
    """Host-side description of one batch: lengths, tables and pool shape."""
    name: str
    num_heads: int
    head_dim: int
    dtype: str
    block_size: int
    num_blocks: int
    context_lens: np.ndarray          # int32 [S]
    block_tables: np.ndarray          # int32 [S, max_blocks], padded with -1
    fills: list                       # per sequence: filled count of each entry
    scale: float
    seed: int
    refcount: np.ndarray = None       # int32 [N], after the tables were built
    extra: dict = field(default_factory=dict)

    @property
    def num_seqs(self) -> int:
        return int(self.context_lens.shape[0])

    @property
    def max_blocks(self) -> int:
        return int(self.block_tables.shape[1])

    def live_mask(self) -> np.ndarray:
        """bool [num_blocks, block_size]: True where a slot holds a token."""
        live = np.zeros((self.num_blocks, self.block_size), dtype=bool)
        for s in range(self.num_seqs):
            for j, f in enumerate(self.fills[s]):
                live[self.block_tables[s, j], :f] = True
        return live

    def kv_tokens(self) -> int:
        return int(self.context_lens.astype(np.int64).sum())


def _rng(index: int, salt: int = 0) -> np.random.Generator:
    return np.random.default_rng(119000 + index + salt)


def draw_lengths(spec, num_seqs: int, rng: np.random.Generator) -> np.ndarray:
    kind = spec[0]
    if kind == "uniform":
        lo, hi = spec[1], spec[2]
        return rng.integers(lo, hi + 1, size=num_seqs).astype(np.int32)
    if kind == "lognormal":
        median, sigma, lo, hi = spec[1:]
        x = np.rint(np.exp(rng.normal(math.log(median), sigma, size=num_seqs)))
        return np.clip(x, lo, hi).astype(np.int32)
    if kind == "fixed":
        return np.asarray(spec[1], dtype=np.int32)
    raise ValueError(kind)


def _blocks_needed(lengths, block_size: int) -> int:
    return int(sum(-(-int(L) // block_size) for L in lengths))


def _pack(alloc: BlockAllocator, sids, max_blocks: int):
    S = len(sids)
    tables = np.full((S, max_blocks), -1, dtype=np.int32)
    fills = []
    lens = np.zeros(S, dtype=np.int32)
    for i, sid in enumerate(sids):
        ids = alloc.block_ids(sid)
        f = alloc.fills(sid)
        if len(ids) > max_blocks:
            raise ValueError("sequence longer than the table width")
        tables[i, :len(ids)] = ids
        fills.append(list(f))
        lens[i] = sum(f)
    return tables, fills, lens


def build_tables(name: str = None, *, params: dict = None, block_size: int = None,
                 num_seqs: int = None, lengths=None, seed_salt: int = 0) -> Tables:
    """Lengths + block tables for a named workload (or explicit ``params``).

    ``block_size`` / ``num_seqs`` / ``lengths`` override the named values (used
    for the block-size sweep and for reduced-size parity cases).
    """
    p = dict(CONFIGS[name]) if name else {}
    if params:
        p.update(params)
    name = name or p.get("name", "custom")
    B = int(block_size or p["block_size"])
    index = int(p.get("index", 0))
    rng = _rng(index, seed_salt)
    kind = p["tables"]

    if kind in ("permute", "churn"):
        S = int(num_seqs or p["num_seqs"])
        lens = np.asarray(lengths, dtype=np.int32) if lengths is not None else draw_lengths(p["lengths"], S, rng)
        S = len(lens)
        needed = _blocks_needed(lens, B)
        if p["pool"][0] == "fixed":
            N = int(p["pool"][1])
        else:
            N = int(math.ceil(p["pool"][1] * needed))
        N = max(N, needed, 1)
        max_len = int(p.get("max_len", max(int(lens.max()) if S else 1, 1)))
        max_blocks = -(-max_len // B)
        if kind == "permute":
            alloc = BlockAllocator.create(N, B, pop_order=rng.permutation(N))
        else:
            alloc = BlockAllocator.create(N, B)
            live = []
            for _ in range(int(p["churn"])):
                if alloc.num_free() == 0:
                    break
                live.append(alloc.allocate())
                if rng.random() < 0.5 and live:
                    j = int(rng.integers(len(live)))
                    alloc.release(live.pop(j))
            for j in rng.permutation(len(live)):
                alloc.release(live[j])
        sids = []
        for L in lens:
            sid = alloc.new_seq()
            alloc.append_tokens(sid, int(L))
            sids.append(sid)
        tables, fills, got = _pack(alloc, sids, max_blocks)
        assert np.array_equal(got, lens)
    elif kind == "fork":
        prompts, prefix, sibs = int(p["prompts"]), int(p["prefix"]), int(p["siblings"])
        lo, hi = p["private"]
        private = rng.integers(lo, hi + 1, size=(prompts, sibs))
        lens = (prefix + private).reshape(-1).astype(np.int32)
        unique = prompts * (-(-prefix // B)) + int(sum(-(-(int(x) + prefix % B) // B) for x in private.reshape(-1)))
        N = int(math.ceil(p["pool"][1] * unique)) + prompts * sibs
        max_blocks = -(-int(lens.max()) // B)
        alloc = BlockAllocator.create(N, B, pop_order=rng.permutation(N))
        sids = []
        for i in range(prompts):
            root = alloc.new_seq()
            alloc.append_tokens(root, prefix)
            group = [root] + [alloc.fork(root) for _ in range(sibs - 1)]
            for j, sid in enumerate(group):
                alloc.append_tokens(sid, int(private[i, j]))
            sids.extend(group)
        tables, fills, got = _pack(alloc, sids, max_blocks)
        assert np.array_equal(got, lens)
        p["private_lens"] = private
    else:
        raise ValueError(kind)

    alloc.check()
    t = Tables(name=name, num_heads=int(p["num_heads"]), head_dim=int(p["head_dim"]), dtype=p["dtype"],
               block_size=B, num_blocks=alloc.num_blocks, context_lens=lens.astype(np.int32),
               block_tables=tables, fills=fills, scale=1.0 / math.sqrt(int(p["head_dim"])),
               seed=119000 + index + seed_salt,
               refcount=np.asarray(alloc.refcount, dtype=np.int32))
    t.extra["copies"] = list(alloc.copies)
    t.extra["free_blocks"] = list(alloc.free_stack)
    if kind == "fork":
        t.extra["prefix_blocks"] = -(-int(p["prefix"]) // B)
        t.extra["siblings"] = int(p["siblings"])
    if "partition_size" in p:
        t.extra["partition_size"] = int(p["partition_size"])
    return t


def duplicate_shared(t: Tables):
    """Control for shared-prefix tables: give every reference to a shared block
    beyond the first its own private block.

    Returns (tables, copies, num_blocks) where ``copies`` lists (src, dst) pool
    blocks whose contents must be copied so the duplicated batch holds the same
    logical K/V as ``t``.
    """
    N = t.num_blocks
    seen = set()
    copies = []
    tables = t.block_tables.copy()
    nxt = N
    for s in range(t.num_seqs):
        for j, f in enumerate(t.fills[s]):
            b = int(tables[s, j])
            if b in seen:
                copies.append((b, nxt))
                tables[s, j] = nxt
                nxt += 1
            else:
                seen.add(b)
    return tables, copies, nxt


# ----------------------------------------------------------------------------
# Values (torch tensors; torch is imported lazily so table-only users need numpy)
# ----------------------------------------------------------------------------

def torch_dtype(dtype: str):
    import torch
    return {"f16": torch.float16, "bf16": torch.bfloat16}[dtype]


def nan_bits(dtype: str) -> int:
    return F16_NAN if dtype == "f16" else BF16_NAN


def _gen(device, seed: int):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return g


def normal_16bit(shape, dtype: str, device, seed: int, chunk_elems: int = 1 << 28):
    """N(0, 1) values drawn in float32 and rounded to the 16-bit type (ties to
    even, torch's cast), filled chunk by chunk to bound temporary memory."""
    import torch
    out = torch.empty(shape, dtype=torch_dtype(dtype), device=device)
    flat = out.view(-1)
    g = _gen(device, seed)
    n = flat.numel()
    for lo in range(0, n, chunk_elems):
        hi = min(n, lo + chunk_elems)
        flat[lo:hi] = torch.randn(hi - lo, generator=g, device=device, dtype=torch.float32).to(out.dtype)
    return out


FP8_NAN = 0x7F  # an e4m3 NaN code (exponent and mantissa all ones)


def random_e4m3(shape, device, seed: int, exp_lo: int = 8, exp_hi: int = 14, chunk_elems: int = 1 << 27):
    """Random e4m3 codes (torch.uint8): uniform sign and mantissa, biased
    exponent uniform in [exp_lo, exp_hi] (0 gives subnormals; the default
    spreads magnitudes over 2 .. 240, about the range of N(0, 1) data
    quantised with a scale near 1/60); never a NaN code."""
    import torch
    out = torch.empty(shape, dtype=torch.uint8, device=device)
    flat = out.view(-1)
    g = _gen(device, seed)
    n = flat.numel()
    for lo in range(0, n, chunk_elems):
        hi = min(n, lo + chunk_elems)
        bits = torch.randint(0, 256, (hi - lo,), generator=g, device=device, dtype=torch.int32)
        e = torch.randint(exp_lo, exp_hi + 1, (hi - lo,), generator=g, device=device, dtype=torch.int32)
        code = (bits & 0x87) | (e << 3)
        code = torch.where((code & 0x7F) == 0x7F, code - 1, code)  # NaN -> 448
        flat[lo:hi] = code.to(torch.uint8)
    return out


def make_fp8_pools(t: Tables, device="cpu", salt: int = 2, poison: bool = True, **kw):
    """e4m3 K and V pools ``[N, H, B, D]`` (uint8 codes) with every live slot
    drawn by ``random_e4m3`` and every other slot set to the NaN code."""
    import torch
    shape = (t.num_blocks, t.num_heads, t.block_size, t.head_dim)
    k = random_e4m3(shape, device, t.seed * 16 + salt, **kw)
    v = random_e4m3(shape, device, t.seed * 16 + salt + 1, **kw)
    if poison:
        dead = torch.from_numpy(~t.live_mask()).to(device)[:, None, :, None].expand(shape)
        for pool in (k, v):
            pool.masked_fill_(dead, FP8_NAN)
    return k, v


def make_query(t: Tables, device="cpu", salt: int = 1):
    return normal_16bit((t.num_seqs, t.num_heads, t.head_dim), t.dtype, device, t.seed * 16 + salt)


def make_pools(t: Tables, device="cpu", salt: int = 2, poison: bool = True):
    """K and V pools ``[N, H, B, D]`` with every live slot ~N(0,1) and every other
    slot set to the NaN poison pattern."""
    import torch
    shape = (t.num_blocks, t.num_heads, t.block_size, t.head_dim)
    k = normal_16bit(shape, t.dtype, device, t.seed * 16 + salt)
    v = normal_16bit(shape, t.dtype, device, t.seed * 16 + salt + 1)
    if poison:
        dead = torch.from_numpy(~t.live_mask()).to(device)          # [N, B]
        dead = dead[:, None, :, None].expand(shape)
        nb = nan_bits(t.dtype)
        nb_signed = nb - 0x10000 if nb >= 0x8000 else nb
        for pool in (k, v):
            pool.view(torch.int16).masked_fill_(dead, nb_signed)
    return k, v


def empty_pools(t: Tables, device="cpu"):
    """Pools filled entirely with the poison pattern (before any append)."""
    import torch
    shape = (t.num_blocks, t.num_heads, t.block_size, t.head_dim)
    nb = nan_bits(t.dtype)
    nb_signed = nb - 0x10000 if nb >= 0x8000 else nb
    k = torch.full(shape, nb_signed, dtype=torch.int16, device=device).view(torch_dtype(t.dtype))
    v = torch.full(shape, nb_signed, dtype=torch.int16, device=device).view(torch_dtype(t.dtype))
    return k, v


def make_history(t: Tables, device="cpu", salt: int = 3):
    """Logical K/V for every token of every sequence, for filling pools through
    the append path: returns (token_seq int32 [T], token_pos int32 [T],
    k [T, H, D], v [T, H, D]) with tokens listed sequence by sequence."""
    import torch
    seq = np.concatenate([np.full(int(L), s, dtype=np.int32) for s, L in enumerate(t.context_lens)]) \
        if t.num_seqs else np.zeros(0, np.int32)
    pos = np.concatenate([np.arange(int(L), dtype=np.int32) for L in t.context_lens]) \
        if t.num_seqs else np.zeros(0, np.int32)
    T = len(seq)
    k = normal_16bit((T, t.num_heads, t.head_dim), t.dtype, device, t.seed * 16 + salt)
    v = normal_16bit((T, t.num_heads, t.head_dim), t.dtype, device, t.seed * 16 + salt + 1)
    return torch.from_numpy(seq), torch.from_numpy(pos), k, v


def to_bits(x) -> np.ndarray:
    """torch 16-bit tensor -> numpy uint16 bit patterns (host copy)."""
    import torch
    return x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
