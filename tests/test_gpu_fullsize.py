"""GPU: the paths the published measurements run, checked against the float64
oracle at the size they are timed at.

* Rows cut into more than 64 pieces by the balanced split (long contexts over
  few heads): the merge then takes several rounds of 64 pieces.  Every output
  of the 16-bit decode, the fused decode step (one call, and split + merge as
  the benchmark times it) and the e4m3 decode and decode step.
* The benchmark's own step on the full OPT-13B batch: the split pass with the
  append fused (``decode_partitions_append``) then ``decode_merge``, every
  output, and both pools bit-exact against the oracle's append.
* The same step on the full LLaMA-13B batch (256 sequences, churned pool):
  appended slots and every other pool byte exact, outputs sampled.
* The long-context batch (96 heads, 16 sequences of 8k-32k tokens) with the
  balanced split at every block size, sampled (the fixed 512-token partitions
  are covered in test_gpu_decode.py).
"""

import math

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from paged_kv_cache_119_amd._binding import pool_desc_of  # noqa: E402
from oracle import paged_oracle as po  # noqa: E402
from synth import build_tables, make_fp8_pools, make_pools, make_query, normal_16bit, to_bits  # noqa: E402

from .gpu_util import DEV, HeadCache, assert_close, device_tables, log, oracle_samples, sample_pairs  # noqa: E402

MIN_SLICE = 8  # smallest balanced-split slice, in chunks


def pieces_per_row(lens, H, TC, G, max_len):
    """Pieces each (sequence, head) row is cut into by the balanced split:
    rows of ceil(L / TC) chunks, sequence major, cut into equal slices of the
    total (at most G workers, each slice at least MIN_SLICE chunks)."""
    chunks = [-(-int(L) // TC) if 0 < L <= max_len else 0 for L in lens]
    total = H * sum(chunks)
    workers = max(1, min(G, total // MIN_SLICE))
    sl = max(1, -(-total // workers))
    out, pos = [], 0
    for n in chunks:
        for _ in range(H):
            if n:
                out.append((pos + n - 1) // sl - pos // sl + 1)
                pos += n
    return out


def _workers(S, H, maxb, desc, fp8=False, append=False):
    info = pkv.decode_launch_info(S, H, maxb, desc, 0, 1, fp8, append)
    return info["workgroups"] * info["waves_per_workgroup"]


def _long_case(lengths, H, D, B, dtype, index):
    return build_tables(params=dict(name="long_rows", index=index, num_heads=H, head_dim=D, dtype=dtype,
                                    block_size=B, num_seqs=len(lengths), lengths=("fixed", lengths),
                                    pool=("slack", 1.1), tables="permute", max_len=max(lengths)))


LONG_CASES = [
    # lengths, heads, head_dim, block size, dtype
    ([16384], 8, 128, 16, "f16"),
    ([32768, 20001], 4, 128, 16, "bf16"),
    ([30000], 4, 64, 32, "f16"),
]


@pytest.mark.parametrize("lengths,H,D,B,dtype", LONG_CASES)
def test_rows_cut_into_more_than_64_pieces(lengths, H, D, B, dtype):
    log(f"long rows: L={lengths} H={H} D={D} B={B} {dtype}")
    t = _long_case(lengths, H, D, B, dtype, 60 + D + B)
    tab, lens = device_tables(t)
    kp, vp = make_pools(t, DEV)
    q = make_query(t, DEV)
    S = t.num_seqs
    TC = 16 if D == 128 else 32
    G = _workers(S, H, t.max_blocks, pool_desc_of(kp))
    pieces = pieces_per_row(t.context_lens, H, TC, G, t.max_blocks * B)
    log(f"  workers {G}, pieces per row {min(pieces)}..{max(pieces)}")
    assert min(pieces) > 64

    out = pkv.paged_attention_decode(q, kp, vp, tab, lens, t.scale)
    torch.cuda.synchronize()
    ref = po.decode(to_bits(q), to_bits(kp), to_bits(vp), t.block_tables, t.context_lens, t.scale, B, dtype)
    assert_close(to_bits(out), ref, dtype, "decode")

    # the decode step: append token L - 1, attend (one call; split + merge)
    knew = normal_16bit((S, H, D), dtype, DEV, 7001 + D)
    vnew = normal_16bit((S, H, D), dtype, DEV, 7002 + D)
    kpo, vpo = to_bits(kp), to_bits(vp)
    kp2, vp2 = kp.clone(), vp.clone()
    one = pkv.paged_attention_decode_append(q, knew, vnew, kp, vp, tab, lens, t.scale)
    ws = pkv.alloc_workspace(S, H, t.max_blocks, kp2, 0)
    two = torch.zeros_like(q)
    pkv.decode_partitions_append(q, knew, vnew, kp2, vp2, tab, lens, t.scale, two, ws)
    pkv.decode_merge(two, lens, t.max_blocks, kp2, ws)
    torch.cuda.synchronize()
    slots = po.slot_mapping(t.block_tables, np.arange(S), t.context_lens - 1, B)
    po.reshape_and_cache(to_bits(knew), to_bits(vnew), kpo, vpo, slots, B)
    assert np.array_equal(to_bits(kp), kpo) and np.array_equal(to_bits(vp), vpo)
    assert np.array_equal(to_bits(kp2), kpo) and np.array_equal(to_bits(vp2), vpo)
    ref = po.decode(to_bits(q), kpo, vpo, t.block_tables, t.context_lens, t.scale, B, dtype)
    assert_close(to_bits(one), ref, dtype, "decode step, one call")
    assert torch.equal(one.view(torch.int16), two.view(torch.int16))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_rows_cut_into_more_than_64_pieces(dtype):
    lengths, H, D, B = [32768, 23000], 4, 128, 16
    log(f"long rows e4m3: L={lengths} H={H} {dtype}")
    t = _long_case(lengths, H, D, B, dtype, 70)
    tab, lens = device_tables(t)
    kp, vp = make_fp8_pools(t, DEV, exp_lo=4, exp_hi=10)
    q = make_query(t, DEV)
    S = t.num_seqs
    desc = pkv.make_pool_desc(t.num_blocks, B, H, D, dtype)
    G = _workers(S, H, t.max_blocks, desc, fp8=True)
    pieces = pieces_per_row(t.context_lens, H, 32, G, t.max_blocks * B)
    log(f"  workers {G}, pieces per row {min(pieces)}..{max(pieces)}")
    assert min(pieces) > 64
    ks, vs = 0.37, 1.9

    def codes(x):
        return x.detach().cpu().contiguous().view(torch.uint8).numpy()

    out = pkv.paged_attention_decode_fp8(q, kp, vp, tab, lens, t.scale, ks, vs)
    torch.cuda.synchronize()
    ref = po.decode_rows_fp8(to_bits(q)[:, None], codes(kp), codes(vp), t.block_tables, t.context_lens,
                             t.scale, B, dtype, ks, vs)[:, 0]
    assert_close(to_bits(out), ref, dtype, "e4m3 decode")

    knew = normal_16bit((S, H, D), dtype, DEV, 7101)
    vnew = normal_16bit((S, H, D), dtype, DEV, 7102)
    kpo, vpo = codes(kp).copy(), codes(vp).copy()
    step = pkv.paged_attention_decode_append_fp8(q, knew, vnew, kp, vp, tab, lens, t.scale, ks, vs)
    torch.cuda.synchronize()
    slots = po.slot_mapping(t.block_tables, np.arange(S), t.context_lens - 1, B)
    po.reshape_and_cache_fp8(to_bits(knew), to_bits(vnew), kpo, vpo, slots, B, dtype, ks, vs)
    assert np.array_equal(codes(kp), kpo) and np.array_equal(codes(vp), vpo)
    ref = po.decode_rows_fp8(to_bits(q)[:, None], kpo, vpo, t.block_tables, t.context_lens, t.scale, B, dtype,
                             ks, vs)[:, 0]
    assert_close(to_bits(step), ref, dtype, "e4m3 decode step")


def _bench_step(t, q, knew, vnew, kp, vp, tab, lens):
    """The benchmark's step: split pass with the append fused, then the merge."""
    ws = pkv.alloc_workspace(t.num_seqs, t.num_heads, t.max_blocks, kp, 0)
    out = torch.full_like(q, float("nan"))
    pkv.decode_partitions_append(q, knew, vnew, kp, vp, tab, lens, t.scale, out, ws)
    pkv.decode_merge(out, lens, t.max_blocks, kp, ws)
    torch.cuda.synchronize()
    return out


def test_opt13b_bench_step_every_output():
    """The exact step bench.py times, on the full OPT-13B batch (same seeds,
    same launch): pools bit-exact against the oracle's append of the 64 new
    rows, every output against the oracle over the updated pools."""
    log("opt13b bench step: decode_partitions_append + decode_merge, full compare")
    t = build_tables("opt13b")
    S, H, D = t.num_seqs, t.num_heads, t.head_dim
    tab, lens = device_tables(t)
    kp, vp = make_pools(t, DEV)
    q = make_query(t, DEV)
    knew = normal_16bit((S, H, D), t.dtype, DEV, t.seed * 16 + 9)
    vnew = normal_16bit((S, H, D), t.dtype, DEV, t.seed * 16 + 10)
    kpo, vpo = to_bits(kp), to_bits(vp)
    out = _bench_step(t, q, knew, vnew, kp, vp, tab, lens)
    slots = po.slot_mapping(t.block_tables, np.arange(S), t.context_lens - 1, t.block_size)
    po.reshape_and_cache(to_bits(knew), to_bits(vnew), kpo, vpo, slots, t.block_size)
    assert np.array_equal(to_bits(kp), kpo) and np.array_equal(to_bits(vp), vpo)
    ref = po.decode(to_bits(q), kpo, vpo, t.block_tables, t.context_lens, t.scale, t.block_size, t.dtype)
    assert_close(to_bits(out), ref, t.dtype, "opt13b bench step")


def test_llama13b_bench_step_sampled():
    """The same step on the full LLaMA-13B batch: every appended slot equals
    its new row and no other pool byte changes; outputs sampled against the
    oracle over the updated pools."""
    log("llama13b bench step: decode_partitions_append + decode_merge, sampled")
    t = build_tables("llama13b")
    S, H, D, B = t.num_seqs, t.num_heads, t.head_dim, t.block_size
    tab, lens = device_tables(t)
    kp, vp = make_pools(t, DEV)
    q = make_query(t, DEV)
    knew = normal_16bit((S, H, D), t.dtype, DEV, t.seed * 16 + 9)
    vnew = normal_16bit((S, H, D), t.dtype, DEV, t.seed * 16 + 10)
    k0, v0 = kp.clone(), vp.clone()
    out = _bench_step(t, q, knew, vnew, kp, vp, tab, lens)
    slots = po.slot_mapping(t.block_tables, np.arange(S), t.context_lens - 1, B)
    assert np.all(slots >= 0)
    blk = torch.from_numpy(slots // B).to(DEV)
    off = torch.from_numpy(slots % B).to(DEV)
    assert torch.equal(kp[blk, :, off, :].view(torch.int16), knew.view(torch.int16))
    assert torch.equal(vp[blk, :, off, :].view(torch.int16), vnew.view(torch.int16))
    k0[blk, :, off, :] = knew
    v0[blk, :, off, :] = vnew
    assert torch.equal(kp.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(vp.view(torch.int16), v0.view(torch.int16))
    del k0, v0
    rng = np.random.default_rng(21)
    pairs = sample_pairs(t, rng)
    ref = oracle_samples(t, to_bits(q), HeadCache(kp, vp), pairs)
    ob = to_bits(out)
    assert_close(np.stack([ob[s, h] for s, h in pairs]), ref, t.dtype, f"llama13b bench step ({len(pairs)} samples)")


@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_longctx_balanced_split_sampled(B):
    """The long-context batch with the default balanced split (partition_size
    0), as its timings are taken, at every block size."""
    log(f"longctx B={B}: 16 seqs x 96 heads, balanced split, sampled oracle")
    t = build_tables("longctx", block_size=B)
    tab, lens = device_tables(t)
    kp, vp = make_pools(t, DEV)
    q = make_query(t, DEV)
    assert pkv.decode_partition_size(t.num_seqs, t.num_heads, t.max_blocks, kp, 0) == 0
    out = pkv.paged_attention_decode(q, kp, vp, tab, lens, t.scale, partition_size=0)
    torch.cuda.synchronize()
    rng = np.random.default_rng(30 + B)
    pairs = sample_pairs(t, rng, heads=[0, 47, 95])
    ref = oracle_samples(t, to_bits(q), HeadCache(kp, vp), pairs)
    ob = to_bits(out)
    assert_close(np.stack([ob[s, h] for s, h in pairs]), ref, t.dtype,
                 f"longctx B={B} balanced ({len(pairs)} samples)")
    del kp, vp
    torch.cuda.empty_cache()


def test_pieces_rule_matches_a_hand_count():
    """The host-side piece count used above, on a case small enough to count
    by hand: 2 rows of 20 chunks, 5 workers -> slices of 8 chunks."""
    got = pieces_per_row([20 * 16], 2, 16, 5, 10 ** 6)
    # chunks 0..19 (row 0) and 20..39 (row 1) over slices [0,8) [8,16) ...
    assert got == [3, 3]
    assert math.ceil(40 / 5) == 8
