"""Host-side logic: the table-building allocator against the pages' worked
examples, the seeded workloads, and the byte accounting against the pages'
closed forms.  CPU only."""

import json
import math
import os

import numpy as np
import pytest

from paged_kv_cache_119_amd import accounting as acc
from synth import BlockAllocator, PoolExhausted, build_tables, duplicate_shared
from synth.configs import CONFIGS


def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


def _pool(N, B, head):
    rest = [b for b in range(N) if b not in head]
    return BlockAllocator.create(N, B, pop_order=list(head) + rest)


def test_fig6_on_demand_allocation(golden_dir):
    g = _load(golden_dir, "fig6_decode_walkthrough.json")
    a = _pool(16, g["block_size"], g["pop_order_head"])
    sid = a.new_seq()
    a.append_tokens(sid, g["after_prompt"]["tokens"])
    assert a.block_ids(sid) == g["after_prompt"]["blocks"]
    assert a.fills(sid) == g["after_prompt"]["filled"]
    free_before = a.num_free()
    a.append(sid)
    assert a.block_ids(sid) == g["after_decode_1"]["blocks"]
    assert a.fills(sid) == g["after_decode_1"]["filled"]
    assert a.num_free() == free_before          # no allocation on decode 1
    a.append(sid)
    assert a.block_ids(sid) == g["after_decode_2"]["blocks"]
    assert a.fills(sid) == g["after_decode_2"]["filled"]
    a.check()


def test_lp_translation_example(golden_dir):
    g = _load(golden_dir, "lp_sec23_translation.json")
    a = _pool(8, g["block_size"], g["pop_order_head"])
    sid = a.new_seq()
    a.append_tokens(sid, g["tokens"])
    assert a.block_ids(sid) == g["blocks"]
    assert a.fills(sid) == g["filled"]


def test_fig7_two_sequences_and_reuse(golden_dir):
    g = _load(golden_dir, "fig7_two_sequences.json")
    B = g["block_size"]
    a = _pool(8, B, g["pop_order_head"])
    A, Bq = a.new_seq(), a.new_seq()
    for _ in range(2):              # interleaved growth, one block each at a time
        a.append_tokens(A, B)
        a.append_tokens(Bq, B)
    assert a.block_ids(A) == g["seq_a_blocks"]
    assert a.block_ids(Bq) == g["seq_b_blocks"]
    a.free_seq(A)
    C = a.new_seq()
    a.append_tokens(C, 2 * B)
    assert sorted(a.block_ids(C)) == sorted(g["reused_after_a_ends"])
    a.check()


def test_fig8_copy_on_write(golden_dir):
    g = _load(golden_dir, "fig8_copy_on_write.json")
    a = _pool(16, g["block_size"], g["pop_order_head"])
    a1 = a.new_seq()
    a.append_tokens(a1, g["prompt_tokens"])
    a2 = a.fork(a1)
    assert a.block_ids(a1) == a.block_ids(a2) == g["shared_blocks"]
    assert all(a.refcount[b] == g["shared_refcount"] for b in g["shared_blocks"])
    a.append(a1)          # A1 writes first: copy-on-write of block 1
    assert a.block_ids(a1) == g["a1_blocks_after"]
    assert [list(c) for c in a.copies] == g["copies"]
    a.append(a2)          # A2 writes in place
    assert a.block_ids(a2) == g["a2_blocks_after"]
    assert len(a.copies) == 1
    for b, cnt in g["refcount_after"].items():
        assert a.refcount[int(b)] == cnt
    a.check()


def test_fig9_beam_search_sharing(golden_dir):
    g = _load(golden_dir, "fig9_beam_search.json")
    B = g["block_size"]
    N = 16
    # Build the "before" state: cand0..2 share [0, 1, 3]; cand3 shares [0].
    head = [0, 1, 3, 5, 6, 7, 2, 4, 8] + list(range(9, 13))
    a = _pool(N, B, head)
    c0 = a.new_seq()
    a.append_tokens(c0, 3 * B)             # blocks 0, 1, 3
    c1 = a.fork(c0)
    c2 = a.fork(c0)
    for c in (c0, c1, c2):
        a.append_tokens(c, B)              # 5, 6, 7
    c3 = a.new_seq()
    a.tables[c3] = [type(a.tables[c0][0])(0, B)]
    a.refcount[0] += 1
    a.append_tokens(c3, 3 * B)             # 2, 4, 8
    cands = {"cand0": c0, "cand1": c1, "cand2": c2, "cand3": c3}
    for name, blocks in g["before"].items():
        assert a.block_ids(cands[name]) == blocks
    a.check()
    # One step: fork survivors, append a token each, then free the old candidates.
    new = {}
    for name, parent in g["survivor_parents"].items():
        new[name] = a.fork(cands[parent])
    for name in sorted(new):
        a.append(new[name])
    freed_before = set(a.free_stack)
    for sid in cands.values():
        a.free_seq(sid)
    freed = sorted(set(a.free_stack) - freed_before)
    assert freed == g["freed"]
    assert sorted(a.block_ids(new[n])[-1] for n in new) == g["new_blocks"]
    for b in g["shared_by_all"]:
        assert all(b in a.block_ids(s) for s in new.values())
        assert a.refcount[b] == 4
    assert a.block_ids(new["new0"])[3] == a.block_ids(new["new1"])[3] == g["shared_01"]
    assert a.block_ids(new["new2"])[3] == a.block_ids(new["new3"])[3] == g["shared_23"]
    a.check()


def test_exhaustion_is_all_or_nothing():
    a = BlockAllocator.create(4, 4)
    s = a.new_seq()
    a.append_tokens(s, 10)                 # 3 blocks
    t = a.new_seq()
    before = (list(a.free_stack), [list(map(lambda e: (e.block, e.filled), a.tables[s]))])
    with pytest.raises(PoolExhausted):
        a.append_tokens(t, 9)              # needs 3, one free
    assert a.tables[t] == []
    assert list(a.free_stack) == before[0]
    a.check()


def test_churn_never_double_owns():
    rng = np.random.default_rng(0)
    a = BlockAllocator.create(64, 8, pop_order=rng.permutation(64))
    live = []
    for step in range(2000):
        r = rng.random()
        if r < 0.4 and a.num_free() > 4:
            s = a.new_seq()
            a.append_tokens(s, int(rng.integers(1, 20)))
            live.append(s)
        elif r < 0.6 and live:
            s = live[int(rng.integers(len(live)))]
            if a.num_free() > 2:
                live.append(a.fork(s))
        elif r < 0.8 and live:
            s = live[int(rng.integers(len(live)))]
            if a.num_free() > 2:
                a.append(s)
        elif live:
            a.free_seq(live.pop(int(rng.integers(len(live)))))
        if step % 100 == 0:
            a.check()
    a.check()


# ---------------------------------------------------------------------------
# seeded workloads
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("name", ["tiny", "opt13b", "shared"])
def test_workload_tables_are_deterministic_and_valid(name):
    t1 = build_tables(name)
    t2 = build_tables(name)
    assert np.array_equal(t1.block_tables, t2.block_tables)
    assert np.array_equal(t1.context_lens, t2.context_lens)
    B = t1.block_size
    seen = {}
    for s in range(t1.num_seqs):
        L = int(t1.context_lens[s])
        nb = -(-L // B)
        row = t1.block_tables[s]
        assert np.all(row[:nb] >= 0) and np.all(row[:nb] < t1.num_blocks)
        assert np.all(row[nb:] == -1)
        for b in row[:nb]:
            seen[int(b)] = seen.get(int(b), 0) + 1
    for b, cnt in seen.items():
        assert t1.refcount[b] == cnt
    if name != "shared":
        assert max(seen.values()) == 1


def test_opt13b_lengths_shape():
    t = build_tables("opt13b")
    L = t.context_lens
    assert L.min() >= 1 and L.max() <= 2048
    assert 150 < np.median(L) < 600
    assert t.num_blocks == math.ceil(1.2 * sum(-(-int(x) // 16) for x in L))


def test_shared_prefix_refcounts():
    t = build_tables("shared")
    pre = t.extra["prefix_blocks"]
    sib = t.extra["siblings"]
    assert pre == 32 and sib == 6 and t.num_seqs == 192
    for g in range(32):
        rows = t.block_tables[g * sib:(g + 1) * sib, :pre]
        assert np.all(rows == rows[0])
        assert np.all(t.refcount[rows[0]] == sib)
        priv = t.block_tables[g * sib:(g + 1) * sib, pre]
        assert len(set(priv.tolist())) == sib
    dup, copies, n = duplicate_shared(t)
    assert len(copies) == 32 * 32 * 5
    flat = [int(b) for s in range(t.num_seqs) for b in dup[s, :-(-int(t.context_lens[s]) // 16)]]
    assert len(flat) == len(set(flat))


def test_llama13b_churn_fragments_pool():
    t = build_tables("llama13b")
    assert t.num_seqs == 256 and t.dtype == "bf16"
    first = t.block_tables[:, 0]
    # after churn, sequence 0's blocks are not simply 0, 1, 2, ...
    nb0 = -(-int(t.context_lens[0]) // 16)
    assert not np.array_equal(t.block_tables[0, :nb0], np.arange(nb0))
    assert len(set(first.tolist())) == 256


@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_longctx_sweep_tables(B):
    t = build_tables("longctx", block_size=B)
    assert t.block_size == B and t.num_seqs == 16
    assert t.context_lens.min() >= 8192 and t.context_lens.max() <= 32768
    assert t.max_blocks == 32768 // B


# ---------------------------------------------------------------------------
# byte accounting against the pages' closed forms
# ---------------------------------------------------------------------------

def test_byte_accounting_closed_forms(golden_dir):
    g = _load(golden_dir, "byte_accounting.json")
    k = g["kv_per_token_opt13b"]
    assert acc.kv_bytes_per_token_hidden(k["layers"], k["hidden"], k["dtype_bytes"]) == k["bytes"] == 800 * 1024
    assert acc.kv_bytes_per_token(40, 40, 128, 2) == k["bytes"]
    seq = g["seq_2048_opt13b"]["tokens"] * k["bytes"]
    assert abs(seq / 2 ** 30 - g["seq_2048_opt13b"]["printed_gb"]) < 0.05
    l = g["llama2_70b"]
    assert acc.kv_bytes_per_token(l["layers"], l["kv_heads"], l["head_dim"], l["dtype_bytes"]) == l["bytes_per_token"]
    for row in g["tail_waste"]:
        B = row["block_size"]
        assert acc.max_tail_waste_tokens(B) == row["max_tokens"]
        mib = row["max_tokens"] * l["bytes_per_token"] / 2 ** 20
        assert abs(mib - row["max_mib"]) < 0.005
        avg = row["avg_tokens_printed"] * l["bytes_per_token"] / 2 ** 20
        assert abs(avg - row["avg_mib"]) < 0.005
    t = g["table"]
    assert acc.num_blocks_for(t["max_model_len"], t["block_size"]) == t["entries"]
    assert acc.table_bytes(t["max_model_len"], t["block_size"]) == t["per_request_kib"] * 1024
    assert acc.table_bytes(t["max_model_len"], t["block_size"], t["requests"]) == t["total_kib"] * 1024
    assert acc.table_bytes(t["max_model_len"], 8, t["requests"]) == t["block_size_8_total_kib"] * 1024


def test_decode_bytes_counts_live_tokens_only():
    d = acc.decode_bytes([1, 16, 17, 0], 40, 128, 2, 16)
    assert d["kv_tokens"] == 34
    assert d["kv"] == 34 * 40 * 128 * 2 * 2
    assert d["table"] == (1 + 1 + 2 + 0) * 4
    assert d["q"] == d["out"] == 4 * 40 * 128 * 2
    assert d["total"] == d["kv"] + d["q"] + d["out"] + d["table"] + 16
