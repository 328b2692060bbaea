"""Pins for the float64 oracle: each check ties the oracle to something other
than itself (brute force, a library routine, a closed form, an invariant the
pages state, or a worked example printed on a page).

The mutation tests at the end plant plausible mistakes into copies of oracle
functions (on the CPU) and show that a pin here catches each of them.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
from oracle import paged_oracle as po
from synth import BlockAllocator

RNG = np.random.default_rng(7)


def _bits(x, dtype="f16"):
    x = np.asarray(x, dtype=np.float32)
    if dtype == "f16":
        return x.astype(np.float16).view(np.uint16)
    import torch
    return torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def _paged_case(lengths, H, D, B, dtype="f16", rng=None, extra_blocks=3, poison=True):
    """Logical K/V per sequence, scattered into pools through the oracle's own
    append, with random physical placement.  Returns everything needed to
    compare paged results with unpaged brute force."""
    rng = rng or RNG
    S = len(lengths)
    # values first, so the same seed gives the same logical K/V at any B
    q = _bits(rng.standard_normal((S, H, D)), dtype)
    kl = [_bits(rng.standard_normal((L, H, D)), dtype) for L in lengths]
    vl = [_bits(rng.standard_normal((L, H, D)), dtype) for L in lengths]
    nb = [-(-L // B) for L in lengths]
    N = sum(nb) + extra_blocks
    perm = rng.permutation(N)
    maxb = max(max(nb), 1)
    tables = np.full((S, maxb), -1, dtype=np.int32)
    c = 0
    for s in range(S):
        tables[s, :nb[s]] = perm[c:c + nb[s]]
        c += nb[s]
    fill = 0x7E55 if dtype == "f16" else 0x7FD5
    kp = np.full((N, H, B, D), fill if poison else 0, dtype=np.uint16)
    vp = kp.copy()
    for s in range(S):
        seq = np.full(lengths[s], s)
        pos = np.arange(lengths[s])
        slots = po.slot_mapping(tables, seq, pos, B)
        po.reshape_and_cache(kl[s], vl[s], kp, vp, slots, B)
    return dict(q=q, kl=kl, vl=vl, kp=kp, vp=vp, tables=tables,
                lens=np.asarray(lengths, dtype=np.int32), B=B, dtype=dtype)


# ---------------------------------------------------------------------------
# brute force and library special cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("B", [1, 2, 4, 16])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_decode_matches_dense_causal_brute_force(B, dtype):
    rng = np.random.default_rng(100 + B)
    lengths = [1, 5, 17, 33, 64]
    H, D = 2, 8
    c = _paged_case(lengths, H, D, B, dtype, rng)
    scale = 1.0 / math.sqrt(D)
    out = po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], scale, B, dtype)
    for s, L in enumerate(lengths):
        for h in range(H):
            K = po.bits_to_f64(c["kl"][s][:, h], dtype)
            V = po.bits_to_f64(c["vl"][s][:, h], dtype)
            Q = np.zeros((L, D))
            Q[:-1] = rng.standard_normal((L - 1, D))  # earlier rows do not matter
            Q[-1] = po.bits_to_f64(c["q"][s, h], dtype)
            ref = po.dense_causal_last_row(Q, K, V, float(np.float32(scale)))
            np.testing.assert_allclose(out[s, h], ref, rtol=1e-12, atol=1e-14)


def test_decode_matches_torch_sdpa_float64():
    torch = pytest.importorskip("torch")
    rng = np.random.default_rng(11)
    lengths = [3, 40, 64]
    H, D, B = 3, 16, 4
    c = _paged_case(lengths, H, D, B, "f16", rng)
    scale = 1.0 / math.sqrt(D)
    out = po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], scale, B, "f16")
    for s, L in enumerate(lengths):
        K = torch.from_numpy(po.bits_to_f64(c["kl"][s], "f16")).permute(1, 0, 2)[None]
        V = torch.from_numpy(po.bits_to_f64(c["vl"][s], "f16")).permute(1, 0, 2)[None]
        Q = torch.zeros((1, H, L, D), dtype=torch.float64)
        Q[0, :, -1] = torch.from_numpy(po.bits_to_f64(c["q"][s], "f16"))
        ref = torch.nn.functional.scaled_dot_product_attention(
            Q, K.contiguous(), V.contiguous(), is_causal=True, scale=float(np.float32(scale)))
        np.testing.assert_allclose(out[s], ref[0, :, -1].numpy(), rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# closed forms and special cases
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_context_one_returns_v_exactly(dtype):
    c = _paged_case([1, 1, 1], 4, 16, 16, dtype, np.random.default_rng(3))
    out = po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.25, 16, dtype)
    for s in range(3):
        assert np.array_equal(out[s], po.bits_to_f64(c["vl"][s][0], dtype))
        assert np.array_equal(po.f64_to_bits(out[s], dtype), c["vl"][s][0])


def test_zero_query_gives_mean_of_values():
    c = _paged_case([37], 2, 8, 4, "f16", np.random.default_rng(4))
    c["q"][:] = 0
    out = po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.3, 4, "f16")
    V = po.bits_to_f64(c["vl"][0], "f16")
    np.testing.assert_allclose(out[0], V.mean(axis=0), rtol=1e-13, atol=1e-15)


def test_equal_keys_give_uniform_weights():
    c = _paged_case([23], 1, 8, 4, "f16", np.random.default_rng(5))
    same = c["kl"][0][0].copy()
    c["kl"][0][:] = same
    for pos in range(23):
        slot = po.slot_of(c["tables"][0], pos, 4)
        c["kp"][slot // 4, :, slot % 4, :] = same
    K = po.bits_to_f64(po.gather(c["kp"], c["tables"][0], 23, 4, 0), "f16")
    q = po.bits_to_f64(c["q"][0, 0], "f16")
    V = po.bits_to_f64(po.gather(c["vp"], c["tables"][0], 23, 4, 0), "f16")
    _, a, _, _ = po.attend(q, K, V, 0.7)
    np.testing.assert_allclose(a, np.full(23, 1 / 23), rtol=1e-14)


def test_dominant_key_and_large_scale_stay_finite():
    rng = np.random.default_rng(6)
    D, L = 16, 50
    q = rng.standard_normal(D)
    K = rng.standard_normal((L, D)) * 0.01
    K[17] = q * 4.0
    V = rng.standard_normal((L, D))
    o, a, m, l = po.attend(q, K, V, 100.0)
    assert np.all(np.isfinite(o))
    assert a[17] > 1 - 1e-12
    np.testing.assert_allclose(o, V[17], atol=1e-10)


def test_softmax_weights_sum_to_one():
    rng = np.random.default_rng(8)
    for L in (1, 2, 7, 300, 2048):
        q = rng.standard_normal(64)
        K = rng.standard_normal((L, 64))
        V = rng.standard_normal((L, 64))
        _, a, _, _ = po.attend(q, K, V, 1 / 8)
        assert abs(a.sum() - 1.0) <= L * 2.0 ** -52 + 2.0 ** -52
        assert np.all(a >= 0)


def test_empty_context_is_zero():
    c = _paged_case([5, 9], 2, 8, 4, "f16", np.random.default_rng(9))
    lens = c["lens"].copy()
    lens[1] = 0
    out = po.decode(c["q"], c["kp"], c["vp"], c["tables"], lens, 0.3, 4, "f16")
    assert np.all(out[1] == 0)
    assert np.all(np.isfinite(out[0]))


# ---------------------------------------------------------------------------
# invariants stated on the pages
# ---------------------------------------------------------------------------

def test_physical_placement_does_not_change_result():
    """Blocks may sit anywhere in the pool ("PagedAttention 完全拆解",
    原理详解（二）: splitting into blocks only reorganises the computation)."""
    rng = np.random.default_rng(12)
    lengths = [9, 31, 64, 1]
    a = _paged_case(lengths, 2, 8, 4, "f16", np.random.default_rng(12))
    # same logical data, different permutation
    b = _paged_case(lengths, 2, 8, 4, "f16", np.random.default_rng(12))
    N = b["kp"].shape[0]
    perm = rng.permutation(N)
    kp2 = np.empty_like(b["kp"])
    vp2 = np.empty_like(b["vp"])
    kp2[perm] = b["kp"]
    vp2[perm] = b["vp"]
    t2 = np.where(b["tables"] >= 0, perm[np.maximum(b["tables"], 0)], -1).astype(np.int32)
    assert not np.array_equal(t2, a["tables"])
    o1 = po.decode(a["q"], a["kp"], a["vp"], a["tables"], a["lens"], 0.35, 4, "f16")
    o2 = po.decode(b["q"], kp2, vp2, t2, b["lens"], 0.35, 4, "f16")
    assert np.array_equal(o1, o2)


def test_identity_table_equals_contiguous_storage():
    rng = np.random.default_rng(13)
    L, H, D, B = 29, 2, 8, 4
    q = _bits(rng.standard_normal((1, H, D)))
    k = _bits(rng.standard_normal((L, H, D)))
    v = _bits(rng.standard_normal((L, H, D)))
    nb = -(-L // B)
    kp = np.zeros((nb, H, B, D), dtype=np.uint16)
    vp = np.zeros_like(kp)
    for pos in range(L):
        kp[pos // B, :, pos % B] = k[pos]
        vp[pos // B, :, pos % B] = v[pos]
    table = np.arange(nb, dtype=np.int32)[None]
    out = po.decode(q, kp, vp, table, np.array([L], np.int32), 0.5, B, "f16")
    for h in range(H):
        ref, _, _, _ = po.attend(po.bits_to_f64(q[0, h], "f16"), po.bits_to_f64(k[:, h], "f16"),
                                 po.bits_to_f64(v[:, h], "f16"), 0.5)
        assert np.array_equal(out[0, h], ref)


def test_shared_prefix_equals_duplicated_blocks():
    """Reading a shared block is the same as reading a private copy
    ("PagedAttention 完全拆解", 内存共享 / 引用计数)."""
    rng = np.random.default_rng(14)
    B, H, D = 4, 2, 8
    prefix = 12            # 3 full blocks shared by 3 siblings
    priv = [3, 6, 1]
    N = 3 + sum(-(-p // B) for p in priv) + 9
    kp = np.full((N, H, B, D), 0x7E55, dtype=np.uint16)
    vp = kp.copy()
    shared_tab = []
    nxt = 0
    pre = [nxt, nxt + 1, nxt + 2]
    nxt += 3
    kpre = _bits(rng.standard_normal((prefix, H, D)))
    vpre = _bits(rng.standard_normal((prefix, H, D)))
    for i in range(prefix):
        kp[pre[i // B], :, i % B] = kpre[i]
        vp[pre[i // B], :, i % B] = vpre[i]
    kpriv, vpriv = [], []
    for p in priv:
        own = list(range(nxt, nxt + (-(-p // B))))
        nxt += len(own)
        kx = _bits(rng.standard_normal((p, H, D)))
        vx = _bits(rng.standard_normal((p, H, D)))
        for i in range(p):
            kp[own[i // B], :, i % B] = kx[i]
            vp[own[i // B], :, i % B] = vx[i]
        shared_tab.append(pre + own)
        kpriv.append(kx)
        vpriv.append(vx)
    maxb = max(len(t) for t in shared_tab)
    tab = np.full((3, maxb), -1, np.int32)
    for s, t in enumerate(shared_tab):
        tab[s, :len(t)] = t
    # duplicated control: siblings 1 and 2 get private copies of the prefix
    dup = tab.copy()
    for s in (1, 2):
        for j in range(3):
            kp[nxt] = kp[pre[j]]
            vp[nxt] = vp[pre[j]]
            dup[s, j] = nxt
            nxt += 1
    lens = np.array([prefix + p for p in priv], np.int32)
    q = _bits(rng.standard_normal((3, H, D)))
    o1 = po.decode(q, kp, vp, tab, lens, 0.4, B, "f16")
    o2 = po.decode(q, kp, vp, dup, lens, 0.4, B, "f16")
    assert np.array_equal(o1, o2)


def test_block_size_does_not_change_result():
    rng = np.random.default_rng(15)
    lengths = [1, 7, 33, 64]
    outs = []
    for B in (1, 2, 4, 8, 16):
        c = _paged_case(lengths, 2, 8, B, "bf16", np.random.default_rng(15))
        outs.append(po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.3, B, "bf16"))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])


@pytest.mark.parametrize("P", [1, 4, 8, 16, 64])
def test_partitioned_merge_equals_unpartitioned(P):
    c = _paged_case([1, 9, 40, 64, 63], 2, 8, 4, "f16", np.random.default_rng(16))
    o1 = po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.3, 4, "f16")
    o2 = po.decode_partitioned(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.3, 4, "f16", P)
    np.testing.assert_allclose(o2, o1, rtol=1e-12, atol=1e-15)


def test_partials_of_one_partition_are_the_plain_softmax_terms():
    c = _paged_case([20], 1, 8, 4, "f16", np.random.default_rng(17))
    m, l, o = po.partials(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.3, 4, "f16", 64, 0, 0)
    K = po.bits_to_f64(c["kl"][0][:, 0], "f16")
    V = po.bits_to_f64(c["vl"][0][:, 0], "f16")
    q = po.bits_to_f64(c["q"][0, 0], "f16")
    z = [float(np.dot(K[j], q)) * float(np.float32(0.3)) for j in range(20)]
    mm = max(z)
    assert m[0] == mm
    np.testing.assert_allclose(l[0], math.fsum(math.exp(x - mm) for x in z), rtol=1e-14)
    np.testing.assert_allclose(o[0], sum(math.exp(z[j] - mm) * V[j] for j in range(20)), rtol=1e-13)


def test_merge_of_equal_halves():
    """Two partitions with equal max and equal sums average their outputs."""
    m = np.array([0.5, 0.5])
    l = np.array([2.0, 2.0])
    o = np.array([[2.0, 4.0], [6.0, 8.0]])
    np.testing.assert_allclose(po.lse_merge(m, l, o), [2.0, 3.0])
    # a partition whose max is far below contributes nothing
    m = np.array([0.0, -800.0])
    np.testing.assert_allclose(po.lse_merge(m, np.array([1.0, 1.0]), np.array([[1.0], [9.0]])), [1.0])


# ---------------------------------------------------------------------------
# translation and the append, against the pages' worked examples
# ---------------------------------------------------------------------------

def _load(golden_dir, name):
    with open(os.path.join(golden_dir, name)) as f:
        return json.load(f)


@pytest.mark.parametrize("name", ["fig6_decode_walkthrough.json", "lp_sec23_translation.json"])
def test_slot_rule_on_worked_examples(golden_dir, name):
    g = _load(golden_dir, name)
    B = g["block_size"]
    blocks = g.get("after_decode_2", g)["blocks"]
    row = np.array(blocks, np.int32)
    for pos, blk, off in g["token_block_offset"]:
        slot = po.slot_of(row, pos, B)
        assert (slot // B, slot % B) == (blk, off)


def test_block_table_ranges_b16(golden_dir):
    g = _load(golden_dir, "ga_table_b16.json")
    B = g["block_size"]
    row = np.array([905, 3, 4242], np.int32)
    for r in g["rows"]:
        for pos in range(r["first_token"], r["last_token"] + 1):
            assert po.slot_of(row, pos, B) // B == row[r["table_index"]]
        assert pos // B == r["logical_block"]


def test_append_writes_exact_rows_and_nothing_else():
    rng = np.random.default_rng(18)
    N, H, B, D = 6, 3, 4, 8
    kp = np.full((N, H, B, D), 0x7E55, np.uint16)
    vp = kp.copy()
    k = rng.integers(0, 0x7C00, size=(5, H, D)).astype(np.uint16)
    v = rng.integers(0, 0x7C00, size=(5, H, D)).astype(np.uint16)
    slots = np.array([5, -1, 23, 0, N * B + 2], np.int64)
    kp0, vp0 = kp.copy(), vp.copy()
    po.reshape_and_cache(k, v, kp, vp, slots, B)
    touched = np.zeros((N, B), bool)
    for t, slot in enumerate(slots):
        if 0 <= slot < N * B:
            assert np.array_equal(kp[slot // B, :, slot % B], k[t])
            assert np.array_equal(vp[slot // B, :, slot % B], v[t])
            touched[slot // B, slot % B] = True
    untouched = ~touched[:, None, :, None].repeat(H, 1).repeat(D, 3)
    assert np.array_equal(kp[untouched], kp0[untouched])
    assert np.array_equal(vp[untouched], vp0[untouched])


def _fig8_copy_on_write_holds(copy_fn, golden_dir) -> bool:
    """Figure 8 of [PA] 内存共享 run through the allocator and the oracle's
    append: after A1's copy-on-write (done by ``copy_fn``) and one new token per
    sample, both samples read the prompt's 7 rows unchanged and their own
    eighth row."""
    with open(os.path.join(golden_dir, "fig8_copy_on_write.json")) as f:
        g = json.load(f)
    B, H, D, N = g["block_size"], 2, 8, 16
    head = g["pop_order_head"]
    a = BlockAllocator.create(N, B, pop_order=list(head) + [b for b in range(N) if b not in head])
    rng = np.random.default_rng(24)
    kp = np.full((N, H, B, D), 0x7E55, np.uint16)
    vp = kp.copy()
    a1 = a.new_seq()
    prompt_k = rng.integers(0, 0x7C00, size=(g["prompt_tokens"], H, D)).astype(np.uint16)
    prompt_v = rng.integers(0, 0x7C00, size=(g["prompt_tokens"], H, D)).astype(np.uint16)
    slots = []
    for _ in range(g["prompt_tokens"]):
        e = a.append(a1)
        slots.append(e.block * B + e.filled - 1)
    po.reshape_and_cache(prompt_k, prompt_v, kp, vp, np.array(slots, np.int64), B)
    a2 = a.fork(a1)
    new = {}
    for sid in (a1, a2):
        e = a.append(sid)
        copy_fn(kp, vp, list(a.copies))
        a.copies.clear()
        k = rng.integers(0, 0x7C00, size=(1, H, D)).astype(np.uint16)
        v = rng.integers(0, 0x7C00, size=(1, H, D)).astype(np.uint16)
        po.reshape_and_cache(k, v, kp, vp, np.array([e.block * B + e.filled - 1], np.int64), B)
        new[sid] = (k[0], v[0])
    L = g["prompt_tokens"] + 1
    for sid in (a1, a2):
        row = np.array(a.block_ids(sid) + [-1] * 4, np.int32)
        for h in range(H):
            K = po.gather(kp, row, L, B, h)
            V = po.gather(vp, row, L, B, h)
            if not (np.array_equal(K[:-1], prompt_k[:, h]) and np.array_equal(V[:-1], prompt_v[:, h])):
                return False
            if not (np.array_equal(K[-1], new[sid][0][h]) and np.array_equal(V[-1], new[sid][1][h])):
                return False
    return True


def test_copy_blocks_completes_fig8_copy_on_write(golden_dir):
    assert _fig8_copy_on_write_holds(po.copy_blocks, golden_dir)


def test_copy_blocks_pin_catches_planted_mistakes(golden_dir):
    def no_copy(kp, vp, pairs):
        pass

    def swapped(kp, vp, pairs):
        po.copy_blocks(kp, vp, [(d, s_) for s_, d in pairs])

    assert not _fig8_copy_on_write_holds(no_copy, golden_dir)
    assert not _fig8_copy_on_write_holds(swapped, golden_dir)


def test_copy_blocks_exact_and_skips_invalid_pairs():
    rng = np.random.default_rng(25)
    N, H, B, D = 9, 2, 4, 8
    kp = rng.integers(0, 0x7C00, size=(N, H, B, D)).astype(np.uint16)
    vp = rng.integers(0, 0x7C00, size=(N, H, B, D)).astype(np.uint16)
    kp0, vp0 = kp.copy(), vp.copy()
    pairs = [(0, 5), (5, 6), (-1, 7), (2, N), (3, 8)]  # 5 is read before it is overwritten
    po.copy_blocks(kp, vp, pairs)
    for b in range(N):
        want = {5: 0, 6: 5, 8: 3}.get(b, b)
        assert np.array_equal(kp[b], kp0[want]) and np.array_equal(vp[b], vp0[want])
    po.copy_blocks(kp, vp, [])
    assert np.array_equal(kp[0], kp0[0])


# ---------------------------------------------------------------------------
# grouped-query heads and multi-token queries
# ---------------------------------------------------------------------------

def _gqa_pools(rng, S, L_max, Hkv, D, B, dtype):
    lengths = [int(x) for x in rng.integers(1, L_max, size=S)]
    c = _paged_case(lengths, Hkv, D, B, dtype, rng)
    return c, lengths


@pytest.mark.parametrize("G", [2, 4, 8])
def test_grouped_query_equals_mha_over_repeated_kv_heads(G):
    """Query head h of a group reads KV head h // G: the same result as plain
    multi-head decode over a pool in which every KV head is repeated G times."""
    rng = np.random.default_rng(40 + G)
    Hkv, D, B = 2, 8, 4
    c, lengths = _gqa_pools(rng, 5, 40, Hkv, D, B, "f16")
    q = _bits(rng.standard_normal((5, 1, Hkv * G, D)), "f16")
    got = po.decode_rows(q, c["kp"], c["vp"], c["tables"], c["lens"], 0.3, B, "f16")[:, 0]
    kr = np.repeat(c["kp"], G, axis=1)
    vr = np.repeat(c["vp"], G, axis=1)
    ref = po.decode(q[:, 0], kr, vr, c["tables"], c["lens"], 0.3, B, "f16")
    assert np.array_equal(got, ref)
    # planted mistake: heads interleaved over KV heads instead of grouped
    bad = po.decode(q[:, 0], np.tile(c["kp"], (1, G, 1, 1)), np.tile(c["vp"], (1, G, 1, 1)), c["tables"],
                    c["lens"], 0.3, B, "f16")
    assert not np.allclose(bad, ref)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_multi_token_queries_match_dense_causal_brute_force(dtype):
    """The last Q tokens of a sequence, attending causally, equal the last Q
    rows of dense causal attention over the unpaged sequence."""
    rng = np.random.default_rng(44)
    H, D, B, Q = 2, 8, 4, 5
    lengths = [5, 9, 23]
    c = _paged_case(lengths, H, D, B, dtype, rng)
    qb = _bits(rng.standard_normal((len(lengths), Q, H, D)), dtype)
    got = po.decode_rows(qb, c["kp"], c["vp"], c["tables"], c["lens"], 0.35, B, dtype)
    s64 = float(np.float32(0.35))
    for s, L in enumerate(lengths):
        for h in range(H):
            Qfull = np.zeros((L, D))
            Qfull[L - Q:] = po.bits_to_f64(qb[s, :, h], dtype)
            ref = po.dense_causal(Qfull, po.bits_to_f64(c["kl"][s][:, h], dtype),
                                  po.bits_to_f64(c["vl"][s][:, h], dtype), s64)[L - Q:]
            assert np.allclose(got[s, :, h], ref, rtol=1e-12, atol=1e-12)


def test_multi_token_query_i_equals_decode_over_its_prefix():
    rng = np.random.default_rng(45)
    H, D, B, Q = 3, 8, 4, 4
    lengths = [4, 11, 30]
    c = _paged_case(lengths, H, D, B, "f16", rng)
    qb = _bits(rng.standard_normal((len(lengths), Q, H, D)), "f16")
    got = po.decode_rows(qb, c["kp"], c["vp"], c["tables"], c["lens"], 0.35, B, "f16")
    for i in range(Q):
        lens_i = c["lens"] - Q + 1 + i
        ref = po.decode(qb[:, i], c["kp"], c["vp"], c["tables"], lens_i, 0.35, B, "f16")
        assert np.array_equal(got[:, i], ref)


def test_slot_mapping_padding():
    tab = np.array([[4, 2], [0, 1]], np.int32)
    got = po.slot_mapping(tab, [0, -1, 1, 1], [5, 3, -2, 4], 4)
    assert list(got) == [2 * 4 + 1, -1, -1, 1 * 4 + 0]


def test_append_then_decode_round_trip_matches_unpaged():
    """End to end on the oracle side: history and a new token appended through
    the slot rule, then decode, equals attention over the unpaged rows."""
    rng = np.random.default_rng(19)
    lengths = [1, 16, 17, 45]
    c = _paged_case(lengths, 2, 16, 16, "f16", rng)
    out = po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.25, 16, "f16")
    for s, L in enumerate(lengths):
        for h in range(2):
            ref, _, _, _ = po.attend(po.bits_to_f64(c["q"][s, h], "f16"),
                                     po.bits_to_f64(c["kl"][s][:, h], "f16"),
                                     po.bits_to_f64(c["vl"][s][:, h], "f16"), 0.25)
            assert np.array_equal(out[s, h], ref)


# ---------------------------------------------------------------------------
# 16-bit conversions against library routines
# ---------------------------------------------------------------------------

def test_bit_conversions_match_numpy_and_torch():
    torch = pytest.importorskip("torch")
    x = np.random.default_rng(20).standard_normal(4096).astype(np.float32) * 3
    assert np.array_equal(po.f64_to_bits(x, "f16"), x.astype(np.float16).view(np.uint16))
    tb = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(po.f64_to_bits(x.astype(np.float64), "bf16"), tb)
    np.testing.assert_array_equal(po.bits_to_f64(tb, "bf16"),
                                  torch.from_numpy(tb.view(np.int16)).view(torch.bfloat16).double().numpy())


# ---------------------------------------------------------------------------
# planted mistakes: copies of oracle functions with one plausible error each
# must fail the pins above
# ---------------------------------------------------------------------------

def _brute_force_disagrees(decode_fn):
    rng = np.random.default_rng(21)
    lengths = [5, 17, 33]
    H, D, B = 2, 8, 4
    c = _paged_case(lengths, H, D, B, "f16", rng)
    scale = 1.0 / math.sqrt(D)
    out = decode_fn(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], scale, B, "f16")
    for s, L in enumerate(lengths):
        for h in range(H):
            K = po.bits_to_f64(c["kl"][s][:, h], "f16")
            V = po.bits_to_f64(c["vl"][s][:, h], "f16")
            Q = np.zeros((L, D))
            Q[-1] = po.bits_to_f64(c["q"][s, h], "f16")
            ref = po.dense_causal_last_row(Q, K, V, float(np.float32(scale)))
            if not np.allclose(out[s, h], ref, rtol=1e-12, atol=1e-14):
                return True
    return False


def _mutant_decode(mutation):
    def attend(q64, K64, V64, scale64):
        if mutation == "drop_scale":
            scale64 = 1.0
        z = (K64 @ q64) * scale64
        if mutation == "neg_sign":
            z = -z
        m = z.max()
        e = np.exp(z - m)
        a = e / e.sum()
        if mutation == "no_normalise":
            a = e
        return a @ V64

    def decode(q, kp, vp, tables, lens, scale, B, dtype):
        S, H, D = q.shape
        out = np.zeros((S, H, D))
        for s in range(S):
            L = int(lens[s])
            if mutation == "off_by_one_len":
                L -= 1
            for h in range(H):
                rows_k, rows_v = [], []
                for pos in range(L):
                    lb, off = pos // B, pos % B
                    if mutation == "wrong_offset":
                        off = (off + 1) % B
                    if mutation == "wrong_table_index":
                        lb = min(lb + 1, -(-L // B) - 1)
                    blk = int(tables[s, lb])
                    rows_k.append(kp[blk, h, off])
                    rows_v.append(vp[blk, h, off])
                K = po.bits_to_f64(np.array(rows_k), dtype)
                V = po.bits_to_f64(np.array(rows_v), dtype)
                if mutation == "swap_kv":
                    K, V = V, K
                out[s, h] = attend(po.bits_to_f64(q[s, h], dtype), K, V, float(np.float32(scale)))
        return out
    return decode


@pytest.mark.parametrize("mutation", ["drop_scale", "neg_sign", "no_normalise", "off_by_one_len",
                                      "wrong_offset", "wrong_table_index", "swap_kv"])
def test_pins_catch_planted_mistakes(mutation):
    assert _brute_force_disagrees(_mutant_decode(mutation))
    assert not _brute_force_disagrees(_mutant_decode("none"))


def test_merge_pin_catches_dropped_rescale():
    c = _paged_case([40, 64], 1, 8, 4, "f16", np.random.default_rng(22))
    ref = po.decode(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.9, 4, "f16")

    def bad_merge(m, l, o):
        return o.sum(axis=0) / l.sum()   # forgets the exp(m_p - M) factors

    for s in range(2):
        m, l, o = po.partials(c["q"], c["kp"], c["vp"], c["tables"], c["lens"], 0.9, 4, "f16", 8, s, 0)
        assert not np.allclose(bad_merge(m, l, o), ref[s, 0], rtol=1e-9)
        np.testing.assert_allclose(po.lse_merge(m, l, o), ref[s, 0], rtol=1e-12)
