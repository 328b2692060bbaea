"""GPU: the FP8 (e4m3) KV cache -- quantising append and decode attention
over e4m3 pools -- against the float64 oracle."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from oracle import paged_oracle as po  # noqa: E402
from synth import (FP8_NAN, build_tables, make_fp8_pools, make_query, normal_16bit, random_e4m3,  # noqa: E402
                   to_bits)

from .gpu_util import DEV, assert_close, log, sample_pairs  # noqa: E402

D = 128


def _codes(x):
    return x.detach().cpu().contiguous().view(torch.uint8).numpy()


def _case(lengths, H, B, seed, slack=3, exp_lo=0, exp_hi=15):
    """e4m3 pools [N, H, B, D] with random codes, a random block placement for
    the given lengths, and every unused slot set to the NaN code."""
    rng = np.random.default_rng(seed)
    nb = [-(-L // B) for L in lengths]
    N = sum(nb) + slack
    perm = rng.permutation(N)
    maxb = max(max(nb), 1)
    tables = np.full((len(lengths), maxb), -1, np.int32)
    live = np.zeros((N, B), bool)
    c = 0
    for s, L in enumerate(lengths):
        tables[s, :nb[s]] = perm[c:c + nb[s]]
        for j in range(L):
            live[perm[c + j // B], j % B] = True
        c += nb[s]
    kp = random_e4m3((N, H, B, D), DEV, seed * 4 + 1, exp_lo, exp_hi)
    vp = random_e4m3((N, H, B, D), DEV, seed * 4 + 2, exp_lo, exp_hi)
    dead = torch.from_numpy(~live).to(DEV)[:, None, :, None].expand(kp.shape)
    for pool in (kp, vp):
        pool.masked_fill_(dead, FP8_NAN)
    return dict(kp=kp, vp=vp, tables=tables, lens=np.asarray(lengths, np.int32), B=B)


def _run(c, q, scale, ks, vs):
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    return pkv.paged_attention_decode_fp8(q, c["kp"], c["vp"], tab, lens, scale, ks, vs)


def _oracle(c, q, scale, ks, vs, dtype):
    return po.decode_rows_fp8(to_bits(q)[:, None], _codes(c["kp"]), _codes(c["vp"]), c["tables"], c["lens"],
                              scale, c["B"], dtype, ks, vs)[:, 0]


LENGTHS = [1, 31, 32, 33, 63, 64, 65, 100, 255, 256, 257, 511, 700, 1025, 40, 3, 16, 17]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_fp8_decode_small_shapes(dtype, B):
    H = 3
    c = _case(LENGTHS, H, B, seed=300 + B)
    q = normal_16bit((len(LENGTHS), H, D), dtype, DEV, 301 + B)
    ks, vs = 0.004, 0.006
    out = _run(c, q, D ** -0.5, ks, vs)
    torch.cuda.synchronize()
    assert_close(to_bits(out), _oracle(c, q, D ** -0.5, ks, vs, dtype), dtype, f"fp8 decode {dtype} B={B}")


@pytest.mark.parametrize("ks,vs", [(1.0, 1.0), (2.0 ** -10, 0.25), (0.037, 3.5)])
def test_fp8_decode_scales(ks, vs):
    """K and V scales far apart, from 2^-10 to 3.5."""
    lengths = [5, 90, 333, 1, 64]
    c = _case(lengths, 2, 16, seed=320, exp_lo=0, exp_hi=10)
    q = normal_16bit((len(lengths), 2, D), "f16", DEV, 321)
    out = _run(c, q, 0.02, ks, vs)
    torch.cuda.synchronize()
    assert_close(to_bits(out), _oracle(c, q, 0.02, ks, vs, "f16"), "f16", f"fp8 scales k={ks} v={vs}")


def test_fp8_decode_opt13b_shape_sampled():
    """The OPT-13B decode batch (64 sequences x 40 heads x 128, B=16, lengths
    43 .. 1824) over e4m3 pools; sampled (sequence, head) pairs against the
    oracle, which walks the real block table over host copies of each head."""
    t = build_tables("opt13b")
    log(f"fp8 opt13b: {t.num_seqs} seqs x {t.num_heads} heads, {t.num_blocks} blocks")
    kp, vp = make_fp8_pools(t, DEV)
    q = make_query(t, DEV)
    tab = torch.from_numpy(np.ascontiguousarray(t.block_tables)).to(DEV)
    lens = torch.from_numpy(np.ascontiguousarray(t.context_lens)).to(DEV)
    ks, vs = 1.0 / 60, 1.0 / 60
    out = pkv.paged_attention_decode_fp8(q, kp, vp, tab, lens, t.scale, ks, vs)
    torch.cuda.synchronize()
    rng = np.random.default_rng(330)
    pairs = sample_pairs(t, rng)
    qb = to_bits(q)
    ob = to_bits(out)
    heads = sorted({h for _, h in pairs})
    for h in heads:
        kh = _codes(kp[:, h:h + 1])
        vh = _codes(vp[:, h:h + 1])
        ss = [s for s, hh in pairs if hh == h]
        ref = po.decode_rows_fp8(qb[ss][:, None, h:h + 1], kh, vh, t.block_tables[ss], t.context_lens[ss],
                                 t.scale, t.block_size, t.dtype, ks, vs)[:, 0, 0]
        assert_close(ob[ss, h], ref, t.dtype, f"fp8 opt13b head {h} ({len(ss)} seqs)")


def test_fp8_decode_edge_cases():
    """L == 0 gives zeros; L past the table and a table entry outside the pool
    give NaN rows; other rows are unaffected; NaN codes in unused slots never
    leak into results."""
    lengths = [0, 37, 80, 5, 3000]
    c = _case([max(L, 1) if L < 3000 else 1 for L in lengths], 2, 16, seed=340)
    c["lens"] = np.asarray(lengths, np.int32)  # 3000 > max_blocks * 16
    c["tables"][2, 3] = 10 ** 6
    q = normal_16bit((len(lengths), 2, D), "bf16", DEV, 341)
    out = po.bits_to_f64(to_bits(_run(c, q, 0.1, 0.01, 0.01)), "bf16")
    assert np.all(out[0] == 0)
    assert np.all(np.isnan(out[2])) and np.all(np.isnan(out[4]))
    good = [1, 3]
    sub = dict(c)
    sub["tables"] = c["tables"][good]
    sub["lens"] = c["lens"][good]
    ref = _oracle(sub, q[good], 0.1, 0.01, 0.01, "bf16")
    assert_close(po.f64_to_bits(out[good], "bf16"), ref, "bf16", "fp8 edge: valid sequences")


def test_fp8_decode_placement_and_run_to_run_bitwise():
    lengths = [300, 17, 1000, 64, 1]
    a = _case(lengths, 4, 16, seed=350)
    q = normal_16bit((len(lengths), 4, D), "f16", DEV, 351)
    o1 = _run(a, q, 0.09, 0.02, 0.03)
    o2 = _run(a, q, 0.09, 0.02, 0.03)
    rng = np.random.default_rng(352)
    N = a["kp"].shape[0]
    perm = rng.permutation(N)
    inv = torch.from_numpy(np.argsort(perm)).to(DEV)
    b = dict(a)
    b["kp"] = a["kp"][inv].contiguous()
    b["vp"] = a["vp"][inv].contiguous()
    b["tables"] = np.where(a["tables"] >= 0, perm[np.maximum(a["tables"], 0)], -1).astype(np.int32)
    o3 = _run(b, q, 0.09, 0.02, 0.03)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))


def _append_inputs(T, H, Dh, dtype, seed, strided):
    g = normal_16bit((T, 3, H, Dh) if strided else (T, 2, H, Dh), dtype, DEV, seed)
    g.mul_(40.0)  # many values past 448 * scale: saturation
    flat = g.view(-1)
    n = flat.numel()
    idx = torch.from_numpy(np.random.default_rng(seed).choice(n, 60, replace=False)).to(DEV)
    specials = torch.tensor([float("inf"), -float("inf"), float("nan"), -0.0, 0.0, 1e-7, -3e-8, 65504.0, -448.0,
                             6e-5, 1e-30, -1e-30] * 5, dtype=g.dtype, device=DEV)
    flat[idx] = specials
    return g[:, 0], g[:, 1]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("Dh,B,strided", [(128, 16, False), (64, 8, True), (128, 64, True), (64, 32, False)])
def test_fp8_append_bit_exact(dtype, Dh, B, strided):
    """Quantised rows land in their slots bit for bit (NaN in, NaN code out);
    negative and out-of-pool slots are skipped; other slots keep their codes."""
    T, H = 301, 3
    N = -(-T // B) + 4
    k, v = _append_inputs(T, H, Dh, dtype, 360 + Dh + B, strided)
    rng = np.random.default_rng(361)
    slots = rng.permutation(N * B)[:T].astype(np.int64)
    slots[rng.choice(T, 20, replace=False)] = -1
    slots[rng.choice(T, 5, replace=False)] = N * B + 7
    kp = random_e4m3((N, H, B, Dh), DEV, 362, 0, 15)
    vp = random_e4m3((N, H, B, Dh), DEV, 363, 0, 15)
    kw, vw = _codes(kp).copy(), _codes(vp).copy()
    ks, vs = 0.05, 0.75
    pkv.reshape_and_cache_fp8(k, v, kp, vp, torch.from_numpy(slots).to(DEV), ks, vs)
    torch.cuda.synchronize()
    po.reshape_and_cache_fp8(to_bits(k.contiguous()), to_bits(v.contiguous()), kw, vw, slots, B, dtype, ks, vs)
    for got, want, name in ((_codes(kp), kw, "k"), (_codes(vp), vw, "v")):
        nan_want = (want & 0x7F) == 0x7F
        assert np.array_equal((got & 0x7F) == 0x7F, nan_want), f"{name}: NaN codes differ"
        assert np.array_equal(got[~nan_want], want[~nan_want]), \
            f"{name}: {int((got != want).sum())} codes differ"


def test_fp8_append_then_decode_round_trip():
    """History appended through the quantising append, then decoded: equal to
    the oracle's append followed by the oracle's attention."""
    lengths = [1, 50, 129, 400]
    B, H = 16, 2
    c = _case(lengths, H, B, seed=370)
    kp, vp = c["kp"], c["vp"]
    kw, vw = _codes(kp).copy(), _codes(vp).copy()
    seq = np.concatenate([np.full(L, s) for s, L in enumerate(lengths)])
    pos = np.concatenate([np.arange(L) for L in lengths])
    slots = np.array([c["tables"][s, p // B] * B + p % B for s, p in zip(seq, pos)], np.int64)
    k = normal_16bit((len(seq), H, D), "f16", DEV, 371)
    v = normal_16bit((len(seq), H, D), "f16", DEV, 372)
    ks, vs = 4.5 / 448, 4.5 / 448
    pkv.reshape_and_cache_fp8(k, v, kp, vp, torch.from_numpy(slots).to(DEV), ks, vs)
    po.reshape_and_cache_fp8(to_bits(k), to_bits(v), kw, vw, slots, B, "f16", ks, vs)
    assert np.array_equal(_codes(kp), kw) and np.array_equal(_codes(vp), vw)
    q = normal_16bit((len(lengths), H, D), "f16", DEV, 373)
    out = _run(c, q, D ** -0.5, ks, vs)
    torch.cuda.synchronize()
    ref = po.decode_rows_fp8(to_bits(q)[:, None], kw, vw, c["tables"], c["lens"], D ** -0.5, B, "f16", ks, vs)
    assert_close(to_bits(out), ref[:, 0], "f16", "fp8 append then decode")


@pytest.mark.parametrize("dtype,B", [("f16", 16), ("bf16", 8), ("f16", 64)])
def test_fp8_fused_append_matches_oracle_and_separate_path(dtype, B):
    """The fused step writes the same codes as the quantising append and
    returns the oracle's append-then-attend result; it equals the separate
    append + decode bit for bit.  L == 0 appends nothing; an out-of-pool last
    block writes nothing and gives NaN."""
    lengths = [1, 31, 32, 33, 200, 0, 77, 1025, 64]
    H = 3
    c = _case([max(L, 1) for L in lengths], H, B, seed=390 + B)
    c["lens"] = np.asarray(lengths, np.int32)
    c["tables"][6, (77 - 1) // B] = 10 ** 6  # sequence 6: its last block is outside the pool
    S = len(lengths)
    kn = normal_16bit((S, H, D), dtype, DEV, 391)
    vn = normal_16bit((S, H, D), dtype, DEV, 392)
    q = normal_16bit((S, H, D), dtype, DEV, 393)
    ks, vs = 0.02, 0.03
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    kw, vw = _codes(c["kp"]).copy(), _codes(c["vp"]).copy()
    k1, v1 = c["kp"].clone(), c["vp"].clone()
    out = pkv.paged_attention_decode_append_fp8(q, kn, vn, k1, v1, tab, lens, D ** -0.5, ks, vs)
    # the separate path: slots of token L - 1, the quantising append, then decode
    k2, v2 = c["kp"].clone(), c["vp"].clone()
    slots = np.array([int(c["tables"][s, (L - 1) // B]) * B + (L - 1) % B if L > 0 else -1
                      for s, L in enumerate(lengths)], np.int64)
    slots[6] = -1
    pkv.reshape_and_cache_fp8(kn, vn, k2, v2, torch.from_numpy(slots).to(DEV), ks, vs)
    out2 = pkv.paged_attention_decode_fp8(q, k2, v2, tab, lens, D ** -0.5, ks, vs)
    torch.cuda.synchronize()
    po.reshape_and_cache_fp8(to_bits(kn), to_bits(vn), kw, vw, slots, B, dtype, ks, vs)
    assert np.array_equal(_codes(k1), kw) and np.array_equal(_codes(v1), vw)
    assert np.array_equal(_codes(k2), kw) and np.array_equal(_codes(v2), vw)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    o = po.bits_to_f64(to_bits(out), dtype)
    assert np.all(o[5] == 0) and np.all(np.isnan(o[6]))
    good = [i for i in range(S) if i not in (5, 6)]
    ref = po.decode_rows_fp8(to_bits(q)[good][:, None], kw, vw, c["tables"][good], c["lens"][good], D ** -0.5, B,
                             dtype, ks, vs)[:, 0]
    assert_close(to_bits(out)[good], ref, dtype, f"fp8 fused append {dtype} B={B}")


def test_fp8_fused_append_many_short_rows():
    """Short contexts put many rows' last chunks into one wavefront's slice
    (a slice is at least 8 chunks): more appends than a wavefront stages, so
    the extra ones take the direct-write path.  Same checks as above."""
    rng = np.random.default_rng(395)
    lengths = [int(x) for x in rng.integers(1, 41, 48)]
    H, B, dtype = 4, 16, "bf16"
    c = _case(lengths, H, B, seed=396)
    S = len(lengths)
    kn = normal_16bit((S, H, D), dtype, DEV, 397)
    vn = normal_16bit((S, H, D), dtype, DEV, 398)
    q = normal_16bit((S, H, D), dtype, DEV, 399)
    ks, vs = 0.05, 0.04
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    kw, vw = _codes(c["kp"]).copy(), _codes(c["vp"]).copy()
    k1, v1 = c["kp"].clone(), c["vp"].clone()
    out = pkv.paged_attention_decode_append_fp8(q, kn, vn, k1, v1, tab, lens, 0.09, ks, vs)
    k2, v2 = c["kp"].clone(), c["vp"].clone()
    slots = np.array([int(c["tables"][s, (L - 1) // B]) * B + (L - 1) % B for s, L in enumerate(lengths)], np.int64)
    pkv.reshape_and_cache_fp8(kn, vn, k2, v2, torch.from_numpy(slots).to(DEV), ks, vs)
    out2 = pkv.paged_attention_decode_fp8(q, k2, v2, tab, lens, 0.09, ks, vs)
    torch.cuda.synchronize()
    po.reshape_and_cache_fp8(to_bits(kn), to_bits(vn), kw, vw, slots, B, dtype, ks, vs)
    assert np.array_equal(_codes(k1), kw) and np.array_equal(_codes(v1), vw)
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    ref = po.decode_rows_fp8(to_bits(q)[:, None], kw, vw, c["tables"], c["lens"], 0.09, B, dtype, ks, vs)[:, 0]
    assert_close(to_bits(out), ref, dtype, "fp8 fused append, short rows")


def test_fp8_unsupported_shapes_are_rejected():
    c = _case([20, 30], 2, 16, seed=380)
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    q = normal_16bit((2, 34, D), "f16", DEV, 381)  # 17 query heads per KV head
    with pytest.raises(pkv.PagedKVError):
        pkv.paged_attention_decode_fp8(q, c["kp"], c["vp"], tab, lens, 0.1, 1.0, 1.0)
    q = normal_16bit((2, 2, D), "f16", DEV, 382)
    with pytest.raises(pkv.PagedKVError):  # a zero scale
        pkv.paged_attention_decode_fp8(q, c["kp"], c["vp"], tab, lens, 0.1, 0.0, 1.0)
