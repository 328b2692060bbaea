"""GPU: the FP8 (e4m3) KV cache at head_dim 64 -- decode over e4m3 pools and
the decode step with the quantising append, one query row per KV head (the
stream kernel: a lane holds 8 codes of a row, 8 lanes a row, a chunk is 64
tokens) and several (the matrix-core kernel) -- against the float64 oracle
(decode_rows_fp8, reshape_and_cache_fp8)."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from oracle import paged_oracle as po  # noqa: E402
from synth import FP8_NAN, normal_16bit, random_e4m3, to_bits  # noqa: E402

from .gpu_util import DEV, assert_close, log  # noqa: E402

D = 64


def _codes(x):
    return x.detach().cpu().contiguous().view(torch.uint8).numpy()


def _case(lengths, H, B, seed, slack=3, exp_lo=0, exp_hi=15):
    """e4m3 pools [N, H, B, 64] with random codes, a random placement, NaN
    codes in every unused slot."""
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


def _oracle(c, q, scale, ks, vs, dtype, kp=None, vp=None):
    kc = _codes(c["kp"]) if kp is None else kp
    vc = _codes(c["vp"]) if vp is None else vp
    return po.decode_rows_fp8(to_bits(q)[:, None], kc, vc, c["tables"], c["lens"], scale, c["B"], dtype, ks,
                              vs)[:, 0]


LENGTHS = [1, 7, 8, 9, 63, 64, 65, 100, 127, 128, 129, 255, 256, 257, 511, 700, 1025, 40, 3, 16, 17]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B", [8, 16, 32, 64])
def test_fp8_d64_decode_every_output(dtype, B):
    H = 3
    c = _case(LENGTHS, H, B, seed=500 + B)
    q = normal_16bit((len(LENGTHS), H, D), dtype, DEV, 501 + B)
    ks, vs = 0.004, 0.006
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    out = pkv.paged_attention_decode_fp8(q, c["kp"], c["vp"], tab, lens, D ** -0.5, ks, vs)
    torch.cuda.synchronize()
    assert_close(to_bits(out), _oracle(c, q, D ** -0.5, ks, vs, dtype), dtype, f"fp8 D=64 decode {dtype} B={B}")


@pytest.mark.parametrize("dtype,B", [("f16", 16), ("bf16", 8), ("f16", 64), ("bf16", 32)])
def test_fp8_d64_decode_step_matches_oracle_and_separate_path(dtype, B):
    """The decode step with the quantising append: the pools get the oracle's
    codes for token L - 1, the output is the oracle's append-then-attend, and
    both equal the separate append + decode bit for bit.  L == 0 appends
    nothing; an out-of-pool last block writes nothing and gives NaN."""
    lengths = [1, 63, 64, 65, 200, 0, 77, 1025, 128, 129]
    H = 4
    c = _case([max(L, 1) for L in lengths], H, B, seed=520 + B)
    c["lens"] = np.asarray(lengths, np.int32)
    c["tables"][6, (77 - 1) // B] = 10 ** 6
    S = len(lengths)
    kn = normal_16bit((S, H, D), dtype, DEV, 521)
    vn = normal_16bit((S, H, D), dtype, DEV, 522)
    q = normal_16bit((S, H, D), dtype, DEV, 523)
    ks, vs = 0.02, 0.03
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    kw, vw = _codes(c["kp"]).copy(), _codes(c["vp"]).copy()
    k1, v1 = c["kp"].clone(), c["vp"].clone()
    out = pkv.paged_attention_decode_append_fp8(q, kn, vn, k1, v1, tab, lens, D ** -0.5, ks, vs)
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
    sub = dict(c, tables=c["tables"][good], lens=c["lens"][good])
    ref = _oracle(sub, q[good], D ** -0.5, ks, vs, dtype, kp=kw, vp=vw)
    assert_close(to_bits(out)[good], ref, dtype, f"fp8 D=64 decode step {dtype} B={B}")


def test_fp8_d64_rows_cut_into_more_than_64_pieces():
    """One 40,000-token sequence over 4 heads: 625 chunks a row, cut into
    about 70 pieces by the balanced split, so the merge takes two rounds."""
    lengths, H, B = [40000], 4, 32
    log("fp8 D=64: one 40k-token row per head")
    c = _case(lengths, H, B, seed=540, exp_lo=4, exp_hi=10)
    q = normal_16bit((1, H, D), "bf16", DEV, 541)
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    desc = pkv.make_pool_desc(c["kp"].shape[0], B, H, D, "bf16")
    info = pkv.decode_launch_info(1, H, c["tables"].shape[1], desc, 0, 1, True, False)
    G = info["workgroups"] * info["waves_per_workgroup"]
    chunks = -(-lengths[0] // 64)
    total = H * chunks
    sl = -(-total // max(1, min(G, total // 8)))
    assert chunks // sl > 64
    out = pkv.paged_attention_decode_fp8(q, c["kp"], c["vp"], tab, lens, D ** -0.5, 0.5, 1.5)
    torch.cuda.synchronize()
    assert_close(to_bits(out), _oracle(c, q, D ** -0.5, 0.5, 1.5, "bf16"), "bf16", "fp8 D=64 long rows")


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B", [8, 16, 32, 64])
@pytest.mark.parametrize("G,Q", [(8, 1), (1, 4), (3, 2)])
def test_fp8_d64_rows_every_output(dtype, B, G, Q):
    """Several query rows per KV head over e4m3 pools at head_dim 64 (the
    matrix-core kernel): grouped heads and several query tokens."""
    Hkv = 2
    lengths = [max(L, Q) for L in LENGTHS]
    c = _case(lengths, Hkv, B, seed=560 + B + G + 10 * Q)
    shape = (len(lengths), Hkv * G, D) if Q == 1 else (len(lengths), Q, Hkv * G, D)
    q = normal_16bit(shape, dtype, DEV, 561 + B)
    ks, vs = 0.004, 0.006
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    if Q == 1:
        out = pkv.paged_attention_decode_fp8(q, c["kp"], c["vp"], tab, lens, D ** -0.5, ks, vs)
    else:
        out = pkv.paged_attention_multi_fp8(q, c["kp"], c["vp"], tab, lens, D ** -0.5, ks, vs)
    torch.cuda.synchronize()
    qb = to_bits(q)
    qb = qb[:, None] if Q == 1 else qb
    ref = po.decode_rows_fp8(qb, _codes(c["kp"]), _codes(c["vp"]), c["tables"], c["lens"], D ** -0.5, B, dtype,
                             ks, vs)
    ref = ref[:, 0] if Q == 1 else ref
    assert_close(to_bits(out), ref, dtype, f"fp8 D=64 rows G={G} Q={Q} {dtype} B={B}")


@pytest.mark.parametrize("G,Q", [(8, 1), (2, 4)])
def test_fp8_d64_rows_long_context_many_pieces(G, Q):
    """Long rows over two KV heads, e4m3 pools at head_dim 64 (the matrix-core
    kernel, 32-token chunks): the longest row is cut into far more than 16
    pieces, so the merge takes their maxima over several rounds before the
    sums; every output against the oracle."""
    Hkv, B, dtype = 2, 16, "bf16"
    lengths = [30000, 17777, 16, 40]
    log(f"fp8 D=64 rows, long contexts: G={G} Q={Q}")
    c = _case(lengths, Hkv, B, seed=580 + 10 * G + Q, exp_lo=4, exp_hi=10)
    desc = pkv.make_pool_desc(c["kp"].shape[0], B, Hkv, D, dtype)
    info = pkv.decode_launch_info(len(lengths), Hkv * G, c["tables"].shape[1], desc, 0, Q, True)
    workers = info["workgroups"] * info["waves_per_workgroup"]
    chunks = [-(-L // 32) for L in lengths]
    total = Hkv * sum(chunks)
    assert max(chunks) // -(-total // max(1, min(workers, total // 8))) > 16
    shape = (len(lengths), Hkv * G, D) if Q == 1 else (len(lengths), Q, Hkv * G, D)
    q = normal_16bit(shape, dtype, DEV, 581 + G + Q)
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    if Q == 1:
        out = pkv.paged_attention_decode_fp8(q, c["kp"], c["vp"], tab, lens, D ** -0.5, 0.5, 1.5)
    else:
        out = pkv.paged_attention_multi_fp8(q, c["kp"], c["vp"], tab, lens, D ** -0.5, 0.5, 1.5)
    torch.cuda.synchronize()
    qb = to_bits(q)
    qb = qb[:, None] if Q == 1 else qb
    ref = po.decode_rows_fp8(qb, _codes(c["kp"]), _codes(c["vp"]), c["tables"], c["lens"], D ** -0.5, B, dtype,
                             0.5, 1.5)
    ref = ref[:, 0] if Q == 1 else ref
    assert_close(to_bits(out), ref, dtype, f"fp8 D=64 rows G={G} Q={Q}, long contexts")


def test_fp8_d64_grouped_decode_step():
    """The decode step with the quantising append and grouped heads at head
    _dim 64 (the append is its own launch): codes and output as the oracle's."""
    lengths = [1, 63, 64, 65, 300, 0]
    H, Hkv, B, dtype = 8, 2, 16, "bf16"
    c = _case([max(L, 1) for L in lengths], Hkv, B, seed=580)
    c["lens"] = np.asarray(lengths, np.int32)
    S = len(lengths)
    kn = normal_16bit((S, Hkv, D), dtype, DEV, 581)
    vn = normal_16bit((S, Hkv, D), dtype, DEV, 582)
    q = normal_16bit((S, H, D), dtype, DEV, 583)
    ks, vs = 0.02, 0.03
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    kw, vw = _codes(c["kp"]).copy(), _codes(c["vp"]).copy()
    out = pkv.paged_attention_decode_append_fp8(q, kn, vn, c["kp"], c["vp"], tab, lens, D ** -0.5, ks, vs)
    torch.cuda.synchronize()
    slots = np.array([int(c["tables"][s, (L - 1) // B]) * B + (L - 1) % B if L > 0 else -1
                      for s, L in enumerate(lengths)], np.int64)
    po.reshape_and_cache_fp8(to_bits(kn), to_bits(vn), kw, vw, slots, B, dtype, ks, vs)
    assert np.array_equal(_codes(c["kp"]), kw) and np.array_equal(_codes(c["vp"]), vw)
    o = po.bits_to_f64(to_bits(out), dtype)
    assert np.all(o[5] == 0)
    good = list(range(5))
    sub = dict(c, tables=c["tables"][good], lens=c["lens"][good])
    ref = po.decode_rows_fp8(to_bits(q)[good][:, None], kw, vw, sub["tables"], sub["lens"], D ** -0.5, B, dtype,
                             ks, vs)[:, 0]
    assert_close(to_bits(out)[good], ref, dtype, "fp8 D=64 grouped decode step")
