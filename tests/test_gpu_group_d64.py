"""GPU: the matrix-core kernel (several query rows per KV head: grouped-query
heads, several query tokens) at head_dim 64, against the float64 oracle's
decode_rows.  At 64, S^T takes two k-slices and O^T four 16-dim slices, whose
operand rows are dims 8(m % 8) + 2s + m / 8; a lane swap then gives each lane
two whole runs of 8 dims."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from oracle import paged_oracle as po  # noqa: E402
from synth import nan_bits, normal_16bit, to_bits  # noqa: E402

from .gpu_util import DEV, assert_close, log  # noqa: E402

D = 64


def _case(lengths, Hkv, B, dtype, seed, slack=3):
    """Pools [N, Hkv, B, 64], a random placement, unused slots NaN."""
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
    kp = normal_16bit((N, Hkv, B, D), dtype, DEV, seed * 4 + 1)
    vp = normal_16bit((N, Hkv, B, D), dtype, DEV, seed * 4 + 2)
    dead = torch.from_numpy(~live).to(DEV)[:, None, :, None].expand(kp.shape)
    nb_ = nan_bits(dtype)
    for pool in (kp, vp):
        pool.view(torch.int16).masked_fill_(dead, nb_ - 0x10000 if nb_ >= 0x8000 else nb_)
    return dict(kp=kp, vp=vp, tables=tables, lens=np.asarray(lengths, np.int32), B=B)


def _run(c, q, scale):
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    if q.dim() == 3:
        return pkv.paged_attention_decode(q, c["kp"], c["vp"], tab, lens, scale)
    return pkv.paged_attention_multi(q, c["kp"], c["vp"], tab, lens, scale)


def _oracle(c, q, scale, dtype):
    qb = to_bits(q)
    if qb.ndim == 3:
        qb = qb[:, None]
    ref = po.decode_rows(qb, to_bits(c["kp"]), to_bits(c["vp"]), c["tables"], c["lens"], scale, c["B"], dtype)
    return ref[:, 0] if q.dim() == 3 else ref


LENGTHS = [1, 15, 16, 17, 31, 33, 64, 100, 255, 256, 257, 511, 700, 1025, 40, 3]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("B", [8, 16, 32, 64])
@pytest.mark.parametrize("G,Q", [(8, 1), (4, 1), (16, 1), (1, 4), (2, 4), (3, 2)])
def test_d64_rows_every_output(dtype, B, G, Q):
    Hkv = 2
    lengths = [max(L, Q) for L in LENGTHS]
    c = _case(lengths, Hkv, B, dtype, seed=2000 + 10 * B + G + 100 * Q)
    shape = (len(lengths), Hkv * G, D) if Q == 1 else (len(lengths), Q, Hkv * G, D)
    q = normal_16bit(shape, dtype, DEV, 177 + G + Q)
    out = _run(c, q, D ** -0.5)
    torch.cuda.synchronize()
    assert_close(to_bits(out), _oracle(c, q, D ** -0.5, dtype), dtype, f"D=64 rows G={G} Q={Q} {dtype} B={B}")


def test_d64_rows_long_context_many_pieces():
    """Two long sequences over 2 KV heads x 8 query heads: rows cut into many
    pieces, merged by the matrix-core merge at head_dim 64."""
    log("D=64 grouped rows, long contexts")
    lengths = [30000, 17777]
    c = _case(lengths, 2, 16, "bf16", seed=2101)
    q = normal_16bit((2, 16, D), "bf16", DEV, 2102)
    out = _run(c, q, D ** -0.5)
    torch.cuda.synchronize()
    assert_close(to_bits(out), _oracle(c, q, D ** -0.5, "bf16"), "bf16", "D=64 rows, long contexts")


def test_d64_rows_edges_and_step_with_append():
    """L = 0 gives zeros, L < Q and an out-of-pool entry give NaN rows; the
    decode step with the append (grouped heads: its own launch) writes the
    oracle's slots and returns the oracle's output."""
    lengths = [0, 37, 80, 5, 200]
    c = _case([max(L, 1) for L in lengths], 2, 16, "f16", seed=2201)
    c["lens"] = np.asarray(lengths, np.int32)
    c["tables"][2, 3] = 10 ** 6
    q = normal_16bit((5, 3, 2 * 4, D), "f16", DEV, 2202)  # 3 query tokens, 4 query heads per KV head
    lens2 = c["lens"].copy()
    lens2[3] = 2  # shorter than the 3 query tokens
    c2 = dict(c, lens=lens2)
    out = po.bits_to_f64(to_bits(_run(c2, q, 0.1)), "f16")
    assert np.all(out[0] == 0)
    assert np.all(np.isnan(out[2])) and np.all(np.isnan(out[3]))
    good = [1, 4]
    sub = dict(c2, tables=c2["tables"][good], lens=c2["lens"][good])
    ref = _oracle(sub, q[good], 0.1, "f16")
    assert_close(to_bits(_run(c2, q, 0.1))[good], ref, "f16", "D=64 edges: valid rows")

    # the decode step with the append, grouped heads (4 query heads per KV head)
    lengths = [1, 33, 64, 65, 300]
    c = _case(lengths, 2, 16, "bf16", seed=2301)
    S, H = len(lengths), 8
    kn = normal_16bit((S, 2, D), "bf16", DEV, 2302)
    vn = normal_16bit((S, 2, D), "bf16", DEV, 2303)
    q = normal_16bit((S, H, D), "bf16", DEV, 2304)
    kpo, vpo = to_bits(c["kp"]), to_bits(c["vp"])
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    out = pkv.paged_attention_decode_append(q, kn, vn, c["kp"], c["vp"], tab, lens, D ** -0.5)
    torch.cuda.synchronize()
    slots = po.slot_mapping(c["tables"], np.arange(S), c["lens"] - 1, 16)
    po.reshape_and_cache(to_bits(kn), to_bits(vn), kpo, vpo, slots, 16)
    assert np.array_equal(to_bits(c["kp"]), kpo) and np.array_equal(to_bits(c["vp"]), vpo)
    ref = po.decode_rows(to_bits(q)[:, None], kpo, vpo, c["tables"], c["lens"], D ** -0.5, 16, "bf16")[:, 0]
    assert_close(to_bits(out), ref, "bf16", "D=64 grouped decode step")


def test_d64_rows_placement_and_repeat_bitwise():
    lengths = [300, 17, 1000, 64, 1]
    a = _case(lengths, 2, 16, "f16", seed=2401)
    q = normal_16bit((len(lengths), 16, D), "f16", DEV, 2402)
    o1 = _run(a, q, 0.1)
    o2 = _run(a, q, 0.1)
    rng = np.random.default_rng(2403)
    N = a["kp"].shape[0]
    perm = rng.permutation(N)
    inv = torch.from_numpy(np.argsort(perm)).to(DEV)
    b = dict(a, kp=a["kp"][inv].contiguous(), vp=a["vp"][inv].contiguous(),
             tables=np.where(a["tables"] >= 0, perm[np.maximum(a["tables"], 0)], -1).astype(np.int32))
    o3 = _run(b, q, 0.1)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16))
