"""GPU: the two passes of the e4m3 decode as separate calls
(pkv_decode_partitions_fp8, then pkv_decode_merge_fp8) against the one call
(pkv_paged_attention_decode_fp8 / pkv_paged_attention_multi_fp8) and the
float64 oracle.  The rows are long enough that the balanced split cuts them
into many pieces, so the merge pass has work; the batch also holds an empty
context (zeros) and rows of a single token."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from oracle import paged_oracle as po  # noqa: E402
from synth import FP8_NAN, normal_16bit, random_e4m3, to_bits  # noqa: E402

from .gpu_util import DEV, assert_close, log  # noqa: E402

LENGTHS = [3000, 1500, 0, 700, 33, 2000, 4]


def _case(D, Hkv, B, seed):
    rng = np.random.default_rng(seed)
    nb = [-(-L // B) for L in LENGTHS]
    N = sum(nb) + 3
    perm = rng.permutation(N)
    tables = np.full((len(LENGTHS), max(nb)), -1, np.int32)
    live = np.zeros((N, B), bool)
    c = 0
    for s, L in enumerate(LENGTHS):
        tables[s, :nb[s]] = perm[c:c + nb[s]]
        for j in range(L):
            live[perm[c + j // B], j % B] = True
        c += nb[s]
    kp = random_e4m3((N, Hkv, B, D), DEV, seed * 4 + 1, 0, 15)
    vp = random_e4m3((N, Hkv, B, D), DEV, seed * 4 + 2, 0, 15)
    dead = torch.from_numpy(~live).to(DEV)[:, None, :, None].expand(kp.shape)
    for pool in (kp, vp):
        pool.masked_fill_(dead, FP8_NAN)
    return kp, vp, tables


@pytest.mark.parametrize("D", [128, 64])
@pytest.mark.parametrize("G,Q", [(1, 1), (8, 1), (4, 1), (1, 4), (2, 4)])
def test_two_passes_equal_the_one_call(G, Q, D):
    dtype = "bf16" if G != 4 else "f16"
    log(f"e4m3 split + merge as two calls: G={G} Q={Q} D={D} {dtype}")
    Hkv, B = 2, 16
    kp, vp, tables = _case(D, Hkv, B, 4100 + 10 * G + Q + D)
    S = len(LENGTHS)
    lens_np = np.asarray([max(L, Q) if L else 0 for L in LENGTHS], np.int32)
    shape = (S, Hkv * G, D) if Q == 1 else (S, Q, Hkv * G, D)
    q = normal_16bit(shape, dtype, DEV, 4200 + G + Q)
    tab = torch.from_numpy(tables).to(DEV)
    lens = torch.from_numpy(lens_np).to(DEV)
    scale, ks, vs = D ** -0.5, 0.004, 0.006
    if Q == 1:
        one = pkv.paged_attention_decode_fp8(q, kp, vp, tab, lens, scale, ks, vs)
        need = pkv.fp8_decode_workspace_bytes(S, Hkv * G, tables.shape[1], kp, dtype)
    else:
        one = pkv.paged_attention_multi_fp8(q, kp, vp, tab, lens, scale, ks, vs)
        need = pkv.fp8_multi_workspace_bytes(S, Q, Hkv * G, tables.shape[1], kp, dtype)
    ws = torch.full((max(need, 256),), 0xA5, dtype=torch.uint8, device=DEV)  # stale bytes: nothing may read them
    two = torch.full_like(q, float("nan"))
    pkv.decode_partitions_fp8(q, kp, vp, tab, lens, scale, ks, vs, two, ws)
    pkv.decode_merge_fp8(two, lens, tables.shape[1], kp, ws)
    torch.cuda.synchronize()
    assert torch.equal(two.view(torch.int16), one.view(torch.int16)), "two calls differ from the one call"
    qb = to_bits(q)
    qb = qb[:, None] if Q == 1 else qb
    codes = [x.cpu().contiguous().view(torch.uint8).numpy() for x in (kp, vp)]
    ref = po.decode_rows_fp8(qb, codes[0], codes[1], tables, lens_np, scale, B, dtype, ks, vs)
    ref = ref[:, 0] if Q == 1 else ref
    assert_close(to_bits(two), ref, dtype, f"two calls G={G} Q={Q} D={D}")
    empty = [s for s, L in enumerate(lens_np) if L == 0]
    assert np.all(to_bits(two)[empty] == 0), "empty contexts give zero rows"
