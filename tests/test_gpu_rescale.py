"""GPU: score profiles that drive the online softmax's running maximum.

With N(0, 1) data a row's maximum settles within its first tiles. These
batches scale each token's K row by a factor that depends on its position:
- rising: the maximum climbs by many times the rescale threshold along every
  row, so the reference max is raised (and the sums rescaled) tile after tile;
- spike: one token in the middle of each row scores far above the rest;
- falling: the first tile holds the largest scores and no later tile raises.
Every path that keeps a running maximum is checked against the float64
oracle: the streaming kernel, the matrix-core kernel with grouped heads and
with several query tokens, over 16-bit and e4m3 pools.  The rows are long
enough that the balanced split cuts them, so the pieces' maxima also differ
at the merge."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from oracle import paged_oracle as po  # noqa: E402
from synth import nan_bits, normal_16bit, to_bits  # noqa: E402

from .gpu_util import DEV, assert_close, log  # noqa: E402

D = 128
LENGTHS = [1000, 1500, 700, 64, 17, 2000, 333]
K_SCALE, V_SCALE = 0.5, 0.05  # e4m3 scales: codes of the scaled rows stay inside +-448


def _factor(profile, t, L):
    if profile == "rising":
        return 1.0 + t / 32.0
    if profile == "falling":
        return 1.0 + (L - 1 - t) / 32.0
    return 40.0 if t == L // 2 else 1.0  # spike


def _case(profile, Hkv, B, dtype, seed):
    """Pools [N, Hkv, B, D]: N(0, 1) rows, each live K row multiplied by the
    profile's factor for its position; unused slots hold NaN."""
    rng = np.random.default_rng(seed)
    nb = [-(-L // B) for L in LENGTHS]
    N = sum(nb) + 3
    perm = rng.permutation(N)
    tables = np.full((len(LENGTHS), max(nb)), -1, np.int32)
    fac = np.zeros((N, B), np.float32)
    c = 0
    for s, L in enumerate(LENGTHS):
        tables[s, :nb[s]] = perm[c:c + nb[s]]
        for j in range(L):
            fac[perm[c + j // B], j % B] = _factor(profile, j, L)
        c += nb[s]
    kp = normal_16bit((N, Hkv, B, D), dtype, DEV, seed * 4 + 1)
    vp = normal_16bit((N, Hkv, B, D), dtype, DEV, seed * 4 + 2)
    f = torch.from_numpy(fac).to(DEV)[:, None, :, None]
    kp = (kp.float() * f).to(kp.dtype)  # rounded once to the pool type: the pool holds these values
    dead = torch.from_numpy(fac == 0).to(DEV)[:, None, :, None].expand(kp.shape)
    nb_ = nan_bits(dtype)
    for pool in (kp, vp):
        pool.view(torch.int16).masked_fill_(dead, nb_ - 0x10000 if nb_ >= 0x8000 else nb_)
    return dict(kp=kp, vp=vp, tables=tables, lens=np.asarray(LENGTHS, np.int32), B=B, dead=dead)


def _fp8(c, dtype):
    """e4m3 pools holding the oracle's codes of the 16-bit pools (NaN codes in unused slots)."""
    out = []
    for pool, sc in ((c["kp"], K_SCALE), (c["vp"], V_SCALE)):
        codes = po.quantize_e4m3(to_bits(pool), dtype, sc)
        t = torch.from_numpy(codes).to(DEV)
        t.masked_fill_(c["dead"], 0x7F)
        out.append(t)
    return out


@pytest.mark.parametrize("profile", ["rising", "spike", "falling"])
@pytest.mark.parametrize("kind", ["mha", "grouped", "multi", "mha_fp8", "grouped_fp8"])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_running_max_profiles(profile, kind, dtype):
    log(f"running max: {profile} {kind} {dtype}")
    B, S = 16, len(LENGTHS)
    G, Q = {"mha": (1, 1), "grouped": (8, 1), "multi": (1, 4), "mha_fp8": (1, 1), "grouped_fp8": (8, 1)}[kind]
    Hkv = 2
    c = _case(profile, Hkv, B, dtype, 700 + len(kind) + (0 if dtype == "f16" else 50))
    shape = (S, Hkv * G, D) if Q == 1 else (S, Q, Hkv * G, D)
    q = normal_16bit(shape, dtype, DEV, 701)
    tab = torch.from_numpy(c["tables"]).to(DEV)
    lens = torch.from_numpy(c["lens"]).to(DEV)
    scale = D ** -0.5
    qb = to_bits(q)
    qb = qb[:, None] if Q == 1 else qb
    if kind.endswith("fp8"):
        kc, vc = _fp8(c, dtype)
        out = pkv.paged_attention_decode_fp8(q, kc, vc, tab, lens, scale, K_SCALE, V_SCALE)
        torch.cuda.synchronize()
        ref = po.decode_rows_fp8(qb, kc.cpu().numpy(), vc.cpu().numpy(), c["tables"], c["lens"], scale, B, dtype,
                                 K_SCALE, V_SCALE)
    else:
        if Q == 1:
            out = pkv.paged_attention_decode(q, c["kp"], c["vp"], tab, lens, scale)
        else:
            out = pkv.paged_attention_multi(q, c["kp"], c["vp"], tab, lens, scale)
        torch.cuda.synchronize()
        ref = po.decode_rows(qb, to_bits(c["kp"]), to_bits(c["vp"]), c["tables"], c["lens"], scale, B, dtype)
    ref = ref[:, 0] if Q == 1 else ref
    assert_close(to_bits(out), ref, dtype, f"{profile} {kind} {dtype}")
