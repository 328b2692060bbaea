"""GPU: a caller's workspace that the kernels could not use is refused by the
binding before anything is launched -- a tensor in host memory (whose address
would reach the kernels as a device address) or a non-contiguous one -- for
every call that takes a workspace."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from synth import normal_16bit, random_e4m3  # noqa: E402

from .gpu_util import DEV  # noqa: E402

D, B, HKV = 128, 16, 2
LENS = [5, 40, 17, 33]


def _batch(fp8):
    rng = np.random.default_rng(77)
    nb = [-(-L // B) for L in LENS]
    N = sum(nb) + 3
    perm = rng.permutation(N)
    tables = np.full((len(LENS), max(nb)), -1, np.int32)
    c = 0
    for s in range(len(LENS)):
        tables[s, :nb[s]] = perm[c:c + nb[s]]
        c += nb[s]
    if fp8:
        kp = random_e4m3((N, HKV, B, D), DEV, 781, 4, 10)
        vp = random_e4m3((N, HKV, B, D), DEV, 782, 4, 10)
    else:
        kp = normal_16bit((N, HKV, B, D), "f16", DEV, 781)
        vp = normal_16bit((N, HKV, B, D), "f16", DEV, 782)
    tab = torch.from_numpy(tables).to(DEV)
    lens = torch.from_numpy(np.asarray(LENS, np.int32)).to(DEV)
    return kp, vp, tab, lens


def _calls(fp8, ws):
    """(name, thunk) for every call over these pools that takes a workspace."""
    kp, vp, tab, lens = _batch(fp8)
    S, maxb, sc = len(LENS), tab.shape[1], D ** -0.5
    q = normal_16bit((S, HKV * 4, D), "f16", DEV, 783)
    q1 = normal_16bit((S, HKV, D), "f16", DEV, 784)
    qm = normal_16bit((S, 3, HKV, D), "f16", DEV, 785)
    k_new = normal_16bit((S, HKV, D), "f16", DEV, 786)
    v_new = normal_16bit((S, HKV, D), "f16", DEV, 787)
    out = torch.empty_like(q1)
    if fp8:
        return [
            ("decode_fp8", lambda: pkv.paged_attention_decode_fp8(q, kp, vp, tab, lens, sc, 0.5, 0.5, workspace=ws)),
            ("multi_fp8", lambda: pkv.paged_attention_multi_fp8(qm, kp, vp, tab, lens, sc, 0.5, 0.5, workspace=ws)),
            ("decode_append_fp8", lambda: pkv.paged_attention_decode_append_fp8(
                q1, k_new, v_new, kp, vp, tab, lens, sc, 0.5, 0.5, workspace=ws)),
            ("partitions_fp8", lambda: pkv.decode_partitions_fp8(q1, kp, vp, tab, lens, sc, 0.5, 0.5, out, ws)),
            ("merge_fp8", lambda: pkv.decode_merge_fp8(out, lens, maxb, kp, ws)),
        ]
    pl = torch.tensor([4, 8], dtype=torch.int32, device=DEV)
    return [
        ("decode", lambda: pkv.paged_attention_decode(q, kp, vp, tab, lens, sc, workspace=ws)),
        ("decode_append", lambda: pkv.paged_attention_decode_append(q1, k_new, v_new, kp, vp, tab, lens, sc,
                                                                    workspace=ws)),
        ("partitions", lambda: pkv.decode_partitions(q1, kp, vp, tab, lens, sc, out, ws)),
        ("partitions_append", lambda: pkv.decode_partitions_append(q1, k_new, v_new, kp, vp, tab, lens, sc, out, ws)),
        ("merge", lambda: pkv.decode_merge(out, lens, maxb, kp, ws)),
        ("multi", lambda: pkv.paged_attention_multi(qm, kp, vp, tab, lens, sc, workspace=ws)),
        ("shared", lambda: pkv.paged_attention_decode_shared(q1, kp, vp, tab, lens, sc, 2, pl, workspace=ws)),
    ]


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("where", ["host", "strided"])
def test_unusable_workspace_is_refused(fp8, where):
    big = 1 << 22
    if where == "host":
        ws = torch.zeros(big, dtype=torch.uint8)
    else:
        ws = torch.zeros(2 * big, dtype=torch.uint8, device=DEV)[::2]
    for name, call in _calls(fp8, ws):
        with pytest.raises(ValueError, match="workspace"):
            call()
    torch.cuda.synchronize()
