"""GPU: the library's calls captured in a HIP graph (torch.cuda.CUDAGraph) and
replayed, as a serving loop runs its decode step.  The library launches only
kernels on the caller's stream (no memsets, no allocations, no host
synchronisation), so a captured call must replay exactly: every replay,
with eager work and a device synchronisation between replays and the outputs
poisoned before each, gives the eager call's outputs bit for bit, and calls
that append leave the pools as the eager call left them."""

import numpy as np
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402
from synth import build_tables, make_fp8_pools, make_pools, make_query, normal_16bit  # noqa: E402

from .gpu_util import DEV, device_tables, log  # noqa: E402

REPLAYS = 3


def _bits(x):
    return x.view(torch.uint8) if x.element_size() == 1 else x.view(torch.int16)


def _check_replays(fn, outs, pools=()):
    """fn() issues the calls under test, writing into the preallocated
    `outs`.  Eager reference first; then one capture and REPLAYS replays."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    pref = [p.clone() for p in pools]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):  # a warm-up on a side stream before the capture
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    other = torch.randn(1 << 20, device=DEV)
    for i in range(REPLAYS):
        for o in outs:
            o.fill_(float("nan"))
        other.mul_(1.0001)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(_bits(o), _bits(r)), f"replay {i}: output differs from the eager call"
        for p, r in zip(pools, pref):
            assert torch.equal(_bits(p), _bits(r)), f"replay {i}: pool differs from the eager call"
    del g


@pytest.fixture(scope="module")
def opt13b():
    t = build_tables("opt13b")
    tab, lens = device_tables(t)
    kp, vp = make_pools(t, DEV)
    q = make_query(t, DEV)
    S, H, D = t.num_seqs, t.num_heads, t.head_dim
    kn = normal_16bit((S, H, D), t.dtype, DEV, 9101)
    vn = normal_16bit((S, H, D), t.dtype, DEV, 9102)
    return dict(t=t, tab=tab, lens=lens, kp=kp, vp=vp, q=q, kn=kn, vn=vn)


def test_graph_decode_one_call_and_split_merge(opt13b):
    c = opt13b
    t = c["t"]
    log("graph: decode, one call and split + merge (opt13b)")
    out = torch.empty_like(c["q"])
    ws = pkv.alloc_workspace(t.num_seqs, t.num_heads, t.max_blocks, c["kp"], 0)
    _check_replays(lambda: pkv.paged_attention_decode(c["q"], c["kp"], c["vp"], c["tab"], c["lens"], t.scale,
                                                      out=out, workspace=ws), [out])
    out2 = torch.empty_like(c["q"])

    def split_merge():
        pkv.decode_partitions(c["q"], c["kp"], c["vp"], c["tab"], c["lens"], t.scale, out2, ws)
        pkv.decode_merge(out2, c["lens"], t.max_blocks, c["kp"], ws)

    _check_replays(split_merge, [out2])
    assert torch.equal(_bits(out), _bits(out2))


def test_graph_decode_step_with_append(opt13b):
    """The benchmark's step (split pass with the append fused, then the
    merge) and the one-call step, on clones of the pools."""
    c = opt13b
    t = c["t"]
    log("graph: decode step with the append (opt13b)")
    kp, vp = c["kp"].clone(), c["vp"].clone()
    out = torch.empty_like(c["q"])
    ws = pkv.alloc_workspace(t.num_seqs, t.num_heads, t.max_blocks, kp, 0)

    def step():
        pkv.decode_partitions_append(c["q"], c["kn"], c["vn"], kp, vp, c["tab"], c["lens"], t.scale, out, ws)
        pkv.decode_merge(out, c["lens"], t.max_blocks, kp, ws)

    _check_replays(step, [out], pools=[kp, vp])
    kp2, vp2 = c["kp"].clone(), c["vp"].clone()
    out2 = torch.empty_like(c["q"])
    _check_replays(lambda: pkv.paged_attention_decode_append(c["q"], c["kn"], c["vn"], kp2, vp2, c["tab"], c["lens"],
                                                             t.scale, out=out2, workspace=ws),
                   [out2], pools=[kp2, vp2])
    assert torch.equal(_bits(out), _bits(out2))
    assert torch.equal(_bits(kp), _bits(kp2)) and torch.equal(_bits(vp), _bits(vp2))


def test_graph_noalloc(opt13b):
    c = opt13b
    t = c["t"]
    log("graph: the no-allocation decode (opt13b)")
    out = torch.empty_like(c["q"])
    _check_replays(lambda: pkv.paged_attention_decode_noalloc(c["q"], c["kp"], c["vp"], c["tab"], c["lens"], t.scale,
                                                              out), [out])


def test_graph_grouped_and_multi_token(opt13b):
    """Four query heads per KV head, and four query tokens per sequence, on
    the matrix-core kernel."""
    c = opt13b
    t = c["t"]
    S, H, D = t.num_seqs, t.num_heads, t.head_dim
    log("graph: grouped heads and multi-token queries (opt13b pools)")
    qg = normal_16bit((S, 4 * H, D), t.dtype, DEV, 9103)
    og = torch.empty_like(qg)
    wsg = pkv.alloc_workspace(S, 4 * H, t.max_blocks, c["kp"], 0)
    _check_replays(lambda: pkv.paged_attention_decode(qg, c["kp"], c["vp"], c["tab"], c["lens"], t.scale, out=og,
                                                      workspace=wsg), [og])
    qm = normal_16bit((S, 4, H, D), t.dtype, DEV, 9104)
    om = torch.empty_like(qm)
    need = pkv.multi_workspace_bytes(S, 4, H, t.max_blocks, c["kp"])
    wsm = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    _check_replays(lambda: pkv.paged_attention_multi(qm, c["kp"], c["vp"], c["tab"], c["lens"], t.scale, out=om,
                                                     workspace=wsm), [om])


def test_graph_fp8_decode_step(opt13b):
    c = opt13b
    t = c["t"]
    log("graph: e4m3 decode step with the quantising append (opt13b)")
    kp, vp = make_fp8_pools(t, DEV)
    out = torch.empty_like(c["q"])
    need = pkv.fp8_decode_workspace_bytes(t.num_seqs, t.num_heads, t.max_blocks, kp, t.dtype)
    ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)
    _check_replays(lambda: pkv.paged_attention_decode_append_fp8(c["q"], c["kn"], c["vn"], kp, vp, c["tab"], c["lens"],
                                                                 t.scale, 1.0 / 60, 1.0 / 60, out=out, workspace=ws),
                   [out], pools=[kp, vp])


def test_graph_shared_prefix():
    log("graph: shared-prefix decode (32 prompts x 6 siblings)")
    t = build_tables("shared")
    k = t.extra["siblings"]
    P = t.extra["prefix_blocks"] * t.block_size
    tab, lens = device_tables(t)
    kp, vp = make_pools(t, DEV)
    q = make_query(t, DEV)
    pl = torch.from_numpy(np.full(t.num_seqs // k, P, np.int32)).to(DEV)
    out = torch.empty_like(q)
    need = pkv.shared_prefix_workspace_bytes(t.num_seqs, t.num_heads, t.max_blocks, kp, k)
    ws = torch.empty(max(need, 256), dtype=torch.uint8, device=DEV)
    _check_replays(lambda: pkv.paged_attention_decode_shared(q, kp, vp, tab, lens, t.scale, k, pl, out=out,
                                                             workspace=ws), [out])


def test_graph_fp8_split_and_merge_calls(opt13b):
    """The e4m3 decode's two passes as separate calls, one query row and four
    query heads per KV head."""
    c = opt13b
    t = c["t"]
    S, H, D = t.num_seqs, t.num_heads, t.head_dim
    log("graph: e4m3 split + merge as two calls (opt13b pools)")
    kp, vp = make_fp8_pools(t, DEV)
    for G in (1, 4):
        q = c["q"] if G == 1 else normal_16bit((S, G * H, D), t.dtype, DEV, 9105)
        out = torch.empty_like(q)
        need = pkv.fp8_decode_workspace_bytes(S, G * H, t.max_blocks, kp, t.dtype)
        ws = torch.zeros(max(need, 256), dtype=torch.uint8, device=DEV)

        def two_calls():
            pkv.decode_partitions_fp8(q, kp, vp, c["tab"], c["lens"], t.scale, 1.0 / 60, 1.0 / 60, out, ws)
            pkv.decode_merge_fp8(out, c["lens"], t.max_blocks, kp, ws)

        _check_replays(two_calls, [out])
        one = pkv.paged_attention_decode_fp8(q, kp, vp, c["tab"], c["lens"], t.scale, 1.0 / 60, 1.0 / 60)
        torch.cuda.synchronize()
        assert torch.equal(_bits(out), _bits(one)), f"G={G}: two calls differ from the one call"
