"""ctypes binding over libpagedkv (include/pagedkv.h).

Argument marshalling only: every computation runs in the library's HIP
kernels.  torch supplies device memory and the current stream.  There is no
fallback: if the library is missing or a call fails, an exception is raised.
"""

from __future__ import annotations

import ctypes
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libpagedkv.so")

PKV_OK = 0
STATUS_NAMES = {0: "PKV_OK", 1: "PKV_ERR_NULL", 2: "PKV_ERR_SHAPE", 3: "PKV_ERR_UNSUPPORTED",
                4: "PKV_ERR_WORKSPACE", 5: "PKV_ERR_HIP", 6: "PKV_ERR_SCRATCH"}
DTYPE_CODES = {"f16": 0, "bf16": 1}

# every symbol include/pagedkv.h declares
EXPORTS = (
    "pkv_version",
    "pkv_status_string",
    "pkv_pool_bytes",
    "pkv_pool_index",
    "pkv_slot_mapping",
    "pkv_reshape_and_cache",
    "pkv_copy_blocks",
    "pkv_decode_partition_size",
    "pkv_decode_workspace_bytes",
    "pkv_decode_launch_info",
    "pkv_paged_attention_decode",
    "pkv_paged_attention_decode_noalloc",
    "pkv_shared_prefix_workspace_bytes",
    "pkv_paged_attention_decode_shared",
    "pkv_paged_attention_decode_append",
    "pkv_decode_partitions_append",
    "pkv_decode_partitions",
    "pkv_decode_merge",
    "pkv_multi_workspace_bytes",
    "pkv_paged_attention_multi",
    "pkv_fp8_pool_bytes",
    "pkv_reshape_and_cache_fp8",
    "pkv_fp8_decode_workspace_bytes",
    "pkv_paged_attention_decode_fp8",
    "pkv_paged_attention_decode_append_fp8",
    "pkv_fp8_multi_workspace_bytes",
    "pkv_paged_attention_multi_fp8",
    "pkv_decode_partitions_fp8",
    "pkv_decode_merge_fp8",
)


class PagedKVError(RuntimeError):
    """A non-OK status returned by libpagedkv."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {STATUS_NAMES.get(status, status)} ({_status_text(status)})")


class PoolDesc(ctypes.Structure):
    _fields_ = [("num_blocks", ctypes.c_int64), ("block_size", ctypes.c_int32),
                ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("flags", ctypes.c_int32)]


class LaunchInfo(ctypes.Structure):
    """pkv_launch_info: the split pass's grid, occupancy and resources."""
    _fields_ = [(n, ctypes.c_int32) for n in (
        "workgroups", "waves_per_workgroup", "waves_per_simd", "compute_units", "registers",
        "lds_static_bytes", "lds_dynamic_bytes", "scratch_bytes", "balanced", "partition_size")]


POOL_REUSE = 1  # pkv_pool.flags: blocks read by several sequences in one call


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libpagedkv.so (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"libpagedkv.so not found at {path}; build it with "
                           "`python -m paged_kv_cache_119_amd.build`")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    vp = ctypes.c_void_p
    i32, i64, sz = ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    pool = P(PoolDesc)
    sig = {
        "pkv_version": (ctypes.c_int, []),
        "pkv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
        "pkv_pool_bytes": (sz, [pool]),
        "pkv_pool_index": (i64, [pool, i64, i32, i32, i32]),
        "pkv_slot_mapping": (ctypes.c_int, [vp, vp, i32, i32, vp, vp, i32, pool, vp]),
        "pkv_reshape_and_cache": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, vp, i32, pool, vp]),
        "pkv_copy_blocks": (ctypes.c_int, [vp, vp, vp, i32, pool, vp]),
        "pkv_decode_partition_size": (i32, [i32, i32, i32, pool, i32]),
        "pkv_decode_launch_info": (ctypes.c_int, [i32, i32, i32, pool, i32, i32, i32, i32, P(LaunchInfo)]),
        "pkv_decode_workspace_bytes": (sz, [i32, i32, i32, pool, i32]),
        "pkv_paged_attention_decode": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32,
                                                      i32, pool, i32, vp, sz, vp]),
        "pkv_paged_attention_decode_noalloc": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32,
                                                              i32, pool, vp]),
        "pkv_shared_prefix_workspace_bytes": (sz, [i32, i32, i32, pool, i32]),
        "pkv_paged_attention_decode_shared": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32,
                                                             pool, i32, vp, vp, sz, vp]),
        "pkv_paged_attention_decode_append": (ctypes.c_int, [vp, vp, vp, vp, i64, vp, vp, vp, vp, ctypes.c_float,
                                                             i32, i32, i32, pool, i32, vp, sz, vp]),
        "pkv_decode_partitions_append": (ctypes.c_int, [vp, vp, vp, vp, i64, vp, vp, vp, vp, ctypes.c_float,
                                                        i32, i32, i32, pool, i32, vp, sz, vp]),
        "pkv_decode_partitions": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32,
                                                 pool, i32, vp, sz, vp]),
        "pkv_decode_merge": (ctypes.c_int, [vp, vp, i32, i32, i32, pool, i32, vp, sz, vp]),
        "pkv_multi_workspace_bytes": (sz, [i32, i32, i32, i32, pool]),
        "pkv_paged_attention_multi": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, i32, i32, i32, i32,
                                                     pool, vp, sz, vp]),
        "pkv_fp8_pool_bytes": (sz, [pool]),
        "pkv_reshape_and_cache_fp8": (ctypes.c_int, [vp, vp, vp, vp, i64, i64, vp, i32, ctypes.c_float,
                                                     ctypes.c_float, pool, vp]),
        "pkv_fp8_decode_workspace_bytes": (sz, [i32, i32, i32, pool]),
        "pkv_paged_attention_decode_fp8": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                                          ctypes.c_float, i32, i32, i32, pool, vp, sz, vp]),
        "pkv_fp8_multi_workspace_bytes": (sz, [i32, i32, i32, i32, pool]),
        "pkv_paged_attention_multi_fp8": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                                         ctypes.c_float, i32, i32, i32, i32, pool, vp, sz, vp]),
        "pkv_paged_attention_decode_append_fp8": (ctypes.c_int, [vp, vp, vp, vp, i64, vp, vp, vp, vp, ctypes.c_float,
                                                                 ctypes.c_float, ctypes.c_float, i32, i32, i32, pool,
                                                                 vp, sz, vp]),
        "pkv_decode_partitions_fp8": (ctypes.c_int, [vp, vp, vp, vp, vp, vp, ctypes.c_float, ctypes.c_float,
                                                     ctypes.c_float, i32, i32, i32, i32, pool, vp, sz, vp]),
        "pkv_decode_merge_fp8": (ctypes.c_int, [vp, vp, i32, i32, i32, i32, pool, vp, sz, vp]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _status_text(status: int) -> str:
    try:
        return load_library().pkv_status_string(status).decode()
    except Exception:  # pragma: no cover - only when the library is absent
        return "?"


def _check(status: int, what: str) -> None:
    if status != PKV_OK:
        raise PagedKVError(status, what)


def make_pool_desc(num_blocks: int, block_size: int, num_kv_heads: int, head_dim: int, dtype: str,
                   reuse_blocks: bool = False) -> PoolDesc:
    return PoolDesc(int(num_blocks), int(block_size), int(num_kv_heads), int(head_dim), DTYPE_CODES[dtype],
                    POOL_REUSE if reuse_blocks else 0)


# ---------------------------------------------------------------------------
# torch plumbing
# ---------------------------------------------------------------------------

def _torch():
    import torch
    return torch


def _dtype_name(t) -> str:
    torch = _torch()
    if t.dtype == torch.float16:
        return "f16"
    if t.dtype == torch.bfloat16:
        return "bf16"
    raise TypeError(f"expected float16 or bfloat16, got {t.dtype}")


def _need(t, name, dtype=None, ndim=None, device=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions, got shape {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _stream_ptr(device) -> int:
    torch = _torch()
    return int(torch.cuda.current_stream(device).cuda_stream)


def pool_desc_of(k_pool, reuse_blocks: bool = False) -> PoolDesc:
    N, H, B, D = (int(x) for x in k_pool.shape)
    return make_pool_desc(N, B, H, D, _dtype_name(k_pool), reuse_blocks)


def _check_pools(k_pool, v_pool, reuse_blocks=False):
    _need(k_pool, "k_pool", ndim=4)
    _need(v_pool, "v_pool", dtype=k_pool.dtype, ndim=4, device=k_pool.device)
    if k_pool.shape != v_pool.shape:
        raise ValueError(f"k_pool {tuple(k_pool.shape)} and v_pool {tuple(v_pool.shape)} differ")
    return pool_desc_of(k_pool, reuse_blocks)


# ---------------------------------------------------------------------------
# public calls (same names as the C entry points, without the prefix)
# ---------------------------------------------------------------------------

def version() -> int:
    return int(load_library().pkv_version())


def status_string(status: int) -> str:
    return load_library().pkv_status_string(int(status)).decode()


def pool_bytes(num_blocks, block_size, num_kv_heads, head_dim, dtype="f16") -> int:
    d = make_pool_desc(num_blocks, block_size, num_kv_heads, head_dim, dtype)
    return int(load_library().pkv_pool_bytes(ctypes.byref(d)))


def pool_index(desc: PoolDesc, block, head, offset, dim) -> int:
    return int(load_library().pkv_pool_index(ctypes.byref(desc), int(block), int(head), int(offset), int(dim)))


def slot_mapping(block_tables, token_seq, token_pos, k_pool, out=None):
    """Pool slot of each (sequence, position) token; -1 for padding."""
    torch = _torch()
    lib = load_library()
    desc = pool_desc_of(k_pool)
    dev = k_pool.device
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=dev)
    _need(token_seq, "token_seq", dtype=torch.int32, ndim=1, device=dev)
    _need(token_pos, "token_pos", dtype=torch.int32, ndim=1, device=dev)
    T = int(token_seq.shape[0])
    if token_pos.shape[0] != T:
        raise ValueError("token_seq and token_pos lengths differ")
    if out is None:
        out = torch.empty(T, dtype=torch.int64, device=dev)
    _need(out, "out", dtype=torch.int64, ndim=1, device=dev)
    S, maxb = (int(x) for x in block_tables.shape)
    st = lib.pkv_slot_mapping(out.data_ptr(), block_tables.data_ptr(), S, maxb, token_seq.data_ptr(),
                              token_pos.data_ptr(), T, ctypes.byref(desc), _stream_ptr(dev))
    _check(st, "pkv_slot_mapping")
    return out


def reshape_and_cache(k, v, k_pool, v_pool, slot_mapping):
    """Write new tokens' K/V rows ``[T, Hkv, D]`` into their pool slots."""
    torch = _torch()
    lib = load_library()
    desc = _check_pools(k_pool, v_pool)
    dev = k_pool.device
    for name, t in (("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
            raise ValueError(f"{name} must be a tensor on {dev}")
        if t.dtype != k_pool.dtype:
            raise TypeError(f"{name} must be {k_pool.dtype}")
        if t.dim() != 3 or tuple(t.shape[1:]) != (desc.num_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [T, {desc.num_kv_heads}, {desc.head_dim}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != desc.head_dim:
            raise ValueError(f"{name} must have heads and dims contiguous")
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1, device=dev)
    T = int(k.shape[0])
    if v.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("k, v and slot_mapping must have the same number of tokens")
    st = lib.pkv_reshape_and_cache(k_pool.data_ptr(), v_pool.data_ptr(), k.data_ptr(), v.data_ptr(),
                                   int(k.stride(0)) if T > 0 else 0, int(v.stride(0)) if T > 0 else 0,
                                   slot_mapping.data_ptr(), T, ctypes.byref(desc), _stream_ptr(dev))
    _check(st, "pkv_reshape_and_cache")


def copy_blocks(k_pool, v_pool, block_pairs):
    """Copy whole pool blocks: ``block_pairs`` is int64 ``[n, 2]`` of (src, dst)."""
    torch = _torch()
    lib = load_library()
    desc = _check_pools(k_pool, v_pool)
    dev = k_pool.device
    _need(block_pairs, "block_pairs", dtype=torch.int64, ndim=2, device=dev)
    if block_pairs.shape[1] != 2 or not block_pairs.is_contiguous():
        raise ValueError("block_pairs must be a contiguous [n, 2] tensor")
    n = int(block_pairs.shape[0])
    st = lib.pkv_copy_blocks(k_pool.data_ptr(), v_pool.data_ptr(), block_pairs.data_ptr(), n, ctypes.byref(desc),
                             _stream_ptr(dev))
    _check(st, "pkv_copy_blocks")


def decode_partition_size(num_seqs, num_heads, max_blocks_per_seq, k_pool, partition_size=0) -> int:
    desc = pool_desc_of(k_pool)
    return int(load_library().pkv_decode_partition_size(int(num_seqs), int(num_heads), int(max_blocks_per_seq),
                                                        ctypes.byref(desc), int(partition_size)))


def decode_launch_info(num_seqs, num_heads, max_blocks_per_seq, desc, partition_size=0, num_queries=1,
                       fp8=False, append=False) -> dict:
    """The split pass a decode call with these arguments launches on the
    current device: grid, resident waves per SIMD, registers, LDS and scratch
    from the library's own code objects (pkv_decode_launch_info).  `desc` is
    the pool's PoolDesc (make_pool_desc / pool_desc_of)."""
    info = LaunchInfo()
    st = load_library().pkv_decode_launch_info(int(num_seqs), int(num_heads), int(max_blocks_per_seq),
                                               ctypes.byref(desc), int(partition_size), int(num_queries),
                                               1 if fp8 else 0, 1 if append else 0, ctypes.byref(info))
    _check(st, "pkv_decode_launch_info")
    return {name: int(getattr(info, name)) for name, _ in LaunchInfo._fields_}


def decode_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq, k_pool, partition_size=0) -> int:
    desc = pool_desc_of(k_pool)
    return int(load_library().pkv_decode_workspace_bytes(int(num_seqs), int(num_heads), int(max_blocks_per_seq),
                                                         ctypes.byref(desc), int(partition_size)))


def alloc_workspace(num_seqs, num_heads, max_blocks_per_seq, k_pool, partition_size=0):
    """A caller-owned workspace tensor of the size the decode call needs
    (zero-filled, which the kernels do not require)."""
    torch = _torch()
    n = decode_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq, k_pool, partition_size)
    return torch.zeros(max(n, 256), dtype=torch.uint8, device=k_pool.device)


def _decode_args(q, k_pool, v_pool, block_tables, context_lens, out, reuse_blocks=False):
    torch = _torch()
    desc = _check_pools(k_pool, v_pool, reuse_blocks)
    dev = k_pool.device
    _need(q, "q", dtype=k_pool.dtype, ndim=3, device=dev)
    S, H, D = (int(x) for x in q.shape)
    if D != desc.head_dim:
        raise ValueError(f"q head_dim {D} != pool head_dim {desc.head_dim}")
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("q, block_tables and context_lens disagree on the number of sequences")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, ndim=3, device=dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    return desc, S, H, int(block_tables.shape[1]), out


def _ws_arg(ws, device):
    """A caller's workspace: a contiguous GPU tensor on the pools' device (any
    dtype; the library checks its size and alignment).  Its pointer and size in
    bytes."""
    _need(ws, "workspace", device=device)
    return ws.data_ptr(), ws.numel() * ws.element_size()


def _workspace(ws, S, H, maxb, k_pool, partition_size):
    need = decode_workspace_bytes(S, H, maxb, k_pool, partition_size)
    if ws is None:
        if need == 0:
            return 0, 0
        ws = alloc_workspace(S, H, maxb, k_pool, partition_size)
    return _ws_arg(ws, k_pool.device)


def paged_attention_decode(q, k_pool, v_pool, block_tables, context_lens, scale, out=None,
                           partition_size=0, workspace=None, reuse_blocks=False):
    """Single-query decode attention over paged K/V; returns ``out`` [S, H, D].
    ``reuse_blocks``: the batch reads some blocks more than once (shared
    prefixes); K/V reads then stay cacheable (speed only)."""
    lib = load_library()
    desc, S, H, maxb, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out, reuse_blocks)
    ws_ptr, ws_bytes = _workspace(workspace, S, H, maxb, k_pool, partition_size)
    st = lib.pkv_paged_attention_decode(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                        block_tables.data_ptr(), context_lens.data_ptr(), float(scale), S, H,
                                        maxb, ctypes.byref(desc), int(partition_size), ws_ptr, ws_bytes,
                                        _stream_ptr(k_pool.device))
    _check(st, "pkv_paged_attention_decode")
    return out


def paged_attention_decode_noalloc(q, k_pool, v_pool, block_tables, context_lens, scale, out,
                                   reuse_blocks=False):
    """pkv_paged_attention_decode_noalloc: the decode of paged_attention_decode
    (balanced split) with its partial results in the library's static device
    scratch; nothing is allocated, so ``out`` must be passed.  Calls that may
    overlap on one GPU race on that scratch."""
    lib = load_library()
    if out is None:
        raise ValueError("out must be given: this call allocates nothing")
    desc, S, H, maxb, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out, reuse_blocks)
    st = lib.pkv_paged_attention_decode_noalloc(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                                block_tables.data_ptr(), context_lens.data_ptr(), float(scale), S, H,
                                                maxb, ctypes.byref(desc), _stream_ptr(k_pool.device))
    _check(st, "pkv_paged_attention_decode_noalloc")
    return out


def shared_prefix_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq, k_pool, group_size) -> int:
    desc = pool_desc_of(k_pool)
    return int(load_library().pkv_shared_prefix_workspace_bytes(int(num_seqs), int(num_heads),
                                                                int(max_blocks_per_seq), ctypes.byref(desc),
                                                                int(group_size)))


def paged_attention_decode_shared(q, k_pool, v_pool, block_tables, context_lens, scale, group_size, prefix_lens,
                                  out=None, workspace=None, reuse_blocks=False):
    """Decode over groups of ``group_size`` consecutive sequences whose first
    ``prefix_lens[g]`` tokens (int32 [S / group_size], device) hold the same
    K/V: each group's prefix is read once for all its sequences
    (pkv_paged_attention_decode_shared)."""
    torch = _torch()
    lib = load_library()
    desc, S, H, maxb, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out, reuse_blocks)
    _need(prefix_lens, "prefix_lens", dtype=torch.int32, ndim=1, device=k_pool.device)
    if group_size < 1 or S % group_size != 0 or prefix_lens.shape[0] != S // group_size:
        raise ValueError("prefix_lens must hold one length per group of group_size sequences")
    need = shared_prefix_workspace_bytes(S, H, maxb, k_pool, group_size)
    if workspace is None:
        workspace = torch.empty(max(need, 256), dtype=torch.uint8, device=k_pool.device)
    st = lib.pkv_paged_attention_decode_shared(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                               block_tables.data_ptr(), context_lens.data_ptr(), float(scale), S, H,
                                               maxb, ctypes.byref(desc), int(group_size), prefix_lens.data_ptr(),
                                               *_ws_arg(workspace, k_pool.device),
                                               _stream_ptr(k_pool.device))
    _check(st, "pkv_paged_attention_decode_shared")
    return out


def multi_workspace_bytes(num_seqs, num_queries, num_heads, max_blocks_per_seq, k_pool) -> int:
    desc = pool_desc_of(k_pool)
    return int(load_library().pkv_multi_workspace_bytes(int(num_seqs), int(num_queries), int(num_heads),
                                                        int(max_blocks_per_seq), ctypes.byref(desc)))


def paged_attention_multi(q, k_pool, v_pool, block_tables, context_lens, scale, out=None, workspace=None,
                          reuse_blocks=False):
    """Several query tokens per sequence over paged K/V: ``q`` is [S, Q, H, D];
    query i of sequence s sits at position context_lens[s] - Q + i and attends
    causally.  Returns ``out`` [S, Q, H, D]."""
    torch = _torch()
    lib = load_library()
    desc = _check_pools(k_pool, v_pool, reuse_blocks)
    dev = k_pool.device
    _need(q, "q", dtype=k_pool.dtype, ndim=4, device=dev)
    S, Q, H, D = (int(x) for x in q.shape)
    if D != desc.head_dim:
        raise ValueError(f"q head_dim {D} != pool head_dim {desc.head_dim}")
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("q, block_tables and context_lens disagree on the number of sequences")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, ndim=4, device=dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    maxb = int(block_tables.shape[1])
    need = multi_workspace_bytes(S, Q, H, maxb, k_pool)
    if workspace is None:
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.pkv_paged_attention_multi(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                       block_tables.data_ptr(), context_lens.data_ptr(), float(scale), S, Q, H, maxb,
                                       ctypes.byref(desc), *_ws_arg(workspace, k_pool.device), _stream_ptr(dev))
    _check(st, "pkv_paged_attention_multi")
    return out


# ---------------------------------------------------------------------------
# FP8 (e4m3) pools: one byte per element, one float32 scale per pool
# ---------------------------------------------------------------------------

def _fp8_pools(k_pool, v_pool, dtype_name, reuse_blocks=False):
    torch = _torch()
    _need(k_pool, "k_pool", ndim=4)
    _need(v_pool, "v_pool", ndim=4, device=k_pool.device)
    for name, t in (("k_pool", k_pool), ("v_pool", v_pool)):
        if t.dtype not in (torch.uint8, torch.float8_e4m3fn):
            raise TypeError(f"{name} must hold e4m3 codes (uint8 or float8_e4m3fn), got {t.dtype}")
    if k_pool.shape != v_pool.shape:
        raise ValueError(f"k_pool {tuple(k_pool.shape)} and v_pool {tuple(v_pool.shape)} differ")
    N, H, B, D = (int(x) for x in k_pool.shape)
    return make_pool_desc(N, B, H, D, dtype_name, reuse_blocks)


def fp8_pool_bytes(num_blocks, block_size, num_kv_heads, head_dim) -> int:
    d = make_pool_desc(num_blocks, block_size, num_kv_heads, head_dim, "f16")
    return int(load_library().pkv_fp8_pool_bytes(ctypes.byref(d)))


def reshape_and_cache_fp8(k, v, k_pool, v_pool, slot_mapping, k_scale, v_scale):
    """Quantise new tokens' K/V rows ``[T, Hkv, D]`` (16-bit) to e4m3 codes
    under the pools' scales and write them into their slots."""
    torch = _torch()
    lib = load_library()
    desc = _fp8_pools(k_pool, v_pool, _dtype_name(k))
    dev = k_pool.device
    for name, t in (("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor) or not t.is_cuda or t.device != dev:
            raise ValueError(f"{name} must be a tensor on {dev}")
        if t.dtype != k.dtype:
            raise TypeError("k and v must have the same dtype")
        if t.dim() != 3 or tuple(t.shape[1:]) != (desc.num_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [T, {desc.num_kv_heads}, {desc.head_dim}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != desc.head_dim:
            raise ValueError(f"{name} must have heads and dims contiguous")
    _need(slot_mapping, "slot_mapping", dtype=torch.int64, ndim=1, device=dev)
    T = int(k.shape[0])
    if v.shape[0] != T or slot_mapping.shape[0] != T:
        raise ValueError("k, v and slot_mapping must have the same number of tokens")
    st = lib.pkv_reshape_and_cache_fp8(k_pool.data_ptr(), v_pool.data_ptr(), k.data_ptr(), v.data_ptr(),
                                       int(k.stride(0)) if T > 0 else 0, int(v.stride(0)) if T > 0 else 0,
                                       slot_mapping.data_ptr(), T, float(k_scale), float(v_scale),
                                       ctypes.byref(desc), _stream_ptr(dev))
    _check(st, "pkv_reshape_and_cache_fp8")


def fp8_decode_workspace_bytes(num_seqs, num_heads, max_blocks_per_seq, k_pool, dtype="f16") -> int:
    N, H, B, D = (int(x) for x in k_pool.shape)
    desc = make_pool_desc(N, B, H, D, dtype)
    return int(load_library().pkv_fp8_decode_workspace_bytes(int(num_seqs), int(num_heads),
                                                             int(max_blocks_per_seq), ctypes.byref(desc)))


def paged_attention_decode_fp8(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out=None,
                               workspace=None, reuse_blocks=False):
    """Single-query decode attention over e4m3 pools (K element = code value *
    k_scale, V element = code value * v_scale); ``q`` and ``out`` [S, H, D]
    16-bit."""
    torch = _torch()
    lib = load_library()
    desc = _fp8_pools(k_pool, v_pool, _dtype_name(q), reuse_blocks)
    dev = k_pool.device
    _need(q, "q", ndim=3, device=dev)
    S, H, D = (int(x) for x in q.shape)
    if D != desc.head_dim:
        raise ValueError(f"q head_dim {D} != pool head_dim {desc.head_dim}")
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("q, block_tables and context_lens disagree on the number of sequences")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, ndim=3, device=dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    maxb = int(block_tables.shape[1])
    if workspace is None:
        need = fp8_decode_workspace_bytes(S, H, maxb, k_pool, _dtype_name(q))
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.pkv_paged_attention_decode_fp8(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                            block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
                                            float(k_scale), float(v_scale), S, H, maxb, ctypes.byref(desc),
                                            *_ws_arg(workspace, k_pool.device),
                                            _stream_ptr(dev))
    _check(st, "pkv_paged_attention_decode_fp8")
    return out


def fp8_multi_workspace_bytes(num_seqs, num_queries, num_heads, max_blocks_per_seq, k_pool, dtype="f16") -> int:
    N, H, B, D = (int(x) for x in k_pool.shape)
    desc = make_pool_desc(N, B, H, D, dtype)
    return int(load_library().pkv_fp8_multi_workspace_bytes(int(num_seqs), int(num_queries), int(num_heads),
                                                            int(max_blocks_per_seq), ctypes.byref(desc)))


def paged_attention_multi_fp8(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out=None,
                              workspace=None, reuse_blocks=False):
    """Several query tokens per sequence over e4m3 pools (see
    paged_attention_multi): ``q`` [S, Q, H, D] 16-bit, returns ``out`` of the
    same shape."""
    torch = _torch()
    lib = load_library()
    desc = _fp8_pools(k_pool, v_pool, _dtype_name(q), reuse_blocks)
    dev = k_pool.device
    _need(q, "q", ndim=4, device=dev)
    S, Q, H, D = (int(x) for x in q.shape)
    if D != desc.head_dim:
        raise ValueError(f"q head_dim {D} != pool head_dim {desc.head_dim}")
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("q, block_tables and context_lens disagree on the number of sequences")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, ndim=4, device=dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    maxb = int(block_tables.shape[1])
    if workspace is None:
        need = fp8_multi_workspace_bytes(S, Q, H, maxb, k_pool, _dtype_name(q))
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.pkv_paged_attention_multi_fp8(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                           block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
                                           float(k_scale), float(v_scale), S, Q, H, maxb, ctypes.byref(desc),
                                           *_ws_arg(workspace, k_pool.device),
                                           _stream_ptr(dev))
    _check(st, "pkv_paged_attention_multi_fp8")
    return out


def _fp8_rows(q, k_pool, v_pool, reuse_blocks):
    """Pool descriptor and (S, Q, H) of a 16-bit query of [S, H, D] (one
    token) or [S, Q, H, D] rows over e4m3 pools."""
    desc = _fp8_pools(k_pool, v_pool, _dtype_name(q), reuse_blocks)
    _need(q, "q", device=k_pool.device)
    if q.dim() == 3:
        S, H, D = (int(x) for x in q.shape)
        Q = 1
    elif q.dim() == 4:
        S, Q, H, D = (int(x) for x in q.shape)
    else:
        raise ValueError(f"q must be [S, H, D] or [S, Q, H, D], got {tuple(q.shape)}")
    if D != desc.head_dim:
        raise ValueError(f"q head_dim {D} != pool head_dim {desc.head_dim}")
    return desc, S, Q, H


def decode_partitions_fp8(q, k_pool, v_pool, block_tables, context_lens, scale, k_scale, v_scale, out, workspace,
                          reuse_blocks=False):
    """The split pass over e4m3 pools alone (see pkv_decode_partitions_fp8):
    ``q`` and ``out`` [S, H, D] or [S, Q, H, D]; decode_merge_fp8 with the same
    workspace completes the call."""
    torch = _torch()
    lib = load_library()
    desc, S, Q, H = _fp8_rows(q, k_pool, v_pool, reuse_blocks)
    dev = k_pool.device
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("q, block_tables and context_lens disagree on the number of sequences")
    _need(out, "out", dtype=q.dtype, device=dev)
    if out.shape != q.shape:
        raise ValueError("out must have q's shape")
    maxb = int(block_tables.shape[1])
    st = lib.pkv_decode_partitions_fp8(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                       block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
                                       float(k_scale), float(v_scale), S, Q, H, maxb, ctypes.byref(desc),
                                       *_ws_arg(workspace, k_pool.device),
                                       _stream_ptr(dev))
    _check(st, "pkv_decode_partitions_fp8")
    return out


def decode_merge_fp8(out, context_lens, max_blocks_per_seq, k_pool, workspace, reuse_blocks=False):
    """The merge pass over e4m3 pools alone (see pkv_decode_merge_fp8);
    ``out`` as given to decode_partitions_fp8."""
    torch = _torch()
    lib = load_library()
    desc, S, Q, H = _fp8_rows(out, k_pool, k_pool, reuse_blocks)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=k_pool.device)
    st = lib.pkv_decode_merge_fp8(out.data_ptr(), context_lens.data_ptr(), S, Q, H, int(max_blocks_per_seq),
                                  ctypes.byref(desc), *_ws_arg(workspace, k_pool.device), _stream_ptr(k_pool.device))
    _check(st, "pkv_decode_merge_fp8")
    return out


def paged_attention_decode_append_fp8(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale, k_scale,
                                      v_scale, out=None, workspace=None, reuse_blocks=False):
    """One decode step over e4m3 pools with the quantising append fused in:
    row s of k_new / v_new ([S, Hkv, D], 16-bit) becomes token
    context_lens[s] - 1 of sequence s, then attention runs."""
    torch = _torch()
    lib = load_library()
    desc = _fp8_pools(k_pool, v_pool, _dtype_name(q), reuse_blocks)
    dev = k_pool.device
    _need(q, "q", ndim=3, device=dev)
    S, H, D = (int(x) for x in q.shape)
    if D != desc.head_dim:
        raise ValueError(f"q head_dim {D} != pool head_dim {desc.head_dim}")
    _need(block_tables, "block_tables", dtype=torch.int32, ndim=2, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    if block_tables.shape[0] != S or context_lens.shape[0] != S:
        raise ValueError("q, block_tables and context_lens disagree on the number of sequences")
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dtype != q.dtype or t.device != dev:
            raise TypeError(f"{name} must be a {q.dtype} tensor on {dev}")
        if t.dim() != 3 or tuple(t.shape) != (S, desc.num_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [{S}, {desc.num_kv_heads}, {desc.head_dim}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != desc.head_dim:
            raise ValueError(f"{name} must have heads and dims contiguous")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must have the same token stride")
    if out is None:
        out = torch.empty_like(q)
    _need(out, "out", dtype=q.dtype, ndim=3, device=dev)
    maxb = int(block_tables.shape[1])
    if workspace is None:
        need = fp8_decode_workspace_bytes(S, H, maxb, k_pool, _dtype_name(q))
        workspace = torch.zeros(max(need, 256), dtype=torch.uint8, device=dev)
    st = lib.pkv_paged_attention_decode_append_fp8(
        out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(), int(k_new.stride(0)) if S > 0 else 0,
        k_pool.data_ptr(), v_pool.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(), float(scale),
        float(k_scale), float(v_scale), S, H, maxb, ctypes.byref(desc), *_ws_arg(workspace, k_pool.device),
        _stream_ptr(dev))
    _check(st, "pkv_paged_attention_decode_append_fp8")
    return out


def paged_attention_decode_append(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale, out=None,
                                  partition_size=0, workspace=None, reuse_blocks=False):
    """One decode step with the append fused in: row s of k_new / v_new
    ([S, Hkv, D]) becomes token context_lens[s] - 1 of sequence s (written to
    its pool slot), then attention runs over the paged K/V."""
    lib = load_library()
    desc, S, H, maxb, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out, reuse_blocks)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dtype != k_pool.dtype or t.device != k_pool.device:
            raise TypeError(f"{name} must be a {k_pool.dtype} tensor on {k_pool.device}")
        if t.dim() != 3 or tuple(t.shape) != (S, desc.num_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [{S}, {desc.num_kv_heads}, {desc.head_dim}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != desc.head_dim:
            raise ValueError(f"{name} must have heads and dims contiguous")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must have the same token stride")
    ws_ptr, ws_bytes = _workspace(workspace, S, H, maxb, k_pool, partition_size)
    st = lib.pkv_paged_attention_decode_append(out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                               int(k_new.stride(0)) if S > 0 else 0, k_pool.data_ptr(),
                                               v_pool.data_ptr(), block_tables.data_ptr(), context_lens.data_ptr(),
                                               float(scale), S, H, maxb, ctypes.byref(desc), int(partition_size),
                                               ws_ptr, ws_bytes, _stream_ptr(k_pool.device))
    _check(st, "pkv_paged_attention_decode_append")
    return out


def decode_partitions(q, k_pool, v_pool, block_tables, context_lens, scale, out, workspace,
                      partition_size=0, reuse_blocks=False):
    """The partition pass alone (see pkv_decode_partitions)."""
    lib = load_library()
    desc, S, H, maxb, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out, reuse_blocks)
    ws_ptr, ws_bytes = _workspace(workspace, S, H, maxb, k_pool, partition_size)
    st = lib.pkv_decode_partitions(out.data_ptr(), q.data_ptr(), k_pool.data_ptr(), v_pool.data_ptr(),
                                   block_tables.data_ptr(), context_lens.data_ptr(), float(scale), S, H, maxb,
                                   ctypes.byref(desc), int(partition_size), ws_ptr, ws_bytes,
                                   _stream_ptr(k_pool.device))
    _check(st, "pkv_decode_partitions")
    return out


def decode_partitions_append(q, k_new, v_new, k_pool, v_pool, block_tables, context_lens, scale, out, workspace,
                             partition_size=0, reuse_blocks=False):
    """The partition pass with the append fused in, alone (see
    pkv_decode_partitions_append); decode_merge completes the step."""
    lib = load_library()
    desc, S, H, maxb, out = _decode_args(q, k_pool, v_pool, block_tables, context_lens, out, reuse_blocks)
    for name, t in (("k_new", k_new), ("v_new", v_new)):
        if t.dtype != k_pool.dtype or t.device != k_pool.device:
            raise TypeError(f"{name} must be a {k_pool.dtype} tensor on {k_pool.device}")
        if t.dim() != 3 or tuple(t.shape) != (S, desc.num_kv_heads, desc.head_dim):
            raise ValueError(f"{name} must be [{S}, {desc.num_kv_heads}, {desc.head_dim}], got {tuple(t.shape)}")
        if t.stride(2) != 1 or t.stride(1) != desc.head_dim:
            raise ValueError(f"{name} must have heads and dims contiguous")
    if k_new.stride(0) != v_new.stride(0):
        raise ValueError("k_new and v_new must have the same token stride")
    ws_ptr, ws_bytes = _workspace(workspace, S, H, maxb, k_pool, partition_size)
    st = lib.pkv_decode_partitions_append(out.data_ptr(), q.data_ptr(), k_new.data_ptr(), v_new.data_ptr(),
                                          int(k_new.stride(0)) if S > 0 else 0, k_pool.data_ptr(), v_pool.data_ptr(),
                                          block_tables.data_ptr(), context_lens.data_ptr(), float(scale), S, H, maxb,
                                          ctypes.byref(desc), int(partition_size), ws_ptr, ws_bytes,
                                          _stream_ptr(k_pool.device))
    _check(st, "pkv_decode_partitions_append")
    return out


def decode_merge(out, context_lens, max_blocks_per_seq, k_pool, workspace, partition_size=0):
    """The merge pass alone (see pkv_decode_merge)."""
    torch = _torch()
    lib = load_library()
    desc = pool_desc_of(k_pool)
    dev = k_pool.device
    _need(out, "out", dtype=k_pool.dtype, ndim=3, device=dev)
    _need(context_lens, "context_lens", dtype=torch.int32, ndim=1, device=dev)
    S, H = int(out.shape[0]), int(out.shape[1])
    ws_ptr, ws_bytes = _workspace(workspace, S, H, max_blocks_per_seq, k_pool, partition_size)
    st = lib.pkv_decode_merge(out.data_ptr(), context_lens.data_ptr(), S, H, int(max_blocks_per_seq),
                              ctypes.byref(desc), int(partition_size), ws_ptr, ws_bytes, _stream_ptr(dev))
    _check(st, "pkv_decode_merge")
    return out


def workspace_views(workspace, num_seqs, num_heads, max_blocks_per_seq, k_pool, partition_size=0):
    """Float32 views (m [S,H,MP], l [S,H,MP], o [S,H,MP,D]) of a workspace
    tensor, following the layout documented in include/pagedkv.h."""
    P = decode_partition_size(num_seqs, num_heads, max_blocks_per_seq, k_pool, partition_size)
    desc = pool_desc_of(k_pool)
    MP = -(-(max_blocks_per_seq * desc.block_size) // P)
    U = num_seqs * num_heads * MP
    sec = -(-(U * 4) // 256) * 256
    f = workspace.view(__import__("torch").float32)
    m = f[:U].view(num_seqs, num_heads, MP)
    l = f[sec // 4: sec // 4 + U].view(num_seqs, num_heads, MP)
    o = f[2 * sec // 4: 2 * sec // 4 + U * desc.head_dim].view(num_seqs, num_heads, MP, desc.head_dim)
    return m, l, o
