#!/usr/bin/env python3
"""Benchmark: paged decode attention on one MI355X, OPT-13B-shaped layer.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config opt13b]

One step is one pass of the whole hot path over one batch, as a serving
engine runs it for one layer: each of the 64 sequences appends its new
token's K/V (token context_len - 1, written into its pool slot through the
block table) and attends over its paged context -- the split pass with the
append fused in (pkv_decode_partitions_append) followed by the log-sum-exp
merge (pkv_decode_merge).  `--separate-append` runs the append as its own
two launches (pkv_slot_mapping + pkv_reshape_and_cache) before the decode
passes instead.  Inputs are built and resident in HBM before timing; each step
uses one of R replicas of the pools (different addresses), cycled, so no step
finds the previous step's KV in the 256 MiB MALL or the L2s.

Prints ONE JSON line.  `value` is algorithmic bytes per step / time per step
(GB/s); `roofline` prices the partition kernel alone (algorithmic decode bytes
per launch / its mean launch time, from a pair of HIP events around each launch
on its stream, created without the system-scope fence so that recording them
adds no cache writeback between launches); `cpu_baseline` times the float64 CPU
oracle on a bounded sample of the same batch.
"""

from __future__ import annotations

import argparse
import ctypes
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "paged decode attention achieved HBM GB/s (% of MI355X peak) + KV tokens/s"
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic_decode_partition_opt13b.json")


def parse(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="opt13b")
    ap.add_argument("--block-size", type=int, default=None)
    ap.add_argument("--partition-size", type=int, default=0)
    ap.add_argument("--replicas", type=int, default=4)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget-s", type=float, default=12.0,
                    help="seconds of oracle work per host core (the one-thread leg takes half)")
    ap.add_argument("--one-call", action="store_true",
                    help="time the whole decode step as one pkv_paged_attention_decode_append call (split + "
                         "merge, the merge launch writing the new rows) instead of the split pass alone")
    ap.add_argument("--separate-append", action="store_true",
                    help="append with pkv_slot_mapping + pkv_reshape_and_cache, then decode")
    ap.add_argument("--duplicate-shared", action="store_true",
                    help="shared workload: give every sibling private copies of the prefix blocks (control)")
    ap.add_argument("--op", choices=("decode", "copy_blocks", "rows"), default="decode",
                    help="decode (the hot path, default), the batched block copy of copy-on-write, or "
                         "several query rows per KV head (grouped-query heads, multi-token queries)")
    ap.add_argument("--shared-prefix", action="store_true",
                    help="shared workload: decode with pkv_paged_attention_decode_shared (each prompt's prefix read "
                         "once for its siblings) instead of the plain decode")
    ap.add_argument("--reuse-blocks", action="store_true",
                    help="pass the pool's reuse hint (cached K/V loads) for batches that share blocks")
    ap.add_argument("--kv", choices=("16bit", "fp8"), default="16bit",
                    help="--op decode: pool element type (fp8: e4m3 codes with per-pool scales)")
    ap.add_argument("--group", type=int, default=None,
                    help="--op rows: query heads per KV head (default: the workload's query_heads / heads)")
    ap.add_argument("--queries", type=int, default=1, help="--op rows: query tokens per sequence")
    ap.add_argument("--copy-pairs", type=int, default=1024, help="block pairs per copy launch (--op copy_blocks)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a plain 1 GiB device copy (for scaling HBM counters)")
    return ap.parse_args(argv)


def main(argv=None) -> int:
    args = parse(argv)
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: this path has no multi-GPU step (heads and sequences shard with "
              "no exchange); run with --gpus 1", file=sys.stderr)
        return 2
    if args.one_call and (args.separate_append or args.op != "decode" or args.kv != "16bit"):
        print("--one-call times the 16-bit decode step with the append fused", file=sys.stderr)
        return 2

    import numpy as np
    import torch

    import paged_kv_cache_119_amd as pkv
    from paged_kv_cache_119_amd import accounting as acc
    from paged_kv_cache_119_amd.rocprof_summary import kernel_hash
    from paged_kv_cache_119_amd._binding import pool_desc_of
    from synth import build_tables, duplicate_shared, make_pools, make_query, normal_16bit

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    if not os.path.exists(pkv.LIB_PATH):
        from paged_kv_cache_119_amd.build import build
        build()
    lib = pkv.load_library()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)

    t = build_tables(args.config, block_size=args.block_size)
    if args.op == "copy_blocks":
        return bench_copy_blocks(args, t, pkv, lib, dev)
    if args.op == "rows":
        return bench_rows(args, t, pkv, lib, dev)
    if args.kv == "fp8":
        return bench_fp8(args, t, pkv, lib, dev)
    if args.shared_prefix:
        return bench_shared(args, t, pkv, lib, dev)
    dup = None
    if args.duplicate_shared:
        dup_tab, copies, n_total = duplicate_shared(t)
        dup = (dup_tab, [c[0] for c in copies], n_total)
    S, H, D, B = t.num_seqs, t.num_heads, t.head_dim, t.block_size
    dsize = 2
    tab = torch.from_numpy(dup[0] if dup is not None else t.block_tables).to(dev)
    lens = torch.from_numpy(t.context_lens).to(dev)
    seq = torch.arange(S, dtype=torch.int32, device=dev)
    pos = torch.from_numpy((t.context_lens - 1).astype(np.int32)).to(dev)
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    print(f"[bench] {args.config}: S={S} H={H} D={D} B={B} N={t.num_blocks} "
          f"kv_tokens={t.kv_tokens()} replicas={args.replicas}", file=sys.stderr, flush=True)

    reps = []
    for r in range(args.replicas):
        t.seed += 1000 * r
        kp, vp = make_pools(t, dev)
        if dup is not None:
            src = torch.tensor(dup[1], device=dev, dtype=torch.long)
            kp, vp = torch.cat([kp, kp[src]], 0), torch.cat([vp, vp[src]], 0)
            assert kp.shape[0] == dup[2]
        q = make_query(t, dev)
        knew = normal_16bit((S, H, D), t.dtype, dev, t.seed * 16 + 9)
        vnew = normal_16bit((S, H, D), t.dtype, dev, t.seed * 16 + 10)
        t.seed -= 1000 * r
        reps.append((kp, vp, q, knew, vnew, torch.empty_like(q)))
    desc = pool_desc_of(reps[0][0], args.reuse_blocks)
    P = pkv.decode_partition_size(S, H, t.max_blocks, reps[0][0], args.partition_size)
    ws = pkv.alloc_workspace(S, H, t.max_blocks, reps[0][0], args.partition_size)
    ws_bytes = ws.numel()
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)
    dref = ctypes.byref(desc)

    # argument marshalling done once; the timed loop only issues the C calls
    calls = []
    for kp, vp, q, knew, vnew, out in reps:
        a_slot = (slots.data_ptr(), tab.data_ptr(), S, t.max_blocks, seq.data_ptr(), pos.data_ptr(), S, dref, sp)
        a_app = (kp.data_ptr(), vp.data_ptr(), knew.data_ptr(), vnew.data_ptr(), 0, 0, slots.data_ptr(), S,
                 dref, sp)
        a_dec = (out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(), tab.data_ptr(), lens.data_ptr(),
                 ctypes.c_float(t.scale), S, H, t.max_blocks, dref, P, ws.data_ptr(), ws_bytes, sp)
        a_fused = (out.data_ptr(), q.data_ptr(), knew.data_ptr(), vnew.data_ptr(), 0, kp.data_ptr(), vp.data_ptr(),
                   tab.data_ptr(), lens.data_ptr(), ctypes.c_float(t.scale), S, H, t.max_blocks, dref, P,
                   ws.data_ptr(), ws_bytes, sp)
        a_mrg = (out.data_ptr(), lens.data_ptr(), S, H, t.max_blocks, dref, P, ws.data_ptr(), ws_bytes, sp)
        calls.append((a_slot, a_app, a_dec, a_fused, a_mrg))

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {pkv.status_string(st)}")

    def step(i, ev=None):
        a_slot, a_app, a_dec, a_fused, a_mrg = calls[i % len(calls)]
        if args.one_call:
            if ev is not None:
                ev[0].record(stream)
            check(lib.pkv_paged_attention_decode_append(*a_fused), "paged_attention_decode_append")
            if ev is not None:
                ev[1].record(stream)
            return
        if args.separate_append:
            check(lib.pkv_slot_mapping(*a_slot), "slot_mapping")
            check(lib.pkv_reshape_and_cache(*a_app), "reshape_and_cache")
        if ev is not None:
            ev[0].record(stream)
        if args.separate_append:
            check(lib.pkv_decode_partitions(*a_dec), "decode_partitions")
        else:
            check(lib.pkv_decode_partitions_append(*a_fused), "decode_partitions_append")
        if ev is not None:
            ev[1].record(stream)
        check(lib.pkv_decode_merge(*a_mrg), "decode_merge")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    evs = [(KernelEvent(), KernelEvent()) for _ in range(args.steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    elapsed = time.perf_counter() - t0
    kern_ms = [a.elapsed_time(b) for a, b in evs]

    # whole-step time without per-kernel events (same work), for ms_per_step
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    print(f"[bench] timed {args.steps} steps ({elapsed * 1e3 / args.steps:.3f} ms/step host clock with events, "
          f"{ms_per_step:.4f} ms/step by events)", file=sys.stderr, flush=True)

    dec = acc.decode_bytes(t.context_lens, H, D, dsize, B)
    if args.separate_append:
        app = acc.append_bytes(S, S, H, D, dsize)
        step_bytes = dec["total"] + app["total"] + acc.slot_mapping_bytes(S)
        kern_bytes = dec["total"]
        kern_name = "decode_balanced_kernel" if P == 0 else "decode_partition_kernel"
    else:
        # the new rows are read once (counted in the KV bytes) and written once
        app_write = 2 * S * H * D * dsize
        step_bytes = dec["total"] + app_write
        kern_bytes = step_bytes
        kern_name = ("decode_balanced_kernel" if P == 0 else "decode_partition_kernel") + " (append fused)"
        if args.one_call:
            kern_name += " + merge, one call"
    value = step_bytes / (ms_per_step * 1e-3) / 1e9
    kern_mean_ms = float(np.mean(kern_ms))
    achieved = kern_bytes / (kern_mean_ms * 1e-3) / 1e9

    traffic = None
    if os.path.exists(TRAFFIC_FILE):
        with open(TRAFFIC_FILE) as f:
            tr = json.load(f)
        if tr.get("kernel_hash") == kernel_hash() and tr.get("config") == args.config and \
                tr.get("partition_size") == P and tr.get("separate_append", False) == args.separate_append \
                and not args.one_call:
            traffic = tr.get("hbm_bytes_per_launch")

    if args.copy_calibration:
        copy_calibration(torch, dev)

    # one parity spot check of the timed configuration (outputs finite)
    assert torch.isfinite(reps[0][5].float()).all().item(), "non-finite output"
    ceiling = read_ceiling(torch, dev, kern_bytes)

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(t, reps[0], args.cpu_budget_s)

    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": t.dtype,
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {S} seqs x {H} heads x {D}, B={B}, "
                               f"context_len {describe_lengths(t)}, one decode step: append of {S} tokens + "
                               f"attention ({'separate append' if args.separate_append else 'append fused'})"
                               + (", prefix blocks duplicated per sibling" if dup is not None else "")
                               + (", reuse hint (cached K/V loads)" if args.reuse_blocks else ""),
                   "global_batch": S, "kv_tokens": t.kv_tokens(), "block_size": B, "partition_size": P,
                   "pool_blocks": t.num_blocks, "replicas": args.replicas, "parallelism": "none (1 GPU)"},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBS, 2),
        "kv_tokens_per_s": round(t.kv_tokens() / (ms_per_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "roofline": {"kernel": kern_name, "bound": "hbm", "achieved": round(achieved, 2),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "bytes_per_launch": kern_bytes,
                     "mean_launch_us": round(kern_mean_ms * 1e3, 2),
                     "median_us": round(float(np.median(kern_ms)) * 1e3, 2),
                     "p10_us": round(float(np.percentile(kern_ms, 10)) * 1e3, 2),
                     "p90_us": round(float(np.percentile(kern_ms, 90)) * 1e3, 2)},
        "cpu_baseline": cpu,
        "read_ceiling": ceiling,
        "occupancy": with_measured(pkv.decode_launch_info(S, H, t.max_blocks, desc, P, 1, False,
                                                          not args.separate_append),
                                   f"{args.config}/B{B}/decode" + (f"/P{P}" if P else "")
                                   + ("/separate" if args.separate_append else "")
                                   + ("/one-call" if args.one_call else "")),
    }
    print(json.dumps(line), flush=True)
    return 0


def copy_calibration(torch, dev) -> None:
    """Three plain 1 GiB device copies: a counter run reads its FETCH_SIZE and
    WRITE_SIZE against the known byte count to scale the kernel's figures."""
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    del src, dst


def probe_lib():
    """The measurement helpers built beside the library (read probe, timing
    events); built here if missing."""
    global _PROBE
    if _PROBE is None:
        from paged_kv_cache_119_amd.build import PROBE_LIB, build_probe
        if not os.path.exists(PROBE_LIB):
            build_probe()
        lib = ctypes.CDLL(PROBE_LIB)
        vp = ctypes.c_void_p
        lib.pkvprobe_stream_read.argtypes = [vp, ctypes.c_int64, vp, ctypes.c_int, ctypes.c_int, vp]
        lib.pkvprobe_event_create.argtypes = [ctypes.POINTER(vp)]
        lib.pkvprobe_event_record.argtypes = [vp, vp]
        lib.pkvprobe_event_elapsed.argtypes = [ctypes.POINTER(ctypes.c_float), vp, vp]
        lib.pkvprobe_event_destroy.argtypes = [vp]
        _PROBE = lib
    return _PROBE


_PROBE = None


class KernelEvent:
    """A HIP timing event for per-launch durations, created with
    hipEventDisableSystemFence: recording it adds no system-scope cache
    writeback and invalidation between the launches it brackets.  Same
    record / elapsed_time use as torch.cuda.Event; read after a device
    synchronisation."""

    def __init__(self):
        self._lib = probe_lib()
        self.h = ctypes.c_void_p()
        st = self._lib.pkvprobe_event_create(ctypes.byref(self.h))
        if st != 0:
            raise RuntimeError(f"hipEventCreateWithFlags: HIP error {st}")

    def record(self, stream=None):
        import torch
        s = torch.cuda.current_stream() if stream is None else stream
        st = self._lib.pkvprobe_event_record(self.h, ctypes.c_void_p(int(s.cuda_stream)))
        if st != 0:
            raise RuntimeError(f"hipEventRecord: HIP error {st}")

    def elapsed_time(self, end) -> float:
        ms = ctypes.c_float()
        st = self._lib.pkvprobe_event_elapsed(ctypes.byref(ms), self.h, end.h)
        if st != 0:
            raise RuntimeError(f"hipEventElapsedTime: HIP error {st}")
        return ms.value

    def __del__(self):
        if getattr(self, "h", None) and self._lib is not None:
            self._lib.pkvprobe_event_destroy(self.h)


def read_ceiling(torch, dev, nbytes: int) -> dict:
    """Context for the roofline: a plain streaming read of the same number of
    bytes from one contiguous buffer (the probe built beside the library),
    cached and non-temporal loads, 32,768 workgroups; the median of 20
    HIP-event-timed launches, the faster of the two load kinds."""
    import numpy as np
    lib = probe_lib()
    n = max(16, nbytes // 16 * 16)
    bufs = [torch.zeros(n, dtype=torch.uint8, device=dev) for _ in range(2)]
    out = torch.zeros(1024, dtype=torch.int32, device=dev)
    sp = int(torch.cuda.current_stream(dev).cuda_stream)
    best = None
    for nt in (0, 1):
        ts = []
        for i in range(23):
            e0, e1 = KernelEvent(), KernelEvent()
            e0.record()
            st = lib.pkvprobe_stream_read(bufs[i % 2].data_ptr(), n, out.data_ptr(), 32768, nt, sp)
            e1.record()
            if st != 0:
                raise RuntimeError(f"read probe: HIP error {st}")
            ts.append((e0, e1))
        torch.cuda.synchronize()
        us = float(np.median([a.elapsed_time(b) for a, b in ts[3:]])) * 1e3
        if best is None or us < best[0]:
            best = (us, nt)
    del bufs
    return {"GB/s": round(n / best[0] / 1e3, 1), "bytes": n, "us": round(best[0], 2),
            "loads": "non-temporal" if best[1] else "cached",
            "how": "plain streaming read of one contiguous buffer of the kernel's byte count (events)"}


def bench_rows(args, t, pkv, lib, dev) -> int:
    """Several query rows per KV head on the matrix-core kernel: G query heads
    per KV head (grouped-query decode) and/or Q query tokens per sequence.
    One step = the split pass and the merge pass; the roofline times the
    split pass (16-bit pools with Q > 1: the whole call, which has no
    separate passes)."""
    import numpy as np
    import torch

    from synth import make_fp8_pools, make_pools, normal_16bit

    Hkv, D, B, S = t.num_heads, t.head_dim, t.block_size, t.num_seqs
    G = args.group or config_query_heads(t) // Hkv
    Q = args.queries
    H = G * Hkv
    dsize = 2
    fp8 = args.kv == "fp8"
    ks = vs = 1.0 / 60
    kvsize = 1 if fp8 else dsize
    tab = torch.from_numpy(t.block_tables).to(dev)
    lens = torch.from_numpy(t.context_lens).to(dev)
    reps = []
    for r in range(args.replicas):
        t.seed += 1000 * r
        kp, vp = make_fp8_pools(t, dev) if fp8 else make_pools(t, dev)
        t.seed -= 1000 * r
        shape = (S, H, D) if Q == 1 else (S, Q, H, D)
        q = normal_16bit(shape, t.dtype, dev, t.seed * 16 + 20 + r)
        reps.append((kp, vp, q, torch.empty_like(q)))
    desc = pkv.make_pool_desc(t.num_blocks, B, Hkv, D, t.dtype, args.reuse_blocks)
    dref = ctypes.byref(desc)
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)
    if fp8:
        wsb = pkv.fp8_multi_workspace_bytes(S, Q, H, t.max_blocks, reps[0][0], t.dtype)
    elif Q == 1:
        wsb = pkv.decode_workspace_bytes(S, H, t.max_blocks, reps[0][0], 0)
    else:
        wsb = pkv.multi_workspace_bytes(S, Q, H, t.max_blocks, reps[0][0])
    if wsb == 0:
        print("unsupported shape for the matrix-core path", file=sys.stderr)
        return 2
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {pkv.status_string(st)}")

    def step(i, ev=None):
        kp, vp, q, out = reps[i % len(reps)]
        if ev is not None:
            ev[0].record(stream)
        if fp8:
            check(lib.pkv_decode_partitions_fp8(out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                                                tab.data_ptr(), lens.data_ptr(), ctypes.c_float(D ** -0.5),
                                                ctypes.c_float(ks), ctypes.c_float(vs), S, Q, H, t.max_blocks,
                                                dref, ws.data_ptr(), wsb, sp), "decode_partitions_fp8")
            if ev is not None:
                ev[1].record(stream)
            check(lib.pkv_decode_merge_fp8(out.data_ptr(), lens.data_ptr(), S, Q, H, t.max_blocks, dref,
                                           ws.data_ptr(), wsb, sp), "decode_merge_fp8")
        elif Q == 1:
            check(lib.pkv_decode_partitions(out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(), tab.data_ptr(),
                                            lens.data_ptr(), ctypes.c_float(D ** -0.5), S, H, t.max_blocks, dref, 0,
                                            ws.data_ptr(), wsb, sp), "decode_partitions")
            if ev is not None:
                ev[1].record(stream)
            check(lib.pkv_decode_merge(out.data_ptr(), lens.data_ptr(), S, H, t.max_blocks, dref, 0, ws.data_ptr(),
                                       wsb, sp), "decode_merge")
        else:
            check(lib.pkv_paged_attention_multi(out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                                                tab.data_ptr(), lens.data_ptr(), ctypes.c_float(D ** -0.5), S, Q, H,
                                                t.max_blocks, dref, ws.data_ptr(), wsb, sp), "paged_attention_multi")
            if ev is not None:
                ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(KernelEvent(), KernelEvent()) for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    L = t.context_lens.astype(np.int64)
    kv = int(L.sum()) * Hkv * D * 2 * kvsize
    nbytes = kv + 2 * S * Q * H * D * dsize + int((-(-L // B)).sum()) * 4 + S * 4
    kern_mean_ms = float(np.mean(kern_ms))
    achieved = nbytes / (kern_mean_ms * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration(torch, dev)
    ceiling = read_ceiling(torch, dev, nbytes)
    kp0, vp0, q0, out0 = reps[0]
    cpu = None
    if not args.no_cpu_baseline:
        qrows = q0 if Q > 1 else q0[:, None]
        cpu = cpu_baseline(t, (kp0, vp0, qrows, None, None, out0), args.cpu_budget_s,
                           "rows_fp8" if fp8 else "rows", ks, vs, rows=(Q, H))
    line = {
        "metric": "paged attention, several query rows per KV head: achieved HBM GB/s + KV tokens/s",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": t.dtype + (" (K/V e4m3)" if fp8 else ""), "data": "synthetic",
        "config": {"workload": f"{args.config}: {S} seqs, {H} query heads over {Hkv} KV heads x {D}, {Q} query "
                               f"token(s) per sequence, B={B}, context_len {describe_lengths(t)}"
                               + (", e4m3 pools (scales 1/60)" if fp8 else ""),
                   "global_batch": S, "kv_tokens": t.kv_tokens(), "query_rows_per_kv_head": G * Q,
                   "parallelism": "none (1 GPU)"},
        "kv_tokens_per_s": round(t.kv_tokens() / (ms_per_step * 1e-3), 1),
        "roofline": {"kernel": (("decode_fp8_kernel" if fp8 else "decode_balanced_kernel") if G * Q == 1
                                else "decode_group_kernel" + (" (e4m3 K/V)" if fp8 else " + merge" if Q > 1 else "")),
                     "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": nbytes,
                     "mean_launch_us": round(kern_mean_ms * 1e3, 2),
                     "median_us": round(float(np.median(kern_ms)) * 1e3, 2),
                     "p10_us": round(float(np.percentile(kern_ms, 10)) * 1e3, 2),
                     "p90_us": round(float(np.percentile(kern_ms, 90)) * 1e3, 2)},
        "cpu_baseline": cpu,
        "read_ceiling": ceiling,
        "occupancy": with_measured(pkv.decode_launch_info(S, H, t.max_blocks, desc, 0, Q, args.kv == "fp8"),
                                   f"{args.config}/B{B}/rows/G{G}/Q{Q}" + ("/fp8" if fp8 else "")),
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_fp8(args, t, pkv, lib, dev) -> int:
    """Decode over an e4m3 KV cache: one step = the quantising append of the
    batch's new tokens and the attention -- by default one
    pkv_paged_attention_decode_append_fp8 call (split pass with the append
    fused in + merge pass); with --separate-append, slot mapping +
    pkv_reshape_and_cache_fp8 + pkv_paged_attention_decode_fp8.  The roofline
    times the decode call (both of its launches) with HIP events."""
    import numpy as np
    import torch

    from paged_kv_cache_119_amd import accounting as acc
    from synth import make_fp8_pools, make_query, normal_16bit

    S, H, D, B = t.num_seqs, t.num_heads, t.head_dim, t.block_size
    ks = vs = 1.0 / 60
    tab = torch.from_numpy(t.block_tables).to(dev)
    lens = torch.from_numpy(t.context_lens).to(dev)
    seq = torch.arange(S, dtype=torch.int32, device=dev)
    pos = torch.from_numpy((t.context_lens - 1).astype(np.int32)).to(dev)
    slots = torch.empty(S, dtype=torch.int64, device=dev)
    reps = []
    for r in range(args.replicas):
        t.seed += 1000 * r
        kp, vp = make_fp8_pools(t, dev)
        q = make_query(t, dev)
        knew = normal_16bit((S, H, D), t.dtype, dev, t.seed * 16 + 9)
        vnew = normal_16bit((S, H, D), t.dtype, dev, t.seed * 16 + 10)
        t.seed -= 1000 * r
        reps.append((kp, vp, q, knew, vnew, torch.empty_like(q)))
    desc = pkv.make_pool_desc(t.num_blocks, B, H, D, t.dtype, args.reuse_blocks)
    dref = ctypes.byref(desc)
    wsb = pkv.fp8_decode_workspace_bytes(S, H, t.max_blocks, reps[0][0], t.dtype)
    if wsb == 0:
        print("unsupported shape for the fp8 path", file=sys.stderr)
        return 2
    ws = torch.zeros(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)
    print(f"[bench] fp8 {args.config}: S={S} H={H} D={D} B={B} N={t.num_blocks} kv_tokens={t.kv_tokens()}",
          file=sys.stderr, flush=True)

    def check(st, what):
        if st != 0:
            raise RuntimeError(f"{what}: {pkv.status_string(st)}")

    def step(i, ev=None):
        kp, vp, q, knew, vnew, out = reps[i % len(reps)]
        if args.separate_append:
            check(lib.pkv_slot_mapping(slots.data_ptr(), tab.data_ptr(), S, t.max_blocks, seq.data_ptr(),
                                       pos.data_ptr(), S, dref, sp), "slot_mapping")
            check(lib.pkv_reshape_and_cache_fp8(kp.data_ptr(), vp.data_ptr(), knew.data_ptr(), vnew.data_ptr(), 0,
                                                0, slots.data_ptr(), S, ctypes.c_float(ks), ctypes.c_float(vs), dref,
                                                sp), "reshape_and_cache_fp8")
        if ev is not None:
            ev[0].record(stream)
        if args.separate_append:
            check(lib.pkv_paged_attention_decode_fp8(out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                                                     tab.data_ptr(), lens.data_ptr(), ctypes.c_float(t.scale),
                                                     ctypes.c_float(ks), ctypes.c_float(vs), S, H, t.max_blocks,
                                                     dref, ws.data_ptr(), wsb, sp), "paged_attention_decode_fp8")
        else:
            check(lib.pkv_paged_attention_decode_append_fp8(
                out.data_ptr(), q.data_ptr(), knew.data_ptr(), vnew.data_ptr(), 0, kp.data_ptr(), vp.data_ptr(),
                tab.data_ptr(), lens.data_ptr(), ctypes.c_float(t.scale), ctypes.c_float(ks), ctypes.c_float(vs),
                S, H, t.max_blocks, dref, ws.data_ptr(), wsb, sp), "paged_attention_decode_append_fp8")
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(KernelEvent(), KernelEvent()) for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    assert torch.isfinite(reps[0][5].float()).all().item(), "non-finite output"

    dec = acc.decode_bytes(t.context_lens, H, D, 2, B, kv_dtype_bytes=1)
    if args.separate_append:
        app = acc.append_bytes(S, S, H, D, 2, pool_dtype_bytes=1)
        step_bytes = dec["total"] + app["total"] + acc.slot_mapping_bytes(S)
        kern_bytes = dec["total"]
    else:
        # the new rows are read once (16-bit) and written once (codes); their
        # codes are counted in the KV bytes
        step_bytes = kern_bytes = dec["total"] + 2 * S * H * D * 2
    kern_mean_ms = float(np.mean(kern_ms))
    achieved = kern_bytes / (kern_mean_ms * 1e-3) / 1e9
    if args.copy_calibration:
        copy_calibration(torch, dev)
    cpu = None if args.no_cpu_baseline else cpu_baseline(t, reps[0], args.cpu_budget_s, "fp8", ks, vs)
    ceiling = read_ceiling(torch, dev, kern_bytes)
    line = {
        "metric": "paged decode attention over an FP8 (e4m3) KV cache: achieved HBM GB/s + KV tokens/s",
        "value": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": f"{t.dtype} (K/V e4m3)",
        "data": "synthetic",
        "config": {"workload": f"{args.config}: {S} seqs x {H} heads x {D}, B={B}, context_len "
                               f"{describe_lengths(t)}, e4m3 pools (scales 1/60), one decode step: quantising "
                               f"append of {S} tokens + attention "
                               f"({'separate append' if args.separate_append else 'append fused'})",
                   "global_batch": S, "kv_tokens": t.kv_tokens(), "block_size": B, "pool_blocks": t.num_blocks,
                   "replicas": args.replicas, "parallelism": "none (1 GPU)"},
        "kv_tokens_per_s": round(t.kv_tokens() / (ms_per_step * 1e-3), 1),
        "step_bytes": step_bytes,
        "roofline": {"kernel": "decode_fp8_kernel" + ("" if args.separate_append else " (append fused)")
                     + " + decode_balanced_merge_kernel", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": kern_bytes,
                     "mean_launch_us": round(kern_mean_ms * 1e3, 2),
                     "median_us": round(float(np.median(kern_ms)) * 1e3, 2),
                     "p10_us": round(float(np.percentile(kern_ms, 10)) * 1e3, 2),
                     "p90_us": round(float(np.percentile(kern_ms, 90)) * 1e3, 2)},
        "cpu_baseline": cpu,
        "read_ceiling": ceiling,
        "occupancy": with_measured(pkv.decode_launch_info(S, H, t.max_blocks, desc, 0, 1, True,
                                                          not args.separate_append),
                                   f"{args.config}/B{B}/fp8" + ("/separate" if args.separate_append else "")),
    }
    print(json.dumps(line), flush=True)
    return 0


def bench_shared(args, t, pkv, lib, dev) -> int:
    """Groups of siblings sharing a prompt prefix, decoded with
    pkv_paged_attention_decode_shared: one step is one call (prefix pass and
    its merge, suffix pass and its merge).  `value` counts the batch's bytes
    by the plain decode formula (every sequence's whole context), so it
    compares with the plain decode of the same batch; `unique` counts the
    bytes the call must move (each prefix once per group), and the roofline
    prices the call on those."""
    import numpy as np
    import torch

    from paged_kv_cache_119_amd import accounting as acc
    from synth import make_pools, make_query

    if "siblings" not in t.extra:
        print("--shared-prefix needs a workload of sibling groups (--config shared)", file=sys.stderr)
        return 2
    S, H, D, B = t.num_seqs, t.num_heads, t.head_dim, t.block_size
    k = t.extra["siblings"]
    P = t.extra["prefix_blocks"] * B
    tab = torch.from_numpy(t.block_tables).to(dev)
    lens = torch.from_numpy(t.context_lens).to(dev)
    pl_np = np.full(S // k, P, np.int32)
    pl = torch.from_numpy(pl_np).to(dev)
    reps = []
    for r in range(args.replicas):
        t.seed += 1000 * r
        kp, vp = make_pools(t, dev)
        q = make_query(t, dev)
        t.seed -= 1000 * r
        reps.append((kp, vp, q, torch.empty_like(q)))
    desc = pkv.pool_desc_of(reps[0][0], args.reuse_blocks)
    dref = ctypes.byref(desc)
    wsb = pkv.shared_prefix_workspace_bytes(S, H, t.max_blocks, reps[0][0], k)
    ws = torch.empty(wsb, dtype=torch.uint8, device=dev)
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)

    def step(i, ev=None):
        kp, vp, q, out = reps[i % len(reps)]
        if ev is not None:
            ev[0].record(stream)
        st = lib.pkv_paged_attention_decode_shared(out.data_ptr(), q.data_ptr(), kp.data_ptr(), vp.data_ptr(),
                                                   tab.data_ptr(), lens.data_ptr(), ctypes.c_float(t.scale), S, H,
                                                   t.max_blocks, dref, k, pl.data_ptr(), ws.data_ptr(), wsb, sp)
        if st != 0:
            raise RuntimeError(f"paged_attention_decode_shared: {pkv.status_string(st)}")
        if ev is not None:
            ev[1].record(stream)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(KernelEvent(), KernelEvent()) for _ in range(args.steps)]
    for i in range(args.steps):
        step(args.warmup + i, evs[i])
    torch.cuda.synchronize()
    call_ms = [a.elapsed_time(b) for a, b in evs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    by = acc.shared_prefix_bytes(t.context_lens, pl_np, k, H, D, 2, B)
    call_mean = float(np.mean(call_ms))
    achieved = by["total"] / (call_mean * 1e-3) / 1e9
    assert torch.isfinite(reps[0][3].float()).all().item(), "non-finite output"
    kp, vp, q, out = reps[0]
    cpu = None if args.no_cpu_baseline else cpu_baseline(t, (kp, vp, q, None, None, out), args.cpu_budget_s)
    line = {
        "metric": METRIC,
        "value": round(by["logical"] / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": t.dtype, "data": "synthetic",
        "config": {"workload": f"{args.config}: {S // k} prompts x {k} siblings ({S} seqs) x {H} heads x {D}, "
                               f"B={B}, {P}-token shared prefix, context_len {describe_lengths(t)}, decode with "
                               f"each prefix read once per group (pkv_paged_attention_decode_shared)",
                   "global_batch": S, "kv_tokens": t.kv_tokens(), "group_size": k, "prefix_tokens": P,
                   "replicas": args.replicas, "parallelism": "none (1 GPU)"},
        "value_counts": "logical bytes (every sequence's whole context, the plain decode formula)",
        "logical_bytes": by["logical"], "unique_bytes": by["total"],
        "unique_gbs": round(by["total"] / (ms_per_step * 1e-3) / 1e9, 2),
        "kv_tokens_per_s": round(t.kv_tokens() / (ms_per_step * 1e-3), 1),
        "roofline": {"kernel": "shared-prefix call: prefix pass (decode_group_kernel) + merge, suffix pass "
                               "(decode_balanced_kernel) + merge", "bound": "hbm",
                     "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBS, 4), "traffic": None, "bytes_per_launch": by["total"],
                     "mean_launch_us": round(call_mean * 1e3, 2),
                     "median_us": round(float(np.median(call_ms)) * 1e3, 2),
                     "p10_us": round(float(np.percentile(call_ms, 10)) * 1e3, 2),
                     "p90_us": round(float(np.percentile(call_ms, 90)) * 1e3, 2)},
        "cpu_baseline": cpu,
        "occupancy": {"prefix_pass": measured_occupancy(f"{args.config}/B{B}/shared-prefix/prefix-pass"),
                      "suffix_pass": measured_occupancy(f"{args.config}/B{B}/shared-prefix/suffix-pass")},
    }
    print(json.dumps(line), flush=True)
    return 0


def measured_occupancy(key: str):
    """Waves per SIMD measured by a rocprofv3 counter pass (recorded in
    profiles/ by rocprof_summary tables --occupancy) for this workload and
    mode, while the library sources are the ones it was measured on."""
    from paged_kv_cache_119_amd.rocprof_summary import OCCUPANCY_FILE, library_hash
    if not os.path.exists(OCCUPANCY_FILE):
        return None
    with open(OCCUPANCY_FILE) as f:
        rec = json.load(f).get(key)
    if not rec or rec.get("library_hash") != library_hash():
        return None
    return {"waves_per_simd": rec["waves_per_simd"], "kernel": rec["kernel"], "counter": rec["counter"],
            "source": rec["summary"]}


def with_measured(info: dict, key: str) -> dict:
    info = dict(info)
    info["measured"] = measured_occupancy(key)
    return info


def config_query_heads(t) -> int:
    from synth.configs import CONFIGS
    return int(CONFIGS.get(t.name, {}).get("query_heads", t.num_heads))


def bench_copy_blocks(args, t, pkv, lib, dev) -> int:
    """Batched block copy (copy-on-write): `--copy-pairs` random (src, dst)
    pairs of the workload's pool per launch, both pools; bytes = every copied
    block read once and written once."""
    import numpy as np
    import torch

    from synth import make_pools

    kp, vp = make_pools(t, dev, poison=False)
    n = args.copy_pairs
    if 2 * n > t.num_blocks:
        print(f"--copy-pairs {n} needs {2 * n} distinct blocks; the pool has {t.num_blocks}", file=sys.stderr)
        return 2
    rng = np.random.default_rng(7)
    sets = []
    for r in range(args.replicas):  # different pairs per launch, so no launch finds the last one's blocks cached
        perm = rng.permutation(t.num_blocks)
        sets.append(torch.from_numpy(np.stack([perm[:n], perm[n:2 * n]], 1).astype(np.int64)).to(dev))
    desc = pkv.pool_desc_of(kp)
    stream = torch.cuda.current_stream(dev)
    sp = int(stream.cuda_stream)
    dref = ctypes.byref(desc)

    def step(i):
        st = lib.pkv_copy_blocks(kp.data_ptr(), vp.data_ptr(), sets[i % len(sets)].data_ptr(), n, dref, sp)
        if st != 0:
            raise RuntimeError(pkv.status_string(st))

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    evs = [(KernelEvent(), KernelEvent()) for _ in range(args.steps)]
    for i in range(args.steps):
        evs[i][0].record(stream)
        step(args.warmup + i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    kern_ms = [a.elapsed_time(b) for a, b in evs]
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for i in range(args.steps):
        step(args.warmup + i)
    e1.record(stream)
    torch.cuda.synchronize()
    ms_per_step = e0.elapsed_time(e1) / args.steps
    block_bytes = t.num_heads * t.block_size * t.head_dim * 2
    nbytes = 2 * 2 * n * block_bytes + n * 16  # both pools, read + write, and the pairs
    kern_mean_ms = float(np.mean(kern_ms))
    # practical ceiling: the runtime's own device-to-device copy of the same
    # bytes (one contiguous buffer), timed the same way
    src_buf = torch.empty(2 * n * block_bytes, dtype=torch.uint8, device=dev)
    dst_buf = torch.empty_like(src_buf)
    for _ in range(3):
        dst_buf.copy_(src_buf)
    torch.cuda.synchronize()
    cev = [(KernelEvent(), KernelEvent()) for _ in range(args.steps)]
    for i in range(args.steps):
        cev[i][0].record(stream)
        dst_buf.copy_(src_buf)
        cev[i][1].record(stream)
    torch.cuda.synchronize()
    copy_ms = float(np.mean([a.elapsed_time(b) for a, b in cev]))
    del src_buf, dst_buf
    line = {
        "metric": "batched block copy (copy-on-write) achieved HBM GB/s, read + write",
        "value": round(nbytes / (ms_per_step * 1e-3) / 1e9, 2), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": t.dtype, "data": "synthetic",
        "config": {"workload": f"{args.config} pool ({t.num_blocks} blocks of {t.num_heads} x {t.block_size} x "
                               f"{t.head_dim}): {n} random block pairs per launch, K and V",
                   "block_pairs": n, "block_bytes": block_bytes, "parallelism": "none (1 GPU)"},
        "roofline": {"kernel": "copy_blocks_kernel", "bound": "hbm",
                     "achieved": round(nbytes / (kern_mean_ms * 1e-3) / 1e9, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(nbytes / (kern_mean_ms * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "traffic": None, "bytes_per_launch": nbytes, "mean_launch_us": round(kern_mean_ms * 1e3, 2)},
        "cpu_baseline": None,
        "copy_ceiling": {"GB/s": round(4 * n * block_bytes / (copy_ms * 1e-3) / 1e9, 1),
                         "bytes": 4 * n * block_bytes, "us": round(copy_ms * 1e3, 2),
                         "how": "the runtime's device-to-device copy of one contiguous buffer of the copied bytes "
                                "(read + write, events)"},
    }
    print(json.dumps(line), flush=True)
    return 0


def describe_lengths(t) -> str:
    L = t.context_lens
    return f"min {int(L.min())} median {int(__import__('numpy').median(L))} max {int(L.max())}"


def _oracle_pass(kind, files, meta, seqs, t_start, budget_s):
    """One oracle timing leg (runs in a worker process, or in the parent for
    the one-thread figure): wait until wall time t_start, then decode the
    given sequences (all heads, in turn, again and again) until budget_s has
    passed.  One BLAS thread.  Returns (sequences done, wall-clock start and
    end of the timed window)."""
    import numpy as np
    from threadpoolctl import threadpool_limits

    from oracle import paged_oracle as po

    kb, vb, qb, tabs, lens = (np.load(f, mmap_mode="r") for f in files)
    tabs, lens = np.asarray(tabs), np.asarray(lens)
    done = []
    with threadpool_limits(limits=1):
        while time.time() < t_start:
            time.sleep(0.001)
        w0 = time.time()
        t0 = time.perf_counter()
        i = 0
        while time.perf_counter() - t0 <= budget_s:
            s = seqs[i % len(seqs)]
            i += 1
            if kind in ("rows", "rows_fp8"):  # q [S, Q, H, D]: every query row of the sequence
                if kind == "rows_fp8":
                    po.decode_rows_fp8(np.asarray(qb[s:s + 1]), kb, vb, tabs[s:s + 1], lens[s:s + 1],
                                       meta["scale"], meta["block_size"], meta["dtype"], meta["k_scale"],
                                       meta["v_scale"])
                else:
                    po.decode_rows(np.asarray(qb[s:s + 1]), kb, vb, tabs[s:s + 1], lens[s:s + 1], meta["scale"],
                                   meta["block_size"], meta["dtype"])
            elif kind == "fp8":
                po.decode_rows_fp8(np.asarray(qb[s:s + 1])[:, None], kb, vb, tabs[s:s + 1], lens[s:s + 1],
                                   meta["scale"], meta["block_size"], meta["dtype"], meta["k_scale"],
                                   meta["v_scale"])
            else:
                for h in range(meta["num_heads"]):
                    po.decode_one(qb, kb, vb, tabs, lens, meta["scale"], meta["block_size"], meta["dtype"], s, h)
            done.append(s)
        dt = time.perf_counter() - t0
    return done, w0, w0 + dt


def _oracle_worker(a):
    return _oracle_pass(*a)


def host_cores() -> tuple:
    """(cores the oracle uses, cores this process may run on): the affinity
    set, capped at the host-core share a one-GPU job gets (OMP_NUM_THREADS,
    else 16)."""
    aff = len(os.sched_getaffinity(0))
    try:
        share = int(os.environ.get("OMP_NUM_THREADS") or 16)
    except ValueError:
        share = 16
    return max(1, min(aff, share)), aff


def cpu_baseline(t, rep, budget_s: float, kind: str = "16bit", ks: float = 1.0, vs: float = 1.0,
                 rows: tuple = None):
    """The float64 oracle timed on the host's cores, on host copies of one
    replica: N worker processes (N from host_cores(), one BLAS thread each)
    take the batch's sequences round-robin and decode them, all heads,
    passing over their share again until the budget is used; all workers
    start at one wall-clock time and the rate is taken over the span from the
    first start to the last end.  A one-thread leg in this process (budget / 2) is
    reported beside it.  GB/s of the same algorithmic bytes, and KV tokens/s.
    kind "rows" / "rows_fp8": q is [S, Q, H, D] over pools of t.num_heads KV
    heads, rows = (Q, H), and the bytes are those of the rows bench line."""
    import multiprocessing as mp
    import shutil
    import tempfile

    import numpy as np

    from paged_kv_cache_119_amd import accounting as acc
    from synth import to_bits

    kp, vp, q, _, _, _ = rep
    if kind in ("fp8", "rows_fp8"):
        kb, vb = kp.cpu().numpy(), vp.cpu().numpy()
    else:
        kb, vb = to_bits(kp), to_bits(vp)
    qb = to_bits(q)
    meta = {"scale": t.scale, "block_size": t.block_size, "dtype": t.dtype, "num_heads": t.num_heads,
            "k_scale": ks, "v_scale": vs}
    kv_bytes = 1 if kind == "fp8" else None
    tmp = tempfile.mkdtemp(prefix="pkv_oracle_", dir="/dev/shm" if os.path.isdir("/dev/shm") else None)
    try:
        files = []
        for name, arr in (("k", kb), ("v", vb), ("q", qb), ("tab", t.block_tables), ("lens", t.context_lens)):
            f = os.path.join(tmp, name + ".npy")
            np.save(f, np.ascontiguousarray(arr))
            files.append(f)
        del kb, vb

        def rate(done, dt):
            lens = t.context_lens[np.asarray(done, dtype=np.int64)]
            if rows is not None:
                Q, H = rows
                L = lens.astype(np.int64)
                by = (int(L.sum()) * t.num_heads * t.head_dim * 2 * (1 if kind == "rows_fp8" else 2)
                      + 2 * len(done) * Q * H * t.head_dim * 2 + int((-(-L // t.block_size)).sum()) * 4
                      + len(done) * 4)
            else:
                by = acc.decode_bytes(lens, t.num_heads, t.head_dim, 2, t.block_size,
                                      kv_dtype_bytes=kv_bytes)["total"]
            return by, int(lens.sum())

        # one thread, in this process
        done1, a1, b1 = _oracle_pass(kind, files, meta, list(range(t.num_seqs)), 0.0, budget_s / 2)
        dt1 = b1 - a1
        by1, tok1 = rate(done1, dt1)

        # N worker processes (started fresh, not forked from this GPU process)
        n, aff = host_cores()
        ctx = mp.get_context("spawn")
        t_start = time.time() + 8.0  # time for the workers to start and import
        jobs = [(kind, files, meta, list(range(w, t.num_seqs, n)) or [w % t.num_seqs], t_start, budget_s)
                for w in range(n)]
        with ctx.Pool(n) as pool:
            res = pool.map(_oracle_worker, jobs)
        done = [s for d, _, _ in res for s in d]
        dt = max(b for _, _, b in res) - min(a for _, a, _ in res)  # span of all windows
        by, tok = rate(done, dt)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    what = "sequence decodes" + (" over e4m3 pools" if kind in ("fp8", "rows_fp8") else "")
    if rows is not None:
        what += f" ({rows[0]} query token(s) x {rows[1]} query heads each)"
    return {"value": round(by / dt / 1e9, 4), "unit": "GB/s", "cores": n, "kind": "oracle",
            "sample": f"{len(done)} {what} ({len(done) / t.num_seqs:.1f} passes over the {t.num_seqs}-sequence "
                      f"batch, all {t.num_heads} {'KV ' if rows is not None else ''}heads), {tok} KV tokens, "
                      f"{dt:.1f} s, numpy float64, {n} worker "
                      f"processes x 1 BLAS thread ({aff} cores in the affinity set); the sequences dealt "
                      f"round-robin to the workers",
            "kv_tokens_per_s": round(tok / dt, 1),
            "one_thread": {"value": round(by1 / dt1 / 1e9, 4), "unit": "GB/s", "cores": 1,
                           "kv_tokens_per_s": round(tok1 / dt1, 1),
                           "sample": f"{len(done1)} {what}, {tok1} KV tokens, {dt1:.1f} s"}}


if __name__ == "__main__":
    sys.exit(main())
