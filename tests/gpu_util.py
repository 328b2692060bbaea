"""Helpers for the GPU parity tests: device copies of generated batches,
oracle evaluation on host copies, and the acceptance check."""

from __future__ import annotations

import math
import sys

import numpy as np

from oracle import paged_oracle as po
from synth import to_bits

DEV = "cuda:0"
TOL_ABS = 2e-3
TOL_REL = 1e-2


def log(msg: str) -> None:
    print(msg, flush=True)
    sys.stdout.flush()


def device_tables(t, device=DEV):
    import torch
    return (torch.from_numpy(np.ascontiguousarray(t.block_tables)).to(device),
            torch.from_numpy(np.ascontiguousarray(t.context_lens)).to(device))


def assert_close(gpu_bits: np.ndarray, ref: np.ndarray, dtype: str, what: str) -> dict:
    """|gpu - ref| <= 2e-3 + 1e-2 |ref| elementwise; returns error statistics."""
    g = po.bits_to_f64(gpu_bits, dtype)
    ref = np.asarray(ref, dtype=np.float64)
    assert g.shape == ref.shape, (g.shape, ref.shape)
    assert np.all(np.isfinite(g)), f"{what}: non-finite GPU output"
    err = np.abs(g - ref)
    bound = TOL_ABS + TOL_REL * np.abs(ref)
    worst = np.unravel_index(np.argmax(err - bound), err.shape)
    stats = {"max_abs": float(err.max()) if err.size else 0.0,
             "max_rel": float((err / np.maximum(np.abs(ref), 1e-30)).max()) if err.size else 0.0}
    assert np.all(err <= bound), (f"{what}: tolerance exceeded at {worst}: gpu={g[worst]} ref={ref[worst]} "
                                  f"err={err[worst]} stats={stats}")
    log(f"  {what}: max|err|={stats['max_abs']:.3e}")
    return stats


class HeadCache:
    """Host copies of single heads of device pools, for oracle samples at full
    size (a whole pool may not fit comfortably in host memory)."""

    def __init__(self, k_pool, v_pool):
        self.k_pool, self.v_pool = k_pool, v_pool
        self.cache = {}

    def get(self, h: int):
        if h not in self.cache:
            self.cache = {}  # keep one head at a time
            kh = to_bits(self.k_pool[:, h:h + 1])
            vh = to_bits(self.v_pool[:, h:h + 1])
            self.cache[h] = (kh, vh)
        return self.cache[h]


def oracle_samples(t, q_bits, heads: HeadCache, pairs, dtype=None):
    """Float64 oracle outputs for the given (s, h) pairs; returns [len(pairs), D].

    The oracle walks the real block table over a host copy of head h of each
    pool (shape [N, 1, B, D])."""
    dtype = dtype or t.dtype
    out = np.zeros((len(pairs), t.head_dim))
    for i, (s, h) in enumerate(pairs):
        kh, vh = heads.get(h)
        qh = q_bits[s:s + 1, h:h + 1]
        lens = np.array([t.context_lens[s]], np.int32)
        out[i] = po.decode_one(qh, kh, vh, t.block_tables[s:s + 1], lens, t.scale, t.block_size, dtype, 0, 0)
    return out


def sample_pairs(t, rng, per_head=None, heads=None):
    """(s, h) pairs covering the shortest and longest sequences, first and last
    heads, plus random ones."""
    S, H = t.num_seqs, t.num_heads
    L = t.context_lens
    heads = heads if heads is not None else sorted({0, H - 1, int(rng.integers(H))})
    seqs = sorted({int(np.argmin(L)), int(np.argmax(L)), *[int(x) for x in rng.integers(0, S, size=6)]})
    if per_head is None:
        return [(s, h) for h in heads for s in seqs]
    return [(s, h) for h in heads for s in range(S)]


def scale_of(D: int) -> float:
    return 1.0 / math.sqrt(D)
