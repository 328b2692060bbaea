"""GPU: pkv_decode_launch_info reports what the split passes launch --
the grid, resident waves per SIMD and the registers, LDS and scratch of the
library's own kernels -- consistently with the documented design (three
waves per SIMD launched for the 16-bit and e4m3 streams, two for the
matrix-core kernel, no spills)."""

import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

import paged_kv_cache_119_amd as pkv  # noqa: E402

from .gpu_util import log  # noqa: E402


def _lds(S):
    return (S + 1) * 8 + S * 4  # chunk prefix (int64) and lengths (int32)


@pytest.mark.parametrize("append", [False, True])
def test_balanced_16bit_stream(append):
    S, H, maxb = 64, 40, 128
    d = pkv.make_pool_desc(2000, 16, H, 128, "f16")
    info = pkv.decode_launch_info(S, H, maxb, d, append=append)
    log(f"16-bit balanced append={append}: {info}")
    assert info["balanced"] == 1 and info["partition_size"] == 0
    assert info["waves_per_workgroup"] == 4
    # the kernel with the append holds 3 waves per SIMD, the one without 4;
    # the split launches for the smaller, so both agree on the worker count
    assert info["waves_per_simd"] == (3 if append else 4)
    assert info["workgroups"] == info["compute_units"] * 3
    assert 0 < info["registers"] <= (168 if append else 128)
    assert info["scratch_bytes"] == 0
    assert info["lds_dynamic_bytes"] == _lds(S)


def test_small_batch_launches_only_the_workers_it_can_use():
    # 2 sequences of at most 32 tokens: 2 * 4 heads * 2 chunks = 16 chunks,
    # slices of at least 8 chunks -> at most 2 workers -> one workgroup
    d = pkv.make_pool_desc(64, 16, 4, 128, "f16")
    info = pkv.decode_launch_info(2, 4, 2, d)
    log(f"small batch: {info}")
    assert info["workgroups"] == 1


def test_fixed_partitions_grid():
    S, H, maxb = 8, 4, 64  # 1024 tokens -> 2 partitions of 512
    d = pkv.make_pool_desc(600, 16, H, 128, "f16")
    info = pkv.decode_launch_info(S, H, maxb, d, partition_size=512)
    log(f"fixed P=512: {info}")
    assert info["balanced"] == 0 and info["partition_size"] == 512
    items = S * H * 2
    assert info["workgroups"] >= items and info["workgroups"] % 128 == 0
    assert info["scratch_bytes"] == 0


def test_matrix_core_and_fp8_kernels():
    S, H, Hkv, maxb = 64, 64, 8, 128
    d = pkv.make_pool_desc(9000, 16, Hkv, 128, "bf16")
    g = pkv.decode_launch_info(S, H, maxb, d)
    log(f"grouped 16-bit: {g}")
    assert g["balanced"] == 1 and g["waves_per_simd"] == 2 and g["scratch_bytes"] == 0
    assert g["lds_static_bytes"] > 0  # the K transpose tiles
    g8 = pkv.decode_launch_info(S, H, maxb, d, fp8=True)
    log(f"grouped e4m3: {g8}")
    assert g8["waves_per_simd"] == 2 and g8["scratch_bytes"] == 0
    dm = pkv.make_pool_desc(2000, 16, 40, 128, "f16")
    f8 = pkv.decode_launch_info(64, 40, 128, dm, fp8=True)
    log(f"e4m3 stream: {f8}")
    assert f8["waves_per_simd"] == 3 and f8["scratch_bytes"] == 0
    assert f8["registers"] <= 168
