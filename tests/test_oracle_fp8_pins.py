"""Pins for the oracle's FP8 (OCP e4m3) cache: the code tables against
PyTorch's float8_e4m3fn conversions (a library routine that shares nothing
with the oracle), closed forms of the format, the rounding error bound, and
the attention over an e4m3 pool against the already pinned 16-bit oracle on
pools that hold the same values exactly."""

import numpy as np
import pytest

from oracle import paged_oracle as po

torch = pytest.importorskip("torch")


def _torch_decode(codes):
    return torch.from_numpy(np.asarray(codes, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode_f32(x32):
    """torch's float32 -> e4m3fn conversion (round to nearest even, no
    saturation: only inputs below 464 in magnitude are meaningful)."""
    return torch.from_numpy(np.asarray(x32, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_e4m3_decode_matches_torch_for_every_code():
    c = np.arange(256, dtype=np.uint8)
    np.testing.assert_array_equal(po.e4m3_to_f64(c), _torch_decode(c))


def test_e4m3_closed_forms():
    v = po.e4m3_to_f64(np.array([0x00, 0x80, 0x01, 0x07, 0x08, 0x38, 0x39, 0xC0, 0x7E, 0xFE, 0x7F, 0xFF,
                                 0x77, 0x78], np.uint8))
    assert v[0] == 0.0 and not np.signbit(v[0])
    assert v[1] == 0.0 and np.signbit(v[1])
    assert v[2] == 2.0 ** -9                  # smallest subnormal
    assert v[3] == 7 * 2.0 ** -9              # largest subnormal
    assert v[4] == 2.0 ** -6                  # smallest normal
    assert v[5] == 1.0 and v[6] == 1.125
    assert v[7] == -2.0
    assert v[8] == 448.0 and v[9] == -448.0   # largest finite
    assert np.isnan(v[10]) and np.isnan(v[11])
    assert v[12] == 240.0 and v[13] == 256.0  # exponent 14 mantissa 7, exponent 15 mantissa 0


def test_e4m3_encode_round_trips_every_finite_code():
    c = np.array([x for x in range(256) if x & 0x7F != 0x7F], np.uint8)
    np.testing.assert_array_equal(po.f64_to_e4m3(po.e4m3_to_f64(c)), c)


def test_e4m3_encode_ties_go_to_the_even_code():
    mags = po.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mid = (mags[:-1] + mags[1:]) / 2  # exact in float64
    got = po.f64_to_e4m3(mid).astype(int)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    np.testing.assert_array_equal(got, want)
    np.testing.assert_array_equal(po.f64_to_e4m3(-mid).astype(int), want | 0x80)
    # just off the midpoint goes to the nearer code
    np.testing.assert_array_equal(po.f64_to_e4m3(np.nextafter(mid, np.inf)).astype(int), lo + 1)
    np.testing.assert_array_equal(po.f64_to_e4m3(np.nextafter(mid, -np.inf)).astype(int), lo)


def test_e4m3_encode_matches_torch_below_saturation():
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.normal(0, 60, 50000), rng.normal(0, 0.01, 50000), rng.normal(0, 1e-3, 20000),
                        rng.uniform(-463.9, 463.9, 20000)]).astype(np.float32)
    mags = po.e4m3_to_f64(np.arange(0x7F, dtype=np.uint8))
    mid = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)  # midpoints are float32 values
    x = np.concatenate([x, mid, -mid])
    np.testing.assert_array_equal(po.f64_to_e4m3(x.astype(np.float64)), _torch_encode_f32(x))


def test_e4m3_encode_saturates_and_keeps_nan_and_sign():
    x = np.array([448.0, 455.9, 464.0, 470.0, 1e6, np.inf, -464.0, -np.inf, np.nan, 2.0 ** -10,
                  -(2.0 ** -10), 2.0 ** -10 * (1 + 1e-9), -1e-30, 0.0, -0.0])
    got = po.f64_to_e4m3(x).astype(int).tolist()
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0xFE, 0x7F, 0x00, 0x80, 0x01, 0x80, 0x00, 0x80]


def test_e4m3_encode_is_monotone_and_within_half_a_step():
    x = np.sort(np.random.default_rng(4).uniform(-500, 500, 20000))
    v = po.e4m3_to_f64(po.f64_to_e4m3(x))
    assert np.all(np.diff(v) >= 0)
    inr = np.abs(x) <= 448
    # relative error at most 2^-4 in the normal range, absolute 2^-10 below it
    bound = np.maximum(np.abs(x) * 2.0 ** -4, 2.0 ** -10)
    assert np.all(np.abs(v - x)[inr] <= bound[inr])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("scale", [1.0, 0.0137, 3.7, 2.0 ** -8])
def test_quantize_matches_torch_float32_product_then_cast(dtype, scale):
    rng = np.random.default_rng(5)
    x = torch.from_numpy(rng.normal(0, 2, 40000).astype(np.float32)).to(
        torch.float16 if dtype == "f16" else torch.bfloat16)
    bits = x.view(torch.int16).numpy().view(np.uint16)
    y = x.float() * (torch.tensor(1.0, dtype=torch.float32) / torch.tensor(scale, dtype=torch.float32))
    ok = y.abs() < 464
    want = y.to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = po.quantize_e4m3(bits, dtype, scale)
    np.testing.assert_array_equal(got[ok.numpy()], want[ok.numpy()])
    assert np.all(got[~ok.numpy()] & 0x7F == 0x7E)


def test_reshape_and_cache_fp8_writes_quantised_rows_only():
    rng = np.random.default_rng(6)
    N, H, B, D, T = 6, 2, 4, 8, 9
    k = rng.normal(0, 1, (T, H, D)).astype(np.float16).view(np.uint16)
    v = rng.normal(0, 1, (T, H, D)).astype(np.float16).view(np.uint16)
    slots = np.array([0, 5, 23, -1, 7, 24, 1000, 13, 2], np.int64)
    kp = rng.integers(0, 256, (N, H, B, D)).astype(np.uint8)
    vp = rng.integers(0, 256, (N, H, B, D)).astype(np.uint8)
    kp0, vp0 = kp.copy(), vp.copy()
    po.reshape_and_cache_fp8(k, v, kp, vp, slots, B, "f16", 0.25, 3.0)
    # the same through the (pinned) 16-bit append of precomputed codes
    kw, vw = kp0.copy(), vp0.copy()
    po.reshape_and_cache(po.quantize_e4m3(k, "f16", 0.25), po.quantize_e4m3(v, "f16", 3.0), kw, vw, slots, B)
    np.testing.assert_array_equal(kp, kw)
    np.testing.assert_array_equal(vp, vw)
    written = np.zeros((N, B), bool)
    for sl in slots:
        if 0 <= sl < N * B:
            written[sl // B, sl % B] = True
    np.testing.assert_array_equal(kp[~written[:, None, :].repeat(H, 1)], kp0[~written[:, None, :].repeat(H, 1)])


def _fp8_case(lengths, Hkv, B, D, seed):
    rng = np.random.default_rng(seed)
    nb = [-(-L // B) for L in lengths]
    N = sum(nb) + 2
    perm = rng.permutation(N)
    tables = np.full((len(lengths), max(nb)), -1, np.int32)
    c = 0
    for s in range(len(lengths)):
        tables[s, :nb[s]] = perm[c:c + nb[s]]
        c += nb[s]
    kc = rng.integers(0, 256, (N, Hkv, B, D)).astype(np.uint8)
    vc = rng.integers(0, 256, (N, Hkv, B, D)).astype(np.uint8)
    for pool in (kc, vc):  # random codes without NaN
        pool[(pool & 0x7F) == 0x7F] ^= 1
    return kc, vc, tables, np.asarray(lengths, np.int32)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fp8_decode_equals_16bit_decode_of_the_same_values(dtype):
    """Every e4m3 value is exactly a binary16 and a bfloat16 value, so with
    unit scales the fp8 attention equals the 16-bit attention over pools
    holding those values."""
    kc, vc, tables, lens = _fp8_case([1, 7, 30, 64], 2, 8, 16, 8)
    q = po.f64_to_bits(np.random.default_rng(9).normal(0, 0.05, (4, 2, 4, 16)), dtype)
    kb = po.f64_to_bits(po.e4m3_to_f64(kc), dtype)
    vb = po.f64_to_bits(po.e4m3_to_f64(vc), dtype)
    assert np.array_equal(po.bits_to_f64(kb, dtype), po.e4m3_to_f64(kc))
    ref = po.decode_rows(q, kb, vb, tables, lens, 0.3, 8, dtype)
    got = po.decode_rows_fp8(q, kc, vc, tables, lens, 0.3, 8, dtype, 1.0, 1.0)
    np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-300)


def test_fp8_decode_scales_act_on_scores_and_values():
    """k_scale multiplies every score (the same as a larger softmax scale) and
    v_scale the output; powers of two keep the float32 scales exact."""
    kc, vc, tables, lens = _fp8_case([5, 33, 17], 2, 8, 16, 10)
    q = po.f64_to_bits(np.random.default_rng(11).normal(0, 0.05, (3, 1, 2, 16)), "f16")
    a = po.decode_rows_fp8(q, kc, vc, tables, lens, 0.1, 8, "f16", 0.5, 4.0)
    b = po.decode_rows_fp8(q, kc, vc, tables, lens, float(np.float32(0.1)) * 0.5, 8, "f16", 1.0, 1.0)
    np.testing.assert_allclose(a, 4.0 * b, rtol=1e-12)
    # a mistake swapping the roles of the scales is caught
    c = po.decode_rows_fp8(q, kc, vc, tables, lens, 0.1, 8, "f16", 4.0, 0.5)
    assert not np.allclose(a, c, rtol=1e-3)
