"""Pins of Philox4x32-10, the dither stream and the dithered INT8 quantizer
(WitCert Sec. 4.2, 6.2.1).  CPU only."""
import os
import shutil
import subprocess

import numpy as np
import pytest

from oracle.numerics import bf16_bits_to_f64, f64_to_bf16_bits
from oracle.philox import dither, dither_counters, philox4x32_10
from oracle.quant import int8_dither_dequant, int8_dither_quantize


HELPER = os.path.join(os.path.dirname(__file__), "helpers", "philox_rocrand_ref.cpp")


@pytest.fixture(scope="module")
def rocrand_ref(tmp_path_factory):
    """rocRAND's Philox4x32-10 engine, compiled from its public header and run
    on the host: an implementation independent of the oracle's."""
    hipcc = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
    if not os.path.exists(hipcc) or not os.path.exists("/opt/rocm/include/rocrand/rocrand_kernel.h"):
        pytest.skip("hipcc / rocRAND headers not available")
    exe = str(tmp_path_factory.mktemp("philox") / "philox_ref")
    subprocess.run([hipcc, "-O1", "-x", "hip", "--offload-arch=gfx950", HELPER, "-o", exe],
                   check=True, capture_output=True, timeout=300)
    return exe


@pytest.mark.parametrize("seed", [0, 1, 0xDEADBEEFCAFEF00D, 20260004])
def test_philox_matches_rocrand_engine(rocrand_ref, seed):
    n = 1024
    out = subprocess.run([rocrand_ref, str(seed), str(n)], check=True, capture_output=True,
                         text=True, timeout=60).stdout
    ref = np.array([[int(x) for x in line.split()] for line in out.strip().splitlines()], np.uint32)
    ctr = np.zeros((n, 4), np.uint64)
    ctr[:, 0] = np.arange(n)
    ours = philox4x32_10(ctr, (seed & 0xFFFFFFFF, seed >> 32))
    np.testing.assert_array_equal(ours, ref)


def test_philox_counter_words_all_matter():
    base = np.zeros((1, 4), np.uint64)
    out0 = philox4x32_10(base, (1, 2))
    for w in range(4):
        c = base.copy(); c[0, w] = 1
        assert not np.array_equal(philox4x32_10(c, (1, 2)), out0)
    assert not np.array_equal(philox4x32_10(base, (1, 3)), out0)
    assert np.array_equal(philox4x32_10(base, (0x100000001, 2)), out0)   # 32-bit key words


def test_dither_stream_unique_over_five_tuple():
    """Distinct (stream, layer, KV head, token, channel group) give distinct
    counters (WitCert Sec. 6.3.1's five-tuple)."""
    seen = set()
    for stream in range(3):
        for layer in (0, 1, 35):
            for kvh in (0, 7):
                ctr = dither_counters(np.arange(300)[:, None], np.arange(0, 128, 4)[None, :],
                                      layer, kvh, stream).reshape(-1, 4)
                for row in map(tuple, ctr.tolist()):
                    assert row not in seen
                    seen.add(row)


def test_keys_and_values_share_the_dither():
    """The five-tuple has no key/value component: a token's keys and values are
    quantized with the same dither, so equal inputs give equal codes, and a
    changed input on one side leaves the other's codes alone."""
    from oracle.pipeline import RegionSpec, encode_region
    rng = np.random.default_rng(3)
    x = _bf16(rng.standard_normal((2, 300, 128)))
    spec = RegionSpec(k_fmt="int8", v_fmt="int8", seed=77, layer=4, stream=1)
    enc = encode_region(x[0], x[0], spec, kv_head=2)
    np.testing.assert_array_equal(enc.k_codes, enc.v_codes)
    enc2 = encode_region(x[0], x[1], spec, kv_head=2)
    np.testing.assert_array_equal(enc2.k_codes, enc.k_codes)
    assert not np.array_equal(enc2.v_codes, enc.v_codes)


def test_dither_range_and_uniformity():
    xi = dither(20260004, 3, 5, 2, np.arange(4096), 128).ravel().astype(np.float64)
    assert xi.min() >= -0.5 and xi.max() < 0.5
    # exact on the 2^-24 grid
    assert np.all((xi + 0.5) * 2 ** 24 == np.round((xi + 0.5) * 2 ** 24))
    # mean 0 and variance 1/12 within 6 standard errors; KS distance small
    n = xi.size
    assert abs(xi.mean()) < 6 * np.sqrt(1 / 12 / n)
    assert abs(xi.var() - 1 / 12) < 6 * np.sqrt(1 / 180 / n)
    srt = np.sort(xi) + 0.5
    ks = np.max(np.abs(srt - (np.arange(1, n + 1) / n)))
    assert ks < 1.95 / np.sqrt(n)          # 0.1% level


def _bf16(x):
    return bf16_bits_to_f64(f64_to_bf16_bits(x))


def test_int8_dither_error_bound_no_clipping_and_moments():
    rng = np.random.default_rng(7)
    T = 1000                                 # three full blocks and a ragged one
    x = rng.standard_normal((T, 128))
    x[:, [5, 9, 60, 101]] *= 8
    x = _bf16(x)
    xi = dither(99, 2, 1, 0, np.arange(T), 128)
    codes, s16, clipped = int8_dither_quantize(x, xi)
    assert clipped == 0 and s16.shape == (4, 128) and s16.dtype == np.float16
    assert np.max(np.abs(codes.astype(int))) <= 127
    xh = int8_dither_dequant(codes, s16, xi)
    s = s16.astype(np.float64)[np.arange(T) // 256]
    ratio = np.abs(xh - x) / (s / 2)
    assert ratio.max() <= 1 + 1e-5            # |err| <= s/2 (WitCert Sec. 6.2.3)
    r = (xh - x) / s                           # residual / step: uniform on [-1/2, 1/2)
    assert abs(r.mean()) < 6 * np.sqrt(1 / 12 / r.size)
    assert abs(r.var() - 1 / 12) < 6 * np.sqrt(1 / 180 / r.size)
    # the residual does not depend on the input (classical subtractive dither)
    assert abs(np.corrcoef(r.ravel(), (x / s).ravel())[0, 1]) < 0.01


def test_int8_scale_is_stored_fp16_of_amax_over_126_5():
    rng = np.random.default_rng(8)
    x = _bf16(rng.standard_normal((300, 128)) * 3)
    xi = np.zeros((300, 128), np.float32)
    _, s16, _ = int8_dither_quantize(x, xi)
    amax0 = np.max(np.abs(x[:256]), axis=0).astype(np.float32)
    np.testing.assert_array_equal(s16[0], (amax0 / np.float32(126.5)).astype(np.float32).astype(np.float16))
    amax1 = np.max(np.abs(x[256:]), axis=0).astype(np.float32)
    np.testing.assert_array_equal(s16[1], (amax1 / np.float32(126.5)).astype(np.float32).astype(np.float16))
    # with zero dither this is plain rounding: codes = rint(x / s)
    c, _, _ = int8_dither_quantize(x, xi)
    s = s16.astype(np.float32)[np.arange(300) // 256]
    np.testing.assert_array_equal(c, np.rint((x.astype(np.float32) / s).astype(np.float32)).astype(np.int8))
