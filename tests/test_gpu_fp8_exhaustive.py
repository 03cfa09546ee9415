"""The GPU's FP8 E4M3 encoder over every fp32 bit pattern it can meet.

The FP8 codec row of the method's oracle (cartridge page, "What fake
quantization does with the other eight bits": each value rounded to the
nearest E4M3 value) is checked exhaustively: every finite fp32 pattern with
|x| <= 448 goes through kvq_quantize (fp32 input) in rows whose absmax is 448,
so the per-token scale is exactly 1 and the encoder rounds y = x itself.
Those are all the values the rounding step can see, since y = x / s lies in
[-448, 448] for every row.  Codes are compared with torch's float8_e4m3fn
cast (round to nearest, ties to even) on every value and with the oracle's
encoder on a sample.  Rows with larger magnitudes exercise the scale path
(s = amax / 448 in fp32) on a seeded sample against the oracle."""
import numpy as np
import pytest
import torch

from oracle.numerics import e4m3_encode
from oracle.quant import fp8_token_quantize

pytestmark = pytest.mark.gpu

FREE = 127                   # values per row; channel 127 holds the 448 anchor
BATCH = 1 << 26              # fp32 patterns per kernel call


def _encode_rows(kvq, rows: torch.Tensor):
    """kvq_quantize of fp32 rows [n, 128] (one sequence, one KV head) to FP8."""
    n = rows.shape[0]
    st = kvq.alloc_stored(1, 1, n, "fp8", None, False, rows.device)
    kvq.quantize_into(st, rows.view(1, 1, n, 128), None)
    return st.k.view(n, 128), st.k_scale.view(n)


@pytest.mark.parametrize("sign", [0, 1])
def test_fp8_encoder_every_fp32_pattern_up_to_448(gpu_lib, sign):
    kvq = gpu_lib
    dev = torch.device("cuda")
    top = 0x43E00000                                  # 448.0
    base = sign << 31
    total = top + 1
    rng = np.random.default_rng(2026 + sign)
    checked = 0
    for start in range(0, total, BATCH):
        stop = min(start + BATCH, total)
        bits = torch.arange(base + start, base + stop, dtype=torch.int64, device=dev).to(torch.int32)
        x = bits.view(torch.float32)
        n = x.numel()
        n_rows = -(-n // FREE)
        flat = torch.zeros(n_rows * FREE, dtype=torch.float32, device=dev)
        flat[:n] = x
        rows = torch.empty((n_rows, 128), dtype=torch.float32, device=dev)
        rows[:, :FREE] = flat.view(n_rows, FREE)
        rows[:, FREE] = 448.0
        del flat
        codes, scales = _encode_rows(kvq, rows)
        assert bool((scales == 1.0).all())
        got = codes[:, :FREE].reshape(-1)[:n]
        want = x.to(torch.float8_e4m3fn).view(torch.uint8)
        bad = (got != want).nonzero()
        assert bad.numel() == 0, f"{bad.numel()} codes differ, first at pattern {hex(base + start + int(bad[0]))}"
        assert bool((codes[:, FREE] == 0x7E).all())
        # the oracle's encoder on a sample of this batch
        idx = torch.from_numpy(rng.integers(0, n, 1 << 14)).to(dev)
        ref = e4m3_encode(x[idx].cpu().numpy())
        np.testing.assert_array_equal(got[idx].cpu().numpy(), ref)
        checked += n
        del rows, codes, scales, got, want, x, bits
    assert checked == total
    print(f"[fp8 exhaustive] sign {sign}: {checked} fp32 patterns, codes equal", flush=True)


def test_fp8_encoder_scale_path_sampled(gpu_lib):
    """Rows whose absmax exceeds 448, from just above 448 to near FLT_MAX (the
    anchor is a random pattern, the other values random patterns up to it):
    codes and scales bit-exact against the oracle's per-token encoder."""
    kvq = gpu_lib
    rng = np.random.default_rng(7)
    n_rows = 1 << 14
    lo, hi = 0x43E00001, 0x7F7FFFFF
    amax_bits = rng.integers(lo, hi + 1, n_rows, dtype=np.int64).astype(np.uint32)
    amax = amax_bits.view(np.float32)
    # other values: random patterns with magnitude below the anchor
    frac = rng.random((n_rows, 127))
    mag = (frac * amax[:, None].astype(np.float64)).astype(np.float32)
    mag = np.minimum(mag, amax[:, None])
    sgn = np.where(rng.random((n_rows, 127)) < 0.5, -1.0, 1.0).astype(np.float32)
    anchor = np.where(rng.random(n_rows) < 0.5, -amax, amax).astype(np.float32)[:, None]
    rows = np.concatenate([mag * sgn, anchor], axis=1).astype(np.float32)
    codes, scales = _encode_rows(kvq, torch.from_numpy(rows).cuda())
    ref_codes, ref_s = fp8_token_quantize(rows.astype(np.float64))
    np.testing.assert_array_equal(scales.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_codes)
    print(f"[fp8 scale path] {n_rows} rows, amax in ({float(amax.min()):.3e}, {float(amax.max()):.3e})", flush=True)
