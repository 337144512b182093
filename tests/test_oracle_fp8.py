"""Pins of the fp8 latent-cache oracle (oracle/fp8_cache.py), CPU only.

E4M3 decoding and encoding are pinned to torch's float8_e4m3fn conversions (a library
routine), the block scale and codes to a hand-computed example (tests/golden), and the
quantiser to its error bound and to exactness on values the format holds."""
import json
import math
import os

import numpy as np
import torch

from oracle import fp8_cache as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_row_example.json")


def _torch_codes(x):
    return torch.from_numpy(np.asarray(x, dtype=np.float32)).to(torch.float8_e4m3fn).view(
        torch.uint8).numpy()


def test_decode_every_code_matches_torch():
    codes = np.arange(256, dtype=np.uint8)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).float().numpy().astype(np.float64)
    got = F.e4m3_decode(codes)
    assert np.array_equal(np.isnan(got), np.isnan(ref))
    assert np.array_equal(got[~np.isnan(got)], ref[~np.isnan(ref)])
    assert np.isnan(got[0x7F]) and np.isnan(got[0xFF]) and got[0x7E] == 448.0


def test_encode_matches_torch_including_ties():
    rng = np.random.default_rng(1)
    x = rng.uniform(-448, 448, 4000).astype(np.float32).astype(np.float64)
    small = (rng.uniform(-1, 1, 2000) * 2.0 ** rng.integers(-12, 0, 2000)).astype(np.float32)
    vals = np.sort(F.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    ties = (vals[:-1] + vals[1:]) / 2  # exact midpoints: round half to the even code
    for arr in (x, small.astype(np.float64), ties, -ties):
        assert np.array_equal(F.e4m3_encode(arr), _torch_codes(arr))


def test_encode_saturates_and_keeps_signed_zero():
    assert list(F.e4m3_encode([500.0, 1e9, -1e9, 0.0, -0.0])) == [0x7E, 0x7E, 0xFE, 0x00, 0x80]


def test_codes_of_representable_values_round_trip():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(F.e4m3_encode(F.e4m3_decode(codes)), codes)


def test_golden_example():
    g = json.load(open(GOLDEN))
    latent = np.zeros(512)
    for b, blk in enumerate(g["blocks"]):
        latent[128 * b:128 * b + len(blk["values"])] = blk["values"]
    codes, scales = F.quantize_latent(latent)
    for b, blk in enumerate(g["blocks"]):
        assert scales[b] == blk["scale"], b
        n = len(blk["codes"])
        assert list(codes[128 * b:128 * b + n]) == blk["codes"], b
        assert not codes[128 * b + n:128 * (b + 1)].any(), b


def test_scale_is_the_smallest_power_of_two():
    rng = np.random.default_rng(2)
    for _ in range(300):
        blk = rng.standard_normal(128) * 2.0 ** rng.integers(-30, 30)
        s = F.block_scale(blk)
        amax = np.max(np.abs(blk))
        k = math.log2(s)
        assert k == int(k)
        assert amax <= 448 * s and amax > 224 * s  # one binade lower would overflow 448
    # an exact boundary: max = 448 * 2^k uses 2^k, not 2^(k+1)
    assert F.block_scale([448 * 2.0 ** -5]) == 2.0 ** -5


def test_round_trip_error_bound():
    """|x - deq(q(x))| <= 2^-4 |x| in the normal range (half an ulp of 3 mantissa bits), and
    <= s 2^-10 below it (half a subnormal step of 2^-9)."""
    rng = np.random.default_rng(3)
    lat = rng.standard_normal((64, 512)) * np.exp(rng.uniform(-8, 8, (64, 1)))
    lat[3, :128] = 0.0
    codes, scales = F.quantize_latent(lat)
    deq = F.dequantize_latent(codes, scales)
    s = np.repeat(scales, 128, axis=-1)
    bound = np.maximum(2.0 ** -4 * np.abs(lat), s * 2.0 ** -10)
    assert np.all(np.abs(lat - deq) <= bound)
    assert np.all(deq[3, :128] == 0.0) and np.all(scales[3, 0] == 1.0)


def test_values_the_format_holds_are_exact():
    """A latent made of E4M3 values times a power of two per block comes back unchanged."""
    rng = np.random.default_rng(4)
    codes = rng.integers(0, 0x7F, (8, 512)).astype(np.uint8) | (rng.integers(0, 2, (8, 512)) << 7).astype(np.uint8)
    codes[:, ::128] = 0x7E  # each block reaches 448, so the scale is the chosen power
    scales = 2.0 ** rng.integers(-20, 20, (8, 4))
    x = F.dequantize_latent(codes, scales)
    c2, s2 = F.quantize_latent(x)
    assert np.array_equal(s2, scales)
    assert np.array_equal(F.dequantize_latent(c2, s2), x)


def test_row_layout():
    rng = np.random.default_rng(5)
    rows = rng.standard_normal((3, 576))
    rows[:, 512:] = torch.from_numpy(rows[:, 512:]).to(torch.bfloat16).double().numpy()
    packed = F.quantize_rows(rows)
    assert packed.shape == (3, 656) and F.ROW_BYTES == 656
    codes, rope, scales = F.unpack_rows(packed)
    assert np.array_equal(rope, rows[:, 512:])
    c2, s2 = F.quantize_latent(rows[:, :512])
    assert np.array_equal(codes, c2) and np.array_equal(scales, s2)
    # k^R bytes are little-endian bf16: the high half of the fp32 pattern
    hi = np.frombuffer(np.float32(rows[0, 512]).tobytes(), dtype=np.uint8)[2:]
    assert np.array_equal(packed[0, 512:514], hi)
    # the scales are the last 16 bytes, fp32
    assert np.array_equal(np.frombuffer(packed[1, 640:656].tobytes(), dtype="<f4"), s2[1])
    assert np.array_equal(F.dequantize_rows(packed)[:, 512:], rows[:, 512:])
