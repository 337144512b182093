"""fp8 latent cache: quantisation, dequantisation and row layout — fp64 CPU oracle.

TEST INFRASTRUCTURE ONLY, like the rest of this package: only the test suite, the smoke
check and the benchmark's CPU-baseline leg may import it.  It shares no code, table or
constant generator with the HIP library.

The pages name quantisation of the KV cache as a technique that combines with MLA's
smaller cache ([kasblo] "GQA・量子化・FlashAttentionとは何が違うのか", the row on KV cache
quantisation; [explainer] "実装のポイント（Implementation）", combining with quantisation)
but fix no format.  The format below is this repository's reading, chosen so that
dequantisation is exact in bf16 and the attention over the dequantised rows is the plain
definition of the bf16 path:

  * One cached token is a 656-byte row:
      bytes   0 .. 511  the latent c^KV (512 values) as OCP FP8 E4M3 codes
                        (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits;
                        subnormals; no infinities; S.1111.111 is NaN; largest 448);
      bytes 512 .. 639  the rotated k^R (64 values) in bf16, unquantised;
      bytes 640 .. 655  four fp32 scales, one per 128-value block of the latent.
  * Block b of the latent is stored as codes of x / s_b with s_b = 2^k, k the smallest
    integer with max|x| <= 448 * 2^k (s_b = 1 for an all-zero block); each code is the
    E4M3 value nearest to x / s_b, ties to the even code, values past 448 saturating.
  * Dequantisation: x' = value(code) * s_b, exact in fp32 and bf16 (a power-of-two
    multiple of a 4-significant-bit value).
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64
E4M3_MAX = 448.0
LATENT = 512
ROPE = 64
BLOCK = 128
ROW_BYTES = LATENT + 2 * ROPE + 4 * (LATENT // BLOCK)  # 656


def e4m3_value(code: int) -> float:
    """The value of one E4M3 code, from the bit fields."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    m = code & 0x7
    if e == 0xF and m == 0x7:
        return math.nan
    if e == 0:  # subnormal: m/8 * 2^(1 - 7)
        return sign * (m / 8.0) * 2.0 ** -6
    return sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)


def e4m3_decode(codes) -> np.ndarray:
    """Values of E4M3 codes: e4m3_value looked up per code."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([e4m3_value(c) for c in range(256)], dtype=F64)
    return table[codes]


def e4m3_encode(x) -> np.ndarray:
    """Nearest E4M3 code to each value (ties to the even code), magnitudes past 448
    saturating to +-448, NaN to 0x7F.  The two grid neighbours of |x| among the 127
    non-negative finite values (codes 0x00 .. 0x7E, increasing with the code) are compared."""
    grid = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    x = np.asarray(x, dtype=F64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    a = np.where(np.isnan(x), 0.0, a)
    hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 0x7E)  # first grid value >= a
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - grid[lo], grid[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(0x7F), code).astype(np.uint8)


def block_scale(block) -> float:
    """s = 2^k with k the smallest integer such that max|x| <= 448 * 2^k (1 for zeros)."""
    amax = float(np.max(np.abs(np.asarray(block, dtype=F64))))
    if amax == 0.0:
        return 1.0
    k = math.ceil(math.log2(amax / E4M3_MAX))
    while amax > E4M3_MAX * 2.0 ** k:  # exact comparisons settle any log2 rounding
        k += 1
    while amax <= E4M3_MAX * 2.0 ** (k - 1):
        k -= 1
    return 2.0 ** k


def quantize_latent(latent):
    """latent [..., 512] -> (codes [..., 512] uint8, scales [..., 4] float64)."""
    latent = np.asarray(latent, dtype=F64)
    lead = latent.shape[:-1]
    blocks = latent.reshape(lead + (LATENT // BLOCK, BLOCK))
    scales = np.empty(lead + (LATENT // BLOCK,), dtype=F64)
    for idx in np.ndindex(*blocks.shape[:-1]):
        scales[idx] = block_scale(blocks[idx])
    codes = e4m3_encode(blocks / scales[..., None])
    return codes.reshape(lead + (LATENT,)), scales


def dequantize_latent(codes, scales) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8)
    lead = codes.shape[:-1]
    vals = e4m3_decode(codes).reshape(lead + (LATENT // BLOCK, BLOCK))
    return (vals * np.asarray(scales, dtype=F64)[..., None]).reshape(lead + (LATENT,))


def _bf16_bits(values) -> np.ndarray:
    """bf16 bit patterns of values that bf16 holds exactly (the stored k^R)."""
    f32 = np.asarray(values, dtype=np.float32)
    assert np.array_equal(f32.astype(F64), np.asarray(values, dtype=F64)), "value not exact in fp32"
    bits = f32.view(np.uint32)
    assert np.all(bits & 0xFFFF == 0), "value not exact in bf16"
    return (bits >> 16).astype(np.uint16)


def pack_rows(codes, rope_values, scales) -> np.ndarray:
    """Rows of 656 bytes: codes, k^R as little-endian bf16 (exact values), fp32 scales."""
    codes = np.asarray(codes, dtype=np.uint8)
    lead = codes.shape[:-1]
    out = np.zeros(lead + (ROW_BYTES,), dtype=np.uint8)
    out[..., :LATENT] = codes
    out[..., LATENT:LATENT + 2 * ROPE] = _bf16_bits(rope_values).astype("<u2").view(np.uint8).reshape(
        lead + (2 * ROPE,))
    out[..., LATENT + 2 * ROPE:] = np.asarray(scales, dtype="<f4").view(np.uint8).reshape(
        lead + (4 * (LATENT // BLOCK),))
    return out


def unpack_rows(rows):
    """656-byte rows -> (codes, k^R values, scales) with the values in float64."""
    rows = np.asarray(rows, dtype=np.uint8)
    codes = rows[..., :LATENT]
    rope_bits = np.ascontiguousarray(rows[..., LATENT:LATENT + 2 * ROPE]).view("<u2").astype(np.uint32)
    rope = (rope_bits << 16).view(np.float32).astype(F64)
    scales = np.ascontiguousarray(rows[..., LATENT + 2 * ROPE:]).view("<f4").astype(F64)
    return codes, rope, scales


def quantize_rows(rows576) -> np.ndarray:
    """Cache rows [..., 576] (latent then k^R; k^R exact in bf16) -> fp8 rows [..., 656]."""
    rows576 = np.asarray(rows576, dtype=F64)
    codes, scales = quantize_latent(rows576[..., :LATENT])
    return pack_rows(codes, rows576[..., LATENT:], scales)


def dequantize_rows(rows656) -> np.ndarray:
    """fp8 rows [..., 656] -> the values they stand for, [..., 576] float64."""
    codes, rope, scales = unpack_rows(rows656)
    return np.concatenate([dequantize_latent(codes, scales), rope], axis=-1)
