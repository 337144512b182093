"""Planted mistakes in the oracle must be caught by its pins (CPU only).

Each mutant swaps one oracle building block for a plausibly wrong variant (a sign, an
index, a transposed operand, a dropped term) and re-runs the pin tests; at least one
pin has to fail.  The mutants live only inside this test and are undone afterwards.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import mla_oracle as M
from tests import test_oracle_pins as pins

PIN_TESTS = [
    pins.test_worked_example_both_orders,
    lambda: pins.test_rope_first_pair_is_plain_rotation(2.5),
    pins.test_rope_frequency_ladder,
    pins.test_rope_invariants,
    pins.test_expanded_matches_library_sdpa,
    pins.test_latent_attention_is_mqa_sdpa,
    pins.test_softmax_weights_sum_to_one,
    pins.test_single_token_returns_its_value,
    pins.test_zero_query_gives_mean,
    lambda: pins.test_absorbed_equals_expanded(0),
    pins.test_head_blocks_are_row_blocks,
    pins.test_combine_equals_unsplit,
    pins.test_combine_closed_form,
    pins.test_page_slot_example,
    pins.test_gather_permuted_pool_equals_contiguous,
    pins.test_append_then_gather,
    pins.test_paged_decode_matches_per_sequence_sdpa,
    pins.test_multi_token_decode_is_causal_sdpa,
    pins.test_multi_token_decode_reduces_to_single,
    pins.test_layer_single_token_closed_form,
    pins.test_layer_matches_sdpa_composition,
    pins.test_cache_sizes_from_pages,
    pins.test_default_scale,
    pins.test_causal_attention_is_masked_sdpa,
    pins.test_expanded_prefill_rows_are_decodes,
]


def _rope_clockwise(x, pos, base=10000.0):
    return M_rope_orig(x, -np.asarray(pos, dtype=float), base)


def _rope_wrong_freq(x, pos, base=10000.0):
    x = np.asarray(x, float)
    d = x.shape[-1]
    k = np.arange(d // 2)
    ang = np.asarray(pos, float)[..., None] * float(base) ** (-k / d)
    c, s = np.cos(ang), np.sin(ang)
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)))
    out[..., 0::2] = x[..., 0::2] * c - x[..., 1::2] * s
    out[..., 1::2] = x[..., 0::2] * s + x[..., 1::2] * c
    return out


def _rope_half_split(x, pos, base=10000.0):
    """rotate-half pairing (i, i + d/2) instead of adjacent pairs"""
    x = np.asarray(x, float)
    d = x.shape[-1]
    perm = np.concatenate([np.arange(0, d, 2), np.arange(1, d, 2)])
    inv = np.argsort(perm)
    y = M_rope_orig(x[..., inv], pos, base)
    return y[..., perm]


def _head_block_interleaved(w, i, d_h):
    w = np.asarray(w, float)
    H = w.shape[0] // d_h
    return w[i::H, :]


def _softmax_no_norm(s, axis=-1):
    s = np.asarray(s, float)
    return np.exp(s - np.max(s, axis=axis, keepdims=True))


def _softmax_wrong_axis(s, axis=-1):
    return M_softmax_orig(s, axis=0)


def _page_slot_swapped(row, pos, P):
    return int(row[pos % P]), pos // P


def _combine_no_shift(o_parts, lse_parts):
    o_parts, lse_parts = np.asarray(o_parts, float), np.asarray(lse_parts, float)
    w = np.where(np.isfinite(lse_parts), lse_parts, 0.0)
    den = np.sum(w, axis=0)
    den_safe = np.where(den != 0, den, 1.0)
    return np.sum(w[..., None] * o_parts, axis=0) / den_safe[..., None], np.log(np.abs(den_safe))


def _cache_bytes_kv_twice(B, T, L, d_c, d_R, s):
    return B * T * L * (2 * d_c + d_R) * s


def _logsumexp_log2(s, axis=-1):
    return M_lse_orig(s, axis) / math.log(2)


def _absorb_no_transpose(q_c, w_uk):
    # uses the column block of W^UK^T instead of the row block's transpose
    q_c = np.asarray(q_c, float)
    H, d_h = q_c.shape[-2], q_c.shape[-1]
    w = np.asarray(w_uk, float)
    out = np.empty(q_c.shape[:-1] + (w.shape[1],))
    for i in range(H):
        blk = w[i * d_h:(i + 1) * d_h, :]
        out[..., i, :] = (q_c[..., i, :][..., ::-1]) @ blk
    return out


def _multi_decode(visible_of):
    """paged_decode_multi with another rule for the tokens a query sees"""
    def f(q_lat, q_pe, cache, block_table, seq_lens, n_q, d_c, scale):
        q_lat, q_pe = np.asarray(q_lat, float), np.asarray(q_pe, float)
        B, _, H, _ = q_lat.shape
        P = np.asarray(cache).shape[1]
        o = np.zeros((B, n_q, H, d_c))
        lse = np.full((B, n_q, H), -np.inf)
        for b in range(B):
            for t in range(n_q):
                v = visible_of(int(seq_lens[b]), n_q, t)
                if v <= 0:
                    continue
                att = M.latent_attention(q_lat[b, t], q_pe[b, t],
                                         M.gather_rows(cache, block_table[b], v, P), d_c, scale)
                o[b, t], lse[b, t] = att["o_lat"], att["lse"]
        return o, lse
    return f


M_rope_orig = M.rope
M_softmax_orig = M.softmax
M_lse_orig = M.logsumexp

M_causal_orig = M.causal_attention


def _causal_misses_itself(q, k, v, scale):
    """each query sees only the tokens strictly before it (and the first one itself)"""
    q, k, v = (np.asarray(a, float) for a in (q, k, v))
    T, H, _ = q.shape
    o = np.empty((T, H, v.shape[-1]))
    lse = np.empty((T, H))
    vis = np.tril(np.ones((T, T), dtype=bool), -1)
    vis[0, 0] = True
    for i in range(H):
        s = np.where(vis, (q[:, i] @ k[:, i].T) * scale, -np.inf)
        o[:, i] = M.softmax(s, axis=-1) @ v[:, i]
        lse[:, i] = M.logsumexp(s, axis=-1)
    return o, lse


def _causal_future(q, k, v, scale):
    """mask transposed: each query sees the tokens at and after it"""
    o, lse = M_causal_orig(np.asarray(q)[::-1], np.asarray(k)[::-1], np.asarray(v)[::-1], scale)
    return o[::-1], lse[::-1]


MUTANTS = {
    "rope_clockwise": ("rope", _rope_clockwise),
    "rope_wrong_frequency": ("rope", _rope_wrong_freq),
    "rope_rotate_half_pairs": ("rope", _rope_half_split),
    "head_block_interleaved": ("head_block", _head_block_interleaved),
    "softmax_unnormalised": ("softmax", _softmax_no_norm),
    "softmax_wrong_axis": ("softmax", _softmax_wrong_axis),
    "page_slot_swapped": ("page_slot", _page_slot_swapped),
    "combine_linear_weights": ("combine_splits", _combine_no_shift),
    "cache_bytes_k_and_v": ("cache_bytes", _cache_bytes_kv_twice),
    "lse_in_log2": ("logsumexp", _logsumexp_log2),
    "absorb_reversed_index": ("absorb_query", _absorb_no_transpose),
    "multi_query_misses_itself": ("paged_decode_multi", _multi_decode(lambda L, n, t: L - n + t)),
    "multi_query_not_causal": ("paged_decode_multi", _multi_decode(lambda L, n, t: L)),
    "multi_query_tokens_reversed": ("paged_decode_multi",
                                    _multi_decode(lambda L, n, t: L - t)),
    "causal_misses_itself": ("causal_attention", _causal_misses_itself),
    "causal_sees_future": ("causal_attention", _causal_future),
}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_mutant_is_caught(name, monkeypatch):
    attr, fn = MUTANTS[name]
    monkeypatch.setattr(M, attr, fn)
    monkeypatch.setattr(oracle, attr, fn)
    failures = 0
    for t in PIN_TESTS:
        try:
            t()
        except Exception:  # an assertion or a shape error: the pin noticed
            failures += 1
    assert failures > 0, f"planted mistake {name} passed every pin"


# ---- the fp8 latent-cache oracle ------------------------------------------------------
from oracle import fp8_cache as F8  # noqa: E402
from tests import test_oracle_fp8 as fp8_pins  # noqa: E402

FP8_PIN_TESTS = [
    fp8_pins.test_decode_every_code_matches_torch,
    fp8_pins.test_encode_matches_torch_including_ties,
    fp8_pins.test_encode_saturates_and_keeps_signed_zero,
    fp8_pins.test_codes_of_representable_values_round_trip,
    fp8_pins.test_golden_example,
    fp8_pins.test_scale_is_the_smallest_power_of_two,
    fp8_pins.test_round_trip_error_bound,
    fp8_pins.test_values_the_format_holds_are_exact,
    fp8_pins.test_row_layout,
]

F8_scale_orig = F8.block_scale
F8_encode_orig = F8.e4m3_encode
F8_value_orig = F8.e4m3_value


def _scale_one_binade_high(block):
    return 2.0 * F8_scale_orig(block)


def _encode_ties_away(x):
    """round half away from zero instead of to the even code"""
    x = np.asarray(x, dtype=float)
    out = F8_encode_orig(x)
    vals = np.sort(F8.e4m3_decode(np.arange(0x7F, dtype=np.uint8)))
    mids = set(((vals[:-1] + vals[1:]) / 2).tolist())
    flat, res = x.reshape(-1), out.reshape(-1)
    for n, v in enumerate(flat):
        if abs(v) in mids:
            res[n] = F8_encode_orig(np.array([math.copysign(np.nextafter(abs(v), np.inf), v)]))[0]
    return out


def _value_bias_8(code):
    code = int(code) & 0xFF
    e, m = (code >> 3) & 0xF, code & 7
    if e == 0xF and m == 7:
        return math.nan
    sign = -1.0 if code & 0x80 else 1.0
    return sign * ((m / 8.0) * 2.0 ** -7 if e == 0 else (1 + m / 8.0) * 2.0 ** (e - 8))


def _encode_flush_subnormals(x):
    out = F8_encode_orig(x)
    out[(out & 0x78) == 0] &= 0x80
    return out


FP8_MUTANTS = {
    "fp8_scale_one_binade_high": ("block_scale", _scale_one_binade_high),
    "fp8_ties_away_from_zero": ("e4m3_encode", _encode_ties_away),
    "fp8_exponent_bias_8": ("e4m3_value", _value_bias_8),
    "fp8_flush_subnormals": ("e4m3_encode", _encode_flush_subnormals),
}


@pytest.mark.parametrize("name", sorted(FP8_MUTANTS))
def test_fp8_mutant_is_caught(name, monkeypatch):
    attr, fn = FP8_MUTANTS[name]
    monkeypatch.setattr(F8, attr, fn)
    failures = 0
    for t in FP8_PIN_TESTS:
        try:
            t()
        except Exception:
            failures += 1
    assert failures > 0, f"planted mistake {name} passed every fp8 pin"
