"""Pins of the fp64 oracle against what the pages and mathematics fix (CPU only).

Each test pins an oracle function to something other than itself: a worked example
printed on the pages, a closed form, an invariant, or a library routine that the
method reduces to in a special case (torch's scaled_dot_product_attention in fp64,
numpy's logaddexp).
"""
import json
import math
import os

import numpy as np
import pytest
import torch

import oracle

GOLD = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


# ---------------------------------------------------------------- worked example (pages)
def test_worked_example_both_orders():
    """kasblo.com/?p=4663, figure '説明用の数値例': c=(2,1), U picks c1, c2, c1+c2, q=(1,2,1).
    Expanding k=Uc then q.k, or absorbing U^T q then (U^T q).c, both give 7."""
    g = json.load(open(os.path.join(GOLD, "worked_example.json")))
    c = np.array(g["c"], float)
    U = np.array(g["U"], float)           # [d_h=3, d_c=2]: one head's W^UK block
    q = np.array(g["q"], float)
    # absorb: q~ = U^T q
    q_lat = oracle.absorb_query(q[None, :], U)
    assert q_lat.shape == (1, 2)
    assert q_lat[0].tolist() == g["UTq"]
    # expanded order: the oracle's own k^C = W^UK c, score = q . k (scale 1, no RoPE part)
    empty = np.zeros((1, 0))
    res = oracle.expanded_decode(q[None, :], empty, c[None, :], np.zeros((1, 0)), U, U, 1.0)
    assert res["scores"][0, 0] == g["score"]
    # latent order over the raw cache row
    lat = oracle.latent_attention(q_lat, empty, c[None, :], 2, 1.0)
    assert lat["scores"][0, 0] == g["score"]
    # one token: softmax weight 1, lse = the score itself
    assert res["lse"][0] == g["score"] and lat["lse"][0] == g["score"]
    assert np.array_equal(res["p"], [[1.0]])
    # k = U c printed on the page: single-token value path returns W^UV c with W^UV = U
    assert res["o"][0].tolist() == g["k"]


# ---------------------------------------------------------------- RoPE closed forms
@pytest.mark.parametrize("p", [0.0, 1.0, 2.5, -3.0, 255.0])
def test_rope_first_pair_is_plain_rotation(p):
    """theta_0 = base**0 = 1: pair (1, 0) at position p goes to (cos p, sin p) — the
    counter-clockwise rotation matrix [[cos, -sin], [sin, cos]] of RoFormer."""
    out = oracle.rope(np.array([1.0, 0.0]), p, base=10000.0)
    assert np.allclose(out, [math.cos(p), math.sin(p)], rtol=0, atol=1e-15)
    out = oracle.rope(np.array([0.0, 1.0]), p, base=10000.0)
    assert np.allclose(out, [-math.sin(p), math.cos(p)], rtol=0, atol=1e-15)


def test_rope_frequency_ladder():
    """d=4, base=100: pair k=1 has theta_1 = 100**(-2/4) = 0.1, so position 10 turns it by
    exactly 1 rad while pair 0 turns by 10 rad."""
    x = np.array([1.0, 0.0, 1.0, 0.0])
    out = oracle.rope(x, 10.0, base=100.0)
    assert np.allclose(out, [math.cos(10), math.sin(10), math.cos(1), math.sin(1)], atol=1e-14)
    # d=64, base=10000: last pair theta_31 = 10000**(-62/64)
    x = np.zeros(64)
    x[62] = 1.0
    out = oracle.rope(x, 1000.0, base=10000.0)
    a = 1000.0 * 10000.0 ** (-62 / 64)
    assert np.allclose(out[62:], [math.cos(a), math.sin(a)], atol=1e-13)
    assert np.all(out[:62] == 0)


def test_rope_invariants():
    """[kasblo] '分離したRoPE': rotation keeps norms and makes the dot product depend only
    on the relative position: <R(m)q, R(n)k> = <R(m-n)q, k>; R(0) = I; R(a)R(b) = R(a+b)."""
    r = _rng(0)
    q, k = r.standard_normal(64), r.standard_normal(64)
    assert np.allclose(oracle.rope(q, 0.0), q, atol=0)
    for m, n in [(5, 3), (4095, 17), (32767, 32000), (7, 7)]:
        lhs = oracle.rope(q, m) @ oracle.rope(k, n)
        rhs = oracle.rope(q, m - n) @ k
        assert abs(lhs - rhs) < 1e-9 * (1 + abs(rhs))
        assert abs(np.linalg.norm(oracle.rope(q, m)) - np.linalg.norm(q)) < 1e-12
    assert np.allclose(oracle.rope(oracle.rope(q, 11.0), 30.0), oracle.rope(q, 41.0), atol=1e-12)


# ---------------------------------------------------------------- softmax attention
def _sdpa(q, k, v, scale):
    """torch SDPA in fp64 on the CPU.  q [H, 1, E], k [H, T, E], v [H, T, Ev]."""
    return torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None], torch.from_numpy(k)[None], torch.from_numpy(v)[None],
        scale=scale)[0].numpy()


def _tiny_expanded_inputs(seed, H=3, d_h=5, d_c=7, d_R=4, T=9):
    r = _rng(seed)
    return dict(q_c=r.standard_normal((H, d_h)), q_pe=r.standard_normal((H, d_R)),
                c_kv=r.standard_normal((T, d_c)), k_pe=r.standard_normal((T, d_R)),
                w_uk=r.standard_normal((H * d_h, d_c)) / 3, w_uv=r.standard_normal((H * d_h, d_c)) / 3,
                w_o=r.standard_normal((11, H * d_h)))


def test_expanded_matches_library_sdpa():
    """The expanded path equals standard scaled dot-product attention over the restored
    per-head keys [W^UK_i c_j ; k^R_j] and values W^UV_i c_j, scale 1/sqrt(d_h + d_R)
    ([qiita] 'Attention 計算').  Keys/values built here with plain matmuls."""
    x = _tiny_expanded_inputs(1)
    H, d_h = x["q_c"].shape
    T = x["c_kv"].shape[0]
    scale = 1 / math.sqrt(d_h + x["q_pe"].shape[1])
    q = np.concatenate([x["q_c"], x["q_pe"]], 1)[:, None, :]
    k = np.stack([np.concatenate([x["c_kv"] @ x["w_uk"][i * d_h:(i + 1) * d_h].T, x["k_pe"]], 1)
                  for i in range(H)])
    v = np.stack([x["c_kv"] @ x["w_uv"][i * d_h:(i + 1) * d_h].T for i in range(H)])
    ref = _sdpa(q, k, v, scale)[:, 0]
    res = oracle.expanded_decode(x["q_c"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_uk"], x["w_uv"],
                                 scale, x["w_o"])
    assert np.allclose(res["o"], ref, rtol=0, atol=1e-13)
    assert np.allclose(res["u"], x["w_o"] @ ref.reshape(-1), rtol=0, atol=1e-12)
    assert res["p"].shape == (H, T)


def test_latent_attention_is_mqa_sdpa():
    """Latent attention is MQA with one KV stream: key = whole 576-style row, value =
    its first d_c entries; compare with torch SDPA (fp64)."""
    r = _rng(2)
    H, d_c, d_R, T = 6, 16, 4, 37
    q_lat, q_pe = r.standard_normal((H, d_c)), r.standard_normal((H, d_R))
    rows = r.standard_normal((T, d_c + d_R))
    scale = 0.3
    res = oracle.latent_attention(q_lat, q_pe, rows, d_c, scale)
    q = np.concatenate([q_lat, q_pe], 1)[:, None, :]
    k = np.broadcast_to(rows, (H, T, d_c + d_R)).copy()
    v = np.broadcast_to(rows[:, :d_c], (H, T, d_c)).copy()
    assert np.allclose(res["o_lat"], _sdpa(q, k, v, scale)[:, 0], rtol=0, atol=1e-13)
    # lse against numpy's logaddexp.reduce of the scaled scores
    s = (q[:, 0] @ rows.T) * scale
    assert np.allclose(res["lse"], np.logaddexp.reduce(s, axis=1), rtol=0, atol=1e-12)


def test_softmax_weights_sum_to_one():
    """[kasblo]: Softmax turns the scores into weights whose sum is 1."""
    x = _tiny_expanded_inputs(3, T=50)
    res = oracle.expanded_decode(x["q_c"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_uk"], x["w_uv"], 0.4)
    assert np.all(res["p"] >= 0)
    assert np.allclose(res["p"].sum(1), 1.0, rtol=0, atol=1e-14)
    huge = oracle.softmax(np.array([1000.0, 999.0, -1e4]))
    assert np.isfinite(huge).all() and abs(huge.sum() - 1) < 1e-15


def test_single_token_returns_its_value():
    """With one cached token the softmax weight is 1, so o_i = W^UV_i c_0 and the latent
    output is c_0 itself."""
    x = _tiny_expanded_inputs(4, T=1)
    H, d_h = x["q_c"].shape
    res = oracle.expanded_decode(x["q_c"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_uk"], x["w_uv"], 0.7)
    for i in range(H):
        assert np.array_equal(res["o"][i], x["w_uv"][i * d_h:(i + 1) * d_h] @ x["c_kv"][0])
    rows = np.concatenate([x["c_kv"], x["k_pe"]], 1)
    lat = oracle.latent_attention(np.ones((H, 7)), np.ones((H, 4)), rows, 7, 0.7)
    assert np.array_equal(lat["o_lat"], np.broadcast_to(x["c_kv"][0], (H, 7)))


def test_zero_query_gives_mean():
    """q = 0 makes every score 0, so p = 1/T and o~ is the mean of the latents."""
    r = _rng(5)
    rows = r.standard_normal((64, 10))
    lat = oracle.latent_attention(np.zeros((2, 8)), np.zeros((2, 2)), rows, 8, 1.0)
    assert np.allclose(lat["o_lat"], rows[:, :8].mean(0), atol=1e-15)
    assert np.allclose(lat["lse"], math.log(64), atol=1e-15)


def test_empty_context_defined():
    lat = oracle.latent_attention(np.ones((3, 4)), np.ones((3, 2)), np.zeros((0, 6)), 4, 1.0)
    assert np.all(lat["o_lat"] == 0) and np.all(lat["lse"] == -np.inf)


# ---------------------------------------------------------------- absorption identity
@pytest.mark.parametrize("seed", [0, 1, 2])
def test_absorbed_equals_expanded(seed):
    """[explainer] '行列吸収トリック' / [kasblo] K side and V side: moving W^UK onto the
    query and W^UV after the weighted sum changes nothing in exact arithmetic."""
    x = _tiny_expanded_inputs(10 + seed, H=4, d_h=6, d_c=9, d_R=4, T=23)
    a = oracle.expanded_decode(x["q_c"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_uk"], x["w_uv"],
                               0.25, x["w_o"])
    b = oracle.absorbed_decode(x["q_c"], x["q_pe"], x["c_kv"], x["k_pe"], x["w_uk"], x["w_uv"],
                               0.25, x["w_o"])
    assert np.max(np.abs(a["o"] - b["o"])) <= 1e-12
    assert np.max(np.abs(a["u"] - b["u"])) <= 1e-12
    assert np.max(np.abs(a["lse"] - b["lse"])) <= 1e-12


def test_head_blocks_are_row_blocks():
    """Head i of an [n_h*d_h, d_c] weight is its i-th row block (nn.Linear layout):
    with a weight whose head-1 block is the identity and the rest zero, only head 1's
    absorbed query is non-zero and equals q^C_1 itself (d_h = d_c)."""
    H, d = 3, 4
    w = np.zeros((H * d, d))
    w[d:2 * d] = np.eye(d)
    q = np.arange(H * d, dtype=float).reshape(H, d) + 1
    out = oracle.absorb_query(q, w)
    assert np.all(out[0] == 0) and np.all(out[2] == 0)
    assert np.array_equal(out[1], q[1])
    o = oracle.up_project_values(q, w)
    assert np.array_equal(o[1], q[1]) and np.all(o[0] == 0)


# ---------------------------------------------------------------- split + combine
def test_combine_equals_unsplit():
    """Softmax over disjoint token ranges merged by log-sum-exp equals the full softmax
    (the denominator is a sum over j)."""
    r = _rng(6)
    H, d_c, d_R, T = 5, 12, 4, 100
    q_lat, q_pe = r.standard_normal((H, d_c)), r.standard_normal((H, d_R))
    rows = r.standard_normal((T, d_c + d_R))
    full = oracle.latent_attention(q_lat, q_pe, rows, d_c, 0.5)
    cuts = [0, 13, 13, 60, 100, 100]           # includes two empty splits
    parts = [oracle.latent_attention(q_lat, q_pe, rows[a:b], d_c, 0.5) for a, b in zip(cuts, cuts[1:])]
    o, lse = oracle.combine_splits([p["o_lat"] for p in parts], [p["lse"] for p in parts])
    assert np.allclose(o, full["o_lat"], rtol=0, atol=1e-14)
    assert np.allclose(lse, full["lse"], rtol=0, atol=1e-13)


def test_combine_closed_form():
    """Two splits with lse a, b: weights e^a, e^b; merged lse = logaddexp(a, b)."""
    o1, o2 = np.array([[1.0, 0.0]]), np.array([[0.0, 1.0]])
    a, b = np.array([0.3]), np.array([2.0])
    o, lse = oracle.combine_splits([o1, o2], [a, b])
    wa = math.exp(0.3) / (math.exp(0.3) + math.exp(2.0))
    assert np.allclose(o, [[wa, 1 - wa]], atol=1e-15)
    assert np.allclose(lse, np.logaddexp(a, b), atol=1e-15)
    o, lse = oracle.combine_splits([o1, o2], [np.array([-np.inf]), np.array([-np.inf])])
    assert np.all(o == 0) and np.all(lse == -np.inf)


# ---------------------------------------------------------------- paged addressing
def test_page_slot_example():
    """Token j of a sequence lives at page block_table[j // P], slot j % P."""
    assert oracle.page_slot([5, 2, 9], 0, 4) == (5, 0)
    assert oracle.page_slot([5, 2, 9], 5, 4) == (2, 1)
    assert oracle.page_slot([5, 2, 9], 11, 4) == (9, 3)


def test_gather_permuted_pool_equals_contiguous():
    r = _rng(7)
    P, T, W = 4, 10, 3
    rows = r.standard_normal((T, W))
    perm = np.array([4, 0, 2])                 # logical page p -> physical page perm[p]
    pool = np.full((6, P, W), np.nan)
    for j in range(T):
        pool[perm[j // P], j % P] = rows[j]
    assert np.array_equal(oracle.gather_rows(pool, perm, T, P), rows)


def test_append_then_gather():
    """Appending rows writes [c ; RoPE(k, pos)] at the token's page/slot and nothing else."""
    r = _rng(8)
    P, d_c, d_R = 4, 3, 2
    pool = np.full((5, P, d_c + d_R), 7.0)
    bt = np.array([[3, 1, 0], [4, 2, -1]])
    before = [5, 2]
    c_new, k_new = r.standard_normal((2, 2, d_c)), r.standard_normal((2, 2, d_R))
    out = oracle.append_rows(pool, bt, before, c_new, k_new, 10000.0)
    # sequence 0: positions 5, 6 -> page 1 slots 1, 2 ; sequence 1: positions 2, 3 -> page 4 slots 2, 3
    assert np.array_equal(out[1, 1, :d_c], c_new[0, 0]) and np.array_equal(out[1, 2, :d_c], c_new[0, 1])
    assert np.array_equal(out[4, 2, :d_c], c_new[1, 0]) and np.array_equal(out[4, 3, :d_c], c_new[1, 1])
    assert np.allclose(out[1, 1, d_c:], oracle.rope(k_new[0, 0], 5))
    assert np.allclose(out[4, 3, d_c:], oracle.rope(k_new[1, 1], 3))
    touched = np.zeros(out.shape[:2], bool)
    touched[1, 1] = touched[1, 2] = touched[4, 2] = touched[4, 3] = True
    assert np.all(out[~touched] == 7.0)


def test_paged_decode_matches_per_sequence_sdpa():
    r = _rng(9)
    P, d_c, d_R, H = 4, 6, 2, 3
    seq_lens = [5, 1, 8]
    pool = r.standard_normal((7, P, d_c + d_R))
    bt = np.array([[6, 1, -1], [3, -1, -1], [0, 5, -1]])
    q_lat, q_pe = r.standard_normal((3, H, d_c)), r.standard_normal((3, H, d_R))
    o, lse = oracle.paged_decode(q_lat, q_pe, pool, bt, seq_lens, d_c, 0.6)
    for b, L in enumerate(seq_lens):
        rows = np.concatenate([pool[bt[b, j // P], j % P][None] for j in range(L)])
        q = np.concatenate([q_lat[b], q_pe[b]], 1)[:, None]
        ref = _sdpa(q, np.broadcast_to(rows, (H, L, d_c + d_R)).copy(),
                    np.broadcast_to(rows[:, :d_c], (H, L, d_c)).copy(), 0.6)[:, 0]
        assert np.allclose(o[b], ref, atol=1e-13)


def test_multi_token_decode_is_causal_sdpa():
    """n_q new tokens per sequence: torch SDPA in fp64 with a boolean mask that lets query t
    see the cached tokens up to its own position (seq_len - n_q + t), over the gathered
    paged rows; pages permuted, one sequence shorter than n_q (its first query sees
    nothing: o = 0, lse = -inf)."""
    r = _rng(12)
    P, d_c, d_R, H, n_q = 4, 6, 2, 3, 3
    seq_lens = [7, 3, 2]
    pool = r.standard_normal((6, P, d_c + d_R))
    bt = np.array([[4, 0], [5, -1], [2, -1]])
    q_lat, q_pe = r.standard_normal((3, n_q, H, d_c)), r.standard_normal((3, n_q, H, d_R))
    o, lse = oracle.paged_decode_multi(q_lat, q_pe, pool, bt, seq_lens, n_q, d_c, 0.45)
    for b, L in enumerate(seq_lens):
        rows = np.concatenate([pool[bt[b, j // P], j % P][None] for j in range(L)])
        for t in range(n_q):
            pos = L - n_q + t
            if pos < 0:
                assert np.all(o[b, t] == 0) and np.all(lse[b, t] == -np.inf)
                continue
            q = torch.from_numpy(np.concatenate([q_lat[b, t], q_pe[b, t]], 1)[:, None])[None]
            k = torch.from_numpy(np.broadcast_to(rows, (H, L, d_c + d_R)).copy())[None]
            v = torch.from_numpy(np.broadcast_to(rows[:, :d_c], (H, L, d_c)).copy())[None]
            mask = torch.arange(L)[None, :] <= pos          # [1, L]: keys up to the query
            ref = torch.nn.functional.scaled_dot_product_attention(
                q, k, v, attn_mask=mask, scale=0.45)[0, :, 0].numpy()
            assert np.allclose(o[b, t], ref, rtol=0, atol=1e-13), (b, t)


def test_multi_token_decode_reduces_to_single():
    """n_q = 1 is paged_decode; the last of n_q tokens sees the whole sequence, so it equals
    paged_decode at the same lengths exactly; rows past a query's position do not change it."""
    r = _rng(13)
    P, d_c, d_R, H = 4, 5, 2, 2
    seq_lens = [9, 6]
    pool = r.standard_normal((6, P, d_c + d_R))
    bt = np.array([[3, 0, 5], [1, 4, -1]])
    q1, p1 = r.standard_normal((2, 1, H, d_c)), r.standard_normal((2, 1, H, d_R))
    o1, l1 = oracle.paged_decode_multi(q1, p1, pool, bt, seq_lens, 1, d_c, 0.5)
    o_ref, l_ref = oracle.paged_decode(q1[:, 0], p1[:, 0], pool, bt, seq_lens, d_c, 0.5)
    assert np.array_equal(o1[:, 0], o_ref) and np.array_equal(l1[:, 0], l_ref)
    n_q = 4
    q4, p4 = r.standard_normal((2, n_q, H, d_c)), r.standard_normal((2, n_q, H, d_R))
    o4, l4 = oracle.paged_decode_multi(q4, p4, pool, bt, seq_lens, n_q, d_c, 0.5)
    o_last, l_last = oracle.paged_decode(q4[:, -1], p4[:, -1], pool, bt, seq_lens, d_c, 0.5)
    assert np.array_equal(o4[:, -1], o_last) and np.array_equal(l4[:, -1], l_last)
    # overwrite the last cached token of sequence 0: only its last query may change
    pool2 = pool.copy()
    j = seq_lens[0] - 1
    pool2[bt[0, j // P], j % P] = r.standard_normal(d_c + d_R) * 5
    o5, _ = oracle.paged_decode_multi(q4, p4, pool2, bt, seq_lens, n_q, d_c, 0.5)
    assert np.array_equal(o5[0, :-1], o4[0, :-1]) and not np.allclose(o5[0, -1], o4[0, -1])
    assert np.array_equal(o5[1], o4[1])


# ---------------------------------------------------------------- full layer
def _tiny_layer(seed, B=2, d=12, H=2, d_h=3, d_c=5, d_cq=4, d_R=2, T=6, P=4):
    r = _rng(seed)
    w = {"w_dq": r.standard_normal((d_cq, d)), "w_uq": r.standard_normal((H * d_h, d_cq)),
         "w_qr": r.standard_normal((H * d_R, d_cq)), "w_dkv": r.standard_normal((d_c, d)),
         "w_kr": r.standard_normal((d_R, d)), "w_uk": r.standard_normal((H * d_h, d_c)),
         "w_uv": r.standard_normal((H * d_h, d_c)), "w_o": r.standard_normal((d, H * d_h))}
    w = {k: v / math.sqrt(v.shape[1]) for k, v in w.items()}
    pp = math.ceil((T + 1) / P)
    pool = r.standard_normal((B * pp, P, d_c + d_R))
    bt = np.arange(B * pp).reshape(B, pp)
    h = r.standard_normal((B, d))
    return h, w, pool, bt, [T] * B, dict(d_h=d_h, d_R=d_R, d_c=d_c, H=H, P=P)


def test_layer_single_token_closed_form():
    """Empty prior cache: the only key is the new token itself, its weight is 1, so
    u = W^O [W^UV_1 c; ...; W^UV_H c] with c = W^DKV h (plain matrix products)."""
    h, w, pool, bt, _, s = _tiny_layer(11)
    res = oracle.decode_layer(h, w, pool, bt, [0, 0], s["d_h"], s["d_R"], 10000.0, 0.5)
    for b in range(h.shape[0]):
        c = w["w_dkv"] @ h[b]
        o = np.concatenate([w["w_uv"][i * s["d_h"]:(i + 1) * s["d_h"]] @ c for i in range(s["H"])])
        assert np.allclose(res["u"][b], w["w_o"] @ o, atol=1e-13)


def test_layer_matches_sdpa_composition():
    """Full layer vs an independent composition: projections by plain matmuls, RoPE from
    the pinned oracle rope, attention from torch SDPA (fp64)."""
    h, w, pool, bt, before, s = _tiny_layer(12)
    d_h, d_R, H, P, d_c = s["d_h"], s["d_R"], s["H"], s["P"], s["d_c"]
    scale = 1 / math.sqrt(d_h + d_R)
    res = oracle.decode_layer(h, w, pool, bt, before, d_h, d_R, 10000.0, scale)
    for b in range(h.shape[0]):
        T = before[b]
        cq = w["w_dq"] @ h[b]
        qc = (w["w_uq"] @ cq).reshape(H, d_h)
        qr = oracle.rope((w["w_qr"] @ cq).reshape(H, d_R), T)
        rows = [pool[bt[b, j // P], j % P] for j in range(T)]
        rows.append(np.concatenate([w["w_dkv"] @ h[b], oracle.rope(w["w_kr"] @ h[b], T)]))
        rows = np.stack(rows)
        k = np.stack([np.concatenate([rows[:, :d_c] @ w["w_uk"][i * d_h:(i + 1) * d_h].T,
                                      rows[:, d_c:]], 1) for i in range(H)])
        v = np.stack([rows[:, :d_c] @ w["w_uv"][i * d_h:(i + 1) * d_h].T for i in range(H)])
        q = np.concatenate([qc, qr], 1)[:, None]
        o = _sdpa(q, k, v, scale)[:, 0]
        assert np.allclose(res["u"][b], w["w_o"] @ o.reshape(-1), atol=1e-12)


# ---------------------------------------------------------------- cache arithmetic (pages)
def test_cache_sizes_from_pages():
    g = json.load(open(os.path.join(GOLD, "cache_sizes.json")))
    d_c, d_R, L, s = g["d_c"], g["d_R"], g["layers"], g["elem_bytes"]
    for case in g["cases"]:
        nbytes = oracle.cache_bytes(case["B"], case["T"], L, d_c, d_R, s)
        if "bytes" in case:
            assert nbytes == case["bytes"]
        assert nbytes == case["MiB"] * 1024 * 1024
    assert oracle.cache_elements_per_token_layer(d_c, d_R) == g["mla_elements_per_token_layer"]
    assert 2 * 128 * 128 == g["mha_elements_per_token_layer"]
    assert round(g["mha_elements_per_token_layer"] / g["mla_elements_per_token_layer"]) == g["mha_over_mla_rounded"]


def test_default_scale():
    """1/sqrt(d_h + d_R): 1/sqrt(192) at DeepSeek-V2 shape, not 1/sqrt(576)."""
    assert oracle.default_scale(128, 64) == 1 / math.sqrt(192)
    assert oracle.default_scale(32, 16) == 1 / math.sqrt(48)


# ---- prefill in the expanded form -----------------------------------------------------

def test_causal_attention_is_masked_sdpa():
    """causal_attention equals torch's SDPA with its causal mask, in fp64 (library routine)."""
    rng = np.random.default_rng(40)
    T, H = 37, 5
    q = rng.standard_normal((T, H, 24))
    k = rng.standard_normal((T, H, 24))
    v = rng.standard_normal((T, H, 7))
    o, lse = oracle.causal_attention(q, k, v, 0.25)
    t = lambda a: torch.from_numpy(a).transpose(0, 1)
    ref = torch.nn.functional.scaled_dot_product_attention(t(q), t(k), t(v), is_causal=True,
                                                           scale=0.25).transpose(0, 1).numpy()
    assert np.max(np.abs(o - ref)) <= 1e-12
    # lse of the visible scores: row 0 sees only itself
    assert np.allclose(lse[0], np.einsum("hd,hd->h", q[0], k[0]) * 0.25, atol=1e-12)


def test_expanded_prefill_rows_are_decodes():
    """Query t of a prompt is the decode of the prompt's first t + 1 tokens: every row of
    expanded_prefill equals expanded_decode over that prefix."""
    rng = np.random.default_rng(41)
    T, H, d_h, d_c, d_R = 11, 3, 8, 16, 4
    q_c = rng.standard_normal((T, H, d_h))
    q_pe = rng.standard_normal((T, H, d_R))
    c_kv = rng.standard_normal((T, d_c))
    k_pe = rng.standard_normal((T, d_R))
    w_uk = rng.standard_normal((H * d_h, d_c)) / 4
    w_uv = rng.standard_normal((H * d_h, d_c)) / 4
    o, lse = oracle.expanded_prefill(q_c, q_pe, c_kv, k_pe, w_uk, w_uv, 0.3)
    for t in (0, 1, 5, T - 1):
        dec = oracle.expanded_decode(q_c[t], q_pe[t], c_kv[:t + 1], k_pe[:t + 1], w_uk, w_uv, 0.3)
        assert np.max(np.abs(o[t] - dec["o"])) <= 1e-12
        assert np.max(np.abs(lse[t] - dec["lse"])) <= 1e-12
    # the first token sees only itself: its values
    assert np.allclose(o[0], np.stack([c_kv[0] @ w_uv[i * d_h:(i + 1) * d_h].T for i in range(H)]))
