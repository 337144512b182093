"""Plain fp64 CPU oracle for weight-absorbed MLA decode.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or link
this module: only the test suite, the smoke check and the benchmark's CPU-baseline
leg use it.  It shares no code, header, table or constant with the HIP library.

Everything here is NumPy in float64 and follows the plain definitions on the
source pages, written for a reader to check by eye.  Page references:

  [explainer]  "論文解説: DeepSeek-V2 — MoEモデルのKVキャッシュを93.3%削減する
               Multi-head Latent Attention" (0h-n0.github.io/posts/paper-2401-06066)
  [kasblo]     kasblo.com/?p=4663 (MLA explainer: stored data, computation order,
               decoupled RoPE, cache-size arithmetic)
  [qiita]      qiita.com/joule/items/57d9b3f4fc27959eaa0d ("Multi-Head Latent
               Attention" article: full equation set and the absorption derivation)

Readings where the pages leave a step open (each one is listed with its reason in
the design notes of the repository):
  * RoPE rotates adjacent pairs (x[2k], x[2k+1]) by pos * base**(-2k/d) with the
    standard 2x2 rotation [[cos, -sin], [sin, cos]] (RoFormer).  The pages only
    say that pairs of numbers are rotated by position ([kasblo] "分離したRoPE").
  * The cache holds k^R after rotation ([qiita] "RoPE の扱い" defines k^R_t as
    already rotated; [explainer] "Decoupled RoPE" caches k^R).
  * The decode query sits at position seq_len - 1 (the sum over j runs up to t,
    [qiita] "Attention 計算"), cache token j sits at position j (0-based).
  * Head i of W^UK / W^UV is the row block i*d_h ... (i+1)*d_h - 1 of the
    [n_h*d_h, d_c] weight, in nn.Linear [out, in] layout ([explainer] code sketch).
  * Softmax scale 1/sqrt(d_h + d_h^R) in both forms ([qiita] "Attention 計算").

Parity pins for every function live in the CPU test suite; every function below
has at least one pin that does not re-type its own formula.
"""

from __future__ import annotations

import math

import numpy as np

F64 = np.float64


def _f64(x) -> np.ndarray:
    return np.asarray(x, dtype=F64)


# --------------------------------------------------------------------------------------
# RoPE
# --------------------------------------------------------------------------------------
def rope(x, pos, base: float = 10000.0) -> np.ndarray:
    """Rotary position embedding of the last axis of ``x``.

    [kasblo] "位置情報は別の経路で持つ：分離したRoPE": pairs of numbers in q and k are
    rotated according to position so that the dot product reflects relative position.
    [qiita] "RoPE の扱い": q^R = RoPE(W^QR c^Q), k^R = RoPE(W^KR h).

    Pair k = (x[2k], x[2k+1]) is rotated by angle pos * theta_k with
    theta_k = base ** (-2k / d), d = x.shape[-1] (must be even).
    ``pos`` broadcasts against x.shape[:-1].
    """
    x = _f64(x)
    d = x.shape[-1]
    if d % 2:
        raise ValueError("RoPE needs an even dimension")
    k = np.arange(d // 2, dtype=F64)
    theta = float(base) ** (-2.0 * k / d)
    ang = _f64(pos)[..., None] * theta
    cos, sin = np.cos(ang), np.sin(ang)
    even, odd = x[..., 0::2], x[..., 1::2]
    out = np.empty(np.broadcast_shapes(x.shape, ang.shape[:-1] + (d,)), dtype=F64)
    out[..., 0::2] = even * cos - odd * sin
    out[..., 1::2] = even * sin + odd * cos
    return out


# --------------------------------------------------------------------------------------
# Softmax attention (the plain definition)
# --------------------------------------------------------------------------------------
def softmax(s, axis: int = -1) -> np.ndarray:
    """softmax_j(s) = exp(s_j - max) / sum exp(s - max); weights sum to one
    ([kasblo] "Qは今回の問い合わせ…": Softmax turns scores into weights summing to 1)."""
    s = _f64(s)
    m = np.max(s, axis=axis, keepdims=True)
    e = np.exp(s - m)
    return e / np.sum(e, axis=axis, keepdims=True)


def logsumexp(s, axis: int = -1) -> np.ndarray:
    """log sum_j exp(s_j), computed with the maximum pulled out."""
    s = _f64(s)
    m = np.max(s, axis=axis, keepdims=True)
    return (m + np.log(np.sum(np.exp(s - m), axis=axis, keepdims=True))).squeeze(axis)


def head_block(w, i: int, d_h: int) -> np.ndarray:
    """W_i: rows i*d_h .. (i+1)*d_h - 1 of an [n_h*d_h, in] weight ([explainer] code
    sketch: W_uk / W_uv are nn.Linear(d_c, n_heads*d_h), so W^UK_i is that row block)."""
    return _f64(w)[i * d_h:(i + 1) * d_h, :]


# --------------------------------------------------------------------------------------
# Expanded ("naive") decode: explicitly restore k^C and v^C for every cached token.
# --------------------------------------------------------------------------------------
def expanded_decode(q_c, q_pe, c_kv, k_pe, w_uk, w_uv, scale, w_o=None):
    """One query token of one sequence, the non-absorbed path.

    [explainer] "MLA: 低ランクKV結合圧縮": k^C_t = W^UK c^KV_t, v^C_t = W^UV c^KV_t.
    [explainer] "Decoupled RoPE": q_{t,i} = [q^C_i; RoPE(q^R_i)], k_{t,i} = [k^C_i; RoPE(k^R_t)].
    [qiita] "Attention 計算": o_i = sum_j softmax_j(q_i . k_{j,i} / sqrt(d_h + d_h^R)) v^C_{j,i},
    u = W^O [o_1; ...; o_{n_h}].

    q_c  [H, d_h]        content query q^C
    q_pe [H, d_R]        rotated position query RoPE(q^R)
    c_kv [T, d_c]        cached latents c^KV_j, j = 0..T-1
    k_pe [T, d_R]        cached rotated shared keys RoPE(k^R_j)
    w_uk, w_uv [H*d_h, d_c];  w_o [d, H*d_h] or None
    Returns dict with o [H, d_h], p [H, T], lse [H] (natural log of the softmax
    denominator of the scaled scores), scores [H, T] and u [d] if w_o is given.
    """
    q_c, q_pe, c_kv, k_pe = _f64(q_c), _f64(q_pe), _f64(c_kv), _f64(k_pe)
    H, d_h = q_c.shape
    T = c_kv.shape[0]
    scores = np.empty((H, T), dtype=F64)
    o = np.empty((H, d_h), dtype=F64)
    p_all = np.empty((H, T), dtype=F64)
    for i in range(H):
        k_c = c_kv @ head_block(w_uk, i, d_h).T          # [T, d_h]   k^C_{j,i}
        v_c = c_kv @ head_block(w_uv, i, d_h).T          # [T, d_h]   v^C_{j,i}
        q_i = np.concatenate([q_c[i], q_pe[i]])          # [d_h + d_R]
        k_i = np.concatenate([k_c, k_pe], axis=1)        # [T, d_h + d_R]
        s = (k_i @ q_i) * scale                          # [T]
        p = softmax(s)
        scores[i] = s
        p_all[i] = p
        o[i] = p @ v_c
    out = {"o": o, "p": p_all, "scores": scores, "lse": logsumexp(scores, axis=-1)}
    if w_o is not None:
        out["u"] = _f64(w_o) @ o.reshape(H * d_h)
    return out


def causal_attention(q, k, v, scale):
    """Causal softmax attention for a prompt, per head ([qiita] "Attention 計算": the sum for
    query t runs over j <= t, o_t = sum_j softmax_j(q_t . k_j * scale) v_j).

    q [T, H, d_qk], k [T, H, d_qk], v [T, H, d_v] -> (o [T, H, d_v], lse [T, H]).
    """
    q, k, v = _f64(q), _f64(k), _f64(v)
    T, H, _ = q.shape
    o = np.empty((T, H, v.shape[-1]), dtype=F64)
    lse = np.empty((T, H), dtype=F64)
    visible = np.tril(np.ones((T, T), dtype=bool))   # [t, j]: j <= t
    for i in range(H):
        s = (q[:, i] @ k[:, i].T) * scale              # [T, T]
        s = np.where(visible, s, -np.inf)
        o[:, i] = softmax(s, axis=-1) @ v[:, i]
        lse[:, i] = logsumexp(s, axis=-1)
    return o, lse


def expanded_prefill(q_c, q_pe, c_kv, k_pe, w_uk, w_uv, scale):
    """A prompt of T tokens through the expanded path, causal ([perforder]
    "極限最適化の代償" and [kasblo] "「キャッシュを減らせた」と「その割合だけ速い」は別の評価":
    for many query tokens the up-projected keys and values are the natural order).

    q_c [T, H, d_h], q_pe [T, H, d_R] (rotated), c_kv [T, d_c], k_pe [T, d_R] (rotated),
    w_uk, w_uv [H*d_h, d_c] -> (o [T, H, d_h], lse [T, H]).
    """
    q_c, q_pe = _f64(q_c), _f64(q_pe)
    T, H, d_h = q_c.shape
    k = np.empty((T, H, d_h + q_pe.shape[-1]), dtype=F64)
    v = np.empty((T, H, d_h), dtype=F64)
    for i in range(H):
        k[:, i, :d_h] = _f64(c_kv) @ head_block(w_uk, i, d_h).T
        k[:, i, d_h:] = _f64(k_pe)
        v[:, i] = _f64(c_kv) @ head_block(w_uv, i, d_h).T
    q = np.concatenate([q_c, q_pe], axis=-1)
    return causal_attention(q, k, v, scale)


# --------------------------------------------------------------------------------------
# Absorbed form, fp64 (used only to check that absorption changes nothing)
# --------------------------------------------------------------------------------------
def absorb_query(q_c, w_uk) -> np.ndarray:
    """q~_i = W^UK_i^T q^C_i for every head i.

    [explainer] "行列吸収トリック": q^C . (W^UK_i c) = (W^UK_i^T q^C) . c, so the key
    up-projection moves onto the query.  [kasblo] "K側は…Qを変換する" gives the same
    reorder with the worked example U^T q = (2, 3).
    q_c [H, d_h] (or [B, H, d_h]); w_uk [H*d_h, d_c] -> [H, d_c] (or [B, H, d_c]).
    """
    q_c = _f64(q_c)
    d_h = q_c.shape[-1]
    H = q_c.shape[-2]
    out = np.empty(q_c.shape[:-1] + (_f64(w_uk).shape[1],), dtype=F64)
    for i in range(H):
        out[..., i, :] = q_c[..., i, :] @ head_block(w_uk, i, d_h)
    return out


def latent_attention(q_lat, q_pe, rows, d_c: int, scale):
    """Attention straight over latent cache rows ([c^KV_j ; k^R_j], 576 = 512 + 64 at
    DeepSeek-V2 shape, [explainer] "Decoupled RoPE": the cache holds 576 elements per
    token per layer).

    Score s_ij = scale * ([q~_i; q_pe_i] . row_j) — the content part is the absorbed
    score of [explainer] "行列吸収トリック", the position part the decoupled RoPE
    score of [kasblo] "分離したRoPE" (the two dot products are added).
    Value: o~_i = sum_j p_ij c_j ([kasblo] "V側は、小さな表現の加重和を先に求める":
    sum the latents with the weights first, up-project afterwards).

    q_lat [H, d_c], q_pe [H, d_R], rows [T, d_c + d_R].
    Returns o_lat [H, d_c], lse [H] (natural log), p [H, T].
    For T = 0 returns o_lat = 0 and lse = -inf.
    """
    q_lat, q_pe, rows = _f64(q_lat), _f64(q_pe), _f64(rows)
    H = q_lat.shape[0]
    T = rows.shape[0]
    if T == 0:
        return {"o_lat": np.zeros((H, d_c)), "lse": np.full(H, -np.inf), "p": np.zeros((H, 0))}
    q = np.concatenate([q_lat, q_pe], axis=1)            # [H, d_c + d_R]
    s = (q @ rows.T) * scale                             # [H, T]
    p = softmax(s)
    return {"o_lat": p @ rows[:, :d_c], "lse": logsumexp(s, axis=-1), "p": p, "scores": s}


def up_project_values(o_lat, w_uv) -> np.ndarray:
    """o_i = W^UV_i o~_i ([kasblo] "V側は…": sum first, transform last)."""
    o_lat = _f64(o_lat)
    H = o_lat.shape[-2]
    d_h = _f64(w_uv).shape[0] // H
    out = np.empty(o_lat.shape[:-1] + (d_h,), dtype=F64)
    for i in range(H):
        out[..., i, :] = o_lat[..., i, :] @ head_block(w_uv, i, d_h).T
    return out


def output_projection(o, w_o) -> np.ndarray:
    """u = W^O [o_1; ...; o_{n_h}] ([qiita] "Attention 計算").  o [..., H, d_h]."""
    o = _f64(o)
    flat = o.reshape(o.shape[:-2] + (o.shape[-2] * o.shape[-1],))
    return flat @ _f64(w_o).T


def absorbed_decode(q_c, q_pe, c_kv, k_pe, w_uk, w_uv, scale, w_o=None):
    """Absorbed order in fp64: q~ = W^UK^T q^C, attention on the latent, then W^UV."""
    q_lat = absorb_query(q_c, w_uk)
    rows = np.concatenate([_f64(c_kv), _f64(k_pe)], axis=1)
    att = latent_attention(q_lat, q_pe, rows, _f64(c_kv).shape[1], scale)
    o = up_project_values(att["o_lat"], w_uv)
    out = {"o": o, "o_lat": att["o_lat"], "lse": att["lse"], "q_lat": q_lat}
    if w_o is not None:
        out["u"] = output_projection(o, w_o)
    return out


# --------------------------------------------------------------------------------------
# Split over tokens + log-sum-exp combine
# --------------------------------------------------------------------------------------
def combine_splits(o_parts, lse_parts):
    """Merge per-split softmax results of the same rows.

    Split s saw tokens J_s and returned o_s = sum_{j in J_s} e^{s_j} c_j / sum_{J_s} e^{s_j}
    and lse_s = log sum_{J_s} e^{s_j}.  The full softmax is then
    o = sum_s e^{lse_s - LSE} o_s with LSE = log sum_s e^{lse_s}: the softmax
    denominator over all tokens is the sum of the per-split denominators
    ([qiita] "Attention 計算", the sum over j split into disjoint ranges).
    Splits with lse = -inf (no tokens) get weight 0.

    o_parts [S, ..., D], lse_parts [S, ...] -> (o [..., D], lse [...]).
    """
    o_parts, lse_parts = _f64(o_parts), _f64(lse_parts)
    m = np.max(lse_parts, axis=0)
    safe_m = np.where(np.isfinite(m), m, 0.0)
    w = np.where(np.isfinite(lse_parts), np.exp(lse_parts - safe_m), 0.0)
    den = np.sum(w, axis=0)
    lse = np.where(den > 0, safe_m + np.log(np.where(den > 0, den, 1.0)), -np.inf)
    num = np.sum(w[..., None] * o_parts, axis=0)
    o = np.where(den[..., None] > 0, num / np.where(den > 0, den, 1.0)[..., None], 0.0)
    return o, lse


# --------------------------------------------------------------------------------------
# Paged latent cache: addressing, append, gather
# --------------------------------------------------------------------------------------
def page_slot(block_table_row, pos: int, page_size: int):
    """Token at position pos of a sequence lives at page block_table_row[pos // P],
    slot pos % P (paged pool; not on the pages, the plainest layout for a pool of
    fixed-size pages)."""
    return int(block_table_row[pos // page_size]), pos % page_size


def gather_rows(cache, block_table_row, seq_len: int, page_size: int) -> np.ndarray:
    """Rows 0..seq_len-1 of one sequence, in token order, from a paged pool
    cache [num_pages, page_size, row]."""
    cache = _f64(cache)
    out = np.empty((seq_len, cache.shape[-1]), dtype=F64)
    for j in range(seq_len):
        page, slot = page_slot(block_table_row, j, page_size)
        out[j] = cache[page, slot]
    return out


def append_rows(cache, block_table, seq_lens_before, c_new, k_new, rope_base: float):
    """Write n new tokens per sequence into a copy of the paged cache.

    Row layout [c^KV ; RoPE(k^R, pos)], pos = seq_lens_before[b] + n ([explainer]
    "Decoupled RoPE": the cache holds c^KV and the rotated shared key k^R; the code
    sketch concatenates the new token's c_kv / k_rope onto the cache along time).
    cache [num_pages, P, d_c + d_R]; c_new [B, n, d_c]; k_new [B, n, d_R] (pre-rotation).
    """
    cache = _f64(cache).copy()
    c_new, k_new = _f64(c_new), _f64(k_new)
    B, n, d_c = c_new.shape
    P = cache.shape[1]
    for b in range(B):
        for t in range(n):
            pos = int(seq_lens_before[b]) + t
            page, slot = page_slot(block_table[b], pos, P)
            cache[page, slot, :d_c] = c_new[b, t]
            cache[page, slot, d_c:] = rope(k_new[b, t], pos, rope_base)
    return cache


def paged_decode(q_lat, q_pe, cache, block_table, seq_lens, d_c: int, scale):
    """Latent attention for every sequence of a paged batch.
    q_lat [B, H, d_c], q_pe [B, H, d_R] (rotated), cache [pages, P, d_c + d_R].
    Returns o_lat [B, H, d_c], lse [B, H]."""
    q_lat, q_pe = _f64(q_lat), _f64(q_pe)
    B, H, _ = q_lat.shape
    P = np.asarray(cache).shape[1]
    o = np.zeros((B, H, d_c), dtype=F64)
    lse = np.full((B, H), -np.inf, dtype=F64)
    for b in range(B):
        rows = gather_rows(cache, block_table[b], int(seq_lens[b]), P)
        att = latent_attention(q_lat[b], q_pe[b], rows, d_c, scale)
        o[b], lse[b] = att["o_lat"], att["lse"]
    return o, lse


def paged_decode_multi(q_lat, q_pe, cache, block_table, seq_lens, n_q: int, d_c: int, scale):
    """Latent attention for n_q new query tokens per sequence, all already in the cache.
    Query t of sequence b sits at position seq_lens[b] - n_q + t and attends to the cached
    tokens 0 .. that position: the sum over tokens runs up to the query's own position
    ([qiita] "Attention 計算"), so the new tokens see each other causally.
    q_lat [B, n_q, H, d_c], q_pe [B, n_q, H, d_R].
    Returns o_lat [B, n_q, H, d_c], lse [B, n_q, H] (no visible token: o = 0, lse = -inf)."""
    q_lat, q_pe = _f64(q_lat), _f64(q_pe)
    B, nq, H, _ = q_lat.shape
    if nq != n_q:
        raise ValueError("q_lat must hold n_q tokens per sequence")
    P = np.asarray(cache).shape[1]
    o = np.zeros((B, n_q, H, d_c), dtype=F64)
    lse = np.full((B, n_q, H), -np.inf, dtype=F64)
    for b in range(B):
        for t in range(n_q):
            visible = int(seq_lens[b]) - n_q + t + 1   # tokens 0 .. position of query t
            if visible <= 0:
                continue
            rows = gather_rows(cache, block_table[b], visible, P)
            att = latent_attention(q_lat[b, t], q_pe[b, t], rows, d_c, scale)
            o[b, t], lse[b, t] = att["o_lat"], att["lse"]
    return o, lse


# --------------------------------------------------------------------------------------
# Projections and the full decode layer
# --------------------------------------------------------------------------------------
def linear(x, w) -> np.ndarray:
    """y = x W^T for an nn.Linear weight w [out, in] ([explainer] code sketch)."""
    return _f64(x) @ _f64(w).T


def decode_layer(h, weights: dict, cache, block_table, seq_lens_before, d_h: int,
                 d_R: int, rope_base: float, scale, batch_index=None):
    """One decode step of one MLA layer for each sequence, expanded ("naive") path.

    Projections ([qiita] "Query の圧縮", "RoPE の扱い"; [explainer] eq. for c^KV):
      c^Q = W^DQ h, q^C = W^UQ c^Q, q^R = RoPE(W^QR c^Q),
      c^KV = W^DKV h, k^R = RoPE(W^KR h)
    The new token (position seq_lens_before[b]) is appended after the cached ones, then
    the expanded attention of ``expanded_decode`` runs over all of them and
    u = W^O [o_1; ...; o_H].  No normalisation layers ([kasblo] omits them).

    h [B, d]; weights: w_dq, w_uq, w_qr, w_dkv, w_kr, w_uk, w_uv, w_o.
    cache [pages, P, d_c + d_R] holds the prior tokens (rotated k^R).
    batch_index: optional iterable of sequences to compute (sampling at full size).
    Returns dict: u [B, d] (rows not computed are NaN), and the new-token projections.
    """
    h = _f64(h)
    w = {k: _f64(v) for k, v in weights.items()}
    B = h.shape[0]
    H = w["w_uq"].shape[0] // d_h
    d_c = w["w_dkv"].shape[0]
    P = np.asarray(cache).shape[1]
    c_q = linear(h, w["w_dq"])
    q_c = linear(c_q, w["w_uq"]).reshape(B, H, d_h)
    q_r = linear(c_q, w["w_qr"]).reshape(B, H, d_R)
    c_new = linear(h, w["w_dkv"])
    k_new = linear(h, w["w_kr"])
    u = np.full((B, w["w_o"].shape[0]), np.nan, dtype=F64)
    idx = range(B) if batch_index is None else batch_index
    for b in idx:
        pos = int(seq_lens_before[b])
        prior = gather_rows(cache, block_table[b], pos, P)
        c_all = np.concatenate([prior[:, :d_c], c_new[b][None]], axis=0)
        k_all = np.concatenate([prior[:, d_c:], rope(k_new[b], pos, rope_base)[None]], axis=0)
        q_pe = rope(q_r[b], pos, rope_base)
        res = expanded_decode(q_c[b], q_pe, c_all, k_all, w["w_uk"], w["w_uv"], scale, w["w_o"])
        u[b] = res["u"]
    return {"u": u, "c_q": c_q, "q_c": q_c, "q_r": q_r, "c_kv_new": c_new, "k_r_new": k_new}


# --------------------------------------------------------------------------------------
# Cache-size arithmetic
# --------------------------------------------------------------------------------------
def cache_elements_per_token_layer(d_c: int, d_R: int) -> int:
    """d_c + d_h^R elements per token per layer ([explainer] Table 6 row MLA; [kasblo]
    "1トークン・1層では「512＋64」個の数値")."""
    return d_c + d_R


def cache_bytes(B: int, T: int, layers: int, d_c: int, d_R: int, elem_bytes: int) -> int:
    """B * T * L * (d_c + d_r) * s bytes ([kasblo] "容量を計算する" formula)."""
    return B * T * layers * cache_elements_per_token_layer(d_c, d_R) * elem_bytes


def default_scale(d_h: int, d_R: int) -> float:
    """1 / sqrt(d_h + d_h^R) ([qiita] "Attention 計算")."""
    return 1.0 / math.sqrt(d_h + d_R)
