"""GPU parity of the one-launch query side (mla_query_path): q~_i = W^UK_i^T W^UQ_i c^Q and
q_pe = RoPE(W^QR c^Q, seq_len - 1) against the oracle's plain products, absorption and RoPE;
closed forms bit-exact (a one-hot c^Q selecting weight columns); runs bit-identical; each
row's result independent of the rest of the batch."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import assert_bf16, dev, host64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_15_amd as m
    return m


def _weights(seed, H, d_cq, d_h=128, d_R=64, d_c=512):
    g = torch.Generator().manual_seed(seed)
    mk = lambda n, k: (torch.randn(n, k, generator=g) / math.sqrt(k)).to(torch.bfloat16)
    return {"w_uq": mk(H * d_h, d_cq), "w_qr": mk(H * d_R, d_cq), "w_uk": mk(H * d_h, d_c)}


def run(mla, c_q, wts, seq_lens, base=10000.0):
    """c_q: a CUDA tensor [B, d_cq] (may be a column range); the weights are packed on the GPU
    first.  Returns (q_lat, q_pe) on the GPU."""
    B, H = c_q.shape[0], wts["w_qr"].shape[0] // 64
    w_pack = mla.mla_pack_query_weights(dev(wts["w_uq"]), dev(wts["w_qr"]), dev(wts["w_uk"]), H)
    q_lat = torch.full((B, H, 512), float("nan"), device="cuda", dtype=torch.bfloat16)
    q_pe = torch.full((B, H, 64), float("nan"), device="cuda", dtype=torch.bfloat16)
    mla.mla_query_path(c_q, w_pack, dev(seq_lens), base, q_lat, q_pe)
    torch.cuda.synchronize()
    return q_lat, q_pe


def test_pack_query_weights_layout(mla):
    """The packed layout, element by element, rebuilt from its definition: fragment
    (c, i, tile, s4), lane l, element e holds row 16 tile + l % 16 of [W^UQ_i; W^QR_i] at
    k = 32 (4 c + s4) + 8 (l / 16) + e; then W^UK piece (i, hf, j, pos) holds
    W^UK[i*128 + j][256 hf + 8 (pos ^ f(j)) ..], f(j) = 2 (j % 4) + 8 ((j / 8) % 2)."""
    H, d_cq = 2, 768
    g = torch.Generator().manual_seed(99)
    w_uq = torch.randn(H * 128, d_cq, generator=g).to(torch.bfloat16)
    w_qr = torch.randn(H * 64, d_cq, generator=g).to(torch.bfloat16)
    w_uk = torch.randn(H * 128, 512, generator=g).to(torch.bfloat16)
    say("pack query weights")
    got = mla.mla_pack_query_weights(dev(w_uq), dev(w_qr), dev(w_uk), H).cpu()
    rows = torch.cat([w_uq.view(H, 128, d_cq), w_qr.view(H, 64, d_cq)], dim=1)  # [H, 192, d_cq]
    nc = d_cq // 128
    # [H, 192, nc, 4, 4, 8] (row, chunk, step, k group, element) -> [H, nc, 12, 4, 64 lanes, 8]
    r6 = rows.view(H, 12, 16, nc, 4, 4, 8)              # i, tile, n, c, s4, g, e
    frags = r6.permute(3, 0, 1, 4, 5, 2, 6).reshape(-1)  # c, i, tile, s4, (g, n), e
    f = lambda j: 2 * (j % 4) + 8 * ((j // 8) % 2)
    uk = torch.empty(H, 2, 128, 32, 8, dtype=torch.bfloat16)
    for i in range(H):
        for hf in range(2):
            for j in range(128):
                for pos in range(32):
                    c0 = 256 * hf + 8 * (pos ^ f(j))
                    uk[i, hf, j, pos] = w_uk[i * 128 + j, c0:c0 + 8]
    assert got.numel() == mla.query_pack_elems(H, d_cq)
    assert torch.equal(got[:frags.numel()], frags)
    assert torch.equal(got[frags.numel():], uk.reshape(-1))


def reference(c_q, wts, seq_lens, base=10000.0):
    """The oracle: q^C = W^UQ c^Q, q^R = W^QR c^Q (fp64 products), absorption, RoPE."""
    B = c_q.shape[0]
    H = wts["w_qr"].shape[0] // 64
    x = W.to_f64(c_q.cpu())
    q_c = oracle.linear(x, W.to_f64(wts["w_uq"])).reshape(B, H, 128)
    q_r = oracle.linear(x, W.to_f64(wts["w_qr"])).reshape(B, H, 64)
    q_lat = oracle.absorb_query(q_c, W.to_f64(wts["w_uk"]))
    pos = (seq_lens.numpy().astype(np.float64) - 1)[:, None]
    return q_lat, oracle.rope(q_r, pos, base)


@pytest.mark.parametrize("B,H,d_cq", [(1, 8, 384), (5, 8, 1536), (64, 16, 768), (100, 8, 1152)])
def test_query_path_against_oracle(mla, B, H, d_cq):
    g = torch.Generator().manual_seed(100 + B)
    c_q = torch.randn(B, d_cq, generator=g)
    wts = _weights(101 + B, H, d_cq)
    seq_lens = torch.randint(1, 200000, (B,), generator=g, dtype=torch.int32)
    seq_lens[0] = 1
    say(f"query path B={B} H={H} d_cq={d_cq}")
    q_lat, q_pe = run(mla, dev(c_q), wts, seq_lens)
    ref_lat, ref_pe = reference(c_q, wts, seq_lens)
    assert_bf16(host64(q_lat), ref_lat, f"q_lat B={B}")
    assert_bf16(host64(q_pe), ref_pe, f"q_pe B={B}")


def test_query_path_reads_a_column_range(mla):
    """c^Q read in place from the stacked projection [c^Q | c^KV | k^R] (rows 2112 apart)."""
    B, H, d_cq = 64, 8, 1536
    g = torch.Generator().manual_seed(110)
    y_a = torch.randn(B, d_cq + 512 + 64, generator=g)
    wts = _weights(111, H, d_cq)
    seq_lens = torch.full((B,), 2049, dtype=torch.int32)
    say("query path column range")
    y = dev(y_a)
    q_lat, q_pe = run(mla, y[:, :d_cq], wts, seq_lens)
    q_lat2, q_pe2 = run(mla, dev(y_a[:, :d_cq]), wts, seq_lens)
    assert torch.equal(q_lat, q_lat2) and torch.equal(q_pe, q_pe2)
    ref_lat, ref_pe = reference(y_a[:, :d_cq], wts, seq_lens)
    assert_bf16(host64(q_lat), ref_lat, "q_lat column range")
    assert_bf16(host64(q_pe), ref_pe, "q_pe column range")


def test_query_path_one_hot_exact(mla):
    """c^Q_b = e_{k_b}: q^C_i = W^UQ_i[:, k_b] and q^R = W^QR[:, k_b] exactly.  With W^UQ_i
    column k holding a single one at row j_i, q~_i is row j_i of W^UK_i bit for bit; at
    position 0 (seq_len 1) q_pe is the W^QR column itself."""
    B, H, d_cq = 9, 16, 384
    g = torch.Generator().manual_seed(120)
    wts = _weights(121, H, d_cq)
    ks = torch.randperm(d_cq, generator=g)[:B]
    js = torch.randint(0, 128, (H,), generator=g)
    w_uq = torch.zeros(H * 128, d_cq)
    for i in range(H):
        w_uq[i * 128 + int(js[i]), :] = 1.0
    wts["w_uq"] = w_uq.to(torch.bfloat16)
    c_q = torch.zeros(B, d_cq)
    c_q[torch.arange(B), ks] = 1.0
    say("query path one-hot")
    q_lat, q_pe = run(mla, dev(c_q), wts, torch.ones(B, dtype=torch.int32))
    q_lat, q_pe = q_lat.cpu(), q_pe.cpu()
    for b in range(B):
        for i in range(H):
            assert torch.equal(q_lat[b, i], wts["w_uk"][i * 128 + int(js[i])]), (b, i)
        assert torch.equal(q_pe[b].reshape(-1), wts["w_qr"][:, int(ks[b])]), b


def test_query_path_bit_identical_runs_and_rows_independent(mla):
    """No atomics: two runs agree bit for bit, and a row's outputs do not depend on the other
    rows of its batch or on which 64-row block it falls in."""
    B, H, d_cq = 100, 16, 1536
    g = torch.Generator().manual_seed(130)
    c_q = dev(torch.randn(B, d_cq, generator=g))
    wts = _weights(131, H, d_cq)
    seq_lens = torch.randint(1, 5000, (B,), generator=g, dtype=torch.int32)
    say("query path determinism")
    a = run(mla, c_q, wts, seq_lens)
    b = run(mla, c_q, wts, seq_lens)
    assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1])
    part = run(mla, c_q[60:67].contiguous(), wts, seq_lens[60:67])
    assert torch.equal(part[0], a[0][60:67]) and torch.equal(part[1], a[1][60:67])


def test_query_path_matches_two_launch_path(mla):
    """Against mla_linear_strided + mla_absorb_q_strided (the same products in two launches,
    q^C rounded to fp32 in between): both within the bf16 bar of the oracle, and of each
    other."""
    B, H, d_cq = 64, 16, 1536
    g = torch.Generator().manual_seed(140)
    c_q = torch.randn(B, d_cq, generator=g)
    wts = _weights(141, H, d_cq)
    seq_lens = torch.randint(1, 3000, (B,), generator=g, dtype=torch.int32)
    say("query path vs two launches")
    q_lat, q_pe = run(mla, dev(c_q), wts, seq_lens)
    w_b = dev(torch.cat([wts["w_uq"], wts["w_qr"]]))
    y_b = torch.empty(B, H * 192, device="cuda")
    mla.mla_linear_strided(dev(c_q), w_b, y_b)
    lat2 = torch.empty(B, H, 512, device="cuda", dtype=torch.bfloat16)
    pe2 = torch.empty(B, H, 64, device="cuda", dtype=torch.bfloat16)
    mla.mla_absorb_q_strided(y_b[:, :H * 128].view(B, H, 128), dev(wts["w_uk"]),
                             y_b[:, H * 128:].view(B, H, 64), dev(seq_lens), 10000.0, lat2, pe2)
    torch.cuda.synchronize()
    assert_bf16(host64(q_lat), host64(lat2), "q_lat one launch vs two")
    assert_bf16(host64(q_pe), host64(pe2), "q_pe one launch vs two")


def test_query_path_dsv2_b64_full(mla):
    """The decode layer's sizes (B=64, H=128, d_cq=1536): every output against the oracle."""
    x = W.layer_b64_t2k()
    wts = {k: x["weights"][k] for k in ("w_uq", "w_qr", "w_uk")}
    g = torch.Generator().manual_seed(150)
    c_q = torch.randn(64, 1536, generator=g)
    seq_lens = x["seq_lens_before"] + 1
    say("query path dsv2 B=64")
    q_lat, q_pe = run(mla, dev(c_q), wts, seq_lens)
    ref_lat, ref_pe = reference(c_q, wts, seq_lens)
    m, r = assert_bf16(host64(q_lat), ref_lat, "q_lat dsv2")
    print(f"query path dsv2 q_lat: max-abs {m:.3e} rel-L2 {r:.3e}")
    assert_bf16(host64(q_pe), ref_pe, "q_pe dsv2")
