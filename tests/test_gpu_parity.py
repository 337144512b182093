"""GPU parity: the HIP path through the C ABI against the fp64 oracle on the same seeded
inputs.  Tolerances: fp32 max-abs <= 1e-5; bf16 max-abs <= 2e-2 and rel-L2 <= 5e-3;
indexing (which tokens are read) bit-exact."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import assert_bf16, assert_fp32, dev, errors, host64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_15_amd as m
    return m


def run_attention(mla, inp, S, lse=True, part=torch.float32):
    """decode_attn (+ combine for S > 1) on device copies of a workloads problem; `part` is
    the dtype of the split partials (float32 or bfloat16)."""
    q_lat, q_pe, cache = dev(inp["q_lat"]), dev(inp["q_pe"]), dev(inp["cache"])
    bt, sl = dev(inp["block_table"]), dev(inp["seq_lens"])
    B, H, d_c = q_lat.shape
    if S == 1:
        out = torch.empty(B, H, d_c, device="cuda")
        lse_t = torch.empty(B, H, device="cuda") if lse else None
        mla.mla_decode_attn(q_lat, q_pe, cache, bt, sl, inp["scale"], 1, out, lse_t)
    else:
        o_part = torch.empty(B, H, S, d_c, device="cuda", dtype=part)
        lse_part = torch.empty(B, H, S, device="cuda")
        mla.mla_decode_attn(q_lat, q_pe, cache, bt, sl, inp["scale"], S, o_part, lse_part)
        out = torch.empty(B, H, d_c, device="cuda")
        lse_t = torch.empty(B, H, device="cuda")
        mla.mla_splitk_combine(o_part, lse_part, out, lse_t)
    torch.cuda.synchronize()
    return out, lse_t


def oracle_attention(inp, batch_index=None):
    d_c = inp["shape"].d_c
    P = inp["cache"].shape[1]
    cache = inp["cache"]
    bt = inp["block_table"].numpy()
    sl = inp["seq_lens"].numpy()
    idx = range(inp["q_lat"].shape[0]) if batch_index is None else batch_index
    o, lse = [], []
    for b in idx:
        # gather only the pages this sequence references, then the oracle's paged gather
        rows = oracle.gather_rows(W.to_f64(cache[torch.from_numpy(np.maximum(bt[b], 0)).long()]),
                                  np.arange(bt.shape[1]), int(sl[b]), P)
        att = oracle.latent_attention(W.to_f64(inp["q_lat"][b]), W.to_f64(inp["q_pe"][b]), rows,
                                      d_c, inp["scale"])
        o.append(att["o_lat"])
        lse.append(att["lse"])
    return np.stack(o), np.stack(lse)


# ------------------------------------------------------------------ tiny fp32 end to end
def test_tiny_fp32_chain(mla):
    """Cache fill with RoPE, query absorption + RoPE, attention (1, 2, 4 splits), combine,
    W^UV: every intermediate and the output against the oracle, max-abs <= 1e-5."""
    x = W.tiny_fp32()
    s = x["shape"]
    B, H, T = s.B, s.H, x["T"]
    say("tiny_fp32 chain")
    pages = T // W.PAGE
    cache = torch.zeros(pages, W.PAGE, s.d_c + s.d_R, device="cuda")
    bt, before = dev(x["block_table"]), dev(x["seq_lens_before"])
    mla.mla_kv_append(dev(x["c_kv"]), dev(x["k_r"]), before, bt, cache, x["rope_base"])
    seq_lens = torch.full((B,), T, dtype=torch.int32, device="cuda")
    q_lat = torch.empty(B, H, s.d_c, device="cuda")
    q_pe = torch.empty(B, H, s.d_R, device="cuda")
    mla.mla_absorb_q(dev(x["q_c"]), dev(x["w_uk"]), dev(x["q_r"]), seq_lens, x["rope_base"],
                     q_lat, q_pe)
    torch.cuda.synchronize()

    # oracle, expanded path with explicit RoPE at positions 0..T-1, query at T-1
    c = W.to_f64(x["c_kv"][0])
    k_pe = oracle.rope(W.to_f64(x["k_r"][0]), np.arange(T), x["rope_base"])
    q_pe_ref = oracle.rope(W.to_f64(x["q_r"][0]), T - 1, x["rope_base"])
    ref = oracle.expanded_decode(W.to_f64(x["q_c"][0]), q_pe_ref, c, k_pe, W.to_f64(x["w_uk"]),
                                 W.to_f64(x["w_uv"]), x["scale"])
    rows_ref = np.concatenate([c, k_pe], 1)
    assert_fp32(host64(cache).reshape(T, -1), rows_ref, 1e-6, "cache rows")
    assert_fp32(host64(q_lat)[0], oracle.absorb_query(W.to_f64(x["q_c"][0]), W.to_f64(x["w_uk"])),
                1e-5, "q_lat")
    assert_fp32(host64(q_pe)[0], q_pe_ref, 1e-6, "q_pe")

    for S in (1, 2, 4):
        inp = {"q_lat": q_lat, "q_pe": q_pe, "cache": cache, "block_table": bt,
               "seq_lens": seq_lens, "scale": x["scale"]}
        o_lat, lse = run_attention(mla, inp, S)
        o_heads = torch.empty(B, H, s.d_h, device="cuda")
        mla.mla_out_proj(o_lat, dev(x["w_uv"]), None, o_heads)
        torch.cuda.synchronize()
        assert_fp32(host64(o_heads)[0], ref["o"], 1e-5, f"o (S={S})")
        assert_fp32(host64(lse)[0], ref["lse"], 1e-5, f"lse (S={S})")


def test_worked_example_on_gpu(mla):
    """kasblo.com/?p=4663 figure '説明用の数値例' zero-padded into the fp32 shapes:
    c=(2,1), U=[[1,0],[0,1],[1,1]] as head 0's W^UK block, q=(1,2,1), scale 1, no RoPE part,
    one cached token.  q~ = U^T q = (2, 3) exactly; lse = score = 7 exactly; o~ = c."""
    say("worked example")
    H, d_h, d_c, d_R = 4, 32, 64, 16
    w_uk = torch.zeros(H * d_h, d_c)
    w_uk[0:3, 0:2] = torch.tensor([[1.0, 0.0], [0.0, 1.0], [1.0, 1.0]])
    q_c = torch.zeros(1, H, d_h)
    q_c[0, 0, 0:3] = torch.tensor([1.0, 2.0, 1.0])
    q_lat = torch.empty(1, H, d_c, device="cuda")
    seq_lens = torch.ones(1, dtype=torch.int32, device="cuda")
    mla.mla_absorb_q(dev(q_c), dev(w_uk), None, seq_lens, 10000.0, q_lat, None)
    cache = torch.zeros(1, W.PAGE, d_c + d_R, device="cuda")
    cache[0, 0, 0:2] = torch.tensor([2.0, 1.0])
    q_pe = torch.zeros(1, H, d_R, device="cuda")
    out = torch.empty(1, H, d_c, device="cuda")
    lse = torch.empty(1, H, device="cuda")
    bt = torch.zeros(1, 1, dtype=torch.int32, device="cuda")
    mla.mla_decode_attn(q_lat, q_pe, cache, bt, seq_lens, 1.0, 1, out, lse)
    torch.cuda.synchronize()
    assert q_lat[0, 0, :2].tolist() == [2.0, 3.0]
    assert torch.all(q_lat[0, 0, 2:] == 0) and torch.all(q_lat[0, 1:] == 0)
    assert lse[0, 0].item() == 7.0
    assert out[0, 0, :2].tolist() == [2.0, 1.0]


# ------------------------------------------------------------------ bf16 latent parity
@pytest.mark.parametrize("H", [128, 64, 16, 20])
@pytest.mark.parametrize("S", [1, 3, 8])
def test_latent_ragged_midsize(mla, H, S):
    """Several pages, a ragged tail, a 1-token sequence, permuted pages."""
    inp = W.paged_attention(100 + H, B=3, H=H, seq_lens=[1, 700, 1500])
    say(f"ragged midsize H={H} S={S}")
    out, lse = run_attention(mla, inp, S)
    o_ref, lse_ref = oracle_attention(inp)
    assert_bf16(host64(out), o_ref, f"o~ H={H} S={S}")
    m, _ = errors(host64(lse), lse_ref)
    assert m <= 2e-2, f"lse max-abs {m}"


@pytest.mark.slow
@pytest.mark.parametrize("part", [torch.float32, torch.bfloat16], ids=["f32part", "bf16part"])
def test_dsv2_b32_t4k_full(mla, part):
    """B=32, T=4096, H=128 (the headline shape), suggested splits, full output; with
    bf16 partials this is the launch configuration the benchmark times."""
    inp = W.dsv2_b32_t4k()
    S = mla.mla_suggest_num_splits(32, 4096, 0, 64, 256)
    say(f"dsv2_b32_t4k S={S} part={part}")
    out, lse = run_attention(mla, inp, S, part=part)
    o_ref, lse_ref = oracle_attention(inp)
    m, r = assert_bf16(host64(out), o_ref, "dsv2_b32_t4k")
    print(f"dsv2_b32_t4k ({part}): max-abs {m:.3e} rel-L2 {r:.3e}")
    assert errors(host64(lse), lse_ref)[0] <= 2e-2


@pytest.mark.slow
def test_long_b4_t32k_full(mla):
    """B=4, T=32768 over a permuted pool, 64 splits, full output."""
    inp = W.long_b4_t32k()
    S = mla.mla_suggest_num_splits(4, 32768, 0, 64, 256)
    say(f"long_b4_t32k S={S}")
    out, lse = run_attention(mla, inp, S)
    o_ref, lse_ref = oracle_attention(inp)
    m, r = assert_bf16(host64(out), o_ref, "long_b4_t32k")
    print(f"long_b4_t32k: max-abs {m:.3e} rel-L2 {r:.3e}")


@pytest.mark.slow
def test_ragged_b128_sampled(mla):
    """B=128 ragged over a shared permuted pool: whole batch on the GPU, sampled
    sequences (shortest, longest, and a seeded draw) against the oracle."""
    inp = W.ragged_b128()
    sl = inp["seq_lens"].tolist()
    S = mla.mla_suggest_num_splits(128, max(sl), sum(sl), 64, 256)
    say(f"ragged_b128 S={S}")
    out, lse = run_attention(mla, inp, S)
    rng = np.random.default_rng(0)
    pick = sorted(set([int(np.argmin(sl)), int(np.argmax(sl))] + rng.choice(128, 10, replace=False).tolist()))
    o_ref, _ = oracle_attention(inp, pick)
    m, r = assert_bf16(host64(out)[pick], o_ref, "ragged_b128")
    print(f"ragged_b128 sample {pick}: max-abs {m:.3e} rel-L2 {r:.3e}")


# ------------------------------------------------------------------ multi-token decode
def run_attention_multi(mla, inp, q_lat, q_pe, n_q, S, part=torch.float32):
    """mla_decode_attn_multi (+ combine over B n_q rows for S > 1)."""
    cache, bt, sl = dev(inp["cache"]), dev(inp["block_table"]), dev(inp["seq_lens"])
    B, _, H, d_c = q_lat.shape
    ql, qp = dev(q_lat), dev(q_pe)
    if S == 1:
        out = torch.empty(B, n_q, H, d_c, device="cuda")
        mla.mla_decode_attn_multi(ql, qp, cache, bt, sl, inp["scale"], 1, out, None)
    else:
        o_part = torch.empty(B, n_q, H, S, d_c, device="cuda", dtype=part)
        lse_part = torch.empty(B, n_q, H, S, device="cuda")
        mla.mla_decode_attn_multi(ql, qp, cache, bt, sl, inp["scale"], S, o_part, lse_part)
        out = torch.empty(B * n_q, H, d_c, device="cuda")
        mla.mla_splitk_combine(o_part.view(B * n_q, H, S, d_c), lse_part.view(B * n_q, H, S), out)
        out = out.view(B, n_q, H, d_c)
    torch.cuda.synchronize()
    return out


@pytest.mark.parametrize("H", [128, 20], ids=["mfma", "generic"])
def test_multi_token_decode(mla, H):
    """n_q new tokens per sequence, causal among them, against the oracle: ragged lengths
    over permuted pages, one sequence shorter than n_q (its first query sees nothing and
    returns exactly 0), split counts 1, 3 and 8 with fp32 and bf16 partials; n_q = 1 equals
    mla_decode_attn bit for bit."""
    n_q = 3
    inp = W.paged_attention(40 + H, B=4, H=H, seq_lens=[2, 97, 700, 1537])
    g = torch.Generator().manual_seed(41)
    q_lat = torch.randn(4, n_q, H, 512, generator=g).to(torch.bfloat16)
    q_pe = torch.randn(4, n_q, H, 64, generator=g).to(torch.bfloat16)
    cache64 = W.to_f64(inp["cache"])
    o_ref, _ = oracle.paged_decode_multi(W.to_f64(q_lat), W.to_f64(q_pe), cache64,
                                         inp["block_table"].numpy(), inp["seq_lens"].numpy(),
                                         n_q, 512, inp["scale"])
    for S, part in [(1, torch.float32), (3, torch.float32), (8, torch.bfloat16)]:
        say(f"multi-token decode H={H} n_q={n_q} S={S} part={part}")
        out = run_attention_multi(mla, inp, q_lat, q_pe, n_q, S, part)
        assert_bf16(host64(out), o_ref, f"S={S}")
        assert float(out[0, 0].abs().max()) == 0.0  # position -1: no visible token
    say(f"multi-token decode H={H} n_q=1 vs single")
    one = run_attention_multi(mla, inp, q_lat[:, :1], q_pe[:, :1], 1, 4)
    single = dict(inp, q_lat=q_lat[:, 0].contiguous(), q_pe=q_pe[:, 0].contiguous())
    ref_one, _ = run_attention(mla, single, 4)
    assert torch.equal(one[:, 0], ref_one)


def test_multi_token_decode_fp32(mla):
    """The fp32 shape (d_c = 64, d_R = 16, H = 4) with n_q = 4: max-abs <= 1e-5."""
    n_q = 4
    inp = W.paged_attention(42, B=2, H=4, seq_lens=[5, 300], d_c=64, d_R=16, d_h=32,
                            dtype=torch.float32)
    g = torch.Generator().manual_seed(43)
    q_lat = torch.randn(2, n_q, 4, 64, generator=g)
    q_pe = torch.randn(2, n_q, 4, 16, generator=g)
    o_ref, _ = oracle.paged_decode_multi(W.to_f64(q_lat), W.to_f64(q_pe), W.to_f64(inp["cache"]),
                                         inp["block_table"].numpy(), inp["seq_lens"].numpy(),
                                         n_q, 64, inp["scale"])
    for S in (1, 2):
        say(f"multi-token decode fp32 n_q={n_q} S={S}")
        out = run_attention_multi(mla, inp, q_lat, q_pe, n_q, S)
        assert_fp32(host64(out), o_ref, what=f"S={S}")


# ------------------------------------------------------------------ indexing exactness
def _spike_problem(B, H, seq_lens, spikes, seed=7):
    """q~ = 0, q_pe = 64 e_0; the rope part of every row is 0 except row j* of each
    sequence, whose k^R[0] = 64: its score is 4096*scale (~296) above all others, so its
    softmax weight is 1 and every other weight underflows to exactly 0."""
    inp = W.paged_attention(seed, B=B, H=H, seq_lens=seq_lens)
    inp["cache"][:, :, 512:] = 0
    inp["q_lat"].zero_()
    inp["q_pe"].zero_()
    inp["q_pe"][:, :, 0] = 64.0
    bt = inp["block_table"]
    for b, j in enumerate(spikes):
        inp["cache"][int(bt[b, j // 64]), j % 64, 512] = 64.0
    return inp


@pytest.mark.parametrize("S", [1, 4])
def test_spike_selects_exact_token(mla, S):
    """o~ equals the selected latent bit-exactly on both sides of page boundaries."""
    seq_lens = [64, 65, 128, 129, 300, 1000, 1000, 4096]
    spikes = [63, 64, 127, 128, 0, 999, 511, 4095]
    inp = _spike_problem(len(seq_lens), 32, seq_lens, spikes)
    say(f"spike S={S}")
    out, _ = run_attention(mla, inp, S)
    out = out.cpu()
    bt = inp["block_table"]
    for b, j in enumerate(spikes):
        want = inp["cache"][int(bt[b, j // 64]), j % 64, :512].float()
        assert torch.equal(out[b], want.expand_as(out[b])), f"seq {b} token {j}"


def test_single_token_bit_exact(mla):
    """seq_len = 1: softmax weight exactly 1, o~ = c_0 bit-exactly."""
    inp = W.paged_attention(8, B=4, H=128, seq_lens=[1, 1, 1, 1])
    say("single token")
    out, lse = run_attention(mla, inp, 1)
    out = out.cpu()
    bt = inp["block_table"]
    for b in range(4):
        want = inp["cache"][int(bt[b, 0]), 0, :512].float().expand_as(out[b])
        bad = (out[b] != want).nonzero()
        assert bad.numel() == 0, (f"seq {b}: {bad.shape[0]} mismatches, first at {bad[:4].tolist()}: "
                                  f"{[(out[b][tuple(i)].item(), want[tuple(i)].item()) for i in bad[:4]]}")


def test_page_permutation_bit_identical(mla):
    """Moving pages in the pool (and the block table with them) changes nothing."""
    inp = W.paged_attention(9, B=3, H=128, seq_lens=[333, 1024, 77], permute_pages=False)
    say("page permutation")
    a, la = run_attention(mla, inp, 2)
    n = inp["cache"].shape[0]
    perm = torch.randperm(n, generator=torch.Generator().manual_seed(1))
    inp2 = dict(inp)
    inp2["cache"] = torch.empty_like(inp["cache"])
    inp2["cache"][perm] = inp["cache"]
    bt = inp["block_table"].clone()
    m = bt >= 0
    bt[m] = perm[bt[m].long()].to(torch.int32)
    inp2["block_table"] = bt
    b, lb = run_attention(mla, inp2, 2)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_nan_poison_outside_context(mla):
    """NaN in pages nobody references and in slots at or past seq_len is never read."""
    inp = W.paged_attention(10, B=3, H=64, seq_lens=[70, 129, 500], extra_pages=3)
    say("nan poison")
    clean, lc = run_attention(mla, inp, 3)
    pois = dict(inp)
    cache = inp["cache"].clone()
    bt = inp["block_table"]
    used = set(int(v) for v in bt.flatten().tolist() if v >= 0)
    for p in range(cache.shape[0]):
        if p not in used:
            cache[p] = float("nan")
    for b, L in enumerate(inp["seq_lens"].tolist()):
        last = int(bt[b, (L - 1) // 64])
        cache[last, (L - 1) % 64 + 1:] = float("nan")
    pois["cache"] = cache
    dirty, ld = run_attention(mla, pois, 3)
    assert torch.equal(clean, dirty) and torch.equal(lc, ld)


def test_splits_agree_fp32_combine(mla):
    """The split-K combine is exact up to fp32 rounding: with the fp32-math path (H=20 is
    not tiled by the MFMA kernel), S = 1 and S in {2, 7, 64, 65} agree to 1e-5, including
    splits entirely past the end of short sequences."""
    inp = W.paged_attention(11, B=4, H=20, seq_lens=[64, 100, 2000, 4096])
    say("splits fp32")
    ref, lref = run_attention(mla, inp, 1)
    for S in (2, 7, 64, 65):  # up to 64 splits one wavefront per head combines; beyond, a workgroup
        out, lse = run_attention(mla, inp, S)
        assert_fp32(host64(out), host64(ref), 1e-5, f"o S={S}")
        assert_fp32(host64(lse), host64(lref), 1e-5, f"lse S={S}")


@pytest.mark.parametrize("part", [torch.float32, torch.bfloat16], ids=["f32part", "bf16part"])
def test_splits_mfma_vs_oracle(mla, part):
    """MFMA path: every split count (including empty splits) meets the bf16 bar, with
    fp32 and with bf16 split partials."""
    inp = W.paged_attention(11, B=4, H=128, seq_lens=[64, 100, 2000, 4096])
    o_ref, lse_ref = oracle_attention(inp)
    for S in (1, 2, 7, 64):
        say(f"splits mfma S={S} part={part}")
        out, lse = run_attention(mla, inp, S, part=part)
        assert_bf16(host64(out), o_ref, f"S={S}")
        assert errors(host64(lse), lse_ref)[0] <= 2e-2
        assert torch.isfinite(lse).all()


def test_bf16_partials_generic_path(mla):
    """bf16 split partials through the VALU path (H=20): the combined output stays within
    bf16 rounding of the fp32-partial result, which itself matches the oracle."""
    inp = W.paged_attention(15, B=3, H=20, seq_lens=[70, 700, 3000])
    o_ref, _ = oracle_attention(inp)
    say("bf16 partials generic")
    a, la = run_attention(mla, inp, 5)
    b, lb = run_attention(mla, inp, 5, part=torch.bfloat16)
    assert_bf16(host64(a), o_ref, "fp32 partials")
    assert_bf16(host64(b), o_ref, "bf16 partials")
    assert torch.equal(la, lb), "lse does not depend on the partial dtype"
    d = (b - a).abs().max().item()
    assert d <= 2.0 ** -8 * a.abs().max().item(), f"bf16 partial rounding {d}"


def test_single_token_generic_path(mla):
    """seq_len = 1 through the fp32-math path (H=20): o~ = c_0 bit-exactly."""
    inp = W.paged_attention(8, B=3, H=20, seq_lens=[1, 1, 1])
    say("single token generic")
    out, lse = run_attention(mla, inp, 1)
    out = out.cpu()
    bt = inp["block_table"]
    for b in range(3):
        want = inp["cache"][int(bt[b, 0]), 0, :512].float().expand_as(out[b])
        bad = (out[b] != want).nonzero()
        assert bad.numel() == 0, (f"seq {b}: {bad.shape[0]} mismatches, first at {bad[:4].tolist()}: "
                                  f"{[(out[b][tuple(i)].item(), want[tuple(i)].item()) for i in bad[:4]]}")


def test_deterministic(mla):
    inp = W.paged_attention(12, B=2, H=128, seq_lens=[3000, 1234])
    say("determinism")
    a, la = run_attention(mla, inp, 5)
    b, lb = run_attention(mla, inp, 5)
    assert torch.equal(a, b) and torch.equal(la, lb)


def test_bound_calls_match_wrappers(mla):
    """bind(): the pre-marshalled attention and combine calls produce bit-identical output
    to the checked wrappers, on repeated calls."""
    inp = W.paged_attention(14, B=3, H=128, seq_lens=[4096, 77, 1500])
    say("bound calls")
    ref, lref = run_attention(mla, inp, 4, part=torch.bfloat16)
    q_lat, q_pe, cache = dev(inp["q_lat"]), dev(inp["q_pe"]), dev(inp["cache"])
    bt, sl = dev(inp["block_table"]), dev(inp["seq_lens"])
    B, H, d_c = q_lat.shape
    o_part = torch.empty(B, H, 4, d_c, device="cuda", dtype=torch.bfloat16)
    lse_part = torch.empty(B, H, 4, device="cuda")
    out = torch.empty(B, H, d_c, device="cuda")
    lse = torch.empty(B, H, device="cuda")
    attn = mla.bind(mla.mla_decode_attn, q_lat, q_pe, cache, bt, sl, inp["scale"], 4, o_part,
                    lse_part)
    comb = mla.bind(mla.mla_splitk_combine, o_part, lse_part, out, lse)
    for _ in range(3):
        out.fill_(float("nan"))
        attn()
        comb()
        torch.cuda.synchronize()
        assert torch.equal(out, ref) and torch.equal(lse, lref)


def test_zero_query_and_ones_latent(mla):
    """q = 0: every weight is 1/T, o~ = mean of the latents.  All-ones latents: o~ = 1."""
    inp = W.paged_attention(13, B=2, H=32, seq_lens=[512, 1000])
    inp["q_lat"].zero_()
    inp["q_pe"].zero_()
    say("zero query")
    out, lse = run_attention(mla, inp, 2)
    o_ref, lse_ref = oracle_attention(inp)
    assert_fp32(host64(out), o_ref, 2e-5, "mean")
    assert_fp32(host64(lse), lse_ref, 1e-5, "lse = ln T")
    inp2 = W.paged_attention(14, B=2, H=32, seq_lens=[512, 1000])
    inp2["cache"][:, :, :512] = 1.0
    out, _ = run_attention(mla, inp2, 3)
    assert_fp32(host64(out), np.ones(out.shape), 1e-5, "ones")


def test_validate_indices(mla):
    say("validate indices")
    inp = W.paged_attention(15, B=3, H=16, seq_lens=[100, 64, 1])
    bt, sl = dev(inp["block_table"]), dev(inp["seq_lens"])
    cnt = torch.full((1,), -1, dtype=torch.int32, device="cuda")
    n = inp["cache"].shape[0]
    mla.mla_validate_indices(bt, sl, 64, n, cnt)
    torch.cuda.synchronize()
    assert cnt.item() == 0
    bt[0, 1] = n          # out of the pool
    sl[2] = 10 ** 6       # longer than the table allows
    mla.mla_validate_indices(bt, sl, 64, n, cnt)
    torch.cuda.synchronize()
    assert cnt.item() == 2


def test_stream_read_runs(mla):
    say("stream read")
    x = torch.ones(1 << 20, dtype=torch.uint8, device="cuda")
    sink = torch.zeros(4096, device="cuda")
    mla.mla_stream_read(x, sink)
    torch.cuda.synchronize()
    assert torch.isfinite(sink).all()


# ------------------------------------------------------------------ full decode layer
def layer_on_gpu(mla, x, S, stacked=False, fused=False, qpath=False, det=False, append_fused=False):
    """The whole decode layer through the C ABI: projections, cache append, absorption,
    attention + combine, W^UV and W^O.  stacked: the projections that share an input run as
    one product over their stacked weights ([W^DQ; W^DKV; W^KR] h, then [W^UQ; W^QR] c^Q
    with c^Q read in place), and the append and absorption read their inputs in place from
    those outputs through the row-strided entry points.  qpath (with stacked): the query
    side (W^UQ, W^QR, RoPE, absorption) is one mla_query_path launch instead.  det (with
    stacked and fused): the two remaining projections run with a fixed summation order.
    append_fused (with det): the cache append runs in the down-projection's summing launch
    (mla_linear_deterministic_append)."""
    s = x["shape"]
    B, H, d_h, d_c, d_R, d, d_cq = s.B, s.H, s.d_h, s.d_c, s.d_R, x["d"], x["d_cq"]
    w = {k: dev(v) for k, v in x["weights"].items()}
    h = dev(x["h"])
    cache = dev(x["cache"])
    bt, before = dev(x["block_table"]), dev(x["seq_lens_before"])
    seq_lens = before + 1
    f32 = dict(device="cuda", dtype=torch.float32)
    q_lat = torch.empty(B, H, d_c, device="cuda", dtype=torch.bfloat16)
    q_pe = torch.empty(B, H, d_R, device="cuda", dtype=torch.bfloat16)
    if stacked:
        w_a = torch.cat([w["w_dq"], w["w_dkv"], w["w_kr"]]).contiguous()
        w_b = torch.cat([w["w_uq"], w["w_qr"]]).contiguous()
        y_a = torch.empty(B, d_cq + d_c + d_R, **f32)
        y_b = torch.empty(B, H * (d_h + d_R), **f32)
        if det:
            ws_lin = torch.empty(max(mla.mla_linear_deterministic_workspace_bytes(B, w_a.shape[0], d),
                                     mla.mla_linear_deterministic_workspace_bytes(B, d, H * d_h)),
                                 dtype=torch.uint8, device="cuda")
            if append_fused:
                mla.mla_linear_deterministic_append(h, w_a, y_a, ws_lin, d_cq, before, bt, cache,
                                                    x["rope_base"])
            else:
                mla.mla_linear_deterministic(h, w_a, y_a, ws_lin)
        else:
            mla.mla_linear(h, w_a, y_a)
        if not append_fused:
            mla.mla_kv_append_strided(y_a[:, d_cq:d_cq + d_c].unsqueeze(1),
                                      y_a[:, d_cq + d_c:].unsqueeze(1), before, bt, cache,
                                      x["rope_base"])
        if qpath:  # the query side in one launch, c^Q read in place
            w_pack = mla.mla_pack_query_weights(w["w_uq"], w["w_qr"], w["w_uk"], H)
            mla.mla_query_path(y_a[:, :d_cq], w_pack, seq_lens, x["rope_base"], q_lat, q_pe)
        else:
            mla.mla_linear_strided(y_a[:, :d_cq], w_b, y_b)
            mla.mla_absorb_q_strided(y_b[:, :H * d_h].view(B, H, d_h), w["w_uk"],
                                     y_b[:, H * d_h:].view(B, H, d_R), seq_lens, x["rope_base"],
                                     q_lat, q_pe)
    else:
        c_q = torch.empty(B, d_cq, **f32)
        q_c = torch.empty(B, H * d_h, **f32)
        q_r = torch.empty(B, H * d_R, **f32)
        c_kv = torch.empty(B, d_c, **f32)
        k_r = torch.empty(B, d_R, **f32)
        mla.mla_linear(h, w["w_dq"], c_q)
        mla.mla_linear(c_q, w["w_uq"], q_c)
        mla.mla_linear(c_q, w["w_qr"], q_r)
        mla.mla_linear(h, w["w_dkv"], c_kv)
        mla.mla_linear(h, w["w_kr"], k_r)
        mla.mla_kv_append(c_kv.view(B, 1, d_c), k_r.view(B, 1, d_R), before, bt, cache,
                          x["rope_base"])
        mla.mla_absorb_q(q_c.view(B, H, d_h), w["w_uk"], q_r.view(B, H, d_R), seq_lens,
                         x["rope_base"], q_lat, q_pe)
    o_heads = torch.empty(B, H, d_h, **f32)
    u = torch.empty(B, d, **f32)
    if fused:  # attention, then the combine fused with W^UV, then W^O
        o_part = torch.empty(B, H, S, d_c, device="cuda", dtype=torch.bfloat16)
        lse_part = torch.empty(B, H, S, **f32)
        mla.mla_decode_attn(q_lat, q_pe, cache, bt, seq_lens, x["scale"], S, o_part, lse_part)
        mla.mla_combine_out_proj(o_part, lse_part, w["w_uv"], o_heads)
        if det:
            mla.mla_linear_deterministic(o_heads.view(B, H * d_h), w["w_o"], u, ws_lin)
        else:
            mla.mla_linear(o_heads.view(B, H * d_h), w["w_o"], u)
    else:
        ws = torch.empty(max(1, mla.mla_decode_workspace_bytes(B, H, d_c, S)), dtype=torch.uint8,
                         device="cuda")
        o_lat = torch.empty(B, H, d_c, **f32)
        mla.mla_decode(q_lat, q_pe, cache, bt, seq_lens, x["scale"], S, ws, o_lat)
        mla.mla_out_proj(o_lat, w["w_uv"], w["w_o"], o_heads, u)
    torch.cuda.synchronize()
    return u, cache


@pytest.mark.slow
@pytest.mark.parametrize("stacked,fused,qpath,det,append_fused",
                         [(False, False, False, False, False), (True, False, False, False, False),
                          (True, True, False, False, False), (True, True, True, True, False),
                          (True, True, True, True, True)],
                         ids=["separate", "stacked", "stacked-fused", "stacked-fused-qpath-det",
                              "bench-chain"])
def test_full_layer_b64_t2k_sampled(mla, stacked, fused, qpath, det, append_fused):
    """Full layer at d=5120, H=128, B=64, 2048 prior tokens + 1 appended: all 64 rows of
    u on the GPU; sequences 0 and 37 through the oracle's expanded path, and every one of
    the 64 sequences for the chain the bench times (bench-chain)."""
    x = W.layer_b64_t2k()
    say(f"layer_b64_t2k stacked={stacked} fused={fused} qpath={qpath} det={det} "
        f"append_fused={append_fused}")
    u, cache = layer_on_gpu(mla, x, S=4, stacked=stacked, fused=fused, qpath=qpath, det=det,
                            append_fused=append_fused)
    pick = list(range(64)) if append_fused else [0, 37]
    ref = oracle.decode_layer(W.to_f64(x["h"]), {k: W.to_f64(v) for k, v in x["weights"].items()},
                              W.to_f64(x["cache"]), x["block_table"].numpy(),
                              x["seq_lens_before"].numpy(), x["shape"].d_h, x["shape"].d_R,
                              x["rope_base"], x["scale"], batch_index=pick)
    m, r = assert_bf16(host64(u)[pick], ref["u"][pick], "layer u")
    print(f"layer_b64_t2k u: max-abs {m:.3e} rel-L2 {r:.3e}")
    # the appended rows: [c^KV ; RoPE(k^R, 2048)] rounded to bf16
    bt = x["block_table"]
    for b in pick:
        row = host64(cache[int(bt[b, 2048 // 64]), 2048 % 64])
        want = np.concatenate([ref["c_kv_new"][b], oracle.rope(ref["k_r_new"][b], 2048, 10000.0)])
        assert_bf16(row, want, "appended row")


@pytest.mark.parametrize("stacked,fused,qpath,det",
                         [(False, False, False, False), (True, False, False, False),
                          (True, True, False, False), (True, True, True, False),
                          (True, True, True, True)],
                         ids=["separate", "stacked", "stacked-fused", "stacked-fused-qpath",
                              "stacked-fused-qpath-det"])
def test_small_layer_chain(mla, stacked, fused, qpath, det):
    """A small layer (d=256, H=16, d_c=512, d_R=64, B=5, 100 prior tokens) end to end on all
    rows (d_c^Q = 384 where the one-launch query side runs, which needs a multiple of 384)."""
    x = W.layer_b64_t2k(seed=21, B=5, T=100, d=256, H=16, d_cq=384 if qpath else 96)
    say(f"small layer stacked={stacked} fused={fused} qpath={qpath} det={det}")
    u, _ = layer_on_gpu(mla, x, S=2, stacked=stacked, fused=fused, qpath=qpath, det=det)
    ref = oracle.decode_layer(W.to_f64(x["h"]), {k: W.to_f64(v) for k, v in x["weights"].items()},
                              W.to_f64(x["cache"]), x["block_table"].numpy(),
                              x["seq_lens_before"].numpy(), x["shape"].d_h, x["shape"].d_R,
                              x["rope_base"], x["scale"])
    assert_bf16(host64(u), ref["u"], "small layer u")


def test_layer_chain_reruns_bit_identical(mla):
    """The decode layer with the fixed-order projections (the append in the first one's
    summing launch), the one-launch query side and the fused combine: two runs from the same cache give u bit for bit (every sum in the chain
    has one order), at the DeepSeek-V2 sizes."""
    x = W.layer_b64_t2k()
    say("layer_b64_t2k rerun determinism")
    cache0 = x["cache"].clone()
    u1, _ = layer_on_gpu(mla, x, S=4, stacked=True, fused=True, qpath=True, det=True,
                         append_fused=True)
    x["cache"] = cache0
    u2, _ = layer_on_gpu(mla, x, S=4, stacked=True, fused=True, qpath=True, det=True,
                         append_fused=True)
    assert torch.equal(u1, u2)


def test_linear_and_outproj_against_matmul(mla):
    """Plain GEMMs against numpy fp64 matmul, including ragged tile edges."""
    g = torch.Generator().manual_seed(3)
    say("linear")
    for (M, N, K) in [(1, 1, 1), (7, 130, 67), (64, 512, 5120), (65, 64, 33)]:
        x = torch.randn(M, K, generator=g)
        w = torch.randn(N, K, generator=g).to(torch.bfloat16)
        y = torch.empty(M, N, device="cuda")
        mla.mla_linear(dev(x), dev(w), y)
        torch.cuda.synchronize()
        ref = W.to_f64(x) @ W.to_f64(w).T
        m, _ = errors(host64(y), ref)
        assert m <= 1e-5 * math.sqrt(K) * 4, (M, N, K, m)


def test_weight_streaming_gemm_paths(mla):
    """The bf16-weight MFMA GEMM (weights [out, in], k a multiple of 128) against numpy
    fp64 matmul over its tile widths, k splits (atomic accumulation), ragged rows and
    columns, bf16 activations and more than 64 rows.  x is fp32 (split hi + lo) or bf16."""
    g = torch.Generator().manual_seed(31)
    for (M, N, K, xdt) in [(64, 5120, 16384, torch.float32),   # wide tiles, 16-way k split
                           (50, 1000, 1536, torch.float32),    # narrow tiles, ragged N
                           (100, 300, 256, torch.bfloat16),    # two row blocks, bf16 x
                           (3, 16, 128, torch.float32)]:       # one chunk
        say(f"weight-streaming GEMM M={M} N={N} K={K} x={xdt}")
        x = torch.randn(M, K, generator=g).to(xdt)
        w = torch.randn(N, K, generator=g).to(torch.bfloat16)
        y = torch.empty(M, N, device="cuda")
        mla.mla_linear(dev(x), dev(w), y)
        torch.cuda.synchronize()
        ref = W.to_f64(x) @ W.to_f64(w).T
        m, r = errors(host64(y), ref)
        # x keeps ~16 significant bits (hi + lo), products are exact, sums are fp32
        assert m <= 2e-5 * float(np.abs(ref).max()) + 1e-4, (M, N, K, m)
        assert r <= 1e-5, (M, N, K, r)


def test_linear_planned_kernels(mla):
    """Both weight-streaming kernels over explicit plans against numpy fp64 matmul: the
    persistent kernel with k slices per XCD (grids that are multiples of 8) and without,
    runs that cross column-tile boundaries, odd runs, ragged M, bf16 and fp32 x, every ring
    depth; the tile-grid kernel over its tile widths, k splits and rings.  Invalid plans are
    refused without launching."""
    g = torch.Generator().manual_seed(34)
    cases = [  # (M, N, K, x dtype, [(kernel, tile, split, ring), ...])
        (64, 1536, 5120, torch.bfloat16, [(1, 1, 240, 16), (1, 2, 240, 8), (1, 4, 240, 4),
                                          (1, 1, 160, 12), (0, 1, 8, 20), (0, 2, 4, 4)]),
        (50, 1024, 1536, torch.float32, [(1, 2, 96, 4), (1, 1, 96, 8), (1, 4, 12, 4),
                                         (1, 2, 48, 8), (0, 2, 2, 12), (0, 4, 3, 4)]),
        (64, 512, 640, torch.float32, [(1, 1, 8, 4), (1, 1, 10, 16), (1, 1, 40, 4),
                                       (1, 2, 20, 4), (0, 1, 5, 4)]),
        (7, 128, 256, torch.bfloat16, [(1, 2, 2, 4), (1, 1, 4, 4), (1, 1, 1, 8), (0, 1, 2, 4)]),
        # activation-stationary: slices of 256 / 384 / 512 k, runs of 1 to 4 tiles, two-tile
        # waves, ragged M, bf16 x with 640-wide slices (copies spanning two rows)
        (64, 2048, 1536, torch.float32, [(2, 1, 64, 12), (2, 1, 32, 12), (2, 1, 48, 16),
                                         (2, 2, 24, 8), (2, 2, 16, 12), (2, 1, 96, 8)]),
        (33, 1024, 5120, torch.bfloat16, [(2, 1, 64, 20), (2, 1, 80, 16), (2, 2, 40, 8),
                                          (2, 1, 8, 20)]),
    ]
    for (M, N, K, xdt, plans) in cases:
        x = torch.randn(M, K, generator=g).to(xdt)
        w = torch.randn(N, K, generator=g).to(torch.bfloat16)
        ref = W.to_f64(x) @ W.to_f64(w).T
        xd, wd = dev(x), dev(w)
        for (kernel, tile, split, ring) in plans:
            say(f"planned GEMM M={M} N={N} K={K} x={xdt} kernel={kernel} plan=({tile},{split},{ring})")
            y = torch.full((M, N), float("nan"), device="cuda")
            mla.mla_linear_planned(xd, wd, y, kernel, tile, split, ring)
            torch.cuda.synchronize()
            m, r = errors(host64(y), ref)
            assert m <= 2e-5 * float(np.abs(ref).max()) + 1e-4, (M, N, K, kernel, tile, split, ring, m)
            assert r <= 1e-5, (M, N, K, kernel, tile, split, ring, r)
    # plans the kernels cannot take are refused (nothing launched, y untouched)
    x = dev(torch.randn(64, 1536, generator=g))
    w = dev(torch.randn(1024, 1536, generator=g).to(torch.bfloat16))
    y = torch.zeros(64, 1024, device="cuda")
    for bad in [(1, 4, 7, 4), (1, 2, 512, 4), (1, 4, 96, 8), (1, 3, 96, 4), (0, 2, 5, 4),
                (0, 4, 2, 16), (2, 1, 7, 12), (2, 1, 32, 20), (2, 4, 8, 8), (3, 1, 1, 4)]:
        with pytest.raises(mla.MLAError):
            mla.mla_linear_planned(x, w, y, *bad)
    torch.cuda.synchronize()
    assert float(y.abs().max()) == 0.0


def test_offline_absorption_gemm(mla):
    """Offline absorption (W~_i = W^UK_i^T W^UQ_i, prepared once in fp64 and rounded to
    bf16) through mla_linear gives the absorbed query of the oracle (W^UK_i^T (W^UQ c^Q)_i
    in fp64) within the bf16 bar: the weight is the only rounding."""
    g = torch.Generator().manual_seed(35)
    B, H, d_h, d_c, d_cq = 8, 4, 128, 512, 1536
    say("offline absorption")
    c_q = torch.randn(B, d_cq, generator=g)
    w_uq = (torch.randn(H * d_h, d_cq, generator=g) / math.sqrt(d_cq)).to(torch.bfloat16)
    w_uk = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_h)).to(torch.bfloat16)
    wuk, wuq = W.to_f64(w_uk), W.to_f64(w_uq)
    w_off = np.concatenate([wuk[i * d_h:(i + 1) * d_h].T @ wuq[i * d_h:(i + 1) * d_h]
                            for i in range(H)])
    w_off = torch.from_numpy(w_off).to(torch.bfloat16)
    y = torch.empty(B, H * d_c, device="cuda")
    mla.mla_linear(dev(c_q), dev(w_off), y)
    torch.cuda.synchronize()
    q_c = oracle.linear(W.to_f64(c_q), wuq).reshape(B, H, d_h)
    ref = np.stack([oracle.absorb_query(q_c[b], wuk) for b in range(B)]).reshape(B, H * d_c)
    assert_bf16(host64(y), ref, "offline q~")


def test_out_proj_full_size(mla):
    """W^UV per head (batched, strided) then W^O at the DeepSeek-V2 sizes, fp64 reference."""
    g = torch.Generator().manual_seed(32)
    B, H, d_h, d_c, d_model = 64, 128, 128, 512, 5120
    say("out_proj full size")
    o_lat = torch.randn(B, H, d_c, generator=g)
    w_uv = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_c)).to(torch.bfloat16)
    w_o = (torch.randn(d_model, H * d_h, generator=g) / math.sqrt(H * d_h)).to(torch.bfloat16)
    o_heads = torch.empty(B, H, d_h, device="cuda")
    u = torch.empty(B, d_model, device="cuda")
    mla.mla_out_proj(dev(o_lat), dev(w_uv), dev(w_o), o_heads, u)
    torch.cuda.synchronize()
    ref_heads = np.stack([W.to_f64(o_lat[:, i]) @ W.to_f64(w_uv[i * d_h:(i + 1) * d_h]).T
                          for i in range(H)], axis=1)
    assert_fp32(host64(o_heads), ref_heads, 1e-4, "o_heads")
    ref_u = ref_heads.reshape(B, H * d_h) @ W.to_f64(w_o).T
    m, r = errors(host64(u), ref_u)
    assert r <= 1e-5 and m <= 1e-4, (m, r)


def test_absorb_mfma_against_oracle(mla):
    """Query absorption on the MFMA path (bf16 W^UK, bf16 q~, d_h = 128) against the
    oracle's absorption in fp64: ragged batch (B = 70: a full and a partial 64-row block),
    four 128-column blocks; q~ is rounded once to bf16.  Then with q^R, whose RoPE the same
    call applies, against the oracle's RoPE at ragged positions."""
    g = torch.Generator().manual_seed(33)
    B, H, d_h, d_c = 70, 6, 128, 512
    say("absorb mfma")
    q_c = torch.randn(B, H, d_h, generator=g)
    w_uk = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_h)).to(torch.bfloat16)
    q_lat = torch.empty(B, H, d_c, device="cuda", dtype=torch.bfloat16)
    seq_lens = torch.full((B,), 5, dtype=torch.int32, device="cuda")
    mla.mla_absorb_q(dev(q_c), dev(w_uk), None, seq_lens, 10000.0, q_lat, None)
    torch.cuda.synchronize()
    ref = np.stack([oracle.absorb_query(W.to_f64(q_c[b]), W.to_f64(w_uk)) for b in range(B)])
    assert_bf16(host64(q_lat), ref, "q~")
    # the bf16 output is the only rounding: within half a bf16 ulp of the fp64 value
    m, _ = errors(host64(q_lat), ref)
    assert m <= float(np.abs(ref).max()) * 2.0 ** -8, m
    # with q^R: the same launch also rotates q_pe at position seq_len - 1 (ragged lengths)
    d_R = 64
    q_r = torch.randn(B, H, d_R, generator=g)
    seq_lens = torch.randint(1, 5000, (B,), generator=g, dtype=torch.int32)
    q_lat2 = torch.empty(B, H, d_c, device="cuda", dtype=torch.bfloat16)
    q_pe = torch.empty(B, H, d_R, device="cuda", dtype=torch.bfloat16)
    mla.mla_absorb_q(dev(q_c), dev(w_uk), dev(q_r), dev(seq_lens), 10000.0, q_lat2, q_pe)
    torch.cuda.synchronize()
    assert torch.equal(q_lat2.cpu(), q_lat.cpu())
    ref_pe = np.stack([oracle.rope(W.to_f64(q_r[b]), int(seq_lens[b]) - 1) for b in range(B)])
    assert_bf16(host64(q_pe), ref_pe, "q_pe")
    m, _ = errors(host64(q_pe), ref_pe)
    assert m <= float(np.abs(ref_pe).max()) * 2.0 ** -8, m


def test_strided_entry_points(mla):
    """The row-strided entry points on views into wider buffers.  mla_linear_strided
    against numpy fp64 matmul on each kernel family (persistent, activation-stationary,
    tile-grid, fp32 VALU), then again with accumulate on top of that result, with the
    columns of y's buffer outside the view left untouched;
    mla_kv_append_strided and mla_absorb_q_strided bit-identical to their dense forms on
    the same values (same kernels, same arithmetic), the query RoPE done inside the
    absorption kernel bit-identical to the RoPE kernel, and the absorption with a row stride
    the MFMA path cannot take (not a multiple of 4) against the oracle."""
    g = torch.Generator().manual_seed(77)
    for (M, N, K, xdt) in [(64, 2112, 5120, torch.float32),    # [W^DQ; W^DKV; W^KR] shape
                           (64, 24576, 1536, torch.float32),   # [W^UQ; W^QR] shape
                           (5, 192, 256, torch.bfloat16),
                           (100, 320, 384, torch.float32),    # two row blocks
                           (3, 70, 33, torch.float32)]:
        say(f"linear strided M={M} N={N} K={K} x={xdt}")
        xb = torch.randn(M, K + 24, generator=g).to(xdt)
        w = (torch.randn(N, K, generator=g) / math.sqrt(K)).to(torch.bfloat16)
        yb = torch.full((M, N + 40), 7.0, device="cuda")
        mla.mla_linear_strided(dev(xb)[:, 8:8 + K], dev(w), yb[:, 16:16 + N])
        torch.cuda.synchronize()
        ref = W.to_f64(xb[:, 8:8 + K]) @ W.to_f64(w).T
        m, r = errors(host64(yb[:, 16:16 + N]), ref)
        assert m <= 2e-5 * float(np.abs(ref).max()) + 1e-4 and r <= 1e-5, (M, N, K, m, r)
        assert bool((yb[:, :16] == 7.0).all()) and bool((yb[:, 16 + N:] == 7.0).all())
        # accumulate: y += x w^T on top of the first result (no zero fill), so y = 2 x w^T
        mla.mla_linear_strided(dev(xb)[:, 8:8 + K], dev(w), yb[:, 16:16 + N], accumulate=True)
        torch.cuda.synchronize()
        m, r = errors(host64(yb[:, 16:16 + N]), 2 * ref)
        assert m <= 4e-5 * float(np.abs(ref).max()) + 2e-4 and r <= 1e-5, ("acc", M, N, K, m, r)
        assert bool((yb[:, :16] == 7.0).all()) and bool((yb[:, 16 + N:] == 7.0).all())

    # cache append: c^KV and k^R as column ranges of one [B, n, 1536 + 576 + 8] buffer
    B, n, d_c, d_R, P = 6, 3, 512, 64, 16
    say("kv_append strided")
    src = torch.randn(B, n, 1536 + d_c + d_R + 8, generator=g)
    before = torch.tensor([0, 5, 16, 29, 47, 60], dtype=torch.int32)
    bt = torch.randperm(B * 5, generator=g).to(torch.int32).view(B, 5)
    caches = [torch.zeros(B * 5, P, d_c + d_R, device="cuda", dtype=torch.bfloat16) for _ in range(2)]
    s_dev = dev(src)
    mla.mla_kv_append_strided(s_dev[:, :, 1536:1536 + d_c], s_dev[:, :, 1536 + d_c:1536 + d_c + d_R],
                              dev(before), dev(bt), caches[0], 10000.0)
    mla.mla_kv_append(dev(src[:, :, 1536:1536 + d_c]), dev(src[:, :, 1536 + d_c:1536 + d_c + d_R]),
                      dev(before), dev(bt), caches[1], 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(caches[0].cpu(), caches[1].cpu())
    assert int((caches[0] != 0).any(-1).sum()) == B * n

    # absorption: q^C and q^R as the two column ranges of one [B, H (d_h + d_R) + pad] buffer
    B, H, d_h = 70, 6, 128
    w_uk = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_h)).to(torch.bfloat16)
    seq_lens = torch.randint(1, 5000, (B,), generator=g, dtype=torch.int32)
    for pad, out_dt in [(8, torch.bfloat16), (8, torch.float32), (2, torch.bfloat16)]:
        say(f"absorb strided pad={pad} out={out_dt}")
        yb = torch.randn(B, H * (d_h + d_R) + pad, generator=g)
        yd = dev(yb)
        q_c, q_r = yd[:, :H * d_h].view(B, H, d_h), yd[:, H * d_h:H * (d_h + d_R)].view(B, H, d_R)
        outs = [(torch.empty(B, H, d_c, device="cuda", dtype=out_dt),
                 torch.empty(B, H, d_R, device="cuda", dtype=out_dt)) for _ in range(2)]
        mla.mla_absorb_q_strided(q_c, dev(w_uk), q_r, dev(seq_lens), 10000.0, *outs[0])
        torch.cuda.synchronize()
        ref_pe = np.stack([oracle.rope(W.to_f64(q_r[b].cpu()), int(seq_lens[b]) - 1)
                           for b in range(B)])
        if pad % 4 == 0:
            mla.mla_absorb_q(q_c.contiguous(), dev(w_uk), q_r.contiguous(), dev(seq_lens), 10000.0,
                             *outs[1])
            torch.cuda.synchronize()
            assert torch.equal(outs[0][0].cpu(), outs[1][0].cpu())
            assert torch.equal(outs[0][1].cpu(), outs[1][1].cpu())
        if pad == 8 and out_dt == torch.bfloat16:
            # q^R at an odd row stride cannot ride along in the absorption kernel: the RoPE
            # then runs as its own kernel and must give the same bits as the fused one
            odd = torch.empty(B, H * d_R + 1, device="cuda")
            odd[:, :H * d_R] = q_r.reshape(B, H * d_R)
            sep = torch.empty(B, H, d_R, device="cuda", dtype=out_dt)
            mla.mla_absorb_q_strided(q_c, dev(w_uk), odd[:, :H * d_R].view(B, H, d_R),
                                     dev(seq_lens), 10000.0, outs[1][0], sep)
            torch.cuda.synchronize()
            assert torch.equal(sep.cpu(), outs[0][1].cpu())
            assert torch.equal(outs[1][0].cpu(), outs[0][0].cpu())
        ref = np.stack([oracle.absorb_query(W.to_f64(q_c[b].cpu()), W.to_f64(w_uk))
                        for b in range(B)])
        assert_bf16(host64(outs[0][0]), ref, "q~ strided")
        assert_bf16(host64(outs[0][1]), ref_pe, "q_pe strided")


@pytest.mark.parametrize("B,H,S,pdt", [(37, 8, 5, torch.bfloat16),   # ragged blocks, 2 chunks
                                       (20, 6, 64, torch.float32),   # H % 8 != 0, most splits
                                       (64, 16, 4, torch.bfloat16),  # the layer's shape class
                                       (1, 8, 1, torch.bfloat16),    # one row, one split
                                       (70, 64, 6, torch.bfloat16),  # 32-row blocks, ragged
                                       (40, 128, 3, torch.float32)]) # 32-row blocks, fp32
def test_combine_out_proj(mla, B, H, S, pdt):
    """The combine fused with W^UV against the oracle's combine and up-projection in fp64 on
    seeded partials: ragged sequence blocks of 16 and of 32 (the kernel takes 32 once 16-row
    blocks would exceed one workgroup per CU), both head numberings, 1 to 64 splits, empty
    splits (lse = -inf) holding NaN that must not leak, and one (sequence, head) with no
    tokens at all (o = 0).  Then against the unfused pair (mla_splitk_combine, mla_out_proj)
    on the same inputs."""
    g = torch.Generator().manual_seed(90 + S)
    d_c, d_h = 512, 128
    say(f"combine_out_proj B={B} H={H} S={S} {pdt}")
    o_part = torch.randn(B, H, S, d_c, generator=g)
    lse = torch.randn(B, H, S, generator=g) * 3
    empty = torch.rand(B, H, S, generator=g) < 0.2
    if B > 1:
        empty[1, 2, :] = True
    lse[empty] = -math.inf
    o_part = o_part.to(pdt)
    w_uv = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_c)).to(torch.bfloat16)
    # weight-0 splits do not enter the sum: the oracle gets zeros there, the GPU gets NaN
    o_ref = W.to_f64(o_part)
    o_ref[empty.numpy()] = 0.0
    o_gpu = o_part.clone()
    o_gpu[empty] = float("nan")
    o_comb, _ = oracle.combine_splits(np.moveaxis(o_ref, 2, 0), np.moveaxis(W.to_f64(lse), 2, 0))
    ref = oracle.up_project_values(o_comb, W.to_f64(w_uv))
    out = torch.empty(B, H, d_h, device="cuda")
    mla.mla_combine_out_proj(dev(o_gpu), dev(lse), dev(w_uv), out)
    torch.cuda.synchronize()
    m, r = errors(host64(out), ref)
    # o~ carried as hi + lo bf16 (about 16 bits), exact products, fp32 sums over 512
    assert r <= 1e-5 and m <= 1e-5 * float(np.abs(ref).max()) + 1e-6, (m, r)
    if B > 1:
        assert bool((out[1, 2] == 0).all())
    # the unfused pair on the same partials
    o_lat = torch.empty(B, H, d_c, device="cuda")
    o_h2 = torch.empty(B, H, d_h, device="cuda")
    mla.mla_splitk_combine(dev(o_gpu), dev(lse), o_lat)
    mla.mla_out_proj(o_lat, dev(w_uv), None, o_h2)
    torch.cuda.synchronize()
    m2, r2 = errors(host64(out), host64(o_h2))
    assert r2 <= 1e-5, (m2, r2)
