"""GPU parity of each bf16 MFMA attention kernel, chosen explicitly through
mla_decode_attn_planned: "heads" (16 heads per wavefront for both products), "cols"
(the latent product partitioned by columns, 128 heads) and "wide" (32 heads per wavefront on
the 32 x 32 x 16 MFMA, 128 heads).  Each kernel against the fp64
oracle on the same seeded inputs; indexing (which tokens are read) bit-exact."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import assert_bf16, dev, errors, host64, say

pytestmark = pytest.mark.gpu

KERNELS = ["heads", "cols", "wide"]


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_15_amd as m
    return m


def attend(mla, inp, S, kernel, part=torch.float32, q_lat=None, q_pe=None):
    """Planned attention (+ combine for S > 1); q_lat / q_pe default to the problem's.
    Returns the combined o~ [rows, H, d_c] and lse [rows, H] (rows = B, or B n_q)."""
    q_lat = dev(inp["q_lat"] if q_lat is None else q_lat)
    q_pe = dev(inp["q_pe"] if q_pe is None else q_pe)
    cache, bt, sl = dev(inp["cache"]), dev(inp["block_table"]), dev(inp["seq_lens"])
    rows = q_lat.shape[0] * (q_lat.shape[1] if q_lat.dim() == 4 else 1)
    H, d_c = q_lat.shape[-2], q_lat.shape[-1]
    o_part = torch.empty(rows, H, S, d_c, device="cuda", dtype=part if S > 1 else torch.float32)
    lse_part = torch.empty(rows, H, S, device="cuda")
    mla.mla_decode_attn_planned(q_lat, q_pe, cache, bt, sl, inp["scale"], S, o_part, lse_part,
                                kernel=kernel)
    if S == 1:
        torch.cuda.synchronize()
        return o_part.view(rows, H, d_c), lse_part.view(rows, H)
    out = torch.empty(rows, H, d_c, device="cuda")
    lse = torch.empty(rows, H, device="cuda")
    mla.mla_splitk_combine(o_part, lse_part, out, lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_attention(inp, batch_index=None):
    P = inp["cache"].shape[1]
    bt = inp["block_table"].numpy()
    sl = inp["seq_lens"].numpy()
    idx = range(inp["q_lat"].shape[0]) if batch_index is None else batch_index
    o, lse = [], []
    for b in idx:
        rows = oracle.gather_rows(W.to_f64(inp["cache"][torch.from_numpy(np.maximum(bt[b], 0)).long()]),
                                  np.arange(bt.shape[1]), int(sl[b]), P)
        att = oracle.latent_attention(W.to_f64(inp["q_lat"][b]), W.to_f64(inp["q_pe"][b]), rows,
                                      inp["shape"].d_c, inp["scale"])
        o.append(att["o_lat"])
        lse.append(att["lse"])
    return np.stack(o), np.stack(lse)


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("S,part", [(1, torch.float32), (3, torch.float32), (8, torch.bfloat16),
                                    (64, torch.bfloat16)])
def test_ragged_against_oracle(mla, kernel, S, part):
    """One-token, sub-tile, mid-page and multi-page sequences over permuted pages, with
    fp32 and bf16 partials and splits past the end of the short sequences."""
    inp = W.paged_attention(200, B=5, H=128, seq_lens=[1, 31, 33, 700, 2050])
    say(f"kernel={kernel} ragged S={S} part={part}")
    out, lse = attend(mla, inp, S, kernel, part)
    o_ref, lse_ref = oracle_attention(inp)
    assert_bf16(host64(out), o_ref, f"{kernel} S={S}")
    assert errors(host64(lse), lse_ref)[0] <= 2e-2
    assert torch.isfinite(lse).all()


@pytest.mark.parametrize("kernel", KERNELS)
def test_kernels_agree_closely(mla, kernel):
    """Both kernels compute the same bf16-weighted sums in a different order: their
    outputs agree far inside the oracle tolerance."""
    inp = W.paged_attention(201, B=3, H=128, seq_lens=[4096, 1000, 65])
    say(f"kernel={kernel} agreement")
    a, la = attend(mla, inp, 4, "heads")
    b, lb = attend(mla, inp, 4, kernel)
    m, r = errors(host64(b), host64(a))
    assert m <= 2e-3 and r <= 1e-3, (m, r)
    assert errors(host64(lb), host64(la))[0] <= 1e-4


def _spike_inputs(seq_lens, spikes, heads_hit, seed=7):
    """Random queries except heads `heads_hit`, whose q~ = 0 and q_pe = 64 e_0; row j* of
    each sequence has k^R[0] = 64 and every other row k^R[0] = 0, so those heads give
    weight 1 to j* and exactly 0 elsewhere (scores ~296 apart), far above any first-tile
    reference: they take the exact fallback while the other heads stay on the MFMA path."""
    inp = W.paged_attention(seed, B=len(seq_lens), H=128, seq_lens=seq_lens)
    inp["cache"][:, :, 512] = 0
    for h in heads_hit:
        inp["q_lat"][:, h].zero_()
        inp["q_pe"][:, h].zero_()
        inp["q_pe"][:, h, 0] = 64.0
    bt = inp["block_table"]
    for b, j in enumerate(spikes):
        inp["cache"][int(bt[b, j // 64]), j % 64, 512] = 64.0
    return inp


@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("S", [1, 4])
def test_spike_exact_on_some_heads(mla, kernel, S):
    """Spike heads select the latent row bit-exactly on both sides of page boundaries;
    the other heads of the same workgroups still match the oracle."""
    seq_lens = [64, 65, 128, 129, 300, 1000, 4096]
    spikes = [63, 64, 127, 128, 0, 999, 4095]
    hit = list(range(48, 64)) + [5, 127]
    inp = _spike_inputs(seq_lens, spikes, hit)
    say(f"kernel={kernel} spike S={S}")
    out, _ = attend(mla, inp, S, kernel)
    out = out.cpu()
    bt = inp["block_table"]
    for b, j in enumerate(spikes):
        want = inp["cache"][int(bt[b, j // 64]), j % 64, :512].float()
        for h in hit:
            assert torch.equal(out[b, h], want), f"seq {b} head {h} token {j}"
    rest = [h for h in range(128) if h not in hit]
    o_ref, _ = oracle_attention(inp)
    assert_bf16(host64(out)[:, rest], o_ref[:, rest], f"{kernel} other heads")


@pytest.mark.parametrize("kernel", KERNELS)
def test_single_token_bit_exact(mla, kernel):
    """seq_len = 1: the weight is exactly 1, o~ = c_0 bit-exactly, lse = the score."""
    inp = W.paged_attention(8, B=4, H=128, seq_lens=[1, 1, 1, 1])
    say(f"kernel={kernel} single token")
    out, _ = attend(mla, inp, 1, kernel)
    out = out.cpu()
    bt = inp["block_table"]
    for b in range(4):
        want = inp["cache"][int(bt[b, 0]), 0, :512].float().expand_as(out[b])
        assert torch.equal(out[b], want), f"seq {b}"


@pytest.mark.parametrize("kernel", KERNELS)
def test_nan_poison_and_page_permutation(mla, kernel):
    """NaN in unreferenced pages and in slots at or past seq_len is never read; moving
    pages in the pool (and the table with them) changes no bit."""
    inp = W.paged_attention(10, B=3, H=128, seq_lens=[70, 129, 500], extra_pages=3,
                            permute_pages=False)
    say(f"kernel={kernel} nan poison / permutation")
    clean, lc = attend(mla, inp, 3, kernel, torch.bfloat16)
    cache = inp["cache"].clone()
    bt = inp["block_table"]
    used = set(int(v) for v in bt.flatten().tolist() if v >= 0)
    for p in range(cache.shape[0]):
        if p not in used:
            cache[p] = float("nan")
    for b, L in enumerate(inp["seq_lens"].tolist()):
        cache[int(bt[b, (L - 1) // 64]), (L - 1) % 64 + 1:] = float("nan")
    dirty, ld = attend(mla, dict(inp, cache=cache), 3, kernel, torch.bfloat16)
    assert torch.equal(clean, dirty) and torch.equal(lc, ld)
    perm = torch.randperm(cache.shape[0], generator=torch.Generator().manual_seed(1))
    moved = torch.empty_like(cache)
    moved[perm] = cache
    bt2 = bt.clone()
    m = bt2 >= 0
    bt2[m] = perm[bt2[m].long()].to(torch.int32)
    again, la = attend(mla, dict(inp, cache=moved, block_table=bt2), 3, kernel, torch.bfloat16)
    assert torch.equal(clean, again) and torch.equal(lc, la)


@pytest.mark.parametrize("kernel", KERNELS)
def test_zero_query_mean(mla, kernel):
    """q = 0: all weights are equal, so o~ = the mean of the latents and lse = ln T."""
    inp = W.paged_attention(13, B=2, H=128, seq_lens=[512, 1000])
    inp["q_lat"].zero_()
    inp["q_pe"].zero_()
    say(f"kernel={kernel} zero query")
    out, lse = attend(mla, inp, 2, kernel)
    o_ref, lse_ref = oracle_attention(inp)
    assert errors(host64(out), o_ref)[0] <= 2e-5
    assert errors(host64(lse), lse_ref)[0] <= 1e-5


@pytest.mark.parametrize("kernel", KERNELS)
def test_multi_token(mla, kernel):
    """n_q = 3 new tokens per sequence, causal among them; a sequence shorter than n_q
    (its first query sees nothing and returns exactly 0)."""
    n_q = 3
    inp = W.paged_attention(44, B=4, H=128, seq_lens=[2, 97, 700, 1537])
    q_lat, q_pe = W.multi_queries(45, 4, n_q, 128)
    o_ref, _ = oracle.paged_decode_multi(W.to_f64(q_lat), W.to_f64(q_pe), W.to_f64(inp["cache"]),
                                         inp["block_table"].numpy(), inp["seq_lens"].numpy(),
                                         n_q, 512, inp["scale"])
    for S, part in [(1, torch.float32), (8, torch.bfloat16)]:
        say(f"kernel={kernel} multi-token S={S}")
        out, _ = attend(mla, inp, S, kernel, part, q_lat=q_lat, q_pe=q_pe)
        out = out.view(4, n_q, 128, 512)
        assert_bf16(host64(out), o_ref, f"{kernel} S={S}")
        assert float(out[0, 0].abs().max()) == 0.0


@pytest.mark.parametrize("kernel", ["cols", "wide"])
def test_128_head_kernels_reject_other_head_counts(mla, kernel):
    inp = W.paged_attention(3, B=1, H=64, seq_lens=[100])
    say(f"{kernel} rejects H=64")
    with pytest.raises(mla.MLAError):
        attend(mla, inp, 1, kernel)


@pytest.mark.slow
@pytest.mark.parametrize("kernel", KERNELS)
@pytest.mark.parametrize("part", [torch.float32, torch.bfloat16], ids=["f32part", "bf16part"])
def test_dsv2_b32_t4k_full(mla, kernel, part):
    """The headline shape B=32, T=4096, H=128 at the suggested split count, every output
    against the oracle, with fp32 and with bf16 partials."""
    inp = W.dsv2_b32_t4k()
    S = mla.mla_suggest_num_splits(32, 4096, 0, 64, 256)
    say(f"kernel={kernel} dsv2_b32_t4k S={S} part={part}")
    out, lse = attend(mla, inp, S, kernel, part)
    o_ref, lse_ref = oracle_attention(inp)
    m, r = assert_bf16(host64(out), o_ref, f"{kernel} dsv2_b32_t4k")
    print(f"{kernel} dsv2_b32_t4k ({part}): max-abs {m:.3e} rel-L2 {r:.3e}")
    assert errors(host64(lse), lse_ref)[0] <= 2e-2
