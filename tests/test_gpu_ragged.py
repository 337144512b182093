"""GPU parity of mla_decode_ragged, the flattened work list for ragged batches: the batch's
cached pages, concatenated, are cut into one equal range per compute unit, and a combine
kernel merges each sequence's pieces.  Every sequence of the ragged 128-sequence workload
against the fp64 oracle; empty and one-token sequences; spikes on both sides of piece
boundaries select their latent row bit-exactly."""
import numpy as np
import pytest
import torch

import oracle
import workloads as W
from tests.gpu_util import assert_bf16, dev, errors, host64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_15_amd as m
    return m


def ragged(mla, inp):
    q_lat, q_pe = dev(inp["q_lat"]), dev(inp["q_pe"])
    cache, bt, sl = dev(inp["cache"]), dev(inp["block_table"]), dev(inp["seq_lens"])
    B, H, d_c = q_lat.shape
    nbytes = mla.mla_decode_ragged_workspace_bytes(cache, bt, H, d_c)
    ws = torch.full((nbytes,), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.full((B, H, d_c), float("nan"), device="cuda")
    lse = torch.full((B, H), float("nan"), device="cuda")
    mla.mla_decode_ragged(q_lat, q_pe, cache, bt, sl, inp["scale"], ws, out, lse)
    torch.cuda.synchronize()
    err = int(ws[8 * B:8 * B + 4].view(torch.int32).item())
    return out, lse, err


def oracle_attention(inp, batch_index=None):
    P = inp["cache"].shape[1]
    bt = inp["block_table"].numpy()
    sl = inp["seq_lens"].numpy()
    idx = range(inp["q_lat"].shape[0]) if batch_index is None else batch_index
    o, lse = [], []
    for b in idx:
        n = int(sl[b])
        if n == 0:
            o.append(np.zeros((inp["q_lat"].shape[1], inp["shape"].d_c)))
            lse.append(np.full(inp["q_lat"].shape[1], -np.inf))
            continue
        pages = bt[b, :(n + P - 1) // P].astype(np.int64)
        rows = oracle.gather_rows(W.to_f64(inp["cache"][torch.from_numpy(pages)]),
                                  np.arange(len(pages)), n, P)
        att = oracle.latent_attention(W.to_f64(inp["q_lat"][b]), W.to_f64(inp["q_pe"][b]), rows,
                                      inp["shape"].d_c, inp["scale"])
        o.append(att["o_lat"])
        lse.append(att["lse"])
    return np.stack(o), np.stack(lse)


def test_ragged_b128_every_sequence(mla):
    """The ragged workload (128 sequences, lengths uniform in 128 .. 8192, shuffled pool):
    every output of every sequence against the oracle."""
    inp = W.ragged_b128()
    say("ragged_b128 all sequences")
    out, lse, err = ragged(mla, inp)
    assert err == 0
    o_ref, lse_ref = oracle_attention(inp)
    m, r = assert_bf16(host64(out), o_ref, "ragged_b128")
    print(f"ragged_b128: max-abs {m:.3e} rel-L2 {r:.3e}")
    assert errors(host64(lse), lse_ref)[0] <= 2e-2


@pytest.mark.parametrize("H", [128, 64, 16])
def test_ragged_edge_lengths(mla, H):
    """Empty sequences (o = 0, lse = -inf), one-token, sub-tile, page-edge and long
    sequences in one batch of more than 64 sequences (several scan chunks)."""
    lens = [0, 1, 31, 32, 63, 64, 65, 127, 128, 129, 4095, 4096, 4097, 20000, 0, 3] * 5
    inp = W.paged_attention(400 + H, B=len(lens), H=H, seq_lens=lens)
    say(f"ragged edge lengths H={H}")
    out, lse, err = ragged(mla, inp)
    assert err == 0
    o_ref, lse_ref = oracle_attention(inp)
    empty = [b for b, n in enumerate(lens) if n == 0]
    full = [b for b, n in enumerate(lens) if n > 0]
    assert float(out[empty].abs().max()) == 0.0
    assert torch.isinf(lse[empty]).all() and (lse[empty] < 0).all()
    assert_bf16(host64(out)[full], o_ref[full], f"ragged edges H={H}")
    assert errors(host64(lse)[full], lse_ref[full])[0] <= 2e-2


def test_ragged_single_token_bit_exact(mla):
    """seq_len = 1 everywhere: each output is its sequence's first latent row, bit for bit."""
    inp = W.paged_attention(410, B=300, H=128, seq_lens=[1] * 300)
    say("ragged single tokens")
    out, _, err = ragged(mla, inp)
    assert err == 0
    out = out.cpu()
    bt = inp["block_table"]
    for b in range(300):
        want = inp["cache"][int(bt[b, 0]), 0, :512].float().expand_as(out[b])
        assert torch.equal(out[b], want), f"seq {b}"


def test_ragged_spikes_across_pieces(mla):
    """Heads whose score singles out one token j* select c_{j*} exactly, with j* on both
    sides of page boundaries inside long sequences that span several ranges."""
    lens = [9000, 70000, 300, 65, 128, 129, 16384]
    spikes = [8999, 40000, 0, 64, 127, 128, 8191]
    hit = list(range(32, 48)) + [0, 127]
    inp = W.paged_attention(411, B=len(lens), H=128, seq_lens=lens)
    inp["cache"][:, :, 512] = 0
    for h in hit:
        inp["q_lat"][:, h].zero_()
        inp["q_pe"][:, h].zero_()
        inp["q_pe"][:, h, 0] = 64.0
    bt = inp["block_table"]
    for b, j in enumerate(spikes):
        inp["cache"][int(bt[b, j // 64]), j % 64, 512] = 64.0
    say("ragged spikes")
    out, _, err = ragged(mla, inp)
    assert err == 0
    out = out.cpu()
    for b, j in enumerate(spikes):
        want = inp["cache"][int(bt[b, j // 64]), j % 64, :512].float()
        for h in hit:
            assert torch.equal(out[b, h], want), f"seq {b} head {h} token {j}"
    rest = [h for h in range(128) if h not in hit]
    o_ref, _ = oracle_attention(inp)
    assert_bf16(host64(out)[:, rest], o_ref[:, rest], "ragged spikes other heads")


def test_ragged_matches_uniform_decode(mla):
    """On a uniform batch the flattened list cuts the same ranges as the split grid: the
    result agrees with mla_decode far inside the oracle tolerance."""
    inp = W.paged_attention(412, B=32, H=128, seq_lens=[2048] * 32)
    say("ragged vs uniform decode")
    out, lse, err = ragged(mla, inp)
    assert err == 0
    q_lat, q_pe = dev(inp["q_lat"]), dev(inp["q_pe"])
    cache, bt, sl = dev(inp["cache"]), dev(inp["block_table"]), dev(inp["seq_lens"])
    S = 8
    ws = torch.empty(mla.mla_decode_workspace_bytes(32, 128, 512, S), dtype=torch.uint8, device="cuda")
    ref = torch.empty(32, 128, 512, device="cuda")
    lref = torch.empty(32, 128, device="cuda")
    mla.mla_decode(q_lat, q_pe, cache, bt, sl, inp["scale"], S, ws, ref, lref)
    torch.cuda.synchronize()
    m, r = errors(host64(out), host64(ref))
    assert m <= 2e-3 and r <= 1e-3, (m, r)


def test_ragged_rejects_bad_workspace(mla):
    inp = W.paged_attention(413, B=2, H=128, seq_lens=[10, 20])
    q_lat, q_pe = dev(inp["q_lat"]), dev(inp["q_pe"])
    cache, bt, sl = dev(inp["cache"]), dev(inp["block_table"]), dev(inp["seq_lens"])
    need = mla.mla_decode_ragged_workspace_bytes(cache, bt, 128, 512)
    ws = torch.empty(need - 256, dtype=torch.uint8, device="cuda")
    out = torch.empty(2, 128, 512, device="cuda")
    say("ragged rejects small workspace")
    with pytest.raises(mla.MLAError):
        mla.mla_decode_ragged(q_lat, q_pe, cache, bt, sl, inp["scale"], ws, out)
