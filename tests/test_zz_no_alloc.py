"""The entry point that allocates nothing (mla_decode_noalloc) against the workspace entry
point it mirrors (mla_decode): same kernels, so bit-identical outputs, on two calls in a
row (the second smaller, so stale partials of the first stay in the scratch), for the bf16
and the fp32 shapes; a request beyond the scratch is rejected before any launch."""
import pytest
import torch

import workloads as W
from tests.gpu_util import dev, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_15_amd as m
    return m


def _both(mla, inp, S):
    q_lat, q_pe, cache = dev(inp["q_lat"]), dev(inp["q_pe"]), dev(inp["cache"])
    bt, sl = dev(inp["block_table"]), dev(inp["seq_lens"])
    B, H, d_c = q_lat.shape
    ws = torch.empty(max(1, mla.mla_decode_workspace_bytes(B, H, d_c, S)), dtype=torch.uint8,
                     device="cuda")
    ref = torch.full((B, H, d_c), float("nan"), device="cuda")
    lref = torch.full((B, H), float("nan"), device="cuda")
    mla.mla_decode(q_lat, q_pe, cache, bt, sl, inp["scale"], S, ws, ref, lref)
    got = torch.full((B, H, d_c), float("nan"), device="cuda")
    lgot = torch.full((B, H), float("nan"), device="cuda")
    mla.mla_decode_noalloc(q_lat, q_pe, cache, bt, sl, inp["scale"], S, got, lgot)
    torch.cuda.synchronize()
    return ref, lref, got, lgot


@pytest.mark.parametrize("shape", ["bf16_h128", "fp32_h4"])
def test_noalloc_matches_workspace_entry(mla, shape):
    if shape == "bf16_h128":
        cases = [(W.paged_attention(300, B=8, H=128, seq_lens=[4096, 1, 33, 700, 2050, 4000, 64, 1500]), 8),
                 (W.paged_attention(301, B=3, H=128, seq_lens=[100, 1000, 31]), 3)]
    else:
        kw = dict(d_c=64, d_R=16, d_h=32, dtype=torch.float32)
        cases = [(W.paged_attention(302, B=4, H=4, seq_lens=[300, 5, 1000, 64], **kw), 6),
                 (W.paged_attention(303, B=2, H=4, seq_lens=[70, 9], **kw), 2)]
    for k, (inp, S) in enumerate(cases):
        say(f"noalloc {shape} call {k} S={S}")
        ref, lref, got, lgot = _both(mla, inp, S)
        assert torch.isfinite(ref).all()
        assert torch.equal(got, ref) and torch.equal(lgot, lref), f"call {k}"


def test_noalloc_rejects_oversize(mla):
    """B=32, H=128, 64 splits: 268 MB of bf16 partials, beyond the 48 MiB scratch."""
    inp = W.paged_attention(304, B=32, H=128, seq_lens=[64] * 32)
    B, H, d_c = inp["q_lat"].shape
    assert mla.mla_decode_workspace_bytes(B, H, d_c, 64) > 48 << 20
    out = torch.zeros(B, H, d_c, device="cuda")
    say("noalloc oversize")
    with pytest.raises(mla.MLAError) as e:
        mla.mla_decode_noalloc(dev(inp["q_lat"]), dev(inp["q_pe"]), dev(inp["cache"]),
                               dev(inp["block_table"]), dev(inp["seq_lens"]), inp["scale"], 64, out)
    assert e.value.status == mla.MLA_ERR_WORKSPACE
    torch.cuda.synchronize()
    assert torch.count_nonzero(out) == 0
