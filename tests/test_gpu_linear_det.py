"""GPU parity of the deterministic projection (mla_linear_deterministic): against numpy fp64
matmul at the decode-layer shapes, bit-identical across reruns, independent of what the
workspace held before (NaN poison), and equal to the atomic split-k product up to the order
of the fp32 additions."""
import math

import numpy as np
import pytest
import torch

import workloads as W
from tests.gpu_util import dev, errors, host64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_15_amd as m
    return m


def det(mla, x, w, y, accumulate=False, poison=False):
    M, K = x.shape
    N = w.shape[0]
    n = mla.mla_linear_deterministic_workspace_bytes(M, N, K)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    if poison:
        ws.view(torch.float32).fill_(float("nan"))
    mla.mla_linear_deterministic(x, w, y, ws, accumulate=accumulate)
    torch.cuda.synchronize()
    return y


# (M, N, K, x dtype): W^O, [W^DQ; W^DKV; W^KR], a short batch, bf16 x, a small product
SHAPES = [(64, 5120, 16384, torch.float32), (64, 2112, 5120, torch.float32),
          (5, 2112, 5120, torch.float32), (64, 1024, 1024, torch.bfloat16), (3, 64, 128, torch.float32)]


@pytest.mark.parametrize("M,N,K,xdt", SHAPES)
def test_deterministic_linear_against_matmul(mla, M, N, K, xdt):
    g = torch.Generator().manual_seed(M + N + K)
    x = torch.randn(M, K, generator=g).to(xdt)
    w = (torch.randn(N, K, generator=g) / math.sqrt(K)).to(torch.bfloat16)
    say(f"deterministic linear M={M} N={N} K={K} x={xdt}")
    y = det(mla, dev(x), dev(w), torch.full((M, N), float("nan"), device="cuda"), poison=True)
    ref = W.to_f64(x) @ W.to_f64(w).T
    m, _ = errors(host64(y), ref)
    # x keeps ~16 significant bits (fp32 as hi + lo) or is exact (bf16): products exact,
    # fp32 sums of K terms of size ~1/sqrt(K)
    assert m <= 4e-5 * math.sqrt(K / 1024) + 1e-6, (M, N, K, m)


def test_deterministic_linear_bit_identical_and_accumulates(mla):
    """Two runs (fresh workspaces, one poisoned) agree bit for bit; accumulate adds onto y
    exactly as y_prev + product in one fixed order; the atomic product differs from it only
    by the order of fp32 additions."""
    M, N, K = 64, 5120, 16384
    g = torch.Generator().manual_seed(7)
    x = dev(torch.randn(M, K, generator=g))
    w = dev((torch.randn(N, K, generator=g) / math.sqrt(K)).to(torch.bfloat16))
    say("deterministic linear reruns")
    a = det(mla, x, w, torch.empty(M, N, device="cuda"))
    b = det(mla, x, w, torch.empty(M, N, device="cuda"), poison=True)
    assert torch.equal(a, b)
    prior = dev(torch.randn(M, N, generator=g))
    c = det(mla, x, w, prior.clone(), accumulate=True)
    c2 = det(mla, x, w, prior.clone(), accumulate=True, poison=True)
    assert torch.equal(c, c2)
    assert errors(host64(c), host64(prior) + host64(a))[0] <= 1e-5
    at = torch.empty(M, N, device="cuda")
    mla.mla_linear_strided(x, w, at)
    torch.cuda.synchronize()
    assert errors(host64(at), host64(a))[0] <= 1e-5


def test_deterministic_linear_strided_views(mla):
    """x read as a column range of a wider buffer, y written into a column range of one."""
    M, N, K = 64, 2112, 5120
    g = torch.Generator().manual_seed(8)
    xb = dev(torch.randn(M, K + 64, generator=g))
    w = dev((torch.randn(N, K, generator=g) / math.sqrt(K)).to(torch.bfloat16))
    yb = torch.full((M, N + 256), 7.0, device="cuda")
    say("deterministic linear strided")
    det(mla, xb[:, :K], w, yb[:, 128:128 + N])
    ref = host64(xb)[:, :K] @ host64(w).T
    assert errors(host64(yb)[:, 128:128 + N], ref)[0] <= 1e-4
    assert torch.all(yb[:, :128] == 7.0) and torch.all(yb[:, 128 + N:] == 7.0)


@pytest.mark.parametrize("B,seq_lens_before", [
    (64, [2048] * 64),                                  # the decode layer: B = 64, 2048 prior tokens
    (5, [0, 63, 64, 700, 1023]),                        # ragged, page boundaries, permuted pages
])
def test_deterministic_linear_append_matches_two_calls(mla, B, seq_lens_before):
    """The fused down-projection + append writes y and the cache exactly as
    mla_linear_deterministic followed by mla_kv_append_strided (n_new = 1) on that y: y bit
    for bit, every cache byte bit for bit (the new rows, and nothing else).  The new rows
    also match the oracle's RoPE of the same fp32 y within bf16 rounding."""
    import oracle
    d, d_cq, d_c, d_R = 5120, 1536, 512, 64
    N = d_cq + d_c + d_R
    g = torch.Generator().manual_seed(90 + B)
    h = torch.randn(B, d, generator=g)
    w = (torch.randn(N, d, generator=g) / math.sqrt(d)).to(torch.bfloat16)
    lens = [s + 1 for s in seq_lens_before]             # room for the appended token
    inp = W.paged_attention(91 + B, B=B, H=1, seq_lens=lens, extra_pages=2)
    cache0 = inp["cache"]
    bt, before = dev(inp["block_table"]), dev(torch.tensor(seq_lens_before, dtype=torch.int32))
    ws = torch.empty(mla.mla_linear_deterministic_workspace_bytes(B, N, d), dtype=torch.uint8,
                     device="cuda")
    say(f"deterministic linear + append B={B}")
    hd, wd = dev(h), dev(w)
    y_ref = torch.full((B, N), float("nan"), device="cuda")
    c_ref = dev(cache0.clone())
    mla.mla_linear_deterministic(hd, wd, y_ref, ws)
    mla.mla_kv_append_strided(y_ref[:, d_cq:d_cq + d_c].unsqueeze(1),
                              y_ref[:, d_cq + d_c:].unsqueeze(1), before, bt, c_ref, 10000.0)
    y = torch.full((B, N), float("nan"), device="cuda")
    c = dev(cache0.clone())
    mla.mla_linear_deterministic_append(hd, wd, y, ws, d_cq, before, bt, c, 10000.0)
    torch.cuda.synchronize()
    assert torch.equal(y.cpu().view(torch.int32), y_ref.cpu().view(torch.int32))
    got, want = c.cpu(), c_ref.cpu()
    assert torch.equal(got.view(torch.int16), want.view(torch.int16))
    yc = y.cpu().double().numpy()
    P = cache0.shape[1]
    changed = (got.view(torch.int16) != cache0.view(torch.int16)).any(dim=2)
    for b, pos in enumerate(seq_lens_before):
        pg, slot = int(inp["block_table"][b, pos // P]), pos % P
        changed[pg, slot] = False
        row = got[pg, slot].double().numpy()
        ref = np.concatenate([yc[b, d_cq:d_cq + d_c],
                              oracle.rope(yc[b, d_cq + d_c:], pos, 10000.0)])
        assert np.all(np.abs(row - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30), b
    assert not bool(changed.any()), "bytes outside the appended rows changed"
