"""GPU parity of the offline weight folds (mla_fold_uq, mla_fold_o_uv): each folded block
against the same product of the bf16 weights in fp64, and the folded projections against
the oracle's unfolded order (absorb_query; up_project_values then output_projection)."""
import math

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


def _bf16_close(gpu, ref):
    """Within one bf16 rounding of the fp64 value (plus the fp32 sum's order)."""
    gpu = host64(gpu)
    err = np.abs(gpu - ref)
    assert np.all(err <= 2.0 ** -7 * np.abs(ref) + 1e-6), float(np.max(err / (np.abs(ref) + 1e-6)))


def _weights(seed, H, d_h, d_c, other):
    g = torch.Generator().manual_seed(seed)
    a = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_h)).to(torch.bfloat16)
    b = (torch.randn(H * d_h, other, generator=g) / math.sqrt(other)).to(torch.bfloat16)
    return a, b


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fold_uq_blocks(mla, out_dtype):
    H, d_h, d_c, d_cq = 4, 128, 512, 1536
    w_uk, w_uq = _weights(50, H, d_h, d_c, d_cq)
    out = torch.empty(H * d_c, d_cq, device="cuda", dtype=out_dtype)
    say(f"fold uq {out_dtype}")
    mla.mla_fold_uq(dev(w_uk), dev(w_uq), H, out)
    torch.cuda.synchronize()
    wuk, wuq = W.to_f64(w_uk), W.to_f64(w_uq)
    ref = np.concatenate([wuk[i * d_h:(i + 1) * d_h].T @ wuq[i * d_h:(i + 1) * d_h]
                          for i in range(H)])
    if out_dtype == torch.float32:
        m, r = errors(host64(out), ref)
        assert r <= 1e-6, r
    else:
        _bf16_close(out, ref)


@pytest.mark.parametrize("out_dtype", [torch.float32, torch.bfloat16])
def test_fold_o_uv_blocks(mla, out_dtype):
    H, d_h, d_c, d_model = 4, 128, 512, 640
    g = torch.Generator().manual_seed(51)
    w_uv = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_c)).to(torch.bfloat16)
    w_o = (torch.randn(d_model, H * d_h, generator=g) / math.sqrt(H * d_h)).to(torch.bfloat16)
    out = torch.empty(d_model, H * d_c, device="cuda", dtype=out_dtype)
    say(f"fold o uv {out_dtype}")
    mla.mla_fold_o_uv(dev(w_o), dev(w_uv), H, out)
    torch.cuda.synchronize()
    wo, wuv = W.to_f64(w_o), W.to_f64(w_uv)
    ref = np.concatenate([wo[:, i * d_h:(i + 1) * d_h] @ wuv[i * d_h:(i + 1) * d_h]
                          for i in range(H)], axis=1)
    if out_dtype == torch.float32:
        m, r = errors(host64(out), ref)
        assert r <= 1e-6, r
    else:
        _bf16_close(out, ref)


def test_folded_query_matches_oracle(mla):
    """q~ = (W^UK^T W^UQ) c^Q with the library's bf16 fold through mla_linear equals the
    oracle's W^UK_i^T (W^UQ c^Q)_i within the bf16 bar."""
    g = torch.Generator().manual_seed(52)
    B, H, d_h, d_c, d_cq = 8, 8, 128, 512, 1536
    c_q = torch.randn(B, d_cq, generator=g)
    w_uk, w_uq = _weights(53, H, d_h, d_c, d_cq)
    w_fold = torch.empty(H * d_c, d_cq, device="cuda", dtype=torch.bfloat16)
    say("folded query")
    mla.mla_fold_uq(dev(w_uk), dev(w_uq), H, w_fold)
    y = torch.empty(B, H * d_c, device="cuda")
    mla.mla_linear(dev(c_q), w_fold, y)
    torch.cuda.synchronize()
    q_c = oracle.linear(W.to_f64(c_q), W.to_f64(w_uq)).reshape(B, H, d_h)
    ref = np.stack([oracle.absorb_query(q_c[b], W.to_f64(w_uk)) for b in range(B)]).reshape(B, H * d_c)
    assert_bf16(host64(y), ref, "folded q~")


def test_folded_output_matches_oracle(mla):
    """u = (W^O W^UV) [o~_1; ...; o~_H] with the library's bf16 fold through mla_linear equals
    the oracle's W^O [W^UV_1 o~_1; ...] within the bf16 bar, at the DeepSeek-V2 widths."""
    g = torch.Generator().manual_seed(54)
    B, H, d_h, d_c, d_model = 16, 128, 128, 512, 5120
    o_lat = torch.randn(B, H, d_c, generator=g) * 0.1
    w_uv = (torch.randn(H * d_h, d_c, generator=g) / math.sqrt(d_c)).to(torch.bfloat16)
    w_o = (torch.randn(d_model, H * d_h, generator=g) / math.sqrt(H * d_h)).to(torch.bfloat16)
    w_fold = torch.empty(d_model, H * d_c, device="cuda", dtype=torch.bfloat16)
    say("folded output projection")
    mla.mla_fold_o_uv(dev(w_o), dev(w_uv), H, w_fold)
    u = torch.empty(B, d_model, device="cuda")
    mla.mla_linear(dev(o_lat).view(B, H * d_c), w_fold, u)
    torch.cuda.synchronize()
    ref = oracle.output_projection(oracle.up_project_values(W.to_f64(o_lat), W.to_f64(w_uv)),
                                   W.to_f64(w_o))
    assert_bf16(host64(u), ref, "folded u")
