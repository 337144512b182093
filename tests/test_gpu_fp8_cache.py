"""GPU parity of the fp8 latent cache (MLA_FP8 rows: 512 E4M3 codes, bf16 k^R, four
power-of-two block scales).  The quantised bytes (bulk quantisation and append) against
oracle/fp8_cache bit for bit; the attention over fp8 rows against the fp64 oracle on the
dequantised rows within the bf16 bar, and bit-exact where a closed form fixes the
result (one token; a spike selecting one row)."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from oracle import fp8_cache as F8
from tests.gpu_util import assert_bf16, dev, errors, host64, say

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def mla():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import head_latent_attention_15_amd as m
    return m


def quantize_gpu(mla, rows):
    """rows [..., 576] (torch, fp32 or bf16) -> uint8 [..., 656] quantised on the GPU."""
    src = dev(rows)
    out = torch.empty(rows.shape[:-1] + (656,), dtype=torch.uint8, device="cuda")
    mla.mla_quantize_cache(src, out)
    torch.cuda.synchronize()
    return out


def _awkward_rows(seed, n):
    """Rows with blocks of very different magnitudes, all-zero blocks, a block whose maximum
    is exactly 448 * 2^k, values on E4M3 rounding midpoints, tiny and subnormal-range values."""
    g = torch.Generator().manual_seed(seed)
    x = torch.randn(n, 576, generator=g)
    mags = 2.0 ** torch.randint(-20, 20, (n, 4), generator=g).float()
    x[:, :512] *= mags.repeat_interleave(128, dim=1)
    x[0, :128] = 0.0
    x[1, 128:256] = 0.0
    x[1, 128] = 448.0 * 2.0 ** -3                  # exact boundary: scale 2^-3
    x[2, :4] = torch.tensor([1.0, 1.0625, 1.1875, -17.0])  # 1.0625 and 1.1875: E4M3 midpoints
    x[2, 4:128] = 0.0
    x[3, 256:384] *= 1e-30
    return x


@pytest.mark.parametrize("src_dtype", [torch.bfloat16, torch.float32])
def test_quantize_rows_bit_exact(mla, src_dtype):
    rows = _awkward_rows(60, 300).to(src_dtype)
    say(f"fp8 quantize {src_dtype}")
    got = quantize_gpu(mla, rows).cpu().numpy()
    vals = rows.double().numpy()
    # k^R is rounded to bf16 on the GPU; the oracle packs the bf16 values
    vals[:, 512:] = rows[:, 512:].to(torch.bfloat16).double().numpy()
    want = F8.quantize_rows(vals)
    assert np.array_equal(got, want), int(np.sum(got != want))


def test_append_fp8_rows(mla):
    """Append of 2 tokens per sequence into fp8 rows: codes and scales of c^KV bit-exact,
    k^R the oracle's RoPE rounded to bf16 (within one bf16 rounding); other slots untouched."""
    g = torch.Generator().manual_seed(61)
    B, n_new, P = 3, 2, 64
    before = torch.tensor([0, 63, 200], dtype=torch.int32)
    pages = [math.ceil((int(b) + n_new) / P) for b in before]
    bt = torch.full((B, max(pages)), -1, dtype=torch.int32)
    k = 0
    for b in range(B):
        for p in range(pages[b]):
            bt[b, p] = k
            k += 1
    cache = torch.full((k, P, 656), 0xA5, dtype=torch.uint8)
    c_kv = torch.randn(B, n_new, 512, generator=g) * 3
    k_r = torch.randn(B, n_new, 64, generator=g)
    cd = dev(cache)
    say("fp8 append")
    mla.mla_kv_append(dev(c_kv), dev(k_r), dev(before), dev(bt), cd, 10000.0)
    torch.cuda.synchronize()
    got = cd.cpu().numpy()
    touched = np.zeros(got.shape[:2], dtype=bool)
    for b in range(B):
        for t in range(n_new):
            pos = int(before[b]) + t
            pg, slot = int(bt[b, pos // P]), pos % P
            touched[pg, slot] = True
            codes, rope, scales = F8.unpack_rows(got[pg, slot])
            c_ref, s_ref = F8.quantize_latent(c_kv[b, t].double().numpy())
            assert np.array_equal(codes, c_ref) and np.array_equal(scales, s_ref)
            r_ref = oracle.rope(k_r[b, t].double().numpy(), pos, 10000.0)
            assert np.all(np.abs(rope - r_ref) <= 2.0 ** -8 * np.abs(r_ref) + 1e-30)
    assert np.all(got[~touched] == 0xA5)


def _fp8_problem(seed, B, seq_lens, H=128):
    inp = W.paged_attention(seed, B=B, H=H, seq_lens=seq_lens)
    rows = inp["cache"].double().numpy()
    inp["fp8"] = F8.quantize_rows(rows)                      # oracle bytes
    inp["deq"] = torch.from_numpy(F8.dequantize_rows(inp["fp8"]))
    return inp


def attend_fp8(mla, inp, S, part, q_lat=None, q_pe=None, cache_bytes=None, kernel="auto"):
    q_lat = dev(inp["q_lat"] if q_lat is None else q_lat)
    q_pe = dev(inp["q_pe"] if q_pe is None else q_pe)
    cache = dev(torch.from_numpy(inp["fp8"]) if cache_bytes is None else cache_bytes)
    bt, sl = dev(inp["block_table"]), dev(inp["seq_lens"])
    rows = q_lat.shape[0] * (q_lat.shape[1] if q_lat.dim() == 4 else 1)
    o_part = torch.empty(rows, 128, S, 512, device="cuda", dtype=part if S > 1 else torch.float32)
    lse_part = torch.empty(rows, 128, S, device="cuda")
    mla.mla_decode_attn_planned(q_lat, q_pe, cache, bt, sl, inp["scale"], S, o_part, lse_part,
                                kernel=kernel)
    if S == 1:
        torch.cuda.synchronize()
        return o_part.view(rows, 128, 512), lse_part.view(rows, 128)
    out = torch.empty(rows, 128, 512, device="cuda")
    lse = torch.empty(rows, 128, device="cuda")
    mla.mla_splitk_combine(o_part, lse_part, out, lse)
    torch.cuda.synchronize()
    return out, lse


def oracle_fp8(inp):
    P = inp["deq"].shape[1]
    bt = inp["block_table"].numpy()
    sl = inp["seq_lens"].numpy()
    o, lse = [], []
    for b in range(inp["q_lat"].shape[0]):
        rows = oracle.gather_rows(inp["deq"][torch.from_numpy(np.maximum(bt[b], 0)).long()].numpy(),
                                  np.arange(bt.shape[1]), int(sl[b]), P)
        att = oracle.latent_attention(W.to_f64(inp["q_lat"][b]), W.to_f64(inp["q_pe"][b]), rows,
                                      512, inp["scale"])
        o.append(att["o_lat"])
        lse.append(att["lse"])
    return np.stack(o), np.stack(lse)


FP8_KERNELS = ["heads", "wide"]


@pytest.mark.parametrize("kernel", FP8_KERNELS)
@pytest.mark.parametrize("S,part", [(1, torch.float32), (3, torch.float32), (8, torch.bfloat16),
                                    (64, torch.bfloat16)])
def test_fp8_attention_against_oracle(mla, S, part, kernel):
    inp = _fp8_problem(70, 5, [1, 31, 33, 700, 2050])
    say(f"fp8 attention S={S} part={part} kernel={kernel}")
    out, lse = attend_fp8(mla, inp, S, part, kernel=kernel)
    o_ref, lse_ref = oracle_fp8(inp)
    assert_bf16(host64(out), o_ref, f"fp8 S={S} {kernel}")
    assert errors(host64(lse), lse_ref)[0] <= 2e-2


@pytest.mark.parametrize("kernel", FP8_KERNELS)
def test_fp8_split_tile_counts(mla, kernel):
    """Splits of one, two, three and four 32-token tiles, full and ragged (the raw-row
    staging runs two tiles ahead of the products, so each short count takes its own
    path through the prologue), against the oracle."""
    lens = [32, 33, 64, 65, 96, 97, 127, 128, 129, 1024, 1025]
    inp = _fp8_problem(76, len(lens), lens)
    say(f"fp8 tile counts kernel={kernel}")
    for S in (1, 4, 8):
        out, lse = attend_fp8(mla, inp, S, torch.float32, kernel=kernel)
        o_ref, lse_ref = oracle_fp8(inp)
        assert_bf16(host64(out), o_ref, f"fp8 tile counts S={S} {kernel}")
        assert errors(host64(lse), lse_ref)[0] <= 2e-2


@pytest.mark.parametrize("kernel", FP8_KERNELS)
def test_fp8_single_token_bit_exact(mla, kernel):
    inp = _fp8_problem(71, 4, [1, 1, 1, 1])
    say(f"fp8 single token kernel={kernel}")
    out, _ = attend_fp8(mla, inp, 1, torch.float32, kernel=kernel)
    out = out.cpu()
    bt = inp["block_table"]
    for b in range(4):
        want = inp["deq"][int(bt[b, 0]), 0, :512].float().expand_as(out[b])
        assert torch.equal(out[b], want), f"seq {b}"


@pytest.mark.parametrize("kernel", FP8_KERNELS)
def test_fp8_spike_takes_exact_fallback(mla, kernel):
    """Heads whose scores jump far above their reference take the exact fallback, which
    reads the fp8 rows itself: they select the dequantised spike row bit for bit."""
    seq_lens = [64, 129, 1000]
    spikes = [63, 128, 999]
    hit = list(range(16, 32)) + [127]
    inp = W.paged_attention(72, B=3, H=128, seq_lens=seq_lens)
    inp["cache"][:, :, 512] = 0
    for h in hit:
        inp["q_lat"][:, h].zero_()
        inp["q_pe"][:, h].zero_()
        inp["q_pe"][:, h, 0] = 64.0
    bt = inp["block_table"]
    for b, j in enumerate(spikes):
        inp["cache"][int(bt[b, j // 64]), j % 64, 512] = 64.0
    inp["fp8"] = F8.quantize_rows(inp["cache"].double().numpy())
    inp["deq"] = torch.from_numpy(F8.dequantize_rows(inp["fp8"]))
    say(f"fp8 spike fallback kernel={kernel}")
    out, _ = attend_fp8(mla, inp, 4, torch.float32, kernel=kernel)
    out = out.cpu()
    for b, j in enumerate(spikes):
        want = inp["deq"][int(bt[b, j // 64]), j % 64, :512].float()
        for h in hit:
            assert torch.equal(out[b, h], want), f"seq {b} head {h}"
    rest = [h for h in range(128) if h not in hit]
    o_ref, _ = oracle_fp8(inp)
    assert_bf16(host64(out)[:, rest], o_ref[:, rest], "fp8 spike other heads")


@pytest.mark.parametrize("kernel", FP8_KERNELS)
def test_fp8_multi_token(mla, kernel):
    n_q = 2
    inp = _fp8_problem(73, 3, [5, 300, 1100])
    q_lat, q_pe = W.multi_queries(74, 3, n_q, 128)
    say(f"fp8 multi-token kernel={kernel}")
    out, _ = attend_fp8(mla, inp, 4, torch.bfloat16, q_lat=q_lat, q_pe=q_pe, kernel=kernel)
    o_ref, _ = oracle.paged_decode_multi(W.to_f64(q_lat), W.to_f64(q_pe), inp["deq"].numpy(),
                                         inp["block_table"].numpy(), inp["seq_lens"].numpy(),
                                         n_q, 512, inp["scale"])
    assert_bf16(host64(out.view(3, n_q, 128, 512)), o_ref, "fp8 multi-token")


@pytest.mark.slow
@pytest.mark.parametrize("kernel", FP8_KERNELS)
def test_fp8_dsv2_b32_t4k_full(mla, kernel):
    """The headline shape over fp8 rows quantised on the GPU: the bytes of 4096 sampled
    rows against the oracle, then every output against the oracle on the dequantised rows."""
    inp = W.dsv2_b32_t4k()
    say(f"fp8 dsv2_b32_t4k kernel={kernel}")
    fp8 = quantize_gpu(mla, inp["cache"])
    flat = fp8.view(-1, 656).cpu().numpy()
    idx = np.random.default_rng(75).choice(flat.shape[0], 4096, replace=False)
    want = F8.quantize_rows(inp["cache"].view(-1, 576)[torch.from_numpy(idx)].double().numpy())
    assert np.array_equal(flat[idx], want)
    inp["fp8"] = flat.reshape(fp8.shape)
    inp["deq"] = torch.from_numpy(F8.dequantize_rows(inp["fp8"]))
    S = mla.mla_suggest_num_splits(32, 4096, 0, 64, 256)
    out, lse = attend_fp8(mla, inp, S, torch.bfloat16, cache_bytes=fp8, kernel=kernel)
    o_ref, lse_ref = oracle_fp8(inp)
    m, r = assert_bf16(host64(out), o_ref, "fp8 dsv2_b32_t4k")
    print(f"fp8 dsv2_b32_t4k: max-abs {m:.3e} rel-L2 {r:.3e}")
    assert errors(host64(lse), lse_ref)[0] <= 2e-2


def test_fp8_ragged_work_list(mla):
    """mla_decode_ragged over fp8 rows (flattened work list, kernel with 32 heads per
    wavefront): ragged lengths incl. an empty sequence and single-tile pieces, a permuted
    pool, every output against the oracle on the dequantised rows."""
    lens = [0, 1, 33, 64, 700, 2050, 4097, 95]
    inp = _fp8_problem(77, len(lens), lens)
    say("fp8 ragged work list")
    q_lat, q_pe = dev(inp["q_lat"]), dev(inp["q_pe"])
    cache = dev(torch.from_numpy(inp["fp8"]))
    bt, sl = dev(inp["block_table"]), dev(inp["seq_lens"])
    B = len(lens)
    ws = torch.full((mla.mla_decode_ragged_workspace_bytes(cache, bt, 128, 512),), 0xFF,
                    dtype=torch.uint8, device="cuda")
    out = torch.full((B, 128, 512), float("nan"), device="cuda")
    lse = torch.full((B, 128), float("nan"), device="cuda")
    mla.mla_decode_ragged(q_lat, q_pe, cache, bt, sl, inp["scale"], ws, out, lse)
    torch.cuda.synchronize()
    assert int(ws[8 * B:8 * B + 4].view(torch.int32).item()) == 0
    o_ref, lse_ref = oracle_fp8(inp)
    empty = [b for b, n in enumerate(lens) if n == 0]
    rest = [b for b, n in enumerate(lens) if n > 0]
    assert torch.all(out[empty] == 0) and torch.all(torch.isinf(lse[empty]))
    assert_bf16(host64(out)[rest], o_ref[rest], "fp8 ragged")
    assert errors(host64(lse)[rest], lse_ref[rest])[0] <= 2e-2
