#!/usr/bin/env python3
"""Benchmark of absorbed MLA decode on one MI355X.

One step = the decode hot path over one batch of the DeepSeek-V2-shaped workload
(B=32 sequences, T=4096 cached tokens each, H=128 heads, d_c=512, d_R=64, bf16 cache and
queries, 64-token pages): split-K attention over the paged latent cache (bf16 split
partials) followed by the log-sum-exp combine, both from libmla.  Inputs are seeded
synthetic data, resident in HBM before timing starts.  Four copies of the 151 MB cache
rotate between steps so the 256 MB Infinity Cache cannot serve a repeat.

Three timed regions on the launch stream, each bracketed by HIP events at its ends only:
K whole steps (the headline value), K attention launches back to back (the attention
kernel's average launch duration, its roofline position), and K combine launches.  Back
to back, the attention kernel runs a little slower than between two combines (the
kernel trace shows both), so its roofline figure is the conservative one.  Every launch is
a pre-marshalled library call (head_latent_attention_15_amd.bind), so the host stays ahead of the GPU.

Prints ONE JSON line: throughput (latent-cache GB/s), the attention kernel's roofline
position, and the fp64 CPU oracle timed on the host cores as a baseline.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "MLA absorbed decode: latent-cache GB/s + MFMA TFLOP/s vs roofline, B32 T4K H128"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16 MFMA
ROW_BYTES = 576 * 2             # one cached token: c^KV (512) + k^R (64), bf16
FLOP_PER_TOKEN_HEAD = 2 * (576 + 512)
N_CACHE_COPIES = 4
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attn_mfma_dsv2_b32_t4k_traffic.json")
KERNEL_SRC = os.path.join(ROOT, "head_latent_attention_15_amd", "csrc", "attn_mfma.hip")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    return hashlib.sha256(open(KERNEL_SRC, "rb").read()).hexdigest()[:16]


def measured_traffic():
    """HBM bytes per attention launch from the committed rocprofv3 counter summary, if it
    was taken on the current kernel source; else None."""
    try:
        t = json.load(open(TRAFFIC_FILE))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, n_seq: int, min_seconds: float = 10.0):
    """The fp64 oracle (unchanged) on the first n_seq sequences of the same workload,
    repeated until at least min_seconds of CPU work has been timed."""
    import numpy as np
    import oracle
    import workloads as W
    try:
        from threadpoolctl import threadpool_info
        threads = max([i.get("num_threads", 1) for i in threadpool_info()] or [1])
    except Exception:  # threadpoolctl missing: report the affinity mask size
        threads = len(os.sched_getaffinity(0))
    bt = inp["block_table"].numpy()
    sl = inp["seq_lens"].numpy()
    P = inp["cache"].shape[1]
    t0 = time.perf_counter()
    toks = 0
    passes = 0
    while passes == 0 or time.perf_counter() - t0 < min_seconds:
        for b in range(n_seq):
            rows = oracle.gather_rows(
                W.to_f64(inp["cache"][bt[b, :math.ceil(sl[b] / P)].astype(np.int64)]),
                np.arange(math.ceil(sl[b] / P)), int(sl[b]), P)
            oracle.latent_attention(W.to_f64(inp["q_lat"][b]), W.to_f64(inp["q_pe"][b]), rows,
                                    512, inp["scale"])
            toks += int(sl[b])
        passes += 1
    dt = time.perf_counter() - t0
    return {"value": round(toks * ROW_BYTES / dt / 1e9, 4), "unit": "GB/s", "cores": int(threads),
            "kind": "oracle",
            "sample": f"{passes} passes over {n_seq} of 32 sequences x 4096 tokens (fp64 NumPy "
                      f"latent attention incl. the paged gather, {dt:.1f} s)"}


def layer_rows(mla, W, torch, oracle_seqs: int):
    """Every step of the path on the full decode layer (DeepSeek-V2 sizes, B=64, 2048 cached
    tokens + the new one): each library call timed alone (20 back-to-back calls after a
    0.3 s warmup of the whole chain), its algorithmic bytes (weights, cache rows,
    activations in and out at their stored dtypes) and its fraction of the 8 TB/s HBM
    roofline (every step is HBM-bound at this batch); then the whole chain, and the fp64
    oracle's layer on a few of the sequences.  The projections that share an input run as
    one product over their stacked weights ([W^DQ; W^DKV; W^KR] h, [W^UQ; W^QR] c^Q; the
    weights are stacked once at load time, outside the timing), the append and the
    absorption read their inputs in place, the split-K combine is fused with W^UV, and in
    the timed chain the products accumulate into outputs cleared by one fill at its start.
    Timed beside it: the chain with dense outputs (each product zeroing its own), the chain
    with the combine and W^UV as two launches, and the chain of separate products.  The
    fused step's algorithmic bytes are W^UV and its output: the combined latent is never
    stored."""
    x = W.layer_b64_t2k()
    s = x["shape"]
    B, H, d_h, d_c, d_R, d, d_cq = s.B, s.H, s.d_h, s.d_c, s.d_R, x["d"], x["d_cq"]
    cu = lambda t: t.to("cuda")
    w = {k: cu(v) for k, v in x["weights"].items()}
    w_a = torch.cat([w["w_dq"], w["w_dkv"], w["w_kr"]]).contiguous()
    w_b = torch.cat([w["w_uq"], w["w_qr"]]).contiguous()
    h, cache, bt, before = cu(x["h"]), cu(x["cache"]), cu(x["block_table"]), cu(x["seq_lens_before"])
    f32 = dict(device="cuda", dtype=torch.float32)
    n_a, n_b = d_cq + d_c + d_R, H * (d_h + d_R)
    outs = torch.empty(B * (n_a + n_b + d), **f32)  # y_a, y_b and u, cleared by one fill
    y_a, y_b = outs[:B * n_a].view(B, n_a), outs[B * n_a:B * (n_a + n_b)].view(B, n_b)
    u = outs[B * (n_a + n_b):].view(B, d)
    c_q, c_kv, k_r = y_a[:, :d_cq], y_a[:, d_cq:d_cq + d_c], y_a[:, d_cq + d_c:]
    q_c, q_r = y_b[:, :H * d_h].view(B, H, d_h), y_b[:, H * d_h:].view(B, H, d_R)
    seq_lens = before + 1
    q_lat = torch.empty(B, H, d_c, device="cuda", dtype=torch.bfloat16)
    q_pe = torch.empty(B, H, d_R, device="cuda", dtype=torch.bfloat16)
    S = mla.mla_suggest_num_splits(B, int(seq_lens.max()), 0, 64, 256)
    ws = torch.empty(max(1, mla.mla_decode_workspace_bytes(B, H, d_c, S)), dtype=torch.uint8, device="cuda")
    o_part = torch.empty(B, H, S, d_c, device="cuda", dtype=torch.bfloat16)
    lse_part = torch.empty(B, H, S, **f32)
    o_lat, o_heads = torch.empty(B, H, d_c, **f32), torch.empty(B, H, d_h, **f32)
    nb = lambda t: t.numel() * t.element_size()
    tokens = int(seq_lens.sum())
    rows = [
        ("7 mla_linear [W^DQ; W^DKV; W^KR] h",
         [mla.bind(mla.mla_linear, h, w_a, y_a)], nb(w_a) + nb(h) + nb(y_a)),
        ("7 mla_linear_strided [W^UQ; W^QR] c^Q",
         [mla.bind(mla.mla_linear_strided, c_q, w_b, y_b)], nb(w_b) + B * d_cq * 4 + nb(y_b)),
        ("2 mla_kv_append_strided", [mla.bind(mla.mla_kv_append_strided, c_kv.unsqueeze(1),
                                              k_r.unsqueeze(1), before, bt, cache, x["rope_base"])],
         B * (d_c + d_R) * 4 + B * (d_c + d_R) * 2),
        ("1 mla_absorb_q_strided", [mla.bind(mla.mla_absorb_q_strided, q_c, w["w_uk"], q_r, seq_lens,
                                             x["rope_base"], q_lat, q_pe)],
         nb(w["w_uk"]) + B * H * (d_h + d_R) * 4 + nb(q_lat) + nb(q_pe)),
        (f"3 mla_decode_attn ({S} splits, bf16 partials)",
         [mla.bind(mla.mla_decode_attn, q_lat, q_pe, cache, bt, seq_lens, x["scale"], S, o_part,
                   lse_part)],
         tokens * (d_c + d_R) * 2 + nb(q_lat) + nb(q_pe)),
        ("4+5 mla_combine_out_proj (combine fused with W^UV)",
         [mla.bind(mla.mla_combine_out_proj, o_part, lse_part, w["w_uv"], o_heads)],
         nb(w["w_uv"]) + nb(o_heads)),
        ("6 W^O (mla_linear on the concatenated heads)",
         [mla.bind(mla.mla_linear, o_heads.view(B, H * d_h), w["w_o"], u)],
         nb(w["w_o"]) + nb(o_heads) + nb(u)),
    ]
    # attention + combine (o~ written to HBM), then W^UV on it, then W^O
    unfused_back = [
        mla.bind(mla.mla_decode, q_lat, q_pe, cache, bt, seq_lens, x["scale"], S, ws, o_lat),
        mla.bind(mla.mla_out_proj, o_lat, w["w_uv"], None, o_heads),
        rows[6][1][0]]
    # the same layer with one product per weight and dense intermediates
    sep = {k: torch.empty(B, n, **f32) for k, n in
           (("c_q", d_cq), ("q_c", H * d_h), ("q_r", H * d_R), ("c_kv", d_c), ("k_r", d_R))}
    separate = [
        mla.bind(mla.mla_linear, h, w["w_dq"], sep["c_q"]),
        mla.bind(mla.mla_linear, sep["c_q"], w["w_uq"], sep["q_c"]),
        mla.bind(mla.mla_linear, sep["c_q"], w["w_qr"], sep["q_r"]),
        mla.bind(mla.mla_linear, h, w["w_dkv"], sep["c_kv"]),
        mla.bind(mla.mla_linear, h, w["w_kr"], sep["k_r"]),
        mla.bind(mla.mla_kv_append, sep["c_kv"].view(B, 1, d_c), sep["k_r"].view(B, 1, d_R),
                 before, bt, cache, x["rope_base"]),
        mla.bind(mla.mla_absorb_q, sep["q_c"].view(B, H, d_h), w["w_uk"], sep["q_r"].view(B, H, d_R),
                 seq_lens, x["rope_base"], q_lat, q_pe),
    ] + unfused_back
    chain = [c for _, calls, _ in rows for c in calls]

    # the same calls with the products accumulating into outputs cleared together by one
    # fill at the start of the layer (y_a, y_b and u share one buffer), so the split-k kernels
    # launch no zero fills of their own: two kernels fewer on the one stream
    acc_chain = ([mla.bind(mla.mla_linear_strided, h, w_a, y_a, accumulate=True),
                  mla.bind(mla.mla_linear_strided, c_q, w_b, y_b, accumulate=True)]
                 + [rows[i][1][0] for i in (2, 3, 4, 5)]
                 + [mla.bind(mla.mla_linear_strided, o_heads.view(B, H * d_h), w["w_o"], u,
                             accumulate=True)])

    def accumulate_chain():
        outs.zero_()
        for c in acc_chain:
            c()

    unfused_chain = acc_chain[:4] + unfused_back[:2] + acc_chain[6:]

    def accumulate_unfused():
        outs.zero_()
        for c in unfused_chain:
            c()

    for c in chain:
        c()
    torch.cuda.synchronize()
    u_dense = u.clone()
    accumulate_chain()
    torch.cuda.synchronize()
    acc_vs_dense = float((u - u_dense).abs().max() / u_dense.abs().max())
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        for c in chain + separate:
            c()
        accumulate_chain()
        accumulate_unfused()
        torch.cuda.synchronize()

    def timed(fn, n=20):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for _ in range(n):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n * 1e3  # us

    out = {}
    total_bytes = 0
    for name, calls, byts in rows:
        us = timed(lambda: [c() for c in calls])
        gbps = byts / us / 1e3
        out[name] = {"us": round(us, 2), "bytes_algorithmic": int(byts), "GBps": round(gbps, 1),
                     "roofline_frac": round(gbps / HBM_PEAK_GBPS, 4)}
        total_bytes += byts
    dense_us = timed(lambda: [c() for c in chain])
    separate_us = timed(lambda: [c() for c in separate])
    chain_us = timed(accumulate_chain)
    unfused_us = timed(accumulate_unfused)

    # the survey's fourth next item, measured only: offline absorption folds W^UK_i^T into
    # W^UQ_i ([H d_c, d_c^Q], 201 MB of bf16 weights, prepared once here in fp32 and rounded
    # once), so q~ = W~ c^Q is one projection instead of W^UQ plus the absorption
    wuk = w["w_uk"].float().view(H, d_h, d_c).transpose(1, 2).contiguous()
    wuq = w["w_uq"].float().view(H, d_h, d_cq)
    w_off = torch.bmm(wuk, wuq).to(torch.bfloat16).view(H * d_c, d_cq)
    del wuk, wuq
    q_off = torch.empty(B, H * d_c, **f32)
    off_us = timed(lambda: mla.mla_linear(sep["c_q"], w_off, q_off))
    rt_calls = [mla.bind(mla.mla_linear, sep["c_q"], w["w_uq"], sep["q_c"]),
                mla.bind(mla.mla_absorb_q, sep["q_c"].view(B, H, d_h), w["w_uk"], None, seq_lens,
                         x["rope_base"], q_lat, None)]
    rt_us = timed(lambda: [c() for c in rt_calls])
    off_bytes = nb(w_off) + nb(sep["c_q"]) + nb(q_off)
    out["next-4 offline absorption (measure only)"] = {
        "us": round(off_us, 2), "bytes_algorithmic": int(off_bytes),
        "GBps": round(off_bytes / off_us / 1e3, 1),
        "roofline_frac": round(off_bytes / off_us / 1e3 / HBM_PEAK_GBPS, 4),
        "runtime_absorption_us": round(rt_us, 2),
        "note": "q~ = (W^UK^T W^UQ) c^Q in one mla_linear; runtime_absorption_us = W^UQ + "
                "mla_absorb_q on the same input"}
    del w_off, q_off
    res = {"workload": "layer_b64_t2k (d=5120, H=128, d_h=128, d_c=512, d_c^Q=1536, d_R=64, "
                       "B=64, 2048 cached tokens + 1, bf16 weights and cache)",
           "steps": out, "chain_us": round(chain_us, 2), "chain_bytes_algorithmic": int(total_bytes),
           "chain_GBps": round(total_bytes / chain_us / 1e3, 1),
           "chain_roofline_frac": round(total_bytes / chain_us / 1e3 / HBM_PEAK_GBPS, 4),
           "sequences_per_s": round(B / (chain_us * 1e-6), 1),
           "chain_schedule": "one stream; stacked products accumulating into outputs cleared "
                             "by one fill at the start; combine fused with W^UV",
           "chain_dense_outputs_us": round(dense_us, 2),
           "chain_unfused_combine_us": round(unfused_us, 2),
           "chain_separate_products_us": round(separate_us, 2),
           "accumulate_vs_dense_max_rel_diff": round(acc_vs_dense, 6)}
    if oracle_seqs > 0:
        import oracle
        wf = {k: W.to_f64(v) for k, v in x["weights"].items()}
        hf, cf = W.to_f64(x["h"]), W.to_f64(x["cache"])
        t0 = time.perf_counter()
        oracle.decode_layer(hf, wf, cf, x["block_table"].numpy(), x["seq_lens_before"].numpy(), d_h, d_R,
                            x["rope_base"], x["scale"], batch_index=list(range(oracle_seqs)))
        dt = time.perf_counter() - t0
        res["cpu_oracle"] = {"sequences_per_s": round(oracle_seqs / dt, 3), "kind": "oracle",
                             "sample": f"{oracle_seqs} of 64 sequences (fp64 expanded layer, {dt:.1f} s)"}
    return res


def multi_token_rows(mla, W, torch, caches, bt, sl, scale, num_cus, n_q: int = 2, steps: int = 20):
    """Multi-token decode on the headline cache: the last n_q cached tokens of every
    sequence are new queries (causal among themselves); attention + combine over B n_q
    query rows.  The cache is counted once in the bytes: the n_q workgroups of a
    (sequence, split) read the same tiles."""
    B, H, T = 32, 128, 4096
    q_lat, q_pe = (t.to("cuda") for t in W.multi_queries(6, B, n_q, H))
    S = mla.mla_suggest_num_splits(B * n_q, T, 0, 64, num_cus)
    o_part = torch.empty(B, n_q, H, S, 512, device="cuda", dtype=torch.bfloat16)
    lse_part = torch.empty(B, n_q, H, S, device="cuda")
    out = torch.empty(B * n_q, H, 512, device="cuda")
    calls = [mla.bind(mla.mla_decode_attn_multi, q_lat, q_pe, c, bt, sl, scale, S, o_part, lse_part)
             for c in caches]
    combine = mla.bind(mla.mla_splitk_combine, o_part.view(B * n_q, H, S, 512),
                       lse_part.view(B * n_q, H, S), out)
    for k in range(8):
        calls[k % len(calls)]()
        combine()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for k in range(steps):
        calls[k % len(calls)]()
        combine()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) / steps * 1e3
    cache_bytes = B * T * ROW_BYTES
    flops = B * n_q * T * H * FLOP_PER_TOKEN_HEAD
    return {"workload": f"decode_nq{n_q}_b32_t4k (B=32, T=4096, H=128, {n_q} query tokens per "
                        "sequence at positions T-n_q .. T-1, causal among them)",
            "n_q": n_q, "num_splits": S, "us_per_step": round(us, 2),
            "query_tokens_per_s": round(B * n_q / (us * 1e-6), 1),
            "cache_GBps": round(cache_bytes / (us * 1e-6) / 1e9, 1),
            "tflops": round(flops / (us * 1e-6) / 1e12, 1)}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep warming up until this much time has passed (clocks settle)")
    ap.add_argument("--splits", type=int, default=0, help="split count (0: library suggestion)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--no-layer", action="store_true", help="skip the per-step layer measurement")
    ap.add_argument("--layer-only", action="store_true",
                    help="run only the full-layer measurement and print its JSON (for profiling "
                         "the layer's kernels)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for --pmc runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path here has no multi-GPU mode "
              "(sequences shard across GPUs with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    import torch
    import head_latent_attention_15_amd as mla
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    num_cus = props.multi_processor_count
    if args.layer_only:
        log("layer_b64_t2k only")
        print(json.dumps({"layer_b64_t2k": layer_rows(mla, W, torch, 0)}), flush=True)
        return

    log("generating dsv2_b32_t4k inputs")
    inp = W.dsv2_b32_t4k()
    B, H, T = 32, 128, 4096
    S = args.splits or mla.mla_suggest_num_splits(B, T, 0, 64, num_cus)
    caches = [inp["cache"].to(dev)]
    for _ in range(N_CACHE_COPIES - 1):
        caches.append(caches[0].clone())
    q_lat, q_pe = inp["q_lat"].to(dev), inp["q_pe"].to(dev)
    bt, sl = inp["block_table"].to(dev), inp["seq_lens"].to(dev)
    o_part = torch.empty(B, H, S, 512, device=dev, dtype=torch.bfloat16)
    lse_part = torch.empty(B, H, S, device=dev)
    out = torch.empty(B, H, 512, device=dev)
    lse = torch.empty(B, H, device=dev)
    scale = inp["scale"]

    # arguments checked and marshalled once per cache copy, so the host issues each launch
    # in a few microseconds and the timed regions measure the GPU, not Python
    attn_calls = [mla.bind(mla.mla_decode_attn, q_lat, q_pe, c, bt, sl, scale, S, o_part, lse_part)
                  for c in caches]
    combine = mla.bind(mla.mla_splitk_combine, o_part, lse_part, out, lse)

    def attn(k):
        attn_calls[k % N_CACHE_COPIES]()

    def timed(fn, n):
        """Average milliseconds of n back-to-back calls between two events."""
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record()
        for k in range(n):
            fn(k)
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / n

    # at least W warmup steps, and at least --warmup-seconds of them: the first tens of
    # milliseconds of back-to-back launches run at lower clocks than the steady state
    t_w = time.perf_counter()
    k = 0
    while k < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        attn(k)
        combine()
        k += 1
        if k % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"warmup {k} steps ({time.perf_counter() - t_w:.2f} s), S={S}, {num_cus} CUs")

    ms_step = timed(lambda k: (attn(k), combine()), args.steps)
    # second and third regions: each kernel alone, back to back, events at the ends only
    # (an event recorded between two kernels stalls the queue for several microseconds,
    # so per-kernel events would time the stall with the kernel)
    attn_avg = timed(attn, args.steps)
    comb_avg = timed(lambda k: combine(), args.steps)
    log(f"step {ms_step * 1e3:.1f} us; attention alone {attn_avg * 1e3:.1f} us; "
        f"combine alone {comb_avg * 1e3:.1f} us")

    # plain streaming read of one cache copy: the practical HBM read ceiling
    sink = torch.empty(4096, device=dev)
    for _ in range(3):
        mla.mla_stream_read(caches[1], sink)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    reps = 10
    e0.record()
    for k in range(reps):
        mla.mla_stream_read(caches[k % N_CACHE_COPIES], sink)
    e1.record()
    torch.cuda.synchronize()
    stream_gbps = caches[0].numel() * 2 * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9

    if args.copy_probe:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
        b_ = torch.empty_like(a)
        b_.copy_(a)
        torch.cuda.synchronize()
        del a, b_

    tokens = B * T
    cache_bytes = tokens * ROW_BYTES
    # cache + queries + block table + seq_lens read once; combined output written once
    step_alg_bytes = cache_bytes + B * H * 576 * 2 + B * H * 512 * 4 + bt.numel() * 4 + B * 4
    flops = tokens * H * FLOP_PER_TOKEN_HEAD
    attn_s = attn_avg * 1e-3
    # what one attention launch must move: the cache rows, the queries, the block table and
    # the lengths (split partials are an implementation choice and are not counted)
    attn_alg_bytes = cache_bytes + B * H * 576 * 2 + bt.numel() * 4 + B * 4
    achieved = attn_alg_bytes / attn_s / 1e9
    traffic = measured_traffic()
    result = {
        "metric": METRIC,
        "value": round(cache_bytes / (ms_step * 1e-3) / 1e9, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "dsv2_b32_t4k", "B": B, "T": T, "H": H, "d_c": 512, "d_R": 64,
                   "page_size": 64, "num_splits": S, "split_partials": "bf16",
                   "cache_copies": N_CACHE_COPIES, "parallelism": "none"},
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "query_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "step_bytes_algorithmic": step_alg_bytes,
        "attn_us": round(attn_avg * 1e3, 2),
        "combine_us": round(comb_avg * 1e3, 2),
        "attn_tflops": round(flops / attn_s / 1e12, 2),
        "mfma_frac_of_peak": round(flops / attn_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        "stream_read_GBps": round(stream_gbps, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "kernel": "attn_mfma_kernel<8, bf16 partials> (8 waves x 16 heads, 32-token tiles)",
                     "bytes_per_launch_algorithmic": attn_alg_bytes},
    }
    log("timing multi-token decode (2 query tokens per sequence)")
    result["multi_token"] = multi_token_rows(mla, W, torch, caches, bt, sl, scale, num_cus)
    if not args.no_cpu_baseline:
        log(f"timing the fp64 oracle on {args.cpu_seqs} sequences")
        result["cpu_baseline"] = cpu_baseline(inp, args.cpu_seqs)
    if not args.no_layer:
        log("timing every step of the path on the full decode layer")
        result["layer_b64_t2k"] = layer_rows(mla, W, torch, 0 if args.no_cpu_baseline else 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
