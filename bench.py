#!/usr/bin/env python3
"""Benchmark of absorbed MLA decode on one MI355X.

One step = the decode hot path over one batch of the DeepSeek-V2-shaped workload
(B=32 sequences, T=4096 cached tokens each, H=128 heads, d_c=512, d_R=64, bf16 cache and
queries, 64-token pages): split-K attention over the paged latent cache (the library's
kernel for 128 heads, bf16 split partials) followed by the log-sum-exp combine, both from
libmla.  Inputs are seeded synthetic data, resident in HBM before timing starts.  Four
copies of the 151 MB cache rotate between steps so the 256 MB Infinity Cache cannot serve
a repeat.

Timed regions on the launch stream, each bracketed by HIP events at its ends only: K whole
steps (the headline value); the same steps with fp32 partials; K single launches that
merge their own splits (mla_decode_fused); K attention launches back to back (the
attention kernel's average launch duration: its roofline position); K combines; and K
launches of the other attention kernel.  Every launch is a pre-marshalled library call
(head_latent_attention_15_amd.bind), so the host stays ahead of the GPU.  Beside the
headline: the long-context and ragged workloads (split grid, flattened work list, single
launch), the headline over fp8 latent rows, multi-token decode, the plain and LDS-DMA
stream-read ceilings, the full decode layer with every step's roofline fraction and the
offline folds, and the fp64 CPU oracle on all host cores and on one thread.

Prints ONE JSON line.

    python bench.py [--gpus 1] [--steps 50] [--warmup 10] [--no-cpu-baseline] [--no-layer]
                    [--no-configs] [--headline-only] [--layer-only] [--prefill-only]
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
# rocprofv3 counter summary and kernel source of each attention kernel the headline can time
TRAFFIC = {
    "wide": ("attn_wide_dsv2_b32_t4k_traffic.json", "attn_wide.hip"),
    "heads": ("attn_mfma_dsv2_b32_t4k_traffic.json", "attn_mfma.hip"),
    "cols": ("attn_cols_dsv2_b32_t4k_traffic.json", "attn_cols.hip"),
}
KERNEL_NAMES = {
    "wide": "attn_wide_kernel<bf16 partials> (4 waves x 32 heads, 32x32x16 MFMA)",
    "heads": "attn_mfma_kernel<8, bf16 partials> (8 waves x 16 heads)",
    "cols": "attn_cols_kernel<bf16 partials> (8 waves: scores by 16-head blocks, latent "
            "product by 64-column blocks)",
}


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


def kernel_source_hash(kernel: str) -> str:
    src = os.path.join(ROOT, "head_latent_attention_15_amd", "csrc", TRAFFIC[kernel][1])
    return hashlib.sha256(open(src, "rb").read()).hexdigest()[:16]


def measured_traffic(kernel: str):
    """HBM bytes per attention launch of `kernel` from the committed rocprofv3 counter
    summary, if it was taken on the current kernel source; else None."""
    try:
        t = json.load(open(os.path.join(ROOT, "profiles", TRAFFIC[kernel][0])))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256_16") != kernel_source_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(inp, n_seq: int, min_seconds: float = 10.0):
    """The fp64 oracle (unchanged) on the first n_seq sequences of the same workload,
    repeated until at least min_seconds of CPU work has been timed, with the BLAS thread
    count the process was started with."""
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


def cpu_baseline_child(n_seq: int, threads: int):
    """The same measurement in a child process whose BLAS and OpenMP pools are limited to
    `threads` (set before NumPy loads); returns its cpu_baseline dict."""
    import subprocess
    env = dict(os.environ)
    for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS", "BLIS_NUM_THREADS"):
        env[k] = str(threads)
    env["HIP_VISIBLE_DEVICES"] = ""  # the child never touches the GPU
    r = subprocess.run([sys.executable, os.path.abspath(__file__), "--cpu-baseline-only",
                        "--cpu-seqs", str(n_seq)], env=env, capture_output=True, text=True,
                       timeout=600)
    if r.returncode != 0:
        return {"error": r.stderr[-400:]}
    return json.loads(r.stdout.strip().splitlines()[-1])


def layer_rows(mla, W, torch, oracle_seqs: int):
    """Every step of the path on the full decode layer (DeepSeek-V2 sizes, B=64, 2048 cached
    tokens + the new one): each library call timed alone (20 back-to-back calls after a
    0.3 s warmup of the whole chain), its algorithmic bytes (weights, cache rows,
    activations in and out at their stored dtypes) and its fraction of the 8 TB/s HBM
    roofline (every step is HBM-bound at this batch); then the whole chain, and the fp64
    oracle's layer on a few of the sequences.  In the chain every result is the same from
    run to run (checked: two runs, u bit for bit): [W^DQ; W^DKV; W^KR] h and W^O are split-k
    products summed in a fixed order (mla_linear_deterministic), the first one's summing
    launch also writes the new token's cache row with its RoPE (mla_linear_deterministic_
    append), the query side ([W^UQ; W^QR] c^Q, RoPE, absorption) is one launch reading c^Q in
    place (its weights packed once at load time, outside the timing), and the split-K combine
    is fused with W^UV.  Timed beside it: the chain with fp32-atomic projections
    accumulating into outputs cleared by one fill, with the query side as two launches (the
    stacked product, then the absorption), with the combine and W^UV as two launches, with
    the first product and the append as two launches, and the chain of separate products.  The fused steps' algorithmic bytes are their weights,
    inputs and outputs: q^C, q^R and the combined latent are never stored."""
    x = W.layer_b64_t2k()
    s = x["shape"]
    B, H, d_h, d_c, d_R, d, d_cq = s.B, s.H, s.d_h, s.d_c, s.d_R, x["d"], x["d_cq"]
    cu = lambda t: t.to("cuda")
    w = {k: cu(v) for k, v in x["weights"].items()}
    w_a = torch.cat([w["w_dq"], w["w_dkv"], w["w_kr"]]).contiguous()
    w_b = torch.cat([w["w_uq"], w["w_qr"]]).contiguous()
    w_pack = mla.mla_pack_query_weights(w["w_uq"], w["w_qr"], w["w_uk"], H)  # load-time packing
    h, cache, bt, before = cu(x["h"]), cu(x["cache"]), cu(x["block_table"]), cu(x["seq_lens_before"])
    f32 = dict(device="cuda", dtype=torch.float32)
    n_a, n_b = d_cq + d_c + d_R, H * (d_h + d_R)
    outs = torch.empty(B * (n_a + d), **f32)  # y_a and u (cleared by one fill where accumulated)
    y_a, u = outs[:B * n_a].view(B, n_a), outs[B * n_a:].view(B, d)
    y_b = torch.empty(B, n_b, **f32)            # q^C | q^R of the two-launch query side
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
    # the projections run with a fixed summation order (split-k partials summed in order):
    # one workspace serves both, since they run one after the other on the stream
    ws_lin = torch.empty(max(mla.mla_linear_deterministic_workspace_bytes(B, n_a, d),
                             mla.mla_linear_deterministic_workspace_bytes(B, d, H * d_h)),
                         dtype=torch.uint8, device="cuda")
    append_bytes = B * (d_c + d_R) * 2  # the new rows written to the cache
    det_a = mla.bind(mla.mla_linear_deterministic, h, w_a, y_a, ws_lin)
    append = mla.bind(mla.mla_kv_append_strided, c_kv.unsqueeze(1), k_r.unsqueeze(1), before, bt,
                      cache, x["rope_base"])
    rows = [
        ("7+2 mla_linear_deterministic_append ([W^DQ; W^DKV; W^KR] h, RoPE and the cache append "
         "in its summing launch)",
         [mla.bind(mla.mla_linear_deterministic_append, h, w_a, y_a, ws_lin, d_cq, before, bt,
                   cache, x["rope_base"])], nb(w_a) + nb(h) + nb(y_a) + append_bytes),
        ("7+1 mla_query_path (W^UQ, W^QR, RoPE, absorption in one launch)",
         [mla.bind(mla.mla_query_path, c_q, w_pack, seq_lens, x["rope_base"], q_lat, q_pe)],
         nb(w_b) + nb(w["w_uk"]) + B * d_cq * 4 + nb(q_lat) + nb(q_pe)),
        (f"3 mla_decode_attn ({S} splits, bf16 partials)",
         [mla.bind(mla.mla_decode_attn, q_lat, q_pe, cache, bt, seq_lens, x["scale"], S, o_part,
                   lse_part)],
         tokens * (d_c + d_R) * 2 + nb(q_lat) + nb(q_pe)),
        ("4+5 mla_combine_out_proj (combine fused with W^UV)",
         [mla.bind(mla.mla_combine_out_proj, o_part, lse_part, w["w_uv"], o_heads)],
         nb(w["w_uv"]) + nb(o_heads)),
        ("6 W^O (mla_linear_deterministic on the concatenated heads)",
         [mla.bind(mla.mla_linear_deterministic, o_heads.view(B, H * d_h), w["w_o"], u, ws_lin)],
         nb(w["w_o"]) + nb(o_heads) + nb(u)),
    ]
    # the fused first step as its two calls, and the same two products with fp32 atomic split-k
    # (not in the main chain)
    split_rows = [
        ("7 mla_linear_deterministic [W^DQ; W^DKV; W^KR] h (the first step's product alone)",
         det_a, nb(w_a) + nb(h) + nb(y_a)),
        ("2 mla_kv_append_strided (the first step's append as its own launch)", append,
         B * (d_c + d_R) * 4 + append_bytes)]
    atomic_rows = [
        ("7 mla_linear [W^DQ; W^DKV; W^KR] h",
         mla.bind(mla.mla_linear, h, w_a, y_a), nb(w_a) + nb(h) + nb(y_a)),
        ("6 W^O (mla_linear)", mla.bind(mla.mla_linear, o_heads.view(B, H * d_h), w["w_o"], u),
         nb(w["w_o"]) + nb(o_heads) + nb(u))]
    # the query side as two launches: the stacked product [W^UQ; W^QR] c^Q, then the
    # absorption (with the RoPE) reading q^C and q^R in place
    two_launch_query = [
        ("7 mla_linear_strided [W^UQ; W^QR] c^Q",
         mla.bind(mla.mla_linear_strided, c_q, w_b, y_b), nb(w_b) + B * d_cq * 4 + nb(y_b)),
        ("1 mla_absorb_q_strided",
         mla.bind(mla.mla_absorb_q_strided, q_c, w["w_uk"], q_r, seq_lens, x["rope_base"], q_lat,
                  q_pe), nb(w["w_uk"]) + B * H * (d_h + d_R) * 4 + nb(q_lat) + nb(q_pe))]
    # attention + combine (o~ written to HBM), then W^UV on it, then W^O
    unfused_back = [
        mla.bind(mla.mla_decode, q_lat, q_pe, cache, bt, seq_lens, x["scale"], S, ws, o_lat),
        mla.bind(mla.mla_out_proj, o_lat, w["w_uv"], None, o_heads),
        rows[4][1][0]]
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
    # the main chain: every step's result is the same from run to run
    chain = [c for _, calls, _ in rows for c in calls]

    def run_calls(calls, fill=False):
        def go():
            if fill:
                outs.zero_()
            for c in calls:
                c()
        return go

    main_chain = run_calls(chain)
    # the atomic split-k products accumulating into outputs cleared together by one fill at
    # the start of the layer (y_a and u share one buffer), so they launch no zero fills
    acc_chain = ([mla.bind(mla.mla_linear_strided, h, w_a, y_a, accumulate=True), append]
                 + chain[1:4] + [mla.bind(mla.mla_linear_strided, o_heads.view(B, H * d_h),
                                          w["w_o"], u, accumulate=True)])
    atomic_chain = run_calls(acc_chain, fill=True)
    # attention + combine, then W^UV: two launches in place of the fused one
    unfused_chain = run_calls(chain[:2] + unfused_back[:2] + chain[4:])
    # the query side as two launches in place of mla_query_path
    two_launch_chain = run_calls(chain[:1] + [c for _, c, _ in two_launch_query] + chain[2:])
    # the product and the append as two launches in place of the fused first step
    split_append_chain = run_calls([det_a, append] + chain[1:])

    main_chain()
    torch.cuda.synchronize()
    u_det = u.clone()
    main_chain()
    torch.cuda.synchronize()
    rerun_identical = bool(torch.equal(u, u_det))
    atomic_chain()
    torch.cuda.synchronize()
    atomic_vs_det = float((u - u_det).abs().max() / u_det.abs().max())
    two_launch_chain()
    torch.cuda.synchronize()
    two_vs_one = float((u - u_det).abs().max() / u_det.abs().max())
    split_append_chain()
    torch.cuda.synchronize()
    split_append_identical = bool(torch.equal(u, u_det))
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        for c in separate:
            c()
        main_chain()
        atomic_chain()
        unfused_chain()
        two_launch_chain()
        split_append_chain()
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
    for name, call, byts in split_rows:
        us = timed(call)
        gbps = byts / us / 1e3
        out[name + " (not in the chain)"] = {
            "us": round(us, 2), "bytes_algorithmic": int(byts), "GBps": round(gbps, 1),
            "roofline_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    for name, call, byts in atomic_rows:
        us = timed(call)
        gbps = byts / us / 1e3
        out[name + " (atomic split-k; not in the chain)"] = {
            "us": round(us, 2), "bytes_algorithmic": int(byts), "GBps": round(gbps, 1),
            "roofline_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    two_us = 0.0
    for name, call, byts in two_launch_query:
        us = timed(call)
        two_us += us
        gbps = byts / us / 1e3
        out[name + " (the query side as two launches; not in the chain)"] = {
            "us": round(us, 2), "bytes_algorithmic": int(byts), "GBps": round(gbps, 1),
            "roofline_frac": round(gbps / HBM_PEAK_GBPS, 4)}
    separate_us = timed(lambda: [c() for c in separate])
    chain_us = timed(main_chain)
    atomic_us = timed(atomic_chain)
    unfused_us = timed(unfused_chain)
    two_launch_us = timed(two_launch_chain)
    split_append_us = timed(split_append_chain)

    # Offline folds, measured only, with the weights prepared once by the library outside the
    # timing.  W~ = W^UK^T W^UQ ([H d_c, d_c^Q], 201 MB of bf16) makes q~ = W~ c^Q one
    # projection instead of W^UQ plus the absorption; W_fold = W^O W^UV ([d, H d_c], 671 MB)
    # makes u = W_fold [o~_1; ...] one projection instead of W^UV plus W^O.
    w_off = torch.empty(H * d_c, d_cq, device="cuda", dtype=torch.bfloat16)
    mla.mla_fold_uq(w["w_uk"], w["w_uq"], H, w_off)
    q_off = torch.empty(B, H * d_c, **f32)
    off_us = timed(lambda: mla.mla_linear(sep["c_q"], w_off, q_off))
    rt_calls = [mla.bind(mla.mla_linear, sep["c_q"], w["w_uq"], sep["q_c"]),
                mla.bind(mla.mla_absorb_q, sep["q_c"].view(B, H, d_h), w["w_uk"], None, seq_lens,
                         x["rope_base"], q_lat, None)]
    rt_us = timed(lambda: [c() for c in rt_calls])
    off_bytes = nb(w_off) + nb(sep["c_q"]) + nb(q_off)
    out["next-4 offline absorption W^UK^T W^UQ (measure only)"] = {
        "us": round(off_us, 2), "bytes_algorithmic": int(off_bytes),
        "GBps": round(off_bytes / off_us / 1e3, 1),
        "roofline_frac": round(off_bytes / off_us / 1e3 / HBM_PEAK_GBPS, 4),
        "runtime_path_us": round(rt_us, 2),
        "note": "q~ = (W^UK^T W^UQ) c^Q in one mla_linear (fold by mla_fold_uq); "
                "runtime_path_us = W^UQ + mla_absorb_q on the same input"}
    del w_off, q_off
    w_fold = torch.empty(d, H * d_c, device="cuda", dtype=torch.bfloat16)
    mla.mla_fold_o_uv(w["w_o"], w["w_uv"], H, w_fold)
    u_fold = torch.empty(B, d, **f32)
    fold_us = timed(lambda: mla.mla_linear(o_lat.view(B, H * d_c), w_fold, u_fold))
    rt2 = [mla.bind(mla.mla_out_proj, o_lat, w["w_uv"], None, o_heads),
           mla.bind(mla.mla_linear, o_heads.view(B, H * d_h), w["w_o"], u)]
    rt2_us = timed(lambda: [c() for c in rt2])
    fold_bytes = nb(w_fold) + nb(o_lat) + nb(u_fold)
    out["next-4 offline fold W^O W^UV (measure only)"] = {
        "us": round(fold_us, 2), "bytes_algorithmic": int(fold_bytes),
        "GBps": round(fold_bytes / fold_us / 1e3, 1),
        "roofline_frac": round(fold_bytes / fold_us / 1e3 / HBM_PEAK_GBPS, 4),
        "runtime_path_us": round(rt2_us, 2),
        "note": "u = (W^O W^UV) [o~_1; ...; o~_H] in one mla_linear (fold by mla_fold_o_uv, "
                "d_c/d_h = 4x the bytes of W^O); runtime_path_us = W^UV (mla_out_proj) + W^O "
                "on the same combined latent"}
    del w_fold, u_fold
    res = {"workload": "layer_b64_t2k (d=5120, H=128, d_h=128, d_c=512, d_c^Q=1536, d_R=64, "
                       "B=64, 2048 cached tokens + 1, bf16 weights and cache)",
           "steps": out, "chain_us": round(chain_us, 2), "chain_bytes_algorithmic": int(total_bytes),
           "chain_GBps": round(total_bytes / chain_us / 1e3, 1),
           "chain_roofline_frac": round(total_bytes / chain_us / 1e3 / HBM_PEAK_GBPS, 4),
           "sequences_per_s": round(B / (chain_us * 1e-6), 1),
           "chain_schedule": "one stream; stacked projections with a fixed summation order, "
                             "the cache append in the first one's summing launch; the query "
                             "side in one launch; combine fused with W^UV",
           "chain_bit_identical_reruns": rerun_identical,
           "chain_atomic_projections_us": round(atomic_us, 2),
           "atomic_vs_deterministic_max_rel_diff_u": round(atomic_vs_det, 6),
           "chain_two_launch_query_us": round(two_launch_us, 2),
           "two_launch_query_vs_one_max_rel_diff_u": round(two_vs_one, 6),
           "chain_unfused_combine_us": round(unfused_us, 2),
           "chain_separate_append_us": round(split_append_us, 2),
           "separate_append_vs_fused_u_bit_identical": split_append_identical,
           "chain_separate_products_us": round(separate_us, 2)}
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


def fp8_rows(mla, torch, inp, num_cus, steps, n_copies):
    """The headline workload over fp8 latent rows (MLA_FP8: 656 bytes per token against
    1152): the bf16 cache quantised once on the GPU (outside the timing), then attention +
    combine (bf16 partials) and the attention alone, back to back over rotating copies.
    GB/s count the fp8 bytes actually stored; the bf16-equivalent rate counts 1152 bytes per
    token for comparison with the bf16 step."""
    dev = torch.device("cuda:0")
    B, H, T = 32, 128, 4096
    S = mla.mla_suggest_num_splits(B, T, 0, 64, num_cus)
    src = inp["cache"].to(dev)
    caches = [torch.empty(src.shape[:-1] + (656,), dtype=torch.uint8, device=dev)]
    mla.mla_quantize_cache(src, caches[0])
    del src
    for _ in range(n_copies - 1):
        caches.append(caches[0].clone())
    q_lat, q_pe = inp["q_lat"].to(dev), inp["q_pe"].to(dev)
    bt, sl = inp["block_table"].to(dev), inp["seq_lens"].to(dev)
    o_part = torch.empty(B, H, S, 512, device=dev, dtype=torch.bfloat16)
    lse_part = torch.empty(B, H, S, device=dev)
    out = torch.empty(B, H, 512, device=dev)
    lse = torch.empty(B, H, device=dev)
    calls = [mla.bind(mla.mla_decode_attn_planned, q_lat, q_pe, c, bt, sl, inp["scale"], S, o_part,
                      lse_part) for c in caches]
    heads = [mla.bind(mla.mla_decode_attn_planned, q_lat, q_pe, c, bt, sl, inp["scale"], S, o_part,
                      lse_part, kernel="heads") for c in caches]
    combine = mla.bind(mla.mla_splitk_combine, o_part, lse_part, out, lse)
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < 0.3:
        calls[k % n_copies]()
        combine()
        k += 1
        if k % 32 == 0:
            torch.cuda.synchronize()
    step_ms = timed_ms(torch, lambda k: (calls[k % n_copies](), combine()), steps)
    attn_ms = timed_ms(torch, lambda k: calls[k % n_copies](), steps)
    heads_ms = timed_ms(torch, lambda k: heads[k % n_copies](), steps)
    tokens = B * T
    fp8_bytes = tokens * 656
    attn_bytes = fp8_bytes + B * H * 576 * 2 + bt.numel() * 4 + B * 4
    del caches
    return {"workload": "dsv2_b32_t4k over fp8 latent rows (MLA_FP8, 656 B per token)",
            "num_splits": S, "attention_kernel": "wide (32 heads per wavefront)",
            "us_per_step": round(step_ms * 1e3, 2), "attn_us": round(attn_ms * 1e3, 2),
            "attn_us_heads_kernel": round(heads_ms * 1e3, 2),
            "cache_bytes": fp8_bytes, "cache_GBps_step": round(fp8_bytes / (step_ms * 1e-3) / 1e9, 1),
            "attn_GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1),
            "attn_frac": round(attn_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "bf16_equivalent_GBps_step": round(tokens * ROW_BYTES / (step_ms * 1e-3) / 1e9, 1),
            "query_tokens_per_s": round(B / (step_ms * 1e-3), 1)}


def prefill_row(mla, torch, steps, T=4096, H=128):
    """Prefill attention in the expanded form (mla_prefill_attn) over one prompt of T tokens
    with H heads: q^C, k^C, v^C [T, H, 128], q_pe [T, H, 64], k_pe [T, 64], seeded bf16, resident
    in HBM.  Matrix-core bound: causal flops = H * T (T + 1) / 2 * (192 + 128) * 2, reported
    against the 2.5 PF bf16 dense peak."""
    dev = torch.device("cuda:0")
    g = torch.Generator(device="cpu").manual_seed(7)
    mk = lambda *shape: torch.randn(*shape, generator=g).to(torch.bfloat16).to(dev)
    q_c, q_pe, k_c, v_c = mk(1, T, H, 128), mk(1, T, H, 64), mk(1, T, H, 128), mk(1, T, H, 128)
    k_pe = mk(1, T, 64)
    out = torch.empty(1, T, H, 128, device=dev)
    call = mla.bind(mla.mla_prefill_attn, q_c, q_pe, k_c, k_pe, v_c, 1.0 / math.sqrt(192), out)
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < 0.3:
        call()
        torch.cuda.synchronize()
    ms = timed_ms(torch, lambda k: call(), max(5, steps // 5))
    flops = H * T * (T + 1) / 2 * (192 + 128) * 2
    return {"workload": f"prefill_t{T}_h{H} (one prompt, expanded form, causal)",
            "T": T, "H": H, "us": round(ms * 1e3, 1),
            "tflops": round(flops / (ms * 1e-3) / 1e12, 1),
            "mfma_frac_of_peak": round(flops / (ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "prompt_tokens_per_s": round(T / (ms * 1e-3), 1)}


def config_row(mla, torch, inp, name, num_cus, steps, n_copies, kernel="auto", flattened=False):
    """One attention workload beside the headline, back to back over n_copies rotating
    caches: the split-grid step (attention + combine, bf16 partials), its attention alone,
    mla_decode_fused (one launch that merges its splits, when the grid fits the device at
    once) and mla_decode_ragged (the flattened work list: one equal page range per compute
    unit, then the combine).  us_per_step is the flattened list's when `flattened`, else the
    split grid's.  Algorithmic bytes: cache rows of every sequence, queries, tables, and the
    combined output for the step; fractions of the 8 TB/s HBM roofline."""
    dev = torch.device("cuda:0")
    B, H, d_c = inp["q_lat"].shape
    sl = inp["seq_lens"]
    S = mla.mla_suggest_num_splits(B, int(sl.max()), int(sl.sum()), 64, num_cus)
    caches = [inp["cache"].to(dev)]
    for _ in range(n_copies - 1):
        caches.append(caches[0].clone())
    q_lat, q_pe = inp["q_lat"].to(dev), inp["q_pe"].to(dev)
    bt, sld = inp["block_table"].to(dev), sl.to(dev)
    o_part = torch.empty(B, H, S, d_c, device=dev, dtype=torch.bfloat16)
    lse_part = torch.empty(B, H, S, device=dev)
    out = torch.empty(B, H, d_c, device=dev)
    lse = torch.empty(B, H, device=dev)
    counters = mla.merge_counters(B)
    calls = [mla.bind(mla.mla_decode_attn_planned, q_lat, q_pe, c, bt, sld, inp["scale"], S,
                      o_part, lse_part, kernel=kernel) for c in caches]
    combine = mla.bind(mla.mla_splitk_combine, o_part, lse_part, out, lse)
    fused = [mla.bind(mla.mla_decode_fused, q_lat, q_pe, c, bt, sld, inp["scale"], S, o_part,
                      lse_part, counters, out, lse) for c in caches]
    t0 = time.perf_counter()
    k = 0
    while time.perf_counter() - t0 < 0.3:
        calls[k % n_copies]()
        combine()
        fused[k % n_copies]()
        k += 1
        if k % 32 == 0:
            torch.cuda.synchronize()
    split_ms = timed_ms(torch, lambda k: (calls[k % n_copies](), combine()), steps)
    attn_ms = timed_ms(torch, lambda k: calls[k % n_copies](), steps)
    fused_ms = timed_ms(torch, lambda k: fused[k % n_copies](), steps)
    # the flattened work list: one equal page range per compute unit
    ws = torch.empty(mla.mla_decode_ragged_workspace_bytes(caches[0], bt, H, d_c), dtype=torch.uint8,
                     device=dev)
    flat = [mla.bind(mla.mla_decode_ragged, q_lat, q_pe, c, bt, sld, inp["scale"], ws, out, lse)
            for c in caches]
    for k in range(2 * n_copies):
        flat[k % n_copies]()
    torch.cuda.synchronize()
    flat_ms = timed_ms(torch, lambda k: flat[k % n_copies](), steps)
    fp8_ms = None
    if flattened:  # the same work list over fp8 rows (quantised on the GPU, outside the timing)
        f8 = []
        for c in caches:
            f8.append(torch.empty(c.shape[:-1] + (656,), dtype=torch.uint8, device=dev))
            mla.mla_quantize_cache(c, f8[-1])
        flat8 = [mla.bind(mla.mla_decode_ragged, q_lat, q_pe, c, bt, sld, inp["scale"], ws, out, lse)
                 for c in f8]
        for k in range(2 * n_copies):
            flat8[k % n_copies]()
        torch.cuda.synchronize()
        fp8_ms = timed_ms(torch, lambda k: flat8[k % n_copies](), steps)
        del flat8, f8
    step_ms = flat_ms if flattened else split_ms
    tokens = int(sl.sum())
    attn_bytes = tokens * ROW_BYTES + B * H * 576 * 2 + bt.numel() * 4 + B * 4
    step_bytes = attn_bytes + B * H * 512 * 4
    single = bool(mla.mla_decode_fused_single_launch(mla.paged_shape(inp["cache"], inp["block_table"], H, d_c),
                                                     1, S))
    del caches
    return {"workload": name, "B": B, "H": H, "tokens": tokens, "num_splits": S,
            "path": "mla_decode_ragged (flattened work list)" if flattened
                    else "mla_decode (split grid: attention + combine)",
            "us_per_step": round(step_ms * 1e3, 2), "attn_us": round(attn_ms * 1e3, 2),
            "us_split_grid": round(split_ms * 1e3, 2), "us_flattened": round(flat_ms * 1e3, 2),
            "us_one_launch_merge": round(fused_ms * 1e3, 2) if single else None,
            "cache_GBps_step": round(tokens * ROW_BYTES / (step_ms * 1e-3) / 1e9, 1),
            "step_frac": round(step_bytes / (step_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "attn_GBps": round(attn_bytes / (attn_ms * 1e-3) / 1e9, 1),
            "attn_frac": round(attn_bytes / (attn_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "query_tokens_per_s": round(B / (step_ms * 1e-3), 1),
            "us_flattened_fp8_rows": round(fp8_ms * 1e3, 2) if fp8_ms else None,
            "fp8_cache_GBps": round(tokens * 656 / (fp8_ms * 1e-3) / 1e9, 1) if fp8_ms else None}


def _us(ms):
    """milliseconds -> microseconds rounded, None for a region not timed (NaN)"""
    return None if ms != ms else round(ms * 1e3, 2)


def timed_ms(torch, fn, n):
    """Average milliseconds of n back-to-back calls fn(0..n-1) between two HIP events on the
    current stream (the stream the library launches on)."""
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record()
    for k in range(n):
        fn(k)
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / n


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--warmup-seconds", type=float, default=0.5,
                    help="keep warming up until this much time has passed (clocks settle)")
    ap.add_argument("--splits", type=int, default=0, help="split count (0: library suggestion)")
    ap.add_argument("--kernel", default="auto", choices=["auto", "wide", "heads", "cols"],
                    help="attention kernel of the step (auto: the library's choice, the kernel "
                         "with 32 heads per wavefront for 128 heads)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seqs", type=int, default=32)
    ap.add_argument("--cpu-baseline-only", action="store_true",
                    help="(internal) time only the oracle on the host and print its JSON")
    ap.add_argument("--no-layer", action="store_true", help="skip the per-step layer measurement")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the long-context and ragged-batch attention lines")
    ap.add_argument("--layer-only", action="store_true",
                    help="run only the full-layer measurement and print its JSON (for profiling "
                         "the layer's kernels)")
    ap.add_argument("--config", choices=["long_b4_t32k", "ragged_b128"], default=None,
                    help="run only this workload line and print its JSON (for a kernel trace)")
    ap.add_argument("--headline-only", action="store_true",
                    help="time only the headline step and its attention alone (for a kernel "
                         "trace of exactly those launches)")
    ap.add_argument("--prefill-only", action="store_true",
                    help="time only the prefill attention (for a kernel trace of its launches)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="also run a plain 1 GiB device copy (counter calibration for --pmc runs)")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the decode path here has no multi-GPU mode "
              "(sequences shard across GPUs with no communication); run with --gpus 1.",
              file=sys.stderr)
        sys.exit(2)

    if args.cpu_baseline_only:
        import workloads as W
        print(json.dumps(cpu_baseline(W.dsv2_b32_t4k(), args.cpu_seqs)), flush=True)
        return

    import torch
    import head_latent_attention_15_amd as mla
    import workloads as W

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    props = torch.cuda.get_device_properties(dev)
    num_cus = props.multi_processor_count
    if args.config is not None:
        log(f"{args.config} only")
        gen = {"long_b4_t32k": (W.long_b4_t32k, N_CACHE_COPIES, False),
               "ragged_b128": (W.ragged_b128, 2, True)}[args.config]
        row = config_row(mla, torch, gen[0](), args.config, num_cus, args.steps, gen[1],
                         flattened=gen[2])
        print(json.dumps({args.config: row}), flush=True)
        return
    if args.prefill_only:
        log("prefill only")
        print(json.dumps({"prefill": prefill_row(mla, torch, args.steps)}), flush=True)
        return
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
    o_part_f32 = torch.empty(B, H, S, 512, device=dev)
    lse_part = torch.empty(B, H, S, device=dev)
    out = torch.empty(B, H, 512, device=dev)
    lse = torch.empty(B, H, device=dev)
    counters = mla.merge_counters(B)
    scale = inp["scale"]

    # arguments checked and marshalled once per cache copy, so the host issues each launch
    # in a few microseconds and the timed regions measure the GPU, not Python
    def attn_calls_for(kernel, part):
        return [mla.bind(mla.mla_decode_attn_planned, q_lat, q_pe, c, bt, sl, scale, S, part,
                         lse_part, kernel=kernel) for c in caches]

    def fused_calls_for(part):
        return [mla.bind(mla.mla_decode_fused, q_lat, q_pe, c, bt, sl, scale, S, part, lse_part,
                         counters, out, lse) for c in caches]
    attn_calls = attn_calls_for(args.kernel, o_part)          # the step: attention + combine
    combine = mla.bind(mla.mla_splitk_combine, o_part, lse_part, out, lse)
    attn_f32_calls = attn_calls_for(args.kernel, o_part_f32)  # the same with fp32 partials
    combine_f32 = mla.bind(mla.mla_splitk_combine, o_part_f32, lse_part, out, lse)
    fused_calls = fused_calls_for(o_part)  # one launch that merges the splits itself
    kernel = "wide" if args.kernel == "auto" else args.kernel  # the library's choice at H = 128
    other = "heads" if kernel != "heads" else "wide"  # timed alone beside it
    other_calls = attn_calls_for(other, o_part)

    def step_fused(k):
        fused_calls[k % N_CACHE_COPIES]()

    def attn(k):
        attn_calls[k % N_CACHE_COPIES]()

    # at least W warmup steps, and at least --warmup-seconds of them: the first tens of
    # milliseconds of back-to-back launches run at lower clocks than the steady state
    t_w = time.perf_counter()
    k = 0
    while k < args.warmup or time.perf_counter() - t_w < args.warmup_seconds:
        attn(k)
        combine()
        if not args.headline_only:
            attn_f32_calls[k % N_CACHE_COPIES]()
            combine_f32()
            step_fused(k)
            other_calls[k % N_CACHE_COPIES]()
        k += 1
        if k % 32 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    log(f"warmup {k} steps ({time.perf_counter() - t_w:.2f} s), S={S}, {num_cus} CUs")

    ms_step = timed_ms(torch, lambda k: (attn(k), combine()), args.steps)
    # the other timed regions, each back to back with events at the ends only (an event
    # recorded between two kernels stalls the queue for several microseconds, so
    # per-kernel events would time the stall with the kernel)
    if args.headline_only:
        ms_step_f32 = ms_fused = other_avg = float("nan")
    else:
        ms_step_f32 = timed_ms(torch, lambda k: (attn_f32_calls[k % N_CACHE_COPIES](), combine_f32()),
                               args.steps)
        ms_fused = timed_ms(torch, step_fused, args.steps)
    attn_avg = timed_ms(torch, attn, args.steps)
    comb_avg = timed_ms(torch, lambda k: combine(), args.steps)
    if not args.headline_only:
        other_avg = timed_ms(torch, lambda k: other_calls[k % N_CACHE_COPIES](), args.steps)
    c = counters.cpu()
    if int(c[-1]) != 0 or int(c[:-1].abs().sum()) != 0 or not bool(torch.isfinite(out).all()):
        raise RuntimeError("in-launch merge left its counters set or a non-finite output")
    log(f"step (attention + combine) {ms_step * 1e3:.1f} us, fp32 partials "
        f"{ms_step_f32 * 1e3:.1f} us; one launch merging its splits {ms_fused * 1e3:.1f} us; "
        f"attention alone {attn_avg * 1e3:.1f} us "
        f"({other} kernel {other_avg * 1e3:.1f} us); combine alone {comb_avg * 1e3:.1f} us")

    # streaming reads of the cache copies: the practical HBM read ceilings, with plain
    # vector loads and with the LDS DMA copy the attention kernels stage tiles with
    sink = torch.empty(4096, device=dev)
    cache_nbytes = caches[0].numel() * 2

    def stream_gbps(fn):
        for j in range(3):
            fn(caches[j % N_CACHE_COPIES], sink)
        reps = 12
        ms = timed_ms(torch, lambda k: fn(caches[k % N_CACHE_COPIES], sink), reps)
        return cache_nbytes / (ms * 1e-3) / 1e9
    stream_gbps_plain = stream_gbps(mla.mla_stream_read)
    stream_gbps_lds = stream_gbps(mla.mla_stream_read_lds)

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
    # what the attention alone must move: the cache rows, the queries, the block table and
    # the lengths (split partials are an implementation choice and are not counted)
    attn_alg_bytes = cache_bytes + B * H * 576 * 2 + bt.numel() * 4 + B * 4
    # the dominant kernel of the step is the attention: its algorithmic bytes per launch
    # over its average back-to-back launch duration
    achieved = attn_alg_bytes / attn_s / 1e9
    traffic = measured_traffic(kernel)
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
                   "split_merge": "combine kernel (mla_splitk_combine)",
                   "attention_kernel": kernel,
                   "cache_copies": N_CACHE_COPIES, "parallelism": "none"},
        "tflops": round(flops / (ms_step * 1e-3) / 1e12, 2),
        "query_tokens_per_s": round(B / (ms_step * 1e-3), 1),
        "step_bytes_algorithmic": step_alg_bytes,
        "step_frac": round(step_alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        # the whole step against the HBM roofline: the figure the headline value is;
        # roofline.frac below is the attention kernel alone
        "step_us_f32_partials": _us(ms_step_f32),
        "step_us_one_launch_merge": _us(ms_fused),
        "attn_us": round(attn_avg * 1e3, 2),
        "combine_us": round(comb_avg * 1e3, 2),
        f"attn_us_{other}_kernel": _us(other_avg),
        "attn_tflops": round(flops / attn_s / 1e12, 2),
        "mfma_frac_of_peak": round(flops / attn_s / 1e12 / BF16_PEAK_TFLOPS, 4),
        "stream_read_GBps": round(stream_gbps_plain, 1),
        "stream_read_lds_dma_GBps": round(stream_gbps_lds, 1),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic,
                     "frac_of_lds_dma_ceiling": round(achieved / stream_gbps_lds, 4),
                     # frac is the attention kernel alone; the whole step (attention +
                     # combine, algorithmic bytes over ms_per_step) is step_frac, the figure
                     # value and ms_per_step describe
                     "step_frac": round(step_alg_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
                     "frac_applies_to": "attention kernel alone (step_frac: attention + combine)",
                     "kernel": KERNEL_NAMES[kernel],
                     "bytes_per_launch_algorithmic": attn_alg_bytes},
    }
    del caches
    if args.headline_only:
        print(json.dumps(result), flush=True)
        return
    if not args.no_configs:
        log("timing long_b4_t32k and ragged_b128")
        result["long_b4_t32k"] = config_row(mla, torch, W.long_b4_t32k(), "long_b4_t32k", num_cus,
                                            args.steps, N_CACHE_COPIES)
        result["ragged_b128"] = config_row(mla, torch, W.ragged_b128(), "ragged_b128", num_cus,
                                           args.steps, 2, flattened=True)
    log("timing the headline workload over fp8 latent rows")
    result["fp8_cache"] = fp8_rows(mla, torch, inp, num_cus, args.steps, N_CACHE_COPIES)
    log("timing prefill attention (expanded form, T=4096, H=128)")
    result["prefill"] = prefill_row(mla, torch, args.steps)
    log("timing multi-token decode (2 query tokens per sequence)")
    caches = [inp["cache"].to(dev)]
    for _ in range(N_CACHE_COPIES - 1):
        caches.append(caches[0].clone())
    result["multi_token"] = multi_token_rows(mla, W, torch, caches, bt, sl, scale, num_cus)
    del caches
    if not args.no_cpu_baseline:
        log(f"timing the fp64 oracle on {args.cpu_seqs} sequences (all cores, then 1 thread)")
        cb = cpu_baseline(inp, args.cpu_seqs)
        cb["single_thread"] = cpu_baseline_child(args.cpu_seqs, 1)
        result["cpu_baseline"] = cb
    if not args.no_layer:
        log("timing every step of the path on the full decode layer")
        result["layer_b64_t2k"] = layer_rows(mla, W, torch, 0 if args.no_cpu_baseline else 4)
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
