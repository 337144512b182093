"""Seeded synthetic inputs for the MLA decode workloads.

This module only draws random numbers and lays them out; it holds none of the
method's arithmetic (no RoPE, no projections, no softmax).  Both the HIP path and
the fp64 oracle consume exactly the tensors made here: the oracle converts them to
float64 (exact for bf16 and fp32), the HIP path copies them to the device.

Every generator uses its own torch.Generator seeded with the workload's seed, and
draws in a fixed, documented order.  bf16 values are fp32 normals rounded to
nearest-even by ``Tensor.to(torch.bfloat16)``.

Workloads (names follow the shapes they carry):
  tiny_fp32        B=1, H=4, d_c=64, d_h=32, d_R=16, T=256, fp32, contiguous cache
  dsv2_b32_t4k     B=32, H=128, d_c=512, d_R=64, T=4096, bf16, identity page table
  long_b4_t32k     B=4, T=32768, pages a seeded permutation of the pool
  ragged_b128      B=128, seq_lens ~ U{128..8192}, shared pool, random permutation
  layer_b64_t2k    full decode layer, d=5120, bf16 weights, B=64, 2048 prior tokens
plus ``paged_attention`` for arbitrary smaller shapes used by the parity tests.
"""

from __future__ import annotations

import math
from dataclasses import dataclass

import torch

PAGE = 64


def _gen(seed: int) -> torch.Generator:
    g = torch.Generator(device="cpu")
    g.manual_seed(int(seed))
    return g


def _normal(g, shape, std=1.0, dtype=torch.bfloat16):
    x = torch.randn(*shape, generator=g, dtype=torch.float32)
    if std != 1.0:
        x = x * std
    return x.to(dtype)


@dataclass
class Shape:
    B: int
    H: int
    d_c: int
    d_R: int
    d_h: int = 128
    page_size: int = PAGE


def identity_block_table(B: int, pages_per_seq: int) -> torch.Tensor:
    """Sequence b owns pages b*pages_per_seq .. (b+1)*pages_per_seq - 1, in order."""
    return torch.arange(B * pages_per_seq, dtype=torch.int32).reshape(B, pages_per_seq)


def paged_attention(seed: int, B: int, H: int, seq_lens, d_c: int = 512, d_R: int = 64,
                    d_h: int = 128, page_size: int = PAGE, dtype=torch.bfloat16,
                    permute_pages: bool = True, extra_pages: int = 0,
                    max_pages: int | None = None):
    """Random latent-attention problem over a paged pool.

    Draw order: page permutation (if permute_pages), cache, q_lat, q_pe.
    seq_lens: list of ints.  Pool = sum ceil(len/P) pages + extra_pages (never referenced).
    Unused block-table entries are -1.
    """
    g = _gen(seed)
    seq_lens = [int(s) for s in seq_lens]
    need = [max(0, math.ceil(s / page_size)) for s in seq_lens]
    n_pages = sum(need) + extra_pages
    maxp = max(1, max(need) if need else 1) if max_pages is None else max_pages
    perm = torch.randperm(n_pages, generator=g) if permute_pages else torch.arange(n_pages)
    bt = torch.full((B, maxp), -1, dtype=torch.int32)
    k = 0
    for b in range(B):
        for p in range(need[b]):
            bt[b, p] = int(perm[k])
            k += 1
    cache = _normal(g, (max(n_pages, 1), page_size, d_c + d_R), dtype=dtype)
    q_lat = _normal(g, (B, H, d_c), dtype=dtype)
    q_pe = _normal(g, (B, H, d_R), dtype=dtype)
    return {
        "cache": cache, "q_lat": q_lat, "q_pe": q_pe, "block_table": bt,
        "seq_lens": torch.tensor(seq_lens, dtype=torch.int32),
        "shape": Shape(B=B, H=H, d_c=d_c, d_R=d_R, d_h=d_h, page_size=page_size),
        "scale": 1.0 / math.sqrt(d_h + d_R),
    }


def tiny_fp32(seed: int = 1):
    """B=1, H=4, d_c=64, d_h=32, d_R=16, T=256, fp32.  Draw order: c_kv, k_r, q_c, q_r,
    W^UK, W^UV.  c, k^R, q^C, q^R ~ N(0,1) (k^R, q^R before rotation); W ~ N(0, 1/sqrt(64)).
    The cache is contiguous: an identity table over 64-token pages."""
    g = _gen(seed)
    B, H, d_c, d_h, d_R, T = 1, 4, 64, 32, 16, 256
    f32 = torch.float32
    d = {
        "c_kv": _normal(g, (B, T, d_c), dtype=f32),
        "k_r": _normal(g, (B, T, d_R), dtype=f32),
        "q_c": _normal(g, (B, H, d_h), dtype=f32),
        "q_r": _normal(g, (B, H, d_R), dtype=f32),
        "w_uk": _normal(g, (H * d_h, d_c), std=1.0 / math.sqrt(d_c), dtype=f32),
        "w_uv": _normal(g, (H * d_h, d_c), std=1.0 / math.sqrt(d_c), dtype=f32),
    }
    d.update(shape=Shape(B=B, H=H, d_c=d_c, d_R=d_R, d_h=d_h), T=T, rope_base=10000.0,
             scale=1.0 / math.sqrt(d_h + d_R),
             block_table=identity_block_table(B, T // PAGE),
             seq_lens_before=torch.zeros(B, dtype=torch.int32))
    return d


def dsv2_b32_t4k(seed: int = 2, B: int = 32, T: int = 4096, H: int = 128):
    """DeepSeek-V2-shaped decode: cache [B*T/64, 64, 576], q_lat [B,H,512], q_pe [B,H,64],
    all N(0,1) -> bf16; identity block table b*T/64 + p.  Draw order: cache, q_lat, q_pe."""
    g = _gen(seed)
    ppseq = T // PAGE
    cache = _normal(g, (B * ppseq, PAGE, 576))
    q_lat = _normal(g, (B, H, 512))
    q_pe = _normal(g, (B, H, 64))
    return {"cache": cache, "q_lat": q_lat, "q_pe": q_pe,
            "block_table": identity_block_table(B, ppseq),
            "seq_lens": torch.full((B,), T, dtype=torch.int32),
            "shape": Shape(B=B, H=H, d_c=512, d_R=64), "scale": 1.0 / math.sqrt(192)}


def multi_queries(seed: int, B: int, n_q: int, H: int, d_c: int = 512, d_R: int = 64,
                  dtype=torch.bfloat16):
    """Absorbed queries for n_q new tokens per sequence (multi-token decode): q~
    [B, n_q, H, d_c] and q_pe [B, n_q, H, d_R] ~ N(0,1), drawn in that order."""
    g = _gen(seed)
    return _normal(g, (B, n_q, H, d_c), dtype=dtype), _normal(g, (B, n_q, H, d_R), dtype=dtype)


def long_b4_t32k(seed: int = 3, B: int = 4, T: int = 32768, H: int = 128):
    """Long context: seq b reads pages perm[512b .. 512b+511] of a 2048-page pool.
    Draw order: permutation, cache, q_lat, q_pe."""
    g = _gen(seed)
    ppseq = T // PAGE
    perm = torch.randperm(B * ppseq, generator=g).to(torch.int32)
    cache = _normal(g, (B * ppseq, PAGE, 576))
    q_lat = _normal(g, (B, H, 512))
    q_pe = _normal(g, (B, H, 64))
    return {"cache": cache, "q_lat": q_lat, "q_pe": q_pe,
            "block_table": perm.reshape(B, ppseq).contiguous(),
            "seq_lens": torch.full((B,), T, dtype=torch.int32),
            "shape": Shape(B=B, H=H, d_c=512, d_R=64), "scale": 1.0 / math.sqrt(192)}


def ragged_b128(seed: int = 4, B: int = 128, lo: int = 128, hi: int = 8192, H: int = 128):
    """Ragged batch: seq_lens ~ U{lo..hi} inclusive; pool of sum ceil(len/64) pages,
    randomly permuted and handed out to sequences in order; max 128 pages per sequence,
    unused entries -1.  Draw order: seq_lens, permutation, cache, q_lat, q_pe."""
    g = _gen(seed)
    seq_lens = torch.randint(lo, hi + 1, (B,), generator=g, dtype=torch.int64).to(torch.int32)
    need = [math.ceil(int(s) / PAGE) for s in seq_lens]
    n_pages = sum(need)
    perm = torch.randperm(n_pages, generator=g).to(torch.int32)
    maxp = math.ceil(hi / PAGE)
    bt = torch.full((B, maxp), -1, dtype=torch.int32)
    k = 0
    for b in range(B):
        bt[b, :need[b]] = perm[k:k + need[b]]
        k += need[b]
    cache = _normal(g, (n_pages, PAGE, 576))
    q_lat = _normal(g, (B, H, 512))
    q_pe = _normal(g, (B, H, 64))
    return {"cache": cache, "q_lat": q_lat, "q_pe": q_pe, "block_table": bt,
            "seq_lens": seq_lens, "shape": Shape(B=B, H=H, d_c=512, d_R=64),
            "scale": 1.0 / math.sqrt(192)}


LAYER_WEIGHTS = ("w_dq", "w_uq", "w_qr", "w_dkv", "w_kr", "w_uk", "w_uv", "w_o")


def layer_b64_t2k(seed: int = 5, B: int = 64, T: int = 2048, d: int = 5120, H: int = 128,
                  d_h: int = 128, d_c: int = 512, d_cq: int = 1536, d_R: int = 64):
    """Full decode layer.  h [B, d] ~ N(0,1); weights nn.Linear [out, in] with
    std 1/sqrt(in); prior cache rows (tokens 0..T-1, rotated k^R) ~ N(0,1); all bf16.
    Pages: sequence b owns ceil((T+1)/64) consecutive pages so the new token fits.
    Draw order: h, w_dq, w_uq, w_qr, w_dkv, w_kr, w_uk, w_uv, w_o, cache."""
    g = _gen(seed)
    shapes = {"w_dq": (d_cq, d), "w_uq": (H * d_h, d_cq), "w_qr": (H * d_R, d_cq),
              "w_dkv": (d_c, d), "w_kr": (d_R, d), "w_uk": (H * d_h, d_c),
              "w_uv": (H * d_h, d_c), "w_o": (d, H * d_h)}
    h = _normal(g, (B, d))
    weights = {k: _normal(g, shapes[k], std=1.0 / math.sqrt(shapes[k][1])) for k in LAYER_WEIGHTS}
    ppseq = math.ceil((T + 1) / PAGE)
    cache = _normal(g, (B * ppseq, PAGE, d_c + d_R))
    return {"h": h, "weights": weights, "cache": cache,
            "block_table": identity_block_table(B, ppseq),
            "seq_lens_before": torch.full((B,), T, dtype=torch.int32),
            "shape": Shape(B=B, H=H, d_c=d_c, d_R=d_R, d_h=d_h), "d": d, "d_cq": d_cq,
            "rope_base": 10000.0, "scale": 1.0 / math.sqrt(d_h + d_R)}


def to_f64(t: torch.Tensor):
    """Exact widening for the oracle (bf16 and fp32 embed in fp64)."""
    return t.to(torch.float64).numpy()
