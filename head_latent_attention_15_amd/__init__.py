"""MI355X (gfx950) weight-absorbed MLA decode.

Thin ctypes binding of ``libmla.so`` (C ABI in ``include/mla.h``).  Every step of the
decode path runs in the library's HIP kernels; this module only checks torch tensors
(device, dtype, contiguity, shapes), passes their device pointers and the current HIP
stream, and raises :class:`MLAError` on a non-OK status.  PyTorch is used for device
memory and streams only.  There is no fallback: if the library is missing, importing the
bindings raises.
"""
from __future__ import annotations

import ctypes
import os
import re

# torch first: it ships its own libamdhip64 (SONAME libamdhip64.so.7).  Loaded before
# libmla.so, that copy satisfies libmla's dependency, so the process has one HIP runtime
# and libmla's kernels run on torch's device context and streams.
import torch  # noqa: F401

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libmla.so")
HEADER_PATH = os.path.join(os.path.dirname(_PKG), "include", "mla.h")

MLA_OK, MLA_ERR_NULL, MLA_ERR_SHAPE, MLA_ERR_UNSUPPORTED = 0, 1, 2, 3
MLA_ERR_WORKSPACE, MLA_ERR_LAUNCH, MLA_ERR_INDEX = 4, 5, 6
MLA_F32, MLA_BF16, MLA_FP8 = 0, 1, 2


class MLAError(RuntimeError):
    def __init__(self, status: int, detail: str):
        super().__init__(f"{_status_name(status)}: {detail}")
        self.status = status
        self.detail = detail


class _PagedShape(ctypes.Structure):
    _fields_ = [("batch", ctypes.c_int32), ("num_heads", ctypes.c_int32),
                ("d_latent", ctypes.c_int32), ("d_rope", ctypes.c_int32),
                ("page_size", ctypes.c_int32), ("max_pages_per_seq", ctypes.c_int32),
                ("num_pages", ctypes.c_int32)]


_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_F = ctypes.c_float
_SZ = ctypes.c_size_t
_SP = ctypes.POINTER(_PagedShape)

_SIGNATURES = {
    "mla_cache_bytes": (_SZ, [_I64, _I64, _I64, _I32, _I32, _I32]),
    "mla_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32]),
    "mla_suggest_num_splits": (_I32, [_I32, _I32, _I64, _I32, _I32]),
    "mla_absorb_q": (_I32, [_P, _P, _P, _P, _F, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                            _I32, _P]),
    "mla_absorb_q_strided": (_I32, [_P, _I64, _P, _P, _I64, _P, _F, _P, _P, _I32, _I32, _I32,
                                    _I32, _I32, _I32, _I32, _P]),
    "mla_pack_query_weights": (_I32, [_P, _P, _P, _I32, _I32, _P, _P]),
    "mla_query_path": (_I32, [_P, _I64, _P, _P, _F, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                              _P]),
    "mla_kv_append": (_I32, [_P, _P, _I32, _P, _P, _P, _F, _SP, _I32, _P]),
    "mla_kv_append_strided": (_I32, [_P, _I64, _P, _I64, _I32, _P, _P, _P, _F, _SP, _I32, _P]),
    "mla_decode_attn": (_I32, [_P, _P, _P, _P, _P, _SP, _F, _I32, _P, _I32, _P, _I32, _P]),
    "mla_decode_attn_multi": (_I32, [_P, _P, _P, _P, _P, _SP, _I32, _F, _I32, _P, _I32, _P, _I32,
                                     _P]),
    "mla_decode_attn_planned": (_I32, [_P, _P, _P, _P, _P, _SP, _I32, _F, _I32, _P, _I32, _P,
                                       _I32, _I32, _P]),
    "mla_decode_fused": (_I32, [_P, _P, _P, _P, _P, _SP, _I32, _F, _I32, _P, _I32, _P, _P, _P,
                                _P, _I32, _P]),
    "mla_decode_fused_single_launch": (_I32, [_SP, _I32, _I32]),
    "mla_decode_ragged_workspace_bytes": (_SZ, [_SP]),
    "mla_decode_ragged": (_I32, [_P, _P, _P, _P, _P, _SP, _F, _P, _SZ, _P, _P, _I32, _P]),
    "mla_splitk_combine": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "mla_fold_uq": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P]),
    "mla_quantize_cache": (_I32, [_P, _I32, _I64, _I64, _P, _P]),
    "mla_prefill_attn": (_I32, [_P, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32, _F, _P, _P, _I32,
                                _P]),
    "mla_fold_o_uv": (_I32, [_P, _P, _I32, _I32, _I32, _I32, _I32, _P, _I32, _P]),
    "mla_combine_out_proj": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _I32, _P, _I32, _I32, _P,
                                    _P]),
    "mla_decode": (_I32, [_P, _P, _P, _P, _P, _SP, _F, _I32, _P, _SZ, _P, _P, _I32, _P]),
    "mla_decode_noalloc": (_I32, [_P, _P, _P, _P, _P, _SP, _F, _I32, _P, _P, _I32, _P]),
    "mla_out_proj": (_I32, [_P, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _P, _P, _P]),
    "mla_linear": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _I32, _P, _P]),
    "mla_linear_deterministic_workspace_bytes": (_SZ, [_I32, _I32, _I32]),
    "mla_linear_deterministic": (_I32, [_P, _I32, _I64, _P, _I32, _I32, _I32, _I32, _P, _I64,
                                        _I32, _P, _SZ, _P]),
    "mla_linear_deterministic_append": (_I32, [_P, _I32, _I64, _P, _I32, _I32, _I32, _I32, _P,
                                               _I64, _P, _SZ, _I32, _P, _P, _P, _F, _SP, _I32,
                                               _P]),
    "mla_linear_strided": (_I32, [_P, _I32, _I64, _P, _I32, _I32, _I32, _I32, _P, _I64, _I32,
                                  _P]),
    "mla_linear_planned": (_I32, [_P, _I32, _P, _I32, _I32, _I32, _I32, _P, _I32, _I32, _I32,
                                  _I32, _P]),
    "mla_validate_indices": (_I32, [_P, _P, _SP, _P, _P]),
    "mla_stream_read": (_I32, [_P, _SZ, _P, _P]),
    "mla_stream_read_lds": (_I32, [_P, _SZ, _P, _P]),
    "mla_status_string": (ctypes.c_char_p, [_I32]),
    "mla_last_error_detail": (ctypes.c_char_p, []),
}


def header_functions() -> list[str]:
    """Names of the functions declared in include/mla.h."""
    text = open(HEADER_PATH).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mla_[a-z0-9_]+)\s*\(", text)))


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python head_latent_attention_15_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def _status_name(st: int) -> str:
    return lib.mla_status_string(st).decode()


def _check(st: int) -> None:
    if st != MLA_OK:
        raise MLAError(st, lib.mla_last_error_detail().decode())


_capture: list | None = None


def _invoke(name: str, *args) -> None:
    """Call lib.<name>(*args) and raise on a non-OK status; inside bind(), record instead."""
    if _capture is not None:
        _capture.append((name, args))
        return
    _check(getattr(lib, name)(*args))


class Bound:
    """A library call whose arguments were checked and marshalled once (see bind)."""

    def __init__(self, name: str, args: tuple):
        fn = getattr(lib, name)
        conv = []
        for a, t in zip(args, fn.argtypes):
            # plain Python numbers become ctypes values once; pointers stay NULL or as given
            conv.append(t(a) if isinstance(a, (int, float)) and not isinstance(a, bool) else a)
        self.name, self._fn, self._args = name, fn, tuple(conv)

    def __call__(self) -> None:
        _check(self._fn(*self._args))


def bind(fn, *args, **kwargs) -> Bound:
    """Check and marshal the arguments of one hot-path wrapper now; return a callable that
    repeats exactly that library call (same tensors, same stream) with no per-call Python
    checks.  The tensors must stay alive and in place while the Bound is used."""
    global _capture
    if _capture is not None:
        raise RuntimeError("bind() is not reentrant")
    _capture = []
    try:
        fn(*args, **kwargs)
        calls = _capture
    finally:
        _capture = None
    if len(calls) != 1:
        raise RuntimeError(f"{getattr(fn, '__name__', fn)} made {len(calls)} library calls")
    return Bound(*calls[0])


# ----------------------------------------------------------------------------- helpers
def _torch():
    import torch
    return torch


def _dtype_code(t) -> int:
    torch = _torch()
    if t.dtype == torch.float32:
        return MLA_F32
    if t.dtype == torch.bfloat16:
        return MLA_BF16
    raise TypeError(f"unsupported dtype {t.dtype}")


def _dev(t, name, dtype=None, ndim=None):
    """Device pointer of a contiguous GPU tensor (None -> NULL)."""
    if t is None:
        return None
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr()


def _row_stride(shape, stride, lead, name="tensor") -> int:
    """Row stride (elements) of a tensor whose first `lead` dims number rows at one common
    stride and whose other dims are dense within a row; raises ValueError otherwise."""
    width = 1
    for i in range(len(shape) - 1, lead - 1, -1):
        if shape[i] > 1 and stride[i] != width:
            raise ValueError(f"{name} must be dense within a row (strides {tuple(stride)})")
        width *= shape[i]
    ld, span = None, 1
    for i in range(lead - 1, -1, -1):
        if shape[i] > 1:
            if ld is None:
                ld = stride[i] // span if stride[i] % span == 0 else -1
            if ld <= 0 or stride[i] != ld * span:
                raise ValueError(f"{name}: rows must be evenly spaced (strides {tuple(stride)})")
        span *= shape[i]
    return ld if ld is not None else width


def _dev_rows(t, name, dtype, ndim, lead):
    """Device pointer and row stride of a GPU tensor laid out as _row_stride describes (a
    column range of a wider buffer, for instance)."""
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    return t.data_ptr(), _row_stride(t.shape, t.stride(), lead, name)


def _stream(stream):
    if stream is None:
        return _torch().cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def _expect(cond, msg):
    if not cond:
        raise ValueError(msg)


FP8_ROW_BYTES = 656  # MLA_FP8 cache rows: 512 E4M3 codes, 64 bf16 k^R, 4 fp32 scales


def is_fp8_cache(kv_cache) -> bool:
    """A uint8 cache of 656-byte rows (the MLA_FP8 format)."""
    torch = _torch()
    return kv_cache.dtype == torch.uint8 and kv_cache.shape[-1] == FP8_ROW_BYTES


def _cache_code(kv_cache) -> int:
    return MLA_FP8 if is_fp8_cache(kv_cache) else _dtype_code(kv_cache)


def _attn_code(q_lat, q_pe, kv_cache) -> int:
    """dtype code of an attention call: the shared dtype, or MLA_FP8 for bf16 queries over
    fp8 rows."""
    torch = _torch()
    if is_fp8_cache(kv_cache):
        _expect(q_lat.dtype == q_pe.dtype == torch.bfloat16, "fp8 rows take bf16 queries")
        return MLA_FP8
    _expect(q_pe.dtype == q_lat.dtype == kv_cache.dtype, "q_lat, q_pe, kv_cache share a dtype")
    return _dtype_code(q_lat)


def _check_row(kv_cache, d_c, d_R):
    if is_fp8_cache(kv_cache):
        _expect(d_c == 512 and d_R == 64, "fp8 rows hold d_c = 512 and d_R = 64")
    else:
        _expect(kv_cache.shape[2] == d_c + d_R, "cache row must be d_c + d_R wide")


def paged_shape(kv_cache, block_table, num_heads: int, d_latent: int) -> _PagedShape:
    pages, P, row = kv_cache.shape
    B, maxp = block_table.shape
    d_rope = 64 if is_fp8_cache(kv_cache) else row - d_latent
    return _PagedShape(B, num_heads, d_latent, d_rope, P, maxp, pages)


# ----------------------------------------------------------------------------- sizes
def mla_cache_bytes(B, T, layers, d_c, d_R, elem_bytes) -> int:
    return int(lib.mla_cache_bytes(B, T, layers, d_c, d_R, elem_bytes))


def mla_decode_workspace_bytes(B, H, d_c, num_splits) -> int:
    return int(lib.mla_decode_workspace_bytes(B, H, d_c, num_splits))


def mla_suggest_num_splits(B, max_seq_len, total_tokens=0, page_size=64, num_cus=256) -> int:
    return int(lib.mla_suggest_num_splits(B, max_seq_len, total_tokens, page_size, num_cus))


def mla_status_string(status: int) -> str:
    return _status_name(status)


def mla_last_error_detail() -> str:
    return lib.mla_last_error_detail().decode()


# ----------------------------------------------------------------------------- hot path
def mla_absorb_q(q_c, w_uk, q_r, seq_lens, rope_base, q_lat, q_pe, stream=None):
    """q_lat = W^UK_i^T q^C_i per head; q_pe = RoPE(q_r, seq_lens - 1).
    q_c [B,H,d_h] f32, w_uk [H*d_h, d_c], q_r [B,H,d_R] f32 or None, q_lat [B,H,d_c],
    q_pe [B,H,d_R] (q_lat / q_pe share one dtype)."""
    torch = _torch()
    B, H, d_h = q_c.shape
    d_c = w_uk.shape[1]
    _expect(w_uk.shape[0] == H * d_h, "w_uk must be [H*d_h, d_c]")
    _expect(tuple(q_lat.shape) == (B, H, d_c), "q_lat must be [B,H,d_c]")
    d_R = q_r.shape[2] if q_r is not None else 0
    if q_r is not None:
        _expect(tuple(q_r.shape) == (B, H, d_R) and tuple(q_pe.shape) == (B, H, d_R),
                "q_r and q_pe must be [B,H,d_R]")
        _expect(q_pe.dtype == q_lat.dtype, "q_pe and q_lat must share a dtype")
        _expect(tuple(seq_lens.shape) == (B,), "seq_lens must be [B]")
    _invoke("mla_absorb_q",
        _dev(q_c, "q_c", torch.float32, 3), _dev(w_uk, "w_uk", None, 2),
        _dev(q_r, "q_r", torch.float32, 3), _dev(seq_lens, "seq_lens", torch.int32, 1),
        float(rope_base), _dev(q_lat, "q_lat", None, 3), _dev(q_pe, "q_pe", None, 3),
        B, H, d_h, d_c, d_R, _dtype_code(w_uk), _dtype_code(q_lat), _stream(stream))


def mla_absorb_q_strided(q_c, w_uk, q_r, seq_lens, rope_base, q_lat, q_pe, stream=None):
    """mla_absorb_q reading q_c [B,H,d_h] and q_r [B,H,d_R] as row-strided views (each
    row's heads contiguous), e.g. column ranges of the stacked [W^UQ; W^QR] projection."""
    torch = _torch()
    B, H, d_h = q_c.shape
    d_c = w_uk.shape[1]
    _expect(w_uk.shape[0] == H * d_h, "w_uk must be [H*d_h, d_c]")
    _expect(tuple(q_lat.shape) == (B, H, d_c), "q_lat must be [B,H,d_c]")
    qc_ptr, ld_qc = _dev_rows(q_c, "q_c", torch.float32, 3, 1)
    qr_ptr, ld_qr, d_R = None, 0, 0
    if q_r is not None:
        d_R = q_r.shape[2]
        _expect(tuple(q_r.shape) == (B, H, d_R) and tuple(q_pe.shape) == (B, H, d_R),
                "q_r and q_pe must be [B,H,d_R]")
        _expect(q_pe.dtype == q_lat.dtype, "q_pe and q_lat must share a dtype")
        _expect(tuple(seq_lens.shape) == (B,), "seq_lens must be [B]")
        qr_ptr, ld_qr = _dev_rows(q_r, "q_r", torch.float32, 3, 1)
    _invoke("mla_absorb_q_strided",
        qc_ptr, ld_qc, _dev(w_uk, "w_uk", None, 2), qr_ptr, ld_qr,
        _dev(seq_lens, "seq_lens", torch.int32, 1), float(rope_base),
        _dev(q_lat, "q_lat", None, 3), _dev(q_pe, "q_pe", None, 3),
        B, H, d_h, d_c, d_R, _dtype_code(w_uk), _dtype_code(q_lat), _stream(stream))


def query_pack_elems(H, d_cq, d_h=128, d_R=64, d_c=512):
    """bf16 elements of the packed query-side weights (mla_pack_query_weights)."""
    return H * ((d_h + d_R) * d_cq + d_h * d_c)


def mla_pack_query_weights(w_uq, w_qr, w_uk, H, w_pack=None, stream=None):
    """Pack W^UQ [H*128, d_cq], W^QR [H*64, d_cq] and W^UK [H*128, 512] (bf16) into the
    layout mla_query_path reads; returns w_pack (a new bf16 tensor unless one is given)."""
    torch = _torch()
    d_cq = w_uq.shape[1]
    _expect(tuple(w_uq.shape) == (H * 128, d_cq) and tuple(w_qr.shape) == (H * 64, d_cq),
            "w_uq must be [H*128, d_cq] and w_qr [H*64, d_cq]")
    _expect(tuple(w_uk.shape) == (H * 128, 512), "w_uk must be [H*128, 512]")
    n = query_pack_elems(H, d_cq)
    if w_pack is None:
        w_pack = torch.empty(n, device=w_uq.device, dtype=torch.bfloat16)
    _expect(w_pack.numel() == n, f"w_pack must hold {n} elements")
    _invoke("mla_pack_query_weights",
        _dev(w_uq, "w_uq", torch.bfloat16, 2), _dev(w_qr, "w_qr", torch.bfloat16, 2),
        _dev(w_uk, "w_uk", torch.bfloat16, 2), H, d_cq, _dev(w_pack, "w_pack", torch.bfloat16),
        _stream(stream))
    return w_pack


def mla_query_path(c_q, w_pack, seq_lens, rope_base, q_lat, q_pe, stream=None):
    """The query side in one launch: q~_i = W^UK_i^T (W^UQ_i c^Q) into q_lat and
    RoPE(W^QR_i c^Q, seq_lens - 1) into q_pe.  c_q [B, d_cq] f32 (rows may be a column
    range of a wider buffer), w_pack from mla_pack_query_weights; q_lat [B,H,512],
    q_pe [B,H,64] bf16."""
    torch = _torch()
    B, d_cq = c_q.shape
    B2, H, d_c = q_lat.shape
    d_R = q_pe.shape[2]
    _expect(B2 == B and tuple(q_pe.shape) == (B, H, d_R), "q_lat / q_pe must be [B,H,*]")
    _expect(w_pack.numel() == query_pack_elems(H, d_cq, 128, d_R, d_c),
            "w_pack does not hold the packed weights of these sizes")
    _expect(tuple(seq_lens.shape) == (B,), "seq_lens must be [B]")
    cq_ptr, ld_cq = _dev_rows(c_q, "c_q", torch.float32, 2, 1)
    _invoke("mla_query_path",
        cq_ptr, ld_cq, _dev(w_pack, "w_pack", torch.bfloat16),
        _dev(seq_lens, "seq_lens", torch.int32, 1), float(rope_base),
        _dev(q_lat, "q_lat", torch.bfloat16, 3), _dev(q_pe, "q_pe", torch.bfloat16, 3),
        B, H, 128, d_R, d_c, d_cq, _stream(stream))


def mla_kv_append(c_kv, k_r, seq_lens_before, block_table, kv_cache, rope_base, stream=None):
    """Write [c_kv | RoPE(k_r, pos)] rows at positions seq_lens_before[b] + t.
    c_kv [B,n,d_c] f32, k_r [B,n,d_R] f32, kv_cache [pages, P, d_c + d_R]."""
    torch = _torch()
    B, n, d_c = c_kv.shape
    _expect(k_r.shape[0] == B and k_r.shape[1] == n, "k_r must be [B,n,d_R]")
    _check_row(kv_cache, d_c, k_r.shape[2])
    _expect(block_table.shape[0] == B and tuple(seq_lens_before.shape) == (B,), "batch mismatch")
    shp = paged_shape(kv_cache, block_table, 1, d_c)
    _invoke("mla_kv_append",
        _dev(c_kv, "c_kv", torch.float32, 3), _dev(k_r, "k_r", torch.float32, 3), n,
        _dev(seq_lens_before, "seq_lens_before", torch.int32, 1),
        _dev(block_table, "block_table", torch.int32, 2), _dev(kv_cache, "kv_cache", None, 3),
        float(rope_base), ctypes.byref(shp), _cache_code(kv_cache), _stream(stream))


def mla_kv_append_strided(c_kv, k_r, seq_lens_before, block_table, kv_cache, rope_base,
                          stream=None):
    """mla_kv_append reading c_kv [B,n,d_c] and k_r [B,n,d_R] as row-strided views (rows
    b n + t evenly spaced), e.g. column ranges of the stacked [W^DQ; W^DKV; W^KR] projection."""
    torch = _torch()
    B, n, d_c = c_kv.shape
    _expect(k_r.shape[0] == B and k_r.shape[1] == n, "k_r must be [B,n,d_R]")
    _check_row(kv_cache, d_c, k_r.shape[2])
    _expect(block_table.shape[0] == B and tuple(seq_lens_before.shape) == (B,), "batch mismatch")
    shp = paged_shape(kv_cache, block_table, 1, d_c)
    c_ptr, ld_c = _dev_rows(c_kv, "c_kv", torch.float32, 3, 2)
    k_ptr, ld_k = _dev_rows(k_r, "k_r", torch.float32, 3, 2)
    _invoke("mla_kv_append_strided", c_ptr, ld_c, k_ptr, ld_k, n,
        _dev(seq_lens_before, "seq_lens_before", torch.int32, 1),
        _dev(block_table, "block_table", torch.int32, 2), _dev(kv_cache, "kv_cache", None, 3),
        float(rope_base), ctypes.byref(shp), _cache_code(kv_cache), _stream(stream))


def mla_decode_attn(q_lat, q_pe, kv_cache, block_table, seq_lens, softmax_scale, num_splits,
                    o_part, lse_part=None, stream=None):
    """Split-K decode attention; o_part [B,H,S,d_c] (or [B,H,d_c] when S == 1), float32 or
    bfloat16 (the partial dtype follows the tensor), lse_part [B,H,S] (or [B,H] / None when
    S == 1)."""
    torch = _torch()
    B, H, d_c = q_lat.shape
    _expect(q_pe.shape[0] == B and q_pe.shape[1] == H, "q_pe must be [B,H,d_R]")
    code = _attn_code(q_lat, q_pe, kv_cache)
    _check_row(kv_cache, d_c, q_pe.shape[2])
    _expect(block_table.shape[0] == B and tuple(seq_lens.shape) == (B,), "batch mismatch")
    S = int(num_splits)
    want = (B, H, d_c) if S == 1 else (B, H, S, d_c)
    _expect(tuple(o_part.shape) == want or (S == 1 and tuple(o_part.shape) == (B, H, 1, d_c)),
            f"o_part must be {want}")
    if lse_part is not None:
        _expect(lse_part.numel() == B * H * S, "lse_part must hold B*H*S floats")
    shp = paged_shape(kv_cache, block_table, H, d_c)
    _invoke("mla_decode_attn",
        _dev(q_lat, "q_lat", None, 3), _dev(q_pe, "q_pe", None, 3),
        _dev(kv_cache, "kv_cache", None, 3), _dev(block_table, "block_table", torch.int32, 2),
        _dev(seq_lens, "seq_lens", torch.int32, 1), ctypes.byref(shp), float(softmax_scale), S,
        _dev(o_part, "o_part"), _dtype_code(o_part), _dev(lse_part, "lse_part", torch.float32),
        code, _stream(stream))



def mla_decode_attn_multi(q_lat, q_pe, kv_cache, block_table, seq_lens, softmax_scale,
                          num_splits, o_part, lse_part=None, stream=None):
    """Decode attention for n_q new tokens per sequence (causal among them): q_lat
    [B,n_q,H,d_c], q_pe [B,n_q,H,d_R]; o_part [B,n_q,H,S,d_c] (or [B,n_q,H,d_c] when S == 1),
    lse_part [B,n_q,H,S] (or None when S == 1)."""
    torch = _torch()
    B, n_q, H, d_c = q_lat.shape
    _expect(tuple(q_pe.shape[:3]) == (B, n_q, H), "q_pe must be [B,n_q,H,d_R]")
    code = _attn_code(q_lat, q_pe, kv_cache)
    _check_row(kv_cache, d_c, q_pe.shape[3])
    _expect(block_table.shape[0] == B and tuple(seq_lens.shape) == (B,), "batch mismatch")
    S = int(num_splits)
    want = (B, n_q, H, d_c) if S == 1 else (B, n_q, H, S, d_c)
    _expect(tuple(o_part.shape) == want, f"o_part must be {want}")
    if lse_part is not None:
        _expect(lse_part.numel() == B * n_q * H * S, "lse_part must hold B*n_q*H*S floats")
    shp = paged_shape(kv_cache, block_table, H, d_c)
    _invoke("mla_decode_attn_multi",
        _dev(q_lat, "q_lat", None, 4), _dev(q_pe, "q_pe", None, 4),
        _dev(kv_cache, "kv_cache", None, 3), _dev(block_table, "block_table", torch.int32, 2),
        _dev(seq_lens, "seq_lens", torch.int32, 1), ctypes.byref(shp), n_q, float(softmax_scale),
        S, _dev(o_part, "o_part"), _dtype_code(o_part), _dev(lse_part, "lse_part", torch.float32),
        code, _stream(stream))

ATTN_KERNELS = {"auto": 0, "heads": 1, "cols": 2, "generic": 3, "wide": 4}


def mla_decode_attn_planned(q_lat, q_pe, kv_cache, block_table, seq_lens, softmax_scale,
                            num_splits, o_part, lse_part=None, kernel="auto", stream=None):
    """mla_decode_attn (q_lat [B,H,d_c]) or mla_decode_attn_multi (q_lat [B,n_q,H,d_c]) on an
    explicit kernel: "auto", "heads" (16 heads per wavefront), "cols" (column-partitioned,
    H = 128), "generic" (VALU) or "wide" (32 heads per wavefront, H = 128), or the integer
    code."""
    torch = _torch()
    if q_lat.dim() == 3:
        B, H, d_c = q_lat.shape
        n_q = 1
    else:
        B, n_q, H, d_c = q_lat.shape
    _expect(tuple(q_pe.shape[:-1]) == tuple(q_lat.shape[:-1]), "q_pe must match q_lat but the last dim")
    code = _attn_code(q_lat, q_pe, kv_cache)
    _check_row(kv_cache, d_c, q_pe.shape[-1])
    _expect(block_table.shape[0] == B and tuple(seq_lens.shape) == (B,), "batch mismatch")
    S = int(num_splits)
    _expect(o_part.numel() == B * n_q * H * S * d_c, "o_part must hold B*n_q*H*S*d_c elements")
    if lse_part is not None:
        _expect(lse_part.numel() == B * n_q * H * S, "lse_part must hold B*n_q*H*S floats")
    k = ATTN_KERNELS[kernel] if isinstance(kernel, str) else int(kernel)
    shp = paged_shape(kv_cache, block_table, H, d_c)
    _invoke("mla_decode_attn_planned",
        _dev(q_lat, "q_lat"), _dev(q_pe, "q_pe"),
        _dev(kv_cache, "kv_cache", None, 3), _dev(block_table, "block_table", torch.int32, 2),
        _dev(seq_lens, "seq_lens", torch.int32, 1), ctypes.byref(shp), n_q, float(softmax_scale),
        S, _dev(o_part, "o_part"), _dtype_code(o_part), _dev(lse_part, "lse_part", torch.float32),
        code, k, _stream(stream))


def merge_counters(rows, device=None):
    """A zeroed int32 counter array for mla_decode_fused with `rows` = B * n_q query rows
    (2 counters per row and the error word); every call leaves it zeroed for the next."""
    torch = _torch()
    return torch.zeros(2 * int(rows) + 1, dtype=torch.int32, device=device or "cuda")


def mla_decode_fused(q_lat, q_pe, kv_cache, block_table, seq_lens, softmax_scale, num_splits,
                     o_part, lse_part, counters, out, lse_out=None, stream=None):
    """Attention and split combine in one launch (q_lat [B,H,d_c] or [B,n_q,H,d_c]); o_part
    [rows,H,S,d_c] (fp32 or bf16) and lse_part [rows,H,S] are scratch, counters from
    merge_counters(rows), out [rows,H,d_c] fp32."""
    torch = _torch()
    if q_lat.dim() == 3:
        B, H, d_c = q_lat.shape
        n_q = 1
    else:
        B, n_q, H, d_c = q_lat.shape
    rows = B * n_q
    _expect(tuple(q_pe.shape[:-1]) == tuple(q_lat.shape[:-1]), "q_pe must match q_lat but the last dim")
    code = _attn_code(q_lat, q_pe, kv_cache)
    _check_row(kv_cache, d_c, q_pe.shape[-1])
    _expect(block_table.shape[0] == B and tuple(seq_lens.shape) == (B,), "batch mismatch")
    S = int(num_splits)
    _expect(out.numel() == rows * H * d_c, "out must hold B*n_q*H*d_c floats")
    if lse_out is not None:
        _expect(lse_out.numel() == rows * H, "lse_out must hold B*n_q*H floats")
    if S > 1:
        _expect(o_part is not None and o_part.numel() == rows * H * S * d_c,
                "o_part must hold B*n_q*H*S*d_c elements")
        _expect(lse_part is not None and lse_part.numel() == rows * H * S,
                "lse_part must hold B*n_q*H*S floats")
        _expect(counters is not None and counters.numel() >= 2 * rows + 1,
                "counters must hold 2*B*n_q + 1 int32 (merge_counters)")
    shp = paged_shape(kv_cache, block_table, H, d_c)
    _invoke("mla_decode_fused",
        _dev(q_lat, "q_lat"), _dev(q_pe, "q_pe"),
        _dev(kv_cache, "kv_cache", None, 3), _dev(block_table, "block_table", torch.int32, 2),
        _dev(seq_lens, "seq_lens", torch.int32, 1), ctypes.byref(shp), n_q, float(softmax_scale),
        S, _dev(o_part, "o_part") if S > 1 else None,
        _dtype_code(o_part) if S > 1 else MLA_F32,
        _dev(lse_part, "lse_part", torch.float32) if S > 1 else None,
        _dev(counters, "counters", torch.int32, 1) if S > 1 else None,
        _dev(out, "out", torch.float32), _dev(lse_out, "lse_out", torch.float32),
        code, _stream(stream))


def mla_decode_fused_single_launch(shape, n_q, num_splits) -> int:
    """1 if mla_decode_fused merges inside the attention launch for this paged shape
    (paged_shape(...)), n_q and split count on the current device; else 0."""
    return int(lib.mla_decode_fused_single_launch(ctypes.byref(shape), int(n_q), int(num_splits)))


def mla_decode_ragged_workspace_bytes(kv_cache, block_table, num_heads, d_latent) -> int:
    """Workspace bytes of mla_decode_ragged for this cache pool and batch."""
    return int(lib.mla_decode_ragged_workspace_bytes(
        ctypes.byref(paged_shape(kv_cache, block_table, num_heads, d_latent))))


def mla_decode_ragged(q_lat, q_pe, kv_cache, block_table, seq_lens, softmax_scale, workspace,
                      out, lse_out=None, stream=None):
    """Decode of a ragged batch over the flattened work list: out [B,H,d_c] fp32; workspace a
    uint8 tensor of >= mla_decode_ragged_workspace_bytes(kv_cache, block_table, H, d_c)
    bytes."""
    torch = _torch()
    B, H, d_c = q_lat.shape
    _expect(tuple(q_pe.shape[:-1]) == (B, H), "q_pe must be [B,H,d_R]")
    code = _attn_code(q_lat, q_pe, kv_cache)
    _check_row(kv_cache, d_c, q_pe.shape[-1])
    _expect(block_table.shape[0] == B and tuple(seq_lens.shape) == (B,), "batch mismatch")
    _expect(tuple(out.shape) == (B, H, d_c), "out must be [B,H,d_c]")
    if lse_out is not None:
        _expect(tuple(lse_out.shape) == (B, H), "lse_out must be [B,H]")
    _expect(workspace.dtype == torch.uint8, "workspace must be a uint8 tensor")
    shp = paged_shape(kv_cache, block_table, H, d_c)
    _invoke("mla_decode_ragged",
        _dev(q_lat, "q_lat"), _dev(q_pe, "q_pe"),
        _dev(kv_cache, "kv_cache", None, 3), _dev(block_table, "block_table", torch.int32, 2),
        _dev(seq_lens, "seq_lens", torch.int32, 1), ctypes.byref(shp), float(softmax_scale),
        _dev(workspace, "workspace", torch.uint8), workspace.numel(),
        _dev(out, "out", torch.float32, 3), _dev(lse_out, "lse_out", torch.float32, 2),
        code, _stream(stream))


def mla_fold_uq(w_uk, w_uq, num_heads, w_out, stream=None):
    """W~ [H*d_c, d_cq]: head i rows = W^UK_i^T W^UQ_i (w_uk [H*d_h, d_c], w_uq [H*d_h, d_cq])."""
    H = int(num_heads)
    _expect(w_uk.dim() == 2 and w_uq.dim() == 2 and w_uk.shape[0] == w_uq.shape[0],
            "w_uk and w_uq must be [H*d_h, .] with the same rows")
    _expect(w_uk.shape[0] % H == 0, "rows of w_uk must be H*d_h")
    d_h, d_c, d_cq = w_uk.shape[0] // H, w_uk.shape[1], w_uq.shape[1]
    _expect(tuple(w_out.shape) == (H * d_c, d_cq), "w_out must be [H*d_c, d_cq]")
    _expect(w_uk.dtype == w_uq.dtype, "w_uk and w_uq share a dtype")
    _invoke("mla_fold_uq", _dev(w_uk, "w_uk", None, 2), _dev(w_uq, "w_uq", None, 2), H, d_h, d_c,
            d_cq, _dtype_code(w_uk), _dev(w_out, "w_out", None, 2), _dtype_code(w_out),
            _stream(stream))


def mla_fold_o_uv(w_o, w_uv, num_heads, w_out, stream=None):
    """W_fold [d_model, H*d_c]: head i columns = W^O_i W^UV_i (w_o [d_model, H*d_h],
    w_uv [H*d_h, d_c])."""
    H = int(num_heads)
    _expect(w_o.dim() == 2 and w_uv.dim() == 2 and w_o.shape[1] == w_uv.shape[0],
            "w_o must be [d_model, H*d_h] and w_uv [H*d_h, d_c]")
    _expect(w_uv.shape[0] % H == 0, "rows of w_uv must be H*d_h")
    d_h, d_c, d_model = w_uv.shape[0] // H, w_uv.shape[1], w_o.shape[0]
    _expect(tuple(w_out.shape) == (d_model, H * d_c), "w_out must be [d_model, H*d_c]")
    _expect(w_o.dtype == w_uv.dtype, "w_o and w_uv share a dtype")
    _invoke("mla_fold_o_uv", _dev(w_o, "w_o", None, 2), _dev(w_uv, "w_uv", None, 2), H, d_h, d_c,
            d_model, _dtype_code(w_o), _dev(w_out, "w_out", None, 2), _dtype_code(w_out),
            _stream(stream))


def mla_quantize_cache(src, dst, stream=None):
    """fp8 rows dst [..., 656] (uint8) from rows src [..., 576] (fp32 or bf16, rows contiguous
    in memory with stride src.stride(-2) elements)."""
    torch = _torch()
    _expect(src.shape[-1] == 576 and dst.shape[-1] == FP8_ROW_BYTES, "rows of 576 -> 656 bytes")
    _expect(dst.dtype == torch.uint8, "dst must be uint8")
    rows = src.numel() // 576
    _expect(dst.numel() == rows * FP8_ROW_BYTES, "dst must hold one row per source row")
    _expect(src.is_contiguous(), "src must be contiguous")
    _invoke("mla_quantize_cache", _dev(src, "src"), _dtype_code(src), 576, rows,
            _dev(dst, "dst", torch.uint8), _stream(stream))


def mla_prefill_attn(q_c, q_pe, k_c, k_pe, v_c, softmax_scale, out, lse_out=None, stream=None):
    """Causal prefill attention, expanded form: q_c, k_c, v_c [B,T,H,d_h], q_pe [B,T,H,d_R],
    k_pe [B,T,d_R] (bf16); out [B,T,H,d_h] fp32, lse_out [B,T,H] or None."""
    torch = _torch()
    B, T, H, d_h = q_c.shape
    d_R = q_pe.shape[-1]
    _expect(tuple(q_pe.shape) == (B, T, H, d_R), "q_pe must be [B,T,H,d_R]")
    _expect(tuple(k_c.shape) == (B, T, H, d_h) and tuple(v_c.shape) == (B, T, H, d_h),
            "k_c and v_c must be [B,T,H,d_h]")
    _expect(tuple(k_pe.shape) == (B, T, d_R), "k_pe must be [B,T,d_R]")
    _expect(tuple(out.shape) == (B, T, H, d_h), "out must be [B,T,H,d_h]")
    if lse_out is not None:
        _expect(tuple(lse_out.shape) == (B, T, H), "lse_out must be [B,T,H]")
    for t in (q_pe, k_c, k_pe, v_c):
        _expect(t.dtype == q_c.dtype, "inputs share a dtype")
    _invoke("mla_prefill_attn", _dev(q_c, "q_c"), _dev(q_pe, "q_pe"), _dev(k_c, "k_c"),
            _dev(k_pe, "k_pe"), _dev(v_c, "v_c"), B, T, H, d_h, d_R, float(softmax_scale),
            _dev(out, "out", torch.float32), _dev(lse_out, "lse_out", torch.float32),
            _dtype_code(q_c), _stream(stream))


def mla_splitk_combine(o_part, lse_part, out, lse_out=None, stream=None):
    """Log-sum-exp combine of float32 or bfloat16 partials o_part [B,H,S,d_c] into out [B,H,d_c]."""
    torch = _torch()
    B, H, S, d_c = o_part.shape
    _expect(tuple(lse_part.shape) == (B, H, S), "lse_part must be [B,H,S]")
    _expect(tuple(out.shape) == (B, H, d_c), "out must be [B,H,d_c]")
    if lse_out is not None:
        _expect(tuple(lse_out.shape) == (B, H), "lse_out must be [B,H]")
    _invoke("mla_splitk_combine",
        _dev(o_part, "o_part", None, 4), _dtype_code(o_part),
        _dev(lse_part, "lse_part", torch.float32, 3), B, H, S, d_c, _dev(out, "out", torch.float32, 3),
        _dev(lse_out, "lse_out", torch.float32, 2), _stream(stream))


def mla_combine_out_proj(o_part, lse_part, w_uv, o_heads, stream=None):
    """o_heads = W^UV_i (combine of the split partials) per head, in one kernel.
    o_part [B,H,S,d_c] f32/bf16, lse_part [B,H,S] f32, w_uv [H*d_h, d_c] bf16,
    o_heads [B,H,d_h] f32."""
    torch = _torch()
    B, H, S, d_c = o_part.shape
    d_h = o_heads.shape[2]
    _expect(tuple(lse_part.shape) == (B, H, S), "lse_part must be [B,H,S]")
    _expect(tuple(w_uv.shape) == (H * d_h, d_c), "w_uv must be [H*d_h, d_c]")
    _expect(tuple(o_heads.shape) == (B, H, d_h), "o_heads must be [B,H,d_h]")
    _invoke("mla_combine_out_proj", _dev(o_part, "o_part", None, 4), _dtype_code(o_part),
            _dev(lse_part, "lse_part", torch.float32, 3), B, H, S, d_c,
            _dev(w_uv, "w_uv", None, 2), _dtype_code(w_uv), d_h,
            _dev(o_heads, "o_heads", torch.float32, 3), _stream(stream))


def mla_decode(q_lat, q_pe, kv_cache, block_table, seq_lens, softmax_scale, num_splits,
               workspace, out, lse_out=None, stream=None):
    """Attention + combine with the split partials in `workspace` (uint8 tensor of at
    least mla_decode_workspace_bytes bytes; may be None when num_splits == 1)."""
    torch = _torch()
    B, H, d_c = q_lat.shape
    code = _attn_code(q_lat, q_pe, kv_cache)
    _expect(tuple(out.shape) == (B, H, d_c), "out must be [B,H,d_c]")
    shp = paged_shape(kv_cache, block_table, H, d_c)
    ws_ptr = _dev(workspace, "workspace") if workspace is not None else None
    ws_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _invoke("mla_decode",
        _dev(q_lat, "q_lat", None, 3), _dev(q_pe, "q_pe", None, 3),
        _dev(kv_cache, "kv_cache", None, 3), _dev(block_table, "block_table", torch.int32, 2),
        _dev(seq_lens, "seq_lens", torch.int32, 1), ctypes.byref(shp), float(softmax_scale),
        int(num_splits), ws_ptr, ws_bytes, _dev(out, "out", torch.float32, 3),
        _dev(lse_out, "lse_out", torch.float32, 2), code, _stream(stream))


def mla_decode_noalloc(q_lat, q_pe, kv_cache, block_table, seq_lens, softmax_scale,
                       num_splits, out, lse_out=None, stream=None):
    """mla_decode with the split partials in the library's fixed device scratch (48 MiB):
    the call allocates no device memory."""
    torch = _torch()
    B, H, d_c = q_lat.shape
    code = _attn_code(q_lat, q_pe, kv_cache)
    _expect(tuple(out.shape) == (B, H, d_c), "out must be [B,H,d_c]")
    shp = paged_shape(kv_cache, block_table, H, d_c)
    _invoke("mla_decode_noalloc",
        _dev(q_lat, "q_lat", None, 3), _dev(q_pe, "q_pe", None, 3),
        _dev(kv_cache, "kv_cache", None, 3), _dev(block_table, "block_table", torch.int32, 2),
        _dev(seq_lens, "seq_lens", torch.int32, 1), ctypes.byref(shp), float(softmax_scale),
        int(num_splits), _dev(out, "out", torch.float32, 3),
        _dev(lse_out, "lse_out", torch.float32, 2), code, _stream(stream))


def mla_out_proj(o_lat, w_uv, w_o, o_heads, u=None, stream=None):
    """o_heads = W^UV_i o_lat_i per head; u = W^O concat(o_heads) when w_o is given."""
    torch = _torch()
    B, H, d_c = o_lat.shape
    d_h = w_uv.shape[0] // H
    _expect(tuple(w_uv.shape) == (H * d_h, d_c), "w_uv must be [H*d_h, d_c]")
    _expect(tuple(o_heads.shape) == (B, H, d_h), "o_heads must be [B,H,d_h]")
    d_model = 0
    if w_o is not None:
        d_model = w_o.shape[0]
        _expect(tuple(w_o.shape) == (d_model, H * d_h), "w_o must be [d_model, H*d_h]")
        _expect(w_o.dtype == w_uv.dtype, "w_o and w_uv share a dtype")
        _expect(u is not None and tuple(u.shape) == (B, d_model), "u must be [B, d_model]")
    _invoke("mla_out_proj",
        _dev(o_lat, "o_lat", torch.float32, 3), _dev(w_uv, "w_uv", None, 2),
        _dev(w_o, "w_o", None, 2), B, H, d_c, d_h, d_model, _dtype_code(w_uv),
        _dev(o_heads, "o_heads", torch.float32, 3), _dev(u, "u", torch.float32, 2),
        _stream(stream))


def mla_linear(x, w, y, stream=None):
    """y = x w^T; x [M,K], w [N,K], y [M,N] fp32."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _expect(w.shape[1] == K and tuple(y.shape) == (M, N), "shapes must be x[M,K] w[N,K] y[M,N]")
    _invoke("mla_linear", _dev(x, "x", None, 2), _dtype_code(x), _dev(w, "w", None, 2),
                          _dtype_code(w), M, N, K, _dev(y, "y", torch.float32, 2),
                          _stream(stream))


def mla_linear_strided(x, w, y, accumulate=False, stream=None):
    """y = x w^T (accumulate: y += x w^T) on row-strided views: x [M,K], y [M,N] fp32 with
    unit column stride (e.g. column ranges of wider buffers); w [N,K] dense (e.g. several
    nn.Linear weights stacked)."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _expect(w.shape[1] == K and tuple(y.shape) == (M, N), "shapes must be x[M,K] w[N,K] y[M,N]")
    x_ptr, ldx = _dev_rows(x, "x", None, 2, 1)
    y_ptr, ldy = _dev_rows(y, "y", torch.float32, 2, 1)
    _invoke("mla_linear_strided", x_ptr, _dtype_code(x), ldx, _dev(w, "w", None, 2),
                                  _dtype_code(w), M, N, K, y_ptr, ldy, int(bool(accumulate)),
                                  _stream(stream))


def mla_linear_deterministic_workspace_bytes(M, N, K):
    """Workspace bytes mla_linear_deterministic needs for an [M,K] x [N,K]^T product (0: the
    shape is not supported)."""
    return int(lib.mla_linear_deterministic_workspace_bytes(int(M), int(N), int(K)))


def mla_linear_deterministic(x, w, y, workspace, accumulate=False, stream=None):
    """mla_linear_strided with a fixed summation order (bit-identical reruns): split-k partial
    tiles go to `workspace` (a uint8 GPU tensor of at least
    mla_linear_deterministic_workspace_bytes(M, N, K) bytes) and are summed in order into y."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _expect(w.shape[1] == K and tuple(y.shape) == (M, N), "shapes must be x[M,K] w[N,K] y[M,N]")
    x_ptr, ldx = _dev_rows(x, "x", None, 2, 1)
    y_ptr, ldy = _dev_rows(y, "y", torch.float32, 2, 1)
    _invoke("mla_linear_deterministic", x_ptr, _dtype_code(x), ldx, _dev(w, "w", None, 2),
            _dtype_code(w), M, N, K, y_ptr, ldy, int(bool(accumulate)),
            _dev(workspace, "workspace", torch.uint8), workspace.numel(), _stream(stream))


def mla_linear_deterministic_append(x, w, y, workspace, append_col, seq_lens_before,
                                    block_table, kv_cache, rope_base, d_latent=512, stream=None):
    """mla_linear_deterministic whose summing launch also appends the new token of each
    sequence: [y[b, c:c+d_c] | RoPE(y[b, c+d_c:c+d_c+d_R], pos)] to the bf16 cache at
    pos = seq_lens_before[b] (c = append_col, d_c = d_latent, d_R = cache row - d_c)."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _expect(w.shape[1] == K and tuple(y.shape) == (M, N), "shapes must be x[M,K] w[N,K] y[M,N]")
    _expect(kv_cache.dtype == torch.bfloat16 and kv_cache.dim() == 3, "kv_cache must be bf16 [pages, P, row]")
    _expect(block_table.shape[0] == M and tuple(seq_lens_before.shape) == (M,), "batch mismatch")
    shp = paged_shape(kv_cache, block_table, 1, int(d_latent))
    x_ptr, ldx = _dev_rows(x, "x", None, 2, 1)
    y_ptr, ldy = _dev_rows(y, "y", torch.float32, 2, 1)
    _invoke("mla_linear_deterministic_append", x_ptr, _dtype_code(x), ldx, _dev(w, "w", None, 2),
            _dtype_code(w), M, N, K, y_ptr, ldy, _dev(workspace, "workspace", torch.uint8),
            workspace.numel(), int(append_col),
            _dev(seq_lens_before, "seq_lens_before", torch.int32, 1),
            _dev(block_table, "block_table", torch.int32, 2), _dev(kv_cache, "kv_cache", None, 3),
            float(rope_base), ctypes.byref(shp), _cache_code(kv_cache), _stream(stream))


def mla_linear_planned(x, w, y, kernel, tile, split, ring, stream=None):
    """mla_linear on an explicit kernel (0 tile grid, 1 persistent) and plan."""
    torch = _torch()
    M, K = x.shape
    N = w.shape[0]
    _expect(w.shape[1] == K and tuple(y.shape) == (M, N), "shapes must be x[M,K] w[N,K] y[M,N]")
    _invoke("mla_linear_planned", _dev(x, "x", None, 2), _dtype_code(x), _dev(w, "w", None, 2),
                                  _dtype_code(w), M, N, K, _dev(y, "y", torch.float32, 2),
                                  kernel, tile, split, ring, _stream(stream))


def mla_validate_indices(block_table, seq_lens, page_size, num_pages, dev_count, stream=None):
    torch = _torch()
    B, maxp = block_table.shape
    shp = _PagedShape(B, 1, 1, 2, page_size, maxp, num_pages)
    _invoke("mla_validate_indices",
        _dev(block_table, "block_table", torch.int32, 2), _dev(seq_lens, "seq_lens", torch.int32, 1),
        ctypes.byref(shp), _dev(dev_count, "dev_count", torch.int32), _stream(stream))


def mla_stream_read(src, sink, stream=None):
    torch = _torch()
    _expect(sink.numel() >= 4096, "sink must hold 4096 floats")
    _invoke("mla_stream_read", _dev(src, "src"), src.numel() * src.element_size(),
                               _dev(sink, "sink", torch.float32), _stream(stream))


def mla_stream_read_lds(src, sink, stream=None):
    torch = _torch()
    cus = torch.cuda.get_device_properties(src.device).multi_processor_count
    _expect(sink.numel() >= cus, f"sink must hold {cus} floats (one per compute unit)")
    _invoke("mla_stream_read_lds", _dev(src, "src"), src.numel() * src.element_size(),
                                   _dev(sink, "sink", torch.float32), _stream(stream))
