"""Python binding of libdattn.so (disentangled-attention forward, MI355X).

Argument marshalling only: torch tensors are turned into device pointers,
element strides and the current HIP stream, and the C entry points of
include/dattn.h are called by the same names. Every step of the
computation runs in the library's HIP kernels; there is no Python or CPU
fallback, and a missing library raises.
"""

from __future__ import annotations

import ctypes
import os
from typing import Optional

PKG_DIR = os.path.dirname(os.path.abspath(__file__))
# the in-tree build; DATTN_LIB may name another build of the same ABI
LIB_PATH = os.environ.get("DATTN_LIB") or os.path.join(PKG_DIR, "libdattn.so")

DATTN_OK = 0
DATTN_ERR_INVALID_ARGUMENT = 1
DATTN_ERR_UNSUPPORTED = 2
DATTN_ERR_HIP = 3
DATTN_ERR_SCRATCH_TOO_SMALL = 4
DATTN_NOALLOC_SCRATCH_BYTES = 128 << 20
DATTN_F32, DATTN_F16, DATTN_BF16 = 0, 1, 2
DATTN_C2P, DATTN_P2C = 1, 2
DATTN_MAX_SEQLEN = 8192

_lib_handle = None


class DattnError(RuntimeError):
    def __init__(self, status: int, fn: str):
        self.status = status
        super().__init__(f"{fn}: status {status} ({strerror(status)})")


def lib() -> ctypes.CDLL:
    """Load libdattn.so (built in-tree by deberta_disentangled_attention_amd.build)."""
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing; build it with "
                               "`python -m deberta_disentangled_attention_amd.build`")
        h = ctypes.CDLL(LIB_PATH)
        vp, i32, i64, u32, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64,
                                  ctypes.c_uint32, ctypes.c_float)
        h.rel_bucket.argtypes = [vp, i32, i32, i32, vp]
        h.rel_bucket.restype = ctypes.c_int
        h.dattn_fwd_padded.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i32, vp, i32,
                                       vp, vp, i32, i32, i32, i32, i32, u32, f32, vp]
        h.dattn_fwd_padded.restype = ctypes.c_int
        h.dattn_fwd_varlen.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i32, vp, i32,
                                       vp, i32, i32, i64, vp, i32, i32, i32, u32, f32, vp]
        h.dattn_fwd_varlen.restype = ctypes.c_int
        h.dattn_fwd_padded_lse.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i32, vp, i32,
                                           vp, vp, vp, i32, i32, i32, i32, i32, u32, f32, vp]
        h.dattn_fwd_padded_lse.restype = ctypes.c_int
        h.dattn_fwd_varlen_lse.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i32, vp, i32,
                                           vp, i32, i32, i64, vp, vp, i32, i32, i32, u32, f32, vp]
        h.dattn_fwd_varlen_lse.restype = ctypes.c_int
        h.dattn_pack_index.argtypes = [vp, i32, i32, vp, vp, vp, vp, vp]
        h.dattn_pack_index.restype = ctypes.c_int
        for fn in (h.dattn_pack_rows, h.dattn_unpack_rows):
            fn.argtypes = [vp, i64, i64, vp, i64, i64, vp, i64, vp]
            fn.restype = ctypes.c_int
        h.dattn_rel_proj.argtypes = [vp, i64, vp, vp, i64, vp, vp, vp, vp, i64, i32, i32, i32, i32,
                                     vp]
        h.dattn_rel_proj.restype = ctypes.c_int
        h.rel_bucket_band.argtypes = [i32, i32, i32]
        h.rel_bucket_band.restype = ctypes.c_int32
        h.dattn_bwd_workspace_size.argtypes = [i64, i32, i32, i32, i32, i32]
        h.dattn_bwd_workspace_size.restype = ctypes.c_int64
        h.dattn_bwd_padded.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp, vp, i64,
                                       i32, vp, i32, i32, vp, vp, vp, vp, vp, vp, vp, i64, i32, i32,
                                       i32, i32, i32, u32, f32, vp]
        h.dattn_bwd_padded.restype = ctypes.c_int
        h.dattn_bwd_varlen.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp, vp, i64,
                                       i32, vp, i32, i32, vp, i32, i32, i64, vp, vp, vp, vp, vp, vp,
                                       i64, i32, i32, i32, u32, f32, vp]
        h.dattn_bwd_varlen.restype = ctypes.c_int
        h.dattn_bwd_varlen_noalloc.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i64, vp, vp,
                                               vp, i64, i32, vp, i32, i32, vp, i32, i32, i64, vp,
                                               vp, vp, vp, vp, i32, i32, i32, u32, f32, vp]
        h.dattn_bwd_varlen_noalloc.restype = ctypes.c_int
        h.dattn_fwd_f32fast_workspace_size.argtypes = [i64, i32, i32, i32]
        h.dattn_fwd_f32fast_workspace_size.restype = ctypes.c_int64
        h.dattn_fwd_padded_f32fast.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i32, vp, i32,
                                               vp, vp, i32, i32, i32, i32, u32, f32, vp, i64, vp]
        h.dattn_fwd_padded_f32fast.restype = ctypes.c_int
        h.dattn_fwd_varlen_f32fast.argtypes = [vp, vp, vp, i64, i64, i64, vp, vp, i64, i32, vp, i32,
                                               vp, i32, i32, i64, vp, i32, i32, u32, f32, vp, i64, vp]
        h.dattn_fwd_varlen_f32fast.restype = ctypes.c_int
        h.dattn_strerror.argtypes = [ctypes.c_int]
        h.dattn_strerror.restype = ctypes.c_char_p
        _lib_handle = h
    return _lib_handle


def strerror(status: int) -> str:
    return lib().dattn_strerror(int(status)).decode()


def _check(status: int, fn: str) -> None:
    if status != DATTN_OK:
        raise DattnError(status, fn)


def _dtype_code(t) -> int:
    import torch
    return {torch.float32: DATTN_F32, torch.float16: DATTN_F16,
            torch.bfloat16: DATTN_BF16}.get(t.dtype, -1)


def _ptr(t) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(t):
    import torch
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _row_stride(t, name: str) -> int:
    if t.stride(-1) != 1:
        raise ValueError(f"{name}: the last dimension must be contiguous")
    return t.stride(-2)


def rel_bucket(max_len: int, position_buckets: int, max_relative_positions: int,
               *, out=None, device=None):
    """int32 table of 2*max_len-1 relative rows (see include/dattn.h)."""
    import torch
    if out is None:
        out = torch.empty(2 * max_len - 1, dtype=torch.int32,
                          device=device if device is not None else "cuda")
    if out.dtype != torch.int32 or out.numel() < 2 * max_len - 1 or not out.is_contiguous():
        raise ValueError("out must be a contiguous int32 tensor of 2*max_len-1 entries")
    _check(lib().rel_bucket(ctypes.c_void_p(out.data_ptr()), max_len, position_buckets,
                            max_relative_positions, _stream(out)), "rel_bucket")
    return out


def _out_tensor(out, rows: int, width: int, like, lead=None):
    """The caller's out, or a new one: a contiguous tensor of `rows` rows of
    `width` elements with like's dtype and device (shape `lead` + [width]
    when lead is given)."""
    import torch
    if out is None:
        shape = (rows, width) if lead is None else (*lead, width)
        return torch.empty(shape, dtype=like.dtype, device=like.device)
    if (out.dtype != like.dtype or out.device != like.device or not out.is_contiguous()
            or out.numel() != rows * width or (out.dim() and out.shape[-1] != width)):
        raise ValueError(f"out must be a contiguous {like.dtype} tensor of {rows} rows of "
                         f"{width} elements on {like.device}")
    return out


def _table_check(rel_idx, rel_max_len: int, flags: int, device) -> None:
    import torch
    if rel_idx is None:
        if flags:
            raise ValueError("rel_idx is required when a position term is enabled")
        return
    if (rel_idx.dtype != torch.int32 or not rel_idx.is_contiguous()
            or rel_idx.numel() != 2 * int(rel_max_len) - 1 or rel_idx.device != device):
        raise ValueError("rel_idx must be a contiguous int32 tensor of 2*rel_max_len-1 "
                         "entries on the inputs' device")


def _lse_tensor(lse, rows: int, H: int, device):
    import torch
    if lse is True:
        return torch.empty((rows, H), dtype=torch.float32, device=device)
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != rows * H:
        raise ValueError("lse must be a contiguous float32 tensor of rows * H entries")
    return lse


def dattn_fwd_padded(q, k, v, qr, kr, rel_idx, rel_max_len: int, mask, H: int, d: int,
                     *, flags: int = DATTN_C2P | DATTN_P2C, scale: float = 0.0, out=None,
                     lse=None):
    """Forward over a padded batch; q, k, v are [B, L, >=H*d] (views of a
    fused QKV buffer are fine), mask is [B, L] uint8/bool or None. With lse
    (True, or a float32 [B*L, H] tensor) also returns each row's log-sum-exp:
    (out, lse)."""
    import torch
    B, L = q.shape[0], q.shape[1]
    for name, t in (("k", k), ("v", v)):
        if t.shape[:2] != q.shape[:2] or t.dtype != q.dtype:
            raise ValueError(f"{name} must match q in [B, L] and dtype")
    ld_q, ld_k, ld_v = _row_stride(q, "q"), _row_stride(k, "k"), _row_stride(v, "v")
    for name, t, ld in (("q", q, ld_q), ("k", k, ld_k), ("v", v, ld_v)):
        if B > 1 and t.stride(0) != L * ld:
            raise ValueError(f"{name}: batch stride must be L * row stride")
    ld_rel = 0
    if qr is not None:
        if kr is None or kr.stride() != qr.stride() or kr.shape != qr.shape:
            raise ValueError("qr and kr must have the same shape and strides")
        ld_rel = _row_stride(qr, "qr")
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or not mask.is_contiguous() or tuple(mask.shape) != (B, L):
            raise ValueError("mask must be a contiguous [B, L] uint8/bool tensor")
    _table_check(rel_idx, rel_max_len, flags, q.device)
    out = _out_tensor(out, B * L, H * d, q, lead=(B, L))
    n_rel = qr.shape[0] if qr is not None else 0
    if lse is None:
        st = lib().dattn_fwd_padded(
            _ptr(q), _ptr(k), _ptr(v), ld_q, ld_k, ld_v, _ptr(qr), _ptr(kr), ld_rel, n_rel,
            _ptr(rel_idx), int(rel_max_len), _ptr(mask), _ptr(out), B, L, H, d,
            _dtype_code(q), int(flags), float(scale), _stream(q))
        _check(st, "dattn_fwd_padded")
        return out
    lse = _lse_tensor(lse, B * L, H, q.device)
    st = lib().dattn_fwd_padded_lse(
        _ptr(q), _ptr(k), _ptr(v), ld_q, ld_k, ld_v, _ptr(qr), _ptr(kr), ld_rel, n_rel,
        _ptr(rel_idx), int(rel_max_len), _ptr(mask), _ptr(out), _ptr(lse), B, L, H, d,
        _dtype_code(q), int(flags), float(scale), _stream(q))
    _check(st, "dattn_fwd_padded_lse")
    return out, lse


def dattn_fwd_varlen(q, k, v, qr, kr, rel_idx, rel_max_len: int, cu_seqlens, max_seqlen: int,
                     H: int, d: int, *, flags: int = DATTN_C2P | DATTN_P2C, scale: float = 0.0,
                     out=None, total_tokens: Optional[int] = None, lse=None):
    """Forward over packed sequences; q, k, v are [total_tokens, >=H*d] and
    cu_seqlens a device int32 [nseq+1]. max_seqlen (and total_tokens, by
    default q.shape[0]) are host values. With lse (True, or a float32
    [total_tokens, H] tensor) also returns each row's log-sum-exp."""
    import torch
    T = q.shape[0] if total_tokens is None else int(total_tokens)
    if T > q.shape[0] or T > k.shape[0] or T > v.shape[0]:
        raise ValueError("total_tokens exceeds the rows of q, k or v")
    for name, t in (("k", k), ("v", v)):
        if t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in dtype and device")
    ld_q, ld_k, ld_v = _row_stride(q, "q"), _row_stride(k, "k"), _row_stride(v, "v")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor")
    ld_rel = 0
    if qr is not None:
        if kr is None or kr.stride() != qr.stride() or kr.shape != qr.shape:
            raise ValueError("qr and kr must have the same shape and strides")
        ld_rel = _row_stride(qr, "qr")
    _table_check(rel_idx, rel_max_len, flags, q.device)
    out = _out_tensor(out, T, H * d, q)
    n_rel = qr.shape[0] if qr is not None else 0
    if lse is None:
        st = lib().dattn_fwd_varlen(
            _ptr(q), _ptr(k), _ptr(v), ld_q, ld_k, ld_v, _ptr(qr), _ptr(kr), ld_rel, n_rel,
            _ptr(rel_idx), int(rel_max_len), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
            int(max_seqlen), T, _ptr(out), H, d, _dtype_code(q), int(flags), float(scale),
            _stream(q))
        _check(st, "dattn_fwd_varlen")
        return out
    lse = _lse_tensor(lse, T, H, q.device)
    st = lib().dattn_fwd_varlen_lse(
        _ptr(q), _ptr(k), _ptr(v), ld_q, ld_k, ld_v, _ptr(qr), _ptr(kr), ld_rel, n_rel,
        _ptr(rel_idx), int(rel_max_len), _ptr(cu_seqlens), cu_seqlens.numel() - 1,
        int(max_seqlen), T, _ptr(out), _ptr(lse), H, d, _dtype_code(q), int(flags),
        float(scale), _stream(q))
    _check(st, "dattn_fwd_varlen_lse")
    return out, lse


def f32fast_workspace_size(rows: int, n_rel: int, H: int, d: int) -> int:
    n = lib().dattn_fwd_f32fast_workspace_size(int(rows), int(n_rel), int(H), int(d))
    if n < 0:
        raise ValueError("invalid sizes for the fast fp32 workspace")
    return n


def dattn_fwd_padded_f32fast(q, k, v, qr, kr, rel_idx, rel_max_len: int, mask, H: int, d: int,
                             *, flags: int = DATTN_C2P | DATTN_P2C, scale: float = 0.0, out=None,
                             workspace=None):
    """Fast fp32 forward over a padded batch: float32 q, k, v, qr, kr; the
    products run on the fp16 MFMA (operands rounded once to fp16)."""
    import torch
    B, L = q.shape[0], q.shape[1]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float32:
            raise ValueError(f"{name} must be float32")
        if t.shape[:2] != q.shape[:2]:
            raise ValueError(f"{name} must match q in [B, L]")
    lds = [_row_stride(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"))]
    for name, t, ld in (("q", q, lds[0]), ("k", k, lds[1]), ("v", v, lds[2])):
        if B > 1 and t.stride(0) != L * ld:
            raise ValueError(f"{name}: batch stride must be L * row stride")
    ld_rel, n_rel = 0, 0
    if qr is not None:
        if kr is None or kr.stride() != qr.stride() or kr.shape != qr.shape or qr.dtype != torch.float32:
            raise ValueError("qr and kr must be float32 with the same shape and strides")
        ld_rel, n_rel = _row_stride(qr, "qr"), qr.shape[0]
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or not mask.is_contiguous() or tuple(mask.shape) != (B, L):
            raise ValueError("mask must be a contiguous [B, L] uint8/bool tensor")
    _table_check(rel_idx, rel_max_len, flags, q.device)
    out = _out_tensor(out, B * L, H * d, q, lead=(B, L))
    if workspace is None:
        need = f32fast_workspace_size(B * L, n_rel if flags else 0, H, d)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().dattn_fwd_padded_f32fast(
        _ptr(q), _ptr(k), _ptr(v), lds[0], lds[1], lds[2], _ptr(qr), _ptr(kr), ld_rel, n_rel,
        _ptr(rel_idx), int(rel_max_len), _ptr(mask), _ptr(out), B, L, H, d, int(flags),
        float(scale), _ptr(workspace), workspace.numel() * workspace.element_size(), _stream(q))
    _check(st, "dattn_fwd_padded_f32fast")
    return out


def dattn_fwd_varlen_f32fast(q, k, v, qr, kr, rel_idx, rel_max_len: int, cu_seqlens,
                             max_seqlen: int, H: int, d: int, *,
                             flags: int = DATTN_C2P | DATTN_P2C, scale: float = 0.0, out=None,
                             workspace=None):
    """Fast fp32 forward over packed sequences (float32 operands)."""
    import torch
    T = q.shape[0]
    for name, t in (("q", q), ("k", k), ("v", v)):
        if t.dtype != torch.float32 or t.shape[0] != T:
            raise ValueError(f"{name} must be float32 with q's rows")
    lds = [_row_stride(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"))]
    ld_rel, n_rel = 0, 0
    if qr is not None:
        if kr is None or kr.stride() != qr.stride() or kr.shape != qr.shape or qr.dtype != torch.float32:
            raise ValueError("qr and kr must be float32 with the same shape and strides")
        ld_rel, n_rel = _row_stride(qr, "qr"), qr.shape[0]
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor")
    _table_check(rel_idx, rel_max_len, flags, q.device)
    out = _out_tensor(out, T, H * d, q)
    if workspace is None:
        need = f32fast_workspace_size(T, n_rel if flags else 0, H, d)
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().dattn_fwd_varlen_f32fast(
        _ptr(q), _ptr(k), _ptr(v), lds[0], lds[1], lds[2], _ptr(qr), _ptr(kr), ld_rel, n_rel,
        _ptr(rel_idx), int(rel_max_len), _ptr(cu_seqlens), cu_seqlens.numel() - 1, int(max_seqlen),
        T, _ptr(out), H, d, int(flags), float(scale), _ptr(workspace),
        workspace.numel() * workspace.element_size(), _stream(q))
    _check(st, "dattn_fwd_varlen_f32fast")
    return out


def rel_bucket_band(max_len: int, position_buckets: int, max_relative_positions: int) -> int:
    """The band of rel_bucket's table: the least W >= 1 beyond which (at
    distances >= W and <= -W) the table is constant (host computation)."""
    w = lib().rel_bucket_band(int(max_len), int(position_buckets), int(max_relative_positions))
    if w < 1:
        raise ValueError("invalid bucket parameters")
    return int(w)


def bwd_workspace_size(total_tokens: int, nseq: int, H: int, d: int, dtype, band: int) -> int:
    import torch
    code = {torch.float32: DATTN_F32, torch.float16: DATTN_F16, torch.bfloat16: DATTN_BF16}[dtype]
    n = lib().dattn_bwd_workspace_size(int(total_tokens), int(nseq), int(H), int(d), code, int(band))
    if n < 0:
        raise ValueError("invalid workspace-size arguments")
    return int(n)


def _bwd_outputs(q, rows: int, H: int, d: int, n_rel: int, flags: int):
    import torch
    mk = lambda *shape: torch.empty(shape, dtype=q.dtype, device=q.device)
    dq, dk, dv = mk(rows, H * d), mk(rows, H * d), mk(rows, H * d)
    dqr = mk(n_rel, H * d) if flags else None
    dkr = mk(n_rel, H * d) if flags else None
    return dq, dk, dv, dqr, dkr


def dattn_bwd_padded(q, k, v, out, dout, lse, qr, kr, rel_idx, rel_max_len: int, band: int, mask,
                     H: int, d: int, *, flags: int = DATTN_C2P | DATTN_P2C, scale: float = 0.0,
                     workspace=None):
    """Backward of dattn_fwd_padded_lse: returns (dq, dk, dv, dqr, dkr); dq, dk,
    dv are [B*L, H*d], dqr / dkr [n_rel, H*d] (None when flags == 0). out and
    lse are the forward's; band bounds the distances where the table varies
    (rel_bucket_band)."""
    import torch
    B, L = q.shape[0], q.shape[1]
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.shape[:2] != q.shape[:2] or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in [B, L], dtype and device")
    lds = [_row_stride(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"))]
    for t, ld, name in zip((q, k, v, out, dout), lds, ("q", "k", "v", "out", "dout")):
        if B > 1 and t.stride(0) != L * ld:
            raise ValueError(f"{name}: batch stride must be L * row stride")
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != B * L * H:
        raise ValueError("lse must be the forward's contiguous float32 [B*L, H] log-sum-exp")
    ld_rel, n_rel = 0, 0
    if qr is not None:
        if kr is None or kr.stride() != qr.stride() or kr.shape != qr.shape:
            raise ValueError("qr and kr must have the same shape and strides")
        ld_rel, n_rel = _row_stride(qr, "qr"), qr.shape[0]
    _table_check(rel_idx, rel_max_len, flags, q.device)
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or not mask.is_contiguous() or tuple(mask.shape) != (B, L):
            raise ValueError("mask must be a contiguous [B, L] uint8/bool tensor")
    band = int(band) if flags else 1
    dq, dk, dv, dqr, dkr = _bwd_outputs(q, B * L, H, d, n_rel, flags)
    need = bwd_workspace_size(B * L, B, H, d, q.dtype, band)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().dattn_bwd_padded(
        _ptr(q), _ptr(k), _ptr(v), lds[0], lds[1], lds[2], _ptr(out), _ptr(dout), lds[3], lds[4],
        _ptr(lse), _ptr(qr), _ptr(kr), ld_rel, n_rel, _ptr(rel_idx), int(rel_max_len), band,
        _ptr(mask), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dqr), _ptr(dkr), _ptr(workspace),
        workspace.numel() * workspace.element_size(), B, L, H, d, _dtype_code(q), int(flags),
        float(scale), _stream(q))
    _check(st, "dattn_bwd_padded")
    return dq, dk, dv, dqr, dkr


def _bwd_varlen_checks(q, k, v, out, dout, lse, qr, kr, rel_idx, rel_max_len, band, cu_seqlens,
                       H, flags):
    import torch
    T = q.shape[0]
    for name, t in (("k", k), ("v", v), ("out", out), ("dout", dout)):
        if t.shape[0] != T or t.dtype != q.dtype or t.device != q.device:
            raise ValueError(f"{name} must match q in rows, dtype and device")
    lds = [_row_stride(t, n) for t, n in ((q, "q"), (k, "k"), (v, "v"), (out, "out"), (dout, "dout"))]
    if lse.dtype != torch.float32 or not lse.is_contiguous() or lse.numel() != T * H:
        raise ValueError("lse must be the forward's contiguous float32 [total_tokens, H] log-sum-exp")
    if cu_seqlens.dtype != torch.int32 or not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous int32 tensor")
    ld_rel, n_rel = 0, 0
    if qr is not None:
        if kr is None or kr.stride() != qr.stride() or kr.shape != qr.shape:
            raise ValueError("qr and kr must have the same shape and strides")
        ld_rel, n_rel = _row_stride(qr, "qr"), qr.shape[0]
    _table_check(rel_idx, rel_max_len, flags, q.device)
    band = int(band) if flags else 1
    return T, lds, ld_rel, n_rel, cu_seqlens.numel() - 1, band


def dattn_bwd_varlen(q, k, v, out, dout, lse, qr, kr, rel_idx, rel_max_len: int, band: int,
                     cu_seqlens, max_seqlen: int, H: int, d: int, *,
                     flags: int = DATTN_C2P | DATTN_P2C, scale: float = 0.0, workspace=None):
    """Backward of dattn_fwd_varlen_lse over packed sequences; returns (dq, dk,
    dv, dqr, dkr) with dq, dk, dv [total_tokens, H*d]."""
    import torch
    T, lds, ld_rel, n_rel, nseq, band = _bwd_varlen_checks(
        q, k, v, out, dout, lse, qr, kr, rel_idx, rel_max_len, band, cu_seqlens, H, flags)
    dq, dk, dv, dqr, dkr = _bwd_outputs(q, T, H, d, n_rel, flags)
    need = bwd_workspace_size(T, nseq, H, d, q.dtype, band)
    if workspace is None:
        workspace = torch.empty(max(need, 16), dtype=torch.uint8, device=q.device)
    st = lib().dattn_bwd_varlen(
        _ptr(q), _ptr(k), _ptr(v), lds[0], lds[1], lds[2], _ptr(out), _ptr(dout), lds[3], lds[4],
        _ptr(lse), _ptr(qr), _ptr(kr), ld_rel, n_rel, _ptr(rel_idx), int(rel_max_len), band,
        _ptr(cu_seqlens), nseq, int(max_seqlen), T, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dqr),
        _ptr(dkr), _ptr(workspace), workspace.numel() * workspace.element_size(), H, d,
        _dtype_code(q), int(flags), float(scale), _stream(q))
    _check(st, "dattn_bwd_varlen")
    return dq, dk, dv, dqr, dkr


def dattn_bwd_varlen_noalloc(q, k, v, out, dout, lse, qr, kr, rel_idx, rel_max_len: int,
                             band: int, cu_seqlens, max_seqlen: int, H: int, d: int, *,
                             flags: int = DATTN_C2P | DATTN_P2C, scale: float = 0.0, grads=None):
    """dattn_bwd_varlen with the library's fixed per-GPU scratch array as its
    workspace (no device allocation in the library call). grads, if given,
    is the (dq, dk, dv, dqr, dkr) tuple to write (contiguous, q's dtype;
    dqr/dkr may be None with flags == 0); otherwise the outputs are allocated
    here. Calls that overlap on one GPU race."""
    T, lds, ld_rel, n_rel, nseq, band = _bwd_varlen_checks(
        q, k, v, out, dout, lse, qr, kr, rel_idx, rel_max_len, band, cu_seqlens, H, flags)
    if grads is None:
        grads = _bwd_outputs(q, T, H, d, n_rel, flags)
    dq, dk, dv, dqr, dkr = grads
    for name, t, rows in (("dq", dq, T), ("dk", dk, T), ("dv", dv, T), ("dqr", dqr, n_rel),
                          ("dkr", dkr, n_rel)):
        if t is None:
            if flags or name in ("dq", "dk", "dv"):
                raise ValueError(f"{name} is required")
            continue
        if (t.dtype != q.dtype or t.device != q.device or not t.is_contiguous()
                or t.numel() != rows * H * d):
            raise ValueError(f"{name} must be a contiguous [{rows}, {H * d}] tensor like q")
    st = lib().dattn_bwd_varlen_noalloc(
        _ptr(q), _ptr(k), _ptr(v), lds[0], lds[1], lds[2], _ptr(out), _ptr(dout), lds[3], lds[4],
        _ptr(lse), _ptr(qr), _ptr(kr), ld_rel, n_rel, _ptr(rel_idx), int(rel_max_len), band,
        _ptr(cu_seqlens), nseq, int(max_seqlen), T, _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dqr),
        _ptr(dkr), H, d, _dtype_code(q), int(flags), float(scale), _stream(q))
    _check(st, "dattn_bwd_varlen_noalloc")
    return dq, dk, dv, dqr, dkr


def pack_index(mask, B: Optional[int] = None, L: Optional[int] = None, *, device=None):
    """Packing metadata of a [B, L] mask (uint8/bool, or None for all valid,
    then B and L are required): returns device int32 tensors (cu_seqlens
    [B+1], token_rows [B*L], row_to_packed [B*L], max_seqlen [1])."""
    import torch
    if mask is not None:
        if mask.dtype == torch.bool:
            mask = mask.view(torch.uint8)
        if mask.dtype != torch.uint8 or mask.dim() != 2 or not mask.is_contiguous():
            raise ValueError("mask must be a contiguous [B, L] uint8/bool tensor")
        B, L = mask.shape
        device = mask.device
    if B is None or L is None:
        raise ValueError("B and L are required without a mask")
    device = device if device is not None else "cuda"
    i32 = dict(dtype=torch.int32, device=device)
    cu = torch.empty(B + 1, **i32)
    token_rows = torch.empty(B * L, **i32)
    row_to_packed = torch.empty(B * L, **i32)
    max_len = torch.empty(1, **i32)
    st = lib().dattn_pack_index(_ptr(mask), int(B), int(L), _ptr(cu), _ptr(token_rows),
                                _ptr(row_to_packed), _ptr(max_len), _stream(cu))
    _check(st, "dattn_pack_index")
    return cu, token_rows, row_to_packed, max_len


def _rows2d(t, name: str):
    """[..., W] with a contiguous last dimension and uniformly strided rows ->
    (n_rows, row_bytes, row_stride_bytes)."""
    if t.dim() < 2 or t.stride(-1) != 1:
        raise ValueError(f"{name}: rows must have a contiguous last dimension")
    ld = t.stride(-2)
    expect = ld
    for i in range(t.dim() - 3, -1, -1):
        expect *= t.shape[i + 1]
        if t.shape[i] > 1 and t.stride(i) != expect:
            raise ValueError(f"{name}: rows must be uniformly strided")
    n = t.numel() // t.shape[-1] if t.shape[-1] else 0
    es = t.element_size()
    return n, t.shape[-1] * es, ld * es


def pack_rows(src, token_rows, total: Optional[int] = None, *, out=None):
    """src [B, L, W] or [B*L, W] -> out [total, W] (out[r] = src[token_rows[r]]).
    total defaults to B*L (rows past cu[B] are then left unwritten)."""
    import torch
    n_src, row_bytes, ld_src = _rows2d(src, "src")
    W = src.shape[-1]
    if out is None:
        out = torch.empty((n_src if total is None else int(total), W), dtype=src.dtype,
                          device=src.device)
    if out.dtype != src.dtype or out.shape[-1] != W:
        raise ValueError("out must match src in dtype and row width")
    n_out, _, ld_dst = _rows2d(out, "out")
    n_rows = min(token_rows.numel(), n_out)
    st = lib().dattn_pack_rows(_ptr(src), ld_src, n_src, _ptr(token_rows), n_rows, row_bytes,
                               _ptr(out), ld_dst, _stream(src))
    _check(st, "dattn_pack_rows")
    return out


def unpack_rows(src, row_to_packed, B: int, L: int, *, out=None):
    """src [T, W] packed rows -> out [B, L, W] with zero rows at the padding."""
    import torch
    n_src, row_bytes, ld_src = _rows2d(src, "src")
    W = src.shape[-1]
    if out is None:
        out = torch.empty((B, L, W), dtype=src.dtype, device=src.device)
    n_out, _, ld_dst = _rows2d(out, "out")
    if n_out != B * L or out.dtype != src.dtype or out.shape[-1] != W:
        raise ValueError("out must hold B*L rows of src's width and dtype")
    if row_to_packed.numel() < B * L:
        raise ValueError("row_to_packed must have B*L entries")
    st = lib().dattn_unpack_rows(_ptr(src), ld_src, n_src, _ptr(row_to_packed), B * L, row_bytes,
                                 _ptr(out), ld_dst, _stream(src))
    _check(st, "dattn_unpack_rows")
    return out


def rel_proj(E, Wq, Wk, bq=None, bk=None, *, qr=None, kr=None):
    """qr = E Wq^T + bq and kr = E Wk^T + bk in one launch. E is [n_rel,
    hidden]; Wq, Wk are [H*d, hidden] (nn.Linear weights); biases [H*d] or
    None. Returns (qr, kr), [n_rel, H*d] in E's dtype."""
    import torch
    n_rel, hidden = E.shape
    HD = Wq.shape[0]
    if Wk.shape != Wq.shape or Wq.shape[1] != hidden:
        raise ValueError("Wq and Wk must be [H*d, hidden]")
    if Wk.stride() != Wq.stride():
        raise ValueError("Wq and Wk must have the same strides")
    for name, t in (("E", E), ("Wq", Wq), ("Wk", Wk)):
        if t.dtype != E.dtype:
            raise ValueError(f"{name} must have E's dtype")
    for name, t in (("bq", bq), ("bk", bk)):
        if t is not None and (t.dtype != E.dtype or t.numel() != HD or not t.is_contiguous()):
            raise ValueError(f"{name} must be a contiguous [H*d] tensor of E's dtype")
    if qr is None:
        qr = torch.empty((n_rel, HD), dtype=E.dtype, device=E.device)
    if kr is None:
        kr = torch.empty((n_rel, HD), dtype=E.dtype, device=E.device)
    if kr.stride() != qr.stride() or kr.shape != qr.shape:
        raise ValueError("qr and kr must have the same shape and strides")
    st = lib().dattn_rel_proj(_ptr(E), _row_stride(E, "E"), _ptr(Wq), _ptr(Wk),
                              _row_stride(Wq, "Wq"), _ptr(bq), _ptr(bk), _ptr(qr), _ptr(kr),
                              _row_stride(qr, "qr"), int(n_rel), int(hidden), int(HD),
                              _dtype_code(E), _stream(E))
    _check(st, "dattn_rel_proj")
    return qr, kr
