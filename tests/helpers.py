"""Shared helpers for the GPU tests: move seeded workloads to the device,
call the HIP path through the binding, and compare with the oracle."""

from __future__ import annotations

import numpy as np

import oracle
import workloads

TOL = {"fp32": 1e-5, "fp16": 5e-3, "bf16": 1.5e-2}


def torch_dtype(dtype: str):
    import torch
    return {"fp32": torch.float32, "fp16": torch.float16, "bf16": torch.bfloat16}[dtype]


def dev(x: np.ndarray, dtype: str):
    """float32 array holding values exact in `dtype` -> device tensor."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32)).to(torch_dtype(dtype)).cuda()


def host(t) -> np.ndarray:
    return t.float().cpu().numpy().astype(np.float64)


def gpu_table(max_len, P, M):
    import deberta_disentangled_attention_amd as dd
    return dd.rel_bucket(max_len, P, M, device="cuda")


def run_padded(w: workloads.Workload, rel_max_len=None, flags=None, scale=0.0, mask=None,
               q=None, k=None, v=None, lse=None, table=None):
    """The padded forward of w on the GPU; `table` (host int array) replaces
    the rel_bucket table."""
    import torch
    import deberta_disentangled_attention_amd as dd
    rel_max_len = rel_max_len or w.L
    flags = w.flags if flags is None else flags
    T = (gpu_table(rel_max_len, w.position_buckets, w.max_relative_positions) if table is None
         else torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda())
    mask = w.mask if mask is None else mask
    if isinstance(mask, torch.Tensor):
        m = mask   # a device tensor, passed as it is (its address included)
    else:
        m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask, np.uint8)).cuda()
    out = dd.dattn_fwd_padded(q if q is not None else dev(w.q, w.dtype),
                              k if k is not None else dev(w.k, w.dtype),
                              v if v is not None else dev(w.v, w.dtype),
                              dev(w.qr, w.dtype), dev(w.kr, w.dtype), T, rel_max_len, m,
                              w.H, w.d, flags=flags, scale=scale, lse=lse)
    torch.cuda.synchronize()
    return out


def run_varlen(w: workloads.Workload, rel_max_len=None, flags=None, scale=0.0, lse=None,
               table=None):
    import torch
    import deberta_disentangled_attention_amd as dd
    rel_max_len = rel_max_len or max(w.max_seqlen, 1)
    flags = w.flags if flags is None else flags
    T = (gpu_table(rel_max_len, w.position_buckets, w.max_relative_positions) if table is None
         else torch.from_numpy(np.ascontiguousarray(table, np.int32)).cuda())
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    out = dd.dattn_fwd_varlen(dev(w.q, w.dtype), dev(w.k, w.dtype), dev(w.v, w.dtype),
                              dev(w.qr, w.dtype), dev(w.kr, w.dtype), T, rel_max_len, cu,
                              w.max_seqlen, w.H, w.d, flags=flags, scale=scale, lse=lse)
    torch.cuda.synchronize()
    return out


def oracle_padded(w, rel_max_len=None, flags=None, scale=0.0, mask="w"):
    rel_max_len = rel_max_len or w.L
    T = oracle.rel_index_table(rel_max_len, w.position_buckets, w.max_relative_positions)
    flags = w.flags if flags is None else flags
    return oracle.dattn_padded(w.q, w.k, w.v, w.qr, w.kr, T, rel_max_len,
                               w.mask if isinstance(mask, str) else mask, w.H, w.d, flags, scale)


def oracle_varlen(w, rel_max_len=None, flags=None, scale=0.0):
    rel_max_len = rel_max_len or max(w.max_seqlen, 1)
    T = oracle.rel_index_table(rel_max_len, w.position_buckets, w.max_relative_positions)
    flags = w.flags if flags is None else flags
    return oracle.dattn_varlen(w.q, w.k, w.v, w.qr, w.kr, T, rel_max_len, w.cu_seqlens,
                               w.H, w.d, flags, scale)


def valid_rows_padded(w, mask=None):
    m = w.mask if mask is None else mask
    if m is None:
        return np.ones((w.B, w.L), dtype=bool)
    return np.asarray(m).astype(bool)


def assert_padded_close(got: np.ndarray, want: np.ndarray, valid: np.ndarray, dtype: str,
                        tag: str = ""):
    """Valid rows within the dtype's max-abs tolerance; padded rows exactly 0."""
    tol = TOL[dtype]
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.all(np.isfinite(got)), f"{tag}: non-finite outputs"
    err = np.abs(got[valid] - want[valid])
    worst = float(err.max()) if err.size else 0.0
    assert worst <= tol, f"{tag}: max abs err {worst:.3e} > {tol:.1e}"
    assert np.all(got[~valid] == 0.0), f"{tag}: padded rows not zero"
    return worst
