"""The allocation-free backward (dattn_bwd_varlen_noalloc, workspace in the
library's fixed per-GPU array) against the workspace entry point
(dattn_bwd_varlen) on the same inputs: two calls in a row, the second on a
smaller batch, so whatever the first call left in the shared array must not
leak into the second. Both run the same kernels, which reduce in a fixed
order, so the outputs must be bitwise identical."""

import sys

import numpy as np
import pytest

import workloads
from tests import helpers as H

pytestmark = pytest.mark.gpu

NAMES = ("dq", "dk", "dv", "dqr", "dkr")


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _both(lens, dtype, flags, seed):
    import torch
    import deberta_disentangled_attention_amd as dd
    lens = np.asarray(lens)
    w = workloads.make_workload(f"noalloc_{dtype}", dtype=dtype, B=len(lens), L=int(lens.max()), H=4,
                                d=64, position_buckets=64, max_relative_positions=128, lens=lens,
                                seed=seed, packed=True, flags=flags)
    rel_max_len = max(w.max_seqlen, 1)
    Tg = H.gpu_table(rel_max_len, w.position_buckets, w.max_relative_positions)
    cu = torch.from_numpy(w.cu_seqlens).cuda()
    q, k, v = H.dev(w.q, dtype), H.dev(w.k, dtype), H.dev(w.v, dtype)
    qr, kr = H.dev(w.qr, dtype), H.dev(w.kr, dtype)
    out, lse = dd.dattn_fwd_varlen(q, k, v, qr, kr, Tg, rel_max_len, cu, w.max_seqlen, w.H, w.d,
                                   flags=flags, lse=True)
    rng = np.random.default_rng(seed + 1)
    dout = H.dev(workloads.round_to(rng.standard_normal(w.q.shape).astype(np.float32), dtype), dtype)
    band = dd.rel_bucket_band(rel_max_len, w.position_buckets, w.max_relative_positions)
    need = dd.bwd_workspace_size(w.total_tokens, len(lens), w.H, w.d, q.dtype, band if flags else 1)
    assert need <= dd.DATTN_NOALLOC_SCRATCH_BYTES
    args = (q, k, v, out, dout, lse, qr, kr, Tg, rel_max_len, band, cu, w.max_seqlen, w.H, w.d)
    ref = dd.dattn_bwd_varlen(*args, flags=flags)
    got = dd.dattn_bwd_varlen_noalloc(*args, flags=flags)
    torch.cuda.synchronize()
    return ref, got


@pytest.mark.parametrize("dtype,flags", [("bf16", 3), ("fp32", 3), ("fp16", 0)])
def test_noalloc_equals_workspace_entry_two_calls(dtype, flags):
    for call, lens in enumerate(([300, 77, 0, 129], [50, 20])):
        _say(f"noalloc {dtype} flags={flags} call {call} lens={lens}")
        ref, got = _both(lens, dtype, flags, seed=40 + call)
        for name, a, b in zip(NAMES, ref, got):
            if a is None:
                assert b is None
                continue
            assert bool((a == b).all()), f"call {call} {name}: differs from dattn_bwd_varlen"
