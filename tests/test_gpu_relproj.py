"""GPU parity of the relative-table projection (dattn_rel_proj) against the
float64 oracle (oracle/relproj.py).

Bar, per output: |got - want| <= 2^-p |want| + 2 hidden 2^-24 bound, with
p = 8 (bf16), 10 (fp16), and no rounding term for fp32: the first term is
the one rounding of the fp32 result to the element type (half an ulp,
doubled), the second bounds the fp32 accumulation over `hidden` products,
bound = sum_i |E_ri W_oi| + |b_o| (oracle.relproj.abs_bound). Shapes cover
the v3-base projection (512 x 768 -> 768), ragged row and column tiles,
no bias, and strided operands. The end-to-end case projects the v3-base
tables on the device and runs the padded forward on them.
"""

import sys

import numpy as np
import pytest

import oracle
import workloads
from oracle import relproj as P
from tests import helpers as H

pytestmark = pytest.mark.gpu

REL_BITS = {"bf16": 8, "fp16": 10}


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _check(got, want, E, W, b, hidden, dtype, tag):
    bound = P.abs_bound(E, W) + (0.0 if b is None else np.abs(b)[None, :])
    tol = 2.0 * hidden * 2.0 ** -24 * bound
    if dtype in REL_BITS:
        tol = tol + 2.0 ** -REL_BITS[dtype] * np.abs(want)
    err = np.abs(got - want)
    assert np.all(np.isfinite(got)), tag
    worst = float((err / np.maximum(tol, 1e-30)).max())
    assert np.all(err <= tol), f"{tag}: worst err/tol {worst:.3f}"
    return worst


@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("n_rel,hidden,HD,bias", [
    (512, 768, 768, True), (100, 64, 96, True), (37, 48, 32, False), (1, 16, 32, True),
    (256, 1024, 1024, True), (130, 1536, 1536, False),
])
def test_rel_proj_matches_oracle(dtype, n_rel, hidden, HD, bias):
    import torch
    import deberta_disentangled_attention_amd as dd
    _say(f"rel_proj {dtype} n_rel={n_rel} hidden={hidden} HD={HD} bias={bias}")
    E, Wq, Wk, bq, bk = workloads.projection_inputs(n_rel + hidden + HD, n_rel, hidden, HD, dtype,
                                                    bias=bias)
    dev = lambda x: None if x is None else H.dev(x, dtype)
    qr, kr = dd.rel_proj(dev(E), dev(Wq), dev(Wk), dev(bq), dev(bk))
    torch.cuda.synchronize()
    wq, wk = P.rel_proj(E, Wq, Wk, bq, bk)
    r1 = _check(H.host(qr), wq, E, Wq, bq, hidden, dtype, "qr")
    r2 = _check(H.host(kr), wk, E, Wk, bk, hidden, dtype, "kr")
    _say(f"  worst err/tol {max(r1, r2):.3f}")


def test_rel_proj_strided_operands():
    """E, the weights and the outputs inside wider buffers."""
    import torch
    import deberta_disentangled_attention_amd as dd
    n_rel, hidden, HD, dtype = 70, 96, 64, "bf16"
    E, Wq, Wk, bq, bk = workloads.projection_inputs(3, n_rel, hidden, HD, dtype)
    Ebig = torch.zeros((n_rel, hidden + 32), dtype=torch.bfloat16, device="cuda")
    Ebig[:, 16:16 + hidden] = H.dev(E, dtype)
    Wbig = torch.zeros((2, HD, hidden + 16), dtype=torch.bfloat16, device="cuda")
    Wbig[0, :, :hidden] = H.dev(Wq, dtype)
    Wbig[1, :, :hidden] = H.dev(Wk, dtype)
    out = torch.full((2, n_rel, HD + 8), 3.0, dtype=torch.bfloat16, device="cuda")
    dd.rel_proj(Ebig[:, 16:16 + hidden], Wbig[0, :, :hidden], Wbig[1, :, :hidden],
                H.dev(bq, dtype), H.dev(bk, dtype), qr=out[0, :, :HD], kr=out[1, :, :HD])
    torch.cuda.synchronize()
    o = H.host(out)
    wq, wk = P.rel_proj(E, Wq, Wk, bq, bk)
    _check(o[0, :, :HD], wq, E, Wq, bq, hidden, dtype, "qr")
    _check(o[1, :, :HD], wk, E, Wk, bk, hidden, dtype, "kr")
    assert np.all(o[:, :, HD:] == 3.0)


def test_projected_tables_feed_the_forward():
    """v3-base shape: tables projected on the device, then the padded
    forward; compared with the oracle forward on the exact projection."""
    import torch
    import deberta_disentangled_attention_amd as dd
    w = workloads.c2_v3base_bf16()
    hidden = w.H * w.d
    E, Wq, Wk, bq, bk = workloads.projection_inputs(11, w.n_rel, hidden, hidden, w.dtype)
    qr, kr = dd.rel_proj(H.dev(E, w.dtype), H.dev(Wq, w.dtype), H.dev(Wk, w.dtype),
                         H.dev(bq, w.dtype), H.dev(bk, w.dtype))
    T = H.gpu_table(w.L, w.position_buckets, w.max_relative_positions)
    m = torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).cuda()
    out = dd.dattn_fwd_padded(H.dev(w.q, w.dtype), H.dev(w.k, w.dtype), H.dev(w.v, w.dtype),
                              qr, kr, T, w.L, m, w.H, w.d, flags=w.flags)
    torch.cuda.synchronize()
    wq, wk = P.rel_proj(E, Wq, Wk, bq, bk)
    Tn = oracle.rel_index_table(w.L, w.position_buckets, w.max_relative_positions)
    want = oracle.dattn_padded(w.q, w.k, w.v, wq, wk, Tn, w.L, w.mask, w.H, w.d, w.flags, 0.0)
    worst = H.assert_padded_close(H.host(out), want, H.valid_rows_padded(w), w.dtype, "proj+fwd")
    _say(f"projected tables + forward: max abs err {worst:.3e}")
