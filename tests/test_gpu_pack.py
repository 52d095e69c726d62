"""GPU parity of the packing entry points against the oracle: bit-exact.

Index arrays (cu_seqlens, token_rows, row_to_packed, max_seqlen) and the
copied rows must equal oracle/pack.py exactly. Masks cover right padding,
holes, empty rows, all-valid and NULL, lengths that are not multiples of
the 64- and 256-token chunks, more rows than the scans' 1024-entry chunk,
the longest supported sequence, and batches on both sides of the
one-workgroup path's limits. Row widths cover 16 bytes, widths below one
wave's 1024 bytes, exact multiples, and fused-QKV rows that take the
four-deep copy loop plus a tail. The end-to-end case packs the c3 batch
(deberta-v2-xlarge shape, 92.6% padding) on the device, runs the packed
forward and unpacks: the result must equal the padded forward bit for bit.
"""

import sys

import numpy as np
import pytest

import workloads
from oracle import pack as P
from tests import helpers as H

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, file=sys.stderr, flush=True)


def _mask(kind, B, L, seed):
    rng = np.random.default_rng(seed)
    if kind == "right":
        lens = rng.integers(0, L + 1, size=B)
        lens[:1] = L
        return workloads.right_pad_mask(lens, L)
    if kind == "holes":
        return (rng.random((B, L)) < 0.3).astype(np.uint8) * rng.integers(1, 256, (B, L)).astype(np.uint8)
    if kind == "empty_rows":
        m = (rng.random((B, L)) < 0.8).astype(np.uint8)
        m[::3] = 0
        return m
    if kind == "zeros":
        return np.zeros((B, L), np.uint8)
    if kind == "ones":
        return np.ones((B, L), np.uint8)
    return None


def _gpu_index(mask, B, L):
    import torch
    import deberta_disentangled_attention_amd as dd
    m = None if mask is None else torch.from_numpy(np.ascontiguousarray(mask)).cuda()
    out = dd.pack_index(m, B, L, device="cuda")
    torch.cuda.synchronize()
    return [t.cpu().numpy().astype(np.int64) for t in out]


@pytest.mark.parametrize("kind", ["right", "holes", "empty_rows", "zeros", "ones", "null"])
@pytest.mark.parametrize("B,L", [(1, 1), (3, 37), (16, 512), (5, 300), (1500, 3), (2, 8192),
                                 (7, 257), (1, 0), (0, 5),
                                 # past the one-workgroup limits (4096 rows, 2^18 tokens)
                                 (5000, 3), (64, 8192), (4096, 64), (4097, 1)])
def test_pack_index_bit_exact(kind, B, L):
    _say(f"pack_index {kind} B={B} L={L}")
    mask = _mask(kind, B, L, seed=B * 131 + L)
    cu, tr, rp, mx = _gpu_index(mask, B, L)
    wcu, wtr, wrp = P.pack_index(mask, B, L)
    assert np.array_equal(cu, wcu)
    assert np.array_equal(tr, wtr)
    assert np.array_equal(rp, wrp)
    assert int(mx[0]) == (int(np.diff(wcu).max()) if B else 0)


@pytest.mark.parametrize("W,dtype", [(8, "fp16"), (40, "fp32"), (1536, "fp16"), (4608, "bf16"),
                                     (520, "fp16"), (2048, "fp32")])
def test_pack_unpack_rows_bit_exact(W, dtype):
    import torch
    import deberta_disentangled_attention_amd as dd
    B, L = 6, 203
    mask = _mask("holes" if W % 3 else "right", B, L, seed=W)
    rng = np.random.default_rng(W)
    x = rng.standard_normal((B, L, W)).astype(np.float32)
    _say(f"pack rows W={W} {dtype}")
    xd = H.dev(x, dtype)
    xh = xd.float().cpu().numpy()
    cu, tr, rp, _ = dd.pack_index(torch.from_numpy(mask).cuda())
    total = int(cu[-1].item())
    packed = dd.pack_rows(xd, tr, total)
    torch.cuda.synchronize()
    wcu, wtr, wrp = P.pack_index(mask, B, L)
    want = P.pack_rows(xh.reshape(B * L, W), wtr, total)
    assert np.array_equal(packed.float().cpu().numpy(), want)
    back = dd.unpack_rows(packed, rp, B, L)
    torch.cuda.synchronize()
    assert np.array_equal(back.float().cpu().numpy().reshape(B * L, W), P.unpack_rows(want, wrp))


def test_strided_views_and_untouched_tail():
    """Source rows that are a slice of wider rows; destination rows inside a
    wider buffer; rows past the packed total keep their old contents."""
    import torch
    import deberta_disentangled_attention_amd as dd
    B, L, W = 4, 100, 64
    mask = _mask("right", B, L, seed=3)
    rng = np.random.default_rng(3)
    base = torch.from_numpy(rng.standard_normal((B, L, 3 * W)).astype(np.float32)).cuda().half()
    src = base[..., W:2 * W]                       # the K third of a fused buffer
    cu, tr, rp, _ = dd.pack_index(torch.from_numpy(mask).cuda())
    total = int(cu[-1].item())
    big = torch.full((B * L, 2 * W), 7.0, dtype=torch.float16, device="cuda")
    dst = big[:, :W]
    dd.pack_rows(src, tr, out=dst)                 # capacity B*L rows, only `total` written
    torch.cuda.synchronize()
    wcu, wtr, wrp = P.pack_index(mask, B, L)
    want = P.pack_rows(src.float().cpu().numpy().reshape(B * L, W), wtr, total)
    got = big.float().cpu().numpy()
    assert np.array_equal(got[:total, :W], want)
    assert np.all(got[total:, :W] == 7.0) and np.all(got[:, W:] == 7.0)
    out = torch.full((B, L, 2 * W), 5.0, dtype=torch.float16, device="cuda")
    dd.unpack_rows(dst[:total], rp, B, L, out=out[..., W:])
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().reshape(B * L, 2 * W)
    assert np.array_equal(o[:, W:], P.unpack_rows(want, wrp))
    assert np.all(o[:, :W] == 5.0)


def test_c3_pack_varlen_unpack_equals_padded():
    """Device packing of the fused QKV buffer -> packed forward -> unpack
    equals the padded forward on the same batch exactly."""
    import torch
    import deberta_disentangled_attention_amd as dd
    w = workloads.c3_v2xlarge_fp16()
    hd = w.H * w.d
    _say("c3 pack -> varlen -> unpack")
    qkv = torch.cat([H.dev(w.q, w.dtype), H.dev(w.k, w.dtype), H.dev(w.v, w.dtype)], dim=-1)
    mask = torch.from_numpy(np.ascontiguousarray(w.mask, np.uint8)).cuda()
    ref = dd.dattn_fwd_padded(qkv[..., :hd], qkv[..., hd:2 * hd], qkv[..., 2 * hd:],
                              H.dev(w.qr, w.dtype), H.dev(w.kr, w.dtype),
                              H.gpu_table(w.L, w.position_buckets, w.max_relative_positions),
                              w.L, mask, w.H, w.d, flags=w.flags)
    cu, tr, rp, mx = dd.pack_index(mask)
    total, max_len = int(cu[-1].item()), int(mx.item())
    assert total == int(np.sum(w.lens)) and max_len == int(np.max(w.lens))
    packed = dd.pack_rows(qkv, tr, total)
    # the same relative table as the padded call, so both take the same tile paths
    T = H.gpu_table(w.L, w.position_buckets, w.max_relative_positions)
    o = dd.dattn_fwd_varlen(packed[:, :hd], packed[:, hd:2 * hd], packed[:, 2 * hd:],
                            H.dev(w.qr, w.dtype), H.dev(w.kr, w.dtype), T, w.L, cu, max_len,
                            w.H, w.d, flags=w.flags)
    back = dd.unpack_rows(o, rp, w.B, w.L)
    torch.cuda.synchronize()
    assert torch.equal(back, ref)
    assert np.array_equal(cu.cpu().numpy(), w.cu_seqlens)
