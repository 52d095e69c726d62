"""C-ABI contract of libdattn.so, on the CPU.

The library must load and export every function include/dattn.h declares.
Argument validation runs on the host before any HIP call, so invalid calls
can be checked here without a GPU: each returns its documented status and
launches nothing. No compute call is made.
"""

import ctypes
import os
import re

import pytest

import deberta_disentangled_attention_amd as dd

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dattn.h")

pytestmark = pytest.mark.skipif(not os.path.exists(dd.LIB_PATH),
                                reason="libdattn.so not built")

INV, UNS = dd.DATTN_ERR_INVALID_ARGUMENT, dd.DATTN_ERR_UNSUPPORTED
A = 4096            # a fake, 16-byte aligned "device address": never dereferenced
MIS = A + 2         # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\(", text, flags=re.M)))


def test_every_declared_symbol_is_exported():
    names = declared_functions()
    assert set(names) >= {"rel_bucket", "dattn_fwd_padded", "dattn_fwd_varlen", "dattn_strerror"}
    h = dd.lib()
    for n in names:
        assert hasattr(h, n), n


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define\s+(DATTN_\w+)\s+(\w+)", text))
    for k, v in consts.items():
        if k in ("DATTN_H",):
            continue
        assert getattr(dd, k) == int(v.rstrip("u")), k


def test_strerror():
    assert dd.strerror(0) == "ok"
    assert dd.strerror(1) == "invalid argument"
    assert dd.strerror(2) == "unsupported configuration"
    assert dd.strerror(3) == "HIP launch failure"
    assert dd.strerror(99) == "unknown status"


def padded(**kw):
    a = dict(q=A, k=A, v=A, ld_q=768, ld_k=768, ld_v=768, qr=A, kr=A, ld_rel=768, n_rel=512,
             rel_idx=A, rel_max_len=512, mask=None, out=A, B=2, L=512, H=12, d=64, dtype=2,
             flags=3, scale=0.0, stream=None)
    a.update(kw)
    return dd.lib().dattn_fwd_padded(*a.values())


def varlen(**kw):
    a = dict(q=A, k=A, v=A, ld_q=768, ld_k=768, ld_v=768, qr=A, kr=A, ld_rel=768, n_rel=512,
             rel_idx=A, rel_max_len=512, cu=A, nseq=2, max_seqlen=512, total=1000, out=A, H=12,
             d=64, dtype=2, flags=3, scale=0.0, stream=None)
    a.update(kw)
    return dd.lib().dattn_fwd_varlen(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INV), (dict(k=None), INV), (dict(v=None), INV), (dict(out=None), INV),
    (dict(qr=None), INV), (dict(kr=None), INV), (dict(rel_idx=None), INV),
    (dict(H=0), INV), (dict(B=-1), INV), (dict(L=-1), INV), (dict(ld_q=767), INV),
    (dict(n_rel=0), INV), (dict(rel_max_len=511), INV), (dict(flags=4), INV),
    (dict(scale=float("nan")), INV),
    (dict(d=48), UNS), (dict(d=256), UNS), (dict(dtype=3), UNS), (dict(L=8193, rel_max_len=9000), UNS),
    (dict(q=MIS), UNS), (dict(out=MIS), UNS), (dict(ld_q=772), UNS), (dict(qr=MIS), UNS),
    (dict(dtype=0, ld_q=770), UNS),
    # relative tables whose row offsets would not fit in 31 bits
    (dict(n_rel=1 << 20, ld_rel=1 << 10), UNS), (dict(n_rel=1 << 20, ld_rel=1 << 10, flags=1), UNS),
    (dict(rel_idx=A + 2), UNS),
])
def test_padded_rejections(kw, status):
    assert padded(**kw) == status


@pytest.mark.parametrize("kw", [dict(B=0), dict(L=0),
                                dict(B=0, flags=0, qr=None, kr=None, rel_idx=None)])
def test_padded_empty_is_noop(kw):
    assert padded(**kw) == dd.DATTN_OK


def test_flags0_needs_no_relative_tables():
    # still rejected for another reason (d) -> proves the tables were not required
    assert padded(flags=0, qr=None, kr=None, rel_idx=None, d=48) == UNS
    assert padded(flags=0, qr=None, kr=None, rel_idx=None, n_rel=0, rel_max_len=0, B=0) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(cu=None), INV), (dict(nseq=-1), INV), (dict(total=-1), INV), (dict(max_seqlen=-1), INV),
    (dict(rel_max_len=100), INV), (dict(max_seqlen=9000, rel_max_len=9000), UNS), (dict(q=None), INV),
    (dict(d=16), UNS), (dict(k=MIS), UNS), (dict(n_rel=1 << 20, ld_rel=1 << 10), UNS),
    (dict(cu=A + 2), UNS),
])
def test_varlen_rejections(kw, status):
    assert varlen(**kw) == status


@pytest.mark.parametrize("kw", [dict(nseq=0), dict(total=0)])
def test_varlen_empty_is_noop(kw):
    assert varlen(**kw) == dd.DATTN_OK


@pytest.mark.parametrize("args,status", [
    ((None, 10, 256, 512), INV), ((A, 0, 256, 512), INV), ((A, 10, 1, 512), INV),
    ((A, 10, 256, 129), INV), ((A, 10, 0, 0), INV), ((A, 70000, 256, 512), UNS),
    ((A + 2, 10, 256, 512), UNS), ((A, 10, 4098, 9000), UNS),
])
def test_rel_bucket_rejections(args, status):
    assert dd.lib().rel_bucket(*args, None) == status


def pack_index(**kw):
    a = dict(mask=A, B=4, L=512, cu=A, token_rows=A, row_to_packed=A, max_seqlen=None,
             stream=None)
    a.update(kw)
    return dd.lib().dattn_pack_index(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(B=-1), INV), (dict(L=-1), INV), (dict(cu=None), INV), (dict(token_rows=None), INV),
    (dict(row_to_packed=None), INV), (dict(B=1 << 16, L=1 << 16), UNS),
    (dict(cu=A + 2), UNS), (dict(token_rows=A + 1), UNS), (dict(max_seqlen=A + 2), UNS),
])
def test_pack_index_rejections(kw, status):
    assert pack_index(**kw) == status


def rows(fn, **kw):
    a = dict(src=A, ld_src=3072, n_src=2048, index=A, n_rows=2048, row_bytes=3072, dst=A,
             ld_dst=3072, stream=None)
    a.update(kw)
    return getattr(dd.lib(), fn)(*a.values())


@pytest.mark.parametrize("fn", ["dattn_pack_rows", "dattn_unpack_rows"])
@pytest.mark.parametrize("kw,status", [
    (dict(src=None), INV), (dict(dst=None), INV), (dict(index=None), INV),
    (dict(n_rows=-1), INV), (dict(n_src=-1), INV), (dict(row_bytes=-16), INV),
    (dict(ld_src=3056), INV), (dict(ld_dst=3056), INV),
    (dict(row_bytes=3064, ld_src=3072, ld_dst=3072), UNS), (dict(ld_src=3080), UNS),
    (dict(ld_dst=3080), UNS), (dict(src=MIS), UNS), (dict(dst=MIS), UNS),
    (dict(index=A + 2), UNS),
])
def test_row_copy_rejections(fn, kw, status):
    assert rows(fn, **kw) == status


@pytest.mark.parametrize("fn", ["dattn_pack_rows", "dattn_unpack_rows"])
@pytest.mark.parametrize("kw", [dict(n_rows=0), dict(row_bytes=0), dict(n_rows=0, src=None)])
def test_row_copy_empty_is_noop(fn, kw):
    assert rows(fn, **kw) == dd.DATTN_OK


def rel_proj(**kw):
    a = dict(E=A, ld_e=768, Wq=A, Wk=A, ld_w=768, bq=None, bk=None, qr=A, kr=A, ld_out=768,
             n_rel=512, hidden=768, HD=768, dtype=2, stream=None)
    a.update(kw)
    return dd.lib().dattn_rel_proj(*a.values())


@pytest.mark.parametrize("kw,status", [
    (dict(n_rel=-1), INV), (dict(hidden=-16), INV), (dict(HD=-1), INV), (dict(E=None), INV),
    (dict(Wq=None), INV), (dict(Wk=None), INV), (dict(qr=None), INV), (dict(kr=None), INV),
    (dict(ld_e=700), INV), (dict(ld_w=700), INV), (dict(ld_out=700), INV),
    (dict(dtype=5), UNS), (dict(hidden=760, ld_e=768, ld_w=768), UNS), (dict(hidden=0), UNS),
    (dict(E=MIS), UNS), (dict(Wk=MIS), UNS), (dict(ld_e=772), UNS), (dict(dtype=0, ld_w=770), UNS),
    (dict(qr=A + 1), UNS), (dict(kr=A + 1), UNS), (dict(bq=A + 1), UNS),
    (dict(dtype=0, kr=A + 2), UNS), (dict(dtype=0, bk=A + 2), UNS),
])
def test_rel_proj_rejections(kw, status):
    assert rel_proj(**kw) == status


@pytest.mark.parametrize("kw", [dict(n_rel=0), dict(HD=0), dict(n_rel=0, E=None)])
def test_rel_proj_empty_is_noop(kw):
    assert rel_proj(**kw) == dd.DATTN_OK


def padded_lse(**kw):
    a = dict(q=A, k=A, v=A, ld_q=768, ld_k=768, ld_v=768, qr=A, kr=A, ld_rel=768, n_rel=512,
             rel_idx=A, rel_max_len=512, mask=None, out=A, lse=A, B=2, L=512, H=12, d=64,
             dtype=2, flags=3, scale=0.0, stream=None)
    a.update(kw)
    return dd.lib().dattn_fwd_padded_lse(*a.values())


def varlen_lse(**kw):
    a = dict(q=A, k=A, v=A, ld_q=768, ld_k=768, ld_v=768, qr=A, kr=A, ld_rel=768, n_rel=512,
             rel_idx=A, rel_max_len=512, cu=A, nseq=2, max_seqlen=512, total=1000, out=A,
             lse=A, H=12, d=64, dtype=2, flags=3, scale=0.0, stream=None)
    a.update(kw)
    return dd.lib().dattn_fwd_varlen_lse(*a.values())


@pytest.mark.parametrize("fn", [padded_lse, varlen_lse])
@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), INV), (dict(lse=A + 2), UNS), (dict(q=None), INV), (dict(d=48), UNS),
])
def test_lse_rejections(fn, kw, status):
    assert fn(**kw) == status


def test_lse_empty_is_noop():
    assert padded_lse(B=0) == dd.DATTN_OK and varlen_lse(nseq=0) == dd.DATTN_OK


# ---------------------------------------------------------------------------
# the Python binding rejects buffers the kernels would overrun (CPU tensors:
# every check runs before the library is called)
# ---------------------------------------------------------------------------

def _cpu_inputs(B=2, L=16, H=2, d=32, n_rel=8, dtype="float16"):
    import torch
    t = getattr(torch, dtype)
    q = torch.zeros(B, L, H * d, dtype=t)
    qr = torch.zeros(n_rel, H * d, dtype=t)
    table = torch.zeros(2 * L - 1, dtype=torch.int32)
    return q, qr, table


@pytest.mark.parametrize("bad", ["shape", "dtype", "strided"])
def test_binding_rejects_bad_out_padded(bad):
    import torch
    q, qr, table = _cpu_inputs()
    out = {"shape": torch.zeros(2, 16, 32, dtype=torch.float16),
           "dtype": torch.zeros(2, 16, 64, dtype=torch.float32),
           "strided": torch.zeros(2, 16, 128, dtype=torch.float16)[..., :64]}[bad]
    with pytest.raises(ValueError, match="out must be"):
        dd.dattn_fwd_padded(q, q, q, qr, qr, table, 16, None, 2, 32, out=out)


def test_binding_rejects_bad_table_and_tokens_varlen():
    import torch
    q, qr, table = _cpu_inputs()
    qp = q.reshape(-1, q.shape[-1])
    cu = torch.tensor([0, 16, 32], dtype=torch.int32)
    with pytest.raises(ValueError, match="total_tokens exceeds"):
        dd.dattn_fwd_varlen(qp, qp, qp, qr, qr, table, 16, cu, 16, 2, 32, total_tokens=33)
    with pytest.raises(ValueError, match="rel_idx must be"):
        dd.dattn_fwd_varlen(qp, qp, qp, qr, qr, table[:-1], 16, cu, 16, 2, 32)
    with pytest.raises(ValueError, match="rel_idx must be"):
        dd.dattn_fwd_varlen(qp, qp, qp, qr, qr, table.to(torch.int64), 16, cu, 16, 2, 32)
    with pytest.raises(ValueError, match="rel_idx is required"):
        dd.dattn_fwd_varlen(qp, qp, qp, qr, qr, None, 16, cu, 16, 2, 32)
    with pytest.raises(ValueError, match="out must be"):
        dd.dattn_fwd_varlen(qp, qp, qp, qr, qr, table, 16, cu, 16, 2, 32,
                            out=torch.zeros(31, 64, dtype=torch.float16))
    with pytest.raises(ValueError, match="k must match"):
        dd.dattn_fwd_varlen(qp, qp.float(), qp, qr, qr, table, 16, cu, 16, 2, 32)


# ---------------------------------------------------------------------------
# backward entry points
# ---------------------------------------------------------------------------

def bwd_padded(**kw):
    a = dict(q=A, k=A, v=A, ld_q=768, ld_k=768, ld_v=768, out=A, dout=A, ld_o=768, ld_do=768,
             lse=A, qr=A, kr=A, ld_rel=768, n_rel=512, rel_idx=A, rel_max_len=512, band=512,
             mask=None, dq=A, dk=A, dv=A, dqr=A, dkr=A, ws=A, ws_bytes=1 << 40, B=2, L=512, H=12,
             d=64, dtype=dd.DATTN_BF16, flags=3, scale=0.0)
    a.update(kw)
    return dd.lib().dattn_bwd_padded(
        a["q"], a["k"], a["v"], a["ld_q"], a["ld_k"], a["ld_v"], a["out"], a["dout"], a["ld_o"],
        a["ld_do"], a["lse"], a["qr"], a["kr"], a["ld_rel"], a["n_rel"], a["rel_idx"],
        a["rel_max_len"], a["band"], a["mask"], a["dq"], a["dk"], a["dv"], a["dqr"], a["dkr"],
        a["ws"], a["ws_bytes"], a["B"], a["L"], a["H"], a["d"], a["dtype"], a["flags"], a["scale"],
        None)


@pytest.mark.parametrize("kw,status", [
    (dict(dout=None), INV), (dict(lse=None), INV), (dict(ws=None), INV), (dict(dkr=None), INV),
    (dict(band=0), INV), (dict(band=513), INV), (dict(ws_bytes=1000), INV), (dict(ld_do=100), INV),
    (dict(d=48), UNS), (dict(dout=MIS), UNS), (dict(ws=A + 8), UNS), (dict(lse=A + 2), UNS),
    (dict(B=-1), INV),
])
def test_bwd_rejections(kw, status):
    assert bwd_padded(**kw) == status


def test_bwd_empty_is_noop_and_flags0_needs_no_tables():
    assert bwd_padded(B=0) == dd.DATTN_OK
    assert bwd_padded(B=0, flags=0, qr=None, kr=None, rel_idx=None, dqr=None, dkr=None,
                      band=0) == dd.DATTN_OK


def test_bwd_workspace_size_and_band():
    lib = dd.lib()
    a = lib.dattn_bwd_workspace_size(131072, 16, 12, 64, dd.DATTN_BF16, 512)
    b = lib.dattn_bwd_workspace_size(131072, 16, 12, 64, dd.DATTN_BF16, 1)
    # the distance store grows by H * 2 * tokens elements per unit of band
    assert a - b >= 12 * 2 * 511 * 131072 * 2
    assert lib.dattn_bwd_workspace_size(10, 1, 1, 48, dd.DATTN_BF16, 1) == -1
    assert lib.dattn_bwd_workspace_size(10, 1, 1, 64, dd.DATTN_BF16, 0) == -1
    assert dd.rel_bucket_band(8192, 256, 512) == 512
    assert dd.rel_bucket_band(128, 0, 64) == 64
    assert lib.rel_bucket_band(10, 1, 512) == -1


def test_rel_bucket_band_matches_the_oracle_table():
    """The band is the least W with a constant table beyond +-W; checked on
    the oracle's exact tables."""
    import oracle
    for args in [(8192, 256, 512), (512, 256, 512), (700, 16, 64), (300, 20, 64), (128, 0, 64),
                 (1000, 0, 40), (3000, 4, 7)]:
        T = oracle.rel_index_table(*args)
        L = args[0]
        w = 1
        for r in range(L - 1, 0, -1):
            if T[r + L - 1] != T[-1] or T[-r + L - 1] != T[0]:
                w = r + 1
                break
        assert dd.rel_bucket_band(*args) == w, args


def test_noalloc_rejects_problems_beyond_its_array_before_any_hip_call():
    lib = dd.lib()
    args = [A, A, A, 768, 768, 768, A, A, 768, 768, A, A, A, 768, 512, A, 8192, 512, A, 16, 8192,
            131072, A, A, A, A, A, 12, 64, dd.DATTN_BF16, 3, 0.0, None]
    assert lib.dattn_bwd_varlen_noalloc(*args) == dd.DATTN_ERR_SCRATCH_TOO_SMALL
    assert b"allocation-free" in lib.dattn_strerror(dd.DATTN_ERR_SCRATCH_TOO_SMALL)
    args[1] = None   # argument errors come first
    assert lib.dattn_bwd_varlen_noalloc(*args) == INV


def fast_padded(**kw):
    a = dict(q=A, k=A, v=A, ld_q=768, ld_k=768, ld_v=768, qr=A, kr=A, ld_rel=768, n_rel=512,
             rel_idx=A, rel_max_len=512, mask=None, out=A, B=2, L=512, H=12, d=64, flags=3,
             scale=0.0, ws=A, ws_bytes=1 << 40)
    a.update(kw)
    return dd.lib().dattn_fwd_padded_f32fast(
        a["q"], a["k"], a["v"], a["ld_q"], a["ld_k"], a["ld_v"], a["qr"], a["kr"], a["ld_rel"],
        a["n_rel"], a["rel_idx"], a["rel_max_len"], a["mask"], a["out"], a["B"], a["L"], a["H"],
        a["d"], a["flags"], a["scale"], a["ws"], a["ws_bytes"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(ws=None), INV), (dict(ws_bytes=100), INV), (dict(ws=A + 8), UNS), (dict(q=A + 4), UNS),
    (dict(ld_q=770), UNS), (dict(d=48), UNS), (dict(L=9000), UNS), (dict(B=-1), INV),
    (dict(out=None), INV),
])
def test_fast_f32_rejections(kw, status):
    assert fast_padded(**kw) == status


def test_fast_f32_workspace_size():
    lib = dd.lib()
    # q, k, v and the fp16 output rows, then the two fp16 tables
    assert lib.dattn_fwd_f32fast_workspace_size(1024, 512, 16, 128) == 4 * 1024 * 2048 * 2 + 2 * 512 * 2048 * 2
    assert lib.dattn_fwd_f32fast_workspace_size(1, 0, 1, 32) == 4 * 256
    assert lib.dattn_fwd_f32fast_workspace_size(10, 0, 1, 48) == -1
    assert fast_padded(B=0) == dd.DATTN_OK
