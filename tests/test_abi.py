"""The C ABI: the library loads, exports every declared entry point, and
rejects bad arguments on the host before any HIP call (runs without a GPU)."""
import ctypes
import math
import os
import re

import pytest

import tiled_attention_04_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
S = fa.FaStrides
CONTIG = S(64 * 128 * 16, 64 * 128, 64, 1)  # [b, h, s=128, d=64]
BF16, F16, F32, E5M2 = fa.FA_DTYPE_BF16, fa.FA_DTYPE_F16, fa.FA_DTYPE_F32, fa.FA_DTYPE_E5M2
VT = S(2 * 64 * 128, 64 * 128, 1, 128)  # key-major V [b, h, d=64, s=128] (e5m2)
P = 1 << 20  # a 16-byte-aligned fake address (never dereferenced: calls fail validation)


def declared_functions():
    text = open(os.path.join(ROOT, "include", "fa.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z_0-9]+)\s*\(", text)))


def test_library_loads_with_all_symbols_resolved():
    lib = ctypes.CDLL(fa.LIB_PATH, mode=os.RTLD_NOW)
    assert lib is not None


def test_every_declared_entry_point_is_exported():
    names = declared_functions()
    assert set(names) == set(fa.EXPORTS), names
    lib = fa.lib()
    for n in names:
        assert hasattr(lib, n), n


def test_status_strings_and_version():
    lib = fa.lib()
    for code, name in fa.STATUS.items():
        assert lib.fa_status_string(code).decode() == name
    assert lib.fa_status_string(99).decode() == "FA_ERR_UNKNOWN"
    assert lib.fa_version() >= 100


def call(q=P, k=P, v=P, o=P, lse=None, batch=1, heads=2, sq=128, sk=128, d=64, qs=CONTIG,
         ks=CONTIG, vs=CONTIG, os_=CONTIG, scale=0.125, causal=0, dtype=BF16):
    return fa.fa_fwd(q, k, v, o, lse, batch, heads, sq, sk, d, qs, ks, vs, os_, scale, causal,
                     dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(batch=-1), 2), (dict(heads=-3), 2), (dict(sq=-1), 2), (dict(sk=0), 2),
    (dict(sk=-5), 2), (dict(sq=1 << 31), 2), (dict(batch=1 << 20, heads=1 << 12), 2),
    (dict(dtype=4), 3), (dict(dtype=-1), 3),
    (dict(d=0), 4), (dict(d=257), 4), (dict(d=12), 4), (dict(d=6, dtype=F32), 4),
    (dict(qs=S(0, 0, 64, 2)), 5), (dict(ks=S(0, -64, 64, 1)), 5), (dict(vs=S(0, 0, 68, 1)), 5),
    (dict(os_=S(0, 0, 1 << 24, 1)), 5), (dict(q=P + 8), 5), (dict(o=P + 2, dtype=F32), 5),
    (dict(lse=P + 2), 5),
    (dict(scale=math.nan), 7), (dict(scale=math.inf), 7), (dict(scale=-math.inf), 7),
    (dict(q=None), 1), (dict(o=None), 1), (dict(v=None, dtype=F32), 1),
])
def test_validation_errors(kwargs, code):
    rc = call(**kwargs)
    assert rc == code, (kwargs, rc, fa.last_error())
    assert fa.last_error() != ""


def test_empty_problem_is_ok_without_pointers():
    for kw in (dict(batch=0), dict(heads=0), dict(sq=0)):
        assert call(q=None, k=None, v=None, o=None, **kw) == 0
        assert fa.last_error() == ""


def test_fp32_accepts_unaligned_strides():
    # fp32 rows need only 4-byte alignment, so a seq stride of 65 passes
    # validation; with a NULL q the call then stops at the pointer check.
    rc = call(q=None, qs=S(0, 0, 65, 1), dtype=F32)
    assert rc == 1


@pytest.mark.parametrize("kwargs,code", [
    (dict(d=264), 4), (dict(d=24), 4), (dict(d=8), 4), (dict(d=200), 4),
    (dict(d=256, vs=S(0, 0, 1, (1 << 24) - 16)), 5),
    (dict(vs=CONTIG), 5), (dict(vs=S(0, 0, 1, 112)), 5), (dict(vs=S(0, 0, 1, 136)), 5),
    (dict(vs=S(8, 0, 1, 128)), 5), (dict(vs=S(0, 0, 1, 1 << 24)), 5),
    (dict(qs=S(0, 0, 72, 1)), 5), (dict(ks=S(0, 8, 64, 1)), 5), (dict(q=P + 8), 5),
    (dict(v=P + 4), 5),
    (dict(q=None), 1), (dict(d=16, q=None), 1), (dict(d=128, q=None, vs=S(0, 0, 1, 144)), 1),
])
def test_e5m2_validation_errors(kwargs, code):
    # q, k, o row-major with 16-byte rows; V key-major (seq stride 1, dim
    # stride a multiple of 16 that holds seq_k keys); head_dim 16..128 by 16
    args = dict(vs=VT, dtype=E5M2)
    args.update(kwargs)
    rc = call(**args)
    assert rc == code, (kwargs, rc, fa.last_error())
    assert fa.last_error() != ""


def call_bwd(q=P, k=P, v=P, o=P, do=P, lse=P, delta=P, dq=P, dk=P, dv=P, batch=1, heads=2,
             sq=128, sk=128, d=64, sts=None, scale=0.125, causal=0, dtype=BF16):
    st = dict(q=CONTIG, k=CONTIG, v=CONTIG, o=CONTIG, do=CONTIG, dq=CONTIG, dk=CONTIG, dv=CONTIG)
    st.update(sts or {})
    return fa.fa_bwd(q, k, v, o, do, lse, delta, dq, dk, dv, batch, heads, sq, sk, d,
                     st["q"], st["k"], st["v"], st["o"], st["do"], st["dq"], st["dk"], st["dv"],
                     scale, causal, dtype, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(batch=-1), 2), (dict(sq=-2), 2), (dict(sk=0), 2), (dict(sq=1 << 31), 2),
    (dict(dtype=E5M2), 3), (dict(dtype=5), 3), (dict(dtype=F32, d=6), 4),
    (dict(dtype=F32, d=132), 4), (dict(dtype=F32, dq=P + 2), 5), (dict(dtype=F32, k=None), 1),
    (dict(d=0), 4), (dict(d=264), 4), (dict(d=260), 4), (dict(d=60), 4),
    (dict(sts={"do": S(0, 0, 64, 2)}), 5), (dict(sts={"dk": S(0, -64, 64, 1)}), 5),
    (dict(sts={"dv": S(0, 0, 68, 1)}), 5), (dict(sts={"o": S(0, 0, 1 << 24, 1)}), 5),
    (dict(dq=P + 8), 5), (dict(do=P + 4), 5), (dict(lse=P + 2), 5), (dict(delta=P + 1), 5),
    (dict(scale=math.nan), 7),
    (dict(k=None), 1), (dict(dv=None), 1), (dict(dout_none=True), 1), (dict(lse=None), 1),
    (dict(delta=None), 1), (dict(dq=None), 1),
])
def test_bwd_validation_errors(kwargs, code):
    if kwargs.pop("dout_none", False):
        kwargs["do"] = None
    rc = call_bwd(**kwargs)
    assert rc == code, (kwargs, rc, fa.last_error())
    assert fa.last_error() != ""


def test_bwd_fp32_accepts_unaligned_strides():
    # fp32 rows need only 4-byte alignment: a seq stride of 65 passes, and
    # the call then stops at the NULL q
    rc = call_bwd(q=None, sts={"q": S(0, 0, 65, 1), "dq": S(0, 0, 65, 1)}, dtype=F32)
    assert rc == 1, fa.last_error()


def test_bwd_empty_problem_is_ok_without_pointers():
    nothing = dict(q=None, k=None, v=None, o=None, do=None, lse=None, delta=None, dq=None,
                   dk=None, dv=None)
    for kw in (dict(batch=0), dict(heads=0)):
        assert call_bwd(**nothing, **kw) == 0
        assert fa.last_error() == ""
    # without queries dk and dv are still written (zeros), so they are required
    assert call_bwd(**nothing, sq=0) == 1


def call_splitk(splits=2, ws=P, ws_bytes=1 << 30, dtype=BF16, **kw):
    args = dict(q=P, k=P, v=P, o=P, lse=None, batch=1, heads=2, sq=128, sk=128, d=64)
    args.update(kw)
    return fa.fa_fwd_splitk(args["q"], args["k"], args["v"], args["o"], args["lse"],
                            args["batch"], args["heads"], args["sq"], args["sk"], args["d"],
                            CONTIG, CONTIG, CONTIG, CONTIG, 0.125, 0, dtype, splits, ws, ws_bytes,
                            None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(splits=-1), 8), (dict(splits=17), 8), (dict(ws=None), 8), (dict(ws=P + 16), 8),
    (dict(ws_bytes=1000), 8), (dict(splits=2, dtype=F32), 3), (dict(splits=2, dtype=E5M2), 3),
    (dict(sk=0), 2),
    (dict(q=None), 1),
])
def test_splitk_validation_errors(kwargs, code):
    rc = call_splitk(**kwargs)
    assert rc == code, (kwargs, rc, fa.last_error())
    assert fa.last_error() != ""


def test_splitk_sizes_and_choice():
    assert fa.fa_fwd_splitk_workspace(1, 2, 128, 64, 1) == 0
    assert fa.fa_fwd_splitk_workspace(1, 2, 128, 64, 3) == 3 * 2 * 128 * 65 * 4
    assert fa.fa_fwd_splitk_workspace(0, 2, 128, 64, 3) == 0
    # a large grid needs no splitting; a few query tiles against many keys does;
    # where two splits would do, the unsplit kernel's two key groups per
    # workgroup do the same without partials (fp16, 16 heads, 1000 x 1537 keys)
    assert fa.fa_fwd_splitk_choose(1, 16, 32768, 32768, 128, 1) == 1
    assert fa.fa_fwd_splitk_choose(1, 12, 100, 4096, 64, 0) == 8
    assert fa.fa_fwd_splitk_choose(1, 16, 1000, 1537, 64, 0) == 1
    assert 1 <= fa.fa_fwd_splitk_choose(1, 1, 10, 100000, 64, 0) <= 16
    assert fa.fa_fwd_splitk_choose(0, 1, 10, 10, 64, 0) == 1
    # an empty problem needs no workspace
    assert call_splitk(batch=0, ws=None, q=None, k=None, v=None, o=None) == 0


def _contig(seq, heads, d=8):
    return S(heads * seq * d, seq * d, d, 1)


def test_fwd_rejects_dispatch_beyond_32bit_work_items():
    # 65536 heads x 128 tiles of 256 queries x 512 threads = 2^32 work-items
    st = _contig(32768, 65536)
    rc = fa.fa_fwd(P, P, P, P, None, 1, 65536, 32768, 32768, 8, st, st, st, st, 0.125, 0, BF16,
                   None)
    assert rc == 2, (rc, fa.last_error())
    assert "work-items" in fa.last_error()


def test_splitk_rejects_merge_beyond_32bit_work_items_before_launching():
    # 2^29 query rows: the split launch fits (2^31 work-items) but the merge
    # (8 threads per row) would need 2^32, so nothing may be enqueued
    st = _contig(32768, 16384)
    rc = fa.fa_fwd_splitk(P, P, P, P, None, 1, 16384, 32768, 32768, 8, st, st, st, st, 0.125, 0,
                          BF16, 2, P, 1 << 40, None)
    assert rc == 2, (rc, fa.last_error())
    assert "work-items" in fa.last_error()


def test_bwd_rejects_delta_launch_beyond_32bit_work_items():
    sq = _contig(32768, 16384)
    sk = _contig(128, 16384)
    rc = fa.fa_bwd(P, P, P, P, P, P, P, P, P, P, 1, 16384, 32768, 128, 8,
                   sq, sk, sk, sq, sq, sq, sk, sk, 0.125, 0, BF16, None)
    assert rc == 2, (rc, fa.last_error())
    assert "work-items" in fa.last_error()


def test_bwd_rejects_key_launch_beyond_32bit_work_items():
    # 2 heads of 2^31 - 512 keys: dK/dV needs 2 threads per key and head
    n = (1 << 31) - 512
    sq = _contig(128, 2)
    sk = _contig(n, 2)
    rc = fa.fa_bwd(P, P, P, P, P, P, P, P, P, P, 1, 2, 128, n, 8,
                   sq, sk, sk, sq, sq, sq, sk, sk, 0.125, 0, BF16, None)
    assert rc == 2, (rc, fa.last_error())
    assert "work-items" in fa.last_error()


def test_splitk_static_rejects_partials_beyond_its_array():
    # 8 splits x 16 heads x 4096 rows x 129 floats = 270 MB > 32 MiB: refused before any HIP call
    st = _contig(4096, 16, 128)
    rc = fa.fa_fwd_splitk_static(P, P, P, P, None, 1, 16, 4096, 4096, 128, st, st, st, st, 0.125, 0,
                                 BF16, 8, None)
    assert rc == 8, (rc, fa.last_error())
    assert "static scratch" in fa.last_error()
    need = fa.fa_fwd_splitk_workspace(1, 16, 4096, 128, 8)
    assert need > fa.SPLITK_STATIC_MAX_BYTES


@pytest.mark.parametrize("kwargs,code", [
    (dict(batch=-1), 2), (dict(sk=0), 2), (dict(dtype=F32), 3), (dict(splits=17), 8),
    (dict(q=None), 1), (dict(d=12), 4),
])
def test_splitk_static_validation_errors(kwargs, code):
    args = dict(q=P, k=P, v=P, o=P, batch=1, heads=2, sq=128, sk=128, d=64, dtype=BF16, splits=2)
    args.update(kwargs)
    rc = fa.fa_fwd_splitk_static(args["q"], args["k"], args["v"], args["o"], None, args["batch"],
                                 args["heads"], args["sq"], args["sk"], args["d"], CONTIG, CONTIG,
                                 CONTIG, CONTIG, 0.125, 0, args["dtype"], args["splits"], None)
    assert rc == code, (kwargs, rc, fa.last_error())


def test_splitk_static_empty_problem_is_ok_without_pointers():
    rc = fa.fa_fwd_splitk_static(None, None, None, None, None, 0, 2, 128, 128, 64, CONTIG, CONTIG,
                                 CONTIG, CONTIG, 0.125, 0, BF16, 2, None)
    assert rc == 0
