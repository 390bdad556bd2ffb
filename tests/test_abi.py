"""The C ABI without a GPU: exports, sizes and every host-side check.

No call here reaches a kernel launch: each call carries exactly one defect
that the host validation rejects before anything is enqueued (fake device
addresses are never dereferenced on the host).
"""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import sharding
from sequence_sharded_mla_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HDR = os.path.join(ROOT, "include", "mla_dcp.h")


@pytest.fixture(scope="module")
def lib():
    return _lib.load()


def header_functions():
    text = open(HDR).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return re.findall(r"^[a-z][\w \*]*?\b(mla_\w+)\s*\(", text, flags=re.M)


def test_every_declared_symbol_is_exported(lib):
    names = header_functions()
    assert len(names) >= 10
    assert set(names) == set(_lib.SIGNATURES)
    for n in names:
        assert hasattr(lib, n), n


def test_header_is_plain_c(tmp_path):
    """The header compiles as strict C99 and as C++ (no torch or HIP types)."""
    import shutil
    import subprocess
    src = tmp_path / "use.c"
    src.write_text('#include "mla_dcp.h"\nint main(void) { return (int)sizeof(mla_decode_desc) > 0 ? 0 : 1; }\n')
    for cc, std in (("gcc", "-std=c99"), ("g++", "-std=c++17")):
        if shutil.which(cc) is None:
            pytest.skip(f"{cc} not available")
        lang = ["-x", "c++"] if cc == "g++" else []
        res = subprocess.run([cc, std, "-Wall", "-Wextra", "-pedantic", "-Werror", *lang, "-I",
                              os.path.dirname(HDR), "-c", str(src), "-o", str(tmp_path / "use.o")],
                             capture_output=True, text=True)
        assert res.returncode == 0, res.stderr


def test_status_strings(lib):
    for code in range(8):
        s = lib.mla_status_string(code)
        assert s and s != b"unknown status"
    assert lib.mla_status_string(99) == b"unknown status"


def test_local_len_matches_oracle(lib):
    for N in (1, 2, 3, 8, 16):
        for L in (0, 1, 2, 7, 8, 9, 1000, 32768, 1048576):
            for s in range(N):
                assert lib.mla_shard_local_len(L, s, N) == int(sharding.local_len(L, s, N))
    assert lib.mla_shard_local_len(10, 3, 3) == -1
    assert lib.mla_shard_local_len(10, -1, 3) == -1
    assert lib.mla_shard_local_len(10, 0, 0) == -1
    assert lib.mla_shard_local_len(-1, 0, 1) == -1


def test_row_bytes(lib):
    assert lib.mla_kv_row_bytes(_lib.MLA_F32) == 2304
    assert lib.mla_kv_row_bytes(_lib.MLA_BF16) == 1152
    assert lib.mla_kv_row_bytes(_lib.MLA_FP8_DS) == 656
    assert lib.mla_kv_row_bytes(7) == -1


def good_desc(**kw):
    d = dict(batch=4, q_len=1, num_heads=64, kv_lora_rank=512, rope_dim=64, block_size=64,
             max_blocks=16, topk=0, q_dtype=_lib.MLA_BF16, kv_dtype=_lib.MLA_FP8_DS,
             out_dtype=_lib.MLA_BF16, softmax_scale=0.07, pool_blocks=100)
    d.update(kw)
    return _lib.MLADecodeDesc(**d)


def ws_size(lib, desc, shards=1):
    out = ctypes.c_int64(-1)
    st = lib.mla_decode_workspace_size(ctypes.byref(desc), shards, ctypes.byref(out))
    return st, out.value


@pytest.mark.parametrize("topk,shards,q_len", [(1, 1, 1), (100, 8, 2), (2048, 3, 1), (2500, 8, 2)])
def test_workspace_holds_the_bf16_topk_lists(lib, topk, shards, q_len):
    """A top-K step over a bf16 cache needs, beyond what the same step over an
    fp8 cache needs, each row's list of owned pool rows (int32, the top-K
    width rounded up to 32) and its count, each region 256-byte aligned."""
    def align(x):
        return (x + 255) // 256 * 256
    kw = dict(batch=5, q_len=q_len, topk=topk, max_blocks=64)
    st8, n8 = ws_size(lib, good_desc(kv_dtype=_lib.MLA_FP8_DS, **kw), shards)
    st16, n16 = ws_size(lib, good_desc(kv_dtype=_lib.MLA_BF16, **kw), shards)
    assert st8 == 0 and st16 == 0
    rows = shards * 5 * q_len
    stride = (topk + 31) // 32 * 32
    assert n16 - n8 == align(rows * stride * 4) + align(rows * 4)


@pytest.mark.parametrize("field,value,code", [
    ("batch", -1, _lib.MLA_ERR_SHAPE),
    ("q_len", 0, _lib.MLA_ERR_SHAPE),
    ("max_blocks", 0, _lib.MLA_ERR_SHAPE),
    ("topk", -1, _lib.MLA_ERR_SHAPE),
    ("topk", 70000, _lib.MLA_ERR_SHAPE),
    ("pool_blocks", 0, _lib.MLA_ERR_SHAPE),
    ("kv_lora_rank", 256, _lib.MLA_ERR_UNSUPPORTED),
    ("rope_dim", 32, _lib.MLA_ERR_UNSUPPORTED),
    ("block_size", 16, _lib.MLA_ERR_UNSUPPORTED),
    ("num_heads", 8, _lib.MLA_ERR_UNSUPPORTED),
    ("num_heads", 96, _lib.MLA_ERR_UNSUPPORTED),
    ("num_heads", 256, _lib.MLA_ERR_UNSUPPORTED),
    ("q_dtype", _lib.MLA_FP8_DS, _lib.MLA_ERR_UNSUPPORTED),
    ("q_dtype", _lib.MLA_F32, _lib.MLA_ERR_UNSUPPORTED),
    ("out_dtype", _lib.MLA_FP8_DS, _lib.MLA_ERR_UNSUPPORTED),
    ("softmax_scale", float("nan"), _lib.MLA_ERR_SHAPE),
    ("softmax_scale", float("inf"), _lib.MLA_ERR_SHAPE),
    ("softmax_scale", 0.0, _lib.MLA_ERR_SHAPE),
    ("softmax_scale", -0.1, _lib.MLA_ERR_SHAPE),
])
def test_workspace_size_validates_desc(lib, field, value, code):
    assert ws_size(lib, good_desc(**{field: value}))[0] == code


def test_workspace_size_values(lib):
    st, n = ws_size(lib, good_desc())
    assert st == 0 and n >= 256 and n % 256 == 0
    assert lib.mla_decode_workspace_size(None, 1, ctypes.byref(ctypes.c_int64())) == _lib.MLA_ERR_NULL
    assert lib.mla_decode_workspace_size(ctypes.byref(good_desc()), 1, None) == _lib.MLA_ERR_NULL
    assert ws_size(lib, good_desc(), 0)[0] == _lib.MLA_ERR_SHARD
    # a long single request is split into chunks, which need scratch
    st, n_long = ws_size(lib, good_desc(batch=1, max_blocks=4096))
    assert st == 0 and n_long > 256
    # f32 pair is accepted
    assert ws_size(lib, good_desc(q_dtype=_lib.MLA_F32, kv_dtype=_lib.MLA_F32,
                                  out_dtype=_lib.MLA_F32, num_heads=16))[0] == 0


FAKE = 1 << 20  # 16-byte aligned, never dereferenced


def call_shards(lib, desc, **kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, ctx=FAKE, topk=None, begin=0, count=8, n=8, o=FAKE,
             lse=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mla_decode_partial_shards(
        ctypes.byref(desc), v(a["q"]), v(a["kv"]), v(a["bt"]), v(a["ctx"]), v(a["topk"]),
        a["begin"], a["count"], a["n"], v(a["o"]), v(a["lse"]), v(a["ws"]), a["ws_bytes"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), _lib.MLA_ERR_NULL),
    (dict(kv=None), _lib.MLA_ERR_NULL),
    (dict(bt=None), _lib.MLA_ERR_NULL),
    (dict(ctx=None), _lib.MLA_ERR_NULL),
    (dict(o=None), _lib.MLA_ERR_NULL),
    (dict(lse=None), _lib.MLA_ERR_NULL),
    (dict(ws=None), _lib.MLA_ERR_NULL),
    (dict(topk=FAKE), _lib.MLA_ERR_SHAPE),
    (dict(begin=1), _lib.MLA_ERR_SHARD),
    (dict(begin=-1), _lib.MLA_ERR_SHARD),
    (dict(count=0), _lib.MLA_ERR_SHARD),
    (dict(n=0, count=1), _lib.MLA_ERR_SHARD),
    (dict(n=4097, count=1), _lib.MLA_ERR_SHARD),
    (dict(q=FAKE + 8), _lib.MLA_ERR_ALIGN),
    (dict(kv=FAKE + 4), _lib.MLA_ERR_ALIGN),
    (dict(o=FAKE + 2), _lib.MLA_ERR_ALIGN),
    (dict(ws=FAKE + 8), _lib.MLA_ERR_ALIGN),
    (dict(lse=FAKE + 2), _lib.MLA_ERR_ALIGN),
    (dict(ws_bytes=100), _lib.MLA_ERR_WORKSPACE),
])
def test_decode_shards_rejects(lib, kw, code):
    assert call_shards(lib, good_desc(), **kw) == code


def test_decode_sparse_needs_indices(lib):
    assert call_shards(lib, good_desc(topk=2048)) == _lib.MLA_ERR_NULL


def test_decode_desc_errors_come_first(lib):
    assert call_shards(lib, good_desc(num_heads=48)) == _lib.MLA_ERR_UNSUPPORTED
    assert call_shards(lib, good_desc(), q=None, n=0) == _lib.MLA_ERR_SHARD


def test_empty_batch_is_a_no_op(lib):
    assert call_shards(lib, good_desc(batch=0)) == 0


def call_varlen(lib, desc, n_q, qsl=FAKE, **kw):
    a = dict(q=FAKE, kv=FAKE, bt=FAKE, ctx=FAKE, topk=None, begin=0, count=8, n=8, o=FAKE,
             lse=FAKE, ws=FAKE, ws_bytes=1 << 30)
    a.update(kw)
    v = lambda x: None if x is None else ctypes.c_void_p(x)
    return lib.mla_decode_partial_shards_varlen(
        ctypes.byref(desc), v(a["q"]), v(a["kv"]), v(a["bt"]), v(a["ctx"]), v(qsl), n_q,
        v(a["topk"]), a["begin"], a["count"], a["n"], v(a["o"]), v(a["lse"]), v(a["ws"]),
        a["ws_bytes"], None)


def test_varlen_checks(lib):
    d = good_desc(q_len=3)                       # at most 4 * 3 query tokens
    assert call_varlen(lib, d, -1) == _lib.MLA_ERR_SHAPE
    assert call_varlen(lib, d, 13) == _lib.MLA_ERR_SHAPE
    assert call_varlen(lib, d, 5, qsl=None) == _lib.MLA_ERR_NULL
    assert call_varlen(lib, d, 5, qsl=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert call_varlen(lib, d, 5, q=None) == _lib.MLA_ERR_NULL
    assert call_varlen(lib, d, 5, begin=1) == _lib.MLA_ERR_SHARD
    assert call_varlen(lib, d, 5, ws_bytes=100) == _lib.MLA_ERR_WORKSPACE
    assert call_varlen(lib, d, 0) == 0           # no query tokens: nothing to do
    assert call_varlen(lib, good_desc(batch=0), 0, qsl=None) == 0
    assert lib.mla_decode_partial_shards_varlen(None, *([None] * 5), 0, *([None]), 0, 1, 1,
                                                None, None, None, 0, None) == _lib.MLA_ERR_NULL


def test_single_shard_entry_checks(lib):
    d = good_desc()
    v = ctypes.c_void_p
    args = lambda sid, n, q=FAKE: (ctypes.byref(d), v(q), v(FAKE), v(FAKE), v(FAKE), None, sid, n,
                                  v(FAKE), v(FAKE), v(FAKE), 1 << 30, None)
    assert lib.mla_decode_partial(*args(8, 8)) == _lib.MLA_ERR_SHARD
    assert lib.mla_decode_partial(*args(-1, 8)) == _lib.MLA_ERR_SHARD
    assert lib.mla_decode_partial(*args(0, 0)) == _lib.MLA_ERR_SHARD
    assert lib.mla_decode_partial(*args(3, 8, q=None)) == _lib.MLA_ERR_NULL


def test_merge_and_localize_checks(lib):
    v = ctypes.c_void_p
    m = lambda n=4, rows=10, dv=512, pd=_lib.MLA_BF16, o=FAKE, l=FAKE, od=_lib.MLA_BF16, out=FAKE: \
        lib.mla_lse_merge(n, rows, dv, pd, v(o), v(l), od, v(out), None, None)
    assert m(n=0) == _lib.MLA_ERR_SHAPE
    assert m(n=65) == _lib.MLA_ERR_SHAPE
    assert m(rows=-1) == _lib.MLA_ERR_SHAPE
    assert m(dv=576) == _lib.MLA_ERR_UNSUPPORTED
    assert m(pd=_lib.MLA_FP8_DS) == _lib.MLA_ERR_UNSUPPORTED
    assert m(od=_lib.MLA_FP8_DS) == _lib.MLA_ERR_UNSUPPORTED
    assert m(o=None) == _lib.MLA_ERR_NULL
    assert m(out=None) == _lib.MLA_ERR_NULL
    assert m(o=FAKE + 4) == _lib.MLA_ERR_ALIGN
    assert m(rows=0) == 0
    loc = lambda cnt=10, s=0, n=8, g=FAKE, o=FAKE: lib.mla_localize_indices(v(g), cnt, s, n, v(o), None)
    assert loc(cnt=-1) == _lib.MLA_ERR_SHAPE
    assert loc(s=8) == _lib.MLA_ERR_SHARD
    assert loc(n=0) == _lib.MLA_ERR_SHARD
    assert loc(g=None) == _lib.MLA_ERR_NULL
    assert loc(cnt=0) == 0
    code = ctypes.c_int32()
    assert lib.mla_get_device_error(None, ctypes.byref(code), None) == _lib.MLA_ERR_NULL
    assert lib.mla_clear_device_error(None, None) == _lib.MLA_ERR_NULL


def test_slot_mapping_checks(lib):
    v = ctypes.c_void_p

    def sm(n=10, B=2, mb=4, pool=100, begin=0, count=8, N=8, req=FAKE, pos=FAKE, bt=FAKE,
           out=FAKE, ws=None):
        return lib.mla_dcp_slot_mapping(v(req), v(pos), n, v(bt), B, mb, pool, begin, count, N,
                                        v(out), None if ws is None else v(ws), None)

    assert sm(n=-1) == _lib.MLA_ERR_SHAPE
    assert sm(n=1 << 31) == _lib.MLA_ERR_SHAPE
    assert sm(B=0) == _lib.MLA_ERR_SHAPE
    assert sm(mb=0) == _lib.MLA_ERR_SHAPE
    assert sm(pool=0) == _lib.MLA_ERR_SHAPE
    assert sm(N=0, count=1) == _lib.MLA_ERR_SHARD
    assert sm(begin=1) == _lib.MLA_ERR_SHARD
    assert sm(begin=-1, count=1) == _lib.MLA_ERR_SHARD
    assert sm(count=0) == _lib.MLA_ERR_SHARD
    assert sm(req=None) == _lib.MLA_ERR_NULL
    assert sm(pos=None) == _lib.MLA_ERR_NULL
    assert sm(bt=None) == _lib.MLA_ERR_NULL
    assert sm(out=None) == _lib.MLA_ERR_NULL
    assert sm(out=FAKE + 4) == _lib.MLA_ERR_ALIGN
    assert sm(pos=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert sm(ws=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert sm(n=0, req=None, pos=None, bt=None, out=None) == 0


def test_kv_write_checks(lib):
    v = ctypes.c_void_p

    def kw(src=FAKE, sd=_lib.MLA_BF16, n=10, slots=FAKE, kd=_lib.MLA_FP8_DS, pool=FAKE,
           blocks=100, ws=None):
        return lib.mla_kv_write(v(src), sd, n, v(slots), kd, v(pool), blocks,
                                None if ws is None else v(ws), None)

    assert kw(n=-1) == _lib.MLA_ERR_SHAPE
    assert kw(n=1 << 31) == _lib.MLA_ERR_SHAPE
    assert kw(blocks=0) == _lib.MLA_ERR_SHAPE
    assert kw(sd=_lib.MLA_FP8_DS) == _lib.MLA_ERR_UNSUPPORTED
    assert kw(kd=3) == _lib.MLA_ERR_UNSUPPORTED
    assert kw(src=None) == _lib.MLA_ERR_NULL
    assert kw(slots=None) == _lib.MLA_ERR_NULL
    assert kw(pool=None) == _lib.MLA_ERR_NULL
    assert kw(src=FAKE + 8) == _lib.MLA_ERR_ALIGN
    assert kw(pool=FAKE + 8) == _lib.MLA_ERR_ALIGN
    assert kw(slots=FAKE + 4) == _lib.MLA_ERR_ALIGN
    assert kw(ws=FAKE + 1) == _lib.MLA_ERR_ALIGN
    assert kw(n=0, src=None, slots=None, pool=None) == 0


def test_fused_write_checks(lib):
    v = ctypes.c_void_p

    def fw(src=FAKE, sd=_lib.MLA_BF16, req=FAKE, pos=FAKE, n=10, bt=FAKE, B=2, mb=4, begin=0,
           count=8, N=8, kd=_lib.MLA_FP8_DS, pool=FAKE, blocks=100, ws=None):
        return lib.mla_dcp_kv_write(v(src), sd, v(req), v(pos), n, v(bt), B, mb, begin, count, N, kd,
                                    v(pool), blocks, None if ws is None else v(ws), None)

    assert fw(n=-1) == _lib.MLA_ERR_SHAPE
    assert fw(blocks=0) == _lib.MLA_ERR_SHAPE
    assert fw(B=0) == _lib.MLA_ERR_SHAPE
    assert fw(mb=0) == _lib.MLA_ERR_SHAPE
    assert fw(sd=_lib.MLA_FP8_DS) == _lib.MLA_ERR_UNSUPPORTED
    assert fw(kd=5) == _lib.MLA_ERR_UNSUPPORTED
    assert fw(N=0, count=1) == _lib.MLA_ERR_SHARD
    assert fw(begin=2) == _lib.MLA_ERR_SHARD
    assert fw(count=0) == _lib.MLA_ERR_SHARD
    assert fw(src=None) == _lib.MLA_ERR_NULL
    assert fw(pool=None) == _lib.MLA_ERR_NULL
    assert fw(req=None) == _lib.MLA_ERR_NULL
    assert fw(pos=None) == _lib.MLA_ERR_NULL
    assert fw(bt=None) == _lib.MLA_ERR_NULL
    assert fw(src=FAKE + 8) == _lib.MLA_ERR_ALIGN
    assert fw(pos=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert fw(ws=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert fw(n=0, src=None, req=None, pos=None, bt=None, pool=None) == 0


def test_topk_checks(lib):
    v = ctypes.c_void_p

    def loc(sc=FAKE, stride=1000, ctx=FAKE, B=2, Tq=1, k=64, begin=0, count=8, N=8, ci=FAKE, cs=FAKE,
            ws=None):
        return lib.mla_topk_local(v(sc), stride, v(ctx), B, Tq, k, begin, count, N, v(ci), v(cs),
                                  None if ws is None else v(ws), None)

    assert loc(stride=0) == _lib.MLA_ERR_SHAPE
    # the longest row whose position bitmap fits in LDS beside the selection state
    assert loc(stride=393216 + 1) == _lib.MLA_ERR_SHAPE
    assert loc(stride=1 << 19) == _lib.MLA_ERR_SHAPE
    assert loc(k=0) == _lib.MLA_ERR_SHAPE
    assert loc(Tq=0) == _lib.MLA_ERR_SHAPE
    assert loc(B=-1) == _lib.MLA_ERR_SHAPE
    assert loc(begin=1) == _lib.MLA_ERR_SHARD
    assert loc(N=0, count=1) == _lib.MLA_ERR_SHARD
    assert loc(sc=None) == _lib.MLA_ERR_NULL
    assert loc(ctx=None) == _lib.MLA_ERR_NULL
    assert loc(ci=None) == _lib.MLA_ERR_NULL
    assert loc(cs=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert loc(ws=FAKE + 1) == _lib.MLA_ERR_ALIGN
    assert loc(B=0, sc=None) == 0

    def var(sc=FAKE, stride=1000, ctx=FAKE, qsl=FAKE, B=2, nq=3, k=64, begin=0, count=8, N=8, ci=FAKE,
            cs=FAKE, ws=None):
        return lib.mla_topk_local_varlen(v(sc), stride, v(ctx), None if qsl is None else v(qsl), B, nq, k,
                                         begin, count, N, v(ci), v(cs), None if ws is None else v(ws), None)

    assert var(nq=-1) == _lib.MLA_ERR_SHAPE
    assert var(B=-1) == _lib.MLA_ERR_SHAPE
    assert var(B=0, nq=1) == _lib.MLA_ERR_SHAPE
    assert var(stride=0) == _lib.MLA_ERR_SHAPE
    assert var(k=0) == _lib.MLA_ERR_SHAPE
    assert var(qsl=None) == _lib.MLA_ERR_NULL
    assert var(qsl=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert var(begin=1) == _lib.MLA_ERR_SHARD
    assert var(ci=None) == _lib.MLA_ERR_NULL
    assert var(nq=0, qsl=None, sc=None) == 0      # no query tokens: nothing to do
    assert var(B=0, nq=0, qsl=None) == 0

    def mer(ci=FAKE, cs=FAKE, n=8, rows=10, ck=2048, k=2048, out=FAKE):
        return lib.mla_topk_merge(v(ci), v(cs), n, rows, ck, k, v(out), None)

    assert mer(n=0) == _lib.MLA_ERR_SHAPE
    assert mer(rows=-1) == _lib.MLA_ERR_SHAPE
    assert mer(k=8193) == _lib.MLA_ERR_SHAPE
    assert mer(n=200) == _lib.MLA_ERR_SHAPE
    assert mer(ck=0) == _lib.MLA_ERR_SHAPE
    assert mer(out=None) == _lib.MLA_ERR_NULL
    assert mer(ci=FAKE + 2) == _lib.MLA_ERR_ALIGN
    assert mer(rows=0) == 0
