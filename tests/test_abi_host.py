"""The C ABI on the host: the library loads, exports what include/amla.h declares, and its
host-only functions and argument checks behave as documented.  No device work is launched
here (every call either is host-only or is rejected before any launch)."""
import ctypes
import os
import re

import pytest

from absorbed_mla_split_amd import binding as b

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "amla.h")
GOLDEN = os.path.join(ROOT, "tests", "golden", "fold_examples.txt")


def golden(kind):
    out = []
    for line in open(GOLDEN):
        line = line.strip()
        if line and not line.startswith("#") and line.split()[0] == kind:
            out.append([int(v) for v in line.split()[1:]])
    return out


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(amla_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol():
    lib = b.load()
    names = declared_functions()
    assert set(names) == set(b.EXPORTS), names
    for name in names:
        assert hasattr(lib, name), name


def test_header_constants_match_binding():
    text = open(HEADER).read()
    consts = dict(re.findall(r"#define (AMLA_\w+) \(?(-?\d+)\)?", text))
    assert int(consts["AMLA_PAGE"]) == b.PAGE and int(consts["AMLA_KDIM"]) == b.KDIM
    assert int(consts["AMLA_VDIM"]) == b.VDIM and int(consts["AMLA_MAX_ROWS"]) == b.MAX_ROWS
    assert int(consts["AMLA_UVDIM"]) == b.UVDIM
    assert int(consts["AMLA_MAX_SOURCES"]) == b.MAX_SOURCES
    assert int(consts["AMLA_MAX_REQS"]) == b.MAX_REQS
    assert int(consts["AMLA_MAX_SPLIT_COST"]) == b.MAX_SPLIT_COST
    assert int(consts["AMLA_SPLIT_COST_ONE_TILE"]) == b.SPLIT_COST_ONE_TILE
    assert int(consts["AMLA_SPLIT_COST_MULTI_TILE"]) == b.SPLIT_COST_MULTI_TILE
    assert b.make_params(448, 128, 256).split_cost_pages == b.SPLIT_COST_MULTI_TILE
    assert b.make_params(448, 64, 256).split_cost_pages == b.SPLIT_COST_MULTI_TILE
    assert b.make_params(56, 64, 256).split_cost_pages == b.SPLIT_COST_ONE_TILE
    assert b.make_params(32, 32, 256).split_cost_pages == b.SPLIT_COST_ONE_TILE
    assert int(consts["AMLA_ERR_WORKSPACE"]) == b.ERR_WORKSPACE
    assert int(consts["AMLA_DEV_BAD_PAGE"]) == b.DEV_BAD_PAGE
    assert int(consts["AMLA_DEV_BAD_POSITION"]) == b.DEV_BAD_POSITION
    assert int(consts["AMLA_PLAN_FIXED"]) == b.PLAN_FIXED


def test_fold_plan_pages_examples():
    for k, heads, need_lse, cap, expect in golden("fold_plan"):
        kk, f = b.fold_plan(False, 2, 2 * k, 2 * k, 2, k, heads, need_lse, cap)
        assert kk == k and f == expect
    for causal, reqs, rows, tokens, bt_rows, mql, expect in golden("foldable"):
        kk, f = b.fold_plan(causal, reqs, rows, tokens, bt_rows, mql, 8, True, 128)
        assert kk == expect and (f == 0) == (expect == 0)


def test_fold_plan_matches_oracle_rules():
    import oracle

    for causal in (0, 1):
        for reqs in (1, 2, 3):
            for rows in (2, 4, 6, 8, 12):
                for mql in (1, 2, 4, 6):
                    for heads in (8, 64):
                        for need_lse in (0, 1):
                            k = oracle.foldable(bool(causal), reqs, rows, rows, reqs, mql)
                            kk, f = b.fold_plan(causal, reqs, rows, rows, reqs, mql, heads,
                                                need_lse, 128)
                            assert kk == k
                            if k:
                                assert f == oracle.fold_plan(k, heads, bool(need_lse), 128)


def test_reducer_bands_pages_example_and_formula():
    for rows, units, expect in golden("reducer_bands"):
        assert b.reducer_bands(rows, units) == expect
    # the rule returns 2 when the rows fill at most half the units, and just above each
    # whole wave (the docstring and the formula differ there; the formula is followed)
    assert b.reducer_bands(74, 148) == 2
    assert b.reducer_bands(75, 148) == 1
    assert b.reducer_bands(148, 148) == 1
    assert b.reducer_bands(200, 148) == 2


def test_bmm_scales_composition():
    b1, b2 = b.bmm_scales(0.125, 0.5, 0.25)
    assert b1 == pytest.approx(0.125 * 0.5 * 0.25) and b2 == 0.25


def test_decode_config():
    assert b.decode_config(256, 32) == (256, 32)
    assert b.decode_config(256, 56) == (256, 64)
    assert b.decode_config(256, 256) == (256, 128)
    assert b.decode_config(256, 448) == (256, 64)        # 7 x 64 rows, no padding
    assert b.decode_config(256, 1024) == (256, 128)
    assert b.decode_config(256, 129) == (256, 64)        # 3 x 64 pads 63 rows, 2 x 128 127
    assert b.decode_config(256, 200) == (256, 128)       # 56 padding rows either way
    with pytest.raises(b.AmlaError):
        b.decode_config(256, 0)
    with pytest.raises(b.AmlaError):
        b.decode_config(0, 32)


def test_workspace_bytes_formula():
    # header 256 B + FP32 partials (R+2W)*M*512*4 + FP32 LSE (R+2W)*M*4 rounded to 256 B
    R, M, W = 64, 32, 256
    S = R + 2 * W
    lse = (S * M * 4 + 255) // 256 * 256
    assert b.workspace_bytes(R, M, W) == 256 + S * M * 512 * 4 + lse
    assert b.workspace_bytes(-1, 32, 256) == 0
    assert b.workspace_bytes(4, 0, 256) == 0
    assert b.workspace_bytes(b.MAX_REQS + 1, 32, 256) == 0


def _call_plan(lib, lengths=1, reqs=2, cols=4, params=None, counts=1, offsets=1, work=1,
               list_len=1024, ws=1, ws_bytes=1 << 30):
    p = params if params is not None else b.make_params(32, 32, 256)
    vp = ctypes.c_void_p
    return lib.amla_plan_splits(vp(lengths), reqs, cols, ctypes.byref(p), vp(counts), vp(offsets),
                                vp(work), list_len, vp(ws), ws_bytes, None)


def test_plan_argument_errors():
    lib = b.load()
    assert _call_plan(lib, lengths=0) == b.ERR_INVALID
    assert _call_plan(lib, offsets=0) == b.ERR_INVALID
    assert _call_plan(lib, ws=0) == b.ERR_INVALID
    assert _call_plan(lib, reqs=-1) == b.ERR_INVALID
    assert _call_plan(lib, reqs=b.MAX_REQS + 1) == b.ERR_INVALID
    assert _call_plan(lib, params=b.make_params(32, 48, 256)) == b.ERR_INVALID     # mtile
    assert _call_plan(lib, params=b.make_params(0, 32, 256)) == b.ERR_INVALID
    assert _call_plan(lib, params=b.make_params(b.MAX_ROWS + 1, 128, 256)) == b.ERR_INVALID
    assert _call_plan(lib, params=b.make_params(32, 32, 256, mode=7)) == b.ERR_INVALID
    assert _call_plan(lib, params=b.make_params(32, 32, 256, max_splits=0)) == b.ERR_INVALID
    assert _call_plan(lib, params=b.make_params(32, 32, 256, split_cost_pages=-1)) == b.ERR_INVALID
    assert _call_plan(lib, params=b.make_params(32, 32, 256,
                                                split_cost_pages=b.MAX_SPLIT_COST + 1)) == b.ERR_INVALID
    assert _call_plan(lib, ws_bytes=100) == b.ERR_WORKSPACE
    assert _call_plan(lib, list_len=2 * (2 + 2 * 256) - 1) == b.ERR_LIST


def test_decode_and_combine_argument_errors():
    lib = b.load()
    p = b.make_params(32, 32, 256)
    vp = ctypes.c_void_p
    good = dict(q=1, kv=1, pool=16, bt=1, stride=4, lengths=1, reqs=2, b1=1.0, b2=1.0, counts=1,
                offsets=1, work=1, list_len=1024, ws=1, ws_bytes=1 << 30)

    def dec(**kw):
        a = dict(good, **kw)
        return lib.amla_folded_decode(vp(a["q"]), vp(a["kv"]), a["pool"], vp(a["bt"]), a["stride"],
                                      vp(a["lengths"]), a["reqs"], ctypes.byref(p), a["b1"], a["b2"],
                                      vp(a["counts"]), vp(a["offsets"]), vp(a["work"]),
                                      a["list_len"], vp(a["ws"]), a["ws_bytes"], None)

    for bad in (dict(q=0), dict(kv=0), dict(bt=0), dict(lengths=0), dict(counts=0),
                dict(offsets=0), dict(work=0), dict(ws=0), dict(pool=0), dict(stride=0),
                dict(reqs=-1), dict(b1=float("nan")), dict(b2=float("inf")), dict(b1=0.0), dict(b1=-1.0)):
        assert dec(**bad) == b.ERR_INVALID, bad
    assert dec(ws_bytes=10) == b.ERR_WORKSPACE
    assert dec(list_len=10) == b.ERR_LIST
    assert dec(reqs=0) == b.OK            # nothing to do, nothing launched

    def comb(ws=1, ws_bytes=1 << 30, counts=1, offsets=1, reqs=2, cus=256, out=1, lse=1):
        return lib.amla_combine(vp(ws), ws_bytes, vp(counts), vp(offsets), reqs, ctypes.byref(p), cus,
                                vp(out), vp(lse), None)

    for bad in (dict(ws=0), dict(counts=0), dict(offsets=0), dict(out=0), dict(lse=0),
                dict(cus=0), dict(reqs=-1)):
        assert comb(**bad) == b.ERR_INVALID, bad
    assert comb(ws_bytes=10) == b.ERR_WORKSPACE
    assert comb(reqs=0) == b.OK


def test_noalloc_argument_errors():
    # rejected on the host before the scratch is looked up or anything is launched
    lib = b.load()
    vp = ctypes.c_void_p
    good = dict(q=1, kv=1, pool=16, bt=1, stride=4, lengths=1, reqs=2, b1=1.0, b2=1.0, cus=256,
                out=1, lse=1, M=32, W=256)

    def call(**kw):
        a = dict(good, **kw)
        p = b.make_params(a["M"], 32 if a["M"] <= 32 else 128, a["W"])
        return lib.amla_folded_decode_noalloc(vp(a["q"]), vp(a["kv"]), a["pool"], vp(a["bt"]),
                                              a["stride"], vp(a["lengths"]), a["reqs"],
                                              ctypes.byref(p), a["b1"], a["b2"], a["cus"],
                                              vp(a["out"]), vp(a["lse"]), None, None)

    for bad in (dict(q=0), dict(kv=0), dict(bt=0), dict(lengths=0), dict(out=0), dict(lse=0),
                dict(pool=0), dict(stride=0), dict(cus=0), dict(reqs=-1), dict(reqs=b.MAX_REQS + 1),
                dict(b1=float("nan")), dict(b1=0.0), dict(b2=float("inf")), dict(M=0),
                dict(M=b.MAX_ROWS + 1)):
        assert call(**bad) == b.ERR_INVALID, bad
    # past the static scratch: 4096 requests of 1024 rows need far more than 64 MiB
    assert call(reqs=b.MAX_REQS, M=b.MAX_ROWS) == b.ERR_WORKSPACE
    assert call(reqs=64, M=256) == b.ERR_WORKSPACE


def test_combine_uv_argument_errors():
    lib = b.load()
    p = b.make_params(32, 32, 256)
    vp = ctypes.c_void_p

    def uv(ws=256, ws_bytes=1 << 30, counts=256, offsets=256, reqs=2, heads=8, w=256, ao=256,
           out=0, lse=0, params=p):
        return lib.amla_combine_uv(vp(ws), ws_bytes, vp(counts), vp(offsets), reqs,
                                   ctypes.byref(params), heads, vp(w), vp(ao), vp(out), vp(lse),
                                   None)

    for bad in (dict(ws=0), dict(counts=0), dict(offsets=0), dict(w=0), dict(ao=0), dict(reqs=-1),
                dict(heads=0), dict(heads=3), dict(heads=64), dict(w=264), dict(ao=260),
                dict(out=258), dict(params=b.make_params(32, 48, 256))):
        assert uv(**bad) == b.ERR_INVALID, bad
    assert uv(ws_bytes=10) == b.ERR_WORKSPACE
    assert uv(reqs=0) == b.OK              # nothing to do, nothing launched
    assert uv(reqs=0, heads=32) == b.OK


def test_dcp_argument_errors():
    lib = b.load()
    p = b.make_params(32, 32, 256)
    vp = ctypes.c_void_p

    def dec(dcp, totals=256, reqs=2, params=p):
        return lib.amla_folded_decode_dcp(vp(256), vp(256), 16, vp(256), 4, vp(256), reqs,
                                          ctypes.byref(params), 1.0, 1.0, vp(256), vp(256),
                                          vp(256), 1024, vp(256), 1 << 30,
                                          ctypes.byref(dcp) if dcp is not None else None,
                                          vp(totals), None)

    ok = dict(heads=8, causal=1, world=2, rank=1, interleave=64)
    for bad in (dict(heads=0), dict(heads=3), dict(world=0), dict(rank=2), dict(rank=-1),
                dict(interleave=0), dict(causal=2), dict(world=1 << 16, interleave=1 << 15)):
        assert dec(b.DcpParams(**dict(ok, **bad))) == b.ERR_INVALID, bad
    assert dec(None) == b.ERR_INVALID
    assert dec(b.DcpParams(**ok), totals=0) == b.ERR_INVALID          # causal needs totals
    assert dec(b.DcpParams(**ok), reqs=0) == b.OK
    assert dec(b.DcpParams(**dict(ok, causal=0)), totals=0, reqs=0) == b.OK

    def merge(n_src=2, rows=256, lse=256, n=4, out=256, lo=256):
        return lib.amla_merge_sources(n_src, vp(rows), vp(lse), n, vp(out), vp(lo), None)

    for bad in (dict(n_src=0), dict(n_src=b.MAX_SOURCES + 1), dict(rows=0), dict(lse=0),
                dict(out=0), dict(lo=0), dict(rows=264), dict(out=248), dict(n=-1)):
        assert merge(**bad) == b.ERR_INVALID, bad
    assert merge(n=0) == b.OK


def test_build_query_cache_argument_errors():
    lib = b.load()
    vp = ctypes.c_void_p

    def call(q=256, w=256, kv=256, pe=256, pos=256, cs=256, max_pos=16, slots=256, n=4, heads=8,
             neox=0, qs=1.0, ks=1.0, qo=256, cache=256, pool=4):
        return lib.amla_build_query_cache(vp(q), vp(w), vp(kv), vp(pe), vp(pos), vp(cs), max_pos,
                                          vp(slots), n, heads, neox, qs, ks, vp(qo), vp(cache),
                                          pool, None, None)

    for bad in (dict(q=0), dict(w=0), dict(kv=0), dict(pe=0), dict(pos=0), dict(cs=0),
                dict(slots=0), dict(qo=0), dict(cache=0), dict(n=-1), dict(heads=0),
                dict(max_pos=0), dict(neox=2), dict(qs=0.0), dict(ks=float("nan")),
                dict(q=264), dict(w=260), dict(kv=258), dict(qo=257), dict(cache=260),
                dict(pool=-1)):
        assert call(**bad) == b.ERR_INVALID, bad
    assert call(n=0) == b.OK


def test_status_strings():
    for code in (b.OK, b.ERR_INVALID, b.ERR_WORKSPACE, b.ERR_LIST, b.ERR_HIP, b.DEV_BAD_LENGTH,
                 b.DEV_BAD_PAGE, b.DEV_BAD_ITEM, b.DEV_BAD_POSITION):
        assert b.status_string(code) and b.status_string(code) != "unknown status"
    assert b.status_string(-99) == "unknown status"
