"""The C-ABI library without a GPU: it loads, exports every function the
header declares, rejects every bad argument before any HIP call, and plans
the prefill schedule the way the pages describe."""
import ctypes
import json
import os
import re

import pytest

import flash_attention_forward_fwd_amd as fa
from flash_attention_forward_fwd_amd import _lib

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa.h")
GOLDEN = os.path.join(ROOT, "tests", "golden")

OK, NULL, SHAPE, UNSUP, ALIGN, SCALE, WS, HIP, ALIAS = range(9)
FAKE = 0x10000000  # a 256-byte aligned address that is never dereferenced


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\s*\*?\s*(fa_[a-z_0-9]+)\s*\(",
                                 src, flags=re.M)))


def test_library_loads_and_exports_header_functions():
    lib = fa.lib()
    names = declared_functions()
    assert set(names) == {"fa_fwd", "fa_fwd_lse", "fa_fwd_varlen", "fa_fwd_plan", "fa_fwd_planned",
                          "fa_decode_workspace_bytes", "fa_decode", "fa_decode_noalloc", "fa_decode_paged",
                          "fa_decode_multi_workspace_bytes", "fa_decode_multi",
                          "fa_decode_paged_multi", "fa_bwd_workspace_bytes", "fa_bwd",
                          "fa_status_string"}
    for n in names:
        assert hasattr(lib, n), n
        assert n in _lib.SIGNATURES


def test_fwd_planned_checks_the_schedule_before_any_hip_call():
    lib = fa.lib()
    plan = _lib.FwdPlan()
    assert lib.fa_fwd_plan(1, 32, 8, 4096, 4096, 128, 1, ctypes.byref(plan)) == OK
    args = [FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, None, 1, 32, 8, 4096, 4096,
            128, 1, 0.1, 0]
    assert lib.fa_fwd_planned(*args, None, None) == NULL
    for field, value in (("persistent", 2), ("hkv_major", -1), ("xcd_map", 3)):
        bad = _lib.FwdPlan()
        ctypes.memmove(ctypes.byref(bad), ctypes.byref(plan), ctypes.sizeof(plan))
        setattr(bad, field, value)
        assert lib.fa_fwd_planned(*args, ctypes.byref(bad), None) == SHAPE, field
    # a key split: never with a persistent grid or another order, not
    # negative, and at most 256 parts (4096 keys / 128 per tile / 1 per part
    # x 16 blocks x 32 heads is far more)
    for fields in (dict(split_tiles=-1), dict(split_tiles=4, persistent=1),
                   dict(split_tiles=4, hkv_major=1), dict(split_tiles=1), dict(queue=2),
                   dict(queue=1), dict(split_tiles=40, queue=1)):
        bad = _lib.FwdPlan()
        for key, value in fields.items():
            setattr(bad, key, value)
        assert lib.fa_fwd_planned(*args, ctypes.byref(bad), None) == SHAPE, fields
    # the XCD dealing needs B * Hkv a multiple of 8
    odd = _lib.FwdPlan()
    odd.persistent, odd.hkv_major, odd.xcd_map = 1, 0, 1
    args_odd = list(args)
    args_odd[7] = 4  # Hkv = 4
    assert lib.fa_fwd_planned(*args_odd, ctypes.byref(odd), None) == SHAPE


def test_status_strings():
    lib = fa.lib()
    for code in range(9):
        assert lib.fa_status_string(code).decode().startswith(_lib.STATUS_NAMES[code])
    assert b"unknown" in lib.fa_status_string(99)


def fwd(**kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000, B=1, Hq=4, Hkv=2,
             Sq=128, Sk=128, D=128, causal=1, scale=0.1, dtype=0, stream=None)
    a.update(kw)
    return fa.lib().fa_fwd(a["q"], a["k"], a["v"], a["o"], a["B"], a["Hq"], a["Hkv"], a["Sq"],
                           a["Sk"], a["D"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(v=None), NULL), (dict(o=None), NULL),
    (dict(B=-1), SHAPE), (dict(Sq=-1), SHAPE), (dict(Sk=-5), SHAPE), (dict(Hq=0), SHAPE),
    (dict(Hkv=0), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(D=96), UNSUP), (dict(D=256), UNSUP),
    (dict(dtype=2), UNSUP), (dict(dtype=-1), UNSUP), (dict(scale=float("nan")), SCALE),
    (dict(scale=float("inf")), SCALE), (dict(q=FAKE + 8), ALIGN), (dict(o=FAKE + 0x3000002), ALIGN),
    (dict(o=FAKE), ALIAS), (dict(o=FAKE + 0x1000000 + 256), ALIAS),
    (dict(B=1 << 20, Hq=1 << 10, Hkv=1 << 10, Sq=1 << 20), SHAPE),
    (dict(Sk=1 << 23), SHAPE),
])
def test_fwd_rejects_bad_arguments(kw, code):
    assert fwd(**kw) == code


def test_fwd_empty_queries_need_no_pointers():
    assert fwd(Sq=0, q=None, o=None) == OK
    assert fwd(B=0, q=None, o=None, k=None, v=None) == OK


def test_fwd_lse_requires_lse_pointer():
    lib = fa.lib()
    st = lib.fa_fwd_lse(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, None, 1, 4, 2,
                        128, 128, 128, 1, 0.1, 0, None)
    assert st == NULL
    st = lib.fa_fwd_lse(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 4, 1,
                        4, 2, 128, 128, 128, 1, 0.1, 0, None)
    assert st == ALIGN
    st = lib.fa_fwd_lse(FAKE, FAKE + 0x1000000, FAKE + 0x2000000, FAKE + 0x3000000, FAKE + 16, 1,
                        4, 2, 128, 128, 128, 1, 0.1, 0, None)
    assert st == ALIAS


def varlen(**kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000, lse=None,
             cq=FAKE + 0x4000000, ck=FAKE + 0x4000100, B=2, Hq=4, Hkv=2, tq=300, tk=500, mq=200,
             mk=300, D=128, causal=1, scale=0.1, dtype=0, stream=None)
    a.update(kw)
    return fa.lib().fa_fwd_varlen(a["q"], a["k"], a["v"], a["o"], a["lse"], a["cq"], a["ck"],
                                  a["B"], a["Hq"], a["Hkv"], a["tq"], a["tk"], a["mq"], a["mk"],
                                  a["D"], a["causal"], a["scale"], a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(k=None), NULL), (dict(o=None), NULL), (dict(cq=None), NULL),
    (dict(ck=None), NULL), (dict(B=-1), SHAPE), (dict(tq=-1), SHAPE), (dict(tk=-1), SHAPE),
    (dict(mq=-1), SHAPE), (dict(mk=-2), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(D=80), UNSUP),
    (dict(dtype=5), UNSUP), (dict(scale=float("nan")), SCALE), (dict(q=FAKE + 8), ALIGN),
    (dict(cq=FAKE + 0x4000002), ALIGN), (dict(lse=FAKE + 0x5000004), ALIGN),
    (dict(o=FAKE), ALIAS), (dict(o=FAKE + 0x4000000 - 64), ALIAS),
    (dict(lse=FAKE + 0x3000000), ALIAS), (dict(mk=1 << 21, Hkv=4), SHAPE),
])
def test_varlen_rejects_bad_arguments(kw, code):
    assert varlen(**kw) == code


def test_varlen_empty_needs_no_pointers():
    assert varlen(B=0, cq=None, ck=None, q=None, o=None, tq=0) == OK
    assert varlen(tq=0, q=None, o=None) == OK


def dec(**kw):
    a = dict(q=FAKE, kc=FAKE + 0x1000000, vc=FAKE + 0x2000000, vl=FAKE + 0x3000000,
             cap=128, o=FAKE + 0x4000000, B=1, Hq=8, Hkv=2, D=128, causal=0, scale=0.1, dtype=0,
             ws=FAKE + 0x5000000, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = fa.decode_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["D"], a["cap"]) or 1
    return fa.lib().fa_decode(a["q"], a["kc"], a["vc"], a["vl"], a["cap"], a["o"], a["B"], a["Hq"],
                              a["Hkv"], a["D"], a["causal"], a["scale"], a["dtype"], a["ws"],
                              a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(kc=None), NULL), (dict(vc=None), NULL), (dict(vl=None), NULL),
    (dict(o=None), NULL), (dict(cap=0), SHAPE), (dict(B=-1), SHAPE), (dict(Hq=6, Hkv=4), SHAPE),
    (dict(D=32), UNSUP), (dict(dtype=3), UNSUP), (dict(scale=float("-inf")), SCALE),
    (dict(ws=None), WS), (dict(wsb=16), WS), (dict(ws=FAKE + 0x5000000 + 128), WS),
    (dict(kc=FAKE + 0x1000000 + 2), ALIGN), (dict(vl=FAKE + 0x3000000 + 2), ALIGN),
    (dict(o=FAKE + 0x1000000), ALIAS), (dict(o=FAKE + 0x5000000), ALIAS),
    (dict(cap=1 << 20, Hq=8, Hkv=8), SHAPE),
])
def test_decode_rejects_bad_arguments(kw, code):
    assert dec(**kw) == code


def dec_noalloc(**kw):
    a = dict(q=FAKE, kc=FAKE + 0x1000000, vc=FAKE + 0x2000000, vl=FAKE + 0x3000000,
             cap=128, o=FAKE + 0x4000000, B=1, Hq=8, Hkv=2, D=128, causal=0, scale=0.1, dtype=0,
             stream=None)
    a.update(kw)
    return fa.lib().fa_decode_noalloc(a["q"], a["kc"], a["vc"], a["vl"], a["cap"], a["o"], a["B"],
                                      a["Hq"], a["Hkv"], a["D"], a["causal"], a["scale"],
                                      a["dtype"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(kc=None), NULL), (dict(vc=None), NULL), (dict(vl=None), NULL),
    (dict(o=None), NULL), (dict(cap=0), SHAPE), (dict(B=-1), SHAPE), (dict(Hq=6, Hkv=4), SHAPE),
    (dict(D=32), UNSUP), (dict(dtype=3), UNSUP), (dict(scale=float("nan")), SCALE),
    (dict(kc=FAKE + 0x1000000 + 2), ALIGN), (dict(o=FAKE + 0x1000000), ALIAS),
    (dict(cap=1 << 20, Hq=8, Hkv=8), SHAPE),
])
def test_decode_noalloc_rejects_bad_arguments_before_any_hip_call(kw, code):
    # every check runs before the entry point's first HIP call (none can run
    # here: no GPU), so each bad argument gets its own status
    assert dec_noalloc(**kw) == code


def test_decode_noalloc_empty_batch_is_ok():
    assert dec_noalloc(B=0) == OK


def paged(**kw):
    a = dict(q=FAKE, kp=FAKE + 0x1000000, vp=FAKE + 0x2000000, pt=FAKE + 0x3000000,
             vl=FAKE + 0x3000100, P=64, pps=4, npages=16, o=FAKE + 0x4000000, B=2, Hq=8, Hkv=2,
             D=128, causal=0, scale=0.1, dtype=0, ws=FAKE + 0x5000000, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        cap = max(a["P"], 1) * max(a["pps"], 1)
        a["wsb"] = fa.decode_workspace_bytes(a["B"], a["Hq"], a["Hkv"], a["D"], cap) or 1
    return fa.lib().fa_decode_paged(a["q"], a["kp"], a["vp"], a["pt"], a["vl"], a["P"], a["pps"],
                                    a["npages"], a["o"], a["B"], a["Hq"], a["Hkv"], a["D"],
                                    a["causal"], a["scale"], a["dtype"], a["ws"], a["wsb"],
                                    a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(pt=None), NULL), (dict(kp=None), NULL), (dict(vl=None), NULL),
    (dict(P=16), SHAPE), (dict(P=48), SHAPE), (dict(P=0), SHAPE), (dict(pps=0), SHAPE),
    (dict(npages=0), SHAPE), (dict(P=1 << 16, pps=64), SHAPE), (dict(D=96), UNSUP),
    (dict(pt=FAKE + 0x3000002), ALIGN), (dict(vp=FAKE + 0x2000008), ALIGN),
    (dict(wsb=64), WS), (dict(o=FAKE + 0x3000000), ALIAS), (dict(o=FAKE + 0x1000000), ALIAS),
    (dict(scale=float("inf")), SCALE), (dict(Hq=6, Hkv=4), SHAPE),
])
def test_decode_paged_rejects_bad_arguments(kw, code):
    assert paged(**kw) == code


def test_decode_paged_empty_batch_is_ok():
    assert paged(B=0) == OK


def multi(**kw):
    a = dict(q=FAKE, kc=FAKE + 0x1000000, vc=FAKE + 0x2000000, vl=FAKE + 0x3000000, cap=4096,
             o=FAKE + 0x4000000, B=2, Sq=4, Hq=8, Hkv=2, D=128, causal=1, scale=0.1, dtype=0,
             ws=FAKE + 0x5000000, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = fa.lib().fa_decode_multi_workspace_bytes(
            a["B"], max(a["Sq"], 1), a["Hq"], a["Hkv"], a["D"], a["cap"]) or 1
    return fa.lib().fa_decode_multi(a["q"], a["kc"], a["vc"], a["vl"], a["cap"], a["o"], a["B"],
                                    a["Sq"], a["Hq"], a["Hkv"], a["D"], a["causal"], a["scale"],
                                    a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(Sq=0), SHAPE), (dict(Sq=33), SHAPE), (dict(q=None), NULL), (dict(cap=0), SHAPE),
    (dict(wsb=256), WS), (dict(o=FAKE + 0x5000000 - 1024), ALIAS),
    (dict(o=FAKE + 0x3000000), ALIAS), (dict(D=32), UNSUP),
])
def test_decode_multi_rejects_bad_arguments(kw, code):
    assert multi(**kw) == code


def test_decode_multi_workspace_grows_with_tokens():
    lib = fa.lib()
    one = lib.fa_decode_workspace_bytes(1, 8, 2, 128, 65536)
    assert lib.fa_decode_multi_workspace_bytes(1, 1, 8, 2, 128, 65536) == one
    four = lib.fa_decode_multi_workspace_bytes(1, 4, 8, 2, 128, 65536)
    assert four >= 3 * one  # records grow with the query tokens; the flags do not
    assert lib.fa_decode_multi_workspace_bytes(1, 0, 8, 2, 128, 65536) == 0
    assert lib.fa_decode_multi_workspace_bytes(1, 33, 8, 2, 128, 65536) == 0


def bwd(**kw):
    a = dict(q=FAKE, k=FAKE + 0x1000000, v=FAKE + 0x2000000, o=FAKE + 0x3000000,
             g=FAKE + 0x4000000, lse=FAKE + 0x5000000, dq=FAKE + 0x6000000, dk=FAKE + 0x7000000,
             dv=FAKE + 0x8000000, B=1, Hq=4, Hkv=2, Sq=128, Sk=128, D=128, causal=1, scale=0.1,
             dtype=0, ws=FAKE + 0x9000000, wsb=None, stream=None)
    a.update(kw)
    if a["wsb"] is None:
        a["wsb"] = fa.lib().fa_bwd_workspace_bytes(max(a["B"], 0), max(a["Hq"], 1),
                                                   max(a["Sq"], 0)) or 1
    return fa.lib().fa_bwd(a["q"], a["k"], a["v"], a["o"], a["g"], a["lse"], a["dq"], a["dk"],
                           a["dv"], a["B"], a["Hq"], a["Hkv"], a["Sq"], a["Sk"], a["D"],
                           a["causal"], a["scale"], a["dtype"], a["ws"], a["wsb"], a["stream"])


@pytest.mark.parametrize("kw,code", [
    (dict(q=None), NULL), (dict(lse=None), NULL), (dict(dk=None), NULL), (dict(g=None), NULL),
    (dict(B=-1), SHAPE), (dict(Hq=6, Hkv=4), SHAPE), (dict(D=96), UNSUP), (dict(dtype=7), UNSUP),
    (dict(scale=float("nan")), SCALE), (dict(dq=FAKE + 0x6000008), ALIGN),
    (dict(lse=FAKE + 0x5000002), ALIGN), (dict(ws=None), WS), (dict(wsb=8), WS),
    (dict(ws=FAKE + 0x9000010), WS), (dict(dq=FAKE), ALIAS), (dict(dk=FAKE + 0x6000000), ALIAS),
    (dict(dv=FAKE + 0x9000000), ALIAS), (dict(dq=FAKE + 0x5000000), ALIAS),
])
def test_bwd_rejects_bad_arguments(kw, code):
    assert bwd(**kw) == code


def test_bwd_empty_is_ok():
    assert bwd(B=0) == OK
    assert bwd(Sq=0, Sk=0) == OK


def test_decode_workspace_sizes():
    assert fa.decode_workspace_bytes(1, 8, 2, 128, 128) > 0
    big = fa.decode_workspace_bytes(1, 8, 2, 128, 65536)
    assert big > fa.decode_workspace_bytes(1, 8, 2, 128, 128)
    assert big % 256 == 0 and big < 8 << 20
    assert fa.decode_workspace_bytes(1, 8, 3, 128, 128) == 0
    assert fa.decode_workspace_bytes(1, 8, 2, 128, 0) == 0
    assert fa.decode_workspace_bytes(1, 8, 2, 80, 64) == 0


# ----------------------------------------------------------------------------
# the schedule, against the counts and rules printed on the prefill page
# ----------------------------------------------------------------------------
FACTS = json.load(open(os.path.join(GOLDEN, "schedule_facts.json")))


def test_mask_free_fraction_at_8192():
    f = FACTS["mask_free_fraction"]
    p = fa.fwd_plan(1, 128, 8, f["Sq"], f["Sk"], 128, True)
    assert p["block_m"] == f["query_block"]
    frac = 1 - p["masked_tiles"] / p["kv_tiles"]
    assert abs(frac - f["value"]) <= f["abs_tol"]


def test_work_items_and_orders():
    w = FACTS["work_items"]
    assert fa.fwd_plan(w["B"], w["Hq"], w["Hkv"], w["Sq"], w["Sq"], 128, True)["work_items"] == \
        w["value"]
    # the page's order rule holds for the static persistent schedule; plans
    # with the work queue (12+ items per workgroup) deal a query-block-major
    # list instead
    for c in FACTS["hkv_major_rule"]["cases"]:
        p = fa.fwd_plan(c["B"], c["Hq"], c["Hkv"], c["Sq"], c["Sq"], 128, True)
        if p["queue"]:
            assert p["work_items"] >= 12 * 256 and p["hkv_major"] == 0 and p["xcd_map"] == 0, c
        else:
            assert p["hkv_major"] == (c["order"] == "hkv_major"), c
    # XCD dealing: on for query-block-major persistent launches when the
    # B * Hkv units split over the 8 XCDs
    assert fa.fwd_plan(1, 128, 8, 8192, 8192, 128, True)["xcd_map"] == 0  # work queue
    assert fa.fwd_plan(4, 32, 8, 4096, 4096, 128, True)["xcd_map"] == 1
    assert fa.fwd_plan(4, 32, 8, 1000, 3000, 128, True)["xcd_map"] == 1
    assert fa.fwd_plan(1, 32, 4, 4096, 4096, 128, True)["xcd_map"] == 0   # 4 units
    assert fa.fwd_plan(1, 16, 16, 2048, 2048, 128, True)["xcd_map"] == 0  # not persistent
    for c in FACTS["persistent_auto"]["cases"]:
        p = fa.fwd_plan(c["B"], c["Hq"], c["Hq"], c["Sq"], c["Sq"], 128, True)
        assert p["persistent"] == int(c["persistent"]), c
        # the work queue for persistent grids of 12+ items per workgroup
        assert p["queue"] == int(c["persistent"] and p["work_items"] >= 12 * 256)
        if c["persistent"]:
            assert p["grid"] == 256 and p["split_tiles"] == 0
        else:  # one workgroup per item, or per part of an item when keys are split
            assert p["grid"] == (p["work_items"] if p["split_tiles"] == 0 else
                                 _split_parts(p, c["B"], c["Hq"], c["Sq"], c["Sq"], True,
                                              p["split_tiles"]))


def _block_tiles(p, Sq, Sk, causal):
    """KV tiles of every query block, from the mask by brute force."""
    BM, BN = p["block_m"], p["block_n"]
    out = []
    for q0 in range(0, Sq, BM):
        last = min(Sq, q0 + BM) - 1
        kv_end = min(max(last + 1 + Sk - Sq, 0), Sk) if causal else Sk
        out.append(-(-kv_end // BN))
    return out


def _split_parts(p, B, Hq, Sq, Sk, causal, T):
    return B * Hq * sum(max(1, -(-nt // T)) for nt in _block_tiles(p, Sq, Sk, causal))


def test_split_plan_brute_force():
    # under-filled launches (fewer items than the 256 CUs): the smallest
    # tiles-per-part T >= 2 whose parts fit 256 workgroups, taken when it cuts
    # the longest item by at least 2 tiles
    for (B, Hq, Sq, Sk, causal) in [(1, 16, 2048, 2048, True), (1, 16, 2048, 2048, False),
                                    (1, 128, 256, 256, True), (1, 2, 256, 256, True),
                                    (2, 8, 1000, 3000, True), (1, 4, 300, 9000, False),
                                    (1, 1, 8192, 8192, True), (1, 3, 700, 100, True),
                                    (1, 64, 64, 65536, True), (1, 32, 512, 512, False)]:
        p = fa.fwd_plan(B, Hq, Hq, Sq, Sk, 128, causal)
        if p["persistent"]:
            assert p["split_tiles"] == 0
            continue
        nts = _block_tiles(p, Sq, Sk, causal)
        max_nt = max(nts)
        T = next((t for t in range(2, max_nt + 1)
                  if _split_parts(p, B, Hq, Sq, Sk, causal, t) <= 256), None)
        if T is not None and T <= max_nt - 2:
            assert p["split_tiles"] == T, (B, Hq, Sq, Sk, causal)
            assert p["grid"] == _split_parts(p, B, Hq, Sq, Sk, causal, T) <= 256
        else:
            assert p["split_tiles"] == 0 and p["grid"] == p["work_items"], (B, Hq, Sq, Sk, causal)
    # the MHA 2048 shapes: 16 heads x 8 query blocks = 128 items
    assert fa.fwd_plan(1, 16, 16, 2048, 2048, 128, True)["split_tiles"] == 6
    assert fa.fwd_plan(1, 16, 16, 2048, 2048, 128, False)["split_tiles"] == 8
    assert fa.fwd_plan(1, 16, 16, 2048, 2048, 128, False)["grid"] == 256


def test_plan_tile_counts_brute_force():
    # count tiles and masked tiles by walking every (query block, tile) pair
    for (Sq, Sk, causal) in [(1000, 3000, True), (700, 300, True), (513, 129, False),
                             (4096, 4096, True), (1, 1, True), (300, 0, True)]:
        p = fa.fwd_plan(1, 1, 1, Sq, Sk, 128, causal)
        BM, BN = p["block_m"], p["block_n"]
        tiles = masked = 0
        for q0 in range(0, Sq, BM):
            rows = range(q0, min(Sq, q0 + BM))
            need = [j for j in range(Sk) if any((not causal) or j <= i + Sk - Sq for i in rows)]
            nt = (max(need) + 1 + BN - 1) // BN if need else 0
            for t in range(nt):
                keys = range(t * BN, t * BN + BN)
                full = all(j < Sk and ((not causal) or j <= q0 + Sk - Sq) for j in keys)
                masked += 0 if full else 1
            tiles += nt
        assert (p["kv_tiles"], p["masked_tiles"]) == (tiles, masked), (Sq, Sk, causal)


def test_plan_rejects():
    lib = fa.lib()
    assert lib.fa_fwd_plan(1, 4, 2, 10, 10, 128, 1, None) == NULL
    with pytest.raises(fa.FaError):
        fa.fwd_plan(1, 4, 3, 10, 10, 128, 1)
