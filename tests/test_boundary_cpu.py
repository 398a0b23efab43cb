"""The C ABI on the CPU: the library loads, exports every function the header
declares, and every host-checkable argument error maps to its documented
status without touching a device."""
import ctypes
import os
import re

import pytest

import paged_fp8_mqa_amd as pm

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pmqa.h")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pmqa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = pm.lib()
    names = _declared()
    assert len(names) >= 11
    for n in names:
        assert hasattr(lib, n), f"{n} declared in pmqa.h but not exported"
    assert set(names) == set(pm.SIGNATURES), "binding signatures out of sync with the header"


def test_workspace_bytes():
    lib = pm.lib()
    b2 = lib.pmqa_workspace_bytes(1, 2, 3, 8000)
    f2 = lib.pmqa_workspace_bytes(2, 2, 3, 8000)
    assert b2 > 0 and b2 % 8 == 0 and f2 <= WS
    # the fused select adds a score buffer of round_up(max_context, 64) floats per row
    assert f2 - b2 == 6 * 8000 * 4
    assert lib.pmqa_workspace_bytes(2, 2, 3, 8001) - b2 == 6 * 8064 * 4
    assert lib.pmqa_workspace_bytes(1, 2, 3, 1) == b2  # the select over a logits matrix keeps none
    assert lib.pmqa_workspace_bytes(1, 64, 1, 0) < lib.pmqa_workspace_bytes(1, 64, 2, 0)
    assert lib.pmqa_workspace_bytes(1, 2, 0, 10) == 0 and lib.pmqa_workspace_bytes(1, -1, 1, 10) == 0
    assert lib.pmqa_workspace_bytes(0, 2, 3, 10) == 0 and lib.pmqa_workspace_bytes(2, 2, 3, -1) == 0


def test_helpers():
    assert pm.padded_seq_len(8000) == 8192
    assert pm.padded_seq_len(0) == 0 and pm.padded_seq_len(256) == 256 and pm.padded_seq_len(257) == 512
    assert pm.min_block_table_width(8000, 32) == 250
    assert pm.min_block_table_width(0, 64) == 0 and pm.min_block_table_width(65, 64) == 2
    assert pm.lib().pmqa_padded_seq_len(-1) == -1 and pm.lib().pmqa_min_block_table_width(5, 0) == -1
    assert pm.lib().pmqa_version() >= 10000
    for s in range(9):
        assert pm.lib().pmqa_status_string(s).startswith(b"PMQA")
    assert pm.keys_per_cta("fused") > 0


A = 0x10000   # a fake 64 KiB-aligned "device" address: the checks never dereference it


def P(off=0):
    return ctypes.c_void_p(A + off)


def logits_args(**kw):
    a = dict(q=P(), kv=P(), w=P(), bt=P(), bts=250, btw=250, sl=P(), sls=1, B=2, nn=3, H=64, D=128, bs=32,
             nb=500, msl=8000, out=P(), outs=8192)
    a.update(kw)
    return [a["q"], a["kv"], a["w"], a["bt"], a["bts"], a["btw"], a["sl"], a["sls"], a["B"], a["nn"], a["H"],
            a["D"], a["bs"], a["nb"], a["msl"], a["out"], a["outs"]]


WS = 1 << 23


def select_args(**kw):
    a = dict(lg=P(), lgs=8192, sl=P(), sls=1, B=2, nn=3, mc=8000, thr=P(), cnt=P(), cand=P(), cap=512, k=512,
             arr=P(), rng=P(), topk=P(), ws=P(), wsb=WS)
    a.update(kw)
    return [a["lg"], a["lgs"], a["sl"], a["sls"], a["B"], a["nn"], a["mc"], a["thr"], a["cnt"], a["cand"],
            a["cap"], a["k"], a["arr"], a["rng"], a["topk"], a["ws"], a["wsb"]]


def fused_args(**kw):
    a = dict(q=P(), kv=P(), w=P(), bt=P(), bts=250, btw=250, sl=P(), sls=1, B=2, nn=3, H=64, D=128, bs=32,
             nb=500, mc=8000, thr=P(), cnt=P(), cand=P(), cap=512, k=512, arr=P(), rng=P(), topk=P(), ws=P(),
             wsb=WS)
    a.update(kw)
    return [a["q"], a["kv"], a["w"], a["bt"], a["bts"], a["btw"], a["sl"], a["sls"], a["B"], a["nn"], a["H"],
            a["D"], a["bs"], a["nb"], a["mc"], a["thr"], a["cnt"], a["cand"], a["cap"], a["k"], a["arr"],
            a["rng"], a["topk"], a["ws"], a["wsb"]]


OK, NULL, SHAPE, STRIDE, UNSUP, ALIGN, OVERFLOW = 0, 1, 2, 3, 4, 5, 6

LOGITS_CASES = [
    ({}, OK),
    ({"B": 0, "q": None, "out": None}, OK),
    ({"q": None}, NULL), ({"kv": None}, NULL), ({"w": None}, NULL), ({"bt": None}, NULL),
    ({"sl": None}, NULL), ({"out": None}, NULL),
    ({"H": 32}, UNSUP), ({"D": 64}, UNSUP), ({"nn": 0}, UNSUP), ({"nn": 5}, UNSUP), ({"bs": 16}, UNSUP),
    ({"bs": 256}, UNSUP),
    ({"B": -1}, SHAPE), ({"nb": 0}, SHAPE), ({"msl": -1}, SHAPE), ({"btw": 0}, SHAPE),
    ({"outs": 8000}, STRIDE), ({"bts": -1}, STRIDE), ({"sls": -2}, STRIDE),
    ({"kv": P(8)}, ALIGN), ({"q": P(4)}, ALIGN), ({"w": P(4)}, ALIGN), ({"out": P(2)}, ALIGN),
    ({"B": 40000, "nn": 4, "outs": 16384, "msl": 16384}, OVERFLOW),
]


@pytest.mark.parametrize("kw,want", LOGITS_CASES)
def test_check_logits_args(kw, want):
    assert pm.lib().pmqa_check_logits_args(*logits_args(**kw)) == want


F32, F16, BF16 = 0, 1, 2
TYPED_CASES = [
    ((F32, F32, F32), {}, OK), ((F16, F16, F16), {}, OK), ((F16, F32, F16), {"out": P(2)}, OK),
    ((F32, F16, F32), {"out": P(2)}, ALIGN), ((F16, F32, F32), {"out": P(1)}, ALIGN),
    ((BF16, F32, F32), {}, UNSUP), ((F32, BF16, F32), {}, UNSUP), ((F32, F32, BF16), {}, UNSUP),
    ((F32, F32, 7), {}, UNSUP), ((-1, F32, F32), {}, UNSUP),
    ((F16, F32, F32), {"outs": 8000}, STRIDE), ((F16, F16, F32), {"q": None}, NULL),
    ((BF16, F32, F32), {"B": 0}, UNSUP),  # the precisions are checked before the empty-batch shortcut
]


@pytest.mark.parametrize("dtypes,kw,want", TYPED_CASES)
def test_check_logits_typed_args(dtypes, kw, want):
    assert pm.lib().pmqa_check_logits_typed_args(*logits_args(**kw), *dtypes) == want


def fp4_args(qsf=P(), sfv=32, inter=0, out_dt=BF16, epi=F32, **kw):
    a = logits_args(**kw)
    # q, q_sf, kv, ... max_seq_len, sf_vec_size, interleaved, out, out_stride, output_dtype, epi_dtype
    return [a[0], qsf] + a[1:15] + [sfv, inter] + a[15:17] + [out_dt, epi]


FP4_CASES = [
    ({}, OK), ({"out_dt": F32}, OK), ({"out_dt": F16, "epi": BF16}, OK), ({"epi": F16, "out": P(2)}, OK),
    ({"sfv": 16}, UNSUP), ({"inter": 1}, UNSUP), ({"inter": 1, "bs": 128}, OK), ({"inter": 2, "bs": 128}, UNSUP),
    ({"out_dt": 3}, UNSUP), ({"epi": -1}, UNSUP), ({"qsf": None}, NULL), ({"qsf": P(2)}, ALIGN),
    ({"out_dt": F32, "out": P(2)}, ALIGN), ({"out": P(1)}, ALIGN), ({"H": 32}, UNSUP), ({"outs": 8000}, STRIDE),
    ({"B": 0, "qsf": None, "out": None}, OK),
]


@pytest.mark.parametrize("kw,want", FP4_CASES)
def test_check_fp4_logits_args(kw, want):
    assert pm.lib().pmqa_check_fp4_logits_args(*fp4_args(**kw)) == want


def test_typed_logits_rejects_before_launch():
    lib = pm.lib()
    assert lib.pmqa_mqa_logits_typed(*logits_args(), BF16, F32, F32, None) == UNSUP
    assert lib.pmqa_mqa_logits_typed(*logits_args(B=0), F16, F16, F16, None) == OK


SELECT_CASES = [
    ({}, OK),
    ({"arr": None, "rng": None, "topk": None, "ws": None, "wsb": 0}, OK),
    ({"ws": None, "wsb": 0}, NULL),
    ({"arr": None, "rng": None, "topk": None}, NULL),
    ({"wsb": 1000}, SHAPE),
    ({"ws": P(4)}, ALIGN),
    ({"topk": None}, OK),
    ({"lg": None}, NULL), ({"thr": None}, NULL), ({"cnt": None}, NULL), ({"cand": None}, NULL),
    ({"rng": None}, NULL), ({"arr": None, "ws": None}, NULL),
    ({"nn": 0}, UNSUP), ({"nn": 5}, UNSUP),
    ({"k": 0}, SHAPE), ({"cap": -1}, SHAPE), ({"cap": 100}, SHAPE), ({"mc": -1}, SHAPE), ({"B": -1}, SHAPE),
    ({"lgs": 7999}, STRIDE), ({"sls": -1}, STRIDE),
    ({"cnt": P(4)}, ALIGN), ({"cand": P(4)}, ALIGN), ({"thr": P(2)}, ALIGN),
    ({"k": 2 ** 30, "cap": 2 ** 30}, OVERFLOW),
    ({"B": 60000, "nn": 4, "lgs": 16384, "mc": 16384, "wsb": 1 << 40}, OVERFLOW),
]


@pytest.mark.parametrize("kw,want", SELECT_CASES)
def test_check_select_args(kw, want):
    assert pm.lib().pmqa_check_select_args(*select_args(**kw)) == want


FUSED_CASES = [
    ({}, OK),
    ({"q": None}, NULL), ({"thr": None}, NULL), ({"rng": None}, NULL),
    ({"arr": None, "rng": None, "topk": P(), "ws": None}, NULL), ({"ws": None}, NULL), ({"wsb": 100}, SHAPE),
    # enough for the select over a logits matrix, not for the fused score buffer
    ({"wsb": "select"}, SHAPE), ({"wsb": "select+", "mc": 100, "btw": 4}, OK),
    ({"H": 128}, UNSUP), ({"bs": 48}, UNSUP),
    ({"btw": 249}, SHAPE), ({"k": 0}, SHAPE), ({"cap": 10}, SHAPE),
    ({"kv": P(4)}, ALIGN), ({"cnt": P(4)}, ALIGN),
]


@pytest.mark.parametrize("kw,want", FUSED_CASES)
def test_check_fused_args(kw, want):
    kw = dict(kw)
    if isinstance(kw.get("wsb"), str):
        # the indexer_topk workspace for the same shape (plus room for the
        # 100-key score buffer with "select+")
        need = pm.lib().pmqa_workspace_bytes(1, 2, 3, 8000)
        kw["wsb"] = need + (6 * 128 * 4 if kw["wsb"] == "select+" else 0)
    assert pm.lib().pmqa_check_fused_args(*fused_args(**kw)) == want


def test_entry_points_reject_before_launch():
    """Invalid arguments return their status from the entry points too, before
    any device call (this container has no GPU)."""
    lib = pm.lib()
    assert lib.pmqa_mqa_logits(*logits_args(H=32), None) == UNSUP
    assert lib.pmqa_indexer_topk(*select_args(k=0), None) == SHAPE
    assert lib.pmqa_fused_logits_select(*fused_args(q=None), None) == NULL
    # a zero batch is a no-op that needs no device either
    assert lib.pmqa_fused_logits_select(*fused_args(B=0), None) == OK


def prefill_args(**kw):
    a = dict(q=P(), kv=P(), w=P(), bt=P(), bts=250, btw=250, nreq=2, treq=P(), re=P(), T=6, tr=4, H=64, D=128,
             bs=32, nb=500, mc=8000, thr=P(), cnt=P(), cand=P(), cap=512, k=512, arr=P(), rng=P(), topk=P(),
             ws=P(), wsb=1 << 24)
    a.update(kw)
    return [a["q"], a["kv"], a["w"], a["bt"], a["bts"], a["btw"], a["nreq"], a["treq"], a["re"], a["T"], a["tr"],
            a["H"], a["D"], a["bs"], a["nb"], a["mc"], a["thr"], a["cnt"], a["cand"], a["cap"], a["k"], a["arr"],
            a["rng"], a["topk"], a["ws"], a["wsb"]]


PREFILL_CASES = [
    ({}, OK),
    ({"T": 0, "q": None, "treq": None}, OK),
    ({"treq": None}, NULL), ({"re": None}, NULL), ({"q": None}, NULL), ({"rng": None}, NULL),
    ({"nreq": 0}, SHAPE), ({"tr": 5}, UNSUP), ({"tr": 0}, UNSUP), ({"btw": 249}, SHAPE), ({"T": -1}, SHAPE),
    ({"wsb": 100}, SHAPE), ({"treq": P(2)}, ALIGN), ({"re": P(2)}, ALIGN),
]


@pytest.mark.parametrize("kw,want", PREFILL_CASES)
def test_check_prefill_args(kw, want):
    assert pm.lib().pmqa_check_prefill_args(*prefill_args(**kw)) == want
    if want != OK:
        assert pm.lib().pmqa_prefill_select(*prefill_args(**kw), None) == want


def test_prefill_workspace_is_the_fused_layout():
    """The prefill select's workspace is the fused select's for num_tiles tiles
    of tile_rows rows: one byte short is rejected."""
    need = pm.workspace_bytes("fused", 6, 4, 8000)
    assert pm.lib().pmqa_check_prefill_args(*prefill_args(wsb=need)) == OK
    assert pm.lib().pmqa_check_prefill_args(*prefill_args(wsb=need - 1)) == SHAPE


def test_binding_fails_loudly_without_the_library(monkeypatch, tmp_path):
    """The binding has no fallback: with the library missing every entry point
    raises instead of computing anything."""
    monkeypatch.setattr(pm, "LIB_PATH", str(tmp_path / "missing" / "libpmqa.so"))
    monkeypatch.setattr(pm, "_lib", None)
    with pytest.raises(RuntimeError, match="not built"):
        pm.lib()
    with pytest.raises(RuntimeError, match="not built"):
        pm.padded_seq_len(8000)
