"""PMQA_VALIDATE=1: the library copies seq_lens, the block table, counters and
arrivals to the host before launching and returns PMQA_ERR_CONTENT, with
nothing written, when a device-content precondition is violated.

Each violating input below is also harmless if it were launched (lengths and
ids stay inside the buffers that exist), so a broken check shows as a wrong
status, never as a stray access."""
import numpy as np
import pytest
import torch

import paged_fp8_mqa_amd as pm
import workloads as W
from gpu_util import SENTINEL_F32_BITS, SENTINEL_I32, SelectBuffers, dev, sentinel_f32

pytestmark = pytest.mark.gpu

ERR_CONTENT = 8


@pytest.fixture
def validate(monkeypatch):
    monkeypatch.setenv("PMQA_VALIDATE", "1")
    yield


def _status(fn):
    try:
        fn()
    except pm.PmqaError as e:
        return e.status
    return 0


def test_validate_passes_good_inputs(validate):
    wl = W.small_random(81, [1000, 300], 2, 64, top_k=32, capacity=64)
    d = dev(wl)
    out = sentinel_f32((wl.rows, pm.padded_seq_len(wl.max_seq_len)))
    assert _status(lambda: pm.mqa_logits(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, out=out)) == 0
    torch.cuda.synchronize()
    assert not np.all(out.cpu().numpy().view(np.int32) == SENTINEL_F32_BITS)


def test_validate_rejects_long_seq_len_before_launch(validate):
    # max_seq_len 1000 (padded 1024 columns); a length of 1001 still writes
    # inside those columns and reads pages the table holds
    wl = W.small_random(82, [1001, 300], 1, 64, top_k=32, capacity=64, max_seq_len=1001)
    d = dev(wl)
    out = sentinel_f32((wl.rows, pm.padded_seq_len(1000)))
    st = _status(lambda: pm.mqa_logits(d["q"], d["kv"], d["w"], d["bt"], d["sl"], 1000, out=out))
    assert st == ERR_CONTENT
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy().view(np.int32) == SENTINEL_F32_BITS), "written despite the error"


def test_validate_rejects_narrow_table_and_bad_ids(validate):
    wl = W.small_random(83, [1000, 300], 1, 64, top_k=32, capacity=64)
    d = dev(wl)
    out = sentinel_f32((wl.rows, pm.padded_seq_len(wl.max_seq_len)))
    # a view one column narrower than request 0 needs (its row stride unchanged)
    narrow = d["bt"][:, : d["bt"].shape[1] - 1]
    st = _status(lambda: pm.mqa_logits(d["q"], d["kv"], d["w"], narrow, d["sl"], wl.max_seq_len, out=out))
    assert st == ERR_CONTENT
    # a pool view one block shorter than an id the table holds
    used = int(wl.block_tables[0, :16].max())
    short = d["kv"][:used]
    st = _status(lambda: pm.mqa_logits(d["q"], short, d["w"], d["bt"], d["sl"], wl.max_seq_len, out=out))
    assert st == ERR_CONTENT
    torch.cuda.synchronize()
    assert np.all(out.cpu().numpy().view(np.int32) == SENTINEL_F32_BITS), "written despite the error"


def test_validate_rejects_dirty_counters_and_arrivals(validate):
    wl = W.small_random(84, [1000, 300], 2, 64, top_k=32, capacity=64)
    d = dev(wl)
    thr = np.full(wl.rows, np.inf, np.float32)
    for which in ("counters", "arrivals"):
        sb = SelectBuffers(wl.rows, wl.batch, wl.top_k, wl.capacity, thr, max_context=wl.max_seq_len)
        getattr(sb, which).view(-1)[1] = 5
        st = _status(lambda: pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len,
                                                    **sb.kwargs()))
        assert st == ERR_CONTENT, which
        torch.cuda.synchronize()
        assert np.all(sb.cand.cpu().numpy() == SENTINEL_I32), f"slots written despite dirty {which}"
