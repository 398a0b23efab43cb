"""GPU parity of pmqa_mqa_logits against the float64 oracle."""
import math

import numpy as np
import pytest
import torch

import oracle
import workloads as W
from gpu_util import SENTINEL_F32_BITS, dev, run_logits
from report import LINES

pytestmark = pytest.mark.gpu


def _check_logits(wl, out, rows=None, cols=None):
    """Every visible column of the chosen rows within tau_r of the oracle; rows of
    empty requests and columns past round_up(seq_len, 64) untouched."""
    got = out.cpu().numpy()
    bits = got.view(np.int32)
    R = wl.rows
    rows = range(R) if rows is None else rows
    ref = oracle.paged_mqa_logits(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                                  wl.max_seq_len, rows=rows)
    tau = oracle.row_tolerance(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                               rows=rows)
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    worst = 0.0
    for r in rows:
        L = int(wl.seq_lens[r // wl.next_n])
        e = int(ends[r])
        if L == 0:
            assert np.all(bits[r] == SENTINEL_F32_BITS), f"row {r} of an empty request was written"
            continue
        written = int(math.ceil(L / 64) * 64)
        assert np.all(bits[r, written:] == SENTINEL_F32_BITS), f"row {r}: write past column {written}"
        if e == 0:
            continue
        err = np.abs(got[r, :e].astype(np.float64) - ref[r, :e])
        assert np.all(np.isfinite(got[r, :e])), f"row {r}: non-finite logits"
        m = float(err.max())
        assert m <= tau[r], f"row {r}: max err {m:.3g} > tau {tau[r]:.3g}"
        worst = max(worst, m / max(tau[r], 1e-30))
    return worst


def _tiny_ones(bs=64, nn=1, L=5):
    """All-ones q and k: every dot is 128, so logit = s_p * 128 * sum_h w."""
    g = torch.Generator().manual_seed(0)
    nb = math.ceil(L / bs) + 1
    vals = torch.full((nb, bs, 128), 0x38, dtype=torch.uint8)
    sc = (torch.arange(nb * bs, dtype=torch.float32).reshape(nb, bs) % 7 + 1) * 0.25
    kv = torch.cat([vals.reshape(nb, -1), sc.view(torch.uint8).reshape(nb, -1)], 1).numpy()
    q = np.full((1, nn, 64, 128), 0x38, np.uint8)
    w = (torch.rand(nn, 64, generator=g) - 0.3).numpy()
    bt = np.arange(nb, dtype=np.int32).reshape(1, nb)[:, :max(1, math.ceil(L / bs))]
    return W.Workload(name="ones", q=q, kv_fused=kv, weights=w, block_tables=np.ascontiguousarray(bt),
                      seq_lens=np.array([L], np.int32), max_seq_len=L, block_size=bs, next_n=nn, top_k=4,
                      capacity=8, threshold_recipe="", description="")


def test_all_ones_closed_form():
    wl = _tiny_ones(L=70)
    out, view = run_logits(wl, dev(wl))
    got = view.cpu().numpy()[0]
    s = np.frombuffer(wl.kv_fused[0, 64 * 128:].tobytes(), dtype="<f4").astype(np.float64)
    s = np.concatenate([s, np.frombuffer(wl.kv_fused[1, 64 * 128:].tobytes(), dtype="<f4")])
    want = s[:70] * 128.0 * wl.weights[0].astype(np.float64).sum()
    assert np.allclose(got[:70], want, rtol=1e-6, atol=1e-5)


@pytest.mark.parametrize("cfg", [1, 2])
def test_logits_small_configs(cfg):
    wl = W.make(cfg)
    out, view = run_logits(wl, dev(wl))
    assert tuple(view.shape) == (wl.rows, wl.max_seq_len)
    _check_logits(wl, out)


EDGE = [
    # (seed, seq_lens, next_n, block_size)
    (11, [1, 17, 64, 65, 200], 1, 32),
    (12, [0, 2, 3, 130, 1000], 3, 64),
    (13, [127, 128, 129, 0, 4096], 2, 128),
    (14, [5, 63, 64, 2049, 3], 4, 64),
    (15, [1, 2, 3, 4, 5, 6, 7, 300], 4, 32),
    (16, [0, 0, 0], 2, 64),
    (17, [2500, 1], 1, 128),
]


def test_logits_large_batch_grid():
    """More than 1024 requests: the batch x chunks grid instead of the located one."""
    rng = np.random.default_rng(5)
    seq = [int(x) for x in rng.integers(0, 300, size=1100)]
    wl = W.small_random(18, seq, 2, 32, top_k=16, capacity=32)
    out, _ = run_logits(wl, dev(wl))
    _check_logits(wl, out, rows=list(range(0, wl.rows, 7)) + [wl.rows - 1])


@pytest.mark.parametrize("seed,seq_lens,next_n,bs", EDGE)
def test_logits_edge_cases(seed, seq_lens, next_n, bs):
    wl = W.small_random(seed, seq_lens, next_n, bs, top_k=16, capacity=32)
    out, _ = run_logits(wl, dev(wl))
    _check_logits(wl, out)


def test_logits_strided_views():
    """Row-strided block table and seq_lens views (zero-copy, as the pages allow)
    and an out buffer wider than padded_seq_len."""
    import paged_fp8_mqa_amd as pm
    wl = W.small_random(21, [300, 77, 1024], 2, 64, top_k=16, capacity=32)
    d = dev(wl)
    bt_wide = torch.zeros(wl.batch * 3, wl.block_tables.shape[1], dtype=torch.int32, device="cuda")
    bt_wide[::3] = d["bt"]
    sl_wide = torch.zeros(wl.batch * 2, dtype=torch.int32, device="cuda")
    sl_wide[::2] = d["sl"]
    cols = pm.padded_seq_len(wl.max_seq_len) + 512
    out = torch.full((wl.rows, cols), SENTINEL_F32_BITS, dtype=torch.int32, device="cuda").view(torch.float32)
    pm.mqa_logits(d["q"], d["kv"], d["w"], bt_wide[::3], sl_wide[::2], wl.max_seq_len, out=out)
    torch.cuda.synchronize()
    _check_logits(wl, out)


@pytest.mark.parametrize("cfg", [3, 4, 5])
def test_logits_large_configs(cfg):
    """Every row and every visible column of the large workloads within tau_r of
    the float64 oracle; untouched columns and empty requests keep the sentinel."""
    wl = W.make(cfg)
    out, _ = run_logits(wl, dev(wl))
    worst = _check_logits(wl, out)
    LINES.append(f"{wl.name}: worst |logit err| / tau_r over all rows = {worst:.3g}")
