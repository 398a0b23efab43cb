"""GPU parity of pmqa_fp4_mqa_logits (MXFP4 pools: E2M1 values, UE8M0 scales
per 32 elements; page "flashinfer.attn_scores", fp4_paged_mqa_logits) against
the float64 oracle of oracle/fp4.py."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_mqa_amd as pm
import workloads as W
from oracle.fp4 import fp4_paged_mqa_logits
from report import LINES

pytestmark = pytest.mark.gpu

F32, F16, BF16 = torch.float32, torch.float16, torch.bfloat16
NAME = {F32: "f32", F16: "f16", BF16: "bf16"}
SENT = {F32: (torch.int32, 0x7FC00BAD), F16: (torch.int16, 0x7E5A), BF16: (torch.int16, 0x7FDA)}
WORST = {}


class _WorstLine:
    def __str__(self):
        return "MXFP4 logits, worst |err| / tol per (output, epi): " + ", ".join(
            f"{'/'.join(k)} {v:.3g}" for k, v in sorted(WORST.items()))


def _dev(wl):
    return {"q": torch.from_numpy(wl.q).cuda(), "qsf": torch.from_numpy(wl.q_sf).cuda(),
            "kv": torch.from_numpy(wl.kv_fused).cuda().view(wl.num_blocks, wl.block_size, 1, 68),
            "w": torch.from_numpy(wl.weights).cuda(), "bt": torch.from_numpy(wl.block_tables).cuda(),
            "sl": torch.from_numpy(wl.seq_lens).cuda()}


def _run(wl, d, out_dtype, epi):
    it, sv = SENT[out_dtype]
    out = torch.empty(wl.rows, pm.padded_seq_len(wl.max_seq_len), dtype=out_dtype, device="cuda")
    out.view(it).fill_(sv)
    pm.fp4_mqa_logits(d["q"], d["qsf"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, out=out,
                      output_dtype=out_dtype, epi_dtype=epi, is_kv_sf_interleaved=wl.interleaved)
    torch.cuda.synchronize()
    return out


def _check(wl, out, out_dtype, epi, exact=False):
    ref = fp4_paged_mqa_logits(wl.q, wl.q_sf, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens,
                               wl.block_size, wl.max_seq_len, output_dtype=NAME[out_dtype], epi_dtype=NAME[epi],
                               interleaved=wl.interleaved)
    it, sv = SENT[out_dtype]
    raw = out.cpu().view(it).numpy()
    sent = np.array(sv).astype(raw.dtype)
    got = out.float().cpu().numpy().astype(np.float64)
    ends = wl.row_ends()
    worst = 0.0
    for r in range(wl.rows):
        L = int(wl.seq_lens[r // wl.next_n])
        if L == 0:
            assert np.all(raw[r] == sent), f"row {r} of an empty request was written"
            continue
        written = int(math.ceil(L / 64) * 64)
        assert np.all(raw[r, written:] == sent), f"row {r}: write past column {written}"
        e = int(ends[r])
        if e == 0:
            continue
        v, t, g = ref["value"][r, :e], ref["tol"][r, :e], got[r, :e]
        must, may = ref["must_inf"][r, :e], ref["may_inf"][r, :e]
        assert np.all(np.isinf(g[must]) & (np.sign(g[must]) == np.sign(v[must])))
        ok = ~may
        assert np.all(np.isfinite(g[ok])), f"row {r}: non-finite logits"
        if exact:
            assert np.array_equal(g[ok], v[ok]), f"row {r}: not exact"
        err = np.abs(g[ok] - v[ok])
        assert np.all(err <= t[ok]), f"row {r}: max err/tol {np.max(err / np.maximum(t[ok], 1e-300)):.3g}"
        if ok.any():
            worst = max(worst, float(np.max(err / np.maximum(t[ok], 1e-300))))
    return worst


MODES = [(BF16, F32), (F32, F32), (F16, F32), (F32, F16), (BF16, BF16), (F16, F16), (F32, BF16)]
CASES = [(1, [300, 0, 1029, 64], 1, 64, False), (2, [777, 2, 4096], 2, 32, False),
         (3, [5000, 3, 129], 3, 128, True), (4, [2100, 0, 1, 1500], 4, 64, False), (5, [640, 130], 4, 128, True)]


@pytest.mark.parametrize("out_dtype,epi", MODES)
@pytest.mark.parametrize("seed,lens,nn,bs,inter", CASES)
def test_fp4_vs_oracle(out_dtype, epi, seed, lens, nn, bs, inter):
    wl = W.fp4_random(seed, lens, nn, bs, interleaved=inter)
    worst = _check(wl, _run(wl, _dev(wl), out_dtype, epi), out_dtype, epi)
    if not WORST:
        LINES.append(_WorstLine())
    key = (NAME[out_dtype], NAME[epi])
    WORST[key] = max(WORST.get(key, 0.0), worst)


def test_pages_example_zero_inputs():
    """The page's Example: two requests of 3000 and 8000 keys, three draft
    slots, 32-key blocks, identity block table, zero-filled quantised tensors:
    every visible logit is exactly zero, in the default bfloat16 output."""
    B, nn, bs = 2, 3, 32
    wl = W.Fp4Workload(name="fp4_example", q=np.zeros((B, nn, 64, 64), np.uint8), q_sf=np.zeros((B, nn, 64), np.int32),
                       kv_fused=np.zeros((500, bs * 68), np.uint8),
                       weights=np.random.default_rng(0).random((B * nn, 64)).astype(np.float32),
                       block_tables=np.arange(500, dtype=np.int32).reshape(2, 250),
                       seq_lens=np.array([3000, 8000], np.int32), max_seq_len=8000, block_size=bs, next_n=nn,
                       interleaved=False, description="")
    d = _dev(wl)
    out = pm.fp4_mqa_logits(d["q"], d["qsf"], d["kv"], d["w"], d["bt"], d["sl"], 8000)
    assert out.dtype == BF16 and out.shape == (6, 8000)
    got = out.float().cpu().numpy()
    for r, e in enumerate(wl.row_ends()):
        assert np.all(got[r, :e] == 0.0)
    _check(wl, _run(wl, d, BF16, F32), BF16, F32, exact=True)


@pytest.mark.parametrize("nn", [1, 4])
def test_rounded_outputs_are_the_rounded_f32_output(nn):
    """With the float32 epilogue, the bfloat16 and float16 outputs are the
    float32 output rounded to nearest even, bit for bit."""
    wl = W.fp4_random(20 + nn, [2500, 64, 1000], nn, 64)
    d = _dev(wl)
    a = _run(wl, d, F32, F32)
    for dt in (BF16, F16):
        h = _run(wl, d, dt, F32)
        for r, e in enumerate(wl.row_ends()):
            assert torch.equal(a[r, :e].to(dt).view(torch.int16), h[r, :e].view(torch.int16)), (dt, r)


def test_interleaved_equals_token_order():
    """The same pool written with token-order and with interleaved scale slots
    gives the same logits bit for bit (block size 128)."""
    a = W.fp4_random(30, [3000, 700], 2, 128, interleaved=False)
    b = W.fp4_random(30, [3000, 700], 2, 128, interleaved=True)
    assert not np.array_equal(a.kv_fused, b.kv_fused)
    ra, rb = _run(a, _dev(a), F32, F32), _run(b, _dev(b), F32, F32)
    for r, e in enumerate(a.row_ends()):
        assert torch.equal(ra[r, :e].view(torch.int32), rb[r, :e].view(torch.int32)), r


def test_rejects_unsupported_arguments():
    wl = W.fp4_random(31, [100], 1, 64)
    d = _dev(wl)
    with pytest.raises(pm.PmqaError):  # interleaved scales need block size 128
        pm.fp4_mqa_logits(d["q"], d["qsf"], d["kv"], d["w"], d["bt"], d["sl"], 100, is_kv_sf_interleaved=True)
    with pytest.raises(pm.PmqaError):
        pm.fp4_mqa_logits(d["q"], d["qsf"], d["kv"], d["w"], d["bt"], d["sl"], 100, sf_vec_size=16)


@pytest.mark.parametrize("cfg", [3, 4])
def test_fp4_bench_shapes_all_rows(cfg):
    """The MXFP4 pools bench.py times (decode batch and MTP batch shapes), in
    the page's default precisions: every visible logit of every row against the
    float64 oracle."""
    wl = W.fp4_config(cfg)
    worst = _check(wl, _run(wl, _dev(wl), BF16, F32), BF16, F32)
    LINES.append(f"{wl.name}: worst |logit err| / tol over all rows = {worst:.3g}")
