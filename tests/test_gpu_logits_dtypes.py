"""GPU parity of pmqa_mqa_logits_typed (float16 accumulator, epilogue and
output options of page "flashinfer.attn_scores", fp8_paged_mqa_logits) against
the float64 oracle of oracle/dtypes.py."""
import math

import numpy as np
import pytest
import torch

import oracle
import paged_fp8_mqa_amd as pm
import workloads as W
from gpu_util import dev
from report import LINES

pytestmark = pytest.mark.gpu

F32, F16 = torch.float32, torch.float16
NAME = {F32: "f32", F16: "f16"}
WORST = {}  # (output, epi, acc) -> worst |err| / tol over the random workloads


class _WorstLine:
    def __str__(self):
        return "typed logits, worst |err| / tol per (output, epi, acc): " + ", ".join(
            f"{'/'.join(k)} {v:.3g}" for k, v in sorted(WORST.items()))
SENT16 = 0x7E5A  # a float16 NaN pattern no kernel writes


def _run(wl, d, out_dtype, epi, acc):
    cols = pm.padded_seq_len(wl.max_seq_len)
    out = torch.empty(wl.rows, cols, dtype=out_dtype, device="cuda")
    if out_dtype == F16:
        out.view(torch.int16).fill_(SENT16)
    else:
        out.view(torch.int32).fill_(0x7FC00BAD)
    pm.mqa_logits(d["q"], d["kv"], d["w"], d["bt"], d["sl"], wl.max_seq_len, out=out, output_dtype=out_dtype,
                  epi_dtype=epi, acc_dtype=acc)
    torch.cuda.synchronize()
    return out


def _check(wl, out, out_dtype, epi, acc, exact=False):
    ref = oracle.mqa_logits_dtypes(wl.q, wl.kv_fused, wl.weights, wl.block_tables, wl.seq_lens, wl.block_size,
                                   wl.max_seq_len, output_dtype=NAME[out_dtype], epi_dtype=NAME[epi],
                                   acc_dtype=NAME[acc])
    got = out.float().cpu().numpy().astype(np.float64)
    raw = out.cpu().view(torch.int16 if out_dtype == F16 else torch.int32).numpy()
    sent = SENT16 if out_dtype == F16 else 0x7FC00BAD
    ends = oracle.row_ends(wl.seq_lens, wl.next_n)
    worst = 0.0
    for r in range(wl.rows):
        L = int(wl.seq_lens[r // wl.next_n])
        if L == 0:
            assert np.all(raw[r] == np.array(sent).astype(raw.dtype)), f"row {r} of an empty request was written"
            continue
        written = int(math.ceil(L / 64) * 64)
        assert np.all(raw[r, written:] == np.array(sent).astype(raw.dtype)), f"row {r}: write past {written}"
        e = int(ends[r])
        if e == 0:
            continue
        v, t = ref["value"][r, :e], ref["tol"][r, :e]
        g = got[r, :e]
        must, may = ref["must_inf"][r, :e], ref["may_inf"][r, :e]
        assert np.all(np.isinf(g[must]) & (np.sign(g[must]) == np.sign(v[must]))), f"row {r}: expected inf"
        ok = ~may
        if exact:
            assert np.array_equal(g[ok], v[ok]), f"row {r}: not exact"
        err = np.abs(g[ok] - v[ok])
        assert np.all(np.isfinite(g[ok])), f"row {r}: non-finite"
        assert np.all(err <= t[ok]), f"row {r}: max err/tol {np.max(err / np.maximum(t[ok], 1e-300)):.3g}"
        loose = may & ~must
        assert np.all(np.isinf(g[loose]) | (np.abs(g[loose] - v[loose]) <= t[loose]))
        worst = max(worst, float(np.max(err / np.maximum(t[ok], 1e-300))) if ok.any() else 0.0)
    return worst


MODES = [(F32, F32, F16), (F32, F16, F32), (F16, F32, F32), (F16, F16, F16), (F16, F32, F16), (F32, F16, F16)]


@pytest.mark.parametrize("out_dtype,epi,acc", MODES)
@pytest.mark.parametrize("seed,lens,nn,bs", [(1, [300, 0, 1029, 64], 1, 64), (2, [777, 2, 4096], 2, 32),
                                             (3, [5000, 3], 3, 128), (4, [2100, 0, 1, 1500], 4, 64)])
def test_typed_vs_oracle(out_dtype, epi, acc, seed, lens, nn, bs):
    wl = W.small_random(seed, lens, nn, bs, top_k=1, capacity=1, key_scale=1.5)
    worst = _check(wl, _run(wl, dev(wl), out_dtype, epi, acc), out_dtype, epi, acc)
    key = (NAME[out_dtype], NAME[epi], NAME[acc])
    if not WORST:
        LINES.append(_WorstLine())  # formatted at the end, with every mode's final figure
    WORST[key] = max(WORST.get(key, 0.0), worst)


@pytest.mark.parametrize("out_dtype,epi,acc", MODES)
@pytest.mark.parametrize("nn", [1, 2, 3, 4])
def test_f16_exact_inputs_give_exact_results(out_dtype, epi, acc, nn):
    """Inputs whose every partial sum is a float16 number: every option gives
    the formula's exact value."""
    wl = W.small_f16_exact(10 + nn, [700, 0, 129, 2050], nn, 64)
    _check(wl, _run(wl, dev(wl), out_dtype, epi, acc), out_dtype, epi, acc, exact=True)


def test_pages_example_all_options():
    wl = W.make(2)
    d = dev(wl)
    for mode in MODES:
        _check(wl, _run(wl, d, *mode), *mode)


def test_f32_options_equal_the_untyped_entry_point():
    wl = W.small_random(5, [3000, 17, 0, 900], 3, 64, top_k=1, capacity=1)
    d = dev(wl)
    a = _run(wl, d, F32, F32, F32)
    cols = pm.padded_seq_len(wl.max_seq_len)
    b = torch.empty(wl.rows, cols, dtype=F32, device="cuda")
    b.view(torch.int32).fill_(0x7FC00BAD)
    pm.lib().pmqa_mqa_logits(*pm._paged(d["q"], d["kv"], d["w"], d["bt"], d["sl"], None)[0], wl.max_seq_len,
                             pm._ptr(b), b.stride(0), pm._stream(None))
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int32), b.view(torch.int32))


@pytest.mark.parametrize("nn", [1, 4])
def test_f16_output_is_the_rounded_f32_output(nn):
    """A float16 output with the float32 epilogue is the float32 result rounded
    to nearest even, bit for bit (torch's conversion does that rounding)."""
    wl = W.small_random(6 + nn, [2500, 64, 1000], nn, 64, top_k=1, capacity=1)
    d = dev(wl)
    for acc in (F32, F16):
        a = _run(wl, d, F32, F32, acc)
        h = _run(wl, d, F16, F32, acc)
        ends = oracle.row_ends(wl.seq_lens, nn)
        for r in range(wl.rows):
            e = int(ends[r])
            assert torch.equal(a[r, :e].half().view(torch.int16), h[r, :e].view(torch.int16)), r


def _overflow_workload(nn):
    """One request of 70 keys: key 0 scores 2^17 in row 0 (head 0's dot product
    256 * 8 = 2048, weight 1, scale 64), every other score is 0."""
    bs, L = 64, 70
    nb = 3
    vals = np.zeros((nb, bs, 128), np.float32)
    vals[0, 0, 0] = 8
    sc = np.ones((nb, bs), np.float32)
    sc[0, 0] = 64
    kv = torch.cat([torch.from_numpy(vals).to(torch.float8_e4m3fn).view(torch.uint8).reshape(nb, -1),
                    torch.from_numpy(sc).view(torch.uint8).reshape(nb, -1)], 1).numpy()
    qv = np.zeros((1, nn, 64, 128), np.float32)
    qv[0, :, 0, 0] = 256
    q = torch.from_numpy(qv).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    w = np.zeros((nn, 64), np.float32)
    w[:, 0] = 1
    return W.Workload(name="overflow", q=q, kv_fused=kv, weights=w, block_tables=np.array([[0, 1]], np.int32),
                      seq_lens=np.array([L], np.int32), max_seq_len=L, block_size=bs, next_n=nn, top_k=1,
                      capacity=1, threshold_recipe="", description="")


@pytest.mark.parametrize("nn", [1, 3])
def test_overflow_to_infinity(nn):
    wl = _overflow_workload(nn)
    d = dev(wl)
    assert float(_run(wl, d, F32, F32, F32)[0, 0]) == 2.0 ** 17
    assert float(_run(wl, d, F32, F32, F16)[0, 0]) == 2.0 ** 17
    assert float(_run(wl, d, F32, F16, F32)[0, 0]) == float("inf")
    assert float(_run(wl, d, F16, F32, F32)[0, 0]) == float("inf")
    for mode in MODES:
        _check(wl, _run(wl, d, *mode), *mode)


@pytest.mark.parametrize("mode", [(F16, F16, F16), (F32, F32, F16)])
def test_typed_bench_shape_all_rows(mode):
    """The MTP draft batch (32 requests x 4 rows, up to 65536 keys) through the
    typed logits: every visible logit of every row within the bound."""
    wl = W.make(4)
    worst = _check(wl, _run(wl, dev(wl), *mode), *mode)
    LINES.append(f"{wl.name} typed {'/'.join(NAME[m] for m in mode)}: worst |err| / tol over all rows = {worst:.3g}")
