"""Helpers for the GPU parity tests: move a workload to the device, call the
library through its binding, and read the select buffers back."""
import json
import os

import numpy as np
import torch

import paged_fp8_mqa_amd as pm

SENTINEL_F32_BITS = 0x7FC00BAD        # a NaN payload nobody computes
SENTINEL_I32 = -0x21524111            # 0xDEADBEEF
GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def dev(wl, device="cuda"):
    d = {
        "q": torch.from_numpy(wl.q).to(device),
        "kv": torch.from_numpy(wl.kv_fused).to(device).view(wl.num_blocks, wl.block_size, 1, 132),
        "w": torch.from_numpy(wl.weights).to(device),
        "bt": torch.from_numpy(wl.block_tables).to(device),
        "sl": torch.from_numpy(wl.seq_lens).to(device),
    }
    return d


def sentinel_f32(shape, device="cuda"):
    return torch.full(shape, SENTINEL_F32_BITS, dtype=torch.int32, device=device).view(torch.float32)


def run_logits(wl, d, out_cols=None, max_seq_len=None):
    msl = wl.max_seq_len if max_seq_len is None else max_seq_len
    cols = pm.padded_seq_len(msl) if out_cols is None else out_cols
    out = sentinel_f32((wl.rows, cols))
    view = pm.mqa_logits(d["q"], d["kv"], d["w"], d["bt"], d["sl"], msl, out=out)
    torch.cuda.synchronize()
    return out, view


class SelectBuffers:
    def __init__(self, rows, batch, top_k, capacity, thresholds, device="cuda", arrivals=True, topk=True,
                 workspace=None, which="fused", max_context=0):
        self.top_k, self.capacity = top_k, capacity
        self.thr = torch.as_tensor(np.asarray(thresholds, dtype=np.float32)).to(device)
        self.thr_in = self.thr.clone()
        self.counters = torch.zeros(rows, 2, dtype=torch.int32, device=device)
        self.cand = torch.full((rows, top_k + capacity, 2), SENTINEL_I32, dtype=torch.int32, device=device)
        self.arrivals = torch.zeros(batch, dtype=torch.int32, device=device) if arrivals else None
        self.ranges = torch.full((2, rows), SENTINEL_I32, dtype=torch.int32, device=device) if arrivals else None
        self.topk = torch.full((rows, top_k), SENTINEL_I32, dtype=torch.int32, device=device) if (arrivals and topk) else None
        self.ws = None if not arrivals else (
            workspace if workspace is not None else
            pm.make_workspace(which, batch, rows // batch if batch else 1, max_context, device))

    def kwargs(self):
        return dict(thresholds=self.thr, counters=self.counters, candidates=self.cand, capacity=self.capacity,
                    top_k=self.top_k, arrivals=self.arrivals, ranges=self.ranges, topk_idx=self.topk,
                    workspace=self.ws)

    def host(self):
        torch.cuda.synchronize()
        return {
            "thr_in": self.thr_in.cpu().numpy(), "thr": self.thr.cpu().numpy(),
            "counters": self.counters.cpu().numpy(), "cand": self.cand.cpu().numpy(),
            "arrivals": None if self.arrivals is None else self.arrivals.cpu().numpy(),
            "ranges": None if self.ranges is None else self.ranges.cpu().numpy(),
            "topk": None if self.topk is None else self.topk.cpu().numpy(),
        }


def run_fused(wl, d, thresholds, capacity=None, arrivals=True, topk=True, max_context=None):
    cap = wl.capacity if capacity is None else capacity
    mc = wl.max_seq_len if max_context is None else max_context
    sb = SelectBuffers(wl.rows, wl.batch, wl.top_k, cap, thresholds, arrivals=arrivals, topk=topk, which="fused",
                       max_context=mc)
    pm.fused_logits_select(d["q"], d["kv"], d["w"], d["bt"], d["sl"], mc, **sb.kwargs())
    return sb.host()


def run_select(wl, logits, thresholds, capacity=None, arrivals=True, topk=True, max_context=None):
    cap = wl.capacity if capacity is None else capacity
    mc = wl.max_seq_len if max_context is None else max_context
    sb = SelectBuffers(wl.rows, wl.batch, wl.top_k, cap, thresholds, arrivals=arrivals, topk=topk,
                       which="indexer_topk", max_context=mc)
    sl = torch.from_numpy(wl.seq_lens).to("cuda")
    pm.indexer_topk(logits, sl, wl.next_n, mc, **sb.kwargs())
    return sb.host()


def slot_sets(res, r, top_k, capacity):
    """(candidate pairs, tie pairs) a row holds, as sets of (index, bits)."""
    nc, nt = (int(x) for x in res["counters"][r])
    c = res["cand"][r]
    cands = {tuple(x) for x in c[top_k:top_k + min(nc, capacity)].tolist()}
    ties = {tuple(x) for x in c[top_k - min(nt, top_k):top_k].tolist()}
    return cands, ties


def golden_thresholds(cfg):
    d = json.load(open(os.path.join(GOLDEN, f"thresholds_cfg{cfg}.json")))
    return d, np.array(d["threshold_bits"], dtype=np.int32).view(np.float32)
