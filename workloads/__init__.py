"""Seeded synthetic inputs for the paged FP8 MQA logits + Top-k select path.

This module only draws random numbers and packs them into the input formats the
pages define; it holds none of the method's arithmetic (no scores, no
selection).  Both the CPU oracle and the HIP path consume what it returns.

Input formats (page "flashinfer.attn_scores", fp8_paged_mqa_logits parameters):
  * ``q``            uint8 [B, next_n, H, D]   e4m3fn codes
  * ``kv_fused``     uint8 [num_blocks, block_size*(D+4)]  per block: all e4m3
                     values token-major, then block_size little-endian f32
                     scales (the Example's torch.cat recipe)
  * ``weights``      f32   [B*next_n, H]
  * ``block_tables`` int32 [B, width]
  * ``seq_lens``     int32 [B]

Random-page workloads put every request's pages at random physical ids of one
shared pool and add one poison page.  Trailing block-table entries point at it,
and every token past a request's length (in its last page and in the poison
page) holds e4m3 NaN (0x7F) with a NaN scale, so a read past a request's pages
or a missing visibility mask shows up as NaN.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional

import numpy as np
import torch

H = 64
D = 128
E4M3_NAN = 0x7F
F32_NAN_BITS = 0x7FC00000


@dataclasses.dataclass
class Workload:
    name: str
    q: np.ndarray             # uint8 [B, next_n, H, D]
    kv_fused: np.ndarray      # uint8 [num_blocks, bs*(D+4)]
    weights: np.ndarray       # float32 [B*next_n, H]
    block_tables: np.ndarray  # int32 [B, width]
    seq_lens: np.ndarray      # int32 [B]
    max_seq_len: int
    block_size: int
    next_n: int
    top_k: int
    capacity: int
    threshold_recipe: str
    description: str

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def rows(self) -> int:
        return self.batch * self.next_n

    @property
    def num_blocks(self) -> int:
        return int(self.kv_fused.shape[0])

    def row_ends(self) -> np.ndarray:
        """Visible length of each row: seq_lens[b] - next_n + t + 1, floored at 0."""
        b = np.repeat(self.seq_lens.astype(np.int64), self.next_n)
        t = np.tile(np.arange(self.next_n, dtype=np.int64), self.batch)
        return np.maximum(0, b - self.next_n + t + 1)


def _e4m3_codes(x: torch.Tensor) -> torch.Tensor:
    """Round to e4m3fn (torch's RNE cast) and return the raw byte codes."""
    return x.to(torch.float8_e4m3fn).view(torch.uint8)


def _pack_kv_fused(values: torch.Tensor, scales: torch.Tensor) -> np.ndarray:
    """The pages' torch.cat recipe: per block, the value bytes then the scale bytes.

    values: uint8 [num_blocks, bs, D]; scales: float32 [num_blocks, bs].
    """
    nb = values.shape[0]
    fused = torch.cat([values.reshape(nb, -1), scales.contiguous().view(torch.uint8).reshape(nb, -1)], dim=1)
    return fused.numpy().copy()


def _random_pool(gen: torch.Generator, seq_lens: List[int], bs: int, width: int):
    """Random physical page ids for every request plus one trailing poison page.

    Returns (block_tables int32 [B, width], num_blocks, page_of) where page_of[b]
    lists request b's physical pages in logical order.
    """
    counts = [int(math.ceil(L / bs)) for L in seq_lens]
    total = sum(counts)
    perm = torch.randperm(total, generator=gen).numpy().astype(np.int32)
    poison = total
    bt = np.full((len(seq_lens), width), poison, dtype=np.int32)
    page_of = []
    off = 0
    for b, n in enumerate(counts):
        bt[b, :n] = perm[off:off + n]
        page_of.append(perm[off:off + n])
        off += n
    return bt, total + 1, page_of


def _poison_tails(values: torch.Tensor, scales: torch.Tensor, seq_lens, page_of, bs: int, poison: int):
    """NaN codes and NaN scales for every token a request does not own."""
    nan_scale = torch.tensor([F32_NAN_BITS], dtype=torch.int32).view(torch.float32)[0]
    for b, L in enumerate(seq_lens):
        if L % bs and len(page_of[b]):
            last = int(page_of[b][-1])
            values[last, L % bs:, :] = E4M3_NAN
            scales[last, L % bs:] = nan_scale
    values[poison] = E4M3_NAN
    scales[poison] = nan_scale


def _uniform(gen, shape, lo, hi):
    return lo + (hi - lo) * torch.rand(shape, generator=gen, dtype=torch.float32)


def _randint_inclusive(gen, lo, hi, n):
    return [int(v) for v in torch.randint(lo, hi + 1, (n,), generator=gen)]


def config1(seed: int = 1001) -> Workload:
    """Single request, plain decode, 2048 keys in 64-token pages, identity table."""
    g = torch.Generator().manual_seed(seed)
    B, nn, bs, L = 1, 1, 64, 2048
    nb = L // bs
    q = _e4m3_codes(torch.clamp(torch.randn(B, nn, H, D, generator=g), -4, 4))
    kv = _e4m3_codes(torch.clamp(torch.randn(nb, bs, D, generator=g), -4, 4))
    s = _uniform(g, (nb, bs), 0.5, 2.0)
    w = _uniform(g, (B * nn, H), -1.0, 1.0)
    return Workload(
        name="cfg1_decode_b1_l2048", q=q.numpy().copy(), kv_fused=_pack_kv_fused(kv, s),
        weights=w.numpy().copy(), block_tables=np.arange(nb, dtype=np.int32).reshape(1, nb),
        seq_lens=np.array([L], dtype=np.int32), max_seq_len=L, block_size=bs, next_n=nn,
        top_k=256, capacity=512, threshold_recipe="inf|sigma_k",
        description="B=1 next_n=1 bs=64 L=2048 identity table; q,k=e4m3(clamp(randn,-4,4)); s~U[0.5,2]; w~U[-1,1]; top_k=256")


def config2(seed: int = 1002) -> Workload:
    """The pages' worked example: two requests, three draft slots, 32-token blocks."""
    g = torch.Generator().manual_seed(seed)
    B, nn, bs, max_len = 2, 3, 32, 8000
    width = int(math.ceil(max_len / bs))
    nb = B * width
    kv = _e4m3_codes(torch.randn(nb, bs, D, generator=g))
    s = torch.ones(nb, bs)
    q = _e4m3_codes(torch.randn(B, nn, H, D, generator=g))
    w = torch.rand(B * nn, H, generator=g)
    return Workload(
        name="cfg2_pages_example", q=q.numpy().copy(), kv_fused=_pack_kv_fused(kv, s),
        weights=w.numpy().copy(), block_tables=np.arange(nb, dtype=np.int32).reshape(B, width),
        seq_lens=np.array([3000, 8000], dtype=np.int32), max_seq_len=max_len, block_size=bs,
        next_n=nn, top_k=512, capacity=1024, threshold_recipe="inf|sigma_k",
        description="pages' example: B=2 next_n=3 bs=32 seq_lens=[3000,8000] table=arange(500).view(2,250); q,k=e4m3(randn); s=1; w=rand; top_k=512")


def _random_page_workload(g, name, seq_lens, bs, nn, max_len, key_fn, scale_fn, q_fn, w_fn,
                          top_k, capacity, recipe, desc) -> Workload:
    B = len(seq_lens)
    width = int(math.ceil(max_len / bs))
    bt, nb, page_of = _random_pool(g, seq_lens, bs, width)
    values = key_fn(nb, bs)
    scales = scale_fn(nb, bs)
    _poison_tails(values, scales, seq_lens, page_of, bs, nb - 1)
    q = q_fn(B, nn)
    w = w_fn(B * nn)
    return Workload(
        name=name, q=q.numpy().copy(), kv_fused=_pack_kv_fused(values, scales), weights=w.numpy().copy(),
        block_tables=bt, seq_lens=np.array(seq_lens, dtype=np.int32), max_seq_len=max_len,
        block_size=bs, next_n=nn, top_k=top_k, capacity=capacity, threshold_recipe=recipe, description=desc)


def config3(seed: int = 1003, batch: int = 64) -> Workload:
    """Decode batch: 64 requests, lengths U[4096,32768], random pages."""
    g = torch.Generator().manual_seed(seed)
    bs, nn, lo, hi = 64, 1, 4096, 32768
    seq_lens = _randint_inclusive(g, lo, hi, batch)
    return _random_page_workload(
        g, "cfg3_decode_b64", seq_lens, bs, nn, hi,
        key_fn=lambda nb, bs_: _e4m3_codes(0.5 * torch.randn(nb, bs_, D, generator=g)),
        scale_fn=lambda nb, bs_: _uniform(g, (nb, bs_), 0.25, 4.0),
        q_fn=lambda b, n: _e4m3_codes(0.5 * torch.randn(b, n, H, D, generator=g)),
        w_fn=lambda r: _uniform(g, (r, H), -1.0, 1.0),
        top_k=2048, capacity=4096, recipe="sigma_k_minus_1e-3",
        desc="B=64 next_n=1 bs=64 seq_lens~U[4096,32768] random pages; q,k=e4m3(0.5 randn); s~U[0.25,4]; w~U[-1,1]; top_k=2048 cap=4096")


def config4(seed: int = 1004, batch: int = 32) -> Workload:
    """MTP draft: 32 requests x 4 draft slots, keys from 8 Gaussian clusters (scale 1)."""
    g = torch.Generator().manual_seed(seed)
    bs, nn, lo, hi = 64, 4, 16384, 65536
    seq_lens = _randint_inclusive(g, lo, hi, batch)
    centroids = torch.randn(8, D, generator=g)

    def keys(nb, bs_):
        n = nb * bs_
        j = torch.randint(0, 8, (n,), generator=g)
        exact = torch.rand(n, generator=g) < 0.5
        x = centroids[j] + 0.25 * torch.randn(n, D, generator=g) * (~exact).unsqueeze(1).float()
        return _e4m3_codes(x).reshape(nb, bs_, D).contiguous()

    return _random_page_workload(
        g, "cfg4_mtp_b32_n4", seq_lens, bs, nn, hi, key_fn=keys,
        scale_fn=lambda nb, bs_: torch.ones(nb, bs_),
        q_fn=lambda b, n: _e4m3_codes(torch.randn(b, n, H, D, generator=g)),
        w_fn=lambda r: _uniform(g, (r, H), -1.0, 1.0),
        top_k=2048, capacity=4096, recipe="sigma_k_minus_1e-3",
        desc="B=32 next_n=4 bs=64 seq_lens~U[16384,65536] random pages; keys from 8 clusters (half exact centroids); s=1; q=e4m3(randn); w~U[-1,1]; top_k=2048 cap=4096")


def config5(seed: int = 1005, capacity: Optional[int] = None) -> Workload:
    """Long context: 8 requests of 131072 keys, request 3 empty, two draft slots."""
    g = torch.Generator().manual_seed(seed)
    bs, nn, L = 64, 2, 131072
    seq_lens = [L] * 8
    seq_lens[3] = 0
    top_k = 2048
    return _random_page_workload(
        g, "cfg5_long_b8_n2", seq_lens, bs, nn, L,
        key_fn=lambda nb, bs_: _e4m3_codes(torch.randn(nb, bs_, D, generator=g)),
        scale_fn=lambda nb, bs_: _uniform(g, (nb, bs_), 0.5, 2.0),
        q_fn=lambda b, n: _e4m3_codes(torch.randn(b, n, H, D, generator=g)),
        w_fn=lambda r: _uniform(g, (r, H), -1.0, 1.0),
        top_k=top_k, capacity=capacity if capacity is not None else 2 * top_k,
        recipe="even_sigma_256_odd_sigma_k_minus_1e-3",
        desc="B=8 next_n=2 bs=64 L=131072 (request 3 empty) random pages; q,k=e4m3(randn); s~U[0.5,2]; w~U[-1,1]; top_k=2048")


def small_random(seed: int, seq_lens: List[int], next_n: int, block_size: int, top_k: int,
                 capacity: int, max_seq_len: Optional[int] = None, key_scale: float = 1.0,
                 scale_lo: float = 0.5, scale_hi: float = 2.0, w_lo: float = -1.0, w_hi: float = 1.0,
                 extra_width: int = 0) -> Workload:
    """Small random-page workload for edge-case parity tests."""
    g = torch.Generator().manual_seed(seed)
    max_len = max_seq_len if max_seq_len is not None else max(max(seq_lens), 1)
    bs = block_size
    width = int(math.ceil(max_len / bs)) + extra_width
    bt, nb, page_of = _random_pool(g, seq_lens, bs, width)
    values = _e4m3_codes(key_scale * torch.randn(nb, bs, D, generator=g))
    scales = _uniform(g, (nb, bs), scale_lo, scale_hi)
    _poison_tails(values, scales, seq_lens, page_of, bs, nb - 1)
    q = _e4m3_codes(key_scale * torch.randn(len(seq_lens), next_n, H, D, generator=g))
    w = _uniform(g, (len(seq_lens) * next_n, H), w_lo, w_hi)
    return Workload(
        name=f"small_s{seed}", q=q.numpy().copy(), kv_fused=_pack_kv_fused(values, scales),
        weights=w.numpy().copy(), block_tables=bt, seq_lens=np.array(seq_lens, dtype=np.int32),
        max_seq_len=max_len, block_size=bs, next_n=next_n, top_k=top_k, capacity=capacity,
        threshold_recipe="test", description=f"small random-page workload seed={seed}")


def small_f16_exact(seed: int, seq_lens: List[int], next_n: int, block_size: int) -> Workload:
    """Small random-page workload whose logits are exact in float16 arithmetic
    in any order: q has at most 4 nonzero entries per head, all q and key
    entries are -1, 0 or 1, weights are +-0.5 or +-1 and scales 0.5, 1 or 2, so
    every dot product is an integer of magnitude at most 4, every partial sum a
    multiple of 0.25 below 2^9 in magnitude."""
    g = torch.Generator().manual_seed(seed)
    max_len = max(max(seq_lens), 1)
    bs = block_size
    width = int(math.ceil(max_len / bs))
    bt, nb, page_of = _random_pool(g, seq_lens, bs, width)
    values = _e4m3_codes(torch.randint(-1, 2, (nb, bs, D), generator=g).float())
    scales = torch.tensor([0.5, 1.0, 2.0])[torch.randint(0, 3, (nb, bs), generator=g)]
    _poison_tails(values, scales, seq_lens, page_of, bs, nb - 1)
    qv = torch.zeros(len(seq_lens), next_n, H, D)
    pos = torch.randint(0, D, (len(seq_lens), next_n, H, 4), generator=g)
    qv.scatter_(3, pos, torch.randint(-1, 2, (len(seq_lens), next_n, H, 4), generator=g).float())
    q = _e4m3_codes(qv)
    w = torch.tensor([-1.0, -0.5, 0.5, 1.0])[torch.randint(0, 4, (len(seq_lens) * next_n, H), generator=g)]
    return Workload(
        name=f"f16exact_s{seed}", q=q.numpy().copy(), kv_fused=_pack_kv_fused(values, scales),
        weights=w.numpy().astype(np.float32).copy(), block_tables=bt, seq_lens=np.array(seq_lens, dtype=np.int32),
        max_seq_len=max_len, block_size=bs, next_n=next_n, top_k=1, capacity=1, threshold_recipe="test",
        description=f"float16-exact small workload seed={seed}")


@dataclasses.dataclass
class PrefillWorkload:
    """Prefill-shaped rows: query tiles of tile_rows rows, each tile on one
    request (tile_requests), each row with its own key end (row_ends)."""
    name: str
    q: np.ndarray              # uint8 [rows, H, D]
    kv_fused: np.ndarray       # uint8 [num_blocks, bs*(D+4)]
    weights: np.ndarray        # float32 [rows, H]
    block_tables: np.ndarray   # int32 [requests, width]
    seq_lens: np.ndarray       # int32 [requests]: the keys each request holds
    tile_requests: np.ndarray  # int32 [tiles]
    row_ends: np.ndarray       # int32 [rows]
    max_context: int
    block_size: int
    tile_rows: int
    top_k: int
    capacity: int
    description: str

    @property
    def tiles(self) -> int:
        return int(self.tile_requests.shape[0])

    @property
    def rows(self) -> int:
        return int(self.row_ends.shape[0])

    @property
    def num_blocks(self) -> int:
        return int(self.kv_fused.shape[0])


def prefill_random(seed: int, prompts: List[tuple], tile_rows: int, block_size: int, top_k: int, capacity: int,
                   key_scale: float = 1.0, shuffle_tiles: bool = True, name: Optional[str] = None) -> PrefillWorkload:
    """Causal prefill rows over random pages.  prompts[i] = (prefix, new):
    request i holds prefix + new keys, and its j-th new token's row sees keys
    below prefix + j + 1.  A request's rows fill tiles of tile_rows in order;
    the last tile is topped up with rows that see nothing.  With shuffle_tiles
    the tiles of all requests come in random order."""
    g = torch.Generator().manual_seed(seed)
    lens = [int(p) + int(n) for p, n in prompts]
    bs = block_size
    max_ctx = max(max(lens), 1)
    width = int(math.ceil(max_ctx / bs))
    bt, nb, page_of = _random_pool(g, lens, bs, width)
    values = _e4m3_codes(key_scale * torch.randn(nb, bs, D, generator=g))
    scales = _uniform(g, (nb, bs), 0.5, 2.0)
    _poison_tails(values, scales, lens, page_of, bs, nb - 1)
    tiles = []  # (request, [row ends])
    for i, (pre, new) in enumerate(prompts):
        ends = [int(pre) + j + 1 for j in range(int(new))]
        for t0 in range(0, len(ends), tile_rows):
            e = ends[t0:t0 + tile_rows]
            tiles.append((i, e + [0] * (tile_rows - len(e))))
    if shuffle_tiles and tiles:
        order = torch.randperm(len(tiles), generator=g).tolist()
        tiles = [tiles[j] for j in order]
    R = len(tiles) * tile_rows
    q = _e4m3_codes(key_scale * torch.randn(R, H, D, generator=g))
    w = _uniform(g, (R, H), -1.0, 1.0)
    return PrefillWorkload(
        name=name or f"prefill_s{seed}", q=q.numpy().copy(), kv_fused=_pack_kv_fused(values, scales),
        weights=w.numpy().copy(), block_tables=bt, seq_lens=np.array(lens, dtype=np.int32),
        tile_requests=np.array([t[0] for t in tiles], dtype=np.int32),
        row_ends=np.array([e for t in tiles for e in t[1]], dtype=np.int32), max_context=max_ctx, block_size=bs,
        tile_rows=tile_rows, top_k=top_k, capacity=capacity,
        description=f"causal prefill rows, prompts (prefix, new) = {list(prompts)}, tiles of {tile_rows} rows")


def prefill_chunk(seed: int = 1006) -> PrefillWorkload:
    """A prefill chunk: two requests, 512 new tokens each on cached prefixes of
    12288 and 4096 keys, tiles of 4 rows in random order, top_k 2048."""
    return prefill_random(seed, [(12288, 512), (4096, 512)], tile_rows=4, block_size=64, top_k=2048,
                          capacity=4096, name="prefill_chunk_2x512")


def prefill_fingerprint(w: PrefillWorkload) -> str:
    import hashlib
    h = hashlib.sha256()
    for a in (w.q, w.kv_fused, w.weights, w.block_tables, w.tile_requests, w.row_ends):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]


CONFIGS = {1: config1, 2: config2, 3: config3, 4: config4, 5: config5}


# ---------------------------------------------------------------- MXFP4 pools

_E2M1_MAGS = torch.tensor([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])


def _mx_quantize(x: torch.Tensor):
    """Synthetic MXFP4 data from float values x [..., 128]: per group of 32 the
    scale exponent e = ceil(log2(amax / 6)) (so the group's largest magnitude
    fits the largest E2M1 value), the UE8M0 byte e + 127, and each element the
    E2M1 code nearest x / 2^e (the lower magnitude on a tie).  Returns (packed
    uint8 [..., 64] with element 2m in the low nibble of byte m, scale bytes
    uint8 [..., 4])."""
    g = x.reshape(*x.shape[:-1], 4, 32)
    amax = g.abs().amax(dim=-1).clamp_min(2.0 ** -100)
    e = torch.ceil(torch.log2(amax / 6.0)).clamp(-127, 127)
    y = g / torch.pow(2.0, e).unsqueeze(-1)
    mag = (y.abs().unsqueeze(-1) - _E2M1_MAGS).abs().argmin(dim=-1)
    codes = (mag | ((y < 0) & (mag > 0)).to(torch.int64) * 8).to(torch.uint8).reshape(x.shape)
    packed = codes[..., 0::2] | (codes[..., 1::2] << 4)
    return packed, (e + 127).to(torch.uint8)


@dataclasses.dataclass
class Fp4Workload:
    """An MXFP4 paged pool (page "flashinfer.attn_scores", fp4_paged_mqa_logits)."""
    name: str
    q: np.ndarray              # uint8 [B, next_n, H, 64]
    q_sf: np.ndarray           # int32 [B, next_n, H] (byte k: group k's scale)
    kv_fused: np.ndarray       # uint8 [num_blocks, bs*68]
    weights: np.ndarray        # float32 [B*next_n, H]
    block_tables: np.ndarray   # int32 [B, width]
    seq_lens: np.ndarray       # int32 [B]
    max_seq_len: int
    block_size: int
    next_n: int
    interleaved: bool
    description: str

    @property
    def batch(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def rows(self) -> int:
        return self.batch * self.next_n

    @property
    def num_blocks(self) -> int:
        return int(self.kv_fused.shape[0])

    def row_ends(self) -> np.ndarray:
        L = np.repeat(self.seq_lens.astype(np.int64), self.next_n)
        t = np.tile(np.arange(self.next_n), self.batch)
        return np.maximum(0, L - self.next_n + t + 1)


def fp4_random(seed: int, seq_lens: List[int], next_n: int, block_size: int, interleaved: bool = False,
               max_seq_len: Optional[int] = None, key_scale: float = 1.0, name: Optional[str] = None) -> Fp4Workload:
    """MXFP4 pool over random pages: q and keys are Gaussian (key_scale times
    randn) quantised per group of 32; weights U[-1, 1].  Every token a request
    does not own (its last page's tail, the poison page) has NaN scale bytes
    (255), so an over-read shows as NaN.  With interleaved, each block's scale
    slots are in the interleaved order (slot k holds token (k % 4) * bs/4 + k / 4)."""
    g = torch.Generator().manual_seed(seed)
    bs = block_size
    max_len = max_seq_len if max_seq_len is not None else max(max(seq_lens), 1)
    width = int(math.ceil(max_len / bs))
    bt, nb, page_of = _random_pool(g, seq_lens, bs, width)
    vals, sf = _mx_quantize(key_scale * torch.randn(nb, bs, D, generator=g))
    for b, L in enumerate(seq_lens):
        if L % bs and len(page_of[b]):
            sf[int(page_of[b][-1]), L % bs:] = 255
    sf[nb - 1] = 255
    if interleaved:
        order = torch.tensor([(k % 4) * (bs // 4) + k // 4 for k in range(bs)])
        sf = sf[:, order]
    kv = torch.cat([vals.reshape(nb, -1), sf.reshape(nb, -1)], dim=1).numpy().copy()
    qv, qs = _mx_quantize(key_scale * torch.randn(len(seq_lens), next_n, H, D, generator=g))
    w = _uniform(g, (len(seq_lens) * next_n, H), -1.0, 1.0)
    return Fp4Workload(
        name=name or f"fp4_s{seed}", q=qv.numpy().copy(), q_sf=qs.contiguous().view(torch.int32).squeeze(-1).numpy().copy(),
        kv_fused=kv, weights=w.numpy().copy(), block_tables=bt, seq_lens=np.array(seq_lens, dtype=np.int32),
        max_seq_len=max_len, block_size=bs, next_n=next_n, interleaved=interleaved,
        description=f"MXFP4 random-page pool seed={seed}, bs={bs}, interleaved scales={interleaved}")


def fp4_config(i: int) -> Fp4Workload:
    """MXFP4 pools of the decode batch (3) and the MTP draft batch (4) shapes:
    the same batch sizes, next_n, block size and length ranges."""
    if i == 3:
        g = torch.Generator().manual_seed(1103)
        return fp4_random(1103, _randint_inclusive(g, 4096, 32768, 64), 1, 64, max_seq_len=32768,
                          name="cfg3_decode_b64_mxfp4")
    if i == 4:
        g = torch.Generator().manual_seed(1104)
        return fp4_random(1104, _randint_inclusive(g, 16384, 65536, 32), 4, 64, max_seq_len=65536,
                          name="cfg4_mtp_b32_n4_mxfp4")
    raise ValueError(f"no MXFP4 configuration {i}")


def make(i: int, **kw) -> Workload:
    return CONFIGS[i](**kw)


def fingerprint(w: Workload) -> str:
    """Short digest of a workload's bytes, to detect generator drift."""
    import hashlib
    h = hashlib.sha256()
    for a in (w.q, w.kv_fused, w.weights, w.block_tables, w.seq_lens):
        h.update(np.ascontiguousarray(a).tobytes())
    return h.hexdigest()[:16]
