"""Python binding of libpmqa: paged FP8 MQA logits and threshold Top-k select
on MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP
kernels of libpmqa.so (built in-tree by ``python -m paged_fp8_mqa_amd.build``).
PyTorch supplies device memory and the current stream.  Loading fails loudly
when the library has not been built; there is no fallback.

Entry points mirror the C ABI in include/pmqa.h:
  mqa_logits(q, kv_fused, weights, block_tables, seq_lens, max_seq_len, out=None,
             output_dtype=None, epi_dtype=None, acc_dtype=None)
  fp4_mqa_logits(q, q_sf, kv_fused, weights, block_tables, seq_lens, max_seq_len, out=None,
             output_dtype=None, epi_dtype=None, is_kv_sf_interleaved=False)
               the MXFP4 pool's logits (bfloat16 output by default)
  indexer_topk(logits, seq_lens, next_n, max_context, thresholds, counters,
               candidates, capacity, top_k, arrivals=None, ranges=None, topk_idx=None,
               workspace=None)
  fused_logits_select(q, kv_fused, weights, block_tables, seq_lens, max_context,
               thresholds, counters, candidates, capacity, top_k,
               arrivals=None, ranges=None, topk_idx=None, workspace=None)
  fused_logits_select_noalloc(...)  as fused_logits_select, without workspace:
               the library's static scratch (NOALLOC_SCRATCH_BYTES) serves
  prefill_select(q, kv_fused, weights, block_tables, tile_requests, row_ends, tile_rows,
               max_context, thresholds, counters, candidates, capacity, top_k,
               arrivals=None, ranges=None, topk_idx=None, workspace=None)
               the fused select over prefill-shaped rows (query tiles of tile_rows
               rows of one request each, explicit row ends)
  make_workspace(which, batch_size, next_n, max_context)
               -> zeroed finish-stage workspace (required with arrivals)
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpmqa.so")

STATUS = {0: "PMQA_OK", 1: "PMQA_ERR_NULL", 2: "PMQA_ERR_SHAPE", 3: "PMQA_ERR_STRIDE",
          4: "PMQA_ERR_UNSUPPORTED", 5: "PMQA_ERR_ALIGN", 6: "PMQA_ERR_OVERFLOW",
          7: "PMQA_ERR_LAUNCH", 8: "PMQA_ERR_CONTENT", 9: "PMQA_ERR_SCRATCH"}

_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

_PAGED = [_P, _P, _P, _P, _I64, _I32, _P, _I64, _I32, _I32, _I32, _I32, _I32, _I64]
_SELECT_OUT = [_P, _P, _P, _I32, _I32, _P, _P, _P, _P, _SZ]
# q, kv, weights, block_tables, stride, width, num_requests, tile_requests, row_ends, num_tiles, tile_rows,
# heads, dim, block_size, num_blocks, max_context
_PREFILL = [_P, _P, _P, _P, _I64, _I32, _I32, _P, _P, _I32, _I32, _I32, _I32, _I32, _I64, _I32]
SIGNATURES = {
    "pmqa_status_string": ([ctypes.c_int], ctypes.c_char_p),
    "pmqa_version": ([], _I32),
    "pmqa_padded_seq_len": ([_I32], _I32),
    "pmqa_min_block_table_width": ([_I32, _I32], _I32),
    "pmqa_keys_per_cta": ([_I32], _I32),
    "pmqa_workspace_bytes": ([_I32, _I32, _I32, _I32], _SZ),
    "pmqa_check_logits_args": (_PAGED + [_I32, _P, _I64], ctypes.c_int),
    "pmqa_mqa_logits": (_PAGED + [_I32, _P, _I64, _P], ctypes.c_int),
    "pmqa_check_logits_typed_args": (_PAGED + [_I32, _P, _I64, _I32, _I32, _I32], ctypes.c_int),
    "pmqa_mqa_logits_typed": (_PAGED + [_I32, _P, _I64, _I32, _I32, _I32, _P], ctypes.c_int),
    "pmqa_check_fp4_logits_args": ([_P, _P] + _PAGED[1:] + [_I32, _I32, _I32, _P, _I64, _I32, _I32], ctypes.c_int),
    "pmqa_fp4_mqa_logits": ([_P, _P] + _PAGED[1:] + [_I32, _I32, _I32, _P, _I64, _I32, _I32, _P], ctypes.c_int),
    "pmqa_check_select_args": ([_P, _I64, _P, _I64, _I32, _I32, _I32] + _SELECT_OUT, ctypes.c_int),
    "pmqa_indexer_topk": ([_P, _I64, _P, _I64, _I32, _I32, _I32] + _SELECT_OUT + [_P], ctypes.c_int),
    "pmqa_check_fused_args": (_PAGED + [_I32] + _SELECT_OUT, ctypes.c_int),
    "pmqa_fused_logits_select": (_PAGED + [_I32] + _SELECT_OUT + [_P], ctypes.c_int),
    "pmqa_fused_logits_select_noalloc": (_PAGED + [_I32] + _SELECT_OUT[:-2] + [_P], ctypes.c_int),
    "pmqa_check_prefill_args": (_PREFILL + _SELECT_OUT, ctypes.c_int),
    "pmqa_prefill_select": (_PREFILL + _SELECT_OUT + [_P], ctypes.c_int),
}

NOALLOC_SCRATCH_BYTES = 96 << 20  # PMQA_NOALLOC_SCRATCH_BYTES

_lib = None


class PmqaError(RuntimeError):
    def __init__(self, status, where):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)}")


def lib():
    """The loaded libpmqa (ctypes.CDLL); raises if it is not built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"libpmqa.so is not built ({LIB_PATH}); run python -m paged_fp8_mqa_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        for name, (args, res) in SIGNATURES.items():
            fn = getattr(L, name)
            fn.argtypes = args
            fn.restype = res
        _lib = L
    return _lib


def padded_seq_len(max_seq_len: int) -> int:
    return int(lib().pmqa_padded_seq_len(int(max_seq_len)))


def min_block_table_width(seq_len: int, block_size: int) -> int:
    return int(lib().pmqa_min_block_table_width(int(seq_len), int(block_size)))


_WHICH = {"logits": 0, "indexer_topk": 1, "fused": 2}


def workspace_bytes(which: str, batch_size: int, next_n: int, max_context: int) -> int:
    """Workspace bytes of entry point `which` ("indexer_topk" or "fused")."""
    return int(lib().pmqa_workspace_bytes(_WHICH[which], int(batch_size), int(next_n), int(max_context)))


def make_workspace(which: str, batch_size: int, next_n: int, max_context: int, device="cuda"):
    """A zeroed workspace for the finish stage of entry point `which`; reuse it
    for later calls (the library keeps state in it) and do not share it between
    concurrent calls."""
    import torch
    n = workspace_bytes(which, batch_size, next_n, max_context)
    return torch.zeros(n, dtype=torch.uint8, device=device)


def keys_per_cta(which: str) -> int:
    return int(lib().pmqa_keys_per_cta(_WHICH[which]))


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, where):
    if status != 0:
        raise PmqaError(status, where)


def _paged(q, kv_fused, weights, block_tables, seq_lens, block_size):
    """Pointers and sizes of the paged inputs (pages' shapes accepted)."""
    B, nn, H, D = q.shape
    if kv_fused.dim() == 4:
        bs = kv_fused.shape[1]
    else:
        if block_size is None:
            raise ValueError("block_size is needed for a 2-D kv_fused")
        bs = block_size
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be 2-D with contiguous rows")
    if not q.is_contiguous() or not weights.is_contiguous() or not kv_fused.is_contiguous():
        raise ValueError("q, weights and kv_fused must be contiguous")
    return [_ptr(q), _ptr(kv_fused), _ptr(weights), _ptr(block_tables), block_tables.stride(0),
            block_tables.shape[1], _ptr(seq_lens), seq_lens.stride(0), B, nn, H, D, bs,
            kv_fused.shape[0]], B, nn


DTYPE_F32, DTYPE_F16, DTYPE_BF16 = 0, 1, 2  # pmqa_dtype


def _dtype_code(dt):
    import torch
    codes = {torch.float32: DTYPE_F32, torch.float16: DTYPE_F16, torch.bfloat16: DTYPE_BF16}
    if dt not in codes:
        raise ValueError(f"unsupported dtype {dt}")
    return codes[dt]


def mqa_logits(q, kv_fused, weights, block_tables, seq_lens, max_seq_len, out=None, block_size=None,
               stream=None, output_dtype=None, epi_dtype=None, acc_dtype=None):
    """FP8 paged MQA logits; returns the [B*next_n, max_seq_len] view of `out`.

    output_dtype (torch.float32 or torch.float16), epi_dtype and acc_dtype
    (torch.float32 or torch.float16) select pmqa_mqa_logits_typed; all three
    float32 (the default) is pmqa_mqa_logits."""
    import torch
    args, B, nn = _paged(q, kv_fused, weights, block_tables, seq_lens, block_size)
    odt = torch.float32 if output_dtype is None else output_dtype
    codes = [_dtype_code(odt), _dtype_code(epi_dtype or torch.float32), _dtype_code(acc_dtype or torch.float32)]
    if out is None:
        out = torch.empty(B * nn, padded_seq_len(max_seq_len), dtype=odt, device=q.device)
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    if out.dtype != odt:
        raise ValueError(f"out is {out.dtype}, output_dtype is {odt}")
    if codes == [DTYPE_F32] * 3:
        _check(lib().pmqa_mqa_logits(*args, int(max_seq_len), _ptr(out), out.stride(0), _stream(stream)),
               "pmqa_mqa_logits")
    else:
        _check(lib().pmqa_mqa_logits_typed(*args, int(max_seq_len), _ptr(out), out.stride(0), *codes,
                                           _stream(stream)), "pmqa_mqa_logits_typed")
    return out[: B * nn, :max_seq_len]


def fp4_mqa_logits(q, q_sf, kv_fused, weights, block_tables, seq_lens, max_seq_len, out=None, sf_vec_size=32,
                   output_dtype=None, epi_dtype=None, is_kv_sf_interleaved=False, block_size=None, stream=None):
    """MXFP4 paged MQA logits; returns the [B*next_n, max_seq_len] view of `out`.

    q uint8 [B, next_n, H, head_dim/2], q_sf int32 [B, next_n, H], kv_fused
    uint8 [num_blocks, block_size, 1, head_dim/2 + 4] (or 2-D with block_size);
    output_dtype torch.bfloat16 (default), float32 or float16; epi_dtype
    torch.float32 (default), float16 or bfloat16."""
    import torch
    B, nn, H, half = q.shape
    if kv_fused.dim() == 4:
        bs = kv_fused.shape[1]
    else:
        if block_size is None:
            raise ValueError("block_size is needed for a 2-D kv_fused")
        bs = block_size
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be 2-D with contiguous rows")
    for name, t in (("q", q), ("q_sf", q_sf), ("weights", weights), ("kv_fused", kv_fused)):
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    odt = torch.bfloat16 if output_dtype is None else output_dtype
    edt = torch.float32 if epi_dtype is None else epi_dtype
    if out is None:
        out = torch.empty(B * nn, padded_seq_len(max_seq_len), dtype=odt, device=q.device)
    if out.stride(1) != 1:
        raise ValueError("out rows must be contiguous")
    if out.dtype != odt:
        raise ValueError(f"out is {out.dtype}, output_dtype is {odt}")
    _check(lib().pmqa_fp4_mqa_logits(_ptr(q), _ptr(q_sf), _ptr(kv_fused), _ptr(weights), _ptr(block_tables),
                                     block_tables.stride(0), block_tables.shape[1], _ptr(seq_lens),
                                     seq_lens.stride(0), B, nn, H, 2 * half, bs, kv_fused.shape[0],
                                     int(max_seq_len), int(sf_vec_size), 1 if is_kv_sf_interleaved else 0,
                                     _ptr(out), out.stride(0), _dtype_code(odt), _dtype_code(edt),
                                     _stream(stream)), "pmqa_fp4_mqa_logits")
    return out[: B * nn, :max_seq_len]


def _select_out(thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx, workspace):
    nbytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return [_ptr(thresholds), _ptr(counters), _ptr(candidates), int(capacity), int(top_k),
            _ptr(arrivals), _ptr(ranges), _ptr(topk_idx), _ptr(workspace), nbytes]


def indexer_topk(logits, seq_lens, next_n, max_context, thresholds, counters, candidates, capacity, top_k,
                 arrivals=None, ranges=None, topk_idx=None, workspace=None, stream=None):
    """Threshold select over a logits matrix (rows contiguous).  With arrivals,
    pass a workspace from make_workspace()."""
    if logits.stride(1) != 1:
        raise ValueError("logits rows must be contiguous")
    B = seq_lens.shape[0]
    _check(lib().pmqa_indexer_topk(_ptr(logits), logits.stride(0), _ptr(seq_lens), seq_lens.stride(0), B,
                                   int(next_n), int(max_context),
                                   *_select_out(thresholds, counters, candidates, capacity, top_k, arrivals,
                                                ranges, topk_idx, workspace), _stream(stream)),
           "pmqa_indexer_topk")


def fused_logits_select(q, kv_fused, weights, block_tables, seq_lens, max_context, thresholds, counters,
                        candidates, capacity, top_k, arrivals=None, ranges=None, topk_idx=None,
                        workspace=None, block_size=None, stream=None):
    """Logits and select in one launch (no score matrix).  With arrivals, pass
    a workspace from make_workspace()."""
    args, B, nn = _paged(q, kv_fused, weights, block_tables, seq_lens, block_size)
    _check(lib().pmqa_fused_logits_select(*args, int(max_context),
                                          *_select_out(thresholds, counters, candidates, capacity, top_k,
                                                       arrivals, ranges, topk_idx, workspace), _stream(stream)),
           "pmqa_fused_logits_select")


def fused_logits_select_noalloc(q, kv_fused, weights, block_tables, seq_lens, max_context, thresholds, counters,
                                candidates, capacity, top_k, arrivals=None, ranges=None, topk_idx=None,
                                block_size=None, stream=None):
    """fused_logits_select with the library's static scratch as its workspace
    (nothing is allocated; calls that overlap on one device race)."""
    args, B, nn = _paged(q, kv_fused, weights, block_tables, seq_lens, block_size)
    out = _select_out(thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx, None)[:-2]
    _check(lib().pmqa_fused_logits_select_noalloc(*args, int(max_context), *out, _stream(stream)),
           "pmqa_fused_logits_select_noalloc")


def prefill_select(q, kv_fused, weights, block_tables, tile_requests, row_ends, tile_rows, max_context, thresholds,
                   counters, candidates, capacity, top_k, arrivals=None, ranges=None, topk_idx=None, workspace=None,
                   block_size=None, stream=None):
    """The fused select over prefill-shaped rows: q [rows, H, D] (or [tiles,
    tile_rows, H, D]), tile i's rows on request tile_requests[i], row r seeing
    keys below row_ends[r].  With arrivals ([tiles]), pass a workspace from
    make_workspace("fused", tiles, tile_rows, max_context)."""
    if q.dim() == 4:
        q = q.reshape(-1, q.shape[2], q.shape[3])
    R, H, D = q.shape
    if kv_fused.dim() == 4:
        bs = kv_fused.shape[1]
    else:
        if block_size is None:
            raise ValueError("block_size is needed for a 2-D kv_fused")
        bs = block_size
    if block_tables.dim() != 2 or block_tables.stride(1) != 1:
        raise ValueError("block_tables must be 2-D with contiguous rows")
    if not q.is_contiguous() or not weights.is_contiguous() or not kv_fused.is_contiguous():
        raise ValueError("q, weights and kv_fused must be contiguous")
    if not tile_requests.is_contiguous() or not row_ends.is_contiguous():
        raise ValueError("tile_requests and row_ends must be contiguous")
    T = int(tile_rows)
    if T < 1 or R % T:
        raise ValueError("rows must be a multiple of tile_rows")
    tiles = R // T
    if tile_requests.numel() != tiles or row_ends.numel() != R:
        raise ValueError("tile_requests must hold one entry per tile and row_ends one per row")
    args = [_ptr(q), _ptr(kv_fused), _ptr(weights), _ptr(block_tables), block_tables.stride(0),
            block_tables.shape[1], block_tables.shape[0], _ptr(tile_requests), _ptr(row_ends), tiles, T, H, D, bs,
            kv_fused.shape[0], int(max_context)]
    _check(lib().pmqa_prefill_select(*args, *_select_out(thresholds, counters, candidates, capacity, top_k,
                                                        arrivals, ranges, topk_idx, workspace), _stream(stream)),
           "pmqa_prefill_select")
