"""CPU oracle for the paged FP8 MQA logits + threshold Top-k select path.

TEST INFRASTRUCTURE ONLY.  Only the tests, the package's smoke check and the
benchmark's CPU-baseline leg may import or run anything in this package.  The
product path (the HIP library and its Python binding) never calls it, and it
shares no code, tables or helpers with that path.

Everything here is plain NumPy in float64, written from the definitions on the
pages ("flashinfer.attn_scores" for the logits, and
"flashinfer.sdsa.indexer_threshold_select" for the select) and from the OCP
FP8 E4M3 and MX (E2M1, UE8M0) bit-field definitions.  Slow and obviously correct by design.

Parity pins (tests that tie it to something other than itself) live in
tests/test_oracle_*.py; every function's header says what pins it.  The only
function without an external pin is the slot score encoding (it follows a
reading of a garbled sentence); it is marked "parity unpinned" there.
"""
from .e4m3 import decode_e4m3, E4M3_TABLE  # noqa: F401
from .layout import (parse_block, gather_request, min_block_table_width,  # noqa: F401
                     padded_seq_len, region2_offset, block_bytes)
from .logits import paged_mqa_logits, request_scores, row_ends, row_tolerance  # noqa: F401
from .prefill import prefill_logits, prefill_tolerance  # noqa: F401
from .dtypes import mqa_logits_dtypes, round_f16  # noqa: F401
from .fp4 import fp4_paged_mqa_logits, round_bf16  # noqa: F401
from .select import (classify, fits, kth_largest, topk_indices, threshold_select,  # noqa: F401
                     encode_candidate, encode_tie, decode_slot, select_with_repair)
