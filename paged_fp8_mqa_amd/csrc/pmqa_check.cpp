// Host-side argument checks and size helpers of libpmqa.  Pure C++: nothing
// here touches a device, so every error path can be exercised without a GPU.
#include <cstdint>

#include "pmqa_internal.h"

using namespace pmqa;

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

bool supported_block_size(int32_t bs) { return bs == 32 || bs == 64 || bs == 128; }

// Checks common to the two entry points that read the paged KV pool.
pmqa_status check_paged_inputs(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                               const int32_t* block_tables, int64_t block_table_stride,
                               int32_t block_table_width, const int32_t* seq_lens,
                               int64_t seq_lens_stride, int32_t batch_size, int32_t next_n,
                               int32_t num_heads, int32_t head_dim, int32_t block_size,
                               int64_t num_blocks) {
  if (batch_size < 0) return PMQA_ERR_SHAPE;
  if (next_n < 1 || next_n > kMaxNextN) return PMQA_ERR_UNSUPPORTED;
  if (num_heads != kHeads || head_dim != kDim) return PMQA_ERR_UNSUPPORTED;
  if (!supported_block_size(block_size)) return PMQA_ERR_UNSUPPORTED;
  if (batch_size == 0) return PMQA_OK;
  if (!q || !kv_fused || !weights || !block_tables || !seq_lens) return PMQA_ERR_NULL;
  if (num_blocks < 1 || block_table_width < 1) return PMQA_ERR_SHAPE;
  if (block_table_stride < 0 || seq_lens_stride < 0) return PMQA_ERR_STRIDE;
  if (!aligned(q, 16) || !aligned(kv_fused, 16) || !aligned(weights, 16)) return PMQA_ERR_ALIGN;
  if (!aligned(block_tables, 4) || !aligned(seq_lens, 4)) return PMQA_ERR_ALIGN;
  return PMQA_OK;
}

pmqa_status check_select_outputs(int64_t batch, int64_t rows, int32_t max_context, bool fused,
                                 const float* thresholds, const int32_t* counters,
                                 const int32_t* candidates, int32_t capacity, int32_t top_k,
                                 const int32_t* arrivals, const int32_t* ranges,
                                 const int32_t* topk_idx, const void* workspace, size_t workspace_bytes) {
  if (top_k < 1 || capacity < 0) return PMQA_ERR_SHAPE;
  if (static_cast<int64_t>(top_k) + capacity > INT32_MAX / 2) return PMQA_ERR_OVERFLOW;
  if (rows == 0) return PMQA_OK;
  if (!thresholds || !counters || !candidates) return PMQA_ERR_NULL;
  if (arrivals && (!ranges || !workspace)) return PMQA_ERR_NULL;
  if (!arrivals && (ranges || topk_idx)) return PMQA_ERR_NULL;
  if (topk_idx && capacity < top_k - 1) return PMQA_ERR_SHAPE;
  if (!aligned(thresholds, 4) || !aligned(counters, 8) || !aligned(candidates, 8)) return PMQA_ERR_ALIGN;
  if ((arrivals && !aligned(arrivals, 4)) || (ranges && !aligned(ranges, 4)) ||
      (topk_idx && !aligned(topk_idx, 4)))
    return PMQA_ERR_ALIGN;
  if (workspace) {
    if (!arrivals) return PMQA_ERR_NULL;
    if (!aligned(workspace, 8)) return PMQA_ERR_ALIGN;
    if (static_cast<int64_t>(workspace_bytes) < 4 * workspace_words(batch, rows, max_context, fused))
      return PMQA_ERR_SHAPE;
  }
  return PMQA_OK;
}

}  // namespace

extern "C" {

const char* pmqa_status_string(int status) {
  switch (status) {
    case PMQA_OK: return "PMQA_OK";
    case PMQA_ERR_NULL: return "PMQA_ERR_NULL: a required pointer is NULL";
    case PMQA_ERR_SHAPE: return "PMQA_ERR_SHAPE: a size or count is out of range";
    case PMQA_ERR_STRIDE: return "PMQA_ERR_STRIDE: a stride is negative or too small";
    case PMQA_ERR_UNSUPPORTED: return "PMQA_ERR_UNSUPPORTED: shape not supported (num_heads 64, head_dim 128, next_n 1..4, block_size 32/64/128)";
    case PMQA_ERR_ALIGN: return "PMQA_ERR_ALIGN: a pointer is misaligned";
    case PMQA_ERR_OVERFLOW: return "PMQA_ERR_OVERFLOW: an output offset exceeds the 32-bit range";
    case PMQA_ERR_LAUNCH: return "PMQA_ERR_LAUNCH: the HIP launch failed";
    case PMQA_ERR_CONTENT: return "PMQA_ERR_CONTENT: PMQA_VALIDATE found a device-content precondition violated";
    case PMQA_ERR_SCRATCH: return "PMQA_ERR_SCRATCH: the call needs more workspace than the static scratch holds";
    default: return "PMQA: unknown status";
  }
}

int32_t pmqa_version(void) { return 10000; }

int32_t pmqa_padded_seq_len(int32_t max_seq_len) {
  if (max_seq_len < 0) return -1;
  int64_t v = ceil_div(max_seq_len, kOutColumnGranule) * kOutColumnGranule;
  return v > INT32_MAX ? -1 : static_cast<int32_t>(v);
}

int32_t pmqa_min_block_table_width(int32_t seq_len, int32_t block_size) {
  if (seq_len < 0 || block_size <= 0) return -1;
  return static_cast<int32_t>(ceil_div(seq_len, block_size));
}

size_t pmqa_workspace_bytes(int32_t which, int32_t batch_size, int32_t next_n, int32_t max_context) {
  if ((which != 1 && which != 2) || batch_size < 0 || next_n < 1 || next_n > kMaxNextN || max_context < 0) return 0;
  return static_cast<size_t>(
      4 * workspace_words(batch_size, static_cast<int64_t>(batch_size) * next_n, max_context, which == 2));
}

int32_t pmqa_keys_per_cta(int32_t which) {
  switch (which) {
    case 0: return kLogitsKeysPerCta;
    case 1: return kSelectKeysPerCta;
    case 2: return kFusedKeysPerCta;
    default: return -1;
  }
}

pmqa_status pmqa_check_logits_typed_args(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                         const int32_t* block_tables, int64_t block_table_stride,
                                         int32_t block_table_width, const int32_t* seq_lens,
                                         int64_t seq_lens_stride, int32_t batch_size, int32_t next_n,
                                         int32_t num_heads, int32_t head_dim, int32_t block_size,
                                         int64_t num_blocks, int32_t max_seq_len, const void* out,
                                         int64_t out_stride, int32_t output_dtype, int32_t epi_dtype,
                                         int32_t acc_dtype) {
  pmqa_status st = check_paged_inputs(q, kv_fused, weights, block_tables, block_table_stride,
                                      block_table_width, seq_lens, seq_lens_stride, batch_size,
                                      next_n, num_heads, head_dim, block_size, num_blocks);
  if (st != PMQA_OK) return st;
  // float32 and float16 for each precision (bfloat16 has no FP8 epilogue)
  for (const int32_t d : {output_dtype, epi_dtype, acc_dtype})
    if (d != PMQA_DTYPE_F32 && d != PMQA_DTYPE_F16) return PMQA_ERR_UNSUPPORTED;
  if (max_seq_len < 0) return PMQA_ERR_SHAPE;
  if (batch_size == 0) return PMQA_OK;
  if (!out) return PMQA_ERR_NULL;
  if (!aligned(out, output_dtype == PMQA_DTYPE_F16 ? 2 : 4)) return PMQA_ERR_ALIGN;
  if (out_stride < pmqa_padded_seq_len(max_seq_len) || out_stride < 0) return PMQA_ERR_STRIDE;
  const int64_t rows = static_cast<int64_t>(batch_size) * next_n;
  if (rows * out_stride >= (int64_t(1) << 31)) return PMQA_ERR_OVERFLOW;
  return PMQA_OK;
}

pmqa_status pmqa_check_fp4_logits_args(const uint8_t* q, const int32_t* q_sf, const uint8_t* kv_fused,
                                       const float* weights, const int32_t* block_tables,
                                       int64_t block_table_stride, int32_t block_table_width,
                                       const int32_t* seq_lens, int64_t seq_lens_stride, int32_t batch_size,
                                       int32_t next_n, int32_t num_heads, int32_t head_dim, int32_t block_size,
                                       int64_t num_blocks, int32_t max_seq_len, int32_t sf_vec_size,
                                       int32_t kv_sf_interleaved, const void* out, int64_t out_stride,
                                       int32_t output_dtype, int32_t epi_dtype) {
  pmqa_status st = check_paged_inputs(q, kv_fused, weights, block_tables, block_table_stride,
                                      block_table_width, seq_lens, seq_lens_stride, batch_size,
                                      next_n, num_heads, head_dim, block_size, num_blocks);
  if (st != PMQA_OK) return st;
  if (sf_vec_size != 32) return PMQA_ERR_UNSUPPORTED;
  if (kv_sf_interleaved != 0 && (kv_sf_interleaved != 1 || block_size != 128)) return PMQA_ERR_UNSUPPORTED;
  for (const int32_t d : {output_dtype, epi_dtype})
    if (d != PMQA_DTYPE_F32 && d != PMQA_DTYPE_F16 && d != PMQA_DTYPE_BF16) return PMQA_ERR_UNSUPPORTED;
  if (max_seq_len < 0) return PMQA_ERR_SHAPE;
  if (batch_size == 0) return PMQA_OK;
  if (!q_sf || !out) return PMQA_ERR_NULL;
  if (!aligned(q_sf, 4) || !aligned(out, output_dtype == PMQA_DTYPE_F32 ? 4 : 2)) return PMQA_ERR_ALIGN;
  if (out_stride < pmqa_padded_seq_len(max_seq_len) || out_stride < 0) return PMQA_ERR_STRIDE;
  const int64_t rows = static_cast<int64_t>(batch_size) * next_n;
  if (rows * out_stride >= (int64_t(1) << 31)) return PMQA_ERR_OVERFLOW;
  return PMQA_OK;
}

pmqa_status pmqa_check_logits_args(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                   const int32_t* block_tables, int64_t block_table_stride,
                                   int32_t block_table_width, const int32_t* seq_lens,
                                   int64_t seq_lens_stride, int32_t batch_size, int32_t next_n,
                                   int32_t num_heads, int32_t head_dim, int32_t block_size,
                                   int64_t num_blocks, int32_t max_seq_len, const float* out,
                                   int64_t out_stride) {
  return pmqa_check_logits_typed_args(q, kv_fused, weights, block_tables, block_table_stride, block_table_width,
                                      seq_lens, seq_lens_stride, batch_size, next_n, num_heads, head_dim,
                                      block_size, num_blocks, max_seq_len, out, out_stride, PMQA_DTYPE_F32,
                                      PMQA_DTYPE_F32, PMQA_DTYPE_F32);
}

pmqa_status pmqa_check_select_args(const float* logits, int64_t logits_stride,
                                   const int32_t* seq_lens, int64_t seq_lens_stride,
                                   int32_t batch_size, int32_t next_n, int32_t max_context,
                                   const float* thresholds, const int32_t* counters,
                                   const int32_t* candidates, int32_t capacity, int32_t top_k,
                                   const int32_t* arrivals, const int32_t* ranges,
                                   const int32_t* topk_idx, const void* workspace,
                                   size_t workspace_bytes) {
  if (batch_size < 0 || max_context < 0) return PMQA_ERR_SHAPE;
  if (next_n < 1 || next_n > kMaxNextN) return PMQA_ERR_UNSUPPORTED;
  const int64_t rows = static_cast<int64_t>(batch_size) * next_n;
  pmqa_status st = check_select_outputs(batch_size, rows, max_context, false, thresholds, counters, candidates,
                                        capacity, top_k, arrivals, ranges, topk_idx, workspace, workspace_bytes);
  if (st != PMQA_OK || rows == 0) return st;
  if (!logits || !seq_lens) return PMQA_ERR_NULL;
  if (!aligned(logits, 4) || !aligned(seq_lens, 4)) return PMQA_ERR_ALIGN;
  if (seq_lens_stride < 0 || logits_stride < max_context) return PMQA_ERR_STRIDE;
  if (rows * logits_stride >= (int64_t(1) << 31)) return PMQA_ERR_OVERFLOW;
  return PMQA_OK;
}

pmqa_status pmqa_check_fused_args(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                  const int32_t* block_tables, int64_t block_table_stride,
                                  int32_t block_table_width, const int32_t* seq_lens,
                                  int64_t seq_lens_stride, int32_t batch_size, int32_t next_n,
                                  int32_t num_heads, int32_t head_dim, int32_t block_size,
                                  int64_t num_blocks, int32_t max_context, const float* thresholds,
                                  const int32_t* counters, const int32_t* candidates,
                                  int32_t capacity, int32_t top_k, const int32_t* arrivals,
                                  const int32_t* ranges, const int32_t* topk_idx, const void* workspace,
                                  size_t workspace_bytes) {
  pmqa_status st = check_paged_inputs(q, kv_fused, weights, block_tables, block_table_stride,
                                      block_table_width, seq_lens, seq_lens_stride, batch_size,
                                      next_n, num_heads, head_dim, block_size, num_blocks);
  if (st != PMQA_OK) return st;
  if (max_context < 0) return PMQA_ERR_SHAPE;
  const int64_t rows = static_cast<int64_t>(batch_size) * next_n;
  st = check_select_outputs(batch_size, rows, max_context, true, thresholds, counters, candidates, capacity, top_k,
                            arrivals, ranges, topk_idx, workspace, workspace_bytes);
  if (st != PMQA_OK || rows == 0) return st;
  if (block_table_width < ceil_div(max_context, block_size)) return PMQA_ERR_SHAPE;
  return PMQA_OK;
}

pmqa_status pmqa_check_prefill_args(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                    const int32_t* block_tables, int64_t block_table_stride,
                                    int32_t block_table_width, int32_t num_requests,
                                    const int32_t* tile_requests, const int32_t* row_ends, int32_t num_tiles,
                                    int32_t tile_rows, int32_t num_heads, int32_t head_dim, int32_t block_size,
                                    int64_t num_blocks, int32_t max_context, const float* thresholds,
                                    const int32_t* counters, const int32_t* candidates, int32_t capacity,
                                    int32_t top_k, const int32_t* arrivals, const int32_t* ranges,
                                    const int32_t* topk_idx, const void* workspace, size_t workspace_bytes) {
  // the fused select's checks, with the row ends in place of the lengths
  pmqa_status st = pmqa_check_fused_args(q, kv_fused, weights, block_tables, block_table_stride, block_table_width,
                                         row_ends, 1, num_tiles, tile_rows, num_heads, head_dim, block_size,
                                         num_blocks, max_context, thresholds, counters, candidates, capacity, top_k,
                                         arrivals, ranges, topk_idx, workspace, workspace_bytes);
  if (st != PMQA_OK || num_tiles == 0) return st;
  if (num_requests < 1) return PMQA_ERR_SHAPE;
  if (!tile_requests) return PMQA_ERR_NULL;
  if (!aligned(tile_requests, 4)) return PMQA_ERR_ALIGN;
  return PMQA_OK;
}

}  // extern "C"
