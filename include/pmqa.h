/*
 * pmqa.h -- C ABI of libpmqa, paged FP8 MQA logits and threshold Top-k select
 * for AMD Instinct MI355X (gfx950).
 *
 * Operations (definitions on the pages cited per entry point):
 *   pmqa_mqa_logits           logits[b*next_n+t, p] =
 *                               s_p * sum_h w[b*next_n+t, h] * relu(q[b,t,h,:] . k_p)
 *   pmqa_mqa_logits_typed     the same with float16 accumulator, epilogue or
 *                             output options
 *   pmqa_fp4_mqa_logits       the logits of an MXFP4 pool (E2M1 values, UE8M0
 *                             scales per 32 elements, no per-token scale)
 *   pmqa_indexer_topk         one-pass threshold select over a logits matrix,
 *                             with last-CTA radix-select repair and Top-k finalize
 *   pmqa_fused_logits_select  both in one pass over the KV pages; no score
 *                             matrix is written
 *
 * Conventions shared by every entry point:
 *   - All buffer pointers are DEVICE pointers on the device that owns `stream`
 *     (a hipStream_t; NULL is the null stream).  The caller owns every buffer:
 *     the library never allocates, frees or synchronises the host, and each
 *     call is one kernel launch on `stream` with no host round trip (so it can
 *     be captured in a HIP graph).  A select call whose workspace was last laid
 *     out for another batch_size or next_n first launches one small kernel that
 *     clears the workspace's state words.
 *   - Rows: R = batch_size * next_n, row r = b*next_n + t pairs with q[b, t].
 *     Row r sees KV positions 0 .. e_r - 1 with e_r = seq_lens[b] - next_n + t + 1
 *     (at least 0): slot t = next_n-1 is the newest draft position and sees the
 *     whole sequence (page "flashinfer.attn_scores", Note and Returns).
 *   - Arguments the host can check are checked before anything is launched and
 *     a status other than PMQA_OK is returned with nothing written.
 *   - Device-content preconditions are the caller's: every seq_lens[b] at most
 *     max_seq_len (max_context for the select calls), block table row b valid
 *     for its first ceil(seq_lens[b]/block_size) entries with ids in
 *     [0, num_blocks), counters zeroed, arrivals zeroed.  A violation is
 *     undefined behaviour (an out-of-bounds read or write), as on the pages
 *     (fp8_paged_mqa_logits, block_tables and max_seq_len).  With the
 *     environment variable PMQA_VALIDATE=1 the library copies those buffers to
 *     the host and returns PMQA_ERR_CONTENT on a violation; that check
 *     synchronises the stream and is skipped while the stream is capturing.
 *   - Launch failures return PMQA_ERR_LAUNCH.
 *   - v1 kernels support num_heads == 64, head_dim == 128, next_n in 1..4 and
 *     block_size in {32, 64, 128}; other shapes return PMQA_ERR_UNSUPPORTED.
 */
#ifndef PMQA_H
#define PMQA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum pmqa_status {
  PMQA_OK = 0,
  PMQA_ERR_NULL = 1,        /* a required pointer is NULL (or an optional one is given without its partner) */
  PMQA_ERR_SHAPE = 2,       /* a size or count is out of range */
  PMQA_ERR_STRIDE = 3,      /* a stride is negative, too small, or rows would overlap */
  PMQA_ERR_UNSUPPORTED = 4, /* a shape the kernels are not built for */
  PMQA_ERR_ALIGN = 5,       /* a pointer is not aligned as its entry point requires */
  PMQA_ERR_OVERFLOW = 6,    /* an output offset would not fit the 32-bit range */
  PMQA_ERR_LAUNCH = 7,      /* the HIP launch failed (no device, bad stream, ...) */
  PMQA_ERR_CONTENT = 8,     /* PMQA_VALIDATE=1 found a device-content precondition violated */
  PMQA_ERR_SCRATCH = 9      /* the call needs more workspace than the library's static scratch holds */
} pmqa_status;

/* Static string naming a status; never NULL. */
const char* pmqa_status_string(int status);

/* Library version as major*10000 + minor*100 + patch. */
int32_t pmqa_version(void);

/* Minimum column count of a logits output buffer for max_seq_len: max_seq_len
 * rounded up to a multiple of 256 (the kernels store whole 64-column groups up
 * to round_up(seq_len, 64) and write those padding columns unconditionally).
 * 8000 -> 8192 as in the Example of page "flashinfer.attn_scores".  Returns -1
 * for a negative argument. */
int32_t pmqa_padded_seq_len(int32_t max_seq_len);

/* Minimum block-table width for a sequence length: ceil(seq_len / block_size)
 * (page "flashinfer.attn_scores", block_tables; 8000, 32 -> 250).  Returns -1
 * for a negative seq_len or a non-positive block_size. */
int32_t pmqa_min_block_table_width(int32_t seq_len, int32_t block_size);

/*
 * pmqa_mqa_logits -- FP8 paged MQA logits (page "flashinfer.attn_scores",
 * fp8_paged_mqa_logits: the formula and its parameters).
 *
 *   q            [batch_size, next_n, num_heads, head_dim] e4m3fn bytes,
 *                contiguous, 16-byte aligned.
 *   kv_fused     [num_blocks, block_size*(head_dim+4)] bytes, 16-byte aligned.
 *                Block j: bytes [0, block_size*head_dim) hold the e4m3 values
 *                token-major (token i at i*head_dim); bytes
 *                [block_size*head_dim, end) hold block_size little-endian f32
 *                per-token scales (token i's at block_size*head_dim + 4*i).
 *   weights      [batch_size*next_n, num_heads] f32, contiguous, 16-byte aligned.
 *   block_tables int32, row b at block_tables + b*block_table_stride, entries
 *                contiguous; block_table_stride >= 0 is free (a row-strided view
 *                is fine).  block_table_width is the number of columns (used by
 *                PMQA_VALIDATE only; the kernel never reads row b past
 *                ceil(seq_lens[b]/block_size) entries).
 *   seq_lens     int32 at seq_lens + b*seq_lens_stride (any stride >= 0).
 *   max_seq_len  >= every seq_lens[b]; sizes the output rows.
 *   out          f32, row r at out + r*out_stride, out_stride >=
 *                pmqa_padded_seq_len(max_seq_len), 4-byte aligned, and
 *                R*out_stride < 2^31.  Row r is written for columns
 *                [0, round_up(seq_lens[b], 64)) of every request with
 *                seq_lens[b] > 0; columns at or past e_r hold unspecified values
 *                (no mask is applied) and rows of requests with seq_lens[b] == 0
 *                are never written.
 */
pmqa_status pmqa_check_logits_args(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_seq_len,
    const float* out, int64_t out_stride);

pmqa_status pmqa_mqa_logits(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_seq_len,
    float* out, int64_t out_stride, void* stream);

/* Element types of pmqa_mqa_logits_typed's precision arguments. */
typedef enum pmqa_dtype {
  PMQA_DTYPE_F32 = 0,
  PMQA_DTYPE_F16 = 1,
  PMQA_DTYPE_BF16 = 2 /* MXFP4 logits only; no FP8 precision takes it */
} pmqa_dtype;

/*
 * pmqa_mqa_logits_typed -- pmqa_mqa_logits with the three precisions of page
 * "flashinfer.attn_scores", fp8_paged_mqa_logits (the formula block and the
 * parameters output_dtype, epi_dtype, acc_dtype, weights):
 *
 *   acc_dtype     each head's dot product q[b,t,h,:] . k_p.  PMQA_DTYPE_F32:
 *                 as pmqa_mqa_logits.  PMQA_DTYPE_F16: the float32 result of
 *                 the FP8 matrix instruction is rounded to float16 (nearest
 *                 even; past 65504 it becomes infinite), the hardware having no
 *                 FP8 instruction that accumulates in float16.
 *   epi_dtype     ReLU, the weight multiply, the head sum and the scale
 *                 multiply.  PMQA_DTYPE_F16: the dot product enters rounded to
 *                 float16 (so acc_dtype makes no difference), the weights and
 *                 the scale are rounded to float16, and every product and sum
 *                 is a float16 operation (packed, two heads at a time), which
 *                 overflows to infinity past 65504.
 *   output_dtype  the stored element: PMQA_DTYPE_F32 (4 bytes) or
 *                 PMQA_DTYPE_F16 (2 bytes, the epilogue's result rounded to
 *                 nearest even).
 *
 * PMQA_DTYPE_BF16, or any other value, for any of the three returns
 * PMQA_ERR_UNSUPPORTED.  `out` is an array of output_dtype elements, aligned to
 * one element; out_stride counts elements.  Everything else is as for
 * pmqa_mqa_logits, which equals this call with all three PMQA_DTYPE_F32.
 */
pmqa_status pmqa_check_logits_typed_args(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_seq_len,
    const void* out, int64_t out_stride, int32_t output_dtype, int32_t epi_dtype, int32_t acc_dtype);

pmqa_status pmqa_mqa_logits_typed(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_seq_len,
    void* out, int64_t out_stride, int32_t output_dtype, int32_t epi_dtype, int32_t acc_dtype,
    void* stream);

/*
 * pmqa_fp4_mqa_logits -- MXFP4 paged MQA logits (page "flashinfer.attn_scores",
 * fp4_paged_mqa_logits: the formula, its parameters, the kv_fused figure and
 * the Restrictions):
 *
 *   logits[b*next_n+t, p] = sum_h w[b*next_n+t, h] * relu(q^[b,t,h,:] . k^_p)
 *
 * with q^ and k^ the dequantised vectors (each element an E2M1 value times the
 * UE8M0 scale 2^(e-127) of its group of 32) and no per-token scale.
 *
 *   q            [batch_size, next_n, num_heads, head_dim/2] bytes, two E2M1
 *                values per byte (element 2m in the low nibble of byte m),
 *                contiguous, 16-byte aligned.
 *   q_sf         [batch_size, next_n, num_heads] int32, contiguous, 4-byte
 *                aligned: byte k (k-th least significant) is the UE8M0 scale
 *                of elements [32k, 32k+32) of that (row, head).
 *   kv_fused     [num_blocks, block_size*(head_dim/2 + head_dim/32)] bytes,
 *                16-byte aligned.  Block j: bytes [0, block_size*head_dim/2)
 *                hold the packed values token-major (token i at i*head_dim/2,
 *                same nibble rule as q); then block_size slots of 4 UE8M0 scale
 *                bytes (byte k for elements [32k, 32k+32)): slot i holds token
 *                i, or with kv_sf_interleaved != 0 slot k holds token
 *                (k % 4) * (block_size / 4) + k / 4.
 *   weights, block_tables, seq_lens, max_seq_len: as for pmqa_mqa_logits.
 *   sf_vec_size  must be 32.
 *   kv_sf_interleaved  0 or 1; 1 only with block_size 128.
 *   output_dtype PMQA_DTYPE_BF16 (the page's default), PMQA_DTYPE_F32 or
 *                PMQA_DTYPE_F16; `out` holds such elements, aligned to one,
 *                out_stride counts them (as for pmqa_mqa_logits_typed).
 *   epi_dtype    PMQA_DTYPE_F32, PMQA_DTYPE_F16 or PMQA_DTYPE_BF16: the
 *                precision of ReLU, the weight multiply and the head sum (each
 *                dot product, accumulated in float32 by the matrix
 *                instruction, is rounded to it first; the weights are rounded
 *                to it; every product and sum is rounded).
 *
 * Unsupported values (sf_vec_size != 32, interleaved scales with another block
 * size, another dtype) return PMQA_ERR_UNSUPPORTED.  Output rows, columns and
 * the empty-request rule are as for pmqa_mqa_logits.
 */
pmqa_status pmqa_check_fp4_logits_args(
    const uint8_t* q, const int32_t* q_sf, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_seq_len,
    int32_t sf_vec_size, int32_t kv_sf_interleaved,
    const void* out, int64_t out_stride, int32_t output_dtype, int32_t epi_dtype);

pmqa_status pmqa_fp4_mqa_logits(
    const uint8_t* q, const int32_t* q_sf, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_seq_len,
    int32_t sf_vec_size, int32_t kv_sf_interleaved,
    void* out, int64_t out_stride, int32_t output_dtype, int32_t epi_dtype, void* stream);

/*
 * Select arguments shared by pmqa_indexer_topk and pmqa_fused_logits_select
 * (page "flashinfer.sdsa.indexer_threshold_select", the description and the
 * parameters thresholds, counters, candidates, max_context, top_k, arrivals,
 * ranges).  A query tile is one request: its next_n rows.
 *
 *   max_context  the most keys a row sees (>= every seq_lens[b]); sizes the grid.
 *   thresholds   [R] f32, in/out.  A key p < e_r of row r scoring above
 *                thresholds[r] is a candidate; one scoring neither above nor
 *                below it (equal, or NaN) is a tie.  A repaired row gets its new
 *                threshold: its min(e_r, top_k)-th largest score.
 *   counters     [R, 2] int32, zeroed by the caller, 8-byte aligned: the row's
 *                candidate and tie counts (all of them, also past the slots).
 *   candidates   [R, top_k + capacity, 2] int32, 8-byte aligned, output.  The
 *                n-th candidate goes to slot top_k + n if n < capacity, the n-th
 *                tie to slot top_k - 1 - n if n < top_k; each slot holds (key
 *                index, score bits).  Slot order within a class is unspecified.
 *                Stored score bits: for a candidate s - t when t > 0 and s <= 2t
 *                (exact, and order-keeping), else s; for a tie s - t.
 *   capacity     >= 0 candidate slots per row.
 *   top_k        >= 1; also the number of tie slots.
 *   arrivals     [batch_size] int32 or NULL, zeroed by the caller once and
 *                left zeroed by every call: the per-tile arrival counters.  A
 *                tile is one request's next_n rows.  Each CTA that scores a
 *                share of a tile's keys counts itself on arrivals[b] once its
 *                candidate and tie stores are complete; the CTA that completes
 *                the count sets it back to zero and finishes the tile in the
 *                same launch.  Finishing means: every row that does not fit
 *                (n_cand > capacity or n_cand + min(n_tie, top_k) <
 *                min(e_r, top_k)) is selected again at its radix-selected
 *                min(e_r, top_k)-th largest score (with capacity >= top_k - 1
 *                every row then fits), and ranges and topk_idx are written.  A
 *                repair too large for one CTA becomes items that the launch's
 *                other CTAs claim.  With NULL no repair runs and
 *                ranges/topk_idx must be NULL.
 *   ranges       [2, R] int32, required with arrivals, output: slots
 *                [ranges[0][r], ranges[1][r]) hold the row's ties and candidates
 *                (ranges[0][r] = top_k - min(n_tie, top_k),
 *                 ranges[1][r] = top_k + min(n_cand, capacity)).
 *   topk_idx     [R, top_k] int32 or NULL (needs arrivals and capacity >=
 *                top_k - 1), output: the row's exact Top-min(e_r, top_k) key
 *                indices in unspecified order, then -1 entries.  Among keys
 *                scoring exactly the k-th largest score any may be chosen.
 *   workspace    pmqa_workspace_bytes(which, batch_size, next_n, max_context)
 *                bytes of device memory, 8-byte aligned, required with arrivals
 *                (NULL without).  Zeroed by the caller before its first use;
 *                after that the library keeps state in it from call to call, so
 *                the caller leaves it alone (zeroing it again is harmless).
 *                Every call leaves its state words (tile jobs, row states,
 *                radix histograms) back at zero; a call laid out for another
 *                batch_size or next_n clears them first (above).  It also holds
 *                per row a bucket of keys at the k-th digit, the candidates past
 *                capacity (up to 8192 per row, so a row with too many
 *                candidates is re-selected from its stored pairs without a
 *                sweep), and the keys in a narrow band just below the
 *                threshold (up to 4096 per row, for rows a few keys short).
 *                The fused select adds a score buffer of round_up(max_context,
 *                64) floats per row, written only for rows whose repair sweeps
 *                their keys again: no score matrix is written for fitting rows.
 *                Calls that share a workspace must not run concurrently.
 */

/* Bytes of the finish-stage workspace of entry point `which` (1
 * pmqa_indexer_topk, 2 pmqa_fused_logits_select) for batch_size requests of
 * next_n rows and max_context keys: 64 bytes per tile, about 256 KB of state
 * per row, plus for the fused select a score buffer of round_up(max_context,
 * 64) floats per row.  Returns 0 for an unknown `which` or a negative size. */
size_t pmqa_workspace_bytes(int32_t which, int32_t batch_size, int32_t next_n, int32_t max_context);

pmqa_status pmqa_check_select_args(
    const float* logits, int64_t logits_stride,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t max_context,
    const float* thresholds, const int32_t* counters, const int32_t* candidates,
    int32_t capacity, int32_t top_k,
    const int32_t* arrivals, const int32_t* ranges, const int32_t* topk_idx,
    const void* workspace, size_t workspace_bytes);

/*
 * pmqa_indexer_topk -- the select over a logits matrix (row r at
 * logits + r*logits_stride, 4-byte aligned, logits_stride >= max_context),
 * e.g. the output of pmqa_mqa_logits.  Columns p < seq_lens[b] of request b's
 * rows may be read; only those below e_r are selected.  The repair re-reads the
 * logits rows it repairs.
 */
pmqa_status pmqa_indexer_topk(
    const float* logits, int64_t logits_stride,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t max_context,
    float* thresholds, int32_t* counters, int32_t* candidates,
    int32_t capacity, int32_t top_k,
    int32_t* arrivals, int32_t* ranges, int32_t* topk_idx,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pmqa_fused_logits_select -- logits and select in one launch: each CTA scores
 * its share of a request's keys exactly as pmqa_mqa_logits does (same
 * arithmetic, bit for bit) and selects them without storing the scores; a
 * repair that sweeps a tile's keys again recomputes their scores.  Arguments as in
 * pmqa_mqa_logits (minus out/out_stride/max_seq_len) and the select arguments
 * above; block_table_width >= ceil(max_context / block_size) (the table has
 * to reach max_context keys: page "flashinfer.sdsa.indexer_threshold_select",
 * Parameters: max_context).
 */
pmqa_status pmqa_check_fused_args(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_context,
    const float* thresholds, const int32_t* counters, const int32_t* candidates,
    int32_t capacity, int32_t top_k,
    const int32_t* arrivals, const int32_t* ranges, const int32_t* topk_idx,
    const void* workspace, size_t workspace_bytes);

pmqa_status pmqa_fused_logits_select(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_context,
    float* thresholds, int32_t* counters, int32_t* candidates,
    int32_t capacity, int32_t top_k,
    int32_t* arrivals, int32_t* ranges, int32_t* topk_idx,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pmqa_prefill_select -- the fused select over prefill-shaped rows (page
 * "flashinfer.sdsa.indexer_threshold_select", the signature and the
 * parameters row_ends and tile_requests): rows come in query tiles of
 * tile_rows rows that all belong to one request, each row has its own key
 * end, and several tiles may share a request (the causal rows of a prompt).
 * The pages build 128-row tiles for their hardware's matrix tile; here a tile
 * is the 1 to 4 rows whose scores share one pass over the request's keys, as
 * the next_n rows of a decode request do (the same kernels).
 *
 *   q            [num_tiles*tile_rows, num_heads, head_dim] e4m3fn bytes, row
 *                r = tile*tile_rows + t, contiguous, 16-byte aligned.
 *   weights      [num_tiles*tile_rows, num_heads] f32.
 *   block_tables int32 [num_requests rows of block_table_stride], as in
 *                pmqa_mqa_logits; block_table_width >= ceil(max_context /
 *                block_size).
 *   tile_requests int32 [num_tiles]: tile i's request, a row of block_tables.
 *   row_ends     int32 [num_tiles*tile_rows]: row r sees keys p < row_ends[r]
 *                of its tile's request (0 <= row_ends[r] <= max_context; a row
 *                with 0 sees nothing).  A tile streams keys up to its largest
 *                row end, so that many of its request's keys must be valid.
 *   Row r's score at key p is the pmqa_mqa_logits formula with q[r] and
 *   weights[r]; the select arguments are those of pmqa_fused_logits_select
 *   with e_r = row_ends[r], batch_size = num_tiles and next_n = tile_rows
 *   (arrivals [num_tiles]; workspace pmqa_workspace_bytes(2, num_tiles,
 *   tile_rows, max_context) bytes).
 *   Errors as in pmqa_fused_logits_select; PMQA_VALIDATE=1 also checks
 *   row_ends and tile_requests against max_context and num_requests.
 */
pmqa_status pmqa_check_prefill_args(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width, int32_t num_requests,
    const int32_t* tile_requests, const int32_t* row_ends, int32_t num_tiles, int32_t tile_rows,
    int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t max_context,
    const float* thresholds, const int32_t* counters, const int32_t* candidates,
    int32_t capacity, int32_t top_k,
    const int32_t* arrivals, const int32_t* ranges, const int32_t* topk_idx,
    const void* workspace, size_t workspace_bytes);

pmqa_status pmqa_prefill_select(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width, int32_t num_requests,
    const int32_t* tile_requests, const int32_t* row_ends, int32_t num_tiles, int32_t tile_rows,
    int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks, int32_t max_context,
    float* thresholds, int32_t* counters, int32_t* candidates,
    int32_t capacity, int32_t top_k,
    int32_t* arrivals, int32_t* ranges, int32_t* topk_idx,
    void* workspace, size_t workspace_bytes, void* stream);

/*
 * pmqa_fused_logits_select_noalloc -- pmqa_fused_logits_select for callers
 * that cannot allocate device memory (code under HIP graph capture, tight
 * serving loops, harnesses that forbid hipMalloc): the same kernels, with the
 * finish-stage workspace taken from a static device array of
 * PMQA_NOALLOC_SCRATCH_BYTES bytes that the library holds on every device it
 * runs on until the process ends.  The call itself allocates nothing.
 *
 *   Arguments and outputs as in pmqa_fused_logits_select, without workspace
 *   and workspace_bytes.  The caller still owns and passes every input and
 *   output buffer (thresholds, counters and arrivals zeroed as there).
 *   PMQA_ERR_SCRATCH: with arrivals, pmqa_workspace_bytes(2, batch_size,
 *   next_n, max_context) exceeds PMQA_NOALLOC_SCRATCH_BYTES (e.g. 32 requests
 *   of next_n 4 over 65536 keys need about 64 MiB and fit; 64 such
 *   requests do not);
 *   nothing is launched.  The scratch is cleared by the library on its first
 *   use on a device and whenever a call lays it out for another batch_size or
 *   next_n (one extra fill kernel on the stream); otherwise each call leaves
 *   it as the next call needs it.  All calls on one device share its scratch:
 *   calls that overlap on a device (two streams, two threads) race and give
 *   undefined results.  PMQA_VALIDATE is not honoured here (its check copies
 *   to host memory).
 */
#define PMQA_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

pmqa_status pmqa_fused_logits_select_noalloc(
    const uint8_t* q, const uint8_t* kv_fused, const float* weights,
    const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
    const int32_t* seq_lens, int64_t seq_lens_stride,
    int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
    int32_t block_size, int64_t num_blocks, int32_t max_context,
    float* thresholds, int32_t* counters, int32_t* candidates,
    int32_t capacity, int32_t top_k,
    int32_t* arrivals, int32_t* ranges, int32_t* topk_idx, void* stream);

/* Keys scored per CTA by the logits/fused kernels and selected per CTA by the
 * indexer_topk kernel (at most batch_size x ceil(max_context / keys) CTAs). */
int32_t pmqa_keys_per_cta(int32_t which /* 0 logits, 1 indexer_topk, 2 fused */);

#ifdef __cplusplus
}
#endif

#endif /* PMQA_H */
