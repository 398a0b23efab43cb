// Internal declarations shared by the host-side argument checks and the HIP
// translation unit.  Not part of the public ABI.
#pragma once
#include <cstdint>

#include "pmqa.h"

namespace pmqa {

constexpr int kHeads = 64;          // num_heads the kernels are built for
constexpr int kDim = 128;           // head_dim the kernels are built for
constexpr int kMaxNextN = 4;
constexpr int kLogitsKeysPerCta = 1024;
constexpr int kFusedKeysPerCta = 1024;
constexpr int kSelectKeysPerCta = 4096;
constexpr int kOutColumnGranule = 256;  // padded_seq_len rounding
constexpr int kRadixBins = 2048;        // radix digits: 10 + 11 + 11 bits from the top
constexpr int kHistCopies = 4;          // repair workspace: copies of a row's radix histogram
constexpr int kFinalizeLds = 4096;      // keys a CTA keeps in LDS for a final radix select
constexpr int kBucketPairs = 16384;     // repair workspace: a row's bucket of keys at the k-th digit
constexpr int kOverflowPairs = 8192;    // repair workspace: a row's candidates past its capacity
constexpr int kNearPairs = 4096;        // repair workspace: a row's keys just below its threshold
constexpr uint32_t kNearBand = 1u << 15;  // the band below a threshold, in radix-key units (about 2^-8 of it)
constexpr int kJobWords = 16;           // repair workspace: words per tile job
constexpr int kRowWords = 16;           // repair workspace: words per row state
constexpr int kRescoreItemKeys = 2048;  // granule of the keys per repair item recomputed from the KV pages
constexpr int kRescoreItems = 16;       // repair items a request's keys are recomputed in (about)
constexpr int kSelectItemKeys = 4096;   // keys per repair item read back as scores

constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Floats per row of the fused repair's score buffer (256-byte rows).
constexpr int64_t score_stride(int64_t max_context) { return ceil_div(max_context, 64) * 64; }

// Workspace of the select entry points, in 32-bit words and in this order:
// one job per tile, then per row -- each kind in an array of its own -- the
// state words, kHistCopies radix histograms, the bucket of keys at the k-th
// digit, the candidates past the capacity (kOverflowPairs pairs) and the keys
// just below the threshold (kNearPairs pairs); the fused
// select adds a score row of score_stride(max_context) floats per row, written
// only for rows whose repair sweeps their keys again.  A job's claim words are
// written by the job's publisher; every other word is set up before it is read
// in the call that reads it, so the workspace needs zeroing only before its
// first use.
struct WsLayout {
  int64_t jobs, row_state, hist, bucket, overflow, near, scores, end;
};
constexpr WsLayout workspace_layout(int64_t batch, int64_t rows, int64_t max_context, bool fused) {
  WsLayout l{};
  l.jobs = 0;
  l.row_state = l.jobs + kJobWords * batch;
  l.hist = l.row_state + kRowWords * rows;
  l.bucket = l.hist + static_cast<int64_t>(kHistCopies) * kRadixBins * rows;
  l.overflow = l.bucket + 2 * static_cast<int64_t>(kBucketPairs) * rows;
  l.near = l.overflow + 2 * static_cast<int64_t>(kOverflowPairs) * rows;
  l.scores = l.near + 2 * static_cast<int64_t>(kNearPairs) * rows;
  l.end = l.scores + (fused ? rows * score_stride(max_context) : 0);
  return l;
}
constexpr int64_t workspace_words(int64_t batch, int64_t rows, int64_t max_context, bool fused) {
  return workspace_layout(batch, rows, max_context, fused).end;
}

}  // namespace pmqa
