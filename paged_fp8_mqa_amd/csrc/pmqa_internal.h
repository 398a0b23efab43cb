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
constexpr int kRadixBins = 2048;        // 11-bit radix digits: 11 + 11 + 10
constexpr int kHistCopies = 8;          // repair workspace: copies of a row's radix histogram
constexpr int kFinalizeLds = 4096;      // keys a CTA keeps in LDS for a final radix select
constexpr int kJobWords = 16;           // repair workspace: words per tile job
constexpr int kRowWords = 16;           // repair workspace: words per row state
constexpr int kDoneFlags = 64;          // repair workspace: copies of the end-of-phase-A flag
constexpr int kDoneFlagStride = 64;     // repair workspace: words between two copies (256 bytes)
constexpr int kRescoreItemKeys = 2048;  // keys per repair item recomputed from the KV pages
constexpr int kSelectItemKeys = 4096;   // keys per repair item read back as scores

constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// Repair job list: one word per tile, rounded up to keep the jobs 64-byte aligned.
constexpr int64_t job_list_words(int64_t batch) { return (batch + 15) / 16 * 16; }

// Floats per row of the fused repair's score buffer (256-byte rows).
constexpr int64_t score_stride(int64_t max_context) { return ceil_div(max_context, 64) * 64; }

// Repair workspace: a header, kDoneFlags copies of a flag, the job list, one
// job per tile, and per row its state, kHistCopies copies of a radix histogram
// and a bucket buffer of (index, score) pairs; this much is the finish stage's
// state (in words).
constexpr int64_t workspace_state_words(int64_t batch, int64_t rows) {
  return 16 + kDoneFlags * kDoneFlagStride + job_list_words(batch) + kJobWords * batch +
         (kRowWords + kHistCopies * kRadixBins + 2 * kFinalizeLds) * rows;
}

// The whole workspace in words: the fused select's repair adds a score buffer
// of score_stride(max_context) floats per row (the scores of a repaired row,
// computed once from the KV pages and read back by the later passes).
constexpr int64_t workspace_words(int64_t batch, int64_t rows, int64_t max_context, bool fused) {
  return workspace_state_words(batch, rows) + (fused ? rows * score_stride(max_context) : 0);
}

}  // namespace pmqa
