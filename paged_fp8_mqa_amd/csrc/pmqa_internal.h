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

constexpr int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

}  // namespace pmqa
