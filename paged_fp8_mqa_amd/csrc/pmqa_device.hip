// libpmqa device code and entry points: paged FP8 MQA logits, threshold Top-k
// select with a grid-wide radix-select repair, and the fused path (logits and
// select in one kernel, plus the repair kernel), for gfx950 (MI355X).
//
// What is computed (page "flashinfer.attn_scores", fp8_paged_mqa_logits):
//   E[r, p] = s_p * sum_h w[r, h] * relu(q[b, t, h, :] . k_p),   r = b*next_n + t
// and the select (page "flashinfer.sdsa.indexer_threshold_select"): keys above
// a row's threshold are candidates, keys neither above nor below it are ties,
// both counted and stored in the row's slots; rows that do not fit are
// selected again at their radix-selected k-th largest score.
//
// Work layout.  A CTA is 4 waves and covers a contiguous chunk of one
// request's key positions for all next_n rows.  A wave scores 64 keys at a time:
// four 16-key column tiles of the 16x16x128 FP8 MFMA, with the 64 heads as four
// 16-row tiles on the M axis and head_dim 128 as the MFMA's K.  Each lane loads
// its own B operand -- 32 bytes of one key -- straight from the page, so one
// wave's 64 lanes read one 2 KiB stretch of a page's value region per tile.
// The C layout leaves 16 heads of one key in each lane, so the ReLU and the
// weighted head sum run in-lane; a two-step reduce-scatter across the four lane
// groups then leaves lane l holding the score of key p0 + l, which is
// multiplied by that key's scale (region 2 of its page).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdint>
#include <cstdlib>
#include <map>
#include <mutex>
#include <type_traits>
#include <vector>

#include "pmqa_internal.h"

namespace pmqa {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v4i __attribute__((ext_vector_type(4)));
typedef float v4f __attribute__((ext_vector_type(4)));

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kGroupKeys = 64;                  // keys a wave scores per step
constexpr int kChunk = kGroupKeys * kWaves * 4;  // keys a CTA scores per chunk
constexpr int kStageInt4 = 512;  // a wave's KV staging area: 64 keys x 128 bytes
// Select kernel: a wave's pending candidates and ties per row (smaller for
// next_n >= 3, whose q operands take LDS instead).
template <int NT> constexpr int kWaveCand = NT >= 3 ? 64 : 256;
template <int NT> constexpr int kWaveTie = NT >= 3 ? 32 : 64;
constexpr int kFewExtra = 3;   // final select by value walk when at most this many keys are left out
// Phase A: the candidate pairs of a row that waves 1-3 preload (pair
// u * kPreThreads + tid - 64 in unit u of thread tid >= 64); wave 0 loads the
// fit test's words and counts the row, with no pair load ahead of its atomic.
constexpr int kPreUnits = 16;
constexpr int kPreThreads = kThreads - 64;
constexpr int kPreCap = kPreUnits * kPreThreads;

struct PagedArgs {
  const uint8_t* q;
  const uint8_t* kv;
  const float* w;
  const int32_t* bt;
  int64_t bt_stride;
  const int32_t* seq_lens;
  int64_t sl_stride;
  int32_t bs_shift;     // log2(block_size)
  int32_t block_bytes;  // block_size * (head_dim + 4)
  int32_t scale_off;    // block_size * head_dim: start of region 2
  int32_t batch;
  int32_t locate;       // balanced grid over all requests' keys (else per_request CTAs per request)
  int32_t per_request;
};

struct LogitsArgs {
  const float* logits;
  int64_t ld;
  const int32_t* seq_lens;
  int64_t sl_stride;
  int32_t batch;
  int32_t locate;
  int32_t per_request;
};

struct SelectArgs {
  float* thresholds;
  int32_t* counters;
  int32_t* candidates;
  int32_t* arrivals;
  int32_t* ranges;
  int32_t* topk_idx;
  uint32_t* ws;         // finish-stage workspace (with arrivals)
  int64_t ws_words;     // its size in 32-bit words
  float* scores;        // fused repair: the workspace's score buffer, row r at scores + r * score_ld
  int64_t score_ld;
  float* keep;          // fused select: the main pass writes every score here too (the score
                        // buffer, next_n >= 2), or null
  int32_t capacity;
  int32_t top_k;
  int32_t rows;
};

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Wavefront minimum (the device library's DPP reduction); every lane gets it.
extern "C" __device__ uint64_t __ockl_wfred_min_u64(uint64_t);

// s_waitcnt vmcnt(0): this wave's loads and stores have completed.
__device__ __forceinline__ void wait_vm_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Words shared between the CTAs of one kernel (on any XCD) are written with
// agent-scope atomic stores, which the storing XCD's L2 writes through, and
// read with agent-scope atomic loads.
__device__ __forceinline__ uint32_t ld_ag(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_ag64(const uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ v8i load32(const uint8_t* p) {
  const int4 lo = *reinterpret_cast<const int4*>(p);
  const int4 hi = *reinterpret_cast<const int4*>(p + 16);
  return v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
}

// One 16x16x128 e4m3 x e4m3 -> f32 MFMA from a zero accumulator.  Lane l holds
// row/column l % 16 and 32 of the 128 K values (the same K values for A and B);
// the result gives lane l rows 4*(l/16) .. 4*(l/16)+3 of column l % 16.
__device__ __forceinline__ v4f mfma_fp8(v8i a, v8i b) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

// max(x, 0) as one integer max on the bit pattern: a float with the sign bit
// set is a negative int32 and becomes +0; any other value passes unchanged.
__device__ __forceinline__ float relu(float x) { return __int_as_float(max(__float_as_int(x), 0)); }

// x[j] is this lane's partial for column tile j; returns, in lane (g, n), the
// sum over the four lane groups of tile g's partials for column n.
__device__ __forceinline__ float reduce_scatter4(float x0, float x1, float x2, float x3, int g) {
  const bool hi2 = (g & 2) != 0;
  const float keep_a = hi2 ? x2 : x0, keep_b = hi2 ? x3 : x1;
  const float send_a = hi2 ? x0 : x2, send_b = hi2 ? x1 : x3;
  const float y0 = keep_a + __shfl_xor(send_a, 32);
  const float y1 = keep_b + __shfl_xor(send_b, 32);
  const bool hi1 = (g & 1) != 0;
  const float keep = hi1 ? y1 : y0, send = hi1 ? y0 : y1;
  return keep + __shfl_xor(send, 16);
}

// ---------------------------------------------------------------- score sources

// Scores computed from the paged KV pool.  A wave reads a group's 64 keys with
// contiguous loads -- lane l takes bytes 16l..16l+15 of each 1 KB run of 8
// keys -- and turns them into MFMA B operands through an 8 KB LDS area of its
// own: each lane writes its 16-byte pieces into the keys' 128-byte rows, the
// row's eight 16-byte columns XOR-swizzled by the row index (so that neither
// the writes nor the operand reads of 16 rows at one column pile onto one
// bank), and reads back the 32 bytes of key n its operand needs.
// Page addressing, key loads and the staging of a group's keys into MFMA B
// operands, shared by the two KV score sources below.
struct KvStream {
  struct Group {
    v4i raw[8];   // lane's 16 bytes of keys 8i + lane/8, column lane % 8
    float s;
  };
  v4i* stage;           // this wave's 8 KB LDS area: 64 rows of 8 16-byte columns
  const uint8_t* kv;
  const int32_t* bt_row;
  int bs_shift, bs_mask, block_bytes, scale_off;
  int lane, n, g;

  // The wave's staging area (kStageInt4 int4 per wave, kWaves waves).
  __device__ __forceinline__ void bind(v4i* lds) { stage = lds + wave_id() * kStageInt4; }

  __device__ __forceinline__ void init_stream(const PagedArgs& a, int b) {
    lane = lane_id();
    n = lane & 15;
    g = lane >> 4;
    kv = a.kv;
    bt_row = a.bt + static_cast<int64_t>(b) * a.bt_stride;
    bs_shift = a.bs_shift;
    bs_mask = (1 << a.bs_shift) - 1;
    block_bytes = a.block_bytes;
    scale_off = a.scale_off;
  }

  // Pages of the 64 keys at p0 (a multiple of 64, below L): keys p0..p0+31 on
  // page a, p0+32..p0+63 on page b (the same page for block_size >= 64).  A
  // column tile at or past L re-reads slots of a page the request owns (values
  // never used), so no block-table entry past ceil(L / block_size) is read.
  // The entries are read with scalar loads (the index is uniform), which wait
  // on their own counter: a group's page lookup never waits for the key loads
  // still in flight.
  struct Pages {
    const uint8_t* a;
    const uint8_t* b;
  };
  __device__ __forceinline__ Pages pages(int p0, int L) const {
    typedef const __attribute__((address_space(4))) int32_t const_i32;
    const const_i32* bt = (const const_i32*)(bt_row);
    const int pb = (p0 + 32 < L) ? p0 + 32 : p0;
    const int ia = __builtin_amdgcn_readfirstlane(p0 >> bs_shift);
    const int ib = __builtin_amdgcn_readfirstlane(pb >> bs_shift);
    return {kv + static_cast<int64_t>(bt[ia]) * block_bytes, kv + static_cast<int64_t>(bt[ib]) * block_bytes};
  }

  // Issue the loads of the 64 keys at p0, on the pages pg: eight contiguous
  // 1 KB runs (keys 8i..8i+7 each, never across a page) and the keys' scales.
  // The key bytes are read once per call: nontemporal loads (measured 1.5 us
  // faster on the 64-request decode batch than ordinary ones).
  __device__ __forceinline__ void load(Group& gr, const Pages& pg, int p0) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint8_t* run = (i < 4 ? pg.a : pg.b) + ((p0 + 8 * i) & bs_mask) * kDim;
      gr.raw[i] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(run + 16 * lane));
    }
    gr.s = *reinterpret_cast<const float*>((g < 2 ? pg.a : pg.b) + scale_off + ((p0 + lane) & bs_mask) * 4);
  }
  __device__ __forceinline__ void load(Group& gr, int p0, int L) const { load(gr, pages(p0, L), p0); }

  // The group into the staging area, then the B operands of its four 16-key
  // column tiles out of it (LDS operations of one wave complete in order).
  __device__ __forceinline__ void operands(const Group& gr, v8i (&bk)[4]) const {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int row = 8 * i + (lane >> 3);
      stage[row * 8 + ((lane & 7) ^ (row & 7))] = gr.raw[i];
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int row = 16 * j + n;
      const v4i lo = stage[row * 8 + ((2 * g) ^ (row & 7))];
      const v4i hi = stage[row * 8 + ((2 * g + 1) ^ (row & 7))];
      bk[j] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
  }
};

// The in-lane epilogue of one MFMA result: the weighted sum of the ReLU of
// this lane's four heads, added to sum in head order.  Both score sources use
// it in the same order (head tiles mt = 0..3, then i = 0..3 within a tile), so
// they give the same bits.
__device__ __forceinline__ float head_sum(v4f acc, float4 w, float sum) {
  sum = __builtin_fmaf(relu(acc[0]), w.x, sum);
  sum = __builtin_fmaf(relu(acc[1]), w.y, sum);
  sum = __builtin_fmaf(relu(acc[2]), w.z, sum);
  return __builtin_fmaf(relu(acc[3]), w.w, sum);
}

// Scores computed from the paged KV pool, the A operands (q) and the lane's 16
// weights per row held in VGPRs (next_n up to 2, and the repair).
template <int NT>
struct QLds;

template <int NT>
struct KvSource : KvStream {
  v8i qa[NT][4];        // A operands: rows t, head tiles mt
  float4 wt[NT][4];     // weights of heads 16*mt + 4*g .. +3

  __device__ __forceinline__ void bind_q(QLds<NT>*) {}

  __device__ __forceinline__ void init(const PagedArgs& a, int b) {
    init_stream(a, b);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = static_cast<int64_t>(b) * NT + t;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        qa[t][mt] = load32(a.q + ((row * kHeads + 16 * mt + n) * kDim + 32 * g));
        wt[t][mt] = *reinterpret_cast<const float4*>(a.w + row * kHeads + 16 * mt + 4 * g);
      }
    }
  }

  // E[t] = score of key p0 + lane for row t.  Fixed operation order, shared by
  // every kernel, so the logits, fused and repair paths agree bit for bit.
  __device__ __forceinline__ void score(const Group& gr, float (&E)[NT]) const {
    v8i bk[4];
    operands(gr, bk);
    float part[NT][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      // all of the tile's MFMAs first, into separate accumulators, so their
      // latencies overlap; then the in-lane epilogue
      v4f acc[NT][4];
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[t][mt] = mfma_fp8(qa[t][mt], bk[j]);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        float sum = 0.f;
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sum = head_sum(acc[t][mt], wt[t][mt], sum);
        part[t][j] = sum;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) E[t] = reduce_scatter4(part[t][0], part[t][1], part[t][2], part[t][3], g) * gr.s;
  }
};

// CTA-shared LDS copy of a request's q operands and weights for KvSourceQ: q of
// row t, head tile mt, half h (16 bytes) for lane l at q[t][mt][h][l]; the
// weights of heads 16*mt + 4*g .. +3 at w[t][mt][g].
template <int NT>
struct QLds {
  v4i q[NT][4][2][64];
  float4 w[NT][4][4];
};

// Scores computed from the paged KV pool with the A operands (q) and weights
// read from LDS per head tile (next_n of 3 and 4): holding 32 VGPRs of q and
// 16 of weights per row left those variants one wave per SIMD; from LDS they
// fit two.  Same operation order as KvSource, so the same bits.
template <int NT>
struct KvSourceQ : KvStream {
  QLds<NT>* ql;

  __device__ __forceinline__ void bind_q(QLds<NT>* q_area) { ql = q_area; }

  // Every thread of the CTA calls it (it ends with a barrier).
  __device__ __forceinline__ void init(const PagedArgs& a, int b) {
    init_stream(a, b);
    const int tid = threadIdx.x;
    // (t, mt, h, l) -> bytes 32*(l/16) + 16*h of head 16*mt + l%16 of row t
    for (int e = tid; e < NT * 4 * 2 * 64; e += kThreads) {
      const int l = e & 63, h = (e >> 6) & 1, mt = (e >> 7) & 3, t = e >> 9;
      const int64_t row = static_cast<int64_t>(b) * NT + t;
      (&ql->q[0][0][0][0])[e] =
          *reinterpret_cast<const v4i*>(a.q + (row * kHeads + 16 * mt + (l & 15)) * kDim + 32 * (l >> 4) + 16 * h);
    }
    for (int e = tid; e < NT * 16; e += kThreads) {
      const int t = e >> 4, head4 = e & 15;  // heads 4*head4 .. +3
      (&ql->w[0][0][0])[e] = *reinterpret_cast<const float4*>(a.w + (static_cast<int64_t>(b) * NT + t) * kHeads + 4 * head4);
    }
    __syncthreads();
  }

  struct Pipe {
    v8i qa[3];
    float4 wv[3];
    v4f acc[2][4];
  };
  template <int k>
  __device__ __forceinline__ void ld(Pipe& p) const {
    constexpr int t = k >> 2, mt = k & 3;
    const v4i lo = ql->q[t][mt][0][lane];
    const v4i hi = ql->q[t][mt][1][lane];
    p.qa[k % 3] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    p.wv[k % 3] = ql->w[t][mt][g];
  }
  template <int k>
  __device__ __forceinline__ void mm(Pipe& p, const v8i (&bk)[4]) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) p.acc[k & 1][j] = mfma_fp8(p.qa[k % 3], bk[j]);
  }
  template <int k>
  __device__ __forceinline__ void steps(Pipe& p, const v8i (&bk)[4], float (&part)[NT][4]) const {
    if constexpr (k < 4 * NT) {
      if constexpr (k + 1 < 4 * NT) mm<k + 1>(p, bk);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k + 2 < 4 * NT) ld<k + 2>(p);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 4; ++j) part[k >> 2][j] = head_sum(p.acc[k & 1][j], p.wv[k % 3], part[k >> 2][j]);
      // (keeps the steps in this order: left to itself the scheduler hoists
      // every LDS read to the top and runs out of registers)
      __builtin_amdgcn_sched_barrier(0);
      steps<k + 1>(p, bk, part);
    }
  }

  __device__ __forceinline__ void score(const Group& gr, float (&E)[NT]) const {
    v8i bk[4];
    operands(gr, bk);
    float part[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[t][j] = 0.f;
    // Software pipeline over the 4*NT (row, head tile) steps k = 4t + mt: the
    // operands of step k+2 are read from LDS and the MFMAs of step k+1 issued
    // before the epilogue of step k (operands triple-, accumulators
    // double-buffered), so LDS latency, MFMA latency and the epilogue overlap.
    // The steps are generated at compile time, so every buffer index is a
    // constant and the buffers live in registers.
    Pipe p;
    ld<0>(p);
    ld<1>(p);
    mm<0>(p, bk);
    __builtin_amdgcn_sched_barrier(0);
    steps<0>(p, bk, part);
#pragma unroll
    for (int t = 0; t < NT; ++t) E[t] = reduce_scatter4(part[t][0], part[t][1], part[t][2], part[t][3], g) * gr.s;
  }
};

// Scores read from a logits matrix.  Columns at or past L are clamped to L - 1
// (read, never used); only columns below each row's end are selected.  The
// kShared variant reads scores that other CTAs of the same kernel wrote (the
// fused repair's score buffer): agent-scope loads, and only the rows in `mask`.
template <int NT, bool kShared = false>
struct LogitsSource {
  struct Group {
    float v[NT];
  };
  const float* rows;
  int64_t ld;
  int lane;
  uint32_t mask;

  __device__ __forceinline__ void bind(v4i*) {}
  __device__ __forceinline__ void bind_q(QLds<NT>*) {}
  __device__ __forceinline__ void init(const LogitsArgs& a, int b) {
    lane = lane_id();
    ld = a.ld;
    rows = a.logits + static_cast<int64_t>(b) * NT * a.ld;
    mask = ~0u;
  }
  __device__ __forceinline__ void init_rows(const float* r, int64_t row_ld, uint32_t row_mask) {
    lane = lane_id();
    ld = row_ld;
    rows = r;
    mask = row_mask;
  }
  struct Pages {
    int L;
  };
  __device__ __forceinline__ Pages pages(int, int L) const { return {L}; }
  __device__ __forceinline__ void load(Group& gr, const Pages& pg, int p0) const {
    const int p = min(p0 + lane, pg.L - 1);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (!kShared)
        gr.v[t] = rows[t * ld + p];
      else
        gr.v[t] = (mask >> t) & 1u ? __uint_as_float(ld_ag(reinterpret_cast<const uint32_t*>(rows + t * ld + p)))
                                   : 0.f;
    }
  }
  __device__ __forceinline__ void load(Group& gr, int p0, int L) const { load(gr, pages(p0, L), p0); }
  __device__ __forceinline__ void score(const Group& gr, float (&E)[NT]) const {
#pragma unroll
    for (int t = 0; t < NT; ++t) E[t] = gr.v[t];
  }
  // Row t's score of key p (clamped to L - 1; jobs exist only for L >= 1).
  __device__ __forceinline__ float value(int t, int p, int L) const {
    const float* a = rows + t * ld + max(0, min(p, L - 1));
    return kShared ? __uint_as_float(ld_ag(reinterpret_cast<const uint32_t*>(a))) : *a;
  }
};

// Wave priority from the fraction of the range done: the waves of the CTAs
// that share a compute unit start together, and the issue arbiter favours the
// oldest waves among those of equal priority; waves that are further along
// step down, so the CTAs on a unit finish their equal shares together instead
// of in dispatch order.
__device__ __forceinline__ void set_priority_by_progress(int done, int total) {
  switch (3 - min(3, (4 * done) / max(total, 1))) {
    case 3: __builtin_amdgcn_s_setprio(3); break;
    case 2: __builtin_amdgcn_s_setprio(2); break;
    case 1: __builtin_amdgcn_s_setprio(1); break;
    default: __builtin_amdgcn_s_setprio(0); break;
  }
}

// Scores keys [k0, k1) of one request (k0 a multiple of 64, k1 <= L) in chunks
// of kChunk keys: wave w takes the chunk's groups w, w+4, w+8, w+12.  store(c,
// p0, E) runs for every group below k1 (c = its chunk's first key); once all
// waves have scored a chunk, chunk_done(c, cend) runs between two barriers
// (when kBarriers).  Loads run two groups ahead of the scoring, across chunk
// boundaries, so the next chunk's first groups are in flight while a chunk is
// finished; each group's page lookup is issued one group before its loads.  A
// group past k1 re-reads the segment's last group (an L2 hit), so every load is
// unconditional.  An empty range scores nothing and calls nothing.
template <int NT, bool kBarriers, class Src, class StoreF, class DoneF>
__device__ __forceinline__ void stream_keys(const Src& src, int k0, int k1, int L, StoreF&& store, DoneF&& done) {
  k0 = __builtin_amdgcn_readfirstlane(k0);
  k1 = __builtin_amdgcn_readfirstlane(k1);
  L = __builtin_amdgcn_readfirstlane(L);
  // an empty segment (a request with no keys) issues no load at all: the
  // clamped group indices below assume at least one group
  if (k1 <= k0) return;
  __builtin_amdgcn_s_setprio(3);
  const int w = wave_id();
  const int ngroups = static_cast<int>(ceil_div(k1 - k0, kGroupKeys));
  const int steps = 4 * static_cast<int>(ceil_div(ngroups, 4 * kWaves));  // groups per wave, padded
  auto key0 = [&](int i) { return k0 + kGroupKeys * min(w + kWaves * i, ngroups - 1); };
  auto valid = [&](int i) { return w + kWaves * i < ngroups; };
  auto chunk0 = [&](int i) { return k0 + kChunk * (i >> 2); };
  typename Src::Group ga, gb;
  typename Src::Pages pa = src.pages(key0(0), L);
  typename Src::Pages pb = src.pages(key0(1), L);
  // (the caller's loads -- q, weights, thresholds -- are older than the key
  // loads, so the first group's wait covers them too)
  // the scheduling barriers keep the groups' loads in issue order, so the
  // waits for a group count only the loads issued after it
  src.load(ga, pa, key0(0));
  __builtin_amdgcn_sched_barrier(0);
  pa = src.pages(key0(2), L);
  src.load(gb, pb, key0(1));
  __builtin_amdgcn_sched_barrier(0);
  pb = src.pages(key0(3), L);
  for (int i = 0; i < steps; i += 2) {
    if (valid(i)) {
      float E[NT];
      src.score(ga, E);
      store(chunk0(i), key0(i), E);
    }
    src.load(ga, pa, key0(i + 2));
    __builtin_amdgcn_sched_barrier(0);
    pa = src.pages(key0(i + 4), L);
    if (valid(i + 1)) {
      float E[NT];
      src.score(gb, E);
      store(chunk0(i + 1), key0(i + 1), E);
    }
    src.load(gb, pb, key0(i + 3));
    __builtin_amdgcn_sched_barrier(0);
    pb = src.pages(key0(i + 5), L);
    if (((i + 2) & 3) == 0) {
      const int c = chunk0(i);
      if (kBarriers) __syncthreads();
      done(c, min(c + kChunk, k1));
      if (kBarriers) __syncthreads();
      set_priority_by_progress(i + 2, steps);
    }
  }
  __builtin_amdgcn_s_setprio(3);
}

// ---------------------------------------------------------------- select pieces

// Stored score of a candidate: s - t where that is exact and order-keeping
// (t > 0 and t < s <= 2t, Sterbenz), else s.  Ties store s - t.
__device__ __forceinline__ float enc_cand(float s, float t) { return (t > 0.f && s <= 2.f * t) ? s - t : s; }
__device__ __forceinline__ float dec_cand(float v, float t) { return (t > 0.f && v <= t) ? v + t : v; }

// Order-preserving radix key: larger score -> larger key, -0 == +0, NaN -> 0.
// A positive score (or zero) maps to its magnitude bits with the top bit set,
// a negative one to 2^31 minus its magnitude bits, a NaN (magnitude bits above
// those of infinity) to 0 -- integer operations only, with no compare, so that
// the keys of several scores compute side by side.
__device__ __forceinline__ uint32_t radix_key(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t mag = u & 0x7fffffffu;
  const uint32_t neg = static_cast<uint32_t>(static_cast<int32_t>(u) >> 31);
  const uint32_t key = (neg & (0x80000000u - mag)) | (~neg & (mag | 0x80000000u));
  const uint32_t nan = static_cast<uint32_t>(static_cast<int32_t>(0x7f800000u - mag) >> 31);
  return key & ~nan;
}
__device__ __forceinline__ float key_to_float(uint32_t k) {
  if (k == 0u) return __uint_as_float(0x7fc00000u);
  return __uint_as_float((k & 0x80000000u) ? (k & 0x7fffffffu) : (0x80000000u | (0x80000000u - k)));
}

// Adds nc candidates and nt ties to a row's (candidate, tie) counter pair with
// one 64-bit atomic (the pair is 8-byte aligned) and returns the old pair, the
// first slot of each class.  The low word never carries into the high one:
// both counts stay below the row's length, under 2^31.
__device__ __forceinline__ uint64_t reserve_pair(int32_t* pair, int nc, int nt) {
  const uint64_t add = (static_cast<uint64_t>(static_cast<uint32_t>(nt)) << 32) | static_cast<uint32_t>(nc);
  return atomicAdd(reinterpret_cast<unsigned long long*>(pair), static_cast<unsigned long long>(add));
}

// A slot store is an agent-scope (relaxed) atomic store: the L2 of the
// storing XCD writes it through, so no dirty slot line is left in any XCD's L2.
// The tile's last CTA (on any XCD) can then read the slots after its acquire,
// and its own later stores to the same slots cannot be overwritten by a stale
// write-back -- without the L2-wide write-back an agent-scope release fence
// costs on every CTA.
__device__ __forceinline__ void store_pair(int32_t* slot, int idx, float v) {
  const uint64_t packed = (static_cast<uint64_t>(__float_as_uint(v)) << 32) | static_cast<uint32_t>(idx);
  __hip_atomic_store(reinterpret_cast<uint64_t*>(slot), packed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// Candidates above the final digit a local repair keeps in LDS (enough for
// k <= kAboveLds: fewer than k keys lie above the digit holding the k-th).
constexpr int kAboveLds = 2048;

// Longest request (in keys) whose rows a finish CTA over stored scores repairs
// by itself: one CTA's sweeps cost about 1 us per thousand keys, while the
// grid-wide repair costs about 100 us however long the request (measured on
// 44K- to 62K-key rows, local wins; on 131K-key rows, the jobs).
constexpr int kLocalRepairKeys = 65536;

// Shared memory of a finish-kernel CTA: a union of the per-row radix
// histograms (repair passes) and one row's keys (final selects), which are
// live at different times.
template <int NT>
struct CtaShared {
  union {
    uint32_t hist[NT][kRadixBins];  // per-row radix histograms
    struct {
      alignas(16) uint32_t hist[kRadixBins];
      uint32_t key[kFinalizeLds];
      int32_t idx[kFinalizeLds];
    } fin;                          // one row's keys (and key indices) for a final radix select
  } u;
  uint32_t wtot[kWaves];
  uint32_t dig[2];
  int32_t wcnt[NT][kWaves][2];
  int32_t wbase[NT][kWaves][2];
  uint32_t pfx[NT];
  uint32_t krem[NT];
  int32_t cnt[NT][2];
  int32_t nc[NT];
  int32_t nt[NT];
  float thr[NT];
  uint32_t repair_mask;
  int32_t len;
  int32_t is_last;
  int32_t pos[2];
  int32_t job[3];      // claimed repair item: tile (or -1: none open, -2: leave), stage, index
  int32_t next_stage;
  // few_extra_topk: each wave's smallest (key, position) pair per round;
  // few_extra_from_regs: each wave's smallest packed keys
  uint64_t low[kFewExtra][kWaves];
};

// Shared memory of a select kernel CTA: each wave's candidate and tie lists,
// per row, of (key index, stored score bits) pairs not yet written to the
// row's slots (the finish stage's structures stay out, so that three CTAs and
// their KV staging areas fit on a compute unit).
template <int NT>
struct MainShared {
  int2 cand[kWaves][NT][kWaveCand<NT>];
  int2 tie[kWaves][NT][kWaveTie<NT>];
  int32_t count[kWaves][NT][2];  // the waves' list lengths at the end
  int32_t base[NT][2];           // the CTA's slot bases per row and class
};

// One wave finds the digit holding the krem-th largest entry of hist[0..nb) and
// the rank left inside it, and returns both in every lane.  The histogram's
// total is at least krem.
__device__ __forceinline__ void find_digit(const uint32_t* hist, int nb, uint32_t krem, uint32_t* digit,
                                           uint32_t* rem) {
  const int lane = lane_id();
  const int per = nb / 64;
  uint32_t local = 0;
#pragma unroll 4
  for (int i = 0; i < per; ++i) local += hist[lane * per + i];
  uint32_t incl = local;  // sum over lanes >= this lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(incl, off);
    if (lane + off < 64) incl += y;
  }
  const uint32_t excl = incl - local;
  uint32_t d = 0, r = 0;
  if (excl < krem && krem <= incl) {
    uint32_t acc = excl;
#pragma unroll 1
    for (int i = per - 1; i >= 0; --i) {
      const uint32_t h = hist[lane * per + i];
      if (acc + h >= krem) {
        d = static_cast<uint32_t>(lane * per + i);
        r = krem - acc;
        break;
      }
      acc += h;
    }
  }
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    d = max(d, static_cast<uint32_t>(__shfl_xor(static_cast<int>(d), off)));
    r = max(r, static_cast<uint32_t>(__shfl_xor(static_cast<int>(r), off)));
  }
  *digit = d;
  *rem = r;
}

// Radix pass layout: 11 bits, 11 bits, 10 bits from the top of the key.
__device__ __forceinline__ int pass_shift(int pass) { return pass == 0 ? 21 : (pass == 1 ? 10 : 0); }
__device__ __forceinline__ int pass_bits(int pass) { return pass == 2 ? 10 : 11; }

// The digit of hist[0..nb) (nb = 1024 or 2048, 16-byte aligned) holding the
// krem-th largest entry, and the rank left inside it, found by the whole CTA:
// each thread sums nb / kThreads consecutive bins held in registers, a suffix
// scan over the threads gives the count above each thread's bins, and the one
// thread whose bins reach krem walks them.  The histogram's total is at least
// krem.  Returns the same values in every thread.
template <int NT>
__device__ __forceinline__ void cta_find_digit(const uint32_t* hist, int nb, uint32_t krem, CtaShared<NT>& sh,
                                               uint32_t& digit, uint32_t& rem) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int per = nb / kThreads;  // 4 or 8
  uint32_t h[8];
  const uint4 lo = *reinterpret_cast<const uint4*>(hist + tid * per);
  const uint4 hi = per == 8 ? *reinterpret_cast<const uint4*>(hist + tid * per + 4) : uint4{0u, 0u, 0u, 0u};
  h[0] = lo.x; h[1] = lo.y; h[2] = lo.z; h[3] = lo.w;
  h[4] = hi.x; h[5] = hi.y; h[6] = hi.z; h[7] = hi.w;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) local += h[i];
  uint32_t incl = local;  // over lanes >= this lane
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_down(incl, off);
    if (lane + off < 64) incl += y;
  }
  if (lane == 0) sh.wtot[w] = incl;
  if (tid == 0) {
    sh.dig[0] = 0u;
    sh.dig[1] = 0u;
  }
  __syncthreads();
  uint32_t above = incl - local;
  for (int q = w + 1; q < kWaves; ++q) above += sh.wtot[q];
  if (above < krem && krem <= above + local) {
    uint32_t acc = above;
    bool found = false;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (!found && i < per && acc + h[i] >= krem) {
        sh.dig[0] = static_cast<uint32_t>(tid * per + i);
        sh.dig[1] = krem - acc;
        found = true;
      }
      if (i < per) acc += h[i];
    }
  }
  __syncthreads();
  digit = sh.dig[0];
  rem = sh.dig[1];
}

// The k-th largest of n radix keys key_of(0..n) (1 <= k <= n), by a 3-pass
// LDS radix select over `hist` (kRadixBins words, 16-byte aligned).  Leaves the
// key in sh.pfx[0] and, in sh.krem[0], how many entries equal to it the k
// largest hold; resets sh.pos[0..1] for the caller.
template <int NT, class KeyOf>
__device__ __forceinline__ void cta_radix_select(KeyOf&& key_of, int n, int k, uint32_t* hist, CtaShared<NT>& sh) {
  const int tid = threadIdx.x;
  uint32_t pf = 0u, krem = static_cast<uint32_t>(k);
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass_shift(pass);
    const int bits = pass_bits(pass);
    #pragma unroll 1
    for (int i = tid; i < kRadixBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    #pragma unroll 1
    for (int i = tid; i < n; i += kThreads) {
      const uint32_t key = key_of(i);
      if (pass > 0 && (key >> (shift + bits)) != pf) continue;
      atomicAdd(&hist[(key >> shift) & ((1u << bits) - 1u)], 1u);
    }
    __syncthreads();
    uint32_t d, rem;
    cta_find_digit(hist, 1 << bits, krem, sh, d, rem);
    pf = pass == 0 ? d : ((pf << bits) | d);
    krem = rem;
  }
  if (tid == 0) {
    sh.pfx[0] = pf;
    sh.krem[0] = krem;
    sh.pos[0] = 0;
    sh.pos[1] = 0;
  }
  __syncthreads();
}

// CTA-wide exclusive prefix sums of a and b over the threads in order (two
// barriers).
template <int NT>
__device__ __forceinline__ void cta_exclusive_scan2(uint32_t& a, uint32_t& b, CtaShared<NT>& sh) {
  const int lane = lane_id();
  const int w = wave_id();
  uint32_t ia = a, ib = b;  // inclusive within the wave
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t ya = __shfl_up(ia, off), yb = __shfl_up(ib, off);
    if (lane >= off) {
      ia += ya;
      ib += yb;
    }
  }
  __syncthreads();
  if (lane == 63) {
    sh.wtot[w] = ia;
    sh.wcnt[0][w][0] = static_cast<int32_t>(ib);
  }
  __syncthreads();
  uint32_t ba = 0u, bb = 0u;
  for (int q = 0; q < w; ++q) {
    ba += sh.wtot[q];
    bb += static_cast<uint32_t>(sh.wcnt[0][q][0]);
  }
  a = ba + ia - a;
  b = bb + ib - b;
}

// Top-k of a row whose nc candidates exceed k by d = nc - k <= kFewExtra (the
// pairs of the slots below npre already in sh.u.fin.idx / sh.u.fin.key): the
// d smallest candidates (by radix key, ties by slot position) are left out
// and every other candidate's index is written in slot order.  Each of the d
// rounds finds the smallest pair not yet left out: a tree over each thread's
// keys, the wavefront minimum (DPP), and the four waves' minima exchanged
// through LDS with one barrier; the output then shifts each index past the
// left-out positions before it, so the stores stay coalesced.
template <int NT>
__device__ __forceinline__ void few_extra_topk(const int32_t* cand, int32_t* out, int nc, int d, float th, int npre,
                                               CtaShared<NT>& sh) {
  const int tid = threadIdx.x;
  constexpr int kPer = kFinalizeLds / kThreads;
  uint32_t* key = sh.u.fin.key;
  int32_t* idx = sh.u.fin.idx;
  if (npre < nc) {
    // the pairs not in LDS yet, all of a thread's loads in flight
    int2 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kThreads + tid;
      if (i >= npre && i < nc) v[u] = *reinterpret_cast<const int2*>(cand + 2 * i);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kThreads + tid;
      if (i >= npre && i < nc) {
        idx[i] = v[u].x;
        key[i] = static_cast<uint32_t>(v[u].y);
      }
    }
  }
  __syncthreads();
  // (LDS reads at clamped indices, unconditional, so that they are all in
  // flight at once instead of one branch and wait each; the nu steps a row
  // needs, out of kPer)
  const int nu = static_cast<int>(ceil_div(nc, kThreads));
  uint32_t kv[kPer] = {};
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (u >= nu) break;
    kv[u] = key[min(u * kThreads + tid, nc - 1)];
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (u >= nu) break;
    kv[u] = radix_key(dec_cand(__uint_as_float(kv[u]), th));
  }
  uint32_t p0 = 0xffffffffu, p1 = 0xffffffffu, p2 = 0xffffffffu;
#pragma unroll 1
  for (int j = 0; j < d; ++j) {
    // this thread's smallest pair still in, by a tree over its keys
    uint64_t m[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const uint32_t i = static_cast<uint32_t>(u * kThreads + tid);
      m[u] = (u < nu && i < static_cast<uint32_t>(nc) && i != p0 && i != p1 && i != p2)
                 ? ((static_cast<uint64_t>(kv[u]) << 32) | i)
                 : ~0ull;
    }
#pragma unroll
    for (int w = kPer / 2; w > 0; w >>= 1)
#pragma unroll
      for (int u = 0; u < w; ++u) m[u] = min(m[u], m[u + w]);
    const uint64_t wm = __ockl_wfred_min_u64(m[0]);
    if (lane_id() == 0) sh.low[j][wave_id()] = wm;
    __syncthreads();
    uint64_t g = sh.low[j][0];
#pragma unroll
    for (int q = 1; q < kWaves; ++q) g = min(g, sh.low[j][q]);
    const uint32_t pj = static_cast<uint32_t>(g);
    if (j == 0) p0 = pj;
    else if (j == 1) p1 = pj;
    else p2 = pj;
  }
  int32_t iv[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (u >= nu) break;
    iv[u] = idx[min(u * kThreads + tid, nc - 1)];
  }
#pragma unroll
  for (int u = 0; u < kPer; ++u) {
    if (u >= nu) break;
    const uint32_t i = static_cast<uint32_t>(u * kThreads + tid);
    if (i < static_cast<uint32_t>(nc) && i != p0 && i != p1 && i != p2)
      out[i - (i > p0) - (i > p1) - (i > p2)] = iv[u];
  }
  __syncthreads();
}

// Exact Top-k of one fitting row from its slots: every candidate when there are
// at most k, topped up with ties from the tie slots; otherwise the k largest
// candidates by decoded score -- all but the few smallest when at most
// kFewExtra are left out, else by a 3-pass radix select over keys kept in LDS
// (read from the slots once).  Entries past k are -1.  The first npre
// candidate pairs may be in sh.u.fin.idx / sh.u.fin.key already.
template <int NT>
__device__ __forceinline__ void finalize_topk(const SelectArgs& s, int r, int k, int nc, float th, int npre,
                                              CtaShared<NT>& sh) {
  const int tid = threadIdx.x;
  constexpr int kPer = kFinalizeLds / kThreads;
  const int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + s.capacity) * 2;
  int32_t* out = s.topk_idx + static_cast<int64_t>(r) * s.top_k;
  for (int i = k + tid; i < s.top_k; i += kThreads) out[i] = -1;
  if (nc <= k) {
    // every candidate, then ties; all of a thread's loads in flight at once
    // (the preloaded candidates read from LDS at clamped indices, unconditional)
    const bool lds = nc <= npre;
    for (int i0 = 0; i0 < k; i0 += kPer * kThreads) {
      const int nu = static_cast<int>(ceil_div(min(k - i0, kPer * kThreads), kThreads));
      int32_t v[kPer];
      if (lds && nc > 0) {
#pragma unroll
        for (int u = 0; u < kPer; ++u) {
          if (u >= nu) break;
          v[u] = sh.u.fin.idx[min(i0 + u * kThreads + tid, nc - 1)];
        }
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (u >= nu) break;
        const int i = i0 + u * kThreads + tid;
        if (i < k && (i >= nc || !lds))
          v[u] = i < nc ? slots[2 * (s.top_k + i)] : slots[2 * (s.top_k - 1 - (i - nc))];
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        if (u >= nu) break;
        const int i = i0 + u * kThreads + tid;
        if (i < k) out[i] = v[u];
      }
    }
    return;
  }
  if (nc - k <= kFewExtra && nc <= kFinalizeLds) {
    few_extra_topk<NT>(slots + 2 * s.top_k, out, nc, nc - k, th, npre, sh);
    return;
  }
  const bool in_lds = nc <= kFinalizeLds;
  uint32_t* hist = sh.u.fin.hist;
  uint32_t* keys = sh.u.fin.key;
  int32_t* idx = sh.u.fin.idx;
  const int32_t* cand = slots + 2 * s.top_k;
  if (in_lds) {
    // (index, score) pairs into LDS, all of a thread's loads in flight at once
    constexpr int kPer = kFinalizeLds / kThreads;
    for (int i0 = 0; i0 < nc; i0 += kPer * kThreads) {
      int2 v[kPer];
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = i0 + u * kThreads + tid;
        if (i < nc) v[u] = *reinterpret_cast<const int2*>(cand + 2 * i);
      }
#pragma unroll
      for (int u = 0; u < kPer; ++u) {
        const int i = i0 + u * kThreads + tid;
        if (i < nc) {
          keys[i] = radix_key(dec_cand(__int_as_float(v[u].y), th));
          idx[i] = v[u].x;
        }
      }
    }
    __syncthreads();
  }
  auto key_of = [&](int i) -> uint32_t {
    return in_lds ? keys[i] : radix_key(dec_cand(__int_as_float(cand[2 * i + 1]), th));
  };
  cta_radix_select(key_of, nc, k, hist, sh);
  const uint32_t kstar = sh.pfx[0];
  const int n_eq = static_cast<int>(sh.krem[0]);
  const int n_gt = k - n_eq;
  if (in_lds) {
    // each thread's keys above k* (and equal to it) counted, one CTA-wide
    // exclusive scan of the counts, then every thread writes at its offsets
    constexpr int kPer = kFinalizeLds / kThreads;
    uint32_t gt = 0u, eq = 0u;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kThreads + tid;
      if (i < nc) {
        gt += keys[i] > kstar ? 1u : 0u;
        eq += keys[i] == kstar ? 1u : 0u;
      }
    }
    uint32_t og = gt, oe = eq;
    cta_exclusive_scan2(og, oe, sh);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kThreads + tid;
      if (i < nc) {
        if (keys[i] > kstar) {
          out[og++] = idx[i];
        } else if (keys[i] == kstar) {
          if (static_cast<int>(oe) < n_eq) out[n_gt + oe] = idx[i];
          ++oe;
        }
      }
    }
    __syncthreads();
    return;
  }
  #pragma unroll 1
  for (int i = tid; i < nc; i += kThreads) {
    const uint32_t key = key_of(i);
    if (key > kstar) {
      out[atomicAdd(&sh.pos[0], 1)] = cand[2 * i];
    } else if (key == kstar) {
      const int e = atomicAdd(&sh.pos[1], 1);
      if (e < n_eq) out[n_gt + e] = cand[2 * i];
    }
  }
  __syncthreads();
}

// Fit test of tile b (its request's length at *len) from its counters: fills
// sh.nc, sh.nt, sh.thr and sh.len and returns the mask of rows that do not
// fit.  It also loads the first npre <= kPreCap candidate pairs of row r_pre
// (index, score bits) into the registers of waves 1-3: pair u * kPreThreads +
// tid - 64 into pre[u].  All of these loads are issued together.
template <int NT>
__device__ __forceinline__ uint32_t tile_fit(const SelectArgs& s, const int32_t* len, int b, CtaShared<NT>& sh,
                                             int r_pre, int npre, int2 (&pre)[kPreUnits]) {
  const int tid = threadIdx.x;
  if (tid == 0) sh.repair_mask = 0u;
  int nc = 0, nt = 0, L = 0;
  float th = 0.f;
  if (tid < NT) {
    const int r = b * NT + tid;
    nc = __hip_atomic_load(s.counters + 2 * r, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    nt = __hip_atomic_load(s.counters + 2 * r + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    th = s.thresholds[r];
    L = *len;
  }
  const int32_t* cand = s.candidates + (static_cast<int64_t>(r_pre) * (s.top_k + s.capacity) + s.top_k) * 2;
  const int pt = tid - 64;
#pragma unroll
  for (int u = 0; u < kPreUnits; ++u) {
    const int i = u * kPreThreads + pt;
    pre[u] = pt >= 0 && i < npre ? *reinterpret_cast<const int2*>(cand + 2 * i) : int2{0, 0};
  }
  __syncthreads();
  if (tid < NT) {
    const int k = min(max(0, L - NT + tid + 1), s.top_k);
    const bool fit = nc <= s.capacity && nc + min(nt, s.top_k) >= k;
    sh.nc[tid] = nc;
    sh.nt[tid] = nt;
    sh.thr[tid] = th;
    if (tid == 0) sh.len = L;
    if (!fit) atomicOr(&sh.repair_mask, 1u << tid);
  }
  __syncthreads();
  return sh.repair_mask;
}

// The D smallest of a set of doubles, kept sorted in m[0..D-1]; kFewBig pads.
constexpr double kFewBig = 1152921504606846976.0;  // 2^60, above every packed key
template <int D>
struct Smallest {
  double m[D];
  __device__ __forceinline__ void init() {
#pragma unroll
    for (int j = 0; j < D; ++j) m[j] = kFewBig;
  }
  __device__ __forceinline__ void insert(double x) {
    if constexpr (D >= 3) m[2] = fmin(m[2], fmax(m[1], x));
    if constexpr (D >= 2) m[1] = fmin(m[1], fmax(m[0], x));
    m[0] = fmin(m[0], x);
  }
  // The D smallest of the union with another sorted set o: the j-th smallest
  // of two sorted lists is the least of the maxima of their (i, j - i) prefixes.
  __device__ __forceinline__ void merge(const Smallest& o) {
    const double a1 = m[0], a2 = o.m[0];
    if constexpr (D >= 3) m[2] = fmin(fmin(m[2], o.m[2]), fmin(fmax(a1, o.m[1]), fmax(m[1], a2)));
    if constexpr (D >= 2) m[1] = fmin(fmax(a1, a2), fmin(m[1], o.m[1]));
    m[0] = fmin(a1, a2);
  }
};

// Lane l's double from the lane the DPP control Ctrl names (kFewBig where it
// names none, or in a row outside RowMask).
template <int Ctrl, int RowMask>
__device__ __forceinline__ double dpp_f64(double v) {
  const uint64_t u = static_cast<uint64_t>(__double_as_longlong(v));
  const uint64_t b = static_cast<uint64_t>(__double_as_longlong(kFewBig));
  const int lo = __builtin_amdgcn_update_dpp(static_cast<int>(static_cast<uint32_t>(b)),
                                             static_cast<int>(static_cast<uint32_t>(u)), Ctrl, RowMask, 0xf, false);
  const int hi = __builtin_amdgcn_update_dpp(static_cast<int>(static_cast<uint32_t>(b >> 32)),
                                             static_cast<int>(static_cast<uint32_t>(u >> 32)), Ctrl, RowMask, 0xf, false);
  return __longlong_as_double(static_cast<long long>((static_cast<uint64_t>(static_cast<uint32_t>(hi)) << 32) |
                                                     static_cast<uint32_t>(lo)));
}
template <int Ctrl, int RowMask, int D>
__device__ __forceinline__ void dpp_merge(Smallest<D>& x) {
  Smallest<D> o;
#pragma unroll
  for (int j = 0; j < D; ++j) o.m[j] = dpp_f64<Ctrl, RowMask>(x.m[j]);
  x.merge(o);
}

// Top-k of a fitting row with D = nc - k in 1 .. kFewExtra extra candidates,
// all of them in the registers of waves 1-3 (pre[u] is pair u * kPreThreads +
// tid - 64, nc <= kPreCap): all but the D smallest, by score and then slot
// position.  Each pair becomes one exact double, order key * 4096 + position
// (below 2^44).  The stored candidate scores order as the scores do (the
// encoding maps (t, 2t] onto (0, t] and keeps the rest, with t > 0; ties stay
// ties) and none is NaN (a NaN never compares above a threshold), so the order
// key is the stored bits' radix key with -0 taken as +0.  One pass: each
// thread keeps its D smallest, a DPP reduction leaves the wave's in lane 63,
// and the four waves' are merged through LDS.  The indices are then written in
// slot order shifted past the left-out positions, so the stores stay coalesced.
template <int NT, int D>
__device__ __forceinline__ void few_extra_from_regs(const SelectArgs& s, int r, int k, int nc,
                                                    const int2 (&pre)[kPreUnits], CtaShared<NT>& sh) {
  const int tid = threadIdx.x;
  const int w = wave_id();
  int32_t* out = s.topk_idx + static_cast<int64_t>(r) * s.top_k;
  const bool has = tid >= 64;  // a thread of waves 1-3
  const int pt = tid - 64;
  const int nu = static_cast<int>(ceil_div(nc, kPreThreads));  // units in use (uniform)
  Smallest<D> sm;
  sm.init();
#pragma unroll
  for (int u = 0; u < kPreUnits; ++u) {
    if (u < nu) {
      const int i = u * kPreThreads + pt;
      uint32_t b = static_cast<uint32_t>(pre[u].y);
      b = b == 0x80000000u ? 0u : b;
      b ^= static_cast<uint32_t>(static_cast<int32_t>(b) >> 31) | 0x80000000u;
      if (has && i < nc) sm.insert(__builtin_fma(static_cast<double>(b), 4096.0, static_cast<double>(i)));
    }
  }
  // the wave's D smallest into lane 63
  dpp_merge<0x111, 0xf>(sm);  // row_shr:1
  dpp_merge<0x112, 0xf>(sm);  // row_shr:2
  dpp_merge<0x114, 0xf>(sm);  // row_shr:4
  dpp_merge<0x118, 0xf>(sm);  // row_shr:8
  dpp_merge<0x142, 0xa>(sm);  // row_bcast:15
  dpp_merge<0x143, 0xc>(sm);  // row_bcast:31
  double* xw = reinterpret_cast<double*>(&sh.low[0][0]);  // the waves' sets (8-byte aligned)
  static_assert(kFewExtra * kWaves >= D * kWaves, "room for every wave's set");
  if (lane_id() == 63) {
#pragma unroll
    for (int j = 0; j < D; ++j) xw[D * w + j] = sm.m[j];
  }
  __syncthreads();
  Smallest<D> all;
#pragma unroll
  for (int j = 0; j < D; ++j) all.m[j] = xw[D + j];  // wave 0 holds none
#pragma unroll
  for (int q = 2; q < kWaves; ++q) {
    Smallest<D> o;
#pragma unroll
    for (int j = 0; j < D; ++j) o.m[j] = xw[D * q + j];
    all.merge(o);
  }
  uint32_t p[D];  // the left-out slot positions
#pragma unroll
  for (int j = 0; j < D; ++j) {
    const double v = all.m[j];
    p[j] = static_cast<uint32_t>(v - 4096.0 * floor(v * (1.0 / 4096.0)));
  }
  // (positions before the first left-out one already hold their index: the
  // select kernel wrote candidate j < top_k to entry j)
#pragma unroll
  for (int u = 0; u < kPreUnits; ++u) {
    const int i = u * kPreThreads + pt;
    if (u < nu && has && i < nc) {
      const uint32_t iu = static_cast<uint32_t>(i);
      bool kept = true;
      uint32_t shift = 0;
#pragma unroll
      for (int j = 0; j < D; ++j) {
        kept = kept && iu != p[j];
        shift += iu > p[j] ? 1u : 0u;
      }
      if (kept && shift) out[i - shift] = pre[u].x;
    }
  }
  for (int i = k + tid; i < s.top_k; i += kThreads) out[i] = -1;
}

// ranges and Top-k finalize of row r (k = min(e_r, top_k)) from its final
// candidate count nc, tie count nt and threshold th (the first npre candidate
// pairs possibly loaded already, as finalize_topk takes them).
template <int NT>
__device__ __forceinline__ void row_outputs(const SelectArgs& s, int r, int k, int nc, int nt, float th, int npre,
                                            CtaShared<NT>& sh) {
  if (threadIdx.x == 0) {
    s.ranges[r] = s.top_k - min(nt, s.top_k);
    s.ranges[s.rows + r] = s.top_k + min(nc, s.capacity);
  }
  if (s.topk_idx) finalize_topk<NT>(s, r, k, nc, th, npre, sh);
  __syncthreads();
}

// Phase A's outputs of a fitting row, its first npre candidate pairs loading
// into the registers of waves 1-3 (pre[u] = pair u * kPreThreads + tid - 64).  A row with exactly k
// candidates has its Top-k from the select kernel already (entries past k
// aside) and waits for none of these loads.
template <int NT>
__device__ __forceinline__ void row_outputs_pre(const SelectArgs& s, int r, int k, int nc, int nt, float th, int npre,
                                                const int2 (&pre)[kPreUnits], CtaShared<NT>& sh) {
  const bool exact = nc == k;
  const bool few = nc > k && nc - k <= kFewExtra && nc <= npre;
  if (!s.topk_idx || exact || few) {
    if (s.topk_idx && exact) {
      int32_t* out = s.topk_idx + static_cast<int64_t>(r) * s.top_k;
      for (int i = k + threadIdx.x; i < s.top_k; i += kThreads) out[i] = -1;
    } else if (s.topk_idx) {
      // waves 1-3: their pairs in at once (the compiler would otherwise wait
      // for all earlier memory operations before each store it predicates);
      // wave 0 holds no pairs and has no store outstanding here but, in the
      // CTA with the last count, the done flags'
      if (threadIdx.x >= 64) wait_vm_done();
      static_assert(kFewExtra == 3, "one instance per count of extra candidates");
      if (nc - k == 1) few_extra_from_regs<NT, 1>(s, r, k, nc, pre, sh);
      else if (nc - k == 2) few_extra_from_regs<NT, 2>(s, r, k, nc, pre, sh);
      else few_extra_from_regs<NT, 3>(s, r, k, nc, pre, sh);
    }
    if (threadIdx.x == 0) {
      s.ranges[r] = s.top_k - min(nt, s.top_k);
      s.ranges[s.rows + r] = s.top_k + min(nc, s.capacity);
    }
    __syncthreads();
    return;
  }
  // the pairs into LDS, where finalize_topk takes them (one wait for all)
  const int tid = threadIdx.x;
  wait_vm_done();
#pragma unroll
  for (int u = 0; u < kPreUnits; ++u) {
    const int i = u * kPreThreads + tid - 64;
    if (tid >= 64 && i < npre) {
      sh.u.fin.idx[i] = pre[u].x;
      sh.u.fin.key[i] = static_cast<uint32_t>(pre[u].y);
    }
  }
  __syncthreads();
  row_outputs<NT>(s, r, k, nc, nt, th, npre, sh);
}

// ---------------------------------------------------------------- finish

// Each tile is finished by a second kernel, launched right after the select
// kernel on the same stream, so it starts with every slot and counter of the
// main pass in memory and the memory system idle.  Phase A: CTA i takes rows
// i, i + grid, ...: the fit test of the row's tile, then either the row's
// ranges and exact Top-k, or, for a row that does not fit, over stored scores
// of a request of at most kLocalRepairKeys keys, the row's repair by this CTA
// alone (local_repair_row), or else, from the CTA with the tile's first row
// that does not fit, a repair job: the mask of those rows, their state words,
// and the tile appended to the job list.  Phase B: every CTA runs
// repair items.  A job runs in stages, each split into items of a few thousand
// keys of the request:
//   stages 1-3  radix histogram pass 0/1/2 (11/11/10 bits) of the repaired
//               rows' keys, into per-row global histograms;
//   stage 4     collect: keys above the selected bucket become candidates
//               (stored raw), keys inside it go to a per-row bucket buffer;
//   stage 5     select again at the now exact k-th largest score;
//   stage 6     one item per row: for a collected row, the exact k-th largest
//               key from its bucket (the bucket's keys appended, the collected
//               candidates re-encoded against it), then the row's ranges and
//               Top-k.
// The fused repair computes the scores from the KV pages once, in stage 1, and
// keeps the repaired rows' scores in the workspace's score buffer; its later
// stages read them back (4 bytes a key instead of 132), as the repair of a
// select over a logits matrix reads the matrix.
// After a histogram pass the digit holding each row's k-th largest key is
// found; if every row's bucket fits the bucket buffer the job moves to stage 4,
// if every key bit is known to stage 5, else to the next pass; stages 4 and 5
// lead to stage 6.  An item is
// claimed by a 64-bit fetch-and-add on one of the job's kClaimWords (stage,
// next) words, word q handing out items q, q + kClaimWords, ...: an item below
// the stage's item count is the caller's, a larger one claims nothing.
// Whoever completes a stage's last item runs the stage change, which rewrites
// the words to (next stage, 0), or after stage 6 clears the job's words.  A CTA with no open item waits (a bounded number of polls)
// while some CTA is still in phase A, a listed job is not yet written, or a job
// is in a stage before 6 (its change opens new items), and leaves otherwise;
// the wait only adds hands, since each job is carried to its end by the CTA that
// completes each of its stages.  Shared words are written with agent-scope
// atomic (write-through) stores or atomic adds and read with agent-scope atomic
// loads.  A job's last step clears its words; the select kernel clears the
// header and the job list at its start, when no finish kernel can be running.
constexpr int kClaimWords = 4;  // claim words per repair job
constexpr int kStageHist0 = 1;
constexpr int kStageCollect = 4;
constexpr int kStageSelect = 5;
constexpr int kStageRows = 6;
constexpr int kIdlePolls = 20000;  // bound on a CTA's polls without an item
constexpr int kHdrBatch = 3, kHdrNextN = 4, kHdrMagic = 5;  // header words of the layout record
constexpr uint32_t kLayoutMagic = 0x41514d50u;
static_assert(2 * kClaimWords + 1 + 6 < kJobWords, "a job's claim words, mask and per-stage counts");

struct Ws {
  uint32_t* base;
  int batch, rows;
  // [0,1] the progress word (below), [3..5] the layout of the last finish
  // kernel (the select kernel clears [0..2], the flags and the list before
  // each finish kernel)
  __device__ uint32_t* hdr() const { return base; }
  // rows through phase A (low half) and job list entries reserved (high half)
  __device__ uint64_t* progress() const { return reinterpret_cast<uint64_t*>(base); }
  // copy i of the done flag: 0 while phase A runs, then 1 + the number of jobs
  // listed (the waiting CTAs poll copy blockIdx % kDoneFlags, 256 bytes apart,
  // so their polls spread over many lines instead of queueing on one)
  __device__ uint32_t* flag(int i) const { return base + 16 + kDoneFlagStride * i; }
  __device__ uint32_t* list(int j) const { return base + 16 + kDoneFlags * kDoneFlagStride + j; }  // tile + 1, 0 until written
  // [2q, 2q + 1] claim word q < kClaimWords, [2 kClaimWords] row mask,
  // [2 kClaimWords + 1 + stage] items done in the stage
  __device__ uint32_t* job(int b) const {
    return base + 16 + kDoneFlags * kDoneFlagStride + job_list_words(batch) + kJobWords * b;
  }
  // Claim word q hands out items q, q + kClaimWords, ... of the job's stage: a
  // CTA claims from word blockIdx % kClaimWords, so the atomics of a stage's
  // claims spread over kClaimWords words instead of queueing on one.
  __device__ uint64_t* claim(int b, int q) const { return reinterpret_cast<uint64_t*>(job(b) + 2 * q); }
  __device__ uint32_t* mask_word(int b) const { return job(b) + 2 * kClaimWords; }
  __device__ uint32_t* done_word(int b, int stage) const { return job(b) + 2 * kClaimWords + 1 + stage; }
  // [0] digit prefix [1] rank left [2] bits known [3] bucket count
  __device__ uint32_t* row(int r) const { return job(batch) + kRowWords * r; }
  // copy c of row r's radix histogram (items add into copy idx % kHistCopies,
  // which spreads the atomics of a pass over kHistCopies times more lines)
  __device__ uint32_t* hist(int r, int c) const {
    return job(batch) + kRowWords * rows + static_cast<int64_t>(kRadixBins) * (kHistCopies * r + c);
  }
  __device__ int32_t* bucket(int r) const {
    return reinterpret_cast<int32_t*>(job(batch) + (kRowWords + kHistCopies * kRadixBins) * rows) +
           static_cast<int64_t>(2) * kFinalizeLds * r;
  }
};

// Items of a stage of a request of L keys: kRescoreItemKeys keys when the
// scores are computed from the KV pages (stage 1 of the fused repair), else
// kSelectItemKeys keys read back from a score row; one per row in stage 6.
template <int NT, bool kFused>
__device__ __forceinline__ int stage_items(int stage, int L) {
  if (stage == kStageRows) return NT;
  const int keys = (kFused && stage == kStageHist0) ? kRescoreItemKeys : kSelectItemKeys;
  return max(1, static_cast<int>(ceil_div(L, keys)));
}

// Phase A hands the rows of tile b in `mask` to phase B: their state words and
// the claim words first, then (once those are complete) the list entry.
template <int NT>
__device__ __forceinline__ void publish_job(const SelectArgs& s, const Ws& ws, int b, const int (&end)[NT], uint32_t mask) {
  const int tid = threadIdx.x;
  if (tid < NT && (mask & (1u << tid))) st_wt(ws.row(b * NT + tid) + 1, static_cast<uint32_t>(min(end[tid], s.top_k)));
  if (tid == 0) st_wt(ws.mask_word(b), mask);
  if (tid < kClaimWords) st_wt64(ws.claim(b, tid), static_cast<uint64_t>(kStageHist0) << 32);
  wait_vm_done();
  __syncthreads();
  if (tid == 0) {
    const uint64_t old = atomicAdd(reinterpret_cast<unsigned long long*>(ws.progress()), 1ull << 32);
    st_wt(ws.list(static_cast<int>(old >> 32)), static_cast<uint32_t>(b + 1));
  }
}

// One row through phase A: the count (thread 0, after every store that lists
// a job of the CTA has completed); it returns the progress word before it.
__device__ __forceinline__ uint64_t count_row(const Ws& ws) {
  return atomicAdd(reinterpret_cast<unsigned long long*>(ws.progress()), 1ull);
}

// Thread 0, with count_row's result: the count of the last row sets every copy
// of the done flag to 1 + the jobs listed (final by then: each publisher lists
// its job before it counts its row).
__device__ __forceinline__ void flag_if_last(const Ws& ws, uint64_t old) {
  if (static_cast<uint32_t>(old) + 1u == static_cast<uint32_t>(ws.rows)) {
    const uint32_t v = static_cast<uint32_t>(old >> 32) + 1u;
    for (int i = 0; i < kDoneFlags; ++i) st_wt(ws.flag(i), v);
  }
}

// Stages 4 and 5 on one whole item of scores held in registers (v[t][u] is row
// t's score of key c0 + 64*(w + 4u) + lane, for the rows in mask): every key
// below min(cend, end[t]) is classified by cls(t, score) -> 0 (none), 1 or 2;
// each wave counts its keys of both classes with ballots, one thread per row
// reserves the CTA's slots with one atomic per class (add1(t, n), add2(t, n)
// return the first), and the keys go to put(t, class, position, key, score).
template <int NT, int kU, class Cls, class Add1, class Add2, class Put>
__device__ __forceinline__ void append_item(int c0, int cend, const int (&end)[NT], uint32_t mask,
                                            const float (&v)[NT][kU], CtaShared<NT>& sh, Cls&& cls, Add1&& add1,
                                            Add2&& add2, Put&& put) {
  const int w = wave_id();
  const int lane = lane_id();
  const int tid = threadIdx.x;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!(mask & (1u << t))) continue;
    const int lim = min(cend, end[t]);
    int n1 = 0, n2 = 0;
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = c0 + kGroupKeys * (w + kWaves * u) + lane;
      const int c = p < lim ? cls(t, v[t][u]) : 0;
      n1 += __popcll(__ballot(c == 1));
      n2 += __popcll(__ballot(c == 2));
    }
    if (lane == 0) {
      sh.wcnt[t][w][0] = n1;
      sh.wcnt[t][w][1] = n2;
    }
  }
  __syncthreads();
  if (tid < NT && (mask & (1u << tid))) {
    int tot[2] = {0, 0};
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      tot[0] += sh.wcnt[tid][q][0];
      tot[1] += sh.wcnt[tid][q][1];
    }
    int base[2];
    base[0] = tot[0] ? add1(tid, tot[0]) : 0;
    base[1] = tot[1] ? add2(tid, tot[1]) : 0;
#pragma unroll
    for (int q = 0; q < kWaves; ++q) {
      sh.wbase[tid][q][0] = base[0];
      sh.wbase[tid][q][1] = base[1];
      base[0] += sh.wcnt[tid][q][0];
      base[1] += sh.wcnt[tid][q][1];
    }
  }
  __syncthreads();
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!(mask & (1u << t))) continue;
    const int lim = min(cend, end[t]);
    int r1 = sh.wbase[t][w][0], r2 = sh.wbase[t][w][1];
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int p = c0 + kGroupKeys * (w + kWaves * u) + lane;
      const int c = p < lim ? cls(t, v[t][u]) : 0;
      const uint64_t m1 = __ballot(c == 1);
      const uint64_t m2 = __ballot(c == 2);
      if (c == 1) put(t, 1, r1 + lanes_below(m1), p, v[t][u]);
      if (c == 2) put(t, 2, r2 + lanes_below(m2), p, v[t][u]);
      r1 += __popcll(m1);
      r2 += __popcll(m2);
    }
  }
}

// Stage change after histogram pass `pass` of tile b's job (run by the CTA that
// completed the pass's last item).
template <int NT>
__device__ __forceinline__ void job_next_stage(const SelectArgs& s, const Ws& ws, int b, int pass, uint32_t mask, CtaShared<NT>& sh) {
  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  const int shift = pass_shift(pass);
  const int bits = pass_bits(pass);
  const int nb = 1 << bits;
  // each row's histogram: the sum of its copies, which are cleared for the next
  // pass.  Every row's copies are loaded together (kHistCopies * nb / kThreads
  // words a thread and row), so the sum costs one round trip, not one per row
  // and half histogram.
  constexpr int kJ = kRadixBins / kThreads;  // bins of a thread
  uint32_t v[NT][kJ][kHistCopies];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!(mask & (1u << t))) continue;
    const uint32_t* gh = ws.hist(b * NT + t, 0);
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c)
        v[t][j][c] = j * kThreads < nb ? ld_ag(gh + c * kRadixBins + j * kThreads + tid) : 0u;
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!(mask & (1u << t))) continue;
    uint32_t* gh = ws.hist(b * NT + t, 0);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (j * kThreads >= nb) continue;
      uint32_t sum = 0u;
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) {
        sum += v[t][j][c];
        if (v[t][j][c]) st_wt(gh + c * kRadixBins + j * kThreads + tid, 0u);
      }
      sh.u.hist[t][j * kThreads + tid] = sum;
    }
  }
  __syncthreads();
  if (wave < NT && (mask & (1u << wave))) {
    uint32_t* row = ws.row(b * NT + wave);
    const uint32_t pfx = ld_ag(row + 0);
    uint32_t d = 0, rem = 0;
    find_digit(sh.u.hist[wave], nb, ld_ag(row + 1), &d, &rem);
    if (lane == 0) {
      sh.pfx[wave] = pass == 0 ? d : ((pfx << bits) | d);
      sh.krem[wave] = rem;
      sh.cnt[wave][0] = static_cast<int32_t>(sh.u.hist[wave][d]);
    }
  }
  __syncthreads();
  const int known = 32 - shift;
  if (tid == 0) {
    bool small = true;
    for (int t = 0; t < NT; ++t)
      if ((mask & (1u << t)) && sh.cnt[t][0] > kFinalizeLds) small = false;
    sh.next_stage = known == 32 ? kStageSelect : (small ? kStageCollect : kStageHist0 + pass + 1);
  }
  __syncthreads();
  const int next = sh.next_stage;
  if (tid < NT && (mask & (1u << tid))) {
    const int r = b * NT + tid;
    uint32_t* row = ws.row(r);
    st_wt(row + 0, sh.pfx[tid]);
    st_wt(row + 1, sh.krem[tid]);
    st_wt(row + 2, static_cast<uint32_t>(known));
    if (next >= kStageCollect) {
      st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r, 0u);
      st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r + 1, 0u);
      st_wt(row + 3, 0u);
    }
    if (next == kStageSelect) st_wt(reinterpret_cast<uint32_t*>(s.thresholds) + r, __float_as_uint(key_to_float(sh.pfx[tid])));
  }
  wait_vm_done();
  __syncthreads();
  if (tid < kClaimWords) st_wt64(ws.claim(b, tid), static_cast<uint64_t>(next) << 32);
}

// Row r after the collect stage: its exact k-th largest key among its bucket
// (kept in LDS), the bucket's candidates and ties appended, the raw candidates
// re-encoded against the new threshold.  Leaves the row's final candidate and
// tie counts and threshold in sh.nc[0], sh.nt[0], sh.thr[0] (and in counters
// and thresholds).
template <int NT>
__device__ __forceinline__ void resolve_row(const SelectArgs& s, const Ws& ws, int r, CtaShared<NT>& sh) {
  const int tid = threadIdx.x;
  const int stride = s.top_k + s.capacity;
  uint32_t* row = ws.row(r);
  // the bucket holds the keys of one digit, at most kFinalizeLds by the stage
  // change's test
  const int nin = min(static_cast<int>(ld_ag(row + 3)), kFinalizeLds);
  const int krem = static_cast<int>(ld_ag(row + 1));
  const int nabove = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r));
  int32_t* bucket = ws.bucket(r);
  // the bucket's (index, score bits) pairs into LDS, all of a thread's loads in
  // flight at once (the radix keys are derived from the bits where needed)
  constexpr int kPer = kFinalizeLds / kThreads;
  uint32_t* bits = sh.u.fin.key;
  int32_t* idxs = sh.u.fin.idx;
  {
    int2 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kThreads + tid;
      if (i < nin) v[u] = *reinterpret_cast<const int2*>(bucket + 2 * i);
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = u * kThreads + tid;
      if (i < nin) {
        idxs[i] = v[u].x;
        bits[i] = static_cast<uint32_t>(v[u].y);
      }
    }
  }
  __syncthreads();
  auto key_of = [&](int i) { return radix_key(__uint_as_float(bits[i])); };
  cta_radix_select(key_of, nin, krem, sh.u.fin.hist, sh);
  const uint32_t kstar = sh.pfx[0];
  const float t2 = key_to_float(kstar);
  int32_t* slots = s.candidates + static_cast<int64_t>(r) * stride * 2;
  #pragma unroll 1
  for (int i = tid; i < nin; i += kThreads) {
    const uint32_t key = key_of(i);
    const int32_t idx = idxs[i];
    const float e = __uint_as_float(bits[i]);
    if (key > kstar) {
      const int k = nabove + atomicAdd(&sh.pos[0], 1);
      if (k < s.capacity) store_pair(slots + 2 * (s.top_k + k), idx, enc_cand(e, t2));
    } else if (key == kstar) {
      const int k = atomicAdd(&sh.pos[1], 1);
      if (k < s.top_k) store_pair(slots + 2 * (s.top_k - 1 - k), idx, e - t2);
    }
  }
  // the candidates collected above the bucket (raw scores) re-encoded against
  // the new threshold, all of a thread's loads in flight at once
  const int nabove_kept = min(nabove, s.capacity);
  for (int i0 = 0; i0 < nabove_kept; i0 += kPer * kThreads) {
    int2 v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = i0 + u * kThreads + tid;
      if (i < nabove_kept) v[u] = *reinterpret_cast<const int2*>(slots + 2 * (s.top_k + i));
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = i0 + u * kThreads + tid;
      if (i < nabove_kept) store_pair(slots + 2 * (s.top_k + i), v[u].x, enc_cand(__int_as_float(v[u].y), t2));
    }
  }
  __syncthreads();
  if (tid == 0) {
    const int nc = nabove + sh.pos[0], nt = sh.pos[1];
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r, static_cast<uint32_t>(nc));
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r + 1, static_cast<uint32_t>(nt));
    st_wt(reinterpret_cast<uint32_t*>(s.thresholds) + r, __float_as_uint(t2));
    sh.nc[0] = nc;
    sh.nt[0] = nt;
    sh.thr[0] = t2;
  }
  // this CTA's slot stores complete before the Top-k reads the slots back
  wait_vm_done();
  __syncthreads();
}

// Stage 6 item t of tile b's job: row t, if repaired, resolved (after a
// collect) and given its ranges and Top-k.  The row's state words are cleared
// for the next call.
template <int NT>
__device__ __forceinline__ void row_end_item(const SelectArgs& s, const Ws& ws, int b, int L, int t, uint32_t mask,
                             CtaShared<NT>& sh) {
  if (!(mask & (1u << t))) return;
  const int tid = threadIdx.x;
  const int r = b * NT + t;
  // the collect stage's stores (other CTAs, written through) become visible
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (ld_ag(ws.row(r) + 2) < 32u) {
    resolve_row<NT>(s, ws, r, sh);
  } else {
    // stage 5 selected the row again at its exact threshold
    if (tid == 0) {
      sh.nc[0] = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r));
      sh.nt[0] = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r + 1));
      sh.thr[0] = __uint_as_float(ld_ag(reinterpret_cast<const uint32_t*>(s.thresholds) + r));
    }
    __syncthreads();
  }
  const int k = min(max(0, L - NT + t + 1), s.top_k);
  row_outputs<NT>(s, r, k, sh.nc[0], sh.nt[0], sh.thr[0], 0, sh);
  if (tid < 4) st_wt(ws.row(r) + tid, 0u);
}

// Adds the LDS histograms sh.u.hist of pass `pass` of the rows in `mask` to
// copy `copy` of their global histograms (nonzero bins only).
template <int NT>
__device__ __forceinline__ void flush_hist(const Ws& ws, int b, int pass, uint32_t mask, int copy,
                                           CtaShared<NT>& sh) {
  const int nb = 1 << pass_bits(pass);
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!(mask & (1u << t))) continue;
    uint32_t* gh = ws.hist(b * NT + t, copy);
    for (int i = threadIdx.x; i < nb; i += kThreads) {
      const uint32_t h = sh.u.hist[t][i];
      if (h) atomicAdd(gh + i, h);
    }
  }
}

// Stage 1 of the fused repair, item idx: keys [c0, c1) of request b scored
// again from the KV pages (the select kernel's loop and arithmetic, so the
// scores are the same bits), the repaired rows' scores written to the score
// buffer for the later passes, and their first radix histogram pass.
template <int NT>
__device__ __forceinline__ void rescore_item(const PagedArgs& a, const SelectArgs& s, const Ws& ws, int b, int L, int idx,
                             uint32_t mask, const int (&end)[NT], CtaShared<NT>& sh, v4i* lds) {
  const int lane = lane_id();
  const int shift = pass_shift(0);
  for (int i = threadIdx.x; i < NT * kRadixBins; i += kThreads) (&sh.u.hist[0][0])[i] = 0u;
  __syncthreads();
  KvSource<NT> src;
  src.bind(lds);
  src.init(a, b);
  float* rows = s.scores + static_cast<int64_t>(b) * NT * s.score_ld;
  const int c0 = idx * kRescoreItemKeys;
  const int c1 = min(c0 + kRescoreItemKeys, L);
  stream_keys<NT, false>(
      src, c0, c1, L,
      [&](int, int p0, const float(&E)[NT]) {
        const int p = p0 + lane;
#pragma unroll
        for (int t = 0; t < NT; ++t) {
          if (!(mask & (1u << t)) || p >= end[t]) continue;
          st_wt(reinterpret_cast<uint32_t*>(rows + t * s.score_ld + p), __float_as_uint(E[t]));
          atomicAdd(&sh.u.hist[t][radix_key(E[t]) >> shift], 1u);
        }
      },
      [](int, int) {});
  __syncthreads();
  flush_hist<NT>(ws, b, 0, mask, idx % kHistCopies, sh);
}

// Repair item `idx` of stage `stage` of tile b's job: its keys' scores (read
// back from the logits matrix or the score buffer, or for stage 1 of the fused
// repair computed again), then their histogram, collect or select pass, then
// the stage bookkeeping.
template <int NT, bool kFused, class Args>
__device__ __forceinline__ void run_item(const Args& a, const SelectArgs& s, const Ws& ws, int b, int L, int stage, int idx,
                         CtaShared<NT>& sh, v4i* lds) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const uint32_t mask = ld_ag(ws.mask_word(b));
  int end[NT];
  uint32_t pfx[NT];
  float thr2[NT];
  int known = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    end[t] = max(0, L - NT + t + 1);
    const int r = b * NT + t;
    const bool m = (mask & (1u << t)) != 0;
    pfx[t] = m ? ld_ag(ws.row(r) + 0) : 0u;
    thr2[t] = m ? __uint_as_float(ld_ag(reinterpret_cast<const uint32_t*>(s.thresholds) + r)) : 0.f;
    if (m) known = static_cast<int>(ld_ag(ws.row(r) + 2));
  }
  bool done = false;
  if (stage == kStageRows) {
    row_end_item<NT>(s, ws, b, L, idx, mask, sh);
    done = true;
  }
  if constexpr (kFused) {
    if (stage == kStageHist0) {
      rescore_item<NT>(a, s, ws, b, L, idx, mask, end, sh, lds);
      done = true;
    }
  }
  if (!done) {
    LogitsSource<NT, kFused> src;
    if constexpr (kFused)
      src.init_rows(s.scores + static_cast<int64_t>(b) * NT * s.score_ld, s.score_ld, mask);
    else
      src.init(a, b);
    const int c0 = idx * kSelectItemKeys;
    const int cend = min(c0 + kSelectItemKeys, L);
    // The item's scores of the repaired rows, all loaded at once: wave w's
    // group u holds keys c0 + 64*(w + 4u) .. +63.
    constexpr int kU = kSelectItemKeys / (kGroupKeys * kWaves);
    const int w = wave_id();
    float v[NT][kU];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      if (!(mask & (1u << t))) continue;
#pragma unroll
      for (int u = 0; u < kU; ++u) v[t][u] = src.value(t, c0 + kGroupKeys * (w + kWaves * u) + lane, L);
    }
    if (stage < kStageCollect) {
      // histogram straight from the scores in registers
      const int pass = stage - kStageHist0;
      const int shift = pass_shift(pass);
      const int bits = pass_bits(pass);
      const uint32_t low = (1u << bits) - 1u;
      for (int i = tid; i < NT * kRadixBins; i += kThreads) (&sh.u.hist[0][0])[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        if (!(mask & (1u << t))) continue;
        const int lim = min(cend, end[t]);
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int p = c0 + kGroupKeys * (w + kWaves * u) + lane;
          if (p >= lim) continue;
          const uint32_t key = radix_key(v[t][u]);
          if (pass > 0 && (key >> (shift + bits)) != pfx[t]) continue;
          atomicAdd(&sh.u.hist[t][(key >> shift) & low], 1u);
        }
      }
      __syncthreads();
      flush_hist<NT>(ws, b, pass, mask, idx % kHistCopies, sh);
    } else if (stage == kStageCollect) {
      // keys above the bucket become candidates (raw scores; re-encoded once
      // the threshold is known), keys inside it go to the row's bucket buffer
      const int stride = s.top_k + s.capacity;
      append_item<NT, kU>(
          c0, cend, end, mask, v, sh,
          [&](int t, float e) {
            const uint32_t top = radix_key(e) >> (32 - known);
            return top > pfx[t] ? 1 : (top == pfx[t] ? 2 : 0);
          },
          [&](int t, int n) { return atomicAdd(s.counters + 2 * (b * NT + t), n); },
          [&](int t, int n) { return static_cast<int>(atomicAdd(ws.row(b * NT + t) + 3, static_cast<uint32_t>(n))); },
          [&](int t, int c, int k, int p, float e) {
            if (c == 1 && k < s.capacity)
              store_pair(s.candidates + (static_cast<int64_t>(b * NT + t) * stride + s.top_k + k) * 2, p, e);
            if (c == 2 && k < kFinalizeLds) store_pair(ws.bucket(b * NT + t) + 2 * k, p, e);
          });
    } else {
      // select again at the now exact threshold
      const int stride = s.top_k + s.capacity;
      int32_t* cnt = s.counters + 2 * b * NT;
      append_item<NT, kU>(
          c0, cend, end, mask, v, sh,
          [&](int t, float e) { return e > thr2[t] ? 1 : (!(e < thr2[t]) ? 2 : 0); },
          [&](int t, int n) { return atomicAdd(cnt + 2 * t, n); },
          [&](int t, int n) { return atomicAdd(cnt + 2 * t + 1, n); },
          [&](int t, int c, int k, int p, float e) {
            int32_t* slots = s.candidates + static_cast<int64_t>(b * NT + t) * stride * 2;
            if (c == 1 && k < s.capacity) store_pair(slots + 2 * (s.top_k + k), p, enc_cand(e, thr2[t]));
            if (c == 2 && k < s.top_k) store_pair(slots + 2 * (s.top_k - 1 - k), p, e - thr2[t]);
          });
    }
  }
  wait_vm_done();
  __syncthreads();
  if (tid == 0)
    sh.is_last = atomicAdd(ws.done_word(b, stage), 1u) + 1 == static_cast<uint32_t>(stage_items<NT, kFused>(stage, L));
  __syncthreads();
  if (!sh.is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (stage < kStageCollect) {
    job_next_stage<NT>(s, ws, b, stage - kStageHist0, mask, sh);
  } else if (stage < kStageRows) {
    if (tid < kClaimWords) st_wt64(ws.claim(b, tid), static_cast<uint64_t>(kStageRows) << 32);
  } else {
    // the job is done: its words cleared for the next call (all but the claim
    // words, which late claim attempts may still increment; the next publish
    // of the tile rewrites them)
    if (tid >= 2 * kClaimWords && tid < kJobWords) st_wt(ws.job(b) + tid, 0u);
  }
}

// Wave 0 claims an item of a listed job; the result goes to sh.job: (tile,
// stage, item), tile -1 when none is open but more may open, -2 when the CTA
// should leave.
template <int NT, bool kFused, class Args>
__device__ __forceinline__ void claim_item(const Args& a, const Ws& ws, int& idle, CtaShared<NT>& sh) {
  if (wave_id() == 0) {
    const int lane = lane_id();
    // (a workspace that was not left zeroed gives wrong results, not stray accesses)
    const uint32_t fl = ld_ag(ws.flag(static_cast<int>(blockIdx.x % kDoneFlags)));
    const int njobs = fl ? min(static_cast<int>(fl - 1u), ws.batch) : 0;
    bool pending = fl == 0u;  // phase A still running
    int got = -1, stage = 0, idx = 0;
    const int q = static_cast<int>(blockIdx.x % kClaimWords);  // this CTA's claim word
    for (int j0 = 0; j0 < njobs && got < 0; j0 += 64) {
      const int j = j0 + lane;
      int b = 0, len = 0;
      uint64_t w = 0;
      bool unwritten = false;
      if (j < njobs) {
        const uint32_t e = ld_ag(ws.list(j));
        unwritten = e == 0u;
        if (!unwritten) {
          b = min(static_cast<int>(e) - 1, ws.batch - 1);
          w = ld_ag64(ws.claim(b, q));
          len = a.seq_lens[static_cast<int64_t>(b) * a.sl_stride];
        }
      }
      const uint32_t st = static_cast<uint32_t>(w >> 32);
      const bool open = st >= kStageHist0 && st <= kStageRows &&
                        q + kClaimWords * static_cast<uint64_t>(static_cast<uint32_t>(w)) <
                            static_cast<uint64_t>(stage_items<NT, kFused>(static_cast<int>(st), len));
      pending = pending || __ballot(unwritten || (st >= kStageHist0 && st < kStageRows)) != 0;
      uint64_t m = __ballot(open);
      const int rot = static_cast<int>(blockIdx.x & 63);  // spread CTAs over the open jobs
      while (m) {
        const uint64_t hi = m & (~0ull << rot);
        const int l = __ffsll(static_cast<long long>(hi ? hi : m)) - 1;
        m &= ~(1ull << l);
        const int bl = __shfl(b, l);
        const int ll = __shfl(len, l);
        unsigned long long old = 0;
        if (lane == 0) old = atomicAdd(reinterpret_cast<unsigned long long*>(ws.claim(bl, q)), 1ull);
        old = __shfl(old, 0);
        const uint32_t st2 = static_cast<uint32_t>(old >> 32);
        const uint64_t i2 = q + kClaimWords * static_cast<uint64_t>(static_cast<uint32_t>(old));
        if (st2 >= kStageHist0 && st2 <= kStageRows &&
            i2 < static_cast<uint64_t>(stage_items<NT, kFused>(static_cast<int>(st2), ll))) {
          got = bl;
          stage = static_cast<int>(st2);
          idx = static_cast<int>(i2);
          break;
        }
      }
    }
    if (got < 0 && (!pending || ++idle > kIdlePolls)) got = -2;
    if (lane == 0) {
      sh.job[0] = got;
      sh.job[1] = stage;
      sh.job[2] = idx;
    }
  }
  __syncthreads();
}

// One key of a sweep batch: its position, score, and 1 if it is below the
// row's end (0 for the clamped loads past it).
struct SweepKey {
  int p;
  float e;
  uint32_t ok;
};

// Sweeps keys [0, end) of one stored score row in batches: batch(at, J) gets a
// thread's J keys of the batch as at(0..J-1).  Where the row is 16-byte
// aligned: 16-byte loads, kSweepVec per thread per batch, the next batch's
// loads issued before the current batch is worked through, and the keys past
// the last whole quad in one more batch (J = 1); otherwise 4-byte loads,
// kSweepLoads per thread per batch, all in flight at once.  Every thread of
// the CTA runs every batch (a batch may synchronise the CTA); nothing at or
// past end is read.
constexpr int kSweepVec = 8;
constexpr int kSweepLoads = 32;
template <class B>
__device__ __forceinline__ void sweep_row(const float* row, int end, B&& batch) {
  const int tid = threadIdx.x;
  if ((reinterpret_cast<uintptr_t>(row) & 15u) == 0u) {
    const v4f* row4 = reinterpret_cast<const v4f*>(row);
    const int n4 = end / 4;
    constexpr int kStep = kSweepVec * kThreads;
    v4f cur[kSweepVec], nxt[kSweepVec];
    if (n4 > 0) {
#pragma unroll
      for (int u = 0; u < kSweepVec; ++u) cur[u] = row4[min(u * kThreads + tid, n4 - 1)];
    }
    #pragma unroll 1
    for (int c0 = 0; c0 < n4; c0 += kStep) {
      const bool more = c0 + kStep < n4;
      if (more) {
#pragma unroll
        for (int u = 0; u < kSweepVec; ++u) nxt[u] = row4[min(c0 + kStep + u * kThreads + tid, n4 - 1)];
      }
      batch(
          [&](int j) {
            const int i = c0 + (j >> 2) * kThreads + tid;
            return SweepKey{4 * i + (j & 3), cur[j >> 2][j & 3], i < n4 ? 1u : 0u};
          },
          std::integral_constant<int, 4 * kSweepVec>{});
      if (more) {
#pragma unroll
        for (int u = 0; u < kSweepVec; ++u) cur[u] = nxt[u];
      }
    }
    if (4 * n4 < end) {
      const int p = 4 * n4 + tid;
      const float e = row[min(p, end - 1)];
      batch([&](int) { return SweepKey{p, e, p < end ? 1u : 0u}; }, std::integral_constant<int, 1>{});
    }
    return;
  }
  #pragma unroll 1
  for (int c0 = 0; c0 < end; c0 += kSweepLoads * kThreads) {
    float v[kSweepLoads];
#pragma unroll
    for (int u = 0; u < kSweepLoads; ++u) v[u] = row[min(c0 + u * kThreads + tid, end - 1)];
    batch(
        [&](int j) {
          const int p = c0 + j * kThreads + tid;
          return SweepKey{p, v[j], p < end ? 1u : 0u};
        },
        std::integral_constant<int, kSweepLoads>{});
  }
}

// Appends a sweep batch's keys of class 1 and 2 (cls(score) -> 0, 1 or 2) in
// whole-CTA order: each thread counts its keys of both classes (packed in one
// word, class 2 in the high half: a batch holds fewer than 2^16 keys), one
// CTA-wide exclusive scan of the counts places each thread's keys after the
// running totals sh.pos[0..1], and each thread passes its keys, in order, to
// put(class, position, key, score) (with kEvery, every key is passed, class 0
// included, and put writes without a branch: on a lone wave per SIMD each
// branch per key costs more than the key's arithmetic).  cls must not branch
// either.  Two barriers a batch; the loads already issued for the next batch
// complete before the stores.
template <int NT, int J, bool kEvery = false, class At, class Cls, class Put>
__device__ __forceinline__ void append_batch(At&& at, Cls&& cls, Put&& put, CtaShared<NT>& sh) {
  static_assert(J * kThreads < 65536, "class counts of a batch fit 16 bits");
  const int w = wave_id();
  const int lane = lane_id();
  uint32_t cnt = 0u;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const SweepKey k = at(j);
    const int c = cls(k.e) & -static_cast<int>(k.ok);
    cnt += (c == 1 ? 1u : 0u) + (c == 2 ? 0x10000u : 0u);
  }
  uint32_t incl = cnt;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t y = __shfl_up(incl, off);
    if (lane >= off) incl += y;
  }
  if (lane == 63) sh.wtot[w] = incl;
  __syncthreads();
  uint32_t below = 0u, tot = 0u;
#pragma unroll
  for (int q = 0; q < kWaves; ++q) {
    if (q < w) below += sh.wtot[q];
    tot += sh.wtot[q];
  }
  const int p1 = sh.pos[0], p2 = sh.pos[1];
  __syncthreads();
  if (threadIdx.x == 0) {
    sh.pos[0] = p1 + static_cast<int>(tot & 0xffffu);
    sh.pos[1] = p2 + static_cast<int>(tot >> 16);
  }
  const uint32_t excl = below + incl - cnt;
  int r1 = p1 + static_cast<int>(excl & 0xffffu), r2 = p2 + static_cast<int>(excl >> 16);
  // one wait for every load in flight (the next batch's included): the
  // compiler would otherwise wait for some before each predicated store
  wait_vm_done();
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const SweepKey k = at(j);
    const int c = cls(k.e) & -static_cast<int>(k.ok);
    if constexpr (kEvery) {
      put(c, c == 1 ? r1 : r2, k.p, k.e);  // every key, no branch (put ignores class 0)
    } else {
      if (c == 1) put(1, r1, k.p, k.e);
      if (c == 2) put(2, r2, k.p, k.e);
    }
    r1 += c == 1 ? 1 : 0;
    r2 += c == 2 ? 1 : 0;
  }
}

// radix_key's mapping in straight-line vector integer operations (the
// compiler would turn the C form back into compares, which serialise on one
// condition register): the key of a positive score, or of a negative one,
// picked by the sign mask, then cleared for a NaN.
__device__ __forceinline__ uint32_t radix_key_alu(float x) {
  uint32_t key, mag, t0, t1;
  asm("v_and_b32 %[mag], 0x7fffffff, %[u]\n\t"
      "v_ashrrev_i32 %[t0], 31, %[u]\n\t"
      "v_sub_u32 %[t1], 0x80000000, %[mag]\n\t"
      "v_or_b32 %[key], 0x80000000, %[mag]\n\t"
      "v_bfi_b32 %[key], %[t0], %[t1], %[key]\n\t"
      "v_sub_u32 %[t1], 0x7f800000, %[mag]\n\t"
      "v_ashrrev_i32 %[t1], 31, %[t1]\n\t"
      "v_bfi_b32 %[key], %[t1], 0, %[key]"
      : [key] "=&v"(key), [mag] "=&v"(mag), [t0] "=&v"(t0), [t1] "=&v"(t1)
      : [u] "v"(__float_as_uint(x)));
  return key;
}

// 1 if x == 0, else 0, without a compare.
__device__ __forceinline__ uint32_t is_zero_alu(uint32_t x) {
  uint32_t r;
  asm("v_min_u32 %0, 1, %1\n\t"
      "v_sub_u32 %0, 1, %0"
      : "=&v"(r)
      : "v"(x));
  return r;
}

// Repair of row r by this CTA alone, from its stored scores row[0, end): the
// exact k-th largest key (1 <= k <= end) by LDS radix histogram sweeps (11, 11
// and 10 bits from the top).  As soon as the digit holding it holds at most
// kFinalizeLds keys, one collect sweep keeps the digit's keys in LDS, where a
// radix select finds the exact key, and the keys above the digit as
// candidates (in LDS too when k <= kAboveLds), stored against that key;
// after the third histogram the row is selected again at the exact score
// instead.  Then the row's counters, threshold, ranges and Top-k.  No other
// CTA takes part, so no repair state is shared.
template <int NT>
__device__ __forceinline__ void local_repair_row(const SelectArgs& s, const float* row, int r, int end, int k,
                                                 CtaShared<NT>& sh) {
  const int tid = threadIdx.x;
  uint32_t* hist = sh.u.fin.hist;
  int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + s.capacity) * 2;
  // the candidates above the final digit and the digit's keys: (key index,
  // score bits), each with one spare entry per lane that takes the writes of
  // the keys of other classes (only the finish kernel over stored scores has
  // these areas)
  __shared__ int2 above[kAboveLds + 64];
  __shared__ int2 digit_keys[kFinalizeLds + 64];
  uint32_t pf = 0u, krem = static_cast<uint32_t>(k);
  int known = 0;
  float t2 = 0.f;
  for (int pass = 0;; ++pass) {
    const int shift = pass_shift(pass);
    const int bits = pass_bits(pass);
    const uint32_t low = (1u << bits) - 1u;
    #pragma unroll 1
    for (int i = tid; i < kRadixBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    // every key adds to its digit's bin, 1 if it has the known prefix, else 0
    // (no branch per key, so that the keys' instructions interleave)
    const int above_shift = pass == 0 ? 31 : shift + bits;
    const uint32_t want = pass == 0 ? 0u : pf;
    const uint32_t keep_mask = pass == 0 ? 0u : ~0u;
    sweep_row(row, end, [&](auto at, auto nj) {
#pragma unroll
      for (int j = 0; j < decltype(nj)::value; ++j) {
        const SweepKey k = at(j);
        const uint32_t key = radix_key_alu(k.e);
        const uint32_t in = k.ok & is_zero_alu(((key >> above_shift) ^ want) & keep_mask);
        atomicAdd(&hist[(key >> shift) & low], in);
      }
    });
    __syncthreads();
    uint32_t d, rem;
    cta_find_digit(hist, 1 << bits, krem, sh, d, rem);
    const uint32_t in_digit = hist[d];
    pf = pass == 0 ? d : ((pf << bits) | d);
    krem = rem;
    known += bits;
    if (tid == 0) {
      sh.pos[0] = 0;
      sh.pos[1] = 0;
    }
    __syncthreads();
    if (known == 32) {
      // every bit known: select again at the exact score
      t2 = key_to_float(pf);
      sweep_row(row, end, [&](auto at, auto nj) {
        append_batch<NT, decltype(nj)::value>(
            at, [&](float e) { return e > t2 ? 1 : (!(e < t2) ? 2 : 0); },
            [&](int c, int i, int p, float e) {
              if (c == 1 && i < s.capacity) store_pair(slots + 2 * (s.top_k + i), p, enc_cand(e, t2));
              if (c == 2 && i < s.top_k) store_pair(slots + 2 * (s.top_k - 1 - i), p, e - t2);
            },
            sh);
      });
      break;
    }
    if (in_digit <= static_cast<uint32_t>(kFinalizeLds)) {
      // collect: the digit's keys go to LDS, keys above it become candidates:
      // kept in LDS too while k <= kAboveLds (stored once the exact score is
      // known), else stored with their raw scores and re-encoded afterwards
      const uint32_t top_pf = pf;
      const int drop = 32 - known;
      const bool above_lds = k <= kAboveLds;
      auto put = [&](int c, int i, int p, float e) {
        if (c == 1 && above_lds) above[i] = make_int2(p, __float_as_int(e));
        if (c == 1 && !above_lds && i < s.capacity) store_pair(slots + 2 * (s.top_k + i), p, e);
        if (c == 2 && i < kFinalizeLds) digit_keys[i] = make_int2(p, __float_as_int(e));
      };
      // both classes to LDS, written by every lane for every key (a key of
      // another class, or past an area's end, to the lane's spare entry)
      const int lane = lane_id();
      auto put_every = [&](int c, int i, int p, float e) {
        const int2 v = make_int2(p, __float_as_int(e));
        above[c == 1 && i < kAboveLds ? i : kAboveLds + lane] = v;
        digit_keys[c == 2 && i < kFinalizeLds ? i : kFinalizeLds + lane] = v;
      };
      // The digit's keys are [lo, hi) = [top_pf, top_pf + 1) << drop.  Where lo
      // is the key of a number (not of the NaN-only low keys), the classes
      // follow from two float compares: key(e) >= K exactly when e >= the
      // float of key K (a NaN float for hi past the largest number's key
      // leaves class 1 empty, as it is).
      const uint64_t lo = static_cast<uint64_t>(top_pf) << drop;
      if (lo >= 0x00800000u) {
        const float lb = key_to_float(static_cast<uint32_t>(lo));
        const uint64_t hi = lo + (uint64_t{1} << drop);
        const float ub = hi > 0xffffffffu ? __uint_as_float(0x7fc00000u) : key_to_float(static_cast<uint32_t>(hi));
        // class 1 above the digit, 2 inside it: 2 (e >= lb) - (e >= ub), no branch
        auto cls = [&](float e) { return 2 * static_cast<int>(e >= lb) - static_cast<int>(e >= ub); };
        if (above_lds) {
          sweep_row(row, end, [&](auto at, auto nj) { append_batch<NT, decltype(nj)::value, true>(at, cls, put_every, sh); });
        } else {
          sweep_row(row, end, [&](auto at, auto nj) { append_batch<NT, decltype(nj)::value>(at, cls, put, sh); });
        }
      } else {
        sweep_row(row, end, [&](auto at, auto nj) {
          append_batch<NT, decltype(nj)::value>(
              at,
              [&](float e) {
                const uint32_t top = radix_key_alu(e) >> drop;
                return top > top_pf ? 1 : (top == top_pf ? 2 : 0);
              },
              put, sh);
        });
      }
      __syncthreads();
      const int nabove = sh.pos[0];
      const int nin = min(sh.pos[1], kFinalizeLds);
      __syncthreads();
      auto key_of = [&](int i) { return radix_key(__int_as_float(digit_keys[i].y)); };
      cta_radix_select(key_of, nin, static_cast<int>(krem), hist, sh);  // resets sh.pos
      const uint32_t kstar = sh.pfx[0];
      t2 = key_to_float(kstar);
      #pragma unroll 1
      for (int i = tid; i < nin; i += kThreads) {
        const uint32_t key = key_of(i);
        const int2 v = digit_keys[i];
        const float e = __int_as_float(v.y);
        if (key > kstar) {
          const int c = nabove + atomicAdd(&sh.pos[0], 1);
          if (c < s.capacity) store_pair(slots + 2 * (s.top_k + c), v.x, enc_cand(e, t2));
        } else if (key == kstar) {
          const int c = atomicAdd(&sh.pos[1], 1);
          if (c < s.top_k) store_pair(slots + 2 * (s.top_k - 1 - c), v.x, e - t2);
        }
      }
      // the candidates above the digit, encoded against the exact score: from
      // LDS, or the raw ones read back from L2 once this CTA's stores complete
      const int nkeep = min(nabove, s.capacity);
      if (above_lds) {
        #pragma unroll 1
        for (int i = tid; i < nkeep; i += kThreads) {
          const int2 v = above[i];
          store_pair(slots + 2 * (s.top_k + i), v.x, enc_cand(__int_as_float(v.y), t2));
        }
      } else {
        wait_vm_done();
        __syncthreads();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        #pragma unroll 1
        for (int i = tid; i < nkeep; i += kThreads) {
          const int2 v = *reinterpret_cast<const int2*>(slots + 2 * (s.top_k + i));
          store_pair(slots + 2 * (s.top_k + i), v.x, enc_cand(__int_as_float(v.y), t2));
        }
      }
      // every wave's digit-key appends above are done before the count moves
      // (a late wave's atomicAdd on sh.pos[0] would otherwise race with it)
      __syncthreads();
      if (tid == 0) sh.pos[0] += nabove;
      break;
    }
  }
  // the slot stores complete (and this CTA's view of the slots is refreshed)
  // before the Top-k reads them back
  wait_vm_done();
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  const int nc = sh.pos[0], nt = sh.pos[1];
  __syncthreads();
  if (tid == 0) {
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r, static_cast<uint32_t>(nc));
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r + 1, static_cast<uint32_t>(nt));
    st_wt(reinterpret_cast<uint32_t*>(s.thresholds) + r, __float_as_uint(t2));
  }
  row_outputs<NT>(s, r, k, nc, nt, t2, 0, sh);
}

// The finish kernel's CTA body: phase A over this CTA's rows, then repair
// items until nothing is left.
template <int NT, bool kFused, class Args>
__device__ __forceinline__ void finish_body(const Args& a, const SelectArgs& s, CtaShared<NT>& sh, v4i* lds) {
  const Ws ws{s.ws, a.batch, s.rows};
  const int tid = threadIdx.x;
  if (blockIdx.x == 0 && tid == 0) {
    // the layout this call's state words use (read by the next select kernel)
    st_wt(ws.hdr() + kHdrBatch, static_cast<uint32_t>(a.batch));
    st_wt(ws.hdr() + kHdrNextN, static_cast<uint32_t>(NT));
    st_wt(ws.hdr() + kHdrMagic, kLayoutMagic);
  }
  bool saw_repair = false;
  for (int r = blockIdx.x; r < s.rows; r += gridDim.x) {
    const int b = r / NT, t = r - b * NT;
    // the row's first candidate pairs (all of them when it has at most top_k +
    // kFewExtra) are loaded together with the fit test's inputs
    const int npre = s.topk_idx ? min(min(s.capacity, s.top_k + kFewExtra), kPreCap) : 0;
    int2 pre[kPreUnits];
    // every CTA working on a row of tile b finds the same mask; the one with
    // its lowest row publishes the job
    const uint32_t mask = tile_fit<NT>(s, a.seq_lens + static_cast<int64_t>(b) * a.sl_stride, b, sh, r, npre, pre);
    const int L = sh.len;
    int end[NT];
#pragma unroll
    for (int u = 0; u < NT; ++u) end[u] = max(0, L - NT + u + 1);
    const int k = min(end[t], s.top_k);
    // Stored scores of requests up to kLocalRepairKeys keys: each CTA repairs
    // its own rows (the same decision for every row of a tile); longer ones,
    // and the re-scoring repair, run as jobs.
    const bool local = !kFused && L <= kLocalRepairKeys;
    saw_repair = saw_repair || (mask != 0u && !local);
    // The row is through phase A once its fit is decided (and its job, if it
    // publishes one, listed): the CTAs waiting for repair items leave as soon
    // as every row is, while the fitting rows' outputs are still being written.
    if (!(mask & (1u << t))) {
      // (wave 0 has no pair load in flight: its count returns after one round trip)
      if (tid == 0) flag_if_last(ws, count_row(ws));
      row_outputs_pre<NT>(s, r, k, sh.nc[t], sh.nt[t], sh.thr[t], npre, pre, sh);
    } else if (local) {
      // counted first: the CTAs waiting for jobs need not wait for the repair
      if (tid == 0) flag_if_last(ws, count_row(ws));
      if constexpr (!kFused) {
        if (k > 0) local_repair_row<NT>(s, a.logits + static_cast<int64_t>(r) * a.ld, r, end[t], k, sh);
        else row_outputs<NT>(s, r, k, 0, 0, sh.thr[t], 0, sh);
      }
    } else {
      if ((mask & ((1u << t) - 1u)) == 0u) publish_job<NT>(s, ws, b, end, mask);
      if (tid == 0) {
        wait_vm_done();  // the job's list entry first
        flag_if_last(ws, count_row(ws));
      }
    }
    __syncthreads();
  }
  // With at least as many CTAs without rows as with, those are the repair's
  // hands: a CTA whose rows all fit (or were repaired here) leaves without
  // polling for items.
  if (!saw_repair && blockIdx.x < s.rows && 2 * static_cast<int64_t>(s.rows) <= gridDim.x) return;
  int idle = 0;
  while (true) {
    claim_item<NT, kFused>(a, ws, idle, sh);
    const int b = sh.job[0];
    const int stage = sh.job[1];
    const int idx = sh.job[2];
    __syncthreads();
    if (b == -2) break;
    if (b < 0) {
      // back off (up to about half a microsecond between polls), so that
      // waiting CTAs keep their loads off the job words the working ones update
      for (int i = 0; i < min(idle, 4); ++i) __builtin_amdgcn_s_sleep(4);
      continue;
    }
    idle = 0;
    const int L = a.seq_lens[static_cast<int64_t>(b) * a.sl_stride];
    run_item<NT, kFused>(a, s, ws, b, L, stage, idx, sh, lds);
    __syncthreads();
  }
}

// Run by every CTA of the select kernel after its keys (so before any finish
// kernel of this call): the finish stage's header, done flags and job list
// start empty.  Between calls the workspace holds
// only zeros in its state words (every job clears its own) -- except where a
// call laid it out differently: the fused repair's score buffer starts right
// after the state words, so another batch size or next_n puts state words
// where an earlier call kept scores.  The header records the layout the last
// finish kernel used (written by that kernel, so every CTA here reads the same
// value); when this call's layout differs, all CTAs clear its state words.
template <int NT>
__device__ __forceinline__ void prepare_workspace(const SelectArgs& s, int batch) {
  const Ws ws{s.ws, batch, s.rows};
  const bool same = s.ws[kHdrMagic] == kLayoutMagic && s.ws[kHdrBatch] == static_cast<uint32_t>(batch) &&
                    s.ws[kHdrNextN] == static_cast<uint32_t>(NT);
  const int tid = threadIdx.x;
  if (!same) {
    const int64_t n = workspace_state_words(batch, s.rows) - 16;
    for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + tid; i < n;
         i += static_cast<int64_t>(gridDim.x) * kThreads)
      s.ws[16 + i] = 0u;
  } else if (blockIdx.x == 0) {
    // the done flags and the job list (the claim words a late claim attempt
    // incremented sit where this call's jobs are, and each publish rewrites
    // its job's)
    for (int i = tid; i < kDoneFlags; i += kThreads) *ws.flag(i) = 0u;
    for (int i = tid; i < job_list_words(batch); i += kThreads) *ws.list(i) = 0u;
  }
  if (blockIdx.x == 0 && tid < 3) s.ws[tid] = 0u;
}

// ---------------------------------------------------------------- work items

// Located launches run G >= 2 * batch CTAs, about as many as fit on the device
// at once.  Every request gets one CTA plus a share of the other G - batch in
// proportion to its 64-key groups (with `empty_group`, a request with seq_len 0
// counts as one group, so that its tile still finishes), the shares rounded
// cumulatively so that they add up; a request's groups are split evenly among
// its CTAs.  So every CTA works on one request only -- a CTA never pays a
// second start-up and arrival -- and streams about the same number of keys as
// every other, whatever the length mix, so none sits idle while others finish
// a second round.  Other launches give each request per_request CTAs of
// keys_per_cta keys (no per-CTA scan of the batch).
__device__ __forceinline__ int groups_of(int L, bool empty_group) {
  return L > 0 ? static_cast<int>(ceil_div(L, kGroupKeys)) : (empty_group ? 1 : 0);
}

__device__ __forceinline__ int64_t uniform64(int64_t v) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(static_cast<uint64_t>(v) >> 32));
  return static_cast<int64_t>((static_cast<uint64_t>(hi) << 32) | lo);
}

// Calls seg(b, L, k0, k1, ctas) for the request b this CTA works on, with
// [k0, k1) the keys of b it handles and ctas the number of CTAs that handle b
// (the arrivals b's tile waits for).  Uniform across the CTA.
template <class F>
__device__ __forceinline__ void for_each_segment(const int32_t* seq_lens, int64_t sl_stride, int batch, bool locate,
                                                 int per_request, int keys_per_cta, bool empty_group, F&& seg) {
  if (!locate) {
    const int b = blockIdx.x / per_request;
    const int c = blockIdx.x % per_request;
    const int L = seq_lens[static_cast<int64_t>(b) * sl_stride];
    const int n = L > 0 ? static_cast<int>(ceil_div(L, keys_per_cta)) : (empty_group ? 1 : 0);
    if (c < n) seg(b, L, c * keys_per_cta, min((c + 1) * keys_per_cta, L), n);
    return;
  }
  const int lane = lane_id();
  if (batch <= 64) {
    // one load of the lengths, kept in registers for both scans
    const int L = lane < batch ? seq_lens[static_cast<int64_t>(lane) * sl_stride] : 0;
    const int g = lane < batch ? groups_of(L, empty_group) : 0;
    int64_t incl = g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int64_t N = uniform64(__shfl(incl, 63));
    const int64_t shared = static_cast<int64_t>(gridDim.x) - batch;
    auto first_cta = [&](int64_t b, int64_t c) { return b + (N > 0 ? (2 * shared * c + N) / (2 * N) : 0); };
    const int64_t i = blockIdx.x;
    const int64_t a0 = first_cta(lane, incl - g), a1 = first_cta(lane + 1, incl);
    const uint64_t hit = __ballot(lane < batch && a0 <= i && i < a1);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      const int bb = __builtin_amdgcn_readfirstlane(l);
      const int LL = __builtin_amdgcn_readfirstlane(__shfl(L, l));
      const int gg = __builtin_amdgcn_readfirstlane(__shfl(g, l));
      const int n = static_cast<int>(uniform64(__shfl(a1 - a0, l)));
      const int p = static_cast<int>(i - uniform64(__shfl(a0, l)));
      const int k0 = static_cast<int>(static_cast<int64_t>(p) * gg / n) * kGroupKeys;
      const int k1 = min(static_cast<int>(static_cast<int64_t>(p + 1) * gg / n) * kGroupKeys, LL);
      seg(bb, LL, k0, max(k0, k1), n);
    }
    return;
  }
  int64_t N = 0;  // groups in all
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    int64_t n = b < batch ? groups_of(seq_lens[static_cast<int64_t>(b) * sl_stride], empty_group) : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
    N += uniform64(n);
  }
  const int64_t shared = static_cast<int64_t>(gridDim.x) - batch;
  // CTAs before a request with c groups before it: its index plus round(shared * c / N)
  auto first_cta = [&](int64_t b, int64_t c) { return b + (N > 0 ? (2 * shared * c + N) / (2 * N) : 0); };
  const int64_t i = blockIdx.x;
  int64_t before = 0;  // groups of the requests before this block of 64
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const int L = b < batch ? seq_lens[static_cast<int64_t>(b) * sl_stride] : 0;
    const int g = b < batch ? groups_of(L, empty_group) : 0;
    int64_t incl = g;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const int64_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    const int64_t a0 = first_cta(b, before + incl - g), a1 = first_cta(b + 1, before + incl);
    const uint64_t hit = __ballot(b < batch && a0 <= i && i < a1);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      const int bb = __builtin_amdgcn_readfirstlane(b0 + l);
      const int LL = __builtin_amdgcn_readfirstlane(__shfl(L, l));
      const int gg = __builtin_amdgcn_readfirstlane(__shfl(g, l));
      const int n = static_cast<int>(uniform64(__shfl(a1 - a0, l)));
      const int p = static_cast<int>(i - uniform64(__shfl(a0, l)));
      const int k0 = static_cast<int>(static_cast<int64_t>(p) * gg / n) * kGroupKeys;
      const int k1 = min(static_cast<int>(static_cast<int64_t>(p + 1) * gg / n) * kGroupKeys, LL);
      seg(bb, LL, k0, max(k0, k1), n);
      return;
    }
    before += uniform64(__shfl(incl, 63));
  }
}

// ---------------------------------------------------------------- kernels

// Waves per SIMD each variant is built for (VGPR budget 512 / waves).
template <int NT>
constexpr int kFusedWaves = NT == 1 ? 3 : 2;


template <int NT, class Src>
__device__ __forceinline__ void logits_body(const PagedArgs& a, float* out, int64_t ld, v4i* stage, QLds<NT>* ql) {
  Src src;
  src.bind(stage);
  src.bind_q(ql);
  const int lane = lane_id();
  for_each_segment(a.seq_lens, a.sl_stride, a.batch, a.locate, a.per_request, kLogitsKeysPerCta, false,
                   [&](int b, int L, int k0, int k1, int) {
    src.init(a, b);
    float* row0 = out + static_cast<int64_t>(b) * NT * ld;
    stream_keys<NT, false>(
        src, k0, k1, L,
        [&](int, int p0, const float(&E)[NT]) {
#pragma unroll
          for (int t = 0; t < NT; ++t) row0[t * ld + p0 + lane] = E[t];
        },
        [](int, int) {});
  });
}

template <int NT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFusedWaves<NT>, 8)))
logits_kernel(PagedArgs a, float* out, int64_t ld) {
  __shared__ v4i stage[kWaves * kStageInt4];
  if constexpr (NT >= 3) {
    __shared__ QLds<NT> ql;
    logits_body<NT, KvSourceQ<NT>>(a, out, ld, stage, &ql);
  } else {
    logits_body<NT, KvSource<NT>>(a, out, ld, stage, nullptr);
  }
}

// A wave's n candidate pairs of row r into slots top_k + base + i (those past
// the capacity dropped).  With a Top-k output, candidate j < top_k also writes
// its index to topk_idx[r][j]: a row that ends with exactly k candidates then
// already holds its Top-k in slot order, which the finish kernel keeps; in
// every other case the finish kernel rewrites entries 0 .. top_k - 1.
__device__ __forceinline__ void store_cands(const SelectArgs& s, int r, int base, const int2* list, int n) {
  int32_t* slots = s.candidates + (static_cast<int64_t>(r) * (s.top_k + s.capacity) + s.top_k) * 2;
  int32_t* out = s.topk_idx ? s.topk_idx + static_cast<int64_t>(r) * s.top_k : nullptr;
  for (int i = lane_id(); i < n; i += 64) {
    const int j = base + i;
    const int2 e = list[i];
    if (j < s.capacity) *reinterpret_cast<int2*>(slots + 2 * j) = e;
    if (out && j < s.top_k) out[j] = e.x;
  }
}

// The select kernels' CTA body: score keys [k0, k1) of the CTA's request and
// select each wave's 64-key groups straight from the scores in registers onto
// the wave's own lists, which reach the slots when nearly full (one counter
// atomic per list) and at the end (one atomic per row and class for the whole
// CTA, after the only barrier).  Whatever follows -- fit test,
// repair, ranges, Top-k -- is the finish kernel's.
template <int NT, int kKeysPerCta, class Src, class Args>
__device__ __forceinline__ void select_body(const Args& a, const SelectArgs& s, MainShared<NT>& sh, v4i* stage,
                                            QLds<NT>* ql) {
  Src src;
  src.bind(stage);
  src.bind_q(ql);
  const int lane = lane_id();
  const int w = wave_id();
  for_each_segment(a.seq_lens, a.sl_stride, a.batch, a.locate, a.per_request, kKeysPerCta, true,
                   [&](int b, int L, int k0, int k1, int) {
    float thr[NT];
    int lim[NT];
    int ncl[NT], ntl[NT];  // entries in this wave's lists (wave-uniform)
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      thr[t] = s.thresholds[b * NT + t];
      lim[t] = min(k1, max(0, L - NT + t + 1));
      ncl[t] = 0;
      ntl[t] = 0;
    }
    // A wave's list of row t into the row's slots: one atomic per class for
    // the base, then the pairs at base + i (dropped past the slots).
    auto flush = [&](int t) {
      const int r = b * NT + t;
      int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + s.capacity) * 2;
      uint64_t old = 0;
      if (lane == 0) old = reserve_pair(s.counters + 2 * r, ncl[t], ntl[t]);
      const int bc = __shfl(static_cast<int>(static_cast<uint32_t>(old)), 0);
      const int bt = __shfl(static_cast<int>(static_cast<uint32_t>(old >> 32)), 0);
      store_cands(s, r, bc, sh.cand[w][t], ncl[t]);
      for (int i = lane; i < ntl[t]; i += 64)
        if (bt + i < s.top_k) *reinterpret_cast<int2*>(slots + 2 * (s.top_k - 1 - bt - i)) = sh.tie[w][t][i];
      ncl[t] = 0;
      ntl[t] = 0;
    };
    src.init(a, b);
    stream_keys<NT, false>(
        src, k0, k1, L,
        [&](int, int p0, const float(&E)[NT]) {
          // this group's candidates and ties onto the wave's lists, positions
          // from the ballots
          const int p = p0 + lane;
          if (s.keep && p < k1) {
#pragma unroll
            for (int t = 0; t < NT; ++t) s.keep[static_cast<int64_t>(b * NT + t) * s.score_ld + p] = E[t];
          }
          bool flushed = false;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float e = E[t];
            const bool vis = p < lim[t];
            const bool cand = vis && e > thr[t];
            const bool tie = vis && !(e > thr[t]) && !(e < thr[t]);
            const uint64_t mc = __ballot(cand);
            const uint64_t mt = __ballot(tie);
            const int nc = __popcll(mc);
            const int nt = __popcll(mt);
            if (ncl[t] + nc > kWaveCand<NT> || ntl[t] + nt > kWaveTie<NT>) {
              flush(t);
              flushed = true;
            }
            if (cand) sh.cand[w][t][ncl[t] + lanes_below(mc)] = int2{p, __float_as_int(enc_cand(e, thr[t]))};
            if (tie) sh.tie[w][t][ntl[t] + lanes_below(mt)] = int2{p, __float_as_int(e - thr[t])};
            ncl[t] += nc;
            ntl[t] += nt;
          }
          // a flush's stores and atomics complete here, so that the loop's
          // waits keep counting only key loads
          if (flushed) wait_vm_done();
        },
        [](int, int) {});
    // the end: the four waves' lists of a row share one counter atomic per
    // class (with every CTA finishing at about the same time, per-wave atomics
    // pile up on the rows' counter words)
    if (lane == 0) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        sh.count[w][t][0] = ncl[t];
        sh.count[w][t][1] = ntl[t];
      }
    }
    __syncthreads();
    if (threadIdx.x < NT) {
      const int t = threadIdx.x;
      int tc = 0, tt = 0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        tc += sh.count[q][t][0];
        tt += sh.count[q][t][1];
      }
      const uint64_t old = (tc | tt) ? reserve_pair(s.counters + 2 * (b * NT + t), tc, tt) : 0;
      sh.base[t][0] = static_cast<int>(static_cast<uint32_t>(old));
      sh.base[t][1] = static_cast<int>(static_cast<uint32_t>(old >> 32));
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int bc = sh.base[t][0], bt = sh.base[t][1];
      for (int q = 0; q < w; ++q) {
        bc += sh.count[q][t][0];
        bt += sh.count[q][t][1];
      }
      int32_t* slots = s.candidates + static_cast<int64_t>(b * NT + t) * (s.top_k + s.capacity) * 2;
      store_cands(s, b * NT + t, bc, sh.cand[w][t], ncl[t]);
      for (int i = lane; i < ntl[t]; i += 64)
        if (bt + i < s.top_k) *reinterpret_cast<int2*>(slots + 2 * (s.top_k - 1 - bt - i)) = sh.tie[w][t][i];
    }
  });
  // (last: its layout check is a load the CTA's start would otherwise wait
  // for before it reads the lengths; the finish kernel starts after this one)
  if (s.ws) prepare_workspace<NT>(s, a.batch);
}


template <int NT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFusedWaves<NT>, 8)))
fused_kernel(PagedArgs a, SelectArgs s) {
  __shared__ MainShared<NT> sh;
  __shared__ v4i stage[kWaves * kStageInt4];
  if constexpr (NT >= 3) {
    __shared__ QLds<NT> ql;
    select_body<NT, kFusedKeysPerCta, KvSourceQ<NT>>(a, s, sh, stage, &ql);
  } else {
    select_body<NT, kFusedKeysPerCta, KvSource<NT>>(a, s, sh, stage, nullptr);
  }
}

template <int NT>
__global__ void __launch_bounds__(kThreads) select_kernel(LogitsArgs a, SelectArgs s) {
  __shared__ MainShared<NT> sh;
  select_body<NT, kSelectKeysPerCta, LogitsSource<NT>>(a, s, sh, nullptr, nullptr);
}

// For next_n = 1 two CTAs fit on a compute unit (by LDS and, capped here, by
// registers).
template <int NT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(NT == 1 ? 2 : 1, 8)))
fused_finish_kernel(PagedArgs a, SelectArgs s) {
  __shared__ CtaShared<NT> sh;
  __shared__ v4i stage[kWaves * kStageInt4];
  finish_body<NT, true>(a, s, sh, stage);
}

template <int NT>
__global__ void __launch_bounds__(kThreads) select_finish_kernel(LogitsArgs a, SelectArgs s) {
  __shared__ CtaShared<NT> sh;
  finish_body<NT, false>(a, s, sh, nullptr);
}

// ---------------------------------------------------------------- host side

namespace {

int log2_exact(int v) {
  int s = 0;
  while ((1 << s) < v) ++s;
  return s;
}

bool validate_enabled() {
  const char* v = std::getenv("PMQA_VALIDATE");
  return v && v[0] == '1' && v[1] == '\0';
}

bool stream_capturing(hipStream_t st) {
  hipStreamCaptureStatus cs = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(st, &cs) != hipSuccess) return true;
  return cs != hipStreamCaptureStatusNone;
}

template <class T>
bool copy_span(std::vector<T>& host, const T* dev, int64_t count, hipStream_t st) {
  host.resize(static_cast<size_t>(count));
  if (count == 0) return true;
  return hipMemcpyAsync(host.data(), dev, sizeof(T) * count, hipMemcpyDeviceToHost, st) == hipSuccess;
}

// PMQA_VALIDATE=1: device-content preconditions, checked on a host copy.
pmqa_status validate_content(hipStream_t st, const int32_t* seq_lens, int64_t sl_stride, int32_t B,
                             int32_t limit, const int32_t* bt, int64_t bt_stride, int32_t bt_width,
                             int32_t bs, int64_t num_blocks, const int32_t* counters, int64_t rows,
                             const int32_t* arrivals) {
  if (!validate_enabled() || stream_capturing(st) || B == 0) return PMQA_OK;
  std::vector<int32_t> L, T, C, A;
  bool ok = copy_span(L, seq_lens, (B - 1) * sl_stride + 1, st);
  if (bt) ok = ok && copy_span(T, bt, (B - 1) * bt_stride + bt_width, st);
  if (counters) ok = ok && copy_span(C, counters, 2 * rows, st);
  if (arrivals) ok = ok && copy_span(A, arrivals, static_cast<int64_t>(B), st);
  if (!ok || hipStreamSynchronize(st) != hipSuccess) return PMQA_ERR_LAUNCH;
  for (int32_t b = 0; b < B; ++b) {
    const int32_t len = L[static_cast<size_t>(b * sl_stride)];
    if (len < 0 || len > limit) return PMQA_ERR_CONTENT;
    if (!bt) continue;
    const int64_t pages = ceil_div(len, bs);
    if (pages > bt_width) return PMQA_ERR_CONTENT;
    for (int64_t j = 0; j < pages; ++j) {
      const int32_t id = T[static_cast<size_t>(b * bt_stride + j)];
      if (id < 0 || id >= num_blocks) return PMQA_ERR_CONTENT;
    }
  }
  for (int32_t v : C)
    if (v != 0) return PMQA_ERR_CONTENT;
  for (int32_t v : A)
    if (v != 0) return PMQA_ERR_CONTENT;
  return PMQA_OK;
}


PagedArgs paged_args(const uint8_t* q, const uint8_t* kv, const float* w, const int32_t* bt,
                     int64_t bt_stride, const int32_t* sl, int64_t sl_stride, int32_t bs, int32_t batch,
                     int64_t per_request) {
  PagedArgs a;
  a.batch = batch;
  a.locate = 0;  // chosen at launch
  a.per_request = static_cast<int32_t>(per_request);
  a.q = q;
  a.kv = kv;
  a.w = w;
  a.bt = bt;
  a.bt_stride = bt_stride;
  a.seq_lens = sl;
  a.sl_stride = sl_stride;
  a.bs_shift = log2_exact(bs);
  a.block_bytes = bs * (kDim + 4);
  a.scale_off = bs * kDim;
  return a;
}

// Compute units of the current device (cached per device).
int device_cus() {
  static std::mutex mu;
  static std::map<int, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
  return cache[dev] = std::max(1, cus);
}

// CTAs of kernel `fn` that fit on the device at once (a repair grid).
int resident_ctas(const void* fn) {
  static std::mutex mu;
  static std::map<std::pair<int, const void*>, int> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 1;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, fn);
  auto it = cache.find(key);
  if (it != cache.end()) return it->second;
  int cus = 0, per_cu = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) cus = 1;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, kThreads, 0) != hipSuccess) per_cu = 1;
  const int n = std::max(1, cus) * std::max(1, per_cu);
  cache[key] = n;
  return n;
}

SelectArgs select_args(float* thr, int32_t* cnt, int32_t* cand, int32_t cap, int32_t top_k, int32_t* arr,
                       int32_t* ranges, int32_t* topk, int32_t batch, int32_t rows, int32_t max_context, bool fused,
                       void* workspace, size_t workspace_bytes) {
  SelectArgs s;
  s.thresholds = thr;
  s.counters = cnt;
  s.candidates = cand;
  s.arrivals = arr;
  s.ranges = ranges;
  s.topk_idx = topk;
  s.ws = arr ? static_cast<uint32_t*>(workspace) : nullptr;
  s.ws_words = s.ws ? static_cast<int64_t>(workspace_bytes / 4) : 0;
  s.scores = s.ws && fused ? reinterpret_cast<float*>(s.ws + workspace_state_words(batch, rows)) : nullptr;
  s.score_ld = score_stride(max_context);
  s.keep = nullptr;
  s.capacity = cap;
  s.top_k = top_k;
  s.rows = rows;
  return s;
}

pmqa_status launched() { return hipGetLastError() == hipSuccess ? PMQA_OK : PMQA_ERR_LAUNCH; }


// One launch of K<nt> with scoring arguments `a` first.  A main kernel runs the
// located grid -- as many CTAs as fit on the device at once, but at most 15/8
// per compute unit -- when that is at least twice the batch, else
// a.per_request CTAs per request (PMQA_ERR_SHAPE if that grid is too large); a
// finish kernel always runs as many CTAs as fit.  (The cap: on the 64-request
// decode batch 480 CTAs stream 2.7 us faster than the 768 that fit, whose
// third CTA on each compute unit gets its first keys some 15 us after the
// first and finishes last; 432 and fewer are slower again.)
template <template <int> class K, class A, class... Rest>
pmqa_status launch_k(int nt, bool main, hipStream_t st, A a, Rest... rest) {
  pmqa_status status = PMQA_OK;
  auto go = [&](auto fn) {
    int64_t g = resident_ctas(reinterpret_cast<const void*>(fn));
    if (main) {
      g = std::min<int64_t>(g, static_cast<int64_t>(device_cus()) * 15 / 8);
      a.locate = g >= 2 * static_cast<int64_t>(a.batch);
      if (!a.locate) g = static_cast<int64_t>(a.per_request) * a.batch;
      if (g > 0x7fffffff) {
        status = PMQA_ERR_SHAPE;
        return;
      }
    }
    hipLaunchKernelGGL(fn, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, st, a, rest...);
  };
  switch (nt) {
    case 1: go(K<1>::fn); break;
    case 2: go(K<2>::fn); break;
    case 3: go(K<3>::fn); break;
    default: go(K<4>::fn); break;
  }
  return status;
}

template <int NT> struct LogitsK { static constexpr auto fn = logits_kernel<NT>; };
template <int NT> struct FusedK { static constexpr auto fn = fused_kernel<NT>; };
template <int NT> struct SelectK { static constexpr auto fn = select_kernel<NT>; };
template <int NT> struct FusedFinishK { static constexpr auto fn = fused_finish_kernel<NT>; };
template <int NT> struct SelectFinishK { static constexpr auto fn = select_finish_kernel<NT>; };

}  // namespace
}  // namespace pmqa

using namespace pmqa;

extern "C" {

pmqa_status pmqa_mqa_logits(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                            const int32_t* block_tables, int64_t block_table_stride,
                            int32_t block_table_width, const int32_t* seq_lens, int64_t seq_lens_stride,
                            int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
                            int32_t block_size, int64_t num_blocks, int32_t max_seq_len, float* out,
                            int64_t out_stride, void* stream) {
  pmqa_status st = pmqa_check_logits_args(q, kv_fused, weights, block_tables, block_table_stride,
                                          block_table_width, seq_lens, seq_lens_stride, batch_size, next_n,
                                          num_heads, head_dim, block_size, num_blocks, max_seq_len, out,
                                          out_stride);
  if (st != PMQA_OK) return st;
  if (batch_size > 65535) return PMQA_ERR_SHAPE;
  const int64_t gx = ceil_div(max_seq_len, kLogitsKeysPerCta);
  if (batch_size == 0 || gx == 0) return PMQA_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = validate_content(hs, seq_lens, seq_lens_stride, batch_size, max_seq_len, block_tables,
                        block_table_stride, block_table_width, block_size, num_blocks, nullptr, 0, nullptr);
  if (st != PMQA_OK) return st;
  const PagedArgs a = paged_args(q, kv_fused, weights, block_tables, block_table_stride, seq_lens,
                                 seq_lens_stride, block_size, batch_size, gx);
  st = launch_k<LogitsK>(next_n, true, hs, a, out, out_stride);
  return st != PMQA_OK ? st : launched();
}

pmqa_status pmqa_indexer_topk(const float* logits, int64_t logits_stride, const int32_t* seq_lens,
                              int64_t seq_lens_stride, int32_t batch_size, int32_t next_n, int32_t max_context,
                              float* thresholds, int32_t* counters, int32_t* candidates, int32_t capacity,
                              int32_t top_k, int32_t* arrivals, int32_t* ranges, int32_t* topk_idx,
                              void* workspace, size_t workspace_bytes, void* stream) {
  pmqa_status st = pmqa_check_select_args(logits, logits_stride, seq_lens, seq_lens_stride, batch_size, next_n,
                                          max_context, thresholds, counters, candidates, capacity, top_k,
                                          arrivals, ranges, topk_idx, workspace, workspace_bytes);
  if (st != PMQA_OK) return st;
  if (batch_size > 65535) return PMQA_ERR_SHAPE;
  if (batch_size == 0) return PMQA_OK;
  const int64_t gx = std::max<int64_t>(1, ceil_div(max_context, kSelectKeysPerCta));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t rows = static_cast<int64_t>(batch_size) * next_n;
  st = validate_content(hs, seq_lens, seq_lens_stride, batch_size, max_context, nullptr, 0, 0, 1, 0, counters,
                        rows, arrivals);
  if (st != PMQA_OK) return st;
  const LogitsArgs a{logits, logits_stride, seq_lens, seq_lens_stride, batch_size, 0, static_cast<int32_t>(gx)};
  const SelectArgs s = select_args(thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx,
                                   batch_size, static_cast<int32_t>(rows), max_context, false, workspace,
                                   workspace_bytes);
  st = launch_k<SelectK>(next_n, true, hs, a, s);
  if (st == PMQA_OK && s.ws) st = launch_k<SelectFinishK>(next_n, false, hs, a, s);
  return st != PMQA_OK ? st : launched();
}

pmqa_status pmqa_fused_logits_select(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                     const int32_t* block_tables, int64_t block_table_stride,
                                     int32_t block_table_width, const int32_t* seq_lens, int64_t seq_lens_stride,
                                     int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
                                     int32_t block_size, int64_t num_blocks, int32_t max_context,
                                     float* thresholds, int32_t* counters, int32_t* candidates, int32_t capacity,
                                     int32_t top_k, int32_t* arrivals, int32_t* ranges, int32_t* topk_idx,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  pmqa_status st = pmqa_check_fused_args(q, kv_fused, weights, block_tables, block_table_stride,
                                         block_table_width, seq_lens, seq_lens_stride, batch_size, next_n,
                                         num_heads, head_dim, block_size, num_blocks, max_context, thresholds,
                                         counters, candidates, capacity, top_k, arrivals, ranges, topk_idx,
                                         workspace, workspace_bytes);
  if (st != PMQA_OK) return st;
  if (batch_size > 65535) return PMQA_ERR_SHAPE;
  if (batch_size == 0) return PMQA_OK;
  const int64_t gx = std::max<int64_t>(1, ceil_div(max_context, kFusedKeysPerCta));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t rows = static_cast<int64_t>(batch_size) * next_n;
  st = validate_content(hs, seq_lens, seq_lens_stride, batch_size, max_context, block_tables, block_table_stride,
                        block_table_width, block_size, num_blocks, counters, rows, arrivals);
  if (st != PMQA_OK) return st;
  const PagedArgs a = paged_args(q, kv_fused, weights, block_tables, block_table_stride, seq_lens,
                                 seq_lens_stride, block_size, batch_size, gx);
  SelectArgs s = select_args(thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx,
                             batch_size, static_cast<int32_t>(rows), max_context, true, workspace, workspace_bytes);
  // With next_n >= 2 the main pass also writes every score into the
  // workspace's score buffer (4 * next_n bytes a key against 132 read), and
  // the finish stage is the one of a select over a logits matrix, run on that
  // buffer: a repair then reads 4-byte scores instead of scoring its requests
  // again from the KV pages (next_n = 1 keeps the re-scoring repair: there
  // the writes would cost more than the rare repair saves).
  const bool keep = s.ws && next_n >= 2;
  if (keep) s.keep = s.scores;
  st = launch_k<FusedK>(next_n, true, hs, a, s);
  if (st == PMQA_OK && s.ws) {
    if (keep) {
      const LogitsArgs la{s.scores, s.score_ld, seq_lens, seq_lens_stride, batch_size, 0, 1};
      SelectArgs sf = s;
      sf.scores = nullptr;
      sf.keep = nullptr;
      st = launch_k<SelectFinishK>(next_n, false, hs, la, sf);
    } else {
      st = launch_k<FusedFinishK>(next_n, false, hs, a, s);
    }
  }
  return st != PMQA_OK ? st : launched();
}

}  // extern "C"
