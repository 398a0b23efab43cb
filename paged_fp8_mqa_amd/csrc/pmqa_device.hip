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
// Entries of a wave's list per row: candidates from the front, ties and
// near-band keys from the back; a list is flushed when a group's entries would
// not fit, so an empty list must hold a whole group's (at most 64).
template <int NT> constexpr int kWaveList = NT >= 3 ? 96 : 320;
static_assert(kWaveList<3> >= 64, "a group's entries fit an empty list");

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
  int32_t fast_ctas;    // located grids: the CTAs dispatched first, one per compute unit
  // prefill-shaped rows (both null for decode rows): tile b's rows b*NT + t
  // see keys below row_ends[b*NT + t] of request tile_req[b]
  const int32_t* row_ends;
  const int32_t* tile_req;
  // MXFP4 pools only: q's UE8M0 scales (one int32 of four per (row, head)) and
  // whether a block's scale slots are interleaved
  const int32_t* qsf;
  int32_t sf_inter;
};

struct LogitsArgs {
  const float* logits;
  int64_t ld;
  const int32_t* seq_lens;
  int64_t sl_stride;
  int32_t batch;
  int32_t locate;
  int32_t per_request;
  int32_t fast_ctas;
};

struct SelectArgs {
  float* thresholds;
  int32_t* counters;
  int32_t* candidates;
  int32_t* arrivals;    // [batch] per-tile arrival counters (with the finish stage), else null
  int32_t* ranges;
  int32_t* topk_idx;
  uint32_t* ws;         // workspace (with arrivals), else null
  int32_t* ovf;         // its overflow pairs, row r at ovf + r * 2 * kOverflowPairs (null without)
  int32_t* nearp;       // its near-band pairs, row r at nearp + r * 2 * kNearPairs (null without)
  uint32_t* nearc;      // row r's near-band count at nearc[r * kRowWords] (a row state word)
  float* scores;        // fused repair: the workspace's score rows, row r at scores + r * score_ld
  int64_t score_ld;
  int32_t capacity;
  int32_t top_k;
  int32_t rows;
  int32_t resident;     // 1 when every CTA of the launch fits on the device at once (CTAs
                        // without work then wait a while for repair items before they leave)
  const int32_t* row_ends;  // prefill-shaped rows: each row's key end (null: derived from the length)
};

// Address-space views.  A generic pointer passed through in_global() is known
// to the compiler to address global memory, and one derived from an LdsByte
// pointer to address LDS, so their accesses compile to global_* and ds_*
// instructions rather than flat_* ones (which wait on both the vector-memory
// and the LDS counters, and reach LDS through the vector-memory path).
typedef __attribute__((address_space(3))) char LdsByte;
typedef __attribute__((address_space(1))) char GlobalByte;
template <class T>
__device__ __forceinline__ T* in_global(T* p) {
  return (T*)((GlobalByte*)((char*)p));
}

__device__ __forceinline__ void global_view(PagedArgs& a) {
  a.q = in_global(a.q);
  a.kv = in_global(a.kv);
  a.w = in_global(a.w);
  a.bt = in_global(a.bt);
  a.seq_lens = in_global(a.seq_lens);
  a.row_ends = in_global(a.row_ends);
  a.tile_req = in_global(a.tile_req);
  a.qsf = in_global(a.qsf);
}
__device__ __forceinline__ void global_view(LogitsArgs& a) {
  a.logits = in_global(a.logits);
  a.seq_lens = in_global(a.seq_lens);
}
__device__ __forceinline__ void global_view(SelectArgs& s) {
  s.thresholds = in_global(s.thresholds);
  s.counters = in_global(s.counters);
  s.candidates = in_global(s.candidates);
  s.arrivals = in_global(s.arrivals);
  s.ranges = in_global(s.ranges);
  s.topk_idx = in_global(s.topk_idx);
  s.ws = in_global(s.ws);
  s.ovf = in_global(s.ovf);
  s.nearp = in_global(s.nearp);
  s.nearc = in_global(s.nearc);
  s.scores = in_global(s.scores);
  s.row_ends = in_global(s.row_ends);
}

// The keys tile b streams: its request's length for decode rows, the largest
// of its rows' ends for prefill-shaped rows.
template <int NT>
__device__ __forceinline__ int tile_keys(const PagedArgs& a, int b) {
  if (a.row_ends) {
    int m = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t) m = max(m, a.row_ends[static_cast<int64_t>(b) * NT + t]);
    return m;
  }
  return a.seq_lens[static_cast<int64_t>(b) * a.sl_stride];
}
template <int NT>
__device__ __forceinline__ int tile_keys(const LogitsArgs& a, int b) {
  return a.seq_lens[static_cast<int64_t>(b) * a.sl_stride];
}

// Row t of tile b (L keys streamed) sees keys below its end: L - NT + t + 1
// for decode rows (page "flashinfer.attn_scores", Note), row_ends[r] for
// prefill-shaped rows (page "flashinfer.sdsa.indexer_threshold_select",
// Parameters: row_ends).
template <int NT>
__device__ __forceinline__ int row_end(const SelectArgs& s, int b, int L, int t) {
  return s.row_ends ? max(0, s.row_ends[static_cast<int64_t>(b) * NT + t]) : max(0, L - NT + t + 1);
}

__device__ __forceinline__ int wave_id() { return __builtin_amdgcn_readfirstlane(threadIdx.x >> 6); }
__device__ __forceinline__ int lane_id() { return threadIdx.x & 63; }

__device__ __forceinline__ int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi(static_cast<uint32_t>(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo(static_cast<uint32_t>(mask), 0));
}

// Wavefront minimum (the device library's DPP reduction); every lane gets it.
extern "C" __device__ uint64_t __ockl_wfred_min_u64(uint64_t);
// Wavefront min / max / prefix sum by DPP lane moves (the device library's
// reductions and scans; no LDS round trips).
extern "C" __device__ uint32_t __ockl_wfred_min_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfred_max_u32(uint32_t);
extern "C" __device__ uint32_t __ockl_wfscan_add_u32(uint32_t, bool inclusive);

// s_waitcnt vmcnt(0): this wave's loads and stores have completed.
__device__ __forceinline__ void wait_vm_done() { __builtin_amdgcn_s_waitcnt(0x0F70); }

// Optional event trace (built only with PMQA_TRACE defined; the product build
// compiles every trace point to nothing): thread 0 of each of the first
// kTraceCtas CTAs records up to kTraceSlots events (kind, two small
// arguments, s_memrealtime) at g_trace[cta * kTraceSlots + i], read back with
// pmqa_trace_read.
#ifdef PMQA_TRACE
constexpr int kTraceCtas = 2048;
constexpr int kTraceSlots = 64;
__device__ uint64_t g_trace[kTraceCtas * kTraceSlots];
// events are kept in the CTA's control words and written out when it ends, so
// that the trace adds no global stores for later barriers to wait on
template <class C>
__device__ __forceinline__ void trace_event(C* c, int kind, int x, int y) {
  if (threadIdx.x == 0 && c->trace_n < kTraceSlots) {
    const uint64_t t = __builtin_amdgcn_s_memrealtime();
    c->trace_ev[c->trace_n] = (static_cast<uint64_t>(kind & 0xff) << 56) | (static_cast<uint64_t>(x & 0xffff) << 40) |
                              (static_cast<uint64_t>(y & 0xff) << 32) | (t & 0xffffffffu);
    ++c->trace_n;
  }
}
template <class C>
__device__ __forceinline__ void trace_flush(C* c) {
  if (threadIdx.x == 0 && blockIdx.x < kTraceCtas)
    for (int i = 0; i < c->trace_n; ++i) g_trace[blockIdx.x * kTraceSlots + i] = c->trace_ev[i];
}
#define PMQA_TR(sh, kind, x, y) trace_event((sh).c, (kind), (x), (y))
#else
#define PMQA_TR(sh, kind, x, y) ((void)0)
#endif

// Words shared between the CTAs of one kernel (on any XCD) are written with
// agent-scope atomic stores, which the storing XCD's L2 writes through, and
// read with agent-scope atomic loads.
typedef __attribute__((address_space(1))) uint32_t GlobalU32;
typedef __attribute__((address_space(1))) uint64_t GlobalU64;
typedef __attribute__((address_space(3))) uint32_t LdsU32;
typedef __attribute__((address_space(3))) int32_t LdsI32;
__device__ __forceinline__ uint32_t ld_ag(const uint32_t* p) {
  return __hip_atomic_load((const GlobalU32*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_ag64(const uint64_t* p) {
  return __hip_atomic_load((const GlobalU64*)p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt(uint32_t* p, uint32_t v) {
  __hip_atomic_store((GlobalU32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_wt64(uint64_t* p, uint64_t v) {
  __hip_atomic_store((GlobalU64*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A slot pair (key index, score bits) from global memory, as one 8-byte load.
__device__ __forceinline__ int2 ld_pair(const int32_t* p) {
  const uint64_t v = *(const GlobalU64*)p;
  return make_int2(static_cast<int>(static_cast<uint32_t>(v)), static_cast<int>(static_cast<uint32_t>(v >> 32)));
}

// Agent-scope atomic adds on global memory; they return the old value.
__device__ __forceinline__ uint32_t add_ag(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add((GlobalU32*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ int32_t add_ag(int32_t* p, int32_t v) {
  return static_cast<int32_t>(add_ag(reinterpret_cast<uint32_t*>(p), static_cast<uint32_t>(v)));
}
__device__ __forceinline__ uint64_t add_ag64(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_add((GlobalU64*)p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// A uniform word read by a returning agent-scope atomic (an add of a zero the
// compiler cannot see, so that it stays an atomic; lane 0 of the wave, every
// lane active, the value broadcast): performed where the device's atomics
// are, it returns the word's current value whatever copy of its line a cache
// may hold.  Slower than an agent-scope load, so kept off the usual paths.
__device__ __forceinline__ uint32_t rd_cur_wave(const uint32_t* p) {
  uint32_t z = 0u;
  asm volatile("" : "+v"(z));
  uint32_t v = 0u;
  if ((threadIdx.x & 63) == 0) v = add_ag(const_cast<uint32_t*>(p), z);
  return __builtin_amdgcn_readfirstlane(v);
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
    const int req = a.tile_req ? a.tile_req[b] : b;
    bt_row = a.bt + static_cast<int64_t>(req) * a.bt_stride;
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

// The epilogue's precision (page "flashinfer.attn_scores", fp8_paged_mqa_logits,
// acc_dtype and epi_dtype).  Each policy turns one MFMA result (four heads of
// one key) into a running partial (head_sum, in head order), and a lane's four
// column tiles' partials into the score of key p0 + lane (finish: the
// reduce-scatter over the four lane groups, then the scale multiply).
//   kEpiF32    float32 throughout (the fused select and pmqa_mqa_logits);
//   kEpiAcc16  each dot product rounded to float16, then the float32 epilogue;
//   kEpiF16    the dot products, weights and scale rounded to float16 and
//              every product and sum a float16 operation, two heads per packed
//              instruction.
constexpr int kEpiF32 = 0;
constexpr int kEpiAcc16 = 1;
constexpr int kEpiF16 = 2;

typedef _Float16 h2 __attribute__((ext_vector_type(2)));
typedef short s2 __attribute__((ext_vector_type(2)));

// max(x, 0) of both halves as a 16-bit integer max on the bit patterns (the
// float32 relu's rule: a negative sign bit gives +0).
__device__ __forceinline__ h2 relu2(h2 x) {
  return __builtin_bit_cast(h2, __builtin_elementwise_max(__builtin_bit_cast(s2, x), s2{0, 0}));
}

__device__ __forceinline__ _Float16 shfl_xor_h(_Float16 v, int m) {
  const int x = __shfl_xor(static_cast<int>(__builtin_bit_cast(unsigned short, v)), m);
  return __builtin_bit_cast(_Float16, static_cast<unsigned short>(x));
}

template <int kEpi>
struct Epi {
  using Acc = float;
  using W = float4;
  __device__ static Acc zero() { return 0.f; }
  __device__ static W weights(float4 w) { return w; }
  __device__ static float dot(float x) {
    if constexpr (kEpi == kEpiAcc16) return static_cast<float>(static_cast<_Float16>(x));
    else return x;
  }
  __device__ static Acc head_sum(v4f acc, W w, Acc sum) {
    if constexpr (kEpi == kEpiF32) {
      return pmqa::head_sum(acc, w, sum);
    } else {
      sum = __builtin_fmaf(relu(dot(acc[0])), w.x, sum);
      sum = __builtin_fmaf(relu(dot(acc[1])), w.y, sum);
      sum = __builtin_fmaf(relu(dot(acc[2])), w.z, sum);
      return __builtin_fmaf(relu(dot(acc[3])), w.w, sum);
    }
  }
  __device__ static float finish(Acc x0, Acc x1, Acc x2, Acc x3, int g, float s) {
    return reduce_scatter4(x0, x1, x2, x3, g) * s;
  }
};

template <>
struct Epi<kEpiF16> {
  using Acc = h2;  // two heads' running sums
  struct W {
    h2 lo, hi;  // weights of the lane's heads 0-1 and 2-3 of a tile
  };
  __device__ static Acc zero() { return h2{0, 0}; }
  __device__ static W weights(float4 w) {
    return W{h2{static_cast<_Float16>(w.x), static_cast<_Float16>(w.y)},
             h2{static_cast<_Float16>(w.z), static_cast<_Float16>(w.w)}};
  }
  __device__ static Acc head_sum(v4f acc, W w, Acc sum) {
    typedef float f2 __attribute__((ext_vector_type(2)));
    const h2 a01 = relu2(__builtin_convertvector((f2{acc[0], acc[1]}), h2));
    const h2 a23 = relu2(__builtin_convertvector((f2{acc[2], acc[3]}), h2));
    sum = __builtin_elementwise_fma(a01, w.lo, sum);
    return __builtin_elementwise_fma(a23, w.hi, sum);
  }
  // the two halves of each tile's partial, then the float32 path's
  // reduce-scatter in float16, then the scale
  __device__ static float finish(Acc x0, Acc x1, Acc x2, Acc x3, int g, float s) {
    const _Float16 y[4] = {x0.x + x0.y, x1.x + x1.y, x2.x + x2.y, x3.x + x3.y};
    const bool hi2 = (g & 2) != 0;
    const _Float16 a = (hi2 ? y[2] : y[0]) + shfl_xor_h(hi2 ? y[0] : y[2], 32);
    const _Float16 b = (hi2 ? y[3] : y[1]) + shfl_xor_h(hi2 ? y[1] : y[3], 32);
    const bool hi1 = (g & 1) != 0;
    const _Float16 r = (hi1 ? b : a) + shfl_xor_h(hi1 ? a : b, 16);
    return static_cast<float>(r * static_cast<_Float16>(s));
  }
};

// bfloat16 epilogue (the MXFP4 logits): the float32 operations with every
// result rounded to bfloat16 (nearest even): the dot products, the weights,
// each fused product-and-sum, each partial of the reduce-scatter, the scale
// multiply.  A fused result rounded from float32 to bfloat16 is rounded twice.
constexpr int kEpiBf16 = 3;

__device__ __forceinline__ float round_bf16(float x) { return static_cast<float>(static_cast<__bf16>(x)); }

template <>
struct Epi<kEpiBf16> {
  using Acc = float;
  using W = float4;
  __device__ static Acc zero() { return 0.f; }
  __device__ static W weights(float4 w) {
    return float4{round_bf16(w.x), round_bf16(w.y), round_bf16(w.z), round_bf16(w.w)};
  }
  __device__ static Acc head_sum(v4f acc, W w, Acc sum) {
    sum = round_bf16(__builtin_fmaf(relu(round_bf16(acc[0])), w.x, sum));
    sum = round_bf16(__builtin_fmaf(relu(round_bf16(acc[1])), w.y, sum));
    sum = round_bf16(__builtin_fmaf(relu(round_bf16(acc[2])), w.z, sum));
    return round_bf16(__builtin_fmaf(relu(round_bf16(acc[3])), w.w, sum));
  }
  __device__ static float finish(Acc x0, Acc x1, Acc x2, Acc x3, int g, float s) {
    const bool hi2 = (g & 2) != 0;
    const float a = round_bf16((hi2 ? x2 : x0) + __shfl_xor(hi2 ? x0 : x2, 32));
    const float b = round_bf16((hi2 ? x3 : x1) + __shfl_xor(hi2 ? x1 : x3, 32));
    const bool hi1 = (g & 1) != 0;
    const float r = round_bf16((hi1 ? b : a) + __shfl_xor(hi1 ? a : b, 16));
    return round_bf16(r * round_bf16(s));
  }
};

// Scores computed from the paged KV pool, the A operands (q) and the lane's 16
// weights per row held in VGPRs (next_n up to 2, and the repair).
template <int NT>
struct QLds;

template <int NT, int kEpi = kEpiF32>
struct KvSource : KvStream {
  using E = Epi<kEpi>;
  v8i qa[NT][4];                 // A operands: rows t, head tiles mt
  typename E::W wt[NT][4];       // weights of heads 16*mt + 4*g .. +3

  __device__ __forceinline__ void bind_q(QLds<NT>*) {}

  __device__ __forceinline__ void init(const PagedArgs& a, int b) {
    init_stream(a, b);
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = static_cast<int64_t>(b) * NT + t;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        qa[t][mt] = load32(a.q + ((row * kHeads + 16 * mt + n) * kDim + 32 * g));
        wt[t][mt] = E::weights(*reinterpret_cast<const float4*>(a.w + row * kHeads + 16 * mt + 4 * g));
      }
    }
  }

  // One row's operands (NT == 1): absolute row r = b * next_n + t of q and the
  // weights, with the stream of request b (the repair's scoring of one row).
  __device__ __forceinline__ void init_row(const PagedArgs& a, int b, int64_t r) {
    static_assert(NT == 1, "one row");
    init_stream(a, b);
#pragma unroll
    for (int mt = 0; mt < 4; ++mt) {
      qa[0][mt] = load32(a.q + ((r * kHeads + 16 * mt + n) * kDim + 32 * g));
      wt[0][mt] = E::weights(*reinterpret_cast<const float4*>(a.w + r * kHeads + 16 * mt + 4 * g));
    }
  }

  // out[t] = score of key p0 + lane for row t.  Fixed operation order, shared
  // by every kernel, so the logits, fused and repair paths agree bit for bit.
  __device__ __forceinline__ void score(const Group& gr, float (&out)[NT]) const {
    v8i bk[4];
    operands(gr, bk);
    typename E::Acc part[NT][4];
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
        typename E::Acc sum = E::zero();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sum = E::head_sum(acc[t][mt], wt[t][mt], sum);
        part[t][j] = sum;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) out[t] = E::finish(part[t][0], part[t][1], part[t][2], part[t][3], g, gr.s);
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
// fit two.  The first kRegRows rows keep their q in VGPRs all the same (only
// their weights are read from LDS): every 64-key group reads each LDS row's q
// (8 KB a wave) again, and those reads bound the loop.  Same operation order
// as KvSource, so the same bits.
template <int NT, int kEpi = kEpiF32, int kRegRows = 0>
struct KvSourceQ : KvStream {
  using E = Epi<kEpi>;
  QLds<NT>* ql;
  v8i qr[kRegRows > 0 ? kRegRows : 1][4];  // A operands of rows t < kRegRows

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
#pragma unroll
    for (int t = 0; t < kRegRows; ++t) {
      const int64_t row = static_cast<int64_t>(b) * NT + t;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) qr[t][mt] = load32(a.q + ((row * kHeads + 16 * mt + n) * kDim + 32 * g));
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
    if constexpr (t >= kRegRows) {
      const v4i lo = ql->q[t][mt][0][lane];
      const v4i hi = ql->q[t][mt][1][lane];
      p.qa[k % 3] = v8i{lo.x, lo.y, lo.z, lo.w, hi.x, hi.y, hi.z, hi.w};
    }
    p.wv[k % 3] = ql->w[t][mt][g];
  }
  template <int k>
  __device__ __forceinline__ void mm(Pipe& p, const v8i (&bk)[4]) const {
    constexpr int t = k >> 2, mt = k & 3;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      if constexpr (t < kRegRows) p.acc[k & 1][j] = mfma_fp8(qr[t < kRegRows ? t : 0][mt], bk[j]);
      else p.acc[k & 1][j] = mfma_fp8(p.qa[k % 3], bk[j]);
    }
  }
  template <int k>
  __device__ __forceinline__ void steps(Pipe& p, const v8i (&bk)[4], typename E::Acc (&part)[NT][4]) const {
    if constexpr (k < 4 * NT) {
      if constexpr (k + 1 < 4 * NT) mm<k + 1>(p, bk);
      __builtin_amdgcn_sched_barrier(0);
      if constexpr (k + 2 < 4 * NT) ld<k + 2>(p);
      __builtin_amdgcn_sched_barrier(0);
      const typename E::W wk = E::weights(p.wv[k % 3]);
#pragma unroll
      for (int j = 0; j < 4; ++j) part[k >> 2][j] = E::head_sum(p.acc[k & 1][j], wk, part[k >> 2][j]);
      // (keeps the steps in this order: left to itself the scheduler hoists
      // every LDS read to the top and runs out of registers)
      __builtin_amdgcn_sched_barrier(0);
      steps<k + 1>(p, bk, part);
    }
  }

  __device__ __forceinline__ void score(const Group& gr, float (&out)[NT]) const {
    v8i bk[4];
    operands(gr, bk);
    typename E::Acc part[NT][4];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
      for (int j = 0; j < 4; ++j) part[t][j] = E::zero();
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
    for (int t = 0; t < NT; ++t) out[t] = E::finish(part[t][0], part[t][1], part[t][2], part[t][3], g, gr.s);
  }
};

// Scores of an MXFP4 pool (page "flashinfer.attn_scores", fp4_paged_mqa_logits:
// the kv_fused figure, q, q_sf and is_kv_sf_interleaved).  A block holds
// block_size * 64 bytes of packed E2M1 values (token i's 64 bytes at i * 64,
// element 2m in the low nibble of byte m) and then block_size * 4 UE8M0 scale
// bytes, token i's at slot i, or with interleaved slots (block size 128) at
// slot 4 * (i % 32) + i / 32; byte k of a token's four scales is the scale of
// elements [32k, 32k + 32).  gfx950's block-scaled MFMA takes exactly that:
// with FP4 operands, lane l of a 16x16x128 step holds 32 elements (16 bytes)
// of row / column l % 16, K block l / 16, and one scale byte for them.  So a
// lane loads its 16 bytes of key p0 + 16j + n straight into the B operand of
// column tile j (each 1 KB run of 16 keys is one wave-wide load), and its scale
// byte g of the key's four; no LDS staging.  The matrix instruction applies
// both sides' scales and accumulates in float32; there is no per-token scale.
struct KvStreamFp4 : KvStream {
  struct Group {
    v4i raw[4];       // column tile j: 16 bytes of key p0 + 16j + n, K block g
    uint32_t sc[4];   // column tile j: the key's four scale bytes
    float s;          // (unused: no per-token scale)
  };
  int sf_inter;

  __device__ __forceinline__ void bind(v4i*) {}
  __device__ __forceinline__ void bind_q(void*) {}

  __device__ __forceinline__ void load(Group& gr, const Pages& pg, int p0) const {
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint8_t* page = j < 2 ? pg.a : pg.b;
      const int slot = (p0 + 16 * j + n) & bs_mask;
      gr.raw[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i*>(page + slot * 64 + 16 * g));
      const int ss = sf_inter ? 4 * (slot & 31) + (slot >> 5) : slot;
      gr.sc[j] = *reinterpret_cast<const uint32_t*>(page + scale_off + 4 * ss);
    }
    gr.s = 1.f;
  }
  __device__ __forceinline__ void load(Group& gr, int p0, int L) const { load(gr, pages(p0, L), p0); }
};

// One 16x16x128 FP4 x FP4 -> f32 MFMA with UE8M0 scales sa (A) and sb (B):
// format code 4 (E2M1) for both operands; only the low 4 dwords of each
// operand are read.
__device__ __forceinline__ v4f mfma_fp4(v8i a, v8i b, int sa, int sb) {
  const v4f z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 4, 4, 0, sa, 0, sb);
}

template <int NT, int kEpi>
struct KvSourceFp4 : KvStreamFp4 {
  using E = Epi<kEpi>;
  v8i qa[NT][4];              // A operands: row t, head tile mt (low 4 dwords)
  int qs[NT][4];              // their scale bytes: head 16*mt + n, K block g
  typename E::W wt[NT][4];    // weights of heads 16*mt + 4*g .. +3

  __device__ __forceinline__ void init(const PagedArgs& a, int b) {
    init_stream(a, b);
    sf_inter = a.sf_inter;
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      const int64_t row = static_cast<int64_t>(b) * NT + t;
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const int64_t head = row * kHeads + 16 * mt + n;
        const v4i v = *reinterpret_cast<const v4i*>(a.q + head * (kDim / 2) + 16 * g);
        qa[t][mt] = v8i{v.x, v.y, v.z, v.w, 0, 0, 0, 0};
        qs[t][mt] = (static_cast<uint32_t>(a.qsf[head]) >> (8 * g)) & 0xff;
        wt[t][mt] = E::weights(*reinterpret_cast<const float4*>(a.w + row * kHeads + 16 * mt + 4 * g));
      }
    }
  }

  // out[t] = score of key p0 + lane for row t.  Per row, the four head tiles'
  // MFMAs of a column tile and then their epilogue (a row's accumulators at a
  // time keep the registers within two waves per SIMD).
  __device__ __forceinline__ void score(const Group& gr, float (&out)[NT]) const {
    typename E::Acc part[NT][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const v8i bk = v8i{gr.raw[j].x, gr.raw[j].y, gr.raw[j].z, gr.raw[j].w, 0, 0, 0, 0};
      const int sb = (gr.sc[j] >> (8 * g)) & 0xff;
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        v4f acc[4];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) acc[mt] = mfma_fp4(qa[t][mt], bk, qs[t][mt], sb);
        typename E::Acc sum = E::zero();
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) sum = E::head_sum(acc[mt], wt[t][mt], sum);
        part[t][j] = sum;
      }
    }
#pragma unroll
    for (int t = 0; t < NT; ++t) out[t] = E::finish(part[t][0], part[t][1], part[t][2], part[t][3], g, 1.f);
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

// The lower end of a threshold's near band: kNearBand radix keys below it
// (about 2^-8 of its magnitude), at least -inf; a NaN threshold has none.
__device__ __forceinline__ float near_floor(float t) {
  const uint32_t k = radix_key(t);
  if (k == 0u) return t;
  return key_to_float(k > 0x00800000u + kNearBand ? k - kNearBand : 0x00800000u);
}

// Adds nc candidates and nt ties to a row's (candidate, tie) counter pair with
// one 64-bit atomic (the pair is 8-byte aligned) and returns the old pair, the
// first slot of each class.  The low word never carries into the high one:
// both counts stay below the row's length, under 2^31.
__device__ __forceinline__ uint64_t reserve_pair(int32_t* pair, int nc, int nt) {
  const uint64_t add = (static_cast<uint64_t>(static_cast<uint32_t>(nt)) << 32) | static_cast<uint32_t>(nc);
  return add_ag64(reinterpret_cast<uint64_t*>(pair), add);
}

// A slot store is an agent-scope (relaxed) atomic store: the L2 of the
// storing XCD writes it through, so no dirty slot line is left in any XCD's L2.
// The tile's last CTA (on any XCD) can then read the slots after its acquire,
// and its own later stores to the same slots cannot be overwritten by a stale
// write-back -- without the L2-wide write-back an agent-scope release fence
// costs on every CTA.
__device__ __forceinline__ void store_pair(int32_t* slot, int idx, float v) {
  const uint64_t packed = (static_cast<uint64_t>(__float_as_uint(v)) << 32) | static_cast<uint32_t>(idx);
  __hip_atomic_store((GlobalU64*)slot, packed, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}


// A slot's final value, written by the row's last writer in the launch and
// read by nothing after it in the launch: an ordinary (write-back) store.  No
// other XCD's L2 holds a dirty copy of the line (every earlier slot store was
// written through), so the write-back at the end of the kernel cannot be
// overwritten by a stale one.
__device__ __forceinline__ void store_final(int32_t* slot, int idx, float v) {
  *(GlobalU64*)slot = (static_cast<uint64_t>(__float_as_uint(v)) << 32) | static_cast<uint32_t>(idx);
}

// Control words of a CTA's finish work (fit test, repair items, row outputs).
template <int NT>
struct Ctl {
  uint32_t wtot[kWaves];
  uint32_t wmin[kWaves];
  uint32_t wmax[kWaves];
  uint32_t sink[64];  // a final select's discarded histogram adds, one word per lane
  uint64_t wmin64[2][kWaves];  // few-extra rounds: each wave's least (key, slot), double-buffered
  uint32_t left_out[8];        // few-extra rounds: the left-out slots
  uint32_t dig[2];
  int32_t wcnt[NT][kWaves][2];
  int32_t wbase[NT][kWaves][2];
  uint32_t pfx[NT];
  uint32_t krem[NT];
  int32_t cnt[NT][2];
  int32_t nc[NT];
  int32_t nt[NT];
  int32_t nn[NT];
  float thr[NT];
  uint32_t repair_mask;
  uint32_t stored_mask;
  int32_t len;
  int32_t is_last;
  int32_t pos[2];
  int32_t job[3];      // claimed repair item: tile (or -1: none open, -2: leave), stage, index
  int32_t next_stage;
  int32_t trace_n;  // events recorded by this CTA (trace builds only)
#ifdef PMQA_TRACE
  uint64_t trace_ev[kTraceSlots];
#endif
};

// The finish work's view of a CTA's LDS: per-row radix histograms (rh, NT of
// them) and, at the same place, one row's radix histogram (fh) with up to
// fin_cap keys or score bits (fk) and key indices (fi) for a final select --
// live at different times -- and the control words (c) in an area of their own.
template <int NT>
struct Sh {
  uint32_t (*rh)[kRadixBins];
  uint32_t* fh;
  uint32_t* fk;
  int32_t* fi;
  int fin_cap;
  Ctl<NT>* c;
};

// Bytes of the finish area for fin_cap final-select entries (at least NT per-row histograms).
__host__ __device__ constexpr int fin_area_bytes(int nt, int fin_cap) {
  return 4 * kRadixBins + 8 * fin_cap > 4 * nt * kRadixBins ? 4 * kRadixBins + 8 * fin_cap : 4 * nt * kRadixBins;
}

template <int NT>
__device__ __forceinline__ Sh<NT> make_sh(char* lds, int fin_cap, int ctl_off) {
  Sh<NT> v;
  v.rh = reinterpret_cast<uint32_t(*)[kRadixBins]>(lds);
  v.fh = reinterpret_cast<uint32_t*>(lds);
  v.fk = v.fh + kRadixBins;
  v.fi = reinterpret_cast<int32_t*>(v.fk + fin_cap);
  v.fin_cap = fin_cap;
  v.c = reinterpret_cast<Ctl<NT>*>(lds + ctl_off);
  return v;
}

// Shared memory of a select kernel CTA: each wave's list per row of (key
// index, stored score bits) pairs not yet written to the row's slots --
// candidates from the front, ties and near-band keys from the back (the finish
// stage's structures stay out, so that the LDS of two CTAs, with their KV
// staging areas, fits on a compute unit).
template <int NT>
struct MainShared {
  int2 list[kWaves][NT][kWaveList<NT>];
  int32_t count[kWaves][NT][3];  // the waves' candidates, ties and near-band keys at the end
  int32_t base[NT][3];           // the CTA's bases per row and class
};

// LDS of a select launch, one buffer seen three ways: the main pass (KV
// staging area, q operands for next_n >= 3, the waves' candidate and tie
// lists), a re-scoring repair item (the same staging area and q operands,
// packed first-pass histograms where the lists were), and the finish view
// (row histograms or one row's final-select keys from offset 0, over the
// staging area); the finish's control words sit after all of them.
template <int NT, bool kFused>
struct Layout {
  static constexpr int kStageBytes = kFused ? kWaves * kStageInt4 * 16 : 0;
  static constexpr int kQBytes = (kFused && NT >= 3) ? static_cast<int>(sizeof(QLds<NT>)) : 0;
  static constexpr int kListOff = kStageBytes + kQBytes;
  static constexpr int kMainEnd = kListOff + static_cast<int>(sizeof(MainShared<NT>));
  static constexpr int kRescoreEnd = kListOff + NT * 2048;
  // the largest final select (a multiple of 256 entries, at least kFinalizeLds)
  // whose area fits where the main pass's buffers are; the select over a
  // logits matrix keeps kFinalizeLds
  static constexpr int kFinCap =
      !kFused ? kFinalizeLds
              : ((kMainEnd - 4 * kRadixBins) / 8 / 256 * 256 < kFinalizeLds ? kFinalizeLds
                                                                               : (kMainEnd - 4 * kRadixBins) / 8 / 256 * 256);
  static constexpr int kFinEnd = fin_area_bytes(NT, kFinCap);
  static constexpr int kCtlOff =
      ((kMainEnd > kFinEnd ? (kMainEnd > kRescoreEnd ? kMainEnd : kRescoreEnd) : (kFinEnd > kRescoreEnd ? kFinEnd : kRescoreEnd)) + 15) / 16 * 16;
  static constexpr int kBytes = kCtlOff + static_cast<int>(sizeof(Ctl<NT>));
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

// Radix pass layout: 10 bits, 11 bits, 11 bits from the top of the key (the
// first pass's 1024 bins fit a re-scoring item's histograms beside the KV
// staging area and the q operands).
__device__ __forceinline__ int pass_shift(int pass) { return pass == 0 ? 22 : (pass == 1 ? 11 : 0); }
__device__ __forceinline__ int pass_bits(int pass) { return pass == 0 ? 10 : 11; }

// The digit of hist[0..nb) (nb = 1024 or 2048, 16-byte aligned) holding the
// krem-th largest entry, and the rank left inside it, found by the whole CTA:
// each thread sums nb / kThreads consecutive bins held in registers, a suffix
// scan over the threads gives the count above each thread's bins, and the one
// thread whose bins reach krem walks them.  The histogram's total is at least
// krem.  Returns the same values in every thread.
template <int NT>
__device__ __forceinline__ void cta_find_digit(uint32_t* hist, int nb, uint32_t krem, const Sh<NT>& sh,
                                               uint32_t& digit, uint32_t& rem, bool zero_after = false) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int per = nb / kThreads;  // 4 or 8
  // thread t holds the per bins below nb - per * t, so that a prefix sum over
  // the threads in order counts from the top bin down
  const int b0 = nb - per * (tid + 1);
  uint32_t h[8];
  const uint4 lo = *reinterpret_cast<const uint4*>(hist + b0);
  const uint4 hi = per == 8 ? *reinterpret_cast<const uint4*>(hist + b0 + 4) : uint4{0u, 0u, 0u, 0u};
  h[0] = lo.x; h[1] = lo.y; h[2] = lo.z; h[3] = lo.w;
  h[4] = hi.x; h[5] = hi.y; h[6] = hi.z; h[7] = hi.w;
  uint32_t local = 0;
#pragma unroll
  for (int i = 0; i < 8; ++i) local += h[i];
  const uint32_t incl = __ockl_wfscan_add_u32(local, true);  // this and the earlier lanes: higher bins
  if (lane == 63) sh.c->wtot[w] = incl;
  if (tid == 0) {
    sh.c->dig[0] = 0u;
    sh.c->dig[1] = 0u;
  }
  __syncthreads();
  // every bin is read: the histogram can be cleared for a next pass (cleared
  // by the barrier below)
  if (zero_after) {
    reinterpret_cast<uint4*>(hist + b0)[0] = uint4{0u, 0u, 0u, 0u};
    if (per == 8) reinterpret_cast<uint4*>(hist + b0)[1] = uint4{0u, 0u, 0u, 0u};
  }
  uint32_t above = incl - local;
  for (int q = 0; q < w; ++q) above += sh.c->wtot[q];
  if (above < krem && krem <= above + local) {
    uint32_t acc = above;
    bool found = false;
#pragma unroll
    for (int i = 7; i >= 0; --i) {
      if (!found && i < per && acc + h[i] >= krem) {
        sh.c->dig[0] = static_cast<uint32_t>(b0 + i);
        sh.c->dig[1] = krem - acc;
        found = true;
      }
      if (i < per) acc += h[i];
    }
  }
  __syncthreads();
  digit = sh.c->dig[0];
  rem = sh.c->dig[1];
}

// The k-th largest of n radix keys key_of(0..n) (1 <= k <= n), by a 3-pass
// LDS radix select over `hist` (kRadixBins words, 16-byte aligned).  Leaves the
// key in sh.c->pfx[0] and, in sh.c->krem[0], how many entries equal to it the k
// largest hold; resets sh.c->pos[0..1] for the caller.
template <int NT, class KeyOf>
__device__ __forceinline__ void cta_radix_select(KeyOf&& key_of, int n, int k, uint32_t* hist, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  uint32_t pf = 0u, krem = static_cast<uint32_t>(k);
#pragma unroll 1
  for (int pass = 0; pass < 3; ++pass) {
    const int shift = pass_shift(pass);
    const int bits = pass_bits(pass);
    #pragma unroll 1
    for (int i = tid; i < kRadixBins; i += kThreads) hist[i] = 0u;
    __syncthreads();
    PMQA_TR(sh, 21, n, pass);
    #pragma unroll 1
    for (int i0 = 0; i0 < n; i0 += 4 * kThreads) {
      // four keys a thread per round, their LDS reads in flight together (the
      // loop bound is uniform, so that the wave's ballots see every lane)
      uint32_t key[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kThreads + tid;
        key[u] = i < n ? key_of(i) : 0u;
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + u * kThreads + tid;
        const bool in = i < n && (pass == 0 || (key[u] >> (shift + bits)) == pf);
        const uint32_t bin = (key[u] >> shift) & ((1u << bits) - 1u);
        // lanes in the bin of the wave's first counted lane add once, together
        // (thousands of equal scores would otherwise serialise on one LDS word)
        const uint64_t act = __ballot(in);
        if (act) {
          const uint32_t lead = __builtin_amdgcn_readlane(bin, __ffsll(static_cast<long long>(act)) - 1);
          const uint64_t same = __ballot(in && bin == lead);
          if (in && bin == lead) {
            if (lanes_below(same) == 0) atomicAdd(&hist[lead], static_cast<uint32_t>(__popcll(same)));
          } else if (in) {
            atomicAdd(&hist[bin], 1u);
          }
        }
      }
    }
    __syncthreads();
    PMQA_TR(sh, 22, 0, pass);
    uint32_t d, rem;
    cta_find_digit(hist, 1 << bits, krem, sh, d, rem);
    PMQA_TR(sh, 23, 0, pass);
    pf = pass == 0 ? d : ((pf << bits) | d);
    krem = rem;
  }
  if (tid == 0) {
    sh.c->pfx[0] = pf;
    sh.c->krem[0] = krem;
    sh.c->pos[0] = 0;
    sh.c->pos[1] = 0;
  }
  __syncthreads();
}

// CTA-wide exclusive prefix sums of a and b over the threads in order (two
// barriers).
template <int NT>
__device__ __forceinline__ void cta_exclusive_scan2(uint32_t& a, uint32_t& b, const Sh<NT>& sh) {
  const int lane = lane_id();
  const int w = wave_id();
  const uint32_t ia = __ockl_wfscan_add_u32(a, true);  // inclusive within the wave
  const uint32_t ib = __ockl_wfscan_add_u32(b, true);
  __syncthreads();
  if (lane == 63) {
    sh.c->wtot[w] = ia;
    sh.c->wcnt[0][w][0] = static_cast<int32_t>(ib);
  }
  __syncthreads();
  uint32_t ba = 0u, bb = 0u;
  for (int q = 0; q < w; ++q) {
    ba += sh.c->wtot[q];
    bb += static_cast<uint32_t>(sh.c->wcnt[0][q][0]);
  }
  a = ba + ia - a;
  b = bb + ib - b;
}

// The k-th largest (1 <= k <= n <= fin_cap) of the radix keys of the score
// bits in LDS (sh.fk[0 .. n)), by radix select over the bits where the keys
// differ: their common prefix (from the least and greatest key) is skipped,
// then 11-bit digits from the top of the rest, one histogram pass each (two
// for keys spread over at most 22 bits; none when all are equal).  Each pass
// reads the keys in runs of four per thread (one 16-byte LDS read), two runs
// at a time (the reads past n stay inside the final-select area and are not
// counted).
template <int NT>
__device__ __forceinline__ uint32_t lds_select(int n, int k, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  constexpr int kPer = 4;  // keys a thread takes per run: one 16-byte LDS read
  constexpr int kRun = kPer * kThreads;
  typedef uint32_t U32x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) U32x4 LdsU32x4;
  auto run = [&](int c, uint32_t (&x)[kPer]) {
    const U32x4 a = *(const LdsU32x4*)((LdsByte*)((char*)(sh.fk + c * kRun + kPer * tid)));
#pragma unroll
    for (int u = 0; u < kPer; ++u) x[u] = radix_key(__uint_as_float(a[u]));
  };
  uint32_t* hist = sh.fh;
  // the first pass's histogram cleared by the same barrier as the extremes
  for (int i = tid; i < kRadixBins / 4; i += kThreads) reinterpret_cast<uint4*>(hist)[i] = uint4{0u, 0u, 0u, 0u};
  uint32_t mn = 0xffffffffu, mx = 0u;
#pragma unroll 1
  for (int c = 0; c * kRun < n; ++c) {
    uint32_t x[kPer];
    run(c, x);
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const bool in = c * kRun + kPer * tid + u < n;
      mn = min(mn, in ? x[u] : 0xffffffffu);
      mx = max(mx, in ? x[u] : 0u);
    }
  }
  mn = __ockl_wfred_min_u32(mn);
  mx = __ockl_wfred_max_u32(mx);
  if (lane == 0) {
    sh.c->wmin[w] = mn;
    sh.c->wmax[w] = mx;
  }
  __syncthreads();
  mn = sh.c->wmin[0];
  mx = sh.c->wmax[0];
#pragma unroll
  for (int q = 1; q < kWaves; ++q) {
    mn = min(mn, sh.c->wmin[q]);
    mx = max(mx, sh.c->wmax[q]);
  }
  PMQA_TR(sh, 21, n, 0);
  int hi = mn == mx ? 0 : 32 - __clz(static_cast<int>(mn ^ mx));  // the low bits where keys differ
  uint32_t pf = hi == 32 ? 0u : mn >> hi;                          // the bits above them, shared
  uint32_t krem = static_cast<uint32_t>(k);
  uint32_t* sink = sh.c->sink + lane;
#pragma unroll 1
  while (hi > 0) {
    const int shift = hi > 11 ? hi - 11 : 0;
    const int bits = hi - shift;
    const uint32_t high = hi == 32 ? 0u : ~0u << hi;  // the bits decided so far, and their value
    const uint32_t want = hi == 32 ? 0u : pf << hi;
    const uint32_t low = (1u << bits) - 1u;
    // two runs at a time, their reads in flight together
#pragma unroll 1
    for (int c = 0; c * kRun < n; c += 2) {
      uint32_t x[2 * kPer];
      uint32_t(&x0)[kPer] = *reinterpret_cast<uint32_t(*)[kPer]>(x);
      uint32_t(&x1)[kPer] = *reinterpret_cast<uint32_t(*)[kPer]>(x + kPer);
      run(c, x0);
      run(c + 1, x1);
      // one LDS add per key, every lane: keys outside the pass (or past n) add
      // to the lane's own sink word, so that no lane masking separates the adds
      uint32_t* at[2 * kPer];
#pragma unroll
      for (int u = 0; u < 2 * kPer; ++u) {
        const int i = (c + u / kPer) * kRun + kPer * tid + u % kPer;
        const bool in = i < n && (x[u] & high) == want;
        at[u] = in ? hist + ((x[u] >> shift) & low) : sink;
      }
#pragma unroll
      for (int u = 0; u < 2 * kPer; ++u) atomicAdd(at[u], 1u);
    }
    __syncthreads();
    PMQA_TR(sh, 22, hi, 0);
    uint32_t d, rem;
    cta_find_digit(hist, kRadixBins, krem, sh, d, rem, shift > 0);
    PMQA_TR(sh, 23, 0, 0);
    pf = (pf << bits) | d;
    krem = rem;
    hi = shift;
  }
  return pf;
}

// ---------------------------------------------------------------- row finish

// A row's final select works on n (key index, score bits) pairs: pair_of(i)
// returns pair i (from LDS -- sh.fi, sh.fk -- or from where they lie).
// Loads pairs [0, n) -- the first n1 from `a`, the rest from `b` -- into LDS,
// the score bits passed through dec(bits); sixteen loads a thread in flight.
template <int NT, class Dec>
__device__ __forceinline__ void load_pairs(const int32_t* a, int n1, const int32_t* b, int n, Dec&& dec,
                                           const Sh<NT>& sh) {
  const int tid = threadIdx.x;
#pragma unroll 1
  for (int i0 = 0; i0 < n; i0 += 16 * kThreads) {
    int2 v[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * kThreads + tid;
      if (i < n) v[u] = ld_pair(i < n1 ? a + 2 * i : b + 2 * (i - n1));
    }
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int i = i0 + u * kThreads + tid;
      if (i < n) {
        ((LdsI32*)sh.fi)[i] = v[u].x;
        ((LdsU32*)sh.fk)[i] = dec(static_cast<uint32_t>(v[u].y));
      }
    }
  }
  __syncthreads();
}

// Where a final select's pairs lie: in LDS (sh.fi, sh.fk, already decoded),
// or in memory at g, their stored values encoded as candidates against th
// when dec is set.  One descriptor for every caller, so that the select's
// code exists once.
struct PairSrc {
  const int32_t* g;
  float th;
  int dec;
  int lds;
};

template <int NT>
__device__ __forceinline__ int2 pair_at(const PairSrc& ps, int i, const Sh<NT>& sh) {
  if (ps.lds) return make_int2(((const LdsI32*)sh.fi)[i], static_cast<int>(((const LdsU32*)sh.fk)[i]));
  int2 p = ld_pair(ps.g + 2 * i);
  if (ps.dec) p.y = __float_as_int(dec_cand(__int_as_float(p.y), ps.th));
  return p;
}

// The k-th largest key k* of n pairs (1 <= k <= n) by an LDS radix select,
// then each thread's pairs above k* and equal to it (i = tid, tid + kThreads,
// ...) counted and placed by one CTA-wide exclusive scan: og and oe are the
// thread's first ranks in each class, n_gt and n_eq the class sizes.  The
// caller then walks its pairs in the same order, handing out ranks og++ and
// oe++.
template <int NT>
__device__ __forceinline__ uint32_t kth_scan(const PairSrc& ps, int n, int k, const Sh<NT>& sh, uint32_t& og,
                                             uint32_t& oe, int& n_gt, int& n_eq) {
  auto key_of = [&](int i) { return radix_key(__int_as_float(pair_at<NT>(ps, i, sh).y)); };
  uint32_t kstar = 0u;
  // The class counts check the k-th key found: fewer than k keys above it and
  // at least k at or above it.  Should the prefix-skipping select ever miss
  // that, the three fixed passes select again over the same keys.
#pragma unroll 1
  for (int attempt = 0; attempt < 2; ++attempt) {
    if (ps.lds && attempt == 0) {
      kstar = lds_select<NT>(n, k, sh);
    } else {
      cta_radix_select(key_of, n, k, sh.fh, sh);
      kstar = sh.c->pfx[0];
    }
    uint32_t gt = 0u, eq = 0u;
#pragma unroll 1
    for (int i = threadIdx.x; i < n; i += kThreads) {
      const uint32_t key = key_of(i);
      gt += key > kstar ? 1u : 0u;
      eq += key == kstar ? 1u : 0u;
    }
    PMQA_TR(sh, 24, 0, 0);
    og = gt;
    oe = eq;
    cta_exclusive_scan2(og, oe, sh);
    if (threadIdx.x == kThreads - 1) {
      sh.c->pos[0] = static_cast<int>(og + gt);
      sh.c->pos[1] = static_cast<int>(oe + eq);
    }
    __syncthreads();
    n_gt = sh.c->pos[0];
    n_eq = sh.c->pos[1];
    if (!ps.lds || (n_gt < k && k <= n_gt + n_eq)) break;
    PMQA_TR(sh, 25, n_gt, 0);
  }
  return kstar;
}

// Top-k of a fitting row with a few candidates past k (1 <= nc - k <=
// kFewExtra, nc <= kFewPer * kThreads): every candidate but the nc - k
// smallest, by stored score and then slot.  The stored candidate values order
// as the scores do (the encoding maps (t, 2t] onto (0, t] and keeps the rest,
// with t > 0), so their radix keys are the order.  Thread t holds the keys of
// slots t + kThreads * u in registers; each round takes the CTA's least (key, slot)
// among those not yet left out (a wavefront minimum, then the four waves'
// through LDS; one barrier a round).  The kept indices are then written in
// slot order shifted past the left-out slots -- entries before the first
// left-out slot already hold their index (the main pass writes candidate
// j < top_k to entry j).
constexpr int kFewExtra = 8;  // at most the control words' left_out entries
constexpr int kFewPer = 16;

template <int NT>
__device__ __forceinline__ void few_extra_topk(const SelectArgs& s, int r, int k, int nc, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int w = wave_id();
  const int32_t* cand = s.candidates + (static_cast<int64_t>(r) * (s.top_k + s.capacity) + s.top_k) * 2;
  int32_t* out = s.topk_idx + static_cast<int64_t>(r) * s.top_k;
  const int d = nc - k;
  uint32_t key[kFewPer];
#pragma unroll
  for (int u = 0; u < kFewPer; ++u) {
    key[u] = 0xffffffffu;  // above every radix key (+inf's is 0xff800000)
    if (u * kThreads < nc) {
      const int i = u * kThreads + tid;
      const uint32_t v = *(const GlobalU32*)(cand + 2 * min(i, nc - 1) + 1);
      if (i < nc) key[u] = radix_key(__uint_as_float(v));
    }
  }
  uint32_t gone = 0u;  // this thread's left-out units
#pragma unroll 1
  for (int j = 0; j < d; ++j) {
    uint64_t m = ~0ull;
#pragma unroll
    for (int u = 0; u < kFewPer; ++u) {
      const uint64_t v = (static_cast<uint64_t>(key[u]) << 32) | static_cast<uint32_t>(u * kThreads + tid);
      if (!((gone >> u) & 1u)) m = min(m, v);
    }
    m = __ockl_wfred_min_u64(m);
    if (lane == 0) sh.c->wmin64[j & 1][w] = m;
    __syncthreads();
#pragma unroll
    for (int q = 0; q < kWaves; ++q) m = min(m, sh.c->wmin64[j & 1][q]);
    const uint32_t slot = static_cast<uint32_t>(m);
    if (tid == 0) sh.c->left_out[j] = slot;
    if (static_cast<int>(slot % kThreads) == tid) gone |= 1u << (slot / kThreads);
  }
  __syncthreads();
  uint32_t first = 0xffffffffu;
  for (int j = 0; j < d; ++j) first = min(first, sh.c->left_out[j]);
#pragma unroll
  for (int u = 0; u < kFewPer; ++u) {
    const uint32_t i = static_cast<uint32_t>(u * kThreads + tid);
    if (u * kThreads < nc && i < static_cast<uint32_t>(nc) && !((gone >> u) & 1u) &&
        (i > first || i >= static_cast<uint32_t>(s.top_k))) {
      uint32_t shift = 0u;
      for (int j = 0; j < d; ++j) shift += sh.c->left_out[j] < i ? 1u : 0u;
      out[i - shift] = *(const GlobalU32*)(cand + 2 * i);  // the slot's key index, read again
    }
  }
}

// Ranges and exact Top-k of a fitting row r (k = min(e_r, top_k)) with nc
// candidates, nt ties and threshold th: all candidates when there are at most
// k of them, completed with ties from the tie slots (cands_out: the candidates'
// indices are in topk_idx already, as the main pass writes candidate j < top_k
// to entry j), else the k largest candidates by decoded score.  Entries past k
// are -1.
template <int NT>
__device__ __forceinline__ void fit_row_outputs(const SelectArgs& s, int r, int k, int nc, int nt, float th,
                                                bool cands_out, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    s.ranges[r] = s.top_k - min(nt, s.top_k);
    s.ranges[s.rows + r] = s.top_k + min(nc, s.capacity);
  }
  if (s.topk_idx) {
    const int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + s.capacity) * 2;
    const int32_t* cand = slots + 2 * s.top_k;
    int32_t* out = s.topk_idx + static_cast<int64_t>(r) * s.top_k;
    for (int i = k + tid; i < s.top_k; i += kThreads) out[i] = -1;
    if (nc <= k) {
#pragma unroll 1
      for (int i = (cands_out ? nc : 0) + tid; i < k; i += kThreads)
        out[i] = i < nc ? cand[2 * i] : slots[2 * (s.top_k - 1 - (i - nc))];
    } else if (NT == 1 && cands_out && nc - k <= kFewExtra && nc <= kFewPer * kThreads) {
      // (next_n = 1 only: in the kernels for more rows the extra registers
      // cost the main loop more than this path saves)
      few_extra_topk<NT>(s, r, k, nc, sh);
    } else {
      // nc <= capacity (the row fits)
      const bool lds = nc <= sh.fin_cap;
      if (lds)
        load_pairs<NT>(cand, nc, cand, nc, [&](uint32_t b) { return __float_as_uint(dec_cand(__uint_as_float(b), th)); },
                       sh);
      const PairSrc ps{cand, th, 1, lds ? 1 : 0};
      auto pair_of = [&](int i) { return pair_at<NT>(ps, i, sh); };
      PMQA_TR(sh, 19, nc, 0);
      uint32_t og, oe;
      int n_gt, n_eq;
      const uint32_t kstar = kth_scan<NT>(ps, nc, k, sh, og, oe, n_gt, n_eq);
      PMQA_TR(sh, 20, 0, 0);
#pragma unroll 1
      for (int i = tid; i < nc; i += kThreads) {
        const int2 p = pair_of(i);
        const uint32_t key = radix_key(__int_as_float(p.y));
        if (key > kstar) out[og++] = p.x;
        else if (key == kstar && n_gt + static_cast<int>(oe) < k) out[n_gt + oe++] = p.x;
      }
    }
  }
  __syncthreads();
}

// Fit test of tile b (request length L) by the tile's last CTA, from the final
// counters (every CTA of the tile counted its keys before it arrived): fills
// sh.c->nc, nt, nn (near-band keys), thr and len, and the masks of the rows
// that do not fit -- stored_mask: rows whose k-th largest score is among pairs
// that are all kept (every candidate, in the slots and the overflow area; or,
// short of k candidates, every candidate, tie and near-band key) and that fit
// in LDS, re-selected from those pairs alone; repair_mask: the other rows,
// whose keys are swept again.
template <int NT>
__device__ __forceinline__ void tile_fit(const SelectArgs& s, int b, int L, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  if (tid == 0) {
    sh.c->repair_mask = 0u;
    sh.c->stored_mask = 0u;
    sh.c->len = L;
  }
  __syncthreads();
  if (tid < NT) {
    const int r = b * NT + tid;
    const int nc = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r));
    const int nt = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r + 1));
    const int nn = s.nearc ? static_cast<int>(ld_ag(s.nearc + static_cast<int64_t>(r) * kRowWords)) : 0;
    const float th = __uint_as_float(ld_ag(reinterpret_cast<const uint32_t*>(s.thresholds) + r));
    const int k = min(row_end<NT>(s, b, L, tid), s.top_k);
    const bool fit = nc <= s.capacity && nc + min(nt, s.top_k) >= k;
    const bool kept = nc <= s.capacity + kOverflowPairs;
    const bool stored =
        kept && (nc >= k ? nc <= sh.fin_cap
                         : (s.nearp && nt <= s.top_k && nn <= kNearPairs && nc + nt + nn >= k &&
                            nc + nt + nn <= sh.fin_cap));
    sh.c->nc[tid] = nc;
    sh.c->nt[tid] = nt;
    sh.c->nn[tid] = nn;
    sh.c->thr[tid] = th;
    if (!fit) atomicOr(stored ? &sh.c->stored_mask : &sh.c->repair_mask, 1u << tid);
  }
  __syncthreads();
}

// ---------------------------------------------------------------- finish

// The finish stage runs in the select launch itself.  Each CTA, once its keys
// are selected, arrives on its tile's arrival counter (an atomic add, after
// its slot stores and counter updates have completed: those are agent-scope
// write-through stores and atomics, so no dirty line of them stays in the
// storing XCD's L2).  The CTA that brings the count to the tile's number of
// CTAs is the tile's last: it re-zeroes the counter, takes an agent-scope
// acquire and runs the fit test on the final counters (page
// "flashinfer.sdsa.indexer_threshold_select", description paragraph 3 and
// parameter arrivals).  A tile whose rows all fit is finished at once (one
// row: by the last CTA itself; more rows: one row item each, the last CTA
// taking the first).  Rows that do not fit are repaired:
//   * a row whose candidates all sit in its slots and the workspace's overflow
//     area is selected again from those candidates alone (its k-th largest
//     candidate becomes its threshold; every key at or above it is one of
//     them), in its row item;
//   * the other rows' keys are swept again by a repair job, in stages split
//     into items of a few thousand keys that every CTA of the launch may run:
//       stages 1-3  radix histogram pass 0/1/2 (10/11/11 bits) of the repaired
//                   rows' keys, into per-row global histograms (the fused
//                   select computes the scores again in stage 1 and keeps the
//                   repaired rows' scores in the workspace's score rows for
//                   the later stages; the select over a logits matrix reads
//                   the matrix);
//       stage 4     collect: keys above the selected bucket become candidates
//                   (stored raw), keys inside it go to the row's bucket;
//       stage 5     select again at the now exact k-th largest score;
//       stage 6     one item per row: a collected row's exact k-th largest key
//                   from its bucket, then every row's ranges and Top-k.
// After a histogram pass the digit holding each row's k-th largest key is
// found; if every row's bucket fits the bucket area the job moves to stage 4,
// if every key bit is known to stage 5, else to the next pass.  An item is
// claimed by a 64-bit fetch-and-add on one of the job's kClaimWords (stage,
// next) words, word q handing out items q, q + kClaimWords, ...: an item below
// the stage's item count is the caller's, a larger one claims nothing.
// Whoever completes a stage's last item runs the stage change.  After its own
// keys (and its tile's finish, if last) a CTA claims items, scanning every
// tile's claim words; with none open it waits -- for a bounded time while a
// job is before its last stage (its next stage opens more items), briefly
// otherwise (tiles still finishing their keys may publish some) -- and only
// when every CTA of the launch is resident (otherwise waiting CTAs could keep
// others from starting); then it leaves.  Each job is carried to its end by
// the CTAs that complete its stages, so nothing depends on the waiting, and
// no word outside the jobs is shared, so nothing needs clearing between calls:
// a finished job's claim words hand out no item.
constexpr int kClaimWords = 4;  // claim words per repair job
constexpr int kStageHist0 = 1;
constexpr int kStageCollect = 4;
constexpr int kStageSelect = 5;
constexpr int kStageRows = 6;
constexpr uint64_t kIdleTicks = 20000;  // s_memrealtime ticks (100 MHz) a CTA waits for a pending job: 200 us
constexpr uint64_t kLingerTicks = 400;  // and without one: 4 us
// after an item, without a job pending: 1 us (the launch ends that much after
// its last item; measured 2-3 us faster per call than kLingerTicks there)
constexpr uint64_t kAfterItemTicks = 100;
static_assert(2 * kClaimWords + 1 + 6 < kJobWords, "a job's claim words, mask and per-stage counts");

struct Ws {
  uint32_t* base;
  int batch, rows;
  __device__ WsLayout lay() const { return workspace_layout(batch, rows, 0, false); }
  // [2q, 2q + 1] claim word q < kClaimWords, [2 kClaimWords] row masks (the
  // swept rows, and in bits 8.. the rows re-selected from their candidates),
  // [2 kClaimWords + 1 + stage] items done in the stage
  __device__ uint32_t* job(int b) const { return base + lay().jobs + kJobWords * b; }
  __device__ uint64_t* claim(int b, int q) const { return reinterpret_cast<uint64_t*>(job(b) + 2 * q); }
  __device__ uint32_t* mask_word(int b) const { return job(b) + 2 * kClaimWords; }
  __device__ uint32_t* done_word(int b, int stage) const { return job(b) + 2 * kClaimWords + 1 + stage; }
  // per row: [0] digit prefix [1] rank left [2] bits known [3] bucket count [4] near-band
  // keys (counted by the main pass, cleared when the row is finished)
  __device__ uint32_t* row(int r) const { return base + lay().row_state + kRowWords * r; }
  // copy c of row r's radix histogram (items add into copy idx % kHistCopies,
  // which spreads the atomics of a pass over kHistCopies times more lines)
  __device__ uint32_t* hist(int r, int c) const {
    return base + lay().hist + static_cast<int64_t>(kRadixBins) * (kHistCopies * r + c);
  }
  __device__ int32_t* bucket(int r) const {
    return reinterpret_cast<int32_t*>(base + lay().bucket) + 2 * static_cast<int64_t>(kBucketPairs) * r;
  }
  __device__ int32_t* overflow(int r) const {
    return reinterpret_cast<int32_t*>(base + lay().overflow) + 2 * static_cast<int64_t>(kOverflowPairs) * r;
  }
};

// Items of a stage of a request of L keys: rescore_item_keys(L) keys when the
// scores are computed from the KV pages (stage 1 of the fused repair), else
// kSelectItemKeys keys read back from a score row; one per row in stage 6.
// Keys of a repair item over stored scores (fewer for next_n >= 3, whose
// items hold every repaired row's scores in registers at once).
template <int NT>
constexpr int kItemKeys = NT >= 3 ? kSelectItemKeys / 2 : kSelectItemKeys;

// Keys of a stage-1 item of a request of L keys: the request in about
// kRescoreItems items of a multiple of kRescoreItemKeys keys, at most 32768
// (the items' packed 16-bit histogram counts).  Every item has fixed costs --
// its claim and completion round trips and its histogram's flush into the
// row's -- so long requests take long items; short ones still spread over
// several CTAs.
__device__ __forceinline__ int rescore_item_keys(int L) {
  const int per = static_cast<int>(ceil_div(ceil_div(L, kRescoreItems), kRescoreItemKeys)) * kRescoreItemKeys;
  return min(max(per, kRescoreItemKeys), 32768);
}

template <int NT, bool kFused>
__device__ __forceinline__ int stage_items(int stage, int L) {
  if (stage == kStageRows) return NT;
  const int keys = (kFused && stage == kStageHist0) ? rescore_item_keys(L) : kItemKeys<NT>;
  return max(1, static_cast<int>(ceil_div(L, keys)));
}

// The tile's last CTA publishes tile b's job: the swept rows' state words and
// histograms set up, the row masks and the per-stage counts cleared, and --
// once all of that is complete -- the claim words opened at `stage` (with item
// 0 kept back for the caller when self0).  Claimers find the job by its claim
// words, so no other word changes hands.
template <int NT>
__device__ __forceinline__ void publish_job(const SelectArgs& s, const Ws& ws, int b, const int (&end)[NT],
                                            uint32_t sweep, uint32_t stored, int stage, bool self0) {
  const int tid = threadIdx.x;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!(sweep & (1u << t))) continue;
    uint32_t* h = ws.hist(b * NT + t, 0);
    for (int i = tid; i < kHistCopies * kRadixBins; i += kThreads) st_wt(h + i, 0u);
  }
  if (tid < NT && (sweep & (1u << tid))) {
    uint32_t* row = ws.row(b * NT + tid);
    st_wt(row + 0, 0u);
    st_wt(row + 1, static_cast<uint32_t>(min(end[tid], s.top_k)));
    st_wt(row + 2, 0u);
    st_wt(row + 3, 0u);
  }
  if (tid == 64) st_wt(ws.mask_word(b), sweep | (stored << 8));
  if (tid >= 128 && tid < 128 + kStageRows) st_wt(ws.done_word(b, tid - 127), 0u);
  wait_vm_done();
  __syncthreads();
  if (tid < kClaimWords)
    st_wt64(ws.claim(b, tid), (static_cast<uint64_t>(stage) << 32) | ((self0 && tid == 0) ? 1u : 0u));
}

// Stages 4 and 5 on one row of one item, its scores in registers (v[u] is the
// score of key c0 + 64*(w + 4u) + lane): every key below lim is classified by
// cls(score) -> 0 (none), 1 or 2; each wave counts its keys of both classes
// with ballots, thread 0 reserves the CTA's positions with one atomic per
// class (add1(n), add2(n) return the first), and the keys go to put(class,
// position, key, score).
template <int NT, int kU, class Cls, class Add1, class Add2, class Put>
__device__ __forceinline__ void append_row(int c0, int lim, const float (&v)[kU], const Sh<NT>& sh, Cls&& cls,
                                           Add1&& add1, Add2&& add2, Put&& put) {
  const int w = wave_id();
  const int lane = lane_id();
  int n1 = 0, n2 = 0;
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int p = c0 + kGroupKeys * (w + kWaves * u) + lane;
    const int c = p < lim ? cls(v[u]) : 0;
    n1 += __popcll(__ballot(c == 1));
    n2 += __popcll(__ballot(c == 2));
  }
  if (lane == 0) {
    sh.c->wcnt[0][w][0] = n1;
    sh.c->wcnt[0][w][1] = n2;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot[2] = {0, 0};
    for (int q = 0; q < kWaves; ++q) {
      tot[0] += sh.c->wcnt[0][q][0];
      tot[1] += sh.c->wcnt[0][q][1];
    }
    int base[2];
    base[0] = tot[0] ? add1(tot[0]) : 0;
    base[1] = tot[1] ? add2(tot[1]) : 0;
    for (int q = 0; q < kWaves; ++q) {
      sh.c->wbase[0][q][0] = base[0];
      sh.c->wbase[0][q][1] = base[1];
      base[0] += sh.c->wcnt[0][q][0];
      base[1] += sh.c->wcnt[0][q][1];
    }
  }
  __syncthreads();
  int r1 = sh.c->wbase[0][w][0], r2 = sh.c->wbase[0][w][1];
#pragma unroll
  for (int u = 0; u < kU; ++u) {
    const int p = c0 + kGroupKeys * (w + kWaves * u) + lane;
    const int c = p < lim ? cls(v[u]) : 0;
    const uint64_t m1 = __ballot(c == 1);
    const uint64_t m2 = __ballot(c == 2);
    if (c == 1) put(1, r1 + lanes_below(m1), p, v[u]);
    if (c == 2) put(2, r2 + lanes_below(m2), p, v[u]);
    r1 += __popcll(m1);
    r2 += __popcll(m2);
  }
  __syncthreads();
}

// Stage change after histogram pass `pass` of tile b's job (run by the CTA that
// completed the pass's last item).
template <int NT>
__device__ __forceinline__ void job_next_stage(const SelectArgs& s, const Ws& ws, int b, int pass, uint32_t mask, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  const int wave = wave_id();
  const int lane = lane_id();
  const int shift = pass_shift(pass);
  const int bits = pass_bits(pass);
  const int nb = 1 << bits;
  // each row's histogram: the sum of its copies, which are cleared for the next
  // pass.  A row's copies are loaded together (kHistCopies * nb / kThreads
  // words a thread), so the sum costs one round trip per row.
  constexpr int kJ = kRadixBins / kThreads;  // bins of a thread
#pragma unroll 1
  for (int t = 0; t < NT; ++t) {
    if (!(mask & (1u << t))) continue;
    uint32_t* gh = ws.hist(b * NT + t, 0);
    uint32_t v[kJ][kHistCopies];
#pragma unroll
    for (int j = 0; j < kJ; ++j)
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c)
        v[j][c] = j * kThreads < nb ? ld_ag(gh + c * kRadixBins + j * kThreads + tid) : 0u;
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      if (j * kThreads >= nb) continue;
      uint32_t sum = 0u;
#pragma unroll
      for (int c = 0; c < kHistCopies; ++c) {
        sum += v[j][c];
        if (v[j][c]) st_wt(gh + c * kRadixBins + j * kThreads + tid, 0u);
      }
      sh.rh[t][j * kThreads + tid] = sum;
    }
  }
  __syncthreads();
  if (wave < NT && (mask & (1u << wave))) {
    uint32_t* row = ws.row(b * NT + wave);
    const uint32_t pfx = ld_ag(row + 0);
    uint32_t d = 0, rem = 0;
    find_digit(sh.rh[wave], nb, ld_ag(row + 1), &d, &rem);
    if (lane == 0) {
      sh.c->pfx[wave] = pass == 0 ? d : ((pfx << bits) | d);
      sh.c->krem[wave] = rem;
      sh.c->cnt[wave][0] = static_cast<int32_t>(sh.rh[wave][d]);
    }
  }
  __syncthreads();
  const int known = 32 - shift;
  if (tid == 0) {
    bool small = true;
    for (int t = 0; t < NT; ++t)
      if ((mask & (1u << t)) && sh.c->cnt[t][0] > kBucketPairs) small = false;
    sh.c->next_stage = known == 32 ? kStageSelect : (small ? kStageCollect : kStageHist0 + pass + 1);
  }
  __syncthreads();
  const int next = sh.c->next_stage;
  if (tid < NT && (mask & (1u << tid))) {
    const int r = b * NT + tid;
    uint32_t* row = ws.row(r);
    st_wt(row + 0, sh.c->pfx[tid]);
    st_wt(row + 1, sh.c->krem[tid]);
    st_wt(row + 2, static_cast<uint32_t>(known));
    if (next >= kStageCollect) {
      st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r, 0u);
      st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r + 1, 0u);
      st_wt(row + 3, 0u);
    }
    if (next == kStageSelect) st_wt(reinterpret_cast<uint32_t*>(s.thresholds) + r, __float_as_uint(key_to_float(sh.c->pfx[tid])));
  }
  wait_vm_done();
  __syncthreads();
  if (tid < kClaimWords) st_wt64(ws.claim(b, tid), static_cast<uint64_t>(next) << 32);
}

// Row r after the collect stage: its exact k-th largest key among its bucket
// (in LDS when it fits, else read from L2 by every pass) becomes its
// threshold; the bucket's keys above it and equal to it are appended as
// candidates (after the nabove collected above the bucket) and ties, the
// collected candidates (stored raw) re-encoded against it.  Writes the row's
// counters and threshold and returns them in sh.c->nc[0], nt[0], thr[0].
template <int NT>
__device__ __forceinline__ void resolve_row(const SelectArgs& s, const Ws& ws, int r, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  uint32_t* row = ws.row(r);
  const int nin = min(static_cast<int>(ld_ag(row + 3)), kBucketPairs);
  const int krem = static_cast<int>(ld_ag(row + 1));
  const int nabove = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r));
  const int32_t* bucket = ws.bucket(r);
  const bool lds = nin <= sh.fin_cap;
  if (lds) load_pairs<NT>(bucket, nin, bucket, nin, [](uint32_t b) { return b; }, sh);
  const PairSrc ps{bucket, 0.f, 0, lds ? 1 : 0};
  auto pair_of = [&](int i) { return pair_at<NT>(ps, i, sh); };
  uint32_t og, oe;
  int n_gt, n_eq;
  const uint32_t kstar = kth_scan<NT>(ps, nin, krem, sh, og, oe, n_gt, n_eq);
  const float t2 = key_to_float(kstar);
  int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + s.capacity) * 2;
#pragma unroll 1
  for (int i = tid; i < nin; i += kThreads) {
    const int2 p = pair_of(i);
    const float e = __int_as_float(p.y);
    const uint32_t key = radix_key(e);
    if (key > kstar) {
      const int c = nabove + static_cast<int>(og++);
      if (c < s.capacity) store_pair(slots + 2 * (s.top_k + c), p.x, enc_cand(e, t2));
    } else if (key == kstar) {
      const int c = static_cast<int>(oe++);
      if (c < s.top_k) store_pair(slots + 2 * (s.top_k - 1 - c), p.x, e - t2);
    }
  }
  // the candidates collected above the bucket (raw scores) re-encoded
#pragma unroll 1
  for (int i = tid; i < min(nabove, s.capacity); i += kThreads) {
    const int2 p = *reinterpret_cast<const int2*>(slots + 2 * (s.top_k + i));
    store_pair(slots + 2 * (s.top_k + i), p.x, enc_cand(__int_as_float(p.y), t2));
  }
  if (tid == 0) {
    const int nc = nabove + n_gt;
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r, static_cast<uint32_t>(nc));
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r + 1, static_cast<uint32_t>(n_eq));
    st_wt(reinterpret_cast<uint32_t*>(s.thresholds) + r, __float_as_uint(t2));
    sh.c->nc[0] = nc;
    sh.c->nt[0] = n_eq;
    sh.c->thr[0] = t2;
  }
  // this CTA's slot stores complete before the Top-k reads the slots back
  wait_vm_done();
  __syncthreads();
}

// Row r (k = min(e_r, top_k) >= 1) selected again from its kept pairs alone.
// With at least k candidates, all nc of them are kept -- the first `capacity`
// in its slots (encoded against the old threshold), the rest in the overflow
// area -- and every key at or above the k-th largest candidate is one of them
// (it scores above the old threshold).  With fewer, the kept pairs are every
// candidate, every tie (in the tie slots) and every key of the near band just
// below the threshold (raw, in the near area), which holds the k-th largest:
// every key at or above it is one of them.  The k-th largest kept score,
// radix-selected in LDS, becomes the row's threshold; the kept pairs above it
// and equal to it are stored again as the row's candidates and ties, and its
// counters, threshold, ranges and Top-k written.  (Scores are NaN-free by
// precondition, so no key outside them is a tie at the new threshold.)
template <int NT>
__device__ __forceinline__ void stored_resolve(const SelectArgs& s, int r, int k, int nc, int nt, int nn, float th,
                                               const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  const int cap = s.capacity;
  int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + cap) * 2;
  const int32_t* cand = slots + 2 * s.top_k;
  const int32_t* ovf = s.ovf + 2 * static_cast<int64_t>(kOverflowPairs) * r;
  const int32_t* nearp = s.nearp + 2 * static_cast<int64_t>(kNearPairs) * r;
  const int n = nc >= k ? nc : nc + nt + nn;  // <= fin_cap
  // every kept pair into LDS with its score, eight loads a thread in flight
#pragma unroll 1
  for (int i0 = 0; i0 < n; i0 += 8 * kThreads) {
    int2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kThreads + tid;
      if (i < n) {
        const int32_t* src = i < nc ? (i < cap ? cand + 2 * i : ovf + 2 * (i - cap))
                                    : (i < nc + nt ? slots + 2 * (s.top_k - 1 - (i - nc)) : nearp + 2 * (i - nc - nt));
        v[u] = *reinterpret_cast<const int2*>(src);
      }
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int i = i0 + u * kThreads + tid;
      if (i < n) {
        const float x = __int_as_float(v[u].y);
        const float e = i < nc ? dec_cand(x, th) : (i < nc + nt ? x + th : x);
        sh.fi[i] = v[u].x;
        sh.fk[i] = __float_as_uint(e);
      }
    }
  }
  __syncthreads();
  const PairSrc ps{nullptr, 0.f, 0, 1};
  auto pair_of = [&](int i) { return pair_at<NT>(ps, i, sh); };
  uint32_t og, oe;
  int n_gt, n_eq;
  const uint32_t kstar = kth_scan<NT>(ps, n, k, sh, og, oe, n_gt, n_eq);
  const float t2 = key_to_float(kstar);
  int32_t* out = s.topk_idx ? s.topk_idx + static_cast<int64_t>(r) * s.top_k : nullptr;
#pragma unroll 1
  for (int i = tid; i < n; i += kThreads) {
    const int2 p = pair_of(i);
    const float e = __int_as_float(p.y);
    const uint32_t key = radix_key(e);
    if (key > kstar) {
      if (static_cast<int>(og) < cap) store_final(slots + 2 * (s.top_k + og), p.x, enc_cand(e, t2));
      if (out) out[og] = p.x;
      ++og;
    } else if (key == kstar) {
      if (static_cast<int>(oe) < s.top_k) store_final(slots + 2 * (s.top_k - 1 - oe), p.x, e - t2);
      if (out && n_gt + static_cast<int>(oe) < k) out[n_gt + oe] = p.x;
      ++oe;
    }
  }
  if (out)
    for (int i = k + tid; i < s.top_k; i += kThreads) out[i] = -1;
  if (tid == 0) {
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r, static_cast<uint32_t>(n_gt));
    st_wt(reinterpret_cast<uint32_t*>(s.counters) + 2 * r + 1, static_cast<uint32_t>(n_eq));
    st_wt(reinterpret_cast<uint32_t*>(s.thresholds) + r, __float_as_uint(t2));
    s.ranges[r] = s.top_k - min(n_eq, s.top_k);
    s.ranges[s.rows + r] = s.top_k + min(n_gt, cap);
  }
  __syncthreads();
}

// Row r of a tile with final counters (nc, nt), nn near-band keys and
// threshold th: its ranges and Top-k when it fits, its re-selection from its
// kept pairs when it is a stored row; its near-band count is left zeroed.
template <int NT>
__device__ __forceinline__ void unswept_row(const SelectArgs& s, int r, int k, int nc, int nt, int nn, float th,
                                            bool stored, const Sh<NT>& sh) {
  if (stored && nc < k && nc + nt + nn < k) {
    // A stored row's fit test counted at least k kept pairs, so counts short of
    // k were not the final ones: they are read again as the words' current
    // values (the near-band count is cleared only after the select, whose last
    // barrier every wave passes after these reads).
    nc = static_cast<int>(rd_cur_wave(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r));
    nt = static_cast<int>(rd_cur_wave(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r + 1));
    nn = s.nearc ? static_cast<int>(rd_cur_wave(s.nearc + static_cast<int64_t>(r) * kRowWords)) : 0;
  }
  if (stored) stored_resolve<NT>(s, r, k, nc, nt, nn, th, sh);
  else fit_row_outputs<NT>(s, r, k, nc, nt, th, true, sh);
  if (threadIdx.x == 0 && s.nearc) st_wt(s.nearc + static_cast<int64_t>(r) * kRowWords, 0u);
}

// Stage-6 item t of tile b's job: row t given its ranges and Top-k -- a swept
// row after its bucket is resolved (or after stage 5 selected it again), a
// stored row after its re-selection from its candidates, a fitting row from
// its slots.  A swept row's state words are cleared for the next call.
template <int NT>
__device__ __forceinline__ void row_item(const SelectArgs& s, const Ws& ws, int b, int L, int t, uint32_t masks,
                                         int nc, int nt, int nn, float th, const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  const int r = b * NT + t;
  const int k = min(row_end<NT>(s, b, L, t), s.top_k);
  if (masks & (1u << t)) {
    if (ld_ag(ws.row(r) + 2) < 32u) {
      resolve_row<NT>(s, ws, r, sh);
      nc = sh.c->nc[0];
      nt = sh.c->nt[0];
      th = sh.c->thr[0];
    }
    // (after a stage-5 select the slots were written by the items: visible
    // after the item's acquire; after a resolve this CTA wrote them)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    fit_row_outputs<NT>(s, r, k, nc, nt, th, false, sh);
    if (tid < 5) st_wt(ws.row(r) + tid, 0u);  // (word 4: the near-band count)
  } else {
    unswept_row<NT>(s, r, k, nc, nt, nn, th, ((masks >> 8) & (1u << t)) != 0, sh);
  }
}

// The bookkeeping after item idx of stage `stage` of tile b's job: the item is
// counted, and whoever completes the stage's last item runs the stage change
// (or, after the last stage, clears the job's words).
template <int NT, bool kFused>
__device__ __forceinline__ void item_done(const SelectArgs& s, const Ws& ws, int b, int L, int stage, uint32_t mask,
                                          const Sh<NT>& sh) {
  const int tid = threadIdx.x;
  wait_vm_done();
  __syncthreads();
  PMQA_TR(sh, 11, 0, stage);
  if (tid == 0)
    sh.c->is_last = add_ag(ws.done_word(b, stage), 1u) + 1 == static_cast<uint32_t>(stage_items<NT, kFused>(stage, L));
  __syncthreads();
  PMQA_TR(sh, 12, sh.c->is_last, stage);
  if (!sh.c->is_last) return;
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  if (stage < kStageCollect) {
    job_next_stage<NT>(s, ws, b, stage - kStageHist0, mask, sh);
  } else if (stage < kStageRows) {
    if (tid < kClaimWords) st_wt64(ws.claim(b, tid), static_cast<uint64_t>(kStageRows) << 32);
  } else {
    // the job is done: all of its words cleared for the next call (a late claim
    // attempt then adds to a word of stage 0, which hands out nothing)
    if (tid < kJobWords) st_wt(ws.job(b) + tid, 0u);
  }
}

// LDS areas a re-scoring item uses beside the finish view: the KV staging
// area, the q operands (next_n >= 3) and NT packed first-pass histograms
// (1024 bins as 512 words of two 16-bit counts: an item has at most 32768
// keys per row).
template <int NT>
struct RescoreLds {
  v4i* stage;
  QLds<NT>* ql;
  uint32_t* ph;
};

// Stage 1 of the fused repair, item idx: keys [c0, c1) of request b scored
// again from the KV pages (the select's loop and arithmetic, so the scores are
// the same bits), the repaired rows' scores written to the score rows for the
// later passes, and their first radix histogram pass.
template <int NT>
__device__ __forceinline__ void rescore_item(const PagedArgs& a, const SelectArgs& s, const Ws& ws, int b, int L, int idx,
                                             uint32_t mask, const int (&end)[NT], const RescoreLds<NT>& rl,
                                             const Sh<NT>& sh) {
  const int lane = lane_id();
  const int tid = threadIdx.x;
  const int shift = pass_shift(0);
  constexpr int kWords = (1 << 10) / 2;
  for (int i = tid; i < NT * kWords; i += kThreads) rl.ph[i] = 0u;
  __syncthreads();
  float* rows = s.scores + static_cast<int64_t>(b) * NT * s.score_ld;
  const int c0 = idx * rescore_item_keys(L);
  const int c1 = min(c0 + rescore_item_keys(L), L);
  auto add = [&](int t, int p, float e) {
    st_wt(reinterpret_cast<uint32_t*>(rows + t * s.score_ld + p), __float_as_uint(e));
    const uint32_t bin = radix_key(e) >> shift;
    atomicAdd(&rl.ph[t * kWords + (bin >> 1)], 1u << (16 * (bin & 1u)));
  };
  if (NT > 1 && __popc(mask) == 1) {
    // one row repaired: only its scores are computed (the same operations, so
    // the same bits, as the row's scores in the tile's scoring)
    const int t1 = __ffs(static_cast<int>(mask)) - 1;
    int e1 = 0;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (t == t1) e1 = end[t];
    KvSource<1> src;
    src.bind(rl.stage);
    src.init_row(a, b, static_cast<int64_t>(b) * NT + t1);
    stream_keys<1, false>(
        src, c0, c1, L,
        [&](int, int p0, const float(&E)[1]) {
          const int p = p0 + lane;
          if (p < e1) add(t1, p, E[0]);
        },
        [](int, int) {});
  } else {
    typename std::conditional<(NT >= 3), KvSourceQ<NT>, KvSource<NT>>::type src;
    src.bind(rl.stage);
    src.bind_q(rl.ql);
    src.init(a, b);
    stream_keys<NT, false>(
        src, c0, c1, L,
        [&](int, int p0, const float(&E)[NT]) {
          const int p = p0 + lane;
#pragma unroll
          for (int t = 0; t < NT; ++t)
            if ((mask & (1u << t)) && p < end[t]) add(t, p, E[t]);
        },
        [](int, int) {});
  }
  __syncthreads();
  PMQA_TR(sh, 18, 0, 0);
  const int copy = idx % kHistCopies;
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    if (!(mask & (1u << t))) continue;
    uint32_t* gh = ws.hist(b * NT + t, copy);
    for (int i = tid; i < kWords; i += kThreads) {
      const uint32_t h = rl.ph[t * kWords + i];
      if (h & 0xffffu) add_ag(gh + 2 * i, h & 0xffffu);
      if (h >> 16) add_ag(gh + 2 * i + 1, h >> 16);
    }
  }
}

// Repair item `idx` of stage `stage` of tile b's job: its keys' scores (read
// back from the logits matrix or the score rows, or for stage 1 of the fused
// repair computed again), then their histogram, collect or select pass; or a
// row item; then the stage bookkeeping.
template <int NT, bool kFused, class Args>
__device__ __forceinline__ void run_item(const Args& a, const SelectArgs& s, const Ws& ws, int b, int L, int stage, int idx,
                                         const Sh<NT>& sh, const RescoreLds<NT>& rl) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  // the stores of the CTAs that ran the tile's main pass and the job's earlier
  // stages (written through, before their counts) become visible
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
  // the job's masks and every row's state words, all loaded at once
  const uint32_t masks = ld_ag(ws.mask_word(b));
  int end[NT];
  uint32_t pfx[NT], kn[NT];
  float thr2[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) {
    end[t] = row_end<NT>(s, b, L, t);
    const int r = b * NT + t;
    pfx[t] = ld_ag(ws.row(r) + 0);
    kn[t] = ld_ag(ws.row(r) + 2);
    thr2[t] = __uint_as_float(ld_ag(reinterpret_cast<const uint32_t*>(s.thresholds) + r));
  }
  // a row item's counts, in the same round trip
  int nc = 0, nt = 0, nn = 0;
  if (stage == kStageRows) {
    const int r = b * NT + idx;
    nc = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r));
    nt = static_cast<int>(ld_ag(reinterpret_cast<const uint32_t*>(s.counters) + 2 * r + 1));
    nn = s.nearc ? static_cast<int>(ld_ag(s.nearc + static_cast<int64_t>(r) * kRowWords)) : 0;
  }
  const uint32_t mask = masks & 0xffu;  // the swept rows
  int known = 0;
#pragma unroll
  for (int t = 0; t < NT; ++t)
    if (mask & (1u << t)) known = static_cast<int>(kn[t]);
  bool done = false;
  if (stage == kStageRows) {
    float th = 0.f;
#pragma unroll
    for (int t = 0; t < NT; ++t)
      if (t == idx) th = thr2[t];
    row_item<NT>(s, ws, b, L, idx, masks, nc, nt, nn, th, sh);
    done = true;
  }
  if constexpr (kFused) {
    if (stage == kStageHist0) {
      rescore_item<NT>(a, s, ws, b, L, idx, mask, end, rl, sh);
      done = true;
    }
  }
  if (!done) {
    LogitsSource<NT, kFused> src;
    if constexpr (kFused)
      src.init_rows(s.scores + static_cast<int64_t>(b) * NT * s.score_ld, s.score_ld, mask);
    else
      src.init(a, b);
    const int c0 = idx * kItemKeys<NT>;
    const int cend = min(c0 + kItemKeys<NT>, L);
    // one repaired row at a time: its item scores all loaded at once (wave w's
    // group u holds keys c0 + 64*(w + 4u) .. +63), then its pass
    constexpr int kU = kItemKeys<NT> / (kGroupKeys * kWaves);
    const int w = wave_id();
#pragma unroll 1
    for (int t = 0; t < NT; ++t) {
      if (!(mask & (1u << t))) continue;
      const int r = b * NT + t;
      uint32_t pf = 0u;
      float th2 = 0.f;
      int lim = 0;
#pragma unroll
      for (int u = 0; u < NT; ++u)
        if (u == t) {
          pf = pfx[u];
          th2 = thr2[u];
          lim = min(cend, end[u]);
        }
      float v[kU];
#pragma unroll
      for (int u = 0; u < kU; ++u) v[u] = src.value(t, c0 + kGroupKeys * (w + kWaves * u) + lane, L);
      PMQA_TR(sh, 9, 0, stage);
      if (stage < kStageCollect) {
        // histogram straight from the scores in registers
        const int pass = stage - kStageHist0;
        const int shift = pass_shift(pass);
        const int bits = pass_bits(pass);
        const uint32_t low = (1u << bits) - 1u;
        uint32_t* h = sh.rh[0];
        for (int i = tid; i < (1 << bits); i += kThreads) h[i] = 0u;
        __syncthreads();
#pragma unroll
        for (int u = 0; u < kU; ++u) {
          const int p = c0 + kGroupKeys * (w + kWaves * u) + lane;
          const uint32_t key = radix_key(v[u]);
          const bool in = p < lim && (pass == 0 || (key >> (shift + bits)) == pf);
          if (in) atomicAdd(&h[(key >> shift) & low], 1u);
        }
        __syncthreads();
        PMQA_TR(sh, 10, 0, stage);
        uint32_t* gh = ws.hist(r, idx % kHistCopies);
        for (int i = tid; i < (1 << bits); i += kThreads) {
          const uint32_t x = h[i];
          if (x) add_ag(gh + i, x);
        }
        __syncthreads();
      } else if (stage == kStageCollect) {
        // keys above the bucket become candidates (raw scores; re-encoded once
        // the threshold is known), keys inside it go to the row's bucket
        int32_t* cslots = s.candidates + (static_cast<int64_t>(r) * (s.top_k + s.capacity) + s.top_k) * 2;
        int32_t* bucket = ws.bucket(r);
        append_row<NT, kU>(
            c0, lim, v, sh,
            [&](float e) {
              const uint32_t top = radix_key(e) >> (32 - known);
              return top > pf ? 1 : (top == pf ? 2 : 0);
            },
            [&](int n) { return add_ag(s.counters + 2 * r, n); },
            [&](int n) { return static_cast<int>(add_ag(ws.row(r) + 3, static_cast<uint32_t>(n))); },
            [&](int c, int k, int p, float e) {
              if (c == 1 && k < s.capacity) store_pair(cslots + 2 * k, p, e);
              if (c == 2 && k < kBucketPairs) store_pair(bucket + 2 * k, p, e);
            });
      } else {
        // select again at the now exact threshold
        int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + s.capacity) * 2;
        append_row<NT, kU>(
            c0, lim, v, sh, [&](float e) { return e > th2 ? 1 : (!(e < th2) ? 2 : 0); },
            [&](int n) { return add_ag(s.counters + 2 * r, n); },
            [&](int n) { return add_ag(s.counters + 2 * r + 1, n); },
            [&](int c, int k, int p, float e) {
              if (c == 1 && k < s.capacity) store_pair(slots + 2 * (s.top_k + k), p, enc_cand(e, th2));
              if (c == 2 && k < s.top_k) store_pair(slots + 2 * (s.top_k - 1 - k), p, e - th2);
            });
      }
    }
  }
  item_done<NT, kFused>(s, ws, b, L, stage, mask, sh);
}

// Wave 0 claims an item of a published job; the result goes to sh.c->job:
// (tile, stage, item), tile -1 when none is open but more may open, -2 when
// the CTA should leave.  `since` is when the CTA last had work (s_memrealtime).
template <int NT, bool kFused, class Args>
__device__ __forceinline__ void claim_item(const Args& a, const SelectArgs& s, const Ws& ws, uint64_t since,
                                           const Sh<NT>& sh) {
  if (wave_id() == 0) {
    const int lane = lane_id();
    bool pending = false;  // a job before its last stage
    int got = -1, stage = 0, idx = 0;
    const int q0 = static_cast<int>(blockIdx.x % kClaimWords);  // this CTA's first claim word
    const int rot = static_cast<int>((blockIdx.x / kClaimWords) & 63);  // spread CTAs over the open jobs
    // every claim word of every job, the CTA's own word first (any CTA can
    // take any item, so no item waits for a CTA that has left)
    for (int qi = 0; qi < kClaimWords && got < 0; ++qi) {
      const int q = (q0 + qi) % kClaimWords;
      for (int j0 = 0; j0 < ws.batch && got < 0; j0 += 64) {
        const int b = j0 + lane;
        int len = 0;
        uint64_t w = 0;
        if (b < ws.batch) {
          w = ld_ag64(ws.claim(b, q));
          len = tile_keys<NT>(a, b);
        }
        const uint32_t st = static_cast<uint32_t>(w >> 32);
        const bool open = st >= kStageHist0 && st <= kStageRows &&
                          q + kClaimWords * static_cast<uint64_t>(static_cast<uint32_t>(w)) <
                              static_cast<uint64_t>(stage_items<NT, kFused>(static_cast<int>(st), len));
        pending = pending || __ballot(st >= kStageHist0 && st < kStageRows) != 0;
        uint64_t m = __ballot(open);
        while (m) {
          const uint64_t hi = m & (~0ull << rot);
          const int l = __ffsll(static_cast<long long>(hi ? hi : m)) - 1;
          m &= ~(1ull << l);
          const int bl = j0 + l;
          const int ll = __shfl(len, l);
          unsigned long long old = 0;
          if (lane == 0) old = add_ag64(reinterpret_cast<uint64_t*>(ws.claim(bl, q)), 1ull);
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
    }
    if (got < 0) {
      const uint64_t idle = __builtin_amdgcn_s_memrealtime() - since;
      if (!s.resident || idle > (pending ? kIdleTicks : kLingerTicks)) got = -2;
    }
    if (lane == 0) {
      sh.c->job[0] = got;
      sh.c->job[1] = stage;
      sh.c->job[2] = idx;
    }
  }
  __syncthreads();
}

// After its own keys (and its tile's fit test, if it was the last): repair
// items until nothing is left, then the CTA leaves.
template <int NT, bool kFused, class Args>
__device__ __forceinline__ void work_loop(const Args& a, const SelectArgs& s, char* lds, bool linger) {
  using Lay = Layout<NT, kFused>;
  // (a CTA that has just finished its tile does not linger for items to come:
  // the CTAs still finishing their keys will)
  uint64_t since = __builtin_amdgcn_s_memrealtime() - (linger ? 0 : kLingerTicks);
  int polls = 0;
  while (true) {
    // the LDS views and the workspace rebuilt from opaque bases in every
    // round, so that no address derived from them is hoisted out of the loop
    // (the compiler would keep hundreds of them live across the items, and
    // spill them)
    uint32_t lo = static_cast<uint32_t>(reinterpret_cast<uintptr_t>((LdsByte*)lds));
    asm volatile("" : "+v"(lo));
    char* base = (char*)((LdsByte*)lo);
    const uint64_t wv = reinterpret_cast<uint64_t>(s.ws);
    uint32_t wlo = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(wv));
    uint32_t whi = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(wv >> 32));
    asm volatile("" : "+s"(wlo), "+s"(whi));
    uint32_t* wsb = in_global(reinterpret_cast<uint32_t*>((static_cast<uint64_t>(whi) << 32) | wlo));
    const Ws ws{wsb, a.batch, s.rows};
    const Sh<NT> sh = make_sh<NT>(base, Lay::kFinCap, Lay::kCtlOff);
    const RescoreLds<NT> rl{reinterpret_cast<v4i*>(base), reinterpret_cast<QLds<NT>*>(base + Lay::kStageBytes),
                            reinterpret_cast<uint32_t*>(base + Lay::kListOff)};
    claim_item<NT, kFused>(a, s, ws, since, sh);
    const int b = sh.c->job[0];
    const int stage = sh.c->job[1];
    const int idx = sh.c->job[2];
    __syncthreads();
    if (b == -2) {
      PMQA_TR(sh, 8, polls, 0);
      break;
    }
    if (b < 0) {
      // back off (up to about half a microsecond between polls), so that
      // waiting CTAs keep their loads off the job words the working ones update
      ++polls;
      for (int i = 0; i < min(polls, 4); ++i) __builtin_amdgcn_s_sleep(4);
      continue;
    }
    polls = 0;
    PMQA_TR(sh, 6, b, stage);
    const int L = tile_keys<NT>(a, b);
    run_item<NT, kFused>(a, s, ws, b, L, stage, idx, sh, rl);
    __syncthreads();
    PMQA_TR(sh, 7, idx, stage);
    since = __builtin_amdgcn_s_memrealtime() - (kLingerTicks - kAfterItemTicks);
  }
}

// The tile's last CTA: arrivals[b] back to zero, the fit test, and then the
// rows: finished here (one row, no sweep), or a job published (the first row
// item kept for this CTA when no sweep comes first).
template <int NT, bool kFused, class Args>
__device__ __forceinline__ void tile_finish(const Args& a, const SelectArgs& s, int b, int L, const Sh<NT>& sh,
                                            const RescoreLds<NT>& rl) {
  const Ws ws{s.ws, a.batch, s.rows};
  const int tid = threadIdx.x;
  if (tid == 0) st_wt(reinterpret_cast<uint32_t*>(s.arrivals) + b, 0u);
  tile_fit<NT>(s, b, L, sh);
  const uint32_t sweep = sh.c->repair_mask;
  const uint32_t stored = sh.c->stored_mask;
  PMQA_TR(sh, 4, sweep, stored);
  int end[NT];
#pragma unroll
  for (int t = 0; t < NT; ++t) end[t] = row_end<NT>(s, b, L, t);
  if (NT == 1 && sweep == 0u) {
    const int k = min(end[0], s.top_k);
    unswept_row<NT>(s, b, k, sh.c->nc[0], sh.c->nt[0], sh.c->nn[0], sh.c->thr[0], stored != 0u, sh);
    return;
  }
  const bool self0 = sweep == 0u;
  publish_job<NT>(s, ws, b, end, sweep, stored, self0 ? kStageRows : kStageHist0, self0);
  if (self0) {
    // the first row item, with the counts the fit test loaded
    unswept_row<NT>(s, b * NT, min(end[0], s.top_k), sh.c->nc[0], sh.c->nt[0], sh.c->nn[0], sh.c->thr[0],
                    (stored & 1u) != 0u, sh);
    item_done<NT, kFused>(s, ws, b, L, kStageRows, 0u, sh);
  }
}



// ---------------------------------------------------------------- work items

// Located launches run G >= 2 * batch CTAs, about as many as fit on the device
// at once.  Every request gets one CTA plus a share of the other G - batch in
// proportion to its 64-key groups (with `empty_group`, a request with seq_len 0
// counts as one group, so that its tile still finishes), the shares rounded
// cumulatively so that they add up; a request's groups are split evenly among
// its CTAs, which are consecutive positions of the grid's walk (GridWalk).  So
// every CTA works on one request only -- a CTA never pays a
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

// The request b this CTA works on, [k0, k1) the keys of b it handles and ctas
// the number of CTAs that handle b (the arrivals b's tile waits for); ok is
// false for a CTA without work.  Uniform across the CTA.
struct Segment {
  int b, L, k0, k1, ctas;
  bool ok;
};

// The order a located grid is walked in.  The first F CTAs (one per compute
// unit: dispatch fills every unit once before it doubles up) stream about an
// eighth faster than the G - F that share a unit with one of them (median
// main pass 58 against 66 us on the 32-request MTP batch, 24 against 28 us on
// the 8-request long batch).  Walked in block order, the requests at the
// front would get only first CTAs and those at the back only second ones, and
// the back requests' tiles would finish last, their finish work running on a
// grid that has mostly left.  Position u of the walk holds a first CTA when
// floor((u + 1) F / G) > floor(u F / G), so that every request's CTAs mix both
// kinds in proportion.  (Measured per fused call: 127 against 140 us on the
// MTP batch, 152 against 202 us on the long batch.  Splitting a request's keys
// 8 : 7 towards its first CTAs evens out the main pass, but the calls took 139
// and 167 us: the first CTAs that finish early take up the finish work.)
struct GridWalk {
  int64_t G, F;  // 1 <= F <= G
  __device__ __forceinline__ int64_t pos_of(int64_t i) const {
    return i < F ? ((i + 1) * G + F - 1) / F - 1 : (i - F) * G / (G - F);
  }
};

template <class LenF>
__device__ __forceinline__ Segment find_segment(LenF&& len_of, int batch, bool locate, int per_request,
                                                int keys_per_cta, bool empty_group, int fast_ctas) {
  Segment sg{0, 0, 0, 0, 0, false};
  if (!locate) {
    const int b = blockIdx.x / per_request;
    const int c = blockIdx.x % per_request;
    const int L = len_of(b);
    const int n = L > 0 ? static_cast<int>(ceil_div(L, keys_per_cta)) : (empty_group ? 1 : 0);
    if (c < n) sg = Segment{b, L, c * keys_per_cta, min((c + 1) * keys_per_cta, L), n, true};
    return sg;
  }
  const int lane = lane_id();
  const int64_t G = gridDim.x;
  const GridWalk walk{G, fast_ctas < 1 ? G : min(static_cast<int64_t>(fast_ctas), G)};
  // the CTA at position i of request b's positions [a0, a1): its even share
  // of the request's gg groups
  auto split = [&](int bb, int LL, int gg, int64_t a0, int64_t a1, int64_t i) {
    const int64_t n = a1 - a0, p = i - a0;
    const int k0 = static_cast<int>(p * gg / n) * kGroupKeys;
    const int k1 = min(static_cast<int>((p + 1) * gg / n) * kGroupKeys, LL);
    return Segment{bb, LL, k0, max(k0, k1), static_cast<int>(n), true};
  };
  if (batch <= 64) {
    // one load of the lengths, kept in registers for both scans
    const int L = lane < batch ? len_of(lane) : 0;
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
    const int64_t i = walk.pos_of(blockIdx.x);
    const int64_t a0 = first_cta(lane, incl - g), a1 = first_cta(lane + 1, incl);
    const uint64_t hit = __ballot(lane < batch && a0 <= i && i < a1);
    if (hit) {
      const int l = __ffsll(static_cast<long long>(hit)) - 1;
      const int bb = __builtin_amdgcn_readfirstlane(l);
      const int LL = __builtin_amdgcn_readfirstlane(__shfl(L, l));
      const int gg = __builtin_amdgcn_readfirstlane(__shfl(g, l));
      sg = split(bb, LL, gg, uniform64(__shfl(a0, l)), uniform64(__shfl(a1, l)), i);
    }
    return sg;
  }
  int64_t N = 0;  // groups in all
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    int64_t n = b < batch ? groups_of(len_of(b), empty_group) : 0;
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) n += __shfl_xor(n, off);
    N += uniform64(n);
  }
  const int64_t shared = static_cast<int64_t>(gridDim.x) - batch;
  // CTAs before a request with c groups before it: its index plus round(shared * c / N)
  auto first_cta = [&](int64_t b, int64_t c) { return b + (N > 0 ? (2 * shared * c + N) / (2 * N) : 0); };
  const int64_t i = walk.pos_of(blockIdx.x);
  int64_t before = 0;  // groups of the requests before this block of 64
  for (int b0 = 0; b0 < batch; b0 += 64) {
    const int b = b0 + lane;
    const int L = b < batch ? len_of(b) : 0;
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
      return split(bb, LL, gg, uniform64(__shfl(a0, l)), uniform64(__shfl(a1, l)), i);
    }
    before += uniform64(__shfl(incl, 63));
  }
  return sg;
}

// Calls seg(b, L, k0, k1, ctas) for this CTA's segment, if it has one (one
// call site, so the body is inlined once).
template <class LenF, class F>
__device__ __forceinline__ void for_each_segment(LenF&& len_of, int batch, bool locate, int per_request,
                                                 int keys_per_cta, bool empty_group, int fast_ctas, F&& seg) {
  const Segment sg = find_segment(len_of, batch, locate, per_request, keys_per_cta, empty_group, fast_ctas);
  if (sg.ok) seg(sg.b, sg.L, sg.k0, sg.k1, sg.ctas);
}

// ---------------------------------------------------------------- kernels

// Waves per SIMD each variant is built for (VGPR budget 512 / waves): two for
// every next_n.  The finish stage's code shares the kernel's register budget;
// built for three waves (168 VGPRs) the next_n = 1 variant spilled inside its
// streaming loop and wrote 34 MB of spill lines per call on the 64-request
// decode batch (9.5 MB at two waves, and 0.8 us faster per call).
template <int NT>
constexpr int kFusedWaves = 2;


// Stored logits element: float32, float16 or bfloat16 (rounded to nearest even).
constexpr int kOutF32 = 0;
constexpr int kOutF16 = 1;
constexpr int kOutBf16 = 2;

// Logits of a request's rows, stored as out_type elements.
template <int NT, class Src, class Q>
__device__ __forceinline__ void logits_body(const PagedArgs& a, void* out, int64_t ld, int out_type, v4i* stage,
                                            Q* ql) {
  Src src;
  src.bind(stage);
  src.bind_q(ql);
  const int lane = lane_id();
  for_each_segment([&](int b) { return tile_keys<NT>(a, b); }, a.batch, a.locate, a.per_request, kLogitsKeysPerCta, false, a.fast_ctas,
                   [&](int b, int L, int k0, int k1, int) {
    src.init(a, b);
    const int64_t off = static_cast<int64_t>(b) * NT * ld;
    float* row0 = in_global(static_cast<float*>(out)) + off;
    _Float16* row0h = in_global(static_cast<_Float16*>(out)) + off;
    __bf16* row0b = in_global(static_cast<__bf16*>(out)) + off;
    stream_keys<NT, false>(
        src, k0, k1, L,
        [&](int, int p0, const float(&E)[NT]) {
          if (out_type == kOutF16) {
#pragma unroll
            for (int t = 0; t < NT; ++t) row0h[t * ld + p0 + lane] = static_cast<_Float16>(E[t]);
          } else if (out_type == kOutBf16) {
#pragma unroll
            for (int t = 0; t < NT; ++t) row0b[t * ld + p0 + lane] = static_cast<__bf16>(E[t]);
          } else {
#pragma unroll
            for (int t = 0; t < NT; ++t) row0[t * ld + p0 + lane] = E[t];
          }
        },
        [](int, int) {});
  });
}

template <int NT, int kEpi>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFusedWaves<NT>, 8)))
logits_kernel(PagedArgs a, void* out, int64_t ld, int out_type) {
  __shared__ v4i stage[kWaves * kStageInt4];
  global_view(a);
  if constexpr (NT >= 3) {
    __shared__ QLds<NT> ql;
    logits_body<NT, KvSourceQ<NT, kEpi>>(a, out, ld, out_type, stage, &ql);
  } else {
    logits_body<NT, KvSource<NT, kEpi>>(a, out, ld, out_type, stage, static_cast<QLds<NT>*>(nullptr));
  }
}

// MXFP4 logits: no LDS (the keys go straight from their loads into the MFMA).
template <int NT, int kEpi>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 8)))
fp4_logits_kernel(PagedArgs a, void* out, int64_t ld, int out_type) {
  global_view(a);
  logits_body<NT, KvSourceFp4<NT, kEpi>>(a, out, ld, out_type, nullptr, static_cast<void*>(nullptr));
}

// A wave's n candidate pairs of row r into slots top_k + base + i, those past
// the capacity into the workspace's overflow area (while it has room; without
// a workspace they are dropped), all with agent-scope write-through stores
// (the tile's last CTA, on any XCD, reads them).  With a Top-k output,
// candidate j < top_k also writes its key index to topk_idx[r][j]: a row that
// ends with exactly k candidates then already holds its Top-k in slot order;
// every other row's finish rewrites entries 0 .. top_k - 1.
__device__ __forceinline__ void store_cands(const SelectArgs& s, int r, int base, const int2* list, int n) {
  int32_t* slots = s.candidates + (static_cast<int64_t>(r) * (s.top_k + s.capacity) + s.top_k) * 2;
  int32_t* ovf = s.ovf ? s.ovf + 2 * static_cast<int64_t>(kOverflowPairs) * r : nullptr;
  int32_t* out = s.topk_idx ? s.topk_idx + static_cast<int64_t>(r) * s.top_k : nullptr;
  for (int i = lane_id(); i < n; i += 64) {
    const int j = base + i;
    const int2 e = list[i];
    if (j < s.capacity) store_pair(slots + 2 * j, e.x, __int_as_float(e.y));
    else if (ovf && j - s.capacity < kOverflowPairs) store_pair(ovf + 2 * (j - s.capacity), e.x, __int_as_float(e.y));
    if (out && j < s.top_k) st_wt(reinterpret_cast<uint32_t*>(out + j), static_cast<uint32_t>(e.x));
  }
}

// A wave's n pairs of row r from its tie list -- ties (stored value 0 or NaN)
// into slots top_k - 1 - bt - i (those past top_k dropped), near-band keys
// (below the threshold th; stored value e - th < 0, exact) with their raw
// scores into the workspace's near area at bn + i (those past it dropped) --
// written through.
__device__ __forceinline__ void store_ties(const SelectArgs& s, int r, int bt, int bn, float th, const int2* list,
                                           int n) {
  int32_t* slots = s.candidates + static_cast<int64_t>(r) * (s.top_k + s.capacity) * 2;
  int32_t* nearp = s.nearp ? s.nearp + 2 * static_cast<int64_t>(kNearPairs) * r : nullptr;
  const int lane = lane_id();
  for (int i0 = 0; i0 < n; i0 += 64) {
    const int i = i0 + lane;
    const int2 e = i < n ? list[i] : int2{0, 0};
    const float v = __int_as_float(e.y);
    const bool near = i < n && v != 0.f && v == v;
    const uint64_t mt = __ballot(i < n && !near);
    const uint64_t mn = __ballot(near);
    if (i < n && !near) {
      const int j = bt + lanes_below(mt);
      if (j < s.top_k) store_pair(slots + 2 * (s.top_k - 1 - j), e.x, v);
    }
    if (near) {
      const int j = bn + lanes_below(mn);
      if (nearp && j < kNearPairs) store_pair(nearp + 2 * j, e.x, v + th);
    }
    bt += __popcll(mt);
    bn += __popcll(mn);
  }
}

// The select launch's CTA body: score keys [k0, k1) of the CTA's request (or
// read them from a logits matrix) and select each wave's 64-key groups straight
// from the scores in registers onto the wave's own lists, which reach the slots
// when nearly full (one counter atomic per list) and at the end (one atomic
// per row and class for the whole CTA).  With arrivals, the CTA then arrives
// on its tile, the tile's last CTA runs the fit test and the rows' finish, and
// every CTA runs repair items until none is left.
template <int NT, bool kFused, int kKeysPerCta, class Src, class Args>
__device__ __forceinline__ void select_body(const Args& a, const SelectArgs& s, char* lds) {
  using Lay = Layout<NT, kFused>;
  MainShared<NT>& ms = *reinterpret_cast<MainShared<NT>*>(lds + Lay::kListOff);
  v4i* stage = reinterpret_cast<v4i*>(lds);
  QLds<NT>* ql = reinterpret_cast<QLds<NT>*>(lds + Lay::kStageBytes);
  const Sh<NT> sh = make_sh<NT>(lds, Lay::kFinCap, Lay::kCtlOff);
  const RescoreLds<NT> rl{stage, ql, reinterpret_cast<uint32_t*>(lds + Lay::kListOff)};
  Src src;
  src.bind(stage);
  src.bind_q(ql);
  const int lane = lane_id();
  const int w = wave_id();
  if (threadIdx.x == 0) sh.c->trace_n = 0;
  bool was_last = false;  // this CTA finished its tile
  for_each_segment([&](int b) { return tile_keys<NT>(a, b); }, a.batch, a.locate, a.per_request, kKeysPerCta, true, a.fast_ctas,
                   [&](int b, int L, int k0, int k1, int nctas) {
    PMQA_TR(sh, 1, b, nctas);
    float thr[NT], tlo[NT];
    int lim[NT];
    int ncl[NT], ntl[NT], nnl[NT];  // this wave's list entries: candidates, tie list (ties and near band), near band
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      thr[t] = s.thresholds[b * NT + t];
      // with a workspace, the keys in a narrow band just below the threshold
      // are kept too (a repair that needs a few more keys than the candidates
      // and ties then finds them there); they share the tie list
      tlo[t] = s.nearp ? near_floor(thr[t]) : thr[t];
      lim[t] = min(k1, row_end<NT>(s, b, L, t));
      ncl[t] = 0;
      ntl[t] = 0;
      nnl[t] = 0;
    }
    // A wave's lists of row t out: one atomic on the row's counter pair for
    // the candidate and tie bases (one more for the near band), then the pairs.
    auto flush = [&](int t) {
      const int r = b * NT + t;
      uint64_t old = 0;
      uint32_t nb = 0;
      if (lane == 0) {
        old = reserve_pair(s.counters + 2 * r, ncl[t], ntl[t] - nnl[t]);
        if (nnl[t]) nb = add_ag(s.nearc + static_cast<int64_t>(r) * kRowWords, static_cast<uint32_t>(nnl[t]));
      }
      const int bc = __shfl(static_cast<int>(static_cast<uint32_t>(old)), 0);
      const int bt = __shfl(static_cast<int>(static_cast<uint32_t>(old >> 32)), 0);
      const int bn = __shfl(static_cast<int>(nb), 0);
      store_cands(s, r, bc, ms.list[w][t], ncl[t]);
      store_ties(s, r, bt, bn, thr[t], ms.list[w][t] + kWaveList<NT> - ntl[t], ntl[t]);
      ncl[t] = 0;
      ntl[t] = 0;
      nnl[t] = 0;
    };
    src.init(a, b);
    stream_keys<NT, false>(
        src, k0, k1, L,
        [&](int, int p0, const float(&E)[NT]) {
          // this group's candidates and ties onto the wave's lists, positions
          // from the ballots
          const int p = p0 + lane;
          bool flushed = false;
#pragma unroll
          for (int t = 0; t < NT; ++t) {
            const float e = E[t];
            const bool vis = p < lim[t];
            const bool cand = vis && e > thr[t];
            const bool tie = vis && !(e > thr[t]) && !(e < tlo[t]);  // a tie, or in the near band
            const uint64_t mc = __ballot(cand);
            const uint64_t mt = __ballot(tie);
            const int nc = __popcll(mc);
            const int nt = __popcll(mt);
            const int nn = mt ? __popcll(__ballot(tie && e < thr[t])) : 0;
            if (ncl[t] + ntl[t] + nc + nt > kWaveList<NT>) {
              flush(t);
              flushed = true;
            }
            if (cand) ms.list[w][t][ncl[t] + lanes_below(mc)] = int2{p, __float_as_int(enc_cand(e, thr[t]))};
            if (tie) ms.list[w][t][kWaveList<NT> - 1 - (ntl[t] + lanes_below(mt))] = int2{p, __float_as_int(e - thr[t])};
            ncl[t] += nc;
            ntl[t] += nt;
            nnl[t] += nn;
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
        ms.count[w][t][0] = ncl[t];
        ms.count[w][t][1] = ntl[t] - nnl[t];
        ms.count[w][t][2] = nnl[t];
      }
    }
    __syncthreads();
    if (threadIdx.x < NT) {
      const int t = threadIdx.x;
      int tc = 0, tt = 0, tn = 0;
#pragma unroll
      for (int q = 0; q < kWaves; ++q) {
        tc += ms.count[q][t][0];
        tt += ms.count[q][t][1];
        tn += ms.count[q][t][2];
      }
      const int r = b * NT + t;
      const uint64_t old = (tc | tt) ? reserve_pair(s.counters + 2 * r, tc, tt) : 0;
      ms.base[t][0] = static_cast<int>(static_cast<uint32_t>(old));
      ms.base[t][1] = static_cast<int>(static_cast<uint32_t>(old >> 32));
      ms.base[t][2] = tn ? static_cast<int>(add_ag(s.nearc + static_cast<int64_t>(r) * kRowWords,
                                                      static_cast<uint32_t>(tn)))
                         : 0;
    }
    __syncthreads();
#pragma unroll
    for (int t = 0; t < NT; ++t) {
      int bc = ms.base[t][0], bt = ms.base[t][1], bn = ms.base[t][2];
      for (int q = 0; q < w; ++q) {
        bc += ms.count[q][t][0];
        bt += ms.count[q][t][1];
        bn += ms.count[q][t][2];
      }
      const int r = b * NT + t;
      store_cands(s, r, bc, ms.list[w][t], ncl[t]);
      store_ties(s, r, bt, bn, thr[t], ms.list[w][t] + kWaveList<NT> - ntl[t], ntl[t]);
    }
    PMQA_TR(sh, 2, b, 0);
    if (!s.ws) return;
    // arrival: this CTA's stores and counts are complete (written through)
    // before its count on the tile; the CTA that completes the count is last
    wait_vm_done();
    __syncthreads();
    if (threadIdx.x == 0) sh.c->is_last = add_ag(s.arrivals + b, 1) + 1 == nctas;
    __syncthreads();
    PMQA_TR(sh, 3, b, sh.c->is_last);
    was_last = sh.c->is_last != 0;
    if (was_last) {
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
      tile_finish<NT, kFused>(a, s, b, L, sh, rl);
      PMQA_TR(sh, 5, b, 0);
    }
  });
  if (s.ws) {
    __syncthreads();
    work_loop<NT, kFused>(a, s, lds, !was_last);
  }
}

template <int NT>
__global__ void __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(kFusedWaves<NT>, 8)))
fused_kernel(PagedArgs a, SelectArgs s) {
  using Lay = Layout<NT, true>;
  __shared__ __attribute__((aligned(16))) char lds[Lay::kBytes];
  global_view(a);
  global_view(s);
  if constexpr (NT >= 3)
    // (row 0's q in VGPRs: 2.3 us faster per call on the MTP batch than none,
    // two rows no faster again; the kernel stays within two waves per SIMD)
    select_body<NT, true, kFusedKeysPerCta, KvSourceQ<NT, kEpiF32, 1>>(a, s, lds);
  else
    select_body<NT, true, kFusedKeysPerCta, KvSource<NT>>(a, s, lds);
#ifdef PMQA_TRACE
  trace_flush(reinterpret_cast<Ctl<NT>*>(lds + Lay::kCtlOff));
#endif
}

template <int NT>
__global__ void __launch_bounds__(kThreads) select_kernel(LogitsArgs a, SelectArgs s) {
  using Lay = Layout<NT, false>;
  __shared__ __attribute__((aligned(16))) char lds[Lay::kBytes];
  global_view(a);
  global_view(s);
  select_body<NT, false, kSelectKeysPerCta, LogitsSource<NT>>(a, s, lds);
}

// LDS of the fused launches: two CTAs per compute unit (the VGPR budget allows two).
static_assert(2 * Layout<1, true>::kBytes <= 160 * 1024, "two next_n = 1 CTAs per compute unit");
static_assert(2 * Layout<2, true>::kBytes <= 160 * 1024, "two next_n = 2 CTAs per compute unit");
static_assert(2 * Layout<3, true>::kBytes <= 160 * 1024, "two next_n = 3 CTAs per compute unit");
static_assert(2 * Layout<4, true>::kBytes <= 160 * 1024, "two next_n = 4 CTAs per compute unit");

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


// PMQA_VALIDATE=1 for prefill-shaped rows: every row end within max_context,
// every tile's request a row of the block table, the table entries a tile
// reads (its largest row end's pages) valid ids, counters and arrivals zero.
pmqa_status validate_prefill(hipStream_t st, const int32_t* tile_req, const int32_t* row_ends, int32_t tiles,
                             int32_t tile_rows, int32_t requests, int32_t max_context, const int32_t* bt,
                             int64_t bt_stride, int32_t bt_width, int32_t bs, int64_t num_blocks,
                             const int32_t* counters, const int32_t* arrivals) {
  if (!validate_enabled() || stream_capturing(st) || tiles == 0) return PMQA_OK;
  const int64_t rows = static_cast<int64_t>(tiles) * tile_rows;
  std::vector<int32_t> TR, E, T, C, A;
  bool ok = copy_span(TR, tile_req, static_cast<int64_t>(tiles), st) && copy_span(E, row_ends, rows, st) &&
            copy_span(T, bt, static_cast<int64_t>(requests - 1) * bt_stride + bt_width, st) &&
            copy_span(C, counters, 2 * rows, st);
  if (arrivals) ok = ok && copy_span(A, arrivals, static_cast<int64_t>(tiles), st);
  if (!ok || hipStreamSynchronize(st) != hipSuccess) return PMQA_ERR_LAUNCH;
  for (int32_t b = 0; b < tiles; ++b) {
    const int32_t req = TR[static_cast<size_t>(b)];
    if (req < 0 || req >= requests) return PMQA_ERR_CONTENT;
    int32_t L = 0;
    for (int32_t t = 0; t < tile_rows; ++t) {
      const int32_t e = E[static_cast<size_t>(b) * tile_rows + t];
      if (e < 0 || e > max_context) return PMQA_ERR_CONTENT;
      L = std::max(L, e);
    }
    const int64_t pages = ceil_div(L, bs);
    if (pages > bt_width) return PMQA_ERR_CONTENT;
    for (int64_t j = 0; j < pages; ++j) {
      const int32_t id = T[static_cast<size_t>(req * bt_stride + j)];
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
  a.fast_ctas = 0;
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
  a.row_ends = nullptr;
  a.tile_req = nullptr;
  a.qsf = nullptr;
  a.sf_inter = 0;
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
                       void* workspace) {
  SelectArgs s;
  s.thresholds = thr;
  s.counters = cnt;
  s.candidates = cand;
  s.arrivals = arr;
  s.ranges = ranges;
  s.topk_idx = topk;
  s.ws = arr ? static_cast<uint32_t*>(workspace) : nullptr;
  const WsLayout lay = workspace_layout(batch, rows, max_context, fused);
  s.ovf = s.ws ? reinterpret_cast<int32_t*>(s.ws + lay.overflow) : nullptr;
  s.nearp = s.ws ? reinterpret_cast<int32_t*>(s.ws + lay.near) : nullptr;
  s.nearc = s.ws ? s.ws + lay.row_state + 4 : nullptr;
  s.scores = s.ws && fused ? reinterpret_cast<float*>(s.ws + lay.scores) : nullptr;
  s.score_ld = score_stride(max_context);
  s.capacity = cap;
  s.top_k = top_k;
  s.rows = rows;
  s.resident = 0;
  s.row_ends = nullptr;
  return s;
}

pmqa_status launched() { return hipGetLastError() == hipSuccess ? PMQA_OK : PMQA_ERR_LAUNCH; }

// One launch of K<nt>.  The located grid -- as many CTAs as fit on the device
// at once, but at most 15/8 per compute unit -- runs when that gives every
// tile a CTA (256 prefill tiles of 4 rows: 3328 CTAs in waves took 412 us per
// call against 480 located), else a.per_request CTAs per request
// (PMQA_ERR_SHAPE if that grid is too large).  (The cap: on the 64-request decode batch 480 CTAs
// stream 2.7 us faster than the 768 that fit, whose third CTA on each compute
// unit gets its first keys some 15 us after the first and finishes last; 432
// and fewer are slower again.)  A select launch learns whether all of its CTAs
// fit on the device at once (only then do CTAs without work wait for repair
// items).
template <template <int> class K, class A, class... Rest>
pmqa_status launch_k(int nt, hipStream_t st, A a, Rest... rest) {
  pmqa_status status = PMQA_OK;
  auto go = [&](auto fn) {
    const int64_t fit = resident_ctas(reinterpret_cast<const void*>(fn));
    int64_t g = std::min<int64_t>(fit, static_cast<int64_t>(device_cus()) * 15 / 8);
    a.locate = g >= static_cast<int64_t>(a.batch);
    a.fast_ctas = static_cast<int32_t>(std::min<int64_t>(g, device_cus()));
    if (!a.locate) g = static_cast<int64_t>(a.per_request) * a.batch;
    if (g > 0x7fffffff) {
      status = PMQA_ERR_SHAPE;
      return;
    }
    auto mark = [&](auto& x) {
      if constexpr (std::is_same<std::decay_t<decltype(x)>, SelectArgs>::value) x.resident = g <= fit ? 1 : 0;
    };
    (mark(rest), ...);
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

// Zeroes words [0, n) of a workspace (a kernel, not a memset: callers may
// capture the call in a graph).
__global__ void __launch_bounds__(kThreads) clear_words_kernel(uint32_t* w, int64_t n) {
  for (int64_t i = static_cast<int64_t>(blockIdx.x) * kThreads + threadIdx.x; i < n;
       i += static_cast<int64_t>(gridDim.x) * kThreads)
    w[i] = 0u;
}

// Every state word of the workspace (jobs, row states, histograms) is back to
// zero when a call ends, but where they lie depends on the batch and next_n of
// the call.  The library remembers the layout each workspace was last used
// with and, when a call lays it out otherwise, clears the new layout's state
// words first (one more launch on the same stream); with clear_first_use it
// does so also the first time it sees the workspace.
pmqa_status prepare_workspace(void* ws, int64_t batch, int64_t rows, int64_t max_context, bool fused,
                              hipStream_t st, bool clear_first_use) {
  static std::mutex mu;
  static std::map<void*, std::vector<int64_t>> last;
  const std::vector<int64_t> key{batch, rows};
  {
    std::lock_guard<std::mutex> lock(mu);
    auto it = last.find(ws);
    if (it == last.end()) {
      last[ws] = key;  // first use: zeroed by the caller, or cleared here
      if (!clear_first_use) return PMQA_OK;
    } else {
      if (it->second == key) return PMQA_OK;
      it->second = key;
    }
  }
  const int64_t n = workspace_layout(batch, rows, max_context, fused).bucket;  // jobs, row states, histograms
  const int64_t g = std::min<int64_t>(1024, ceil_div(n, kThreads));
  hipLaunchKernelGGL(clear_words_kernel, dim3(static_cast<unsigned>(g)), dim3(kThreads), 0, st,
                     static_cast<uint32_t*>(ws), n);
  return launched();
}

// The finish-stage workspace of pmqa_fused_logits_select_noalloc, for callers
// that cannot allocate.  Every device the library runs on holds its own copy
// from the code object's load until the process ends.  Host code never passes
// the array's name to a kernel or a copy (on the host it is only a stand-in
// for the symbol): it uses the device address scratch_address() looked up.
constexpr size_t kScratchBytes = PMQA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes % 256 == 0, "scratch size");
static __device__ __align__(256) uint32_t scratch[kScratchBytes / 4];

// Device address of `scratch` on device `dev`, looked up once per device with
// that device current; nullptr if the lookup fails.
void* scratch_address(int dev) {
  static std::mutex mu;
  static std::map<int, void*> cache;
  std::lock_guard<std::mutex> lock(mu);
  auto it = cache.find(dev);
  if (it != cache.end()) return it->second;
  int cur = 0;
  if (hipGetDevice(&cur) != hipSuccess) return nullptr;
  if (cur != dev && hipSetDevice(dev) != hipSuccess) {
    (void)hipGetLastError();
    return nullptr;
  }
  void* p = nullptr;
  const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (cur != dev) (void)hipSetDevice(cur);
  if (e != hipSuccess || p == nullptr) {
    (void)hipGetLastError();
    return nullptr;
  }
  cache[dev] = p;
  return p;
}

template <int NT> struct LogitsK { static constexpr auto fn = logits_kernel<NT, kEpiF32>; };
template <int NT> struct LogitsAcc16K { static constexpr auto fn = logits_kernel<NT, kEpiAcc16>; };
template <int NT> struct LogitsF16K { static constexpr auto fn = logits_kernel<NT, kEpiF16>; };
template <int NT> struct Fp4K { static constexpr auto fn = fp4_logits_kernel<NT, kEpiF32>; };
template <int NT> struct Fp4F16K { static constexpr auto fn = fp4_logits_kernel<NT, kEpiF16>; };
template <int NT> struct Fp4Bf16K { static constexpr auto fn = fp4_logits_kernel<NT, kEpiBf16>; };
template <int NT> struct FusedK { static constexpr auto fn = fused_kernel<NT>; };
template <int NT> struct SelectK { static constexpr auto fn = select_kernel<NT>; };

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
  st = launch_k<LogitsK>(next_n, hs, a, static_cast<void*>(out), out_stride, kOutF32);
  return st != PMQA_OK ? st : launched();
}

pmqa_status pmqa_mqa_logits_typed(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                  const int32_t* block_tables, int64_t block_table_stride,
                                  int32_t block_table_width, const int32_t* seq_lens, int64_t seq_lens_stride,
                                  int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
                                  int32_t block_size, int64_t num_blocks, int32_t max_seq_len, void* out,
                                  int64_t out_stride, int32_t output_dtype, int32_t epi_dtype, int32_t acc_dtype,
                                  void* stream) {
  pmqa_status st = pmqa_check_logits_typed_args(q, kv_fused, weights, block_tables, block_table_stride,
                                                block_table_width, seq_lens, seq_lens_stride, batch_size, next_n,
                                                num_heads, head_dim, block_size, num_blocks, max_seq_len, out,
                                                out_stride, output_dtype, epi_dtype, acc_dtype);
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
  const int out_type = output_dtype == PMQA_DTYPE_F16 ? kOutF16 : kOutF32;
  // a float16 epilogue starts from float16 dot products: acc_dtype changes nothing then
  if (epi_dtype == PMQA_DTYPE_F16)
    st = launch_k<LogitsF16K>(next_n, hs, a, out, out_stride, out_type);
  else if (acc_dtype == PMQA_DTYPE_F16)
    st = launch_k<LogitsAcc16K>(next_n, hs, a, out, out_stride, out_type);
  else
    st = launch_k<LogitsK>(next_n, hs, a, out, out_stride, out_type);
  return st != PMQA_OK ? st : launched();
}

pmqa_status pmqa_fp4_mqa_logits(const uint8_t* q, const int32_t* q_sf, const uint8_t* kv_fused, const float* weights,
                                const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
                                const int32_t* seq_lens, int64_t seq_lens_stride, int32_t batch_size,
                                int32_t next_n, int32_t num_heads, int32_t head_dim, int32_t block_size,
                                int64_t num_blocks, int32_t max_seq_len, int32_t sf_vec_size,
                                int32_t kv_sf_interleaved, void* out, int64_t out_stride, int32_t output_dtype,
                                int32_t epi_dtype, void* stream) {
  pmqa_status st = pmqa_check_fp4_logits_args(q, q_sf, kv_fused, weights, block_tables, block_table_stride,
                                              block_table_width, seq_lens, seq_lens_stride, batch_size, next_n,
                                              num_heads, head_dim, block_size, num_blocks, max_seq_len,
                                              sf_vec_size, kv_sf_interleaved, out, out_stride, output_dtype,
                                              epi_dtype);
  if (st != PMQA_OK) return st;
  if (batch_size > 65535) return PMQA_ERR_SHAPE;
  const int64_t gx = ceil_div(max_seq_len, kLogitsKeysPerCta);
  if (batch_size == 0 || gx == 0) return PMQA_OK;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  st = validate_content(hs, seq_lens, seq_lens_stride, batch_size, max_seq_len, block_tables,
                        block_table_stride, block_table_width, block_size, num_blocks, nullptr, 0, nullptr);
  if (st != PMQA_OK) return st;
  PagedArgs a = paged_args(q, kv_fused, weights, block_tables, block_table_stride, seq_lens, seq_lens_stride,
                           block_size, batch_size, gx);
  a.block_bytes = block_size * (kDim / 2 + kDim / 32);
  a.scale_off = block_size * (kDim / 2);
  a.qsf = q_sf;
  a.sf_inter = kv_sf_interleaved ? 1 : 0;
  const int out_type =
      output_dtype == PMQA_DTYPE_F16 ? kOutF16 : (output_dtype == PMQA_DTYPE_BF16 ? kOutBf16 : kOutF32);
  if (epi_dtype == PMQA_DTYPE_F16)
    st = launch_k<Fp4F16K>(next_n, hs, a, out, out_stride, out_type);
  else if (epi_dtype == PMQA_DTYPE_BF16)
    st = launch_k<Fp4Bf16K>(next_n, hs, a, out, out_stride, out_type);
  else
    st = launch_k<Fp4K>(next_n, hs, a, out, out_stride, out_type);
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
  const LogitsArgs a{logits, logits_stride, seq_lens, seq_lens_stride, batch_size, 0, static_cast<int32_t>(gx), 0};
  const SelectArgs s = select_args(thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx,
                                   batch_size, static_cast<int32_t>(rows), max_context, false, workspace);
  if (s.ws) st = prepare_workspace(workspace, batch_size, rows, max_context, false, hs, false);
  if (st == PMQA_OK) st = launch_k<SelectK>(next_n, hs, a, s);
  return st != PMQA_OK ? st : launched();
}

}  // extern "C"

namespace {

// pmqa_fused_logits_select with a choice: scratch_mode marks the library's
// static scratch as the workspace (cleared on its first use per device, no
// PMQA_VALIDATE host copies).
pmqa_status fused_select(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                         const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
                         const int32_t* seq_lens, int64_t seq_lens_stride, int32_t batch_size, int32_t next_n,
                         int32_t num_heads, int32_t head_dim, int32_t block_size, int64_t num_blocks,
                         int32_t max_context, float* thresholds, int32_t* counters, int32_t* candidates,
                         int32_t capacity, int32_t top_k, int32_t* arrivals, int32_t* ranges, int32_t* topk_idx,
                         void* workspace, size_t workspace_bytes, void* stream, bool scratch_mode) {
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
  if (!scratch_mode) {
    st = validate_content(hs, seq_lens, seq_lens_stride, batch_size, max_context, block_tables, block_table_stride,
                          block_table_width, block_size, num_blocks, counters, rows, arrivals);
    if (st != PMQA_OK) return st;
  }
  const PagedArgs a = paged_args(q, kv_fused, weights, block_tables, block_table_stride, seq_lens,
                                 seq_lens_stride, block_size, batch_size, gx);
  const SelectArgs s = select_args(thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx,
                                   batch_size, static_cast<int32_t>(rows), max_context, true, workspace);
  if (s.ws) st = prepare_workspace(workspace, batch_size, rows, max_context, true, hs, scratch_mode);
  if (st == PMQA_OK) st = launch_k<FusedK>(next_n, hs, a, s);
  return st != PMQA_OK ? st : launched();
}

}  // namespace

extern "C" {

pmqa_status pmqa_fused_logits_select(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                     const int32_t* block_tables, int64_t block_table_stride,
                                     int32_t block_table_width, const int32_t* seq_lens, int64_t seq_lens_stride,
                                     int32_t batch_size, int32_t next_n, int32_t num_heads, int32_t head_dim,
                                     int32_t block_size, int64_t num_blocks, int32_t max_context,
                                     float* thresholds, int32_t* counters, int32_t* candidates, int32_t capacity,
                                     int32_t top_k, int32_t* arrivals, int32_t* ranges, int32_t* topk_idx,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  return fused_select(q, kv_fused, weights, block_tables, block_table_stride, block_table_width, seq_lens,
                      seq_lens_stride, batch_size, next_n, num_heads, head_dim, block_size, num_blocks, max_context,
                      thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx, workspace,
                      workspace_bytes, stream, false);
}

pmqa_status pmqa_prefill_select(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                const int32_t* block_tables, int64_t block_table_stride, int32_t block_table_width,
                                int32_t num_requests, const int32_t* tile_requests, const int32_t* row_ends,
                                int32_t num_tiles, int32_t tile_rows, int32_t num_heads, int32_t head_dim,
                                int32_t block_size, int64_t num_blocks, int32_t max_context, float* thresholds,
                                int32_t* counters, int32_t* candidates, int32_t capacity, int32_t top_k,
                                int32_t* arrivals, int32_t* ranges, int32_t* topk_idx, void* workspace,
                                size_t workspace_bytes, void* stream) {
  pmqa_status st = pmqa_check_prefill_args(q, kv_fused, weights, block_tables, block_table_stride, block_table_width,
                                           num_requests, tile_requests, row_ends, num_tiles, tile_rows, num_heads,
                                           head_dim, block_size, num_blocks, max_context, thresholds, counters,
                                           candidates, capacity, top_k, arrivals, ranges, topk_idx, workspace,
                                           workspace_bytes);
  if (st != PMQA_OK) return st;
  if (num_tiles > 65535) return PMQA_ERR_SHAPE;
  if (num_tiles == 0) return PMQA_OK;
  const int64_t gx = std::max<int64_t>(1, ceil_div(max_context, kFusedKeysPerCta));
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int64_t rows = static_cast<int64_t>(num_tiles) * tile_rows;
  st = validate_prefill(hs, tile_requests, row_ends, num_tiles, tile_rows, num_requests, max_context, block_tables,
                        block_table_stride, block_table_width, block_size, num_blocks, counters, arrivals);
  if (st != PMQA_OK) return st;
  PagedArgs a = paged_args(q, kv_fused, weights, block_tables, block_table_stride, nullptr, 0, block_size, num_tiles,
                           gx);
  a.row_ends = row_ends;
  a.tile_req = tile_requests;
  SelectArgs s = select_args(thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx, num_tiles,
                             static_cast<int32_t>(rows), max_context, true, workspace);
  s.row_ends = row_ends;
  if (s.ws) st = prepare_workspace(workspace, num_tiles, rows, max_context, true, hs, false);
  if (st == PMQA_OK) st = launch_k<FusedK>(tile_rows, hs, a, s);
  return st != PMQA_OK ? st : launched();
}

pmqa_status pmqa_fused_logits_select_noalloc(const uint8_t* q, const uint8_t* kv_fused, const float* weights,
                                             const int32_t* block_tables, int64_t block_table_stride,
                                             int32_t block_table_width, const int32_t* seq_lens,
                                             int64_t seq_lens_stride, int32_t batch_size, int32_t next_n,
                                             int32_t num_heads, int32_t head_dim, int32_t block_size,
                                             int64_t num_blocks, int32_t max_context, float* thresholds,
                                             int32_t* counters, int32_t* candidates, int32_t capacity, int32_t top_k,
                                             int32_t* arrivals, int32_t* ranges, int32_t* topk_idx, void* stream) {
  void* ws = nullptr;
  size_t bytes = 0;
  if (arrivals) {
    // an invalid size gives 0 here and its own status from the argument check
    if (pmqa_workspace_bytes(2, batch_size, next_n, max_context) > kScratchBytes) return PMQA_ERR_SCRATCH;
    int dev = 0;
    if (hipStreamGetDevice(static_cast<hipStream_t>(stream), &dev) != hipSuccess) {
      (void)hipGetLastError();
      return PMQA_ERR_LAUNCH;
    }
    ws = scratch_address(dev);
    if (!ws) return PMQA_ERR_LAUNCH;
    bytes = kScratchBytes;
  }
  return fused_select(q, kv_fused, weights, block_tables, block_table_stride, block_table_width, seq_lens,
                      seq_lens_stride, batch_size, next_n, num_heads, head_dim, block_size, num_blocks, max_context,
                      thresholds, counters, candidates, capacity, top_k, arrivals, ranges, topk_idx, ws, bytes,
                      stream, true);
}

#ifdef PMQA_TRACE
int32_t pmqa_trace_read(void* host, size_t bytes) {
  const size_t n = std::min(bytes, sizeof(g_trace));
  if (hipMemcpyFromSymbol(host, HIP_SYMBOL(g_trace), n, 0, hipMemcpyDeviceToHost) != hipSuccess) return -1;
  static const std::vector<uint64_t> zero(sizeof(g_trace) / sizeof(uint64_t), 0);
  if (hipMemcpyToSymbol(HIP_SYMBOL(g_trace), zero.data(), sizeof(g_trace), 0, hipMemcpyHostToDevice) != hipSuccess) return -1;
  return static_cast<int32_t>(n);
}
#endif

}  // extern "C"
