// pda_internal.h -- argument blocks and launchers shared by the host entry
// points (pda_host.cpp) and the kernels (pda_gqa.hip, pda_mla.hip).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace pda {

// Tokens processed per wave iteration of the GQA kernel ("tile").  Page sizes
// must be multiples of it, so a tile never crosses a page boundary.
constexpr int kTileTokens = 16;
// Waves per workgroup of the GQA kernel and tiles each wave keeps in flight
// ahead of the one it computes (register buffers).  Tuning constants.
#ifndef PDA_GQA_WAVES
#define PDA_GQA_WAVES 4
#endif
#ifndef PDA_GQA_PREFETCH
#define PDA_GQA_PREFETCH 2
#endif
// Matrix-core GQA kernel: tiles per step (loads of a step are issued back to
// back) and steps in flight per wave (1: no prefetch beyond the current
// step), for grid calls (uniform work: fewer loads in flight contend less,
// B=64 42.4 against 42.7 us, B=4 85.1 against 86.2) and for ordered calls
// (units of mixed sizes start with their loads in flight: ragged fp8 97.6
// against 100.1).
#ifndef PDA_GQA_STEP_TILES
#define PDA_GQA_STEP_TILES 1
#endif
#ifndef PDA_GQA_STEPS_IN_FLIGHT
#define PDA_GQA_STEPS_IN_FLIGHT 1
#endif
// Tiles per step and grid steps in flight for 1-byte (fp8) caches: their tiles
// hold half the bytes of a 16-bit tile, so a step of two tiles issues as many
// bytes as one 16-bit tile does.
#ifndef PDA_GQA_STEP_TILES_FP8
#define PDA_GQA_STEP_TILES_FP8 2
#endif
#ifndef PDA_GQA_STEPS_IN_FLIGHT_FP8
#define PDA_GQA_STEPS_IN_FLIGHT_FP8 1
#endif
#ifndef PDA_GQA_STEPS_IN_FLIGHT_ORDERED
#define PDA_GQA_STEPS_IN_FLIGHT_ORDERED 2
#endif
// Steps in flight per wave when one wave owns a work unit (no other wave of
// the workgroup covers its latency).
#ifndef PDA_GQA_STEPS_IN_FLIGHT_WAVE
#define PDA_GQA_STEPS_IN_FLIGHT_WAVE 2
#endif
// Registers the GQA kernels may spend on the ring of in-flight tiles (caps
// the prefetch depth for wide rows).
#ifndef PDA_GQA_RING_REGS
#define PDA_GQA_RING_REGS 96
#endif
// 1: each lane loads its K rows of a tile in a lane-dependent order so that
// every step of the score reduce-scatter is a single DPP add (a load
// instruction then covers pieces of several rows instead of whole rows).
#ifndef PDA_GQA_PERMUTE_ROWS
#define PDA_GQA_PERMUTE_ROWS 0
#endif
constexpr int kGqaWaves = PDA_GQA_WAVES;
constexpr bool kGqaPermuteRows = PDA_GQA_PERMUTE_ROWS != 0;
constexpr int kGqaPrefetch = PDA_GQA_PREFETCH;
constexpr int kGqaRingRegs = PDA_GQA_RING_REGS;
constexpr int kGqaStepTiles = PDA_GQA_STEP_TILES;
constexpr int kGqaStepsInFlight = PDA_GQA_STEPS_IN_FLIGHT;
constexpr int kGqaStepsInFlightOrdered = PDA_GQA_STEPS_IN_FLIGHT_ORDERED;
constexpr int kGqaStepTilesFp8 = PDA_GQA_STEP_TILES_FP8;
constexpr int kGqaStepsInFlightFp8 = PDA_GQA_STEPS_IN_FLIGHT_FP8;
constexpr int kGqaStepsInFlightWave = PDA_GQA_STEPS_IN_FLIGHT_WAVE;

// Split layout shared by the attention kernels and the combine kernel.  For
// sequence b with n = context_lens[b] tokens and pages = ceil(n / P):
//   n <= split_min_tokens or max_splits == 1: one split over every page, the
//   kernel writes the final output directly;
//   otherwise S_b = ceil(pages / pages_per_split) splits of pages_per_split
//   pages each (the last one shorter), written as partials and combined.
struct SplitLayout {
  int32_t pages_per_split;
  int32_t max_splits;
  int32_t split_min_tokens;
};

// The rules of an ordered call's work-unit list (see OrderArgs): the
// sequences' splits and the longest-first order.
struct UnitPlan {
  int32_t batch, page_size, balanced, target_units, min_chunk_pages;
  SplitLayout split;
};

// Largest batch whose workgroups plan their own units (each reads every
// length; beyond it a planning kernel writes the list).
constexpr int kInKernelPlanMaxBatch = 1024;

struct GqaArgs {
  const void* q;
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;
  float* lse;       // nullable
  float* part_o;    // [B, s_q, Hq, max_splits, dv] fp32 (when max_splits > 1)
  float* part_lse;  // [B, s_q, Hq, max_splits] fp32
  int32_t batch, num_q_heads, num_kv_heads, group, head_tiles;
  // query tokens per sequence; the rows of a KV group are (query i, head g)
  // pairs, row i * group + g; causal: query i sees n - (q_len - 1 - i) tokens
  int32_t q_len, causal;
  int32_t page_size, max_pages;
  int32_t log2_page;     // page_size == 1 << log2_page
  // cache strides in elements: token-major pages [P, Hkv, d] have tok_stride
  // Hkv * d and head_stride d, head-major pages [Hkv, P, d] tok_stride d and
  // head_stride P * d; page_stride is P * Hkv * d either way
  int32_t tok_stride;
  int32_t head_stride;
  int64_t page_stride;
  float qk_scale_log2;   // scale * k_scale * log2(e)
  float v_scale;
  SplitLayout split;
  // Ordered work: units[4u .. 4u + 3] = {b, split (-1: only split), t0, t1}
  // for the listed units, b = -1 after (see WorkUnit); the grid is (kv heads
  // * head tiles) x unit_count in x.  Null: the grid is (batch, kv head, head
  // tile) in x and the split in y, ranges from SplitLayout.
  const int32_t* units;
  int32_t unit_count;
  // Ordered calls whose workgroups derive their own unit from context_lens
  // (no planning launch; units is null then): the list's rules, and where
  // each sequence's split count goes for the combine kernel.
  int32_t plan_in_kernel;
  UnitPlan plan;
  int32_t* seq_splits;
  // waves per workgroup of the matrix-core kernel: 4 (a unit's tiles dealt
  // over four waves, merged in LDS) or 1 (one wave per unit; grid calls with
  // one column tile)
  int32_t waves;
};

struct CombineArgs {
  const void* part_o;  // fp32, or binary16 when part_f16 (see launch_combine)
  const float* part_lse;
  const int32_t* context_lens;
  void* out;
  float* lse;  // nullable
  int32_t batch, num_q_heads, head_dim_v, page_size;
  int32_t q_len;  // partial rows are (b, query i, head h); lse is [B, Hq, q_len]
  SplitLayout split;
  // ordered calls: the number of splits of each sequence, written by the
  // planning kernel (null: from SplitLayout)
  const int32_t* seq_splits;
};

struct MlaArgs {
  const void* q;           // [B, q_len, Hq, 576 or 320] bf16
  const void* kv_cache;    // [num_pages, P, 576 or 320] bf16 or fp8 (E4M3)
  const int32_t* block_tables;
  const int32_t* context_lens;
  void* out;               // [B, q_len, Hq, 512 or 256] bf16
  float* lse;
  float* part_o;           // binary16 partial rows [B, q_len, Hq, max_splits, dv]
                           // (in the workspace's fp32-sized area)
  float* part_lse;
  int32_t batch, num_q_heads, head_tiles;
  int32_t q_len, causal;   // as in GqaArgs; tile rows are (query i, head h), i * Hq + h
  int32_t page_size, max_pages;
  int32_t log2_page;       // page_size == 1 << log2_page
  float qk_scale_log2;     // scale * kv_scale * log2(e)
  float v_scale;           // the latent's dequantization scale (1 for bf16)
  SplitLayout split;
  const int32_t* units;    // as in GqaArgs (x = head tiles * unit_count)
  int32_t unit_count;
};

// The planning pass of ordered calls: splits every sequence, lists every
// (sequence, split) work unit by decreasing token count (WorkUnit layout,
// [batch * max_splits] units) and records each sequence's split count.
//   grid schedule: the SplitLayout (pages_per_split, split threshold);
//   balanced schedule: a chunk of max(min_chunk_pages, ceil(total pages /
//   target_units)) pages; sequences longer than a chunk (and than the split
//   threshold) take ceil(pages / chunk) splits, at most max_splits, of
//   ceil(pages / splits) pages each.
struct OrderArgs {
  const int32_t* context_lens;
  int32_t* units;          // [capacity * 4]
  int32_t* seq_splits;     // [batch]
  int32_t capacity;        // listed units never exceed it (see the planner)
  int32_t batch, page_size;
  int32_t balanced, target_units, min_chunk_pages;
  SplitLayout split;
};

// KV append: s_new new tokens per sequence into the paged K (and V) cache.
struct AppendArgs {
  const void* k_new;             // [B, s_new, Hkv, head_dim]
  const void* v_new;             // [B, s_new, Hkv, head_dim_v] (null with v_cache)
  void* k_cache;                 // [num_pages, P, Hkv, head_dim] or [num_pages, Hkv, P, head_dim]
  void* v_cache;                 // the same with head_dim_v, or null
  int32_t head_major;            // 1: pages are [Hkv, P, width]
  const int32_t* block_tables;   // [B, max_pages]
  const int32_t* positions;      // [B]: first new token's position, < 0 skips b
  int32_t batch, s_new, num_kv_heads, head_dim, head_dim_v, page_size, max_pages;
  float k_scale, v_scale;        // E4M3 caches: stored byte = e4m3(x / scale)
};

// Streaming-read probe (pda_stream_probe): the K/V reads of a GQA grid call.
struct ProbeArgs {
  // (the first 16 dwords arrive preloaded in scalar registers: everything the
  // first loads need)
  const void* k_cache;
  const void* v_cache;
  const int32_t* block_tables;
  const int32_t* context_lens;
  SplitLayout split;
  int32_t num_kv_heads, page_size, max_pages, log2_page, tok_stride;  // tok_stride: elements
  uint32_t* sink;  // [max_splits][B * Hkv]: one word per workgroup
  int32_t batch, elem_bytes, head_stride;  // head_stride: elements, as in GqaArgs
  int64_t page_stride;
};
static_assert(offsetof(ProbeArgs, sink) == 64, "probe arguments: prologue values preloaded");

// Precondition check of device-resident inputs (see pda_check_inputs).
struct CheckArgs {
  const int32_t* block_tables;  // [batch, max_pages]
  const int32_t* context_lens;  // [batch]
  const int32_t* positions;     // [batch] or null (append positions)
  int32_t* result;              // [3]: bad lengths, bad table entries, bad positions
  int32_t batch, max_pages, page_size, num_pages, s_new;
};

// Column tiles of 16 rows in a workgroup of the GQA matrix-core kernel for
// `rows` (query token, head) rows per KV group: two when there are more than
// 16 (and d <= 128, for registers), so that one K/V load serves 32 rows --
// unless the table holds fewer than 2048 tokens per sequence and 17 to 32
// rows: there, twice the workgroups with half the rows each finish sooner
// (MQA with 32 heads, B=64: 17.6 against 19.6 us at 1024 tokens, even at
// 2048, 34.5 against 37.2 us at 4096).
inline int gqa_mfma_col_tiles(int rows, int head_dim, int64_t max_tokens) {
  return rows > 16 && head_dim <= 128 && (rows > 32 || max_tokens >= 2048) ? 2 : 1;
}

// Column groups of 16 rows in a workgroup of the MLA matrix-core kernel for
// `rows` (query token, head) rows per sequence: two (512 threads) once there
// are more than 16, so that one staged block serves 32 rows.
inline int mla_column_groups(int rows) { return rows > 16 ? 2 : 1; }

// Host-side support queries (no HIP calls).
bool gqa_supported(int q_dtype, int kv_dtype, int head_dim, int head_dim_v);
int gqa_tile_heads(int group);  // query heads per workgroup tile for a group size

bool gqa_mfma_supported(int q_dtype, int kv_dtype, int head_dim);
bool append_supported(int src_dtype, int cache_dtype);

// Launchers (return the launch error, hipSuccess otherwise).
hipError_t launch_gqa_mfma(const GqaArgs& a, int q_dtype, int kv_dtype, int head_dim,
                           int max_splits, hipStream_t stream);
hipError_t launch_gqa(const GqaArgs& a, int q_dtype, int kv_dtype, int head_dim,
                      int tile_heads, int max_splits, hipStream_t stream);
// part_f16: the partial outputs are binary16 (the MLA kernels write them so;
// the GQA kernels write fp32)
hipError_t launch_combine(const CombineArgs& a, int out_dtype, bool part_f16, hipStream_t stream);
hipError_t launch_order(const OrderArgs& a, hipStream_t stream);
hipError_t launch_mla(const MlaArgs& a, int variant, int kv_dtype, int head_dim, int max_splits,
                      hipStream_t stream);
hipError_t launch_append(const AppendArgs& a, int src_dtype, int cache_dtype, hipStream_t stream);
hipError_t launch_check(const CheckArgs& a, hipStream_t stream);
hipError_t launch_probe(const ProbeArgs& a, int row_bytes, int max_splits, int steps_in_flight,
                        int waves, hipStream_t stream);

}  // namespace pda
