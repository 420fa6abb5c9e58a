// pda_host.cpp -- the C ABI of libpda (include/pda.h): argument validation,
// the split planner and kernel dispatch.  Every host-checkable argument is
// validated before any work is queued, so invalid calls never touch a device
// (the planner may only ask the runtime for the device's compute units).
#include "pda.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <atomic>
#include <cstdint>

#include "pda_internal.h"

namespace {

constexpr int kMaxDevices = 64;
// (calls from several host threads may fill an entry at once, with the same value)
std::atomic<int> g_cu_count[kMaxDevices];

// Compute units of the current device (cached per device id); 0 on failure.
int device_cus() {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return 0;
  if (dev < kMaxDevices) {
    const int cached = g_cu_count[dev].load(std::memory_order_relaxed);
    if (cached > 0) return cached;
  }
  int n = 0;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (dev < kMaxDevices) g_cu_count[dev].store(n, std::memory_order_relaxed);
  return n;
}

int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool valid_dtype(int d) { return d >= PDA_F32 && d <= PDA_FP8_E4M3; }

// Query tokens per sequence (q_len 0 stands for 1).
int query_len(const pda_shape* s) { return s->q_len > 1 ? s->q_len : 1; }

// Shape checks common to both entry points.
int check_shape(const pda_shape* s, bool mla) {
  if (!s) return PDA_ERR_INVALID_ARG;
  if (s->batch < 0 || s->num_q_heads <= 0 || s->num_kv_heads <= 0 || s->head_dim <= 0 ||
      s->head_dim_v <= 0 || s->page_size <= 0 || s->max_pages_per_seq <= 0 ||
      s->num_pages <= 0 || s->split_min_tokens < 0 || s->q_len < 0 ||
      (s->causal != 0 && s->causal != 1) ||
      (s->schedule != PDA_SCHEDULE_GRID && s->schedule != PDA_SCHEDULE_BALANCED) ||
      (s->kv_layout != PDA_KV_TOKEN_MAJOR && s->kv_layout != PDA_KV_HEAD_MAJOR))
    return PDA_ERR_INVALID_ARG;
  // (query, head) rows of a sequence stay well inside 32-bit indexing
  if ((int64_t)query_len(s) * s->num_q_heads > (1 << 20)) return PDA_ERR_UNSUPPORTED;
  if (!valid_dtype(s->q_dtype) || !valid_dtype(s->kv_dtype)) return PDA_ERR_INVALID_ARG;
  if (s->num_q_heads % s->num_kv_heads != 0) return PDA_ERR_INVALID_ARG;
  if ((int64_t)s->max_pages_per_seq * s->page_size > INT32_MAX) return PDA_ERR_INVALID_ARG;
  if (mla) {
    if (s->num_kv_heads != 1) return PDA_ERR_INVALID_ARG;
    // (576, 512) and (320, 256): latent 512 or 256 + rope 64
    if (!((s->head_dim == 576 && s->head_dim_v == 512) ||
          (s->head_dim == 320 && s->head_dim_v == 256)))
      return PDA_ERR_UNSUPPORTED;
    if (s->head_dim != 576 && s->variant == PDA_MLA_VALU) return PDA_ERR_UNSUPPORTED;
    if (s->q_dtype != PDA_BF16 || (s->kv_dtype != PDA_BF16 && s->kv_dtype != PDA_FP8_E4M3))
      return PDA_ERR_UNSUPPORTED;
    if (s->kv_dtype == PDA_FP8_E4M3 && !(s->k_scale > 0.f)) return PDA_ERR_INVALID_ARG;
    if (s->page_size % 64 != 0 || (s->page_size & (s->page_size - 1)) != 0)
      return PDA_ERR_UNSUPPORTED;
    if (s->num_q_heads > 16 && s->num_q_heads % 16 != 0) return PDA_ERR_UNSUPPORTED;
    if (s->variant < PDA_MLA_DEFAULT || s->variant > PDA_MLA_MFMA_QM) return PDA_ERR_INVALID_ARG;
    // several query tokens: the matrix-core kernel only
    if (query_len(s) > 1 && s->variant == PDA_MLA_VALU) return PDA_ERR_UNSUPPORTED;
  } else {
    if (!pda::gqa_supported(s->q_dtype, s->kv_dtype, s->head_dim, s->head_dim_v))
      return PDA_ERR_UNSUPPORTED;
    if (s->variant < PDA_GQA_DEFAULT || s->variant > PDA_GQA_MFMA_1WAVE) return PDA_ERR_INVALID_ARG;
    if (s->variant != PDA_GQA_DEFAULT && s->variant != PDA_GQA_VALU &&
        !pda::gqa_mfma_supported(s->q_dtype, s->kv_dtype, s->head_dim))
      return PDA_ERR_UNSUPPORTED;
    // several query tokens: the matrix-core kernel only
    if (query_len(s) > 1 &&
        (s->variant == PDA_GQA_VALU || !pda::gqa_mfma_supported(s->q_dtype, s->kv_dtype, s->head_dim)))
      return PDA_ERR_UNSUPPORTED;
    if (s->page_size % pda::kTileTokens != 0 || (s->page_size & (s->page_size - 1)) != 0)
      return PDA_ERR_UNSUPPORTED;
    if (s->kv_dtype == PDA_FP8_E4M3 && !(s->k_scale > 0.f && s->v_scale > 0.f))
      return PDA_ERR_INVALID_ARG;
    // per-tile buffer ranges are 32-bit: 16 token rows of every KV head
    const int64_t elem = s->kv_dtype == PDA_F32 ? 4 : s->kv_dtype == PDA_FP8_E4M3 ? 1 : 2;
    if ((int64_t)pda::kTileTokens * s->num_kv_heads * s->head_dim * elem > INT32_MAX)
      return PDA_ERR_UNSUPPORTED;
    // the head stride of head-major pages (P * d elements) is 32-bit
    if ((int64_t)s->page_size * s->head_dim > INT32_MAX) return PDA_ERR_UNSUPPORTED;
  }
  return PDA_OK;
}

// Smallest chunk of the balanced schedule, in pages.
constexpr int kMinChunkPages = 16;

// One-wave GQA workgroups the split planner aims at per compute unit.
constexpr int kOneWaveUnitsPerCu = 2;

// Whether a call that may give each work unit to one wave of the matrix-core
// GQA kernel does so by default (units: (sequence, KV head, head tile)
// units before splitting).  Measured on MI355X (us per step, one wave against
// four): B=64 Hq=32 Hkv=8 d=128 fp16 at 128..4096 tokens 8.1 / 8.6 ..
// 158.0 / 164.3, token-major pages at 1024 tokens 41.1 / 44.3, bfloat16 44.4 /
// 44.9, d=256 45.9 / 47.1, two query tokens 41.2 / 43.6, B=128 at 512 tokens
// 42.5 / 47.8; with splits B=1 at 32768 tokens (64 splits against 32) 26.3 /
// 27.1, B=2 45.1 / 45.8, B=4 equal, B=16 at 8192 tokens 83.7 / 86.2.  A lone
// wave computes its tiles with no other wave of its unit to hide their
// latency: fp8 caches (66.1 / 43.4 at 2048 tokens) and d=64 (62.1 / 44.0)
// stay with four waves, and so do calls whose units fill the compute units
// with four-wave workgroups but not with two one-wave ones per unit of work
// (B=32 at 4096 tokens: one wave would split, 83.7 against 80.0).  With an
// explicit split count (num_splits > 0) one wave needs two units per compute
// unit after splitting (B=1 with 32 splits: 39.5 against 27.1).  Several
// head tiles per KV group count as units (B=64, G=8, three query tokens at
// 1024 tokens, two 16-row tiles: 48.1 against 67.3 us).  Two column tiles
// (32 rows per unit) double a wave's arithmetic per tile and keep four waves
// (MQA, B=64, 32 heads, 8192 tokens, 8 splits: 53.2 against 51.0 us).
bool one_wave_default(const pda_shape* s, int64_t units, int col_tiles, int num_splits,
                      int num_cus) {
  const bool wide16 = (s->kv_dtype == PDA_F16 || s->kv_dtype == PDA_BF16) && s->head_dim >= 128;
  const int64_t fill = (int64_t)kOneWaveUnitsPerCu * num_cus;
  if (!wide16 || col_tiles > 1) return false;
  if (num_splits > 0) return units * std::min(num_splits, s->max_pages_per_seq) >= fill;
  return units >= fill || units < num_cus;
}

// Smallest group size for which the default GQA variant takes the matrix-core
// kernel (its 16 head columns are mostly padding below that).
constexpr int kMfmaMinGroup = 3;

// Whether a (validated) GQA call runs the matrix-core kernel (its columns
// are the q_len * group rows of a KV group).
bool gqa_use_mfma(const pda_shape* s) {
  if (s->variant == PDA_GQA_VALU) return false;
  if (s->variant != PDA_GQA_DEFAULT || query_len(s) > 1) return true;
  return pda::gqa_mfma_supported(s->q_dtype, s->kv_dtype, s->head_dim) &&
         s->num_q_heads / s->num_kv_heads >= kMfmaMinGroup;
}

// The plan of a call: the public summary plus what only the library uses.
struct Plan {
  pda_plan_info info;  // (info.waves_per_unit: 1 selects the one-wave GQA kernel)
  int32_t unit_capacity;  // ordered calls: length of the work-unit list
  int32_t target_units;   // balanced schedule: chunks per KV head and head tile
};

// Balanced schedules split a sequence at most this many times (the unit list
// and the grid are bounded by batch + target units either way).
constexpr int kBalancedMaxSplits = 64;

int plan_impl(const pda_shape* s, bool mla, int num_splits, int num_cus, Plan* plan) {
  if (!plan || num_splits < 0 || num_cus < 0) return PDA_ERR_INVALID_ARG;
  pda_plan_info* p = &plan->info;
  int rc = check_shape(s, mla);
  if (rc != PDA_OK) return rc;
  const int group = s->num_q_heads / s->num_kv_heads;
  const int ql = query_len(s);
  // MLA matrix-core tiles hold 16 rows per column group (two groups in a
  // 512-thread workgroup, which then runs one per compute unit)
  const int mla_groups =
      mla && s->variant != PDA_MLA_VALU ? pda::mla_column_groups(ql * s->num_q_heads) : 1;
  const bool mfma_gqa = !mla && gqa_use_mfma(s);
  const int col_tiles = mfma_gqa ? pda::gqa_mfma_col_tiles(ql * group, s->head_dim,
                                                           (int64_t)s->max_pages_per_seq *
                                                               s->page_size)
                                 : 1;
  const int head_tiles = mla      ? (int)ceil_div(ql * s->num_q_heads, 16 * mla_groups)
                         : mfma_gqa ? (int)ceil_div(ql * group, 16 * col_tiles)
                                    : (int)ceil_div(group, pda::gqa_tile_heads(group));
  const int64_t units = (int64_t)s->batch * s->num_kv_heads * head_tiles;
  const int max_pages = s->max_pages_per_seq;
  const bool balanced = s->schedule == PDA_SCHEDULE_BALANCED;
  // Eight waves per compute unit (two four-wave workgroups, or one of eight)
  const int wg_per_cu = mla_groups == 2 ? 1 : 2;
  // The matrix-core GQA kernel can give each work unit to one wave
  // (workgroups of one wave, no merge) on the GRID schedule without a
  // threshold (no ordered work).
  const bool one_wave_ok = mfma_gqa && !balanced && s->split_min_tokens == 0;
  if (s->variant == PDA_GQA_MFMA_1WAVE && !mla && !one_wave_ok) return PDA_ERR_UNSUPPORTED;
  // (the default choice needs the compute units; with an explicit split
  // count and no device to ask, the call keeps four waves)
  int wave_cus = num_cus;
  if (one_wave_ok && s->variant != PDA_GQA_MFMA_1WAVE && s->variant != PDA_GQA_MFMA_4WAVE &&
      wave_cus == 0)
    wave_cus = device_cus();
  const bool one_wave =
      !mla && one_wave_ok &&
      (s->variant == PDA_GQA_MFMA_1WAVE ||
       (s->variant != PDA_GQA_MFMA_4WAVE && wave_cus > 0 &&
        one_wave_default(s, units, col_tiles, num_splits, wave_cus)));

  if ((num_splits == 0 || balanced) && num_cus == 0) {
    num_cus = device_cus();
    if (num_cus <= 0) return PDA_ERR_HIP;
  }
  int splits = 1;
  if (num_splits > 0) {
    splits = std::min(num_splits, max_pages);
    if (balanced) splits = std::min(splits, kBalancedMaxSplits);
  } else if (balanced) {
    // at most as many splits as units per KV head and head tile fill the
    // GPU, and no more than chunks of the smallest size fit a table row
    splits = (int)std::min<int64_t>(
        std::max<int64_t>(1, (int64_t)wg_per_cu * num_cus / (s->num_kv_heads * head_tiles)),
        std::min<int64_t>(ceil_div(max_pages, kMinChunkPages), kBalancedMaxSplits));
  } else {
    // split only when the (sequence, head tile) units alone cannot fill the
    // compute units.  The matrix-core GQA kernel with one column tile fills
    // one workgroup per CU: at 32768 tokens that measured 0-6% faster than
    // two at every batch from 1 to 32 in both page layouts (B=8: 161 against
    // 168-170 us, B=32 with no split: 624-626 against 645-663 us).  Two
    // column tiles (MQA) carry twice the arithmetic per tile and keep two
    // workgroups per CU (4 splits against 8 at B=64 measured from equal to
    // 2 us slower).
    // One-wave workgroups fill two per compute unit.
    const int fill_per_cu = one_wave ? kOneWaveUnitsPerCu
                            : (mfma_gqa && col_tiles == 1) ? 1 : wg_per_cu;
    const int64_t target = fill_per_cu * (int64_t)num_cus;
    if (units > 0 && units < target)
      splits = (int)std::min<int64_t>(ceil_div(target, units), max_pages);
  }
  // No sequence longer than the threshold fits the table: nothing splits.
  if ((int64_t)max_pages * s->page_size <= s->split_min_tokens) splits = 1;
  splits = std::min(splits, 65535);  // grid y extent
  int pps = (int)ceil_div(max_pages, splits);
  splits = (int)ceil_div(max_pages, pps);

  p->max_splits = splits;
  p->pages_per_split = balanced ? 0 : pps;
  p->waves_per_unit = one_wave ? 1 : mla ? 4 * mla_groups : mfma_gqa ? 4 : pda::kGqaWaves;
  p->reserved = 0;
  p->head_tiles = head_tiles;
  p->num_cus = num_cus;
  // The balanced schedule aims at twice the (sequence, split) units that fill
  // the compute units (per KV head and head tile), so that the longest-first
  // order can even out the units' different sizes; its units number at most
  // B + target (each sequence adds at most pages / chunk splits beyond its
  // first, and the chunk is at least total pages / target).
  const int64_t fill = std::max<int64_t>(1, (int64_t)wg_per_cu * num_cus /
                                                (s->num_kv_heads * head_tiles));
  plan->target_units = (int)std::min<int64_t>(2 * fill, 1 << 20);
  int64_t ucap = (int64_t)s->batch * splits;
  if (balanced) ucap = std::min<int64_t>(ucap, (int64_t)s->batch + plan->target_units);
  // work ordering for mixed-length batches (the threshold signals them) and
  // for the balanced schedule
  p->ordered = (s->split_min_tokens > 0 || balanced) &&
               ucap * s->num_kv_heads * head_tiles <= INT32_MAX;
  // a balanced schedule exists only as ordered work (its split sizes are
  // chosen on the device)
  if (balanced && !p->ordered) return PDA_ERR_UNSUPPORTED;
  plan->unit_capacity = p->ordered ? (int32_t)ucap : 0;
  p->workgroups = (int)std::min<int64_t>(
      p->ordered ? ucap * s->num_kv_heads * head_tiles : units * splits, INT32_MAX);
  uint64_t ws = 0;
  if (splits > 1) {
    const uint64_t rows = (uint64_t)s->batch * ql * s->num_q_heads;
    const uint64_t o_bytes = rows * splits * s->head_dim_v * sizeof(float);
    ws = ((o_bytes + 255) / 256) * 256 + ((rows * splits * sizeof(float) + 255) / 256) * 256;
  }
  if (p->ordered)
    ws += (((uint64_t)ucap * 4 * sizeof(int32_t) + 255) / 256) * 256 +
          (uint64_t)s->batch * sizeof(int32_t);
  p->workspace_bytes = ws;
  return PDA_OK;
}

// Workspace layout: partial outputs [B, q_len, Hq, S, dv] fp32, partial LSE
// [B, q_len, Hq, S] fp32 (both only when S > 1), then for ordered calls the
// work units [units][4] int32 and the split count of each sequence [B]
// int32; every part starts 256-byte aligned.
void workspace_parts(const pda_shape* s, const Plan& plan, void* ws, float** po, float** pl,
                     int32_t** un, int32_t** ss) {
  const pda_plan_info& p = plan.info;
  const uint64_t rows = (uint64_t)s->batch * query_len(s) * s->num_q_heads;
  char* c = (char*)ws;
  *po = nullptr;
  *pl = nullptr;
  *un = nullptr;
  *ss = nullptr;
  if (p.max_splits > 1) {
    const uint64_t o_bytes = rows * p.max_splits * s->head_dim_v * sizeof(float);
    *po = (float*)c;
    c += ((o_bytes + 255) / 256) * 256;
    *pl = (float*)c;
    c += ((rows * p.max_splits * sizeof(float) + 255) / 256) * 256;
  }
  if (p.ordered) {
    *un = (int32_t*)c;
    c += (((uint64_t)plan.unit_capacity * 4 * sizeof(int32_t) + 255) / 256) * 256;
    *ss = (int32_t*)c;
  }
}

// The planning pass of an ordered call (before the attention kernel).
int run_order(const pda_shape& s, const Plan& plan, const int32_t* context_lens, int32_t* units,
              int32_t* seq_splits, const pda::SplitLayout& sp, hipStream_t st) {
  pda::OrderArgs o{};
  o.context_lens = context_lens;
  o.units = units;
  o.seq_splits = seq_splits;
  o.capacity = plan.unit_capacity;
  o.batch = s.batch;
  o.page_size = s.page_size;
  o.balanced = s.schedule == PDA_SCHEDULE_BALANCED;
  o.target_units = plan.target_units;
  o.min_chunk_pages = kMinChunkPages;
  o.split = sp;
  return pda::launch_order(o, st) == hipSuccess ? PDA_OK : PDA_ERR_HIP;
}

}  // namespace

extern "C" {

int pda_check_inputs(const pda_shape* shape, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* positions, int32_t* result,
                     void* stream) {
  if (!shape || !result) return PDA_ERR_INVALID_ARG;
  const pda_shape& s = *shape;
  if (s.batch < 0 || s.page_size <= 0 || s.max_pages_per_seq <= 0 || s.num_pages <= 0 ||
      s.q_len < 0)
    return PDA_ERR_INVALID_ARG;
  if (s.batch > 0 && (!block_tables || !context_lens)) return PDA_ERR_INVALID_ARG;
  if ((int64_t)s.max_pages_per_seq * s.page_size > INT32_MAX) return PDA_ERR_INVALID_ARG;
  pda::CheckArgs a{};
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.positions = s.batch > 0 ? positions : nullptr;
  a.result = result;
  a.batch = s.batch;
  a.max_pages = s.max_pages_per_seq;
  a.page_size = s.page_size;
  a.num_pages = s.num_pages;
  a.s_new = query_len(shape);
  return pda::launch_check(a, (hipStream_t)stream) == hipSuccess ? PDA_OK : PDA_ERR_HIP;
}

int pda_stream_probe(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, const pda_shape* shape, int num_splits,
                     int steps_in_flight, uint32_t* sink, void* stream) {
  if (!k_cache || !v_cache || !block_tables || !context_lens || !sink || !shape)
    return PDA_ERR_INVALID_ARG;
  if (steps_in_flight < 1 || steps_in_flight > 4 || num_splits < 0) return PDA_ERR_INVALID_ARG;
  int rc = check_shape(shape, false);
  if (rc != PDA_OK) return rc;
  const pda_shape& s = *shape;
  if (s.schedule != PDA_SCHEDULE_GRID) return PDA_ERR_UNSUPPORTED;
  if (s.head_dim != s.head_dim_v) return PDA_ERR_UNSUPPORTED;
  const int elem = s.kv_dtype == PDA_F32 ? 4 : s.kv_dtype == PDA_FP8_E4M3 ? 1 : 2;
  const int row_bytes = s.head_dim * elem;
  if (row_bytes != 64 && row_bytes != 128 && row_bytes != 256 && row_bytes != 512)
    return PDA_ERR_UNSUPPORTED;
  if (s.batch == 0) return PDA_OK;
  // the split layout and wave layout the call itself would take (the probe
  // reads each KV head's rows once per split, whatever its head tiles)
  Plan plan;
  rc = plan_impl(&s, false, num_splits, 0, &plan);
  if (rc != PDA_OK) return rc;
  pda::ProbeArgs a{};
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.sink = sink;
  a.batch = s.batch;
  a.num_kv_heads = s.num_kv_heads;
  a.page_size = s.page_size;
  a.max_pages = s.max_pages_per_seq;
  a.log2_page = 0;
  while ((1 << a.log2_page) < s.page_size) ++a.log2_page;
  a.elem_bytes = elem;
  const bool head_major = s.kv_layout == PDA_KV_HEAD_MAJOR;
  a.tok_stride = head_major ? s.head_dim : s.num_kv_heads * s.head_dim;
  a.head_stride = head_major ? s.page_size * s.head_dim : s.head_dim;
  a.page_stride = (int64_t)s.page_size * s.num_kv_heads * s.head_dim;
  a.split.pages_per_split = plan.info.pages_per_split;
  a.split.max_splits = plan.info.max_splits;
  a.split.split_min_tokens = s.split_min_tokens;
  return pda::launch_probe(a, row_bytes, plan.info.max_splits, steps_in_flight,
                           plan.info.waves_per_unit == 1 ? 1 : 4, (hipStream_t)stream) == hipSuccess
             ? PDA_OK
             : PDA_ERR_HIP;
}

int pda_version(void) { return 400; }

const char* pda_status_string(int status) {
  switch (status) {
    case PDA_OK: return "ok";
    case PDA_ERR_INVALID_ARG: return "invalid argument";
    case PDA_ERR_UNSUPPORTED: return "unsupported configuration";
    case PDA_ERR_WORKSPACE: return "workspace missing or too small";
    case PDA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int pda_plan(const pda_shape* shape, int is_mla, int num_splits, int num_cus,
             pda_plan_info* plan) {
  if (!plan) return PDA_ERR_INVALID_ARG;
  Plan p;
  const int rc = plan_impl(shape, is_mla != 0, num_splits, num_cus, &p);
  if (rc == PDA_OK) *plan = p.info;
  return rc;
}

size_t pda_workspace_bytes(const pda_shape* shape, int is_mla, int num_splits) {
  Plan p;
  if (plan_impl(shape, is_mla != 0, num_splits, 0, &p) != PDA_OK) return 0;
  return (size_t)p.info.workspace_bytes;
}

int paged_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int group,
                      float scale, int num_splits, void* out, float* lse,
                      const pda_shape* shape, void* workspace, size_t workspace_bytes,
                      void* stream) {
  if (!q || !k_cache || !v_cache || !block_tables || !context_lens || !out || !shape)
    return PDA_ERR_INVALID_ARG;
  int rc = check_shape(shape, false);
  if (rc != PDA_OK) return rc;
  if (group <= 0 || group * shape->num_kv_heads != shape->num_q_heads) return PDA_ERR_INVALID_ARG;
  if (!(scale == scale) || num_splits < 0) return PDA_ERR_INVALID_ARG;
  if (shape->batch == 0) return PDA_OK;

  Plan plan;
  rc = plan_impl(shape, false, num_splits, 0, &plan);
  if (rc != PDA_OK) return rc;
  const pda_plan_info& p = plan.info;
  if (p.workspace_bytes > 0 && (!workspace || workspace_bytes < p.workspace_bytes))
    return PDA_ERR_WORKSPACE;

  const pda_shape& s = *shape;
  pda::GqaArgs a{};
  a.q = q;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.lse = lse;
  int32_t* units = nullptr;
  int32_t* seq_splits = nullptr;
  workspace_parts(shape, plan, workspace, &a.part_o, &a.part_lse, &units, &seq_splits);
  a.units = units;
  a.unit_count = plan.unit_capacity;
  a.batch = s.batch;
  a.num_q_heads = s.num_q_heads;
  a.num_kv_heads = s.num_kv_heads;
  a.group = group;
  a.head_tiles = p.head_tiles;
  a.q_len = query_len(shape);
  a.causal = shape->causal;
  a.page_size = s.page_size;
  a.max_pages = s.max_pages_per_seq;
  a.log2_page = 0;
  while ((1 << a.log2_page) < s.page_size) ++a.log2_page;
  const bool head_major = s.kv_layout == PDA_KV_HEAD_MAJOR;
  a.tok_stride = head_major ? s.head_dim : s.num_kv_heads * s.head_dim;
  a.head_stride = head_major ? s.page_size * s.head_dim : s.head_dim;
  a.page_stride = (int64_t)s.page_size * s.num_kv_heads * s.head_dim;
  const float ks = s.kv_dtype == PDA_FP8_E4M3 ? s.k_scale : 1.0f;
  a.qk_scale_log2 = scale * ks * 1.4426950408889634f;
  a.v_scale = s.kv_dtype == PDA_FP8_E4M3 ? s.v_scale : 1.0f;
  a.split.pages_per_split = p.pages_per_split;
  a.split.max_splits = p.max_splits;
  a.split.split_min_tokens = s.split_min_tokens;
  a.waves = p.waves_per_unit;

  hipStream_t st = (hipStream_t)stream;
  // BALANCED calls on the matrix-core kernel with a moderate batch: each
  // workgroup derives its unit from the lengths (no planning launch).  Their
  // grid is bounded by batch + target units, close to the real unit count;
  // a GRID schedule with a threshold launches batch x splits workgroups for
  // far fewer units, where the planning kernel's list lets the surplus
  // workgroups leave after one load.
  if (units && s.schedule == PDA_SCHEDULE_BALANCED && gqa_use_mfma(shape) &&
      s.batch <= pda::kInKernelPlanMaxBatch) {
    a.plan_in_kernel = 1;
    a.plan.batch = s.batch;
    a.plan.page_size = s.page_size;
    a.plan.balanced = s.schedule == PDA_SCHEDULE_BALANCED;
    a.plan.target_units = plan.target_units;
    a.plan.min_chunk_pages = kMinChunkPages;
    a.plan.split = a.split;
    a.seq_splits = seq_splits;
    a.units = nullptr;
  } else if (units) {
    rc = run_order(s, plan, context_lens, units, seq_splits, a.split, st);
    if (rc != PDA_OK) return rc;
  }
  const hipError_t le =
      gqa_use_mfma(shape)
          ? pda::launch_gqa_mfma(a, s.q_dtype, s.kv_dtype, s.head_dim, p.max_splits, st)
          : pda::launch_gqa(a, s.q_dtype, s.kv_dtype, s.head_dim, pda::gqa_tile_heads(group),
                            p.max_splits, st);
  if (le != hipSuccess) return PDA_ERR_HIP;
  if (p.max_splits > 1) {
    pda::CombineArgs c{};
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.context_lens = context_lens;
    c.out = out;
    c.lse = lse;
    c.batch = s.batch;
    c.num_q_heads = s.num_q_heads;
    c.q_len = query_len(shape);
    c.head_dim_v = s.head_dim_v;
    c.page_size = s.page_size;
    c.split = a.split;
    c.seq_splits = seq_splits;
    if (pda::launch_combine(c, s.q_dtype, false, st) != hipSuccess) return PDA_ERR_HIP;
  }
  return PDA_OK;
}

int paged_decode_attn_mla(const void* q, const void* kv_cache, const int32_t* block_tables,
                          const int32_t* context_lens, float scale, int num_splits, void* out,
                          float* lse, const pda_shape* shape, void* workspace,
                          size_t workspace_bytes, void* stream) {
  if (!q || !kv_cache || !block_tables || !context_lens || !out || !shape)
    return PDA_ERR_INVALID_ARG;
  int rc = check_shape(shape, true);
  if (rc != PDA_OK) return rc;
  if (!(scale == scale) || num_splits < 0) return PDA_ERR_INVALID_ARG;
  if (shape->batch == 0) return PDA_OK;

  Plan plan;
  rc = plan_impl(shape, true, num_splits, 0, &plan);
  if (rc != PDA_OK) return rc;
  const pda_plan_info& p = plan.info;
  if (p.workspace_bytes > 0 && (!workspace || workspace_bytes < p.workspace_bytes))
    return PDA_ERR_WORKSPACE;

  const pda_shape& s = *shape;
  pda::MlaArgs a{};
  a.q = q;
  a.kv_cache = kv_cache;
  a.block_tables = block_tables;
  a.context_lens = context_lens;
  a.out = out;
  a.lse = lse;
  int32_t* units = nullptr;
  int32_t* seq_splits = nullptr;
  workspace_parts(shape, plan, workspace, &a.part_o, &a.part_lse, &units, &seq_splits);
  a.units = units;
  a.unit_count = plan.unit_capacity;
  a.batch = s.batch;
  a.num_q_heads = s.num_q_heads;
  a.head_tiles = p.head_tiles;
  a.q_len = query_len(shape);
  a.causal = shape->causal;
  a.page_size = s.page_size;
  a.max_pages = s.max_pages_per_seq;
  a.log2_page = 0;
  while ((1 << a.log2_page) < s.page_size) ++a.log2_page;
  // an fp8 latent: K and V are the same dequantized values (one scale)
  const float kvs = s.kv_dtype == PDA_FP8_E4M3 ? s.k_scale : 1.0f;
  a.qk_scale_log2 = scale * kvs * 1.4426950408889634f;
  a.v_scale = kvs;
  a.split.pages_per_split = p.pages_per_split;
  a.split.max_splits = p.max_splits;
  a.split.split_min_tokens = s.split_min_tokens;

  hipStream_t st = (hipStream_t)stream;
  if (units) {
    rc = run_order(s, plan, context_lens, units, seq_splits, a.split, st);
    if (rc != PDA_OK) return rc;
  }
  if (pda::launch_mla(a, s.variant, s.kv_dtype, s.head_dim, p.max_splits, st) != hipSuccess)
    return PDA_ERR_HIP;
  if (p.max_splits > 1) {
    pda::CombineArgs c{};
    c.part_o = a.part_o;
    c.part_lse = a.part_lse;
    c.context_lens = context_lens;
    c.out = out;
    c.lse = lse;
    c.batch = s.batch;
    c.num_q_heads = s.num_q_heads;
    c.q_len = query_len(shape);
    c.head_dim_v = s.head_dim_v;
    c.page_size = s.page_size;
    c.split = a.split;
    c.seq_splits = seq_splits;
    if (pda::launch_combine(c, s.q_dtype, true, st) != hipSuccess) return PDA_ERR_HIP;
  }
  return PDA_OK;
}

int paged_kv_append(const void* k_new, const void* v_new, const int32_t* block_tables,
                    const int32_t* positions, void* k_cache, void* v_cache,
                    const pda_shape* shape, void* stream) {
  if (!shape || !k_new || !k_cache || !block_tables || !positions) return PDA_ERR_INVALID_ARG;
  const bool has_v = v_cache != nullptr;
  if ((v_new != nullptr) != has_v) return PDA_ERR_INVALID_ARG;
  const pda_shape& s = *shape;
  if (s.batch < 0 || s.num_kv_heads <= 0 || s.head_dim <= 0 || s.page_size <= 0 ||
      s.max_pages_per_seq <= 0 || s.num_pages <= 0 || s.q_len < 0 ||
      (has_v && s.head_dim_v <= 0) ||
      (s.kv_layout != PDA_KV_TOKEN_MAJOR && s.kv_layout != PDA_KV_HEAD_MAJOR))
    return PDA_ERR_INVALID_ARG;
  if (!valid_dtype(s.q_dtype) || !valid_dtype(s.kv_dtype)) return PDA_ERR_INVALID_ARG;
  if ((int64_t)s.max_pages_per_seq * s.page_size > INT32_MAX) return PDA_ERR_INVALID_ARG;
  if (!pda::append_supported(s.q_dtype, s.kv_dtype)) return PDA_ERR_UNSUPPORTED;
  if (s.head_dim % 8 != 0 || (has_v && s.head_dim_v % 8 != 0)) return PDA_ERR_UNSUPPORTED;
  if (s.kv_dtype == PDA_FP8_E4M3 && !(s.k_scale > 0.f && (!has_v || s.v_scale > 0.f)))
    return PDA_ERR_INVALID_ARG;
  // rows move in 16-byte pieces
  for (const void* ptr : {k_new, v_new, (const void*)k_cache, (const void*)v_cache})
    if ((uintptr_t)ptr % 16 != 0) return PDA_ERR_INVALID_ARG;
  if (s.batch == 0) return PDA_OK;

  pda::AppendArgs a{};
  a.k_new = k_new;
  a.v_new = v_new;
  a.k_cache = k_cache;
  a.v_cache = v_cache;
  a.block_tables = block_tables;
  a.positions = positions;
  a.batch = s.batch;
  a.s_new = query_len(shape);
  a.num_kv_heads = s.num_kv_heads;
  a.head_dim = s.head_dim;
  a.head_dim_v = has_v ? s.head_dim_v : 0;
  a.page_size = s.page_size;
  a.max_pages = s.max_pages_per_seq;
  a.head_major = s.kv_layout == PDA_KV_HEAD_MAJOR && s.num_kv_heads > 1;
  a.k_scale = s.k_scale;
  a.v_scale = s.v_scale;
  return pda::launch_append(a, s.q_dtype, s.kv_dtype, (hipStream_t)stream) == hipSuccess
             ? PDA_OK
             : PDA_ERR_HIP;
}

}  // extern "C"
