/*
 * pda.h -- C ABI of libpda: single-token decode attention over a paged KV
 * cache on MI355X (gfx950).
 *
 * The operation (pages: "From MHA to MLA: KV Caches and Attention Kernels",
 * sec. 2-6; "GPU kernel drills" L2 paged-decode page, sec. 2-5; FlashMLA-ETAP
 * README, "Usage"):
 *
 *   for each sequence b < B and query head h < Hq, with G = Hq / Hkv and the
 *   KV head kvh = floor(h / G) (contiguous grouping),
 *     K_j = k_cache[block_tables[b][j / P], j % P, kvh, :] * k_scale
 *     V_j = v_cache[block_tables[b][j / P], j % P, kvh, :] * v_scale
 *     s_j = scale * q[b, h, :] . K_j                   for j < context_lens[b]
 *     out[b, h, :] = sum_j softmax(s)_j V_j
 *     lse[b, h]    = ln sum_j exp(s_j)                 (natural log, fp32)
 *
 *   MLA ("From MHA to MLA" sec. 6, "Attention Kernel Variants" MLA section):
 *   one latent record per token [c (512) | k_R (64)] shared by all query
 *   heads; K_j = the 576-wide record, V_j = its first 512 values.
 *
 *   Several query tokens per sequence (multi-token decode, e.g. speculative
 *   or MTP drafts: FlashMLA-ETAP README, "Supported configurations" and
 *   "Usage"): with shape->q_len = s_q > 1 the s_q queries of sequence b are
 *   its last s_q tokens, query i at position n - s_q + i.  With the causal
 *   mask aligned bottom-right ("From MHA to MLA" sec. 2, the reference
 *   kernel's causal branch) query i attends to the first n - (s_q - 1 - i)
 *   tokens; without it every query attends to all n.  A query that sees no
 *   token gets out = 0 and lse = -inf.
 *
 * Long sequences may be cut into page-aligned splits (Flash-Decoding,
 * "From MHA to MLA" sec. 4); each split writes a normalized partial output
 * and its LSE to the workspace and a combine pass merges them with weights
 * exp(L_s - L).  The result does not depend on the split count beyond
 * floating-point rounding.
 *
 * Conventions shared by every entry point:
 *  - Pointers named *_cache, q, out, lse, block_tables, context_lens and
 *    workspace are DEVICE pointers owned by the caller; the library neither
 *    allocates nor retains memory.  `shape` and `plan` are HOST pointers.
 *  - All arrays are dense row-major with the last dimension contiguous
 *    (s_q = shape->q_len; for s_q = 1 the layouts below are [B, Hq, ...]):
 *      q            [B, s_q, Hq, head_dim]     of shape->q_dtype
 *      k_cache      [num_pages, P, Hkv, head_dim]   of shape->kv_dtype
 *                   ([num_pages, Hkv, P, head_dim] with PDA_KV_HEAD_MAJOR)
 *      v_cache      [num_pages, P, Hkv, head_dim_v] of shape->kv_dtype
 *                   ([num_pages, Hkv, P, head_dim_v] with PDA_KV_HEAD_MAJOR)
 *      kv_cache     [num_pages, P, head_dim]   (MLA, K and V share it)
 *      block_tables [B, max_pages_per_seq] int32 (logical -> physical page)
 *      context_lens [B] int32, the number of cached tokens of each sequence
 *      out          [B, s_q, Hq, head_dim_v]   of shape->q_dtype
 *      lse          [B, Hq, s_q] float32, may be NULL
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls are
 *    asynchronous on that stream and never synchronize.  Calls that share a
 *    workspace must be ordered on one stream.
 *  - Errors are returned as pda_status codes; nothing aborts or throws.
 *    Host-checkable arguments are validated before any device work:
 *    NULL pointers, head/group divisibility, supported (dtype, head_dim,
 *    page_size) combinations, num_splits >= 0, workspace size.
 *  - Device-resident values are PRECONDITIONS, not checked: 0 <=
 *    context_lens[b] <= max_pages_per_seq * P, and the first
 *    ceil(context_lens[b] / P) entries of block_tables[b] lie in
 *    [0, num_pages).  Entries past those may be loaded (the table row
 *    is read in blocks) but never address the cache, whatever they hold;
 *    cache slots past context_lens[b] in the last page are never read.
 *    context_lens[b] == 0 gives out = 0 and lse = -inf for that sequence.
 */
#ifndef PDA_H
#define PDA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element types.  PDA_FP8_E4M3 is OCP FP8 E4M3FN (bias 7, max 448, no
 * infinities), stored one byte per element, dequantized as
 * value = e4m3(byte) * scale with one fp32 scale per cache tensor. */
typedef enum pda_dtype {
  PDA_F32 = 0,
  PDA_F16 = 1,
  PDA_BF16 = 2,
  PDA_FP8_E4M3 = 3
} pda_dtype;

typedef enum pda_status {
  PDA_OK = 0,
  PDA_ERR_INVALID_ARG = 1, /* NULL pointer, bad size, Hq % Hkv != 0, ...    */
  PDA_ERR_UNSUPPORTED = 2, /* no kernel for this dtype / head_dim / page    */
  PDA_ERR_WORKSPACE = 3,   /* workspace NULL or smaller than required       */
  PDA_ERR_HIP = 4          /* a HIP runtime call failed (launch, attribute) */
} pda_status;

/* Problem description, passed by host pointer. */
typedef struct pda_shape {
  int32_t batch;             /* B                                          */
  int32_t num_q_heads;       /* Hq                                         */
  int32_t num_kv_heads;      /* Hkv (1 for MLA)                            */
  int32_t head_dim;          /* width of q and K rows (576 for MLA)        */
  int32_t head_dim_v;        /* width of V rows and of out (512 for MLA)   */
  int32_t page_size;         /* P, tokens per page                         */
  int32_t max_pages_per_seq; /* columns of block_tables                    */
  int32_t num_pages;         /* pages in the pool                          */
  int32_t q_dtype;           /* pda_dtype of q and out                     */
  int32_t kv_dtype;          /* pda_dtype of the cache                     */
  float k_scale;             /* K dequant scale (1.0f unless FP8)          */
  float v_scale;             /* V dequant scale (1.0f unless FP8)          */
  int32_t split_min_tokens;  /* sequences with context_lens[b] <= this are */
                             /* never split (0: any sequence may split)    */
  int32_t variant;           /* kernel variant, 0 = default (see below)    */
  int32_t q_len;             /* s_q, query tokens per sequence (0 means 1;  */
                             /* q_len * num_q_heads at most 2^20)          */
  int32_t causal;            /* s_q > 1: 1 = bottom-right causal mask,      */
                             /* 0 = every query sees all n tokens           */
  int32_t schedule;          /* PDA_SCHEDULE_* (below)                       */
  int32_t kv_layout;         /* PDA_KV_* (below): axis order inside a page   */
} pda_shape;

/* Order of a cache page's axes (pda_shape.kv_layout).  The pages address a
 * cached element through separate page, slot and head strides ("From MHA
 * to MLA" sec. 5, paged loads; the drill page sec. 4, the page loop), so
 * both orders describe the same cache:
 * TOKEN_MAJOR: k_cache [num_pages, P, Hkv, head_dim] (a token's KV heads are
 *   adjacent);
 * HEAD_MAJOR:  k_cache [num_pages, Hkv, P, head_dim] (one KV head's P rows
 *   of a page are one contiguous block, so a workgroup that serves one KV
 *   head reads whole blocks); likewise v_cache with head_dim_v.
 * With Hkv = 1 (MLA) the two orders coincide. */
#define PDA_KV_TOKEN_MAJOR 0
#define PDA_KV_HEAD_MAJOR 1

/* How a call cuts sequences into splits (pda_shape.schedule).
 * GRID: every sequence longer than split_min_tokens takes ceil(pages /
 *   pages_per_split) splits of one common size (pda_plan_info); with
 *   split_min_tokens > 0 the work units are listed longest first.
 * BALANCED: a device-side planning pass, run at the start of each call
 *   from context_lens, cuts the batch's total pages into near-equal chunks
 *   of max(16, ceil(total pages / units)) pages, where units is the number
 *   of (sequence, split) units per KV head and head tile that fill the
 *   compute units (two workgroups per CU).  A sequence longer than a chunk
 *   and than split_min_tokens takes ceil(pages / chunk) splits (at most the
 *   planned max_splits) of equal size; the units are listed longest first.
 *   Short sequences stay whole, so a batch of mixed lengths becomes units of
 *   at most one chunk each (load balance across the compute units). */
#define PDA_SCHEDULE_GRID 0
#define PDA_SCHEDULE_BALANCED 1

/* GQA kernel variants (pda_shape.variant for paged_decode_attn). */
#define PDA_GQA_DEFAULT 0 /* matrix cores when available and the group has   */
                          /* at least 3 query heads, else vector ALUs       */
#define PDA_GQA_MFMA 1    /* matrix cores (F16/BF16 queries only)           */
#define PDA_GQA_VALU 2    /* vector dot products                            */
#define PDA_GQA_MFMA_4WAVE 3 /* matrix cores, four waves per work unit        */
#define PDA_GQA_MFMA_1WAVE 4 /* matrix cores, one wave per work unit (GRID    */
                             /* schedule without a split threshold; else     */
                             /* PDA_ERR_UNSUPPORTED)                         */

/* MLA kernel variants (pda_shape.variant for paged_decode_attn_mla). */
#define PDA_MLA_DEFAULT 0 /* the fastest available                          */
#define PDA_MLA_MFMA 1    /* bf16 matrix cores, keys on the M dimension     */
#define PDA_MLA_VALU 2    /* plain vector dot products (reference path)     */
#define PDA_MLA_MFMA_QM 3 /* bf16 matrix cores, queries on the M dimension  */

/* What the planner chose for a call (host struct). */
typedef struct pda_plan_info {
  int32_t max_splits;      /* split-axis extent of the launch grid          */
  int32_t pages_per_split; /* pages per split for sequences that split      */
                           /* (GRID; 0 with BALANCED: chosen on the device) */
  int32_t head_tiles;      /* query-head tiles per KV head (workgroups per   */
                           /* KV head and split: 8 heads a tile for the     */
                           /* vector kernel, 16 or 32 (query, head) rows    */
                           /* for the matrix-core kernels)                  */
  int32_t workgroups;      /* workgroups of the main kernel                  */
  int32_t num_cus;         /* compute units the plan was made for           */
  int32_t ordered;         /* 1: the call orders its work longest first     */
  uint64_t workspace_bytes; /* bytes the call needs in `workspace`          */
  int32_t waves_per_unit;  /* waves of a main-kernel workgroup, which share */
                           /* one work unit: 1 (the matrix-core GQA kernel  */
                           /* with a unit per wave), 4, or 8 (MLA with two  */
                           /* column groups)                                */
  int32_t reserved;
} pda_plan_info;

/* Choose the split layout for a call (host only, no device work).  The pages
 * leave the split count to the caller and its heuristic: "From MHA to MLA"
 * sec. 4 (the closing paragraph) chooses num_splits from the batch size, the
 * head tiles, the context length and the number of SMs, splitting only when
 * the (sequence, head) work alone leaves compute units idle; the drill page
 * sec. 6 shows the cost of not splitting at batch 1.  This planner splits
 * until the grid fills one workgroup per compute unit for the matrix-core
 * GQA kernel with 16-row tiles, and two for its 32-row tiles, the vector
 * kernel and MLA (one of MLA's 512-thread workgroups).  The matrix-core GQA
 * kernel gives each work unit to one wave instead of four (waves_per_unit
 * 1, two units per compute unit) for GRID calls without a threshold on
 * 16-bit caches with head_dim >= 128 and 16-row tiles when the units fill
 * two per compute unit unsplit, or less than one (then split to two per
 * compute unit); with an explicit num_splits, when the split units fill two
 * per compute unit.  PDA_GQA_MFMA_1WAVE and
 * PDA_GQA_MFMA_4WAVE fix the choice.  That choice needs the compute units:
 * with an explicit num_splits and num_cus = 0 the device is asked, and when
 * it cannot answer the call keeps four waves.
 * num_splits: 0 = automatic (fill the GPU's compute units), otherwise the
 * largest number of splits any sequence may use (at most 64 with the BALANCED
 * schedule).  num_cus: compute units to plan for; 0 = query the current HIP
 * device.  Sequences longer than shape->split_min_tokens use ceil(pages /
 * pages_per_split) splits, others one.  is_mla selects the MLA kernel's
 * tiling.  Returns PDA_OK or an error code (PDA_ERR_UNSUPPORTED when a
 * BALANCED call's unit list would exceed 32-bit grid indexing). */
int pda_plan(const pda_shape* shape, int is_mla, int num_splits, int num_cus,
             pda_plan_info* plan);

/* Workspace bytes a call with these arguments needs (0 when no sequence can
 * split and the work is not ordered): the split partials of "From MHA to MLA"
 * sec. 4 (an output row and an fp32 LSE per split and query row) and the
 * ordered work list.  The output rows are fp32 for GQA calls; MLA calls,
 * whose output is bfloat16, store them as binary16 in the first half of the
 * same fp32-sized area.  Queries the current device's CU count when
 * num_splits == 0 or the schedule is BALANCED.  Returns 0 on invalid
 * arguments as well.  The workspace needs no initialization: every call
 * writes what it reads.
 *
 * Work ordering: when shape->split_min_tokens > 0 (a batch of mixed lengths,
 * as the threshold signals) or the schedule is BALANCED, each call first
 * runs one small planning kernel that lists the (sequence, split) work
 * units, with their token ranges, by decreasing token count (in the
 * workspace), and the attention workgroups take units in that order, so the
 * longest units start first (longest-processing-time order; the pages do not
 * prescribe a schedule).  The result does not depend on the order. */
size_t pda_workspace_bytes(const pda_shape* shape, int is_mla, int num_splits);

/* GQA / MQA / MHA paged decode attention (layouts above; the caches' page
 * order is shape->kv_layout's).
 * group must equal num_q_heads / num_kv_heads.  scale multiplies q.K before
 * the softmax (k_scale/v_scale are applied on top for FP8 caches).
 * Supported: (q, kv) dtypes (F32,F32), (F16,F16), (BF16,BF16), (F16,FP8),
 * (BF16,FP8); head_dim == head_dim_v in {64, 128, 256} (256 not for F32);
 * page_size a power of two, at least 16.  q_len > 1 needs F16 or BF16
 * queries and a variant other than PDA_GQA_VALU (the matrix-core kernel,
 * whose columns are the q_len * group (query, head) rows of a KV group).
 * workspace: at least pda_workspace_bytes(shape, 0, num_splits) bytes, may
 * be NULL when that is 0.  Calls that share a workspace must not overlap
 * (order them on one stream). */
int paged_decode_attn(const void* q, const void* k_cache, const void* v_cache,
                      const int32_t* block_tables, const int32_t* context_lens, int group,
                      float scale, int num_splits, void* out, float* lse,
                      const pda_shape* shape, void* workspace, size_t workspace_bytes,
                      void* stream);

/* paged_decode_attn for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, hosts that forbid hipMalloc):
 * the same arguments without the workspace.  The call's workspace (split
 * partials, the ordered work list) lives in a device array that the library
 * holds on each GPU it runs on until the process ends: 64 MiB
 * (67,108,864 bytes) per GPU.  A call whose plan needs more
 * (pda_plan_info.workspace_bytes) returns PDA_ERR_WORKSPACE before any
 * device work.  The call allocates nothing; its first call on a device
 * looks up that device's array once.  Every call on one GPU uses the same
 * array: calls that overlap on one GPU (on different streams) race, so order
 * them on one stream.  Nothing in the array needs initializing: each call
 * writes what it reads. */
int paged_decode_attn_noalloc(const void* q, const void* k_cache, const void* v_cache,
                              const int32_t* block_tables, const int32_t* context_lens,
                              int group, float scale, int num_splits, void* out, float* lse,
                              const pda_shape* shape, void* stream);

/* MLA paged decode attention over a latent cache (FlashMLA-ETAP "Usage";
 * "From MHA to MLA" sec. 6).  shape->num_kv_heads must be 1, (head_dim,
 * head_dim_v) (576, 512) or (320, 256) (a 512- or 256-wide latent + 64 rope
 * values; FlashMLA-ETAP "Supported configurations"; 320 with the matrix-core
 * variant only), q_dtype PDA_BF16, page_size a power of two, at least 64,
 * num_q_heads a multiple of 16 or at most 16.  kv_dtype PDA_BF16, or
 * PDA_FP8_E4M3 for an fp8 latent (the variants page's halved MLA record)
 * dequantized as e4m3(byte) * k_scale -- K and V are the same values, so
 * v_scale is ignored; k_scale is ignored for a bf16 latent.  The variant
 * field picks the kernel (PDA_MLA_*); q_len > 1 needs PDA_MLA_DEFAULT or
 * PDA_MLA_MFMA. */
int paged_decode_attn_mla(const void* q, const void* kv_cache, const int32_t* block_tables,
                          const int32_t* context_lens, float scale, int num_splits,
                          void* out, float* lse, const pda_shape* shape, void* workspace,
                          size_t workspace_bytes, void* stream);

/* Append the new tokens' K and V rows to the paged cache, the step before
 * attention ("From MHA to MLA" sec. 2: the new token's key and value join the
 * cache first; sec. 5 and the drill page sec. 4: a token's page is
 * block_tables[b][position / P], its slot position % P).
 *   k_new      [B, s_new, Hkv, head_dim]   of shape->q_dtype (s_new = q_len,
 *   v_new      [B, s_new, Hkv, head_dim_v]  0 meaning 1), device
 *   positions  [B] int32, device: position of sequence b's first new token;
 *              token t goes to position positions[b] + t; a negative entry
 *              skips the sequence (nothing is written for it)
 *   k_cache, v_cache: the caches of paged_decode_attn (updated in place)
 * v_new and v_cache are both NULL for a cache with K only (an MLA latent
 * cache: num_kv_heads 1, head_dim 576; V is the start of each record).
 * Same-type caches receive the elements unchanged.  A PDA_FP8_E4M3 cache
 * receives the E4M3FN code nearest to the fp32 quotient x / k_scale (v_scale
 * for V): ties to even, magnitudes at or beyond 448 saturate to 448, NaN
 * gives 0x7F.
 * Supported: (q_dtype, kv_dtype) = (F32, F32), (F16, F16), (BF16, BF16), or
 * any of F32/F16/BF16 with FP8_E4M3; head_dim and head_dim_v multiples of 8;
 * any page_size.  The four data pointers must be 16-byte aligned.  Only
 * batch, num_kv_heads, head_dim, head_dim_v, page_size, max_pages_per_seq,
 * num_pages, q_dtype, kv_dtype, k_scale, v_scale and q_len are read from
 * shape.  Preconditions (not checked): positions[b] + s_new <=
 * max_pages_per_seq * P, and the table entries of the pages written lie in
 * [0, num_pages).  Calls whose positions overlap write the same slots in an
 * unspecified order.  No workspace; asynchronous on `stream`. */
int paged_kv_append(const void* k_new, const void* v_new, const int32_t* block_tables,
                    const int32_t* positions, void* k_cache, void* v_cache,
                    const pda_shape* shape, void* stream);

/* Check, on the device, the preconditions the calls above take on trust
 * (the drill page sec. 4 and 8: lengths bound the pages read, and each
 * table entry a call follows is a page index into the pool).  Writes three
 * int32 counts to the DEVICE pointer `result`:
 *   result[0]  sequences with context_lens[b] outside [0, max_pages_per_seq * P];
 *   result[1]  table entries outside [0, num_pages) among those a call would
 *              follow: the first ceil(context_lens[b] / P) of row b (rows of
 *              sequences counted in result[0] are skipped), and, when
 *              `positions` is not NULL, the pages an append of q_len tokens at
 *              positions[b] writes;
 *   result[2]  sequences (positions not NULL, positions[b] >= 0) with
 *              positions[b] + q_len > max_pages_per_seq * P.
 * Reads batch, page_size, max_pages_per_seq, num_pages and q_len (the
 * append's s_new; 0 means 1) from shape.  `positions` may be NULL.  The
 * values read are only compared, never followed, so any contents are safe.
 * One workgroup reads every length and table entry: a debugging aid, not
 * for the decode loop.  Asynchronous on `stream`; read `result` after
 * synchronizing.  Errors: PDA_ERR_INVALID_ARG for a NULL shape or result, a
 * NULL table or length array with batch > 0, or non-positive sizes. */
int pda_check_inputs(const pda_shape* shape, const int32_t* block_tables,
                     const int32_t* context_lens, const int32_t* positions, int32_t* result,
                     void* stream);

/* Streaming-read probe: a measurement aid, not a step of the decode path.
 * Reads exactly the K and V bytes that paged_decode_attn reads for the same
 * arguments (the pages of each sequence through block_tables, the valid
 * rows of the last page; "From MHA to MLA" sec. 5, the drill page sec. 4)
 * with the attention kernels' access pattern -- one workgroup per
 * (sequence, KV head, split) with the split count and the wave layout that
 * pda_plan gives the same call (GRID schedule, num_splits), 16-token tiles,
 * row pieces of up to 16 bytes per lane, non-temporal loads -- but does no
 * arithmetic: each wave of a workgroup (four, or one when the plan's
 * waves_per_unit is 1) folds the words it loads into one 32-bit word of
 * `sink`.  Its duration is the practical ceiling for that access pattern on
 * the device (the attention kernel's time over it is the fraction of that
 * ceiling the kernel reaches).
 *   steps_in_flight: 1..4, tiles each wave keeps in flight;
 *   sink: DEVICE array of at least 4 * batch * num_kv_heads * max_splits
 *         uint32 (pda_plan_info.max_splits of the same call), contents
 *         unspecified; word ((split * batch + b) * num_kv_heads + kvh) * W +
 *         w is the XOR of the 32-bit words wave w of that workgroup read
 *         (W: its waves, 4 or 1).
 * Needs head_dim == head_dim_v with rows of 64, 128, 256 or 512 bytes and the
 * GRID schedule; other shape fields as for paged_decode_attn (they select
 * the plan as they would for the call).  Asynchronous on `stream`; returns a
 * pda_status. */
int pda_stream_probe(const void* k_cache, const void* v_cache, const int32_t* block_tables,
                     const int32_t* context_lens, const pda_shape* shape, int num_splits,
                     int steps_in_flight, uint32_t* sink, void* stream);

/* Static description of a status code. */
const char* pda_status_string(int status);

/* Library version, major * 10000 + minor * 100 + patch: 400 (0.4.0).  0.2
 * appended kv_layout to pda_shape and added pda_check_inputs (a caller built
 * against an older header passes a shorter pda_shape and must be rebuilt);
 * 0.3 added pda_stream_probe and caps BALANCED calls at 64 splits; 0.4 added
 * the one-wave GQA variant and appended waves_per_unit to pda_plan_info (a
 * caller built against an older header must be rebuilt). */
int pda_version(void);

#ifdef __cplusplus
}
#endif

#endif /* PDA_H */
