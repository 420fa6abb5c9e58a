// pda_gqa_mfma.hip -- paged decode attention for the GQA family on the gfx950
// matrix cores ("From MHA to MLA" sec. 3-5; the drill page sec. 3-5).
//
// Same contract as gqa_split_kernel (pda_gqa.hip): a workgroup owns a tile of
// up to 16 query heads of one KV group of one sequence (one split of its
// pages).  Either four waves walk its 16-token tiles (wave w takes tiles w,
// w+4, ...), keep an online softmax each and merge through LDS at the end, or
// (NW = 1, grid calls) one wave walks them all with two
// steps in flight and writes its result from registers.  A lone wave per
// unit keeps fewer bytes in flight per compute unit and has no merge; on
// MI355X it streams the B=64 / 1024-token fp16 cache in 40.6-41.1 us against
// 42.0-42.5 with four waves (token-major pages 40.7-41.4 against 43.9-44.3).
// What changes against the vector kernel is the arithmetic of a tile:
//
//  - scores as S^T = K Q^T with the tile's 16 tokens on the MFMA M dimension
//    and the 16 heads on N (v_mfma_f32_16x16x32, D/32 of them).  The result
//    gives lane (head = lane % 16, group g = lane / 16) the scores of tokens
//    4g..4g+3, which is exactly the B-operand layout of the 16x16x16 MFMA
//    with the tokens as the contraction, so P^T needs no lane exchange;
//  - O^T += V^T P^T (v_mfma_f32_16x16x16, D/16 of them; for bfloat16 queries
//    twice, with p split into two bfloat16 terms), the output rows being
//    value dimensions and the columns heads, so a lane rescales only its own
//    head's accumulators when the running max moves.
//
// Loads stay row-coalesced: load j of a tile gives lane (g, u) token 4j + g
// (fp8 caches: 4g + j), elements [u D/16, (u+1) D/16) of the row, so every
// load instruction covers four whole token rows (consecutive ones for 16-bit
// caches).  That is already the A-operand layout of V^T (lane row u,
// contraction over 4 tokens: two v_perm_b32 per operand), with contraction
// index 4g + i standing for token g + 4i (fp8: 4g + i).  K needs the
// transposed assignment (lane row = token), so each wave writes its K tile
// into its own padded LDS tile and reads it back in the MFMA layout; it is
// written in the same permuted row order, so the score rows S^T come out in
// the contraction order of V^T and P^T needs no exchange.
// Rows are padded by 32 bytes: the hardware's bank-conflict counter reads
// zero for the tile's writes and reads at d = 128 (with 16 or 64 bytes of
// padding it counts 16 conflict cycles per tile and wave, with none 112).
//
// The columns are the (query token, head) rows of the KV group: row
// i * group + g is query token i of head g (one token per sequence in plain
// decode, q_len with multi-token decode), so q_len * group rows are tiled by
// 16.  Spare MFMA columns are computed on zero queries and never written.  A
// causal mask gives each column its own token limit (query i of q_len sees
// the first n - (q_len - 1 - i) tokens).
#include "pda_device.h"

namespace pda {
namespace {

typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));

constexpr int kMWaves = 4;
constexpr int kMHeads = 16;  // MFMA N: heads per workgroup tile

// Pieces of a token row held by one lane: D/16 elements.
template <class KT, int D>
struct Piece {
  static constexpr int bytes = D / 16 * Elem<KT>::bytes;
  static constexpr int words = bytes / 4;
};

template <int W>
struct Words {
  uint32_t w[W];
};

// Row piece of `W` words at byte `off` of a tile resource (non-temporal).
template <int W>
__device__ __forceinline__ Words<W> load_piece(__amdgpu_buffer_rsrc_t r, int off) {
  Words<W> p;
  if constexpr (W == 1) {
    p.w[0] = __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, PDA_KV_LOAD_POLICY);
  } else if constexpr (W == 2) {
    const u32x2 x = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, PDA_KV_LOAD_POLICY);
    p.w[0] = x[0];
    p.w[1] = x[1];
  } else {
#pragma unroll
    for (int h = 0; h < W / 4; ++h) {
      const u32x4 x = __builtin_amdgcn_raw_buffer_load_b128(r, off + 16 * h, 0, PDA_KV_LOAD_POLICY);
      p.w[4 * h] = x[0];
      p.w[4 * h + 1] = x[1];
      p.w[4 * h + 2] = x[2];
      p.w[4 * h + 3] = x[3];
    }
  }
  return p;
}

// A 16-bit row piece of W words (2 or a multiple of 4) into LDS.
template <int W>
__device__ __forceinline__ void store_piece(char* dst, const Words<W>& p) {
  if constexpr (W == 2) {
    *(u32x2*)dst = u32x2{p.w[0], p.w[1]};
  } else {
    static_assert(W % 4 == 0, "piece width");
#pragma unroll
    for (int w = 0; w < W; w += 4) *(u32x4*)(dst + 4 * w) = u32x4{p.w[w], p.w[w + 1], p.w[w + 2], p.w[w + 3]};
  }
}

// Four fp8 values (one word) as two 16-bit-float pairs in the query's type.
template <class QT>
__device__ __forceinline__ uint32_t fp8_pair(uint32_t x, bool hi) {
  if constexpr (std::is_same<QT, F16>::value) {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false));
  } else {
    return __builtin_bit_cast(uint32_t, hi ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true)
                                           : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false));
  }
}

// N consecutive outputs (N = 4, 8 or 16) in the query's 16-bit type, rounded
// to nearest even, with 8- or 16-byte stores.
template <class QT, int N>
__device__ __forceinline__ void store_row(void* out, int64_t i, const float (&o)[N]) {
  uint32_t w[N / 2];
#pragma unroll
  for (int k = 0; k < N / 2; ++k) {
    if constexpr (std::is_same<QT, F16>::value) {
      w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{o[2 * k], o[2 * k + 1]}), f16x2));
    } else {
      w[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{o[2 * k], o[2 * k + 1]}), bf16x2));
    }
  }
  char* p = (char*)out + i * 2;
  if constexpr (N == 4) {
    *(u32x2*)p = u32x2{w[0], w[1]};
  } else {
#pragma unroll
    for (int k = 0; k < N / 2; k += 4) *(u32x4*)(p + 4 * k) = u32x4{w[k], w[k + 1], w[k + 2], w[k + 3]};
  }
}

template <class QT>
__device__ __forceinline__ f32x4 mfma_qk(const u32x4& k, const u32x4& q, f32x4 c) {
  if constexpr (std::is_same<QT, F16>::value) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, k),
                                                  __builtin_bit_cast(f16x8, q), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k),
                                                   __builtin_bit_cast(bf16x8, q), c, 0, 0, 0);
  }
}

template <class QT>
__device__ __forceinline__ f32x4 mfma_pv(const u32x2& v, const u32x2& p, f32x4 c) {
  if constexpr (std::is_same<QT, F16>::value) {
    return __builtin_amdgcn_mfma_f32_16x16x16f16(__builtin_bit_cast(f16x4, v),
                                                 __builtin_bit_cast(f16x4, p), c, 0, 0, 0);
  } else {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(__builtin_bit_cast(s16x4, v),
                                                     __builtin_bit_cast(s16x4, p), c, 0, 0, 0);
  }
}

// The values the prologue needs come first as separate arguments: with kernel
// argument preloading (gfx950) they arrive in scalar registers when the wave
// starts, so the length, table and q requests go out without waiting for a
// kernel-argument load.  GqaArgs carries everything (the same values too).
// CT column tiles of 16 rows per workgroup: one, or two for groups of more
// than 16 rows (d <= 128), so that one load of a K/V tile serves 32 rows.
// SD steps of tiles in flight per wave (see kGqaStepsInFlight), ST tiles per
// step.
template <class QT, class KT, int D, int CT, int SD, int ST, int NW>
__global__ __launch_bounds__(NW * 64, 2) void gqa_mfma_kernel(
    const int32_t* context_lens, const int32_t* block_tables, const void* q, int32_t head_tiles,
    int32_t num_kv_heads, int32_t group, int32_t q_len, int32_t max_pages, int32_t log2_page,
    int32_t pages_per_split, int32_t max_splits, const int32_t* units, GqaArgs a) {
  constexpr int ESZ = Elem<KT>::bytes;
  constexpr int PW = Piece<KT, D>::words;       // words of a loaded row piece
  constexpr int NE = D / 16;                    // elements per piece = PV MFMAs
  constexpr int NQK = D / 32;                   // QK MFMAs (32 contraction each)
  constexpr int kRowB = D * 2 + 32;             // LDS bytes per K row (16-bit, padded)
  constexpr int kTileB = kTileTokens * kRowB;   // one wave's K tile
  constexpr bool kFp8 = std::is_same<KT, E4M3>::value;
  constexpr bool kBf16 = std::is_same<QT, BF16>::value;
  constexpr int kAccStride = D + 4;             // floats per head row of the merge area
  constexpr int kMergeB = NW > 1 ? NW * kMHeads * kAccStride * 4 : 0;
  // the merge area gets its own LDS when both fit two workgroups per CU
  constexpr bool kSeparateMerge = NW * kTileB + kMergeB <= 72 * 1024;
  constexpr int kMergeOff = kSeparateMerge ? NW * kTileB : 0;
  constexpr int kLdsB = kSeparateMerge ? NW * kTileB + kMergeB
                        : (NW * kTileB > kMergeB ? NW * kTileB : kMergeB);
  static_assert(D == 64 || D == 128 || D == 256, "head_dim");
  static_assert(CT == 1 || (CT == 2 && D <= 128), "column tiles");
  constexpr int kRowsWG = kMHeads * CT;         // (query token, head) rows of a workgroup
  static_assert(kFp8 || std::is_same<QT, KT>::value, "q / cache types");

  __shared__ __attribute__((aligned(16))) char lds[kLdsB];
  __shared__ float m_sh[NW][kMHeads], l_sh[NW][kMHeads];

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;  // MFMA column (head) / V^T row piece / K row token
  const int grp = lane >> 4;  // lane group

  // which (sequence, KV head, head tile, split) this workgroup computes
  // One-wave workgroups serve grid calls only: their grid is (units, splits).
  // An ordered launch (x = KV heads x head tiles x listed units) would map
  // workgroups past the batch, so such a launch leaves at once (launch_sd
  // never makes one).
  if constexpr (NW == 1) {
    if (units != nullptr || a.plan_in_kernel) return;
  }
  const bool ordered = NW > 1 && (units != nullptr || a.plan_in_kernel);
  int tile, kvh, b, split, ut0 = 0, ut1 = 0;
  if (ordered) {
    // ordered: the unit list gives (sequence, split, token range) longest
    // first; the (unit, KV head) groups follow it, each with its head tiles
    // (group_tile)
    int g;
    group_tile(blockIdx.x, gridDim.x / head_tiles, head_tiles, g, tile);
    g = __builtin_amdgcn_readfirstlane(g);  // (uniform: scalar registers)
    tile = __builtin_amdgcn_readfirstlane(tile);
    WorkUnit w;
    if (units) {  // the planning kernel's list
      w = load_unit(units, g / num_kv_heads);
    } else {      // this workgroup derives its unit from the lengths
      __shared__ PlanShared plan_sh;
      int ns_b;
      w = plan_unit<NW * 64>(context_lens, a.plan, g / num_kv_heads, plan_sh, ns_b);
      w.b = __builtin_amdgcn_readfirstlane(w.b);
      w.split = __builtin_amdgcn_readfirstlane(w.split);
      w.t0 = __builtin_amdgcn_readfirstlane(w.t0);
      w.t1 = __builtin_amdgcn_readfirstlane(w.t1);
      // the sequence's split count, for the combine kernel (written once)
      if (w.b >= 0 && w.split <= 0 && g % num_kv_heads == 0 && tile == 0 && threadIdx.x == 0)
        a.seq_splits[w.b] = ns_b;
    }
    if (w.b < 0) return;
    b = w.b;
    split = w.split;
    ut0 = w.t0;
    ut1 = w.t1;
    kvh = g % num_kv_heads;
  } else {
    int bk;
    group_tile(blockIdx.x, gridDim.x / head_tiles, head_tiles, bk, tile);
    bk = __builtin_amdgcn_readfirstlane(bk);  // (uniform: scalar registers)
    tile = __builtin_amdgcn_readfirstlane(tile);
    kvh = bk % num_kv_heads;
    b = bk / num_kv_heads;
    split = blockIdx.y;
  }

  const int num_q_heads = group * num_kv_heads;
  const int g0 = tile * kRowsWG;                   // the tile's first row
  const int gvalid = min(kRowsWG, q_len * group - g0);
  const int log2P = log2_page;
  const int32_t* table = block_tables + (int64_t)b * max_pages;
  const int t0_hint = ordered ? ut0 : max_splits > 1 ? split * pages_per_split << log2P : 0;

  // The range is walked in steps of ST consecutive tiles; wave w takes steps
  // w, w + NW, ...  Sequence length, block-table entries (lane j: tile
  // j % ST of the wave's step sbase + j / ST, clamped into the row, unused
  // past the sequence) and q are requested together.
  constexpr int kStepsPerChunk = 64 / ST;
  auto load_table = [&](int sbase) -> int {
    const int T = (wave + (sbase + lane / ST) * NW) * ST + lane % ST;
    const int64_t tok = (int64_t)t0_hint + (int64_t)T * kTileTokens;
    const int64_t pg = tok >> log2P;
    return table[pg < max_pages ? pg : max_pages - 1];
  };
  // Every workgroup requests its length, its first table entries and q
  // together, and only then decides whether its split has pages at all (a
  // split past the end of a short sequence leaves after that one round trip;
  // the entries it loaded lie in the table row and are never used).
  int vtbl = load_table(0);
  int n = load_uniform(context_lens + b);

  // Q^T as the B operand of the QK MFMAs: lane (col, grp) holds, for column
  // tile c, q[row 16 c + col][32 j + 8 grp .. +8] for MFMA j; rows past the
  // group are zero.  Row g0 + 16 c + col is query token qi[c] of head g of
  // the group.
  int qi[CT];
  u32x4 qb[CT][NQK];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const bool hv = 16 * c + col < gvalid;
    const int r = g0 + (hv ? 16 * c + col : 0);
    int g = r;
    qi[c] = 0;
    if (q_len > 1) {
      qi[c] = r / group;
      g = r - qi[c] * group;
    }
    const char* qrow =
        (const char*)q + ((((int64_t)b * q_len + qi[c]) * num_q_heads + kvh * group + g) * D) * 2;
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      const u32x4 w = *(const u32x4*)(qrow + (32 * j + 8 * grp) * 2);
      qb[c][j] = hv ? w : u32x4{0u, 0u, 0u, 0u};
    }
  }

  __builtin_amdgcn_sched_barrier(0);  // the loads above go out before waiting for n
  int nsplit, t0, t1;
  if (ordered) {  // the unit's range; split -1: the sequence's only split
    nsplit = split < 0 ? 1 : 2;
    t0 = ut0;
    t1 = ut1;
  } else {
    split_range(a.split, n, a.page_size, split, nsplit, t0, t1);
    if (split >= nsplit) return;
  }
  // end of the tokens this lane's query tokens may see (t1 without a mask)
  int lim[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) lim[c] = min(t1, a.causal ? n - (q_len - 1 - qi[c]) : n);

  const int tok_bytes = a.tok_stride * ESZ;
  // load j of a tile, 16-bit caches: token 4 j + grp, piece col of the row
  // (relative to the tile's first token row of this KV head), so that one
  // load instruction covers four consecutive rows (1 KiB at d = 128: with
  // head-major pages one contiguous run; B=64 41.8 against 42.0 us with
  // four runs of 256 bytes).  The tokens of the MFMA k index follow from it:
  // k = 4 grp + i is token grp + 4 i, in V^T (load i) and in S^T alike.
  // fp8 caches keep token 4 grp + j (k = 4 grp + i is token 4 grp + i): with
  // their 128-byte rows consecutive rows measured 0.2% slower.
  constexpr bool kConsec = !kFp8;
  const int off0 = (kConsec ? grp : 4 * grp) * tok_bytes + (col * NE) * ESZ;
  const int row_step = kConsec ? 4 * tok_bytes : tok_bytes;
  // this KV head's rows in page 0, and the bytes of a page: a tile's rows
  // start at page * page_bytes + slot * tok_bytes from there (page indices
  // are non-negative, so one unsigned 32 x 64-bit product per tile)
  const char* kbase = (const char*)a.k_cache + (int64_t)kvh * a.head_stride * ESZ;
  const char* vbase = (const char*)a.v_cache + (int64_t)kvh * a.head_stride * ESZ;
  const uint64_t page_bytes = (uint64_t)a.page_stride * ESZ;

  // O^T of column tile c: rows (4 grp + i) * NE + e of the value, column =
  // row 16 c + col of the workgroup
  f32x4 acc[CT][NE];
  float m_run[CT], l_run[CT];
#pragma unroll
  for (int c = 0; c < CT; ++c) {
#pragma unroll
    for (int e = 0; e < NE; ++e) acc[c][e] = f32x4{0.f, 0.f, 0.f, 0.f};
    m_run[c] = kMaxStart;
    l_run[c] = 0.f;
  }
  const float pinf = opaque_inf();

  const int ntiles = (t1 - t0 + kTileTokens - 1) / kTileTokens;
  const int nsteps = (ntiles + ST - 1) / ST;
  const int ns_wave = nsteps > wave ? (nsteps - wave + NW - 1) / NW : 0;

  char* ktile = lds + wave * kTileB;

  // rows: valid token rows of the tile, tok: its first token
  auto compute_tile = [&](const Words<PW> (&kf)[4], const Words<PW> (&vf)[4], int rows, int tok) {
    // ---- K tile into LDS in 16-bit form: LDS row 4 grp + j holds load j
    // (token 4 j + grp, or 4 grp + j for fp8), piece col at 2 NE col bytes;
    // so S^T row r is token (r % 4) * 4 + r / 4 (fp8: r)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      char* dst = ktile + (4 * grp + j) * kRowB + col * NE * 2;
      if constexpr (kFp8) {
        Words<2 * PW> h;
#pragma unroll
        for (int w = 0; w < PW; ++w) {
          h.w[2 * w] = fp8_pair<QT>(kf[j].w[w], false);
          h.w[2 * w + 1] = fp8_pair<QT>(kf[j].w[w], true);
        }
        store_piece<2 * PW>(dst, h);
      } else {
        store_piece<PW>(dst, kf[j]);
      }
    }
    // ---- S^T = K Q^T: lane reads token col, elements 32 j + 8 grp .. +8 (one
    // K operand for every column tile)
    f32x4 st[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) st[c] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j = 0; j < NQK; ++j) {
      const u32x4 kk = *(const u32x4*)(ktile + col * kRowB + (32 * j + 8 * grp) * 2);
#pragma unroll
      for (int c = 0; c < CT; ++c) st[c] = mfma_qk<QT>(kk, qb[c][j], st[c]);
    }
    // ---- online softmax per column tile (log2 domain, lazily moved
    // reference max); this lane holds S^T rows 4 grp + i (tokens grp + 4 i;
    // fp8: 4 grp + i) of row 16 c + col
    u32x2 pb[CT], pb_lo[CT];
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const int rl = min(rows, lim[c] - tok);
      float s[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        s[i] = fminf(st[c][i] * a.qk_scale_log2,
                     (kConsec ? grp + 4 * i : 4 * grp + i) < rl ? INFINITY : -INFINITY);
      float tmax = max2(max2(s[0], s[1], pinf), max2(s[2], s[3], pinf), pinf);
      {
        float x, y;
        swap16(tmax, tmax, x, y);
        tmax = max2(x, y, pinf);
        swap32(tmax, tmax, x, y);
        tmax = max2(x, y, pinf);
      }
      const bool move = tmax > m_run[c] + kLazyMax;
      const float m_new = move ? tmax : m_run[c];
      const float alpha = __builtin_amdgcn_exp2f(m_run[c] - m_new);
      m_run[c] = m_new;
      float p[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) p[i] = __builtin_amdgcn_exp2f(s[i] - m_new);
      if constexpr (!kBf16) {
        // binary16 probabilities (round to nearest even); the denominator sums
        // the same rounded values
        const f16x2 p01 = __builtin_convertvector((f32x2{p[0], p[1]}), f16x2);
        const f16x2 p23 = __builtin_convertvector((f32x2{p[2], p[3]}), f16x2);
        const f16x2 one = {(_Float16)1.0f, (_Float16)1.0f};
        l_run[c] = __builtin_amdgcn_fdot2(
            p23, one, __builtin_amdgcn_fdot2(p01, one, l_run[c] * alpha, false), false);
        pb[c] = u32x2{__builtin_bit_cast(uint32_t, p01), __builtin_bit_cast(uint32_t, p23)};
      } else {
        // p = p_hi + p_lo, two bfloat16 terms (bfloat16 alone leaves 2^-9
        // relative error per weight)
        uint16_t hi[4], lo[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const __bf16 h = (__bf16)p[i];
          const __bf16 l = (__bf16)(p[i] - (float)h);
          hi[i] = __builtin_bit_cast(uint16_t, h);
          lo[i] = __builtin_bit_cast(uint16_t, l);
        }
        l_run[c] = l_run[c] * alpha + ((p[0] + p[1]) + (p[2] + p[3]));
        pb[c] = u32x2{(uint32_t)hi[0] | ((uint32_t)hi[1] << 16),
                      (uint32_t)hi[2] | ((uint32_t)hi[3] << 16)};
        pb_lo[c] = u32x2{(uint32_t)lo[0] | ((uint32_t)lo[1] << 16),
                         (uint32_t)lo[2] | ((uint32_t)lo[3] << 16)};
      }
      // alpha is exactly 1 while the reference max stays.  With one column
      // tile the multiplies are skipped unless a lane's max moved (a wave-
      // uniform branch; one wave, B=64: bfloat16 41.5 against 42.3 us,
      // float16 0.1-0.2 us faster; four waves: the ragged fp8 batch 0.2-1.2
      // us faster, fp8 B=64 at 2048 tokens 0.2-0.4).  Two column tiles
      // multiply unconditionally: there a branch made the compiler copy both
      // tiles' accumulators on every tile (0.4 us of the MQA step).
      if constexpr (NW == 1 || CT == 1) {
        if (__builtin_amdgcn_ballot_w64(move)) {
#pragma unroll
          for (int e = 0; e < NE; ++e) acc[c][e] *= alpha;
        }
      } else {
#pragma unroll
        for (int e = 0; e < NE; ++e) acc[c][e] *= alpha;
      }
    }
    // ---- O^T += V^T P^T.  A operand of MFMA e: V^T row col (value element
    // col NE + e) at k = 4 grp + i (the token of load i) = element e of the
    // four loads (one V operand for every column tile).
#pragma unroll
    for (int e = 0; e < NE; ++e) {
      u32x2 va;
      if constexpr (kFp8) {
        // bytes e of loads (0, 1) and (2, 3), widened exactly
        const int w = e >> 2, sh = e & 3;
        const uint32_t sel = 0x0c0c0000u | ((4u + sh) << 8) | (uint32_t)sh;  // [a.e, b.e, 0, 0]
        const uint32_t x01 = __builtin_amdgcn_perm(vf[1].w[w], vf[0].w[w], sel);
        const uint32_t x23 = __builtin_amdgcn_perm(vf[3].w[w], vf[2].w[w], sel);
        va = u32x2{fp8_pair<QT>(x01, false), fp8_pair<QT>(x23, false)};
      } else {
        const int w = e >> 1;
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;  // hi / lo halves of {b : a}
        va = u32x2{__builtin_amdgcn_perm(vf[1].w[w], vf[0].w[w], sel),
                   __builtin_amdgcn_perm(vf[3].w[w], vf[2].w[w], sel)};
      }
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        acc[c][e] = mfma_pv<QT>(va, pb[c], acc[c][e]);
        if constexpr (kBf16) acc[c][e] = mfma_pv<QT>(va, pb_lo[c], acc[c][e]);
      }
    }
  };

  // Steps in flight per wave: SD (1: a step's loads are issued right before
  // it is computed; other waves cover the latency).  Each step issues the
  // loads of its ST tiles back to back.  Steps are grouped in chunks of
  // kStepsPerChunk (one table entry per lane per tile).
  Words<PW> kb[SD][ST][4], vb[SD][ST][4];
  int rows_b[SD][ST], tok_b[SD][ST];
  auto issue = [&](int sidx, int send, int u) {
#pragma unroll
    for (int t = 0; t < ST; ++t) {
      const int T = (wave + sidx * NW) * ST + t;
      const bool live = sidx < send && T < ntiles;
      const int entry = __builtin_amdgcn_readlane(vtbl, ((sidx % kStepsPerChunk) * ST + t) & 63);
      const int phys = live ? entry : 0;
      const int tok = t0 + T * kTileTokens;
      const int rows = live ? min(kTileTokens, t1 - tok) : 0;
      rows_b[u][t] = rows;
      tok_b[u][t] = tok;
      const int slot = tok & ((1 << log2P) - 1);
      const uint64_t off = (uint64_t)(uint32_t)phys * page_bytes + (uint32_t)(slot * tok_bytes);
      const __amdgpu_buffer_rsrc_t rk = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(kbase + off), 0, rows * tok_bytes, kRsrcFlags);
      const __amdgpu_buffer_rsrc_t rv = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(vbase + off), 0, rows * tok_bytes, kRsrcFlags);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kb[u][t][j] = load_piece<PW>(rk, off0 + j * row_step);
        vb[u][t][j] = load_piece<PW>(rv, off0 + j * row_step);
      }
    }
  };
  for (int sbase = 0; sbase < ns_wave;) {
    const int send = min(sbase + kStepsPerChunk, ns_wave);
    // (in order: the loop's wait counts assume the oldest step is issued first)
#pragma unroll
    for (int u = 0; u < SD - 1; ++u) {
      issue(sbase + u, send, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int sc = sbase;; sc += SD) {
#pragma unroll
      for (int u = 0; u < SD; ++u) {
        const int sidx = sc + u;
        if (sidx >= send) goto chunk_done;
        issue(sidx + SD - 1, send, (u + SD - 1) % SD);
        __builtin_amdgcn_sched_barrier(0);  // all of a step's loads go out before any wait
        // (a step's tiles past the range are computed on zero rows, fully
        // masked: no branch that would let the compiler sink their loads)
#pragma unroll
        for (int t = 0; t < ST; ++t) compute_tile(kb[u][t], vb[u][t], rows_b[u][t], tok_b[u][t]);
      }
    }
  chunk_done:
    sbase = send;
    if (sbase < ns_wave) vtbl = load_table(sbase);
  }

  // ---- epilogue
  if constexpr (NW == 1) {
    // One wave owns the unit: nothing to merge.  Lane (col, grp) holds, for
    // column tile c, values (4 grp + i) NE .. + NE of row 16 c + col (i = 0..3),
    // and a quarter of that row's sum (its four lane groups add it up); the
    // running max is the same in the four.
#pragma unroll
    for (int c = 0; c < CT; ++c) {
      const float den = pair_sum<5>(pair_sum<4>(l_run[c]));
      if (16 * c + col >= gvalid) continue;
      const float inv = den > 0.f ? a.v_scale * __builtin_amdgcn_rcpf(den) : 0.f;
      const float lse_v = den > 0.f ? (m_run[c] + __log2f(den)) * kLn2 : -INFINITY;
      int i = 0, gh = g0 + 16 * c + col;
      if (q_len > 1) {
        i = gh / group;
        gh -= i * group;
      }
      const int h = kvh * group + gh;
      const int64_t row = ((int64_t)b * q_len + i) * num_q_heads + h;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int d0 = (4 * grp + r) * NE;
        float o[NE];
#pragma unroll
        for (int e = 0; e < NE; ++e) o[e] = acc[c][e][r] * inv;
        if (nsplit == 1) {
          store_row<QT, NE>(a.out, row * D + d0, o);
        } else {
          float* po = a.part_o + (row * a.split.max_splits + split) * D + d0;
#pragma unroll
          for (int e = 0; e < NE; e += 4) *(f32x4*)(po + e) = f32x4{o[e], o[e + 1], o[e + 2], o[e + 3]};
        }
      }
      if (grp == 0) {
        if (nsplit == 1) {
          if (a.lse) a.lse[((int64_t)b * num_q_heads + h) * q_len + i] = lse_v;
        } else {
          a.part_lse[row * a.split.max_splits + split] = lse_v;
        }
      }
    }
    return;
  }
  // ---- merge the four waves (the split-combine algebra) through LDS, one
  // column tile after the other through the same 16-row area.  When the
  // merge area overlays the K tiles, every wave must be done with them; a
  // second column tile waits for the readers of the first.
  float* acc_sh = (float*)(lds + kMergeOff);  // [wave][head][kAccStride]
  constexpr int kQ = D / 4;                   // four-value items per row
#pragma unroll
  for (int c = 0; c < CT; ++c) {
    const float l_c = pair_sum<5>(pair_sum<4>(l_run[c]));
    if (c > 0 || !kSeparateMerge) __syncthreads();
    const int gv = min(kMHeads, gvalid - 16 * c);  // valid rows of this column tile
    if (grp == 0) {
      m_sh[wave][col] = m_run[c];
      l_sh[wave][col] = l_c;
    }
    if (col < gv) {  // only the rows of the group
      float* dst = acc_sh + (wave * kMHeads + col) * kAccStride;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int e = 0; e < NE; e += 4)
          *(f32x4*)(dst + (4 * grp + i) * NE + e) =
              f32x4{acc[c][e][i], acc[c][e + 1][i], acc[c][e + 2][i], acc[c][e + 3][i]};
    }
    __syncthreads();

    // Work items: four consecutive values of one valid row, spread over all
    // threads; each item issues its LDS reads (the four waves' max, sum and
    // values) before any arithmetic: weights exp2(m_w - max), one reciprocal.
    // (A row no wave saw a token of keeps max kMaxStart and sum 0: out 0.)
    for (int it = threadIdx.x; it < gv * kQ; it += NW * 64) {
      const int g = it / kQ, d0 = 4 * (it % kQ);
      float mw[NW], lw[NW];
      f32x4 xw[NW];
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        mw[w] = m_sh[w][g];
        lw[w] = l_sh[w][g];
        xw[w] = *(const f32x4*)(acc_sh + (w * kMHeads + g) * kAccStride + d0);
      }
      float mx = mw[0];
#pragma unroll
      for (int w = 1; w < NW; ++w) mx = fmaxf(mx, mw[w]);
      f32x4 num = {0.f, 0.f, 0.f, 0.f};
      float den = 0.f;
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float wt = mx == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mw[w] - mx);
        den += wt * lw[w];
        num += wt * xw[w];
      }
      const float inv = den > 0.f ? a.v_scale * __builtin_amdgcn_rcpf(den) : 0.f;
      const float o[4] = {num.x * inv, num.y * inv, num.z * inv, num.w * inv};
      // row g0 + 16 c + g of the group: query token i, head h; out row
      // (b, i, h), lse [B, Hq, q_len]
      int i = 0, gh = g0 + 16 * c + g;
      if (q_len > 1) {
        i = gh / group;
        gh -= i * group;
      }
      const int h = kvh * group + gh;
      const int64_t row = ((int64_t)b * q_len + i) * num_q_heads + h;
      if (nsplit == 1) {
        store_row<QT, 4>(a.out, row * D + d0, o);
        if (d0 == 0 && a.lse)
          a.lse[((int64_t)b * num_q_heads + h) * q_len + i] =
              den > 0.f ? (mx + __log2f(den)) * kLn2 : -INFINITY;
      } else {
        float* po = a.part_o + (row * a.split.max_splits + split) * D + d0;
        const f32x4 ov = {o[0], o[1], o[2], o[3]};
        if constexpr (CT == 2) {
          // 32-row workgroups write 16 KiB of partials each (MQA: 8.4 MB
          // per call, most of it in the last microseconds): written through
          // to memory (sc0 sc1) rather than left dirty in L2 for the end of
          // the kernel, 51.0-51.3 against 51.7-51.9 us per MQA step.  With
          // 16-row workgroups (2 KiB) plain stores measured faster.
          asm volatile("global_store_dwordx4 %0, %1, off sc0 sc1" ::"v"(po), "v"(ov) : "memory");
        } else {
          *(f32x4*)po = ov;
        }
        if (d0 == 0)
          a.part_lse[row * a.split.max_splits + split] =
              den > 0.f ? (mx + __log2f(den)) * kLn2 : -INFINITY;
      }
    }
  }
}

// grid calls with kGqaStepsInFlight steps in flight (kGqaStepsInFlightFp8 for
// fp8 caches), ordered ones with kGqaStepsInFlightOrdered; ST tiles per step.
// Workgroups of four waves, or of one (a.waves == 1: grid calls) with
// kGqaStepsInFlightWave steps in flight.
template <class QT, class KT, int D, int CT, int ST>
void launch_sd(const GqaArgs& a, dim3 grid, hipStream_t s) {
  constexpr int kGridSD = std::is_same<KT, E4M3>::value ? kGqaStepsInFlightFp8 : kGqaStepsInFlight;
#define PDA_MFMA_ARGS                                                                        \
  a.context_lens, a.block_tables, a.q, a.head_tiles, a.num_kv_heads, a.group, a.q_len,        \
      a.max_pages, a.log2_page, a.split.pages_per_split, a.split.max_splits, a.units, a
  const bool ordered = a.units || a.plan_in_kernel;
  if (ordered)
    hipLaunchKernelGGL((gqa_mfma_kernel<QT, KT, D, CT, kGqaStepsInFlightOrdered, ST, kMWaves>),
                       grid, dim3(kMWaves * 64), 0, s, PDA_MFMA_ARGS);
  else if (a.waves == 1)
    hipLaunchKernelGGL((gqa_mfma_kernel<QT, KT, D, CT, kGqaStepsInFlightWave, ST, 1>), grid,
                       dim3(64), 0, s, PDA_MFMA_ARGS);
  else
    hipLaunchKernelGGL((gqa_mfma_kernel<QT, KT, D, CT, kGridSD, ST, kMWaves>), grid,
                       dim3(kMWaves * 64), 0, s, PDA_MFMA_ARGS);
#undef PDA_MFMA_ARGS
}

// Tiles per step: kGqaStepTilesFp8 for fp8 caches whose tile rows are
// contiguous (head-major pages, or a single KV head), else kGqaStepTiles.  An
// fp8 tile is half the bytes of a 16-bit one; two per step issue as many
// (head-major B=64 at 2048 tokens: 43.3 against 44.2 us; the ragged batch,
// balanced: 86.6 against 88.0) -- but with token-major rows 1 KiB apart they
// slow down (48.1 against 44.9 us; ragged 95.5 against 93.9).
template <class QT, class KT, int D, int CT>
void launch_st(const GqaArgs& a, dim3 grid, hipStream_t s) {
  if constexpr (std::is_same<KT, E4M3>::value && kGqaStepTilesFp8 != kGqaStepTiles) {
    if (a.tok_stride == D) {
      launch_sd<QT, KT, D, CT, kGqaStepTilesFp8>(a, grid, s);
      return;
    }
  }
  launch_sd<QT, KT, D, CT, kGqaStepTiles>(a, grid, s);
}

template <class QT, class KT>
hipError_t launch_mfma_qk(const GqaArgs& a, int head_dim, int max_splits, hipStream_t s) {
  const unsigned units = (unsigned)(a.batch * a.num_kv_heads * a.head_tiles);
  const unsigned nhu = (unsigned)(a.num_kv_heads * a.head_tiles);
  const bool ordered = a.units || a.plan_in_kernel;
  dim3 grid(ordered ? nhu * (unsigned)a.unit_count : units, ordered ? 1u : (unsigned)max_splits);
  const bool two =
      gqa_mfma_col_tiles(a.q_len * a.group, head_dim, (int64_t)a.max_pages * a.page_size) == 2;
  switch (head_dim) {
    case 64:
      if (two) launch_st<QT, KT, 64, 2>(a, grid, s);
      else launch_st<QT, KT, 64, 1>(a, grid, s);
      break;
    case 128:
      if (two) launch_st<QT, KT, 128, 2>(a, grid, s);
      else launch_st<QT, KT, 128, 1>(a, grid, s);
      break;
    case 256: launch_st<QT, KT, 256, 1>(a, grid, s); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

bool gqa_mfma_supported(int q_dtype, int kv_dtype, int head_dim) {
  const bool pair_ok = (q_dtype == 1 && (kv_dtype == 1 || kv_dtype == 3)) ||
                       (q_dtype == 2 && (kv_dtype == 2 || kv_dtype == 3));
  return pair_ok && (head_dim == 64 || head_dim == 128 || head_dim == 256);
}

hipError_t launch_gqa_mfma(const GqaArgs& a, int q_dtype, int kv_dtype, int head_dim,
                           int max_splits, hipStream_t s) {
  if (q_dtype == 1 && kv_dtype == 1) return launch_mfma_qk<F16, F16>(a, head_dim, max_splits, s);
  if (q_dtype == 2 && kv_dtype == 2) return launch_mfma_qk<BF16, BF16>(a, head_dim, max_splits, s);
  if (q_dtype == 1 && kv_dtype == 3) return launch_mfma_qk<F16, E4M3>(a, head_dim, max_splits, s);
  if (q_dtype == 2 && kv_dtype == 3) return launch_mfma_qk<BF16, E4M3>(a, head_dim, max_splits, s);
  return hipErrorInvalidValue;
}

}  // namespace pda
