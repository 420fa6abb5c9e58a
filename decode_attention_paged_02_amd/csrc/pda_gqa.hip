// pda_gqa.hip -- paged decode attention for the GQA family (MHA / GQA / MQA)
// on gfx950, plus the split-KV combine kernel.
//
// What is computed ("From MHA to MLA" sec. 3-5; the drill page sec. 3-5):
// one workgroup owns a tile of GT query heads of one KV group of one sequence
// (and one split of its pages), so every K/V row it loads from HBM serves all
// GT heads; scores go through an online softmax; the result is either the
// final output (one split) or a normalized partial plus its LSE (several
// splits, merged by combine_kernel, "From MHA to MLA" sec. 4).
//
// Layout of the work inside a workgroup (4 waves of 64 lanes):
//  - a "tile" is 16 consecutive tokens of one page (pages are multiples of
//    16 tokens); wave w walks tiles w, w+4, w+8, ... of the workgroup's range
//    with its own online-softmax state, and the four states are merged
//    through LDS at the end (the same LSE algebra as the split combine);
//  - a token row of one KV head (d elements) is spread over LPR consecutive
//    lanes, each holding EPL elements loaded with one 128-bit (64-bit for
//    fp8) buffer load; one wave load covers RPL = 64 / LPR rows, a tile
//    NLD = 16 / RPL loads for K and as many for V;
//  - the per-lane partial dot products (NLD rows x GT heads) are combined
//    across the LPR lanes of a row with a reduce-scatter of DPP lane swaps,
//    leaving each lane with the full scores of VPL (row, head) pairs;
//  - the softmax probabilities are handed back to the lanes that hold the V
//    rows through a 1-2 KiB per-wave LDS slot, and the PV product
//    accumulates into GT x EPL fp32 registers per lane.
// Scores are kept in the log2 domain (q.k * scale * log2 e) so that every
// exponential is a native exp2.
//
// Addressing: each tile's K and V rows are read through a buffer resource
// whose base is the tile's first row in its physical page and whose size
// covers exactly the tile's valid rows, so rows past the context (stale
// slots of a last partial page) read as zero and are never fetched, and the
// per-lane byte offsets are loop invariant.  A wave reads the block-table
// entries of its next 64 tiles with one vector load (one entry per lane) and
// takes each tile's entry with a lane read; entries past the sequence's pages
// may be loaded that way but never address the cache.
#include "pda_device.h"

#include <type_traits>

namespace pda {
namespace {

// ------------------------------------------------------------ main kernel

template <class QT, class KT, int D, int GT>
__global__ __launch_bounds__(kGqaWaves * 64, 2) void gqa_split_kernel(GqaArgs a) {
  using frag_t = typename Elem<KT>::frag;
  constexpr int EPL = Elem<KT>::epl;
  constexpr int ESZ = Elem<KT>::bytes;
  constexpr int LPR = D / EPL;
  constexpr int RPL = 64 / LPR;
  constexpr int NLD = kTileTokens / RPL;
  constexpr int NV = NLD * GT;
  constexpr int LOG_LPR = ilog2(LPR);
  constexpr int STEPS = ilog2(NV) < LOG_LPR ? ilog2(NV) : LOG_LPR;
  constexpr int VPL = NV >> STEPS;
  constexpr int DUPBITS = LOG_LPR - STEPS;
  // Scores with packed dot2 when q and K meet in one 16-bit type (fp8 K is
  // widened to q's type, exactly: every E4M3 value is a binary16 / bfloat16
  // value); P.V with dot2 over token pairs when V widens exactly to binary16.
  constexpr bool kQf16 = std::is_same<QT, F16>::value &&
                         (std::is_same<KT, F16>::value || std::is_same<KT, E4M3>::value);
  constexpr bool kQbf16 = std::is_same<QT, BF16>::value &&
                          (std::is_same<KT, BF16>::value || std::is_same<KT, E4M3>::value);
  constexpr bool kPacked = kQf16 || kQbf16;
  // binary16 probabilities carry ~2^-12 relative error per weight: fine for a
  // binary16 output, too coarse next to the rounding of a bfloat16 output
  // at very short contexts, so bf16-q calls keep fp32 probabilities
  constexpr bool kDotPV = std::is_same<QT, F16>::value &&
                          (std::is_same<KT, F16>::value || std::is_same<KT, E4M3>::value);
  static_assert(!kDotPV || NLD % 2 == 0, "token pairs");
  static_assert(LPR * RPL == 64 && NLD * RPL == kTileTokens, "row layout");
  static_assert(VPL == (GT >= 4 ? GT / 4 : 1) && DUPBITS <= 2, "score layout");
  static_assert(LPR >= 4 && LPR <= 32, "head_dim / dtype combination");

  __shared__ f32x4 pbuf[kGqaWaves][RPL][NV / 4 > 0 ? NV / 4 : 1];
  __shared__ float m_sh[kGqaWaves][GT], l_sh[kGqaWaves][GT];
  __shared__ float acc_sh[kGqaWaves][GT][D];

  // Every kernel argument is fetched in one batch of scalar loads up front
  // (the empty asm needs them all in registers here), instead of in several
  // dependent round trips as the code below first touches them.
  asm volatile("" ::"s"(a.q), "s"(a.k_cache), "s"(a.v_cache), "s"(a.block_tables),
               "s"(a.context_lens), "s"(a.batch), "s"(a.num_q_heads), "s"(a.num_kv_heads),
               "s"(a.group), "s"(a.head_tiles), "s"(a.page_size), "s"(a.max_pages),
               "s"(a.log2_page), "s"(a.tok_stride), "s"(a.head_stride), "s"(a.page_stride), "s"(a.qk_scale_log2),
               "s"(a.split.pages_per_split), "s"(a.split.max_splits),
               "s"(a.split.split_min_tokens));
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = lane / LPR;
  const int c = lane % LPR;
  const int seg = c >> DUPBITS;
  // Per-lane order of the score array for the select-free reduce-scatter:
  // slot s holds the score of logical value s ^ flip (value v = row ordinal
  // * GT + head), where flip carries the lane bits that are exchanged with
  // DPP, each at the index bit its reduction step splits.  A value index
  // decomposes into (row ordinal, head), so the lane loads its K rows in the
  // order i ^ flip_row and its q heads in the order g ^ flip_head.
  constexpr int kLG = ilog2(GT);
  constexpr int kDppSeg = (4 - DUPBITS) < STEPS ? (4 - DUPBITS) : STEPS;
  const int flip = (seg & ((1 << kDppSeg) - 1)) * VPL;
  const int flip_row = kGqaPermuteRows ? flip >> kLG : 0;
  const int flip_head = flip & (GT - 1);
  // steps on arrays up to kPerm values use the flipped order (all of them
  // when the K rows are permuted too, else the head steps only)
  constexpr int kPerm = kGqaPermuteRows ? NV : GT;

  // which (sequence, KV head, head tile, split) this workgroup computes
  // (ordered: from the unit list, as in gqa_mfma_kernel)
  const bool ordered = a.units != nullptr;
  int tile, kvh, b, split, ut0 = 0, ut1 = 0;
  if (ordered) {
    int g;
    group_tile(blockIdx.x, gridDim.x / a.head_tiles, a.head_tiles, g, tile);
    g = __builtin_amdgcn_readfirstlane(g);  // (uniform: scalar registers)
    tile = __builtin_amdgcn_readfirstlane(tile);
    const WorkUnit w = load_unit(a.units, g / a.num_kv_heads);
    if (w.b < 0) return;
    b = w.b;
    split = w.split;
    ut0 = w.t0;
    ut1 = w.t1;
    kvh = g % a.num_kv_heads;
  } else {
    int bk;
    group_tile(blockIdx.x, gridDim.x / a.head_tiles, a.head_tiles, bk, tile);
    bk = __builtin_amdgcn_readfirstlane(bk);
    tile = __builtin_amdgcn_readfirstlane(tile);
    kvh = bk % a.num_kv_heads;
    b = bk / a.num_kv_heads;
    split = blockIdx.y;
  }

  const int g0 = tile * GT;                 // first group-local head of the tile
  const int hbase = kvh * a.group + g0;     // first query head of the tile
  const int gvalid = min(GT, a.group - g0); // heads of the tile inside the group
  const int log2P = a.log2_page;
  const int32_t* table = a.block_tables + (int64_t)b * a.max_pages;
  // First token of this split when the sequence is split (a split that ends
  // up unused exits below before anything depends on it).
  const int t0_hint = ordered                  ? ut0
                      : a.split.max_splits > 1 ? split * a.split.pages_per_split << log2P
                                               : 0;

  // The sequence length, this wave's block-table entries and q are requested
  // together, before anything waits for one of them.  Lane j holds the entry
  // of the wave's tile ordinal kbase + j; indices are clamped into the
  // sequence's table row, and entries past its pages are loaded but never
  // used.
  auto load_table = [&](int kbase) -> int {
    const int64_t tok = (int64_t)t0_hint + (int64_t)(wave + (kbase + lane) * kGqaWaves) * kTileTokens;
    const int64_t pg = tok >> log2P;
    return table[pg < a.max_pages ? pg : a.max_pages - 1];
  };
  // A split past the end of a short sequence finds out from the length,
  // requested together with its first table entries and q (entries in the
  // table row, never used then), and leaves after that one round trip.
  int n = 0;
  int vtbl = load_table(0);
  if (!ordered) n = load_uniform(a.context_lens + b);

  // q of the tile's heads (slot g holds head g ^ flip_head), the EPL elements
  // this lane multiplies.  Heads past the group are loaded from a valid row
  // (no branch around the load) and zeroed.
  uint32_t qp[GT][EPL / 2];
  float qf[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const int gh = g ^ flip_head;
    const bool hv = gh < gvalid;
    const int64_t e0 = ((int64_t)b * a.num_q_heads + hbase + (hv ? gh : 0)) * D + c * EPL;
    if constexpr (kPacked) {
      u32x4 w = *(const u32x4*)((const char*)a.q + e0 * 2);
#pragma unroll
      for (int j = 0; j < EPL / 2; ++j) qp[g][j] = hv ? (uint32_t)w[j] : 0u;
    } else {
      load_q_f32<QT, EPL>(a.q, e0, qf[g]);
#pragma unroll
      for (int j = 0; j < EPL; ++j) qf[g][j] = hv ? qf[g][j] : 0.f;
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

  // loop-invariant byte offsets of this lane's rows inside a tile (K in the
  // permuted row order of the score array, V in plain order)
  const int tok_bytes = a.tok_stride * ESZ;
  int koff[NLD], voff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) {
    koff[i] = (rg + RPL * (i ^ flip_row)) * tok_bytes + (c * EPL) * ESZ;
    voff[i] = (rg + RPL * i) * tok_bytes + (c * EPL) * ESZ;
  }

  float m_run[VPL], l_run[VPL];
  float acc[GT][EPL];
#pragma unroll
  for (int k = 0; k < VPL; ++k) {
    m_run[k] = -INFINITY;
    l_run[k] = 0.f;
  }
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = 0.f;

  const int ntiles = (t1 - t0 + kTileTokens - 1) / kTileTokens;
  // tile ordinals of this wave: tiles wave, wave + kGqaWaves, ...
  const int nt_wave = ntiles > wave ? (ntiles - wave + kGqaWaves - 1) / kGqaWaves : 0;

  // Buffer resources of tile ordinal k (tile wave + k * kGqaWaves) in physical
  // page `phys`; empty ones for dead tiles (their loads return zero without
  // touching memory).
  auto tile_rsrc = [&](int k, bool live, int phys, __amdgpu_buffer_rsrc_t& rk,
                       __amdgpu_buffer_rsrc_t& rv, int& rows) {
    const int T = wave + k * kGqaWaves;
    const int tok = t0 + T * kTileTokens;
    rows = live ? min(kTileTokens, t1 - tok) : 0;
    const int slot = tok & ((1 << log2P) - 1);
    const int64_t elem = (int64_t)(live ? phys : 0) * a.page_stride + (int64_t)slot * a.tok_stride +
                         (int64_t)kvh * a.head_stride;
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.k_cache + elem * ESZ), 0,
                                           rows * tok_bytes, kRsrcFlags);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.v_cache + elem * ESZ), 0,
                                           rows * tok_bytes, kRsrcFlags);
  };

  const float pinf = opaque_inf();
  auto compute_tile = [&](const frag_t (&kf)[NLD], const frag_t (&vf)[NLD], int rows) {
    // partial scores of this lane: NLD rows x GT heads over its EPL elements
    float sc[NV];
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      if constexpr (kPacked) {
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          float s = 0.f;
#pragma unroll
          for (int j = 0; j < EPL / 2; ++j) {
            if constexpr (kQf16) {
              s = __builtin_amdgcn_fdot2(as_f16x2(qp[g][j]), k_pair_f16(kf[i], j), s, false);
            } else {
              s = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qp[g][j]), k_pair_bf16(kf[i], j), s,
                                                  false);
            }
          }
          sc[i * GT + g] = s;
        }
      } else {
        float kv[EPL];
        to_f32(KT{}, kf[i], kv);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          float s = 0.f;
#pragma unroll
          for (int e = 0; e < EPL; ++e) s = fmaf(qf[g][e], kv[e], s);
          sc[i * GT + g] = s;
        }
      }
    }
    reduce_scatter<NV, LOG_LPR - 1, kPerm>(sc, lane);

    // this lane now holds the full scores of values seg*VPL + k.
    // Lazy running max: the reference max moves only when the tile's max
    // exceeds it by more than kLazyMax (log2 units), so p <= 2^kLazyMax and
    // the accumulators are rescaled rarely; numerator and denominator share
    // the reference, so the result is unchanged.
    float p[VPL], alpha[VPL];
    bool changed = false;
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int v = seg * VPL + k;
      const int row = rg + RPL * (v / GT);
      // (a min against +-inf masks rows past the context without a branch)
      const float s = fminf(sc[k] * a.qk_scale_log2, row < rows ? INFINITY : -INFINITY);
      const float tmax = wave_max_bits2to5(s, pinf);
      const bool move = tmax > m_run[k] + kLazyMax;
      const float m_new = move ? tmax : m_run[k];
      alpha[k] = __builtin_amdgcn_exp2f(m_run[k] - m_new);
      p[k] = __builtin_amdgcn_exp2f(s - m_new);
      // P.V runs on binary16 probabilities: round here so that the sum l uses
      // exactly the weights the numerator gets
      if constexpr (kDotPV) p[k] = (float)(_Float16)p[k];
      l_run[k] = l_run[k] * alpha[k] + p[k];
      changed |= move;
      m_run[k] = m_new;
    }
    // hand the probabilities to the lanes that hold the V rows
    float* prow = (float*)&pbuf[wave][rg][0];
#pragma unroll
    for (int k = 0; k < VPL; ++k) prow[seg * VPL + k] = p[k];
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");

    // rescale the accumulators when any running max moved
    if (__builtin_amdgcn_read_exec() & __ballot(changed)) {
#pragma unroll
      for (int g = 0; g < GT; ++g) {
        const int al_bits = __builtin_amdgcn_readlane(
            __builtin_bit_cast(int, alpha[g % VPL]), (g / VPL) << DUPBITS);
        const float al = __builtin_bit_cast(float, al_bits);
#pragma unroll
        for (int e = 0; e < EPL; ++e) acc[g][e] *= al;
      }
    }
    float pv[NV];
#pragma unroll
    for (int j = 0; j < NV / 4; ++j) {
      f32x4 t = pbuf[wave][rg][j];
      pv[4 * j] = t.x;
      pv[4 * j + 1] = t.y;
      pv[4 * j + 2] = t.z;
      pv[4 * j + 3] = t.w;
    }
    if constexpr (NV < 4) {
#pragma unroll
      for (int j = 0; j < NV; ++j) pv[j] = prow[j];
    }
    __builtin_amdgcn_wave_barrier();
    if constexpr (kDotPV) {
      // rows (2ip, 2ip + 1) of the lane: acc[g][e] += (p0, p1) . (V0[e], V1[e])
#pragma unroll
      for (int ip = 0; ip < NLD / 2; ++ip) {
        uint32_t vp[EPL];
        v_pairs(vf[2 * ip], vf[2 * ip + 1], vp);
#pragma unroll
        for (int g = 0; g < GT; ++g) {
          const f16x2 pp = __builtin_bit_cast(
              f16x2, __builtin_amdgcn_cvt_pkrtz(pv[(2 * ip) * GT + g], pv[(2 * ip + 1) * GT + g]));
#pragma unroll
          for (int e = 0; e < EPL; ++e)
            acc[g][e] = __builtin_amdgcn_fdot2(pp, as_f16x2(vp[e]), acc[g][e], false);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < NLD; ++i) {
        float vv[EPL];
        to_f32(KT{}, vf[i], vv);
#pragma unroll
        for (int g = 0; g < GT; ++g)
#pragma unroll
          for (int e = 0; e < EPL; ++e) acc[g][e] = fmaf(pv[i * GT + g], vv[e], acc[g][e]);
      }
    }
  };

  // A ring of kPF + 1 register buffers: while the tile in buffer u is
  // computed, the loads of the next kPF tiles are in flight.  The
  // ring index is a compile-time constant inside the unrolled body.
  // Deep rows (d = 256, or fp32 at d = 128) keep one tile in flight, so the
  // ring stays within ~96 registers.
  constexpr int kTileRegs = 2 * NLD * (int)(sizeof(frag_t) / 4);
  constexpr int kPF = (kGqaRingRegs / kTileRegs - 1) < 1 ? 1
                      : ((kGqaRingRegs / kTileRegs - 1) < kGqaPrefetch ? (kGqaRingRegs / kTileRegs - 1)
                                                                       : kGqaPrefetch);
  constexpr int NB = kPF + 1;
  frag_t kb[NB][NLD], vb[NB][NLD];
  int rows_b[NB];
  // Issue the loads of tile ordinal k into ring buffer u; ordinals at or past
  // kend (the end of the current 64-tile table chunk) get empty resources.
  auto issue = [&](int k, int kend, int u) {
    __amdgpu_buffer_rsrc_t rk, rv;
    const bool live = k < kend;
    const int entry = __builtin_amdgcn_readlane(vtbl, k & 63);
    const int phys = live ? entry : 0;
    tile_rsrc(k, live, phys, rk, rv, rows_b[u]);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kb[u][i] = buf_load(rk, koff[i], (frag_t*)nullptr);
      vb[u][i] = buf_load(rv, voff[i], (frag_t*)nullptr);
    }
  };
  // The wave's tiles in chunks of 64 ordinals, one table entry per lane; the
  // ring restarts at each chunk (one pipeline drain per 64 tiles of a wave).
  for (int kbase = 0; kbase < nt_wave;) {
    const int kend = min(kbase + 64, nt_wave);
    // (in order: the loop's wait counts assume the oldest tile is issued first)
#pragma unroll
    for (int u = 0; u < kPF; ++u) {
      issue(kbase + u, kend, u);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int kc = kbase;; kc += NB) {
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int k = kc + u;
        if (k >= kend) goto chunk_done;
        issue(k + kPF, kend, (u + kPF) % NB);
        compute_tile(kb[u], vb[u], rows_b[u]);
      }
    }
  chunk_done:
    kbase = kend;
    if (kbase < nt_wave) vtbl = load_table(kbase);
  }

  // ---- merge the waves' states (the split-combine algebra, in LDS)
#pragma unroll
  for (int k = 0; k < VPL; ++k) l_run[k] = wave_sum_bits2to5(l_run[k]);
#pragma unroll
  for (int g = 0; g < GT; ++g)
#pragma unroll
    for (int e = 0; e < EPL; ++e) acc[g][e] = wave_sum_from<LOG_LPR>(acc[g][e]);
  if (rg == 0) {
#pragma unroll
    for (int k = 0; k < VPL; ++k) {
      const int v = seg * VPL + k;
      if ((c & ((1 << DUPBITS) - 1)) == 0 && v < GT) {
        m_sh[wave][v] = m_run[k];
        l_sh[wave][v] = l_run[k];
      }
    }
#pragma unroll
    for (int g = 0; g < GT; ++g)
#pragma unroll
      for (int e = 0; e < EPL; ++e) acc_sh[wave][g][c * EPL + e] = acc[g][e];
  }
  __syncthreads();

  const bool final_out = nsplit == 1;
  for (int idx = threadIdx.x; idx < GT * D; idx += kGqaWaves * 64) {
    const int g = idx / D, d = idx % D;
    if (g >= gvalid) continue;
    float mx = -INFINITY;
#pragma unroll
    for (int w = 0; w < kGqaWaves; ++w) mx = fmaxf(mx, m_sh[w][g]);
    float num = 0.f, den = 0.f;
    if (mx != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kGqaWaves; ++w) {
        const float wt = exp2f(m_sh[w][g] - mx);
        num += wt * acc_sh[w][g][d];
        den += wt * l_sh[w][g];
      }
    }
    const float o = den > 0.f ? num / den * a.v_scale : 0.f;
    const float lse = den > 0.f ? (mx + __log2f(den)) * kLn2 : -INFINITY;
    const int h = hbase + g;
    const int64_t row = (int64_t)b * a.num_q_heads + h;
    if (final_out) {
      store_out<QT>(a.out, row * D + d, o);
      if (d == 0 && a.lse) a.lse[row] = lse;
    } else {
      a.part_o[(row * a.split.max_splits + split) * D + d] = o;
      if (d == 0) a.part_lse[row * a.split.max_splits + split] = lse;
    }
  }
}

// ---------------------------------------------------------------- combine

constexpr int kCombineThreads = 256;
// Split counts up to this take combine_rows_kernel (every split of a row in
// one thread), larger ones combine_kernel (a row's splits spread over threads).
#ifndef PDA_COMBINE_ROWS_MAX_SPLITS
#define PDA_COMBINE_ROWS_MAX_SPLITS 16
#endif
constexpr int kCombineRowsMaxSplits = PDA_COMBINE_ROWS_MAX_SPLITS;

// One workgroup per (sequence, query token, query head) row whose sequence
// was split and per CW-wide column chunk of it (CW = min(DV, 128)):
// L = M + ln sum_s exp(L_s - M), O = sum_s exp(L_s - M) O_s / sum_s exp(L_s - M)
// with M = max_s L_s ("From MHA to MLA" sec. 4).  Rows of unsplit sequences
// were written by the attention kernel and are skipped.  The threads form
// kCombineThreads / (CW / 4) split groups x (CW / 4) four-float chunks; each
// group weights its splits against its own maximum, and the groups are
// merged through LDS with the same algebra.  The sequence length and the
// first partials are loaded together, so a chunk costs one memory round trip
// for up to MAXL splits per group.
// The values needed before the first loads come as separate (preloaded)
// arguments ahead of CombineArgs, as in the attention kernels.
template <class OT, int DV, class PT>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(
    const void* part_o, const float* part_lse, const int32_t* context_lens, int32_t rows_per_seq,
    int32_t max_splits, int32_t pages_per_split, int32_t split_min_tokens, int32_t page_size,
    CombineArgs a) {
  constexpr int CW = DV > 128 ? 128 : DV;       // columns per workgroup
  constexpr int NCH = DV / CW;                  // column chunks per row
  constexpr int DC = CW / 4;                    // float4 chunks per workgroup
  constexpr int SG = kCombineThreads / DC;      // split groups
  constexpr int MAXL = 8;                       // splits a thread keeps in flight
  static_assert(DC * SG == kCombineThreads && NCH * CW == DV, "row width");
  __shared__ f32x4 acc_sh[SG][DC];
  __shared__ float den_sh[SG], mx_sh[SG];

  const int64_t row = blockIdx.x / NCH;  // (b, query token i, head h)
  const int chunk = blockIdx.x % NCH;
  const int b = (int)(row / rows_per_seq);
  const int S = max_splits;
  const SplitLayout sp{pages_per_split, max_splits, split_min_tokens};
  const float* pl = part_lse + row * S;
  // split s of this chunk starts at element s * DV
  using PE = typename PartElem<PT>::type;
  const PE* po = (const PE*)part_o + row * S * DV + chunk * CW + 4 * (threadIdx.x % DC);
  const int sg = threadIdx.x / DC, dc = threadIdx.x % DC;

  // In ordered calls (ragged batches) many rows belong to unsplit sequences:
  // the split count is read first and only existing partials are read.
  // Otherwise the length and this thread's first MAXL partials are requested
  // together (slots past the split count hold stale data and are ignored
  // below), so the row costs one memory round trip.
  const bool guarded = split_min_tokens > 0 || a.seq_splits;
  int n = 0, nsplit = 0, t0, t1;
  if (a.seq_splits) {  // ordered call: the planning pass recorded the count
    nsplit = load_uniform(a.seq_splits + b);
    if (nsplit <= 1) return;
  } else if (guarded) {
    n = load_uniform(context_lens + b);
    split_range(sp, n, page_size, 0, nsplit, t0, t1);
    if (nsplit <= 1) return;
  }
  const int bound = guarded ? nsplit : S;
  float l[MAXL];
  f32x4 o[MAXL];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    const int s2 = sg + j * SG;
    l[j] = s2 < bound ? pl[s2] : -INFINITY;
    o[j] = s2 < bound ? load_part4(po + (int64_t)s2 * DV) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (!guarded) {
    __builtin_amdgcn_sched_barrier(0);  // the partial loads go out before waiting for n
    n = load_uniform(context_lens + b);
    split_range(sp, n, page_size, 0, nsplit, t0, t1);
    if (nsplit <= 1) return;
  }

  // this thread's splits: local max, then weighted sums against it
  float mx = -INFINITY;
#pragma unroll
  for (int j = 0; j < MAXL; ++j)
    if (sg + j * SG < nsplit) mx = fmaxf(mx, l[j]);
  for (int s2 = sg + MAXL * SG; s2 < nsplit; s2 += SG) mx = fmaxf(mx, pl[s2]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (mx != -INFINITY) {
#pragma unroll
    for (int j = 0; j < MAXL; ++j) {
      if (sg + j * SG < nsplit && l[j] != -INFINITY) {
        const float w = __expf(l[j] - mx);
        den += w;
        acc += w * o[j];
      }
    }
    for (int s2 = sg + MAXL * SG; s2 < nsplit; s2 += SG) {
      const float ls = pl[s2];
      if (ls == -INFINITY) continue;
      const float w = __expf(ls - mx);
      den += w;
      acc += w * load_part4(po + (int64_t)s2 * DV);
    }
  }
  acc_sh[sg][dc] = acc;
  if (dc == 0) {
    den_sh[sg] = den;
    mx_sh[sg] = mx;
  }
  __syncthreads();
  // merge the split groups (each relative to its own max)
  if (threadIdx.x < DC) {
    float M = -INFINITY;
#pragma unroll
    for (int g = 0; g < SG; ++g) M = fmaxf(M, mx_sh[g]);
    f32x4 t = {0.f, 0.f, 0.f, 0.f};
    float d = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int g = 0; g < SG; ++g) {
        if (mx_sh[g] == -INFINITY) continue;
        const float w = __expf(mx_sh[g] - M);
        t += w * acc_sh[g][threadIdx.x];
        d += w * den_sh[g];
      }
    }
    const float inv = d > 0.f ? 1.f / d : 0.f;
    const int64_t o0 = row * DV + chunk * CW + threadIdx.x * 4;
    store_out<OT>(a.out, o0, t.x * inv);
    store_out<OT>(a.out, o0 + 1, t.y * inv);
    store_out<OT>(a.out, o0 + 2, t.z * inv);
    store_out<OT>(a.out, o0 + 3, t.w * inv);
    if (threadIdx.x == 0 && chunk == 0 && a.lse) {
      // lse is [B, Hq, q_len]
      const int ih = (int)(row - (int64_t)b * rows_per_seq);
      const int i = ih / a.num_q_heads, h = ih - i * a.num_q_heads;
      a.lse[((int64_t)b * a.num_q_heads + h) * a.q_len + i] = d > 0.f ? M + __logf(d) : -INFINITY;
    }
  }
}

// Combine for calls with at most MAXS splits per sequence: a workgroup takes
// kCombineThreads / (DV / 4) consecutive rows, each thread one four-column
// chunk of one row and every split of it at once (one memory round trip after
// the split count is known, no LDS, no barrier).  The same algebra as
// combine_kernel: L = M + ln sum_s exp(L_s - M), O = sum_s exp(L_s - M) O_s /
// sum_s exp(L_s - M), M = max_s L_s, in split order.
template <class OT, int DV, int MAXS, class PT>
__global__ __launch_bounds__(kCombineThreads) void combine_rows_kernel(
    const void* part_o, const float* part_lse, const int32_t* context_lens, int32_t rows_per_seq,
    int32_t max_splits, int32_t pages_per_split, int32_t split_min_tokens, int32_t page_size,
    CombineArgs a) {
  constexpr int DC = DV / 4;                  // four-float chunks per row
  constexpr int RPW = kCombineThreads / DC;   // rows per workgroup
  static_assert(RPW * DC == kCombineThreads, "row width");
  const int64_t row = (int64_t)blockIdx.x * RPW + threadIdx.x / DC;
  const int c = threadIdx.x % DC;
  const int64_t nrows = (int64_t)a.batch * rows_per_seq;
  if (row >= nrows) return;
  const int b = (int)(row / rows_per_seq);
  const int S = max_splits;
  const SplitLayout sp{pages_per_split, max_splits, split_min_tokens};
  const float* pl = part_lse + row * S;
  using PE = typename PartElem<PT>::type;
  const PE* po = (const PE*)part_o + row * S * DV + 4 * c;
  const bool guarded = split_min_tokens > 0 || a.seq_splits;
  int nsplit = S, t0, t1;
  if (a.seq_splits) {
    nsplit = load_uniform_v(a.seq_splits + b);
  } else if (guarded) {
    split_range(sp, load_uniform_v(context_lens + b), page_size, 0, nsplit, t0, t1);
  }
  if (guarded && nsplit <= 1) return;  // the attention kernel wrote this row
  float l[MAXS];
  f32x4 o[MAXS];
#pragma unroll
  for (int j = 0; j < MAXS; ++j) {
    const bool ok = j < (guarded ? nsplit : S);
    l[j] = ok ? pl[j] : -INFINITY;
    o[j] = ok ? load_part4(po + (int64_t)j * DV) : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  if (!guarded) {  // (the length comes with the partials, in the same round trip)
    split_range(sp, load_uniform_v(context_lens + b), page_size, 0, nsplit, t0, t1);
    if (nsplit <= 1) return;
  }
  float M = -INFINITY;
#pragma unroll
  for (int j = 0; j < MAXS; ++j)
    if (j < nsplit) M = fmaxf(M, l[j]);
  f32x4 acc = {0.f, 0.f, 0.f, 0.f};
  float den = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int j = 0; j < MAXS; ++j) {
      if (j < nsplit && l[j] != -INFINITY) {
        const float w = __expf(l[j] - M);
        den += w;
        acc += w * o[j];
      }
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  const int64_t o0 = row * DV + 4 * c;
  store_out<OT>(a.out, o0, acc.x * inv);
  store_out<OT>(a.out, o0 + 1, acc.y * inv);
  store_out<OT>(a.out, o0 + 2, acc.z * inv);
  store_out<OT>(a.out, o0 + 3, acc.w * inv);
  if (c == 0 && a.lse) {  // lse is [B, Hq, q_len]
    const int ih = (int)(row - (int64_t)b * rows_per_seq);
    const int i = ih / a.num_q_heads, h = ih - i * a.num_q_heads;
    a.lse[((int64_t)b * a.num_q_heads + h) * a.q_len + i] = den > 0.f ? M + __logf(den) : -INFINITY;
  }
}

// ------------------------------------------------------- work ordering

constexpr int kOrderThreads = 1024;
constexpr int kOrderStagedLens = 8192;  // sequence lengths the planning pass keeps in LDS

// The planning pass of an ordered call (one workgroup).  Each sequence is cut
// into splits -- by the SplitLayout (grid schedule), or into near-equal
// chunks of the batch's total pages (balanced schedule) -- and the resulting
// (sequence, split) work units are listed in longest-processing-time order:
// bucketed by the bit length of their token count (a counting sort, buckets
// taken from the longest down), so that the attention workgroups that start
// first get the longest ranges.  A sequence's only split is listed even when
// empty (it writes out = 0, LSE = -inf).  Order inside a bucket follows the
// LDS atomics; each unit's result does not depend on it.  The pages do not
// prescribe a schedule (FlashMLA-ETAP "Usage" shows only that one is
// computed from the sequence lengths, once per decoding step).
__global__ __launch_bounds__(kOrderThreads) void order_kernel(OrderArgs a) {
  constexpr int NBK = 33;  // bit lengths 0..32
  __shared__ int cnt[NBK];
  __shared__ int total_sh;
  __shared__ unsigned long long pages_sh;
  __shared__ int lens_sh[kOrderStagedLens];
  const int S = a.split.max_splits;
  const int64_t U = (int64_t)a.batch * S;  // (b, split) candidates; may pass 2^31
  const int P = a.page_size;
  // the lengths are read from memory once (staged in LDS up to
  // kOrderStagedLens sequences), together with the batch's page count
  const bool staged = a.batch <= kOrderStagedLens;
  if (threadIdx.x < NBK) cnt[threadIdx.x] = 0;
  if (threadIdx.x == 0) pages_sh = 0;
  __syncthreads();
  unsigned long long part = 0;
  for (int b = threadIdx.x; b < a.batch; b += kOrderThreads) {
    const int n = load_uniform_v(a.context_lens + b);
    if (staged) lens_sh[b] = n;
    part += (unsigned)((n + P - 1) / P);
  }
  if (a.balanced) {  // a wave sums its part, then one LDS atomic per wave
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) part += __shfl_xor(part, o, 64);
    if ((threadIdx.x & 63) == 0 && part) atomicAdd(&pages_sh, part);
  }
  __syncthreads();
  auto len_of = [&](int b) { return staged ? lens_sh[b] : load_uniform_v(a.context_lens + b); };
  // balanced schedule: the chunk size from the batch's total pages
  int chunk = 0;
  if (a.balanced) {
    const unsigned long long c = (pages_sh + a.target_units - 1) / a.target_units;
    chunk = (int)(c > (unsigned long long)a.min_chunk_pages ? c : a.min_chunk_pages);
  }
  // splits of sequence b (n tokens) and the pages each one covers
  auto layout = [&](int n, int& ns, int& pps) {
    const int pages = (n + P - 1) / P;
    if (S <= 1 || n <= a.split.split_min_tokens || (a.balanced && pages <= chunk)) {
      ns = 1;
      pps = pages > 0 ? pages : 1;
    } else if (!a.balanced) {
      pps = a.split.pages_per_split;
      ns = (pages + pps - 1) / pps;
    } else {
      ns = min(S, (pages + chunk - 1) / chunk);
      pps = (pages + ns - 1) / ns;
      ns = (pages + pps - 1) / pps;
    }
  };
  // unit u = (b, s): its token range, or false past the sequence's splits
  auto unit_of = [&](int64_t u, WorkUnit& w, int& ns) -> bool {
    const int b = (int)(u / S), s = (int)(u % S);
    const int n = len_of(b);
    int pps;
    layout(n, ns, pps);
    if (s >= ns) return false;
    w.b = b;
    w.split = ns == 1 ? -1 : s;
    w.t0 = s * pps * P;
    w.t1 = (int)min((int64_t)(s + 1) * pps * P, (int64_t)n);
    return true;
  };
  auto bucket = [](const WorkUnit& w) {
    const int tok = w.t1 - w.t0;
    return tok > 0 ? 32 - __clz(tok) : 0;
  };
  for (int64_t u = threadIdx.x; u < U; u += kOrderThreads) {
    WorkUnit w;
    int ns;
    if (unit_of(u, w, ns)) {
      atomicAdd(&cnt[bucket(w)], 1);
      if (u % S == 0) a.seq_splits[u / S] = ns;
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) {  // bucket offsets, longest bucket first
    int pos = 0;
    for (int k = NBK - 1; k >= 0; --k) {
      const int c = cnt[k];
      cnt[k] = pos;
      pos += c;
    }
    total_sh = pos;
  }
  __syncthreads();
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  for (int64_t u = threadIdx.x; u < U; u += kOrderThreads) {
    WorkUnit w;
    int ns;
    if (unit_of(u, w, ns)) {
      const int slot = atomicAdd(&cnt[bucket(w)], 1);
      if (slot < a.capacity) *(i32x4*)(a.units + 4 * slot) = i32x4{w.b, w.split, w.t0, w.t1};
    }
  }
  for (int u = total_sh + threadIdx.x; u < a.capacity; u += kOrderThreads)
    *(i32x4*)(a.units + 4 * u) = i32x4{-1, -1, 0, 0};
}

template <class QT, class KT, int D>
hipError_t launch_d(const GqaArgs& a, int tile_heads, int max_splits, hipStream_t s) {
  const unsigned units = (unsigned)(a.batch * a.num_kv_heads * a.head_tiles);
  const unsigned nhu = (unsigned)(a.num_kv_heads * a.head_tiles);
  dim3 grid(a.units ? nhu * (unsigned)a.unit_count : units, a.units ? 1u : (unsigned)max_splits);
  dim3 block(kGqaWaves * 64);
  switch (tile_heads) {
    case 1: hipLaunchKernelGGL((gqa_split_kernel<QT, KT, D, 1>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((gqa_split_kernel<QT, KT, D, 2>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((gqa_split_kernel<QT, KT, D, 4>), grid, block, 0, s, a); break;
    case 8: hipLaunchKernelGGL((gqa_split_kernel<QT, KT, D, 8>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <class QT, class KT>
hipError_t launch_qk(const GqaArgs& a, int head_dim, int tile_heads, int max_splits,
                     hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<QT, KT, 64>(a, tile_heads, max_splits, s);
    case 128: return launch_d<QT, KT, 128>(a, tile_heads, max_splits, s);
    case 256:
      if constexpr (!std::is_same<KT, F32>::value)
        return launch_d<QT, KT, 256>(a, tile_heads, max_splits, s);
      return hipErrorInvalidValue;
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

bool gqa_supported(int q_dtype, int kv_dtype, int head_dim, int head_dim_v) {
  if (head_dim != head_dim_v) return false;
  const bool pair_ok = (q_dtype == 0 && kv_dtype == 0) || (q_dtype == 1 && kv_dtype == 1) ||
                       (q_dtype == 2 && kv_dtype == 2) ||
                       ((q_dtype == 1 || q_dtype == 2) && kv_dtype == 3);
  if (!pair_ok) return false;
  if (head_dim == 64 || head_dim == 128) return true;
  return head_dim == 256 && kv_dtype != 0;
}

int gqa_tile_heads(int group) {
  if (group >= 8) return 8;
  if (group > 2) return group > 4 ? 8 : 4;
  return group;  // 1 or 2
}

hipError_t launch_gqa(const GqaArgs& a, int q_dtype, int kv_dtype, int head_dim,
                      int tile_heads, int max_splits, hipStream_t s) {
  if (q_dtype == 0 && kv_dtype == 0) return launch_qk<F32, F32>(a, head_dim, tile_heads, max_splits, s);
  if (q_dtype == 1 && kv_dtype == 1) return launch_qk<F16, F16>(a, head_dim, tile_heads, max_splits, s);
  if (q_dtype == 2 && kv_dtype == 2) return launch_qk<BF16, BF16>(a, head_dim, tile_heads, max_splits, s);
  if (q_dtype == 1 && kv_dtype == 3) return launch_qk<F16, E4M3>(a, head_dim, tile_heads, max_splits, s);
  if (q_dtype == 2 && kv_dtype == 3) return launch_qk<BF16, E4M3>(a, head_dim, tile_heads, max_splits, s);
  return hipErrorInvalidValue;
}

// Rows kernel for up to MAXS splits (rows of DV columns, RPW per workgroup).
template <class OT, int DV, class PT>
hipError_t launch_combine_rows(const CombineArgs& a, hipStream_t s) {
  constexpr int RPW = kCombineThreads / (DV / 4);
  const int64_t rows = (int64_t)a.batch * a.q_len * a.num_q_heads;
  dim3 grid((unsigned)((rows + RPW - 1) / RPW));
  dim3 block(kCombineThreads);
#define PDA_COMBINE_ARGS                                                                    \
  a.part_o, a.part_lse, a.context_lens, a.q_len * a.num_q_heads, a.split.max_splits,       \
      a.split.pages_per_split, a.split.split_min_tokens, a.page_size, a
  if (a.split.max_splits <= 8)
    hipLaunchKernelGGL((combine_rows_kernel<OT, DV, 8, PT>), grid, block, 0, s, PDA_COMBINE_ARGS);
  else
    hipLaunchKernelGGL((combine_rows_kernel<OT, DV, 16, PT>), grid, block, 0, s, PDA_COMBINE_ARGS);
  return hipGetLastError();
}

template <class OT, class PT>
hipError_t launch_combine_t(const CombineArgs& a, hipStream_t s) {
  // rows kernel: few splits and enough rows for at least 64 workgroups (with
  // fewer rows, one workgroup per row and its splits spread over the threads
  // finish sooner: B=4 at 32768 tokens, 16 splits, 84.5 against 85.2 us)
  const int64_t row_wgs = (int64_t)a.batch * a.q_len * a.num_q_heads * a.head_dim_v / 4 /
                          kCombineThreads;
  if (a.split.max_splits <= kCombineRowsMaxSplits && row_wgs >= 64) {
    switch (a.head_dim_v) {
      case 64: return launch_combine_rows<OT, 64, PT>(a, s);
      case 128: return launch_combine_rows<OT, 128, PT>(a, s);
      case 256: return launch_combine_rows<OT, 256, PT>(a, s);
      case 512: return launch_combine_rows<OT, 512, PT>(a, s);
      default: return hipErrorInvalidValue;
    }
  }
  const int nch = a.head_dim_v > 128 ? a.head_dim_v / 128 : 1;
  dim3 grid((unsigned)(a.batch * a.q_len * a.num_q_heads * nch));
  dim3 block(kCombineThreads);
  switch (a.head_dim_v) {
    case 64: hipLaunchKernelGGL((combine_kernel<OT, 64, PT>), grid, block, 0, s, PDA_COMBINE_ARGS); break;
    case 128: hipLaunchKernelGGL((combine_kernel<OT, 128, PT>), grid, block, 0, s, PDA_COMBINE_ARGS); break;
    case 256: hipLaunchKernelGGL((combine_kernel<OT, 256, PT>), grid, block, 0, s, PDA_COMBINE_ARGS); break;
    case 512: hipLaunchKernelGGL((combine_kernel<OT, 512, PT>), grid, block, 0, s, PDA_COMBINE_ARGS); break;
    default: return hipErrorInvalidValue;
  }
#undef PDA_COMBINE_ARGS
  return hipGetLastError();
}

hipError_t launch_order(const OrderArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(order_kernel, dim3(1), dim3(kOrderThreads), 0, s, a);
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int out_dtype, bool part_f16, hipStream_t s) {
  if (part_f16) {
    if (out_dtype == 2) return launch_combine_t<BF16, F16>(a, s);
    return hipErrorInvalidValue;
  }
  switch (out_dtype) {
    case 0: return launch_combine_t<F32, F32>(a, s);
    case 1: return launch_combine_t<F16, F32>(a, s);
    case 2: return launch_combine_t<BF16, F32>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pda
