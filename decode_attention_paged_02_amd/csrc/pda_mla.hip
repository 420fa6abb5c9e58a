// pda_mla.hip -- MLA latent decode on gfx950 ("From MHA to MLA" sec. 6;
// "Attention Kernel Variants", MLA section; FlashMLA-ETAP "Method").
//
// One cached record per token, [c (512) | k_R (64)] in bf16, shared by every
// query head: K_j is the whole 576-wide record and V_j its first 512 values.
// A workgroup owns one sequence (or one split of its pages) and a tile of up
// to 16 query heads, and walks the range in blocks of 32 tokens staged in LDS
// (double-buffered; rows past the context read as zero through a buffer
// resource sized to the valid rows).
//
// Two kernels compute the same thing:
//
//  mla_mfma_kernel -- bf16 matrix cores with the keys on the M dimension
//    (the transposed pipeline of FlashMLA-ETAP).  Per 16-key half-block each
//    wave forms S^T = K Q^T (16 keys x 16 heads, 18 MFMA 16x16x32 over the
//    576-wide record, K read from LDS, Q^T held in registers).  The MFMA
//    result puts one head per lane column and four keys per lane, which is
//    exactly the B-operand layout of a 16x16x16 MFMA with the keys as the
//    contraction, so P^T feeds O^T += V^T P^T without moving between lanes.
//    V^T comes from LDS with the gfx950 transposing read (ds_read_b64_tr_b16),
//    one read per 16x16 operand.  Every wave computes the same S^T and softmax
//    (so the running max agrees bitwise) and owns 128 of the 512 output
//    columns, so the waves never merge.  On CDNA the 16-row MFMA needs no
//    query padding, so the ETAP motivation (Hopper's 64-row WGMMA minimum)
//    does not apply; the layout is kept because the softmax reduction then
//    lands on two lane swaps and the probabilities need no exchange.
//
//  mla_valu_kernel -- plain dot products on the vector ALUs (packed bf16 dot2
//    for the scores, fp32 FMA for P V), the reference the MFMA path is
//    measured against.
//
// Both keep the online softmax in the log2 domain with a lazily moved
// reference max (see the GQA kernel) and write either the final bf16 output
// or normalized fp32 partials + LSE for the split combine.
//
// Multi-token decode (mla_mfma_kernel only): the 16 MFMA columns of a tile
// are (query token, head) rows, row i * Hq + h for query token i of q_len,
// and each column masks the tokens its query token may not see (causal:
// query i sees the first n - (q_len - 1 - i) tokens).  When a sequence has
// more than 16 rows (q_len * Hq > 16), a workgroup of two four-wave groups
// carries 32 rows over every staged block: each group computes its own 16
// columns from the shared LDS block, so the cache is read once per 32 rows
// rather than once per 16.
#include "pda_device.h"

namespace pda {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short ldsv4s __attribute__((__vector_size__(4 * sizeof(short))));

constexpr int kHeads = 16;          // query heads per workgroup tile
constexpr int kBlock = 32;          // tokens per LDS block
constexpr int kThreads = 256;       // 4 waves: one column group of 16 rows
constexpr int kLoadPolicy = 2;      // non-temporal: each record is read once per row tile

// Widths of the cached record (K: latent + rope) and of its value prefix (V):
// (576, 512) for a 512-wide latent, (320, 256) for a 256-wide one (FlashMLA-
// ETAP "Supported configurations", head dimensions).
template <int REC, int DV>
struct Dims {
  static constexpr int kRec = REC, kDv = DV;
  static constexpr int kRowBytes = REC * 2;          // one record per LDS row (bf16)
  static constexpr int kRowChunks = kRowBytes / 16;  // 16-byte chunks, swizzled
  static constexpr int kBlockChunks = kBlock * kRowChunks;
  static constexpr int kQkChunks = REC / 32;         // 32-wide contraction chunks of a score
  static constexpr int kColsPerWave = DV / 4;        // value columns a wave owns
  static constexpr int kMB = kColsPerWave / 16;      // 16-row MFMA tiles of them
  static_assert(kRowChunks % 8 == 0 && REC % 32 == 0 && DV % 64 == 0, "record widths");
};
typedef Dims<576, 512> Dims576;
typedef Dims<320, 256> Dims320;

__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }
// max / sum over the four lanes {l, l^16, l^32, l^48}
__device__ __forceinline__ float max_x4(float x) {
  float a, b;
  swap16(x, x, a, b);
  x = fmaxf(a, b);
  swap32(x, x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float sum_x4(float x) {
  float a, b;
  swap16(x, x, a, b);
  x = a + b;
  swap32(x, x, a, b);
  return a + b;
}

// LDS placement of 16-byte chunk c of row r: the chunk index is XORed with a
// permutation of r mod 8 inside its aligned group of eight (rows hold 72 or
// 40 chunks, multiples of 8), so eight consecutive rows read at one chunk hit
// distinct banks, and so do four consecutive rows reading an aligned chunk
// pair (the transposing V reads).
__device__ __forceinline__ int swz(int r) { return ((r & 3) << 1) | ((r >> 2) & 1); }
template <class DM>
__device__ __forceinline__ int lds_off(int r, int c) {
  return r * DM::kRowBytes + 16 * (c ^ swz(r));
}

// Block-table entries of a workgroup's range, one per lane: lane j holds the
// entry of page base + j (clamped into the table row; entries past the
// sequence are loaded but never used).  A block's page is then a lane read.
struct PageTable {
  const int32_t* row;
  int max_pages, base, entries;

  __device__ __forceinline__ void load(int page0, int lane) {
    base = page0;
    const int p = min(page0 + lane, max_pages - 1);
    entries = row[p];
  }
  // entry of page p (p >= base); moves the window when p is past it.  The
  // moved window is waited for inside the branch, so the common path reads
  // the lane without waiting on the block loads in flight.
  __device__ __forceinline__ int entry(int p, int lane) {
    if (p - base >= 64) {
      load(p, lane);
      asm volatile("" ::"v"(entries));
    }
    return __builtin_amdgcn_readlane(entries, p - base);
  }
};

// Shared block staging: the workgroup's T threads bring one block of 32
// records into registers, then into LDS as bf16 rows: 16-byte loads of a
// bf16 latent (36 KiB per block), or 8-byte loads of an fp8 latent (18 KiB),
// each widened exactly to the same 16-byte bf16 LDS chunk.  With T = 512 the
// last load of a thread may lie past the block: its offset is outside the
// buffer resource (zero, no memory access) and it is not stored.
template <int T, class KT, class DM>
struct BlockLoader {
  static constexpr bool kFp8 = std::is_same<KT, E4M3>::value;
  static constexpr int kBlockChunks = DM::kBlockChunks, kRowChunks = DM::kRowChunks;
  static constexpr int kRecBytes = kFp8 ? DM::kRec : 2 * DM::kRec;  // a record in memory
  static constexpr int kN = (kBlockChunks + T - 1) / T;              // loads per thread
  typedef typename std::conditional<kFp8, u32x2, u32x4>::type piece_t;
  piece_t r[kN];

  // Load block `blk` of the range [t0, t1) (tokens t0 + 32 blk ...).  Rows
  // past t1 (and a block past the range) read as zero without memory access.
  __device__ __forceinline__ void load(const MlaArgs& a, PageTable& pt, int t0, int t1, int blk,
                                       int log2P, int tid) {
    const int tok = t0 + blk * kBlock;
    // (uniform; read into a scalar register so the resource stays scalar)
    const int rows = __builtin_amdgcn_readfirstlane(max(0, min(kBlock, t1 - tok)));
    // (blocks past the range look up the range's last page and load nothing)
    const int e = pt.entry(min(tok, t1 - 1) >> log2P, tid & 63);
    const int phys = rows > 0 ? e : 0;
    const int slot = tok & ((1 << log2P) - 1);
    const int64_t rec0 = (int64_t)phys * a.page_size + slot;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        (void*)((const char*)a.kv_cache + rec0 * kRecBytes), 0, rows * kRecBytes, kRsrcFlags);
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      if constexpr (kFp8)
        r[i] = __builtin_amdgcn_raw_buffer_load_b64(rs, (tid + i * T) * 8, 0, kLoadPolicy);
      else
        r[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (tid + i * T) * 16, 0, kLoadPolicy);
    }
  }

  __device__ __forceinline__ void store(char* lds, int tid) const {
#pragma unroll
    for (int i = 0; i < kN; ++i) {
      const int q = tid + i * T;
      if (kN * T == kBlockChunks || q < kBlockChunks) {
        const int row = q / kRowChunks, col = q % kRowChunks;
        u32x4 w;
        if constexpr (kFp8) {
          // bytes 0..7 -> bf16 pairs (0, 1), (2, 3), (4, 5), (6, 7); every
          // E4M3 value is a bf16 value, the conversion is exact
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            w[2 * h] = __builtin_bit_cast(uint32_t,
                                          __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[i][h], 1.0f, false));
            w[2 * h + 1] = __builtin_bit_cast(uint32_t,
                                              __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(r[i][h], 1.0f, true));
          }
        } else {
          w = r[i];
        }
        *(u32x4*)(lds + lds_off<DM>(row, col)) = w;
      }
    }
  }
};

template <int WHICH>
__device__ __forceinline__ void store_bf16x4(void* out, int64_t i, f32x4 v) {
  const uint32_t lo = __builtin_bit_cast(uint16_t, (__bf16)v.x) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.y) << 16);
  const uint32_t hi = __builtin_bit_cast(uint16_t, (__bf16)v.z) |
                      ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)v.w) << 16);
  uint2 w;
  w.x = lo;
  w.y = hi;
  *(uint2*)((char*)out + i * 2) = w;
}

// ------------------------------------------------------------ MFMA kernel

// NG column groups of four waves; a workgroup owns 16 NG rows.  KT: the
// latent's storage type (BF16, or E4M3 with a dequantization scale); DM: the
// record widths.  QM: queries on the MFMA M dimension instead of the keys
// (FlashMLA's own layout): S = Q K^T with Q the A operand (rows of the tile)
// and K the B operand (16 keys), then O = P V with P the A operand and V the
// B operand.  The four waves' shares of S go through LDS as a [row][key]
// tile and are read back one row per lane, which is the softmax layout of the
// keys-on-M pipeline, so the softmax and the P operand are the same
// registers; the accumulator then holds rows 4 grp + i of 16 value columns,
// and the rescale factors and 1 / l of those rows come from the rows' lanes.
template <int NG, class KT, class DM, bool QM>
__global__ __launch_bounds__(kThreads * NG, 2 / NG) void mla_mfma_kernel(MlaArgs a) {
  constexpr int T = kThreads * NG;
  constexpr int kRec = DM::kRec, kDv = DM::kDv;
  constexpr int QC = DM::kQkChunks;      // contraction chunks of a score
  constexpr int NWMAX = (QC + 3) / 4;    // most chunks a wave contracts
  constexpr int MB = DM::kMB;            // 16-column MFMA tiles of a wave's values
  constexpr int CPW = DM::kColsPerWave;  // value columns a wave owns
  __shared__ __attribute__((aligned(16))) char lds[2][kBlock * DM::kRowBytes];
  // per-wave partial S^T of a block (QM: a [16 rows][32 keys] float tile in
  // the same bytes, 4-key groups placed at group ^ (row % 8))
  __shared__ f32x4 spart[4 * NG][2][64];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int cg = wid >> 2;        // column group: rows 16 cg .. 16 cg + 15 of the tile
  const int wave = wid & 3;       // wave within the group
  const int col = lane & 15;      // MFMA column: the row
  const int grp = lane >> 4;      // lane group: rows 4*grp..4*grp+3 of an MFMA tile

  // (ordered: the unit list gives (sequence, split, token range), see
  // WorkUnit)
  const bool ordered = a.units != nullptr;
  int tile, b, split, ut0 = 0, ut1 = 0;
  if (ordered) {
    int u;  // head tiles of one unit on one XCD (group_tile)
    group_tile(blockIdx.x, gridDim.x / a.head_tiles, a.head_tiles, u, tile);
    u = __builtin_amdgcn_readfirstlane(u);
    tile = __builtin_amdgcn_readfirstlane(tile);
    const WorkUnit w = load_unit(a.units, u);
    if (w.b < 0) return;
    b = w.b;
    split = w.split;
    ut0 = w.t0;
    ut1 = w.t1;
  } else {
    group_tile(blockIdx.x, gridDim.x / a.head_tiles, a.head_tiles, b, tile);
    b = __builtin_amdgcn_readfirstlane(b);
    tile = __builtin_amdgcn_readfirstlane(tile);
    split = blockIdx.y;
  }
  // One batch of kernel-argument loads; then the sequence length, the
  // range's block-table entries and q are requested together (a split past
  // the end of a short sequence finds out from the length and leaves after
  // that one round trip; the entries it loaded lie in the table row).
  asm volatile("" ::"s"(a.q), "s"(a.kv_cache), "s"(a.block_tables), "s"(a.context_lens),
               "s"(a.num_q_heads), "s"(a.head_tiles), "s"(a.page_size), "s"(a.max_pages),
               "s"(a.log2_page), "s"(a.qk_scale_log2), "s"(a.split.pages_per_split),
               "s"(a.split.max_splits), "s"(a.split.split_min_tokens), "s"(a.q_len));
  const int log2P = a.log2_page;
  PageTable pt{a.block_tables + (int64_t)b * a.max_pages, a.max_pages, 0, 0};
  pt.load(ordered                  ? ut0 >> log2P
          : a.split.max_splits > 1 ? split * a.split.pages_per_split
                                   : 0,
          lane);
  int n = load_uniform(a.context_lens + b);

  // this lane's column: row r = query token qi, head h (rows past the last
  // one compute on zero queries and are not written)
  const int q_len = a.q_len;
  const int r = tile * (kHeads * NG) + kHeads * cg + col;
  const bool hvalid = r < q_len * a.num_q_heads;
  int qi = 0, h = r;
  if (q_len > 1) {
    qi = r / a.num_q_heads;
    h = r - qi * a.num_q_heads;
  }
  // The QC chunks of 32 record values are shared out over the waves (18:
  // 5, 5, 4, 4; 10: 3, 3, 2, 2): wave w contracts chunks [c_lo, c_lo + n_w)
  // of every key and the four partial S^T are summed through LDS in a fixed
  // order.
  const int n_w = QC / 4 + (wave < QC % 4 ? 1 : 0);
  const int c_lo = wave * (QC / 4) + min(wave, QC % 4);
  // Q^T as the B operand: lane (col, grp) holds q[h][32 (c_lo + j) + 8 grp + 0..7]
  // (loaded from valid addresses without branches, then zeroed where unused)
  bf16x8 qb[NWMAX];
  {
    const uint16_t* qrow =
        (const uint16_t*)a.q +
        (hvalid ? (((int64_t)b * q_len + qi) * a.num_q_heads + h) * kRec : 0);
#pragma unroll
    for (int j = 0; j < NWMAX; ++j) {
      const bool use = hvalid && j < n_w;
      const u32x4 w = *(const u32x4*)(qrow + 32 * (c_lo + (j < n_w ? j : 0)) + 8 * grp);
      qb[j] = __builtin_bit_cast(bf16x8, use ? w : u32x4{0u, 0u, 0u, 0u});
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
  const int nblocks = (t1 - t0 + kBlock - 1) / kBlock;
  // end of the tokens this column's query token may see (t1 without a mask)
  const int lim = min(t1, a.causal ? n - (q_len - 1 - qi) : n);

  f32x4 acc[MB];  // O^T rows CPW*wave + 16*mb + 4*grp + i, column = head
#pragma unroll
  for (int mb = 0; mb < MB; ++mb) acc[mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float m_run = kMaxStart, l_run = 0.f;

  // kRing blocks in flight in registers while one is computed from LDS.
  // With one (four-wave workgroups, two per CU), block k + 1 is loaded while
  // block k is computed and staged right after; with two (the 512-thread
  // workgroups, one per CU), block k sits in ld[k % 2] until it is staged and
  // the loads of block k + 2 go into the registers it leaves.  Fewer loads in
  // flight contend less where two workgroups share a CU (bf16 record 195
  // against 200 us, (320, 256) 119 against 121); the lone 512-thread
  // workgroup keeps two (a deeper ring measured no gain, a shallower one
  // 1% less).  Loads of blocks past the range have empty resources (no
  // memory access), so they need no branch.
  constexpr int kRing = NG == 1 ? 1 : 2;
  BlockLoader<T, KT, DM> ld[kRing];
  ld[0].load(a, pt, t0, t1, 0, log2P, tid);
  ld[0].store(lds[0], tid);
  ld[kRing - 1].load(a, pt, t0, t1, 1, log2P, tid);
  if constexpr (kRing == 2) ld[0].load(a, pt, t0, t1, 2, log2P, tid);
  __syncthreads();

  // block blk from LDS
  auto compute = [&](int blk) {
    const char* L = lds[blk & 1];
    const int rows = min(kBlock, lim - (t0 + blk * kBlock));  // per column

    // this wave's share of S^T for the two 16-key halves, then the sum of the
    // four shares (every wave adds them in the same order: identical S^T)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      f32x4 sp = {0.f, 0.f, 0.f, 0.f};
      const int r = 16 * kb + col;
#pragma unroll
      for (int j = 0; j < NWMAX; ++j) {
        if (j < n_w) {
          const bf16x8 kv = *(const bf16x8*)(L + lds_off<DM>(r, 4 * (c_lo + j) + grp));
          if constexpr (QM)  // S = Q K^T: rows 4 grp + i, key 16 kb + col
            sp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(qb[j], kv, sp, 0, 0, 0);
          else               // S^T = K Q^T: keys 16 kb + 4 grp + i, row col
            sp = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kv, qb[j], sp, 0, 0, 0);
        }
      }
      if constexpr (QM) {
        float* sq = (float*)&spart[wid][0][0];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int row = 4 * grp + i, kg = 4 * kb + (col >> 2);
          sq[row * 32 + 4 * (kg ^ (row & 7)) + (col & 3)] = sp[i];
        }
      } else {
        spart[wid][kb][lane] = sp;
      }
    }
    __syncthreads();
    f32x4 st[2];
    const int w0 = 4 * cg;  // the group's four shares
    if constexpr (QM) {
      // row col, keys 16 kb + 4 grp + 0..3 (the keys-on-M layout), summed over
      // the four shares in the same order
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const int off = col * 32 + 4 * ((4 * kb + grp) ^ (col & 7));
        const f32x4* s0 = (const f32x4*)((const float*)&spart[w0][0][0] + off);
        const f32x4* s1 = (const f32x4*)((const float*)&spart[w0 + 1][0][0] + off);
        const f32x4* s2 = (const f32x4*)((const float*)&spart[w0 + 2][0][0] + off);
        const f32x4* s3 = (const f32x4*)((const float*)&spart[w0 + 3][0][0] + off);
        st[kb] = ((*s0 + *s1) + *s2) + *s3;
      }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        st[kb] = ((spart[w0][kb][lane] + spart[w0 + 1][kb][lane]) + spart[w0 + 2][kb][lane]) +
                 spart[w0 + 3][kb][lane];
    }
    // scale, mask rows past the context; lane holds keys 16 kb + 4 grp + i of head `col`
    // (a block whose 32 rows every column sees skips the mask: one wave vote)
    float s[8];
    float tmax = -INFINITY;
    if (__builtin_amdgcn_ballot_w64(rows < kBlock) == 0) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          s[kb * 4 + i] = st[kb][i] * a.qk_scale_log2;
          tmax = fmaxf(tmax, s[kb * 4 + i]);
        }
    } else {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int key = 16 * kb + 4 * grp + i;
          const float v = key < rows ? st[kb][i] * a.qk_scale_log2 : -INFINITY;
          s[kb * 4 + i] = v;
          tmax = fmaxf(tmax, v);
        }
    }
    tmax = max_x4(tmax);
    if constexpr (QM) {
      // per row; the accumulator rows 4 grp + i take their factors from the
      // rows' lanes (only when some row's reference moved)
      const bool move = tmax > m_run + kLazyMax;
      float alpha = 1.f;
      if (move) {
        alpha = __builtin_amdgcn_exp2f(m_run - tmax);
        m_run = tmax;
        l_run *= alpha;
      }
      if (__builtin_amdgcn_ballot_w64(move)) {
        float al[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) al[i] = __shfl(alpha, 4 * grp + i, 64);
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[mb][i] *= al[i];
      }
    } else if (tmax > m_run + kLazyMax) {  // per head; lanes of one head agree
      const float alpha = __builtin_amdgcn_exp2f(m_run - tmax);
      m_run = tmax;
      l_run *= alpha;
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) acc[mb] *= alpha;
    }
    // P^T as the B operand of the PV MFMA, split into two bf16 terms
    // p = p_hi + p_lo (bf16 alone would leave a 2^-9 relative error per
    // weight); both terms multiply the same V^T operand.
    s16x4 pb_hi[2], pb_lo[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float p = __builtin_amdgcn_exp2f(s[kb * 4 + i] - m_run);
        l_run += p;
        const __bf16 hi = (__bf16)p;
        const __bf16 lo = (__bf16)(p - (float)hi);
        pb_hi[kb][i] = __builtin_bit_cast(short, hi);
        pb_lo[kb][i] = __builtin_bit_cast(short, lo);
      }
    // O^T += V^T P^T over this wave's CPW value columns, one 16x16x32 MFMA
    // per term over all 32 keys of the block.  The contraction index k of
    // lane group g covers keys 4 g + 0..3 (k = 8 g + 0..3) and 16 + 4 g + 0..3
    // (k = 8 g + 4..7): that is where the S^T layout left this lane's
    // probabilities, and the two transposing reads below give the V^T
    // operand the same key order (a sum over k does not depend on it).
    const bf16x8 pk_hi = __builtin_bit_cast(bf16x8, __builtin_shufflevector(
                                                        pb_hi[0], pb_hi[1], 0, 1, 2, 3, 4, 5, 6, 7));
    const bf16x8 pk_lo = __builtin_bit_cast(bf16x8, __builtin_shufflevector(
                                                        pb_lo[0], pb_lo[1], 0, 1, 2, 3, 4, 5, 6, 7));
    bf16x8 va[MB];
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      s16x4 vt[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        // transposing read: lane q of group g points at key 16 kb + 4 g + q/4,
        // column CPW wave + 16 mb + 4 (q % 4); it returns V^T rows 16 mb + q
        // (value columns) x keys 16 kb + 4 g + 0..3
        const int q = col;
        const int r = 16 * kb + 4 * grp + (q >> 2);
        const int byte = (CPW * wave + 16 * mb + 4 * (q & 3)) * 2;
        const char* p = L + lds_off<DM>(r, byte >> 4) + (byte & 15);
        vt[kb] = __builtin_bit_cast(s16x4, __builtin_amdgcn_ds_read_tr16_b64_v4i16(
                                               (__attribute__((address_space(3))) ldsv4s*)(p)));
      }
      va[mb] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(vt[0], vt[1], 0, 1, 2, 3, 4, 5,
                                                                  6, 7));
    }
    if constexpr (QM) {  // O = P V: rows 4 grp + i, value column col of tile mb
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pk_hi, va[mb], acc[mb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(pk_lo, va[mb], acc[mb], 0, 0, 0);
    } else {
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mb], pk_hi, acc[mb], 0, 0, 0);
#pragma unroll
      for (int mb = 0; mb < MB; ++mb)
        acc[mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[mb], pk_lo, acc[mb], 0, 0, 0);
    }
  };
  // block blk, then: stage the next block, start loading the one 1 + kRing
  // ahead, hand over the buffer (`nxt` holds block blk + 1 and then receives
  // blk + 1 + kRing).  No branches around loads and stores (nor exits from the
  // unrolled pair): the wait counts then stay exact across iterations, and a
  // block past the range is all zero rows (an odd block count computes one
  // such block, fully masked).
  auto body = [&](int blk, BlockLoader<T, KT, DM>& nxt) {
    compute(blk);
    nxt.store(lds[(blk + 1) & 1], tid);
    nxt.load(a, pt, t0, t1, blk + 1 + kRing, log2P, tid);
    __syncthreads();
  };
  for (int blk = 0; blk < nblocks; blk += 2) {
    body(blk, ld[kRing - 1]);
    body(blk + 1, ld[0]);
  }

  // epilogue: l over the four lane groups; lane holds 4 consecutive columns
  // (out row (b, qi, h); lse [B, Hq, q_len])
  const float l = sum_x4(l_run);
  if constexpr (QM) {
    // lane: rows 4 grp + i of value column col of each tile mb; their 1 / l
    // from the rows' lanes (every lane takes part in the exchange)
    const float inv_row = l > 0.f ? a.v_scale / l : 0.f;
    float inv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) inv[i] = __shfl(inv_row, 4 * grp + i, 64);
    const int nrows = q_len * a.num_q_heads;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ri = tile * (kHeads * NG) + kHeads * cg + 4 * grp + i;
      if (ri >= nrows) continue;
      int qi_i = 0, h_i = ri;
      if (q_len > 1) {
        qi_i = ri / a.num_q_heads;
        h_i = ri - qi_i * a.num_q_heads;
      }
      const int64_t row_i = ((int64_t)b * q_len + qi_i) * a.num_q_heads + h_i;
      if (nsplit == 1) {
#pragma unroll
        for (int mb = 0; mb < MB; ++mb)
          store_out<BF16>(a.out, row_i * kDv + CPW * wave + 16 * mb + col, acc[mb][i] * inv[i]);
      } else {
        _Float16* po = (_Float16*)a.part_o + (row_i * a.split.max_splits + split) * kDv + CPW * wave + col;
#pragma unroll
        for (int mb = 0; mb < MB; ++mb) po[16 * mb] = (_Float16)(acc[mb][i] * inv[i]);
      }
    }
    if (!hvalid || wave != 0 || grp != 0) return;
    const float lse = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
    const int64_t row = ((int64_t)b * q_len + qi) * a.num_q_heads + h;
    if (nsplit == 1) {
      if (a.lse) a.lse[((int64_t)b * a.num_q_heads + h) * q_len + qi] = lse;
    } else {
      a.part_lse[row * a.split.max_splits + split] = lse;
    }
    return;
  }
  if (!hvalid) return;
  const float inv = l > 0.f ? a.v_scale / l : 0.f;
  const float lse = l > 0.f ? (m_run + __log2f(l)) * kLn2 : -INFINITY;
  const int64_t row = ((int64_t)b * q_len + qi) * a.num_q_heads + h;
  if (nsplit == 1) {
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
      store_bf16x4<0>(a.out, row * kDv + CPW * wave + 16 * mb + 4 * grp, acc[mb] * inv);
    if (wave == 0 && grp == 0 && a.lse) a.lse[((int64_t)b * a.num_q_heads + h) * q_len + qi] = lse;
  } else {
    _Float16* po = (_Float16*)a.part_o + (row * a.split.max_splits + split) * kDv;
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) store_part4(po + CPW * wave + 16 * mb + 4 * grp, acc[mb] * inv);
    if (wave == 0 && grp == 0) a.part_lse[row * a.split.max_splits + split] = lse;
  }
}

// ------------------------------------------------------------ VALU kernel

// Scores: wave w holds heads 4w..4w+3, lane (head 4w + lane/16, key pair
// lane%16): the two dot products over 576 values from LDS (packed bf16 dot2).
// The block max of a head is a 16-lane row reduction.  P V: thread t owns
// value columns 8 (t%64) .. +8 of heads 4 (t/64) .. +3 and reads P from LDS.
template <class KT>
__global__ __launch_bounds__(kThreads, 1) void mla_valu_kernel(MlaArgs a) {
  // (the 576 / 512 record only: 64 threads cover a 512-wide value row)
  using DM = Dims576;
  constexpr int kRec = DM::kRec, kDv = DM::kDv, kRowBytes = DM::kRowBytes;
  __shared__ __attribute__((aligned(16))) char lds[2][kBlock * kRowBytes];
  __shared__ __attribute__((aligned(16))) uint32_t q_sh[kHeads][kRec / 2];
  __shared__ __attribute__((aligned(16))) float p_sh[kBlock][kHeads];
  __shared__ float alpha_sh[kHeads];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;

  // (ordered: the unit list gives (sequence, split, token range), see
  // WorkUnit)
  const bool ordered = a.units != nullptr;
  int tile, b, split, ut0 = 0, ut1 = 0;
  if (ordered) {
    int u;  // head tiles of one unit on one XCD (group_tile)
    group_tile(blockIdx.x, gridDim.x / a.head_tiles, a.head_tiles, u, tile);
    u = __builtin_amdgcn_readfirstlane(u);
    tile = __builtin_amdgcn_readfirstlane(tile);
    const WorkUnit w = load_unit(a.units, u);
    if (w.b < 0) return;
    b = w.b;
    split = w.split;
    ut0 = w.t0;
    ut1 = w.t1;
  } else {
    group_tile(blockIdx.x, gridDim.x / a.head_tiles, a.head_tiles, b, tile);
    b = __builtin_amdgcn_readfirstlane(b);
    tile = __builtin_amdgcn_readfirstlane(tile);
    split = blockIdx.y;
  }
  // One batch of kernel-argument loads; then the sequence length, the
  // range's block-table entries and q are requested together (a split past
  // the end of a short sequence finds out from the length and leaves after
  // that one round trip; the entries it loaded lie in the table row).
  asm volatile("" ::"s"(a.q), "s"(a.kv_cache), "s"(a.block_tables), "s"(a.context_lens),
               "s"(a.num_q_heads), "s"(a.head_tiles), "s"(a.page_size), "s"(a.max_pages),
               "s"(a.log2_page), "s"(a.qk_scale_log2), "s"(a.split.pages_per_split),
               "s"(a.split.max_splits), "s"(a.split.split_min_tokens));
  const int log2P = a.log2_page;
  PageTable pt{a.block_tables + (int64_t)b * a.max_pages, a.max_pages, 0, 0};
  pt.load(ordered                  ? ut0 >> log2P
          : a.split.max_splits > 1 ? split * a.split.pages_per_split
                                   : 0,
          lane);
  int n = load_uniform(a.context_lens + b);
  const int hvalid_n = min(kHeads, a.num_q_heads - tile * kHeads);

  // q of the tile's heads into LDS (zero for padded heads)
  for (int i = tid; i < kHeads * kRec / 2; i += kThreads) {
    const int hh = i / (kRec / 2), w = i % (kRec / 2);
    uint32_t v = 0;
    if (hh < hvalid_n)
      v = ((const uint32_t*)a.q)[(((int64_t)b * a.num_q_heads + tile * kHeads + hh) * kRec) / 2 + w];
    q_sh[hh][w] = v;
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
  const int nblocks = (t1 - t0 + kBlock - 1) / kBlock;

  // score-phase identity
  const int sh = 4 * wave + (lane >> 4);  // head
  const int kp = lane & 15;               // keys 2kp, 2kp+1
  float m_run = -INFINITY, l_run = 0.f;   // of head sh (lanes of a row agree)
  // PV-phase identity
  const int c8 = tid & 63;                // value columns 8 c8 .. 8 c8 + 7
  const int hq = tid >> 6;                // heads 4 hq .. 4 hq + 3
  float acc[4][8];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[j][e] = 0.f;

  BlockLoader<kThreads, KT, DM> ld;
  ld.load(a, pt, t0, t1, 0, log2P, tid);
  ld.store(lds[0], tid);
  ld.load(a, pt, t0, t1, 1, log2P, tid);
  __syncthreads();

  for (int blk = 0; blk < nblocks; ++blk) {
    const char* L = lds[blk & 1];
    const int rows = min(kBlock, t1 - (t0 + blk * kBlock));
    // scores of (head sh, keys 2kp, 2kp+1)
    float s0 = 0.f, s1 = 0.f;
#pragma unroll 4
    for (int c = 0; c < kRec / 8; ++c) {
      const u32x4 qv = *(const u32x4*)&q_sh[sh][4 * c];
      const u32x4 a0 = *(const u32x4*)(L + lds_off<DM>(2 * kp, c));
      const u32x4 a1 = *(const u32x4*)(L + lds_off<DM>(2 * kp + 1, c));
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t qj = qv[j], x0 = a0[j], x1 = a1[j];
        s0 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qj), as_bf16x2(x0), s0, false);
        s1 = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(qj), as_bf16x2(x1), s1, false);
      }
    }
    s0 = 2 * kp < rows ? s0 * a.qk_scale_log2 : -INFINITY;
    s1 = 2 * kp + 1 < rows ? s1 * a.qk_scale_log2 : -INFINITY;
    float tmax = fmaxf(s0, s1);
#pragma unroll
    for (int o = 1; o < 16; o <<= 1) tmax = fmaxf(tmax, __shfl_xor(tmax, o, 64));
    float alpha = 1.f;
    if (tmax > m_run + kLazyMax) {
      alpha = exp2f(m_run - tmax);
      m_run = tmax;
    }
    const float p0 = exp2f(s0 - m_run), p1 = exp2f(s1 - m_run);
    l_run = l_run * alpha + p0 + p1;
    p_sh[2 * kp][sh] = p0;
    p_sh[2 * kp + 1][sh] = p1;
    if (kp == 0) alpha_sh[sh] = alpha;
    __syncthreads();
    // P V for value columns 8 c8.. of heads 4 hq..
    float al[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) al[j] = alpha_sh[4 * hq + j];
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[j][e] *= al[j];
#pragma unroll 4
    for (int key = 0; key < kBlock; ++key) {
      const u32x4 v = *(const u32x4*)(L + lds_off<DM>(key, c8));
      const f32x4 p4 = *(const f32x4*)&p_sh[key][4 * hq];
      float vf[8];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const uint32_t vj = v[j];
        vf[2 * j] = bf16_lo(vj);
        vf[2 * j + 1] = bf16_hi(vj);
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        acc[0][e] = fmaf(p4.x, vf[e], acc[0][e]);
        acc[1][e] = fmaf(p4.y, vf[e], acc[1][e]);
        acc[2][e] = fmaf(p4.z, vf[e], acc[2][e]);
        acc[3][e] = fmaf(p4.w, vf[e], acc[3][e]);
      }
    }
    if (blk + 1 < nblocks) ld.store(lds[(blk + 1) & 1], tid);
    if (blk + 2 < nblocks) ld.load(a, pt, t0, t1, blk + 2, log2P, tid);
    __syncthreads();
  }

  // l and m of each head to LDS, then normalize
  float lsum = l_run;
#pragma unroll
  for (int o = 1; o < 16; o <<= 1) lsum += __shfl_xor(lsum, o, 64);
  __shared__ float l_sh[kHeads], m_sh[kHeads];
  if (kp == 0) {
    l_sh[sh] = lsum;
    m_sh[sh] = m_run;
  }
  __syncthreads();
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int hh = 4 * hq + j;
    if (hh >= hvalid_n) continue;
    const float l = l_sh[hh];
    const float inv = l > 0.f ? a.v_scale / l : 0.f;
    const int64_t row = (int64_t)b * a.num_q_heads + tile * kHeads + hh;
    const f32x4 o0 = {acc[j][0] * inv, acc[j][1] * inv, acc[j][2] * inv, acc[j][3] * inv};
    const f32x4 o1 = {acc[j][4] * inv, acc[j][5] * inv, acc[j][6] * inv, acc[j][7] * inv};
    const float lse = l > 0.f ? (m_sh[hh] + __log2f(l)) * kLn2 : -INFINITY;
    if (nsplit == 1) {
      store_bf16x4<0>(a.out, row * kDv + 8 * c8, o0);
      store_bf16x4<0>(a.out, row * kDv + 8 * c8 + 4, o1);
      if (c8 == 0 && a.lse) a.lse[row] = lse;
    } else {
      _Float16* po = (_Float16*)a.part_o + (row * a.split.max_splits + split) * kDv + 8 * c8;
      store_part4(po, o0);
      store_part4(po + 4, o1);
      if (c8 == 0) a.part_lse[row * a.split.max_splits + split] = lse;
    }
  }
}

template <class DM, bool QM>
void launch_mfma(const MlaArgs& a, bool two, bool fp8, dim3 grid, hipStream_t s) {
  if (two) {
    if (fp8) hipLaunchKernelGGL((mla_mfma_kernel<2, E4M3, DM, QM>), grid, dim3(2 * kThreads), 0, s, a);
    else hipLaunchKernelGGL((mla_mfma_kernel<2, BF16, DM, QM>), grid, dim3(2 * kThreads), 0, s, a);
  } else {
    if (fp8) hipLaunchKernelGGL((mla_mfma_kernel<1, E4M3, DM, QM>), grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL((mla_mfma_kernel<1, BF16, DM, QM>), grid, dim3(kThreads), 0, s, a);
  }
}

}  // namespace

hipError_t launch_mla(const MlaArgs& a, int variant, int kv_dtype, int head_dim, int max_splits,
                      hipStream_t s) {
  const unsigned units = (unsigned)(a.batch * a.head_tiles);
  dim3 grid(a.units ? (unsigned)(a.head_tiles * a.unit_count) : units,
            a.units ? 1u : (unsigned)max_splits);
  const bool fp8 = kv_dtype == 3;
  const bool two = mla_column_groups(a.q_len * a.num_q_heads) == 2;
  if (variant == 2) {
    if (head_dim != 576) return hipErrorInvalidValue;
    if (fp8) hipLaunchKernelGGL(mla_valu_kernel<E4M3>, grid, dim3(kThreads), 0, s, a);
    else hipLaunchKernelGGL(mla_valu_kernel<BF16>, grid, dim3(kThreads), 0, s, a);
  } else if (head_dim == 576) {
    if (variant == 3) launch_mfma<Dims576, true>(a, two, fp8, grid, s);
    else launch_mfma<Dims576, false>(a, two, fp8, grid, s);
  } else if (head_dim == 320) {
    if (variant == 3) launch_mfma<Dims320, true>(a, two, fp8, grid, s);
    else launch_mfma<Dims320, false>(a, two, fp8, grid, s);
  } else {
    return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace pda
