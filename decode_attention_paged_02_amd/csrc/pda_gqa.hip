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
// per-lane byte offsets are loop invariant.  Block-table entries past the
// sequence's pages are never read.
#include "pda_internal.h"

#include <type_traits>

namespace pda {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
// Growth of a tile's max over the running reference (log2 units) that
// triggers a rescale; probabilities stay below 2^kLazyMax.
constexpr float kLazyMax = 8.0f;
// dword 3 of a gfx9-family buffer resource: 32-bit data format, raw access.
constexpr int kRsrcFlags = 0x00020000;

struct F32 {};
struct F16 {};
struct BF16 {};
struct E4M3 {};

template <class T> struct Elem;
template <> struct Elem<F32> { static constexpr int bytes = 4, epl = 4; using frag = u32x4; };
template <> struct Elem<F16> { static constexpr int bytes = 2, epl = 8; using frag = u32x4; };
template <> struct Elem<BF16> { static constexpr int bytes = 2, epl = 8; using frag = u32x4; };
template <> struct Elem<E4M3> { static constexpr int bytes = 1, epl = 8; using frag = u32x2; };

constexpr int ilog2(int x) { return x <= 1 ? 0 : 1 + ilog2(x / 2); }

// Reinterpret one 32-bit word as a pair of 16-bit floats.  The word is taken
// by value: hipcc's __builtin_bit_cast applied directly to an ext_vector
// element (v[j]) reads element 0 whatever j is, so every vector element goes
// through a scalar first.
__device__ __forceinline__ f16x2 as_f16x2(uint32_t w) { return __builtin_bit_cast(f16x2, w); }
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

// Cache policy of the K/V stream loads (the buffer instruction's cache-policy
// field; 2 marks them non-temporal).
#ifndef PDA_KV_LOAD_POLICY
#define PDA_KV_LOAD_POLICY 2  // non-temporal: K/V rows are read once
#endif

__device__ __forceinline__ u32x4 buf_load(__amdgpu_buffer_rsrc_t r, int off, u32x4*) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, PDA_KV_LOAD_POLICY);
}
__device__ __forceinline__ u32x2 buf_load(__amdgpu_buffer_rsrc_t r, int off, u32x2*) {
  return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, PDA_KV_LOAD_POLICY);
}

// ---------------------------------------------------------------- decoding

__device__ __forceinline__ void to_f32(F32, const u32x4& w, float (&o)[4]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) o[i] = __uint_as_float(w[i]);
}
__device__ __forceinline__ void to_f32(F16, const u32x4& w, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 h = as_f16x2(w[i]);
    o[2 * i] = (float)h.x;
    o[2 * i + 1] = (float)h.y;
  }
}
__device__ __forceinline__ void to_f32(BF16, const u32x4& w, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    o[2 * i] = __uint_as_float(w[i] << 16);
    o[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ __forceinline__ void to_f32(E4M3, const u32x2& w, float (&o)[8]) {
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], false);
    f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(w[i], true);
    o[4 * i] = lo.x;
    o[4 * i + 1] = lo.y;
    o[4 * i + 2] = hi.x;
    o[4 * i + 3] = hi.y;
  }
}

// Element pair j (elements 2j, 2j+1) of a K row fragment in q's 16-bit type.
__device__ __forceinline__ f16x2 k_pair_f16(const u32x4& w, int j) {
  const uint32_t x = w[j];
  return as_f16x2(x);
}
__device__ __forceinline__ f16x2 k_pair_f16(const u32x2& w, int j) {
  const uint32_t x = w[j >> 1];
  return (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(x, 1.0f, false);
}
__device__ __forceinline__ bf16x2 k_pair_bf16(const u32x4& w, int j) {
  const uint32_t x = w[j];
  return as_bf16x2(x);
}
__device__ __forceinline__ bf16x2 k_pair_bf16(const u32x2& w, int j) {
  const uint32_t x = w[j >> 1];
  return (j & 1) ? __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, true)
                 : __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(x, 1.0f, false);
}

// V of two token rows a, b regrouped into binary16 pairs per element:
// out[e] = (a[e], b[e]).  v_perm_b32 picks bytes of {b : a} (selector values
// 0-3 address a, 4-7 address b).
__device__ __forceinline__ void v_pairs(const u32x4& a, const u32x4& b, uint32_t (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint32_t x = a[j], y = b[j];
    out[2 * j] = __builtin_amdgcn_perm(y, x, 0x05040100u);      // (a.lo, b.lo)
    out[2 * j + 1] = __builtin_amdgcn_perm(y, x, 0x07060302u);  // (a.hi, b.hi)
  }
}
__device__ __forceinline__ void v_pairs(const u32x2& a, const u32x2& b, uint32_t (&out)[8]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const uint32_t x = a[j], y = b[j];
    const uint32_t lo = __builtin_amdgcn_perm(y, x, 0x05010400u);  // a0 b0 a1 b1
    const uint32_t hi = __builtin_amdgcn_perm(y, x, 0x07030602u);  // a2 b2 a3 b3
    out[4 * j] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, false));
    out[4 * j + 1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(lo, 1.0f, true));
    out[4 * j + 2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, false));
    out[4 * j + 3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_f16_fp8(hi, 1.0f, true));
  }
}

// q row fragment (EPL elements starting at element `e0` of a q row) as floats.
template <class QT, int EPL>
__device__ __forceinline__ void load_q_f32(const void* q, int64_t e0, float (&o)[EPL]) {
  if constexpr (std::is_same<QT, F32>::value) {
    const float* p = (const float*)q + e0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = p[i];
  } else if constexpr (std::is_same<QT, F16>::value) {
    const _Float16* p = (const _Float16*)q + e0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = (float)p[i];
  } else {
    const uint16_t* p = (const uint16_t*)q + e0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) o[i] = __uint_as_float((uint32_t)p[i] << 16);
  }
}

template <class T>
__device__ __forceinline__ void store_out(void* out, int64_t i, float v) {
  if constexpr (std::is_same<T, F32>::value) {
    ((float*)out)[i] = v;
  } else if constexpr (std::is_same<T, F16>::value) {
    ((_Float16*)out)[i] = (_Float16)v;
  } else {
    ((__bf16*)out)[i] = (__bf16)v;
  }
}

// --------------------------------------------------------- lane exchanges

// Cross-row exchanges use the gfx950 lane swaps:
//   permlane16_swap(a, b): rows 1 and 3 of a trade places with rows 0 and 2 of b;
//   permlane32_swap(a, b): lanes 32-63 of a trade places with lanes 0-31 of b.
// With a == b == x every lane ends up holding {x_self, x_partner} (partner =
// lane ^ 16, resp. lane ^ 32) in the two results, in an order that depends on
// the row; commutative reductions just combine both.
__device__ __forceinline__ void swap16(float a, float b, float& ra, float& rb) {
  auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  ra = __uint_as_float(r[0]);
  rb = __uint_as_float(r[1]);
}
__device__ __forceinline__ void swap32(float a, float b, float& ra, float& rb) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(a), __float_as_uint(b), false, false);
  ra = __uint_as_float(r[0]);
  rb = __uint_as_float(r[1]);
}

// DPP lane move (every lane written: rows and banks all enabled).
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), CTRL, 0xF, 0xF, true));
}

// Value of x held by lane (this lane XOR 2^BIT) for BIT 0..3 (inside a row of
// 16 lanes, DPP).
template <int BIT>
__device__ __forceinline__ float lane_xor(float x) {
  static_assert(BIT >= 0 && BIT <= 3, "row-local exchange");
  if constexpr (BIT == 0) {
    return dpp<0xB1>(x);  // quad_perm 1,0,3,2
  } else if constexpr (BIT == 1) {
    return dpp<0x4E>(x);  // quad_perm 2,3,0,1
  } else if constexpr (BIT == 2) {
    // row_half_mirror gives lane ^ 7, then quad_perm 3,2,1,0 gives ^ 3: ^ 4
    return dpp<0x1B>(dpp<0x141>(x));
  } else {
    return dpp<0x128>(x);  // row_ror 8
  }
}

// Sum of x over the lane pair {lane, lane ^ 2^BIT}, for any BIT 0..5.
template <int BIT>
__device__ __forceinline__ float pair_sum(float x) {
  if constexpr (BIT <= 3) {
    return x + lane_xor<BIT>(x);
  } else {
    float a, b;
    if constexpr (BIT == 4) swap16(x, x, a, b); else swap32(x, x, a, b);
    return a + b;
  }
}

// Reduce-scatter of N partial sums across the lanes that differ in lane bits
// BIT, BIT-1, ..., 0 (most significant first).  Each step halves the array:
// lanes with the bit clear keep the first half, lanes with it set the second,
// each adding its partner's copy of the half it keeps.  Once one value is
// left, the remaining bits are summed as an all-reduce (duplicated values).
template <int N, int BIT>
__device__ __forceinline__ void reduce_scatter(float* v, int lane) {
  if constexpr (BIT >= 0) {
    if constexpr (N > 1) {
      if constexpr (BIT >= 4) {
        // the swap hands even rows {first half: self, partner} and odd rows
        // {second half: partner, self}; adding them is the scatter step
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
          float a, b;
          if constexpr (BIT == 4) swap16(v[k], v[k + N / 2], a, b);
          else swap32(v[k], v[k + N / 2], a, b);
          v[k] = a + b;
        }
      } else {
        const bool hi = (lane >> BIT) & 1;
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
          float keep = hi ? v[k + N / 2] : v[k];
          float send = hi ? v[k] : v[k + N / 2];
          v[k] = keep + lane_xor<BIT>(send);
        }
      }
      reduce_scatter<N / 2, BIT - 1>(v, lane);
    } else {
      v[0] = pair_sum<BIT>(v[0]);
      reduce_scatter<1, BIT - 1>(v, lane);
    }
  }
}

// Max / sum over the lanes that differ in bits 2..5 (the lanes that hold the
// same head's scores).  Bits 2 and 3 use row rotations by 4 and 8, which
// visit all four lanes with equal bits 0-1 in a row of 16.
__device__ __forceinline__ float wave_max_bits2to5(float x) {
  float a, b;
  x = fmaxf(x, dpp<0x124>(x));  // row_ror 4
  x = fmaxf(x, dpp<0x128>(x));  // row_ror 8
  swap16(x, x, a, b);
  x = fmaxf(a, b);
  swap32(x, x, a, b);
  return fmaxf(a, b);
}
__device__ __forceinline__ float wave_sum_bits2to5(float x) {
  x += dpp<0x124>(x);
  x += dpp<0x128>(x);
  return pair_sum<5>(pair_sum<4>(x));
}

// Sum over lane bits FROM..5.
template <int FROM>
__device__ __forceinline__ float wave_sum_from(float x) {
  if constexpr (FROM <= 3) x = pair_sum<3>(x);
  if constexpr (FROM <= 4) x = pair_sum<4>(x);
  if constexpr (FROM <= 5) x = pair_sum<5>(x);
  return x;
}

__device__ __forceinline__ void split_range(const SplitLayout& sp, int n, int P, int split,
                                            int& nsplit, int& t0, int& t1) {
  const int pages = (n + P - 1) / P;
  if (sp.max_splits <= 1 || n <= sp.split_min_tokens) {
    nsplit = 1;
    t0 = 0;
    t1 = n;
  } else {
    nsplit = (pages + sp.pages_per_split - 1) / sp.pages_per_split;
    const int p0 = split * sp.pages_per_split;
    t0 = p0 * P;
    t1 = min((p0 + sp.pages_per_split) * P, n);
  }
}

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

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int rg = lane / LPR;
  const int c = lane % LPR;
  const int seg = c >> DUPBITS;

  const int wg = blockIdx.x;
  const int tile = wg % a.head_tiles;
  const int bk = wg / a.head_tiles;
  const int kvh = bk % a.num_kv_heads;
  const int b = bk / a.num_kv_heads;
  const int split = blockIdx.y;

  const int n = a.context_lens[b];
  int nsplit, t0, t1;
  split_range(a.split, n, a.page_size, split, nsplit, t0, t1);
  if (split >= nsplit) return;

  const int g0 = tile * GT;                 // first group-local head of the tile
  const int hbase = kvh * a.group + g0;     // first query head of the tile
  const int gvalid = min(GT, a.group - g0); // heads of the tile inside the group

  // q of the tile's heads, the EPL elements this lane multiplies
  uint32_t qp[GT][EPL / 2];
  float qf[GT][EPL];
#pragma unroll
  for (int g = 0; g < GT; ++g) {
    const int64_t e0 = ((int64_t)b * a.num_q_heads + hbase + g) * D + c * EPL;
    if constexpr (kPacked) {
      if (g < gvalid) {
        u32x4 w = *(const u32x4*)((const char*)a.q + e0 * 2);
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) qp[g][j] = w[j];
      } else {
#pragma unroll
        for (int j = 0; j < EPL / 2; ++j) qp[g][j] = 0u;
      }
    } else {
      if (g < gvalid) {
        load_q_f32<QT, EPL>(a.q, e0, qf[g]);
      } else {
#pragma unroll
        for (int j = 0; j < EPL; ++j) qf[g][j] = 0.f;
      }
    }
  }

  // loop-invariant byte offsets of this lane's rows inside a tile
  const int tok_bytes = a.tok_stride * ESZ;
  int voff[NLD];
#pragma unroll
  for (int i = 0; i < NLD; ++i) voff[i] = (rg + RPL * i) * tok_bytes + (kvh * D + c * EPL) * ESZ;

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
  const int32_t* table = a.block_tables + (int64_t)b * a.max_pages;

  // Page of a tile: pages hold 2^log2_page tokens (a multiple of the tile).
  const int log2P = a.log2_page;
  auto page_of = [&](int T) { return (t0 + T * kTileTokens) >> log2P; };

  // Buffer resources of tile ordinal k (tile wave + k * kGqaWaves) in physical
  // page `phys`; empty ones past the range (their loads return zero without
  // touching memory).
  auto tile_rsrc = [&](int k, int phys, __amdgpu_buffer_rsrc_t& rk, __amdgpu_buffer_rsrc_t& rv,
                       int& rows) {
    const int T = wave + k * kGqaWaves;
    const bool live = T < ntiles;
    const int tok = t0 + T * kTileTokens;
    rows = live ? min(kTileTokens, t1 - tok) : 0;
    const int slot = tok & ((1 << log2P) - 1);
    const int64_t elem = (int64_t)(live ? phys : 0) * a.page_stride + (int64_t)slot * a.tok_stride;
    rk = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.k_cache + elem * ESZ), 0,
                                           rows * tok_bytes, kRsrcFlags);
    rv = __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.v_cache + elem * ESZ), 0,
                                           rows * tok_bytes, kRsrcFlags);
  };
  // Block-table entry of tile ordinal k (a scalar load; entries of tiles past
  // the range are not read).
  auto table_entry = [&](int k) {
    const int T = wave + k * kGqaWaves;
    return T < ntiles ? table[page_of(T)] : 0;
  };

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
    reduce_scatter<NV, LOG_LPR - 1>(sc, lane);

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
      const float s = row < rows ? sc[k] * a.qk_scale_log2 : -INFINITY;
      const float tmax = wave_max_bits2to5(s);
      const bool move = tmax > m_run[k] + kLazyMax;
      const float m_new = move ? tmax : m_run[k];
      alpha[k] = exp2f(m_run[k] - m_new);
      p[k] = exp2f(s - m_new);
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
  constexpr int kPF = (96 / kTileRegs - 1) < 1 ? 1
                      : ((96 / kTileRegs - 1) < kGqaPrefetch ? (96 / kTileRegs - 1) : kGqaPrefetch);
  constexpr int NB = kPF + 1;
  frag_t kb[NB][NLD], vb[NB][NLD];
  int rows_b[NB];
  // The table entry of the next tile to issue is loaded one issue ahead, so
  // its scalar-load latency hides behind a tile's compute.
  int phys_next = table_entry(0);
  auto issue = [&](int k, int u) {
    __amdgpu_buffer_rsrc_t rk, rv;
    const int phys = __builtin_amdgcn_readfirstlane(phys_next);
    phys_next = table_entry(k + 1);
    tile_rsrc(k, phys, rk, rv, rows_b[u]);
#pragma unroll
    for (int i = 0; i < NLD; ++i) {
      kb[u][i] = buf_load(rk, voff[i], (frag_t*)nullptr);
      vb[u][i] = buf_load(rv, voff[i], (frag_t*)nullptr);
    }
  };
#pragma unroll
  for (int u = 0; u < kPF; ++u) issue(u, u);
  for (int kc = 0;; kc += NB) {
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      const int k = kc + u;
      if (wave + k * kGqaWaves >= ntiles) goto tiles_done;
      issue(k + kPF, (u + kPF) % NB);
      compute_tile(kb[u], vb[u], rows_b[u]);
    }
  }
tiles_done:

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

// One workgroup per (sequence, query head) row whose sequence was split:
// L = M + ln sum_s exp(L_s - M), O = sum_s exp(L_s - M) O_s / sum_s exp(L_s - M)
// with M = max_s L_s ("From MHA to MLA" sec. 4).  Rows of unsplit sequences
// were written by the attention kernel and are skipped.  The threads form
// kCombineThreads / (DV / 4) split groups x (DV / 4) four-float chunks of the
// row; each group weights its splits against its own maximum, and the groups
// are merged through LDS with the same algebra.  The sequence length and the
// first partials are loaded together, so the row costs one memory round trip.
template <class OT, int DV>
__global__ __launch_bounds__(kCombineThreads) void combine_kernel(CombineArgs a) {
  constexpr int DC = DV / 4;                    // float4 chunks per row
  constexpr int SG = kCombineThreads / DC;      // split groups
  constexpr int MAXL = 8;                       // splits a thread keeps in flight
  static_assert(DC * SG == kCombineThreads, "row width");
  __shared__ f32x4 acc_sh[SG][DC];
  __shared__ float den_sh[SG], mx_sh[SG];

  const int64_t row = blockIdx.x;
  const int b = (int)(row / a.num_q_heads);
  const int S = a.split.max_splits;
  const float* pl = a.part_lse + row * S;
  const f32x4* po = (const f32x4*)(a.part_o + row * S * DV);
  const int sg = threadIdx.x / DC, dc = threadIdx.x % DC;

  // Issue the sequence length and this thread's first MAXL partials together
  // (slots past the split count hold stale data and are ignored below).
  const int n = a.context_lens[b];
  float l[MAXL];
  f32x4 o[MAXL];
#pragma unroll
  for (int j = 0; j < MAXL; ++j) {
    const int s2 = sg + j * SG;
    l[j] = s2 < S ? pl[s2] : -INFINITY;
    o[j] = s2 < S ? po[(int64_t)s2 * DC + dc] : f32x4{0.f, 0.f, 0.f, 0.f};
  }
  int nsplit, t0, t1;
  split_range(a.split, n, a.page_size, 0, nsplit, t0, t1);
  if (nsplit <= 1) return;

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
      acc += w * po[(int64_t)s2 * DC + dc];
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
    const int64_t o0 = row * DV + threadIdx.x * 4;
    store_out<OT>(a.out, o0, t.x * inv);
    store_out<OT>(a.out, o0 + 1, t.y * inv);
    store_out<OT>(a.out, o0 + 2, t.z * inv);
    store_out<OT>(a.out, o0 + 3, t.w * inv);
    if (threadIdx.x == 0 && a.lse) a.lse[row] = d > 0.f ? M + __logf(d) : -INFINITY;
  }
}

template <class QT, class KT, int D>
hipError_t launch_d(const GqaArgs& a, int tile_heads, int max_splits, hipStream_t s) {
  dim3 grid((unsigned)(a.batch * a.num_kv_heads * a.head_tiles), (unsigned)max_splits);
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

template <class OT>
hipError_t launch_combine_t(const CombineArgs& a, hipStream_t s) {
  dim3 grid((unsigned)(a.batch * a.num_q_heads));
  dim3 block(kCombineThreads);
  switch (a.head_dim_v) {
    case 64: hipLaunchKernelGGL((combine_kernel<OT, 64>), grid, block, 0, s, a); break;
    case 128: hipLaunchKernelGGL((combine_kernel<OT, 128>), grid, block, 0, s, a); break;
    case 256: hipLaunchKernelGGL((combine_kernel<OT, 256>), grid, block, 0, s, a); break;
    case 512: hipLaunchKernelGGL((combine_kernel<OT, 512>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

hipError_t launch_combine(const CombineArgs& a, int out_dtype, hipStream_t s) {
  switch (out_dtype) {
    case 0: return launch_combine_t<F32>(a, s);
    case 1: return launch_combine_t<F16>(a, s);
    case 2: return launch_combine_t<BF16>(a, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pda
