// pda_device.h -- device-side building blocks shared by the GQA kernels
// (pda_gqa.hip, pda_gqa_mfma.hip): element types and decoding, buffer loads,
// cross-lane exchanges of the wave64 execution model, and the split layout.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "pda_internal.h"

namespace pda {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.6931471805599453f;
// Growth of a tile's max over the running reference (log2 units) that
// triggers a rescale; probabilities stay below 2^kLazyMax.
constexpr float kLazyMax = 8.0f;
// Start of a running max: the most negative finite float instead of -inf, so
// that a query row whose tokens are all masked so far (a causal mask can hide
// a whole tile or range from the early queries) keeps a rescale factor of
// exp2(0) = 1 and probabilities exp2(-inf) = 0 rather than exp2(-inf + inf).
constexpr float kMaxStart = -3.40282346638528859812e+38f;
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

// A 32-bit value the kernel never writes, read with a scalar load (through
// the constant address space) so that uniform control flow can wait for it
// where it is first used.
__device__ __forceinline__ int load_uniform(const int32_t* p) {
  return *(const __attribute__((address_space(4))) int32_t*)p;
}

// The same read where the address differs per lane (a vector load).
__device__ __forceinline__ int load_uniform_v(const int32_t* p) { return *p; }

// Split partial outputs: fp32, or binary16 for calls whose output is
// bfloat16, whose rounding step is 8 times binary16's.  Four consecutive
// values at p (16- or 8-byte aligned).  Kernels name the format by the tags
// F32 / F16 (PartElem gives the element type).
template <class PT>
struct PartElem {
  using type = float;
};
template <>
struct PartElem<F16> {
  using type = _Float16;
};
template <class PT>
__device__ __forceinline__ f32x4 load_part4(const PT* p) {
  if constexpr (std::is_same<PT, float>::value) return *(const f32x4*)p;
  else return __builtin_convertvector(*(const f16x4*)p, f32x4);
}
template <class PT>
__device__ __forceinline__ void store_part4(PT* p, f32x4 v) {
  if constexpr (std::is_same<PT, float>::value) *(f32x4*)p = v;
  else *(f16x4*)p = __builtin_convertvector(v, f16x4);
}

// A work unit of an ordered call (written by the planning kernel): sequence
// b (negative: no unit, the workgroup exits), split index (-1: the
// sequence's only split, whose result is the final output) and the token
// range [t0, t1).  Read with one scalar load.
struct WorkUnit {
  int b, split, t0, t1;
};
__device__ __forceinline__ WorkUnit load_unit(const int32_t* units, int idx) {
  typedef int32_t i32x4 __attribute__((ext_vector_type(4)));
  const i32x4 w = *(const __attribute__((address_space(4))) i32x4*)(units + 4 * idx);
  return WorkUnit{w[0], w[1], w[2], w[3]};
}

// Workgroup index i of `groups` x `tiles` workgroups -> (group, tile), where
// a group is one (sequence or unit, KV head) whose K/V rows each of its
// `tiles` head tiles reads.  The tiles of a group are placed 8 indices apart:
// workgroups are dealt to the 8 XCDs in index order, so they run on one XCD,
// about together, and the tiles after the first find the rows in that XCD's
// L2.  A last set of fewer than 8 groups keeps its tiles adjacent.  With one
// tile this is the identity.
__device__ __forceinline__ void group_tile(int i, int groups, int tiles, int& g, int& t) {
  if (tiles == 1) {
    g = i;
    t = 0;
    return;
  }
  const int g8 = groups & ~7;
  if (i < g8 * tiles) {
    const int blk = i / (8 * tiles), rem = i - blk * 8 * tiles;
    t = rem >> 3;
    g = blk * 8 + (rem & 7);
  } else {
    const int j = i - g8 * tiles;
    g = g8 + j / tiles;
    t = j - (j / tiles) * tiles;
  }
}

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
// lanes with the bit clear end up with the first half, lanes with it set with
// the second, each adding its partner's copy of the half it keeps.  Once one
// value is left, the remaining bits are summed as an all-reduce (duplicated
// values).
//
// Lane bits 0-3 are exchanged with DPP, which sends every lane the same
// register of its partner.  Steps on arrays of at most PERM values expect
// each lane's array stored with the step's index bit flipped whenever the
// lane's own bit is set (the halves swapped), so every lane keeps its
// register v[k] and receives its partner's v[k + N/2]: one DPP add per value.
// Larger arrays are stored in plain order and the halves are picked with
// selects.  Bits 4 and 5 use the lane swaps, which already hand even rows the
// first half and odd rows the second, so those steps take plain order.
template <int N, int BIT, int PERM>
__device__ __forceinline__ void reduce_scatter(float* v, int lane) {
  if constexpr (BIT >= 0) {
    if constexpr (N > 1) {
      if constexpr (BIT >= 4) {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
          float a, b;
          if constexpr (BIT == 4) swap16(v[k], v[k + N / 2], a, b);
          else swap32(v[k], v[k + N / 2], a, b);
          v[k] = a + b;
        }
      } else if constexpr (N <= PERM) {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) v[k] += lane_xor<BIT>(v[k + N / 2]);
      } else {
        const bool hi = (lane >> BIT) & 1;
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
          const float keep = hi ? v[k + N / 2] : v[k];
          const float send = hi ? v[k] : v[k + N / 2];
          v[k] = keep + lane_xor<BIT>(send);
        }
      }
      reduce_scatter<N / 2, BIT - 1, PERM>(v, lane);
    } else {
      v[0] = pair_sum<BIT>(v[0]);
      reduce_scatter<1, BIT - 1, PERM>(v, lane);
    }
  }
}

// +infinity in a scalar register, opaque to the compiler: med3(x, y, +inf)
// is max(x, y) in one instruction, where a plain fmaxf on lane-exchanged
// values costs two extra canonicalizing maxes.
__device__ __forceinline__ float opaque_inf() {
  int bits;
  asm volatile("s_mov_b32 %0, 0x7f800000" : "=s"(bits));
  return __int_as_float(bits);
}
__device__ __forceinline__ float max2(float x, float y, float pinf) {
  return __builtin_amdgcn_fmed3f(x, y, pinf);
}

// Max / sum over the lanes that differ in bits 2..5 (the lanes that hold the
// same head's scores).  Bits 2 and 3 use row rotations by 4 and 8, which
// visit all four lanes with equal bits 0-1 in a row of 16.
__device__ __forceinline__ float wave_max_bits2to5(float x, float pinf) {
  float a, b;
  x = max2(x, dpp<0x124>(x), pinf);  // row_ror 4
  x = max2(x, dpp<0x128>(x), pinf);  // row_ror 8
  swap16(x, x, a, b);
  x = max2(a, b, pinf);
  swap32(x, x, a, b);
  return max2(a, b, pinf);
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

// ------------------------------------------------------------ unit planning

// LDS scratch of plan_unit.
struct PlanShared {
  unsigned long long pages[16];  // per-wave page sums
  int bucket_count[33];          // units per token-count bit length
  int wave_sum[16];              // per-wave unit counts of the chosen bucket
  int result[5];                 // b, split, t0, t1, split count of b
};

// Splits of a sequence of n tokens under an ordered call's rules (the same
// rules as the planning kernel): ns splits of pps pages.
__device__ __forceinline__ void unit_layout(const UnitPlan& p, int n, int chunk, int& ns,
                                            int& pps) {
  const int P = p.page_size;
  const int pages = (n + P - 1) / P;
  const int S = p.split.max_splits;
  if (S <= 1 || n <= p.split.split_min_tokens || (p.balanced && pages <= chunk)) {
    ns = 1;
    pps = pages > 0 ? pages : 1;
  } else if (!p.balanced) {
    pps = p.split.pages_per_split;
    ns = (pages + pps - 1) / pps;
  } else {
    ns = min(S, (pages + chunk - 1) / chunk);
    pps = (pages + ns - 1) / ns;
    ns = (pages + pps - 1) / pps;
  }
}

__device__ __forceinline__ int token_bucket(int tok) { return tok > 0 ? 32 - __clz(tok) : 0; }

// Work unit `rank` of an ordered call, computed by a whole workgroup of NT
// threads from the sequence lengths (batch <= kInKernelPlanMaxBatch), so that
// no planning launch precedes the attention kernel.  The units are the
// planning kernel's: every sequence cut into its splits, listed by decreasing
// bit length of their token count (longest first).  Inside a bit length they
// follow (sequence, split) order, so the list is a function of the lengths
// alone and every workgroup derives the same one.  Returns b = -1 past the
// last unit; ns_b is the unit's sequence's split count.  Every thread of the
// workgroup must call it (it synchronizes the workgroup).
template <int NT>
__device__ WorkUnit plan_unit(const int32_t* lens, const UnitPlan& p, int rank, PlanShared& sh,
                              int& ns_b) {
  constexpr int NW = NT / 64;
  constexpr int PERMAX = (kInKernelPlanMaxBatch + NT - 1) / NT;
  static_assert(NW <= 16, "workgroup size");
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int B = p.batch;
  const int per = (B + NT - 1) / NT;  // sequences per thread, contiguous
  int n[PERMAX];
  unsigned long long my_pages = 0;
#pragma unroll
  for (int i = 0; i < PERMAX; ++i) {
    const int b = tid * per + i;
    n[i] = (i < per && b < B) ? load_uniform_v(lens + b) : -1;
    if (n[i] >= 0) my_pages += (unsigned)((n[i] + p.page_size - 1) / p.page_size);
  }
  if (tid < 33) sh.bucket_count[tid] = 0;
  if (p.balanced) {
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) my_pages += __shfl_xor(my_pages, o, 64);
    if (lane == 0) sh.pages[wave] = my_pages;
  }
  __syncthreads();
  int chunk = 0;
  if (p.balanced) {  // a chunk of the batch's total pages over the target unit count
    unsigned long long total = 0;
    for (int w = 0; w < NW; ++w) total += sh.pages[w];
    const unsigned long long c = (total + p.target_units - 1) / p.target_units;
    chunk = (int)(c > (unsigned long long)p.min_chunk_pages ? c : p.min_chunk_pages);
  }
  // splits of this thread's sequences; units per token-count bucket: the
  // ns - 1 full splits and the last one
  int ns[PERMAX], pps[PERMAX], bf[PERMAX], bl[PERMAX];
#pragma unroll
  for (int i = 0; i < PERMAX; ++i) {
    ns[i] = 0;
    pps[i] = 1;
    bf[i] = bl[i] = -1;
    if (n[i] < 0) continue;
    unit_layout(p, n[i], chunk, ns[i], pps[i]);
    const int full = pps[i] * p.page_size;
    bf[i] = token_bucket(full);
    bl[i] = token_bucket(n[i] - (ns[i] - 1) * full);
    if (ns[i] > 1) atomicAdd(&sh.bucket_count[bf[i]], ns[i] - 1);
    atomicAdd(&sh.bucket_count[bl[i]], 1);
  }
  __syncthreads();
  // the bucket that holds `rank`, from the longest down, and the rank in it:
  // lane j takes bucket 32 - j, a scan over the lanes gives the units up to
  // and including each bucket, and the first lane whose total exceeds `rank`
  // holds it (one LDS read per lane instead of a dependent walk)
  int bucket = -1, k = rank;
  {
    const int c = lane <= 32 ? sh.bucket_count[32 - lane] : 0;
    int upto = c;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
      const int y = __shfl_up(upto, o, 64);
      if (lane >= o) upto += y;
    }
    const unsigned long long hit = __ballot(rank < upto);
    if (hit != 0) {
      const int j = __builtin_ctzll(hit);
      bucket = 32 - j;
      k = rank - __shfl(upto - c, j, 64);
    }
  }
  if (bucket < 0) {  // (the same for every thread)
    ns_b = 0;
    return WorkUnit{-1, -1, 0, 0};
  }
  // this thread's units in that bucket, then an exclusive scan over the
  // threads (sequence order)
  int cnt[PERMAX], mine = 0;
#pragma unroll
  for (int i = 0; i < PERMAX; ++i) {
    cnt[i] = ns[i] == 0 ? 0
                        : (ns[i] > 1 && bf[i] == bucket ? ns[i] - 1 : 0) + (bl[i] == bucket ? 1 : 0);
    mine += cnt[i];
  }
  int incl = mine;
#pragma unroll
  for (int o = 1; o < 64; o <<= 1) {
    const int y = __shfl_up(incl, o, 64);
    if (lane >= o) incl += y;
  }
  if (lane == 63) sh.wave_sum[wave] = incl;
  __syncthreads();
  int before = incl - mine;
  for (int w = 0; w < wave; ++w) before += sh.wave_sum[w];
  if (k >= before && k < before + mine) {  // exactly one thread
    int kk = k - before;
#pragma unroll
    for (int i = 0; i < PERMAX; ++i) {
      if (kk >= 0 && kk < cnt[i]) {
        // the full splits of the bucket come first, then the last split
        const int sp = (ns[i] > 1 && bf[i] == bucket && kk < ns[i] - 1) ? kk : ns[i] - 1;
        const int full = pps[i] * p.page_size;
        sh.result[0] = tid * per + i;
        sh.result[1] = ns[i] == 1 ? -1 : sp;
        sh.result[2] = sp * full;
        sh.result[3] = min((sp + 1) * full, n[i]);
        sh.result[4] = ns[i];
      }
      kk -= cnt[i];
    }
  }
  __syncthreads();
  ns_b = sh.result[4];
  return WorkUnit{sh.result[0], sh.result[1], sh.result[2], sh.result[3]};
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

}  // namespace pda
