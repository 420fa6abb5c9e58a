// pda_append.hip -- writes the new tokens' K and V rows into the paged cache,
// the step before attention ("From MHA to MLA" sec. 2: the new token's key and
// value join the cache first; sec. 5 and the drill page sec. 4: a token's
// page comes from the block table, its slot is the position modulo P).
//
// One thread moves eight consecutive elements of one token row (a 16-byte
// load for 16-bit sources, two for fp32): the rows of all KV heads of a
// token are contiguous in the source [B, s_new, Hkv, d] and in a token-major
// page [P, Hkv, d], so consecutive threads write consecutive bytes of one
// slot; in a head-major page [Hkv, P, d] they write the token's d-wide row
// of each head (a head width is a multiple of 8, so no piece straddles two
// heads).  Same-type caches get the elements copied; an E4M3 cache gets the
// nearest E4M3FN code of the fp32 quotient x / scale (ties to even,
// saturated at +-448), from the format's definition (bias 7, 3 mantissa
// bits, subnormal step 2^-9, no infinities).
#include "pda_device.h"

namespace pda {
namespace {

constexpr int kAppendThreads = 256;

// E4M3FN code of x: round to nearest even, |x| >= 448 (infinities included)
// saturates to 448, NaN gives 0x7F.
__device__ __forceinline__ uint32_t e4m3_code(float x) {
  const uint32_t u = __float_as_uint(x);
  const uint32_t a = u & 0x7fffffffu;
  if (a > 0x7f800000u) return 0x7fu;
  const uint32_t sign = (u >> 24) & 0x80u;
  const float f = __uint_as_float(a);
  uint32_t code;
  if (f >= 448.0f) {
    code = 0x7eu;
  } else if (f < 0.015625f) {
    // below 2^-6: the subnormal grid m * 2^-9 (f * 512 is exact); m = 8 is
    // 2^-6, whose code 0x08 is the smallest normal
    code = (uint32_t)__builtin_rintf(f * 512.0f);
  } else {
    const uint32_t e = (a >> 23) - 120u;  // unbiased + 7: 1 .. 15
    const uint32_t m = a & 0x7fffffu;
    const uint32_t keep = m >> 20, rem = m & 0xfffffu;
    const uint32_t up = (rem > 0x80000u || (rem == 0x80000u && (keep & 1u))) ? 1u : 0u;
    code = (e << 3) + keep + up;          // a mantissa carry moves to the next exponent
  }
  return sign | code;
}

template <class T>
__device__ __forceinline__ void load8(const void* src, int64_t e, float (&v)[8]) {
  if constexpr (std::is_same<T, F32>::value) {
    const u32x4 a = *(const u32x4*)((const char*)src + e * 4);
    const u32x4 b = *(const u32x4*)((const char*)src + e * 4 + 16);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
    }
  } else {
    const u32x4 w = *(const u32x4*)((const char*)src + e * 2);
    to_f32(T{}, w, v);
  }
}

// s_new tokens per sequence, one tensor (K or V); blockIdx.y picks it.
template <class ST, class CT>
__global__ __launch_bounds__(kAppendThreads) void append_kernel(AppendArgs a) {
  const bool is_v = blockIdx.y == 1;
  const int width = is_v ? a.head_dim_v : a.head_dim;
  const int64_t row = (int64_t)a.num_kv_heads * width;  // elements of one token
  const int64_t row_chunks = row / 8;
  const int64_t chunk = (int64_t)blockIdx.x * kAppendThreads + threadIdx.x;
  if (chunk >= (int64_t)a.batch * a.s_new * row_chunks) return;
  const int64_t tok = chunk / row_chunks;  // b * s_new + t
  const int64_t off = (chunk - tok * row_chunks) * 8;
  const int b = (int)(tok / a.s_new), t = (int)(tok - (int64_t)b * a.s_new);
  const int pos = a.positions[b];
  if (pos < 0) return;
  const int p = pos + t;
  const int page = a.block_tables[(int64_t)b * a.max_pages + p / a.page_size];
  const int slot = p % a.page_size;
  // token-major pages [P, Hkv, width]: the token's row is contiguous;
  // head-major pages [Hkv, P, width]: head h's piece sits at h * P * width
  int64_t dst;
  if (a.head_major) {
    const int h = (int)(off / width), e = (int)(off - (int64_t)h * width);
    dst = (int64_t)page * a.page_size * row + ((int64_t)h * a.page_size + slot) * width + e;
  } else {
    dst = ((int64_t)page * a.page_size + slot) * row + off;
  }
  const int64_t src = tok * row + off;
  const void* from = is_v ? a.v_new : a.k_new;
  void* to = is_v ? a.v_cache : a.k_cache;
  if constexpr (std::is_same<CT, E4M3>::value) {
    const float s = is_v ? a.v_scale : a.k_scale;
    float v[8];
    load8<ST>(from, src, v);
    uint32_t w[2] = {0u, 0u};
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i / 4] |= e4m3_code(__fdiv_rn(v[i], s)) << (8 * (i % 4));
    *(u32x2*)((char*)to + dst) = u32x2{w[0], w[1]};
  } else {
    static_assert(std::is_same<ST, CT>::value, "same-type copy");
    constexpr int bytes = 8 * Elem<CT>::bytes;
#pragma unroll
    for (int k = 0; k < bytes; k += 16)
      *(u32x4*)((char*)to + dst * Elem<CT>::bytes + k) =
          *(const u32x4*)((const char*)from + src * Elem<CT>::bytes + k);
  }
}

template <class ST, class CT>
hipError_t launch_t(const AppendArgs& a, hipStream_t s) {
  const int64_t wmax = a.v_cache ? (a.head_dim > a.head_dim_v ? a.head_dim : a.head_dim_v)
                                 : a.head_dim;
  const int64_t chunks = (int64_t)a.batch * a.s_new * a.num_kv_heads * wmax / 8;
  const int64_t blocks = (chunks + kAppendThreads - 1) / kAppendThreads;
  if (blocks == 0) return hipSuccess;
  if (blocks > INT32_MAX) return hipErrorInvalidValue;
  hipLaunchKernelGGL((append_kernel<ST, CT>), dim3((unsigned)blocks, a.v_cache ? 2u : 1u),
                     dim3(kAppendThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace

bool append_supported(int src_dtype, int cache_dtype) {
  if (cache_dtype == 3) return src_dtype >= 0 && src_dtype <= 2;
  return src_dtype == cache_dtype && src_dtype >= 0 && src_dtype <= 2;
}

hipError_t launch_append(const AppendArgs& a, int src_dtype, int cache_dtype, hipStream_t s) {
  if (cache_dtype == 3) {
    if (src_dtype == 0) return launch_t<F32, E4M3>(a, s);
    if (src_dtype == 1) return launch_t<F16, E4M3>(a, s);
    if (src_dtype == 2) return launch_t<BF16, E4M3>(a, s);
  } else if (src_dtype == cache_dtype) {
    if (src_dtype == 0) return launch_t<F32, F32>(a, s);
    if (src_dtype == 1) return launch_t<F16, F16>(a, s);
    if (src_dtype == 2) return launch_t<BF16, BF16>(a, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace pda
