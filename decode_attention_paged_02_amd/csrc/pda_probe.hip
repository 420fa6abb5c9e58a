// pda_probe.hip -- a streaming-read probe: the practical HBM ceiling of a
// GQA paged decode call on this GPU.
//
// The kernel reads exactly the K and V bytes a GQA decode call reads ("From
// MHA to MLA" sec. 5 and the drill page sec. 4: the pages of each sequence
// through its block-table row, the valid rows of the last page only), with
// the attention kernels' access pattern: one workgroup per (sequence, KV
// head, split), of four waves taking 16-token tiles w, w + 4, ... or of one
// wave taking them all (the wave layout the call's plan picks), a tile read
// as four 16-byte (or 8-/4-byte) row pieces per lane of K and of V with
// non-temporal buffer loads sized to the valid rows, the wave's block-table
// entries fetched 64 at a time and handed out with v_readlane.  Instead of
// attention each wave folds the words it loaded into one word (written to
// `sink`, so no load is dead).  The time of such a launch is the floor any
// kernel with this access pattern that writes a result can reach: bench.py
// reports the attention kernels against it ("fraction of the practical
// ceiling").  (Writing nothing at all would be ~0.4 us faster at B=64: the
// last stores' completion is part of any such kernel's time.)
#include "pda_device.h"

namespace pda {
namespace {

template <int W>
struct PWords {
  uint32_t w[W];
};

template <int W>
__device__ __forceinline__ PWords<W> probe_load(__amdgpu_buffer_rsrc_t r, int off) {
  PWords<W> p;
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

// PW: words of a lane's row piece (row bytes / 64); SD: tiles in flight per
// wave (the loads of tile i + SD - 1 are issued before tile i is folded); NW:
// waves per workgroup (4 or 1).
template <int PW, int SD, int NW>
__global__ __launch_bounds__(NW * 64, 2) void stream_probe_kernel(ProbeArgs a) {
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15, grp = lane >> 4;
  const int bk = blockIdx.x;
  const int kvh = bk % a.num_kv_heads, b = bk / a.num_kv_heads;
  const int split = blockIdx.y;
  const int log2P = a.log2_page;
  const int32_t* table = a.block_tables + (int64_t)b * a.max_pages;
  // The first 64 table entries of this wave (lane j: tile wave + NW j of the
  // split) are requested together with the length, as the attention kernels
  // do, before the split's range is known (entries past the sequence are
  // loaded from the table row but never used).
  const int t0_hint = a.split.max_splits > 1 ? split * a.split.pages_per_split << log2P : 0;
  auto load_entries = [&](int base) -> int {
    const int64_t tok = (int64_t)t0_hint + (int64_t)(wave + (base + lane) * NW) * kTileTokens;
    const int64_t pg = tok >> log2P;
    return table[pg < a.max_pages ? pg : a.max_pages - 1];
  };
  int vtbl = load_entries(0);
  const int n = load_uniform(a.context_lens + b);
  __builtin_amdgcn_sched_barrier(0);  // the table request goes out before waiting for n
  int nsplit, t0, t1;
  split_range(a.split, n, a.page_size, split, nsplit, t0, t1);  // (t0 == t0_hint)
  // one sink word per wave: [split][workgroup][wave]
  uint32_t* sink = a.sink + ((int64_t)blockIdx.y * gridDim.x + blockIdx.x) * NW + wave;
  if (split >= nsplit) {
    if (lane == 0) *sink = 0;
    return;
  }
  const int ntiles = (t1 - t0 + kTileTokens - 1) / kTileTokens;
  const int nw = ntiles > wave ? (ntiles - wave + NW - 1) / NW : 0;
  const int tok_bytes = a.tok_stride * a.elem_bytes;
  // load j: token 4 j + grp for 16-bit caches (four consecutive rows per
  // load instruction), 4 grp + j for fp8 ones, as the attention kernel
  const bool consec = a.elem_bytes != 1;
  const int off0 = (consec ? grp : 4 * grp) * tok_bytes + col * PW * 4;
  const int row_step = consec ? 4 * tok_bytes : tok_bytes;
  const int64_t head_elem = (int64_t)kvh * a.head_stride;
  uint32_t acc = 0;
  PWords<PW> kb[SD][4], vb[SD][4];
  for (int base = 0; base < nw; base += 64) {
    // lane j: the page of this wave's tile base + j
    if (base > 0) vtbl = load_entries(base);
    const int cnt = min(64, nw - base);
    // A tile's two resources, computed one tile ahead: the scalar address
    // arithmetic of tile i + 1 runs while tile i's loads are in flight,
    // not between its data's arrival and the next loads.
    struct TileRes {
      __amdgpu_buffer_rsrc_t k, v;
    };
    auto prep = [&](int i) -> TileRes {
      const bool live = i < cnt;
      const int entry = __builtin_amdgcn_readlane(vtbl, i & 63);
      const int tk = t0 + (wave + (base + i) * NW) * kTileTokens;
      const int rows = live ? min(kTileTokens, t1 - tk) : 0;
      const int slot = tk & ((1 << log2P) - 1);
      const int64_t elem =
          (int64_t)(live ? entry : 0) * a.page_stride + (int64_t)slot * a.tok_stride + head_elem;
      return TileRes{__builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.k_cache + elem * a.elem_bytes),
                                                       0, rows * tok_bytes, kRsrcFlags),
                     __builtin_amdgcn_make_buffer_rsrc((void*)((const char*)a.v_cache + elem * a.elem_bytes),
                                                       0, rows * tok_bytes, kRsrcFlags)};
    };
    auto fire = [&](const TileRes& r, int u) {
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kb[u][j] = probe_load<PW>(r.k, off0 + j * row_step);
        vb[u][j] = probe_load<PW>(r.v, off0 + j * row_step);
      }
    };
    TileRes pend = prep(0);  // the next tile to issue
#pragma unroll
    for (int u = 0; u < SD - 1; ++u) {
      fire(pend, u);
      pend = prep(u + 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    for (int i0 = 0; i0 < cnt; i0 += SD) {
#pragma unroll
      for (int u = 0; u < SD; ++u) {
        const int i = i0 + u;
        if (i >= cnt) break;
        fire(pend, (u + SD - 1) % SD);  // tile i + SD - 1
        pend = prep(i + SD);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
          for (int w = 0; w < PW; ++w) acc ^= kb[u][j].w[w] ^ vb[u][j].w[w];
      }
    }
  }
  // one word per wave keeps every load live: the XOR of every 32-bit word the
  // wave read (so a host can check which bytes were read).  Per wave, with no
  // barrier or LDS: a merge across the waves at the end costs the step time
  // of such a kernel (0.6-1 us at B=64), which a read ceiling should not pay.
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) acc ^= (uint32_t)__shfl_xor((int)acc, o, 64);
  if (lane == 0) *sink = acc;
}

template <int PW, int NW>
hipError_t launch_pw(const ProbeArgs& a, int max_splits, int sd, hipStream_t s) {
  dim3 grid((unsigned)(a.batch * a.num_kv_heads), (unsigned)max_splits);
  dim3 block(NW * 64);
  switch (sd) {
    case 1: hipLaunchKernelGGL((stream_probe_kernel<PW, 1, NW>), grid, block, 0, s, a); break;
    case 2: hipLaunchKernelGGL((stream_probe_kernel<PW, 2, NW>), grid, block, 0, s, a); break;
    case 3: hipLaunchKernelGGL((stream_probe_kernel<PW, 3, NW>), grid, block, 0, s, a); break;
    case 4: hipLaunchKernelGGL((stream_probe_kernel<PW, 4, NW>), grid, block, 0, s, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

template <int PW>
hipError_t launch_nw(const ProbeArgs& a, int max_splits, int sd, int waves, hipStream_t s) {
  return waves == 1 ? launch_pw<PW, 1>(a, max_splits, sd, s) : launch_pw<PW, 4>(a, max_splits, sd, s);
}

}  // namespace

hipError_t launch_probe(const ProbeArgs& a, int row_bytes, int max_splits, int steps_in_flight,
                        int waves, hipStream_t s) {
  switch (row_bytes) {
    case 64: return launch_nw<1>(a, max_splits, steps_in_flight, waves, s);
    case 128: return launch_nw<2>(a, max_splits, steps_in_flight, waves, s);
    case 256: return launch_nw<4>(a, max_splits, steps_in_flight, waves, s);
    case 512: return launch_nw<8>(a, max_splits, steps_in_flight, waves, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace pda
