// pda_check.hip -- on-device check of the preconditions the attention and
// append entry points take on trust: every length lies in [0, max_pages * P]
// and every block-table entry a call would follow lies in [0, num_pages)
// (the drill page sec. 4 and 8: a page index is a dependent load whose value
// addresses the cache; out-of-range lengths or entries are the pitfalls it
// lists).  Only lengths, table entries and positions are read: no value
// found here addresses anything, whatever it holds.
//
// One workgroup walks every length and every table entry of the batch, counts
// violations in LDS and writes the three counts with plain stores, so the
// result buffer needs no clearing and a call is deterministic.
#include "pda_device.h"

namespace pda {
namespace {

constexpr int kCheckThreads = 1024;

__global__ __launch_bounds__(kCheckThreads) void check_kernel(CheckArgs a) {
  __shared__ int counts[3];
  if (threadIdx.x < 3) counts[threadIdx.x] = 0;
  __syncthreads();
  const int64_t cap = (int64_t)a.max_pages * a.page_size;
  int bad_len = 0, bad_entry = 0, bad_pos = 0;
  for (int b = threadIdx.x; b < a.batch; b += kCheckThreads) {
    const int n = a.context_lens[b];
    if (n < 0 || n > cap) ++bad_len;
    if (a.positions) {
      const int p = a.positions[b];
      if (p >= 0 && (int64_t)p + a.s_new > cap) ++bad_pos;
    }
  }
  const int64_t total = (int64_t)a.batch * a.max_pages;
  for (int64_t i = threadIdx.x; i < total; i += kCheckThreads) {
    const int b = (int)(i / a.max_pages);
    const int pg = (int)(i - (int64_t)b * a.max_pages);
    const int n = a.context_lens[b];
    // pages an attention call reads (a sequence with a bad length is
    // counted once above and its entries are not judged)
    bool used = n >= 0 && n <= cap && (int64_t)pg * a.page_size < n;
    if (a.positions) {  // pages an append writes
      const int p = a.positions[b];
      if (p >= 0 && (int64_t)p + a.s_new <= cap)
        used = used || (pg >= p / a.page_size && pg <= (p + a.s_new - 1) / a.page_size);
    }
    if (used) {
      const int e = a.block_tables[i];
      if (e < 0 || e >= a.num_pages) ++bad_entry;
    }
  }
  if (bad_len) atomicAdd(&counts[0], bad_len);
  if (bad_entry) atomicAdd(&counts[1], bad_entry);
  if (bad_pos) atomicAdd(&counts[2], bad_pos);
  __syncthreads();
  if (threadIdx.x < 3) a.result[threadIdx.x] = counts[threadIdx.x];
}

}  // namespace

hipError_t launch_check(const CheckArgs& a, hipStream_t s) {
  hipLaunchKernelGGL(check_kernel, dim3(1), dim3(kCheckThreads), 0, s, a);
  return hipGetLastError();
}

}  // namespace pda
