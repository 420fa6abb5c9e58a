// c_abi_decode.cpp -- one paged decode step through the C ABI alone (HIP
// runtime + libpda, no Python): the calls a C or C++ serving loop makes.
//
//   c_abi_decode OUT.bin
//
// (Built also as libc_abi_decode.so exporting pda_example_decode_step, so
// that a test can run the same calls in its own process.)
//
// Builds a small GQA case on the host (B = 3 sequences of 1, 37 and 300
// tokens, Hq = 8, Hkv = 2, d = 128, pages of 16 tokens laid out head-major,
// fp16 values from a fixed linear congruential sequence), plans the call,
// allocates the workspace the plan asks for, runs paged_decode_attn with up
// to two splits and writes the inputs and results to OUT.bin so that they
// can be checked against an independent implementation.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <vector>

#include "pda.h"

namespace {

#define CHECK_HIP(x)                                                              \
  do {                                                                            \
    hipError_t e_ = (x);                                                          \
    if (e_ != hipSuccess) {                                                       \
      std::fprintf(stderr, "%s failed: %s\n", #x, hipGetErrorString(e_));         \
      return 1;                                                                   \
    }                                                                             \
  } while (0)

struct Lcg {
  uint64_t s;
  float next() {  // uniform in [-1, 1)
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return (float)((s >> 40) * (1.0 / 16777216.0)) * 2.0f - 1.0f;
  }
};

template <class T>
int to_device(const std::vector<T>& h, void** d) {
  CHECK_HIP(hipMalloc(d, h.size() * sizeof(T)));
  CHECK_HIP(hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return 0;
}

}  // namespace

extern "C" int pda_example_decode_step(const char* out_path) {
  const int B = 3, Hq = 8, Hkv = 2, D = 128, P = 16;
  const std::vector<int32_t> lens = {1, 37, 300};
  int max_pages = 0, used = 0;
  for (int n : lens) {
    max_pages = std::max(max_pages, (n + P - 1) / P);
    used += (n + P - 1) / P;
  }
  const int num_pages = used + 2;
  // block tables: the pool's pages handed out from the end, so logical and
  // physical order differ; unused entries -1 (never followed)
  std::vector<int32_t> table((size_t)B * max_pages, -1);
  int next = num_pages - 1;
  for (int b = 0; b < B; ++b)
    for (int p = 0; p < (lens[b] + P - 1) / P; ++p) table[(size_t)b * max_pages + p] = next--;

  Lcg g{12345};
  std::vector<_Float16> q((size_t)B * Hq * D), k((size_t)num_pages * Hkv * P * D),
      v((size_t)num_pages * Hkv * P * D);
  for (auto& x : q) x = (_Float16)g.next();
  for (auto& x : k) x = (_Float16)g.next();
  for (auto& x : v) x = (_Float16)g.next();

  pda_shape s{};
  s.batch = B;
  s.num_q_heads = Hq;
  s.num_kv_heads = Hkv;
  s.head_dim = D;
  s.head_dim_v = D;
  s.page_size = P;
  s.max_pages_per_seq = max_pages;
  s.num_pages = num_pages;
  s.q_dtype = PDA_F16;
  s.kv_dtype = PDA_F16;
  s.k_scale = 1.0f;
  s.v_scale = 1.0f;
  s.kv_layout = PDA_KV_HEAD_MAJOR;  // k/v: [num_pages, Hkv, P, D]

  const int num_splits = 2;
  pda_plan_info info{};
  int rc = pda_plan(&s, 0, num_splits, 0, &info);
  if (rc != PDA_OK) {
    std::fprintf(stderr, "pda_plan: %s\n", pda_status_string(rc));
    return 1;
  }
  void *dq, *dk, *dv, *dt, *dl, *dout, *dlse, *ws = nullptr;
  if (to_device(q, &dq) || to_device(k, &dk) || to_device(v, &dv) || to_device(table, &dt) ||
      to_device(lens, &dl))
    return 1;
  CHECK_HIP(hipMalloc(&dout, q.size() * sizeof(_Float16)));
  CHECK_HIP(hipMalloc(&dlse, (size_t)B * Hq * sizeof(float)));
  if (info.workspace_bytes) CHECK_HIP(hipMalloc(&ws, info.workspace_bytes));
  hipStream_t stream;
  CHECK_HIP(hipStreamCreate(&stream));

  rc = paged_decode_attn(dq, dk, dv, (const int32_t*)dt, (const int32_t*)dl, Hq / Hkv,
                         1.0f / std::sqrt((float)D), num_splits, dout, (float*)dlse, &s, ws,
                         info.workspace_bytes, stream);
  if (rc != PDA_OK) {
    std::fprintf(stderr, "paged_decode_attn: %s\n", pda_status_string(rc));
    return 1;
  }
  CHECK_HIP(hipStreamSynchronize(stream));
  std::vector<_Float16> out(q.size());
  std::vector<float> lse((size_t)B * Hq);
  CHECK_HIP(hipMemcpy(out.data(), dout, out.size() * sizeof(_Float16), hipMemcpyDeviceToHost));
  CHECK_HIP(hipMemcpy(lse.data(), dlse, lse.size() * sizeof(float), hipMemcpyDeviceToHost));

  FILE* f = std::fopen(out_path, "wb");
  if (!f) {
    std::perror(out_path);
    return 1;
  }
  const int32_t hdr[8] = {B, Hq, Hkv, D, P, max_pages, num_pages, num_splits};
  std::fwrite(hdr, sizeof(hdr), 1, f);
  std::fwrite(table.data(), sizeof(int32_t), table.size(), f);
  std::fwrite(lens.data(), sizeof(int32_t), lens.size(), f);
  std::fwrite(q.data(), sizeof(_Float16), q.size(), f);
  std::fwrite(k.data(), sizeof(_Float16), k.size(), f);
  std::fwrite(v.data(), sizeof(_Float16), v.size(), f);
  std::fwrite(out.data(), sizeof(_Float16), out.size(), f);
  std::fwrite(lse.data(), sizeof(float), lse.size(), f);
  std::fclose(f);
  std::printf("paged_decode_attn: %s; max_splits %d, workspace %llu bytes\n", pda_status_string(rc),
              info.max_splits, (unsigned long long)info.workspace_bytes);

  for (void* p : {dq, dk, dv, dt, dl, dout, dlse}) CHECK_HIP(hipFree(p));
  if (ws) CHECK_HIP(hipFree(ws));
  CHECK_HIP(hipStreamDestroy(stream));
  return 0;
}

#ifndef PDA_EXAMPLE_LIBRARY
int main(int argc, char** argv) {
  if (argc != 2) {
    std::fprintf(stderr, "usage: %s OUT.bin\n", argv[0]);
    return 2;
  }
  return pda_example_decode_step(argv[1]);
}
#endif
