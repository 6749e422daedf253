// Host-side argument fuzzing of the C ABI, built with AddressSanitizer and
// UndefinedBehaviorSanitizer on the host code of the library (no device code
// is compiled into this build).  Every entry point is called with dims drawn
// from edge values (negative, zero, limits, values that overflow 32-bit size
// products, odd strides), null or misaligned pointers, and small workspaces.
// Calls that pass validation reach the HIP runtime, which has no device here
// and reports an error; the program refuses to run if a device is visible,
// so no kernel can ever be launched on the fake pointers it passes.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <limits>

#include "sparsepr.h"

namespace {

uint64_t rng_state = 0x9e3779b97f4a7c15ull;
uint64_t next() {  // splitmix64
  uint64_t z = (rng_state += 0x9e3779b97f4a7c15ull);
  z = (z ^ (z >> 30)) * 0xbf58476d1ce4e5b9ull;
  z = (z ^ (z >> 27)) * 0x94d049bb133111ebull;
  return z ^ (z >> 31);
}
template <typename T, size_t N>
T pick(const T (&v)[N]) { return v[next() % N]; }

const int32_t kInts[] = {-2147483647 - 1, -1, 0, 1, 2, 7, 16, 63, 64, 65, 96, 127, 128, 256,
                         1023, 1024, 1025, 4096, 17550, 75600, 118800, 1 << 20, 1 << 24,
                         2147483647};
const int32_t kDims[] = {-1, 0, 32, 64, 96, 128, 256};
const int32_t kSmall[] = {-1, 0, 1, 2, 10, 15, 16, 17, 48, 63, 64, 64, 64, 65, 1000, 2147483647};
const int64_t kStrides[] = {-16, 0, 8, 16, 64, 128, 130, 256, 8192, 1ll << 20, 1ll << 33,
                            std::numeric_limits<int64_t>::max()};
const size_t kWs[] = {0, 16, 4096, size_t(1) << 30, std::numeric_limits<size_t>::max(),
                      std::numeric_limits<size_t>::max()};

const int32_t kHeads[] = {1, 2, 8, 40};
const int32_t kTokens[] = {1, 17, 300, 4096, 17550, 75600, 118800, 16777215, 16777216};
const int32_t kGroups[] = {1, 8, 64, 256, 1024};

sparsepr_dims random_dims() {
  sparsepr_dims d{};
  if (next() % 2) {
    // mostly valid shapes with packed strides
    d.heads = pick(kHeads);
    d.n_q = pick(kTokens);
    d.n_k = next() % 2 ? d.n_q : pick(kTokens);
    d.head_dim = next() % 2 ? 64 : 128;
    d.dtype = int32_t(next() % 2);
    d.c_q = pick(kGroups);
    d.c_k = pick(kGroups);
    d.q_stride_tok = d.kv_stride_tok = d.head_dim;
    d.q_stride_head = int64_t(d.n_q) * d.head_dim;
    d.kv_stride_head = int64_t(d.n_k) * d.head_dim;
    return d;
  }
  d.heads = pick(kInts);
  d.n_q = pick(kInts);
  d.n_k = next() % 2 ? d.n_q : pick(kInts);
  d.head_dim = pick(kDims);
  d.dtype = int32_t(next() % 4) - 1;
  d.c_q = pick(kInts);
  d.c_k = pick(kInts);
  d.reserved = next() % 8 == 0 ? 1 : 0;
  if (next() % 2) {
    d.q_stride_head = d.q_stride_tok = d.kv_stride_head = d.kv_stride_tok = 0;  // packed
  } else {
    d.q_stride_head = pick(kStrides);
    d.q_stride_tok = pick(kStrides);
    d.kv_stride_head = pick(kStrides);
    d.kv_stride_tok = pick(kStrides);
  }
  return d;
}

void* ptr() {
  switch (next() % 16) {
    case 0: return nullptr;
    case 1: return reinterpret_cast<void*>(uintptr_t(4100));  // misaligned
    default: return reinterpret_cast<void*>(uintptr_t(1) << 20);
  }
}
template <typename T>
T* p() { return static_cast<T*>(ptr()); }

int checked(int32_t st) {
  if (st < 0 || st > SPARSEPR_ERR_HIP) {
    std::fprintf(stderr, "unexpected status %d\n", st);
    std::exit(3);
  }
  return st;
}

}  // namespace

int main(int argc, char** argv) {
  int devices = 0;
  if (hipGetDeviceCount(&devices) == hipSuccess && devices > 0) {
    std::printf("a device is visible: not run\n");
    return 0;
  }
  const int iters = argc > 1 ? std::atoi(argv[1]) : 20000;
  long long counts[5] = {};
  for (int it = 0; it < iters; ++it) {
    const sparsepr_dims d = random_dims();
    const sparsepr_dims* dp = next() % 64 == 0 ? nullptr : &d;
    const int32_t m = pick(kSmall), rank = pick(kSmall), feat = pick(kSmall);
    const size_t ws = pick(kWs);
    for (int32_t call = -1; call <= 9; ++call) (void)sparsepr_workspace_bytes(call, dp, m, rank);
    int32_t st[15];
    st[0] = sparsepr_partition_layout(dp, p<int32_t>(), p<int32_t>(), ptr(), ptr(), ptr(),
                                      p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                      ptr(), ptr(), ptr(), p<int32_t>(), p<double>(),
                                      p<double>(), ptr(), ws, nullptr);
    st[1] = sparsepr_route_cells(dp, p<int32_t>(), p<int32_t>(), p<double>(), p<double>(),
                                 int64_t(next() % 3) - 1 + (int64_t(next() % 2) << 40),
                                 p<int32_t>(), p<int32_t>(), p<int64_t>(), ptr(), ws, nullptr);
    st[2] = sparsepr_route_cells_ex(dp, int32_t(next() % 4) - 1, p<int32_t>(), p<int32_t>(),
                                    p<double>(), p<double>(), int64_t(next() % 100000),
                                    p<int32_t>(), p<int32_t>(), p<int64_t>(), ptr(), ws,
                                    nullptr);
    const float scale = next() % 8 == 0 ? -1.f : 0.125f;
    st[3] = sparsepr_sparse_attn(dp, p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                 ptr(), ptr(), ptr(), p<int32_t>(), scale, p<float>(),
                                 p<float>(), ptr(), ws, nullptr);
    st[4] = sparsepr_sparse_attn_noalloc(dp, p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                         p<int32_t>(), ptr(), ptr(), ptr(), p<int32_t>(), scale,
                                         p<float>(), p<float>(), nullptr);
    const double lam = next() % 6 == 0 ? 0.0 : (next() % 6 == 0 ? -1.0 : 0.1);
    st[5] = sparsepr_probe_fit(dp, m, rank, lam, p<int32_t>(), p<int32_t>(), p<int32_t>(),
                               p<int32_t>(), p<int32_t>(), p<double>(), ptr(), ptr(), ptr(),
                               p<int32_t>(), scale, p<int32_t>(), p<int32_t>(), p<float>(),
                               p<float>(), p<float>(), p<float>(), p<float>(), ptr(), ws,
                               nullptr);
    const int32_t odt = int32_t(next() % 4) - 1;
    const int64_t osh = pick(kStrides), ost = pick(kStrides);
    st[6] = sparsepr_correct(dp, m, rank, p<int32_t>(), p<float>(), p<int32_t>(), p<float>(),
                             p<float>(), p<float>(), p<float>(), ptr(), odt, osh, ost, ptr(), ws,
                             nullptr);
    st[7] = sparsepr_sparse_attn_correct(dp, m, rank, p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                         p<int32_t>(), ptr(), ptr(), ptr(), p<int32_t>(), scale,
                                         p<int32_t>(), p<int32_t>(), p<float>(), p<float>(),
                                         p<float>(), p<float>(), p<float>(), ptr(), odt, osh,
                                         ost, p<float>(), ptr(), ws, nullptr);
    const int32_t iters_k = pick(kSmall);
    st[8] = sparsepr_rcp_partition(dp, pick(kSmall), pick(kSmall), pick(kSmall), iters_k, ptr(),
                                   ptr(), p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                   p<float>(), p<float>(), ptr(), ws, nullptr);
    st[9] = sparsepr_rcp_partition_ex(dp, pick(kSmall), pick(kSmall), pick(kSmall), iters_k,
                                      int32_t(next() % 3) - 1 + 1, ptr(), ptr(), p<int32_t>(),
                                      p<int32_t>(), p<float>(), p<float>(), p<float>(),
                                      p<float>(), p<int32_t>(), p<int32_t>(), p<float>(),
                                      p<float>(), ptr(), ws, nullptr);
    st[10] = sparsepr_probe_fit_ex(dp, m, rank, lam, int32_t(next() % 6) - 1, p<int32_t>(),
                                   p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                   p<double>(), p<float>(), feat, ptr(), ptr(), ptr(),
                                   p<int32_t>(), scale, p<int32_t>(), p<int32_t>(), p<float>(),
                                   p<float>(), p<float>(), p<float>(), p<float>(), p<float>(),
                                   ptr(), ws, nullptr);
    st[11] = sparsepr_correct_ex(dp, m, rank, p<int32_t>(), p<float>(), p<int32_t>(),
                                 p<float>(), p<float>(), p<float>(), p<float>(), p<float>(),
                                 ptr(), odt, osh, ost, ptr(), ws, nullptr);
    st[12] = sparsepr_debug_check(dp, m, p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                  p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                  p<int64_t>(), p<int32_t>(), p<int32_t>(), p<uint32_t>(),
                                  nullptr);
    st[13] = sparsepr_probe_select(dp, m, p<int32_t>(), p<int32_t>(), p<double>(), p<float>(),
                                   feat, ptr(), p<int32_t>(), p<int32_t>(), ptr(), ws, nullptr);
    st[14] = sparsepr_probe_fit_selected(dp, m, rank, lam, int32_t(next() % 6) - 1,
                                         p<int32_t>(), p<int32_t>(), p<int32_t>(), p<int32_t>(),
                                         ptr(), ptr(), ptr(), p<int32_t>(), scale, p<int32_t>(),
                                         p<float>(), p<float>(), p<float>(), p<float>(),
                                         p<float>(), p<float>(), ptr(), ws, nullptr);
    for (int i = 0; i < 15; ++i) ++counts[checked(st[i])];
  }
  for (int32_t s = -1; s <= 5; ++s) (void)sparsepr_status_string(s);
  std::printf("calls by status: ok %lld invalid %lld unsupported %lld workspace %lld hip %lld\n",
              counts[0], counts[1], counts[2], counts[3], counts[4]);
  return 0;
}
