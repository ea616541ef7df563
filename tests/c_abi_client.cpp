// A C++ caller of libgqa.so that uses nothing but include/gqa.h and the HIP runtime: it
// builds seeded bf16 inputs on the host, copies them into device memory it allocates itself,
// runs a causal prefill (with an LSE output) and a ragged split-KV decode through the C ABI,
// and checks both against the fp64 oracle (oracle/oracle.c, linked as liboracle.so, test
// infrastructure only). It also checks that a bad argument is rejected before any launch.
// Exit status 0 and a final "OK" line on success.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "gqa.h"

extern "C" {
int oracle_prefill(int dtype, const void* q, const void* k, const void* v, const int32_t* seqlens,
                   int B, int S, int Hq, int Hkv, int d, double scale, int causal, double* o,
                   double* lse, int n_threads);
int oracle_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* lens, int B, int Hq, int Hkv, int d, int max_len, double scale,
                  double* o, double* lse, int n_threads);
}
// The oracle's element-type codes (its own numbering, not gqa_dtype_t).
constexpr int kOracleBf16 = 2;

namespace {

#define CHECK_HIP(x)                                                            \
  do {                                                                          \
    hipError_t e_ = (x);                                                        \
    if (e_ != hipSuccess) {                                                     \
      std::fprintf(stderr, "HIP error %s at %s:%d\n", hipGetErrorString(e_),    \
                   __FILE__, __LINE__);                                         \
      return 1;                                                                 \
    }                                                                           \
  } while (0)

// Seeded standard normal values (64-bit LCG, Box-Muller), rounded to bf16 (nearest even).
struct Rng {
  uint64_t s;
  double uniform() {
    s = s * 6364136223846793005ull + 1442695040888963407ull;
    return ((s >> 11) + 0.5) * (1.0 / 9007199254740992.0);
  }
  double normal() {
    const double u1 = uniform(), u2 = uniform();
    return std::sqrt(-2.0 * std::log(u1)) * std::cos(6.283185307179586 * u2);
  }
};

uint16_t to_bf16(float x) {
  uint32_t u;
  std::memcpy(&u, &x, 4);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

float from_bf16(uint16_t h) {
  const uint32_t u = (uint32_t)h << 16;
  float x;
  std::memcpy(&x, &u, 4);
  return x;
}

std::vector<uint16_t> randn_bf16(size_t n, uint64_t seed) {
  Rng r{seed};
  std::vector<uint16_t> v(n);
  for (auto& x : v) x = to_bf16((float)r.normal());
  return v;
}

template <class T>
int to_device(const std::vector<T>& h, void** d) {
  CHECK_HIP(hipMalloc(d, h.size() * sizeof(T)));
  CHECK_HIP(hipMemcpy(*d, h.data(), h.size() * sizeof(T), hipMemcpyHostToDevice));
  return 0;
}

double max_err_bf16(const std::vector<uint16_t>& got, const std::vector<double>& ref) {
  double e = 0.0;
  for (size_t i = 0; i < got.size(); ++i)
    e = std::fmax(e, std::fabs(from_bf16(got[i]) - ref[i]));
  return e;
}

int run() {
  int fails = 0;
  // ---- prefill: B 2, S 200, 8 query heads over 2, d 128, causal, key lengths {200, 77}
  {
    const int B = 2, S = 200, Hq = 8, Hkv = 2, d = 128;
    const double scale = 1.0 / std::sqrt((double)d);
    const auto q = randn_bf16((size_t)B * S * Hq * d, 11);
    const auto k = randn_bf16((size_t)B * S * Hkv * d, 12);
    const auto v = randn_bf16((size_t)B * S * Hkv * d, 13);
    const std::vector<int32_t> lens = {200, 77};
    void *dq, *dk, *dv, *dl, *dO, *dL;
    if (to_device(q, &dq) || to_device(k, &dk) || to_device(v, &dv) || to_device(lens, &dl))
      return 1;
    CHECK_HIP(hipMalloc(&dO, q.size() * 2));
    CHECK_HIP(hipMalloc(&dL, (size_t)B * Hq * S * 4));
    int st = gqa_prefill(GQA_DTYPE_BF16, dq, dk, dv, dO, (float*)dL, (const int32_t*)dl, B, S,
                         Hq, Hkv, d, (float)scale, 1, nullptr);
    if (st != GQA_OK) {
      std::printf("prefill: %s\n", gqa_status_string(st));
      return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    std::vector<uint16_t> o(q.size());
    std::vector<float> lse((size_t)B * Hq * S);
    CHECK_HIP(hipMemcpy(o.data(), dO, o.size() * 2, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemcpy(lse.data(), dL, lse.size() * 4, hipMemcpyDeviceToHost));
    std::vector<double> ro(q.size()), rl(lse.size());
    if (oracle_prefill(kOracleBf16, q.data(), k.data(), v.data(), lens.data(), B, S, Hq, Hkv, d,
                       scale, 1, ro.data(), rl.data(), 0) != 0)
      return 1;
    const double e = max_err_bf16(o, ro);
    double le = 0.0;
    for (size_t i = 0; i < lse.size(); ++i) le = std::fmax(le, std::fabs(lse[i] - rl[i]));
    std::printf("prefill bf16 causal: max_abs_err=%.3e lse_err=%.3e\n", e, le);
    fails += !(e <= 2e-2 && le <= 1e-3);
    // A bad argument (Hq not a multiple of Hkv) is rejected on the host.
    st = gqa_prefill(GQA_DTYPE_BF16, dq, dk, dv, dO, nullptr, nullptr, B, S, 7, Hkv, d, 0.1f, 0,
                     nullptr);
    std::printf("prefill with Hq %% Hkv != 0: %s\n", gqa_status_string(st));
    fails += st != GQA_ERR_INVALID_ARG;
    for (void* p : {dq, dk, dv, dl, dO, dL}) CHECK_HIP(hipFree(p));
  }
  // ---- decode: B 3, 16 query heads over 2, d 128, cache 600, lengths {600, 1, 333}, 3 splits
  {
    const int B = 3, Hq = 16, Hkv = 2, d = 128, max_len = 600, splits = 3;
    const double scale = 1.0 / std::sqrt((double)d);
    const auto q = randn_bf16((size_t)B * Hq * d, 21);
    const auto kc = randn_bf16((size_t)B * Hkv * max_len * d, 22);
    const auto vc = randn_bf16((size_t)B * Hkv * max_len * d, 23);
    const std::vector<int32_t> lens = {600, 1, 333};
    void *dq, *dk, *dv, *dl, *dO, *dW;
    if (to_device(q, &dq) || to_device(kc, &dk) || to_device(vc, &dv) || to_device(lens, &dl))
      return 1;
    CHECK_HIP(hipMalloc(&dO, q.size() * 2));
    const size_t ws = gqa_decode_workspace_bytes(B, Hq, Hkv, d, max_len, splits);
    CHECK_HIP(hipMalloc(&dW, ws));
    const int st = gqa_decode(GQA_DTYPE_BF16, dq, dk, dv, (const int32_t*)dl, dO, nullptr, B, Hq,
                              Hkv, d, max_len, (float)scale, splits, dW, ws, nullptr);
    if (st != GQA_OK) {
      std::printf("decode: %s\n", gqa_status_string(st));
      return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    std::vector<uint16_t> o(q.size());
    CHECK_HIP(hipMemcpy(o.data(), dO, o.size() * 2, hipMemcpyDeviceToHost));
    std::vector<double> ro(q.size()), rl((size_t)B * Hq);
    if (oracle_decode(kOracleBf16, q.data(), kc.data(), vc.data(), lens.data(), B, Hq, Hkv, d,
                      max_len, scale, ro.data(), rl.data(), 0) != 0)
      return 1;
    const double e = max_err_bf16(o, ro);
    std::printf("decode bf16 split-KV (%d splits, workspace %zu bytes): max_abs_err=%.3e\n",
                splits, ws, e);
    fails += !(e <= 2e-2);
    for (void* p : {dq, dk, dv, dl, dO, dW}) CHECK_HIP(hipFree(p));
  }
  std::printf(fails ? "FAILED\n" : "OK\n");
  return fails ? 1 : 0;
}

}  // namespace

int main() {
  std::printf("libgqa version %d\n", gqa_version());
  return run();
}
