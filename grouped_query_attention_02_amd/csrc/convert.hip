// convert.hip - MHA -> GQA conversion of per-head projection weights by mean pooling.
//
// A multi-head checkpoint becomes a grouped one by replacing the K (and V) projection
// of each group of H/G consecutive heads with the mean of those heads' projections
// (azimuth.plus GQA digest, "Idea 1", step 1 and its code listing). The work is a plain
// streaming reduction: every input byte is read once and every output byte written
// once, so the kernel is bound by HBM bandwidth. Each thread owns 8 consecutive
// elements of one group's output (one 16-byte bf16 vector, two for fp32), loads the
// same 8 elements of each of the group's heads, sums them in fp32 and writes the mean.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int CV_THREADS = 256;

template <bool BF16>
__global__ __launch_bounds__(CV_THREADS) void mean_pool_kernel(MeanPoolParams p) {
  const int64_t vec = (int64_t)blockIdx.x * CV_THREADS + threadIdx.x;  // 8-element vector
  const int64_t nvec = p.per_head / 8;
  const int grp = blockIdx.y;
  if (vec >= nvec) return;
  const int hpg = p.H / p.G;
  const float inv = 1.f / (float)hpg;
  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  for (int t = 0; t < hpg; ++t) {
    const int64_t src = ((int64_t)(grp * hpg + t) * p.per_head) + vec * 8;
    if constexpr (BF16) {
      // Non-temporal: a wave reads 1 KB contiguous per head, every line of it once.
      const u32x4 x = __builtin_nontemporal_load(
          reinterpret_cast<const u32x4*>(static_cast<const uint16_t*>(p.w) + src));
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(x[e] << 16);
        acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u);
      }
    } else {
      const float* f = static_cast<const float*>(p.w) + src;
      const u32x4 a = ldg16(f), b = ldg16(f + 4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[e] += __uint_as_float(a[e]);
        acc[4 + e] += __uint_as_float(b[e]);
      }
    }
  }
  const int64_t dst = (int64_t)grp * p.per_head + vec * 8;
  if constexpr (BF16) {
    u32x4 y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    // (non-temporal loads and stores: 30.1 -> 28.9 us on the Llama-2-70B-shaped K projection)
    __builtin_nontemporal_store(y, reinterpret_cast<u32x4*>(static_cast<uint16_t*>(p.out) + dst));
  } else {
    u32x4 a, b;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      a[e] = __float_as_uint(acc[e] * inv);
      b[e] = __float_as_uint(acc[4 + e] * inv);
    }
    float* o = static_cast<float*>(p.out) + dst;
    *reinterpret_cast<u32x4*>(o) = a;
    *reinterpret_cast<u32x4*>(o + 4) = b;
  }
}

}  // namespace

hipError_t launch_mean_pool(const MeanPoolParams& p, bool bf16, hipStream_t stream) {
  const int64_t nvec = p.per_head / 8;
  const dim3 grid((unsigned)((nvec + CV_THREADS - 1) / CV_THREADS), (unsigned)p.G);
  if (bf16)
    hipLaunchKernelGGL(mean_pool_kernel<true>, grid, dim3(CV_THREADS), 0, stream, p);
  else
    hipLaunchKernelGGL(mean_pool_kernel<false>, grid, dim3(CV_THREADS), 0, stream, p);
  return hipGetLastError();
}

}  // namespace gqa
