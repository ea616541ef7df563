// probes.hip - microbenchmarks for the achievable peaks the measurements are compared
// with (libgqa_probes.so; used by bench.py only, not part of the attention library).
//
//   gqa_probe_mfma_bf16: back-to-back v_mfma_f32_32x32x16_bf16 with four independent
//     accumulator chains per wave; one launch does blocks x 4 waves x iters x 4 products
//     of 32 x 32 x 16 (2 x 16384 FLOP each).
//   gqa_probe_mfma_bf16_rand: the same products on random operands cycled over four register
//     sets (the multipliers toggle as on real data; the fixed operands above barely do).
//   gqa_probe_read / gqa_probe_read_nt: every 16-byte chunk of a buffer read once (grid-stride), XOR-folded
//     so nothing is optimised away; the achievable HBM read rate for a buffer far larger
//     than the last-level cache.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(unsigned)))) unsigned u32x4;

constexpr int kChains = 4;

__global__ __launch_bounds__(256, 4) void mfma_probe(int iters, float* out) {
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (float)((threadIdx.x + i) & 15));
    b[i] = (__bf16)(0.002f * (float)((threadIdx.x * 3 + i) & 7));
  }
  f32x16 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < kChains; ++k)
      acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

// Random-operand variant: four sets of A and B operands with random bf16 values (sign and
// mantissa from a hash of the lane, magnitudes in [0.5, 2)), cycled so that consecutive
// products see different data, as the multipliers do on real inputs.
__device__ unsigned mix32(unsigned x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__device__ unsigned rand_bf16x2(unsigned seed) {
  const unsigned h = mix32(seed);
  const unsigned lo = ((h & 1u) << 15) | ((126u + ((h >> 1) & 1u)) << 7) | ((h >> 2) & 0x7fu);
  const unsigned hi = (((h >> 9) & 1u) << 15) | ((126u + ((h >> 10) & 1u)) << 7) | ((h >> 11) & 0x7fu);
  return lo | (hi << 16);
}

constexpr int kSets = 4;

__global__ __launch_bounds__(256, 4) void mfma_probe_rand(int iters, float* out) {
  u32x4 a[kSets], b[kSets];
  const unsigned t = blockIdx.x * blockDim.x + threadIdx.x;
#pragma unroll
  for (int s = 0; s < kSets; ++s)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[s][i] = rand_bf16x2(t * 64u + s * 8u + i);
      b[s][i] = rand_bf16x2(t * 64u + s * 8u + 4u + i + 0x9e3779b9u);
    }
  f32x16 acc[kChains];
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[k][r] = 0.f;
  for (int it = 0; it < iters; it += kSets) {
#pragma unroll
    for (int u = 0; u < kSets; ++u)
#pragma unroll
      for (int k = 0; k < kChains; ++k)
        acc[k] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
            __builtin_bit_cast(bf16x8, a[(u + k) % kSets]),
            __builtin_bit_cast(bf16x8, b[(u + 2 * k + 1) % kSets]), acc[k], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int k = 0; k < kChains; ++k)
#pragma unroll
    for (int r = 0; r < 16; ++r) s += acc[k][r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void read_probe(const u32x4* buf, size_t n, unsigned* out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) acc ^= buf[i];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

// The same read with non-temporal loads (`nt`: lines read once are not kept).
__global__ __launch_bounds__(256) void read_probe_nt(const u32x4* buf, size_t n, unsigned* out) {
  u32x4 acc = {0u, 0u, 0u, 0u};
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  for (size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride)
    acc ^= __builtin_nontemporal_load(buf + i);
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = acc[0] ^ acc[1] ^ acc[2] ^ acc[3];
}

}  // namespace

extern "C" {

// FLOPs of one gqa_probe_mfma_bf16 launch.
double gqa_probe_mfma_flops(int blocks, int iters) {
  return (double)blocks * 4.0 * iters * kChains * 2.0 * 32 * 32 * 16;
}

// out: blocks * 256 floats (device). Returns 0 or a HIP error code.
int gqa_probe_mfma_bf16(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_probe, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     iters, out);
  return (int)hipGetLastError();
}

// As gqa_probe_mfma_bf16 with random operands cycled over four register sets; iters must be
// a multiple of 4 (same FLOPs per launch as gqa_probe_mfma_flops gives).
int gqa_probe_mfma_bf16_rand(int blocks, int iters, float* out, void* stream) {
  if (blocks <= 0 || iters <= 0 || iters % kSets || !out) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(mfma_probe_rand, dim3(blocks), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, out);
  return (int)hipGetLastError();
}

// buf: n16 16-byte chunks (device, 16-byte aligned); out: blocks * 256 words (device).
int gqa_probe_read(const void* buf, size_t n16, unsigned* out, int blocks, void* stream) {
  if (!buf || !out || blocks <= 0 || ((uintptr_t)buf & 15u)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), n16, out);
  return (int)hipGetLastError();
}

// As gqa_probe_read with non-temporal loads.
int gqa_probe_read_nt(const void* buf, size_t n16, unsigned* out, int blocks, void* stream) {
  if (!buf || !out || blocks <= 0 || ((uintptr_t)buf & 15u)) return (int)hipErrorInvalidValue;
  hipLaunchKernelGGL(read_probe_nt, dim3(blocks), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), n16, out);
  return (int)hipGetLastError();
}

}  // extern "C"
