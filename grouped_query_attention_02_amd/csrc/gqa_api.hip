// gqa_api.hip - C ABI of libgqa.so: argument validation, launch planning, dispatch.
//
// Every argument check runs on the host before anything touches the HIP runtime,
// so invalid calls return a status code without a device present.
#include <limits.h>
#include <math.h>
#include <stddef.h>
#include <stdint.h>

#include "gqa.h"
#include "gqa_kernels.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0
constexpr int kDecodeTile = 32;  // keys per decode tile
constexpr int kDecodeAutoShares = 256;  // auto split: one 8-wave workgroup per CU of a 256-CU GPU
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kMinScaleLog2 = 1e-30f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

bool supported_prefill_d(int dtype, int d) {
  (void)dtype;
  return d == 32 || d == 64 || d == 128;
}

bool supported_decode_d(int d) { return d == 64 || d == 128; }

struct DecodePlan {
  int nqb;
  int n_units;
  int n_wg;
  size_t ws_bytes;
  size_t ws_lse_offset;
};

// Shapes only; returns false for invalid arguments.
bool plan_decode(int B, int Hq, int Hkv, int d, int max_len, int num_splits, DecodePlan* out) {
  if (B <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0 || max_len <= 0 || num_splits < 0) return false;
  if (Hq % Hkv != 0) return false;
  const int g = Hq / Hkv;
  const long long nqb = (g + 31) / 32;
  const long long units = (long long)B * Hkv * nqb;
  const long long max_tiles = (max_len + kDecodeTile - 1) / kDecodeTile;
  long long wg;
  if (num_splits == 0) {
    wg = units > kDecodeAutoShares ? units : kDecodeAutoShares;
  } else {
    wg = (long long)num_splits * units;
  }
  if (wg > units * max_tiles) wg = units * max_tiles;  // never more shares than tiles
  if (units > INT_MAX / 2 || wg > INT_MAX / 2) return false;
  const long long slots = wg + units;
  out->nqb = (int)nqb;
  out->n_units = (int)units;
  out->n_wg = (int)wg;
  out->ws_lse_offset = (size_t)slots * 32 * d * sizeof(float);
  out->ws_bytes = out->ws_lse_offset + (size_t)slots * 32 * sizeof(float);
  return true;
}

}  // namespace

namespace gqa {

hipError_t current_device(int* dev_out, int* cus_out) {
  static int cus_cache[kMaxDevices];  // 0 = not queried yet
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  *dev_out = dev;
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int c = __atomic_load_n(&cus_cache[dev], __ATOMIC_ACQUIRE);
    if (c > 0) {
      *cus_out = c;
      return hipSuccess;
    }
  }
  int c = 0;
  if ((e = hipDeviceGetAttribute(&c, hipDeviceAttributeMultiprocessorCount, dev)) != hipSuccess)
    return e;
  if (c <= 0) c = 1;
  // Two threads racing here store the same value.
  if (cached) __atomic_store_n(&cus_cache[dev], c, __ATOMIC_RELEASE);
  *cus_out = c;
  return hipSuccess;
}

hipError_t setup_kernel(KernelSetup& s, const void* kern, int threads, size_t lds, int dev,
                        int* per_cu_out) {
  const bool cached = dev >= 0 && dev < kMaxDevices;
  if (cached) {
    const int v = __atomic_load_n(&s.per_cu[dev], __ATOMIC_ACQUIRE);
    if (v > 0) {
      *per_cu_out = v;
      return hipSuccess;
    }
  }
  hipError_t e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  int nb = 0;
  if ((e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&nb, kern, threads, lds)) != hipSuccess)
    return e;
  if (nb <= 0) nb = 1;
  if (cached) __atomic_store_n(&s.per_cu[dev], nb, __ATOMIC_RELEASE);
  *per_cu_out = nb;
  return hipSuccess;
}

}  // namespace gqa

namespace {

// Device scratch of gqa_decode_noalloc: the split partials of one call, in place of a
// caller's workspace. Each device the library runs on holds its own copy of this array
// until the process ends. In host code the name is only a stand-in: its device address is
// looked up once per device (scratch_address) and only that address is ever passed on.
static __device__ __align__(256) uint8_t scratch[GQA_DECODE_SCRATCH_BYTES];

// Device address of `scratch` on the current device, looked up on the first call on each
// device and cached.
hipError_t scratch_address(void** out) {
  static void* cache[gqa::kMaxDevices];
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < gqa::kMaxDevices;
  if (cached) {
    void* ptr = __atomic_load_n(&cache[dev], __ATOMIC_ACQUIRE);
    if (ptr) {
      *out = ptr;
      return hipSuccess;
    }
  }
  void* ptr = nullptr;
  if ((e = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch))) != hipSuccess) return e;
  if (!ptr) return hipErrorInvalidSymbol;
  if (cached) __atomic_store_n(&cache[dev], ptr, __ATOMIC_RELEASE);
  *out = ptr;
  return hipSuccess;
}

// Every argument check of a decode call except the workspace's (host only, no HIP call).
int check_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
                 const int32_t* cache_lens, const int32_t* block_table, int page_size,
                 int max_blocks, int num_pages, const void* o, const float* lse, int B, int Hq,
                 int Hkv, int d, int max_len, float softmax_scale, int window,
                 const float* alibi_slopes, int num_splits, DecodePlan* plan) {
  if (!plan_decode(B, Hq, Hkv, d > 0 ? d : 1, max_len, num_splits, plan))
    return GQA_ERR_INVALID_ARG;
  if (!q || !k_cache || !v_cache || !o) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o))
    return GQA_ERR_INVALID_ARG;
  if ((lse && ((uintptr_t)lse & 3u)) || (cache_lens && ((uintptr_t)cache_lens & 3u)) ||
      (alibi_slopes && ((uintptr_t)alibi_slopes & 3u)) ||
      (block_table && ((uintptr_t)block_table & 3u)))
    return GQA_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale) || window < 0) return GQA_ERR_INVALID_ARG;
  if (block_table) {
    // Paged cache: tiles of 32 keys must not straddle pages, and the table covers max_len.
    if (page_size <= 0 || page_size % kDecodeTile != 0 || max_blocks <= 0 || num_pages <= 0 ||
        (long long)page_size * max_blocks != max_len)
      return GQA_ERR_INVALID_ARG;
  }
  if (dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  if (!supported_decode_d(d)) return GQA_ERR_UNSUPPORTED;
  return GQA_OK;
}

// Launch of a checked decode call; `workspace` holds at least plan.ws_bytes bytes.
int launch_decode(const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* cache_lens, const int32_t* block_table, int page_size,
                  int max_blocks, int num_pages, void* o, float* lse, int B, int Hq, int Hkv,
                  int d, int max_len, float softmax_scale, int window,
                  const float* alibi_slopes, const DecodePlan& plan, void* workspace,
                  void* stream) {
  gqa::DecodeParams p;
  p.q = q; p.kc = k_cache; p.vc = v_cache; p.lens = cache_lens; p.o = o; p.lse = lse;
  p.ws_o = static_cast<float*>(workspace);
  p.ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + plan.ws_lse_offset);
  p.B = B; p.Hq = Hq; p.Hkv = Hkv; p.g = Hq / Hkv; p.d = d; p.max_len = max_len;
  p.nqb = plan.nqb; p.n_units = plan.n_units; p.n_wg = plan.n_wg;
  // A zero scale (uniform weights) still gets a positive exponent factor, tiny enough
  // that every valid weight rounds to exp2(0) = 1 while masked scores (-inf) give 0.
  p.scale_log2 = fmaxf(fabsf(softmax_scale) * kLog2e, kMinScaleLog2);
  // The LSE converts the kernels' running max (raw-score units) with the scale that factor
  // stands for, not |softmax_scale|: with a zero scale and ALiBi the max holds a bias of
  // slope / scale_log2 per key and must still come out as slope * distance.
  p.scale_abs = p.scale_log2 / kLog2e;
  p.negate_q = softmax_scale < 0.f ? 1 : 0;
  p.window = window < max_len ? window : 0;  // a window of max_len or more keys hides nothing
  p.alibi = alibi_slopes;
  p.block_table = block_table;
  p.page_size = block_table ? page_size : 0;
  p.max_blocks = block_table ? max_blocks : 0;
  p.num_pages = block_table ? num_pages : 0;
  // With no length array every unit has the same tile count; one share per unit then
  // maps each workgroup onto exactly one whole unit and no merge pass is needed.
  const bool need_combine = !(cache_lens == nullptr && plan.n_wg == plan.n_units);
  hipError_t e = gqa::launch_decode_bf16(p, need_combine, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // namespace

extern "C" {

int gqa_version(void) { return kVersion; }

const char* gqa_status_string(int status) {
  switch (status) {
    case GQA_OK: return "ok";
    case GQA_ERR_INVALID_ARG: return "invalid argument";
    case GQA_ERR_UNSUPPORTED: return "unsupported head size or dtype";
    case GQA_ERR_WORKSPACE:
      return "decode workspace missing or too small (gqa_decode_noalloc: the call needs more "
             "than the library's static scratch of GQA_DECODE_SCRATCH_BYTES)";
    case GQA_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

int gqa_prefill_ex(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                   const int32_t* seqlens, int B, int S, int Hq, int Hkv, int d,
                   float softmax_scale, int causal, int window, const float* alibi_slopes,
                   void* stream) {
  if (B <= 0 || S <= 0 || Hq <= 0 || Hkv <= 0 || d <= 0) return GQA_ERR_INVALID_ARG;
  if (Hq % Hkv != 0) return GQA_ERR_INVALID_ARG;
  if (!q || !k || !v || !o) return GQA_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o)) return GQA_ERR_INVALID_ARG;
  if ((lse && ((uintptr_t)lse & 3u)) || (seqlens && ((uintptr_t)seqlens & 3u)) ||
      (alibi_slopes && ((uintptr_t)alibi_slopes & 3u)))
    return GQA_ERR_INVALID_ARG;
  if (!isfinite(softmax_scale)) return GQA_ERR_INVALID_ARG;
  if (causal != 0 && causal != 1) return GQA_ERR_INVALID_ARG;
  if (window < 0) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  if (!supported_prefill_d(dtype, d)) return GQA_ERR_UNSUPPORTED;
  const int g = Hq / Hkv;
  if ((long long)S * g > INT_MAX / 2 || (long long)B * S * Hq > (long long)INT_MAX * 64)
    return GQA_ERR_INVALID_ARG;
  // The bf16 kernel addresses one sequence's K or V rows with 32-bit byte offsets.
  if (dtype == GQA_DTYPE_BF16 && (long long)S * Hkv * d * 2 > (long long)INT_MAX)
    return GQA_ERR_UNSUPPORTED;

  gqa::PrefillParams p;
  p.q = q; p.k = k; p.v = v; p.o = o; p.lse = lse; p.seqlens = seqlens;
  p.B = B; p.S = S; p.Hq = Hq; p.Hkv = Hkv; p.g = g; p.d = d;
  p.window = window < S ? window : 0;  // a window of S or more keys hides nothing
  p.alibi = alibi_slopes;
  if (p.window > 0 && !causal) return GQA_ERR_UNSUPPORTED;
  // A zero scale (uniform weights) still gets a positive exponent factor, tiny enough
  // that every valid weight rounds to exp2(0) = 1 while masked scores (-inf) give 0.
  p.scale_log2 = fmaxf(fabsf(softmax_scale) * kLog2e, kMinScaleLog2);
  // The LSE converts the kernels' running max (raw-score units) with the scale that factor
  // stands for, not |softmax_scale|: with a zero scale and ALiBi the max holds a bias of
  // slope / scale_log2 per key and must still come out as slope * distance.
  p.scale_abs = p.scale_log2 / kLog2e;
  p.negate_q = softmax_scale < 0.f ? 1 : 0;
  p.rows_per_wg = dtype == GQA_DTYPE_BF16 ? gqa::prefill_rows_per_wg_bf16(d)
                                          : gqa::prefill_rows_per_wg_f32();
  const long long rows = (long long)S * g;
  const long long nrb = (rows + p.rows_per_wg - 1) / p.rows_per_wg;
  const long long n_wg = nrb * B * Hkv;
  if (n_wg > INT_MAX / 2) return GQA_ERR_INVALID_ARG;
  p.nrb = (int)nrb;
  p.n_wg = (int)n_wg;
  p.per_xcd = (int)((n_wg + 7) / 8);
  // With ragged lengths the bf16 kernel sorts the (b, kvh) units by length and deals
  // them to the 8 XCD queues in snake order: each queue gets ceil(units / 8) units.
  p.lpt = (dtype == GQA_DTYPE_BF16 && seqlens && B <= gqa::kPrefillLptMaxB) ? 1 : 0;
  if (p.lpt) p.per_xcd = (int)(((long long)B * Hkv + 7) / 8 * nrb);

  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t e = dtype == GQA_DTYPE_BF16 ? gqa::launch_prefill_bf16(p, causal, s)
                                         : gqa::launch_prefill_f32(p, causal, s);
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

int gqa_prefill(int dtype, const void* q, const void* k, const void* v, void* o, float* lse,
                const int32_t* seqlens, int B, int S, int Hq, int Hkv, int d,
                float softmax_scale, int causal, void* stream) {
  return gqa_prefill_ex(dtype, q, k, v, o, lse, seqlens, B, S, Hq, Hkv, d, softmax_scale, causal,
                        0, nullptr, stream);
}

size_t gqa_decode_workspace_bytes(int B, int Hq, int Hkv, int d, int max_len, int num_splits) {
  DecodePlan plan;
  if (!plan_decode(B, Hq, Hkv, d, max_len, num_splits, &plan)) return 0;
  return plan.ws_bytes;
}

int gqa_decode_num_workgroups(int B, int Hq, int Hkv, int max_len, int num_splits) {
  DecodePlan plan;
  if (!plan_decode(B, Hq, Hkv, 32, max_len, num_splits, &plan)) return 0;
  return plan.n_wg;
}

int gqa_decode_ex(int dtype, const void* q, const void* k_cache, const void* v_cache,
                  const int32_t* cache_lens, const int32_t* block_table, int page_size,
                  int max_blocks, int num_pages, void* o, float* lse, int B, int Hq, int Hkv,
                  int d, int max_len, float softmax_scale, int window,
                  const float* alibi_slopes, int num_splits, void* workspace,
                  size_t workspace_bytes, void* stream) {
  DecodePlan plan;
  const int st = check_decode(dtype, q, k_cache, v_cache, cache_lens, block_table, page_size,
                              max_blocks, num_pages, o, lse, B, Hq, Hkv, d, max_len,
                              softmax_scale, window, alibi_slopes, num_splits, &plan);
  if (st != GQA_OK) return st;
  if (!workspace || workspace_bytes < plan.ws_bytes || !aligned16(workspace))
    return GQA_ERR_WORKSPACE;
  return launch_decode(q, k_cache, v_cache, cache_lens, block_table, page_size, max_blocks,
                       num_pages, o, lse, B, Hq, Hkv, d, max_len, softmax_scale, window,
                       alibi_slopes, plan, workspace, stream);
}

int gqa_decode_noalloc(int dtype, const void* q, const void* k_cache, const void* v_cache,
                       const int32_t* cache_lens, const int32_t* block_table, int page_size,
                       int max_blocks, int num_pages, void* o, float* lse, int B, int Hq,
                       int Hkv, int d, int max_len, float softmax_scale, int window,
                       const float* alibi_slopes, int num_splits, void* stream) {
  DecodePlan plan;
  const int st = check_decode(dtype, q, k_cache, v_cache, cache_lens, block_table, page_size,
                              max_blocks, num_pages, o, lse, B, Hq, Hkv, d, max_len,
                              softmax_scale, window, alibi_slopes, num_splits, &plan);
  if (st != GQA_OK) return st;
  if (plan.ws_bytes > (size_t)GQA_DECODE_SCRATCH_BYTES) return GQA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (scratch_address(&ws) != hipSuccess) return GQA_ERR_HIP;
  return launch_decode(q, k_cache, v_cache, cache_lens, block_table, page_size, max_blocks,
                       num_pages, o, lse, B, Hq, Hkv, d, max_len, softmax_scale, window,
                       alibi_slopes, plan, ws, stream);
}

int gqa_decode(int dtype, const void* q, const void* k_cache, const void* v_cache,
               const int32_t* cache_lens, void* o, float* lse, int B, int Hq, int Hkv, int d,
               int max_len, float softmax_scale, int num_splits, void* workspace,
               size_t workspace_bytes, void* stream) {
  return gqa_decode_ex(dtype, q, k_cache, v_cache, cache_lens, nullptr, 0, 0, 0, o, lse, B, Hq,
                       Hkv, d, max_len, softmax_scale, 0, nullptr, num_splits, workspace,
                       workspace_bytes, stream);
}

int gqa_mean_pool_heads(int dtype, const void* w, int H, int G, int64_t per_head, void* out,
                        void* stream) {
  if (!w || !out || H <= 0 || G <= 0 || H % G != 0 || per_head <= 0 || per_head % 8 != 0)
    return GQA_ERR_INVALID_ARG;
  if (!aligned16(w) || !aligned16(out)) return GQA_ERR_INVALID_ARG;
  if (per_head / 8 > (int64_t)INT_MAX * 256 || G > 65535) return GQA_ERR_INVALID_ARG;
  if (dtype != GQA_DTYPE_F32 && dtype != GQA_DTYPE_BF16) return GQA_ERR_UNSUPPORTED;
  gqa::MeanPoolParams p;
  p.w = w; p.out = out; p.H = H; p.G = G; p.per_head = per_head;
  hipError_t e =
      gqa::launch_mean_pool(p, dtype == GQA_DTYPE_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? GQA_OK : GQA_ERR_HIP;
}

}  // extern "C"
