// gqa_kernels.h - kernel parameter blocks and launchers (internal to libgqa.so).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gqa {

// Prefill: one workgroup owns (sequence b, K/V head kvh, block of ROWS flattened
// query rows). Flattened row f = i * g + head_in_group, so a block holds whole query
// positions for every head of the group and they all share each K/V tile.
struct PrefillParams {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  const int32_t* seqlens;
  int B, S, Hq, Hkv, g, d;
  float scale_log2;   // |softmax_scale| * log2(e), at least 1e-30
  float scale_abs;    // scale_log2 / log2(e): |softmax_scale|, or the tiny stand-in for 0
  int negate_q;       // 1 when softmax_scale < 0 (the kernel negates q or the scores)
  int rows_per_wg;    // flattened rows per workgroup
  int nrb;            // row blocks per (b, kvh) unit
  int n_wg;           // B * Hkv * nrb
  int per_xcd;        // workgroups per XCD queue
  int lpt;            // 1: deal (b, kvh) units to XCDs longest sequence first (needs seqlens)
  int window;         // > 0: key j is visible to query i only if j > i - window
  const float* alibi; // [Hq] ALiBi slopes (score -= slope * |i - j|), or null
};

// Largest batch for which the bf16 prefill orders its work by sequence length.
constexpr int kPrefillLptMaxB = 256;

// Decode: workgroups split the concatenated key tiles of all units
// u = (b, kvh, query block) into equal shares (see decode_bf16.hip).
struct DecodeParams {
  const void* q;
  const void* kc;
  const void* vc;
  const int32_t* lens;
  void* o;
  float* lse;
  float* ws_o;        // [slots][32][d] normalised split outputs
  float* ws_lse;      // [slots][32] split log-sum-exp (natural log)
  int B, Hq, Hkv, g, d, max_len;
  int nqb;            // query blocks per K/V head: ceil(g / 32)
  int n_units;        // B * Hkv * nqb
  int n_wg;           // split workgroups
  float scale_log2;
  float scale_abs;
  int negate_q;
  int window;                 // > 0: only the last `window` keys (j > L_b - 1 - window)
  const float* alibi;         // [Hq] ALiBi slopes (score -= slope * (L_b - 1 - j)), or null
  const int32_t* block_table; // paged cache: [B, max_blocks] page ids, or null (contiguous)
  int page_size;              // keys per page (multiple of 32)
  int max_blocks;             // columns of block_table
  int num_pages;              // pages in each of the K and V pools
};

// MHA -> GQA weight conversion: out[g] = mean of w[g * H/G .. (g + 1) * H/G - 1].
struct MeanPoolParams {
  const void* w;      // [H, per_head]
  void* out;          // [G, per_head]
  int H, G;
  int64_t per_head;   // elements per head, a multiple of 8
};

// Per-device launch facts, found on the first launch on each device and kept until the
// process ends (the only state the library keeps between calls).
constexpr int kMaxDevices = 64;

// The current device and its compute-unit count (queried once per device).
hipError_t current_device(int* dev_out, int* cus_out);

// One kernel's per-device set-up: the dynamic-LDS attribute is set and the number of its
// workgroups a CU holds at once is found on the first launch on each device. A zero entry
// means "not set up yet"; keep one zero-initialised object with static storage per kernel.
struct KernelSetup {
  int per_cu[kMaxDevices];
};
hipError_t setup_kernel(KernelSetup& s, const void* kern, int threads, size_t lds, int dev,
                        int* per_cu_out);

hipError_t launch_prefill_bf16(const PrefillParams& p, int causal, hipStream_t stream);
hipError_t launch_prefill_f32(const PrefillParams& p, int causal, hipStream_t stream);
hipError_t launch_decode_bf16(const DecodeParams& p, bool need_combine, hipStream_t stream);
hipError_t launch_mean_pool(const MeanPoolParams& p, bool bf16, hipStream_t stream);

int prefill_rows_per_wg_bf16(int d);
int prefill_rows_per_wg_f32();

}  // namespace gqa
