// prefill_f32.hip - fp32 grouped-query attention prefill (fp32 in, fp32 out).
//
// Same work split and online softmax as the bf16 kernel (one workgroup per
// (b, kvh, block of flattened rows f = i * g + h_local), K/V tiles in LDS shared by
// the whole query-head group, running max / running sum), but every product runs on
// the fp32 matrix-core instruction v_mfma_f32_32x32x2_f32, so no operand is ever
// rounded below fp32. Products of 2 keys at a time let P feed the PV product
// straight from the score accumulators and V be read from LDS in its stored
// [key][d] layout (no transpose).
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int PF32_WAVES = 4;
constexpr int PF32_THREADS = 64 * PF32_WAVES;
constexpr int PF32_ROWS = 32 * PF32_WAVES;
constexpr int PF32_BN = 32;

template <int D, bool CAUSAL>
__global__ __launch_bounds__(PF32_THREADS) void prefill_f32_kernel(PrefillParams p) {
  // K rows: lanes read one column of 32 rows -> stride = 2 mod 64 banks
  constexpr int KSTR = D + 2;
  constexpr int VSTR = D + 8;  // V rows: the two lane halves read rows 4 apart -> 32-bank offset
  __shared__ float ks_[PF32_BN * KSTR];
  __shared__ __attribute__((aligned(16))) float vs_[PF32_BN * VSTR];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const int lin = blockIdx.x;
  const int logical = (lin & 7) * p.per_xcd + (lin >> 3);
  if (logical >= p.n_wg) return;
  const int unit = logical / p.nrb;
  int rb = logical - unit * p.nrb;
  if (CAUSAL) rb = p.nrb - 1 - rb;
  const int b = unit / p.Hkv;
  const int kvh = unit - b * p.Hkv;
  const int g = p.g, S = p.S, Hq = p.Hq, Hkv = p.Hkv;

  int Lb = S;
  if (p.seqlens) {
    Lb = p.seqlens[b];
    Lb = Lb < 0 ? 0 : (Lb > S ? S : Lb);
  }
  const int R = S * g;
  const int f0 = rb * PF32_ROWS;
  const int fw = f0 + wave * 32;
  const int f = fw + l32;
  const bool row_ok = f < R;
  const int qi = row_ok ? f / g : 0;
  const int hq = kvh * g + (row_ok ? f - qi * g : 0);

  int kv_end = Lb, wave_kv_end = Lb, wave_mask_from = Lb;
  if (CAUSAL) {
    const int last_f = min(f0 + PF32_ROWS, R) - 1;
    kv_end = min(Lb, last_f / g + 1);
    const int wf_last = min(fw + 31, R - 1);
    wave_kv_end = (fw < R) ? min(Lb, wf_last / g + 1) : 0;
    wave_mask_from = min(Lb, fw / g + 1);
  }
  const int lim = CAUSAL ? min(Lb, qi + 1) : Lb;
  const int ntiles = (kv_end + PF32_BN - 1) / PF32_BN;
  // Sliding window: keys j >= lo = i - window + 1 only; tiles below every row's bound are
  // skipped. ALiBi: the score gets -slope_h * |i - j| (beta: the slope in raw-score units).
  constexpr int kNoLo = -(1 << 30);
  int lo = kNoLo, t_first = 0, wave_lo_min = kNoLo, wave_lo_hi = kNoLo;
  if (p.window > 0) {
    lo = qi - p.window + 1;
    t_first = max(0, f0 / g - p.window + 1) / PF32_BN;
    if (fw < R) {
      wave_lo_min = fw / g - p.window + 1;
      wave_lo_hi = min(fw + 31, R - 1) / g - p.window + 1;
    }
  }
  const float slope = p.alibi ? p.alibi[hq] : 0.f;
  const float beta = slope * kLog2e / p.scale_log2;
  // The bias is measured from key a = min(i, L_b - 1), the visible key nearest to the query:
  // when i >= L_b every key lies below a, so |i - j| = |a - j| + (i - a). The constant
  // slope * (i - a) drops out of the softmax and is added back to the LSE; without it, the
  // scores of a row far past a short key range would all carry a large bias, and fp32 would
  // resolve their differences only to the ulp of that bias.
  const int qa = min(qi, Lb - 1);

  // B operand of S^T = K Q^T: lane holds Q[row][2*ks + hh].
  float qf[D / 2];
  {
    const float* qrow = static_cast<const float*>(p.q) + (((size_t)b * S + qi) * Hq + hq) * D;
    const float sgn = p.negate_q ? -1.f : 1.f;
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks) qf[ks] = row_ok ? sgn * qrow[2 * ks + hh] : 0.f;
  }

  const size_t rstride = (size_t)Hkv * D;
  const float* kbase = static_cast<const float*>(p.k) + ((size_t)b * S * Hkv + kvh) * D;
  const float* vbase = static_cast<const float*>(p.v) + ((size_t)b * S * Hkv + kvh) * D;

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;
  constexpr int CPR = D / 4;  // float4 chunks per row

  for (int t = t_first; t < ntiles; ++t) {
    const int t0 = t * PF32_BN;
    __syncthreads();  // previous tile fully consumed
    for (int ch = tid; ch < PF32_BN * CPR; ch += PF32_THREADS) {
      const int key = ch / CPR, col = ch - key * CPR;
      const int j = t0 + key;
      u32x4 kv = j < Lb ? ldg16(kbase + (size_t)j * rstride + col * 4) : zero_u32x4();
      u32x4 vv = j < Lb ? ldg16(vbase + (size_t)j * rstride + col * 4) : zero_u32x4();
#pragma unroll
      for (int e = 0; e < 4; ++e) ks_[key * KSTR + col * 4 + e] = __uint_as_float(kv[e]);
      *reinterpret_cast<u32x4*>(vs_ + key * VSTR + col * 4) = vv;
    }
    __syncthreads();
    if (t0 >= wave_kv_end || t0 + PF32_BN <= wave_lo_min) continue;

    f32x16 s = zero16();
#pragma unroll
    for (int ks = 0; ks < D / 2; ++ks)
      s = mfma_f32_32x32x2(ks_[l32 * KSTR + 2 * ks + hh], qf[ks], s);

    if (p.alibi) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        s[r] = fmaf(-beta, fabsf((float)(qa - j)), s[r]);
      }
    }
    const bool need_mask = t0 + PF32_BN > wave_mask_from || t0 < wave_lo_hi;
    if (need_mask) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int j = t0 + 8 * (r >> 2) + 4 * hh + (r & 3);
        if (j >= lim || j < lo) s[r] = -INFINITY;
      }
    }
    float mx = -INFINITY;
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    mx = fmaxf(mx, xor32(mx));
    const float m_new = fmaxf(m_run, mx);
    if (wave_any(m_new > m_run)) {
      const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * c);
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    const float msc = (m_run == -INFINITY ? 0.f : m_run) * c;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float pv = fast_exp2(fmaf(s[r], c, -msc));
      if (need_mask) pv = (s[r] == -INFINITY) ? 0.f : pv;
      s[r] = pv;
      l_run += pv;
    }
    // O^T += V^T P^T two keys at a time: step r uses key 8(r/4)+(r%4) in lanes 0-31 and
    // key 8(r/4)+4+(r%4) in lanes 32-63, exactly the keys of this lane's s[r].
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = 8 * (r >> 2) + 4 * hh + (r & 3);
        oacc[db] = mfma_f32_32x32x2(vs_[key * VSTR + db * 32 + l32], s[r], oacc[db]);
      }
  }

  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    float* orow = static_cast<float*>(p.o) + (((size_t)b * S + qi) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        u32x4 w;
#pragma unroll
        for (int e = 0; e < 4; ++e) w[e] = __float_as_uint(oacc[db][4 * j + e] * inv);
        *reinterpret_cast<u32x4*>(orow + db * 32 + 8 * j + 4 * hh) = w;
      }
    if (p.lse && hh == 0)
      p.lse[((size_t)b * Hq + hq) * S + qi] =
          l_tot > 0.f ? m_run * p.scale_abs + logf(l_tot) - slope * (float)(qi - qa) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((prefill_f32_kernel<D, CAUSAL>), dim3(8 * p.per_xcd), dim3(PF32_THREADS), 0,
                     stream, p);
  return hipGetLastError();
}

}  // namespace

int prefill_rows_per_wg_f32() { return PF32_ROWS; }

hipError_t launch_prefill_f32(const PrefillParams& p, int causal, hipStream_t stream) {
  switch (p.d) {
    case 32: return causal ? launch_one<32, true>(p, stream) : launch_one<32, false>(p, stream);
    case 64: return causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
    case 128: return causal ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
