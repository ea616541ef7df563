// prefill_bf16.hip - bf16 grouped-query attention prefill on gfx950 matrix cores.
//
// Work split: one workgroup per (sequence b, K/V head kvh, block of 256 flattened
// query rows). A flattened row f = i * g + h_local stands for query position i of
// head kvh * g + h_local, so every row of a block reads the same K/V head
// (kv_head = q_head / g, blog.gitcode.com "3个GQA核心优化技巧", section
// "Flash-Attention的稀疏分组优化") and each K/V tile is staged in LDS once and
// reused by all g heads of the group (same section: K/V reuse in on-chip memory,
// access granularity raised from a head to a block).
//
// Per K/V tile of 64 keys, each of the 8 waves (32 rows each):
//   S^T = K Q^T          2 x (d/16) MFMA 32x32x16 (A = K rows from LDS, B = Q in VGPRs)
//   mask, online softmax running max / running sum (webturing.pages.dev
//   "FlashAttention Serisi", section "Ana fikir": the softmax is built as a
//   running sum so the score matrix never leaves the chip)
//   O^T += V^T P^T       (d/32) x 4 MFMA (A = V^T from LDS, B = P straight from the
//                        score accumulators, no LDS round trip)
// The result equals textbook softmax(scale Q K^T) V over the valid keys (aifullclass.xyz
// BERT self-attention article, LowRankSelfAttention example; the FlashAttention page's
// FAQ: the computed result is mathematically the same).
//
// Masks: key j is visible to query i iff j < L_b and (not causal or j <= i). K/V rows
// at or past L_b are never read (zero-filled in LDS), so padding may hold anything.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_ROWS = 32 * PF_WAVES;  // flattened query rows per workgroup
constexpr int PF_BN = 64;               // keys per K/V tile

template <int D>
struct PfLayout {
  static constexpr int KSTR = D + 8;       // bf16 per K row in LDS (pad: conflict-free b128 reads)
  static constexpr int VSTR = PF_BN + 4;   // bf16 per V^T row in LDS (pad: conflict-free b64 reads)
  static constexpr int K_ELEMS = PF_BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int CPR = D / 8;                               // 16-byte chunks per row
  static constexpr int KCH = PF_BN * CPR;                         // K chunks per tile
  static constexpr int KPT = (KCH + PF_THREADS - 1) / PF_THREADS;
  static constexpr int VBL = (PF_BN / 2) * CPR;                   // (2 keys x 8 d) V blocks
  static constexpr int VPT = (VBL + PF_THREADS - 1) / PF_THREADS;
};

template <int D, bool CAUSAL>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_bf16_kernel(PrefillParams p) {
  using Lay = PfLayout<D>;
  extern __shared__ __attribute__((aligned(16))) uint16_t smem[];

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // Launch index -> logical block. Workgroups are dealt round-robin to the 8 XCDs;
  // giving each XCD a contiguous range of logical blocks keeps the blocks of one
  // (b, kvh) unit, which share K/V, in the same L2.
  const int lin = blockIdx.x;
  const int logical = (lin & 7) * p.per_xcd + (lin >> 3);
  if (logical >= p.n_wg) return;
  const int unit = logical / p.nrb;
  int rb = logical - unit * p.nrb;
  if (CAUSAL) rb = p.nrb - 1 - rb;  // heaviest row blocks first
  const int b = unit / p.Hkv;
  const int kvh = unit - b * p.Hkv;
  const int g = p.g, S = p.S, Hq = p.Hq, Hkv = p.Hkv;

  int Lb = S;
  if (p.seqlens) {
    Lb = p.seqlens[b];
    Lb = Lb < 0 ? 0 : (Lb > S ? S : Lb);
  }
  const int R = S * g;
  const int f0 = rb * PF_ROWS;
  const int fw = f0 + wave * 32;
  const int f = fw + l32;
  const bool row_ok = f < R;
  const int qi = row_ok ? f / g : 0;
  const int hq = kvh * g + (row_ok ? f - qi * g : 0);

  int kv_end = Lb;                 // keys the workgroup visits
  int wave_kv_end = kv_end;        // keys this wave needs
  int wave_mask_from = Lb;         // first key at which some row of the wave is masked
  if (CAUSAL) {
    const int last_f = min(f0 + PF_ROWS, R) - 1;
    kv_end = min(Lb, last_f / g + 1);
    const int wf_last = min(fw + 31, R - 1);
    wave_kv_end = (fw < R) ? min(Lb, wf_last / g + 1) : 0;
    wave_mask_from = min(Lb, fw / g + 1);
  }
  const int lim = CAUSAL ? min(Lb, qi + 1) : Lb;  // keys j < lim are visible to this row
  const int ntiles = (kv_end + PF_BN - 1) / PF_BN;

  // Q^T as the B operand: lane holds query row f, d = ks*16 + hh*8 .. +7.
  bf16x8 qf[D / 16];
  {
    const uint16_t* qrow =
        static_cast<const uint16_t*>(p.q) + (((size_t)b * S + qi) * Hq + hq) * D;
    const uint32_t flip = p.negate_q ? 0x80008000u : 0u;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      u32x4 v = row_ok ? ldg16(qrow + ks * 16 + hh * 8) : zero_u32x4();
      v[0] ^= flip; v[1] ^= flip; v[2] ^= flip; v[3] ^= flip;
      qf[ks] = as_bf16x8(v);
    }
  }

  const size_t rstride = (size_t)Hkv * D;  // elements between consecutive keys (BSHD)
  const uint16_t* kbase = static_cast<const uint16_t*>(p.k) + ((size_t)b * S * Hkv + kvh) * D;
  const uint16_t* vbase = static_cast<const uint16_t*>(p.v) + ((size_t)b * S * Hkv + kvh) * D;

  u32x4 kreg[Lay::KPT], va[Lay::VPT], vb[Lay::VPT];

  auto gload = [&](int t0) {
#pragma unroll
    for (int r = 0; r < Lay::KPT; ++r) {
      const int c = tid + r * PF_THREADS;
      if (Lay::KCH % PF_THREADS == 0 || c < Lay::KCH) {
        const int key = c / Lay::CPR, col = c - key * Lay::CPR;
        const int j = t0 + key;
        kreg[r] = j < Lb ? ldg16(kbase + (size_t)j * rstride + col * 8) : zero_u32x4();
      }
    }
#pragma unroll
    for (int r = 0; r < Lay::VPT; ++r) {
      const int c = tid + r * PF_THREADS;
      if (Lay::VBL % PF_THREADS == 0 || c < Lay::VBL) {
        const int pr = c / Lay::CPR, col = c - pr * Lay::CPR;
        const int j = t0 + 2 * pr;
        va[r] = j < Lb ? ldg16(vbase + (size_t)j * rstride + col * 8) : zero_u32x4();
        vb[r] = j + 1 < Lb ? ldg16(vbase + (size_t)(j + 1) * rstride + col * 8) : zero_u32x4();
      }
    }
  };

  // K rows as loaded; V transposed in registers so each LDS row holds one d for all keys.
  auto lstore = [&](int stage) {
    uint16_t* ks_ = smem + stage * Lay::STAGE;
    uint16_t* vs_ = ks_ + Lay::K_ELEMS;
#pragma unroll
    for (int r = 0; r < Lay::KPT; ++r) {
      const int c = tid + r * PF_THREADS;
      if (Lay::KCH % PF_THREADS == 0 || c < Lay::KCH) {
        const int key = c / Lay::CPR, col = c - key * Lay::CPR;
        *reinterpret_cast<u32x4*>(ks_ + key * Lay::KSTR + col * 8) = kreg[r];
      }
    }
#pragma unroll
    for (int r = 0; r < Lay::VPT; ++r) {
      const int c = tid + r * PF_THREADS;
      if (Lay::VBL % PF_THREADS == 0 || c < Lay::VBL) {
        const int pr = c / Lay::CPR, col = c - pr * Lay::CPR;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const uint32_t a = va[r][e], bb = vb[r][e];
          const uint32_t lo = (a & 0xffffu) | (bb << 16);
          const uint32_t hi = (a >> 16) | (bb & 0xffff0000u);
          *reinterpret_cast<uint32_t*>(vs_ + (col * 8 + 2 * e) * Lay::VSTR + 2 * pr) = lo;
          *reinterpret_cast<uint32_t*>(vs_ + (col * 8 + 2 * e + 1) * Lay::VSTR + 2 * pr) = hi;
        }
      }
    }
  };

  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  if (ntiles > 0) {
    gload(0);
    lstore(0);
  }
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int t0 = t * PF_BN;
    const bool has_next = t + 1 < ntiles;
    if (has_next) gload(t0 + PF_BN);
    const uint16_t* ks_ = smem + (t & 1) * Lay::STAGE;
    const uint16_t* vs_ = ks_ + Lay::K_ELEMS;

    if (t0 < wave_kv_end) {
      // S^T = K Q^T for two 32-key blocks: lane holds query l32, keys 8(r/4)+4hh+(r%4).
      f32x16 s[2];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        s[kb] = zero16();
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks) {
          const u32x4 a =
              *reinterpret_cast<const u32x4*>(ks_ + (kb * 32 + l32) * Lay::KSTR + ks * 16 + hh * 8);
          s[kb] = mfma_bf16_32x32x16(as_bf16x8(a), qf[ks], s[kb]);
        }
      }

      const bool need_mask = t0 + PF_BN > wave_mask_from;
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int j = t0 + kb * 32 + 8 * (r >> 2) + 4 * hh + (r & 3);
            if (j >= lim) s[kb][r] = -INFINITY;
          }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
      mx = fmaxf(mx, xor32(mx));  // the other 32 keys of this query sit in lane l ^ 32
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
      float lsum = 0.f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float pv = fast_exp2(fmaf(s[kb][r], c, -msc));
          if (need_mask) pv = (s[kb][r] == -INFINITY) ? 0.f : pv;
          s[kb][r] = pv;
          lsum += pv;
        }
      l_run += lsum;

      // O^T += V^T P^T, 16 keys per MFMA: B slot i <-> key 16ks + 8(i/4) + 4hh + (i%4).
#pragma unroll
      for (int ks = 0; ks < PF_BN / 16; ++ks) {
        const int kb = ks >> 1, r0 = 8 * (ks & 1);
        const bf16x8 pb = pack_bf16x8(s[kb][r0 + 0], s[kb][r0 + 1], s[kb][r0 + 2], s[kb][r0 + 3],
                                      s[kb][r0 + 4], s[kb][r0 + 5], s[kb][r0 + 6], s[kb][r0 + 7]);
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint16_t* vp = vs_ + (db * 32 + l32) * Lay::VSTR + ks * 16 + 4 * hh;
          const u32x2 lo = *reinterpret_cast<const u32x2*>(vp);
          const u32x2 hi = *reinterpret_cast<const u32x2*>(vp + 8);
          const u32x4 a = {lo[0], lo[1], hi[0], hi[1]};
          oacc[db] = mfma_bf16_32x32x16(as_bf16x8(a), pb, oacc[db]);
        }
      }
    }
    if (has_next) lstore((t + 1) & 1);
    __syncthreads();
  }

  // Epilogue: O = O^T / l, rounded to bf16; LSE = m*|scale| + ln l.
  const float l_tot = l_run + xor32(l_run);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (row_ok) {
    uint16_t* orow = static_cast<uint16_t*>(p.o) + (((size_t)b * S + qi) * Hq + hq) * D;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int d0 = db * 32 + 8 * j + 4 * hh;
        u32x2 w;
        w[0] = pack_bf16x2(oacc[db][4 * j + 0] * inv, oacc[db][4 * j + 1] * inv);
        w[1] = pack_bf16x2(oacc[db][4 * j + 2] * inv, oacc[db][4 * j + 3] * inv);
        *reinterpret_cast<u32x2*>(orow + d0) = w;
      }
    if (p.lse && hh == 0)
      p.lse[((size_t)b * Hq + hq) * S + qi] =
          l_tot > 0.f ? m_run * p.scale_abs + logf(l_tot) : -INFINITY;
  }
}

template <int D, bool CAUSAL>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  const size_t lds = 2 * PfLayout<D>::STAGE * sizeof(uint16_t);
  auto kern = prefill_bf16_kernel<D, CAUSAL>;
  hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(kern, dim3(8 * p.per_xcd), dim3(PF_THREADS), lds, stream, p);
  return hipGetLastError();
}

}  // namespace

int prefill_rows_per_wg_bf16() { return PF_ROWS; }

hipError_t launch_prefill_bf16(const PrefillParams& p, int causal, hipStream_t stream) {
  switch (p.d) {
    case 32: return causal ? launch_one<32, true>(p, stream) : launch_one<32, false>(p, stream);
    case 64: return causal ? launch_one<64, true>(p, stream) : launch_one<64, false>(p, stream);
    case 128: return causal ? launch_one<128, true>(p, stream) : launch_one<128, false>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
