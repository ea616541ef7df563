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
// Per K/V tile of 64 keys, each of the 8 waves (32 rows each) computes
//   S^T = K Q^T          (A = K rows from LDS, B = Q held in VGPRs)
//   mask, online softmax with a running max and running sum (webturing.pages.dev
//   "FlashAttention Serisi", section "Ana fikir": the softmax is accumulated as a
//   running sum so the score matrix never leaves the chip)
//   O^T += V^T P^T       (A = V^T read from row-major LDS with the transposing
//                        ds_read_b64_tr_b16, B = P taken straight from the score
//                        accumulators)
// on v_mfma_f32_32x32x16_bf16. The loop is software-pipelined: iteration t issues the
// PV product of tile t-1 and the QK^T product of tile t+1 on the matrix cores while the
// vector ALUs run the softmax of tile t. The running max used as the exponent offset is
// refreshed only when a row's max grows by more than 2^8 (in exp2 units), so the O
// rescale is rare; the result is the same normalised softmax because every term of a
// row always shares one offset. The result equals textbook softmax(scale Q K^T) V over
// the valid keys (aifullclass.xyz BERT self-attention article, LowRankSelfAttention
// example; FlashAttention page FAQ: the computed result is mathematically the same).
//
// Masks: key j is visible to query i iff j < L_b and (not causal or j <= i). K/V rows
// at or past L_b are never read (zero-filled in LDS), so padding may hold anything.
#include "gqa_device.h"
#include "gqa_kernels.h"

#include <type_traits>

namespace gqa {
namespace {

constexpr int PF_WAVES = 8;
constexpr int PF_THREADS = 64 * PF_WAVES;
constexpr int PF_ROWS = 32 * PF_WAVES;  // flattened query rows per workgroup
// Keys per K/V tile: 64 for d <= 64, 32 for d = 128 (keeps the score and P registers of
// two tiles within the 256-VGPR budget of two waves per SIMD).
template <int D>
constexpr int kBN = D == 128 ? 32 : 64;
constexpr float kTau = 8.0f;            // exp2 headroom before the running max is refreshed
constexpr int kNK = 3;                  // K tile ring: K(t+1) read while K(t+2), K(t+3) land
constexpr int kNV = 4;                  // V tile ring: V(t-1) read while V(t..t+2) land

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;

template <int D>
struct PfLayout {
  static constexpr int BN = kBN<D>;
  static constexpr int NKB = BN / 32;               // 32-key blocks per tile
  static constexpr int NKS = BN / 16;               // 16-key MFMA steps per tile
  static constexpr int CPR = D / 8;                 // 16-byte chunks per row
  static constexpr int ROWB = D * 2;                // bytes per K or V row
  static constexpr int TILE_B = BN * ROWB;          // bytes per K or V tile
  static constexpr int NWI = BN * CPR / 64;         // 1 KB DMA wave-instructions per tile
  static constexpr int LDS_BYTES = (kNK + kNV) * TILE_B;
  // Tiles are stored unpadded (DMA writes 1 KB contiguous per wave instruction); the
  // 16-byte chunk q of row r sits at chunk position q ^ f(r). fk makes the K fragment
  // reads (16 rows x one chunk per pass) hit 16 different bank groups; fv does the same
  // for the transposing V reads (4 rows x 4 chunks per pass).
  static __device__ __forceinline__ int fk(int r) {
    return D == 128 ? (r & 15) : (D == 64 ? ((r >> 1) & 7) : ((r >> 2) & 3));
  }
  static __device__ __forceinline__ int fv(int r) {
    return D == 128 ? 4 * (r & 3) : (D == 64 ? 4 * ((r >> 1) & 1) : 0);
  }
};

typedef int i32x4 __attribute__((ext_vector_type(4)));

// Buffer resource over [base, base + num_bytes): loads at or past num_bytes return 0.
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t num_bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  i32x4 r;
  r[0] = __builtin_amdgcn_readfirstlane((uint32_t)a);
  r[1] = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32) & 0xffffu);  // stride 0
  r[2] = __builtin_amdgcn_readfirstlane(num_bytes);
  r[3] = 0x00020000;  // 32-bit data format, raw (untyped) access
  return r;
}

// Global -> LDS copy of one 16-byte chunk per lane (byte offset voff in the resource),
// 1 KB per wave, straight into LDS at m0 + 16 * lane with no VGPR staging. Out-of-range
// chunks arrive as zeros. Issued as inline asm so the compiler does not turn every later
// LDS read into a wait for all outstanding copies; the kernel waits on the
// vector-memory counter itself before each barrier.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// Wait until at most n of this wave's vector-memory operations are outstanding.
__device__ __forceinline__ void wait_vm(int n) {
  switch (n) {
    case 0: asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); break;
    case 1: asm volatile("s_waitcnt vmcnt(1)" ::: "memory"); break;
    case 2: asm volatile("s_waitcnt vmcnt(2)" ::: "memory"); break;
    case 3: asm volatile("s_waitcnt vmcnt(3)" ::: "memory"); break;
    case 4: asm volatile("s_waitcnt vmcnt(4)" ::: "memory"); break;
    case 5: asm volatile("s_waitcnt vmcnt(5)" ::: "memory"); break;
    default: asm volatile("s_waitcnt vmcnt(6)" ::: "memory"); break;
  }
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, bool CAUSAL>
__global__ __launch_bounds__(PF_THREADS, 1) void prefill_bf16_kernel(PrefillParams p) {
  using Lay = PfLayout<D>;
  constexpr int PF_BN = Lay::BN;
  constexpr int NKB = Lay::NKB, NKS = Lay::NKS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // LDS: K slots 0..kNK-1, then V slots 0..kNV-1 (byte offsets).
  auto kslot = [&](int t) { return (t % kNK) * Lay::TILE_B; };
  auto vslot = [&](int t) { return (kNK + t % kNV) * Lay::TILE_B; };

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
  const int wave_nt = (wave_kv_end + PF_BN - 1) / PF_BN;

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

  // ---- DMA of one K/V tile pair. A group is this wave's share of K(tk) then V(tv):
  // wave-instruction k (of 2 * NWI per group) is taken by wave k % 8; k < NWI copies K
  // chunk block k, otherwise V chunk block k - NWI. Each copy goes through a buffer
  // resource that ends at row L_b, so rows past the valid range land as zeros and
  // nothing outside [0, L_b) is ever read.
  constexpr int kJ = (2 * Lay::NWI + PF_WAVES - 1) / PF_WAVES;
  uint32_t voff[kJ];
  int n_k = 0, n_v = 0;
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int k = wave + PF_WAVES * j;
    const bool is_k = k < Lay::NWI;
    const int kk = is_k ? k : k - Lay::NWI;
    const int c = kk * 64 + lane;
    const int row = c / Lay::CPR, pos = c - row * Lay::CPR;
    const int q = pos ^ (is_k ? Lay::fk(row) : Lay::fv(row));
    voff[j] = (uint32_t)row * (uint32_t)(rstride * 2) + 16u * q;
    if (k < 2 * Lay::NWI) (is_k ? n_k : n_v) += 1;
  }
  const int vm_allow = n_v + n_k + n_v;  // group t-1's V part and all of group t
  const uint32_t row_bytes = (uint32_t)(rstride * 2);
  auto issue_group = [&](int tk, int tv, bool with_v) {
    const int tk0 = tk * PF_BN, tv0 = tv * PF_BN;
    const i32x4 rk = make_rsrc(kbase + (size_t)tk0 * rstride, (uint32_t)max(Lb - tk0, 0) * row_bytes);
    const i32x4 rv = make_rsrc(vbase + (size_t)tv0 * rstride, (uint32_t)max(Lb - tv0, 0) * row_bytes);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int k = wave + PF_WAVES * j;
      if (k < Lay::NWI)
        dma16(rk, voff[j], lds_base + kslot(tk) + k * 1024);
      else if (with_v && k < 2 * Lay::NWI)
        dma16(rv, voff[j], lds_base + vslot(tv) + (k - Lay::NWI) * 1024);
    }
  };

  // ---- matrix-core phases
  f32x16 oacc[D / 32];
#pragma unroll
  for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();

  // S^T = K Q^T for two 32-key blocks: lane holds query l32, keys 8(r/4)+4hh+(r%4).
  // Chunk (2ks + hh) of row kb*32 + l32 sits at position (2ks + hh) ^ fk(l32).
  const int k_lane = l32 * Lay::ROWB + 16 * (hh ^ (Lay::fk(l32) & 1));
  const int k_swz = Lay::fk(l32) & ~1;
  auto qk = [&](f32x16 (&s)[NKB], int slot_off) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const int off = slot_off + k_lane + 16 * ((2 * ks) ^ k_swz);
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(smem + off + kb * 32 * Lay::ROWB);
        s[kb] = mfma_bf16_32x32x16(as_bf16x8(a), qf[ks], ks == 0 ? zero16() : s[kb]);
      }
    }
  };
  // O^T += V^T P^T, 16 keys per MFMA; B slot i <-> key 16ks + 8(i/4) + 4hh + (i%4).
  // The transposing read hands lane (group G = lane/16, i = lane%16) keys
  // 16ks + 4(G/2) + {0..3} (and +8) of output column d = db*32 + (lane % 32): lane i of a
  // group supplies the address of row 4(G/2) + i/4, columns db*32 + 16(G%2) + 4(i%4) .. +3.
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_q = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within the 32 columns
  const int v_lane = tr_row * Lay::ROWB + 8 * (lane & 1);
  const int v_swz = Lay::fv(tr_row);  // the same for every (ks, db, +8 rows)
  auto pv = [&](const bf16x8 (&pp)[NKS], int slot_off) {
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int off = slot_off + ks * 16 * Lay::ROWB + v_lane + 16 * ((4 * db + tr_q) ^ v_swz);
        const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + off));
        const s16x4 hi =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + off + 8 * Lay::ROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo), h2 = __builtin_bit_cast(u32x2, hi);
        const u32x4 a = {l2[0], l2[1], h2[0], h2[1]};
        oacc[db] = mfma_bf16_32x32x16(as_bf16x8(a), pp[ks], oacc[db]);
      }
    }
  };

  // ---- online softmax state (one query row per lane; lanes l and l^32 share a row)
  float m_run = -INFINITY, l_run = 0.f;
  const float c = p.scale_log2;

  // Key j = t0 + kb*32 + 8(r/4) + 4hh + (r%4) is kept iff j < lim: the sign of j - lim
  // selects between the score and -inf bit patterns (no compare masks in SGPRs).
  auto mask = [&](f32x16 (&s)[NKB], int t0) {
    const int base = t0 + 4 * hh - lim;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t keep = (uint32_t)((base + kb * 32 + 8 * (r >> 2) + (r & 3)) >> 31);
        s[kb][r] = __uint_as_float((__float_as_uint(s[kb][r]) & keep) | (0xff800000u & ~keep));
      }
  };
  // Returns this lane's rescale factor for O; P goes to pp as bf16.
  auto softmax = [&](f32x16 (&s)[NKB], bf16x8 (&pp)[NKS]) -> float {
    float mx = m_run;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    mx = fmaxf(mx, xor32(mx));  // the other 32 keys of this row sit in lane l ^ 32
    const bool fresh = m_run == -INFINITY;
    const bool refresh = fresh ? (mx != -INFINITY) : ((mx - m_run) * c > kTau);
    const float m_new = refresh ? mx : m_run;
    const float alpha = refresh ? (fresh ? 0.f : fast_exp2((m_run - m_new) * c)) : 1.f;
    m_run = m_new;
    const float msc = (m_new == -INFINITY ? 0.f : m_new) * c;
    float lsum = 0.f;
#pragma unroll
    for (int ks = 0; ks < NKS; ++ks) {
      const int kb = ks >> 1, r0 = 8 * (ks & 1);
      float e[8];
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        e[i] = fast_exp2(fmaf(s[kb][r0 + i], c, -msc));  // masked: exp2(-inf) = 0 as c > 0
      }
      u32x4 u;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        u[i] = pack_bf16x2(e[2 * i], e[2 * i + 1]);
        lsum += e[2 * i] + e[2 * i + 1];
      }
      pp[ks] = as_bf16x8(u);
    }
    l_run = l_run * alpha + lsum;
    return alpha;
  };
  auto rescale = [&](float alpha) {
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
  };

  // ---- pipeline: iteration t runs PV(t-1), QK(t+1) and softmax(t) while the DMA of
  // K(t+3) and V(t+2) is in flight (K(t+1), V(t-1) are read; K(t+2), V(t), V(t+1) may
  // still be landing). Every wave runs every tile of the workgroup (tiles past a causal
  // wave's rows are fully masked and add nothing); the QK of the last iteration reads a
  // tile that is not used. The loop is unrolled by two with the register roles swapped,
  // so no accumulator is ever copied.
  f32x16 s_a[NKB], s_b[NKB];
  bf16x8 pp_a[NKS], pp_b[NKS];
  if (ntiles > 0) {
    issue_group(0, 0, false);
    issue_group(1, 0, true);
    issue_group(2, 1, true);
    wait_vm(0);
  }
  block_barrier();
  if (ntiles > 0) qk(s_a, kslot(0));
  block_barrier();  // every wave has read K(0) before K(3) replaces it

  auto step = [&](auto do_pv, int t, f32x16 (&s_cur)[NKB], f32x16 (&s_nxt)[NKB],
                  bf16x8 (&pp_prev)[NKS], bf16x8 (&pp_cur)[NKS]) {
    __builtin_amdgcn_sched_barrier(0);
    issue_group(t + 3, t + 2, true);
    if (t * PF_BN + PF_BN > wave_mask_from) mask(s_cur, t * PF_BN);
    __builtin_amdgcn_sched_barrier(0);
    // One scheduling region: matrix-core products of tiles t-1 and t+1 interleaved with
    // the vector-ALU softmax of tile t (each MFMA is followed by a slice of the VALU work).
    constexpr bool kPV = decltype(do_pv)::value;
    if constexpr (kPV) pv(pp_prev, vslot(t - 1));
    qk(s_nxt, kslot(t + 1));
    const float alpha = softmax(s_cur, pp_cur);
    constexpr int kMfma = (kPV ? NKS * (D / 32) : 0) + NKB * (D / 16);
    constexpr int kValuPer = (kMfma >= 32 ? 4 : (kMfma >= 16 ? 7 : 14));
#pragma unroll
    for (int i = 0; i < kMfma; ++i) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
      __builtin_amdgcn_sched_group_barrier(0x002, kValuPer, 0);
    }
    // Pin P(t) here: without a use inside the region the compiler sinks the exponentials
    // into the next step, next to their consumer, and nothing overlaps the MFMAs.
#pragma unroll
    for (int i = 0; i < NKS; ++i) asm volatile("" ::"v"(pp_cur[i]));
    __builtin_amdgcn_sched_barrier(0);
    if (wave_any(alpha != 1.f)) rescale(alpha);  // after PV(t-1), before PV(t)
    wait_vm(vm_allow);  // this wave's copies of K(t+2) and V(t) have landed
    block_barrier();    // ... and every other wave's
  };
  using no_pv = std::integral_constant<bool, false>;
  using with_pv = std::integral_constant<bool, true>;
  int t = 1;
  if (ntiles > 0) {
    step(no_pv{}, 0, s_a, s_b, pp_b, pp_a);
    for (; t + 1 < ntiles; t += 2) {
      step(with_pv{}, t, s_b, s_a, pp_a, pp_b);
      step(with_pv{}, t + 1, s_a, s_b, pp_b, pp_a);
    }
    if (t < ntiles) step(with_pv{}, t, s_b, s_a, pp_a, pp_b);
    // PV of the last tile: its P sits in pp_a when ntiles is odd, pp_b when even.
    if (ntiles & 1)
      pv(pp_a, vslot(ntiles - 1));
    else
      pv(pp_b, vslot(ntiles - 1));
    wait_vm(0);  // drain the copies issued for tiles past the end
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
  const size_t lds = PfLayout<D>::LDS_BYTES;
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
