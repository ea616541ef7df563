// prefill_bf16.hip - bf16 grouped-query attention prefill on gfx950 matrix cores.
//
// Work split: one work item per (sequence b, K/V head kvh, block of flattened query
// rows), one workgroup per item (d <= 64) or a resident workgroup working through a
// share of the items (d = 128). A flattened row f = i * g + h_local stands for query
// position i of head kvh * g + h_local, so every row of a block reads the same K/V head
// (kv_head = q_head / g, blog.gitcode.com "3个GQA核心优化技巧", section
// "Flash-Attention的稀疏分组优化") and each K/V tile is staged in LDS once and reused by
// all g heads of the group (same section: K/V reuse in on-chip memory, access
// granularity raised from a head to a block).
//
// Per K/V tile (64 keys, 32 for d = 128), each wave (32 rows) computes
//   S^T = K Q^T          (A = K rows from LDS, B = Q held in VGPRs)
//   mask, online softmax with a running max and running sum (webturing.pages.dev
//   "FlashAttention Serisi", section "Ana fikir": the softmax is accumulated as a
//   running sum so the score matrix never leaves the chip)
//   O^T += V^T P^T       (A = V^T read from row-major LDS with the transposing
//                        ds_read_b64_tr_b16, B = P taken straight from the score
//                        accumulators)
// on v_mfma_f32_32x32x16_bf16. The kernel is kept small (at most 128 VGPRs for d <= 64,
// 168 for d = 128 without ALiBi) so that several waves share each SIMD (four, or three for
// d = 128; two for d = 128 with ALiBi) and the hardware overlaps one wave's matrix
// products with another wave's softmax. K/V tiles stream from HBM/L2 straight into an LDS
// ring (4 slots, 3 with three workgroups per CU), RING - 1 tiles ahead of their use. The
// exponent offset is a row max that is raised only when a tile's weights would exceed
// 2^32, so the O rescale is rare; every term of a row always shares one offset, so the
// normalised result is unchanged. The result equals textbook softmax(scale Q K^T) V
// over the valid keys (aifullclass.xyz BERT self-attention article, LowRankSelfAttention
// example; FlashAttention page FAQ: the computed result is mathematically the same).
//
// Masks: key j is visible to query i iff j < L_b and (not causal or j <= i). K/V rows
// at or past L_b are never read (they arrive in LDS as zeros), so padding may hold
// anything. Options (template flags, so the plain kernels carry none of their code): a
// causal sliding window (keys j > i - w; tiles below every row's window are skipped) and
// ALiBi (score - slope_h |i - j|). Causal ALiBi visits each item's tiles from the diagonal
// down, with the bias folded into the accumulators and the exponent offset.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr float kSumCap = 4294967296.0f;  // 2^32: a tile's weights stay at most this large

// Waves per workgroup and workgroups per CU for head size D (and the ALiBi flag, whose
// extra registers change the d = 128 choice).
template <int D, bool ALIBI = false>
struct PfShape {
  // Keys per K/V tile: 64 while the registers allow four waves per SIMD, 32 for d = 128.
  static constexpr int BN = D == 128 ? 32 : 64;
  static constexpr int WAVES = D == 128 ? 4 : 8;
  // d = 128: three 4-wave workgroups per CU, so three waves share each SIMD (at most 168
  // VGPRs each) and hide each other's LDS and matrix-core latencies (5 % faster than two
  // workgroups on the causal Llama-shaped prefill). The ALiBi kernels spill 16-23
  // registers at that budget, so they keep two workgroups per CU (256 VGPRs, no spills).
  // d <= 64: two 8-wave workgroups (four waves per SIMD at 128 VGPRs).
  static constexpr bool THREE = D == 128 && !ALIBI;
  static constexpr int WG_PER_CU = THREE ? 3 : 2;
  static constexpr int THREADS = 64 * WAVES;
  static constexpr int ROWS = 32 * WAVES;
  static constexpr int WAVES_PER_SIMD = WG_PER_CU * WAVES / 4;  // register budget 512 / this
  // LDS slots per K and per V ring, and tiles in flight ahead of the one being read.
  // With two workgroups per CU the 64 KB ring (4 slots) lets both share it (a 3-slot ring
  // measured slower); with three (d = 128), 3-slot rings (48 KB each).
  static constexpr int RING = THREE ? 3 : 4;
  // Read all of a tile's K or V^T fragments before its products: ~3 % faster at d = 128
  // with two waves per SIMD, but beyond the 168-register budget of three.
  static constexpr bool BATCH_READS = D == 128 && !THREE;
  static constexpr int AHEAD = RING - 1;
  // Persistent launch: one resident workgroup per slot works through a share of its XCD's
  // queue. Used for d = 128 (one wave per SIMD per workgroup), where the two workgroups
  // of a CU progress at the same rate. With two waves per SIMD per workgroup (d <= 64) the
  // older workgroup of a CU takes most issue slots and a static share leaves the younger
  // one finishing alone, so there every item gets its own workgroup and the hardware
  // dispatcher balances the queue.
  static constexpr bool PERSISTENT = D == 128;
};

typedef __attribute__((__vector_size__(4 * sizeof(short)))) short s16x4;
typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
typedef int i32x4 __attribute__((ext_vector_type(4)));

template <int D, bool ALIBI>
struct PfLayout {
  static constexpr int BN = PfShape<D, ALIBI>::BN;
  static constexpr int NKB = BN / 32;            // 32-key score blocks per tile
  static constexpr int NKS = BN / 16;            // 16-key MFMA steps per tile
  static constexpr int CPR = D / 8;              // 16-byte chunks per row
  static constexpr int ROWB = D * 2;             // bytes per K or V row
  static constexpr int TILE_B = BN * ROWB;       // bytes per K or V tile
  static constexpr int NWI = BN * CPR / 64;      // 1 KB DMA wave-instructions per tile
  static constexpr int LDS_BYTES = 2 * PfShape<D, ALIBI>::RING * TILE_B;
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
// vector-memory counter itself before each barrier. The compiler inserts no hazard waits
// around inline asm, so the asm carries them: on GFX9 a buffer instruction must issue at
// least 5 wait states after a vector instruction wrote one of its descriptor's SGPRs
// (make_rsrc's readfirstlane calls) and an LDS copy at least 1 after a scalar write of M0.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_addr) {
  asm volatile("s_nop 4\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(voff), "s"(rsrc),
               "{m0}"(__builtin_amdgcn_readfirstlane(lds_addr))
               : "memory");
}

// Wait until at most n (a compile-time constant) vector-memory operations of this wave
// are outstanding.
template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N <= 63, "vmcnt range");
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}

__device__ __forceinline__ void block_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

template <int D, bool CAUSAL, bool WINDOW, bool ALIBI, bool EXACT_SUM>
__global__ __launch_bounds__((PfShape<D, ALIBI>::THREADS),
                             (PfShape<D, ALIBI>::WAVES_PER_SIMD)) void
prefill_bf16_kernel(PrefillParams p) {
  using Lay = PfLayout<D, ALIBI>;
  using Shp = PfShape<D, ALIBI>;
  constexpr int WAVES = Shp::WAVES;
  constexpr int ROWS = Shp::ROWS;
  constexpr int PF_BN = Lay::BN;
  constexpr int NKB = Lay::NKB, NKS = Lay::NKS;
  constexpr bool kBatchReads = Shp::BATCH_READS;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const uint32_t lds_base = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint8_t*)smem;
  // LDS: K slots 0..RING-1, then V slots 0..RING-1 (byte offsets).
  constexpr int kRing = Shp::RING, kAhead = Shp::AHEAD;
  auto kslot = [](int t) { return (t % kRing) * Lay::TILE_B; };
  auto vslot = [](int t) { return (kRing + t % kRing) * Lay::TILE_B; };

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  // ---- Work list. The (b, kvh, row block) items are dealt to 8 XCD queues (launch index
  // lin runs on XCD lin % 8); all row blocks of one (b, kvh) unit, which share K/V, sit in
  // one queue so the unit's K/V stays in that XCD's L2. The grid holds P = gridDim.x / 8
  // resident workgroups per XCD; slot s of an XCD takes queue positions s, 2P-1-s, 2P+s,
  // 4P-1-s, ... (snake order), so with each queue ordered heaviest first every slot gets
  // about the same amount of work. A workgroup streams the K/V tiles of all its items
  // through one LDS ring: the next item's first tiles are in flight while the current item
  // finishes, and no workgroup start-up or tail is paid per item.
  const int g = p.g, S = p.S, Hq = p.Hq, Hkv = p.Hkv;
  const int R = S * g;
  const int lin = blockIdx.x;
  const int xcd = lin & 7, slot = lin >> 3, P = gridDim.x >> 3;
  int* s_len = reinterpret_cast<int*>(smem + Lay::LDS_BYTES);  // [B] clamped L_b
  int* s_order = s_len + kPrefillLptMaxB;                       // [rank] -> sequence
  if (p.lpt) {
    // Ragged batch: sort the sequences by length (longest first, ties by index); the
    // units of that order are dealt to the XCD queues in snake order 0..7, 7..0, ..., so
    // every queue gets about the same number of key tiles, longest units first.
    for (int i = tid; i < p.B; i += Shp::THREADS) {
      const int L = p.seqlens[i];
      s_len[i] = L < 0 ? 0 : (L > S ? S : L);
    }
    __syncthreads();
    for (int i = tid; i < p.B; i += Shp::THREADS) {
      const int Li = s_len[i];
      int rank = 0;
      for (int j = 0; j < p.B; ++j) {
        const int Lj = s_len[j];
        rank += (Lj > Li) | ((Lj == Li) & (j < i));
      }
      s_order[rank] = i;
    }
    __syncthreads();
  }
  // Sequence lengths read with a uniform index go through the scalar cache (the array
  // does not change during the kernel), so they never wait on the vector-memory counter.
  const __attribute__((address_space(4))) int* seqlens_k =
      (const __attribute__((address_space(4))) int*)p.seqlens;
  struct Item {
    int b, kvh, rb, Lb;
  };
  // Item k of this workgroup; false past the end of its share (positions grow with k).
  auto get_item = [&](int k, Item& it) -> bool {
    const int qpos = (k & 1) ? (k + 1) * P - 1 - slot : k * P + slot;
    if (qpos >= p.per_xcd) return false;
    if (p.lpt) {
      const int upos = qpos / p.nrb;                          // unit slot in this queue
      const int r = 8 * upos + ((upos & 1) ? 7 - xcd : xcd);  // rank of the unit
      if (r >= p.B * Hkv) return false;
      const int rank_b = r / Hkv;
      it.kvh = r - rank_b * Hkv;
      it.rb = qpos - upos * p.nrb;
      it.b = __builtin_amdgcn_readfirstlane(s_order[rank_b]);
      it.Lb = __builtin_amdgcn_readfirstlane(s_len[it.b]);
    } else {
      const int logical = xcd * p.per_xcd + qpos;  // each XCD: a contiguous range
      if (logical >= p.n_wg) return false;
      const int unit = logical / p.nrb;
      it.rb = logical - unit * p.nrb;
      it.b = unit / Hkv;
      it.kvh = unit - it.b * Hkv;
      it.Lb = S;
      if (p.seqlens) {
        const int L = seqlens_k[it.b];
        it.Lb = L < 0 ? 0 : (L > S ? S : L);
      }
    }
    if (CAUSAL) it.rb = p.nrb - 1 - it.rb;  // heaviest row blocks first
    return true;
  };
  // Key tiles [t_first, ntiles) that the workgroup visits for an item. With a sliding
  // window, key j must also satisfy j >= i - window + 1: tiles below the lowest row's
  // bound are skipped.
  auto item_tiles = [&](const Item& it, int& t_first, int& ntiles) {
    const int f0 = it.rb * ROWS;
    int kv_end = it.Lb;
    if (CAUSAL) kv_end = min(it.Lb, (min(f0 + ROWS, R) - 1) / g + 1);
    ntiles = (kv_end + PF_BN - 1) / PF_BN;
    t_first = WINDOW ? max(0, f0 / g - p.window + 1) / PF_BN : 0;
  };

  const size_t rstride = (size_t)Hkv * D;  // elements between consecutive keys (BSHD)
  const uint32_t row_bytes = (uint32_t)(rstride * 2);
  const uint16_t* const k_all = static_cast<const uint16_t*>(p.k);
  const uint16_t* const v_all = static_cast<const uint16_t*>(p.v);

  // ---- DMA of one K/V tile pair. Wave-instruction k (of 2 * NWI per tile pair) is taken
  // by wave k % WAVES; k < NWI copies K chunk block k, otherwise V chunk block k - NWI.
  // Each copy goes through a buffer resource that ends at row L_b, so rows past the valid
  // range land as zeros and nothing outside [0, L_b) is ever read.
  // With fewer copies than waves (d = 32) the extra waves repeat a copy (same bytes to
  // the same place), so every wave issues exactly kJ copies and waits on the same count.
  constexpr int kCopies = 2 * Lay::NWI;
  static_assert(kCopies % WAVES == 0 || WAVES % kCopies == 0, "uniform copy count");
  constexpr int kJ = kCopies >= WAVES ? kCopies / WAVES : 1;  // copies per wave per tile pair
  uint32_t voff[kJ];
  int kidx[kJ];
#pragma unroll
  for (int j = 0; j < kJ; ++j) {
    const int k = (wave + WAVES * j) % kCopies;
    kidx[j] = k;
    const bool is_k = k < Lay::NWI;
    const int c = (is_k ? k : k - Lay::NWI) * 64 + lane;
    const int row = c / Lay::CPR, pos = c - row * Lay::CPR;
    const int q = pos ^ (is_k ? Lay::fk(row) : Lay::fv(row));
    voff[j] = (uint32_t)row * row_bytes + 16u * q;
  }
  // Causal ALiBi visits an item's key tiles nearest-first (from the diagonal down to key
  // 0): the bias then only falls from one tile to the next, so the exponent offset taken
  // from the first tile a row sees keys in stays above the later tiles' scores as it does
  // without a bias. (In key order each tile nearer the diagonal would raise the scores by
  // up to slope * tile width and could force the redo below on many tiles.)
  constexpr bool kNearFirst = CAUSAL && ALIBI;
  // Issue cursor: the next tile to copy is position it_t of item it_k's tiles [it_first,
  // it_end) (key tile it_t, or it_first + it_end - 1 - it_t when nearest-first); it_kp /
  // it_vp point at the item's K and V rows, it_L is its length.
  int it_k = -1, it_t = 0, it_first = 0, it_end = 0, it_L = 0;
  bool live = true;
  const uint16_t* it_kp = k_all;
  const uint16_t* it_vp = v_all;
  auto seek = [&]() {  // move the cursor to the next item that has tiles
    for (;;) {
      Item n;
      if (!get_item(++it_k, n)) {
        live = false;
        it_t = 0;
        it_L = 0;
        return;
      }
      int t0, nt;
      item_tiles(n, t0, nt);
      if (t0 < nt) {
        it_t = t0;
        it_first = t0;
        it_end = nt;
        it_L = n.Lb;
        it_kp = k_all + ((size_t)n.b * S * Hkv + n.kvh) * D;
        it_vp = v_all + ((size_t)n.b * S * Hkv + n.kvh) * D;
        return;
      }
    }
  };
  // Copy the cursor's tile into ring position u and advance. Past the last item the copy
  // has an empty resource and zeros land in the (free) slot: every wave issues the same
  // number of copies per ring position, which keeps the waits below exact.
  auto issue = [&](int u) {
    // (past the last tile it_L is 0, so the copy is empty whatever tile it names)
    const int t0 = (kNearFirst && live ? it_first + it_end - 1 - it_t : it_t) * PF_BN;
    const uint32_t valid = (uint32_t)max(it_L - t0, 0) * row_bytes;
    const i32x4 rk = make_rsrc(it_kp + (size_t)t0 * rstride, valid);
    const i32x4 rv = make_rsrc(it_vp + (size_t)t0 * rstride, valid);
#pragma unroll
    for (int j = 0; j < kJ; ++j) {
      const int k = kidx[j];
      if (k < Lay::NWI)
        dma16(rk, voff[j], lds_base + kslot(u) + k * 1024);
      else
        dma16(rv, voff[j], lds_base + vslot(u) + (k - Lay::NWI) * 1024);
    }
    if (live && ++it_t == it_end) {
      if constexpr (Shp::PERSISTENT)
        seek();
      else
        live = false, it_L = 0;  // one item per workgroup
    }
  };

  // ---- per-lane constants of the fragment layouts
  // S^T = K Q^T for a 32-key block: lane holds query l32, keys 8(r/4)+4hh+(r%4).
  // Chunk (2ks + hh) of row l32 sits at position (2ks + hh) ^ fk(l32).
  const int k_lane = l32 * Lay::ROWB + 16 * (hh ^ (Lay::fk(l32) & 1));
  const int k_swz = Lay::fk(l32) & ~1;
  // O^T += V^T P^T, 16 keys per MFMA; B slot i <-> key 16ks + 8(i/4) + 4hh + (i%4).
  // The transposing read hands lane (group G = lane/16, i = lane%16) keys
  // 16ks + 4(G/2) + {0..3} (and +8) of output column d = db*32 + (lane % 32): lane i of a
  // group supplies the address of row 4(G/2) + i/4, columns db*32 + 16(G%2) + 4(i%4) .. +3.
  const int tr_row = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tr_q = 2 * ((lane >> 4) & 1) + ((lane & 3) >> 1);  // chunk within the 32 columns
  const int v_lane = tr_row * Lay::ROWB + 8 * (lane & 1);
  const int v_swz = Lay::fv(tr_row);  // the same for every (ks, db, +8 rows)
  const float c = p.scale_log2;
  const bf16x2 ones2 = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  // A negative softmax scale: the kernel works with the negated scores -q.k (and |scale|),
  // so masked scores are +inf before the sign is applied.
  const float sgn = p.negate_q ? -1.f : 1.f;
  const float cs = c * sgn;
  const uint32_t masked_bits = p.negate_q ? 0x7f800000u : 0xff800000u;

  Item cur;
  if (!get_item(0, cur)) return;  // uniform: no work for this workgroup
  seek();
  // ---- pipeline: the copy of ring position u + kAhead is issued while position u is
  // computed (after its scores are read, so a wait for Q never covers it); after position
  // u each wave waits for its own copies of u + 1 and the barrier publishes everyone's.
  // The first copies are issued after the first item's Q loads, so the two overlap.
  int u = 0;

  for (int item_no = 0;; ++item_no) {
    if (item_no > 0 && (!Shp::PERSISTENT || !get_item(item_no, cur))) break;
    const int b = cur.b, kvh = cur.kvh, Lb = cur.Lb;
    const int f0 = cur.rb * ROWS;
    const int fw = f0 + wave * 32;
    const int f = fw + l32;
    const bool row_ok = f < R;
    const int qi = row_ok ? f / g : 0;  // rows past the end compute row 0, never stored
    const int hq = kvh * g + (row_ok ? f - qi * g : 0);

    int wave_kv_end = Lb;     // keys this wave needs
    int wave_mask_from = Lb;  // first key at which some row of the wave is masked
    if (CAUSAL) {
      const int wf_last = min(fw + 31, R - 1);
      wave_kv_end = (fw < R) ? min(Lb, wf_last / g + 1) : 0;
      wave_mask_from = min(Lb, fw / g + 1);
    }
    const int lim = CAUSAL ? min(Lb, qi + 1) : Lb;  // keys j < lim are visible to this row
    int t_first, ntiles;
    item_tiles(cur, t_first, ntiles);
    const int wave_nt = (wave_kv_end + PF_BN - 1) / PF_BN;
    constexpr int kNoLo = -(1 << 30);
    int lo = kNoLo, wave_t0 = 0, wave_lo_hi = kNoLo;
    if constexpr (WINDOW) {
      lo = qi - p.window + 1;
      if (fw < R) {
        wave_t0 = max(0, fw / g - p.window + 1) / PF_BN;
        wave_lo_hi = min(fw + 31, R - 1) / g - p.window + 1;  // highest bound in the wave
      }
    }

    // Q^T as the B operand: lane holds query row f, d = ks*16 + hh*8 .. +7.
    bf16x8 qf[D / 16];
    {
      const uint16_t* qrow =
          static_cast<const uint16_t*>(p.q) + (((size_t)b * S + qi) * Hq + hq) * D;
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) qf[ks] = as_bf16x8(ldg16(qrow + ks * 16 + hh * 8));
    }
    if (item_no == 0) {
#pragma unroll
      for (int a = 0; a < kAhead; ++a) issue(a);
      wait_vm<kJ * (kAhead - 1)>();  // position 0 has landed
      block_barrier();
    }
    // Take the compiler's wait for the Q loads here, once per item: its first real use is
    // inside the tile loop, where the wait would otherwise be repeated on every tile (and,
    // not knowing about the copies, it waits for all of them).
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) asm volatile("" ::"v"(qf[ks]));

    f32x16 oacc[D / 32];
#pragma unroll
    for (int i = 0; i < D / 32; ++i) oacc[i] = zero16();

    // ALiBi: the score gets -slope_h * |i - j|, i.e. -beta * |i - j| in the units of the
    // raw dot product that c = |scale| * log2(e) scales into exp2 units.
    const float slope = ALIBI ? p.alibi[hq] : 0.f;
    const float beta = slope * kLog2e / c;
    // The bias is measured from key qa = min(i, L_b - 1), the visible key nearest to the
    // query: when i >= L_b every key lies below qa, so |i - j| = |qa - j| + (i - qa). The
    // constant slope * (i - qa) drops out of the softmax and is added back to the LSE; it
    // keeps the offsets of rows far past a short key range near the size of their scores.
    const int qa = ALIBI ? min(qi, Lb - 1) : qi;
    // Causal ALiBi is linear in the key: every visible key has j <= qa, so the bias is
    // beta * (j - qa) = beta * (t0 + 4hh - qa) + beta * jj(kb, r), a per-tile term plus a
    // per-slot term that does not change between tiles. The per-slot term starts the score
    // accumulators (the products add onto it: sgn * jj * beta, so that sgn * s comes out
    // biased), and the per-tile term joins the exponent offset, so the bias costs no
    // instruction per score. Masked keys are overwritten by the mask.
    constexpr bool kLinBias = CAUSAL && ALIBI;
    const float sbeta = sgn * beta;
    auto alibi_off = [](int kb, int i) { return (float)(32 * kb + 8 * (i >> 2) + (i & 3)); };

    // S^T = K Q^T. Each fragment read feeds its product directly, which keeps the register
    // budgets (four waves per SIMD at d <= 64, three at d = 128); kBatchReads reads all of
    // a tile's fragments first.
    auto qk = [&](f32x16 (&sc)[NKB], int slot_off) {
      auto kfrag = [&](int ks, int kb) {
        return *reinterpret_cast<const u32x4*>(smem + slot_off + kb * 32 * Lay::ROWB + k_lane +
                                               16 * ((2 * ks) ^ k_swz));
      };
      if constexpr (kLinBias) {
        float sb = sbeta;
        // (d <= 64: recomputed per tile rather than kept live across the loop)
        if constexpr (D <= 64) asm volatile("" : "+v"(sb));
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int i = 0; i < 16; ++i) sc[kb][i] = sb * alibi_off(kb, i);
      } else {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) sc[kb] = zero16();
      }
      if constexpr (kBatchReads) {
        u32x4 kf[D / 16][NKB];
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb) kf[ks][kb] = kfrag(ks, kb);
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            sc[kb] = mfma_bf16_32x32x16(as_bf16x8(kf[ks][kb]), qf[ks], sc[kb]);
      } else {
#pragma unroll
        for (int ks = 0; ks < D / 16; ++ks)
#pragma unroll
          for (int kb = 0; kb < NKB; ++kb)
            sc[kb] = mfma_bf16_32x32x16(as_bf16x8(kfrag(ks, kb)), qf[ks], sc[kb]);
      }
    };
    // O^T += V^T P^T, 16 keys per MFMA; B slot i <-> key 16ks + 8(i/4) + 4hh + (i%4). The
    // V^T fragments come from transposing reads.
    auto pv = [&](const bf16x8 (&pp)[NKS], int slot_off) {
      auto vfrag = [&](int ks, int db) {
        const int off = slot_off + ks * 16 * Lay::ROWB + v_lane + 16 * ((4 * db + tr_q) ^ v_swz);
        const s16x4 lo4 = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + off));
        const s16x4 hi4 =
            __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4*)(smem + off + 8 * Lay::ROWB));
        const u32x2 l2 = __builtin_bit_cast(u32x2, lo4), h2 = __builtin_bit_cast(u32x2, hi4);
        return u32x4{l2[0], l2[1], h2[0], h2[1]};
      };
      if constexpr (kBatchReads) {
        u32x4 vf[NKS][D / 32];
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int db = 0; db < D / 32; ++db) vf[ks][db] = vfrag(ks, db);
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            oacc[db] = mfma_bf16_32x32x16(as_bf16x8(vf[ks][db]), pp[ks], oacc[db]);
      } else {
#pragma unroll
        for (int ks = 0; ks < NKS; ++ks)
#pragma unroll
          for (int db = 0; db < D / 32; ++db)
            oacc[db] = mfma_bf16_32x32x16(as_bf16x8(vfrag(ks, db)), pp[ks], oacc[db]);
      }
    };

    // ---- online softmax state (one query row per lane; lanes l and l^32 share a row)
    // With a window or nearest-first order, m_run stays -inf until the row sees a key;
    // otherwise key 0 is visible to every row and the first tile always sets it.
    constexpr bool kLateStart = WINDOW || kNearFirst;
    float m_run = kLateStart ? -INFINITY : 0.f, l_run = 0.f;
    float lx_run = 0.f;  // EXACT_SUM: running sum of the fp32 weights (for the LSE)

    // Key j = t0 + 32kb + 8(i/4) + 4hh + (i%4) is kept iff lo <= j < lim: the signs of
    // j - lim and j - lo select between the score and the masked bit pattern (no compare
    // masks in SGPRs).
    auto mask = [&](f32x16 (&sc)[NKB], int t0) {
      const int base = t0 + 4 * hh - lim;
      const int base_lo = t0 + 4 * hh - lo;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int jj = 32 * kb + 8 * (i >> 2) + (i & 3);
          uint32_t keep = (uint32_t)((base + jj) >> 31);
          if constexpr (WINDOW) keep &= ~(uint32_t)((base_lo + jj) >> 31);
          sc[kb][i] = __uint_as_float((__float_as_uint(sc[kb][i]) & keep) | (masked_bits & ~keep));
        }
    };
    // Mask tile t's scores if any key of the wave's rows is masked in it.
    auto prep = [&](f32x16 (&sc)[NKB], int t) {
      const int t0 = t * PF_BN;
      if (t0 + PF_BN > wave_mask_from || (WINDOW && t0 < wave_lo_hi)) mask(sc, t0);
    };
    // ALiBi distance |qa - j| of this lane's score (kb, i) in tile t: key j = t0 + 32kb +
    // 8(i/4) + 4hh + (i%4), so qa - j = dq(t) - (32kb + 8(i/4) + i%4).
    // (The empty asm hides where dq came from, so the compiler recomputes the distances in
    // each use instead of keeping 32 of them live between the row max and the weights.)
    auto alibi_dq = [&](int t) {
      float dq = (float)(qa - t * PF_BN - 4 * hh);
      asm volatile("" : "+v"(dq));
      return dq;
    };
    // Row max of the (signed, biased) scores over the tile (the row's other keys sit in lane
    // l ^ 32).
    auto row_max = [&](const f32x16 (&sc)[NKB], int t) {
      float mx = -INFINITY;
      const float dq = ALIBI ? alibi_dq(t) : 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          float x = sc[kb][i] * sgn;
          if constexpr (ALIBI && !kLinBias) x = fmaf(-beta, fabsf(dq - alibi_off(kb, i)), x);
          mx = fmaxf(mx, x);
        }
      if constexpr (kLinBias) mx = fmaf(-beta, dq, mx);  // the per-tile bias term
      return pair_max(mx);
    };
    // A new exponent offset from tile t's scores: their row max, and with non-causal ALiBi
    // that max raised by the tile's largest bias |i - j| * beta (at least 0, at most kLift
    // exp2 units). The tiles walk towards the diagonal and then away from it, and the lift
    // keeps the nearer tiles under the offset, where the plain max of far, strongly biased
    // keys would be passed by each of them. The cap keeps the tile's largest weight at or
    // above 2^-kLift, so a row's weights never all underflow; the floor keeps a negative
    // slope from lowering the offset below the tile's own max.
    auto new_offset = [&](const f32x16 (&sc)[NKB], int t) {
      float mx = row_max(sc, t);
      if constexpr (ALIBI && !CAUSAL) {
        constexpr float kLift = 64.f;
        const float t0 = (float)(t * PF_BN), fq = (float)qa;
        const float reach = fmaxf(fabsf(fq - t0), fabsf(fq - t0 - (float)(PF_BN - 1)));
        mx += fminf(fmaxf(beta * reach, 0.f), kLift / c);
      }
      return mx;
    };
    // Weights exp2(c sgn s - c m) rounded to bf16 as the PV operand; returns this lane's sum
    // of the rounded weights (the values the PV product uses, one dot2 per pair: the output
    // is normalised by exactly the weights it sums, so a row dominated by one key keeps that
    // key's value whatever the rounding). With EXACT_SUM (the caller asked for the LSE) the
    // fp32 weights are summed as well, into xsum: that sum carries no bf16 rounding into the
    // LSE. exp2(-inf) = 0.
    auto weights = [&](const f32x16 (&sc)[NKB], bf16x8 (&pp)[NKS], int t, float& xsum) {
      const float msc = ((kLateStart && m_run == -INFINITY) ? 0.f : m_run) * c;  // no key yet
      const float dq = ALIBI ? alibi_dq(t) : 0.f;
      const float bc = beta * c;  // the bias slope in exp2 units
      // exp2 argument of score (kb, i): c * (sgn s - beta |i - j|) - c * m
      const float base = kLinBias ? fmaf(-bc, dq, -msc) : -msc;
      auto arg = [&](int kb, int i) {
        float x = fmaf(sc[kb][i], cs, base);
        if constexpr (ALIBI && !kLinBias) x = fmaf(-bc, fabsf(dq - alibi_off(kb, i)), x);
        return x;
      };
      float lsum = 0.f;
#pragma unroll
      for (int ks = 0; ks < NKS; ++ks) {
        u32x4 w;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int kb = ks >> 1, i0 = 8 * (ks & 1) + 2 * i;
          const f32x2 e = {fast_exp2(arg(kb, i0)), fast_exp2(arg(kb, i0 + 1))};
          const bf16x2 h = __builtin_convertvector(e, bf16x2);
          w[i] = __builtin_bit_cast(uint32_t, h);
          // The dot operand is the converted pair itself: bit-casting it back out of w[i]
          // makes this compiler feed the same register to every dot instruction.
          lsum = __builtin_amdgcn_fdot2_f32_bf16(h, ones2, lsum, false);
          if constexpr (EXACT_SUM) {
            xsum += e[0];
            xsum += e[1];
          }
        }
        pp[ks] = as_bf16x8(w);
      }
      return lsum;
    };

    // The exponent offset m_run comes from the first tile in which the row sees a key
    // (new_offset: its row max, lifted for non-causal ALiBi), and stays fixed while every
    // weight of a tile is at most 2^32 (checked through the tile's weight sum, which bounds
    // each weight). A tile that breaks this (scores grown past the offset) is redone with
    // the offset raised to at least its row max, after rescaling what was accumulated.
    // Every term of a row always shares one offset, so the normalised result is that of
    // the exact max.
    auto tile = [&](int t, int u) {
      f32x16 sc[NKB];
      qk(sc, kslot(u));
      issue(u + kAhead);
      prep(sc, t);
      if constexpr (kLateStart) {
        if (wave_any(m_run == -INFINITY)) {  // rows that have not seen a key yet
          const float mx = new_offset(sc, t);
          if (m_run == -INFINITY) m_run = mx;  // stays -inf while all the row's keys are masked
        }
      } else if (t == 0) {
        m_run = new_offset(sc, t);  // key 0 is visible to every row, so this is finite
      }
      bf16x8 pp[NKS];
      // The softmax runs at raised wave priority, so a SIMD prefers this wave's vector work
      // while other waves' matrix products are in flight (measured ~2% faster for d = 128,
      // neutral for d = 64).
      __builtin_amdgcn_s_setprio(1);
      float xsum = 0.f;
      float lsum = weights(sc, pp, t, xsum);
      __builtin_amdgcn_s_setprio(0);
      if (wave_any(!(lsum <= kSumCap))) {
        // Recompute the scores from the K tile (still in LDS) rather than keeping them live
        // through the common path: the empty asm keeps the compiler from reusing them.
        asm volatile("" ::: "memory");
        qk(sc, kslot(u));
        prep(sc, t);
        const float m_new = fmaxf(m_run, new_offset(sc, t));
        const float alpha = m_new == m_run ? 1.f : fast_exp2((m_run - m_new) * c);
        l_run *= alpha;
        if constexpr (EXACT_SUM) lx_run *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int i = 0; i < 16; ++i) oacc[db][i] *= alpha;
        m_run = m_new;
        xsum = 0.f;
        lsum = weights(sc, pp, t, xsum);
      }
      l_run += lsum;
      if constexpr (EXACT_SUM) lx_run += xsum;
      pv(pp, vslot(u));
    };

    for (int n = t_first; n < ntiles; ++n, ++u) {
      const int t = kNearFirst ? t_first + ntiles - 1 - n : n;  // key tile of position n
      if (t >= wave_t0 && t < wave_nt)
        tile(t, u);
      else
        issue(u + kAhead);
      wait_vm<kJ * kAhead - kJ>();  // this wave's copies of position u + 1 have landed
      block_barrier();              // ... and every wave's; slot u may be overwritten next
    }

    // Epilogue: O = O^T / l, rounded to bf16; LSE = m*|scale| + ln l (l of the fp32 weights).
    const float l_tot = pair_sum(l_run);
    const float lx_tot = EXACT_SUM ? pair_sum(lx_run) : 0.f;
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
      if constexpr (EXACT_SUM) {
        if (hh == 0)
          p.lse[((size_t)b * Hq + hq) * S + qi] =
              l_tot > 0.f ? m_run * p.scale_abs + logf(lx_tot) - slope * (float)(qi - qa)
                          : -INFINITY;
      }
    }
  }
  wait_vm<0>();  // drain the copies issued past the last tile
}

// Dynamic LDS of the kernel: the K/V ring, then the length-order tables.
template <int D, bool ALIBI>
constexpr size_t prefill_lds_bytes() {
  return PfLayout<D, ALIBI>::LDS_BYTES + 2 * kPrefillLptMaxB * sizeof(int);
}

template <int D, bool CAUSAL, bool WINDOW, bool ALIBI>
hipError_t launch_one(const PrefillParams& p, hipStream_t stream) {
  using Shp = PfShape<D, ALIBI>;
  const size_t lds = prefill_lds_bytes<D, ALIBI>();
  // With an LSE output the weight sums are taken in fp32 (a separate instantiation, so the
  // plain kernel keeps its dot2 sums).
  auto kern = p.lse ? prefill_bf16_kernel<D, CAUSAL, WINDOW, ALIBI, true>
                    : prefill_bf16_kernel<D, CAUSAL, WINDOW, ALIBI, false>;
  static KernelSetup setups[2];  // per device and variant: LDS attribute, workgroups per CU
  KernelSetup& setup = setups[p.lse ? 1 : 0];
  int dev = 0, cus = 0, per_cu = 1;
  hipError_t e = current_device(&dev, &cus);
  if (e != hipSuccess) return e;
  if ((e = setup_kernel(setup, reinterpret_cast<const void*>(kern), Shp::THREADS, lds, dev,
                        &per_cu)) != hipSuccess)
    return e;
  // One resident workgroup per slot: P slots per XCD, each working through its share of
  // the XCD's queue (no more slots than queue positions).
  const int slots = Shp::PERSISTENT ? per_cu * (cus / 8 > 0 ? cus / 8 : 1) : p.per_xcd;
  const int P = p.per_xcd < slots ? p.per_xcd : slots;
  hipLaunchKernelGGL(kern, dim3(8 * (P > 0 ? P : 1)), dim3(Shp::THREADS), lds, stream, p);
  return hipGetLastError();
}

// The sliding window is built for causal attention only (the host rejects it otherwise).
template <int D>
hipError_t launch_d(const PrefillParams& p, int causal, hipStream_t stream) {
  const bool al = p.alibi != nullptr;
  if (!causal)
    return al ? launch_one<D, false, false, true>(p, stream)
              : launch_one<D, false, false, false>(p, stream);
  if (p.window > 0)
    return al ? launch_one<D, true, true, true>(p, stream)
              : launch_one<D, true, true, false>(p, stream);
  return al ? launch_one<D, true, false, true>(p, stream)
            : launch_one<D, true, false, false>(p, stream);
}

}  // namespace

static_assert(PfShape<128, true>::ROWS == PfShape<128, false>::ROWS,
              "the host plans one row count per head size");

int prefill_rows_per_wg_bf16(int d) {
  return d == 128 ? PfShape<128>::ROWS : (d == 64 ? PfShape<64>::ROWS : PfShape<32>::ROWS);
}

hipError_t launch_prefill_bf16(const PrefillParams& p, int causal, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_d<32>(p, causal, stream);
    case 64: return launch_d<64>(p, causal, stream);
    case 128: return launch_d<128>(p, causal, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
