// decode_bf16.hip - bf16 grouped-query attention decode over a ragged KV cache.
//
// One new query token per sequence reads every cached K/V row of its K/V head, so
// decode is bound by HBM bandwidth, and with grouping each K/V row read serves all
// g query heads of the group (azimuth.plus GQA digest, "the bottleneck" section and
// the KV-cache size formula 2 x L x G x d_k x n).
//
// Work split (split-KV with a log-sum-exp merge; the pages' `num_splits` knob,
// blog.gitcode.com "3个GQA核心优化技巧", section "阶段二：高级优化参数"):
//   * unit u = (b, kvh, query block of <= 32 heads); unit u has T_u = ceil(L_b / 32)
//     key tiles of 32 rows; all units' tiles are concatenated (T tiles in total);
//   * workgroup w of W = min(launched, T) takes tiles [floor(w T / W), floor((w+1) T / W)),
//     so every workgroup streams the same number of rows whatever the length mix,
//     and a sequence is split into as many pieces as shares overlap it;
//   * a workgroup covering a whole unit writes the final output; otherwise it writes
//     a normalised fp32 partial and its LSE to slot (w + u) (w and u never both
//     decrease along the tile order, so w + u is unique), and the combine kernel
//     merges a unit's partials in workgroup order with weights exp(lse_s - max).
// Inside a workgroup the 8 waves take each segment's tiles (the part of one unit inside
// the share) round-robin and merge their running (max, sum, O) through LDS. A wave
// requests its first tile of the next segment, and the workgroup that segment's Q,
// before the current segment's merge, so a share spanning several units streams on.
//
// Per 32-key tile, per wave (lane l: query l % 32 of the block, key half l / 32):
//   S^T = K Q^T   (d/16) MFMA 32x32x16; K rows come straight from HBM as the A
//                 operand (16 bytes per lane), Q^T is read back from LDS;
//   online softmax over the 32 keys (running max / running sum);
//   O^T += V^T P^T  2 x (d/32) MFMA; each lane loads d/32 consecutive values of 8
//                 keys (one full row per 32 lanes, coalesced, non-temporal), and byte
//                 permutes build the V^T operand for output columns d = (d/32) * m + c.
// Rows at or past L_b are never read.
#include "gqa_device.h"
#include "gqa_kernels.h"

namespace gqa {
namespace {

constexpr int DC_WAVES = 8;  // one workgroup fills a CU (2 waves per SIMD)
constexpr int DC_THREADS = 64 * DC_WAVES;
constexpr int DC_TILE = 32;

__device__ __forceinline__ int clamp_len(const int32_t* lens, int b, int cap) {
  if (!lens) return cap;
  int L = lens[b];
  return L < 0 ? 0 : (L > cap ? cap : L);
}

// A sequence's key tiles: with a sliding window only the last `window` keys are visited,
// from tile first_tile(L) on.
__device__ __forceinline__ int first_tile(int L, int window) {
  return window > 0 ? max(0, L - window) / DC_TILE : 0;
}
__device__ __forceinline__ int tiles_of(int L, int window) {
  return L > 0 ? (L + DC_TILE - 1) / DC_TILE - first_tile(L, window) : 0;
}

// Sum over a workgroup of NT threads (all threads get the result).
template <int NT>
__device__ long long block_sum(long long v, long long* scratch) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off, 64);
  const int wave = threadIdx.x >> 6;
  __syncthreads();
  if ((threadIdx.x & 63) == 0) scratch[wave] = v;
  __syncthreads();
  long long t = 0;
#pragma unroll
  for (int w = 0; w < NT / 64; ++w) t += scratch[w];
  return t;
}

// Tiles of sequences [0, B) (per K/V unit of one sequence) and of [0, b_end).
template <int NT>
__device__ void tile_prefix(const int32_t* lens, int B, int cap, int window, int b_end,
                            long long* total, long long* before, long long* scratch) {
  long long tot = 0, bef = 0;
  for (int base = 0; base < B; base += NT) {
    const int bb = base + threadIdx.x;
    const long long tb = bb < B ? tiles_of(clamp_len(lens, bb, cap), window) : 0;
    tot += block_sum<NT>(tb, scratch);
    bef += block_sum<NT>(bb < b_end ? tb : 0, scratch);
  }
  *total = tot;
  *before = bef;
}

// First sequence whose tile range (in concatenated unit order) ends after tile t0,
// and the first tile of that sequence.
__device__ void find_seq(const int32_t* lens, int B, int cap, int window, long long HU,
                         long long t0, int* b_out, long long* start_out, long long* scratch) {
  long long run = 0;  // tiles of sequences before this chunk
  if (threadIdx.x == 0) {
    scratch[DC_WAVES] = 0;
    scratch[DC_WAVES + 1] = 0;
  }
  for (int base = 0; base < B; base += DC_THREADS) {
    const int bb = base + threadIdx.x;
    const long long tb = bb < B ? HU * tiles_of(clamp_len(lens, bb, cap), window) : 0;
    // inclusive scan of tb across the workgroup
    long long x = tb;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    __syncthreads();
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    long long wave_off = 0;
    for (int w = 0; w < wave; ++w) wave_off += scratch[w];
    long long chunk_total = 0;
#pragma unroll
    for (int w = 0; w < DC_WAVES; ++w) chunk_total += scratch[w];
    const long long incl = run + wave_off + x;  // tiles through sequence bb
    const long long excl = incl - tb;
    // the sequence containing tile t0: excl <= t0 < incl
    const bool hit = bb < B && excl <= t0 && t0 < incl;
    __syncthreads();
    if (hit) {
      scratch[DC_WAVES] = bb;
      scratch[DC_WAVES + 1] = excl;
    }
    __syncthreads();
    if (run + chunk_total > t0) break;  // uniform: the hit was in this chunk
    run += chunk_total;
  }
  *b_out = (int)scratch[DC_WAVES];
  *start_out = scratch[DC_WAVES + 1];
}

// The workgroup's share [t_begin, t_end) of the concatenated unit tiles (T of them, W =
// min(T, n_wg) equal shares) and the sequence b it starts in, with bstart that sequence's
// first tile. With at most one length per thread this is one pass over the lengths (a
// workgroup-wide scan: the total, then the sequence holding t_begin); longer length
// arrays take the two-pass path. False when the workgroup has no share (uniform).
__device__ bool find_share(const DecodeParams& p, int cap, long long HU, int w,
                           long long* t_begin, long long* t_end, int* b_out,
                           long long* bstart_out, long long* scratch) {
  long long T;
  if (p.B <= DC_THREADS) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const long long tb = tid < p.B ? HU * tiles_of(clamp_len(p.lens, tid, cap), p.window) : 0;
    long long x = tb;  // inclusive scan within the wave
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const long long y = __shfl_up(x, off, 64);
      if (lane >= off) x += y;
    }
    if (lane == 63) scratch[wave] = x;
    __syncthreads();
    long long wave_off = 0;
    T = 0;
#pragma unroll
    for (int i = 0; i < DC_WAVES; ++i) {
      const long long v = scratch[i];
      wave_off += i < wave ? v : 0;
      T += v;
    }
    const long long W = T < p.n_wg ? T : p.n_wg;
    if (w >= W) return false;
    *t_begin = (long long)w * T / W;
    *t_end = (long long)(w + 1) * T / W;
    const long long incl = wave_off + x, excl = incl - tb;
    if (tid < p.B && excl <= *t_begin && *t_begin < incl) {
      scratch[DC_WAVES] = tid;
      scratch[DC_WAVES + 1] = excl;
    }
    __syncthreads();
    *b_out = (int)scratch[DC_WAVES];
    *bstart_out = scratch[DC_WAVES + 1];
    return true;
  }
  long long unused;
  tile_prefix<DC_THREADS>(p.lens, p.B, cap, p.window, 0, &T, &unused, scratch);
  T *= HU;
  const long long W = T < p.n_wg ? T : p.n_wg;
  if (w >= W) return false;
  *t_begin = (long long)w * T / W;
  *t_end = (long long)(w + 1) * T / W;
  find_seq(p.lens, p.B, cap, p.window, HU, *t_begin, b_out, bstart_out, scratch);
  return true;
}

template <int D>
struct DcLayout {
  static constexpr int OSTR = D + 4;  // floats per query row of a wave's O in LDS
  static constexpr int O_FLOATS = DC_WAVES * 32 * OSTR;
  static constexpr int QSTR = D + 8;  // bf16 per query row of Q in LDS (conflict-free reads)
  static constexpr int Q_BYTES = 32 * QSTR * 2;
  // Q, the merge area (O, m, l per wave), the share-search scratch, then the clamped
  // lengths of up to DC_THREADS sequences (kept when the share search read them all).
  static constexpr size_t SCRATCH_OFF = Q_BYTES + (O_FLOATS + 2 * DC_WAVES * 32) * 4;
  static constexpr size_t LEN_OFF = SCRATCH_OFF + (DC_WAVES + 4) * sizeof(long long);
  static constexpr size_t LDS = LEN_OFF + DC_THREADS * sizeof(int);
  static_assert(LDS <= 160 * 1024, "one workgroup's LDS must fit a CU");
  static_assert(32 * (D / 8) <= DC_THREADS, "one Q chunk per thread at most");
};

template <int D, bool ALIBI, bool PAGED>
__global__ __launch_bounds__(DC_THREADS, 2) void decode_split_kernel(DecodeParams p) {
  constexpr int DPL = D / 32;  // output columns per lane in the V^T operand
  using Lay = DcLayout<D>;
  extern __shared__ __attribute__((aligned(16))) float dsm[];
  uint8_t* const dsm8 = reinterpret_cast<uint8_t*>(dsm);
  uint16_t* s_q = reinterpret_cast<uint16_t*>(dsm);                       // [32][QSTR] bf16
  float* s_o = dsm + Lay::Q_BYTES / 4;     // [wave][32][OSTR]
  float* s_m = s_o + Lay::O_FLOATS;        // [wave][32]
  float* s_l = s_m + DC_WAVES * 32;        // [wave][32]
  long long* scratch = reinterpret_cast<long long*>(dsm8 + Lay::SCRATCH_OFF);  // 8 + 4 entries
  int* s_len = reinterpret_cast<int*>(dsm8 + Lay::LEN_OFF);                    // [B] clamped

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63;
  const int l32 = lane & 31;
  const int hh = lane >> 5;
  const int w = blockIdx.x;
  const int cap = p.max_len;
  const long long HU = (long long)p.Hkv * p.nqb;
  const float c = p.scale_log2;

  // With one length per thread the lengths stay in LDS for the segment lookups below.
  const bool lens_in_lds = p.B <= DC_THREADS;
  if (lens_in_lds && tid < p.B) s_len[tid] = clamp_len(p.lens, tid, cap);

  // Never more shares than tiles, so every share is non-empty and the shares
  // overlapping a unit form one run of consecutive workgroups.
  long long t_begin, t_end, bstart;
  int b;
  if (!find_share(p, cap, HU, w, &t_begin, &t_end, &b, &bstart, scratch)) return;
  if (t_begin >= t_end) return;  // (find_share's barriers also publish s_len)

  // A segment: the tiles [ta, te) of one unit u = (b, kvh, query block) that fall inside
  // the share; next_t is the share position after it. All fields are wave-uniform.
  struct Seg {
    int b, Lb, Tb, ft, klo, ta, te, kvh, hbase, nh, u;
    long long next_t;
  };
  // The segment holding share position t; b_/bstart_ (the sequence reached so far and its
  // first position) move forward past sequences that end before t. False at the end of
  // the share or of the batch.
  auto find_seg = [&](long long t, int& b_, long long& bstart_, Seg& sg) -> bool {
    while (t < t_end && b_ < p.B) {
      const int Lb = lens_in_lds ? s_len[b_] : clamp_len(p.lens, b_, cap);
      const int Tb = tiles_of(Lb, p.window);
      const long long bend = bstart_ + HU * Tb;
      if (Tb == 0 || t >= bend) {
        bstart_ = bend;
        ++b_;
        continue;
      }
      const int ui = (int)((t - bstart_) / Tb);
      const long long ustart = bstart_ + (long long)ui * Tb;
      const int kvh = ui / p.nqb, qb = ui - kvh * p.nqb;
      sg.b = b_;
      sg.Lb = Lb;
      sg.Tb = Tb;
      sg.ft = first_tile(Lb, p.window);                   // unit tile tt is key tile ft + tt
      sg.klo = p.window > 0 ? max(0, Lb - p.window) : 0;  // keys j < klo are outside
      sg.ta = (int)(t - ustart);
      sg.te = (int)(min(t_end, ustart + Tb) - ustart);
      sg.kvh = kvh;
      sg.hbase = kvh * p.g + qb * 32;
      sg.nh = min(32, p.g - qb * 32);
      sg.u = (b_ * p.Hkv + kvh) * p.nqb + qb;
      sg.next_t = ustart + sg.te;
      return true;
    }
    return false;
  };

  // One tile's K rows (A operand: lane reads 16 bytes of row j0 + l32) and V rows (for
  // 16-key step ks2 and slot i, key j0 + 16ks2 + 8(i/4) + 4hh + (i%4); the lane reads DPL
  // consecutive values starting at d = DPL * l32). Loads go through a buffer resource that
  // starts at the tile and ends at row L_b, so rows at or past L_b read as zeros, the lane
  // offsets are the same for every tile and no load needs a predicate.
  struct TileRegs {
    u32x4 kf[D / 16];
    uint32_t vl[2][8][DPL / 2];
  };
  const uint32_t row_b = D * 2;
  const uint32_t k_lane = l32 * row_b + hh * 16;
  const uint32_t v_lane = (4 * hh) * row_b + DPL * 2 * l32;
  // Element offset (from the start of the cache or page pool) of segment tile tt's first
  // key row and the bytes of its valid rows. A paged cache looks the tile's page up in the
  // block table (a tile never straddles pages); a page id outside the pool leaves no valid
  // bytes, so its rows read as zeros.
  auto tile_src = [&](const Seg& sg, int tt, uint32_t* valid) -> size_t {
    const int j0 = (sg.ft + tt) * DC_TILE;
    const int nv = max(min(sg.Lb - j0, DC_TILE), 0);
    if constexpr (PAGED) {
      const int page = p.block_table[(size_t)sg.b * p.max_blocks + j0 / p.page_size];
      const bool ok = page >= 0 && page < p.num_pages;
      *valid = ok ? (uint32_t)nv * row_b : 0u;
      return ok ? (((size_t)page * p.Hkv + sg.kvh) * p.page_size + j0 % p.page_size) * D : 0;
    } else {
      *valid = (uint32_t)nv * row_b;
      return (((size_t)sg.b * p.Hkv + sg.kvh) * cap + j0) * D;
    }
  };
  // Every input of the descriptor is wave-uniform; reading each through readfirstlane
  // tells the compiler so, which keeps every buffer load a single instruction (a
  // descriptor it cannot prove uniform gets a loop over the distinct values per load).
  auto rsrc = [&](const void* base, const Seg& sg, int tt) {
    uint32_t valid;
    const size_t off = tile_src(sg, tt, &valid);
    // (readfirstlane returns a signed int: go through uint32_t so that an address whose
    // low word has bit 31 set is not sign-extended into the high word.)
    const uint64_t a = reinterpret_cast<uint64_t>(static_cast<const uint16_t*>(base) + off);
    const uint64_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint64_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void*>(lo | (hi << 32)), 0,
                                             __builtin_amdgcn_readfirstlane(valid), 0x00020000);
  };
  auto load_k_from = [&](TileRegs& r, __amdgpu_buffer_rsrc_t rk) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks)
      r.kf[ks] = __builtin_bit_cast(
          u32x4, __builtin_amdgcn_raw_buffer_load_b128(rk, k_lane + ks * 32, 0, 0));
  };
  // V loads are non-temporal (cache-policy bit 1, `nt`): each instruction reads whole rows
  // (32 lanes cover one 256-byte row at d = 128), so every cache line it touches is consumed
  // at once and keeping it is of no use. Measured 11 % faster on the uniform 8k decode and
  // 6 % on the ragged multi-query one. K keeps the default policy: an A-operand load takes
  // 32 bytes from each of 32 rows and the rest of each line is read by the next products,
  // which with `nt` fetched the lines again (15 % slower).
  constexpr int kVPolicy = 2;
  auto load_v_from = [&](TileRegs& r, __amdgpu_buffer_rsrc_t rv) {
#pragma unroll
    for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const uint32_t off = v_lane + (16 * ks2 + 8 * (i >> 2) + (i & 3)) * row_b;
        if constexpr (DPL == 4) {
          const u32x2 x = __builtin_bit_cast(
              u32x2, __builtin_amdgcn_raw_buffer_load_b64(rv, off, 0, kVPolicy));
          r.vl[ks2][i][0] = x[0];
          r.vl[ks2][i][1] = x[1];
        } else {
          r.vl[ks2][i][0] = __builtin_amdgcn_raw_buffer_load_b32(rv, off, 0, kVPolicy);
        }
      }
  };
  auto load_k = [&](TileRegs& r, const Seg& sg, int tt) { load_k_from(r, rsrc(p.kc, sg, tt)); };
  auto load_v = [&](TileRegs& r, const Seg& sg, int tt) { load_v_from(r, rsrc(p.vc, sg, tt)); };
  // Q of a segment's heads (rows past nh are zeros): thread tid holds 16-byte chunk tid;
  // it is written to LDS (the B operand of S^T = K Q^T, read back per tile: lane holds
  // head l32, d = ks*16 + hh*8 .. +7) once the previous segment is done with it.
  const uint32_t flip = p.negate_q ? 0x80008000u : 0u;
  const int q_row = tid / (D / 8), q_col = tid - q_row * (D / 8);
  auto load_q = [&](const Seg& sg) -> u32x4 {
    u32x4 v = zero_u32x4();
    if (q_row < 32 && q_row < sg.nh) {
      v = ldg16(static_cast<const uint16_t*>(p.q) + ((size_t)sg.b * p.Hq + sg.hbase + q_row) * D +
                q_col * 8);
      v[0] ^= flip; v[1] ^= flip; v[2] ^= flip; v[3] ^= flip;
    }
    return v;
  };
  auto store_q = [&](const u32x4& v) {
    if (q_row < 32) *reinterpret_cast<u32x4*>(s_q + q_row * Lay::QSTR + q_col * 8) = v;
  };

  Seg cur;
  if (!find_seg(t_begin, b, bstart, cur)) return;  // uniform
  TileRegs r0;
  // The wave's first K/V tile is requested before the Q staging so both round trips
  // overlap. Later segments' first tiles are requested while the previous segment ends.
  if (cur.ta + wave < cur.te) {
    load_k(r0, cur, cur.ta + wave);
    load_v(r0, cur, cur.ta + wave);
  }
  store_q(load_q(cur));
  __syncthreads();

  for (;;) {
    // The next segment, if any: only the descriptors of this wave's first tile there stay
    // live through the tile loop (the segment itself is looked up again at the switch).
    bool pre_next = false;
    __amdgpu_buffer_rsrc_t rk_next = __builtin_amdgcn_make_buffer_rsrc(nullptr, 0, 0, 0);
    __amdgpu_buffer_rsrc_t rv_next = rk_next;
    {
      Seg nxt;
      int bn = b;
      long long bsn = bstart;
      if (find_seg(cur.next_t, bn, bsn, nxt) && nxt.ta + wave < nxt.te) {
        pre_next = true;
        rk_next = rsrc(p.kc, nxt, nxt.ta + wave);
        rv_next = rsrc(p.vc, nxt, nxt.ta + wave);
      }
    }

    f32x16 oacc[DPL];
#pragma unroll
    for (int i = 0; i < DPL; ++i) oacc[i] = zero16();
    float m_run = -INFINITY, l_run = 0.f;
    float beta = 0.f;  // ALiBi slope of this lane's head in raw-score units
    if constexpr (ALIBI) beta = l32 < cur.nh ? p.alibi[cur.hbase + l32] * kLog2e / c : 0.f;

    // Each tile's K (V) registers are refilled as soon as QK^T (PV) has consumed them:
    // with this wave's next tile of the segment, or after its last one with its first tile
    // of the next segment.
    auto compute_tile = [&](TileRegs& r, int tt, bool more) {
      const int j0 = (cur.ft + tt) * DC_TILE;
      f32x16 s = zero16();
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        const u32x4 qv = *reinterpret_cast<const u32x4*>(s_q + l32 * Lay::QSTR + ks * 16 + hh * 8);
        s = mfma_bf16_32x32x16(as_bf16x8(r.kf[ks]), as_bf16x8(qv), s);
      }
      if (more)
        load_k(r, cur, tt + DC_WAVES);
      else if (pre_next)
        load_k_from(r, rk_next);
      if constexpr (ALIBI) {  // the query sits at L_b - 1: bias -slope * (L_b - 1 - j)
        const float dq = (float)(cur.Lb - 1 - j0 - 4 * hh);
#pragma unroll
        for (int rr = 0; rr < 16; ++rr)
          s[rr] = fmaf(-beta, dq - (float)(8 * (rr >> 2) + (rr & 3)), s[rr]);
      }
      const bool need_mask = j0 + DC_TILE > cur.Lb || j0 < cur.klo;
      if (need_mask) {
#pragma unroll
        for (int rr = 0; rr < 16; ++rr) {
          const int j = j0 + 8 * (rr >> 2) + 4 * hh + (rr & 3);
          if (j >= cur.Lb || j < cur.klo) s[rr] = -INFINITY;
        }
      }
      float mx = -INFINITY;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) mx = fmaxf(mx, s[rr]);
      mx = pair_max(mx);
      const float m_new = fmaxf(m_run, mx);
      if (wave_any(m_new > m_run)) {
        const float alpha = (m_run == -INFINITY) ? 0.f : fast_exp2((m_run - m_new) * c);
        l_run *= alpha;
#pragma unroll
        for (int i = 0; i < DPL; ++i)
#pragma unroll
          for (int rr = 0; rr < 16; ++rr) oacc[i][rr] *= alpha;
        m_run = m_new;
      }
      const float msc = (m_run == -INFINITY ? 0.f : m_run) * c;
#pragma unroll
      for (int rr = 0; rr < 16; ++rr) {
        float pv = fast_exp2(fmaf(s[rr], c, -msc));
        if (need_mask) pv = (s[rr] == -INFINITY) ? 0.f : pv;
        s[rr] = pv;
        l_run += pv;
      }
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2) {
        const int e0 = 8 * ks2;
        const bf16x8 pb = pack_bf16x8(s[e0 + 0], s[e0 + 1], s[e0 + 2], s[e0 + 3], s[e0 + 4],
                                      s[e0 + 5], s[e0 + 6], s[e0 + 7]);
#pragma unroll
        for (int cc = 0; cc < DPL; ++cc) {
          const int word = cc >> 1;       // which dword of the lane's DPL values
          const bool upper = cc & 1;      // low or high bf16 of that dword
          u32x4 a;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            const uint32_t x0 = r.vl[ks2][2 * jj][word], x1 = r.vl[ks2][2 * jj + 1][word];
            a[jj] = upper ? ((x0 >> 16) | (x1 & 0xffff0000u)) : ((x0 & 0xffffu) | (x1 << 16));
          }
          oacc[cc] = mfma_bf16_32x32x16(as_bf16x8(a), pb, oacc[cc]);
        }
      }
      if (more)
        load_v(r, cur, tt + DC_WAVES);  // V registers are free again
      else if (pre_next)
        load_v_from(r, rv_next);
    };

    // The wave's tiles of the segment are ta + wave, ta + wave + DC_WAVES, ...
    for (int tt = cur.ta + wave; tt < cur.te; tt += DC_WAVES)
      compute_tile(r0, tt, tt + DC_WAVES < cur.te);
    if (cur.ta + wave >= cur.te && pre_next) {  // no tile here: request the next one now
      load_k_from(r0, rk_next);
      load_v_from(r0, rv_next);
    }
    // The next segment (b and bstart move on to it); its Q is requested before the merge
    // and stored after it.
    Seg nxt;
    const bool has_next = find_seg(cur.next_t, b, bstart, nxt);
    const u32x4 q_next = has_next ? load_q(nxt) : zero_u32x4();

    // Merge the waves' running states through LDS.
    const float l_tot = pair_sum(l_run);
    if (hh == 0) {
      s_m[wave * 32 + l32] = m_run;
      s_l[wave * 32 + l32] = l_tot;
    }
    // Accumulator slot r of the DPL column blocks holds columns DPL * (8(r/4) + 4hh + r%4)
    // + 0 .. DPL-1: one vector store each.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      float* dst = s_o + (wave * 32 + l32) * Lay::OSTR + DPL * (8 * (r >> 2) + 4 * hh + (r & 3));
      if constexpr (DPL == 4) {
        *reinterpret_cast<u32x4*>(dst) =
            u32x4{__float_as_uint(oacc[0][r]), __float_as_uint(oacc[1][r]),
                  __float_as_uint(oacc[2][r]), __float_as_uint(oacc[3][r])};
      } else {
        *reinterpret_cast<u32x2*>(dst) =
            u32x2{__float_as_uint(oacc[0][r]), __float_as_uint(oacc[1][r])};
      }
    }
    __syncthreads();
    {
      constexpr int SEGS = DC_THREADS / 32;  // threads per query row
      constexpr int CPT = D / SEGS;          // output columns per thread
      const int n = tid / SEGS;              // query of the block
      const int dseg = (tid % SEGS) * CPT;
      float M = -INFINITY;
#pragma unroll
      for (int wv = 0; wv < DC_WAVES; ++wv) M = fmaxf(M, s_m[wv * 32 + n]);
      float wgt[DC_WAVES];
      float lsum = 0.f;
#pragma unroll
      for (int wv = 0; wv < DC_WAVES; ++wv) {
        const float mw = s_m[wv * 32 + n];
        wgt[wv] = (mw == -INFINITY) ? 0.f : fast_exp2((mw - M) * c);
        lsum += wgt[wv] * s_l[wv * 32 + n];
      }
      const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
      const float lse_v = lsum > 0.f ? M * p.scale_abs + logf(lsum) : -INFINITY;
      if (n < cur.nh) {
        float val[CPT];
#pragma unroll
        for (int dd = 0; dd < CPT; ++dd) val[dd] = 0.f;
#pragma unroll
        for (int wv = 0; wv < DC_WAVES; ++wv)
#pragma unroll
          for (int q4 = 0; q4 < CPT / 4; ++q4) {
            const u32x4 x =
                *reinterpret_cast<const u32x4*>(s_o + (wv * 32 + n) * Lay::OSTR + dseg + 4 * q4);
#pragma unroll
            for (int e = 0; e < 4; ++e) val[4 * q4 + e] += wgt[wv] * __uint_as_float(x[e]);
          }
#pragma unroll
        for (int dd = 0; dd < CPT; ++dd) val[dd] *= inv;
        if (cur.ta == 0 && cur.te == cur.Tb) {
          uint16_t* orow =
              static_cast<uint16_t*>(p.o) + ((size_t)cur.b * p.Hq + cur.hbase + n) * D + dseg;
#pragma unroll
          for (int q4 = 0; q4 < CPT / 4; ++q4) {
            u32x2 w2;
            w2[0] = pack_bf16x2(val[4 * q4], val[4 * q4 + 1]);
            w2[1] = pack_bf16x2(val[4 * q4 + 2], val[4 * q4 + 3]);
            *reinterpret_cast<u32x2*>(orow + 4 * q4) = w2;
          }
          if (p.lse && (tid % SEGS) == 0) p.lse[(size_t)cur.b * p.Hq + cur.hbase + n] = lse_v;
        } else {
          const size_t slot = (size_t)w + cur.u;
          float* dst = p.ws_o + (slot * 32 + n) * D + dseg;
#pragma unroll
          for (int q4 = 0; q4 < CPT / 4; ++q4) {
            u32x4 wv4;
#pragma unroll
            for (int e = 0; e < 4; ++e) wv4[e] = __float_as_uint(val[4 * q4 + e]);
            *reinterpret_cast<u32x4*>(dst + 4 * q4) = wv4;
          }
          if ((tid % SEGS) == 0) p.ws_lse[slot * 32 + n] = lse_v;
        }
      }
    }
    __syncthreads();  // the merge area and Q are free for the next segment
    if (!has_next) break;
    store_q(q_next);
    __syncthreads();
    cur = nxt;
  }
}

// Merge the split partials of one unit (b, kvh, query block): workgroup (u, head block),
// one thread per (head, 4 output columns). Partials are visited in workgroup order with
// a running max, so the merge order is fixed and the result deterministic.
constexpr int CB_THREADS = 64;  // one wave per combine workgroup
constexpr int CB_BATCH = 16;    // partials whose loads are issued together

template <int D>
__global__ __launch_bounds__(CB_THREADS) void decode_combine_kernel(DecodeParams p) {
  constexpr int TPH = D / 4;              // threads per head
  constexpr int HPB = CB_THREADS / TPH;   // heads per workgroup
  __shared__ long long scratch[CB_THREADS / 64];
  const int u = blockIdx.x;
  const int qb = u % p.nqb;
  const int kvh = (u / p.nqb) % p.Hkv;
  const int b = u / (p.nqb * p.Hkv);
  const int cap = p.max_len;
  const long long HU = (long long)p.Hkv * p.nqb;
  long long T, before;
  tile_prefix<CB_THREADS>(p.lens, p.B, cap, p.window, b, &T, &before, scratch);
  T *= HU;
  const int Tb = tiles_of(clamp_len(p.lens, b, cap), p.window);
  const int hbase = kvh * p.g + qb * 32;
  const int nh = min(32, p.g - qb * 32);
  const int n = blockIdx.y * HPB + threadIdx.x / TPH;
  const int d0 = (threadIdx.x % TPH) * 4;
  if (n >= nh) return;
  uint16_t* orow = static_cast<uint16_t*>(p.o) + ((size_t)b * p.Hq + hbase + n) * D + d0;
  float* lse_out = p.lse ? p.lse + (size_t)b * p.Hq + hbase + n : nullptr;

  if (Tb == 0) {  // empty cache: O = 0, LSE = -inf
    *reinterpret_cast<u32x2*>(orow) = u32x2{0u, 0u};
    if (lse_out && d0 == 0) *lse_out = -INFINITY;
    return;
  }
  const long long W = T < p.n_wg ? T : p.n_wg;  // the split kernel's effective share count
  const long long ustart = before * HU + (long long)(kvh * p.nqb + qb) * Tb;
  const long long ulast = ustart + Tb - 1;
  const int wa = (int)(((ustart + 1) * W - 1) / T);
  const int wb = (int)(((ulast + 1) * W - 1) / T);
  if (wa == wb) return;  // one workgroup covered the unit and wrote the output

  float m = -INFINITY, den = 0.f, acc[4] = {0.f, 0.f, 0.f, 0.f};
  for (int s0 = wa; s0 <= wb; s0 += CB_BATCH) {
    float lw[CB_BATCH];
    u32x4 ov[CB_BATCH];
#pragma unroll
    for (int k = 0; k < CB_BATCH; ++k) {
      const int s = s0 + k;
      if (s <= wb) {
        const size_t slot = (size_t)s + u;
        lw[k] = p.ws_lse[slot * 32 + n];
        ov[k] = ldg16(p.ws_o + (slot * 32 + n) * D + d0);
      } else {
        lw[k] = -INFINITY;
        ov[k] = zero_u32x4();
      }
    }
#pragma unroll
    for (int k = 0; k < CB_BATCH; ++k) {
      if (lw[k] == -INFINITY) continue;
      const float m_new = fmaxf(m, lw[k]);
      const float sc = (m == -INFINITY) ? 0.f : fast_exp2((m - m_new) * kLog2e);
      const float e = fast_exp2((lw[k] - m_new) * kLog2e);
      den = den * sc + e;
#pragma unroll
      for (int c = 0; c < 4; ++c) acc[c] = acc[c] * sc + e * __uint_as_float(ov[k][c]);
      m = m_new;
    }
  }
  const float inv = den > 0.f ? 1.f / den : 0.f;
  u32x2 o2;
  o2[0] = pack_bf16x2(acc[0] * inv, acc[1] * inv);
  o2[1] = pack_bf16x2(acc[2] * inv, acc[3] * inv);
  *reinterpret_cast<u32x2*>(orow) = o2;
  if (lse_out && d0 == 0) *lse_out = den > 0.f ? m + logf(den) : -INFINITY;
}

template <int D, bool ALIBI, bool PAGED>
hipError_t launch_d(const DecodeParams& p, bool need_combine, hipStream_t stream) {
  using Lay = DcLayout<D>;
  const size_t lds = Lay::LDS;
  auto kern = decode_split_kernel<D, ALIBI, PAGED>;
  static KernelSetup setup;  // per device: LDS attribute set
  int dev = 0, cus = 0, per_cu = 1;
  hipError_t e = current_device(&dev, &cus);
  if (e != hipSuccess) return e;
  if ((e = setup_kernel(setup, reinterpret_cast<const void*>(kern), DC_THREADS, lds, dev,
                        &per_cu)) != hipSuccess)
    return e;
  hipLaunchKernelGGL(kern, dim3(p.n_wg), dim3(DC_THREADS), lds, stream, p);
  e = hipGetLastError();
  if (e != hipSuccess || !need_combine) return e;
  constexpr int HPB = CB_THREADS / (D / 4);
  const int heads = p.g < 32 ? p.g : 32;
  hipLaunchKernelGGL((decode_combine_kernel<D>), dim3(p.n_units, (heads + HPB - 1) / HPB),
                     dim3(CB_THREADS), 0, stream, p);
  return hipGetLastError();
}

template <int D>
hipError_t launch_opts(const DecodeParams& p, bool need_combine, hipStream_t stream) {
  const bool paged = p.block_table != nullptr;
  if (p.alibi)
    return paged ? launch_d<D, true, true>(p, need_combine, stream)
                 : launch_d<D, true, false>(p, need_combine, stream);
  return paged ? launch_d<D, false, true>(p, need_combine, stream)
               : launch_d<D, false, false>(p, need_combine, stream);
}

}  // namespace

hipError_t launch_decode_bf16(const DecodeParams& p, bool need_combine, hipStream_t stream) {
  switch (p.d) {
    case 64: return launch_opts<64>(p, need_combine, stream);
    case 128: return launch_opts<128>(p, need_combine, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gqa
