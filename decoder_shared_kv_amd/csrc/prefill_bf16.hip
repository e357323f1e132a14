// Prefill: causal cross-attention of every prompt row, bf16 storage, MFMA,
// with K^/V^ tiles copied HBM -> LDS by the load unit (no registers, no VALU)
// through a multi-stage LDS pipeline.
//
// Attn_l = softmax(Q^l K^T * scale + M_causal) V^ over the whole prompt (page
// "YOCO", section "Cross-Decoder", Attn_l equation; causal rule j <= i from
// section "架构总览"). Both products run on v_mfma_f32_32x32x16_bf16.
//
// Workgroup = W waves x 32 query rows of one KV group (up to W query heads at
// the same positions, or fewer heads over more positions), so every K^/V^ tile
// in LDS serves all heads of the group. Per 64-key tile and per wave:
//   S^T[key][query] = K^ . Q^T      A = K^ rows from LDS (16-byte reads),
//                                   B = Q^T in registers
//   online softmax on S^T           one query per lane pair (lane, lane ^ 32)
//   O^T[dim][query] += V^T . P^T    B = P^T straight from the S^T registers,
//                                   A = V^T read from the row-major V^ tile by
//                                   ds_read_b64_tr_b16 (transposing LDS reads)
// The accumulator layout of a 32x32 MFMA gives lane l the keys
// 8*(r/4) + 4*(l/32) + (r%4) of query l%32; registers 8c..8c+7 are the B
// operand of PV step c, whose k-slot e of lane half h is key
// 16c + 8*(e/4) + 4h + (e%4): two 4-key groups, each one transposing read.
//
// LDS tiles are stored unpadded (the load unit writes 16 bytes per lane,
// contiguous), with XOR swizzles of the 16-byte chunks chosen on the source
// side: K^ row r keeps chunk c at c ^ (r mod chunks-per-row), V^ row r at
// c ^ v_swizzle(r mod 4); both make the reads bank-conflict-free. The K^ tiles
// of all stages fill the first half of the LDS and the V^ tiles the second, and
// the tile loop is unrolled by the stage count, so every operand read is a
// lane-constant register plus an immediate offset (no address arithmetic per
// tile).
//
// Softmax: online, with the running reference moved lazily (only when a row's
// max passed it by a slack) and the max itself taken only when the weights
// computed against the current reference could be too large (see sv_step).
//
// Pipeline: tile t + S - 1 is requested while tile t is computed, so a tile has
// S - 1 tile-compute times to arrive. One workgroup barrier per tile. Within a
// tile each wave keeps its LDS operand reads a few MFMAs ahead (scheduling
// fences stop the compiler from sinking them to their use), and spreads half
// of the exponentials between the PV MFMAs, which execute while they issue.
#include <hip/hip_bf16.h>

#include <type_traits>
#include <utility>

#include "internal.h"
#include "lds_copy.h"
#include "tile_common.h"

namespace yoco {

namespace {

#ifndef YOCO_PREFILL_STAGES
#define YOCO_PREFILL_STAGES 4
#endif
constexpr int kStages = YOCO_PREFILL_STAGES;
#ifndef YOCO_PREFILL_SCHED
#define YOCO_PREFILL_SCHED 1
#endif



constexpr int kBN = 64;                 // keys per tile
constexpr float kRescaleSlack = 8.0f;   // base-2 growth of the running max tolerated before a rescale
constexpr float kWeightCap = 65536.0f;  // largest sum of one lane's half-tile weights taken without a max

// Wait until at most `ahead` (< kStages - 1) tiles of L loads each are still in flight.
template <int L>
__device__ __forceinline__ void wait_tiles(int ahead) {
  if (kStages >= 5 && ahead >= 3) wait_vm_lgkm0<(kStages >= 5 ? 3 * L : 0)>();
  else if (kStages >= 4 && ahead >= 2) wait_vm_lgkm0<(kStages >= 4 ? 2 * L : 0)>();
  else if (kStages >= 3 && ahead >= 1) wait_vm_lgkm0<L>();
  else wait_vm_lgkm0<0>();
}

template <int D>
struct Geom {
  static constexpr int kCpr = D / 8;                         // 16-byte chunks per row
  static constexpr int kChunks = kBN * kCpr;                 // chunks per tile and matrix
  static constexpr int kLoads = kChunks / kPrefillThreads;   // loads per thread, tile and matrix
  static constexpr int kTileBytes = kChunks * 16;
  static constexpr int kStageBytes = 2 * kTileBytes;         // one K^ and one V^ tile
  // V^ tiles start here, K^ tiles at 0; with kStages * kTileBytes <= 64 KB every
  // read's stage and row offsets fit the LDS instructions' 16-bit immediate
  static constexpr int kVRegion = kStages * kTileBytes;
  static_assert(kChunks % kPrefillThreads == 0, "every thread issues the same number of loads");
};

// Source offsets of this thread's chunks, relative to the tile's first row:
// LDS chunk p = i * threads + t holds row p / cpr, swizzled chunk p % cpr.
template <int D>
struct Issue {
  int row[Geom<D>::kLoads];
  int kcol[Geom<D>::kLoads];       // element offset of the K^ chunk within its row
  int vcol[Geom<D>::kLoads];
  uint32_t koff[Geom<D>::kLoads];  // byte offset of the K^ chunk from the tile's first row
  uint32_t voff[Geom<D>::kLoads];
};

template <int D>
__device__ __forceinline__ void make_issue(Issue<D>& is, int64_t row_stride) {
  constexpr int cpr = Geom<D>::kCpr;
#pragma unroll
  for (int i = 0; i < Geom<D>::kLoads; ++i) {
    const int p = i * kPrefillThreads + (int)threadIdx.x;
    const int r = p / cpr, cs = p % cpr;
    is.row[i] = r;
    is.kcol[i] = 8 * (cs ^ (r & (cpr - 1)));
    is.vcol[i] = 8 * (cs ^ v_swizzle<D>(r));
    is.koff[i] = (uint32_t)((r * row_stride + is.kcol[i]) * 2);
    is.voff[i] = (uint32_t)((r * row_stride + is.vcol[i]) * 2);
  }
}

// Request one K^/V^ tile into stage st (K^ at smem + st * tile bytes, V^ that
// far into the V^ region). Rows past `last` repeat row `last`.
template <int D>
__device__ __forceinline__ void issue_tile(const Issue<D>& is, const __bf16* kbase, const __bf16* vbase,
                                           int64_t row_stride, int key0, int last, YOCO_LDS char* smem, int st) {
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const uint32_t lds0 = (uint32_t)(uintptr_t)smem + st * Geom<D>::kTileBytes + wave * 64 * 16;
  if (key0 + kBN - 1 <= last) {
    // whole tile inside the sequence: one scalar base per matrix
    const int64_t toff = (int64_t)key0 * row_stride;
    const char* kt = reinterpret_cast<const char*>(kbase + toff);
    const char* vt = reinterpret_cast<const char*>(vbase + toff);
#pragma unroll
    for (int i = 0; i < Geom<D>::kLoads; ++i) {
      const uint32_t kd = lds0 + i * kPrefillThreads * 16;
      dma16(kt, is.koff[i], kd);
      dma16(vt, is.voff[i], kd + Geom<D>::kVRegion);
    }
  } else {
#pragma unroll
    for (int i = 0; i < Geom<D>::kLoads; ++i) {
      int key = key0 + is.row[i];
      key = key < last ? key : last;
      const int64_t roff = (int64_t)key * row_stride;
      const uint32_t kd = lds0 + i * kPrefillThreads * 16;
      dma16(kbase + roff + is.kcol[i], kd);
      dma16(vbase + roff + is.vcol[i], kd + Geom<D>::kVRegion);
    }
  }
}

// Lane-constant LDS byte offsets of the reads of one tile, relative to its
// stage's K^ tile (the V^ offsets include the distance to the V^ region).
template <int D>
struct ReadOffs {
  int k[D / 16];   // K^ A operand, step kk: row qj, chunk (2kk + hf) swizzled (+ kb * 32 rows)
  int v[D / 32];   // V^ transposing read, dim tile t (+ row offsets of kb, c, group)
};

template <int D>
__device__ __forceinline__ void make_read_offs(ReadOffs<D>& ro, int lane) {
  constexpr int cpr = Geom<D>::kCpr;
  const int qj = lane & 31, hf = lane >> 5;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) ro.k[kk] = qj * (D * 2) + 16 * ((2 * kk + hf) ^ (qj & (cpr - 1)));
  const int i = lane & 15, g = lane >> 4, h = lane >> 5;
  const int q = i >> 2, w = i & 3;
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
    // source row 4h + q of the 4-key group; dims 32t + 16(g%2) + 4w .. +3
    const int chunk = (4 * t + 2 * (g & 1) + (w >> 1)) ^ v_swizzle<D>(q);   // row 4h + q: r & 3 = q
    ro.v[t] = Geom<D>::kVRegion + (4 * h + q) * (D * 2) + 16 * chunk + 8 * (w & 1);
  }
}

// Calls f(integral_constant<int, 0>), f(..1>), ... in order while it returns true.
template <class F, int... I>
__device__ __forceinline__ bool each_stage(F& f, std::integer_sequence<int, I...>) {
  return (f(std::integral_constant<int, I>{}) && ...);
}

// Keeps the compiler's scheduler from moving instructions across this point,
// so LDS reads stay where they are issued, ahead of the MFMAs that use them.
__device__ __forceinline__ void sched_fence() {
#if YOCO_PREFILL_SCHED
  __builtin_amdgcn_sched_barrier(0);
#endif
}

// One K^ A-operand read of QK step i: kk = i / 2, kb = i % 2.
template <int D>
__device__ __forceinline__ bf16x8 read_k(const YOCO_LDS char* ks, const ReadOffs<D>& ro, int i) {
  return *reinterpret_cast<const YOCO_LDS bf16x8*>(ks + (i & 1) * 32 * (D * 2) + ro.k[i >> 1]);
}

// V^T A operand of PV step j (keys 32kb + 16cc + {0..3, 8..11} + 4h, dims of
// tile t): two transposing reads, rows +0 and +8. `tile` is the stage's K^ tile.
template <int D>
__device__ __forceinline__ bf16x8 read_v(const YOCO_LDS char* tile, const ReadOffs<D>& ro, int kb, int cc, int t) {
  const YOCO_LDS char* base = tile + (32 * kb + 16 * cc) * (D * 2) + ro.v[t];
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(base));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(base + 8 * (D * 2)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

#ifndef YOCO_PREFILL_RA
#define YOCO_PREFILL_RA 4
#endif
constexpr int kReadsAhead = YOCO_PREFILL_RA;  // LDS operand reads kept in flight ahead of the MFMAs

// S^T = K^ Q^T of one 64-key tile for one wave (16 or 8 MFMAs, two chains).
template <int D>
__device__ __forceinline__ void qk_step(const YOCO_LDS char* ks, const ReadOffs<D>& ro, const bf16x8 (&qf)[D / 16],
                                        f32x16 (&s)[2]) {
  constexpr int NQ = D / 8;
  constexpr int RA = kReadsAhead;
  s[0] = s[1] = f32x16{};
  bf16x8 ka[NQ];
#pragma unroll
  for (int i = 0; i < RA; ++i) ka[i] = read_k<D>(ks, ro, i);
#pragma unroll
  for (int i = 0; i < NQ; ++i) {
    if (i + RA < NQ) ka[i + RA] = read_k<D>(ks, ro, i + RA);
    s[i & 1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[i], qf[i >> 1], s[i & 1], 0, 0, 0);
    sched_fence();
  }
}

// Causal (MASK 1) and window (MASK 2) masks of a tile: register r of chain kb
// holds key key0 + 32kb + 8(r/4) + 4hf + r%4; keys past the row's (clamped)
// position pos, or before pos - window + 1, become -inf (compares with
// constants per register).
template <int MASK>
__device__ __forceinline__ void apply_mask(f32x16 (&s)[2], int key0, int pos, int window, int hf) {
  if constexpr (MASK != 0) {
    const int lim = pos - key0 - 4 * hf;
    const int lim_lo = lim - window + 1;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int rel = kb * 32 + 8 * (r >> 2) + (r & 3);
        if constexpr (MASK == 1) {
          if (rel > lim) s[kb][r] = -INFINITY;
        } else {
          if (rel > lim || rel < lim_lo) s[kb][r] = -INFINITY;
        }
      }
    }
  }
}

// Row max over chains kb0..1 of a tile and the lazy rescale of the running
// state: the reference m moves (and l, acc shrink by exp2(m - m_new)) only
// where the row's max passed m + slack. Returns -m for the exponentials.
template <int D>
__device__ __forceinline__ float rescale_to_max(const f32x16 (&s)[2], int kb0, f32x16 (&acc)[D / 32], float& m,
                                                float& l, float c) {
  float mx = -INFINITY;
#pragma unroll
  for (int kb = kb0; kb < 2; ++kb)
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  // lanes l and l ^ 32 hold the two key halves of one query row; the exchange
  // stays out of LDS, so it waits on none of the operand reads in flight
  mx = max_xor32(mx);
  const float mx2 = mx * c;  // c > 0: the max commutes with the scale
  // only the lanes whose own max grew move their reference, so every row's
  // arithmetic stays independent of the other rows of the wave
  const bool grow = mx2 > m + kRescaleSlack;
  if (__builtin_amdgcn_ballot_w64(grow) != 0) {
    const float m_new = grow ? mx2 : m;
    const float alpha = grow ? __builtin_amdgcn_exp2f(m - m_new) : 1.0f;  // exp2(-inf) = 0 on the first tile
    m = m_new;
    l *= alpha;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] *= alpha;
  }
  return m == -INFINITY ? 0.f : -m;
}

// P^T word w[kb][cc][i]: the weights of S^T registers 8cc + 2i and 8cc + 2i + 1
// of chain kb, as two bf16. Returns their unrounded fp32 sum (the row sum is
// kept from unrounded weights, so the LSE stays fp32-accurate).
__device__ __forceinline__ float softmax_word(const f32x16 (&s)[2], uint32_t (&w)[2][2][4], float c, float neg_m,
                                              int kb, int cc, int i) {
  const float e0 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * cc + 2 * i], c, neg_m));
  const float e1 = __builtin_amdgcn_exp2f(fmaf(s[kb][8 * cc + 2 * i + 1], c, neg_m));
  w[kb][cc][i] = pack2(e0, e1);
  return e0 + e1;
}

// PV step j of a tile: (kb, cc, t) with the dim tile t fastest, so consecutive
// MFMAs update different accumulators.
template <int D>
__device__ __forceinline__ void pv_index(int j, int& kb, int& cc, int& t) {
  constexpr int NT = D / 32;
  kb = j / (2 * NT);
  cc = (j / NT) & 1;
  t = j % NT;
}

// Softmax and O^T += V^T P^T of one tile whose S^T is in s. The exponentials
// of keys 32..63 are spread between the PV MFMAs of keys 0..31, which run
// while they issue.
//
// The weights of each 32-key half are first taken against the row's current
// reference m, without a max. Their sum bounds every one of them, so where a
// lane's half sums to at most kWeightCap every weight is at most that, well
// inside fp32 and bf16 range; softmax does not depend on the reference. Only if
// some lane's half sums to more (or to inf or NaN) does the wave take the row
// max of the tile (or of its second half), move m where it grew past the slack,
// and redo that half's exponentials; a wave with a row that has no reference
// yet (m = -inf) takes the max at once. Either way the weights that reach the
// MFMAs and the row sum use one m, and the running max itself is no longer
// computed on most tiles (about 20 VALU instructions per tile and wave fewer).
// neg_m is kept with m (-m, or 0 while m = -inf) and changes only with it.
template <int D, int MASK>
__device__ __forceinline__ void sv_step(const YOCO_LDS char* tile, const ReadOffs<D>& ro, f32x16 (&s)[2],
                                        f32x16 (&acc)[D / 32], float& m, float& neg_m, float& l, int key0, int pos,
                                        int window, float c, int hf) {
  constexpr int NV = D / 8;        // PV steps: (kb, cc, t)
  constexpr int RA = kReadsAhead;
  // the first V^ operands go out before the softmax, which hides their latency
  bf16x8 va[NV];
#pragma unroll
  for (int j = 0; j < RA; ++j) {
    int kb, cc, t;
    pv_index<D>(j, kb, cc, t);
    va[j] = read_v<D>(tile, ro, kb, cc, t);
  }
  sched_fence();
  apply_mask<MASK>(s, key0, pos, window, hf);
  uint32_t w[2][2][4];
  // a row without a reference yet (m = -inf: its first keys) takes the max first
  bool exact = __builtin_amdgcn_ballot_w64(m == -INFINITY) != 0;
  float la;
  for (;;) {   // at most twice: after a rescale the weights are taken as they are
    if (exact) neg_m = rescale_to_max<D>(s, 0, acc, m, l, c);
    la = softmax_word(s, w, c, neg_m, 0, 0, 0);
#pragma unroll
    for (int wi = 1; wi < 8; ++wi) la += softmax_word(s, w, c, neg_m, 0, wi >> 2, wi & 3);
    if (exact || __builtin_amdgcn_ballot_w64(!(la <= kWeightCap)) == 0) break;
    exact = true;
  }
  l += la;
  float lb;
  sched_fence();
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    int kb, cc, t;
    pv_index<D>(j, kb, cc, t);
    if (j == NV / 2) {
      // the second half's weights are checked before its first MFMA
      if (__builtin_amdgcn_ballot_w64(!(lb <= kWeightCap)) != 0) {
        neg_m = rescale_to_max<D>(s, 1, acc, m, l, c);
        lb = softmax_word(s, w, c, neg_m, 1, 0, 0);
#pragma unroll
        for (int wi = 1; wi < 8; ++wi) lb += softmax_word(s, w, c, neg_m, 1, wi >> 2, wi & 3);
      }
      l += lb;
      sched_fence();
    }
    if (j + RA < NV) {
      int kb2, cc2, t2;
      pv_index<D>(j + RA, kb2, cc2, t2);
      va[j + RA] = read_v<D>(tile, ro, kb2, cc2, t2);
    }
    const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w[kb][cc][0], w[kb][cc][1], w[kb][cc][2], w[kb][cc][3]));
    acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[j], pb, acc[t], 0, 0, 0);
    // keys 32..63: 8 words over the NV / 2 MFMAs of keys 0..31
    if (j < NV / 2) {
#pragma unroll
      for (int q = 0; q < 8 / (NV / 2); ++q) {
        const int wi = j * (8 / (NV / 2)) + q;
        const float e = softmax_word(s, w, c, neg_m, 1, wi >> 2, wi & 3);
        lb = wi == 0 ? e : lb + e;
      }
    }
    sched_fence();
  }
}

// 0 in a vector register, unknown to the optimiser. Added to the address of the
// claim made ahead, it keeps the compiler from combining that atomic across the
// wave (which reads its result back at once and so waits for its round trip
// and every copy in flight): the result is then first awaited where it is used,
// at the end of the item.
__device__ __forceinline__ int lane_zero() {
  int z = 0;
  asm volatile("" : "+v"(z));
  return z;
}

// Work-queue fetch (thread 0 of a workgroup): the next item of this XCD's
// queue, else of the first other queue that still has items; n_items when all
// are empty. The counters of all queues are read in one round trip, then one
// is incremented; a lost race (the queue emptied meanwhile) reads again.
__device__ __forceinline__ int queue_fetch(int* q, int xcd, int n_items) {
  for (;;) {
    int cnt[kXcds];
#pragma unroll
    for (int x = 0; x < kXcds; ++x)
      cnt[x] = __hip_atomic_load(q + x * kQueueStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    int pick = -1, len = 0;
#pragma unroll
    for (int k = 0; k < kXcds; ++k) {
      const int x = (xcd + k) & (kXcds - 1);
      const int lx = n_items > x ? (n_items - x + kXcds - 1) / kXcds : 0;
      if (pick < 0 && cnt[x] < lx) pick = x, len = lx;
    }
    if (pick < 0) return n_items;
    const int j = __hip_atomic_fetch_add(q + pick * kQueueStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (j < len) return pick + kXcds * j;
  }
}

// With units a multiple of the XCD count, queue x lists its units one after
// the other, P = pos_blocks items each. An empty item means that its unit's
// sequence has fewer position blocks (nb) than P: the unit's other empty items
// are skipped at once by raising the queue's counter past them (causal order:
// the first P - nb items of a unit are empty; window order: the last P - nb).
__device__ __forceinline__ void skip_empty_items(const AttnParams& p, int item, int units, int nb) {
  if (units % kXcds != 0) return;
  const int x = item % kXcds, j = item / kXcds;
  const int P = p.pos_blocks;
  const int first = (j / P) * P;
  int target;
  if (p.window > 0 || nb <= 0 || nb >= P) target = first + P;   // the unit's remaining items are empty
  else target = first + (P - nb);                                 // its first non-empty item
  if (target > j + 1)
    __hip_atomic_fetch_max(p.queue + x * kQueueStride, target, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int D>
__global__ __launch_bounds__(kPrefillThreads, 2) void prefill_bf16_kernel(AttnParams p) {
  constexpr int kStage = Geom<D>::kStageBytes;
  constexpr int kOStride = D + 8;  // output staging row (elements)
  static_assert(kPrefillWaves * kPrefillRowsPerWave * kOStride * 2 <= kStages * kStage, "staging fits");
  __shared__ __attribute__((aligned(16))) char smem_raw[kStages * kStage];
  YOCO_LDS char* smem = (YOCO_LDS char*)smem_raw;

  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int qj = lane & 31;
  const int hf = lane >> 5;

  const int hpw = prefill_heads_per_wg(p.group);
  const int ppw = kPrefillWaves / hpw;
  const int hchunks = p.group / hpw;
  const int units = p.batch * p.hkv * hchunks;
  const int pos_per_wg = kPrefillRowsPerWave * ppw;
  const float c = p.scale_log2;
  const int64_t row_stride = (int64_t)p.hkv * D;
  const __bf16* qbase = static_cast<const __bf16*>(p.q);

  Issue<D> is;
  make_issue<D>(is, row_stride);
  ReadOffs<D> ro;
  make_read_offs<D>(ro, lane);
  constexpr int L = 2 * Geom<D>::kLoads;   // loads per thread and tile

  // Work items: with a queue, this (persistent) workgroup takes items until
  // every queue is empty; the next item is fetched by thread 0 while the
  // current one's first tiles are in flight and handed over through LDS
  // (two slots, alternating, so a slot is rewritten only after a later barrier).
  __shared__ int s_item[2];
  const bool dyn = p.queue != nullptr;
  const int xcd = blockIdx.x % kXcds;
  int par = 0;
  int item = blockIdx.x;
  if (dyn) {
    if (threadIdx.x == 0) s_item[0] = queue_fetch(p.queue, xcd, p.n_items);
    __syncthreads();
    item = __builtin_amdgcn_readfirstlane(s_item[0]);   // uniform: everything derived stays scalar
    par = 1;
  }
  while (item < p.n_items) {
  int unit, rank;
  prefill_schedule(item, units, p.pos_blocks, &unit, &rank);
  const int hc = unit % hchunks;
  const int kh = (unit / hchunks) % p.hkv;
  const int b = unit / (hchunks * p.hkv);
  // wave -> (head, position block): heads fastest
  const int h = kh * p.group + hc * hpw + wave % hpw;
  const int pbl = wave / hpw;

  int64_t start = 0;
  int32_t n_kv = 0, n_q = 0;
  if (rank < p.pos_blocks && b < p.batch) {
    n_kv = readable_rows(p.seq_start, p.seq_len, p.seq_cap, p.pool_rows, b, &start);
    int64_t q0_ = p.cu_seqlens[b];
    int64_t q1_ = p.cu_seqlens[b + 1];
    if (q1_ > p.total_q) q1_ = p.total_q;
    if (q0_ >= 0 && q0_ <= q1_) n_q = (int32_t)(q1_ - q0_);
  }
  const int64_t q0 = n_q > 0 ? p.cu_seqlens[b] : 0;
  const int32_t offset = n_kv > n_q ? n_kv - n_q : 0;

  const __bf16* kbase = static_cast<const __bf16*>(p.k) + start * row_stride + (int64_t)kh * D;
  const __bf16* vbase = static_cast<const __bf16*>(p.v) + start * row_stride + (int64_t)kh * D;

  // causal: longest position blocks first (the last finish with the short ones).
  // Sliding window: blocks are (nearly) equally long, so workgroups started
  // together would also load and store together, each round; shortest first
  // (the first window's blocks are shorter) spreads their phases after round
  // one (+2-3% at C = 1024)
  const int pw0 = p.window > 0 ? rank : p.pos_blocks - 1 - rank;
  // The next item of this XCD's queue is claimed while this one runs (thread 0,
  // once this item's first tiles are in) and its index read only at the end,
  // so the atomic's round trip overlaps this item. Not near the end of the
  // queue (within 4 items per workgroup of this XCD, as the counter read when
  // the item starts shows): an item claimed ahead can no longer go to an idle
  // workgroup, and held behind a long one it would end the launch late; there
  // the next item is taken when this one is done.
  const int own = p.n_items > xcd ? (p.n_items - xcd + kXcds - 1) / kXcds : 0;   // this XCD's queue length
  int spec = -1, seen = 0;
  if (dyn && threadIdx.x == 0) {
    seen = __hip_atomic_load(p.queue + xcd * kQueueStride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (pw0 < 0 || pw0 * pos_per_wg >= n_q)   // an empty item (a position block past its sequence's end)
      skip_empty_items(p, item, units, (n_q + pos_per_wg - 1) / pos_per_wg);
  }
  for (int pw = pw0; pw >= 0 && pw * pos_per_wg < n_q; pw += p.pos_blocks) {
    const int wg_last_row = min(n_q, (pw + 1) * pos_per_wg) - 1;
    const int wg_last_key = min(wg_last_row + offset, n_kv - 1);
    const int n_tiles = wg_last_key >= 0 ? wg_last_key / kBN + 1 : 0;
    const int r0 = pw * pos_per_wg + pbl * kPrefillRowsPerWave;
    // a row whose position has no cache row of its own (more query rows than
    // cache rows) gets the empty result, O = 0 and LSE = -inf: its own row is
    // written before any Cross-Decoder layer reads the cache, so nothing else
    // is defined for it; the clamp only keeps its (discarded) masking in range
    const int my_pos = min(r0 + qj + offset, n_kv - 1);
    const bool own_row = r0 + qj + offset < n_kv;
    const bool wave_active = r0 < n_q && r0 + offset < n_kv;
    const int wave_max_pos = min(r0 + kPrefillRowsPerWave, n_q) - 1 + offset;
    // tiles below full_tiles need no causal mask for any row of this wave
    const int full_tiles = min((r0 + offset + 1) / kBN, n_kv / kBN);
    // sliding window: the workgroup starts at the first tile its first row sees;
    // a wave skips tiles wholly before its rows' windows and masks the lower
    // edge below band_full (keys from there on lie in every row's window)
    const int win = p.window;
    const int kt_lo = win > 0 ? max(0, min(pw * pos_per_wg + offset, n_kv - 1) - win + 1) / kBN : 0;
    const int wave_key_lo = win > 0 ? max(0, min(r0 + offset, n_kv - 1) - win + 1) : 0;
    const int band_full = win > 0 ? min(wave_max_pos, n_kv - 1) - win + 1 : 0;

    // the tiles ahead go out first: they have the longest way. Tile kt of this
    // pass goes to stage (kt - kt_lo) mod S
#pragma unroll
    for (int st = 0; st < kStages - 1; ++st)
      if (kt_lo + st < n_tiles)
        issue_tile<D>(is, kbase, vbase, row_stride, (kt_lo + st) * kBN, n_kv - 1, smem, st);

    bf16x8 qf[D / 16];
    {
      const int my_row = min(r0 + qj, n_q - 1);
      const __bf16* qsrc = qbase + ((q0 + my_row) * p.hq + h) * D + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk)
        qf[kk] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qsrc + 16 * kk));
    }
    // Q^ (and the first tiles) in: from here on the only loads in flight are
    // tile copies, which the loop awaits by count
    wait_vm_lgkm0<0>();
    if (dyn && threadIdx.x == 0 && pw == pw0 && seen < own - 4 * (int)(gridDim.x / kXcds))
      spec = __hip_atomic_fetch_add(p.queue + xcd * kQueueStride + lane_zero(), 1, __ATOMIC_RELAXED,
                                    __HIP_MEMORY_SCOPE_AGENT);
    f32x16 acc[D / 32];
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
    float m = -INFINITY, neg_m = 0.f, l = 0.f;

    // One tile, from stage U (a constant, so every operand read is a register
    // plus an immediate offset); false once the pass has no tile kt0 + U.
    int kt0 = kt_lo;
    auto tile_step = [&](auto stage) __attribute__((always_inline)) -> bool {
      constexpr int u = decltype(stage)::value;
      const int kt = kt0 + u;
      if (kt >= n_tiles) return false;
      // tile kt has landed in LDS (this thread's part): at most the tiles
      // requested after it may still be in flight
      wait_tiles<L>(min(kStages - 2, n_tiles - 1 - kt));
      barrier_only();  // every thread's part of tile kt is in; the stage of tile kt - 1 is free
      if (kt + kStages - 1 < n_tiles)
        issue_tile<D>(is, kbase, vbase, row_stride, (kt + kStages - 1) * kBN, n_kv - 1, smem,
                      (u + kStages - 1) % kStages);
      const int key0 = kt * kBN;
      if (wave_active && key0 <= wave_max_pos && key0 + kBN > wave_key_lo) {
        const YOCO_LDS char* tile = smem + u * Geom<D>::kTileBytes;   // K^ here, V^ by the offsets in ro.v
        f32x16 s[2];
        qk_step<D>(tile, ro, qf, s);
        if (win > 0 && key0 < band_full)
          sv_step<D, 2>(tile, ro, s, acc, m, neg_m, l, key0, my_pos, win, c, hf);
        else if (kt >= full_tiles)
          sv_step<D, 1>(tile, ro, s, acc, m, neg_m, l, key0, my_pos, win, c, hf);
        else
          sv_step<D, 0>(tile, ro, s, acc, m, neg_m, l, key0, my_pos, win, c, hf);
      }
      return true;
    };
    for (; kt0 < n_tiles; kt0 += kStages)
      if (!each_stage(tile_step, std::make_integer_sequence<int, kStages>{})) break;
    wait_vm_lgkm0<0>();
    barrier_only();  // every wave is done with the tiles: the stages become the output staging area

    // Epilogue: normalise, stage the wave's 32 x D output tile in LDS, then
    // store whole rows with 16-byte writes.
    const float l_tot = own_row ? sum_xor32(l) : 0.f;
    const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
    YOCO_LDS __bf16* ot = (YOCO_LDS __bf16*)smem + wave * (kPrefillRowsPerWave * kOStride);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const u32x2 wv = {pack2(acc[t][4 * g4 + 0] * inv, acc[t][4 * g4 + 1] * inv),
                          pack2(acc[t][4 * g4 + 2] * inv, acc[t][4 * g4 + 3] * inv)};
        *reinterpret_cast<YOCO_LDS u32x2*>(ot + qj * kOStride + 32 * t + 8 * g4 + 4 * hf) = wv;
      }
    }
    if (hf == 0 && p.lse != nullptr && r0 + qj < n_q)
      p.lse[(int64_t)h * p.total_q + q0 + r0 + qj] =
          l_tot > 0.f ? (m + log2f(l_tot)) * 0.6931471805599453f : -INFINITY;
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __bf16* obase = static_cast<__bf16*>(p.out);
#pragma unroll
    for (int i = 0; i < kPrefillRowsPerWave * (D / 8) / 64; ++i) {
      const int ci = lane + 64 * i;
      const int row = ci / (D / 8);
      const int c8 = ci % (D / 8);
      if (r0 + row < n_q)
        *reinterpret_cast<u32x4*>(obase + ((q0 + r0 + row) * p.hq + h) * D + 8 * c8) =
            *reinterpret_cast<const YOCO_LDS u32x4*>(ot + row * kOStride + 8 * c8);
    }
    __syncthreads();  // the staging area is the next pass's first stage
  }
  if (!dyn) break;
  if (threadIdx.x == 0)
    s_item[par] = spec >= 0 && spec < own ? xcd + kXcds * spec : queue_fetch(p.queue, xcd, p.n_items);
  __syncthreads();
  item = __builtin_amdgcn_readfirstlane(s_item[par]);
  par ^= 1;
  }
  if (dyn && threadIdx.x == 0) {
    // every workgroup has left its fetch loop once the done count reaches the
    // grid: the last one zeroes the counters for the next call
    int* q = p.queue;
    const int done = __hip_atomic_fetch_add(q + kXcds * kQueueStride, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done == (int)gridDim.x - 1)
      for (int i = 0; i < kQueueCounters; ++i)
        __hip_atomic_store(q + i * kQueueStride, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace

namespace {

// With a work queue the grid is persistent: as many workgroups as the device
// holds at once (CUs times the kernel's occupancy), each taking items until
// the queues are empty; without one, one workgroup per item.
template <int D>
hipError_t launch_prefill(const AttnParams& p, int items, hipStream_t stream) {
  int grid = items;
  if (p.queue != nullptr) {
    int dev = 0, cus = 0, per_cu = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err == hipSuccess) err = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (err == hipSuccess)
      err = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, reinterpret_cast<const void*>(prefill_bf16_kernel<D>),
                                                         kPrefillThreads, 0);
    if (err != hipSuccess) return err;
    const int64_t wgs = (int64_t)(cus > 0 ? cus : 1) * (per_cu > 0 ? per_cu : 1);
    if (grid > wgs) grid = (int)wgs;
  }
  hipLaunchKernelGGL(prefill_bf16_kernel<D>, dim3(grid), dim3(kPrefillThreads), 0, stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_bf16(const AttnParams& p, int head_dim, int items, hipStream_t stream) {
  return head_dim == 64 ? launch_prefill<64>(p, items, stream) : launch_prefill<128>(p, items, stream);
}

}  // namespace yoco
