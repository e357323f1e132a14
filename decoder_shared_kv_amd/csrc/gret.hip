// Gated retention (gRet), the Self-Decoder's default attention ("YOCO 深度技术分析",
// liuhc.cn, section 2.2: the parallel form (Q K^T ⊙ D) V with the data-controlled
// decay D[n][m] = γ_{m+1} ... γ_n, the recurrent form S_n = γ_n S_{n-1} + K_n^T V_n,
// o_n = Q_n S_n, and the chunkwise form; section 5.3.2: chunks of 256 rows).
//
// Prefill runs the chunkwise form in three launches. A sequence's chunks are
// grouped into segments of seg_chunks consecutive chunks (the segments of all
// sequences numbered one after the other and located on the device, so every
// row is computed whatever the lengths); every (segment, head) works in
// parallel and only the recurrence across segments is serial:
//   1. gret_segstate_kernel: per segment, its contribution to the state, U, and
//      its total decay, by the chunk recurrence U <- G_c U + sum_m w_m k_m^T v_m
//      (w_m the decay from row m to the chunk's end; MFMA: U = (w ⊙ K)^T V, both
//      operands by transposing LDS reads, U in fp32 accumulators);
//   2. gret_segscan_kernel: S_{s+1} = G_s S_s + U_s over the segments (fp32),
//      writing each segment's incoming state and the final state;
//   3. gret_out_kernel: per segment, chunk after chunk, carrying the state
//      in fp32 accumulators: o_j = e_j q_j S_c + sum_{m <= j} (e_j / e_m)
//      (q_j . k_m) v_m with e_j the decay from the chunk's start to row j (the
//      first term one MFMA product with S_c staged in LDS as bf16, the second
//      the intra-chunk parallel form, tiled like attention: S^T = K Q^T, decay
//      and causal mask on the accumulator registers, O^T += V^T P^T, without a
//      softmax), then S_{c+1} = G_c S_c + (w ⊙ K)^T V from the same LDS tiles.
// Decays are handled as base-2 logarithms, accumulated along the chunk; a gate
// below 2^-126 counts as 2^-126 (its products vanish below fp32's range).
// Decode is the recurrent form's step on the fp32 state (gret_decode_kernel).

#include "internal.h"
#include "lds_copy.h"
#include "tile_common.h"

namespace yoco {

namespace {

constexpr int kGC = 256;           // rows per chunk
constexpr int kGT = 64;            // keys per LDS tile in the output kernel
constexpr int kGThreads = 512;     // 8 waves, 32 rows each
constexpr float kLogGateFloor = -126.0f;

// LDS barrier that leaves the tile copies in flight: waits for this wave's own
// LDS accesses (lgkmcnt 0, vmcnt left at its maximum), then s_barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
  barrier_only();
}

// Inclusive prefix sum over a wave's lanes on DPP lane moves, no LDS: the same
// pattern as wave_incl_scan_i32, on fp32 values.
template <int CTRL, int ROW_MASK, bool BOUND>
__device__ __forceinline__ float dpp_add(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, ROW_MASK, 0xf, BOUND));
}
__device__ __forceinline__ float wave_incl_scan_f32(float x) {
  x += dpp_add<0x111, 0xf, true>(x);    // row_shr:1 (lanes shifted in read 0)
  x += dpp_add<0x112, 0xf, true>(x);    // row_shr:2
  x += dpp_add<0x114, 0xf, true>(x);    // row_shr:4
  x += dpp_add<0x118, 0xf, true>(x);    // row_shr:8
  x += dpp_add<0x142, 0xa, false>(x);   // row_bcast:15 into rows 1 and 3
  x += dpp_add<0x143, 0xc, false>(x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// inclusive prefix sum of 256 values held by threads 0..255 (one each); every
// thread of the workgroup must call it. Returns the sum up to and including
// this thread's value (threads >= 256 get garbage). kWaitAll: the barrier also
// waits for every memory access in flight (__syncthreads); otherwise copies
// to LDS may stay in flight across it.
template <bool kWaitAll = true>
__device__ __forceinline__ float chunk_prefix(float x, float* wsum) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  x = wave_incl_scan_f32(x);
  if (lane == 63 && wave < 4) wsum[wave] = x;
  if constexpr (kWaitAll) __syncthreads();
  else lds_barrier();
  float add = 0.f;
  for (int w = 0; w < wave && w < 4; ++w) add += wsum[w];
  return x + add;
}

// base-2 log of the gate of chunk row j (rows past the chunk's end: gate 1)
__device__ __forceinline__ float log2_gate(const float* gamma, int64_t row, int h, int H, bool valid) {
  if (!valid) return 0.f;
  const float g = gamma[row * H + h];
  const float l = __log2f(g);
  return l > kLogGateFloor ? l : kLogGateFloor;   // also catches g = 0 (log -inf) and NaN-free clamps
}

// LDS byte offset of 16-byte chunk c of row r of a row-major [rows][D] bf16 tile
// that is read with transposing reads
template <int D>
__device__ __forceinline__ uint32_t tr_slot(int r, int c) {
  return (uint32_t)(r * (D * 2) + 16 * (c ^ v_swizzle<D>(r)));
}
// ... and of one that is read row-wise (16 bytes per lane): chunk c at c ^ (r mod chunks)
template <int D>
__device__ __forceinline__ uint32_t row_slot(int r, int c) {
  return (uint32_t)(r * (D * 2) + 16 * (c ^ (r & (D / 8 - 1))));
}
// ... and of a K tile of the output pass, read both ways (row-wise for the
// scores, transposed for the state update): chunk c at c ^ kd_swizzle(r), a map
// linear in the bits of r mod 16 under which 16 consecutive rows at one chunk
// and the 8 rows x 64 bytes of a transposing read both fall on distinct banks
// (D = 128, for 32 and for 64 banks, checked by enumeration on the host; for
// D = 64 no such map exists and this one keeps the transposing reads whole)
template <int D>
__device__ __forceinline__ int kd_swizzle(int r) {
  if constexpr (D == 128) {
    return ((r >> 2) & 3) ^ (12 * (r & 1)) ^ (6 * ((r >> 1) & 1));
  } else {
    return (4 * (r & 1)) ^ (2 * ((r >> 1) & 1)) ^ ((r >> 2) & 1);
  }
}
template <int D>
__device__ __forceinline__ uint32_t kd_slot(int r, int c) {
  return (uint32_t)(r * (D * 2) + 16 * (c ^ kd_swizzle<D>(r)));
}

// ... and of the output pass's V tile, read transposed both by the state update
// (4 rows x 64 bytes per 16 lanes) and by the products with the scores (16 lanes
// at 4 rows x 32 bytes, the lane groups 4 rows apart): a map linear in the bits
// of r mod 8 under which both fall on distinct banks (32 lanes x 8 bytes; 32
// and 64 banks, checked by enumeration on the host)
template <int D>
__device__ __forceinline__ int pv_swizzle(int r) {
  if constexpr (D == 128) {
    return (4 * (r & 1)) ^ (10 * ((r >> 1) & 1)) ^ (2 * ((r >> 2) & 1));
  } else {
    return (2 * (r & 1)) ^ (4 * ((r >> 1) & 1)) ^ (2 * ((r >> 2) & 1));
  }
}

enum TileLayout { kRowLayout, kTrLayout, kKdLayout, kPvLayout };

// x, hidden from the optimiser: per-lane offsets derived from it are computed
// where they are used instead of being kept live (or spilled) across a loop
__device__ __forceinline__ int opaque(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

template <int D, int LAYOUT>
__device__ __forceinline__ int tile_swizzle(int r) {
  if constexpr (LAYOUT == kRowLayout) return r & (D / 8 - 1);
  else if constexpr (LAYOUT == kTrLayout) return v_swizzle<D>(r);
  else if constexpr (LAYOUT == kPvLayout) return pv_swizzle<D>(r);
  else return kd_swizzle<D>(r);
}

// Transposing read: 8 bf16 of one column (dim 32t + lane col) at rows
// base + 4h + {0..3} and base + 8 + 4h + {0..3} of a tr_slot (or kd_slot) tile.
template <int D, int LAYOUT = kTrLayout>
__device__ __forceinline__ bf16x8 read_tr(const YOCO_LDS char* tile, int base_row, int t, int lane) {
  const int i = lane & 15, g = lane >> 4, h = lane >> 5;
  const int q = i >> 2, w = i & 3;
  const int r = base_row + 4 * h + q;
  const int chunk = 4 * t + 2 * (g & 1) + (w >> 1);
  // rows r and r + 8 (the kd swizzle depends on bit 3 of the row, the
  // transposing one only on r mod 4)
  const YOCO_LDS char* p = tile + r * (D * 2) + 16 * (chunk ^ tile_swizzle<D, LAYOUT>(r)) + 8 * (w & 1);
  const YOCO_LDS char* p8 = tile + (r + 8) * (D * 2) + 16 * (chunk ^ tile_swizzle<D, LAYOUT>(r + 8)) + 8 * (w & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(p8));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Transposing read of a 16 x 32 A operand V^T of a 16 x 16 x 32 product from a
// kPvLayout tile: dims 16t + (lane & 15) at rows base + 4g + {0..3} and
// base + 16 + 4g + {0..3}, g = lane / 16 (k slots 8g .. 8g + 7 in that order).
template <int D>
__device__ __forceinline__ bf16x8 read_pv(const YOCO_LDS char* tile, int base_row, int t, int lane) {
  const int i = lane & 15, g = lane >> 4;
  const int r = base_row + 4 * g + (i >> 2);
  const int chunk = 2 * t + ((i & 3) >> 1);
  const YOCO_LDS char* p = tile + r * (D * 2) + 16 * (chunk ^ pv_swizzle<D>(r)) + 8 * (i & 1);
  const YOCO_LDS char* p16 = tile + (r + 16) * (D * 2) + 16 * (chunk ^ pv_swizzle<D>(r + 16)) + 8 * (i & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(p16));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Copy tile rows [first, first + rows) of a [rows, H, D] bf16 tensor (row
// stride H*D) whose row 0 is global row `row0` (rows >= n_rows, n_rows >= 1,
// repeat row n_rows - 1) into LDS at `lds` (tile row `first` at offset 0), in
// the given layout, by the load unit (tid: this thread's index in the
// workgroup). rows * D / 8 must be a multiple of the thread count, `first` a
// multiple of 16. STREAM: with the nontemporal hint, for rows not read again
// soon (the state pass's K and V, the output pass's Q rows: measured 7% faster
// per call at 32K rows than cached copies; the output pass's K and V tiles stay
// cached, the hint there was slower on ragged batches).
// (copy i of this thread alone: load_tile_one)
template <int D, int LAYOUT, bool STREAM = false>
__device__ __forceinline__ void load_tile_one(const __bf16* src, int64_t row0, int n_rows, int first, int H, int h,
                                              uint32_t lds, int tid, int i) {
  constexpr int cpr = D / 8;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int p = i * kGThreads + tid;
  const int r = first + p / cpr, slot = p % cpr;
  const int c = slot ^ tile_swizzle<D, LAYOUT>(r);
  const int rr = r < n_rows ? r : n_rows - 1;
  if constexpr (STREAM) dma16_nt(src + ((row0 + rr) * H + h) * D + 8 * c, lds + (i * kGThreads + wave * 64) * 16);
  else dma16(src + ((row0 + rr) * H + h) * D + 8 * c, lds + (i * kGThreads + wave * 64) * 16);
}
template <int D, int LAYOUT, bool STREAM = false>
__device__ __forceinline__ void load_tile(const __bf16* src, int64_t row0, int n_rows, int first, int rows, int H,
                                          int h, uint32_t lds, int tid) {
  for (int i = 0; i < rows * (D / 8) / kGThreads; ++i)
    load_tile_one<D, LAYOUT, STREAM>(src, row0, n_rows, first, H, h, lds, tid, i);
}

// The A operand of a state-update product, U += (w ⊙ K)^T V over 16 keys: the
// K columns read transposed (elements 4z..4z+3 at keys base + 8z + 4h + {0..3}),
// each times its key's weight (w0: keys base + 4h + {0..3}, w1: base + 8 + ...).
__device__ __forceinline__ bf16x8 weight_keys(const bf16x8 kb, const f32x4 w0, const f32x4 w1) {
  uint32_t wv[4];
#pragma unroll
  for (int z = 0; z < 2; ++z) {
    const f32x4 ww = z == 0 ? w0 : w1;
    wv[2 * z] = pack2((float)kb[4 * z + 0] * ww[0], (float)kb[4 * z + 1] * ww[1]);
    wv[2 * z + 1] = pack2((float)kb[4 * z + 2] * ww[2], (float)kb[4 * z + 3] * ww[3]);
  }
  return __builtin_bit_cast(bf16x8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
}

// Keeps the scheduler from moving instructions across this point, so that LDS
// operand reads stay issued ahead of the MFMAs that use them.
__device__ __forceinline__ void sched_fence() { __builtin_amdgcn_sched_barrier(0); }
constexpr int kGReadsAhead = 4;   // LDS operand reads kept in flight ahead of the MFMAs (output pass)

struct ChunkInfo {
  int64_t row0;   // first global row of the chunk
  int n;          // rows of the chunk (0: no chunk)
};

// Rows of sequence b (clamped to the packed rows), its chunks and its segments
// (runs of p.seg_chunks consecutive chunks, the unit of work of both passes
// that read K and V).
__device__ __forceinline__ int64_t seq_rows(const GretParams& p, int b) {
  int64_t r0 = p.cu_seqlens[b], r1 = p.cu_seqlens[b + 1];
  if (r1 > p.total_rows) r1 = p.total_rows;
  return (r0 >= 0 && r1 > r0) ? r1 - r0 : 0;
}
__device__ __forceinline__ int seq_chunks(const GretParams& p, int b) {
  return (int)((seq_rows(p, b) + kGC - 1) / kGC);
}
__device__ __forceinline__ int seq_segs(const GretParams& p, int b) {
  return (seq_chunks(p, b) + p.seg_chunks - 1) / p.seg_chunks;
}

// The segments of all sequences are numbered one after the other (sequence 0's
// first), so a grid over the workspace's slots covers every row whatever the
// lengths. Global segment g -> (sequence b, its segment s), counted by the
// whole wave (64 sequences per step: segment counts, a DPP prefix sum, a ballot
// for the first sequence whose prefix passes g). All 64 lanes must be active.
// False if g is past the last segment.
__device__ __forceinline__ bool locate_segment(const GretParams& p, int g, int* b_out, int* s_out) {
  const int lane = threadIdx.x & 63;
  int before = 0;   // segments of the sequences before this group of 64
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int bb = b0 + lane;
    const int n = bb < p.batch ? seq_segs(p, bb) : 0;
    const int incl = wave_incl_scan_i32(n);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (g < before + total) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(before + incl > g);
      const int l = __builtin_ctzll(m);
      *b_out = b0 + l;
      *s_out = g - before - (__builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(n, l));
      return true;
    }
    before += total;
  }
  return false;
}

// First global segment of sequence b (scalar loop over the sequences before it).
__device__ __forceinline__ int64_t seg_start(const GretParams& p, int b) {
  int64_t g = 0;
  for (int i = 0; i < b; ++i) g += seq_segs(p, i);
  return g;
}

// Rows [r0, r1) of a sequence (clamped to the packed rows; r1 <= r0: none).
struct SeqRows {
  int64_t r0, r1;
};
__device__ __forceinline__ SeqRows seq_range(const GretParams& p, int b) {
  SeqRows sr{p.cu_seqlens[b], p.cu_seqlens[b + 1]};
  if (sr.r1 > p.total_rows) sr.r1 = p.total_rows;
  return sr;
}
// Chunk c of a sequence, from its row range (no memory access)
__device__ __forceinline__ ChunkInfo chunk_of(const SeqRows& sr, int c) {
  ChunkInfo ci{sr.r0 + (int64_t)c * kGC, 0};
  if (sr.r0 < 0 || sr.r1 <= sr.r0) return ci;
  const int64_t left = sr.r1 - ci.row0;
  ci.n = left <= 0 ? 0 : (left < kGC ? (int)left : kGC);
  return ci;
}
__device__ __forceinline__ ChunkInfo chunk_info(const GretParams& p, int b, int c) {
  return chunk_of(seq_range(p, b), c);
}

// This wave's blocks of a head_dim x head_dim state held as MFMA accumulators:
// blocks (bi, bj) of 32 x 32, rows dk = 32 bi + 8(r/4) + 4hf + r%4 in register r,
// column dv = 32 bj + lane % 32. D = 128: 16 blocks, two per wave (same bi);
// D = 64: 4 blocks, waves 0..3 (waves 4..7 hold none).
template <int D>
struct StateBlocks {
  static constexpr int NB = D / 32;
  static constexpr int PER = (NB * NB) / 8 > 0 ? (NB * NB) / 8 : 1;
  bool idle;
  int blk0, bi;
  __device__ explicit StateBlocks(int wave) {
    idle = wave * PER >= NB * NB;
    blk0 = idle ? 0 : wave * PER;
    bi = blk0 / NB;
  }
  __device__ int bj(int e) const { return (blk0 + e) % NB; }
};

// One 16-key step of a state update S += (w ⊙ K)^T V for this wave's blocks:
// its LDS operands (K columns of block row bi, transposed; the keys' weights;
// V columns of each block column, transposed), read ahead of the MFMAs.
template <int PER>
struct StepOps {
  bf16x8 k;
  f32x4 w0, w1;
  bf16x8 v[PER];
  template <int D, int KLAYOUT, int VLAYOUT = kTrLayout>
  __device__ __forceinline__ void read(const YOCO_LDS char* kt, const YOCO_LDS char* vt, const YOCO_LDS float* w,
                                       int key0, int base_row, const StateBlocks<D>& sb, int lane) {
    const int hf = lane >> 5;
    k = read_tr<D, KLAYOUT>(kt, base_row, sb.bi, lane);
    w0 = *reinterpret_cast<const YOCO_LDS f32x4*>(w + key0 + base_row + 4 * hf);
    w1 = *reinterpret_cast<const YOCO_LDS f32x4*>(w + key0 + base_row + 8 + 4 * hf);
#pragma unroll
    for (int e = 0; e < PER; ++e) v[e] = read_tr<D, VLAYOUT>(vt, base_row, sb.bj(e), lane);
  }
  __device__ __forceinline__ void mfma(f32x16 (&acc)[PER]) const {
    const bf16x8 kw = weight_keys(k, w0, w1);
#pragma unroll
    for (int e = 0; e < PER; ++e) acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kw, v[e], acc[e], 0, 0, 0);
  }
};

// Wait until at most n of this wave's copies are in flight (n from a short list
// of wave-uniform values: the waits need an immediate).
template <int LQ>
__device__ __forceinline__ void wait_copies(int n) {
  if (n == 0) wait_vm_lgkm0<0>();
  else if (n == LQ) wait_vm_lgkm0<LQ>();
  else if (n == LQ + 1) wait_vm_lgkm0<LQ + 1>();
  else if (n == 2 * LQ) wait_vm_lgkm0<2 * LQ>();
  else wait_vm_lgkm0<2 * LQ + 1>();
}

// ---------------------------------------------------------------------------
// 1. per segment: its state contribution and total decay
// ---------------------------------------------------------------------------
// U = sum over the segment's rows m of (decay from m to the segment's end)
// k_m^T v_m, built chunk by chunk as U <- G_c U + sum_{m in c} w_m k_m^T v_m, with
// w_m the decay from row m to the chunk's end and G_c the chunk's total decay
// (the recurrence itself, in fp32 accumulators). K and V stream through
// kSStages LDS stages in quarters of 64 rows, kSStages - 1 quarters ahead and
// across chunk boundaries; each chunk's gates come in by the load unit with its
// first quarter (every thread one dword, so that all waves count the same
// copies), into one of two buffers by chunk parity.
constexpr int kSStages = 4;

template <int D>
struct SegLds {
  static constexpr int kQ = kGC / 4;                        // rows per quarter
  static constexpr int kQBytes = kQ * D * 2;                // one matrix's quarter
  static constexpr int kStage = 2 * kQBytes;                // K then V
  static constexpr int kGates = kSStages * kStage;          // 2 x kGThreads dwords
  static constexpr int kWgt = kGates + 2 * kGThreads * 4;   // 2 x kGC weights
  static constexpr int kBytes = kWgt + 2 * kGC * 4;
};

template <int D>
__global__ __launch_bounds__(kGThreads, 1) void gret_segstate_kernel(GretParams p) {
  typedef SegLds<D> LY;
  constexpr int kQ = LY::kQ;
  constexpr int LQ = 2 * (kQ * D / 8 / kGThreads);   // tile copies per thread and quarter
  constexpr int kAhead = kSStages - 1;
  __shared__ __attribute__((aligned(16))) char smem_raw[LY::kBytes];
  __shared__ float wsum[4];
  YOCO_LDS char* smem = (YOCO_LDS char*)smem_raw;
  const int h = blockIdx.x % p.heads, g = blockIdx.x / p.heads;
  int b, s;
  if (!locate_segment(p, g, &b, &s)) return;
  const int c0 = s * p.seg_chunks;
  const int left = seq_chunks(p, b) - c0;
  const int nc = left < p.seg_chunks ? left : p.seg_chunks;
  const ChunkInfo first = chunk_info(p, b, c0);
  const int n_last = chunk_info(p, b, c0 + nc - 1).n;
  const int nq = 4 * (nc - 1) + (n_last + kQ - 1) / kQ;    // quarters holding rows
  const int64_t slot = (int64_t)h * p.slots + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5;
  const int H = p.heads;
  const uint32_t base = (uint32_t)(uintptr_t)smem;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
  const __bf16* kg = static_cast<const __bf16*>(p.k);
  const __bf16* vg = static_cast<const __bf16*>(p.v);
  auto issue = [&](int f) {
    const int cf = f >> 2;
    const int64_t row0 = first.row0 + (int64_t)cf * kGC;
    const int n = cf == nc - 1 ? n_last : kGC;
    if ((f & 3) == 0) {
      const int r = (tid & (kGC - 1)) < n ? (tid & (kGC - 1)) : n - 1;
      dma4(p.gamma + (row0 + r) * H + h, base + LY::kGates + (cf & 1) * (kGThreads * 4) + wv * 256);
    }
    const uint32_t st = base + (f % kSStages) * LY::kStage;
    load_tile<D, kTrLayout, true>(kg, row0, n, kQ * (f & 3), kQ, H, h, st, tid);
    load_tile<D, kTrLayout, true>(vg, row0, n, kQ * (f & 3), kQ, H, h, st + LY::kQBytes, tid);
  };
  for (int f = 0; f < kAhead && f < nq; ++f) issue(f);

  const StateBlocks<D> sb(wave);
  constexpr int PER = StateBlocks<D>::PER;
  f32x16 acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = f32x16{};
  float a_seg = 0.f;   // the segment's log2 decay
  for (int f = 0; f < nq; ++f) {
    // quarter f is in when at most the copies of the quarters issued after it
    // (up to kAhead - 1, one of them perhaps a chunk's first) are in flight
    const int later = nq - 1 - f < kAhead - 1 ? nq - 1 - f : kAhead - 1;
    int pending = later * LQ;
    for (int j = 1; j <= later; ++j) pending += ((f + j) & 3) == 0 ? 1 : 0;
    wait_copies<LQ>(pending);
    barrier_only();
    // the next quarter goes out at once: its stage held quarter f - 1, which
    // every wave finished before the barrier above
    if (f + kAhead < nq) issue(f + kAhead);
    const int cf = f >> 2;
    YOCO_LDS float* wgt = (YOCO_LDS float*)(smem + LY::kWgt + (cf & 1) * (kGC * 4));
    if ((f & 3) == 0) {
      // the chunk's decay prefix, its weights and total decay
      const int n = cf == nc - 1 ? n_last : kGC;
      const YOCO_LDS float* gt = (const YOCO_LDS float*)(smem + LY::kGates + (cf & 1) * (kGThreads * 4));
      float a = 0.f;
      if (tid < kGC && tid < n) {
        const float l = __log2f(gt[tid]);
        a = l > kLogGateFloor ? l : kLogGateFloor;
      }
      const float A = chunk_prefix<false>(a, wsum);
      const float a_last = wsum[0] + wsum[1] + wsum[2] + wsum[3];   // rows past the end count gate 1
      if (tid < kGC) wgt[tid] = tid < n ? exp2f(a_last - A) : 0.f;
      const float G = exp2f(a_last);
#pragma unroll
      for (int e = 0; e < PER; ++e) acc[e] *= G;
      a_seg += a_last;
      lds_barrier();   // the weights are in for every wave
    }
    if (!sb.idle) {
      // U += (w ⊙ K)^T V over the quarter in steps of 16 keys, each step's LDS
      // reads issued one step ahead of its MFMAs
      const YOCO_LDS char* kt = smem + (f % kSStages) * LY::kStage;
      const YOCO_LDS char* vt = kt + LY::kQBytes;
      const int key0 = kQ * (f & 3);
      StepOps<PER> op[2];
      op[0].template read<D, kTrLayout>(kt, vt, wgt, key0, 0, sb, lane);
#pragma unroll
      for (int s4 = 0; s4 < kQ / 16; ++s4) {
        if (s4 + 1 < kQ / 16) op[(s4 + 1) & 1].template read<D, kTrLayout>(kt, vt, wgt, key0, 16 * (s4 + 1), sb, lane);
        sched_fence();
        op[s4 & 1].mfma(acc);
        sched_fence();
      }
    }
  }
  if (tid == 0) p.seg_decay[slot] = exp2f(a_seg);
  if (sb.idle) return;
  float* u = p.seg_u + slot * (D * D);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dk = 32 * sb.bi + 8 * (r >> 2) + 4 * hf + (r & 3);
      u[dk * D + 32 * sb.bj(e) + (lane & 31)] = acc[e][r];
    }
  }
}

// ---------------------------------------------------------------------------
// 2. the state recurrence across segments
// ---------------------------------------------------------------------------
// S_{s+1} = G_s S_s + U_s (fp32), writing each segment's incoming state and the
// final state; each thread holds 4 consecutive elements of S [dk][dv].
template <int D>
__global__ __launch_bounds__(256) void gret_segscan_kernel(GretParams p) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int e0 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (e0 >= D * D) return;
  const int64_t g0 = seg_start(p, b);
  int64_t ns = seq_segs(p, b);
  // non-decreasing cu_seqlens keep every segment within the slots; others are clamped to them
  if (g0 + ns > p.slots) ns = g0 < p.slots ? p.slots - g0 : 0;
  const int64_t bh = (int64_t)b * p.heads + h;
  f32x4 st = {0.f, 0.f, 0.f, 0.f};
  if (p.state_in != nullptr) st = *reinterpret_cast<const f32x4*>(p.state_in + bh * (D * D) + e0);
  // the loads do not depend on the state: fetch a group of segments ahead,
  // then run the (serial) recurrence over the group
  constexpr int kAhead = 8;
  const int64_t slot0 = (int64_t)h * p.slots + g0;
  const float* __restrict__ us = p.seg_u + slot0 * (D * D) + e0;
  const float* __restrict__ gs = p.seg_decay + slot0;
  float* __restrict__ sin = p.seg_s + slot0 * (D * D) + e0;
  for (int64_t s0 = 0; s0 < ns; s0 += kAhead) {
    f32x4 u[kAhead];
    float gd[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int64_t s = s0 + i < ns ? s0 + i : ns - 1;
      u[i] = *reinterpret_cast<const f32x4*>(us + s * (D * D));
      gd[i] = gs[s];
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (s0 + i >= ns) break;
      *reinterpret_cast<f32x4*>(sin + (s0 + i) * (D * D)) = st;
#pragma unroll
      for (int j = 0; j < 4; ++j) st[j] = fmaf(gd[i], st[j], u[i][j]);
    }
  }
  if (p.state_out != nullptr) *reinterpret_cast<f32x4*>(p.state_out + bh * (D * D) + e0) = st;
}

// ---------------------------------------------------------------------------
// 3. outputs: one segment per workgroup, its chunks one after the other
// ---------------------------------------------------------------------------
// The workgroup starts from the segment's incoming state (fp32, in its MFMA
// accumulators) and carries it across its chunks: each chunk's state goes into
// LDS as bf16 for the inter-chunk product, and the chunk's own contribution is
// added tile by tile from the K and V tiles already staged for the outputs.
// LDS (head_dim D, T = one stage, a K and a V tile of 64 rows):
//   [0, 2T)         Q^ rows of the chunk, then tiles 1 and 2; during the
//                   chunk's last tile, the next chunk's Q^ rows
//   [2T, 3T)        tile 0
//   [3T, 4T)        S_c^T (bf16, written from the running state), then tile 3
//   [2T, 2T + O)    the outputs, staged for whole-row stores (tiles 0 and 3
//                   done with; past 4T for head_dim 128)
//   then the gates / their prefix A (two buffers, chunk parity: the next
//   chunk's gates come in while this chunk's prefix is in use) and the
//   state-update weights.
// K tiles are in the kd layout (read both ways), V tiles in the transposing one.
template <int D>
struct OutLds {
  static constexpr int kTile = kGT * D * 2;        // one K or V tile
  static constexpr int kStage = 2 * kTile;          // K then V
  static constexpr int kQ = 0;                      // Q^ area (2 stages)
  static constexpr int kS = 3 * kStage;             // state area (stage 3)
  static constexpr int kO = 2 * kStage;             // output staging
  static constexpr int kOStride = D + 8;            // staged output row (elements)
  static constexpr int kOBytes = 8 * 32 * kOStride * 2;
  static constexpr int kEnd = kO + kOBytes > 4 * kStage ? kO + kOBytes : 4 * kStage;
  static constexpr int kA = (kEnd + 15) / 16 * 16;  // gates / prefix, 2 x kGC floats
  static constexpr int kW = kA + 2 * kGC * 4;       // weights
  static constexpr int kBytes = kW + kGC * 4;
  static_assert(kGC * D * 2 == 2 * kStage, "the chunk's Q^ rows fill two stages");
  static_assert(D * D * 2 <= kStage, "the state fits a stage");
};
// tile t's stage: 0 after Q^, 1 and 2 in the Q^ area, 3 in the state area
__device__ __forceinline__ uint32_t out_stage_off(int t, int stage) {
  return (uint32_t)(t == 0 ? 2 * stage : t == 3 ? 3 * stage : (t - 1) * stage);
}

template <int D>
__global__ __launch_bounds__(kGThreads, 1) void gret_out_kernel(GretParams p) {
  typedef OutLds<D> LY;
  constexpr int kTile = LY::kTile;
  constexpr int kStage = LY::kStage;
  constexpr int kOStride = LY::kOStride;
  __shared__ __attribute__((aligned(16))) char smem_raw[LY::kBytes];
  __shared__ float wsum[4];
  YOCO_LDS char* smem = (YOCO_LDS char*)smem_raw;
  YOCO_LDS float* W_lds = (YOCO_LDS float*)(smem + LY::kW);
  const int h = blockIdx.x % p.heads, g = blockIdx.x / p.heads;
  int b, s;
  if (!locate_segment(p, g, &b, &s)) return;
  const int c0 = s * p.seg_chunks;
  const int left = seq_chunks(p, b) - c0;
  const int nc = left < p.seg_chunks ? left : p.seg_chunks;
  const SeqRows sr = seq_range(p, b);   // loaded once: a load in the chunk loop would wait for the copies in flight
  const int64_t slot = (int64_t)h * p.slots + g;
  const bool has_state0 = s > 0 || p.state_in != nullptr;
  const int tid0 = threadIdx.x, wave = tid0 >> 6;
  const int H = p.heads;
  const uint32_t base_lds = (uint32_t)(uintptr_t)smem;
  const __bf16* kg = static_cast<const __bf16*>(p.k);
  const __bf16* vg = static_cast<const __bf16*>(p.v);
  const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
  constexpr int L = 2 * (kGT * D / 8 / kGThreads);   // copies per thread and tile
  constexpr int kQHalf = (kGC / 2) * D / 8 / kGThreads;   // copies per thread of half a chunk's Q^ rows

  // the running state S (fp32): the segment's incoming state, then after each chunk
  const StateBlocks<D> sb(wave);
  constexpr int PER = StateBlocks<D>::PER;
  f32x16 sacc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) sacc[e] = f32x16{};
  if (has_state0 && !sb.idle) {
    const int lane = tid0 & 63, hf = lane >> 5;
    const float* src = p.seg_s + slot * (D * D);
#pragma unroll
    for (int e = 0; e < PER; ++e) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int dk = 32 * sb.bi + 8 * (r >> 2) + 4 * hf + (r & 3);
        sacc[e][r] = src[dk * D + 32 * sb.bj(e) + (lane & 31)];
      }
    }
  }

  for (int cc = 0; cc < nc; ++cc) {
    // the per-lane LDS offsets of the chunk's prologue and epilogue are
    // recomputed per chunk (kept live across the loop they would not fit)
    const int tid = opaque(tid0), lane = tid & 63;
    const int hf = lane >> 5;
    const ChunkInfo ci = chunk_of(sr, c0 + cc);
    const bool has_state = has_state0 || cc > 0;
    const int n_tiles = (ci.n + kGT - 1) / kGT;
    YOCO_LDS float* A_lds = (YOCO_LDS float*)(smem + LY::kA + (cc & 1) * (kGC * 4));
    // the gates and Q^ rows of chunk c (one dword per row; Q^ in the row_slot layout)
    // (in two halves: Q^ rows 0 .. kGC/2 - 1, then the rest and the gates)
    auto issue_q_half = [&](const ChunkInfo& c, int parity, int half) {
      const int tq = opaque(tid0);   // offsets computed here, not kept live across the tile loop
      if (half == 1 && tq < kGC) {
        const int r = tq < c.n ? tq : c.n - 1;
        dma4(p.gamma + (c.row0 + r) * H + h, base_lds + LY::kA + parity * (kGC * 4) + wv * 256);
      }
      load_tile<D, kRowLayout, true>(static_cast<const __bf16*>(p.q), c.row0, c.n, half * (kGC / 2), kGC / 2, H, h,
                                     base_lds + LY::kQ + half * (kGC / 2) * (D * 2), tq);
    };
    auto issue_q = [&](const ChunkInfo& c, int parity) {
      issue_q_half(c, parity, 0);
      issue_q_half(c, parity, 1);
    };
    auto issue = [&](int t) {
      const uint32_t st = base_lds + out_stage_off(t, kStage);
      const int n_t = ci.n - t * kGT < kGT ? ci.n - t * kGT : kGT;
      load_tile<D, kKdLayout>(kg, ci.row0 + t * kGT, n_t, 0, kGT, H, h, st, tid);
      load_tile<D, kPvLayout>(vg, ci.row0 + t * kGT, n_t, 0, kGT, H, h, st + kTile, tid);
    };
    // copy j (of L) of tile t: K's copies first, then V's
    auto issue_one = [&](int t, int j) {
      const uint32_t st = base_lds + out_stage_off(t, kStage);
      const int n_t = ci.n - t * kGT < kGT ? ci.n - t * kGT : kGT;
      if (j < L / 2) load_tile_one<D, kKdLayout>(kg, ci.row0 + t * kGT, n_t, 0, H, h, st, tid, j);
      else load_tile_one<D, kPvLayout>(vg, ci.row0 + t * kGT, n_t, 0, H, h, st + kTile, tid, j - L / 2);
    };
    // S_c^T into the state area as bf16 (row dv, 16-byte chunk dk / 8; each lane
    // 4 consecutive dk of one dv), once the previous chunk's staged outputs are
    // read (they cover this area for head_dim 128)
    lds_barrier();   // every wave has read its staged outputs of the previous chunk
    if (has_state && !sb.idle) {
#pragma unroll
      for (int e = 0; e < PER; ++e) {
        const int dv = 32 * sb.bj(e) + (lane & 31);
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const u32x2 w2 = {pack2(sacc[e][4 * g4 + 0], sacc[e][4 * g4 + 1]),
                            pack2(sacc[e][4 * g4 + 2], sacc[e][4 * g4 + 3])};
          *reinterpret_cast<YOCO_LDS u32x2*>(smem + LY::kS + row_slot<D>(dv, 4 * sb.bi + g4) + 8 * hf) = w2;
        }
      }
    }
    // copies: the gates and Q^ (unless requested during the previous chunk), tile 0
    if (cc == 0) issue_q(ci, 0);
    issue(0);
    wait_vm_lgkm0<L>();   // all but tile 0 (and the state's LDS writes)
    barrier_only();

    // decay prefix A_j (base 2) of the chunk's rows, in place of the gates; the
    // state-update weights 2^(A_last - A_m) and the chunk's total decay
    float a = 0.f;
    if (tid < kGC && tid < ci.n) {
      const float l = __log2f(A_lds[tid]);
      a = l > kLogGateFloor ? l : kLogGateFloor;
    }
    const float A = chunk_prefix<false>(a, wsum);
    const float a_last = wsum[0] + wsum[1] + wsum[2] + wsum[3];
    if (tid < kGC) {
      A_lds[tid] = A;
      W_lds[tid] = tid < ci.n ? exp2f(a_last - A) : 0.f;
    }

    // This wave's query rows: two blocks of 16, lo = chunk rows 16w .. 16w + 15
    // and hi = rows 16(15 - w) .., so that every wave meets the same share of the
    // causal triangle (2.5 of the chunk's 64-key tiles; blocks of 32 rows would
    // meet 1 to 4). Products on 16 x 16 x 32 MFMAs with query row 16 blk + (lane
    // & 15) as the column: Q^T as the B operand, dims 32ks + 8qg .. +7.
    constexpr int KS = D / 32;   // 32-dim steps
    constexpr int NT = D / 16;   // 16-dim output blocks
    const int ql = lane & 15, qg = lane >> 4;
    const int blo = wave, bhi = 15 - wave;
    const int jr0 = 16 * blo + ql, jr1 = 16 * bhi + ql;   // rows within the chunk
    const int jl0 = jr0 < ci.n ? jr0 : ci.n - 1, jl1 = jr1 < ci.n ? jr1 : ci.n - 1;
    bf16x8 qf[2][KS];
    {
      const YOCO_LDS char* qs = smem + LY::kQ;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        qf[0][ks] = *reinterpret_cast<const YOCO_LDS bf16x8*>(qs + row_slot<D>(jl0, 4 * ks + qg));
        qf[1][ks] = *reinterpret_cast<const YOCO_LDS bf16x8*>(qs + row_slot<D>(jl1, 4 * ks + qg));
      }
    }
    lds_barrier();   // Q^ read by every wave (its area takes tiles 1 and 2); A in LDS
    const bool prefetch = cc + 1 < nc;   // then this chunk is whole: four tiles

    // block hi holds rows only if block lo does; a block without rows is still
    // computed beside a block with rows (on clamped rows, never stored)
    const bool lo_rows = 16 * blo < ci.n, hi_rows = 16 * bhi < ci.n;
    const float Aj0 = A_lds[jl0], Aj1 = A_lds[jl1];
    f32x4 acc[2][NT];   // O^T of block b: dims 16t + 4qg + r (register r), query row jr_b
#pragma unroll
    for (int b = 0; b < 2; ++b)
#pragma unroll
      for (int t = 0; t < NT; ++t) acc[b][t] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (has_state && lo_rows) {
      // inter-chunk term: O^T[dv][j] = sum_dk S^T[dv][dk] q_j[dk], then times 2^A_j;
      // steps (ks, t) with the output block t fastest, each state operand serving
      // both query blocks, the state reads kGReadsAhead steps ahead. The copies
      // of tiles 1 and 2 go out one every kEvery steps (issued together, they
      // held every wave at the load unit)
      constexpr int NS = KS * NT;
      constexpr int kEvery = NS / (2 * L);
      static_assert(NS % (2 * L) == 0, "the inter-chunk steps spread the copies of two tiles");
      constexpr int RA = kGReadsAhead;
      const YOCO_LDS char* sl = smem + LY::kS;
      auto read_s = [&](int i) {
        return *reinterpret_cast<const YOCO_LDS bf16x8*>(sl + row_slot<D>(16 * (i % NT) + ql, 4 * (i / NT) + qg));
      };
      bf16x8 sa[NS];
#pragma unroll
      for (int i = 0; i < RA; ++i) sa[i] = read_s(i);
#pragma unroll
      for (int i = 0; i < NS; ++i) {
        if (i + RA < NS) sa[i + RA] = read_s(i + RA);
        acc[0][i % NT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa[i], qf[0][i / NT], acc[0][i % NT], 0, 0, 0);
        acc[1][i % NT] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(sa[i], qf[1][i / NT], acc[1][i % NT], 0, 0, 0);
        sched_fence();
        if (i % kEvery == 0 && 1 + (i / kEvery) / L < n_tiles) issue_one(1 + (i / kEvery) / L, (i / kEvery) % L);
      }
      const float e0 = exp2f(Aj0), e1 = exp2f(Aj1);
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        acc[0][t] *= e0;
        acc[1][t] *= e1;
      }
    } else {
      if (n_tiles > 1) issue(1);
      if (n_tiles > 2) issue(2);
    }
    if (n_tiles > 3) {
      lds_barrier();   // the state is read by every wave: its area takes tile 3
      issue(3);
    }
    // S_{c+1} = G_c S_c + (the chunk's contribution, added tile by tile below)
    const float G = exp2f(a_last);
#pragma unroll
    for (int e = 0; e < PER; ++e) sacc[e] *= G;

    // One key tile against the query blocks in MASK (bit 0: lo, bit 1: hi), the
    // causal mask applied to those in CAUSAL (the others lie wholly below the
    // diagonal)
    auto tile_body = [&](auto mask_c, auto causal_c, const YOCO_LDS char* kt, const YOCO_LDS char* vt, int key0) {
      constexpr int MASK = decltype(mask_c)::value;
      constexpr int CAUSAL = decltype(causal_c)::value;
      constexpr int RA = kGReadsAhead;
      // S^T[m][j] = K Q^T per group kb of 16 keys: steps (ks, kb) with kb fastest,
      // each K operand serving the blocks in MASK, the reads RA steps ahead
      constexpr int NQ = 4 * KS;
      auto read_k = [&](int i) {
        return *reinterpret_cast<const YOCO_LDS bf16x8*>(kt + kd_slot<D>(16 * (i & 3) + ql, 4 * (i >> 2) + qg));
      };
      f32x4 sc[2][4];
#pragma unroll
      for (int b = 0; b < 2; ++b)
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) sc[b][kb] = f32x4{0.f, 0.f, 0.f, 0.f};
      bf16x8 ka[NQ];
#pragma unroll
      for (int i = 0; i < RA; ++i) ka[i] = read_k(i);
#pragma unroll
      for (int i = 0; i < NQ; ++i) {
        if (i + RA < NQ) ka[i + RA] = read_k(i + RA);
        if constexpr ((MASK & 1) != 0)
          sc[0][i & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qf[0][i >> 2], sc[0][i & 3], 0, 0, 0);
        if constexpr ((MASK & 2) != 0)
          sc[1][i & 3] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ka[i], qf[1][i >> 2], sc[1][i & 3], 0, 0, 0);
        sched_fence();
      }
      // O^T += V^T P^T in steps (s, t), t fastest: the A operand is V^T at dims
      // 16t .. 16t + 15 and keys 32s + 4qg + {0..3}, 32s + 16 + 4qg + {0..3}; the
      // first V reads go out before the decay, whose VALU work hides their latency
      constexpr int NV = 2 * NT;
      auto read_v = [&](int j) { return read_pv<D>(vt, 32 * (j / NT), j % NT, lane); };
      bf16x8 va[NV];
#pragma unroll
      for (int j = 0; j < RA; ++j) va[j] = read_v(j);
      sched_fence();
      // P^T = S^T * 2^(A_j - A_m) for m <= j, else 0; register r of group kb is key
      // key0 + 16kb + 4qg + r, so words 0..3 of w[b][s] are the B operand of step s
      uint32_t w[2][2][4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int m0 = key0 + 16 * kb + 4 * qg;
        const f32x4 am = *reinterpret_cast<const YOCO_LDS f32x4*>((const YOCO_LDS char*)A_lds + 4 * m0);
#pragma unroll
        for (int b = 0; b < 2; ++b) {
          if (((MASK >> b) & 1) == 0) continue;
          const float Ajb = b == 0 ? Aj0 : Aj1;
          const int jrb = b == 0 ? jr0 : jr1;
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = __builtin_amdgcn_exp2f(Ajb - am[e]);   // below 2^-126: 0 or denormal, as the product vanishes
            if (((CAUSAL >> b) & 1) != 0) pv[e] = (m0 + e <= jrb) ? sc[b][kb][e] * d : 0.f;
            else pv[e] = sc[b][kb][e] * d;
          }
          w[b][kb >> 1][2 * (kb & 1)] = pack2(pv[0], pv[1]);
          w[b][kb >> 1][2 * (kb & 1) + 1] = pack2(pv[2], pv[3]);
        }
      }
      sched_fence();
#pragma unroll
      for (int j = 0; j < NV; ++j) {
        const int s = j / NT, tt = j % NT;
        if (j + RA < NV) va[j + RA] = read_v(j + RA);
        if constexpr ((MASK & 1) != 0) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w[0][s][0], w[0][s][1], w[0][s][2], w[0][s][3]));
          acc[0][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[j], pb, acc[0][tt], 0, 0, 0);
        }
        if constexpr ((MASK & 2) != 0) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w[1][s][0], w[1][s][1], w[1][s][2], w[1][s][3]));
          acc[1][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[j], pb, acc[1][tt], 0, 0, 0);
        }
        sched_fence();
      }
    };

    // intra-chunk term and state update, tile by tile; tile t is in when at
    // most the copies of the tiles requested after it (n_tiles - 1 - t of them)
    // are in flight
    static_assert(kGC / kGT == 4, "the waits below assume four tiles per chunk");
    for (int t = 0; t < n_tiles; ++t) {
      const int after = n_tiles - 1 - t;
      if (after >= 3) wait_vm_lgkm0<3 * L>();
      else if (after == 2) wait_vm_lgkm0<2 * L>();
      else if (after == 1) wait_vm_lgkm0<L>();
      else if (prefetch) wait_vm_lgkm0<kQHalf>();   // the next chunk's first Q^ rows may stay in flight
      else wait_vm_lgkm0<0>();
      barrier_only();
      // the next chunk's Q^ rows go out as their stages free up: the first half
      // once tile 1 is done with, the rest and the gates once tile 2 is
      if (t == 2 && prefetch) issue_q_half(chunk_of(sr, c0 + cc + 1), (cc + 1) & 1, 0);
      if (t == 3 && prefetch) issue_q_half(chunk_of(sr, c0 + cc + 1), (cc + 1) & 1, 1);
      const int key0 = t * kGT;
      const YOCO_LDS char* ks = smem + out_stage_off(t, kStage);
      const YOCO_LDS char* vs = ks + kTile;
      // the blocks whose rows reach this tile (hi's whenever lo's do; a tile
      // that reaches lo's rows lies wholly below hi's)
      using I0 = std::integral_constant<int, 0>;
      using I1 = std::integral_constant<int, 1>;
      using I2 = std::integral_constant<int, 2>;
      using I3 = std::integral_constant<int, 3>;
      if (lo_rows && key0 <= 16 * blo + 15) {
        if (key0 + kGT - 1 > 16 * blo) tile_body(I3{}, I1{}, ks, vs, key0);
        else tile_body(I3{}, I0{}, ks, vs, key0);
      } else if (hi_rows && key0 <= 16 * bhi + 15) {
        if (key0 + kGT - 1 > 16 * bhi) tile_body(I2{}, I2{}, ks, vs, key0);
        else tile_body(I2{}, I0{}, ks, vs, key0);
      }
      // the state update from this tile: S += (w ⊙ K)^T V over its 64 keys (rows
      // past the chunk's end have weight 0), in steps of 16 keys whose LDS reads
      // are issued one step ahead of their MFMAs
      if (!sb.idle) {
        StepOps<PER> op[2];
        op[0].template read<D, kKdLayout, kPvLayout>(ks, vs, W_lds, key0, 0, sb, lane);
#pragma unroll
        for (int s4 = 0; s4 < kGT / 16; ++s4) {
          if (s4 + 1 < kGT / 16)
            op[(s4 + 1) & 1].template read<D, kKdLayout, kPvLayout>(ks, vs, W_lds, key0, 16 * (s4 + 1), sb, lane);
          sched_fence();
          op[s4 & 1].mfma(sacc);
          sched_fence();
        }
      }
    }
    lds_barrier();   // tiles 0 and 3 are done with: stage the outputs there (the next chunk's copies stay in flight)

    // staged row 16b + ql holds block b's row; then whole rows are stored
    YOCO_LDS __bf16* ot = (YOCO_LDS __bf16*)(smem + LY::kO) + wave * (32 * kOStride);
#pragma unroll
    for (int b = 0; b < 2; ++b) {
#pragma unroll
      for (int t = 0; t < NT; ++t) {
        const u32x2 w2 = {pack2(acc[b][t][0], acc[b][t][1]), pack2(acc[b][t][2], acc[b][t][3])};
        *reinterpret_cast<YOCO_LDS u32x2*>(ot + (16 * b + ql) * kOStride + 16 * t + 4 * qg) = w2;
      }
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    __bf16* obase = static_cast<__bf16*>(p.out);
#pragma unroll
    for (int i = 0; i < 32 * (D / 8) / 64; ++i) {
      const int ci8 = lane + 64 * i;
      const int row = ci8 / (D / 8), c8 = ci8 % (D / 8);
      const int jr = row < 16 ? 16 * blo + row : 16 * bhi + (row - 16);
      if (jr < ci.n)
        __builtin_nontemporal_store(*reinterpret_cast<const YOCO_LDS u32x4*>(ot + row * kOStride + 8 * c8),
                                    reinterpret_cast<u32x4*>(obase + ((ci.row0 + jr) * H + h) * D + 8 * c8));
    }
  }
}

// ---------------------------------------------------------------------------
// decode: one recurrent step, S <- g S + k^T v and o = q S (fp32 state)
// ---------------------------------------------------------------------------
// A workgroup owns 32 state columns (dv) of one (sequence, head): 8 lanes of 4
// columns cover the block's 128 bytes of a state row, and 32 row groups take
// every 32nd dk row from their own. Each thread issues all of its state loads
// before using any, so the step costs about one memory round trip; the row
// groups' partial outputs are added in LDS.
constexpr int kDecCols = 32;                       // state columns per workgroup
constexpr int kDecGroups = 256 / (kDecCols / 4);   // row groups

template <int D>
__global__ __launch_bounds__(256) void gret_decode_kernel(GretParams p) {
  constexpr int kRows = D / kDecGroups;            // dk rows per thread
  __shared__ f32x4 part[kDecGroups][kDecCols / 4];
  const int cb = blockIdx.x % (D / kDecCols);
  const int h = blockIdx.x / (D / kDecCols), b = blockIdx.y;
  const int64_t bh = (int64_t)b * p.heads + h;
  const int tid = threadIdx.x;
  const int c4 = tid & 7, grp = tid >> 3;
  const int col = cb * kDecCols + 4 * c4;
  const __bf16* q = static_cast<const __bf16*>(p.q) + bh * D;
  const __bf16* k = static_cast<const __bf16*>(p.k) + bh * D;
  const __bf16* v = static_cast<const __bf16*>(p.v) + bh * D;
  float* st = p.state_out + bh * D * D + col;
  f32x4 s[kRows];
  float qi[kRows], ki[kRows];
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
    const int i = grp + kDecGroups * r;
    s[r] = *reinterpret_cast<const f32x4*>(st + (int64_t)i * D);
    qi[r] = (float)q[i];
    ki[r] = (float)k[i];
  }
  const float g = p.gamma[bh];
  float vv[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) vv[e] = (float)v[col + e];
  f32x4 o = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int r = 0; r < kRows; ++r) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      s[r][e] = fmaf(g, s[r][e], ki[r] * vv[e]);
      o[e] = fmaf(qi[r], s[r][e], o[e]);
    }
    *reinterpret_cast<f32x4*>(st + (int64_t)(grp + kDecGroups * r) * D) = s[r];
  }
  part[grp][c4] = o;
  __syncthreads();
  if (tid < kDecCols) {
    float sum = 0.f;
#pragma unroll 8
    for (int g2 = 0; g2 < kDecGroups; ++g2) sum += part[g2][tid >> 2][tid & 3];
    static_cast<__bf16*>(p.out)[bh * D + cb * kDecCols + tid] = (__bf16)sum;
  }
}

}  // namespace

hipError_t launch_gret_prefill(const GretParams& p, int head_dim, hipStream_t stream) {
  // one workgroup per (segment slot, head), heads fastest: the slots past the
  // last segment come last in dispatch order, so that they never take a place
  // that a real segment waits for (within an XCD, workgroups are dealt to the
  // shader engines in turn)
  const dim3 grid_c((unsigned)p.slots * (unsigned)p.heads);
  const dim3 grid_s((head_dim * head_dim / 4 + 255) / 256, p.heads, p.batch);
  if (head_dim == 64) {
    hipLaunchKernelGGL(gret_segstate_kernel<64>, grid_c, dim3(kGThreads), 0, stream, p);
    hipLaunchKernelGGL(gret_segscan_kernel<64>, grid_s, dim3(256), 0, stream, p);
    hipLaunchKernelGGL(gret_out_kernel<64>, grid_c, dim3(kGThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(gret_segstate_kernel<128>, grid_c, dim3(kGThreads), 0, stream, p);
    hipLaunchKernelGGL(gret_segscan_kernel<128>, grid_s, dim3(256), 0, stream, p);
    hipLaunchKernelGGL(gret_out_kernel<128>, grid_c, dim3(kGThreads), 0, stream, p);
  }
  return hipGetLastError();
}

hipError_t launch_gret_decode(const GretParams& p, int head_dim, hipStream_t stream) {
  const dim3 grid((unsigned)(p.heads * (head_dim / kDecCols)), (unsigned)p.batch);
  if (head_dim == 64)
    hipLaunchKernelGGL(gret_decode_kernel<64>, grid, dim3(256), 0, stream, p);
  else
    hipLaunchKernelGGL(gret_decode_kernel<128>, grid, dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace yoco
