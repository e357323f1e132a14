// Gated retention (gRet), the Self-Decoder's default attention ("YOCO 深度技术分析",
// liuhc.cn, section 2.2: the parallel form (Q K^T ⊙ D) V with the data-controlled
// decay D[n][m] = γ_{m+1} ... γ_n, the recurrent form S_n = γ_n S_{n-1} + K_n^T V_n,
// o_n = Q_n S_n, and the chunkwise form; section 5.3.2: chunks of 256 rows).
//
// Prefill runs the chunkwise form in three launches, so that every (sequence,
// head, chunk) works in parallel and only the cheap state recurrence is serial
// (the chunks of all sequences are numbered one after the other and located on
// the device, so every row is computed whatever the lengths):
//   1. gret_state_kernel: per chunk, U = sum_m w_m k_m^T v_m with w_m the decay
//      from row m to the chunk's end, and the chunk's total decay G
//      (MFMA: U^T = V^T diag(w) K, both operands by transposing LDS reads);
//   2. gret_scan_kernel: S_{c+1} = G_c S_c + U_c over the chunks (fp32), writing
//      each chunk's incoming state S_c (bf16, for the MFMA of step 3) and the
//      final state;
//   3. gret_out_kernel: o_j = e_j q_j S_c + sum_{m <= j} (e_j / e_m) (q_j . k_m) v_m
//      with e_j the decay from the chunk's start to row j: the first term is one
//      MFMA product with the staged S_c, the second the intra-chunk parallel
//      form, tiled like attention (S^T = K Q^T, decay and causal mask on the
//      accumulator registers, O^T += V^T P^T) but without a softmax.
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

// Transposing read: 8 bf16 of one column (dim 32t + lane col) at rows
// base + 4h + {0..3} and base + 8 + 4h + {0..3} of a tr_slot tile.
template <int D>
__device__ __forceinline__ bf16x8 read_tr(const YOCO_LDS char* tile, int base_row, int t, int lane) {
  const int i = lane & 15, g = lane >> 4, h = lane >> 5;
  const int q = i >> 2, w = i & 3;
  const int r = base_row + 4 * h + q;
  const int chunk = 4 * t + 2 * (g & 1) + (w >> 1);
  const YOCO_LDS char* p = tile + tr_slot<D>(r, chunk) + 8 * (w & 1);
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(p));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((YOCO_LDS s16x4*)(p + 8 * (D * 2)));
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Copy tile rows [first, first + rows) of a [rows, H, D] bf16 tensor (row
// stride H*D) whose row 0 is global row `row0` (rows >= n_rows, n_rows >= 1,
// repeat row n_rows - 1) into LDS at `lds` (tile row `first` at offset 0), in
// the tr_slot (TR) or row_slot layout, by the load unit. rows * D / 8 must be a
// multiple of the thread count.
template <int D, bool TR>
__device__ __forceinline__ void load_tile(const __bf16* src, int64_t row0, int n_rows, int first, int rows, int H,
                                          int h, uint32_t lds) {
  constexpr int cpr = D / 8;
  const uint32_t wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  for (int i = 0; i < rows * cpr / kGThreads; ++i) {
    const int p = i * kGThreads + (int)threadIdx.x;
    const int r = first + p / cpr, slot = p % cpr;
    const int c = TR ? (slot ^ v_swizzle<D>(r)) : (slot ^ (r & (cpr - 1)));
    const int rr = r < n_rows ? r : n_rows - 1;
    dma16(src + ((row0 + rr) * H + h) * D + 8 * c, lds + (i * kGThreads + wave * 64) * 16);
  }
}

struct ChunkInfo {
  int64_t row0;   // first global row of the chunk
  int n;          // rows of the chunk (0: no chunk)
};

// Rows of sequence b (clamped to the packed rows) and its chunks.
__device__ __forceinline__ int64_t seq_rows(const GretParams& p, int b) {
  int64_t r0 = p.cu_seqlens[b], r1 = p.cu_seqlens[b + 1];
  if (r1 > p.total_rows) r1 = p.total_rows;
  return (r0 >= 0 && r1 > r0) ? r1 - r0 : 0;
}
__device__ __forceinline__ int seq_chunks(const GretParams& p, int b) {
  return (int)((seq_rows(p, b) + kGC - 1) / kGC);
}

// The chunks of all sequences are numbered one after the other (sequence 0's
// first), so a grid over the workspace's slots covers every row whatever the
// lengths. Global chunk g -> (sequence b, its chunk c), counted by the whole
// wave (64 sequences per step: chunk counts, a DPP prefix sum, a ballot for the
// first sequence whose prefix passes g). All 64 lanes must be active. False if
// g is past the last chunk.
__device__ __forceinline__ bool locate_chunk(const GretParams& p, int g, int* b_out, int* c_out) {
  const int lane = threadIdx.x & 63;
  int before = 0;   // chunks of the sequences before this group of 64
  for (int b0 = 0; b0 < p.batch; b0 += 64) {
    const int bb = b0 + lane;
    const int n = bb < p.batch ? seq_chunks(p, bb) : 0;
    const int incl = wave_incl_scan_i32(n);
    const int total = __builtin_amdgcn_readlane(incl, 63);
    if (g < before + total) {
      const uint64_t m = __builtin_amdgcn_ballot_w64(before + incl > g);
      const int l = __builtin_ctzll(m);
      *b_out = b0 + l;
      *c_out = g - before - (__builtin_amdgcn_readlane(incl, l) - __builtin_amdgcn_readlane(n, l));
      return true;
    }
    before += total;
  }
  return false;
}

// First global chunk of sequence b (scalar loop over the sequences before it).
__device__ __forceinline__ int64_t chunk_start(const GretParams& p, int b) {
  int64_t g = 0;
  for (int i = 0; i < b; ++i) g += seq_chunks(p, i);
  return g;
}

__device__ __forceinline__ ChunkInfo chunk_info(const GretParams& p, int b, int c) {
  int64_t r0 = p.cu_seqlens[b], r1 = p.cu_seqlens[b + 1];
  if (r1 > p.total_rows) r1 = p.total_rows;
  ChunkInfo ci{r0 + (int64_t)c * kGC, 0};
  if (r0 < 0 || r1 <= r0) return ci;
  const int64_t left = r1 - ci.row0;
  ci.n = left <= 0 ? 0 : (left < kGC ? (int)left : kGC);
  return ci;
}

// ---------------------------------------------------------------------------
// 1. per-chunk state contribution U^T[dv][dk] and total decay
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(kGThreads, 2) void gret_state_kernel(GretParams p) {
  constexpr int kQ = kGC / 4;                        // rows per quarter
  constexpr int kQBytes = kQ * D * 2;                // one matrix's quarter
  __shared__ __attribute__((aligned(16))) char smem_raw[2 * 2 * kQBytes];   // 2 stages x (K, V)
  __shared__ __attribute__((aligned(16))) float wgt[kGC];
  __shared__ float wsum[4];
  YOCO_LDS char* smem = (YOCO_LDS char*)smem_raw;
  const int g = blockIdx.x, h = blockIdx.y;
  int b, c;
  if (!locate_chunk(p, g, &b, &c)) return;
  const ChunkInfo ci = chunk_info(p, b, c);
  if (ci.n == 0) return;
  const int64_t slot = (int64_t)h * p.slots + g;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  // decay from row m to the chunk's end: 2^(A_last - A_m), A = prefix of log2 gates
  const float a = log2_gate(p.gamma, ci.row0 + tid, h, p.heads, tid < ci.n);
  const float A = chunk_prefix(a, wsum);
  const float a_last = wsum[0] + wsum[1] + wsum[2] + wsum[3];   // gates past the end count 1
  if (tid < kGC) wgt[tid] = tid < ci.n ? exp2f(a_last - A) : 0.f;
  if (tid == 0) p.chunk_decay[slot] = exp2f(a_last);
  wait_vm_lgkm0<0>();   // the gates are in: from here on only the tile copies are in flight

  // K and V of the chunk in quarters of 64 rows through two stages (64 KB of LDS,
  // so two workgroups share a CU and one's copies overlap the other's MFMAs)
  const uint32_t base = (uint32_t)(uintptr_t)smem;
  constexpr int LQ = 2 * (kQ * D / 8 / kGThreads);   // copies per thread and quarter
  const __bf16* kg = static_cast<const __bf16*>(p.k);
  const __bf16* vg = static_cast<const __bf16*>(p.v);
  auto issue = [&](int f) {
    const uint32_t st = base + (f & 1) * 2 * kQBytes;
    load_tile<D, true>(kg, ci.row0, ci.n, kQ * f, kQ, p.heads, h, st);
    load_tile<D, true>(vg, ci.row0, ci.n, kQ * f, kQ, p.heads, h, st + kQBytes);
  };
  const int n_q = (ci.n + kQ - 1) / kQ;              // quarters holding rows
  issue(0);
  if (n_q > 1) issue(1);

  // output blocks (dv block i, dk block j) of 32 x 32; D = 128: 16 blocks, two per
  // wave (same i); D = 64: 4 blocks, waves 0..3
  constexpr int NB = D / 32;
  constexpr int PER = (NB * NB) / 8 > 0 ? (NB * NB) / 8 : 1;
  const bool idle = wave * PER >= NB * NB;     // D = 64: waves 4..7 only join the barriers
  const int blk0 = idle ? 0 : wave * PER;
  const int bi = blk0 / NB;
  f32x16 acc[PER];
#pragma unroll
  for (int e = 0; e < PER; ++e) acc[e] = f32x16{};
  const int hf = lane >> 5;
  for (int f = 0; f < n_q; ++f) {
    // quarter f is in when at most the next one's copies are in flight
    if (f + 1 < n_q) wait_vm_lgkm0<LQ>(); else wait_vm_lgkm0<0>();
    barrier_only();
    const YOCO_LDS char* kt = smem + (f & 1) * 2 * kQBytes;
    const YOCO_LDS char* vt = kt + kQBytes;
    if (!idle) {
#pragma unroll
      for (int s4 = 0; s4 < kQ / 16; ++s4) {
        // keys 16 s + {0..3, 8..11} + 4h of the chunk, s = 4f + s4 (two 4-key runs per lane)
        const int base_q = 16 * s4;               // row within the quarter
        const int key = kQ * f + base_q;          // row within the chunk
        const bf16x8 av = read_tr<D>(vt, base_q, bi, lane);            // V^T rows dv, 8 keys
        const f32x4 w0 = *reinterpret_cast<const YOCO_LDS f32x4*>((const YOCO_LDS char*)wgt + 4 * (key + 4 * hf));
        const f32x4 w1 = *reinterpret_cast<const YOCO_LDS f32x4*>((const YOCO_LDS char*)wgt + 4 * (key + 8 + 4 * hf));
#pragma unroll
        for (int e = 0; e < PER; ++e) {
          const int bj = (blk0 + e) % NB;
          const bf16x8 kb = read_tr<D>(kt, base_q, bj, lane);          // K columns dk, same 8 keys
          uint32_t wv[4];
#pragma unroll
          for (int z = 0; z < 2; ++z) {
            const f32x4 ww = z == 0 ? w0 : w1;
            wv[2 * z] = pack2((float)kb[4 * z + 0] * ww[0], (float)kb[4 * z + 1] * ww[1]);
            wv[2 * z + 1] = pack2((float)kb[4 * z + 2] * ww[2], (float)kb[4 * z + 3] * ww[3]);
          }
          const bf16x8 kw = __builtin_bit_cast(bf16x8, make_uint4(wv[0], wv[1], wv[2], wv[3]));
          acc[e] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, kw, acc[e], 0, 0, 0);
        }
      }
    }
    if (f + 2 < n_q) {
      barrier_only();   // every wave is done with stage f & 1
      issue(f + 2);
    }
  }
  if (idle) return;
  // lane holds dk = 32 bj + lane % 32, dv rows 32 bi + 8(r/4) + 4hf + r%4; stored
  // as bf16 (the scan adds it to an fp32 state): half the bytes of fp32 for the
  // store here and the scan's read, for one more rounding of the contribution
  __bf16* u = reinterpret_cast<__bf16*>(p.chunk_state) + slot * (D * D);
#pragma unroll
  for (int e = 0; e < PER; ++e) {
    const int bj = (blk0 + e) % NB;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int dv = 32 * bi + 8 * (r >> 2) + 4 * hf + (r & 3);
      u[dv * D + 32 * bj + (lane & 31)] = (__bf16)acc[e][r];
    }
  }
}

// ---------------------------------------------------------------------------
// 2. the state recurrence across chunks
// ---------------------------------------------------------------------------
template <int D>
__global__ __launch_bounds__(256) void gret_scan_kernel(GretParams p) {
  const int h = blockIdx.y, b = blockIdx.z;
  const int e0 = (blockIdx.x * 256 + threadIdx.x) * 4;   // element (dv, dk..dk+3) of S^T
  if (e0 >= D * D) return;
  const int dv = e0 / D, dk = e0 % D;
  const int64_t g0 = chunk_start(p, b);
  int64_t nc = seq_chunks(p, b);
  // non-decreasing cu_seqlens keep every chunk within the slots; others are clamped to them
  if (g0 + nc > p.slots) nc = g0 < p.slots ? p.slots - g0 : 0;
  const int64_t bh = (int64_t)b * p.heads + h;
  float s[4] = {0.f, 0.f, 0.f, 0.f};
  if (p.state_in != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) s[i] = p.state_in[(bh * D + dk + i) * D + dv];
  }
  // the loads do not depend on the state: fetch a group of chunks ahead, then
  // run the (serial) recurrence over the group
  constexpr int kAhead = 8;
  const int64_t slot0 = (int64_t)h * p.slots + g0;
  const uint16_t* __restrict__ us = p.chunk_state + slot0 * (D * D) + e0;
  const float* __restrict__ gs = p.chunk_decay + slot0;
  uint16_t* __restrict__ sin = p.chunk_in + slot0 * (D * D) + e0;
  for (int c0 = 0; c0 < nc; c0 += kAhead) {
    u32x2 u[kAhead];   // four bf16 contributions
    float g[kAhead];
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      const int c = c0 + i < nc ? c0 + i : nc - 1;
      u[i] = *reinterpret_cast<const u32x2*>(us + (int64_t)c * (D * D));
      g[i] = gs[c];
    }
#pragma unroll
    for (int i = 0; i < kAhead; ++i) {
      if (c0 + i >= nc) break;
      *reinterpret_cast<u32x2*>(sin + (int64_t)(c0 + i) * (D * D)) = u32x2{pack2(s[0], s[1]), pack2(s[2], s[3])};
      const float uf[4] = {bf16_lo(u[i][0]), bf16_hi(u[i][0]), bf16_lo(u[i][1]), bf16_hi(u[i][1])};
#pragma unroll
      for (int j = 0; j < 4; ++j) s[j] = fmaf(g[i], s[j], uf[j]);
    }
  }
  if (p.state_out != nullptr) {
#pragma unroll
    for (int i = 0; i < 4; ++i) p.state_out[(bh * D + dk + i) * D + dv] = s[i];
  }
}

// ---------------------------------------------------------------------------
// 3. outputs of one chunk
// ---------------------------------------------------------------------------
// LDS of the output kernel (head_dim D): every K/V tile of the chunk has its
// own stage, Q^ and the incoming state come in by the load unit too and their
// space is handed to tiles 1, 2 (Q^) and 3 (state) once read:
//   [0, T)          tile 0
//   [T, 3T)         Q^ rows of the chunk, then tiles 1 and 2
//   [3T, 4T)        S_c^T, then tile 3
//   [4T, 4T + 1 KB) the gates, then their prefix A
template <int D>
struct OutLds {
  static constexpr int kTile = kGT * D * 2;        // one K or V tile
  static constexpr int kStage = 2 * kTile;          // K then V
  static constexpr int kQ = kStage;                 // Q^ area (2 stages)
  static constexpr int kS = 3 * kStage;             // state area (stage 3)
  static constexpr int kA = 4 * kStage;             // gates / prefix
  static constexpr int kBytes = kA + kGC * 4;
  static_assert(kGC * D * 2 == 2 * kStage, "the chunk's Q^ rows fill two stages");
  static_assert(D * D * 2 <= kStage, "the state fits a stage");
};
__device__ __forceinline__ uint32_t out_stage_off(int t, int stage) {
  return (uint32_t)(t == 0 ? 0 : t * stage);   // tiles 1, 2 in the Q^ area, 3 in the state area
}

template <int D>
__global__ __launch_bounds__(kGThreads, 1) void gret_out_kernel(GretParams p) {
  typedef OutLds<D> LY;
  constexpr int kTile = LY::kTile;
  constexpr int kStage = LY::kStage;
  constexpr int kOStride = D + 8;
  static_assert(8 * 32 * kOStride * 2 <= LY::kS, "output staging fits tiles 0..2");
  __shared__ __attribute__((aligned(16))) char smem_raw[LY::kBytes];
  __shared__ float wsum[4];
  YOCO_LDS char* smem = (YOCO_LDS char*)smem_raw;
  YOCO_LDS float* A_lds = (YOCO_LDS float*)(smem + LY::kA);
  const int g = blockIdx.x, h = blockIdx.y;
  int b, c;
  if (!locate_chunk(p, g, &b, &c)) return;
  const ChunkInfo ci = chunk_info(p, b, c);
  if (ci.n == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qj = lane & 31, hf = lane >> 5;
  const int H = p.heads;
  const uint32_t base_lds = (uint32_t)(uintptr_t)smem;
  const int n_tiles = (ci.n + kGT - 1) / kGT;
  const __bf16* kg = static_cast<const __bf16*>(p.k);
  const __bf16* vg = static_cast<const __bf16*>(p.v);
  const bool has_state = c > 0 || p.state_in != nullptr;
  const uint32_t wv = __builtin_amdgcn_readfirstlane(wave);
  auto issue = [&](int t) {
    const uint32_t st = base_lds + out_stage_off(t, kStage);
    const int n_t = ci.n - t * kGT < kGT ? ci.n - t * kGT : kGT;
    load_tile<D, false>(kg, ci.row0 + t * kGT, n_t, 0, kGT, H, h, st);
    load_tile<D, true>(vg, ci.row0 + t * kGT, n_t, 0, kGT, H, h, st + kTile);
  };

  // copies, in this order: the gates (one dword per row), the incoming state
  // (bf16 [dv][dk] in the workspace), Q^ (row_slot layout), tile 0
  if (tid < kGC) {
    const int r = tid < ci.n ? tid : ci.n - 1;
    dma4(p.gamma + (ci.row0 + r) * H + h, base_lds + LY::kA + wv * 256);
  }
  if (has_state) {
    constexpr int cpr = D / 8;
    const __bf16* sg = reinterpret_cast<const __bf16*>(p.chunk_in) + ((int64_t)h * p.slots + g) * (D * D);
    for (int i = 0; i < D * cpr / kGThreads; ++i) {
      const int q = i * kGThreads + tid;
      const int r = q / cpr, slot = q % cpr;
      dma16(sg + r * D + 8 * (slot ^ (r & (cpr - 1))), base_lds + LY::kS + (i * kGThreads + wv * 64) * 16);
    }
  }
  load_tile<D, false>(static_cast<const __bf16*>(p.q), ci.row0, ci.n, 0, kGC, H, h, base_lds + LY::kQ);
  issue(0);
  constexpr int L = 2 * (kGT * D / 8 / kGThreads);   // copies per thread and tile
  wait_vm_lgkm0<L>();   // all but tile 0
  barrier_only();

  // decay prefix A_j (base 2) of the chunk's rows, in place of the gates
  float a = 0.f;
  if (tid < kGC && tid < ci.n) {
    const float l = __log2f(A_lds[tid]);
    a = l > kLogGateFloor ? l : kLogGateFloor;
  }
  const float A = chunk_prefix<false>(a, wsum);
  if (tid < kGC) A_lds[tid] = A;

  // Q^T as the B operand: query row qj of this wave, dims 16kk + 8hf .. +7
  const int j_row = 32 * wave + qj;                         // row within the chunk
  const int j_load = j_row < ci.n ? j_row : ci.n - 1;
  bf16x8 qf[D / 16];
  {
    const YOCO_LDS char* qs = smem + LY::kQ;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qf[kk] = *reinterpret_cast<const YOCO_LDS bf16x8*>(qs + row_slot<D>(j_load, 2 * kk + hf));
  }
  lds_barrier();   // Q^ read by every wave (its area takes tiles 1 and 2); A in LDS
  if (n_tiles > 1) issue(1);
  if (n_tiles > 2) issue(2);

  const bool wave_active = 32 * wave < ci.n;
  const float Aj = A_lds[j_load];
  f32x16 acc[D / 32];
#pragma unroll
  for (int t = 0; t < D / 32; ++t) acc[t] = f32x16{};
  if (has_state && wave_active) {
    // inter-chunk term: O^T[dv][j] = sum_dk S^T[dv][dk] q_j[dk], then times 2^A_j
    const YOCO_LDS char* sl = smem + LY::kS;
#pragma unroll
    for (int t = 0; t < D / 32; ++t) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 sa = *reinterpret_cast<const YOCO_LDS bf16x8*>(sl + row_slot<D>(32 * t + qj, 2 * kk + hf));
        acc[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(sa, qf[kk], acc[t], 0, 0, 0);
      }
    }
    const float e = exp2f(Aj);
#pragma unroll
    for (int t = 0; t < D / 32; ++t) acc[t] *= e;
  }
  if (n_tiles > 3) {
    lds_barrier();   // the state is read by every wave: its area takes tile 3
    issue(3);
  }

  // intra-chunk term, tile by tile; tile t is in when at most the copies of
  // the tiles requested after it (n_tiles - 1 - t of them) are in flight
  static_assert(kGC / kGT == 4, "the waits below assume four tiles per chunk");
  for (int t = 0; t < n_tiles; ++t) {
    const int after = n_tiles - 1 - t;
    if (after >= 3) wait_vm_lgkm0<3 * L>();
    else if (after == 2) wait_vm_lgkm0<2 * L>();
    else if (after == 1) wait_vm_lgkm0<L>();
    else wait_vm_lgkm0<0>();
    barrier_only();
    const int key0 = t * kGT;
    if (wave_active && key0 <= j_row) {
      const YOCO_LDS char* ks = smem + out_stage_off(t, kStage);
      const YOCO_LDS char* vs = ks + kTile;
      // S^T[m][j] = K Q^T: two 32-key chains
      f32x16 s[2] = {f32x16{}, f32x16{}};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) {
          const bf16x8 ka = *reinterpret_cast<const YOCO_LDS bf16x8*>(ks + row_slot<D>(32 * kb + qj, 2 * kk + hf));
          s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qf[kk], s[kb], 0, 0, 0);
        }
      }
      // P^T = S^T * 2^(A_j - A_m) for m <= j, else 0; register r of chain kb is
      // key key0 + 32kb + 8(r/4) + 4hf + r%4
      uint32_t w[2][2][4];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int m0 = key0 + 32 * kb + 8 * g4 + 4 * hf;
          const f32x4 am = *reinterpret_cast<const YOCO_LDS f32x4*>((const YOCO_LDS char*)A_lds + 4 * m0);
          float pv[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float d = __builtin_amdgcn_exp2f(Aj - am[e]);   // below 2^-126: 0 or denormal, as the product vanishes
            pv[e] = (m0 + e <= j_row) ? s[kb][4 * g4 + e] * d : 0.f;
          }
          w[kb][g4 >> 1][2 * (g4 & 1)] = pack2(pv[0], pv[1]);
          w[kb][g4 >> 1][2 * (g4 & 1) + 1] = pack2(pv[2], pv[3]);
        }
      }
      // O^T += V^T P^T: B operand of step (kb, cc) = registers 8cc .. 8cc + 7 of chain kb
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int cc = 0; cc < 2; ++cc) {
          const bf16x8 pb = __builtin_bit_cast(bf16x8, make_uint4(w[kb][cc][0], w[kb][cc][1], w[kb][cc][2],
                                                                  w[kb][cc][3]));
#pragma unroll
          for (int tt = 0; tt < D / 32; ++tt) {
            const bf16x8 va = read_tr<D>(vs, 32 * kb + 16 * cc, tt, lane);
            acc[tt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, pb, acc[tt], 0, 0, 0);
          }
        }
      }
    }
  }
  wait_vm_lgkm0<0>();
  __syncthreads();   // the tiles are done with: stage the outputs in LDS

  YOCO_LDS __bf16* ot = (YOCO_LDS __bf16*)smem + wave * (32 * kOStride);
#pragma unroll
  for (int t = 0; t < D / 32; ++t) {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const u32x2 wv = {pack2(acc[t][4 * g4 + 0], acc[t][4 * g4 + 1]), pack2(acc[t][4 * g4 + 2], acc[t][4 * g4 + 3])};
      *reinterpret_cast<YOCO_LDS u32x2*>(ot + qj * kOStride + 32 * t + 8 * g4 + 4 * hf) = wv;
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
    const int jr = 32 * wave + row;
    if (jr < ci.n)
      *reinterpret_cast<u32x4*>(obase + ((ci.row0 + jr) * H + h) * D + 8 * c8) =
          *reinterpret_cast<const YOCO_LDS u32x4*>(ot + row * kOStride + 8 * c8);
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
  const dim3 grid_c(p.slots, p.heads);
  const dim3 grid_s((head_dim * head_dim / 4 + 255) / 256, p.heads, p.batch);
  if (head_dim == 64) {
    hipLaunchKernelGGL(gret_state_kernel<64>, grid_c, dim3(kGThreads), 0, stream, p);
    hipLaunchKernelGGL(gret_scan_kernel<64>, grid_s, dim3(256), 0, stream, p);
    hipLaunchKernelGGL(gret_out_kernel<64>, grid_c, dim3(kGThreads), 0, stream, p);
  } else {
    hipLaunchKernelGGL(gret_state_kernel<128>, grid_c, dim3(kGThreads), 0, stream, p);
    hipLaunchKernelGGL(gret_scan_kernel<128>, grid_s, dim3(256), 0, stream, p);
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
