// The shared cache's producer: K^ = RMSNorm(X) W_K, V^ = RMSNorm(X) W_V for the
// rows of the last Self-Decoder output, written straight into each sequence's
// rows of the shared cache (page "YOCO", section "架构总览", the K^, V^
// equations; LN is RMSNorm: xingfushuangcheng.com explainer of YOCO, section
// "自解码器"). Optionally the YOCO++ residual with the bottom layer's rows,
// K' = lambda (a1 K_1 + a2 K^), is formed in the same epilogue, so the cache holds
// the combined rows and decode reads no more than YOCO (gist.science explainer
// of YOCO++, sections 2.1 and 2.2).
//
// One GEMM on v_mfma_f32_32x32x16_bf16: C[t][n] = X[t][:] . W'[n][:], with
// W' = (gamma * [W_K | W_V])^T packed once (kv_pack_kernel): the gain is
// folded into the weights, and since RMSNorm's 1/rms is a per-row scalar the
// GEMM runs on the raw rows and the epilogue multiplies by it. The row sums of
// squares come from the A operands already in registers (v_dot2_f32_bf16).
//
// Workgroup: 8 waves, a 256 (rows) x 128 (columns) tile, each wave 64 x 64
// (2 x 2 MFMA blocks). X and W' tiles of 64 k stream HBM -> LDS by the load
// unit through 3 stages, 16-byte chunks XOR-swizzled by the row (conflict-free
// A/B reads). A sequence whose rows do not all fit its capacity is skipped
// (kv_commit_kernel raises the flag; it also advances seq_len afterwards).
#include <hip/hip_bf16.h>

#include "internal.h"
#include "lds_copy.h"
#include "tile_common.h"

namespace yoco {

namespace {

constexpr int kPM = 256;           // rows per workgroup tile
constexpr int kPN = 128;           // columns per workgroup tile
constexpr int kPK = 64;            // k per stage
constexpr int kPStages = 3;
constexpr int kPThreads = 512;
constexpr int kXBytes = kPM * kPK * 2;     // 32 KB
constexpr int kWBytes = kPN * kPK * 2;     // 16 KB
constexpr int kPStage = kXBytes + kWBytes;
constexpr int kXLoads = kPM * kPK / 8 / kPThreads;   // 16-byte chunks per thread and stage
constexpr int kWLoads = kPN * kPK / 8 / kPThreads;
static_assert(kXLoads == 4 && kWLoads == 2, "tile split");

// byte offset of 16-byte chunk c of tile row r (64 k = 8 chunks per row)
__device__ __forceinline__ uint32_t swz(int r, int c) { return (uint32_t)(r * 128 + 16 * (c ^ (r & 7))); }

__global__ __launch_bounds__(kPThreads, 1) void kv_project_kernel(ProjectParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kPStages * kPStage];
  __shared__ int64_t prow[kPM];     // pool row of each tile row, -1: not written
  __shared__ float ss_part[2][kPM]; // sums of squares of each row, two halves of k
  __shared__ float inv_rms[kPM];
  YOCO_LDS char* smem = (YOCO_LDS char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wm = wave >> 1;          // 0..3: rows wm*64 ..
  const int wn = wave & 1;           // 0..1: columns wn*64 ..
  // XCD-aware raster: workgroup i runs on XCD i % 8; each XCD takes a
  // contiguous range of tiles in row-block-major order, so the resident
  // workgroups of an XCD share their X row blocks in its L2
  const int n_tiles = p.n_cols / kPN;
  const int grid = (int)gridDim.x;
  const int xcd = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
  const int tile = xcd * (grid / kXcds) + min(xcd, grid % kXcds) + j;
  const int nt = tile % n_tiles;
  const int mt = tile / n_tiles;
  const int64_t m0 = (int64_t)mt * kPM;
  const int n0 = nt * kPN;

  // where each tile row goes: sequence b by binary search over cu_seqlens
  if (tid < kPM) {
    const int64_t t = m0 + tid;
    int64_t dst = -1;
    if (t < p.total_rows) {
      int lo = 0, hi = p.batch;       // find b with cu[b] <= t < cu[b + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int64_t c0 = p.cu_seqlens[b], c1 = p.cu_seqlens[b + 1];
      const int64_t len = p.seq_len[b], cap = p.seq_cap[b], start = p.seq_start[b];
      const bool fits = t >= c0 && t < c1 && c1 <= p.total_rows && len >= 0 && start >= 0 &&
                        len + (c1 - c0) <= cap && start + len + (c1 - c0) <= p.pool_rows;
      if (fits) dst = start + len + (t - c0);
    }
    prow[tid] = dst;
  }

  // this thread's chunks: X chunk q = i * threads + tid -> row q / 8, chunk q % 8
  uint32_t xoff[kXLoads], xdst[kXLoads], woff[kWLoads], wdst[kWLoads];
  const uint32_t wave_lds = (uint32_t)(uintptr_t)smem + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 64 * 16;
#pragma unroll
  for (int i = 0; i < kXLoads; ++i) {
    const int q = i * kPThreads + tid;
    int64_t row = m0 + q / 8;
    if (row >= p.total_rows) row = p.total_rows - 1;     // rows past the end repeat the last one
    const int c = (q % 8) ^ ((q / 8) & 7);               // the chunk that belongs at this LDS slot
    xoff[i] = (uint32_t)((row - m0) * p.k_dim * 2 + c * 16);
    xdst[i] = i * kPThreads * 16;
  }
#pragma unroll
  for (int i = 0; i < kWLoads; ++i) {
    const int q = i * kPThreads + tid;
    const int c = (q % 8) ^ ((q / 8) & 7);
    woff[i] = (uint32_t)((q / 8) * p.k_dim * 2 + c * 16);
    wdst[i] = kXBytes + i * kPThreads * 16;
  }
  const char* xbase = static_cast<const char*>(p.x) + m0 * p.k_dim * 2;
  const char* wbase = static_cast<const char*>(p.w) + (int64_t)n0 * p.k_dim * 2;
  const int k_steps = p.k_dim / kPK;

  auto issue = [&](int ks) {
    const uint32_t st = wave_lds + (ks % kPStages) * kPStage;
    const char* xb = xbase + (int64_t)ks * kPK * 2;
    const char* wb = wbase + (int64_t)ks * kPK * 2;
#pragma unroll
    for (int i = 0; i < kXLoads; ++i) dma16(xb, xoff[i], st + xdst[i]);
#pragma unroll
    for (int i = 0; i < kWLoads; ++i) dma16(wb, woff[i], st + wdst[i]);
  };
  constexpr int L = kXLoads + kWLoads;

#pragma unroll
  for (int s = 0; s < kPStages - 1; ++s)
    if (s < k_steps) issue(s);

  f32x16 acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i) acc[i][0] = acc[i][1] = f32x16{};
  float ss[2] = {0.f, 0.f};
  const int qr = lane & 31, hf = lane >> 5;

  for (int ks = 0; ks < k_steps; ++ks) {
    if (ks + 1 < k_steps) wait_vm_lgkm0<L>(); else wait_vm_lgkm0<0>();
    barrier_only();   // stage ks is in for every thread; stage (ks - 1) % S is free
    if (ks + kPStages - 1 < k_steps) issue(ks + kPStages - 1);
    const YOCO_LDS char* xs = smem + (ks % kPStages) * kPStage;
    const YOCO_LDS char* ws = xs + kXBytes;
#pragma unroll
    for (int kk = 0; kk < kPK / 16; ++kk) {
      bf16x8 a[2], b[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int r = wm * 64 + 32 * i + qr;
        a[i] = *reinterpret_cast<const YOCO_LDS bf16x8*>(xs + swz(r, 2 * kk + hf));
      }
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int r = wn * 64 + 32 * j + qr;
        b[j] = *reinterpret_cast<const YOCO_LDS bf16x8*>(ws + swz(r, 2 * kk + hf));
      }
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j) acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[j], acc[i][j], 0, 0, 0);
      if ((kk >> 1) == wn) {
        // sum of squares of this lane's 8 values of row r (k half hf); the two
        // waves that read the same rows take half of the k steps each
#pragma unroll
        for (int i = 0; i < 2; ++i) {
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const bf16x2 v2 = {a[i][2 * e], a[i][2 * e + 1]};
            ss[i] = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, ss[i], false);
          }
        }
      }
    }
  }
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const float tot = ss[i] + __shfl_xor(ss[i], 32);
    if (hf == 0) ss_part[wn][wm * 64 + 32 * i + qr] = tot;
  }
  __syncthreads();
  if (tid < kPM) inv_rms[tid] = 1.0f / sqrtf((ss_part[0][tid] + ss_part[1][tid]) / (float)p.k_dim + p.eps);
  __syncthreads();

  // epilogue: lane holds column n0 + wn*64 + 32j + qr, rows 8(r/4) + 4hf + r%4 of block i
  const int hd = p.n_cols / 2;                 // K^ columns, then V^ columns
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int n = n0 + wn * 64 + 32 * j + qr;
    const bool is_v = n >= hd;
    const int nc = is_v ? n - hd : n;
    __bf16* dst = static_cast<__bf16*>(is_v ? p.v : p.k);
    const __bf16* bottom = static_cast<const __bf16*>(is_v ? p.v1 : p.k1);
    const float a1 = is_v ? p.av1 : p.ak1, a2 = is_v ? p.av2 : p.ak2;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int lr = wm * 64 + 32 * i + 8 * (r >> 2) + 4 * hf + (r & 3);
        const int64_t pr = prow[lr];
        if (pr < 0) continue;
        float val = acc[i][j][r] * inv_rms[lr];
        if (bottom != nullptr) val = p.lam * (a1 * (float)bottom[(m0 + lr) * hd + nc] + a2 * val);
        dst[pr * hd + nc] = (__bf16)val;
      }
    }
  }
}

// Wide tile (n_cols a multiple of 256): 256 rows x 256 columns per workgroup,
// 64 k per stage through 2 stages (64 KB each; 32 k through 4 stages measured
// 5-7% slower: twice the barriers), so each row block of X is read
// half as often as with 128 columns and every byte brought into LDS feeds
// twice the MFMA work. The product is formed transposed, C^T = W' X^T (A = W'
// rows, B = X rows), so a lane ends up with 4 consecutive output columns per
// register group; the tile is staged in LDS (the stages' 128 KB) and written
// as whole rows, 16 bytes per lane. Waves: 4 (rows) x 2 (columns), each
// 64 rows x 128 columns (2 x 4 MFMA blocks).
constexpr int kWM = 256;
constexpr int kWN = 256;
#ifndef YOCO_PROJ_WK
#define YOCO_PROJ_WK 64
#endif
constexpr int kWK = YOCO_PROJ_WK;
constexpr int kWStages = 128 / kWK;          // 128 KB of stages
constexpr int kWCpr = kWK / 8;              // 16-byte chunks per tile row
constexpr int kWXBytes = kWM * kWK * 2;
constexpr int kWWBytes = kWN * kWK * 2;
constexpr int kWStage = kWXBytes + kWWBytes;
constexpr int kWXLoads = kWM * kWK / 8 / kPThreads;
constexpr int kWWLoads = kWN * kWK / 8 / kPThreads;
static_assert(kWStages * kWStage == kWM * kWN * 2, "the output tile is staged in the stages");

// XOR applied to the 16-byte chunks of tile row r so that 16 lanes reading one
// chunk of 16 consecutive rows hit distinct banks (rows of 64 or 128 bytes)
__device__ __forceinline__ int wswz(int r) { return kWK == 32 ? ((r >> 2) & 3) : ((r >> 1) & 7); }
__device__ __forceinline__ uint32_t swz32(int r, int c) { return (uint32_t)(r * (kWK * 2) + 16 * (c ^ wswz(r))); }
// 16-byte chunk c (of 32) of row r of the [256][256] bf16 output staging tile
__device__ __forceinline__ uint32_t swz_out(int r, int c) { return (uint32_t)(r * 512 + 16 * (c ^ (r & 31))); }

__global__ __launch_bounds__(kPThreads, 1) void kv_project_wide_kernel(ProjectParams p) {
  __shared__ __attribute__((aligned(16))) char smem_raw[kWStages * kWStage];
  __shared__ int64_t prow[kWM];
  __shared__ float ss_part[2][kWM];
  __shared__ float inv_rms[kWM];
  YOCO_LDS char* smem = (YOCO_LDS char*)smem_raw;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int wt = wave >> 1;          // 0..3: rows wt*64 ..
  const int wn = wave & 1;           // 0..1: columns wn*128 ..
  const int n_tiles = p.n_cols / kWN;
  const int grid = (int)gridDim.x;
  const int xcd = (int)blockIdx.x % kXcds, j = (int)blockIdx.x / kXcds;
  const int tile = xcd * (grid / kXcds) + min(xcd, grid % kXcds) + j;
  const int nt = tile % n_tiles;
  const int mt = tile / n_tiles;
  const int64_t m0 = (int64_t)mt * kWM;
  const int n0 = nt * kWN;

  if (tid < kWM) {
    const int64_t t = m0 + tid;
    int64_t dst = -1;
    if (t < p.total_rows) {
      int lo = 0, hi = p.batch;       // find b with cu[b] <= t < cu[b + 1]
      while (hi - lo > 1) {
        const int mid = (lo + hi) >> 1;
        if (p.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
      }
      const int b = lo;
      const int64_t c0 = p.cu_seqlens[b], c1 = p.cu_seqlens[b + 1];
      const int64_t len = p.seq_len[b], cap = p.seq_cap[b], start = p.seq_start[b];
      const bool fits = t >= c0 && t < c1 && c1 <= p.total_rows && len >= 0 && start >= 0 &&
                        len + (c1 - c0) <= cap && start + len + (c1 - c0) <= p.pool_rows;
      if (fits) dst = start + len + (t - c0);
    }
    prow[tid] = dst;
  }
  // the row lookups' loads are done: from here on the only loads in flight are
  // the tile copies, which the loop awaits by count (a load of the compiler's
  // own still pending at the loop would make it wait for everything there)
  wait_vm_lgkm0<0>();

  // this thread's chunks: chunk q = i * threads + tid -> tile row q / cpr, slot q % cpr
  uint32_t xoff[kWXLoads], woff[kWWLoads];
  const uint32_t wave_lds = (uint32_t)(uintptr_t)smem + (uint32_t)__builtin_amdgcn_readfirstlane(wave) * 64 * 16;
#pragma unroll
  for (int i = 0; i < kWXLoads; ++i) {
    const int q = i * kPThreads + tid;
    int64_t row = m0 + q / kWCpr;
    if (row >= p.total_rows) row = p.total_rows - 1;     // rows past the end repeat the last one
    const int c = (q % kWCpr) ^ wswz(q / kWCpr);         // the chunk that belongs at this LDS slot
    xoff[i] = (uint32_t)((row - m0) * p.k_dim * 2 + c * 16);
  }
#pragma unroll
  for (int i = 0; i < kWWLoads; ++i) {
    const int q = i * kPThreads + tid;
    const int c = (q % kWCpr) ^ wswz(q / kWCpr);
    woff[i] = (uint32_t)((q / kWCpr) * p.k_dim * 2 + c * 16);
  }
  const char* xbase = static_cast<const char*>(p.x) + m0 * p.k_dim * 2;
  const char* wbase = static_cast<const char*>(p.w) + (int64_t)n0 * p.k_dim * 2;
  const int k_steps = p.k_dim / kWK;

  auto issue = [&](int ks) {
    const uint32_t st = wave_lds + (ks % kWStages) * kWStage;
    const char* xb = xbase + (int64_t)ks * kWK * 2;
    const char* wb = wbase + (int64_t)ks * kWK * 2;
#pragma unroll
    for (int i = 0; i < kWXLoads; ++i) dma16(xb, xoff[i], st + i * kPThreads * 16);
#pragma unroll
    for (int i = 0; i < kWWLoads; ++i) dma16(wb, woff[i], st + kWXBytes + i * kPThreads * 16);
  };
  constexpr int L = kWXLoads + kWWLoads;

#pragma unroll
  for (int s = 0; s < kWStages - 1; ++s)
    if (s < k_steps) issue(s);

  // acc[tb][nb]: C^T block (output columns 32 nb .., rows 32 tb ..) of this wave
  f32x16 acc[2][4];
#pragma unroll
  for (int tb = 0; tb < 2; ++tb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[tb][nb] = f32x16{};
  float ss[2] = {0.f, 0.f};
  const int qr = lane & 31, hf = lane >> 5;

  for (int ks = 0; ks < k_steps; ++ks) {
    // stage ks is in when at most the stages requested after it are in flight
    const int ahead = min(kWStages - 2, k_steps - 1 - ks);
    if (kWStages >= 4 && ahead >= 2) wait_vm_lgkm0<(kWStages >= 4 ? 2 * L : 0)>();
    else if (kWStages >= 3 && ahead >= 1) wait_vm_lgkm0<(kWStages >= 3 ? L : 0)>();
    else wait_vm_lgkm0<0>();
    barrier_only();   // stage ks is in for every thread; stage (ks - 1) % S is free
    if (ks + kWStages - 1 < k_steps) issue(ks + kWStages - 1);
    const YOCO_LDS char* xs = smem + (ks % kWStages) * kWStage;
    const YOCO_LDS char* ws = xs + kWXBytes;
    // all operand reads of the stage first (both 16-k steps), then the MFMAs,
    // so the second step's reads are in flight during the first step's MFMAs
    bf16x8 xb[kWK / 16][2], wa[kWK / 16][4];
#pragma unroll
    for (int kk = 0; kk < kWK / 16; ++kk) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
        xb[kk][tb] = *reinterpret_cast<const YOCO_LDS bf16x8*>(xs + swz32(wt * 64 + 32 * tb + qr, 2 * kk + hf));
#pragma unroll
      for (int nb = 0; nb < 4; ++nb)
        wa[kk][nb] = *reinterpret_cast<const YOCO_LDS bf16x8*>(ws + swz32(wn * 128 + 32 * nb + qr, 2 * kk + hf));
    }
#pragma unroll
    for (int kk = 0; kk < kWK / 16; ++kk) {
#pragma unroll
      for (int tb = 0; tb < 2; ++tb)
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[tb][nb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(wa[kk][nb], xb[kk][tb], acc[tb][nb], 0, 0, 0);
    }
    // sum of squares of this lane's 8 values of row qr (k half hf); the two
    // waves that read the same rows take half of the 16-k steps each
#pragma unroll
    for (int kk = 0; kk < kWK / 16; ++kk) {
      if ((2 * kk) / (kWK / 16) != wn) continue;   // wave-uniform; constant indices keep xb in registers
#pragma unroll
      for (int tb = 0; tb < 2; ++tb) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const bf16x2 v2 = {xb[kk][tb][2 * e], xb[kk][tb][2 * e + 1]};
          ss[tb] = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, ss[tb], false);
        }
      }
    }
  }
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const float tot = ss[tb] + __shfl_xor(ss[tb], 32);
    if (hf == 0) ss_part[wn][wt * 64 + 32 * tb + qr] = tot;
  }
  wait_vm_lgkm0<0>();
  __syncthreads();   // every wave is done with the stages: they become the output tile
  if (tid < kWM) inv_rms[tid] = 1.0f / sqrtf((ss_part[0][tid] + ss_part[1][tid]) / (float)p.k_dim + p.eps);
  __syncthreads();

  // stage: lane holds output row t = wt*64 + 32tb + qr, columns
  // wn*128 + 32nb + 8g + 4hf .. +3 in registers 4g .. 4g + 3
#pragma unroll
  for (int tb = 0; tb < 2; ++tb) {
    const int t = wt * 64 + 32 * tb + qr;
    const float s = inv_rms[t];
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int col = wn * 128 + 32 * nb + 8 * g;     // 16-byte chunk col / 8, half hf
        const u32x2 v = {pack2(acc[tb][nb][4 * g + 0] * s, acc[tb][nb][4 * g + 1] * s),
                         pack2(acc[tb][nb][4 * g + 2] * s, acc[tb][nb][4 * g + 3] * s)};
        *reinterpret_cast<YOCO_LDS u32x2*>(smem + swz_out(t, col / 8) + 8 * hf) = v;
      }
    }
  }
  __syncthreads();

  // write whole rows: 32 lanes per row, 16 bytes (8 columns) each
  const int hd = p.n_cols / 2;                 // K^ columns, then V^ columns
#pragma unroll 4
  for (int it = 0; it < kWM * 32 / kPThreads; ++it) {
    const int q = it * kPThreads + tid;
    const int t = q / 32, c = q % 32;
    const int64_t pr = prow[t];
    if (pr < 0) continue;
    const int n = n0 + 8 * c;
    const bool is_v = n >= hd;
    const int nc = is_v ? n - hd : n;
    u32x4 v = *reinterpret_cast<const YOCO_LDS u32x4*>(smem + swz_out(t, c));
    const __bf16* bottom = static_cast<const __bf16*>(is_v ? p.v1 : p.k1);
    if (bottom != nullptr) {
      const float a1 = is_v ? p.av1 : p.ak1, a2 = is_v ? p.av2 : p.ak2;
      const u32x4 bv = *reinterpret_cast<const u32x4*>(bottom + (m0 + t) * hd + nc);
      const bf16x8 x8 = __builtin_bit_cast(bf16x8, v), b8 = __builtin_bit_cast(bf16x8, bv);
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e)
        w[e] = pack2(p.lam * (a1 * (float)b8[2 * e] + a2 * (float)x8[2 * e]),
                     p.lam * (a1 * (float)b8[2 * e + 1] + a2 * (float)x8[2 * e + 1]));
      v = u32x4{w[0], w[1], w[2], w[3]};
    }
    __bf16* dst = static_cast<__bf16*>(is_v ? p.v : p.k);
    *reinterpret_cast<u32x4*>(dst + pr * hd + nc) = v;
  }
}

// Few rows (decode: one per sequence): the tile above would leave most CUs idle
// and stream the weights through one pipeline per 128 columns. Here a workgroup
// owns 16 columns and all (<= 16) rows; its 8 waves split d_model, read their
// A (rows) and B (weights) operands straight from memory (16 bytes per lane;
// the 12.6 MB of weights of the 3B geometry stay cached between calls), run
// v_mfma_f32_16x16x32_bf16 and add their partial tiles in LDS.
constexpr int kSmallRows = 16;
constexpr int kSmallWaves = 8;

__global__ __launch_bounds__(64 * kSmallWaves) void kv_project_small_kernel(ProjectParams p) {
  __shared__ float part[kSmallWaves][kSmallRows][17];
  __shared__ float ssq[kSmallWaves][kSmallRows];
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int n0 = blockIdx.x * 16;
  const int col = lane & 15, grp = lane >> 4;          // MFMA 16x16x32: k = 8 grp .. 8 grp + 7
  int64_t row = col < p.total_rows ? col : p.total_rows - 1;   // rows past the end repeat the last one
  const __bf16* xr = static_cast<const __bf16*>(p.x) + row * p.k_dim;
  const __bf16* wr = static_cast<const __bf16*>(p.w) + (int64_t)(n0 + col) * p.k_dim;
  const int per_wave = p.k_dim / kSmallWaves;          // a multiple of 8; steps of 32 k plus a tail of 8-k groups
  const int k_lo = wave * per_wave, k_hi = k_lo + per_wave;
  f32x4 acc = f32x4{};
  float ss = 0.f;
  for (int k = k_lo; k < k_hi; k += 32) {
    const int kk = k + 8 * grp;
    bf16x8 a = bf16x8{}, b = bf16x8{};
    if (kk < k_hi) {
      a = *reinterpret_cast<const bf16x8*>(xr + kk);
      b = *reinterpret_cast<const bf16x8*>(wr + kk);
    }
    acc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const bf16x2 v2 = {a[2 * e], a[2 * e + 1]};
      ss = __builtin_amdgcn_fdot2_f32_bf16(v2, v2, ss, false);
    }
  }
  // lane holds column col, rows 4 grp .. 4 grp + 3 (D layout of the 16x16 MFMA);
  // the sum of squares of row `col` over this wave's k is spread over the 4 groups
  ss += __shfl_xor(ss, 16);
  ss += __shfl_xor(ss, 32);
#pragma unroll
  for (int r = 0; r < 4; ++r) part[wave][4 * grp + r][col] = acc[r];
  if (grp == 0) ssq[wave][col] = ss;
  __syncthreads();
  if (wave != 0) return;
  // wave 0: sum the waves' partial tiles and write 16 columns x 16 rows
  const int hd = p.n_cols / 2;
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int rr = 4 * grp + r;
    float v = 0.f, sq = 0.f;
#pragma unroll
    for (int w = 0; w < kSmallWaves; ++w) {
      v += part[w][rr][col];
      sq += ssq[w][rr];
    }
    const int64_t t = rr;
    if (t >= p.total_rows) continue;
    int lo = 0, hi = p.batch;
    while (hi - lo > 1) {
      const int mid = (lo + hi) >> 1;
      if (p.cu_seqlens[mid] <= t) lo = mid; else hi = mid;
    }
    const int64_t c0 = p.cu_seqlens[lo], c1 = p.cu_seqlens[lo + 1];
    const int64_t len = p.seq_len[lo], cap = p.seq_cap[lo], start = p.seq_start[lo];
    const bool fits = t >= c0 && t < c1 && c1 <= p.total_rows && len >= 0 && start >= 0 &&
                      len + (c1 - c0) <= cap && start + len + (c1 - c0) <= p.pool_rows;
    if (!fits) continue;
    const int64_t pr = start + len + (t - c0);
    const int n = n0 + col;
    const bool is_v = n >= hd;
    const int nc = is_v ? n - hd : n;
    float val = v * (1.0f / sqrtf(sq / (float)p.k_dim + p.eps));
    const __bf16* bottom = static_cast<const __bf16*>(is_v ? p.v1 : p.k1);
    if (bottom != nullptr)
      val = p.lam * ((is_v ? p.av1 : p.ak1) * (float)bottom[t * hd + nc] + (is_v ? p.av2 : p.ak2) * val);
    static_cast<__bf16*>(is_v ? p.v : p.k)[pr * hd + nc] = (__bf16)val;
  }
}

// seq_len[b] += rows of sequence b if they fit (the projection wrote them),
// else the flag.
__global__ void kv_commit_kernel(ProjectParams p) {
  const int b = blockIdx.x * blockDim.x + threadIdx.x;
  if (b >= p.batch) return;
  const int64_t c0 = p.cu_seqlens[b], c1 = p.cu_seqlens[b + 1];
  const int64_t len = p.seq_len[b], cap = p.seq_cap[b], start = p.seq_start[b];
  const bool fits = c1 >= c0 && c1 <= p.total_rows && len >= 0 && start >= 0 && len + (c1 - c0) <= cap &&
                    start + len + (c1 - c0) <= p.pool_rows;
  if (fits) p.seq_len[b] = (int32_t)(len + (c1 - c0));
  else if (p.overflow != nullptr) p.overflow[0] = 1;
}

// W'[n][k] = gain[k] * (n < hd ? W_K[k][n] : W_V[k][n - hd]), through a 32 x 32 LDS tile.
__global__ __launch_bounds__(256) void kv_pack_kernel(const __bf16* gain, const __bf16* wk, const __bf16* wv,
                                                      __bf16* out, int k_dim, int hd) {
  __shared__ float tile[32][33];
  const int n_cols = 2 * hd;
  const int tk = blockIdx.y * 32, tn = blockIdx.x * 32;
  const int tx = threadIdx.x & 31, ty = threadIdx.x >> 5;   // 32 x 8
  for (int r = ty; r < 32; r += 8) {
    const int k = tk + r, n = tn + tx;
    float v = 0.f;
    if (k < k_dim && n < n_cols)
      v = (float)gain[k] * (float)(n < hd ? wk[(int64_t)k * hd + n] : wv[(int64_t)k * hd + n - hd]);
    tile[r][tx] = v;
  }
  __syncthreads();
  for (int r = ty; r < 32; r += 8) {
    const int n = tn + r, k = tk + tx;
    if (n < n_cols && k < k_dim) out[(int64_t)n * k_dim + k] = (__bf16)tile[tx][r];
  }
}

}  // namespace

hipError_t launch_kv_project(const ProjectParams& p, hipStream_t stream) {
  if (p.total_rows > 0 && p.total_rows <= kSmallRows) {
    hipLaunchKernelGGL(kv_project_small_kernel, dim3(p.n_cols / 16), dim3(64 * kSmallWaves), 0, stream, p);
  } else if (p.total_rows > 0 && p.n_cols % kWN == 0 && p.k_dim % kWK == 0) {
    const int64_t m_tiles = (p.total_rows + kWM - 1) / kWM;
    const int64_t grid = m_tiles * (p.n_cols / kWN);
    hipLaunchKernelGGL(kv_project_wide_kernel, dim3((unsigned)grid), dim3(kPThreads), 0, stream, p);
  } else if (p.total_rows > 0) {
    const int64_t m_tiles = (p.total_rows + kPM - 1) / kPM;
    const int64_t grid = m_tiles * (p.n_cols / kPN);
    hipLaunchKernelGGL(kv_project_kernel, dim3((unsigned)grid), dim3(kPThreads), 0, stream, p);
  }
  hipLaunchKernelGGL(kv_commit_kernel, dim3((p.batch + 255) / 256), dim3(256), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_kv_pack(const void* gain, const void* wk, const void* wv, void* out, int k_dim, int hd,
                          hipStream_t stream) {
  dim3 grid((2 * hd + 31) / 32, (k_dim + 31) / 32);
  hipLaunchKernelGGL(kv_pack_kernel, grid, dim3(256), 0, stream, static_cast<const __bf16*>(gain),
                     static_cast<const __bf16*>(wk), static_cast<const __bf16*>(wv), static_cast<__bf16*>(out), k_dim,
                     hd);
  return hipGetLastError();
}

}  // namespace yoco
