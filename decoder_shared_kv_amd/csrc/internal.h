// Internal launch parameters and device helpers shared by the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace yoco {

// Everything a kernel needs, by value (kernel argument).
struct AttnParams {
  const void* q;
  void* out;
  float* lse;
  const void* k;
  const void* v;
  const int64_t* seq_start;
  const int32_t* seq_len;
  const int32_t* seq_cap;
  const int32_t* cu_seqlens;  // prefill only
  int64_t pool_rows;
  int64_t total_q;            // prefill: rows of q/out, columns of lse
  int32_t batch;
  int32_t hq;
  int32_t hkv;
  int32_t group;              // hq / hkv
  float scale_log2;           // scale * log2(e): scores are kept in the base-2 domain
  int32_t window;             // sliding window in positions (0: none, plain causal)
  // prefill grid
  int32_t pos_blocks;         // position blocks covering max_q_len
  int32_t n_items;            // (unit, position block) work items of the prefill schedule
  int32_t* queue;             // prefill work queue counters (workspace), or null for the static grid
  // decode split plan: the row blocks of all sequences are cut into `splits`
  // equal shares per column (bf16: KV head x head chunk; f32: query head)
  int32_t splits;
  int32_t slots;              // partial slots per query head: splits + batch
  int32_t head_chunks;        // query-head chunks of <= 16 per KV head (decode)
  float* part_o;              // [Hq, slots, D] unnormalised partial outputs
  float* part_ml;             // [Hq, slots, 2] (running max in base 2, sum of weights)
  int32_t* decode_meta;       // [B, 2]: each sequence's first partial slot and its number of pieces
};

struct AppendParams {
  void* k;
  void* v;
  const void* k_new;
  const void* v_new;
  const int64_t* seq_start;
  int32_t* seq_len;
  const int32_t* seq_cap;
  int32_t* overflow;
  int64_t pool_rows;
  int32_t row_bytes;          // Hkv * head_dim * element size (multiple of 16)
  int32_t ring;               // 1: ring window cache, the row goes to slot seq_len mod seq_cap
};

// The shared cache's producer: RMSNorm + [W_K | W_V] projection + append.
struct ProjectParams {
  const void* x;              // [total_rows, k_dim] bf16, the Self-Decoder output rows
  const void* w;              // [n_cols, k_dim] bf16, gain-folded packed weights
  void* k;                    // cache pools [pool_rows, n_cols / 2] bf16
  void* v;
  const void* k1;             // YOCO++ bottom-layer rows [total_rows, n_cols / 2] or null
  const void* v1;
  const int64_t* seq_start;
  int32_t* seq_len;
  const int32_t* seq_cap;
  const int32_t* cu_seqlens;  // [batch + 1]
  int32_t* overflow;
  int64_t pool_rows;
  int64_t total_rows;
  int32_t batch;
  int32_t k_dim;              // d_model, a multiple of 64
  int32_t n_cols;             // 2 * Hkv * head_dim, a multiple of 128
  float eps;
  float lam, ak1, ak2, av1, av2;
};

// Gated retention (gRet): chunkwise prefill and recurrent decode.
struct GretParams {
  const void* q;              // [T, H, D] bf16 (decode: [B, H, D])
  const void* k;
  const void* v;
  const float* gamma;         // [T, H] (decode: [B, H]) per-token, per-head gates
  void* out;                  // [T, H, D] bf16 (decode: [B, H, D])
  const int32_t* cu_seqlens;  // [B + 1] (prefill)
  const float* state_in;      // [B, H, D(dk), D(dv)] fp32 or null (prefill)
  float* state_out;           // [B, H, D, D]: prefill's final states; decode's states, updated in place
  float* seg_u;               // workspace: per segment slot, its state contribution U [D(dk)][D(dv)]
  float* seg_s;               // workspace: per segment slot, its incoming state S [D(dk)][D(dv)]
  float* seg_decay;           // workspace: per segment slot, its total decay
  int64_t total_rows;
  int32_t batch;
  int32_t heads;
  int32_t slots;              // segment slots per head in the workspace, at least the segments of
                              // all sequences together for any lengths
  int32_t seg_chunks;         // chunks (of 256 rows) per segment, >= 1
};

// Host launchers (one per kernel family); each returns the hipGetLastError code.
hipError_t launch_kv_append(const AppendParams& p, int batch, hipStream_t stream);
hipError_t launch_prefill_bf16(const AttnParams& p, int head_dim, int items, hipStream_t stream);
hipError_t launch_prefill_f32(const AttnParams& p, int head_dim, int grid, hipStream_t stream);
hipError_t launch_decode_split_bf16(const AttnParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_split_f32(const AttnParams& p, int head_dim, hipStream_t stream);
hipError_t launch_decode_merge(const AttnParams& p, int head_dim, int dtype, hipStream_t stream);
hipError_t launch_kv_project(const ProjectParams& p, hipStream_t stream);
hipError_t launch_gret_prefill(const GretParams& p, int head_dim, hipStream_t stream);
hipError_t launch_gret_decode(const GretParams& p, int head_dim, hipStream_t stream);
// Device address of this device's no-allocation scratch (YOCO_NOALLOC_SCRATCH_BYTES,
// 256-byte aligned), looked up once per device.
hipError_t noalloc_scratch(void** ptr);
hipError_t launch_kv_pack(const void* gain, const void* wk, const void* wv, void* out, int k_dim, int hd,
                          hipStream_t stream);

// Prefill tiling shared between the planner and the kernels.
#ifndef YOCO_PREFILL_WAVES
#define YOCO_PREFILL_WAVES 8
#endif
constexpr int kPrefillRowsPerWave = 32;
constexpr int kPrefillWaves = YOCO_PREFILL_WAVES;
constexpr int kPrefillThreads = 64 * kPrefillWaves;
// heads of one KV group that one prefill workgroup serves: the largest power of
// two that divides the group and does not exceed the wave count
__host__ __device__ inline int prefill_heads_per_wg(int group) {
  int h = kPrefillWaves;
  while (h > 1 && group % h != 0) h >>= 1;
  return h;
}
__host__ __device__ inline int prefill_positions_per_wg(int group) {
  return kPrefillRowsPerWave * (kPrefillWaves / prefill_heads_per_wg(group));
}

// XCD-affine order of the prefill grid. Workgroup i runs on XCD i % 8. With U
// units of P position blocks each:
//  * U % 8 == 0: XCD x takes units x, x+8, ... one after the other, each unit's
//    blocks longest first (grid U*P);
//  * 8 % U == 0: the 8/U XCDs sharing unit x % U take its blocks round-robin
//    (grid 8 * ceil(P / (8/U)); blocks past P are empty);
//  * otherwise: unit-major order (grid U*P).
constexpr int kXcds = 8;
__host__ __device__ inline int64_t prefill_grid(int units, int pos_blocks) {
  if (units % kXcds != 0 && kXcds % units == 0) {
    const int per = kXcds / units;
    return (int64_t)kXcds * ((pos_blocks + per - 1) / per);
  }
  return (int64_t)units * pos_blocks;
}
__host__ __device__ inline void prefill_schedule(int bid, int units, int pos_blocks, int* unit, int* rank) {
  if (units % kXcds == 0) {
    const int x = bid % kXcds, j = bid / kXcds;
    *unit = x + kXcds * (j / pos_blocks);
    *rank = j % pos_blocks;
  } else if (kXcds % units == 0) {
    const int x = bid % kXcds, j = bid / kXcds;
    *unit = x % units;
    *rank = x / units + (kXcds / units) * j;
  } else {
    *unit = bid / pos_blocks;
    *rank = bid % pos_blocks;
  }
}

// Prefill work queue (bf16 prefill with a workspace). The items are the
// workgroups of the static schedule above, item i belonging to XCD i % 8; a
// persistent grid of one workgroup per CU takes them from per-XCD queues
// (queue x holds items x, x + 8, ... in schedule order) through atomic
// counters, and a workgroup whose own queue is empty takes items from the
// others, so faster XCDs absorb the tail. Counter layout (int32, one per
// 128-byte line): queues 0..7, then the count of workgroups done; the last
// workgroup to finish sets all of them back to zero, so the counters are zero
// between calls (the caller zeroes them once, when the workspace is allocated).
constexpr int kQueueStride = 32;                       // int32 per counter line
constexpr int kQueueCounters = kXcds + 1;
constexpr size_t kPrefillQueueBytes = 2048;            // >= kQueueCounters * kQueueStride * 4

// fp32 prefill: one thread per query row, 64 rows per workgroup
constexpr int kPrefillF32Rows = 64;

// Readable rows of sequence b: min(seq_len, seq_cap), limited to the pool.
__device__ __forceinline__ int32_t readable_rows(const int64_t* seq_start, const int32_t* seq_len,
                                                 const int32_t* seq_cap, int64_t pool_rows, int b,
                                                 int64_t* start_out) {
  int64_t s = seq_start[b];
  int64_t n = seq_len[b];
  int64_t c = seq_cap[b];
  if (n > c) n = c;
  if (s < 0 || s > pool_rows) s = 0, n = 0;
  if (n > pool_rows - s) n = pool_rows - s;
  if (n < 0) n = 0;
  *start_out = s;
  return (int32_t)n;
}

// Decode under a sliding window: of the n readable rows only the last `window`
// are visible to the query at position n - 1.
__device__ __forceinline__ int32_t window_rows(int32_t n, int32_t window, int64_t* start) {
  if (window > 0 && n > window) {
    *start += n - window;
    return window;
  }
  return n;
}

// Decode work unit: blocks of 128 rows of one sequence (a multiple of every
// decode kernel's rows per iteration).
constexpr int kDecodeBlockRows = 128;

// Rows of sequence b that its decode query sees (0 for b >= batch) and the
// pool row of the first of them.
__device__ __forceinline__ int32_t decode_rows(const AttnParams& p, int b, int64_t* start) {
  *start = 0;
  if (b >= p.batch) return 0;
  return window_rows(readable_rows(p.seq_start, p.seq_len, p.seq_cap, p.pool_rows, b, start), p.window, start);
}
__device__ __forceinline__ int decode_blocks(int32_t rows) { return (rows + kDecodeBlockRows - 1) / kDecodeBlockRows; }

// The balanced decode split. Each column cuts the `total` blocks of all
// sequences into parts = min(shares planned, total) shares, so none is empty.
// Share w of `parts` equal shares of `total` blocks starts at block
// floor(w * total / parts); block x belongs to the last share starting at or
// before it, share floor(((x + 1) * parts - 1) / total). Both quotients are
// taken in fp64 (an emulated int64 division costs ~100 instructions): the
// products are exact and a correctly rounded quotient of integers floors to
// the exact result while total * parts < 2^52 (parts <= 4096 here, so up to
// 2^40 blocks).
__host__ __device__ inline int64_t share_begin(int64_t w, int64_t total, int parts) {
  return (int64_t)((double)(w * total) / (double)parts);
}
__host__ __device__ inline int64_t share_of_block(int64_t x, int64_t total, int parts) {
  return (int64_t)((double)((x + 1) * parts - 1) / (double)total);
}

// A value equal in every lane, moved to scalar registers.
__device__ __forceinline__ int64_t uniform_i64(int64_t x) {
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)x);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// Wave-wide integer sum and inclusive prefix sum (64 lanes, all active).
__device__ __forceinline__ int wave_incl_scan_i32(int x);
__device__ __forceinline__ int wave_sum_i32(int x) {
  return __builtin_amdgcn_readlane(wave_incl_scan_i32(x), 63);
}
// The scan runs on DPP lane moves (no LDS): shifts right by 1, 2, 4, 8 within
// each row of 16 lanes (lanes shifted in read 0), then the last lane of row 0
// is added to row 1, of row 2 to row 3 (row_bcast:15, rows 1 and 3), and the
// last lane of row 1 to rows 2 and 3 (row_bcast:31).
__device__ __forceinline__ int wave_incl_scan_i32(int x) {
  x += __builtin_amdgcn_update_dpp(0, x, 0x111, 0xf, 0xf, true);   // row_shr:1
  x += __builtin_amdgcn_update_dpp(0, x, 0x112, 0xf, 0xf, true);   // row_shr:2
  x += __builtin_amdgcn_update_dpp(0, x, 0x114, 0xf, 0xf, true);   // row_shr:4
  x += __builtin_amdgcn_update_dpp(0, x, 0x118, 0xf, 0xf, true);   // row_shr:8
  x += __builtin_amdgcn_update_dpp(0, x, 0x142, 0xa, 0xf, false);  // row_bcast:15
  x += __builtin_amdgcn_update_dpp(0, x, 0x143, 0xc, 0xf, false);  // row_bcast:31
  return x;
}

}  // namespace yoco
