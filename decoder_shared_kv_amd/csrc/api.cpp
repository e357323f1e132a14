// C ABI entry points: host-side argument checks, launch planning, dispatch.
//
// Every check runs before the first launch, so a call that returns an error has
// launched nothing. All launches go to the caller's stream; nothing here
// synchronises, allocates or keeps state between calls.
#include <cmath>
#include <cstdint>

#include "yoco_xattn.h"
#include "internal.h"

namespace {

using yoco::AttnParams;

constexpr float kLog2e = 1.4426950408889634f;
// bf16 decode: workgroups of all columns together. Two fit one CU, so 512 are
// one round on 256 CUs. Measured on MI355X (8 x 131072, 1 x 1048576, 4 x 131072
// and 16 x 17292 rows): one round is fastest with one or two columns (KV
// heads x head chunks), two rounds with four or more.
#ifndef YOCO_DECODE_TARGET_WGS
#define YOCO_DECODE_TARGET_WGS 0
#endif
int64_t decode_target_wgs(int64_t columns) {
  if (YOCO_DECODE_TARGET_WGS > 0) return YOCO_DECODE_TARGET_WGS;
  return columns <= 2 ? 512 : 1024;
}
// f32 decode: threads of all columns together
constexpr int kDecodeTargetThreadsF32 = 4096;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

int elem_size(int dtype) { return dtype == YOCO_DTYPE_BF16 ? 2 : 4; }

yoco_status check_dims(const yoco_dims* d) {
  if (d == nullptr) return YOCO_ERR_INVALID_ARG;
  if (d->batch < 1 || d->num_q_heads < 1 || d->num_kv_heads < 1) return YOCO_ERR_INVALID_ARG;
  if (d->num_q_heads % d->num_kv_heads != 0) return YOCO_ERR_INVALID_ARG;
  if (!std::isfinite(d->scale) || !(d->scale > 0.f)) return YOCO_ERR_INVALID_ARG;
  if (d->dtype != YOCO_DTYPE_F32 && d->dtype != YOCO_DTYPE_BF16) return YOCO_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return YOCO_ERR_UNSUPPORTED;
  return YOCO_OK;
}

yoco_status check_cache(const yoco_kv_cache* c) {
  if (c == nullptr) return YOCO_ERR_INVALID_ARG;
  if (c->k == nullptr || c->v == nullptr || !aligned16(c->k) || !aligned16(c->v)) return YOCO_ERR_INVALID_ARG;
  if (c->seq_start == nullptr || c->seq_len == nullptr || c->seq_cap == nullptr) return YOCO_ERR_INVALID_ARG;
  if (!aligned4(c->seq_len) || !aligned4(c->seq_cap) || (reinterpret_cast<uintptr_t>(c->seq_start) & 7u))
    return YOCO_ERR_INVALID_ARG;
  if (c->pool_rows < 0) return YOCO_ERR_INVALID_ARG;
  return YOCO_OK;
}

int head_chunks(const yoco_dims* d) {
  const int g = d->num_q_heads / d->num_kv_heads;
  return (g + 15) / 16;
}

// Columns of the balanced decode split: workgroups of one (KV head, head chunk)
// for bf16, threads of one query head for f32.
int64_t decode_columns(const yoco_dims* d) {
  return d->dtype == YOCO_DTYPE_BF16 ? (int64_t)d->num_kv_heads * head_chunks(d) : (int64_t)d->num_q_heads;
}

// Most shares per column any plan uses.
int32_t decode_share_cap(const yoco_dims* d) {
  const int64_t cols = decode_columns(d);
  const int64_t target = d->dtype == YOCO_DTYPE_BF16 ? decode_target_wgs(cols) : kDecodeTargetThreadsF32;
  const int64_t c = target / cols;
  return (int32_t)(c < 1 ? 1 : c);
}

// Blocks of 128 rows the hints describe: total_kv_len (0: B * max_kv_len),
// kept within max_kv_len .. B * max_kv_len.
int64_t decode_hint_blocks(const yoco_dims* d, int32_t max_kv_len, int64_t total_kv_len) {
  const int64_t n = max_kv_len > 0 ? max_kv_len : 1;
  const int64_t all = (int64_t)d->batch * n;
  int64_t total = total_kv_len > 0 && total_kv_len < all ? total_kv_len : all;
  if (total < n) total = n;
  return (total + yoco::kDecodeBlockRows - 1) / yoco::kDecodeBlockRows;
}

// Split plan: every column cuts the 128-row blocks of all sequences into
// `shares` equal shares; about decode_target_wgs workgroups in all, fewer when
// the hinted rows hold fewer blocks, so that no share is planned empty. The
// hints size the plan only: the kernels count the blocks on the device. The
// plan grows with max_kv_len, so a workspace sized for max_kv_len fits every
// call with a smaller one and any total_kv_len.
int32_t decode_shares(const yoco_dims* d, int32_t max_kv_len, int64_t total_kv_len) {
  const int64_t blocks = decode_hint_blocks(d, max_kv_len, total_kv_len);
  const int64_t cap = decode_share_cap(d);
  return (int32_t)(blocks < cap ? blocks : cap);
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Workspace: part_o [Hq, shares + B, D] fp32, part_ml [Hq, shares + B, 2] fp32,
// meta [B, 2] int32.
size_t decode_ml_offset(const yoco_dims* d, int32_t shares) {
  return align256((size_t)d->num_q_heads * (shares + d->batch) * d->head_dim * sizeof(float));
}
size_t decode_meta_offset(const yoco_dims* d, int32_t shares) {
  return decode_ml_offset(d, shares) + align256((size_t)d->num_q_heads * (shares + d->batch) * 2 * sizeof(float));
}
size_t decode_workspace(const yoco_dims* d, int32_t shares) {
  return decode_meta_offset(d, shares) + (size_t)d->batch * 2 * sizeof(int32_t);
}

AttnParams base_params(const yoco_dims* d, const yoco_kv_cache* c) {
  AttnParams p{};
  p.k = c->k;
  p.v = c->v;
  p.seq_start = c->seq_start;
  p.seq_len = c->seq_len;
  p.seq_cap = c->seq_cap;
  p.pool_rows = c->pool_rows;
  p.batch = d->batch;
  p.hq = d->num_q_heads;
  p.hkv = d->num_kv_heads;
  p.group = d->num_q_heads / d->num_kv_heads;
  p.scale_log2 = d->scale * kLog2e;
  return p;
}

yoco_status append_impl(const yoco_dims* dims, const yoco_kv_cache* cache, const void* k_new, const void* v_new,
                        int32_t* overflow_flag, int ring, void* stream) {
  yoco_status st = check_dims(dims);
  if (st != YOCO_OK) return st;
  st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (k_new == nullptr || v_new == nullptr || !aligned16(k_new) || !aligned16(v_new)) return YOCO_ERR_INVALID_ARG;
  if (overflow_flag != nullptr && !aligned4(overflow_flag)) return YOCO_ERR_INVALID_ARG;
  yoco::AppendParams p{};
  p.k = cache->k;
  p.v = cache->v;
  p.k_new = k_new;
  p.v_new = v_new;
  p.seq_start = cache->seq_start;
  p.seq_len = cache->seq_len;
  p.seq_cap = cache->seq_cap;
  p.overflow = overflow_flag;
  p.pool_rows = cache->pool_rows;
  p.row_bytes = dims->num_kv_heads * dims->head_dim * elem_size(dims->dtype);
  p.ring = ring;
  if (yoco::launch_kv_append(p, dims->batch, static_cast<hipStream_t>(stream)) != hipSuccess) return YOCO_ERR_HIP;
  return YOCO_OK;
}

yoco_status prefill_impl(const yoco_dims* dims, const yoco_kv_cache* cache, const void* q,
                         const int32_t* cu_seqlens_q, int32_t max_q_len, int64_t total_q, int32_t window, void* out,
                         float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  yoco_status st = check_dims(dims);
  if (st != YOCO_OK) return st;
  st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (q == nullptr || out == nullptr || cu_seqlens_q == nullptr) return YOCO_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(out) || !aligned4(cu_seqlens_q)) return YOCO_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned4(lse)) return YOCO_ERR_INVALID_ARG;
  if (max_q_len < 0 || total_q < 0) return YOCO_ERR_INVALID_ARG;
  const bool queue = workspace != nullptr && dims->dtype == YOCO_DTYPE_BF16;
  if (queue && (!aligned16(workspace) || workspace_bytes < yoco::kPrefillQueueBytes)) return YOCO_ERR_WORKSPACE;
  if (total_q == 0) return YOCO_OK;
  AttnParams p = base_params(dims, cache);
  p.q = q;
  p.out = out;
  p.lse = lse;
  p.cu_seqlens = cu_seqlens_q;
  p.total_q = total_q;
  p.window = window;
  const int64_t len = max_q_len > 0 ? max_q_len : 1;
  hipError_t err;
  if (dims->dtype == YOCO_DTYPE_BF16) {
    const int ppw = yoco::prefill_positions_per_wg(p.group);
    const int64_t units = (int64_t)dims->batch * dims->num_kv_heads * (p.group / yoco::prefill_heads_per_wg(p.group));
    const int64_t blocks = (len + ppw - 1) / ppw;
    if (blocks * units > INT32_MAX / 2 || units > INT32_MAX) return YOCO_ERR_UNSUPPORTED;
    p.pos_blocks = (int32_t)blocks;
    const int64_t items = yoco::prefill_grid((int)units, (int)blocks);
    p.n_items = (int32_t)items;
    if (queue) p.queue = static_cast<int32_t*>(workspace);   // the launcher sizes the persistent grid
    err = yoco::launch_prefill_bf16(p, dims->head_dim, (int)items, static_cast<hipStream_t>(stream));
  } else {
    const int64_t units = (int64_t)dims->batch * dims->num_q_heads;
    const int64_t blocks = (len + yoco::kPrefillF32Rows - 1) / yoco::kPrefillF32Rows;
    if (blocks * units > INT32_MAX) return YOCO_ERR_UNSUPPORTED;
    p.pos_blocks = (int32_t)blocks;
    err = yoco::launch_prefill_f32(p, dims->head_dim, (int)(blocks * units), static_cast<hipStream_t>(stream));
  }
  return err == hipSuccess ? YOCO_OK : YOCO_ERR_HIP;
}

// noalloc: the partials go to the library's device-resident scratch (of
// YOCO_NOALLOC_SCRATCH_BYTES on each device) instead of a caller workspace.
yoco_status decode_impl(const yoco_dims* dims, const yoco_kv_cache* cache, const void* q, int32_t max_kv_len,
                        int64_t total_kv_len, int32_t window, void* out, float* lse, void* workspace,
                        size_t workspace_bytes, void* stream, bool noalloc = false) {
  yoco_status st = check_dims(dims);
  if (st != YOCO_OK) return st;
  st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (q == nullptr || out == nullptr || !aligned16(q) || !aligned16(out)) return YOCO_ERR_INVALID_ARG;
  if (lse != nullptr && !aligned4(lse)) return YOCO_ERR_INVALID_ARG;
  if (max_kv_len < 0 || total_kv_len < 0) return YOCO_ERR_INVALID_ARG;
  if (window > 0) {
    // only the last `window` rows of each sequence are read: plan for those
    if (max_kv_len > window) max_kv_len = window;
    const int64_t cap = (int64_t)dims->batch * window;
    if (total_kv_len > cap) total_kv_len = cap;
  }
  const int32_t shares = decode_shares(dims, max_kv_len, total_kv_len);
  const size_t need = decode_workspace(dims, shares);
  if (noalloc) {
    if (need > (size_t)YOCO_NOALLOC_SCRATCH_BYTES) return YOCO_ERR_WORKSPACE;
    if (yoco::noalloc_scratch(&workspace) != hipSuccess) return YOCO_ERR_HIP;
    workspace_bytes = YOCO_NOALLOC_SCRATCH_BYTES;
  }
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < need) return YOCO_ERR_WORKSPACE;
  AttnParams p = base_params(dims, cache);
  p.q = q;
  p.out = out;
  p.lse = lse;
  p.window = window;
  p.splits = shares;
  p.slots = shares + dims->batch;
  p.head_chunks = head_chunks(dims);
  p.part_o = static_cast<float*>(workspace);
  p.part_ml = reinterpret_cast<float*>(static_cast<char*>(workspace) + decode_ml_offset(dims, shares));
  p.decode_meta = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + decode_meta_offset(dims, shares));
  hipStream_t s = static_cast<hipStream_t>(stream);
  hipError_t err = dims->dtype == YOCO_DTYPE_BF16 ? yoco::launch_decode_split_bf16(p, dims->head_dim, s)
                                                  : yoco::launch_decode_split_f32(p, dims->head_dim, s);
  if (err != hipSuccess) return YOCO_ERR_HIP;
  if (yoco::launch_decode_merge(p, dims->head_dim, dims->dtype, s) != hipSuccess) return YOCO_ERR_HIP;
  return YOCO_OK;
}

}  // namespace

extern "C" {

yoco_status yoco_kv_append(const yoco_dims* dims, const yoco_kv_cache* cache, const void* k_new,
                           const void* v_new, int32_t* overflow_flag, void* stream) {
  return append_impl(dims, cache, k_new, v_new, overflow_flag, 0, stream);
}

yoco_status yoco_kv_append_ring(const yoco_dims* dims, const yoco_kv_cache* cache, const void* k_new,
                                const void* v_new, int32_t* flag, void* stream) {
  return append_impl(dims, cache, k_new, v_new, flag, 1, stream);
}

yoco_status yoco_xattn_prefill(const yoco_dims* dims, const yoco_kv_cache* cache, const void* q,
                               const int32_t* cu_seqlens_q, int32_t max_q_len, int64_t total_q, void* out,
                               float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  return prefill_impl(dims, cache, q, cu_seqlens_q, max_q_len, total_q, 0, out, lse, workspace, workspace_bytes,
                      stream);
}

yoco_status yoco_xattn_prefill_window(const yoco_dims* dims, const yoco_kv_cache* cache, const void* q,
                                      const int32_t* cu_seqlens_q, int32_t max_q_len, int64_t total_q,
                                      int32_t window, void* out, float* lse, void* workspace,
                                      size_t workspace_bytes, void* stream) {
  if (window < 1) return YOCO_ERR_INVALID_ARG;
  return prefill_impl(dims, cache, q, cu_seqlens_q, max_q_len, total_q, window, out, lse, workspace,
                      workspace_bytes, stream);
}

yoco_status yoco_xattn_decode_splits(const yoco_dims* dims, int32_t max_kv_len, int64_t total_kv_len,
                                     int32_t* splits, int32_t* rows_per_split) {
  yoco_status st = check_dims(dims);
  if (st != YOCO_OK) return st;
  if (splits == nullptr || rows_per_split == nullptr || max_kv_len < 0 || total_kv_len < 0) return YOCO_ERR_INVALID_ARG;
  const int32_t shares = decode_shares(dims, max_kv_len, total_kv_len);
  const int64_t blocks = decode_hint_blocks(dims, max_kv_len, total_kv_len);
  *splits = shares;
  *rows_per_split = (int32_t)((blocks + shares - 1) / shares * yoco::kDecodeBlockRows);
  return YOCO_OK;
}

yoco_status yoco_xattn_workspace_size(const yoco_dims* dims, int32_t max_len, int32_t is_decode, size_t* bytes) {
  yoco_status st = check_dims(dims);
  if (st != YOCO_OK) return st;
  if (bytes == nullptr || max_len < 0) return YOCO_ERR_INVALID_ARG;
  if (is_decode)
    *bytes = decode_workspace(dims, decode_shares(dims, max_len, 0));
  else
    *bytes = dims->dtype == YOCO_DTYPE_BF16 ? yoco::kPrefillQueueBytes : 0;
  return YOCO_OK;
}

yoco_status yoco_xattn_decode(const yoco_dims* dims, const yoco_kv_cache* cache, const void* q,
                              int32_t max_kv_len, int64_t total_kv_len, void* out, float* lse, void* workspace,
                              size_t workspace_bytes, void* stream) {
  return decode_impl(dims, cache, q, max_kv_len, total_kv_len, 0, out, lse, workspace, workspace_bytes, stream);
}

yoco_status yoco_xattn_decode_noalloc(const yoco_dims* dims, const yoco_kv_cache* cache, const void* q,
                                      int32_t max_kv_len, int64_t total_kv_len, void* out, float* lse,
                                      void* stream) {
  return decode_impl(dims, cache, q, max_kv_len, total_kv_len, 0, out, lse, nullptr, 0, stream, true);
}

yoco_status yoco_xattn_decode_window(const yoco_dims* dims, const yoco_kv_cache* cache, const void* q,
                                     int32_t max_kv_len, int64_t total_kv_len, int32_t window, void* out,
                                     float* lse, void* workspace, size_t workspace_bytes, void* stream) {
  if (window < 1) return YOCO_ERR_INVALID_ARG;
  return decode_impl(dims, cache, q, max_kv_len, total_kv_len, window, out, lse, workspace, workspace_bytes, stream);
}

yoco_status yoco_kv_project_pack(const yoco_dims* dims, int32_t d_model, const void* gain, const void* w_k,
                                 const void* w_v, void* w_packed, void* stream) {
  yoco_status st = check_dims(dims);
  if (st != YOCO_OK) return st;
  if (dims->dtype != YOCO_DTYPE_BF16) return YOCO_ERR_UNSUPPORTED;
  if (d_model < 64 || d_model % 64 != 0) return YOCO_ERR_UNSUPPORTED;
  if (gain == nullptr || w_k == nullptr || w_v == nullptr || w_packed == nullptr) return YOCO_ERR_INVALID_ARG;
  if (!aligned16(w_packed)) return YOCO_ERR_INVALID_ARG;
  const int hd = dims->num_kv_heads * dims->head_dim;
  if (yoco::launch_kv_pack(gain, w_k, w_v, w_packed, d_model, hd, static_cast<hipStream_t>(stream)) != hipSuccess)
    return YOCO_ERR_HIP;
  return YOCO_OK;
}

yoco_status yoco_kv_project_append(const yoco_dims* dims, const yoco_kv_cache* cache, const void* x,
                                   const int32_t* cu_seqlens, int64_t total_rows, int32_t d_model,
                                   const void* w_packed, float eps, const yoco_kv_residual* residual,
                                   int32_t* overflow_flag, void* stream) {
  yoco_status st = check_dims(dims);
  if (st != YOCO_OK) return st;
  st = check_cache(cache);
  if (st != YOCO_OK) return st;
  if (dims->dtype != YOCO_DTYPE_BF16) return YOCO_ERR_UNSUPPORTED;
  if (d_model < 64 || d_model % 64 != 0 || d_model > (1 << 20)) return YOCO_ERR_UNSUPPORTED;
  if (x == nullptr || cu_seqlens == nullptr || w_packed == nullptr) return YOCO_ERR_INVALID_ARG;
  if (!aligned16(x) || !aligned16(w_packed) || !aligned4(cu_seqlens)) return YOCO_ERR_INVALID_ARG;
  if (overflow_flag != nullptr && !aligned4(overflow_flag)) return YOCO_ERR_INVALID_ARG;
  if (total_rows < 0 || !std::isfinite(eps) || eps < 0.f) return YOCO_ERR_INVALID_ARG;
  if (residual != nullptr) {
    if (residual->k1 == nullptr || residual->v1 == nullptr) return YOCO_ERR_INVALID_ARG;
    if (!std::isfinite(residual->lambda) || !std::isfinite(residual->a_k[0]) || !std::isfinite(residual->a_k[1]) ||
        !std::isfinite(residual->a_v[0]) || !std::isfinite(residual->a_v[1]))
      return YOCO_ERR_INVALID_ARG;
  }
  yoco::ProjectParams p{};
  p.x = x;
  p.w = w_packed;
  p.k = cache->k;
  p.v = cache->v;
  p.seq_start = cache->seq_start;
  p.seq_len = cache->seq_len;
  p.seq_cap = cache->seq_cap;
  p.cu_seqlens = cu_seqlens;
  p.overflow = overflow_flag;
  p.pool_rows = cache->pool_rows;
  p.total_rows = total_rows;
  p.batch = dims->batch;
  p.k_dim = d_model;
  p.n_cols = 2 * dims->num_kv_heads * dims->head_dim;
  p.eps = eps;
  if (residual != nullptr) {
    p.k1 = residual->k1;
    p.v1 = residual->v1;
    p.lam = residual->lambda;
    p.ak1 = residual->a_k[0];
    p.ak2 = residual->a_k[1];
    p.av1 = residual->a_v[0];
    p.av2 = residual->a_v[1];
  }
  if (yoco::launch_kv_project(p, static_cast<hipStream_t>(stream)) != hipSuccess) return YOCO_ERR_HIP;
  return YOCO_OK;
}

}  // extern "C"

namespace {

constexpr int kGretChunk = 256;

yoco_status check_gret(const yoco_gret_dims* d) {
  if (d == nullptr) return YOCO_ERR_INVALID_ARG;
  if (d->batch < 1 || d->num_heads < 1) return YOCO_ERR_INVALID_ARG;
  if (d->dtype != YOCO_DTYPE_BF16) return YOCO_ERR_UNSUPPORTED;
  if (d->head_dim != 64 && d->head_dim != 128) return YOCO_ERR_UNSUPPORTED;
  return YOCO_OK;
}

struct GretWorkspace {
  size_t u_off, s_off, decay_off, total;
};

// Chunks per segment: the largest power of two (at most 64) that still leaves
// one segment per compute unit (256 on MI355X) over all heads, counting the
// rows' chunks; 1 for short inputs.
constexpr int64_t kGretTargetSegs = 256;
int gret_seg_chunks(const yoco_gret_dims* d, int64_t total_rows) {
  const int64_t ch = (total_rows + kGretChunk - 1) / kGretChunk * d->num_heads;
  int seg = 1;
  while (seg < 64 && ch >= kGretTargetSegs * 2 * seg) seg *= 2;
  return seg;
}

// Segment slots per head: every sequence's segments, numbered one after the
// other, fit ceil(chunks / seg) + batch slots whatever the lengths, chunks =
// ceil(total_rows / 256) + batch (each sequence adds at most one partial chunk
// and one partial segment).
int64_t gret_slots(const yoco_gret_dims* d, int64_t total_rows, int seg) {
  const int64_t chunks = (total_rows + kGretChunk - 1) / kGretChunk + d->batch;
  return (chunks + seg - 1) / seg + d->batch;
}

GretWorkspace gret_workspace(const yoco_gret_dims* d, int64_t slots) {
  const size_t per = (size_t)d->num_heads * slots;
  const size_t dd = (size_t)d->head_dim * d->head_dim;
  GretWorkspace w;
  w.u_off = 0;
  w.s_off = (per * dd * 4 + 255) & ~(size_t)255;
  w.decay_off = (w.s_off + per * dd * 4 + 255) & ~(size_t)255;
  w.total = w.decay_off + per * 4;
  return w;
}

// The most slots any call with at most total_rows rows uses (the segment
// length grows with the rows, so fewer rows can need more slots): the reported
// workspace size never shrinks as total_rows grows.
int64_t gret_max_slots(const yoco_gret_dims* d, int64_t total_rows) {
  const int seg = gret_seg_chunks(d, total_rows);
  int64_t most = gret_slots(d, total_rows, seg);
  for (int s = 1; s < seg; s *= 2) {
    // the most rows that still take segments of s chunks
    const int64_t ch_max = kGretTargetSegs * 2 * s - 1;               // chunk count over all heads
    const int64_t rows = ch_max / d->num_heads * kGretChunk;
    const int64_t r = rows < total_rows ? rows : total_rows;
    const int64_t n = gret_slots(d, r, gret_seg_chunks(d, r));
    if (n > most) most = n;
  }
  return most;
}

}  // namespace

extern "C" {

yoco_status yoco_gret_workspace_size(const yoco_gret_dims* dims, int64_t total_rows, size_t* bytes) {
  yoco_status st = check_gret(dims);
  if (st != YOCO_OK) return st;
  if (bytes == nullptr || total_rows < 0) return YOCO_ERR_INVALID_ARG;
  *bytes = gret_workspace(dims, gret_max_slots(dims, total_rows)).total;
  return YOCO_OK;
}

yoco_status yoco_gret_prefill(const yoco_gret_dims* dims, const void* q, const void* k, const void* v,
                              const float* gamma, const int32_t* cu_seqlens, int64_t total_rows,
                              const float* state_in, float* state_out, void* out, void* workspace,
                              size_t workspace_bytes, void* stream) {
  yoco_status st = check_gret(dims);
  if (st != YOCO_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || gamma == nullptr || cu_seqlens == nullptr || out == nullptr)
    return YOCO_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(gamma) ||
      !aligned4(cu_seqlens))
    return YOCO_ERR_INVALID_ARG;
  if ((state_in != nullptr && !aligned16(state_in)) || (state_out != nullptr && !aligned16(state_out)))
    return YOCO_ERR_INVALID_ARG;
  if (total_rows < 0) return YOCO_ERR_INVALID_ARG;
  const int seg = gret_seg_chunks(dims, total_rows);
  const int64_t slots = gret_slots(dims, total_rows, seg);
  if (slots * dims->num_heads > INT32_MAX || dims->num_heads > 65535) return YOCO_ERR_UNSUPPORTED;
  if (total_rows == 0 && state_out == nullptr) return YOCO_OK;   // nothing to compute or pass on
  const GretWorkspace w = gret_workspace(dims, slots);
  if (workspace == nullptr || !aligned16(workspace) || workspace_bytes < w.total) return YOCO_ERR_WORKSPACE;
  yoco::GretParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.gamma = gamma;
  p.out = out;
  p.cu_seqlens = cu_seqlens;
  p.state_in = state_in;
  p.state_out = state_out;
  char* ws = static_cast<char*>(workspace);
  p.seg_u = reinterpret_cast<float*>(ws + w.u_off);
  p.seg_s = reinterpret_cast<float*>(ws + w.s_off);
  p.seg_decay = reinterpret_cast<float*>(ws + w.decay_off);
  p.total_rows = total_rows;
  p.batch = dims->batch;
  p.heads = dims->num_heads;
  p.slots = (int32_t)slots;
  p.seg_chunks = seg;
  if (yoco::launch_gret_prefill(p, dims->head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
    return YOCO_ERR_HIP;
  return YOCO_OK;
}

yoco_status yoco_gret_decode(const yoco_gret_dims* dims, const void* q, const void* k, const void* v,
                             const float* gamma, float* state, void* out, void* stream) {
  yoco_status st = check_gret(dims);
  if (st != YOCO_OK) return st;
  if (q == nullptr || k == nullptr || v == nullptr || gamma == nullptr || state == nullptr || out == nullptr)
    return YOCO_ERR_INVALID_ARG;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(out) || !aligned4(gamma) || !aligned16(state))
    return YOCO_ERR_INVALID_ARG;
  yoco::GretParams p{};
  p.q = q;
  p.k = k;
  p.v = v;
  p.gamma = gamma;
  p.out = out;
  p.state_out = state;
  p.batch = dims->batch;
  p.heads = dims->num_heads;
  if (yoco::launch_gret_decode(p, dims->head_dim, static_cast<hipStream_t>(stream)) != hipSuccess)
    return YOCO_ERR_HIP;
  return YOCO_OK;
}

const char* yoco_status_string(yoco_status status) {
  switch (status) {
    case YOCO_OK: return "ok";
    case YOCO_ERR_INVALID_ARG: return "invalid argument";
    case YOCO_ERR_UNSUPPORTED: return "unsupported dtype or head_dim";
    case YOCO_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case YOCO_ERR_HIP: return "HIP launch failed";
  }
  return "unknown status";
}

}  // extern "C"
