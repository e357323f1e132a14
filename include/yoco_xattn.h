/*
 * yoco_xattn.h -- C ABI of the shared-KV cross-attention library for MI355X (gfx950).
 *
 * The operation: YOCO's Cross-Decoder layers each send their own queries Q^l
 * against ONE shared pair K^, V^ that the Self-Decoder output produced once
 * (page "YOCO", zdszero.github.io: section "架构总览" (architecture overview),
 * equations for K^, V^ and Q^l; section "Cross-Decoder：共享 KV，但不共享 Query",
 * the Attn_l equation):
 *
 *     Attn_l = softmax(Q^l K^T * scale + M_causal) V^
 *
 * M_causal lets the query at position i see cache rows j <= i (same page, end of
 * "架构总览"). Several query heads share one KV head (page "YOCO 深度技术分析",
 * liuhc.cn, section 2.1, Cross-Decoder bullets): query head h reads KV head
 * h / (Hq / Hkv). No positional transform is applied inside these calls.
 *
 * Conventions shared by every call
 * --------------------------------
 *  - Pointers marked [device] are device (HBM) addresses; [host] are host memory.
 *  - Tensors are dense, row-major, head_dim contiguous:
 *      shared cache  K, V   : [pool_rows, Hkv, head_dim]
 *      prefill queries/out  : [total_q, Hq, head_dim], sequences packed back to back
 *      decode queries/out   : [batch, Hq, head_dim]
 *  - Q, K, V, O share one storage dtype (fp32 or bf16); scores, softmax and
 *    accumulation are fp32; O is rounded once (round-to-nearest-even) on store.
 *    LSE (natural log of the sum of exp of the scaled scores) is fp32.
 *  - Every call is asynchronous on `stream` (a hipStream_t, NULL = the null
 *    stream); nothing is synchronised inside the library. Host-side argument
 *    checks run before any launch: a call that returns an error launched
 *    nothing and touched no output.
 *  - The library allocates and frees nothing and keeps no global state: all
 *    buffers belong to the caller. Calls are re-entrant. The one exception is
 *    yoco_xattn_decode_noalloc, whose partials live in a device-resident
 *    scratch array of the library (one per GPU).
 *  - Device-side sequence metadata is clamped, never trusted, for memory
 *    safety: a sequence's readable rows are seq_start[b] .. seq_start[b] +
 *    min(seq_len[b], seq_cap[b]) - 1, further limited to the pool. Metadata
 *    outside these limits yields clamped results, never an out-of-bounds access.
 *  - Pointers to Q, K, V, O and the appended rows must be 16-byte aligned.
 */
#ifndef YOCO_XATTN_H
#define YOCO_XATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  YOCO_OK = 0,
  YOCO_ERR_INVALID_ARG = 1,  /* null/misaligned pointer, bad size or count */
  YOCO_ERR_UNSUPPORTED = 2,  /* valid but not built: dtype, head_dim */
  YOCO_ERR_WORKSPACE = 3,    /* workspace missing or smaller than yoco_xattn_workspace_size */
  YOCO_ERR_HIP = 4           /* a kernel launch failed (hipGetLastError after launch) */
} yoco_status;

typedef enum { YOCO_DTYPE_F32 = 0, YOCO_DTYPE_BF16 = 1 } yoco_dtype;

/* [host] Problem dimensions. */
typedef struct {
  int32_t batch;         /* B >= 1: sequences */
  int32_t num_q_heads;   /* Hq >= 1 */
  int32_t num_kv_heads;  /* Hkv >= 1, Hq % Hkv == 0 */
  int32_t head_dim;      /* 64 or 128 */
  int32_t dtype;         /* yoco_dtype of Q, K, V, O */
  float scale;           /* softmax scale, finite and > 0; 1/sqrt(head_dim) for the usual d_k reading */
} yoco_dims;

/* [host] Descriptor of the ONE shared K^,V^ cache read by every layer. */
typedef struct {
  void* k;                   /* [device] [pool_rows, Hkv, head_dim] */
  void* v;                   /* [device] same layout as k */
  int64_t pool_rows;         /* rows allocated in k and v (bounds every access) */
  const int64_t* seq_start;  /* [device] [B] first pool row of sequence b */
  int32_t* seq_len;          /* [device] [B] valid rows of sequence b (kv_append increments) */
  const int32_t* seq_cap;    /* [device] [B] rows reserved for sequence b */
} yoco_kv_cache;

/*
 * yoco_kv_append -- write each sequence's new K^,V^ row into the shared cache.
 *
 * Decode order on the pages: the new token passes the Self-Decoder, which yields
 * its K^,V^ row, before any Cross-Decoder layer reads the cache (page "YOCO",
 * section "Decode：新 token 仍需经过两部分"). For each b: if seq_len[b] <
 * seq_cap[b] (and the row lies inside the pool) the row k_new[b], v_new[b] is
 * copied to pool row seq_start[b] + seq_len[b] and seq_len[b] is incremented;
 * otherwise nothing of sequence b changes and *overflow_flag is set to 1 (the
 * flag is never cleared by the library; NULL disables it).
 *   k_new, v_new  [device] [B, Hkv, head_dim], same dtype as the cache.
 */
yoco_status yoco_kv_append(const yoco_dims* dims, const yoco_kv_cache* cache,
                           const void* k_new, const void* v_new,
                           int32_t* overflow_flag, void* stream);

/*
 * yoco_xattn_prefill -- causal cross-attention of every packed query row.
 *
 * Sequence b's queries are packed rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1 of
 * q. With n = its readable cache rows and m = its query rows, query row r sits
 * at position r + max(n - m, 0) (r itself when m == n, the full-prompt case)
 * and attends rows 0 .. that position. A query row whose position is n or
 * later (more query rows than readable rows, n == 0 included) has no K^,V^ row
 * of its own in the cache: a token's row is written before any Cross-Decoder
 * layer reads (page "YOCO", section "Decode：新 token 仍需经过两部分"), so no
 * attention is defined for it, and it gets the empty key set's result,
 * O = 0 and LSE = -inf.
 *   q          [device] [total_q, Hq, head_dim]
 *   cu_seqlens_q [device] int32 [B+1], non-decreasing, cu_seqlens_q[B] <= total_q
 *   max_q_len  [host] sizing hint for the grid (longer sequences are still
 *              computed in full, by more passes)
 *   total_q    [host] rows of q, out and columns of lse
 *   out        [device] [total_q, Hq, head_dim]
 *   lse        [device] fp32 [Hq, total_q] or NULL
 *   workspace  [device] the bf16 kernels' work queue: >=
 *              yoco_xattn_workspace_size(dims, max_q_len, 0) bytes (2 KB),
 *              16-byte aligned, ALL ZERO before its first use (allocate it
 *              zeroed); every call that completes leaves it zero again (the
 *              last workgroup resets the counters), so it is reused as is.
 *              Calls that share it must be serialised, and it must not be
 *              shared with a decode call (whose partials would overwrite it)
 *              unless zeroed again. With a queue, one persistent workgroup per
 *              CU takes (KV group, position block) items from per-XCD queues
 *              and takes over other XCDs' items when its own run out, so no
 *              XCD waits for a slower one at the end. NULL: the static grid
 *              (one workgroup per item), same results. fp32 ignores it.
 * YOCO_ERR_WORKSPACE: workspace misaligned or smaller than needed.
 */
yoco_status yoco_xattn_prefill(const yoco_dims* dims, const yoco_kv_cache* cache,
                               const void* q, const int32_t* cu_seqlens_q,
                               int32_t max_q_len, int64_t total_q,
                               void* out, float* lse,
                               void* workspace, size_t workspace_bytes, void* stream);

/*
 * yoco_xattn_decode -- one query per sequence against the whole shared cache.
 *
 * Call after yoco_kv_append: sequence b's query sits at position seq_len[b]-1
 * and attends rows 0 .. seq_len[b]-1 (every Cross-Decoder layer re-reads the
 * shared cache: page "YOCO", section "KV Cache 与计算量分析", cost table).
 * Rows are split across workgroups (split-K) and merged by log-sum-exp: the
 * 128-row blocks of all sequences together are cut into equal shares, one per
 * workgroup of each KV head (a share may span several sequences), so every
 * workgroup reads the same number of rows whatever the mix of lengths.
 *   q          [device] [B, Hq, head_dim]
 *   max_kv_len [host] sizing hint for the split plan: the longest sequence's
 *              rows; the kernels count the rows on the device, so every row is
 *              computed whatever the hints say
 *   total_kv_len [host] sizing hint: the rows of all sequences together, or 0
 *              for B * max_kv_len (values above B * max_kv_len count as that);
 *              the number of shares follows it (at most 512 or 1024 workgroups)
 *   out        [device] [B, Hq, head_dim]; a sequence with no rows gets O = 0
 *   lse        [device] fp32 [B, Hq] or NULL; -inf for a sequence with no rows
 *   workspace  [device] >= yoco_xattn_workspace_size(dims, max_kv_len, 1) bytes,
 *              16-byte aligned; contents need no initialisation and are
 *              overwritten. Calls that share a workspace must be serialised.
 */
yoco_status yoco_xattn_decode(const yoco_dims* dims, const yoco_kv_cache* cache,
                              const void* q, int32_t max_kv_len, int64_t total_kv_len,
                              void* out, float* lse,
                              void* workspace, size_t workspace_bytes, void* stream);

/* Bytes of the device-resident scratch yoco_xattn_decode_noalloc uses on each GPU. */
#define YOCO_NOALLOC_SCRATCH_BYTES (8u << 20)

/*
 * yoco_xattn_decode_noalloc -- yoco_xattn_decode without a workspace, for
 * callers that cannot allocate device memory: code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc. Same operation,
 * arguments, kernels and results as yoco_xattn_decode; the split-K partials
 * go to a scratch array of YOCO_NOALLOC_SCRATCH_BYTES that the library holds
 * on each GPU it runs on until the process ends (its device address is looked
 * up on the first call on that device, which must be the current device of
 * the calling thread). Calls whose plan needs more partial space than that
 * (yoco_xattn_workspace_size(dims, max_kv_len, 1) > YOCO_NOALLOC_SCRATCH_BYTES,
 * e.g. hundreds of sequences) return YOCO_ERR_WORKSPACE and launch nothing.
 * The call allocates and frees nothing (no hipMalloc, no library allocator).
 * Every call on one GPU shares that GPU's scratch, which keeps the last call's
 * contents (nothing in it needs to start at zero): calls that may overlap on
 * one GPU (different streams, or different threads) race and must be
 * serialised by the caller. YOCO_ERR_HIP if the device or the scratch address
 * cannot be obtained.
 */
yoco_status yoco_xattn_decode_noalloc(const yoco_dims* dims, const yoco_kv_cache* cache,
                                      const void* q, int32_t max_kv_len, int64_t total_kv_len,
                                      void* out, float* lse, void* stream);

/*
 * Sliding-window attention (the Self-Decoder's efficient attention)
 * -----------------------------------------------------------------
 * The current position sees only the tokens of a fixed window of size C, so a
 * layer's decode cache is O(C) rather than O(N) (page "YOCO", section
 * "Self-Decoder：把历史编码成可复用的全局表示"; page "YOCO 深度技术分析", section
 * 2.3, C = 1024). Reading: a window of size C holds the C most recent positions,
 * the query's own included: position p attends rows max(0, p - C + 1) .. p.
 * Here the cache descriptor describes one layer's K, V; everything else is as
 * in the calls above.
 */

/*
 * yoco_xattn_prefill_window -- yoco_xattn_prefill with the band mask: query row
 * r at position p (as in yoco_xattn_prefill) attends rows max(0, p - window + 1)
 * .. p. window >= 1 (YOCO_ERR_INVALID_ARG otherwise); a window of at least the
 * sequence length gives yoco_xattn_prefill's result. Tiles wholly outside every
 * row's window are neither loaded nor computed. Workspace as for
 * yoco_xattn_prefill.
 */
yoco_status yoco_xattn_prefill_window(const yoco_dims* dims, const yoco_kv_cache* cache,
                                      const void* q, const int32_t* cu_seqlens_q,
                                      int32_t max_q_len, int64_t total_q, int32_t window,
                                      void* out, float* lse,
                                      void* workspace, size_t workspace_bytes, void* stream);

/*
 * yoco_xattn_decode_window -- yoco_xattn_decode over a full (linear) cache with
 * the band mask: the query at position seq_len[b]-1 attends the last
 * min(seq_len[b], window) readable rows only; only those are read. window >= 1.
 * Workspace as for yoco_xattn_decode with the same max_kv_len.
 */
yoco_status yoco_xattn_decode_window(const yoco_dims* dims, const yoco_kv_cache* cache,
                                     const void* q, int32_t max_kv_len, int64_t total_kv_len,
                                     int32_t window, void* out, float* lse,
                                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * yoco_kv_append_ring -- append to ring window caches (decode cache of a window
 * of C = seq_cap[b] positions). Sequence b's row goes to pool row seq_start[b] +
 * (seq_len[b] mod seq_cap[b]), replacing the token C positions older, and
 * seq_len[b] (which counts every token appended so far) is incremented. A
 * sequence with seq_cap[b] <= 0 (or whose slot lies outside the pool) stores
 * nothing and sets *flag to 1 (never cleared; NULL disables it).
 * Decode over a ring is plain yoco_xattn_decode on the same descriptor: its
 * readable rows min(seq_len, seq_cap) are exactly the last C tokens (in rotated
 * slot order, which softmax attention does not depend on); pass max_kv_len =
 * the largest seq_cap.
 *   k_new, v_new  [device] [B, Hkv, head_dim], same dtype as the cache.
 */
yoco_status yoco_kv_append_ring(const yoco_dims* dims, const yoco_kv_cache* cache,
                                const void* k_new, const void* v_new,
                                int32_t* flag, void* stream);

/*
 * The shared cache's producer (bf16 only)
 * ---------------------------------------
 * The Self-Decoder output X^{L/2} is normalised and projected once into the
 * global pair K^ = LN(X) W_K, V^ = LN(X) W_V (page "YOCO", section "架构总览",
 * the K^, V^ equations), LN being RMSNorm (xingfushuangcheng.com explainer of
 * YOCO, section "自解码器"): y = x / sqrt(mean(x^2) + eps) * gain. The rows go
 * straight into each sequence's rows of the shared cache.
 */

/*
 * yoco_kv_project_pack -- prepack the projection once per model:
 * w_packed[n][k] = gain[k] * W[k][n] rounded to bf16, for n < Hkv*head_dim from
 * W_K and after that from W_V (the gain folds into the weights because 1/rms is
 * a per-row factor).
 *   gain      [device] bf16 [d_model]
 *   w_k, w_v  [device] bf16 [d_model, Hkv * head_dim] (row-major: x @ W)
 *   w_packed  [device] bf16 [2 * Hkv * head_dim, d_model] (caller-owned,
 *             2 * Hkv * head_dim * d_model * 2 bytes), 16-byte aligned
 * d_model must be a positive multiple of 64 (YOCO_ERR_UNSUPPORTED otherwise).
 */
yoco_status yoco_kv_project_pack(const yoco_dims* dims, int32_t d_model, const void* gain,
                                 const void* w_k, const void* w_v, void* w_packed, void* stream);

/* [host] YOCO++ residual with the bottom layer's rows (gist.science explainer of
 * YOCO++ (2604.13556), sections 2.1 and 2.2): K' = lambda (a_k[0] K_1 + a_k[1] K^),
 * V' = lambda (a_v[0] V_1 + a_v[1] V^); the pages fix lambda = 35 and start
 * from a[0] = 0, a[1] = 1/lambda (which gives YOCO's rows). The combined rows are
 * what the cache holds, so decode reads no more than YOCO. */
typedef struct {
  const void* k1;            /* [device] bf16 [total_rows, Hkv * head_dim], bottom-layer K rows */
  const void* v1;            /* [device] bf16 [total_rows, Hkv * head_dim] */
  float lambda;
  float a_k[2];
  float a_v[2];
} yoco_kv_residual;

/*
 * yoco_kv_project_append -- K^, V^ of the packed rows x and their append to the
 * shared cache in one GEMM (MFMA) with the RMSNorm and the optional YOCO++
 * combine in its epilogue. Sequence b owns rows cu_seqlens[b] .. cu_seqlens[b+1]-1
 * of x; its i-th row lands at pool row seq_start[b] + seq_len[b] + i, and then
 * seq_len[b] grows by its row count (one row per sequence is the per-token
 * append after the Self-Decoder; a whole prompt, the prefill). A sequence whose
 * rows do not all fit seq_cap[b] (or the pool) is left untouched and sets
 * *overflow_flag to 1 (never cleared; NULL disables it).
 *   x          [device] bf16 [total_rows, d_model]
 *   cu_seqlens [device] int32 [B+1], non-decreasing
 *   w_packed   [device] from yoco_kv_project_pack with the same dims and d_model
 *   eps        RMSNorm epsilon, finite and >= 0
 *   residual   [host] YOCO++ combine or NULL
 * The normalised rows are not rounded before the product; scores of the GEMM
 * accumulate in fp32 and each cache element is rounded once to bf16.
 */
yoco_status yoco_kv_project_append(const yoco_dims* dims, const yoco_kv_cache* cache,
                                   const void* x, const int32_t* cu_seqlens, int64_t total_rows,
                                   int32_t d_model, const void* w_packed, float eps,
                                   const yoco_kv_residual* residual, int32_t* overflow_flag,
                                   void* stream);

/*
 * Gated retention (gRet), the Self-Decoder's default attention
 * -------------------------------------------------------------
 * Page "YOCO 深度技术分析", section 2.2 (three equivalent forms) and 5.3.2
 * (chunkwise for prefill, chunk size 256; recurrent for decode):
 *   parallel   O = (Q K^T ⊙ D) V,  D[n][m] = γ_{m+1} γ_{m+2} ... γ_n (m <= n), 0 (m > n)
 *   recurrent  S_n = γ_n S_{n-1} + K_n^T V_n,  o_n = Q_n S_n
 * Q and K come already multiplied by the caller's Θ; γ is one gate per token
 * and head (the head-wise γ = sigmoid(X W_γ)^(1/τ)), in (0, 1]; a gate below
 * 2^-126 counts as 2^-126. No scale, no normalisation inside (GroupNorm and the
 * swish gate are outside). Layouts: q, k, v, out [T, H, head_dim] bf16 (one head
 * dim for K and V); gamma [T, H] fp32; states [B, H, head_dim (k), head_dim (v)]
 * fp32, the recurrent form's S. Products are bf16 MFMA with fp32 accumulation;
 * the state recurrence is fp32; outputs are rounded once to bf16.
 */
typedef struct {
  int32_t batch;       /* B >= 1 */
  int32_t num_heads;   /* H >= 1 */
  int32_t head_dim;    /* d_k = d_v, 64 or 128 */
  int32_t dtype;       /* YOCO_DTYPE_BF16 (fp32 storage: YOCO_ERR_UNSUPPORTED) */
} yoco_gret_dims;

/* [host] Workspace bytes of yoco_gret_prefill for total_rows packed rows (any
 * number of sequences up to dims->batch, any lengths): per head and segment
 * slot two fp32 head_dim^2 states (the segment's contribution and its incoming
 * state) and one fp32 decay. A segment is a run of consecutive 256-row chunks
 * of one sequence (1 to 64 chunks, more as the rows grow); the size covers
 * every call with at most total_rows rows, so it never shrinks as total_rows
 * grows. */
yoco_status yoco_gret_workspace_size(const yoco_gret_dims* dims, int64_t total_rows, size_t* bytes);

/*
 * yoco_gret_prefill -- the chunkwise form over packed sequences: sequence b owns
 * rows cu_seqlens[b] .. cu_seqlens[b+1]-1 (clamped to total_rows). Three
 * launches: per-segment state contributions, the state recurrence across
 * segments, and the outputs, each segment's chunks in turn with the state
 * carried from chunk to chunk. The segments of all sequences are numbered one
 * after the other and found on the device, so every row of every sequence is
 * computed whatever the lengths; cu_seqlens must be non-decreasing (otherwise
 * segments beyond the workspace's slots are left out, never written out of
 * bounds).
 *   total_rows [host] rows of q, k, v, gamma and out
 *   state_in   [device] [B, H, d, d] fp32 initial states, or NULL for zero
 *   state_out  [device] [B, H, d, d] fp32 states after each sequence's last row,
 *              or NULL; may be the same buffer as state_in
 *   workspace  [device] >= yoco_gret_workspace_size(dims, total_rows), 16-byte
 *              aligned; needs no initialisation; serialise calls that share it
 */
yoco_status yoco_gret_prefill(const yoco_gret_dims* dims, const void* q, const void* k, const void* v,
                              const float* gamma, const int32_t* cu_seqlens, int64_t total_rows,
                              const float* state_in, float* state_out, void* out,
                              void* workspace, size_t workspace_bytes, void* stream);

/*
 * yoco_gret_decode -- one recurrent step per sequence and head: q, k, v
 * [B, H, d] bf16, gamma [B, H] fp32; state [B, H, d, d] fp32 is updated in
 * place (S = γ S + k^T v) and out [B, H, d] bf16 gets q S.
 */
yoco_status yoco_gret_decode(const yoco_gret_dims* dims, const void* q, const void* k, const void* v,
                             const float* gamma, float* state, void* out, void* stream);

/* [host] Workspace bytes of a call. is_decode != 0: yoco_xattn_decode (and
 * yoco_xattn_decode_window) with this max_kv_len (any total_kv_len, any smaller
 * max_kv_len): per query head one fp32 partial (head_dim + 2 values) per share
 * and sequence, and two int32 per sequence. is_decode == 0: yoco_xattn_prefill
 * (and _window) with any max_q_len: the work queue's counters, 2 KB for bf16,
 * 0 for fp32. */
yoco_status yoco_xattn_workspace_size(const yoco_dims* dims, int32_t max_len, int32_t is_decode,
                                      size_t* bytes);

/* [host] The split plan yoco_xattn_decode uses (for reports and tests):
 * *splits = shares per KV head (bf16) or per query head (fp32),
 * *rows_per_split = rows of one share for rows as the hints describe them. */
yoco_status yoco_xattn_decode_splits(const yoco_dims* dims, int32_t max_kv_len,
                                     int64_t total_kv_len, int32_t* splits,
                                     int32_t* rows_per_split);

/* Static description of a status code; never NULL. */
const char* yoco_status_string(yoco_status status);

#ifdef __cplusplus
}
#endif

#endif /* YOCO_XATTN_H */
