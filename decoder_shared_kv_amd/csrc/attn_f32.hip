// fp32 storage path: plain VALU kernels for prefill and the decode split pass.
//
// Same operation as the bf16 kernels (page "YOCO", section "Cross-Decoder",
// Attn_l equation, causal mask j <= i), in true fp32 arithmetic throughout so
// that fp32 inputs keep fp32 accuracy. One thread owns one query row (prefill)
// or one (share of the rows, head) pair (decode) and keeps a running max, a
// running sum of weights and an unnormalised output vector (online softmax in
// the base-2 domain: exp(s*scale) = exp2(s*scale*log2 e)).
#include "internal.h"

namespace yoco {

namespace {

template <int D>
__device__ __forceinline__ float dot_row(const float* qr, const float* kr) {
  const float4* k4 = reinterpret_cast<const float4*>(kr);
  float acc = 0.f;
#pragma unroll
  for (int i = 0; i < D / 4; ++i) {
    float4 kv = k4[i];
    acc = fmaf(qr[4 * i + 0], kv.x, acc);
    acc = fmaf(qr[4 * i + 1], kv.y, acc);
    acc = fmaf(qr[4 * i + 2], kv.z, acc);
    acc = fmaf(qr[4 * i + 3], kv.w, acc);
  }
  return acc;
}

// Online-softmax accumulation over rows [j0, j1) of one KV head.
template <int D>
__device__ __forceinline__ void accumulate_rows(const float* qr, const float* kbase, const float* vbase,
                                                int64_t row_stride, int j0, int j1, float scale_log2,
                                                float& m, float& l, float* acc) {
  for (int j = j0; j < j1; ++j) {
    const float t = dot_row<D>(qr, kbase + (int64_t)j * row_stride) * scale_log2;
    const float m_new = fmaxf(m, t);
    const float alpha = exp2f(m - m_new);  // m == -inf on the first row: alpha = 0
    const float w = exp2f(t - m_new);
    l = l * alpha + w;
    const float4* v4 = reinterpret_cast<const float4*>(vbase + (int64_t)j * row_stride);
#pragma unroll
    for (int i = 0; i < D / 4; ++i) {
      float4 vv = v4[i];
      acc[4 * i + 0] = fmaf(w, vv.x, acc[4 * i + 0] * alpha);
      acc[4 * i + 1] = fmaf(w, vv.y, acc[4 * i + 1] * alpha);
      acc[4 * i + 2] = fmaf(w, vv.z, acc[4 * i + 2] * alpha);
      acc[4 * i + 3] = fmaf(w, vv.w, acc[4 * i + 3] * alpha);
    }
    m = m_new;
  }
}

template <int D>
__global__ __launch_bounds__(kPrefillF32Rows) void prefill_f32_kernel(AttnParams p) {
  const int bh_count = p.batch * p.hq;
  const int bh = blockIdx.x % bh_count;
  const int rank = blockIdx.x / bh_count;
  const int b = bh / p.hq;
  const int h = bh % p.hq;
  const int kh = h / p.group;
  int64_t start;
  const int32_t n_kv = readable_rows(p.seq_start, p.seq_len, p.seq_cap, p.pool_rows, b, &start);
  int64_t q0 = p.cu_seqlens[b];
  int64_t q1 = p.cu_seqlens[b + 1];
  if (q1 > p.total_q) q1 = p.total_q;
  if (q0 < 0 || q0 > q1) return;
  const int32_t n_q = (int32_t)(q1 - q0);
  const int32_t offset = n_kv > n_q ? n_kv - n_q : 0;
  const int64_t row_stride = (int64_t)p.hkv * D;
  const float* kbase = static_cast<const float*>(p.k) + start * row_stride + (int64_t)kh * D;
  const float* vbase = static_cast<const float*>(p.v) + start * row_stride + (int64_t)kh * D;
  // longest position blocks first; later passes cover sequences longer than the grid
  for (int pb = p.pos_blocks - 1 - rank; pb >= 0 && pb * kPrefillF32Rows < n_q; pb += p.pos_blocks) {
    const int r = pb * kPrefillF32Rows + threadIdx.x;
    if (r >= n_q) continue;
    const int64_t qrow = q0 + r;
    const float* qsrc = static_cast<const float*>(p.q) + (qrow * p.hq + h) * D;
    float qr[D];
#pragma unroll
    for (int i = 0; i < D; ++i) qr[i] = qsrc[i];
    float acc[D];
#pragma unroll
    for (int i = 0; i < D; ++i) acc[i] = 0.f;
    float m = -INFINITY, l = 0.f;
    // a row whose position has no cache row of its own (more query rows than
    // cache rows) sees no rows: O = 0, LSE = -inf
    int vis = r + offset + 1;
    if (vis > n_kv) vis = 0;
    // sliding window: rows vis - window .. vis - 1 only
    const int lo = p.window > 0 && vis > p.window ? vis - p.window : 0;
    accumulate_rows<D>(qr, kbase, vbase, row_stride, lo, vis, p.scale_log2, m, l, acc);
    float* dst = static_cast<float*>(p.out) + (qrow * p.hq + h) * D;
    const float inv = l > 0.f ? 1.f / l : 0.f;
#pragma unroll
    for (int i = 0; i < D; ++i) dst[i] = acc[i] * inv;
    if (p.lse != nullptr)
      p.lse[(int64_t)h * p.total_q + qrow] = l > 0.f ? (m + log2f(l)) * 0.6931471805599453f : -INFINITY;
  }
}

// One thread per (share, query head): the share's rows of every sequence it
// spans, one partial (m, l, unnormalised O) per piece, in slot share + sequence
// (the balanced split of the bf16 decode kernel, walked sequentially).
template <int D>
__global__ __launch_bounds__(64) void decode_split_f32_kernel(AttnParams p) {
  const int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= (int64_t)p.splits * p.hq) return;
  const int share = (int)(t % p.splits);
  const int h = (int)(t / p.splits);
  const int kh = h / p.group;
  int64_t total = 0;
  for (int b = 0; b < p.batch; ++b) {
    int64_t st;
    total += decode_blocks(decode_rows(p, b, &st));
  }
  const int parts = total < p.splits ? (int)total : p.splits;
  if (share >= parts) return;
  const int64_t first = share_begin(share, total, parts);
  const int64_t last = share_begin(share + 1, total, parts);
  const int64_t row_stride = (int64_t)p.hkv * D;
  int64_t pre = 0;
  for (int b = 0; b < p.batch && pre < last; ++b) {
    int64_t start;
    const int32_t n_kv = decode_rows(p, b, &start);
    const int u = decode_blocks(n_kv);
    if (u > 0 && pre + u > first) {
      const int64_t lo = (first > pre ? first : pre) - pre;
      const int64_t hi = (last < pre + u ? last : pre + u) - pre;
      if (lo == 0 && h == 0) {
        p.decode_meta[2 * b + 0] = share + b;
        p.decode_meta[2 * b + 1] = (int32_t)(share_of_block(pre + u - 1, total, parts) - share + 1);
      }
      const int j0 = (int)(lo * kDecodeBlockRows);
      const int j1 = hi * kDecodeBlockRows < n_kv ? (int)(hi * kDecodeBlockRows) : n_kv;
      const float* kbase = static_cast<const float*>(p.k) + start * row_stride + (int64_t)kh * D;
      const float* vbase = static_cast<const float*>(p.v) + start * row_stride + (int64_t)kh * D;
      const float* qsrc = static_cast<const float*>(p.q) + ((int64_t)b * p.hq + h) * D;
      float qr[D];
#pragma unroll
      for (int i = 0; i < D; ++i) qr[i] = qsrc[i];
      float acc[D];
#pragma unroll
      for (int i = 0; i < D; ++i) acc[i] = 0.f;
      float m = -INFINITY, l = 0.f;
      accumulate_rows<D>(qr, kbase, vbase, row_stride, j0, j1, p.scale_log2, m, l, acc);
      const int64_t ps = (int64_t)h * p.slots + share + b;
      float* po = p.part_o + ps * D;
#pragma unroll
      for (int i = 0; i < D; ++i) po[i] = acc[i];
      p.part_ml[2 * ps + 0] = m;
      p.part_ml[2 * ps + 1] = l;
    }
    pre += u;
  }
}

}  // namespace

hipError_t launch_prefill_f32(const AttnParams& p, int head_dim, int grid, hipStream_t stream) {
  if (head_dim == 64)
    hipLaunchKernelGGL(prefill_f32_kernel<64>, dim3(grid), dim3(kPrefillF32Rows), 0, stream, p);
  else
    hipLaunchKernelGGL(prefill_f32_kernel<128>, dim3(grid), dim3(kPrefillF32Rows), 0, stream, p);
  return hipGetLastError();
}

hipError_t launch_decode_split_f32(const AttnParams& p, int head_dim, hipStream_t stream) {
  const int64_t total = (int64_t)p.splits * p.hq;
  const dim3 grid((unsigned)((total + 63) / 64));
  if (head_dim == 64)
    hipLaunchKernelGGL(decode_split_f32_kernel<64>, grid, dim3(64), 0, stream, p);
  else
    hipLaunchKernelGGL(decode_split_f32_kernel<128>, grid, dim3(64), 0, stream, p);
  return hipGetLastError();
}

}  // namespace yoco
