// Decode merge: combine the partial softmax states of one query.
//
// Each piece s of a sequence's rows (one share of the balanced split) left
// (m_s, l_s, O_s): its running max of the base-2 scores, its sum of weights
// exp2(t - m_s) and its unnormalised weighted sum of V rows. The exact softmax
// over all rows is then
//   M = max_s m_s,  L = sum_s l_s exp2(m_s - M),  O = sum_s O_s exp2(m_s - M) / L,
// and LSE = (M + log2 L) ln 2. The pieces of sequence b sit in consecutive
// slots, which the split pass recorded (first slot, count); a sequence with no
// rows gets O = 0 and LSE = -inf.
#include <hip/hip_bf16.h>

#include "internal.h"

namespace yoco {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kMergeDims = 16;                            // dims per workgroup
constexpr int kMergeGroups = kMergeThreads / kMergeDims;  // piece groups per workgroup

// One workgroup per (sequence, query head, 16-dim chunk): many workgroups even
// for one long sequence. The pieces' maxima are reduced by the whole workgroup;
// then 16 groups of 16 threads each sum a strided subset of the pieces (with
// independent loads in flight), and the groups are added in LDS.
template <int D, typename OutT>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(AttnParams p) {
  __shared__ float red[kMergeThreads / 64];
  __shared__ float part_o[kMergeGroups][kMergeDims];
  __shared__ float part_l[kMergeGroups];
  const int bh = blockIdx.x;  // b * hq + h
  const int b = bh / p.hq;
  const int h = bh % p.hq;
  const int d0 = blockIdx.y * kMergeDims;
  const int tid = threadIdx.x;
  // the sequence's rows and where the split pass left its pieces (loaded together)
  int64_t start;
  const int32_t n = decode_rows(p, b, &start);
  const int32_t s0 = p.decode_meta[2 * b + 0];
  int pieces = p.decode_meta[2 * b + 1];
  if (n == 0 || s0 < 0 || pieces < 1 || (int64_t)s0 + pieces > p.slots) pieces = 0;   // (stale when n == 0)
  const int64_t base = (int64_t)h * p.slots + (pieces > 0 ? s0 : 0);
  const float* ml = p.part_ml + 2 * base;

  float mx = -INFINITY;
  for (int s = tid; s < pieces; s += kMergeThreads) mx = fmaxf(mx, ml[2 * s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mx = fmaxf(mx, __shfl_xor(mx, off));
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  float M = red[0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red[w]);

  const int g = tid / kMergeDims;
  const int d = tid % kMergeDims;
  float o = 0.f, lsum = 0.f;
  if (M != -INFINITY) {
    const float* po = p.part_o + base * D + d0 + d;
#pragma unroll 8
    for (int s = g; s < pieces; s += kMergeGroups) {
      const float ms = ml[2 * s];
      const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
      lsum = fmaf(ml[2 * s + 1], w, lsum);
      o = fmaf(po[(int64_t)s * D], w, o);
    }
  }
  part_o[g][d] = o;
  if (d == 0) part_l[g] = lsum;
  __syncthreads();
  if (tid < kMergeDims) {
    float os = 0.f, ls = 0.f;
#pragma unroll
    for (int i = 0; i < kMergeGroups; ++i) {
      os += part_o[i][tid];
      ls += part_l[i];
    }
    const float res = ls > 0.f ? os / ls : 0.f;
    OutT* dst = static_cast<OutT*>(p.out) + (int64_t)bh * D + d0 + tid;
    if constexpr (sizeof(OutT) == 2) {
      *dst = __float2bfloat16(res);
    } else {
      *dst = res;
    }
    if (tid == 0 && blockIdx.y == 0 && p.lse != nullptr)
      p.lse[bh] = ls > 0.f ? (M + log2f(ls)) * 0.6931471805599453f : -INFINITY;
  }
}

}  // namespace

hipError_t launch_decode_merge(const AttnParams& p, int head_dim, int dtype, hipStream_t stream) {
  const dim3 grid((unsigned)(p.batch * p.hq), (unsigned)(head_dim / kMergeDims));
  const dim3 block(kMergeThreads);
  if (dtype == 1) {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_merge_kernel<64, __hip_bfloat16>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<128, __hip_bfloat16>), grid, block, 0, stream, p);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_merge_kernel<64, float>), grid, block, 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<128, float>), grid, block, 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace yoco
