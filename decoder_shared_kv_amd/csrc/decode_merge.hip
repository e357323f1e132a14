// Decode merge: combine the per-split partial softmax states of one query.
//
// Each split s of the shared-cache rows left (m_s, l_s, O_s): its running max
// of the base-2 scores, its sum of weights exp2(t - m_s) and its unnormalised
// weighted sum of V rows. The exact softmax over all rows is then
//   M = max_s m_s,  L = sum_s l_s exp2(m_s - M),  O = sum_s O_s exp2(m_s - M) / L,
// and LSE = (M + log2 L) ln 2. Splits with no rows carry m_s = -inf and weigh 0.
#include <hip/hip_bf16.h>

#include "internal.h"

namespace yoco {

namespace {

template <int D, typename OutT>
__global__ __launch_bounds__(D) void decode_merge_kernel(AttnParams p) {
  const int bh = blockIdx.x;  // b * hq + h
  const int d = threadIdx.x;
  const int64_t base = (int64_t)bh * p.splits;
  const float* ml = p.part_ml + 2 * base;
  float mx = -INFINITY;
  for (int s = 0; s < p.splits; ++s) mx = fmaxf(mx, ml[2 * s]);
  float lsum = 0.f, o = 0.f;
  if (mx != -INFINITY) {
    const float* po = p.part_o + base * D + d;
    for (int s = 0; s < p.splits; ++s) {
      const float ms = ml[2 * s];
      if (ms == -INFINITY) continue;
      const float w = exp2f(ms - mx);
      lsum = fmaf(ml[2 * s + 1], w, lsum);
      o = fmaf(po[(int64_t)s * D], w, o);
    }
  }
  const float res = lsum > 0.f ? o / lsum : 0.f;
  OutT* dst = static_cast<OutT*>(p.out) + (int64_t)bh * D + d;
  if constexpr (sizeof(OutT) == 2) {
    *dst = __float2bfloat16(res);
  } else {
    *dst = res;
  }
  if (d == 0 && p.lse != nullptr) p.lse[bh] = lsum > 0.f ? (mx + log2f(lsum)) * 0.6931471805599453f : -INFINITY;
}

}  // namespace

hipError_t launch_decode_merge(const AttnParams& p, int head_dim, int dtype, hipStream_t stream) {
  const dim3 grid((unsigned)(p.batch * p.hq));
  if (dtype == 1) {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_merge_kernel<64, __hip_bfloat16>), grid, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<128, __hip_bfloat16>), grid, dim3(128), 0, stream, p);
  } else {
    if (head_dim == 64)
      hipLaunchKernelGGL((decode_merge_kernel<64, float>), grid, dim3(64), 0, stream, p);
    else
      hipLaunchKernelGGL((decode_merge_kernel<128, float>), grid, dim3(128), 0, stream, p);
  }
  return hipGetLastError();
}

}  // namespace yoco
