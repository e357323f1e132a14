// Decode merge: combine the partial softmax states of one query.
//
// Each piece s of a sequence's rows (one share of the balanced split) left
// (m_s, l_s, O_s): its running max of the base-2 scores, its sum of weights
// exp2(t - m_s) and its unnormalised weighted sum of V rows. The exact softmax
// over all rows is then
//   M = max_s m_s,  L = sum_s l_s exp2(m_s - M),  O = sum_s O_s exp2(m_s - M) / L,
// and LSE = (M + log2 L) ln 2. The pieces of sequence b sit in
// consecutive slots, which the split pass recorded (first slot, count); a
// sequence with no rows gets O = 0 and LSE = -inf.
#include <hip/hip_bf16.h>

#include "internal.h"
#include "tile_common.h"

namespace yoco {

namespace {

constexpr int kMergeThreads = 256;
constexpr int kRegPieces = 4;   // pieces per thread group held in registers

// One workgroup per (sequence, query head, chunk of DW dims); threads hold V
// dims each (V = 1 or 4), so a piece group has DW / V threads and the
// workgroup 256 V / DW groups. Group g sums pieces g, g + G, ... against the
// max over all pieces (reduced across the workgroup); its first pieces are
// loaded together with their maxima, so a sequence with up to 4 G pieces
// costs one round of loads after its slot record. The groups' sums are added
// in LDS. Few pieces per sequence (many
// sequences): 64 dims, 4 per thread, fewer and fuller workgroups; many pieces
// (few long sequences): 16 dims, 1 per thread, more workgroups.
template <int V>
struct MergeVec;
template <>
struct MergeVec<1> {
  typedef float T;
};
template <>
struct MergeVec<4> {
  typedef f32x4 T;
};

template <int D, int DW, int V, typename OutT>
__global__ __launch_bounds__(kMergeThreads) void decode_merge_kernel(AttnParams p) {
  typedef typename MergeVec<V>::T VecT;
  constexpr int TPG = DW / V;                     // threads per piece group
  constexpr int G = kMergeThreads / TPG;          // piece groups
  static_assert(D % DW == 0 && kMergeThreads % TPG == 0, "dim chunks");
  __shared__ __attribute__((aligned(16))) float red_o[G][DW];
  __shared__ __attribute__((aligned(16))) float red_ml[G][2];
  const int bh = blockIdx.x;  // b * hq + h
  const int b = bh / p.hq;
  const int h = bh % p.hq;
  const int d0 = blockIdx.y * DW;
  const int tid = threadIdx.x;
  const int g = tid / TPG;
  const int dl = V * (tid % TPG);   // first of this thread's dims within the chunk
  // the sequence's rows and where the split pass left its pieces (loaded together)
  int64_t start;
  const int32_t n = decode_rows(p, b, &start);
  const int32_t s0 = p.decode_meta[2 * b + 0];
  int pieces = p.decode_meta[2 * b + 1];
  if (n == 0 || s0 < 0 || pieces < 1 || (int64_t)s0 + pieces > p.slots) pieces = 0;   // (stale when n == 0)
  const int64_t base = (int64_t)h * p.slots + (pieces > 0 ? s0 : 0);
  const float* ml = p.part_ml + 2 * base;
  const float* po = p.part_o + base * D + d0 + dl;

  // group g's first kRegPieces pieces (g, g + G, ...) go into registers with
  // their maxima in one round of loads; the maxima of any further pieces are
  // read by every thread of the workgroup. The workgroup's max over both is the
  // sequence's max M.
  float ms_r[kRegPieces], ls_r[kRegPieces];
  VecT o_r[kRegPieces];
  float m = -INFINITY;
#pragma unroll
  for (int i = 0; i < kRegPieces; ++i) {
    const int s = g + G * i;
    ms_r[i] = -INFINITY;
    ls_r[i] = 0.f;
    o_r[i] = VecT{};
    if (s < pieces) {
      ms_r[i] = ml[2 * s];
      ls_r[i] = ml[2 * s + 1];
      o_r[i] = *reinterpret_cast<const VecT*>(po + (int64_t)s * D);
    }
    m = fmaxf(m, ms_r[i]);
  }
  for (int s = G * kRegPieces + tid; s < pieces; s += kMergeThreads) m = fmaxf(m, ml[2 * s]);
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) m = fmaxf(m, __shfl_xor(m, off));
  if ((tid & 63) == 0) red_ml[tid >> 6][0] = m;
  __syncthreads();
  float M = red_ml[0][0];
#pragma unroll
  for (int w = 1; w < kMergeThreads / 64; ++w) M = fmaxf(M, red_ml[w][0]);
  // the weighted sums against it, in piece order
  float l = 0.f;
  VecT o = {};
  if (M != -INFINITY) {
#pragma unroll
    for (int i = 0; i < kRegPieces; ++i) {
      const float w = ms_r[i] == -INFINITY ? 0.f : exp2f(ms_r[i] - M);
      l = fmaf(ls_r[i], w, l);
      o += o_r[i] * w;
    }
#pragma unroll 4
    for (int s = g + G * kRegPieces; s < pieces; s += G) {
      const float ms = ml[2 * s];
      const float w = ms == -INFINITY ? 0.f : exp2f(ms - M);
      l = fmaf(ml[2 * s + 1], w, l);
      o += *reinterpret_cast<const VecT*>(po + (int64_t)s * D) * w;
    }
  }
  if (tid % TPG == 0) red_ml[g][1] = l;
  *reinterpret_cast<VecT*>(&red_o[g][dl]) = o;
  __syncthreads();
  if (tid < TPG) {
    float L = 0.f;
    VecT O = {};
#pragma unroll 8
    for (int i = 0; i < G; ++i) {
      L += red_ml[i][1];
      O += *reinterpret_cast<const VecT*>(&red_o[i][dl]);
    }
    const float inv = L > 0.f ? 1.f / L : 0.f;
    OutT* dst = static_cast<OutT*>(p.out) + (int64_t)bh * D + d0 + dl;
    if constexpr (V == 4) {
      if constexpr (sizeof(OutT) == 2) {
        *reinterpret_cast<uint2*>(dst) = make_uint2(pack2(O[0] * inv, O[1] * inv), pack2(O[2] * inv, O[3] * inv));
      } else {
        *reinterpret_cast<f32x4*>(dst) = O * inv;
      }
    } else {
      if constexpr (sizeof(OutT) == 2) {
        *dst = __float2bfloat16(O * inv);
      } else {
        *dst = O * inv;
      }
    }
    if (tid == 0 && blockIdx.y == 0 && p.lse != nullptr)
      p.lse[bh] = L > 0.f ? (M + log2f(L)) * 0.6931471805599453f : -INFINITY;
  }
}

template <int D, typename OutT>
void launch_merge_d(const AttnParams& p, hipStream_t stream) {
  const bool many = p.splits >= 32 * p.batch;   // pieces per sequence, roughly
  const dim3 block(kMergeThreads);
  if (many)
    hipLaunchKernelGGL((decode_merge_kernel<D, 16, 1, OutT>), dim3(p.batch * p.hq, D / 16), block, 0, stream, p);
  else
    hipLaunchKernelGGL((decode_merge_kernel<D, 64, 4, OutT>), dim3(p.batch * p.hq, D / 64), block, 0, stream, p);
}

}  // namespace

hipError_t launch_decode_merge(const AttnParams& p, int head_dim, int dtype, hipStream_t stream) {
  if (dtype == 1) {
    if (head_dim == 64) launch_merge_d<64, __hip_bfloat16>(p, stream);
    else launch_merge_d<128, __hip_bfloat16>(p, stream);
  } else {
    if (head_dim == 64) launch_merge_d<64, float>(p, stream);
    else launch_merge_d<128, float>(p, stream);
  }
  return hipGetLastError();
}

}  // namespace yoco
