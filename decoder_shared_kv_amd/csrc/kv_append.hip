// kv_append: one new K^,V^ row per sequence into the shared cache, or into a
// ring window cache (the Self-Decoder's sliding-window layers keep only the last
// C tokens: page "YOCO", section "Self-Decoder：把历史编码成可复用的全局表示").
//
// The new token's row exists before any Cross-Decoder layer reads the cache
// (page "YOCO", section "Decode：新 token 仍需经过两部分"). One workgroup per
// sequence copies the row with 16-byte vector stores, then bumps seq_len.
#include "internal.h"

namespace yoco {

__global__ __launch_bounds__(256) void kv_append_kernel(AppendParams p) {
  const int b = blockIdx.x;
  const int n16 = p.row_bytes / 16;
  const uint4* ks = reinterpret_cast<const uint4*>(static_cast<const char*>(p.k_new) + (int64_t)b * p.row_bytes);
  const uint4* vs = reinterpret_cast<const uint4*>(static_cast<const char*>(p.v_new) + (int64_t)b * p.row_bytes);
  // the first 16-byte pieces of the new rows are requested together with the
  // sequence's record (they do not depend on it)
  const int i0 = threadIdx.x;
  uint4 k0 = make_uint4(0, 0, 0, 0), v0 = make_uint4(0, 0, 0, 0);
  if (i0 < n16) {
    k0 = ks[i0];
    v0 = vs[i0];
  }
  const int64_t start = p.seq_start[b];
  const int32_t len = p.seq_len[b];
  const int32_t cap = p.seq_cap[b];
  // shared cache: the next free row; ring window cache: slot len mod cap, which
  // holds the token cap positions older (or nothing yet)
  const int64_t slot = p.ring ? (cap > 0 && len >= 0 ? len % cap : -1) : (len < cap ? len : -1);
  const bool ok = len >= 0 && slot >= 0 && start >= 0 && start + slot < p.pool_rows;
  if (!ok) {
    if (threadIdx.x == 0 && p.overflow != nullptr) p.overflow[0] = 1;
    return;
  }
  const int64_t row = start + slot;
  uint4* kd = reinterpret_cast<uint4*>(static_cast<char*>(p.k) + row * p.row_bytes);
  uint4* vd = reinterpret_cast<uint4*>(static_cast<char*>(p.v) + row * p.row_bytes);
  if (i0 < n16) {
    kd[i0] = k0;
    vd[i0] = v0;
  }
  for (int i = i0 + (int)blockDim.x; i < n16; i += blockDim.x) {
    kd[i] = ks[i];
    vd[i] = vs[i];
  }
  // every thread has read seq_len above; the increment comes after all of them
  __syncthreads();
  if (threadIdx.x == 0) p.seq_len[b] = len + 1;
}

hipError_t launch_kv_append(const AppendParams& p, int batch, hipStream_t stream) {
  hipLaunchKernelGGL(kv_append_kernel, dim3(batch), dim3(256), 0, stream, p);
  return hipGetLastError();
}

}  // namespace yoco
