// Streaming-read bandwidth probe: a measuring instrument for the benchmark,
// not part of the attention path (built into its own library,
// lib/libyoco_probe.so, which the attention library never loads).
//
// Every workgroup of a grid-stride loop reads 16 KB per iteration as four
// rounds of 16-byte nontemporal loads (the decode kernel's load width and
// cache policy), each round a contiguous 4 KB (lane l of a wave reads bytes
// 16 l .. 16 l + 15 of its wave's 1 KB), and folds them into a running XOR;
// each workgroup stores one word, so the loads cannot be dropped and the
// writes are negligible. The buffer should be far larger than the 256 MB
// Infinity Cache so that the rate is HBM's.
//
//   extern "C" int yoco_probe_read(const void* buf, size_t bytes, unsigned* sink,
//                                  int grid, void* stream)
//     buf   [device] 16-byte aligned, bytes a multiple of 64 * 256
//     sink  [device] at least `grid` words
//     grid  workgroups of 256 threads (>= 1)
//   returns 0 on success, 1 on a bad argument, 2 if the launch failed.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

__global__ __launch_bounds__(kThreads) void read_probe_kernel(const u32x4* __restrict__ buf, uint64_t n16,
                                                              uint32_t* __restrict__ sink) {
  const uint64_t stride = (uint64_t)gridDim.x * kThreads * 4;
  u32x4 acc = {0u, 0u, 0u, 0u};
  // chunk i + u * kThreads for u = 0..3: the workgroup's 4 * kThreads chunks
  // start at i - threadIdx.x; n16 is a multiple of 4 * kThreads
  for (uint64_t i = (uint64_t)blockIdx.x * kThreads * 4 + threadIdx.x; i < n16; i += stride) {
    const u32x4 a = __builtin_nontemporal_load(buf + i);
    const u32x4 b = __builtin_nontemporal_load(buf + i + kThreads);
    const u32x4 c = __builtin_nontemporal_load(buf + i + 2 * kThreads);
    const u32x4 d = __builtin_nontemporal_load(buf + i + 3 * kThreads);
    acc ^= a ^ b ^ c ^ d;
  }
  uint32_t x = acc.x ^ acc.y ^ acc.z ^ acc.w;
  for (int o = 32; o > 0; o >>= 1) x ^= __shfl_xor(x, o);
  __shared__ uint32_t part[kThreads / 64];
  if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = x;
  __syncthreads();
  if (threadIdx.x == 0) sink[blockIdx.x] = part[0] ^ part[1] ^ part[2] ^ part[3];
}

}  // namespace

extern "C" int yoco_probe_read(const void* buf, size_t bytes, unsigned* sink, int grid, void* stream) {
  if (buf == nullptr || sink == nullptr || grid < 1) return 1;
  if ((reinterpret_cast<uintptr_t>(buf) & 15u) != 0 || bytes == 0 || bytes % (64 * kThreads) != 0) return 1;
  hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(kThreads), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(buf), (uint64_t)(bytes / 16), sink);
  return hipGetLastError() == hipSuccess ? 0 : 2;
}
