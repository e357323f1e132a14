// Device-resident scratch of the decode entry point that allocates nothing.
//
// The split-K decode needs partial results between its two launches (per
// share and query head: an unnormalised output and its (max, sum), plus two
// integers per sequence). yoco_xattn_decode takes them in a caller-owned
// workspace; callers that cannot allocate (code under graph capture, tight
// serving loops) use yoco_xattn_decode_noalloc instead, whose partials live in
// the file-scope array below: one copy per GPU, held for the life of the
// process. Host code must never pass the array's name to a kernel (on the host
// it is only a stand-in for the symbol); it passes the device address that
// hipGetSymbolAddress returns for the current device, looked up once per
// device and kept here.
#include <mutex>

#include "internal.h"
#include "yoco_xattn.h"

namespace yoco {

namespace {

static __device__ __align__(256) unsigned char scratch[YOCO_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t noalloc_scratch(void** ptr) {
  int dev = -1;
  hipError_t err = hipGetDevice(&dev);
  if (err != hipSuccess) return err;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (err != hipSuccess) return err;
    if (p == nullptr || (reinterpret_cast<uintptr_t>(p) & 255u) != 0) return hipErrorInvalidSymbol;
    g_scratch_ptr[dev] = p;
  }
  *ptr = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace yoco
