// Static device scratch for the entry point that allocates nothing (attn_fwd_noalloc).
//
// The split-K decode writes per-split partial outputs and log-sum-exps to a scratch buffer
// before its combine kernel merges them. attn_fwd keeps that buffer in a grow-only workspace it
// allocates on first use; attn_fwd_noalloc uses this fixed array instead, which every device the
// library runs on holds from module load until the process ends. Its size, kScratchFloats
// floats (16 MiB), caps the split count (splits * B * Hq * (d + 1) floats must fit).
//
// In host code the array's name is only a stand-in for its device address, so the address is
// looked up once per device, with that device current, and only the looked-up pointer is ever
// handed to a kernel. Every call on one GPU shares that GPU's array: calls that overlap on one
// GPU (two streams, two threads) race on it. Nothing in it needs to start at zero: the partial
// kernel writes every split's output and log-sum-exp before the combine reads them.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <mutex>

#include "kernels.h"

namespace fattn {
namespace {

static __device__ __align__(256) float scratch[kScratchFloats];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mutex;
float* g_scratch_ptr[kMaxDevices] = {};

}  // namespace

hipError_t static_scratch(int dev, float** out) {
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(g_scratch_mutex);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    g_scratch_ptr[dev] = static_cast<float*>(p);
  }
  *out = g_scratch_ptr[dev];
  return hipSuccess;
}

}  // namespace fattn
