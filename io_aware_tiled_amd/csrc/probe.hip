// Measurement probes, built into their own library (libfattn_probe.so) that only the benchmark
// loads: the matrix-core and HBM-read rates this chip reaches on trivial work, so that the
// attention kernels' rates can be quoted against what is achievable as well as against the
// published peaks. Not part of libfattn or of its C ABI.
//
//  int probe_mfma_bf16(float* out, int workgroups, int iters, int random, void* stream);
//    Enqueues `workgroups` workgroups of 8 wavefronts on `stream`; every wavefront runs four
//    independent chains of v_mfma_f32_32x32x16_bf16 (the prefill kernel's instruction, 32768
//    FLOPs each), 32 * iters of them, on register operands, then writes one float per thread to
//    `out` (device memory of at least workgroups * 512 floats, owned by the caller).
//    FLOPs per launch: workgroups * 8 * 32 * iters * 32768. With random = 0 the operands are
//    small slowly varying values; with random = 1 every element is a hashed uniform(-1, 1)
//    value, as the attention inputs are. The matrix cores run measurably slower on the second
//    (the chip's clock under matrix load depends on how many operand bits toggle).
//  int probe_hbm_read(const void* buf, size_t bytes, unsigned* out, int workgroups, void* stream);
//    Enqueues `workgroups` workgroups of 256 threads that read the `bytes` bytes at device
//    pointer `buf` once with 16-byte nontemporal loads (the decode kernel's load form),
//    workgroup w the w-th of `workgroups` equal contiguous chunks, and write one XOR-reduced word
//    per wavefront to `out` (at least workgroups * 4 words). `buf` must be 16-byte aligned and
//    `bytes` a positive multiple of 16.
//  Both return -1 for a NULL pointer or a non-positive count (and, for the read probe, a
//  misaligned buffer or size), -3 for a launch failure, else 0.
#include <hip/hip_runtime.h>

#include <cstddef>
#include <cstdint>


namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// uniform(-1, 1) from a 32-bit integer hash (xorshift-multiply mixing)
__device__ __forceinline__ float hashed_uniform(uint32_t x) {
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return (float)(x & 0xffffu) * (1.0f / 32768.0f) - 1.0f;
}

template <bool RANDOM>
__global__ __launch_bounds__(512) void probe_mfma_kernel(float* __restrict__ out, int iters) {
  f32x16 c0 = {}, c1 = {}, c2 = {}, c3 = {};
  bf16x8 a, b;
  const uint32_t id = blockIdx.x * blockDim.x + threadIdx.x;
  for (int i = 0; i < 8; ++i) {
    if (RANDOM) {
      a[i] = (__bf16)hashed_uniform(16 * id + i);
      b[i] = (__bf16)hashed_uniform(16 * id + 8 + i);
    } else {
      a[i] = (__bf16)(0.001f * (float)(threadIdx.x + i));
      b[i] = (__bf16)(0.002f * (float)((int)threadIdx.x - i));
    }
  }
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      c0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c0, 0, 0, 0);
      c1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c1, 0, 0, 0);
      c2 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c2, 0, 0, 0);
      c3 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c3, 0, 0, 0);
    }
  }
  float s = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) s += c0[r] + c1[r] + c2[r] + c3[r];
  out[(size_t)blockIdx.x * blockDim.x + threadIdx.x] = s;
}

__global__ __launch_bounds__(256) void probe_read_kernel(const u32x4* __restrict__ p, size_t n,
                                                         unsigned* __restrict__ out) {
  // workgroup w reads the contiguous chunk [w * chunk, (w + 1) * chunk), eight loads in flight
  // per thread (measured: about 7.1 TB/s with 8192-16384 workgroups over 4 GiB, against
  // 6.3-6.8 for a grid-stride walk)
  const size_t chunk = (n + gridDim.x - 1) / gridDim.x;
  const size_t beg = (size_t)blockIdx.x * chunk;
  const size_t end = beg + chunk < n ? beg + chunk : n;
  u32x4 acc = {0u, 0u, 0u, 0u};
  size_t i = beg + threadIdx.x;
  for (; i + 7 * 256 < end; i += 8 * 256) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = __builtin_nontemporal_load(p + i + u * 256);
#pragma unroll
    for (int u = 0; u < 8; ++u) acc ^= v[u];
  }
  for (; i < end; i += 256) acc ^= __builtin_nontemporal_load(p + i);
  // one word per wavefront (a word per thread added measurable write traffic at this grid size)
  unsigned w = acc.x ^ acc.y ^ acc.z ^ acc.w;
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) w ^= __shfl_xor(w, m);
  if ((threadIdx.x & 63) == 0) out[(size_t)blockIdx.x * 4 + (threadIdx.x >> 6)] = w;
}

}  // namespace

constexpr int kOk = 0, kInvalid = -1, kLaunch = -3;

#define PROBE_API extern "C" __attribute__((visibility("default")))

PROBE_API int probe_mfma_bf16(float* out, int workgroups, int iters, int random, void* stream) {
  if (!out || workgroups <= 0 || iters <= 0 || (random != 0 && random != 1)) return kInvalid;
  const hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  if (random)
    hipLaunchKernelGGL(probe_mfma_kernel<true>, dim3((unsigned)workgroups), dim3(512), 0, s, out,
                       iters);
  else
    hipLaunchKernelGGL(probe_mfma_kernel<false>, dim3((unsigned)workgroups), dim3(512), 0, s, out,
                       iters);
  return hipGetLastError() == hipSuccess ? kOk : kLaunch;
}

PROBE_API int probe_hbm_read(const void* buf, size_t bytes, unsigned* out, int workgroups,
                             void* stream) {
  if (!buf || !out || workgroups <= 0 || bytes < 16 || (bytes & 15) != 0 ||
      (reinterpret_cast<uintptr_t>(buf) & 15) != 0)
    return kInvalid;
  hipLaunchKernelGGL(probe_read_kernel, dim3((unsigned)workgroups), dim3(256), 0,
                     reinterpret_cast<hipStream_t>(stream), static_cast<const u32x4*>(buf),
                     bytes / 16, out);
  return hipGetLastError() == hipSuccess ? kOk : kLaunch;
}
