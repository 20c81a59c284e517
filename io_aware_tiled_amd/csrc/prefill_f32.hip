// fp32 forward pass on the vector ALU: one workgroup (one wavefront) per (batch, query head,
// block of 64 query rows), one lane per query row.
//
// Same tiled online-softmax recurrence as the bf16 matrix-core kernel ("4.2 FlashAttention I:
// IO-Awareness & The Online Softmax", section "FlashAttention forward: tiling + online softmax
// fused into one pass"): 32-key tiles of K and V are staged in LDS and read by every lane as
// broadcasts, each lane keeps its row's running max, running sum and d accumulators in
// registers, and causal blocks past the diagonal are not visited (nor, under a sliding window,
// blocks before the window of the block's first row). Everything is fp32 with the
// accurate exp/log, because this path is held to a 1e-5 absolute bound; the dense fp32 MFMA
// rate on gfx950 equals the VALU rate, so matrix cores would not make it faster.
#include <hip/hip_runtime.h>

#include "kernels.h"

namespace fattn {
namespace {

constexpr int BR = 64;  // query rows per workgroup
constexpr int BC = 32;  // keys per tile
constexpr float kNegInf = -__builtin_inff();

template <int D>
__global__ __launch_bounds__(64) void prefill_f32_kernel(
    const float* __restrict__ Q, const float* __restrict__ K, const float* __restrict__ V,
    float* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Tq, int Tk,
    int causal, int window, float abs_scale, int qsign) {
  __shared__ float4 Ks[BC * D / 4];
  __shared__ float4 Vs[BC * D / 4];

  const int lane = threadIdx.x;
  const int nqb = (Tq + BR - 1) / BR;
  const int bh = blockIdx.x / nqb;
  const int qb = blockIdx.x - bh * nqb;
  const int b = bh / Hq, h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const int off = Tk - Tq;

  const float* Kh = K + ((size_t)b * Hkv + g) * (size_t)Tk * D;
  const float* Vh = V + ((size_t)b * Hkv + g) * (size_t)Tk * D;
  const int i0 = qb * BR;
  const int q_end = min(i0 + BR, Tq);
  const int kv_end = causal ? min(Tk, q_end + off) : Tk;
  // sliding window: the block starts at the tile holding its first row's first visible key
  const int kv_beg = window > 0 ? max(0, i0 + off - window + 1) / BC * BC : 0;
  const int row = i0 + lane;
  const bool valid = row < Tq;
  const int last = causal ? min(Tk - 1, row + off) : Tk - 1;
  const int first = window > 0 ? row + off - window + 1 : 0;

  float q[D];
  {
    const float* Qr = Q + (((size_t)b * Hq + h) * (size_t)Tq + (valid ? row : 0)) * D;
    const float sgn = (float)qsign;
#pragma unroll
    for (int c = 0; c < D; c += 4) {
      float4 x = valid ? *reinterpret_cast<const float4*>(Qr + c) : float4{0.f, 0.f, 0.f, 0.f};
      q[c] = sgn * x.x; q[c + 1] = sgn * x.y; q[c + 2] = sgn * x.z; q[c + 3] = sgn * x.w;
    }
  }
  float acc[D];
#pragma unroll
  for (int c = 0; c < D; ++c) acc[c] = 0.f;
  float m = kNegInf, l = 0.f;

  for (int j0 = kv_beg; j0 < kv_end; j0 += BC) {
    for (int i = lane; i < BC * D / 4; i += 64) {
      const int key = j0 + i / (D / 4);
      const int c4 = i % (D / 4);
      float4 kx = {0.f, 0.f, 0.f, 0.f}, vx = {0.f, 0.f, 0.f, 0.f};
      if (key < Tk) {
        kx = *reinterpret_cast<const float4*>(Kh + (size_t)key * D + 4 * c4);
        vx = *reinterpret_cast<const float4*>(Vh + (size_t)key * D + 4 * c4);
      }
      Ks[i] = kx;
      Vs[i] = vx;
    }
    __syncthreads();

    float s[BC];
    float mt = kNegInf;
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      float dot = 0.f;
#pragma unroll
      for (int c = 0; c < D / 4; ++c) {
        const float4 kx = Ks[jj * (D / 4) + c];
        dot = fmaf(q[4 * c], kx.x, dot);
        dot = fmaf(q[4 * c + 1], kx.y, dot);
        dot = fmaf(q[4 * c + 2], kx.z, dot);
        dot = fmaf(q[4 * c + 3], kx.w, dot);
      }
      s[jj] = (j0 + jj <= last && j0 + jj >= first) ? dot * abs_scale : kNegInf;
      mt = fmaxf(mt, s[jj]);
    }
    const float m_new = fmaxf(m, mt);
    const float base = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = (m == kNegInf) ? 0.f : expf(m - base);
    float ps = 0.f;
#pragma unroll
    for (int jj = 0; jj < BC; ++jj) {
      s[jj] = expf(s[jj] - base);
      ps += s[jj];
    }
    l = alpha * l + ps;
#pragma unroll
    for (int c = 0; c < D / 4; ++c) {
      float a0 = acc[4 * c] * alpha, a1 = acc[4 * c + 1] * alpha;
      float a2 = acc[4 * c + 2] * alpha, a3 = acc[4 * c + 3] * alpha;
#pragma unroll
      for (int jj = 0; jj < BC; ++jj) {
        const float4 vx = Vs[jj * (D / 4) + c];
        a0 = fmaf(s[jj], vx.x, a0);
        a1 = fmaf(s[jj], vx.y, a1);
        a2 = fmaf(s[jj], vx.z, a2);
        a3 = fmaf(s[jj], vx.w, a3);
      }
      acc[4 * c] = a0; acc[4 * c + 1] = a1; acc[4 * c + 2] = a2; acc[4 * c + 3] = a3;
    }
    m = m_new;
    __syncthreads();
  }

  if (!valid) return;
  const float inv = 1.f / l;
  float* Or = O + (((size_t)b * Hq + h) * (size_t)Tq + row) * D;
#pragma unroll
  for (int c = 0; c < D; c += 4) {
    *reinterpret_cast<float4*>(Or + c) =
        float4{acc[c] * inv, acc[c + 1] * inv, acc[c + 2] * inv, acc[c + 3] * inv};
  }
  LSE[((size_t)b * Hq + h) * (size_t)Tq + row] = m + logf(l);
}

template <int D>
hipError_t launch_t(const Problem& p, hipStream_t stream) {
  const int nqb = (p.Tq + BR - 1) / BR;
  const long long grid = (long long)p.B * p.Hq * nqb;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(prefill_f32_kernel<D>, dim3((unsigned)grid), dim3(64), 0, stream,
                     static_cast<const float*>(p.Q), static_cast<const float*>(p.K),
                     static_cast<const float*>(p.V), static_cast<float*>(p.O), p.LSE, p.B, p.Hq,
                     p.Hkv, p.Tq, p.Tk, p.causal, p.window, p.abs_scale, p.qsign);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_f32(const Problem& p, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_t<32>(p, stream);
    case 64: return launch_t<64>(p, stream);
    case 128: return launch_t<128>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fattn
