// bf16 prefill kernel for gfx950: one workgroup per (batch, query head, query block).
//
// The algorithm is the tiled online-softmax forward of "4.2 FlashAttention I: IO-Awareness &
// The Online Softmax" (section "FlashAttention forward: tiling + online softmax fused into one
// pass") and of "Efficient attention & KV cache" (section 3): the query block stays on chip,
// key/value tiles stream past it, and each row keeps a running max m, a running sum l and an
// unnormalised accumulator that are rescaled by exp(m_old - m_new) whenever m grows; blocks past
// the causal diagonal are never visited ("Causal masking is free" in the same chapter).
//
// Mapping onto CDNA4:
//  * every wavefront owns 32 query rows; both products run on v_mfma_f32_32x32x16_bf16 with fp32
//    accumulation. The scores are formed transposed, S^T = K Q^T, so a lane holds one query row
//    (lane % 32) and 16 keys per 32x32 tile: the row max and row sum are in-lane except for one
//    exchange between the two half-waves.
//  * the output is accumulated transposed as well, O^T = V^T P^T. The P^T operand is the S^T
//    accumulator itself converted to bf16 (no LDS round trip), because the MFMA reduction index
//    may be any permutation of the keys as long as both operands use the same one; V is stored
//    transposed in LDS in exactly that key order.
//  * K and V tiles are double-buffered in LDS: the next tile's global loads are in flight in
//    registers while the current tile is consumed, then written to the other LDS stage.
//  * the exponentials run on the fp32 VALU as exp2 with log2(e) folded into the scale.
//  * the reference maximum is re-based lazily: the exponent base only moves when a row's maximum
//    grows by more than kRebase (log2 units), so the 64-register accumulator rescale is rare.
//    Any reference gives the same O = acc / l and LSE = m + log l ("Efficient attention & KV
//    cache", section 2.1: the max is there only for numerical safety); the weights stay below
//    2^kRebase, far inside fp32 and bf16 range.
//  * the row sum is taken from the bf16 weights the PV product uses (v_dot2 against ones), so the
//    normaliser matches the weights exactly and costs half the adds.
//  * K and V are read with buffer loads: rows past Tk come back as zeros from the hardware range
//    check, so ragged tiles need no branches.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace fattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();
constexpr float kRebase = 8.0f;               // lazy re-base threshold, log2 units
constexpr int kBufferFlags = 0x00020000;      // raw buffer, 32-bit data format

template <int D, int BC, int NW>
struct Shape {
  static constexpr int BR = 32 * NW;       // query rows per workgroup
  static constexpr int NT = 64 * NW;       // threads per workgroup
  static constexpr int KS = D + 8;         // LDS row pitch of K (elements): +16 bytes
  static constexpr int VS = BC + 8;        // LDS row pitch of V^T (elements): +16 bytes
  static constexpr int K_ELEMS = BC * KS;
  static constexpr int V_ELEMS = D * VS;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int LDS_BYTES = 2 * STAGE * 2;
  static constexpr int K_CHUNKS = BC * D / 8;           // 16-byte pieces of a K tile
  static constexpr int K_PER = (K_CHUNKS + NT - 1) / NT;
  static constexpr int V_ITEMS = (BC / 4) * (D / 8);    // 4 keys x 8 dims per item
  static constexpr int V_PER = (V_ITEMS + NT - 1) / NT;
  static_assert(D % 32 == 0 && BC % 32 == 0, "tile shape");
};

// Position of tile-local key k inside a V^T row. Within each group of 16 keys the order is
// {0-3, 8-11, 4-7, 12-15}: that is the order in which one half-wave holds its eight keys of a
// 16-key chunk in the S^T accumulator (rows 4h..4h+3 and 8+4h..8+4h+3 for half h).
__device__ __forceinline__ int vt_pos_of_group(int kg) {  // start of keys 4kg..4kg+3
  return 16 * (kg >> 2) + 8 * (kg & 1) + 4 * ((kg >> 1) & 1);
}

// Low halves of a and b as one word (a low), and the high halves likewise.
__device__ __forceinline__ uint32_t pack_lo(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x05040100u);
}
__device__ __forceinline__ uint32_t pack_hi(uint32_t a, uint32_t b) {
  return __builtin_amdgcn_perm(b, a, 0x07060302u);
}

// Buffer resource for rows [row0, T) of a [T, D] bf16 slice: reads past T return zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const __bf16* slice, int row0, int T) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(slice + (size_t)row0 * D),
                                           (short)0, (T - row0) * D * 2, kBufferFlags);
}

// Two floats rounded to bf16 (nearest-even) and packed low/high.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

template <int D, int BC, int NW>
__global__ __launch_bounds__(64 * NW, 2) void prefill_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Tq, int Tk,
    int causal, float log2_scale, int qsign, int schedule) {
  using S = Shape<D, BC, NW>;
  extern __shared__ __align__(16) __bf16 lds[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int col = lane & 31;   // query row within the wave (MFMA column)
  const int hf = lane >> 5;    // half-wave

  // ---- which (batch, head, query block) this workgroup owns
  const int nqb = (Tq + S::BR - 1) / S::BR;
  const int total = gridDim.x;
  int lin = blockIdx.x;
  if (schedule == 2) {
    // Workgroups are dealt round-robin to the 8 XCDs; give each XCD a contiguous range of the
    // logical order so the query blocks of one head share that XCD's L2 for K and V.
    const int xcd = lin & 7, k = lin >> 3;
    const int q8 = total >> 3, r8 = total & 7;
    lin = xcd * q8 + (xcd < r8 ? xcd : r8) + k;
  }
  const int bh = lin / nqb;
  int qb = lin - bh * nqb;
  if (schedule == 2 && causal) qb = nqb - 1 - qb;  // longest causal blocks first
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  const int off = Tk - Tq;

  const __bf16* Qh = Q + ((size_t)b * Hq + h) * (size_t)Tq * D;
  const __bf16* Kh = K + ((size_t)b * Hkv + g) * (size_t)Tk * D;
  const __bf16* Vh = V + ((size_t)b * Hkv + g) * (size_t)Tk * D;

  const int i0 = qb * S::BR;
  const int q_end = min(i0 + S::BR, Tq);
  const int kv_end = causal ? min(Tk, q_end + off) : Tk;
  const int ntiles = (kv_end + BC - 1) / BC;

  // ---- this wave's query rows; Q^T operand held in registers for the whole loop
  const int qw0 = i0 + 32 * wave;
  const int qrow = qw0 + col;
  const bool wave_has_rows = qw0 < Tq;
  const int wave_last = min(qw0 + 31, Tq - 1);
  bf16x8 qb8[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qrow < Tq && qsign != 0) {
      raw = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * D + 16 * kk + 8 * hf);
      if (qsign < 0) raw ^= 0x80008000u;  // exact negation of both bf16 halves
    }
    qb8[kk] = __builtin_bit_cast(bf16x8, raw);
  }

  // ---- staging registers for the next tile; byte offsets within a tile are fixed per thread
  u32x4 kreg[S::K_PER];
  u32x4 vreg[S::V_PER][4];
  int koff[S::K_PER], voff[S::V_PER];
#pragma unroll
  for (int i = 0; i < S::K_PER; ++i) koff[i] = (tid + i * S::NT) * 16;
#pragma unroll
  for (int i = 0; i < S::V_PER; ++i) {
    const int it = tid + i * S::NT;
    voff[i] = (4 * (it % (BC / 4))) * D * 2 + (it / (BC / 4)) * 16;
  }

  auto load_tile = [&](int j0) {
    const __amdgpu_buffer_rsrc_t kr = rows_rsrc<D>(Kh, j0, Tk);
    const __amdgpu_buffer_rsrc_t vr = rows_rsrc<D>(Vh, j0, Tk);
#pragma unroll
    for (int i = 0; i < S::K_PER; ++i)
      if (S::K_CHUNKS % S::NT == 0 || tid + i * S::NT < S::K_CHUNKS)
        kreg[i] = __builtin_amdgcn_raw_buffer_load_b128(kr, koff[i], 0, 0);
#pragma unroll
    for (int i = 0; i < S::V_PER; ++i)
      if (S::V_ITEMS % S::NT == 0 || tid + i * S::NT < S::V_ITEMS) {
#pragma unroll
        for (int r = 0; r < 4; ++r)
          vreg[i][r] = __builtin_amdgcn_raw_buffer_load_b128(vr, voff[i] + r * D * 2, 0, 0);
      }
  };

  auto store_tile = [&](int stage) {
    __bf16* Ks = lds + stage * S::STAGE;
    __bf16* Vs = Ks + S::K_ELEMS;
#pragma unroll
    for (int i = 0; i < S::K_PER; ++i) {
      const int c = tid + i * S::NT;
      if (c < S::K_CHUNKS) {
        const int row = c / (D / 8), cc = c % (D / 8);
        *reinterpret_cast<u32x4*>(Ks + row * S::KS + cc * 8) = kreg[i];
      }
    }
#pragma unroll
    for (int i = 0; i < S::V_PER; ++i) {
      const int it = tid + i * S::NT;
      if (it < S::V_ITEMS) {
        const int kg = it % (BC / 4), dg = it / (BC / 4);
        const int pos = vt_pos_of_group(kg);
        // 4 keys x 8 dims -> 8 rows of V^T, 4 consecutive key positions each
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const uint32_t a0 = vreg[i][0][w], a1 = vreg[i][1][w];
          const uint32_t a2 = vreg[i][2][w], a3 = vreg[i][3][w];
          u32x2 even = {pack_lo(a0, a1), pack_lo(a2, a3)};
          u32x2 odd = {pack_hi(a0, a1), pack_hi(a2, a3)};
          const int d = 8 * dg + 2 * w;
          *reinterpret_cast<u32x2*>(Vs + d * S::VS + pos) = even;
          *reinterpret_cast<u32x2*>(Vs + (d + 1) * S::VS + pos) = odd;
        }
      }
    }
  };

  // ---- running statistics (log2 domain: M = max of log2_scale * s over the keys seen)
  float M = kNegInf;
  float lsum = 0.f;  // this lane's share of the row sum (half of the keys of each tile)
  // M is the exponent base of this lane's row, in log2 units of the scaled scores
  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int j = 0; j < ntiles; ++j) {
    const int j0 = j * BC;
    if (j + 1 < ntiles) load_tile(j0 + BC);

    const bool active = wave_has_rows && (!causal || j0 <= wave_last + off);
    if (active) {
      const __bf16* Ks = lds + (j & 1) * S::STAGE;
      const __bf16* Vs = Ks + S::K_ELEMS;

      // S^T tile: rows = keys (32 per MFMA tile), columns = this wave's 32 queries. The K
      // operands of a 32-key half are all read from LDS before its MFMA chain starts, so the
      // read latency is paid once per chain rather than once per MFMA.
      f32x16 s[BC / 32];
#pragma unroll
      for (int t = 0; t < BC / 32; ++t) {
        bf16x8 ka[D / 16];
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          ka[kk] = *reinterpret_cast<const bf16x8*>(Ks + (32 * t + col) * S::KS + 16 * kk + 8 * hf);
        s[t] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk)
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka[kk], qb8[kk], s[t], 0, 0, 0);
      }
      // issue order: the first half's reads, then its MFMAs alternating with the second half's
      // reads, then the second half's MFMAs
      __builtin_amdgcn_sched_group_barrier(0x100, D / 16, 0);
#pragma unroll
      for (int i = 0; i < (BC / 32 - 1) * (D / 16); ++i) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
      }
      __builtin_amdgcn_sched_group_barrier(0x008, D / 16, 0);

      // mask only on the diagonal and ragged tiles
      const bool need_mask = (j0 + BC > Tk) || (causal && j0 + BC - 1 > qw0 + off);
      if (need_mask) {
        const int last = causal ? min(Tk - 1, qrow + off) : Tk - 1;
#pragma unroll
        for (int t = 0; t < BC / 32; ++t)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = j0 + 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
            if (key > last) s[t][r] = kNegInf;
          }
      }

      // online softmax update for this lane's query row
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < BC / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      mx = fmaxf(mx, __shfl_xor(mx, 32));
      const float mt = mx * log2_scale;
      const bool grow = mt > M + kRebase;  // always true on the first tile a row sees
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mt : M;
        const float alpha = __builtin_amdgcn_exp2f(M - m_new);  // 0 while M is -inf
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
        M = m_new;
      }
      const float base = (M == kNegInf) ? 0.f : M;

      // Per 16-key chunk: weights exp2(s * log2_scale - base) <= 2^kRebase rounded to bf16 (the
      // row sum adds exactly those bf16 weights), then O^T += V^T P^T for that chunk, so the
      // chunk's MFMAs can run while the next chunk's exponentials are computed.
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int ch = 0; ch < BC / 16; ++ch) {
        const int t = ch >> 1, c2 = ch & 1;
        bf16x8 pb;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t][8 * c2 + i], log2_scale, -base));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t][8 * c2 + i + 1], log2_scale, -base));
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
          pb[i] = pp[0];
          pb[i + 1] = pp[1];
        }
        bf16x8 va[D / 32];
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          va[dt] = *reinterpret_cast<const bf16x8*>(Vs + (32 * dt + col) * S::VS + 16 * ch + 8 * hf);
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[dt], pb, acc[dt], 0, 0, 0);
      }
    }

    if (j + 1 < ntiles) store_tile((j + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: O = acc / l, LSE = ln 2 * (M + log2 l)
  if (!wave_has_rows) return;
  const float l = lsum + __shfl_xor(lsum, 32);
  if (qrow >= Tq) return;
  const float inv = 1.f / l;
  __bf16* Orow = O + (((size_t)b * Hq + h) * (size_t)Tq + qrow) * D;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      const int d0 = 32 * dt + 8 * g4 + 4 * hf;
      u32x2 packed = {pack2_bf16(acc[dt][4 * g4 + 0] * inv, acc[dt][4 * g4 + 1] * inv),
                      pack2_bf16(acc[dt][4 * g4 + 2] * inv, acc[dt][4 * g4 + 3] * inv)};
      *reinterpret_cast<u32x2*>(Orow + d0) = packed;
    }
  if (hf == 0) {
    LSE[((size_t)b * Hq + h) * (size_t)Tq + qrow] = (M + __builtin_amdgcn_logf(l)) * kLn2;
  }
}

template <int D, int BC, int NW>
hipError_t launch_t(const Problem& p, int schedule, hipStream_t stream) {
  using S = Shape<D, BC, NW>;
  const int nqb = (p.Tq + S::BR - 1) / S::BR;
  const long long grid = (long long)p.B * p.Hq * nqb;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, NW>), dim3((unsigned)grid), dim3(S::NT),
                     S::LDS_BYTES, stream, static_cast<const __bf16*>(p.Q),
                     static_cast<const __bf16*>(p.K), static_cast<const __bf16*>(p.V),
                     static_cast<__bf16*>(p.O), p.LSE, p.B, p.Hq, p.Hkv, p.Tq, p.Tk, p.causal,
                     p.log2_scale, p.qsign, schedule);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const Problem& p, int block_kv, int waves, int schedule, hipStream_t stream) {
  if (block_kv == 64 && waves == 4) return launch_t<D, 64, 4>(p, schedule, stream);
  if (block_kv == 64 && waves == 8) return launch_t<D, 64, 8>(p, schedule, stream);
  if (block_kv == 32 && waves == 4) return launch_t<D, 32, 4>(p, schedule, stream);
  if (block_kv == 32 && waves == 8) return launch_t<D, 32, 8>(p, schedule, stream);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_prefill_bf16(const Problem& p, int block_kv, int waves, int schedule,
                               hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_d<32>(p, block_kv, waves, schedule, stream);
    case 64: return launch_d<64>(p, block_kv, waves, schedule, stream);
    case 128: return launch_d<128>(p, block_kv, waves, schedule, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fattn
