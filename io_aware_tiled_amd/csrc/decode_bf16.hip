// bf16 decode (one query token per head) for gfx950: split-K partial kernel + LSE combine.
//
// A decode step reads every cached key and value once and does about eight FLOPs per byte under
// 8-way grouped-query attention, so it is bound by HBM bandwidth ("Attention from scratch +
// roofline", section "Classify prefill vs decode", and its exercise 1 on GQA). The key range of
// each (batch, kv head) is therefore split into `splits` chunks processed by independent
// single-wavefront workgroups, so that thousands of wavefronts keep loads in flight. Each chunk
// runs the online-softmax recurrence of "4.2 FlashAttention I" over its keys and writes a
// normalised partial output O_s with its log-sum-exp LSE_s; the combine kernel then merges the
// chunks exactly, O = sum_s exp(LSE_s - LSE) O_s with LSE = log sum_s exp(LSE_s), which holds
// because any reference maximum gives the same final ratio ("Efficient attention & KV cache",
// section 2.1).
//
// Inside a chunk the G query heads that share a kv head form the 16-wide N side of
// v_mfma_f32_16x16x32_bf16 (padded with zero rows when G < 16): S^T = K Q^T reads K from a
// per-wave LDS copy of the block (loaded from global memory as whole rows, 1 KB per load
// instruction: reading the operand layout straight from memory, 16 rows a quarter each, streamed
// about 10% slower), and O^T = V^T P^T reads V^T from a small per-wave LDS transpose whose key
// order matches the S^T accumulator, as in the prefill kernel.
//
// The same kernels serve a paged cache ("Efficient attention & KV cache", section 2.5 and the
// interview question on what PagedAttention changes in the kernel): keys and values sit in
// fixed-size pages located through a per-sequence block table, and the kernel fetches each
// 16-key half of its 32-key blocks from the page the table names, one table read per half.
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"

namespace fattn {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();
constexpr int KB = 32;       // keys per block

// LDS layouts of the per-wave K rows and V^T block. Measured on gfx950 with a probe of the
// counter SQ_LDS_BANK_CONFLICT: a 16-byte LDS read (ds_read_b128) is served in four passes of 16
// lanes, each pass one half of the wave (lanes 0-31 or 32-63) and, within it, the 4-lane quads
// whose index has even (or odd) parity, against 64 four-byte banks; a 16-byte write
// (ds_write_b128) in passes of 8 consecutive lanes against 32 banks. The element offsets below
// give every pass of the kernel's reads and writes distinct banks.
//
// K: key row r (D elements, no padding), logical 16-byte chunk c stored at chunk c ^ f(r).
template <int D>
__device__ __forceinline__ int k_at(int r, int c) {
  const int f = D >= 64 ? r % (D / 8) : ((r >> 3) & 1) << 1;
  return r * D + 8 * (c ^ f);
}
// V^T: dim row r of 32 keys (4 chunks), rows 8 apart in the writes moved to the other half of
// the 32 banks (r ^ bit 3 of r), chunks of odd rows swapped in pairs for the reads.
__device__ __forceinline__ int vt_at(int r, int c) {
  return (r ^ ((r >> 3) & 1)) * KB + 8 * (c ^ ((r & 1) << 1));
}

__device__ __forceinline__ uint32_t pick_half(uint32_t a, uint32_t b, int hi) {
  return hi ? ((a >> 16) | (b & 0xffff0000u)) : ((a & 0xffffu) | (b << 16));
}

template <int D>
struct Block {
  // K of half t: load c covers rows 16t + c*RPI .. +RPI-1 whole (RPI = 512 / D rows of D/8
  // 16-byte chunks each), lane -> row c*RPI + lane/(D/8), chunk lane%(D/8)
  u32x4 k[2][D / 32];
  u32x4 v[8];          // V rows of keys 4gg+r and 16+4gg+r, dims 8dg .. 8dg+8
};

// Where the 16-key halves of a 32-key block live. Keys kb + 16h + r (r < 16) are rows
// row[h] + r of the K and V bases; a half whose rows are not readable has ok[h] false.
// Contiguous caches: the [Tk, D] slice of one (batch, kv head), row[h] = kb + 16h.
// Paged caches [num_blocks, Hkv, bs, D] (bs a power of two >= 16, so a 16-key half never
// crosses a page): row[h] = (page * Hkv + kv head) * bs + (kb + 16h) mod bs with page read from
// the sequence's block table.
struct Halves {
  size_t row[2];
  bool ok[2];
};

// One 32-key block of K and V into registers. Every key and value is read exactly once per
// decode step, so the loads carry the nontemporal hint: they stream past the caches instead of
// evicting lines that other wavefronts still use (measured: 5.8 -> 6.5 TB/s on the GQA shape).
template <int D>
__device__ __forceinline__ void load_block(Block<D>& blk, const __bf16* Kb, const __bf16* Vb,
                                           const Halves& hv, int kb, int kend, int lane) {
  // K: each load reads whole rows (64 lanes x 16 bytes contiguous), which streams faster than
  // reading 16 rows a quarter each in the operand layout; the rows go through LDS (kt_store)
  constexpr int CPR = D / 8, RPI = 64 / CPR;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
#pragma unroll
    for (int c = 0; c < D / 32; ++c) {
      const int r = c * RPI + lane / CPR;
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kb + 16 * t + r < kend && hv.ok[t])
        x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(
            Kb + (hv.row[t] + r) * D + 8 * (lane % CPR)));
      blk.k[t][c] = x;
    }
  }
  if (lane < D / 2) {
    const int gg = lane & 3, dg = lane >> 2;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const int h = i >> 2, r = 4 * gg + (i & 3);
      u32x4 x = {0u, 0u, 0u, 0u};
      if (kb + 16 * h + r < kend && hv.ok[h])
        x = __builtin_nontemporal_load(
            reinterpret_cast<const u32x4*>(Vb + (hv.row[h] + r) * D + 8 * dg));
      blk.v[i] = x;
    }
  }
}

// Block-table view of one sequence of a paged cache (unused by contiguous launches).
struct PageMap {
  const int* table;  // this sequence's row of the block table
  int nblocks;       // physical blocks in the cache; entries outside [0, nblocks) read as zeros
  int Hkv, g;        // kv heads per page and this workgroup's kv head
  int sh;            // log2(block size)
};

template <bool PAGED>
__device__ __forceinline__ Halves halves_of(int kb, int kend, const PageMap& pm) {
  Halves hv;
  if (!PAGED) {
    hv.row[0] = (size_t)kb;
    hv.row[1] = (size_t)kb + 16;
    hv.ok[0] = hv.ok[1] = true;
    return hv;
  }
  const int mask = (1 << pm.sh) - 1;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int key = kb + 16 * h;
    const int page = key < kend ? pm.table[key >> pm.sh] : 0;
    hv.ok[h] = key < kend && page >= 0 && page < pm.nblocks;
    hv.row[h] = hv.ok[h] ? (((size_t)page * pm.Hkv + pm.g) << pm.sh) + (key & mask) : 0;
  }
  return hv;
}

// PAGED: K and V are paged caches [num_blocks, Hkv, bs, D] read through `table`
// ([B, max_blocks] physical block ids) with seq_lens[b] keys for batch b (clamped to
// max_blocks * bs); Tk and k0 are then unused. Otherwise K, V are [B, Hkv, Tk, D] and the keys
// [k0, Tk) are read.
template <int D, bool PAGED>
__global__ __launch_bounds__(64, 2) void decode_partial_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    float* __restrict__ ws_o, float* __restrict__ ws_lse, int Hq, int Hkv, int Tk, int k0,
    int splits, int chunk, float log2_scale, int qsign, const int* __restrict__ table,
    const int* __restrict__ seq_lens, int max_blocks, int bs_shift, int nblocks) {
  __shared__ __align__(16) __bf16 Vt[D * KB];
  __shared__ __align__(16) __bf16 Kt[KB * D];

  const int lane = threadIdx.x;
  const int c16 = lane & 15, g4 = lane >> 4;
  const int G = Hq / Hkv;
  const int nqg = (G + 15) / 16;
  int w = blockIdx.x;
  const int s = w % splits;
  w /= splits;
  const int qg = w % nqg;
  w /= nqg;
  const int hk = w % Hkv;
  const int b = w / Hkv;
  PageMap pm = {nullptr, nblocks, Hkv, hk, bs_shift};
  int kv_len = Tk;
  if (PAGED) {
    pm.table = table + (size_t)b * max_blocks;
    kv_len = max(0, min(seq_lens[b], max_blocks << bs_shift));
    k0 = 0;
  }
  const int kbeg = k0 + s * chunk;  // k0 > 0: a sliding window starts at key Tk - window
  const int kend = min(kv_len, kbeg + chunk);
  const int qi = qg * 16 + c16;
  const bool qvalid = qi < G;
  const int hq = hk * G + qi;

  // Q^T operand: column = query qi, dims 32c + 8*g4 .. +8
  bf16x8 qb[D / 32];
#pragma unroll
  for (int c = 0; c < D / 32; ++c) {
    u32x4 raw = {0u, 0u, 0u, 0u};
    if (qvalid && qsign != 0) {
      raw = *reinterpret_cast<const u32x4*>(Q + ((size_t)b * Hq + hq) * D + 32 * c + 8 * g4);
      if (qsign < 0) raw ^= 0x80008000u;
    }
    qb[c] = __builtin_bit_cast(bf16x8, raw);
  }

  const __bf16* Kh = PAGED ? K : K + ((size_t)b * Hkv + hk) * (size_t)Tk * D;
  const __bf16* Vh = PAGED ? V : V + ((size_t)b * Hkv + hk) * (size_t)Tk * D;

  float M = kNegInf, lsum = 0.f;
  f32x4 acc[D / 16];
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt) acc[mt] = f32x4{};

  Block<D> cur;
  if (kbeg < kend) load_block<D>(cur, Kh, Vh, halves_of<PAGED>(kbeg, kend, pm), kbeg, kend, lane);

  // page lookups run one block ahead of the loads that use them
  Halves hv_next = halves_of<PAGED>(kbeg + KB, kend, pm);
  for (int kb = kbeg; kb < kend; kb += KB) {
    const bool more = kb + KB < kend;
    Block<D> nxt;
    if (more) load_block<D>(nxt, Kh, Vh, hv_next, kb + KB, kend, lane);
    hv_next = halves_of<PAGED>(kb + 2 * KB, kend, pm);

    __syncthreads();  // the previous block's V^T reads are done
    if (lane < D / 2) {
      const int gg = lane & 3, dg = lane >> 2;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1, hi = e & 1;
        u32x4 row = {pick_half(cur.v[0][wd], cur.v[1][wd], hi),
                     pick_half(cur.v[2][wd], cur.v[3][wd], hi),
                     pick_half(cur.v[4][wd], cur.v[5][wd], hi),
                     pick_half(cur.v[6][wd], cur.v[7][wd], hi)};
        *reinterpret_cast<u32x4*>(Vt + vt_at(8 * dg + e, gg)) = row;
      }
    }

    {
      constexpr int CPR = D / 8, RPI = 64 / CPR;
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int c = 0; c < D / 32; ++c)
          *reinterpret_cast<u32x4*>(Kt + k_at<D>(16 * t + c * RPI + lane / CPR, lane % CPR)) =
              cur.k[t][c];
    }
    __syncthreads();  // K rows of this block are in LDS

    // S^T: rows = keys kb + 16t + 4*g4 + r, column = query qi
    f32x4 st[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      st[t] = f32x4{};
#pragma unroll
      for (int c = 0; c < D / 32; ++c) {
        const bf16x8 a =
            *reinterpret_cast<const bf16x8*>(Kt + k_at<D>(16 * t + c16, 4 * c + g4));
        st[t] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, qb[c], st[t], 0, 0, 0);
      }
    }
    if (kb + KB > kend) {
#pragma unroll
      for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int r = 0; r < 4; ++r)
          if (kb + 16 * t + 4 * g4 + r >= kend) st[t][r] = kNegInf;
    }

    float mx = kNegInf;
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int r = 0; r < 4; ++r) mx = fmaxf(mx, st[t][r]);
    mx = fmaxf(mx, __shfl_xor(mx, 16));
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float m_new = fmaxf(M, mx * log2_scale);
    const float base = (m_new == kNegInf) ? 0.f : m_new;
    const float alpha = __builtin_amdgcn_exp2f(M - base);
    M = m_new;
    bf16x8 pb;
    float psum = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float p = __builtin_amdgcn_exp2f(fmaf(st[i >> 2][i & 3], log2_scale, -base));
      psum += p;
      pb[i] = (__bf16)p;
    }
    lsum = fmaf(alpha, lsum, psum);
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) acc[mt] *= alpha;

    __syncthreads();  // V^T of this block is in LDS
#pragma unroll
    for (int mt = 0; mt < D / 16; ++mt) {
      const bf16x8 a = *reinterpret_cast<const bf16x8*>(Vt + vt_at(16 * mt + c16, g4));
      acc[mt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, pb, acc[mt], 0, 0, 0);
    }
    if (more) cur = nxt;
  }

  float l = lsum + __shfl_xor(lsum, 16);
  l += __shfl_xor(l, 32);
  if (!qvalid) return;
  const size_t slot = ((size_t)b * Hq + hq) * splits + s;
  const float inv = (l > 0.f) ? 1.f / l : 0.f;
#pragma unroll
  for (int mt = 0; mt < D / 16; ++mt)
    *reinterpret_cast<f32x4*>(ws_o + slot * D + 16 * mt + 4 * g4) = acc[mt] * inv;
  if (g4 == 0) ws_lse[slot] = (l > 0.f) ? (M + __builtin_amdgcn_logf(l)) * kLn2 : kNegInf;
}

template <int D>
__global__ __launch_bounds__(128) void decode_combine_kernel(const float* __restrict__ ws_o,
                                                             const float* __restrict__ ws_lse,
                                                             __bf16* __restrict__ O,
                                                             float* __restrict__ LSE,
                                                             int splits) {
  const size_t row = blockIdx.x;  // b * Hq + h
  const int d = threadIdx.x;
  const float* lp = ws_lse + row * splits;
  float mx = kNegInf;
  for (int s = 0; s < splits; ++s) mx = fmaxf(mx, lp[s]);
  const float base = (mx == kNegInf) ? 0.f : mx;
  float tot = 0.f, o = 0.f;
  for (int s = 0; s < splits; ++s) {
    const float w = expf(lp[s] - base);
    tot += w;
    o = fmaf(w, ws_o[(row * splits + s) * D + d], o);
  }
  // no key at all (a paged sequence of length 0): O = 0, LSE = -inf
  O[row * D + d] = (__bf16)(tot > 0.f ? o / tot : 0.f);
  if (d == 0) LSE[row] = tot > 0.f ? base + logf(tot) : kNegInf;
}

template <int D>
hipError_t launch_t(const Problem& p, int k0, int splits, int chunk, float* ws_o, float* ws_lse,
                    hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const int nqg = (G + 15) / 16;
  const long long grid = (long long)p.B * p.Hkv * nqg * splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL || (long long)p.B * p.Hq > 0x7fffffffLL)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_partial_kernel<D, false>), dim3((unsigned)grid), dim3(64), 0,
                     stream, static_cast<const __bf16*>(p.Q), static_cast<const __bf16*>(p.K),
                     static_cast<const __bf16*>(p.V), ws_o, ws_lse, p.Hq, p.Hkv, p.Tk, k0,
                     splits, chunk, p.log2_scale, p.qsign, nullptr, nullptr, 0, 0, 0);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)(p.B * p.Hq)), dim3(D), 0, stream,
                     ws_o, ws_lse, static_cast<__bf16*>(p.O), p.LSE, splits);
  return hipGetLastError();
}

template <int D>
hipError_t launch_paged_t(const Problem& p, const PagedKV& pk, int splits, int chunk,
                          float* ws_o, float* ws_lse, hipStream_t stream) {
  const int G = p.Hq / p.Hkv;
  const int nqg = (G + 15) / 16;
  const long long grid = (long long)p.B * p.Hkv * nqg * splits;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL || (long long)p.B * p.Hq > 0x7fffffffLL)
    return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((decode_partial_kernel<D, true>), dim3((unsigned)grid), dim3(64), 0, stream,
                     static_cast<const __bf16*>(p.Q), static_cast<const __bf16*>(p.K),
                     static_cast<const __bf16*>(p.V), ws_o, ws_lse, p.Hq, p.Hkv, 0, 0, splits,
                     chunk, p.log2_scale, p.qsign, pk.table, pk.seq_lens, pk.max_blocks,
                     pk.bs_shift, pk.num_blocks);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(decode_combine_kernel<D>, dim3((unsigned)(p.B * p.Hq)), dim3(D), 0, stream,
                     ws_o, ws_lse, static_cast<__bf16*>(p.O), p.LSE, splits);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_decode_paged_bf16(const Problem& p, const PagedKV& pk, int splits, int chunk,
                                    float* ws_o, float* ws_lse, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_paged_t<32>(p, pk, splits, chunk, ws_o, ws_lse, stream);
    case 64: return launch_paged_t<64>(p, pk, splits, chunk, ws_o, ws_lse, stream);
    case 128: return launch_paged_t<128>(p, pk, splits, chunk, ws_o, ws_lse, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_decode_bf16(const Problem& p, int k0, int splits, int chunk, float* ws_o,
                              float* ws_lse, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_t<32>(p, k0, splits, chunk, ws_o, ws_lse, stream);
    case 64: return launch_t<64>(p, k0, splits, chunk, ws_o, ws_lse, stream);
    case 128: return launch_t<128>(p, k0, splits, chunk, ws_o, ws_lse, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace fattn
