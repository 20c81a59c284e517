// Backward pass of attention with recomputation, bf16 in and out, fp32 accumulation.
//
// "4.2 FlashAttention I: IO-Awareness & The Online Softmax" (section "The backward pass:
// recomputation instead of storage") and "Efficient attention & KV cache" (section 2.2, the
// backward with recomputation): the forward keeps only O and the per-row log-sum-exp L; the
// backward rebuilds each probability tile as P = exp(scale * Q K^T - L) instead of reading a
// stored T x T matrix, and with D_i = rowsum(dO o O)_i:
//   dV = P^T dO,   dP = dO V^T,   dS = P o (dP - D),   dQ = scale * dS K,   dK = scale * dS^T Q.
//
// Two kernels, none with atomics, so every result is bitwise reproducible run to run:
//  * bwd_dq_kernel (query-block outer loop, like the forward): a lane owns a query row. It first
//    forms its row's D_i and L_i * log2(e) and writes them to the workspace for the second
//    kernel, in 32-row blocks [L (32 floats), D (32 floats)] with rows past Tq holding L = +inf
//    and D = 0 (so their recomputed probabilities are exactly 0); packed batches use
//    [Hq, total_q] planes. It then streams the K and V tiles of its head; per tile S^T and dP^T
//    come from two MFMA products against Q^T and dO^T held in registers, dS is formed on the
//    VALU, and dQ^T += K^T dS^T reads the same K tile transposed. Software-pipelined like the
//    forward: the products of the next tile are issued together with the current tile's
//    exponentials.
//  * bwd_dkdv_kernel (key-block outer loop): a lane owns a key and holds V^T in registers; at
//    d = 128 the workgroup's K rows sit in LDS for its whole life (read as the K^T operand), which
//    keeps the kernel within 256 registers and so at two waves per SIMD (K^T stays in registers
//    at d <= 64, which fits two waves per SIMD anyway). It streams the Q, dO and (L, D)
//    tiles of every query head of its group, forms S and dP, then dV^T += dO^T P and
//    dK^T += Q^T dS. dK and dV of a key are accumulated in registers over all the query heads
//    that share it, so GQA needs no reduction pass.
// The split recomputes S and dP once per kernel (7 products instead of 5) in exchange for no
// atomic accumulation of dQ: the first page above notes that the usual key-outer order adds dQ
// with atomics and is therefore not reproducible run to run, and that a deterministic mode pays
// for reproducibility.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <type_traits>

#include "kernels.h"
#include "grid_order.h"
#include "lds_tiles.h"

namespace fattn {
namespace {

using namespace lds;

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2eF = 1.44269504088896340736f;
constexpr float kPosInf = __builtin_inff();

// A wave's 32 gradient rows (lane (col, hf) holds dims 32dt + 8g4 + 4hf .. +3 of row col in
// acc[dt][4g4 .. 4g4+3], the MFMA accumulator layout), times `mul`, rounded to bf16 and stored as
// whole rows: 16 rows at a time through the wave's 16-row share of four idle LDS stage arrays,
// 16-byte chunks XOR-swizzled by row, then one row-contiguous chunk per lane per store (instead
// of 8-byte pieces of 32 rows per instruction). Rows r < nvalid go to base + r * stride.
// Every wave of the workgroup must call it (it starts with a barrier: the stages are free).
template <int D, int BC, int NW>
__device__ __forceinline__ void store_rows(unsigned char* a0, unsigned char* a1,
                                           unsigned char* a2, unsigned char* a3, int wave,
                                           int lane, const f32x16 (&acc)[D / 32], float mul,
                                           __bf16* base, size_t stride, int nvalid) {
  using S = Shape<D, BC, NW>;
  constexpr int C = D / 8, HALF = 16 * S::RB, PER = S::TILE / HALF;
  static_assert(PER >= 1 && NW <= 4 * PER, "stage arrays too small for the row staging");
  const int col = lane & 31, hf = lane >> 5;
  const int arr = wave / PER;
  unsigned char* ob = (arr == 0 ? a0 : arr == 1 ? a1 : arr == 2 ? a2 : a3) + (wave % PER) * HALF;
  __syncthreads();
#pragma unroll
  for (int half = 0; half < 2; ++half) {
    if ((col >> 4) == half) {
      const int r = col & 15;
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const int c = 4 * dt + g4;
          u32x2 packed = {pack2_bf16(acc[dt][4 * g4 + 0] * mul, acc[dt][4 * g4 + 1] * mul),
                          pack2_bf16(acc[dt][4 * g4 + 2] * mul, acc[dt][4 * g4 + 3] * mul)};
          *(LDS_AS u32x2*)(ob + r * S::RB + ((c ^ (r % C)) << 4) + 8 * hf) = packed;
        }
    }
    // the wave's own LDS operations run in order: only the compiler must keep this order
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
#pragma unroll
    for (int i = 0; i < C / 4; ++i) {
      const int r = i * (64 / C) + lane / C, lc = lane % C;
      const u32x4 v = *(LDS_AS u32x4*)(ob + r * S::RB + ((lc ^ (r % C)) << 4));
      const int row = 16 * half + r;
      if (row < nvalid) *reinterpret_cast<u32x4*>(base + (size_t)row * stride + 8 * lc) = v;
    }
    __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
  }
}

// ---- dQ: one workgroup per (batch, query head, block of 32 * NW query rows).
// VARLEN: packed batch (Q, O, dO, dQ [total_q, Hq, D], K, V [total_k, Hkv, D], LSE
// [Hq, total_q]); blockIdx covers (sequence, head, query block) with Tq and Tk the longest
// lengths, and each workgroup takes its sequence's lengths from the offsets.
template <int D, int BC, int NW, bool VARLEN>
__global__ __launch_bounds__(64 * NW, 2) void bwd_dq_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ O, const __bf16* __restrict__ dO, const float* __restrict__ LSE,
    float* __restrict__ ws, __bf16* __restrict__ dQ, int Hq, int Hkv, int Tq, int Tk, int causal,
    int window, float scale, float c, const int* __restrict__ cu_q, const int* __restrict__ cu_k,
    int total_q, int total_k) {
  using S = Shape<D, BC, NW>;
  // One array per stage (K rotates through four, V through two; see the pipeline below), so
  // the compiler can tell a direct-to-LDS load into one stage from reads of another.
  __shared__ __align__(1024) unsigned char k_st0[S::TILE], k_st1[S::TILE];
  __shared__ __align__(1024) unsigned char k_st2[S::TILE], k_st3[S::TILE];
  __shared__ __align__(1024) unsigned char v_st0[S::TILE], v_st1[S::TILE];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;

  const int nqb = (Tq + S::BR - 1) / S::BR;
  // Dense batches: each XCD a contiguous range of whole heads, 4 heads at a time block-major
  // (blocks of one size dispatched together). Packed batches, whose sequences differ in length:
  // pairs dealt to the XCDs by head, 4 at a time block-major.
  int bh, qb;
  if (VARLEN) {
    xcd_grouped_pairs<4>(blockIdx.x, gridDim.x / nqb, nqb, bh, qb);
  } else {
    xcd_pair_groups<4>(blockIdx.x, gridDim.x, nqb, bh, qb);
  }
  if (causal) qb = nqb - 1 - qb;  // longest causal blocks first
  const int b = bh / Hq;
  const int h = bh - b * Hq;
  const int g = h / (Hq / Hkv);
  int q_begin = 0, k_begin = 0;
  if constexpr (VARLEN) {
    q_begin = min(max(cu_q[b], 0), total_q);
    const int q_stop = min(max(cu_q[b + 1], q_begin), total_q);
    k_begin = min(max(cu_k[b], 0), total_k);
    const int k_stop = min(max(cu_k[b + 1], k_begin), total_k);
    Tq = min(q_stop - q_begin, Tq);
    Tk = min(k_stop - k_begin, Tk);
    if (qb * S::BR >= Tq) return;  // the whole workgroup: past this sequence's rows
  }
  const int off = Tk - Tq;
  const int nqt = (Tq + 31) / 32;
  const size_t qstr = VARLEN ? (size_t)Hq * D : (size_t)D;   // elements between rows
  const size_t kstr = VARLEN ? (size_t)Hkv * D : (size_t)D;

  const __bf16* Qh = VARLEN ? Q + ((size_t)q_begin * Hq + h) * D : Q + (size_t)bh * Tq * D;
  const __bf16* dOh = VARLEN ? dO + ((size_t)q_begin * Hq + h) * D : dO + (size_t)bh * Tq * D;
  const __bf16* Kh = VARLEN ? K + ((size_t)k_begin * Hkv + g) * D
                            : K + ((size_t)b * Hkv + g) * (size_t)Tk * D;
  const __bf16* Vh = VARLEN ? V + ((size_t)k_begin * Hkv + g) * D
                            : V + ((size_t)b * Hkv + g) * (size_t)Tk * D;

  // key tiles: the same ranges as the forward pass of this query block
  const int i0 = qb * S::BR;
  const int q_end = min(i0 + S::BR, Tq);
  const int kv_end = causal ? min(Tk, q_end + off) : Tk;
  const int ntiles = (kv_end + BC - 1) / BC;
  int jm = Tk / BC;
  if (causal) jm = min(jm, (i0 + off + 1) / BC);
  jm = min(jm, ntiles);
  const int kv_beg = window > 0 ? max(0, i0 + off - window + 1) : 0;
  const int j_lo = kv_beg / BC;
  const int j_ul = window > 0 ? (max(0, q_end - 1 + off - window + 1) + BC - 1) / BC : 0;
  auto clean = [&](int j) { return j >= j_ul && j < jm; };

  // ---- this lane's query row: Q^T and dO^T operands, L and D
  const int qw0 = i0 + 32 * wave;
  const int qrow = qw0 + col;
  const bool wave_has_rows = qw0 < Tq;
  const int wave_last = min(qw0 + 31, Tq - 1);
  bf16x8 qb8[D / 16], ob8[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 rq = {0u, 0u, 0u, 0u}, ro = {0u, 0u, 0u, 0u};
    if (qrow < Tq) {
      rq = *reinterpret_cast<const u32x4*>(Qh + (size_t)qrow * qstr + 16 * kk + 8 * hf);
      ro = *reinterpret_cast<const u32x4*>(dOh + (size_t)qrow * qstr + 16 * kk + 8 * hf);
    }
    qb8[kk] = __builtin_bit_cast(bf16x8, rq);
    ob8[kk] = __builtin_bit_cast(bf16x8, ro);
  }
  // L * log2(e) and D = rowsum(dO * O) of this lane's row: this lane holds half of the row's
  // dims of dO (the other half is in lane ^ 32) and reads the same dims of O. They are written
  // to the workspace, in the layout the dK/dV kernel that follows on the stream reads (dense:
  // per 32-row block, 32 L then 32 D, rows past Tq +inf and 0; packed: [Hq, total_q] planes).
  float Lr = kPosInf, Dr = 0.f;
  {
    const __bf16* Oh = VARLEN ? O + ((size_t)q_begin * Hq + h) * D : O + (size_t)bh * Tq * D;
    float acc = 0.f;
    if (qrow < Tq) {
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 o = *reinterpret_cast<const bf16x8*>(Oh + (size_t)qrow * qstr + 16 * kk +
                                                          8 * hf);
#pragma unroll
        for (int k = 0; k < 8; ++k) acc = fmaf((float)o[k], (float)ob8[kk][k], acc);
      }
    }
    acc += __shfl_xor(acc, 32);
    if constexpr (VARLEN) {
      const size_t r = (size_t)h * total_q + q_begin + qrow;
      if (qrow < Tq) {
        Lr = LSE[r] * kLog2eF;
        Dr = acc;
        if (hf == 0) {
          ws[r] = Lr;
          ws[(size_t)Hq * total_q + r] = Dr;
        }
      }
    } else {
      if (qrow < Tq) {
        Lr = LSE[(size_t)bh * Tq + qrow] * kLog2eF;
        Dr = acc;
      }
      if (hf == 0 && qrow < nqt * 32) {
        float* blk = ws + ((size_t)bh * nqt + qrow / 32) * 64;
        blk[qrow % 32] = Lr;
        blk[32 + qrow % 32] = Dr;
      }
    }
  }

  const int krb = VARLEN ? (int)(kstr * 2) : S::RB;  // bytes between K (V) rows in memory
  int dvo[S::NI_W];
#pragma unroll
  for (int i = 0; i < S::NI_W; ++i) {
    const int q = wave + i * NW;
    const int r = q * S::RPI + lane / S::C;
    dvo[i] = r * krb + (((lane % S::C) ^ swz<D, BC, NW>(r)) << 4);
  }
  auto load_tile = [&](const __bf16* head, int j0, unsigned char* dst) {
    if constexpr (VARLEN)
      dma_tile_strided<D, BC, NW>(head, j0, Tk, (int)kstr, dst, wave, dvo);
    else
      dma_tile<D, BC, NW>(head, j0, Tk, dst, wave, dvo);
  };
  const int ka = rowbase<D, BC, NW>(col) ^ (hf << 4);
  const int vq = lane >> 5, vg = (lane >> 4) & 1, ve = (lane >> 2) & 3, va = lane & 3;
  int vab[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
    vab[rr] = (rowbase<D, BC, NW>(8 * rr + 4 * vq + ve) ^ ((2 * vg + (va >> 1)) << 4)) + 8 * (va & 1);

  // tile rows (keys) x this lane's row, against a register operand
  auto rows_x = [&](f32x16 (&s)[BC / 32], const unsigned char* st, const bf16x8 (&op)[D / 16]) {
#pragma unroll
    for (int t = 0; t < BC / 32; ++t) {
      s[t] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *(const LDS_AS bf16x8*)(st + ((ka ^ (kk << 5)) + 32 * t * S::RB));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op[kk], s[t], 0, 0, 0);
      }
    }
  };

  f32x16 acc[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

  auto active = [&](int j) {
    return wave_has_rows && (!causal || j * BC <= wave_last + off) &&
           (window == 0 || (j + 1) * BC - 1 >= qw0 + off - window + 1);
  };

  // S^T and dP^T of one key tile from its K and V stages
  auto sdp = [&](f32x16 (&s)[BC / 32], f32x16 (&dp)[BC / 32], const unsigned char* kst,
                 const unsigned char* vst) {
    rows_x(s, kst, qb8);
    rows_x(dp, vst, ob8);
  };
  // dS of key tile j, rounded to bf16. Two copies of the element loop, with and without the
  // mask, so that neither holds a branch.
  auto dsoft = [&](int j, const f32x16 (&s)[BC / 32], const f32x16 (&dp)[BC / 32],
                   bf16x8 (&ds)[BC / 16], auto with_mask) {
    // visible keys of the tile for this lane's row (relative to the tile start): key_lo..key_hi
    const int j0 = j * BC;
    const int key_hi = (causal ? min(Tk - 1, qrow + off) : Tk - 1) - j0;
    const int key_lo = (window > 0 ? qrow + off - window + 1 : 0) - j0;
#pragma unroll
    for (int ch = 0; ch < BC / 16; ++ch) {
      const int t = ch >> 1, c2 = ch & 1;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        const int r = 8 * c2 + i;
        float p = __builtin_amdgcn_exp2f(fmaf(s[t][r], c, -Lr));
        float v = p * (dp[t][r] - Dr);
        if constexpr (decltype(with_mask)::value) {
          const int kk = 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
          v = (kk > key_hi || kk < key_lo) ? 0.f : v;
        }
        ds[ch][i] = (__bf16)v;
      }
    }
  };
  // dQ^T += K^T dS^T: the K stage of the tile read transposed
  auto dq = [&](const bf16x8 (&ds)[BC / 16], const unsigned char* kst) {
#pragma unroll
    for (int ch = 0; ch < BC / 16; ++ch)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(kst + ((vab[0] ^ (dt << 6)) + 16 * ch * S::RB)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(kst + ((vab[1] ^ (dt << 6)) + 16 * ch * S::RB)));
        const bf16x8 a = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, ds[ch], acc[dt], 0, 0, 0);
      }
  };

  // Software pipeline over the key tiles: the step of tile j forms S^T and dP^T of tile j+1
  // (matrix cores) while it forms dS of tile j (VALU), then adds K^T dS^T of tile j, and loads
  // the K and V tiles of j+2. Tile j's K stage is still read (transposed) while tile j+2 loads,
  // so K rotates through four stages (three would do; four keep the rotation in step with the
  // two V stages and the two score buffers, so the unrolled steady state names every buffer
  // statically); V's stage of tile j is free once S^T and dP^T of tile j were formed a step
  // earlier, so V needs two.
  auto kst = [&](int i) { return i == 0 ? k_st0 : i == 1 ? k_st1 : i == 2 ? k_st2 : k_st3; };
  auto vst = [&](int i) { return i == 0 ? v_st0 : v_st1; };

  // Stages start cleared: a stage row past Tk is then zero or a finite leftover of an earlier
  // tile, and meets a zero dS.
  for (int i = tid; i < S::TILE / 16; i += S::NT) {
#pragma unroll
    for (int k = 0; k < 4; ++k) *(LDS_AS u32x4*)(kst(k) + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    *(LDS_AS u32x4*)(v_st0 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    *(LDS_AS u32x4*)(v_st1 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
  // prologue: tiles j_lo and j_lo+1 in stages 0 and 1; S^T and dP^T of tile j_lo
  if (j_lo < ntiles) {
    load_tile(Kh, j_lo * BC, k_st0);
    load_tile(Vh, j_lo * BC, v_st0);
  }
  if (j_lo + 1 < ntiles) {
    load_tile(Kh, (j_lo + 1) * BC, k_st1);
    load_tile(Vh, (j_lo + 1) * BC, v_st1);
  }
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  f32x16 sa[BC / 32], pa[BC / 32], sb[BC / 32], pb[BC / 32];
  if (j_lo < ntiles && active(j_lo)) sdp(sa, pa, k_st0, v_st0);
  __syncthreads();  // V stage 0 is free for tile j_lo + 2

  // steady state: tiles j, j+1 and j+2 are clean (every wave active, no mask)
  auto fast_step = [&](f32x16 (&sc)[BC / 32], f32x16 (&pc)[BC / 32], f32x16 (&sn)[BC / 32],
                       f32x16 (&pn)[BC / 32], int j, const unsigned char* k_cur,
                       const unsigned char* k_nxt, unsigned char* k_far,
                       const unsigned char* v_nxt, unsigned char* v_far) {
    load_tile(Kh, (j + 2) * BC, k_far);
    load_tile(Vh, (j + 2) * BC, v_far);
    bf16x8 ds[BC / 16];
    sdp(sn, pn, k_nxt, v_nxt);
    dsoft(j, sc, pc, ds, std::false_type{});
    dq(ds, k_cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  // general step: masks, inactive waves, the window's left band and the end of the pipeline
  auto general_step = [&](int j) {
    const int u = j - j_lo;
    const unsigned char* k_cur = kst(u & 3);
    const unsigned char* k_nxt = kst((u + 1) & 3);
    const unsigned char* v_nxt = vst((u + 1) & 1);
    if (j + 2 < ntiles) {
      load_tile(Kh, (j + 2) * BC, kst((u + 2) & 3));
      load_tile(Vh, (j + 2) * BC, vst(u & 1));
    }
    if (j + 1 < ntiles && active(j + 1)) sdp(sb, pb, k_nxt, v_nxt);
    if (active(j)) {
      bf16x8 ds[BC / 16];
      if (clean(j)) {
        dsoft(j, sa, pa, ds, std::false_type{});
      } else {
        dsoft(j, sa, pa, ds, std::true_type{});
      }
      dq(ds, k_cur);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
#pragma unroll
    for (int t = 0; t < BC / 32; ++t) {
      sa[t] = sb[t];
      pa[t] = pb[t];
    }
  };
  // left band of a window and the steps up to a multiple of four from j_lo, then the steady
  // state over clean tiles, then the rest
  int j = j_lo;
  for (; j < ntiles && (j < j_ul || ((j - j_lo) & 3) != 0); ++j) general_step(j);
  for (; j + 5 < jm; j += 4) {
    fast_step(sa, pa, sb, pb, j, k_st0, k_st1, k_st2, v_st1, v_st0);
    fast_step(sb, pb, sa, pa, j + 1, k_st1, k_st2, k_st3, v_st0, v_st1);
    fast_step(sa, pa, sb, pb, j + 2, k_st2, k_st3, k_st0, v_st1, v_st0);
    fast_step(sb, pb, sa, pa, j + 3, k_st3, k_st0, k_st1, v_st0, v_st1);
  }
  for (; j < ntiles; ++j) general_step(j);

  // rows qw0 .. qw0+31 of this head (packed batches keep Hq * D elements between rows)
  __bf16* rows = VARLEN ? dQ + ((size_t)(q_begin + qw0) * Hq + h) * D
                        : dQ + ((size_t)bh * Tq + qw0) * D;
  store_rows<D, BC, NW>(k_st0, k_st1, v_st0, v_st1, wave, lane, acc, scale, rows,
                        VARLEN ? (size_t)Hq * D : (size_t)D, Tq - qw0);
}

// ---- dK, dV: one workgroup per (batch, kv head, block of 32 * NW keys); the loop runs over the
// query heads of the group and the query tiles of BC rows that see a key of the block (the order
// is given with the step mapping below).
// VARLEN: packed batch, as for the dQ kernel; blockIdx covers (sequence, kv head, key block).
// KLDS: the workgroup's K rows live in LDS and are read as the K^T operand of every tile, instead
// of K^T in registers. At d = 128 this frees the 32 registers that bring the kernel within 256,
// so two waves run per SIMD instead of one.
template <int D, int BC, int NW, int MINW, bool KLDS, bool VARLEN>
__global__ __launch_bounds__(64 * NW, MINW) void bwd_dkdv_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    const __bf16* __restrict__ dO, const float* __restrict__ ws, __bf16* __restrict__ dK,
    __bf16* __restrict__ dV, int Hq, int Hkv, int Tq, int Tk, int causal, int window, float scale,
    float c, const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q,
    int total_k) {
  using S = Shape<D, BC, NW>;
  constexpr int BK = 32 * NW;     // keys per workgroup
  constexpr int LWB = BC / 32;    // (L, D) blocks per query tile
  static_assert(LWB <= NW, "one wave per (L, D) block");
  __shared__ __align__(1024) unsigned char q_st0[S::TILE], q_st1[S::TILE];
  __shared__ __align__(1024) unsigned char o_st0[S::TILE], o_st1[S::TILE];
  __shared__ __align__(16) float lw_st0[64 * LWB], lw_st1[64 * LWB];
  __shared__ __align__(1024) unsigned char k_blk[KLDS ? NW * S::TILE : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int col = lane & 31;
  const int hf = lane >> 5;

  const int nkb = (Tk + BK - 1) / BK;
  // grid order as in the dQ kernel; key blocks ascending: longest causal blocks first
  int bg, kb;
  if (VARLEN) {
    xcd_grouped_pairs<4>(blockIdx.x, gridDim.x / nkb, nkb, bg, kb);
  } else {
    xcd_pair_groups<4>(blockIdx.x, gridDim.x, nkb, bg, kb);
  }
  const int b = bg / Hkv;
  const int g = bg - b * Hkv;
  const int G = Hq / Hkv;
  const int k0 = kb * BK;
  int q_begin = 0, k_begin = 0;
  if constexpr (VARLEN) {
    q_begin = min(max(cu_q[b], 0), total_q);
    const int q_stop = min(max(cu_q[b + 1], q_begin), total_q);
    k_begin = min(max(cu_k[b], 0), total_k);
    const int k_stop = min(max(cu_k[b + 1], k_begin), total_k);
    Tq = min(q_stop - q_begin, Tq);
    Tk = min(k_stop - k_begin, Tk);
    if (k0 >= Tk) return;  // the whole workgroup: past this sequence's keys
  }
  const int off = Tk - Tq;
  const int nqt = (Tq + 31) / 32;
  const size_t qstr = VARLEN ? (size_t)Hq * D : (size_t)D;   // elements between rows
  const size_t kstr = VARLEN ? (size_t)Hkv * D : (size_t)D;

  const int kw0 = k0 + 32 * wave;
  const int kcol = kw0 + col;
  const int k_last = min(Tk - 1, k0 + BK - 1);
  const __bf16* Kh = VARLEN ? K + ((size_t)k_begin * Hkv + g) * D : K + (size_t)bg * Tk * D;
  const __bf16* Vh = VARLEN ? V + ((size_t)k_begin * Hkv + g) * D : V + (size_t)bg * Tk * D;

  // ---- this lane's key: the V^T operand, and K^T unless the K block is loaded into LDS below
  bf16x8 kb8[KLDS ? 1 : D / 16], vb8[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    u32x4 rv = {0u, 0u, 0u, 0u};
    if (kcol < Tk)
      rv = *reinterpret_cast<const u32x4*>(Vh + (size_t)kcol * kstr + 16 * kk + 8 * hf);
    vb8[kk] = __builtin_bit_cast(bf16x8, rv);
    if constexpr (!KLDS) {
      u32x4 rk = {0u, 0u, 0u, 0u};
      if (kcol < Tk)
        rk = *reinterpret_cast<const u32x4*>(Kh + (size_t)kcol * kstr + 16 * kk + 8 * hf);
      kb8[kk] = __builtin_bit_cast(bf16x8, rk);
    }
  }

  // ---- query rows that see a key of this block: causal rows from k0 - off on; under a window
  // rows up to k_last + window - 1 - off
  const int i_lo = causal ? max(0, k0 - off) : 0;
  const int i_hi = window > 0 ? min(Tq - 1, k_last + window - 1 - off) : Tq - 1;
  const int t_lo = i_lo / BC;
  const int ntq = i_lo <= i_hi ? i_hi / BC - t_lo + 1 : 0;
  const int nsteps = G * ntq;

  const int qrb = VARLEN ? (int)(qstr * 2) : S::RB;  // bytes between Q (dO) rows in memory
  int dvo[S::NI_W];
#pragma unroll
  for (int i = 0; i < S::NI_W; ++i) {
    const int q = wave + i * NW;
    const int r = q * S::RPI + lane / S::C;
    dvo[i] = r * qrb + (((lane % S::C) ^ swz<D, BC, NW>(r)) << 4);
  }
  int dvk[S::NI_W];
#pragma unroll
  for (int i = 0; i < S::NI_W; ++i) {
    const int q = wave + i * NW;
    const int r = q * S::RPI + lane / S::C;
    dvk[i] = r * (VARLEN ? (int)(kstr * 2) : S::RB) + (((lane % S::C) ^ swz<D, BC, NW>(r)) << 4);
  }
  const int ka = rowbase<D, BC, NW>(col) ^ (hf << 4);
  const int vq = lane >> 5, vg = (lane >> 4) & 1, ve = (lane >> 2) & 3, va = lane & 3;
  int vab[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
    vab[rr] = (rowbase<D, BC, NW>(8 * rr + 4 * vq + ve) ^ ((2 * vg + (va >> 1)) << 4)) + 8 * (va & 1);

  // Step s takes query tile t_lo + ntq - 1 - s / G of query head g*G + s % G: the tiles run from
  // the last one down, the heads of the group inner, so that the workgroups of one kv head, whose
  // first tiles differ under a causal mask, read the same Q and dO tiles at the same time (they
  // meet in L2) instead of each streaming the group's tiles from its own first tile.
  auto tile_of = [&](int s) { return t_lo + ntq - 1 - s / G; };
  // Q, dO and (L, D) tiles of step s
  auto issue = [&](int s, unsigned char* qst, unsigned char* ost, float* lw) {
    const int hh = g * G + s % G;
    const int q0 = tile_of(s) * BC;
    if constexpr (VARLEN) {
      const size_t head = (size_t)q_begin * Hq + hh;
      dma_tile_strided<D, BC, NW>(Q + head * D, q0, Tq, (int)qstr, qst, wave, dvo);
      dma_tile_strided<D, BC, NW>(dO + head * D, q0, Tq, (int)qstr, ost, wave, dvo);
      if (wave < LWB) {
        // lanes 0-31: L of rows q0 + 32*wave + lane, lanes 32-63: D of the same rows; rows past
        // the sequence are masked, rows past the batch read as zeros
        const size_t plane = (size_t)Hq * total_q;
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(ws), (short)0, (int)min(plane * 8, (size_t)0x7fffffff),
            kBufferFlags);
        const size_t r = (size_t)hh * total_q + q_begin + q0 + 32 * wave + (lane & 31);
        const size_t at = (lane < 32 ? r : plane + r) * 4;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lw + 64 * wave), 4,
                                                 (int)at, 0, 0, 0);
      }
    } else {
      const size_t bh = (size_t)b * Hq + hh;
      dma_tile<D, BC, NW>(Q + bh * Tq * D, q0, Tq, qst, wave, dvo);
      dma_tile<D, BC, NW>(dO + bh * Tq * D, q0, Tq, ost, wave, dvo);
      if (wave < LWB) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            const_cast<float*>(ws + bh * nqt * 64), (short)0, nqt * 256, kBufferFlags);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(lw + 64 * wave), 4,
                                                 (q0 / 32 + wave) * 256 + 4 * lane, 0, 0, 0);
      }
    }
  };

  f32x16 dk[D / 32], dv[D / 32];
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }

  // tile rows (queries) x this lane's key, against a register operand
  auto rows_x = [&](f32x16 (&s)[BC / 32], const unsigned char* st, const bf16x8 (&op)[D / 16]) {
#pragma unroll
    for (int t = 0; t < BC / 32; ++t) {
      s[t] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *(const LDS_AS bf16x8*)(st + ((ka ^ (kk << 5)) + 32 * t * S::RB));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, op[kk], s[t], 0, 0, 0);
      }
    }
  };
  // tile rows (queries) x this lane's key, against this wave's K tile in LDS
  auto rows_xk = [&](f32x16 (&s)[BC / 32], const unsigned char* st) {
    const unsigned char* kst = k_blk + wave * S::TILE;
#pragma unroll
    for (int t = 0; t < BC / 32; ++t) {
      s[t] = f32x16{};
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        const bf16x8 a = *(const LDS_AS bf16x8*)(st + ((ka ^ (kk << 5)) + 32 * t * S::RB));
        const bf16x8 bk = *(const LDS_AS bf16x8*)(kst + (ka ^ (kk << 5)));
        s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, bk, s[t], 0, 0, 0);
      }
    }
  };
  // acc^T += tile^T x (bf16 operand whose k index runs over the tile rows)
  auto tr_x = [&](f32x16 (&a)[D / 32], const bf16x8 (&pb)[BC / 16], const unsigned char* st) {
#pragma unroll
    for (int ch = 0; ch < BC / 16; ++ch)
#pragma unroll
      for (int dt = 0; dt < D / 32; ++dt) {
        const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(st + ((vab[0] ^ (dt << 6)) + 16 * ch * S::RB)));
        const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (LDS_AS i16x4*)(st + ((vab[1] ^ (dt << 6)) + 16 * ch * S::RB)));
        const bf16x8 m = __builtin_bit_cast(
            bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        a[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(m, pb[ch], a[dt], 0, 0, 0);
      }
  };

  auto compute = [&](int s, const unsigned char* qst, const unsigned char* ost, const float* lw) {
    const int q0 = tile_of(s) * BC;
    if (kw0 >= Tk || (causal && q0 + BC - 1 + off < kw0) ||
        (window > 0 && q0 + off - window + 1 > kw0 + 31))
      return;  // no row of the tile sees a key of this wave
    const bool masked = q0 + BC > Tq || (causal && q0 + off < kw0 + 31) ||
                        (window > 0 && q0 + BC - 1 + off - window + 1 > kw0);
    f32x16 sc[BC / 32], dp[BC / 32];
    if constexpr (KLDS) {
      rows_xk(sc, qst);
    } else {
      rows_x(sc, qst, kb8);
    }
    rows_x(dp, ost, vb8);
    bf16x8 pb[BC / 16], db[BC / 16];
    // visible rows of the tile for this lane's key (relative to q0); empty when row_hi < row_lo
    const int row_lo = causal ? max(0, kcol - off - q0) : 0;
    int row_hi = min(BC - 1, Tq - 1 - q0);
    if (window > 0) row_hi = min(row_hi, kcol - off + window - 1 - q0);
    // The element loop exists twice, with and without the mask, so that neither holds a branch:
    // a uniform test inside an unrolled element loop splits it into many small blocks.
    auto elements = [&](auto with_mask) {
#pragma unroll
      for (int ch = 0; ch < BC / 16; ++ch) {
        const int t = ch >> 1, c2 = ch & 1;
        // rows 32t + 16c2 + 4hf + {0..3} and 32t + 16c2 + 8 + 4hf + {0..3} of the tile
        const float* lb = lw + 64 * t + 16 * c2 + 4 * hf;
        const f32x4 l0 = *(const LDS_AS f32x4*)(lb), l1 = *(const LDS_AS f32x4*)(lb + 8);
        const f32x4 d0 = *(const LDS_AS f32x4*)(lb + 32), d1 = *(const LDS_AS f32x4*)(lb + 40);
        const float Lv[8] = {l0[0], l0[1], l0[2], l0[3], l1[0], l1[1], l1[2], l1[3]};
        const float Dv[8] = {d0[0], d0[1], d0[2], d0[3], d1[0], d1[1], d1[2], d1[3]};
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          const int r = 8 * c2 + i;
          float p = __builtin_amdgcn_exp2f(fmaf(sc[t][r], c, -Lv[i]));
          float v = p * (dp[t][r] - Dv[i]);
          if constexpr (decltype(with_mask)::value) {
            // rows row_lo .. row_hi of the query tile see this lane's key
            const int rr = 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
            const bool vis = rr >= row_lo && rr <= row_hi;
            p = vis ? p : 0.f;
            v = vis ? v : 0.f;
          }
          pb[ch][i] = (__bf16)p;
          db[ch][i] = (__bf16)v;
        }
      }
    };
    if (masked) {
      elements(std::true_type{});
    } else {
      elements(std::false_type{});
    }
    tr_x(dv, pb, ost);  // dV^T += dO^T P
    tr_x(dk, db, qst);  // dK^T += Q^T dS
  };

  // Stages start cleared (see the dQ kernel).
  for (int i = tid; i < S::TILE / 16; i += S::NT) {
    *(LDS_AS u32x4*)(q_st0 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    *(LDS_AS u32x4*)(q_st1 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    *(LDS_AS u32x4*)(o_st0 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    *(LDS_AS u32x4*)(o_st1 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < (KLDS ? NW : 0); ++w) {
    if constexpr (VARLEN) {
      dma_tile_strided<D, BC, NW>(Kh, k0 + 32 * w, Tk, (int)kstr, k_blk + w * S::TILE, wave, dvk);
    } else {
      dma_tile<D, BC, NW>(Kh, k0 + 32 * w, Tk, k_blk + w * S::TILE, wave, dvk);
    }
  }
  if (nsteps > 0) issue(0, q_st0, o_st0, lw_st0);
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  auto step = [&](int s, const unsigned char* q_cur, const unsigned char* o_cur,
                  const float* lw_cur, unsigned char* q_nxt, unsigned char* o_nxt, float* lw_nxt) {
    if (s + 1 < nsteps) issue(s + 1, q_nxt, o_nxt, lw_nxt);
    compute(s, q_cur, o_cur, lw_cur);
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
  };
  int s = 0;
  for (; s + 1 < nsteps; s += 2) {
    step(s, q_st0, o_st0, lw_st0, q_st1, o_st1, lw_st1);
    step(s + 1, q_st1, o_st1, lw_st1, q_st0, o_st0, lw_st0);
  }
  if (s < nsteps) step(s, q_st0, o_st0, lw_st0, q_st1, o_st1, lw_st1);

  // keys kw0 .. kw0+31 of this kv head (packed batches keep Hkv * D elements between rows)
  const size_t kstride = VARLEN ? (size_t)Hkv * D : (size_t)D;
  const size_t k_off = VARLEN ? ((size_t)(k_begin + kw0) * Hkv + g) * D : ((size_t)bg * Tk + kw0) * D;
  store_rows<D, BC, NW>(q_st0, q_st1, o_st0, o_st1, wave, lane, dk, scale, dK + k_off, kstride,
                        Tk - kw0);
  store_rows<D, BC, NW>(q_st0, q_st1, o_st0, o_st1, wave, lane, dv, 1.f, dV + k_off, kstride,
                        Tk - kw0);
}

// dQ and dK/dV launches with DQ_NW waves per dQ workgroup (32 * DQ_NW query rows) and KV_NW
// waves per dK/dV workgroup (32 * KV_NW keys).
template <int D, int DQ_NW, int KV_NW>
hipError_t launch_grads(const BwdProblem& p, const Packed* pk, float* ws, float c,
                        hipStream_t stream) {
  const __bf16* Q = static_cast<const __bf16*>(p.Q);
  const __bf16* K = static_cast<const __bf16*>(p.K);
  const __bf16* V = static_cast<const __bf16*>(p.V);
  const __bf16* dO = static_cast<const __bf16*>(p.dO);
  const int* cu_q = pk ? pk->cu_q : nullptr;
  const int* cu_k = pk ? pk->cu_k : nullptr;
  const int total_q = pk ? pk->total_q : 0, total_k = pk ? pk->total_k : 0;
  constexpr int DQ_BC = 32;
  const int nqb = (p.Tq + 32 * DQ_NW - 1) / (32 * DQ_NW);
  const dim3 dq_grid((unsigned)(p.B * p.Hq * nqb)), dq_block(64 * DQ_NW);
  const __bf16* O = static_cast<const __bf16*>(p.O);
  if (pk)
    bwd_dq_kernel<D, DQ_BC, DQ_NW, true><<<dq_grid, dq_block, 0, stream>>>(
        Q, K, V, O, dO, p.LSE, ws, static_cast<__bf16*>(p.dQ), p.Hq, p.Hkv, p.Tq, p.Tk,
        p.causal, p.window, p.scale, c, cu_q, cu_k, total_q, total_k);
  else
    bwd_dq_kernel<D, DQ_BC, DQ_NW, false><<<dq_grid, dq_block, 0, stream>>>(
        Q, K, V, O, dO, p.LSE, ws, static_cast<__bf16*>(p.dQ), p.Hq, p.Hkv, p.Tq, p.Tk,
        p.causal, p.window, p.scale, c, nullptr, nullptr, 0, 0);

  // K in LDS for the dK/dV workgroups of 4 and 8 waves at d = 128 (two waves per SIMD); K^T in
  // registers below (two waves per SIMD already at d <= 64)
  constexpr bool KLDS = D >= 128 && KV_NW >= 4;
  constexpr int KV_BC = 32, KV_MINW = (KLDS || D < 128) ? 2 : 1;
  const int nkb = (p.Tk + 32 * KV_NW - 1) / (32 * KV_NW);
  const dim3 kv_grid((unsigned)(p.B * p.Hkv * nkb)), kv_block(64 * KV_NW);
  if (pk)
    bwd_dkdv_kernel<D, KV_BC, KV_NW, KV_MINW, KLDS, true><<<kv_grid, kv_block, 0, stream>>>(
        Q, K, V, dO, ws, static_cast<__bf16*>(p.dK), static_cast<__bf16*>(p.dV), p.Hq, p.Hkv,
        p.Tq, p.Tk, p.causal, p.window, p.scale, c, cu_q, cu_k, total_q, total_k);
  else
    bwd_dkdv_kernel<D, KV_BC, KV_NW, KV_MINW, KLDS, false><<<kv_grid, kv_block, 0, stream>>>(
        Q, K, V, dO, ws, static_cast<__bf16*>(p.dK), static_cast<__bf16*>(p.dV), p.Hq, p.Hkv,
        p.Tq, p.Tk, p.causal, p.window, p.scale, c, nullptr, nullptr, 0, 0);
  return hipGetLastError();
}

template <int D>
hipError_t launch_d(const BwdProblem& p, const Packed* pk, float* ws, hipStream_t stream) {
  const float c = p.scale * kLog2eF;
  // (L, D) of every row are formed by the dQ kernel itself, which writes them to the workspace
  // for the dK/dV kernel that follows (no separate pass over O and dO).
  // Workgroup size by the keys an average row sees (half the longest sequence when causal, at
  // most the window). Up to 2048: 4-wave dQ workgroups (128 query rows), whose doubled workgroup
  // count balances the CUs better (against 8 waves 16-21% faster on causal d = 64 and 128 at
  // T = 1024 and 2048 and 5% on a packed batch of 35 documents up to 4096 tokens). Beyond,
  // 8-wave dQ workgroups, which read K and V half as often per query row. dK/dV workgroups at
  // d = 128 keep their K block in LDS and run two waves per SIMD: 4 waves up to 2048 (3-9%
  // faster than 2 waves with K^T in registers at T = 1024 to 4096), 8 beyond (one workgroup per
  // CU: causal T = 8192 and 16384 8% faster than 4 waves with K^T in registers). At d <= 64, 2
  // and 4 waves with K^T in registers.
  long long seen = p.causal ? p.Tk / 2 : p.Tk;
  if (p.window > 0 && p.window < seen) seen = p.window;
  if constexpr (D >= 128) {
    if (seen <= 2048) return launch_grads<D, 4, 4>(p, pk, ws, c, stream);
    return launch_grads<D, 8, 8>(p, pk, ws, c, stream);
  } else {
    if (seen <= 2048) return launch_grads<D, 4, 2>(p, pk, ws, c, stream);
    return launch_grads<D, 8, 4>(p, pk, ws, c, stream);
  }
}

hipError_t launch_any(const BwdProblem& p, const Packed* pk, float* ws, hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_d<32>(p, pk, ws, stream);
    case 64: return launch_d<64>(p, pk, ws, stream);
    case 128: return launch_d<128>(p, pk, ws, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_backward_bf16(const BwdProblem& p, float* ws, hipStream_t stream) {
  return launch_any(p, nullptr, ws, stream);
}

hipError_t launch_backward_varlen_bf16(const BwdProblem& p, const Packed& pk, float* ws,
                                       hipStream_t stream) {
  return launch_any(p, &pk, ws, stream);
}

}  // namespace fattn
