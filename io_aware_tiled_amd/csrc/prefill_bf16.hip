// bf16 prefill kernel for gfx950: one workgroup per (batch, query head, query block), or per
// pair of query blocks of one (batch, head).
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
//    accumulation. Scores are formed transposed, S^T = K Q^T, so a lane holds one query row
//    (lane % 32) and 16 keys per 32x32 tile: row max and row sum are in-lane except for one
//    exchange between the half-waves (v_permlane32_swap).
//  * the output is accumulated transposed too, O^T = V^T P^T. The P^T operand is the S^T
//    accumulator converted to bf16 in place; the MFMA reduction index may be any permutation of
//    the keys as long as both operands use it, and the V^T operand is assembled in that key order
//    by LDS transpose reads (ds_read_b64_tr_b16) from V stored row-major.
//  * K and V tiles travel global -> LDS by direct-to-LDS buffer loads (no registers, no LDS store
//    instructions), two stages each, with K one tile ahead of V. Rows are stored with their
//    16-byte chunks XOR-swizzled so both the K operand reads and the transpose reads of V are
//    free of bank conflicts. Rows past Tk come back as zeros from the buffer range check.
//  * software pipeline: while the exponentials of tile j run on the VALU, the matrix cores
//    compute the scores of tile j+1; while the PV products of tile j run, the VALU takes the row
//    maxima of tile j+1. Tiles that need a mask (causal diagonal, ragged end) take a separate,
//    non-interleaved path.
//  * exponentials are exp2 with log2(e) folded into the scale. The exponent base moves lazily:
//    only when a row's maximum exceeds it by more than kRebase (log2 units) are l and the
//    accumulator rescaled. Any base gives the same O = acc / l and LSE = base + log l
//    ("Efficient attention & KV cache", section 2.1: the max is there only for numerical
//    safety); weights stay below 2^kRebase. For d <= 64 the steady state skips the row maximum
//    altogether: it forms the weights against the current base and falls back to the maximum
//    and a re-base only when a lane's sum of them (which bounds each one) exceeds 2^13.
//  * the row sum adds the bf16 weights the PV product uses (v_dot2 against ones).
#include <hip/hip_runtime.h>

#include <cstdint>

#include "kernels.h"
#include "grid_order.h"
#include "lds_tiles.h"

namespace fattn {
namespace {

using namespace lds;

constexpr float kRebase = 8.0f;  // lazy re-base threshold, log2 units

// VARLEN: packed variable-length batch. Q, O are [total_q, Hq, D], K, V [total_k, Hkv, D] and
// LSE [Hq, total_q]; sequence b owns query rows cu_q[b] .. cu_q[b+1]-1 and key rows
// cu_k[b] .. cu_k[b+1]-1 (clamped to the totals), B is the number of sequences and Tq_in, Tk_in
// arrive as the longest lengths the grid was sized for. Otherwise Q, O are [B, Hq, Tq, D], K, V
// [B, Hkv, Tk, D] and LSE [B, Hq, Tq].
//
// PAIRED (dense batches only): every workgroup runs two query blocks of one (batch, head), block
// qb and its mirror nqb-1-qb, one after the other. Under a causal mask the two together always
// span nqb+1 block lengths of keys, so every workgroup has the same work and the rounds of the
// grid stay balanced; the second block's Q is loaded into LDS while the first runs and its first
// K and V tiles are issued as soon as the first block's output has left the stages, so the
// second block starts without a workgroup's launch, drain and cold loads. The two iterations are
// unrolled: a loop back-edge around the tile loops would keep its loop-carried and hoisted
// values live through every tile step, past what two waves per SIMD can hold.
template <int D, int BC, int NW, bool VARLEN, bool PAIRED>
__global__ __launch_bounds__(64 * NW, 2) void prefill_bf16_kernel(
    const __bf16* __restrict__ Q, const __bf16* __restrict__ K, const __bf16* __restrict__ V,
    __bf16* __restrict__ O, float* __restrict__ LSE, int B, int Hq, int Hkv, int Tq_in, int Tk_in,
    int causal, int window, float log2_scale, int qsign, int schedule,
    const int* __restrict__ cu_q, const int* __restrict__ cu_k, int total_q, int total_k) {
  using S = Shape<D, BC, NW>;
  static_assert(!(PAIRED && VARLEN), "paired blocks serve dense batches");
  // d <= 64: the steady state takes no row maximum unless the weights could grow too large (the
  // exponentials and the few other VALU instructions per score bound the step at these sizes;
  // at d = 128 the scores kept live for the check would spill)
  constexpr bool NOMAX = D <= 64;
  // One array per stage, so the compiler can tell a direct-to-LDS load into one stage from reads
  // of another and does not make those reads wait for the load.
  __shared__ __align__(1024) unsigned char k_st0[S::TILE], k_st1[S::TILE];
  __shared__ __align__(1024) unsigned char v_st0[S::TILE], v_st1[S::TILE];
  // paired blocks: the second block's Q (rows laid out like a K tile). (Its smaller alignment
  // keeps it after the stages, whose reads then fit the 16-bit offset field of ds_read.)
  using QS = Shape<D, S::BR, NW>;
  __shared__ __align__(256) unsigned char q_st[PAIRED ? QS::TILE : 16];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int col = lane & 31;   // query row within the wave (MFMA column)
  const int hf = lane >> 5;    // half-wave

  const int nqb = (Tq_in + S::BR - 1) / S::BR;
  const int total = B * Hq * nqb;
  // elements between consecutive rows of one head
  const size_t qstr = VARLEN ? (size_t)Hq * D : (size_t)D;
  const size_t kstr = VARLEN ? (size_t)Hkv * D : (size_t)D;

  // ---- per-lane constant offsets
  // direct-to-LDS loads: LDS slot `lane` of load q holds row q*RPI + lane/C, physical chunk
  // lane%C, i.e. logical chunk (lane%C) ^ swz(row) of that row
  const int krb = VARLEN ? (int)(kstr * 2) : S::RB;  // bytes between K (V) rows in memory
  int dvo[S::NI_W];
#pragma unroll
  for (int i = 0; i < S::NI_W; ++i) {
    const int q = wave + i * NW;
    const int r = q * S::RPI + lane / S::C;
    dvo[i] = r * krb + (((lane % S::C) ^ swz<D, BC, NW>(r)) << 4);
  }
  // K operand of row col, chunk 2kk+hf: ka ^ (kk << 5), plus 32t rows for the t-th key half
  const int ka = rowbase<D, BC, NW>(col) ^ (hf << 4);
  // V^T operand by transpose reads: lane = 16*(2*vq + vg) + 4*ve + va reads 4 d-values starting
  // at 32*dt + 16*vg + 4*va of key row 16*ch + 8*rr + 4*vq + ve (rr = 0, 1 for the two reads)
  const int vq = lane >> 5, vg = (lane >> 4) & 1, ve = (lane >> 2) & 3, va = lane & 3;
  int vab[2];
#pragma unroll
  for (int rr = 0; rr < 2; ++rr)
    vab[rr] = (rowbase<D, BC, NW>(8 * rr + 4 * vq + ve) ^ ((2 * vg + (va >> 1)) << 4)) + 8 * (va & 1);

  // The block geometry below divides by runtime sizes. With paired blocks each block reads
  // copies of those sizes made opaque at its start, so the compiler computes the second
  // block's values where they are needed instead of sharing them with the first block's and
  // keeping them live (or spilled) through the first block's tile steps.
  int dHq = Hq, dHkv = Hkv, dTq = Tq_in, dTk = Tk_in;
  auto opaque_sizes = [&]() {
    if constexpr (PAIRED) asm volatile("" : "+s"(dHq), "+s"(dHkv), "+s"(dTq), "+s"(dTk));
  };

  // ---- which (batch, head, query block) position `id` of the grid order names
  auto locate = [&](int id, int& bh, int& qb) {
    bh = id / nqb;
    qb = id - bh * nqb;
    // schedule 2: whole heads per XCD, 8 heads at a time query-block-major
    if (schedule == 2) xcd_pair_groups<8>(id, total, nqb, bh, qb);
    // schedule 3, for packed batches: pairs dealt to the XCDs by head, 4 at a time block-major
    if (schedule == 3) xcd_grouped_pairs<4>(id, total / nqb, nqb, bh, qb);
    if (schedule >= 2 && causal) qb = nqb - 1 - qb;  // longest causal blocks first
  };

  // ---- one block's geometry
  struct Item {
    int b, h, Tq, Tk, q_begin, i0, q_end, ntiles, jm, j_lo, j_ul;
    const __bf16 *Qh, *Kh, *Vh;
  };
  auto make_item = [&](int bh, int qb) {
    Item it;
    it.b = bh / dHq;
    it.h = bh - it.b * dHq;
    const int g = it.h / (dHq / dHkv);
    int Tq = dTq, Tk = dTk;
    // packed batches: this sequence's rows and lengths (the documents do not see each other)
    int q_begin = 0, k_begin = 0;
    if constexpr (VARLEN) {
      q_begin = min(max(cu_q[it.b], 0), total_q);
      const int q_stop = min(max(cu_q[it.b + 1], q_begin), total_q);
      k_begin = min(max(cu_k[it.b], 0), total_k);
      const int k_stop = min(max(cu_k[it.b + 1], k_begin), total_k);
      Tq = min(q_stop - q_begin, Tq);
      Tk = min(k_stop - k_begin, Tk);
    }
    it.Tq = Tq;
    it.Tk = Tk;
    it.q_begin = q_begin;
    const int off = Tk - Tq;
    it.Qh = VARLEN ? Q + ((size_t)q_begin * dHq + it.h) * D
                   : Q + ((size_t)it.b * dHq + it.h) * (size_t)Tq * D;
    it.Kh = VARLEN ? K + ((size_t)k_begin * dHkv + g) * D
                   : K + ((size_t)it.b * dHkv + g) * (size_t)Tk * D;
    it.Vh = VARLEN ? V + ((size_t)k_begin * dHkv + g) * D
                   : V + ((size_t)it.b * dHkv + g) * (size_t)Tk * D;
    it.i0 = qb * S::BR;
    it.q_end = min(it.i0 + S::BR, Tq);
    const int kv_end = causal ? min(Tk, it.q_end + off) : Tk;
    it.ntiles = (kv_end + BC - 1) / BC;
    // tiles [0, jm) hold no key past any row's diagonal or past Tk
    int jm = Tk / BC;
    if (causal) jm = min(jm, (it.i0 + off + 1) / BC);
    it.jm = min(jm, it.ntiles);
    // Sliding window: the first row's window starts at key kv_beg, so the loop starts at tile
    // j_lo; tiles from j_ul on start at or after the last row's window edge, so no row hides
    // any of their keys on the left. Tiles in [j_ul, jm) need no mask at all.
    const int kv_beg = window > 0 ? max(0, it.i0 + off - window + 1) : 0;
    it.j_lo = kv_beg / BC;
    it.j_ul = window > 0 ? (max(0, it.q_end - 1 + off - window + 1) + BC - 1) / BC : 0;
    return it;
  };

  auto issue_tile = [&](const __bf16* head, int j0, int Tk, unsigned char* dst) {
    if constexpr (VARLEN)
      dma_tile_strided<D, BC, NW>(head, j0, Tk, (int)kstr, dst, wave, dvo);
    else
      dma_tile<D, BC, NW>(head, j0, Tk, dst, wave, dvo);
  };
  // first tiles of a block: K(j_lo), V(j_lo) into stage 0, K(j_lo + 1) into stage 1
  auto issue_prologue = [&](const Item& it) {
    issue_tile(it.Kh, it.j_lo * BC, it.Tk, k_st0);
    issue_tile(it.Vh, it.j_lo * BC, it.Tk, v_st0);
    if (it.j_lo + 1 < it.ntiles) issue_tile(it.Kh, (it.j_lo + 1) * BC, it.Tk, k_st1);
  };
  // persistent grid: a block's BR query rows into q_st by direct-to-LDS loads (rows past Tq are
  // not read)
  // (The per-lane offsets of the block-boundary work below are derived from an opaque copy of
  // the lane index: otherwise the compiler hoists them out of the persistent block loop and
  // keeps them live, or spilled, through every tile step.)
  auto opaque_lane = [&]() {
    int l = lane;
    if constexpr (PAIRED) asm volatile("" : "+v"(l));
    return l;
  };
  auto issue_q = [&](const Item& it) {
    if constexpr (PAIRED) {
      const __amdgpu_buffer_rsrc_t rs = rows_rsrc<D>(it.Qh, it.i0, it.Tq);
      const int ln = opaque_lane();
#pragma unroll
      for (int i = 0; i < QS::NI_W; ++i) {
        const int q = wave + i * NW;
        const int r = q * QS::RPI + ln / QS::C;
        const int off = r * QS::RB + (((ln % QS::C) ^ swz<D, S::BR, NW>(r)) << 4);
        if (QS::NI % NW == 0 || q < QS::NI)
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(q_st + q * 1024), 16, off,
                                                   0, 0, 0);
      }
    }
  };
  // rows past the sequence or a zero scale read as zeros; a negative scale negates Q exactly
  auto signed_q = [&](u32x4 raw, bool valid) {
    if (!valid || qsign == 0) raw = u32x4{0u, 0u, 0u, 0u};
    if (qsign < 0) raw ^= 0x80008000u;  // exact negation of both bf16 halves
    return __builtin_bit_cast(bf16x8, raw);
  };
  // the Q^T operand of this lane's row from q_st
  bf16x8 qb8[D / 16];
  auto q_from_lds = [&](const Item& it) {
    const int ln = opaque_lane();
    const int r = 32 * wave + (ln & 31);
    const int qa = rowbase<D, S::BR, NW>(r) ^ ((ln >> 5) << 4);
    const bool valid = it.i0 + r < it.Tq;
#pragma unroll
    for (int kk = 0; kk < D / 16; ++kk)
      qb8[kk] = signed_q(*(const LDS_AS u32x4*)(q_st + (qa ^ (kk << 5))), valid);
  };
  auto clear_v = [&]() {
    for (int i = tid; i < S::TILE / 16; i += S::NT) {
      *(LDS_AS u32x4*)(v_st0 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
      *(LDS_AS u32x4*)(v_st1 + 16 * i) = u32x4{0u, 0u, 0u, 0u};
    }
  };

  // ---- this workgroup's block(s)
  int bh, qb, qb2 = -1;
  if constexpr (PAIRED) {
    // pair p of a (batch, head): blocks nqb-1-p (the longer under a causal mask) and p; the
    // pairs of the grid are dealt to the XCDs in contiguous ranges, so each XCD works through
    // whole heads
    const int npb = (nqb + 1) / 2;
    const int id = xcd_contiguous(blockIdx.x, B * Hq * npb);
    bh = id / npb;
    const int pr = id - bh * npb;
    qb = nqb - 1 - pr;
    if (pr != qb) qb2 = pr;
  } else {
    locate(blockIdx.x, bh, qb);
  }
  {
    const Item cur = make_item(bh, qb);
    if constexpr (VARLEN) {
      if (cur.i0 >= cur.Tq) return;  // the whole workgroup: past this sequence's rows
    }
    if constexpr (PAIRED) {
      issue_q(cur);
      // (with Tk a multiple of BC every row a PV product reads is loaded; otherwise the V
      // stages start cleared, and the first block leaves only finite V rows behind)
      if (cur.Tk % BC != 0) {
        clear_v();
        __syncthreads();
      }
    } else {
      // ---- this wave's query rows; Q^T operand held in registers for the whole loop
      const int qrow = cur.i0 + 32 * wave + col;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        u32x4 raw = {0u, 0u, 0u, 0u};
        if (qrow < cur.Tq && qsign != 0)
          raw = *reinterpret_cast<const u32x4*>(cur.Qh + (size_t)qrow * qstr + 16 * kk + 8 * hf);
        qb8[kk] = signed_q(raw, qrow < cur.Tq);
      }
      // rows past Tk must never hold non-finite leftovers in a V stage (with Tk a multiple of
      // BC every row a PV product reads is loaded, and the clear is skipped)
      if (cur.Tk % BC != 0) {
        clear_v();
        __syncthreads();
      }
    }
    issue_prologue(cur);
  }

#pragma unroll
  for (int it = 0; it < (PAIRED ? 2 : 1); ++it) {
    if (it == 1 && qb2 < 0) break;
    opaque_sizes();
    const Item cur = make_item(bh, it == 0 ? qb : qb2);
    const int Tq = cur.Tq, Tk = cur.Tk, off = Tk - Tq;
    const int i0 = cur.i0, ntiles = cur.ntiles, jm = cur.jm;
    const int j_lo = cur.j_lo, j_ul = cur.j_ul;
    const __bf16 *Kh = cur.Kh, *Vh = cur.Vh;
    auto clean = [&](int j) { return j >= j_ul && j < jm; };

    const int qw0 = i0 + 32 * wave;
    const int qrow = qw0 + col;
    const bool wave_has_rows = qw0 < Tq;
    const int wave_last = min(qw0 + 31, Tq - 1);

    // S^T for one tile from a K stage
    auto qk = [&](f32x16 (&s)[BC / 32], const unsigned char* kst) {
#pragma unroll
      for (int t = 0; t < BC / 32; ++t) {
        s[t] = f32x16{};
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          const bf16x8 a = *(const LDS_AS bf16x8*)(kst + ((ka ^ (kk << 5)) + 32 * t * S::RB));
          s[t] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, qb8[kk], s[t], 0, 0, 0);
        }
      }
    };

    // d = 128: key j0 + 4*hf + k of element (t, r) has k = 32t + 8(r/4) + r%4, a constant; the
    // bounds move into this lane's frame once, and without a window only the upper one is
    // tested (0.5% on causal shapes; at d <= 64 the two versions cost registers and occupancy)
    auto mask_tile = [&](f32x16 (&s)[BC / 32], int j0) {
      if constexpr (D == 128) {
        const int base = j0 + 4 * hf;
        const int hi = (causal ? min(Tk - 1, qrow + off) : Tk - 1) - base;
        if (window == 0) {
#pragma unroll
          for (int t = 0; t < BC / 32; ++t)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (32 * t + 8 * (r >> 2) + (r & 3) > hi) s[t][r] = kNegInf;
          return;
        }
      }
      const int last = causal ? min(Tk - 1, qrow + off) : Tk - 1;
      const int first_key = window > 0 ? qrow + off - window + 1 : 0;
#pragma unroll
      for (int t = 0; t < BC / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = j0 + 32 * t + 8 * (r >> 2) + 4 * hf + (r & 3);
          if (key > last || key < first_key) s[t][r] = kNegInf;
        }
    };

    // ---- running state (M: exponent base of this lane's row, log2 units of the scaled scores)
    float M = kNegInf;
    float lsum = 0.f;  // this lane's share of the row sum (half of the keys of each tile)
    f32x16 acc[D / 32];
#pragma unroll
    for (int dt = 0; dt < D / 32; ++dt) acc[dt] = f32x16{};

    // row maximum of a score tile and the lazy re-base of the running state
    auto rebase = [&](f32x16 (&s)[BC / 32]) {
      float mx = kNegInf;
#pragma unroll
      for (int t = 0; t < BC / 32; ++t)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[t][r]);
      float m_lo, m_hi;
      halves(mx, m_lo, m_hi);
      mx = fmaxf(m_lo, m_hi);
      const float mt = mx * log2_scale;
      const bool grow = mt > M + kRebase;  // always true on the first tile a row sees
      if (__builtin_amdgcn_ballot_w64(grow) != 0) {
        const float m_new = grow ? mt : M;
        // 0 when M leaves -inf; 1 for a row that still has seen no key (under a sliding window
        // a row's first tiles can be fully masked while other rows of the wave move their base)
        const float alpha = m_new == kNegInf ? 1.f : __builtin_amdgcn_exp2f(M - m_new);
        lsum *= alpha;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) acc[dt] *= alpha;
        M = m_new;
      }
    };

    // weights of a score tile (bf16) and their row sum
    auto weights = [&](f32x16 (&s)[BC / 32], bf16x8 (&pb)[BC / 16]) {
      const float base = (M == kNegInf) ? 0.f : M;
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
#pragma unroll
      for (int ch = 0; ch < BC / 16; ++ch) {
        const int t = ch >> 1, c2 = ch & 1;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t][8 * c2 + i], log2_scale, -base));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t][8 * c2 + i + 1], log2_scale, -base));
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          lsum = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, lsum, false);
          pb[ch][i] = pp[0];
          pb[ch][i + 1] = pp[1];
        }
      }
    };

    // weights of a score tile against the current base, with this lane's sum of them
    auto weights_sum = [&](f32x16 (&s)[BC / 32], bf16x8 (&pb)[BC / 16]) {
      const float base = (M == kNegInf) ? 0.f : M;
      const bf16x2 ones = {(__bf16)1.f, (__bf16)1.f};
      float ts = 0.f;
#pragma unroll
      for (int ch = 0; ch < BC / 16; ++ch) {
        const int t = ch >> 1, c2 = ch & 1;
#pragma unroll
        for (int i = 0; i < 8; i += 2) {
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[t][8 * c2 + i], log2_scale, -base));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[t][8 * c2 + i + 1], log2_scale, -base));
          const bf16x2 pp = {(__bf16)p0, (__bf16)p1};
          ts = __builtin_amdgcn_fdot2_f32_bf16(pp, ones, ts, false);
          pb[ch][i] = pp[0];
          pb[ch][i + 1] = pp[1];
        }
      }
      return ts;
    };

    // O^T += V^T P^T for one tile from a V stage
    auto pv = [&](const bf16x8 (&pb)[BC / 16], const unsigned char* vst) {
#pragma unroll
      for (int ch = 0; ch < BC / 16; ++ch)
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt) {
          const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (LDS_AS i16x4*)(vst + ((vab[0] ^ (dt << 6)) + 16 * ch * S::RB)));
          const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
              (LDS_AS i16x4*)(vst + ((vab[1] ^ (dt << 6)) + 16 * ch * S::RB)));
          const bf16x8 a = __builtin_bit_cast(
              bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
          acc[dt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, pb[ch], acc[dt], 0, 0, 0);
        }
    };

    // this wave's rows see a key of tile j: not past the diagonal of its last row, not before
    // the window of its first row
    auto active = [&](int j) {
      return wave_has_rows && (!causal || j * BC <= wave_last + off) &&
             (window == 0 || (j + 1) * BC - 1 >= qw0 + off - window + 1);
    };

    // ---- prologue: K(j_lo), V(j_lo), K(j_lo+1) are in flight (issued above, or at the end of
    // the first block of a pair); scores, mask and maximum of tile j_lo. Stages alternate with
    // j - j_lo.
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();
    if constexpr (PAIRED) q_from_lds(cur);
    f32x16 sa[BC / 32], sb[BC / 32];
    if (active(j_lo)) {
      qk(sa, k_st0);
      if (!clean(j_lo)) mask_tile(sa, j_lo * BC);
      rebase(sa);
    }
    __syncthreads();
    // paired blocks: every wave has its Q in registers, so q_st takes the second block's rows
    if constexpr (PAIRED) {
      if (it == 0 && qb2 >= 0) {
        opaque_sizes();
        issue_q(make_item(bh, qb2));
      }
    }

    // ---- steady state: tiles j, j+1 and j+2 need no mask (so every wave is active). Unrolled
    // by two so the score buffers and LDS stages alternate without copies.
    auto fast_step = [&](f32x16 (&sc)[BC / 32], f32x16 (&sn)[BC / 32], int j,
                         unsigned char* k_cur, unsigned char* k_nxt, unsigned char* v_cur,
                         unsigned char* v_nxt) {
      const int j0 = j * BC;
      issue_tile(Vh, j0 + BC, Tk, v_nxt);
      issue_tile(Kh, j0 + 2 * BC, Tk, k_cur);
      bf16x8 pb[BC / 16];
      qk(sn, k_nxt);
      if constexpr (NOMAX) {
        // weights against the current base; the row maximum only when a lane's weights could
        // exceed 2^13 (their sum bounds each of them)
        float ts = weights_sum(sc, pb);
        if (__builtin_amdgcn_ballot_w64(!(ts <= 8192.f)) != 0) {
          rebase(sc);
          ts = weights_sum(sc, pb);
        }
        lsum += ts;
        pv(pb, v_cur);
      } else {
        weights(sc, pb);
        pv(pb, v_cur);
        rebase(sn);
      }
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
    };
    // ---- general step: masks, inactive waves, the window's left band and the end of the
    // pipeline
    auto general_step = [&](int j) {
      const int j0 = j * BC;
      const bool odd = ((j - j_lo) & 1) != 0;
      unsigned char* k_cur = odd ? k_st1 : k_st0;
      unsigned char* k_nxt = odd ? k_st0 : k_st1;
      unsigned char* v_cur = odd ? v_st1 : v_st0;
      unsigned char* v_nxt = odd ? v_st0 : v_st1;
      // no loads of tiles past the last one: the step's closing wait would wait for them
      if (j + 1 < ntiles) issue_tile(Vh, j0 + BC, Tk, v_nxt);
      if (j + 2 < ntiles) issue_tile(Kh, j0 + 2 * BC, Tk, k_cur);
      const bool act_next = (j + 1 < ntiles) && active(j + 1);
      if (act_next) {
        qk(sb, k_nxt);
        if (!clean(j + 1)) mask_tile(sb, j0 + BC);
      }
      if (active(j)) {
        bf16x8 pb[BC / 16];
        weights(sa, pb);
        pv(pb, v_cur);
      }
      if (act_next) rebase(sb);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
#pragma unroll
      for (int t = 0; t < BC / 32; ++t) sa[t] = sb[t];
    };
    // left band of a window (and one step to reach an even stage parity), then the steady
    // state over clean tiles, then the rest
    int j = j_lo;
    for (; j < ntiles && (j < j_ul || ((j - j_lo) & 1) != 0); ++j) general_step(j);
    for (; j + 2 < jm; j += 2) {
      fast_step(sa, sb, j, k_st0, k_st1, v_st0, v_st1);
      fast_step(sb, sa, j + 1, k_st1, k_st0, v_st1, v_st0);
    }
    // the steady state leaves the scores of tile j without their maximum
    if constexpr (NOMAX) {
      if (j < ntiles && active(j)) rebase(sa);
    }
    for (; j < ntiles; ++j) general_step(j);

    // ---- epilogue: O = acc / l, LSE = ln 2 * (M + log2 l)
    float l_lo, l_hi;
    halves(lsum, l_lo, l_hi);
    const float l = l_lo + l_hi;
    // a packed sequence can have rows that see no key (causal, fewer keys than queries, or
    // none): O = 0 and LSE = -inf for them
    const bool empty = VARLEN && !(l > 0.f);
    const float inv = empty ? 0.f : 1.f / l;
    // O goes out row-major through the wave's share of the (now idle) K/V stages: each store
    // instruction writes whole rows (1 KB, contiguous for dense O), instead of 8-byte pieces of
    // 32 different rows. Measured: causal T = 8192 +1.3%, T = 1024 +7%.
    constexpr int WAVE_BYTES = 32 * S::RB;
    constexpr int PER_ARR = S::TILE / WAVE_BYTES;
    const int el = opaque_lane();
    const int ecol = el & 31, ehf = el >> 5;
    if constexpr (PER_ARR >= 1 && NW <= 4 * PER_ARR) {
      if (wave_has_rows) {
        constexpr int C = D / 8;  // 16-byte chunks per row; chunk c of row r sits at c ^ (r % C)
        const int arr = wave / PER_ARR;
        unsigned char* ob = (arr == 0 ? k_st0 : arr == 1 ? k_st1 : arr == 2 ? v_st0 : v_st1) +
                            (wave % PER_ARR) * WAVE_BYTES;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int c = 4 * dt + g4;
            u32x2 packed = {pack2_bf16(acc[dt][4 * g4 + 0] * inv, acc[dt][4 * g4 + 1] * inv),
                            pack2_bf16(acc[dt][4 * g4 + 2] * inv, acc[dt][4 * g4 + 3] * inv)};
            *(LDS_AS u32x2*)(ob + ecol * S::RB + ((c ^ (ecol % C)) << 4) + 8 * ehf) = packed;
          }
        // the wave's own LDS operations run in order: only the compiler must not move the
        // reads up
        __builtin_amdgcn_fence(__ATOMIC_SEQ_CST, "wavefront");
        // row qw0 + r of this head: packed batches keep Hq * D elements between rows
        __bf16* Ow = VARLEN ? O + ((size_t)(cur.q_begin + qw0) * Hq + cur.h) * D
                            : O + (((size_t)cur.b * Hq + cur.h) * (size_t)Tq + qw0) * D;
#pragma unroll
        for (int i = 0; i < C / 2; ++i) {
          const int r = i * (64 / C) + el / C, lc = el % C;
          const u32x4 v = *(LDS_AS u32x4*)(ob + r * S::RB + ((lc ^ (r % C)) << 4));
          if (qw0 + r < Tq) *reinterpret_cast<u32x4*>(Ow + (size_t)r * qstr + 8 * lc) = v;
        }
      }
    } else {
      if (qrow < Tq) {
        __bf16* Orow = VARLEN ? O + ((size_t)(cur.q_begin + qrow) * Hq + cur.h) * D
                              : O + (((size_t)cur.b * Hq + cur.h) * (size_t)Tq + qrow) * D;
#pragma unroll
        for (int dt = 0; dt < D / 32; ++dt)
#pragma unroll
          for (int g4 = 0; g4 < 4; ++g4) {
            const int d0 = 32 * dt + 8 * g4 + 4 * hf;
            u32x2 packed = {pack2_bf16(acc[dt][4 * g4 + 0] * inv, acc[dt][4 * g4 + 1] * inv),
                            pack2_bf16(acc[dt][4 * g4 + 2] * inv, acc[dt][4 * g4 + 3] * inv)};
            *reinterpret_cast<u32x2*>(Orow + d0) = packed;
          }
      }
    }
    if (hf == 0 && qrow < Tq) {
      const float lse = empty ? kNegInf : (M + __builtin_amdgcn_logf(l)) * kLn2;
      if constexpr (VARLEN)
        LSE[(size_t)cur.h * total_q + cur.q_begin + qrow] = lse;
      else
        LSE[((size_t)cur.b * Hq + cur.h) * (size_t)Tq + qrow] = lse;
    }
    if constexpr (!PAIRED) break;
    // paired blocks: once every wave has read its O back out of the stages, the second block's
    // first K and V tiles go in (its Q is already in q_st)
    if (it == 0 && qb2 >= 0) {
      opaque_sizes();
      const Item nxt = make_item(bh, qb2);
      __syncthreads();
      if (nxt.Tk % BC != 0) {
        clear_v();
        __syncthreads();
      }
      issue_prologue(nxt);
    }
  }
}

template <int D, int BC, int NW, bool VARLEN, bool PAIRED>
hipError_t launch_t(const Problem& p, int schedule, const Packed* pk, hipStream_t stream) {
  using S = Shape<D, BC, NW>;
  const int nqb = (p.Tq + S::BR - 1) / S::BR;
  // one workgroup per query block, or per pair of blocks
  const long long grid = (long long)p.B * p.Hq * (PAIRED ? (nqb + 1) / 2 : nqb);
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((prefill_bf16_kernel<D, BC, NW, VARLEN, PAIRED>), dim3((unsigned)grid),
                     dim3(S::NT), 0, stream, static_cast<const __bf16*>(p.Q),
                     static_cast<const __bf16*>(p.K), static_cast<const __bf16*>(p.V),
                     static_cast<__bf16*>(p.O), p.LSE, p.B, p.Hq, p.Hkv, p.Tq, p.Tk, p.causal,
                     p.window, p.log2_scale, p.qsign, schedule, pk ? pk->cu_q : nullptr,
                     pk ? pk->cu_k : nullptr, pk ? pk->total_q : 0, pk ? pk->total_k : 0);
  return hipGetLastError();
}

template <int D, bool VARLEN, bool PAIRED>
hipError_t launch_shape(const Problem& p, int block_kv, int waves, int schedule, const Packed* pk,
                        hipStream_t stream) {
  if (block_kv == 64 && waves == 4) return launch_t<D, 64, 4, VARLEN, PAIRED>(p, schedule, pk, stream);
  if (block_kv == 64 && waves == 8) return launch_t<D, 64, 8, VARLEN, PAIRED>(p, schedule, pk, stream);
  if (block_kv == 32 && waves == 4) return launch_t<D, 32, 4, VARLEN, PAIRED>(p, schedule, pk, stream);
  if (block_kv == 32 && waves == 8) return launch_t<D, 32, 8, VARLEN, PAIRED>(p, schedule, pk, stream);
  return hipErrorInvalidValue;
}

// schedule 4: paired blocks (dense batches)
template <int D>
hipError_t launch_d(const Problem& p, int block_kv, int waves, int schedule, const Packed* pk,
                    hipStream_t stream) {
  if (pk) {
    if (schedule == 4) return hipErrorInvalidValue;
    return launch_shape<D, true, false>(p, block_kv, waves, schedule, pk, stream);
  }
  // paired blocks only with 8-wave workgroups: the second block's Q in LDS leaves 4-wave
  // workgroups one per CU, where two fit otherwise
  if (schedule == 4) {
    if (waves != 8) return hipErrorInvalidValue;
    if (block_kv == 64) return launch_t<D, 64, 8, false, true>(p, schedule, pk, stream);
    if (block_kv == 32) return launch_t<D, 32, 8, false, true>(p, schedule, pk, stream);
    return hipErrorInvalidValue;
  }
  return launch_shape<D, false, false>(p, block_kv, waves, schedule, pk, stream);
}

hipError_t launch_any(const Problem& p, int block_kv, int waves, int schedule, const Packed* pk,
                      hipStream_t stream) {
  switch (p.d) {
    case 32: return launch_d<32>(p, block_kv, waves, schedule, pk, stream);
    case 64: return launch_d<64>(p, block_kv, waves, schedule, pk, stream);
    case 128: return launch_d<128>(p, block_kv, waves, schedule, pk, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace

hipError_t launch_prefill_bf16(const Problem& p, int block_kv, int waves, int schedule,
                               hipStream_t stream) {
  return launch_any(p, block_kv, waves, schedule, nullptr, stream);
}

hipError_t launch_prefill_varlen_bf16(const Problem& p, const Packed& pk, int block_kv,
                                      int waves, int schedule, hipStream_t stream) {
  return launch_any(p, block_kv, waves, schedule, &pk, stream);
}

}  // namespace fattn
