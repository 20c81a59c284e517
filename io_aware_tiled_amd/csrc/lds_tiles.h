// LDS tile machinery shared by the bf16 matrix-core kernels (forward prefill and backward):
// vector types, the swizzled row layout of a K, V (or Q, dO) tile in LDS, its direct-to-LDS
// loads, and two small lane-exchange and packing helpers.
//
// A tile of BC rows of D bf16 elements is stored row by row, each 256-byte-or-smaller row as
// 16-byte chunks permuted by an XOR with a function of the row (`swz`), so that both operand
// reads a kernel makes of it are free of bank conflicts: 16 consecutive rows read at the same
// logical chunk (the A operand of an MFMA taken row-wise, `ds_read_b128`), and the four rows a
// transpose read (`ds_read_b64_tr_b16`) takes at once.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace fattn {
namespace lds {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
#ifndef LDS_AS
#define LDS_AS __attribute__((address_space(3)))
#endif

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kNegInf = -__builtin_inff();
constexpr int kBufferFlags = 0x00020000;  // raw buffer, 32-bit data format

template <int D, int BC, int NW>
struct Shape {
  static constexpr int BR = 32 * NW;               // lane-owned rows per workgroup
  static constexpr int NT = 64 * NW;               // threads per workgroup
  static constexpr int RB = 2 * D;                 // bytes per K or V row
  static constexpr int C = D / 8;                  // 16-byte chunks per row
  static constexpr int R256 = RB >= 256 ? 1 : 256 / RB;  // rows per 256 bytes
  static constexpr int G = C / 4;
  static constexpr int TILE = BC * RB;             // bytes per K or V tile
  static constexpr int NI = TILE / 1024;           // direct-to-LDS loads (1 KB each) per tile
  static constexpr int NI_W = (NI + NW - 1) / NW;  // per wave
  static constexpr int RPI = 1024 / RB;            // rows per direct-to-LDS load
  static constexpr int LDS_BYTES = 4 * TILE;       // K and V, two stages each
  static_assert(D % 32 == 0 && D <= 128 && BC % 32 == 0 && TILE % 1024 == 0, "tile shape");
};

// Chunk swizzle of row r: a bijection on the chunk index so that 16 consecutive rows read at the
// same logical chunk, and the four rows a transpose read takes at once, hit distinct banks.
template <int D, int BC, int NW>
__device__ __forceinline__ int swz(int r) {
  using S = Shape<D, BC, NW>;
  const int u = (r / S::R256) % S::C;
  return 4 * (u % S::G) + (u / S::G) % 4;
}
// Byte offset of row r inside a tile; logical chunk c of that row is at rowbase(r) ^ (c << 4).
template <int D, int BC, int NW>
__device__ __forceinline__ int rowbase(int r) {
  using S = Shape<D, BC, NW>;
  return r * S::RB + (swz<D, BC, NW>(r) << 4);
}

// Buffer resource for rows [row0, T) of a [T, D] bf16 slice: reads past T return zeros.
template <int D>
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rows_rsrc(const __bf16* slice, int row0, int T) {
  const int rows = T - row0;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<__bf16*>(slice + (size_t)row0 * D),
                                           (short)0, rows > 0 ? rows * D * 2 : 0, kBufferFlags);
}

// One K or V tile, global -> LDS by direct-to-LDS loads: this wave's share of the 1 KB loads.
// dvo[i] (i < NI_W) is this lane's LDS byte offset within the tile for the wave's i-th load.
// (A device function rather than a lambda: the builtin exists only in the device pass.)
template <int D, int BC, int NW>
__device__ __forceinline__ void dma_tile(const __bf16* head, int j0, int Tk, unsigned char* dst,
                                         int wave, const int* dvo) {
  using S = Shape<D, BC, NW>;
  const __amdgpu_buffer_rsrc_t rs = rows_rsrc<D>(head, j0, Tk);
#pragma unroll
  for (int i = 0; i < S::NI_W; ++i) {
    const int q = wave + i * NW;
    if (S::NI % NW == 0 || q < S::NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + q * 1024), 16, dvo[i], 0,
                                               0, 0);
  }
}

// One tile of rows j0 .. j0+BC-1 of a slice whose consecutive rows are row_elems elements apart
// (row_elems >= D: packed [total, H, D] tensors), global -> LDS like dma_tile. dvo[i] must have
// been computed with row stride row_elems * 2 bytes. Rows at or past T read as zeros.
template <int D, int BC, int NW>
__device__ __forceinline__ void dma_tile_strided(const __bf16* head, int j0, int T, int row_elems,
                                                 unsigned char* dst, int wave, const int* dvo) {
  using S = Shape<D, BC, NW>;
  const int rows = min(T - j0, BC);
  const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<__bf16*>(head + (size_t)j0 * row_elems), (short)0,
      rows > 0 ? ((rows - 1) * row_elems + D) * 2 : 0, kBufferFlags);
#pragma unroll
  for (int i = 0; i < S::NI_W; ++i) {
    const int q = wave + i * NW;
    if (S::NI % NW == 0 || q < S::NI)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + q * 1024), 16, dvo[i], 0,
                                               0, 0);
  }
}

// Values of lane l and lane l ^ 32 (the same query row in the other half-wave), via
// v_permlane32_swap on two copies of x. Written as inline asm because the compiler folds the
// two results of the builtin into one when both inputs are the same value.
__device__ __forceinline__ void halves(float x, float& lo_half, float& hi_half) {
  uint32_t a = __builtin_bit_cast(uint32_t, x), b = a;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1" : "+v"(a), "+v"(b));
  lo_half = __builtin_bit_cast(float, a);  // lanes 0-31: own; lanes 32-63: lane - 32
  hi_half = __builtin_bit_cast(float, b);  // lanes 0-31: lane + 32; lanes 32-63: own
}

// Two floats rounded to bf16 (nearest-even) and packed low/high.
__device__ __forceinline__ uint32_t pack2_bf16(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, (__bf16)lo) |
         ((uint32_t)__builtin_bit_cast(uint16_t, (__bf16)hi) << 16);
}

}  // namespace lds
}  // namespace fattn
