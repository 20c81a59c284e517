// Internal launch interface between the host library (api.cpp) and the HIP kernels.
// Every launcher enqueues on `stream`, returns the launch status and performs no allocation.
#pragma once

#include <hip/hip_runtime.h>

namespace fattn {

// Host-side view of one forward problem. Pointers are device pointers; element type is implied
// by the launcher. `log2_scale` is |scale| * log2(e) (1 when scale == 0) and `qsign` is the
// sign of scale (-1, 0 or +1): the kernels multiply Q by qsign as they load it, which is exact,
// so every kernel works with a positive scale.
struct Problem {
  const void* Q;
  const void* K;
  const void* V;
  void* O;
  float* LSE;
  int B, Hq, Hkv, Tq, Tk, d;
  int causal;
  int window;        // sliding window width (causal only): row at p sees keys p-window < j <= p;
                     // 0 = no window
  float abs_scale;   // |scale|, or 1 when scale == 0
  float log2_scale;  // abs_scale * log2(e)
  int qsign;
};

// bf16 matrix-core prefill. block_kv in {32, 64}, waves in {4, 8}, d in {32, 64, 128};
// schedule 1 = row-major grid, 2 = whole heads per XCD, 8 heads at a time query-block-major with
// the longest causal blocks first (grid_order.h), 4 = one workgroup per pair of blocks of a
// (batch, head), block nqb-1-p then block p, pairs dealt to the XCDs in contiguous ranges.
hipError_t launch_prefill_bf16(const Problem& p, int block_kv, int waves, int schedule,
                               hipStream_t stream);

// A packed variable-length batch: sequence b owns rows cu_q[b] .. cu_q[b+1]-1 of the
// [total_q, Hq, d] query tensor and rows cu_k[b] .. cu_k[b+1]-1 of the [total_k, Hkv, d] key and
// value tensors (device int32 arrays of B + 1 entries).
struct Packed {
  const int* cu_q;
  const int* cu_k;
  int total_q, total_k;
};

// bf16 matrix-core prefill over a packed batch: p.B is the number of sequences, p.Tq and p.Tk
// the longest lengths (the grid covers p.Tq rows per sequence; longer sequences are cut there),
// LSE is [Hq, total_q]. block_kv, waves as for launch_prefill_bf16; schedule 3 deals the
// (sequence, head) pairs to the XCDs by head, so every XCD gets a share of every sequence
// (grid_order.h).
hipError_t launch_prefill_varlen_bf16(const Problem& p, const Packed& pk, int block_kv,
                                      int waves, int schedule, hipStream_t stream);

// fp32 vector-ALU path, any Tq (also Tq == 1), d in {32, 64, 128}.
hipError_t launch_prefill_f32(const Problem& p, hipStream_t stream);

// bf16 split-K decode (Tq == 1): partial kernel + combine kernel on the same stream.
// ws_o holds splits * B * Hq * d floats, ws_lse splits * B * Hq floats.
// The keys [k0, Tk) are split into chunks of `chunk` keys (a multiple of 32);
// splits = ceil((Tk - k0) / chunk). k0 > 0 under a sliding window.
hipError_t launch_decode_bf16(const Problem& p, int k0, int splits, int chunk, float* ws_o,
                              float* ws_lse, hipStream_t stream);

// A paged KV cache: K and V are [num_blocks, Hkv, block_size, d]; table is [B, max_blocks]
// physical block ids (int32), seq_lens [B] keys per sequence (int32); all device pointers.
struct PagedKV {
  const int* table;
  const int* seq_lens;
  int num_blocks;
  int max_blocks;
  int bs_shift;  // log2(block_size), block_size >= 16
};

// bf16 split-K decode over a paged cache: as launch_decode_bf16 with the keys of batch b read
// through its block-table row; p.K and p.V are the cache bases, p.Tk is unused. The split plan
// covers max_blocks * block_size keys; splits past a sequence's length write empty partials.
hipError_t launch_decode_paged_bf16(const Problem& p, const PagedKV& pk, int splits, int chunk,
                                    float* ws_o, float* ws_lse, hipStream_t stream);

// Host-side view of one backward problem (bf16 tensors, fp32 LSE). Layouts as the forward:
// Q, O, dO, dQ [B, Hq, Tq, d]; K, V, dK, dV [B, Hkv, Tk, d]; LSE [B, Hq, Tq].
struct BwdProblem {
  const void* Q;
  const void* K;
  const void* V;
  const void* O;
  const void* dO;
  const float* LSE;
  void* dQ;
  void* dK;
  void* dV;
  int B, Hq, Hkv, Tq, Tk, d;
  int causal;
  int window;   // as in Problem
  float scale;  // signed softmax scale
};

// Static scratch of the entry point that allocates nothing: kScratchFloats floats per device,
// a file-scope device array (noalloc.hip). static_scratch returns its device address on device
// `dev`, which must be current; the first call per device looks it up, later calls return it.
constexpr size_t kScratchFloats = size_t(4) << 20;  // 16 MiB
hipError_t static_scratch(int dev, float** out);

// Floats of backward workspace: (L, D) in 32-row blocks for every (batch, query head).
inline size_t backward_workspace_floats(int B, int Hq, int Tq) {
  return (size_t)B * Hq * (size_t)((Tq + 31) / 32) * 64;
}

// bf16 backward: the (L, D) kernel, then the dQ and the dK/dV kernels, on `stream`.
// ws holds backward_workspace_floats(B, Hq, Tq) floats. d in {32, 64, 128}.
hipError_t launch_backward_bf16(const BwdProblem& p, float* ws, hipStream_t stream);

// The same over a packed batch: p.B is the number of sequences, p.Tq and p.Tk the longest
// lengths; Q, O, dO, dQ are [total_q, Hq, d], K, V, dK, dV [total_k, Hkv, d], LSE [Hq, total_q];
// ws holds 2 * Hq * total_q floats.
hipError_t launch_backward_varlen_bf16(const BwdProblem& p, const Packed& pk, float* ws,
                                       hipStream_t stream);

}  // namespace fattn
