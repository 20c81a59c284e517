// Launch-configuration table of libfattn.
//
// The block size is a performance choice, not a numerical one ("SDPA and FlashAttention's
// tiling", section "A softmax you can compute one block at a time"; "Explain tiled attention and
// verify its output", section "Separate storage savings from runtime": tile size, register
// pressure and cache reuse decide the speed). Every entry computes the same function; the
// parity tests run each one.
//
// Prefill rows are matched in order: the first row whose d matches, whose causal flag matches
// (-1 = either) and whose Tk is at most tk_max (0 = no bound) wins.
#pragma once

namespace fattn {

struct PrefillEntry {
  int d;
  int causal;   // -1 = any
  int tk_max;   // 0 = unbounded
  int block_kv;
  int waves;
  int schedule;
};

// Measured on MI355X with `python -m io_aware_tiled_amd.tune` (C3-like shapes): 64-key tiles beat
// 32-key tiles everywhere; 8 waves (256 query rows) per workgroup win at d = 128 and 4 waves at
// d = 64 for long sequences; the XCD-grouped, longest-first order is 1.3-1.5x faster than
// row-major for causal masks and no slower without one.
static const PrefillEntry kPrefillTable[] = {
    // d, causal, tk_max, block_kv, waves, schedule
    {64, -1, 2048, 64, 8, 2},
    {64, -1, 0, 64, 4, 2},
    {128, -1, 0, 64, 8, 2},
    {32, -1, 0, 64, 4, 2},
};

// Decode: number of workgroups to aim for across the whole grid and the smallest key chunk a
// split may have (keys, multiple of 32).
struct DecodeEntry {
  int d;
  int target_workgroups;
  int min_chunk;
};

static const DecodeEntry kDecodeTable[] = {
    {128, 2048, 256},
    {64, 2048, 256},
    {32, 2048, 256},
};

}  // namespace fattn
