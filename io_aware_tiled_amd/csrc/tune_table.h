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

// Measured on MI355X with `python -m io_aware_tiled_amd.tune` (TFLOP/s of the best entry against
// the next best in parentheses where it matters):
//  * d = 128, causal: 4 waves (128 query rows per workgroup) up to Tk = 4096 (T = 1024: 572 vs
//    456 with 8 waves; 4096: 836 vs 712), 8 waves beyond (8192: 1072 vs 1019).
//  * d = 128, no mask: 4 waves up to Tk = 1024 (880 vs 830), 8 waves beyond.
//  * d = 64, causal: 4 waves with 64-key tiles (T = 8192: 852 vs 757 with 8 waves).
//  * d = 64, no mask: 32-key tiles with 4 waves up to Tk = 1024, with 8 waves beyond
//    (T = 8192: 995 vs 968).
// 64-key tiles win everywhere else; the XCD-grouped, longest-first order is 1.3-1.5x faster
// than row-major for causal masks and no slower without one.
static const PrefillEntry kPrefillTable[] = {
    // d, causal, tk_max, block_kv, waves, schedule
    {128, 1, 4096, 64, 4, 2},
    {128, 1, 0, 64, 8, 2},
    {128, 0, 1024, 64, 4, 2},
    {128, 0, 0, 64, 8, 2},
    {64, 1, 0, 64, 4, 2},
    {64, 0, 1024, 32, 4, 2},
    {64, 0, 0, 32, 8, 2},
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
