// Launch-configuration table of libfattn.
//
// The block size is a performance choice, not a numerical one ("SDPA and FlashAttention's
// tiling", section "A softmax you can compute one block at a time"; "Explain tiled attention and
// verify its output", section "Separate storage savings from runtime": tile size, register
// pressure and cache reuse decide the speed). Every entry computes the same function; the
// parity tests run each one.
//
// Prefill rows are matched in order: the first row whose d matches, whose causal flag matches
// (-1 = either), whose Tk is at most tk_max (0 = no bound) and whose batch x query heads is at
// least min_bh wins.
#pragma once

namespace fattn {

struct PrefillEntry {
  int d;
  int causal;   // -1 = any
  int tk_max;   // 0 = unbounded
  int min_bh;   // B * Hq at least this (0 = any)
  int block_kv;
  int waves;
  int schedule;
};

// Measured on MI355X with `python -m io_aware_tiled_amd.tune` and the head-group grid order
// (TFLOP/s of the chosen entry against the next best in parentheses where it matters):
//  * d = 128, causal: 4 waves (128 query rows per workgroup) up to Tk = 2048 (B = 1, T = 2048:
//    633 vs 541 with 8 waves; B = 16, T = 1024: 635 vs 604), 8 waves beyond (B = 1, T = 4096:
//    966 vs 913; T = 8192: 1108 vs 1074).
//  * d = 128, no mask: 4 waves up to Tk = 1024 (887 vs 860), 8 waves beyond.
//  * d = 64, causal: up to Tk = 1024, 32-key tiles with 4 waves for at least 256 (batch, head)
//    pairs (B = 16, H = 32: 637 vs 606 with 64-key tiles), 64-key tiles with 4 waves for fewer
//    (B = 4, H = 16: 326 vs 316); 32-key tiles with 4 waves beyond (T = 2048 to 16384 with 32
//    heads: 2-3% faster, e.g. T = 8192: 946 vs 932).
//  * d = 64, no mask: 32-key tiles with 4 waves up to Tk = 1024, with 8 waves beyond
//    (T = 2048: 932 vs 908; T = 8192: 1008 vs 975).
// 64-key tiles win everywhere else; the XCD-grouped, longest-first order is 1.3-1.5x faster
// than row-major for causal masks and no slower without one.
static const PrefillEntry kPrefillTable[] = {
    // d, causal, tk_max, min_bh, block_kv, waves, schedule
    {128, 1, 2048, 0, 64, 4, 2},
    {128, 1, 0, 0, 64, 8, 2},
    {128, 0, 1024, 0, 64, 4, 2},
    {128, 0, 0, 0, 64, 8, 2},
    {64, 1, 1024, 256, 32, 4, 2},
    {64, 1, 1024, 0, 64, 4, 2},
    {64, 1, 0, 0, 32, 4, 2},
    {64, 0, 1024, 0, 32, 4, 2},
    {64, 0, 0, 0, 32, 8, 2},
    {32, -1, 0, 0, 64, 4, 2},
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
