/*
 * libfattn: fused attention for AMD Instinct MI355X (gfx950): the forward pass (attn_fwd,
 * attn_fwd_window, attn_fwd_varlen, attn_fwd_paged) and its backward (attn_bwd).
 *
 * Computes, for every batch b, query head h and query row i,
 *   O[b,h,i,:] = softmax_j(scale * Q[b,h,i,:] . K[b,g,j,:] + mask(i,j)) V[b,g,j,:]
 *   LSE[b,h,i] = log sum_j exp(scale * Q[b,h,i,:] . K[b,g,j,:] + mask(i,j))
 * with g = h / (Hq / Hkv), one query tile at a time: key/value tiles stream through on-chip
 * memory while a running row maximum, a running sum and an unnormalised accumulator are kept and
 * rescaled whenever the maximum grows; the Tq x Tk score matrix never reaches device memory.
 *
 * Sources of the definition: the online-softmax update and tiled forward of
 * "4.2 FlashAttention I: IO-Awareness & The Online Softmax" (sections "The key idea: a running
 * max and a correction factor" and "FlashAttention forward: tiling + online softmax fused into
 * one pass"), the blockwise forward returning (out, lse) of "Efficient attention & KV cache"
 * (section 3), and the argument set of the fused attention call on "SDPA and FlashAttention's
 * tiling" (section "The tiled sketch, in Python": is_causal, scale, enable_gqa).
 *
 * Plain C ABI: no HIP or torch types appear here. All entry points are thread-safe.
 */
#ifndef FATTN_H
#define FATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

/* The library is built with hidden symbol visibility; exactly the calls declared here are
   exported. */
#pragma GCC visibility push(default)

/* Return codes. */
#define FATTN_OK 0
#define FATTN_ERR_INVALID (-1)     /* an argument is out of its documented range */
#define FATTN_ERR_UNSUPPORTED (-2) /* valid but not implemented (head dim not 32, 64 or 128) */
#define FATTN_ERR_HIP (-3)         /* the HIP runtime reported an error at launch */
#define FATTN_ERR_NOMEM (-4)       /* a workspace could not be allocated */

/* Element types of Q, K, V and O. LSE is always float32. */
#define FATTN_F32 0
#define FATTN_BF16 1

/* Kernel families a configuration can name. */
#define FATTN_KERNEL_AUTO 0
#define FATTN_KERNEL_PREFILL_MFMA 1 /* bf16 matrix-core prefill */
#define FATTN_KERNEL_PREFILL_F32 2  /* fp32 vector-ALU path (any Tq) */
#define FATTN_KERNEL_DECODE_SPLITK 3 /* bf16 split-K decode + LSE combine (Tq == 1) */

/* Launch configuration. A zero field means "use the tuned table's value". */
typedef struct fattn_cfg {
  int kernel;   /* FATTN_KERNEL_* */
  int block_q;  /* query rows per workgroup (prefill: 32 * waves) */
  int block_kv; /* keys per tile (prefill MFMA: 32 or 64; decode: 32) */
  int waves;    /* wavefronts (64 lanes) per workgroup */
  int splits;   /* decode: key-range splits per (batch, kv head) */
  int schedule; /* prefill grid order: 1 = row-major, 2 = XCD-grouped, longest causal first,
                   4 = one workgroup per pair of query blocks of a (batch, head), the longer
                   causal block first (dense batches, 8 waves only) */
} fattn_cfg_t;

/*
 * attn_fwd: enqueue one forward pass on `stream` and return without waiting.
 *
 *   Q    [B, Hq,  Tq, d] contiguous, element type `dtype`
 *   K, V [B, Hkv, Tk, d] contiguous, element type `dtype`
 *   O    [B, Hq,  Tq, d] contiguous, element type `dtype` (written)
 *   LSE  [B, Hq,  Tq]    contiguous float32, natural-log log-sum-exp of the scaled, masked
 *                        scores of each row (written)
 *
 * All five pointers are device pointers on the current HIP device, owned by the caller, and must
 * be 16-byte aligned. `scale` multiplies the dot products as given (callers usually pass
 * 1/sqrt(d)); it must be finite. `causal` = 1 masks key j for query row i when
 * j > i + (Tk - Tq): causal masks align at the bottom-right, so a single query row (Tq == 1)
 * sees every key, the decode case. Hq must be a multiple of Hkv (grouped-query attention:
 * query head h reads kv head h / (Hq / Hkv)). Tq == 1 with dtype bf16 runs the split-K decode
 * kernels; any other shape runs the prefill kernels. `stream` is a hipStream_t (NULL = the
 * default stream). O and LSE are valid once the stream reaches this point.
 *
 * Errors, all detected on the host before any HIP call:
 *   FATTN_ERR_INVALID     a NULL pointer; B, Hq, Hkv, Tq, Tk or d negative; Tk == 0 with work
 *                         to do; Hkv == 0 or Hq % Hkv != 0; causal not 0 or 1; causal with
 *                         Tq > Tk (a row would see no key); a non-finite scale; an unknown
 *                         dtype; a pointer not 16-byte aligned; Tq*d or Tk*d above 2^31 - 1.
 *   FATTN_ERR_UNSUPPORTED d not in {32, 64, 128}.
 * B == 0 or Tq == 0 (or Hq == 0) is a no-op that returns FATTN_OK.
 * A launch failure returns FATTN_ERR_HIP; device faults surface at the caller's next
 * synchronisation. The decode path allocates a grow-only workspace per (device, stream) on first
 * use (FATTN_ERR_NOMEM if that fails); fattn_release() frees it.
 */
int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
             int Hkv, int Tq, int Tk, int d, int causal, float scale, int dtype, void* stream);

/*
 * attn_fwd_cfg: attn_fwd with an explicit launch configuration (NULL = the tuned table).
 * Non-zero fields override the table; a combination the kernels do not implement returns
 * FATTN_ERR_UNSUPPORTED (for example block_kv not in {32, 64}, waves not in {4, 8}, or a decode
 * kernel for a shape with Tq != 1). Used by the autotune sweep and the parity tests.
 */
int attn_fwd_cfg(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
                 int Hkv, int Tq, int Tk, int d, int causal, float scale, int dtype, void* stream,
                 const fattn_cfg_t* cfg);

/*
 * attn_fwd_noalloc: attn_fwd for callers that cannot allocate device memory: code under HIP
 * graph capture, tight serving loops, harnesses that forbid allocation. Same arguments, layouts,
 * results and error codes as attn_fwd, and it calls no hipMalloc, hipFree or other allocating
 * routine. The split-K decode (Tq == 1, bf16) keeps its per-split partial outputs in a static
 * device array of 16 MiB (4 * 2^20 floats) that each GPU holds from library load until the
 * process ends, instead of attn_fwd's grow-only workspace; the split count is lowered where
 * needed so that splits * B * Hq * (d + 1) floats fit, and a shape with B * Hq * (d + 1) above
 * 4 * 2^20 is rejected with FATTN_ERR_INVALID before any HIP call. Every call on one GPU shares
 * that array, so calls that overlap on one GPU (different streams or threads) race: serialise
 * them. The prefill paths use no scratch memory and run as in attn_fwd.
 */
int attn_fwd_noalloc(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                     int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale, int dtype,
                     void* stream);

/*
 * attn_fwd_plan: host-only query of the configuration attn_fwd would launch for this shape
 * (after validation, with `cfg` overrides applied when non-NULL); writes it to *out.
 * Same return codes as attn_fwd; makes no HIP call.
 */
int attn_fwd_plan(int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int dtype,
                  const fattn_cfg_t* cfg, fattn_cfg_t* out);

/*
 * attn_fwd_window: sliding-window causal attention ("4.2 FlashAttention I: IO-Awareness & The
 * Online Softmax", Exercises, exercise 4: a query sees only keys inside a causal window of width
 * W; "Efficient attention & KV cache", section 7, exercises 1 and 2: the rolling window and the
 * key loop that starts at the window's left edge). With the bottom-right alignment of attn_fwd,
 * query row i sits at position p = i + Tk - Tq and sees keys j with p - window < j <= p; key
 * blocks wholly outside every row's window of a query block are never read.
 *
 * Arguments, layouts, ownership, stream semantics and error codes are those of attn_fwd with
 * causal = 1, plus `window` (keys per row, >= 1; FATTN_ERR_INVALID otherwise). A window of Tk or
 * more hides nothing beyond the causal mask and gives exactly the result of attn_fwd with
 * causal = 1. With Tq == 1 and bf16 the split-K decode path reads only the last `window` keys.
 * A prefill under a window takes the launch table's configuration for a key length of `window`
 * (the most keys a row sees), with schedule 2 in place of schedule 4.
 */
int attn_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                    int Hq, int Hkv, int Tq, int Tk, int d, int window, float scale, int dtype,
                    void* stream);

/* attn_fwd_window with an explicit launch configuration, as attn_fwd_cfg is to attn_fwd. */
int attn_fwd_window_cfg(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                        int Hq, int Hkv, int Tq, int Tk, int d, int window, float scale,
                        int dtype, void* stream, const fattn_cfg_t* cfg);

/*
 * attn_fwd_varlen: causal or full attention over a packed batch of sequences of different
 * lengths, concatenated without padding and described by cumulative lengths, so that no score
 * between two sequences is ever formed ("4.2 FlashAttention I: IO-Awareness & The Online
 * Softmax", section "Practical use: you almost never write this yourself": the packed call with
 * cumulative sequence offsets; "Efficient attention & KV cache", section 4, document masks
 * through the variable-length interface for training).
 *
 *   Q, O          [total_q, Hq, d]  bf16 (O written)
 *   K, V          [total_k, Hkv, d] bf16
 *   LSE           [Hq, total_q]     float32 (written)
 *   cu_seqlens_q  [num_seqs + 1]    int32 device array: sequence b owns query rows
 *                                   cu_seqlens_q[b] .. cu_seqlens_q[b+1] - 1
 *   cu_seqlens_k  [num_seqs + 1]    int32, the same for key/value rows
 *
 * Within sequence b everything is attn_fwd (or attn_fwd_window when window > 0) on its slices,
 * with bottom-right causal alignment when its query and key lengths differ. max_seqlen_q and
 * max_seqlen_k must be at least every sequence's lengths (rows past max_seqlen_q are not
 * computed). Device-side contents are the caller's contract: offsets are clamped to
 * [0, total]; a row that sees no key (a causal sequence with fewer keys than queries, or no
 * keys) gets O = 0 and LSE = -inf. Pointers are caller-owned device pointers, tensors 16-byte
 * aligned, cu arrays 4-byte aligned.
 *
 * Errors (host-side): FATTN_ERR_INVALID for NULL or misaligned pointers, negative sizes, Hq not a
 * multiple of Hkv, causal not 0/1, a window without causal, a non-finite scale;
 * FATTN_ERR_UNSUPPORTED for d not in {32, 64, 128} or dtype FATTN_F32. num_seqs == 0,
 * Hq == 0 or total_q == 0 is a no-op.
 */
int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                    const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs, int total_q,
                    int total_k, int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d,
                    int causal, int window, float scale, int dtype, void* stream);

/*
 * attn_fwd_paged: one decode step (one query token per sequence) over a paged KV cache
 * ("Efficient attention & KV cache", section 2.5 and the interview question on what
 * PagedAttention changes in the attention kernel: keys and values live in fixed-size blocks
 * located through a per-sequence block table, and the kernel gathers each block from its
 * physical location instead of reading one contiguous slice).
 *
 *   Q            [B, Hq, d]                          bf16
 *   K_cache,
 *   V_cache      [num_blocks, Hkv, block_size, d]    bf16; physical block n holds, for every kv
 *                                                    head, block_size consecutive positions
 *   block_table  [B, max_blocks_per_seq]             int32; entry (b, i) is the physical block
 *                                                    holding positions i*block_size ..
 *                                                    (i+1)*block_size - 1 of sequence b
 *   seq_lens     [B]                                 int32; cached positions of sequence b
 *   O            [B, Hq, d] bf16 and LSE [B, Hq] float32 (written)
 *
 * Sequence b attends, without a mask, to its positions 0 .. seq_lens[b] - 1 (the decode case of
 * attn_fwd with Tq = 1): O and LSE equal attn_fwd on the gathered contiguous cache. GQA as in
 * attn_fwd. All pointers are caller-owned device pointers on the current device; the tensors
 * must be 16-byte aligned, block_table and seq_lens 4-byte aligned.
 *
 * Errors (host-side, before any HIP call): FATTN_ERR_INVALID for a NULL pointer, a misaligned
 * pointer, block_size not a power of two in [16, 4096], num_blocks or max_blocks_per_seq < 1,
 * max_blocks_per_seq * block_size above 2^31 - 1, and the shape errors of attn_fwd;
 * FATTN_ERR_UNSUPPORTED for d not in {32, 64, 128} or dtype FATTN_F32. B == 0 or Hq == 0 is a
 * no-op. The device-side contents are the caller's contract: seq_lens[b] is clamped to
 * [0, max_blocks_per_seq * block_size]; a sequence of length 0 gets O = 0 and LSE = -inf; a
 * table entry outside [0, num_blocks) is never dereferenced (its positions read as zero keys and
 * values). Shares the split-K decode kernels and workspace of attn_fwd; the split plan covers
 * max_blocks_per_seq * block_size keys.
 */
int attn_fwd_paged(const void* Q, const void* K_cache, const void* V_cache,
                   const int* block_table, const int* seq_lens, void* O, float* LSE, int B,
                   int Hq, int Hkv, int d, int num_blocks, int block_size, int max_blocks_per_seq,
                   float scale, int dtype, void* stream);

/*
 * attn_bwd: enqueue the backward pass of attn_fwd (or attn_fwd_window) on `stream`: the
 * gradients of a scalar loss with respect to Q, K and V, given its gradient dO with respect to
 * O. The probabilities are recomputed tile by tile from Q, K and the saved LSE instead of being
 * stored ("4.2 FlashAttention I: IO-Awareness & The Online Softmax", section "The backward pass:
 * recomputation instead of storage"; "Efficient attention & KV cache", section 2.2):
 *   P = exp(scale * Q K^T + mask - LSE),  D_i = sum_c dO[i,c] O[i,c],
 *   dV = P^T dO,  dS = P o (dO V^T - D),  dQ = scale * dS K,  dK = scale * dS^T Q,
 * with the gradients of kv head g summed over the query heads h / (Hq / Hkv) == g that read it.
 *
 *   Q, dO, O, dQ  [B, Hq,  Tq, d] contiguous bf16 (dQ written)
 *   K, V, dK, dV  [B, Hkv, Tk, d] contiguous bf16 (dK, dV written)
 *   LSE           [B, Hq,  Tq]    contiguous float32, as written by the forward call
 * O and LSE must be the forward outputs for the same Q, K, V, causal, window and scale. `window`
 * is 0 for none, else the sliding-window width of attn_fwd_window (causal must then be 1).
 * All pointers are caller-owned device pointers on the current device, 16-byte aligned. dQ, dK
 * and dV must not overlap the inputs. The result is bitwise reproducible: no atomics, fixed
 * summation order.
 *
 * Errors: those of attn_fwd, plus FATTN_ERR_INVALID for a negative window or a window without
 * causal; dtype FATTN_F32 returns FATTN_ERR_UNSUPPORTED. B == 0, Hq == 0 or Tq == 0 is a no-op.
 * The call uses a grow-only workspace per (device, stream) of B * Hq * ceil(Tq / 32) * 256 bytes
 * (FATTN_ERR_NOMEM if it cannot be allocated), shared with the decode path and freed by
 * fattn_release().
 */
int attn_bwd(const void* Q, const void* K, const void* V, const void* O, const void* dO,
             const float* LSE, void* dQ, void* dK, void* dV, int B, int Hq, int Hkv, int Tq,
             int Tk, int d, int causal, int window, float scale, int dtype, void* stream);

/*
 * attn_bwd_varlen: attn_bwd over a packed batch, the backward of attn_fwd_varlen: each sequence's
 * gradients are those of attn_bwd on its slices (no gradient flows between sequences).
 *
 *   Q, O, dO, dQ  [total_q, Hq, d]  bf16 (dQ written)
 *   K, V, dK, dV  [total_k, Hkv, d] bf16 (dK, dV written)
 *   LSE           [Hq, total_q]     float32, as written by attn_fwd_varlen
 *   cu_seqlens_q, cu_seqlens_k, num_seqs, total_q, total_k, max_seqlen_q, max_seqlen_k, causal,
 *   window: as for attn_fwd_varlen.
 *
 * Rows that see no key contribute nothing and get dQ = 0; keys no row sees get dK = dV = 0.
 * Errors: those of attn_fwd_varlen and attn_bwd, plus FATTN_ERR_INVALID when Hq * total_q
 * exceeds 2^28 - 1. Uses the per-(device, stream) workspace (2 * Hq * total_q floats).
 */
int attn_bwd_varlen(const void* Q, const void* K, const void* V, const void* O, const void* dO,
                    const float* LSE, void* dQ, void* dK, void* dV, const int* cu_seqlens_q,
                    const int* cu_seqlens_k, int num_seqs, int total_q, int total_k,
                    int max_seqlen_q, int max_seqlen_k, int Hq, int Hkv, int d, int causal,
                    int window, float scale, int dtype, void* stream);

/* Text for a return code (static storage). */
const char* fattn_strerror(int code);

/*
 * Text describing the most recent failure of a call on the calling thread: which check failed or
 * which HIP call returned which error. Empty after a successful call. Thread-local storage, valid
 * until the thread's next call into the library.
 */
const char* fattn_last_error(void);

/* Library version as major * 10000 + minor * 100 + patch. */
int fattn_version(void);

/*
 * Free the workspaces (split-K decode, backward) of every device after synchronising each device.
 * Safe to call at any time when no call of this library is in flight; later calls allocate again.
 */
int fattn_release(void);

#pragma GCC visibility pop

#ifdef __cplusplus
}
#endif

#endif /* FATTN_H */
