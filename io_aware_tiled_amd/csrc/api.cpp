// Host side of libfattn: argument validation, launch planning, the workspaces and the
// exported C entry points. Validation and planning make no HIP call, so every argument error is
// reported identically on a machine without a GPU.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <map>
#include <mutex>
#include <utility>

#include "fattn.h"
#include "kernels.h"
#include "tune_table.h"

namespace fattn {
namespace {

constexpr int kVersion = 1 * 10000 + 0 * 100 + 0;
constexpr float kLog2e = 1.44269504088896340736f;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

thread_local char g_last_error[256] = "";

// Records why a call failed (per thread) and returns `code`.
int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_last_error, sizeof g_last_error, fmt, ap);
  va_end(ap);
  return code;
}

int hip_fail(int code, const char* what, hipError_t e) {
  return fail(code, "%s: %s (%d)", what, hipGetErrorString(e), (int)e);
}

// Shape checks shared by attn_fwd_cfg and attn_fwd_plan. Sets *noop when there is no work.
int validate_shape(int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int dtype,
                   bool* noop) {
  *noop = false;
  if (B < 0 || Hq < 0 || Hkv < 0 || Tq < 0 || Tk < 0 || d < 0)
    return fail(FATTN_ERR_INVALID, "negative dimension");
  if (causal != 0 && causal != 1) return fail(FATTN_ERR_INVALID, "causal must be 0 or 1");
  if (dtype != FATTN_F32 && dtype != FATTN_BF16) return fail(FATTN_ERR_INVALID, "unknown dtype");
  if (B == 0 || Hq == 0 || Tq == 0) {
    *noop = true;
    return FATTN_OK;
  }
  if (Hkv == 0 || Hq % Hkv != 0) return fail(FATTN_ERR_INVALID, "Hq must be a multiple of Hkv");
  if (Tk == 0) return fail(FATTN_ERR_INVALID, "Tk == 0: softmax over no keys");
  if (d == 0) return fail(FATTN_ERR_INVALID, "d == 0");
  if (causal && Tq > Tk) return fail(FATTN_ERR_INVALID, "causal with Tq > Tk");
  if (d != 32 && d != 64 && d != 128) return fail(FATTN_ERR_UNSUPPORTED, "head dim %d", d);
  if ((long long)Tq * d > 0x7fffffffLL || (long long)Tk * d > 0x7fffffffLL)
    return fail(FATTN_ERR_INVALID, "T*d exceeds 2^31-1");
  return FATTN_OK;
}

// The configuration to launch: table defaults, then non-zero overrides from `cfg`.
int make_plan(int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int dtype,
              const fattn_cfg_t* cfg, fattn_cfg_t* out) {
  fattn_cfg_t p = {};
  const bool decode_shape = (Tq == 1 && dtype == FATTN_BF16);
  int kernel = (cfg && cfg->kernel) ? cfg->kernel : FATTN_KERNEL_AUTO;
  if (kernel == FATTN_KERNEL_AUTO) {
    kernel = dtype == FATTN_F32 ? FATTN_KERNEL_PREFILL_F32
                                : (decode_shape ? FATTN_KERNEL_DECODE_SPLITK
                                                : FATTN_KERNEL_PREFILL_MFMA);
  }
  p.kernel = kernel;
  switch (kernel) {
    case FATTN_KERNEL_PREFILL_F32:
      if (dtype != FATTN_F32) return FATTN_ERR_UNSUPPORTED;
      p.block_q = 64;
      p.block_kv = 32;
      p.waves = 1;
      p.splits = 1;
      p.schedule = 1;
      if (cfg && ((cfg->block_q && cfg->block_q != 64) || (cfg->block_kv && cfg->block_kv != 32) ||
                  (cfg->waves && cfg->waves != 1) || (cfg->splits && cfg->splits != 1)))
        return FATTN_ERR_UNSUPPORTED;
      break;
    case FATTN_KERNEL_PREFILL_MFMA: {
      if (dtype != FATTN_BF16) return FATTN_ERR_UNSUPPORTED;
      const PrefillEntry* e = nullptr;
      for (const PrefillEntry& r : kPrefillTable) {
        if (r.d == d && (r.causal < 0 || r.causal == causal) && (r.tk_max == 0 || Tk <= r.tk_max) &&
            (long long)B * Hq >= r.min_bh) {
          e = &r;
          break;
        }
      }
      if (!e) return FATTN_ERR_UNSUPPORTED;
      p.block_kv = e->block_kv;
      p.waves = e->waves;
      p.schedule = e->schedule;
      p.splits = 1;
      if (cfg) {
        if (cfg->block_kv) p.block_kv = cfg->block_kv;
        if (cfg->waves) p.waves = cfg->waves;
        if (cfg->schedule) p.schedule = cfg->schedule;
        if (cfg->splits && cfg->splits != 1) return FATTN_ERR_UNSUPPORTED;
      }
      if (p.block_kv != 32 && p.block_kv != 64) return FATTN_ERR_UNSUPPORTED;
      if (p.waves != 4 && p.waves != 8) return FATTN_ERR_UNSUPPORTED;
      if (p.schedule != 1 && p.schedule != 2 && p.schedule != 4) return FATTN_ERR_UNSUPPORTED;
      if (p.schedule == 4 && p.waves != 8) return FATTN_ERR_UNSUPPORTED;
      p.block_q = 32 * p.waves;
      if (cfg && cfg->block_q && cfg->block_q != p.block_q) return FATTN_ERR_UNSUPPORTED;
      break;
    }
    case FATTN_KERNEL_DECODE_SPLITK: {
      if (dtype != FATTN_BF16 || Tq != 1) return FATTN_ERR_UNSUPPORTED;
      const DecodeEntry* e = nullptr;
      for (const DecodeEntry& r : kDecodeTable)
        if (r.d == d) e = &r;
      if (!e) return FATTN_ERR_UNSUPPORTED;
      const int G = Hq / Hkv;
      const long long units = (long long)B * Hkv * ((G + 15) / 16);
      const int max_splits = (Tk + 31) / 32;
      int splits;
      if (cfg && cfg->splits) {
        splits = cfg->splits;
        if (splits < 1) return FATTN_ERR_UNSUPPORTED;
      } else {
        long long want = (e->target_workgroups + units - 1) / units;
        const int by_chunk = (Tk + e->min_chunk - 1) / e->min_chunk;
        if (want > by_chunk) want = by_chunk;
        if (want < 1) want = 1;
        splits = (int)want;
      }
      if (splits > max_splits) splits = max_splits;
      // keys per split, rounded up to the 32-key block; drop splits that would be empty
      int chunk = ((Tk + splits - 1) / splits + 31) / 32 * 32;
      splits = (Tk + chunk - 1) / chunk;
      p.splits = splits;
      p.block_kv = 32;
      p.block_q = 16;
      p.waves = 1;
      p.schedule = 1;
      if (cfg && ((cfg->block_kv && cfg->block_kv != 32) || (cfg->waves && cfg->waves != 1)))
        return FATTN_ERR_UNSUPPORTED;
      break;
    }
    default:
      return FATTN_ERR_UNSUPPORTED;
  }
  *out = p;
  return FATTN_OK;
}

// Grow-only workspace per (device, stream), shared by the split-K decode (partial outputs) and
// the backward ((L, D) blocks). The lock is held across the launches that use it, so a buffer is
// never replaced while a call is between lookup and enqueue.
struct Workspace {
  float* ptr = nullptr;
  size_t floats = 0;
};
std::mutex g_ws_mutex;
std::map<std::pair<int, uintptr_t>, Workspace> g_ws;

// The workspace of (dev, stream), grown to at least `need` floats. Call with g_ws_mutex held.
// Growing waits for the stream (earlier work may still read the old buffer) and frees it.
int workspace(int dev, hipStream_t s, size_t need, float** out) {
  Workspace& ws = g_ws[{dev, reinterpret_cast<uintptr_t>(s)}];
  if (ws.floats < need) {
    if (ws.ptr) {
      hipError_t he = hipStreamSynchronize(s);
      if (he != hipSuccess) return hip_fail(FATTN_ERR_HIP, "hipStreamSynchronize", he);
      (void)hipFree(ws.ptr);
      ws.ptr = nullptr;
      ws.floats = 0;
    }
    void* mem = nullptr;
    hipError_t he = hipMalloc(&mem, need * sizeof(float));
    if (he != hipSuccess) {
      (void)hipGetLastError();
      return hip_fail(FATTN_ERR_NOMEM, "hipMalloc of the workspace", he);
    }
    ws.ptr = static_cast<float*>(mem);
    ws.floats = need;
  }
  *out = ws.ptr;
  return FATTN_OK;
}

}  // namespace
}  // namespace fattn

using namespace fattn;

extern "C" int attn_fwd_plan(int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, int dtype,
                             const fattn_cfg_t* cfg, fattn_cfg_t* out) {
  g_last_error[0] = 0;
  if (!out) return fail(FATTN_ERR_INVALID, "out is NULL");
  bool noop;
  int rc = validate_shape(B, Hq, Hkv, Tq, Tk, d, causal, dtype, &noop);
  if (rc != FATTN_OK) return rc;
  if (noop) {
    *out = fattn_cfg_t{};
    return FATTN_OK;
  }
  rc = make_plan(B, Hq, Hkv, Tq, Tk, d, causal, dtype, cfg, out);
  return rc == FATTN_OK ? rc : fail(rc, "launch configuration not implemented for this shape");
}

namespace fattn {
namespace {

// The forward pass behind every entry point. window == 0: no window; window >= 1: sliding
// window, causal implied (checked by the callers).
// noalloc: the split-K decode uses the static scratch (noalloc.hip) instead of the workspace,
// with its split count capped to fit; nothing is allocated.
int forward(const void* Q, const void* K, const void* V, void* O, float* LSE, int B, int Hq,
            int Hkv, int Tq, int Tk, int d, int causal, int window, float scale, int dtype,
            void* stream, const fattn_cfg_t* cfg, bool noalloc = false) {
  bool noop;
  int rc = validate_shape(B, Hq, Hkv, Tq, Tk, d, causal, dtype, &noop);
  if (rc != FATTN_OK) return rc;
  if (!std::isfinite(scale)) return fail(FATTN_ERR_INVALID, "scale is not finite");
  if (noop) return FATTN_OK;
  if (!Q || !K || !V || !O || !LSE) return fail(FATTN_ERR_INVALID, "NULL tensor pointer");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return fail(FATTN_ERR_INVALID, "tensor pointer not 16-byte aligned");
  // A window at least Tk wide hides nothing the causal mask does not: every row's position is
  // below Tk. Such calls run the plain causal path.
  if (window >= Tk) window = 0;
  // Under a window a decode row reads only the last `window` keys: plan the splits on those.
  const int k0 = (window > 0 && Tq == 1) ? Tk - window : 0;
  // A windowed prefill row sees at most `window` keys: the table's row for that key length, and
  // the XCD-grouped order in place of paired blocks (pairing evens out the causal triangle; past
  // the first `window` rows every query block of a window holds the same work).
  const bool window_prefill = window > 0 && Tq > 1;
  fattn_cfg_t plan;
  rc = make_plan(B, Hq, Hkv, Tq, window_prefill ? window : Tk - k0, d, causal, dtype, cfg, &plan);
  if (rc != FATTN_OK) return fail(rc, "launch configuration not implemented for this shape");
  if (window_prefill && plan.kernel == FATTN_KERNEL_PREFILL_MFMA && plan.schedule == 4 &&
      !(cfg && cfg->schedule))
    plan.schedule = 2;
  if (noalloc && plan.kernel == FATTN_KERNEL_DECODE_SPLITK) {
    // the partials of every split must fit the static scratch: fewer splits if needed
    const size_t per_split = (size_t)B * Hq * (size_t)(d + 1);
    const size_t fit = kScratchFloats / per_split;
    if (fit < 1)
      return fail(FATTN_ERR_INVALID,
                  "B*Hq*(d+1) = %zu floats exceeds the static scratch of %zu floats", per_split,
                  kScratchFloats);
    if ((size_t)plan.splits > fit) {
      fattn_cfg_t c = cfg ? *cfg : fattn_cfg_t{};
      c.kernel = FATTN_KERNEL_DECODE_SPLITK;
      c.splits = (int)fit;
      rc = make_plan(B, Hq, Hkv, Tq, Tk - k0, d, causal, dtype, &c, &plan);
      if (rc != FATTN_OK) return fail(rc, "launch configuration not implemented for this shape");
    }
  }

  Problem p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.LSE = LSE;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tq = Tq;
  p.Tk = Tk;
  p.d = d;
  p.causal = causal;
  p.window = window;
  p.qsign = scale > 0.f ? 1 : (scale < 0.f ? -1 : 0);
  p.abs_scale = scale == 0.f ? 1.f : std::fabs(scale);
  p.log2_scale = p.abs_scale * kLog2e;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);

  hipError_t e = hipSuccess;
  switch (plan.kernel) {
    case FATTN_KERNEL_PREFILL_F32:
      e = launch_prefill_f32(p, s);
      break;
    case FATTN_KERNEL_PREFILL_MFMA:
      e = launch_prefill_bf16(p, plan.block_kv, plan.waves, plan.schedule, s);
      break;
    case FATTN_KERNEL_DECODE_SPLITK: {
      int dev = 0;
      hipError_t he = hipGetDevice(&dev);
      if (he != hipSuccess) return hip_fail(FATTN_ERR_HIP, "hipGetDevice", he);
      const int nkeys = Tk - k0;
      const int chunk = ((nkeys + plan.splits - 1) / plan.splits + 31) / 32 * 32;
      const size_t rows = (size_t)B * Hq * plan.splits;
      const size_t need = rows * (size_t)d + rows;
      float* ws = nullptr;
      if (noalloc) {
        he = static_scratch(dev, &ws);
        if (he != hipSuccess) return hip_fail(FATTN_ERR_HIP, "hipGetSymbolAddress", he);
        e = launch_decode_bf16(p, k0, plan.splits, chunk, ws, ws + rows * (size_t)d, s);
        break;
      }
      std::lock_guard<std::mutex> lock(g_ws_mutex);
      rc = workspace(dev, s, need, &ws);
      if (rc != FATTN_OK) return rc;
      e = launch_decode_bf16(p, k0, plan.splits, chunk, ws, ws + rows * (size_t)d, s);
      break;
    }
    default:
      return fail(FATTN_ERR_UNSUPPORTED, "unknown kernel family");
  }
  return e == hipSuccess ? FATTN_OK : hip_fail(FATTN_ERR_HIP, "kernel launch", e);
}

}  // namespace
}  // namespace fattn

extern "C" int attn_fwd_cfg(const void* Q, const void* K, const void* V, void* O, float* LSE,
                            int B, int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale,
                            int dtype, void* stream, const fattn_cfg_t* cfg) {
  g_last_error[0] = 0;
  return forward(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, causal, 0, scale, dtype, stream, cfg);
}

extern "C" int attn_fwd(const void* Q, const void* K, const void* V, void* O, float* LSE, int B,
                        int Hq, int Hkv, int Tq, int Tk, int d, int causal, float scale, int dtype,
                        void* stream) {
  return attn_fwd_cfg(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, causal, scale, dtype, stream,
                      nullptr);
}

extern "C" int attn_fwd_noalloc(const void* Q, const void* K, const void* V, void* O,
                                float* LSE, int B, int Hq, int Hkv, int Tq, int Tk, int d,
                                int causal, float scale, int dtype, void* stream) {
  g_last_error[0] = 0;
  return forward(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, causal, 0, scale, dtype, stream,
                 nullptr, true);
}

extern "C" int attn_fwd_window_cfg(const void* Q, const void* K, const void* V, void* O,
                                   float* LSE, int B, int Hq, int Hkv, int Tq, int Tk, int d,
                                   int window, float scale, int dtype, void* stream,
                                   const fattn_cfg_t* cfg) {
  g_last_error[0] = 0;
  if (window < 1) return fail(FATTN_ERR_INVALID, "window must be >= 1");
  return forward(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, 1, window, scale, dtype, stream, cfg);
}

extern "C" int attn_fwd_window(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               int B, int Hq, int Hkv, int Tq, int Tk, int d, int window,
                               float scale, int dtype, void* stream) {
  return attn_fwd_window_cfg(Q, K, V, O, LSE, B, Hq, Hkv, Tq, Tk, d, window, scale, dtype,
                             stream, nullptr);
}

extern "C" int attn_fwd_varlen(const void* Q, const void* K, const void* V, void* O, float* LSE,
                               const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                               int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                               int Hq, int Hkv, int d, int causal, int window, float scale,
                               int dtype, void* stream) {
  g_last_error[0] = 0;
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(FATTN_ERR_INVALID, "negative size");
  if (window < 0) return fail(FATTN_ERR_INVALID, "window must be >= 0");
  if (window > 0 && causal != 1) return fail(FATTN_ERR_INVALID, "a window needs causal = 1");
  // Per-sequence lengths live on the device; shape checks use the longest ones. A causal row
  // that sees no key (a sequence with fewer keys than queries) is not an error here.
  const int tk_check = max_seqlen_k > max_seqlen_q ? max_seqlen_k : max_seqlen_q;
  bool noop;
  int rc = validate_shape(num_seqs, Hq, Hkv, max_seqlen_q, tk_check > 0 ? tk_check : 1, d,
                          causal, dtype, &noop);
  if (rc != FATTN_OK) return rc;
  if (!std::isfinite(scale)) return fail(FATTN_ERR_INVALID, "scale is not finite");
  if (noop || total_q == 0) return FATTN_OK;
  if (dtype != FATTN_BF16) return fail(FATTN_ERR_UNSUPPORTED, "packed batches are bf16 only");
  if ((long long)total_q * Hq * d > 0x7fffffffffffLL || (long long)total_k * Hkv * d > 0x7fffffffffffLL)
    return fail(FATTN_ERR_INVALID, "packed tensors too large");
  if ((long long)Hkv * d * 2 * 64 > 0x7fffffffLL) return fail(FATTN_ERR_INVALID, "Hkv * d too large");
  if (!Q || !K || !V || !O || !LSE || !cu_seqlens_q || !cu_seqlens_k)
    return fail(FATTN_ERR_INVALID, "NULL pointer");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(LSE))
    return fail(FATTN_ERR_INVALID, "tensor pointer not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return fail(FATTN_ERR_INVALID, "cu_seqlens not 4-byte aligned");
  if (window >= max_seqlen_k) window = 0;

  Problem p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.LSE = LSE;
  p.B = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tq = max_seqlen_q;
  p.Tk = max_seqlen_k;
  p.d = d;
  p.causal = causal;
  p.window = window;
  p.qsign = scale > 0.f ? 1 : (scale < 0.f ? -1 : 0);
  p.abs_scale = scale == 0.f ? 1.f : std::fabs(scale);
  p.log2_scale = p.abs_scale * kLog2e;
  Packed pk;
  pk.cu_q = cu_seqlens_q;
  pk.cu_k = cu_seqlens_k;
  pk.total_q = total_q;
  pk.total_k = total_k;
  // tile shape from the table for the longest lengths (under a window, for the window: the most
  // keys a row sees); the grid order is always 3
  fattn_cfg_t cfg = {};
  cfg.kernel = FATTN_KERNEL_PREFILL_MFMA;
  fattn_cfg_t plan;
  const int plan_tk = window > 0 ? window : (max_seqlen_k > 0 ? max_seqlen_k : 1);
  rc = make_plan(num_seqs, Hq, Hkv, max_seqlen_q > 0 ? max_seqlen_q : 1, plan_tk, d, causal, dtype,
                 &cfg, &plan);
  if (rc != FATTN_OK) return fail(rc, "launch configuration not implemented for this shape");
  hipError_t e = launch_prefill_varlen_bf16(p, pk, plan.block_kv, plan.waves, 3,
                                            reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? FATTN_OK : hip_fail(FATTN_ERR_HIP, "kernel launch", e);
}

extern "C" int attn_bwd_varlen(const void* Q, const void* K, const void* V, const void* O,
                               const void* dO, const float* LSE, void* dQ, void* dK, void* dV,
                               const int* cu_seqlens_q, const int* cu_seqlens_k, int num_seqs,
                               int total_q, int total_k, int max_seqlen_q, int max_seqlen_k,
                               int Hq, int Hkv, int d, int causal, int window, float scale,
                               int dtype, void* stream) {
  g_last_error[0] = 0;
  if (num_seqs < 0 || total_q < 0 || total_k < 0 || max_seqlen_q < 0 || max_seqlen_k < 0)
    return fail(FATTN_ERR_INVALID, "negative size");
  if (window < 0) return fail(FATTN_ERR_INVALID, "window must be >= 0");
  if (window > 0 && causal != 1) return fail(FATTN_ERR_INVALID, "a window needs causal = 1");
  const int tk_check = max_seqlen_k > max_seqlen_q ? max_seqlen_k : max_seqlen_q;
  bool noop;
  int rc = validate_shape(num_seqs, Hq, Hkv, max_seqlen_q, tk_check > 0 ? tk_check : 1, d,
                          causal, dtype, &noop);
  if (rc != FATTN_OK) return rc;
  if (!std::isfinite(scale)) return fail(FATTN_ERR_INVALID, "scale is not finite");
  if (noop || total_q == 0) return FATTN_OK;
  if (dtype != FATTN_BF16) return fail(FATTN_ERR_UNSUPPORTED, "backward is bf16 only");
  if ((long long)Hq * total_q * 8 > 0x7fffffffLL)
    return fail(FATTN_ERR_INVALID, "Hq * total_q too large for the packed backward");
  if ((long long)Hq * d * 2 * 64 > 0x7fffffffLL || (long long)Hkv * d * 2 * 64 > 0x7fffffffLL)
    return fail(FATTN_ERR_INVALID, "H * d too large");
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV || !cu_seqlens_q ||
      !cu_seqlens_k)
    return fail(FATTN_ERR_INVALID, "NULL pointer");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
    return fail(FATTN_ERR_INVALID, "tensor pointer not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(cu_seqlens_q) & 3u) ||
      (reinterpret_cast<uintptr_t>(cu_seqlens_k) & 3u))
    return fail(FATTN_ERR_INVALID, "cu_seqlens not 4-byte aligned");
  if (window >= max_seqlen_k) window = 0;

  BwdProblem p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.dO = dO;
  p.LSE = LSE;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.B = num_seqs;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tq = max_seqlen_q;
  p.Tk = max_seqlen_k;
  p.d = d;
  p.causal = causal;
  p.window = window;
  p.scale = scale;
  Packed pk;
  pk.cu_q = cu_seqlens_q;
  pk.cu_k = cu_seqlens_k;
  pk.total_q = total_q;
  pk.total_k = total_k;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(FATTN_ERR_HIP, "hipGetDevice", he);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  float* ws = nullptr;
  rc = workspace(dev, s, (size_t)2 * Hq * total_q, &ws);
  if (rc != FATTN_OK) return rc;
  he = launch_backward_varlen_bf16(p, pk, ws, s);
  return he == hipSuccess ? FATTN_OK : hip_fail(FATTN_ERR_HIP, "kernel launch", he);
}

extern "C" int attn_fwd_paged(const void* Q, const void* K_cache, const void* V_cache,
                              const int* block_table, const int* seq_lens, void* O, float* LSE,
                              int B, int Hq, int Hkv, int d, int num_blocks, int block_size,
                              int max_blocks_per_seq, float scale, int dtype, void* stream) {
  g_last_error[0] = 0;
  if (block_size < 16 || block_size > 4096 || (block_size & (block_size - 1)) != 0)
    return fail(FATTN_ERR_INVALID, "block_size must be a power of two in [16, 4096]");
  if (num_blocks < 1) return fail(FATTN_ERR_INVALID, "num_blocks must be >= 1");
  if (max_blocks_per_seq < 1) return fail(FATTN_ERR_INVALID, "max_blocks_per_seq must be >= 1");
  const long long max_keys = (long long)max_blocks_per_seq * block_size;
  if (max_keys > 0x7fffffffLL) return fail(FATTN_ERR_INVALID, "max_blocks_per_seq too large");
  if ((long long)num_blocks * Hkv * block_size * (d > 0 ? d : 1) > (1LL << 62))
    return fail(FATTN_ERR_INVALID, "cache too large");
  bool noop;
  int rc = validate_shape(B, Hq, Hkv, 1, (int)max_keys, d, 0, dtype, &noop);
  if (rc != FATTN_OK) return rc;
  if (!std::isfinite(scale)) return fail(FATTN_ERR_INVALID, "scale is not finite");
  if (noop) return FATTN_OK;
  if (dtype != FATTN_BF16) return fail(FATTN_ERR_UNSUPPORTED, "paged decode is bf16 only");
  if (!Q || !K_cache || !V_cache || !block_table || !seq_lens || !O || !LSE)
    return fail(FATTN_ERR_INVALID, "NULL pointer");
  if (!aligned16(Q) || !aligned16(K_cache) || !aligned16(V_cache) || !aligned16(O) ||
      !aligned16(LSE))
    return fail(FATTN_ERR_INVALID, "tensor pointer not 16-byte aligned");
  if ((reinterpret_cast<uintptr_t>(block_table) & 3u) || (reinterpret_cast<uintptr_t>(seq_lens) & 3u))
    return fail(FATTN_ERR_INVALID, "block_table or seq_lens not 4-byte aligned");
  fattn_cfg_t plan;
  rc = make_plan(B, Hq, Hkv, 1, (int)max_keys, d, 0, dtype, nullptr, &plan);
  if (rc != FATTN_OK) return fail(rc, "launch configuration not implemented for this shape");

  Problem p;
  p.Q = Q;
  p.K = K_cache;
  p.V = V_cache;
  p.O = O;
  p.LSE = LSE;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tq = 1;
  p.Tk = (int)max_keys;
  p.d = d;
  p.causal = 0;
  p.window = 0;
  p.qsign = scale > 0.f ? 1 : (scale < 0.f ? -1 : 0);
  p.abs_scale = scale == 0.f ? 1.f : std::fabs(scale);
  p.log2_scale = p.abs_scale * kLog2e;
  PagedKV pk;
  pk.table = block_table;
  pk.seq_lens = seq_lens;
  pk.num_blocks = num_blocks;
  pk.max_blocks = max_blocks_per_seq;
  pk.bs_shift = 0;
  while ((1 << pk.bs_shift) < block_size) ++pk.bs_shift;
  const int chunk = ((int)((max_keys + plan.splits - 1) / plan.splits) + 31) / 32 * 32;

  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(FATTN_ERR_HIP, "hipGetDevice", he);
  const size_t rows = (size_t)B * Hq * plan.splits;
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  float* ws = nullptr;
  rc = workspace(dev, s, rows * (size_t)d + rows, &ws);
  if (rc != FATTN_OK) return rc;
  he = launch_decode_paged_bf16(p, pk, plan.splits, chunk, ws, ws + rows * (size_t)d, s);
  return he == hipSuccess ? FATTN_OK : hip_fail(FATTN_ERR_HIP, "kernel launch", he);
}

extern "C" int attn_bwd(const void* Q, const void* K, const void* V, const void* O,
                        const void* dO, const float* LSE, void* dQ, void* dK, void* dV, int B,
                        int Hq, int Hkv, int Tq, int Tk, int d, int causal, int window,
                        float scale, int dtype, void* stream) {
  g_last_error[0] = 0;
  bool noop;
  int rc = validate_shape(B, Hq, Hkv, Tq, Tk, d, causal, dtype, &noop);
  if (rc != FATTN_OK) return rc;
  if (!std::isfinite(scale)) return fail(FATTN_ERR_INVALID, "scale is not finite");
  if (window < 0) return fail(FATTN_ERR_INVALID, "window must be >= 0");
  if (window > 0 && !causal) return fail(FATTN_ERR_INVALID, "a window needs causal = 1");
  if (noop) return FATTN_OK;
  if (dtype != FATTN_BF16) return fail(FATTN_ERR_UNSUPPORTED, "backward is bf16 only");
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV)
    return fail(FATTN_ERR_INVALID, "NULL tensor pointer");
  if (!aligned16(Q) || !aligned16(K) || !aligned16(V) || !aligned16(O) || !aligned16(dO) ||
      !aligned16(LSE) || !aligned16(dQ) || !aligned16(dK) || !aligned16(dV))
    return fail(FATTN_ERR_INVALID, "tensor pointer not 16-byte aligned");
  if (window >= Tk) window = 0;

  BwdProblem p;
  p.Q = Q;
  p.K = K;
  p.V = V;
  p.O = O;
  p.dO = dO;
  p.LSE = LSE;
  p.dQ = dQ;
  p.dK = dK;
  p.dV = dV;
  p.B = B;
  p.Hq = Hq;
  p.Hkv = Hkv;
  p.Tq = Tq;
  p.Tk = Tk;
  p.d = d;
  p.causal = causal;
  p.window = window;
  p.scale = scale;
  hipStream_t s = reinterpret_cast<hipStream_t>(stream);
  int dev = 0;
  hipError_t he = hipGetDevice(&dev);
  if (he != hipSuccess) return hip_fail(FATTN_ERR_HIP, "hipGetDevice", he);
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  float* ws = nullptr;
  rc = workspace(dev, s, backward_workspace_floats(B, Hq, Tq), &ws);
  if (rc != FATTN_OK) return rc;
  he = launch_backward_bf16(p, ws, s);
  return he == hipSuccess ? FATTN_OK : hip_fail(FATTN_ERR_HIP, "kernel launch", he);
}

extern "C" const char* fattn_strerror(int code) {
  switch (code) {
    case FATTN_OK: return "ok";
    case FATTN_ERR_INVALID: return "invalid argument";
    case FATTN_ERR_UNSUPPORTED: return "unsupported configuration";
    case FATTN_ERR_HIP: return "HIP runtime error";
    case FATTN_ERR_NOMEM: return "out of device memory for the workspace";
    default: return "unknown error code";
  }
}

extern "C" const char* fattn_last_error(void) { return g_last_error; }

extern "C" int fattn_version(void) { return kVersion; }

extern "C" int fattn_release(void) {
  std::lock_guard<std::mutex> lock(g_ws_mutex);
  int rc = FATTN_OK;
  int cur = -1;
  const bool have_cur = hipGetDevice(&cur) == hipSuccess;
  for (auto& kv : g_ws) {
    if (!kv.second.ptr) continue;
    if (hipSetDevice(kv.first.first) != hipSuccess || hipDeviceSynchronize() != hipSuccess ||
        hipFree(kv.second.ptr) != hipSuccess)
      rc = FATTN_ERR_HIP;
  }
  g_ws.clear();
  if (have_cur) (void)hipSetDevice(cur);
  return rc;
}
