// Host side of the C ABI declared in include/dsa.h: argument validation,
// workspace sizing, kernel dispatch, the IndexShare layer driver and the
// thread-local error text.  Every host-checkable condition is checked before
// anything is enqueued.
#include <unistd.h>
#include <cmath>

#include <atomic>
#include <chrono>
#include <cstdarg>
#include <cstdio>
#include <cstring>

#include "common.h"

#include <mutex>

// Scratch of the allocation-free indexer entry point: one copy per GPU, held
// until the process ends.  In host code this name is only a stand-in for the
// device array: its device address comes from hipGetSymbolAddress, once per
// device (see scratch_on_current_device), and only that address is used.
static __device__ __align__(256) uint8_t scratch[DSA_NOALLOC_SCRATCH_BYTES];

namespace {

thread_local char g_err[512] = "";

int fail(int code, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof(g_err), fmt, ap);
  va_end(ap);
  return code;
}

int ok() {
  g_err[0] = '\0';
  return DSA_OK;
}

// Prepends "<what>: " to the current error text.
int prefix_error(int code, const char* what, int layer) {
  char prev[sizeof(g_err)];
  memcpy(prev, g_err, sizeof(prev));
  char head[64];
  snprintf(head, sizeof(head), what, layer);
  return fail(code, "%s: %s", head, prev);
}

int hip_fail(hipError_t e, const char* what) {
  return fail(DSA_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

constexpr size_t kAlign = 256;
size_t round_up(size_t n) { return (n + kAlign - 1) / kAlign * kAlign; }

int check_batch(const dsa_batch* b) {
  if (!b) return fail(DSA_ERR_INVALID_ARG, "batch is NULL");
  if (b->num_reqs < 1) return fail(DSA_ERR_INVALID_ARG, "num_reqs must be >= 1");
  if (b->num_q_tokens < 0 || b->max_q_len < 0 || b->max_seq_len < 0)
    return fail(DSA_ERR_INVALID_ARG, "negative token count or length");
  if (b->num_q_tokens > 0 && b->max_q_len < 1)
    return fail(DSA_ERR_INVALID_ARG, "max_q_len must be >= 1");
  if (b->max_q_len > b->max_seq_len)
    return fail(DSA_ERR_INVALID_ARG, "max_q_len %d exceeds max_seq_len %d",
                b->max_q_len, b->max_seq_len);
  if (b->block_size < 1 || b->max_blocks < 1 || b->num_slots < 1)
    return fail(DSA_ERR_INVALID_ARG, "block_size, max_blocks and num_slots must be >= 1");
  if (b->block_size % 32 != 0)
    return fail(DSA_ERR_UNSUPPORTED, "block_size %d is not a multiple of 32",
                b->block_size);
  if (static_cast<int64_t>(b->max_blocks) * b->block_size < b->max_seq_len)
    return fail(DSA_ERR_INVALID_ARG,
                "max_blocks * block_size (%lld) < max_seq_len (%d)",
                static_cast<long long>(b->max_blocks) * b->block_size,
                b->max_seq_len);
  if (!b->seq_lens || !b->cu_q || !b->block_table)
    return fail(DSA_ERR_INVALID_ARG, "batch device pointers must be non-NULL");
  if (static_cast<int64_t>(b->num_q_tokens) * b->max_seq_len > (int64_t(1) << 40))
    return fail(DSA_ERR_UNSUPPORTED, "num_q_tokens * max_seq_len too large");
  return DSA_OK;
}

bool known_dtype(int d) {
  return d == DSA_F32 || d == DSA_BF16 || d == DSA_FP8_E4M3;
}

// score rows are padded to 64 floats so that every row starts 256-byte aligned
int64_t score_row_stride(const dsa_batch* b) {
  return (static_cast<int64_t>(b->max_seq_len) + 63) / 64 * 64;
}

// fp32 score rows, then the per-chunk score ranges, of a window of n query
// tokens
size_t topk_scores_bytes(const dsa_batch* b, int64_t n) {
  return round_up(static_cast<size_t>(n) * static_cast<size_t>(score_row_stride(b)) *
                  sizeof(float));
}
size_t topk_ws_n(const dsa_batch* b, int64_t n) {
  return topk_scores_bytes(b, n) +
         round_up(static_cast<size_t>(n) *
                  static_cast<size_t>(dsa::indexer_range_stride_max(b->max_seq_len)) *
                  2 * sizeof(float));
}
// the whole batch in one window (the fastest), and the least accepted: a
// window of kMinWindow tokens (fewer when the batch has fewer)
constexpr int64_t kMinWindow = 16;
size_t topk_ws(const dsa_batch* b) { return topk_ws_n(b, b->num_q_tokens); }
size_t topk_ws_min(const dsa_batch* b) {
  return topk_ws_n(b, b->num_q_tokens < kMinWindow ? b->num_q_tokens : kMinWindow);
}
// the query tokens per window that a workspace of ws_bytes holds (>= 1 when
// ws_bytes >= topk_ws_min): the whole batch, else whole blocks of 16 tokens
int64_t topk_window(const dsa_batch* b, size_t ws_bytes) {
  const int64_t n = b->num_q_tokens;
  if (topk_ws_n(b, n) <= ws_bytes) return n;
  const size_t per = static_cast<size_t>(score_row_stride(b)) * sizeof(float) +
                     static_cast<size_t>(dsa::indexer_range_stride_max(b->max_seq_len)) *
                         2 * sizeof(float);
  int64_t w = static_cast<int64_t>(ws_bytes / per);
  if (w >= kMinWindow) w = w / kMinWindow * kMinWindow;
  while (w > 1 && topk_ws_n(b, w) > ws_bytes) w -= (w > kMinWindow ? kMinWindow : 1);
  return w < 1 ? 1 : (w > n ? n : w);
}

size_t mla_ws(const dsa_batch* b, int n_heads, int R, int P, int topk, int dtype) {
  const int split = dsa::mla_choose_split(b, dtype, n_heads, R, P, topk);
  if (split <= 1) return 0;
  const size_t th = static_cast<size_t>(b->num_q_tokens) * split * n_heads;
  return round_up(th * R * sizeof(uint16_t)) + round_up(th * sizeof(float)) +
         round_up(static_cast<size_t>(b->num_q_tokens) * 128);   // a 128-byte line per token
}

// 48-bit tag of a sparse MLA call: split arrivals counted under another tag
// (an earlier call, or whatever the workspace held) do not count.  Starts
// from a clock- and process-dependent value and never returns 0.
unsigned long long next_call_tag() {
  static std::atomic<unsigned long long> next{
      (static_cast<unsigned long long>(
           std::chrono::steady_clock::now().time_since_epoch().count()) ^
       (static_cast<unsigned long long>(getpid()) << 24)) * 0x9E3779B97F4A7C15ull};
  for (;;) {
    const unsigned long long tag = next.fetch_add(1) & ((1ull << 48) - 1);
    if (tag) return tag;
  }
}

int check_indexer(const dsa_batch* b, const void* q, int q_dtype,
                  const float* w, int n_heads, int d_idx, const void* k_cache,
                  const float* k_scale, int cache_dtype, int topk,
                  const int32_t* topk_idx, const void* ws, size_t ws_bytes,
                  bool check_ws = true, const float* q_scale = nullptr) {
  int st = check_batch(b);
  if (st) return st;
  if (!q || !w || !k_cache || !topk_idx)
    return fail(DSA_ERR_INVALID_ARG, "q, w, k_cache and topk_idx must be non-NULL");
  if (!known_dtype(q_dtype) || !known_dtype(cache_dtype))
    return fail(DSA_ERR_INVALID_ARG, "unknown dtype");
  if (q_dtype == DSA_FP8_E4M3) {
    if (!q_scale)
      return fail(DSA_ERR_UNSUPPORTED, "FP8 queries go through dsa_indexer_topk_fp8q");
    if (cache_dtype != DSA_FP8_E4M3)
      return fail(DSA_ERR_UNSUPPORTED, "FP8 queries need an FP8 cache");
  }
  if (cache_dtype == DSA_FP8_E4M3) {
    if (q_dtype != DSA_BF16 && q_dtype != DSA_FP8_E4M3)
      return fail(DSA_ERR_UNSUPPORTED, "an FP8 cache needs bf16 or FP8 queries");
    if (!k_scale) return fail(DSA_ERR_INVALID_ARG, "FP8 cache needs k_scale");
  } else if (cache_dtype != q_dtype) {
    return fail(DSA_ERR_UNSUPPORTED, "q dtype %d with cache dtype %d", q_dtype,
                cache_dtype);
  }
  if (n_heads < 1 || n_heads > 64 || d_idx < 1 || d_idx > 256)
    return fail(DSA_ERR_UNSUPPORTED, "n_heads %d / d_idx %d outside 1..64 / 1..256",
                n_heads, d_idx);
  if (n_heads * d_idx > 8192)
    return fail(DSA_ERR_UNSUPPORTED, "n_heads * d_idx > 8192");
  if (topk < 1 || topk > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "topk %d outside 1..%d", topk, DSA_MAX_TOPK);
  if (!check_ws) return DSA_OK;
  if (b->num_q_tokens > 0 && (!ws || ws_bytes < topk_ws_min(b)))
    return fail(DSA_ERR_WORKSPACE,
                "workspace needs at least %zu bytes (%zu for the batch in one pass), got %zu",
                topk_ws_min(b), topk_ws(b), ws ? ws_bytes : static_cast<size_t>(0));
  if (reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return DSA_OK;
}

int check_mla(const dsa_batch* b, const void* q, const void* kv, int dtype,
              int n_heads, int R, int P, const int32_t* idx, int topk, float scale,
              const void* out, const void* ws, size_t ws_bytes) {
  int st = check_batch(b);
  if (st) return st;
  if (!q || !kv || !idx || !out)
    return fail(DSA_ERR_INVALID_ARG, "q, kv_cache, topk_idx and out must be non-NULL");
  if (dtype != DSA_F32 && dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "sparse_mla_attn dtype must be F32 or BF16");
  if (n_heads < 1 || n_heads > 128 || R < 1 || P < 0 || R + P > 1024)
    return fail(DSA_ERR_UNSUPPORTED, "n_heads %d, kv_lora_rank %d, rope_dim %d",
                n_heads, R, P);
  if (topk < 1 || topk > DSA_MAX_TOPK)
    return fail(DSA_ERR_UNSUPPORTED, "topk %d outside 1..%d", topk, DSA_MAX_TOPK);
  if (!(scale > 0.0f) || !std::isfinite(scale))
    return fail(DSA_ERR_INVALID_ARG, "softmax_scale must be finite and > 0");
  const size_t need = mla_ws(b, n_heads, R, P, topk, dtype);
  if (need && (!ws || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                ws ? ws_bytes : static_cast<size_t>(0));
  if (need && reinterpret_cast<uintptr_t>(ws) % kAlign)
    return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
  return DSA_OK;
}

// Score + top-k over the batch's query tokens, in windows of as many
// tokens as the workspace holds (one window when it holds the batch).
int run_indexer(const dsa_batch* b, const void* q, int q_dtype, const float* w,
                int n_heads, int d_idx, const void* k_cache, const float* k_scale,
                int cache_dtype, int topk, int32_t* topk_idx, void* ws, size_t ws_bytes,
                hipStream_t stream, const float* q_scale = nullptr) {
  dsa::IndexerArgs a;
  a.b = *b;
  a.q = q;
  a.q_dtype = q_dtype;
  a.q_scale = q_scale;
  a.w = w;
  a.n_heads = n_heads;
  a.d_idx = d_idx;
  a.k_cache = k_cache;
  a.k_scale = k_scale;
  a.cache_dtype = cache_dtype;
  a.topk = topk;
  a.topk_idx = topk_idx;
  a.row_stride = score_row_stride(b);
  const int64_t n = b->num_q_tokens;
  const int64_t win = n > 0 ? topk_window(b, ws_bytes) : 0;
  hipError_t e;
#ifdef DSA_DEBUG
  // checked build: metadata validated, output and workspace filled with
  // canaries before the call, every row checked after it
  e = dsa::debug_check_batch(*b, stream);
  if (e == hipSuccess)
    e = dsa::debug_fill(topk_idx, static_cast<size_t>(n) * topk * sizeof(int32_t),
                        static_cast<uint32_t>(dsa::kCanaryIdx), stream);
  if (e == hipSuccess && win > 0)
    e = dsa::debug_fill(ws, topk_ws_n(b, win), dsa::kPoisonWorkspace, stream);
  if (e != hipSuccess) return hip_fail(e, "checked-build launch");
#endif
  for (int64_t w0 = 0; w0 < n; w0 += win) {
    a.win_lo = static_cast<int32_t>(w0);
    a.win_hi = static_cast<int32_t>(w0 + win < n ? w0 + win : n);
    a.scores = static_cast<float*>(ws);
    a.chunk_range = reinterpret_cast<float2*>(static_cast<char*>(ws) + topk_scores_bytes(b, win));
    a.range_stride = 0;
    a.chunk_keys = 0;
    e = dsa::launch_indexer_score(a, stream);
    if (e != hipSuccess) return hip_fail(e, "indexer score launch");
    e = dsa::launch_topk(a, stream);
    if (e != hipSuccess) return hip_fail(e, "top-k launch");
  }
#ifdef DSA_DEBUG
  e = dsa::debug_check_topk_out(*b, topk_idx, topk, stream);
  if (e != hipSuccess) return hip_fail(e, "checked-build launch");
#endif
  return ok();
}

int run_mla(const dsa_batch* b, const void* q, const void* kv, int dtype,
            int n_heads, int R, int P, const int32_t* idx, int topk, float scale,
            void* out, float* lse, void* ws, hipStream_t stream) {
  dsa::MlaArgs a;
  a.b = *b;
  a.q = q;
  a.kv = kv;
  a.dtype = dtype;
  a.n_heads = n_heads;
  a.R = R;
  a.P = P;
  a.idx = idx;
  a.topk = topk;
  a.scale = scale;
  a.out = out;
  a.lse = lse;
  a.n_split = dsa::mla_choose_split(b, dtype, n_heads, R, P, topk);
  a.part_o = nullptr;
  a.part_lse = nullptr;
  a.arrivals = nullptr;
  a.call_tag = 0;
  if (a.n_split > 1) {
    const size_t th = static_cast<size_t>(b->num_q_tokens) * a.n_split * n_heads;
    a.part_o = static_cast<uint16_t*>(ws);
    a.part_lse = reinterpret_cast<float*>(static_cast<char*>(ws) +
                                          round_up(th * R * sizeof(uint16_t)));
    a.arrivals = reinterpret_cast<unsigned long long*>(
        static_cast<char*>(ws) + round_up(th * R * sizeof(uint16_t)) +
        round_up(th * sizeof(float)));
    a.call_tag = next_call_tag();
  }
  hipError_t e;
#ifdef DSA_DEBUG
  const size_t n_out = static_cast<size_t>(b->num_q_tokens) * n_heads * R;
  const int out_bytes = dtype == DSA_BF16 ? 2 : 4;
  const uint32_t out_canary = out_bytes == 2 ? dsa::kCanaryBf16 : dsa::kCanaryF32;
  e = dsa::debug_check_batch(*b, stream);
  if (e == hipSuccess) e = dsa::debug_check_topk_in(*b, idx, topk, stream);
  if (e == hipSuccess)
    e = dsa::debug_fill(out, n_out * out_bytes,
                        out_bytes == 2 ? (out_canary | (out_canary << 16)) : out_canary, stream);
  if (e == hipSuccess && lse)
    e = dsa::debug_fill(lse, static_cast<size_t>(b->num_q_tokens) * n_heads * sizeof(float),
                        dsa::kCanaryF32, stream);
  if (e == hipSuccess)
    e = dsa::debug_fill(ws, mla_ws(b, n_heads, R, P, topk, dtype), dsa::kPoisonWorkspace, stream);
  if (e != hipSuccess) return hip_fail(e, "checked-build launch");
#endif
  e = dsa::launch_sparse_mla(a, stream);
  if (e != hipSuccess) return hip_fail(e, "sparse MLA launch");
#ifdef DSA_DEBUG
  e = dsa::debug_check_unwritten(out, n_out, out_bytes, out_canary, stream);
  if (e == hipSuccess && lse)
    e = dsa::debug_check_unwritten(lse, static_cast<size_t>(b->num_q_tokens) * n_heads, 4,
                                   dsa::kCanaryF32, stream);
  if (e != hipSuccess) return hip_fail(e, "checked-build launch");
#endif
  return ok();
}

int resolve_sources(int32_t n_layers, const int32_t* types, int32_t n_types,
                    int32_t* src) {
  if (n_layers < 0) return fail(DSA_ERR_INVALID_ARG, "n_layers < 0");
  if (n_layers > 0 && (!types || !src))
    return fail(DSA_ERR_INVALID_ARG, "types and src must be non-NULL");
  if (n_types < n_layers)
    return fail(DSA_ERR_INDEXER_TYPES,
                "indexer_types has %d entries for %d layers", n_types, n_layers);
  for (int i = 0; i < n_types; ++i)
    if (types[i] != DSA_LAYER_FULL && types[i] != DSA_LAYER_SHARED)
      return fail(DSA_ERR_INDEXER_TYPES, "unknown indexer type %d at layer %d",
                  types[i], i);
  int last_full = -1;
  for (int i = 0; i < n_layers; ++i) {
    if (types[i] == DSA_LAYER_FULL) last_full = i;
    else if (last_full < 0)
      return fail(DSA_ERR_INDEXER_TYPES,
                  "shared layer %d has no preceding full layer", i);
  }
  last_full = -1;
  for (int i = 0; i < n_layers; ++i) {
    if (types[i] == DSA_LAYER_FULL) last_full = i;
    src[i] = last_full;
  }
  return DSA_OK;
}

// Device address of `scratch` on the current device, looked up on the first
// call on that device and kept.  The stream (if any) must belong to the
// current device.  Returns DSA_OK or an error code with the text set.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

int scratch_on_current_device(hipStream_t stream, void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(DSA_ERR_UNSUPPORTED, "device %d beyond the %d devices supported", dev,
                kMaxDevices);
  if (stream) {
    hipDevice_t sdev = -1;
    e = hipStreamGetDevice(stream, &sdev);
    if (e != hipSuccess) return hip_fail(e, "hipStreamGetDevice");
    if (sdev != dev)
      return fail(DSA_ERR_INVALID_ARG,
                  "the stream belongs to device %d but device %d is current", sdev, dev);
  }
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e, "hipGetSymbolAddress(scratch)");
    if (!p || reinterpret_cast<uintptr_t>(p) % kAlign)
      return fail(DSA_ERR_HIP, "scratch address %p is not 256-byte aligned", p);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return DSA_OK;
}

}  // namespace

extern "C" {

int dsa_indexer_cache_write(const void* k_new, int32_t k_dtype, int32_t n_new,
                            int32_t d_idx, const int64_t* slot_mapping,
                            int64_t num_slots, void* k_cache, float* k_scale,
                            int32_t cache_dtype, void* stream) {
  if (n_new < 0 || d_idx < 1 || d_idx > 1024 || num_slots < 1)
    return fail(DSA_ERR_INVALID_ARG, "n_new %d, d_idx %d, num_slots %lld", n_new,
                d_idx, static_cast<long long>(num_slots));
  if (n_new > 0 && (!k_new || !slot_mapping || !k_cache))
    return fail(DSA_ERR_INVALID_ARG, "k_new, slot_mapping and k_cache must be non-NULL");
  if (!known_dtype(k_dtype) || !known_dtype(cache_dtype))
    return fail(DSA_ERR_INVALID_ARG, "unknown dtype");
  if (k_dtype == DSA_FP8_E4M3)
    return fail(DSA_ERR_UNSUPPORTED, "new keys must be F32 or BF16");
  if (cache_dtype == DSA_FP8_E4M3) {
    if (n_new > 0 && !k_scale)
      return fail(DSA_ERR_INVALID_ARG, "FP8 cache needs k_scale");
  } else if (cache_dtype != k_dtype) {
    return fail(DSA_ERR_UNSUPPORTED, "a %s cache stores keys unchanged; key dtype differs",
                cache_dtype == DSA_BF16 ? "BF16" : "F32");
  }
#ifdef DSA_DEBUG
  {
    const hipError_t ec = dsa::debug_check_slots(slot_mapping, n_new, num_slots,
                                                 static_cast<hipStream_t>(stream));
    if (ec != hipSuccess) return hip_fail(ec, "checked-build launch");
  }
#endif
  hipError_t e = dsa::launch_cache_write(k_new, k_dtype, n_new, d_idx,
                                         slot_mapping, num_slots, k_cache,
                                         k_scale, cache_dtype,
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "cache write launch");
  return ok();
}

size_t dsa_indexer_topk_workspace_size(const dsa_batch* batch, int32_t topk) {
  (void)topk;
  if (!batch || batch->num_q_tokens < 0 || batch->max_seq_len < 0) return 0;
  return topk_ws(batch);
}

size_t dsa_indexer_topk_workspace_min(const dsa_batch* batch, int32_t topk) {
  (void)topk;
  if (!batch || batch->num_q_tokens < 0 || batch->max_seq_len < 0) return 0;
  return topk_ws_min(batch);
}

int dsa_indexer_topk(const dsa_batch* batch, const void* q, int32_t q_dtype,
                     const float* w, int32_t n_heads, int32_t d_idx,
                     const void* k_cache, const float* k_scale,
                     int32_t cache_dtype, int32_t topk, int32_t* topk_idx,
                     void* workspace, size_t ws_bytes, void* stream) {
  int st = check_indexer(batch, q, q_dtype, w, n_heads, d_idx, k_cache, k_scale,
                         cache_dtype, topk, topk_idx, workspace, ws_bytes);
  if (st) return st;
  return run_indexer(batch, q, q_dtype, w, n_heads, d_idx, k_cache, k_scale,
                     cache_dtype, topk, topk_idx, workspace, ws_bytes,
                     static_cast<hipStream_t>(stream));
}

int dsa_rotate_quantize(const void* x, int32_t x_dtype, int64_t n_rows, int32_t d,
                        const int64_t* row_slots, int64_t num_out, uint8_t* codes,
                        float* scales, void* stream) {
  if (n_rows < 0 || num_out < 1)
    return fail(DSA_ERR_INVALID_ARG, "n_rows %lld / num_out %lld",
                static_cast<long long>(n_rows), static_cast<long long>(num_out));
  if (d < 32 || d > 256 || (d & (d - 1)))
    return fail(DSA_ERR_UNSUPPORTED, "d %d is not a power of two in 32..256", d);
  if (x_dtype != DSA_F32 && x_dtype != DSA_BF16)
    return fail(DSA_ERR_UNSUPPORTED, "rows must be F32 or BF16");
  if (n_rows > 0 && (!x || !codes || !scales))
    return fail(DSA_ERR_INVALID_ARG, "x, codes and scales must be non-NULL");
  if (!row_slots && n_rows > num_out)
    return fail(DSA_ERR_INVALID_ARG, "n_rows exceeds num_out without row_slots");
  hipError_t e = dsa::launch_rotate_quantize(x, x_dtype, n_rows, d, row_slots, num_out,
                                             codes, scales, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "rotate-quantize launch");
  return ok();
}

int dsa_indexer_topk_fp8q(const dsa_batch* batch, const uint8_t* q_codes,
                          const float* q_scale, const float* w, int32_t n_heads,
                          int32_t d_idx, const void* k_cache, const float* k_scale,
                          int32_t topk, int32_t* topk_idx, void* workspace,
                          size_t ws_bytes, void* stream) {
  if (!q_scale) return fail(DSA_ERR_INVALID_ARG, "q_scale must be non-NULL");
  int st = check_indexer(batch, q_codes, DSA_FP8_E4M3, w, n_heads, d_idx, k_cache, k_scale,
                         DSA_FP8_E4M3, topk, topk_idx, workspace, ws_bytes, true, q_scale);
  if (st) return st;
  return run_indexer(batch, q_codes, DSA_FP8_E4M3, w, n_heads, d_idx, k_cache, k_scale,
                     DSA_FP8_E4M3, topk, topk_idx, workspace, ws_bytes,
                     static_cast<hipStream_t>(stream), q_scale);
}

size_t dsa_indexer_prologue_workspace_size(int32_t n_tokens, const dsa_prologue_dims* d) {
  if (n_tokens < 0 || !d || d->n_heads < 1 || d->head_dim < 1) return 0;
  return round_up(dsa::prologue_part_floats(n_tokens, d) * sizeof(float));
}

int dsa_indexer_prologue(int32_t n_tokens, const dsa_prologue_dims* d, const void* hidden,
                         const void* qa_normed, const float* cos, const float* sin,
                         const void* wq_b, const void* wk, const void* weights_proj,
                         const float* k_norm_weight, const int64_t* slot_mapping,
                         int64_t num_slots, void* k_cache, float* k_scale,
                         int32_t cache_dtype, void* q_out, void* k_out, float* w_out,
                         void* workspace, size_t ws_bytes, void* stream) {
  if (!d) return fail(DSA_ERR_INVALID_ARG, "dims is NULL");
  if (n_tokens < 0) return fail(DSA_ERR_INVALID_ARG, "n_tokens < 0");
  if (d->head_dim != 128)
    return fail(DSA_ERR_UNSUPPORTED, "head_dim %d (the prologue supports 128)", d->head_dim);
  if (d->n_heads < 1 || d->n_heads > 64)
    return fail(DSA_ERR_UNSUPPORTED, "n_heads %d outside 1..64", d->n_heads);
  if (d->rope_dim < 0 || d->rope_dim > d->head_dim || d->rope_dim % 2)
    return fail(DSA_ERR_UNSUPPORTED, "rope_dim %d must be even and <= head_dim", d->rope_dim);
  if (d->q_lora_rank < 32 || d->q_lora_rank % 32 || d->hidden_dim < 32 || d->hidden_dim % 32)
    return fail(DSA_ERR_UNSUPPORTED, "q_lora_rank %d and hidden_dim %d must be multiples of 32",
                d->q_lora_rank, d->hidden_dim);
  if (!(d->eps >= 0.0f) || !std::isfinite(d->eps))
    return fail(DSA_ERR_INVALID_ARG, "eps must be finite and >= 0");
  if (n_tokens > 0 && (!hidden || !qa_normed || !wq_b || !wk || !weights_proj ||
                       !k_norm_weight || !q_out || !w_out || (d->rope_dim && (!cos || !sin))))
    return fail(DSA_ERR_INVALID_ARG, "input, weight and output pointers must be non-NULL");
  if (slot_mapping) {
    if (!k_cache || num_slots < 1)
      return fail(DSA_ERR_INVALID_ARG, "a cache write needs k_cache and num_slots");
    if (cache_dtype != DSA_BF16 && cache_dtype != DSA_FP8_E4M3)
      return fail(DSA_ERR_UNSUPPORTED, "prologue cache dtype must be BF16 or FP8_E4M3");
    if (cache_dtype == DSA_FP8_E4M3 && !k_scale)
      return fail(DSA_ERR_INVALID_ARG, "FP8 cache needs k_scale");
  }
  const size_t need = dsa_indexer_prologue_workspace_size(n_tokens, d);
  if (n_tokens > 0 && (!workspace || ws_bytes < need))
    return fail(DSA_ERR_WORKSPACE, "workspace needs %zu bytes, got %zu", need,
                workspace ? ws_bytes : static_cast<size_t>(0));
  if (reinterpret_cast<uintptr_t>(workspace) % kAlign)
    return fail(DSA_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
#ifdef DSA_DEBUG
  if (slot_mapping) {
    const hipError_t ec = dsa::debug_check_slots(slot_mapping, n_tokens, num_slots,
                                                 static_cast<hipStream_t>(stream));
    if (ec != hipSuccess) return hip_fail(ec, "checked-build launch");
  }
#endif
  hipError_t e = dsa::launch_prologue(n_tokens, d, hidden, qa_normed, cos, sin, wq_b, wk,
                                      weights_proj, k_norm_weight, slot_mapping, num_slots,
                                      k_cache, k_scale, cache_dtype, q_out, k_out, w_out,
                                      static_cast<float*>(workspace),
                                      static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "prologue launch");
  return ok();
}

int dsa_indexer_topk_noalloc(const dsa_batch* batch, const void* q, int32_t q_dtype,
                             const float* w, int32_t n_heads, int32_t d_idx,
                             const void* k_cache, const float* k_scale,
                             int32_t cache_dtype, int32_t topk, int32_t* topk_idx,
                             void* stream) {
  // every host-side check first, the scratch's size included
  if (batch && batch->num_q_tokens >= 0 && batch->max_seq_len >= 0 &&
      topk_ws(batch) > static_cast<size_t>(DSA_NOALLOC_SCRATCH_BYTES))
    return fail(DSA_ERR_WORKSPACE,
                "this batch needs %zu bytes of scratch; the allocation-free entry point "
                "holds %d (use dsa_indexer_topk with a workspace)",
                topk_ws(batch), DSA_NOALLOC_SCRATCH_BYTES);
  int st = check_indexer(batch, q, q_dtype, w, n_heads, d_idx, k_cache, k_scale,
                         cache_dtype, topk, topk_idx, nullptr, 0, /*check_ws=*/false);
  if (st) return st;
  void* ws = nullptr;
  st = scratch_on_current_device(static_cast<hipStream_t>(stream), &ws);
  if (st) return st;
  return run_indexer(batch, q, q_dtype, w, n_heads, d_idx, k_cache, k_scale,
                     cache_dtype, topk, topk_idx, ws, topk_ws(batch),
                     static_cast<hipStream_t>(stream));
}

size_t sparse_mla_attn_workspace_size(const dsa_batch* batch, int32_t n_heads,
                                      int32_t kv_lora_rank, int32_t rope_dim,
                                      int32_t topk, int32_t dtype) {
  if (!batch || batch->num_q_tokens < 0) return 0;
  return mla_ws(batch, n_heads, kv_lora_rank, rope_dim, topk, dtype);
}

int sparse_mla_attn(const dsa_batch* batch, const void* q, const void* kv_cache,
                    int32_t dtype, int32_t n_heads, int32_t kv_lora_rank,
                    int32_t rope_dim, const int32_t* topk_idx, int32_t topk,
                    float softmax_scale, void* out, float* lse, void* workspace,
                    size_t ws_bytes, void* stream) {
  int st = check_mla(batch, q, kv_cache, dtype, n_heads, kv_lora_rank, rope_dim,
                     topk_idx, topk, softmax_scale, out, workspace, ws_bytes);
  if (st) return st;
  return run_mla(batch, q, kv_cache, dtype, n_heads, kv_lora_rank, rope_dim,
                 topk_idx, topk, softmax_scale, out, lse, workspace,
                 static_cast<hipStream_t>(stream));
}

int dsa_resolve_indexer_sources(int32_t n_layers, const int32_t* types,
                                int32_t n_types, int32_t* src) {
  int st = resolve_sources(n_layers, types, n_types, src);
  return st ? st : ok();
}

size_t indexshare_forward_workspace_size(const dsa_batch* batch,
                                         const dsa_stack_dims* d) {
  if (!batch || !d || batch->num_q_tokens < 0) return 0;
  size_t a = topk_ws(batch);
  size_t m = mla_ws(batch, d->n_heads, d->kv_lora_rank, d->rope_dim, d->topk,
                    d->mla_dtype);
  return a > m ? a : m;
}

int indexshare_forward(const dsa_batch* batch, int32_t n_layers,
                       const int32_t* types, int32_t n_types,
                       const dsa_layer* layers, const dsa_stack_dims* d,
                       const int32_t** active_topk, void* workspace,
                       size_t ws_bytes, void* stream) {
  if (!d) return fail(DSA_ERR_INVALID_ARG, "dims is NULL");
  if (n_layers < 1) return fail(DSA_ERR_INVALID_ARG, "n_layers must be >= 1");
  if (!layers) return fail(DSA_ERR_INVALID_ARG, "layers is NULL");
  int32_t src_stack[256];
  if (n_layers > 256) return fail(DSA_ERR_UNSUPPORTED, "more than 256 layers");
  int st = resolve_sources(n_layers, types, n_types, src_stack);
  if (st) return st;
  // validate every layer before enqueuing anything
  for (int i = 0; i < n_layers; ++i) {
    const dsa_layer& L = layers[i];
    if (src_stack[i] == i) {
      if (!L.topk_idx)
        return fail(DSA_ERR_MISSING_TOPK, "full layer %d has no topk_idx buffer", i);
      st = check_indexer(batch, L.q_idx, d->q_idx_dtype, L.w, d->n_idx_heads,
                         d->d_idx, L.k_cache, L.k_scale, d->idx_cache_dtype,
                         d->topk, L.topk_idx, workspace, ws_bytes);
      if (st) return prefix_error(st, "layer %d indexer", i);
    }
    st = check_mla(batch, L.q_mla, L.kv_cache, d->mla_dtype, d->n_heads,
                   d->kv_lora_rank, d->rope_dim, layers[src_stack[i]].topk_idx,
                   d->topk, d->softmax_scale, L.out, workspace, ws_bytes);
    if (st) return prefix_error(st, "layer %d attention", i);
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int32_t* active = nullptr;
  for (int i = 0; i < n_layers; ++i) {
    const dsa_layer& L = layers[i];
    if (src_stack[i] == i) {
      st = run_indexer(batch, L.q_idx, d->q_idx_dtype, L.w, d->n_idx_heads,
                       d->d_idx, L.k_cache, L.k_scale, d->idx_cache_dtype,
                       d->topk, L.topk_idx, workspace, ws_bytes, s);
      if (st) return st;
      active = L.topk_idx;
    }
    // a shared layer keeps `active`, the buffer of layer src_stack[i]
    if (active_topk) active_topk[i] = active;
    st = run_mla(batch, L.q_mla, L.kv_cache, d->mla_dtype, d->n_heads,
                 d->kv_lora_rank, d->rope_dim, active, d->topk,
                 d->softmax_scale, L.out, L.lse, workspace, s);
    if (st) return st;
  }
  return ok();
}

int dsa_fp8_decode_check(const uint8_t* codes, float* out, int32_t n,
                         void* stream) {
  if (n < 0 || n % 8 != 0)
    return fail(DSA_ERR_INVALID_ARG, "n must be a non-negative multiple of 8");
  if (n > 0 && (!codes || !out))
    return fail(DSA_ERR_INVALID_ARG, "codes and out must be non-NULL");
  hipError_t e = dsa::launch_fp8_decode_check(codes, out, n,
                                              static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "fp8 decode launch");
  return ok();
}

int dsa_debug_faults(uint32_t* faults, int32_t clear) {
  if (!faults) return fail(DSA_ERR_INVALID_ARG, "faults is NULL");
#ifdef DSA_DEBUG
  const hipError_t e = dsa::debug_faults(faults, clear != 0);
  if (e != hipSuccess) return hip_fail(e, "reading the fault word");
  return ok();
#else
  (void)clear;
  *faults = 0;
  return fail(DSA_ERR_UNSUPPORTED, "not the checked build (libdsa_debug.so)");
#endif
}

const char* dsa_last_error(void) { return g_err; }

}  // extern "C"
