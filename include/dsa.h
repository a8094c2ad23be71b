/*
 * dsa.h - C ABI of the MI355X (gfx950) DSA indexer + top-k + absorbed
 * sparse-MLA library (libdsa.so).
 *
 * The method: for each query token, a light "lightning" indexer with H_I
 * heads scores every causal cached token,
 *     score[t, s] = sum_h w[t, h] * ReLU(q[t, h, :] . k[s, :]),
 * the top `topk` positions are kept (ties go to the lower position), and
 * absorbed multi-head latent attention then runs only over the latent rows
 * cached at those positions.  With GLM-5.2 IndexShare, "shared" layers reuse
 * the top-k of the nearest preceding "full" layer.
 *
 * Passages the operations follow (page "GLM5 TensorCast 适配设计", i.e. the
 * GLM5 TensorCast adaptation design, unless another page is named):
 *   - section "DSA Indexer fused semantic op": one op covers cache write,
 *     scoring, head-weight mixing, head reduction and top-k; the indexer
 *     cache is a mutable argument addressed by slot_mapping, block_tables and
 *     seq_lens; the result has shape (batch, seq_len, min(topk_limit,
 *     active_seq_len)) with a static width topk_limit; topk_limit and
 *     topk_indices are handed to the MLA backend;
 *   - section "Performance model design": score MMA, head-weight multiply /
 *     head reduce / ReLU and scale shaping, top-k selection, key-cache and
 *     FP8 scale-cache traffic; the sparse attention length is the top-k width;
 *   - section "KV cache dtype and parallel-linear boundary fix": the indexer
 *     cache is FP8 when attention is FP8, else the model dtype; only full
 *     IndexShare layers own an indexer cache;
 *   - section "GLM-5.2 IndexShare": full / shared layer types, the nearest
 *     preceding full layer is the source, invalid type lists are rejected;
 *   - page "GLM5 full-stack LoRA", section 1 and section 2.1: top-k must be
 *     deterministic (torch.topk tie order differs between builds);
 *     section 2.2: absorbed MLA over the latent rows.
 *
 * Conventions for every entry point
 *   - Pointers are DEVICE pointers unless marked [host].  All device buffers
 *     belong to the caller; the library never allocates or frees device
 *     memory and never synchronises the device (dsa_debug_faults of the
 *     checked build excepted).  State kept between calls: the thread-local
 *     error text, a process-wide counter that tags each sparse_mla_attn
 *     call, once dsa_indexer_topk_noalloc has run on a device, that
 *     device's static scratch array and its address, and each device's
 *     fault word (checked build).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Every call only
 *     enqueues work on it; inputs must stay valid until that work completes.
 *   - Return value: DSA_OK (0) or a negative dsa_status.  Every condition
 *     that can be checked on the host (null pointers, sizes, dtypes, the
 *     workspace size, IndexShare type lists) is checked BEFORE anything is
 *     enqueued, so a failed call has no effect.  dsa_last_error() then
 *     describes the failure.
 *   - Device-resident metadata (seq_lens, cu_q, block_table, slot_mapping,
 *     topk indices) must agree with the host-side bounds in dsa_batch.
 *     Kernels clamp or skip values outside those bounds so that no memory
 *     outside the given buffers is touched, but results are then unspecified.
 *   - Row-major layouts throughout; "[A, B]" lists dims outer to inner.
 *   - Positions are logical per-request positions 0..seq_len-1; the physical
 *     cache row (slot) of position s of request b is
 *         block_table[b * max_blocks + s / block_size] * block_size
 *         + s % block_size.
 */
#ifndef DSA_H
#define DSA_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* storage / arithmetic types */
typedef enum {
  DSA_F32 = 0,      /* IEEE binary32                                      */
  DSA_BF16 = 1,     /* bfloat16 (upper half of binary32)                  */
  DSA_FP8_E4M3 = 2  /* OCP e4m3fn: bias 7, max 448, 0x7F/0xFF = NaN       */
} dsa_dtype;

typedef enum {
  DSA_OK = 0,
  DSA_ERR_INVALID_ARG = -1,   /* null pointer, negative or inconsistent size */
  DSA_ERR_UNSUPPORTED = -2,   /* valid but not implemented (dtype, shape)    */
  DSA_ERR_INDEXER_TYPES = -3, /* bad IndexShare type list (the ValueError
                                 case of section "GLM-5.2 IndexShare")       */
  DSA_ERR_MISSING_TOPK = -4,  /* a full layer has no top-k buffer to fill    */
  DSA_ERR_WORKSPACE = -5,     /* workspace null or smaller than required     */
  DSA_ERR_HIP = -6            /* a HIP launch failed                         */
} dsa_status;

enum { DSA_LAYER_FULL = 0, DSA_LAYER_SHARED = 1 };

/* Largest supported top-k width and the latent-row limits. */
enum { DSA_MAX_TOPK = 4096 };

/*
 * Ragged batch and paged-cache geometry (section "DSA Indexer fused
 * semantic op": slot_mapping / block_tables / seq_lens address the cache).
 * Request b has q_len_b = cu_q[b+1] - cu_q[b] query tokens, the last q_len_b
 * tokens of its seq_lens[b] cached tokens: query i sits at position
 * seq_lens[b] - q_len_b + i and attends to positions 0..that position (the
 * cache already holds this step's tokens).  Prefill is q_len_b = seq_lens[b].
 */
typedef struct dsa_batch {
  int32_t num_reqs;            /* B >= 1                                    */
  int32_t num_q_tokens;        /* N = cu_q[B]            (host copy)        */
  int32_t max_q_len;           /* >= every q_len_b       (host copy)        */
  int32_t max_seq_len;         /* >= every seq_lens[b]   (host copy)        */
  int32_t max_blocks;          /* row length of block_table                 */
  int32_t block_size;          /* tokens per cache block, multiple of 32    */
  int64_t num_slots;           /* rows of every paged cache buffer          */
  const int32_t* seq_lens;     /* [B]                                       */
  const int32_t* cu_q;         /* [B+1], cu_q[0] = 0, non-decreasing        */
  const int32_t* block_table;  /* [B, max_blocks] physical block ids        */
} dsa_batch;

/*
 * Indexer key-cache write (section "DSA Indexer fused semantic op", the
 * cache write of both paths; section "KV cache dtype ..." for the dtype).
 *   k_new        [n_new, d_idx] new keys, k_dtype DSA_F32 or DSA_BF16
 *   slot_mapping [n_new] int64 destination rows; -1 = padding token, skipped;
 *                rows >= num_slots are skipped too
 *   k_cache      [num_slots, d_idx] of cache_dtype
 *   k_scale      [num_slots] fp32, required iff cache_dtype == DSA_FP8_E4M3,
 *                else ignored
 * F32 / BF16 cache: the key is stored unchanged (k_dtype must equal
 * cache_dtype).  FP8 cache: per token amax = max_d |k_d| (in fp32),
 * scale = fl32(amax / 448) (1 if amax == 0), code_d = e4m3(fl32(k_d / scale))
 * with round-to-nearest-even, saturating at +-448, the sign kept; k_scale gets
 * scale.  Only the listed rows are written.  d_idx: 1..1024.
 */
int dsa_indexer_cache_write(const void* k_new, int32_t k_dtype, int32_t n_new,
                            int32_t d_idx, const int64_t* slot_mapping,
                            int64_t num_slots, void* k_cache, float* k_scale,
                            int32_t cache_dtype, void* stream);

/*
 * Indexer score + deterministic top-k (section "DSA Indexer fused semantic
 * op"; section "Performance model design", score MMA, head mixing / reduce /
 * ReLU shaping and top-k buckets; tie rule after page "GLM5 full-stack LoRA"
 * section 1).
 *   q        [N, n_heads, d_idx] query, q_dtype DSA_F32 or DSA_BF16
 *   w        [N, n_heads] fp32 head weights
 *   k_cache  [num_slots, d_idx] of cache_dtype (F32, BF16 or FP8_E4M3)
 *   k_scale  [num_slots] fp32 for an FP8 cache (the key's value is
 *            code * scale), else ignored
 *   topk_idx [N, topk] int32 output: row t holds the n = min(topk, pos_t + 1)
 *            selected positions in ascending order, then -1 up to topk.
 *            Selection order is (score descending, position ascending), so
 *            the set is unique.
 * Scores use fp32 accumulation (bf16 / fp8 operands are widened exactly).
 * Supported: q_dtype == cache_dtype for F32/BF16, q BF16 with an FP8 cache
 * (FP8 queries: dsa_indexer_topk_fp8q);
 * n_heads 1..64 and d_idx 1..256 (the matrix-core path needs n_heads % 32 == 0
 * and d_idx == 128; other shapes take a slower vector path); topk 1..4096.
 * workspace: 256-byte aligned; contents on entry are ignored.  Per query
 * token it holds an fp32 score row (max_seq_len rounded up to 64) and,
 * behind the rows, the range (min, max) of the token's scores in each key
 * chunk, which the score pass writes when rows can exceed 32768 keys so that
 * the selection, which then streams its rows from memory, needs no range
 * pass of its own.  With dsa_indexer_topk_workspace_size() bytes the whole
 * batch is scored and selected in one pass.  A smaller workspace, of at
 * least dsa_indexer_topk_workspace_min() bytes (the rows of 16 query tokens,
 * or of all of them when there are fewer), is used window by window: the
 * query tokens go through score + selection in consecutive windows of as
 * many tokens as it holds (whole blocks of 16 when it can), with the same
 * result.  Below the minimum: DSA_ERR_WORKSPACE.
 */
size_t dsa_indexer_topk_workspace_size(const dsa_batch* batch, int32_t topk);
size_t dsa_indexer_topk_workspace_min(const dsa_batch* batch, int32_t topk);
int dsa_indexer_topk(const dsa_batch* batch, const void* q, int32_t q_dtype,
                     const float* w, int32_t n_heads, int32_t d_idx,
                     const void* k_cache, const float* k_scale,
                     int32_t cache_dtype, int32_t topk, int32_t* topk_idx,
                     void* workspace, size_t ws_bytes, void* stream);

/*
 * Activation rotation and quantisation of the FP8 indexer path (section
 * "DSA Indexer fused semantic op": the DeepSeek-V3.2 FP8 path applies
 * rotate_activation and activation quantisation before the FP8 key cache /
 * scale cache write and the FP8 index score; section "Performance model
 * design", bucket 5).  Each row of d elements is rotated by the orthonormal
 * Hadamard transform (Sylvester order, scaled by d^-1/2: butterflies over
 * strides 1, 2, ..., d/2 in fp32, then one multiply by fl32(d^-1/2)) and
 * quantised like a key of an FP8 cache: scale = fl32(amax / 448) (1 if
 * amax == 0), code = e4m3(fl32(v / scale)), round to nearest even,
 * saturating.
 *   x          [n_rows, d] F32 or BF16
 *   row_slots  [n_rows] int64 output rows (-1 or >= num_out: skipped), or
 *              NULL: row i goes to output row i (n_rows <= num_out)
 *   codes      [num_out, d] e4m3 codes; scales [num_out] fp32
 * Queries: rows are the heads of each token (n_rows = N * n_heads, one scale
 * per token and head), row_slots NULL.  Keys: rows are tokens, row_slots the
 * slot mapping, codes / scales the FP8 indexer cache and its scale cache.
 * d: a power of two in 32..256.
 */
int dsa_rotate_quantize(const void* x, int32_t x_dtype, int64_t n_rows, int32_t d,
                        const int64_t* row_slots, int64_t num_out, uint8_t* codes,
                        float* scales, void* stream);

/*
 * Indexer score + top-k over e4m3 queries and an e4m3 cache (the FP8 path of
 * section "DSA Indexer fused semantic op"; section "Performance model
 * design", bucket 7: ReLU / q-scale / k-scale shaping):
 *     score[t, s] = k_scale[s] * sum_h w[t, h] * q_scale[t, h] *
 *                   ReLU(qv[t, h, :] . kv[s, :])
 * with qv, kv the values of the e4m3 codes (both rotated by
 * dsa_rotate_quantize, which keeps every dot product).  Selection, output
 * rows, workspace and errors as dsa_indexer_topk.
 *   q_codes  [N, n_heads, d_idx] e4m3;  q_scale [N, n_heads] fp32 (> 0)
 *   k_cache  [num_slots, d_idx] e4m3;  k_scale [num_slots] fp32
 * d_idx == 128 with n_heads 32 or 64 runs on the fp8 matrix cores; other
 * shapes within dsa_indexer_topk's limits take the vector path.
 */
int dsa_indexer_topk_fp8q(const dsa_batch* batch, const uint8_t* q_codes,
                          const float* q_scale, const float* w, int32_t n_heads,
                          int32_t d_idx, const void* k_cache, const float* k_scale,
                          int32_t topk, int32_t* topk_idx, void* workspace,
                          size_t ws_bytes, void* stream);

/*
 * Indexer prologue (section "DSA Indexer fused semantic op": the op's inputs
 * hidden_states, qa_normed (the MLA path's normalised query low-rank
 * activation, section "mlapo / mlapo_quant and qa_normed"), RoPE cos / sin,
 * wq_b, wk, weights_proj, the k_norm weight, head_dim and qk_rope_head_dim,
 * and the indexer cache it writes; section "Performance model design",
 * buckets 1-4).  For N new tokens:
 *     q = RoPE(qa_normed wq_b^T)                          -> q_out [N, H, D] bf16
 *     k = RoPE(RMSNorm(hidden wk^T, eps) * k_norm_weight)  -> k_out [N, D] bf16
 *     w = hidden weights_proj^T                           -> w_out [N, H] fp32
 * and k is written to the indexer cache at slot_mapping[t] (skipped when -1
 * or >= num_slots): a bf16 copy for a BF16 cache; for an FP8 cache the
 * bf16 key rotated and quantised exactly as dsa_rotate_quantize does (the
 * FP8 path), codes into k_cache and the scale into k_scale.
 *   hidden        [N, hidden_dim] bf16;  qa_normed [N, q_lora_rank] bf16
 *   cos, sin      [N, rope_dim / 2] fp32, the token's RoPE angles: dims j and
 *                 j + rope_dim / 2 (j < rope_dim / 2) of each query head and
 *                 of the key turn by angle j (rotate-half); dims past
 *                 rope_dim are left alone
 *   wq_b          [n_heads * head_dim, q_lora_rank] bf16 (linear-layer
 *                 layout [out, in]); wk [head_dim, hidden_dim] bf16;
 *                 weights_proj [n_heads, hidden_dim] bf16
 *   k_norm_weight [head_dim] fp32
 *   k_out         may be NULL; slot_mapping may be NULL (no cache write)
 * Products accumulate in fp32 over the bf16 inputs, in a fixed order (the
 * results are deterministic).  Supported: head_dim 128, rope_dim even and
 * <= head_dim, q_lora_rank and hidden_dim multiples of 32, n_heads 1..64.
 * workspace: at least dsa_indexer_prologue_workspace_size() bytes (fp32
 * partial sums), 256-byte aligned, contents ignored.
 */
typedef struct dsa_prologue_dims {
  int32_t hidden_dim, q_lora_rank, n_heads, head_dim, rope_dim;
  float eps;
} dsa_prologue_dims;
size_t dsa_indexer_prologue_workspace_size(int32_t n_tokens, const dsa_prologue_dims* dims);
int dsa_indexer_prologue(int32_t n_tokens, const dsa_prologue_dims* dims, const void* hidden,
                         const void* qa_normed, const float* cos, const float* sin,
                         const void* wq_b, const void* wk, const void* weights_proj,
                         const float* k_norm_weight, const int64_t* slot_mapping,
                         int64_t num_slots, void* k_cache, float* k_scale,
                         int32_t cache_dtype, void* q_out, void* k_out, float* w_out,
                         void* workspace, size_t ws_bytes, void* stream);

/*
 * Allocation-free variant of dsa_indexer_topk, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  Same arguments, results and errors as
 * dsa_indexer_topk, minus the workspace: its scratch (the score rows and
 * chunk ranges) lives in a static device array of
 * DSA_NOALLOC_SCRATCH_BYTES that every GPU the library runs on holds until
 * the process ends.  Nothing is allocated or freed.
 *   - A batch whose dsa_indexer_topk_workspace_size() exceeds
 *     DSA_NOALLOC_SCRATCH_BYTES is rejected with DSA_ERR_WORKSPACE before
 *     anything is enqueued (e.g. 128 query tokens of up to 64K keys fit).
 *   - `stream` must belong to the current device (else
 *     DSA_ERR_INVALID_ARG); the first call on a device looks up that
 *     device's copy of the array.
 *   - Calls share their device's array and need nothing cleared between
 *     them (every entry a call reads was written earlier in the same call);
 *     calls that may overlap on one GPU (other streams, other threads) race
 *     on it and must not be issued.
 */
enum { DSA_NOALLOC_SCRATCH_BYTES = 32 << 20 };
int dsa_indexer_topk_noalloc(const dsa_batch* batch, const void* q, int32_t q_dtype,
                             const float* w, int32_t n_heads, int32_t d_idx,
                             const void* k_cache, const float* k_scale,
                             int32_t cache_dtype, int32_t topk, int32_t* topk_idx,
                             void* stream);

/*
 * Absorbed sparse MLA over the selected latent rows (section "DSA Indexer
 * fused semantic op": topk_limit / topk_indices reach the MLA backend;
 * section "Performance model design": attention length = top-k width; page
 * "GLM5 full-stack LoRA" section 2.2: absorbed MLA).
 *   q        [N, n_heads, R + P] absorbed queries (R = kv_lora_rank,
 *            P = rope_dim)
 *   kv_cache [num_slots, R + P] latent rows: R latent dims then P rope dims
 *   topk_idx [N, topk] logical positions; entries < 0 are ignored; entries
 *            beyond the token's position are out of contract
 *   out      [N, n_heads, R] (same dtype as q): for each head
 *            sum_j softmax_j(softmax_scale * q . kv_j) * kv_j[0:R]
 *   lse      [N, n_heads] fp32 log-sum-exp of the scaled logits, or NULL
 *   softmax_scale  finite and > 0 (else DSA_ERR_INVALID_ARG)
 * A token with no valid index gets out = 0 and lse = -inf.
 * Supported: dtype DSA_F32 or DSA_BF16.  The matrix-core path takes BF16
 * with R = 512, P = 64 and n_heads == 64; other shapes (R + P <= 1024,
 * n_heads <= 128) take a vector path.
 * workspace: at least sparse_mla_attn_workspace_size() bytes (may be 0, in
 * which case workspace may be NULL), 256-byte aligned.  When the keys of a
 * token are split over several workgroups it holds their normalised bf16
 * partial outputs [N, n_split, n_heads, R], fp32 log-sum-exps [N, n_split,
 * n_heads] and, per token, a 128-byte line holding its arrival word; its
 * prior contents do not matter (arrivals are counted under a tag unique to
 * the call, and a word in which every split of the call has counted counts
 * as none, so a call captured into a HIP graph may be replayed with the tag
 * it was captured with).  Calls that may run at the same time must not
 * share a workspace.
 * The splits of a token merge their partials a part of the heads each:
 * when every workgroup of the launch fits the device at once, a split waits
 * for its token's other splits for at most DSA_MERGE_WAIT_TICKS (from the
 * environment, read at each call; ticks of 10 ns; default 2000, 0 for no
 * wait) and otherwise leaves its part to the last split.  The result does
 * not depend on the wait.
 */
size_t sparse_mla_attn_workspace_size(const dsa_batch* batch, int32_t n_heads,
                                      int32_t kv_lora_rank, int32_t rope_dim,
                                      int32_t topk, int32_t dtype);
int sparse_mla_attn(const dsa_batch* batch, const void* q,
                    const void* kv_cache, int32_t dtype, int32_t n_heads,
                    int32_t kv_lora_rank, int32_t rope_dim,
                    const int32_t* topk_idx, int32_t topk, float softmax_scale,
                    void* out, float* lse, void* workspace, size_t ws_bytes,
                    void* stream);

/*
 * GLM-5.2 IndexShare source resolution (section "GLM-5.2 IndexShare";
 * section "Configuration constraints", item 6).  Host only.
 *   types [host] n_types values, DSA_LAYER_FULL or DSA_LAYER_SHARED
 *   src   [host] out, n_layers entries: src[i] = i for a full layer, the
 *         index of the nearest preceding full layer for a shared one
 * DSA_ERR_INDEXER_TYPES if n_types < n_layers, any of the n_types values is
 * unknown, or a shared layer among the first n_layers has no preceding full
 * layer (src is then left unchanged).
 */
int dsa_resolve_indexer_sources(int32_t n_layers, const int32_t* types,
                                int32_t n_types, int32_t* src);

/* One decoder layer's tensors for indexshare_forward. */
typedef struct dsa_layer {
  const void* q_idx;     /* full: [N, n_idx_heads, d_idx]; shared: unused  */
  const float* w;        /* full: [N, n_idx_heads];       shared: unused   */
  const void* k_cache;   /* full: indexer cache [num_slots, d_idx]; shared:
                            unused (shared layers own no indexer cache)     */
  const float* k_scale;  /* full with an FP8 cache: [num_slots]             */
  int32_t* topk_idx;     /* full: [N, topk] buffer to fill; shared: unused  */
  const void* q_mla;     /* [N, n_heads, R + P]                             */
  const void* kv_cache;  /* [num_slots, R + P]                              */
  void* out;             /* [N, n_heads, R]                                 */
  float* lse;            /* [N, n_heads] or NULL                            */
} dsa_layer;

/* Dimensions shared by every layer of the stack. */
typedef struct dsa_stack_dims {
  int32_t n_idx_heads, d_idx, q_idx_dtype, idx_cache_dtype, topk;
  int32_t n_heads, kv_lora_rank, rope_dim, mla_dtype;
  float softmax_scale;
} dsa_stack_dims;

/*
 * IndexShare layer stack (section "GLM-5.2 IndexShare"; section "Trace and
 * performance results": shared layers add no indexer op, latency or cache
 * traffic).  For each layer i in order: a full layer runs
 * dsa_indexer_topk into layers[i].topk_idx; a shared layer runs no indexer
 * and uses the active top-k of its source layer unchanged; every layer then
 * runs sparse_mla_attn with its own q_mla / kv_cache.
 *   types       [host] as for dsa_resolve_indexer_sources
 *   layers      [host] n_layers entries
 *   active_topk [host] out, n_layers entries (may be NULL): the device
 *               buffer each layer attended with (the source layer's buffer)
 * Errors: DSA_ERR_INDEXER_TYPES as above; DSA_ERR_MISSING_TOPK if a full
 * layer has topk_idx == NULL; the per-op argument errors otherwise.
 * workspace: at least indexshare_forward_workspace_size() bytes.
 */
size_t indexshare_forward_workspace_size(const dsa_batch* batch,
                                         const dsa_stack_dims* dims);
int indexshare_forward(const dsa_batch* batch, int32_t n_layers,
                       const int32_t* types, int32_t n_types,
                       const dsa_layer* layers, const dsa_stack_dims* dims,
                       const int32_t** active_topk, void* workspace,
                       size_t ws_bytes, void* stream);

/*
 * Diagnostic: decode n e4m3fn codes with the same device conversion the
 * indexer's FP8 path uses (codes -> bf16 -> fp32).  For checking that
 * conversion against the format definition; not on the hot path.
 */
int dsa_fp8_decode_check(const uint8_t* codes, float* out, int32_t n,
                         void* stream);

/*
 * Checked build.  libdsa_debug.so is the same library compiled with
 * -DDSA_DEBUG: around every call it enqueues, on the call's stream, a
 * validation of the device-resident metadata the call reads against the
 * host-side bounds (the conditions the release library only clamps), canary
 * fills of the outputs and the workspace, and after the call a check that
 * every output element was written and every indexer row is a valid
 * selection.  Violations accumulate in a per-device fault word:
 */
typedef enum {
  DSA_FAULT_SEQ_LENS = 1,      /* a seq_len outside [0, max_seq_len]                 */
  DSA_FAULT_CU_Q = 2,          /* cu_q not 0 .. num_q_tokens ascending, or a q_len
                                  above max_q_len or above its request's seq_len    */
  DSA_FAULT_BLOCK_TABLE = 4,   /* a block in use past max_blocks, negative, or with
                                  rows past num_slots                                */
  DSA_FAULT_SLOT_MAPPING = 8,  /* a cache-write slot neither -1 nor in [0, num_slots) */
  DSA_FAULT_TOPK_INPUT = 16,   /* an attention index neither -1 nor in [0, pos]      */
  DSA_FAULT_TOPK_OUTPUT = 32,  /* an indexer row that is not min(topk, pos + 1)
                                  ascending positions in [0, pos] followed by -1     */
  DSA_FAULT_UNWRITTEN = 64     /* an output element still holds its canary           */
} dsa_fault;

/*
 * The calling device's fault word (OR of dsa_fault bits since the last
 * clear) into *faults [host]; clear != 0 resets it.  Waits for the device
 * to finish all queued work first (checked build only: the one call that
 * synchronises).  The release library sets *faults = 0 and returns
 * DSA_ERR_UNSUPPORTED.  NULL faults: DSA_ERR_INVALID_ARG.
 */
int dsa_debug_faults(uint32_t* faults, int32_t clear);

/* Text of the last error raised on the calling thread ("" if none). */
const char* dsa_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* DSA_H */
