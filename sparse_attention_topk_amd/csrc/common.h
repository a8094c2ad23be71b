// Shared device helpers and internal launch declarations for libdsa.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "dsa.h"

namespace dsa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;

__device__ __forceinline__ float bf16_bits_to_f32(uint16_t b) {
  return __uint_as_float(static_cast<uint32_t>(b) << 16);
}

// e4m3fn x8 (two dwords, byte order = element order) -> bf16 x8.  Exact:
// every e4m3 value is a bf16 value.
__device__ __forceinline__ bf16x8 fp8x8_to_bf16x8(uint32_t lo, uint32_t hi) {
  auto a = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, false);
  auto b = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(lo, 1.0f, true);
  auto c = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, false);
  auto d = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(hi, 1.0f, true);
  bf16x8 r;
  r[0] = a[0]; r[1] = a[1]; r[2] = b[0]; r[3] = b[1];
  r[4] = c[0]; r[5] = c[1]; r[6] = d[0]; r[7] = d[1];
  return r;
}

__device__ __forceinline__ float fp8_to_f32(uint8_t code) {
  auto v = __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(static_cast<uint32_t>(code),
                                                      1.0f, false);
  return static_cast<float>(v[0]);
}

// Workgroup barrier ordering LDS accesses only.  __syncthreads() also waits
// for every outstanding global load of the wave, which would serialise a
// register prefetch with the barrier; this one leaves them in flight.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Inclusive prefix sum over the 64 lanes of a wave with DPP moves: shifts
// within each 16-lane row, then the gfx9 row broadcasts (lane 15 of a row
// into the next row, lane 31 into the upper half).  Lanes a move does not
// reach keep 0, so each step adds only what lies below them.
__device__ __forceinline__ uint32_t wave_scan_incl(uint32_t v) {
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x111, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x112, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x114, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x118, 0xF, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x142, 0xA, 0xF, false));
  v += static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, static_cast<int>(v), 0x143, 0xC, 0xF, false));
  return v;
}

// Cross-lane reductions inside a wave with VALU moves only (no LDS round
// trip, unlike a shuffle): DPP permutations inside each 16-lane row (lane
// l ^ 1, l ^ 2, then the half-row and row mirrors), then gfx950's permlane
// swaps between rows (lanes l ^ 16, l ^ 32).
template <int Ctrl>
__device__ __forceinline__ float dpp_move(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), Ctrl, 0xF, 0xF, false));
}
// x[l] + x[l ^ 32] in every lane (the same bits as in either order)
__device__ __forceinline__ float lane_sum_x32(float x) {
  const auto c = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(c[0]) + __uint_as_float(c[1]);
}
// min and max over each 32-lane half of the wave (NaN skipped, as fminf /
// fmaxf do), in every lane of the half
__device__ __forceinline__ void half_minmax(float& lo, float& hi) {
  lo = fminf(lo, dpp_move<0xB1>(lo));    // quad_perm [1, 0, 3, 2]: lane l ^ 1
  hi = fmaxf(hi, dpp_move<0xB1>(hi));
  lo = fminf(lo, dpp_move<0x4E>(lo));    // quad_perm [2, 3, 0, 1]: lane l ^ 2
  hi = fmaxf(hi, dpp_move<0x4E>(hi));
  lo = fminf(lo, dpp_move<0x141>(lo));   // row_half_mirror: the other quad of 8
  hi = fmaxf(hi, dpp_move<0x141>(hi));
  lo = fminf(lo, dpp_move<0x140>(lo));   // row_mirror: the other 8 of 16
  hi = fmaxf(hi, dpp_move<0x140>(hi));
  const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(lo), __float_as_uint(lo), false, false);
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(hi), __float_as_uint(hi), false, false);
  lo = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  hi = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
// min and max over the whole wave, in every lane
__device__ __forceinline__ void wave_minmax(float& lo, float& hi) {
  half_minmax(lo, hi);
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(lo), __float_as_uint(lo), false, false);
  const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(hi), __float_as_uint(hi), false, false);
  lo = fminf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  hi = fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// fp32 -> OCP e4m3fn, round to nearest even, saturating, sign kept.
// NaN is outside the contract (it saturates like a large value).
__device__ __forceinline__ uint32_t f32_to_e4m3(float v) {
  uint32_t bits = __float_as_uint(v);
  uint32_t sign = (bits >> 24) & 0x80u;
  uint32_t a = bits & 0x7FFFFFFFu;
  if (a >= 0x43E00000u) return sign | 0x7Eu;          // |v| >= 448
  if (a >= 0x3C800000u) {                             // |v| >= 2^-6: normal
    // keep 3 mantissa bits: round the 20 dropped bits to nearest even; a
    // carry moves into the exponent, which is the right result
    uint32_t r = a + 0x7FFFFu + ((a >> 20) & 1u);
    return sign | ((r >> 20) - (120u << 3));          // rebias 127 -> 7
  }
  // subnormal: value = m * 2^-9 with m = rne(|v| * 512) in 0..8
  // (m == 8 is the smallest normal, code 0x08, which is also correct)
  float m = rintf(__uint_as_float(a) * 512.0f);
  return sign | static_cast<uint32_t>(m);
}

// Activation rotation and quantisation of one row by one wave (the FP8
// indexer path's rotate_activation and activation quantisation): element
// l + 64 m of the row sits in lane l, slot m (EPL = max(1, d / 64) slots;
// for d < 64 lanes d .. 63 hold zeros).  The orthonormal Hadamard transform
// runs as butterflies over h = 1, 2, ..., d / 2 in that order, (a, b) ->
// (a + b, a - b) for the pair (i, i + h) in each block of 2 h, rounded to
// fp32 at every stage, then one multiply by inv_sqrt_d = fl32(d^-1/2);
// pairs of h < 64 meet across lanes l and l ^ h, pairs of h >= 64 inside a
// lane.  The rotated row is then quantised like a key: amax, scale =
// fl32(amax / 448) (1 if amax == 0), code = e4m3(v / scale); the codes go to
// codes_row[0 .. d) and the scale to *scale_out.  Every lane of the wave
// must call it (it exchanges values across lanes).
template <int EPL>
__device__ __forceinline__ void wave_rotate_quantize(float (&v)[EPL], int d, float inv_sqrt_d,
                                                     uint8_t* __restrict__ codes_row,
                                                     float* __restrict__ scale_out) {
  const int lane = threadIdx.x & 63;
  for (int h = 1; h < 64 && h < d; h <<= 1) {
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      const float other = __shfl_xor(v[m], h);
      v[m] = (lane & h) ? other - v[m] : v[m] + other;
    }
  }
#pragma unroll
  for (int h = 1; h < EPL; h <<= 1) {    // element strides 64 h
#pragma unroll
    for (int m = 0; m < EPL; ++m) {
      if (m & h) continue;
      const float a = v[m], b = v[m + h];
      v[m] = a + b;
      v[m + h] = a - b;
    }
  }
  float amax = 0.0f;
#pragma unroll
  for (int m = 0; m < EPL; ++m) {
    v[m] *= inv_sqrt_d;
    amax = fmaxf(amax, fabsf(v[m]));
  }
  for (int off = 32; off > 0; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off));
  const float sc = (amax == 0.0f) ? 1.0f : amax / 448.0f;
  if (lane < d) {
#pragma unroll
    for (int m = 0; m < EPL; ++m)
      codes_row[lane + 64 * m] = static_cast<uint8_t>(f32_to_e4m3(v[m] / sc));
  }
  if (lane == 0) *scale_out = sc;
}

// Physical cache row of logical position s of a request, or -1 when the
// block id or slot falls outside the cache (treated as "no key").
__device__ __forceinline__ int64_t slot_of(const int32_t* bt_row, int32_t s,
                                           int32_t block_size,
                                           int32_t max_blocks,
                                           int64_t num_slots) {
  int32_t blk = s / block_size;
  if (s < 0 || blk >= max_blocks) return -1;
  int64_t slot = static_cast<int64_t>(bt_row[blk]) * block_size + s % block_size;
  return (slot >= 0 && slot < num_slots) ? slot : -1;
}

// Request that owns query token t: the largest b with cu_q[b] <= t.
__device__ __forceinline__ int request_of(const int32_t* cu_q, int32_t B,
                                          int32_t t) {
  int lo = 0, hi = B - 1;
  while (lo < hi) {
    int mid = (lo + hi + 1) >> 1;
    if (cu_q[mid] <= t) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// Same as request_of, computed by one wave on its own: cu_q is read 64
// entries per load and the entries <= t are counted with a ballot (no LDS,
// no barrier; every wave of a workgroup gets the same, wave-uniform value).
__device__ __forceinline__ int request_of_wave(const int32_t* cu_q, int32_t B, int32_t t) {
  const int lane = threadIdx.x & 63;
  int n = 0;
  for (int b0 = 0; b0 < B; b0 += 64) {
    const int b = b0 + lane;
    const int32_t c = cu_q[b < B ? b : B];      // cu_q has B + 1 entries
    n += __popcll(__ballot(b < B && c <= t));
  }
  const int r = n - 1;
  return r < 0 ? 0 : (r >= B ? B - 1 : r);
}

// Request b and position of query token t in one memory round trip when
// B < 128: cu_q[0..127] and seq_lens[0..127] are read two entries per lane
// up front, b is counted with ballots and the entries it needs are taken
// with v_readlane (every wave gets the same, wave-uniform values).  Larger
// batches take request_of_wave and query_pos.
__device__ __forceinline__ int32_t query_pos(const int32_t* seq_lens,
                                             const int32_t* cu_q, int b,
                                             int32_t t, int32_t max_seq_len);
__device__ __forceinline__ void token_place(const int32_t* cu_q, const int32_t* seq_lens,
                                            int32_t B, int32_t t, int32_t max_seq_len,
                                            int& b, int32_t& pos) {
  if (B < 128) {
    const int lane = threadIdx.x & 63;
    const int32_t c0 = cu_q[min(lane, B)], c1 = cu_q[min(lane + 64, B)];   // B + 1 entries
    const int32_t s0 = seq_lens[min(lane, B - 1)], s1 = seq_lens[min(lane + 64, B - 1)];
    const int n = __popcll(__ballot(lane < B && c0 <= t)) +
                  __popcll(__ballot(lane + 64 < B && c1 <= t));
    const int bb = n - 1 < 0 ? 0 : (n - 1 >= B ? B - 1 : n - 1);
    auto pick = [&](int32_t v0, int32_t v1, int i) {
      return i < 64 ? __builtin_amdgcn_readlane(v0, i) : __builtin_amdgcn_readlane(v1, i - 64);
    };
    const int32_t cb = pick(c0, c1, bb), ce = pick(c0, c1, bb + 1);
    const int32_t L = min(pick(s0, s1, bb), max_seq_len);
    pos = min(L - (ce - cb) + (t - cb), L - 1);
    b = bb;
    return;
  }
  b = request_of_wave(cu_q, B, t);
  pos = query_pos(seq_lens, cu_q, b, t, max_seq_len);
}

// Position of query token t of request b, clamped into [-1, max_seq_len-1].
__device__ __forceinline__ int32_t query_pos(const int32_t* seq_lens,
                                             const int32_t* cu_q, int b,
                                             int32_t t, int32_t max_seq_len) {
  int32_t L = min(seq_lens[b], max_seq_len);
  int32_t qlen = cu_q[b + 1] - cu_q[b];
  return min(L - qlen + (t - cu_q[b]), L - 1);
}

// Checked build (debug.hip): launched around every call when compiled with
// -DDSA_DEBUG.  Canaries: an index no row can hold, and NaNs with payloads
// the arithmetic does not produce from finite inputs.
constexpr int32_t kCanaryIdx = 0x7FFFFFF7;
constexpr uint32_t kCanaryBf16 = 0xFFC1u;
constexpr uint32_t kCanaryF32 = 0xFFC00001u;
constexpr uint32_t kPoisonWorkspace = 0xA5A5A5A5u;
hipError_t debug_check_batch(const dsa_batch& b, hipStream_t stream);
hipError_t debug_check_slots(const int64_t* slots, int32_t n, int64_t num_slots,
                             hipStream_t stream);
hipError_t debug_check_topk_in(const dsa_batch& b, const int32_t* idx, int32_t topk,
                               hipStream_t stream);
hipError_t debug_check_topk_out(const dsa_batch& b, const int32_t* idx, int32_t topk,
                                hipStream_t stream);
hipError_t debug_fill(void* p, size_t bytes, uint32_t pattern, hipStream_t stream);
hipError_t debug_check_unwritten(const void* p, size_t n, int elem_bytes, uint32_t canary,
                                 hipStream_t stream);
hipError_t debug_faults(uint32_t* faults, bool clear);   // synchronises the device

// Launchers (each returns hipGetLastError() after its launches).
hipError_t launch_cache_write(const void* k_new, int k_dtype, int n_new,
                              int d_idx, const int64_t* slot_mapping,
                              int64_t num_slots, void* k_cache, float* k_scale,
                              int cache_dtype, hipStream_t stream);

struct IndexerArgs {
  dsa_batch b;
  const void* q;
  int q_dtype;
  const float* q_scale;   // e4m3 queries: [N, n_heads] scales; else null
  const float* w;
  int n_heads, d_idx;
  const void* k_cache;
  const float* k_scale;
  int cache_dtype;
  int topk;
  int32_t* topk_idx;
  float* scores;          // workspace [N, max_seq_len]
  int64_t row_stride;
  // Per-chunk score ranges (workspace [N, range_stride] of (min, max)): the
  // matrix-core score pass writes, for each key chunk of kRangeParts waves,
  // the range of each token's causal scores there, so the top-k needs no
  // range pass.  Set by launch_indexer_score; null when rows are short
  // enough for the top-k's register path (see kTopkRegCap) or that pass
  // took the vector path (the top-k then finds the range itself).
  float2* chunk_range;
  int32_t range_stride;   // entries per token
  int32_t chunk_keys;     // keys per chunk
  // Query-token window of this launch pair: only tokens t in [win_lo,
  // win_hi) are scored and selected, and their score and range rows sit at
  // row t - win_lo of the workspace (a workspace smaller than the whole
  // batch's is used window by window).
  int32_t win_lo = 0, win_hi = 0;
};
constexpr int kRangeParts = 4;   // entries per chunk (one per score wave)
// Rows up to this many keys are selected from registers, where finding the
// range costs next to nothing; the score pass records ranges only for
// batches with longer rows (they are streamed in every pass).
constexpr int kTopkRegCap = 32768;
// entries per token the chunk ranges can need (chunks of at least 128 keys)
inline int64_t indexer_range_stride_max(int32_t max_seq_len) {
  return (static_cast<int64_t>(max_seq_len) + 127) / 128 * kRangeParts;
}
bool indexer_mfma_ok(const IndexerArgs& a);
hipError_t launch_indexer_score(IndexerArgs& a, hipStream_t stream);
// prefill-shaped batches (bf16 queries and keys, 32 heads of 128 dims,
// blocks of a multiple of 64 keys, at least 16 query tokens in a request):
// each key tile is reused across 16 query tokens
bool prefill_score_ok(const IndexerArgs& a);
hipError_t launch_score_prefill(IndexerArgs& a, hipStream_t stream);
hipError_t launch_topk(const IndexerArgs& a, hipStream_t stream);

struct MlaArgs {
  dsa_batch b;
  const void* q;
  const void* kv;
  int dtype;
  int n_heads, R, P;
  const int32_t* idx;
  int topk;
  float scale;
  void* out;
  float* lse;
  uint16_t* part_o;       // workspace [N, n_split, H, R] bf16 when n_split > 1
  float* part_lse;        // workspace [N, n_split, H]
  unsigned long long* arrivals;   // workspace [N] x 128 B: the token's split arrivals
  unsigned long long call_tag;    // 48-bit tag of this call, never 0
  int n_split;
};
// compute units of the current device (cached per device; 256 if the
// runtime cannot say)
inline int device_cus() {
  static int cached[64] = {0};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  if (cached[dev] == 0) {
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        n <= 0)
      n = 256;
    cached[dev] = n;
  }
  return cached[dev];
}
bool mla_mfma_ok(const dsa_batch& b, int dtype, int n_heads, int R, int P);
int mla_choose_split(const dsa_batch* b, int dtype, int n_heads, int R, int P,
                     int topk);
hipError_t launch_sparse_mla(const MlaArgs& a, hipStream_t stream);

// Hadamard-rotates and quantises rows of d (a power of two, 32 .. 256)
// elements; row i goes to output row row_slots[i] (or i when row_slots is
// null), skipped when that is negative or >= num_out.
hipError_t launch_rotate_quantize(const void* x, int x_dtype, int64_t n_rows, int d,
                                  const int64_t* row_slots, int64_t num_out, uint8_t* codes,
                                  float* scales, hipStream_t stream);

// indexer prologue: split counts, partial-sum floats, launch
void prologue_splits(int32_t N, const dsa_prologue_dims* d, int* sq, int* sk);
size_t prologue_part_floats(int32_t N, const dsa_prologue_dims* d);
hipError_t launch_prologue(int32_t N, const dsa_prologue_dims* d, const void* hidden,
                           const void* qa, const float* cos, const float* sin,
                           const void* wq_b, const void* wk, const void* wp,
                           const float* k_norm, const int64_t* slots, int64_t num_slots,
                           void* k_cache, float* k_scale, int cache_dtype, void* q_out,
                           void* k_out, float* w_out, float* part, hipStream_t stream);

hipError_t launch_fp8_decode_check(const uint8_t* codes, float* out, int n,
                                   hipStream_t stream);

}  // namespace dsa
